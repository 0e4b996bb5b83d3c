// Residual-window append: one new fp16 token per sequence written at slot
// `pos` of its full-precision residual.
// [NSNQuant summary (gist.science), Methodology §4: recent tokens are kept
//  in full precision until the residual is full; then it is quantized and
//  appended to the cache.]
#include "nsn_device.h"
#include "nsn_launch.h"

namespace nsn {

namespace {

// 16 lanes per token, 16 bytes each.
__global__ __launch_bounds__(256) void append_kernel(const uint4* __restrict__ tok, int64_t n_seq,
                                                     uint16_t* __restrict__ resid,
                                                     int64_t resid_seq_stride, int64_t pos) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n_seq * 16) return;
  const int64_t s = i / 16, part = i % 16;
  uint4* dst = reinterpret_cast<uint4*>(resid + s * resid_seq_stride + pos * kD);
  dst[part] = tok[i];
}

}  // namespace

hipError_t launch_residual_append(const uint16_t* tok, int64_t n_seq, uint16_t* resid,
                                  int64_t resid_seq_stride, int64_t pos, hipStream_t s) {
  const int64_t threads = n_seq * 16;
  const unsigned blocks = static_cast<unsigned>((threads + 255) / 256);
  hipLaunchKernelGGL(append_kernel, dim3(blocks), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(tok), n_seq, resid, resid_seq_stride, pos);
  return hipGetLastError();
}

}  // namespace nsn
