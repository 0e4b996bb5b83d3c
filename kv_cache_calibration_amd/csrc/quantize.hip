// NSNQuant quantize and dequantize kernels for gfx950.
//
// Quantize [NSNQuant summary (gist.science), Methodology §1 NSN, §2 Hadamard,
// §3 VQ with one global codebook and scale adjustment], for the shapes the
// matrix-core kernels do not take (fp32 input, groups of 256): one workgroup
// per (sequence, token group), one lane per token.  The token's 128 channels
// live in VGPRs for the whole pass, so the input is read from HBM exactly
// once and every intermediate stays on chip.
//
// The rotation is applied first and NSN then runs in the rotated domain.
// This is the same result as the pages' order (NSN, then rotation): the
// orthonormal rotation keeps token norms (s1, s2 unchanged) and commutes
// with the group mean (the stored shift is the rotated mean, which is what
// dequantization and attention consume).  The randomized rotation (§2)
// negates the channels its signs select before the transform; the inverse
// negates them after it.
#include "nsn_device.h"
#include "nsn_launch.h"

namespace nsn {

namespace {

constexpr float kInvSqrtD = 0.08838834764831845f;  // 1/sqrt(128)

// Load one 128-channel row into fp32 registers with 16-byte loads.
__device__ __forceinline__ void load_row(const __half* __restrict__ row, float (&v)[kD]) {
#pragma unroll
  for (int i = 0; i < kD / 8; ++i) {
    const u32x4 w = load_nt16(row + 8 * i);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[8 * i + 2 * k] = h2f(static_cast<uint16_t>(u[k] & 0xffffu));
      v[8 * i + 2 * k + 1] = h2f(static_cast<uint16_t>(u[k] >> 16));
    }
  }
}
__device__ __forceinline__ void load_row(const float* __restrict__ row, float (&v)[kD]) {
#pragma unroll
  for (int i = 0; i < kD / 4; ++i) {
    const f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + 4 * i));
    v[4 * i] = w.x;
    v[4 * i + 1] = w.y;
    v[4 * i + 2] = w.z;
    v[4 * i + 3] = w.w;
  }
}

template <typename TIn, int M, int G>
__global__ __launch_bounds__(G) void quantize_kernel(
    const TIn* __restrict__ x, int64_t n_groups, int64_t x_seq_stride,
    const uint8_t* __restrict__ table, uint8_t* __restrict__ codes,
    int64_t codes_seq_stride, uint16_t* __restrict__ meta,
    int64_t meta_seq_stride, uint16_t* __restrict__ shift,
    int64_t shift_seq_stride, int scale_adjust, Signs sg) {
  constexpr int NSUB = kD / M;
  __shared__ float cb[kCodes * M];
  __shared__ float tile[G][33];
  __shared__ float part[G / 32][32];
  __shared__ float osh[kD];
  __shared__ __attribute__((aligned(16))) uint8_t binlut[M == 4 ? kFine : 4];   // quantile bin of each fine cell

  const int tid = threadIdx.x;
  const int64_t seq = blockIdx.x / n_groups;
  const int64_t grp = blockIdx.x - seq * n_groups;
  const int64_t tok = grp * G + tid;

  const float* cbg = reinterpret_cast<const float*>(table + kTabCodebook);
  for (int i = tid; i < kCodes * M; i += G) cb[i] = cbg[i];
  if constexpr (M == 4) {
    const uint32_t* bl = reinterpret_cast<const uint32_t*>(table + kTabBinLut);
    for (int i = tid; i < kFine / 4; i += G) reinterpret_cast<uint32_t*>(binlut)[i] = bl[i];
  }

  float v[kD];
  load_row(x + seq * x_seq_stride + tok * kD, v);
  if (any_sign(sg)) {
#pragma unroll
    for (int i = 0; i < kD; ++i) v[i] = flip_sign(v[i], sign_bit(sg, i));
  }

  // Rotation (unnormalized Sylvester transform, then 1/sqrt(d)) and the
  // first token-wise normalization: s1 = ||x|| / sqrt(d).
  fwht_regs<kD>(v);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kD; ++i) {
    v[i] *= kInvSqrtD;
    ss = fmaf(v[i], v[i], ss);
  }
  const float s1 = sqrtf(ss * (1.0f / kD));
  const float inv1 = s1 > 0.f ? 1.0f / s1 : 0.f;
#pragma unroll
  for (int i = 0; i < kD; ++i) v[i] *= inv1;

  // Shift: per-channel mean over the G tokens of the group, reduced through
  // LDS in four 32-channel slices (padded rows avoid bank conflicts).
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int k = 0; k < 32; ++k) tile[tid][k] = v[32 * q + k];
    __syncthreads();
    {
      const int c = tid & 31, b = tid >> 5;
      float s = 0.f;
#pragma unroll 8
      for (int r = 0; r < 32; ++r) s += tile[b * 32 + r][c];
      part[b][c] = s;
    }
    __syncthreads();
    if (tid < 32) {
      float t = 0.f;
#pragma unroll
      for (int b = 0; b < G / 32; ++b) t += part[b][tid];
      osh[32 * q + tid] = t * (1.0f / G);
    }
  }
  __syncthreads();

  // Second normalization.
  float ss2 = 0.f;
#pragma unroll
  for (int i = 0; i < kD; ++i) {
    v[i] -= osh[i];
    ss2 = fmaf(v[i], v[i], ss2);
  }
  const float s2 = sqrtf(ss2 * (1.0f / kD));
  const float inv2 = s2 > 0.f ? 1.0f / s2 : 0.f;
  float hh = 0.f;
#pragma unroll
  for (int i = 0; i < kD; ++i) {
    v[i] *= inv2;
    hh = fmaf(v[i], v[i], hh);
  }

  // Nearest codeword of every sub-vector: the smallest exact squared
  // distance, ties to the lowest index (the key (distance bits, code) is
  // minimized; distances are >= 0, so their bits order like their values).
  // m = 4: the sub-vector's cell of the quantile grid lists every code that
  // can be nearest anywhere in it (up to eight, one L2-resident u64); cells
  // with more and points off the grid scan all 256 codes, as m = 8 always
  // does.
  uint32_t packed[NSUB / 4];
#pragma unroll
  for (int w = 0; w < NSUB / 4; ++w) packed[w] = 0u;
  float dot = 0.f;
  const uint64_t* tmain = reinterpret_cast<const uint64_t*>(table + kTabMain);
  // m = 4: the cells of eight sub-vectors are located first and their eight
  // table words loaded together, so the lookups' latencies overlap.
  constexpr int kBatch = M == 4 ? 8 : 1;
#pragma unroll
  for (int j0 = 0; j0 < NSUB; j0 += kBatch) {
    uint64_t wv[kBatch];
    bool off[kBatch];
    if constexpr (M == 4) {
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        int cell = 0;
        off[b] = false;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float fe = floorf(fmaf(v[M * (j0 + b) + e], kFineInv, 512.0f));
          const bool oe = !(fe >= 0.f && fe < static_cast<float>(kFine));   // off the grid or NaN
          off[b] |= oe;
          cell = cell * kNB + binlut[oe ? 0 : static_cast<int>(fe)];
        }
        wv[b] = tmain[off[b] ? 0 : min(cell, kCells - 1)];
      }
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int j = j0 + b;
      uint64_t best = ~uint64_t(0);
      auto eval = [&](uint32_t k) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < M; ++e) {
          const float t = v[M * j + e] - cb[k * M + e];
          d = fmaf(t, t, d);
        }
        const uint64_t key = (static_cast<uint64_t>(__float_as_uint(d)) << 32) | k;
        best = key < best ? key : best;
      };
      bool scan = true;
      if constexpr (M == 4) {
        scan = off[b] || cand_more_than_8(wv[b]);
        if (!scan) {
#pragma unroll
          for (int i = 0; i < 4; ++i) eval(static_cast<uint32_t>(wv[b] >> (8 * i)) & 0xffu);
          if (cand_more_than_4(wv[b])) {
#pragma unroll
            for (int i = 4; i < 8; ++i) eval(static_cast<uint32_t>(wv[b] >> (8 * i)) & 0xffu);
          }
        }
      }
      if constexpr (M == 4) {
        // The rare sub-vectors that need all 256 codes are scanned by the
        // whole wave, one at a time: broadcast, four codes per lane, then the
        // wave minimum of the (distance, code) key.
        const int lane = tid & (kWave - 1);
        uint64_t need = __ballot(scan);
        while (need) {
          const int l = __builtin_ctzll(need);
          need &= need - 1;
          float hb[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            hb[e] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[M * j + e]), l));
          uint32_t dk = 0xffffffffu, ck = 0xffffffffu;   // this lane's best (distance bits, code)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t k = static_cast<uint32_t>(lane + kWave * r);
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float t = hb[e] - cb[k * 4 + e];
              d = fmaf(t, t, d);
            }
            const uint32_t db = __float_as_uint(d);
            ck = (db < dk || (db == dk && k < ck)) ? k : ck;
            dk = db < dk ? db : dk;
          }
#pragma unroll
          for (int o = kWave / 2; o >= 1; o >>= 1) {
            const uint32_t d2 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(dk), o, kWave));
            const uint32_t c2 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(ck), o, kWave));
            ck = (d2 < dk || (d2 == dk && c2 < ck)) ? c2 : ck;
            dk = d2 < dk ? d2 : dk;
          }
          if (lane == l) best = (static_cast<uint64_t>(dk) << 32) | ck;
        }
      } else if (scan) {
#pragma unroll 4
        for (uint32_t k = 0; k < kCodes; ++k) eval(k);
      }
      const uint32_t bi = static_cast<uint32_t>(best & 0xffu);
#pragma unroll
      for (int e = 0; e < M; ++e) dot = fmaf(v[M * j + e], cb[bi * M + e], dot);
      packed[j / 4] |= bi << (8 * (j % 4));
    }
  }

  // Scale adjustment: alpha = ||h||^2 / <h, h_hat>, folded into s2.
  const float alpha = (scale_adjust && dot > 0.f) ? hh / dot : 1.0f;

  uint4* cdst = reinterpret_cast<uint4*>(codes + seq * codes_seq_stride + tok * NSUB);
#pragma unroll
  for (int w = 0; w < NSUB / 16; ++w)
    cdst[w] = make_uint4(packed[4 * w], packed[4 * w + 1], packed[4 * w + 2], packed[4 * w + 3]);
  const uint32_t mv = static_cast<uint32_t>(f2h(s1)) |
                      (static_cast<uint32_t>(f2h(s2 * alpha)) << 16);
  *reinterpret_cast<uint32_t*>(meta + seq * meta_seq_stride + 2 * tok) = mv;
  if (tid < kD) shift[seq * shift_seq_stride + grp * kD + tid] = f2h(osh[tid]);
}

template <typename TOut> __device__ __forceinline__ void store_row(TOut* row, const float (&v)[kD]);
template <> __device__ __forceinline__ void store_row<float>(float* row, const float (&v)[kD]) {
  float4* p = reinterpret_cast<float4*>(row);
#pragma unroll
  for (int i = 0; i < kD / 4; ++i)
    p[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}
template <> __device__ __forceinline__ void store_row<__half>(__half* row, const float (&v)[kD]) {
  uint4* p = reinterpret_cast<uint4*>(row);
#pragma unroll
  for (int i = 0; i < kD / 8; ++i) {
    uint32_t u[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      u[k] = static_cast<uint32_t>(f2h(v[8 * i + 2 * k])) |
             (static_cast<uint32_t>(f2h(v[8 * i + 2 * k + 1])) << 16);
    p[i] = make_uint4(u[0], u[1], u[2], u[3]);
  }
}

// Dequantize [NSNQuant summary §1: the byproducts reconstruct the tensor;
// §4: dequantization kernel]: x_hat = R^T [ s1 (s2' c + o') ], R^T = H/sqrt(d)
// (D H / sqrt(d) for the randomized rotation).
// DQ: s1 and o' come from the group's 4-bit record (§3, Double
// Quantization), s2' from the one-fp16-per-token meta.
template <typename TOut, int M, int G, bool DQ>
__global__ __launch_bounds__(G) void dequantize_kernel(
    const uint8_t* __restrict__ codes, int64_t codes_seq_stride,
    const uint16_t* __restrict__ meta, int64_t meta_seq_stride,
    const uint16_t* __restrict__ shift, int64_t shift_seq_stride,
    const uint8_t* __restrict__ table, int64_t n_groups, TOut* __restrict__ out,
    int64_t out_seq_stride, Signs sg) {
  constexpr int NSUB = kD / M;
  __shared__ float cb[kCodes * M];
  __shared__ float osh[kD];
  const int tid = threadIdx.x;
  const int64_t seq = blockIdx.x / n_groups;
  const int64_t grp = blockIdx.x - seq * n_groups;
  const int64_t tok = grp * G + tid;

  const float* cbg = reinterpret_cast<const float*>(table + kTabCodebook);
  for (int i = tid; i < kCodes * M; i += G) cb[i] = cbg[i];
  float s1, s2;
  if constexpr (DQ) {
    static_assert(G == kD, "one thread per channel and per token");
    const uint8_t* rec = reinterpret_cast<const uint8_t*>(shift + seq * shift_seq_stride + grp * kDqRecU16);
    const uint2 hd = *reinterpret_cast<const uint2*>(rec);
    osh[tid] = dq_nibble_o(rec[8 + tid / 2], tid & 1, h2f(static_cast<uint16_t>(hd.y & 0xffffu)));
    s1 = dq_nibble_s1(rec[8 + kD / 2 + tid / 2], tid & 1, h2f(static_cast<uint16_t>(hd.x & 0xffffu)),
                      h2f(static_cast<uint16_t>(hd.x >> 16)));
    s2 = h2f(meta[seq * meta_seq_stride + tok]);
  } else {
    if (tid < kD) osh[tid] = h2f(shift[seq * shift_seq_stride + grp * kD + tid]);
    const uint32_t mv = *reinterpret_cast<const uint32_t*>(meta + seq * meta_seq_stride + 2 * tok);
    s1 = h2f(static_cast<uint16_t>(mv & 0xffffu));
    s2 = h2f(static_cast<uint16_t>(mv >> 16));
  }

  uint32_t packed[NSUB / 4];
  const uint4* csrc = reinterpret_cast<const uint4*>(codes + seq * codes_seq_stride + tok * NSUB);
#pragma unroll
  for (int w = 0; w < NSUB / 16; ++w) {
    const uint4 c = csrc[w];
    packed[4 * w] = c.x;
    packed[4 * w + 1] = c.y;
    packed[4 * w + 2] = c.z;
    packed[4 * w + 3] = c.w;
  }
  __syncthreads();

  float v[kD];
#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    const int code = (packed[j / 4] >> (8 * (j % 4))) & 0xff;
#pragma unroll
    for (int e = 0; e < M; ++e) v[M * j + e] = s1 * fmaf(s2, cb[code * M + e], osh[M * j + e]);
  }
  fwht_regs<kD>(v);
#pragma unroll
  for (int i = 0; i < kD; ++i) v[i] *= kInvSqrtD;
  if (any_sign(sg)) {
#pragma unroll
    for (int i = 0; i < kD; ++i) v[i] = flip_sign(v[i], sign_bit(sg, i));
  }
  store_row<TOut>(out + seq * out_seq_stride + tok * kD, v);
}

template <typename TIn, int M, int G>
hipError_t quant_launch(const QuantArgs& a, hipStream_t s) {
  const int64_t n_groups = a.n_tok / G;
  const int64_t blocks = a.n_seq * n_groups;
  hipLaunchKernelGGL((quantize_kernel<TIn, M, G>), dim3(static_cast<unsigned>(blocks)), dim3(G), 0, s,
                     static_cast<const TIn*>(a.x), n_groups, a.x_seq_stride,
                     static_cast<const uint8_t*>(a.table), a.codes, a.codes_seq_stride, a.meta,
                     a.meta_seq_stride, a.shift, a.shift_seq_stride, a.scale_adjust, a.rht);
  return hipGetLastError();
}

template <typename TOut, int M, int G, bool DQ = false>
hipError_t dequant_launch(const DequantArgs& a, hipStream_t s) {
  const int64_t n_groups = a.n_tok / G;
  const int64_t blocks = a.n_seq * n_groups;
  hipLaunchKernelGGL((dequantize_kernel<TOut, M, G, DQ>), dim3(static_cast<unsigned>(blocks)), dim3(G), 0, s,
                     a.codes, a.codes_seq_stride, a.meta, a.meta_seq_stride, a.shift,
                     a.shift_seq_stride, static_cast<const uint8_t*>(a.table), n_groups,
                     static_cast<TOut*>(a.out), a.out_seq_stride, a.rht);
  return hipGetLastError();
}

template <typename TIn, int M>
hipError_t quant_g(const QuantArgs& a, hipStream_t s) {
  return a.group_size == 128 ? quant_launch<TIn, M, 128>(a, s) : quant_launch<TIn, M, 256>(a, s);
}
template <typename TOut, int M>
hipError_t dequant_g(const DequantArgs& a, hipStream_t s) {
  if (a.dq) return a.group_size == 128 ? dequant_launch<TOut, M, 128, true>(a, s) : hipErrorInvalidValue;
  return a.group_size == 128 ? dequant_launch<TOut, M, 128>(a, s)
                             : dequant_launch<TOut, M, 256>(a, s);
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  if (a.n_seq == 0 || a.n_tok == 0) return hipSuccess;
  if (quantize_mfma_supported(a.in_f32, a.sub_dim, a.group_size)) return launch_quantize_mfma(a, s);
  if (a.dq) return hipErrorInvalidValue;   // double quantization runs on the matrix-core kernels only
  if (a.in_f32) return a.sub_dim == 4 ? quant_g<float, 4>(a, s) : quant_g<float, 8>(a, s);
  return a.sub_dim == 4 ? quant_g<__half, 4>(a, s) : quant_g<__half, 8>(a, s);
}

hipError_t launch_dequantize(const DequantArgs& a, hipStream_t s) {
  if (a.n_seq == 0 || a.n_tok == 0) return hipSuccess;
  if (a.out_f32) return a.sub_dim == 4 ? dequant_g<float, 4>(a, s) : dequant_g<float, 8>(a, s);
  return a.sub_dim == 4 ? dequant_g<__half, 4>(a, s) : dequant_g<__half, 8>(a, s);
}

}  // namespace nsn
