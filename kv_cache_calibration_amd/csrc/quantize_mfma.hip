// Quantize for fp16 input, 2-bit codes (m = 4) and groups of 128 tokens, on
// the matrix cores and the certified candidate tables.
// [NSNQuant summary (gist.science), Methodology §1 NSN, §2 Hadamard
//  rotation, §3 nearest codeword in one global codebook, scale adjustment.]
//
// One workgroup (4 waves) per (sequence, group of 128 tokens); wave w owns
// tokens 32w .. 32w+31, lane (t = lane % 32, half = lane / 32).
//
// 1. Rotation on MFMA.  The Sylvester matrix factors as H128 = H8 (x) H16, so
//    every 32x16 block of H is +-(one fixed 16-column pattern) with a sign
//    that depends only on the block and on bit 4 of the row; the +-1 entries
//    and the fp16 input are exact, and v_mfma_f32_32x32x16_f16 accumulates in
//    fp32.  Token-major pass: D[c][t] = (H x_t)[c] -- lane (t, half) gets the
//    channels {32mb + 8q + 4half + e}, i.e. sub-vectors j = 8mb + 2q + half,
//    each as four consecutive registers.  Channel-major pass (same operand
//    registers, roles swapped): D[t][c], used for the per-channel group sums.
// 2. NSN in the rotated domain: s1 from the token norm, the group mean from
//    the channel-major pass weighted by 1/s1 (exactly the pages' Shift, since
//    the rotation is linear and orthonormal), z = y - o', s2 = ||z||/sqrt(d).
// 3. Nearest codeword: the sub-vector's box in the 24^4 quantile grid gives
//    four candidate codes (one L2-resident u32); the exact squared distance
//    in fp32 and a lexicographic (distance bits, code) key pick the lowest
//    code among equal distances.  Boxes with more candidates and points off
//    the grid go to a per-wave LDS queue, finished cooperatively (extra
//    candidates from the pool, or a full scan) with an LDS 64-bit atomic min
//    on the same key.
// 4. Scale adjustment alpha = ||h||^2 / <h, h_hat>, codes, (s1, s2'), o'.
#include "nsn_device.h"
#include "nsn_launch.h"

namespace nsn {

namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kG = 128;
constexpr int kNW = kG / 32;       // waves per workgroup
constexpr int kQCap = 256;         // overflow queue entries per wave
constexpr float kSqrtD = 11.313708498984761f;

struct QEntry {
  float h[4];
  uint32_t slot;   // sub-vector * 32 + token
  int32_t cell;    // -1: off the grid (full scan)
};

__device__ __forceinline__ uint64_t dist_key(float d, uint32_t code) {
  return (static_cast<uint64_t>(__float_as_uint(d)) << 32) | code;
}

__device__ __forceinline__ float sqdist4(const float* h, const float* c) {
  const float d0 = h[0] - c[0], d1 = h[1] - c[1], d2 = h[2] - c[2], d3 = h[3] - c[3];
  return fmaf(d3, d3, fmaf(d2, d2, fmaf(d1, d1, d0 * d0)));
}

__device__ __forceinline__ v8h as_v8h(u32x4 v) { return __builtin_bit_cast(v8h, v); }

__global__ __launch_bounds__(kG * 2) void quantize_mfma_kernel(
    const __half* __restrict__ x, int64_t n_groups, int64_t x_seq_stride,
    const uint8_t* __restrict__ table, uint8_t* __restrict__ codes, int64_t codes_seq_stride,
    uint16_t* __restrict__ meta, int64_t meta_seq_stride, uint16_t* __restrict__ shift,
    int64_t shift_seq_stride, int scale_adjust) {
  __shared__ __attribute__((aligned(16))) float cb[kCodes * 4];
  __shared__ __attribute__((aligned(16))) uint8_t binlut[kFine];
  __shared__ float ascale[kG];
  __shared__ float csum[kNW][kD];
  __shared__ __attribute__((aligned(16))) float osh[kD];
  __shared__ uint64_t res[kNW][32 * 32];   // [sub-vector][token]: lanes hit distinct banks
  __shared__ QEntry queue[kNW][kQCap];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int t = lane & 31, hf = lane >> 5;
  const int64_t seq = blockIdx.x / n_groups;
  const int64_t grp = blockIdx.x - seq * n_groups;
  const int tg = 32 * w + t;                          // token within the group
  const int64_t tok = grp * kG + tg;

  {
    const float* cbg = reinterpret_cast<const float*>(table + kTabCodebook);
    for (int i = tid; i < kCodes * 4; i += kG * 2) cb[i] = cbg[i];
    const uint32_t* bl = reinterpret_cast<const uint32_t*>(table + kTabBinLut);
    uint32_t* bd = reinterpret_cast<uint32_t*>(binlut);
    for (int i = tid; i < kFine / 4; i += kG * 2) bd[i] = bl[i];
  }

  // ---- operands: x (fp16, 8 x 16 bytes per lane) and the H16 sign pattern
  const __half* row = x + seq * x_seq_stride + tok * kD;
  u32x4 xv[8];
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) xv[kb] = load_nt16(row + 16 * kb + 8 * hf);
  u32x4 P0, P1;
  {
    const int r16 = lane & 15, r4 = (lane >> 4) & 1;
    uint32_t wv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c0 = 8 * hf + 2 * i, c1 = c0 + 1;
      const uint32_t lo = (__popc(r16 & c0) & 1) ? 0xBC00u : 0x3C00u;
      const uint32_t hi = (__popc(r16 & c1) & 1) ? 0xBC00u : 0x3C00u;
      wv[i] = lo | (hi << 16);
    }
    P0 = u32x4{wv[0], wv[1], wv[2], wv[3]};
    const uint32_t f = r4 ? 0x80008000u : 0u;   // odd blocks: sign of bit 4 of the row
    P1 = u32x4{wv[0] ^ f, wv[1] ^ f, wv[2] ^ f, wv[3] ^ f};
  }
  const u32x4 N0 = P0 ^ 0x80008000u, N1 = P1 ^ 0x80008000u;
  // block (a, kb) of H: sign (-1)^popcount(2a & kb), times bit-4 sign for odd kb
#define HBLK(a, kb) as_v8h((__popc((2 * (a)) & (kb)) & 1) ? (((kb) & 1) ? N1 : N0) : (((kb) & 1) ? P1 : P0))

  // ---- token-major rotation: acc[mb][r] = (H x_t)[32mb + 8(r/4) + 4hf + r%4]
  v16f acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) acc[mb] = v16f{};
#pragma unroll
  for (int kb = 0; kb < 8; ++kb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(HBLK(mb, kb), as_v8h(xv[kb]), acc[mb], 0, 0, 0);

  // s1 = ||x|| / sqrt(d) = ||H x|| / d ;  y = acc * a with a = sqrt(d) / ||H x||
  float ss = 0.f;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) ss = fmaf(acc[mb][r], acc[mb][r], ss);
  ss += __shfl_xor(ss, 32, kWave);
  const float nrm = sqrtf(ss);
  const float s1 = nrm * (1.0f / kD);
  const float a_t = nrm > 0.f ? kSqrtD / nrm : 0.f;
  if (hf == 0) ascale[tg] = a_t;
  __syncthreads();

  // ---- channel-major rotation for the group mean: lane holds tokens
  //      {8q + 4hf + e} of this wave for channel 32nb + t
  {
    float av[16];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) av[4 * q + e] = ascale[32 * w + 8 * q + 4 * hf + e];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      v16f c2 = v16f{};
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_v8h(xv[kb]), HBLK(nb, kb), c2, 0, 0, 0);
      float s = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) s = fmaf(av[r], c2[r], s);
      s += __shfl_xor(s, 32, kWave);
      if (hf == 0) csum[w][32 * nb + t] = s;
    }
  }
#undef HBLK
  __syncthreads();
  if (tid < kD) {
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < kNW; ++ww) s += csum[ww][tid];
    osh[tid] = s * (1.0f / kG);
  }
  __syncthreads();

  // ---- z = y - o' (in place), s2
  float ss2 = 0.f;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 o = *reinterpret_cast<const float4*>(&osh[32 * mb + 8 * q + 4 * hf]);
      const float ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float z = fmaf(acc[mb][4 * q + e], a_t, -ov[e]);
        acc[mb][4 * q + e] = z;
        ss2 = fmaf(z, z, ss2);
      }
    }
  ss2 += __shfl_xor(ss2, 32, kWave);
  const float s2 = sqrtf(ss2 * (1.0f / kD));
  const float inv2 = s2 > 0.f ? 1.0f / s2 : 0.f;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][r] *= inv2;   // h

  // ---- nearest codeword, four sub-vectors (one mb block) at a time
  const uint32_t* tmain = reinterpret_cast<const uint32_t*>(table + kTabMain);
  const uint32_t* text = reinterpret_cast<const uint32_t*>(table + kTabExt);
  const uint8_t* tpool = table + kTabPool;
  uint64_t* myres = res[w];
  QEntry* myq = queue[w];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    int cell[4];
    bool off[4];
    uint32_t mainv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int c = 0;
      bool o = false;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float fe = floorf(fmaf(acc[mb][4 * q + e], kFineInv, 512.0f));
        o |= !(fe >= 0.f && fe < static_cast<float>(kFine));   // also catches NaN
        const int fi = o ? 0 : static_cast<int>(fe);
        c = c * kNB + binlut[fi];
      }
      cell[q] = min(c, kCells - 1);   // in bounds even for an unprepared table
      off[q] = o;
      mainv[q] = o ? 0u : tmain[cell[q]];
    }
    uint32_t flagged = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float hv[4] = {acc[mb][4 * q], acc[mb][4 * q + 1], acc[mb][4 * q + 2], acc[mb][4 * q + 3]};
      uint64_t best = ~uint64_t(0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t k = (mainv[q] >> (8 * i)) & 0xffu;
        const float4 cw = *reinterpret_cast<const float4*>(&cb[4 * k]);
        const float cv[4] = {cw.x, cw.y, cw.z, cw.w};
        const uint64_t key = dist_key(sqdist4(hv, cv), k);
        best = key < best ? key : best;
      }
      const int j = 8 * mb + 2 * q + hf;
      myres[j * 32 + t] = best;
      const bool over = off[q] || ((mainv[q] & 0xffu) > ((mainv[q] >> 8) & 0xffu));
      flagged |= over ? (1u << q) : 0u;
    }
    // push overflow entries (wave-uniform bookkeeping, no atomics)
    int qn = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool over = (flagged >> q) & 1u;
      const uint64_t bal = __ballot(over);
      if (over) {
        const int rank = qn + __popcll(bal & ((uint64_t(1) << lane) - 1));
        QEntry e;
        e.h[0] = acc[mb][4 * q];
        e.h[1] = acc[mb][4 * q + 1];
        e.h[2] = acc[mb][4 * q + 2];
        e.h[3] = acc[mb][4 * q + 3];
        e.slot = static_cast<uint32_t>((8 * mb + 2 * q + hf) * 32 + t);
        e.cell = off[q] ? -1 : cell[q];
        myq[rank] = e;
      }
      qn += __popcll(bal);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // finish the queued sub-vectors cooperatively
    for (int qi = lane; qi < qn; qi += kWave) {
      const QEntry e = myq[qi];
      uint64_t best = ~uint64_t(0);
      uint32_t ext = kExtBrute;
      if (e.cell >= 0) ext = text[e.cell];
      if (ext != kExtBrute && (ext >> 8) + (ext & 0xffu) > kPoolBytes) ext = kExtBrute;
      if (ext == kExtBrute) {
        for (int k = 0; k < kCodes; ++k) {
          const float4 cw = *reinterpret_cast<const float4*>(&cb[4 * k]);
          const float cv[4] = {cw.x, cw.y, cw.z, cw.w};
          const uint64_t key = dist_key(sqdist4(e.h, cv), static_cast<uint32_t>(k));
          best = key < best ? key : best;
        }
      } else {
        const uint32_t o = ext >> 8, n = ext & 0xffu;
        for (uint32_t i = 0; i < n; ++i) {
          const uint32_t k = tpool[o + i];
          const float4 cw = *reinterpret_cast<const float4*>(&cb[4 * k]);
          const float cv[4] = {cw.x, cw.y, cw.z, cw.w};
          const uint64_t key = dist_key(sqdist4(e.h, cv), k);
          best = key < best ? key : best;
        }
      }
      atomicMin(reinterpret_cast<unsigned long long*>(&myres[e.slot]),
                static_cast<unsigned long long>(best));
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- scale adjustment, codes, metadata
  float dot = 0.f, hh = 0.f;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t k = static_cast<uint32_t>(myres[(8 * mb + 2 * q + hf) * 32 + t]) & 0xffu;
      const float4 cw = *reinterpret_cast<const float4*>(&cb[4 * k]);
      const float cv[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dot = fmaf(acc[mb][4 * q + e], cv[e], dot);
        hh = fmaf(acc[mb][4 * q + e], acc[mb][4 * q + e], hh);
      }
    }
  dot += __shfl_xor(dot, 32, kWave);
  hh += __shfl_xor(hh, 32, kWave);
  const float alpha = (scale_adjust && dot > 0.f) ? hh / dot : 1.0f;

  uint32_t pk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      v |= (static_cast<uint32_t>(myres[(16 * hf + 4 * i + b) * 32 + t]) & 0xffu) << (8 * b);
    pk[i] = v;
  }
  *reinterpret_cast<u32x4*>(codes + seq * codes_seq_stride + tok * 32 + 16 * hf) =
      u32x4{pk[0], pk[1], pk[2], pk[3]};
  if (hf == 0) {
    const uint32_t mv = static_cast<uint32_t>(f2h(s1)) |
                        (static_cast<uint32_t>(f2h(s2 * alpha)) << 16);
    *reinterpret_cast<uint32_t*>(meta + seq * meta_seq_stride + 2 * tok) = mv;
  }
  if (tid < kD) shift[seq * shift_seq_stride + grp * kD + tid] = f2h(osh[tid]);
}

}  // namespace

bool quantize_mfma_supported(int in_f32, int sub_dim, int group_size) {
  return !in_f32 && sub_dim == 4 && group_size == kG;
}

hipError_t launch_quantize_mfma(const QuantArgs& a, hipStream_t s) {
  const int64_t n_groups = a.n_tok / kG;
  const int64_t blocks = a.n_seq * n_groups;
  hipLaunchKernelGGL(quantize_mfma_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kG * 2), 0, s,
                     static_cast<const __half*>(a.x), n_groups, a.x_seq_stride,
                     static_cast<const uint8_t*>(a.table), a.codes, a.codes_seq_stride, a.meta,
                     a.meta_seq_stride, a.shift, a.shift_seq_stride, a.scale_adjust);
  return hipGetLastError();
}

}  // namespace nsn
