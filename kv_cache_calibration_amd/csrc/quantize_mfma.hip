// Quantize for fp16 input and groups of 128 tokens on the matrix cores:
// 2-bit codes (m = 4) through certified candidate tables, 1-bit codes (m = 8)
// through an exhaustive matrix-core search.
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
//    channels {32mb + 8q + 4half + e}: for m = 4 the sub-vectors
//    j = 8mb + 2q + half, each as four consecutive registers; for m = 8 half
//    of sub-vector j = 4mb + q.  Channel-major pass (same operand registers,
//    roles swapped): D[t][c], used for the per-channel group sums.
//    The randomized rotation (signs given) negates the selected channels of
//    the staged fp16 input first (sign-bit flips, exact).
// 2. NSN in the rotated domain: s1 from the token norm, the group mean from
//    the channel-major pass weighted by 1/s1 (exactly the pages' Shift, since
//    the rotation is linear and orthonormal), z = y - o', s2 = ||z||/sqrt(d).
// 3a. Nearest codeword, m = 4: h = z / s2 is never formed: the search
//    compares ||z - s2 c||^2, which orders the codewords as ||h - c||^2 does.
//    The sub-vector's box in the 24^4 quantile grid gives up to eight
//    candidate codes (one L2-resident u64), evaluated in place with the exact
//    squared distance in fp32 in ascending code order, so ties keep the
//    lowest index (the second four only when some lane of the wave has more
//    than four).  Boxes with more than eight candidates and points off the
//    grid are rare: the whole wave scans all 256 codes for them, one
//    sub-vector at a time (broadcast by readlane, then a wave minimum of the
//    distance and of the code among equal distances).
// 3b. Nearest codeword, m = 8: for each sub-vector index j the wave forms
//    D[c][t] = ||c||^2 + H_t - 2 <c, h_t> for all 256 codes c and its 32
//    tokens t with two MFMAs per 32-code tile.  h enters as an fp16 pair
//    (hi + lo, 22 significant bits), the codebook is exact in fp16, ||c||^2
//    as an fp16 pair, and H_t >= ||h_t||^2 (rounded up) keeps every value
//    non-negative.  Each lane then takes the minimum of its 16 values per
//    tile with the row number in the four low mantissa bits (a key that
//    orders like the distance to within 15 ulp, ties to the lowest code),
//    keeps the best tile, and the two lane halves of a token settle the
//    final code.
// 4. Scale adjustment alpha = ||h||^2 / <h, h_hat>, codes, (s1, s2'), o';
//    with double quantization (template flag DQ) s2' alone per token and one
//    4-bit group record of s1 and o' (write_dq_record).
#include "nsn_device.h"
#include "nsn_launch.h"

namespace nsn {

namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kG = 128;
constexpr int kNW = kG / 32;       // waves per workgroup
constexpr float kSqrtD = 11.313708498984761f;
constexpr int kRing = 128;         // queue entries per wave (a ring; 4 KB of the staging tile)

struct alignas(16) QEntry {
  float h[4];
  uint32_t codes;  // candidates five to eight, ascending
  float best;      // best distance among the first four
  uint32_t dst;    // byte of the owner's result row
  float s;         // s2 of the owner's token (1 when it is 0)
};

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef _Float16 h2v __attribute__((ext_vector_type(2)));

// z - s c for c the low (HI = 0) or high (HI = 1) fp16 half of w: one
// v_fma_mix_f32 (c widened exactly, s negated by the source modifier, one
// rounding).  Arithmetic only.
template <int HI>
__device__ __forceinline__ float fma_f16(uint32_t w, float s, float z) {
  float d;
  if constexpr (HI)
    asm("v_fma_mix_f32 %0, %1, -%2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "=v"(d) : "v"(w), "v"(s), "v"(z));
  else
    asm("v_fma_mix_f32 %0, %1, -%2, %3 op_sel:[0,0,0] op_sel_hi:[1,0,0]"
        : "=v"(d) : "v"(w), "v"(s), "v"(z));
  return d;
}

// The shift count 3 in a VGPR that the compiler cannot rematerialize: made
// once per kernel, so the SDWA shifts below share one register instead of a
// fresh constant move each.
__device__ __forceinline__ uint32_t vgpr_three() {
  uint32_t r;
  asm volatile("v_mov_b32 %0, 3" : "=v"(r));
  return r;
}

// 8 x byte i of w: the byte offset in the fp16 codebook of the code held in
// that byte, by one SDWA shift (three = vgpr_three()).  The compiler forms
// bytes 1-3 that way with a constant register of its own but byte 0 with a
// shift and a mask; all four go through the one shared register here.
__device__ __forceinline__ uint32_t code_byte_off(uint32_t w, int i, uint32_t three) {
  uint32_t r;
  if (i == 0)
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0"
        : "=v"(r) : "v"(three), "v"(w));
  else if (i == 1)
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1"
        : "=v"(r) : "v"(three), "v"(w));
  else if (i == 2)
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2"
        : "=v"(r) : "v"(three), "v"(w));
  else
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
        : "=v"(r) : "v"(three), "v"(w));
  return r;
}

// ||z - s c||^2 for the codeword at byte offset `off` (8 x its code) of the
// fp16 codebook in LDS.  With z = s h this is s^2 ||h - c||^2: the same order
// over codewords as the distance to h, without forming h.
__device__ __forceinline__ float sqdist_cb(const float (&z)[4], const uint32_t* cbh, uint32_t off,
                                           float s) {
  const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(cbh) + off);
  const float d0 = fma_f16<0>(w.x, s, z[0]), d1 = fma_f16<1>(w.x, s, z[1]);
  const float d2 = fma_f16<0>(w.y, s, z[2]), d3 = fma_f16<1>(w.y, s, z[3]);
  return fmaf(d3, d3, fmaf(d2, d2, fmaf(d1, d1, d0 * d0)));
}

// the codeword at byte offset `off` (8 x its code) of the fp16 codebook in
// LDS, as fp32 (exact)
__device__ __forceinline__ void codeword(const uint32_t* cbh, uint32_t off, float (&cv)[4]) {
  const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(cbh) + off);
  const h2v a = __builtin_bit_cast(h2v, w.x), b = __builtin_bit_cast(h2v, w.y);
  cv[0] = static_cast<float>(a.x);
  cv[1] = static_cast<float>(a.y);
  cv[2] = static_cast<float>(b.x);
  cv[3] = static_cast<float>(b.y);
}

__device__ __forceinline__ v8h as_v8h(u32x4 v) { return __builtin_bit_cast(v8h, v); }

// Shared memory of the front end (steps 1 and 2).
struct FrontSmem {
  float ascale[kG];
  float csum[kNW][kD];
  __attribute__((aligned(16))) float osh[kD];
  // per-wave staging of the wave's 32 input tokens: 16-byte chunk c of token
  // t at slot 16 t + (c ^ (t % 16)), so both the coalesced writes and the
  // operand-layout reads touch 16 different 4-bank groups per 16 lanes
  __attribute__((aligned(16))) u32x4 xs[kNW][32 * 16];
};

// Steps 1 and 2 for the group (seq, grp).  On return acc[mb][4q + e] holds z
// of channel 32mb + 8q + 4hf + e of the lane's token; fs.osh holds the group's
// rotated shift o'.  Contains block barriers: every thread of the workgroup
// calls it.
__device__ __forceinline__ void nsn_front(const __half* __restrict__ x, int64_t x_seq_stride,
                                          int64_t seq, int64_t grp, FrontSmem& fs,
                                          v16f (&acc)[4], float& s1, float& s2, const Signs& sg) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int t = lane & 31, hf = lane >> 5;
  const int tg = 32 * w + t;                          // token within the group

  // ---- operands: x (fp16, 8 x 16 bytes per lane) and the H16 sign pattern
  // the wave's 32 tokens are 8 KB of contiguous input: eight fully coalesced
  // 1 KB loads, through LDS into the operand layout (lane (t, hf) needs the
  // 16-byte chunks 2 kb + hf of token t)
  u32x4 xv[8];
  {
    const __half* wrow = x + seq * x_seq_stride + (grp * kG + 32 * w) * kD;
    u32x4 ld[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ld[i] = load_nt16(wrow + 8 * (kWave * i + lane));
    if (any_sign(sg)) {
      // randomized rotation: every load of this lane holds channels 8c ..
      // 8c + 7 (c = lane % 16) of some token; negate the selected ones by
      // their fp16 sign bits
      const int c = lane & 15;
      const uint32_t byte = (sign_word(sg, c >> 2) >> (8 * (c & 3))) & 0xffu;
      uint32_t mk[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        mk[k] = (((byte >> (2 * k)) & 1u) << 15) | (((byte >> (2 * k + 1)) & 1u) << 31);
      const u32x4 m4 = u32x4{mk[0], mk[1], mk[2], mk[3]};
#pragma unroll
      for (int i = 0; i < 8; ++i) ld[i] ^= m4;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tt = 4 * i + (lane >> 4), c = lane & 15;
      fs.xs[w][16 * tt + (c ^ (tt & 15))] = ld[i];
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) xv[kb] = fs.xs[w][16 * t + ((2 * kb + hf) ^ (t & 15))];
  }
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
  ss = half_pair_sum(ss);
  const float nrm = sqrtf(ss);
  s1 = nrm * (1.0f / kD);
  const float a_t = nrm > 0.f ? kSqrtD / nrm : 0.f;
  if (hf == 0) fs.ascale[tg] = a_t;
  __syncthreads();

  // ---- channel-major rotation for the group mean: lane holds tokens
  //      {8q + 4hf + e} of this wave for channel 32nb + t
  {
    float av[16];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) av[4 * q + e] = fs.ascale[32 * w + 8 * q + 4 * hf + e];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      v16f c2 = v16f{};
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_v8h(xv[kb]), HBLK(nb, kb), c2, 0, 0, 0);
      float s = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) s = fmaf(av[r], c2[r], s);
      s = half_pair_sum(s);
      if (hf == 0) fs.csum[w][32 * nb + t] = s;
    }
  }
#undef HBLK
  __syncthreads();
  if (tid < kD) {
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < kNW; ++ww) s += fs.csum[ww][tid];
    fs.osh[tid] = s * (1.0f / kG);
  }
  __syncthreads();

  // ---- z = y - o' (in place), s2
  float ss2 = 0.f;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 o = *reinterpret_cast<const float4*>(&fs.osh[32 * mb + 8 * q + 4 * hf]);
      const float ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float z = fmaf(acc[mb][4 * q + e], a_t, -ov[e]);
        acc[mb][4 * q + e] = z;
        ss2 = fmaf(z, z, ss2);
      }
    }
  ss2 = half_pair_sum(ss2);
  s2 = sqrtf(ss2 * (1.0f / kD));
}

// Double quantization of the group's byproducts (flag NSN_DQ), written after
// every token's s1 is in s1g: a record of 8 + 64 + 64 bytes per group --
// fp16 (lo, hi) = min and max of s1, fp16 scale = max |o'| / 7, 0; the o'
// codes (channel c in byte c / 2, low nibble for even c: round(o'/scale)
// in [-7, 7] plus 8, 0 for a zero scale); the s1 codes (token t likewise:
// round((s1 - lo) * 15 / (hi - lo)) in [0, 15], 0 when hi == lo).  Codes
// are taken in fp32 with round-half-even.  Contains block barriers.
// [NSNQuant summary, Methodology §3, Double Quantization: s1 and o at 4
//  bits; grids and second-level scales are this library's reading.]
struct DqSmem {
  float s1g[kG];
  uint16_t par[4];
};
__device__ __forceinline__ void write_dq_record(const float* osh, DqSmem& dq, uint8_t* rec) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  if (w == 0) {
    const float a = dq.s1g[lane], b = dq.s1g[lane + kWave];
    const float mn = wave_min_fast(fminf(a, b)), mx = wave_max_fast(fmaxf(a, b));
    if (lane == 0) {
      dq.par[0] = f2h(mn);
      dq.par[1] = f2h(mx);
    }
  } else if (w == 1) {
    const float m = wave_max_fast(fmaxf(fabsf(osh[lane]), fabsf(osh[lane + kWave])));
    if (lane == 0) {
      dq.par[2] = f2h(m / 7.0f);
      dq.par[3] = 0;
    }
  }
  __syncthreads();
  const float lo = h2f(dq.par[0]), hi = h2f(dq.par[1]), sc = h2f(dq.par[2]);
  if (tid < kD / 2) {
    // o' codes of channels 2 tid, 2 tid + 1
    uint32_t c[2] = {0u, 0u};
    if (sc > 0.f) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float t = rintf(osh[2 * tid + e] / sc);
        c[e] = static_cast<uint32_t>(static_cast<int>(fminf(fmaxf(t, -7.f), 7.f)) + 8);
      }
    }
    rec[8 + tid] = static_cast<uint8_t>(c[0] | (c[1] << 4));
  } else if (tid < kD / 2 + kG / 2) {
    // s1 codes of tokens 2k, 2k + 1
    const int k = tid - kD / 2;
    uint32_t c[2] = {0u, 0u};
    if (hi > lo) {
      const float inv = 15.0f / (hi - lo);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float t = rintf((dq.s1g[2 * k + e] - lo) * inv);
        c[e] = static_cast<uint32_t>(fminf(fmaxf(t, 0.f), 15.f));
      }
    }
    rec[8 + kD / 2 + k] = static_cast<uint8_t>(c[0] | (c[1] << 4));
  } else if (tid == kD / 2 + kG / 2) {
    *reinterpret_cast<uint2*>(rec) = make_uint2(static_cast<uint32_t>(dq.par[0]) | (static_cast<uint32_t>(dq.par[1]) << 16),
                                                static_cast<uint32_t>(dq.par[2]));
  }
}
static_assert(kDqRecU16 * 2 == 8 + kD / 2 + kG / 2, "record size");

template <bool DQ>
__global__ __launch_bounds__(kG * 2, 2) void quantize_mfma_kernel(
    const __half* __restrict__ x, int64_t n_groups, int64_t x_seq_stride,
    const uint8_t* __restrict__ table, uint8_t* __restrict__ codes, int64_t codes_seq_stride,
    uint16_t* __restrict__ meta, int64_t meta_seq_stride, uint16_t* __restrict__ shift,
    int64_t shift_seq_stride, int scale_adjust, Signs sg) {
  // fp16 codebook (the prepared codebook's entries are fp16 values, so this
  // copy is exact and half the LDS traffic of fp32)
  __shared__ __attribute__((aligned(16))) uint32_t cbh[kCodes * 2];
  __shared__ __attribute__((aligned(16))) uint8_t binlut[3 * kFine];   // sentinels around the grid
  __shared__ FrontSmem fs;
  // per-lane result row (16 code bytes) that queued sub-vectors update
  __shared__ __attribute__((aligned(16))) uint32_t res[kNW][kWave][4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int t = lane & 31, hf = lane >> 5;
  const int64_t seq = blockIdx.x / n_groups;
  const int64_t grp = blockIdx.x - seq * n_groups;
  const int tg = 32 * w + t;                          // token within the group
  const int64_t tok = grp * kG + tg;

  {
    const uint32_t* cbg = reinterpret_cast<const uint32_t*>(table + kTabCodebookH);
    for (int i = tid; i < kCodes * 2; i += kG * 2) cbh[i] = cbg[i];
    const uint32_t* bl = reinterpret_cast<const uint32_t*>(table + kTabBinLut);
    uint32_t* bd = reinterpret_cast<uint32_t*>(binlut);
    for (int i = tid; i < 3 * kFine / 4; i += kG * 2)
      bd[i] = (i >= kFine / 4 && i < 2 * kFine / 4) ? bl[i - kFine / 4] : 0x80808080u;
  }

  v16f acc[4];
  float s1, s2;
  nsn_front(x, x_seq_stride, seq, grp, fs, acc, s1, s2, sg);

  // The search runs on z = s2 h directly: distances ||z - s2 c||^2 and bins
  // of z / s2.  A zero z (s2 = 0) is h = 0: scale 1 gives the same answer.
  const float sc = s2 > 0.f ? s2 : 1.0f;
  const float fine_scale = kFineInv / sc;

  // ---- nearest codeword, four sub-vectors (one mb block) per step; the
  //      candidate words of the next block are fetched while the current one
  //      is evaluated.
  const uint64_t* tmain = reinterpret_cast<const uint64_t*>(table + kTabMain);
  auto locate = [&](int mb, int q, bool& off) -> int {
    uint32_t bins[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // fine index + 1024; off-grid and non-finite values land on sentinels
      const uint32_t fi = static_cast<uint32_t>(
          static_cast<int>(fmaf(acc[mb][4 * q + e], fine_scale, 512.0f + kFine)));
      bins[e] = binlut[min(fi, static_cast<uint32_t>(3 * kFine - 1))];
    }
    off = ((bins[0] | bins[1] | bins[2] | bins[3]) & 0x80u) != 0;
    return min(static_cast<int>(((bins[0] * kNB + bins[1]) * kNB + bins[2]) * kNB + bins[3]),
               kCells - 1);
  };
  bool offv[2][4];
  uint64_t wordv[2][4];
#pragma unroll
  for (int q = 0; q < 4; ++q) wordv[0][q] = tmain[locate(0, q, offv[0][q])];

  // Boxes with five to eight candidates: the first four are evaluated in
  // place; the sub-vector, its other four candidates and its best distance
  // so far go to a per-wave ring (in the staging tile, free by now).
  // Whenever 64 entries are waiting the wave works through them, one entry
  // per lane, writing an improved code straight into the owner's result row
  // (every code is stored as its own byte as soon as it is known, so an
  // entry may be resolved at any later point).
  uint8_t* resb = reinterpret_cast<uint8_t*>(&res[w][0][0]);   // lane l: bytes 16 l .. 16 l + 15
  QEntry* ring = reinterpret_cast<QEntry*>(&fs.xs[w][0]);
  const uint32_t three = vgpr_three();
  int qhead = 0, qtail = 0;   // wave-uniform ring positions
  auto flush = [&](int n) {
    wave_lds_sync();
    if (lane < n) {
      // candidates five to eight are ascending and above the first four, so
      // a strict '<' against the best so far keeps the lowest code on ties
      const QEntry e = ring[(qhead + lane) & (kRing - 1)];
      float bd = e.best;
      uint32_t bc = 0xffffffffu;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t code = (e.codes >> (8 * i)) & 0xffu;
        const float d = sqdist_cb(e.h, cbh, code_byte_off(e.codes, i, three), e.s);
        bc = d < bd ? code : bc;
        bd = d < bd ? d : bd;
      }
      if (bc != 0xffffffffu) resb[e.dst] = static_cast<uint8_t>(bc);
    }
    wave_lds_sync();
    qhead += n;
  };
  const uint64_t below = (uint64_t(1) << lane) - 1;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int cur = mb & 1, nxt = cur ^ 1;
    if (mb < 3) {
#pragma unroll
      for (int q = 0; q < 4; ++q) wordv[nxt][q] = tmain[locate(mb + 1, q, offv[nxt][q])];
    }
    uint32_t scanmask = 0;   // bit q: sub-vector (mb, q) of this lane needs the full scan
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float hv[4] = {acc[mb][4 * q], acc[mb][4 * q + 1], acc[mb][4 * q + 2], acc[mb][4 * q + 3]};
      const uint64_t wv = wordv[cur][q];
      const uint32_t lo = static_cast<uint32_t>(wv), hi = static_cast<uint32_t>(wv >> 32);
      const bool more4 = cand_more_than_4_lo(lo);
      const bool scan = offv[cur][q] || cand_more_than_8_hi(hi);
      // the four lowest candidates in ascending code order (byte-reversed
      // when there are more than four)
      const uint32_t asc = more4 ? __builtin_amdgcn_perm(0u, lo, 0x00010203u) : lo;
      // distance >= 0 with the candidate's slot in its two low bits: the
      // integer minimum is the smallest distance (to within 3 ulp) and, among
      // equal keys, the lowest slot, i.e. the lowest code
      uint32_t best = 0xffffffffu;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float d = sqdist_cb(hv, cbh, code_byte_off(asc, i, three), sc);
        best = min(best, (__float_as_uint(d) & ~3u) | static_cast<uint32_t>(i));
      }
      const uint32_t bc = (asc >> (8 * (best & 3u))) & 0xffu;
      const uint32_t dst = static_cast<uint32_t>(lane * 16 + 4 * mb + q);
      resb[dst] = static_cast<uint8_t>(bc);
      scanmask |= scan ? (1u << q) : 0u;
      const bool enq = more4 && !scan;
      const uint64_t bq = __ballot(enq);
      if (enq) {
        QEntry e;
        e.h[0] = hv[0];
        e.h[1] = hv[1];
        e.h[2] = hv[2];
        e.h[3] = hv[3];
        e.codes = hi;
        e.best = __uint_as_float(best & ~3u);
        e.dst = dst;
        e.s = sc;
        ring[(qtail + __popcll(bq & below)) & (kRing - 1)] = e;
      }
      qtail += __popcll(bq);
      if (qtail - qhead >= kWave) flush(kWave);
    }
    // sub-vectors whose box has more than eight candidates or that lie off
    // the grid: the whole wave scans all codes for one of them at a time
    if (__ballot(scanmask != 0)) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint64_t pend = __ballot((scanmask >> q) & 1u);
        while (pend) {
          const int src = __builtin_ctzll(pend);
          pend &= pend - 1;
          float hv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            hv[e] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc[mb][4 * q + e]), src));
          const float ss = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc), src));
          float bd = __builtin_huge_valf();
          uint32_t bc = 0;
#pragma unroll
          for (int r = 0; r < kCodes / kWave; ++r) {
            const uint32_t code = static_cast<uint32_t>(lane + kWave * r);
            const float d = sqdist_cb(hv, cbh, code << 3, ss);
            bc = d < bd ? code : bc;
            bd = d < bd ? d : bd;
          }
          const float dmin = wave_min_fast(bd);
          const float cmin = wave_min_fast(bd == dmin ? static_cast<float>(bc) : 1e9f);
          if (lane == src) resb[lane * 16 + 4 * mb + q] = static_cast<uint8_t>(static_cast<uint32_t>(cmin) & 0xffu);
        }
      }
    }
  }
  if (qtail > qhead) flush(qtail - qhead);
  uint32_t codes4[4];
  {
    wave_lds_sync();
    const u32x4 r = *reinterpret_cast<const u32x4*>(&res[w][lane][0]);
    codes4[0] = r.x;
    codes4[1] = r.y;
    codes4[2] = r.z;
    codes4[3] = r.w;
  }

  // ---- scale adjustment, codes, metadata
  float dot = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int mb = k >> 2, q = k & 3;
    float cv[4];
    codeword(cbh, code_byte_off(codes4[mb], q, three), cv);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dot = fmaf(acc[mb][4 * q + e], cv[e], dot);
    }
  }
  // <h, h_hat> = <z, h_hat> / s2 and ||h||^2 = d exactly (Normalize #2)
  dot = half_pair_sum(dot);
  const float alpha = (scale_adjust && dot > 0.f) ? (kD * s2) / dot : 1.0f;
  const uint32_t own[4] = {codes4[0], codes4[1], codes4[2], codes4[3]};

  // Lane half 0 holds the even sub-vectors, half 1 the odd ones.  After the
  // swap, half 0 has (own even, partner odd) codes of sub-vectors 0..15 and
  // half 1 (partner even, own odd) of 16..31: interleave bytes and store.
  uint32_t lo01[2] = {own[0], own[1]}, hi23[2] = {own[2], own[3]};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(lo01[i], hi23[i], false, false);
    lo01[i] = r[0];
    hi23[i] = r[1];
  }
  // half 0: even = lo01 (own), odd = hi23 (partner's codes 0..15)
  // half 1: even = lo01 (partner's 16..31), odd = hi23 (own)
  uint32_t pk[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t ev = lo01[d >> 1], od = hi23[d >> 1];
    pk[d] = __builtin_amdgcn_perm(od, ev, (d & 1) ? 0x07030602u : 0x05010400u);
  }
  *reinterpret_cast<u32x4*>(codes + seq * codes_seq_stride + tok * 32 + 16 * hf) =
      u32x4{pk[0], pk[1], pk[2], pk[3]};
  if constexpr (DQ) {
    __shared__ DqSmem dqs;
    if (hf == 0) {
      dqs.s1g[tg] = s1;
      meta[seq * meta_seq_stride + tok] = f2h(s2 * alpha);
    }
    __syncthreads();
    write_dq_record(fs.osh, dqs, reinterpret_cast<uint8_t*>(shift + seq * shift_seq_stride + grp * kDqRecU16));
  } else {
    if (hf == 0) {
      const uint32_t mv = static_cast<uint32_t>(f2h(s1)) |
                          (static_cast<uint32_t>(f2h(s2 * alpha)) << 16);
      *reinterpret_cast<uint32_t*>(meta + seq * meta_seq_stride + 2 * tok) = mv;
    }
    if (tid < kD) shift[seq * shift_seq_stride + grp * kD + tid] = f2h(fs.osh[tid]);
  }
}


__device__ __forceinline__ uint32_t pack_h2(_Float16 lo, _Float16 hi) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
}

// fp16 pair (RNE) of (z0 s, z1 s), each rounded once from the exact product.
// Arithmetic only.
__device__ __forceinline__ uint32_t split_hi(float z0, float z1, float s) {
  uint32_t h;
  asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,0,0]" : "=v"(h) : "v"(z0), "v"(s));
  asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel_hi:[0,0,0]" : "+v"(h) : "v"(z1), "v"(s));
  return h;
}
// fp16 pair (RNE) of (z0 s - hi0, z1 s - hi1) for hi = split_hi(z0, z1, s),
// each an fma with one rounding.  Arithmetic only.
__device__ __forceinline__ uint32_t split_lo(float z0, float z1, float s, uint32_t hi) {
  uint32_t l;
  asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel:[0,0,0] op_sel_hi:[0,0,1]"
      : "=v"(l) : "v"(z0), "v"(s), "v"(hi));
  asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
      : "+v"(l) : "v"(z1), "v"(s), "v"(hi));
  return l;
}
// acc + z c for c the low (HI = 0) or high (HI = 1) fp16 half of w (c
// widened exactly).  Arithmetic only.
template <int HI>
__device__ __forceinline__ float fma_acc_f16(float z, uint32_t w, float acc) {
  float d;
  if constexpr (HI)
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(d) : "v"(z), "v"(w), "v"(acc));
  else
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,0,0] op_sel_hi:[0,1,0]" : "=v"(d) : "v"(z), "v"(w), "v"(acc));
  return d;
}

template <bool DQ>
__global__ __launch_bounds__(kG * 2, 2) void quantize_mfma8_kernel(
    const __half* __restrict__ x, int64_t n_groups, int64_t x_seq_stride,
    const uint8_t* __restrict__ table, uint8_t* __restrict__ codes, int64_t codes_seq_stride,
    uint16_t* __restrict__ meta, int64_t meta_seq_stride, uint16_t* __restrict__ shift,
    int64_t shift_seq_stride, int scale_adjust, Signs sg) {
  constexpr int kTiles = kCodes / 32;
  __shared__ __attribute__((aligned(16))) u32x4 cb8[kCodes];        // fp16 codebook [256][8]
  // norm operand of tile T for lane l: fp16 (||c||^2 hi, ||c||^2 lo, 1, 0,
  // 0, ...) of code 32T + l for l < 32, zero for lanes 32..63
  __shared__ __attribute__((aligned(16))) u32x4 a2s[kTiles][kWave];
  __shared__ FrontSmem fs;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int t = lane & 31, hf = lane >> 5;
  const int64_t seq = blockIdx.x / n_groups;
  const int64_t grp = blockIdx.x - seq * n_groups;
  const int64_t tok = grp * kG + 32 * (tid >> 6) + t;

  // Codebook operand of tile T: code 32T + t in every lane (K 0..7 in lanes
  // 0..31 and K 8..15 in lanes 32..63: the same c meets the hi and the lo
  // part of -2h).
  const u32x4* cbg = reinterpret_cast<const u32x4*>(table + kTabCodebookH);
  {
    const u32x4 c = cbg[tid];                          // 256 threads, one code each
    cb8[tid] = c;
    const v8h ch = as_v8h(c);
    float n2 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) n2 = fmaf(static_cast<float>(ch[e]), static_cast<float>(ch[e]), n2);
    const _Float16 nh = static_cast<_Float16>(n2);
    const _Float16 nl = static_cast<_Float16>(n2 - static_cast<float>(nh));   // n2 - nh is exact
    a2s[tid >> 5][tid & 31] = u32x4{pack_h2(nh, nl), 0x3C00u, 0u, 0u};
    a2s[tid >> 5][32 + (tid & 31)] = u32x4{0u, 0u, 0u, 0u};
  }

  v16f acc[4];
  float s1, s2;
  nsn_front(x, x_seq_stride, seq, grp, fs, acc, s1, s2, sg);   // its barriers publish cb8, a2s
  // The search runs on g = -2h = z * (-2 / s2) (the factor -2 is exact).  A zero
  // z (s2 = 0) is h = 0: scale 1 gives the same answer.
  const float ginv = -2.0f / (s2 > 0.f ? s2 : 1.0f);

  uint32_t cw[4] = {0u, 0u, 0u, 0u};   // code of sub-vector j in byte j % 4 of word j / 4
  float dot = 0.f;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // sub-vector j = 4mb + q of the lane's token: this lane holds z of
      // elements 4hf .. 4hf+3, the other half the rest
      float zf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t v = __float_as_uint(acc[mb][4 * q + e]);
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        zf[e] = __uint_as_float(r[0]);
        zf[4 + e] = __uint_as_float(r[1]);
      }
      // B1: fp16 hi part of g (lanes 0..31, K 0..7) or lo part g - hi
      // (lanes 32..63, K 8..15), each rounded once from the exact z * ginv
      uint32_t b1[4];
      float gg = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t hi = split_hi(zf[2 * i], zf[2 * i + 1], ginv);
        const uint32_t lo = split_lo(zf[2 * i], zf[2 * i + 1], ginv, hi);
        b1[i] = hf ? lo : hi;
        gg = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, hi), __builtin_bit_cast(h2v, hi), gg,
                                    false);
      }
      const v8h B1 = as_v8h(u32x4{b1[0], b1[1], b1[2], b1[3]});
      // B2: (1, 1, H, 0, ...) in lanes 0..31, H an upper bound of
      // ||h_j||^2 = ||g||^2 / 4: ||hi||^2 >= (1 - 2^-10) ||g||^2, the 2^-8
      // increase covers that and the fp16 rounding of H.  Then
      // D = ||h - c||^2 + (H - ||h_j||^2) >= 0 and its float bits order like
      // its value.
      const _Float16 Hh = static_cast<_Float16>(gg * (0.25f * (1.0f + 0x1p-8f)));
      const v8h B2 = as_v8h(u32x4{hf ? 0u : 0x3C003C00u, hf ? 0u : pack_h2(Hh, 0), 0u, 0u});

      // lane (t, hf) holds D for codes 32T + 8(r/4) + 4hf + r%4, r = 0..15;
      // the products of tile T + 1 are issued before the minimum of tile T.
      // (The compiler keeps the loop-invariant operands in registers; forcing
      // per-tile LDS reads for a third wave per SIMD, or fencing the schedule,
      // measured slower.)
      auto tile = [&](int T) {
        const v16f n = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_v8h(a2s[T][lane]), B2, v16f{},
                                                              0, 0, 0);
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(as_v8h(cb8[32 * T + t]), B1, n, 0, 0, 0);
      };
      int best = 0x7fffffff, bt = 0;
      v16f dcur = tile(0);
#pragma unroll
      for (int T = 0; T < kTiles; ++T) {
        v16f dnext;
        if (T + 1 < kTiles) dnext = tile(T + 1);
        int m = 0x7fffffff;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          m = min(m, static_cast<int>((__float_as_uint(dcur[r]) & ~15u) | static_cast<uint32_t>(r)));
        bt = m < best ? T : bt;
        best = min(best, m);
        if (T + 1 < kTiles) dcur = dnext;
      }
      const uint32_t p = static_cast<uint32_t>(best) & 15u;
      const uint32_t code = (static_cast<uint32_t>(bt) << 5) | ((p >> 2) << 3) |
                            (static_cast<uint32_t>(hf) << 2) | (p & 3u);
      // the two halves hold disjoint code sets of the same token
      const auto rk = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(best),
                                                       static_cast<uint32_t>(best), false, false);
      const auto rc = __builtin_amdgcn_permlane32_swap(code, code, false, false);
      const int k0 = static_cast<int>(rk[0]), k1 = static_cast<int>(rk[1]);
      const uint32_t c0 = rc[0], c1 = rc[1];
      const uint32_t win = (k1 < k0 || (k1 == k0 && c1 < c0)) ? c1 : c0;
      cw[mb] |= win << (8 * q);
      // <z_j, c> over all eight elements, for the scale adjustment (both
      // halves form the same sum in the same order)
      const u32x4 cv = cb8[win];
      dot = fma_acc_f16<0>(zf[0], cv.x, dot);
      dot = fma_acc_f16<1>(zf[1], cv.x, dot);
      dot = fma_acc_f16<0>(zf[2], cv.y, dot);
      dot = fma_acc_f16<1>(zf[3], cv.y, dot);
      dot = fma_acc_f16<0>(zf[4], cv.z, dot);
      dot = fma_acc_f16<1>(zf[5], cv.z, dot);
      dot = fma_acc_f16<0>(zf[6], cv.w, dot);
      dot = fma_acc_f16<1>(zf[7], cv.w, dot);
    }
  }

  // <h, h_hat> = <z, h_hat> / s2 and ||h||^2 = d exactly (Normalize #2)
  const float alpha = (scale_adjust && dot > 0.f) ? (kD * s2) / dot : 1.0f;
  if (hf == 0)
    *reinterpret_cast<u32x4*>(codes + seq * codes_seq_stride + tok * 16) =
        u32x4{cw[0], cw[1], cw[2], cw[3]};
  if constexpr (DQ) {
    __shared__ DqSmem dqs;
    if (hf == 0) {
      dqs.s1g[tok - grp * kG] = s1;
      meta[seq * meta_seq_stride + tok] = f2h(s2 * alpha);
    }
    __syncthreads();
    write_dq_record(fs.osh, dqs, reinterpret_cast<uint8_t*>(shift + seq * shift_seq_stride + grp * kDqRecU16));
  } else {
    if (hf == 0) {
      const uint32_t mv = static_cast<uint32_t>(f2h(s1)) |
                          (static_cast<uint32_t>(f2h(s2 * alpha)) << 16);
      *reinterpret_cast<uint32_t*>(meta + seq * meta_seq_stride + 2 * tok) = mv;
    }
    if (tid < kD) shift[seq * shift_seq_stride + grp * kD + tid] = f2h(fs.osh[tid]);
  }
}

}  // namespace

bool quantize_mfma_supported(int in_f32, int sub_dim, int group_size) {
  return !in_f32 && (sub_dim == 4 || sub_dim == 8) && group_size == kG;
}

hipError_t launch_quantize_mfma(const QuantArgs& a, hipStream_t s) {
  const int64_t n_groups = a.n_tok / kG;
  const int64_t blocks = a.n_seq * n_groups;
  auto kernel = a.sub_dim == 8 ? (a.dq ? quantize_mfma8_kernel<true> : quantize_mfma8_kernel<false>)
                                : (a.dq ? quantize_mfma_kernel<true> : quantize_mfma_kernel<false>);
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(blocks)), dim3(kG * 2), 0, s,
                     static_cast<const __half*>(a.x), n_groups, a.x_seq_stride,
                     static_cast<const uint8_t*>(a.table), a.codes, a.codes_seq_stride, a.meta,
                     a.meta_seq_stride, a.shift, a.shift_seq_stride, a.scale_adjust, a.rht);
  return hipGetLastError();
}

}  // namespace nsn
