// Decode attention over an NSN-quantized KV cache plus an fp16 residual
// window, for gfx950.
// [NSNQuant summary (gist.science), Methodology §4: KIVI-style split of the
//  cache into a quantized part and a full-precision residual; the attention
//  score takes the NSN byproducts s1, s2, o directly.]
//
// Everything on quantized tokens happens in the rotated domain: with
// q' = H q / sqrt(d) (computed once per workgroup),
//   <q, x_hat_t> = s1_t (s2'_t <q', c(codes_t)> + <q', o'_g>),
// so a key is never dequantized.  <q', c(codes_t)> is a sum over the token's
// sub-vectors of a per-workgroup lookup table
//   T[j][code] = ( <q'_h[m j : m j + m], C[code]> )_{h < 4}
// (one 16-byte LDS read gives all four heads).  Values are accumulated in the
// rotated domain and rotated back once per query head in the combine kernel.
//
// attn_split_kernel: one workgroup (16 waves) per (token chunk, kv head,
//   block of up to 4 query heads, batch).  After the shared set-up (rotated
//   queries, per-group <q', o'_g>, lookup table) every wave runs its own
//   online softmax over 64-token tiles with no workgroup barrier:
//     score phase  lane = token: table lookups, scale, wave max, exp;
//                  weights w = p s1 s2' go to a per-wave LDS buffer (fp16);
//     value phase  lane = (16-channel unit, token slot): tokens are taken in
//                  pairs so one v_dot2_f32_f16 does w_a c_a + w_b c_b into an
//                  fp32 accumulator (codewords are exact fp16 values);
//     shift term   p s1 o'_g, from the wave-summed p s1 of the tile.
//   The 16 wave partials are merged through LDS at the end and one
//   (acc[128], max, sum) partial per head is written.
// attn_combine_kernel: one workgroup per (kv head block, batch): the
//   residual window's exact fp16 attention, a log-sum-exp merge with the
//   chunk partials, one inverse rotation, normalization.
#include "nsn_device.h"
#include "nsn_launch.h"

namespace nsn {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kHB = 4;              // query heads per workgroup
constexpr int kMaxChunk = 8192;     // quantized tokens per workgroup, at most
constexpr int kMinChunk = 1024;
constexpr int kPartStride = 132;    // acc[128], m, l, pad
constexpr float kInvSqrtD = 0.08838834764831845f;

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

struct SplitParams {
  const uint16_t* q;
  const uint8_t* kc;
  const uint8_t* vc;
  const uint16_t* km;
  const uint16_t* vm;
  const uint16_t* ks;
  const uint16_t* vs;
  const uint8_t* table;
  float* work;
  int Hq, Hkv, grp, hblocks, n_quant, n_split, chunk;
  int64_t cap;
  float scale;
};

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a), __builtin_bit_cast(h2_t, b), c, false);
}
// (lo half of a, lo half of b) and (hi half of a, hi half of b)
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Global data one wave needs for one 64-token tile, loaded one tile ahead.
struct TileData {
  u32x4 kc[2][2];   // score phase: this lane's token codes, blocks 0 and 1
  uint32_t km, vm;  // metadata of token t0 + lane
  uint32_t vc[8];   // value phase: unit u of tokens slot + 8 i
  u32x4 osh;        // 8 fp16 of the group's V shift for the shift term
};

template <int M>
__device__ __forceinline__ void load_tile(TileData& d, int t0, int c1, int lane, int u, int slot,
                                          int sh_c, const uint8_t* kcrow, const uint8_t* vcrow,
                                          const uint32_t* kmrow, const uint32_t* vmrow,
                                          const uint16_t* vs_g) {
  constexpr int CODE_BYTES = kD / M;
  const int t32 = lane & 31;
#pragma unroll
  for (int bk = 0; bk < 2; ++bk) {
    const int tt = t0 + 32 * bk + t32;
#pragma unroll
    for (int i = 0; i < 2; ++i) d.kc[bk][i] = u32x4{0u, 0u, 0u, 0u};
    if (tt < c1) {
      const uint8_t* src = kcrow + static_cast<int64_t>(tt) * CODE_BYTES;
#pragma unroll
      for (int i = 0; i < CODE_BYTES / 16; ++i) d.kc[bk][i] = load_nt16(src + 16 * i);
    }
  }
  const int t = t0 + lane;
  d.km = t < c1 ? __builtin_nontemporal_load(kmrow + t) : 0u;
  d.vm = t < c1 ? __builtin_nontemporal_load(vmrow + t) : 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int tv = t0 + slot + 8 * i;
    uint32_t v = 0;
    if (tv < c1) {
      if constexpr (M == 4)
        v = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(vcrow + static_cast<int64_t>(tv) * CODE_BYTES) + u);
      else
        v = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(vcrow + static_cast<int64_t>(tv) * CODE_BYTES) + u);
    }
    d.vc[i] = v;
  }
  d.osh = load_nt16(vs_g + sh_c);
}

// One 16-channel MFMA step of the scores, for compile-time step ST (keeps
// every register index constant), then the next step.
template <int M, int ST>
__device__ __forceinline__ void score_steps(v16f& sc, const u32x4 (&qa)[8], const uint32_t (&w8)[8],
                                            int hf, const uint32_t* cbh) {
  if constexpr (ST < 8) {
    u32x4 bv;
    if constexpr (M == 4) {
      // sub-vectors 4 ST + 2 hf and + 1: bytes 2 hf, 2 hf + 1 of code word ST
      const uint32_t wd = w8[ST];
      const uint32_t ca = (wd >> (16 * hf)) & 0xffu;
      const uint32_t cb2 = (wd >> (16 * hf + 8)) & 0xffu;
      const uint2 xa = *reinterpret_cast<const uint2*>(&cbh[ca * 2]);
      const uint2 xb = *reinterpret_cast<const uint2*>(&cbh[cb2 * 2]);
      bv = u32x4{xa.x, xa.y, xb.x, xb.y};
    } else {
      // sub-vector 2 ST + hf: byte (2 ST + hf) & 3 of code word (2 ST + hf) / 4
      const uint32_t wd = w8[ST >> 1];
      const uint32_t ca = (wd >> (8 * (((2 * ST) & 3) + hf))) & 0xffu;
      const uint4 xa = *reinterpret_cast<const uint4*>(&cbh[ca * 4]);
      bv = u32x4{xa.x, xa.y, xa.z, xa.w};
    }
    sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, qa[ST]),
                                                 __builtin_bit_cast(v8h, bv), sc, 0, 0, 0);
    score_steps<M, ST + 1>(sc, qa, w8, hf, cbh);
  }
}

template <int M, int G>
__global__ __launch_bounds__(kThreads, 2) void attn_split_kernel(SplitParams p) {
  constexpr int NSUB = kD / M;
  constexpr int CODE_BYTES = NSUB;   // bytes of codes per token
  constexpr int UPOS = 16 / M;       // sub-vector positions per 16-channel unit
  constexpr int CW = M / 2;          // dwords per fp16 codeword
  constexpr int kMaxGroups = kMaxChunk / G;

  __shared__ __attribute__((aligned(16))) uint32_t cbh[kCodes * CW];   // fp16 codebook
  __shared__ float qr[kHB][kD];
  __shared__ float qo[kMaxGroups][kHB];
  __shared__ uint2 wbuf[kWaves][64];      // per-wave fp16 weights of the tile's tokens
  __shared__ float wm[kWaves][kHB];
  __shared__ float wl[kWaves][kHB];
  __shared__ float wacc[kWaves][kHB][kD];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int t32 = lane & 31, hf = lane >> 5;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y / p.hblocks;
  const int hb = blockIdx.y - kvh * p.hblocks;
  const int b = blockIdx.z;
  const int h0 = kvh * p.grp + hb * kHB;
  const int nh = min(kHB, p.grp - hb * kHB);
  const int c0 = split * p.chunk;
  const int c1 = min(p.n_quant, c0 + p.chunk);
  const int64_t row = static_cast<int64_t>(b) * p.Hkv + kvh;  // (b, kvh) cache row

  // ---- set-up: fp16 codebook, rotated queries, per-group <q', o'_g>
  const uint32_t* cbg = reinterpret_cast<const uint32_t*>(p.table + kTabCodebookH);
  for (int i = tid; i < kCodes * CW; i += kThreads) cbh[i] = cbg[i];
  for (int i = tid; i < kHB * kD; i += kThreads) {
    const int h = i / kD, c = i % kD;
    qr[h][c] = h < nh ? h2f(p.q[(static_cast<int64_t>(b) * p.Hq + h0 + h) * kD + c]) : 0.f;
  }
  __syncthreads();
#pragma unroll 1
  for (int st = 1; st < kD; st <<= 1) {
    for (int i = tid; i < kHB * kD / 2; i += kThreads) {
      const int h = i / (kD / 2), pr = i % (kD / 2);
      const int k = ((pr / st) * 2 * st) + (pr % st);
      const float a = qr[h][k], bb = qr[h][k + st];
      qr[h][k] = a + bb;
      qr[h][k + st] = a - bb;
    }
    __syncthreads();
  }
  for (int i = tid; i < kHB * kD; i += kThreads) qr[i / kD][i % kD] *= kInvSqrtD;
  __syncthreads();

  const int ng = (c1 - c0) / G;
  const uint16_t* ksrow = p.ks + row * (p.cap / G) * kD;
  for (int pair = wave; pair < ng * kHB; pair += kWaves) {
    const int g = pair / kHB, h = pair % kHB;
    const uint16_t* o = ksrow + static_cast<int64_t>(c0 / G + g) * kD;
    float s = qr[h][lane] * h2f(o[lane]) + qr[h][lane + 64] * h2f(o[lane + 64]);
    s = wave_sum(s);
    if (lane == 0) qo[g][h] = s;
  }
  // MFMA A operand, one per 16-channel step: rows 0..3 = fp16(q'_h),
  // rows 8..11 = fp16(q'_h - fp16(q'_h)) (so the pair carries ~22 bits), other
  // rows zero; lane (row t32, channels 16 s + 8 hf .. + 7)
  u32x4 qa[8];
  {
    const bool is_hi = t32 < kHB, is_lo = t32 >= 8 && t32 < 8 + kHB;
    const int hq = is_hi ? t32 : (is_lo ? t32 - 8 : 0);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      uint32_t wv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t pk = 0;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float v = qr[hq][16 * st + 8 * hf + 2 * i + e];
          const uint16_t hi = f2h(v);
          const uint16_t lo = f2h(v - h2f(hi));
          const uint16_t val = is_hi ? hi : (is_lo ? lo : 0);
          pk |= static_cast<uint32_t>(val) << (16 * e);
        }
        wv[i] = pk;
      }
      qa[st] = u32x4{wv[0], wv[1], wv[2], wv[3]};
    }
  }
  __syncthreads();

  // ---- per-wave online softmax over 64-token tiles
  const int u = lane & 7;        // 16-channel unit (value phase)
  const int slot = lane >> 3;    // token slot (value phase)
  const int sh_h = slot >> 1;                 // shift term: this lane's head
  const int sh_c = 16 * u + 8 * (slot & 1);   // and its 8 channels
  float m_run[kHB], l_lane[kHB];
  float acc[kHB][16];
  float sh[8];
#pragma unroll
  for (int h = 0; h < kHB; ++h) {
    m_run[h] = -__builtin_huge_valf();
    l_lane[h] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[h][i] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) sh[i] = 0.f;

  const uint8_t* kcrow = p.kc + row * p.cap * CODE_BYTES;
  const uint8_t* vcrow = p.vc + row * p.cap * CODE_BYTES;
  const uint32_t* kmrow = reinterpret_cast<const uint32_t*>(p.km + row * p.cap * 2);
  const uint32_t* vmrow = reinterpret_cast<const uint32_t*>(p.vm + row * p.cap * 2);
  const uint16_t* vsrow = p.vs + row * (p.cap / G) * kD;

  TileData cur;
  if (c0 + 64 * wave < c1)
    load_tile<M>(cur, c0 + 64 * wave, c1, lane, u, slot, sh_c, kcrow, vcrow, kmrow, vmrow,
                 vsrow + static_cast<int64_t>((c0 + 64 * wave) / G) * kD);
  for (int t0 = c0 + 64 * wave; t0 < c1; t0 += 64 * kWaves) {
    TileData nxt;
    const int tn = t0 + 64 * kWaves;
    if (tn < c1)
      load_tile<M>(nxt, tn, c1, lane, u, slot, sh_c, kcrow, vcrow, kmrow, vmrow,
                   vsrow + static_cast<int64_t>(tn / G) * kD);
    // -- scores on MFMA: block bk covers tokens t0 + 32 bk + t32
    float sblk[2][kHB];
#pragma unroll
    for (int bk = 0; bk < 2; ++bk) {
      uint32_t w8[8];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        w8[4 * i] = cur.kc[bk][i].x;
        w8[4 * i + 1] = cur.kc[bk][i].y;
        w8[4 * i + 2] = cur.kc[bk][i].z;
        w8[4 * i + 3] = cur.kc[bk][i].w;
      }
      v16f sc = v16f{};
      score_steps<M, 0>(sc, qa, w8, hf, cbh);
#pragma unroll
      for (int h = 0; h < kHB; ++h) sblk[bk][h] = sc[h] + sc[4 + h];   // hi + lo rows (lanes < 32)
    }
    // lanes 32..63 take block 1's tokens: lane l now holds token t0 + l
    float dotq[kHB];
#pragma unroll
    for (int h = 0; h < kHB; ++h) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(sblk[0][h]),
                                                      __float_as_uint(sblk[1][h]), false, false);
      dotq[h] = __uint_as_float(r[0]);
    }
    const int t = t0 + lane;
    const bool valid = t < c1;
    const uint32_t kmv = cur.km, vmv = cur.vm;
    const int g = (t0 - c0) / G;  // one group per tile (64 divides G)
    const float s1k = h2f(kmv & 0xffffu), s2k = h2f(kmv >> 16);
    const float s1v = h2f(vmv & 0xffffu), s2v = h2f(vmv >> 16);
    const float ks1 = p.scale * s1k;
    float s[kHB];
#pragma unroll
    for (int h = 0; h < kHB; ++h) s[h] = ks1 * fmaf(s2k, dotq[h], qo[g][h]);
    float pw[kHB], gs[kHB];
#pragma unroll
    for (int h = 0; h < kHB; ++h) {
      if (!valid) s[h] = -__builtin_huge_valf();
      const float mnew = fmaxf(m_run[h], wave_max_fast(s[h]));  // wave-uniform
      if (mnew > m_run[h]) {
        const float f = __expf(m_run[h] - mnew);
        m_run[h] = mnew;
        l_lane[h] *= f;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[h][i] *= f;
        if (sh_h == h) {
#pragma unroll
          for (int i = 0; i < 8; ++i) sh[i] *= f;
        }
      }
      pw[h] = valid ? __expf(s[h] - m_run[h]) : 0.f;
      l_lane[h] += pw[h];
      gs[h] = wave_sum_fast(pw[h] * s1v);
    }
    const float sv = s1v * s2v;
    wbuf[wave][lane] = make_uint2(
        static_cast<uint32_t>(f2h(pw[0] * sv)) | (static_cast<uint32_t>(f2h(pw[1] * sv)) << 16),
        static_cast<uint32_t>(f2h(pw[2] * sv)) | (static_cast<uint32_t>(f2h(pw[3] * sv)) << 16));
    // shift term p s1 o'_g: this lane owns head sh_h, channels sh_c .. sh_c + 7
    {
      const u32x4 o = cur.osh;
      const float gsh = sh_h == 0 ? gs[0] : sh_h == 1 ? gs[1] : sh_h == 2 ? gs[2] : gs[3];
      const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sh[2 * i] = fmaf(gsh, h2f(ow[i] & 0xffffu), sh[2 * i]);
        sh[2 * i + 1] = fmaf(gsh, h2f(ow[i] >> 16), sh[2 * i + 1]);
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // -- value phase: lane = (unit u, slot); token pairs (a, a + 8)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int ia = slot + 16 * k, ib = ia + 8;
      const uint32_t va = cur.vc[2 * k], vb = cur.vc[2 * k + 1];
      const uint2 wa = wbuf[wave][ia], wb = wbuf[wave][ib];
      const uint32_t wp[kHB] = {pair_lo(wa.x, wb.x), pair_hi(wa.x, wb.x), pair_lo(wa.y, wb.y),
                                pair_hi(wa.y, wb.y)};
#pragma unroll
      for (int pos = 0; pos < UPOS; ++pos) {
        const uint32_t ca = (va >> (8 * pos)) & 0xffu, cb = (vb >> (8 * pos)) & 0xffu;
        uint32_t xa[CW], xb[CW];
#pragma unroll
        for (int i = 0; i < CW; ++i) {
          xa[i] = cbh[ca * CW + i];
          xb[i] = cbh[cb * CW + i];
        }
#pragma unroll
        for (int i = 0; i < CW; ++i) {
          const uint32_t plo = pair_lo(xa[i], xb[i]), phi = pair_hi(xa[i], xb[i]);
#pragma unroll
          for (int h = 0; h < kHB; ++h) {
            acc[h][pos * M + 2 * i] = dot2(wp[h], plo, acc[h][pos * M + 2 * i]);
            acc[h][pos * M + 2 * i + 1] = dot2(wp[h], phi, acc[h][pos * M + 2 * i + 1]);
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    cur = nxt;
  }

  // ---- merge: slots inside each wave, then the waves
#pragma unroll
  for (int h = 0; h < kHB; ++h) {
    l_lane[h] = wave_sum(l_lane[h]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = acc[h][i];
      v += __shfl_xor(v, 8, kWave);
      v += __shfl_xor(v, 16, kWave);
      v += __shfl_xor(v, 32, kWave);
      acc[h][i] = v;
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int h = 0; h < kHB; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) wacc[wave][h][16 * u + i] = acc[h][i];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < kHB; ++h) {
      wm[wave][h] = m_run[h];
      wl[wave][h] = l_lane[h];
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // the shift-term accumulators: each (head, channel) of a wave's row has
  // exactly one owner lane, so a plain read-modify-write is race free
#pragma unroll
  for (int i = 0; i < 8; ++i) wacc[wave][sh_h][sh_c + i] += sh[i];
  __syncthreads();
  for (int idx = tid; idx < kHB * kD; idx += kThreads) {
    const int h = idx / kD, c = idx % kD;
    float M_ = -__builtin_huge_valf();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M_ = fmaxf(M_, wm[w][h]);
    float a = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float e = wm[w][h] == -__builtin_huge_valf() ? 0.f : __expf(wm[w][h] - M_);
      a = fmaf(e, wacc[w][h][c], a);
      l = fmaf(e, wl[w][h], l);
    }
    if (h < nh) {
      float* dst = p.work + ((static_cast<int64_t>(b) * p.Hq + h0 + h) * p.n_split + split) * kPartStride;
      dst[c] = a;
      if (c == 0) {
        dst[128] = M_;
        dst[129] = l;
      }
    }
  }
}

struct CombineParams {
  const uint16_t* q;
  const uint16_t* kr;
  const uint16_t* vr;
  const float* work;
  float* out;
  int Hq, Hkv, grp, hblocks, n_resid, n_split;
  int64_t rcap;
  float scale;
};

constexpr int kCombThreads = 256;
constexpr int kMaxResid = 1024;

__global__ __launch_bounds__(kCombThreads) void attn_combine_kernel(CombineParams p) {
  __shared__ float qf[kHB][kD];
  __shared__ float sres[kHB][kMaxResid];
  __shared__ float rot[kHB][kD];
  __shared__ float red[kCombThreads / kWave][kHB];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int kvh = blockIdx.x / p.hblocks;
  const int hb = blockIdx.x - kvh * p.hblocks;
  const int b = blockIdx.y;
  const int h0 = kvh * p.grp + hb * kHB;
  const int nh = min(kHB, p.grp - hb * kHB);
  const int64_t row = static_cast<int64_t>(b) * p.Hkv + kvh;
  const uint16_t* krow = p.kr + row * p.rcap * kD;
  const uint16_t* vrow = p.vr + row * p.rcap * kD;

  for (int i = tid; i < kHB * kD; i += kCombThreads) {
    const int h = i / kD, c = i % kD;
    qf[h][c] = h < nh ? h2f(p.q[(static_cast<int64_t>(b) * p.Hq + h0 + h) * kD + c]) : 0.f;
  }
  __syncthreads();

  // residual scores
  for (int r = tid; r < p.n_resid; r += kCombThreads) {
    float s[kHB] = {0.f, 0.f, 0.f, 0.f};
    const uint4* kp = reinterpret_cast<const uint4*>(krow + static_cast<int64_t>(r) * kD);
#pragma unroll 4
    for (int i = 0; i < kD / 8; ++i) {
      const uint4 w = kp[i];
      const uint32_t uu[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float a = h2f(uu[k] & 0xffffu), bb = h2f(uu[k] >> 16);
        const int c = 8 * i + 2 * k;
#pragma unroll
        for (int h = 0; h < kHB; ++h) s[h] = fmaf(qf[h][c], a, fmaf(qf[h][c + 1], bb, s[h]));
      }
    }
#pragma unroll
    for (int h = 0; h < kHB; ++h) sres[h][r] = s[h] * p.scale;
  }
  __syncthreads();
  float mres[kHB], lres[kHB];
#pragma unroll
  for (int h = 0; h < kHB; ++h) {
    float mx = -__builtin_huge_valf();
    for (int r = tid; r < p.n_resid; r += kCombThreads) mx = fmaxf(mx, sres[h][r]);
    mx = wave_max(mx);
    if (lane == 0) red[wave][h] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < kHB; ++h) {
    float mx = red[0][h];
#pragma unroll
    for (int w = 1; w < kCombThreads / kWave; ++w) mx = fmaxf(mx, red[w][h]);
    mres[h] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < kHB; ++h) {
    float ls = 0.f;
    for (int r = tid; r < p.n_resid; r += kCombThreads) {
      const float e = __expf(sres[h][r] - mres[h]);
      sres[h][r] = e;
      ls += e;
    }
    ls = wave_sum(ls);
    if (lane == 0) red[wave][h] = ls;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < kHB; ++h) {
    float ls = 0.f;
#pragma unroll
    for (int w = 0; w < kCombThreads / kWave; ++w) ls += red[w][h];
    lres[h] = ls;
  }

  // merge: every thread owns (h, c) for two (h, c) pairs
  float res_acc[2], scale_res[2], L[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int idx = tid + k * kCombThreads;
    const int h = idx / kD, c = idx % kD;
    float ra = 0.f;
    for (int r = 0; r < p.n_resid; ++r) ra = fmaf(sres[h][r], h2f(vrow[static_cast<int64_t>(r) * kD + c]), ra);
    float M = mres[h];
    const float* part = p.work + (static_cast<int64_t>(b) * p.Hq + h0 + min(h, nh - 1)) * p.n_split * kPartStride;
    for (int i = 0; i < p.n_split; ++i) M = fmaxf(M, part[i * kPartStride + 128]);
    float a = 0.f, l = 0.f;
    for (int i = 0; i < p.n_split; ++i) {
      const float e = __expf(part[i * kPartStride + 128] - M);
      a = fmaf(e, part[i * kPartStride + c], a);
      l = fmaf(e, part[i * kPartStride + 129], l);
    }
    const float er = __expf(mres[h] - M);
    rot[h][c] = a;
    res_acc[k] = ra;
    scale_res[k] = er;
    L[k] = fmaf(er, lres[h], l);
  }
  __syncthreads();
#pragma unroll 1
  for (int st = 1; st < kD; st <<= 1) {
    const int h = tid / (kD / 2), pr = tid % (kD / 2);
    const int i = ((pr / st) * 2 * st) + (pr % st);
    const float a = rot[h][i], bb = rot[h][i + st];
    rot[h][i] = a + bb;
    rot[h][i + st] = a - bb;
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int idx = tid + k * kCombThreads;
    const int h = idx / kD, c = idx % kD;
    if (h < nh)
      p.out[(static_cast<int64_t>(b) * p.Hq + h0 + h) * kD + c] =
          fmaf(rot[h][c], kInvSqrtD, scale_res[k] * res_acc[k]) / L[k];
  }
}

template <int M, int G>
hipError_t split_launch(const AttnArgs& a, const SplitParams& sp, hipStream_t s) {
  dim3 grid(a.n_split, a.Hkv * sp.hblocks, a.B);
  hipLaunchKernelGGL((attn_split_kernel<M, G>), grid, dim3(kThreads), 0, s, sp);
  return hipGetLastError();
}

}  // namespace

void attn_plan(int B, int Hq, int Hkv, int n_quant, int group_size, int* n_split, int* chunk) {
  if (n_quant <= 0) {
    *n_split = 0;
    *chunk = 0;
    return;
  }
  const int grp = Hq / Hkv;
  const int64_t units = static_cast<int64_t>(B) * Hkv * ((grp + kHB - 1) / kHB);
  const int max_split = (n_quant + kMinChunk - 1) / kMinChunk;
  int64_t want = (3072 + units - 1) / units;  // about four rounds of three workgroups per CU
  if (want > max_split) want = max_split;
  if (want < 1) want = 1;
  int64_t c = (n_quant + want - 1) / want;
  c = (c + group_size - 1) / group_size * group_size;
  if (c > kMaxChunk) c = kMaxChunk;
  *chunk = static_cast<int>(c);
  *n_split = static_cast<int>((n_quant + c - 1) / c);
}

size_t attn_workspace_bytes(int B, int Hq, int n_split) {
  return static_cast<size_t>(B) * Hq * (n_split > 0 ? n_split : 1) * kPartStride * sizeof(float);
}

hipError_t launch_decode_attention(const AttnArgs& a, hipStream_t s) {
  const int grp = a.Hq / a.Hkv;
  const int hblocks = (grp + kHB - 1) / kHB;
  if (a.n_split > 0) {
    SplitParams sp{a.q, a.kc, a.vc, a.km, a.vm, a.ks, a.vs, static_cast<const uint8_t*>(a.table),
                   a.work, a.Hq, a.Hkv, grp, hblocks, a.n_quant, a.n_split, a.chunk, a.cap, a.scale};
    hipError_t e;
    if (a.sub_dim == 4)
      e = a.group_size == 128 ? split_launch<4, 128>(a, sp, s) : split_launch<4, 256>(a, sp, s);
    else
      e = a.group_size == 128 ? split_launch<8, 128>(a, sp, s) : split_launch<8, 256>(a, sp, s);
    if (e != hipSuccess) return e;
  }
  CombineParams cp{a.q, a.kr, a.vr, a.work, a.out, a.Hq, a.Hkv, grp, hblocks, a.n_resid,
                   a.n_split, a.rcap, a.scale};
  hipLaunchKernelGGL(attn_combine_kernel, dim3(a.Hkv * hblocks, a.B), dim3(kCombThreads), 0, s, cp);
  return hipGetLastError();
}

int attn_max_resid() { return kMaxResid; }

}  // namespace nsn
