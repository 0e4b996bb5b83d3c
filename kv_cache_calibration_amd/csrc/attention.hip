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

constexpr int kThreads = 512;
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

template <int M, int G>
__global__ __launch_bounds__(kThreads) void attn_split_kernel(SplitParams p) {
  constexpr int NSUB = kD / M;
  constexpr int CODE_BYTES = NSUB;   // bytes of codes per token
  constexpr int UPOS = 16 / M;       // sub-vector positions per 16-channel unit
  constexpr int CW = M / 2;          // dwords per fp16 codeword
  constexpr int kMaxGroups = kMaxChunk / G;

  __shared__ float4 lut[NSUB * kCodes];   // T[j][code] -> 4 heads (also the merge scratch)
  __shared__ uint32_t cbh[kCodes * CW];   // fp16 codebook, CW dwords per code
  __shared__ float qr[kHB][kD];
  __shared__ float qo[kMaxGroups][kHB];
  __shared__ uint2 wbuf[kWaves][64];      // per-wave fp16 weights of the tile's tokens
  __shared__ float wm[kWaves][kHB];       // per-wave running max, for the merge

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y / p.hblocks;
  const int hb = blockIdx.y - kvh * p.hblocks;
  const int b = blockIdx.z;
  const int h0 = kvh * p.grp + hb * kHB;
  const int nh = min(kHB, p.grp - hb * kHB);
  const int c0 = split * p.chunk;
  const int c1 = min(p.n_quant, c0 + p.chunk);
  const int64_t row = static_cast<int64_t>(b) * p.Hkv + kvh;  // (b, kvh) cache row

  // ---- set-up: fp16 codebook, rotated queries, per-group <q', o'_g>, table
  const uint32_t* cbg = reinterpret_cast<const uint32_t*>(p.table + kTabCodebookH);
  for (int i = tid; i < kCodes * CW; i += kThreads) cbh[i] = cbg[i];
  if (tid < kHB * kD) {
    const int h = tid / kD, c = tid % kD;
    qr[h][c] = h < nh ? h2f(p.q[(static_cast<int64_t>(b) * p.Hq + h0 + h) * kD + c]) : 0.f;
  }
  __syncthreads();
#pragma unroll 1
  for (int st = 1; st < kD; st <<= 1) {
    if (tid < kHB * kD / 2) {
      const int h = tid / (kD / 2), pr = tid % (kD / 2);
      const int i = ((pr / st) * 2 * st) + (pr % st);
      const float a = qr[h][i], bb = qr[h][i + st];
      qr[h][i] = a + bb;
      qr[h][i + st] = a - bb;
    }
    __syncthreads();
  }
  if (tid < kHB * kD) qr[tid / kD][tid % kD] *= kInvSqrtD;
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
  {
    const float* cbf = reinterpret_cast<const float*>(p.table + kTabCodebook);
    for (int e = tid; e < NSUB * kCodes; e += kThreads) {
      const int j = e / kCodes, k = e % kCodes;
      float c[M];
#pragma unroll
      for (int i = 0; i < M; ++i) c[i] = cbf[k * M + i];
      float t[kHB];
#pragma unroll
      for (int h = 0; h < kHB; ++h) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < M; ++i) s = fmaf(qr[h][M * j + i], c[i], s);
        t[h] = s;
      }
      lut[e] = make_float4(t[0], t[1], t[2], t[3]);
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

  for (int t0 = c0 + 64 * wave; t0 < c1; t0 += 64 * kWaves) {
    // -- score phase: lane = token
    const int t = t0 + lane;
    const bool valid = t < c1;
    uint32_t w8[8];
    uint32_t kmv = 0, vmv = 0;
    if (valid) {
      const uint8_t* src = kcrow + static_cast<int64_t>(t) * CODE_BYTES;
#pragma unroll
      for (int i = 0; i < CODE_BYTES / 16; ++i) {
        const u32x4 c = load_nt16(src + 16 * i);
        w8[4 * i] = c.x;
        w8[4 * i + 1] = c.y;
        w8[4 * i + 2] = c.z;
        w8[4 * i + 3] = c.w;
      }
      kmv = __builtin_nontemporal_load(kmrow + t);
      vmv = __builtin_nontemporal_load(vmrow + t);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) w8[i] = 0u;
    }
    float4 dot = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < NSUB; ++j) {
      const uint32_t code = (w8[j >> 2] >> (8 * (j & 3))) & 0xffu;
      const float4 L = lut[j * kCodes + code];
      dot.x += L.x;
      dot.y += L.y;
      dot.z += L.z;
      dot.w += L.w;
      // keep at most 8 table reads in flight (register pressure)
      if ((j & 7) == 7) __builtin_amdgcn_sched_barrier(0);
    }
    const int g = (t0 - c0) / G;  // one group per tile (64 divides G)
    const float s1k = h2f(kmv & 0xffffu), s2k = h2f(kmv >> 16);
    const float s1v = h2f(vmv & 0xffffu), s2v = h2f(vmv >> 16);
    const float ks1 = p.scale * s1k;
    float s[kHB];
    s[0] = ks1 * fmaf(s2k, dot.x, qo[g][0]);
    s[1] = ks1 * fmaf(s2k, dot.y, qo[g][1]);
    s[2] = ks1 * fmaf(s2k, dot.z, qo[g][2]);
    s[3] = ks1 * fmaf(s2k, dot.w, qo[g][3]);
    float pw[kHB], gs[kHB];
#pragma unroll
    for (int h = 0; h < kHB; ++h) {
      if (!valid) s[h] = -__builtin_huge_valf();
      const float mnew = fmaxf(m_run[h], wave_max(s[h]));  // wave-uniform
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
      gs[h] = wave_sum(pw[h] * s1v);
    }
    const float sv = s1v * s2v;
    wbuf[wave][lane] = make_uint2(
        static_cast<uint32_t>(f2h(pw[0] * sv)) | (static_cast<uint32_t>(f2h(pw[1] * sv)) << 16),
        static_cast<uint32_t>(f2h(pw[2] * sv)) | (static_cast<uint32_t>(f2h(pw[3] * sv)) << 16));
    // shift term p s1 o'_g: this lane owns head sh_h, channels sh_c .. sh_c + 7
    {
      const u32x4 o = load_nt16(vsrow + static_cast<int64_t>(c0 / G + g) * kD + sh_c);
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
#pragma unroll 2
    for (int k = 0; k < 4; ++k) {
      const int ia = slot + 16 * k, ib = ia + 8;
      const int ta = t0 + ia, tb = t0 + ib;
      uint32_t va = 0, vb = 0;
      if constexpr (M == 4) {
        if (ta < c1) va = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(vcrow + static_cast<int64_t>(ta) * CODE_BYTES) + u);
        if (tb < c1) vb = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(vcrow + static_cast<int64_t>(tb) * CODE_BYTES) + u);
      } else {
        if (ta < c1) va = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(vcrow + static_cast<int64_t>(ta) * CODE_BYTES) + u);
        if (tb < c1) vb = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(vcrow + static_cast<int64_t>(tb) * CODE_BYTES) + u);
      }
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
  }

  // ---- merge: slots inside each wave, then the 16 waves
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
  __syncthreads();  // every wave is done with the lookup table
  float* wacc = reinterpret_cast<float*>(lut);        // [kWaves][4][128]
  float* wl = wacc + kWaves * kHB * kD;               // [kWaves][4]
  if (slot == 0) {
#pragma unroll
    for (int h = 0; h < kHB; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) wacc[(wave * kHB + h) * kD + 16 * u + i] = acc[h][i];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < kHB; ++h) {
      wm[wave][h] = m_run[h];
      wl[wave * kHB + h] = l_lane[h];
    }
  }
  __syncthreads();
  // the shift-term accumulators: each (head, channel) of a wave's row has
  // exactly one owner lane, so a plain read-modify-write is race free
#pragma unroll
  for (int i = 0; i < 8; ++i) wacc[(wave * kHB + sh_h) * kD + sh_c + i] += sh[i];
  __syncthreads();
  if (tid < kHB * kD) {
    const int h = tid / kD, c = tid % kD;
    float M_ = -__builtin_huge_valf();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M_ = fmaxf(M_, wm[w][h]);
    float a = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float e = wm[w][h] == -__builtin_huge_valf() ? 0.f : __expf(wm[w][h] - M_);
      a = fmaf(e, wacc[(w * kHB + h) * kD + c], a);
      l = fmaf(e, wl[w * kHB + h], l);
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
  int64_t want = (1024 + units - 1) / units;  // about four workgroups per CU
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
