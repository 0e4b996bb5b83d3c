// Decode attention over an NSN-quantized KV cache plus an fp16 residual
// window, for gfx950.
// [NSNQuant summary (gist.science), Methodology §4: KIVI-style split of the
//  cache into a quantized part and a full-precision residual; the attention
//  score takes the NSN byproducts s1, s2, o directly.]
//
// Everything on quantized tokens happens in the rotated domain: with
// q' = H q / sqrt(d) (computed once per workgroup),
//   <q, x_hat_t> = s1_t (s2'_t <q', c(codes_t)> + <q', o'_g>),
// so a key never has to be dequantized.  <q', c(codes_t)> is a sum over the
// token's sub-vectors of a per-workgroup lookup table
//   T[j][code][h] = <q'_h[m j : m j + m], C[code]>
// (one LDS read of all heads' entries per code).  Values are accumulated in
// the rotated domain too, and rotated back once per query head at the end.
//
// attn_split_kernel: one workgroup (1024 threads) per (token chunk, kv head,
//   block of up to 4 query heads, batch).  Per 1024-token tile it scores
//   every token (one thread per token), updates the running max, and
//   accumulates p * s1 * s2' * c(codes) into per-thread rotated-domain
//   accumulators (thread = 16-channel slice x token slot) plus the per-group
//   shift term p * s1 * o'_g.  It writes (acc[128], max, sum) per head.
// attn_combine_kernel: one workgroup per (kv head block, batch): the
//   residual window's exact fp16 attention, a log-sum-exp merge with the
//   chunk partials, one inverse rotation, normalization.
#include "nsn_device.h"
#include "nsn_launch.h"

namespace nsn {

namespace {

constexpr int kThreads = 1024;
constexpr int kTile = 1024;         // tokens per tile (one per thread in the score phase)
constexpr int kHB = 4;              // query heads per workgroup
constexpr int kMaxChunk = 8192;     // quantized tokens per workgroup, at most
constexpr int kMinChunk = 1024;
constexpr int kPartStride = 132;    // acc[128], m, l, pad
constexpr int kWaves = kThreads / kWave;
constexpr int kSlots = kThreads / 8;  // token slots in the value phase
constexpr float kInvSqrtD = 0.08838834764831845f;

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

__device__ __forceinline__ uint32_t byte_of(const uint32_t (&w)[8], int j) {
  return (w[j >> 2] >> (8 * (j & 3))) & 0xffu;
}

template <int M, int G>
__global__ __launch_bounds__(kThreads) void attn_split_kernel(SplitParams p) {
  constexpr int NSUB = kD / M;
  constexpr int CODE_BYTES = NSUB;              // bytes of codes per token
  constexpr int UNIT_POS = 16 / M;              // sub-vector positions per 16-channel unit
  constexpr int kMaxGroups = kMaxChunk / G;
  constexpr int kTileGroups = kTile / G;

  __shared__ float4 lut[NSUB * kCodes];         // T[j][code] -> 4 heads
  __shared__ float cbs[kCodes * M];
  __shared__ float qr[kHB][kD];
  __shared__ float4 wts[kTile];
  __shared__ float qo[kMaxGroups][kHB];
  __shared__ float red[kWaves][kHB];
  __shared__ float gred[kWaves][kHB];

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

  // ---- setup: codebook, rotated queries, per-group <q', o'_g>, lookup table
  const float* cbg = reinterpret_cast<const float*>(p.table + kTabCodebook);
  for (int i = tid; i < kCodes * M; i += kThreads) cbs[i] = cbg[i];
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
  for (int e = tid; e < NSUB * kCodes; e += kThreads) {
    const int j = e / kCodes, k = e % kCodes;
    float t[kHB];
#pragma unroll
    for (int h = 0; h < kHB; ++h) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < M; ++i) s = fmaf(qr[h][M * j + i], cbs[k * M + i], s);
      t[h] = s;
    }
    lut[e] = make_float4(t[0], t[1], t[2], t[3]);
  }
  __syncthreads();

  // ---- main loop
  float m_run[kHB], l_part[kHB];
#pragma unroll
  for (int h = 0; h < kHB; ++h) {
    m_run[h] = -__builtin_huge_valf();
    l_part[h] = 0.f;
  }
  float acc[kHB][16];
#pragma unroll
  for (int h = 0; h < kHB; ++h)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[h][i] = 0.f;
  float acc_sh = 0.f;  // shift term for (h, c) = (tid / 128, tid % 128), tid < 512
  const int u = tid & 7;       // 16-channel unit of the value phase
  const int slot = tid >> 3;   // token slot of the value phase

  const uint8_t* kcrow = p.kc + row * p.cap * CODE_BYTES;
  const uint8_t* vcrow = p.vc + row * p.cap * CODE_BYTES;
  const uint32_t* kmrow = reinterpret_cast<const uint32_t*>(p.km + row * p.cap * 2);
  const uint32_t* vmrow = reinterpret_cast<const uint32_t*>(p.vm + row * p.cap * 2);
  const uint16_t* vsrow = p.vs + row * (p.cap / G) * kD;

  for (int t0 = c0; t0 < c1; t0 += kTile) {
    // -- score phase: one thread per token
    const int t = t0 + tid;
    const bool valid = t < c1;
    float s[kHB];
    float s1v = 0.f, s2v = 0.f;
    if (valid) {
      uint32_t w[8];
      const uint8_t* src = kcrow + static_cast<int64_t>(t) * CODE_BYTES;
#pragma unroll
      for (int i = 0; i < CODE_BYTES / 16; ++i) {
        const u32x4 c = load_nt16(src + 16 * i);
        w[4 * i] = c.x;
        w[4 * i + 1] = c.y;
        w[4 * i + 2] = c.z;
        w[4 * i + 3] = c.w;
      }
      float4 dot = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int j = 0; j < NSUB; ++j) {
        const float4 L = lut[j * kCodes + byte_of(w, j)];
        dot.x += L.x;
        dot.y += L.y;
        dot.z += L.z;
        dot.w += L.w;
      }
      const uint32_t kmv = __builtin_nontemporal_load(kmrow + t);
      const uint32_t vmv = __builtin_nontemporal_load(vmrow + t);
      const float s1k = h2f(kmv & 0xffffu), s2k = h2f(kmv >> 16);
      s1v = h2f(vmv & 0xffffu);
      s2v = h2f(vmv >> 16);
      const int g = (t - c0) / G;
      const float ks1 = p.scale * s1k;
      s[0] = ks1 * fmaf(s2k, dot.x, qo[g][0]);
      s[1] = ks1 * fmaf(s2k, dot.y, qo[g][1]);
      s[2] = ks1 * fmaf(s2k, dot.z, qo[g][2]);
      s[3] = ks1 * fmaf(s2k, dot.w, qo[g][3]);
    } else {
#pragma unroll
      for (int h = 0; h < kHB; ++h) s[h] = -__builtin_huge_valf();
    }
    // tile max per head
#pragma unroll
    for (int h = 0; h < kHB; ++h) {
      const float mx = wave_max(s[h]);
      if (lane == 0) red[wave][h] = mx;
    }
    __syncthreads();
    float f[kHB], pw[kHB];
#pragma unroll
    for (int h = 0; h < kHB; ++h) {
      float mx = red[0][h];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, red[w][h]);
      const float mnew = fmaxf(m_run[h], mx);
      f[h] = __expf(m_run[h] - mnew);
      m_run[h] = mnew;
      pw[h] = valid ? __expf(s[h] - mnew) : 0.f;
      l_part[h] = fmaf(l_part[h], f[h], pw[h]);
    }
    wts[tid] = make_float4(pw[0] * s1v * s2v, pw[1] * s1v * s2v, pw[2] * s1v * s2v,
                           pw[3] * s1v * s2v);
    // per-group sums of p * s1 for the shift term (a group spans G/64 waves)
#pragma unroll
    for (int h = 0; h < kHB; ++h) {
      const float gs = wave_sum(pw[h] * s1v);
      if (lane == 0) gred[wave][h] = gs;
    }
    __syncthreads();
    if (tid < kHB * kD) {
      const int h = tid / kD, c = tid % kD;
      float a = acc_sh * f[h];
      const int gt0 = (t0 - c0) / G;
      for (int gg = 0; gg < kTileGroups; ++gg) {
        if (t0 + gg * G >= c1) break;
        float gs = 0.f;
#pragma unroll
        for (int w = 0; w < G / kWave; ++w) gs += gred[gg * (G / kWave) + w][h];
        a = fmaf(gs, h2f(vsrow[static_cast<int64_t>(c0 / G + gt0 + gg) * kD + c]), a);
      }
      acc_sh = a;
    }
    // -- value phase: thread = (16-channel unit u, token slot)
#pragma unroll
    for (int h = 0; h < kHB; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[h][i] *= f[h];
    for (int i = 0; i < kTile / kSlots; ++i) {
      const int tt = t0 + slot + kSlots * i;
      if (tt >= c1) break;
      const float4 wv = wts[tt - t0];
      uint32_t cw;
      if constexpr (M == 4)
        cw = __builtin_nontemporal_load(
            reinterpret_cast<const uint32_t*>(vcrow + static_cast<int64_t>(tt) * CODE_BYTES) + u);
      else
        cw = __builtin_nontemporal_load(
            reinterpret_cast<const uint16_t*>(vcrow + static_cast<int64_t>(tt) * CODE_BYTES) + u);
#pragma unroll
      for (int pos = 0; pos < UNIT_POS; ++pos) {
        const int code = (cw >> (8 * pos)) & 0xff;
#pragma unroll
        for (int e = 0; e < M; ++e) {
          const float c = cbs[code * M + e];
          acc[0][pos * M + e] = fmaf(wv.x, c, acc[0][pos * M + e]);
          acc[1][pos * M + e] = fmaf(wv.y, c, acc[1][pos * M + e]);
          acc[2][pos * M + e] = fmaf(wv.z, c, acc[2][pos * M + e]);
          acc[3][pos * M + e] = fmaf(wv.w, c, acc[3][pos * M + e]);
        }
      }
    }
    __syncthreads();
  }

  // ---- reductions and partial output
  // sum over token slots: lanes with equal u inside a wave, then over waves
#pragma unroll
  for (int h = 0; h < kHB; ++h)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = acc[h][i];
      v += __shfl_xor(v, 8, kWave);
      v += __shfl_xor(v, 16, kWave);
      v += __shfl_xor(v, 32, kWave);
      acc[h][i] = v;
    }
  float* racc = reinterpret_cast<float*>(lut);  // [kWaves][8 units][64]
  if (lane < 8) {
#pragma unroll
    for (int h = 0; h < kHB; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) racc[(wave * 8 + lane) * 64 + h * 16 + i] = acc[h][i];
  }
#pragma unroll
  for (int h = 0; h < kHB; ++h) {
    const float ls = wave_sum(l_part[h]);
    if (lane == 0) red[wave][h] = ls;
  }
  __syncthreads();
  if (tid < kHB * kD) {
    const int h = tid / kD, c = tid % kD;
    const int uu = c / 16, ii = c % 16;
    float a = acc_sh;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) a += racc[(w * 8 + uu) * 64 + h * 16 + ii];
    if (h < nh) {
      float* dst = p.work + ((static_cast<int64_t>(b) * p.Hq + h0 + h) * p.n_split + split) * kPartStride;
      dst[c] = a;
      if (c == 0) {
        float l = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) l += red[w][h];
        dst[128] = m_run[h];
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
