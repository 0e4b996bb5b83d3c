// Decode attention over an NSN-quantized KV cache plus an fp16 residual
// window, for gfx950.
// [NSNQuant summary (gist.science), Methodology §4: KIVI-style split of the
//  cache into a quantized part and a full-precision residual; the attention
//  score takes the NSN byproducts s1, s2, o directly.]
//
// Quantized tokens are handled in the rotated domain.  With q' = H q / sqrt(d),
//   <q, x_hat_t> = s1_t (s2'_t <q', c(codes_t)> + <q', o'_g>),
// so keys are never dequantized, and the rotated value sum splits into
//   sum_t p_t s1_t s2'_t c(codes_t)  +  sum_g o'_g sum_{t in g} p_t s1_t;
// one inverse rotation per query head at the end gives the output.  The
// randomized rotation (§2) only changes the two ends: q' = H D q / sqrt(d),
// and the inverse rotation is followed by D.
//
// attn_split_kernel: one workgroup (4 waves) per (token chunk, kv head, block
//   of up to 4 query heads, batch).  Tile i (64 tokens) of the chunk belongs
//   to wave i mod 4; each wave runs its own online softmax with no workgroup
//   barrier:
//     scores   16 MFMA 16x16x32 (fp16 in, fp32 out): rows = the 4 heads' q'
//              split into an fp16 high and low part, columns = 16 tokens,
//              K = 32 channels; the B operand is two fp16 codewords per lane
//              read straight from the codebook in LDS.  Two permlane swaps
//              leave lane l with token l's 4 scores.
//     softmax  base-2 exponent; the running max is raised (and the
//              accumulators rescaled) only when some score exceeds it.
//     values   16 MFMA: A = codewords, transposed on the fly by
//              ds_read_b64_tr_b16 from the codebook (the lanes' addresses
//              select the codes), B = the tile's fp16 high/low weights
//              p s1 s2' from a per-wave LDS row buffer.
//     shift    the tile's sum of p s1 per head (fp32) is kept in LDS with the
//              max it refers to and applied to the group shifts at the end.
//   The workgroup of the last chunk first takes the fp16 residual window
//   (exact scores, original domain), written as partial n_split.
//   Variants (template flags): ROPE -- keys stored before rotary embedding
//   (NSNQuant summary §4), scored in the original domain: codewords through
//   a matrix-core Hadamard, shift, rotation by the key's position, dot
//   products with the turned queries on the matrix cores; the value side is
//   unchanged.  DQ -- double-quantized metadata (§3, Double Quantization):
//   s1 and o' decoded from the 4-bit group records on the fly.
// attn_combine_kernel: one wave per (batch, query head): log-sum-exp merge of
//   the chunk partials, inverse rotation, residual partial, normalization.
#include <type_traits>

#include "nsn_device.h"
#include "nsn_launch.h"

namespace nsn {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kHB = 4;               // query heads per workgroup
constexpr int kTile = 64;            // tokens per wave iteration
constexpr int kMaxChunk = 8192;      // quantized tokens per workgroup, at most
constexpr int kMaxTiles = kMaxChunk / kTile;
constexpr int kMaxGroups = kMaxChunk / 128;
constexpr int kMinChunk = 512;
constexpr int kMaxResid = 1024;
constexpr int kResidWeight = 7;      // residual token ~ this many quantized ones (split plan)
constexpr int kPartStride = 132;     // acc[128], m, l, pad
constexpr int kBlocksPerCU = 4;      // split workgroups one CU can hold (<= 128 VGPRs)
constexpr int kPlanBlocksPerCU = 3;  // workgroups per CU the split count aims at (measured best)
constexpr int kPlanBlocksPerCURope = 2;  // the rotary kernel: two fit per CU (LDS, registers)
constexpr int kPlanCUs = 256;
constexpr float kInvSqrtD = 0.08838834764831845f;
constexpr float kLog2e = 1.4426950408889634f;

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

struct SplitParams {
  const uint16_t* q;
  const uint8_t* kc;
  const uint8_t* vc;
  const uint16_t* km;
  const uint16_t* vm;
  const uint16_t* ks;
  const uint16_t* vs;
  const uint16_t* kr;
  const uint16_t* vr;
  const uint8_t* table;
  float* work;
  int Hq, Hkv, grp, hblocks, n_quant, n_split, chunk, n_resid;
  int64_t cap, rcap;
  float scale;
  int64_t q_pos;     // query position (keys stored before rotary embedding)
  float rope_base;   // rotary base, theta_i = base^(-i/64)
  Signs sg;          // randomized rotation: q' = H D q / sqrt(d) (plain kernel only)
};

// Double-quantized metadata: per group of the chunk, (lo, step) of the s1
// grid of keys and of values, and the value shift's scale.
struct DqSmem {
  float2 kls[kMaxGroups];
  float2 vls[kMaxGroups];
  float vsc[kMaxGroups];
};

template <int M>
struct SplitSmem {
  uint32_t cbh[kCodes * M / 2];      // fp16 codebook, 2m bytes per code
  float qr[kHB][kD];                 // rotated queries
  float qo[kMaxGroups][kHB];         // <q'_h, o'_g> per group of the chunk
  float sg[kMaxGroups][kHB];         // per group: sum of p s1, relative to the final max
  float ssum[kMaxTiles][kHB];        // per tile: sum of p s1 ...
  float smax[kMaxTiles][kHB];        // ... relative to this max
  // per-wave weight rows [token][slot] (slots 0..3 fp16 high part of p s1 s2'
  // of heads 0..3, 4..7 low part, 8..15 zero); after the tile loop the same
  // 2 KB hold the wave's value sums as float[kHB][kD]
  uint16_t wrow[kWaves][kTile][16];
  float wm[kWaves][kHB];
  float wl[kWaves][kHB];
  DqSmem dq;                         // double-quantized metadata (the union's
                                     // residual half is larger, so free)
};
struct ResidSmem {
  float4 sres[kMaxResid];          // per token: scores of the 4 heads (base 2)
  float vpart[kWaves][kHB][kD];
};
template <int M>
union AttnSmem {
  SplitSmem<M> s;
  ResidSmem r;
};
// Keys stored before rotary embedding: every tile of 64 keys (positions
// P .. P + 63) is scored as <R(q_pos - P) q, R(t) k_t> = <R(q_pos) q,
// R(P + t) k_t>, so the per-key rotation R(t) depends only on the key's
// offset t in the tile (a table built once per workgroup) and the query is
// turned once per tile.
struct RopeSmem {
  float2 tab[kD / 2][kTile];     // (cos, sin) of t * theta_i, [pair i][offset t]
  float q[kHB][kD];              // the block's queries, original domain
  float qp[kWaves][kHB][kD];     // per wave: the queries turned by q_pos - P
  float og[kWaves][kD];          // per wave: the tile's group shift, original domain
  u32x4 qkl[kWaves][8][2][8];   // per wave: the query MFMA operand, [slice][lane half][row]
};
struct NoRopeSmem {
  int unused;
};
// ds_read_b64_tr_b16: inside each group of 16 lanes, lane 4a + b receives
// element b of the 8-byte chunks addressed by lanes 4k + a, k = 0..3.  With
// chunk (lane 4k + a) = 4 channels of token k, lane 4a + b gets one channel
// of 4 consecutive tokens: the k-major layout of an MFMA operand.
__device__ __forceinline__ uint2 ds_tr16(uint32_t lds_byte_addr) {
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<lds_v4s*>(static_cast<uintptr_t>(lds_byte_addr)));
  return __builtin_bit_cast(uint2, r);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// byte K of w, times 2^S (a byte offset into the codebook).  The compiler
// takes bytes 1-3 with one SDWA shift but byte 0 with a shift and a mask;
// SDWA0 selects one SDWA shift for byte 0 too (the shift count sits in a
// VGPR, hoisted out of the tile loop).  The rotary kernels keep the
// compiler's form.
template <int K, int S, bool SDWA0 = false>
__device__ __forceinline__ uint32_t code_off(uint32_t w) {
  if constexpr (K == 0 && SDWA0) {
    uint32_t r;
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0"
        : "=v"(r)
        : "v"(static_cast<uint32_t>(S)), "v"(w));
    return r;
  } else {
    return ((w >> (8 * K)) & 0xffu) << S;
  }
}

__device__ __forceinline__ v4f mfma16(const u32x4& a, const u32x4& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b),
                                                c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int M>
struct TileData {
  using CT = std::conditional_t<M == 4, u32x2, uint32_t>;
  // key codes of token 16 tb + lane % 16: bytes 8R.. (m = 4) or 4R.. (m = 8)
  // of the token, R = lane / 16
  CT kc[4];
  // value codes of token 32 (i / 2) + 8R + 4 (i % 2) + (lane % 16) / 4:
  // bytes 8a.. (m = 4) or 4a.. (m = 8), a = lane % 4
  CT vc[4];
  uint32_t km, vm;  // (s1, s2') of token `lane`
};

// The three parts of a tile are loaded separately, each right after the
// last use of the current tile's part (a full phase ahead of the next use
// with one set of registers).
template <int M>
__device__ __forceinline__ void load_keys(TileData<M>& d, const uint8_t* kb, uint32_t koff) {
  using CT = typename TileData<M>::CT;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
    d.kc[tb] = __builtin_nontemporal_load(reinterpret_cast<const CT*>(kb + koff + 16 * tb * (kD / M)));
}
template <int M>
__device__ __forceinline__ void load_values(TileData<M>& d, const uint8_t* vb, uint32_t voff) {
  using CT = typename TileData<M>::CT;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    d.vc[i] = __builtin_nontemporal_load(
        reinterpret_cast<const CT*>(vb + voff + (32 * (i >> 1) + 4 * (i & 1)) * (kD / M)));
}
template <int M>
__device__ __forceinline__ void load_meta(TileData<M>& d, const uint32_t* kmb, const uint32_t* vmb, int lane) {
  d.km = __builtin_nontemporal_load(kmb + lane);
  d.vm = __builtin_nontemporal_load(vmb + lane);
}

// Score B operand of step s for token block tb: the channels 32R + 8s .. + 7
// (R = lane / 16) of the lane's token, i.e. sub-vectors 8R + 2s, 8R + 2s + 1
// (m = 4) or 4R + s (m = 8).
template <int M, int S>
__device__ __forceinline__ u32x4 score_b(const typename TileData<M>::CT& kc, const uint32_t* cbh) {
  const char* base = reinterpret_cast<const char*>(cbh);
  if constexpr (M == 4) {
    const uint32_t w = kc[S >> 1];
    const u32x2 c0 = *reinterpret_cast<const u32x2*>(base + code_off<2 * (S & 1), 3, true>(w));
    const u32x2 c1 = *reinterpret_cast<const u32x2*>(base + code_off<2 * (S & 1) + 1, 3, true>(w));
    return u32x4{c0.x, c0.y, c1.x, c1.y};
  } else {
    return *reinterpret_cast<const u32x4*>(base + code_off<S, 4, true>(kc));
  }
}

// Value A operand chunk of channel block CB for one token: channels
// 4 (8a + CB) .. + 3 (a = lane % 4): code byte CB (m = 4) or half CB % 2 of
// code byte CB / 2 (m = 8) of the lane's value-code bytes.
template <int M, int CB, bool SDWA0>
__device__ __forceinline__ uint32_t value_chunk_off(const typename TileData<M>::CT& vc) {
  if constexpr (M == 4)
    return code_off<CB & 3, 3, SDWA0>(vc[CB >> 2]);
  else
    return code_off<(CB >> 1), 4, SDWA0>(vc) + 8u * (CB & 1);
}

template <int M, int CB, bool SDWA0>
__device__ __forceinline__ void value_steps(v4f (&acc)[8], const TileData<M>& d, int kb, const u32x4& bw,
                                            uint32_t cbh_base) {
  if constexpr (CB < 8) {
    const uint2 a0 = ds_tr16(cbh_base + value_chunk_off<M, CB, SDWA0>(d.vc[2 * kb]));
    const uint2 a1 = ds_tr16(cbh_base + value_chunk_off<M, CB, SDWA0>(d.vc[2 * kb + 1]));
    acc[CB] = mfma16(u32x4{a0.x, a0.y, a1.x, a1.y}, bw, acc[CB]);
    value_steps<M, CB + 1, SDWA0>(acc, d, kb, bw, cbh_base);
  }
}

template <int M, int S>
__device__ __forceinline__ void score_steps(v4f& sa, const u32x4 (&qa)[4], const typename TileData<M>::CT& kc,
                                            const uint32_t* cbh) {
  if constexpr (S < 4) {
    sa = mfma16(qa[S], score_b<M, S>(kc, cbh), sa);
    score_steps<M, S + 1>(sa, qa, kc, cbh);
  }
}
__device__ __forceinline__ float dpp_row_shr4(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, false));
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A operands of the Sylvester matrix H128 = H8 (x) H16 for
// v_mfma_f32_32x32x16_f16: block (a, kb) (rows 32a.., K slice 16kb..) is
// +-(one 16-column pattern), the sign (-1)^popcount(2a & kb), times the
// bit-4 row sign for odd kb.  +-1 are exact in fp16.
struct HOps {
  u32x4 P0, P1, N0, N1;
};
__device__ __forceinline__ HOps hadamard_ops(int lane) {
  const int r16 = lane & 15, r4 = (lane >> 4) & 1, hf = lane >> 5;
  uint32_t wv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c0 = 8 * hf + 2 * i, c1 = c0 + 1;
    const uint32_t lo = (__popc(r16 & c0) & 1) ? 0xBC00u : 0x3C00u;
    const uint32_t hi = (__popc(r16 & c1) & 1) ? 0xBC00u : 0x3C00u;
    wv[i] = lo | (hi << 16);
  }
  HOps o;
  o.P0 = u32x4{wv[0], wv[1], wv[2], wv[3]};
  const uint32_t f = r4 ? 0x80008000u : 0u;
  o.P1 = u32x4{wv[0] ^ f, wv[1] ^ f, wv[2] ^ f, wv[3] ^ f};
  o.N0 = o.P0 ^ 0x80008000u;
  o.N1 = o.P1 ^ 0x80008000u;
  return o;
}
typedef float v16f __attribute__((ext_vector_type(16)));
// block (a, kb); a and kb are constants once the caller's loops unroll
__device__ __forceinline__ v8h hblk(const HOps& o, int a, int kb) {
  const bool neg = (__popc((2 * a) & kb) & 1) != 0;
  return __builtin_bit_cast(v8h, (kb & 1) ? (neg ? o.N1 : o.P1) : (neg ? o.N0 : o.P0));
}

// fp16 pair of (z0, z1), each rounded once toward zero (one instruction for
// the pair), and the fp16 pair of the remainders (z0 - hi0, z1 - hi1),
// rounded to nearest even: together about 22 significant bits (the
// remainder is below one fp16 ulp of z).  Arithmetic only.
__device__ __forceinline__ uint32_t f16_hi2(float z0, float z1) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(z0, z1));
}
// The result feeds matrix-core operands.  A VALU write of a VGPR needs two
// wait states before an MFMA reads it; the compiler inserts them after its
// own VALU instructions but does not count an inline-asm instruction as
// such a write, so the asm block ends with them.
__device__ __forceinline__ uint32_t f16_lo2(float z0, float z1, uint32_t hi) {
  uint32_t l;
  asm("v_fma_mixlo_f16 %0, %1, 1.0, -%2 op_sel:[0,0,0] op_sel_hi:[0,0,1]" : "=v"(l) : "v"(z0), "v"(hi));
  asm("v_fma_mixhi_f16 %0, %1, 1.0, -%2 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\ts_nop 1"
      : "+v"(l) : "v"(z1), "v"(hi));
  return l;
}

// Rotary angle: theta_i = base^(-i/64) for channel pair (i, i + 64).
__device__ __forceinline__ double rope_theta(float base, int i) {
  return pow(static_cast<double>(base), -static_cast<double>(i) / 64.0);
}
// (cos a, sin a), the angle reduced to [-pi, pi] in double first.
__device__ __forceinline__ float2 rope_cs(double a) {
  const double two_pi = 6.283185307179586476925;
  const double r = a - two_pi * rint(a * (1.0 / two_pi));
  float sn, cs;
  sincosf(static_cast<float>(r), &sn, &cs);
  return make_float2(cs, sn);
}
// The wave's queries turned by the angle delta * theta (lane = pair i):
// pair (x, y) -> (x cos - y sin, y cos + x sin).  The caller syncs the wave.
__device__ __forceinline__ void rope_query(const RopeSmem& rs, float (&qp)[kHB][kD], int lane,
                                           double theta, int64_t delta) {
  const float2 cs = rope_cs(static_cast<double>(delta) * theta);
#pragma unroll
  for (int h = 0; h < kHB; ++h) {
    const float x = rs.q[h][lane], y = rs.q[h][lane + kD / 2];
    qp[h][lane] = x * cs.x - y * cs.y;
    qp[h][lane + kD / 2] = y * cs.x + x * cs.y;
  }
}
// Scores (base-2 units) of the lane's key k (original domain, before the
// rotary embedding; k[c] = a hc[c] + b og[c]) at offset `lane` of its tile
// against the turned queries qp.
__device__ __forceinline__ void rope_dot(float (&s)[kHB], const float (&hc)[kD], float a, float bo,
                                         const float* og, const RopeSmem& rs,
                                         const float (&qp)[kHB][kD], int lane, float qscale) {
  float acc[kHB] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i0 = 0; i0 < kD / 2; i0 += 4) {
    float ox[4] = {0.f, 0.f, 0.f, 0.f}, oy[4] = {0.f, 0.f, 0.f, 0.f};
    if (og) {
      const float4 u = *reinterpret_cast<const float4*>(og + i0);
      const float4 v = *reinterpret_cast<const float4*>(og + kD / 2 + i0);
      ox[0] = u.x; ox[1] = u.y; ox[2] = u.z; ox[3] = u.w;
      oy[0] = v.x; oy[1] = v.y; oy[2] = v.z; oy[3] = v.w;
    }
    float qx[kHB][4], qy[kHB][4];
#pragma unroll
    for (int h = 0; h < kHB; ++h) {
      const float4 u = *reinterpret_cast<const float4*>(&qp[h][i0]);
      const float4 v = *reinterpret_cast<const float4*>(&qp[h][kD / 2 + i0]);
      qx[h][0] = u.x; qx[h][1] = u.y; qx[h][2] = u.z; qx[h][3] = u.w;
      qy[h][0] = v.x; qy[h][1] = v.y; qy[h][2] = v.z; qy[h][3] = v.w;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = i0 + e;
      const float2 cs = rs.tab[i][lane];
      const float x = fmaf(a, hc[i], bo * ox[e]);
      const float y = fmaf(a, hc[i + kD / 2], bo * oy[e]);
      const float kx = x * cs.x - y * cs.y;
      const float ky = y * cs.x + x * cs.y;
#pragma unroll
      for (int h = 0; h < kHB; ++h) acc[h] = fmaf(qy[h][e], ky, fmaf(qx[h][e], kx, acc[h]));
    }
  }
#pragma unroll
  for (int h = 0; h < kHB; ++h) s[h] = acc[h] * qscale;
}

// The fp16 residual window of one (batch, kv head, head block), in the
// original domain, written as partial n_split.  Every load is issued first;
// scores are exact MFMA products of the fp16 q and k (fp32 sums) into LDS;
// after one barrier every wave takes the per-head max and sum itself; values
// run one thread per (channel pair, token residue mod 4) with weights formed
// on the fly, and the four residue classes are summed through LDS.
template <bool ROPE>
__device__ void resid_block(const SplitParams& p, ResidSmem& sm, RopeSmem* rs, double theta, int b,
                            int kvh, int hb) {
  constexpr int kVPre = 32;              // value words held in registers per thread
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int R = lane >> 4, c16 = lane & 15;
  const int h0 = kvh * p.grp + hb * kHB;
  const int nh = min(kHB, p.grp - hb * kHB);
  const int64_t row = static_cast<int64_t>(b) * p.Hkv + kvh;
  const uint16_t* krow = p.kr + row * p.rcap * kD;
  const uint32_t* vrow = reinterpret_cast<const uint32_t*>(p.vr + row * p.rcap * kD);
  const int nr = p.n_resid;
  const float qscale = p.scale * kLog2e;   // scores in base-2 units
  const float ninf = -__builtin_huge_valf();

  // ---- all loads: this thread's value words, the wave's key blocks, q
  uint32_t vpre[kVPre];
#pragma unroll
  for (int i = 0; i < kVPre; ++i) {
    const int t = wave + kWaves * i;
    vpre[i] = t < nr ? vrow[static_cast<int64_t>(t) * (kD / 2) + lane] : 0u;
  }
  if constexpr (ROPE) {
    // keys before rotary embedding, positions n_quant + t: tiles of 64, lane
    // = token, wave w takes tiles w, w + 4, ...
    for (int rt = wave; rt * kTile < nr; rt += kWaves) {
      const int t = rt * kTile + lane;
      rope_query(*rs, rs->qp[wave], lane, theta, p.q_pos - (static_cast<int64_t>(p.n_quant) + rt * kTile));
      float hc[kD];
#pragma unroll
      for (int i = 0; i < kD / 8; ++i) {
        const u32x4 w = t < nr ? *reinterpret_cast<const u32x4*>(krow + static_cast<int64_t>(t) * kD + 8 * i)
                               : u32x4{0u, 0u, 0u, 0u};
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          hc[8 * i + 2 * k] = h2f(ww[k] & 0xffffu);
          hc[8 * i + 2 * k + 1] = h2f(ww[k] >> 16);
        }
      }
      wave_lds_sync();
      float sc[kHB];
      rope_dot(sc, hc, 1.0f, 0.f, nullptr, *rs, rs->qp[wave], lane, qscale);
      if (t < nr) sm.sres[t] = make_float4(sc[0], sc[1], sc[2], sc[3]);
      wave_lds_sync();
    }
  } else {
  // A operand per step s: row c16 = head c16 (< nh), K index 8R + v =
  // channel 32 s + 8R + v
  u32x4 qa[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    qa[s] = c16 < nh ? *reinterpret_cast<const u32x4*>(
                           p.q + (static_cast<int64_t>(b) * p.Hq + h0 + c16) * kD + 32 * s + 8 * R)
                     : u32x4{0u, 0u, 0u, 0u};
  for (int tb0 = 2 * wave; tb0 * 16 < nr; tb0 += 2 * kWaves) {
    u32x4 kb[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = (tb0 + u) * 16 + c16;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        kb[u][s] = t < nr ? *reinterpret_cast<const u32x4*>(krow + static_cast<int64_t>(t) * kD + 32 * s + 8 * R)
                          : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = (tb0 + u) * 16 + c16;
      v4f d = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) d = mfma16(qa[s], kb[u][s], d);
      if (R == 0 && t < nr)
        sm.sres[t] = make_float4(d[0] * qscale, d[1] * qscale, d[2] * qscale, d[3] * qscale);
    }
  }
  }
  __syncthreads();
  // ---- per-head max and sum, every wave over all tokens
  float mres[kHB] = {ninf, ninf, ninf, ninf};
  for (int t = lane; t < nr; t += kWave) {
    const float4 v = sm.sres[t];
    mres[0] = fmaxf(mres[0], v.x);
    mres[1] = fmaxf(mres[1], v.y);
    mres[2] = fmaxf(mres[2], v.z);
    mres[3] = fmaxf(mres[3], v.w);
  }
#pragma unroll
  for (int h = 0; h < kHB; ++h) mres[h] = wave_max_fast(mres[h]);
  float lres[kHB] = {0.f, 0.f, 0.f, 0.f};
  for (int t = lane; t < nr; t += kWave) {
    const float4 v = sm.sres[t];
    lres[0] += exp2_fast(v.x - mres[0]);
    lres[1] += exp2_fast(v.y - mres[1]);
    lres[2] += exp2_fast(v.z - mres[2]);
    lres[3] += exp2_fast(v.w - mres[3]);
  }
#pragma unroll
  for (int h = 0; h < kHB; ++h) lres[h] = wave_sum_fast(lres[h]);
  // ---- values: channels 2 lane, 2 lane + 1; tokens wave, wave + 4, ...
  float a[kHB][2] = {};
  auto accumulate = [&](int t, uint32_t v) {
    const float v0 = h2f(v & 0xffffu), v1 = h2f(v >> 16);
    const float4 sv = sm.sres[t];
    const float pw[kHB] = {exp2_fast(sv.x - mres[0]), exp2_fast(sv.y - mres[1]),
                           exp2_fast(sv.z - mres[2]), exp2_fast(sv.w - mres[3])};
#pragma unroll
    for (int h = 0; h < kHB; ++h) {
      a[h][0] = fmaf(pw[h], v0, a[h][0]);
      a[h][1] = fmaf(pw[h], v1, a[h][1]);
    }
  };
#pragma unroll
  for (int i = 0; i < kVPre; ++i) {
    const int t = wave + kWaves * i;
    if (t < nr) accumulate(t, vpre[i]);
  }
  for (int t = wave + kWaves * kVPre; t < nr; t += kWaves)
    accumulate(t, vrow[static_cast<int64_t>(t) * (kD / 2) + lane]);
#pragma unroll
  for (int h = 0; h < kHB; ++h)
    *reinterpret_cast<float2*>(&sm.vpart[wave][h][2 * lane]) = make_float2(a[h][0], a[h][1]);
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int idx = tid + k * kThreads;
    const int h = idx / kD, c = idx % kD;   // h is uniform in a wave
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) acc += sm.vpart[w][h][c];
    float mh = mres[0], lh = lres[0];
#pragma unroll
    for (int kk = 1; kk < kHB; ++kk) {
      mh = h == kk ? mres[kk] : mh;
      lh = h == kk ? lres[kk] : lh;
    }
    if (h < nh) {
      float* dst = p.work + ((static_cast<int64_t>(b) * p.Hq + h0 + h) * (p.n_split + 1) + p.n_split) * kPartStride;
      dst[c] = acc;
      if (c == 0) {
        dst[128] = mh;
        dst[129] = lh;
      }
    }
  }
}

// DQ: meta holds one fp16 s2' per token, the shift arrays hold the group
// records of the double quantization (4-bit s1 and o', decoded on the fly:
// o' into <q', o'> at set-up and into the value shift at the end, s1 with
// each tile's metadata).
template <int M, int G, bool ROPE, bool DQ>
__global__ __launch_bounds__(kThreads, ROPE ? 2 : kBlocksPerCU) void attn_split_kernel(SplitParams p) {
  static_assert(!DQ || G == 128, "double quantization uses groups of 128");
  constexpr int CB = kD / M;            // code bytes per token
  constexpr int TPG = G / kTile;        // tiles per group
  constexpr int RB = 2 * kDqRecU16;     // record bytes
  __shared__ AttnSmem<M> smem;
  __shared__ std::conditional_t<ROPE, RopeSmem, NoRopeSmem> rsm;
  SplitSmem<M>& sm = smem.s;
  DqSmem& dsm = sm.dq;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int R = lane >> 4, c16 = lane & 15;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y / p.hblocks;
  const int hb = blockIdx.y - kvh * p.hblocks;
  const int b = blockIdx.z;
  const int h0 = kvh * p.grp + hb * kHB;
  const int nh = min(kHB, p.grp - hb * kHB);
  double theta = 0.0;   // rotary frequency of pair `lane`
  RopeSmem* rsp = nullptr;
  if constexpr (ROPE) {
    rsp = &rsm;
    theta = rope_theta(p.rope_base, lane);
    static_assert(kTile == kWave && kThreads % kWave == 0, "one table row per wave pass");
    for (int idx = tid; idx < (kD / 2) * kTile; idx += kThreads) {
      // i is the same in the whole wave: its frequency is lane i's theta
      const int i = idx / kTile, t = idx % kTile;
      rsm.tab[i][t] = rope_cs(static_cast<double>(t) * __shfl(theta, i, kWave));
    }
    for (int idx = tid; idx < kHB * kD; idx += kThreads) {
      const int h = idx / kD, c = idx % kD;
      rsm.q[h][c] = h < nh ? h2f(p.q[(static_cast<int64_t>(b) * p.Hq + h0 + h) * kD + c]) : 0.f;
    }
    __syncthreads();
  }
  if (split == (p.n_split > 0 ? p.n_split - 1 : 0)) {
    // the residual window first, in the workgroup of the last chunk (the
    // plan's shortest): its load latency overlaps the other workgroups' work
    // instead of ending the kernel
    resid_block<ROPE>(p, smem.r, rsp, theta, b, kvh, hb);
    if (p.n_split == 0) return;
    __syncthreads();   // the LDS is reused
  }
  const int c0 = split * p.chunk;
  const int c1 = min(p.n_quant, c0 + p.chunk);
  const int ntiles = (c1 - c0) / kTile;   // chunks hold whole groups, groups whole tiles
  const int ng = (c1 - c0) / G;
  const int64_t row = static_cast<int64_t>(b) * p.Hkv + kvh;  // (b, kv head) cache row
  const uint16_t* ksg = p.ks + (row * (p.cap / G) + c0 / G) * kD;
  const uint16_t* vsg = p.vs + (row * (p.cap / G) + c0 / G) * kD;
  const uint8_t* krec = reinterpret_cast<const uint8_t*>(p.ks + (row * (p.cap / G) + c0 / G) * kDqRecU16);
  const uint8_t* vrec = reinterpret_cast<const uint8_t*>(p.vs + (row * (p.cap / G) + c0 / G) * kDqRecU16);

  // ---- set-up: fp16 codebook, rotated queries (wave = head), zero weight slots
  {
    const uint32_t* cbg = reinterpret_cast<const uint32_t*>(p.table + kTabCodebookH);
    for (int i = tid; i < kCodes * M / 2; i += kThreads) sm.cbh[i] = cbg[i];
    float x0 = 0.f, x1 = 0.f;
    if (wave < nh) {
      const uint32_t qq =
          reinterpret_cast<const uint32_t*>(p.q + (static_cast<int64_t>(b) * p.Hq + h0 + wave) * kD)[lane];
      x0 = h2f(qq & 0xffffu);
      x1 = h2f(qq >> 16);
    }
    if (any_sign(p.sg)) {   // randomized rotation: D first
      const uint32_t wd = sign_word(p.sg, lane >> 4) >> (2 * (lane & 15));
      x0 = flip_sign(x0, (wd & 1u) << 31);
      x1 = flip_sign(x1, ((wd >> 1) & 1u) << 31);
    }
    // Walsh-Hadamard transform, channels 2 lane and 2 lane + 1 in this lane
    const float u0 = x0 + x1, u1 = x0 - x1;
    x0 = u0;
    x1 = u1;
#pragma unroll
    for (int e = 1; e < kWave; e <<= 1) {
      const float y0 = __shfl_xor(x0, e, kWave), y1 = __shfl_xor(x1, e, kWave);
      const bool up = (lane & e) != 0;
      x0 = up ? y0 - x0 : x0 + y0;
      x1 = up ? y1 - x1 : x1 + y1;
    }
    sm.qr[wave][2 * lane] = x0 * kInvSqrtD;
    sm.qr[wave][2 * lane + 1] = x1 * kInvSqrtD;
    *reinterpret_cast<u32x4*>(&sm.wrow[wave][lane][8]) = u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  // <q'_h, o'_g> for every group of the chunk, one thread per (g, h)
  if constexpr (DQ) {
    for (int idx = tid; idx < (ROPE ? 0 : ng * kHB); idx += kThreads) {
      const int g = idx / kHB, h = idx % kHB;
      const uint8_t* rec = krec + static_cast<int64_t>(g) * RB;
      const uint32_t* w32 = reinterpret_cast<const uint32_t*>(rec + 8);
      float s = 0.f;
#pragma unroll 4
      for (int i = 0; i < kD / 8; ++i) {
        const uint32_t w = w32[i];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int c = static_cast<int>((w >> (4 * k)) & 15u);
          s = fmaf(sm.qr[h][8 * i + k], c ? static_cast<float>(c - 8) : 0.f, s);
        }
      }
      sm.qo[g][h] = s * h2f(reinterpret_cast<const uint16_t*>(rec)[2]);
    }
    for (int g = tid; g < ng; g += kThreads) {
      const uint2 kh = *reinterpret_cast<const uint2*>(krec + static_cast<int64_t>(g) * RB);
      const uint2 vh = *reinterpret_cast<const uint2*>(vrec + static_cast<int64_t>(g) * RB);
      const float klo = h2f(kh.x & 0xffffu), khi = h2f(kh.x >> 16);
      const float vlo = h2f(vh.x & 0xffffu), vhi = h2f(vh.x >> 16);
      dsm.kls[g] = make_float2(klo, dq_step(klo, khi));
      dsm.vls[g] = make_float2(vlo, dq_step(vlo, vhi));
      dsm.vsc[g] = h2f(vh.y & 0xffffu);
    }
  }
  for (int idx = tid; idx < (ROPE || DQ ? 0 : ng * kHB); idx += kThreads) {
    const int g = idx / kHB, h = idx % kHB;
    const uint4* o = reinterpret_cast<const uint4*>(ksg + static_cast<int64_t>(g) * kD);
    float s = 0.f;
#pragma unroll 4
    for (int i = 0; i < kD / 8; ++i) {
      const uint4 w = o[i];
      const uint32_t uu[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        s = fmaf(sm.qr[h][8 * i + 2 * k], h2f(uu[k] & 0xffffu), s);
        s = fmaf(sm.qr[h][8 * i + 2 * k + 1], h2f(uu[k] >> 16), s);
      }
    }
    sm.qo[g][h] = s;
  }
  // score A operand per step s: row = slot c16 (0..3: fp16(q'_h), 4..7:
  // fp16(q'_h - fp16(q'_h)), the pair carries ~22 bits; 8..15: 0), K index
  // 8R + v = channel 32R + 8s + v
  u32x4 qa[4];
  if constexpr (!ROPE) {
    const int hq = c16 & 3;
    const bool is_hi = c16 < 4, is_lo = c16 >= 4 && c16 < 8;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t wv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t pk = 0;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float v = sm.qr[hq][32 * R + 8 * s + 2 * i + e];
          const uint16_t hi = f2h(v);
          const uint16_t lo = f2h(v - h2f(hi));
          const uint16_t val = is_hi ? hi : (is_lo ? lo : 0);
          pk |= static_cast<uint32_t>(val) << (16 * e);
        }
        wv[i] = pk;
      }
      qa[s] = u32x4{wv[0], wv[1], wv[2], wv[3]};
    }
  }
  __syncthreads();

  // ---- per-wave online softmax over the wave's tiles
  float m_run[kHB], l_lane[kHB];
#pragma unroll
  for (int h = 0; h < kHB; ++h) {
    m_run[h] = -__builtin_huge_valf();
    l_lane[h] = 0.f;
  }
  v4f acc[8];   // rows: channels 32R + 4cb + j; columns: weight slot c16
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) acc[cb] = v4f{0.f, 0.f, 0.f, 0.f};
  const int slot_head = c16 & 3;
  const float qscale = p.scale * kLog2e;
  const int a4 = lane & 3, k4 = (lane & 15) >> 2;

  const uint8_t* kcrow = p.kc + row * p.cap * CB + static_cast<int64_t>(c0) * CB;
  const uint8_t* vcrow = p.vc + row * p.cap * CB + static_cast<int64_t>(c0) * CB;
  const uint32_t* kmrow = reinterpret_cast<const uint32_t*>(p.km + row * p.cap * 2) + c0;
  const uint32_t* vmrow = reinterpret_cast<const uint32_t*>(p.vm + row * p.cap * 2) + c0;
  const uint16_t* kmrow16 = p.km + row * p.cap + c0;   // DQ: s2' per token
  const uint16_t* vmrow16 = p.vm + row * p.cap + c0;
  const uint32_t koff = c16 * CB + (M == 4 ? 8 : 4) * R;
  const uint32_t voff = (8 * R + k4) * CB + (M == 4 ? 8 : 4) * a4;
  const uint32_t cbh_base = lds_addr(sm.cbh);   // codebook copy of this lane
  const uint32_t wtr = lds_addr(&sm.wrow[wave][8 * R + k4][4 * a4]);

  TileData<M> d;
  // metadata of token `lane` of a tile: (s1, s2') fp16 pair, or with DQ
  // s2' in the low half and the 4-bit s1 code in bits 16..19
  auto lmeta = [&](int tile) {
    if constexpr (DQ) {
      const int t = tile * kTile + lane;
      const int64_t rb = static_cast<int64_t>(tile / TPG) * RB + 8 + kD / 2 + (t % G) / 2;
      const int sh = 4 * (t & 1);
      d.km = static_cast<uint32_t>(__builtin_nontemporal_load(kmrow16 + t)) | (((krec[rb] >> sh) & 15u) << 16);
      d.vm = static_cast<uint32_t>(__builtin_nontemporal_load(vmrow16 + t)) | (((vrec[rb] >> sh) & 15u) << 16);
    } else {
      load_meta<M>(d, kmrow + tile * kTile, vmrow + tile * kTile, lane);
    }
  };
  // (s1, s2') from a metadata word of tile `tile`'s group
  auto umeta = [&](uint32_t w, int tile, bool is_v, float& s1, float& s2) {
    if constexpr (DQ) {
      const float2 ls = is_v ? dsm.vls[tile / TPG] : dsm.kls[tile / TPG];
      s1 = dq_s1(w >> 16, ls.x, ls.y);
      s2 = h2f(w & 0xffffu);
    } else {
      s1 = h2f(w & 0xffffu);
      s2 = h2f(w >> 16);
    }
  };
  HOps ho{};
  // rotary path: key codes of keys t32 and 32 + t32 of the tile, and this
  // lane's word (channels 2 lane, 2 lane + 1) of the tile's group shift,
  // fetched one tile ahead
  u32x4 kpre[2][CB / 16];
  uint32_t opre = 0;
  auto load_rope = [&](int tile) {
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int i = 0; i < CB / 16; ++i)
        kpre[ht][i] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(kcrow + (tile * kTile + 32 * ht + (lane & 31)) * CB) + i);
    if constexpr (DQ) {
      const uint8_t* rec = krec + static_cast<int64_t>(tile / TPG) * RB;
      opre = static_cast<uint32_t>(rec[8 + lane]) | (static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(rec)[2]) << 16);
    } else {
      opre = reinterpret_cast<const uint32_t*>(ksg + static_cast<int64_t>(tile / TPG) * kD)[lane];
    }
  };
  if constexpr (ROPE) ho = hadamard_ops(lane);
  for (int tau = wave; tau < ntiles; tau += kWaves) {
    const int tn = tau + kWaves;
    const bool more = tn < ntiles;
    if (tau == wave) {
      if constexpr (ROPE)
        load_rope(tau);
      else
        load_keys<M>(d, kcrow + tau * kTile * CB, koff);
      lmeta(tau);
      load_values<M>(d, vcrow + tau * kTile * CB, voff);
    }
    float s[kHB];
    float s1v, s2v;
    if constexpr (ROPE) {
      // the tile's group shift in the original domain, (H / sqrt(d)) o'_g,
      // lane holding channels 2 lane, 2 lane + 1; the queries turned to the
      // tile's first position
      {
        float x0, x1;
        if constexpr (DQ) {
          // the o' code byte of channels 2 lane, 2 lane + 1 and the record's scale
          const float osc = h2f(opre >> 16);
          x0 = dq_nibble_o(opre & 0xffu, 0, osc);
          x1 = dq_nibble_o(opre & 0xffu, 1, osc);
        } else {
          x0 = h2f(opre & 0xffffu);
          x1 = h2f(opre >> 16);
        }
        const float u0 = x0 + x1, u1 = x0 - x1;
        x0 = u0;
        x1 = u1;
#pragma unroll
        for (int e = 1; e < kWave; e <<= 1) {
          const float y0 = __shfl_xor(x0, e, kWave), y1 = __shfl_xor(x1, e, kWave);
          const bool up = (lane & e) != 0;
          x0 = up ? y0 - x0 : x0 + y0;
          x1 = up ? y1 - x1 : x1 + y1;
        }
        *reinterpret_cast<float2*>(&rsm.og[wave][2 * lane]) = make_float2(x0 * kInvSqrtD, x1 * kInvSqrtD);
      }
      rope_query(rsm, rsm.qp[wave], lane, theta, p.q_pos - (static_cast<int64_t>(c0) + tau * kTile));
      wave_lds_sync();
      // The turned queries as the A operand of v_mfma_f32_32x32x16_f16 for
      // the key dot products: row l % 32 = slot (0..3: fp16 high part of
      // head 0..3, 4..7: low part); K slice s = 4pm + q holds channels
      // 32pm + 8q + [0, 8) and those + 64, lane half hA supplying K = 8hA + v:
      // v < 4 channel 32pm + 8q + 4hA + v, v >= 4 the same channel + 64 (the
      // key operand below uses the same order).  Kept in LDS (registers are
      // the limit here); lanes of rows 8..31 read a copy of row l % 8, whose
      // output rows are never used.  The 128 entries (8 rows x 8 slices x 2
      // lane halves) are made by the whole wave, two per lane: lane l takes
      // row l % 8, half (l / 8) % 2 and slices l / 16 and l / 16 + 4.
      {
        const int row = lane & 7, hA = (lane >> 3) & 1, sp = lane >> 4;
        const int hq = row & 3;
        const bool lo_part = row >= 4;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int sl = sp + 4 * j;
          const int c = 32 * (sl >> 2) + 8 * (sl & 3) + 4 * hA;
          const float4 u = *reinterpret_cast<const float4*>(&rsm.qp[wave][hq][c]);
          const float4 v = *reinterpret_cast<const float4*>(&rsm.qp[wave][hq][c + kD / 2]);
          uint32_t w4[4] = {f16_hi2(u.x, u.y), f16_hi2(u.z, u.w), f16_hi2(v.x, v.y), f16_hi2(v.z, v.w)};
          const uint32_t l4[4] = {f16_lo2(u.x, u.y, w4[0]), f16_lo2(u.z, u.w, w4[1]),
                                  f16_lo2(v.x, v.y, w4[2]), f16_lo2(v.z, v.w, w4[3])};
#pragma unroll
          for (int i = 0; i < 4; ++i) w4[i] = lo_part ? l4[i] : w4[i];
          rsm.qkl[wave][sl][hA][row] = u32x4{w4[0], w4[1], w4[2], w4[3]};
        }
        wave_lds_sync();
      }
      // Two halves of 32 keys.  The MFMA token-major pass gives lane
      // (t32, hf) the channels {32mb + 8(r/4) + 4hf + r%4} of key 32ht + t32:
      // both members of every rotary pair (c, c + 64) sit in one lane.
      const int t32 = lane & 31, hf = lane >> 5;
      // (scheduling fences around the two halves and the two row-block pairs
      // keep their registers from overlapping; without them the kernel spills)
      __builtin_amdgcn_sched_barrier(0);
      float sh[kHB];   // key 32 hf + t32 ends up in this lane: half ht == hf keeps its sums
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        const int tok = 32 * ht + t32;   // key of the tile
        u32x4 xv[8];   // channels 16kb + 8hf .. + 7 of the key, codewords (fp16, exact)
        if constexpr (M == 4) {
          const u32x4 w0 = kpre[ht][0];
          const u32x4 w1 = kpre[ht][CB / 16 - 1];
          const uint32_t ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
          for (int kb = 0; kb < 8; ++kb) {
            // sub-vectors 4kb + 2hf and + 1: bytes 2hf, 2hf + 1 of word kb
            const uint32_t wq = ww[kb] >> (16 * hf);
            const uint32_t c0i = wq & 0xffu, c1i = (wq >> 8) & 0xffu;
            const u32x2 a0 = *reinterpret_cast<const u32x2*>(&sm.cbh[2 * c0i]);
            const u32x2 a1 = *reinterpret_cast<const u32x2*>(&sm.cbh[2 * c1i]);
            xv[kb] = u32x4{a0.x, a0.y, a1.x, a1.y};
          }
        } else {
          const u32x4 w0 = kpre[ht][0];
          const uint32_t ww[4] = {w0.x, w0.y, w0.z, w0.w};
#pragma unroll
          for (int kb = 0; kb < 8; ++kb) {
            // sub-vector 2kb + hf: byte 2(kb % 2) + hf of word kb / 2
            const uint32_t ci = (ww[kb >> 1] >> (8 * (2 * (kb & 1) + hf))) & 0xffu;
            xv[kb] = *reinterpret_cast<const u32x4*>(&sm.cbh[4 * ci]);
          }
        }
        // k = s1 (s2' H c / sqrt(d) + og), turned by the key's offset (s1
        // applied to the score); row blocks (pm, pm + 2) hold the pairs
        // (c, c + 64) of channels 32pm ..  The turned key, split into fp16
        // high and low parts, is the B operand (K = this lane's channels,
        // N = its key) of the dot products with the queries: rows 0..3 of
        // the result (lane half 0) and 4..7 (half 1) are the high and low
        // query parts of heads 0..3.
        const uint32_t kmt = __shfl(d.km, tok, kWave);
        float s1k, s2k;
        umeta(kmt, tau, false, s1k, s2k);
        const float a = s2k * kInvSqrtD;
        v16f dq = v16f{};
#pragma unroll
        for (int pm = 0; pm < 2; ++pm) {
          v16f hx = v16f{}, hy = v16f{};
#pragma unroll
          for (int kb = 0; kb < 8; ++kb) {
            hx = __builtin_amdgcn_mfma_f32_32x32x16_f16(hblk(ho, pm, kb), __builtin_bit_cast(v8h, xv[kb]), hx, 0, 0, 0);
            hy = __builtin_amdgcn_mfma_f32_32x32x16_f16(hblk(ho, pm + 2, kb), __builtin_bit_cast(v8h, xv[kb]), hy, 0, 0, 0);
          }
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int cb0 = 32 * pm + 8 * g4 + 4 * hf;   // channels cb0 .. cb0 + 3 and + 64
            const float4 ox = *reinterpret_cast<const float4*>(&rsm.og[wave][cb0]);
            const float4 oy = *reinterpret_cast<const float4*>(&rsm.og[wave][cb0 + kD / 2]);
            const float oxv[4] = {ox.x, ox.y, ox.z, ox.w}, oyv[4] = {oy.x, oy.y, oy.z, oy.w};
            float kx[4], ky[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * g4 + e;
              const float2 cs = rsm.tab[cb0 + e][tok];
              const float x = fmaf(a, hx[r], oxv[e]);
              const float y = fmaf(a, hy[r], oyv[e]);
              kx[e] = x * cs.x - y * cs.y;
              ky[e] = y * cs.x + x * cs.y;
            }
            const uint32_t h0 = f16_hi2(kx[0], kx[1]), h1 = f16_hi2(kx[2], kx[3]);
            const uint32_t h2 = f16_hi2(ky[0], ky[1]), h3 = f16_hi2(ky[2], ky[3]);
            const u32x4 bh = u32x4{h0, h1, h2, h3};
            const u32x4 bl = u32x4{f16_lo2(kx[0], kx[1], h0), f16_lo2(kx[2], kx[3], h1),
                                   f16_lo2(ky[0], ky[1], h2), f16_lo2(ky[2], ky[3], h3)};
            const v8h qa = __builtin_bit_cast(v8h, rsm.qkl[wave][4 * pm + g4][hf][lane & 7]);
            dq = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa, __builtin_bit_cast(v8h, bh), dq, 0, 0, 0);
            dq = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa, __builtin_bit_cast(v8h, bl), dq, 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int h = 0; h < kHB; ++h) {
          const float v = half_pair_sum(dq[h]) * s1k;
          sh[h] = ht == hf ? v : sh[h];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int h = 0; h < kHB; ++h) s[h] = sh[h] * qscale;
      if (more) load_rope(tn);
      umeta(d.vm, tau, true, s1v, s2v);
      if (more) lmeta(tn);
    } else {
    // -- scores
    v4f sacc[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      sacc[tb] = v4f{0.f, 0.f, 0.f, 0.f};
      score_steps<M, 0>(sacc[tb], qa, d.kc[tb], sm.cbh);
    }
    if (more) load_keys<M>(d, kcrow + tn * kTile * CB, koff);
    // rows 0..3 (lanes 0..15) hold high-part scores of heads 0..3, rows 4..7
    // (lanes 16..31) low-part ones; swap so that lane l holds token l
    float dot[kHB];
#pragma unroll
    for (int j = 0; j < kHB; ++j) {
      const auto r01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(sacc[0][j]),
                                                        __float_as_uint(sacc[1][j]), false, false);
      const auto r23 = __builtin_amdgcn_permlane16_swap(__float_as_uint(sacc[2][j]),
                                                        __float_as_uint(sacc[3][j]), false, false);
      const float t01 = __uint_as_float(r01[0]) + __uint_as_float(r01[1]);
      const float t23 = __uint_as_float(r23[0]) + __uint_as_float(r23[1]);
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(t01), __float_as_uint(t23), false, false);
      dot[j] = __uint_as_float(r[0]);
    }
    const int g = tau / TPG;
    const float4 qo4 = *reinterpret_cast<const float4*>(&sm.qo[g][0]);
    const float qov[kHB] = {qo4.x, qo4.y, qo4.z, qo4.w};
    float s1k, s2k;
    umeta(d.km, tau, false, s1k, s2k);
    umeta(d.vm, tau, true, s1v, s2v);
    if (more) lmeta(tn);
    const float ks = qscale * s1k;
#pragma unroll
    for (int h = 0; h < kHB; ++h) s[h] = ks * fmaf(s2k, dot[h], qov[h]);
    }
    // -- running max, raised only when a score exceeds it.  From here to the
    //    end of the value phase the wave runs at raised issue priority, so a
    //    wave that holds its scores finishes the tile while the others gather
    //    codewords for theirs (measured 2-3.5 % faster than one priority;
    //    the rotary kernel, whose score phase dominates, keeps one).
    if constexpr (!ROPE) __builtin_amdgcn_s_setprio(1);
    bool raised = false;
    float fl = 1.f;
#pragma unroll
    for (int h = 0; h < kHB; ++h) {
      if (__ballot(s[h] > m_run[h])) {
        const float mn = fmaxf(m_run[h], wave_max_fast(s[h]));
        const float f = exp2_fast(m_run[h] - mn);
        m_run[h] = mn;
        l_lane[h] *= f;
        fl = slot_head == h ? f : fl;
        raised = true;
      }
    }
    if (raised) {
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) acc[cb] *= fl;
    }
    // -- weights: p s1 s2' as fp16 high + low parts into the wave's rows;
    //    p s1 per head summed over the tile for the shift term
    float sp[kHB];
    uint32_t wk[4];
#pragma unroll
    for (int h = 0; h < kHB; ++h) {
      const float pw = exp2_fast(s[h] - m_run[h]);
      l_lane[h] += pw;
      sp[h] = pw * s1v;
      const float w = sp[h] * s2v;
      const _Float16 hi = static_cast<_Float16>(w);
      const _Float16 lo = static_cast<_Float16>(w - static_cast<float>(hi));
      const uint32_t hb16 = __builtin_bit_cast(uint16_t, hi), lb16 = __builtin_bit_cast(uint16_t, lo);
      if (h & 1) {
        wk[h >> 1] |= hb16 << 16;
        wk[2 + (h >> 1)] |= lb16 << 16;
      } else {
        wk[h >> 1] = hb16;
        wk[2 + (h >> 1)] = lb16;
      }
    }
    *reinterpret_cast<u32x4*>(&sm.wrow[wave][lane][0]) = u32x4{wk[0], wk[1], wk[2], wk[3]};
    {
      // four wave sums at once: halves, then rows, then within rows; row R
      // ends with head (0, 2, 1, 3)[R]
      const auto x01 = __builtin_amdgcn_permlane32_swap(__float_as_uint(sp[0]), __float_as_uint(sp[1]), false, false);
      const auto x23 = __builtin_amdgcn_permlane32_swap(__float_as_uint(sp[2]), __float_as_uint(sp[3]), false, false);
      const float u = __uint_as_float(x01[0]) + __uint_as_float(x01[1]);
      const float w = __uint_as_float(x23[0]) + __uint_as_float(x23[1]);
      const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(u), __float_as_uint(w), false, false);
      float z = __uint_as_float(y[0]) + __uint_as_float(y[1]);
      auto dpp = [](float v, auto ctrl_c) {
        constexpr int ctrl = decltype(ctrl_c)::value;
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xf, 0xf, false));
      };
      z += dpp(z, std::integral_constant<int, 0xB1>{});
      z += dpp(z, std::integral_constant<int, 0x4E>{});
      z += dpp(z, std::integral_constant<int, 0x124>{});
      z += dpp(z, std::integral_constant<int, 0x128>{});
      if (c16 == 0) sm.ssum[tau][((R & 1) << 1) | (R >> 1)] = z;
      if (lane == 0) *reinterpret_cast<float4*>(&sm.smax[tau][0]) = make_float4(m_run[0], m_run[1], m_run[2], m_run[3]);
    }
    wave_lds_sync();
    // -- values: acc[cb] += C^T (32 channels x 32 tokens) W (32 tokens x 16 slots)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint2 w0 = ds_tr16(wtr + (32 * kb) * 32);
      const uint2 w1 = ds_tr16(wtr + (32 * kb + 4) * 32);
      const u32x4 bw = u32x4{w0.x, w0.y, w1.x, w1.y};
      value_steps<M, 0, !ROPE>(acc, d, kb, bw, cbh_base);
    }
    if constexpr (!ROPE) __builtin_amdgcn_s_setprio(0);
    if (more) load_values<M>(d, vcrow + tn * kTile * CB, voff);
    wave_lds_sync();
  }

  // ---- merge: high + low slots (lanes c16 = 4..7 end with the sum), waves
  float* wacc = reinterpret_cast<float*>(&sm.wrow[wave][0][0]);   // [kHB][kD]
#pragma unroll
  for (int cb = 0; cb < 8; ++cb)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[cb][j] += dpp_row_shr4(acc[cb][j]);
  wave_lds_sync();
  if (c16 >= 4 && c16 < 8) {
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
      *reinterpret_cast<v4f*>(&wacc[(c16 - 4) * kD + 32 * R + 4 * cb]) = acc[cb];
  }
  float lsum[kHB];
#pragma unroll
  for (int h = 0; h < kHB; ++h) lsum[h] = wave_sum_fast(l_lane[h]);
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < kHB; ++h) {
      sm.wm[wave][h] = m_run[h];
      sm.wl[wave][h] = lsum[h];
    }
  }
  __syncthreads();
  float Mh[kHB];
#pragma unroll
  for (int h = 0; h < kHB; ++h) {
    float mx = sm.wm[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, sm.wm[w][h]);
    Mh[h] = mx;
  }
  for (int idx = tid; idx < ng * kHB; idx += kThreads) {
    const int g = idx / kHB, h = idx % kHB;
    float mh = Mh[0];
#pragma unroll
    for (int k = 1; k < kHB; ++k) mh = h == k ? Mh[k] : mh;
    float S = 0.f;
#pragma unroll
    for (int t = 0; t < TPG; ++t) {
      S = fmaf(sm.ssum[g * TPG + t][h], exp2_fast(sm.smax[g * TPG + t][h] - mh), S);
    }
    sm.sg[g][h] = S;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int idx = tid + k * kThreads;
    const int h = idx / kD, c = idx % kD;   // h is uniform in a wave
    float mh = Mh[0];
#pragma unroll
    for (int kk = 1; kk < kHB; ++kk) mh = h == kk ? Mh[kk] : mh;
    float a = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm.wm[w][h];
      const float e = mw == -__builtin_huge_valf() ? 0.f : exp2_fast(mw - mh);
      a = fmaf(e, reinterpret_cast<const float*>(&sm.wrow[w][0][0])[h * kD + c], a);
      l = fmaf(e, sm.wl[w][h], l);
    }
    if constexpr (DQ) {
#pragma unroll 8
      for (int g = 0; g < ng; ++g)
        a = fmaf(sm.sg[g][h], dq_nibble_o(vrec[static_cast<int64_t>(g) * RB + 8 + c / 2], c & 1, dsm.vsc[g]), a);
    } else {
#pragma unroll 8
      for (int g = 0; g < ng; ++g) a = fmaf(sm.sg[g][h], h2f(vsg[static_cast<int64_t>(g) * kD + c]), a);
    }
    if (h < nh) {
      float* dst = p.work + ((static_cast<int64_t>(b) * p.Hq + h0 + h) * (p.n_split + 1) + split) * kPartStride;
      dst[c] = a;
      if (c == 0) {
        dst[128] = mh;
        dst[129] = l;
      }
    }
  }
}

struct CombineParams {
  const float* work;
  float* out;
  int Hq, n_split;
  Signs sg;   // randomized rotation: the inverse ends with D
};

constexpr int kCombThreads = 256;

// One wave per (batch, query head): lane holds rotated channels 2 lane and
// 2 lane + 1.
__global__ __launch_bounds__(kCombThreads) void attn_combine_kernel(CombineParams p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int hq = blockIdx.x * (kCombThreads / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (hq >= p.Hq) return;
  const int64_t gh = static_cast<int64_t>(blockIdx.y) * p.Hq + hq;
  const float* part = p.work + gh * (p.n_split + 1) * kPartStride;
  const float ninf = -__builtin_huge_valf();
  float M = ninf;
  for (int i = 0; i <= p.n_split; ++i) M = fmaxf(M, part[i * kPartStride + 128]);
  float a0 = 0.f, a1 = 0.f, L = 0.f;
  for (int i = 0; i < p.n_split; ++i) {
    const float* pi = part + i * kPartStride;
    const float mi = pi[128];
    const float e = mi == ninf ? 0.f : exp2_fast(mi - M);
    L = fmaf(e, pi[129], L);
    const float2 v = reinterpret_cast<const float2*>(pi)[lane];
    a0 = fmaf(e, v.x, a0);
    a1 = fmaf(e, v.y, a1);
  }
  // inverse rotation (the transform is its own inverse up to 1/sqrt(d))
  {
    const float u0 = a0 + a1, u1 = a0 - a1;
    a0 = u0;
    a1 = u1;
#pragma unroll
    for (int e = 1; e < kWave; e <<= 1) {
      const float y0 = __shfl_xor(a0, e, kWave), y1 = __shfl_xor(a1, e, kWave);
      const bool up = (lane & e) != 0;
      a0 = up ? y0 - a0 : a0 + y0;
      a1 = up ? y1 - a1 : a1 + y1;
    }
    if (any_sign(p.sg)) {
      const uint32_t wd = sign_word(p.sg, lane >> 4) >> (2 * (lane & 15));
      a0 = flip_sign(a0, (wd & 1u) << 31);
      a1 = flip_sign(a1, ((wd >> 1) & 1u) << 31);
    }
  }
  const float* pr = part + p.n_split * kPartStride;
  const float mr = pr[128];
  const float er = mr == ninf ? 0.f : exp2_fast(mr - M);
  L = fmaf(er, pr[129], L);
  const float2 rv = reinterpret_cast<const float2*>(pr)[lane];
  const float inv = 1.f / L;
  float2 o;
  o.x = fmaf(a0, kInvSqrtD, er * rv.x) * inv;
  o.y = fmaf(a1, kInvSqrtD, er * rv.y) * inv;
  reinterpret_cast<float2*>(p.out + gh * kD)[lane] = o;
}

template <int M, int G>
hipError_t split_launch(const AttnArgs& a, const SplitParams& sp, hipStream_t s) {
  dim3 grid(a.n_split > 0 ? a.n_split : 1, a.Hkv * sp.hblocks, a.B);
  if constexpr (G == 128) {
    if (a.rope && a.dq) {
      hipLaunchKernelGGL((attn_split_kernel<M, G, true, true>), grid, dim3(kThreads), 0, s, sp);
      return hipGetLastError();
    }
  }
  if (a.dq && G != 128) return hipErrorInvalidValue;
  if (a.rope)
    hipLaunchKernelGGL((attn_split_kernel<M, G, true, false>), grid, dim3(kThreads), 0, s, sp);
  else if constexpr (G == 128) {
    if (a.dq)
      hipLaunchKernelGGL((attn_split_kernel<M, G, false, true>), grid, dim3(kThreads), 0, s, sp);
    else
      hipLaunchKernelGGL((attn_split_kernel<M, G, false, false>), grid, dim3(kThreads), 0, s, sp);
  } else {
    if (a.dq) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_split_kernel<M, G, false, false>), grid, dim3(kThreads), 0, s, sp);
  }
  return hipGetLastError();
}

}  // namespace

void attn_plan(int B, int Hq, int Hkv, int n_quant, int n_resid, int group_size, int rope,
               int* n_split, int* chunk) {
  if (n_quant <= 0) {
    *n_split = 0;
    *chunk = 0;
    return;
  }
  const int grp = Hq / Hkv;
  const int64_t units = static_cast<int64_t>(B) * Hkv * ((grp + kHB - 1) / kHB);
  // about three workgroups per CU in one round: every CU equally busy, with
  // room left for one more workgroup per CU while the others finish
  const int64_t slots = static_cast<int64_t>(kPlanCUs) * (rope ? kPlanBlocksPerCURope : kPlanBlocksPerCU);
  int64_t want = slots / units;
  const int64_t max_split = (n_quant + kMinChunk - 1) / kMinChunk;
  if (want > max_split) want = max_split;
  if (want < 1) want = 1;
  // The last chunk's workgroup also takes the residual window: count each
  // residual token as kResidWeight quantized ones (its K and V are 512 fp16
  // bytes against 72 of 2-bit codes and metadata; a 1-bit token takes the
  // time of a 2-bit one, its codeword gathers being the same size), so that
  // the chunks come out larger and the last one short by about that much.
  const int64_t work = n_quant + static_cast<int64_t>(n_resid) * kResidWeight;
  int64_t c = (work + want - 1) / want;
  c = (c + group_size - 1) / group_size * group_size;
  if (c > kMaxChunk) c = kMaxChunk;
  *chunk = static_cast<int>(c);
  *n_split = static_cast<int>((n_quant + c - 1) / c);
}

int attn_split_bound(int B, int Hq, int Hkv, int n_quant) {
  // attn_plan's count is at most want <= min(slots / units, ceil(n /
  // kMinChunk)) (taken at least 1), unless the chunk is capped at kMaxChunk,
  // when it is ceil(n / kMaxChunk).  Both terms grow with n, and the plain
  // plan has the most slots, so this bounds every plan (plain or rotary) for
  // every count up to n_quant -- unlike the plan itself, whose rounding of
  // the chunk to whole groups can need more partials at a smaller count.
  if (n_quant <= 0) return 0;
  const int grp = Hq / Hkv;
  const int64_t units = static_cast<int64_t>(B) * Hkv * ((grp + kHB - 1) / kHB);
  const int64_t slots = static_cast<int64_t>(kPlanCUs) * kPlanBlocksPerCU;
  int64_t w = slots / units;
  if (w < 1) w = 1;
  const int64_t by_min = (n_quant + kMinChunk - 1) / kMinChunk;
  if (w > by_min) w = by_min;
  const int64_t by_max = (n_quant + kMaxChunk - 1) / kMaxChunk;
  return static_cast<int>(w > by_max ? w : by_max);
}

size_t attn_workspace_bytes(int B, int Hq, int n_split) {
  return static_cast<size_t>(B) * Hq * (n_split + 1) * kPartStride * sizeof(float);
}

hipError_t launch_decode_attention(const AttnArgs& a, hipStream_t s) {
  const int grp = a.Hq / a.Hkv;
  const int hblocks = (grp + kHB - 1) / kHB;
  SplitParams sp{a.q,     a.kc,       a.vc,    a.km,      a.vm,      a.ks,    a.vs,
                 a.kr,    a.vr,       static_cast<const uint8_t*>(a.table), a.work,
                 a.Hq,    a.Hkv,      grp,     hblocks,   a.n_quant, a.n_split, a.chunk,
                 a.n_resid, a.cap,    a.rcap,  a.scale,   a.q_pos,   a.rope_base, a.rht};
  hipError_t e;
  if (a.sub_dim == 4)
    e = a.group_size == 128 ? split_launch<4, 128>(a, sp, s) : split_launch<4, 256>(a, sp, s);
  else
    e = a.group_size == 128 ? split_launch<8, 128>(a, sp, s) : split_launch<8, 256>(a, sp, s);
  if (e != hipSuccess) return e;
  CombineParams cp{a.work, a.out, a.Hq, a.n_split, a.rht};
  const int per_block = kCombThreads / kWave;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((a.Hq + per_block - 1) / per_block, a.B),
                     dim3(kCombThreads), 0, s, cp);
  return hipGetLastError();
}

int attn_max_resid() { return kMaxResid; }

}  // namespace nsn
