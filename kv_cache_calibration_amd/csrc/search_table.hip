// Certified candidate tables for the exact nearest-codeword search of 4-d
// sub-vectors (2-bit codes).
// [NSNQuant summary (gist.science), Methodology §3: every rotated sub-vector
//  is replaced by its nearest codeword in one global codebook built for
//  N(0,1) data.]
//
// The space [-4.5, 4.5)^4 is cut into 24^4 boxes whose edges are the N(0,1)
// quantiles k/24 (rounded to multiples of 9/1024, so a 1024-entry table maps
// a coordinate to its bin exactly).  For every box the table lists each
// codeword c that is not *dominated*: c is dropped only if some c' is
// strictly closer than c at every point of the box, i.e. if
//   min over the box of  ||x - c||^2 - ||x - c'||^2
//     = sum_d min(2 lo_d (c'_d - c_d), 2 hi_d (c'_d - c_d)) + ||c||^2 - ||c'||^2  > 0.
// The test runs in float64 on the box widened by one fine cell on each side
// (covers the rounding of the bin computation), so the true nearest codeword
// of any point of the box -- including every lowest-index tie -- is always
// in its list.  Points outside the grid take a full scan.
//
// Per box: one u64 of eight candidate codes (encoding in nsn_device.h):
// up to four ascending; five to eight split in two halves whose byte order
// flags the overflow; more than eight (rare, far tails) tells the search to
// scan all codes.
#include <cmath>

#include "nsn_device.h"
#include "nsn_launch.h"

namespace nsn {

namespace {

struct Edges {
  float e[kNB + 1];
};

// Inverse N(0,1) CDF by bisection on erfc (host, once per prepare call).
double norm_ppf(double p) {
  double lo = -10.0, hi = 10.0;
  for (int it = 0; it < 200; ++it) {
    const double mid = 0.5 * (lo + hi);
    const double cdf = 0.5 * std::erfc(-mid / std::sqrt(2.0));
    if (cdf < p) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

Edges make_edges() {
  Edges E;
  E.e[0] = kGridLo;
  E.e[kNB] = -kGridLo;
  for (int k = 1; k < kNB; ++k) {
    const double q = norm_ppf(static_cast<double>(k) / kNB);
    const double f = std::nearbyint((q - kGridLo) / kFineW);
    E.e[k] = static_cast<float>(kGridLo + f * static_cast<double>(kFineW));
  }
  return E;
}

__global__ void tab_init_kernel(Edges E, uint8_t* __restrict__ table) {
  const int f = blockIdx.x * blockDim.x + threadIdx.x;
  if (f < kFine) {
    const float x = kGridLo + f * kFineW;   // left end of fine cell f (exact)
    int b = 0;
    for (int k = 1; k < kNB; ++k) b += (E.e[k] <= x) ? 1 : 0;
    table[kTabBinLut + f] = static_cast<uint8_t>(b);
  }
  if (f <= kNB) reinterpret_cast<float*>(table + kTabEdges)[f] = E.e[f];
}

// One block per box, one thread per codeword: is codeword `c` dominated?
__device__ bool alive_in_box(const double (*cw)[4], const double* n2, int c, const double* lo,
                             const double* hi) {
  for (int k = 0; k < kCodes; ++k) {
    double m = n2[c] - n2[k];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const double dl = cw[k][d] - cw[c][d];
      m += fmin(2.0 * lo[d] * dl, 2.0 * hi[d] * dl);
    }
    if (m > 1e-9) return false;
  }
  return true;
}

__device__ void box_of(int cell, const float* edges, double* lo, double* hi) {
  int r = cell;
  for (int d = 3; d >= 0; --d) {
    const int b = r % kNB;
    r /= kNB;
    lo[d] = static_cast<double>(edges[b]) - kFineW;
    hi[d] = static_cast<double>(edges[b + 1]) + kFineW;
  }
}

__device__ void load_codebook64(const uint8_t* table, double (*cw)[4], double* n2) {
  const float* cb = reinterpret_cast<const float*>(table + kTabCodebook);
  const int t = threadIdx.x;
  double s = 0.0;
  for (int d = 0; d < 4; ++d) {
    cw[t][d] = cb[t * 4 + d];
    s += cw[t][d] * cw[t][d];
  }
  n2[t] = s;
}

__global__ __launch_bounds__(256) void tab_write_kernel(uint8_t* __restrict__ table) {
  __shared__ double cw[kCodes][4];
  __shared__ double n2[kCodes];
  __shared__ uint32_t wave_cnt[kCodes / kWave];
  __shared__ uint8_t list[kCodes];
  const int cell = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  load_codebook64(table, cw, n2);
  __syncthreads();
  double lo[4], hi[4];
  box_of(cell, reinterpret_cast<const float*>(table + kTabEdges), lo, hi);
  const bool a = alive_in_box(cw, n2, t, lo, hi);
  const uint64_t bal = __ballot(a);
  if (lane == 0) wave_cnt[wave] = static_cast<uint32_t>(__popcll(bal));
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < wave; ++w) base += wave_cnt[w];
  const uint32_t rank = base + static_cast<uint32_t>(__popcll(bal & ((uint64_t(1) << lane) - 1)));
  if (a) list[rank] = static_cast<uint8_t>(t);
  __syncthreads();
  if (t == 0) {
    const uint32_t n = wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
    uint64_t w = 0;
    if (n <= 4) {
      for (int i = 0; i < 4; ++i) {
        const uint64_t c = list[min<uint32_t>(i, n - 1)];
        w |= c << (8 * i);
        w |= c << (8 * (i + 4));
      }
    } else {
      for (int i = 0; i < 4; ++i) w |= static_cast<uint64_t>(list[3 - i]) << (8 * i);
      if (n <= 8) {
        for (int i = 0; i < 4; ++i) w |= static_cast<uint64_t>(list[min<uint32_t>(4 + i, n - 1)]) << (8 * (i + 4));
      } else {
        for (int i = 0; i < 4; ++i) w |= static_cast<uint64_t>(list[7 - i]) << (8 * (i + 4));
      }
    }
    reinterpret_cast<uint64_t*>(table + kTabMain)[cell] = w;
  }
}

// Stand-alone nearest codeword of arbitrary sub-vectors (one thread each),
// using the same tables and the same lexicographic (distance, code) key.
// m = 4: a sub-vector in a crowded or off-grid cell is scanned over all 256
// codes by the whole wave (four codes per lane, then the wave minimum), as
// the quantizers do; m = 8 scans per lane.
template <int M>
__global__ __launch_bounds__(256) void nearest_kernel(const uint8_t* __restrict__ table,
                                                      const float* __restrict__ v, int64_t n,
                                                      uint8_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) float cb[kCodes * M];
  const float* cbg = reinterpret_cast<const float*>(table + kTabCodebook);
  for (int i = threadIdx.x; i < kCodes * M; i += 256) cb[i] = cbg[i];
  __syncthreads();
  const int64_t id = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const bool valid = id < n;   // lanes past the end still join the wave scans
  float h[M];
#pragma unroll
  for (int e = 0; e < M; ++e) h[e] = valid ? v[id * M + e] : 0.f;
  uint64_t best = ~uint64_t(0);
  auto dist = [&](const float (&x)[M], uint32_t k) {
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < M; ++e) {
      const float t = x[e] - cb[k * M + e];
      d = (e == 0) ? t * t : fmaf(t, t, d);
    }
    return d;
  };
  auto eval = [&](uint32_t k) {
    const uint64_t key = (static_cast<uint64_t>(__float_as_uint(dist(h, k))) << 32) | k;
    best = key < best ? key : best;
  };
  if constexpr (M == 4) {
    int cell = 0;
    bool off = false;
    for (int e = 0; e < 4; ++e) {
      const float fe = floorf(fmaf(h[e], kFineInv, 512.0f));
      off |= !(fe >= 0.f && fe < static_cast<float>(kFine));
      cell = cell * kNB + (off ? 0 : table[kTabBinLut + static_cast<int>(fe)]);
    }
    cell = min(cell, kCells - 1);   // in bounds even for an unprepared table
    bool brute = true;
    if (!off) {
      const uint64_t wv = reinterpret_cast<const uint64_t*>(table + kTabMain)[cell];
      brute = cand_more_than_8(wv);
      if (!brute) {
        for (int i = 0; i < 4; ++i) eval(static_cast<uint32_t>(wv >> (8 * i)) & 0xffu);
        if (cand_more_than_4(wv))
          for (int i = 4; i < 8; ++i) eval(static_cast<uint32_t>(wv >> (8 * i)) & 0xffu);
      }
    }
    const int lane = threadIdx.x & (kWave - 1);
    uint64_t need = __ballot(valid && brute);
    while (need) {
      const int l = __builtin_ctzll(need);
      need &= need - 1;
      float hb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) hb[e] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(h[e]), l));
      uint32_t dk = 0xffffffffu, ck = 0xffffffffu;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t k = static_cast<uint32_t>(lane + kWave * r);
        const uint32_t db = __float_as_uint(dist(hb, k));
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
  } else {
    for (uint32_t k = 0; k < kCodes; ++k) eval(k);
  }
  if (valid) out[id] = static_cast<uint8_t>(best & 0xffu);
}

}  // namespace

hipError_t launch_nearest(const void* table, int sub_dim, const float* v, int64_t n, uint8_t* out,
                          hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
  const uint8_t* t = static_cast<const uint8_t*>(table);
  if (sub_dim == 4)
    hipLaunchKernelGGL(nearest_kernel<4>, dim3(blocks), dim3(256), 0, s, t, v, n, out);
  else
    hipLaunchKernelGGL(nearest_kernel<8>, dim3(blocks), dim3(256), 0, s, t, v, n, out);
  return hipGetLastError();
}

hipError_t launch_search_table(void* table, hipStream_t s) {
  uint8_t* t = static_cast<uint8_t*>(table);
  const Edges E = make_edges();
  hipLaunchKernelGGL(tab_init_kernel, dim3((kFine + 255) / 256), dim3(256), 0, s, E, t);
  hipLaunchKernelGGL(tab_write_kernel, dim3(kCells), dim3(256), 0, s, t);
  return hipGetLastError();
}

}  // namespace nsn
