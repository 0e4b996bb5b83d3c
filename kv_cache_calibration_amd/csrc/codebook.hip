// Codebook kernels: Lloyd k-means on standard-normal samples, fp16 rounding,
// and the prepared-codebook table.
// [NSNQuant summary (gist.science), Methodology §3, codebook construction:
//  one global codebook from k-means over synthetic N(0,1) data; authors'
//  README, Overview.]
//
// Everything here is float64 with contraction disabled, so distances are
// the exact-form sum of rounded squares and each centroid is the sequential
// sum of its members in sample order divided by the member count.  The
// result is deterministic and reproducible bit for bit.
#include "nsn_device.h"
#include "nsn_launch.h"

namespace nsn {

namespace {

constexpr int kAssignThreads = 256;

// Label every sample with its nearest centroid (lowest index on ties).
template <int M>
__global__ __launch_bounds__(kAssignThreads) void kmeans_assign(
    const double* __restrict__ x, int64_t n, const double* __restrict__ cent,
    int32_t* __restrict__ labels) {
#pragma clang fp contract(off)
  __shared__ double c[kCodes * M];
  for (int i = threadIdx.x; i < kCodes * M; i += kAssignThreads) c[i] = cent[i];
  __syncthreads();
  const int64_t s = static_cast<int64_t>(blockIdx.x) * kAssignThreads + threadIdx.x;
  if (s >= n) return;
  double v[M];
#pragma unroll
  for (int e = 0; e < M; ++e) v[e] = x[s * M + e];
  double best = 0.0;
  int bi = 0;
  for (int k = 0; k < kCodes; ++k) {
    double d = 0.0;
#pragma unroll
    for (int e = 0; e < M; ++e) {
      const double t = v[e] - c[k * M + e];
      const double sq = t * t;
      d = (e == 0) ? sq : d + sq;
    }
    if (k == 0 || d < best) {
      best = d;
      bi = k;
    }
  }
  labels[s] = bi;
}

// New centroid (k, e) = sequential sum over samples with label k, in sample
// order, divided by the count; an empty cluster keeps its centroid.
template <int M>
__global__ __launch_bounds__(256) void kmeans_update(const double* __restrict__ x, int64_t n,
                                                     const int32_t* __restrict__ labels,
                                                     double* __restrict__ cent) {
#pragma clang fp contract(off)
  const int id = blockIdx.x * 256 + threadIdx.x;
  if (id >= kCodes * M) return;
  const int k = id / M, e = id % M;
  double s = 0.0;
  int64_t cnt = 0;
  for (int64_t i = 0; i < n; ++i) {
    if (labels[i] == k) {
      s = s + x[i * M + e];
      ++cnt;
    }
  }
  if (cnt > 0) cent[id] = s / static_cast<double>(cnt);
}

template <int M>
__global__ void kmeans_init(const double* __restrict__ x, double* __restrict__ cent) {
  const int id = blockIdx.x * 256 + threadIdx.x;
  if (id < kCodes * M) cent[id] = x[id];
}

// Round a double to the nearest fp16 value (ties to even), returned exactly
// as a float.  Normal fp16 range: 11 significant bits; below 2^-14 the
// spacing is 2^-24; beyond 65504 (after rounding) the result is infinite.
__device__ float round_to_half(double v) {
  if (!(v == v)) return __builtin_nanf("");
  const double a = fabs(v);
  double r;
  if (a < 6.103515625e-05) {  // 2^-14: subnormal spacing 2^-24
    r = rint(v * 16777216.0) / 16777216.0;
  } else {
    const int e = ilogb(a);                 // 2^e <= a < 2^(e+1)
    const double q = ldexp(1.0, e - 10);    // spacing of fp16 at this binade
    r = rint(v / q) * q;
  }
  if (fabs(r) > 65504.0) r = v > 0 ? __builtin_huge_val() : -__builtin_huge_val();
  return static_cast<float>(r);
}

template <int M>
__global__ void kmeans_finish(const double* __restrict__ cent, float* __restrict__ out) {
  const int id = blockIdx.x * 256 + threadIdx.x;
  if (id < kCodes * M) out[id] = round_to_half(cent[id]);
}

// Nearest of the 16 levels (k - 7.5) * 3/8 of the double-quantized codebook
// [NSNQuant summary, Methodology §3, Double Quantization: codebook entries
//  at 4 bits; the level grid is this library's reading].  Magnitude level
// j (3/16 + 3j/8) owns |v| in (3j/8, 3(j+1)/8]; the bounds are exact in fp32,
// so a tie goes to the smaller magnitude, and 0 goes to +3/16.
__device__ __forceinline__ float level4(float v) {
  const float a = fabsf(v);
  int j = 0;
#pragma unroll
  for (int k = 1; k < 8; ++k) j = a > 0.375f * static_cast<float>(k) ? k : j;
  const float m = 0.1875f + 0.375f * static_cast<float>(j);
  return v < 0.f ? -m : m;
}

template <int M>
__global__ void prepare_kernel(const float* __restrict__ cb, int dq, uint8_t* __restrict__ table) {
  const int k = threadIdx.x;  // 256 threads, one per codeword
  float* tc = reinterpret_cast<float*>(table + kTabCodebook);
  float* tn = reinterpret_cast<float*>(table + kTabNorm2);
  uint16_t* th = reinterpret_cast<uint16_t*>(table + kTabCodebookH);
  float n2 = 0.f;
#pragma unroll
  for (int e = 0; e < M; ++e) {
    // one codebook for every consumer: the entry rounded once to fp16
    // (nearest, ties to even) or, double-quantized, to its 4-bit level (an
    // fp16 value too); the fp32 and fp16 copies then hold the same numbers
    const float c = dq ? level4(cb[k * M + e]) : h2f(f2h(cb[k * M + e]));
    tc[k * M + e] = c;
    th[k * M + e] = f2h(c);
    n2 = fmaf(c, c, n2);
  }
  tn[k] = n2;
}

// ---- fine-tuning on cosine distance
// [NSNQuant summary, Methodology §3, codebook construction: the k-means
//  codebook is fine-tuned to minimize the cosine distance between original
//  and quantized vectors, without any model.]
// Full d-dimensional vectors (d = 128) are split into d/m sub-vectors, each
// assigned its nearest codeword (kmeans_assign on the same memory viewed as
// sub-vectors).  Loss: mean over vectors of 1 - cos(h, h_hat).  With the
// assignment held fixed, dL/dc_k = -(1/n) sum over the sub-vectors (i, j)
// assigned to k of w_i (h_ij - r_i c_k), w_i = 1/sqrt(|h_i|^2 |h_hat_i|^2),
// r_i = <h_i, h_hat_i>/|h_hat_i|^2 (both 0 when a norm is 0).  One
// full-batch Adam step per iteration (Kingma and Ba, bias-corrected
// moments).  Float64 without contraction, every sum left to right in a
// fixed order: coordinates in index order, gradient terms in sample order.

// Per vector: (w_i, r_i).
template <int M>
__global__ __launch_bounds__(256) void tune_stats(const double* __restrict__ h, int64_t n_vec,
                                                  const int32_t* __restrict__ labels,
                                                  const double* __restrict__ cent,
                                                  double* __restrict__ wr) {
#pragma clang fp contract(off)
  constexpr int NS = kD / M;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n_vec) return;
  double p = 0.0, a = 0.0, b = 0.0;
  for (int j = 0; j < NS; ++j) {
    const int k = labels[i * NS + j];
#pragma unroll
    for (int e = 0; e < M; ++e) {
      const double x = h[i * kD + j * M + e], c = cent[k * M + e];
      p = p + x * c;
      a = a + x * x;
      b = b + c * c;
    }
  }
  const double ab = a * b;
  double w = 0.0, r = 0.0;
  if (ab > 0.0) {
    w = 1.0 / sqrt(ab);
    r = p / b;
  }
  wr[2 * i] = w;
  wr[2 * i + 1] = r;
}

// Gradient of coordinate (k, e), summed over the members of k in sample
// order, and the Adam update of that coordinate (it reads only its own
// codeword, so the update is in place).
struct AdamArgs {
  double lr, b1, b2, eps, b1t, b2t;   // b1t, b2t = beta^t of this step
};
template <int M>
__global__ __launch_bounds__(256) void tune_update(const double* __restrict__ h, int64_t n_vec,
                                                   const int32_t* __restrict__ labels,
                                                   const double* __restrict__ wr,
                                                   double* __restrict__ cent, double* __restrict__ mom,
                                                   double* __restrict__ vel, AdamArgs ad) {
#pragma clang fp contract(off)
  constexpr int NS = kD / M;
  const int id = blockIdx.x * 256 + threadIdx.x;
  if (id >= kCodes * M) return;
  const int k = id / M, e = id % M;
  const double c = cent[id];
  const int64_t ns = n_vec * NS;
  double s = 0.0;
  for (int64_t i = 0; i < ns; ++i) {
    if (labels[i] == k) {
      const int64_t v = i / NS;
      s = s + (h[i * M + e] - wr[2 * v + 1] * c) * wr[2 * v];
    }
  }
  const double g = -s / static_cast<double>(n_vec);
  const double mo = ad.b1 * mom[id] + (1.0 - ad.b1) * g;
  const double ve = ad.b2 * vel[id] + (1.0 - ad.b2) * (g * g);
  mom[id] = mo;
  vel[id] = ve;
  const double mhat = mo / (1.0 - ad.b1t);
  const double vhat = ve / (1.0 - ad.b2t);
  cent[id] = c - ad.lr * mhat / (sqrt(vhat) + ad.eps);
}

template <int M>
__global__ void tune_init(const float* __restrict__ cb, double* __restrict__ cent,
                          double* __restrict__ mom, double* __restrict__ vel) {
  const int id = blockIdx.x * 256 + threadIdx.x;
  if (id < kCodes * M) {
    cent[id] = static_cast<double>(cb[id]);
    mom[id] = 0.0;
    vel[id] = 0.0;
  }
}

struct TuneWs {
  int32_t* labels;
  double* wr;
  double* cent;
  double* mom;
  double* vel;
  size_t bytes;
};
TuneWs tune_ws(void* base, int sub_dim, int64_t n_vec) {
  auto pad = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
  const size_t lab = pad(static_cast<size_t>(n_vec) * (kD / sub_dim) * 4);
  const size_t wr = pad(static_cast<size_t>(n_vec) * 2 * 8);
  const size_t cb = pad(static_cast<size_t>(kCodes) * sub_dim * 8);
  uint8_t* p = static_cast<uint8_t*>(base);
  TuneWs w{};
  w.labels = reinterpret_cast<int32_t*>(p);
  w.wr = reinterpret_cast<double*>(p + lab);
  w.cent = reinterpret_cast<double*>(p + lab + wr);
  w.mom = reinterpret_cast<double*>(p + lab + wr + cb);
  w.vel = reinterpret_cast<double*>(p + lab + wr + 2 * cb);
  w.bytes = lab + wr + 3 * cb;
  return w;
}

template <int M>
hipError_t tune(int64_t n_vec, int iters, double lr, const double* vec, float* codebook, void* ws,
                hipStream_t s) {
  const TuneWs w = tune_ws(ws, M, n_vec);
  const int cb_blocks = (kCodes * M + 255) / 256;
  const int64_t ns = n_vec * (kD / M);
  const unsigned ab = static_cast<unsigned>((ns + kAssignThreads - 1) / kAssignThreads);
  const unsigned vb = static_cast<unsigned>((n_vec + 255) / 256);
  hipLaunchKernelGGL(tune_init<M>, dim3(cb_blocks), dim3(256), 0, s, codebook, w.cent, w.mom, w.vel);
  AdamArgs ad{lr, 0.9, 0.999, 1e-8, 1.0, 1.0};
  for (int it = 0; it < iters; ++it) {
    ad.b1t = ad.b1t * ad.b1;
    ad.b2t = ad.b2t * ad.b2;
    hipLaunchKernelGGL(kmeans_assign<M>, dim3(ab), dim3(kAssignThreads), 0, s, vec, ns, w.cent,
                       w.labels);
    hipLaunchKernelGGL(tune_stats<M>, dim3(vb), dim3(256), 0, s, vec, n_vec, w.labels, w.cent, w.wr);
    hipLaunchKernelGGL(tune_update<M>, dim3(cb_blocks), dim3(256), 0, s, vec, n_vec, w.labels, w.wr,
                       w.cent, w.mom, w.vel, ad);
  }
  hipLaunchKernelGGL(kmeans_finish<M>, dim3(cb_blocks), dim3(256), 0, s, w.cent, codebook);
  return hipGetLastError();
}

template <int M>
hipError_t build(int64_t n, int iters, const double* samples, float* codebook, void* ws,
                 hipStream_t s) {
  int32_t* labels = static_cast<int32_t*>(ws);
  const size_t lab_bytes = (static_cast<size_t>(n) * 4 + 255) & ~static_cast<size_t>(255);
  double* cent = reinterpret_cast<double*>(static_cast<uint8_t*>(ws) + lab_bytes);
  const int cb_blocks = (kCodes * M + 255) / 256;
  hipLaunchKernelGGL(kmeans_init<M>, dim3(cb_blocks), dim3(256), 0, s, samples, cent);
  const unsigned ab = static_cast<unsigned>((n + kAssignThreads - 1) / kAssignThreads);
  for (int it = 0; it < iters; ++it) {
    hipLaunchKernelGGL(kmeans_assign<M>, dim3(ab), dim3(kAssignThreads), 0, s, samples, n, cent,
                       labels);
    hipLaunchKernelGGL(kmeans_update<M>, dim3(cb_blocks), dim3(256), 0, s, samples, n, labels,
                       cent);
  }
  hipLaunchKernelGGL(kmeans_finish<M>, dim3(cb_blocks), dim3(256), 0, s, cent, codebook);
  return hipGetLastError();
}

}  // namespace

size_t build_codebook_workspace(int sub_dim, int n_codes, int64_t n) {
  const size_t lab_bytes = (static_cast<size_t>(n) * 4 + 255) & ~static_cast<size_t>(255);
  return lab_bytes + static_cast<size_t>(n_codes) * sub_dim * sizeof(double);
}

hipError_t launch_build_codebook(int sub_dim, int n_codes, int64_t n, int iters,
                                 const double* samples, float* codebook, void* ws,
                                 hipStream_t s) {
  (void)n_codes;
  return sub_dim == 4 ? build<4>(n, iters, samples, codebook, ws, s)
                      : build<8>(n, iters, samples, codebook, ws, s);
}

size_t tune_codebook_workspace(int sub_dim, int64_t n_vec) {
  return tune_ws(nullptr, sub_dim, n_vec).bytes;
}

hipError_t launch_tune_codebook(int sub_dim, int64_t n_vec, int iters, double lr,
                                const double* vectors, float* codebook, void* ws, hipStream_t s) {
  return sub_dim == 4 ? tune<4>(n_vec, iters, lr, vectors, codebook, ws, s)
                      : tune<8>(n_vec, iters, lr, vectors, codebook, ws, s);
}

hipError_t launch_prepare_codebook(const float* codebook, int sub_dim, int dq, void* table,
                                   hipStream_t s) {
  uint8_t* t = static_cast<uint8_t*>(table);
  if (sub_dim == 4) {
    hipLaunchKernelGGL(prepare_kernel<4>, dim3(1), dim3(256), 0, s, codebook, dq, t);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_search_table(table, s);
  }
  hipLaunchKernelGGL(prepare_kernel<8>, dim3(1), dim3(256), 0, s, codebook, dq, t);
  return hipGetLastError();
}

}  // namespace nsn
