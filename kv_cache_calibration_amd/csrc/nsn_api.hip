// C ABI of the NSNQuant library: argument validation, then kernel launch.
// The contract of every entry point is documented in include/nsn.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include <cmath>
#include <mutex>

#include "nsn.h"
#include "nsn_device.h"
#include "nsn_launch.h"

namespace nsn {
int attn_max_resid();
}

namespace {

thread_local char g_err[512] = "";

nsn_status fail(nsn_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

nsn_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) {
    g_err[0] = '\0';
    return NSN_OK;
  }
  return fail(NSN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// One launch covers a call: its work-items (workgroups x threads, at most
// 256 threads per workgroup) must stay below 2^32.
constexpr int64_t kMaxGroups = (int64_t(1) << 24) - 1;     // workgroup per token group
constexpr int64_t kMaxNearest = (int64_t(1) << 32) - 256;  // one work-item per sub-vector
constexpr int64_t kMaxAppendSeq = (int64_t(1) << 28) - 16;  // 16 work-items per sequence

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// The shift argument: 16 bytes, or 8 with NSN_DQ (the 136-byte group records
// are 8-byte aligned, so a cache advanced by an odd number of groups is too).
bool shift_aligned(const nsn_params* p, const void* q) {
  return (reinterpret_cast<uintptr_t>(q) & ((p->flags & NSN_DQ) ? 7u : 15u)) == 0;
}

nsn_status check_params(const nsn_params* p) {
  if (!p) return fail(NSN_ERR_INVALID_ARG, "params is NULL");
  if (p->head_dim != 128) return fail(NSN_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", p->head_dim);
  if (p->sub_dim != 4 && p->sub_dim != 8)
    return fail(NSN_ERR_UNSUPPORTED, "sub_dim must be 4 or 8 (got %d)", p->sub_dim);
  if (p->n_codes != 256) return fail(NSN_ERR_UNSUPPORTED, "n_codes must be 256 (got %d)", p->n_codes);
  if (p->group_size != 128 && p->group_size != 256)
    return fail(NSN_ERR_UNSUPPORTED, "group_size must be 128 or 256 (got %d)", p->group_size);
  if (p->flags & ~(NSN_SCALE_ADJUST | NSN_DQ | NSN_RHT))
    return fail(NSN_ERR_INVALID_ARG, "unknown flags 0x%x", p->flags);
  if ((p->flags & NSN_DQ) && p->group_size != 128)
    return fail(NSN_ERR_UNSUPPORTED, "NSN_DQ needs group_size 128 (got %d)", p->group_size);
  return NSN_OK;
}

// The kernels' sign mask: the caller's with NSN_RHT, else all zero (plain
// rotation).
nsn::RhtSigns signs_of(const nsn_params* p) {
  nsn::RhtSigns r{};
  if (p->flags & NSN_RHT)
    for (int i = 0; i < 4; ++i) r.w[i] = p->rht_signs[i];
  return r;
}

#define NSN_TRY(expr)            \
  do {                           \
    nsn_status st_ = (expr);     \
    if (st_ != NSN_OK) return st_; \
  } while (0)

}  // namespace

extern "C" {

const char* nsn_version(void) { return "nsnq-gfx950 0.2"; }

const char* nsn_last_error(void) { return g_err; }

const char* nsn_status_string(nsn_status s) {
  switch (s) {
    case NSN_OK: return "ok";
    case NSN_ERR_INVALID_ARG: return "invalid argument";
    case NSN_ERR_UNSUPPORTED: return "unsupported shape or parameter";
    case NSN_ERR_WORKSPACE: return "workspace too small";
    case NSN_ERR_HIP: return "HIP runtime error";
    case NSN_ERR_INTERNAL: return "internal error";
    default: break;
  }
  return "unknown status";
}

size_t nsn_table_size(const nsn_params* p) {
  if (check_params(p) != NSN_OK) return 0;
  return nsn::kTabBytes;
}

size_t nsn_build_codebook_workspace_size(int32_t sub_dim, int32_t n_codes, int64_t n_samples) {
  if ((sub_dim != 4 && sub_dim != 8) || n_codes != 256 || n_samples < n_codes ||
      n_samples > (int64_t(1) << 26))
    return 0;
  return nsn::build_codebook_workspace(sub_dim, n_codes, n_samples);
}

nsn_status nsn_build_codebook(int32_t sub_dim, int32_t n_codes, int64_t n_samples, int32_t iters,
                              const double* samples, float* codebook, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (sub_dim != 4 && sub_dim != 8)
    return fail(NSN_ERR_UNSUPPORTED, "sub_dim must be 4 or 8 (got %d)", sub_dim);
  if (n_codes != 256) return fail(NSN_ERR_UNSUPPORTED, "n_codes must be 256 (got %d)", n_codes);
  if (n_samples < n_codes || n_samples > (int64_t(1) << 26))
    return fail(NSN_ERR_INVALID_ARG, "n_samples must be in [n_codes, 2^26] (got %lld)",
                static_cast<long long>(n_samples));
  if (iters < 1 || iters > 1000) return fail(NSN_ERR_INVALID_ARG, "iters must be in [1, 1000]");
  if (!samples || !codebook || !workspace)
    return fail(NSN_ERR_INVALID_ARG, "samples, codebook and workspace must be non-NULL");
  if (!aligned16(samples) || !aligned16(codebook) || !aligned16(workspace))
    return fail(NSN_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  const size_t need = nsn::build_codebook_workspace(sub_dim, n_codes, n_samples);
  if (workspace_bytes < need)
    return fail(NSN_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
  return hip_status(nsn::launch_build_codebook(sub_dim, n_codes, n_samples, iters, samples, codebook,
                                               workspace, static_cast<hipStream_t>(stream)),
                    "nsn_build_codebook launch");
}

size_t nsn_tune_codebook_workspace_size(int32_t sub_dim, int32_t n_codes, int64_t n_vec) {
  if ((sub_dim != 4 && sub_dim != 8) || n_codes != 256 || n_vec < 1) return 0;
  return nsn::tune_codebook_workspace(sub_dim, n_vec);
}

nsn_status nsn_tune_codebook(int32_t sub_dim, int32_t n_codes, int64_t n_vec, int32_t iters,
                             double lr, const double* vectors, float* codebook, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (sub_dim != 4 && sub_dim != 8)
    return fail(NSN_ERR_UNSUPPORTED, "sub_dim must be 4 or 8 (got %d)", sub_dim);
  if (n_codes != 256) return fail(NSN_ERR_UNSUPPORTED, "n_codes must be 256 (got %d)", n_codes);
  if (n_vec < 1 || n_vec > ((int64_t(1) << 26) / (128 / sub_dim)))
    return fail(NSN_ERR_INVALID_ARG, "n_vec must be in [1, 2^26 * sub_dim / 128] (got %lld)",
                static_cast<long long>(n_vec));
  if (iters < 0 || iters > 100000) return fail(NSN_ERR_INVALID_ARG, "iters must be in [0, 100000]");
  if (!(lr > 0.0 && lr <= 1.0)) return fail(NSN_ERR_INVALID_ARG, "lr must be in (0, 1], got %g", lr);
  if (!vectors || !codebook || !workspace)
    return fail(NSN_ERR_INVALID_ARG, "vectors, codebook and workspace must be non-NULL");
  if (!aligned16(vectors) || !aligned16(codebook) || !aligned16(workspace))
    return fail(NSN_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  const size_t need = nsn::tune_codebook_workspace(sub_dim, n_vec);
  if (workspace_bytes < need)
    return fail(NSN_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
  return hip_status(nsn::launch_tune_codebook(sub_dim, n_vec, iters, lr, vectors, codebook, workspace,
                                              static_cast<hipStream_t>(stream)),
                    "nsn_tune_codebook launch");
}

nsn_status nsn_prepare_codebook(const nsn_params* p, const float* codebook, void* table,
                                size_t table_bytes, void* stream) {
  NSN_TRY(check_params(p));
  if (!codebook || !table) return fail(NSN_ERR_INVALID_ARG, "codebook and table must be non-NULL");
  if (!aligned16(codebook) || !aligned16(table))
    return fail(NSN_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  if (table_bytes < nsn::kTabBytes)
    return fail(NSN_ERR_WORKSPACE, "table needs %zu bytes, got %zu", nsn::kTabBytes, table_bytes);
  return hip_status(nsn::launch_prepare_codebook(codebook, p->sub_dim, (p->flags & NSN_DQ) ? 1 : 0, table,
                                                 static_cast<hipStream_t>(stream)),
                    "nsn_prepare_codebook launch");
}

nsn_status nsn_nearest_codeword(const nsn_params* p, const void* table, const float* v, int64_t n,
                                uint8_t* out, void* stream) {
  NSN_TRY(check_params(p));
  if (n < 0) return fail(NSN_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) {
    g_err[0] = '\0';
    return NSN_OK;
  }
  if (n > kMaxNearest)
    return fail(NSN_ERR_UNSUPPORTED, "n above %lld", static_cast<long long>(kMaxNearest));
  if (!table || !v || !out) return fail(NSN_ERR_INVALID_ARG, "table, v and out must be non-NULL");
  if (!aligned16(table) || !aligned16(v) || !aligned16(out))
    return fail(NSN_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  return hip_status(nsn::launch_nearest(table, p->sub_dim, v, n, out,
                                        static_cast<hipStream_t>(stream)),
                    "nsn_nearest_codeword launch");
}

// Sequence strides of meta and shift (uint16 units) for the plain and the
// double-quantized layouts.
static nsn_status check_meta_strides(const nsn_params* p, int64_t n_tok, int64_t meta_seq_stride,
                                     int64_t shift_seq_stride) {
  const int64_t G = p->group_size;
  if (p->flags & NSN_DQ) {
    if (meta_seq_stride < n_tok || meta_seq_stride % 8)
      return fail(NSN_ERR_INVALID_ARG, "meta_seq_stride must be >= n_tok and a multiple of 8 (NSN_DQ)");
    if (shift_seq_stride < (n_tok / G) * nsn::kDqRecU16 || shift_seq_stride % 4)
      return fail(NSN_ERR_INVALID_ARG, "shift_seq_stride must be >= (n_tok/128)*%d and a multiple of 4 (NSN_DQ)",
                  nsn::kDqRecU16);
    return NSN_OK;
  }
  if (meta_seq_stride < n_tok * 2 || meta_seq_stride % 8)
    return fail(NSN_ERR_INVALID_ARG, "meta_seq_stride must be >= 2*n_tok and a multiple of 8");
  if (shift_seq_stride < (n_tok / G) * 128 || shift_seq_stride % 8)
    return fail(NSN_ERR_INVALID_ARG, "shift_seq_stride must be >= (n_tok/G)*128 and a multiple of 8");
  return NSN_OK;
}

nsn_status nsn_quantize(const nsn_params* p, nsn_dtype in_dtype, const void* x, int64_t n_seq,
                        int64_t n_tok, int64_t x_seq_stride, const void* table, uint8_t* codes,
                        int64_t codes_seq_stride, uint16_t* meta, int64_t meta_seq_stride,
                        uint16_t* shift, int64_t shift_seq_stride, void* stream) {
  NSN_TRY(check_params(p));
  if (in_dtype != NSN_F16 && in_dtype != NSN_F32)
    return fail(NSN_ERR_INVALID_ARG, "in_dtype must be NSN_F16 or NSN_F32");
  if ((p->flags & NSN_DQ) && in_dtype != NSN_F16)
    return fail(NSN_ERR_UNSUPPORTED, "NSN_DQ quantizes fp16 input only");
  if (n_seq < 0 || n_tok < 0) return fail(NSN_ERR_INVALID_ARG, "n_seq and n_tok must be >= 0");
  if (n_tok % p->group_size)
    return fail(NSN_ERR_INVALID_ARG, "n_tok (%lld) must be a multiple of group_size (%d)",
                static_cast<long long>(n_tok), p->group_size);
  if (n_seq == 0 || n_tok == 0) {
    g_err[0] = '\0';
    return NSN_OK;
  }
  const int64_t G = p->group_size, nsub = 128 / p->sub_dim;
  const int64_t esz = in_dtype == NSN_F16 ? 2 : 4;
  if (!x || !table || !codes || !meta || !shift)
    return fail(NSN_ERR_INVALID_ARG, "x, table, codes, meta and shift must be non-NULL");
  if (!aligned16(x) || !aligned16(table) || !aligned16(codes) || !aligned16(meta) || !shift_aligned(p, shift))
    return fail(NSN_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  if (n_seq > 1) {
    if (x_seq_stride < n_tok * 128 || (x_seq_stride * esz) % 16)
      return fail(NSN_ERR_INVALID_ARG, "x_seq_stride must be >= n_tok*128 and a multiple of 16 bytes");
    if (codes_seq_stride < n_tok * nsub || codes_seq_stride % 16)
      return fail(NSN_ERR_INVALID_ARG, "codes_seq_stride must be >= n_tok*%lld and a multiple of 16",
                  static_cast<long long>(nsub));
    NSN_TRY(check_meta_strides(p, n_tok, meta_seq_stride, shift_seq_stride));
  }
  if (n_seq > kMaxGroups || n_seq * (n_tok / G) > kMaxGroups)
    return fail(NSN_ERR_UNSUPPORTED, "%lld token groups in one call (at most %lld)",
                static_cast<long long>(n_seq * (n_tok / G)), static_cast<long long>(kMaxGroups));
  nsn::QuantArgs a{x, in_dtype == NSN_F32, n_seq, n_tok, x_seq_stride, table, codes,
                   codes_seq_stride, meta, meta_seq_stride, shift, shift_seq_stride,
                   p->sub_dim, p->group_size, static_cast<int>(p->flags & NSN_SCALE_ADJUST),
                   (p->flags & NSN_DQ) ? 1 : 0};
  a.rht = signs_of(p);
  return hip_status(nsn::launch_quantize(a, static_cast<hipStream_t>(stream)), "nsn_quantize launch");
}

nsn_status nsn_dequantize(const nsn_params* p, const uint8_t* codes, int64_t codes_seq_stride,
                          const uint16_t* meta, int64_t meta_seq_stride, const uint16_t* shift,
                          int64_t shift_seq_stride, const void* table, int64_t n_seq, int64_t n_tok,
                          nsn_dtype out_dtype, void* x_hat, int64_t out_seq_stride, void* stream) {
  NSN_TRY(check_params(p));
  if (out_dtype != NSN_F16 && out_dtype != NSN_F32)
    return fail(NSN_ERR_INVALID_ARG, "out_dtype must be NSN_F16 or NSN_F32");
  if (n_seq < 0 || n_tok < 0) return fail(NSN_ERR_INVALID_ARG, "n_seq and n_tok must be >= 0");
  if (n_tok % p->group_size)
    return fail(NSN_ERR_INVALID_ARG, "n_tok (%lld) must be a multiple of group_size (%d)",
                static_cast<long long>(n_tok), p->group_size);
  if (n_seq == 0 || n_tok == 0) {
    g_err[0] = '\0';
    return NSN_OK;
  }
  const int64_t G = p->group_size, nsub = 128 / p->sub_dim;
  const int64_t esz = out_dtype == NSN_F16 ? 2 : 4;
  if (!x_hat || !table || !codes || !meta || !shift)
    return fail(NSN_ERR_INVALID_ARG, "codes, meta, shift, table and x_hat must be non-NULL");
  if (!aligned16(x_hat) || !aligned16(table) || !aligned16(codes) || !aligned16(meta) || !shift_aligned(p, shift))
    return fail(NSN_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  if (n_seq > 1) {
    if (out_seq_stride < n_tok * 128 || (out_seq_stride * esz) % 16)
      return fail(NSN_ERR_INVALID_ARG, "out_seq_stride must be >= n_tok*128 and a multiple of 16 bytes");
    if (codes_seq_stride < n_tok * nsub || codes_seq_stride % 16)
      return fail(NSN_ERR_INVALID_ARG, "codes_seq_stride must be >= n_tok*%lld and a multiple of 16",
                  static_cast<long long>(nsub));
    NSN_TRY(check_meta_strides(p, n_tok, meta_seq_stride, shift_seq_stride));
  }
  if (n_seq > kMaxGroups || n_seq * (n_tok / G) > kMaxGroups)
    return fail(NSN_ERR_UNSUPPORTED, "%lld token groups in one call (at most %lld)",
                static_cast<long long>(n_seq * (n_tok / G)), static_cast<long long>(kMaxGroups));
  nsn::DequantArgs a{codes, codes_seq_stride, meta, meta_seq_stride, shift, shift_seq_stride, table,
                     n_seq, n_tok, out_dtype == NSN_F32, x_hat, out_seq_stride, p->sub_dim,
                     p->group_size, (p->flags & NSN_DQ) ? 1 : 0};
  a.rht = signs_of(p);
  return hip_status(nsn::launch_dequantize(a, static_cast<hipStream_t>(stream)),
                    "nsn_dequantize launch");
}

nsn_status nsn_residual_append(const uint16_t* tok, int64_t n_seq, uint16_t* resid,
                               int64_t resid_seq_stride, int64_t resid_capacity, int64_t pos,
                               void* stream) {
  if (n_seq < 0) return fail(NSN_ERR_INVALID_ARG, "n_seq must be >= 0");
  if (pos < 0 || pos >= resid_capacity)
    return fail(NSN_ERR_INVALID_ARG, "pos (%lld) must be in [0, resid_capacity=%lld)",
                static_cast<long long>(pos), static_cast<long long>(resid_capacity));
  if (n_seq == 0) {
    g_err[0] = '\0';
    return NSN_OK;
  }
  if (!tok || !resid) return fail(NSN_ERR_INVALID_ARG, "tok and resid must be non-NULL");
  if (!aligned16(tok) || !aligned16(resid))
    return fail(NSN_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  if (n_seq > kMaxAppendSeq)   // 16 work-items per sequence in one launch
    return fail(NSN_ERR_UNSUPPORTED, "n_seq above %lld", static_cast<long long>(kMaxAppendSeq));
  if (n_seq > 1 && (resid_seq_stride < resid_capacity * 128 || resid_seq_stride % 8))
    return fail(NSN_ERR_INVALID_ARG,
                "resid_seq_stride must be >= resid_capacity*128 and a multiple of 8");
  return hip_status(nsn::launch_residual_append(tok, n_seq, resid, resid_seq_stride, pos,
                                                static_cast<hipStream_t>(stream)),
                    "nsn_residual_append launch");
}

static nsn_status check_attn(const nsn_params* p, const nsn_attn_shape* s) {
  NSN_TRY(check_params(p));
  if (!s) return fail(NSN_ERR_INVALID_ARG, "shape is NULL");
  if (s->batch < 1 || s->n_kv_heads < 1 || s->n_q_heads < 1)
    return fail(NSN_ERR_INVALID_ARG, "batch, n_q_heads and n_kv_heads must be >= 1");
  if (s->n_q_heads % s->n_kv_heads)
    return fail(NSN_ERR_INVALID_ARG, "n_q_heads must be a multiple of n_kv_heads");
  if (s->batch > 65535 || static_cast<int64_t>(s->n_kv_heads) * s->n_q_heads > (1 << 20))
    return fail(NSN_ERR_UNSUPPORTED, "batch or head count too large");
  // the split launch's second grid dimension: one workgroup row per (kv
  // head, block of up to four of its query heads), at most 65535
  if (static_cast<int64_t>(s->n_kv_heads) * ((s->n_q_heads / s->n_kv_heads + 3) / 4) > 65535)
    return fail(NSN_ERR_UNSUPPORTED, "too many (kv head, query-head block) rows for one launch");
  if (s->n_quant_tok < 0 || s->n_resid_tok < 0)
    return fail(NSN_ERR_INVALID_ARG, "token counts must be >= 0");
  if (s->n_quant_tok + static_cast<int64_t>(s->n_resid_tok) < 1)
    return fail(NSN_ERR_INVALID_ARG, "need at least one quantized or residual token");
  if (s->n_quant_tok % p->group_size)
    return fail(NSN_ERR_INVALID_ARG, "n_quant_tok must be a multiple of group_size");
  if (s->cache_capacity < s->n_quant_tok || s->cache_capacity % p->group_size)
    return fail(NSN_ERR_INVALID_ARG,
                "cache_capacity must be >= n_quant_tok and a multiple of group_size");
  if (s->resid_capacity < s->n_resid_tok)
    return fail(NSN_ERR_INVALID_ARG, "resid_capacity must be >= n_resid_tok");
  if (s->n_resid_tok > nsn::attn_max_resid())
    return fail(NSN_ERR_UNSUPPORTED, "n_resid_tok above %d", nsn::attn_max_resid());
  if (!(s->softmax_scale > 0.f) || !(s->softmax_scale < 1e30f))
    return fail(NSN_ERR_INVALID_ARG, "softmax_scale must be positive and finite");
  return NSN_OK;
}

size_t nsn_decode_attention_workspace_size(const nsn_params* p, const nsn_attn_shape* s) {
  if (check_attn(p, s) != NSN_OK) return 0;
  return nsn::attn_workspace_bytes(
      s->batch, s->n_q_heads, nsn::attn_split_bound(s->batch, s->n_q_heads, s->n_kv_heads, s->n_quant_tok));
}

// Scratch of nsn_decode_attention_noalloc: the split partials live in a
// static device array instead of a caller workspace.  In host code `scratch`
// names a host-side stand-in, so its device address is looked up once per
// device (with that device current) and only that address is used.
namespace {
constexpr size_t kScratchBytes = size_t(4) << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

hipError_t scratch_of_current_device(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
  });
  *out = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}
}  // namespace

static nsn_status decode_attention_impl(const nsn_params* p, const nsn_attn_shape* s,
                                        const nsn_rope* r, const uint16_t* q,
                                        const uint8_t* k_codes, const uint16_t* k_meta,
                                        const uint16_t* k_shift, const uint8_t* v_codes,
                                        const uint16_t* v_meta, const uint16_t* v_shift,
                                        const uint16_t* k_resid, const uint16_t* v_resid,
                                        const void* table, void* workspace, size_t workspace_bytes,
                                        float* out, void* stream, const char* what,
                                        bool use_scratch = false) {
  NSN_TRY(check_attn(p, s));
  if (r && (p->flags & NSN_RHT))
    return fail(NSN_ERR_UNSUPPORTED, "NSN_RHT is not supported with rotary keys");
  if (!q || !table || (!workspace && !use_scratch) || !out)
    return fail(NSN_ERR_INVALID_ARG, "q, table, workspace and out must be non-NULL");
  if (s->n_quant_tok > 0 && (!k_codes || !k_meta || !k_shift || !v_codes || !v_meta || !v_shift))
    return fail(NSN_ERR_INVALID_ARG, "cache arrays must be non-NULL when n_quant_tok > 0");
  if (s->n_resid_tok > 0 && (!k_resid || !v_resid))
    return fail(NSN_ERR_INVALID_ARG, "residual arrays must be non-NULL when n_resid_tok > 0");
  const void* ptrs[] = {q, k_codes, k_meta, v_codes, v_meta, k_resid, v_resid, table, workspace, out};
  // (workspace is NULL on the no-allocation path: skipped here)
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(NSN_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  if ((k_shift && !shift_aligned(p, k_shift)) || (v_shift && !shift_aligned(p, v_shift)))
    return fail(NSN_ERR_INVALID_ARG, "shift pointers must be 16-byte aligned (8 with NSN_DQ)");
  int n_split = 0, chunk = 0;
  nsn::attn_plan(s->batch, s->n_q_heads, s->n_kv_heads, s->n_quant_tok, s->n_resid_tok, p->group_size,
                 r ? 1 : 0, &n_split, &chunk);
  // the size query's monotone bound, so one workspace sized for a cache
  // serves every fill level of it
  const size_t need = nsn::attn_workspace_bytes(
      s->batch, s->n_q_heads, nsn::attn_split_bound(s->batch, s->n_q_heads, s->n_kv_heads, s->n_quant_tok));
  if (n_split > nsn::attn_split_bound(s->batch, s->n_q_heads, s->n_kv_heads, s->n_quant_tok))
    return fail(NSN_ERR_INTERNAL, "split plan above its bound");
  if (use_scratch && need > kScratchBytes)
    return fail(NSN_ERR_UNSUPPORTED,
                "this shape needs %zu bytes of split partials, above the %zu bytes of static "
                "scratch of nsn_decode_attention_noalloc (use nsn_decode_attention)",
                need, kScratchBytes);
  if (workspace_bytes < need)
    return fail(NSN_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
  if (use_scratch) {
    const hipError_t e = scratch_of_current_device(&workspace);
    if (e != hipSuccess) return hip_status(e, "nsn_decode_attention_noalloc scratch lookup");
  }
  nsn::AttnArgs a{};
  a.B = s->batch;
  a.Hq = s->n_q_heads;
  a.Hkv = s->n_kv_heads;
  a.n_quant = s->n_quant_tok;
  a.n_resid = s->n_resid_tok;
  a.cap = s->cache_capacity;
  a.rcap = s->resid_capacity;
  a.scale = s->softmax_scale;
  a.sub_dim = p->sub_dim;
  a.group_size = p->group_size;
  a.q = q;
  a.kc = k_codes;
  a.vc = v_codes;
  a.km = k_meta;
  a.vm = v_meta;
  a.ks = k_shift;
  a.vs = v_shift;
  a.kr = k_resid;
  a.vr = v_resid;
  a.table = table;
  a.work = static_cast<float*>(workspace);
  a.out = out;
  a.n_split = n_split;
  a.chunk = chunk;
  a.rope = r ? 1 : 0;
  a.rope_base = r ? r->base : 0.f;
  a.q_pos = r ? r->q_pos : 0;
  a.dq = (p->flags & NSN_DQ) ? 1 : 0;
  a.rht = signs_of(p);
  return hip_status(nsn::launch_decode_attention(a, static_cast<hipStream_t>(stream)), what);
}

nsn_status nsn_decode_attention(const nsn_params* p, const nsn_attn_shape* s, const uint16_t* q,
                                const uint8_t* k_codes, const uint16_t* k_meta,
                                const uint16_t* k_shift, const uint8_t* v_codes,
                                const uint16_t* v_meta, const uint16_t* v_shift,
                                const uint16_t* k_resid, const uint16_t* v_resid, const void* table,
                                void* workspace, size_t workspace_bytes, float* out, void* stream) {
  return decode_attention_impl(p, s, nullptr, q, k_codes, k_meta, k_shift, v_codes, v_meta, v_shift,
                               k_resid, v_resid, table, workspace, workspace_bytes, out, stream,
                               "nsn_decode_attention launch");
}

nsn_status nsn_decode_attention_noalloc(const nsn_params* p, const nsn_attn_shape* s,
                                        const uint16_t* q, const uint8_t* k_codes,
                                        const uint16_t* k_meta, const uint16_t* k_shift,
                                        const uint8_t* v_codes, const uint16_t* v_meta,
                                        const uint16_t* v_shift, const uint16_t* k_resid,
                                        const uint16_t* v_resid, const void* table, float* out,
                                        void* stream) {
  return decode_attention_impl(p, s, nullptr, q, k_codes, k_meta, k_shift, v_codes, v_meta, v_shift,
                               k_resid, v_resid, table, nullptr, kScratchBytes, out, stream,
                               "nsn_decode_attention_noalloc launch", true);
}

nsn_status nsn_decode_attention_rope(const nsn_params* p, const nsn_attn_shape* s,
                                     const nsn_rope* r, const uint16_t* q,
                                     const uint8_t* k_codes, const uint16_t* k_meta,
                                     const uint16_t* k_shift, const uint8_t* v_codes,
                                     const uint16_t* v_meta, const uint16_t* v_shift,
                                     const uint16_t* k_resid, const uint16_t* v_resid,
                                     const void* table, void* workspace, size_t workspace_bytes,
                                     float* out, void* stream) {
  if (!r) return fail(NSN_ERR_INVALID_ARG, "rope must be non-NULL");
  if (!(r->base > 1.0f) || !std::isfinite(r->base))
    return fail(NSN_ERR_INVALID_ARG, "rope base must be finite and > 1, got %g", static_cast<double>(r->base));
  if (r->q_pos < 0 || r->q_pos > (int64_t(1) << 40))
    return fail(NSN_ERR_INVALID_ARG, "q_pos must lie in [0, 2^40], got %lld", static_cast<long long>(r->q_pos));
  return decode_attention_impl(p, s, r, q, k_codes, k_meta, k_shift, v_codes, v_meta, v_shift,
                               k_resid, v_resid, table, workspace, workspace_bytes, out, stream,
                               "nsn_decode_attention_rope launch");
}

}  // extern "C"
