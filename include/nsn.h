/*
 * nsn.h -- C ABI of the NSNQuant KV-cache quantization library (gfx950).
 *
 * The method: each KV token of one head (d = 128 channels) is normalized to
 * norm sqrt(d) (scale s1), centred by the per-channel mean of its token
 * group (o), normalized again (s2), rotated by the orthonormal Hadamard
 * transform (optionally randomized by channel signs, NSN_RHT), and every
 * m-dimensional sub-vector (m = 4: 2 bits per value,
 * m = 8: 1 bit) is replaced by the index of its nearest codeword in one
 * 256-entry codebook built by k-means on standard-normal samples.
 * [NSNQuant technical summary (gist.science, es/de), Methodology §1 NSN,
 *  §2 Hadamard transform, §3 vector quantization and codebook,
 *  §4 implementation details; authors' README (DHdroid/NSNQuant), Overview.]
 *
 * Conventions for every call
 *  - Pointers documented "device" are HIP device memory owned by the caller;
 *    the library never allocates, frees or retains them.  Every device
 *    pointer must be 16-byte aligned, except that with NSN_DQ the shift
 *    (group record) pointers need only 8 (records are 136 bytes, so a
 *    cache advanced by an odd number of groups is 8-byte aligned).
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream) and never synchronize.  Kernel faults surface at the caller's
 *    next synchronization.
 *  - All arguments are validated before any HIP call.  Invalid values
 *    return NSN_ERR_INVALID_ARG, supported-but-unimplemented shapes
 *    NSN_ERR_UNSUPPORTED, a too-small workspace NSN_ERR_WORKSPACE; a failed
 *    launch returns NSN_ERR_HIP.  A detail string for the most recent error
 *    on the calling thread is available from nsn_last_error().
 *  - Inputs must be finite.  Non-finite inputs give unspecified output but
 *    never an out-of-bounds access.
 *  - The library keeps no mutable global state besides the thread-local
 *    error string and the static device scratch of
 *    nsn_decode_attention_noalloc; calls on different streams may run
 *    concurrently as long as their output buffers do not overlap (and, for
 *    nsn_decode_attention_noalloc, not on the same GPU at all).
 */
#ifndef NSN_H
#define NSN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NSN_OK = 0,
  NSN_ERR_INVALID_ARG = 1,
  NSN_ERR_UNSUPPORTED = 2,
  NSN_ERR_WORKSPACE = 3,
  NSN_ERR_HIP = 4,
  NSN_ERR_INTERNAL = 5,  /* a library invariant failed (a bug); nothing launched */
  NSN_STATUS_MAX_ENUM = 0x7fffffff   /* not a status: makes every int value valid */
} nsn_status;

typedef enum {
  NSN_F16 = 0,
  NSN_F32 = 1,
  NSN_DTYPE_MAX_ENUM = 0x7fffffff    /* not a dtype: makes every int value valid */
} nsn_dtype;

/* nsn_params.flags: per-token scale adjustment (NSNQuant summary, §3:
 * the quantized vector is rescaled so that its component along the
 * original vector is preserved; folded into the stored s2). */
#define NSN_SCALE_ADJUST 1u

/* nsn_params.flags: double quantization (NSNQuant summary, §3, Double
 * Quantization: the NSN byproducts s1 and o, and the codebook entries, are
 * themselves stored at 4 bits).  The pages fix no grids; this library reads
 * them as follows.  Requires group_size 128 (else NSN_ERR_UNSUPPORTED).
 *   meta   one fp16 s2' per token (s1 moves into the group record):
 *          meta + s*meta_seq_stride + t.
 *   shift  one record of 136 bytes (68 uint16) per group of 128 tokens, at
 *          shift + s*shift_seq_stride + (t/128)*68:
 *            bytes 0..7    fp16 lo, hi (min and max of the group's s1),
 *                          fp16 sc = max |o'| / 7, fp16 0;
 *            bytes 8..71   o' codes, channel c in byte 8 + c/2 (low nibble
 *                          for even c): round(o'_c / sc) clamped to [-7, 7]
 *                          plus 8; 0 when sc == 0; decodes to (code-8)*sc,
 *                          a code of 0 to 0;
 *            bytes 72..135 s1 codes, token t of the group in byte 72 + t/2
 *                          likewise: round((s1 - lo) * 15 / (hi - lo))
 *                          clamped to [0, 15], 0 when hi == lo; decodes to
 *                          lo + code * (hi - lo) / 15.
 *          Codes are decided in fp32, round half to even, from the
 *          unrounded s1 and o'.
 *   codebook  nsn_prepare_codebook rounds every entry to the nearest of the
 *          16 levels (k - 7.5) * 3/8, k = 0..15 (ties to the smaller
 *          magnitude, an entry of 0 to +3/16); the search, dequantization
 *          and attention use the rounded codebook.
 * nsn_quantize with this flag takes fp16 input only.  Dequantization and
 * the attention calls (with or without rotary keys) take the decoded values
 * as exact.  Metadata cost:
 * (2 + 136/128) bytes per token, 0.19 bits per value against 0.375 for
 * the fp16 (s1, s2', o') layout. */
#define NSN_DQ 2u

/* nsn_params.flags: randomized Hadamard rotation (NSNQuant summary,
 * Methodology §2: the analysis pairs NSN with the randomized transform --
 * random channel sign flips, then the Hadamard matrix -- which guarantees
 * channel variances close to 1; the pages' own implementation keeps the
 * plain transform, which is this library's default).  With this flag the
 * rotation is R = H D / sqrt(d), D = diag(+-1) given by
 * nsn_params.rht_signs: bit c % 32 of word c / 32 set means channel c is
 * negated before H.  The caller draws the signs (any generator) and passes
 * the same ones to every call on one cache; all zero is the plain rotation.
 * nsn_quantize stores h and o' in R's frame; nsn_dequantize and
 * nsn_decode_attention (and _noalloc) invert with D H / sqrt(d).  The
 * layouts are unchanged and NSN_DQ combines with it.
 * nsn_decode_attention_rope returns NSN_ERR_UNSUPPORTED with this flag. */
#define NSN_RHT 4u

typedef struct {
  int32_t head_dim;   /* d: must be 128 */
  int32_t sub_dim;    /* m: 4 (2-bit codes) or 8 (1-bit codes) */
  int32_t n_codes;    /* K: must be 256 (one byte per code) */
  int32_t group_size; /* G: tokens per Shift group; 128 or 256 */
  uint32_t flags;     /* NSN_SCALE_ADJUST | NSN_DQ | NSN_RHT, or 0 */
  uint32_t rht_signs[4]; /* NSN_RHT channel signs (see there); ignored
                            without that flag */
} nsn_params;

/* Size in bytes of a prepared codebook for these params (codebook, squared
 * norms and search tables); constant for the supported shapes, 0 for
 * invalid or unsupported params. */
size_t nsn_table_size(const nsn_params* p);

/*
 * nsn_build_codebook -- Lloyd k-means codebook on standard-normal samples.
 * [NSNQuant summary §3, codebook construction: k-means over synthetic
 *  N(0,1) data, no calibration set; README, Overview.]
 *
 * samples   device, float64 [n_samples][sub_dim], row-major; the random
 *           N(0,1) draw is the caller's (any generator).
 * codebook  device, float32 [n_codes][sub_dim], written.
 * Steps: init = the first n_codes samples; `iters` times: assign every
 * sample to its nearest centroid (exact squared distance in float64, lowest
 * index on ties), then set each centroid to the mean of its members summed
 * in sample order (a centroid with no members keeps its value).  The final
 * centroids are rounded to the nearest fp16 value (ties to even) and stored
 * as float32.  Deterministic.
 * workspace device, >= nsn_build_codebook_workspace_size() bytes (the
 *           query returns 0 for arguments outside the requirements).
 * Requires n_codes == 256, sub_dim in {4, 8}, n_codes <= n_samples
 * <= 2^26, 1 <= iters <= 1000.
 */
size_t nsn_build_codebook_workspace_size(int32_t sub_dim, int32_t n_codes,
                                         int64_t n_samples);
nsn_status nsn_build_codebook(int32_t sub_dim, int32_t n_codes,
                              int64_t n_samples, int32_t iters,
                              const double* samples, float* codebook,
                              void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * nsn_tune_codebook -- fine-tune a codebook for cosine distance.
 * [NSNQuant summary §3, codebook construction: the k-means codebook is
 *  fine-tuned to minimize the cosine distance between the original and
 *  the quantized vectors, with no model involved; README, Codebook tuning.]
 *
 * The pages give the objective only; this call reads it as follows.
 * vectors   device, float64 [n_vec][128]: training vectors (the NSN +
 *           Hadamard output is standard normal, so N(0,1) draws; the
 *           caller's generator).  Each is split into 128/sub_dim contiguous
 *           sub-vectors, as the quantizer splits a token.
 * codebook  device, float32 [n_codes][sub_dim]: the start (e.g. the output
 *           of nsn_build_codebook) on entry, the tuned codebook on return,
 *           rounded to the nearest fp16 value (ties to even).
 * Each of `iters` iterations: assign every sub-vector its nearest codeword
 * (exact squared distance in float64, lowest index on ties); with that
 * assignment held fixed, take the gradient of the mean over vectors of
 * 1 - cos(h, h_hat), h_hat the concatenated codewords; one Adam step on the
 * whole batch (beta1 = 0.9, beta2 = 0.999, eps = 1e-8, bias-corrected
 * moments starting at zero, learning rate lr).  Float64, sums in a fixed
 * order: deterministic and reproducible bit for bit.  iters = 0 only
 * rounds.  The README's 2-bit "--abs" option is not described on the pages
 * and is not provided.
 * Requires sub_dim in {4, 8}, n_codes == 256 (else NSN_ERR_UNSUPPORTED),
 * 1 <= n_vec with n_vec*128/sub_dim <= 2^26, 0 <= iters <= 100000,
 * 0 < lr <= 1, 16-byte aligned non-NULL pointers (else
 * NSN_ERR_INVALID_ARG), workspace >= nsn_tune_codebook_workspace_size()
 * (else NSN_ERR_WORKSPACE; the size query returns 0 for invalid shapes).
 */
size_t nsn_tune_codebook_workspace_size(int32_t sub_dim, int32_t n_codes,
                                        int64_t n_vec);
nsn_status nsn_tune_codebook(int32_t sub_dim, int32_t n_codes, int64_t n_vec,
                             int32_t iters, double lr, const double* vectors,
                             float* codebook, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * nsn_prepare_codebook -- derive the device search tables from a codebook.
 * codebook  device, float32 [256][sub_dim]; entries must be finite with
 *           |c| <= 65504 (the fp16 range).
 * table     device, nsn_table_size(p) bytes, written; passed to every
 *           quantize / dequantize / attention call using this codebook.
 * Every entry is first rounded once: to the nearest fp16 value (ties to
 * even), or with NSN_DQ in p->flags to the 4-bit level given at that flag.
 * The table holds only the rounded codebook, and the search, the scale
 * adjustment, dequantization and attention all use it (a codebook from
 * nsn_build_codebook or nsn_tune_codebook is already fp16-valued and passes
 * unchanged).  A table is used with params of the same flags and sub_dim it
 * was prepared with; the table lives in device memory, so a mismatch is not
 * detected.
 * Returns NSN_ERR_WORKSPACE when table_bytes < nsn_table_size(p).
 */
nsn_status nsn_prepare_codebook(const nsn_params* p, const float* codebook,
                                void* table, size_t table_bytes,
                                void* stream);

/*
 * nsn_nearest_codeword -- index of the nearest codeword of each of n
 * arbitrary sub-vectors, through the same search the quantizer uses.
 * [NSNQuant summary §3: each rotated sub-vector is replaced by its nearest
 *  codeword in one global codebook.]
 * v      device float32 [n][sub_dim]; out device uint8 [n].
 * Nearest = smallest exact squared distance in float32, lowest index among
 * equal distances.  Requires 0 <= n <= 2^32 - 256 (else
 * NSN_ERR_UNSUPPORTED).
 */
nsn_status nsn_nearest_codeword(const nsn_params* p, const void* table,
                                const float* v, int64_t n, uint8_t* out,
                                void* stream);

/*
 * nsn_quantize -- compress whole token groups.
 * [NSNQuant summary §1 (Normalize, Shift over the group, Normalize),
 *  §2 (Hadamard rotation), §3 (nearest codeword, scale adjustment),
 *  §4 (a full residual is quantized and appended).]
 *
 * x       device, [n_seq][n_tok][128] of in_dtype (fp16 or fp32); tokens of
 *         one sequence are contiguous (row stride 128 elements), sequences
 *         `x_seq_stride` elements apart.  A "sequence" is one (batch, layer,
 *         head) of K or of V; any leading dims are flattened into n_seq.
 * n_tok   multiple of group_size (only whole groups are quantized); 0 is a
 *         no-op.
 * Outputs (device; token t of sequence s):
 *   codes  uint8 at codes + s*codes_seq_stride + t*(128/m) + j, j < 128/m:
 *          the code of sub-vector j = rotated channels [m*j, m*j+m).
 *   meta   fp16 pair at meta + s*meta_seq_stride + 2*t: (s1, s2'), where
 *          s1 = ||x_t||/sqrt(128) and s2' = s2 * alpha (alpha = 1 without
 *          NSN_SCALE_ADJUST).
 *   shift  fp16 [128] at shift + s*shift_seq_stride + (t/G)*128: the group's
 *          channel mean o, stored rotated (H o / sqrt(128); with NSN_RHT
 *          H D o / sqrt(128), and the codes likewise index the sub-vectors
 *          of the randomized rotation).
 *   With NSN_DQ, meta and shift hold the layouts given at that flag; the
 *   strides are then at least n_tok and (n_tok/128)*68 (multiples of 8 and
 *   4), and in_dtype must be NSN_F16.
 * Strides let a flush write into a preallocated cache at a group offset:
 * pass pointers advanced to the offset and the cache's sequence strides.
 * At most 2^24 - 1 token groups (n_seq * n_tok / group_size) per call, else
 * NSN_ERR_UNSUPPORTED (one launch covers the call).
 */
nsn_status nsn_quantize(const nsn_params* p, nsn_dtype in_dtype,
                        const void* x, int64_t n_seq, int64_t n_tok,
                        int64_t x_seq_stride, const void* table,
                        uint8_t* codes, int64_t codes_seq_stride,
                        uint16_t* meta, int64_t meta_seq_stride,
                        uint16_t* shift, int64_t shift_seq_stride,
                        void* stream);

/*
 * nsn_dequantize -- reconstruct tokens from codes and stored byproducts.
 * [NSNQuant summary §1 (the byproducts reconstruct the tensor), §4
 *  (dequantization kernels).]
 * x_hat_t = (H/sqrt(128)) [ s1 (s2' c(codes_t) + o'_g) ] (with NSN_RHT
 * D H/sqrt(128) [...]), the stored fp16 values taken as exact.  Layouts as
 * nsn_quantize; output x_hat
 * [n_seq][n_tok][128] of out_dtype, sequences out_seq_stride elements apart.
 * n_tok must be a multiple of group_size; at most 2^24 - 1 token groups per
 * call, as for nsn_quantize.
 */
nsn_status nsn_dequantize(const nsn_params* p, const uint8_t* codes,
                          int64_t codes_seq_stride, const uint16_t* meta,
                          int64_t meta_seq_stride, const uint16_t* shift,
                          int64_t shift_seq_stride, const void* table,
                          int64_t n_seq, int64_t n_tok, nsn_dtype out_dtype,
                          void* x_hat, int64_t out_seq_stride, void* stream);

/*
 * nsn_residual_append -- write one new fp16 token per sequence into the
 * full-precision residual window at position `pos`.
 * [NSNQuant summary §4: recent tokens stay in full precision until the
 *  residual is full, then it is quantized and appended to the cache.]
 * tok    device fp16 [n_seq][128] (contiguous).
 * resid  device fp16, token t of sequence s at resid + s*resid_seq_stride
 *        + t*128; requires 0 <= pos < resid_capacity.
 * n_seq above 2^28 - 16 (one launch) returns NSN_ERR_UNSUPPORTED.
 */
nsn_status nsn_residual_append(const uint16_t* tok, int64_t n_seq,
                               uint16_t* resid, int64_t resid_seq_stride,
                               int64_t resid_capacity, int64_t pos,
                               void* stream);

typedef struct {
  int32_t batch;          /* B, at most 65535 (else NSN_ERR_UNSUPPORTED) */
  int32_t n_q_heads;      /* Hq, a multiple of n_kv_heads; Hkv * Hq at most
                             2^20 and Hkv * ceil(Hq / Hkv / 4) at most 65535
                             (else NSN_ERR_UNSUPPORTED) */
  int32_t n_kv_heads;     /* Hkv; q head h reads kv head h / (Hq/Hkv) */
  int32_t n_quant_tok;    /* quantized tokens per (b, kv head); multiple of G */
  int32_t n_resid_tok;    /* valid fp16 residual tokens, 0..resid_capacity */
  int64_t cache_capacity; /* token slots per (b, kv head) in the code/meta
                             arrays; multiple of G, >= n_quant_tok */
  int64_t resid_capacity; /* token slots per (b, kv head) in the residual */
  float softmax_scale;    /* e.g. 1/sqrt(128) */
} nsn_attn_shape;

/*
 * nsn_decode_attention -- one query token per (batch, q head) attends over
 * its kv head's quantized cache plus the fp16 residual window.
 * [NSNQuant summary §4: quantized part plus full-precision residual; the
 *  score uses the NSN byproducts s1, s2, o directly.]
 *
 * With q' = H q / sqrt(128), on quantized token t of group g:
 *   score_t = scale * s1_t * (s2'_t <q', c(codes_t)> + <q', o'_g>)
 * and on residual token r: score_r = scale * <q, k_r>.  Softmax over all
 * n_quant_tok + n_resid_tok scores (float32, max-subtracted); values are
 * the dequantized V tokens and the residual V tokens.  No mask, no RoPE.
 * With NSN_RHT, q' = H D q / sqrt(128) and the values dequantize through
 * D H / sqrt(128) (the caches must have been quantized with the same signs).
 *
 * q        device fp16 [B][Hq][128].
 * k_codes, v_codes   device uint8 [B][Hkv][cache_capacity][128/m].
 * k_meta,  v_meta    device fp16  [B][Hkv][cache_capacity][2]
 *                    (NSN_DQ: [B][Hkv][cache_capacity], s2' only).
 * k_shift, v_shift   device fp16  [B][Hkv][cache_capacity/G][128]
 *                    (NSN_DQ: uint16 [B][Hkv][cache_capacity/128][68], the
 *                    group records).
 * k_resid, v_resid   device fp16  [B][Hkv][resid_capacity][128].
 * workspace          device, >= nsn_decode_attention_workspace_size() for
 *                    this shape.  The size is non-decreasing in n_quant_tok,
 *                    so a workspace sized for a cache's capacity (n_quant_tok
 *                    = cache_capacity, same batch and heads) serves every
 *                    fill level of that cache, with or without rotary keys.
 * out      device fp32 [B][Hq][128].
 * Requires n_quant_tok + n_resid_tok >= 1.
 */
size_t nsn_decode_attention_workspace_size(const nsn_params* p,
                                           const nsn_attn_shape* s);
nsn_status nsn_decode_attention(const nsn_params* p, const nsn_attn_shape* s,
                                const uint16_t* q, const uint8_t* k_codes,
                                const uint16_t* k_meta, const uint16_t* k_shift,
                                const uint8_t* v_codes, const uint16_t* v_meta,
                                const uint16_t* v_shift, const uint16_t* k_resid,
                                const uint16_t* v_resid, const void* table,
                                void* workspace, size_t workspace_bytes,
                                float* out, void* stream);

/*
 * nsn_decode_attention_rope -- nsn_decode_attention for keys stored before
 * rotary position embedding.
 * [NSNQuant summary §4: for keys, NSN is applied before RoPE; the score
 *  still takes the NSN byproducts.]
 *
 * The pages fix neither the RoPE form, its base nor the positions.  This
 * call uses the rotate-half form: for i < 64 the channel pair (i, i + 64)
 * of a vector at position pos turns by the angle pos * base^(-i/64)
 * ((x, y) -> (x cos - y sin, y cos + x sin)).  Quantized key t of a (b, kv
 * head) row sits at position t, residual key r at n_quant_tok + r, the
 * query at rope->q_pos; the query and every key are turned before the dot
 * product (the query arrives un-rotated, like the keys).  Values are
 * unchanged.  Everything else -- arguments, layouts, workspace size (the
 * same nsn_decode_attention_workspace_size()), ordering and errors -- is as
 * for nsn_decode_attention.
 *
 * rope     host; base finite and > 1, 0 <= q_pos <= 2^40, else
 *          NSN_ERR_INVALID_ARG.  With NSN_DQ the cache holds the
 *          double-quantized layout, as for nsn_decode_attention.
 */
typedef struct {
  int64_t q_pos;   /* position of the query token */
  float base;      /* rotary base, e.g. 10000 */
} nsn_rope;
nsn_status nsn_decode_attention_rope(const nsn_params* p, const nsn_attn_shape* s,
                                     const nsn_rope* rope, const uint16_t* q,
                                     const uint8_t* k_codes, const uint16_t* k_meta,
                                     const uint16_t* k_shift, const uint8_t* v_codes,
                                     const uint16_t* v_meta, const uint16_t* v_shift,
                                     const uint16_t* k_resid, const uint16_t* v_resid,
                                     const void* table, void* workspace, size_t workspace_bytes,
                                     float* out, void* stream);

/*
 * nsn_decode_attention_noalloc -- nsn_decode_attention without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * The split partials go to a static device array of the library, 4 MiB
 * (4194304 bytes) per GPU, held from the first call on that GPU until the
 * process ends.  Shapes whose nsn_decode_attention_workspace_size() exceeds
 * that return NSN_ERR_UNSUPPORTED (use nsn_decode_attention); the decode
 * workload B = 16, 32 q heads on 8 kv heads needs 1.9 MB at any cache
 * length.  Nothing is allocated or freed, by the library or any library it
 * calls.  Every call on one GPU shares that GPU's array (nothing in it needs
 * to start at zero: every partial is written before it is read), so calls
 * that overlap on one GPU -- on different streams, or from different
 * threads -- race and must be serialized by the caller.  Arguments, layouts,
 * results and errors are otherwise those of nsn_decode_attention, and the
 * output equals its output for the same inputs.
 */
nsn_status nsn_decode_attention_noalloc(const nsn_params* p, const nsn_attn_shape* s,
                                        const uint16_t* q, const uint8_t* k_codes,
                                        const uint16_t* k_meta, const uint16_t* k_shift,
                                        const uint8_t* v_codes, const uint16_t* v_meta,
                                        const uint16_t* v_shift, const uint16_t* k_resid,
                                        const uint16_t* v_resid, const void* table,
                                        float* out, void* stream);

/* Static description of a status code. */
const char* nsn_status_string(nsn_status s);
/* Detail of the last error returned on the calling thread ("" if none). */
const char* nsn_last_error(void);
/* Library version string. */
const char* nsn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* NSN_H */
