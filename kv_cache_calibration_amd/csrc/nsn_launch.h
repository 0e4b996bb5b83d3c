// Host-side launchers of the NSNQuant kernels.  Arguments are validated by
// the C ABI layer (nsn_api.hip) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nsn {

// Double-quantized group record (G = 128): 8 header bytes, 64 bytes of o'
// codes, 64 bytes of s1 codes, in uint16 units.
constexpr int kDqRecU16 = 68;

// Channel signs of the randomized rotation (bit c = channel c negated before
// the Hadamard transform); all zero for the plain rotation.  Passed to the
// kernels by value.
struct RhtSigns {
  uint32_t w[4];
};

struct QuantArgs {
  const void* x;
  int in_f32;
  int64_t n_seq, n_tok, x_seq_stride;
  const void* table;
  uint8_t* codes;
  int64_t codes_seq_stride;
  uint16_t* meta;
  int64_t meta_seq_stride;
  uint16_t* shift;
  int64_t shift_seq_stride;
  int sub_dim, group_size, scale_adjust;
  int dq;   // 1: double-quantized metadata (meta = s2' per token, shift = group records)
  RhtSigns rht;
};
hipError_t launch_quantize(const QuantArgs& a, hipStream_t s);
bool quantize_mfma_supported(int in_f32, int sub_dim, int group_size);
hipError_t launch_quantize_mfma(const QuantArgs& a, hipStream_t s);
hipError_t launch_search_table(void* table, hipStream_t s);
hipError_t launch_nearest(const void* table, int sub_dim, const float* v, int64_t n, uint8_t* out,
                          hipStream_t s);

struct DequantArgs {
  const uint8_t* codes;
  int64_t codes_seq_stride;
  const uint16_t* meta;
  int64_t meta_seq_stride;
  const uint16_t* shift;
  int64_t shift_seq_stride;
  const void* table;
  int64_t n_seq, n_tok;
  int out_f32;
  void* out;
  int64_t out_seq_stride;
  int sub_dim, group_size;
  int dq;   // 1: double-quantized metadata
  RhtSigns rht;
};
hipError_t launch_dequantize(const DequantArgs& a, hipStream_t s);

hipError_t launch_prepare_codebook(const float* codebook, int sub_dim, int dq,
                                   void* table, hipStream_t s);

hipError_t launch_build_codebook(int sub_dim, int n_codes, int64_t n,
                                 int iters, const double* samples,
                                 float* codebook, void* workspace,
                                 hipStream_t s);
size_t build_codebook_workspace(int sub_dim, int n_codes, int64_t n);
hipError_t launch_tune_codebook(int sub_dim, int64_t n_vec, int iters, double lr,
                                const double* vectors, float* codebook, void* workspace,
                                hipStream_t s);
size_t tune_codebook_workspace(int sub_dim, int64_t n_vec);

hipError_t launch_residual_append(const uint16_t* tok, int64_t n_seq,
                                  uint16_t* resid, int64_t resid_seq_stride,
                                  int64_t pos, hipStream_t s);

struct AttnArgs {
  int B, Hq, Hkv, n_quant, n_resid;
  int64_t cap, rcap;
  float scale;
  int sub_dim, group_size;
  const uint16_t* q;
  const uint8_t *kc, *vc;
  const uint16_t *km, *vm, *ks, *vs, *kr, *vr;
  const void* table;
  float* work;
  float* out;
  int n_split;   // chunks per (b, kv-head block)
  int chunk;     // quantized tokens per chunk (multiple of group_size)
  int rope;          // 1: keys are stored before rotary embedding
  float rope_base;   // rotary base (rope = 1)
  int64_t q_pos;     // query position (rope = 1)
  int dq;            // 1: double-quantized metadata (group_size 128)
  RhtSigns rht;      // randomized rotation's signs (rope = 0 only)
};
// Split choice of one launch: chunks of whole groups, the last one shortened
// for the residual window its workgroup also takes (n_resid); the rotary
// kernel (rope = 1) aims at fewer workgroups per CU.  Never above
// attn_split_bound, which sizes the workspace.
void attn_plan(int B, int Hq, int Hkv, int n_quant, int n_resid, int group_size, int rope,
               int* n_split, int* chunk);
// Upper bound of the split count over both plans and every quantized-token
// count in [0, n_quant]; non-decreasing in n_quant.  The workspace size the
// library asks for and checks.
int attn_split_bound(int B, int Hq, int Hkv, int n_quant);
size_t attn_workspace_bytes(int B, int Hq, int n_split);
hipError_t launch_decode_attention(const AttnArgs& a, hipStream_t s);

}  // namespace nsn
