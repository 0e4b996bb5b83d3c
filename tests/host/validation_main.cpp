// Host-side driver of the C ABI's argument validation, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code (see
// tests/test_host_sanitizers.py).  Every call here fails validation, so no
// device memory is touched and nothing is launched; fake device pointers are
// never dereferenced.  With no HIP device visible, one call with valid
// arguments also exercises the failed-launch path (NSN_ERR_HIP).
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "nsn.h"

static int g_fail = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::printf("FAILED line %d: %s (last error: %s)\n", __LINE__, #cond, \
                  nsn_last_error());                                   \
      ++g_fail;                                                        \
    }                                                                  \
  } while (0)

int main(int argc, char** argv) {
  const bool no_device = argc > 1 && std::strcmp(argv[1], "--no-device") == 0;
  void* F = reinterpret_cast<void*>(uintptr_t(0x10000));     // aligned, never dereferenced
  void* MIS = reinterpret_cast<void*>(uintptr_t(0x10004));
  uint8_t* F8 = static_cast<uint8_t*>(F);
  uint16_t* F16 = static_cast<uint16_t*>(F);
  nsn_params p{128, 4, 256, 128, NSN_SCALE_ADJUST};
  nsn_params bad = p;

  // status strings, version
  for (int s = 0; s <= 5; ++s) EXPECT(std::strlen(nsn_status_string(static_cast<nsn_status>(s))) > 0);
  EXPECT(std::strcmp(nsn_status_string(static_cast<nsn_status>(77)), "unknown status") == 0);
  EXPECT(std::strncmp(nsn_version(), "nsnq", 4) == 0);

  // params
  EXPECT(nsn_quantize(nullptr, NSN_F16, F, 1, 128, 0, F, F8, 0, F16, 0, F16, 0, nullptr) == NSN_ERR_INVALID_ARG);
  bad.head_dim = 64;
  EXPECT(nsn_quantize(&bad, NSN_F16, F, 1, 128, 0, F, F8, 0, F16, 0, F16, 0, nullptr) == NSN_ERR_UNSUPPORTED);
  bad = p;
  bad.flags = 0x80;
  EXPECT(nsn_quantize(&bad, NSN_F16, F, 1, 128, 0, F, F8, 0, F16, 0, F16, 0, nullptr) == NSN_ERR_INVALID_ARG);
  // a long error message is truncated, not overflowed
  EXPECT(nsn_quantize(&p, NSN_F16, F, 1, 100, 0, F, F8, 0, F16, 0, F16, 0, nullptr) == NSN_ERR_INVALID_ARG);
  EXPECT(std::strlen(nsn_last_error()) < 512);

  // quantize / dequantize
  EXPECT(nsn_quantize(&p, static_cast<nsn_dtype>(7), F, 1, 128, 0, F, F8, 0, F16, 0, F16, 0, nullptr) == NSN_ERR_INVALID_ARG);
  EXPECT(nsn_quantize(&p, NSN_F16, nullptr, 1, 128, 0, F, F8, 0, F16, 0, F16, 0, nullptr) == NSN_ERR_INVALID_ARG);
  EXPECT(nsn_quantize(&p, NSN_F16, MIS, 1, 128, 0, F, F8, 0, F16, 0, F16, 0, nullptr) == NSN_ERR_INVALID_ARG);
  EXPECT(nsn_quantize(&p, NSN_F16, F, 2, 128, 100, F, F8, 4096, F16, 256, F16, 128, nullptr) == NSN_ERR_INVALID_ARG);
  EXPECT(nsn_quantize(&p, NSN_F16, F, -1, 128, 0, F, F8, 0, F16, 0, F16, 0, nullptr) == NSN_ERR_INVALID_ARG);
  EXPECT(nsn_quantize(&p, NSN_F16, F, 1, int64_t(1) << 40, 0, F, F8, 0, F16, 0, F16, 0, nullptr) == NSN_ERR_UNSUPPORTED);
  EXPECT(nsn_quantize(&p, NSN_F16, F, 0, 128, 0, F, F8, 0, F16, 0, F16, 0, nullptr) == NSN_OK);
  EXPECT(nsn_dequantize(&p, F8, 0, F16, 0, F16, 0, F, 1, 200, NSN_F32, F, 0, nullptr) == NSN_ERR_INVALID_ARG);
  EXPECT(nsn_dequantize(&p, F8, 0, F16, 0, F16, 0, nullptr, 1, 128, NSN_F32, F, 0, nullptr) == NSN_ERR_INVALID_ARG);
  {
    nsn_params dq = p;
    dq.flags |= NSN_DQ;
    EXPECT(nsn_quantize(&dq, NSN_F32, F, 1, 128, 0, F, F8, 0, F16, 0, F16, 0, nullptr) == NSN_ERR_UNSUPPORTED);
    dq.group_size = 256;
    EXPECT(nsn_quantize(&dq, NSN_F16, F, 1, 256, 0, F, F8, 0, F16, 0, F16, 0, nullptr) == NSN_ERR_UNSUPPORTED);
  }

  // codebook calls
  EXPECT(nsn_build_codebook_workspace_size(3, 256, 1000) == 0);
  EXPECT(nsn_build_codebook(4, 256, 100, 20, static_cast<const double*>(F), static_cast<float*>(F), F, 1 << 20, nullptr) == NSN_ERR_INVALID_ARG);
  EXPECT(nsn_tune_codebook(4, 256, 10, 5, 0.0, static_cast<const double*>(F), static_cast<float*>(F), F, 1 << 20, nullptr) == NSN_ERR_INVALID_ARG);
  EXPECT(nsn_prepare_codebook(&p, static_cast<const float*>(F), F, 16, nullptr) == NSN_ERR_WORKSPACE);
  EXPECT(nsn_table_size(&p) > 0);
  EXPECT(nsn_table_size(nullptr) == 0);
  EXPECT(nsn_nearest_codeword(&p, F, static_cast<const float*>(F), -1, F8, nullptr) == NSN_ERR_INVALID_ARG);
  EXPECT(nsn_nearest_codeword(&p, F, static_cast<const float*>(F), (int64_t(1) << 32), F8, nullptr) == NSN_ERR_UNSUPPORTED);
  EXPECT(nsn_residual_append(F16, 1, F16, 0, 4, 4, nullptr) == NSN_ERR_INVALID_ARG);

  // attention
  nsn_attn_shape s{2, 8, 2, 1024, 16, 1024, 16, 0.0884f};
  const size_t ws = nsn_decode_attention_workspace_size(&p, &s);
  EXPECT(ws > 0);
  EXPECT(nsn_decode_attention(&p, &s, F16, F8, F16, F16, F8, F16, F16, F16, F16, F, F, ws - 1,
                              static_cast<float*>(F), nullptr) == NSN_ERR_WORKSPACE);
  nsn_attn_shape s2 = s;
  s2.n_q_heads = 7;
  EXPECT(nsn_decode_attention_workspace_size(&p, &s2) == 0);
  EXPECT(nsn_decode_attention(&p, &s2, F16, F8, F16, F16, F8, F16, F16, F16, F16, F, F, ws,
                              static_cast<float*>(F), nullptr) == NSN_ERR_INVALID_ARG);
  nsn_rope r{10, 1.0f};
  EXPECT(nsn_decode_attention_rope(&p, &s, &r, F16, F8, F16, F16, F8, F16, F16, F16, F16, F, F, ws,
                                   static_cast<float*>(F), nullptr) == NSN_ERR_INVALID_ARG);
  // monotone workspace over every fill level of one capacity
  {
    nsn_attn_shape c{1, 32, 8, 0, 1, 65536, 1, 0.0884f};
    size_t prev = 0;
    for (int n = 0; n <= 65536; n += 128) {
      c.n_quant_tok = n;
      const size_t w = nsn_decode_attention_workspace_size(&p, &c);
      EXPECT(w >= prev);
      prev = w;
    }
  }

  if (no_device) {
    EXPECT(nsn_residual_append(F16, 1, F16, 0, 4, 0, nullptr) == NSN_ERR_HIP);
    EXPECT(std::strstr(nsn_last_error(), "launch") != nullptr);
  }
  std::printf("%s: %d failure(s)\n", g_fail ? "FAILED" : "ok", g_fail);
  return g_fail ? 1 : 0;
}
