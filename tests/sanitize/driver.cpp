// Argument paths of the C ABI under the address and undefined-behaviour
// sanitizers: every entry point with null, negative, oversized or otherwise
// invalid arguments must return its documented error code. Exits non-zero on
// the first mismatch (the sanitizers abort on their own findings).
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "tri_attn.h"

static int failures = 0;
#define EXPECT(call, code)                                                              \
  do {                                                                                  \
    const int rc_ = (call);                                                             \
    if (rc_ != (code)) {                                                                \
      std::fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, \
                   #call, rc_, (int)(code));                                            \
      ++failures;                                                                       \
    }                                                                                   \
  } while (0)

int main() {
  for (int c = -12; c <= 2; ++c)
    if (!tri_attn_strerror(c) || !std::strlen(tri_attn_strerror(c))) ++failures;

  float host[4] = {0.f, 0.f, 0.f, 0.f};
  tri_attn_weights w;
  w.ln_weight = w.ln_bias = w.w_query = w.w_key = w.w_value = host;
  w.w_gate = w.b_gate = w.w_bias_proj = w.w_out = w.b_out = host;
  tri_attn_config ok = {128, 4, TRI_ATTN_F32, 1e-5f, -1e9f, 0};
  tri_attn_t h = nullptr;

  // create: null arguments and every invalid config field
  EXPECT(tri_attn_create(&ok, &w, nullptr, nullptr), TRI_ATTN_ERR_INVALID_ARG);
  EXPECT(tri_attn_create(nullptr, &w, nullptr, &h), TRI_ATTN_ERR_INVALID_ARG);
  EXPECT(tri_attn_create(&ok, nullptr, nullptr, &h), TRI_ATTN_ERR_INVALID_ARG);
  tri_attn_weights wn = w;
  wn.b_out = nullptr;
  EXPECT(tri_attn_create(&ok, &wn, nullptr, &h), TRI_ATTN_ERR_INVALID_ARG);
  struct Bad {
    tri_attn_config c;
    int code;
  } bad[] = {
      {{0, 4, TRI_ATTN_F32, 1e-5f, -1e9f, 0}, TRI_ATTN_ERR_INVALID_ARG},
      {{-128, 4, TRI_ATTN_F32, 1e-5f, -1e9f, 0}, TRI_ATTN_ERR_INVALID_ARG},
      {{128, 0, TRI_ATTN_F32, 1e-5f, -1e9f, 0}, TRI_ATTN_ERR_INVALID_ARG},
      {{128, -4, TRI_ATTN_F32, 1e-5f, -1e9f, 0}, TRI_ATTN_ERR_INVALID_ARG},
      {{128, 3, TRI_ATTN_F32, 1e-5f, -1e9f, 0}, TRI_ATTN_ERR_INVALID_ARG},
      {{128, 4, 7, 1e-5f, -1e9f, 0}, TRI_ATTN_ERR_INVALID_ARG},
      {{128, 4, TRI_ATTN_F32, 0.f, -1e9f, 0}, TRI_ATTN_ERR_INVALID_ARG},
      {{128, 4, TRI_ATTN_F32, -1e-5f, -1e9f, 0}, TRI_ATTN_ERR_INVALID_ARG},
      {{128, 4, TRI_ATTN_F32, NAN, -1e9f, 0}, TRI_ATTN_ERR_INVALID_ARG},
      {{128, 4, TRI_ATTN_F32, INFINITY, -1e9f, 0}, TRI_ATTN_ERR_INVALID_ARG},
      {{128, 4, TRI_ATTN_F32, 1e-5f, NAN, 0}, TRI_ATTN_ERR_INVALID_ARG},
      {{128, 4, TRI_ATTN_F32, 1e-5f, 1.f, 0}, TRI_ATTN_ERR_INVALID_ARG},
      {{128, 4, TRI_ATTN_F32, 1e-5f, -1.f, 0}, TRI_ATTN_ERR_INVALID_ARG},
      {{128, 4, TRI_ATTN_F32, 1e-5f, INFINITY, 0}, TRI_ATTN_ERR_INVALID_ARG},
      {{128, 4, TRI_ATTN_F32, 1e-5f, -1e9f, 2}, TRI_ATTN_ERR_INVALID_ARG},
      {{128, 4, TRI_ATTN_F32, 1e-5f, -1e9f, -1}, TRI_ATTN_ERR_INVALID_ARG},
      {{256, 8, TRI_ATTN_F32, 1e-5f, -1e9f, 0}, TRI_ATTN_ERR_UNSUPPORTED},
      {{128, 2, TRI_ATTN_BF16, 1e-5f, -1e9f, 0}, TRI_ATTN_ERR_UNSUPPORTED},
      {{96, 6, TRI_ATTN_BF16, 1e-5f, -1e9f, 0}, TRI_ATTN_ERR_UNSUPPORTED},
  };
  for (const Bad &b : bad) {
    h = reinterpret_cast<tri_attn_t>(&failures);  // must be reset to null
    EXPECT(tri_attn_create(&b.c, &w, nullptr, &h), b.code);
    if (h != nullptr) ++failures;
  }
  // a valid config on a machine without a GPU: the handle is built and freed
  // again when the runtime reports no device
  {
    const char *gpu = std::getenv("TRI_ATTN_EXPECT_NO_GPU");
    if (gpu && gpu[0] == '1') {
      h = nullptr;
      EXPECT(tri_attn_create(&ok, &w, nullptr, &h), TRI_ATTN_ERR_HIP);
      if (h != nullptr) ++failures;
    }
  }
  // fault-injection hook
  EXPECT(tri_attn_set_alloc_fault(-1), TRI_ATTN_ERR_INVALID_ARG);
  EXPECT(tri_attn_set_alloc_fault(0), TRI_ATTN_OK);

  // every entry point with a null handle
  size_t n = 0;
  tri_attn_workspace_layout lay;
  tri_attn_grads g;
  std::memset(&g, 0, sizeof(g));
  void *p = host;
  const unsigned char *m = reinterpret_cast<const unsigned char *>(host);
  EXPECT(tri_attn_workspace_size(nullptr, 1, 8, &n), TRI_ATTN_ERR_INVALID_ARG);
  EXPECT(tri_attn_workspace_size(nullptr, 1, 8, nullptr), TRI_ATTN_ERR_INVALID_ARG);
  EXPECT(tri_attn_get_workspace_layout(nullptr, 1, 8, &lay), TRI_ATTN_ERR_INVALID_ARG);
  EXPECT(tri_attn_get_workspace_layout(nullptr, 1, 8, nullptr), TRI_ATTN_ERR_INVALID_ARG);
  EXPECT(tri_attn_forward(nullptr, p, m, p, 1, 8, p, 1 << 20, nullptr), TRI_ATTN_ERR_INVALID_ARG);
  EXPECT(tri_attn_project(nullptr, p, m, 1, 8, p, 1 << 20, nullptr), TRI_ATTN_ERR_INVALID_ARG);
  EXPECT(tri_attn_attend(nullptr, 1, 8, p, 1 << 20, nullptr), TRI_ATTN_ERR_INVALID_ARG);
  EXPECT(tri_attn_output(nullptr, p, 1, 8, p, 1 << 20, nullptr), TRI_ATTN_ERR_INVALID_ARG);
  EXPECT(tri_attn_forward_train(nullptr, p, m, p, nullptr, 1, 8, 0.1, 1, 0, p, 1 << 20, nullptr),
         TRI_ATTN_ERR_INVALID_ARG);
  EXPECT(tri_attn_forward_train(nullptr, p, m, p, nullptr, 1, 8, NAN, 1, 0, p, 1 << 20, nullptr),
         TRI_ATTN_ERR_INVALID_ARG);
  EXPECT(tri_attn_backward_workspace_size(nullptr, 1, 8, &n), TRI_ATTN_ERR_INVALID_ARG);
  EXPECT(tri_attn_backward_workspace_size(nullptr, 1, 8, nullptr), TRI_ATTN_ERR_INVALID_ARG);
  EXPECT(tri_attn_backward_train(nullptr, p, m, p, 1, 8, 0.1, 1, 0, &g, p, 1 << 20, nullptr),
         TRI_ATTN_ERR_INVALID_ARG);
  EXPECT(tri_attn_backward_train(nullptr, p, m, p, 1, 8, 1.5, 1, 0, nullptr, p, 1 << 20, nullptr),
         TRI_ATTN_ERR_INVALID_ARG);
  EXPECT(tri_attn_onepass_workspace_size(nullptr, 1, 8, &n), TRI_ATTN_ERR_INVALID_ARG);
  EXPECT(tri_attn_onepass_workspace_size(nullptr, 1, 8, nullptr), TRI_ATTN_ERR_INVALID_ARG);
  EXPECT(tri_attn_forward_onepass(nullptr, p, m, p, 1, 8, p, 1 << 20, nullptr), TRI_ATTN_ERR_INVALID_ARG);
  EXPECT(tri_attn_forward_noalloc(nullptr, p, m, p, 1, 8, nullptr), TRI_ATTN_ERR_INVALID_ARG);
  EXPECT(tri_attn_set_shift_slack(nullptr, 1.f), TRI_ATTN_ERR_INVALID_ARG);
  EXPECT(tri_attn_set_backward_dz_ranges(nullptr, 2), TRI_ATTN_ERR_INVALID_ARG);
  EXPECT(tri_attn_destroy(nullptr), TRI_ATTN_OK);

  if (failures) std::fprintf(stderr, "%d failures\n", failures);
  else std::printf("argument paths: all codes as documented\n");
  return failures ? 1 : 0;
}
