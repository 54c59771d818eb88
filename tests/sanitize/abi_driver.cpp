// Host-side driver for the sanitizer build of libh3x: every call here either fails validation
// (so nothing reaches the GPU) or only computes sizes, schedules and strings. Built and run
// with AddressSanitizer and UndefinedBehaviorSanitizer on the host code; a report or a wrong
// status ends the run with a non-zero exit code.
#include <cmath>
#include <cstdio>
#include <cstring>

#include "h3x.h"
#include "h3x_kernels.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "line %d: %s (%s)\n", __LINE__, #cond, h3x_last_error()); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

int main() {
  void* const F = reinterpret_cast<void*>(0x10000);  // never dereferenced: every call fails first
  const float* const Ff = static_cast<const float*>(F);
  h3x_block_cfg c = {512, 4, 128, 768, H3X_BF16, H3X_BF16, 1e-6f, 10000.f};
  h3x_block_cfg big = {6144, 48, 128, 24576, H3X_BF16, H3X_BF16, 1e-6f, 10000.f};
  h3x_geom g = {3, 8, 12, 30, 45, 0};
  h3x_geom g6912 = {6, 32, 32, 256, 512, 0};

  // Size queries (layouts computed without a workspace), every weight type and geometry.
  for (int wt : {H3X_BF16, H3X_I8, H3X_I8A8}) {
    h3x_block_cfg cw = big;
    cw.weight = wt;
    for (int merged : {0, 1}) {
      h3x_geom gg = g6912;
      gg.merged = merged;
      EXPECT(h3x_block_workspace_bytes(&cw, &gg) > 0);
    }
    EXPECT(h3x_step_workspace_bytes(&cw, &g6912) > h3x_block_workspace_bytes(&cw, &g6912));
    for (int k = 0; k < 4; ++k) EXPECT(h3x_packed_rows(&cw, k) > 0);
  }
  EXPECT(h3x_packed_weight_bytes(&big, H3X_W_GATE_UP, 2 * 24576, 6144) == size_t(2) * 24576 * 6144 * 2);
  EXPECT(h3x_packed_weight_bytes(&big, H3X_W_GATE_UP, 24576, 6144) == 0);
  EXPECT(h3x_packed_weight_bytes(&big, 7, 6144, 6144) == 0);
  EXPECT(h3x_geom_tokens(&g6912) == 6912);
  h3x_geom bad = {1, 3, 5, 0, 0, 1};
  EXPECT(h3x_geom_tokens(&bad) == -1);
  h3x_geom huge = {2147483647, 2147483647, 2147483647, 0, 0, 0};  // product beyond 64 bits
  EXPECT(h3x_geom_tokens(&huge) == -1);
  EXPECT(h3x_attention_workspace_bytes(&big, 6912, 0) == 0 || h3x_attention_workspace_bytes(&big, 6912, 256) > 0);
  EXPECT(h3x_rope_table_bytes(&big, &g6912) > 0);

  // Validation failures before any launch.
  const size_t need = h3x_block_workspace_bytes(&c, &g);
  h3x_block_weights w = {F, F, F, F, nullptr, nullptr, nullptr, nullptr};
  EXPECT(h3x_dit_block_forward(&c, &g, &w, Ff, F, F, need - 1, nullptr) == H3X_EWORKSPACE);
  EXPECT(h3x_dit_block_forward(nullptr, &g, &w, Ff, F, F, need, nullptr) == H3X_EINVAL);
  EXPECT(h3x_dit_block_forward(&c, nullptr, &w, Ff, F, F, need, nullptr) == H3X_EINVAL);
  EXPECT(h3x_dit_block_forward(&c, &g, nullptr, Ff, F, F, need, nullptr) == H3X_EINVAL);
  EXPECT(h3x_dit_block_forward_noalloc(&big, &g6912, &w, Ff, F, nullptr) == H3X_EWORKSPACE);
  h3x_block_cfg odd = c;
  odd.head_dim = 64;
  EXPECT(h3x_dit_block_forward(&odd, &g, &w, Ff, F, F, need, nullptr) == H3X_EINVAL);
  odd = c;
  odd.norm_eps = NAN;
  EXPECT(h3x_norm_mod(&odd, 4, F, Ff, Ff, F, nullptr) == H3X_EINVAL);
  EXPECT(h3x_pack_weights_bf16(&c, H3X_W_OUT, F, 512, 513, F, nullptr) == H3X_EINVAL);
  EXPECT(h3x_pack_int8_weights(&c, H3X_W_OUT, F, 512, 512, F, F, nullptr) == H3X_EINVAL);

  h3x_block_weights blocks[4] = {w, w, w, w};
  const size_t step_need = h3x_step_workspace_bytes(&c, &g);
  h3x_step st;
  std::memset(&st, 0, sizeof(st));
  st.step = 0; st.n_steps = 4; st.reuse = 1; st.sigma = 1.0f; st.sigma_next = 0.75f;
  st.n_blocks = 4; st.blocks = blocks; st.mod = Ff; st.tr_first = -1; st.tr_last = -1;
  float* z = static_cast<float*>(F);
  EXPECT(h3x_denoise_step(&c, &g, &st, z, F, F, F, step_need - 1, nullptr) == H3X_EWORKSPACE);
  st.tr_first = 1; st.tr_last = 2; st.core_reuse = 2; st.core_first = 0; st.core_last = 1;
  st.core_delta = z;
  EXPECT(h3x_denoise_step(&c, &g, &st, z, F, F, F, step_need, nullptr) == H3X_EINVAL);  // straddles
  st.core_first = 1; st.core_last = 2;
  EXPECT(h3x_denoise_step(&c, &g, &st, z, F, F, F, step_need - 1, nullptr) == H3X_EWORKSPACE);
  st.sigma = NAN;
  EXPECT(h3x_denoise_step(&c, &g, &st, z, F, F, F, step_need, nullptr) == H3X_EINVAL);

  // Schedules, fresh rule, strings.
  float sig[21];
  for (int kind = 0; kind < 3; ++kind) EXPECT(h3x_sigma_schedule(kind, 20, kind == 2 ? 29.0 : 2.0, sig) == H3X_OK);
  EXPECT(h3x_sigma_schedule(5, 20, 1.0, sig) == H3X_EINVAL);
  int fresh = 0;
  for (int i = 0; i < 20; ++i) fresh += h3x_step_is_fresh(i, 20, 2);
  EXPECT(fresh == 11);
  EXPECT(std::isnan(h3x_extrapolation_weight(0.5f, 0.6f, 0.6f)));
  for (int s = 0; s < 6; ++s) EXPECT(std::strlen(h3x_status_string(static_cast<h3x_status>(s))) > 0);
  EXPECT(h3x_abi_version() == H3X_ABI_VERSION);

  std::printf("abi driver: %d failure(s)\n", failures);
  return failures == 0 ? 0 : 1;
}
