// Host-side checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code only: every entry point that
// validates or lays out on the host (status strings, shape checks, workspace
// layouts over a sweep of shapes, argument checks before any device work) is
// called; a sanitizer report or a wrong status ends the program with a non-zero
// exit code.  No device work is done, so no GPU is needed.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/latentmoe.h"
#include "../../include/ssm_replay.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static latentmoe_config cfg(int d, int l, int n, int k, int m, int ms, int T, int ef = 0, int sf = 0, int pf = 0) {
  latentmoe_config c;
  std::memset(&c, 0, sizeof c);
  c.d = d; c.latent = l; c.n_experts = n; c.top_k = k; c.expert_hidden = m; c.shared_hidden = ms;
  c.max_tokens = T; c.expert_format = ef; c.shared_format = sf; c.proj_format = pf;
  return c;
}

int main() {
  for (int st = -6; st <= 1; ++st) EXPECT(latentmoe_status_string(st) != nullptr);
  EXPECT(std::strcmp(latentmoe_status_string(0), "ok") == 0);

  // workspace layouts over shapes and formats, every T class the plans use
  const int Ts[] = {1, 7, 16, 17, 33, 64, 65, 255, 256, 1100, 8192};
  const int shapes[][6] = {{256, 64, 16, 4, 128, 256}, {4096, 1024, 512, 22, 2688, 5376},
                           {8192, 2048, 512, 22, 5120, 10240}, {512, 128, 1024, 64, 192, 320},
                           {256, 64, 16, 1, 64, 64}, {208, 80, 32, 4, 112, 144},
                           {256, 64, 4096, 64, 128, 256}};
  for (const auto& sh : shapes)
    for (int T : Ts)
      for (int ef = 0; ef < 2; ++ef)
        for (int sf = 0; sf < 2; ++sf)
          for (int pf = 0; pf <= 2; pf += 2) {
            latentmoe_config c = cfg(sh[0], sh[1], sh[2], sh[3], sh[4], sh[5], T, ef, sf, pf);
            size_t n = 0;
            EXPECT(latentmoe_workspace_bytes(&c, &n) == LATENTMOE_OK);
            EXPECT(n > 0);
          }
  // rejected shapes and formats
  size_t n = 0;
  latentmoe_config bad[] = {cfg(250, 64, 16, 4, 128, 256, 8), cfg(256, 64, 16, 17, 128, 256, 8),
                            cfg(256, 64, 20, 4, 128, 256, 8), cfg(256, 64, 4112, 4, 128, 256, 8),
                            cfg(256, 64, 128, 65, 128, 256, 8), cfg(256, 64, 16, 4, 128, 256, 8, 7),
                            cfg(256, 64, 16, 4, 128, 256, 8, 0, 2), cfg(256, 64, 16, 4, 128, 256, 8, 0, 0, 1),
                            cfg(4096, 1024, 512, 22, 2688, 5376, 36315), cfg(200, 64, 16, 4, 128, 256, 8),
                            cfg(256, 64, 16, 4, 120, 256, 8)};
  for (auto& c : bad) EXPECT(latentmoe_workspace_bytes(&c, &n) == LATENTMOE_ERR_UNSUPPORTED);
  latentmoe_config zero = cfg(256, 64, 16, 4, 128, 256, 0);
  EXPECT(latentmoe_workspace_bytes(&zero, &n) == LATENTMOE_ERR_INVALID_ARG);
  EXPECT(latentmoe_workspace_bytes(nullptr, &n) == LATENTMOE_ERR_INVALID_ARG);
  latentmoe_config ok = cfg(256, 64, 16, 4, 128, 256, 8);
  EXPECT(latentmoe_workspace_bytes(&ok, nullptr) == LATENTMOE_ERR_INVALID_ARG);

  // argument checks that return before any device work
  latentmoe_weights w;
  std::memset(&w, 0, sizeof w);
  latentmoe_handle_t h = reinterpret_cast<latentmoe_handle_t>(0x1);
  EXPECT(latentmoe_init(&ok, &w, nullptr, &h) == LATENTMOE_ERR_INVALID_ARG);
  EXPECT(h == nullptr);
  EXPECT(latentmoe_init(&ok, &w, nullptr, nullptr) == LATENTMOE_ERR_INVALID_ARG);
  EXPECT(latentmoe_forward(nullptr, nullptr, 1, nullptr, nullptr, nullptr, nullptr) == LATENTMOE_ERR_INVALID_ARG);
  EXPECT(latentmoe_forward_graph(nullptr, nullptr, 1, nullptr, nullptr, nullptr, nullptr) ==
         LATENTMOE_ERR_INVALID_ARG);
  EXPECT(latentmoe_destroy(nullptr) == LATENTMOE_OK);
  EXPECT(latentmoe_debug_copy(nullptr, 0, nullptr, 0, nullptr) == LATENTMOE_ERR_INVALID_ARG);
  EXPECT(latentmoe_profile_begin(nullptr, 1, 1) == LATENTMOE_ERR_INVALID_ARG);
  EXPECT(latentmoe_fp4_decode(nullptr, nullptr, 1, nullptr, nullptr) == LATENTMOE_ERR_INVALID_ARG);
  EXPECT(latentmoe_fp8_decode(nullptr, 1, nullptr, nullptr) == LATENTMOE_ERR_INVALID_ARG);
  EXPECT(latentmoe_forward_static(nullptr, &w, nullptr, 1, nullptr, nullptr, nullptr, nullptr) ==
         LATENTMOE_ERR_INVALID_ARG);
  EXPECT(latentmoe_forward_static(&ok, &w, nullptr, 1, nullptr, nullptr, nullptr, nullptr) ==
         LATENTMOE_ERR_INVALID_ARG);
  latentmoe_config fp4 = cfg(256, 64, 16, 4, 128, 256, 8, 1);
  EXPECT(latentmoe_forward_static(&fp4, &w, nullptr, 1, nullptr, nullptr, nullptr, nullptr) ==
         LATENTMOE_ERR_UNSUPPORTED);

  // Mamba verify shapes
  for (int P : {32, 64, 128})
    for (int N : {64, 96, 128})
      for (int cap : {1, 16, 32, 33}) {
        ssm_shape s{128, 8, P, N, cap};
        const int st = ssm_check_shape(&s);
        const bool supported = (P == 64 || P == 128) && (N == 64 || N == 128) && cap <= 32;
        EXPECT((st == SSM_OK) == supported);
      }
  ssm_shape s{128, 8, 64, 128, 16};
  EXPECT(ssm_replay_verify(&s, 1, 17, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                           nullptr, nullptr, nullptr) == SSM_ERR_INVALID_ARG);
  EXPECT(ssm_check_shape(nullptr) == SSM_ERR_INVALID_ARG);

  if (failures) {
    std::fprintf(stderr, "%d host checks failed\n", failures);
    return 1;
  }
  std::printf("host checks ok\n");
  return 0;
}
