// Host-only driver for the sanitizer test (tests/test_host_sanitizers.py):
// plan creation, queries and destruction in a loop, malformed irreps strings,
// the dense CG builder for every (l1, l2, l3) up to 4, and the argument errors
// of the launch entry points, which return before any HIP call.  Built with
// AddressSanitizer (leak checking on) and UndefinedBehaviorSanitizer over the
// C ABI's host code; exits 0 when every check holds.
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>
#include "tpconv.h"
static int fails = 0;
#define CHECK(c) do { if (!(c)) { std::printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c); ++fails; } } while (0)
int main() {
  const char* good[][1] = {{"8x0e+8x1o"}, {"32x0e+32x1o+32x2e"}, {"64x0e+64x1o+64x2e+64x3o"}};
  const int ls[] = {2, 2, 3};
  for (int round = 0; round < 50; ++round)
    for (int g = 0; g < 3; ++g) {
      tp_plan_t p = nullptr;
      CHECK(tp_conv_plan_create(&p, good[g][0], ls[g], ls[g], 0, nullptr) == 0 && p);
      int32_t P, U, xd, ysh, od, nnz;
      char out_irr[256];
      CHECK(tp_conv_plan_info(p, &P, &U, &xd, &ysh, &od, &nnz, out_irr, sizeof(out_irr)) == 0);
      std::vector<int32_t> paths(4 * P);
      CHECK(tp_conv_plan_paths(p, paths.data()) == 0);
      std::vector<int16_t> abc(4 * nnz);
      std::vector<double> val(nnz);
      CHECK(tp_conv_plan_cg(p, abc.data(), val.data()) == 0);
      char tiny[4];
      tp_conv_plan_info(p, &P, &U, &xd, &ysh, &od, &nnz, tiny, sizeof(tiny));   // short buffer: truncated or error
      size_t b = 0;
      tp_conv_fc_workspace(p, 100, 8, &b);
      tp_conv_fc_backward_workspace(p, 100, 8, &b);
      tp_conv_radial_workspace(p, 100, 1, &b);
      tp_conv_uvw_workspace(p, &b);
      tp_conv_plan_destroy(p);
      tp_plan_t q = nullptr;
      if (tp_conv_plan_create(&q, good[g][0], ls[g] < 2 ? ls[g] : 2, ls[g] < 2 ? ls[g] : 2, 1, nullptr) == 0) {
        int32_t o, w, pts;
        CHECK(tp_conv_gaunt_dims(q, &o, &w, &pts) == 0);
        tp_conv_plan_destroy(q);
      }
    }
  const char* bad[] = {"", "x", "32x0e+16x1o", "32x9e", "32x1e", "0x0e", "-4x0e", "32x0e+", "+", "32x0q",
                       "99999999999x0e", "32x0e+32x1o+32x2e+32x3o+32x4e+32x5o+32x6e+32x7o+32x8e", "32X0E"};
  for (const char* s : bad) {
    tp_plan_t p = nullptr;
    const tp_status st = tp_conv_plan_create(&p, s, 2, 2, 0, nullptr);
    CHECK(st < 0 && p == nullptr);
    CHECK(std::strlen(tp_conv_last_error()) > 0);
  }
  std::string longs(100000, '1');
  { tp_plan_t p = nullptr; CHECK(tp_conv_plan_create(&p, longs.c_str(), 2, 2, 0, nullptr) < 0); }
  { tp_plan_t p = nullptr; CHECK(tp_conv_plan_create(&p, nullptr, 2, 2, 0, nullptr) < 0); }
  CHECK(tp_conv_plan_create(nullptr, "8x0e", 2, 2, 0, nullptr) < 0);
  { tp_plan_t p = nullptr; CHECK(tp_conv_plan_create(&p, "8x0e", -1, 2, 0, nullptr) < 0); }
  { tp_plan_t p = nullptr; CHECK(tp_conv_plan_create(&p, "8x0e", 2, 2, 7, nullptr) < 0); }
  std::vector<double> cg(9 * 9 * 9);
  for (int l1 = 0; l1 <= 4; ++l1)
    for (int l2 = 0; l2 <= 4; ++l2)
      for (int l3 = 0; l3 <= 4; ++l3) {
        std::vector<double> o((2 * l1 + 1) * (2 * l2 + 1) * (2 * l3 + 1));
        tp_cg_real(l1, l2, l3, o.data());
      }
  CHECK(tp_cg_real(-1, 0, 0, cg.data()) < 0);
  size_t ws = 0;
  CHECK(tp_conv_graph_workspace(-1, 5, &ws) < 0);
  CHECK(tp_conv_graph_workspace(5, -1, &ws) < 0);
  tp_conv_graph_workspace(2147483647, 2147483647, &ws);
  CHECK(tp_conv_forward(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) < 0);
  tp_plan_t p = nullptr;
  tp_conv_plan_create(&p, "32x0e+32x1o+32x2e", 2, 2, 0, nullptr);
  CHECK(tp_conv_forward(p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) < 0);
  tp_graph g{};
  g.n_nodes = -3;
  CHECK(tp_conv_forward(p, &g, nullptr, nullptr, nullptr, nullptr, nullptr) < 0);
  CHECK(tp_conv_backward(p, &g, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) < 0);
  tp_conv_plan_destroy(p);
  tp_conv_plan_destroy(nullptr);
  std::printf("%s (%d failures)\n", fails ? "FAILED" : "OK", fails);
  return fails ? 1 : 0;
}
