// Driver for the host-side library code (codebooks, seeded matrices, status
// strings, argument checks) built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py.  It prints
// every result with 17 significant digits so that the test can compare them
// with the shipped library's.
#include <cstdio>
#include <vector>

#include "tq.h"

static void put(const char *tag, const std::vector<double> &v) {
  std::printf("%s", tag);
  for (double x : v) std::printf(" %.17g", x);
  std::printf("\n");
}

int main() {
  int bad = 0;
  const int cb[][2] = {{3, 1}, {3, 3}, {16, 2}, {64, 2}, {128, 3}, {256, 4}};
  for (const auto &c : cb) {
    const int k = 1 << c[1];
    std::vector<double> cen(k), bnd(k - 1), mse(1);
    if (tq_make_codebook(c[0], c[1], cen.data(), bnd.data(), mse.data()) != TQ_OK) ++bad;
    char tag[64];
    std::snprintf(tag, sizeof tag, "codebook %d %d", c[0], c[1]);
    cen.insert(cen.end(), bnd.begin(), bnd.end());
    cen.push_back(mse[0]);
    put(tag, cen);
  }
  for (int d : {2, 3, 64, 128}) {
    for (int kind = 0; kind < 3; ++kind) {
      std::vector<double> m((size_t)d * d);
      if (tq_make_rotation(d, 7, kind, m.data()) != TQ_OK) ++bad;
      char tag[64];
      std::snprintf(tag, sizeof tag, "rotation %d %d", d, kind);
      put(tag, std::vector<double>(m.begin(), m.begin() + (d < 4 ? d * d : 8)));
    }
  }
  for (int d : {64, 256}) {
    int lv = 0;
    while ((1 << lv) < d) ++lv;
    std::vector<double> c(4 * (lv - 1)), t(3 * (lv - 1));
    if (tq_make_polar_codebook(d, c.data(), t.data()) != TQ_OK) ++bad;
    char tag[64];
    std::snprintf(tag, sizeof tag, "polar %d", d);
    c.insert(c.end(), t.begin(), t.end());
    put(tag, c);
  }
  // argument checks: every one refused, nothing written
  double buf[16];
  if (tq_make_codebook(2, 2, buf, buf, nullptr) != TQ_ERR_INVALID) ++bad;
  if (tq_make_codebook(128, 9, buf, buf, nullptr) != TQ_ERR_INVALID) ++bad;
  if (tq_make_codebook(128, 2, nullptr, buf, nullptr) != TQ_ERR_INVALID) ++bad;
  if (tq_make_rotation(1, 0, 0, buf) != TQ_ERR_INVALID) ++bad;
  if (tq_make_rotation(4, 0, 3, buf) != TQ_ERR_INVALID) ++bad;
  if (tq_make_rotation(4, 0, 0, nullptr) != TQ_ERR_INVALID) ++bad;
  if (tq_make_polar_codebook(96, buf, buf) != TQ_ERR_INVALID) ++bad;
  if (tq_make_polar_codebook(32, buf, buf) != TQ_ERR_INVALID) ++bad;
  for (int s = -5; s <= 0; ++s) std::printf("status %d %s\n", s, tq_status_string(s));
  std::printf("bad %d\n", bad);
  return bad == 0 ? 0 : 1;
}
