// Host-only driver of the bit-allocation search (ddg_pd_allocate), built by
// tests/test_host_sanitizers.py with the host code under ThreadSanitizer or
// AddressSanitizer + UndefinedBehaviorSanitizer.  The search runs its restarts
// on host threads that share read-only tables and write one result slot each;
// this driver calls it on a synthetic 40-tensor table at several targets and
// checks that every allocation keeps its budget.  No GPU call is made.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "ddg.h"

int main() {
  const int n = 40, nc = 5, restarts = 16, iters = 200;
  const int cand[nc] = {3, 4, 5, 6, 7};
  std::vector<double> sse((size_t)n * nc), tinit((size_t)restarts * n);
  std::vector<int64_t> nparams(n);
  unsigned state = 12345u;
  auto uniform = [&]() {                                   // a small LCG: values in [0, 1)
    state = state * 1103515245u + 12345u;
    return (double)((state >> 8) & 0xFFFF) / 65536.0;
  };
  for (int i = 0; i < n; ++i) {
    nparams[i] = 1000 + (int64_t)(uniform() * 100000.0);
    double e = (0.5 + uniform()) * (double)nparams[i];   // error sums falling with the width
    for (int c = 0; c < nc; ++c) {
      sse[(size_t)i * nc + c] = e;
      e *= 0.25 + 0.05 * uniform();
    }
  }
  for (double& t : tinit) t = (uniform() - 0.5) * 4.0;
  std::vector<int> bits(n);
  double info[3];
  for (double target : {3.0, 4.0, 4.5, 5.0, 6.5, 7.0}) {
    const int st = ddg_pd_allocate(sse.data(), nparams.data(), n, cand, nc, target, tinit.data(),
                                   restarts, iters, bits.data(), info);
    if (st != DDG_OK) {
      std::printf("ddg_pd_allocate returned %d at target %.1f\n", st, target);
      return 1;
    }
    double p = 0.0, tot = 0.0;
    for (int i = 0; i < n; ++i) {
      p += (double)nparams[i] * bits[i];
      tot += (double)nparams[i];
    }
    std::printf("target %.1f: %.4f bits per weight, restart %d kept\n", target, p / tot, (int)info[2]);
    if (p / tot > target + 1e-9) return 2;
  }
  // argument checks on the same threads' entry point
  if (ddg_pd_allocate(nullptr, nparams.data(), n, cand, nc, 4.0, tinit.data(), restarts, iters,
                      bits.data(), info) != DDG_ERR_ARG)
    return 3;
  return 0;
}
