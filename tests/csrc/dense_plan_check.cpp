// Host check of the decode-width dense linear's launch plan over every shape the C ABI admits for it
// (M in [1, 64], N and K multiples of 128 up to 65536): prints the first violation and exits 1, else prints
// the largest LDS request and exits 0.
#include <stdio.h>

#include "dense_plan.h"

int main() {
  size_t worst = 0;
  long long plans = 0;
  for (int M = 1; M <= 64; ++M)
    for (int N = 128; N <= 65536; N += 128)
      for (int K = 128; K <= 65536; K += 128) {
        const moe::DensePlan p = moe::dense_plan(M, N, K);
        const int nk = K / 128;
        const bool ok = p.runs >= 1 && p.steps_per_run >= 1 && p.steps_per_run <= nk &&
                        (long long)p.runs * p.steps_per_run >= nk && (long long)(p.runs - 1) * p.steps_per_run < nk &&
                        p.lds == moe::dense_run_lds(M, p.steps_per_run) && p.lds <= (size_t)moe::kDenseLdsBudget &&
                        p.runs <= 65535;
        if (!ok) {
          printf("bad plan M=%d N=%d K=%d: runs=%d steps=%d lds=%zu\n", M, N, K, p.runs, p.steps_per_run, p.lds);
          return 1;
        }
        if (p.lds > worst) worst = p.lds;
        ++plans;
      }
  printf("%lld plans, largest LDS %zu bytes\n", plans, worst);
  return 0;
}
