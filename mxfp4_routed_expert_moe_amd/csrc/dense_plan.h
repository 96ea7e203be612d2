// Launch plan of the decode-width dense FP8 linear (dense.hip): plain host C++ with no HIP types, so that
// host tests can check it over every admitted shape.
#pragma once

#include <stddef.h>

#include <algorithm>

namespace moe {

constexpr int kDenseBlocks = 1024;       // blocks the K split aims for
constexpr int kDenseMinSteps = 4;        // fewest K steps per run when K is split
constexpr int kDenseLdsBudget = 49152;   // dynamic LDS bytes a block may take

// The K steps (128 wide) are split into `runs` runs of `steps_per_run` (one block column per run); lds =
// dynamic LDS bytes per block. runs > 1 needs fp32 partials [runs, M, N]. For M in [1, 64], N and K
// multiples of 128: lds <= kDenseLdsBudget, runs * steps_per_run >= K / 128 and no run is empty.
struct DensePlan {
  int runs;
  int steps_per_run;
  size_t lds;
};

inline size_t dense_run_lds(int M, int steps) { return (size_t)M * steps * 132 + 2 * (size_t)steps * 4; }

inline DensePlan dense_plan(int M, int N, int K) {
  const int nk = K / 128, cols = N / 64;
  const int m16 = ((M + 15) / 16) * 16;
  // LDS of one run: activation codes and scales of the M rows plus two weight-scale rows
  const int max_steps = std::max(1, kDenseLdsBudget / (m16 * 132 + 8));
  int runs = std::max(1, std::min(nk, (kDenseBlocks + cols - 1) / cols));
  // a block per CU already and the whole K fits in one run's LDS: no split, so no second launch
  // (wq_b, 16384 x 1280 at M = 8: 8.4 us against 10.5 us in three runs)
  if (cols >= 256 && nk <= max_steps) runs = 1;
  int spr = (nk + runs - 1) / runs;
  if (runs > 1) spr = std::max(spr, kDenseMinSteps);
  // the LDS cap holds for every plan, also where the block count alone asked for one run
  spr = std::min(std::min(spr, nk), max_steps);
  DensePlan pl{};
  pl.runs = (nk + spr - 1) / spr;
  pl.steps_per_run = spr;
  pl.lds = dense_run_lds(M, spr);
  return pl;
}

}  // namespace moe
