// Stepwise AllReduce schedules that run as descriptor steps (k_gsteps):
// tree, double binary tree, 2-port ring, and halving-doubling / butterfly for
// N not a power of two.  Host-side only.
#pragma once

#include <stdint.h>

#include <vector>

#include "cc_launch.h"

namespace cc {

enum SchedAlg { SCHED_TREE, SCHED_DBT, SCHED_RING2, SCHED_HD_PAIRS, SCHED_BFLY_PAIRS };

struct Plan {
  // what the kernels run: per step, descriptors with disjoint destinations
  // and no descriptor reading what another of the same step writes
  std::vector<std::vector<GDesc>> steps;
  // the simulated network: values each rank sends, and the number of steps
  std::vector<uint64_t> sent;
  int net_steps = 0;
};

// N >= 2; M elements per rank.
Plan build_plan(SchedAlg alg, int N, uint64_t M);

// the two complementary trees (children lists, left first) and their tops
struct Trees {
  std::vector<std::vector<int>> ch[2];
  int top[2];
};
Trees dbt_trees(int N);

}  // namespace cc
