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
  // hierarchical schedules: values each rank sends at each level
  std::vector<std::vector<uint64_t>> level_sent;
};

// Hierarchical AllReduce over dims (level 0 innermost, rank r = r_0 +
// p_0 (r_1 + p_1 (...))): standalone ring ReduceScatters inside the groups of
// levels 0 .. d-2, a ring AllReduce inside the outermost groups, ring
// AllGathers back.  Levels of size 1 do nothing (with an outermost level of
// size 1 no AllReduce runs); prod(dims) >= 2.  level_sent is indexed by the
// levels of size > 1.
Plan build_hier_plan(const std::vector<int>& dims, uint64_t M);

// The non-trivial levels of dims: their sizes and rank strides.
void hier_levels(const std::vector<int>& dims, std::vector<int>* p, std::vector<int>* stride);

// N >= 2; M elements per rank.
Plan build_plan(SchedAlg alg, int N, uint64_t M);

// the two complementary trees (children lists, left first) and their tops
struct Trees {
  std::vector<std::vector<int>> ch[2];
  int top[2];
};
Trees dbt_trees(int N);

}  // namespace cc
