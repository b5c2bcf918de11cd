// Launch plan of the prefill GEMM (plan.cpp, host code): which tile heights,
// segments, split-K pieces and tail a grouped launch of gemm.hip runs.
#pragma once

#include "dmq_common.h"

#include <vector>

namespace dmq {

constexpr int GEMM_MAX_GROUP = 8;                  // problems per launch
constexpr int GEMM_MAX_SEG = 2 * GEMM_MAX_GROUP;   // segments per launch

// One segment of a launch: n-tiles [n_begin, n_begin + nt) of problem prob,
// all at the kernel's tall (alt = 0) or short (alt = 1) tile height, with K
// split into ks pieces of kbs super-blocks each (ks = 1: unsplit).
struct Seg {
  int prob, alt, n_begin, nt, ks, kbs;
};
// A launch: the tall and short heights in units of 32 activation rows, the
// segments in dispatch order, the formats present (bit 0 Q4_K, bit 1 Q6_K)
// and whether the problem is a SwiGLU gate|up pair.
struct Plan {
  int jba = 1, jbb = 1, nseg = 0, fmt_mask = 0;
  bool swiglu = false;
  Seg seg[GEMM_MAX_SEG];
};

// Tiles of a problem along M at height jb (32*jb rows) and along N (256
// weight rows; SwiGLU pairs: 128 gate + 128 up rows).
int m_tiles(const GemmProblem& p, int jb);
int n_tiles(const GemmProblem& p);
// The plan for these problems (count <= GEMM_MAX_GROUP) on ncu compute units.
Plan make_plan(const GemmProblem* probs, int count, int ncu);
// make_plan for the current device, cached by the problems' shapes.
Plan get_plan(const GemmProblem* probs, int count);
// Simulated time of a plan in shader cycles (the greedy dispatch of its
// tiles over ncu CUs, plus the split-K combine); buf is scratch.
double simulate(const Plan& pl, const GemmProblem* probs, int ncu, std::vector<double>& buf);

}  // namespace dmq
