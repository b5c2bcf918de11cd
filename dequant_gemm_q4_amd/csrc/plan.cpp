// Launch planner of the prefill GEMM (host code; the kernels are in
// gemm.hip).
//
// Workgroups hold one CU each (the LDS of one tile exceeds half a CU's) and
// the dispatcher hands them to CUs in index order as CUs fall free, so a
// launch is a greedy list schedule of its tiles.  When the tiles do not
// fill whole rounds, or a long-K problem's tiles outlast the rest, CUs idle
// at the end of the launch.  The plan picks, per group of problems, the tile
// height pair (tall, short), which height each problem uses, and how many of
// the last problem's n-tile columns to run at the short height, by
// simulating that schedule with per-tile times measured on gfx950.

#include "plan.h"

#include <algorithm>
#include <cstring>
#include <mutex>
#include <utility>
#include <vector>

namespace dmq {

// Time of one tile in shader cycles, measured on MI355X (timestamps of every
// workgroup in launches full of tiles): a fixed part (prologue, first block,
// epilogue) plus a part per 256-wide K block, per format and tile height.
static double tile_cost(int fmt, int jb, int nb) {
  static const double a4[4] = {5000, 7700, 14300, 27600}, b4[4] = {5700, 6500, 8430, 12800};
  static const double a6[4] = {8000, 9000, 17300, 30600}, b6[4] = {9400, 11100, 14000, 17550};
  const int i = jb == 1 ? 0 : jb == 2 ? 1 : jb == 4 ? 2 : 3;
  return fmt == 0 ? a4[i] + b4[i] * nb : a6[i] + b6[i] * nb;
}

int m_tiles(const GemmProblem& p, int jb) { return (p.M + 32 * jb - 1) / (32 * jb); }
int n_tiles(const GemmProblem& p) {
  return p.swiglu ? (p.N / 2 + 127) / 128 : (p.N + 255) / 256;   // SwiGLU: 128 gate + 128 up rows per tile
}

// Time of the split-K combine (shader cycles, as tile_cost): a launch plus
// reading ks partial slices and writing y at about 5.5 TB/s.
static double reduce_cost(const Plan& pl, const GemmProblem* probs) {
  double bytes = 0.0;
  bool any = false;
  for (int i = 0; i < pl.nseg; ++i) {
    const Seg& sg = pl.seg[i];
    if (sg.ks == 1) continue;
    any = true;
    bytes += 4.0 * (sg.ks + 1) * probs[sg.prob].M * (double)probs[sg.prob].N;
  }
  return any ? 4000.0 + bytes / 2900.0 : 0.0;
}

// Greedy dispatch of the segments' tiles, in order, over ncu CUs (plus the
// split-K combine): the time the last CU falls idle.  The tiles of one
// segment cost the same, so the CU free times they produce come out in
// increasing order: a sorted array plus a FIFO replace a heap.
double simulate(const Plan& pl, const GemmProblem* probs, int ncu, std::vector<double>& buf) {
  buf.assign(3 * (size_t)ncu, 0.0);
  double* cur = buf.data();              // sorted free times of the CUs not yet used by this segment
  double* fifo = buf.data() + ncu;       // ring of free times produced by this segment
  double* tmp = buf.data() + 2 * ncu;
  for (int i = 0; i < pl.nseg; ++i) {
    const Seg& sg = pl.seg[i];
    const GemmProblem& p = probs[sg.prob];
    const int jb = sg.alt ? pl.jbb : pl.jba;
    const double c = tile_cost(p.fmt, jb, sg.kbs);
    const int64_t n = (int64_t)m_tiles(p, jb) * sg.nt * sg.ks;
    int a = 0, head = 0, len = 0;
    for (int64_t t = 0; t < n; ++t) {
      double f;
      if (len > 0 && (a == ncu || fifo[head] < cur[a])) {
        f = fifo[head];
        head = head + 1 == ncu ? 0 : head + 1;
        --len;
      } else {
        f = cur[a++];
      }
      int tail = head + len;
      fifo[tail >= ncu ? tail - ncu : tail] = f + c;
      ++len;
    }
    // merge the untouched CUs with the segment's output (both sorted)
    int o = 0;
    while (a < ncu || len > 0) {
      if (len > 0 && (a == ncu || fifo[head] < cur[a])) {
        tmp[o++] = fifo[head];
        head = head + 1 == ncu ? 0 : head + 1;
        --len;
      } else {
        tmp[o++] = cur[a++];
      }
    }
    std::copy(tmp, tmp + ncu, cur);
  }
  return cur[ncu - 1] + reduce_cost(pl, probs);
}

// Piece length in K blocks for a split into about ks pieces (Q6_K pieces
// start on even blocks, keeping the weight rows' 4-byte alignment).
static int piece_blocks(const GemmProblem& p, int ks) {
  const int nb = p.K / QK;
  int kbs = (nb + ks - 1) / ks;
  if (p.fmt == 1 && (kbs & 1) && kbs < nb) ++kbs;
  return kbs;
}

Plan make_plan(const GemmProblem* probs, int count, int ncu) {
  int mmax = 0, kmax = 0, fmt_mask = 0;
  for (int i = 0; i < count; ++i) {
    mmax = probs[i].M > mmax ? probs[i].M : mmax;
    kmax = probs[i].K > kmax ? probs[i].K : kmax;
    fmt_mask |= 1 << probs[i].fmt;
  }
  const bool swiglu = probs[0].swiglu != 0;
  static const int pairs[5][2] = {{8, 4}, {8, 2}, {4, 2}, {2, 1}, {1, 1}};
  static const int splits[8] = {1, 2, 3, 4, 6, 8, 12, 16};
  std::vector<double> heap;

  // Phase 1: tile heights, which problems run short tiles, and the split of
  // the deepest-K problems; no tail.
  struct Cand {
    Plan pl;
    double t;
  };
  std::vector<Cand> cands;
  for (const auto& hp : pairs) {
    const int jba = hp[0], jbb = hp[1];
    if (jba > 1 && 32 * (jba / 2) >= mmax) continue;   // taller than needed
    // which problems run short tiles: none, Q6_K ones (mixed groups), all
    for (int short_set = 0; short_set < 3; ++short_set) {
      if (jba == jbb && short_set) break;
      if (short_set == 1 && fmt_mask != 3) continue;
      for (int ks : splits) {
        if (ks > 1 && (swiglu || ks > kmax / QK)) break;
        Plan pl;
        pl.jba = jba;
        pl.jbb = jbb;
        pl.fmt_mask = fmt_mask;
        pl.swiglu = swiglu;
        bool ok = true;
        int order[GEMM_MAX_GROUP];
        Seg sg[GEMM_MAX_GROUP];
        for (int i = 0; i < count; ++i) {
          const GemmProblem& p = probs[i];
          const int alt = short_set == 2 || (short_set == 1 && p.fmt == 1) ? 1 : 0;
          const int kbs = p.K == kmax ? piece_blocks(p, ks) : p.K / QK;
          const int pks = (p.K / QK + kbs - 1) / kbs;
          // the partial sums must fit a bounded workspace
          if (pks > 1 && (double)pks * p.M * (double)p.N * 4.0 > (double)(512 << 20)) ok = false;
          sg[i] = Seg{i, alt, 0, n_tiles(p), pks, kbs};
          order[i] = i;
        }
        if (!ok) continue;
        // longest tiles first
        auto cost_of = [&](int i) { return tile_cost(probs[i].fmt, sg[i].alt ? jbb : jba, sg[i].kbs); };
        std::stable_sort(order, order + count, [&](int a, int b) { return cost_of(a) > cost_of(b); });
        for (int i = 0; i < count; ++i) pl.seg[pl.nseg++] = sg[order[i]];
        cands.push_back(Cand{pl, simulate(pl, probs, ncu, heap)});
      }
    }
  }
  std::stable_sort(cands.begin(), cands.end(), [](const Cand& a, const Cand& b) { return a.t < b.t; });

  // Phase 2, for every candidate within 25% of the best: the last k n-tile
  // columns of the last tall, unsplit segment at the short height.
  Plan best = cands[0].pl;
  double best_t = cands[0].t;
  for (const Cand& cd : cands) {
    if (cd.t > 1.25 * cands[0].t) break;
    const Plan& pl = cd.pl;
    const Seg last = pl.seg[pl.nseg - 1];
    const int kmx = (pl.jba != pl.jbb && !last.alt && last.ks == 1) ? last.nt : 0;
    const int kstep = kmx > 32 ? (kmx + 31) / 32 : 1;
    for (int k = kstep; k <= kmx; k += kstep) {
      Plan q = pl;
      q.seg[q.nseg - 1].nt = last.nt - k;
      q.seg[q.nseg++] = Seg{last.prob, 1, last.nt - k, k, 1, last.kbs};
      if (k == last.nt) q.seg[q.nseg - 2] = q.seg[q.nseg - 1], --q.nseg;
      const double t = simulate(q, probs, ncu, heap);
      if (t < best_t * 0.995) {
        best_t = t;
        best = q;
      }
    }
  }
  return best;
}

// Plans are cached by the problems' shapes (a serving loop repeats a few).
struct PlanKey {
  int count;
  int32_t shape[GEMM_MAX_GROUP][5];
  bool operator==(const PlanKey& o) const {
    return count == o.count && std::memcmp(shape, o.shape, sizeof(int32_t) * 5 * count) == 0;
  }
};

Plan get_plan(const GemmProblem* probs, int count) {
  static std::mutex mu;
  static std::vector<std::pair<PlanKey, Plan>> cache;
  PlanKey key{};
  key.count = count;
  for (int i = 0; i < count; ++i) {
    const GemmProblem& p = probs[i];
    key.shape[i][0] = p.fmt;
    key.shape[i][1] = p.swiglu;
    key.shape[i][2] = p.M;
    key.shape[i][3] = p.N;
    key.shape[i][4] = p.K;
  }
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& e : cache)
    if (e.first == key) return e.second;
  Plan pl = make_plan(probs, count, device_cu_count());
  if (cache.size() >= 256) cache.erase(cache.begin());
  cache.emplace_back(key, pl);
  return pl;
}

}  // namespace dmq
