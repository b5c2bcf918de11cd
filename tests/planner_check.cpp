// Invariants of the prefill launch planner (dequant_gemm_q4_amd/csrc/plan.cpp),
// checked on the host over many groups of problems.  Built and run by
// tests/test_planner_cpu.py; prints one line per failure and "ok <plans>".
#include "plan.h"

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <utility>
#include <vector>

namespace dmq {
int device_cu_count() { return 256; }
}  // namespace dmq

using namespace dmq;

static int failures = 0;
#define CHECK(cond, ...)                      \
  do {                                        \
    if (!(cond)) {                            \
      ++failures;                             \
      std::printf("FAIL %s: ", #cond);        \
      std::printf(__VA_ARGS__);               \
      std::printf("\n");                      \
    }                                         \
  } while (0)

static GemmProblem P(int fmt, int swiglu, int M, int N, int K) {
  return GemmProblem{nullptr, nullptr, nullptr, fmt, swiglu, M, N, K, nullptr, 0.0f, nullptr};
}

static bool same(const Plan& a, const Plan& b) {
  if (a.jba != b.jba || a.jbb != b.jbb || a.nseg != b.nseg || a.fmt_mask != b.fmt_mask || a.swiglu != b.swiglu)
    return false;
  for (int i = 0; i < a.nseg; ++i)
    if (std::memcmp(&a.seg[i], &b.seg[i], sizeof(Seg)) != 0) return false;
  return true;
}

static void check(const char* name, const std::vector<GemmProblem>& ps) {
  const int count = (int)ps.size();
  const Plan pl = make_plan(ps.data(), count, 256);
  int mmax = 0, fmt_mask = 0;
  for (const auto& p : ps) {
    mmax = p.M > mmax ? p.M : mmax;
    fmt_mask |= 1 << p.fmt;
  }
  CHECK(pl.nseg >= count && pl.nseg <= GEMM_MAX_SEG, "%s: %d segments", name, pl.nseg);
  CHECK(pl.jba == 1 || pl.jba == 2 || pl.jba == 4 || pl.jba == 8, "%s: jba %d", name, pl.jba);
  CHECK(pl.jbb >= 1 && pl.jbb <= pl.jba, "%s: jbb %d jba %d", name, pl.jbb, pl.jba);
  CHECK(pl.jba == 1 || 32 * (pl.jba / 2) < mmax, "%s: tall height %d for M <= %d", name, 32 * pl.jba, mmax);
  CHECK(pl.fmt_mask == fmt_mask, "%s: format mask %d, want %d", name, pl.fmt_mask, fmt_mask);
  CHECK(pl.swiglu == (ps[0].swiglu != 0), "%s: SwiGLU flag", name);
  for (int i = 0; i < count; ++i) {
    const GemmProblem& p = ps[i];
    const int nb = p.K / 256, nt = n_tiles(p);
    // the problem's segments cover its n-tiles exactly once
    std::vector<int> cover(nt, 0);
    for (int s = 0; s < pl.nseg; ++s) {
      const Seg& sg = pl.seg[s];
      CHECK(sg.prob >= 0 && sg.prob < count, "%s: segment %d names problem %d", name, s, sg.prob);
      if (sg.prob != i) continue;
      CHECK(sg.nt >= 1 && sg.n_begin >= 0 && sg.n_begin + sg.nt <= nt, "%s: segment %d n-range [%d, %d) of %d", name,
            s, sg.n_begin, sg.n_begin + sg.nt, nt);
      for (int n = sg.n_begin; n < sg.n_begin + sg.nt && n < nt; ++n)
        if (n >= 0) ++cover[n];
      // K pieces: every piece non-empty, together exactly the K blocks
      CHECK(sg.ks >= 1 && sg.kbs >= 1 && (int64_t)(sg.ks - 1) * sg.kbs < nb && (int64_t)sg.ks * sg.kbs >= nb,
            "%s: segment %d splits %d blocks as %d x %d", name, s, nb, sg.ks, sg.kbs);
      CHECK(sg.ks == 1 || p.fmt == 0 || sg.kbs % 2 == 0, "%s: Q6_K pieces of %d blocks start on odd blocks", name,
            sg.kbs);
      CHECK(sg.ks == 1 || !p.swiglu, "%s: a SwiGLU problem split", name);
      CHECK(sg.ks == 1 || (double)sg.ks * p.M * (double)p.N * 4.0 <= (double)(512 << 20),
            "%s: partial sums of %d pieces exceed the workspace bound", name, sg.ks);
      CHECK(sg.alt == 0 || sg.alt == 1, "%s: height flag %d", name, sg.alt);
      CHECK(m_tiles(p, sg.alt ? pl.jbb : pl.jba) >= 1, "%s: no m-tiles", name);
    }
    for (int n = 0; n < nt; ++n) CHECK(cover[n] == 1, "%s: problem %d n-tile %d covered %d times", name, i, n, cover[n]);
  }
  // the same shapes give the same plan, from the cache too; and the plan is
  // no slower (in the simulation) than every problem unsplit at 32 rows
  CHECK(same(pl, make_plan(ps.data(), count, 256)), "%s: plan not deterministic", name);
  CHECK(same(pl, get_plan(ps.data(), count)), "%s: cached plan differs", name);
  CHECK(same(get_plan(ps.data(), count), get_plan(ps.data(), count)), "%s: cache lookups differ", name);
  // (the base plan orders its segments as the planner does: longest tiles
  // first, ties in problem order; a tile's time is one tile column's
  // simulated time on one CU divided by its tiles)
  std::vector<double> buf;
  std::vector<std::pair<double, int>> order;
  for (int i = 0; i < count; ++i) {
    Plan one;
    one.jba = one.jbb = 1;
    one.seg[one.nseg++] = Seg{i, 0, 0, 1, 1, ps[i].K / 256};
    order.push_back({simulate(one, ps.data(), 1, buf) / m_tiles(ps[i], 1), i});
  }
  std::stable_sort(order.begin(), order.end(), [](const std::pair<double, int>& a, const std::pair<double, int>& b) {
    return a.first > b.first;
  });
  Plan base;
  base.jba = base.jbb = 1;
  base.fmt_mask = fmt_mask;
  base.swiglu = ps[0].swiglu != 0;
  for (const auto& o : order) base.seg[base.nseg++] = Seg{o.second, 0, 0, n_tiles(ps[o.second]), 1, ps[o.second].K / 256};
  CHECK(simulate(pl, ps.data(), 256, buf) <= simulate(base, ps.data(), 256, buf) * (1.0 + 1e-9),
        "%s: plan simulated slower than the unsplit 32-row plan", name);
}

int main() {
  int plans = 0;
  char name[128];
  // one decoder layer's seven projections (Q|K|V|O|gate|up Q4_K, down Q6_K)
  for (int M : {2, 5, 16, 17, 33, 100, 256, 300, 1024, 2048, 4096, 8192}) {
    std::snprintf(name, sizeof name, "layer M=%d", M);
    check(name, {P(0, 0, M, 3072, 3072), P(0, 0, M, 1024, 3072), P(0, 0, M, 1024, 3072), P(0, 0, M, 3072, 3072),
                 P(0, 0, M, 8192, 3072), P(0, 0, M, 8192, 3072), P(1, 0, M, 3072, 8192)});
    ++plans;
  }
  // single projections, ragged sizes, deep and shallow K, both formats
  for (int fmt : {0, 1})
    for (int M : {2, 40, 129, 1024, 5000})
      for (int N : {16, 37, 250, 333, 3072, 128256})
        for (int K : {256, 768, 3072, 4864, 8192, 32768}) {
          if ((double)M * N > 2e8 || (double)N * K > 2e9) continue;
          std::snprintf(name, sizeof name, "fmt%d M=%d N=%d K=%d", fmt, M, N, K);
          check(name, {P(fmt, 0, M, N, K)});
          ++plans;
        }
  // SwiGLU gate|up pairs (run alone)
  for (int M : {2, 16, 300, 1024, 4096})
    for (int F : {256, 1024, 8192}) {
      std::snprintf(name, sizeof name, "swiglu M=%d F=%d", M, F);
      check(name, {P(0, 1, M, 2 * F, 3072)});
      ++plans;
    }
  // mixed groups of up to eight problems with different K
  check("mixed 8", {P(0, 0, 700, 1000, 3072), P(1, 0, 700, 37, 8192), P(0, 0, 700, 4096, 256),
                    P(1, 0, 700, 512, 4864), P(0, 0, 700, 96, 768), P(0, 0, 700, 3072, 3072),
                    P(1, 0, 700, 2048, 2048), P(0, 0, 700, 16, 32768)});
  check("LM head", {P(1, 0, 1024, 128256, 3072)});
  check("wide split bound", {P(1, 0, 65536, 3072, 8192)});
  plans += 3;
  std::printf("ok %d plans, %d failures\n", plans, failures);
  return failures == 0 ? 0 : 1;
}
