// Contiguous, byte-balanced placement of a model's blocks over devices, each stage within its own
// device's budget (host only; see include/placement.h for the rule and its sources).
//
// A stage's requirement depends only on its block count and on whether it is first and/or last
// (blocks are alike), so stage_plan runs once per (count, first, last).  An exact dynamic program
// over cut positions then minimises the largest requirement / budget ratio:
//   best[i][c] = min over c' < c of max(best[i - 1][c'], ratio(device i - 1, blocks [c', c)))
// for i devices covering blocks [0, c), each with >= 1 block.
#include <cstring>
#include <vector>

#include "placement.h"

namespace {

// a / b as an exact fraction; "infinite" when the stage does not fit its device
struct Ratio {
  uint64_t num = 0, den = 1;
  bool inf = false;
};

bool less(const Ratio& x, const Ratio& y) {
  if (x.inf || y.inf) return !x.inf && y.inf;
  return (unsigned __int128)x.num * y.den < (unsigned __int128)y.num * x.den;
}

Ratio max_of(const Ratio& x, const Ratio& y) { return less(x, y) ? y : x; }

}  // namespace

extern "C" int stage_place(const stage_model_cfg* model, const stage_stage_cfg* shape, int n_devices,
                           const uint64_t* budgets, int32_t* cuts, uint64_t* required) {
  if (!model || !shape || !budgets || !cuts || n_devices <= 0) return STAGE_E_INVALID;
  const int L = model->n_blocks_total;
  if (L <= 0 || n_devices > L) return STAGE_E_INVALID;
  const int n = n_devices;

  // requirement of a stage of `len` blocks with the given endpoint flags, memoised
  std::vector<uint64_t> memo((size_t)4 * (L + 1), 0);
  std::vector<char> have((size_t)4 * (L + 1), 0);
  int plan_rc = STAGE_OK;
  auto need = [&](int len, bool first, bool last) -> uint64_t {
    const size_t key = (size_t)((first ? 1 : 0) | (last ? 2 : 0)) * (L + 1) + len;
    if (!have[key]) {
      stage_stage_cfg s = *shape;
      s.block_begin = first ? 0 : L - len;    // any range of `len` blocks; only the count matters
      s.block_end = s.block_begin + len;
      s.flags = (shape->flags & STAGE_KV_F32) | (first ? STAGE_FIRST : 0u) | (last ? STAGE_LAST : 0u);
      stage_plan_t p;
      const int rc = stage_plan(model, &s, &p);
      if (rc != STAGE_OK && plan_rc == STAGE_OK) plan_rc = rc;
      memo[key] = rc == STAGE_OK ? p.total_bytes : UINT64_MAX;
      have[key] = 1;
    }
    return memo[key];
  };
  auto ratio = [&](int dev, int len) {
    Ratio r;
    const uint64_t b = budgets[dev];
    const uint64_t q = need(len, dev == 0, dev == n - 1);
    if (q == UINT64_MAX || b == 0 || q > b) {
      r.inf = true;
    } else {
      r.num = q;
      r.den = b;
    }
    return r;
  };

  // best[i][c]: i devices cover blocks [0, c); from[i][c]: the cut before the last of them
  Ratio unreachable;
  unreachable.inf = true;
  std::vector<Ratio> best((size_t)(n + 1) * (L + 1), unreachable);
  std::vector<int> from((size_t)(n + 1) * (L + 1), -1);
  auto B = [&](int i, int c) -> Ratio& { return best[(size_t)i * (L + 1) + c]; };
  auto F = [&](int i, int c) -> int& { return from[(size_t)i * (L + 1) + c]; };
  B(0, 0) = Ratio{};
  F(0, 0) = 0;
  for (int i = 1; i <= n; ++i) {
    // device i - 1 ends at c; the last device must end at L, earlier ones leave a block per device
    const int c_lo = i, c_hi = (i == n) ? L : L - (n - i);
    for (int c = c_lo; c <= c_hi; ++c) {
      if (i == n && c != L) continue;
      for (int cp = i - 1; cp < c; ++cp) {
        if (F(i - 1, cp) < 0) continue;
        const Ratio prev = B(i - 1, cp);
        if (prev.inf) continue;
        const Ratio here = ratio(i - 1, c - cp);
        if (here.inf) continue;
        const Ratio cand = max_of(prev, here);
        if (F(i, c) < 0 || less(cand, B(i, c))) {
          B(i, c) = cand;
          F(i, c) = cp;
        }
      }
    }
  }
  if (plan_rc != STAGE_OK) return plan_rc;   // the stage configuration itself is refused
  if (F(n, L) < 0) return STAGE_E_DOES_NOT_FIT;
  std::vector<int32_t> cut(n + 1);
  cut[n] = L;
  for (int i = n; i >= 1; --i) cut[i - 1] = F(i, cut[i]);
  std::memcpy(cuts, cut.data(), sizeof(int32_t) * (n + 1));
  if (required)
    for (int i = 0; i < n; ++i) required[i] = need(cut[i + 1] - cut[i], i == 0, i == n - 1);
  return STAGE_OK;
}
