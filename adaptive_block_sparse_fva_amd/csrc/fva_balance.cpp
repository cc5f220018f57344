// Runtime load balancing (RLB) plan search and slack-aware sparse
// augmentation (SASA) budgets, on the host.
//
// FVAttn paper S3.2: after routing, every rank knows every head's workload;
// a migration plan is a permutation sigma of the ranks in which rank r sends
// one of its heads to sigma(r) and receives one from sigma^-1(r) (Eq 5), and
// the plan minimises the largest rank load, then the load variance (Eq 6).
// The search is deterministic so that every rank computes the same plan.
// S3.3: slack to the critical rank (Eq 7) becomes a discounted block budget
// (Eq 8-9) where it exceeds a trigger; S3.3's gating picks no mechanism,
// SASA only, or RLB then SASA from the imbalance rho (Eq 2).
//
// Pairing topology: every involution sigma (disjoint rank pairs that swap one
// head each way) is enumerated.  For a fixed pairing the objective splits
// over the pairs: the smallest reachable maximum M is the larger of the
// unpaired loads and each pair's best pair-maximum, and given M each pair
// independently takes its lowest sum of squares among the swaps that keep
// both loads <= M.  A per-pair table of swaps sorted by pair-maximum with a
// running best makes that a binary search.
//
// Ring topology: sigma is the identity or r -> r+1 mod R with every rank
// sending one head; rank r's new load depends on its own choice and its
// predecessor's, so the best maximum is found by bisection over the candidate
// values with a reachability pass around the cycle, and the sum of squares by
// a dynamic programme around the cycle for each choice of rank 0's head.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

#include "fva.h"

namespace {

using i64 = int64_t;
constexpr i64 INF = std::numeric_limits<i64>::max();

struct Plan {
  i64 mx = INF, sq = INF;
  int moves = 0;
  std::vector<int32_t> sigma, send;
  std::vector<i64> loads;
};

// (max, sum of squares, moves, sigma, send) in lexicographic order
bool better(const Plan& a, const Plan& b) {
  if (a.mx != b.mx) return a.mx < b.mx;
  if (a.sq != b.sq) return a.sq < b.sq;
  if (a.moves != b.moves) return a.moves < b.moves;
  if (a.sigma != b.sigma) return a.sigma < b.sigma;
  return a.send < b.send;
}

struct Problem {
  int R, Hl;
  std::vector<i64> w;  // [R][Hl]
  std::vector<i64> L;  // [R]
  i64 at(int r, int h) const { return w[(size_t)r * Hl + h]; }
};

Plan identity_plan(const Problem& P) {
  Plan p;
  p.sigma.resize(P.R);
  p.send.assign(P.R, -1);
  p.loads = P.L;
  p.mx = 0;
  p.sq = 0;
  for (int r = 0; r < P.R; ++r) {
    p.sigma[r] = r;
    p.mx = std::max(p.mx, P.L[r]);
    p.sq += P.L[r] * P.L[r];
  }
  return p;
}

// ---------------------------------------------------------------- pairs
struct PairOpt {
  i64 pmax, sq;
  int ha, hb;
};

struct PairTable {
  std::vector<i64> pmax;      // ascending
  std::vector<PairOpt> best;  // best[c]: lowest (sq, ha, hb) among the first c+1
};

class PairSearch {
 public:
  explicit PairSearch(const Problem& P) : P_(P), tab_((size_t)P.R * P.R) {
    const int R = P.R, Hl = P.Hl;
    std::vector<PairOpt> opts((size_t)Hl * Hl);
    for (int a = 0; a < R; ++a)
      for (int b = a + 1; b < R; ++b) {
        size_t n = 0;
        for (int ha = 0; ha < Hl; ++ha)
          for (int hb = 0; hb < Hl; ++hb) {
            const i64 la = P.L[a] - P.at(a, ha) + P.at(b, hb);
            const i64 lb = P.L[b] - P.at(b, hb) + P.at(a, ha);
            opts[n++] = PairOpt{std::max(la, lb), la * la + lb * lb, ha, hb};
          }
        std::stable_sort(opts.begin(), opts.end(),
                         [](const PairOpt& x, const PairOpt& y) { return x.pmax < y.pmax; });
        PairTable& t = tab_[(size_t)a * R + b];
        t.pmax.resize(n);
        t.best.resize(n);
        PairOpt run = opts[0];
        for (size_t i = 0; i < n; ++i) {
          const PairOpt& o = opts[i];
          if (o.sq < run.sq || (o.sq == run.sq && (o.ha < run.ha || (o.ha == run.ha && o.hb < run.hb))))
            run = o;
          t.pmax[i] = o.pmax;
          t.best[i] = run;
        }
      }
    best_ = identity_plan(P);
    sigma_.resize(R);
    for (int r = 0; r < R; ++r) sigma_[r] = r;
    cand_.sigma.resize(R);
    cand_.send.resize(R);
    cand_.loads.resize(R);
  }

  Plan run() {
    std::vector<int> free_ranks(P_.R);
    for (int r = 0; r < P_.R; ++r) free_ranks[r] = r;
    recurse(free_ranks);
    return best_;
  }

 private:
  const PairOpt& under(int a, int b, i64 M) const {
    const PairTable& t = tab_[(size_t)a * P_.R + b];
    const size_t c = std::upper_bound(t.pmax.begin(), t.pmax.end(), M) - t.pmax.begin();
    return t.best[c - 1];  // c >= 1 because M >= the pair's smallest maximum
  }

  void evaluate() {
    const int R = P_.R;
    i64 M = 0;
    int npairs = 0;
    for (int r = 0; r < R; ++r) {
      const int s = sigma_[r];
      if (s == r)
        M = std::max(M, P_.L[r]);
      else if (r < s) {
        M = std::max(M, tab_[(size_t)r * R + s].pmax[0]);
        ++npairs;
      }
    }
    if (M > best_.mx) return;
    i64 sq = 0;
    for (int r = 0; r < R; ++r) {
      const int s = sigma_[r];
      if (s == r)
        sq += P_.L[r] * P_.L[r];
      else if (r < s)
        sq += under(r, s, M).sq;
    }
    const int moves = 2 * npairs;
    if (M == best_.mx && (sq > best_.sq || (sq == best_.sq && moves > best_.moves))) return;
    cand_.mx = M;
    cand_.sq = sq;
    cand_.moves = moves;
    for (int r = 0; r < R; ++r) {
      const int s = sigma_[r];
      cand_.sigma[r] = s;
      if (s == r) {
        cand_.send[r] = -1;
        cand_.loads[r] = P_.L[r];
      } else if (r < s) {
        const PairOpt& o = under(r, s, M);
        cand_.send[r] = o.ha;
        cand_.send[s] = o.hb;
        cand_.loads[r] = P_.L[r] - P_.at(r, o.ha) + P_.at(s, o.hb);
        cand_.loads[s] = P_.L[s] - P_.at(s, o.hb) + P_.at(r, o.ha);
      }
    }
    if (better(cand_, best_)) best_ = cand_;
  }

  // pair the lowest free rank with nobody, or with each higher free rank
  void recurse(std::vector<int>& free_ranks) {
    if (free_ranks.empty()) {
      evaluate();
      return;
    }
    const int r = free_ranks[0];
    std::vector<int> rest(free_ranks.begin() + 1, free_ranks.end());
    recurse(rest);
    for (size_t i = 0; i < rest.size(); ++i) {
      const int s = rest[i];
      std::vector<int> left;
      left.reserve(rest.size() - 1);
      for (size_t j = 0; j < rest.size(); ++j)
        if (j != i) left.push_back(rest[j]);
      sigma_[r] = s;
      sigma_[s] = r;
      recurse(left);
      sigma_[r] = r;
      sigma_[s] = s;
    }
  }

  const Problem& P_;
  std::vector<PairTable> tab_;
  std::vector<int> sigma_;
  Plan best_, cand_;
};

// ----------------------------------------------------------------- ring
// new load of rank r when it sends head x and its predecessor sends head y
i64 ring_load(const Problem& P, int r, int x, int y) {
  const int p = (r + P.R - 1) % P.R;
  return P.L[r] - P.at(r, x) + P.at(p, y);
}

bool ring_feasible(const Problem& P, i64 M) {
  const int R = P.R, Hl = P.Hl;
  std::vector<char> cur(Hl), nxt(Hl);
  for (int h0 = 0; h0 < Hl; ++h0) {
    std::fill(cur.begin(), cur.end(), 0);
    cur[h0] = 1;  // reachable heads of rank r-1 (r = 1 first)
    for (int r = 1; r < R; ++r) {
      std::fill(nxt.begin(), nxt.end(), 0);
      for (int y = 0; y < Hl; ++y)
        if (cur[y])
          for (int x = 0; x < Hl; ++x)
            if (!nxt[x] && ring_load(P, r, x, y) <= M) nxt[x] = 1;
      std::swap(cur, nxt);
    }
    for (int y = 0; y < Hl; ++y)
      if (cur[y] && ring_load(P, 0, h0, y) <= M) return true;
  }
  return false;
}

Plan ring_search(const Problem& P) {
  const int R = P.R, Hl = P.Hl;
  Plan best = identity_plan(P);
  if (R < 2) return best;
  // smallest feasible maximum among the candidate values
  std::vector<i64> vals;
  vals.reserve((size_t)R * Hl * Hl);
  for (int r = 0; r < R; ++r)
    for (int x = 0; x < Hl; ++x)
      for (int y = 0; y < Hl; ++y) vals.push_back(ring_load(P, r, x, y));
  std::sort(vals.begin(), vals.end());
  vals.erase(std::unique(vals.begin(), vals.end()), vals.end());
  size_t lo = 0, hi = vals.size() - 1;  // the largest value is always feasible
  while (lo < hi) {
    const size_t mid = (lo + hi) / 2;
    if (ring_feasible(P, vals[mid]))
      hi = mid;
    else
      lo = mid + 1;
  }
  const i64 M = vals[lo];
  if (M > best.mx) return best;

  // for each head of rank 0: G[r][x] = lowest sum of squares of the new loads
  // of ranks r+1 .. R-1 and rank 0, given rank r sends x
  std::vector<i64> G((size_t)R * Hl);
  auto sqr_if = [&](i64 l) { return l <= M ? l * l : INF; };
  i64 best_sq = INF;
  int best_h0 = -1;
  std::vector<int32_t> send(R);
  for (int h0 = 0; h0 < Hl; ++h0) {
    for (int x = 0; x < Hl; ++x) G[(size_t)(R - 1) * Hl + x] = sqr_if(ring_load(P, 0, h0, x));
    for (int r = R - 2; r >= 0; --r)
      for (int x = 0; x < Hl; ++x) {
        i64 g = INF;
        if (r == 0 && x != h0) {
          G[x] = INF;
          continue;
        }
        for (int y = 0; y < Hl; ++y) {
          const i64 a = sqr_if(ring_load(P, r + 1, y, x)), b = G[(size_t)(r + 1) * Hl + y];
          if (a != INF && b != INF) g = std::min(g, a + b);
        }
        G[(size_t)r * Hl + x] = g;
      }
    const i64 total = G[h0];
    if (total >= best_sq) continue;  // ties keep the smaller h0
    best_sq = total;
    best_h0 = h0;
    // lexicographically smallest head vector reaching the optimum
    send[0] = h0;
    for (int r = 0; r < R - 1; ++r) {
      const i64 need = G[(size_t)r * Hl + send[r]];
      for (int y = 0; y < Hl; ++y) {
        const i64 a = sqr_if(ring_load(P, r + 1, y, send[r])), b = G[(size_t)(r + 1) * Hl + y];
        if (a != INF && b != INF && a + b == need) {
          send[r + 1] = y;
          break;
        }
      }
    }
    Plan p;
    p.mx = M;
    p.sq = total;
    p.moves = R;
    p.sigma.resize(R);
    p.loads.resize(R);
    p.send = send;
    for (int r = 0; r < R; ++r) {
      p.sigma[r] = (r + 1) % R;
      p.loads[r] = ring_load(P, r, send[r], send[(r + R - 1) % R]);
    }
    if (better(p, best)) best = p;
  }
  (void)best_h0;
  return best;
}

int gate(const std::vector<i64>& L, int k1, int k2) {
  const i64 R = (i64)L.size();
  i64 tot = 0, mx = 0;
  for (i64 x : L) {
    tot += x;
    mx = std::max(mx, x);
  }
  if (tot == 0) return FVA_BALANCE_NONE;
  if (1000 * R * mx >= (i64)k2 * tot) return FVA_BALANCE_RLB_SASA;
  if (1000 * R * mx >= (i64)k1 * tot) return FVA_BALANCE_SASA;
  return FVA_BALANCE_NONE;
}

int32_t rho_per_mille(const std::vector<i64>& L) {
  i64 tot = 0, mx = 0;
  for (i64 x : L) {
    tot += x;
    mx = std::max(mx, x);
  }
  return tot == 0 ? 0 : (int32_t)((1000 * (i64)L.size() * mx) / tot);
}

int check_params(const fva_balance_params* p) {
  if (!p) return FVA_ERR_ARG;
  if (p->reserved != 0) return FVA_ERR_ARG;
  if (p->num_ranks < 1 || p->heads_per_rank < 1) return FVA_ERR_ARG;
  if (p->topology != FVA_RLB_PAIRS && p->topology != FVA_RLB_RING) return FVA_ERR_ARG;
  if (p->k1_per_mille < 0 || p->k2_per_mille < p->k1_per_mille ||
      p->k2_per_mille > FVA_RLB_MAX_PER_MILLE)
    return FVA_ERR_ARG;
  if (p->n1_per_mille < 0 || p->n1_per_mille > 1000 || p->n2_per_mille < 0 ||
      p->n2_per_mille > FVA_RLB_MAX_PER_MILLE)
    return FVA_ERR_ARG;
  if (p->heads_per_rank > FVA_RLB_MAX_HEADS) return FVA_ERR_UNSUPPORTED;
  const int max_r = p->topology == FVA_RLB_PAIRS ? FVA_RLB_MAX_PAIR_RANKS : FVA_RLB_MAX_RANKS;
  if (p->num_ranks > max_r) return FVA_ERR_UNSUPPORTED;
  return FVA_OK;
}

}  // namespace

extern "C" int fva_balance(const fva_balance_params* prm, const int32_t* head_load, int32_t* sigma,
                           int32_t* send_head, int64_t* load_new, int64_t* slack, int64_t* budget,
                           fva_balance_info* info) {
  int st = check_params(prm);
  if (st) return st;
  if (!head_load || !sigma || !send_head || !load_new || !slack || !budget || !info) return FVA_ERR_ARG;
  Problem P;
  P.R = prm->num_ranks;
  P.Hl = prm->heads_per_rank;
  P.w.resize((size_t)P.R * P.Hl);
  P.L.assign(P.R, 0);
  for (int r = 0; r < P.R; ++r)
    for (int h = 0; h < P.Hl; ++h) {
      const int32_t x = head_load[(size_t)r * P.Hl + h];
      if (x < 0 || x > FVA_RLB_MAX_HEAD_LOAD) return FVA_ERR_ARG;
      P.w[(size_t)r * P.Hl + h] = x;
      P.L[r] += x;
    }
  const int mode = gate(P.L, prm->k1_per_mille, prm->k2_per_mille);
  Plan plan;
  if (mode == FVA_BALANCE_RLB_SASA)
    plan = prm->topology == FVA_RLB_PAIRS ? PairSearch(P).run() : ring_search(P);
  else
    plan = identity_plan(P);

  i64 lmax = 0;
  for (int r = 0; r < P.R; ++r) lmax = std::max(lmax, plan.loads[r]);
  i64 aug_max = 0, tot = 0;
  for (int r = 0; r < P.R; ++r) {
    const i64 d = lmax - plan.loads[r];
    const bool trig = mode != FVA_BALANCE_NONE && 1000 * d > (i64)prm->n2_per_mille * lmax;
    sigma[r] = plan.sigma[r];
    send_head[r] = plan.send[r];
    load_new[r] = plan.loads[r];
    slack[r] = d;
    budget[r] = trig ? ((i64)prm->n1_per_mille * d) / 1000 : 0;
    aug_max = std::max(aug_max, plan.loads[r] + budget[r]);
    tot += P.L[r];
  }
  info->mode = mode;
  info->moves = plan.moves;
  info->rho_per_mille = rho_per_mille(P.L);
  info->rho_new_per_mille = rho_per_mille(plan.loads);
  info->load_total = tot;
  info->load_max = *std::max_element(P.L.begin(), P.L.end());
  info->load_new_max = lmax;
  info->load_aug_max = aug_max;
  return FVA_OK;
}

extern "C" int fva_sasa_refill(const fva_balance_params* prm, int32_t nb, const int32_t* row_count,
                               const int32_t* send_head, const int64_t* budget, int32_t* head_refill,
                               int64_t* added) {
  int st = check_params(prm);
  if (st) return st;
  if (!row_count || !send_head || !budget || !head_refill || !added) return FVA_ERR_ARG;
  if (nb < 1 || nb > FVA_MAX_BLOCKS) return FVA_ERR_ARG;
  const int R = prm->num_ranks, Hl = prm->heads_per_rank;
  for (int r = 0; r < R; ++r)
    if (send_head[r] < -1 || send_head[r] >= Hl || budget[r] < 0) return FVA_ERR_ARG;
  const size_t rows = (size_t)R * Hl * nb;
  for (size_t i = 0; i < rows; ++i)
    if (row_count[i] < 0 || row_count[i] > nb) return FVA_ERR_ARG;

  const i64 fmax = 1000 * (i64)(nb - 1);
  std::vector<i64> hist(nb + 1);
  for (int r = 0; r < R; ++r) {
    // kept-count histogram of the rank's eligible rows
    std::fill(hist.begin(), hist.end(), 0);
    for (int h = 0; h < Hl; ++h) {
      if (h == send_head[r]) continue;
      const int32_t* rc = row_count + ((size_t)r * Hl + h) * nb;
      for (int i = 0; i < nb; ++i) ++hist[rc[i]];
    }
    auto added_at = [&](i64 f) {
      i64 a = 0;
      for (int k = 1; k < nb; ++k)
        if (hist[k]) a += hist[k] * std::min<i64>(nb - k, (k * f) / 1000);
      return a;
    };
    const i64 B = budget[r];
    i64 lo = 0, hi = fmax;  // largest f whose refill fits the budget
    while (lo < hi) {
      const i64 mid = (lo + hi + 1) / 2;
      if (added_at(mid) <= B)
        lo = mid;
      else
        hi = mid - 1;
    }
    const i64 best = added_at(lo);
    i64 a = 0, b = lo;  // smallest f adding as many blocks
    while (a < b) {
      const i64 mid = (a + b) / 2;
      if (added_at(mid) >= best)
        b = mid;
      else
        a = mid + 1;
    }
    for (int h = 0; h < Hl; ++h) head_refill[(size_t)r * Hl + h] = h == send_head[r] ? 0 : (int32_t)a;
    added[r] = best;
  }
  return FVA_OK;
}
