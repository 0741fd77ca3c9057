// Planner step of PagedWeight §3.2 (Algorithm 1, Eqs. 3-8), host code.
//
// For each bitwidth-floor stage the planner builds a candidate plan by a
// greedy over one-bit reductions ("steps") of routed linear-blocks, cheapest
// predicted damage per released byte first, until the byte target D derived
// from KV-cache pressure is met; the newest plan of every stage forms the
// plan queue, and under pressure one plan is selected for page movement.
// Every floating-point value is formed in a fixed order (no contraction), so
// the result is reproducible bit for bit.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <queue>
#include <vector>

#include "mpb.h"
#include "mpb_internal.h"

#pragma clang fp contract(off)

namespace {

constexpr int kMinBits = 3, kMaxBits = 8;

int64_t block_bytes(int64_t N, int64_t Kd, int b) { return N * Kd * b / 8 + N * (int64_t(1) << b) * 2; }

struct Step {
  double ratio;  // predicted damage / released bytes
  int i;
  bool operator>(const Step& o) const { return ratio > o.ratio || (ratio == o.ratio && i > o.i); }
};

bool params_ok(const mpb_planner_params& p, const char** why) {
  if (p.n_buckets < 1 || p.n_buckets > 8) { *why = "n_buckets must be in 1..8"; return false; }
  for (int k = 0; k < p.n_buckets; ++k) {
    const double lo = k ? p.bucket_frac[k - 1] : 0.0;
    if (!(p.bucket_frac[k] > lo) || p.bucket_frac[k] > 1.0) {
      *why = "bucket_frac must increase within (0, 1]";
      return false;
    }
    if (!(p.mu[k] > 0.0) || !std::isfinite(p.mu[k])) { *why = "mu must be positive"; return false; }
    if (p.floor[k] < kMinBits || p.floor[k] > kMaxBits) { *why = "bucket floors must be in 3..8"; return false; }
  }
  if (p.bucket_frac[p.n_buckets - 1] != 1.0) { *why = "the last bucket_frac must be 1"; return false; }
  if (p.n_stages < 1 || p.n_stages > 6) { *why = "n_stages must be in 1..6"; return false; }
  for (int s = 0; s < p.n_stages; ++s) {
    if (p.stage_floor[s] < kMinBits || p.stage_floor[s] > kMaxBits) { *why = "stage floors must be in 3..8"; return false; }
    if (s && p.stage_floor[s] >= p.stage_floor[s - 1]) { *why = "stage floors must decrease"; return false; }
  }
  if (!(p.eps > 0.0) || !std::isfinite(p.eps)) { *why = "eps must be positive"; return false; }
  if (!std::isfinite(p.alpha) || !(p.rho_min <= p.rho_max)) { *why = "alpha / rho range invalid"; return false; }
  if (p.T_blk < 0 || p.F_blk < 0 || p.P_blk < 0 || p.B_kv < 0) { *why = "block counts must be >= 0"; return false; }
  return true;
}

// Predicted damage of the step (i, b -> b-1): global damage (Eq. 4) times the
// bucket multiplier and the prompt-residual factor (Eqs. 5, 6), floored (Eq. 8).
double step_damage(const mpb_planner_params& p, const double* sens, const double* phi, int i, int b, double mu) {
  const int u = i & 1, t = b - 4;
  const double* s = sens + (size_t)i * 6;
  const double g = std::fmax(s[b - 1 - kMinBits] - s[b - kMinBits], 0.0);
  const double* f = phi + (size_t)i * 3;
  double rho = 0.0;
  for (int j = 0; j < 3; ++j) rho = rho + p.head_w[u][t][j] * f[j];
  rho = rho + p.head_a[u][t];
  const double clipped = std::fmin(std::fmax(rho, p.rho_min), p.rho_max);
  const double eta = std::exp(p.alpha * p.head_c[u][t] * clipped);
  return std::fmax(p.eps, mu * g * eta);
}

}  // namespace

extern "C" int mpb_plan_step(const mpb_layer_desc* d, const int32_t* q, const uint8_t* movable,
                             const double* sens, const double* mass, const double* phi,
                             const mpb_planner_params* prm, int32_t* queue, mpb_plan_entry* plan,
                             mpb_plan_summary* summary) try {
  using mpb::set_error;
  if (!d || !q || !sens || !mass || !phi || !prm || !plan || !summary)
    return set_error(MPB_E_ARG, "mpb_plan_step: null pointer");
  const char* why = "";
  if (!mpb::geometry_ok(d->H, d->I, d->E, d->S, d->K, &why)) return set_error(MPB_E_SHAPE, why);
  const mpb_planner_params& p = *prm;
  if (!params_ok(p, &why)) return set_error(MPB_E_ARG, why);
  const int E = d->E, nb = 2 * (d->E + d->S), nr = 2 * E;
  for (int i = 0; i < nb; ++i)
    if (q[i] < kMinBits || q[i] > kMaxBits) return set_error(MPB_E_RANGE, "mpb_plan_step: q outside 3..8");
  auto rows = [&](int i) { return (int64_t)(i & 1 ? d->H : 2 * d->I); };
  auto cols = [&](int i) { return (int64_t)(i & 1 ? d->I : d->H); };

  // TargetBytesFromKVPressure (Eq. 7), on the free count after pending growth
  const int64_t short_blk = p.T_blk + 1 - (p.F_blk - p.P_blk);
  const int64_t D = short_blk > 0 ? short_blk * p.B_kv : 0;

  // routing buckets: experts by routing mass, hottest first, ties to lower index
  std::vector<int> order(E), bucket(E, 0);
  for (int e = 0; e < E; ++e) order[e] = e;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return mass[a] > mass[b]; });
  for (int k = 0, lo = 0; k < p.n_buckets; ++k) {
    const int hi = std::min(E, (int)std::ceil(p.bucket_frac[k] * E));
    for (int r = lo; r < hi; ++r) bucket[order[r]] = k;
    lo = std::max(lo, hi);
  }

  std::vector<int32_t> cur(nb), floor_(nb);
  std::vector<double> dmg(nb);
  std::vector<std::vector<int32_t>> stage_bits(p.n_stages);
  std::vector<std::vector<double>> stage_dmg(p.n_stages);
  int64_t released_s[6] = {0};
  double damage_s[6] = {0};
  for (int s = 0; s < p.n_stages; ++s) {
    // ScoreActions: the floors of this stage and every block's first step
    std::priority_queue<Step, std::vector<Step>, std::greater<Step>> heap;
    auto push = [&](int i) {
      if (cur[i] <= floor_[i]) return;
      const int64_t delta = block_bytes(rows(i), cols(i), cur[i]) - block_bytes(rows(i), cols(i), cur[i] - 1);
      const double dd = step_damage(p, sens, phi, i, cur[i], p.mu[bucket[i >> 1]]);
      heap.push(Step{dd / (double)delta, i});
    };
    for (int i = 0; i < nb; ++i) {
      cur[i] = q[i];
      dmg[i] = 0.0;
      const bool cand = i < nr && (!movable || movable[i]);
      floor_[i] = cand ? std::max(p.stage_floor[s], p.floor[bucket[i >> 1]]) : kMaxBits + 1;
      push(i);
    }
    // GreedySelect: cheapest step per released byte until D is met
    int64_t released = 0;
    double damage = 0.0;
    while (released < D && !heap.empty()) {
      const int i = heap.top().i;
      heap.pop();
      const int64_t delta = block_bytes(rows(i), cols(i), cur[i]) - block_bytes(rows(i), cols(i), cur[i] - 1);
      const double dd = step_damage(p, sens, phi, i, cur[i], p.mu[bucket[i >> 1]]);
      released += delta;
      damage = damage + dd;
      dmg[i] = dmg[i] + dd;
      --cur[i];
      push(i);
    }
    // RefreshPlanQueue: the newest plan of this stage
    stage_bits[s] = cur;
    stage_dmg[s] = dmg;
    released_s[s] = released;
    damage_s[s] = damage;
    if (queue) std::memcpy(queue + (size_t)s * nb, cur.data(), sizeof(int32_t) * nb);
  }

  // SelectBestPlan: first stage that meets D, else the largest reduction
  int pick = -1;
  for (int s = 0; s < p.n_stages && pick < 0; ++s)
    if (released_s[s] >= D) pick = s;
  if (pick < 0) {
    pick = 0;
    for (int s = 1; s < p.n_stages; ++s)
      if (released_s[s] > released_s[pick]) pick = s;
  }
  const bool triggered = p.F_blk <= p.T_blk;  // PressureTriggered
  std::memset(summary, 0, sizeof(*summary));
  summary->D = D;
  summary->triggered = triggered ? 1 : 0;
  summary->stage = triggered ? pick : -1;
  for (int s = 0; s < p.n_stages; ++s) {
    summary->stage_released[s] = released_s[s];
    summary->stage_damage[s] = damage_s[s];
  }
  int n = 0;
  if (triggered) {
    for (int i = 0; i < nb; ++i) {
      const int to = stage_bits[pick][i];
      if (to == q[i]) continue;
      mpb_plan_entry& en = plan[n++];
      en.i = i;
      en.from = q[i];
      en.to = to;
      en.delta = block_bytes(rows(i), cols(i), q[i]) - block_bytes(rows(i), cols(i), to);
      en.damage = stage_dmg[pick][i];
      summary->released += en.delta;
      summary->damage = summary->damage + en.damage;
    }
  }
  summary->n_plan = n;
  return MPB_OK;
} catch (...) {
  return mpb::set_error(MPB_E_ARG, "mpb_plan_step: unexpected exception");
}
