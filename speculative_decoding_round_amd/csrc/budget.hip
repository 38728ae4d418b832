// Speculative-budget controller ([P5] 执行控制器): host code, one state per request stream.
// The policy (lower on low acceptance or costly drafting, raise cautiously on stable
// acceptance with verification room, revert a raise that costs goodput, cooldown and bounds)
// is stated with the entry points in eagle3.h.
#include <cmath>

#include "internal.h"

namespace {

bool finite_nonneg(float x) { return std::isfinite(x) && x >= 0.f; }

int params_ok(const eagle3_budget_params* p) {
  if (!p) return EAGLE3_EINVAL;
  if (p->n_levels < 1 || p->n_levels > EAGLE3_BUDGET_MAX_LEVELS) return EAGLE3_EINVAL;
  if (p->start_level < 0 || p->start_level >= p->n_levels) return EAGLE3_EINVAL;
  if (p->cooldown < 1 || p->window < 1 || p->window > EAGLE3_BUDGET_MAX_WINDOW) return EAGLE3_EINVAL;
  if (!finite_nonneg(p->low_frac) || !finite_nonneg(p->high_frac) || !finite_nonneg(p->max_cv) ||
      !finite_nonneg(p->draft_share_max) || !finite_nonneg(p->verify_ms_max) || !finite_nonneg(p->revert_drop))
    return EAGLE3_EINVAL;
  for (int l = 0; l < p->n_levels; ++l) {
    const eagle3_tree_cfg& t = p->levels[l];
    if (t.depth < 1 || t.topk < 1 || t.width < 1 || t.n_nodes < 1) return EAGLE3_EINVAL;
  }
  return EAGLE3_OK;
}

void change(eagle3_budget_state* s, int level) {
  s->level = level;
  s->since = 0;
  s->count = 0;
  s->head = 0;
}

}  // namespace

extern "C" {

int eagle3_budget_init(const eagle3_budget_params* p, eagle3_budget_state* s) {
  if (const int st = params_ok(p)) return st;
  if (!s) return EAGLE3_EINVAL;
  s->level = p->start_level;
  s->since = 0;
  s->block = 0;
  s->check = 0;
  s->count = 0;
  s->head = 0;
  s->g_before = 0.0;
  return EAGLE3_OK;
}

int eagle3_budget_update(const eagle3_budget_params* p, eagle3_budget_state* s, int32_t accept_len,
                         float draft_ms, float verify_ms, eagle3_tree_cfg* next) {
  if (const int st = params_ok(p)) return st;
  if (!s || accept_len < 0 || !finite_nonneg(draft_ms) || !finite_nonneg(verify_ms)) return EAGLE3_EINVAL;
  if (s->level < 0 || s->level >= p->n_levels || s->count < 0 || s->count > p->window || s->head < 0 ||
      s->head >= EAGLE3_BUDGET_MAX_WINDOW)
    return EAGLE3_EINVAL;   // not a state this controller wrote
  const int W = p->window;
  // append; a full window drops its oldest round
  if (s->count == W) {
    s->head = (s->head + 1) % W;
    s->count = W - 1;
  }
  const int slot = (s->head + s->count) % W;
  s->committed[slot] = (double)accept_len + 1.0;
  s->draft_ms[slot] = (double)draft_ms;
  s->verify_ms[slot] = (double)verify_ms;
  s->count += 1;
  s->since += 1;
  if (s->block > 0) s->block -= 1;
  if (s->count == W && s->since >= p->cooldown) {
    const double n = (double)s->count;
    double sc = 0.0, sd = 0.0, sv = 0.0, sr = 0.0;
    for (int i = 0; i < s->count; ++i) {
      const int j = (s->head + i) % W;
      sc += s->committed[j];
      sd += s->draft_ms[j];
      sv += s->verify_ms[j];
      sr += s->draft_ms[j] + s->verify_ms[j];
    }
    const double mc = sc / n;
    double ss = 0.0;
    for (int i = 0; i < s->count; ++i) {
      const double e = s->committed[(s->head + i) % W] - mc;
      ss += e * e;
    }
    const double cv = std::sqrt(ss / n) / mc;
    const double md = sd / n, mv = sv / n, mr = sr / n;
    const double frac = mc / (double)(p->levels[s->level].depth + 1);
    const double good = mc / mr;
    bool done = false;
    if (s->check) {
      s->check = 0;
      if (good < s->g_before * (1.0 - (double)p->revert_drop) && s->level > 0) {
        s->block = 4 * p->cooldown;
        change(s, s->level - 1);
        done = true;
      }
    }
    if (!done) {
      if ((frac < (double)p->low_frac || md / mr > (double)p->draft_share_max) && s->level > 0) {
        change(s, s->level - 1);
      } else if (frac >= (double)p->high_frac && cv <= (double)p->max_cv && mv < (double)p->verify_ms_max &&
                 s->block == 0 && s->level < p->n_levels - 1) {
        s->g_before = good;
        s->check = 1;
        change(s, s->level + 1);
      }
    }
  }
  if (next) *next = p->levels[s->level];
  return s->level;
}

}  // extern "C"
