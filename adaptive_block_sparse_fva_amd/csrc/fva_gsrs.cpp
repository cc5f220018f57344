// Step schedule of growing sparsity with reduced search, on the host.
//
// GSRS paper S5.1 and A.5: the first denoising steps run full attention
// (warm-up); the first search evaluates every key block; later searches
// evaluate only the early candidate set (the first search's mask) unless
// reduced search is off; between searches the latest mask is reused; the
// Top-p threshold of each search is given per search (decreasing p is the
// growing sparsity of S5.1).  S6.1's default: 50 steps, 10 warm-up steps,
// searches at steps 10, 20, 30, 40 with p = 0.95, 0.9, 0.85, 0.8.
#include <cmath>

#include "fva.h"

extern "C" int fva_gsrs_action(const fva_gsrs_schedule* s, int32_t step, int32_t* action,
                               float* top_p) {
  if (!s || !action || !top_p) return FVA_ERR_ARG;
  if (s->num_steps < 1 || s->warmup_steps < 0 || s->num_searches < 0 ||
      s->num_searches > FVA_GSRS_MAX_SEARCHES || (s->reduced != 0 && s->reduced != 1))
    return FVA_ERR_ARG;
  for (int j = 0; j < s->num_searches; ++j) {
    if (s->search_step[j] < 0 || s->search_step[j] >= s->num_steps) return FVA_ERR_ARG;
    if (j > 0 && s->search_step[j] <= s->search_step[j - 1]) return FVA_ERR_ARG;
    if (std::isnan(s->top_p[j])) return FVA_ERR_ARG;
  }
  if (step < 0 || step >= s->num_steps) return FVA_ERR_ARG;

  *top_p = 1.0f;
  if (step < s->warmup_steps) {
    *action = FVA_GSRS_DENSE;
    return FVA_OK;
  }
  int first = -1;  // first search step past the warm-up
  for (int j = 0; j < s->num_searches; ++j)
    if (s->search_step[j] >= s->warmup_steps) {
      first = s->search_step[j];
      break;
    }
  for (int j = 0; j < s->num_searches; ++j)
    if (s->search_step[j] == step) {
      *top_p = s->top_p[j];
      *action = (step == first || !s->reduced) ? FVA_GSRS_FULL_SEARCH : FVA_GSRS_CANDIDATE_SEARCH;
      return FVA_OK;
    }
  *action = (first < 0 || step < first) ? FVA_GSRS_DENSE : FVA_GSRS_REUSE;
  return FVA_OK;
}
