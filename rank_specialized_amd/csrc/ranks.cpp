// Retained-rank allocation (host only): how many ranks each adapter factor
// pair keeps after compression.
//
// "LoRAForge: Co-Designing Compression and Execution for More Efficient
// Multi-LoRA Serving", section "LoRAForge's Core Design: Explicit
// Retained-Rank Representation and Dual Strategies": a uniform ratio of the
// original rank (with a floor), or a spectral budget that keeps the
// components carrying the most energy.  The pages give no formula; the
// readings: uniform r = min(r_orig, max(floor, ceil(ratio r_orig))); spectral
// keeps min(floor, r_orig) per unit, then gives the remaining budget one rank
// at a time to the unit whose next sigma^2 is largest (ties: lower unit).
// With every unit's sigma non-increasing, that is the first k candidates
// (unit u, component j >= its floor) in the order (sigma^2 descending, u, j),
// found here with one selection, O(candidates).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "../../include/lora.h"

extern "C" {

int lora_ranks_uniform(int m, const int32_t* r_orig_host, double ratio, int floor_rank, int32_t* r_out_host) {
  if (m < 0 || (m > 0 && (!r_orig_host || !r_out_host)) || !(ratio >= 0.0 && ratio <= 1.0) || floor_rank < 0)
    return LORA_ERR_INVALID_ARG;
  for (int u = 0; u < m; ++u)
    if (r_orig_host[u] < 0) return LORA_ERR_INVALID_ARG;
  for (int u = 0; u < m; ++u) {
    const int r = r_orig_host[u];
    // ceil of ratio * r; the tolerance keeps a product that rounding puts a
    // hair above an integer (0.3 * 10) at that integer
    const int c = (int)std::ceil(ratio * r - 1e-12);
    r_out_host[u] = std::min(r, std::max(floor_rank, c));
  }
  return LORA_OK;
}

int lora_ranks_spectral(int m, const int32_t* r_orig_host, const float* sigma_host, const int64_t* sigma_off_host,
                        int floor_rank, int64_t budget, int32_t* r_out_host) {
  if (m < 0 || (m > 0 && (!r_orig_host || !sigma_off_host || !r_out_host)) || floor_rank < 0 || budget < 0)
    return LORA_ERR_INVALID_ARG;
  if (m == 0) return LORA_OK;
  if (sigma_off_host[0] != 0) return LORA_ERR_INVALID_ARG;
  int64_t floors = 0, cands = 0;
  for (int u = 0; u < m; ++u) {
    const int r = r_orig_host[u];
    if (r < 0 || sigma_off_host[u + 1] - sigma_off_host[u] != r) return LORA_ERR_INVALID_ARG;
    const float* s = sigma_host + sigma_off_host[u];
    for (int j = 0; j < r; ++j) {
      if (!(std::isfinite(s[j]) && s[j] >= 0.f)) return LORA_ERR_INVALID_ARG;
      if (j > 0 && s[j] > s[j - 1]) return LORA_ERR_INVALID_ARG;  // non-increasing per unit
    }
    const int f = std::min(floor_rank, r);
    r_out_host[u] = f;
    floors += f;
    cands += r - f;
  }
  if (sigma_off_host[m] > 0 && !sigma_host) return LORA_ERR_INVALID_ARG;
  int64_t k = std::min(budget - floors, cands);
  if (k <= 0) return LORA_OK;
  struct Cand {
    double e;
    int32_t u, j;
  };
  std::vector<Cand> c;
  c.reserve((size_t)cands);
  for (int u = 0; u < m; ++u) {
    const float* s = sigma_host + sigma_off_host[u];
    for (int j = r_out_host[u]; j < r_orig_host[u]; ++j) c.push_back({(double)s[j] * (double)s[j], u, j});
  }
  auto before = [](const Cand& a, const Cand& b) {
    if (a.e != b.e) return a.e > b.e;
    if (a.u != b.u) return a.u < b.u;
    return a.j < b.j;
  };
  if (k < (int64_t)c.size()) std::nth_element(c.begin(), c.begin() + (k - 1), c.end(), before);
  for (int64_t i = 0; i < k; ++i) ++r_out_host[c[(size_t)i].u];
  return LORA_OK;
}

}  // extern "C"
