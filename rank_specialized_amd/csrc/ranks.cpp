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
// found here by a radix selection over the values' bits, O(candidates).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
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
  for (int u = 0; u < m; ++u)
    if (r_orig_host[u] < 0 || sigma_off_host[u + 1] - sigma_off_host[u] != r_orig_host[u]) return LORA_ERR_INVALID_ARG;
  if (sigma_off_host[m] > 0 && !sigma_host) return LORA_ERR_INVALID_ARG;
  int64_t floors = 0, cands = 0;
  for (int u = 0; u < m; ++u) {
    const int r = r_orig_host[u];
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
  const int64_t k = std::min(budget - floors, cands);
  if (k <= 0) return LORA_OK;
  // sigma >= 0, so sigma^2 orders as sigma does, and a non-negative float
  // orders as its bit pattern.  Radix-select the bits T of the k-th largest
  // candidate (two 16-bit histogram passes), then give each unit its
  // candidates above T and, in (unit, component) order, the ties at T that
  // the budget still allows: the same first k as sorting by (sigma^2
  // descending, unit, component).
  auto bits = [](float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return f == 0.f ? 0u : u;  // -0 orders as +0
  };
  std::vector<int64_t> hist(1 << 16);
  int64_t need = k;  // rank of the threshold among candidates, from the top
  uint32_t hi = 0;
  for (int pass = 0; pass < 2; ++pass) {
    std::fill(hist.begin(), hist.end(), 0);
    for (int u = 0; u < m; ++u) {
      const float* s = sigma_host + sigma_off_host[u];
      for (int j = r_out_host[u]; j < r_orig_host[u]; ++j) {
        const uint32_t b = bits(s[j]);
        if (pass == 0) ++hist[b >> 16];
        else if ((b >> 16) == hi) ++hist[b & 0xffffu];
      }
    }
    int bin = (1 << 16) - 1;
    for (; bin > 0 && hist[bin] < need; --bin) need -= hist[bin];
    hi = pass == 0 ? (uint32_t)bin : (hi << 16) | (uint32_t)bin;
  }
  const uint32_t thr = hi;  // bits of the k-th largest; need = how many ties at thr are taken
  for (int u = 0; u < m; ++u) {
    const float* s = sigma_host + sigma_off_host[u];
    int add = 0;
    for (int j = r_out_host[u]; j < r_orig_host[u]; ++j) {
      const uint32_t b = bits(s[j]);
      if (b > thr) {
        ++add;
      } else if (b == thr && need > 0) {
        ++add;
        --need;
      } else {
        break;  // non-increasing: nothing further in this unit qualifies
      }
    }
    r_out_host[u] += add;
  }
  return LORA_OK;
}

}  // extern "C"
