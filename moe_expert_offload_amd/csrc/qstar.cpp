// The bandwidth-adaptive split of a decode step's cache misses.
//
// [FT] "FreeToken: Efficient Edge-Native MoE Serving with Bandwidth-Adaptive
// Execution", §3.2 Eqs. (1)-(4): misses split into q fills over PCIe (rate B_P)
// and m - q host executions at the residual rate B_H - B_P; balance gives
// q* ~= m B_P / B_H, rounded to an integer, with at least one fill kept.
// [AIN] "FreeToken: bandwidth-adaptive edge MoE serving", section "The split,
// and what it is actually optimising": the integer pick is done in Q16 between
// lo = floor(m fq / 2^16) and lo + 1 by the two-branch makespan, lo on a tie.
#include <cfenv>
#include <cmath>

#include "internal.h"

extern "C" uint32_t ft_frac_q16(double B_P, double B_H) {
  if (!(B_P > 0.0)) return 0u;
  if (B_P >= B_H) return 65536u;
  // nearbyint under the default rounding mode: ties to even
  const double v = std::nearbyint((B_P / B_H) * 65536.0);
  if (v <= 0.0) return 0u;
  if (v >= 65536.0) return 65536u;
  return (uint32_t)v;
}

extern "C" int32_t ft_qstar_split(int32_t m, uint32_t frac_q16, int32_t min_fill,
                                  int32_t max_fetch, int32_t avail) {
  if (m < 0 || frac_q16 > 65536u) return FT_EINVAL;
  if (m == 0) return 0;
  const int64_t fq = frac_q16;
  const int64_t one = 65536;
  // makespan of f fills next to m - f host experts, in Q16 units
  auto makespan = [&](int64_t f) {
    const int64_t fill = f * (one - fq);
    const int64_t host = (int64_t)(m - f) * fq;
    return fill > host ? fill : host;
  };
  const int64_t lo = ((int64_t)m * fq) >> 16;
  int64_t q = makespan(lo + 1) < makespan(lo) ? lo + 1 : lo;
  if (q > m) q = m;
  const int64_t floor_fill = min_fill < m ? min_fill : m;
  if (q < floor_fill) q = floor_fill;
  if (max_fetch >= 0 && q > max_fetch) q = max_fetch;
  if (avail < 0) avail = 0;
  if (q > avail) q = avail;
  if (q < 0) q = 0;
  return (int32_t)q;
}

// ---- the bandwidth profile's fraction and the hybrid gate -----------------------------
// [AIN] "How to maintain it": the preferred fraction uses the contended pair,
// pcie_ov / (pcie_ov + cpu_ov); a profile without it falls back to Eq. (4).
extern "C" uint32_t ft_frac_q16_contended(double pcie_ov, double cpu_ov) {
  if (!(pcie_ov > 0.0)) return 0u;
  if (!(cpu_ov > 0.0)) return 65536u;
  const double v = std::nearbyint(pcie_ov / (pcie_ov + cpu_ov) * 65536.0);
  if (v <= 0.0) return 0u;
  if (v >= 65536.0) return 65536u;
  return (uint32_t)v;
}

extern "C" uint32_t ft_fetch_fraction_q16(const ft_bw_profile* p) {
  if (!p) return 0u;
  if (p->pcie_ov > 0.0 && p->cpu_ov > 0.0) return ft_frac_q16_contended(p->pcie_ov, p->cpu_ov);
  return ft_frac_q16(p->B_P, p->B_H);
}

// [AIN] "Why use it": hybrid only when B_H > threshold * B_P for every benched
// workload of the format ("unanimous or offload").
extern "C" int32_t ft_recommend_hybrid(const double* B_P, const double* B_H, int32_t n, double threshold) {
  if (n < 0 || (n > 0 && (!B_P || !B_H)) || !(threshold > 0.0)) return FT_EINVAL;
  if (n == 0) return 0;
  for (int32_t i = 0; i < n; ++i)
    if (!(B_H[i] > threshold * B_P[i])) return 0;
  return 1;
}
