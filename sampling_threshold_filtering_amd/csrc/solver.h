// Internal declarations of the host-side parameter solver (solver.cpp).
#pragma once
#include <cstdint>

#include "profk.h"

namespace profk {

// F_{N,K,S}(j) = Pr(X <= j), X ~ Hypergeometric(N, K, S).
double hyp_cdf(int64_t j, int64_t N, int64_t K, int64_t S);
// Pr(X > j).
double hyp_upper_tail(int64_t j, int64_t N, int64_t K, int64_t S);
// min{j : F(j) >= p}.
int64_t hyp_quantile(double p, int64_t N, int64_t K, int64_t S);
// z with Pr(Z > z) = q for a standard normal Z.
double normal_upper_quantile(double q);
// Phi^-1(p) by Acklam's rational approximation.
double acklam_inv_phi(double p);
// 1 / r(k) of the cost model (0 when r is infinite).
double cost_ratio_inverse(int64_t k, double a, double b);

int solve(int64_t N, int64_t k, double eps, const profk_options* opt, profk_params* out);
int solve_memo(int64_t N, int64_t k, double eps, const profk_options* opt, profk_params* out);

}  // namespace profk
