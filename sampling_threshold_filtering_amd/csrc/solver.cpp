// Host-side parameter choice of Prof-K, in double precision.
//
// Pages: P1 = "Prof-K: Probabilistic One-Pass Filtering for Efficient Top-k
// Selection" (arXiv HTML page); P2 = its earlier version (bittide mirror).
//
//  * eps_A = eps_B = eps / 2                            (P1 §4, after Theorem 4)
//  * z_A = Phi^-1(1 - eps_A), z = z_A + z_B             (P2 Algorithm 1, step 1)
//  * S*_raw = c (k (N-k))^(1/3), default c = 1; S = round-to-nearest, clamped to
//    [S_min, S_max] = [32768, 131072], at most N         (P2 Theorem 5, Eq. 14 and
//    the text after it; the prefactor c = 1 is the one that reproduces the worked
//    example N = 1e9, k = 100 -> S* about 4,600)
//  * t* = F^-1_{N,k-1,S}(1 - eps_A) + 1,
//    M* = min{M in [k, N] : F_{N,M,S}(t* - 1) <= eps_B}  (P1 Theorem 4, Eq. 7),
//    M* by binary search since G(M) = F_{N,M,S}(t-1) is nonincreasing in M (P1 Lemma 1)
//  * M_cf = k + z sqrt(k (N-k) / S (1 - S/N))          (P2 Corollary 4, Eq. 12)
//  * operating t = t*, M = max(M*, ceil(M_cf)); the closed form is kept as a lower
//    bound only, since with P2's own t it exceeds the budget in the sparse regime
//  * Pr(R < k) = 1 - F_{N,k-1,S}(t-1)  (P1 Eq. 5);  Pr(R > M) = F_{N,M,S}(t-1)  (P1 Eq. 6)
//  * E[R], Var[R] of the negative hypergeometric rank  (P2 Lemma 1, Eq. 2)
//
//  * optional (profk_options.param_mode / s_rule): the closed-form surrogates and the
//    cost-model S rule of P1 Algorithm 1 (App. B Eq. 10-12, Proposition 7)
//
// Hypergeometric CDF numerics: log P(X = 0) = sum_{i<S} log1p(-K / (N - i)), then the
// ratio recurrence P(j+1)/P(j) = (K-j)(S-j) / ((j+1)(N-K-S+j+1)) in log space.  lgamma
// differences are avoided in the main regime: at N = 2^30 they lose about 1e-6.
#include "solver.h"

#include <algorithm>
#include <cmath>
#include <map>
#include <mutex>
#include <tuple>

namespace profk {

namespace {

// log P(X = jmin) for X ~ Hyp(N, K, S), jmin = max(0, S + K - N).
double log_pmf_at_min(int64_t N, int64_t K, int64_t S, int64_t jmin) {
  if (jmin == 0) {
    // P(X = 0) = prod_{i<S} (N - K - i) / (N - i)
    if (K == 0) return 0.0;
    long double acc = 0.0L;
    const double Kd = (double)K;
    for (int64_t i = 0; i < S; ++i) acc += (long double)std::log1p(-Kd / (double)(N - i));
    return (double)acc;
  }
  // K + S > N: P(X = jmin) = C(K, jmin) C(N-K, S-jmin) / C(N, S) with S - jmin = N - K,
  // so C(N-K, N-K) = 1.  Only reached far from the operating point (M near N).
  auto lc = [](double n, double r) { return std::lgamma(n + 1) - std::lgamma(r + 1) - std::lgamma(n - r + 1); };
  return lc((double)K, (double)jmin) - lc((double)N, (double)S);
}

}  // namespace

double hyp_cdf(int64_t j, int64_t N, int64_t K, int64_t S) {
  if (j < 0) return 0.0;
  const int64_t jmin = std::max<int64_t>(0, S + K - N);
  const int64_t jmax = std::min<int64_t>(K, S);
  if (j >= jmax) return 1.0;
  if (j < jmin) return 0.0;
  double lp = log_pmf_at_min(N, K, S, jmin);
  // sum_{i=jmin}^{j} exp(lp_i), with a running max shift
  double mx = lp, sum = 1.0;  // sum of exp(lp_i - mx)
  for (int64_t i = jmin; i < j; ++i) {
    const double num = (double)(K - i) * (double)(S - i);
    const double den = (double)(i + 1) * (double)(N - K - S + i + 1);
    lp += std::log(num) - std::log(den);
    if (lp > mx) {
      sum = sum * std::exp(mx - lp) + 1.0;
      mx = lp;
    } else {
      sum += std::exp(lp - mx);
    }
  }
  const double r = std::exp(mx + std::log(sum));
  return r > 1.0 ? 1.0 : r;
}

double hyp_upper_tail(int64_t j, int64_t N, int64_t K, int64_t S) {
  // Pr(X > j) = 1 - F(j)
  return 1.0 - hyp_cdf(j, N, K, S);
}

int64_t hyp_quantile(double p, int64_t N, int64_t K, int64_t S) {
  // min{j in 0..min(K,S) : F(j) >= p} (P1 Eq. 2), walking the pmf upward
  const int64_t jmin = std::max<int64_t>(0, S + K - N);
  const int64_t jmax = std::min<int64_t>(K, S);
  double lp = log_pmf_at_min(N, K, S, jmin);
  double cdf = std::exp(lp);
  int64_t j = jmin;
  while (j < jmax && cdf < p) {
    const double num = (double)(K - j) * (double)(S - j);
    const double den = (double)(j + 1) * (double)(N - K - S + j + 1);
    lp += std::log(num) - std::log(den);
    ++j;
    cdf += std::exp(lp);
  }
  return j;
}

double normal_upper_quantile(double q) {
  // z with Q(z) = 0.5 erfc(z / sqrt 2) = q, 0 < q < 1, by bisection (Q is decreasing)
  double lo = -40.0, hi = 40.0;
  for (int it = 0; it < 200; ++it) {
    const double mid = 0.5 * (lo + hi);
    const double Q = 0.5 * std::erfc(mid / std::sqrt(2.0));
    if (Q > q)
      lo = mid;
    else
      hi = mid;
    if (hi - lo <= 1e-15 * std::max(1.0, std::fabs(mid))) break;
  }
  return 0.5 * (lo + hi);
}

// Phi^-1(p), 0 < p < 1, by P. J. Acklam's rational approximation (relative error below
// 1.15e-9): one rational function of (p - 1/2)^2 in the centre and one of
// sqrt(-2 log(tail)) in each tail.  This is the "rational approximation" of P1
// Algorithm 1, line 1; it needs elementary arithmetic only.
double acklam_inv_phi(double p) {
  static const double a[6] = {-3.969683028665376e+01, 2.209460984245205e+02, -2.759285104469687e+02,
                              1.383577518672690e+02,  -3.066479806614716e+01, 2.506628277459239e+00};
  static const double b[5] = {-5.447609879822406e+01, 1.615858368580409e+02, -1.556989798598866e+02,
                              6.680131188771972e+01,  -1.328068155288572e+01};
  static const double c[6] = {-7.784894002430293e-03, -3.223964580411365e-01, -2.400758277161838e+00,
                              -2.549732539343734e+00, 4.374664141464968e+00,  2.938163982698783e+00};
  static const double d[4] = {7.784695709041462e-03, 3.224671290700398e-01, 2.445134137142996e+00,
                              3.754408661907416e+00};
  const double p_low = 0.02425;
  auto tail = [&](double q) {  // q = sqrt(-2 log(tail probability))
    return (((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
           ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1.0);
  };
  if (p < p_low) return tail(std::sqrt(-2.0 * std::log(p)));
  if (p > 1.0 - p_low) return -tail(std::sqrt(-2.0 * std::log1p(-p)));
  const double q = p - 0.5, r = q * q;
  return (((((a[0] * r + a[1]) * r + a[2]) * r + a[3]) * r + a[4]) * r + a[5]) * q /
         (((((b[0] * r + b[1]) * r + b[2]) * r + b[3]) * r + b[4]) * r + 1.0);
}

// 1 / r(k), the calibrated ratio of the per-element costs of selecting from the
// buffer and of sampling (P1 App. E.1): 1/r = a log2 k - b for k > 2^7, r infinite
// (returned as 0) below.  The page prints a = 0.59, b = 4.3; its Table 3 S column is
// reproduced exactly, for all 21 rows, only by the unrounded a = 0.594, b = 4.29.
double cost_ratio_inverse(int64_t k, double a, double b) {
  if (k <= 128) return 0.0;
  if (a <= 0.0 && b <= 0.0) {
    a = 0.594;
    b = 4.29;
  }
  const double v = a * std::log2((double)k) - b;
  return v > 0.0 ? v : 0.0;
}

namespace {

// The cost model's ratio measured on MI355X (P1 App. E.1's procedure: a sweep of S =
// 2^12 .. 2^18 over N = 2^22 .. 2^30 and k = 2^5 .. 2^19, exact (t*, M*), eps = 1e-3,
// standard normal inputs).  The refinement here is a binned selection whose cost per
// buffer slot hardly changes with k, so one constant 1/r serves every k: r is about
// 45, i.e. one sampled element (a random gather plus a hash-set insert) costs as much
// as selecting some 45 buffer slots.  The page's floor for k/N > 2^-10 is dropped: the
// threshold select here does not grow costlier with t, and the floor cost 13% at
// N = 2^28, k = 2^19.  With S in [2^12, 2^17] the rule lands within 0.4% of the
// sweep's best latency on average and 5.4% at worst.
constexpr double kMi355xInvR = 0.022;
constexpr int64_t kMi355xSMin = int64_t(1) << 12;
constexpr int64_t kMi355xSMax = int64_t(1) << 17;

// P1 Algorithm 1 lines 1-4: S from the cost model of Proposition 7, clipped, for a
// given 1/r; `dense_floor`: S_min once k/N > 2^-10 (line 4's second clause).
int64_t s_prop7(int64_t N, int64_t k, double z, double inv_r, int64_t s_min, int64_t s_max, bool dense_floor,
                double* raw) {
  const double kappa = z * z + 0.5;
  if (inv_r <= 0.0 || (dense_floor && (double)k / (double)N > std::ldexp(1.0, -10))) {
    *raw = 0.0;
    return s_min;
  }
  const double s1 = std::pow(z * inv_r, 2.0 / 3.0) * std::cbrt((double)k * (double)N);
  const double s2 = std::sqrt(kappa * (double)N * inv_r);
  *raw = std::max(s1, s2);
  const int64_t S = (int64_t)std::floor(*raw);
  return std::max(s_min, std::min(s_max, S));
}

int64_t s_cost_model(int64_t N, int64_t k, double z, int64_t s_min, int64_t s_max, double a, double b,
                     double* raw) {
  return s_prop7(N, k, z, cost_ratio_inverse(k, a, b), s_min, s_max, true, raw);
}

// P1 Algorithm 1 lines 5-15: threshold rank by the skewness-corrected normal quantile
// (Eq. 10, mu >= 15) or the Poisson quantile (Eq. 11), then the Wilson-Hilferty
// quantile of the Gamma approximation of R for the buffer (Eq. 12).
void fast_t_m(int64_t N, int64_t k, int64_t S, double eps, double z, int64_t* t_out, int64_t* m_out) {
  const double mu = (double)(k - 1) * (double)S / (double)N;
  int64_t t;
  if (mu >= 15.0) {
    const double sigma = std::sqrt(mu * (1.0 - (double)(k - 1) / (double)N) * (double)(N - S) / (double)(N - 1));
    t = (int64_t)std::ceil(mu + z * sigma + (z * z - 1.0) / 6.0) + 1;
  } else {
    double p = std::exp(-mu), c = p;
    int64_t j = 0;
    while (c < 1.0 - eps / 2.0 && j < S) {
      ++j;
      p = p * mu / (double)j;
      c += p;
    }
    t = j + 1;
  }
  const double h = 1.0 / (9.0 * (double)t);
  const double w = 1.0 - h + z * std::sqrt(h);
  *t_out = t;
  *m_out = (int64_t)std::ceil((double)(N + 1) / (double)(S + 1) * (double)t * w * w * w);
}

}  // namespace

int solve(int64_t N, int64_t k, double eps, const profk_options* opt, profk_params* out) {
  if (!out) return PROFK_EINVAL;
  if (N < 1 || k < 1 || k > N || !(eps > 0.0 && eps < 1.0)) return PROFK_EINVAL;
  if (N >= (int64_t(1) << 32)) return PROFK_EUNSUPPORTED;
  profk_params p{};
  p.N = N;
  p.k = k;
  p.eps = eps;
  p.eps_a = eps / 2.0;
  p.eps_b = eps / 2.0;
  p.z_a = normal_upper_quantile(p.eps_a);
  p.z = 2.0 * p.z_a;

  const bool fast = opt && opt->param_mode == PROFK_PARAMS_FAST;
  const bool cost_model = opt && opt->s_rule == PROFK_S_RULE_COST_MODEL;
  // Algorithm 1 of P1 uses a single z = Phi^-1(1 - eps/2) from a rational approximation
  const double z1 = fast ? -acklam_inv_phi(p.eps_a) : p.z_a;
  int64_t S;
  if (cost_model) {
    const int64_t s_min = (opt->s_min > 0) ? opt->s_min : (int64_t(1) << 14);
    const int64_t s_max = (opt->s_max > 0) ? opt->s_max : (int64_t(1) << 18);
    S = s_cost_model(N, k, z1, s_min, s_max, opt->cost_a, opt->cost_b, &p.S_raw);
  } else if (opt && opt->s_rule == PROFK_S_RULE_MI355X) {
    const int64_t s_min = (opt->s_min > 0) ? opt->s_min : kMi355xSMin;
    const int64_t s_max = (opt->s_max > 0) ? opt->s_max : kMi355xSMax;
    S = s_prop7(N, k, z1, kMi355xInvR, s_min, s_max, false, &p.S_raw);
  } else {
    const int64_t s_min = (opt && opt->s_min > 0) ? opt->s_min : 32768;
    const int64_t s_max = (opt && opt->s_max > 0) ? opt->s_max : 131072;
    const double c = (opt && opt->s_prefactor > 0.0) ? opt->s_prefactor : 1.0;
    p.S_raw = c * std::cbrt((double)k * (double)(N - k));
    S = (int64_t)std::floor(p.S_raw + 0.5);
    S = std::max(s_min, std::min(s_max, S));
  }
  // Short inputs: at most N/128 samples (P1 App. B Table 3 samples N/128 = 8192 at
  // N = 2^20; the clamp above is stated for large tensors).  No effect for N >= 2^22.
  S = std::min<int64_t>(S, std::max<int64_t>(1, N / 128));
  if (opt && opt->s_override > 0) S = opt->s_override;
  S = std::min(S, N);
  p.S = S;

  if (fast) {
    // closed forms only: no hypergeometric sums (P1 Algorithm 1)
    int64_t tf = 0, mf = 0;
    fast_t_m(N, k, S, eps, z1, &tf, &mf);
    p.z_a = z1;  // the approximated quantile is the one reported
    p.z = 2.0 * z1;
    p.t_star = -1;
    p.M_star = -1;
    p.M_cf = (double)k + p.z * std::sqrt((double)k * (double)(N - k) / (double)S * (1.0 - (double)S / (double)N));
    const double a = (double)k / (double)N, f = 1.0 - (double)S / (double)N;
    p.t_eq6 = (int64_t)std::ceil((double)S * a + p.z_a * std::sqrt((double)S * a * (1.0 - a) * f));
    const bool t_ok = tf <= S;
    p.t = std::min<int64_t>(tf, S);
    p.M = std::max<int64_t>(mf, k);
    if (opt->force_t > 0) p.t = std::min<int64_t>(opt->force_t, S);
    if (opt->force_M > 0) p.M = std::max<int64_t>(opt->force_M, k);
    p.M = std::min<int64_t>(p.M, N);
    p.p_recall = -1.0;
    p.p_overflow = -1.0;
    p.E_R = (double)(N + 1) * (double)p.t / (double)(S + 1);
    p.Var_R = (double)p.t * (double)(S - p.t + 1) * (double)(N + 1) * (double)(N - S) /
              (((double)S + 1.0) * ((double)S + 1.0) * ((double)S + 2.0));
    const bool forced = opt->force_t > 0 || opt->force_M > 0;
    p.direct_exact = (!t_ok || 2 * S > N || (!forced && 2 * p.M > N)) ? 1 : 0;
    *out = p;
    return PROFK_OK;
  }

  p.t_star = hyp_quantile(1.0 - p.eps_a, N, k - 1, S) + 1;
  // If t* > S the recall budget cannot be met (Theorem 4's condition on eps_A fails).
  const bool t_ok = p.t_star <= S;
  if (t_ok) {
    int64_t lo = k, hi = N;  // F_{N,N,S}(t-1) = 0 since X = S >= t
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo) / 2;
      if (hyp_cdf(p.t_star - 1, N, mid, S) <= p.eps_b)
        hi = mid;
      else
        lo = mid + 1;
    }
    p.M_star = lo;
  } else {
    p.M_star = N;
  }
  p.M_cf = (double)k + p.z * std::sqrt((double)k * (double)(N - k) / (double)S * (1.0 - (double)S / (double)N));
  const double a = (double)k / (double)N, f = 1.0 - (double)S / (double)N;
  p.t_eq6 = (int64_t)std::ceil((double)S * a + p.z_a * std::sqrt((double)S * a * (1.0 - a) * f));

  p.t = std::min<int64_t>(p.t_star, S);
  p.M = std::max<int64_t>(p.M_star, (int64_t)std::ceil(p.M_cf));
  if (opt && opt->force_t > 0) p.t = std::min<int64_t>(opt->force_t, S);
  if (opt && opt->force_M > 0) p.M = std::max<int64_t>(opt->force_M, k);
  p.M = std::min<int64_t>(p.M, N);

  p.p_recall = hyp_upper_tail(p.t - 1, N, k - 1, S);
  p.p_overflow = hyp_cdf(p.t - 1, N, p.M, S);
  p.E_R = (double)(N + 1) * (double)p.t / (double)(S + 1);
  p.Var_R = (double)p.t * (double)(S - p.t + 1) * (double)(N + 1) * (double)(N - S) /
            (((double)S + 1.0) * ((double)S + 1.0) * ((double)S + 2.0));

  // The sampled path pays for itself only while sample and buffer are small next to N
  // (P2 "Graceful Degradation via Fallback": fall back to the exact selection when
  // the conditions are not met economically).
  const bool forced = opt && (opt->force_t > 0 || opt->force_M > 0);
  p.direct_exact = (!t_ok || 2 * S > N || (!forced && 2 * p.M > N)) ? 1 : 0;
  *out = p;
  return PROFK_OK;
}

namespace {
std::mutex g_memo_mu;
std::map<std::tuple<int64_t, int64_t, double, int64_t, int64_t, int64_t, double, int64_t, int64_t, int32_t, double,
                    double>,
         profk_params>
    g_memo;
}  // namespace

int solve_memo(int64_t N, int64_t k, double eps, const profk_options* opt, profk_params* out) {
  profk_options o{};
  if (opt) o = *opt;
  // the closed forms cost microseconds: computed on every call (P1 §4, for
  // configurations that change from call to call)
  if (o.param_mode == PROFK_PARAMS_FAST) return solve(N, k, eps, &o, out);
  auto key = std::make_tuple(N, k, eps, o.s_override, o.s_min, o.s_max, o.s_prefactor, o.force_t, o.force_M,
                             o.s_rule, o.cost_a, o.cost_b);
  {
    std::lock_guard<std::mutex> g(g_memo_mu);
    auto it = g_memo.find(key);
    if (it != g_memo.end()) {
      if (out) *out = it->second;
      return PROFK_OK;
    }
  }
  profk_params p{};
  int rc = solve(N, k, eps, opt, &p);
  if (rc != PROFK_OK) return rc;
  {
    std::lock_guard<std::mutex> g(g_memo_mu);
    if (g_memo.size() > 4096) g_memo.clear();
    g_memo[key] = p;
  }
  if (out) *out = p;
  return PROFK_OK;
}

}  // namespace profk
