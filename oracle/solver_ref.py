"""Double-precision reference for the Prof-K parameter choice: TEST INFRASTRUCTURE ONLY.

Pages: P1 = "Prof-K: Probabilistic One-Pass Filtering for Efficient Top-k
Selection" (arXiv HTML page); P2 = the earlier version (bittide mirror).
Every probability goes through scipy.stats.hypergeom; the GPU library has
its own C++ implementation and the two share nothing.

Definitions followed (plain readings, listed again in the design notes):

* budget split eps_A = eps_B = eps/2 (P1 §4 after Theorem 4; P1 Algorithm 1
  header).
* z_A = Phi^-1(1 - eps/2), z = z_A + z_B = 2 z_A (P2 Algorithm 1, step 1).
* S rule: S*_raw = c (k (N-k))^(1/3) with default prefactor c = 1, the
  (kN)^(1/3) rule of P2 Theorem 5, whose worked example (N = 1e9, k = 100,
  S* about 4,600) only this prefactor reproduces; P2 Eq. 14's own prefactor
  (z rho log2 k / 2)^(2/3) is kept as an option.  S = clamp(round(S*_raw),
  S_min, S_max), S_min = 32768, S_max = 131072 (P2 §4 "Optimal Sample
  Size"), round to nearest (P2 Algorithm 1, step 4), then at most N/128 (the
  S column of P1 App. B Table 3 at N = 2^20 is 8192 = N/128; the cap only
  bites below N = 2^22).
* t* = F^-1_{N,k-1,S}(1 - eps_A) + 1 and
  M* = min{M in [k, N] : F_{N,M,S}(t* - 1) <= eps_B}  (P1 §4 Theorem 4, Eq. 7),
  with F the hypergeometric CDF of P1 Eq. 1-2.
* M_cf = k + z sqrt(k (N-k) / S * (1 - S/N))  (P2 Corollary 4, Eq. 12);
  operating M = max(M*, ceil(M_cf)), operating t = t*.
* t_eq6 = ceil(S a + z_A sqrt(S a (1-a) f)), a = k/N, f = 1 - S/N (P2 Eq. 6),
  reported only.
* Pr(R < k) = 1 - F_{N,k-1,S}(t-1)  (P1 Proposition 2, Eq. 5);
  Pr(R > M) = F_{N,M,S}(t-1)  (P1 Proposition 3, Eq. 6).
* E[R] = (N+1) t / (S+1),
  Var[R] = t (S-t+1)(N+1)(N-S) / ((S+1)^2 (S+2))  (P2 Lemma 1, Eq. 2).

Parity unpinned: s_rule_mi355x (its cost ratio and clip range are measured on
MI355X, see MI355X_INV_R).  Every other function here is pinned by the tests
(P1 Table 3, the worked examples, exhaustive enumeration, Corollary 5).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

from scipy.stats import hypergeom, norm

S_MIN_DEFAULT = 32768
S_MAX_DEFAULT = 131072


def hyp_cdf(j: int, N: int, K: int, S: int) -> float:
    """F_{N,K,S}(j) = Pr(X <= j), X ~ Hypergeometric(N, K, S) (P1 Eq. 1)."""
    if j < 0:
        return 0.0
    return float(hypergeom.cdf(j, N, K, S))


def hyp_sf(j: int, N: int, K: int, S: int) -> float:
    """Pr(X > j) for X ~ Hypergeometric(N, K, S)."""
    if j < 0:
        return 1.0
    return float(hypergeom.sf(j, N, K, S))


def hyp_quantile(p: float, N: int, K: int, S: int) -> int:
    """F^-1_{N,K,S}(p) = min{j in 0..S : F(j) >= p} (P1 Eq. 2), by direct scan."""
    j = 0
    hi = min(K, S)
    while j < hi and hyp_cdf(j, N, K, S) < p:
        j += 1
    return j


def z_upper(eps_half: float) -> float:
    """Phi^-1(1 - eps_half)."""
    return float(norm.isf(eps_half))


def s_rule(N: int, k: int, eps: float, s_min: int = S_MIN_DEFAULT, s_max: int = S_MAX_DEFAULT,
           prefactor: float = 1.0, eq14_rho: float | None = None) -> tuple[float, int]:
    """(S*_raw, S).  With eq14_rho given, P2 Eq. 14's prefactor with log2 k is used."""
    z = 2.0 * z_upper(eps / 2.0)
    base = (k * (N - k)) ** (1.0 / 3.0)
    if eq14_rho is not None:
        lg = math.log2(k) if k > 1 else 0.0
        raw = ((z * eq14_rho * lg) / 2.0) ** (2.0 / 3.0) * base
    else:
        raw = prefactor * base
    S = int(math.floor(raw + 0.5))
    S = max(s_min, min(s_max, S))
    # short inputs: at most N/128 samples (P1 App. B Table 3 uses S = 8192 = N/128 at
    # N = 2^20); no effect for N >= 2^22
    S = min(S, max(1, N // 128))
    S = min(S, N)
    return raw, S


def t_star(N: int, k: int, S: int, eps_a: float) -> int:
    """P1 Theorem 4, Eq. 7 (first line)."""
    return hyp_quantile(1.0 - eps_a, N, k - 1, S) + 1


def m_star(N: int, k: int, S: int, t: int, eps_b: float) -> int:
    """P1 Theorem 4, Eq. 7 (second line), by binary search over {k..N}; G(M) =
    F_{N,M,S}(t-1) is nonincreasing in M (P1 Lemma 1)."""
    lo, hi = k, N  # F_{N,N,S}(t-1) = 0 <= eps_b, so hi is feasible
    while lo < hi:
        mid = (lo + hi) // 2
        if hyp_cdf(t - 1, N, mid, S) <= eps_b:
            hi = mid
        else:
            lo = mid + 1
    return lo


@dataclass
class RefParams:
    N: int
    k: int
    eps: float
    S_raw: float
    S: int
    z_a: float
    z: float
    t_star: int
    M_star: int
    M_cf: float
    t_eq6: int
    t: int
    M: int
    p_recall: float
    p_overflow: float
    E_R: float
    Var_R: float


def solve(N: int, k: int, eps: float, S: int | None = None, s_min: int = S_MIN_DEFAULT,
          s_max: int = S_MAX_DEFAULT, prefactor: float = 1.0) -> RefParams:
    eps_a = eps_b = eps / 2.0
    z_a = z_upper(eps_a)
    z = 2.0 * z_a
    raw, s_auto = s_rule(N, k, eps, s_min, s_max, prefactor)
    if S is None:
        S = s_auto
    ts = t_star(N, k, S, eps_a)
    ms = m_star(N, k, S, ts, eps_b)
    m_cf = k + z * math.sqrt(k * (N - k) / S * (1.0 - S / N))
    a = k / N
    f = 1.0 - S / N
    t6 = int(math.ceil(S * a + z_a * math.sqrt(S * a * (1.0 - a) * f)))
    t = ts
    M = max(ms, int(math.ceil(m_cf)))
    M = min(M, N)
    p_rec = hyp_sf(t - 1, N, k - 1, S)
    p_ovf = hyp_cdf(t - 1, N, M, S)
    e_r = (N + 1) * t / (S + 1)
    var_r = t * (S - t + 1) * (N + 1) * (N - S) / ((S + 1) ** 2 * (S + 2))
    return RefParams(N, k, eps, raw, S, z_a, z, ts, ms, m_cf, t6, t, M, p_rec, p_ovf, e_r, var_r)


def inv_cost_ratio(k: int, a: float = 0.594, b: float = 4.29) -> float:
    """1/r(k) of the cost model (P1 App. E.1): a log2 k - b for k > 2^7, and 0
    (r infinite) below.  The page prints a = 0.59, b = 4.3; the unrounded
    a = 0.594, b = 4.29 are the reading, because only they reproduce the S
    column of P1 App. B Table 3 (all 21 rows)."""
    if k <= 128:
        return 0.0
    return max(0.0, a * math.log2(k) - b)


def s_rule_cost_model(N: int, k: int, eps: float, s_min: int = 1 << 14, s_max: int = 1 << 18,
                      a: float = 0.594, b: float = 4.29, inv_r: float | None = None,
                      dense_floor: bool = True) -> int:
    """P1 Algorithm 1 lines 1-4 (Proposition 7): S1 = (z/r)^(2/3) (kN)^(1/3),
    S2 = (kappa N / r)^(1/2), kappa = z^2 + 1/2, z = Phi^-1(1 - eps/2);
    S = clip(floor(max(S1, S2)), S_min, S_max), and S_min when r is infinite or
    k/N > 2^-10.  Then at most N/128 and at most N, as for the default rule.
    1/r is a log2 k - b, or the given constant inv_r for every k; without
    dense_floor the k/N > 2^-10 clause is left out."""
    z = z_upper(eps / 2.0)
    kappa = z * z + 0.5
    if inv_r is None:
        inv_r = inv_cost_ratio(k, a, b)
    if inv_r <= 0.0 or (dense_floor and k / N > 2.0 ** -10):
        S = s_min
    else:
        s1 = (z * inv_r) ** (2.0 / 3.0) * (k * N) ** (1.0 / 3.0)
        s2 = math.sqrt(kappa * N * inv_r)
        S = max(s_min, min(s_max, int(math.floor(max(s1, s2)))))
    S = min(S, max(1, N // 128))
    return min(S, N)


# The cost ratio measured on MI355X with the sweep of P1 App. E.1 (bench.py
# --calibrate-s): one constant for every k, its clip range, and no floor for dense k.
# PARITY UNPINNED: these three numbers are a measured input (timings of the HIP path
# on one MI355X), not something the pages print or the mathematics fixes, so the
# library's PROFK_S_RULE_MI355X agreeing with s_rule_mi355x only checks that both
# sides apply the same formula to the same constants.  S changes the speed of a call,
# never its result: no parity of the top-k output depends on these values.
MI355X_INV_R = 0.022
MI355X_S_MIN = 1 << 12
MI355X_S_MAX = 1 << 17


def s_rule_mi355x(N: int, k: int, eps: float) -> int:
    """Algorithm 1 lines 1-4 with the MI355X cost ratio."""
    return s_rule_cost_model(N, k, eps, s_min=MI355X_S_MIN, s_max=MI355X_S_MAX, inv_r=MI355X_INV_R,
                             dense_floor=False)


def surrogate_params(N: int, k: int, S: int, eps: float) -> tuple[int, int]:
    """P1 Algorithm 1 / App. B closed forms (Eq. 10, 11, 12) for a given S: (t, M).
    Phi^-1 comes from scipy here (the page uses a rational approximation)."""
    z = z_upper(eps / 2.0)
    mu = (k - 1) * S / N
    if mu >= 15:
        sigma = math.sqrt(mu * (1.0 - (k - 1) / N) * (N - S) / (N - 1))
        t = int(math.ceil(mu + z * sigma + (z * z - 1.0) / 6.0)) + 1
    else:
        p = math.exp(-mu)
        c = p
        j = 0
        while c < 1.0 - eps / 2.0:
            j += 1
            p = p * mu / j
            c += p
        t = j + 1
    h = 1.0 / (9.0 * t)
    M = int(math.ceil((N + 1) / (S + 1) * t * (1.0 - h + z * math.sqrt(h)) ** 3))
    return t, M
