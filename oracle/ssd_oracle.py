"""Plain float64 reference of the verification hot path (test infrastructure only; see package doc).

Sources, by page title:
  [SSD]  "论文阅读：Speculative Speculative Decoding — 消除推测解码的最后一个顺序瓶颈"
         (xiaohongrsx.github.io/posts/ssd-paper-reading)
  [SD7.3] "7.3 Speculative Decoding：投机采样加速" (aiknowledge.cn)
  [HW]   "推测解码：用一个“小模型”骗出 3 倍推理速度" (bbs.huaweicloud.com/blogs/510880)

Readings where the pages are silent or garbled (each the plainest one the rest supports):
  * temperature: both distributions are softmax(z / T) with one T > 0;
  * acceptance: accept x iff u * q'(x) < p(x), u in [0, 1) (so p >= q' always accepts);
  * a rejection resamples from the normalised residual max(p - q', 0), the only choice that keeps
    the output distribution equal to p as all three pages assert;
  * the bonus uses its own uniform u[K]; the inverse CDF runs in ascending token order and picks the
    first token whose cumulative residual exceeds u * R;
  * if every draft token is accepted, the bonus is drawn from the target row K (0-based) with R = 1;
    an all-zero residual (reachable only through rounding) falls back to the target row, R = 1;
  * Saguaro: the draft probability of each token of the set S is multiplied by C, the others keep
    their weight, and the row is renormalised;
  * top-F orders raw logits descending, ties to the smaller index, never returns -inf, pads with -1;
  * geometric acceptance law P(k) = (1 - a) a^k for k < K and a^K for k = K; power-law miss model
    sum_k P(k) F_k^-r; integer fan-out by largest remainder, ties to the smaller k.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np


# ----------------------------------------------------------------------------------------------
# inputs
# ----------------------------------------------------------------------------------------------
def logits_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored logits: fp32 arrays, or bf16 carried as uint16 bit patterns."""
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------------------
# distributions
# ----------------------------------------------------------------------------------------------
def softmax_t(z: np.ndarray, T: float) -> np.ndarray:
    """Temperature softmax of one logit row: each position's output is a probability distribution
    over the vocabulary ([SSD] "为什么大模型能并行验证"; [SD7.3] 7.3.3 names q(x), p(x))."""
    if not (T > 0.0 and math.isfinite(T)):
        raise ValueError("temperature must be finite and > 0")
    y = np.asarray(z, dtype=np.float64) / T
    m = np.max(y)
    e = np.exp(y - m)
    return e / np.sum(e)


def _valid_set(S: Optional[Sequence[int]], V: int) -> list:
    """Distinct in-range entries of a Saguaro set, in their given order (-1 and duplicates ignored)."""
    out = []
    if S is None:
        return out
    for s in S:
        s = int(s)
        if 0 <= s < V and s not in out:
            out.append(s)
    return out


def saguaro(q: np.ndarray, S: Optional[Sequence[int]], C: float):
    """Saguaro sampling ([SSD] "Saguaro 优化二", "解法：操纵草稿分布"): multiply the draft probability
    of the F cached tokens by C, leave the rest, renormalise.

    Returns (q', sigma, N) with sigma = sum_{s in S} q(s) and N = 1 - (1 - C) sigma.
    """
    if not (0.0 <= C <= 1.0):
        raise ValueError("C must lie in [0, 1]")
    V = q.shape[0]
    idx = _valid_set(S, V)
    sigma = float(np.sum(q[idx])) if idx else 0.0
    N = 1.0 - (1.0 - C) * sigma
    if not N > 0.0:
        raise ValueError("Saguaro normaliser is not positive")
    w = np.ones(V)
    w[idx] = C
    return q * w / N, sigma, N


# ----------------------------------------------------------------------------------------------
# verification of one sequence
# ----------------------------------------------------------------------------------------------
@dataclass
class VerifyResult:
    k: int                 # accepted draft tokens, 0..K
    bonus: int             # the token emitted after them
    a: np.ndarray          # [K] min(1, p_i(x_i) / q'_i(x_i)) at every position
    R: float               # residual mass at the rejected position (1.0 when k == K)
    c_lo: float            # cumulative residual fraction just before the bonus token
    c_hi: float            # ... and including it (decision boundaries of the bonus uniform)
    fallback: bool         # residual was all zero and the target row was used instead


def verify_sequence(zq: np.ndarray, zp: np.ndarray, x: Sequence[int], u: Sequence[float], T: float,
                    sets: Optional[Sequence[Sequence[int]]] = None, C=1.0) -> VerifyResult:
    """Verify K draft tokens of one sequence.

    zq [K, V]   draft logits of the K drafted positions (float64 values)
    zp [K+1, V] target logits; row K scores the position after the last draft token
    x  [K]      draft tokens;  u [K+1] uniforms, u[K] samples the bonus token
    sets        per-position Saguaro sets (or None), C the Saguaro factor: one value for every
                position, or K values, position i down-weighting its set by C[i] ([SSD] "关于逐位置
                的思考": the pages' C is global and a per-position C is the direction they name)

    Steps ([SD7.3] 7.3.2 steps 3-4 and 7.3.3; [HW] "三、接受概率为什么是对的"; [SSD] "接受-拒绝机制"):
    accept x_i with probability min(1, p(x_i)/q(x_i)); stop at the first rejection and discard the
    later drafts; on a rejection sample the bonus from the normalised max(p - q, 0); if every draft
    is accepted, sample it from the target's extra position.
    """
    K = len(x)
    V = zq.shape[1]
    assert zq.shape[0] >= K and zp.shape == (K + 1, V) and len(u) == K + 1
    p = [softmax_t(zp[i], T) for i in range(K + 1)]
    Cs = [float(C)] * K if np.ndim(C) == 0 else [float(c) for c in C]
    assert len(Cs) == K
    qd = []
    for i in range(K):
        q = softmax_t(zq[i], T)
        if sets is not None:
            q, _, _ = saguaro(q, sets[i], Cs[i])
        qd.append(q)

    a = np.empty(K)
    k = K
    for i in range(K):
        xi = int(x[i])
        px, qx = p[i][xi], qd[i][xi]
        if qx > 0.0:
            a[i] = min(1.0, px / qx)
        else:
            a[i] = 1.0 if px > 0.0 else 0.0
        if k == K and not (float(u[i]) * qx < px):
            k = i  # first rejection: positions after it are discarded

    fallback = False
    if k < K:
        r = np.maximum(p[k] - qd[k], 0.0)
        R = float(np.sum(r))
        R_out = R
        if R == 0.0:
            r, R, fallback = p[k], 1.0, True
    else:
        r, R, R_out = p[K], 1.0, 1.0

    cum = np.cumsum(r)
    target = float(u[K]) * R
    t = int(np.searchsorted(cum, target, side="right"))  # first index with cum > target
    if t >= V:
        t = int(np.nonzero(r > 0.0)[0][-1])
    c_lo = (cum[t - 1] if t > 0 else 0.0) / R
    c_hi = cum[t] / R
    return VerifyResult(k=k, bonus=t, a=a, R=R_out, c_lo=float(c_lo), c_hi=float(c_hi),
                        fallback=fallback)


def verify_batch(draft: np.ndarray, target: np.ndarray, dtype: str, x: np.ndarray, u: np.ndarray,
                 T: float, sets: Optional[np.ndarray] = None, C=1.0, seqs=None):
    """verify_sequence over sequences of stored logits; draft [B, >=K, V], target [B, K+1, V];
    C one value or K per-position values."""
    B, K = x.shape
    seqs = range(B) if seqs is None else seqs
    out = {}
    for b in seqs:
        zq = logits_f64(draft[b, :K], dtype)
        zp = logits_f64(target[b], dtype)
        out[b] = verify_sequence(zq, zp, x[b], u[b], T, None if sets is None else sets[b], C)
    return out


# ----------------------------------------------------------------------------------------------
# SSD: bonus-token guesses, fan-out, speculation cache
# ----------------------------------------------------------------------------------------------
def topf(z: np.ndarray, F: int, exclude: int = -1) -> np.ndarray:
    """Top-F bonus-token guesses of one draft row, excluding the sampled token
    ([SSD] "怎么猜奖励 token"). Raw logits descending, ties to the smaller index; -inf never
    returned; -1 pads when fewer than F tokens remain."""
    z = np.asarray(z, dtype=np.float64)
    V = z.shape[0]
    order = np.lexsort((np.arange(V), -z))
    keep = order[(order != exclude) & (z[order] > -np.inf)]
    out = np.full(F, -1, dtype=np.int64)
    take = keep[:F]
    out[: len(take)] = take
    return out


@dataclass
class SampleResult:
    S: np.ndarray     # the Saguaro set: top-F of the row (-1 pads)
    sigma: float      # q mass of S
    N: float          # normaliser 1 - (1 - C) sigma
    x: int            # sampled draft token, -1 when q' has no mass
    qx: float         # q'(x)
    c_lo: float       # cumulative q' before x; the draw is x exactly when c_lo <= u < c_hi
    c_hi: float       # cumulative q' through x


def saguaro_sample(z: np.ndarray, T: float, F: int, C: float, u: float) -> SampleResult:
    """Draft-side Saguaro sampling of one row ([SSD] "Saguaro 优化二：Saguaro 采样",
    "解法：操纵草稿分布"): the down-weighted set is the row's own top F (raw logits, nothing
    excluded), the draft distribution is q' = saguaro(softmax_t(z, T), S, C), and the draft token
    is drawn from q' with the uniform u by the inverse CDF in ascending token order, the reading
    used for the bonus token: the first token whose cumulative q' exceeds u, or the last token of
    positive mass when u is not below the total."""
    z = np.asarray(z, dtype=np.float64)
    S = topf(z, F)
    q = softmax_t(z, T)
    qs, sigma, N = saguaro(q, [int(v) for v in S if v >= 0], C)
    cum = np.cumsum(qs)
    x = int(np.searchsorted(cum, float(u), side="right"))  # first index with cum > u
    if x >= len(qs):
        x = int(np.nonzero(qs > 0.0)[0][-1])
    c_lo = float(cum[x - 1]) if x > 0 else 0.0
    return SampleResult(S=S, sigma=float(sigma), N=float(N), x=x, qx=float(qs[x]), c_lo=c_lo,
                        c_hi=float(cum[x]))


def geometric_pk(K: int, a: float) -> np.ndarray:
    """Geometric acceptance law ([SSD] "最优扇出度分配"): P(k) = (1-a) a^k for k < K, a^K for k = K."""
    P = np.array([(1.0 - a) * a ** k for k in range(K)] + [a ** K], dtype=np.float64)
    return P


def fanout(K: int, a: float, r: float, budget: int):
    """Geometric fan-out ([SSD] "最优扇出度分配"): minimise sum_k P(k) F_k^-r subject to
    sum_k F_k = budget. Setting the Lagrangian's derivative in F_k to zero gives
    F_k proportional to P(k)^(1/(1+r)); substituting P gives F_k = F_0 a^(k/(1+r)) for k < K.

    Returns (integer F [K+1], continuous F [K+1]). Integers: floor, then the remaining units to the
    largest fractional parts, ties to the smaller k.
    """
    if K < 0 or not (0.0 < a < 1.0) or not (r > 0.0) or budget < 0:
        raise ValueError("bad fan-out arguments")
    P = geometric_pk(K, a)
    ratio = (P / P[0]) ** (1.0 / (1.0 + r))   # F_k / F_0
    F0 = budget / np.sum(ratio)              # from the budget constraint
    Fc = F0 * ratio
    Fi = np.floor(Fc).astype(np.int64)
    left = budget - int(Fi.sum())
    frac = Fc - Fi
    order = sorted(range(K + 1), key=lambda k: (-frac[k], k))
    for k in order[:left]:
        Fi[k] += 1
    return Fi, Fc


def batch_speedup(h: float, E_hit: float, E_miss: float, T_p: float, T_b: float, b: float) -> float:
    """Expected speedup over autoregressive decoding for a batch of b sequences ([SSD] "SSD 的核心思想"
    speedup formula; "解法：根据 batch 大小切换备用推测器"). The page's formulas are lost; this reading
    keeps every quantity its text names: h the cache hit rate of one sequence, E_hit / E_miss the
    expected tokens a round yields on a hit / a miss, T_p / T_b the primary / backup speculator
    latencies in units of one target verification. A round costs the verification (or the primary
    speculator when it is the slower), and the whole batch waits for the backup whenever any of its b
    sequences misses, with probability 1 - h^b:
        S(b) = (h E_hit + (1 - h) E_miss) / (max(1, T_p) + (1 - h^b) T_b).
    As b grows the miss term tends to T_b: the backup's latency bounds the speedup."""
    if not (0.0 <= h <= 1.0) or min(E_hit, E_miss, T_p, T_b) < 0.0 or not (b > 0):
        raise ValueError("bad speedup arguments")
    A = h * E_hit + (1.0 - h) * E_miss
    return A / (max(1.0, T_p) + (1.0 - h ** b) * T_b)


def backup_crossover(h: float, E_hit: float, E_miss_neural: float, T_neural: float, E_miss_fast: float,
                     T_fast: float, T_p: float):
    """Where a fast backup speculator overtakes a neural one as the batch grows ([SSD] "解法：根据
    batch 大小切换备用推测器"; "消融实验": the fast backup wins from the critical size on). Writing
    x = 1 - h^b and A = h E_hit + (1 - h) E_miss, batch_speedup equal for the two backups means
    A_n (D + x T_fast) = A_f (D + x T_neural), D = max(1, T_p), so x* = D (A_n - A_f) / (A_f T_neural -
    A_n T_fast) and b* = ln(1 - x*) / ln h.
    Returns (b_star, fast_wins_large): b_star the real batch size where the two speedups are equal
    (nan when they do not cross at any b > 0), fast_wins_large whether the fast backup is at least
    as good in the limit of large batches."""
    D = max(1.0, T_p)
    A_n = h * E_hit + (1.0 - h) * E_miss_neural
    A_f = h * E_hit + (1.0 - h) * E_miss_fast
    fast_large = A_f * (D + T_neural) >= A_n * (D + T_fast)
    den = A_f * T_neural - A_n * T_fast
    if den == 0.0 or not (0.0 < h < 1.0):
        return math.nan, bool(fast_large)
    xs = D * (A_n - A_f) / den
    if not (0.0 < xs < 1.0):
        return math.nan, bool(fast_large)
    return math.log(1.0 - xs) / math.log(h), bool(fast_large)


def cache_keys(guesses: Sequence[Sequence[int]], F: Sequence[int]):
    """Keys of one sequence's speculation cache ([SSD] "SSD 的核心思想": an outcome is (k, t), k
    drafts accepted and t the bonus token). For each k the F_k guesses of draft position k
    (0-based; position K is the extra draft row) occupy consecutive slots; a missing guess (-1)
    leaves its slot empty as (-1, -1)."""
    kk, tt = [], []
    for k, Fk in enumerate(F):
        for j in range(int(Fk)):
            t = int(guesses[k][j]) if j < len(guesses[k]) else -1
            kk.append(k if t >= 0 else -1)
            tt.append(t if t >= 0 else -1)
    return np.array(kk, dtype=np.int64), np.array(tt, dtype=np.int64)


def cache_lookup(keys_k: np.ndarray, keys_t: np.ndarray, k: int, bonus: int) -> int:
    """First slot holding the outcome (k, bonus), or -1 on a miss."""
    for j in range(len(keys_k)):
        if int(keys_k[j]) == k and int(keys_t[j]) == bonus:
            return j
    return -1


def all_hit_probability(h: float, B: int) -> float:
    """[SSD] "问题：大 batch 下缓存未命中不可避免": the batch proceeds with zero wait only if every
    one of its B sequences hits; with independent per-sequence hit rate h that is h^B."""
    return float(h) ** int(B)


def branch_layout(budget: int, K: int) -> dict:
    """Shape arithmetic of the cache build ([SSD] "并行生成所有分支", "两层 batch"): each of the
    `budget` outcomes owns a K-token continuation; drafting them one token at a time across all
    branches takes K batched forwards of `budget` rows instead of budget*K serial ones."""
    return dict(branches=budget, K=K, serial_forwards=budget * K, batched_forwards=K,
                batch_size=budget, branch_rows=budget * K)


def ssd_round(draft, target, dtype, x, u, T, sets, C, F, branch=None, seqs=None, branch_u=None):
    """One SSD round for the sampled sequences:
    guesses (top-F_k of draft row k excluding x_k for k < K, of the extra row K without exclusion),
    cache keys, Saguaro verification, cache lookup; and, for the branch rows, the Saguaro set
    (top-F of the row) with its mass and normaliser, and with branch_u ([B, budget, K] uniforms)
    the draft token each branch row draws from its q' (saguaro_sample).

    Returns {b: dict(k, bonus, guesses, keys_k, keys_t, slot, branch_sigma, branch_N
    [, branch_sample])}.
    """
    B, K = x.shape
    seqs = range(B) if seqs is None else seqs
    out = {}
    for b in seqs:
        zq = logits_f64(draft[b], dtype)
        zp = logits_f64(target[b], dtype)
        res = verify_sequence(zq[:K], zp, x[b], u[b], T, None if sets is None else sets[b], C)
        guesses = [topf(zq[i], int(F[i]), int(x[b, i])) for i in range(K)]
        guesses.append(topf(zq[K], int(F[K])))
        kk, tt = cache_keys(guesses, F)
        slot = cache_lookup(kk, tt, res.k, res.bonus)
        d = dict(verify=res, k=res.k, bonus=res.bonus, guesses=guesses, keys_k=kk, keys_t=tt, slot=slot)
        if branch is not None:
            nbr = branch.shape[1]
            sig = np.empty((nbr, K))
            nrm = np.empty((nbr, K))
            sets_b = np.empty((nbr, K, max(1, int(max(F[:K])))), dtype=np.int64)
            samples = {}
            for j in range(nbr):
                for i in range(K):
                    zb = logits_f64(branch[b, j, i], dtype)
                    if branch_u is None:
                        S = topf(zb, int(F[i]))
                        _, sig[j, i], nrm[j, i] = saguaro(softmax_t(zb, T), S, C)
                    else:
                        smp = saguaro_sample(zb, T, int(F[i]), C, float(branch_u[b, j, i]))
                        S, sig[j, i], nrm[j, i] = smp.S, smp.sigma, smp.N
                        samples[(j, i)] = smp
                    sets_b[j, i, :] = -1
                    sets_b[j, i, : len(S)] = S
            d.update(branch_sets=sets_b, branch_sigma=sig, branch_N=nrm)
            if branch_u is not None:
                d["branch_sample"] = samples
        out[b] = d
    return out
