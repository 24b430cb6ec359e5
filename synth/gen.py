"""Seeded synthetic inputs with the shapes and value distributions of the verification workloads.

The speculative-decoding pages measure on real models (a 70B-class target with a ~1B draft,
vocabularies of 128256 / 152064 tokens) over GSM8k; no weights or dataset exist here, so these
generators stand in for them:

* draft logits  z_q ~ N(0, sigma_d^2)  (or a Zipf-shaped rank profile plus N(0,1) jitter);
* target logits z_p = z_q + N(0, sigma_n^2), added in fp32 before any bf16 cast;
* draft tokens  x_i drawn from the draft distribution at temperature T (Gumbel-max), or, when a
  Saguaro set S_i is given, from the draft distribution with the weight of S_i scaled by C;
* verification uniforms u in [0, 1), fp32, one per draft position plus one for the bonus token.

Random streams: ``SeedSequence(seed).spawn(6)`` gives, in order, draft logits, target noise,
draft-token sampling, verification uniforms, speculation-branch rows and the branch rows' sampling
uniforms (a child stream depends only on its index, so adding the sixth left the others as they
were).  bf16 values are made by round-to-nearest-even from fp32 and are carried as their uint16
bit patterns.

Nothing here computes a softmax, an acceptance test, a residual or a sampler inverse CDF.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

BF16 = "bf16"
F32 = "f32"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    # +-inf survive the rounding above; NaN is not produced by these generators.
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _streams(seed: int, n: int = 6):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def _as_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(a) if dtype == BF16 else a


@dataclass
class VerifyBatch:
    """One verification batch.

    draft   [B, K+1, V]  draft logits; rows 0..K-1 are verified, row K feeds the k=K guesses.
    target  [B, K+1, V]  target logits.
    x       [B, K]       int32 draft tokens.
    u       [B, K+1]     fp32 uniforms; u[:, K] samples the bonus token.
    sets    [B, K, F]    int32 Saguaro sets (-1 padded) or None.
    Logit arrays are float32, or uint16 bf16 bit patterns when dtype == "bf16".
    """

    dtype: str
    B: int
    K: int
    V: int
    T: float
    draft: np.ndarray
    target: np.ndarray
    x: np.ndarray
    u: np.ndarray
    sets: Optional[np.ndarray] = None
    C: float = 1.0
    meta: dict = field(default_factory=dict)


def _draft_logits(rng, rows: int, V: int, sigma: float, zipf_s: Optional[float]) -> np.ndarray:
    if zipf_s is None:
        out = rng.standard_normal((rows, V), dtype=np.float32)
        out *= np.float32(sigma)
        return out
    # Zipf-shaped rank profile: z = -s * ln(rank) + N(0, 1), ranks a per-row random permutation.
    ln_rank = np.log(np.arange(1, V + 1, dtype=np.float64)).astype(np.float32)
    out = np.empty((rows, V), dtype=np.float32)
    for r in range(rows):
        perm = rng.permutation(V)
        np.multiply(ln_rank[perm], np.float32(-zipf_s), out=out[r])
        out[r] += rng.standard_normal(V, dtype=np.float32)
    return out


def _top_by_logit(z: np.ndarray, F: int) -> np.ndarray:
    """Indices of the F largest values of one row, ties to the smaller index (the draft side's
    choice of tokens to cache)."""
    if F <= 0:
        return np.empty(0, dtype=np.int64)
    order = np.argsort(-z.astype(np.float64), kind="stable")
    return order[:F]


def make_verify_batch(
    B: int,
    K: int,
    V: int,
    dtype: str,
    seed: int,
    *,
    T: float = 1.0,
    draft_sigma: float = 2.0,
    noise_sigma: float = 0.5,
    zipf_s: Optional[float] = None,
    sag_sizes: Optional[Sequence[int]] = None,
    C: float = 1.0,
) -> VerifyBatch:
    """Draw a verification batch.

    ``sag_sizes`` (length K) turns on Saguaro sampling: the set of draft row i holds its
    ``sag_sizes[i]`` largest raw logits, and x_i is drawn with those tokens' weight scaled by C.
    """
    assert dtype in (BF16, F32)
    r_logit, r_noise, r_draw, r_unif = _streams(seed)[:4]
    rows = B * (K + 1)
    zq = _draft_logits(r_logit, rows, V, draft_sigma, zipf_s)
    zp = zq + np.float32(noise_sigma) * r_noise.standard_normal((rows, V), dtype=np.float32)
    if dtype == BF16:
        draft = f32_to_bf16_bits(zq).reshape(B, K + 1, V)
        target = f32_to_bf16_bits(zp).reshape(B, K + 1, V)
    else:
        draft = zq.reshape(B, K + 1, V)
        target = zp.astype(np.float32).reshape(B, K + 1, V)
    del zq, zp

    sets = None
    if sag_sizes is not None:
        sag_sizes = [int(f) for f in sag_sizes]
        assert len(sag_sizes) == K
        Fm = max(1, max(sag_sizes))
        sets = np.full((B, K, Fm), -1, dtype=np.int32)

    x = np.empty((B, K), dtype=np.int32)
    inv_t = 1.0 / float(T)
    for b in range(B):
        for i in range(K):
            z = _as_f32(draft[b, i], dtype).astype(np.float64)
            score = z * inv_t
            if sets is not None and sag_sizes[i] > 0:
                s = _top_by_logit(z, sag_sizes[i])
                sets[b, i, : len(s)] = s
                with np.errstate(divide="ignore"):
                    score[s] += np.log(C)
            g = -np.log(-np.log(r_draw.random(V)))
            x[b, i] = int(np.argmax(score + g))
    u = r_unif.random((B, K + 1), dtype=np.float32)
    return VerifyBatch(dtype=dtype, B=B, K=K, V=V, T=float(T), draft=draft, target=target, x=x, u=u,
                       sets=sets, C=float(C))


def make_branch_rows(B: int, budget: int, K: int, V: int, dtype: str, seed: int,
                     draft_sigma: float = 2.0) -> np.ndarray:
    """Draft logits of the speculation-cache branches: [B, budget, K, V] (one K-token continuation
    per cached outcome), same value distribution as the draft rows."""
    rng = _streams(seed)[4]
    z = rng.standard_normal((B * budget * K, V), dtype=np.float32)
    z *= np.float32(draft_sigma)
    if dtype == BF16:
        return f32_to_bf16_bits(z).reshape(B, budget, K, V)
    return z.reshape(B, budget, K, V)


def make_branch_uniforms(B: int, budget: int, K: int, seed: int) -> np.ndarray:
    """Uniforms in [0, 1), fp32, [B, budget, K]: one per branch row, for drawing its draft token."""
    return _streams(seed)[5].random((B, budget, K), dtype=np.float32)


# The five workloads: verification at several scales, and two SSD rounds (cache build and full round).
WORKLOADS = {
    "b1_k4_v32000_f32": dict(B=1, K=4, V=32000, dtype=F32, T=1.0),
    "b16_k4_v128256_bf16_top3": dict(B=16, K=4, V=128256, dtype=BF16, T=1.0, topf=3),
    "ssd_build_b16x12_k4_v128256_bf16": dict(B=16, K=4, V=128256, dtype=BF16, T=1.0, budget=12, a=0.7,
                                              r=1.0, C=0.5),
    "b128_k8_v152064_f32_zipf_top4": dict(B=128, K=8, V=152064, dtype=F32, T=0.7, zipf_s=1.1,
                                          noise_sigma=0.8, topf=4),
    "ssd_round_b64x32_k4_v128256_f32": dict(B=64, K=4, V=128256, dtype=F32, T=1.0, budget=32, a=0.7,
                                             r=1.0, C=0.3),
}


def workload(name: str) -> dict:
    return dict(WORKLOADS[name])
