"""Shared helpers for the GPU parity tests: device copies of seeded batches and comparison with the
oracle under the boundary-case rule.

Rule: accepted lengths, bonus tokens and top-F sets must equal the oracle's bit for bit, except
where a uniform lies within BOUNDARY = 1e-5 of a decision boundary computed by the oracle in
float64: |u_i - a_i| for a position the decision passed through, or |u_K - c| for the cumulative
residual fractions c on either side of the oracle's bonus token. Such cases are counted and
reported; every other case must match. Probabilities must agree to PROB_ATOL = 1e-5.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
import synth

BOUNDARY = 1e-5
PROB_ATOL = 1e-5
DEV = "cuda:0"


def logits_to_device(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == synth.BF16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def batch_to_device(bt: synth.VerifyBatch, verify_rows_only: bool = True) -> dict:
    d = dict(
        draft=logits_to_device(bt.draft[:, : bt.K] if verify_rows_only else bt.draft, bt.dtype),
        target=logits_to_device(bt.target, bt.dtype),
        x=torch.from_numpy(bt.x).to(DEV),
        u=torch.from_numpy(bt.u).to(DEV),
    )
    if bt.sets is not None:
        d["sets"] = torch.from_numpy(bt.sets).to(DEV)
    return d


def compare_verify(bt: synth.VerifyBatch, out: dict, ref: dict, aprob=None, rmass=None) -> dict:
    """Compare GPU outputs with oracle results {b: VerifyResult}; raise on a non-boundary mismatch."""
    k_gpu = out["accepted_len"].cpu().numpy()
    t_gpu = out["bonus_token"].cpu().numpy()
    ap = None if aprob is None else aprob.cpu().numpy()
    rm = None if rmass is None else rmass.cpu().numpy()
    stats = dict(compared=0, boundary_k=0, boundary_bonus=0, k_diff_boundary=0, bonus_diff_boundary=0)
    K = bt.K
    for b, r in ref.items():
        stats["compared"] += 1
        last = min(r.k, K - 1)
        k_boundary = any(abs(float(bt.u[b, i]) - r.a[i]) < BOUNDARY for i in range(last + 1))
        stats["boundary_k"] += k_boundary
        if ap is not None:
            np.testing.assert_allclose(ap[b], r.a, atol=PROB_ATOL, rtol=0,
                                       err_msg=f"accept_prob of sequence {b}")
        if int(k_gpu[b]) != r.k:
            assert k_boundary, f"sequence {b}: k gpu={k_gpu[b]} oracle={r.k} a={r.a} u={bt.u[b]}"
            stats["k_diff_boundary"] += 1
            continue
        if rm is not None:
            assert abs(rm[b] - r.R) < PROB_ATOL, f"residual mass of sequence {b}: {rm[b]} vs {r.R}"
        ub = float(bt.u[b, K])
        b_boundary = abs(ub - r.c_lo) < BOUNDARY or abs(ub - r.c_hi) < BOUNDARY
        stats["boundary_bonus"] += b_boundary
        if int(t_gpu[b]) != r.bonus:
            assert b_boundary, (f"sequence {b}: bonus gpu={t_gpu[b]} oracle={r.bonus} k={r.k} "
                                f"u={ub} c=[{r.c_lo}, {r.c_hi}]")
            stats["bonus_diff_boundary"] += 1
    return stats


def oracle_topf_rows(z64: np.ndarray, F: int, exclude=None) -> np.ndarray:
    out = np.full((z64.shape[0], F), -1, dtype=np.int64)
    for r in range(z64.shape[0]):
        ex = -1 if exclude is None else int(exclude[r])
        out[r] = O.topf(z64[r], F, ex)
    return out


def report(name: str, stats: dict) -> None:
    print(f"[parity] {name}: {stats}", flush=True)
