"""GPU parity of ssd_saguaro_sample, the draft's sampling step with Saguaro, against the oracle.

The sampled token must equal the oracle's unless the row's uniform lies within BOUNDARY of the
cumulative q' on either side of the oracle's token (such rows are counted and printed); q' of the
GPU's token, the set, its mass and the normaliser must agree to PROB_ATOL.
"""
import numpy as np
import pytest
import torch

import draft_verification_ssd_amd as ssd
import oracle as O
import synth
from gpu_helpers import BOUNDARY, DEV, PROB_ATOL, logits_to_device

pytestmark = pytest.mark.gpu


def _rows(R, V, dtype, seed, ties=False):
    rng = np.random.default_rng(seed)
    if ties:
        z = rng.integers(-4, 5, size=(R, V)).astype(np.float32) * np.float32(0.5)
    else:
        z = rng.standard_normal(size=(R, V), dtype=np.float32) * np.float32(2.0)
    z[rng.random((R, V)) < 0.03] = -np.inf
    return synth.f32_to_bf16_bits(z) if dtype == "bf16" else z


def _uniforms(R, seed):
    u = np.random.default_rng(seed).random(R).astype(np.float32)
    if R > 2:
        u[0] = 0.0
        u[1] = np.nextafter(np.float32(1.0), np.float32(0.0))
    return u


def _check(z64, T, F, Fr, C_eff, u, out, rows):
    tok, prob, S, sig, N = (x.cpu().numpy() for x in out)
    near = 0
    for r in rows:
        res = O.saguaro_sample(z64[r], T, int(Fr[r]), float(C_eff[r]), float(u[r]))
        assert list(S[r]) == list(res.S) + [-1] * (F - len(res.S)), f"set of row {r}"
        assert abs(sig[r] - res.sigma) < PROB_ATOL and abs(N[r] - res.N) < PROB_ATOL, f"row {r}"
        if int(tok[r]) != res.x:
            assert min(abs(float(u[r]) - res.c_lo), abs(float(u[r]) - res.c_hi)) < BOUNDARY, \
                f"row {r}: gpu {tok[r]} oracle {res.x} u {u[r]} [{res.c_lo}, {res.c_hi})"
            near += 1
        qs, _, _ = O.saguaro(O.softmax_t(z64[r], T), [int(v) for v in res.S if v >= 0], float(C_eff[r]))
        assert 0 <= int(tok[r]) < len(qs) and qs[int(tok[r])] > 0.0, f"row {r}: token {tok[r]} has no mass"
        assert abs(prob[r] - qs[int(tok[r])]) < PROB_ATOL, f"row {r}"
    return near


@pytest.mark.parametrize("R,V,F,C,T,dtype", [(1, 1, 1, 0.5, 1.0, "f32"), (3, 5, 7, 0.3, 1.0, "bf16"),
                                             (17, 2049, 4, 0.3, 0.7, "bf16"), (4, 40000, 16, 0.5, 1.0, "f32"),
                                             (300, 9000, 8, 1.0, 1.0, "bf16"), (2, 128256, 3, 0.5, 1.0, "bf16"),
                                             (800, 20000, 0, 1.0, 1.0, "f32"), (3, 77777, 5, 0.0, 2.0, "f32"),
                                             (64, 128256, 3, 0.5, 1.0, "f32"), (3, 100000, 0, 1.0, 1.0, "bf16"),
                                             (2, 1 << 20, 4, 0.5, 1.0, "f32"), (2, 300000, 16, 0.4, 1.0, "f32")])
def test_sample_matches_oracle(R, V, F, C, T, dtype):
    """Rows cut into several chunks (few rows) and whole-row chunks (many rows), tie-heavy rows,
    F = 0 (plain sampling), C = 0 and C = 1, per-row F, u = 0 and u just below 1."""
    print(f"[case] sample R{R} V{V} F{F} C{C} T{T} {dtype}", flush=True)
    z = _rows(R, V, dtype, seed=R * 13 + V, ties=(R % 2 == 1))
    rng = np.random.default_rng(R + V)
    Fr = rng.integers(0, F + 1, size=R).astype(np.int32) if F > 0 else np.zeros(R, np.int32)
    u = _uniforms(R, R * 7 + V)
    ws = ssd.Workspace(ssd.ssd_saguaro_sample_workspace_bytes(R, V, F))
    out = ssd.ssd_saguaro_sample(logits_to_device(z, dtype), T, F, C, torch.from_numpy(u).to(DEV),
                                 F_per_row=torch.from_numpy(Fr).to(DEV) if F > 0 else None, workspace=ws)
    z64 = O.logits_f64(z, dtype)
    rows = [r for r in range(R) if np.isfinite(z64[r]).any()]
    if C == 0.0:  # rows whose set holds all the mass have no q' (covered by the degenerate test)
        rows = [r for r in rows
                if O.softmax_t(z64[r], T)[[v for v in O.topf(z64[r], int(Fr[r]))]].sum() < 1.0 - 1e-9]
    if len(rows) > 48:
        rows = sorted(np.random.default_rng(1).choice(rows, 48, replace=False).tolist())
    near = _check(z64, T, F, Fr, np.full(R, C), u, out, rows)
    print(f"  compared {len(rows)} rows, {near} within {BOUNDARY} of a boundary", flush=True)
    assert ssd.ssd_read_flags(ws) & ~ssd.FLAG_SAGUARO_NORM == 0


def test_sample_with_segments_of_several_batches():
    """Whole-row chunks longer than 16 batches of 8192 tokens: each segment spans two batches."""
    R, V, F = 800, 140000, 4
    print(f"[case] sample long rows R{R} V{V}", flush=True)
    z = _rows(R, V, "bf16", seed=5)
    u = _uniforms(R, 6)
    Cr = np.random.default_rng(7).uniform(0.0, 1.0, size=R).astype(np.float32)
    out = ssd.ssd_saguaro_sample(logits_to_device(z, "bf16"), 0.9, F, 1.0, torch.from_numpy(u).to(DEV),
                                 C_per_row=torch.from_numpy(Cr).to(DEV))
    z64 = O.logits_f64(z[:40], "bf16")
    near = _check(z64, 0.9, F, np.full(R, F), Cr.astype(np.float64), u, out, range(40))
    print(f"  {near} within {BOUNDARY} of a boundary", flush=True)


def test_sample_on_unaligned_strided_rows():
    """Rows 8 bytes apart from 16-byte alignment take the element-wise path."""
    R, V, F = 6, 10001, 3
    z = _rows(R, V + 1, "f32", seed=9)
    view = logits_to_device(z, "f32")[:, :V]
    u = _uniforms(R, 10)
    print("[case] sample unaligned rows", flush=True)
    out = ssd.ssd_saguaro_sample(view, 1.0, F, 0.4, torch.from_numpy(u).to(DEV))
    z64 = O.logits_f64(np.ascontiguousarray(z[:, :V]), "f32")
    _check(z64, 1.0, F, np.full(R, F), np.full(R, 0.4), u, out, range(R))


def test_sample_on_unaligned_rows_cut_into_chunks():
    """Few unaligned rows: several chunks a row, element-wise loads, the draw in the merge kernel."""
    R, V, F = 2, 50001, 5
    z = _rows(R, V + 1, "f32", seed=19)
    view = logits_to_device(z, "f32")[:, :V]
    u = np.array([0.37, 0.91], dtype=np.float32)
    print("[case] sample unaligned chunked rows", flush=True)
    out = ssd.ssd_saguaro_sample(view, 0.8, F, 0.2, torch.from_numpy(u).to(DEV))
    z64 = O.logits_f64(np.ascontiguousarray(z[:, :V]), "f32")
    _check(z64, 0.8, F, np.full(R, F), np.full(R, 0.2), u, out, range(R))


def test_sample_grid_frequencies_are_q_prime():
    """Identical rows with uniforms on a midpoint grid: token v is drawn about G q'(v) times."""
    G, V, F, C = 4096, 3000, 5, 0.25
    base = _rows(1, V, "f32", seed=12)[0] * np.float32(0.6)
    z = np.tile(base, (G, 1))
    u = ((np.arange(G) + 0.5) / G).astype(np.float32)
    print("[case] sample grid frequencies", flush=True)
    tok = ssd.ssd_saguaro_sample(logits_to_device(z, "f32"), 1.0, F, C, torch.from_numpy(u).to(DEV))[0]
    z64 = O.logits_f64(base, "f32")
    qs, _, _ = O.saguaro(O.softmax_t(z64, 1.0), list(O.topf(z64, F)), C)
    counts = np.bincount(tok.cpu().numpy(), minlength=V)
    assert np.abs(counts - G * qs).max() <= 2.0


def test_sample_degenerate_rows():
    """A fully masked row and a row whose set holds all the mass with C = 0 draw nothing (-1, q' 0);
    the second is flagged."""
    z = np.full((3, 5000), -np.inf, dtype=np.float32)
    z[1, [7, 4000]] = 1.0                       # the set (F = 2) holds all the mass
    z[2] = _rows(1, 5000, "f32", seed=13)[0]    # an ordinary row beside them
    u = np.array([0.5, 0.5, 0.5], dtype=np.float32)
    ws = ssd.Workspace(ssd.ssd_saguaro_sample_workspace_bytes(3, 5000, 2))
    print("[case] sample degenerate rows", flush=True)
    tok, prob, S, sig, N = ssd.ssd_saguaro_sample(logits_to_device(z, "f32"), 1.0, 2, 0.0,
                                                  torch.from_numpy(u).to(DEV), workspace=ws)
    tok, prob = tok.cpu().numpy(), prob.cpu().numpy()
    assert tok[0] == -1 and prob[0] == 0.0
    assert tok[1] == -1 and prob[1] == 0.0
    assert ssd.ssd_read_flags(ws) == ssd.FLAG_SAGUARO_NORM
    res = O.saguaro_sample(O.logits_f64(z[2], "f32"), 1.0, 2, 0.0, 0.5)
    assert tok[2] == res.x and abs(prob[2] - res.qx) < PROB_ATOL


def test_sample_agrees_with_saguaro_topf_and_repeats():
    """The set is ssd_saguaro_topf's and the mass and normaliser agree with it (the two sum the
    statistics in different orders); repeated calls give the same tokens."""
    R, V, F = 192, 128256, 3
    z = _rows(R, V, "bf16", seed=14)
    zd = logits_to_device(z, "bf16")
    ud = torch.from_numpy(_uniforms(R, 15)).to(DEV)
    print("[case] sample vs saguaro_topf", flush=True)
    S0, s0, n0 = ssd.ssd_saguaro_topf(zd, 1.0, F, 0.5)
    first = ssd.ssd_saguaro_sample(zd, 1.0, F, 0.5, ud)
    assert torch.equal(first[2], S0)
    assert (first[3] - s0).abs().max().item() < 1e-6 and (first[4] - n0).abs().max().item() < 1e-6
    for _ in range(5):
        again = ssd.ssd_saguaro_sample(zd, 1.0, F, 0.5, ud)
        assert torch.equal(again[0], first[0]) and torch.equal(again[1], first[1])
