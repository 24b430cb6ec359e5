"""GPU parity of the standalone top-F guesses, Saguaro adjust and speculation-cache calls."""
import numpy as np
import pytest
import torch

import draft_verification_ssd_amd as ssd
import oracle as O
import synth
from gpu_helpers import DEV, PROB_ATOL, logits_to_device, oracle_topf_rows

pytestmark = pytest.mark.gpu


def tie_heavy_rows(R, V, dtype, seed):
    rng = np.random.default_rng(seed)
    z = rng.integers(-4, 5, size=(R, V)).astype(np.float32) * np.float32(0.5)
    z[rng.random((R, V)) < 0.05] = -np.inf
    return synth.f32_to_bf16_bits(z) if dtype == "bf16" else z


@pytest.mark.parametrize("R,V,F,dtype", [(1, 1, 1, "f32"), (3, 5, 7, "bf16"), (5, 300, 3, "f32"),
                                         (17, 2049, 4, "bf16"), (4, 40000, 16, "f32"),
                                         (300, 9000, 8, "bf16"), (2, 128256, 3, "bf16"),
                                         (3, 77777, 5, "f32"), (2, 300000, 16, "f32")])
def test_topf_matches_oracle_with_ties_masks_and_exclusion(R, V, F, dtype):
    print(f"[case] topf R{R} V{V} F{F} {dtype}", flush=True)
    z = tie_heavy_rows(R, V, dtype, seed=R * 7 + V)
    rng = np.random.default_rng(V)
    ex = rng.integers(-1, V, size=R).astype(np.int32)
    Fr = rng.integers(0, F + 1, size=R).astype(np.int32)
    zd = logits_to_device(z, dtype)
    got = ssd.ssd_topf_guess(zd, F, exclude=torch.from_numpy(ex).to(DEV),
                             F_per_row=torch.from_numpy(Fr).to(DEV)).cpu().numpy()
    z64 = O.logits_f64(z, dtype)
    for r in range(R):
        want = list(O.topf(z64[r], int(Fr[r]), int(ex[r]))) + [-1] * (F - int(Fr[r]))
        assert list(got[r]) == want, f"row {r}"


def test_topf_on_a_strided_row_view():
    bt = synth.make_verify_batch(6, 4, 20000, synth.BF16, 2)
    d = logits_to_device(bt.draft, bt.dtype)                 # [B, K+1, V]
    view = d[:, bt.K, :]                                      # row K of every sequence
    print("[case] topf strided view", flush=True)
    got = ssd.ssd_topf_guess(view, 4).cpu().numpy()
    want = oracle_topf_rows(O.logits_f64(bt.draft[:, bt.K], bt.dtype), 4)
    assert np.array_equal(got, want)


def test_topf_bad_f_is_clamped_and_flagged():
    z = tie_heavy_rows(3, 500, "f32", 1)
    Fr = np.array([2, 9, -1], dtype=np.int32)
    ws = ssd.Workspace(ssd.ssd_topf_workspace_bytes(3, 500, 4))
    print("[case] topf bad F", flush=True)
    got = ssd.ssd_topf_guess(logits_to_device(z, "f32"), 4, F_per_row=torch.from_numpy(Fr).to(DEV),
                             workspace=ws).cpu().numpy()
    assert ssd.ssd_read_flags(ws) & ssd.FLAG_BAD_F
    z64 = O.logits_f64(z, "f32")
    assert list(got[0]) == list(O.topf(z64[0], 2)) + [-1, -1]
    assert list(got[1]) == list(O.topf(z64[1], 4))
    assert list(got[2]) == [-1] * 4


@pytest.mark.parametrize("R,V,F,C,T,dtype", [(4, 1000, 3, 0.5, 1.0, "f32"), (7, 4099, 8, 0.0, 0.7, "bf16"),
                                             (3, 32000, 4, 1.0, 1.0, "f32"), (9, 128256, 5, 0.3, 1.0, "bf16"),
                                             (2, 777, 0, 0.5, 1.0, "f32"), (5, 2048, 16, 0.9, 2.0, "bf16")])
def test_saguaro_matches_oracle(R, V, F, C, T, dtype):
    print(f"[case] saguaro R{R} V{V} F{F} C{C} {dtype}", flush=True)
    rng = np.random.default_rng(R + V)
    z = (rng.normal(0, 2, size=(R, V))).astype(np.float32)
    if dtype == "bf16":
        z = synth.f32_to_bf16_bits(z)
    z64 = O.logits_f64(z, dtype)
    sets = np.full((R, max(F, 1)), -1, dtype=np.int32)
    for r in range(R):
        s = O.topf(z64[r], F) if F else []
        sets[r, : len(s)] = s
        if F >= 3 and r % 2 == 0:
            sets[r, 2] = sets[r, 0]          # repeated entry: ignored
        if F >= 2 and r % 3 == 0:
            sets[r, 1] = V + 3               # out of range: ignored
    zd = logits_to_device(z, dtype)
    sd = torch.from_numpy(sets[:, :F].copy()).to(DEV) if F else None
    qp, sig, N = ssd.ssd_saguaro_adjust(zd, T, sd, C, materialise=True)
    qp, sig, N = qp.cpu().numpy(), sig.cpu().numpy(), N.cpu().numpy()
    for r in range(R):
        q = O.softmax_t(z64[r], T)
        want, s_ref, n_ref = O.saguaro(q, sets[r, :F] if F else None, C)
        assert abs(sig[r] - s_ref) < PROB_ATOL and abs(N[r] - n_ref) < PROB_ATOL
        np.testing.assert_allclose(qp[r], want, atol=PROB_ATOL, rtol=0)


def test_saguaro_compact_outputs_only():
    z = np.random.default_rng(3).normal(0, 2, size=(5, 3001)).astype(np.float32)
    sets = np.array([O.topf(z[r].astype(np.float64), 2) for r in range(5)], dtype=np.int32)
    print("[case] saguaro compact", flush=True)
    qp, sig, N = ssd.ssd_saguaro_adjust(logits_to_device(z, "f32"), 1.0, torch.from_numpy(sets).to(DEV), 0.5)
    assert qp is None
    for r in range(5):
        _, s_ref, n_ref = O.saguaro(O.softmax_t(z[r].astype(np.float64), 1.0), sets[r], 0.5)
        assert abs(sig[r].item() - s_ref) < PROB_ATOL and abs(N[r].item() - n_ref) < PROB_ATOL


def test_saguaro_degenerate_normaliser_is_flagged():
    z = np.full((1, 4), -np.inf, dtype=np.float32)
    z[0, :2] = 0.0
    sets = np.array([[0, 1]], dtype=np.int32)
    ws = ssd.Workspace(ssd.ssd_saguaro_workspace_bytes(1, 4))
    print("[case] saguaro N<=0", flush=True)
    ssd.ssd_saguaro_adjust(logits_to_device(z, "f32"), 1.0, torch.from_numpy(sets).to(DEV), 0.0, workspace=ws)
    assert ssd.ssd_read_flags(ws) & ssd.FLAG_SAGUARO_NORM


@pytest.mark.parametrize("R,V,F,C,T,dtype", [(1, 1, 1, 0.5, 1.0, "f32"), (3, 5, 7, 0.0, 1.0, "bf16"),
                                             (17, 2049, 4, 0.3, 0.7, "bf16"), (4, 40000, 16, 0.5, 1.0, "f32"),
                                             (300, 9000, 8, 1.0, 1.0, "bf16"), (2, 128256, 3, 0.5, 1.0, "bf16"),
                                             (800, 20000, 3, 0.5, 1.0, "f32"), (3, 77777, 5, 0.3, 2.0, "f32"),
                                             (2, 300000, 16, 0.5, 1.0, "bf16")])
def test_saguaro_topf_matches_topf_then_saguaro(R, V, F, C, T, dtype):
    """One pass (set = the row's top F, then sigma and N) against the oracle's top-F and Saguaro;
    the shapes cover rows cut into several chunks (few rows) and whole-row chunks (many rows)."""
    print(f"[case] saguaro_topf R{R} V{V} F{F} C{C} T{T} {dtype}", flush=True)
    rng = np.random.default_rng(R * 31 + V)
    if R % 2:
        z = tie_heavy_rows(R, V, dtype, seed=R + V)
    else:
        z = rng.normal(0, 2, size=(R, V)).astype(np.float32)
        z[rng.random((R, V)) < 0.02] = -np.inf
        if dtype == "bf16":
            z = synth.f32_to_bf16_bits(z)
    Fr = rng.integers(0, F + 1, size=R).astype(np.int32)
    ws = ssd.Workspace(ssd.ssd_saguaro_topf_workspace_bytes(R, V, F))
    S, sig, N = ssd.ssd_saguaro_topf(logits_to_device(z, dtype), T, F, C, F_per_row=torch.from_numpy(Fr).to(DEV),
                                     workspace=ws)
    S, sig, N = S.cpu().numpy(), sig.cpu().numpy(), N.cpu().numpy()
    z64 = O.logits_f64(z, dtype)
    for r in range(R):
        want = O.topf(z64[r], int(Fr[r]))
        assert list(S[r]) == list(want) + [-1] * (F - len(want)), f"set of row {r}"
        if not np.isfinite(z64[r]).any():
            continue
        q = O.softmax_t(z64[r], T)
        if C == 0.0 and abs(q[list(want)].sum() - 1.0) < 1e-12:  # the set holds all the mass: N = 0
            assert abs(N[r]) < PROB_ATOL, f"row {r}"
            assert ssd.ssd_read_flags(ws, clear=False) & ssd.FLAG_SAGUARO_NORM
            continue
        _, s_ref, n_ref = O.saguaro(q, want, C)
        assert abs(sig[r] - s_ref) < PROB_ATOL and abs(N[r] - n_ref) < PROB_ATOL, f"row {r}"
    flags = ssd.ssd_read_flags(ws)
    assert flags & ~ssd.FLAG_SAGUARO_NORM == 0


def test_saguaro_topf_on_a_strided_row_view_and_degenerate_norm():
    bt = synth.make_verify_batch(6, 4, 20000, synth.BF16, 3)
    view = logits_to_device(bt.draft, bt.dtype)[:, bt.K, :]   # row K of every sequence
    print("[case] saguaro_topf strided view", flush=True)
    S, sig, N = ssd.ssd_saguaro_topf(view, 1.0, 4, 0.5)
    z64 = O.logits_f64(bt.draft[:, bt.K], bt.dtype)
    for r in range(6):
        want = O.topf(z64[r], 4)
        assert list(S[r].cpu().numpy()) == list(want)
        _, s_ref, n_ref = O.saguaro(O.softmax_t(z64[r], 1.0), want, 0.5)
        assert abs(sig[r].item() - s_ref) < PROB_ATOL and abs(N[r].item() - n_ref) < PROB_ATOL
    z = np.full((1, 4), -np.inf, dtype=np.float32)
    z[0, :2] = 0.0                                            # the set holds all the mass; C = 0
    ws = ssd.Workspace(ssd.ssd_saguaro_topf_workspace_bytes(1, 4, 2))
    ssd.ssd_saguaro_topf(logits_to_device(z, "f32"), 1.0, 2, 0.0, workspace=ws)
    assert ssd.ssd_read_flags(ws) & ssd.FLAG_SAGUARO_NORM


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_saguaro_statistics_with_a_long_masked_prefix(dtype):
    """Rows whose first tens of thousands of tokens are -inf: every lane's first batches hold no
    finite token, which the running statistics must skip (regression: they turned the lane's sum
    into NaN and lost its tokens)."""
    R, V = 4, 60000
    rng = np.random.default_rng(11)
    z = rng.normal(0, 2, size=(R, V)).astype(np.float32)
    for r in range(R):
        z[r, : 20000 + 9000 * r] = -np.inf
    zz = synth.f32_to_bf16_bits(z) if dtype == "bf16" else z
    z64 = O.logits_f64(zz, dtype)
    zd = logits_to_device(zz, dtype)
    print(f"[case] masked prefix {dtype}", flush=True)
    sets = np.stack([O.topf(z64[r], 3) for r in range(R)]).astype(np.int32)
    _, sig_a, N_a = ssd.ssd_saguaro_adjust(zd, 1.0, torch.from_numpy(sets).to(DEV), 0.5)
    S, sig_b, N_b = ssd.ssd_saguaro_topf(zd, 1.0, 3, 0.5)
    assert np.array_equal(S.cpu().numpy(), sets)
    for r in range(R):
        _, s_ref, n_ref = O.saguaro(O.softmax_t(z64[r], 1.0), sets[r], 0.5)
        for sig, N in ((sig_a, N_a), (sig_b, N_b)):
            assert abs(sig[r].item() - s_ref) < PROB_ATOL and abs(N[r].item() - n_ref) < PROB_ATOL, f"row {r}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_per_row_saguaro_c_in_both_saguaro_calls(dtype):
    """A Saguaro factor per row (the branch rows of different draft positions): both entry points
    against the oracle; an out-of-range factor is clamped (NaN taken as 1) and flagged."""
    R, V, F = 40, 5000, 3
    rng = np.random.default_rng(21)
    z = rng.normal(0, 2, size=(R, V)).astype(np.float32)
    zz = synth.f32_to_bf16_bits(z) if dtype == "bf16" else z
    z64 = O.logits_f64(zz, dtype)
    Cr = rng.uniform(0.0, 1.0, size=R).astype(np.float32)
    Cr[0], Cr[1], Cr[5], Cr[9] = 0.0, 1.0, 1.5, np.nan
    C_eff = np.where(np.isnan(Cr), 1.0, np.clip(Cr, 0.0, 1.0))
    sets = np.stack([O.topf(z64[r], F) for r in range(R)]).astype(np.int32)
    zd = logits_to_device(zz, dtype)
    Cd = torch.from_numpy(Cr).to(DEV)
    print(f"[case] per-row C {dtype}", flush=True)
    ws_a = ssd.Workspace(ssd.ssd_saguaro_workspace_bytes(R, V))
    qp, sig_a, N_a = ssd.ssd_saguaro_adjust(zd, 1.0, torch.from_numpy(sets).to(DEV), 0.5, C_per_row=Cd,
                                            materialise=True, workspace=ws_a)
    ws_b = ssd.Workspace(ssd.ssd_saguaro_topf_workspace_bytes(R, V, F))
    S, sig_b, N_b = ssd.ssd_saguaro_topf(zd, 1.0, F, 0.5, C_per_row=Cd, workspace=ws_b)
    assert ssd.ssd_read_flags(ws_a) == ssd.FLAG_BAD_C
    assert ssd.ssd_read_flags(ws_b) == ssd.FLAG_BAD_C
    assert np.array_equal(S.cpu().numpy(), sets)
    qp = qp.cpu().numpy()
    for r in range(R):
        want, s_ref, n_ref = O.saguaro(O.softmax_t(z64[r], 1.0), sets[r], float(C_eff[r]))
        for sig, N in ((sig_a, N_a), (sig_b, N_b)):
            assert abs(sig[r].item() - s_ref) < PROB_ATOL and abs(N[r].item() - n_ref) < PROB_ATOL, f"row {r}"
        np.testing.assert_allclose(qp[r], want, atol=PROB_ATOL, rtol=0)


@pytest.mark.parametrize("B,K,G,fan", [(3, 4, 3, [3, 2, 2, 2, 3]), (5, 4, 8, [8, 7, 5, 5, 7]),
                                       (2, 2, 2, [0, 2, 1]), (1, 1, 1, [1, 0])])
def test_cache_keys_and_lookup_match_oracle(B, K, G, fan):
    print(f"[case] cache B{B} K{K} fan{fan}", flush=True)
    rng = np.random.default_rng(B * 10 + K)
    guesses = np.full((B, K + 1, G), -1, dtype=np.int32)
    for b in range(B):
        for k in range(K + 1):
            n = rng.integers(0, G + 1)
            guesses[b, k, :n] = rng.permutation(50)[:n]
    gd = torch.from_numpy(guesses).to(DEV)
    ck, ct = ssd.ssd_cache_keys(gd, fan)
    # the same keys from position K's guesses held apart (a narrower array, as ssd_topf_guess gives)
    ck2, ct2 = ssd.ssd_cache_keys(gd[:, :K].contiguous(), fan, guesses_last=gd[:, K, : max(1, fan[K])].contiguous())
    assert torch.equal(ck, ck2) and torch.equal(ct, ct2)
    ck, ct = ck.cpu().numpy(), ct.cpu().numpy()
    kk_all, tt_all = [], []
    for b in range(B):
        kk, tt = O.cache_keys([list(guesses[b, k]) for k in range(K + 1)], fan)
        assert list(ck[b]) == list(kk) and list(ct[b]) == list(tt)
        kk_all.append(kk)
        tt_all.append(tt)
    # outcomes: half of them drawn from the cache, half at random
    acc = np.empty(B, dtype=np.int32)
    bon = np.empty(B, dtype=np.int32)
    for b in range(B):
        valid = np.nonzero(ck[b] >= 0)[0]
        if b % 2 == 0 and len(valid):
            j = rng.choice(valid)
            acc[b], bon[b] = ck[b, j], ct[b, j]
        else:
            acc[b], bon[b] = rng.integers(0, K + 1), rng.integers(0, 50)
    slot, miss = ssd.ssd_cache_lookup(torch.from_numpy(ck).to(DEV), torch.from_numpy(ct).to(DEV),
                                      torch.from_numpy(acc).to(DEV), torch.from_numpy(bon).to(DEV))
    slot = slot.cpu().numpy()
    want = [O.cache_lookup(kk_all[b], tt_all[b], int(acc[b]), int(bon[b])) for b in range(B)]
    assert list(slot) == want
    assert int(miss.item()) == sum(s < 0 for s in want)
    # keys and lookup in one launch: the same keys, slots and miss count, with position K's guesses
    # in the array or held apart
    for args in ((gd, fan), (gd[:, :K].contiguous(), fan)):
        kw = {} if args[0] is gd else dict(guesses_last=gd[:, K, : max(1, fan[K])].contiguous())
        fk, ft, fs, fm = ssd.ssd_cache_keys_lookup(args[0], args[1], torch.from_numpy(acc).to(DEV),
                                                  torch.from_numpy(bon).to(DEV), **kw)
        assert np.array_equal(fk.cpu().numpy(), ck) and np.array_equal(ft.cpu().numpy(), ct)
        assert list(fs.cpu().numpy()) == want and int(fm.item()) == sum(s < 0 for s in want)


def test_lookup_with_empty_cache_counts_every_miss():
    B = 1000
    z = torch.zeros(B, dtype=torch.int32, device=DEV)
    ck = torch.empty((B, 0), dtype=torch.int32, device=DEV)
    print("[case] lookup empty cache", flush=True)
    slot, miss = ssd.ssd_cache_lookup(ck, ck, z, z)
    assert int(miss.item()) == B and bool((slot == -1).all())
