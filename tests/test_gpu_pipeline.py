"""Full-size workloads on the GPU against the oracle (every outer sequence; branch rows sampled), with
every call's device-error flags read back:

  * SSD cache build: B=16 outer x 12 branches, K=4, V=128256 bf16, fan-out budget 12 (a=0.7, r=1),
    Saguaro C=0.5 — guesses, keys, Saguaro verification, the branch rows' draft step (top-F set,
    Saguaro mass and normaliser, sampled token), lookup and hit rate;
  * large batch: B=128, K=8, V=152064 fp32 Zipf-shaped rows, T=0.7, top-4 guesses (several launch
    rounds of the verification kernel);
  * full SSD round: B=64 x budget 32 = 2048 branches (8192 branch rows) plus the outer rows,
    V=128256 fp32, C=0.3 — the draft step on every branch row, verification, lookup, miss count.
"""
import numpy as np
import pytest
import torch

import draft_verification_ssd_amd as ssd
import oracle as O
import synth
from gpu_helpers import BOUNDARY, DEV, PROB_ATOL, compare_verify, logits_to_device, report

pytestmark = pytest.mark.gpu


def ssd_round_gpu(bt, fan, branch=None, branch_u=None):
    """One SSD round through the library: guesses of the outer draft rows (rows 0..K and the extra
    row K, all in the verification's pass), cache keys, Saguaro verification, lookup; and the branch rows'
    draft step in one pass each (ssd_saguaro_sample: set = the row's top F_j, its mass and
    normaliser, and the token drawn from q' with the row's uniform)."""
    B, K, V = bt.B, bt.K, bt.V
    draft = logits_to_device(bt.draft, bt.dtype)          # [B, K+1, V]
    target = logits_to_device(bt.target, bt.dtype)
    x = torch.from_numpy(bt.x).to(DEV)
    u = torch.from_numpy(bt.u).to(DEV)
    sets = torch.from_numpy(bt.sets).to(DEV)
    Gm = max(fan)
    guesses = torch.full((B, K + 1, Gm), -1, dtype=torch.int32, device=DEV)
    topf = torch.empty((B, K, Gm), dtype=torch.int32, device=DEV)
    # explicit workspaces, so that every call's device-error flags are read afterwards
    ws_v = ssd.Workspace(ssd.ssd_verify_workspace_bytes(B, K, V, Gm), DEV)
    # draft row K's guesses (nothing excluded) come from the same pass as the verification
    out = ssd.ssd_verify(draft, target, x, u, bt.T, sag_set=sets, sag_C=bt.C, topf_F=fan[:K],
                         topf_F_max=Gm, topf_out=topf,
                         accept_prob=torch.empty((B, K), device=DEV), residual_mass=torch.empty(B, device=DEV),
                         topf_last_F=fan[K], workspace=ws_v)
    guesses[:, :K] = topf
    last = out["topf_last"]
    if fan[K] > 0:
        guesses[:, K, : fan[K]] = last[:, : fan[K]]
    # keys straight from the two calls' outputs (no copy into one buffer)
    ck, ct, slot, miss = ssd.ssd_cache_keys_lookup(topf, fan, out["accepted_len"], out["bonus_token"],
                                                   guesses_last=last)
    # the two-launch form gives the same keys and slots
    ck2, ct2 = ssd.ssd_cache_keys(topf, fan, guesses_last=last)
    slot2, miss2 = ssd.ssd_cache_lookup(ck2, ct2, out["accepted_len"], out["bonus_token"])
    assert torch.equal(ck, ck2) and torch.equal(ct, ct2) and torch.equal(slot, slot2) and torch.equal(miss, miss2)
    res = dict(k=out["accepted_len"], bonus=out["bonus_token"], guesses=guesses, ck=ck, ct=ct,
               slot=slot, miss=miss, out=out)
    if branch is not None:
        nb = branch.shape[1]
        bd = logits_to_device(branch, bt.dtype).view(B * nb * K, V)
        Fr = torch.tensor(fan[:K], dtype=torch.int32, device=DEV).repeat(B * nb)
        ub = torch.from_numpy(np.ascontiguousarray(branch_u).reshape(-1)).to(DEV)
        ws_s = ssd.Workspace(ssd.ssd_saguaro_sample_workspace_bytes(B * nb * K, V, Gm), DEV)
        tok, prob, bsets, sig, N = ssd.ssd_saguaro_sample(bd, bt.T, Gm, bt.C, ub, F_per_row=Fr, workspace=ws_s)
        res.update(branch_sets=bsets.view(B, nb, K, Gm), branch_sigma=sig.view(B, nb, K),
                   branch_N=N.view(B, nb, K), branch_token=tok.view(B, nb, K), branch_prob=prob.view(B, nb, K))
        assert ssd.ssd_read_flags(ws_s) == 0, "ssd_saguaro_sample device flags"
    torch.cuda.synchronize()
    assert ssd.ssd_read_flags(ws_v) == 0, "ssd_verify device flags"
    return res


def check_round(bt, fan, res, seqs, branch=None, branch_seqs=(), name="", branch_u=None):
    ref = O.ssd_round(bt.draft, bt.target, bt.dtype, bt.x, bt.u, bt.T, bt.sets, bt.C, fan,
                      branch=None, seqs=seqs)
    st = compare_verify(bt, res["out"], {b: ref[b]["verify"] for b in seqs},
                        res["out"]["accept_prob"], res["out"]["residual_mass"])
    g = res["guesses"].cpu().numpy()
    ck, ct, slot = res["ck"].cpu().numpy(), res["ct"].cpu().numpy(), res["slot"].cpu().numpy()
    k_gpu, t_gpu = res["k"].cpu().numpy(), res["bonus"].cpu().numpy()
    for b in seqs:
        d = ref[b]
        for i in range(bt.K + 1):
            assert list(g[b, i, : fan[i]]) == list(d["guesses"][i]), f"guesses seq {b} pos {i}"
        assert list(ck[b]) == list(d["keys_k"]) and list(ct[b]) == list(d["keys_t"]), f"keys seq {b}"
        # lookup must agree with the oracle's lookup of the GPU's own outcome (bit-exact int work)
        assert slot[b] == O.cache_lookup(d["keys_k"], d["keys_t"], int(k_gpu[b]), int(t_gpu[b]))
    miss = int(res["miss"].item())
    assert miss == int((slot < 0).sum())
    if branch is not None:
        bs = res["branch_sets"].cpu().numpy()
        sig = res["branch_sigma"].cpu().numpy()
        nrm = res["branch_N"].cpu().numpy()
        tok = res["branch_token"].cpu().numpy()
        prob = res["branch_prob"].cpu().numpy()
        st["branch_rows"] = st["branch_token_near_boundary"] = 0
        for b, j in branch_seqs:
            for i in range(bt.K):
                zb = O.logits_f64(branch[b, j, i], bt.dtype)
                smp = O.saguaro_sample(zb, bt.T, fan[i], bt.C, float(branch_u[b, j, i]))
                assert list(bs[b, j, i, : fan[i]]) == list(smp.S), f"branch set {b},{j},{i}"
                assert abs(sig[b, j, i] - smp.sigma) < PROB_ATOL and abs(nrm[b, j, i] - smp.N) < PROB_ATOL
                st["branch_rows"] += 1
                if int(tok[b, j, i]) != smp.x:
                    uu = float(branch_u[b, j, i])
                    assert min(abs(uu - smp.c_lo), abs(uu - smp.c_hi)) < BOUNDARY, f"branch token {b},{j},{i}"
                    st["branch_token_near_boundary"] += 1
                qs, _, _ = O.saguaro(O.softmax_t(zb, bt.T), [int(v) for v in smp.S if v >= 0], bt.C)
                assert abs(prob[b, j, i] - qs[int(tok[b, j, i])]) < PROB_ATOL, f"branch q' {b},{j},{i}"
    st["hits"] = int((slot >= 0).sum())
    st["miss_count"] = miss
    report(name, st)
    return st


@pytest.mark.parametrize("seed", [0, 1])
def test_ssd_cache_build_b16x12_k4_v128256_bf16(seed):
    w = synth.workload("ssd_build_b16x12_k4_v128256_bf16")
    fan, _ = ssd.ssd_fanout_alloc(w["K"], w["a"], w["r"], w["budget"])
    fo, _ = O.fanout(w["K"], w["a"], w["r"], w["budget"])
    assert fan == [int(v) for v in fo] == [3, 2, 2, 2, 3]
    bt = synth.make_verify_batch(w["B"], w["K"], w["V"], w["dtype"], seed, T=w["T"], sag_sizes=fan[: w["K"]],
                                 C=w["C"])
    branch = synth.make_branch_rows(w["B"], w["budget"], w["K"], w["V"], w["dtype"], seed)
    bu = synth.make_branch_uniforms(w["B"], w["budget"], w["K"], seed)
    print(f"[case] ssd cache build seed {seed}", flush=True)
    res = ssd_round_gpu(bt, fan, branch, bu)
    check_round(bt, fan, res, range(w["B"]), branch, [(b, j) for b in (0, 7, 15) for j in (0, 5, 11)],
                branch_u=bu,
                name=f"ssd_build seed{seed}")


@pytest.mark.parametrize("seed", [0])
def test_large_batch_b128_k8_v152064_f32_zipf_top4(seed):
    w = synth.workload("b128_k8_v152064_f32_zipf_top4")
    bt = synth.make_verify_batch(w["B"], w["K"], w["V"], w["dtype"], seed, T=w["T"], zipf_s=w["zipf_s"],
                                 noise_sigma=w["noise_sigma"])
    print("[case] b128_k8_v152064 verify", flush=True)
    draft = logits_to_device(bt.draft[:, : bt.K], bt.dtype)
    target = logits_to_device(bt.target, bt.dtype)
    B, K = bt.B, bt.K
    aprob = torch.empty((B, K), device=DEV)
    rmass = torch.empty(B, device=DEV)
    ws = ssd.Workspace(ssd.ssd_verify_workspace_bytes(B, K, bt.V, w["topf"]), DEV)
    out = ssd.ssd_verify(draft, target, torch.from_numpy(bt.x).to(DEV), torch.from_numpy(bt.u).to(DEV), bt.T,
                         topf_F_max=w["topf"], accept_prob=aprob, residual_mass=rmass, workspace=ws)
    torch.cuda.synchronize()
    assert ssd.ssd_read_flags(ws) == 0, "ssd_verify device flags"
    seqs = list(range(B))  # every sequence of the batch
    ref = O.verify_batch(bt.draft, bt.target, bt.dtype, bt.x, bt.u, bt.T, seqs=seqs)
    st = compare_verify(bt, out, ref, aprob, rmass)
    g = out["topf"].cpu().numpy()
    for b in seqs:
        for i in range(K):
            want = O.topf(O.logits_f64(bt.draft[b, i], bt.dtype), w["topf"], int(bt.x[b, i]))
            assert list(g[b, i]) == list(want), f"top-F seq {b} pos {i}"
    assert st["compared"] == B
    report("b128_k8_v152064_f32_zipf", st)


def test_full_ssd_round_b64x32_k4_v128256_f32():
    w = synth.workload("ssd_round_b64x32_k4_v128256_f32")
    fan, _ = ssd.ssd_fanout_alloc(w["K"], w["a"], w["r"], w["budget"])
    assert fan == [int(v) for v in O.fanout(w["K"], w["a"], w["r"], w["budget"])[0]] == [8, 7, 5, 5, 7]
    bt = synth.make_verify_batch(w["B"], w["K"], w["V"], w["dtype"], 0, T=w["T"], sag_sizes=fan[: w["K"]],
                                 C=w["C"])
    branch = synth.make_branch_rows(w["B"], w["budget"], w["K"], w["V"], w["dtype"], 0)
    bu = synth.make_branch_uniforms(w["B"], w["budget"], w["K"], 0)
    print("[case] full ssd round b64x32", flush=True)
    res = ssd_round_gpu(bt, fan, branch, bu)
    seqs = list(range(w["B"]))  # every outer sequence; branch rows sampled across the batch
    branch_seqs = [(0, 0), (13, 31), (40, 17), (63, 5), (7, 9), (22, 0), (51, 30), (33, 12)]
    st = check_round(bt, fan, res, seqs, branch, branch_seqs, branch_u=bu, name="ssd_round b64x32")
    assert st["compared"] == w["B"]
    # host-side choice of the path from the miss count ([SSD] Saguaro 优化三): zero-wait only if
    # every sequence hit
    miss = st["miss_count"]
    path = "zero-wait" if miss == 0 else "fallback"
    print(f"[ssd round] misses {miss}/{w['B']} -> {path} path", flush=True)


@pytest.mark.parametrize("T", [0.5, 2.0])
def test_fanout_ablation_lookups_match_oracle(T):
    """The fan-out ablation's pieces: both fan-outs' caches built from one set of top-8 guesses and
    the batch's outcomes looked up, slot for slot against the oracle's guesses and lookup."""
    import bench
    B, K, V, budget = 24, 4, 32000, 12
    bt = synth.make_verify_batch(B, K, V, synth.BF16, 5, T=T)
    draft = logits_to_device(bt.draft, bt.dtype)
    target = logits_to_device(bt.target, bt.dtype)
    ap = torch.empty((B, K), device=DEV)
    print(f"[case] fan-out ablation T{T}", flush=True)
    ws = ssd.Workspace(ssd.ssd_verify_workspace_bytes(B, K, V, 8), DEV)
    out = ssd.ssd_verify(draft[:, :K], target, torch.from_numpy(bt.x).to(DEV), torch.from_numpy(bt.u).to(DEV), T,
                         topf_F_max=8, accept_prob=ap, residual_mass=torch.empty(B, device=DEV), workspace=ws)
    torch.cuda.synchronize()
    assert ssd.ssd_read_flags(ws) == 0, "ssd_verify device flags"
    guesses = torch.cat([out["topf"], ssd.ssd_topf_guess(draft[:, K, :], 8)[:, None, :]], dim=1).contiguous()
    ref = O.verify_batch(bt.draft, bt.target, bt.dtype, bt.x, bt.u, T)
    compare_verify(bt, out, ref, ap, out["residual_mass"])
    a_hat = float(ap.mean().item())
    k_gpu, t_gpu = out["accepted_len"].cpu().numpy(), out["bonus_token"].cpu().numpy()
    for fan in (ssd.ssd_fanout_alloc(K, a_hat, 1.0, budget)[0], bench.uniform_fanout(K, budget)):
        ck, ct = ssd.ssd_cache_keys(guesses, fan)
        slot, miss = ssd.ssd_cache_lookup(ck, ct, out["accepted_len"], out["bonus_token"])
        slot = slot.cpu().numpy()
        for b in range(B):
            z = O.logits_f64(bt.draft[b], bt.dtype)
            g = [O.topf(z[i], fan[i], int(bt.x[b, i])) for i in range(K)] + [O.topf(z[K], fan[K])]
            kk, tt = O.cache_keys(g, fan)
            assert slot[b] == O.cache_lookup(kk, tt, int(k_gpu[b]), int(t_gpu[b])), f"T {T} fan {fan} seq {b}"
        assert int(miss.item()) == int((slot < 0).sum())
