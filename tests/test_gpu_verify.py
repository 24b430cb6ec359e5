"""GPU parity of ssd_verify against the float64 oracle (accept decisions, bonus token, accept
probabilities, residual mass, fused top-F guesses), plus edge cases and determinism."""
import numpy as np
import pytest
import torch

import draft_verification_ssd_amd as ssd
import oracle as O
import synth
from gpu_helpers import DEV, batch_to_device, compare_verify, oracle_topf_rows, report

pytestmark = pytest.mark.gpu


def run_verify(bt, topf_F_max=0, topf_F=None, extra_draft_row=False):
    d = batch_to_device(bt, verify_rows_only=not extra_draft_row)
    B, K = bt.B, bt.K
    aprob = torch.empty((B, K), dtype=torch.float32, device=DEV)
    rmass = torch.empty(B, dtype=torch.float32, device=DEV)
    call = ssd.VerifyCall(d["draft"], d["target"], d["x"], d["u"], bt.T, sag_set=d.get("sets"),
                          sag_C=bt.C, topf_F=topf_F, topf_F_max=topf_F_max, accept_prob=aprob,
                          residual_mass=rmass)
    out = call()
    torch.cuda.synchronize()
    flags = ssd.ssd_read_flags(call.workspace)
    return out, aprob, rmass, flags


def check_batch(bt, name, topf_F_max=0, topf_F=None, extra_draft_row=False):
    print(f"[case] {name}", flush=True)
    out, aprob, rmass, flags = run_verify(bt, topf_F_max, topf_F, extra_draft_row)
    assert flags == 0, f"device flags {flags:#x}"
    ref = O.verify_batch(bt.draft, bt.target, bt.dtype, bt.x, bt.u, bt.T, bt.sets, bt.C)
    st = compare_verify(bt, out, ref, aprob, rmass)
    report(name, st)
    if topf_F_max:
        got = out["topf"].cpu().numpy()
        for b in range(bt.B):
            for i in range(bt.K):
                F = topf_F_max if topf_F is None else topf_F[i]
                z = O.logits_f64(bt.draft[b, i], bt.dtype)
                want = list(O.topf(z, F, int(bt.x[b, i]))) + [-1] * (topf_F_max - F)
                assert list(got[b, i]) == want, f"top-F of sequence {b} position {i}"
    return st


# --- shapes spanning several chunks, ragged tails, tiny vocabularies --------------------------
SMALL = [
    # B, K, V, dtype, T, topf
    (1, 1, 1, "f32", 1.0, 0),
    (2, 3, 2, "bf16", 1.0, 1),
    (3, 4, 7, "f32", 0.7, 3),
    (4, 2, 8, "bf16", 1.0, 2),
    (5, 4, 9, "bf16", 1.3, 3),
    (3, 8, 100, "f32", 1.0, 4),
    (7, 4, 1000, "bf16", 0.8, 3),
    (2, 4, 2047, "f32", 1.0, 3),
    (2, 4, 2048, "bf16", 1.0, 3),
    (2, 4, 2049, "bf16", 1.0, 5),
    (6, 5, 4099, "f32", 2.0, 8),
    (3, 16, 16385, "bf16", 1.0, 16),
    (17, 4, 50021, "f32", 1.0, 3),
    (4, 8, 65536, "bf16", 0.7, 4),
]


@pytest.mark.parametrize("B,K,V,dtype,T,topf", SMALL)
@pytest.mark.parametrize("seed", [0, 1])
def test_verify_matches_oracle(B, K, V, dtype, T, topf, seed):
    bt = synth.make_verify_batch(B, K, V, dtype, seed, T=T)
    check_batch(bt, f"B{B} K{K} V{V} {dtype} T{T} F{topf} seed{seed}", topf_F_max=topf)


@pytest.mark.parametrize("C", [0.0, 0.3, 1.0])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_verify_with_saguaro_sets(C, dtype):
    sizes = [3, 2, 2, 1]
    bt = synth.make_verify_batch(9, 4, 30011, dtype, 5, sag_sizes=sizes, C=C)
    # set hygiene: repeat an entry and add out-of-range ones, both ignored by definition
    bt.sets[0, 0, 1] = bt.sets[0, 0, 0]
    bt.sets[1, 1, 1] = 30011 + 7
    check_batch(bt, f"saguaro C{C} {dtype}", topf_F_max=3, topf_F=[3, 2, 2, 2])


def test_config_b1_k4_v32000_f32():
    st = dict(compared=0, boundary_k=0, boundary_bonus=0)
    for seed in range(32):
        bt = synth.make_verify_batch(1, 4, 32000, synth.F32, seed)
        s = check_batch(bt, f"b1_k4_v32000_f32 seed{seed}")
        for k in st:
            st[k] += s[k]
    report("b1_k4_v32000_f32 x32 seeds", st)


@pytest.mark.parametrize("seed", range(32))
def test_config_b16_k4_v128256_bf16_top3(seed):
    bt = synth.make_verify_batch(16, 4, 128256, synth.BF16, seed)
    check_batch(bt, f"b16_k4_v128256_bf16_top3 seed{seed}", topf_F_max=3)


def test_strided_draft_rows_and_misaligned_vocab():
    # draft tensor keeps its K+1-th row (seq stride (K+1) V); odd V makes bf16 rows misaligned
    bt = synth.make_verify_batch(5, 4, 12345, synth.BF16, 9)
    check_batch(bt, "strided draft, V=12345 bf16", topf_F_max=2, extra_draft_row=True)
    bt = synth.make_verify_batch(4, 3, 5003, synth.F32, 10)
    check_batch(bt, "strided draft, V=5003 f32", topf_F_max=3, extra_draft_row=True)


def test_identical_draft_and_target_accepts_everything():
    bt = synth.make_verify_batch(8, 6, 7777, synth.BF16, 3)
    bt.target[:, : bt.K] = bt.draft[:, : bt.K]
    bt.u[:, : bt.K] = np.float32(1 - 2 ** -24)
    out, _, rmass, flags = run_verify(bt)
    assert flags == 0
    assert np.all(out["accepted_len"].cpu().numpy() == bt.K)
    assert np.all(rmass.cpu().numpy() == 1.0)
    ref = O.verify_batch(bt.draft, bt.target, bt.dtype, bt.x, bt.u, bt.T)
    compare_verify(bt, out, ref)


def test_masked_logits_and_extreme_uniforms():
    bt = synth.make_verify_batch(6, 4, 3000, synth.F32, 12)
    bt.draft[:, :, 100:2000] = -np.inf          # masked vocabulary in both models
    bt.target[:, :, 100:2000] = -np.inf
    for b in range(bt.B):
        for i in range(bt.K):
            bt.x[b, i] = (b * 7 + i) % 100       # drafts from the unmasked part
    bt.u[0, :] = 0.0
    bt.u[1, :] = np.float32(1 - 2 ** -24)
    check_batch(bt, "masked logits / u extremes", topf_F_max=4)


def test_bad_draft_token_is_flagged_not_dereferenced():
    bt = synth.make_verify_batch(3, 4, 1000, synth.F32, 4)
    bt.x[1, 2] = 1000 + 5
    bt.x[2, 0] = -3
    print("[case] bad draft token", flush=True)
    out, aprob, _, flags = run_verify(bt, topf_F_max=2)
    assert flags & ssd.FLAG_BAD_TOKEN
    k = out["accepted_len"].cpu().numpy()
    assert k[1] <= 2 and k[2] == 0
    assert aprob.cpu().numpy()[1, 2] == 0.0


def test_determinism_over_repeated_calls():
    bt = synth.make_verify_batch(16, 4, 128256, synth.BF16, 21)
    d = batch_to_device(bt)
    call = ssd.VerifyCall(d["draft"], d["target"], d["x"], d["u"], 1.0, topf_F_max=3,
                          accept_prob=torch.empty((16, 4), device=DEV),
                          residual_mass=torch.empty(16, device=DEV))
    print("[case] determinism x50", flush=True)
    first = {k: v.clone() for k, v in call().items() if v is not None}
    for _ in range(49):
        out = call()
        for k, v in first.items():
            assert torch.equal(out[k], v), k


def test_output_marginal_is_the_target_distribution():
    """Lossless property on the GPU: enumerate every draft token with weight q(x) and a midpoint
    grid of both uniforms; the emitted first token's distribution must be p."""
    V, G = 6, 64
    rng = np.random.default_rng(0)
    zq = rng.normal(0, 1.5, size=V).astype(np.float32)
    zp = (zq + rng.normal(0, 1.0, size=V)).astype(np.float32)
    zb = rng.normal(0, 1.0, size=V).astype(np.float32)
    grid = ((np.arange(G) + 0.5) / G).astype(np.float32)
    xs, u1, u2 = np.meshgrid(np.arange(V), grid, grid, indexing="ij")
    B = xs.size
    draft = np.broadcast_to(zq, (B, 1, V)).copy()
    target = np.broadcast_to(np.stack([zp, zb]), (B, 2, V)).copy()
    x = xs.reshape(B, 1).astype(np.int32)
    u = np.stack([u1.ravel(), u2.ravel()], axis=1).astype(np.float32)
    print(f"[case] marginal quadrature B={B}", flush=True)
    out = ssd.ssd_verify(torch.from_numpy(draft).to(DEV), torch.from_numpy(target).to(DEV),
                         torch.from_numpy(x).to(DEV), torch.from_numpy(u).to(DEV), 1.0)
    k = out["accepted_len"].cpu().numpy()
    t = out["bonus_token"].cpu().numpy()
    first = np.where(k >= 1, x[:, 0], t)
    q = O.softmax_t(zq.astype(np.float64), 1.0)
    p = O.softmax_t(zp.astype(np.float64), 1.0)
    w = q[x[:, 0]] / (G * G)
    emp = np.bincount(first, weights=w, minlength=V)
    assert np.abs(emp - p).max() < 3.0 / G


def test_empty_batch_is_a_no_op():
    L = ssd.lib()
    ws = ssd.Workspace(256)
    st = L.ssd_verify(None, 400, None, 500, 0, 0, 4, 100, 1.0, None, None, None, 0, 1.0, None, None, 0, None,
                      None, None, None, None, ws.ptr, ws.nbytes, None)
    assert st == ssd.SSD_OK


def test_launch_count_and_tiles():
    # one launch while the batch's tiles fit on the device at once (MI355X: 256 CUs x 2), two beyond;
    # tiles per row follow the plan (bf16 4096-token tiles for the headline shape, smaller tiles when
    # the batch alone would leave CUs idle)
    assert ssd.ssd_verify_launches(16, 4, 128256, ssd.SSD_BF16, 3) == 1
    assert ssd.ssd_verify_launches(4096, 4, 128256, ssd.SSD_BF16, 3) == 2
    assert ssd.ssd_verify_launches(0, 4, 128256, ssd.SSD_BF16, 3) == 0
    assert ssd.ssd_verify_tiles(16, 4, 128256, ssd.SSD_BF16) == 32
    assert ssd.ssd_verify_tiles(1, 4, 32000, ssd.SSD_F32) == 32


def test_bf16_batch_of_64_sequences():
    bt = synth.make_verify_batch(64, 4, 128256, synth.BF16, 7)
    check_batch(bt, "b64_k4_v128256_bf16_top3", topf_F_max=3)


# --- per-position Saguaro factor ---------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_per_position_saguaro_c_matches_oracle(dtype):
    B, K, V = 8, 4, 30000
    bt = synth.make_verify_batch(B, K, V, dtype, 5, sag_sizes=[3, 2, 2, 2], C=0.5)
    Cs = [0.2, 0.5, 0.0, 1.0]
    d = batch_to_device(bt)
    aprob = torch.empty((B, K), dtype=torch.float32, device=DEV)
    rmass = torch.empty(B, dtype=torch.float32, device=DEV)
    print(f"[case] per-position C {dtype}", flush=True)
    call = ssd.VerifyCall(d["draft"], d["target"], d["x"], d["u"], bt.T, sag_set=d["sets"], sag_C=Cs,
                          topf_F_max=3, accept_prob=aprob, residual_mass=rmass)
    out = call()
    torch.cuda.synchronize()
    assert ssd.ssd_read_flags(call.workspace) == 0
    ref = O.verify_batch(bt.draft, bt.target, bt.dtype, bt.x, bt.u, bt.T, bt.sets, Cs)
    report(f"per-position C {dtype}", compare_verify(bt, out, ref, aprob, rmass))


def test_uniform_per_position_c_gives_the_single_value_bits():
    B, K, V = 8, 4, 50000
    bt = synth.make_verify_batch(B, K, V, synth.BF16, 6, sag_sizes=[3, 2, 2, 2], C=0.3)
    d = batch_to_device(bt)
    print("[case] uniform per-position C", flush=True)
    res = []
    for C in (0.3, [0.3] * K):
        aprob = torch.empty((B, K), dtype=torch.float32, device=DEV)
        rmass = torch.empty(B, dtype=torch.float32, device=DEV)
        out = ssd.ssd_verify(d["draft"], d["target"], d["x"], d["u"], bt.T, sag_set=d["sets"], sag_C=C,
                             topf_F_max=3, accept_prob=aprob, residual_mass=rmass)
        torch.cuda.synchronize()
        res.append([out["accepted_len"].cpu().numpy(), out["bonus_token"].cpu().numpy(),
                    aprob.cpu().numpy().view(np.int32), rmass.cpu().numpy().view(np.int32),
                    out["topf"].cpu().numpy()])
    for a, b in zip(*res):
        assert np.array_equal(a, b)
