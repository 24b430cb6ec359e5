"""GPU tests of ssd_verify's exchange between the workgroups of a sequence: every duty a tile hands
over (wait_polls = 0) lands in the sequence's last tile with the same result bits; one workspace
serves calls of different shapes in turn; the all-zero residual falls back to the target row;
and the result is the oracle's while another stream keeps the device busy."""
import numpy as np
import pytest
import torch

import draft_verification_ssd_amd as ssd
import oracle as O
import synth
from gpu_helpers import DEV, batch_to_device, compare_verify, report

pytestmark = pytest.mark.gpu


def call_verify(bt, topf_F_max=3, wait_polls=None, workspace=None, stream=None):
    d = batch_to_device(bt)
    B, K = bt.B, bt.K
    aprob = torch.empty((B, K), dtype=torch.float32, device=DEV)
    rmass = torch.empty(B, dtype=torch.float32, device=DEV)
    call = ssd.VerifyCall(d["draft"], d["target"], d["x"], d["u"], bt.T, sag_set=d.get("sets"), sag_C=bt.C,
                          topf_F_max=topf_F_max, accept_prob=aprob, residual_mass=rmass, wait_polls=wait_polls,
                          workspace=workspace, stream=stream)
    out = call()
    return call, out, aprob, rmass


def outputs_host(out, aprob, rmass):
    res = [out["accepted_len"].cpu().numpy(), out["bonus_token"].cpu().numpy(), aprob.cpu().numpy().view(np.int32),
           rmass.cpu().numpy().view(np.int32)]
    if out["topf"] is not None:
        res.append(out["topf"].cpu().numpy())
    return res


def check_oracle(bt, out, aprob, rmass, topf_F_max, name):
    ref = O.verify_batch(bt.draft, bt.target, bt.dtype, bt.x, bt.u, bt.T, bt.sets, bt.C)
    st = compare_verify(bt, out, ref, aprob, rmass)
    if topf_F_max:
        got = out["topf"].cpu().numpy()
        for b in range(bt.B):
            for i in range(bt.K):
                want = O.topf(O.logits_f64(bt.draft[b, i], bt.dtype), topf_F_max, int(bt.x[b, i]))
                assert list(got[b, i]) == list(want), f"{name}: top-F of sequence {b} position {i}"
    report(name, st)


HANDOVER = [
    # B, K, V, dtype, T, topf, saguaro
    (16, 4, 128256, "bf16", 1.0, 3, False),
    (3, 4, 50021, "f32", 0.8, 4, True),
    (5, 8, 65536, "bf16", 1.0, 2, False),
    (2, 16, 16385, "f32", 1.0, 5, False),
    (1, 4, 32000, "f32", 1.0, 0, False),
]


@pytest.mark.parametrize("B,K,V,dtype,T,topf,sag", HANDOVER)
def test_every_tile_hands_over_to_the_last(B, K, V, dtype, T, topf, sag):
    """wait_polls = 0: tiles do not wait for each other; the last tile of each sequence computes the
    residual of the others and draws the bonus. Same bits as the default call, and the oracle's."""
    kw = dict(sag_sizes=[3] * K, C=0.4) if sag else {}
    bt = synth.make_verify_batch(B, K, V, dtype, 11, T=T, **kw)
    print(f"[case] hand-over B{B} K{K} V{V} {dtype}", flush=True)
    c0, o0, a0, r0 = call_verify(bt, topf, wait_polls=None)
    torch.cuda.synchronize()
    assert c0.flags() == 0
    h0 = outputs_host(o0, a0, r0)
    c1, o1, a1, r1 = call_verify(bt, topf, wait_polls=0)
    torch.cuda.synchronize()
    assert c1.flags() == 0
    h1 = outputs_host(o1, a1, r1)
    for x, y in zip(h0, h1):
        assert np.array_equal(x, y)
    check_oracle(bt, o1, a1, r1, topf, f"hand-over B{B} K{K} V{V} {dtype}")


def test_one_workspace_serves_calls_of_different_shapes():
    """B = 16, then 8, then 16 again (and other K, V, dtypes) on one workspace, every call against the
    oracle: a smaller call must not leave words that a later larger call takes as its own."""
    shapes = [(16, 4, 128256, "bf16"), (8, 4, 128256, "bf16"), (16, 4, 128256, "bf16"), (6, 2, 70001, "f32"),
              (16, 4, 128256, "bf16"), (9, 8, 40000, "bf16"), (16, 4, 128256, "bf16")]
    need = max(ssd.ssd_verify_workspace_bytes(B, K, V, 3) for B, K, V, _ in shapes)
    ws = ssd.Workspace(need, DEV)
    for n, (B, K, V, dtype) in enumerate(shapes):
        bt = synth.make_verify_batch(B, K, V, dtype, 100 + n)
        print(f"[case] shared workspace call {n}: B{B} K{K} V{V} {dtype}", flush=True)
        for wp in (None, 0):
            c, o, a, r = call_verify(bt, 3, wait_polls=wp, workspace=ws)
            torch.cuda.synchronize()
            assert c.flags() == 0
            check_oracle(bt, o, a, r, 3, f"shared workspace call {n} wait_polls={wp}")


@pytest.mark.parametrize("wait_polls", [None, 0])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_zero_residual_falls_back_to_the_target_row(wait_polls, dtype):
    """Identical draft and target rows with u_0 = 1: u q = q = p is not < p, so position 0 rejects,
    and max(p - q, 0) is zero everywhere. The bonus is drawn from p_0 with u_K (R reported 0)."""
    B, K, V = 6, 4, 20011
    bt = synth.make_verify_batch(B, K, V, dtype, 42)
    bt.target[:, :K] = bt.draft[:, :K]
    bt.u[:, 0] = np.float32(1.0)
    ref = O.verify_batch(bt.draft, bt.target, bt.dtype, bt.x, bt.u, bt.T)
    assert all(r.fallback and r.k == 0 and r.R == 0.0 for r in ref.values())
    print(f"[case] all-zero residual {dtype} wait_polls={wait_polls}", flush=True)
    c, o, a, r = call_verify(bt, 2, wait_polls=wait_polls)
    torch.cuda.synchronize()
    assert c.flags() == 0
    assert np.all(o["accepted_len"].cpu().numpy() == 0)
    assert np.all(r.cpu().numpy() == 0.0)
    check_oracle(bt, o, a, r, 2, f"all-zero residual {dtype}")


@pytest.mark.parametrize("wait_polls", [None, 4])
def test_verify_while_another_stream_holds_the_device(wait_polls):
    """A long read-only kernel on a second stream occupies the CUs while ssd_verify is launched: its
    workgroups start in whatever slots free up. The outputs must be the oracle's, with no flag."""
    bt = synth.make_verify_batch(16, 4, 128256, synth.BF16, 5)
    busy = torch.empty(6 << 30, dtype=torch.uint8, device=DEV)  # ~1 ms of streaming
    sink = torch.zeros(8192, dtype=torch.int32, device=DEV)
    side = torch.cuda.Stream(device=DEV)
    d = batch_to_device(bt)
    aprob = torch.empty((16, 4), dtype=torch.float32, device=DEV)
    rmass = torch.empty(16, dtype=torch.float32, device=DEV)
    call = ssd.VerifyCall(d["draft"], d["target"], d["x"], d["u"], bt.T, topf_F_max=3, accept_prob=aprob,
                          residual_mass=rmass, wait_polls=wait_polls)
    torch.cuda.synchronize()
    print(f"[case] busy device wait_polls={wait_polls}", flush=True)
    for rep in range(3):
        with torch.cuda.stream(side):
            ssd.ssd_stream_read(busy, sink, stream=side)
        out = call()
        torch.cuda.synchronize()
        assert call.flags() == 0
        check_oracle(bt, out, aprob, rmass, 3, f"busy device rep {rep} wait_polls={wait_polls}")
    del busy
