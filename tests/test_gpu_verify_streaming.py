"""GPU tests of ssd_verify's streaming form (two grids: statistics and guesses of every tile; then,
over runs of tiles, the decision, the residual masses, the guess merge and the bonus): forced on
small shapes it gives the one-launch form's bits, and the oracle's results; chosen by shape for a
batch with more tiles than the device runs at once; one workspace serves both forms in turn."""
import numpy as np
import pytest
import torch

import draft_verification_ssd_amd as ssd
import oracle as O
import synth
from gpu_helpers import DEV, batch_to_device, compare_verify, report

pytestmark = pytest.mark.gpu

ONE, STREAM, BY_SHAPE = 1, 2, 0


def call_verify(bt, topf_F_max, launch_mode, workspace=None, last_F=0, stream=None):
    d = batch_to_device(bt, verify_rows_only=last_F == 0)
    B, K = bt.B, bt.K
    aprob = torch.empty((B, K), dtype=torch.float32, device=DEV)
    rmass = torch.empty(B, dtype=torch.float32, device=DEV)
    call = ssd.VerifyCall(d["draft"], d["target"], d["x"], d["u"], bt.T, sag_set=d.get("sets"), sag_C=bt.C,
                          topf_F_max=topf_F_max, accept_prob=aprob, residual_mass=rmass, workspace=workspace,
                          topf_last_F=last_F, launch_mode=launch_mode, stream=stream)
    out = call()
    torch.cuda.synchronize()
    assert call.flags() == 0, f"device flags {call.flags():#x}"
    host = [out["accepted_len"].cpu().numpy(), out["bonus_token"].cpu().numpy(), aprob.cpu().numpy().view(np.int32),
            rmass.cpu().numpy().view(np.int32)]
    for key in ("topf", "topf_last"):
        if out[key] is not None:
            host.append(out[key].cpu().numpy())
    return out, aprob, rmass, host


def check_oracle(bt, out, aprob, rmass, topf_F_max, name, last_F=0):
    ref = O.verify_batch(bt.draft, bt.target, bt.dtype, bt.x, bt.u, bt.T, bt.sets, bt.C)
    st = compare_verify(bt, out, ref, aprob, rmass)
    got = None if not topf_F_max else out["topf"].cpu().numpy()
    last = None if not last_F else out["topf_last"].cpu().numpy()
    for b in range(bt.B):
        for i in range(bt.K if topf_F_max else 0):
            want = O.topf(O.logits_f64(bt.draft[b, i], bt.dtype), topf_F_max, int(bt.x[b, i]))
            assert list(got[b, i]) == list(want), f"{name}: top-F of sequence {b} position {i}"
        if last_F:
            want = O.topf(O.logits_f64(bt.draft[b, bt.K], bt.dtype), last_F, -1)
            assert list(last[b]) == list(want), f"{name}: guesses of draft row K, sequence {b}"
    report(name, st)


def same_bits(h1, h2, name):
    assert len(h1) == len(h2)
    for n, (x, y) in enumerate(zip(h1, h2)):
        assert np.array_equal(x, y), f"{name}: output {n} differs between the one-launch and streaming forms"


FORCED = [
    # B, K, V, dtype, T, topf, saguaro, last_F
    (16, 4, 128256, "bf16", 1.0, 3, False, 0),
    (3, 4, 50021, "f32", 0.8, 4, True, 0),
    (5, 8, 65536, "bf16", 1.0, 2, False, 0),
    (2, 16, 16385, "f32", 1.0, 5, False, 0),
    (1, 4, 32000, "f32", 1.0, 0, False, 0),
    (1, 1, 1, "f32", 1.0, 0, False, 0),
    (2, 4, 2049, "bf16", 1.0, 5, False, 0),
    (7, 4, 1000, "bf16", 0.8, 3, True, 0),
    (5, 4, 12345, "bf16", 1.0, 2, False, 3),    # odd V: rows not 16-byte aligned; extra draft row
    (4, 3, 5003, "f32", 1.0, 3, False, 4),
    (4, 4, 40000, "f32", 1.0, 0, False, 3),     # guesses of the extra row only
]


@pytest.mark.parametrize("B,K,V,dtype,T,topf,sag,last_F", FORCED)
def test_streaming_form_gives_the_one_launch_bits(B, K, V, dtype, T, topf, sag, last_F):
    kw = dict(sag_sizes=[3] * K, C=0.4) if sag else {}
    bt = synth.make_verify_batch(B, K, V, dtype, 13, T=T, **kw)
    name = f"streaming B{B} K{K} V{V} {dtype} F{topf} last{last_F}"
    print(f"[case] {name}", flush=True)
    _, _, _, h1 = call_verify(bt, topf, ONE, last_F=last_F)
    o2, a2, r2, h2 = call_verify(bt, topf, STREAM, last_F=last_F)
    same_bits(h1, h2, name)
    check_oracle(bt, o2, a2, r2, topf, name, last_F)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_streaming_all_zero_residual_falls_back_to_the_target_row(dtype):
    """Identical draft and target rows with u_0 = 1: position 0 rejects and max(p - q, 0) is zero
    everywhere, so the last workgroup of the sequence in the second grid draws the bonus from p_0 (R reported 0)."""
    B, K, V = 6, 4, 20011
    bt = synth.make_verify_batch(B, K, V, dtype, 42)
    bt.target[:, :K] = bt.draft[:, :K]
    bt.u[:, 0] = np.float32(1.0)
    ref = O.verify_batch(bt.draft, bt.target, bt.dtype, bt.x, bt.u, bt.T)
    assert all(r.fallback and r.k == 0 and r.R == 0.0 for r in ref.values())
    print(f"[case] streaming, all-zero residual {dtype}", flush=True)
    _, _, _, h1 = call_verify(bt, 2, ONE)
    o2, a2, r2, h2 = call_verify(bt, 2, STREAM)
    same_bits(h1, h2, f"all-zero residual {dtype}")
    assert np.all(r2.cpu().numpy() == 0.0)
    check_oracle(bt, o2, a2, r2, 2, f"streaming, all-zero residual {dtype}")


def test_identical_rows_accept_everything_in_the_streaming_form():
    bt = synth.make_verify_batch(8, 6, 7777, synth.BF16, 3)
    bt.target[:, : bt.K] = bt.draft[:, : bt.K]
    bt.u[:, : bt.K] = np.float32(1 - 2 ** -24)
    print("[case] streaming, every draft accepted", flush=True)
    _, _, _, h1 = call_verify(bt, 3, ONE)
    o2, a2, r2, h2 = call_verify(bt, 3, STREAM)
    same_bits(h1, h2, "every draft accepted")
    assert np.all(o2["accepted_len"].cpu().numpy() == bt.K)
    check_oracle(bt, o2, a2, r2, 3, "streaming, every draft accepted")


@pytest.mark.parametrize("B", [17, 24])
def test_batch_beyond_the_device_takes_the_streaming_form(B):
    """17 and 24 sequences of the headline rows (32 tiles each): more tiles than 256 CUs run at once,
    so the shape picks the streaming form; the bits are the forced one-launch call's, and the oracle's."""
    assert ssd.ssd_verify_launches(B, 4, 128256, ssd.SSD_BF16, 3) == 2
    bt = synth.make_verify_batch(B, 4, 128256, synth.BF16, 30 + B)
    print(f"[case] B={B} headline rows by shape", flush=True)
    o0, a0, r0, h0 = call_verify(bt, 3, BY_SHAPE)
    _, _, _, h1 = call_verify(bt, 3, ONE)
    same_bits(h0, h1, f"B={B} by shape")
    check_oracle(bt, o0, a0, r0, 3, f"B={B} headline rows, streaming form by shape")


def test_one_workspace_serves_both_forms_in_turn():
    """Calls of both forms and of different shapes on one workspace, every one against the oracle:
    the streaming form's tag and counters must leave the workspace as a one-launch call expects it."""
    calls = [(16, 4, 128256, "bf16", ONE), (16, 4, 128256, "bf16", STREAM), (8, 4, 128256, "bf16", STREAM),
             (16, 4, 128256, "bf16", ONE), (6, 2, 70001, "f32", STREAM), (9, 8, 40000, "bf16", ONE),
             (24, 4, 128256, "bf16", BY_SHAPE), (16, 4, 128256, "bf16", BY_SHAPE)]
    need = max(ssd.ssd_verify_workspace_bytes(B, K, V, 3) for B, K, V, _, _ in calls)
    ws = ssd.Workspace(need, DEV)
    for n, (B, K, V, dtype, mode) in enumerate(calls):
        bt = synth.make_verify_batch(B, K, V, dtype, 200 + n)
        name = f"shared workspace call {n}: B{B} K{K} V{V} {dtype} mode {mode}"
        print(f"[case] {name}", flush=True)
        o, a, r, _ = call_verify(bt, 3, mode, workspace=ws)
        check_oracle(bt, o, a, r, 3, name)


def test_streaming_form_while_another_stream_holds_the_device():
    """A long read-only kernel on a second stream occupies the CUs while both grids are launched."""
    bt = synth.make_verify_batch(16, 4, 128256, synth.BF16, 5)
    busy = torch.empty(6 << 30, dtype=torch.uint8, device=DEV)  # ~1 ms of streaming
    sink = torch.zeros(8192, dtype=torch.int32, device=DEV)
    side = torch.cuda.Stream(device=DEV)
    torch.cuda.synchronize()
    print("[case] streaming form on a busy device", flush=True)
    for rep in range(2):
        with torch.cuda.stream(side):
            ssd.ssd_stream_read(busy, sink, stream=side)
        o, a, r, _ = call_verify(bt, 3, STREAM)
        check_oracle(bt, o, a, r, 3, f"streaming form, busy device rep {rep}")
    del busy
