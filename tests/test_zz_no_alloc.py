"""ssd_verify_noalloc, the allocation-free variant of ssd_verify (its workspace is the library's
static device array): its outputs equal ssd_verify's bit for bit on calls in a row, the second with
a smaller batch, vocabulary and dtype, and the caller's flags word stays zero."""
import numpy as np
import pytest
import torch

import draft_verification_ssd_amd as ssd
import synth
from gpu_helpers import DEV, batch_to_device

pytestmark = pytest.mark.gpu


def run(bt, topf, noalloc_flags=None):
    d = batch_to_device(bt)
    B, K = bt.B, bt.K
    aprob = torch.full((B, K), -1.0, dtype=torch.float32, device=DEV)
    rmass = torch.full((B,), -1.0, dtype=torch.float32, device=DEV)
    topf_out = torch.full((B, K, topf), -7, dtype=torch.int32, device=DEV) if topf else None
    call = ssd.VerifyCall(d["draft"], d["target"], d["x"], d["u"], bt.T, sag_set=d.get("sets"), sag_C=bt.C,
                          topf_F_max=topf, topf_out=topf_out, accept_prob=aprob, residual_mass=rmass,
                          noalloc_flags=noalloc_flags)
    out = call()
    torch.cuda.synchronize()
    res = [out["accepted_len"].cpu().numpy(), out["bonus_token"].cpu().numpy(),
           aprob.cpu().numpy().view(np.int32), rmass.cpu().numpy().view(np.int32)]
    if topf:
        res.append(topf_out.cpu().numpy())
    if noalloc_flags is None:
        assert call.flags() == 0
    return res


def test_noalloc_matches_ssd_verify_on_calls_of_shrinking_shape():
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    cases = [
        (synth.make_verify_batch(16, 4, 128256, synth.BF16, 3), 3, "B16 K4 V128256 bf16"),
        (synth.make_verify_batch(3, 2, 5003, synth.F32, 4, sag_sizes=[2, 2], C=0.3), 2, "B3 K2 V5003 f32"),
        (synth.make_verify_batch(16, 4, 128256, synth.BF16, 5), 3, "B16 K4 V128256 bf16 again"),
    ]
    for bt, topf, name in cases:
        print(f"[case] noalloc {name}", flush=True)
        want = run(bt, topf)
        got = run(bt, topf, noalloc_flags=flags)
        assert int(flags.item()) == 0, f"{name}: device flags {int(flags.item()):#x}"
        for i, (w, g) in enumerate(zip(want, got)):
            assert np.array_equal(w, g), f"{name}: output {i} differs"
