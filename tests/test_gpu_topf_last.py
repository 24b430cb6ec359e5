"""GPU parity of the extra draft row's guesses inside ssd_verify (ssd_verify_opts.topf_last_F): the
top-F of draft row K with nothing excluded ([SSD] "怎么猜奖励 token": the outcome k = K), read in
the same pass as the verification. Against the oracle's topf, and the rest of the call's outputs
bit for bit as without the option."""
import numpy as np
import pytest
import torch

import draft_verification_ssd_amd as ssd
import oracle as O
import synth
from gpu_helpers import DEV, batch_to_device

pytestmark = pytest.mark.gpu


def _call(bt, topf, last_F, sets=True):
    d = batch_to_device(bt, verify_rows_only=False)  # the draft keeps its row K
    B, K = bt.B, bt.K
    aprob = torch.empty((B, K), dtype=torch.float32, device=DEV)
    rmass = torch.empty(B, dtype=torch.float32, device=DEV)
    call = ssd.VerifyCall(d["draft"], d["target"], d["x"], d["u"], bt.T, sag_set=d.get("sets") if sets else None,
                          sag_C=bt.C, topf_F_max=topf, accept_prob=aprob, residual_mass=rmass,
                          topf_last_F=last_F)
    out = call()
    torch.cuda.synchronize()
    assert call.flags() == 0
    res = [out["accepted_len"].cpu().numpy(), out["bonus_token"].cpu().numpy(), aprob.cpu().numpy().view(np.int32),
           rmass.cpu().numpy().view(np.int32)]
    if topf:
        res.append(out["topf"].cpu().numpy())
    return res, (out["topf_last"].cpu().numpy() if last_F else None)


CASES = [
    # B, K, V, dtype, topf, last_F, ties
    (16, 4, 128256, "bf16", 3, 3, False),     # the cache-build shape
    (16, 4, 128256, "bf16", 3, 3, True),
    (5, 4, 50021, "f32", 2, 7, False),        # more guesses for the extra row than for the others
    (3, 8, 65536, "bf16", 0, 4, False),       # only the extra row
    (4, 2, 12345, "bf16", 2, 3, True),        # rows not 16-byte aligned
    (2, 16, 20000, "f32", 1, 12, True),       # more guesses than hot-lane slots: compaction
    (1, 1, 7, "f32", 1, 9, False),            # fewer tokens than guesses: -1 padding
]


@pytest.mark.parametrize("B,K,V,dtype,topf,last_F,ties", CASES)
def test_extra_row_guesses_match_oracle(B, K, V, dtype, topf, last_F, ties):
    bt = synth.make_verify_batch(B, K, V, dtype, 21 + K)
    if ties:  # integer-valued draft rows: many equal logits
        z = np.round(O.logits_f64(bt.draft, dtype)).astype(np.float32)
        bt.draft = synth.f32_to_bf16_bits(z) if dtype == "bf16" else z
    print(f"[case] extra-row guesses B{B} K{K} V{V} {dtype} F{topf} last{last_F} ties={ties}", flush=True)
    base, _ = _call(bt, topf, 0)
    got, last = _call(bt, topf, last_F)
    for i, (x, y) in enumerate(zip(base, got)):
        assert np.array_equal(x, y), f"output {i} changed with the extra row's guesses"
    for b in range(B):
        want = O.topf(O.logits_f64(bt.draft[b, K], dtype), last_F)
        assert list(last[b]) == list(want), f"sequence {b}: {list(last[b])} != {list(want)}"
