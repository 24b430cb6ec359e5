"""The seeded generators: determinism, shapes, bf16 rounding, and draft tokens that follow q'."""
import numpy as np
import torch

import synth


def test_bf16_round_to_nearest_even_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 3, 100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.0e38, 1e-40], np.float32)])
    bits = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    back = synth.bf16_bits_to_f32(bits)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_batch_is_deterministic_and_shaped():
    a = synth.make_verify_batch(3, 4, 1000, synth.BF16, seed=7)
    b = synth.make_verify_batch(3, 4, 1000, synth.BF16, seed=7)
    c = synth.make_verify_batch(3, 4, 1000, synth.BF16, seed=8)
    for f in ["draft", "target", "x", "u"]:
        assert np.array_equal(getattr(a, f), getattr(b, f))
    assert not np.array_equal(a.draft, c.draft)
    assert a.draft.shape == (3, 5, 1000) and a.target.shape == (3, 5, 1000)
    assert a.draft.dtype == np.uint16 and a.x.dtype == np.int32 and a.u.dtype == np.float32
    assert a.x.shape == (3, 4) and a.u.shape == (3, 5)
    assert np.all((a.u >= 0) & (a.u < 1)) and np.all((a.x >= 0) & (a.x < 1000))


def test_saguaro_sets_hold_the_top_logits_and_c0_excludes_them():
    bt = synth.make_verify_batch(4, 3, 500, synth.F32, seed=3, sag_sizes=[3, 2, 1], C=0.0)
    for b in range(4):
        for i, F in enumerate([3, 2, 1]):
            z = bt.draft[b, i]
            assert set(bt.sets[b, i, :F]) == set(np.argsort(-z)[:F])
            assert np.all(bt.sets[b, i, F:] == -1)
            assert bt.x[b, i] not in set(bt.sets[b, i, :F])


def test_draft_tokens_follow_the_draft_distribution():
    # Gumbel-max draws: frequencies over a small vocabulary match softmax(z / T).
    V, B = 5, 4000
    bt = synth.make_verify_batch(B, 1, V, synth.F32, seed=11, draft_sigma=1.0, T=0.7)
    # each sequence has its own row; pool the per-row probabilities
    z = bt.draft[:, 0].astype(np.float64) / 0.7
    p = np.exp(z - z.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    hits = p[np.arange(B), bt.x[:, 0]].mean()
    expect = (p ** 2).sum(1).mean()   # E[p(x)] when x ~ p
    assert abs(hits - expect) < 0.02


def test_branch_uniforms_are_seeded_and_leave_the_other_streams_alone():
    """The branch rows' sampling uniforms come from a sixth child stream: deterministic, in [0, 1),
    and adding that stream left the five earlier ones (and so every earlier input) unchanged."""
    import numpy as np
    a = synth.make_branch_uniforms(3, 4, 2, seed=5)
    b = synth.make_branch_uniforms(3, 4, 2, seed=5)
    assert a.shape == (3, 4, 2) and a.dtype == np.float32
    assert np.array_equal(a, b) and (a >= 0).all() and (a < 1).all()
    assert not np.array_equal(a, synth.make_branch_uniforms(3, 4, 2, seed=6))
    five = np.random.SeedSequence(5).spawn(5)
    six = np.random.SeedSequence(5).spawn(6)
    for x, y in zip(five, six[:5]):
        assert np.array_equal(np.random.Generator(np.random.PCG64(x)).random(8),
                              np.random.Generator(np.random.PCG64(y)).random(8))
