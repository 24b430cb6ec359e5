"""C-ABI contract tests that need no GPU: exports, argument validation, host-side fan-out.

No call here reaches a kernel launch: every device entry point is called with at least one invalid
argument, and the workspace pointer is NULL wherever the expected error comes earlier, so a
validation slip surfaces as a wrong status code rather than a launch.
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import draft_verification_ssd_amd as ssd
import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "ssd.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ssd.LIB_PATH), reason="libssd.so not built")

OK, INV, UNS, WS = ssd.SSD_OK, ssd.SSD_ERR_INVALID_ARG, ssd.SSD_ERR_UNSUPPORTED, ssd.SSD_ERR_WORKSPACE
FAKE = 0x1000          # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 10
    L = ssd.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(ssd.EXPORTS) == names


def test_status_strings():
    L = ssd.lib()
    for s in range(6):
        assert L.ssd_status_string(s)
    assert L.ssd_status_string(99) == b"unknown status"


def _verify(**over):
    B, K, V = 2, 4, 1000
    a = dict(draft=FAKE, dstride=K * V, target=FAKE, tstride=(K + 1) * V, dtype=ssd.SSD_F32, B=B, K=K,
             V=V, T=1.0, x=FAKE, u=FAKE, sset=None, sF=0, C=1.0, Cpos=None, topfF=None, topfFmax=0,
             topf_out=None, k=FAKE, bonus=FAKE, aprob=None, rmass=None, ws=None, wsb=0, stream=None)
    a.update(over)
    return ssd.lib().ssd_verify(*a.values())


@pytest.mark.parametrize("over,want", [
    (dict(dtype=7), UNS),
    (dict(B=-1), INV), (dict(B=70000), INV),
    (dict(K=0), INV), (dict(K=17), INV),
    (dict(V=0), INV), (dict(V=(1 << 20) + 1), INV),
    (dict(T=0.0), INV), (dict(T=-1.0), INV), (dict(T=float("inf")), INV), (dict(T=float("nan")), INV),
    (dict(sF=-1), INV), (dict(sF=17), INV), (dict(sF=2, sset=None), INV),
    (dict(sF=2, sset=FAKE, C=1.5), INV), (dict(sF=2, sset=FAKE, C=float("nan")), INV),
    (dict(topfFmax=17, topf_out=FAKE), INV), (dict(topfFmax=3, topf_out=None), INV),
    (dict(dstride=3999), INV), (dict(tstride=4999), INV),
    (dict(draft=None), INV), (dict(target=None), INV), (dict(x=None), INV), (dict(u=None), INV),
    (dict(k=None), INV), (dict(bonus=None), INV),
    (dict(), WS),                                       # no workspace
    (dict(ws=FAKE + 8, wsb=1 << 30), WS),               # misaligned workspace
    (dict(ws=FAKE * 16, wsb=64), WS),                   # too small
    (dict(B=0), OK),                                    # empty batch: nothing to do
])
def test_verify_argument_validation(over, want):
    assert _verify(**over) == want


def _verify_ex(opts, **over):
    B, K, V = 2, 4, 1000
    a = dict(draft=FAKE, dstride=K * V, target=FAKE, tstride=(K + 1) * V, dtype=ssd.SSD_F32, B=B, K=K,
             V=V, T=1.0, x=FAKE, u=FAKE, sset=None, sF=0, C=1.0, Cpos=None, topfF=None, topfFmax=0,
             topf_out=None, k=FAKE, bonus=FAKE, aprob=None, rmass=None, opts=ctypes.addressof(opts), ws=None,
             wsb=0, stream=None)
    a.update(over)
    return ssd.lib().ssd_verify_ex(*a.values())


@pytest.mark.parametrize("fields,over,want", [
    (dict(launch_mode=3), {}, INV), (dict(launch_mode=-1), {}, INV),
    (dict(wait_polls=(1 << 20) + 1), {}, INV),
    (dict(topf_last_F=17, topf_last_out=FAKE), dict(dstride=5000), INV),
    (dict(topf_last_F=2), dict(dstride=5000), INV),                   # no output for the extra row
    (dict(topf_last_F=2, topf_last_out=FAKE), {}, INV),                # draft stride without row K
    (dict(topf_last_F=2, topf_last_out=FAKE), dict(dstride=5000), WS),  # valid: fails at the workspace
    (dict(launch_mode=0), {}, WS), (dict(launch_mode=1), {}, WS), (dict(launch_mode=2), {}, WS),
    (dict(wait_polls=-5), {}, WS),                                     # < 0: the default
])
def test_verify_options_are_checked(fields, over, want):
    o = ssd.VerifyOpts(-1, 0, None, 0)
    for k, v in fields.items():
        setattr(o, k, v)
    assert _verify_ex(o, **over) == want


def test_verify_per_position_c_is_checked():
    good = (ctypes.c_float * 4)(0.5, 0.3, 1.0, 0.0)
    bad = (ctypes.c_float * 4)(0.5, 1.2, 1.0, 0.0)
    nan = (ctypes.c_float * 4)(0.5, float("nan"), 1.0, 0.0)
    assert _verify(sset=FAKE, sF=2, Cpos=ctypes.addressof(bad)) == INV
    assert _verify(sset=FAKE, sF=2, Cpos=ctypes.addressof(nan)) == INV
    assert _verify(sset=FAKE, sF=2, Cpos=ctypes.addressof(good)) == WS   # valid: fails at the workspace


def test_verify_topf_per_position_range_is_checked():
    F = (ctypes.c_int32 * 4)(1, 2, 4, 1)                  # 4 > topf_F_max = 3
    assert _verify(topfF=ctypes.addressof(F), topfFmax=3, topf_out=FAKE) == INV
    F2 = (ctypes.c_int32 * 4)(1, -1, 2, 1)
    assert _verify(topfF=ctypes.addressof(F2), topfFmax=3, topf_out=FAKE) == INV


def test_topf_and_saguaro_validation():
    L = ssd.lib()
    assert L.ssd_topf_guess(FAKE, 100, 9, 4, 100, None, None, 3, FAKE, None, 0, None) == UNS
    assert L.ssd_topf_guess(FAKE, 99, 0, 4, 100, None, None, 3, FAKE, None, 0, None) == INV
    assert L.ssd_topf_guess(FAKE, 100, 0, 4, 100, None, None, 0, FAKE, None, 0, None) == INV
    assert L.ssd_topf_guess(FAKE, 100, 0, 4, 100, None, None, 17, FAKE, None, 0, None) == INV
    assert L.ssd_topf_guess(None, 100, 0, 4, 100, None, None, 3, FAKE, None, 0, None) == INV
    assert L.ssd_topf_guess(FAKE, 100, 0, 4, 100, None, None, 3, None, None, 0, None) == INV
    assert L.ssd_topf_guess(FAKE, 100, 0, 4, 100, None, None, 3, FAKE, None, 0, None) == WS
    assert L.ssd_topf_guess(FAKE, 100, 0, 0, 100, None, None, 3, FAKE, None, 0, None) == OK
    sag = L.ssd_saguaro_adjust
    assert sag(FAKE, 100, 0, 4, 100, 0.0, None, 0, 0.5, None, None, None, None, None, 0, None) == INV
    assert sag(FAKE, 100, 0, 4, 100, 1.0, None, 2, 0.5, None, None, None, None, None, 0, None) == INV
    assert sag(FAKE, 100, 0, 4, 100, 1.0, FAKE, 2, -0.1, None, None, None, None, None, 0, None) == INV
    assert sag(FAKE, 100, 0, 4, 100, 1.0, FAKE, 17, 0.5, None, None, None, None, None, 0, None) == INV
    assert sag(FAKE, 99, 0, 4, 100, 1.0, FAKE, 2, 0.5, None, None, None, None, None, 0, None) == INV
    assert sag(FAKE, 100, 0, 4, 100, 1.0, FAKE, 2, 0.5, None, None, None, None, None, 0, None) == WS
    assert sag(FAKE, 100, 5, 4, 100, 1.0, FAKE, 2, 0.5, None, None, None, None, None, 0, None) == UNS
    assert sag(FAKE, 100, 0, 0, 100, 1.0, FAKE, 2, 0.5, None, None, None, None, None, 0, None) == OK


def test_saguaro_topf_validation():
    st = ssd.lib().ssd_saguaro_topf
    # (logits, stride, dtype, R, V, T, F_per_row, F_max, C, out_set, sigma, N, ws, bytes, stream)
    assert st(FAKE, 100, 9, 4, 100, 1.0, None, 3, 0.5, None, FAKE, None, None, None, 0, None) == UNS
    assert st(FAKE, 99, 0, 4, 100, 1.0, None, 3, 0.5, None, FAKE, None, None, None, 0, None) == INV
    assert st(FAKE, 100, 0, 4, 100, 0.0, None, 3, 0.5, None, FAKE, None, None, None, 0, None) == INV
    assert st(FAKE, 100, 0, 4, 100, float("inf"), None, 3, 0.5, None, FAKE, None, None, None, 0, None) == INV
    assert st(FAKE, 100, 0, 4, 100, 1.0, None, 0, 0.5, None, FAKE, None, None, None, 0, None) == INV
    assert st(FAKE, 100, 0, 4, 100, 1.0, None, 17, 0.5, None, FAKE, None, None, None, 0, None) == INV
    assert st(FAKE, 100, 0, 4, 100, 1.0, None, 3, 1.5, None, FAKE, None, None, None, 0, None) == INV
    assert st(FAKE, 100, 0, 4, 100, 1.0, None, 3, float("nan"), None, FAKE, None, None, None, 0, None) == INV
    assert st(None, 100, 0, 4, 100, 1.0, None, 3, 0.5, None, FAKE, None, None, None, 0, None) == INV
    assert st(FAKE, 100, 0, 4, 100, 1.0, None, 3, 0.5, None, None, None, None, None, 0, None) == INV
    assert st(FAKE, 100, 0, 4, 100, 1.0, None, 3, 0.5, None, FAKE, None, None, None, 0, None) == WS
    assert st(FAKE, 100, 0, 0, 100, 1.0, None, 3, 0.5, None, FAKE, None, None, None, 0, None) == OK
    assert ssd.ssd_saguaro_topf_workspace_bytes(768, 128256, 3) > 0
    assert ssd.ssd_saguaro_topf_workspace_bytes(4, 100, 0) == 0


def test_saguaro_sample_validation():
    st = ssd.lib().ssd_saguaro_sample
    # (logits, stride, dtype, R, V, T, F_per_row, F_max, C, C_per_row, u, token, prob, set, sigma, N,
    #  ws, bytes, stream)
    def call(**kw):
        a = dict(logits=FAKE, stride=100, dtype=0, R=4, V=100, T=1.0, Fr=None, Fmax=3, C=0.5, Cr=None,
                 u=FAKE, tok=FAKE, prob=None, set_=FAKE, sig=None, N=None, ws=None, nb=0, stream=None)
        a.update(kw)
        return st(*a.values())
    assert call(dtype=9) == UNS
    assert call(stride=99) == INV
    assert call(T=0.0) == INV
    assert call(Fmax=17) == INV
    assert call(Fmax=-1) == INV
    assert call(C=-0.1) == INV
    assert call(logits=None) == INV
    assert call(u=None) == INV
    assert call(tok=None) == INV
    assert call(set_=None) == INV
    assert call(set_=None, Fmax=0) == WS        # plain sampling needs no set buffer
    assert call() == WS
    assert call(R=0, u=None, tok=None) == OK
    assert ssd.ssd_saguaro_sample_workspace_bytes(2048, 128256, 3) > 0
    assert ssd.ssd_saguaro_sample_workspace_bytes(4, 100, 0) > 0
    assert ssd.ssd_saguaro_sample_workspace_bytes(4, 100, 17) == 0
    # few rows are cut into chunks, which then keep per-segment pairs in the workspace
    assert ssd.ssd_saguaro_sample_workspace_bytes(4, 128256, 3) > ssd.ssd_saguaro_topf_workspace_bytes(4, 128256, 3)


def test_cache_validation():
    L = ssd.lib()
    F = (ctypes.c_int32 * 5)(3, 2, 2, 2, 3)
    # fan-out must sum to the budget and fit the guess width
    assert L.ssd_cache_keys(2, 4, 3, FAKE, None, 0, ctypes.addressof(F), 11, FAKE, FAKE, None) == INV
    assert L.ssd_cache_keys(2, 4, 2, FAKE, None, 0, ctypes.addressof(F), 12, FAKE, FAKE, None) == INV
    assert L.ssd_cache_keys(2, 4, 3, FAKE, None, 0, None, 12, FAKE, FAKE, None) == INV
    assert L.ssd_cache_keys(2, 4, 3, None, None, 0, ctypes.addressof(F), 12, FAKE, FAKE, None) == INV
    assert L.ssd_cache_keys(0, 4, 3, FAKE, None, 0, ctypes.addressof(F), 12, FAKE, FAKE, None) == OK
    # position K's guesses apart: their width bounds F_K (3 here), not G_max
    assert L.ssd_cache_keys(2, 4, 3, FAKE, FAKE, 2, ctypes.addressof(F), 12, FAKE, FAKE, None) == INV
    assert L.ssd_cache_keys(2, 4, 3, FAKE, FAKE, 0, ctypes.addressof(F), 12, FAKE, FAKE, None) == INV
    assert L.ssd_cache_keys(0, 4, 2, FAKE, FAKE, 3, ctypes.addressof((ctypes.c_int32 * 5)(2, 2, 2, 2, 3)), 11, FAKE, FAKE, None) == OK
    assert L.ssd_cache_lookup(2, 12, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == INV
    assert L.ssd_cache_lookup(2, 12, None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == INV
    assert L.ssd_cache_lookup(-1, 12, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == INV
    assert L.ssd_read_flags(None, FAKE, 1, None) == INV


def test_workspace_sizes():
    a = ssd.ssd_verify_workspace_bytes(16, 4, 128256, 3)
    b = ssd.ssd_verify_workspace_bytes(128, 8, 152064, 4)
    assert 0 < a < b and a % 256 == 0
    assert ssd.ssd_verify_workspace_bytes(16, 0, 128256, 3) == 0
    assert ssd.ssd_topf_workspace_bytes(768, 128256, 3) > 0
    assert ssd.ssd_saguaro_workspace_bytes(8192, 128256) > 0


def test_verify_launch_count_rejects_what_verify_rejects():
    for args in [(-1, 4, 1000, ssd.SSD_BF16, 3), (1, 0, 1000, ssd.SSD_BF16, 3), (1, 17, 1000, ssd.SSD_F32, 0),
                 (1, 4, 0, ssd.SSD_F32, 0), (1, 4, (1 << 20) + 1, ssd.SSD_F32, 0), (1, 4, 1000, 7, 0),
                 (1, 4, 1000, ssd.SSD_BF16, 17), (1, 4, 1000, ssd.SSD_BF16, -1)]:
        assert ssd.ssd_verify_launches(*args) == -1, args
    assert ssd.ssd_verify_launches(0, 4, 1000, ssd.SSD_BF16, 3) == 0


def test_verify_launch_count_follows_the_tiles_the_device_runs_at_once():
    # 256 CUs x 2 workgroups (the count the library assumes when no device answers, and MI355X's):
    # 16 x 32 tiles fit, 17 x 32 do not
    assert ssd.ssd_verify_tiles(16, 4, 128256, ssd.SSD_BF16) == 32
    assert ssd.ssd_verify_launches(16, 4, 128256, ssd.SSD_BF16, 3) == 1
    assert ssd.ssd_verify_launches(17, 4, 128256, ssd.SSD_BF16, 3) == 2
    assert ssd.ssd_verify_launches(128, 8, 152064, ssd.SSD_F32, 4) == 2
    assert ssd.ssd_verify_launches(1, 4, 32000, ssd.SSD_F32, 0) == 1


@pytest.mark.parametrize("K,a,r,budget", [(4, 0.7, 1.0, 12), (4, 0.7, 1.0, 32), (8, 0.55, 0.5, 100),
                                          (2, 0.9, 2.0, 7), (0, 0.5, 1.0, 5), (6, 0.3, 1.5, 0),
                                          (16, 0.8, 1.0, 1000), (3, 0.99, 0.1, 9)])
def test_fanout_matches_the_oracle(K, a, r, budget):
    F, Fc = ssd.ssd_fanout_alloc(K, a, r, budget)
    Fo, Fco = O.fanout(K, a, r, budget)
    assert F == [int(v) for v in Fo]
    np.testing.assert_allclose(Fc, Fco, rtol=1e-12, atol=1e-12)


def test_fanout_validation():
    L = ssd.lib()
    out = (ctypes.c_int32 * 5)()
    for args in [(4, 1.0, 1.0, 3), (4, 0.0, 1.0, 3), (4, 0.5, 0.0, 3), (4, 0.5, 1.0, -1), (-1, 0.5, 1.0, 3)]:
        assert L.ssd_fanout_alloc(*args, ctypes.addressof(out), None) == INV
    assert L.ssd_fanout_alloc(4, 0.5, 1.0, 3, None, None) == INV


# ------------------------------------------------------------------------------------------
# host-only speedup model against the oracle
# ------------------------------------------------------------------------------------------
def test_batch_speedup_matches_the_oracle():
    rng = np.random.default_rng(3)
    for _ in range(300):
        h, Eh, Em = rng.uniform(0, 1), rng.uniform(0, 8), rng.uniform(0, 4)
        Tp, Tb, b = rng.uniform(0, 2), rng.uniform(0, 3), int(rng.integers(1, 500))
        got = ssd.ssd_batch_speedup(h, Eh, Em, Tp, Tb, b)
        assert abs(got - O.batch_speedup(h, Eh, Em, Tp, Tb, b)) <= 1e-12 * max(1.0, got)
    assert ssd.ssd_batch_speedup(1.0, 5.0, 1.0, 0.2, 3.0, 64) == 5.0


def test_backup_crossover_matches_the_oracle():
    rng = np.random.default_rng(4)
    crossed = 0
    for _ in range(500):
        args = (rng.uniform(0.3, 0.999), rng.uniform(1, 6), rng.uniform(1, 4), rng.uniform(0, 2),
                rng.uniform(0.5, 2), rng.uniform(0, 0.5), rng.uniform(0, 1.5))
        b, fl = ssd.ssd_backup_crossover(*args)
        b_ref, fl_ref = O.backup_crossover(*args)
        assert fl == fl_ref
        if math.isnan(b_ref):
            assert math.isnan(b)
        else:
            crossed += 1
            assert abs(b - b_ref) <= 1e-9 * max(1.0, b_ref)
    assert crossed > 50
    b, fl = ssd.ssd_backup_crossover(1.0, 4, 3, 1, 1, 0, 0.5)      # no misses: never cross
    assert math.isnan(b)


def test_speedup_validation():
    L = ssd.lib()
    out = ctypes.c_double()
    assert L.ssd_batch_speedup(1.5, 1, 1, 0, 0, 1, ctypes.byref(out)) == INV
    assert L.ssd_batch_speedup(0.5, -1, 1, 0, 0, 1, ctypes.byref(out)) == INV
    assert L.ssd_batch_speedup(0.5, 1, 1, 0, float("inf"), 1, ctypes.byref(out)) == INV
    assert L.ssd_batch_speedup(0.5, 1, 1, 0, 0, 0, ctypes.byref(out)) == INV
    assert L.ssd_batch_speedup(0.5, 1, 1, 0, 0, 1, None) == INV
    assert L.ssd_backup_crossover(0.5, 1, 1, 0, 1, 0, float("nan"), ctypes.byref(out), None) == INV
    assert L.ssd_backup_crossover(0.5, 1, 1, 0, 1, 0, 0, None, None) == INV


def _verify_noalloc(**over):
    B, K, V = 2, 4, 1000
    a = dict(draft=FAKE, dstride=K * V, target=FAKE, tstride=(K + 1) * V, dtype=ssd.SSD_F32, B=B, K=K,
             V=V, T=1.0, x=FAKE, u=FAKE, sset=None, sF=0, C=1.0, Cpos=None, topfF=None, topfFmax=0,
             topf_out=None, k=FAKE, bonus=FAKE, aprob=None, rmass=None, flags=FAKE, stream=None)
    a.update(over)
    return ssd.lib().ssd_verify_noalloc(*a.values())


@pytest.mark.parametrize("over,want", [
    (dict(flags=None), INV), (dict(dtype=7), UNS), (dict(B=-1), INV), (dict(T=0.0), INV),
    (dict(k=None), INV),
    # past the static array: B = 4096 sequences of K = 16 at V = 2^20 need far more than 32 MiB
    (dict(B=4096, K=16, V=1 << 20, dstride=16 << 20, tstride=17 << 20), ssd.SSD_ERR_SCRATCH_LIMIT),
])
def test_verify_noalloc_rejects_before_any_launch(over, want):
    assert _verify_noalloc(**over) == want


def test_verify_noalloc_limit_matches_the_workspace_size():
    # the headline shape fits the static array; the limit is the workspace size itself
    assert ssd.ssd_verify_workspace_bytes(16, 4, 128256, 3) <= ssd.SSD_NOALLOC_SCRATCH_BYTES
    assert ssd.ssd_verify_workspace_bytes(4096, 16, 1 << 20, 16) > ssd.SSD_NOALLOC_SCRATCH_BYTES
    assert _verify_noalloc(B=0) == OK  # an empty batch is a no-op, before the array is touched


def test_cache_keys_lookup_validates_like_its_two_calls():
    L = ssd.lib()
    F = (ctypes.c_int32 * 3)(2, 1, 1)
    call = lambda B, K, G, g, budget, k, t, ck, ct, sl, m: L.ssd_cache_keys_lookup(
        B, K, G, g, None, 0, ctypes.addressof(F), budget, k, t, ck, ct, sl, m, None)
    assert call(2, 2, 2, FAKE, 3, FAKE, FAKE, FAKE, FAKE, FAKE, None) == INV   # no miss-count output
    assert call(2, 2, 2, FAKE, 5, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE) == INV   # budget != sum(fanout)
    assert call(2, 2, 1, FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE) == INV   # F_0 = 2 > G_max = 1
    assert call(2, 2, 2, None, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE) == INV   # no guesses
    assert call(2, 2, 2, FAKE, 4, None, FAKE, FAKE, FAKE, FAKE, FAKE) == INV   # no outcomes
    assert call(-1, 2, 2, FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE) == INV
