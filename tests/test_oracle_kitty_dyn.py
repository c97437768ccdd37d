"""Pins of the oracle's Kitty dynamic boost (per-page channel selection).

Kitty summary, "Channel-Wise Precision Boost Mechanism": within a group the
channels are ranked by mean absolute value and the top K are boosted to 4
bits.  Reading taken: the group is one 64-token page of the cache; ties go to
the lower channel; offsets follow ascending channel order, the sentinel is
D_b + 1 (as for the static boost).  Pins: the selection equals a brute-force
top-K over exact sums; with a selection that is the same on every page the
scheme equals the static Kitty scheme bit for bit; a page's selection depends
on its own tokens only; streaming equals bulk prefill; boosted channels take
16 levels within the error bound of the quantizer.
"""
import numpy as np
import pytest

from oracle import oracle as O

D = 128
NB = 16


def f16(x):
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def f32(h):
    return np.asarray(h, np.uint16).view(np.float16).astype(np.float32)


def brute_select(k, nb):
    imp = np.abs(f32(k).astype(np.float64)).sum(axis=0)      # exact for fp16 inputs
    order = np.lexsort((np.arange(D), -imp))                  # mean |x| desc, channel asc
    chosen = np.sort(order[:nb])
    idx = np.full(D, nb + 1, np.uint8)
    idx[chosen] = np.arange(nb)
    return idx


def test_selection_is_topk_of_mean_abs():
    rng = np.random.default_rng(11)
    for trial in range(30):
        x = rng.standard_normal((64, D)).astype(np.float32) * rng.uniform(0.05, 8, D).astype(np.float32)
        if trial % 3 == 1:                       # exact ties: equal sums, lower channel first
            x[:, 40] = 3.0; x[:, 41] = -3.0; x[:, 90] = 3.0
            x[:, 40:42] *= 1.0
        if trial % 3 == 2:                       # sign does not matter, only |x|
            x[:, 7] = -np.abs(x[:, 7]) * 50
        k = f16(x)
        assert np.array_equal(O.kitty_select_dyn(k, NB), brute_select(k, NB)), trial


def test_tie_goes_to_lower_channel():
    x = np.ones((64, D), np.float32) * 0.5
    x[:, 100:120] = 2.0                          # 20 tied channels, 16 places
    idx = O.kitty_select_dyn(f16(x), NB)
    assert np.array_equal(np.nonzero(idx < NB)[0], np.arange(100, 116))
    assert np.array_equal(idx[100:116], np.arange(NB))
    assert np.all(idx[116:120] == NB + 1)


def test_constant_selection_equals_static_kitty():
    rng = np.random.default_rng(12)
    n = 900
    big = np.array([1, 5, 9, 20, 33, 34, 47, 60, 64, 71, 88, 99, 100, 111, 120, 127])
    K = rng.standard_normal((n, D)).astype(np.float32)
    K[:, big] = 40.0 + rng.uniform(0, 1, (n, big.size)).astype(np.float32)   # top 16 on every page
    V = rng.standard_normal((n, D)).astype(np.float32)
    K, V = f16(K), f16(V)
    idx = np.full(D, NB + 1, np.uint8)
    idx[big] = np.arange(NB)
    a = O.Stream(O.KITTY, 1024, nb=NB, idx=idx)
    b = O.Stream(O.KITTY_DYN, 1024, nb=NB, sel=64)
    a.prefill(K, V)
    b.prefill(K, V)
    l, n_kq, _ = b.state
    assert np.array_equal(a.key_codes(), b.key_codes())
    assert all(np.array_equal(x, y) for x, y in zip(a.key_stats(), b.key_stats()))
    assert np.all(b.unit_index()[: n_kq // 64] == idx)


def test_each_page_selects_from_its_own_tokens():
    rng = np.random.default_rng(13)
    n = 600
    K = rng.standard_normal((n, D)).astype(np.float32)
    K[0:64, 0:16] *= 30.0                        # page 0: channels 0..15 dominate
    K[64:128, 100:116] *= 30.0                   # page 1: channels 100..115 dominate
    V = rng.standard_normal((n, D)).astype(np.float32)
    s = O.Stream(O.KITTY_DYN, 1024, nb=NB, sel=64)
    s.prefill(f16(K), f16(V))
    u = s.unit_index()
    assert np.array_equal(np.nonzero(u[0] < NB)[0], np.arange(16))
    assert np.array_equal(np.nonzero(u[1] < NB)[0], np.arange(100, 116))
    # changing page 1 leaves page 0's selection and codes alone
    K2 = K.copy()
    K2[64:128] = rng.standard_normal((64, D)).astype(np.float32)
    t = O.Stream(O.KITTY_DYN, 1024, nb=NB, sel=64)
    t.prefill(f16(K2), f16(V))
    assert np.array_equal(t.unit_index()[0], u[0])
    assert np.array_equal(t.key_codes()[:64], s.key_codes()[:64])
    for n_ in range(2, 4):                       # later pages follow brute force too
        assert np.array_equal(u[n_], brute_select(f16(K)[64 * n_:64 * n_ + 64], NB))


def test_streaming_equals_bulk_prefill():
    rng = np.random.default_rng(14)
    n0, extra = 300, 200
    K = f16(rng.standard_normal((n0 + extra, D)) * rng.uniform(0.1, 5, D))
    V = f16(rng.standard_normal((n0 + extra, D)))
    a = O.Stream(O.KITTY_DYN, 1024, nb=NB, sel=64)
    a.prefill(K[:n0], V[:n0])
    for t in range(n0, n0 + extra):
        a.flush()
        assert a.append(K[t], V[t]) == 0
    b = O.Stream(O.KITTY_DYN, 1024, nb=NB, sel=64)
    b.prefill(K, V)
    assert a.state == b.state
    assert np.array_equal(a.key_codes(), b.key_codes())
    assert np.array_equal(a.value_codes(), b.value_codes())
    assert np.array_equal(a.unit_index(), b.unit_index())
    assert all(np.array_equal(x, y) for x, y in zip(a.key_stats() + a.value_stats(),
                                                     b.key_stats() + b.value_stats()))


def test_boosted_channels_take_sixteen_levels_within_bound():
    rng = np.random.default_rng(15)
    K = f16(rng.standard_normal((640, D)) * rng.uniform(0.1, 6, D))
    V = f16(rng.standard_normal((640, D)))
    s = O.Stream(O.KITTY_DYN, 1024, nb=NB, sel=64)
    s.prefill(K, V)
    l, n_kq, _ = s.state
    codes = s.key_codes()[:n_kq]
    u = s.unit_index()
    for p in range(n_kq // 64):
        boosted = u[p] < NB
        assert boosted.sum() == NB
        page = codes[64 * p:64 * p + 64]
        assert page[:, ~boosted].max() <= 3 and page[:, boosted].max() > 3
    Kt, _ = s.dequant(0, n_kq)
    ks, _ = s.key_stats()
    step = f32(ks[: n_kq // 32]).repeat(32, axis=0).astype(np.float64)
    err = np.abs(f32(K[:n_kq]).astype(np.float64) - Kt)
    assert np.all(err <= step / 2 * (1 + 2.0 ** -20) + 1e-30)


@pytest.mark.parametrize("sel", [0, 48, 256])
def test_selection_unit_must_divide_the_residual(sel):
    with pytest.raises(ValueError):
        O.Stream(O.KITTY_DYN, 1024, nb=NB, sel=sel)       # R = 128, G = 32


def brute_select_amax(k, nb):
    amax = np.abs(f32(k)).max(axis=0)
    order = np.lexsort((np.arange(D), -amax))
    chosen = np.sort(order[:nb])
    idx = np.full(D, nb + 1, np.uint8)
    idx[chosen] = np.arange(nb)
    return idx


@pytest.mark.parametrize("scheme", [O.KITTY, O.KITTY_DYN])
def test_kitty_pro_boosts_a_quarter_of_the_channels(scheme):
    # Kitty-Pro reading: alpha = 1/4, 32 of 128 key channels at 4 bits
    rng = np.random.default_rng(16)
    K = f16(rng.standard_normal((700, D)) * rng.uniform(0.1, 6, D))
    V = f16(rng.standard_normal((700, D)))
    idx = O.kitty_select(K[:512], 32) if scheme == O.KITTY else None
    if idx is not None:
        assert np.array_equal(idx, brute_select_amax(K[:512], 32))
    s = O.Stream(scheme, 1024, nb=32, idx=idx, sel=64)
    s.prefill(K, V)
    l, n_kq, _ = s.state
    codes = s.key_codes()[:n_kq]
    for p in range(n_kq // 64):
        pidx = idx if scheme == O.KITTY else s.unit_index()[p]
        if scheme == O.KITTY_DYN:
            assert np.array_equal(pidx, brute_select(K[64 * p:64 * p + 64], 32))
        boosted = pidx < 32
        assert boosted.sum() == 32
        page = codes[64 * p:64 * p + 64]
        assert page[:, ~boosted].max() <= 3 and page[:, boosted].max() > 3
    Kt, _ = s.dequant(0, n_kq)
    ks, _ = s.key_stats()
    step = f32(ks[: n_kq // 32]).repeat(32, axis=0).astype(np.float64)
    err = np.abs(f32(K[:n_kq]).astype(np.float64) - Kt)
    assert np.all(err <= step / 2 * (1 + 2.0 ** -20) + 1e-30)
