"""Pins of the oracle's KIVI-4 scheme (the KIVI quantizer at 4 bits for keys
and values; "KIVI" explainer, the 2- and 4-bit variants).  Pins: keys equal
Kitty with every channel boosted (the 4-bit branch of the same quantizer);
values are 16-level per token and group, each within half its step; a
constant group gives code 0 and the exact value; streaming equals bulk
prefill; 4 bits are at least as accurate as 2 bits on every element's
group step."""
import numpy as np

from oracle import oracle as O

D = 128


def f16(x):
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def f32(h):
    return np.asarray(h, np.uint16).view(np.float16).astype(np.float32)


def kv(seed, n):
    rng = np.random.default_rng(seed)
    K = f16(rng.standard_normal((n, D)) * rng.uniform(0.1, 8, D))
    V = f16(rng.standard_normal((n, D)) * 3)
    return K, V


def test_keys_equal_kitty_with_every_channel_boosted():
    K, V = kv(31, 800)
    a = O.Stream(O.KIVI4, 1024)
    b = O.Stream(O.KITTY, 1024, nb=128, idx=np.arange(D, dtype=np.uint8))
    a.prefill(K, V)
    b.prefill(K, V)
    assert a.state == b.state
    assert np.array_equal(a.key_codes(), b.key_codes())
    assert all(np.array_equal(x, y) for x, y in zip(a.key_stats(), b.key_stats()))


def test_values_sixteen_levels_within_half_step():
    K, V = kv(32, 900)
    s = O.Stream(O.KIVI4, 1024)
    s.prefill(K, V)
    l, n_kq, n_vq = s.state
    vc = s.value_codes()[:n_vq]
    assert vc.max() == 15 and vc.min() == 0
    _, Vt = s.dequant(0, n_vq)
    vs, _ = s.value_stats()
    step = f32(vs[:n_vq]).repeat(32, axis=1).astype(np.float64)
    err = np.abs(f32(V[:n_vq]).astype(np.float64) - Vt)
    assert np.all(err <= step / 2 * (1 + 2.0 ** -20) + 1e-30)
    # the 4-bit step is the 2-bit step over 5 (15 levels vs 3 over the same range)
    t = O.Stream(O.KIVI, 1024)
    t.prefill(K, V)
    vs2, _ = t.value_stats()
    r = f32(vs2[:n_vq]).astype(np.float64) / np.maximum(f32(vs[:n_vq]).astype(np.float64), 1e-30)
    assert np.all(np.abs(r - 5.0) < 0.01)


def test_constant_group_is_exact():
    K = np.full((300, D), f16(1.25), np.uint16)
    V = np.full((300, D), f16(-0.5), np.uint16)
    s = O.Stream(O.KIVI4, 512)
    s.prefill(K, V)
    l, n_kq, n_vq = s.state
    Kt, Vt = s.dequant(0, l)
    assert np.all(Kt == 1.25) and np.all(Vt == -0.5)
    assert s.key_codes()[:n_kq].max() == 0 and s.value_codes()[:n_vq].max() == 0


def test_streaming_equals_bulk():
    K, V = kv(33, 520)
    a = O.Stream(O.KIVI4, 1024)
    a.prefill(K[:300], V[:300])
    for t in range(300, 520):
        a.flush()
        assert a.append(K[t], V[t]) == 0
    b = O.Stream(O.KIVI4, 1024)
    b.prefill(K, V)
    assert a.state == b.state
    assert np.array_equal(a.key_codes(), b.key_codes())
    assert np.array_equal(a.value_codes(), b.value_codes())
    assert all(np.array_equal(x, y) for x, y in zip(a.key_stats() + a.value_stats(),
                                                     b.key_stats() + b.value_stats()))
