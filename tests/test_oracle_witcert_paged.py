"""Pins of the oracle's paging-safe WitCert storage (scheme WITCERT_TOK).

WitCert page, certified-deployment paragraphs:
* every token is quantized when written, one scale per (token, group of
  G_c = 32 channels), s = amax/126.5 over the group stored fp16 and reused
  (same rule as the block scheme): |x - x_hat| <= s/2, no clipping;
* the fixed outlier RoPE pairs are kept fp16 and left out of their group's
  amax: a huge bypassed channel does not raise the other channels' scale;
* the dither is keyed by the cache slot (layer, KV head, slot, channel):
  a token's record depends on its values and its slot only, so requests that
  share a prefix in the same slots share its records bit for bit, whatever
  the request id or what follows;
* byte account: 136 B per token and side at G_c = 32, + 16 B for m = 4 pairs
  (tests/golden/witcert_paged.json);
* certificate: bypassed channels carry no error; a single token gives the
  closed form A = e^u; kappa = 0 gives A = 1.
The pair selection (top m by the pair's largest squared norm over the
calibration tokens, ties to the lower pair) is checked against a numpy brute
force, a planted outlier pair, and swap/negation invariance within a pair.
"""
import json
import os

import numpy as np
import pytest
from scipy import stats

HERE = os.path.dirname(__file__)
GOLD = os.path.join(HERE, "golden")
D = 128
SM = float(np.float32(1.0 / np.sqrt(128)))


def f16(x):
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def f32(h):
    return np.asarray(h, np.uint16).view(np.float16).astype(np.float32)


def gold():
    with open(os.path.join(GOLD, "witcert_paged.json")) as f:
        return json.load(f)


def _tokens(seed, n, pairs=(), factor=50.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, D)).astype(np.float32)
    for i in pairs:
        x[:, i] *= np.float32(factor)
        x[:, i + D // 2] *= np.float32(factor)
    return f16(x)


def _mask(pairs):
    m = np.zeros(D, np.uint8)
    for i in pairs:
        m[i] = m[i + D // 2] = 1
    return m


def _stream(O, n, mask=None, slots=None, seed=7, req=0, kvh=3, layer=2):
    return O.Stream(O.WITCERT_TOK, n, VG=gold()["G_c"], idx=mask, seed=seed, req=req,
                    layer=layer, kvh=kvh, slots=slots)


def test_byte_account_matches_the_page():
    g = gold()
    per_side = D + 2 * (D // g["G_c"])        # int8 codes + fp16 scales per group
    assert per_side == g["bytes_per_token_per_side"]
    assert 2 * per_side == g["bytes_per_token_kv"]
    assert 2 * g["m"] * 2 == g["bypass_bytes"]  # 2m fp16 values


def test_half_step_bound_no_clipping_and_exact_bypass(O):
    pairs = (5, 17, 40, 63)
    mask = _mask(pairs)
    K = _tokens(1, 300, pairs)
    V = _tokens(2, 300)
    s = _stream(O, 300, mask)
    s.prefill(K, V)
    assert s.state == (300, 300, 300)
    Kt, Vt = s.dequant()
    ks, _ = s.key_stats()
    vs, _ = s.value_stats()
    kc = s.key_codes().view(np.int8)
    vc = s.value_codes().view(np.int8)
    for side, raw, got, sc, codes in ((0, K, Kt, ks, kc), (1, V, Vt, vs, vc)):
        xv = f32(raw).astype(np.float64)
        step = np.repeat(f32(sc).astype(np.float64), 32, axis=1)
        quant = np.ones(D, bool) if side else mask == 0
        err = np.abs(xv - got.astype(np.float64))[:, quant]
        assert np.all(err <= step[:, quant] / 2 * (1 + 2.0 ** -20) + 2.0 ** -30)
        assert np.abs(codes[:, quant]).max() <= 127
        # s = amax / 126.5 over the group's quantized channels, fp16
        for g in range(4):
            cols = [c for c in range(32 * g, 32 * g + 32) if quant[c]]
            amax = np.abs(f32(raw)[:, cols]).max(axis=1)
            assert np.array_equal(sc[:, g], f16(amax / np.float32(126.5)))
    # bypassed keys come back exactly; their codes are 0; values have no bypass
    assert np.array_equal(Kt[:, mask == 1], f32(K)[:, mask == 1])
    assert np.all(kc[:, mask == 1] == 0)
    assert np.any(Vt[:, mask == 1] != f32(V)[:, mask == 1])


def test_bypassed_channel_left_out_of_the_amax(O):
    # worked example: one group holds a bypassed channel at 1000 and others
    # whose largest magnitude is exactly 1; the group's step follows the 1
    x = np.full((1, D), 0.25, np.float32)
    x[0, 3] = -1.0
    x[0, 10] = 1000.0
    x[0, 10 + D // 2] = 0.5
    K = f16(x)
    with_b = _stream(O, 1, _mask((10,)))
    with_b.prefill(K, K)
    without = _stream(O, 1, None)
    without.prefill(K, K)
    div = np.float32(126.5)
    assert with_b.key_stats()[0][0, 0] == f16(np.float32(1.0) / div)
    assert without.key_stats()[0][0, 0] == f16(np.float32(1000.0) / div)
    assert with_b.value_stats()[0][0, 0] == f16(np.float32(1000.0) / div)   # values: no bypass


def test_record_depends_on_values_and_slot_only(O):
    # two requests share a 150-token prefix in the same slots; their suffixes
    # and slots differ.  The prefix records agree bit for bit.
    P, n = 150, 260
    pre = _tokens(3, P)
    Ka = np.concatenate([pre, _tokens(4, n - P)])
    Kb = np.concatenate([pre, _tokens(5, n - P)])
    slots_a = np.arange(n, dtype=np.uint64) + 1000
    slots_b = slots_a.copy()
    slots_b[P:] += 5000
    a = _stream(O, n, slots=slots_a, req=0)
    b = _stream(O, n, slots=slots_b, req=9)
    a.prefill(Ka, Ka)
    b.prefill(Kb, Kb)
    for get in ("key_codes", "value_codes"):
        assert np.array_equal(getattr(a, get)()[:P], getattr(b, get)()[:P])
    assert np.array_equal(a.key_stats()[0][:P], b.key_stats()[0][:P])
    # one token alone, written to the same slot, gets the same record
    t = 77
    one = _stream(O, 1, slots=slots_a[t:t + 1])
    one.prefill(Ka[t:t + 1], Ka[t:t + 1])
    assert np.array_equal(one.key_codes()[0], a.key_codes()[t])
    assert np.array_equal(one.value_codes()[0], a.value_codes()[t])
    # the same tokens in other slots get another dither
    c = _stream(O, n, slots=slots_a + 64)
    c.prefill(Ka, Ka)
    assert not np.array_equal(c.key_codes(), a.key_codes())
    assert np.array_equal(c.key_stats()[0], a.key_stats()[0])     # scales: values only


def test_slot_dither_uniform_and_word_layout(O):
    xs = np.array([O.dither_slot(11, side, 2, 3, slot, ch)
                   for side in (0, 1) for slot in range(0, 40000, 97) for ch in range(0, 128, 9)])
    assert abs(xs.mean()) < 0.01 and abs(xs.var() - 1 / 12) < 0.003
    assert stats.kstest(xs + 0.5, "uniform").pvalue > 1e-3
    # the four channels of a quad read the four words of one Philox block
    # whose counter is (slot_lo, quad, (layer << 16) | kv_head, slot_hi)
    slot = (5 << 32) | 123
    out = O.philox([123, 7, (2 << 16) | 3, 5], [11, 0])
    for w in range(4):
        want = np.float32(int(out[w]) >> 8) * np.float32(2.0 ** -24) - np.float32(0.5)
        assert O.dither_slot(11, 0, 2, 3, slot, 28 + w) == want


def test_streaming_equals_bulk(O):
    mask = _mask((1, 33))
    K, V = _tokens(6, 200, (1, 33)), _tokens(7, 200)
    slots = np.random.default_rng(0).permutation(4096)[:200].astype(np.uint64)
    bulk = _stream(O, 200, mask, slots)
    bulk.prefill(K, V)
    st = _stream(O, 200, mask, slots)
    st.prefill(K[:50], V[:50])
    for t in range(50, 200):
        assert not st.flush()                   # nothing waits for a flush
        assert st.append(K[t], V[t]) == 0
    assert st.state == bulk.state == (200, 200, 200)
    for get in ("key_codes", "value_codes"):
        assert np.array_equal(getattr(st, get)(), getattr(bulk, get)())
    assert np.array_equal(st.key_stats()[0], bulk.key_stats()[0])
    assert np.array_equal(st.value_stats()[0], bulk.value_stats()[0])


def test_certificate_closed_forms(O):
    mask = _mask((2, 9))
    K, V = _tokens(8, 1, (2, 9)), _tokens(9, 1)
    s = _stream(O, 1, mask)
    s.prefill(K, V)
    q = f16(np.random.default_rng(1).standard_normal((3, D)))
    kappa = float(np.float32(1.7))          # crosses the ABI as binary32
    _, cert = s.decode(q, SM, kappa)
    sc = np.repeat(f32(s.key_stats()[0][0]).astype(np.float64), 32)
    sc[mask == 1] = 0.0
    qf = f32(q).astype(np.float64)
    u = kappa * np.sqrt(SM * SM / 12.0 * (qf * qf * sc * sc).sum(axis=1))
    np.testing.assert_allclose(cert, np.exp(u), rtol=1e-12)
    # a query on bypassed channels only sees no quantization noise: A = 1
    s2 = _stream(O, 40, mask)
    s2.prefill(_tokens(10, 40, (2, 9)), _tokens(11, 40))
    qb = np.zeros((1, D), np.float32)
    qb[0, mask == 1] = 1.0
    _, c1 = s2.decode(f16(qb), SM, 3.0)
    assert c1[0] == 1.0
    _, c0 = s2.decode(q, SM, 0.0)
    assert np.all(c0 == 1.0)


def _imp_numpy(k):
    x = f32(k)
    a, b = x[:, :D // 2], x[:, D // 2:]
    e = (a * a + b * b).astype(np.float32)
    return e.max(axis=0)


@pytest.mark.parametrize("seed", range(6))
def test_pair_selection_brute_force(O, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((64, D)).astype(np.float32)
    if seed % 2:
        x = np.round(x * 2) / 2                 # many ties
    k = f16(x)
    imp = _imp_numpy(k)
    order = np.lexsort((np.arange(D // 2), -imp))
    want = _mask(order[:4])
    assert np.array_equal(O.witcert_select_pairs(k, 4), want)


def test_pair_selection_outlier_and_invariance(O):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((100, D)).astype(np.float32)
    x[40, 21] = 300.0                           # one massive activation in pair 21
    k = f16(x)
    m = O.witcert_select_pairs(k, 4)
    assert m[21] == 1 and m[21 + D // 2] == 1 and m.sum() == 8
    # swapping or negating the two channels of every pair keeps the choice
    xs = np.concatenate([x[:, D // 2:], -x[:, :D // 2]], axis=1)
    assert np.array_equal(O.witcert_select_pairs(f16(xs), 4), m)
