"""Pins of the oracle's sink tokens (Kitty summary: the first tokens of a
sequence kept in full precision, keys and values alike).

Reading taken: the first S tokens stay fp16 for keys and values; key groups,
Kitty selection units and the value FIFO start at token S.  Pins: sink
tokens dequantize to their exact fp16 values; the quantized record after the
sink equals an ordinary stream fed the tokens after the sink (so the scheme
is "fp16 sink + unchanged method"); attention equals torch float64 attention
over [sink fp16 ; that stream's dequantized tensors]; streaming equals bulk
prefill for lengths below, at and past the sink; the first flush comes R
tokens after the sink; WitCert takes no sink.
"""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as O

D = 128
S = 32
SM = float(np.float32(1 / math.sqrt(D)))


def f16(x):
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def f32(h):
    return np.asarray(h, np.uint16).view(np.float16).astype(np.float32)


def kv(seed, n):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((n, D)).astype(np.float32) * rng.uniform(0.2, 6, D).astype(np.float32)
    V = rng.standard_normal((n, D)).astype(np.float32)
    return f16(K), f16(V)


@pytest.mark.parametrize("scheme", [O.KIVI, O.KITTY, O.KITTY_DYN])
def test_sink_plus_ordinary_stream(scheme):
    n = 700
    K, V = kv(21, n)
    idx = O.kitty_select(K[:256], 16) if scheme == O.KITTY else None
    nb = 16 if scheme != O.KIVI else 0
    a = O.Stream(scheme, 1024, nb=nb, idx=idx, sink=S)
    a.prefill(K, V)
    b = O.Stream(scheme, 1024, nb=nb, idx=idx)            # the tokens after the sink
    b.prefill(K[S:], V[S:])
    la, ka, va = a.state
    lb, kb, vb = b.state
    assert (la - S, ka - S, va - S) == (lb, kb, vb)
    Ka, Va = a.dequant(0, la)
    Kb, Vb = b.dequant(0, lb)
    assert np.array_equal(Ka[:S], f32(K[:S])) and np.array_equal(Va[:S], f32(V[:S]))
    assert np.array_equal(Ka[S:], Kb) and np.array_equal(Va[S:], Vb)
    assert np.array_equal(a.key_codes()[S:la], b.key_codes()[:lb])
    assert np.array_equal(a.value_codes()[S:la], b.value_codes()[:lb])
    assert all(np.array_equal(x, y) for x, y in zip(a.key_stats(), b.key_stats()))
    if scheme == O.KITTY_DYN:
        assert np.array_equal(a.unit_index(), b.unit_index())


def test_attention_over_sink_and_dequantized_rest_matches_torch():
    n = 650
    K, V = kv(22, n)
    s = O.Stream(O.KIVI, 1024, sink=S)
    s.prefill(K, V)
    q = f16(np.random.default_rng(23).standard_normal((4, D)))
    out, _ = s.decode(q, SM)
    Kt, Vt = s.dequant(0, n)
    assert np.array_equal(Kt[:S], f32(K[:S]))
    qt = torch.tensor(f32(q), dtype=torch.float64)
    p = torch.softmax(SM * (qt @ torch.tensor(Kt, dtype=torch.float64).T), dim=-1)
    ref = (p @ torch.tensor(Vt, dtype=torch.float64)).numpy()
    assert np.abs(out - ref).max() < 1e-12


@pytest.mark.parametrize("n0", [0, 1, 31, 32, 33, 100, 160, 161, 300])
def test_streaming_equals_bulk_with_sink(n0):
    extra = 300
    K, V = kv(24, n0 + extra)
    a = O.Stream(O.KIVI, 1024, sink=S)
    a.prefill(K[:n0], V[:n0])
    flushes = []
    for t in range(n0, n0 + extra):
        if a.flush():
            flushes.append(t)
        assert a.append(K[t], V[t]) == 0
    b = O.Stream(O.KIVI, 1024, sink=S)
    b.prefill(K, V)
    assert a.state == b.state
    assert np.array_equal(a.key_codes(), b.key_codes())
    assert np.array_equal(a.value_codes(), b.value_codes())
    assert all(np.array_equal(x, y) for x, y in zip(a.key_stats() + a.value_stats(),
                                                     b.key_stats() + b.value_stats()))
    # a flush happens exactly when R keys after the sink have gathered
    assert all((t - S) % 128 == 0 and t > S for t in flushes)


def test_state_inside_the_sink():
    K, V = kv(25, 40)
    s = O.Stream(O.KIVI, 256, sink=S)
    for t in range(40):
        assert not s.flush()
        s.append(K[t], V[t])
        l, n_kq, n_vq = s.state
        if t < S:
            assert (l, n_kq, n_vq) == (t + 1, t + 1, t + 1)   # nothing pending
        else:
            assert (n_kq, n_vq) == (S, S)                     # residual and FIFO hold the rest
    Kt, Vt = s.dequant()
    assert np.array_equal(Kt, f32(K)) and np.array_equal(Vt, f32(V))


def test_witcert_takes_no_sink():
    with pytest.raises(ValueError):
        O.Stream(O.WITCERT, 1024, sink=S)
