"""The algorithmic byte accounts that bench.py divides by the measured time
(host only).  The per-token figures must match the page layout the library
reports, the window terms must match a hand count of what a decode step
reads, and the per-launch figures recorded next to the rocprofv3 traffic
counters must be the ones the accounting gives at bench.py's default
warm-up and step counts."""
import json
import os

import numpy as np
import pytest

import bench
from bit_kv_cache_kivi_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def K():
    from bit_kv_cache_kivi_amd import kvq
    if not os.path.exists(kvq.LIB_PATH):
        from bit_kv_cache_kivi_amd import build
        build.build()
    kvq.lib()
    return kvq


@pytest.mark.parametrize("scheme,nb", [("kivi2", 16), ("kivi4", 16), ("kitty", 16), ("kitty", 32),
                                       ("kitty_dyn", 16), ("kitty_dyn", 32)])
def test_paged_bytes_are_the_layouts_pages(K, scheme, nb):
    # a paged prefix of whole 64-token pages costs exactly its pages' bytes
    L = K.make_layout(scheme, B=1, Hq=1, Hkv=1, max_pages=1, n_pages=1,
                      nb=nb if scheme.startswith("kitty") else None)
    for pages in (1, 3, 17):
        n = 64 * pages
        got = bench.key_q_bytes(scheme, n, nb) + n * bench.value_q_bytes(scheme)
        assert got == pages * K.page_bytes(L)


@pytest.mark.parametrize("nb", [0, 4])
def test_witcert_paged_bytes_are_the_layouts_tokens(K, nb):
    L = K.make_layout("witcert_paged", B=1, Hq=1, Hkv=1, max_pages=1, n_pages=1, nb=nb)
    for l in (1, 64, 1000):
        assert bench.witcert_paged_bytes(l, 4, nb)["stage1"] == l * K.bytes_per_token(L)


def test_kivi_window_terms_by_hand():
    # l = 1000, R = 128: values quantized below 872, keys below 896 (the key
    # residual holds 104 tokens).  Stage 1 reads 872 tokens x 96 B of pages,
    # the keys of tokens 872..895 quantized (48 B each), the fp16 keys of
    # 896..999 and the fp16 values of 872..999 (256 B each)
    l, n_kq, R = 1000, 896, 128
    d = bench.kivi_bytes(l, n_kq, R, 4, "kivi2")
    assert d["stage1"] == 872 * 96 + 24 * 48 + 104 * 256 + 128 * 256
    # the decode adds four fp16 queries, four fp32 output rows and the page
    # table row (16 entries of 4 B)
    assert d["decode"] == d["stage1"] + 4 * (256 + 512) + 16 * 4
    # 32 sink tokens: fp16 keys and values, the quantized positions start
    # after them
    d = bench.kivi_bytes(l, n_kq, R, 1, "kivi2", sink=32)
    n_vq = l - 32 - R
    assert d["stage1"] == (n_vq * 96 + (n_kq - 32 - n_vq) * 48 + (l - n_kq) * 256
                           + (l - 32 - n_vq) * 256 + 32 * 512)


def _stage1_mean(w, warmup=5, steps=50, every=4):
    # the mean over the timed steps whose stage-1 launch the HIP events
    # bracket (every `every`-th, bench.event_steps), as the bench line records
    sampled = set(bench.event_steps(steps, every))
    states = [bench.state_after_prefill(w, l) for l in w.ctx]
    for _ in range(warmup):
        _, _, states = bench.step_bytes(w, states)
    s1 = []
    for j in range(steps):
        _, b, states = bench.step_bytes(w, states)
        if j in sampled:
            s1.append(b)
    return int(np.mean(s1))


def test_recorded_per_launch_bytes_match_the_accounting():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)
    names = {inputs.workload(i).name: i for i in range(1, 12)}
    assert rec
    for key, e in rec.items():
        wname = key.split("@")[1]
        w = inputs.workload(names[wname])
        assert e["algorithmic_bytes_per_launch"] == _stage1_mean(w), key
