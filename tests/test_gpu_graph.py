"""One decode step (flush -> append -> decode through the C ABI) captured in
a HIP graph and replayed: every replay advances the cache exactly as the
same step run eagerly on a twin cache does (outputs, certificate and the
whole pool bit for bit).  The library allocates, frees and synchronizes
nothing and records no memset, so the captured step needs no setup of its
own.  Eager work and host synchronizations run between the replays."""
import numpy as np
import pytest

from bit_kv_cache_kivi_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_kv_cache_kivi_amd import kvq
    kvq.lib()


def _cache(w, max_pages):
    import torch
    from bit_kv_cache_kivi_amd import kvq
    table = inputs.page_permutation(w, w.B * max_pages).reshape(w.B, max_pages)
    layout = kvq.make_layout(w.scheme, w.B, w.Hq, w.Hkv, max_pages, w.B * max_pages, R=w.R,
                             seed=0x5EED_0000_0000_0000 | w.seed, split_pages=3,
                             nb=w.nb if (w.nb or w.scheme == "witcert_paged") else None)
    cache = kvq.KVCache(layout, table, poison=True)
    if w.scheme == "kitty" or (w.scheme == "witcert_paged" and w.nb):
        calib = torch.from_numpy(np.stack([inputs.kitty_calibration(w, h)
                                           for h in range(w.Hkv)]).view(np.float16)).cuda()
        if w.scheme == "kitty":
            cache.kitty_calibrate(calib)
        else:
            cache.witcert_calibrate(calib)
    for b in range(w.B):
        K = np.stack([inputs.context_kv(w, b, h)[0] for h in range(w.Hkv)])[None]
        V = np.stack([inputs.context_kv(w, b, h)[1] for h in range(w.Hkv)])[None]
        cache.prefill(b, torch.from_numpy(K.view(np.float16)).cuda(),
                      torch.from_numpy(V.view(np.float16)).cuda(),
                      torch.tensor([w.ctx[b]], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    return cache


@pytest.mark.parametrize("wid", [3, 4, 10])
def test_captured_step_replays_like_eager(wid):
    import torch
    # key residuals of 127 and 128 tokens after the prefill: the replays
    # include flushes that quantize a whole residual
    w = inputs.workload(wid, B=2, Hq=8, Hkv=2, ctx=(767, 1024))
    graph_cache, eager_cache = _cache(w, 20), _cache(w, 20)
    k, v = inputs.step_kv(w, 0)
    q = inputs.step_q(w, 0)
    kt = torch.from_numpy(k.view(np.float16)).cuda()
    vt = torch.from_numpy(v.view(np.float16)).cuda()
    qt = torch.from_numpy(q.view(np.float16)).cuda()
    kappa = 1.0 if w.scheme.startswith("witcert") else 0.0
    outs = [torch.zeros((w.B, w.Hq, 128), dtype=torch.float32, device="cuda") for _ in range(2)]
    certs = [torch.zeros((w.B, w.Hq), dtype=torch.float32, device="cuda") for _ in range(2)]

    def step(cache, i):
        cache.flush()
        cache.append(kt, vt)
        cache.decode(qt, outs[i], certs[i], sm_scale=w.sm_scale, kappa=kappa)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(graph_cache, 0)
    torch.cuda.synchronize()
    # capturing runs nothing: both caches still hold the prefill state
    assert torch.equal(graph_cache.state, eager_cache.state)
    for r in range(5):
        graph.replay()
        step(eager_cache, 1)                    # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1]), ("output", r)
        assert torch.equal(certs[0], certs[1]), ("certificate", r)
        assert torch.equal(graph_cache.state, eager_cache.state), ("state", r)
    assert torch.equal(graph_cache.pool, eager_cache.pool)
    assert graph_cache.status_word() == 0 and eager_cache.status_word() == 0
