"""kvq_stage1_load_floor, the group kernel's load-only copy (a measurement
aid): it runs the work-list plan and stage 1 with the page step's arithmetic
taken out, writes only the workspace, and leaves the cache as it was -- the
state is unchanged and a decode after it gives the same output bit for bit.
It writes every partial row of the paged splits that a decode writes (folded
words, finite, weight slot 1); the work list it plans is the decode's."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

PT = 64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_kv_cache_kivi_amd import kvq
    kvq.lib()


@pytest.mark.parametrize("B,Hq,Hkv,split,sink", [
    (6, 8, 2, 8, 0),              # group of 4
    (5, 4, 2, 12, 32),            # group of 2 (one quad), sink tokens
    (4, 16, 2, 8, 0),             # group of 8: two waves per workgroup
])
def test_load_floor_leaves_the_cache_and_decode_unchanged(B, Hq, Hkv, split, sink):
    import torch
    from bit_kv_cache_kivi_amd import kvq
    R = 128
    rng = np.random.default_rng(B * 100 + Hq)
    ctx = np.concatenate([[1, R + sink + 1], rng.integers(200, 3000, size=B)])[:B].astype(np.int32)
    max_pages = (int(ctx.max()) + PT - 1) // PT + 1
    n_pages = B * max_pages
    table = rng.permutation(n_pages).astype(np.int32).reshape(B, max_pages)
    layout = kvq.make_layout("kivi2", B, Hq, Hkv, max_pages, n_pages, R=R, seed=0x5EED,
                             split_pages=split, sink=sink)
    cache = kvq.KVCache(layout, table)
    print(f"load floor case B={B} Hq={Hq} Hkv={Hkv} split={split} sink={sink}", flush=True)
    ld = int(ctx.max())
    g = torch.Generator(device="cuda").manual_seed(B + Hq)
    K = torch.randn((B, Hkv, ld, 128), generator=g, device="cuda").to(torch.float16)
    V = torch.randn((B, Hkv, ld, 128), generator=g, device="cuda").to(torch.float16)
    cache.prefill(0, K, V, torch.from_numpy(ctx).cuda())
    del K, V
    q = torch.randn((B, Hq, 128), generator=g, device="cuda").to(torch.float16)
    out1 = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
    out2 = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    cache.decode(q, out1)
    torch.cuda.synchronize()
    ws_decode = cache.workspace.cpu().numpy().copy()
    state0 = cache.state.cpu().numpy().copy()
    pool0 = cache.pool.clone()

    cache.stage1_load_floor(q)
    cache.stage1_load_floor(q)
    torch.cuda.synchronize()
    assert cache.status_word() == 0
    assert np.array_equal(cache.state.cpu().numpy(), state0)
    assert torch.equal(cache.pool, pool0)

    # the workspace: the same work list, and on every paged row the decode
    # wrote, one folded value (finite) and the weight slot 1
    ws = cache.workspace.cpu().numpy()
    n_win = R // PT + (1 if sink else 0)
    total = cache.ws_bytes - 256
    # rows = B Hq (ms + n_win); bytes = rows (512 + 8) + B Hkv ms 16
    ms = (total // B - Hq * n_win * 520) // (Hq * 520 + Hkv * 16)
    rows = B * Hq * (ms + n_win)
    assert rows * 520 + B * Hkv * ms * 16 + 256 == cache.ws_bytes
    off = rows * 520
    assert np.array_equal(ws[off:], ws_decode[off:])          # work list and its length
    items = ws[off:off + B * Hkv * ms * 16].view(np.uint32).reshape(-1, 4)
    n_items = int(ws[off + B * Hkv * ms * 16:][:4].view(np.uint32)[0])
    o = ws[:rows * 512].view(np.float32).reshape(B, Hq, ms + n_win, 128)
    ml = ws[rows * 512:rows * 520].view(np.float32).reshape(B, Hq, ms + n_win, 2)
    qpk = Hq // Hkv
    for pr, r, _, _ in items[:n_items]:
        b, h = divmod(int(pr), Hkv)
        for hq in range(h * qpk, (h + 1) * qpk):
            row = o[b, hq, r]
            assert np.isfinite(row).all() and np.isfinite(ml[b, hq, r, 0]), (b, hq, r)
            assert ml[b, hq, r, 1] == 1.0, (b, hq, r)

    cache.decode(q, out2)
    torch.cuda.synchronize()
    assert cache.status_word() == 0
    assert torch.equal(out1, out2)
