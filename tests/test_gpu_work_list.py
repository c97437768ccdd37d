"""The group kernel's stage-1 work list, read back from the workspace after a
decode and compared item by item (bit-exact) with the list built on the host
from its definition: per (request, KV head) pair of npg quantized pages, body
splits of sp pages over all but the last min(npg / 8, 2 sp) pages, then tail
splits of sp / 4 pages, the last one shorter; the list holds every body
split, then every full tail split, each in (pair, split) order, then the
short splits by length, longest first, each length in pair order.  An item is
{pair, partial row, first page, pages | valid tokens of the pair's last page
<< 8 when it ends the pair}; a group of 8 runs both query quads of an item in
one workgroup."""
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


def _tail_pages(sp):
    return sp // 4 if sp >= 4 else 1


def _split_counts(npg, sp):
    tt = min(npg // 8, 2 * sp)
    nb = (npg - tt) // sp
    rest = npg - nb * sp
    tp = _tail_pages(sp)
    return nb, rest // tp, rest % tp


def _max_splits(max_pages, sp):
    tt = min(max_pages // 8, 2 * sp)
    tp = _tail_pages(sp)
    return (max_pages - tt) // sp + (tt + sp - 1 + tp - 1) // tp


def _expected(lengths, Hkv, sp, R, sink, max_pages):
    tp = _tail_pages(sp)
    body, tail, short = [], [], {n: [] for n in range(1, tp)}
    for b, row in enumerate(lengths):
        for h in range(Hkv):
            nvq = max(0, int(row[h]) - sink - R)
            npg = min((nvq + PT - 1) // PT, max_pages)
            last = min(PT, nvq - (npg - 1) * PT) if npg else 0
            nb, nt, rem = _split_counts(npg, sp)
            pr = b * Hkv + h

            def item(r, p0, n):
                return (pr, r, p0, n | ((last << 8) if p0 + n == npg else 0))
            body += [item(k, k * sp, sp) for k in range(nb)]
            tail += [item(nb + k, nb * sp + k * tp, tp) for k in range(nt)]
            if rem:
                short[rem].append(item(nb + nt, nb * sp + nt * tp, rem))
    out = body + tail
    for n in range(tp - 1, 0, -1):
        out += short[n]
    return np.array(out, dtype=np.uint32).reshape(-1, 4)


@pytest.mark.parametrize("B,Hq,Hkv,split,sink,cmax", [
    (12, 8, 2, 8, 0, 4100),       # one row of pairs, one short length
    (12, 16, 2, 48, 0, 9000),     # a group of 8, eleven short lengths
    (11, 4, 2, 12, 32, 3000),     # group of 2 (one quad), sink tokens
    (260, 16, 4, 8, 0, 1400),     # 1040 pairs: 17 rows, more than one batch of counts
    (520, 32, 8, 16, 0, 900),     # 4160 pairs: 65 rows, two rows for some workgroups
])
def test_gqa4_work_list_exact(B, Hq, Hkv, split, sink, cmax):
    import torch
    from bit_kv_cache_kivi_amd import kvq
    R = 128
    rng = np.random.default_rng(B * 1000 + split)
    edge = [1, R + sink, R + sink + 1, R + sink + PT, R + sink + PT + 1, cmax]
    ctx = np.concatenate([edge, rng.integers(1, cmax + 1, size=B)])[:B].astype(np.int32)
    max_pages = (int(ctx.max()) + 16 + PT - 1) // PT
    n_pages = B * max_pages
    table = rng.permutation(n_pages).astype(np.int32).reshape(B, max_pages)
    layout = kvq.make_layout("kivi2", B, Hq, Hkv, max_pages, n_pages, R=R, seed=0x5EED, split_pages=split,
                             sink=sink)
    cache = kvq.KVCache(layout, table)
    assert cache.cache.split_pages == split
    ld = int(ctx.max())
    print(f"work list case B={B} Hq={Hq} Hkv={Hkv} split={split} sink={sink}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(B)
    K = torch.randn((B, Hkv, ld, 128), generator=g, device="cuda").to(torch.float16)
    V = torch.randn((B, Hkv, ld, 128), generator=g, device="cuda").to(torch.float16)
    cache.prefill(0, K, V, torch.from_numpy(ctx).cuda())
    del K, V
    q = torch.randn((B, Hq, 128), generator=g, device="cuda").to(torch.float16)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
    cache.decode(q, out)
    torch.cuda.synchronize()
    assert cache.status_word() == 0
    assert torch.isfinite(out).all()
    state = cache.state.cpu().numpy()
    assert np.array_equal(state[:, :, 0], np.repeat(ctx[:, None], Hkv, 1))

    ms = _max_splits(max_pages, split)
    n_win = R // PT + (1 if sink else 0)
    rows = B * Hq * (ms + n_win)
    cap = B * Hkv * ms
    assert cache.ws_bytes == rows * 128 * 4 + rows * 8 + cap * 16 + 256
    ws = cache.workspace.cpu().numpy()
    off = rows * 128 * 4 + rows * 8
    items = ws[off:off + cap * 16].view(np.uint32).reshape(cap, 4)
    n_items = int(ws[off + cap * 16:off + cap * 16 + 4].view(np.uint32)[0])
    exp = _expected(state[:, :, 0], Hkv, split, R, sink, max_pages)
    assert n_items == len(exp)
    bad = np.nonzero((items[:n_items] != exp).any(1))[0]
    assert bad.size == 0, (bad[:5], items[bad[:5]], exp[bad[:5]])
