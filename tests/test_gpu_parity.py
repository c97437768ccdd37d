"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Codes, statistics, fp16 windows and state: bit-exact.  Attention output:
max |delta o| <= 1e-5 absolute; certificate: relative 1e-5 (+inf equal).
Pools are filled with 0xFF (NaN statistics) so a read of unwritten memory
poisons the output."""
import numpy as np
import pytest

from bit_kv_cache_kivi_amd import inputs

pytestmark = pytest.mark.gpu

TOL_O = 1e-5
TOL_CERT = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_kv_cache_kivi_amd import kvq
    kvq.lib()          # the HIP library must load: no fallback


def _case(*a, **k):
    from gpu_harness import Case
    return Case(*a, **k)


def _check_decode(case, out, cert, q, kappa=0.0, cert_check=False):
    w = case.w
    g = w.group
    o = out.cpu().numpy()
    c = cert.cpu().numpy()
    worst = 0.0
    for (b, h) in case.streams:
        ref, rc = case.oracle_decode(q, b, h, kappa)
        got = o[b, h * g:(h + 1) * g]
        assert np.all(np.isfinite(got)), (b, h)
        err = np.abs(got.astype(np.float64) - ref).max()
        worst = max(worst, err)
        assert err <= TOL_O, (b, h, err)
        if cert_check:
            gc = c[b, h * g:(h + 1) * g].astype(np.float64)
            both_inf = np.isinf(gc) & np.isinf(rc)
            rel = np.abs(gc - rc) / np.maximum(np.abs(rc), 1e-30)
            assert np.all(both_inf | (rel <= TOL_CERT)), (b, h, gc, rc)
    return worst


@pytest.mark.parametrize("Hq,Hkv,flags", [(2, 2, 0), (2, 2, 1), (8, 2, 0), (8, 2, 1), (16, 4, 0), (6, 3, 0),
                                           (16, 2, 0), (16, 2, 1)])
def test_kivi_prefill_decode_small(Hq, Hkv, flags):
    # flags 0: matrix-core stage 1 (group of 4: one wave per KV head; other
    # group sizes: one wave per query head); flags 1: the VALU stage 1
    w = inputs.workload(3, B=3, Hq=Hq, Hkv=Hkv, ctx=(700, 1301, 2113), steps=3)
    case = _case(w, extra_tokens=300, split_pages=4, flags=flags)
    case.check_status()
    case.check_state()
    case.check_store()
    out, cert, q = case.decode_now(99)
    _check_decode(case, out, cert, q)


@pytest.mark.parametrize("Hq,Hkv,split", [(8, 2, 0), (8, 2, 5), (8, 2, 8), (8, 2, 12), (8, 2, 16),
                                           (16, 2, 0), (16, 2, 12), (4, 2, 0), (4, 2, 8), (24, 3, 5)])
def test_gqa4_body_and_tail_splits(Hq, Hkv, split):
    # the group kernel's work list: body splits of `split` pages, then tail
    # splits of a quarter of that (the last one shorter), over requests
    # holding 0, 9, 19, 32, 45 and 63 quantized pages; every split's partial
    # row merged (split 0: the default for a cache this short).  Groups of 8
    # run as two query quads per KV head, groups of 2 as one quad with two
    # zero queries
    w = inputs.workload(3, B=6, Hq=Hq, Hkv=Hkv, ctx=(70, 700, 1301, 2113, 3000, 4100), steps=3)
    case = _case(w, extra_tokens=80, split_pages=split)
    case.check_status()
    out, cert, q = case.decode_now(7)
    _check_decode(case, out, cert, q)
    for i in range(3):
        out, cert, q = case.step(decode=True)
        _check_decode(case, out, cert, q)
    case.check_status()


def test_gqa4_work_list_over_one_plan_pass():
    # 1040 (request, KV head) pairs, more than one pass of the plan kernel
    # (1024): the list's regions are placed from every pair's counts first,
    # then each pass's items after the earlier passes'
    rng = np.random.default_rng(5)
    ctx = tuple(int(x) for x in rng.integers(100, 1400, size=260))
    w = inputs.workload(3, B=260, Hq=16, Hkv=4, ctx=ctx, steps=2)
    sample = [(0, 0), (17, 3), (129, 1), (200, 2), (255, 2), (259, 3)]
    case = _case(w, extra_tokens=64, split_pages=8, sample=sample)
    case.check_status()
    out, cert, q = case.decode_now(3)
    _check_decode(case, out, cert, q)
    case.check_status()


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2)])
def test_kivi_streaming_crosses_flush_and_pages(Hq, Hkv):
    w = inputs.workload(2, B=2, Hq=Hq, Hkv=Hkv, ctx=(250, 383))
    case = _case(w, extra_tokens=300, split_pages=2)
    for i in range(140):                 # crosses a flush on both requests
        out, cert, q = case.step(decode=(i % 35 == 34 or i in (0, 1, 127, 128, 129)))
        if out is not None:
            _check_decode(case, out, cert, q)
    case.check_status()
    case.check_state()
    case.check_store()


def test_workload1_exact_config():
    w = inputs.workload(1)
    case = _case(w, extra_tokens=64)
    case.check_state()
    case.check_store()
    out, cert, q = case.decode_now(0)
    err = _check_decode(case, out, cert, q)
    print(f"workload 1 max|do| = {err:.3e}")


@pytest.mark.parametrize("ctx", [(1,), (64,), (128,), (129,), (191,), (192,), (257,), (1000,)])
def test_kivi_short_contexts(ctx):
    w = inputs.workload(2, B=1, Hq=4, Hkv=1, ctx=ctx)
    case = _case(w, extra_tokens=200, split_pages=1)
    case.check_state()
    case.check_store()
    out, cert, q = case.decode_now(5)
    _check_decode(case, out, cert, q)
    for i in range(3):
        out, cert, q = case.step()
        _check_decode(case, out, cert, q)
    case.check_store()


@pytest.mark.parametrize("flags", [0, 1])
def test_kitty_calibrate_store_decode(flags):
    w = inputs.workload(4, B=2, Hq=2, Hkv=2, ctx=(1100, 1500))
    case = _case(w, extra_tokens=200, split_pages=3, flags=flags)
    idx_gpu = case.cache.boost_idx.cpu().numpy()
    assert np.array_equal(idx_gpu, case.idx)
    case.check_state()
    case.check_store()
    out, cert, q = case.decode_now(1)
    _check_decode(case, out, cert, q)
    for i in range(130):
        out, cert, q = case.step(decode=(i % 64 == 63))
        if out is not None:
            _check_decode(case, out, cert, q)
    case.check_store()


@pytest.mark.parametrize("wid,Hq,Hkv", [(2, 2, 2), (3, 8, 2), (3, 16, 2), (4, 2, 2), (6, 4, 1), (9, 8, 2)])
def test_sink_tokens_store_decode(wid, Hq, Hkv):
    # the first 32 tokens stay fp16: bit-exact store (sink buffers included)
    # and decode through prefill and two flushes, for KIVI-2 (one query head
    # per wave and the group-of-4 kernel), both Kitty schemes and KIVI-4
    w = inputs.workload(wid, B=2, Hq=Hq, Hkv=Hkv, ctx=(700, 1129))
    case = _case(w, extra_tokens=300, split_pages=3, sink=32)
    case.check_state()
    case.check_store()
    out, cert, q = case.decode_now(2)
    _check_decode(case, out, cert, q)
    for i in range(260):
        out, cert, q = case.step(decode=(i % 64 == 63 or i in (0, 1, 127, 128)))
        if out is not None:
            _check_decode(case, out, cert, q)
    case.check_status()
    case.check_state()
    case.check_store()


@pytest.mark.parametrize("ctx", [(1,), (2,), (31,), (32,), (33,), (159,), (160,), (161,), (290,)])
def test_sink_short_contexts(ctx):
    # contexts inside, at and just past the sink, and around the first flush
    w = inputs.workload(2, B=1, Hq=4, Hkv=1, ctx=ctx)
    case = _case(w, extra_tokens=200, split_pages=1, sink=32)
    case.check_state()
    case.check_store()
    if ctx[0] > 0:
        out, cert, q = case.decode_now(5)
        _check_decode(case, out, cert, q)
    for i in range(40):
        out, cert, q = case.step(decode=(i % 7 == 6 or i in (0, 1)))
        if out is not None:
            _check_decode(case, out, cert, q)
    case.check_status()
    case.check_store()


@pytest.mark.parametrize("wid,Hq,Hkv", [(8, 2, 2), (8, 8, 2)])
def test_kitty_pro_32_boosted_store_decode(wid, Hq, Hkv):
    # 32 boosted channels (two high planes), static set from the calibration
    w = inputs.workload(wid, B=2, Hq=Hq, Hkv=Hkv, ctx=(1100, 1500))
    case = _case(w, extra_tokens=200, split_pages=3)
    idx_gpu = case.cache.boost_idx.cpu().numpy()
    assert np.array_equal(idx_gpu, case.idx)
    assert (idx_gpu < 32).sum(axis=1).tolist() == [32] * Hkv
    case.check_state()
    case.check_store()
    out, cert, q = case.decode_now(1)
    _check_decode(case, out, cert, q)
    for i in range(130):
        out, cert, q = case.step(decode=(i % 64 == 63))
        if out is not None:
            _check_decode(case, out, cert, q)
    case.check_store()


def test_kitty_pro_dynamic_with_sink():
    # 32 boosted channels chosen per page, behind 32 sink tokens
    w = inputs.workload(6, B=2, Hq=4, Hkv=2, ctx=(900, 1300), nb=32)
    case = _case(w, extra_tokens=200, split_pages=2, sink=32)
    case.check_state()
    case.check_store()
    out, cert, q = case.decode_now(1)
    _check_decode(case, out, cert, q)
    for i in range(140):
        out, cert, q = case.step(decode=(i % 64 == 63 or i == 0))
        if out is not None:
            _check_decode(case, out, cert, q)
    case.check_status()
    case.check_store()


@pytest.mark.parametrize("Hq,Hkv,split", [(2, 2, 3), (8, 2, 2), (6, 3, 1), (4, 4, 64)])
def test_kivi4_store_decode(Hq, Hkv, split):
    # 4-bit keys and values: bit-exact codes and statistics through prefill,
    # two flushes and per-token value quantization; decode to the tolerance
    # (one query head per wave for every group size)
    w = inputs.workload(9, B=3, Hq=Hq, Hkv=Hkv, ctx=(700, 1301, 2113))
    case = _case(w, extra_tokens=300, split_pages=split)
    case.check_state()
    case.check_store()
    out, cert, q = case.decode_now(1)
    _check_decode(case, out, cert, q)
    for i in range(260):
        out, cert, q = case.step(decode=(i % 64 == 63 or i in (0, 1, 127, 128)))
        if out is not None:
            _check_decode(case, out, cert, q)
    case.check_status()
    case.check_state()
    case.check_store()


@pytest.mark.parametrize("R", [64, 192, 256])
@pytest.mark.parametrize("wid,Hq,Hkv", [(3, 8, 2), (3, 16, 2), (2, 2, 2), (4, 4, 1), (9, 2, 1), (6, 4, 1),
                                        (8, 2, 2)])
def test_residual_sizes(R, wid, Hq, Hkv):
    # fp16 windows of 64, 192 and 256 tokens (one to four pages flushed at
    # once, as many window chunks): bit-exact store through prefill and
    # flushes, decode to the tolerance, for the group kernel (groups of 4
    # and 8), the one-query-head kernel, Kitty and KIVI-4
    w = inputs.workload(wid, B=2, Hq=Hq, Hkv=Hkv, ctx=(700, R + 37), R=R)
    case = _case(w, extra_tokens=2 * R + 40, split_pages=3)
    case.check_state()
    case.check_store()
    out, cert, q = case.decode_now(1)
    _check_decode(case, out, cert, q)
    for i in range(2 * R + 20):
        out, cert, q = case.step(decode=(i % 37 == 36 or i in (0, R - 1, R)))
        if out is not None:
            _check_decode(case, out, cert, q)
    case.check_status()
    case.check_state()
    case.check_store()


@pytest.mark.parametrize("wid,Hq,Hkv", [(7, 8, 2), (7, 16, 2), (7, 2, 2)])
def test_merge_most_entries(wid, Hq, Hkv):
    # the largest merge a layout allows: a 256-token window plus the sink
    # chunk (five window chunks) and one-page splits over a request that
    # fills a 256-page table (252 paged splits: the window's 256 tokens and
    # the sink occupy the rest of its capacity), for the group kernel (groups
    # of 4 and 8) and the one-query-head kernel; then steps up to the capacity
    w = inputs.workload(wid, B=2, Hq=Hq, Hkv=Hkv, ctx=(16384 - 16, 900), R=256, sink=32)
    case = _case(w, extra_tokens=16, split_pages=1)
    assert case.max_pages == 256
    case.check_state()
    case.check_store()
    out, cert, q = case.decode_now(2)
    _check_decode(case, out, cert, q)
    for i in range(16):
        out, cert, q = case.step(decode=(i in (0, 15)))
        if out is not None:
            _check_decode(case, out, cert, q)
    case.check_status()
    case.check_state()


@pytest.mark.parametrize("ctx", [(1,), (63,), (128,), (129,), (192,), (193,), (300,)])
def test_kivi4_short_contexts(ctx):
    # contexts inside the fp16 windows, at their edges and past the first flush
    w = inputs.workload(9, B=1, Hq=2, Hkv=1, ctx=ctx)
    case = _case(w, extra_tokens=200, split_pages=1)
    case.check_state()
    case.check_store()
    out, cert, q = case.decode_now(3)
    _check_decode(case, out, cert, q)
    for i in range(70):
        out, cert, q = case.step(decode=(i % 9 == 8 or i in (0, 1)))
        if out is not None:
            _check_decode(case, out, cert, q)
    case.check_status()
    case.check_store()


@pytest.mark.parametrize("Hq,Hkv,split", [(2, 2, 3), (8, 2, 2)])
def test_kitty_dynamic_store_decode(Hq, Hkv, split):
    # boosted set chosen per page: bit-exact codes, high plane and per-page
    # channel ids through prefill and two flushes, decode to the tolerance
    w = inputs.workload(6, B=2, Hq=Hq, Hkv=Hkv, ctx=(1100, 1500))
    case = _case(w, extra_tokens=300, split_pages=split)
    case.check_state()
    case.check_store()
    out, cert, q = case.decode_now(1)
    _check_decode(case, out, cert, q)
    for i in range(260):
        out, cert, q = case.step(decode=(i % 64 == 63 or i in (0, 1, 127, 128)))
        if out is not None:
            _check_decode(case, out, cert, q)
    case.check_status()
    case.check_state()
    case.check_store()


@pytest.mark.parametrize("Hq,Hkv,nb,split", [(8, 2, 4, 0), (2, 2, 4, 3), (4, 4, 0, 1), (16, 2, 2, 2),
                                             (1, 1, 4, 64)])
def test_witcert_paged_store_decode_certificate(Hq, Hkv, nb, split):
    # every token quantized on write with slot-keyed dither: bit-exact codes,
    # per-token group scales and bypass rows through prefill and appends that
    # cross pages; decode and certificate to the tolerance
    w = inputs.workload(10, B=3, Hq=Hq, Hkv=Hkv, ctx=(700, 1301, 2113), nb=nb)
    case = _case(w, extra_tokens=200, split_pages=split)
    if nb:
        idx = case.cache.boost_idx.cpu().numpy()
        assert np.array_equal((idx < 2 * nb).astype(np.uint8), case.bypass)
        for h in range(Hkv):                          # offsets in ascending channel order
            ch = np.nonzero(case.bypass[h])[0]
            assert idx[h, ch].tolist() == list(range(2 * nb))
    case.check_state()
    case.check_store()
    out, cert, q = case.decode_now(1, kappa=2.0)
    _check_decode(case, out, cert, q, kappa=2.0, cert_check=True)
    for i in range(130):
        out, cert, q = case.step(decode=(i % 16 == 15 or i in (0, 1)), kappa=1.0)
        if out is not None:
            _check_decode(case, out, cert, q, kappa=1.0, cert_check=True)
    case.check_status()
    case.check_state()
    case.check_store()


@pytest.mark.parametrize("ctx", [(1,), (2,), (63,), (64,), (65,), (130,)])
def test_witcert_paged_short_contexts(ctx):
    w = inputs.workload(10, B=1, Hq=4, Hkv=1, ctx=ctx)
    case = _case(w, extra_tokens=140, split_pages=1)
    case.check_state()
    case.check_store()
    out, cert, q = case.decode_now(2, kappa=1.5)
    _check_decode(case, out, cert, q, kappa=1.5, cert_check=True)
    for i in range(70):
        out, cert, q = case.step(decode=(i % 5 == 4 or i in (0, 1)), kappa=1.5)
        if out is not None:
            _check_decode(case, out, cert, q, kappa=1.5, cert_check=True)
    case.check_status()
    case.check_store()


def test_witcert_paged_prefix_sharing():
    # two requests share the pages of a 512-token prefix (the same slots): the
    # second request's prefill rewrites them with the same bytes, because a
    # token's record depends only on its values and its slot; both requests
    # decode to the oracle, each stream keyed by its own page table
    import torch
    from bit_kv_cache_kivi_amd import kvq
    from oracle import oracle as O
    w = inputs.workload(10, B=2, Hq=4, Hkv=2, ctx=(900, 1100))
    shared, max_pages = 8, 20
    table = np.zeros((2, max_pages), np.int32)
    table[0] = np.arange(max_pages)
    table[1, :shared] = np.arange(shared)
    table[1, shared:] = max_pages + np.arange(max_pages - shared)
    n_pages = 2 * max_pages
    layout = kvq.make_layout("witcert_paged", 2, w.Hq, w.Hkv, max_pages, n_pages,
                             seed=0x5EED_0000_0000_0000 | w.seed, split_pages=3, nb=w.nb)
    cache = kvq.KVCache(layout, table, poison=True)
    calib = np.stack([inputs.kitty_calibration(w, h) for h in range(w.Hkv)])
    cache.witcert_calibrate(torch.from_numpy(calib.view(np.float16)).cuda())
    masks = [O.witcert_select_pairs(calib[h], w.nb) for h in range(w.Hkv)]
    K0 = np.stack([inputs.context_kv(w, 0, h)[0] for h in range(w.Hkv)])
    V0 = np.stack([inputs.context_kv(w, 0, h)[1] for h in range(w.Hkv)])
    K1 = np.stack([inputs.context_kv(w, 1, h)[0] for h in range(w.Hkv)])
    V1 = np.stack([inputs.context_kv(w, 1, h)[1] for h in range(w.Hkv)])
    P = shared * 64
    K1[:, :P], V1[:, :P] = K0[:, :P], V0[:, :P]             # the shared prefix
    ctx = (900, 1100)
    for b, (K, V) in enumerate(((K0, V0), (K1, V1))):
        cache.prefill(b, torch.from_numpy(K.view(np.float16)).cuda()[None].contiguous(),
                      torch.from_numpy(V.view(np.float16)).cuda()[None].contiguous(),
                      torch.tensor([ctx[b]], dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        if b == 0:
            pool0 = cache.pool.cpu().numpy().copy()
    pool1 = cache.pool.cpu().numpy()
    pb = cache.page_bytes * w.Hkv
    assert np.array_equal(pool1[:shared * pb], pool0[:shared * pb])    # rewritten identically
    assert cache.status_word() == 0
    q = inputs.step_q(w, 0)
    out = torch.full((2, w.Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    cert = torch.full((2, w.Hq), float("nan"), dtype=torch.float32, device="cuda")
    cache.decode(torch.from_numpy(q.view(np.float16)).cuda(), out, cert, sm_scale=w.sm_scale,
                 kappa=1.0)
    torch.cuda.synchronize()
    o, c = out.cpu().numpy(), cert.cpu().numpy()
    g = w.group
    for b, (K, V) in enumerate(((K0, V0), (K1, V1))):
        t = np.arange(ctx[b] + 8)
        slots = (table[b][t // 64].astype(np.uint64) * 64 + (t % 64)).astype(np.uint64)
        for h in range(w.Hkv):
            s = O.Stream(O.WITCERT_TOK, ctx[b] + 8, VG=32, idx=masks[h],
                         seed=0x5EED_0000_0000_0000 | w.seed, req=b, layer=0, kvh=h, slots=slots)
            s.prefill(K[h, :ctx[b]], V[h, :ctx[b]])
            ref, rc = s.decode(q[b, h * g:(h + 1) * g], w.sm_scale, 1.0)
            assert np.abs(o[b, h * g:(h + 1) * g] - ref).max() <= TOL_O, (b, h)
            assert np.all(np.abs(c[b, h * g:(h + 1) * g] - rc) <= TOL_CERT * np.abs(rc))


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (2, 2)])
def test_witcert_store_decode_certificate(Hq, Hkv):
    w = inputs.workload(5, B=2, Hq=Hq, Hkv=Hkv, ctx=(700, 1024))
    case = _case(w, extra_tokens=300)
    case.check_state()
    case.check_store()
    for kappa in (0.0, 1.7):
        out, cert, q = case.decode_now(3, kappa=kappa)
        _check_decode(case, out, cert, q, kappa=kappa, cert_check=True)
    for i in range(260):                 # crosses a block flush
        out, cert, q = case.step(decode=(i % 100 == 99), kappa=2.0)
        if out is not None:
            _check_decode(case, out, cert, q, kappa=2.0, cert_check=True)
    case.check_status()
    case.check_state()
    case.check_store()


def test_append_refuses_full_residual_and_flags():
    import torch
    w = inputs.workload(2, B=1, Hq=1, Hkv=1, ctx=(256,))
    case = _case(w, extra_tokens=64, poison=False)
    k, v = inputs.step_kv(w, 0)
    st0 = case.cache.state.clone()
    case.cache.append(torch.from_numpy(k.view(np.float16)).cuda(),
                      torch.from_numpy(v.view(np.float16)).cuda())
    torch.cuda.synchronize()
    assert int(case.cache.status[0].item()) & 1
    assert torch.equal(case.cache.state, st0)


def test_witcert_paged_capacity_and_unmapped_page_flags():
    # WitCert paging-safe: an append past max_pages * 64 tokens sets CAPACITY,
    # one into a page whose table entry is out of range sets UNMAPPED_PAGE;
    # both leave the state as it was
    import torch
    from bit_kv_cache_kivi_amd import kvq
    w = inputs.workload(10, B=1, Hq=4, Hkv=1, ctx=(128,))
    k, v = inputs.step_kv(w, 0)
    kt = torch.from_numpy(k.view(np.float16)).cuda()
    vt = torch.from_numpy(v.view(np.float16)).cuda()
    case = _case(w, extra_tokens=0, poison=False)           # capacity 2 pages = 128 tokens
    st0 = case.cache.state.clone()
    case.cache.append(kt, vt)
    torch.cuda.synchronize()
    assert int(case.cache.status[0].item()) == kvq.STATUS_CAPACITY
    assert torch.equal(case.cache.state, st0)
    # a table whose third entry is out of range: the 129th token has no page
    case2 = _case(w, extra_tokens=64, poison=False)
    case2.cache.page_table[0, 2] = 10 ** 6
    st0 = case2.cache.state.clone()
    case2.cache.append(kt, vt)
    torch.cuda.synchronize()
    assert int(case2.cache.status[0].item()) == kvq.STATUS_UNMAPPED_PAGE
    assert torch.equal(case2.cache.state, st0)


@pytest.mark.parametrize("wid,Hq,Hkv,flags", [(3, 8, 2, 0), (2, 2, 2, 0), (2, 2, 2, 1), (5, 8, 2, 0),
                                              (10, 8, 2, 0)])
def test_decode_flags_unmapped_page(wid, Hq, Hkv, flags):
    # a page-table entry of the quantized prefix out of range: decode reads
    # another page instead (never the entry), sets UNMAPPED_PAGE and still
    # writes finite outputs for every query head
    import torch
    from bit_kv_cache_kivi_amd import kvq
    ctx = (1500, 1500) if wid != 5 else (1300, 1300)
    w = inputs.workload(wid, B=2, Hq=Hq, Hkv=Hkv, ctx=ctx)
    case = _case(w, extra_tokens=64, split_pages=2, poison=False, flags=flags)
    case.check_status()
    case.cache.page_table[1, 1] = case.n_pages + 5           # inside the quantized prefix
    torch.cuda.synchronize()
    out, cert, q = case.decode_now(0, kappa=1.0)
    assert int(case.cache.status[0].item()) == kvq.STATUS_UNMAPPED_PAGE
    assert torch.isfinite(out).all()
    # request 0 does not touch the entry: its outputs still match the oracle
    g = w.group
    for (b, h) in case.streams:
        if b != 0:
            continue
        ref, _ = case.oracle_decode(q, b, h, 1.0)
        assert np.abs(out.cpu().numpy()[b, h * g:(h + 1) * g] - ref).max() <= TOL_O


def test_range_flag_value_scale_and_operand_overflow():
    # leaving the matrix-core stage 1's operand range is reported, and every
    # kernel still exits normally: (a) values x300 give value scales of a few
    # hundred (above 255), flagged when the prefill stores them; (b) queries
    # x2000 against the outlier key channels make |q_c s_c| overflow the f16
    # operand head, and the stage-1 splits come out non-finite and flag it.
    # The VALU stage 1 (binary32) has no such range: the same inputs raise no
    # flag there and decode to finite outputs.
    import torch
    from bit_kv_cache_kivi_amd import kvq
    w = inputs.workload(3, B=2, Hq=8, Hkv=2, ctx=(700, 1301))
    big_v = _case(w, extra_tokens=64, split_pages=4, kv_scale=(1.0, 300.0))
    assert big_v.cache.status_word() == kvq.STATUS_RANGE
    big_v.decode_now(0)
    assert big_v.cache.status_word() == kvq.STATUS_RANGE
    generic = _case(w, extra_tokens=64, split_pages=4, kv_scale=(1.0, 300.0),
                    flags=kvq.FLAG_GENERIC_STAGE1)
    out, _, _ = generic.decode_now(0)
    generic.check_status()
    assert torch.isfinite(out).all()

    plain = _case(w, extra_tokens=64, split_pages=4)
    plain.check_status()
    q = (inputs.step_q(w, 0).view(np.float16).astype(np.float32) * 2000.0).astype(np.float16)
    assert np.isfinite(q.astype(np.float32)).all()
    qt = torch.from_numpy(q).cuda()
    out = torch.empty((w.B, w.Hq, 128), dtype=torch.float32, device="cuda")
    plain.cache.decode(qt, out, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    assert plain.cache.status_word() == kvq.STATUS_RANGE
    g2 = _case(w, extra_tokens=64, split_pages=4, flags=kvq.FLAG_GENERIC_STAGE1)
    g2.cache.decode(qt, out, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    g2.check_status()
    assert torch.isfinite(out).all()


def test_prefill_flags_bad_length():
    # a prefill length beyond the capacity sets BAD_LENGTH and writes nothing
    import torch
    from bit_kv_cache_kivi_amd import kvq
    w = inputs.workload(3, B=1, Hq=4, Hkv=1, ctx=(300,))
    case = _case(w, extra_tokens=0, poison=False)            # capacity 320 tokens
    pool0 = case.cache.pool.clone()
    state0 = case.cache.state.clone()
    K = torch.zeros((1, 1, 400, 128), dtype=torch.float16, device="cuda")
    case.cache.prefill(0, K, K, torch.tensor([400], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert int(case.cache.status[0].item()) == kvq.STATUS_BAD_LENGTH
    assert torch.equal(case.cache.pool, pool0) and torch.equal(case.cache.state, state0)


@pytest.mark.parametrize("wid,Hq,Hkv", [(2, 2, 2), (3, 8, 2), (3, 16, 2), (4, 2, 2), (5, 8, 2), (6, 4, 1),
                                        (7, 8, 2), (9, 4, 2), (10, 8, 2)])
def test_empty_request_decodes_to_zero_then_grows(wid, Hq, Hkv):
    # request 1 holds no token: attention over an empty set is taken as a zero
    # output, a zero certificate and no effect on the other request; then it
    # receives its first tokens through the ordinary step (request 0 keeps its
    # context: the calibration slice of the boosted or bypassed channels is
    # drawn from it)
    w = inputs.workload(wid, B=2, Hq=Hq, Hkv=Hkv, ctx=(300, 0))
    case = _case(w, extra_tokens=64, split_pages=2)
    case.check_status()
    out, cert, q = case.decode_now(3, kappa=1.0)
    assert np.all(out.cpu().numpy()[1] == 0.0) and np.all(cert.cpu().numpy()[1] == 0.0)
    wit = w.scheme in ("witcert", "witcert_paged")
    _check_decode(case, out, cert, q, kappa=1.0, cert_check=wit)
    for i in range(3):
        out, cert, q = case.step(kappa=1.0)
        _check_decode(case, out, cert, q, kappa=1.0, cert_check=wit)
    case.check_status()


@pytest.mark.parametrize("KS,VS", [(1.0, 60.0), (20.0, 1.0)])
@pytest.mark.parametrize("wid,Hq,Hkv", [(3, 8, 2), (3, 16, 2), (2, 2, 2), (4, 2, 2), (9, 2, 2), (6, 4, 1)])
def test_large_magnitudes_inside_the_operand_range(wid, Hq, Hkv, KS, VS):
    # values x60: value scales up to ~150, inside the P.V operands' range
    # (at most 255); keys x20: |q s| up to ~3300 and scores twenty times wider
    # (|q s| below 65504).  Errors grow with the values (the output's scale)
    # and with the keys (the scores' scale), so the bound is 1e-5 x KS x VS.
    w = inputs.workload(wid, B=2, Hq=Hq, Hkv=Hkv, ctx=(700, 1129))
    case = _case(w, extra_tokens=160, split_pages=3, kv_scale=(KS, VS))
    case.check_state()
    case.check_store()
    g = w.group
    tol = TOL_O * KS * VS
    for i in range(130):                        # crosses a key flush
        out, cert, q = case.step(decode=(i % 43 == 42 or i in (0, 129)))
        if out is None:
            continue
        o = out.cpu().numpy()
        for (b, h) in case.streams:
            ref, _ = case.oracle_decode(q, b, h)
            got = o[b, h * g:(h + 1) * g].astype(np.float64)
            assert np.all(np.isfinite(got)), (b, h)
            assert np.abs(got - ref).max() <= tol, (b, h, np.abs(got - ref).max())
    case.check_store()
    case.check_status()
