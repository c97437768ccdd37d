"""The C ABI of libkvq.so on the host (no GPU): every symbol the header
declares is exported, and the host-only entry points (layout validation,
geometry, workspace sizing, error strings) behave as include/kvq.h states.
No call here launches device work."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


@pytest.fixture(scope="module")
def K():
    from bit_kv_cache_kivi_amd import kvq
    if not os.path.exists(kvq.LIB_PATH):
        from bit_kv_cache_kivi_amd import build
        build.build()
    kvq.lib()
    return kvq


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("kvq_set_layout", "kvq_append_token", "kvq_flush_key_group", "kvq_decode_attention"):
        assert n in names


def test_every_declared_symbol_is_exported(K):
    lib = C.CDLL(K.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(declared_functions()) == set(K.EXPORTS)


# fake, suitably aligned device addresses: kvq_set_layout only checks them
A256 = 0x7f0000000000


def bufs(K, **over):
    b = dict(pool=A256, page_table=A256 + 0x1000, state=A256 + 0x2000, res_k=A256 + 0x3000,
             res_v=A256 + 0x4000, boost_idx=A256 + 0x5000, status=A256 + 0x6000,
             sink_k=A256 + 0x7000, sink_v=A256 + 0x8000)
    b.update(over)
    return K.kvq_buffers_t(**b)


def ws_bytes(B, Hq, Hkv, splits, n_win):
    """Workspace of kvq_decode_attention: a partial row (128 fp32 + {lse, A})
    per query head and split or window chunk, a stage-1 work-list item (16 B)
    per (request, KV head, split), and 256 bytes for the list's length."""
    rows = B * Hq * (splits + n_win)
    return rows * (128 * 4 + 8) + B * Hkv * splits * 16 + 256


def gqa_splits(npg, sp):
    """Splits of one (request, KV head) pair of npg pages in the group-of-4
    kernel's work list: body splits of sp pages over all but the last
    min(npg // 8, 2 sp) pages, then tail splits of sp // 4 pages (1 below 4)."""
    tp = sp // 4 if sp >= 4 else 1
    body = (npg - min(npg // 8, 2 * sp)) // sp
    return body + -(-(npg - body * sp) // tp)


def gqa_rows(max_pages, sp):
    """Partial rows per query head the workspace holds: the most any pair of
    at most max_pages pages needs, by brute force."""
    return max(gqa_splits(n, sp) for n in range(max_pages + 1))


def set_layout(K, L, B=None):
    cache = K.kvq_cache_t()
    rc = K.lib().kvq_set_layout(C.byref(cache), C.byref(L), C.byref(B if B is not None else bufs(K)))
    return rc, cache


@pytest.mark.parametrize("scheme", ["kivi2", "kitty", "witcert", "kitty_dyn", "kivi4", "witcert_paged"])
def test_valid_layouts(K, scheme):
    L = K.make_layout(scheme, B=64, Hq=32, Hkv=8, max_pages=512, n_pages=32768)
    rc, cache = set_layout(K, L)
    assert rc == K.KVQ_OK
    assert cache.page_tokens == (256 if scheme == "witcert" else 64)
    assert cache.page_bytes == {"kivi2": 6144, "kitty": 6400, "witcert": 66048,
                                "kitty_dyn": 6416, "kivi4": 10240, "witcert_paged": 18432}[scheme]


def test_page_geometry_and_bytes_per_token(K):
    # 96 B/token/KV head for KIVI-2 (codes + fp16 statistics of keys and
    # values), 100 with Kitty's 16-channel high plane, 258 for the INT8 block
    # scheme (128 codes + an fp16 scale per 256-token block and channel, twice);
    # Kitty dynamic adds the page's 16 boosted channel ids (0.25 B/token)
    # Kitty-Pro (32 boosted channels): one more 256-B high plane, 104 B/token;
    # KIVI-4: 64 + 64 B of codes and the same 32 B of statistics, 160 B/token
    for scheme, nb, bpt in (("kivi2", None, 96.0), ("kitty", None, 100.0), ("witcert", None, 258.0),
                            ("kitty_dyn", None, 100.25), ("kitty", 32, 104.0),
                            ("kitty_dyn", 32, 104.5), ("kivi4", None, 160.0)):
        L = K.make_layout(scheme, B=1, Hq=1, Hkv=1, max_pages=1, n_pages=1, nb=nb)
        assert K.bytes_per_token(L) == bpt
        assert K.page_bytes(L) == bpt * K.page_tokens(L)
    bad = K.make_layout("kivi2", B=1, Hq=1, Hkv=1, max_pages=1, n_pages=1)
    bad.scheme = 7
    assert K.page_bytes(bad) == 0 and K.page_tokens(bad) == 0 and K.bytes_per_token(bad) == 0.0


INVALID = [
    ("head_dim", 64), ("n_kv_heads", 0), ("n_kv_heads", 65536), ("n_q_heads", 12),
    ("n_q_heads", 72), ("batch", 0), ("batch", 65536), ("max_pages", 0), ("n_pages", 0),
    ("split_pages", -1), ("split_pages", 65), ("flags", 2), ("scheme", 6), ("scheme", -1),
    ("group", 64), ("value_group", 16), ("residual", 96), ("residual", 100),
    ("residual", 0), ("residual", 320), ("n_boost", 4),
]


@pytest.mark.parametrize("field,value", INVALID)
def test_invalid_kivi_fields(K, field, value):
    L = K.make_layout("kivi2", B=8, Hq=8, Hkv=8, max_pages=64, n_pages=512)
    setattr(L, field, value)
    rc, cache = set_layout(K, L)
    assert rc == K.KVQ_EINVAL
    assert cache.magic == 0


def test_residual_must_hold_whole_key_groups(K):
    # R % G == 0 is required ("KIVI" explainer 3.3); with G = 32 and whole
    # 64-token pages the accepted residuals are 64, 128, 192, 256
    ok = []
    for R in range(0, 300, 16):
        L = K.make_layout("kivi2", B=1, Hq=1, Hkv=1, max_pages=8, n_pages=8, R=R)
        ok.append(R) if set_layout(K, L)[0] == K.KVQ_OK else None
    assert ok == [64, 128, 192, 256]


def test_kitty_and_witcert_fields(K):
    L = K.make_layout("kitty", B=1, Hq=4, Hkv=4, max_pages=8, n_pages=8, nb=0)
    assert set_layout(K, L)[0] == K.KVQ_EINVAL
    for scheme in ("kitty", "kitty_dyn"):
        for nb, want in ((8, K.KVQ_EINVAL), (16, K.KVQ_OK), (24, K.KVQ_EINVAL), (32, K.KVQ_OK),
                         (64, K.KVQ_EINVAL)):
            L = K.make_layout(scheme, B=1, Hq=4, Hkv=4, max_pages=8, n_pages=8, nb=nb)
            assert set_layout(K, L)[0] == want, (scheme, nb)
    L = K.make_layout("kitty", B=1, Hq=4, Hkv=4, max_pages=8, n_pages=8, nb=32,
                      flags=K.FLAG_GENERIC_STAGE1)          # the VALU stage 1: 16 only
    assert set_layout(K, L)[0] == K.KVQ_EINVAL
    # the VALU stage 1 knows only the static boost table
    L = K.make_layout("kitty_dyn", B=1, Hq=4, Hkv=4, max_pages=8, n_pages=8,
                      flags=K.FLAG_GENERIC_STAGE1)
    assert set_layout(K, L)[0] == K.KVQ_EINVAL
    L = K.make_layout("kitty", B=1, Hq=4, Hkv=4, max_pages=8, n_pages=8,
                      flags=K.FLAG_GENERIC_STAGE1)
    assert set_layout(K, L)[0] == K.KVQ_OK
    L = K.make_layout("witcert", B=1, Hq=32, Hkv=8, max_pages=8, n_pages=8)
    L.block = 128
    assert set_layout(K, L)[0] == K.KVQ_EINVAL
    L = K.make_layout("witcert", B=1, Hq=32, Hkv=8, max_pages=8, n_pages=8, layer=65536)
    assert set_layout(K, L)[0] == K.KVQ_EINVAL
    L = K.make_layout("witcert", B=1, Hq=24, Hkv=8, max_pages=8, n_pages=8)    # 3 per KV head
    assert set_layout(K, L)[0] == K.KVQ_EINVAL
    L = K.make_layout("kivi2", B=1, Hq=24, Hkv=8, max_pages=8, n_pages=8)      # fine for KIVI-2
    assert set_layout(K, L)[0] == K.KVQ_OK


def test_byte_accounts_match_the_pages(K):
    # Kitty: the high plane adds 2 bits per boosted channel, 2 + 2 alpha bits
    # per key element; WitCert blocks: 128 int8 codes + an fp16 scale per
    # 256-token block and channel = 129 B per token and side
    import json
    with open(os.path.join(ROOT, "tests", "golden", "byte_accounts.json")) as f:
        g = json.load(f)
    base = K.page_bytes(K.make_layout("kivi2", B=1, Hq=1, Hkv=1, max_pages=1, n_pages=1))
    for alpha, bits in g["kitty_bits_per_key_element"].items():
        nb = int(float(alpha) * 128)
        L = K.make_layout("kitty", B=1, Hq=1, Hkv=1, max_pages=1, n_pages=1, nb=nb)
        high_bits = (K.page_bytes(L) - base) * 8 / (64 * 128)   # per key element
        assert 2 + high_bits == bits, (alpha, 2 + high_bits)
    L = K.make_layout("witcert", B=1, Hq=1, Hkv=1, max_pages=1, n_pages=1)
    assert K.bytes_per_token(L) == 2 * g["witcert_int8_bytes_per_token_per_side"]


def test_witcert_paged_bytes_match_the_page(K):
    # WitCert certified deployment: 136 B per token, head and side at G_c = 32
    # (K+V 272 B), and 16 B of fp16 bypass values for m = 4 pairs
    import json
    with open(os.path.join(ROOT, "tests", "golden", "witcert_paged.json")) as f:
        g = json.load(f)
    L = K.make_layout("witcert_paged", B=1, Hq=1, Hkv=1, max_pages=1, n_pages=1, nb=0)
    assert K.bytes_per_token(L) == g["bytes_per_token_kv"]
    L = K.make_layout("witcert_paged", B=1, Hq=1, Hkv=1, max_pages=1, n_pages=1, nb=g["m"])
    assert K.bytes_per_token(L) == g["bytes_per_token_kv"] + g["bypass_bytes"]
    assert K.page_tokens(L) == 64


def test_witcert_paged_fields(K):
    def lay(**kw):
        args = dict(B=1, Hq=8, Hkv=2, max_pages=8, n_pages=8)
        args.update(kw)
        return K.make_layout("witcert_paged", **args)
    for nb, want in ((0, K.KVQ_OK), (1, K.KVQ_OK), (4, K.KVQ_OK), (5, K.KVQ_EINVAL), (-1, K.KVQ_EINVAL)):
        assert set_layout(K, lay(nb=nb))[0] == want, nb
    assert set_layout(K, lay(Hq=6))[0] == K.KVQ_EINVAL              # 3 query heads per KV head
    assert set_layout(K, lay(sink=16))[0] == K.KVQ_EINVAL
    assert set_layout(K, lay(flags=K.FLAG_GENERIC_STAGE1))[0] == K.KVQ_EINVAL
    assert set_layout(K, lay(layer=65536))[0] == K.KVQ_EINVAL
    for field, value in (("group", 64), ("value_group", 16)):
        L = lay()
        setattr(L, field, value)
        assert set_layout(K, L)[0] == K.KVQ_EINVAL
    # no fp16 residual buffers; the bypass index only with bypassed pairs
    assert set_layout(K, lay(), bufs(K, res_k=0, res_v=0))[0] == K.KVQ_OK
    assert set_layout(K, lay(), bufs(K, boost_idx=0))[0] == K.KVQ_ENULL
    assert set_layout(K, lay(nb=0), bufs(K, boost_idx=0))[0] == K.KVQ_OK
    # default split 4 pages (256 tokens); no window chunks in the workspace
    rc, cache = set_layout(K, lay(max_pages=100, n_pages=100))
    assert rc == K.KVQ_OK and cache.split_pages == 4
    assert K.kvq_workspace_bytes(cache) == ws_bytes(B=1, Hq=8, Hkv=2, splits=25, n_win=0)
    # calibration: the scheme and m > 0 are checked before any launch
    lib = K.lib()
    a = C.c_void_p(A256 + 0x20000)
    assert lib.kvq_witcert_calibrate(C.byref(cache), a, 0, a, None) == K.KVQ_EINVAL
    assert lib.kvq_witcert_calibrate(C.byref(cache), None, 8, a, None) == K.KVQ_ENULL
    rc0, c0 = set_layout(K, lay(nb=0))
    assert lib.kvq_witcert_calibrate(C.byref(c0), a, 8, a, None) == K.KVQ_EINVAL
    rc2, c2 = set_layout(K, K.make_layout("kivi2", B=1, Hq=8, Hkv=2, max_pages=8, n_pages=8))
    assert lib.kvq_witcert_calibrate(C.byref(c2), a, 8, a, None) == K.KVQ_EINVAL


def test_kivi4_fields(K):
    # KIVI-4 shares KIVI-2's groups and windows, has no boosted channels, and
    # its 4-bit codes have no VALU stage 1
    L = K.make_layout("kivi4", B=1, Hq=24, Hkv=8, max_pages=8, n_pages=8, sink=16)
    assert set_layout(K, L)[0] == K.KVQ_OK
    for nb in (16, 32):
        L = K.make_layout("kivi4", B=1, Hq=4, Hkv=4, max_pages=8, n_pages=8, nb=nb)
        assert set_layout(K, L)[0] == K.KVQ_EINVAL
    L = K.make_layout("kivi4", B=1, Hq=4, Hkv=4, max_pages=8, n_pages=8, flags=K.FLAG_GENERIC_STAGE1)
    assert set_layout(K, L)[0] == K.KVQ_EINVAL
    for field, value in (("group", 64), ("value_group", 16), ("residual", 96)):
        L = K.make_layout("kivi4", B=1, Hq=4, Hkv=4, max_pages=8, n_pages=8)
        setattr(L, field, value)
        assert set_layout(K, L)[0] == K.KVQ_EINVAL


def test_null_and_alignment(K):
    L = K.make_layout("kivi2", B=1, Hq=1, Hkv=1, max_pages=8, n_pages=8)
    cache = K.kvq_cache_t()
    lib = K.lib()
    assert lib.kvq_set_layout(None, C.byref(L), C.byref(bufs(K))) == K.KVQ_ENULL
    assert lib.kvq_set_layout(C.byref(cache), None, C.byref(bufs(K))) == K.KVQ_ENULL
    assert lib.kvq_set_layout(C.byref(cache), C.byref(L), None) == K.KVQ_ENULL
    for f in ("pool", "page_table", "state", "res_k", "res_v", "status"):
        assert set_layout(K, L, bufs(K, **{f: 0}))[0] == K.KVQ_ENULL, f
    assert set_layout(K, L, bufs(K, boost_idx=0))[0] == K.KVQ_OK      # only Kitty needs it
    Lk = K.make_layout("kitty", B=1, Hq=1, Hkv=1, max_pages=8, n_pages=8)
    assert set_layout(K, Lk, bufs(K, boost_idx=0))[0] == K.KVQ_ENULL
    Ld = K.make_layout("kitty_dyn", B=1, Hq=1, Hkv=1, max_pages=8, n_pages=8)
    assert set_layout(K, Ld, bufs(K, boost_idx=0))[0] == K.KVQ_OK    # chosen per page
    for f, off in (("pool", 16), ("page_table", 4), ("state", 8), ("res_k", 2), ("res_v", 8),
                   ("status", 2)):
        b = bufs(K)
        setattr(b, f, getattr(b, f) + off)
        assert set_layout(K, L, b)[0] == K.KVQ_EALIGN, f


def test_split_resolution_and_workspace(K):
    # default split: 4 pages up to 32 pages of cache, 8 up to 128, above that
    # 32 (12 for KIVI4; 1 for WITCERT's 256-token pages); for the KIVI2 group kernel bodies
    # of 8 and 48 pages with quarter-length tail splits; raised to what keeps
    # at most 256 splits
    cases = (("kivi2", 8, 100, 8), ("kivi2", 8, 128, 8), ("kitty", 8, 32, 4), ("kitty", 8, 33, 8),
             ("kitty", 8, 129, 32), ("kivi2", 8, 129, 48), ("kivi2", 8, 512, 48), ("kivi2", 8, 4096, 48),
             ("kivi2", 8, 8000, 48), ("kivi2", 8, 15807, 64),
             ("kivi2", 2, 16, 4), ("kivi2", 2, 100, 8), ("kivi2", 2, 129, 32), ("kivi2", 2, 512, 32),
             ("kivi2", 2, 8192, 32), ("kivi2", 2, 8193, 33), ("kivi2", 4, 512, 48), ("kivi2", 16, 512, 48),
             ("kivi2", 6, 512, 32), ("kivi4", 8, 512, 12), ("kivi4", 8, 100, 8),
             ("witcert", 8, 64, 1), ("witcert", 8, 1024, 4))
    for scheme, Hq, max_pages, want in cases:
        L = K.make_layout(scheme, B=2, Hq=Hq, Hkv=2, max_pages=max_pages, n_pages=max_pages)
        rc, cache = set_layout(K, L)
        assert rc == K.KVQ_OK and cache.split_pages == want, (scheme, Hq, max_pages)
        gqa = scheme == "kivi2" and Hq // 2 in (2, 4, 8)    # the group kernel
        rows = gqa_rows(max_pages, want) if gqa else -(-max_pages // want)
        n_win = 4 if scheme == "witcert" else 128 // 64     # 64-token chunks of the fp16 window
        ws = K.kvq_workspace_bytes(cache)
        if gqa:     # a closed-form bound on the rows: exact or at most two rows over
            assert any(ws == ws_bytes(B=2, Hq=Hq, Hkv=2, splits=rows + d, n_win=n_win) for d in (0, 1, 2))
        else:
            assert ws == ws_bytes(B=2, Hq=Hq, Hkv=2, splits=rows, n_win=n_win)
        assert rows <= 256
    # past what 256 group-of-4 splits of 64-page bodies and their tails hold
    L = K.make_layout("kivi2", B=2, Hq=8, Hkv=2, max_pages=15808, n_pages=8)
    assert set_layout(K, L)[0] == K.KVQ_EINVAL
    # the VALU stage 1 takes the one-query-head kernel's default
    L = K.make_layout("kivi2", B=2, Hq=8, Hkv=2, max_pages=512, n_pages=512, flags=K.FLAG_GENERIC_STAGE1)
    assert set_layout(K, L)[1].split_pages == 32
    L = K.make_layout("kivi2", B=1, Hq=1, Hkv=1, max_pages=16385, n_pages=8)
    assert set_layout(K, L)[0] == K.KVQ_EINVAL          # would need splits of 128 pages
    L = K.make_layout("kivi2", B=1, Hq=1, Hkv=1, max_pages=100, n_pages=8, split_pages=3)
    rc, cache = set_layout(K, L)
    assert rc == K.KVQ_OK and cache.split_pages == 3


def test_calls_on_an_unset_cache_launch_nothing(K):
    lib = K.lib()
    cache = K.kvq_cache_t()                      # zeroed: not filled by kvq_set_layout
    assert K.kvq_workspace_bytes(cache) == 0
    assert lib.kvq_append_token(C.byref(cache), None, None, None) == K.KVQ_ENOLAYOUT
    assert lib.kvq_flush_key_group(C.byref(cache), None) == K.KVQ_ENOLAYOUT
    assert lib.kvq_decode_attention(C.byref(cache), None, None, None, C.c_float(1.0),
                                    C.c_float(0.0), None, C.c_size_t(0), None) == K.KVQ_ENOLAYOUT
    assert lib.kvq_prefill(C.byref(cache), 0, 1, None, None, C.c_int64(1), None,
                           None) == K.KVQ_ENOLAYOUT
    assert lib.kvq_kitty_calibrate(C.byref(cache), None, 1, None, None) == K.KVQ_ENOLAYOUT
    assert lib.kvq_witcert_calibrate(C.byref(cache), None, 1, None, None) == K.KVQ_ENOLAYOUT
    assert lib.kvq_append_token(None, None, None, None) == K.KVQ_ENULL


def test_decode_rejects_small_workspace_before_launching(K):
    L = K.make_layout("kivi2", B=2, Hq=8, Hkv=2, max_pages=64, n_pages=128)
    rc, cache = set_layout(K, L)
    assert rc == K.KVQ_OK
    need = K.kvq_workspace_bytes(cache)
    a = A256 + 0x10000
    rc = K.lib().kvq_decode_attention(C.byref(cache), C.c_void_p(a), C.c_void_p(a + 0x1000), None,
                                      C.c_float(1.0), C.c_float(0.0), C.c_void_p(a + 0x100000),
                                      C.c_size_t(need - 1), None)
    assert rc == K.KVQ_EWORKSPACE


def test_load_floor_host_checks_launch_nothing(K):
    # kvq_stage1_load_floor runs only the group kernel's copy: every check
    # that fails returns before any device call (these addresses are fake)
    lib = K.lib()
    a = A256 + 0x10000
    q, ws = C.c_void_p(a), C.c_void_p(a + 0x100000)
    one = C.c_float(1.0)
    unset = K.kvq_cache_t()
    assert lib.kvq_stage1_load_floor(C.byref(unset), q, one, ws, C.c_size_t(1 << 30),
                                     None) == K.KVQ_ENOLAYOUT
    # layouts that do not run the group kernel
    for scheme, Hq, flags in (("kivi2", 2, 0), ("kivi2", 8, K.FLAG_GENERIC_STAGE1),
                              ("kitty", 8, 0), ("kivi4", 8, 0), ("witcert", 8, 0)):
        L = K.make_layout(scheme, B=2, Hq=Hq, Hkv=2, max_pages=64, n_pages=128)
        L.flags = flags
        rc, cache = set_layout(K, L)
        assert rc == K.KVQ_OK, scheme
        assert lib.kvq_stage1_load_floor(C.byref(cache), q, one, ws, C.c_size_t(1 << 30),
                                         None) == K.KVQ_EINVAL, (scheme, Hq, flags)
    L = K.make_layout("kivi2", B=2, Hq=8, Hkv=2, max_pages=64, n_pages=128)
    rc, cache = set_layout(K, L)
    assert rc == K.KVQ_OK
    need = K.kvq_workspace_bytes(cache)
    assert lib.kvq_stage1_load_floor(C.byref(cache), None, one, ws, C.c_size_t(need),
                                     None) == K.KVQ_ENULL
    assert lib.kvq_stage1_load_floor(C.byref(cache), q, one, None, C.c_size_t(need),
                                     None) == K.KVQ_ENULL
    assert lib.kvq_stage1_load_floor(C.byref(cache), C.c_void_p(a + 8), one, ws, C.c_size_t(need),
                                     None) == K.KVQ_EALIGN
    assert lib.kvq_stage1_load_floor(C.byref(cache), q, one, C.c_void_p(a + 0x100040),
                                     C.c_size_t(need), None) == K.KVQ_EALIGN
    assert lib.kvq_stage1_load_floor(C.byref(cache), q, one, ws, C.c_size_t(need - 1),
                                     None) == K.KVQ_EWORKSPACE


def test_error_strings(K):
    lib = K.lib()
    lib.kvq_strerror.restype = C.c_char_p
    codes = (K.KVQ_OK, K.KVQ_EINVAL, K.KVQ_ENULL, K.KVQ_EALIGN, K.KVQ_ENOLAYOUT,
             K.KVQ_EWORKSPACE, K.KVQ_ELAUNCH, K.KVQ_ENOSCRATCH)
    texts = [lib.kvq_strerror(c) for c in codes]
    assert all(isinstance(t, bytes) and len(t) > 0 for t in texts)
    assert len(set(texts)) == len(codes)                    # one text per return code
    assert lib.kvq_strerror(-99) == b"unknown"
    # device status words: each bit its own text, several bits one text,
    # undefined bits "unknown"
    bits = (K.STATUS_RESIDUAL_FULL, K.STATUS_CAPACITY, K.STATUS_UNMAPPED_PAGE,
            K.STATUS_BAD_LENGTH, K.STATUS_RANGE)
    btexts = [lib.kvq_strerror(b) for b in bits]
    assert len(set(btexts)) == len(bits) and not set(btexts) & set(texts)
    assert b"unknown" not in btexts
    many = lib.kvq_strerror(K.STATUS_CAPACITY | K.STATUS_RANGE)
    assert many == b"several device status bits" and many not in btexts
    assert lib.kvq_strerror(32) == b"unknown" and lib.kvq_strerror(1 | 64) == b"unknown"
    # the header declares each bit the binding names
    text = open(HEADER).read()
    for name, val in (("RESIDUAL_FULL", 1), ("CAPACITY", 2), ("UNMAPPED_PAGE", 4),
                      ("BAD_LENGTH", 8), ("RANGE", 16)):
        assert re.search(rf"KVQ_STATUS_{name}\s*=\s*{val}u", text), name


def test_sink_fields_and_workspace(K):
    # sink tokens: 0 .. 64 for KIVI2 / Kitty, none for WITCERT; the sink
    # buffers are required and aligned when sink > 0; one more window chunk
    for sink, rc_want in ((0, K.KVQ_OK), (32, K.KVQ_OK), (64, K.KVQ_OK), (65, K.KVQ_EINVAL),
                          (-1, K.KVQ_EINVAL)):
        L = K.make_layout("kivi2", B=2, Hq=8, Hkv=2, max_pages=64, n_pages=64, sink=sink)
        assert set_layout(K, L)[0] == rc_want, sink
    L = K.make_layout("witcert", B=2, Hq=8, Hkv=2, max_pages=8, n_pages=8, sink=32)
    assert set_layout(K, L)[0] == K.KVQ_EINVAL
    L = K.make_layout("kivi2", B=2, Hq=8, Hkv=2, max_pages=64, n_pages=64)
    L.reserved = 1
    assert set_layout(K, L)[0] == K.KVQ_EINVAL
    L = K.make_layout("kitty_dyn", B=2, Hq=8, Hkv=2, max_pages=64, n_pages=64, sink=32)
    assert set_layout(K, L, bufs(K, sink_k=0))[0] == K.KVQ_ENULL
    assert set_layout(K, L, bufs(K, sink_v=0))[0] == K.KVQ_ENULL
    b = bufs(K)
    b.sink_k += 8
    assert set_layout(K, L, b)[0] == K.KVQ_EALIGN
    rc, cache = set_layout(K, L)
    assert rc == K.KVQ_OK
    splits = -(-64 // cache.split_pages)
    # window chunks + the sink chunk
    assert K.kvq_workspace_bytes(cache) == ws_bytes(B=2, Hq=8, Hkv=2, splits=splits, n_win=128 // 64 + 1)


def test_noalloc_rejects_oversized_cache_before_device_work(K):
    # kvq_decode_attention_noalloc refuses a cache whose workspace exceeds the
    # scratch array, before any HIP call (no GPU needed to see it)
    L = K.make_layout("kivi2", B=256, Hq=32, Hkv=8, max_pages=512, n_pages=256 * 512)
    rc, cache = set_layout(K, L)
    assert rc == K.KVQ_OK
    assert K.kvq_workspace_bytes(cache) > K.NOALLOC_SCRATCH_BYTES
    a = A256 + 0x10000
    lib = K.lib()
    rc = lib.kvq_decode_attention_noalloc(C.byref(cache), C.c_void_p(a), C.c_void_p(a + 0x1000),
                                          None, C.c_float(1.0), C.c_float(0.0), None)
    assert rc == K.KVQ_ENOSCRATCH
    assert lib.kvq_decode_attention_noalloc(C.byref(cache), None, C.c_void_p(a), None,
                                            C.c_float(1.0), C.c_float(0.0), None) == K.KVQ_ENULL
    s = lib.kvq_strerror(K.KVQ_ENOSCRATCH)
    assert s and s != lib.kvq_strerror(K.KVQ_EWORKSPACE)
    # the header's size and the binding's agree
    text = open(HEADER).read()
    assert "KVQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in text
    assert K.NOALLOC_SCRATCH_BYTES == 64 << 20
