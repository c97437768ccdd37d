"""Test-side reader of the library's page layout (as documented in
bit_kv_cache_kivi_amd/csrc/kvq_common.hpp): maps the packed bytes of a
(page, KV head) block back to logical codes and statistics so they can be
compared with the oracle's.  Written independently of the HIP code."""
from __future__ import annotations

import numpy as np

D = 128
PT = 64
WPT = 256

def geom(scheme: int, nb: int = 16) -> dict:
    """Block layout: KIVI-2 (0), Kitty (1, nb boosted channels: one 256-B high
    plane per 16), WitCert (2), Kitty dynamic (3: Kitty + the page's nb
    channel ids, at least 16 bytes), KIVI-4 (4: 4-bit key and value codes),
    WitCert paging-safe (5: per-token int8 rows, scales per 32-channel group,
    an 8-entry fp16 bypass row per token when nb pairs > 0)."""
    if scheme == 5:
        return dict(kc=0, vc=8192, ks=16384, vs=16896, kb=17408,
                    bytes=17408 + (1024 if nb > 0 else 0), tokens=PT)
    if scheme == 4:
        return dict(kc=0, kh=0, ks=4096, vc=5120, vs=9216, bytes=10240, tokens=PT)
    if scheme == 0:
        return dict(kc=0, kh=0, ks=2048, vc=3072, vs=5120, bytes=6144, tokens=PT)
    if scheme == 2:
        return dict(kc=0, kh=0, ks=32768, vc=33024, vs=65792, bytes=66048, tokens=WPT)
    ks = 2048 + 16 * nb
    g = dict(kc=0, kh=2048, ks=ks, vc=ks + 1024, vs=ks + 3072, bytes=ks + 4096, tokens=PT)
    if scheme == 3:
        g["ki"] = g["bytes"]
        g["bytes"] += max(16, nb)
    return g


GEOM = {s: geom(s) for s in range(5)}
KITTY_SCHEMES = (1, 3)


def _key_index():
    t = np.arange(PT)[:, None]
    c = np.arange(D)[None, :]
    n, r, kc, g, j = t >> 4, t & 15, c >> 5, (c >> 3) & 3, c & 7
    lane = 16 * g + r
    d = 2 * n + (kc >> 1)
    h = kc & 1
    dword = (d >> 2) * 256 + lane * 4 + (d & 3)
    shift = 4 * j + 2 * h
    return dword, shift


def _value_index():
    t = np.arange(PT)[:, None]
    c = np.arange(D)[None, :]
    nt, r, ks, g, j = c >> 4, c & 15, t >> 5, (t >> 3) & 3, t & 7
    lane = 16 * g + r
    dword = (nt >> 2) * 256 + lane * 4 + (nt & 3)
    shift = 4 * j + 2 * ks
    return dword, shift


def _nibble_shift(k):
    """4-bit code k (0..7) of a KIVI-4 dword: byte k % 4, nibble k // 4."""
    return 8 * (k & 3) + 4 * (k >> 2)


def _key_index4():
    """KIVI-4 keys: token t, channel c -> dword 256 (t // 16) + 4 lane +
    c // 32 with lane = 16 ((c // 8) % 4) + t % 16; code c % 8 of the dword."""
    t = np.arange(PT)[:, None]
    c = np.arange(D)[None, :]
    lane = 16 * ((c >> 3) & 3) + (t & 15)
    return 256 * (t >> 4) + 4 * lane + (c >> 5), _nibble_shift(c & 7)


def _value_index4():
    """KIVI-4 values: dword d = 8 (t // 32) + c // 16 of lane 16 ((t // 8) % 4)
    + c % 16 at 256 (d // 4) + 4 lane + d % 4; code t % 8 of the dword."""
    t = np.arange(PT)[:, None]
    c = np.arange(D)[None, :]
    lane = 16 * ((t >> 3) & 3) + (c & 15)
    d = 8 * (t >> 5) + (c >> 4)
    return 256 * (d >> 2) + 4 * lane + (d & 3), _nibble_shift(t & 7)


def _high_index(nb=16):
    t = np.arange(PT)[:, None]
    o = np.arange(nb)[None, :]
    n, r, q, g, i = t >> 4, t & 15, o >> 4, (o & 15) >> 2, o & 3
    dword = 64 * q + 16 * g + r
    shift = 4 * (4 * (n & 1) + i) + 2 * (n >> 1)
    return dword, shift


KEY_DW, KEY_SH = _key_index()
VAL_DW, VAL_SH = _value_index()
HI_DW, HI_SH = _high_index()
KEY4_DW, KEY4_SH = _key_index4()
VAL4_DW, VAL4_SH = _value_index4()
KEY_SLOT = np.arange(D)            # key statistics in channel order


def _u32(block: np.ndarray, off: int, n: int) -> np.ndarray:
    return block[off:off + 4 * n].view(np.uint32)


def key_codes(block: np.ndarray, scheme: int) -> np.ndarray:
    """Low 2-bit key codes [64][128] (KIVI-4: the 4-bit codes)."""
    g = geom(scheme)
    if scheme == 4:
        return ((_u32(block, g["kc"], 1024)[KEY4_DW] >> KEY4_SH) & 15).astype(np.uint8)
    kc = _u32(block, g["kc"], 512)
    return ((kc[KEY_DW] >> KEY_SH) & 3).astype(np.uint8)


def key_high(block: np.ndarray, nb: int = 16) -> np.ndarray:
    """Kitty high planes [64][nb] by boosted offset (same place in both Kitty schemes)."""
    g = geom(1, nb)
    kh = _u32(block, g["kh"], 4 * nb)
    dw, sh = _high_index(nb)
    return ((kh[dw] >> sh) & 3).astype(np.uint8)


def key_stats(block: np.ndarray, scheme: int, nb: int = 16):
    """(scale, zero) fp16 bits [2 groups][128 channels]."""
    g = geom(scheme, nb)
    ks = _u32(block, g["ks"], 256).reshape(2, 128)[:, KEY_SLOT]
    return (ks & 0xFFFF).astype(np.uint16), (ks >> 16).astype(np.uint16)


def page_boost_index(block: np.ndarray, nb: int = 16) -> np.ndarray:
    """Kitty dynamic: the page's boost index per channel (offset, or nb + 1)
    from its stored channel ids."""
    ki = geom(3, nb)["ki"]
    ids = block[ki:ki + nb]
    idx = np.full(D, nb + 1, np.uint8)
    idx[ids.astype(np.int64)] = np.arange(nb, dtype=np.uint8)
    return idx


def value_codes(block: np.ndarray, scheme: int, nb: int = 16) -> np.ndarray:
    g = geom(scheme, nb)
    if scheme == 4:
        return ((_u32(block, g["vc"], 1024)[VAL4_DW] >> VAL4_SH) & 15).astype(np.uint8)
    vc = _u32(block, g["vc"], 512)
    return ((vc[VAL_DW] >> VAL_SH) & 3).astype(np.uint8)


def value_stats(block: np.ndarray, scheme: int, nb: int = 16):
    """(scale, zero) fp16 bits [64 tokens][4 groups]."""
    g = geom(scheme, nb)
    vs = _u32(block, g["vs"], 256).reshape(64, 4)
    return (vs & 0xFFFF).astype(np.uint16), (vs >> 16).astype(np.uint16)


def witcert_paged_block(block: np.ndarray, nb: int):
    """(key codes int8 [64][128], key scales [64][4], value codes, value
    scales, bypass rows fp16 [64][8] or None)."""
    g = geom(5, nb)
    kc = block[g["kc"]:g["kc"] + PT * D].view(np.int8).reshape(PT, D)
    vc = block[g["vc"]:g["vc"] + PT * D].view(np.int8).reshape(PT, D)
    ks = block[g["ks"]:g["ks"] + PT * 8].view(np.uint16).reshape(PT, 4)
    vs = block[g["vs"]:g["vs"] + PT * 8].view(np.uint16).reshape(PT, 4)
    kb = block[g["kb"]:g["kb"] + PT * 16].view(np.uint16).reshape(PT, 8) if nb > 0 else None
    return kc, ks, vc, vs, kb


def witcert_block(block: np.ndarray):
    """(key codes int8 [256][128], key scales [128], value codes, value scales)."""
    g = GEOM[2]
    kc = block[g["kc"]:g["kc"] + WPT * D].view(np.int8).reshape(WPT, D)
    ks = block[g["ks"]:g["ks"] + 2 * D].view(np.uint16)
    vc = block[g["vc"]:g["vc"] + WPT * D].view(np.int8).reshape(WPT, D)
    vs = block[g["vs"]:g["vs"] + 2 * D].view(np.uint16)
    return kc, ks, vc, vs


def page_block(pool: np.ndarray, pid: int, h: int, Hkv: int, scheme: int, nb: int = 16) -> np.ndarray:
    nbytes = geom(scheme, nb)["bytes"]
    off = (pid * Hkv + h) * nbytes
    return pool[off:off + nbytes]


def gather_kivi(pool, table_row, h, Hkv, scheme, n_kq, n_vq, idx=None, page_idx=None, nb=16):
    """Logical record of one (request, KV head) for tokens below n_kq / n_vq:
    key codes (4-bit for Kitty boosted channels) [n_kq][128], key stats
    [n_kq/32][128] x2, value codes [n_vq][128], value stats [n_vq][4] x2.
    Kitty dynamic: each page's own index; pass a list as page_idx to receive
    the indices of the key pages."""
    kcodes = np.zeros((n_kq, D), np.uint8)
    ks = np.zeros((n_kq // 32, D), np.uint16)
    kz = np.zeros((n_kq // 32, D), np.uint16)
    vcodes = np.zeros((n_vq, D), np.uint8)
    vs = np.zeros((n_vq, 4), np.uint16)
    vz = np.zeros((n_vq, 4), np.uint16)
    for p in range((max(n_kq, n_vq) + PT - 1) // PT):
        blk = page_block(pool, int(table_row[p]), h, Hkv, scheme, nb)
        t0 = p * PT
        if t0 < n_kq:
            codes = key_codes(blk, scheme).astype(np.uint8)
            if scheme in KITTY_SCHEMES:
                pidx = idx if scheme == 1 else page_boost_index(blk, nb)
                if page_idx is not None:
                    page_idx.append(pidx)
                hi = key_high(blk, nb)
                for c in range(D):
                    if pidx[c] < nb:
                        codes[:, c] |= hi[:, pidx[c]] << 2
            kcodes[t0:t0 + PT] = codes
            s, z = key_stats(blk, scheme, nb)
            ks[t0 // 32:t0 // 32 + 2] = s
            kz[t0 // 32:t0 // 32 + 2] = z
        if t0 < n_vq:
            n = min(PT, n_vq - t0)
            vcodes[t0:t0 + n] = value_codes(blk, scheme, nb)[:n]
            s, z = value_stats(blk, scheme, nb)
            vs[t0:t0 + n] = s[:n]
            vz[t0:t0 + n] = z[:n]
    return kcodes, ks, kz, vcodes, vs, vz
