"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no quantization or attention arithmetic: it only draws
fp16 tensors and workload shapes.  Every tensor is a function of
(workload seed, purpose, request, KV head) so any slice can be regenerated
alone, bit for bit, on the host.

Recipe: float32 standard normals from ``numpy.random.default_rng``, outlier
key channels multiplied by a fixed factor in float32, then rounded to fp16
(round-to-nearest-even, numpy ``astype``).  Values cross as ``uint16`` bit
patterns.

Workloads (shapes of the decode batches the pages measure on; the pages'
own datasets and models are not used):
  1  one decode step, B=1, one head, D=128, context 1024; key channels
     {3, 77} x20.
  2  Llama-2-7B-shaped MHA: B=16, 32 heads, context 4096, four seeded
     outlier key channels per head x15 (shared by all requests); steps
     append one token each.
  3  Llama-3-8B-shaped GQA: B=64, 32 query heads over 8 KV heads, contexts
     drawn uniformly from [8192, 32768], four outlier channels per KV head
     x15, 64-token pages in a shuffled page table.
  4  Kitty: workload 2's shapes at context 32768, 16 of 128 key channels per
     head boosted to 4 bits (largest amax over the first 1024 context tokens
     of request 0).
  5  WitCert INT8 dither: B=32, 32 query / 8 KV heads, context 16384 plus
     one appended token, plain N(0,1).
  6  workload 4 with the Kitty boosted set chosen per 64-token page.
  7  workload 3 with 32 fp16 sink tokens per request.
  8  workload 4 with 32 boosted channels (Kitty-Pro).
  9  workload 4's shapes with 4-bit keys and values (KIVI-4).
 10  WitCert paging-safe storage: workload 5's shapes, keys with four seeded
     outlier RoPE pairs (channels i and i + 64, x15) that the four-pair
     bypass set should find.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# purposes (part of every seed)
_CTX_K, _CTX_V, _STEP_Q, _STEP_K, _STEP_V, _OUTLIERS, _LENGTHS, _PAGES, _QDEC = range(1, 10)


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    scheme: str            # "kivi2" | "kitty" | "witcert" | "kitty_dyn" | "kivi4" | "witcert_paged"
    B: int
    Hq: int
    Hkv: int
    D: int = 128
    G: int = 32
    R: int = 128
    VG: int = 32
    BLK: int = 256
    page_tokens: int = 64
    nb: int = 0            # Kitty boosted channels per head
    sink: int = 0          # leading tokens kept fp16 (keys and values)
    ctx: tuple = ()        # per-request context length before the first step
    outlier_ch: tuple = ()  # fixed channels (workload 1) or () for seeded
    n_outliers: int = 0
    outlier_pairs: bool = False  # seeded outliers are RoPE pairs (i, i + D/2)
    outlier_factor: float = 1.0
    steps: int = 1
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    @property
    def sm_scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.D)))


def _lengths3(B: int, lo: int, hi: int, seed: int) -> tuple:
    return tuple(int(v) for v in np.random.default_rng(seed).integers(lo, hi + 1, B))


def workload(wid: int, **over) -> Workload:
    """The workloads at full size; keyword overrides give scaled-down cases."""
    if wid == 1:
        w = dict(wid=1, name="kivi2-b1-h1-ctx1024", scheme="kivi2", B=1, Hq=1, Hkv=1,
                 ctx=(1024,), outlier_ch=(3, 77), outlier_factor=20.0, steps=1, seed=1)
    elif wid == 2:
        w = dict(wid=2, name="kivi2-mha-b16-h32-ctx4096", scheme="kivi2", B=16, Hq=32, Hkv=32,
                 ctx=(4096,) * 16, n_outliers=4, outlier_factor=15.0, steps=1000, seed=2)
    elif wid == 3:
        w = dict(wid=3, name="kivi2-gqa-b64-32q8kv-ctx8k-32k-paged", scheme="kivi2", B=64,
                 Hq=32, Hkv=8, ctx=_lengths3(64, 8192, 32768, 3), n_outliers=4,
                 outlier_factor=15.0, steps=1, seed=3)
    elif wid == 4:
        w = dict(wid=4, name="kitty-mha-b16-h32-ctx32768", scheme="kitty", B=16, Hq=32, Hkv=32,
                 ctx=(32768,) * 16, n_outliers=4, outlier_factor=15.0, nb=16, steps=1, seed=4)
    elif wid == 5:
        w = dict(wid=5, name="witcert-int8-b32-32q8kv-ctx16384", scheme="witcert", B=32, Hq=32,
                 Hkv=8, ctx=(16384,) * 32, steps=1, seed=5)
    elif wid == 6:
        # workload 4's shapes with the boosted set chosen per page
        w = dict(wid=6, name="kitty-dyn-mha-b16-h32-ctx32768", scheme="kitty_dyn", B=16, Hq=32,
                 Hkv=32, ctx=(32768,) * 16, n_outliers=4, outlier_factor=15.0, nb=16, steps=1,
                 seed=6)
    elif wid == 8:
        # Kitty-Pro: workload 4 with a quarter of the key channels boosted
        w = dict(wid=8, name="kitty-pro-mha-b16-h32-ctx32768", scheme="kitty", B=16, Hq=32,
                 Hkv=32, ctx=(32768,) * 16, n_outliers=4, outlier_factor=15.0, nb=32, steps=1,
                 seed=8)
    elif wid == 7:
        # workload 3's shapes and lengths with 32 fp16 sink tokens per request
        w = dict(wid=7, name="kivi2-sink32-gqa-b64-32q8kv-ctx8k-32k-paged", scheme="kivi2", B=64,
                 Hq=32, Hkv=8, ctx=_lengths3(64, 8192, 32768, 3), n_outliers=4,
                 outlier_factor=15.0, sink=32, steps=1, seed=7)
    elif wid == 10:
        # WitCert paging-safe storage at workload 5's shapes, 4 bypassed pairs
        w = dict(wid=10, name="witcert-paged-b32-32q8kv-ctx16384", scheme="witcert_paged", B=32,
                 Hq=32, Hkv=8, ctx=(16384,) * 32, n_outliers=4, outlier_pairs=True,
                 outlier_factor=15.0, nb=4, steps=1, seed=10)
    elif wid == 11:
        # a group of 8 query heads per KV head (64q/8kv), 32 requests with
        # lengths drawn like workload 3's (uniform over 8K..32K)
        w = dict(wid=11, name="kivi2-gqa8-b32-64q8kv-ctx8k-32k-paged", scheme="kivi2", B=32,
                 Hq=64, Hkv=8, ctx=_lengths3(32, 8192, 32768, 11), n_outliers=4,
                 outlier_factor=15.0, steps=1, seed=11)
    elif wid == 9:
        # KIVI-4: workload 4's shapes with 4-bit keys and values, no boosting
        w = dict(wid=9, name="kivi4-mha-b16-h32-ctx32768", scheme="kivi4", B=16, Hq=32,
                 Hkv=32, ctx=(32768,) * 16, n_outliers=4, outlier_factor=15.0, steps=1, seed=9)
    else:
        raise ValueError(wid)
    w.update(over)
    if "B" in over and "ctx" not in over:
        w["ctx"] = tuple(w["ctx"][i % len(w["ctx"])] for i in range(w["B"]))
    return Workload(**w)


def _rng(w: Workload, purpose: int, *ids: int) -> np.random.Generator:
    return np.random.default_rng([w.seed, purpose, *ids])


def to_fp16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x.astype(np.float16)).view(np.uint16)


def outlier_channels(w: Workload, kvh: int) -> tuple:
    """Fixed outlier key channels of one KV head (shared by every request)."""
    if w.outlier_ch:
        return tuple(w.outlier_ch)
    if w.n_outliers == 0:
        return ()
    if w.outlier_pairs:
        pr = _rng(w, _OUTLIERS, kvh).choice(w.D // 2, w.n_outliers, replace=False)
        return tuple(sorted(int(c) for i in pr for c in (i, i + w.D // 2)))
    ch = _rng(w, _OUTLIERS, kvh).choice(w.D, w.n_outliers, replace=False)
    return tuple(int(c) for c in sorted(ch))


def _draw(w: Workload, purpose: int, shape, ids, outliers=()) -> np.ndarray:
    x = _rng(w, purpose, *ids).standard_normal(shape, dtype=np.float32)
    if outliers:
        x[..., list(outliers)] *= np.float32(w.outlier_factor)
    return to_fp16_bits(x)


def context_kv(w: Workload, req: int, kvh: int, n: int | None = None):
    """Context keys/values of one (request, KV head): two uint16 [n][D]."""
    if n is None:
        n = w.ctx[req]
    K = _draw(w, _CTX_K, (n, w.D), (req, kvh), outlier_channels(w, kvh))
    V = _draw(w, _CTX_V, (n, w.D), (req, kvh))
    return K, V


def step_kv(w: Workload, step: int):
    """New key/value of every (request, KV head) at one decode step: [B][Hkv][D]."""
    K = np.empty((w.B, w.Hkv, w.D), np.uint16)
    for h in range(w.Hkv):
        K[:, h] = _draw(w, _STEP_K, (w.B, w.D), (step, h), outlier_channels(w, h))
    V = _draw(w, _STEP_V, (w.B, w.Hkv, w.D), (step,))
    return K, V


def step_q(w: Workload, step: int) -> np.ndarray:
    """Queries of one decode step: [B][Hq][D]."""
    return _draw(w, _STEP_Q, (w.B, w.Hq, w.D), (step,))


def page_permutation(w: Workload, n_pages: int) -> np.ndarray:
    """Seeded shuffle of physical page ids (the page table's randomness)."""
    return _rng(w, _PAGES).permutation(n_pages).astype(np.int32)


def kitty_calibration(w: Workload, kvh: int, n: int = 1024) -> np.ndarray:
    """Calibration slice for a static channel set (Kitty's boost set, WitCert's
    bypassed pairs): the first n context keys of request 0 for this KV head."""
    K, _ = context_kv(w, 0, kvh, n=min(n, w.ctx[0]))
    return K
