"""ctypes binding of libkvq.so (include/kvq.h).

Argument marshalling only: every step of the path runs in the HIP library.
PyTorch supplies device memory and the stream.  ``KVCache`` allocates the
caller-owned buffers the C ABI expects (pool, page table, state, residuals,
status, workspace) as torch tensors on ``cuda``.

Importing this module loads ``libkvq.so`` and fails loudly if it has not been
built (``python bit_kv_cache_kivi_amd/build.py``); there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkvq.so")

(KVQ_SCHEME_KIVI2, KVQ_SCHEME_KITTY, KVQ_SCHEME_WITCERT, KVQ_SCHEME_KITTY_DYN, KVQ_SCHEME_KIVI4,
 KVQ_SCHEME_WITCERT_PAGED) = 0, 1, 2, 3, 4, 5
SCHEMES = {"kivi2": KVQ_SCHEME_KIVI2, "kitty": KVQ_SCHEME_KITTY, "witcert": KVQ_SCHEME_WITCERT,
           "kitty_dyn": KVQ_SCHEME_KITTY_DYN, "kivi4": KVQ_SCHEME_KIVI4,
           "witcert_paged": KVQ_SCHEME_WITCERT_PAGED}

KVQ_OK, KVQ_EINVAL, KVQ_ENULL, KVQ_EALIGN, KVQ_ENOLAYOUT, KVQ_EWORKSPACE, KVQ_ELAUNCH, \
    KVQ_ENOSCRATCH = 0, -1, -2, -3, -4, -5, -6, -7
NOALLOC_SCRATCH_BYTES = 64 << 20          # KVQ_NOALLOC_SCRATCH_BYTES
STATUS_RESIDUAL_FULL, STATUS_CAPACITY, STATUS_UNMAPPED_PAGE, STATUS_BAD_LENGTH, STATUS_RANGE = \
    1, 2, 4, 8, 16
FLAG_GENERIC_STAGE1 = 1

EXPORTS = ("kvq_set_layout", "kvq_append_token", "kvq_flush_key_group",
           "kvq_decode_attention", "kvq_decode_attention_noalloc", "kvq_page_bytes",
           "kvq_page_tokens", "kvq_bytes_per_token", "kvq_workspace_bytes", "kvq_prefill",
           "kvq_kitty_calibrate", "kvq_witcert_calibrate", "kvq_set_stage1_events",
           "kvq_stage1_load_floor", "kvq_strerror")


class kvq_layout_t(C.Structure):
    _fields_ = [("scheme", C.c_int32), ("head_dim", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("batch", C.c_int32), ("group", C.c_int32),
                ("value_group", C.c_int32), ("residual", C.c_int32), ("block", C.c_int32),
                ("n_boost", C.c_int32), ("max_pages", C.c_int32), ("n_pages", C.c_int32),
                ("split_pages", C.c_int32), ("flags", C.c_int32), ("layer", C.c_uint32),
                ("seed", C.c_uint64), ("sink", C.c_int32), ("reserved", C.c_int32)]


class kvq_buffers_t(C.Structure):
    _fields_ = [("pool", C.c_void_p), ("page_table", C.c_void_p), ("state", C.c_void_p),
                ("res_k", C.c_void_p), ("res_v", C.c_void_p), ("boost_idx", C.c_void_p),
                ("status", C.c_void_p), ("sink_k", C.c_void_p), ("sink_v", C.c_void_p)]


class kvq_cache_t(C.Structure):
    _fields_ = [("layout", kvq_layout_t), ("bufs", kvq_buffers_t), ("page_tokens", C.c_int32),
                ("split_pages", C.c_int32), ("page_bytes", C.c_int64), ("magic", C.c_int32),
                ("reserved", C.c_int32), ("ev_stage1_begin", C.c_void_p),
                ("ev_stage1_end", C.c_void_p)]


_lib = None


def lib():
    """Load libkvq.so (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run bit_kv_cache_kivi_amd/build.py")
        L = C.CDLL(LIB_PATH)
        P, S = C.c_void_p, C.c_void_p
        L.kvq_set_layout.argtypes = [C.POINTER(kvq_cache_t), C.POINTER(kvq_layout_t),
                                     C.POINTER(kvq_buffers_t)]
        L.kvq_append_token.argtypes = [C.POINTER(kvq_cache_t), P, P, S]
        L.kvq_flush_key_group.argtypes = [C.POINTER(kvq_cache_t), S]
        L.kvq_decode_attention.argtypes = [C.POINTER(kvq_cache_t), P, P, P, C.c_float,
                                           C.c_float, P, C.c_size_t, S]
        L.kvq_stage1_load_floor.argtypes = [C.POINTER(kvq_cache_t), P, C.c_float, P, C.c_size_t, S]
        L.kvq_decode_attention_noalloc.argtypes = [C.POINTER(kvq_cache_t), P, P, P, C.c_float,
                                                   C.c_float, S]
        L.kvq_page_bytes.argtypes = [C.POINTER(kvq_layout_t)]
        L.kvq_page_bytes.restype = C.c_int64
        L.kvq_page_tokens.argtypes = [C.POINTER(kvq_layout_t)]
        L.kvq_page_tokens.restype = C.c_int32
        L.kvq_bytes_per_token.argtypes = [C.POINTER(kvq_layout_t)]
        L.kvq_bytes_per_token.restype = C.c_double
        L.kvq_workspace_bytes.argtypes = [C.POINTER(kvq_cache_t)]
        L.kvq_workspace_bytes.restype = C.c_size_t
        L.kvq_prefill.argtypes = [C.POINTER(kvq_cache_t), C.c_int32, C.c_int32, P, P,
                                  C.c_int64, P, S]
        L.kvq_kitty_calibrate.argtypes = [C.POINTER(kvq_cache_t), P, C.c_int32, P, S]
        L.kvq_witcert_calibrate.argtypes = [C.POINTER(kvq_cache_t), P, C.c_int32, P, S]
        L.kvq_set_stage1_events.argtypes = [C.POINTER(kvq_cache_t), P, P]
        L.kvq_strerror.argtypes = [C.c_int]
        L.kvq_strerror.restype = C.c_char_p
        _lib = L
    return _lib


class KVQError(RuntimeError):
    pass


def _check(rc: int, what: str):
    if rc != KVQ_OK:
        raise KVQError(f"{what}: {lib().kvq_strerror(rc).decode()} ({rc})")


# --------------------------------------------------------------------------
# thin wrappers with the C names
# --------------------------------------------------------------------------

def kvq_set_layout(layout: kvq_layout_t, bufs: kvq_buffers_t) -> kvq_cache_t:
    cache = kvq_cache_t()
    _check(lib().kvq_set_layout(C.byref(cache), C.byref(layout), C.byref(bufs)), "kvq_set_layout")
    return cache


def kvq_append_token(cache: kvq_cache_t, k_ptr: int, v_ptr: int, stream: int):
    _check(lib().kvq_append_token(C.byref(cache), k_ptr, v_ptr, stream), "kvq_append_token")


def kvq_flush_key_group(cache: kvq_cache_t, stream: int):
    _check(lib().kvq_flush_key_group(C.byref(cache), stream), "kvq_flush_key_group")


def kvq_decode_attention(cache: kvq_cache_t, q_ptr: int, out_ptr: int, cert_ptr: int | None,
                         sm_scale: float, kappa: float, ws_ptr: int, ws_bytes: int, stream: int):
    _check(lib().kvq_decode_attention(C.byref(cache), q_ptr, out_ptr, cert_ptr, sm_scale, kappa,
                                      ws_ptr, ws_bytes, stream), "kvq_decode_attention")


def kvq_decode_attention_noalloc(cache: kvq_cache_t, q_ptr: int, out_ptr: int,
                                 cert_ptr: int | None, sm_scale: float, kappa: float,
                                 stream: int):
    _check(lib().kvq_decode_attention_noalloc(C.byref(cache), q_ptr, out_ptr, cert_ptr, sm_scale,
                                              kappa, stream), "kvq_decode_attention_noalloc")


def kvq_stage1_load_floor(cache: kvq_cache_t, q_ptr: int, sm_scale: float, ws_ptr: int,
                          ws_bytes: int, stream: int):
    _check(lib().kvq_stage1_load_floor(C.byref(cache), q_ptr, sm_scale, ws_ptr, ws_bytes, stream),
           "kvq_stage1_load_floor")


def kvq_prefill(cache: kvq_cache_t, req0: int, n_req: int, k_ptr: int, v_ptr: int,
                ld_tokens: int, lengths_ptr: int, stream: int):
    _check(lib().kvq_prefill(C.byref(cache), req0, n_req, k_ptr, v_ptr, ld_tokens, lengths_ptr,
                             stream), "kvq_prefill")


def kvq_kitty_calibrate(cache: kvq_cache_t, calib_ptr: int, n_tokens: int, idx_ptr: int,
                        stream: int):
    _check(lib().kvq_kitty_calibrate(C.byref(cache), calib_ptr, n_tokens, idx_ptr, stream),
           "kvq_kitty_calibrate")


def kvq_witcert_calibrate(cache: kvq_cache_t, calib_ptr: int, n_tokens: int, idx_ptr: int,
                          stream: int):
    _check(lib().kvq_witcert_calibrate(C.byref(cache), calib_ptr, n_tokens, idx_ptr, stream),
           "kvq_witcert_calibrate")


def kvq_set_stage1_events(cache: kvq_cache_t, begin: int | None, end: int | None):
    _check(lib().kvq_set_stage1_events(C.byref(cache), begin, end), "kvq_set_stage1_events")


def kvq_workspace_bytes(cache: kvq_cache_t) -> int:
    return int(lib().kvq_workspace_bytes(C.byref(cache)))


def make_layout(scheme: str, B: int, Hq: int, Hkv: int, max_pages: int, n_pages: int,
                R: int = 128, seed: int = 0, layer: int = 0, split_pages: int = 0,
                nb: int | None = None, flags: int = 0, sink: int = 0) -> kvq_layout_t:
    s = SCHEMES[scheme]
    return kvq_layout_t(scheme=s, head_dim=128, n_q_heads=Hq, n_kv_heads=Hkv, batch=B, group=32,
                        value_group=32, residual=R, block=256,
                        n_boost=(16 if s in (KVQ_SCHEME_KITTY, KVQ_SCHEME_KITTY_DYN)
                                 else 4 if s == KVQ_SCHEME_WITCERT_PAGED else 0)
                        if nb is None else nb,
                        max_pages=max_pages, n_pages=n_pages, split_pages=split_pages,
                        flags=flags, layer=layer, seed=seed, sink=sink, reserved=0)


def page_bytes(layout: kvq_layout_t) -> int:
    return int(lib().kvq_page_bytes(C.byref(layout)))


def page_tokens(layout: kvq_layout_t) -> int:
    return int(lib().kvq_page_tokens(C.byref(layout)))


def bytes_per_token(layout: kvq_layout_t) -> float:
    return float(lib().kvq_bytes_per_token(C.byref(layout)))


# --------------------------------------------------------------------------
# buffer owner (torch tensors on the GPU)
# --------------------------------------------------------------------------

class KVCache:
    """Allocates the caller-owned buffers of one cache and holds its kvq_cache_t.

    page_table: int32 [B][max_pages] numpy array of physical page ids (the
    caller decides the mapping, e.g. a seeded permutation)."""

    def __init__(self, layout: kvq_layout_t, page_table: np.ndarray, device: str = "cuda",
                 boost_idx: np.ndarray | None = None, poison: bool = False):
        import torch
        self.torch = torch
        self.layout = layout
        self.device = device
        B, Hkv = layout.batch, layout.n_kv_heads
        self.page_bytes = page_bytes(layout)
        self.page_tokens = page_tokens(layout)
        W = 256 if layout.scheme == KVQ_SCHEME_WITCERT else layout.residual
        wtok = layout.scheme == KVQ_SCHEME_WITCERT_PAGED    # no fp16 residual buffers
        fill = 0xFF if poison else 0
        self.pool = torch.full((layout.n_pages * Hkv * self.page_bytes,), fill, dtype=torch.uint8,
                               device=device)
        pt = np.ascontiguousarray(page_table, dtype=np.int32).reshape(B, layout.max_pages)
        self.page_table = torch.from_numpy(pt).to(device)
        self.state = torch.zeros((B, Hkv, 4), dtype=torch.int32, device=device)
        self.res_k = None if wtok else torch.zeros((B, Hkv, W, 128), dtype=torch.int16, device=device)
        self.res_v = None if wtok else torch.zeros((B, Hkv, W, 128), dtype=torch.int16, device=device)
        self.status = torch.zeros((4,), dtype=torch.int32, device=device)
        S = layout.sink
        self.sink_k = torch.zeros((B, Hkv, S, 128), dtype=torch.int16, device=device) if S else None
        self.sink_v = torch.zeros((B, Hkv, S, 128), dtype=torch.int16, device=device) if S else None
        if layout.scheme == KVQ_SCHEME_KITTY or (wtok and layout.n_boost > 0):
            sentinel = layout.n_boost + 1 if not wtok else 2 * layout.n_boost + 1
            idx = np.full((Hkv, 128), sentinel, np.uint8) if boost_idx is None else boost_idx
            self.boost_idx = torch.from_numpy(np.ascontiguousarray(idx, np.uint8)).to(device)
        else:
            self.boost_idx = None
        self.bufs = kvq_buffers_t(
            pool=self.pool.data_ptr(), page_table=self.page_table.data_ptr(),
            state=self.state.data_ptr(),
            res_k=None if wtok else self.res_k.data_ptr(),
            res_v=None if wtok else self.res_v.data_ptr(),
            boost_idx=self.boost_idx.data_ptr() if self.boost_idx is not None else None,
            status=self.status.data_ptr(),
            sink_k=self.sink_k.data_ptr() if S else None, sink_v=self.sink_v.data_ptr() if S else None)
        self.cache = kvq_set_layout(layout, self.bufs)
        self.ws_bytes = kvq_workspace_bytes(self.cache)
        self.workspace = torch.empty((self.ws_bytes,), dtype=torch.uint8, device=device)

    def stream(self) -> int:
        return self.torch.cuda.current_stream().cuda_stream

    # the four calls ---------------------------------------------------------
    def flush(self):
        kvq_flush_key_group(self.cache, self.stream())

    def append(self, k, v):
        assert k.dtype == self.torch.float16 and k.is_contiguous() and v.is_contiguous()
        kvq_append_token(self.cache, k.data_ptr(), v.data_ptr(), self.stream())

    def decode(self, q, out, cert=None, sm_scale: float = 1.0 / 128 ** 0.5, kappa: float = 0.0):
        assert q.dtype == self.torch.float16 and q.is_contiguous()
        assert out.dtype == self.torch.float32 and out.is_contiguous()
        kvq_decode_attention(self.cache, q.data_ptr(), out.data_ptr(),
                             None if cert is None else cert.data_ptr(), sm_scale, kappa,
                             self.workspace.data_ptr(), self.ws_bytes, self.stream())

    def decode_noalloc(self, q, out, cert=None, sm_scale: float = 1.0 / 128 ** 0.5,
                       kappa: float = 0.0):
        """decode() through kvq_decode_attention_noalloc: the library's
        per-device scratch array instead of this cache's workspace."""
        assert q.dtype == self.torch.float16 and q.is_contiguous()
        assert out.dtype == self.torch.float32 and out.is_contiguous()
        kvq_decode_attention_noalloc(self.cache, q.data_ptr(), out.data_ptr(),
                                     None if cert is None else cert.data_ptr(), sm_scale, kappa,
                                     self.stream())

    def stage1_load_floor(self, q, sm_scale: float = 1.0 / 128 ** 0.5):
        """The group kernel's load-only stage 1 on the current state (a
        measurement aid): overwrites this cache's workspace, nothing else."""
        assert q.dtype == self.torch.float16 and q.is_contiguous()
        kvq_stage1_load_floor(self.cache, q.data_ptr(), sm_scale, self.workspace.data_ptr(),
                              self.ws_bytes, self.stream())

    def prefill(self, req0: int, K, V, lengths):
        """K, V: fp16 [n_req][Hkv][ld][128] on the device; lengths int32 [n_req]."""
        assert K.is_contiguous() and V.is_contiguous() and K.dtype == self.torch.float16
        kvq_prefill(self.cache, req0, K.shape[0], K.data_ptr(), V.data_ptr(), K.shape[2],
                    lengths.data_ptr(), self.stream())

    def kitty_calibrate(self, calib):
        """calib: fp16 [Hkv][T][128] on the device; fills the boost index."""
        assert self.boost_idx is not None
        kvq_kitty_calibrate(self.cache, calib.data_ptr(), calib.shape[1],
                            self.boost_idx.data_ptr(), self.stream())

    def witcert_calibrate(self, calib):
        """calib: fp16 [Hkv][T][128] on the device; fills the bypass index
        (WitCert paging-safe storage)."""
        assert self.boost_idx is not None
        kvq_witcert_calibrate(self.cache, calib.data_ptr(), calib.shape[1],
                              self.boost_idx.data_ptr(), self.stream())

    def status_word(self) -> int:
        return int(self.status[0].item())
