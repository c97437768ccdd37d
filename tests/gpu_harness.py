"""Shared set-up for the GPU parity tests: builds a device cache through the
C ABI and the matching oracle streams from the same seeded inputs."""
from __future__ import annotations

import numpy as np

from bit_kv_cache_kivi_amd import inputs
from layout_unpack import PT, WPT, gather_kivi, page_block, witcert_block, witcert_paged_block

SCHEME_ID = {"kivi2": 0, "kitty": 1, "witcert": 2, "kitty_dyn": 3, "kivi4": 4, "witcert_paged": 5}


class Case:
    """One workload on the GPU plus its oracle streams."""

    def __init__(self, w: inputs.Workload, extra_tokens: int = 0, split_pages: int = 0,
                 poison: bool = True, sample=None, flags: int = 0, sink: int | None = None,
                 kv_scale=(1.0, 1.0)):
        import torch
        from bit_kv_cache_kivi_amd import kvq
        from oracle import oracle as O
        self.torch, self.kvq, self.O = torch, kvq, O
        self.w = w
        self.kv_scale = kv_scale
        sink = w.sink if sink is None else sink
        self.S = sink
        self.sid = SCHEME_ID[w.scheme]
        self.pt = WPT if w.scheme == "witcert" else PT
        self.cap = max(w.ctx) + extra_tokens
        self.max_pages = (self.cap + self.pt - 1) // self.pt
        self.n_pages = w.B * self.max_pages
        perm = inputs.page_permutation(w, self.n_pages)
        self.table = perm.reshape(w.B, self.max_pages)
        # Kitty boost set: host oracle (for the oracle streams) and GPU kernel
        self.idx = None
        self.sample = sample if sample is not None else [(b, h) for b in range(w.B)
                                                          for h in range(w.Hkv)]
        if w.scheme == "kitty":
            self.idx = np.stack([O.kitty_select(inputs.kitty_calibration(w, h), w.nb)
                                 for h in range(w.Hkv)])
        self.bypass = None                           # WitCert paging-safe: bypass mask per head
        if w.scheme == "witcert_paged" and w.nb > 0:
            self.bypass = np.stack([O.witcert_select_pairs(inputs.kitty_calibration(w, h), w.nb)
                                    for h in range(w.Hkv)])
        layout = kvq.make_layout(w.scheme, w.B, w.Hq, w.Hkv, self.max_pages, self.n_pages,
                                 R=w.R, seed=self.seed, split_pages=split_pages, flags=flags,
                                 sink=sink,
                                 nb=w.nb if (w.nb or w.scheme == "witcert_paged") else None)
        self.cache = kvq.KVCache(layout, self.table, poison=poison)
        if w.scheme in ("kitty", "witcert_paged") and (w.scheme == "kitty" or w.nb > 0):
            calib = np.stack([inputs.kitty_calibration(w, h) for h in range(w.Hkv)])
            ct = torch.from_numpy(calib.view(np.float16)).cuda()
            if w.scheme == "kitty":
                self.cache.kitty_calibrate(ct)
            else:
                self.cache.witcert_calibrate(ct)
        # prefill, one request at a time (host inputs drawn by a thread pool)
        def gen(b):
            K = np.stack([self._kv(*inputs.context_kv(w, b, h))[0] for h in range(w.Hkv)])
            V = np.stack([self._kv(*inputs.context_kv(w, b, h))[1] for h in range(w.Hkv)])
            return K, V
        import concurrent.futures as cf
        with cf.ThreadPoolExecutor(min(16, w.B)) as ex:
            for b, (K, V) in enumerate(ex.map(gen, range(w.B))):
                if w.ctx[b] == 0:                    # a fresh cache already holds no token
                    continue
                Kt = torch.from_numpy(K.view(np.float16)).cuda()[None].contiguous()
                Vt = torch.from_numpy(V.view(np.float16)).cuda()[None].contiguous()
                lens = torch.tensor([w.ctx[b]], dtype=torch.int32, device="cuda")
                self.cache.prefill(b, Kt, Vt, lens)
        torch.cuda.synchronize()
        # oracle streams for the sampled (request, KV head) pairs
        self.streams = {}
        for b, h in self.sample:
            idx, slots = (None if self.idx is None else self.idx[h]), None
            if w.scheme == "witcert_paged":
                idx = None if self.bypass is None else self.bypass[h]
                t = np.arange(self.cap)
                slots = (self.table[b][t // PT].astype(np.uint64) * PT + (t % PT)).astype(np.uint64)
            s = O.Stream(self.sid, self.cap, D=128, G=w.G, R=w.R, VG=w.VG, BLK=w.BLK,
                         nb=w.nb, idx=idx, seed=self.seed, req=b, layer=0, kvh=h, sel=PT,
                         sink=sink, slots=slots)
            K, V = self._kv(*inputs.context_kv(w, b, h))
            s.prefill(K, V)
            self.streams[(b, h)] = s
        self.steps_done = 0

    def _kv(self, K, V):
        """The generated fp16 keys and values times the case's kv_scale (the
        same fp16 arrays go to the GPU and to the oracle)."""
        ks, vs = self.kv_scale
        def sc(x, f):
            if f == 1.0:
                return x
            return (x.view(np.float16).astype(np.float32) * np.float32(f)).astype(np.float16).view(np.uint16)
        return sc(K, ks), sc(V, vs)

    @property
    def seed(self) -> int:
        return 0x5EED_0000_0000_0000 | self.w.seed

    # ---------------------------------------------------------------------
    def step(self, decode: bool = True, kappa: float = 0.0):
        """flush -> append -> decode on both sides; returns (gpu_out, gpu_cert, q).
        Step ids run 0, 1, 2, ... (they seed the new tokens and queries)."""
        torch = self.torch
        w = self.w
        step_id = self.steps_done
        k, v = self._kv(*inputs.step_kv(w, step_id))
        q = inputs.step_q(w, step_id)
        self.cache.flush()
        kt = torch.from_numpy(k.view(np.float16)).cuda()
        vt = torch.from_numpy(v.view(np.float16)).cuda()
        self.cache.append(kt, vt)
        for (b, h), s in self.streams.items():
            s.flush()
            assert s.append(k[b, h], v[b, h]) == 0
        out = cert = None
        if decode:
            qt = torch.from_numpy(q.view(np.float16)).cuda()
            out = torch.full((w.B, w.Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
            cert = torch.full((w.B, w.Hq), float("nan"), dtype=torch.float32, device="cuda")
            self.cache.decode(qt, out, cert, sm_scale=w.sm_scale, kappa=kappa)
        torch.cuda.synchronize()
        self.steps_done += 1
        return out, cert, q

    def decode_now(self, step_id: int, kappa: float = 0.0):
        torch = self.torch
        w = self.w
        q = inputs.step_q(w, step_id)
        qt = torch.from_numpy(q.view(np.float16)).cuda()
        out = torch.full((w.B, w.Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
        cert = torch.full((w.B, w.Hq), float("nan"), dtype=torch.float32, device="cuda")
        self.cache.decode(qt, out, cert, sm_scale=w.sm_scale, kappa=kappa)
        torch.cuda.synchronize()
        return out, cert, q

    # ---------------------------------------------------------------------
    def oracle_decode(self, q: np.ndarray, b: int, h: int, kappa: float = 0.0):
        g = self.w.group
        return self.streams[(b, h)].decode(q[b, h * g:(h + 1) * g], self.w.sm_scale, kappa)

    def check_status(self):
        st = int(self.cache.status[0].item())
        assert st == 0, f"device status bits {st:#x}"

    def check_state(self):
        st = self.cache.state.cpu().numpy()
        for (b, h), s in self.streams.items():
            l, n_kq, _ = s.state
            assert (st[b, h, 0], st[b, h, 1]) == (l, n_kq), ((b, h), st[b, h], s.state)

    def check_store(self):
        """Bit-exact codes, statistics and fp16 windows against the oracle."""
        pool = self.cache.pool.cpu().numpy()
        w = self.w
        if w.scheme == "witcert_paged":
            return self._check_store_paged(pool)
        rk = self.cache.res_k.cpu().numpy().view(np.uint16)
        rv = self.cache.res_v.cpu().numpy().view(np.uint16)
        for (b, h), s in self.streams.items():
            l, n_kq, n_vq = s.state
            Kraw, Vraw = self._raw(s, l)
            if w.scheme == "witcert":
                okc, ovc = s.key_codes().view(np.int8), s.value_codes().view(np.int8)
                oks, _ = s.key_stats()
                ovs, _ = s.value_stats()
                for blk in range(n_kq // WPT):
                    kc, ks, vc, vs = witcert_block(page_block(pool, int(self.table[b, blk]), h,
                                                              w.Hkv, 2))
                    sl = slice(blk * WPT, (blk + 1) * WPT)
                    assert np.array_equal(kc, okc[sl]), ("wit key codes", b, h, blk)
                    assert np.array_equal(vc, ovc[sl]), ("wit value codes", b, h, blk)
                    assert np.array_equal(ks, oks[blk]) and np.array_equal(vs, ovs[blk])
                n = l - n_kq
                assert np.array_equal(rk[b, h, :n], Kraw[n_kq:l])
                assert np.array_equal(rv[b, h, :n], Vraw[n_kq:l])
                continue
            # pages hold quantized positions t - S; the sink tokens sit apart
            S = self.S
            qk, qv = max(0, n_kq - S), max(0, n_vq - S)
            pidx = []
            kc, ks, kz, vc, vs, vz = gather_kivi(pool, self.table[b], h, w.Hkv, self.sid, qk,
                                                 qv, None if self.idx is None else self.idx[h],
                                                 page_idx=pidx, nb=w.nb if w.nb else 16)
            if w.scheme == "kitty_dyn":               # each key page's boosted channel set
                ou = s.unit_index()
                for p in range(qk // PT):
                    assert np.array_equal(pidx[p], ou[p]), ("page boost index", b, h, p)
            okc, ovc = s.key_codes(), s.value_codes()
            oks, okz = s.key_stats()
            ovs, ovz = s.value_stats()
            assert np.array_equal(kc, okc[S:S + qk]), ("key codes", b, h)
            assert np.array_equal(ks, oks[:qk // 32]) and np.array_equal(kz, okz[:qk // 32])
            assert np.array_equal(vc, ovc[S:S + qv]), ("value codes", b, h)
            assert np.array_equal(vs, ovs[S:S + qv]) and np.array_equal(vz, ovz[S:S + qv])
            if S:
                ns = min(l, S)
                sk = self.cache.sink_k.cpu().numpy().view(np.uint16)
                sv = self.cache.sink_v.cpu().numpy().view(np.uint16)
                assert np.array_equal(sk[b, h, :ns], Kraw[:ns]), ("sink keys", b, h)
                assert np.array_equal(sv[b, h, :ns], Vraw[:ns]), ("sink values", b, h)
            assert np.array_equal(rk[b, h, :l - n_kq], Kraw[n_kq:l]), ("key residual", b, h)
            for t in range(n_vq, l):
                assert np.array_equal(rv[b, h, t % w.R], Vraw[t]), ("value window", b, h, t)

    def _check_store_paged(self, pool):
        """WitCert paging-safe: every token's int8 codes, group scales and
        bypass row against the oracle, bit for bit."""
        w = self.w
        for (b, h), s in self.streams.items():
            l, n_kq, _ = s.state
            assert n_kq == l
            Kraw, _ = self._raw(s, l)
            okc, ovc = s.key_codes().view(np.int8), s.value_codes().view(np.int8)
            oks, _ = s.key_stats()
            ovs, _ = s.value_stats()
            for p in range((l + PT - 1) // PT):
                n = min(PT, l - p * PT)
                kc, ks, vc, vs, kb = witcert_paged_block(
                    page_block(pool, int(self.table[b, p]), h, w.Hkv, 5, w.nb), w.nb)
                sl = slice(p * PT, p * PT + n)
                assert np.array_equal(kc[:n], okc[sl]), ("key codes", b, h, p)
                assert np.array_equal(vc[:n], ovc[sl]), ("value codes", b, h, p)
                assert np.array_equal(ks[:n], oks[sl]) and np.array_equal(vs[:n], ovs[sl]), \
                    ("scales", b, h, p)
                if self.bypass is not None:
                    ch = np.nonzero(self.bypass[h])[0]          # offsets in ascending channel order
                    assert np.array_equal(kb[:n, :len(ch)], Kraw[sl][:, ch]), ("bypass row", b, h, p)

    def _raw(self, s, l):
        # raw fp16 history, rebuilt from the seeded inputs
        b, h = [k for k, v in self.streams.items() if v is s][0]
        K0, V0 = self._kv(*inputs.context_kv(self.w, b, h))
        ks, vs = [K0], [V0]
        for i in range(self.steps_done):
            k, v = self._kv(*inputs.step_kv(self.w, i))
            ks.append(k[b, h][None])
            vs.append(v[b, h][None])
        return np.concatenate(ks)[:l], np.concatenate(vs)[:l]
