#!/usr/bin/env python3
"""Quantized-KV decode attention benchmark on one MI355X.

One step = kvq_flush_key_group -> kvq_append_token -> kvq_decode_attention for
one attention layer of a whole decode batch (every request appends one token
and attends once).  Inputs are seeded synthetic fp16 tensors shaped like the
pages' workloads (bit_kv_cache_kivi_amd/inputs.py); the cache is prefilled
and every step's q/k/v is resident in HBM before the timed region.

Prints ONE JSON line: effective KV GB/s (algorithmic bytes of the step / step
time) as `value`, with tokens/s, the stage-1 kernel's roofline (HIP events
around it inside the timed steps) and the CPU oracle timed on a bounded
sample of the same workload on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1..11]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from bit_kv_cache_kivi_amd import inputs  # noqa: E402

METRIC = "quantized-KV decode attn: effective KV GB/s (% of HBM peak) + tokens/s, 1 GPU"
HBM_PEAK_GBS = 8000.0
# host CPUs a one-GPU job is given (the oracle baseline runs on as many threads)
BOX_CPU_SHARE = 16
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12         # full-rate 32-bit VALU lane ops, all CUs
PHILOX_VALU_OPS = 40                              # per Philox4x32-10 call on gfx950 (see below)


def witcert_ops_per_call(qpk: int) -> int:
    """Algorithmic VALU lane operations per Philox call (= per 4 quantized
    elements of one side), counted in operations gfx950 runs at full rate:
    the generator, 10 rounds x (2 32x32->64 multiply-adds + 2 three-input
    XORs), the key schedule being per block and scalar; then per element the
    dither from its word (shift, convert), the dequantization (code convert,
    code + 1/2, fused subtraction of the dither, times the scale) and one FMA
    per query head (the score on the key side, P.V on the value side)."""
    return PHILOX_VALU_OPS + 4 * (2 + 4 + qpk)
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["bit_kv_cache_kivi_amd/csrc/kvq_decode.hip",
                  "bit_kv_cache_kivi_amd/csrc/kvq_common.hpp"]


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic byte accounts (per (request, KV head) at decode time)
# ---------------------------------------------------------------------------

def key_q_bytes(scheme: str, n: int, nb: int = 16) -> int:
    """Quantized key bytes of n tokens: codes + stats (48 B) + the Kitty high
    plane (nb/4 B), and for Kitty dynamic the channel ids of each 64-token
    page touched (max(16, nb) B); KIVI-4: 64 B of codes + 16 B of stats."""
    if scheme == "kivi4":
        return n * 80
    if scheme == "kitty_dyn":
        return n * (48 + nb // 4) + ((n + 63) // 64) * max(16, nb)
    return n * (48 + nb // 4) if scheme == "kitty" else n * 48


def value_q_bytes(scheme: str) -> int:
    """Quantized value bytes per token: codes (2 or 4 bits x 128) + 4 groups'
    fp16 (scale, zero)."""
    return 80 if scheme == "kivi4" else 48


def kivi_bytes(l: int, n_kq: int, R: int, qpk: int, scheme: str, sink: int = 0,
               nb: int = 16) -> dict:
    """n_kq: absolute (keys below it are quantized or sink tokens)."""
    ns = min(l, sink)                              # fp16 sink tokens, keys and values
    n_vq = max(0, l - sink - R)                    # quantized values after the sink
    kq = max(0, n_kq - sink)                       # quantized keys after the sink
    paged = key_q_bytes(scheme, n_vq, nb) + n_vq * value_q_bytes(scheme)
    window = key_q_bytes(scheme, kq - n_vq, nb) + (l - max(n_kq, ns)) * 256 + (l - ns - n_vq) * 256
    window += ns * 512
    qo = qpk * (256 + 512)
    table = ((l + 63) // 64) * 4
    # stage 1 streams the paged prefix and, as one more split, the fp16 window
    return dict(stage1=paged + window, decode=paged + window + qo + table)


def witcert_paged_bytes(l: int, qpk: int, nb: int) -> dict:
    """Every token quantized: 136 B per side (int8 codes + four fp16 group
    scales) + 16 B of bypassed key values when there are bypassed pairs."""
    paged = l * (272 + (16 if nb > 0 else 0))
    qo = qpk * (256 + 512 + 4)
    table = ((l + 63) // 64) * 4
    return dict(stage1=paged, decode=paged + qo + table)


def witcert_bytes(l: int, n_q: int, qpk: int) -> dict:
    paged = n_q * 258
    window = (l - n_q) * 512
    qo = qpk * (256 + 512 + 4)
    table = ((l + 255) // 256) * 4
    return dict(stage1=paged + window, decode=paged + window + qo + table)


def write_bytes(w: inputs.Workload, l_before: int, n_kq_before: int) -> int:
    """Append (+ value pack) and flush-if-due bytes of one (request, KV head)."""
    if w.scheme == "witcert_paged":    # new k, v in; the token's record out
        return 512 + 272 + (16 if w.nb > 0 else 0)
    b = 512 + 512                      # new k, v in; fp16 windows out
    if w.scheme == "witcert":
        if l_before - n_kq_before == w.BLK:
            b += 2 * w.BLK * 256 + 2 * (w.BLK * 128 + 256)
        return b
    if l_before < w.sink:
        return b                       # a sink token: fp16 only
    if l_before - w.sink >= w.R:
        b += 256 + value_q_bytes(w.scheme)     # value leaving the window, its codes + stats
    if l_before - n_kq_before == w.R:
        b += w.R * 256 + key_q_bytes(w.scheme, w.R, w.nb or 16)
    return b


def state_after_prefill(w: inputs.Workload, l0: int):
    if w.scheme == "witcert_paged":
        return l0, l0
    W = w.BLK if w.scheme == "witcert" else w.R
    if l0 <= w.sink:
        return l0, l0
    lq = l0 - w.sink
    r = ((lq - 1) % W) + 1
    return l0, l0 - r


def step_state(w: inputs.Workload, l: int, n_kq: int):
    if w.scheme == "witcert_paged":
        return l + 1, l + 1
    W = w.BLK if w.scheme == "witcert" else w.R
    if l < w.sink:
        return l + 1, l + 1
    if l - n_kq == W:
        n_kq += W
    return l + 1, n_kq


def step_bytes(w: inputs.Workload, states):
    """states: list over requests of (l, n_kq) before the step.  Returns
    (total algorithmic bytes of the step, stage-1 bytes, new states)."""
    tot = 0
    s1 = 0
    new = []
    for (l, n_kq) in states:
        wb = write_bytes(w, l, n_kq)
        l2, k2 = step_state(w, l, n_kq)
        if w.scheme == "witcert":
            d = witcert_bytes(l2, k2, w.group)
        elif w.scheme == "witcert_paged":
            d = witcert_paged_bytes(l2, w.group, w.nb)
        else:
            d = kivi_bytes(l2, k2, w.R, w.group, w.scheme, w.sink, w.nb or 16)
        tot += w.Hkv * (wb + d["decode"])
        s1 += w.Hkv * d["stage1"]
        new.append((l2, k2))
    return tot, s1, new


# ---------------------------------------------------------------------------
# GPU side
# ---------------------------------------------------------------------------

def gen_request(w: inputs.Workload, b: int):
    K = np.stack([inputs.context_kv(w, b, h)[0] for h in range(w.Hkv)])
    V = np.stack([inputs.context_kv(w, b, h)[1] for h in range(w.Hkv)])
    return K, V


def setup_gpu(w: inputs.Workload, extra: int, split_pages: int):
    import torch
    from bit_kv_cache_kivi_amd import kvq
    pt = 256 if w.scheme == "witcert" else 64
    cap = max(w.ctx) + extra
    max_pages = (cap + pt - 1) // pt
    n_pages = w.B * max_pages
    table = inputs.page_permutation(w, n_pages).reshape(w.B, max_pages)
    layout = kvq.make_layout(w.scheme, w.B, w.Hq, w.Hkv, max_pages, n_pages, R=w.R,
                             seed=0x5EED_0000_0000_0000 | w.seed, split_pages=split_pages,
                             sink=w.sink, nb=w.nb if (w.nb or w.scheme == "witcert_paged") else None)
    cache = kvq.KVCache(layout, table)
    if w.scheme == "kitty" or (w.scheme == "witcert_paged" and w.nb > 0):
        calib = np.stack([inputs.kitty_calibration(w, h) for h in range(w.Hkv)])
        ct = torch.from_numpy(calib.view(np.float16)).cuda()
        if w.scheme == "kitty":
            cache.kitty_calibrate(ct)
        else:
            cache.witcert_calibrate(ct)
    threads = min(16, os.cpu_count() or 1)
    t0 = time.time()
    with cf.ThreadPoolExecutor(threads) as ex:
        futs = {b: ex.submit(gen_request, w, b) for b in range(min(w.B, threads))}
        nxt = len(futs)
        for b in range(w.B):
            K, V = futs.pop(b).result()
            if nxt < w.B:
                futs[nxt] = ex.submit(gen_request, w, nxt)
                nxt += 1
            Kt = torch.from_numpy(K.view(np.float16)).cuda(non_blocking=False)[None]
            Vt = torch.from_numpy(V.view(np.float16)).cuda(non_blocking=False)[None]
            lens = torch.tensor([w.ctx[b]], dtype=torch.int32, device="cuda")
            cache.prefill(b, Kt.contiguous(), Vt.contiguous(), lens)
    torch.cuda.synchronize()
    if cache.status_word() != 0:
        raise RuntimeError(f"prefill status {cache.status_word():#x}")
    log(f"prefill of {w.B} requests x {w.Hkv} KV heads done in {time.time() - t0:.1f}s")
    return cache


def event_steps(steps: int, every: int) -> list:
    """The timed steps whose stage-1 launch is bracketed by HIP events."""
    return [j for j in range(steps) if j % max(1, every) == 0]


def run_gpu(w: inputs.Workload, steps: int, warmup: int, split_pages: int, copies: int = 1,
            settle_s: float = 0.06, latency_steps: int = 0, event_every: int = 4,
            floor_launches: int = 0):
    """copies > 1: that many independent caches of the workload, used in turn
    (step i on copy i mod copies), so that no cache stays resident in the
    memory-side cache between its steps (a cold-cache figure).

    settle_s: before the warm-up steps, decode-only passes over the caches
    (they read the caches and change no state) for about this long.  The GPU
    idles during the host-side prefill and needs some 20 ms of work to return
    to its working clock; without this the few timed steps of a short run
    would measure that ramp instead of the kernels.

    event_every: HIP events bracket the stage-1 launch of every event_every-th
    timed step (event_steps): recording them costs the stream about 5 us of
    a step on this chip, so bracketing every step would slow the timed loop.

    latency_steps: after the timed steps, that many more steps one at a time,
    each bracketed by events on the stream and followed by a host
    synchronisation (the latency of one whole step: flush, append, decode).

    floor_launches: after the timed steps (group kernel only), that many
    launches of its load-only copy (kvq_stage1_load_floor) on the state the
    timed steps left, each bracketed by the same stage-1 events: the floor of
    the group kernel's access pattern."""
    import torch
    from bit_kv_cache_kivi_amd import kvq
    n = steps + warmup + latency_steps
    caches = [setup_gpu(w, extra=n + 8, split_pages=split_pages) for _ in range(copies)]
    # every step's inputs resident in HBM before timing
    ks, vs, qs = [], [], []
    for i in range(n):
        k, v = inputs.step_kv(w, i)
        ks.append(torch.from_numpy(k.view(np.float16)).cuda())
        vs.append(torch.from_numpy(v.view(np.float16)).cuda())
        qs.append(torch.from_numpy(inputs.step_q(w, i).view(np.float16)).cuda())
    out = torch.empty((w.B, w.Hq, 128), dtype=torch.float32, device="cuda")
    cert = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    sampled = event_steps(steps, event_every)
    ev1 = {j: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for j in sampled}
    kappa = 1.0 if w.scheme in ("witcert", "witcert_paged") else 0.0
    for a, b in ev1.values():   # torch creates the HIP event at its first record
        a.record()
        b.record()
    torch.cuda.synchronize()
    assert all(a.cuda_event and b.cuda_event for a, b in ev1.values())

    def one(i, evs=None):
        cache = caches[i % copies]
        j = i // copies                     # this copy's own step number
        if evs is not None:
            kvq.kvq_set_stage1_events(cache.cache, evs[0].cuda_event, evs[1].cuda_event)
        else:
            kvq.kvq_set_stage1_events(cache.cache, None, None)
        cache.flush()
        cache.append(ks[j], vs[j])
        cache.decode(qs[j], out, cert, sm_scale=w.sm_scale, kappa=kappa)

    n_settle = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < settle_s:
        for _ in range(20):
            caches[n_settle % copies].decode(qs[0], out, cert, sm_scale=w.sm_scale, kappa=kappa)
            n_settle += 1
        torch.cuda.synchronize()
    settle = {"decode_passes": n_settle, "ms": round((time.perf_counter() - t_settle) * 1e3, 1)}
    for i in range(warmup):
        one(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(steps):
        one(warmup + j, ev1.get(j))
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    for cache in caches:
        kvq.kvq_set_stage1_events(cache.cache, None, None)
        st = cache.status_word()
        if st != 0:
            raise RuntimeError(f"device status {st:#x}")
    if not torch.isfinite(out).all():
        raise RuntimeError("non-finite output")
    s1_ms = [ev1[j][0].elapsed_time(ev1[j][1]) for j in sampled]
    floor_ms = []
    if floor_launches:
        fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(floor_launches + 2)]
        for a, b in fev:
            a.record()
            b.record()
        torch.cuda.synchronize()
        cache = caches[(warmup + steps - 1) % copies]
        for a, b in fev:                    # the first two warm the copy up, untimed
            kvq.kvq_set_stage1_events(cache.cache, a.cuda_event, b.cuda_event)
            cache.stage1_load_floor(qs[0], sm_scale=w.sm_scale)
        kvq.kvq_set_stage1_events(cache.cache, None, None)
        torch.cuda.synchronize()
        floor_ms = [a.elapsed_time(b) for a, b in fev[2:]]
        if cache.status_word() != 0:
            raise RuntimeError(f"device status {cache.status_word():#x}")
    lat = None
    if latency_steps:
        dev_us, host_us = [], []
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(latency_steps)]
        for j, (a, b) in enumerate(pairs):
            t1 = time.perf_counter()
            a.record()
            one(warmup + steps + j)
            b.record()
            b.synchronize()
            host_us.append((time.perf_counter() - t1) * 1e6)
            dev_us.append(a.elapsed_time(b) * 1e3)
        for cache in caches:
            if cache.status_word() != 0:
                raise RuntimeError(f"device status {cache.status_word():#x}")
        lat = {"steps": latency_steps,
               "device_us_median": round(float(np.median(dev_us)), 2),
               "device_us_p90": round(float(np.percentile(dev_us, 90)), 2),
               "device_us_min": round(float(np.min(dev_us)), 2),
               "host_us_median": round(float(np.median(host_us)), 2),
               "host_us_p90": round(float(np.percentile(host_us, 90)), 2)}
    del stream
    return dt, s1_ms, settle, lat, floor_ms


# ---------------------------------------------------------------------------
# CPU oracle baseline (bounded sample of the same workload)
# ---------------------------------------------------------------------------

def cpu_baseline(w: inputs.Workload, warmup: int, target_s: float = 15.0, threads: int = 0,
                 n_pairs: int = 0):
    from oracle import oracle as O
    sid = {"kivi2": O.KIVI, "kitty": O.KITTY, "witcert": O.WITCERT, "kitty_dyn": O.KITTY_DYN,
           "kivi4": O.KIVI4, "witcert_paged": O.WITCERT_TOK}[w.scheme]
    affinity = len(os.sched_getaffinity(0))
    if threads <= 0:
        # the host CPUs a one-GPU job is given (16) where the process may
        # use more; all of them where it may use fewer
        threads = max(1, min(BOX_CPU_SHARE, affinity))
    idx = None
    if w.scheme == "kitty":
        idx = [O.kitty_select(inputs.kitty_calibration(w, h), w.nb) for h in range(w.Hkv)]
    if w.scheme == "witcert_paged" and w.nb > 0:     # bypass masks (slots: token index)
        idx = [O.witcert_select_pairs(inputs.kitty_calibration(w, h), w.nb) for h in range(w.Hkv)]
    # the whole step (every request and KV head) unless a smaller sample is asked for
    pairs = ([(b, b % w.Hkv) for b in range(min(n_pairs, w.B))] if n_pairs > 0
             else [(b, h) for b in range(w.B) for h in range(w.Hkv)])
    seed = 0x5EED_0000_0000_0000 | w.seed

    def make(pair):
        b, h = pair
        s = O.Stream(sid, w.ctx[b] + warmup + 210, G=w.G, R=w.R, VG=w.VG, BLK=w.BLK, nb=w.nb,
                     idx=None if idx is None else idx[h], seed=seed, req=b, kvh=h,
                     sink=w.sink)
        K, V = inputs.context_kv(w, b, h)
        s.prefill(K, V)
        return s, b, h

    def run(item, k, v, q):
        s, b, h = item
        s.flush()
        s.append(k[b, h], v[b, h])
        s.decode(q[b, h * w.group:(h + 1) * w.group], w.sm_scale,
                 1.0 if w.scheme in ("witcert", "witcert_paged") else 0.0)

    # rounds of one flush/append/decode step on every sampled pair, until the
    # timed work reaches about target_s (at least one round; at most max_rounds)
    max_rounds = 200
    with cf.ThreadPoolExecutor(threads) as ex:
        items = list(ex.map(make, pairs))
        states = [state_after_prefill(w, w.ctx[b]) for (b, h) in pairs]
        total_t = 0.0
        done_bytes = 0
        rounds = 0
        while rounds < max_rounds and total_t < target_s:
            k, v = inputs.step_kv(w, warmup + rounds)
            q = inputs.step_q(w, warmup + rounds)
            t0 = time.perf_counter()
            list(ex.map(lambda it: run(it, k, v, q), items))
            total_t += time.perf_counter() - t0
            for i, (l, n_kq) in enumerate(states):
                wb = write_bytes(w, l, n_kq)
                l2, k2 = step_state(w, l, n_kq)
                d = (witcert_bytes(l2, k2, w.group) if w.scheme == "witcert"
                     else witcert_paged_bytes(l2, w.group, w.nb) if w.scheme == "witcert_paged"
                     else kivi_bytes(l2, k2, w.R, w.group, w.scheme, w.sink, w.nb or 16))
                done_bytes += wb + d["decode"]
                states[i] = (l2, k2)
            rounds += 1
    done_pairs = len(pairs) * rounds
    gbs = done_bytes / total_t / 1e9
    whole = len(pairs) == w.B * w.Hkv
    what = ("every (request, KV head) pair of the workload, i.e. whole steps at full shape" if whole
            else f"{len(pairs)} (request, KV head) pairs of the workload (one per request)")
    return {"value": gbs, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{what} x {rounds} flush/append/decode steps ({done_bytes / 1e6:.1f} MB "
                      f"algorithmic), {total_t:.1f}s on {threads} host threads",
            "affinity_cpus": affinity, "lscpu": lscpu_counts(),
            "step_s": round(total_t / rounds, 3) if whole else None,
            "tokens_per_s_equiv": done_pairs / w.Hkv / total_t}


def lscpu_counts() -> dict:
    """Sockets, cores and hardware threads of the host, as lscpu reports them."""
    try:
        out = subprocess.run(["lscpu", "-p=SOCKET,CORE,CPU"], capture_output=True, text=True,
                             timeout=10).stdout
    except (OSError, subprocess.SubprocessError):
        return {}
    rows = [ln.split(",") for ln in out.splitlines() if ln and not ln.startswith("#")]
    return {"sockets": len({r[0] for r in rows}), "cores": len({(r[0], r[1]) for r in rows}),
            "cpus": len(rows)}


# ---------------------------------------------------------------------------

def source_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_entry(kernel: str, workload: str):
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    e = data.get(f"{kernel}@{workload}")
    if not e or e.get("source_sha") != source_sha():
        return None
    return e.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--split-pages", type=int, default=0)
    ap.add_argument("--cold", action="store_true",
                    help="two cache copies used in turn, so the memory-side cache holds neither")
    ap.add_argument("--settle-ms", type=float, default=80.0,
                    help="decode-only passes before the warm-up steps, to bring the clock up")
    ap.add_argument("--event-every", type=int, default=4,
                    help="bracket the stage-1 launch of every N-th timed step with HIP events")
    ap.add_argument("--latency", type=int, default=-1,
                    help="steps timed one at a time after the timed loop (default: 200 for "
                         "workload 1, else 0)")
    ap.add_argument("--floor-launches", type=int, default=8,
                    help="launches of the group kernel's load-only copy after the timed steps "
                         "(0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 1 GiB (scales FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        x = torch.ones(1 << 28, dtype=torch.float32, device="cuda")      # 1 GiB
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": x.numel() * 4, "copies": 3}))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)
    w = inputs.workload(args.workload)
    log(f"workload {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} ctx mean "
        f"{np.mean(w.ctx):.0f}, steps={args.steps} warmup={args.warmup}")
    copies = 2 if args.cold else 1
    lat_steps = args.latency if args.latency >= 0 else (200 if args.workload == 1 else 0)
    group_kernel = w.scheme == "kivi2" and w.group in (2, 4, 8)
    dt, s1_ms, settle, lat, floor_ms = run_gpu(w, args.steps, args.warmup, args.split_pages, copies,
                                               args.settle_ms * 1e-3, lat_steps, args.event_every,
                                               args.floor_launches if group_kernel else 0)
    sampled = set(event_steps(args.steps, args.event_every))

    # algorithmic bytes of the timed steps (step i advances copy i mod copies)
    cstates = [[state_after_prefill(w, l) for l in w.ctx] for _ in range(copies)]
    for i in range(args.warmup):
        _, _, cstates[i % copies] = step_bytes(w, cstates[i % copies])
    tot = 0
    s1_bytes = []
    s1_calls = []
    for i in range(args.warmup, args.warmup + args.steps):
        states = cstates[i % copies]
        nxt = [step_state(w, l, k) for (l, k) in states]
        if w.scheme == "witcert":        # tokens of the quantized blocks x quads x sides
            s1_calls.append(sum(w.Hkv * 2 * (n_kq // w.BLK) * w.BLK * (w.D // 4) for (_, n_kq) in nxt))
        elif w.scheme == "witcert_paged":   # every token
            s1_calls.append(sum(w.Hkv * 2 * l * (w.D // 4) for (l, _) in nxt))
        else:
            s1_calls.append(0)
        b, s1, cstates[i % copies] = step_bytes(w, states)
        tot += b
        if i - args.warmup in sampled:     # the launches the events timed
            s1_bytes.append(s1)
        else:
            s1_calls.pop()
    gbs = tot / dt / 1e9
    ms_step = dt / args.steps * 1e3
    s1_avg_ms = float(np.mean(s1_ms))
    s1_gbs = float(np.mean(s1_bytes)) / (s1_avg_ms * 1e-3) / 1e9
    kernel = ("stage1_witcert" if w.scheme == "witcert" else
              "stage1_witcert_paged" if w.scheme == "witcert_paged" else
              "stage1_gqa4_mfma" if group_kernel else "stage1_head_mfma")
    if w.scheme in ("witcert", "witcert_paged"):
        # VALU bound: Philox4x32-10 calls (one per token, channel quad and
        # side of every quantized block) x the algorithmic VALU operations per
        # call, against 256 CUs x 64 lanes x 2.4 GHz of full-rate VALU ops
        calls = float(np.mean(s1_calls))
        ops_call = witcert_ops_per_call(w.group)
        tops = calls * ops_call / (s1_avg_ms * 1e-3) / 1e12
        roof = {"kernel": kernel, "bound": "alu", "achieved": round(tops, 2),
                "peak": VALU_PEAK_TOPS, "unit": "TOP/s",
                "frac": round(tops / VALU_PEAK_TOPS, 4),
                "valu_ops_per_philox_call": ops_call,
                "traffic": traffic_entry(kernel, w.name),
                "avg_launch_us": round(s1_avg_ms * 1e3, 2),
                "timed_launches": len(s1_ms),
                "median_launch_us": round(float(np.median(s1_ms)) * 1e3, 2),
                "philox_calls_per_launch": int(calls),
                "algorithmic_bytes_per_launch": int(np.mean(s1_bytes)),
                "hbm_gbs": round(s1_gbs, 1)}
    else:
        roof = {"kernel": kernel, "bound": "hbm",
                "achieved": round(s1_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(s1_gbs / HBM_PEAK_GBS, 4),
                "traffic": traffic_entry(kernel, w.name),
                "avg_launch_us": round(s1_avg_ms * 1e3, 2),
                "timed_launches": len(s1_ms),
                "median_launch_us": round(float(np.median(s1_ms)) * 1e3, 2),
                "algorithmic_bytes_per_launch": int(np.mean(s1_bytes))}
        if floor_ms:
            # the same launch with the page step's arithmetic taken out
            # (kvq_stage1_load_floor), on the state the timed steps left
            roof["load_floor_us"] = round(float(np.mean(floor_ms)) * 1e3, 2)
            roof["of_load_floor"] = round(float(np.mean(floor_ms)) / s1_avg_ms, 4)
    rec = {"metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": {"witcert": "i8+f32", "witcert_paged": "i8+f32", "kivi4": "u4+f32"}.get(w.scheme, "u2+f32"),
           "data": "synthetic",
           "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                      "head_dim": w.D, "ctx_mean": float(np.mean(w.ctx)),
                      "ctx_min": int(min(w.ctx)), "ctx_max": int(max(w.ctx)),
                      "page_tokens": 256 if w.scheme == "witcert" else 64,
                      "G": w.G, "R": w.R, "layers": 1, "cache_copies": copies},
           "tokens_per_s": round(w.B / (ms_step * 1e-3), 1),
           # the same step time for 32 such attention layers and nothing else
           "tokens_per_s_attention_only_32_layers": round(w.B / (ms_step * 1e-3) / 32, 1),
           "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
           "settle": settle,
           "roofline": roof}
    if lat is not None:
        rec["latency"] = lat
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        rec["cpu_baseline"] = cpu_baseline(w, args.warmup, args.cpu_seconds)
        one_t = cpu_baseline(w, args.warmup, max(2.0, args.cpu_seconds / 4), threads=1, n_pairs=4)
        rec["cpu_baseline"]["single_thread"] = {"value": one_t["value"], "unit": one_t["unit"],
                                                "sample": one_t["sample"]}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
