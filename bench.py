"""Benchmark of the TurboQuant KV-cache hot path on one MI355X.

One step = the whole path for one decode step of the workload: encode the
step's new K and V token of every KV head into the cache (append), prepare
the queries (rotation + QJL projection), and run split-K decode attention over
the full compressed context. Steps read rotating device copies of the cache
(together at least 1 GiB, four times the 256 MB Infinity Cache) so the stream
comes from HBM. Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]
"""

from __future__ import annotations

import argparse
import dataclasses
import ctypes as C
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compressed-KV decode attention GB/s (% HBM peak) + ctx tokens/s; encode vec/s"
HBM_PEAK_GBS = 8000.0
ROTATE_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.txt")


def kv_bytes_per_token_head(d: int, v_bits: int = 3, k_bits: int = 3) -> int:
    """Algorithmic compressed bytes read per (token, KV head): K record (k_bits
    code planes and the signs) + its two fp16 sidecars, V record (v_bits-bit
    codes) + its fp16 sidecar."""
    return ((k_bits + 1) * d // 8 + 4) + (v_bits * d // 8 + 2)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_vector_07_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per decode launch measured with rocprofv3 counters, if they were
    taken on the current kernel sources (else None)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.strip().split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_hash") != kernel_source_hash() or kv.get("workload") != workload:
        return None
    return float(kv["hbm_bytes_per_launch"])


def platform_info():
    """ROCm/HIP version, GPU name and the current clock levels (best effort). The
    clocks are read from the amdgpu sysfs files (the level marked '*'), so no
    helper program is started from this GPU process."""
    import glob
    import torch
    info = {"hip": torch.version.hip, "torch": torch.__version__,
            "gpu": torch.cuda.get_device_name(0)}
    clk = []
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_[sm]clk")):
        try:
            with open(path) as f:
                cur = [ln.strip() for ln in f if ln.strip().endswith("*")]
            if cur:
                clk.append(f"{os.path.basename(path)[7:]} {cur[0]}")
        except OSError:
            pass
    info["clocks"] = clk[:4] if clk else "unavailable"
    return info


def dense_baseline(dense, qs, seq, scale, tq_dec_ms, sh, log, v_bits=3, k_bits=3):
    """The uncompressed bf16 decode kernel on the same K, V and queries, over
    rotating device copies (>= 1 GiB), against the compressed split kernel."""
    import torch
    from kv_cache_vector_07_amd import tq
    k0, v0 = dense
    B, H, Lm, d = k0.shape
    nbytes = 2 * k0.numel() * 2
    R = max(1, math.ceil(ROTATE_BYTES / nbytes))
    ks = [k0] + [k0.clone() for _ in range(R - 1)]
    vs = [v0] + [v0.clone() for _ in range(R - 1)]
    out = torch.empty(qs[0].shape, dtype=torch.float32, device=k0.device)
    L_ = tq.lib()
    size = C.c_size_t(0)
    n_q, Hq = qs[0].shape[1], qs[0].shape[2]
    qdt = tq._dtype_code(qs[0])
    args = lambda i, ws: (ks[i % R].data_ptr(), vs[i % R].data_ptr(), d, H, Lm, qs[i % len(qs)].data_ptr(),
                          qdt, B, n_q, Hq, seq.data_ptr(), scale, out.data_ptr(), ws)
    assert L_.tq_dense_attn_decode(*args(0, None), C.byref(size), None) == 0
    ws = torch.empty(size.value, dtype=torch.uint8, device=k0.device)
    for i in range(8):
        sz = C.c_size_t(ws.numel())
        assert L_.tq_dense_attn_decode(*args(i, ws.data_ptr()), C.byref(sz), sh) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 64
    torch.cuda.synchronize()
    e0.record()
    for i in range(n):
        sz = C.c_size_t(ws.numel())
        L_.tq_dense_attn_decode(*args(i, ws.data_ptr()), C.byref(sz), sh)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    gbs = nbytes / (ms / 1e3) / 1e9
    log(f"[bench] dense bf16 baseline: {ms * 1e3:.2f} us/step ({gbs:.0f} GB/s), {R} copies")
    return {"kernel": "dense_decode_kernel + merge", "us_per_step": round(ms * 1e3, 3),
            "bytes_per_step": nbytes, "achieved_GBps": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4), "rotating_copies": R,
            "speedup_compressed_split_vs_dense": round(ms / tq_dec_ms, 3),
            "speedup_vs_dense_at_hbm_peak": round(nbytes / (HBM_PEAK_GBS * 1e9) * 1e3 / tq_dec_ms, 3),
            "ideal_byte_ratio": round(nbytes / (Lm * B * H * kv_bytes_per_token_head(d, v_bits, k_bits)), 3)}


def _host_cpu():
    """CPU model, logical CPUs and the ones this process may run on (no helper
    program is started)."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "cpu_count": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def cpu_baseline(w, lens, n_pages_total, kp, vp, table, q, budget_s=12.0, budget_1t_s=6.0,
                 v_bits=3, k_bits=3):
    """The CPU reference (numpy float64, as it stands) timed on this host on a
    bounded sample: whole decode steps over every KV head of sequence 0 with the
    BLAS thread pool as it is, then again on one BLAS thread, and an encode of a
    slice of the K/V inputs."""
    import oracle as O
    from kv_cache_vector_07_amd import inputs as I
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threadpool_limits = None
        threads = 1
    cb = O.codebook(w.head_dim, k_bits)
    S = O.qjl_matrix(w.head_dim, w.qjl_seed)
    d, H = w.head_dim, w.n_kv_heads
    L = int(lens[0])

    def decode_rate(budget):
        t0 = time.perf_counter()
        done = 0
        while time.perf_counter() - t0 < budget and done < 64 * H:
            O.attn_decode(kp, vp, cb, S, q[:1].astype(np.float64), table[:1], lens[:1], H,
                          w.page_size, 1 / math.sqrt(d), pairs=[(0, done % H)],
                          cb_v=O.codebook(d, v_bits), v_bits=v_bits, k_bits=k_bits)
            done += 1
        dt = time.perf_counter() - t0
        return done, dt, done * L * kv_bytes_per_token_head(d, v_bits, k_bits) / dt / 1e9

    heads_done, dt, gbs = decode_rate(budget_s)
    one = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            one = decode_rate(budget_1t_s)
    n_enc = 2048
    x = I.kv_tokens(w, "k", 0, 0, n_enc // H + 1)[: n_enc // H].astype(np.float64)
    cb_v = O.codebook(d, v_bits)
    t1 = time.perf_counter()
    O.encode(x, cb, S)
    O.encode(x, cb_v)
    enc_dt = time.perf_counter() - t1
    out = {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{heads_done} (sequence, KV head) decode passes over L={L} "
                     f"({heads_done * w.group} query rows) in {dt:.1f} s; "
                     f"encode of {x.shape[0] * H} K and V vectors",
           "encode_vec_per_s": round(2 * x.shape[0] * H / enc_dt, 1),
           "host": _host_cpu()}
    if one is not None:
        out["value_1_thread"] = round(one[2], 4)
        out["sample_1_thread"] = f"{one[0]} decode passes in {one[1]:.1f} s on one BLAS thread"
    return out


def prefill_attention(copies, table, lens, w, chunk, tdt, scale, sh, log):
    """Chunked-prefill attention: the last `chunk` tokens of each sequence are
    appended again (encoding is idempotent) and their chunk x Hq/Hkv query rows
    attend causally over the whole compressed cache, in one tq_append_decode.
    Reported against the time its MFMA instructions need at the published
    rates (16 clocks per 16x16x128 fp6 x fp4 and per 16x16x64 int8 MFMA on
    1024 SIMDs at 2.4 GHz), counted over the 64-token blocks each workgroup's
    rows can see."""
    import torch
    from kv_cache_vector_07_amd import inputs as I
    from kv_cache_vector_07_amd import tq
    dev = table.device
    d, H, Hq, B = w.head_dim, w.n_kv_heads, w.n_q_heads, w.batch
    g = Hq // H
    rows = chunk * g
    R = len(copies)
    pos = np.concatenate([np.arange(int(L) - chunk, int(L)) for L in lens])
    seq_np = np.repeat(np.arange(B), chunk)
    tbl = table.cpu().numpy()
    slots = torch.from_numpy((tbl[seq_np, pos // 256].astype(np.int64) * 256 + pos % 256)
                             .astype(np.int32)).to(dev)
    k = torch.from_numpy(np.concatenate([I.kv_tokens(w, "k", b, int(L) - chunk, int(L))
                                         for b, L in enumerate(lens)])).to(dev, tdt)
    v = torch.from_numpy(np.concatenate([I.kv_tokens(w, "v", b, int(L) - chunk, int(L))
                                         for b, L in enumerate(lens)])).to(dev, tdt)
    rng = np.random.default_rng([w.data_seed, 7, chunk])
    q = torch.from_numpy(rng.standard_normal((B, chunk, Hq, d)).astype(np.float32)).to(dev, tdt)
    seq = torch.from_numpy(lens.astype(np.int32)).to(dev)
    out = torch.empty(B, chunk, Hq, d, dtype=torch.float32, device=dev)
    size = C.c_size_t(0)
    L_ = tq.lib()
    qdt = tq._dtype_code(q)
    args = lambda i, wsp: (copies[i % R].ref, k.data_ptr(), v.data_ptr(), qdt, slots.data_ptr(),
                           B * chunk, q.data_ptr(), qdt, B, chunk, Hq, table.data_ptr(),
                           table.shape[1], seq.data_ptr(), 1, scale, out.data_ptr(), wsp)
    st = L_.tq_append_decode(*args(0, None), C.byref(size), None)
    if st:
        log(f"[bench] prefill attention: chunk {chunk} not supported (status {st})")
        return None
    ws = torch.empty(size.value, dtype=torch.uint8, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def run(i):
        sz = C.c_size_t(ws.numel())
        r = L_.tq_append_decode(*args(i, ws.data_ptr()), C.byref(sz), sh)
        if r:
            raise RuntimeError(f"prefill attention launch failed with status {r}")
    for i in range(3):
        run(i)
    torch.cuda.synchronize()
    n = 8
    e0.record()
    for i in range(n):
        run(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    # MFMA instructions: per visible 64-token block and query group of 4 rows,
    # 4 tiles x 5 d/128 fp6 x fp4 MFMAs and 4 planes x d/16 int8 MFMAs
    per_blk = 4 * 5 * (d // 128) + 4 * (d // 16)
    groups = (rows + 3) // 4
    blocks = 0
    useful = 0
    for L in lens:
        for gi in range(groups):
            t_last = min(4 * gi + 3, rows - 1) // g
            vis = int(L) - (chunk - 1 - t_last)
            blocks += (vis + 63) // 64
        t = np.arange(chunk)
        useful += g * int(np.sum(int(L) - (chunk - 1 - t)))
    blocks *= H
    mfma_us = blocks * per_blk * 16 / (1024 * 2.4e9) * 1e6
    flops = 4.0 * d * useful * H
    log(f"[bench] prefill attention: chunk {chunk}, {rows} rows per KV head: {ms * 1e3:.1f} us "
        f"(MFMA issue bound {mfma_us:.1f} us)")
    return {"entry": "tq_append_decode (causal tail)", "chunk": chunk, "rows_per_kv_head": rows,
            "us": round(ms * 1e3, 2), "query_tokens_per_s": round(B * chunk / (ms / 1e3), 1),
            "dense_equiv_tflops": round(flops / (ms / 1e3) / 1e12, 2),
            "mfma_issue_bound_us": round(mfma_us, 2), "frac_of_mfma_bound": round(mfma_us / (ms * 1e3), 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-launches", type=int, default=512)
    ap.add_argument("--v-bits", type=int, default=3, choices=(2, 3, 4),
                    help="V code width (3: the method's V path; 2 and 4: the bit-width variant)")
    ap.add_argument("--k-bits", type=int, default=3, choices=(2, 3, 4),
                    help="K code width (3: the method's K path; 2 and 4: the bit-width variant)")
    ap.add_argument("--prefill-chunk", type=int, default=512,
                    help="chunk length of the chunked-prefill attention measurement (0: skip)")
    ap.add_argument("--no-dense-baseline", action="store_true",
                    help="skip the uncompressed bf16 decode baseline")
    ap.add_argument("--context", type=int, default=0,
                    help="override the context length of an equal-length workload (a sweep "
                         "point, named <workload>_ctx<L>; not the headline configuration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import torch

    from kv_cache_vector_07_amd import inputs as I
    from kv_cache_vector_07_amd import tq

    L_ = tq.lib()
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    w = I.workload(args.workload)
    if args.context:
        if not w.fixed_len:
            print(json.dumps({"error": "--context needs an equal-length workload"}))
            sys.exit(2)
        w = dataclasses.replace(w, name=f"{w.name}_ctx{args.context}", fixed_len=args.context)
    d, H, Hq, B, nq = w.head_dim, w.n_kv_heads, w.n_q_heads, w.batch, w.n_q
    lens = I.seq_lens(w)
    table_np, n_pages = I.page_table(w, lens, shuffle=w.batch > 1)
    vbits, kbits = args.v_bits, args.k_bits
    kpb, vpb = tq.tq_k_page_bytes(d, bits=kbits), tq.tq_v_page_bytes(d, bits=vbits)
    copy_bytes = n_pages * H * (kpb + vpb)
    R = max(1, math.ceil(ROTATE_BYTES / copy_bytes))
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    log(f"[bench] workload {w.name}: B={B} Hq={Hq} Hkv={H} d={d} n_q={nq} "
        f"L={lens.tolist() if B <= 4 else (int(lens.min()), int(lens.max()))}, "
        f"{n_pages} pages, {R} rotating copies of {copy_bytes / 1e6:.1f} MB")

    # ---- build the compressed cache once (timed: encode vec/s), then copy it
    base = tq.Cache(d, H, n_pages, qjl_seed=w.qjl_seed, device=dev, v_bits=vbits, k_bits=kbits)
    table = torch.from_numpy(table_np).to(dev)
    seq = torch.from_numpy(lens.astype(np.int32)).to(dev)
    stream = torch.cuda.current_stream()
    # every chunk's inputs are staged on the device first, so the timed region
    # holds only back-to-back encode launches (all K calls, then all V calls)
    calls = []
    if w.prefill_chunk:
        # chunked prefill: one call per chunk position covers every sequence
        CH = w.prefill_chunk
        for t0 in range(0, int(lens.min()), CH):
            t = torch.arange(t0, t0 + CH, device=dev)
            slots = torch.cat([(table[b, t // 256] * 256 + t % 256) for b in range(B)]).to(torch.int32)
            k = torch.from_numpy(np.concatenate([I.kv_tokens(w, "k", b, t0, t0 + CH) for b in range(B)])).to(dev, tdt)
            v = torch.from_numpy(np.concatenate([I.kv_tokens(w, "v", b, t0, t0 + CH) for b in range(B)])).to(dev, tdt)
            calls.append((k, v, slots))
    else:
        chunk = 32768
        for b in range(B):
            Lb = int(lens[b])
            for t0 in range(0, Lb, chunk):
                t1 = min(Lb, t0 + chunk)
                k = torch.from_numpy(I.kv_tokens(w, "k", b, t0, t1)).to(dev, tdt)
                v = torch.from_numpy(I.kv_tokens(w, "v", b, t0, t1)).to(dev, tdt)
                t = torch.arange(t0, t1, device=dev)
                slots = (table[b, t // 256] * 256 + t % 256).to(torch.int32)
                calls.append((k, v, slots))
    n_vec = sum(c[2].numel() for c in calls) * H
    # one untimed call first (encoding is idempotent): the first launch of a
    # kernel also loads its code object
    tq.tq_encode_k(base, *calls[0][0::2])
    tq.tq_encode_v(base, *calls[0][1:])
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    torch.cuda.synchronize()
    e0.record()
    for k, v, slots in calls:
        tq.tq_encode_k(base, k, slots)
    e1.record()
    for k, v, slots in calls:
        tq.tq_encode_v(base, v, slots)
    e2.record()
    e2.synchronize()
    enc_k_ms, enc_v_ms = e0.elapsed_time(e1), e1.elapsed_time(e2)
    # the uncompressed bf16 baseline reads the same K and V densely (single
    # sequence workloads: the staged chunks are the sequence in order)
    dense = None
    if B == 1 and not args.no_dense_baseline and tdt == torch.bfloat16:
        # [1][Hkv][L][d]: each KV head's tokens contiguous
        dense = tuple(torch.cat([c[i] for c in calls]).transpose(0, 1).contiguous().unsqueeze(0)
                      for i in (0, 1))
    del calls
    log(f"[bench] cache encoded: {n_vec} K and V vectors")
    copies = [base]
    for _ in range(R - 1):
        c = tq.Cache(d, H, n_pages, device=dev, zero=False,
                     codebook=(base.levels, base.thresholds, base.qjl_host), v_bits=vbits,
                     v_codebook=(base.v_levels, base.v_thresholds), k_bits=kbits,
                     k_codebook=(base.k_levels, base.k_thresholds))
        c.k_pool.copy_(base.k_pool)
        c.v_pool.copy_(base.v_pool)
        copies.append(c)
    torch.cuda.synchronize()

    # ---- per-step inputs: fresh queries and one new K/V token per sequence
    n_q_sets = 16
    qs = [torch.from_numpy(I.queries(w, s)).to(dev, tdt) for s in range(n_q_sets)]
    app_k = [torch.from_numpy(I.kv_tokens(w, "k", b, int(lens[b]) - 1, int(lens[b]))).to(dev, tdt)
             for b in range(B)]
    app_v = [torch.from_numpy(I.kv_tokens(w, "v", b, int(lens[b]) - 1, int(lens[b]))).to(dev, tdt)
             for b in range(B)]
    new_k = torch.cat(app_k, 0).contiguous()
    new_v = torch.cat(app_v, 0).contiguous()
    last = torch.from_numpy(lens - 1).to(dev)
    app_slots = (table[torch.arange(B, device=dev), last // 256] * 256 + last % 256).to(torch.int32)
    size = C.c_size_t(0)
    scale = 1.0 / math.sqrt(d)
    out = torch.empty(B, nq, Hq, d, dtype=torch.float32, device=dev)
    st = L_.tq_attn_decode(copies[0].ref, qs[0].data_ptr(), tq._dtype_code(qs[0]), B, nq, Hq,
                           table.data_ptr(), table.shape[1], seq.data_ptr(), 0, scale,
                           out.data_ptr(), None, C.byref(size), None)
    assert st == 0, st
    ws = torch.zeros(size.value, dtype=torch.uint8, device=dev)
    sh = stream.cuda_stream
    qdt = tq._dtype_code(qs[0])
    mp = table.shape[1]

    def step(i):
        c = copies[i % R]
        q = qs[i % n_q_sets]
        # append one token per sequence (encode K and V), then decode: one call
        sz = C.c_size_t(ws.numel())
        r = L_.tq_append_decode(c.ref, new_k.data_ptr(), new_v.data_ptr(), qdt, app_slots.data_ptr(),
                                B, q.data_ptr(), qdt, B, nq, Hq, table.data_ptr(), mp,
                                seq.data_ptr(), 0, scale, out.data_ptr(), ws.data_ptr(),
                                C.byref(sz), sh)
        if r:
            raise RuntimeError(f"launch failed with status {r}")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    step_ms = ev0.elapsed_time(ev1) / args.steps
    log(f"[bench] timed {args.steps} steps: {step_ms * 1e3:.2f} us/step (host wall {wall:.3f} s)")

    # ---- the split-K decode kernel alone (the dominant kernel): back-to-back launches
    prep = tq.tq_query_prepare(copies[0], qs[0])
    size_p = C.c_size_t(0)
    L_.tq_attn_decode_split(copies[0].ref, prep.data_ptr(), B, nq, Hq, table.data_ptr(), mp,
                            seq.data_ptr(), 0, scale, None, C.byref(size_p), None)
    ws_p = torch.zeros(size_p.value, dtype=torch.uint8, device=dev)

    def dec(i):
        c = copies[i % R]
        sz = C.c_size_t(ws_p.numel())
        r = L_.tq_attn_decode_split(c.ref, prep.data_ptr(), B, nq, Hq, table.data_ptr(), mp,
                                    seq.data_ptr(), 0, scale, ws_p.data_ptr(), C.byref(sz), sh)
        if r:
            raise RuntimeError(f"decode launch failed with status {r}")

    def merge(i):
        r = L_.tq_attn_decode_merge(copies[0].ref, B, nq, Hq, mp, out.data_ptr(), ws_p.data_ptr(),
                                    ws_p.numel(), sh)
        if r:
            raise RuntimeError(f"merge launch failed with status {r}")

    def timed(fn, n):
        for i in range(8):
            fn(i)
        torch.cuda.synchronize()
        ev0.record()
        for i in range(n):
            fn(i)
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n

    dec_ms = timed(dec, args.decode_launches)
    merge_ms = timed(merge, 64)
    dec_kernel = "decode_mfma_kernel"

    # the same split kernel on one copy only: its data can stay in the 256 MB
    # Infinity Cache, so this is the "warm" figure, not the HBM-bound one
    def dec_warm(i):
        dec(0)
    dec_warm_ms = timed(dec_warm, 64)

    # the append encode of one step alone (one K and one V vector per sequence
    # and KV head), as separate tq_encode_k / tq_encode_v calls
    def append(i):
        c = copies[i % R]
        tq.tq_encode_k(c, new_k, app_slots, stream=sh)
        tq.tq_encode_v(c, new_v, app_slots, stream=sh)
    append_ms = timed(append, 64)

    ctx_tokens = int(lens.sum())
    kv_bytes = ctx_tokens * H * kv_bytes_per_token_head(d, vbits, kbits)
    app_bytes = B * H * (2 * d * (2 if w.dtype == "bf16" else 4) + kv_bytes_per_token_head(d, vbits, kbits))
    step_s = step_ms / 1e3
    value = (kv_bytes + app_bytes) / step_s / 1e9
    dec_gbs = kv_bytes / (dec_ms / 1e3) / 1e9
    traffic = read_traffic(w.name) if vbits == 3 and kbits == 3 else None
    in_bytes = 2 if w.dtype == "bf16" else 4
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; outlier-channel K where the workload says so)",
        "config": {"workload": w.name, "batch": B, "n_q_heads": Hq, "n_kv_heads": H,
                   "head_dim": d, "n_q": nq, "context": int(lens.max()) if B == 1 else
                   [int(lens.min()), int(lens.max())], "ctx_tokens": ctx_tokens,
                   "input_dtype": w.dtype, "page_size": 256, "rotating_copies": R,
                   "v_bits": vbits, "k_bits": kbits,
                   "step": "tq_append_decode: append 1 token/seq (encode K+V) and decode (prologue, split-K, merge)"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "ctx_tokens_per_s": round(ctx_tokens / step_s, 1),
        "encode_k_vec_per_s": round(n_vec / (enc_k_ms / 1e3), 1),
        "encode_v_vec_per_s": round(n_vec / (enc_v_ms / 1e3), 1),
        # input + record bytes per vector; S r is m x d = d^2 multiply-adds per K vector
        "encode_k_GBps": round(n_vec * (d * in_bytes + d // 2 + 4) / (enc_k_ms / 1e3) / 1e9, 2),
        "encode_v_GBps": round(n_vec * (d * in_bytes + 3 * d // 8 + 2) / (enc_v_ms / 1e3) / 1e9, 2),
        "encode_k_sr_tflops": round(n_vec * 2 * d * d / (enc_k_ms / 1e3) / 1e12, 2),
        "encode_k_sr_frac_fp32_peak": round(n_vec * 2 * d * d / (enc_k_ms / 1e3) / 157.3e12, 4),
        "decode_kernel_us": round(dec_ms * 1e3, 3),
        "decode_kernel_us_warm_single_copy": round(dec_warm_ms * 1e3, 3),
        "merge_kernel_us": round(merge_ms * 1e3, 3),
        "append_encode_us": round(append_ms * 1e3, 3),
        "platform": platform_info(),
        "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": dec_kernel,
                     "bytes_per_launch": kv_bytes},
    }
    if args.prefill_chunk > 0 and int(lens.min()) >= args.prefill_chunk:
        pa = prefill_attention(copies, table, lens, w, args.prefill_chunk, tdt, scale, sh, log)
        if pa is not None:
            result["prefill_attention"] = pa
    if dense is not None:
        result["dense_bf16_baseline"] = dense_baseline(dense, qs, seq, scale, dec_ms, sh, log, vbits, kbits)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU reference on a bounded sample")
        kp = base.k_pool.cpu().numpy()
        vp = base.v_pool.cpu().numpy()
        result["cpu_baseline"] = cpu_baseline(w, lens, n_pages, kp, vp, table_np,
                                              I.queries(w, 0), v_bits=vbits, k_bits=kbits)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
