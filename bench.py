"""Benchmark of the TurboQuant KV-cache hot path on one MI355X.

One step = the whole path for one decode step of the workload: encode the
step's new K and V tokens of every KV head into the cache (append), prepare
the queries (rotation + QJL projection), and run split-K decode attention over
the full compressed context. Steps read rotating device copies of the cache
(together at least 1 GiB, four times the 256 MB Infinity Cache) so the stream
comes from HBM. Prints one JSON line.

The headline workload (--workload, default 2: GQA decode at 32K context) is
timed over exactly --steps steps after --warmup untimed ones. The other
workloads named by --also (default 3,4,5: 100K context, batched paged serving,
chunked prefill + 4-token verify) each get a record under "workloads" with the
median of 5 event-timed repeats of the step and of the decode kernel, and, for
single-sequence bf16 workloads, the uncompressed bf16 decode baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--also 3,4,5]
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import ctypes as C
import dataclasses
import hashlib
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compressed-KV decode attention GB/s (% HBM peak) + ctx tokens/s; encode vec/s"
HBM_PEAK_GBS = 8000.0
ROTATE_BYTES = 1 << 30
REPEATS = 5
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.txt")
# what the path computes in: scores on block-scaled MFMA (fp6 query limbs x fp4
# key bit planes, fp32 accumulation), V on int8 MFMA (int8 weight limbs x V bit
# planes, int32 accumulation), softmax and outputs in fp32
DTYPE = "fp6x4-limb x fp4 scores, int8x4-limb V, fp32 softmax/accum/out"


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


class Timer:
    """Event timing of back-to-back launches on the stream they are issued on."""

    def __init__(self):
        import torch
        self.torch = torch
        self.e0 = torch.cuda.Event(enable_timing=True)
        self.e1 = torch.cuda.Event(enable_timing=True)

    def once(self, fn, n, start=0):
        """Average ms per call of fn(start), ..., fn(start + n - 1)."""
        self.torch.cuda.synchronize()
        self.e0.record()
        for i in range(n):
            fn(start + i)
        self.e1.record()
        self.torch.cuda.synchronize()
        return self.e0.elapsed_time(self.e1) / n

    def median(self, fn, n, warm=8, repeats=REPEATS):
        """Median over `repeats` repeats of the average ms per call over n calls
        (after `warm` untimed calls); also returns every repeat."""
        for i in range(warm):
            fn(i)
        runs = [self.once(fn, n, start=warm + r * n) for r in range(repeats)]
        return statistics.median(runs), runs


# ---------------------------------------------------------------- cache build
def _call_specs(w, lens):
    """Encode calls of the initial cache build: one per 4096-token chunk position
    over every sequence for chunked-prefill workloads, else per sequence and
    32768-token range."""
    if w.prefill_chunk:
        CH = w.prefill_chunk
        return [("all", t0, t0 + CH) for t0 in range(0, int(lens.min()), CH)]
    specs = []
    for b in range(w.batch):
        Lb = int(lens[b])
        for t0 in range(0, Lb, 32768):
            specs.append((b, t0, min(Lb, t0 + 32768)))
    return specs


def _host_call(w, table_np, spec):
    from kv_cache_vector_07_amd import inputs as I
    b, t0, t1 = spec
    seqs = range(w.batch) if b == "all" else [b]
    t = np.arange(t0, t1)
    k = np.concatenate([I.kv_tokens(w, "k", s, t0, t1) for s in seqs])
    v = np.concatenate([I.kv_tokens(w, "v", s, t0, t1) for s in seqs])
    slots = np.concatenate([table_np[s][t // 256].astype(np.int64) * 256 + t % 256 for s in seqs])
    return k, v, slots.astype(np.int32)


def build_cache(w, dev, vbits, kbits, log, keep_dense=False):
    """Encode the whole workload into a fresh paged cache. Inputs are drawn on the
    host by a thread pool (the generator is chunked and seeded per chunk) and
    staged on the device first, so the timed encode region holds only
    back-to-back encode launches: every K call, then every V call."""
    import torch
    from kv_cache_vector_07_amd import inputs as I
    from kv_cache_vector_07_amd import tq
    lens = I.seq_lens(w)
    table_np, n_pages = I.page_table(w, lens, shuffle=w.batch > 1)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    base = tq.Cache(w.head_dim, w.n_kv_heads, n_pages, qjl_seed=w.qjl_seed, device=dev,
                    v_bits=vbits, k_bits=kbits)
    specs = _call_specs(w, lens)
    calls = []
    workers = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 8))
    window = workers + 4
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        futs = [ex.submit(_host_call, w, table_np, s) for s in specs[:window]]
        nxt = window
        while futs:
            k, v, slots = futs.pop(0).result()
            calls.append((torch.from_numpy(k).to(dev, tdt), torch.from_numpy(v).to(dev, tdt),
                          torch.from_numpy(slots).to(dev)))
            if nxt < len(specs):
                futs.append(ex.submit(_host_call, w, table_np, specs[nxt]))
                nxt += 1
    n_vec = sum(c[2].numel() for c in calls) * w.n_kv_heads
    # one untimed pass over every call first (encoding is idempotent): it loads
    # the kernels' code objects and brings the GPU out of its idle clocks
    for k, v, slots in calls:
        tq.tq_encode_k(base, k, slots)
        tq.tq_encode_v(base, v, slots)
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
    enc = {"n_vec": n_vec, "k_ms": e0.elapsed_time(e1), "v_ms": e1.elapsed_time(e2),
           "calls": len(calls)}
    dense = None
    if keep_dense and w.batch == 1 and tdt == torch.bfloat16:
        # [1][Hkv][L][d]: each KV head's tokens contiguous (single sequence: the
        # staged calls are the sequence in order)
        dense = tuple(torch.cat([c[i] for c in calls]).transpose(0, 1).contiguous().unsqueeze(0)
                      for i in (0, 1))
    del calls
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: cache encoded, {n_vec} K and V vectors")
    return base, table_np, lens, n_pages, enc, dense


def rotating_copies(base, w, n_pages, vbits, kbits, dev):
    import torch
    from kv_cache_vector_07_amd import tq
    copy_bytes = n_pages * w.n_kv_heads * (tq.tq_k_page_bytes(w.head_dim, bits=kbits)
                                           + tq.tq_v_page_bytes(w.head_dim, bits=vbits))
    R = max(1, math.ceil(ROTATE_BYTES / copy_bytes))
    copies = [base]
    for _ in range(R - 1):
        c = tq.Cache(w.head_dim, w.n_kv_heads, n_pages, device=dev, zero=False,
                     codebook=(base.levels, base.thresholds, base.qjl_host), v_bits=vbits,
                     v_codebook=(base.v_levels, base.v_thresholds), k_bits=kbits,
                     k_codebook=(base.k_levels, base.k_thresholds))
        c.k_pool.copy_(base.k_pool)
        c.v_pool.copy_(base.v_pool)
        copies.append(c)
    torch.cuda.synchronize()
    return copies, copy_bytes


class Workload:
    """Device state of one workload for timing: rotating cache copies, queries,
    the tokens appended per step, and the calls that one step makes."""

    def __init__(self, w, dev, vbits, kbits, log, keep_dense=False):
        import torch
        from kv_cache_vector_07_amd import inputs as I
        from kv_cache_vector_07_amd import tq
        self.w, self.vbits, self.kbits = w, vbits, kbits
        d, H, Hq, B, nq = w.head_dim, w.n_kv_heads, w.n_q_heads, w.batch, w.n_q
        base, self.table_np, self.lens, self.n_pages, self.enc, self.dense = build_cache(
            w, dev, vbits, kbits, log, keep_dense)
        self.copies, self.copy_bytes = rotating_copies(base, w, self.n_pages, vbits, kbits, dev)
        self.R = len(self.copies)
        log(f"[bench] {w.name}: B={B} Hq={Hq} Hkv={H} d={d} n_q={nq} "
            f"L={self.lens.tolist() if B <= 4 else (int(self.lens.min()), int(self.lens.max()))}, "
            f"{self.n_pages} pages, {self.R} rotating copies of {self.copy_bytes / 1e6:.1f} MB")
        self.tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.table = torch.from_numpy(self.table_np).to(dev)
        self.seq = torch.from_numpy(self.lens.astype(np.int32)).to(dev)
        self.n_q_sets = 16
        self.qs = [torch.from_numpy(I.queries(w, s)).to(dev, self.tdt) for s in range(self.n_q_sets)]
        # tokens appended per step: the last `a` tokens of each sequence are encoded
        # again (encoding is idempotent); one per sequence, or the n_q verify tokens
        a = max(1, nq)
        pos = np.concatenate([np.arange(int(L) - a, int(L)) for L in self.lens])
        seq_of = np.repeat(np.arange(B), a)
        self.new_k = torch.from_numpy(np.concatenate(
            [I.kv_tokens(w, "k", b, int(L) - a, int(L)) for b, L in enumerate(self.lens)])).to(dev, self.tdt)
        self.new_v = torch.from_numpy(np.concatenate(
            [I.kv_tokens(w, "v", b, int(L) - a, int(L)) for b, L in enumerate(self.lens)])).to(dev, self.tdt)
        self.app_slots = torch.from_numpy((self.table_np[seq_of, pos // 256].astype(np.int64) * 256
                                           + pos % 256).astype(np.int32)).to(dev)
        self.n_new = int(self.app_slots.numel())
        self.scale = 1.0 / math.sqrt(d)
        self.out = torch.empty(B, nq, Hq, d, dtype=torch.float32, device=dev)
        self.L_ = tq.lib()
        self.qdt = tq._dtype_code(self.qs[0])
        self.mp = self.table.shape[1]
        size = C.c_size_t(0)
        st = self.L_.tq_append_decode(self.copies[0].ref, None, None, self.qdt, None, 0,
                                      self.qs[0].data_ptr(), self.qdt, B, nq, Hq, self.table.data_ptr(),
                                      self.mp, self.seq.data_ptr(), 0, self.scale, self.out.data_ptr(),
                                      None, C.byref(size), None)
        assert st == 0, st
        self.ws = torch.zeros(size.value, dtype=torch.uint8, device=dev)
        self.sh = torch.cuda.current_stream().cuda_stream
        # the decode kernels alone, on a prepared query
        self.prep = tq.tq_query_prepare(self.copies[0], self.qs[0])
        size_p = C.c_size_t(0)
        self.L_.tq_attn_decode_split(self.copies[0].ref, self.prep.data_ptr(), B, nq, Hq,
                                     self.table.data_ptr(), self.mp, self.seq.data_ptr(), 0,
                                     self.scale, None, C.byref(size_p), None)
        self.ws_p = torch.zeros(size_p.value, dtype=torch.uint8, device=dev)
        self.ctx_tokens = int(self.lens.sum())
        self.kv_bytes = self.ctx_tokens * H * kv_bytes_per_token_head(d, vbits, kbits)
        in_b = 2 if w.dtype == "bf16" else 4
        self.app_bytes = self.n_new * H * (2 * d * in_b + kv_bytes_per_token_head(d, vbits, kbits))

    def step(self, i):
        """One decode step: append (encode K and V) and decode, one call."""
        w = self.w
        c = self.copies[i % self.R]
        q = self.qs[i % self.n_q_sets]
        sz = C.c_size_t(self.ws.numel())
        r = self.L_.tq_append_decode(c.ref, self.new_k.data_ptr(), self.new_v.data_ptr(), self.qdt,
                                     self.app_slots.data_ptr(), self.n_new, q.data_ptr(), self.qdt,
                                     w.batch, w.n_q, w.n_q_heads, self.table.data_ptr(), self.mp,
                                     self.seq.data_ptr(), 0, self.scale, self.out.data_ptr(),
                                     self.ws.data_ptr(), C.byref(sz), self.sh)
        if r:
            raise RuntimeError(f"launch failed with status {r}")

    def split(self, i):
        """The split-K decode kernel alone (the dominant kernel)."""
        w = self.w
        c = self.copies[i % self.R]
        sz = C.c_size_t(self.ws_p.numel())
        r = self.L_.tq_attn_decode_split(c.ref, self.prep.data_ptr(), w.batch, w.n_q, w.n_q_heads,
                                         self.table.data_ptr(), self.mp, self.seq.data_ptr(), 0,
                                         self.scale, self.ws_p.data_ptr(), C.byref(sz), self.sh)
        if r:
            raise RuntimeError(f"decode launch failed with status {r}")

    def merge(self, i):
        w = self.w
        r = self.L_.tq_attn_decode_merge(self.copies[0].ref, w.batch, w.n_q, w.n_q_heads, self.mp,
                                         self.out.data_ptr(), self.ws_p.data_ptr(), self.ws_p.numel(),
                                         self.sh)
        if r:
            raise RuntimeError(f"merge launch failed with status {r}")

    def append(self, i):
        """One step's append encode alone, as separate tq_encode_k / tq_encode_v calls."""
        from kv_cache_vector_07_amd import tq
        c = self.copies[i % self.R]
        tq.tq_encode_k(c, self.new_k, self.app_slots, stream=self.sh)
        tq.tq_encode_v(c, self.new_v, self.app_slots, stream=self.sh)

    def encode_rates(self):
        d = self.w.head_dim
        in_b = 2 if self.w.dtype == "bf16" else 4
        n = self.enc["n_vec"]
        kb = (self.kbits + 1) * d // 8 + 4
        vb = self.vbits * d // 8 + 2
        return {
            "encode_k_vec_per_s": round(n / (self.enc["k_ms"] / 1e3), 1),
            "encode_v_vec_per_s": round(n / (self.enc["v_ms"] / 1e3), 1),
            # input + record bytes per vector; S r is m x d = d^2 multiply-adds per K vector
            "encode_k_GBps": round(n * (d * in_b + kb) / (self.enc["k_ms"] / 1e3) / 1e9, 2),
            "encode_v_GBps": round(n * (d * in_b + vb) / (self.enc["v_ms"] / 1e3) / 1e9, 2),
            "encode_v_frac_hbm": round(n * (d * in_b + vb) / (self.enc["v_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "encode_k_sr_tflops": round(n * 2 * d * d / (self.enc["k_ms"] / 1e3) / 1e12, 2),
            "encode_k_sr_frac_fp32_peak": round(n * 2 * d * d / (self.enc["k_ms"] / 1e3) / 157.3e12, 4),
            "encode_calls": self.enc["calls"],
        }


def dense_baseline(wl, tm, tq_dec_ms, log):
    """The uncompressed bf16 decode kernel on the same K, V and queries, over
    rotating device copies (>= 1 GiB), against the compressed split kernel;
    median of 5 repeats."""
    import torch
    from kv_cache_vector_07_amd import tq
    k0, v0 = wl.dense
    B, H, Lm, d = k0.shape
    nbytes = 2 * k0.numel() * 2
    R = max(1, math.ceil(ROTATE_BYTES / nbytes))
    ks = [k0] + [k0.clone() for _ in range(R - 1)]
    vs = [v0] + [v0.clone() for _ in range(R - 1)]
    out = torch.empty(wl.qs[0].shape, dtype=torch.float32, device=k0.device)
    L_ = tq.lib()
    size = C.c_size_t(0)
    n_q, Hq = wl.qs[0].shape[1], wl.qs[0].shape[2]
    args = lambda i, ws: (ks[i % R].data_ptr(), vs[i % R].data_ptr(), d, H, Lm,
                          wl.qs[i % wl.n_q_sets].data_ptr(), wl.qdt, B, n_q, Hq, wl.seq.data_ptr(),
                          wl.scale, out.data_ptr(), ws)
    assert L_.tq_dense_attn_decode(*args(0, None), C.byref(size), None) == 0
    ws = torch.empty(size.value, dtype=torch.uint8, device=k0.device)

    def run(i):
        sz = C.c_size_t(ws.numel())
        r = L_.tq_dense_attn_decode(*args(i, ws.data_ptr()), C.byref(sz), wl.sh)
        if r:
            raise RuntimeError(f"dense baseline launch failed with status {r}")
    ms, runs = tm.median(run, 32)
    gbs = nbytes / (ms / 1e3) / 1e9
    log(f"[bench] {wl.w.name}: dense bf16 baseline {ms * 1e3:.2f} us/step ({gbs:.0f} GB/s), {R} copies")
    del ks, vs
    return {"kernel": "dense_decode_kernel + merge", "us_per_step": round(ms * 1e3, 3),
            "us_repeats": [round(r * 1e3, 3) for r in runs],
            "bytes_per_step": nbytes, "achieved_GBps": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4), "rotating_copies": R,
            "speedup_compressed_split_vs_dense": round(ms / tq_dec_ms, 3),
            "speedup_vs_dense_at_hbm_peak": round(nbytes / (HBM_PEAK_GBS * 1e9) * 1e3 / tq_dec_ms, 3),
            "ideal_byte_ratio": round(nbytes / (Lm * B * H * kv_bytes_per_token_head(d, wl.vbits, wl.kbits)), 3)}


def workload_record(wl, tm, log, steps=64, launches=128):
    """Median-of-5 figures of one workload: whole step, decode split kernel,
    their HBM fractions and ctx tokens/s, encode rates, and the bf16 baseline
    where the workload has one bf16 sequence."""
    w = wl.w
    step_ms, step_runs = tm.median(wl.step, steps)
    dec_ms, dec_runs = tm.median(wl.split, launches)
    step_gbs = (wl.kv_bytes + wl.app_bytes) / (step_ms / 1e3) / 1e9
    dec_gbs = wl.kv_bytes / (dec_ms / 1e3) / 1e9
    log(f"[bench] {w.name}: step {step_ms * 1e3:.2f} us, decode kernel {dec_ms * 1e3:.2f} us "
        f"({100 * dec_gbs / HBM_PEAK_GBS:.1f}% of HBM peak)")
    rec = {
        "config": {"batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "n_q": w.n_q,
                   "context": int(wl.lens.max()) if w.batch == 1 else [int(wl.lens.min()), int(wl.lens.max())],
                   "ctx_tokens": wl.ctx_tokens, "input_dtype": w.dtype, "rotating_copies": wl.R,
                   "appended_tokens_per_step": wl.n_new},
        "step_us": round(step_ms * 1e3, 3),
        "step_us_repeats": [round(r * 1e3, 3) for r in step_runs],
        "step_GBps": round(step_gbs, 1),
        "step_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "ctx_tokens_per_s": round(wl.ctx_tokens / (step_ms / 1e3), 1),
        "decode_kernel_us": round(dec_ms * 1e3, 3),
        "decode_kernel_us_repeats": [round(r * 1e3, 3) for r in dec_runs],
        "decode_kernel_GBps": round(dec_gbs, 1),
        "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
        "bytes_per_launch": wl.kv_bytes,
    }
    rec.update(wl.encode_rates())
    if wl.dense is not None:
        rec["dense_bf16_baseline"] = dense_baseline(wl, tm, dec_ms, log)
    return rec


def cpu_baseline(w, lens, kp, vp, table, q, budget_s=12.0, budget_1t_s=6.0, v_bits=3, k_bits=3):
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


def prefill_attention(wl, chunk, tm, log):
    """Chunked-prefill attention: the last `chunk` tokens of each sequence are
    appended again (encoding is idempotent) and their chunk x Hq/Hkv query rows
    attend causally over the whole compressed cache, in one tq_append_decode.
    Reported against the time its MFMA instructions need at the published
    rates (16 clocks per 16x16x128 fp6 x fp4 and per 16x16x64 int8 MFMA on
    1024 SIMDs at 2.4 GHz), counted over the 64-token blocks each workgroup's
    rows can see, for the kernel the row count selects."""
    import torch
    from kv_cache_vector_07_amd import inputs as I
    w, lens = wl.w, wl.lens
    dev = wl.table.device
    d, H, Hq, B = w.head_dim, w.n_kv_heads, w.n_q_heads, w.batch
    g = Hq // H
    rows = chunk * g
    pos = np.concatenate([np.arange(int(L) - chunk, int(L)) for L in lens])
    seq_np = np.repeat(np.arange(B), chunk)
    slots = torch.from_numpy((wl.table_np[seq_np, pos // 256].astype(np.int64) * 256 + pos % 256)
                             .astype(np.int32)).to(dev)
    k = torch.from_numpy(np.concatenate([I.kv_tokens(w, "k", b, int(L) - chunk, int(L))
                                         for b, L in enumerate(lens)])).to(dev, wl.tdt)
    v = torch.from_numpy(np.concatenate([I.kv_tokens(w, "v", b, int(L) - chunk, int(L))
                                         for b, L in enumerate(lens)])).to(dev, wl.tdt)
    rng = np.random.default_rng([w.data_seed, 7, chunk])
    q = torch.from_numpy(rng.standard_normal((B, chunk, Hq, d)).astype(np.float32)).to(dev, wl.tdt)
    out = torch.empty(B, chunk, Hq, d, dtype=torch.float32, device=dev)
    size = C.c_size_t(0)
    L_ = wl.L_
    qdt = wl.qdt
    args = lambda i, wsp: (wl.copies[i % wl.R].ref, k.data_ptr(), v.data_ptr(), qdt, slots.data_ptr(),
                           B * chunk, q.data_ptr(), qdt, B, chunk, Hq, wl.table.data_ptr(),
                           wl.mp, wl.seq.data_ptr(), 1, wl.scale, out.data_ptr(), wsp)
    st = L_.tq_append_decode(*args(0, None), C.byref(size), None)
    if st:
        log(f"[bench] prefill attention: chunk {chunk} not supported (status {st})")
        return None
    ws = torch.empty(size.value, dtype=torch.uint8, device=dev)

    def run(i):
        sz = C.c_size_t(ws.numel())
        r = L_.tq_append_decode(*args(i, ws.data_ptr()), C.byref(sz), wl.sh)
        if r:
            raise RuntimeError(f"prefill attention launch failed with status {r}")
    ms, runs = tm.median(run, 4, warm=3)
    # MFMA instructions per visible 64-token block. Wide groups (16 rows or
    # more, 3-bit K and V): per 16 rows, 4 tiles x 5 d/128 x 4 limbs fp6 x fp4
    # MFMAs and 4 planes x 3 limbs x d/16 int8 MFMAs. Narrow groups of 4 rows:
    # 4 tiles x 5 d/128 fp6 x fp4 MFMAs and 4 planes x d/16 int8 MFMAs.
    wide = rows >= 16 and wl.kbits == 3 and wl.vbits == 3
    RW = 16 if wide else 4
    if wide:
        per_blk = 4 * 5 * (d // 128) * 4 + 4 * 3 * (d // 16)
    else:
        per_blk = 4 * 5 * (d // 128) + 4 * (d // 16)
    groups = (rows + RW - 1) // RW
    blocks = 0
    useful = 0
    for L in lens:
        for gi in range(groups):
            t_last = min(RW * gi + RW - 1, rows - 1) // g
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
            "us": round(ms * 1e3, 2), "us_repeats": [round(r * 1e3, 2) for r in runs],
            "query_tokens_per_s": round(B * chunk / (ms / 1e3), 1),
            "dense_equiv_tflops": round(flops / (ms / 1e3) / 1e12, 2),
            "mfma_issue_bound_us": round(mfma_us, 2), "frac_of_mfma_bound": round(mfma_us / (ms * 1e3), 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--also", default="3,4,5",
                    help="other workloads measured into the 'workloads' record (comma list, or 'none')")
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

    tq.lib()
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    w = I.workload(args.workload)
    if args.context:
        if not w.fixed_len:
            print(json.dumps({"error": "--context needs an equal-length workload"}))
            sys.exit(2)
        w = dataclasses.replace(w, name=f"{w.name}_ctx{args.context}", fixed_len=args.context)
    vbits, kbits = args.v_bits, args.k_bits
    d = w.head_dim
    tm = Timer()
    wl = Workload(w, dev, vbits, kbits, log, keep_dense=not args.no_dense_baseline)

    # ---- the headline: exactly --steps timed steps after --warmup untimed ones
    for i in range(args.warmup):
        wl.step(i)
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")
    t_wall = time.perf_counter()
    step_ms = tm.once(wl.step, args.steps, start=args.warmup)
    wall = time.perf_counter() - t_wall
    log(f"[bench] timed {args.steps} steps: {step_ms * 1e3:.2f} us/step (host wall {wall:.3f} s)")

    dec_ms, dec_runs = tm.median(wl.split, args.decode_launches)
    merge_ms = tm.once(wl.merge, 64)
    step_med_ms, step_runs = tm.median(wl.step, 64)
    # the same split kernel on one copy only: its data can stay in the 256 MB
    # Infinity Cache, so this is the "warm" figure, not the HBM-bound one
    dec_warm_ms = tm.once(lambda i: wl.split(0), 64)
    append_ms = tm.once(wl.append, 64)

    step_s = step_ms / 1e3
    value = (wl.kv_bytes + wl.app_bytes) / step_s / 1e9
    dec_gbs = wl.kv_bytes / (dec_ms / 1e3) / 1e9
    traffic = read_traffic(w.name) if vbits == 3 and kbits == 3 else None
    B, H = w.batch, w.n_kv_heads
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
        "dtype": DTYPE,
        "data": "synthetic (seeded; outlier-channel K where the workload says so)",
        "config": {"workload": w.name, "batch": B, "n_q_heads": w.n_q_heads, "n_kv_heads": H,
                   "head_dim": d, "n_q": w.n_q, "context": int(wl.lens.max()) if B == 1 else
                   [int(wl.lens.min()), int(wl.lens.max())], "ctx_tokens": wl.ctx_tokens,
                   "input_dtype": w.dtype, "page_size": 256, "rotating_copies": wl.R,
                   "v_bits": vbits, "k_bits": kbits,
                   "step": "tq_append_decode: append the step's tokens (encode K+V) and decode "
                           "(prologue, split-K, merge)"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "ctx_tokens_per_s": round(wl.ctx_tokens / step_s, 1),
        "step_us_median5": round(step_med_ms * 1e3, 3),
        "step_us_repeats": [round(r * 1e3, 3) for r in step_runs],
        "decode_kernel_us": round(dec_ms * 1e3, 3),
        "decode_kernel_us_repeats": [round(r * 1e3, 3) for r in dec_runs],
        "decode_kernel_us_warm_single_copy": round(dec_warm_ms * 1e3, 3),
        "merge_kernel_us": round(merge_ms * 1e3, 3),
        "append_encode_us": round(append_ms * 1e3, 3),
        "platform": platform_info(),
        "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "decode_mfma_kernel",
                     "bytes_per_launch": wl.kv_bytes},
    }
    result.update(wl.encode_rates())
    if args.prefill_chunk > 0 and int(wl.lens.min()) >= args.prefill_chunk:
        pa = prefill_attention(wl, args.prefill_chunk, tm, log)
        if pa is not None:
            result["prefill_attention"] = pa
    if wl.dense is not None:
        result["dense_bf16_baseline"] = dense_baseline(wl, tm, dec_ms, log)
    cpu_inputs = None
    if not args.no_cpu_baseline:
        cpu_inputs = (wl.copies[0].k_pool.cpu().numpy(), wl.copies[0].v_pool.cpu().numpy())
    head = (w, wl.lens, wl.table_np)
    del wl
    torch.cuda.empty_cache()

    # ---- the other workloads: median-of-5 records
    others = [] if args.also.strip().lower() in ("", "none") else [int(x) for x in args.also.split(",")]
    records = {}
    for n in others:
        if n == args.workload:
            continue
        wo = I.workload(n)
        wlo = Workload(wo, dev, vbits, kbits, log, keep_dense=not args.no_dense_baseline)
        big = wo.head_dim * wo.batch * int(wlo.lens.max()) > 128 * 200000
        records[wo.name] = workload_record(wlo, tm, log, steps=16 if big else 64,
                                           launches=32 if big else 128)
        del wlo
        torch.cuda.empty_cache()
    if records:
        result["workloads"] = records

    if cpu_inputs is not None:
        log("[bench] timing the CPU reference on a bounded sample")
        hw, hlens, htable = head
        result["cpu_baseline"] = cpu_baseline(hw, hlens, cpu_inputs[0], cpu_inputs[1], htable,
                                              I.queries(hw, 0), v_bits=vbits, k_bits=kbits)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
