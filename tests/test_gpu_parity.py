"""GPU parity: the HIP path (through the C ABI) against the CPU reference on
the same seeded inputs, at sizes the reference finishes in seconds that still
span several pages and ragged tails."""

import math

import numpy as np
import pytest

import oracle as O
from kv_cache_vector_07_amd import inputs as I
from tests import harness as Hn

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_vector_07_amd import tq as _tq
    _tq.lib()
    return _tq


def _wl(d, dtype, dist, seed, H=8, Hq=32):
    return I.Workload(f"t{seed}", 1, Hq, H, d, dtype, dist, seed, fixed_len=1)


ENC_CASES = [
    # (d, dtype, k_dist, n_tokens, H, seed)
    (128, "f32", "normal", 1024, 1, 1),     # tiny reference workload, full size
    (128, "bf16", "outlier", 1500, 8, 2),
    (256, "bf16", "outlier", 700, 8, 5),
    (128, "bf16", "normal", 333, 3, 4),
]


def _enc_inputs(d, dtype, dist, n, H, seed):
    w = _wl(d, dtype, dist, seed, H=H)
    k = I.kv_tokens(w, "k", 0, 0, n)
    v = I.kv_tokens(w, "v", 0, 0, n)
    return w, k, v


@pytest.mark.parametrize("case", ENC_CASES, ids=lambda c: f"d{c[0]}-{c[1]}-{c[2]}-n{c[3]}-H{c[4]}")
def test_encode_parity(tq, case):
    d, dtype, dist, n, H, seed = case
    print(f"[encode parity] d={d} {dtype} {dist} n={n} H={H}", flush=True)
    w, k, v = _enc_inputs(*case)
    n_pages = (n + 255) // 256 + 2
    cache = tq.Cache(d, H, n_pages, zero=False)
    g0 = torch.Generator(device="cpu").manual_seed(seed)
    kp0 = torch.randint(0, 256, (cache.k_pool.numel(),), generator=g0, dtype=torch.uint8)
    vp0 = torch.randint(0, 256, (cache.v_pool.numel(),), generator=g0, dtype=torch.uint8)
    cache.k_pool.copy_(kp0)
    cache.v_pool.copy_(vp0)
    slots = np.random.default_rng(seed).permutation(n_pages * 256)[:n].astype(np.int32)
    ts = torch.from_numpy(slots).cuda()
    tq.tq_encode_k(cache, Hn.torch_input(k, dtype), ts)
    tq.tq_encode_v(cache, Hn.torch_input(v, dtype), ts)
    torch.cuda.synchronize()
    kp, vp = cache.k_pool.cpu().numpy(), cache.v_pool.cpu().numpy()
    cb = Hn.codebook_from_cache(cache)
    gk = O.unpack_k(kp, slots, H, d, 256)
    gv = O.unpack_v(vp, slots, H, d, 256)
    rk = Hn.compare_encode_k(gk, k.astype(np.float64), cb, Hn.oracle_qjl(cache))
    rv = Hn.compare_encode_v(gv, v.astype(np.float64), cb)
    print("K boundary report", rk, "V boundary report", rv)
    # untouched records keep their bytes
    others = np.setdiff1d(np.arange(n_pages * 256), slots)[:200].astype(np.int64)
    a, b = O.unpack_k(kp, others, H, d, 256), O.unpack_k(kp0.numpy(), others, H, d, 256)
    assert np.array_equal(a["idx"], b["idx"]) and np.array_equal(a["sign"], b["sign"])
    assert np.array_equal(a["N"].view(np.uint16), b["N"].view(np.uint16))
    a, b = O.unpack_v(vp, others, H, d, 256), O.unpack_v(vp0.numpy(), others, H, d, 256)
    assert np.array_equal(a["idx"], b["idx"])
    assert np.array_equal(a["N"].view(np.uint16), b["N"].view(np.uint16))


@pytest.mark.parametrize("n", [70, 2100], ids=["append-path", "bulk-path"])
def test_encode_deterministic_and_edge_vectors(tq, n):
    """Zero, one-hot and fp16-overflowing vectors, on the short-append kernels
    (n * H < 4096) and on the bulk ones."""
    d, H = 128, 2
    rng = np.random.default_rng(9)
    k = rng.standard_normal((n, H, d)).astype(np.float32)
    k[3, 0] = 0.0                  # zero vector: N = 0, all codes 4
    k[5, 1] *= 1e4                 # norm above the fp16 range: N = +inf
    k[6, 0, :] = 0.0
    k[6, 0, 17] = 2.5              # one-hot vector
    cache = tq.Cache(d, H, (n + 100 + 255) // 256)
    ts = torch.arange(n, dtype=torch.int32, device="cuda") + 100
    kt = torch.from_numpy(k).cuda()
    tq.tq_encode_k(cache, kt, ts)
    tq.tq_encode_v(cache, kt, ts)
    first_k, first_v = cache.k_pool.clone(), cache.v_pool.clone()
    tq.tq_encode_k(cache, kt, ts)
    tq.tq_encode_v(cache, kt, ts)
    torch.cuda.synchronize()
    assert torch.equal(first_k, cache.k_pool) and torch.equal(first_v, cache.v_pool)
    cb = Hn.codebook_from_cache(cache)
    slots = ts.cpu().numpy()
    gk = O.unpack_k(cache.k_pool.cpu().numpy(), slots, H, d, 256)
    gv = O.unpack_v(cache.v_pool.cpu().numpy(), slots, H, d, 256)
    assert gk["N"][3, 0] == 0 and np.all(gk["idx"][3, 0] == 4)
    assert np.isinf(gk["N"][5, 1]) and np.isinf(gv["N"][5, 1])
    finite = np.ones((n, H), bool)
    finite[5, 1] = False
    sub = lambda dct: {kk: vv[finite][:, None] for kk, vv in dct.items()}
    Hn.compare_encode_k(sub(gk), k.astype(np.float64)[finite][:, None], cb, Hn.oracle_qjl(cache))
    Hn.compare_encode_v(sub(gv), k.astype(np.float64)[finite][:, None], cb)


def _oracle_cache(d, H, lens, dtype, dist, seed, npages_extra=3):
    """Reference-encoded, reference-packed cache and the inputs it came from."""
    w = I.Workload(f"dec{seed}", len(lens), H, H, d, dtype, dist, seed, fixed_len=1)
    table, total = I.page_table(w, np.asarray(lens), shuffle=True)
    n_pages = total + npages_extra
    cb = O.codebook(d)
    S = O.qjl_matrix(d, I.QJL_SEED)
    kp = np.zeros(n_pages * H * O.k_page_bytes(d, 256), np.uint8)
    vp = np.zeros(n_pages * H * O.v_page_bytes(d, 256), np.uint8)
    for b, L in enumerate(lens):
        if L == 0:
            continue
        k = I.kv_tokens(w, "k", b, 0, L).astype(np.float64)
        v = I.kv_tokens(w, "v", b, 0, L).astype(np.float64)
        t = np.arange(L)
        slots = table[b][t // 256].astype(np.int64) * 256 + t % 256
        ek = O.encode(k, cb, S)
        ev = O.encode(v, cb)
        O.pack_k(kp, slots, ek["idx"], ek["sign"], ek["N"], ek["G"], 256)
        O.pack_v(vp, slots, ev["idx"], ev["N"], 256)
    return table, n_pages, kp, vp, cb, S


DEC_CASES = [
    # (d, Hkv, Hq, n_q, lens, dtype, dist, causal, seed)
    (128, 1, 1, 1, [1024], "f32", "normal", 0, 1),                    # tiny workload, full size
    (128, 8, 32, 1, [2000], "bf16", "outlier", 0, 2),                 # GQA g=4
    (128, 8, 16, 1, [1500], "bf16", "outlier", 0, 3),                 # g=2
    (128, 8, 32, 1, [1, 255, 256, 257, 700, 0], "bf16", "normal", 0, 4),  # ragged, paged, empty
    (256, 8, 32, 4, [600, 300], "bf16", "outlier", 0, 5),             # d=256, 16 rows per KV head
    (256, 8, 32, 4, [600, 3], "bf16", "outlier", 1, 6),               # causal tail
    (128, 2, 6, 1, [513], "bf16", "normal", 0, 7),                    # g=3 (padded group)
    (256, 4, 16, 1, [700, 256], "bf16", "outlier", 0, 8),             # d=256, one query group
    (128, 4, 8, 2, [400, 2, 257], "bf16", "outlier", 1, 9),           # n_q=2 causal, MFMA path
    (128, 2, 16, 1, [300], "bf16", "normal", 0, 10),                  # 8 rows: two query groups
    (128, 2, 12, 1, [700, 300], "bf16", "outlier", 0, 11),            # 6 rows: two groups, one partial
    (128, 2, 24, 1, [600, 5], "bf16", "normal", 0, 12),               # 12 rows: three groups, the second workgroup half empty
    (128, 1, 16, 1, [900], "bf16", "outlier", 0, 13),                 # 16 rows at d=128: two workgroups of two groups
    (128, 2, 8, 40, [700, 300], "bf16", "normal", 0, 14),             # 160 rows per KV head
    (128, 1, 4, 64, [30, 600], "bf16", "outlier", 1, 15),             # 256 causal rows, L < n_q: zero rows
    # 8 x 8 x 20 pages: 3 pages per split, so d=128 takes the kernel that loads one block
    # ahead into two register sets (odd page counts, short and empty sequences)
    (128, 8, 32, 1, [5000, 4700, 1, 300, 5120, 4000, 0, 2500], "bf16", "outlier", 0, 30),
    (256, 2, 4, 48, [520, 47], "bf16", "outlier", 1, 16),             # d=256, 96 causal rows
]


@pytest.mark.parametrize("d", [128, 256])
def test_decode_query_extremes(tq, d):
    """The query operand is four fp6 limbs with power-of-two block scales (about
    2^-18 of each 32-coordinate block's largest term), so the score error grows
    with the logits: a zero query, a query scaled by 1e-4 or by 1e3 (logits near
    1e4, softmax near one-hot) and queries with one large coordinate before or
    after the rotation all stay within tolerance. (At 1e4 times the workloads'
    query norm the error passes 2e-3.)"""
    H, Hq, lens = 2, 8, [700, 300]
    table, n_pages, kp, vp, cb, S = _oracle_cache(d, H, lens, "f32", "outlier", 21)
    cache = tq.Cache(d, H, n_pages)
    cache.k_pool.copy_(torch.from_numpy(kp))
    cache.v_pool.copy_(torch.from_numpy(vp))
    bt = torch.from_numpy(table).cuda()
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(21)
    base = rng.standard_normal((len(lens), 1, Hq, d)).astype(np.float32)
    spike = np.full_like(base, 1e-6)
    spike[..., 5] = 3.0
    # a spike after the rotation: row 5 of the Sylvester Hadamard matrix, so the
    # rotated query has one large coordinate in one 32-coordinate block
    hrow = np.array([(-1) ** bin(5 & j).count("1") for j in range(d)], np.float32) / math.sqrt(d)
    rot_spike = (base * 1e-6 + 3.0 * hrow).astype(np.float32)
    for name, q in [("zero", np.zeros_like(base)), ("small", base * 1e-4), ("large", base * 1e3),
                    ("spike", spike), ("rotated spike", rot_spike)]:
        print(f"[query extremes] d={d} {name}", flush=True)
        ref = O.attn_decode(kp, vp, cb, S, q.astype(np.float64), table, lens, H, 256, Hn.scale_of(d))
        out = tq.tq_attn_decode(cache, Hn.torch_input(q, "f32"), bt, sl)
        torch.cuda.synchronize()
        err = Hn.attn_rel_err(out.cpu().numpy(), ref)
        print(f"  max rel err {err:.3e}")
        assert err <= Hn.ATTN_TOL, name


@pytest.mark.parametrize("case", DEC_CASES, ids=lambda c: f"d{c[0]}-H{c[1]}-Hq{c[2]}-nq{c[3]}-L{len(c[4])}-c{c[7]}")
def test_decode_parity(tq, case):
    d, H, Hq, nq, lens, dtype, dist, causal, seed = case
    print(f"[decode parity] {case}", flush=True)
    table, n_pages, kp, vp, cb, S = _oracle_cache(d, H, lens, dtype, dist, seed)
    w = I.Workload(f"q{seed}", len(lens), Hq, H, d, dtype, dist, seed, n_q=nq, fixed_len=1)
    q = I.queries(w, 0)
    ref = O.attn_decode(kp, vp, cb, S, q.astype(np.float64), table, lens, H, 256,
                        Hn.scale_of(d), causal_tail=bool(causal))
    cache = tq.Cache(d, H, n_pages)
    cache.k_pool.copy_(torch.from_numpy(kp))
    cache.v_pool.copy_(torch.from_numpy(vp))
    bt = torch.from_numpy(table).cuda()
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    qt = Hn.torch_input(q, dtype)
    out = tq.tq_attn_decode(cache, qt, bt, sl, causal_tail=causal)
    out2 = tq.tq_attn_decode(cache, qt, bt, sl, causal_tail=causal)   # workspace reuse
    torch.cuda.synchronize()
    err = Hn.attn_rel_err(out.cpu().numpy(), ref)
    print(f"max rel err {err:.3e}")
    assert err <= Hn.ATTN_TOL
    assert torch.equal(out, out2)
    # the prepared-query path gives the same bits
    prep = tq.tq_query_prepare(cache, qt)
    out3 = tq.tq_attn_decode_prepared(cache, prep, tuple(qt.shape), bt, sl, causal_tail=causal)
    # the split pass and the merge as separate calls
    ws = torch.empty(cache.workspace(0).numel(), dtype=torch.uint8, device="cuda")
    tq.tq_attn_decode_split(cache, prep, tuple(qt.shape), bt, sl, ws, causal_tail=causal)
    out4 = tq.tq_attn_decode_merge(cache, tuple(qt.shape), bt.shape[1], ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out3)
    assert torch.equal(out, out4)


@pytest.mark.parametrize("d", [128, 256])
def test_query_prepare_parity(tq, d):
    cache = tq.Cache(d, 2, 1)
    q = np.random.default_rng(3).standard_normal((3, 2, 4, d)).astype(np.float32)
    prep = tq.tq_query_prepare(cache, torch.from_numpy(q).cuda())
    rows = tq.prepared_rows(prep, q.shape).cpu().numpy()
    qt, p = O.rotate_query(q.astype(np.float64), Hn.oracle_qjl(cache))
    assert np.max(np.abs(rows[..., 0, :] - qt)) < 1e-5 * np.max(np.abs(qt))
    assert np.max(np.abs(rows[..., 1, :] - p)) < 1e-5 * np.max(np.abs(p))


@pytest.mark.parametrize("d", [128, 256])
def test_dequant_parity(tq, d):
    H, lens = 4, [700]
    table, n_pages, kp, vp, cb, S = _oracle_cache(d, H, lens, "bf16", "outlier", 11)
    cache = tq.Cache(d, H, n_pages)
    cache.k_pool.copy_(torch.from_numpy(kp))
    cache.v_pool.copy_(torch.from_numpy(vp))
    t = np.arange(lens[0])
    slots = (table[0][t // 256].astype(np.int64) * 256 + t % 256).astype(np.int32)
    ts = torch.from_numpy(slots).cuda()
    uk, uv = O.unpack_k(kp, slots, H, d, 256), O.unpack_v(vp, slots, H, d, 256)
    for which, qjl in ((0, 1), (0, 0), (1, 0)):
        got = tq.tq_dequant(cache, which, qjl, ts).cpu().numpy()
        if which == 0:
            ref = O.dequant_k(uk["idx"], uk["sign"], uk["N"], uk["G"], cb, S, bool(qjl))
        else:
            ref = O.dequant_v(uv["idx"], uv["N"], cb)
        den = np.max(np.abs(ref), axis=-1, keepdims=True)
        assert np.max(np.abs(got - ref) / den) < 1e-5, (which, qjl)
    # identity: <q, K_tilde_j> is the attention score estimate
    q = np.random.default_rng(1).standard_normal(d)
    Kt = O.dequant_k(uk["idx"], uk["sign"], uk["N"], uk["G"], cb, S)[:, 2]
    qt_, p_ = O.rotate_query(q, S)
    s = O.score(qt_, p_, uk["idx"][:, 2], uk["sign"][:, 2], uk["N"][:, 2].astype(float),
                uk["G"][:, 2].astype(float), cb, d)
    assert np.max(np.abs(Kt @ q - s)) < 1e-9 * np.max(np.abs(s))


@pytest.mark.parametrize("start", [256, 288], ids=["aligned-blocks", "unaligned"])
def test_encode_whole_blocks_and_unaligned(tq, start):
    """Bulk encode into consecutive slots: from a 64-token boundary every block is
    stored whole; from an unaligned start no block is whole (per-bit path)."""
    d, H, n, seed = 128, 8, 640, 11
    print(f"[encode blocks] start={start}", flush=True)
    w, k, v = _enc_inputs(d, "bf16", "outlier", n, H, seed)
    cache = tq.Cache(d, H, 5)
    slots = np.arange(start, start + n, dtype=np.int32)
    ts = torch.from_numpy(slots).cuda()
    tq.tq_encode_k(cache, Hn.torch_input(k, "bf16"), ts)
    tq.tq_encode_v(cache, Hn.torch_input(v, "bf16"), ts)
    torch.cuda.synchronize()
    kp, vp = cache.k_pool.cpu().numpy(), cache.v_pool.cpu().numpy()
    cb = Hn.codebook_from_cache(cache)
    Hn.compare_encode_k(O.unpack_k(kp, slots, H, d, 256), k.astype(np.float64), cb, Hn.oracle_qjl(cache))
    Hn.compare_encode_v(O.unpack_v(vp, slots, H, d, 256), v.astype(np.float64), cb)
    # slots outside the written range stay zero
    rest = np.setdiff1d(np.arange(5 * 256), slots).astype(np.int64)
    assert np.all(O.unpack_v(vp, rest, H, d, 256)["idx"] == 0)
    assert np.all(O.unpack_k(kp, rest, H, d, 256)["idx"] == 0)


@pytest.mark.parametrize("d,Hq,nq", [(128, 32, 1), (256, 32, 4)])
def test_append_decode_matches_separate_calls_and_reference(tq, d, Hq, nq):
    """tq_append_decode (encode of the appended tokens and query prepare in one
    launch) against tq_encode_k + tq_encode_v + tq_attn_decode on a twin cache,
    bit for bit, and against the reference over the updated cache."""
    H, lens0 = 8, np.array([700, 257, 64])
    print(f"[append decode] d={d} Hq={Hq} n_q={nq}", flush=True)
    w = I.Workload(f"app{d}", len(lens0), Hq, H, d, "bf16", "outlier", 31, n_q=nq, fixed_len=1)
    table, n_pages = I.page_table(w, lens0, extra_tokens=1, shuffle=True)
    caches = [tq.Cache(d, H, n_pages) for _ in range(2)]
    bt = torch.from_numpy(table).cuda()
    for c in caches:
        for b, L in enumerate(lens0):
            t = torch.arange(0, int(L), device="cuda")
            sl = (bt[b, t // 256] * 256 + t % 256).to(torch.int32)
            c_k = torch.from_numpy(I.kv_tokens(w, "k", b, 0, int(L))).to("cuda", torch.bfloat16)
            c_v = torch.from_numpy(I.kv_tokens(w, "v", b, 0, int(L))).to("cuda", torch.bfloat16)
            tq.tq_encode_k(c, c_k, sl)
            tq.tq_encode_v(c, c_v, sl)
    pos = torch.from_numpy(lens0).cuda()
    slots = (bt[torch.arange(len(lens0), device="cuda"), pos // 256] * 256 + pos % 256).to(torch.int32)
    nk = np.concatenate([I.kv_tokens(w, "k", b, int(L), int(L) + 1) for b, L in enumerate(lens0)])
    nv = np.concatenate([I.kv_tokens(w, "v", b, int(L), int(L) + 1) for b, L in enumerate(lens0)])
    nk_t = torch.from_numpy(nk).to("cuda", torch.bfloat16)
    nv_t = torch.from_numpy(nv).to("cuda", torch.bfloat16)
    lens = lens0 + 1
    sl = torch.from_numpy(lens.astype(np.int32)).cuda()
    q = I.queries(w, 0)
    qt = torch.from_numpy(q).to("cuda", torch.bfloat16)
    out_a = tq.tq_append_decode(caches[0], nk_t, nv_t, slots, qt, bt, sl)
    tq.tq_encode_k(caches[1], nk_t, slots)
    tq.tq_encode_v(caches[1], nv_t, slots)
    out_b = tq.tq_attn_decode(caches[1], qt, bt, sl)
    torch.cuda.synchronize()
    assert torch.equal(caches[0].k_pool, caches[1].k_pool)
    assert torch.equal(caches[0].v_pool, caches[1].v_pool)
    assert torch.equal(out_a, out_b)
    kp, vp = caches[0].k_pool.cpu().numpy(), caches[0].v_pool.cpu().numpy()
    cb = Hn.codebook_from_cache(caches[0])
    s_np = slots.cpu().numpy()
    Hn.compare_encode_k(O.unpack_k(kp, s_np, H, d, 256), nk.astype(np.float64), cb, Hn.oracle_qjl(caches[0]))
    Hn.compare_encode_v(O.unpack_v(vp, s_np, H, d, 256), nv.astype(np.float64), cb)
    ref = O.attn_decode(kp, vp, cb, Hn.oracle_qjl(caches[0]), q.astype(np.float64), table, lens, H, 256,
                        Hn.scale_of(d))
    err = Hn.attn_rel_err(out_a.cpu().numpy(), ref)
    print(f"  max rel err {err:.3e}", flush=True)
    assert err <= Hn.ATTN_TOL


def test_speculative_verify_and_rollback(tq):
    """Speculative verify: append n_q = 4 draft tokens per sequence, score the four
    draft queries against the cache with the causal tail (query t sees
    L - (n_q - 1 - t) tokens) and check them against the reference; then roll back
    by rewinding seq_lens. Earlier slots are never rewritten, so decoding after the
    rollback gives the same bits as before the drafts were appended."""
    d, H, Hq, nq = 128, 4, 8, 4
    lens0 = np.array([600, 255, 256])
    print("[verify rollback]", flush=True)
    w = I.Workload("spec", len(lens0), Hq, H, d, "bf16", "outlier", 41, n_q=nq, fixed_len=1)
    table, n_pages = I.page_table(w, lens0, extra_tokens=nq, shuffle=True)
    cache = tq.Cache(d, H, n_pages)
    bt = torch.from_numpy(table).cuda()
    for b, L in enumerate(lens0):
        t = torch.arange(0, int(L), device="cuda")
        sl = (bt[b, t // 256] * 256 + t % 256).to(torch.int32)
        tq.tq_encode_k(cache, torch.from_numpy(I.kv_tokens(w, "k", b, 0, int(L))).to("cuda", torch.bfloat16), sl)
        tq.tq_encode_v(cache, torch.from_numpy(I.kv_tokens(w, "v", b, 0, int(L))).to("cuda", torch.bfloat16), sl)
    # one decode step (a single query token per sequence) before the drafts
    w1 = I.Workload("spec1", len(lens0), Hq, H, d, "bf16", "outlier", 41, n_q=1, fixed_len=1)
    q1 = torch.from_numpy(I.queries(w1, 0)).to("cuda", torch.bfloat16)
    sl0 = torch.from_numpy(lens0.astype(np.int32)).cuda()
    before = tq.tq_attn_decode(cache, q1, bt, sl0).clone()
    # append the drafts and verify them in one call
    pos = np.concatenate([np.arange(L, L + nq) for L in lens0])
    bidx = np.repeat(np.arange(len(lens0)), nq)
    slots = torch.from_numpy((table[bidx, pos // 256].astype(np.int64) * 256 + pos % 256).astype(np.int32)).cuda()
    dk = np.concatenate([I.kv_tokens(w, "k", b, int(L), int(L) + nq) for b, L in enumerate(lens0)])
    dv = np.concatenate([I.kv_tokens(w, "v", b, int(L), int(L) + nq) for b, L in enumerate(lens0)])
    q = I.queries(w, 0)
    lens = lens0 + nq
    sl = torch.from_numpy(lens.astype(np.int32)).cuda()
    out = tq.tq_append_decode(cache, torch.from_numpy(dk).to("cuda", torch.bfloat16),
                              torch.from_numpy(dv).to("cuda", torch.bfloat16), slots,
                              torch.from_numpy(q).to("cuda", torch.bfloat16), bt, sl, causal_tail=1)
    torch.cuda.synchronize()
    kp, vp = cache.k_pool.cpu().numpy(), cache.v_pool.cpu().numpy()
    cb = Hn.codebook_from_cache(cache)
    ref = O.attn_decode(kp, vp, cb, Hn.oracle_qjl(cache), q.astype(np.float64), table, lens, H, 256,
                        Hn.scale_of(d), causal_tail=True)
    err = Hn.attn_rel_err(out.cpu().numpy(), ref)
    print(f"  verify max rel err {err:.3e}", flush=True)
    assert err <= Hn.ATTN_TOL
    # rollback: the drafts are rejected, seq_lens go back; the same step again
    after = tq.tq_attn_decode(cache, q1, bt, sl0)
    torch.cuda.synchronize()
    assert torch.equal(before, after)


@pytest.mark.parametrize("d,H,Hq,C", [(128, 2, 8, 128), (256, 8, 8, 200), (128, 2, 6, 67)],
                         ids=["d128-512rows-fused-prologue", "d256-200rows-separate-encode",
                              "d128-201rows-ragged-groups"])
def test_chunked_prefill_attention(tq, d, H, Hq, C):
    """Chunked prefill: C new tokens per sequence are appended (encoded) and their
    C x Hq/Hkv query rows attend causally over the compressed history and the
    chunk (causal tail: chunk token t sees the history and chunk tokens <= t).
    One sequence starts empty, so its first chunk attends to itself only. Checked
    bit for bit against separate encode + decode calls on a twin cache, and
    against the reference over the updated cache."""
    lens0 = np.array([900, 0, 37])
    print(f"[chunked prefill] d={d} Hkv={H} Hq={Hq} chunk={C}", flush=True)
    w = I.Workload(f"pre{d}", len(lens0), Hq, H, d, "bf16", "outlier", 41, n_q=C, fixed_len=1)
    table, n_pages = I.page_table(w, lens0, extra_tokens=C, shuffle=True)
    caches = [tq.Cache(d, H, n_pages) for _ in range(2)]
    bt = torch.from_numpy(table).cuda()
    for c in caches:
        for b, L in enumerate(lens0):
            if L == 0:
                continue
            t = torch.arange(0, int(L), device="cuda")
            sl = (bt[b, t // 256] * 256 + t % 256).to(torch.int32)
            tq.tq_encode_k(c, torch.from_numpy(I.kv_tokens(w, "k", b, 0, int(L))).to("cuda", torch.bfloat16), sl)
            tq.tq_encode_v(c, torch.from_numpy(I.kv_tokens(w, "v", b, 0, int(L))).to("cuda", torch.bfloat16), sl)
    pos = np.concatenate([np.arange(L, L + C) for L in lens0])
    seq = np.repeat(np.arange(len(lens0)), C)
    slots = torch.from_numpy((table[seq, pos // 256].astype(np.int64) * 256 + pos % 256).astype(np.int32)).cuda()
    nk = np.concatenate([I.kv_tokens(w, "k", b, int(L), int(L) + C) for b, L in enumerate(lens0)])
    nv = np.concatenate([I.kv_tokens(w, "v", b, int(L), int(L) + C) for b, L in enumerate(lens0)])
    nk_t = torch.from_numpy(nk).to("cuda", torch.bfloat16)
    nv_t = torch.from_numpy(nv).to("cuda", torch.bfloat16)
    lens = lens0 + C
    sl = torch.from_numpy(lens.astype(np.int32)).cuda()
    q = I.queries(w, 0)
    qt = torch.from_numpy(q).to("cuda", torch.bfloat16)
    out_a = tq.tq_append_decode(caches[0], nk_t, nv_t, slots, qt, bt, sl, causal_tail=1)
    tq.tq_encode_k(caches[1], nk_t, slots)
    tq.tq_encode_v(caches[1], nv_t, slots)
    out_b = tq.tq_attn_decode(caches[1], qt, bt, sl, causal_tail=1)
    torch.cuda.synchronize()
    assert torch.equal(caches[0].k_pool, caches[1].k_pool)
    assert torch.equal(caches[0].v_pool, caches[1].v_pool)
    assert torch.equal(out_a, out_b)
    kp, vp = caches[0].k_pool.cpu().numpy(), caches[0].v_pool.cpu().numpy()
    cb = Hn.codebook_from_cache(caches[0])
    s_np = slots.cpu().numpy()
    Hn.compare_encode_k(O.unpack_k(kp, s_np, H, d, 256), nk.astype(np.float64), cb, Hn.oracle_qjl(caches[0]))
    Hn.compare_encode_v(O.unpack_v(vp, s_np, H, d, 256), nv.astype(np.float64), cb)
    ref = O.attn_decode(kp, vp, cb, Hn.oracle_qjl(caches[0]), q.astype(np.float64), table, lens, H, 256,
                        Hn.scale_of(d), causal_tail=True)
    err = Hn.attn_rel_err(out_a.cpu().numpy(), ref)
    print(f"  max rel err {err:.3e}", flush=True)
    assert err <= Hn.ATTN_TOL


@pytest.mark.parametrize("d", [128, 256])
def test_sphere_codebook_encode_and_decode(tq, d):
    """The kernels take the codebook by value: a cache built with the exact
    sphere-coordinate codebook encodes and decodes to the reference fitted on
    that density (codes bit-exact up to boundary cases, attention within
    tolerance)."""
    H, Hq, lens = 2, 8, [700, 300]
    print(f"[sphere codebook] d={d}", flush=True)
    w = I.Workload(f"sph{d}", len(lens), Hq, H, d, "bf16", "outlier", 51, fixed_len=1)
    table, n_pages = I.page_table(w, np.asarray(lens), shuffle=True)
    cache = tq.Cache(d, H, n_pages, codebook=tq.tq_build_codebook(d, 3, 12345, density="sphere"))
    cb = Hn.codebook_from_cache(cache, density="sphere")
    bt = torch.from_numpy(table).cuda()
    for b, L in enumerate(lens):
        k = I.kv_tokens(w, "k", b, 0, L)
        v = I.kv_tokens(w, "v", b, 0, L)
        t = np.arange(L)
        slots = (table[b][t // 256].astype(np.int64) * 256 + t % 256).astype(np.int32)
        ts = torch.from_numpy(slots).cuda()
        tq.tq_encode_k(cache, Hn.torch_input(k, "bf16"), ts)
        tq.tq_encode_v(cache, Hn.torch_input(v, "bf16"), ts)
        torch.cuda.synchronize()
        kp, vp = cache.k_pool.cpu().numpy(), cache.v_pool.cpu().numpy()
        rk = Hn.compare_encode_k(O.unpack_k(kp, slots, H, d, 256), k.astype(np.float64), cb, Hn.oracle_qjl(cache))
        rv = Hn.compare_encode_v(O.unpack_v(vp, slots, H, d, 256), v.astype(np.float64), cb)
        print("  K", rk, "V", rv)
    q = I.queries(w, 0)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = tq.tq_attn_decode(cache, Hn.torch_input(q, "bf16"), bt, sl)
    torch.cuda.synchronize()
    ref = O.attn_decode(kp, vp, cb, Hn.oracle_qjl(cache), q.astype(np.float64), table, lens, H, 256,
                        Hn.scale_of(d))
    err = Hn.attn_rel_err(out.cpu().numpy(), ref)
    print(f"  max rel err {err:.3e}", flush=True)
    assert err <= Hn.ATTN_TOL


@pytest.mark.parametrize("d", [128, 256])
def test_mse_only_keys_encode_and_decode(tq, d):
    """Keys without the QJL stage (k_mse_only = 1, no S on the device): codes, N
    and G as the reference, a zero sign plane, and attention that keeps only
    the codebook term. The fused append step takes the same path."""
    H, Hq, lens = 2, 8, [700, 300]
    print(f"[mse-only keys] d={d}", flush=True)
    w = I.Workload(f"mse{d}", len(lens), Hq, H, d, "bf16", "outlier", 61, fixed_len=1)
    table, n_pages = I.page_table(w, np.asarray(lens), extra_tokens=1, shuffle=True)
    # S stays on the device: were it read, the signs or the scores would show it
    cache = tq.Cache(d, H, n_pages, k_mse_only=True)
    cb = Hn.codebook_from_cache(cache)
    bt = torch.from_numpy(table).cuda()
    for b, L in enumerate(lens):
        k = I.kv_tokens(w, "k", b, 0, L - 1)
        v = I.kv_tokens(w, "v", b, 0, L - 1)
        t = np.arange(L - 1)
        slots = (table[b][t // 256].astype(np.int64) * 256 + t % 256).astype(np.int32)
        ts = torch.from_numpy(slots).cuda()
        tq.tq_encode_k(cache, Hn.torch_input(k, "bf16"), ts)
        tq.tq_encode_v(cache, Hn.torch_input(v, "bf16"), ts)
        torch.cuda.synchronize()
        rk = Hn.compare_encode_k_mse_only(O.unpack_k(cache.k_pool.cpu().numpy(), slots, H, d, 256),
                                          k.astype(np.float64), cb)
        print("  K", rk)
    # one appended token per sequence through the fused step, then the reference
    pos = np.asarray(lens) - 1
    slots = torch.from_numpy((table[np.arange(len(lens)), pos // 256].astype(np.int64) * 256
                              + pos % 256).astype(np.int32)).cuda()
    nk = np.concatenate([I.kv_tokens(w, "k", b, L - 1, L) for b, L in enumerate(lens)])
    nv = np.concatenate([I.kv_tokens(w, "v", b, L - 1, L) for b, L in enumerate(lens)])
    q = I.queries(w, 0)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = tq.tq_append_decode(cache, Hn.torch_input(nk, "bf16"), Hn.torch_input(nv, "bf16"), slots,
                              Hn.torch_input(q, "bf16"), bt, sl)
    out2 = tq.tq_attn_decode(cache, Hn.torch_input(q, "bf16"), bt, sl)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    kp, vp = cache.k_pool.cpu().numpy(), cache.v_pool.cpu().numpy()
    Hn.compare_encode_k_mse_only(O.unpack_k(kp, slots.cpu().numpy(), H, d, 256), nk.astype(np.float64), cb)
    ref = O.attn_decode(kp, vp, cb, None, q.astype(np.float64), table, lens, H, 256, Hn.scale_of(d))
    err = Hn.attn_rel_err(out.cpu().numpy(), ref)
    print(f"  max rel err {err:.3e}", flush=True)
    assert err <= Hn.ATTN_TOL


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("Hq", [8, 32], ids=["4rows", "16rows"])
@pytest.mark.parametrize("mse", [False, True], ids=["qjl", "mse-only"])
def test_codebook_with_a_negative_parity_weight(tq, d, Hq, mse):
    """An odd codebook whose parity plane weighs less than nothing
    (c4 + c7 < c5 + c6): the 16-row kernel takes that plane's V bits
    complemented. Groups of 4 and of 16 rows, with and without the QJL stage,
    against the reference on the same codebook (float32 levels, midpoint
    thresholds)."""
    H, lens = 2, [700, 300]
    c = (np.array([0.3, 0.9, 1.4, 1.9]) / np.sqrt(d)).astype(np.float32)
    levels = np.concatenate([-c[::-1], c]).astype(np.float32)
    thr = (0.5 * (levels[:-1].astype(np.float64) + levels[1:])).astype(np.float32)
    thr[3] = 0.0
    assert 0.5 * (float(c[0]) + float(c[3]) - float(c[1]) - float(c[2])) < 0   # parity plane weight
    S = tq.tq_build_codebook(d, 3, 12345)[2]   # the cache's QJL seed: oracle_qjl checks it
    cb = O.Codebook(d, levels.astype(np.float64), thr.astype(np.float64), levels.astype(np.float64),
                    thr.astype(np.float64), 0)
    print(f"[negative parity weight] d={d} rows={Hq // H} mse_only={mse}", flush=True)
    w = I.Workload(f"npw{d}", len(lens), Hq, H, d, "bf16", "outlier", 91, fixed_len=1)
    table, n_pages = I.page_table(w, np.asarray(lens), shuffle=True)
    cache = tq.Cache(d, H, n_pages, qjl_seed=12345, codebook=(levels, thr, S), k_mse_only=mse)
    bt = torch.from_numpy(table).cuda()
    S64 = None if mse else Hn.oracle_qjl(cache)   # the oracle's own S, equal to the cache's
    for b, L in enumerate(lens):
        k = I.kv_tokens(w, "k", b, 0, L)
        v = I.kv_tokens(w, "v", b, 0, L)
        t = np.arange(L)
        slots = (table[b][t // 256].astype(np.int64) * 256 + t % 256).astype(np.int32)
        ts = torch.from_numpy(slots).cuda()
        tq.tq_encode_k(cache, Hn.torch_input(k, "bf16"), ts)
        tq.tq_encode_v(cache, Hn.torch_input(v, "bf16"), ts)
        torch.cuda.synchronize()
        kp, vp = cache.k_pool.cpu().numpy(), cache.v_pool.cpu().numpy()
        uk = O.unpack_k(kp, slots, H, d, 256)
        if mse:
            Hn.compare_encode_k_mse_only(uk, k.astype(np.float64), cb)
        else:
            Hn.compare_encode_k(uk, k.astype(np.float64), cb, S64)
        Hn.compare_encode_v(O.unpack_v(vp, slots, H, d, 256), v.astype(np.float64), cb)
    q = I.queries(w, 0)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = tq.tq_attn_decode(cache, Hn.torch_input(q, "bf16"), bt, sl)
    torch.cuda.synchronize()
    ref = O.attn_decode(kp, vp, cb, S64, q.astype(np.float64), table, lens, H, 256, Hn.scale_of(d))
    err = Hn.attn_rel_err(out.cpu().numpy(), ref)
    print(f"  max rel err {err:.3e}", flush=True)
    assert err <= Hn.ATTN_TOL


def _decode_wide_table(tq, cache, q, bt, sl):
    """Decode with the block table padded to 72 columns (the padding is never
    read): two sequences x 8 KV heads x 72 pages make 3 pages per split, so at
    d = 128 the kernel that loads one block ahead into two register sets runs."""
    wide = torch.zeros(bt.shape[0], 72, dtype=bt.dtype, device=bt.device)
    wide[:, :bt.shape[1]] = bt
    return tq.tq_attn_decode(cache, Hn.torch_input(q, "bf16"), wide, sl)


@pytest.mark.parametrize("d,vb", [(128, 2), (128, 4), (256, 2), (256, 4)])
def test_v_code_widths(tq, d, vb):
    """V codes of 2 and 4 bits (v_bits): the encode's codes and norms against the
    reference with the 4- or 16-level codebook (whole 64-token blocks and single
    tokens), dequant, the fused append step, and attention for one query row
    group, for two groups per workgroup (16 rows) and with the causal tail."""
    H, lens = 8, np.array([700, 300])
    print(f"[v bits] d={d} vb={vb}", flush=True)
    w = I.Workload(f"vb{d}{vb}", len(lens), 32, H, d, "bf16", "outlier", 70 + vb, n_q=4, fixed_len=1)
    table, n_pages = I.page_table(w, lens, extra_tokens=1, shuffle=True)
    cache = tq.Cache(d, H, n_pages, v_bits=vb)
    cb = Hn.codebook_from_cache(cache)
    cbv = O.codebook(d, vb)
    assert np.array_equal(cache.v_levels.astype(np.float64), cbv.levels)
    bt = torch.from_numpy(table).cuda()
    for b, L in enumerate(lens):
        t = np.arange(L)
        slots = (table[b][t // 256].astype(np.int64) * 256 + t % 256).astype(np.int32)
        ts = torch.from_numpy(slots).cuda()
        k = I.kv_tokens(w, "k", b, 0, L)
        v = I.kv_tokens(w, "v", b, 0, L)
        tq.tq_encode_k(cache, Hn.torch_input(k, "bf16"), ts)
        tq.tq_encode_v(cache, Hn.torch_input(v, "bf16"), ts)   # 700 x 8 vectors: whole blocks
        torch.cuda.synchronize()
        vp = cache.v_pool.cpu().numpy()
        rv = Hn.compare_encode_v(O.unpack_v(vp, slots, H, d, 256, vb), v.astype(np.float64), cbv)
        print(f"  seq {b}: V {rv}", flush=True)
        if b == 0:
            uv = O.unpack_v(vp, slots, H, d, 256, vb)
            got = tq.tq_dequant(cache, 1, 0, ts).cpu().numpy()
            ref = O.dequant_v(uv["idx"], uv["N"], cbv)
            assert np.max(np.abs(got - ref) / np.max(np.abs(ref), axis=-1, keepdims=True)) < 1e-5
    # one appended token per sequence through the fused step (single-token V encode)
    pos = lens.copy()
    aslots = torch.from_numpy((table[np.arange(2), pos // 256].astype(np.int64) * 256 + pos % 256)
                              .astype(np.int32)).cuda()
    nk = np.concatenate([I.kv_tokens(w, "k", b, int(L), int(L) + 1) for b, L in enumerate(lens)])
    nv = np.concatenate([I.kv_tokens(w, "v", b, int(L), int(L) + 1) for b, L in enumerate(lens)])
    lens1 = lens + 1
    sl = torch.from_numpy(lens1.astype(np.int32)).cuda()
    q1 = I.queries(w, 0)[:, :1].copy()                     # 4 rows per KV head
    out1 = tq.tq_append_decode(cache, Hn.torch_input(nk, "bf16"), Hn.torch_input(nv, "bf16"), aslots,
                               Hn.torch_input(q1, "bf16"), bt, sl)
    q4 = I.queries(w, 1)                                     # 16 rows, causal tail
    out4 = tq.tq_attn_decode(cache, Hn.torch_input(q4, "bf16"), bt, sl, causal_tail=1)
    out1w = _decode_wide_table(tq, cache, q1, bt, sl)
    torch.cuda.synchronize()
    kp, vp = cache.k_pool.cpu().numpy(), cache.v_pool.cpu().numpy()
    Hn.compare_encode_v(O.unpack_v(vp, aslots.cpu().numpy(), H, d, 256, vb), nv.astype(np.float64), cbv)
    for q, out, causal in ((q1, out1, False), (q4, out4, True), (q1, out1w, False)):
        ref = O.attn_decode(kp, vp, cb, Hn.oracle_qjl(cache), q.astype(np.float64), table, lens1, H, 256,
                            Hn.scale_of(d), causal_tail=causal, cb_v=cbv, v_bits=vb)
        err = Hn.attn_rel_err(out.cpu().numpy(), ref)
        print(f"  rows {q.shape[1] * 4} causal {causal}: max rel err {err:.3e}", flush=True)
        assert err <= Hn.ATTN_TOL


@pytest.mark.parametrize("d,kb,vb", [(128, 2, 3), (128, 4, 3), (256, 2, 3), (256, 4, 3),
                                     (128, 2, 2), (256, 4, 4)])
def test_k_code_widths(tq, d, kb, vb):
    """K codes of 2 and 4 bits with the QJL signs (k_bits; alone and with V of the
    same width): codes, signs, N and G of whole-block and single-token encodes
    against the reference with the 4- or 16-level codebook, dequant with and
    without the QJL term, the fused append step, and attention for 4 rows and
    16 causal rows."""
    H, lens = 8, np.array([700, 300])
    print(f"[k bits] d={d} kb={kb} vb={vb}", flush=True)
    w = I.Workload(f"kb{d}{kb}{vb}", len(lens), 32, H, d, "bf16", "outlier", 80 + kb, n_q=4, fixed_len=1)
    table, n_pages = I.page_table(w, lens, extra_tokens=1, shuffle=True)
    cache = tq.Cache(d, H, n_pages, k_bits=kb, v_bits=vb)
    cbk, cbv = O.codebook(d, kb), O.codebook(d, vb)
    assert np.array_equal(cache.k_levels.astype(np.float64), cbk.levels)
    S = Hn.oracle_qjl(cache)
    bt = torch.from_numpy(table).cuda()
    for b, L in enumerate(lens):
        t = np.arange(L)
        slots = (table[b][t // 256].astype(np.int64) * 256 + t % 256).astype(np.int32)
        ts = torch.from_numpy(slots).cuda()
        k = I.kv_tokens(w, "k", b, 0, L)
        v = I.kv_tokens(w, "v", b, 0, L)
        tq.tq_encode_k(cache, Hn.torch_input(k, "bf16"), ts)   # 700 x 8 vectors: the bulk kernel
        tq.tq_encode_v(cache, Hn.torch_input(v, "bf16"), ts)
        torch.cuda.synchronize()
        kp = cache.k_pool.cpu().numpy()
        uk = O.unpack_k(kp, slots, H, d, 256, kb)
        rk = Hn.compare_encode_k(uk, k.astype(np.float64), cbk, S)
        print(f"  seq {b}: K {rk}", flush=True)
        if b == 0:
            for qjl in (1, 0):
                got = tq.tq_dequant(cache, 0, qjl, ts).cpu().numpy()
                ref = O.dequant_k(uk["idx"], uk["sign"], uk["N"], uk["G"], cbk, S, bool(qjl))
                assert np.max(np.abs(got - ref) / np.max(np.abs(ref), axis=-1, keepdims=True)) < 1e-5
    pos = lens.copy()
    aslots = torch.from_numpy((table[np.arange(2), pos // 256].astype(np.int64) * 256 + pos % 256)
                              .astype(np.int32)).cuda()
    nk = np.concatenate([I.kv_tokens(w, "k", b, int(L), int(L) + 1) for b, L in enumerate(lens)])
    nv = np.concatenate([I.kv_tokens(w, "v", b, int(L), int(L) + 1) for b, L in enumerate(lens)])
    lens1 = lens + 1
    sl = torch.from_numpy(lens1.astype(np.int32)).cuda()
    q1 = I.queries(w, 0)[:, :1].copy()
    out1 = tq.tq_append_decode(cache, Hn.torch_input(nk, "bf16"), Hn.torch_input(nv, "bf16"), aslots,
                               Hn.torch_input(q1, "bf16"), bt, sl)
    q4 = I.queries(w, 1)
    out4 = tq.tq_attn_decode(cache, Hn.torch_input(q4, "bf16"), bt, sl, causal_tail=1)
    out1w = _decode_wide_table(tq, cache, q1, bt, sl)
    torch.cuda.synchronize()
    kp, vp = cache.k_pool.cpu().numpy(), cache.v_pool.cpu().numpy()
    Hn.compare_encode_k(O.unpack_k(kp, aslots.cpu().numpy(), H, d, 256, kb), nk.astype(np.float64), cbk, S)
    for q, out, causal in ((q1, out1, False), (q4, out4, True), (q1, out1w, False)):
        ref = O.attn_decode(kp, vp, cbk, S, q.astype(np.float64), table, lens1, H, 256, Hn.scale_of(d),
                            causal_tail=causal, cb_v=cbv, v_bits=vb, k_bits=kb)
        err = Hn.attn_rel_err(out.cpu().numpy(), ref)
        print(f"  rows {q.shape[1] * 4} causal {causal}: max rel err {err:.3e}", flush=True)
        assert err <= Hn.ATTN_TOL


WIN_CASES = [
    # (d, Hkv, Hq, n_q, lens, starts, causal, seed)
    # mid-page, page-aligned, the last token only, a start past the length (zero rows)
    (128, 2, 8, 1, [1000, 700, 300, 5], [300, 256, 299, 10], 0, 31),
    # d = 256, causal tail: the second sequence's first row sees no token
    (256, 2, 8, 4, [600, 300], [520, 297], 1, 32),
    # 16 rows at d = 128 (two workgroups per KV head), a long window
    (128, 1, 16, 1, [2100, 900], [1300, 1], 0, 33),
]


@pytest.mark.parametrize("case", WIN_CASES, ids=lambda c: f"d{c[0]}-Hq{c[2]}-nq{c[3]}-c{c[6]}")
def test_window_decode_parity(tq, case):
    """A per-sequence first visible token (a sliding window): pages wholly before
    it are not read, so their block-table entries name recycled pages here."""
    d, H, Hq, nq, lens, starts, causal, seed = case
    print(f"[window parity] {case}", flush=True)
    table, n_pages, kp, vp, cb, S = _oracle_cache(d, H, lens, "bf16", "outlier", seed)
    w = I.Workload(f"w{seed}", len(lens), Hq, H, d, "bf16", "outlier", seed, n_q=nq, fixed_len=1)
    q = I.queries(w, 0)
    recycled = table.copy()
    for b, s0 in enumerate(starts):
        # in-range pages of other sequences stand in for pages handed to them
        recycled[b, :s0 // 256] = table[(b + 1) % len(lens), 0]
    ref = O.attn_decode(kp, vp, cb, S, q.astype(np.float64), table, lens, H, 256, Hn.scale_of(d),
                        causal_tail=bool(causal), seq_starts=np.asarray(starts))
    cache = tq.Cache(d, H, n_pages)
    cache.k_pool.copy_(torch.from_numpy(kp))
    cache.v_pool.copy_(torch.from_numpy(vp))
    bt = torch.from_numpy(recycled).cuda()
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    st = torch.tensor(starts, dtype=torch.int32, device="cuda")
    qt = Hn.torch_input(q, "bf16")
    out = tq.tq_attn_decode_window(cache, qt, bt, sl, st, causal_tail=causal)
    # a window starting at token 0 is the plain call, bit for bit
    z = torch.zeros_like(st)
    bt0 = torch.from_numpy(table).cuda()
    outz = tq.tq_attn_decode_window(cache, qt, bt0, sl, z, causal_tail=causal)
    plain = tq.tq_attn_decode(cache, qt, bt0, sl, causal_tail=causal)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    err = Hn.attn_rel_err(o, ref)
    print(f"max rel err {err:.3e}")
    assert err <= Hn.ATTN_TOL
    empty = np.all(ref == 0, axis=-1)           # rows with no visible token
    assert np.all(o[empty] == 0) and not np.any(np.all(o[~empty] == 0, axis=-1))
    assert torch.equal(outz, plain)


@pytest.mark.parametrize("d,Hq,nq,lens", [(128, 16, 1, [700, 257]), (128, 32, 1, [1000, 1]),
                                          (256, 16, 2, [300, 64]), (128, 8, 2, [513, 0])])
def test_dense_baseline_parity(tq, d, Hq, nq, lens):
    """The uncompressed bf16 baseline kernel against plain softmax attention."""
    H = 8
    print(f"[dense baseline] d={d} Hq={Hq} n_q={nq} lens={lens}", flush=True)
    w = I.Workload(f"dense{d}", len(lens), Hq, H, d, "bf16", "outlier", 41, n_q=nq, fixed_len=1)
    Lm = max(max(lens), 1)
    k = np.zeros((len(lens), Lm, H, d), np.float32)
    v = np.zeros_like(k)
    for b, L in enumerate(lens):
        if L:
            k[b, :L] = I.kv_tokens(w, "k", b, 0, L)
            v[b, :L] = I.kv_tokens(w, "v", b, 0, L)
    q = I.queries(w, 0)
    # the kernel takes [B][Hkv][max_len][d]
    kt = torch.from_numpy(k).to("cuda", torch.bfloat16).permute(0, 2, 1, 3).contiguous()
    vt = torch.from_numpy(v).to("cuda", torch.bfloat16).permute(0, 2, 1, 3).contiguous()
    qt = torch.from_numpy(q).to("cuda", torch.bfloat16)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = tq.tq_dense_attn_decode(kt, vt, qt, sl).cpu().numpy()
    ref = O.dense_attn_decode(k, v, q, lens, Hn.scale_of(d))
    err = Hn.attn_rel_err(out, ref)
    print(f"  max rel err {err:.3e}", flush=True)
    assert err <= Hn.ATTN_TOL


def _fp6_e2m3(code):
    """Value of OCP fp6 e2m3 codes (sign bit 5; 1/8 steps below 2, then 1/4, 1/2)."""
    m = code & 0x1F
    v = np.where(m < 16, m / 8.0, np.where(m < 24, 2.0 + (m - 16) / 4.0, 4.0 + (m - 24) / 2.0))
    return np.where(code & 0x20, -v, v)


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("n_q", [1, 5])
def test_query_operand_layout(tq, d, n_q):
    """The packed scoring operand reconstructs its inputs. Per 32-slot block of
    MFMA mu (coordinate chunk c = mu // 5, plane pl = mu % 5), slot f holds
    y_i / value(f) as four fp6 limbs with E8M0 scales, i = 32 (block + 4 c) +
    4 (f & 7) + (f >> 3), value 0.5, 1, 2, 2 for f >> 3 = 0..3, and y = w_pl q~_i
    (code planes) or 2 kappa p_i (signs); the limbs sum to it within 2^-17 of the
    block's largest term. With 4 rows per KV head (n_q = 1) a query group has 4
    rows and MFMA mu holds row r's limbs on rows 4 r + limb; with 20 (n_q = 5)
    the rows form wide groups of 16 (the second one ragged), and limb l of row r
    sits on row r of operand (mu, l). Rows past the group are zero with unit
    scales; q~ and p come from the same buffer (checked against the oracle in
    test_query_prepare_parity)."""
    B, Hkv, Hq = 2, 2, 8
    g = Hq // Hkv
    G = g * n_q
    cache = tq.Cache(d, Hkv, 1)
    q = np.random.default_rng(40 + n_q).standard_normal((B, n_q, Hq, d)).astype(np.float32)
    prep = tq.tq_query_prepare(cache, torch.from_numpy(q).cuda())
    torch.cuda.synchronize()
    rows = tq.prepared_rows(prep, q.shape).cpu().numpy().astype(np.float64)
    raw = prep.cpu().numpy()
    wide = G >= 16
    NMU = 5 * d // 128
    RG = 16 if wide else 4
    NOP = 4 * NMU if wide else NMU
    QG = -(-G // RG)
    gbytes = NOP * (2048 + 256) + (16 * 8 if wide else 64)
    off0 = -(-(B * n_q * Hq * 2 * d * 4) // 256) * 256
    lv = cache.k_levels.astype(np.float64)
    a2 = 0.25 * (lv[4] + lv[5] + lv[6] + lv[7])
    w = [2 * (0.5 * (lv[5] + lv[7]) - a2), 2 * (0.5 * (lv[6] + lv[7]) - a2), 2 * a2,
         2 * (0.5 * (lv[4] + lv[7]) - a2)]
    kap2 = 2 * math.sqrt(math.pi / 2) / d
    f = np.arange(32)
    fv, fm = f >> 3, f & 7
    val = np.where(fv == 0, 0.5, np.where(fv == 1, 1.0, 2.0))
    worst = 0.0
    for b in range(B):
        for kvh in range(Hkv):
            for rho in range(QG):
                grp = raw[off0 + ((b * Hkv + kvh) * QG + rho) * gbytes:][:gbytes]
                ops = grp[:NOP * 2048].reshape(NOP, 64, 32)
                scl = grp[NOP * 2048:NOP * 2304].view(np.uint32).reshape(NOP, 64)
                for qloc in range(RG):
                    qq = rho * RG + qloc
                    lanes = [(mu, kb, [((mu * 4 + l) if wide else mu,
                                        16 * kb + (qloc if wide else 4 * qloc + l)) for l in range(4)])
                             for mu in range(NMU) for kb in range(4)]
                    for mu, kb, where in lanes:
                        recon = np.zeros(32)
                        for o, lane in where:
                            bits = int.from_bytes(ops[o, lane, :24].tobytes(), "little")
                            codes = np.array([(bits >> (6 * k)) & 63 for k in range(32)])
                            assert not ops[o, lane, 24:].any()
                            recon += _fp6_e2m3(codes) * 2.0 ** (int(scl[o, lane]) - 127)
                        if qq >= G:
                            assert not recon.any()
                            assert all(int(scl[o, lane]) == 127 for o, lane in where)
                            continue
                        t, hh = qq // g, qq % g
                        qt = rows[b, t, kvh * g + hh, 0]
                        p = rows[b, t, kvh * g + hh, 1]
                        c, pl = mu // 5, mu % 5
                        i = 32 * (kb + 4 * c) + 4 * fm + fv
                        y = (w[pl] * qt[i] if pl < 4 else kap2 * p[i]) / val
                        den = max(np.max(np.abs(y)), 1e-30)
                        err = np.max(np.abs(recon - y)) / den
                        worst = max(worst, err)
                        assert err < 2.0 ** -17, (b, kvh, qq, mu, kb, err)
    print(f"[operand layout] d={d} rows={G} wide={wide}: worst limb-sum error {worst:.2e} of block max")
