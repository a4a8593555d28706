"""tq_append_decode_static (the decode step with the library's static device
scratch, for callers that cannot allocate) against tq_append_decode with a
caller workspace: three calls in a row, each smaller than the one before (the
first with 16 query rows per KV head). Both entry points run the same kernels, so
outputs and pools must be bit-equal."""

import ctypes as C
import math

import numpy as np
import pytest

from kv_cache_vector_07_amd import inputs as I

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _caches(tq, w, lens, n_pages, table):
    """Two caches with the same encoded history (one per entry point)."""
    out = []
    bt = torch.from_numpy(table).cuda()
    for _ in range(2):
        cache = tq.Cache(w.head_dim, w.n_kv_heads, n_pages, qjl_seed=w.qjl_seed)
        for b, L in enumerate(lens):
            t = torch.arange(0, int(L) - 1, device="cuda")
            slots = (bt[b, t // 256] * 256 + t % 256).to(torch.int32)
            tq.tq_encode_k(cache, torch.from_numpy(I.kv_tokens(w, "k", b, 0, int(L) - 1)).to("cuda", torch.bfloat16), slots)
            tq.tq_encode_v(cache, torch.from_numpy(I.kv_tokens(w, "v", b, 0, int(L) - 1)).to("cuda", torch.bfloat16), slots)
        out.append(cache)
    return out, bt


def _step(tq, caches, w, bt, lens, B, n_q, step):
    """One append + decode step through both entry points: the last token of each
    of the first B sequences is appended, and n_q query tokens attend."""
    lens = np.asarray(lens[:B])
    pos = lens - 1
    slots = (bt[torch.arange(B, device="cuda"), torch.from_numpy(pos // 256).cuda()] * 256
             + torch.from_numpy(pos % 256).cuda()).to(torch.int32)
    nk = torch.from_numpy(np.concatenate([I.kv_tokens(w, "k", b, int(L) - 1, int(L)) for b, L in enumerate(lens)])).to("cuda", torch.bfloat16)
    nv = torch.from_numpy(np.concatenate([I.kv_tokens(w, "v", b, int(L) - 1, int(L)) for b, L in enumerate(lens)])).to("cuda", torch.bfloat16)
    rng = np.random.default_rng([w.data_seed, 11, step])
    q = torch.from_numpy(I.round_to_dtype(rng.standard_normal((B, n_q, w.n_q_heads, w.head_dim)).astype(np.float32),
                                          "bf16")).to("cuda", torch.bfloat16)
    sl = torch.from_numpy(lens.astype(np.int32)).cuda()
    table = bt[:B].contiguous()
    ref = tq.tq_append_decode(caches[0], nk, nv, slots, q, table, sl, causal_tail=1)
    got = tq.tq_append_decode_static(caches[1], nk, nv, slots, q, table, sl, causal_tail=1)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


def test_static_scratch_entry_matches_caller_workspace():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_vector_07_amd import tq
    tq.lib()
    w = I.Workload("no_alloc", 3, 16, 4, 128, "bf16", "outlier", 31, fixed_len=1)
    lens = [1500, 700, 2100]
    table, n_pages = I.page_table(w, np.asarray(lens), shuffle=True)
    caches, bt = _caches(tq, w, lens, n_pages, table)
    # first call: 3 sequences, 4 query tokens (16 causal rows per KV head: the
    # 16-row kernel)
    print("[no-alloc] call 1: B=3, n_q=4, L=[1500, 700, 2100]", flush=True)
    ref, got = _step(tq, caches, w, bt, lens, 3, 4, 2)
    assert np.array_equal(ref, got) and np.abs(ref).max() > 0
    assert torch.equal(caches[0].k_pool, caches[1].k_pool) and torch.equal(caches[0].v_pool, caches[1].v_pool)
    # then smaller calls, each after one that left more in the scratch: 3
    # sequences with 2 query tokens (8 causal rows per KV head, groups of 4)
    print("[no-alloc] call 2: B=3, n_q=2, L=[1500, 700, 2100]", flush=True)
    ref, got = _step(tq, caches, w, bt, lens, 3, 2, 0)
    assert np.array_equal(ref, got) and np.abs(ref).max() > 0
    assert torch.equal(caches[0].k_pool, caches[1].k_pool) and torch.equal(caches[0].v_pool, caches[1].v_pool)
    # 1 sequence, 1 query token; the scratch keeps the earlier calls' contents,
    # which this one must not depend on
    print("[no-alloc] call 3: B=1, n_q=1, L=[1500]", flush=True)
    ref, got = _step(tq, caches, w, bt, lens, 1, 1, 1)
    assert np.array_equal(ref, got) and np.abs(ref).max() > 0
    assert torch.equal(caches[0].k_pool, caches[1].k_pool) and torch.equal(caches[0].v_pool, caches[1].v_pool)
