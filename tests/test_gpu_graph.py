"""A decode step captured in a HIP graph: the C entry points launch kernels only
(no allocation, no memset, no host synchronisation), so a caller can capture
tq_append_decode once and replay it. Every replay, with fresh queries copied
into the captured buffers and eager work between replays, must give the eager
call's bits."""

import numpy as np
import pytest

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


def test_append_decode_step_replays_in_a_graph(tq):
    d, H, Hq, L = 128, 8, 32, 4000
    w = I.Workload("graph", 1, Hq, H, d, "bf16", "outlier", 91, fixed_len=L)
    table, n_pages = I.page_table(w, np.array([L]), shuffle=True)
    cache = tq.Cache(d, H, n_pages)
    bt = torch.from_numpy(table).cuda()
    t = torch.arange(0, L, device="cuda")
    slots_all = (bt[0, t // 256] * 256 + t % 256).to(torch.int32)
    tq.tq_encode_k(cache, Hn.torch_input(I.kv_tokens(w, "k", 0, 0, L), "bf16"), slots_all)
    tq.tq_encode_v(cache, Hn.torch_input(I.kv_tokens(w, "v", 0, 0, L), "bf16"), slots_all)
    # the step re-appends the last token (idempotent) and decodes a fresh query
    slot = slots_all[L - 1:L].contiguous()
    k_new = Hn.torch_input(I.kv_tokens(w, "k", 0, L - 1, L), "bf16")
    v_new = Hn.torch_input(I.kv_tokens(w, "v", 0, L - 1, L), "bf16")
    sl = torch.tensor([L], dtype=torch.int32, device="cuda")
    qs = [Hn.torch_input(I.queries(w, s), "bf16") for s in range(3)]
    q_buf = torch.empty_like(qs[0])
    out_e = torch.empty(1, 1, Hq, d, dtype=torch.float32, device="cuda")
    out_g = torch.empty_like(out_e)
    probe = tq.tq_append_decode(cache, k_new, v_new, slot, qs[0], bt, sl)   # sizes the workspace
    ws = cache.workspace(0)
    torch.cuda.synchronize()

    eager = []
    for q in qs:
        q_buf.copy_(q)
        tq.tq_append_decode(cache, k_new, v_new, slot, q_buf, bt, sl, out=out_e, workspace=ws)
        torch.cuda.synchronize()
        eager.append(out_e.clone())
    assert torch.equal(eager[0], probe)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):   # warm up on the capture stream
            tq.tq_append_decode(cache, k_new, v_new, slot, q_buf, bt, sl, out=out_g, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        tq.tq_append_decode(cache, k_new, v_new, slot, q_buf, bt, sl, out=out_g, workspace=ws)
    torch.cuda.synchronize()
    other = torch.empty_like(out_e)
    for rep in range(2):
        for i, q in enumerate(qs):
            q_buf.copy_(q)
            out_g.zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            print(f"[graph] replay {rep}.{i}", flush=True)
            assert torch.equal(out_g, eager[i])
            # eager work on the same buffers between replays
            tq.tq_attn_decode(cache, qs[(i + 1) % 3], bt, sl, out=other, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(other, eager[(i + 1) % 3])
