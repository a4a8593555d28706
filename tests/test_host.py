"""Host-side logic on the CPU: the seeded input generator, the binding's loud
failure without the library, the one-GPU guard of the benchmark, and the
decode plan as the C ABI reports it through workspace sizes."""

import ctypes as C
import subprocess
import sys

import numpy as np
import pytest

from kv_cache_vector_07_amd import inputs as I
from kv_cache_vector_07_amd import tq


# ---- seeded inputs ------------------------------------------------------------

def test_token_ranges_are_reproducible_and_chunk_independent():
    w = I.workload(2)
    whole = I.kv_tokens(w, "k", 0, 4000, 4200)      # crosses a generation chunk
    left = I.kv_tokens(w, "k", 0, 4000, 4096)
    right = I.kv_tokens(w, "k", 0, 4096, 4200)
    assert np.array_equal(whole, np.concatenate([left, right]))
    assert np.array_equal(whole, I.kv_tokens(w, "k", 0, 4000, 4200))
    assert not np.array_equal(I.kv_tokens(w, "v", 0, 0, 8), I.kv_tokens(w, "k", 0, 0, 8))
    assert I.kv_tokens(w, "k", 0, 5, 5).shape == (0, w.n_kv_heads, w.head_dim)


def test_bf16_inputs_are_exact_bf16_values():
    w = I.workload(3)
    x = I.kv_tokens(w, "v", 0, 0, 64)
    assert np.array_equal(x.view(np.uint32) & np.uint32(0xFFFF), np.zeros(x.shape, np.uint32))
    # round to nearest even on the dropped half
    v = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9], np.float32)
    r = I.round_to_dtype(v, "bf16")
    assert r.tolist() == [1.0, 1.0 + 2.0 ** -6, 1.0]


def test_outlier_channel_scales():
    w = I.workload(2)
    s = I.k_channel_scales(w)
    assert s.shape == (w.n_kv_heads, w.head_dim)
    for h in range(w.n_kv_heads):
        big = s[h] > 2.0
        assert big.sum() == 4                                  # four outlier channels
        assert np.all((s[h][big] >= 10.0) & (s[h][big] <= 40.0))
        assert np.all((s[h][~big] >= 0.5) & (s[h][~big] <= 2.0))
    assert np.all(I.k_channel_scales(I.workload(4)) == 1.0)     # "normal" workload


def test_page_table_hands_out_every_page_once():
    w = I.workload(4)
    lens = I.seq_lens(w)
    assert lens.min() >= 4096 and lens.max() <= 16384
    table, total = I.page_table(w, lens, extra_tokens=1)
    need = [(int(L) + 1 + 255) // 256 for L in lens]
    used = np.concatenate([table[b, :n] for b, n in enumerate(need)])
    assert total == sum(need) and np.array_equal(np.sort(used), np.arange(total))
    assert not np.array_equal(used, np.arange(total))          # shuffled


# ---- the binding and the benchmark -------------------------------------------

def test_binding_fails_loudly_without_the_library(monkeypatch):
    monkeypatch.setattr(tq, "_lib", None)
    monkeypatch.setattr(tq, "_LIB_PATH", "/nonexistent/libtq.so")
    with pytest.raises(ImportError):
        tq.lib()


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stdout


# ---- the decode plan through the ABI -------------------------------------------

def _desc(d=128, H=8):
    levels, thr, _ = tq.tq_build_codebook(d, 3, 1, with_qjl=False)
    return tq.TqCacheDesc(d, H, 256, 64, 0x100000, 0x200000, 0x300000,
                          (C.c_float * 8)(*levels.tolist()), (C.c_float * 7)(*thr.tolist()))


def _prepared_ws(dsc, B, nq, Hq, maxp):
    sz = C.c_size_t(0)
    st = tq.lib().tq_attn_decode_prepared(C.byref(dsc), 0x400000, B, nq, Hq, 0x400000, maxp,
                                          0x400000, 0, 0.1, 0x400000, None, C.byref(sz), None)
    assert st == tq.TQ_OK
    return sz.value


@pytest.mark.parametrize("d", [128, 256])
def test_split_workspace_follows_the_plan(d):
    """The prepared call's workspace is the split partials alone:
    B * Hkv * n_split * rows * (d + 4) floats, rounded up to 256 B, with
    n_split = ceil(max_pages / pps) and pps = clamp(ceil(B Hkv max_pages W / T), 1, 256)
    (T = 768 for a single group of 4 rows at d = 128, else 512)
    (W = workgroups per sequence: one per wide group of 16 rows when there are 16
    rows or more, else one per one or two (d = 128) groups of 4)."""
    dsc = _desc(d)
    for B, nq, Hq, maxp in [(1, 1, 32, 128), (1, 1, 16, 391), (32, 1, 32, 64), (4, 4, 32, 512),
                            (1, 512, 32, 130), (2, 1, 8, 1)]:
        rows = Hq // 8 * nq
        if rows >= 16:
            wz = (rows + 15) // 16
        else:
            qg = (rows + 3) // 4
            per_wg = (2 if d == 128 else 1) if qg > 1 else 1
            wz = (qg + per_wg - 1) // per_wg
        # 768 workgroups for the one-group kernel at d = 128, else 512
        target = 768 if d == 128 and rows <= 4 else 512
        pps = min(256, max(1, -(-(B * 8 * maxp * wz) // target)))
        n_split = -(-maxp // pps)
        want = -(-(B * 8 * n_split * rows * (d + 4) * 4) // 256) * 256
        assert _prepared_ws(dsc, B, nq, Hq, maxp) == want, (B, nq, Hq, maxp)


# ---- the product path stands apart from the oracle ----------------------------

def test_package_never_imports_the_oracle():
    """The binding and the HIP sources name nothing under oracle/, and importing
    the package (binding included) leaves the oracle unloaded."""
    import pathlib
    root = pathlib.Path(__file__).resolve().parent.parent
    pkg = root / "kv_cache_vector_07_amd"
    for f in list(pkg.glob("*.py")) + list((pkg / "csrc").glob("*")):
        if f.is_file() and f.suffix in (".py", ".hip", ".cpp", ".h"):
            text = f.read_text()
            assert "import oracle" not in text and "from oracle" not in text, f
            assert "tq_oracle" not in text, f
    code = ("import sys; import kv_cache_vector_07_amd, kv_cache_vector_07_amd.tq, "
            "kv_cache_vector_07_amd.inputs; "
            "print(any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules))")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=120, cwd=str(root))
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "False"
