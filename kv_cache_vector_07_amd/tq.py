"""ctypes binding of libtq.so: one Python function per C entry point, same names.

Only argument marshalling happens here: every step of encode, decode and
dequantisation runs in the HIP kernels behind the C ABI. torch supplies device
memory and the current HIP stream. If the library is not built this module
raises instead of computing anything another way.
"""

from __future__ import annotations

import ctypes as C
import math
import os

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtq.so")
_lib = None

TQ_OK, TQ_EINVAL, TQ_EUNSUPPORTED, TQ_EALIGN, TQ_EWORKSPACE, TQ_EHIP = 0, -1, -2, -3, -4, -5
TQ_ESCRATCH = -6
TQ_STATIC_SCRATCH_BYTES = 64 << 20
TQ_F32, TQ_BF16 = 0, 1
TQ_PAGE_SIZE = 256
TQ_MAX_GROUP = 4096
EXPORTS = ("tq_k_page_bytes", "tq_v_page_bytes", "tq_k_page_bytes_bits", "tq_v_page_bytes_bits",
           "tq_build_codebook",
           "tq_build_codebook_sphere",
           "tq_encode_k",
           "tq_encode_v", "tq_query_prepare", "tq_attn_decode", "tq_attn_decode_window",
           "tq_append_decode", "tq_append_decode_static",
           "tq_attn_decode_prepared", "tq_attn_decode_split", "tq_attn_decode_merge",
           "tq_dense_attn_decode", "tq_dequant", "tq_status_string")


class TqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class TqCacheDesc(C.Structure):
    """Mirror of struct tq_cache."""
    _fields_ = [("head_dim", C.c_int32), ("n_kv_heads", C.c_int32), ("page_size", C.c_int32),
                ("n_pages", C.c_int32), ("k_pool", C.c_void_p), ("v_pool", C.c_void_p),
                ("qjl", C.c_void_p), ("levels", C.c_float * 8), ("thresholds", C.c_float * 7),
                ("k_mse_only", C.c_int32), ("v_bits", C.c_int32), ("v_levels", C.c_float * 16),
                ("v_thresholds", C.c_float * 15), ("k_bits", C.c_int32), ("k_levels", C.c_float * 16),
                ("k_thresholds", C.c_float * 15)]


def lib():
    """Load libtq.so once; raise loudly when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m kv_cache_vector_07_amd.build` (hipcc, gfx950)")
    L = C.CDLL(_LIB_PATH)
    vp, i32, f32, sz = C.c_void_p, C.c_int32, C.c_float, C.c_size_t
    L.tq_k_page_bytes.argtypes = [i32, i32]
    L.tq_k_page_bytes.restype = sz
    L.tq_v_page_bytes.argtypes = [i32, i32]
    L.tq_v_page_bytes.restype = sz
    L.tq_v_page_bytes_bits.argtypes = [i32, i32, i32]
    L.tq_v_page_bytes_bits.restype = sz
    L.tq_k_page_bytes_bits.argtypes = [i32, i32, i32]
    L.tq_k_page_bytes_bits.restype = sz
    L.tq_status_string.argtypes = [i32]
    L.tq_status_string.restype = C.c_char_p
    L.tq_build_codebook.argtypes = [i32, i32, C.c_uint64, vp, vp, vp]
    L.tq_build_codebook_sphere.argtypes = [i32, i32, C.c_uint64, vp, vp, vp]
    L.tq_encode_k.argtypes = [vp, vp, i32, vp, i32, vp]
    L.tq_encode_v.argtypes = [vp, vp, i32, vp, i32, vp]
    L.tq_query_prepare.argtypes = [vp, vp, i32, i32, i32, i32, vp, C.POINTER(sz), vp]
    L.tq_attn_decode.argtypes = [vp, vp, i32, i32, i32, i32, vp, i32, vp, i32, f32, vp, vp,
                                 C.POINTER(sz), vp]
    L.tq_attn_decode_window.argtypes = [vp, vp, i32, i32, i32, i32, vp, i32, vp, vp, i32, f32, vp,
                                        vp, C.POINTER(sz), vp]
    L.tq_append_decode.argtypes = [vp, vp, vp, i32, vp, i32, vp, i32, i32, i32, i32, vp, i32, vp,
                                   i32, f32, vp, vp, C.POINTER(sz), vp]
    L.tq_append_decode_static.argtypes = [vp, vp, vp, i32, vp, i32, vp, i32, i32, i32, i32, vp, i32,
                                          vp, i32, f32, vp, vp]
    L.tq_attn_decode_prepared.argtypes = [vp, vp, i32, i32, i32, vp, i32, vp, i32, f32, vp, vp,
                                          C.POINTER(sz), vp]
    L.tq_attn_decode_split.argtypes = [vp, vp, i32, i32, i32, vp, i32, vp, i32, f32, vp,
                                       C.POINTER(sz), vp]
    L.tq_attn_decode_merge.argtypes = [vp, i32, i32, i32, i32, vp, vp, sz, vp]
    L.tq_dequant.argtypes = [vp, i32, i32, vp, i32, vp, vp]
    L.tq_dense_attn_decode.argtypes = [vp, vp, i32, i32, i32, vp, i32, i32, i32, i32, vp, f32,
                                       vp, vp, C.POINTER(sz), vp]
    for name in ("tq_build_codebook", "tq_build_codebook_sphere", "tq_encode_k", "tq_encode_v", "tq_query_prepare",
                 "tq_attn_decode", "tq_attn_decode_window", "tq_append_decode", "tq_append_decode_static",
                 "tq_attn_decode_prepared",
                 "tq_attn_decode_split",
                 "tq_attn_decode_merge", "tq_dense_attn_decode", "tq_dequant"):
        getattr(L, name).restype = i32
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().tq_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != TQ_OK:
        raise TqError(status, where)


def _stream(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return TQ_F32
    if t.dtype == torch.bfloat16:
        return TQ_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def tq_k_page_bytes(head_dim: int, page_size: int = TQ_PAGE_SIZE, bits: int = 3) -> int:
    return int(lib().tq_k_page_bytes_bits(head_dim, page_size, bits))


def tq_v_page_bytes(head_dim: int, page_size: int = TQ_PAGE_SIZE, bits: int = 3) -> int:
    return int(lib().tq_v_page_bytes_bits(head_dim, page_size, bits))


def tq_build_codebook(head_dim: int, bits: int = 3, qjl_seed: int = 12345, with_qjl: bool = True,
                      density: str = "gaussian"):
    """Host-only: (levels float32[2^bits], thresholds float32[2^bits - 1], S float32[d][d]
    or None). density "gaussian" fits N(0, 1/d); "sphere" the exact law of a
    coordinate of a uniform unit vector (tq_build_codebook_sphere)."""
    n = 1 << bits if 2 <= bits <= 4 else 16
    levels = np.zeros(n, np.float32)
    thr = np.zeros(n - 1, np.float32)
    S = np.zeros((head_dim, head_dim), np.float32) if with_qjl and head_dim > 0 else None
    fn = {"gaussian": "tq_build_codebook", "sphere": "tq_build_codebook_sphere"}[density]
    st = getattr(lib(), fn)(head_dim, bits, qjl_seed, levels.ctypes.data, thr.ctypes.data,
                            S.ctypes.data if S is not None else None)
    _check(st, fn)
    return levels, thr, S


class Cache:
    """Caller-side owner of one packed cache: device pools, the QJL matrix and
    the descriptor passed to every call. Pools are allocated with torch."""

    def __init__(self, head_dim: int, n_kv_heads: int, n_pages: int, qjl_seed: int = 12345,
                 device="cuda", codebook=None, zero: bool = True, k_mse_only: bool = False,
                 v_bits: int = 3, v_codebook=None, k_bits: int = 3, k_codebook=None):
        import torch
        self.head_dim, self.n_kv_heads, self.n_pages = head_dim, n_kv_heads, n_pages
        self.page_size = TQ_PAGE_SIZE
        self.qjl_seed = qjl_seed
        levels, thr, S = codebook if codebook is not None else tq_build_codebook(head_dim, 3, qjl_seed)
        self.levels, self.thresholds, self.qjl_host = levels, thr, S
        # V codes of v_bits bits: 3 shares the K codebook; 2 and 4 bring their own
        self.v_bits = int(v_bits)
        if self.v_bits == 3:
            vlev, vthr = levels, thr
        else:
            vlev, vthr = (v_codebook if v_codebook is not None
                          else tq_build_codebook(head_dim, self.v_bits, qjl_seed, with_qjl=False)[:2])
        self.v_levels, self.v_thresholds = vlev, vthr
        # K codes of k_bits bits: 3 uses the codebook above; 2 and 4 bring their own
        self.k_bits = int(k_bits)
        if self.k_bits == 3:
            klev, kthr = levels, thr
        else:
            klev, kthr = (k_codebook if k_codebook is not None
                          else tq_build_codebook(head_dim, self.k_bits, qjl_seed, with_qjl=False)[:2])
        self.k_levels, self.k_thresholds = klev, kthr
        kpb = tq_k_page_bytes(head_dim, bits=self.k_bits)
        vpb = tq_v_page_bytes(head_dim, bits=self.v_bits)
        alloc = torch.zeros if zero else torch.empty
        self.k_pool = alloc(n_pages * n_kv_heads * kpb, dtype=torch.uint8, device=device)
        self.v_pool = alloc(n_pages * n_kv_heads * vpb, dtype=torch.uint8, device=device)
        self.qjl = torch.from_numpy(S).to(device)
        vl = np.zeros(16, np.float32)
        vt = np.zeros(15, np.float32)
        vl[:len(vlev)] = vlev
        vt[:len(vthr)] = vthr
        kl = np.zeros(16, np.float32)
        kt = np.zeros(15, np.float32)
        kl[:len(klev)] = klev
        kt[:len(kthr)] = kthr
        self.desc = TqCacheDesc(head_dim, n_kv_heads, self.page_size, n_pages,
                                self.k_pool.data_ptr(), self.v_pool.data_ptr(), self.qjl.data_ptr(),
                                (C.c_float * 8)(*levels.tolist()), (C.c_float * 7)(*thr.tolist()),
                                int(k_mse_only), self.v_bits, (C.c_float * 16)(*vl.tolist()),
                                (C.c_float * 15)(*vt.tolist()), self.k_bits,
                                (C.c_float * 16)(*kl.tolist()), (C.c_float * 15)(*kt.tolist()))
        self.k_mse_only = bool(k_mse_only)
        self._ws = None

    @property
    def ref(self):
        return C.byref(self.desc)

    def workspace(self, nbytes: int):
        """A zero-initialised decode workspace of at least nbytes, reused across calls."""
        import torch
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=self.k_pool.device)
        return self._ws


def tq_encode_k(cache: Cache, k, slots, stream=None) -> None:
    """k: [n_tokens][Hkv][d] float32/bfloat16 on the device; slots: int32 [n_tokens]."""
    st = lib().tq_encode_k(cache.ref, k.data_ptr(), _dtype_code(k), slots.data_ptr(),
                           int(slots.numel()), _stream(stream))
    _check(st, "tq_encode_k")


def tq_encode_v(cache: Cache, v, slots, stream=None) -> None:
    st = lib().tq_encode_v(cache.ref, v.data_ptr(), _dtype_code(v), slots.data_ptr(),
                           int(slots.numel()), _stream(stream))
    _check(st, "tq_encode_v")


def tq_query_prepare(cache: Cache, q, prep=None, stream=None):
    """q: [B][n_q][Hq][d] -> the prepared-query buffer (uint8 device tensor) whose
    first B*n_q*Hq*2*d float32 values are (Pi q, S Pi q) per row."""
    import torch
    B, n_q, Hq, d = q.shape
    size = C.c_size_t(0)
    L = lib()
    _check(L.tq_query_prepare(cache.ref, q.data_ptr(), _dtype_code(q), B, n_q, Hq, None,
                              C.byref(size), None), "tq_query_prepare (size query)")
    if prep is None:
        prep = torch.empty(size.value, dtype=torch.uint8, device=q.device)
    size = C.c_size_t(prep.numel())
    _check(L.tq_query_prepare(cache.ref, q.data_ptr(), _dtype_code(q), B, n_q, Hq, prep.data_ptr(),
                              C.byref(size), _stream(stream)), "tq_query_prepare")
    return prep


def prepared_rows(prep, shape):
    """View of the (Pi q, S Pi q) rows of a prepared-query buffer: [..., 2, d] float32."""
    B, n_q, Hq, d = shape
    n = B * n_q * Hq * 2 * d
    return prep[: 4 * n].view(dtype=__import__("torch").float32).view(B, n_q, Hq, 2, d)


def _decode_ws(cache, fn, args, workspace):
    size = C.c_size_t(0)
    st = fn(*args(None), C.byref(size), None)
    _check(st, fn.__name__ + " (workspace query)")
    ws = workspace if workspace is not None else cache.workspace(size.value)
    return ws, size


def tq_attn_decode(cache: Cache, q, block_table, seq_lens, causal_tail: int = 0, scale=None,
                   out=None, workspace=None, stream=None):
    """q: [B][n_q][Hq][d]; block_table: int32 [B][max_pages]; seq_lens: int32 [B]."""
    import torch
    B, n_q, Hq, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty(B, n_q, Hq, d, dtype=torch.float32, device=q.device)
    L = lib()
    args = lambda ws: (cache.ref, q.data_ptr(), _dtype_code(q), B, n_q, Hq, block_table.data_ptr(),
                       int(block_table.shape[1]), seq_lens.data_ptr(), int(causal_tail), scale,
                       out.data_ptr(), ws)
    ws, size = _decode_ws(cache, L.tq_attn_decode, args, workspace)
    size = C.c_size_t(ws.numel())
    st = L.tq_attn_decode(*args(ws.data_ptr()), C.byref(size), _stream(stream))
    _check(st, "tq_attn_decode")
    return out


def tq_attn_decode_window(cache: Cache, q, block_table, seq_lens, seq_starts, causal_tail: int = 0,
                          scale=None, out=None, workspace=None, stream=None):
    """tq_attn_decode where sequence b sees only tokens j >= seq_starts[b] (int32 [B])."""
    import torch
    B, n_q, Hq, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty(B, n_q, Hq, d, dtype=torch.float32, device=q.device)
    L = lib()
    args = lambda ws: (cache.ref, q.data_ptr(), _dtype_code(q), B, n_q, Hq, block_table.data_ptr(),
                       int(block_table.shape[1]), seq_lens.data_ptr(), seq_starts.data_ptr(),
                       int(causal_tail), scale, out.data_ptr(), ws)
    ws, size = _decode_ws(cache, L.tq_attn_decode_window, args, workspace)
    size = C.c_size_t(ws.numel())
    st = L.tq_attn_decode_window(*args(ws.data_ptr()), C.byref(size), _stream(stream))
    _check(st, "tq_attn_decode_window")
    return out


def tq_append_decode(cache: Cache, k_new, v_new, slots, q, block_table, seq_lens,
                     causal_tail: int = 0, scale=None, out=None, workspace=None, stream=None):
    """Encode k_new / v_new ([n][Hkv][d]) into `slots`, then decode q ([B][n_q][Hq][d])
    over the updated cache; seq_lens must already count the new tokens."""
    import torch
    B, n_q, Hq, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty(B, n_q, Hq, d, dtype=torch.float32, device=q.device)
    n_new = int(slots.numel())
    L = lib()
    args = lambda ws: (cache.ref, k_new.data_ptr(), v_new.data_ptr(), _dtype_code(k_new),
                       slots.data_ptr(), n_new, q.data_ptr(), _dtype_code(q), B, n_q, Hq,
                       block_table.data_ptr(), int(block_table.shape[1]), seq_lens.data_ptr(),
                       int(causal_tail), scale, out.data_ptr(), ws)
    ws, size = _decode_ws(cache, L.tq_append_decode, args, workspace)
    size = C.c_size_t(ws.numel())
    st = L.tq_append_decode(*args(ws.data_ptr()), C.byref(size), _stream(stream))
    _check(st, "tq_append_decode")
    return out


def tq_append_decode_static(cache: Cache, k_new, v_new, slots, q, block_table, seq_lens,
                            causal_tail: int = 0, scale=None, out=None, stream=None):
    """tq_append_decode with the library's static device scratch instead of a
    workspace: the call allocates nothing (out is allocated here only when not
    given)."""
    import torch
    B, n_q, Hq, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty(B, n_q, Hq, d, dtype=torch.float32, device=q.device)
    n_new = int(slots.numel())
    st = lib().tq_append_decode_static(cache.ref, k_new.data_ptr(), v_new.data_ptr(), _dtype_code(k_new),
                                       slots.data_ptr(), n_new, q.data_ptr(), _dtype_code(q), B, n_q, Hq,
                                       block_table.data_ptr(), int(block_table.shape[1]),
                                       seq_lens.data_ptr(), int(causal_tail), scale, out.data_ptr(),
                                       _stream(stream))
    _check(st, "tq_append_decode_static")
    return out


def tq_attn_decode_prepared(cache: Cache, prep, q_shape, block_table, seq_lens,
                            causal_tail: int = 0, scale=None, out=None, workspace=None,
                            stream=None):
    """prep: buffer from tq_query_prepare for queries of shape q_shape = (B, n_q, Hq, d)."""
    import torch
    B, n_q, Hq, d = q_shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty(B, n_q, Hq, d, dtype=torch.float32, device=prep.device)
    L = lib()
    args = lambda ws: (cache.ref, prep.data_ptr(), B, n_q, Hq, block_table.data_ptr(),
                       int(block_table.shape[1]), seq_lens.data_ptr(), int(causal_tail), scale,
                       out.data_ptr(), ws)
    ws, size = _decode_ws(cache, L.tq_attn_decode_prepared, args, workspace)
    size = C.c_size_t(ws.numel())
    st = L.tq_attn_decode_prepared(*args(ws.data_ptr()), C.byref(size), _stream(stream))
    _check(st, "tq_attn_decode_prepared")
    return out


def tq_attn_decode_split(cache: Cache, prep, q_shape, block_table, seq_lens, workspace,
                         causal_tail: int = 0, scale=None, stream=None) -> None:
    """Split-K pass only: partials land in `workspace` (uint8 device tensor)."""
    B, n_q, Hq, d = q_shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    size = C.c_size_t(workspace.numel())
    st = lib().tq_attn_decode_split(cache.ref, prep.data_ptr(), B, n_q, Hq, block_table.data_ptr(),
                                    int(block_table.shape[1]), seq_lens.data_ptr(), int(causal_tail),
                                    scale, workspace.data_ptr(), C.byref(size), _stream(stream))
    _check(st, "tq_attn_decode_split")


def tq_attn_decode_merge(cache: Cache, q_shape, max_pages: int, workspace, out=None, stream=None):
    """Merge pass only: combines the partials in `workspace` into out [B][n_q][Hq][d]."""
    import torch
    B, n_q, Hq, d = q_shape
    if out is None:
        out = torch.empty(B, n_q, Hq, d, dtype=torch.float32, device=workspace.device)
    st = lib().tq_attn_decode_merge(cache.ref, B, n_q, Hq, int(max_pages), out.data_ptr(),
                                    workspace.data_ptr(), int(workspace.numel()), _stream(stream))
    _check(st, "tq_attn_decode_merge")
    return out


def tq_dequant(cache: Cache, which: int, with_qjl: int, slots, out=None, stream=None):
    """which 0 = K, 1 = V; returns float32 [n_tokens][Hkv][d] in the original domain."""
    import torch
    n = int(slots.numel())
    if out is None:
        out = torch.empty(n, cache.n_kv_heads, cache.head_dim, dtype=torch.float32,
                          device=slots.device)
    st = lib().tq_dequant(cache.ref, int(which), int(with_qjl), slots.data_ptr(), n,
                          out.data_ptr(), _stream(stream))
    _check(st, "tq_dequant")
    return out


def tq_dense_attn_decode(k, v, q, seq_lens, scale=None, out=None, workspace=None, stream=None):
    """Uncompressed baseline. k, v: bf16 [B][Hkv][max_len][d]; q: [B][n_q][Hq][d]."""
    import torch
    B, Hkv, max_len, d = k.shape
    _, n_q, Hq, _ = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty(B, n_q, Hq, d, dtype=torch.float32, device=q.device)
    L = lib()
    args = lambda ws: (k.data_ptr(), v.data_ptr(), d, Hkv, max_len, q.data_ptr(), _dtype_code(q), B,
                       n_q, Hq, seq_lens.data_ptr(), scale, out.data_ptr(), ws)
    size = C.c_size_t(0)
    _check(L.tq_dense_attn_decode(*args(None), C.byref(size), None), "tq_dense_attn_decode (size)")
    ws = workspace if workspace is not None else torch.empty(size.value, dtype=torch.uint8, device=q.device)
    size = C.c_size_t(ws.numel())
    _check(L.tq_dense_attn_decode(*args(ws.data_ptr()), C.byref(size), _stream(stream)),
           "tq_dense_attn_decode")
    return out
