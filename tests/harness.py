"""Shared helpers of the GPU parity tests: build caches from the seeded
workloads, run the HIP path through the C ABI, and compare it with the CPU
reference under the stated tolerances."""

from __future__ import annotations

import math

import numpy as np

import oracle as O
from kv_cache_vector_07_amd import inputs as I

BOUNDARY = 1e-6          # codes / signs within this of a decision boundary may differ
ATTN_TOL = 2e-3          # max over rows of max|o_gpu - o_ref| / max|o_ref|
MAX_EXCEPTION_RATE = 1e-4


def torch_input(x32: np.ndarray, dtype: str, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.to(device)


def _fp16_near_midpoint(v64: np.ndarray) -> np.ndarray:
    """True where v64 is within relative 1e-6 of a binary16 rounding midpoint."""
    v64 = np.asarray(v64, np.float64)
    h = v64.astype(np.float16).astype(np.float64)
    up = np.nextafter(v64.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(v64.astype(np.float16), np.float16(-np.inf)).astype(np.float64)
    mids = np.stack([(h + up) / 2, (h + dn) / 2])
    return np.any(np.abs(mids - v64) <= 1e-6 * np.abs(v64) + 1e-30, axis=0)


def _fp16_match(gpu: np.ndarray, ref64: np.ndarray):
    """Bitwise match of fp16 sidecars, or 1 ulp where the value sits at a midpoint."""
    g = np.asarray(gpu, np.float16)
    r = np.asarray(ref64, np.float64).astype(np.float16)
    same = g.view(np.uint16) == r.view(np.uint16)
    ulp1 = np.abs(g.view(np.uint16).astype(np.int32) - r.view(np.uint16).astype(np.int32)) == 1
    excused = ~same & ulp1 & _fp16_near_midpoint(ref64)
    return same | excused, excused


def check_codes(gidx, e, cb):
    """Codes bitwise equal except next to a threshold (|y - t| < 1e-6)."""
    oidx = e["idx"]
    diff = gidx != oidx
    if not diff.any():
        return diff
    y = e["y"][diff]
    lo = np.minimum(gidx[diff], oidx[diff]).astype(np.int64)
    hi = np.maximum(gidx[diff], oidx[diff]).astype(np.int64)
    assert np.all(hi - lo == 1), "codes differ by more than one cell"
    t = cb.thresholds[lo]
    assert np.all(np.abs(y - t) < BOUNDARY), f"code mismatch away from a threshold: {np.max(np.abs(y - t))}"
    return diff


def compare_encode_k(gpu: dict, x64: np.ndarray, cb, S, rate_check: bool = True) -> dict:
    """gpu: unpacked K records [n][H][...]; x64: the exact inputs [n][H][d].
    rate_check=False leaves the exception-rate gate to a caller that sums the
    counts over many calls (a short range has too few values for a rate)."""
    e = O.encode(x64, cb, S)
    code_diff = check_codes(gpu["idx"], e, cb)
    vec_cascade = code_diff.any(axis=-1)
    S64 = S.astype(np.float64)
    z = e["z"].copy()
    gamma = e["gamma"].copy()
    if vec_cascade.any():
        # re-derive the residual from the GPU's codes, then compare signs and G to that
        r = e["y"][vec_cascade] - cb.levels[gpu["idx"][vec_cascade]]
        gamma[vec_cascade] = np.sqrt((r * r).sum(-1))
        z[vec_cascade] = r @ S64.T
    sign_ref = z >= 0
    sdiff = gpu["sign"] != sign_ref
    assert np.all(np.abs(z[sdiff]) < BOUNDARY), "QJL sign mismatch away from zero"
    okN, exN = _fp16_match(gpu["N"], e["norm"])
    okG, exG = _fp16_match(gpu["G"], gamma)
    assert okN.all(), "N sidecar mismatch"
    assert okG.all(), "G sidecar mismatch"
    n_coded = gpu["idx"].size + gpu["sign"].size + 2 * gpu["N"].size
    exc = int(code_diff.sum() + sdiff.sum() + exN.sum() + exG.sum())
    assert not rate_check or exc / n_coded < MAX_EXCEPTION_RATE, f"boundary exceptions {exc}/{n_coded}"
    return {"code_boundary": int(code_diff.sum()), "sign_boundary": int(sdiff.sum()),
            "sidecar_midpoint": int(exN.sum() + exG.sum()), "values": n_coded, "exceptions": exc}


def compare_encode_k_mse_only(gpu: dict, x64: np.ndarray, cb) -> dict:
    """K records written without the QJL stage: codes and N as compare_encode_v,
    G from the residual of the GPU's own codes (the cascade rule), and an all-zero
    sign plane."""
    e = O.encode_k_mse_only(x64, cb)
    code_diff = check_codes(gpu["idx"], e, cb)
    r = e["y"] - cb.levels[gpu["idx"]]
    gamma = np.sqrt((r * r).sum(-1))
    assert not gpu["sign"].any(), "sign plane of MSE-only keys is not zero"
    okN, exN = _fp16_match(gpu["N"], e["norm"])
    okG, exG = _fp16_match(gpu["G"], gamma)
    assert okN.all(), "N sidecar mismatch"
    assert okG.all(), "G sidecar mismatch"
    n_coded = gpu["idx"].size + 2 * gpu["N"].size
    exc = int(code_diff.sum() + exN.sum() + exG.sum())
    assert exc / n_coded < MAX_EXCEPTION_RATE, f"boundary exceptions {exc}/{n_coded}"
    return {"code_boundary": int(code_diff.sum()), "sidecar_midpoint": int(exN.sum() + exG.sum()),
            "values": n_coded}


def compare_encode_v(gpu: dict, x64: np.ndarray, cb, rate_check: bool = True) -> dict:
    e = O.encode(x64, cb)
    code_diff = check_codes(gpu["idx"], e, cb)
    okN, exN = _fp16_match(gpu["N"], e["norm"])
    assert okN.all(), "N sidecar mismatch"
    n_coded = gpu["idx"].size + gpu["N"].size
    exc = int(code_diff.sum() + exN.sum())
    assert not rate_check or exc / n_coded < MAX_EXCEPTION_RATE, f"boundary exceptions {exc}/{n_coded}"
    return {"code_boundary": int(code_diff.sum()), "sidecar_midpoint": int(exN.sum()),
            "values": n_coded, "exceptions": exc}


def attn_rel_err(gpu_out: np.ndarray, ref_out: np.ndarray) -> float:
    """max over query rows of max_i |o_gpu - o_ref| / max_i |o_ref| (zero rows
    must be exactly zero on both sides)."""
    g = np.asarray(gpu_out, np.float64).reshape(-1, gpu_out.shape[-1])
    r = np.asarray(ref_out, np.float64).reshape(-1, ref_out.shape[-1])
    den = np.max(np.abs(r), axis=1)
    num = np.max(np.abs(g - r), axis=1)
    zero = den == 0
    assert np.all(num[zero] == 0), "rows that must be zero are not"
    return float(np.max(num[~zero] / den[~zero])) if (~zero).any() else 0.0


def codebook_from_cache(cache, density: str = "gaussian"):
    """The reference's view of the codebook the cache descriptor carries (the
    reference fits it itself and checks that the descriptor holds the same bits)."""
    cb = O.codebook(cache.head_dim, density=density)
    assert np.array_equal(cache.levels.astype(np.float64), cb.levels)
    assert np.array_equal(cache.thresholds.astype(np.float64), cb.thresholds)
    return cb


def oracle_qjl(cache):
    """The reference's own QJL matrix for the cache's seed. It must equal, bit for
    bit, the matrix the cache descriptor points at (built by the library's host
    code), so the reference and the GPU see the same S without the reference
    taking it from the library."""
    S = O.qjl_matrix(cache.head_dim, cache.qjl_seed)
    assert np.array_equal(S, cache.qjl_host), "library S differs from the reference's S"
    return S


def scale_of(d: int) -> float:
    return 1.0 / math.sqrt(d)
