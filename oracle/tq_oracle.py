"""Plain, slow, float64 CPU reference ("oracle") of the TurboQuant KV-cache path.

TEST INFRASTRUCTURE ONLY: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may use it. It shares no code with the HIP library or its
binding and imports nothing from them.

Sources (cited below by the short names in brackets):
  [AH]  AI Heartland news, "Apple Silicon向けSwiftLM、TurboQuant KVキャッシュ圧縮と
        SSD Expert Streamingを実装", section 技術的な詳細:
          - "TurboQuant KVキャッシュ圧縮アーキテクチャ" (Lloyd-Max codebook, fused dequant)
          - "K-Cache圧縮: 3-bit PolarQuant + 1-bit QJL = 4.25 bits/dim" (flow steps 1-5
            and the reason QJL is kept: inner-product attention scoring)
          - "V-Cache圧縮: 3-bit PolarQuant = 3.125 bits/dim" (V skips QJL)
  [TF]  techfi24, "SwiftLM : serveur d'inférence MLX natif pour Apple Silicon",
        section "Contexte Technique" (polar quantisation + QJL residual correction)
  [AL]  agentlenshq project page "SharpAI/SwiftLM", section 주요 기능 및 혁신,
        TurboQuant bullet (long-context decode is bandwidth bound)

Readings of points the pages leave open are listed in the repository's design
notes; the ones that shape arithmetic are restated where they are used:
  R1  sidecars: K keeps two fp16 scalars (norm N, residual norm G), V one (N);
      the only split that yields exactly 4.25 and 3.125 bits/dim at d = 128.
  R3  the rotation is the plain normalised Sylvester Hadamard matrix H_d/sqrt(d)
      (no random sign diagonal).
  R4  the codebook is the 8-level Lloyd-Max quantiser of N(0, 1/d), fitted on the
      continuous density; both encoder and decoder use its float32 rounding.
  R5  a coordinate equal to a threshold goes to the upper cell.
  R6  the QJL sign bit is 1 when the projection is >= 0.
  R7  the residual is taken in the rotated domain, r = y - c[idx].
  R8  the JL matrix is square, m = d, entries i.i.d. N(0, 1).
  R9  the inner-product estimator is the QJL one with constant sqrt(pi/2)/m.
  R10 x/||x|| and r use the unrounded norms; only the stored sidecars are fp16.
  R11 a zero vector has N = 0 and x_hat = 0 (no other special case).
  R13 softmax scale is an argument, no soft capping.
  R15 query head h reads KV head h // (Hq / Hkv).
  R16 by default every query of a step sees all L cached tokens; with
      causal_tail query t sees the first L - (n_q - 1 - t).
  R22 an empty visible range yields an all-zero output row.
  R25 (variant) the codebook may instead be fitted to the exact law of one
      coordinate of a uniform unit vector in R^d, whose large-d limit is R4's.
  R26 (variant) keys may skip the QJL stage: the record keeps codes, N and G,
      its sign plane is zero, and the score keeps only the codebook term.
  R27 (variant) K and V codes may have 2 or 4 bits (4 or 16 Lloyd-Max levels of
      the same density), stored as that many bit planes (K: kb + 1 words per 32
      coordinates, the signs last).
"""

from __future__ import annotations

import functools
import math
from dataclasses import dataclass

import numpy as np
from scipy.special import betaincc, gammaln, ndtr, ndtri

__all__ = [
    "QJL_KAPPA_NUM", "bits_per_dim", "fwht", "lloyd_max_gaussian", "lloyd_max_sphere",
    "sphere_coordinate_pdf", "Codebook",
    "codebook", "splitmix64", "qjl_matrix", "fp16_rne", "quantize", "encode",
    "k_page_bytes", "v_page_bytes", "pack_k", "pack_v", "unpack_k", "unpack_v",
    "gather_k", "gather_v", "rotate_query", "score", "attn_decode", "dequant_k",
    "dequant_v", "dense_attn_decode", "encode_k_mse_only",
]

# sqrt(pi/2): the QJL estimator constant numerator (R9); divided by m at use.
QJL_KAPPA_NUM = math.sqrt(math.pi / 2.0)


# --------------------------------------------------------------------------
# Bit budget  [AH] K-Cache圧縮 title (4.25 bits/dim), V-Cache圧縮 title (3.125)
# --------------------------------------------------------------------------
def bits_per_dim(head_dim: int, which: str, m: int | None = None) -> float:
    """Stored bits per coordinate.

    K: 3 code bits + m/d QJL sign bits + two fp16 sidecars per vector (R1).
    V: 3 code bits + one fp16 sidecar per vector (no QJL, [AH] V-Cache圧縮).
    """
    m = head_dim if m is None else m
    if which == "k":
        return (3 * head_dim + m + 32) / head_dim
    if which == "v":
        return (3 * head_dim + 16) / head_dim
    raise ValueError(which)


# --------------------------------------------------------------------------
# Fast Walsh-Hadamard rotation  [AH] K-Cache圧縮 flow step 2 (R3)
# --------------------------------------------------------------------------
def fwht(x) -> np.ndarray:
    """y = H_d x / sqrt(d) along the last axis, H_d Sylvester (natural order).

    Butterfly stages h = 1, 2, 4, ..., d/2; in each block of 2h entries the pair
    (a, b) = (x[i], x[i + h]) becomes (a + b, a - b).
    """
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("length must be a power of two")
    lead = y.shape[:-1]
    h = 1
    while h < d:
        blocks = y.reshape(*lead, d // (2 * h), 2, h)
        a = blocks[..., 0, :]
        b = blocks[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2).reshape(*lead, d)
        h *= 2
    return y / math.sqrt(d)


# --------------------------------------------------------------------------
# Lloyd-Max codebook  [AH] アーキテクチャ item 1 and K-Cache圧縮 flow step 3 (R4)
# --------------------------------------------------------------------------
def _phi(u):
    u = np.asarray(u, dtype=np.float64)
    out = np.zeros_like(u)
    fin = np.isfinite(u)
    out[fin] = np.exp(-0.5 * u[fin] ** 2) / math.sqrt(2.0 * math.pi)
    return out


def _cell_mass(a, b):
    """P(a < Z <= b) for Z ~ N(0,1), taking tails from the side that avoids
    cancellation."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    upper = a >= 0
    return np.where(upper, ndtr(-a) - ndtr(-b), ndtr(b) - ndtr(a))


def lloyd_max_gaussian(sigma: float, n_levels: int = 8, init=None,
                       tol: float = 1e-14, max_iter: int = 10000):
    """Lloyd iteration for the n-level MSE quantiser of N(0, sigma^2).

    Alternates the two optimality conditions: thresholds at midpoints of
    adjacent levels, levels at the conditional mean of their cell, i.e.
    c_k = sigma (phi(a/sigma) - phi(b/sigma)) / (Phi(b/sigma) - Phi(a/sigma)).
    Starts from the quantiles sigma * Phi^-1((k + 1/2)/n) unless `init` is given,
    stops when no level moves by tol*sigma, then symmetrises (c_k = -c_{n-1-k})
    and puts the middle threshold at exactly 0.
    Returns (levels, thresholds, iterations), all float64.
    """
    k = np.arange(n_levels, dtype=np.float64)
    c = sigma * ndtri((k + 0.5) / n_levels) if init is None else np.array(init, np.float64)
    it = 0
    for it in range(1, max_iter + 1):
        t = 0.5 * (c[:-1] + c[1:])
        a = np.concatenate([[-np.inf], t]) / sigma
        b = np.concatenate([t, [np.inf]]) / sigma
        c_new = sigma * (_phi(a) - _phi(b)) / _cell_mass(a, b)
        delta = np.max(np.abs(c_new - c))
        c = c_new
        if delta < tol * sigma:
            break
    c = 0.5 * (c - c[::-1])
    t = 0.5 * (c[:-1] + c[1:])
    t[n_levels // 2 - 1] = 0.0
    return c, t, it


@dataclass(frozen=True)
class Codebook:
    head_dim: int
    levels64: np.ndarray       # fp64 fixed point
    thresholds64: np.ndarray
    levels: np.ndarray         # float32 rounding, promoted to fp64: what both sides use
    thresholds: np.ndarray
    iterations: int


def sphere_coordinate_pdf(x, d: int):
    """Density of one coordinate of a point drawn uniformly from the unit sphere
    in R^d (d >= 2): Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) (1 - x^2)^((d-3)/2)
    on (-1, 1). N(0, 1/d) is its large-d limit. A unit vector x_hat that the
    rotation leaves in general position has coordinates of this law when x is
    isotropic, which is the setting the Lloyd-Max codebook is fitted for."""
    x = np.asarray(x, dtype=np.float64)
    lc = gammaln(d / 2.0) - 0.5 * math.log(math.pi) - gammaln((d - 1) / 2.0)
    inside = np.abs(x) < 1.0
    out = np.zeros_like(x)
    out[inside] = np.exp(lc + 0.5 * (d - 3) * np.log1p(-x[inside] ** 2))
    return out


def _sphere_tail(u, d: int):
    """P(X > u) for one sphere coordinate X: by symmetry and X^2 ~ Beta(1/2, (d-1)/2),
    P(X > u) = (1 - I_{u^2}(1/2, (d-1)/2)) / 2 for u >= 0."""
    u = np.asarray(u, dtype=np.float64)
    uc = np.clip(np.abs(u), 0.0, 1.0)
    half = 0.5 * betaincc(0.5, 0.5 * (d - 1), uc ** 2)
    return np.where(u >= 0, half, 1.0 - half)


def _sphere_first_moment(a, b, d: int):
    """Integral of x f(x) over (a, b): the antiderivative of x (1 - x^2)^m is
    -(1 - x^2)^(m+1) / (2 (m + 1)) with m = (d - 3)/2."""
    m1 = 0.5 * (d - 1)
    k = math.exp(gammaln(d / 2.0) - 0.5 * math.log(math.pi) - gammaln((d - 1) / 2.0)) / (2.0 * m1)

    def F(x):
        x = np.clip(np.asarray(x, dtype=np.float64), -1.0, 1.0)
        return -k * np.power(1.0 - x * x, m1)
    return F(b) - F(a)


def lloyd_max_sphere(d: int, n_levels: int = 8, init=None, tol: float = 1e-14,
                     max_iter: int = 20000):
    """Lloyd iteration for the n-level MSE quantiser of one coordinate of a
    uniform point on the unit sphere in R^d (density sphere_coordinate_pdf).
    The same two conditions as lloyd_max_gaussian: thresholds at midpoints,
    levels at the conditional mean of their cell, the mean taken from the
    closed-form first moment and the cell mass from the incomplete beta
    function. Starts from the N(0, 1/d) levels unless `init` is given;
    symmetrises at the end. Returns (levels, thresholds, iterations), float64."""
    if init is None:
        c = lloyd_max_gaussian(1.0 / math.sqrt(d), n_levels)[0]
        c = np.clip(c, -0.999, 0.999)
    else:
        c = np.array(init, np.float64)
    scale = float(np.max(np.abs(c)))
    it = 0
    for it in range(1, max_iter + 1):
        t = 0.5 * (c[:-1] + c[1:])
        a = np.concatenate([[-1.0], t])
        b = np.concatenate([t, [1.0]])
        mass = _sphere_tail(a, d) - _sphere_tail(b, d)
        c_new = _sphere_first_moment(a, b, d) / mass
        delta = np.max(np.abs(c_new - c))
        c = c_new
        if delta < tol * scale:
            break
    c = 0.5 * (c - c[::-1])
    t = 0.5 * (c[:-1] + c[1:])
    t[n_levels // 2 - 1] = 0.0
    return c, t, it


def codebook(head_dim: int, bits: int = 3, density: str = "gaussian") -> Codebook:
    """8-level Lloyd-Max codebook (R4); stored values are float32. density
    "gaussian" fits N(0, 1/d) (the default, R4); "sphere" fits the exact
    marginal of a coordinate of a uniform unit vector in R^d (R25)."""
    if bits not in (2, 3, 4):
        raise ValueError("codes of 2, 3 or 4 bits (3 for K, R27 for V)")
    if density == "gaussian":
        c, t, it = lloyd_max_gaussian(1.0 / math.sqrt(head_dim), 1 << bits)
    elif density == "sphere":
        c, t, it = lloyd_max_sphere(head_dim, 1 << bits)
    else:
        raise ValueError(f"unknown density {density!r}")
    return Codebook(head_dim, c, t,
                    c.astype(np.float32).astype(np.float64),
                    t.astype(np.float32).astype(np.float64), it)


# --------------------------------------------------------------------------
# QJL projection matrix  [AH] K-Cache圧縮 flow step 5 (R8)
# --------------------------------------------------------------------------
_SM_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_SM_M1 = np.uint64(0xBF58476D1CE4E5B9)
_SM_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, n: int) -> np.ndarray:
    """First n outputs of SplitMix64 (Steele, Lea & Flood, OOPSLA 2014).

    Output i (0-based) mixes the counter state seed + (i+1)*0x9E3779B97F4A7C15
    through z ^= z>>30, z *= 0xBF58476D1CE4E5B9, z ^= z>>27,
    z *= 0x94D049BB133111EB, z ^= z>>31 (all mod 2^64).
    """
    with np.errstate(over="ignore"):
        ctr = np.arange(1, n + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + ctr * _SM_GAMMA
        z = (z ^ (z >> np.uint64(30))) * _SM_M1
        z = (z ^ (z >> np.uint64(27))) * _SM_M2
        return z ^ (z >> np.uint64(31))


def qjl_matrix(head_dim: int, seed: int) -> np.ndarray:
    """S[l][i] (m = d rows), row-major, float32.

    Pairs of SplitMix64 outputs (x1, x2) become u = ((x >> 11) + 1) * 2^-53 in
    (0, 1]; Box-Muller gives sqrt(-2 ln u1) cos(2 pi u2), then the matching sin,
    filled in order; each value is rounded to float32.
    """
    n = head_dim * head_dim
    raw = splitmix64(seed, n + (n & 1))
    out = np.empty(n, dtype=np.float32)
    for p in range(0, n, 2):
        u1 = (int(raw[p]) >> 11) + 1
        u2 = (int(raw[p + 1]) >> 11) + 1
        u1 = u1 * 2.0 ** -53
        u2 = u2 * 2.0 ** -53
        rad = math.sqrt(-2.0 * math.log(u1))
        ang = 2.0 * math.pi * u2
        out[p] = rad * math.cos(ang)
        if p + 1 < n:
            out[p + 1] = rad * math.sin(ang)
    return out.reshape(head_dim, head_dim)


# --------------------------------------------------------------------------
# Encoding  [AH] K-Cache圧縮 flow steps 1-5; V-Cache圧縮 (steps 1-3 only)
# --------------------------------------------------------------------------
def fp16_rne(x) -> np.ndarray:
    """IEEE binary16 round-to-nearest-even of float64 values (overflow -> inf)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16)


def quantize(y, thresholds) -> np.ndarray:
    """idx = number of thresholds t_k with t_k <= y (ties go up, R5)."""
    y = np.asarray(y, dtype=np.float64)
    return (y[..., None] >= np.asarray(thresholds)).sum(-1).astype(np.uint8)


def encode(x, cb: Codebook, S=None) -> dict:
    """Encode rows of x (any leading shape, last axis d).

    Step 1: n = ||x||, x_hat = x / n (0 when n = 0, R11).
    Step 2: y = Pi x_hat.
    Step 3: idx = 3-bit Lloyd-Max cell of each y_i; N = fp16(n).
    V stops here. For K (S given):
    Step 4: r = y - c[idx], gamma = ||r||, G = fp16(gamma).
    Step 5: z = S r, sign bit = [z >= 0] (R6).
    """
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1))
    safe = np.where(n > 0, n, 1.0)
    xhat = np.where((n > 0)[..., None], x / safe[..., None], 0.0)
    y = fwht(xhat)
    idx = quantize(y, cb.thresholds)
    out = {"norm": n, "y": y, "idx": idx, "N": fp16_rne(n)}
    if S is not None:
        S = np.asarray(S, dtype=np.float64)
        r = y - cb.levels[idx]
        gamma = np.sqrt(np.sum(r * r, axis=-1))
        z = r @ S.T
        out.update(r=r, gamma=gamma, G=fp16_rne(gamma), z=z, sign=(z >= 0))
    return out


def encode_k_mse_only(x, cb: Codebook) -> dict:
    """K without the QJL stage (R26): steps 1-4 of encode(); the record keeps
    G = fp16(||r||) and its sign plane is all zero."""
    out = encode(x, cb)
    r = out["y"] - cb.levels[out["idx"]]
    gamma = np.sqrt(np.sum(r * r, axis=-1))
    out.update(r=r, gamma=gamma, G=fp16_rne(gamma), sign=np.zeros(r.shape, dtype=bool))
    return out


# --------------------------------------------------------------------------
# Packed page layout (frozen format of this library; not given by the pages)
#   Offsets t within a page are split as t = 64 b + 16 tau + 4 k + r
#   (b = 64-token block, tau, k, r = 0..3).
#   K section of one (page, kv-head), P tokens, kb-bit codes (kb = 3 by default):
#     token t record ((kb+1) d/8 bytes) at t*(kb+1)*d/8: for group s = 0..d/32-1,
#     kb + 1 little-endian u32 words [code bit0, ..., code bit kb-1, QJL sign];
#     bit e of a word belongs to coordinate 32 s + e;
#     then N[P] fp16 at P*(kb+1)*d/8, then G[P] fp16 2P bytes later, each array in
#     side order: token t at entry 64 b + 16 k + 4 r + tau.
#   V section of one (page, kv-head): code bits, then N[P] fp16 at 3*d*P/8 in
#     side order. Code bits are little-endian u32 words; bit j of the code of
#     coordinate i = 16 (2 kp + h) + n (h = 0..1, n = 0..15) of token t is bit
#     8 r + 4 h + tau of word  b*(6 d) + j*(2 d) + (16 k + n)*(d/32) + kp.
#   Pools are [n_pages][n_kv_heads][section bytes]; slot = page * P + offset.
# --------------------------------------------------------------------------
def _split_offset(t):
    t = np.asarray(t, dtype=np.int64)
    return t // 64, (t % 64) // 16, (t % 16) // 4, t % 4        # b, tau, k, r


def side_entry(t):
    """Entry of offset t in the per-page N / G arrays."""
    b, tau, k, r = _split_offset(t)
    return 64 * b + 16 * k + 4 * r + tau


@functools.lru_cache(maxsize=None)
def _v_bit_table(d: int, P: int, vb: int = 3) -> np.ndarray:
    """[vb][d][P] -> index of that bit in the section's code bits (as a flat
    little-endian bit string, bit 32 w + p = bit p of word w). A 64-token block
    holds vb planes of 2 d words each."""
    j = np.arange(vb)[:, None, None]
    i = np.arange(d)[None, :, None]
    b, tau, k, r = _split_offset(np.arange(P)[None, None, :])
    kk, n = i // 16, i % 16
    kp, h = kk // 2, kk % 2
    word = b * (2 * vb * d) + j * (2 * d) + (16 * k + n) * (d // 32) + kp
    bit = 8 * r + 4 * h + tau
    return (32 * word + bit).astype(np.int64)


def k_page_bytes(d: int, P: int, kb: int = 3) -> int:
    """K section of one (page, KV head) with kb-bit codes."""
    return P * (kb + 1) * d // 8 + 4 * P


def v_page_bytes(d: int, P: int, vb: int = 3) -> int:
    """V section of one (page, KV head) with vb-bit codes."""
    return vb * d * P // 8 + 2 * P


def pack_k(pool: np.ndarray, slots, idx, sign, N, G, P: int, kb: int = 3) -> None:
    """Write kb-bit K records of tokens [n][H][d] into a uint8 pool at `slots`."""
    idx = np.asarray(idx, dtype=np.uint8)
    n, H, d = idx.shape
    kpb = k_page_bytes(d, P, kb)
    rb = (kb + 1) * d // 8                                               # record bytes
    slots = np.asarray(slots, dtype=np.int64)
    planes = np.stack([(idx >> j) & 1 for j in range(kb)] + [np.asarray(sign, dtype=np.uint8)],
                      axis=2)                                            # [n][H][kb+1][d]
    planes = planes.reshape(n, H, kb + 1, d // 32, 32).transpose(0, 1, 3, 2, 4)
    rec = np.packbits(planes, axis=-1, bitorder="little").reshape(n, H, rb)
    page, off = slots // P, slots % P
    base = (page[:, None] * H + np.arange(H)[None, :]) * kpb             # [n][H]
    pool[(base + off[:, None] * rb)[..., None] + np.arange(rb)] = rec
    nb = np.asarray(N, dtype=np.float16).reshape(n, H, 1).view(np.uint8)
    gb = np.asarray(G, dtype=np.float16).reshape(n, H, 1).view(np.uint8)
    side = base + P * rb + 2 * side_entry(off)[:, None]
    pool[side[..., None] + np.arange(2)] = nb
    pool[(side + 2 * P)[..., None] + np.arange(2)] = gb


def pack_v(pool: np.ndarray, slots, idx, N, P: int, vb: int = 3) -> None:
    """Write vb-bit V records of tokens [n][H][d] into a uint8 pool at `slots`
    (only the addressed tokens' bits change)."""
    idx = np.asarray(idx, dtype=np.uint8)
    n, H, d = idx.shape
    vpb = v_page_bytes(d, P, vb)
    cbytes = vb * d * P // 8
    tab = _v_bit_table(d, P, vb)
    slots = np.asarray(slots, dtype=np.int64)
    page, off = slots // P, slots % P
    for pg in np.unique(page):
        sel = np.nonzero(page == pg)[0]
        for h in range(H):
            base = (int(pg) * H + h) * vpb
            bits = np.unpackbits(pool[base:base + cbytes], bitorder="little")
            for j in range(vb):
                bits[tab[j][:, off[sel]]] = ((idx[sel, h, :] >> j) & 1).T
            pool[base:base + cbytes] = np.packbits(bits, bitorder="little")
            nb = np.asarray(N, dtype=np.float16)[sel, h].view(np.uint8).reshape(-1, 2)
            pos = base + cbytes + 2 * side_entry(off[sel])
            pool[pos[:, None] + np.arange(2)] = nb


def unpack_k(pool: np.ndarray, slots, H: int, d: int, P: int, kb: int = 3) -> dict:
    """Read kb-bit K records of `slots` for all heads: idx [n][H][d], sign, N, G."""
    kpb = k_page_bytes(d, P, kb)
    rb = (kb + 1) * d // 8
    slots = np.asarray(slots, dtype=np.int64)
    page, off = slots // P, slots % P
    base = (page[:, None] * H + np.arange(H)[None, :]) * kpb
    rec = pool[(base + off[:, None] * rb)[..., None] + np.arange(rb)]
    bits = np.unpackbits(rec.reshape(len(slots), H, d // 32, kb + 1, 4), axis=-1,
                         bitorder="little")                                # [n][H][S][kb+1][32]
    bits = bits.transpose(0, 1, 3, 2, 4).reshape(len(slots), H, kb + 1, d)
    idx = sum(bits[:, :, j].astype(np.uint8) << j for j in range(kb))
    side = base + P * rb + 2 * side_entry(off)[:, None]
    N = pool[side[..., None] + np.arange(2)].copy().view(np.float16)[..., 0]
    G = pool[(side + 2 * P)[..., None] + np.arange(2)].copy().view(np.float16)[..., 0]
    return {"idx": idx.astype(np.uint8), "sign": bits[:, :, kb].astype(bool), "N": N, "G": G}


def unpack_v(pool: np.ndarray, slots, H: int, d: int, P: int, vb: int = 3) -> dict:
    """Read vb-bit V records of `slots` for all heads: idx [n][H][d], N [n][H]."""
    vpb = v_page_bytes(d, P, vb)
    cbytes = vb * d * P // 8
    tab = _v_bit_table(d, P, vb)
    slots = np.asarray(slots, dtype=np.int64)
    page, off = slots // P, slots % P
    n = len(slots)
    idx = np.zeros((n, H, d), dtype=np.uint8)
    N = np.zeros((n, H), dtype=np.float16)
    for pg in np.unique(page):
        sel = np.nonzero(page == pg)[0]
        for h in range(H):
            base = (int(pg) * H + h) * vpb
            bits = np.unpackbits(pool[base:base + cbytes], bitorder="little")
            sub = bits[tab[:, :, off[sel]]]                                # [vb][d][k]
            idx[sel, h, :] = sum(sub[j].astype(np.uint8) << j for j in range(vb)).T
            pos = base + cbytes + 2 * side_entry(off[sel])
            N[sel, h] = pool[pos[:, None] + np.arange(2)].copy().view(np.float16)[:, 0]
    return {"idx": idx, "N": N}


def gather_k(pool, block_table_row, L, kv_head, H, d, P, kb: int = 3):
    """kb-bit K records of tokens 0..L-1 of one sequence and one KV head."""
    kpb = k_page_bytes(d, P, kb)
    rb = (kb + 1) * d // 8
    t = np.arange(L, dtype=np.int64)
    page = np.asarray(block_table_row, dtype=np.int64)[t // P]
    off = t % P
    base = (page * H + kv_head) * kpb
    rec = pool[(base + off * rb)[:, None] + np.arange(rb)]
    bits = np.unpackbits(rec.reshape(L, d // 32, kb + 1, 4), axis=-1, bitorder="little")
    bits = bits.transpose(0, 2, 1, 3).reshape(L, kb + 1, d)
    idx = sum(bits[:, j].astype(np.uint8) << j for j in range(kb))
    side = base + P * rb + 2 * side_entry(off)
    N = pool[side[:, None] + np.arange(2)].copy().view(np.float16)[:, 0]
    G = pool[(side + 2 * P)[:, None] + np.arange(2)].copy().view(np.float16)[:, 0]
    return idx, bits[:, kb].astype(bool), N.astype(np.float64), G.astype(np.float64)


def gather_v(pool, block_table_row, L, kv_head, H, d, P, vb: int = 3):
    """vb-bit V records of tokens 0..L-1 of one sequence and one KV head."""
    vpb = v_page_bytes(d, P, vb)
    cbytes = vb * d * P // 8
    npg = (L + P - 1) // P
    pages = np.asarray(block_table_row, dtype=np.int64)[:npg]
    base = (pages * H + kv_head) * vpb
    codes = pool[base[:, None] + np.arange(cbytes)]                     # [pg][cbytes]
    bits = np.unpackbits(codes, axis=-1, bitorder="little")[:, _v_bit_table(d, P, vb)]  # [pg][vb][d][P]
    idx = sum(bits[:, j].astype(np.uint8) << j for j in range(vb))          # [pg][d][P]
    idx = idx.transpose(0, 2, 1).reshape(npg * P, d)[:L]
    t = np.arange(L, dtype=np.int64)
    side = base[t // P] + cbytes + 2 * side_entry(t % P)
    N = pool[side[:, None] + np.arange(2)].copy().view(np.float16)[:, 0]
    return idx, N.astype(np.float64)


# --------------------------------------------------------------------------
# Scoring and attention  [AH] K-Cache圧縮 (QJL keeps inner-product scoring
# accurate), V-Cache圧縮 (V is not scored); [TF] Contexte Technique
# --------------------------------------------------------------------------
def rotate_query(q, S):
    """q_tilde = Pi q and p = S q_tilde (the query-side work, done once)."""
    qt = fwht(q)
    return qt, qt @ np.asarray(S, dtype=np.float64).T


def score(qt, p, idx, sign, N, G, cb: Codebook, m: int):
    """QJL inner-product estimate of <q, k> for each record (R9):
    N * (<q_tilde, c[idx]> + sqrt(pi/2)/m * G * <p, sigma>), sigma = 2 bit - 1."""
    sig = np.where(sign, 1.0, -1.0)
    return N * (cb.levels[idx] @ qt + (QJL_KAPPA_NUM / m) * G * (sig @ p))


def attn_decode(k_pool, v_pool, cb: Codebook, S, q, block_table, seq_lens,
                n_kv_heads: int, page_size: int, scale: float,
                causal_tail: bool = False, pairs=None, seq_starts=None,
                cb_v: Codebook | None = None, v_bits: int = 3, k_bits: int = 3) -> np.ndarray:
    """Naive two-pass softmax attention over the packed cache, float64.

    For query (b, t, h) with KV head h // (Hq/Hkv) (R15) and visible tokens
    s_b <= j < L_b (or L_b - (n_q-1-t) with causal_tail, R16), s_b = seq_starts[b]
    (0 without a window):
      w = softmax_j(scale * score_j),  a = sum_j w_j N^V_j c[idxV_j],  o = Pi a.
    A row with no visible token is zero. Records of tokens before s_b are not
    read. `pairs` restricts the work to the listed (b, kv_head) pairs; other
    rows stay zero. K records hold k_bits-bit codes of cb; V records hold
    v_bits-bit codes of the codebook cb_v (cb when None; R27). Returns
    out [B][n_q][Hq][d].
    """
    q = np.asarray(q, dtype=np.float64)
    B, n_q, Hq, d = q.shape
    g = Hq // n_kv_heads
    # S None: MSE-only keys (R26), the score keeps only the codebook term
    S64 = np.asarray(S, dtype=np.float64) if S is not None else np.zeros((d, d))
    m = S64.shape[0]
    qjl_w = QJL_KAPPA_NUM / m if S is not None else 0.0
    out = np.zeros((B, n_q, Hq, d))
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(n_kv_heads)]
    for b, kvh in pairs:
        L = int(seq_lens[b])
        s0 = max(0, int(seq_starts[b])) if seq_starts is not None else 0
        if L <= s0:
            continue
        # the visible range starts on page s0 // P: earlier pages are not read
        p0 = s0 // page_size
        base = p0 * page_size
        idx, sign, N, G = gather_k(k_pool, block_table[b][p0:], L - base, kvh, n_kv_heads, d, page_size,
                                   k_bits)
        vidx, NV = gather_v(v_pool, block_table[b][p0:], L - base, kvh, n_kv_heads, d, page_size,
                            v_bits)
        vals = NV[:, None] * (cb_v or cb).levels[vidx]                     # [L - base][d]
        ckey = cb.levels[idx]                                              # [L - base][d]
        sig = np.where(sign, 1.0, -1.0)
        lo = s0 - base
        for t in range(n_q):
            vis = (L - (n_q - 1 - t) if causal_tail else L) - base
            if vis <= lo:
                continue
            for h in range(kvh * g, (kvh + 1) * g):
                qt, p = rotate_query(q[b, t, h], S64)
                # the estimate of score() with c[idx] and sigma evaluated once per head
                est = N[lo:vis] * (ckey[lo:vis] @ qt + qjl_w * G[lo:vis] * (sig[lo:vis] @ p))
                logits = scale * est
                w = np.exp(logits - logits.max())
                w /= w.sum()
                out[b, t, h] = fwht(w @ vals[lo:vis])
    return out


def dequant_k(idx, sign, N, G, cb: Codebook, S, with_qjl: bool = True) -> np.ndarray:
    """K_tilde = N * Pi (c[idx] + sqrt(pi/2)/m * G * S^T sigma), or N * Pi c[idx]."""
    S64 = np.asarray(S, dtype=np.float64)
    v = cb.levels[np.asarray(idx)]
    if with_qjl:
        sig = np.where(sign, 1.0, -1.0)
        v = v + (QJL_KAPPA_NUM / S64.shape[0]) * np.asarray(G, np.float64)[..., None] * (sig @ S64)
    return np.asarray(N, np.float64)[..., None] * fwht(v)


def dequant_v(idx, N, cb: Codebook) -> np.ndarray:
    """V_tilde = N * Pi c[idx]."""
    return np.asarray(N, np.float64)[..., None] * fwht(cb.levels[np.asarray(idx)])


def dense_attn_decode(k, v, q, seq_lens, scale):
    """Plain softmax(q K^T * scale) V over dense, uncompressed K and V
    ([B][max_len][Hkv][d]); q [B][n_q][Hq][d]; query head h reads KV head
    h // (Hq / Hkv) (R15); every query sees seq_lens[b] tokens. The baseline the
    compressed path is measured against, not part of the method."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    q = np.asarray(q, np.float64)
    B, n_q, Hq, d = q.shape
    H = k.shape[2]
    g = Hq // H
    out = np.zeros((B, n_q, Hq, d))
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        for t in range(n_q):
            for h in range(Hq):
                lg = scale * (k[b, :L, h // g] @ q[b, t, h])
                w = np.exp(lg - lg.max())
                out[b, t, h] = (w / w.sum()) @ v[b, :L, h // g]
    return out
