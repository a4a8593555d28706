"""Pins of the CPU reference against facts fixed outside it: the pages' bit
budgets, textbook values, closed forms, invariants and brute force."""

import json
import math
import os

import numpy as np
import pytest
from scipy import integrate, stats
from scipy.linalg import hadamard

import oracle as O
from tests.conftest import GOLDEN


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- bit budget
def test_bits_per_dim_match_pages():
    g = _golden("bits_per_dim.json")
    d = g["head_dim"]
    assert O.bits_per_dim(d, "k") == g["k_bits_per_dim"]          # exact 4.25
    assert O.bits_per_dim(d, "v") == g["v_bits_per_dim"]          # exact 3.125
    saving = (O.bits_per_dim(d, "k") - O.bits_per_dim(d, "v")) / O.bits_per_dim(d, "k")
    assert abs(saving - g["v_extra_saving_approx"]) < 0.02
    # the packed sections hold exactly those bits (plus nothing else)
    P = 256
    assert O.k_page_bytes(d, P) * 8 == P * d * g["k_bits_per_dim"]
    assert O.v_page_bytes(d, P) * 8 == P * d * g["v_bits_per_dim"]


def test_bits_per_dim_d256_and_d8():
    assert O.bits_per_dim(256, "k") * 256 == 1056
    assert O.bits_per_dim(256, "v") * 256 == 784
    assert O.bits_per_dim(8, "k") * 8 == 64
    assert O.bits_per_dim(8, "v") * 8 == 40


# ---------------------------------------------------------------- rotation
@pytest.mark.parametrize("d", [8, 16, 32, 64, 128, 256])
def test_fwht_equals_sylvester_matrix(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((5, d))
    ref = x @ (hadamard(d) / math.sqrt(d)).T
    assert np.max(np.abs(O.fwht(x) - ref)) < 1e-14 * d


@pytest.mark.parametrize("d", [8, 128, 256])
def test_fwht_orthonormal_involution(d):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((4, d))
    y = O.fwht(x)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    assert np.max(np.abs(O.fwht(y) - x)) < 1e-13
    e0 = np.zeros(d)
    e0[0] = 1
    assert np.allclose(O.fwht(e0), np.full(d, 1 / math.sqrt(d)), atol=1e-15)
    assert np.allclose(O.fwht(np.ones(d)), math.sqrt(d) * e0, atol=1e-12)
    # an outlier channel is spread evenly over every coordinate
    ej = np.zeros(d)
    ej[d // 3] = 20.0
    assert np.allclose(np.abs(O.fwht(ej)), 20.0 / math.sqrt(d), atol=1e-12)


# ---------------------------------------------------------------- Lloyd-Max
@pytest.mark.parametrize("n", [4, 8, 16])
def test_lloyd_max_matches_max_1960(n):
    """Max's printed optimum quantisers of the unit Gaussian for 4, 8 and 16
    levels (the 2-, 3- and 4-bit codebooks up to the scale 1/sqrt(d))."""
    g = _golden(f"max1960_gaussian_n{n}.json")
    c, t, it = O.lloyd_max_gaussian(1.0, n)
    h = n // 2
    assert it < 10000
    assert np.allclose(c[h:], g["levels_positive"], atol=g["printed_abs_tol"])
    assert np.allclose(c[:h], -np.array(g["levels_positive"][::-1]), atol=g["printed_abs_tol"])
    assert np.allclose(t[h - 1:], g["thresholds_positive"], atol=g["printed_abs_tol"])
    # distortion by numerical integration, not by the iteration's own formula
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    mse = sum(integrate.quad(lambda x, ck=ck: (x - ck) ** 2 * stats.norm.pdf(x), a, b,
                             epsabs=1e-13)[0] for ck, a, b in zip(c, edges[:-1], edges[1:]))
    assert abs(mse - g["mse"]) < 5e-5 * max(1.0, g["mse"] / 0.03)


@pytest.mark.parametrize("d", [8, 128, 256])
def test_lloyd_max_centroid_and_midpoint_conditions(d):
    cb = O.codebook(d)
    s = 1 / math.sqrt(d)
    c, t = cb.levels64, cb.thresholds64
    assert np.all(np.diff(c) > 0)
    assert np.array_equal(c, -c[::-1])
    assert t[3] == 0.0
    assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=1e-17)
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    for k in range(8):
        a, b = edges[k], edges[k + 1]
        mass = integrate.quad(lambda x: stats.norm.pdf(x, scale=s), a, b, epsabs=1e-15)[0]
        mom = integrate.quad(lambda x: x * stats.norm.pdf(x, scale=s), a, b, epsabs=1e-15)[0]
        assert abs(mom / mass - c[k]) < 1e-10 * s


def test_lloyd_max_unique_fixed_point_from_other_start():
    # the Gaussian is log-concave, so Lloyd's fixed point does not depend on the start
    c1, _, _ = O.lloyd_max_gaussian(1.0, 8)
    c2, _, _ = O.lloyd_max_gaussian(1.0, 8, init=np.linspace(-0.5, 0.5, 8))
    assert np.max(np.abs(c1 - c2)) < 1e-11


def test_codebook_stored_values_are_float32_roundings():
    cb = O.codebook(128)
    assert np.array_equal(cb.levels, cb.levels64.astype(np.float32).astype(np.float64))
    assert np.array_equal(cb.levels, -cb.levels[::-1])
    assert cb.thresholds[3] == 0.0


# ---------------------------------------------------------------- quantiser
def test_quantize_is_nearest_level_and_ties_go_up():
    cb = O.codebook(128)
    rng = np.random.default_rng(3)
    y = rng.standard_normal(20000) / math.sqrt(128) * 1.5
    idx = O.quantize(y, cb.thresholds)
    nearest = np.argmin(np.abs(y[:, None] - cb.levels[None, :]), axis=1)
    # away from the float32-rounded thresholds nearest level == threshold count
    far = np.min(np.abs(y[:, None] - cb.thresholds[None, :]), axis=1) > 1e-9
    assert np.array_equal(idx[far], nearest[far])
    assert np.array_equal(O.quantize(cb.thresholds, cb.thresholds), np.arange(1, 8))
    assert O.quantize(np.array([0.0]), cb.thresholds)[0] == 4


def test_product_codebook_brute_force_d8():
    """argmin over all 8^8 codewords of ||y - c[idx]|| equals the per-coordinate code."""
    d = 8
    cb = O.codebook(d)
    rng = np.random.default_rng(11)
    lv = cb.levels
    grid = np.stack(np.meshgrid(*([np.arange(8)] * d), indexing="ij"), -1).reshape(-1, d)
    for _ in range(2):
        y = O.encode(rng.standard_normal(d), cb)["y"]
        best, best_i = np.inf, None
        for lo in range(0, len(grid), 1 << 21):
            g = grid[lo:lo + (1 << 21)]
            dist = ((y[None, :] - lv[g]) ** 2).sum(1)
            j = int(np.argmin(dist))
            if dist[j] < best:
                best, best_i = dist[j], g[j]
        assert np.array_equal(best_i, O.quantize(y, cb.thresholds))


# ---------------------------------------------------------------- RNG
def test_splitmix64_reference_outputs():
    g = _golden("splitmix64.json")
    assert int(O.splitmix64(0, 1)[0]) == int(g["seed0_first"], 16)
    assert [int(v) for v in O.splitmix64(1234567, 5)] == [int(v) for v in g["seed1234567_first5"]]


def test_qjl_matrix_is_standard_gaussian():
    S = O.qjl_matrix(128, 12345).astype(np.float64).ravel()
    n = S.size
    assert S.dtype == np.float64 and O.qjl_matrix(128, 12345).dtype == np.float32
    assert abs(S.mean()) < 5 / math.sqrt(n)
    assert abs(S.var() - 1) < 5 * math.sqrt(2 / n)
    assert stats.kstest(S, "norm").pvalue > 1e-3
    assert abs(np.corrcoef(S[0::2], S[1::2])[0, 1]) < 5 / math.sqrt(n / 2)
    assert not np.array_equal(O.qjl_matrix(128, 12346), O.qjl_matrix(128, 12345))
    assert np.array_equal(O.qjl_matrix(128, 12345), O.qjl_matrix(128, 12345))


# ---------------------------------------------------------------- fp16 sidecars
def test_fp16_rne_cases():
    f = lambda v: float(O.fp16_rne(v))
    assert f(1 + 2 ** -11) == 1.0                       # tie -> even
    assert f(1 + 3 * 2 ** -11) == 1 + 2 ** -9           # tie -> even (up)
    assert f(1 + 2 ** -11 + 2 ** -40) == 1 + 2 ** -10   # no double rounding via fp32
    assert f(65504.0) == 65504.0
    assert f(65519.99) == 65504.0
    assert math.isinf(f(65520.0))
    assert f(0.0) == 0.0


# ---------------------------------------------------------------- QJL estimator
def test_qjl_constant_by_quadrature():
    """E[<s,q> sign<s,r>] = sqrt(2/pi) <q,r>/||r|| for s ~ N(0, I): reduce to the
    plane of (r, q) and integrate over the two independent coordinates."""
    q1, q2 = 0.7, -1.3          # components of q along r/||r|| and its normal
    val = integrate.dblquad(
        lambda b, a: (q1 * a + q2 * b) * np.sign(a) * stats.norm.pdf(a) * stats.norm.pdf(b),
        -12, 12, -12, 12, epsabs=1e-13, epsrel=1e-13)[0]
    assert abs(val - math.sqrt(2 / math.pi) * q1) < 1e-10
    assert abs(O.QJL_KAPPA_NUM * math.sqrt(2 / math.pi) - 1.0) < 1e-15


def test_qjl_estimator_unbiased_monte_carlo():
    """With x, q and the codes fixed (they do not depend on S), over draws of S:
    E[s_hat] = <q, x> exactly, Var = (n^2/m)((pi/2)|q~|^2 gamma^2 - <q~, r>^2)."""
    d = 32
    cb = O.codebook(d)
    rng = np.random.default_rng(2024)
    x = rng.standard_normal(d) * np.exp(rng.uniform(-0.7, 0.7, d))
    q = rng.standard_normal(d)
    base = O.encode(x, cb)                       # codes, y: independent of S
    r = base["y"] - cb.levels[base["idx"]]
    gamma, n = np.linalg.norm(r), base["norm"]
    qt = O.fwht(q)
    K = 40000
    ests = np.empty(K)
    for lo in range(0, K, 5000):
        Ss = rng.standard_normal((5000, d, d))
        z = np.einsum("kli,i->kl", Ss, r)
        sign = z >= 0
        p = np.einsum("kli,i->kl", Ss, qt)
        sig = np.where(sign, 1.0, -1.0)
        ests[lo:lo + 5000] = n * (cb.levels[base["idx"]] @ qt
                                  + O.QJL_KAPPA_NUM / d * gamma * (sig * p).sum(1))
    # the same estimate through the oracle's scoring routine for one draw
    Ss = rng.standard_normal((d, d))
    e = O.encode(x, cb, Ss)
    qt2, p2 = O.rotate_query(q, Ss)
    one = O.score(qt2, p2, e["idx"], e["sign"], n, e["gamma"], cb, d)
    sig = np.where(e["sign"], 1.0, -1.0)
    assert abs(one - n * (cb.levels[e["idx"]] @ qt + O.QJL_KAPPA_NUM / d * gamma * sig @ (Ss @ qt))) < 1e-12
    var = n ** 2 / d * ((math.pi / 2) * (qt @ qt) * gamma ** 2 - (qt @ r) ** 2)
    assert abs(ests.mean() - q @ x) < 4 * math.sqrt(var / K)
    assert abs(ests.var() / var - 1) < 0.05


def test_qjl_sign_step_end_to_end_monte_carlo():
    """The whole K path of the reference, unchanged, over K independent draws of
    S: O.encode(x, cb, S) writes the codes, norms and signs, O.rotate_query and
    O.score read them back. The codes, r and gamma do not depend on S, so over
    the draws the estimate has mean <q, x> exactly and the variance
    (n^2/m)((pi/2)|q~|^2 gamma^2 - <q~, r>^2) of the QJL estimator. The query is
    chosen with q~ close to r, where that variance is far below the (pi/2)
    |q~|^2 gamma^2 / m that signs taken from any projection other than S r
    (e.g. S^T r) would give, so a transposed or otherwise wrong projection in
    the sign step fails the variance gate. AI Heartland, K-Cache圧縮 flow step 5
    and the reason for QJL (inner-product scoring stays accurate)."""
    d = 32
    cb = O.codebook(d)
    rng = np.random.default_rng(77)
    x = rng.standard_normal(d) * np.exp(rng.uniform(-0.7, 0.7, d))
    base = O.encode(x, cb)                        # S-free part: codes, y, norm
    r = base["y"] - cb.levels[base["idx"]]
    gamma, n = np.linalg.norm(r), float(base["norm"])
    q = O.fwht(r / gamma + 0.35 * rng.standard_normal(d) / math.sqrt(d))   # q~ = Pi q near r
    qt = O.fwht(q)
    K = 12000
    ests = np.empty(K)
    for k in range(K):
        S = rng.standard_normal((d, d))
        e = O.encode(x, cb, S)
        qt_k, p_k = O.rotate_query(q, S)
        ests[k] = O.score(qt_k, p_k, e["idx"], e["sign"], e["norm"], e["gamma"], cb, d)
    var = n ** 2 / d * ((math.pi / 2) * (qt @ qt) * gamma ** 2 - (qt @ r) ** 2)
    var_wrong = n ** 2 / d * (math.pi / 2) * (qt @ qt) * gamma ** 2
    assert var < 0.6 * var_wrong                  # the gate separates the two
    assert abs(ests.mean() - q @ x) < 4 * math.sqrt(var / K)
    assert abs(ests.var() / var - 1) < 0.05


def test_qjl_sign_orientation_with_a_triangular_projection():
    """With S the upper-triangular all-ones matrix, (S r)_l is the suffix sum
    r_l + ... + r_{d-1}, which differs from the prefix sums of r @ S: the sign
    plane of O.encode must be [suffix sum >= 0] (sign bit 1 at zero, R6)."""
    d = 16
    cb = O.codebook(d)
    rng = np.random.default_rng(5)
    S = np.triu(np.ones((d, d)))
    differs = 0
    for _ in range(20):
        x = rng.standard_normal(d)
        e = O.encode(x, cb, S)
        r = e["y"] - cb.levels[e["idx"]]
        suffix = np.cumsum(r[::-1])[::-1]
        assert np.array_equal(e["sign"], suffix >= 0)
        differs += not np.array_equal(suffix >= 0, np.cumsum(r) >= 0)
    assert differs >= 15                           # the two orientations are told apart


def test_residual_energy_band():
    """E[gamma^2] ~ Lloyd-Max distortion of a unit vector (0.0345), sanity band."""
    cb = O.codebook(128)
    x = np.random.default_rng(5).standard_normal((4000, 128))
    e = O.encode(x, cb, np.eye(128))
    assert 0.030 < np.mean(e["gamma"] ** 2) < 0.038


def test_zero_vector():
    cb = O.codebook(128)
    S = O.qjl_matrix(128, 1)
    e = O.encode(np.zeros((1, 128)), cb, S)
    assert e["N"][0] == 0 and np.all(e["idx"] == 4)
    assert abs(e["gamma"][0] - abs(cb.levels[4]) * math.sqrt(128)) < 1e-12
    assert np.all(O.dequant_k(e["idx"], e["sign"], e["N"], e["G"], cb, S) == 0)


# ---------------------------------------------------------------- packed format
def test_pack_layout_hand_fixture():
    g = _golden("pack_layout_d32_p64.json")
    d, P, slot = g["head_dim"], g["page_size"], g["k_slot"]
    assert O.k_page_bytes(d, P) == g["k_section_bytes"]
    assert O.v_page_bytes(d, P) == g["v_section_bytes"]
    i = np.arange(d)
    idx = (i % 8).astype(np.uint8)[None, None]
    sign = (i % 3 == 0)[None, None]
    kp = np.zeros(g["k_section_bytes"], np.uint8)
    O.pack_k(kp, [slot], idx, sign, np.array([[1.0]], np.float16), np.array([[0.5]], np.float16), P)
    want = np.zeros_like(kp)
    for off, hx in g["k_nonzero"].items():
        want[int(off)] = int(hx, 16)
    assert np.array_equal(kp, want)
    vp = np.zeros(g["v_section_bytes"], np.uint8)
    idx3 = np.stack([idx[0], np.full((1, d), 7, np.uint8), np.full((1, d), 7, np.uint8)])
    O.pack_v(vp, [1, 13, 37], idx3, np.array([[1.0], [2.0], [0.5]], np.float16), P)
    wantv = np.zeros_like(vp)
    for off, hx in g["v_nonzero"].items():
        wantv[int(off)] = int(hx, 16)
    assert np.array_equal(vp, wantv)


@pytest.mark.parametrize("d", [128, 256])
def test_pack_unpack_roundtrip_and_isolation(d):
    P, H = 256, 3
    rng = np.random.default_rng(d)
    n = 300
    slots = rng.choice(4 * P, size=n, replace=False)
    idx = rng.integers(0, 8, (n, H, d)).astype(np.uint8)
    sign = rng.integers(0, 2, (n, H, d)).astype(bool)
    N = rng.standard_normal((n, H)).astype(np.float16)
    G = rng.standard_normal((n, H)).astype(np.float16)
    kp = rng.integers(0, 256, 4 * H * O.k_page_bytes(d, P)).astype(np.uint8)
    vp = rng.integers(0, 256, 4 * H * O.v_page_bytes(d, P)).astype(np.uint8)
    kp0, vp0 = kp.copy(), vp.copy()
    O.pack_k(kp, slots, idx, sign, N, G, P)
    O.pack_v(vp, slots, idx, N, P)
    uk = O.unpack_k(kp, slots, H, d, P)
    uv = O.unpack_v(vp, slots, H, d, P)
    assert np.array_equal(uk["idx"], idx) and np.array_equal(uk["sign"], sign)
    assert np.array_equal(uk["N"].view(np.uint16), N.view(np.uint16))
    assert np.array_equal(uk["G"].view(np.uint16), G.view(np.uint16))
    assert np.array_equal(uv["idx"], idx) and np.array_equal(uv["N"].view(np.uint16), N.view(np.uint16))
    # untouched slots keep their bytes
    others = np.setdiff1d(np.arange(4 * P), slots)[:50]
    a = O.unpack_k(kp, others, H, d, P)
    b = O.unpack_k(kp0, others, H, d, P)
    assert np.array_equal(a["idx"], b["idx"]) and np.array_equal(a["sign"], b["sign"])
    a = O.unpack_v(vp, others, H, d, P)
    b = O.unpack_v(vp0, others, H, d, P)
    assert np.array_equal(a["idx"], b["idx"])


@pytest.mark.parametrize("vb", [2, 4])
def test_v_pack_unpack_other_widths(vb):
    """vb-bit V records: round trip, untouched neighbours, the section size, and
    the plane layout (bit j of a code sits in plane j of its 64-token block)."""
    d, P, H = 128, 256, 2
    rng = np.random.default_rng(vb)
    n = 200
    slots = rng.choice(3 * P, size=n, replace=False)
    idx = rng.integers(0, 1 << vb, (n, H, d)).astype(np.uint8)
    N = rng.standard_normal((n, H)).astype(np.float16)
    assert O.v_page_bytes(d, P, vb) == vb * d * P // 8 + 2 * P
    vp = rng.integers(0, 256, 3 * H * O.v_page_bytes(d, P, vb)).astype(np.uint8)
    vp0 = vp.copy()
    O.pack_v(vp, slots, idx, N, P, vb)
    uv = O.unpack_v(vp, slots, H, d, P, vb)
    assert np.array_equal(uv["idx"], idx) and np.array_equal(uv["N"].view(np.uint16), N.view(np.uint16))
    others = np.setdiff1d(np.arange(3 * P), slots)[:50]
    assert np.array_equal(O.unpack_v(vp, others, H, d, P, vb)["idx"],
                          O.unpack_v(vp0, others, H, d, P, vb)["idx"])
    # one set bit: code 2^j of coordinate 0, token 0 of page 0, head 0 -> bit 0 of word j * 2d
    for j in range(vb):
        z = np.zeros(3 * H * O.v_page_bytes(d, P, vb), np.uint8)
        one = np.zeros((1, H, d), np.uint8)
        one[0, 0, 0] = 1 << j
        O.pack_v(z, [0], one, np.zeros((1, H), np.float16), P, vb)
        words = z[:vb * d * P // 8].view("<u4")
        assert np.flatnonzero(words).tolist() == [j * 2 * d] and words[j * 2 * d] == 1


@pytest.mark.parametrize("vb", [2, 4])
def test_attention_with_other_v_widths_equals_dense_softmax(vb):
    """Attention over vb-bit V records (R27) is softmax attention over the keys'
    dequantised values and V dequantised with the vb-bit codebook."""
    d, H, P, L, g = 32, 2, 64, 150, 2
    rng = np.random.default_rng(20 + vb)
    cb, cbv = O.codebook(d), O.codebook(d, vb)
    assert len(cbv.levels) == 1 << vb
    S = O.qjl_matrix(d, 3).astype(np.float64)
    k = rng.standard_normal((L, H, d)) * 2
    v = rng.standard_normal((L, H, d))
    ek, ev = O.encode(k, cb, S), O.encode(v, cbv)
    assert ev["idx"].max() == (1 << vb) - 1
    npg = (L + P - 1) // P
    table = np.arange(npg, dtype=np.int32)[::-1].copy()[None, :]
    t = np.arange(L)
    slots = table[0][t // P] * P + t % P
    kp = np.zeros(npg * H * O.k_page_bytes(d, P), np.uint8)
    vp = np.zeros(npg * H * O.v_page_bytes(d, P, vb), np.uint8)
    O.pack_k(kp, slots, ek["idx"], ek["sign"], ek["N"], ek["G"], P)
    O.pack_v(vp, slots, ev["idx"], ev["N"], P, vb)
    q = rng.standard_normal((1, 2, H * g, d))
    out = O.attn_decode(kp, vp, cb, S, q, table, [L], H, P, 0.3, causal_tail=True,
                        cb_v=cbv, v_bits=vb)
    Kt = O.dequant_k(ek["idx"], ek["sign"], ek["N"], ek["G"], cb, S)
    Vt = O.dequant_v(ev["idx"], ev["N"], cbv)
    for tq_ in range(2):
        vis = L - (1 - tq_)
        for h in range(H * g):
            lg = 0.3 * (Kt[:vis, h // g] @ q[0, tq_, h])
            w = np.exp(lg - lg.max())
            w /= w.sum()
            assert np.max(np.abs(out[0, tq_, h] - w @ Vt[:vis, h // g])) < 1e-12


@pytest.mark.parametrize("kb", [2, 4])
def test_k_pack_unpack_other_widths(kb):
    """kb-bit K records: round trip, untouched neighbours, the section size, and
    the word order (kb code planes, then the signs, per 32 coordinates)."""
    d, P, H = 128, 256, 2
    rng = np.random.default_rng(30 + kb)
    n = 200
    slots = rng.choice(3 * P, size=n, replace=False)
    idx = rng.integers(0, 1 << kb, (n, H, d)).astype(np.uint8)
    sign = rng.integers(0, 2, (n, H, d)).astype(bool)
    N = rng.standard_normal((n, H)).astype(np.float16)
    G = rng.standard_normal((n, H)).astype(np.float16)
    assert O.k_page_bytes(d, P, kb) == (kb + 1) * d * P // 8 + 4 * P
    kp = rng.integers(0, 256, 3 * H * O.k_page_bytes(d, P, kb)).astype(np.uint8)
    kp0 = kp.copy()
    O.pack_k(kp, slots, idx, sign, N, G, P, kb)
    u = O.unpack_k(kp, slots, H, d, P, kb)
    assert np.array_equal(u["idx"], idx) and np.array_equal(u["sign"], sign)
    assert np.array_equal(u["N"].view(np.uint16), N.view(np.uint16))
    assert np.array_equal(u["G"].view(np.uint16), G.view(np.uint16))
    others = np.setdiff1d(np.arange(3 * P), slots)[:50]
    a, b = O.unpack_k(kp, others, H, d, P, kb), O.unpack_k(kp0, others, H, d, P, kb)
    assert np.array_equal(a["idx"], b["idx"]) and np.array_equal(a["sign"], b["sign"])
    # one set bit: code bit j (or the sign) of coordinate 33 of token 1, head 0
    for j in range(kb + 1):
        z = np.zeros(3 * H * O.k_page_bytes(d, P, kb), np.uint8)
        one = np.zeros((1, H, d), np.uint8)
        sg = np.zeros((1, H, d), bool)
        if j < kb:
            one[0, 0, 33] = 1 << j
        else:
            sg[0, 0, 33] = True
        O.pack_k(z, [1], one, sg, np.zeros((1, H), np.float16), np.zeros((1, H), np.float16), P, kb)
        words = z[:(kb + 1) * d * P // 8].view("<u4")
        rec_words = (kb + 1) * d // 32
        assert np.flatnonzero(words).tolist() == [rec_words + (kb + 1) * 1 + j]
        assert words[rec_words + (kb + 1) + j] == 2


@pytest.mark.parametrize("kb", [2, 4])
def test_attention_with_other_k_widths_equals_dense_softmax(kb):
    """Attention over kb-bit K records with QJL (R27) is softmax attention over
    the keys dequantised with the kb-bit codebook and the QJL term."""
    d, H, P, L, g = 32, 2, 64, 150, 2
    rng = np.random.default_rng(40 + kb)
    cbk, cb = O.codebook(d, kb), O.codebook(d)
    S = O.qjl_matrix(d, 4).astype(np.float64)
    k = rng.standard_normal((L, H, d)) * 2
    v = rng.standard_normal((L, H, d))
    ek, ev = O.encode(k, cbk, S), O.encode(v, cb)
    assert ek["idx"].max() == (1 << kb) - 1
    npg = (L + P - 1) // P
    table = np.arange(npg, dtype=np.int32)[::-1].copy()[None, :]
    t = np.arange(L)
    slots = table[0][t // P] * P + t % P
    kp = np.zeros(npg * H * O.k_page_bytes(d, P, kb), np.uint8)
    vp = np.zeros(npg * H * O.v_page_bytes(d, P), np.uint8)
    O.pack_k(kp, slots, ek["idx"], ek["sign"], ek["N"], ek["G"], P, kb)
    O.pack_v(vp, slots, ev["idx"], ev["N"], P)
    q = rng.standard_normal((1, 1, H * g, d))
    out = O.attn_decode(kp, vp, cbk, S, q, table, [L], H, P, 0.3, cb_v=cb, k_bits=kb)
    Kt = O.dequant_k(ek["idx"], ek["sign"], ek["N"], ek["G"], cbk, S)
    Vt = O.dequant_v(ev["idx"], ev["N"], cb)
    for h in range(H * g):
        lg = 0.3 * (Kt[:, h // g] @ q[0, 0, h])
        w = np.exp(lg - lg.max())
        w /= w.sum()
        assert np.max(np.abs(out[0, 0, h] - w @ Vt[:, h // g])) < 1e-12


# ---------------------------------------------------------------- attention
def _small_cache(d=32, L=150, H=2, P=64, seed=0, nq=3, g=2, B=2):
    rng = np.random.default_rng(seed)
    cb = O.codebook(d)
    S = O.qjl_matrix(d, 77).astype(np.float64)
    lens = np.array([L, L // 2 + 3][:B])
    npg = (L + P - 1) // P
    table = np.arange(B * npg, dtype=np.int32).reshape(B, npg)[:, ::-1].copy()
    kp = np.zeros(B * npg * H * O.k_page_bytes(d, P), np.uint8)
    vp = np.zeros(B * npg * H * O.v_page_bytes(d, P), np.uint8)
    dense = []
    for b in range(B):
        Lb = int(lens[b])
        t = np.arange(Lb)
        slots = table[b][t // P] * P + t % P
        k = rng.standard_normal((Lb, H, d)) * 3
        v = rng.standard_normal((Lb, H, d))
        ek = O.encode(k, cb, S)
        ev = O.encode(v, cb)
        O.pack_k(kp, slots, ek["idx"], ek["sign"], ek["N"], ek["G"], P)
        O.pack_v(vp, slots, ev["idx"], ev["N"], P)
        Kt = O.dequant_k(ek["idx"], ek["sign"], ek["N"], ek["G"], cb, S)
        Vt = O.dequant_v(ev["idx"], ev["N"], cb)
        dense.append((Kt, Vt))
    q = rng.standard_normal((B, nq, H * g, d))
    return dict(cb=cb, S=S, lens=lens, table=table, kp=kp, vp=vp, dense=dense, q=q,
                H=H, P=P, d=d, g=g)


def test_score_equals_inner_product_with_dequantised_key():
    c = _small_cache()
    cb, S, d = c["cb"], c["S"], c["d"]
    idx, sign, N, G = O.gather_k(c["kp"], c["table"][0], int(c["lens"][0]), 1, c["H"], d, c["P"])
    q = c["q"][0, 0, 2]
    qt, p = O.rotate_query(q, S)
    s = O.score(qt, p, idx, sign, N, G, cb, d)
    Kt = c["dense"][0][0][:, 1]
    assert np.max(np.abs(s - Kt @ q)) < 1e-12 * np.max(np.abs(s))


@pytest.mark.parametrize("causal", [False, True])
def test_attention_equals_dense_softmax_over_dequantised_cache(causal):
    c = _small_cache()
    scale = 1 / math.sqrt(c["d"])
    out = O.attn_decode(c["kp"], c["vp"], c["cb"], c["S"], c["q"], c["table"], c["lens"],
                        c["H"], c["P"], scale, causal_tail=causal)
    B, nq, Hq, d = c["q"].shape
    for b in range(B):
        Kt, Vt = c["dense"][b]
        for t in range(nq):
            vis = int(c["lens"][b]) - (nq - 1 - t) if causal else int(c["lens"][b])
            for h in range(Hq):
                kv = h // c["g"]
                lg = scale * (Kt[:vis, kv] @ c["q"][b, t, h])
                w = np.exp(lg - lg.max())
                w /= w.sum()
                assert np.max(np.abs(out[b, t, h] - w @ Vt[:vis, kv])) < 1e-12


def test_attention_special_cases():
    c = _small_cache()
    scale = 1 / math.sqrt(c["d"])
    lens1 = np.array([1, 1])
    out = O.attn_decode(c["kp"], c["vp"], c["cb"], c["S"], c["q"], c["table"], lens1,
                        c["H"], c["P"], scale)
    for b in range(2):
        Vt = c["dense"][b][1]
        for h in range(c["q"].shape[2]):
            assert np.allclose(out[b, 0, h], Vt[0, h // c["g"]], atol=1e-12)
    q0 = np.zeros_like(c["q"])
    out = O.attn_decode(c["kp"], c["vp"], c["cb"], c["S"], q0, c["table"], c["lens"],
                        c["H"], c["P"], scale)
    for b in range(2):
        Vt = c["dense"][b][1]
        L = int(c["lens"][b])
        assert np.allclose(out[b, 1, 3], Vt[:L, 1].mean(0), atol=1e-12)
    out = O.attn_decode(c["kp"], c["vp"], c["cb"], c["S"], c["q"], c["table"], np.array([0, 5]),
                        c["H"], c["P"], scale)
    assert np.all(out[0] == 0) and np.any(out[1] != 0)


def test_dequant_without_qjl_drops_only_the_sign_term():
    cb = O.codebook(64)
    S = O.qjl_matrix(64, 5)
    x = np.random.default_rng(1).standard_normal((10, 64))
    e = O.encode(x, cb, S)
    full = O.dequant_k(e["idx"], e["sign"], e["N"], e["G"], cb, S, True)
    mse = O.dequant_k(e["idx"], e["sign"], e["N"], e["G"], cb, S, False)
    assert np.allclose(mse, e["N"].astype(float)[:, None] * O.fwht(cb.levels[e["idx"]]))
    # reconstruction is close to x in the MSE-only form (relative error ~ sqrt(0.0345))
    rel = np.linalg.norm(mse - x, axis=1) / np.linalg.norm(x, axis=1)
    assert np.all(rel < 0.3)
    assert not np.allclose(full, mse)


def test_dense_attention_matches_compressed_attention_over_dequantised_cache():
    """Two independent formulas: the dense baseline run on the dequantised K and
    V equals the compressed-cache attention (scores from the packed bits)."""
    c = _small_cache()
    scale = 1 / math.sqrt(c["d"])
    out = O.attn_decode(c["kp"], c["vp"], c["cb"], c["S"], c["q"], c["table"], c["lens"],
                        c["H"], c["P"], scale)
    B = len(c["lens"])
    Lm = int(max(c["lens"]))
    k = np.zeros((B, Lm, c["H"], c["d"]))
    v = np.zeros_like(k)
    for b in range(B):
        Kt, Vt = c["dense"][b]
        k[b, :len(Kt)] = Kt
        v[b, :len(Vt)] = Vt
    ref = O.dense_attn_decode(k, v, c["q"], c["lens"], scale)
    assert np.max(np.abs(out - ref)) < 1e-12


def test_dense_attention_special_cases():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((1, 5, 2, 8))
    v = rng.standard_normal((1, 5, 2, 8))
    q = rng.standard_normal((1, 1, 4, 8))
    out = O.dense_attn_decode(k, v, q, [1], 0.3)
    assert np.allclose(out[0, 0, 3], v[0, 0, 1])
    out = O.dense_attn_decode(k, v, np.zeros_like(q), [5], 0.3)
    assert np.allclose(out[0, 0, 0], v[0, :, 0].mean(0))


@pytest.mark.parametrize("causal", [False, True])
def test_window_equals_dense_softmax_over_the_visible_tokens(causal):
    """A per-sequence first visible token s_b: the result is softmax attention
    over the dequantised tokens s_b <= j < vis only, and pages wholly before s_b
    are never read (their block-table entries may name any page)."""
    c = _small_cache(L=150, P=64)
    scale = 1 / math.sqrt(c["d"])
    B, nq, Hq, d = c["q"].shape
    for starts in ([0, 0], [70, 3], [149, 64], [128, 40]):
        starts = np.array(starts)
        table = c["table"].copy()
        for b in range(B):
            # recycled pages: entries before the window's first page name another page
            table[b, :starts[b] // c["P"]] = table[1 - b, 0]
        out = O.attn_decode(c["kp"], c["vp"], c["cb"], c["S"], c["q"], table, c["lens"],
                            c["H"], c["P"], scale, causal_tail=causal, seq_starts=starts)
        for b in range(B):
            Kt, Vt = c["dense"][b]
            for t in range(nq):
                vis = int(c["lens"][b]) - (nq - 1 - t) if causal else int(c["lens"][b])
                s0 = int(starts[b])
                for h in range(Hq):
                    if vis <= s0:
                        assert np.all(out[b, t, h] == 0)
                        continue
                    kv = h // c["g"]
                    lg = scale * (Kt[s0:vis, kv] @ c["q"][b, t, h])
                    w = np.exp(lg - lg.max())
                    w /= w.sum()
                    assert np.max(np.abs(out[b, t, h] - w @ Vt[s0:vis, kv])) < 1e-12
    # a start of 0 is the plain call; a start at or past the length gives zero rows
    plain = O.attn_decode(c["kp"], c["vp"], c["cb"], c["S"], c["q"], c["table"], c["lens"],
                          c["H"], c["P"], scale)
    zero = O.attn_decode(c["kp"], c["vp"], c["cb"], c["S"], c["q"], c["table"], c["lens"],
                         c["H"], c["P"], scale, seq_starts=np.array([0, 0]))
    assert np.array_equal(plain, zero)
    past = O.attn_decode(c["kp"], c["vp"], c["cb"], c["S"], c["q"], c["table"], c["lens"],
                         c["H"], c["P"], scale, seq_starts=c["lens"].copy())
    assert np.all(past == 0)


# ---- the codebook of the exact sphere-coordinate law --------------------------

def test_sphere_codebook_d3_is_the_uniform_quantiser():
    """At d = 3 a coordinate of a uniform point on the sphere is uniform on
    (-1, 1) (Archimedes), whose 8-level Lloyd-Max quantiser is the uniform one:
    levels (2k - 7)/8 and thresholds at multiples of 1/4."""
    c, t, _ = O.lloyd_max_sphere(3)
    assert np.allclose(c, (2 * np.arange(8) - 7) / 8, atol=1e-13)
    assert np.allclose(t, (np.arange(7) - 3) / 4, atol=1e-13)


@pytest.mark.parametrize("d", [4, 16, 128, 256])
def test_sphere_density_normalised_with_second_moment_one_over_d(d):
    from scipy.integrate import quad
    f = lambda x: float(O.sphere_coordinate_pdf(np.array([x]), d)[0])
    assert abs(quad(f, -1, 1, limit=200)[0] - 1) < 1e-10
    # the d coordinates of a unit vector have squares summing to one
    assert abs(quad(lambda x: x * x * f(x), -1, 1, limit=200)[0] - 1 / d) < 1e-12


@pytest.mark.parametrize("d", [8, 128])
def test_sphere_codebook_centroid_and_midpoint_conditions(d):
    from scipy.integrate import quad
    cb = O.codebook(d, density="sphere")
    c, t = cb.levels64, cb.thresholds64
    f = lambda x: float(O.sphere_coordinate_pdf(np.array([x]), d)[0])
    edges = np.concatenate([[-1.0], t, [1.0]])
    for k in range(8):
        m0 = quad(f, edges[k], edges[k + 1], limit=200, epsabs=1e-15)[0]
        m1 = quad(lambda x: x * f(x), edges[k], edges[k + 1], limit=200, epsabs=1e-15)[0]
        assert abs(m1 / m0 - c[k]) < 1e-9 * np.max(np.abs(c))
    assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), atol=1e-15)
    assert np.array_equal(c, -c[::-1]) and t[3] == 0.0


def test_sphere_codebook_tends_to_the_gaussian_one():
    """N(0, 1/d) is the large-d limit; the gap in units of 1/sqrt(d) shrinks like 1/d."""
    gap = {}
    for d in (256, 1024, 4096):
        s = O.codebook(d, density="sphere").levels64
        g = O.codebook(d).levels64
        gap[d] = np.max(np.abs(s - g)) * math.sqrt(d)
    assert gap[4096] < 1e-3
    assert 3.0 < gap[256] / gap[1024] < 5.0 and 3.0 < gap[1024] / gap[4096] < 5.0


def test_sphere_codebook_against_sampled_unit_vectors():
    """Monte Carlo from the definition: coordinates of normalised Gaussian
    vectors in R^8. Each level is the mean of the samples in its cell (within
    sampling error), and the sphere codebook's MSE is below the Gaussian one's."""
    d = 8
    rng = np.random.default_rng(5)
    z = rng.standard_normal((400_000, d))
    x = (z / np.linalg.norm(z, axis=1, keepdims=True)).ravel()
    sph = O.codebook(d, density="sphere")
    gau = O.codebook(d)
    idx = np.searchsorted(sph.thresholds64, x, side="right")
    for k in range(8):
        sel = x[idx == k]
        se = sel.std() / math.sqrt(len(sel))
        assert abs(sel.mean() - sph.levels64[k]) < 5 * se
    mse_s = np.mean((x - sph.levels64[idx]) ** 2)
    ig = np.searchsorted(gau.thresholds64, x, side="right")
    mse_g = np.mean((x - gau.levels64[ig]) ** 2)
    assert mse_s < 0.99 * mse_g


# ---- keys without the QJL stage ----------------------------------------------

def test_mse_only_keys_drop_only_the_qjl_stage_and_term():
    """encode_k_mse_only keeps codes, N and G of the full K encode with a zero
    sign plane, and attention over such records with no S is dense softmax over
    the MSE-only dequantised keys."""
    d, H, P, L, g = 32, 2, 64, 150, 2
    rng = np.random.default_rng(8)
    cb = O.codebook(d)
    S = O.qjl_matrix(d, 9).astype(np.float64)
    k = rng.standard_normal((L, H, d)) * 2
    v = rng.standard_normal((L, H, d))
    full = O.encode(k, cb, S)
    mse = O.encode_k_mse_only(k, cb)
    assert np.array_equal(full["idx"], mse["idx"]) and not mse["sign"].any()
    assert np.array_equal(full["N"], mse["N"]) and np.array_equal(full["G"], mse["G"])
    npg = (L + P - 1) // P
    table = np.arange(npg, dtype=np.int32)[::-1].copy()[None, :]
    t = np.arange(L)
    slots = table[0][t // P] * P + t % P
    kp = np.zeros(npg * H * O.k_page_bytes(d, P), np.uint8)
    vp = np.zeros(npg * H * O.v_page_bytes(d, P), np.uint8)
    O.pack_k(kp, slots, mse["idx"], mse["sign"], mse["N"], mse["G"], P)
    ev = O.encode(v, cb)
    O.pack_v(vp, slots, ev["idx"], ev["N"], P)
    q = rng.standard_normal((1, 1, H * g, d))
    scale = 0.4
    out = O.attn_decode(kp, vp, cb, None, q, table, [L], H, P, scale)
    Kt = O.dequant_k(mse["idx"], mse["sign"], mse["N"], mse["G"], cb, S, with_qjl=False)
    Vt = O.dequant_v(ev["idx"], ev["N"], cb)
    for h in range(H * g):
        lg = scale * (Kt[:, h // g] @ q[0, 0, h])
        w = np.exp(lg - lg.max())
        w /= w.sum()
        assert np.max(np.abs(out[0, 0, h] - w @ Vt[:, h // g])) < 1e-12
    # with S the same records score differently (the zero plane reads as sigma = -1)
    out_q = O.attn_decode(kp, vp, cb, S, q, table, [L], H, P, scale)
    assert np.max(np.abs(out_q - out)) > 1e-6
