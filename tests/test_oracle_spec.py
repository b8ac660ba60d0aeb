"""Pins of the oracle's bit-exact parts (router logits, exp_spec, selection,
FP8 E4M3 encoding and block quantisation) against things other than the
oracle itself: closed forms, brute force, exhaustive scans and independent
library routines (libm exp, numpy matmul, torch's float8_e4m3fn cast)."""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle

F32 = np.float32


# ---------------------------------------------------------------- exp_spec

def test_exp_spec_exhaustive_within_2ulp():
    """Every fp32 input in [-86, 88] (about 2.1e9 patterns): |exp_spec - exp| <= 2 ulp."""
    n = oracle.ctypes.c_int64(0)
    worst = oracle.lib().orc_exp_spec_max_ulp(0, 0xFFFFFFFF, oracle.ctypes.byref(n))
    assert n.value > 2_000_000_000
    assert worst <= 2.0, worst


def test_exp_spec_special_values():
    e = oracle.exp_spec
    assert e(np.array([0.0], F32))[0] == 1.0
    assert e(np.array([-0.0], F32))[0] == 1.0
    assert np.isnan(e(np.array([np.nan], F32))[0])
    assert e(np.array([88.5], F32))[0] == np.inf
    assert e(np.array([-86.5], F32))[0] == 0.0
    # exact powers of two: r = 0 after reduction only when x is a multiple of
    # ln 2 to fp32 precision; exp(ln 2) must be 2 within 1 ulp
    assert abs(float(e(np.array([math.log(2.0)], F32))[0]) - 2.0) <= 2.0 ** -22
    s = oracle.sigmoid_spec(np.array([0.0, 100.0, -100.0], F32))
    assert s[0] == 0.5 and s[1] == 1.0 and s[2] == 0.0


# ------------------------------------------------------------ router logits

def test_logits_exact_on_integer_inputs():
    """Integer inputs keep every partial sum exact in fp32, so the result must
    equal the integer matrix product: pins indexing and operand roles."""
    rng = np.random.default_rng(0)
    x = rng.integers(-8, 9, size=(37, 53)).astype(F32)
    w = rng.integers(-8, 9, size=(11, 53)).astype(F32)
    b = rng.integers(-4, 5, size=11).astype(F32)
    L = oracle.router_logits(x, w, b)
    ref = x.astype(np.int64) @ w.astype(np.int64).T + b.astype(np.int64)
    assert np.array_equal(L, ref.astype(F32))


def test_logits_sequential_order():
    """[2^24, 1, -2^24] * [1, 1, 1]: in ascending order 2^24 + 1 rounds to
    2^24 (tie to even) and the result is 0; any other order gives 1."""
    x = np.array([[2.0 ** 24, 1.0, -(2.0 ** 24)]], F32)
    w = np.ones((1, 3), F32)
    assert oracle.router_logits(x, w)[0, 0] == 0.0
    x2 = np.array([[1.0, -(2.0 ** 24), 2.0 ** 24]], F32)
    assert oracle.router_logits(x2, w)[0, 0] == 1.0


def test_logits_fused_multiply_add():
    """a = 1 + 2^-12: a*a = 1 + 2^-11 + 2^-24. Step 1 rounds to 1 + 2^-11
    (tie to even); step 2 adds a*a exactly to -(1 + 2^-11) only if fused,
    giving 2^-24 (unfused: 0)."""
    a = 1.0 + 2.0 ** -12
    x = np.array([[a, a]], F32)
    w = np.array([[a, -a]], F32)
    # sequential: acc = fma(a, a, 0) = 1 + 2^-11; acc = fma(a, -a, acc) = -2^-24
    assert oracle.router_logits(x, w)[0, 0] == F32(-(2.0 ** -24))


def test_logits_higham_bound():
    """|L - L64| <= gamma_d * sum_i |x_i w_i| with gamma_d = d u / (1 - d u),
    u = 2^-24, against numpy's fp64 product."""
    rng = np.random.default_rng(1)
    d = 4096
    x = torch.randn(64, d, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    w = (rng.standard_normal((8, d)) * 0.02).astype(F32)
    L = oracle.router_logits(x, w).astype(np.float64)
    x64 = oracle.as_f64(x)
    ref = x64 @ w.astype(np.float64).T
    u = 2.0 ** -24
    gamma = d * u / (1 - d * u)
    bound = gamma * (np.abs(x64) @ np.abs(w.astype(np.float64)).T)
    assert np.all(np.abs(L - ref) <= bound)
    assert np.max(np.abs(L - ref)) > 0  # it really is fp32


# --------------------------------------------------------------- selection

def _key(L, e):
    """Sort key: larger logit first, NaN last, then lower index."""
    v = float(L)
    return (1 if math.isnan(v) else 0, -v if not math.isnan(v) else 0.0, e)


def _brute_topk(L, k, allowed=None):
    """The k-subset whose members, sorted by rank, are lexicographically best."""
    E = len(L)
    cand = [e for e in range(E) if allowed is None or allowed[e]]
    best = None
    for sub in itertools.combinations(cand, k):
        ks = sorted((_key(L[e], e) for e in sub))
        if best is None or ks < best[0]:
            best = (ks, [kk[2] for kk in ks])
    return best[1]


@pytest.mark.parametrize("E,k", [(4, 1), (5, 2), (8, 2), (8, 3), (6, 6), (10, 4)])
def test_topk_bruteforce(E, k):
    rng = np.random.default_rng(E * 10 + k)
    for trial in range(3):
        if trial == 0:
            L = rng.standard_normal((40, E)).astype(F32)
        else:  # heavy ties, signed zeros
            L = rng.integers(-2, 3, size=(40, E)).astype(F32)
            L[L == 0] = np.where(rng.random(int((L == 0).sum())) < 0.5, -0.0, 0.0).astype(F32)
        idx = oracle.route_select(L, k)
        for t in range(L.shape[0]):
            assert list(idx[t]) == _brute_topk(L[t], k), (t, L[t], idx[t])


def test_topk_special_cases():
    L = np.zeros((3, 8), F32)
    assert np.array_equal(oracle.route_select(L, 3), np.tile(np.arange(3), (3, 1)))
    L = np.array([[-0.0, 0.0, -0.0, 0.0]], F32)
    assert list(oracle.route_select(L, 4)[0]) == [0, 1, 2, 3]
    L = np.array([[0.5, np.nan, 2.0, -1.0]], F32)
    assert list(oracle.route_select(L, 4)[0]) == [2, 0, 3, 1]  # NaN last
    rng = np.random.default_rng(5)
    L = rng.standard_normal((10, 7)).astype(F32)
    assert np.array_equal(oracle.route_select(L, 7), np.argsort(-L, axis=1, kind="stable"))


def _brute_grouped(L, k, G, TG, group_score):
    E = len(L)
    gs = E // G
    s = oracle.sigmoid_spec(L.astype(F32))
    scores = []
    for g in range(G):
        members = sorted(range(g * gs, (g + 1) * gs), key=lambda e: _key(L[e], e))
        sc = s[members[0]]
        if group_score == "top2_sum" and gs > 1:
            sc = F32(sc + s[members[1]])
        scores.append(F32(sc))
    best = None
    for sub in itertools.combinations(range(G), TG):
        ks = sorted(_key(scores[g], g) for g in sub)
        if best is None or ks < best[0]:
            best = (ks, set(sub))
    allowed = [(e // gs) in best[1] for e in range(E)]
    return _brute_topk(L, k, allowed)


@pytest.mark.parametrize("E,G,TG,k,gsc", [(16, 4, 2, 3, "top2_sum"), (16, 4, 1, 4, "top2_sum"),
                                          (24, 8, 4, 5, "top2_sum"), (16, 4, 2, 3, "max"),
                                          (12, 6, 3, 2, "top2_sum")])
def test_group_limited_bruteforce(E, G, TG, k, gsc):
    rng = np.random.default_rng(E + G + TG + k)
    for trial in range(2):
        if trial == 0:
            L = (rng.standard_normal((30, E)) * 0.6).astype(F32)
        else:
            L = rng.integers(-2, 3, size=(30, E)).astype(F32) * F32(0.5)
        idx = oracle.route_select(L, k, G, TG, gsc)
        for t in range(L.shape[0]):
            assert list(idx[t]) == _brute_grouped(L[t], k, G, TG, gsc), t


def test_group_limit_all_groups_is_plain_topk():
    rng = np.random.default_rng(9)
    L = rng.standard_normal((50, 32)).astype(F32)
    assert np.array_equal(oracle.route_select(L, 6, 8, 8), oracle.route_select(L, 6))


def test_group_limit_rejects_bad_arguments():
    L = np.zeros((2, 16), F32)
    with pytest.raises(ValueError):
        oracle.route_select(L, 9, 4, 2)   # 2 groups of 4 hold fewer than 9
    with pytest.raises(ValueError):
        oracle.route_select(L, 2, 5, 2)   # 5 does not divide 16


# ------------------------------------------------------------------- gates

def test_gates_closed_forms():
    rng = np.random.default_rng(2)
    L = rng.standard_normal((20, 8)).astype(F32)
    idx = oracle.route_select(L, 3)
    g = oracle.route_gates(L, idx, "softmax", True, 1.0)
    sel = np.take_along_axis(L.astype(np.float64), idx.astype(np.int64), axis=1)
    assert np.allclose(g.sum(1), 1.0, atol=1e-15)
    # ratio of two gates is exp of the logit difference
    assert np.allclose(g[:, 1] / g[:, 0], np.exp(sel[:, 1] - sel[:, 0]), rtol=1e-13)
    # plain softmax gates equal torch's softmax over all experts
    gp = oracle.route_gates(L, idx, "softmax", False, 1.0)
    ref = torch.softmax(torch.tensor(L, dtype=torch.float64), dim=1).numpy()
    assert np.allclose(gp, np.take_along_axis(ref, idx.astype(np.int64), axis=1), rtol=1e-14)
    # sigmoid renormalised times 2.5 sums to 2.5; k = 1 gives exactly the scale
    gs = oracle.route_gates(L, idx, "sigmoid", True, 2.5)
    assert np.allclose(gs.sum(1), 2.5, atol=1e-14)
    sig = torch.sigmoid(torch.tensor(sel, dtype=torch.float64)).numpy()
    assert np.allclose(gs / 2.5, sig / sig.sum(1, keepdims=True), rtol=1e-14)
    idx1 = oracle.route_select(L, 1)
    assert np.all(oracle.route_gates(L, idx1, "softmax", True, 1.0) == 1.0)
    assert np.all(oracle.route_gates(L, idx1, "sigmoid", True, 2.5) == 2.5)


# ---------------------------------------------------------------- FP8 E4M3

def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.all(both_nan | (ours == ref))
    assert ours[0x7E] == 448.0 and np.isnan(ours[0x7F]) and ours[0x01] == 2.0 ** -9


def test_e4m3_encode_exhaustive_vs_torch():
    """Every fp32 bit pattern with |v| <= 448 (and both signs): our encoder
    equals torch's round-to-nearest-even float8_e4m3fn cast."""
    top = int(np.array(448.0, F32).view(np.uint32))
    chunk = 1 << 25
    for sign in (0, 1 << 31):
        for lo in range(0, top + 1, chunk):
            hi = min(lo + chunk, top + 1)
            bits = (np.arange(lo, hi, dtype=np.uint64) | sign).astype(np.uint32)
            v = bits.view(F32)
            ours = oracle.e4m3_encode(v)
            ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            bad = np.nonzero(ours != ref)[0]
            assert bad.size == 0, (hex(int(bits[bad[0]])), ours[bad[0]], ref[bad[0]])


def test_e4m3_encode_saturates_and_nan():
    v = np.array([448.0, 463.9, 464.0, 1e30, np.inf, -500.0, np.nan], F32)
    assert list(oracle.e4m3_encode(v)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7F]


def test_quant_blocks_properties():
    rng = np.random.default_rng(4)
    src = (rng.standard_normal((300, 260)) * np.exp(rng.standard_normal((300, 1)))).astype(F32)
    src[5, :128] = 0.0                        # an all-zero block -> scale 1
    for br, bc in [(1, 128), (128, 128), (128, 1)]:
        q, s = oracle.quant_blocks(src, br, bc)
        assert s.shape == (-(-300 // br), -(-260 // bc))
        # scale = amax / 448 with one fp32 division, 1 for a zero block
        for I in range(0, s.shape[0], max(1, s.shape[0] // 7)):
            for J in range(s.shape[1]):
                blk = src[I * br:(I + 1) * br, J * bc:(J + 1) * bc]
                amax = np.max(np.abs(blk))
                exp_s = F32(1.0) if amax == 0 else F32(amax) / F32(448.0)
                assert s[I, J] == exp_s
                # the amax element encodes as +-448
                if amax > 0:
                    r, c = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
                    assert q[I * br + r, J * bc + c] & 0x7F == 0x7E
        # codes equal torch's cast of v / scale (fp32 division)
        S = np.repeat(np.repeat(s, br, 0)[:300], bc, 1)[:, :260]
        ref = torch.from_numpy((src / S).astype(F32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(q, ref)
        # dequantisation error: at most half an E4M3 step of each block
        deq = oracle.dequant_blocks(q, s, br, bc)
        err = np.abs(deq - src.astype(np.float64))
        assert np.all(err <= np.maximum(np.abs(src) * 2.0 ** -4, S * 2.0 ** -10) * (1 + 1e-7))


# ---------------------------------------------------------------- MXFP8

def _e4m3_values_by_definition():
    """All 256 E4M3FN code values from the format's definition (1 sign, 4
    exponent bits with bias 7, 3 mantissa bits; exponent 0 is subnormal; only
    S.1111.111 is NaN): an enumeration independent of the oracle's tables."""
    vals = np.empty(256)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = (-1) ** s * m / 8 * 2.0 ** -6
        else:
            vals[c] = (-1) ** s * (1 + m / 8) * 2.0 ** (e - 7)
    return vals


def _mx_exp_brute(amax):
    """Smallest integer x in [-127, 127] with amax * 2^-x <= 448, by search."""
    if amax == 0:
        return 0
    for x in range(-127, 128):
        if float(amax) * 2.0 ** -x <= 448.0:
            return x
    raise AssertionError


def test_mx_scale_exponent_bruteforce():
    rng = np.random.default_rng(21)
    cases = [0.0, 448.0, 449.0, 447.99997, 1.0, 0.875, 0.875 * 2 ** 9, 0.87500006 * 2 ** 9, 1.75, 3.5,
             2.0 ** -126, 2.0 ** -140, 1e-45, 3.0e38, 2.0 ** 120 * 1.7]
    cases += list((np.exp(rng.uniform(-90, 88, 3000))).astype(F32))
    cases += list(F32(448) * F32(2.0) ** rng.integers(-130, 120, 500).astype(F32))  # power-of-two multiples
    for a in cases:
        a = F32(a)
        assert oracle.lib().orc_mx_scale_exp(a) == _mx_exp_brute(a), a


def test_mx_rows_nearest_code_bruteforce():
    """Every code is the E4M3 value nearest to v * 2^-x (ties to an even
    mantissa), found by scanning all 256 codes; the E8M0 byte is x + 127."""
    vals = _e4m3_values_by_definition()
    finite = ~np.isnan(vals)
    rng = np.random.default_rng(22)
    R, C = 24, 128
    src = (rng.standard_normal((R, C)) * np.exp(rng.uniform(-30, 30, (R, 1)))).astype(F32)
    src[3, 32:64] = 0.0                      # an all-zero block
    src[4, :32] = 0.0
    src[4, 7] = -3.0e-41                     # a lone fp32 subnormal
    src[5, 64:96] = 1e-3
    src[5, 70] = 1e3                         # one large element among small ones
    src[6, :32] = np.linspace(-448, 448, 32)  # exact E4M3 range
    q, e = oracle.quant_mx_rows(src)
    assert q.shape == (R, C) and e.shape == (R, C // 32)
    for r in range(R):
        for b in range(C // 32):
            blk = src[r, 32 * b:32 * b + 32]
            x = _mx_exp_brute(np.max(np.abs(blk)))
            assert e[r, b] == x + 127
            for i, v in enumerate(blk):
                t = float(v) * 2.0 ** -x
                assert abs(t) <= 448.0
                dist = np.where(finite, np.abs(vals - t), np.inf)
                best = np.nonzero(dist == dist.min())[0]
                code = q[r, 32 * b + i]
                if t == 0.0:
                    assert vals[code] == 0.0 and (code >> 7) == (np.signbit(v))
                    continue
                best = [c for c in best if (c >> 7) == (t < 0) or vals[c] == 0]
                if len(best) > 1:  # a tie: the even mantissa
                    best = [c for c in best if c & 1 == 0]
                assert code in best, (r, b, i, v, t, code, best)


def test_mx_properties_and_roundtrip():
    rng = np.random.default_rng(23)
    src = (rng.standard_normal((64, 256)) * np.exp(rng.standard_normal((64, 1)) * 4)).astype(F32)
    q, e = oracle.quant_mx_rows(src)
    deq = oracle.dequant_mx_rows(q, e)
    X = np.repeat(oracle.mx_scale(e), 32, axis=1)
    # every block's largest element lands in [224, 448] after scaling: one
    # more halving of the scale would push it past 448
    amax_code = np.abs(oracle.e4m3_decode(q)).reshape(64, 8, 32).max(axis=2)
    assert np.all((amax_code >= 224) & (amax_code <= 448))
    # error of round-to-nearest: half a step, relative 2^-4 in the normal
    # range, absolute 2^-10 X in the subnormal one
    err = np.abs(deq - src.astype(np.float64))
    assert np.all(err <= np.maximum(np.abs(src) * 2.0 ** -4, X * 2.0 ** -10) * (1 + 1e-12))
    # exact values survive: small integers times a power of two
    ex = (rng.integers(-15, 16, (8, 64)) * 2.0 ** rng.integers(-20, 20, (8, 1))).astype(F32)
    assert np.array_equal(oracle.mx_roundtrip_rows(ex), ex.astype(np.float64))
    # column blocks are the row blocks of the transpose
    qc, ec = oracle.quant_mx_cols(src[:, :64].T.copy())
    assert np.array_equal(qc, q[:, :64].T) and np.array_equal(ec, e[:, :2].T)
    with pytest.raises(ValueError):
        oracle.quant_mx_rows(np.zeros((2, 48), F32))


def test_mx_cols_are_the_rows_of_the_transpose():
    """The column-block MXFP8 quantiser equals the row-block one applied to
    the transpose, codes and scales, over magnitudes across the fp32 range."""
    rng = np.random.default_rng(13)
    a = (rng.normal(size=(96, 70)) * np.exp(rng.normal(size=(1, 70)) * 15)).astype(np.float32)
    a[:32, 3] = 0.0
    a[40, 5] = -3.0e-41
    q, e = oracle.quant_mx_cols(a)
    qt, et = oracle.quant_mx_rows(np.ascontiguousarray(a.T))
    assert np.array_equal(q, qt.T) and np.array_equal(e, et.T)
