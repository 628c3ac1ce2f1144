"""Pins for the CPU oracle: checks that do not re-use the oracle's own code.

Each test ties one oracle function to something fixed outside it: the
hand-worked example, exact rational arithmetic, closed forms of the Gaussian
workload, textbook identities, independent library routines (numpy / torch)
or the pages' own popcount formulations of the ternary product.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads


def f32(v):
    return np.float32(v)


def next_up(v):
    return np.nextafter(np.float32(v), np.float32(np.inf))


# ------------------------------------------------------------- hand example
@pytest.fixture(scope="module")
def hand(golden_dir):
    with open(os.path.join(golden_dir, "hand_4x4.json")) as f:
        return json.load(f)


def test_hand_example_every_step(hand):
    w = np.array(hand["w"], dtype=np.float32)
    x = np.array(hand["x"], dtype=np.float32)
    beta = oracle.absmean(w)
    assert beta == f32(hand["beta"])
    t = oracle.ternarize(w, beta)
    np.testing.assert_array_equal(t, np.array(hand["t"]))
    # round-half-to-even is pinned: half-away-from-zero gives different codes
    assert not np.array_equal(t, np.array(hand["t_if_half_away_from_zero"]))
    q, ds, rs = oracle.quant_act(x)
    np.testing.assert_array_equal(q, np.array(hand["q"]))
    assert not np.array_equal(q, np.array(hand["q_if_half_away_from_zero"]))
    np.testing.assert_array_equal(ds, np.array(hand["ds"], dtype=np.float32))
    np.testing.assert_array_equal(rs, np.array(hand["rowsum"]))
    acc = oracle.matmul_i32(q, t)
    np.testing.assert_array_equal(acc, np.array(hand["acc"]))
    y = oracle.dequant(acc, ds, beta)
    np.testing.assert_array_equal(y, np.array(hand["y"], dtype=np.float32))


def test_hand_example_through_bf16_entry(hand):
    x = np.array(hand["x"], dtype=np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)  # every value is bf16-exact
    assert np.array_equal(workloads.bf16_bits_to_f32(xb), x)
    out = oracle.bitlinear_forward(xb, np.array(hand["w"], dtype=np.float32))
    np.testing.assert_array_equal(out["y"], np.array(hand["y"], dtype=np.float32))
    np.testing.assert_array_equal(out["acc"], np.array(hand["acc"]))


# --------------------------------------------------------------------- beta
def exact_mean_f32(w):
    """Exact rational mean of |w|, correctly rounded to fp32 (via Fraction)."""
    s = sum(Fraction(float(abs(v))) for v in w.ravel())
    m = s / w.size
    lo = np.float32(float(m))  # double rounding can be off by one fp32 ulp
    best = min((lo, np.nextafter(lo, np.float32(-1)), np.nextafter(lo, np.float32(2))),
               key=lambda c: abs(Fraction(float(c)) - m))
    return best


@pytest.mark.parametrize("count", [1, 7, 4096, 4097, 3 * 4096 + 17])
def test_absmean_vs_exact_rational(count):
    rng = np.random.default_rng(count)
    w = (rng.standard_normal(count) * 0.02).astype(np.float32)
    assert abs(int(oracle.absmean(w).view(np.int32)) - int(exact_mean_f32(w).view(np.int32))) <= 1


def test_absmean_vs_numpy_fp64_mean():
    w = workloads.gen_weights(512, 512, seed=0)
    ref = np.float32(np.mean(np.abs(w.astype(np.float64))))
    assert abs(int(oracle.absmean(w).view(np.int32)) - int(ref.view(np.int32))) <= 1


def test_absmean_symmetry_and_exact_scaling():
    w = workloads.gen_weights(64, 300, seed=3)
    b = oracle.absmean(w)
    assert oracle.absmean(-w) == b
    assert oracle.absmean(w * np.float32(2.0)) == np.float32(2.0) * b
    assert oracle.absmean(w * np.float32(0.25)) == np.float32(0.25) * b


def test_absmean_constant_tensor():
    assert oracle.absmean(np.full(10000, -0.375, dtype=np.float32)) == f32(0.375)
    assert oracle.absmean(np.zeros(100, dtype=np.float32)) == f32(0.0)


def test_absmean_closed_form_gaussian():
    # E|w| = sigma * sqrt(2/pi); sd of the mean = sigma*sqrt(1-2/pi)/sqrt(n)
    n_rows, k = 512, 512
    w = workloads.gen_weights(n_rows, k, seed=0)
    sigma = workloads.W_STD
    mean = sigma * math.sqrt(2.0 / math.pi)
    sd = sigma * math.sqrt(1.0 - 2.0 / math.pi) / math.sqrt(n_rows * k)
    assert abs(float(oracle.absmean(w)) - mean) < 5 * sd


# ---------------------------------------------------------------- ternarize
def test_ternarize_ties_round_half_even():
    beta = f32(0.5)  # d = 0.5 exactly
    w = np.array([0.25, -0.25, 0.75, -0.75, 1.25, -1.25, 0.0, -0.0, 0.1, 5.0, -5.0],
                 dtype=np.float32)
    # w/d = 0.5 -> 0, -0.5 -> 0, 1.5 -> 2 -> 1, -1.5 -> -1, 2.5 -> 2 -> 1, ...
    np.testing.assert_array_equal(oracle.ternarize(w, beta), [0, 0, 1, -1, 1, -1, 0, 0, 0, 1, -1])


def test_ternarize_epsilon_matters_at_workload_scale():
    # at beta ~ 0.016 an ulp is ~1.9e-9, so the +1e-8 moves d by several ulps;
    # an element at w = d_without_eps / 2 rounds differently with and without it
    beta = f32(0.016)
    d = f32(beta + f32(1e-8))
    assert d != beta
    w_tie_noeps = f32(beta * f32(0.5))  # exactly beta/2 (power-of-two scaling)
    # w/beta = 0.5 exactly -> 0 either way; take the next float up: w/beta > 0.5
    w = next_up(w_tie_noeps)
    assert w / beta > f32(0.5)
    assert np.rint(w / beta) == 1.0   # without the guard the code would be +1
    assert oracle.ternarize(np.array([w]), beta)[0] == 0  # with it, w/d < 0.5


def test_ternarize_zero_tensor():
    w = np.zeros((4, 8), dtype=np.float32)
    beta = oracle.absmean(w)
    assert beta == 0.0
    assert not oracle.ternarize(w, beta).any()


def test_ternarize_invariants_gaussian():
    w = workloads.gen_weights(512, 512, seed=0)
    beta = oracle.absmean(w)
    t = oracle.ternarize(w, beta)
    assert set(np.unique(t)) <= {-1, 0, 1}
    # sign(t) is sign(w) or 0
    assert np.all((t == 0) | (np.sign(t) == np.sign(w)))
    # monotone in w: sorting w sorts t
    order = np.argsort(w.ravel(), kind="stable")
    assert np.all(np.diff(t.ravel()[order].astype(np.int32)) >= 0)
    # scale invariance (exact for power-of-two scales)
    np.testing.assert_array_equal(oracle.ternarize(w * np.float32(8), oracle.absmean(w * np.float32(8))), t)
    # zero fraction: P(|w| < beta/2) = 2*Phi(sqrt(2/pi)/2) - 1 = 0.31006 for Gaussian w
    p0 = math.erf(math.sqrt(2.0 / math.pi) / 2.0 / math.sqrt(2.0))
    n = t.size
    assert abs(float(np.mean(t == 0)) - p0) < 5 * math.sqrt(p0 * (1 - p0) / n)


def test_ternarize_against_torch_round():
    # torch.round is half-to-even; an independent library routine for the codes
    w = workloads.gen_weights(128, 384, seed=11)
    beta = oracle.absmean(w)
    ref = torch.clamp(torch.round(torch.from_numpy(w) / (torch.tensor(beta) + torch.tensor(1e-8, dtype=torch.float32))), -1, 1)
    np.testing.assert_array_equal(oracle.ternarize(w, beta), ref.numpy().astype(np.int8))


# ---------------------------------------------------------- activation quant
def test_quant_act_exact_rational_bound():
    x = workloads.bf16_bits_to_f32(workloads.gen_acts_bf16(6, 700, seed=5, outliers=True))
    q, ds, rs = oracle.quant_act(x)
    for m in range(x.shape[0]):
        gamma = float(np.max(np.abs(x[m])))
        assert ds[m] == np.float32(np.float32(gamma) / np.float32(127.0))
        for k in range(0, x.shape[1], 7):
            r = Fraction(float(x[m, k])) * 127 / Fraction(gamma)
            # fp32 rounding of 127/gamma and of the product stays far below 1/2
            assert abs(Fraction(int(q[m, k])) - r) <= Fraction(1, 2) + Fraction(1, 10**4)
        assert rs[m] == int(q[m].astype(np.int64).sum())


def test_quant_act_invariants():
    xb = workloads.gen_acts_bf16(16, 2560, seed=1, outliers=True)
    x = workloads.bf16_bits_to_f32(xb)
    q, ds, rs = oracle.quant_act(xb, bf16_bits=True)
    q2, ds2, rs2 = oracle.quant_act(x)
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(ds, ds2)
    assert q.min() >= -127 and q.max() <= 127
    for m in range(x.shape[0]):
        am = np.argmax(np.abs(x[m]))
        assert abs(int(q[m, am])) == 127 and np.sign(q[m, am]) == np.sign(x[m, am])
    assert np.all(np.sign(q) * np.sign(x) >= 0)  # never flips sign
    assert np.all(q[x == 0] == 0)
    err = np.abs(x - q.astype(np.float32) * ds[:, None])
    assert np.all(err <= ds[:, None] * 0.5 * (1 + 1e-5))
    for m in range(4):  # monotone within a token
        order = np.argsort(x[m], kind="stable")
        assert np.all(np.diff(q[m, order].astype(np.int32)) >= 0)


def test_quant_act_zero_row_and_ties():
    x = np.zeros((2, 5), dtype=np.float32)
    x[1] = [254.0, 5.0, -3.0, 1.0, -1.0]
    q, ds, rs = oracle.quant_act(x)
    assert not q[0].any() and rs[0] == 0
    assert ds[0] == np.float32(np.float32(1e-5) / np.float32(127.0))
    np.testing.assert_array_equal(q[1], [127, 2, -2, 0, 0])  # 2.5->2, -1.5->-2, +-0.5->0


# ------------------------------------------------------------------ products
def brute_acc(q, t):
    M, K = q.shape
    N = t.shape[0]
    return [[sum(int(q[m][k]) * int(t[n][k]) for k in range(K)) for n in range(N)] for m in range(M)]


def addsub_skip(qrow, trow):
    """The pages' form: activations where w=+1, minus those where w=-1, others skipped."""
    s = 0
    for a, w in zip(qrow, trow):
        if w == 1:
            s += int(a)
        elif w == -1:
            s -= int(a)
    return s


def masks(vals):
    plus = sum(1 << i for i, v in enumerate(vals) if v == 1)
    minus = sum(1 << i for i, v in enumerate(vals) if v == -1)
    return plus, minus


def popc(v):
    return bin(v).count("1")


def dot_sign_value(a, b):
    """Sign/value 2-bit code, popcount form (post #132 of the BitNet HN thread)."""
    va, sa = masks(a)[0] | masks(a)[1], masks(a)[1]
    vb, sb = masks(b)[0] | masks(b)[1], masks(b)[1]
    actv = va & vb
    sign = sa ^ sb
    return popc(actv & ~sign) - popc(actv & sign)


def dot_bitplanes(a, b):
    """Two bit-planes per operand: Cp=(Ap&Bp)|(An&Bn), Cn=(An&Bp)|(Ap&Bn)."""
    ap, an = masks(a)
    bp, bn = masks(b)
    cp = (ap & bp) | (an & bn)
    cn = (an & bp) | (ap & bn)
    return popc(cp) - popc(cn)


def dot_sign_magnitude(a, b):
    """sum = popcount(mag) - 2*popcount(mag & sgn) with mag = Am&Bm, sgn = As^Bs."""
    ap, an = masks(a)
    bp, bn = masks(b)
    mag = (ap | an) & (bp | bn)
    sgn = an ^ bn
    return popc(mag) - 2 * popc(mag & sgn)


def dot_int8_bitplanes(qrow, trow):
    """int8 activations as two's-complement bit-planes against +1/-1 weight masks."""
    plus, minus = masks(trow)
    total = 0
    for bit in range(8):
        plane = sum(1 << i for i, v in enumerate(qrow) if (int(v) & 0xFF) >> bit & 1)
        weight = -(1 << 7) if bit == 7 else (1 << bit)
        total += weight * (popc(plus & plane) - popc(minus & plane))
    return total


def test_matmul_brute_and_pages_forms_ternary_acts():
    rng = np.random.default_rng(7)
    for K in (1, 3, 31, 64, 65):
        q = rng.integers(-1, 2, size=(3, K)).astype(np.int8)
        t = rng.integers(-1, 2, size=(5, K)).astype(np.int8)
        acc = oracle.matmul_i32(q, t)
        assert acc.tolist() == brute_acc(q, t)
        for m in range(3):
            for n in range(5):
                a, b = q[m].tolist(), t[n].tolist()
                assert acc[m, n] == addsub_skip(a, b)
                assert acc[m, n] == dot_sign_value(a, b)
                assert acc[m, n] == dot_bitplanes(a, b)
                assert acc[m, n] == dot_sign_magnitude(a, b)


def test_matmul_int8_acts_brute_and_bitplanes():
    rng = np.random.default_rng(8)
    q = rng.integers(-127, 128, size=(4, 97)).astype(np.int8)
    t = rng.integers(-1, 2, size=(6, 97)).astype(np.int8)
    acc = oracle.matmul_i32(q, t)
    assert acc.tolist() == brute_acc(q, t)
    for m in range(4):
        for n in range(6):
            assert acc[m, n] == addsub_skip(q[m], t[n])
            assert acc[m, n] == dot_int8_bitplanes(q[m].tolist(), t[n].tolist())


def test_matmul_exhaustive_k4():
    # every ternary row of length 4 against every activation row over {-127,-1,0,1,127}^4
    import itertools
    trows = np.array(list(itertools.product((-1, 0, 1), repeat=4)), dtype=np.int8)
    qrows = np.array(list(itertools.product((-127, -1, 0, 1, 127), repeat=4)), dtype=np.int8)
    acc = oracle.matmul_i32(qrows, trows)
    ref = qrows.astype(np.int64) @ trows.astype(np.int64).T
    np.testing.assert_array_equal(acc, ref)


def test_matmul_extremes_no_overflow():
    K = 28672
    q = np.full((2, K), 127, dtype=np.int8)
    q[1] = -127
    t = np.ones((3, K), dtype=np.int8)
    t[1] = -1
    t[2, ::2] = 0
    acc = oracle.matmul_i32(q, t, threads=4)
    np.testing.assert_array_equal(acc, [[127 * K, -127 * K, 127 * K // 2], [-127 * K, 127 * K, -127 * K // 2]])


def test_matmul_threads_and_pairs_agree():
    rng = np.random.default_rng(9)
    q = rng.integers(-127, 128, size=(5, 300)).astype(np.int8)
    t = rng.integers(-1, 2, size=(40, 300)).astype(np.int8)
    a1 = oracle.matmul_i32(q, t, threads=1)
    a4 = oracle.matmul_i32(q, t, threads=4)
    np.testing.assert_array_equal(a1, a4)
    np.testing.assert_array_equal(a1, q.astype(np.int64) @ t.astype(np.int64).T)
    ms = rng.integers(0, 5, size=50)
    ns = rng.integers(0, 40, size=50)
    np.testing.assert_array_equal(oracle.matmul_i32_pairs(q, t, ms, ns), a1[ms, ns])


# ------------------------------------------------------------------- dequant
def test_dequant_error_bound_and_zero():
    rng = np.random.default_rng(10)
    acc = rng.integers(-3_000_000, 3_000_000, size=(3, 50)).astype(np.int32)
    acc[0, :5] = 0
    ds = rng.uniform(0.01, 1.0, size=3).astype(np.float32)
    beta = np.float32(0.0159)
    y = oracle.dequant(acc, ds, beta)
    assert np.all(y[0, :5] == 0)
    exact = acc.astype(np.float64) * ds.astype(np.float64)[:, None] * float(beta)
    rel = np.abs(y.astype(np.float64) - exact) / np.maximum(np.abs(exact), 1e-30)
    assert np.all(rel[acc != 0] <= 2.0 ** -23)  # two roundings of half an ulp each


def test_bf16_rounding_against_torch():
    rng = np.random.default_rng(12)
    y = np.concatenate([
        rng.standard_normal(5000).astype(np.float32) * 100,
        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0, -0.0, np.inf, -np.inf,
                  1e-40, -1e-40, 3.4e38], dtype=np.float32),
    ])
    ref = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.to_bf16_bits(y), ref)
    nan = oracle.to_bf16_bits(np.array([np.nan], dtype=np.float32))
    assert (nan[0] & 0x7F80) == 0x7F80 and (nan[0] & 0x7F) != 0


# ------------------------------------------------------------------- packing
def test_pack_layout_single_weights():
    # a single nonzero weight lands exactly where the format specification says
    N, K = 35, 700
    Kt = (K + 255) // 256
    for (n, k, tv) in [(0, 0, 1), (0, 1, -1), (17, 255, 1), (34, 699, -1), (5, 64 + 16 + 4 + 1, 1),
                       (20, 256 + 3 * 64 + 2 * 16 + 3 * 4 + 2, -1)]:
        t = np.zeros((N, K), dtype=np.int8)
        t[n, k] = tv
        p = oracle.pack_t2(t)
        nb, kb, r, c = n // 16, k // 256, n % 16, k % 256
        i, g, d, b = c // 64, (c % 64) // 16, (c % 16) // 4, c % 4
        byte = (nb * Kt + kb) * 1024 + 16 * (16 * g + r) + 4 * d + b
        expect = np.zeros_like(p)
        expect[byte] = (1 if tv == 1 else 3) << (2 * i)
        np.testing.assert_array_equal(p, expect)


def test_pack_exhaustive_byte_patterns_round_trip():
    import itertools
    # four weights sharing one byte: k = b + 64*i for i in 0..3 (same n, g, d, b)
    for b in (0, 3):
        for combo in itertools.product((-1, 0, 1), repeat=4):
            t = np.zeros((1, 256), dtype=np.int8)
            for i, v in enumerate(combo):
                t[0, 64 * i + b] = v
            p = oracle.pack_t2(t)
            assert np.count_nonzero(p) <= 1
            back, bad = oracle.unpack_t2(p, 1, 256)
            assert bad == 0
            np.testing.assert_array_equal(back, t)


@pytest.mark.parametrize("N,K", [(1, 1), (16, 256), (17, 257), (50, 700), (64, 2560)])
def test_pack_round_trip_random(N, K):
    rng = np.random.default_rng(N * 1000 + K)
    t = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    p = oracle.pack_t2(t)
    assert p.size == ((N + 15) // 16) * ((K + 255) // 256) * 1024 == oracle.t2_bytes(N, K)
    back, bad = oracle.unpack_t2(p, N, K)
    assert bad == 0
    np.testing.assert_array_equal(back, t)
    # no field ever holds the unused code 10
    fields = np.stack([(p >> s) & 3 for s in (0, 2, 4, 6)])
    assert not np.any(fields == 2)
    # padding holds only zero codes: count nonzero fields == count nonzero weights
    assert int(np.count_nonzero(fields)) == int(np.count_nonzero(t))


def test_unpack_reports_invalid_code():
    p = np.zeros(1024, dtype=np.uint8)
    p[0] = 0b10
    t, bad = oracle.unpack_t2(p, 16, 256)
    assert bad == 1 and not t.any()


# ------------------------------------------------------------ whole forward
def test_forward_single_4x512():
    lin = workloads.SINGLE_4x512.linears[0]
    w = workloads.gen_weights(lin.N, lin.K, seed=0)
    xb = workloads.gen_acts_bf16(lin.M, lin.K, seed=1)
    out = oracle.bitlinear_forward(xb, w)
    x = workloads.bf16_bits_to_f32(xb).astype(np.float64)
    # the quantized product approximates the fp64 product of x and beta*t
    approx = x @ (float(out["beta"]) * out["t"].astype(np.float64)).T
    err = np.abs(out["y"] - approx)
    # per element the int8 rounding error is at most ds/2 per term
    bound = (out["ds"][:, None].astype(np.float64) / 2) * float(out["beta"]) * np.abs(out["t"]).sum(1)[None, :]
    assert np.all(err <= bound * (1 + 1e-6) + 1e-6)
    np.testing.assert_array_equal(out["y_bf16"],
                                  torch.from_numpy(out["y"]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


# ------------------------------------------------------------- decoder glue
def test_relu2_mul_special_values():
    # exact small integers and dyadic values: every product is representable
    g = np.array([-3.0, -0.0, 0.0, 0.5, 1.0, 2.0, 3.0, -1e30, 1e-20], dtype=np.float32)
    u = np.array([5.0, 7.0, -2.0, 4.0, -1.0, 3.0, -2.5, 9.0, 1.0], dtype=np.float32)
    h = oracle.relu2_mul(g, u)
    tiny = np.float32(1e-20) * np.float32(1e-20)  # underflows to a subnormal, one rounding
    np.testing.assert_array_equal(h, np.array([0, 0, 0, 1.0, -1.0, 12.0, -22.5, 0, tiny], dtype=np.float32))
    # the ReLU side never lets a negative gate through, whatever u is
    assert not np.any(h[g <= 0])


def test_relu2_mul_reduces_to_library_square():
    rng = np.random.default_rng(11)
    g = rng.standard_normal(4096).astype(np.float32) * 3
    # u = 1: h is the library's single-rounding square of max(g, 0)
    h = oracle.relu2_mul(g, np.ones_like(g))
    np.testing.assert_array_equal(h, np.square(np.maximum(g, np.float32(0))))
    # scaling u by a power of two scales h exactly; a sign flip of u flips h
    u = rng.standard_normal(4096).astype(np.float32)
    base = oracle.relu2_mul(g, u)
    np.testing.assert_array_equal(oracle.relu2_mul(g, u * np.float32(8)), base * np.float32(8))
    np.testing.assert_array_equal(oracle.relu2_mul(g, -u), -base)
    # within one rounding of the fp64 value (two fp32 roundings: <= 2^-23 relative)
    ref = np.square(np.maximum(g, 0).astype(np.float64)) * u.astype(np.float64)
    assert np.all(np.abs(base - ref) <= np.abs(ref) * 2.0 ** -22.9 + 1e-45)


def test_add_f32_matches_library_add():
    rng = np.random.default_rng(12)
    x = rng.standard_normal(5000).astype(np.float32)
    r = rng.standard_normal(5000).astype(np.float32) * 1e3
    np.testing.assert_array_equal(oracle.add_f32(x, r), np.add(x, r))
    # exact on integers; the input is left untouched
    xi = np.arange(-50, 50, dtype=np.float32)
    np.testing.assert_array_equal(oracle.add_f32(xi, xi), 2 * xi)
    assert xi[0] == -50


# ------------------------------------------------------------- RMS normalization
def test_rmsnorm_constant_and_zero_rows():
    x = np.zeros((3, 64), dtype=np.float32)
    x[0] = 2.0          # mean square 4: r = 1 / sqrt(4 + 1e-5)
    x[1, ::2] = -0.5    # mean square 0.125
    out = oracle.rmsnorm(x)
    r0 = np.float32(1) / np.sqrt(np.float32(4) + oracle.EPS_NORM)
    np.testing.assert_array_equal(out[0], np.full(64, np.float32(2) * r0, dtype=np.float32))
    r1 = np.float32(1) / np.sqrt(np.float32(0.125) + oracle.EPS_NORM)
    np.testing.assert_array_equal(out[1, ::2], np.float32(-0.5) * r1)
    assert not out[1, 1::2].any()
    assert not out[2].any()  # zero row stays zero (r = 1 / sqrt(eps) finite)
    # without the epsilon the constant row would map to exactly 1
    assert abs(float(out[0, 0]) - 1.0) < 2e-6


def test_rmsnorm_unit_rms_and_fp64_bound():
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((5, 2560)) * np.array([[1e-2], [1.0], [3.0], [40.0], [1e3]])).astype(np.float32)
    out = oracle.rmsnorm(x)
    x64 = x.astype(np.float64)
    ref = x64 / np.sqrt((x64 ** 2).mean(1, keepdims=True) + 1e-5)
    # three fp32 roundings of r and one of the product: a few ulp
    assert np.all(np.abs(out - ref) <= np.abs(ref) * 4 * 2.0 ** -23 + 1e-30)
    rms = np.sqrt((out.astype(np.float64) ** 2).mean(1))
    np.testing.assert_allclose(rms[1:], 1.0, rtol=1e-5)
    # the small row is pulled below 1 by the epsilon: rms = s / sqrt(s^2 + eps)
    s = np.sqrt((x64[0] ** 2).mean())
    assert abs(rms[0] - s / np.sqrt(s * s + 1e-5)) < 1e-5


def test_rmsnorm_sign_symmetry_and_row_independence():
    rng = np.random.default_rng(22)
    x = rng.standard_normal((4, 300)).astype(np.float32)
    out = oracle.rmsnorm(x)
    np.testing.assert_array_equal(oracle.rmsnorm(-x), -out)
    np.testing.assert_array_equal(oracle.rmsnorm(x[2:3]), out[2:3])
    np.testing.assert_array_equal(oracle.rmsnorm(x[:, ::-1].copy())[:, ::-1] != 0, out != 0)


# ------------------------------------------------------------- binary weights (b1)
def test_binarize_signs_and_zero():
    w = np.array([-2.0, -1e-30, -0.0, 0.0, 1e-30, 3.0, np.float32(-1e-45)], dtype=np.float32)
    np.testing.assert_array_equal(oracle.binarize(w), [-1, -1, 1, 1, 1, 1, -1])
    rng = np.random.default_rng(31)
    x = rng.standard_normal(100000).astype(np.float32)
    t = oracle.binarize(x)
    assert set(np.unique(t)) == {-1, 1}
    np.testing.assert_array_equal(t, np.where(np.signbit(x) & (x != 0), -1, 1))
    np.testing.assert_array_equal(oracle.binarize(-x), -t)  # no zeros drawn
    # half of a symmetric distribution is positive: within 5 sigma
    assert abs((t == 1).mean() - 0.5) < 5 * 0.5 / np.sqrt(x.size)


def _mfma_sim_b1(packed, q, N, K):
    """acc = q . t^T computed the way a 16x16x64 int8 matrix core consumes the
    1-bit tiles: for step s of a 512-column tile, lane (n, g) supplies the 16
    bits 16*(s%2) .. +15 of its dword s//2, which must be the codes of
    columns 64 s + 16 g + j of row n (bit 1 = +1, bit 0 = -1)."""
    M = q.shape[0]
    Kt, Nt = -(-K // 512), -(-N // 16)
    qp = np.zeros((M, Kt * 512), dtype=np.int64)
    qp[:, :K] = q
    acc = np.zeros((M, Nt * 16), dtype=np.int64)
    tiles = packed.reshape(Nt, Kt, 64, 16)
    for nb in range(Nt):
        for kb in range(Kt):
            words = tiles[nb, kb].copy().view("<u4").reshape(64, 4)
            for s in range(8):
                for lane in range(64):
                    n, g = lane % 16, lane // 16
                    bits = (int(words[lane, s // 2]) >> (16 * (s % 2))) & 0xFFFF
                    b = np.array([(bits >> j) & 1 for j in range(16)], dtype=np.int64) * 2 - 1
                    cols = kb * 512 + 64 * s + 16 * g + np.arange(16)
                    acc[:, nb * 16 + n] += qp[:, cols] @ b
    return acc[:, :N]


@pytest.mark.parametrize("N,K", [(16, 512), (17, 600), (5, 1030)])
def test_pack_b1_feeds_the_matrix_core_contraction(N, K):
    rng = np.random.default_rng(N + K)
    t = np.where(rng.random((N, K)) < 0.5, 1, -1).astype(np.int8)
    q = rng.integers(-127, 128, size=(3, K)).astype(np.int8)
    p = oracle.pack_b1(t)
    assert p.size == -(-N // 16) * -(-K // 512) * 1024 == oracle.b1_bytes(N, K)
    sim = _mfma_sim_b1(p, q, N, K)
    # padded columns read -1 codes against zero activations: no contribution
    np.testing.assert_array_equal(sim, q.astype(np.int64) @ t.astype(np.int64).T)
    np.testing.assert_array_equal(oracle.matmul_i32(q, t), sim)


def test_pack_b1_round_trip_and_padding():
    rng = np.random.default_rng(5)
    for N, K in ((1, 1), (16, 512), (33, 1100), (7, 513)):
        t = np.where(rng.random((N, K)) < 0.5, 1, -1).astype(np.int8)
        p = oracle.pack_b1(t)
        np.testing.assert_array_equal(oracle.unpack_b1(p, N, K), t)
        # one set bit per +1 weight, none in the padding
        assert int(np.unpackbits(p).sum()) == int((t == 1).sum())
    t = -np.ones((16, 512), dtype=np.int8)
    t[3, 200] = 1  # column 200: step 3, group 0, bit 8 of the high half of dword 1 of lane 3
    p = oracle.pack_b1(t)
    assert np.flatnonzero(p).tolist() == [16 * 3 + 4 * 1 + (16 + 8) // 8]
    assert p[16 * 3 + 4 + 3] == 1 << ((16 + 8) % 8)


def test_b1_product_equals_xnor_popcount():
    # textbook identity for +-1 vectors: a . w = K - 2 * popcount(a xor w) on their sign bits
    rng = np.random.default_rng(8)
    K = 777
    a = np.where(rng.random((4, K)) < 0.5, 1, -1).astype(np.int8)
    w = rng.standard_normal((9, K)).astype(np.float32)
    t = oracle.binarize(w)
    acc = oracle.matmul_i32(a, t)
    for m in range(4):
        for n in range(9):
            x = int(np.sum((a[m] > 0) != (t[n] > 0)))
            assert acc[m, n] == K - 2 * x


def test_forward_b1_bound():
    w = workloads.gen_weights(64, 512, seed=3)
    xb = workloads.gen_acts_bf16(4, 512, seed=4)
    out = oracle.bitlinear_forward_b1(xb, w)
    assert set(np.unique(out["t"])) == {-1, 1}
    x = workloads.bf16_bits_to_f32(xb).astype(np.float64)
    approx = x @ (float(out["beta"]) * out["t"].astype(np.float64)).T
    bound = (out["ds"][:, None].astype(np.float64) / 2) * float(out["beta"]) * 512
    assert np.all(np.abs(out["y"] - approx) <= bound * (1 + 1e-6) + 1e-6)


# ------------------------------------------------------------- base-3 packing (b3)
def _mfma_sim_b3(packed, q, N, K):
    """acc = q . t^T computed the way the matrix cores consume base-3 tiles:
    for step s of a 320-column tile, lane (n, g) supplies the base-3 digit s
    of its 16 bytes as operand bytes c in {0, 1, 2} (column 64 s + 16 g + j
    from byte j), and sum q * c - rowsum(q) = sum q * (c - 1)."""
    M = q.shape[0]
    Kt, Nt = -(-K // 320), -(-N // 16)
    qp = np.zeros((M, Kt * 320), dtype=np.int64)
    qp[:, :K] = q
    acc = np.zeros((M, Nt * 16), dtype=np.int64)
    tiles = packed.reshape(Nt, Kt, 64, 16).astype(np.int64)
    for nb in range(Nt):
        for kb in range(Kt):
            for s in range(5):
                digits = (tiles[nb, kb] // 3 ** s) % 3  # [lane][byte]
                for lane in range(64):
                    n, g = lane % 16, lane // 16
                    cols = kb * 320 + 64 * s + 16 * g + np.arange(16)
                    acc[:, nb * 16 + n] += qp[:, cols] @ digits[lane]
    return acc[:, :N] - q.astype(np.int64).sum(1, keepdims=True)


@pytest.mark.parametrize("N,K", [(16, 320), (17, 700), (5, 1030)])
def test_pack_b3_feeds_the_matrix_core_contraction(N, K):
    rng = np.random.default_rng(N * 3 + K)
    t = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    q = rng.integers(-127, 128, size=(3, K)).astype(np.int8)
    p = oracle.pack_b3(t)
    assert p.size == -(-N // 16) * -(-K // 320) * 1024 == oracle.b3_bytes(N, K)
    assert p.max() <= 242
    np.testing.assert_array_equal(_mfma_sim_b3(p, q, N, K), q.astype(np.int64) @ t.astype(np.int64).T)


def test_pack_b3_closed_forms_and_round_trip():
    # all-zero weights: every byte of a full tile is 1 + 3 + 9 + 27 + 81 = 121
    p = oracle.pack_b3(np.zeros((16, 320), dtype=np.int8))
    assert np.all(p == 121)
    # all +1: 2 * 121 = 242, all -1: 0
    assert np.all(oracle.pack_b3(np.ones((16, 320), dtype=np.int8)) == 242)
    assert not oracle.pack_b3(-np.ones((16, 320), dtype=np.int8)).any()
    # padding contributes nothing: a 1 x 1 zero weight sets digit 0 of byte 0 only
    p = oracle.pack_b3(np.zeros((1, 1), dtype=np.int8))
    assert p[0] == 1 and not p[1:].any()
    # one weight at (3, 200): step 3, group 0, byte 8 of lane 3 -> +2 * 27 over the -1 background
    t = -np.ones((16, 320), dtype=np.int8)
    t[3, 200] = 1
    p = oracle.pack_b3(t)
    assert np.flatnonzero(p).tolist() == [16 * 3 + 8] and p[16 * 3 + 8] == 2 * 27
    rng = np.random.default_rng(13)
    for N, K in ((1, 1), (33, 1100), (7, 321), (64, 2560)):
        t = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
        np.testing.assert_array_equal(oracle.unpack_b3(oracle.pack_b3(t), N, K), t)


def test_b3_digits_cover_every_byte_value():
    # every byte value 0..242 is reachable and decodes to its base-3 digits
    vals = np.arange(243)
    digits = np.stack([(vals // 3 ** s) % 3 for s in range(5)], 1)  # [243][5]
    t = np.zeros((16, 320), dtype=np.int8)
    for v in range(243):
        lane, i = divmod(v, 16)
        if lane >= 64:
            break
        n, g = lane % 16, lane // 16
        for s in range(5):
            t[n, 64 * s + 16 * g + i] = digits[v, s] - 1
    p = oracle.pack_b3(t).reshape(64, 16)
    np.testing.assert_array_equal(p.reshape(-1)[:243], vals)


# ------------------------------------------------------------- training products (STE)
def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_train_products_small_exact():
    # integers: every product and sum is exact, beta a power of two
    x = np.array([[1, 2, 3], [-1, 0, 4]], dtype=np.float32)
    t = np.array([[1, 0, -1], [-1, 1, 1], [0, 0, 1], [1, 1, 1]], dtype=np.int8)
    dy = np.array([[1, -2, 0, 3], [2, 1, -1, 0]], dtype=np.float32)
    beta = np.float32(0.5)
    np.testing.assert_array_equal(oracle.train_forward(_bf16(x), t, beta), 0.5 * (x @ t.T.astype(np.float32)))
    np.testing.assert_array_equal(oracle.train_dx(_bf16(dy), t, beta), 0.5 * (dy @ t.astype(np.float32)))
    np.testing.assert_array_equal(oracle.train_dw(_bf16(dy), _bf16(x)), dy.T @ x)


def test_train_products_match_library_matmul_and_adjoints():
    rng = np.random.default_rng(41)
    M, K, N = 7, 300, 13
    xb = _bf16(rng.standard_normal((M, K)))
    dyb = _bf16(rng.standard_normal((M, N)))
    w = rng.standard_normal((N, K)).astype(np.float32) * 0.02
    beta = oracle.absmean(w)
    t = oracle.ternarize(w, beta)
    x = workloads.bf16_bits_to_f32(xb).astype(np.float64)
    dy = workloads.bf16_bits_to_f32(dyb).astype(np.float64)
    wq = float(beta) * t.astype(np.float64)
    y = oracle.train_forward(xb, t, beta, threads=4)
    dx = oracle.train_dx(dyb, t, beta, threads=4)
    dw = oracle.train_dw(dyb, xb, threads=4)
    # one fp32 rounding of the exact value (numpy's fp64 products as the independent routine)
    for got, ref in ((y, x @ wq.T), (dx, dy @ wq), (dw, dy.T @ x)):
        assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -23 + 1e-30)
    # adjoint identities tie the three products together: <dy, y> = <dx, x> = <dw, wq>
    a = float((dy * y.astype(np.float64)).sum())
    b = float((dx.astype(np.float64) * x).sum())
    c = float((dw.astype(np.float64) * wq).sum())
    scale = float(np.abs(dy).sum() * np.abs(x).sum())
    assert abs(a - b) <= 1e-6 * scale and abs(a - c) <= 1e-6 * scale
