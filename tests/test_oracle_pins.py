"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's formulas: each checks the oracle against a
closed form, an invariant, a special case that reduces to a library routine,
or brute force over a tiny domain.  A plausible mistake in the oracle (a wrong
divisor, a dropped scale, a transposed operand, a wrong block or group index,
truncation instead of round-half-even) fails at least one of them.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from w4a8_quantized_gemm_quantize_amd import inputs

U = 2.0 ** -24  # binary32 unit roundoff


def bf16(values):
    return inputs.f32_to_bf16_bits(np.asarray(values, np.float32))


def f32(bits):
    return inputs.bf16_bits_to_f32(bits)


def rne_fraction(fr: Fraction) -> int:
    """Round an exact rational half to even."""
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


# ------------------------------------------------------------ activations --

def test_act_zero_block_gives_zero_codes_and_scale():
    x = bf16(np.zeros((3, 64)))
    q, s = oracle.quantize_act_blockwise(x, 32)
    assert (q == 0).all() and (s == 0).all()


def test_act_integer_block_is_identity_with_unit_scale():
    # A block of integers whose absmax is 127: scale is exactly 1, codes equal x.
    g = np.random.default_rng(1)
    vals = g.integers(-127, 128, size=(4, 128)).astype(np.float32)
    vals[:, 5] = 127.0
    vals[2, 5] = -127.0
    q, s = oracle.quantize_act_blockwise(bf16(vals), 128)
    assert (s == 1.0).all()
    assert np.array_equal(q.astype(np.float32), vals)


def test_act_sign_symmetry():
    x = inputs.activations(8, 256, seed=3)
    q, s = oracle.quantize_act_blockwise(x, 32)
    qn, sn = oracle.quantize_act_blockwise(x ^ np.uint16(0x8000), 32)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)


@pytest.mark.parametrize("j", [-3, 5])
def test_act_power_of_two_scaling(j):
    # Scaling by 2^j commutes with every binary32 rounding (no over/underflow here).
    x = inputs.activations(8, 256, seed=4)
    xs = bf16(f32(x) * np.float32(2.0 ** j))
    q, s = oracle.quantize_act_blockwise(x, 64)
    q2, s2 = oracle.quantize_act_blockwise(xs, 64)
    assert np.array_equal(q2, q)
    assert np.array_equal(s2, (s * np.float32(2.0 ** j)).astype(np.float32))


def test_act_argmax_maps_to_full_scale_code():
    x = inputs.activations(64, 512, seed=5)
    q, _ = oracle.quantize_act_blockwise(x, 32)
    xf = f32(x).reshape(-1, 32)
    qb = q.reshape(-1, 32).astype(np.int32)
    idx = np.abs(xf).argmax(axis=1)
    rows = np.arange(xf.shape[0])
    assert (np.abs(qb[rows, idx]) == 127).all()
    assert (np.sign(qb[rows, idx]) == np.sign(xf[rows, idx])).all()
    assert (np.abs(qb) <= 127).all()


@pytest.mark.parametrize("block", [8, 32, 128, 1024])
def test_act_reconstruction_bound(block):
    # |q*s - x| <= s * (1/2 + 381 u): three binary32 roundings on |x*inv| <= 127.
    x = inputs.activations(64, 1024, seed=6, outlier_frac=0.001)
    q, s = oracle.quantize_act_blockwise(x, block)
    xf = f32(x).astype(np.float64).reshape(-1, block)
    sf = s.astype(np.float64).reshape(-1, 1)
    err = np.abs(q.astype(np.float64).reshape(-1, block) * sf - xf)
    assert (err <= sf * (0.5 + 381 * U * 1.001)).all()


def test_act_block_indexing_matches_rows_of_one_block():
    # Quantizing [r, c] with blocks of b equals quantizing [r*c/b, b] with one block per row.
    x = inputs.activations(16, 512, seed=7)
    q, s = oracle.quantize_act_blockwise(x, 64)
    q2, s2 = oracle.quantize_act_blockwise(x.reshape(-1, 64), 64)
    assert np.array_equal(q.reshape(-1, 64), q2)
    assert np.array_equal(s.reshape(-1), s2.reshape(-1))


def test_act_brute_force_against_exact_rational_rounding():
    # Every bf16 value in [-3, 3] in one block whose absmax is 3: the code is the
    # round-half-even of the exact x * 127 / 3 unless that value lies within
    # 1e-4 of a tie (where the binary32 product may fall on either side).
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = f32(allbits)
    keep = np.isfinite(vals) & (np.abs(vals) <= 3.0)
    xbits = allbits[keep]
    xbits = np.concatenate([xbits, bf16([3.0])])
    q, s = oracle.quantize_act_blockwise(xbits.reshape(1, -1), xbits.size)
    assert s[0, 0] == np.float32(3.0) / np.float32(127.0)
    checked = 0
    for b, code in zip(xbits.tolist(), q.reshape(-1).tolist()):
        xv = Fraction(float(f32(np.array([b], np.uint16))[0]))
        exact = xv * 127 / 3
        frac = exact - (exact.numerator // exact.denominator)
        if abs(frac - Fraction(1, 2)) < Fraction(1, 10000):
            assert code in (exact.numerator // exact.denominator,
                            exact.numerator // exact.denominator + 1)
        else:
            assert code == rne_fraction(exact), (b, code, float(exact))
            checked += 1
    assert checked > 30000


def test_act_exact_ties_round_to_even():
    # amax = 63.5 makes 127/amax exactly 2, so x = j + 1/4 lands exactly on a
    # half-integer: the code must round half to even (0.5 -> 0, 1.5 -> 2, -2.5 -> -2).
    xs = [63.5, 0.25, 0.75, 1.25, -0.25, -0.75, -1.25, 2.25]
    q, s = oracle.quantize_act_blockwise(bf16([xs]), 8)
    assert s[0, 0] == np.float32(63.5) / np.float32(127.0)
    assert q.tolist() == [[127, 0, 2, 2, 0, -2, -2, 4]]


def test_weight_level1_exact_ties_round_to_even():
    # c = 56 makes 112/c exactly 2: w = j + 1/4 is an exact tie.
    xs = np.zeros((1, 64), np.float32)
    xs[0, :6] = [56.0, 0.25, 0.75, -0.25, -1.25, 1.25]
    w8, s_ch = oracle.weight_level1(bf16(xs))
    assert s_ch[0] == 0.5
    assert w8[0, :6].tolist() == [112, 0, 2, 0, -2, 2]


def test_act_tiny_amax_saturates_and_zero_stays_zero():
    # amax below 127/FLT_MAX makes 127/amax overflow: non-zero codes saturate, 0 stays 0.
    tiny = np.float32(2.0 ** -126)
    x = bf16(np.array([[tiny, -tiny, 0.0, tiny / 2, 0.0, 0.0, 0.0, 0.0]], np.float32))
    q, s = oracle.quantize_act_blockwise(x, 8)
    assert q.tolist() == [[127, -127, 0, 127, 0, 0, 0, 0]]
    assert s[0, 0] == np.float32(tiny) / np.float32(127.0)


@pytest.mark.parametrize("block,lo,hi", [(32, 2.6e-5, 3.1e-5), (128, 3.9e-5, 4.5e-5)])
def test_act_round_trip_mse_closed_form(block, lo, hi):
    # Uniform rounding error: MSE ~= E[s^2] / 12 (s = amax/127 per block) on N(0,1).
    x = inputs.activations(1024, 1024, seed=0)
    q, s = oracle.quantize_act_blockwise(x, block)
    xf = f32(x).astype(np.float64)
    xh, xh_bf16 = oracle.dequantize_act_blockwise(q, s, block)
    mse = float(np.mean((xh.astype(np.float64) - xf) ** 2))
    predicted = float(np.mean(s.astype(np.float64) ** 2)) / 12.0
    assert abs(mse / predicted - 1.0) < 0.05
    assert lo < mse < hi
    mse_bf16 = float(np.mean((f32(xh_bf16).astype(np.float64) - xf) ** 2))
    assert mse < mse_bf16 < 1.2 * mse


def test_dequant_is_the_rounded_product():
    x = inputs.activations(32, 256, seed=8)
    q, s = oracle.quantize_act_blockwise(x, 32)
    xh, xb = oracle.dequantize_act_blockwise(q, s, 32)
    exact = q.astype(np.float64) * np.repeat(s.astype(np.float64), 32, axis=1)
    # one rounding of an exact product
    assert (np.abs(xh.astype(np.float64) - exact) <= U * np.abs(exact)).all()
    # bf16 output is within half a bf16 ulp (unit roundoff 2^-8) of the binary32 value
    assert (np.abs(f32(xb).astype(np.float64) - xh) <= 2.0 ** -8 * np.abs(xh)).all()


# ---------------------------------------------------------------- weights --

def test_weight_level2_exhaustive_brute_force():
    # Every int8 value |v| <= 112 in a group of 64 for every group absmax m in 0..112:
    # s_g is the least s >= 1 with 7 s >= m, and q the nearest multiple index, ties even.
    rows = []
    for m in range(0, 113):
        vals = np.arange(-m, m + 1)
        reps = int(np.ceil(len(vals) / 63))
        for r in range(reps):
            chunk = vals[r * 63:(r + 1) * 63]
            row = np.zeros(64, np.int64)
            row[:len(chunk)] = chunk
            row[63] = m
            rows.append(row)
    w8 = np.array(rows, np.int8)
    q, sg = oracle.weight_level2(w8, 64)
    for i in range(w8.shape[0]):
        m = int(np.abs(w8[i]).max())
        s_expect = next(s for s in range(1, 17) if 7 * s >= m)
        assert sg[i, 0] == s_expect
        for v, code in zip(w8[i].tolist(), q[i].tolist()):
            best = min(range(-7, 8), key=lambda c: (abs(2 * v - 2 * c * s_expect), c % 2))
            assert code == best, (v, s_expect, code, best)


def test_weight_level1_integer_row_and_symmetry():
    vals = np.zeros((2, 128), np.float32)
    vals[0, :5] = [112, -56, 3, 0, -111]
    vals[1, :3] = [-112, 1, 2]
    w8, s_ch = oracle.weight_level1(bf16(vals))
    assert (s_ch == 1.0).all()
    assert np.array_equal(w8.astype(np.float32), vals)
    w = inputs.weights(16, 256, seed=2)
    a8, ac = oracle.weight_level1(w)
    b8, bc = oracle.weight_level1(w ^ np.uint16(0x8000))
    assert np.array_equal(b8, -a8) and np.array_equal(bc, ac)


def test_weight_invariants():
    w = inputs.weights(64, 512, seed=9)
    q, sg, sch = oracle.quantize_w4_grouped(w, 64)
    w8, sch1 = oracle.weight_level1(w)
    assert np.array_equal(sch, sch1)
    wf = f32(w).astype(np.float64)
    # level 1 reconstruction bound
    err1 = np.abs(w8.astype(np.float64) * sch.astype(np.float64)[:, None] - wf)
    assert (err1 <= sch.astype(np.float64)[:, None] * (0.5 + 336 * U * 1.001)).all()
    # level 2: codes in range, |W8 - q s_g| <= s_g / 2, |q s_g| <= 112
    sgx = np.repeat(sg.astype(np.int64), 64, axis=1)
    assert (np.abs(q) <= 7).all() and (sg >= 1).all() and (sg <= 16).all()
    assert (2 * np.abs(w8.astype(np.int64) - q.astype(np.int64) * sgx) <= sgx).all()
    assert (np.abs(q.astype(np.int64) * sgx) <= 112).all()
    # every non-zero row reaches the full protective range in some group -> s_g = 16
    assert (np.abs(w8).max(axis=1) == 112).all()
    assert (sg.max(axis=1) == 16).all()


def test_weight_error_magnitude():
    # Two-level 4-bit weights on N(0, 0.02^2): relative Frobenius error ~0.11.
    w = inputs.weights(256, 1024, seed=0)
    q, sg, sch = oracle.quantize_w4_grouped(w, 64)
    wh = oracle.dequantize_w4_grouped(q, sg, sch, 64)
    wf = f32(w).astype(np.float64)
    rel = np.linalg.norm(wh - wf) / np.linalg.norm(wf)
    assert 0.08 < rel < 0.15


def test_zero_weight_row():
    w = inputs.weights(4, 128, seed=1)
    w[2] = 0
    q, sg, sch = oracle.quantize_w4_grouped(w, 64)
    assert sch[2] == 0 and (q[2] == 0).all() and (sg[2] == 1).all()


# ------------------------------------------------------------------- GEMM --

def _operands(m, n, k, seed):
    a = inputs.activations(m, k, seed=seed)
    w = inputs.weights(n, k, seed=seed)
    a_q, a_s = oracle.quantize_act_blockwise(a, k)
    q, sg, sch = oracle.quantize_w4_grouped(w, 64)
    return a, w, a_q, a_s.reshape(-1), q, sg, sch


def test_group_sums_match_numpy_int64():
    _, _, a_q, _, q, _, _ = _operands(5, 48, 256, 11)
    P = oracle.group_sums(a_q, q, 64)
    ref = np.einsum("mgk,ngk->mng", a_q.astype(np.int64).reshape(5, 4, 64),
                    q.astype(np.int64).reshape(48, 4, 64))
    assert np.array_equal(P.astype(np.int64), ref)


def test_accumulator_matches_numpy_matmul():
    _, _, a_q, a_s, q, sg, sch = _operands(7, 80, 320, 12)
    acc, _ = oracle.w4a8_gemm(a_q, a_s, q, sg, sch, 64)
    w_int = q.astype(np.int64) * np.repeat(sg.astype(np.int64), 64, axis=1)
    assert np.array_equal(acc.astype(np.int64), a_q.astype(np.int64) @ w_int.T)


def test_one_hot_rows_select_single_weights():
    n, k = 32, 256
    w = inputs.weights(n, k, seed=13)
    q, sg, sch = oracle.quantize_w4_grouped(w, 64)
    a_q = np.eye(k, dtype=np.int8)[[0, 63, 64, 130, 255]]
    acc, _ = oracle.w4a8_gemm(a_q, np.ones(5, np.float32), q, sg, sch, 64)
    for i, kk in enumerate([0, 63, 64, 130, 255]):
        assert np.array_equal(acc[i], q[:, kk].astype(np.int32) * sg[:, kk // 64])


def test_all_ones_gives_group_scale_sum():
    n, k = 16, 384
    q = np.ones((n, k), np.int8)
    sg = np.random.default_rng(3).integers(1, 17, size=(n, k // 64)).astype(np.uint8)
    acc, _ = oracle.w4a8_gemm(np.ones((2, k), np.int8), np.ones(2, np.float32), q, sg,
                              np.ones(n, np.float32), 64)
    assert np.array_equal(acc[0], 64 * sg.astype(np.int32).sum(axis=1))


def test_split_k_is_exact():
    _, _, a_q, a_s, q, sg, sch = _operands(3, 32, 512, 14)
    acc, _ = oracle.w4a8_gemm(a_q, a_s, q, sg, sch, 64)
    acc1, _ = oracle.w4a8_gemm(a_q[:, :192], a_s, q[:, :192], sg[:, :3], sch, 64)
    acc2, _ = oracle.w4a8_gemm(a_q[:, 192:], a_s, q[:, 192:], sg[:, 3:], sch, 64)
    assert np.array_equal(acc, acc1 + acc2)


def test_output_equals_product_of_dequantized_operands():
    # y must equal (a_q * s_a) @ w_hat^T computed by numpy in float64.
    _, _, a_q, a_s, q, sg, sch = _operands(6, 64, 256, 15)
    _, y = oracle.w4a8_gemm(a_q, a_s, q, sg, sch, 64)
    wh = oracle.dequantize_w4_grouped(q, sg, sch, 64)
    ref = (a_q.astype(np.float64) * a_s.astype(np.float64)[:, None]) @ wh.T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_end_to_end_error_against_unquantized_matmul():
    a, w, a_q, a_s, q, sg, sch = _operands(16, 256, 256, 0)
    _, y = oracle.w4a8_gemm(a_q, a_s, q, sg, sch, 64)
    ref = f32(a).astype(np.float64) @ f32(w).astype(np.float64).T
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert 0.05 < rel < 0.2


def test_fused_equals_quantize_then_gemm():
    a, w, a_q, a_s, q, sg, sch = _operands(9, 32, 192, 16)
    fq, fs, facc, fy = oracle.w4a8_gemm_bf16act(a, q, sg, sch, 64)
    acc, y = oracle.w4a8_gemm(a_q, a_s, q, sg, sch, 64)
    assert np.array_equal(fq, a_q) and np.array_equal(fs, a_s)
    assert np.array_equal(facc, acc) and np.array_equal(fy, y)


def test_k_max_bound_rejected():
    with pytest.raises(ValueError):
        oracle.w4a8_gemm(np.zeros((1, 150976 + 64), np.int8), np.ones(1, np.float32),
                         np.zeros((16, 150976 + 64), np.int8),
                         np.ones((16, (150976 + 64) // 64), np.uint8),
                         np.ones(16, np.float32), 64, want_y=False)


def test_extreme_accumulator_fits_int32():
    # |acc| <= K * 127 * 112 at K_MAX: all codes at their extremes.
    k = oracle.K_MAX
    a_q = np.full((1, k), -127, np.int8)
    q = np.full((16, k), 7, np.int8)
    sg = np.full((16, k // 64), 16, np.uint8)
    acc, _ = oracle.w4a8_gemm(a_q, np.ones(1, np.float32), q, sg, np.ones(16, np.float32),
                              64, want_y=False)
    assert (acc.astype(np.int64) == -127 * 112 * k).all()
    assert -127 * 112 * k >= -(2 ** 31)
