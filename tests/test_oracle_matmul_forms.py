"""The oracle's matmul forms of the three GEMMs (a binary64 library matmul of
the integer operands) against its plain C loops: accumulators and binary64
outputs equal bit for bit on ragged shapes, including the largest accumulators
(extreme codes at K_MAX) and a trailing half chunk.  The C loops themselves are
pinned in test_oracle_pins.py / test_oracle_ext_pins.py."""
import numpy as np
import pytest

import oracle
from w4a8_quantized_gemm_quantize_amd import inputs


def _act(m, k, seed):
    return oracle.quantize_act_blockwise(inputs.activations(m, k, seed, outlier_frac=0.001), k)


@pytest.mark.parametrize("m,n,k", [(5, 48, 192), (33, 80, 1088), (70, 64, 4160), (1, 16, 64)])
def test_w4_matmul_form_equals_loops(m, n, k):
    q, s_g, s_ch = oracle.quantize_w4_grouped(inputs.weights(n, k, seed=m + n), 64)
    a_q, a_s = _act(m, k, seed=k)
    acc1, y1 = oracle.w4a8_gemm(a_q, a_s, q, s_g, s_ch, 64)
    acc2, y2 = oracle.w4a8_gemm_matmul(a_q, a_s, q, s_g, s_ch, 64)
    assert np.array_equal(acc1, acc2)
    assert np.array_equal(y1.view(np.uint64), y2.view(np.uint64))


@pytest.mark.parametrize("m,n,k", [(5, 48, 192), (33, 80, 1088)])
def test_lqq_matmul_form_equals_loops(m, n, k):
    q_u4, s_u8, w_min, s_ch = oracle.quantize_w4_lqq(inputs.weights(n, k, seed=n), 64)
    a_q, a_s = _act(m, k, seed=m)
    acc1, y1 = oracle.w4a8_gemm_lqq(a_q, a_s, q_u4, s_u8, w_min, s_ch, 64)
    acc2, y2 = oracle.w4a8_gemm_lqq_matmul(a_q, a_s, q_u4, s_u8, w_min, s_ch, 64)
    assert np.array_equal(acc1, acc2)
    assert np.array_equal(y1.view(np.uint64), y2.view(np.uint64))


@pytest.mark.parametrize("m,n,k", [(5, 48, 192), (33, 80, 1088)])
def test_w8_matmul_form_equals_loops(m, n, k):
    q8, s_ch = oracle.quantize_w8_channel(inputs.weights(n, k, seed=k))
    a_q, a_s = _act(m, k, seed=n)
    acc1, y1 = oracle.w8a8_gemm(a_q, a_s, q8, s_ch)
    acc2, y2 = oracle.w8a8_gemm_matmul(a_q, a_s, q8, s_ch)
    assert np.array_equal(acc1, acc2)
    assert np.array_equal(y1.view(np.uint64), y2.view(np.uint64))


def test_matmul_form_exact_at_the_accumulator_bound():
    # all codes at their extremes over K_MAX: |acc| = K_MAX * 127 * 112, the
    # largest value the int32 bound allows; binary64 still holds it exactly
    k = oracle.K_MAX
    a_q = np.full((2, k), -127, np.int8)
    a_q[1] = 127
    q = np.full((16, k), 7, np.int8)
    s_g = np.full((16, k // 64), 16, np.uint8)
    s_ch = np.ones(16, np.float32)
    a_s = np.ones(2, np.float32)
    acc, _ = oracle.w4a8_gemm_matmul(a_q, a_s, q, s_g, s_ch, 64)
    assert (acc[0] == -127 * 112 * k).all() and (acc[1] == 127 * 112 * k).all()
    acc_loop, _ = oracle.w4a8_gemm(a_q, a_s, q, s_g, s_ch, 64, want_y=False)
    assert np.array_equal(acc, acc_loop)
