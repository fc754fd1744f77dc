"""Pins of the oracle's quantize formula: codes are rne(x * fl(127 / amax)), one
binary32 multiply by the rounded reciprocal ("EQuARX" verdict page,
pith_extraction.key_machinery: the second phase scales the data by the block's
factor; the reading fixes that factor as the binary32 reciprocal 127 / amax).

The reference here is numpy's IEEE binary32 arithmetic on the same bf16 inputs
(one rounding per operation, no fused multiply-add) and numpy's rint (round
half to even): a library special case, independent of the oracle's C code.
The same holds for the weights' first level with its protective range 112
("LiquidGEMM" verdict page, referee_report.major_comments[2]).

Each pin has a control: the other plausible reading, dividing by the stored
scale (rne(x / fl(amax / 127))), gives different codes on the same sample, so
an oracle written in that form fails these tests.
"""
import numpy as np
import pytest

import oracle
from w4a8_quantized_gemm_quantize_amd import inputs

F32 = np.float32


def _sample(rows, cols, seed):
    """Rows of N(0,1) with 0.1 % outliers x20, then rows of unit Student t(3)."""
    half = rows // 2
    a = inputs.activations(half, cols, seed, "normal", outlier_frac=0.001)
    b = inputs.activations(rows - half, cols, seed + 1, "student_t")
    return np.ascontiguousarray(np.concatenate([a, b], axis=0))


def _numpy_blockwise(x_bits, block, divide=False):
    """Block absmax quantization in numpy binary32.  divide=False: the pinned
    reading rne(x * fl(127/amax)); divide=True: the control rne(x / fl(amax/127))."""
    x = inputs.bf16_bits_to_f32(x_bits)
    rows, cols = x.shape
    xb = x.reshape(rows, cols // block, block)
    amax = np.abs(xb).max(axis=2).astype(F32)
    s = (amax / F32(127)).astype(F32)
    pos = amax > 0
    if divide:
        safe = np.where(pos, s, F32(1)).astype(F32)
        v = (xb / safe[:, :, None]).astype(F32)
    else:
        inv = np.where(pos, F32(127) / np.where(pos, amax, F32(1)), F32(0)).astype(F32)
        v = (xb * inv[:, :, None]).astype(F32)
    q = np.clip(np.rint(v), -127, 127).astype(np.int8)
    q[~pos] = 0
    return q.reshape(rows, cols), s


ROWS, COLS = 256, 4096            # 1,048,576 elements per sample


@pytest.mark.parametrize("block", [8, 32, 128, 1024, COLS])
def test_act_codes_are_rne_of_product_with_rounded_reciprocal(block):
    x = _sample(ROWS, COLS, seed=11)
    q, s = oracle.quantize_act_blockwise(x, block)
    q_ref, s_ref = _numpy_blockwise(x, block)
    assert np.array_equal(s, s_ref), "scales differ from fl(amax / 127)"
    diff = int((q != q_ref).sum())
    assert diff == 0, f"{diff} codes differ from rne(x * fl(127/amax))"


@pytest.mark.parametrize("block", [8, 32, 128, 1024, COLS])
@pytest.mark.parametrize("dist", ["mixed", "normal"])
def test_act_divide_form_is_told_apart(block, dist):
    # Control: on these samples the divide-by-scale reading disagrees with the
    # pinned one, so the bit-exact test above fails for an oracle written that
    # way (one differing code is enough).  Per-token blocks of heavy-tailed rows
    # have large scales and few near-ties (a handful of disagreements per
    # million codes); N(0,1) rows give hundreds.
    if dist == "mixed":
        x = _sample(ROWS, COLS, seed=11)
    else:
        x = inputs.activations(ROWS, COLS, 11, "normal")
    q, q_ref = oracle.quantize_act_blockwise(x, block)[0], _numpy_blockwise(x, block)[0]
    assert np.array_equal(q, q_ref)
    q_div, _ = _numpy_blockwise(x, block, divide=True)
    differ = int((q != q_div).sum())
    assert differ >= (5 if dist == "mixed" else 100), \
        f"only {differ} codes separate the two readings"
    # the two readings differ by one code step, at near-ties only
    assert int(np.abs(q.astype(np.int32) - q_div.astype(np.int32)).max()) == 1


def _numpy_level1(w_bits, rng_val, divide=False):
    w = inputs.bf16_bits_to_f32(w_bits)
    c = np.abs(w).max(axis=1).astype(F32)
    s_ch = (c / F32(rng_val)).astype(F32)
    pos = c > 0
    if divide:
        v = (w / np.where(pos, s_ch, F32(1))[:, None]).astype(F32)
    else:
        inv = np.where(pos, F32(rng_val) / np.where(pos, c, F32(1)), F32(0)).astype(F32)
        v = (w * inv[:, None]).astype(F32)
    q = np.clip(np.rint(v), -rng_val, rng_val).astype(np.int32)
    q[~pos] = 0
    return q, s_ch


def test_weight_level1_is_rne_of_product_with_rounded_reciprocal():
    w = inputs.weights(256, 4096, seed=5)
    w8, s_ch = oracle.weight_level1(w)
    q_ref, s_ref = _numpy_level1(w, 112)
    assert np.array_equal(s_ch, s_ref)
    diff = int((w8.astype(np.int32) != q_ref).sum())
    assert diff == 0, f"{diff} level-1 codes differ from rne(w * fl(112/c))"


def test_weight_level1_divide_form_is_told_apart():
    w = inputs.weights(256, 4096, seed=5)
    w8, _ = oracle.weight_level1(w)
    q_div, _ = _numpy_level1(w, 112, divide=True)
    differ = int((w8.astype(np.int32) != q_div).sum())
    assert differ >= 50, f"only {differ} level-1 codes separate the two readings"


def test_pack_uses_the_pinned_first_level():
    # The two-level quantizer starts from the same first level: its effective
    # int8 weight s_g * q stays within s_g / 2 of the pinned level-1 codes.
    w = inputs.weights(64, 1024, seed=7)
    q, s_g, s_ch = oracle.quantize_w4_grouped(w, 64)
    q_ref, s_ref = _numpy_level1(w, 112)
    assert np.array_equal(s_ch, s_ref)
    sg = np.repeat(s_g.astype(np.int32), 64, axis=1)
    err = np.abs(q.astype(np.int32) * sg - q_ref)
    assert (2 * err <= sg).all()


def test_fused_codes_follow_the_pinned_formula():
    # The fused call's per-token codes are the block == k case of the pin.
    a = _sample(16, 2048, seed=3)
    w = inputs.weights(32, 2048, seed=3)
    q, s_g, s_ch = oracle.quantize_w4_grouped(w, 64)
    a_q, a_s, _, _ = oracle.w4a8_gemm_bf16act(a, q, s_g, s_ch, 64)
    q_ref, s_ref = _numpy_blockwise(a, 2048)
    assert np.array_equal(a_q, q_ref)
    assert np.array_equal(a_s.reshape(-1), s_ref.reshape(-1))
