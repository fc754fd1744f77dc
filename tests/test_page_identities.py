"""The dequantization identity the pages print, checked exhaustively.

LiquidGEMM verdict page, pith_extraction.key_machinery: a 4-bit code u is
turned back into the INT8 weight by (u * s + a) XOR 0x80 with a = 2^7 + min,
and referee_report.summary / desk_editor.letter: the computation stays inside
UINT8 (no overflow).  The symmetric instance used by the W4A8 path (codes
q in [-7, 7] stored as u = q + 8, integer group scale s in [1, 16], offset
128 - 8 s) is checked the same way; it is what lets four weights be rebuilt
with one packed 16-bit multiply-add and one XOR per 32-bit word.
"""
import json
import os

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
C = json.load(open(os.path.join(HERE, "golden", "page_constants.json")))


def rne_div(a, b):
    """Exact a / b rounded half to even (integers, b > 0)."""
    q, r = divmod(a, b)
    if 2 * r > b or (2 * r == b and q % 2 == 1):
        q += 1
    return q


def test_symmetric_identity_exhaustive():
    for s in range(1, C["lqq_group_scale_bound"]["value"] + 1):
        for q in range(-7, 8):
            u = q + 8
            v = u * s + 128 - 8 * s
            assert 0 <= v <= 255                      # stays inside UINT8: no carry between bytes
            r = v ^ C["lqq_xor_constant"]["value"]
            r = r - 256 if r >= 128 else r             # read the byte as int8
            assert r == q * s


def test_symmetric_protective_range_is_the_largest_with_scale_le_16():
    # ceil(R / 7) <= 16 holds exactly for R <= 112; the page's 119 would need s = 17.
    bound = C["lqq_group_scale_bound"]["value"]
    assert max(R for R in range(1, 128) if -(-R // 7) <= bound) == 112
    assert -(-C["lqq_protective_range"]["value"] // 7) == 17


@pytest.mark.parametrize("rule", ["round", "floor", "ceil"])
def test_lqq_asymmetric_identity_exhaustive(rule):
    # Every (min, max) inside the protective range and every weight between them.
    R = C["lqq_protective_range"]["value"]
    levels = C["lqq_uint4_levels"]["value"]
    max_s = 0
    for lo in range(-R, R + 1):
        for hi in range(lo, R + 1):
            span = hi - lo
            if rule == "round":
                s = rne_div(span, levels)
            elif rule == "floor":
                s = span // levels
            else:
                s = -(-span // levels)
            s = max(s, 1)
            max_s = max(max_s, s)
            a = 128 + lo
            u_max = min(levels, rne_div(span, s))   # largest code quantization emits
            for u in range(0, u_max + 1):
                v = u * s + a
                rec = u * s + lo
                assert 0 <= v <= 255
                r = v ^ C["lqq_xor_constant"]["value"]
                r = r - 256 if r >= 128 else r
                assert r == rec
    if rule == "round":
        assert max_s == C["lqq_group_scale_bound"]["value"]
    if rule == "floor":
        assert max_s == C["lqq_group_scale_floor_of_range"]["value"]
