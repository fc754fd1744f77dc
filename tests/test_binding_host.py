"""Host checks of the Python binding's argument marshalling (no GPU needed): the
library takes raw pointers, so the binding rejects host tensors, wrong dtypes and
undersized buffers before any call reaches it."""
import os

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "w4a8_quantized_gemm_quantize_amd", "libw4a8.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libw4a8.so not built")


@pytest.fixture(scope="module")
def b():
    from w4a8_quantized_gemm_quantize_amd import binding
    return binding


def test_host_tensors_are_rejected(b):
    m, n, k = 4, 16, 128
    a_q = torch.zeros((m, k), dtype=torch.int8)
    with pytest.raises(ValueError):
        b.w4a8_gemm(a_q, torch.ones(m), torch.zeros(n * k // 2, dtype=torch.uint8),
                    torch.ones(n * k // 64, dtype=torch.uint8), torch.ones(n), n)
    with pytest.raises(ValueError):
        b.quantize_act_blockwise(torch.zeros((m, k), dtype=torch.bfloat16), 32)
    with pytest.raises(ValueError):
        b.pack_w4_grouped(torch.zeros((n, k), dtype=torch.bfloat16))


def test_sized_rules(b):
    # None passes through: the library itself reports a missing pointer
    b._sized("f", None, b._F32, 10, "x")
    with pytest.raises(ValueError):
        b._sized("f", torch.zeros(16), b._F32, 4, "x")          # host tensor
    with pytest.raises(ValueError):
        b._sized("f", [1.0] * 16, b._F32, 4, "x")               # not a tensor
    assert b._per(192, 64) == 3 and b._per(192, 0) == 0 and b._per(100, 48) == 2
    err = b.W4A8SizeError("w4a8_gemm", "out", 10, 64)
    assert isinstance(err, b.W4A8Error) and err.status == b.ERR_SHAPE
    assert "out holds 10 elements" in str(err)
