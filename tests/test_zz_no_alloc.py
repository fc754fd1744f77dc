"""The no-allocation fused entry point (w4a8_gemm_bf16act_noalloc, workspace in
the library's static device array) against w4a8_gemm_bf16act with a caller
workspace: identical outputs, for two calls in a row on the same array, the
second with a smaller input, over the fused one-kernel path (m <= 16), the
split-K path (partials in the array) and the tiled path; and the size limit."""
import numpy as np
import pytest
import torch

from w4a8_quantized_gemm_quantize_amd import inputs

from gpu_util import to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4a8():
    from w4a8_quantized_gemm_quantize_amd import binding
    torch.cuda.init()
    return binding


def _case(w4a8, m, n, k, seed):
    w = to_dev_bf16(inputs.weights(n, k, seed=seed))
    a = to_dev_bf16(inputs.activations(m, k, seed=seed + 1, dist="student_t"))
    return a, w4a8.pack_w4_grouped(w)


def _compare(w4a8, a, packed, n, dt):
    m, k = a.shape
    ws = torch.empty(w4a8.workspace_bytes(m, k, n), dtype=torch.uint8, device="cuda")
    ref = w4a8.w4a8_gemm_bf16act(a, *packed, n, out_dtype=dt, workspace=ws)
    out = torch.full((m, n), -7, dtype=dt, device="cuda")
    w4a8.w4a8_gemm_bf16act_noalloc(a, *packed, n, out=out)
    torch.cuda.synchronize()
    view = torch.int16 if dt == torch.bfloat16 else torch.int32
    assert torch.equal(out.view(view), ref.view(view))


@pytest.mark.parametrize("first,second", [
    ((64, 8192, 28672), (24, 14352, 4096)),   # split K both times (partials in the array)
    ((300, 2048, 1024), (8, 4096, 4096)),     # tiled path, then the fused one-kernel path
    ((2048, 512, 28672), (64, 512, 8192)),    # 56 MiB of codes (no room for the partials:
                                              # one pass), then a smaller split call
])
def test_noalloc_equals_fused_with_workspace(w4a8, first, second):
    if first == (2048, 512, 28672):
        assert w4a8.workspace_bytes(2048, 28672, 512) > w4a8.NOALLOC_SCRATCH_BYTES
    for (m, n, k), seed in ((first, 3), (second, 5)):
        print("CASE noalloc", m, n, k, flush=True)
        assert w4a8.workspace_bytes(m, k) <= w4a8.NOALLOC_SCRATCH_BYTES
        a, packed = _case(w4a8, m, n, k, seed)
        for dt in (torch.int32, torch.bfloat16, torch.float32):
            _compare(w4a8, a, packed, n, dt)


def test_noalloc_rejects_workspace_beyond_the_array(w4a8):
    m, n, k = 4096, 64, 32768                  # 128 MiB of activation codes
    print("CASE noalloc too large", m, n, k, flush=True)
    assert w4a8.workspace_bytes(m, k, n) > w4a8.NOALLOC_SCRATCH_BYTES
    a = torch.zeros((m, k), dtype=torch.bfloat16, device="cuda")
    wp = torch.zeros((n * k // 2,), dtype=torch.uint8, device="cuda")
    gs = torch.ones((n * k // 64,), dtype=torch.uint8, device="cuda")
    cs = torch.ones((n,), dtype=torch.float32, device="cuda")
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(w4a8.W4A8Error) as e:
        w4a8.w4a8_gemm_bf16act_noalloc(a, wp, gs, cs, n, out=out)
    assert e.value.status == w4a8.ERR_UNSUPPORTED
