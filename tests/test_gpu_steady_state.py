"""Element-by-element parity of the launch variants that shorter shapes never
reach, through the C ABI, against the oracle:

- the 256 x 256 tiled GEMM (16 wavefronts) in its steady state: shapes with more
  than one round of 256 x 256 tiles (so the launcher keeps them) and 8.5 or 16
  K chunks (every LDS stage and register set reused, the clamped requests past
  the last chunk), ragged M and N, followed by the 128 x 256 tail launch; int32
  accumulators bit-exact, binary32 within 1e-5 relative, bf16 within 1 ulp, for
  the three weight formats;
- every form of the fused quantize + GEMM kernel (vectors per thread, 8 or 16
  wavefronts, widened activations kept in registers or not);
- the binding's own allocations when the call runs on a side stream;
- the debug mode's check for non-finite inputs.

The oracle's accumulators here come from its matmul forms (a binary64 library
matmul of the integer operands, equal to its C loops bit for bit), so full
outputs of these sizes are affordable.
"""
import numpy as np
import pytest
import torch

import oracle
from w4a8_quantized_gemm_quantize_amd import inputs

from gpu_util import assert_bf16_within_ulp, assert_f32_close, bits_of, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4a8():
    from w4a8_quantized_gemm_quantize_amd import binding
    torch.cuda.init()
    return binding


def announce(*what):
    print("CASE", *what, flush=True)


def large_tile_columns(m, n, ncu):
    """The launcher's split of an m > 128 product: output columns [0, 256 c) in
    256 x 256 tiles, the rest in 128 x 256 tiles, c minimising the cost in rounds
    of large tiles (a round of small tiles costs half)."""
    mt, ntb = -(-m // 256), -(-n // 256)

    def rounds(tiles):
        return -(-tiles // ncu)

    best_cols, best = ntb, float(rounds(mt * ntb))
    for cols in range(ntb - 1, -1, -1):
        c = rounds(mt * cols) + 0.5 * rounds(2 * mt * (ntb - cols))
        if c < best - 1e-9:
            best, best_cols = c, cols
    return min(best_cols * 256, n)


STEADY_SHAPES = [
    (4000, 4368, 1088),   # 16 x 16 large tiles (ragged M), 272-column tail, 8.5 chunks
    (2000, 8448, 2048),   # 8 x 32 large tiles (ragged M), 256-column tail, 16 chunks
]


@pytest.mark.parametrize("fmt", ["w4", "lqq", "w8"])
@pytest.mark.parametrize("m,n,k", STEADY_SHAPES)
def test_tiled_256_steady_state(w4a8, m, n, k, fmt):
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    n_large = large_tile_columns(m, n, ncu)
    announce("tiled 256x256 steady state", fmt, m, n, k, "large cols", n_large, "cus", ncu)
    assert 0 < n_large < n, "the shape must reach both the 256 x 256 and the tail launch"
    assert k // 128 >= 8
    w = inputs.weights(n, k, seed=n + k)
    wd = to_dev_bf16(w)
    a_q, a_s = oracle.quantize_act_blockwise(
        inputs.activations(m, k, seed=m, outlier_frac=0.001), k)
    aq_d = torch.from_numpy(a_q).cuda()
    as_d = torch.from_numpy(a_s.reshape(-1)).cuda()
    if fmt == "w4":
        packed = w4a8.pack_w4_grouped(wd)
        fn = w4a8.w4a8_gemm
        acc_ref, y_ref = oracle.w4a8_gemm_matmul(a_q, a_s, *oracle.quantize_w4_grouped(w, 64))
    elif fmt == "lqq":
        packed = w4a8.pack_w4_lqq(wd)
        fn = w4a8.w4a8_gemm_lqq
        acc_ref, y_ref = oracle.w4a8_gemm_lqq_matmul(a_q, a_s, *oracle.quantize_w4_lqq(w, 64))
    else:
        packed = w4a8.pack_w8_channel(wd)
        fn = w4a8.w8a8_gemm
        acc_ref, y_ref = oracle.w8a8_gemm_matmul(a_q, a_s, *oracle.quantize_w8_channel(w))
    acc = fn(aq_d, as_d, *packed, n, out_dtype=torch.int32)
    y32 = fn(aq_d, as_d, *packed, n, out_dtype=torch.float32)
    y16 = fn(aq_d, as_d, *packed, n, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    got = acc.cpu().numpy()
    bad = np.argwhere(got != acc_ref)
    assert bad.size == 0, f"{len(bad)} accumulators differ, first at {bad[:4].tolist()}"
    assert_f32_close(y32.cpu().numpy(), y_ref)
    assert_bf16_within_ulp(bits_of(y16), y_ref)


# ---------------------------------------------------- fused kernel forms --

def fused_form(m, n, k, ncu):
    """The launcher's form of the fused kernel: (vectors per thread, wavefronts,
    widened activations kept in registers, 16-channel tiles per workgroup), or
    None when the shape runs quantize then GEMM (m > 16, activations past 48 KB
    of LDS, or more than 8 vectors per thread)."""
    if m < 1 or m > 16 or k < 128 or m * (k + 16) > 48 * 1024:
        return None

    def need(waves):
        tpr = 64 * waves
        while tpr * m > 64 * waves:
            tpr //= 2
        return -(-(k // 8) // tpr)
    # 8 wavefronts for k > 2048, unless they would need more than 8 vectors per
    # thread, or more than 4 with at most one workgroup per CU
    if k <= 2048 or need(8) > 8 or (need(8) > 4 and n // 16 <= ncu):
        waves = 16
    else:
        waves = 8
    av = 4 if need(waves) <= 4 else 8 if need(waves) <= 8 else None
    if av is None:
        return None
    keep = av == 4 and waves == 16 and n // 16 <= ncu
    # two tiles per workgroup: 4 vectors, 8 wavefronts, more than two
    # workgroups per CU, at least 8192 activations per workgroup
    tiles = 2 if av == 4 and waves == 8 and n // 16 > 2 * ncu and m * k >= 8192 else 1
    return av, waves, keep, tiles


FUSED_FORMS = [
    ((8, 4096, 4096), (4, 16, True, 1)),     # decode: one workgroup per CU
    ((4, 8192, 2048), (4, 16, False, 1)),    # short rows, more workgroups than CUs
    ((16, 64, 2560), (8, 16, False, 1)),     # 8 wavefronts would need 10 vectors
    ((1, 64, 12288), (4, 8, False, 1)),
    ((8, 8192, 4096), (8, 8, False, 1)),     # more workgroups than CUs
    ((1, 512, 28672), (4, 16, True, 1)),     # FFN-down M = 1 row length, few channels
    ((3, 48, 8192), (4, 16, True, 1)),
    ((2, 14352, 4096), (4, 8, False, 2)),    # two tiles per workgroup, the last one alone
    ((2, 4096, 4160), (4, 8, False, 1)),     # 8 wavefronts with a trailing 64-wide chunk
    ((2, 14352, 4160), (4, 8, False, 2)),    # two tiles and a trailing 64-wide chunk
]


@pytest.mark.parametrize("shape,form", FUSED_FORMS)
def test_fused_kernel_forms(w4a8, shape, form):
    m, n, k = shape
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    announce("fused form", m, n, k, form)
    assert fused_form(m, n, k, ncu) == form
    w = inputs.weights(n, k, seed=k + 3)
    a = inputs.activations(m, k, seed=m + 5, dist="student_t")
    ref_w = oracle.quantize_w4_grouped(w, 64)
    packed = w4a8.pack_w4_grouped(to_dev_bf16(w))
    ad = to_dev_bf16(a)
    ws = torch.empty(w4a8.workspace_bytes(m, k), dtype=torch.uint8, device="cuda")
    acc = w4a8.w4a8_gemm_bf16act(ad, *packed, n, out_dtype=torch.int32, workspace=ws)
    torch.cuda.synchronize()
    ws_q, ws_s = [t.clone() for t in w4a8.workspace_views(ws, m, k)]
    y16 = w4a8.w4a8_gemm_bf16act(ad, *packed, n, out_dtype=torch.bfloat16, workspace=ws)
    y32 = w4a8.w4a8_gemm_bf16act(ad, *packed, n, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    a_q, a_s, acc_ref, y_ref = oracle.w4a8_gemm_bf16act(a, *ref_w, 64)
    assert np.array_equal(ws_q.cpu().numpy(), a_q)
    assert np.array_equal(ws_s.cpu().numpy().view(np.uint32), a_s.view(np.uint32))
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert_f32_close(y32.cpu().numpy(), y_ref)
    assert_bf16_within_ulp(bits_of(y16), y_ref)


# ------------------------------------------------- binding on a side stream --

@pytest.mark.parametrize("m,n,k", [(33, 8208, 8448), (8, 4096, 4096), (300, 2048, 4096)])
def test_side_stream_without_workspace(w4a8, m, n, k):
    """The binding creates the workspace (and the output) itself and the call runs
    on a side stream; work allocated and written on the current stream right
    after must not land in memory the call's kernels still use."""
    announce("side stream, binding-made workspace", m, n, k)
    w = inputs.weights(n, k, seed=41)
    a = inputs.activations(m, k, seed=43, outlier_frac=0.001)
    ref_w = oracle.quantize_w4_grouped(w, 64)
    packed = w4a8.pack_w4_grouped(to_dev_bf16(w))
    ad = to_dev_bf16(a)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    need = w4a8.workspace_bytes(m, k, n)
    y = w4a8.w4a8_gemm_bf16act(ad, *packed, n, out_dtype=torch.int32, stream=side)
    # the workspace tensor the binding made is released now; fill fresh blocks
    # of the same size on the current stream while the side stream may still run
    junk = [torch.full((need,), 0x5a, dtype=torch.uint8, device="cuda") for _ in range(4)]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    _, _, acc_ref, _ = oracle.w4a8_gemm_bf16act(a, *ref_w, 64, want_y=False)
    assert np.array_equal(y.cpu().numpy(), acc_ref)
    del junk


# ------------------------------------------------------------- debug mode --

def test_debug_mode_reports_non_finite_inputs(w4a8, monkeypatch):
    announce("debug mode non-finite inputs")
    m, n, k = 4, 64, 256
    w = inputs.weights(n, k, seed=1)
    packed = w4a8.pack_w4_grouped(to_dev_bf16(w))
    a = inputs.activations(m, k, seed=2)
    good = to_dev_bf16(a)
    bad = a.copy()
    bad[2, 17] = 0x7fc0                               # a bf16 NaN
    inf = a.copy()
    inf[0, 3] = 0xff80                                # bf16 -inf
    monkeypatch.setenv("W4A8_DEBUG", "1")
    w4a8.quantize_act_blockwise(good, 32)             # finite: runs
    w4a8.w4a8_gemm_bf16act(good, *packed, n)
    torch.cuda.synchronize()
    for x in (bad, inf):
        with pytest.raises(w4a8.W4A8Error) as e:
            w4a8.quantize_act_blockwise(to_dev_bf16(x), 32)
        assert e.value.status == w4a8.ERR_NONFINITE
        with pytest.raises(w4a8.W4A8Error) as e:
            w4a8.w4a8_gemm_bf16act(to_dev_bf16(x), *packed, n)
        assert e.value.status == w4a8.ERR_NONFINITE
    wbad = w.copy()
    wbad[5, 5] = 0x7f80                               # +inf weight
    with pytest.raises(w4a8.W4A8Error) as e:
        w4a8.pack_w4_grouped(to_dev_bf16(wbad))
    assert e.value.status == w4a8.ERR_NONFINITE
    monkeypatch.delenv("W4A8_DEBUG")
    w4a8.quantize_act_blockwise(to_dev_bf16(bad), 32)  # outside debug mode: no check
    torch.cuda.synchronize()
