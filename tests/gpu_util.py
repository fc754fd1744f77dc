"""Helpers shared by the GPU parity tests: moving seeded inputs to the device and
comparing device results with the CPU oracle."""
import numpy as np
import torch


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> torch.bfloat16 CUDA tensor with identical bits."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def bits_of(t: torch.Tensor) -> np.ndarray:
    """bfloat16 tensor -> uint16 bit patterns on the host."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (8 significant bits)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return 2.0 ** (e - 7)


def assert_f32_close(got: np.ndarray, ref: np.ndarray, rtol=1e-5):
    """Elementwise |got - ref| <= rtol * |ref|; exact zero where ref is zero."""
    got = got.astype(np.float64)
    zero = ref == 0
    assert (got[zero] == 0).all(), "non-zero output where the oracle is exactly zero"
    rel = np.abs(got[~zero] - ref[~zero]) / np.abs(ref[~zero])
    assert rel.size == 0 or rel.max() <= rtol, f"max relative error {rel.max():.3e}"


def assert_bf16_within_ulp(got_bits: np.ndarray, ref: np.ndarray):
    """bf16 output within 1 bf16 ulp of the fp64 reference."""
    got = bf16_bits_to_f64(got_bits)
    err = np.abs(got - ref)
    assert (err <= bf16_ulp(ref)).all(), f"max error {(err / bf16_ulp(ref)).max():.3f} ulp"
