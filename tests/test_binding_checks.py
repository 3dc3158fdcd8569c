"""Binding-level argument checks that need no GPU.

The C ABI sees raw pointers and a row stride only, so the Python binding must
reject, before any launch, outputs of the wrong dtype, shape or stride,
operands in the wrong role, and mismatched devices: otherwise a kernel would
write past a buffer or store bf16 into a float32 tensor.  Every case below
raises ValueError from the binding itself (CPU tensors never reach the
library)."""
import pytest
import torch

import precision_quantized_linear_amd as pql


def _cpu_q(scheme, role, rows, cols, seed):
    """A QTensor with buffers of the right shapes on the CPU (contents irrelevant here)."""
    return pql._alloc_q(scheme, role, rows, cols, "cpu")


@pytest.fixture(scope="module")
def ops():
    return _cpu_q("fp8_row", "activation", 16, 256, 1), _cpu_q("fp8_row", "weight", 32, 256, 2)


@pytest.mark.parametrize("bad", [
    torch.empty((16, 32), dtype=torch.float32),              # wrong dtype
    torch.empty((16, 31), dtype=torch.bfloat16),             # wrong shape
    torch.empty((32, 16), dtype=torch.bfloat16),             # transposed shape
    torch.empty((32, 16), dtype=torch.bfloat16).t(),         # column stride != 1
    torch.empty((16, 64), dtype=torch.bfloat16)[:, ::2],     # strided columns
    torch.empty((512,), dtype=torch.bfloat16),               # 1-D
])
def test_qgemm_rejects_bad_out(ops, bad):
    a, w = ops
    with pytest.raises(ValueError):
        pql.qgemm(a, w, out=bad)


def test_qgemm_rejects_weight_as_activation(ops):
    _, w = ops
    with pytest.raises(ValueError, match="activation"):
        pql.qgemm(w, w)


def test_qgemm_rejects_activation_as_weight(ops):
    a, _ = ops
    with pytest.raises(ValueError, match="weight"):
        pql.qgemm(a, a)


def test_qgemm_rejects_scheme_mismatch(ops):
    a, _ = ops
    w = _cpu_q("fp8_tensor", "weight", 32, 256, 3)
    with pytest.raises(ValueError, match="schemes differ"):
        pql.qgemm(a, w)


def test_qgemm_rejects_k_mismatch(ops):
    a, _ = ops
    w = _cpu_q("fp8_row", "weight", 32, 512, 4)
    with pytest.raises(ValueError, match="K mismatch"):
        pql.qgemm(a, w)


def test_qgemm_w4a16_rejects_quantized_activation(ops):
    a, _ = ops
    w = _cpu_q("w4a16_asym", "weight", 32, 256, 5)
    with pytest.raises(ValueError):
        pql.qgemm(a, w)


def test_qgemm_fp8_rejects_bf16_activation(ops):
    _, w = ops
    with pytest.raises(ValueError, match="quantized activation"):
        pql.qgemm(torch.zeros((16, 256), dtype=torch.bfloat16), w)


def test_cpu_operands_never_reach_the_library(ops):
    a, w = ops
    with pytest.raises(ValueError, match="HIP device"):
        pql.qgemm(a, w, out=torch.empty((16, 32), dtype=torch.bfloat16))


@pytest.mark.parametrize("bad", [
    torch.empty((16, 256), dtype=torch.float16),
    torch.empty((16, 128), dtype=torch.bfloat16),
    torch.empty((256, 16), dtype=torch.bfloat16).t(),
])
def test_dequantize_rejects_bad_out(ops, bad):
    a, _ = ops
    with pytest.raises(ValueError):
        pql.dequantize(a, out=bad)


def test_wide_row_stride_out_is_accepted_until_the_device_check(ops):
    a, w = ops
    wide = torch.empty((16, 48), dtype=torch.bfloat16)[:, 8:40]    # [16, 32] view, row stride 48
    with pytest.raises(ValueError, match="HIP device"):            # shape and strides passed
        pql.qgemm(a, w, out=wide)


def test_from_numpy_needs_a_device():
    import oracle
    import workloads as wl
    q = oracle.quantize(wl.small_case(1, 4, 64), "mxfp8", "activation")
    with pytest.raises(ValueError, match="HIP device"):
        pql.from_numpy(q, "cpu")
