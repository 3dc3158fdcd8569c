"""GPU parity of dual-scale MXFP4 (two online scale levels: a coarse fp32 scale
per 512 K-elements, a fine e8m0 exponent per 32; "vLLM-Omni Online
Quantization complete guide", section "How online quantization works
underneath") through the C ABI, against the CPU oracle:

* codes, fine exponents and coarse scales bit-exact (hard inputs: zero blocks,
  ties, subnormals, -0, outliers), at small shapes and on sampled rows of the
  full-size video-DiT activation and weight;
* dequantize bit-exact;
* the GEMM within the Frobenius gate and the per-element bound on
  power-of-two scaled operands, bit-exact on grid-valued operands (every
  element, ragged multi-tile shapes), into sentinel-guarded strided outputs,
  and on tile-covering samples of the full-size workload;
* qlinear equal to quantize + qgemm bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_quantized_linear_amd as pql
import workloads as wl
from gemm_check import assert_gemm, check_gemm, check_gemm_exact, exact_operand, exact_precondition, tile_sample
from test_gpu_parity import _first_diff, down_bf16, hard_input, up

pytestmark = pytest.mark.gpu

DEV = "cuda"
SCHEME = "mxfp4_dual"


def assert_dual_equal(got: dict, ref: dict, what=""):
    assert np.array_equal(got["codes"], ref["codes"]), f"codes differ {what}: " + _first_diff(got["codes"], ref["codes"])
    assert np.array_equal(got["scales"], ref["scales"]), f"fine exponents differ {what}: " + \
        _first_diff(got["scales"], ref["scales"])
    gc, rc = np.asarray(got["coarse"], np.float32).view(np.uint32), np.asarray(ref["coarse"], np.float32).view(np.uint32)
    assert np.array_equal(gc, rc), f"coarse scales differ {what}: " + _first_diff(gc, rc)


@pytest.mark.parametrize("role", ["activation", "weight"])
@pytest.mark.parametrize("rows,cols", [(1, 512), (37, 1024), (300, 2048), (384, 1536), (5, 5120)])
def test_dual_quantize_bit_exact(role, rows, cols):
    x = hard_input(rows * 11 + cols, rows, cols, 0.02 if role == "weight" else 1.0)
    ref = oracle.quantize(x, SCHEME, role)
    assert pql.kernel_name("quantize", SCHEME, role, rows, 0, cols) == "k_mx4_dual"
    assert_dual_equal(pql.to_numpy(pql.quantize(up(x), SCHEME, role)), ref, f"{role} {rows}x{cols}")


def test_dual_quantize_strided_and_zero():
    wide = hard_input(5, 64, 1536)
    x = up(wide)[:, 512:1536]
    assert_dual_equal(pql.to_numpy(pql.quantize(x, SCHEME)), oracle.quantize(np.ascontiguousarray(wide[:, 512:]), SCHEME))
    z = np.zeros((16, 1024), np.uint16)
    assert_dual_equal(pql.to_numpy(pql.quantize(up(z), SCHEME, "weight")), oracle.quantize(z, SCHEME, "weight"))


def test_dual_dequantize_bit_exact():
    x = hard_input(17, 256, 1024)
    ref_q = oracle.quantize(x, SCHEME, "activation")
    y = pql.dequantize(pql.from_numpy(ref_q, DEV))
    assert np.array_equal(down_bf16(y), oracle.dequantize(ref_q))


@pytest.mark.parametrize("M,N,K", [(1, 256, 512), (77, 384, 1024), (300, 520, 1536), (4300, 4200, 1024)])
def test_dual_qgemm_matches_oracle(M, N, K):
    a = wl.pow2_blocks(wl.small_case(9100 + M, M, K, 1.0), M, 1, 32)
    w = wl.pow2_blocks(wl.small_case(9200 + N, N, K, 0.02), N, 1, 512)
    aq, wq = oracle.quantize(a, SCHEME, "activation"), oracle.quantize(w, SCHEME, "weight")
    assert pql.kernel_name("qgemm", SCHEME, "activation", M, N, K) == "k_gemm_mx4_dual"
    c = pql.qgemm(pql.from_numpy(aq, DEV), pql.from_numpy(wq, DEV))
    assert_gemm(down_bf16(c), aq, wq, f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 128, 512), (300, 520, 1024), (4300, 4200, 512), (129, 4100, 2048)])
def test_dual_exact_every_element(M, N, K):
    a = exact_operand(SCHEME, "activation", M, K, 40 + M)
    w = exact_operand(SCHEME, "weight", N, K, 41 + N)
    exact_precondition(a, w)
    c = pql.qgemm(pql.from_numpy(a, DEV), pql.from_numpy(w, DEV))
    check_gemm_exact(down_bf16(c), oracle.gemm_ref(a, w), f"{M}x{N}x{K}")


@pytest.mark.parametrize("aligned", [True, False])
def test_dual_strided_output_keeps_sentinels(aligned):
    from test_gpu_exact import _check_sentinels, _sentinel_buffer
    M, N, K = 300, 520, 1024
    a, w = exact_operand(SCHEME, "activation", M, K, 3), exact_operand(SCHEME, "weight", N, K, 4)
    col0, ld = (8, N + 40) if aligned else (3, N + 37)
    buf, out = _sentinel_buffer(M, N, 2, col0, ld)
    pql.qgemm(pql.from_numpy(a, DEV), pql.from_numpy(w, DEV), out=out)
    _check_sentinels(buf, M, N, 2, col0, f"ldc={ld}")
    check_gemm_exact(down_bf16(out), oracle.gemm_ref(a, w), f"ldc={ld}")


def test_dual_qlinear_equals_quantize_then_qgemm():
    M, N, K = 300, 384, 1024
    a = up(wl.small_case(5, M, K))
    wq = pql.quantize(up(wl.small_case(6, N, K, 0.02)), SCHEME, "weight")
    y = pql.qlinear(a.reshape(3, 100, K), wq)
    ref = pql.qgemm(pql.quantize(a, SCHEME, "activation"), wq)
    assert torch.equal(y.reshape(M, N).view(torch.int16), ref.view(torch.int16))


def test_dual_rejects_epilogue_and_bad_k():
    x = up(wl.small_case(1, 64, 1024))
    wq = pql.quantize(up(wl.small_case(2, 128, 1024, 0.02)), SCHEME, "weight")
    with pytest.raises(NotImplementedError):
        pql.qlinear(x, wq, alpha=0.5)
    with pytest.raises(ValueError):
        pql.quantize(up(wl.small_case(3, 8, 768)), SCHEME)


def test_full_size_dual_workload():
    w_ = wl.WORKLOADS["mx_video_dit"]
    a_bits, w_bits = wl.activation(w_), wl.weight(w_)
    a_t, w_t = up(a_bits), up(w_bits)
    wq = pql.quantize(w_t, SCHEME, "weight")
    aq = pql.quantize(a_t, SCHEME, "activation")
    y = pql.qlinear(a_t, wq)
    c = pql.qgemm(aq, wq)
    assert torch.equal(y.view(torch.int16), c.view(torch.int16)), "qlinear != quantize + qgemm"
    aq_np, wq_np = pql.to_numpy(aq), pql.to_numpy(wq)
    ra = tile_sample(w_.M, 21, extra=range(w_.M - 24, w_.M))
    rw = tile_sample(w_.N, 22)

    def rows_of(q, rows):
        return dict(q, codes=q["codes"][rows], scales=q["scales"][rows], coarse=q["coarse"][rows], rows=len(rows))
    assert_dual_equal(rows_of(aq_np, ra[::3]), oracle.quantize(np.ascontiguousarray(a_bits[ra[::3]]), SCHEME), "A rows")
    assert_dual_equal(rows_of(wq_np, rw[::3]), oracle.quantize(np.ascontiguousarray(w_bits[rw[::3]]), SCHEME,
                                                               "weight"), "W rows")
    a_rows, w_rows = rows_of(aq_np, ra), rows_of(wq_np, rw)
    c64 = oracle.gemm_ref(a_rows, w_rows)
    t = oracle.gemm_abs_ref(a_rows, w_rows)
    check_gemm(down_bf16(c)[np.ix_(ra, rw)], c64, t, w_.K, "mx_video_dit dual")
