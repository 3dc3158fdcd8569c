"""pql_qlinear_noalloc through the C ABI: the same output as pql_qlinear_ex (same
kernels, workspace replaced by the library's static device buffer), bit for bit,
on two calls in a row on one device, the second with a smaller activation, for
every scheme; and the size limit of that buffer rejected before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import precision_quantized_linear_amd as pql
import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda"


def up(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def _noalloc(scheme, x, wq, out, alpha=1.0, bias=None, act_scales=None):
    L = pql.lib()
    M, K = x.shape
    st = L.pql_qlinear_noalloc(pql.SCHEMES[scheme], x.data_ptr(), M, K, x.stride(0),
                               None if act_scales is None else act_scales.data_ptr(),
                               wq.codes.data_ptr(), wq.scales.data_ptr(),
                               None if wq.zeros is None else wq.zeros.data_ptr(), wq.rows, ctypes.c_float(alpha),
                               None if bias is None else bias.data_ptr(), out.data_ptr(), out.stride(0),
                               torch.cuda.current_stream().cuda_stream)
    return st


def _ex(scheme, x, wq, out, alpha=1.0, bias=None, act_scales=None):
    M, K = x.shape
    ws_b = pql.workspace_size("qlinear", scheme, "activation", M, wq.rows, K)
    ws = torch.empty(max(ws_b, 1), dtype=torch.uint8, device=DEV)
    L = pql.lib()
    st = L.pql_qlinear_ex(pql.SCHEMES[scheme], x.data_ptr(), M, K, x.stride(0),
                          None if act_scales is None else act_scales.data_ptr(),
                          wq.codes.data_ptr(), wq.scales.data_ptr(), None if wq.zeros is None else wq.zeros.data_ptr(),
                          wq.rows, ctypes.c_float(alpha), None if bias is None else bias.data_ptr(),
                          out.data_ptr(), out.stride(0), ws.data_ptr(), ws_b, torch.cuda.current_stream().cuda_stream)
    return st


@pytest.mark.parametrize("scheme", ["fp8_tensor", "fp8_row", "fp8_block128", "mxfp8", "mxfp4", "int8_row",
                                    "w4a16_asym"])
def test_noalloc_matches_qlinear_ex_twice(scheme):
    N, K = 640, 1152
    wq = pql.quantize(up(wl.small_case(51, N, K, 0.02)), scheme, "weight")
    epi = scheme in ("fp8_tensor", "fp8_row", "fp8_block128", "int8_row")
    bias = up(wl.small_case(52, 1, N, 0.5)[0]) if epi else None
    alpha = 0.75 if epi else 1.0
    for call, M in enumerate((1000, 77)):      # the second call is smaller
        x = up(wl.small_case(53 + call, M, K))
        got = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        want = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        assert _noalloc(scheme, x, wq, got, alpha, bias) == 0, pql.lib().pql_last_error()
        assert _ex(scheme, x, wq, want, alpha, bias) == 0, pql.lib().pql_last_error()
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{scheme} call {call} (M={M})"


@pytest.mark.parametrize("scheme", ["fp8_row", "fp8_block128", "int8_row", "mxfp8"])
def test_noalloc_few_tokens_twice(scheme):
    """1-16 tokens run the fused kernel for the FP8 / int8 schemes (no scratch needed) and
    the quantize + GEMM pair for MX: both entry points agree on two calls in a row, the
    second smaller, after a large call has left the static buffer dirty."""
    N, K = 512, 1024
    wq = pql.quantize(up(wl.small_case(81, N, K, 0.02)), scheme, "weight")
    for call, M in enumerate((600, 16, 3)):
        x = up(wl.small_case(82 + call, M, K))
        got = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        want = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        assert _noalloc(scheme, x, wq, got) == 0, pql.lib().pql_last_error()
        assert _ex(scheme, x, wq, want) == 0, pql.lib().pql_last_error()
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{scheme} call {call} (M={M})"


def test_noalloc_static_scales_and_binding():
    N, K, M = 256, 512, 300
    wq = pql.quantize(up(wl.small_case(61, N, K, 0.02)), "fp8_block128", "weight")
    x = up(wl.small_case(62, M, K))
    sa = pql.quantize(x, "fp8_block128", "activation").scales.clone()
    got = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    pql.qlinear_noalloc(x, wq, got, act_scales=sa)
    want = pql.qlinear(x, wq, act_scales=sa)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))


def test_noalloc_rejects_activation_beyond_the_buffer():
    cap = pql.noalloc_scratch_bytes()
    assert cap == 64 << 20
    K, N = 4096, 128
    M = cap // K + 1                      # fp8 codes alone exceed the buffer
    x = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    wq = pql.quantize(up(wl.small_case(71, N, K, 0.02)), "fp8_row", "weight")
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    assert _noalloc("fp8_row", x, wq, out) == pql.PQL_ERR_WORKSPACE
    assert "static scratch" in pql.lib().pql_last_error().decode()
