"""GPU parity: the HIP path through the C ABI against the CPU oracle.

* Quantized codes, scales and zero-points must match the oracle bit for bit.
* Dequantized bf16 must match bit for bit.
* GEMM outputs, given identical quantized inputs, must satisfy
  ||C_gpu - C_oracle||_F / ||C_oracle||_F <= 1e-2 (the tolerance the
  quantized-linear target states) and, element by element, the bound of
  tests/gemm_check.py (bf16 output rounding plus the worst case of fp32
  accumulation); the oracle is the exact float64 product.  The operands are
  scaled by powers of two per row / K-block / weight block so that a scale
  taken from a neighbouring block is off by at least 2x.
Small cases span several 256x256 tiles with ragged M / N tails; the full-size
workloads (the shapes the benchmark times) are checked on sampled rows and
columns covering every 256 x 256 output tile, which the oracle computes one
by one.  tests/test_gpu_exact.py adds bit-exact GEMM checks of every element.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_quantized_linear_amd as pql
import workloads as wl
from gemm_check import assert_gemm, check_gemm, tile_sample, w4a16_terms
from oracle import formats as F

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 1e-2
FP_SCHEMES = ("fp8_tensor", "fp8_row", "fp8_block128", "mxfp8", "mxfp4")
MX_CHUNK = {"mxfp8": 4, "mxfp4": 8}   # exponent bytes per packed chunk (128 bytes of codes)


def up(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def down_bf16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_q_equal(gpu: dict, ref: dict, what=""):
    assert np.array_equal(gpu["codes"], ref["codes"]), f"codes differ {what}: " + _first_diff(gpu["codes"], ref["codes"])
    gs, rs = np.asarray(gpu["scales"]), np.asarray(ref["scales"])
    if gs.dtype == np.float32:
        gs, rs = gs.view(np.uint32), rs.astype(np.float32).view(np.uint32)
    assert np.array_equal(gs.reshape(rs.shape), rs), f"scales differ {what}: " + _first_diff(gs.reshape(rs.shape), rs)
    if ref["zeros"] is not None:
        assert np.array_equal(gpu["zeros"], ref["zeros"]), f"zeros differ {what}"


def _first_diff(a, b):
    idx = np.argwhere(a != b)
    if len(idx) == 0:
        return "shapes " + str(a.shape) + " vs " + str(b.shape)
    i = tuple(idx[0])
    return f"{len(idx)} entries, first at {i}: gpu {a[i]!r} oracle {b[i]!r}"


def hard_input(seed, rows, cols, std=1.0):
    """Normal data plus the cases the casts must get right: zero rows / groups, exact
    ties after scaling, tiny and subnormal values, negative zeros, one huge outlier."""
    x = wl.bf16_bits_to_f32(wl.small_case(seed, rows, cols, std)).copy()
    rng = np.random.default_rng(seed + 1)
    if rows > 2:
        x[1, :] = 0.0
    x[0, : min(cols, 128)] = np.float32(0.0)
    x[0, 0] = 448.0 * std
    x[0, 1] = 0.53125 * std
    x[0, 2] = 0.59375 * std
    if rows > 3:
        x[2, 32:64] = np.float32(1e-39)          # bf16 subnormal range
        x[3, 5] = np.float32(3.0e38)
    idx = rng.integers(0, rows * cols, 50)
    x.reshape(-1)[idx] *= np.float32(7.5)
    bits = wl.f32_to_bf16_bits(x)
    bits.reshape(-1)[rng.integers(0, rows * cols, 20)] = 0x8000   # -0
    return bits


# ----------------------------------------------------------------- quantize
QUANT_CASES = []
for scheme in FP_SCHEMES + ("w4a16_asym", "w4a16_sym"):
    for role in ("activation", "weight"):
        if scheme.startswith("w4a16") and role == "activation":
            continue
        for rows, cols in ((1, 128), (37, 384), (300, 1152), (384, 640)):
            if scheme == "fp8_block128" and role == "weight" and rows % 128:
                continue
            QUANT_CASES.append((scheme, role, rows, cols))


@pytest.mark.parametrize("scheme,role,rows,cols", QUANT_CASES)
def test_quantize_bit_exact(scheme, role, rows, cols):
    x = hard_input(rows * 7 + cols, rows, cols, 0.02 if role == "weight" else 1.0)
    ref = oracle.quantize(x, scheme, role)
    q = pql.quantize(up(x), scheme, role)
    got = pql.to_numpy(q)
    assert_q_equal(got, ref, f"{scheme}/{role} {rows}x{cols}")
    if scheme in MX_CHUNK:   # the packed device layout itself, pad bytes included
        assert np.array_equal(got["scales_packed"], F.pack_mx_scales(ref["scales"], MX_CHUNK[scheme]))
    if scheme.startswith("w4a16"):   # device layout: group-major [cols / 128, rows]
        assert tuple(q.scales.shape) == (cols // 128, rows) and tuple(q.zeros.shape) == (cols // 128, rows)
        assert np.array_equal(q.scales.view(torch.int16).cpu().numpy().view(np.uint16), ref["scales"].T)
        assert np.array_equal(q.zeros.cpu().numpy(), ref["zeros"].T)


REPACK_CASES = [("mxfp8", "activation", 37, 384), ("mxfp8", "weight", 5, 96), ("mxfp4", "weight", 300, 1152),
                ("mxfp4", "activation", 1, 64), ("w4a16_asym", "weight", 300, 1152), ("w4a16_sym", "weight", 7, 128),
                ("w4a16_asym", "weight", 33, 4096), ("fp8_block128", "activation", 9, 256),
                ("fp8_block128", "weight", 128, 384), ("fp8_row", "weight", 3, 64), ("int8_row", "activation", 6, 640),
                ("mxfp4_dual", "activation", 37, 1024), ("mxfp4_dual", "weight", 300, 2048)]


def _bytes(t):
    return t.contiguous().view(torch.uint8).cpu().numpy().reshape(-1)


@pytest.mark.parametrize("scheme,role,rows,cols", REPACK_CASES)
def test_repack_canonical_bytes_on_device(scheme, role, rows, cols):
    """The device repack (pql_repack) turns the packed scales of a GPU quantization into
    the canonical layout bit for bit against the oracle, and back into the same packed
    bytes (MX pad bytes included); no host-side permutation is involved."""
    x = hard_input(rows * 3 + cols, rows, cols, 0.02 if role == "weight" else 1.0)
    ref = oracle.quantize(x, scheme, role)                       # canonical by definition
    q = pql.quantize(up(x), scheme, role)                       # packed device layout
    codes, scales, zeros = pql.to_canonical(q)
    assert np.array_equal(_bytes(codes), np.ascontiguousarray(ref["codes"]).view(np.uint8).reshape(-1))
    want = np.ascontiguousarray(ref["scales"]).view(np.uint8).reshape(-1)
    got = _bytes(scales)
    if scheme == "mxfp4_dual":   # fine exponents, then the coarse scales from the next 256-byte boundary
        off = -(-want.size // 256) * 256
        assert np.array_equal(got[off:], np.ascontiguousarray(ref["coarse"], np.float32).view(np.uint8).reshape(-1))
        got = got[:want.size]
    assert np.array_equal(got, want)
    if ref["zeros"] is not None:
        assert np.array_equal(_bytes(zeros), np.ascontiguousarray(ref["zeros"]).view(np.uint8).reshape(-1))
    back = pql.from_canonical(scheme, role, rows, cols, codes, scales, zeros)
    b, p = _bytes(back.scales), _bytes(q.scales)
    if scheme == "mxfp4_dual":   # the bytes between the two levels are padding, not part of either
        assert np.array_equal(b[:want.size], p[:want.size]) and np.array_equal(b[off:], p[off:])
    else:
        assert np.array_equal(b, p)
    if q.zeros is not None:
        assert np.array_equal(_bytes(back.zeros), _bytes(q.zeros))


@pytest.mark.parametrize("M,N,K", [(257, 388, 384), (1000, 260, 640), (512, 1024, 256), (130, 390, 384),
                                   (2304, 4100, 256), (300, 4100, 512), (200, 8300, 384), (256, 8448, 256)])
def test_w4a16_gemm_tile_shapes(M, N, K):
    # ragged M and N tails across several 256 x 64 tiles (few tiles) and 256 x 128
    # tiles (2304 x 4100: more than 128 of them), an odd number of K-groups, and
    # N % 4 != 0 (which takes the older tile kernel)
    narrow = -(-M // 256) * -(-N // 128) <= 128
    if N % 4 == 0:
        assert pql.kernel_name("qgemm", "w4a16_asym", "activation", M, N, K) == \
            ("k_w4a16_mm_256x64x64" if narrow else "k_w4a16_mm_256x128x64")
    a = wl.pow2_blocks(wl.small_case(5000 + M, M, K, 1.0), M, 1, 128)
    w = wl.pow2_blocks(wl.small_case(6000 + N, N, K, 0.02), N, 1, 128)
    wq = oracle.quantize(w, "w4a16_asym", "weight")
    c = pql.qgemm(up(a), pql.from_numpy(wq, DEV))
    assert_gemm(down_bf16(c), a, wq, f"{M}x{N}x{K}")


@pytest.mark.parametrize("scheme", FP_SCHEMES + ("w4a16_asym",))
def test_quantize_strided_rows(scheme):
    role = "weight" if scheme == "w4a16_asym" else "activation"
    wide = hard_input(99, 256, 768)
    x = up(wide)[:, 128:128 + 512]
    ref = oracle.quantize(np.ascontiguousarray(wide[:, 128:128 + 512]), scheme, role)
    assert_q_equal(pql.to_numpy(pql.quantize(x, scheme, role)), ref, "strided")


def test_quantize_row_longer_than_register_tile():
    # per-row FP8 keeps up to 8192 elements per row in registers; longer rows take the two-pass path
    x = hard_input(5, 9, 12288)
    assert_q_equal(pql.to_numpy(pql.quantize(up(x), "fp8_row")), oracle.quantize(x, "fp8_row"), "long rows")


@pytest.mark.parametrize("scheme", FP_SCHEMES)
def test_quantize_all_zero(scheme):
    x = np.zeros((128, 256), np.uint16)
    assert_q_equal(pql.to_numpy(pql.quantize(up(x), scheme, "weight")), oracle.quantize(x, scheme, "weight"))


# ----------------------------------------------------------------- dequantize
@pytest.mark.parametrize("scheme,role", [(s, r) for s in FP_SCHEMES for r in ("activation", "weight")]
                         + [("w4a16_asym", "weight"), ("w4a16_sym", "weight")])
def test_dequantize_bit_exact(scheme, role):
    x = hard_input(17, 256, 640, 0.02 if role == "weight" else 1.0)
    ref_q = oracle.quantize(x, scheme, role)
    y = pql.dequantize(pql.from_numpy(ref_q, DEV))
    assert np.array_equal(down_bf16(y), oracle.dequantize(ref_q))


# ----------------------------------------------------------------- GEMM, small shapes
GEMM_SHAPES = [(1, 256, 128), (77, 384, 256), (256, 256, 640), (300, 640, 1152), (513, 128, 384)]


def _gemm_operands(scheme, M, N, K, seed):
    """Seeded operands, scaled by powers of two per row and 32-block (activation) and
    per 128 x 128 block (weight), quantized by the oracle."""
    a = wl.pow2_blocks(wl.small_case(seed + M, M, K, 1.0), seed, 1, 32)
    w = wl.pow2_blocks(wl.small_case(seed + 1 + N, N, K, 0.02), seed + 1, 128 if scheme == "fp8_block128" else 1, 128)
    return oracle.quantize(a, scheme, "activation"), oracle.quantize(w, scheme, "weight")


@pytest.mark.parametrize("scheme", FP_SCHEMES)
@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_qgemm_matches_oracle(scheme, M, N, K):
    aq, wq = _gemm_operands(scheme, M, N, K, 1000)
    c = pql.qgemm(pql.from_numpy(aq, DEV), pql.from_numpy(wq, DEV))
    assert_gemm(down_bf16(c), aq, wq, f"{scheme} {M}x{N}x{K}")


# More output tiles than the 256 persistent workgroups, so some workgroups walk
# two tiles through one load stream (the next tile's first K regions are
# fetched while the current one finishes); ragged M and N tails included.  K is
# a multiple of 256 so MXFP4 runs its region-pipelined kernel too.
@pytest.mark.parametrize("scheme", FP_SCHEMES)
def test_qgemm_multi_tile_workgroups(scheme):
    M, N, K = 4300, 4200 if scheme != "fp8_block128" else 4224, 512
    aq, wq = _gemm_operands(scheme, M, N, K, 7100)
    c = pql.qgemm(pql.from_numpy(aq, DEV), pql.from_numpy(wq, DEV))
    assert_gemm(down_bf16(c), aq, wq, f"{scheme} {M}x{N}x{K}")


# The block-128 GEMM's two kernels: 256 x 128 tiles on 4 waves (here 272 tiles,
# so some workgroups walk two), and 256 x 256 tiles on 8 waves once those fill
# a round of the CUs (here 289, with a ragged M tail and a last tile column
# half past N, whose waves take the last weight-scale block).
@pytest.mark.parametrize("M,N,K,kernel", [(4300, 2048, 640, "k_gemm_block"), (4300, 4224, 384, "k_gemm_block256"),
                                          (4096, 4096, 128, "k_gemm_block256")])
def test_block128_kernels(M, N, K, kernel):
    assert pql.kernel_name("qgemm", "fp8_block128", "activation", M, N, K) == kernel
    aq, wq = _gemm_operands("fp8_block128", M, N, K, 7300)
    c = pql.qgemm(pql.from_numpy(aq, DEV), pql.from_numpy(wq, DEV))
    assert_gemm(down_bf16(c), aq, wq, f"{M}x{N}x{K}")


@pytest.mark.parametrize("M", [1, 5, 16, 33, 64, 65, 300])
@pytest.mark.parametrize("sym", [False, True])
def test_w4a16_gemm_matches_oracle(M, sym):
    N, K = 384, 1152
    a = wl.pow2_blocks(wl.small_case(3000 + M, M, K, 1.0), M, 1, 128)
    w = wl.pow2_blocks(wl.small_case(4000, N, K, 0.02), 7, 1, 128)
    wq = oracle.quantize(w, "w4a16_sym" if sym else "w4a16_asym", "weight")
    c = pql.qgemm(up(a), pql.from_numpy(wq, DEV))
    assert_gemm(down_bf16(c), a, wq, f"M={M}")


@pytest.mark.parametrize("scheme", FP_SCHEMES + ("w4a16_asym",))
def test_qlinear_equals_quantize_then_qgemm(scheme):
    M, N, K = 300, 384, 640
    a = up(wl.small_case(5, M, K))
    wq = pql.quantize(up(wl.small_case(6, N, K, 0.02)), scheme, "weight")
    y = pql.qlinear(a.reshape(3, 100, K), wq)
    assert y.shape == (3, 100, N)
    if scheme.startswith("w4a16"):
        ref = pql.qgemm(a, wq)
    else:
        ref = pql.qgemm(pql.quantize(a, scheme, "activation"), wq)
    assert torch.equal(y.reshape(M, N).view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("M,N,K", [(4300, 4224, 384), (4096, 4096, 1024)])
def test_block128_qlinear_equals_quantize_then_qgemm(M, N, K):
    """qlinear on shapes that run the 256 x 256 kernel (its own quantize into the
    workspace, then the GEMM) equals quantize + qgemm bit for bit, with and without the
    alpha / bias epilogue."""
    assert pql.kernel_name("qgemm", "fp8_block128", "activation", M, N, K) == "k_gemm_block256"
    a = up(wl.small_case(31, M, K))
    wq = pql.quantize(up(wl.small_case(32, N, K, 0.02)), "fp8_block128", "weight")
    aq = pql.quantize(a, "fp8_block128", "activation")
    assert torch.equal(pql.qlinear(a, wq).view(torch.int16), pql.qgemm(aq, wq).view(torch.int16))
    bias = up(wl.small_case(33, 1, N, 0.5)[0])
    assert torch.equal(pql.qlinear(a, wq, alpha=0.75, bias=bias).view(torch.int16),
                       pql.qgemm(aq, wq, alpha=0.75, bias=bias).view(torch.int16))


def test_schemes_give_different_outputs():
    """The pages' no-silent-fallback check: each scheme is a real, different computation."""
    M, N, K = 256, 256, 512
    a = up(wl.small_case(7, M, K))
    w = up(wl.small_case(8, N, K, 0.02))
    outs = {s: pql.qlinear(a, pql.quantize(w, s, "weight")) for s in FP_SCHEMES + ("w4a16_asym",)}
    keys = list(outs)
    for i in range(len(keys)):
        for j in range(i + 1, len(keys)):
            assert not torch.equal(outs[keys[i]], outs[keys[j]]), (keys[i], keys[j])


# ----------------------------------------------------------------- full-size workloads
def _sample_rows(n, k, seed, extra=()):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(n, min(k, n), replace=False).tolist()) | {0, n - 1} | set(extra)
    return np.array(sorted(r for r in rows if 0 <= r < n))


def _take(q_np: dict, rows: np.ndarray, role: str) -> dict:
    """Rows of a downloaded GPU quantization (canonical layout) as an oracle-style dict."""
    out = dict(q_np)
    out["codes"] = q_np["codes"][rows]
    if q_np["scheme"] == "fp8_tensor":
        out["scales"] = q_np["scales"]
    elif q_np["scheme"] == "fp8_block128" and role == "weight":
        out["scales"] = q_np["scales"][rows // 128]
    else:
        out["scales"] = q_np["scales"][rows]
    if q_np["zeros"] is not None:
        out["zeros"] = q_np["zeros"][rows]
    out["rows"] = len(rows)
    return out


def _check_rows(xbits, q_gpu_np, scheme, role, rows):
    if scheme == "fp8_block128" and role == "weight":
        blocks = np.unique(rows // 128)
        for b in blocks:
            r = np.arange(b * 128, b * 128 + 128)
            ref = oracle.quantize(np.ascontiguousarray(xbits[r]), scheme, role)
            got = dict(_take(q_gpu_np, r, role))
            got["scales"] = q_gpu_np["scales"][b:b + 1]
            assert_q_equal(got, ref, f"block {b}")
        return
    ref = oracle.quantize(np.ascontiguousarray(xbits[rows]), scheme, role)
    assert_q_equal(_take(q_gpu_np, rows, role), ref, "sampled rows")


def _sample_check(c_bits, a_rows, w_rows, K, what, a_bits_rows=None):
    """Per-element check of sampled outputs; a_rows / w_rows are row subsets (for a
    128x128-block weight, its rows with the block scale repeated per row)."""
    if a_bits_rows is not None:       # W4A16: the activation is bf16 itself
        c64 = oracle.gemm_ref(a_bits_rows, w_rows)
        t = oracle.gemm_abs_ref(a_bits_rows, w_rows)
        wr, t_off = w4a16_terms(a_bits_rows, w_rows)
        return check_gemm(c_bits, c64, t, K, what, weight_round=wr, t_acc=t_off)
    c64 = oracle.gemm_ref(a_rows, w_rows)
    t = oracle.gemm_abs_ref(a_rows, w_rows)
    return check_gemm(c_bits, c64, t, K, what)


def _block_weight_rows(wq_np: dict, rw: np.ndarray) -> dict:
    """Rows of a 128x128-block weight as a per-(row, 128-group) scaled operand."""
    w = _take(wq_np, rw, "weight")
    w["scales"] = np.asarray(wq_np["scales"], np.float32)[rw // 128]
    w["role"] = "activation"
    return w


@pytest.mark.parametrize("name,scheme", [("fp8_tensor_small", "fp8_tensor"), ("fp8_row_dit", "fp8_row"),
                                         ("fp8_block_dit", "fp8_block128"), ("mx_video_dit", "mxfp8"),
                                         ("mx_video_dit", "mxfp4")])
def test_full_size_workload(name, scheme):
    w_ = wl.WORKLOADS[name]
    a_bits, w_bits = wl.activation(w_), wl.weight(w_)
    a_t, w_t = up(a_bits), up(w_bits)
    wq = pql.quantize(w_t, scheme, "weight")
    aq = pql.quantize(a_t, scheme, "activation")
    y = pql.qlinear(a_t, wq)
    c = pql.qgemm(aq, wq)
    assert torch.equal(y.view(torch.int16), c.view(torch.int16)), "qlinear != quantize + qgemm"
    aq_np, wq_np = pql.to_numpy(aq), pql.to_numpy(wq)
    if scheme == "fp8_tensor":
        assert_q_equal(aq_np, oracle.quantize(a_bits, scheme, "activation"), "A")
        assert_q_equal(wq_np, oracle.quantize(w_bits, scheme, "weight"), "W")
        assert_gemm(down_bf16(c), aq_np, wq_np, name)
        return
    # every 256 x 256 output tile: its first and last rows and columns plus two random
    # ones each, and the ragged tail rows
    ra = tile_sample(w_.M, 11, extra=range(w_.M - 24, w_.M))
    rw = tile_sample(w_.N, 12)
    _check_rows(a_bits, aq_np, scheme, "activation", ra[::3])
    _check_rows(w_bits, wq_np, scheme, "weight", rw[::3])
    a_rows = _take(aq_np, ra, "activation")
    w_rows = _block_weight_rows(wq_np, rw) if scheme == "fp8_block128" else _take(wq_np, rw, "weight")
    _sample_check(down_bf16(c)[np.ix_(ra, rw)], a_rows, w_rows, w_.K, f"{name}/{scheme}")


@pytest.mark.parametrize("M", [1, 16, 256, 4096])
def test_full_size_w4a16(M):
    w_ = wl.WORKLOADS["w4a16_dit"]
    codes, zeros, scales = wl.int4_weight_parts(w_)
    wq_np = {"scheme": "w4a16_asym", "role": "weight", "rows": w_.N, "cols": w_.K,
             "codes": F.pack_int4(codes), "scales": scales, "zeros": zeros}
    wq = pql.from_numpy(wq_np, DEV)
    a_bits = wl.activation(w_, M)
    c = pql.qlinear(up(a_bits), wq)
    ra = tile_sample(M, 13)
    rw = tile_sample(w_.N, 14, tile=128, per_tile=1)
    w_rows = {k: (v[rw] if isinstance(v, np.ndarray) else v) for k, v in wq_np.items()}
    w_rows["rows"] = len(rw)
    _sample_check(down_bf16(c)[np.ix_(ra, rw)], None, w_rows, w_.K, f"M={M}",
                  a_bits_rows=np.ascontiguousarray(a_bits[ra]))


def test_full_size_int4_weight_quantizer():
    w_ = wl.WORKLOADS["w4a16_dit"]
    w_bits = wl.weight(w_)
    q = pql.to_numpy(pql.quantize(up(w_bits), "w4a16_asym", "weight"))
    rw = _sample_rows(w_.N, 128, 15)
    _check_rows(w_bits, q, "w4a16_asym", "weight", rw)
