"""8-bit floating-point operands on the GPU against oracle.fp8: the
per-tensor quantizer bit for bit (codes and inverse scale), the fp8
product on the oracle's codes within the fp32 tolerance (exact products,
fp32 accumulation), and the quantize + product chain on fp32 originals
within the closed-form error bound of the formats."""
import numpy as np
import pytest
import torch

from oracle import fp8 as ofp8
from bwd_rmsnorm_qkv_amd import qblk
from bwd_rmsnorm_qkv_amd.runtime import byte_buffer, dev, empty
from gpu_util import FP32_TOL, announce, check, need_gpu

pytestmark = pytest.mark.gpu

FMTS = ["e4m3", "e5m2"]


def _quantize_gpu(x, fmt):
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    inv = empty(1)
    scratch = byte_buffer(qblk.fp8_quantize_workspace_size(rows, cols))
    qblk.fp8_quantize(rows, cols, dev(x), cols, fmt == "e5m2", q, cols, inv, scratch)
    torch.cuda.synchronize()
    return q, inv


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape,sigma", [((64, 256), 1.0), ((77, 130), 0.02), ((512, 2560), 3.0),
                                         ((3, 5), 1e-3), ((1024, 1408), 0.5)])
def test_fp8_quantize_bit_exact(fmt, shape, sigma):
    """Codes and 1/s bit for bit against the oracle (both take the scale and
    the rounding decision in fp32); 130 and 5 columns run the scalar path,
    the others the 4-wide one; values span subnormals to FMAX."""
    need_gpu()
    announce(f"fp8 quantize {fmt} {shape} sigma={sigma}")
    rng = np.random.default_rng(shape[0] * 7 + shape[1])
    x = (rng.standard_normal(shape) * sigma).astype(np.float32)
    x.flat[::97] *= 1e-4  # small values: subnormal codes
    q, inv = _quantize_gpu(x, fmt)
    ref_q, ref_inv = ofp8.quantize(x, fmt)
    got = q.cpu().numpy()
    assert np.array_equal(got, ref_q), f"{np.count_nonzero(got != ref_q)} codes differ"
    assert np.float32(inv.item()).view(np.uint32) == np.float32(ref_inv).view(np.uint32)


@pytest.mark.parametrize("fmt", FMTS)
def test_fp8_quantize_zero_and_nan(fmt):
    """An all-zero tensor: zero codes and 1/s = 1. A NaN element stays a NaN
    code; the rest of the tensor quantizes as without it."""
    need_gpu()
    announce(f"fp8 quantize zeros / NaN {fmt}")
    q, inv = _quantize_gpu(np.zeros((8, 64), np.float32), fmt)
    assert not q.any().item() and inv.item() == 1.0
    rng = np.random.default_rng(5)
    x = rng.standard_normal((16, 64)).astype(np.float32)
    ref_q, ref_inv = ofp8.quantize(x, fmt)
    x[3, 7] = np.nan
    q, inv = _quantize_gpu(x, fmt)
    got = q.cpu().numpy()
    assert np.isnan(ofp8.decode(got[3, 7], fmt))
    mask = np.ones(x.shape, bool)
    mask[3, 7] = False
    assert np.array_equal(got[mask], ref_q[mask]) and inv.item() == ref_inv


GEMM_SHAPES = [
    (64, 64, 128),       # one tile, one K tile
    (77, 200, 384),      # ragged M and N
    (256, 384, 1024),    # several tiles
    (64, 96, 8192),      # few tiles, long K: split K
    (512, 6144, 2560),   # the Qwen3-4B QKV projection
    (512, 2560, 9728),   # the down projection
]


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e5m2")])
@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_fp8_matches_oracle(fa, fb, M, N, K):
    """The product of the oracle's codes: the fp8 products are exact in
    fp32, so only fp32 accumulation order separates the two sides."""
    need_gpu()
    if (fa, fb) != ("e4m3", "e4m3") and K > 2560:
        pytest.skip("format combinations at the small shapes")
    announce(f"gemm fp8 {fa} x {fb} {M}x{N}x{K}")
    rng = np.random.default_rng(M + N + K)
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    qa, ia = ofp8.quantize(a, fa)
    qb, ib = ofp8.quantize(b, fb)
    A = torch.from_numpy(qa).cuda()
    B = torch.from_numpy(qb).cuda()
    IA = dev(np.array([ia], np.float32))
    IB = dev(np.array([ib], np.float32))
    Cm = empty((M, N))
    ws = qblk.gemm_fp8_workspace_size(M, N, K)
    scratch = byte_buffer(ws) if ws else None
    qblk.gemm_fp8(M, N, K, A, K, fa == "e5m2", B, K, fb == "e5m2", IA, IB, Cm, N, scratch=scratch)
    ref = ofp8.gemm_nt(qa, fa, ia, qb, fb, ib)
    check(f"C fp8 {fa}x{fb}", Cm, ref, FP32_TOL)
    # accumulate: C += the same product
    qblk.gemm_fp8(M, N, K, A, K, fa == "e5m2", B, K, fb == "e5m2", IA, IB, Cm, N, accumulate=1, scratch=scratch)
    check(f"2C fp8 {fa}x{fb}", Cm, 2 * ref, FP32_TOL)


@pytest.mark.parametrize("fmt", FMTS)
def test_fp8_chain_within_format_bound(fmt):
    """GPU quantizer + GPU product on fp32 originals against the exact
    product: every element within the oracle pin's closed-form bound
    (both operands' rounding, their subnormal terms) plus fp32 accumulation."""
    need_gpu()
    M, N, K = 256, 512, 2560
    announce(f"fp8 chain {fmt} {M}x{N}x{K}")
    rng = np.random.default_rng(9)
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    qa, ia = _quantize_gpu(a, fmt)
    qb, ib = _quantize_gpu(b, fmt)
    Cm = empty((M, N))
    qblk.gemm_fp8(M, N, K, qa, K, fmt == "e5m2", qb, K, fmt == "e5m2", ia, ib, Cm, N)
    got = Cm.cpu().numpy().astype(np.float64)
    exact = a.astype(np.float64) @ b.astype(np.float64).T
    _, m, bias, _ = ofp8.FORMATS[fmt]
    u = 2.0 ** -(m + 1)
    sub_a = 2.0 ** (1 - bias - m) / 2 * ia.item()
    sub_b = 2.0 ** (1 - bias - m) / 2 * ib.item()
    absprod = np.abs(a).astype(np.float64) @ np.abs(b).astype(np.float64).T
    bound = absprod * (2 * u + u * u) * 1.001 + sub_a * np.abs(b).sum(1)[None, :] * (1 + u) \
        + sub_b * np.abs(a).sum(1)[:, None] * (1 + u) + K * sub_a * sub_b + absprod * K * 2.0 ** -23
    err = np.abs(got - exact)
    assert np.all(err <= bound), float(np.max(err / bound))
    rel = float(np.max(err) / np.max(np.abs(exact)))
    announce(f"  max|err|/max|ref| = {rel:.3e} (u = {u})")


def test_gemm_fp8_refuses_bad_shapes():
    """K not a multiple of 128 and misaligned strides are refused on the
    host before any device work."""
    need_gpu()
    A = torch.zeros((64, 256), dtype=torch.uint8, device="cuda")
    Cm = empty((64, 64))
    with pytest.raises(qblk.QblkError):
        qblk.gemm_fp8(64, 64, 200, A, 256, 0, A, 256, 0, None, None, Cm, 64)
    with pytest.raises(qblk.QblkError):
        qblk.gemm_fp8(64, 64, 128, A, 136, 0, A, 256, 0, None, None, Cm, 64)
