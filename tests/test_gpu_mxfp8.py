"""FP8 tier on the GPU: the MXFP8 quantizer bit for bit, and the scaled-FP8 MFMA GEMM, against the oracle.

Each case logs its name and shape before touching the GPU."""
import numpy as np
import pytest

import oracle as O
from synth import bf16_normal_bits, f32_to_bf16_bits
from tests.gpu_util import dev_bf16, log, rel_l2

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
dt = pytest.importorskip("diffusion_transformer_text_amd")


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3 byte -> value (bias 7, 3 mantissa bits, exponent field 0 = subnormal, S.1111.111 = NaN)."""
    c = codes.astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def unpack_scales(words: np.ndarray, rows: int, K: int, ld: int) -> np.ndarray:
    """Scale words -> biased exponents [rows, K / 32]: word (2g + h) * ld + r, byte q = block 8g + 2q + h."""
    b = words.view(np.uint8).reshape(K // 256, 2, ld, 4)[:, :, :rows, :]        # [g, h, r, q]
    return b.transpose(2, 0, 3, 1).reshape(rows, K // 32).astype(np.int64)     # block = 8g + 2q + h


def blocky_bf16(rng, rows, K, std=1.0, spread=8):
    """bf16 bits of normal values whose 32-element blocks carry scales 2^[-spread, spread]: every block
    gets its own E8M0 exponent, so a scale applied to the wrong block shows."""
    x = rng.standard_normal((rows, K // 32, 32)) * std
    x *= np.ldexp(1.0, rng.integers(-spread, spread + 1, (rows, K // 32)))[..., None]
    return f32_to_bf16_bits(x.reshape(rows, K).astype(np.float32))


def quantize(bits, ld=None):
    rows, K = bits.shape
    ld = rows if ld is None else ld
    codes = torch.empty((rows, K), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((K // 128 * ld,), dtype=torch.int32, device="cuda")
    dt.moss_mx_quantize(dev_bf16(bits, torch), codes, scales, ld)
    return codes, scales


@pytest.mark.parametrize("rows,K", [(1, 256), (300, 512), (1000, 3072)])
def test_mx_quantize_matches_oracle_bitwise(rows, K):
    log(f"mx_quantize rows={rows} K={K}")
    rng = np.random.default_rng(rows + K)
    bits = blocky_bf16(rng, rows, K)
    # special blocks: all zero, tiny (bf16 subnormal amax), huge, exact E4M3 ties and the saturation edge
    x = O.from_bf16_bits(bits)
    if rows > 4:
        x[1, :32] = 0.0
        x[2, 32:64] = np.ldexp(rng.standard_normal(32), -130)
        x[3, 64:96] = np.ldexp(rng.standard_normal(32), 100)
        tie = np.ldexp(1.0, 8) * np.array([1.0 + 1 / 16, 1.0 + 3 / 16, 1.75 + 1 / 16, 1.0 + 15 / 16] * 8)
        x[4, :32] = tie * np.where(np.arange(32) % 2, 1.0, -1.0)     # amax 2^8 * 1.9375: exponent 0
        x[4, 31] = np.ldexp(1.75, 8)
        bits = f32_to_bf16_bits(x.astype(np.float32))
        x = O.from_bf16_bits(bits)
    ld = (rows + 255) // 256 * 256
    codes, scales = quantize(bits, ld)
    torch.cuda.synchronize()
    q_ref, ex_ref = O.mx_quantize(x)
    got_q = e4m3_decode(codes.cpu().numpy())
    got_s = unpack_scales(scales.cpu().numpy(), rows, K, ld)
    assert not np.isnan(got_q).any()
    np.testing.assert_array_equal(got_s, ex_ref + 127)
    np.testing.assert_array_equal(got_q, q_ref)


@pytest.mark.parametrize("M,N,K", [(1, 256, 256), (300, 256, 512), (1000, 768, 1280), (8704, 3072, 8192),
                                   (8704, 16384, 3072)])
def test_gemm_mxfp8_vs_oracle(M, N, K):
    """The GEMM of the quantizer's output (pinned bit for bit above) against the fp64 product of the
    oracle's MXFP8 values. The scaled FP8 MFMA does not sum a k-tile's 64 products in fp32: measured,
    its result deviates by up to 2^-15.7 of sum |a w| (relative L2 about 1.4e-5 whatever K), where an
    fp32 sum would stay near 1e-7. The bound: |error| <= 2^-14 sum_k |a_k w_k| per element."""
    log(f"gemm_mxfp8 M={M} N={N} K={K}")
    rng = np.random.default_rng(M * 7 + N + K)
    A = blocky_bf16(rng, M, K, 1.0, 4)
    W = blocky_bf16(rng, N, K, 0.02, 4)
    lds_a = (M + 255) // 256 * 256
    qa, sa = quantize(A, lds_a)
    qw, sw = quantize(W, N)
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    dt.moss_gemm_mxfp8(qa, sa, lds_a, qw, sw, N, out)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([rng.integers(0, M, 96), [0, M - 1]]))
    a = O.mx_dequantize(O.from_bf16_bits(A[rows]))
    w = O.mx_dequantize(O.from_bf16_bits(W))
    ref = a @ w.T
    bound = np.ldexp(np.abs(a) @ np.abs(w).T, -14)
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    err = rel_l2(got[rows], ref)
    worst = float(np.max(np.abs(got[rows] - ref) / bound))
    log(f"  rel_l2 {err:.3e}, worst error / bound {worst:.3f}")
    assert worst <= 1.0
    assert err < 5e-5


def test_gemm_mxfp8_small_integers_bitwise():
    """Integers of magnitude <= 8 in blocks whose amax is 8 quantize exactly (scale 2^-5, codes k * 32
    <= 256) and their fp32 sums are exact, so the GEMM must match bit for bit."""
    M, N, K = 520, 512, 1024
    log(f"gemm_mxfp8 int M={M} N={N} K={K}")
    rng = np.random.default_rng(3)

    def ints(rows):
        v = rng.integers(-8, 9, (rows, K // 32, 32)).astype(np.float64)
        v[:, :, 0] = 8.0                                    # amax 8: scale exponent 3 - 8 = -5
        return f32_to_bf16_bits(v.reshape(rows, K).astype(np.float32)), v.reshape(rows, K)

    A, av = ints(M)
    W, wv = ints(N)
    lds_a = (M + 255) // 256 * 256
    qa, sa = quantize(A, lds_a)
    qw, sw = quantize(W, N)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    dt.moss_gemm_mxfp8(qa, sa, lds_a, qw, sw, N, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), av @ wv.T)


def test_gemm_mxfp8_rejects_bad_shapes():
    log("gemm_mxfp8 invalid shapes")
    qa = torch.zeros((256, 256), dtype=torch.uint8, device="cuda")
    sa = torch.zeros((2 * 256,), dtype=torch.int32, device="cuda")
    qw = torch.zeros((128, 256), dtype=torch.uint8, device="cuda")
    sw = torch.zeros((2 * 128,), dtype=torch.int32, device="cuda")
    out = torch.empty((256, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(dt.MossError):
        dt.moss_gemm_mxfp8(qa, sa, 256, qw, sw, 128, out)      # N % 256 != 0
    x = torch.zeros((4, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dt.MossError):
        dt.moss_mx_quantize(x, torch.empty((4, 96), dtype=torch.uint8, device="cuda"),
                            torch.zeros((64,), dtype=torch.int32, device="cuda"))   # K % 256 != 0
