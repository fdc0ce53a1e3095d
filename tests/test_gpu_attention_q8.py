"""8-bit attention on the GPU (moss_attention_q8: INT8 Q K^T, FP8 P V) against the oracle's attention_q8.

* The quantizers, bit for bit: INT8 codes of Q (per token and head) and K (per 64-key block and
  head), the E4M3 codes of V (per channel) in the kernel's transposed, permuted V^T layout, and the
  three amax arrays, read back from the workspace.
* The attention: sequences of 1, 70 (a ragged second block) and 200 keys, two samples, and the full
  shape (batch 2, 24 heads, S = 4352 = 256 text + 4096 image tokens; and S = 20480, the 2048^2 length)
  on sampled query rows; bf16 N(0, 1) inputs. The GPU rounds its output to bf16; the oracle's exact
  value is compared after the same rounding. Remaining differences: fp32 vs fp64 score and exp2
  arithmetic (a probability may land on the other side of an E4M3 rounding boundary) and fp32
  accumulation: bound 4e-3 relative L2.
* Special cases: one key and V constant over keys give V exactly (convex weights); a dominant key
  gives its dequantized V row (to the bf16 rounding of the output).
* Independently of the online schedule (the oracle's attention_q8 runs the same blocked softmax with
  the same lazy reference max, so it cannot catch a schedule error both share): the exact fp64 softmax
  attention on the dequantized operands, and a per-element bound that holds for any schedule that
  rounds each probability to E4M3 on the 224 scale against a reference max at most the row max and
  normalises by the sum of the same rounded probabilities (tests/q8_bound.py).

Each case logs its name and shape before touching the GPU."""
import numpy as np
import pytest

import oracle as O
from synth import bf16_normal_bits, f32_to_bf16_bits
from tests.gpu_util import dev_bf16, host_bf16, host_bits, log, rel_l2
from tests.q8_bound import exact_on_quantized

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
dt = pytest.importorskip("diffusion_transformer_text_amd")

TOL = 4e-3


def _run(bits, B, S, H):
    qkv = dev_bf16(bits, torch)
    out = torch.empty((B, S, H * 128), dtype=torch.bfloat16, device="cuda")
    ws = dt.moss_attention_q8(qkv, out, B, S, H)
    torch.cuda.synchronize()
    return host_bf16(out).reshape(B, S, H * 128), ws


def _al(x):
    return (x + 255) // 256 * 256


def test_q8_quantizers_bitwise():
    B, S, H = 2, 70, 2
    log(f"q8 quantizers B={B} S={S} H={H}")
    rng = np.random.default_rng(80)
    bits = bf16_normal_bits(rng, (B, S, 3 * H * 128))
    x = O.from_bf16_bits(bits)
    x[0, 3, :128] = 0.0                                   # an all-zero q row
    bits = f32_to_bf16_bits(x.astype(np.float32))
    x = O.from_bf16_bits(bits)
    _, ws = _run(bits, B, S, H)
    raw = ws.cpu().numpy()
    raw = raw[(-ws.data_ptr()) % 256:]
    M, DM, nblk = B * S, H * 128, (S + 63) // 64
    q8 = raw[:M * DM].view(np.int8).reshape(B, S, DM).astype(np.float64)
    k8 = raw[_al(M * DM):_al(M * DM) + M * DM].view(np.int8).reshape(B, S, DM).astype(np.float64)
    o_vt = 2 * _al(M * DM)
    vt = raw[o_vt:o_vt + B * H * 128 * nblk * 64].reshape(B, H, 128, nblk * 64)
    o_qa = o_vt + _al(B * H * 128 * nblk * 64)
    qa = raw[o_qa:o_qa + M * H * 4].view(np.float32).reshape(B, S, H)
    o_ka = o_qa + _al(M * H * 4)
    ka = raw[o_ka:o_ka + B * H * nblk * 4].view(np.float32).reshape(B, H, nblk)
    o_va = o_ka + _al(B * H * nblk * 4)
    va = raw[o_va:o_va + B * H * 128 * 4].view(np.float32).reshape(B, H, 128)
    # key kk of a block sits at position 32 h + 16 kb + 4 j + i for kk = 32 kb + 8 j + 4 h + i
    kk = np.arange(64)
    pos = 32 * ((kk >> 2) & 1) + 16 * (kk >> 5) + 4 * ((kk >> 3) & 3) + (kk & 3)
    for b in range(B):
        for h in range(H):
            sl = slice(h * 128, (h + 1) * 128)
            qc, qam = O.q8_quantize_q(x[b][:, sl])
            np.testing.assert_array_equal(q8[b][:, sl], qc)
            np.testing.assert_array_equal(qa[b][:, h], qam)
            kc, kam = O.q8_quantize_k(x[b][:, 128 * H + h * 128:128 * H + (h + 1) * 128])
            np.testing.assert_array_equal(k8[b][:, sl], kc)
            np.testing.assert_array_equal(ka[b, h], kam)
            vc, vam = O.fp8_quantize_v(x[b][:, 256 * H + h * 128:256 * H + (h + 1) * 128])
            np.testing.assert_array_equal(va[b, h], vam)
            codes = np.zeros((nblk * 64, 128))
            codes[:S] = vc
            for t in range(nblk):
                got_t = vt[b, h][:, t * 64 + pos]            # [128 dims, 64 keys]
                dec = _e4m3_decode(got_t)
                np.testing.assert_array_equal(dec.T, codes[t * 64:(t + 1) * 64])


def _e4m3_decode(c):
    c = c.astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e, m = (c >> 3) & 0xF, c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    return sign * mag


def _check(bits, B, S, H, rows=None, heads=None):
    got, _ = _run(bits, B, S, H)
    x = O.from_bf16_bits(bits)
    errs = []
    for b in range(B):
        for h in (range(H) if heads is None else heads):
            q = x[b][:, h * 128:(h + 1) * 128]
            k = x[b][:, (H + h) * 128:(H + h + 1) * 128]
            v = x[b][:, (2 * H + h) * 128:(2 * H + h + 1) * 128]
            r = np.arange(S) if rows is None else rows
            ref = O.bf16_round(O.attention_q8(q[r], k, v, 1, 128))
            errs.append(rel_l2(got[b][r][:, h * 128:(h + 1) * 128], ref))
    return max(errs), got


@pytest.mark.parametrize("B,S,H", [(1, 1, 1), (2, 70, 2), (1, 200, 3)])
def test_attention_q8_small_vs_oracle(B, S, H):
    log(f"attention_q8 B={B} S={S} H={H}")
    rng = np.random.default_rng(B * 100 + S + H)
    bits = bf16_normal_bits(rng, (B, S, 3 * H * 128))
    err, _ = _check(bits, B, S, H)
    log(f"  rel_l2 {err:.2e}")
    assert err <= TOL


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B,S", [(2, 4352), (1, 20480)])
def test_attention_q8_full_shape_sampled_rows(B, S):
    H = 24
    log(f"attention_q8 full B={B} S={S} H={H}")
    g = torch.Generator(device="cuda")
    g.manual_seed(S)
    qkv = torch.randn((B, S, 3 * H * 128), generator=g, device="cuda").to(torch.bfloat16)
    bits = host_bits(qkv)
    rng = np.random.default_rng(S)
    rows = np.unique(np.concatenate([rng.integers(0, S, 12), [0, S - 1]]))
    err, _ = _check(bits, B, S, H, rows=rows, heads=[0, 11, 23])
    log(f"  rel_l2 {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("B,S", [(2, 4352), (1, 20480), (1, 2781)])
def test_attention_q8_repeat_bitwise_and_fully_written(B, S):
    """Two calls on the same input give the same bits (no atomics, no timing-dependent reduction
    order, the workspace fully rewritten by each call) and every output element is written."""
    H = 24
    log(f"8-bit attention twice B={B} S={S} H={H}")
    g = torch.Generator(device="cuda")
    g.manual_seed(12)
    qkv = torch.randn((B, S, 3 * H * 128), generator=g, device="cuda").to(torch.bfloat16)
    outs, ws = [], None
    for _ in range(2):
        out = torch.full((B, S, H * 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        ws = dt.moss_attention_q8(qkv, out, B, S, H, ws=ws)
        outs.append(out)
    torch.cuda.synchronize()
    assert not torch.isnan(outs[0]).any()
    assert torch.equal(outs[0], outs[1])


def test_attention_q8_special_cases():
    log("attention_q8 special cases")
    rng = np.random.default_rng(81)
    H = 1
    # V constant over keys (and a single key): the output is V exactly, bit for bit after bf16 rounding
    S = 130
    x = O.from_bf16_bits(bf16_normal_bits(rng, (1, S, 3 * 128)))
    x[0, :, 256:] = x[0, 0, 256:]
    bits = f32_to_bf16_bits(x.astype(np.float32))
    got, _ = _run(bits, 1, S, H)
    np.testing.assert_array_equal(got[0], np.tile(O.from_bf16_bits(bits)[0, 0, 256:], (S, 1)))
    one = bf16_normal_bits(rng, (1, 1, 3 * 128))
    got, _ = _run(one, 1, 1, H)
    np.testing.assert_array_equal(got[0, 0], O.from_bf16_bits(one)[0, 0, 256:])
    # a dominant key: every query attends to key 37 only
    S = 70
    x = O.from_bf16_bits(bf16_normal_bits(rng, (1, S, 3 * 128)))
    x[0, :, :128] = x[0, 0, :128]                          # all queries equal
    x[0, :, 128:256] *= 0.01
    x[0, 37, 128:256] = x[0, 0, :128] * 8.0
    bits = f32_to_bf16_bits(x.astype(np.float32))
    got, _ = _run(bits, 1, S, H)
    xv = O.from_bf16_bits(bits)[0]
    vc, va = O.fp8_quantize_v(xv[:, 256:])
    # v_hat has up to 12 significant bits: the bf16 output is within half a bf16 unit of it
    np.testing.assert_allclose(got[0], np.tile(vc[37] * va / O.E4M3_MAX, (S, 1)), rtol=2.0 ** -8, atol=0)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B,S,amp", [(2, 200, 1.0), (1, 333, 4.0), (2, 4352, 1.0), (1, 4352, 4.0), (1, 20480, 1.0)])
def test_attention_q8_within_p_rounding_bound_of_exact_softmax(B, S, amp):
    """amp scales q and k (amp 4: scores spread over about +-60, the running max moves by far more than
    a factor 2 in many blocks, so the rescales carry most of the result)."""
    H = 24 if S >= 4352 else 2
    log(f"8-bit attention vs exact softmax on quantized operands B={B} S={S} H={H} amp={amp}")
    rng = np.random.default_rng(90 + S)
    x = O.from_bf16_bits(bf16_normal_bits(rng, (B, S, 3 * H * 128)))
    x[..., :2 * H * 128] *= amp
    bits = f32_to_bf16_bits(x.astype(np.float32))
    got, _ = _run(bits, B, S, H)
    x = O.from_bf16_bits(bits)
    rows = np.arange(S) if S <= 512 else np.unique(np.concatenate([rng.integers(0, S, 10), [0, S - 1]]))
    worst = 0.0
    for b in range(B):
        for h in ([0, 1] if H == 2 else [0, 11, 23]):
            q = x[b][rows, h * 128:(h + 1) * 128]
            k = x[b][:, (H + h) * 128:(H + h + 1) * 128]
            v = x[b][:, (2 * H + h) * 128:(2 * H + h + 1) * 128]
            ref, bound = exact_on_quantized(q, k, v)
            g = got[b][rows][:, h * 128:(h + 1) * 128]
            allowed = bound + np.abs(g) * 2.0 ** -8 + 1e-6     # + the bf16 rounding of the output
            err = np.abs(g - ref)
            worst = max(worst, float((err / allowed).max()))
            assert np.all(err <= allowed), (b, h, float((err - allowed).max()))
    log(f"  largest error / bound {worst:.3f}")

