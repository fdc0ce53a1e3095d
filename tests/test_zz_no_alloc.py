"""moss_attention_noalloc (the no-allocation variant of the standalone exact attention, on the library's
static per-GPU scratch) against moss_attention through the C ABI: two calls in a row, the second on a
smaller input, each bit for bit equal to moss_attention on the same input (rotated q/k and output),
and on sampled query rows within the bf16 bound of the oracle's attention.

Shapes: batch 2 x 24 heads x (256 text + 4096 image tokens on a 64 x 64 grid) -- the 1024^2 block's
attention -- then batch 1 x 24 heads x (100 text + 2600 image tokens on a 52-wide grid). On a 256-CU
chip both leave the last round of query tiles partly empty, so both run the key-split tail whose
partial results live in the static scratch (the second call reuses it after the first)."""
import numpy as np
import pytest

import oracle as O
from tests.gpu_util import REL_L2_BF16, host_bf16, log, rel_l2

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
dt = pytest.importorskip("diffusion_transformer_text_amd")

H = 24
CASES = [(2, 256, 64, 64), (1, 100, 50, 52)]      # batch, text_len, grid_h, grid_w


def test_noalloc_attention_matches_moss_attention_twice():
    g = torch.Generator(device="cuda")
    g.manual_seed(21)
    for batch, T, gh, gw in CASES:
        S = T + gh * gw
        log(f"moss_attention_noalloc: B={batch} S={S} H={H} grid {gh}x{gw}")
        qkv = torch.randn((batch, S, 3 * H * 128), generator=g, device="cuda").to(torch.bfloat16)
        qa, qb = qkv.clone(), qkv.clone()
        oa = torch.empty((batch, S, H * 128), dtype=torch.bfloat16, device="cuda")
        ob = torch.full_like(oa, float("nan"))
        dt.moss_attention(qa, oa, batch, S, H, T, gw, rope=True)
        dt.moss_attention_noalloc(qb, ob, batch, S, H, T, gw, rope=True)
        torch.cuda.synchronize()
        assert torch.equal(qa, qb), "rotated q/k differ"
        assert torch.equal(oa, ob), "outputs differ"
        # the third bar: sampled query rows against the oracle from the same rotated q, k, v
        rng = np.random.default_rng(S)
        for b in range(batch):
            rows = np.unique(np.concatenate([rng.integers(0, S, 6), [0, T, S - 1]]))
            x = host_bf16(qb[b])
            D = H * 128
            ref = O.attention(x[rows, :D], x[:, D:2 * D], x[:, 2 * D:], H, 128)
            e = rel_l2(host_bf16(ob[b])[rows], ref)
            log(f"  sample {b}: rel-L2 vs oracle {e:.2e}")
            assert e <= REL_L2_BF16
        del qkv, qa, qb, oa, ob
