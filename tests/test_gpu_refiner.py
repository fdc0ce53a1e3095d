"""The text refiner on the GPU (moss_text_refine): projection text_dim -> hidden and two unmodulated
text-only joint blocks, run once per prompt.

* Tiny: the tiny DiT's widths (hidden 256, 2 heads, FFN 704) with 320-wide encoder states, weights
  N(0, 0.02) from the refiner's own seed, encoder states N(0, 1); prompt lengths 32 (two samples) and
  5 (a ragged tile), against the oracle; batch invariance bit for bit; zero output projections reduce
  it to the projection; permuting the prompt's rows permutes the output.
* Full size: hidden 3072, 24 heads, FFN 8192, 4096-wide states, two samples of 256 tokens, against the
  oracle on every row.
"""
import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_util import REL_L2_BF16, dev_bf16, dev_weights, host_bf16, log, oracle_cfg, rel_l2

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
dt = pytest.importorskip("diffusion_transformer_text_amd")


def _cfg(shape):
    return dt.moss_dit_config_init(num_layers=shape.num_layers, hidden=shape.hidden, num_heads=shape.num_heads,
                                   ffn_hidden=shape.ffn_hidden, text_dim=shape.text_dim,
                                   refiner_layers=shape.refiner_layers)


def _tiny_model(zero_branches=False):
    s = synth.TINY
    w, _ = synth.tiny_workload()
    rw = synth.refiner_weights(s, seed=100)
    if zero_branches:
        rw["refiner_out_w"] = [np.zeros_like(a) for a in rw["refiner_out_w"]]
        rw["refiner_down_w"] = [np.zeros_like(a) for a in rw["refiner_down_w"]]
    d = dev_weights(w, torch)
    d["text_proj_w"] = dev_bf16(rw["text_proj_w"], torch)
    for k in ("refiner_qkv_w", "refiner_out_w", "refiner_gate_up_w", "refiner_down_w"):
        d[k] = [dev_bf16(a, torch) for a in rw[k]]
    cfg = _cfg(s)
    W = {"text_proj_w": O.from_bf16_bits(rw["text_proj_w"])}
    for k in ("refiner_qkv_w", "refiner_out_w", "refiner_gate_up_w", "refiner_down_w"):
        W[k] = [O.from_bf16_bits(a) for a in rw[k]]
    return dt.MossDiT(cfg, d), W, oracle_cfg(cfg)


def _refine(model, enc):
    out = torch.empty((enc.shape[0], enc.shape[1], model.cfg.hidden), dtype=torch.float32, device="cuda")
    model.moss_text_refine(enc, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("B,T", [(2, 32), (1, 5)])
def test_refine_tiny_vs_oracle(B, T):
    model, W, ocfg = _tiny_model()
    rng = np.random.default_rng(40 + T)
    enc = rng.standard_normal((B, T, ocfg.text_dim)).astype(np.float32)
    got = _refine(model, torch.from_numpy(enc).cuda())
    errs = [rel_l2(got[b], O.text_refine(enc[b].astype(np.float64), W, ocfg, mirror=True)) for b in range(B)]
    log(f"refiner tiny B={B} T={T}: rel-L2 {max(errs):.2e}")
    assert max(errs) <= REL_L2_BF16
    # every value is an exact bf16 (the refiner's output is the bf16 residual stream)
    assert np.array_equal(got, O.bf16_round(got))
    if B > 1:
        # batch invariance: each sample alone gives the same bits
        for b in range(B):
            np.testing.assert_array_equal(_refine(model, torch.from_numpy(enc[b:b + 1].copy()).cuda())[0], got[b])
    model.close()


def test_refine_tiny_zero_branches_and_permutation():
    model, W, ocfg = _tiny_model(zero_branches=True)
    rng = np.random.default_rng(50)
    enc = rng.standard_normal((1, 12, ocfg.text_dim)).astype(np.float32)
    got = _refine(model, torch.from_numpy(enc).cuda())[0]
    proj = O.bf16_round(O.bf16_round(enc[0].astype(np.float64)) @ W["text_proj_w"].T)
    log(f"refiner zero branches: rel-L2 {rel_l2(got, proj):.2e}, equal {np.mean(got == proj):.4f}")
    assert rel_l2(got, proj) <= 1e-2 and np.mean(got == proj) > 0.99
    model.close()
    model, W, ocfg = _tiny_model()
    perm = rng.permutation(12)
    a = _refine(model, torch.from_numpy(enc).cuda())[0]
    b = _refine(model, torch.from_numpy(enc[:, perm].copy()).cuda())[0]
    assert rel_l2(b, a[perm]) <= REL_L2_BF16
    model.close()


def test_refine_needs_its_weights():
    w, _ = synth.tiny_workload()
    model = dt.MossDiT(_cfg(synth.TINY), dev_weights(w, torch))
    enc = torch.zeros((1, 4, synth.TINY.text_dim), dtype=torch.float32, device="cuda")
    out = torch.empty((1, 4, synth.TINY.hidden), dtype=torch.float32, device="cuda")
    with pytest.raises(dt.MossError) as e:
        model.moss_text_refine(enc, out)
    assert e.value.status == dt.MOSS_ERR_NOT_SUPPORTED
    model.close()


@pytest.mark.timeout(600)
def test_refine_full_size_vs_oracle():
    s = synth.FULL
    log("refiner full size: hidden 3072, 24 heads, FFN 8192, 4096-wide states, B=2, T=256")
    w = synth.torch_weights(s, seed=0, device="cuda")
    w.update(synth.torch_refiner_weights(s, seed=100, device="cuda"))
    cfg = _cfg(s)
    model = dt.MossDiT(cfg, w)
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    enc = torch.randn((2, 256, s.text_dim), generator=g, device="cuda", dtype=torch.float32)
    got = _refine(model, enc)
    W = {"text_proj_w": host_bf16(w["text_proj_w"])}
    for k in ("refiner_qkv_w", "refiner_out_w", "refiner_gate_up_w", "refiner_down_w"):
        W[k] = [host_bf16(a) for a in w[k]]
    ocfg = oracle_cfg(cfg)
    e_np = enc.cpu().numpy().astype(np.float64)
    errs = [rel_l2(got[b], O.text_refine(e_np[b], W, ocfg, mirror=True)) for b in range(2)]
    log(f"  rel-L2 {max(errs):.2e}")
    model.close()
    assert max(errs) <= REL_L2_BF16
