"""The FP8 tier (gemm_precision = 1: the four projections of every joint block on MXFP8 operands) on
the GPU, against the oracle run with gemm_precision "mxfp8".

* Tiny: 2 blocks, hidden 256, 2 heads x 128, FFN 768 (the tier needs FFN % 256 == 0), 16x16 latent
  (64 image tokens) + 32 text tokens, seed 0, modulation weights x1 and x50. One block stage by stage
  (each stage from the GPU's previous one) and whole; the forward of a CFG pair (the unconditional row
  skipping block 1); the text refiner (320-wide states, two text-only blocks); and the drift of the
  FP8 forward from the bf16 forward of the same weights, which is the tier's loss.
* 8-bit attention (attention_mode = 1, alone and with the MXFP8 GEMMs): the block's attention tap
  against the oracle's attention_q8 of the GPU's own q, k, v; the forward against the oracle in the
  same mode.
* Full size: one joint block (hidden 3072, 24 heads, FFN 8192, batch 2, 256 text + 4096 image tokens)
  on sampled rows against the oracle's MXFP8 block from the same input, with exact and with 8-bit
  attention.
* The fused MXFP8 producers (LN-modulation, SwiGLU epilogue, attention output) against the separate
  quantizer, bit for bit (tiny, 1024^2 and 2048^2); the sampling step and the step cache in the tier
  against the tier's own forward and uncached steps.

The projections' own error bound: the scaled FP8 MFMA's result on identical MXFP8 operands deviates
from the exact product by a relative L2 of about 1.4e-5 (it does not sum a 64-product k-tile in
fp32), so a branch output computed from the GPU's own input is held to 5e-5.

Quantities the oracle computes through its own chain of quantized activations (a branch output, a
block's update, the difference of two passes) carry rounding noise amplified by the E4M3 grid: an
activation that differs from the oracle's by delta crosses an E4M3 rounding boundary with probability
about delta / u (u = 1/16, the E4M3 unit) and then moves by u, an rms change of sqrt(delta * u). With
delta one bf16 unit (1/256) that is 4 x the bf16 tier's rounding noise, so those comparisons take
4 x the bf16 tier's bound.
"""
import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_util import (REL_L2_BF16, REL_L2_FP32, dev_bf16, dev_weights, forward_block_chain, host_bf16, log,
                            oracle_cfg, rel_l2)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
dt = pytest.importorskip("diffusion_transformer_text_amd")

MODES = [1.0, 50.0]
REL_L2_MX_GEMM = 5e-5
REL_L2_FP8_CHAIN = 4 * REL_L2_BF16


def mx(a):
    return O.mx_dequantize(a)


def _cfg(shape, precision, attention_mode=0):
    return dt.moss_dit_config_init(num_layers=shape.num_layers, hidden=shape.hidden, num_heads=shape.num_heads,
                                   ffn_hidden=shape.ffn_hidden, text_dim=shape.text_dim,
                                   refiner_layers=shape.refiner_layers, gemm_precision=precision,
                                   attention_mode=attention_mode)


_cache = {}


def tiny(mod_scale, precision=1, attention_mode=0):
    key = (mod_scale, precision, attention_mode)
    if key not in _cache:
        log(f"create tiny FP8-shape model mod_scale={mod_scale} precision={precision} attention={attention_mode}")
        s = synth.TINY_FP8
        w, inp = synth.tiny_workload(mod_scale=mod_scale, shape=s)
        rw = synth.refiner_weights(s, seed=100)
        d = dev_weights(w, torch)
        d["text_proj_w"] = dev_bf16(rw["text_proj_w"], torch)
        for k in ("refiner_qkv_w", "refiner_out_w", "refiner_gate_up_w", "refiner_down_w"):
            d[k] = [dev_bf16(a, torch) for a in rw[k]]
        cfg = _cfg(s, precision, attention_mode)
        W = O.weights_to_f64(w)
        W["text_proj_w"] = O.from_bf16_bits(rw["text_proj_w"])
        for k in ("refiner_qkv_w", "refiner_out_w", "refiner_gate_up_w", "refiner_down_w"):
            W[k] = [O.from_bf16_bits(a) for a in rw[k]]
        _cache[key] = (dt.MossDiT(cfg, d), inp, W, oracle_cfg(cfg))
    return _cache[key]


def test_oracle_cfg_carries_the_tier():
    assert oracle_cfg(_cfg(synth.TINY_FP8, 1)).gemm_precision == "mxfp8"
    assert oracle_cfg(_cfg(synth.TINY_FP8, 0)).gemm_precision == "bf16"


@pytest.mark.parametrize("mod_scale", MODES)
def test_fp8_block_stages_vs_oracle(mod_scale):
    m, inp, W, ocfg = tiny(mod_scale)
    D, F, T, gh, gw = ocfg.hidden, ocfg.ffn_hidden, 32, 8, 8
    S, B = T + gh * gw, 2
    rng = np.random.default_rng(5)
    xbits = synth.bf16_normal_bits(rng, (B, S, D))
    x = dev_bf16(xbits, torch)
    mod = torch.empty((B, m.mod_stride), dtype=torch.bfloat16, device="cuda")
    m.moss_dit_modulation([0.8, 0.3], mod)
    M = B * S
    taps = {k: torch.empty((M, n), dtype=t, device="cuda") for k, n, t in
            [("a", D, torch.bfloat16), ("qkv", 3 * D, torch.bfloat16), ("o", D, torch.bfloat16),
             ("attn", D, torch.float32), ("x1", D, torch.bfloat16), ("a2", D, torch.bfloat16),
             ("h", F, torch.bfloat16), ("ffn", D, torch.float32)]}
    layer = 1
    log(f"fp8 block taps layer={layer} mod_scale={mod_scale}")
    m.moss_dit_block(layer, x, T, gh, gw, mod, taps=taps)
    torch.cuda.synchronize()
    g = {k: (host_bf16(v) if v.dtype == torch.bfloat16 else v.cpu().numpy().astype(np.float64)) for k, v in taps.items()}
    x0 = O.from_bf16_bits(xbits).reshape(M, D)
    modv = host_bf16(mod)
    wq, wo = mx(W["qkv_w"][layer]), mx(W["out_w"][layer])
    wgu, wd = mx(W["gate_up_w"][layer]), mx(W["down_w"][layer])
    errs = {}
    for b in range(B):
        rs = slice(b * S, (b + 1) * S)
        mb = modv[b, layer * 6 * D:(layer + 1) * 6 * D].reshape(6, D)
        errs.setdefault("a", []).append(rel_l2(g["a"][rs], O.bf16_round(O.ln_modulate(x0[rs], mb[0], mb[1], 1e-6))))
        qkv = O.bf16_round(mx(g["a"][rs]) @ wq.T)
        q = O.bf16_round(O.rope_rows(qkv[:, :D], T, gw, 128, 1e4))
        k = O.bf16_round(O.rope_rows(qkv[:, D:2 * D], T, gw, 128, 1e4))
        errs.setdefault("qkv", []).append(rel_l2(g["qkv"][rs], np.concatenate([q, k, qkv[:, 2 * D:]], 1)))
        gq = g["qkv"][rs]
        errs.setdefault("o", []).append(rel_l2(g["o"][rs], O.attention(gq[:, :D], gq[:, D:2 * D], gq[:, 2 * D:], 2, 128)))
        errs.setdefault("attn", []).append(rel_l2(g["attn"][rs], mx(g["o"][rs]) @ wo.T))
        errs.setdefault("x1", []).append(rel_l2(g["x1"][rs], O.bf16_round(x0[rs] + mb[2] * g["attn"][rs])))
        errs.setdefault("a2", []).append(rel_l2(g["a2"][rs], O.bf16_round(O.ln_modulate(g["x1"][rs], mb[3], mb[4], 1e-6))))
        gu = mx(g["a2"][rs]) @ wgu.T
        errs.setdefault("h", []).append(rel_l2(g["h"][rs], O.bf16_round(O.silu(gu[:, :F]) * gu[:, F:])))
        errs.setdefault("ffn", []).append(rel_l2(g["ffn"][rs], mx(g["h"][rs]) @ wd.T))
        taps_o = {}
        ref = O.block(x0[rs], mb, W, layer, ocfg, T, gw, mirror=True, taps=taps_o)
        errs.setdefault("block", []).append(rel_l2(host_bf16(x).reshape(M, D)[rs], ref))
        errs.setdefault("attn_branch", []).append(rel_l2(g["attn"][rs], taps_o["attn_out"]))
        errs.setdefault("ffn_branch", []).append(rel_l2(g["ffn"][rs], taps_o["ffn_out"]))
    log({k: f"{max(v):.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        tol = REL_L2_MX_GEMM if k in ("attn", "ffn") else REL_L2_BF16
        assert max(v) <= tol, (k, v)


def _forward(m, inp, sigma, skip):
    lat = torch.from_numpy(np.concatenate([inp.latents, inp.latents])).cuda()
    txt = torch.from_numpy(np.concatenate([inp.text_cond, inp.text_uncond])).cuda()
    vel = torch.empty_like(lat)
    m.moss_dit_forward(lat, txt, sigma, vel, skip_mask=skip)
    torch.cuda.synchronize()
    return vel.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("mod_scale", MODES)
def test_fp8_forward_vs_oracle(mod_scale):
    """The tier's CFG-pair forward against the oracle in the same tier: v, v_c - v_u (x50 mode only:
    under the literal init the difference is mostly bf16 rounding of tiny updates, as in the bf16
    tier's test_forward_vs_oracle), and each block of the same forward from the GPU's own input
    (branch outputs, gated residual adds, block output; the update in the x50 mode)."""
    m, inp, W, ocfg = tiny(mod_scale)
    log(f"fp8 tiny forward mod_scale={mod_scale}")
    L, D, T, gh, gw = ocfg.num_layers, ocfg.hidden, 32, 8, 8
    S = T + gh * gw
    lat = torch.from_numpy(np.concatenate([inp.latents, inp.latents])).cuda()
    txt = torch.from_numpy(np.concatenate([inp.text_cond, inp.text_uncond])).cuda()
    vel = torch.empty_like(lat)
    dump = torch.empty((L + 1, 2, S, D), dtype=torch.bfloat16, device="cuda")
    m.moss_dit_forward(lat, txt, [0.6, 0.6], vel, skip_mask=[0, 1 << 1], residual_dump=dump)
    torch.cuda.synchronize()
    v = vel.cpu().numpy().astype(np.float64)
    latn = np.concatenate([inp.latents, inp.latents]).astype(np.float64)
    txtn = np.concatenate([inp.text_cond, inp.text_uncond]).astype(np.float64)
    ref = O.forward(latn, txtn, [0.6, 0.6], W, ocfg, skip=[set(), {1}], mirror=True)
    e_v = rel_l2(v, ref)
    e_d = rel_l2(v[0] - v[1], ref[0] - ref[1])
    log(f"rel-L2 v {e_v:.3e}  (v_c - v_u) {e_d:.3e}")
    assert e_v <= REL_L2_BF16
    if mod_scale != 1.0:
        # v_c - v_u is the effect of one skipped block and the text: the two passes' rounding noise
        assert e_d <= REL_L2_FP8_CHAIN
    mod = torch.empty((2, m.mod_stride), dtype=torch.bfloat16, device="cuda")
    m.moss_dit_modulation([0.6, 0.6], mod)
    m_ref = [O.modulation(0.6, W, ocfg, mirror=True)[0]] * 2
    errs, mism = forward_block_chain(m, torch, dump, mod, [(0, [0, 1]), (1, [0])], T, gh, gw, W, ocfg, m_ref,
                                     lambda l, b: list(range(S)))
    log({k: f"{max(e):.2e}" for k, e in {**errs, **mism}.items()})
    # branch outputs and the update come through the oracle's own chain of E4M3-quantized activations:
    # the chain bound of this file's header; the block output itself holds the bf16 bound
    for k in ("attn_branch", "ffn_branch"):
        assert max(errs[k]) <= REL_L2_FP8_CHAIN, (k, errs[k])
    assert max(errs["block"]) <= REL_L2_BF16, errs["block"]
    if mod_scale != 1.0:
        assert max(errs["update"]) <= REL_L2_FP8_CHAIN, errs["update"]
    assert max(mism["gated_res"]) <= 1e-3, mism


@pytest.mark.parametrize("mod_scale", MODES)
def test_fp8_drift_from_bf16(mod_scale):
    """The tier's loss: FP8 against bf16 forward of the same weights (a report with a loose bound)."""
    m8, inp, _, _ = tiny(mod_scale, 1)
    m16, _, _, _ = tiny(mod_scale, 0)
    v8 = _forward(m8, inp, [0.6, 0.6], [0, 1 << 1])
    v16 = _forward(m16, inp, [0.6, 0.6], [0, 1 << 1])
    e_v = rel_l2(v8, v16)
    e_d = rel_l2(v8[0] - v8[1], v16[0] - v16[1])
    log(f"fp8 vs bf16 forward mod_scale={mod_scale}: rel-L2 v {e_v:.3e}  (v_c - v_u) {e_d:.3e}")
    assert 0 < e_v < 0.1


@pytest.mark.parametrize("attention_mode,T", [(0, 32), (1, 32), (1, 77)])
def test_fp8_text_refiner_vs_oracle(attention_mode, T):
    m, _, W, ocfg = tiny(1.0, precision=1, attention_mode=attention_mode)
    rng = np.random.default_rng(41 + T)
    B = 2
    enc = rng.standard_normal((B, T, ocfg.text_dim)).astype(np.float32)
    log(f"fp8 refiner B={B} T={T} attention_mode={attention_mode}")
    out = torch.empty((B, T, ocfg.hidden), dtype=torch.float32, device="cuda")
    m.moss_text_refine(torch.from_numpy(enc).cuda(), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(B):
        ref = O.text_refine(enc[b].astype(np.float64), W, ocfg, mirror=True)
        assert rel_l2(got[b], ref) <= REL_L2_BF16


# ------------------------------------------------------------------------------------------------
# full size
# ------------------------------------------------------------------------------------------------

FT, FGH, FGW = 256, 64, 64
FS = FT + FGH * FGW


@pytest.mark.timeout(600)
def test_fp8_full_block_sampled_rows():
    log(f"fp8 full block: D=3072 F=8192 H=24, B=2, S={FS}")
    shape = synth.Shape(num_layers=1)
    w = synth.torch_weights(shape, seed=3, device="cuda", mod_scale=50.0)
    cfg = dt.moss_dit_config_init(num_layers=1, gemm_precision=1)
    model = dt.MossDiT(cfg, w)
    ocfg = oracle_cfg(cfg)
    D, F = ocfg.hidden, ocfg.ffn_hidden
    rng = np.random.default_rng(12)
    B = 2
    xbits = synth.bf16_normal_bits(rng, (B, FS, D))
    sig = synth.uniform_f32(rng, (B,))
    x = dev_bf16(xbits, torch)
    mod = torch.empty((B, model.mod_stride), dtype=torch.bfloat16, device="cuda")
    model.moss_dit_modulation([float(s) for s in sig], mod)
    M = B * FS
    taps = {k: torch.empty((M, n), dtype=t, device="cuda") for k, n, t in
            [("o", D, torch.bfloat16), ("attn", D, torch.float32),
             ("h", F, torch.bfloat16), ("ffn", D, torch.float32)]}
    model.moss_dit_block(0, x, FT, FGH, FGW, mod, taps=taps)
    torch.cuda.synchronize()
    W = {"qkv_w": [host_bf16(w["qkv_w"][0])], "out_w": [host_bf16(w["out_w"][0])],
         "gate_up_w": [host_bf16(w["gate_up_w"][0])], "down_w": [host_bf16(w["down_w"][0])]}
    wo, wd = mx(W["out_w"][0]), mx(W["down_w"][0])
    modv = host_bf16(mod)
    x_out = host_bf16(x).reshape(B, FS, D)
    g = {k: (host_bf16(v) if v.dtype == torch.bfloat16 else v.cpu().numpy().astype(np.float64)).reshape(B, FS, -1)
         for k, v in taps.items()}
    x0 = O.from_bf16_bits(xbits)
    errs = {}
    for b in range(B):
        mb = modv[b, :6 * D].reshape(6, D)
        rows = np.unique(np.concatenate([rng.integers(0, FS, 16), [0, FT - 1, FT, FS - 1]]))
        errs.setdefault("out_proj", []).append(rel_l2(g["attn"][b][rows], mx(g["o"][b][rows]) @ wo.T))
        errs.setdefault("down_proj", []).append(rel_l2(g["ffn"][b][rows], mx(g["h"][b][rows]) @ wd.T))
        taps_o = {}
        ref = O.block(x0[b], mb, W, 0, ocfg, FT, FGW, mirror=True, rows=rows, taps=taps_o)
        errs.setdefault("block", []).append(rel_l2(x_out[b][rows], ref))
        errs.setdefault("block_update", []).append(rel_l2(x_out[b][rows] - x0[b][rows], ref - x0[b][rows]))
        errs.setdefault("attn_branch", []).append(rel_l2(g["attn"][b][rows], taps_o["attn_out"]))
        errs.setdefault("ffn_branch", []).append(rel_l2(g["ffn"][b][rows], taps_o["ffn_out"]))
    log({k: f"{max(v):.2e}" for k, v in errs.items()})
    model.close()
    for k, v in errs.items():
        tol = {"out_proj": REL_L2_MX_GEMM, "down_proj": REL_L2_MX_GEMM, "block": REL_L2_BF16}.get(k, REL_L2_FP8_CHAIN)
        assert max(v) <= tol, (k, v)


# ------------------------------------------------------------------------------------------------
# 8-bit attention in the model
# ------------------------------------------------------------------------------------------------

REL_L2_Q8_ATTN = 4e-3      # the attention kernel's own bound on identical inputs (bf16 output rounding)


@pytest.mark.parametrize("precision", [0, 1])
def test_q8_attention_block_tap_and_forward_vs_oracle(precision):
    mod_scale = 50.0
    m, inp, W, ocfg = tiny(mod_scale, precision, 1)
    assert ocfg.attention_mode == "q8"
    D, T, gh, gw = ocfg.hidden, 32, 8, 8
    S, B = T + gh * gw, 2
    rng = np.random.default_rng(6)
    x = dev_bf16(synth.bf16_normal_bits(rng, (B, S, D)), torch)
    mod = torch.empty((B, m.mod_stride), dtype=torch.bfloat16, device="cuda")
    m.moss_dit_modulation([0.8, 0.3], mod)
    M = B * S
    taps = {"qkv": torch.empty((M, 3 * D), dtype=torch.bfloat16, device="cuda"),
            "o": torch.empty((M, D), dtype=torch.bfloat16, device="cuda")}
    log(f"q8 attention block tap precision={precision}")
    m.moss_dit_block(1, x, T, gh, gw, mod, taps=taps)
    torch.cuda.synchronize()
    qkv, o = host_bf16(taps["qkv"]), host_bf16(taps["o"])
    errs = []
    for b in range(B):
        rs = slice(b * S, (b + 1) * S)
        ref = O.bf16_round(O.attention_q8(qkv[rs, :D], qkv[rs, D:2 * D], qkv[rs, 2 * D:], 2, 128))
        errs.append(rel_l2(o[rs], ref))
    log(f"  attention tap rel_l2 {max(errs):.2e}")
    assert max(errs) <= REL_L2_Q8_ATTN
    v = _forward(m, inp, [0.6, 0.6], [0, 1 << 1])
    lat = np.concatenate([inp.latents, inp.latents]).astype(np.float64)
    txt = np.concatenate([inp.text_cond, inp.text_uncond]).astype(np.float64)
    ref = O.forward(lat, txt, [0.6, 0.6], W, ocfg, skip=[set(), {1}], mirror=True)
    e_v = rel_l2(v, ref)
    e_d = rel_l2(v[0] - v[1], ref[0] - ref[1])
    log(f"  forward rel-L2 v {e_v:.3e}  (v_c - v_u) {e_d:.3e}")
    assert e_v <= REL_L2_BF16
    assert e_d <= REL_L2_FP8_CHAIN


@pytest.mark.timeout(600)
def test_q8_attention_full_block_sampled_rows():
    log(f"fp8 + q8 attention full block: D=3072 F=8192 H=24, B=2, S={FS}")
    shape = synth.Shape(num_layers=1)
    w = synth.torch_weights(shape, seed=3, device="cuda", mod_scale=50.0)
    cfg = dt.moss_dit_config_init(num_layers=1, gemm_precision=1, attention_mode=1)
    model = dt.MossDiT(cfg, w)
    ocfg = oracle_cfg(cfg)
    D = ocfg.hidden
    rng = np.random.default_rng(13)
    B = 2
    xbits = synth.bf16_normal_bits(rng, (B, FS, D))
    sig = synth.uniform_f32(rng, (B,))
    x = dev_bf16(xbits, torch)
    mod = torch.empty((B, model.mod_stride), dtype=torch.bfloat16, device="cuda")
    model.moss_dit_modulation([float(s_) for s_ in sig], mod)
    M = B * FS
    taps = {"qkv": torch.empty((M, 3 * D), dtype=torch.bfloat16, device="cuda"),
            "o": torch.empty((M, D), dtype=torch.bfloat16, device="cuda")}
    model.moss_dit_block(0, x, FT, FGH, FGW, mod, taps=taps)
    torch.cuda.synchronize()
    W = {"qkv_w": [host_bf16(w["qkv_w"][0])], "out_w": [host_bf16(w["out_w"][0])],
         "gate_up_w": [host_bf16(w["gate_up_w"][0])], "down_w": [host_bf16(w["down_w"][0])]}
    modv = host_bf16(mod)
    x_out = host_bf16(x).reshape(B, FS, D)
    qkv = host_bf16(taps["qkv"]).reshape(B, FS, 3 * D)
    o = host_bf16(taps["o"]).reshape(B, FS, D)
    x0 = O.from_bf16_bits(xbits)
    errs = {}
    for b in range(B):
        rows = np.unique(np.concatenate([rng.integers(0, FS, 12), [0, FT - 1, FT, FS - 1]]))
        for h in (0, 13, 23):
            sl = slice(h * 128, (h + 1) * 128)
            ref = O.bf16_round(O.attention_q8(qkv[b][rows, sl], qkv[b][:, D + h * 128:D + (h + 1) * 128],
                                              qkv[b][:, 2 * D + h * 128:2 * D + (h + 1) * 128], 1, 128))
            errs.setdefault("attention", []).append(rel_l2(o[b][rows, sl], ref))
        mb = modv[b, :6 * D].reshape(6, D)
        ref = O.block(x0[b], mb, W, 0, ocfg, FT, FGW, mirror=True, rows=rows)
        errs.setdefault("block", []).append(rel_l2(x_out[b][rows], ref))
        errs.setdefault("block_update", []).append(rel_l2(x_out[b][rows] - x0[b][rows], ref - x0[b][rows]))
    log({k: f"{max(v):.2e}" for k, v in errs.items()})
    model.close()
    assert max(errs["attention"]) <= REL_L2_Q8_ATTN
    assert max(errs["block"]) <= REL_L2_BF16
    assert max(errs["block_update"]) <= REL_L2_FP8_CHAIN


def _block_twice(model, layer, xbits, T, gh, gw, mod, taps_spec):
    """The block on two copies of x: once with taps (every MXFP8 activation written by the separate
    quantizer from its bf16 value) and once without (the producers write the codes themselves)."""
    x_fused = dev_bf16(xbits, torch)
    x_sep = dev_bf16(xbits, torch)
    M = xbits.shape[0] * xbits.shape[1]
    taps = {k: torch.empty((M, n), dtype=t, device="cuda") for k, n, t in taps_spec}
    model.moss_dit_block(layer, x_fused, T, gh, gw, mod)
    model.moss_dit_block(layer, x_sep, T, gh, gw, mod, taps=taps)
    torch.cuda.synchronize()
    return x_fused, x_sep


@pytest.mark.parametrize("attention_mode,T", [(0, 32), (1, 32), (1, 64)])
def test_fp8_fused_quantization_equals_separate_quantizer_bitwise(attention_mode, T):
    """Without taps the LayerNorm-modulation kernel, the SwiGLU epilogue and the attention kernels write
    the MXFP8 codes and scales of their bf16-rounded outputs themselves; with taps every activation
    goes through the separate quantizer. Both quantize the same bf16 values, so the block's output
    must be the same bits (T = 64: S = 128, whole 64-key blocks for the 8-bit attention)."""
    m, inp, W, ocfg = tiny(1.0, precision=1, attention_mode=attention_mode)
    D, gh, gw, B = ocfg.hidden, 8, 8, 2
    S = T + gh * gw
    rng = np.random.default_rng(21)
    xbits = synth.bf16_normal_bits(rng, (B, S, D))
    mod = torch.empty((B, m.mod_stride), dtype=torch.bfloat16, device="cuda")
    m.moss_dit_modulation([0.7, 0.2], mod)
    log(f"fp8 fused vs separate quantizers, tiny, attention_mode={attention_mode} T={T}")
    a, b = _block_twice(m, 1, xbits, T, gh, gw, mod, [("o", D, torch.bfloat16)])
    assert torch.equal(a, b)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("attention_mode", [0, 1])
@pytest.mark.parametrize("B,T,G", [(2, FT, FGH), (1, 4096, 128)])
def test_fp8_fused_quantization_equals_separate_quantizer_full_size(attention_mode, B, T, G):
    """The same at the full sizes: batch 2 with 256 text + 4096 image tokens (the exact attention's
    key-split tail and merge are in play), and one sample at 2048^2 with a 4096-token prompt
    (S = 20480: 320 key blocks for the 8-bit attention)."""
    log(f"fp8 fused vs separate quantizers, full size B={B} T={T} grid {G}x{G}, attention_mode={attention_mode}")
    shape = synth.Shape(num_layers=1)
    w = synth.torch_weights(shape, seed=4, device="cuda", mod_scale=50.0)
    cfg = dt.moss_dit_config_init(num_layers=1, gemm_precision=1, attention_mode=attention_mode)
    model = dt.MossDiT(cfg, w)
    D = cfg.hidden
    rng = np.random.default_rng(22)
    xbits = synth.bf16_normal_bits(rng, (B, T + G * G, D))
    mod = torch.empty((B, model.mod_stride), dtype=torch.bfloat16, device="cuda")
    model.moss_dit_modulation([0.9, 0.4][:B], mod)
    a, b = _block_twice(model, 0, xbits, T, G, G, mod, [("o", D, torch.bfloat16)])
    model.close()
    assert torch.equal(a, b)


@pytest.mark.parametrize("attention_mode", [0, 1])
@pytest.mark.parametrize("slg_scale", [0.0, 2.5])
def test_fp8_sample_step_equals_guidance_of_its_forward(attention_mode, slg_scale):
    """The FP8 tier through moss_sample_step (CFG 3, the negative pass skipping block 1, and with
    slg_scale > 0 a third row: the conditional pass skipping block 1) against the guidance combine
    and Euler update of the same rows' velocities from moss_dit_forward, in fp64: rows are computed
    independently, so only the fp32 guidance arithmetic may differ."""
    m, inp, W, ocfg = tiny(50.0, precision=1, attention_mode=attention_mode)
    log(f"fp8 sample step vs forward, attention_mode={attention_mode} slg={slg_scale}")
    step = 1
    sig = dt.moss_sigmas(2, 5.0)
    x0 = torch.from_numpy(inp.latents).cuda()
    tc = torch.from_numpy(inp.text_cond).cuda()
    tu = torch.from_numpy(inp.text_uncond).cuda()
    x = x0.clone()
    m.moss_sample_step(x, tc, tu, sig, step, cfg_scale=3.0, uncond_skip_layers=[1], slg_scale=slg_scale)
    rows = 3 if slg_scale > 0 else 2
    lat = torch.cat([x0] * rows).contiguous()
    txt = torch.cat([tc, tu, tc][:rows]).contiguous()
    vel = torch.empty_like(lat)
    m.moss_dit_forward(lat, txt, [float(sig[step])] * rows, vel, skip_mask=[0, 1 << 1, 1 << 1][:rows])
    torch.cuda.synchronize()
    v = vel.cpu().numpy().astype(np.float64)
    guided = v[1:2] + 3.0 * (v[0:1] - v[1:2])
    if rows == 3:
        guided = guided + slg_scale * (v[0:1] - v[2:3])
    x0n = x0.cpu().numpy().astype(np.float64)
    d_ref = float(sig[step + 1] - sig[step]) * guided
    d_got = x.cpu().numpy().astype(np.float64) - x0n
    assert np.isfinite(d_got).all()
    assert rel_l2(d_got, d_ref) <= REL_L2_FP32


@pytest.mark.parametrize("attention_mode", [0, 1])
def test_fp8_step_cache_threshold_zero_bitwise(attention_mode):
    """The step cache in the FP8 tier: with a threshold no change can fall below, every call runs in
    full and the three steps equal the uncached steps bit for bit."""
    m, inp, W, ocfg = tiny(50.0, precision=1, attention_mode=attention_mode)
    log(f"fp8 step cache threshold ~0, attention_mode={attention_mode}")
    sig = dt.moss_sigmas(3, 5.0)
    tc = torch.from_numpy(inp.text_cond).cuda()
    tu = torch.from_numpy(inp.text_uncond).cuda()

    def run(**kw):
        x = torch.from_numpy(inp.latents.copy()).cuda()
        xs = []
        for i in range(3):
            m.moss_sample_step(x, tc, tu, sig, i, cfg_scale=3.0, uncond_skip_layers=[1], **kw)
            torch.cuda.synchronize()
            xs.append(x.cpu().numpy().copy())
        return xs

    plain = run()
    cached = run(step_cache=True, step_cache_threshold=1e-30)
    for a, b in zip(plain, cached):
        np.testing.assert_array_equal(a, b)
    full, reused, _ = m.moss_step_cache_stats()
    assert (full, reused) == (3, 0)
