"""Model-level parity on the GPU at the tiny configuration: 2 blocks, hidden 256, 2 heads x 128,
FFN 704, 16x16 latent (64 image tokens) + 32 text tokens, seed 0; 2 Euler steps (shift 5) with
CFG 3 and uncond_skip_layers=[1]. Every case runs twice: with the literal N(0, 0.02) init and with
the modulation weights scaled by 50 (gates ~0.25), where a block's update survives the bf16 residual.
"""
import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_util import (REL_L2_BF16, REL_L2_FP32, dev_bf16, dev_weights, forward_block_chain, host_bf16, host_bits,
                            log, oracle_cfg, rel_l2)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
dt = pytest.importorskip("diffusion_transformer_text_amd")

MODES = [1.0, 50.0]


def tiny_cfg():
    s = synth.TINY
    return dt.moss_dit_config_init(num_layers=s.num_layers, hidden=s.hidden, num_heads=s.num_heads,
                                   ffn_hidden=s.ffn_hidden)


_cache = {}


def model(mod_scale):
    if mod_scale not in _cache:
        log(f"create tiny model mod_scale={mod_scale}")
        w, inp = synth.tiny_workload(mod_scale=mod_scale)
        cfg = tiny_cfg()
        dw = dev_weights(w, torch)
        m = dt.MossDiT(cfg, dw)
        _cache[mod_scale] = (m, w, inp, O.weights_to_f64(w), oracle_cfg(cfg), dw)
    return _cache[mod_scale]


@pytest.mark.parametrize("mod_scale", MODES)
def test_modulation_vs_oracle(mod_scale):
    m, w, inp, W, ocfg, _ = model(mod_scale)
    sig = [0.0, 0.37, 1.0]
    mod = torch.empty((3, m.mod_stride), dtype=torch.bfloat16, device="cuda")
    m.moss_dit_modulation(sig, mod)
    torch.cuda.synchronize()
    got = host_bf16(mod)
    D, L = ocfg.hidden, ocfg.num_layers
    for b, s in enumerate(sig):
        ml, mf = O.modulation(s, W, ocfg, mirror=True)
        ref = np.concatenate([ml.reshape(-1), mf.reshape(-1)])
        assert rel_l2(got[b], ref) < 1e-2
        # most entries identical after the final bf16 rounding
        assert np.mean(got[b] == ref) > 0.9


@pytest.mark.parametrize("mod_scale", MODES)
def test_block_taps_vs_oracle(mod_scale):
    """Every stage of one block on identical inputs (the GPU's own previous stage), then the whole
    block against the oracle from the same x and modulation."""
    m, w, inp, W, ocfg, _ = model(mod_scale)
    D, F, T, gh, gw = ocfg.hidden, ocfg.ffn_hidden, 32, 8, 8
    S, B = T + gh * gw, 2
    rng = np.random.default_rng(5)
    xbits = synth.bf16_normal_bits(rng, (B, S, D))
    x = dev_bf16(xbits, torch)
    mod = torch.empty((B, m.mod_stride), dtype=torch.bfloat16, device="cuda")
    m.moss_dit_modulation([0.8, 0.3], mod)
    M = B * S
    taps = {"a": torch.empty((M, D), dtype=torch.bfloat16, device="cuda"),
            "qkv": torch.empty((M, 3 * D), dtype=torch.bfloat16, device="cuda"),
            "o": torch.empty((M, D), dtype=torch.bfloat16, device="cuda"),
            "attn": torch.empty((M, D), dtype=torch.float32, device="cuda"),
            "x1": torch.empty((M, D), dtype=torch.bfloat16, device="cuda"),
            "a2": torch.empty((M, D), dtype=torch.bfloat16, device="cuda"),
            "h": torch.empty((M, F), dtype=torch.bfloat16, device="cuda"),
            "ffn": torch.empty((M, D), dtype=torch.float32, device="cuda")}
    layer = 1
    log(f"block taps layer={layer} mod_scale={mod_scale}")
    m.moss_dit_block(layer, x, T, gh, gw, mod, taps=taps)
    torch.cuda.synchronize()
    g = {k: (host_bf16(v) if v.dtype == torch.bfloat16 else v.cpu().numpy().astype(np.float64)) for k, v in taps.items()}
    x0 = O.from_bf16_bits(xbits).reshape(M, D)
    modv = host_bf16(mod)
    errs = {}
    for b in range(B):
        rs = slice(b * S, (b + 1) * S)
        mb = modv[b, layer * 6 * D:(layer + 1) * 6 * D].reshape(6, D)
        # stage by stage, each from the GPU's previous stage
        errs.setdefault("a", []).append(rel_l2(g["a"][rs], O.bf16_round(O.ln_modulate(x0[rs], mb[0], mb[1], 1e-6))))
        qkv = O.bf16_round(g["a"][rs] @ W["qkv_w"][layer].T)
        q = O.bf16_round(O.rope_rows(qkv[:, :D], T, gw, 128, 1e4))
        k = O.bf16_round(O.rope_rows(qkv[:, D:2 * D], T, gw, 128, 1e4))
        errs.setdefault("qkv", []).append(rel_l2(g["qkv"][rs], np.concatenate([q, k, qkv[:, 2 * D:]], 1)))
        gq = g["qkv"][rs]
        errs.setdefault("o", []).append(rel_l2(g["o"][rs], O.attention(gq[:, :D], gq[:, D:2 * D], gq[:, 2 * D:], 2, 128)))
        errs.setdefault("attn", []).append(rel_l2(g["attn"][rs], g["o"][rs] @ W["out_w"][layer].T))
        errs.setdefault("x1", []).append(rel_l2(g["x1"][rs], O.bf16_round(x0[rs] + mb[2] * g["attn"][rs])))
        errs.setdefault("a2", []).append(rel_l2(g["a2"][rs], O.bf16_round(O.ln_modulate(g["x1"][rs], mb[3], mb[4], 1e-6))))
        gu = g["a2"][rs] @ W["gate_up_w"][layer].T
        errs.setdefault("h", []).append(rel_l2(g["h"][rs], O.bf16_round(O.silu(gu[:, :F]) * gu[:, F:])))
        errs.setdefault("ffn", []).append(rel_l2(g["ffn"][rs], g["h"][rs] @ W["down_w"][layer].T))
        # whole block from the same input
        taps_o = {}
        ref = O.block(x0[rs], mb, W, layer, ocfg, T, gw, mirror=True, taps=taps_o)
        errs.setdefault("block", []).append(rel_l2(host_bf16(x).reshape(M, D)[rs], ref))
        errs.setdefault("attn_branch", []).append(rel_l2(g["attn"][rs], taps_o["attn_out"]))
        errs.setdefault("ffn_branch", []).append(rel_l2(g["ffn"][rs], taps_o["ffn_out"]))
    log({k: max(v) for k, v in errs.items()})
    for k, v in errs.items():
        tol = 1e-5 if k in ("attn", "ffn") else REL_L2_BF16
        assert max(v) <= tol, (k, v)


def _forward(m, inp, sigma, skip):
    lat = torch.from_numpy(np.concatenate([inp.latents, inp.latents])).cuda()
    txt = torch.from_numpy(np.concatenate([inp.text_cond, inp.text_uncond])).cuda()
    vel = torch.empty_like(lat)
    m.moss_dit_forward(lat, txt, sigma, vel, skip_mask=skip)
    torch.cuda.synchronize()
    return vel.cpu().numpy()


@pytest.mark.parametrize("mod_scale", MODES)
def test_forward_vs_oracle(mod_scale):
    """The CFG pair's forward (the unconditional row skipping block 1) against the oracle: v, the
    guidance difference v_c - v_u, and every block of the same forward from the GPU's own input to it
    (branch outputs, gated residual adds, block output and update; tests/gpu_util.forward_block_chain).

    v_c - v_u is gated in the x50 mode only. Under the literal N(0, 0.02) init the gates are ~5e-3, a
    block's update is ~6e-4 of the residual and below half a bf16 ulp for most elements, so the two
    rows' difference is mostly which elements happened to round up: an independent fp64 chain and the
    GPU's fp32 one disagree on a few 1e-4 of those roundings, which alone is a few percent of that
    difference. What the literal mode can check sharply is checked per block instead: the branch
    outputs (their size does not depend on the gates) and the residual adds recomputed from them."""
    m, w, inp, W, ocfg, _ = model(mod_scale)
    log(f"tiny forward mod_scale={mod_scale}")
    L, D, T, gh, gw = ocfg.num_layers, ocfg.hidden, 32, 8, 8
    S = T + gh * gw
    lat = torch.from_numpy(np.concatenate([inp.latents, inp.latents])).cuda()
    txt = torch.from_numpy(np.concatenate([inp.text_cond, inp.text_uncond])).cuda()
    vel = torch.empty_like(lat)
    dump = torch.empty((L + 1, 2, S, D), dtype=torch.bfloat16, device="cuda")
    m.moss_dit_forward(lat, txt, [0.6, 0.6], vel, skip_mask=[0, 1 << 1], residual_dump=dump)
    torch.cuda.synchronize()
    v = vel.cpu().numpy()
    latn = np.concatenate([inp.latents, inp.latents]).astype(np.float64)
    txtn = np.concatenate([inp.text_cond, inp.text_uncond]).astype(np.float64)
    ref = O.forward(latn, txtn, [0.6, 0.6], W, ocfg, skip=[set(), {1}], mirror=True)
    e_v = rel_l2(v, ref)
    e_d = rel_l2(v[0] - v[1], ref[0] - ref[1])
    log(f"rel-L2 v {e_v:.3e}  (v_c - v_u) {e_d:.3e}{'' if mod_scale != 1.0 else ' (not gated at the literal init)'}")
    assert e_v <= REL_L2_BF16
    if mod_scale != 1.0:
        assert e_d <= REL_L2_BF16
    mod = torch.empty((2, m.mod_stride), dtype=torch.bfloat16, device="cuda")
    m.moss_dit_modulation([0.6, 0.6], mod)
    m_ref = [O.modulation(0.6, W, ocfg, mirror=True)[0]] * 2
    errs, mism = forward_block_chain(m, torch, dump, mod, [(0, [0, 1]), (1, [0])], T, gh, gw, W, ocfg, m_ref,
                                     lambda l, b: list(range(S)))
    log({k: f"{max(e):.2e}" for k, e in {**errs, **mism}.items()})
    for k in ("attn_branch", "ffn_branch", "block"):
        assert max(errs[k]) <= REL_L2_BF16, (k, errs[k])
    if mod_scale != 1.0:
        assert max(errs["update"]) <= REL_L2_BF16, errs["update"]
    assert max(mism["gated_res"]) <= 1e-3, mism


@pytest.mark.parametrize("lat_h,lat_w,T,B", [(16, 24, 7, 3), (24, 8, 1, 1)])
def test_forward_non_square_latent_odd_text_vs_oracle(lat_h, lat_w, T, B):
    """Aspect ratios other than 1:1 (a 8x12 and a 12x4 patch grid: the rotary rows and columns and
    the unpatchify differ), odd text lengths (7 and 1 text tokens: a ragged attention tile) and
    batches of 3 and 1 with different sigmas and skip sets per sample, against the oracle."""
    m, w, inp, W, ocfg, _ = model(50.0)
    log(f"tiny forward latent {lat_h}x{lat_w} T={T} B={B}")
    rng = np.random.default_rng(lat_h * 100 + lat_w + T)
    lat = rng.standard_normal((B, ocfg.latent_channels, lat_h, lat_w)).astype(np.float32)
    txt = rng.standard_normal((B, T, ocfg.hidden)).astype(np.float32)
    sig = [0.9, 0.4, 0.1][:B]
    skips = [set(), {1}, {0, 1}][:B]
    vel = torch.empty((B, ocfg.latent_channels, lat_h, lat_w), dtype=torch.float32, device="cuda")
    m.moss_dit_forward(torch.from_numpy(lat).cuda(), torch.from_numpy(txt).cuda(), sig, vel,
                       skip_mask=[sum(1 << l for l in sk) for sk in skips])
    torch.cuda.synchronize()
    ref = O.forward(lat.astype(np.float64), txt.astype(np.float64), sig, W, ocfg, skip=skips, mirror=True)
    v = vel.cpu().numpy().astype(np.float64)
    errs = [rel_l2(v[b], ref[b]) for b in range(B)]
    log(f"rel-L2 per sample {[f'{e:.2e}' for e in errs]}")
    assert max(errs) <= REL_L2_BF16


@pytest.mark.parametrize("mod_scale", MODES)
def test_two_sampling_steps_vs_oracle(mod_scale):
    """2 Euler steps, shift 5, CFG 3, uncond_skip_layers=[1], window 0.01..1.0: step 0 runs full
    CFG, step 1 skips block 1 in the negative pass."""
    m, w, inp, W, ocfg, _ = model(mod_scale)
    log(f"tiny sampling mod_scale={mod_scale}")
    sig = dt.moss_sigmas(2, 5.0)
    x = torch.from_numpy(inp.latents.copy()).cuda()
    tc = torch.from_numpy(inp.text_cond).cuda()
    tu = torch.from_numpy(inp.text_uncond).cuda()
    xs = []
    for i in range(2):
        m.moss_sample_step(x, tc, tu, sig, i, cfg_scale=3.0, uncond_skip_layers=[1])
        torch.cuda.synchronize()
        xs.append(x.cpu().numpy().copy())
    xr = inp.latents.astype(np.float64)
    refs = []
    for i in range(2):
        # the oracle continues from the GPU's x_i so each step is compared on identical inputs
        xin = xs[i - 1].astype(np.float64) if i > 0 else xr
        refs.append(O.sample_step(xin, inp.text_cond.astype(np.float64), inp.text_uncond.astype(np.float64), W, ocfg,
                                  i, sig.astype(np.float64), 3.0, (1,), 0.01, 1.0, mirror=True))
    x0 = inp.latents.astype(np.float64)
    for i in range(2):
        prev = xs[i - 1] if i > 0 else x0
        e = rel_l2(xs[i] - prev, refs[i] - prev)
        log(f"step {i}: rel-L2 of the update {e:.3e}")
        assert e <= REL_L2_BF16
    # an uninterrupted oracle run from x_0 stays within the bar too
    x_or = xr
    for i in range(2):
        x_or = O.sample_step(x_or, inp.text_cond.astype(np.float64), inp.text_uncond.astype(np.float64), W, ocfg, i,
                             sig.astype(np.float64), 3.0, (1,), 0.01, 1.0, mirror=True)
    assert rel_l2(xs[1] - x0, x_or - x0) <= REL_L2_BF16


def test_invariants_bitwise():
    m, w, inp, W, ocfg, dw = model(50.0)
    log("invariants")
    # determinism
    a = _forward(m, inp, [0.5, 0.5], [0, 2])
    b = _forward(m, inp, [0.5, 0.5], [0, 2])
    np.testing.assert_array_equal(a, b)
    # batch invariance: the cond sample alone equals the cond sample of the pair
    lat = torch.from_numpy(inp.latents).cuda()
    txt = torch.from_numpy(inp.text_cond).cuda()
    vel = torch.empty_like(lat)
    m.moss_dit_forward(lat, txt, [0.5], vel)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(vel.cpu().numpy()[0], a[0])
    # skip of block 1 == zero gate rows of block 1's modulation (x + 0*y = x)
    mw1 = dw["mod_w"][1].clone()
    D = ocfg.hidden
    mw1[2 * D:3 * D] = 0
    mw1[5 * D:] = 0
    dw2 = dict(dw)
    dw2["mod_w"] = [dw["mod_w"][0], mw1]
    m2 = dt.MossDiT(tiny_cfg(), dw2)
    c = _forward(m2, inp, [0.5, 0.5], [0, 0])
    np.testing.assert_array_equal(c[1], a[1])
    m2.close()


def test_sample_step_guidance_paths_bitwise():
    m, w, inp, W, ocfg, _ = model(50.0)
    log("guidance paths")
    sig = dt.moss_sigmas(2, 5.0)
    tc = torch.from_numpy(inp.text_cond).cuda()
    tu = torch.from_numpy(inp.text_uncond).cuda()
    lat = torch.from_numpy(np.concatenate([inp.latents, inp.latents])).cuda()
    # cfg = 1: x1 = x0 + dsigma * v_c exactly, and no negative text is needed
    x = torch.from_numpy(inp.latents.copy()).cuda()
    m.moss_sample_step(x, tc, None, sig, 0, cfg_scale=1.0, uncond_skip_layers=[])
    vc = torch.empty_like(lat[:1])
    m.moss_dit_forward(lat[:1].contiguous(), tc, [float(sig[0])], vc)
    x_ref = torch.from_numpy(inp.latents.copy()).cuda()
    dt.moss_cfg_euler(vc, None, x_ref, 1.0, float(sig[0]), float(sig[1]))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(x.cpu().numpy(), x_ref.cpu().numpy())
    # step 1 with [] equals step 1 with the window closed (slg_start above the progress)
    x1 = torch.from_numpy(inp.latents.copy()).cuda()
    m.moss_sample_step(x1, tc, tu, sig, 1, cfg_scale=3.0, uncond_skip_layers=[])
    x2 = torch.from_numpy(inp.latents.copy()).cuda()
    m.moss_sample_step(x2, tc, tu, sig, 1, cfg_scale=3.0, uncond_skip_layers=[1], slg_start=0.9)
    x3 = torch.from_numpy(inp.latents.copy()).cuda()
    m.moss_sample_step(x3, tc, tu, sig, 1, cfg_scale=3.0, uncond_skip_layers=[1])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(x1.cpu().numpy(), x2.cpu().numpy())
    assert not np.array_equal(x1.cpu().numpy(), x3.cpu().numpy())
    # resume: two steps in a row == one step, copy out, copy back, second step
    xa = torch.from_numpy(inp.latents.copy()).cuda()
    for i in range(2):
        m.moss_sample_step(xa, tc, tu, sig, i, uncond_skip_layers=[1])
    xb = torch.from_numpy(inp.latents.copy()).cuda()
    m.moss_sample_step(xb, tc, tu, sig, 0, uncond_skip_layers=[1])
    saved = xb.cpu().numpy().copy()
    xc = torch.from_numpy(saved).cuda()
    m.moss_sample_step(xc, tc, tu, sig, 1, uncond_skip_layers=[1])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(xa.cpu().numpy(), xc.cpu().numpy())


@pytest.mark.parametrize("mod_scale", MODES)
@pytest.mark.parametrize("step,slg_scale,trunc", [(1, 2.5, 1.0), (1, 2.5, 0.5), (1, 0.0, 0.5), (0, 2.5, 0.5)])
def test_guidance_variants_vs_oracle(mod_scale, step, slg_scale, trunc):
    """Three-pass skip-layer guidance (a third, skipped conditional pass inside the window: step 1 of 2;
    step 0 is outside) and CFG truncation (X = 0.5 of 2 steps drops the negative branch at step 1),
    one step from identical inputs against the oracle. With the x50 modulation the skip-layer term
    itself (three-pass minus two-pass update) is compared too."""
    m, w, inp, W, ocfg, _ = model(mod_scale)
    log(f"guidance variant mod_scale={mod_scale} step={step} slg={slg_scale} trunc={trunc}")
    sig = dt.moss_sigmas(2, 5.0)
    tc = torch.from_numpy(inp.text_cond).cuda()
    tu = torch.from_numpy(inp.text_uncond).cuda()
    args = dict(cfg_scale=3.0, uncond_skip_layers=[1])

    def gpu(**kw):
        x = torch.from_numpy(inp.latents.copy()).cuda()
        m.moss_sample_step(x, tc, tu, sig, step, **kw)
        torch.cuda.synchronize()
        return x.cpu().numpy()

    def ref(**kw):
        f = lambda a: a.astype(np.float64)
        return O.sample_step(f(inp.latents), f(inp.text_cond), f(inp.text_uncond), W, ocfg, step, f(sig), 3.0, (1,),
                             0.01, 1.0, mirror=True, **kw)

    x0 = inp.latents.astype(np.float64)
    got = gpu(slg_scale=slg_scale, cfg_truncation=trunc, **args)
    want = ref(slg_scale=slg_scale, cfg_truncation=trunc)
    e = rel_l2(got - x0, want - x0)
    log(f"  rel-L2 of the update {e:.3e}")
    assert e <= REL_L2_BF16
    if slg_scale > 0 and step == 1 and mod_scale == 50.0:
        d_got = got - gpu(slg_scale=0.0, cfg_truncation=trunc, **args)
        d_want = want - ref(slg_scale=0.0, cfg_truncation=trunc)
        e2 = rel_l2(d_got, d_want)
        log(f"  rel-L2 of the skip-layer term {e2:.3e}")
        assert e2 <= REL_L2_BF16


def test_guidance_variants_bitwise():
    m, w, inp, W, ocfg, _ = model(50.0)
    log("guidance variants bitwise")
    sig = dt.moss_sigmas(2, 5.0)
    tc = torch.from_numpy(inp.text_cond).cuda()
    tu = torch.from_numpy(inp.text_uncond).cuda()

    def step(i, **kw):
        x = torch.from_numpy(inp.latents.copy()).cuda()
        m.moss_sample_step(x, tc, tu if kw.get("cfg_scale", 3.0) > 1 else None, sig, i, **kw)
        torch.cuda.synchronize()
        return x.cpu().numpy()

    # no third pass: outside the window (step 0), an empty skip list, or slg 0
    np.testing.assert_array_equal(step(0, uncond_skip_layers=[1], slg_scale=2.5), step(0, uncond_skip_layers=[1]))
    np.testing.assert_array_equal(step(1, uncond_skip_layers=[], slg_scale=2.5), step(1, uncond_skip_layers=[]))
    # a truncated step is the CFG-1 step; before the truncation point nothing changes
    np.testing.assert_array_equal(step(1, uncond_skip_layers=[1], cfg_truncation=0.5),
                                  step(1, cfg_scale=1.0, uncond_skip_layers=[1]))
    np.testing.assert_array_equal(step(0, uncond_skip_layers=[1], cfg_truncation=0.5), step(0, uncond_skip_layers=[1]))
    # the three-pass step from the library's own predictions: rows [cond, uncond skipping 1, cond
    # skipping 1] of one forward give v_c, v_u, v_s; the step applies v_u + 3 (v_c - v_u) + 2.5 (v_c - v_s)
    lat = torch.from_numpy(np.concatenate([inp.latents] * 3)).cuda()
    txt = torch.from_numpy(np.concatenate([inp.text_cond, inp.text_uncond, inp.text_cond])).cuda()
    vel = torch.empty_like(lat)
    m.moss_dit_forward(lat, txt, [float(sig[1])] * 3, vel, skip_mask=[0, 1 << 1, 1 << 1])
    torch.cuda.synchronize()
    v = vel.cpu().numpy().astype(np.float64)
    vc, vu, vs = v[0:1], v[1:2], v[2:3]
    assert not np.array_equal(vc, vs)
    x3 = step(1, uncond_skip_layers=[1], slg_scale=2.5)
    x_ref = inp.latents.astype(np.float64) + float(sig[2] - sig[1]) * (vu + 3.0 * (vc - vu) + 2.5 * (vc - vs))
    assert rel_l2(x3, x_ref) <= REL_L2_FP32
    # and the same step through the standalone combine entry point, bit for bit
    xk = torch.from_numpy(inp.latents.copy()).cuda()
    dt.moss_guidance_euler(vel[0:1].contiguous(), vel[1:2].contiguous(), vel[2:3].contiguous(), xk, 3.0, 2.5,
                           float(sig[1]), float(sig[2]))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(xk.cpu().numpy(), x3)


def test_residual_dump_and_skip_rows():
    m, w, inp, W, ocfg, _ = model(50.0)
    log("residual dump")
    L, D = ocfg.num_layers, ocfg.hidden
    S = 32 + 64
    lat = torch.from_numpy(np.concatenate([inp.latents, inp.latents])).cuda()
    txt = torch.from_numpy(np.concatenate([inp.text_cond, inp.text_uncond])).cuda()
    vel = torch.empty_like(lat)
    dump = torch.empty((L + 1, 2, S, D), dtype=torch.bfloat16, device="cuda")
    m.moss_dit_forward(lat, txt, [0.5, 0.5], vel, skip_mask=[0, 1 << 1], residual_dump=dump)
    torch.cuda.synchronize()
    d = host_bits(dump)
    np.testing.assert_array_equal(d[2, 1], d[1, 1])     # sample 1 skips block 1: unchanged
    assert not np.array_equal(d[2, 0], d[1, 0])
    # the embedding rows: text cast and patch embedding
    x0 = O.embed(inp.latents[0].astype(np.float64), inp.text_cond[0].astype(np.float64), W, ocfg, mirror=True)
    assert rel_l2(O.from_bf16_bits(d[0, 0]), x0) <= 1e-2
