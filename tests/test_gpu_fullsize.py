"""Parity at the full sizes, in the launch configuration the benchmark times.

* One full joint block: hidden 3072, 24 heads x 128, FFN 8192, batch 2, 256 text + 4096 image tokens
  (64 x 64 grid), bf16 weights ~N(0, 0.02), bf16 activations ~N(0, 1), per-sample modulation from
  sigma ~U(0, 1). Every stage is checked on sampled rows against the oracle run on the GPU's own
  previous stage (identical inputs), and the whole block against the oracle from the same input.
* The full 42-block forward at 1024^2 (batch 2, the unconditional row skipping block 22), weights
  from the benchmark's seeded draw: the residual stream is dumped after every block and blocks
  0, 21, 22 and 41 are recomputed by the oracle on sampled rows from the GPU's input to that block;
  the embedding and the final layer + unpatchify are checked in full.
* The largest batch (8 samples at 1024^2, each with its own sigma, prompt and skip set) equals eight
  one-sample forwards bit for bit.
* Whole sampling steps at the benchmark's shapes (the three-pass skip-layer guidance step at 1024^2,
  three rows; a step at 2048^2 with a 4096-token prompt): the step equals the guidance combine of the
  library's own batched forward (rows are computed independently, so the step's rows and the
  forward's rows are the same numbers) up to fp32 rounding.

The oracle computes a sampled row exactly: its keys and values come from every row of the sequence.
"""
import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_util import (REL_L2_BF16, REL_L2_FP32, dev_bf16, forward_block_chain, host_bf16, host_bits, log,
                            oracle_cfg, rel_l2)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
dt = pytest.importorskip("diffusion_transformer_text_amd")

T, GH, GW = 256, 64, 64
S = T + GH * GW


def sample_rows(rng, n=20, T=T, GW=GW, S=S):
    return np.unique(np.concatenate([rng.integers(0, S, n), [0, T - 1, T, T + GW, S - 1]]))


def block_model(mod_scale, seed=3):
    shape = synth.Shape(num_layers=1)
    w = synth.torch_weights(shape, seed=seed, device="cuda", mod_scale=mod_scale)
    cfg = dt.moss_dit_config_init(num_layers=1)
    return dt.MossDiT(cfg, w), w, oracle_cfg(cfg)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mod_scale,T,GH,GW", [(1.0, T, GH, GW), (50.0, T, GH, GW), (50.0, 4096, 128, 128),
                                               (50.0, 256, 64, 128)])
def test_full_block_sampled_rows(mod_scale, T, GH, GW):
    """One joint block at full width, stage by stage and whole. The 2048^2 case (4096 text + 16384
    image tokens, S = 20480, M = 40960 rows per GEMM) is the sampling benchmark's block shape; the
    1024 x 2048 case (a 64 x 128 patch grid, S = 8448) puts the rotary rows and columns on a
    non-square grid at full width, with the attention's key-split tail on (2 x 24 x 66 query tiles
    leave 96 for the last round)."""
    S = T + GH * GW
    log(f"full block: D=3072 F=8192 H=24, B=2, S={S}, mod_scale={mod_scale}")
    model, w, ocfg = block_model(mod_scale)
    D, F = ocfg.hidden, ocfg.ffn_hidden
    rng = np.random.default_rng(11)
    B = 2
    xbits = synth.bf16_normal_bits(rng, (B, S, D))
    sig = synth.uniform_f32(rng, (B,))
    x = dev_bf16(xbits, torch)
    mod = torch.empty((B, model.mod_stride), dtype=torch.bfloat16, device="cuda")
    model.moss_dit_modulation([float(s) for s in sig], mod)
    M = B * S
    taps = {k: torch.empty((M, n), dtype=dt_, device="cuda") for k, n, dt_ in
            [("a", D, torch.bfloat16), ("qkv", 3 * D, torch.bfloat16), ("o", D, torch.bfloat16),
             ("attn", D, torch.float32), ("x1", D, torch.bfloat16), ("a2", D, torch.bfloat16),
             ("h", F, torch.bfloat16), ("ffn", D, torch.float32)]}
    model.moss_dit_block(0, x, T, GH, GW, mod, taps=taps)
    torch.cuda.synchronize()
    W = {"qkv_w": [host_bf16(w["qkv_w"][0])], "out_w": [host_bf16(w["out_w"][0])],
         "gate_up_w": [host_bf16(w["gate_up_w"][0])], "down_w": [host_bf16(w["down_w"][0])],
         "t_w1": host_bf16(w["t_w1"]), "t_w2": host_bf16(w["t_w2"]), "mod_w": [host_bf16(w["mod_w"][0])],
         "final_mod_w": host_bf16(w["final_mod_w"])}
    modv = host_bf16(mod)
    x_out = host_bf16(x).reshape(B, S, D)
    g = {k: (host_bf16(v) if v.dtype == torch.bfloat16 else v.cpu().numpy().astype(np.float64)).reshape(B, S, -1)
         for k, v in taps.items()}
    x0 = O.from_bf16_bits(xbits)
    errs = {}
    for b in range(B):
        m_ref, mf_ref = O.modulation(float(sig[b]), W, ocfg, mirror=True)
        errs.setdefault("modulation", []).append(rel_l2(modv[b], np.concatenate([m_ref.reshape(-1), mf_ref.reshape(-1)])))
        mb = modv[b, :6 * D].reshape(6, D)
        rows = sample_rows(rng, T=T, GW=GW, S=S)
        a_ref = O.bf16_round(O.ln_modulate(x0[b][rows], mb[0], mb[1], 1e-6))
        errs.setdefault("ln1", []).append(rel_l2(g["a"][b][rows], a_ref))
        # qkv + RoPE from the GPU's own LN output
        qkv = O.bf16_round(g["a"][b][rows] @ W["qkv_w"][0].T)
        q = O.bf16_round(O.rope_rows(qkv[:, :D], T, GW, 128, 1e4, rows=rows))
        k = O.bf16_round(O.rope_rows(qkv[:, D:2 * D], T, GW, 128, 1e4, rows=rows))
        errs.setdefault("qkv_rope", []).append(rel_l2(g["qkv"][b][rows], np.concatenate([q, k, qkv[:, 2 * D:]], 1)))
        # attention of sampled queries over every key/value row of the GPU's qkv
        gq = g["qkv"][b]
        errs.setdefault("attention", []).append(
            rel_l2(g["o"][b][rows], O.attention(gq[rows, :D], gq[:, D:2 * D], gq[:, 2 * D:], 24, 128)))
        errs.setdefault("out_proj", []).append(rel_l2(g["attn"][b][rows], g["o"][b][rows] @ W["out_w"][0].T))
        errs.setdefault("gated_res1", []).append(rel_l2(g["x1"][b][rows], O.bf16_round(x0[b][rows] + mb[2] * g["attn"][b][rows])))
        errs.setdefault("ln2", []).append(rel_l2(g["a2"][b][rows], O.bf16_round(O.ln_modulate(g["x1"][b][rows], mb[3], mb[4], 1e-6))))
        gu = g["a2"][b][rows] @ W["gate_up_w"][0].T
        errs.setdefault("swiglu", []).append(rel_l2(g["h"][b][rows], O.bf16_round(O.silu(gu[:, :F]) * gu[:, F:])))
        errs.setdefault("down_proj", []).append(rel_l2(g["ffn"][b][rows], g["h"][b][rows] @ W["down_w"][0].T))
        # the whole block from the same input
        taps_o = {}
        ref = O.block(x0[b], mb, W, 0, ocfg, T, GW, mirror=True, rows=rows, taps=taps_o)
        errs.setdefault("block", []).append(rel_l2(x_out[b][rows], ref))
        errs.setdefault("attn_branch", []).append(rel_l2(g["attn"][b][rows], taps_o["attn_out"]))
        errs.setdefault("ffn_branch", []).append(rel_l2(g["ffn"][b][rows], taps_o["ffn_out"]))
        errs.setdefault("block_update", []).append(rel_l2(x_out[b][rows] - x0[b][rows], ref - x0[b][rows]))
    log({k: f"{max(v):.2e}" for k, v in errs.items()})
    model.close()
    for k, v in errs.items():
        if k in ("out_proj", "down_proj"):
            assert max(v) <= 1e-5, (k, v)
        elif k == "block_update" and mod_scale == 1.0:
            continue      # the literal-init update is mostly bf16 rounding of the residual (see the 50x run)
        else:
            assert max(v) <= REL_L2_BF16, (k, v)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mod_scale", [1.0, 50.0])
def test_full_forward_1024_block_chain(mod_scale):
    """The full 42-block forward at 1024^2 (batch 2, the unconditional row skipping block 22), with the
    literal N(0, 0.02) weights and with the modulation weights x50. Blocks 0, 21 (the last block before
    the skip), 22 (run on the conditional row alone: M = 4352) and 41 (the last modulation offset) are
    re-run from the forward's own residual dump with branch taps (tests/gpu_util.forward_block_chain):
    bitwise equal to the forward's block, gated residual adds recomputed from the taps, and branch
    outputs, block output and (x50) block update against the oracle on sampled rows. The modulation of
    all 42 blocks, the embedding and the final layer + unpatchify are checked against the oracle too."""
    log(f"full forward 1024^2: 42 blocks, B=2 (uncond skips block 22), T=256, mod_scale={mod_scale}")
    L, D = 42, 3072
    w = synth.torch_weights(synth.FULL, seed=0, device="cuda", mod_scale=mod_scale)
    cfg = dt.moss_dit_config_init()
    model = dt.MossDiT(cfg, w)
    ocfg = oracle_cfg(cfg)
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    text_cond = torch.randn((1, T, D), generator=g, device="cuda", dtype=torch.float32)
    lat1 = torch.randn((1, 32, 128, 128), generator=g, device="cuda", dtype=torch.float32)
    lat = torch.cat([lat1, lat1]).contiguous()
    text = torch.cat([text_cond, torch.zeros_like(text_cond)]).contiguous()
    vel = torch.empty_like(lat)
    dump = torch.empty((L + 1, 2, S, D), dtype=torch.bfloat16, device="cuda")
    model.moss_dit_forward(lat, text, [0.5, 0.5], vel, skip_mask=[0, 1 << 22], residual_dump=dump)
    torch.cuda.synchronize()
    assert torch.isfinite(vel).all().item()
    # run-to-run determinism at full size, and the residual dump does not change the result
    vel2 = torch.full_like(lat, float("nan"))
    model.moss_dit_forward(lat, text, [0.5, 0.5], vel2, skip_mask=[0, 1 << 22])
    torch.cuda.synchronize()
    assert torch.equal(vel, vel2)
    # the skipped block leaves the unconditional row bit for bit unchanged
    assert torch.equal(dump[23, 1], dump[22, 1])
    assert not torch.equal(dump[23, 0], dump[22, 0])
    rng = np.random.default_rng(5)
    Wsmall = {"t_w1": host_bf16(w["t_w1"]), "t_w2": host_bf16(w["t_w2"]), "x_embed_w": host_bf16(w["x_embed_w"]),
              "final_mod_w": host_bf16(w["final_mod_w"]), "final_w": host_bf16(w["final_w"])}
    layers = [0, 21, 22, 41]
    W = dict(Wsmall)
    for k in ("mod_w", "qkv_w", "out_w", "gate_up_w", "down_w"):
        W[k] = [host_bf16(w[k][l]) if l in layers else np.zeros((1, 1)) for l in range(L)]
    W["mod_w"] = [host_bf16(w["mod_w"][l]) for l in range(L)]
    m, mf = O.modulation(0.5, W, ocfg, mirror=True)
    errs = {}
    # the modulation the forward used, every block's offset, against the oracle
    mod = torch.empty((2, model.mod_stride), dtype=torch.bfloat16, device="cuda")
    model.moss_dit_modulation([0.5, 0.5], mod)
    torch.cuda.synchronize()
    modv = host_bf16(mod)
    mref = np.concatenate([m.reshape(-1), mf.reshape(-1)])
    errs["modulation"] = max(rel_l2(modv[b], mref) for b in range(2))
    # embedding: text cast + patch embedding of sample 0
    x0_ref = O.embed(lat1[0].double().cpu().numpy(), text_cond[0].double().cpu().numpy(), W, ocfg, mirror=True)
    errs["embed"] = rel_l2(host_bf16(dump[0, 0]), x0_ref)
    rows = {(l, b): sample_rows(rng, 12) for l in layers for b in range(2)}
    runs = [(l, [0] if l == 22 else [0, 1]) for l in layers]
    chain, mism = forward_block_chain(model, torch, dump, mod, runs, T, GH, GW, W, ocfg, [m, m],
                                      lambda l, b: rows[(l, b)])
    # final layer + unpatchify of both samples from the GPU's last residual
    v = vel.cpu().numpy()
    for b in range(2):
        xl = host_bf16(dump[L, b])
        y = O.final_layer(xl[T:], mf, W, ocfg, mirror=True)
        errs[f"final_s{b}"] = rel_l2(v[b], O.unpatchify(y, 32, 128, 128))
    log({k: f"{e:.2e}" for k, e in errs.items()})
    log({k: [f"{x:.2e}" for x in e] for k, e in {**chain, **mism}.items()})
    model.close()
    for k, e in errs.items():
        assert e <= REL_L2_BF16, (k, e)
    for k in ("attn_branch", "ffn_branch", "block"):
        assert max(chain[k]) <= REL_L2_BF16, (k, chain[k])
    if mod_scale != 1.0:       # literal init: the update is mostly bf16 rounding (see forward_block_chain)
        assert max(chain["update"]) <= REL_L2_BF16, chain["update"]
    assert max(mism["gated_res"]) <= 1e-3, mism


@pytest.mark.timeout(600)
def test_full_forward_batch_8_equals_single_samples():
    """The largest batch: 8 samples at 1024^2 (M = 34816 rows per GEMM) with their own latents, prompts,
    sigmas and skip sets equal eight one-sample forwards bit for bit, so the batched launches, the
    per-sample modulation offsets and the runs of samples that a skip set cuts all hold at full size.
    Every kernel computes a row the same whatever rows run beside it; the attention's key split is the
    one batch-dependent choice, and with 816 query tiles per sample on 512 slots none is made in runs
    of 1, 3, 5, 6 or 8 samples, the only run lengths these skip sets leave in any block."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the run lengths are chosen for 256 compute units (512 attention slots)")
    D, B = 3072, 8
    log("full forward 1024^2, batch 8 vs single samples")
    w = synth.torch_weights(synth.FULL, seed=0, device="cuda")
    model = dt.MossDiT(dt.moss_dit_config_init(), w)
    g = torch.Generator(device="cuda")
    g.manual_seed(21)
    lat = torch.randn((B, 32, 128, 128), generator=g, device="cuda", dtype=torch.float32)
    text = torch.randn((B, T, D), generator=g, device="cuda", dtype=torch.float32)
    sig = [0.05 + 0.12 * b for b in range(B)]
    # block 0: samples 1, 2 skip (runs of 1 and 5); block 10: 1, 7 (1 and 5); block 22: 1 (1 and 6);
    # block 41: 6 (6 and 1); every other block: one run of 8
    skips = [0, (1 << 22) | (1 << 10) | 1, 1, 0, 0, 0, 1 << 41, 1 << 10]
    vel = torch.full_like(lat, float("nan"))
    model.moss_dit_forward(lat, text, sig, vel, skip_mask=skips)
    torch.cuda.synchronize()
    assert torch.isfinite(vel).all().item()
    for b in range(B):
        v1 = torch.full_like(lat[b:b + 1], float("nan"))
        model.moss_dit_forward(lat[b:b + 1].contiguous(), text[b:b + 1].contiguous(), [sig[b]], v1,
                               skip_mask=[skips[b]])
        torch.cuda.synchronize()
        assert torch.equal(vel[b:b + 1], v1), b
    model.close()


def _step_vs_forward(model, T, side, step, slg_scale, seed):
    D = 3072
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    tc = torch.randn((1, T, D), generator=g, device="cuda", dtype=torch.float32)
    tu = torch.zeros_like(tc)
    x0 = torch.randn((1, 32, side, side), generator=g, device="cuda", dtype=torch.float32)
    sig = dt.moss_sigmas(50, 5.0)
    x = x0.clone()
    model.moss_sample_step(x, tc, tu, sig, step, cfg_scale=3.0, uncond_skip_layers=[22], slg_scale=slg_scale)
    rows = 3 if slg_scale > 0 else 2
    lat = torch.cat([x0] * rows).contiguous()
    txt = torch.cat([tc, tu, tc][:rows]).contiguous()
    vel = torch.empty_like(lat)
    skip = [0, 1 << 22, 1 << 22][:rows]
    model.moss_dit_forward(lat, txt, [float(sig[step])] * rows, vel, skip_mask=skip)
    torch.cuda.synchronize()
    assert torch.isfinite(x).all().item() and torch.isfinite(vel).all().item()
    v = vel.cpu().numpy().astype(np.float64)
    guided = v[1:2] + 3.0 * (v[0:1] - v[1:2])
    if rows == 3:
        guided = guided + slg_scale * (v[0:1] - v[2:3])
    x_ref = x0.cpu().numpy().astype(np.float64) + float(sig[step + 1] - sig[step]) * guided
    d_got = x.cpu().numpy().astype(np.float64) - x0.cpu().numpy()
    d_ref = x_ref - x0.cpu().numpy()
    return rel_l2(d_got, d_ref)


@pytest.mark.timeout(600)
def test_three_pass_step_1024_and_step_2048():
    w = synth.torch_weights(synth.FULL, seed=0, device="cuda")
    model = dt.MossDiT(dt.moss_dit_config_init(), w)
    log("three-pass SLG step at 1024^2 (rows: cond, uncond skipping 22, cond skipping 22)")
    e3 = _step_vs_forward(model, 256, 128, 5, 2.5, seed=7)
    log(f"  update vs forward-based combine: rel-L2 {e3:.2e}")
    log("step at 2048^2 with 4096 text tokens (S = 20480)")
    e2 = _step_vs_forward(model, 4096, 256, 5, 0.0, seed=8)
    log(f"  update vs forward-based combine: rel-L2 {e2:.2e}")
    model.close()
    assert e3 <= REL_L2_FP32 and e2 <= REL_L2_FP32
