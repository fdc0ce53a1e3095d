"""Helpers of the GPU parity tests: moving bf16 bit patterns between numpy and torch, error metrics."""
import sys

import numpy as np

import oracle as O

REL_L2_BF16 = 2e-2      # bf16 block / forward outputs against the oracle
REL_L2_FP32 = 1e-5      # FP32 guidance / scheduler arithmetic on identical inputs


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def dev_bf16(bits, torch):
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 tensor on the GPU."""
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def host_bf16(t) -> np.ndarray:
    """torch.bfloat16 tensor -> float64 numpy values."""
    import torch
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return O.from_bf16_bits(bits)


def host_bits(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev_weights(w, torch):
    """synth.Weights (bit patterns) -> dict of device bf16 tensors with the C struct's field names."""
    d = {}
    for k in ("t_w1", "t_w2", "x_embed_w", "final_mod_w", "final_w"):
        d[k] = dev_bf16(getattr(w, k), torch)
    for k in ("mod_w", "qkv_w", "out_w", "gate_up_w", "down_w"):
        d[k] = [dev_bf16(a, torch) for a in getattr(w, k)]
    return d


def oracle_weights_from_device(d, layers=None) -> dict:
    """Device weight dict -> float64 dict for the oracle (optionally only some blocks)."""
    out = {k: host_bf16(d[k]) for k in ("t_w1", "t_w2", "x_embed_w", "final_mod_w", "final_w")}
    n = len(d["qkv_w"])
    for k in ("mod_w", "qkv_w", "out_w", "gate_up_w", "down_w"):
        out[k] = [host_bf16(d[k][l]) if (layers is None or l in layers) else None for l in range(n)]
    return out


def oracle_cfg(cfg) -> O.Config:
    return O.Config(num_layers=cfg.num_layers, hidden=cfg.hidden, num_heads=cfg.num_heads, head_dim=cfg.head_dim,
                    ffn_hidden=cfg.ffn_hidden, latent_channels=cfg.latent_channels, patch=cfg.patch,
                    temb_dim=cfg.temb_dim, text_dim=cfg.text_dim, refiner_layers=cfg.refiner_layers,
                    gemm_precision="mxfp8" if cfg.gemm_precision == 1 else "bf16",
                    attention_mode="q8" if cfg.attention_mode == 1 else "exact")


def bf16_ulp(x) -> np.ndarray:
    """One unit in the last place of bf16 values x (8 significant bits), for |x| in the normal range."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(x > 0, x, 1.0)))
    return np.where(x > 0, 2.0 ** (e - 7), 2.0 ** -133)


def residual_add_mismatch(x_new, x_old, gate, branch):
    """A gated residual add x_new = bf16(x_old + gate * branch), recomputed on the host from the GPU's own
    fp32 branch output and bf16 gate: (fraction of elements that differ, largest difference in units of
    x_new's bf16 ulp). The GPU adds in fp32 and rounds once to bf16, so a difference can only come from
    an fp32 rounding that lands next to a bf16 rounding boundary: about 2^-16 of the elements, one ulp."""
    ref = O.bf16_round(x_old + gate * branch)
    d = np.abs(x_new - ref)
    frac = float(np.mean(d > 0))
    ulps = float(np.max(d / np.maximum(bf16_ulp(ref), bf16_ulp(x_new)))) if frac > 0 else 0.0
    return frac, ulps


def forward_block_chain(model, torch, dump, mod, runs, T, gh, gw, W, ocfg, m_ref, rows_of):
    """Parity of single blocks inside one forward pass, from the GPU's own input to each block.

    dump: the forward's residual stream after the embedding and after every block, bf16 [L + 1, B, S, D]
    on the device; mod: the forward's modulation, bf16 [B, mod_stride] (moss_dit_modulation at the same
    sigmas); runs: [(l, [samples that ran block l])]; m_ref[b]: the oracle's [L, 6, D] modulation of
    sample b; rows_of(l, b): the rows to compare.

    Block l is re-run on dump[l] through moss_dit_block (the samples that ran it, i.e. the same row count
    as in the forward) with taps of its two fp32 branch outputs and its intermediate residual. Checked:
    * the re-run's output equals dump[l + 1] bit for bit (so the taps are those of the forward's block);
    * both gated residual adds, recomputed on the host from the taps and the GPU's modulation at block
      l's offset (a wrong gate or layer offset changes most elements; a correct one at most ~1e-4 of
      them, by one bf16 ulp);
    * against the oracle's block from the same input on the sampled rows: the attention and FFN branch
      outputs (before the residual add; their size does not depend on the gates, so they are sensitive
      under the literal init too), the block output and the block's update x_{l+1} - x_l.
    Returns {name: [errors]} and {name: [residual-add mismatch fractions]}."""
    D = ocfg.hidden
    errs, mism = {}, {}
    for l, samples in runs:
        nb = len(samples)
        idx = torch.tensor(samples, device=dump.device)
        x = dump[l].index_select(0, idx).contiguous()
        x_next = dump[l + 1].index_select(0, idx)
        msel = mod.index_select(0, idx).contiguous()
        M = nb * x.shape[1]
        taps = {"attn": torch.empty((M, D), dtype=torch.float32, device=x.device),
                "x1": torch.empty((M, D), dtype=torch.bfloat16, device=x.device),
                "ffn": torch.empty((M, D), dtype=torch.float32, device=x.device)}
        model.moss_dit_block(l, x, T, gh, gw, msel, taps=taps)
        torch.cuda.synchronize()
        assert torch.equal(x, x_next), f"block {l}: the re-run differs from the forward's block"
        S = x.shape[1]
        attn = taps["attn"].cpu().numpy().astype(np.float64).reshape(nb, S, D)
        ffn = taps["ffn"].cpu().numpy().astype(np.float64).reshape(nb, S, D)
        x1 = host_bf16(taps["x1"]).reshape(nb, S, D)
        xo = host_bf16(x).reshape(nb, S, D)
        mv = host_bf16(msel)
        for j, b in enumerate(samples):
            xin = host_bf16(dump[l, b])
            mb = mv[j, l * 6 * D:(l + 1) * 6 * D].reshape(6, D)
            f1, u1 = residual_add_mismatch(x1[j], xin, mb[2], attn[j])
            f2, u2 = residual_add_mismatch(xo[j], x1[j], mb[5], ffn[j])
            mism.setdefault("gated_res", []).append(max(f1, f2))
            assert max(u1, u2) <= 1.0, (l, b, u1, u2)
            rows = rows_of(l, b)
            taps_o = {}
            ref = O.block(xin, m_ref[b][l], W, l, ocfg, T, gw, mirror=True, rows=rows, taps=taps_o)
            errs.setdefault("attn_branch", []).append(rel_l2(attn[j][rows], taps_o["attn_out"]))
            errs.setdefault("ffn_branch", []).append(rel_l2(ffn[j][rows], taps_o["ffn_out"]))
            errs.setdefault("block", []).append(rel_l2(xo[j][rows], ref))
            errs.setdefault("update", []).append(rel_l2(xo[j][rows] - xin[rows], ref - xin[rows]))
        del taps, x
    return errs, mism
