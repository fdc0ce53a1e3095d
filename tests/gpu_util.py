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
