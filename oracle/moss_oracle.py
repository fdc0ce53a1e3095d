"""CPU oracle of one MOSS-Image denoising step (single-stream DiT + FP32 CFG/SLG + Euler).

TEST INFRASTRUCTURE ONLY. Only the test-suite, the package's smoke check and the benchmark's
``cpu_baseline`` leg may import this module. The product path never calls it and shares no code with
it: this file imports nothing but numpy.

Plain, slow and obviously correct: numpy float64, one step of the method after another, in the
pages' order and notation. A library matmul/exp serves as a step; nothing is blocked, fused or
reordered. ``mirror_bf16=True`` rounds (float64 -> float32 -> bfloat16, round-to-nearest-even) at the
points where a bf16 DiT stores a tensor between operations; everything else stays float64.

Pages (titles as published):
  [SG]  "MOSS-Image" -- SGLang diffusion cookbook, section 3 "Guidance and precision".
  [WP]  "MOSS-Image: specs, settings, VRAM and text rendering tested" -- sections "Architecture and
        specs" and "Recommended settings".
  [IV]  InvokeAI user guide "MOSS-Image" -- sections "Transformer formats", "Generation settings",
        "Skip layers".
  [QI]  "Qwen-Image 2.1" -- SGLang cookbook, sections "Lossless RoPE fusion", "Lossless MLP and
        residual fusion", "Lossless LayerNorm modulation" (fused-op idioms of a single-stream DiT).
  [MI]  "MossInfer integration guide" -- the feature table (rows "Generation", "Lossy accelerators")
        and its list of opt-in accelerators (CFG truncation).

Where the pages leave a step open the plainest reading is taken; each such reading is named at the
function that makes it. Pins: every function here is checked in tests/test_oracle_pins.py against
closed forms, hand values, library routines, invariants and an independent scalar brute force.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Set

import numpy as np


# ----------------------------------------------------------------------------------------------
# numbers and rounding
# ----------------------------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """float64 -> float32 (RNE) -> bfloat16 (RNE), returned as float64 values.

    The bf16 DiT keeps weights and activations in bfloat16 while latents, guidance and the scheduler
    stay float32 ([SG] "Guidance and precision")."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    out = r.astype(np.uint32).view(np.float32).astype(np.float64)
    return np.where(np.isnan(x32), np.nan, out)


def from_bf16_bits(bits) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _store(x, mirror: bool):
    return bf16_round(x) if mirror else np.asarray(x, dtype=np.float64)


def silu(x):
    return x / (1.0 + np.exp(-x))


# ----------------------------------------------------------------------------------------------
# configuration
# ----------------------------------------------------------------------------------------------

@dataclass(frozen=True)
class Config:
    """[WP] "Architecture and specs": 42 joint blocks, hidden 3072, 24 heads of 128, FFN 8192,
    32 latent channels, 2x2 latent patches, two text-only blocks after the text projection. temb_dim,
    rope_theta, norm_eps, flow_multiplier and text_dim (the encoder's state width) are readings (the
    pages do not give them)."""
    num_layers: int = 42
    hidden: int = 3072
    num_heads: int = 24
    head_dim: int = 128
    ffn_hidden: int = 8192
    latent_channels: int = 32
    patch: int = 2
    temb_dim: int = 256
    rope_theta: float = 1.0e4
    norm_eps: float = 1.0e-6
    flow_multiplier: float = 1000.0
    text_dim: int = 4096
    refiner_layers: int = 2
    gemm_precision: str = "bf16"        # "bf16", or "mxfp8" for the FP8 tier of the block projections
    attention_mode: str = "exact"       # "exact", or "q8" for the 8-bit attention of the FP8 tier

    @property
    def patch_dim(self) -> int:
        return self.latent_channels * self.patch * self.patch


# ----------------------------------------------------------------------------------------------
# A1  sigma schedule and skip-layer-guidance window
# ----------------------------------------------------------------------------------------------

def sigmas(num_steps: int, shift: float = 5.0) -> np.ndarray:
    """Flow-matching Euler schedule with shift ([SG] "Guidance and precision": 50 steps, flow shift 5;
    [IV] "Generation settings": the model's own Euler schedule).

    s_i = (N - i)/N for i = 0..N, sigma_i = shift*s_i / (1 + (shift-1)*s_i); sigma_0 = 1, sigma_N = 0.
    Reading: the grid is uniform in s and computed as a ratio, not by accumulating a step."""
    if num_steps < 1:
        raise ValueError("num_steps must be >= 1")
    s = np.array([(num_steps - i) / num_steps for i in range(num_steps + 1)], dtype=np.float64)
    return shift * s / (1.0 + (shift - 1.0) * s)


def slg_active(step: int, num_steps: int, slg_start: float = 0.01, slg_stop: float = 1.0) -> bool:
    """Whether the unconditional pass skips its layers at this step ([SG] "Guidance and precision":
    the window slg_start=0.01 .. slg_stop=1.0 leaves the first step at full CFG; slg_start=0.0 starts
    at zero). Reading: progress p = step/num_steps, inclusive at both ends."""
    p = step / num_steps
    return slg_start <= p <= slg_stop


# ----------------------------------------------------------------------------------------------
# A2  timestep embedding and modulation
# ----------------------------------------------------------------------------------------------

def time_features(sigma: float, cfg: Config) -> np.ndarray:
    """Sinusoidal features of t = flow_multiplier*sigma: e = [cos(t f_k) | sin(t f_k)], k = 0..127,
    f_k = exp(-ln(1e4) k / 128). Reading (the pages name a flow multiplier but no embedding)."""
    half = cfg.temb_dim // 2
    t = cfg.flow_multiplier * float(sigma)
    f = np.exp(-math.log(1.0e4) * np.arange(half, dtype=np.float64) / half)
    return np.concatenate([np.cos(t * f), np.sin(t * f)])


def modulation(sigma: float, W: Dict, cfg: Config, mirror: bool = False):
    """Time MLP and per-block modulation ([IV] "Transformer formats" lists the time-embedding and
    modulation layers). Reading: temb = W_t2 SiLU(W_t1 e), u = SiLU(temb); block l gets
    m_l = W_mod,l u = (shift1, scale1, gate1, shift2, scale2, gate2), each of size D; the final layer
    gets m_f = W_fmod u = (shift_f, scale_f). No biases anywhere (the pages mention none).

    Returns (m [L, 6, D], m_f [2, D])."""
    D = cfg.hidden
    e = _store(time_features(sigma, cfg), mirror)
    a1 = _store(silu(W["t_w1"] @ e), mirror)
    temb = _store(W["t_w2"] @ a1, mirror)
    u = _store(silu(temb), mirror)
    m = np.stack([_store(W["mod_w"][l] @ u, mirror).reshape(6, D) for l in range(cfg.num_layers)])
    m_f = _store(W["final_mod_w"] @ u, mirror).reshape(2, D)
    return m, m_f


# ----------------------------------------------------------------------------------------------
# A3 / A11  patchify, unpatchify
# ----------------------------------------------------------------------------------------------

def patchify(latent: np.ndarray, p: int = 2) -> np.ndarray:
    """[C, h, w] -> [N, C*p*p]: 2x2 latent patches, one token per 16x16 pixels ([WP] "Architecture and
    specs"). Token n = r*(w/p) + c for grid cell (r, c), row-major; feature j = ch*p*p + dy*p + dx
    holds latent[ch, p*r+dy, p*c+dx] (reading: channel-major within a patch)."""
    C, h, w = latent.shape
    gh, gw = h // p, w // p
    out = np.zeros((gh * gw, C * p * p), dtype=np.float64)
    for r in range(gh):
        for c in range(gw):
            n = r * gw + c
            for ch in range(C):
                for dy in range(p):
                    for dx in range(p):
                        out[n, ch * p * p + dy * p + dx] = latent[ch, p * r + dy, p * c + dx]
    return out


def unpatchify(tokens: np.ndarray, C: int, h: int, w: int, p: int = 2) -> np.ndarray:
    """Inverse of :func:`patchify`: [N, C*p*p] -> [C, h, w]."""
    gw = w // p
    out = np.zeros((C, h, w), dtype=np.float64)
    for n in range(tokens.shape[0]):
        r, c = divmod(n, gw)
        for ch in range(C):
            for dy in range(p):
                for dx in range(p):
                    out[ch, p * r + dy, p * c + dx] = tokens[n, ch * p * p + dy * p + dx]
    return out


# ----------------------------------------------------------------------------------------------
# A4 / A8  LayerNorm + modulation
# ----------------------------------------------------------------------------------------------

def layernorm(x: np.ndarray, eps: float) -> np.ndarray:
    """Affine-free LayerNorm over the last axis: (x - mean) / sqrt(var + eps), population variance
    ([QI] "Lossless LayerNorm modulation" describes this affine-free form)."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def ln_modulate(x: np.ndarray, shift: np.ndarray, scale: np.ndarray, eps: float) -> np.ndarray:
    """LN(x) * (1 + scale) + shift."""
    return layernorm(x, eps) * (1.0 + scale) + shift


# ----------------------------------------------------------------------------------------------
# RoPE (inside A6)
# ----------------------------------------------------------------------------------------------

def rope_angles(pos_r: int, pos_c: int, head_dim: int, theta: float) -> np.ndarray:
    """Angles of the 2-D axial rotary embedding for image token (pos_r, pos_c): dims [0, d/2) use the
    grid row, dims [d/2, d) the grid column; within each half, pair (2k, 2k+1), k = 0..d/4-1, turns by
    pos * theta^(-k/(d/4)). Reading (the pages name a complex rotary multiplication, [QI] "Lossless
    RoPE fusion", and the attention workload ropes image positions of a 64x64 grid)."""
    quarter = head_dim // 4
    k = np.arange(quarter, dtype=np.float64)
    inv = theta ** (-k / quarter)
    return np.concatenate([pos_r * inv, pos_c * inv])          # [d/2] angles, pair index order


def apply_rope(v: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Rotate interleaved pairs (v[2k], v[2k+1]) by angles[k]."""
    out = v.astype(np.float64).copy()
    a = v[..., 0::2]
    b = v[..., 1::2]
    cs, sn = np.cos(angles), np.sin(angles)
    out[..., 0::2] = a * cs - b * sn
    out[..., 1::2] = a * sn + b * cs
    return out


def rope_rows(x: np.ndarray, text_len: int, grid_w: int, head_dim: int, theta: float,
              rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Apply RoPE per head to the image rows of x [S, H*d]; text rows (the first text_len) stay as
    they are. ``rows`` gives the sequence index of each row of x (default: 0..S-1)."""
    S, HD = x.shape
    H = HD // head_dim
    rows = range(S) if rows is None else rows
    out = x.astype(np.float64).copy()
    for i, s in enumerate(rows):
        if s < text_len:
            continue
        pr, pc = divmod(s - text_len, grid_w)
        ang = rope_angles(pr, pc, head_dim, theta)
        for h in range(H):
            sl = slice(h * head_dim, (h + 1) * head_dim)
            out[i, sl] = apply_rope(x[i, sl], ang)
    return out


# ----------------------------------------------------------------------------------------------
# A6  attention
# ----------------------------------------------------------------------------------------------

def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, num_heads: int, head_dim: int) -> np.ndarray:
    """Exact softmax attention per head over all keys, no mask, scale 1/sqrt(d) ([WP] "Architecture
    and specs": single-stream joint blocks attend over text and image tokens together).
    q [Sq, H*d], k/v [Sk, H*d] -> [Sq, H*d]."""
    out = np.zeros((q.shape[0], num_heads * head_dim), dtype=np.float64)
    scale = 1.0 / math.sqrt(head_dim)
    for h in range(num_heads):
        sl = slice(h * head_dim, (h + 1) * head_dim)
        s = (q[:, sl] @ k[:, sl].T) * scale
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        out[:, sl] = (p @ v[:, sl]) / p.sum(axis=1, keepdims=True)
    return out


# ----------------------------------------------------------------------------------------------
# FP8 tier: OCP microscaling (MX) FP8 operands of the block projections
# ----------------------------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_round(x) -> np.ndarray:
    """Nearest OCP FP8 E4M3 value (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; subnormal step
    2^-9; largest finite 448; no infinities), round half to even, saturating at +-448. Float64 values."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, E = np.frexp(a)                                   # a = f 2^E, f in [0.5, 1)
    e = np.maximum(E - 1, -6)                            # binade exponent; subnormals share 2^-6's
    step = np.ldexp(1.0, e - 3)
    q = np.rint(a / step) * step                         # rint: half to even on the mantissa integer
    return np.sign(x) * np.minimum(q, E4M3_MAX)


def mx_quantize(x: np.ndarray, block: int = 32):
    """OCP MX block quantization along the last axis (blocks of 32): scale exponent
    floor(log2(amax)) - 8 (8 = E4M3's largest exponent), E8M0 range [-127, 127] (an all-zero block takes
    -127), elements e4m3_round(x / 2^scale). Returns (codes as float64, scale exponents)."""
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    assert K % block == 0
    xb = x.reshape(x.shape[:-1] + (K // block, block))
    amax = np.abs(xb).max(axis=-1)
    _, E = np.frexp(np.where(amax > 0, amax, 1.0))
    ex = np.where(amax > 0, E - 1 - 8, -127)
    ex = np.clip(ex, -127, 127)
    q = e4m3_round(xb * np.ldexp(1.0, -ex)[..., None])
    return q.reshape(x.shape), ex


def mx_dequantize(x: np.ndarray, block: int = 32) -> np.ndarray:
    """x -> its MXFP8 value (quantize then scale back)."""
    q, ex = mx_quantize(x, block)
    K = q.shape[-1]
    return (q.reshape(q.shape[:-1] + (K // block, block)) * np.ldexp(1.0, ex)[..., None]).reshape(q.shape)


# ----------------------------------------------------------------------------------------------
# FP8 tier: 8-bit attention (Q K^T on INT8 codes, P V on FP8 E4M3 codes)
# ----------------------------------------------------------------------------------------------
# The pages name 8-bit attention modes (q8_fp8: 8-bit Q and K, FP8 P V; fp32-accumulating variants;
# MossInfer integration guide, "Quality tier" and the feature table's attention modes) and give no
# formula. Reading, step by step below: Q symmetric INT8 per token and head, K symmetric INT8 per
# block of 64 consecutive keys and head, V FP8 E4M3 per channel (head dimension) with scale amax/448;
# the integer dot products are exact; the softmax runs online over the 64-key blocks in order, each
# query's reference max moving to a block's max only when that exceeds it by more than one unit in
# log2 (a factor 2 in probability), so every probability is <= 2 and rounds to E4M3 on the scale 224
# (<= 448); the normaliser sums the same rounded probabilities, so the output is a convex combination
# of the dequantized V rows. Codes are decided in float32 (x * 127 and x * 448 are exact for bf16
# inputs; one correctly rounded division), as the GPU decides them.

Q8_KEY_BLOCK = 64
Q8_P_SCALE = 224.0      # probabilities <= 2 -> E4M3 codes <= 448


def int8_codes(x32: np.ndarray, amax32) -> np.ndarray:
    """rint(x * 127 / amax) with float32 operations (round half to even); all-zero input gives zeros."""
    x32 = np.asarray(x32, dtype=np.float32)
    amax32 = np.asarray(amax32, dtype=np.float32)
    safe = np.where(amax32 > 0, amax32, np.float32(1.0))
    return np.rint((x32 * np.float32(127.0)) / safe).astype(np.float64)


def q8_quantize_q(q: np.ndarray):
    """Per-row INT8 of q [S, d]: codes [S, d] and the row amax [S] (dequantized q = code * amax / 127)."""
    q32 = np.asarray(q, dtype=np.float32)
    amax = np.abs(q32).max(axis=1)
    return int8_codes(q32, amax[:, None]), amax.astype(np.float64)


def q8_quantize_k(k: np.ndarray, block: int = Q8_KEY_BLOCK):
    """INT8 of k [S, d] per block of `block` consecutive rows: codes [S, d], block amax [ceil(S/block)]."""
    k32 = np.asarray(k, dtype=np.float32)
    S = k32.shape[0]
    nb = (S + block - 1) // block
    codes = np.zeros(k32.shape, dtype=np.float64)
    amax = np.zeros(nb, dtype=np.float64)
    for t in range(nb):
        blk = k32[t * block:(t + 1) * block]
        a = np.abs(blk).max()
        amax[t] = a
        codes[t * block:(t + 1) * block] = int8_codes(blk, a)
    return codes, amax


def fp8_quantize_v(v: np.ndarray):
    """Per-channel E4M3 of v [S, d]: codes e4m3_round(v * 448 / amax_channel) (float32 ops), amax [d]."""
    v32 = np.asarray(v, dtype=np.float32)
    amax = np.abs(v32).max(axis=0)
    safe = np.where(amax > 0, amax, np.float32(1.0))
    codes = e4m3_round(((v32 * np.float32(E4M3_MAX)) / safe[None, :]).astype(np.float64))
    return codes, amax.astype(np.float64)


def attention_q8(q: np.ndarray, k: np.ndarray, v: np.ndarray, num_heads: int, head_dim: int,
                 quantize_p: bool = True) -> np.ndarray:
    """8-bit attention per head (reading above). q [Sq, H*d], k/v [Sk, H*d] -> [Sq, H*d].
    quantize_p=False keeps the probabilities exact (the same online algorithm, for the pins)."""
    out = np.zeros((q.shape[0], num_heads * head_dim), dtype=np.float64)
    scale = 1.0 / math.sqrt(head_dim)
    Sk = k.shape[0]
    nb = (Sk + Q8_KEY_BLOCK - 1) // Q8_KEY_BLOCK
    for h in range(num_heads):
        sl = slice(h * head_dim, (h + 1) * head_dim)
        qc, qa = q8_quantize_q(q[:, sl])
        kc, ka = q8_quantize_k(k[:, sl])
        vc, va = fp8_quantize_v(v[:, sl])
        v_hat = vc * (va / E4M3_MAX)[None, :]
        Sq = q.shape[0]
        m = np.full(Sq, -np.inf)
        o = np.zeros((Sq, head_dim))
        l = np.zeros(Sq)
        for t in range(nb):
            ks = slice(t * Q8_KEY_BLOCK, min((t + 1) * Q8_KEY_BLOCK, Sk))
            s = (qc @ kc[ks].T) * (qa / 127.0)[:, None] * (ka[t] / 127.0) * scale
            mx = s.max(axis=1)
            with np.errstate(invalid="ignore"):
                move = ~np.isfinite(m) | ((mx - m) / math.log(2.0) > 1.0)     # more than a factor 2 above
            m_new = np.where(move, mx, m)
            alpha = np.where(np.isfinite(m), np.exp(m - m_new), 0.0)
            p = np.exp(s - m_new[:, None])                                     # <= 2
            if quantize_p:
                p = e4m3_round(p * Q8_P_SCALE) / Q8_P_SCALE
            o = o * alpha[:, None] + p @ v_hat[ks]
            l = l * alpha + p.sum(axis=1)
            m = m_new
        out[:, sl] = o / l[:, None]
    return out


def projection(a: np.ndarray, w: np.ndarray, cfg: "Config") -> np.ndarray:
    """a w^T of a block projection: bf16 operands as they are, or both operands MXFP8-quantized along
    the reduction axis (the FP8 tier)."""
    if cfg.gemm_precision == "mxfp8":
        return mx_dequantize(a) @ mx_dequantize(w).T
    return a @ w.T


# ----------------------------------------------------------------------------------------------
# A4..A10  one joint block
# ----------------------------------------------------------------------------------------------

def block(x: np.ndarray, m: np.ndarray, W: Dict, l: int, cfg: Config, text_len: int, grid_w: int,
          mirror: bool = False, rows: Optional[Sequence[int]] = None, taps: Optional[Dict] = None):
    """One single-stream joint block on one sample ([WP] "Architecture and specs").

    x [S, D] (the residual stream, bf16 values), m [6, D] = (shift1, scale1, gate1, shift2, scale2,
    gate2). Reading: pre-norm; attention branch then SwiGLU FFN branch, each gated into the residual:
        A  = LN(x)(1+scale1) + shift1;  [Q|K|V] = A W_qkv^T;  RoPE on image rows of Q, K
        x += gate1 * (softmax(Q K^T/sqrt d) V) W_o^T
        A2 = LN(x)(1+scale2) + shift2;  x += gate2 * (SiLU(A2 W_g^T) * (A2 W_u^T)) W_down^T
    with W_qkv rows [q | k | v] ([IV] "Transformer formats": a fused qkv weight splits into three)
    and W_gate_up rows [gate | up]. FFN width 8192 = 8/3 of 3072 reads as SwiGLU.

    ``rows``: compute only these output rows (K and V still use every row). Returns x' for those rows.
    ``taps``: dict that receives the branch outputs before the residual add (fp64, for tests)."""
    D, F, H, d = cfg.hidden, cfg.ffn_hidden, cfg.num_heads, cfg.head_dim
    eps, theta = cfg.norm_eps, cfg.rope_theta
    S = x.shape[0]
    rows = list(range(S)) if rows is None else list(rows)
    shift1, scale1, gate1, shift2, scale2, gate2 = m
    r = lambda t: _store(t, mirror)

    a_all = r(ln_modulate(x, shift1, scale1, eps))
    wqkv = W["qkv_w"][l]
    kv = r(projection(a_all, wqkv[D:3 * D], cfg))               # K | V for every row
    k_all = r(rope_rows(kv[:, :D], text_len, grid_w, d, theta))
    v_all = kv[:, D:]
    q = r(projection(a_all[rows], wqkv[:D], cfg))
    q = r(rope_rows(q, text_len, grid_w, d, theta, rows=rows))
    attn = attention_q8 if cfg.attention_mode == "q8" else attention
    o = r(attn(q, k_all, v_all, H, d))
    attn_out = projection(o, W["out_w"][l], cfg)
    x1 = r(x[rows] + gate1 * attn_out)
    a2 = r(ln_modulate(x1, shift2, scale2, eps))
    wgu = W["gate_up_w"][l]
    g = projection(a2, wgu[:F], cfg)
    u = projection(a2, wgu[F:], cfg)
    hf = r(silu(g) * u)
    ffn_out = projection(hf, W["down_w"][l], cfg)
    x2 = r(x1 + gate2 * ffn_out)
    if taps is not None:
        taps.update(dict(a=a_all[rows], q=q, k=k_all, v=v_all, o=o, attn_out=attn_out, x1=x1,
                         a2=a2, h=hf, ffn_out=ffn_out))
    return x2


# ----------------------------------------------------------------------------------------------
# text refiner (runs once per prompt, before the denoising loop)
# ----------------------------------------------------------------------------------------------

def text_refine(enc: np.ndarray, W: Dict, cfg: Config, mirror: bool = False) -> np.ndarray:
    """The step before the DiT on the text side ([WP] "Architecture and specs": a projection and two
    blocks over the text rows alone turn the encoder's last hidden states into the DiT's text rows).
    enc [T, text_dim] -> [T, D].

    Readings (the pages give no more): the projection is a linear map text_dim -> hidden without bias
    (no linear mentions one); the text-only blocks are joint blocks of the same widths applied to the
    text rows alone, without timestep modulation (LN(x) unmodulated, gates 1: they depend on the
    prompt only and run once per prompt), and without RoPE (text rows are never rotated)."""
    D = cfg.hidden
    x = _store(_store(enc, mirror) @ W["text_proj_w"].T, mirror)
    m = np.zeros((6, D))
    m[2] = 1.0                                            # gate1
    m[5] = 1.0                                            # gate2
    Wr = {"qkv_w": W["refiner_qkv_w"], "out_w": W["refiner_out_w"], "gate_up_w": W["refiner_gate_up_w"],
          "down_w": W["refiner_down_w"]}
    T = x.shape[0]
    for l in range(len(Wr["qkv_w"])):
        x = block(x, m, Wr, l, cfg, T, 1, mirror=mirror)   # text_len = T: no row is rotated
    return x


# ----------------------------------------------------------------------------------------------
# A3..A11  one DiT forward
# ----------------------------------------------------------------------------------------------

def embed(latent: np.ndarray, text: np.ndarray, W: Dict, cfg: Config, mirror: bool = False):
    """Sequence [text (T rows) | image tokens (N rows)] of one sample. text [T, D] stands in for the
    text refiner's output; the image tokens are patch features times W_x^T (no bias)."""
    p = _store(patchify(latent, cfg.patch), mirror)
    z = _store(p @ W["x_embed_w"].T, mirror)
    return np.concatenate([_store(text, mirror), z], axis=0)


def final_layer(x_img: np.ndarray, m_f: np.ndarray, W: Dict, cfg: Config, mirror: bool = False):
    """Image rows only: Y = (LN(x)(1+scale_f) + shift_f) W_f^T, kept in float32/64 (latents are FP32,
    [SG] "Guidance and precision"). Returns Y [N, C*p*p]."""
    shift_f, scale_f = m_f
    a = _store(ln_modulate(x_img, shift_f, scale_f, cfg.norm_eps), mirror)
    return a @ W["final_w"].T


def forward(latents: np.ndarray, text: np.ndarray, sigma: Sequence[float], W: Dict, cfg: Config,
            skip: Optional[Sequence[Set[int]]] = None, mirror: bool = False,
            taps: Optional[List] = None) -> np.ndarray:
    """DiT velocity for a batch. latents [B, C, h, w], text [B, T, D], sigma [B]; skip[b] = the
    blocks sample b leaves out ([IV] "Skip layers": the listed blocks are skipped by that pass, which
    reads as the identity on that sample's residual stream). Returns v [B, C, h, w] (float64)."""
    B, C, h, w = latents.shape
    T = text.shape[1]
    gw = w // cfg.patch
    skip = [set() for _ in range(B)] if skip is None else [set(s) for s in skip]
    out = np.zeros((B, C, h, w), dtype=np.float64)
    for b in range(B):
        m, m_f = modulation(sigma[b], W, cfg, mirror)
        x = embed(latents[b], text[b], W, cfg, mirror)
        per_layer = []
        for l in range(cfg.num_layers):
            if l in skip[b]:
                per_layer.append(None)
                continue
            x = block(x, m[l], W, l, cfg, T, gw, mirror)
            per_layer.append(x)
        y = final_layer(x[T:], m_f, W, cfg, mirror)
        out[b] = unpatchify(y, C, h, w, cfg.patch)
        if taps is not None:
            taps.append(per_layer)
    return out


# ----------------------------------------------------------------------------------------------
# A12  guidance and Euler
# ----------------------------------------------------------------------------------------------

def cfg_combine(v_cond: np.ndarray, v_uncond: Optional[np.ndarray], cfg_scale: float) -> np.ndarray:
    """Classifier-free guidance as the ordinary linear combination ([QI] "5. Runtime features" names
    it for a sibling single-stream DiT): v = v_u + cfg (v_c - v_u). CFG 1 turns guidance off and
    runs no negative pass ([IV] "Generation settings"), so v = v_c exactly; CFG < 1 is refused."""
    if cfg_scale < 1.0:
        raise ValueError("CFG scale below 1 is not accepted")
    if cfg_scale == 1.0:
        return np.asarray(v_cond, dtype=np.float64)
    return v_uncond + cfg_scale * (v_cond - v_uncond)


def euler_step(x: np.ndarray, v: np.ndarray, sigma: float, sigma_next: float) -> np.ndarray:
    """Flow-matching Euler update x_{i+1} = x_i + (sigma_{i+1} - sigma_i) v."""
    return x + (sigma_next - sigma) * v


def negative_pass_runs(step: int, num_steps: int, cfg_scale: float, cfg_truncation: float = 1.0) -> bool:
    """Whether the negative (unconditional) branch runs at this step. CFG 1 runs none ([IV]
    "Generation settings"). CFG truncation X in [0, 1] (default 1 = off): the last (1 - X) of the steps
    run without the negative branch ([MI] feature table, "Lossy accelerators", and its list of opt-in
    accelerators). Reading: with steps numbered from 0, the branch runs iff step < X*steps."""
    return cfg_scale > 1.0 and step < cfg_truncation * num_steps


def guidance_combine(v_cond: np.ndarray, v_uncond: Optional[np.ndarray], v_skip: Optional[np.ndarray],
                     cfg_scale: float, slg_scale: float) -> np.ndarray:
    """Guided velocity from up to three predictions. Without a negative branch (v_uncond None) the
    guided part is v_c, else the ordinary linear combination v_u + cfg (v_c - v_u) (see cfg_combine).
    Three-pass skip-layer guidance adds a skipped conditional prediction v_s ([SG] "3. Guidance and
    precision"; [MI] feature table lists skip-layer guidance and its scale). The pages give no formula:
    reading, the skip-layer guidance form v + slg (v_c - v_s), with v_s absent (None) meaning no term."""
    if v_uncond is None:
        v = np.asarray(v_cond, dtype=np.float64)
    else:
        v = cfg_combine(v_cond, v_uncond, cfg_scale)
    if v_skip is not None:
        v = v + slg_scale * (v_cond - v_skip)
    return v


def sample_step(x: np.ndarray, text_cond: np.ndarray, text_uncond: Optional[np.ndarray], W: Dict,
                cfg: Config, step: int, sigma_table: np.ndarray, cfg_scale: float = 3.0,
                uncond_skip_layers: Sequence[int] = (22,), slg_start: float = 0.01,
                slg_stop: float = 1.0, mirror: bool = False, velocities: Optional[List] = None,
                slg_scale: float = 0.0, cfg_truncation: float = 1.0):
    """One denoising step: DiT(cond); DiT(uncond) when the negative branch runs (CFG > 1 and not
    truncated), skipping uncond_skip_layers inside the SLG window; with slg_scale > 0 (three-pass
    skip-layer guidance) inside the same window, DiT(cond) skipping the same layers; the guidance
    combine; Euler. x [1, C, h, w]. Readings: the third pass skips the same list in the same window
    (the cookbook's advice to set uncond_skip_layers also for three-pass SLG), and it is the negative
    branch alone that CFG 1 or truncation removes."""
    N = len(sigma_table) - 1
    s, s_next = float(sigma_table[step]), float(sigma_table[step + 1])
    window = slg_active(step, N, slg_start, slg_stop)
    skip = set(uncond_skip_layers) if window else set()
    neg = negative_pass_runs(step, N, cfg_scale, cfg_truncation)
    third = slg_scale > 0.0 and len(skip) > 0
    lat, txt, sig, skips = [x], [text_cond], [s], [set()]
    if neg:
        lat.append(x), txt.append(text_uncond), sig.append(s), skips.append(skip)
    if third:
        lat.append(x), txt.append(text_cond), sig.append(s), skips.append(skip)
    vv = forward(np.concatenate(lat, axis=0), np.concatenate(txt, axis=0), sig, W, cfg, skip=skips,
                 mirror=mirror)
    v_c = vv[0:1]
    v_u = vv[1:2] if neg else None
    v_s = vv[len(lat) - 1:len(lat)] if third else None
    v = guidance_combine(v_c, v_u, v_s, cfg_scale, slg_scale)
    if velocities is not None:
        velocities.append((v_c, v_u, v_s))
    return euler_step(x, v, s, s_next)


# ----------------------------------------------------------------------------------------------
# step cache (First-Block Cache): a lossy accelerator, off by default
# ----------------------------------------------------------------------------------------------

def first_block_change(r: np.ndarray, r_prev: np.ndarray) -> float:
    """Relative mean absolute change of block 0's residual between two calls,
    sum|r - r_prev| / sum|r_prev| over every element (all rows of all samples of the call)."""
    return float(np.abs(r - r_prev).sum() / np.abs(r_prev).sum())


@dataclass
class StepCache:
    """State of the First-Block Cache across the steps of one sampling run."""
    key: Optional[tuple] = None
    r_prev: Optional[np.ndarray] = None        # block 0's residual at the last full call [B, S, D]
    rest: Optional[np.ndarray] = None          # x after the last block minus x after block 0, same call
    full_calls: int = 0
    reused_calls: int = 0
    last_change: float = float("nan")


def forward_cached(latents: np.ndarray, text: np.ndarray, sigma: Sequence[float], W: Dict, cfg: Config,
                   skip: Sequence[Set[int]], cache: StepCache, threshold: float, mirror: bool = False):
    """DiT velocity with the step cache ([MI] opt-in accelerators: as long as block 0's output moves
    less than a threshold between calls, 0.02 for the base model, blocks 1..41 are taken from the last
    call that ran them). Readings: the change is the First-Block Cache measure of block 0's
    residual r = x_after_block0 - x_before (first_block_change), one decision per call over all its
    rows; a reused call sets the stream after the last block to x_after_block0 + rest, rest = the
    difference of the same two streams at the last full call (a bf16 rounding, the residual being
    bf16); a call whose rows (batch, sequence, per-sample skip sets) differ from the cached call's runs
    in full and restarts the cache. ``cache`` is updated in place."""
    B, C, h, w = latents.shape
    T = text.shape[1]
    gw = w // cfg.patch
    skip = [set(s) for s in skip]
    mods, x0s, x1s = [], [], []
    for b in range(B):
        m, m_f = modulation(sigma[b], W, cfg, mirror)
        x = embed(latents[b], text[b], W, cfg, mirror)
        x0s.append(x)
        x1s.append(x if 0 in skip[b] else block(x, m[0], W, 0, cfg, T, gw, mirror))
        mods.append((m, m_f))
    r = np.stack(x1s) - np.stack(x0s)
    key = (B, T, h, w, tuple(frozenset(s) for s in skip))
    reuse = cache.key == key and cache.r_prev is not None
    if reuse:
        cache.last_change = first_block_change(r, cache.r_prev)
        reuse = cache.last_change < threshold
    out = np.zeros((B, C, h, w), dtype=np.float64)
    xls = []
    for b in range(B):
        m, m_f = mods[b]
        if reuse:
            x = _store(x1s[b] + cache.rest[b], mirror)
        else:
            x = x1s[b]
            for l in range(1, cfg.num_layers):
                if l not in skip[b]:
                    x = block(x, m[l], W, l, cfg, T, gw, mirror)
        xls.append(x)
        out[b] = unpatchify(final_layer(x[T:], m_f, W, cfg, mirror), C, h, w, cfg.patch)
    if reuse:
        cache.reused_calls += 1
    else:
        cache.full_calls += 1
        cache.key, cache.r_prev, cache.rest = key, r, np.stack(xls) - np.stack(x1s)
    return out


def sample_step_cached(x: np.ndarray, text_cond: np.ndarray, text_uncond: Optional[np.ndarray], W: Dict,
                       cfg: Config, step: int, sigma_table: np.ndarray, cache: StepCache, threshold: float = 0.02,
                       cfg_scale: float = 3.0, uncond_skip_layers: Sequence[int] = (22,), slg_start: float = 0.01,
                       slg_stop: float = 1.0, mirror: bool = False):
    """sample_step (two-pass recipe) with the step cache; step 0 starts a new sampling run and clears
    the cache."""
    if step == 0:
        cache.key = cache.r_prev = cache.rest = None
    N = len(sigma_table) - 1
    s, s_next = float(sigma_table[step]), float(sigma_table[step + 1])
    skip_u = set(uncond_skip_layers) if slg_active(step, N, slg_start, slg_stop) else set()
    neg = negative_pass_runs(step, N, cfg_scale)
    lat, txt, sig, skips = [x], [text_cond], [s], [set()]
    if neg:
        lat.append(x), txt.append(text_uncond), sig.append(s), skips.append(skip_u)
    vv = forward_cached(np.concatenate(lat, axis=0), np.concatenate(txt, axis=0), sig, W, cfg, skips, cache,
                        threshold, mirror=mirror)
    v = guidance_combine(vv[0:1], vv[1:2] if neg else None, None, cfg_scale, 0.0)
    return euler_step(x, v, s, s_next)


def weights_to_f64(w) -> Dict:
    """bf16 bit-pattern weights (an object with the C ABI's field names) -> float64 arrays. The text
    refiner's weights are converted when present."""
    get = (lambda k: w[k]) if isinstance(w, dict) else (lambda k: getattr(w, k))
    has = (lambda k: k in w) if isinstance(w, dict) else (lambda k: getattr(w, k, None) is not None)
    out = {k: from_bf16_bits(get(k)) for k in ("t_w1", "t_w2", "x_embed_w", "final_mod_w", "final_w")}
    for k in ("mod_w", "qkv_w", "out_w", "gate_up_w", "down_w"):
        out[k] = [from_bf16_bits(a) for a in get(k)]
    if has("text_proj_w"):
        out["text_proj_w"] = from_bf16_bits(get("text_proj_w"))
        for k in ("refiner_qkv_w", "refiner_out_w", "refiner_gate_up_w", "refiner_down_w"):
            out[k] = [from_bf16_bits(a) for a in get(k)]
    return out
