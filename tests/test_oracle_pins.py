"""Pins of the CPU oracle against what the pages and the mathematics fix (runs without a GPU).

Each test names the passage or the mathematical fact it checks. The brute-force references below are
scalar Python loops written from the definition, not calls of the oracle's own routines, so a dropped
term, a wrong sign or index, or a transposed operand in the oracle fails one of them.
"""
import json
import math
import os
import statistics

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ------------------------------------------------------------------------------------------------
# bfloat16 rounding
# ------------------------------------------------------------------------------------------------

def test_bf16_round_matches_torch_cast():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0, -1.0, 65504.0, 3.0e38, 1e-40, -1e-42]])
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.bf16_round(x32), ref)


def test_bf16_round_hand_ties():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins -> 1.
    assert O.bf16_round(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 (odd) and 1 + 2^-6 (even) -> 1 + 2^-6.
    assert O.bf16_round(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert O.bf16_round(1.0 + 2.0 ** -8 + 2.0 ** -20) == 1.0 + 2.0 ** -7
    assert O.from_bf16_bits(np.array([0x3F80, 0xC000, 0x0000], dtype=np.uint16)).tolist() == [1.0, -2.0, 0.0]


# ------------------------------------------------------------------------------------------------
# A1: schedule and SLG window
# ------------------------------------------------------------------------------------------------

def test_sigmas_hand_fractions_shift5():
    # sigma = 5 s / (1 + 4 s) on s = 1, 3/4, 1/2, 1/4, 0 (fractions worked by hand)
    np.testing.assert_allclose(O.sigmas(4, 5.0), [1.0, 15 / 16, 5 / 6, 5 / 8, 0.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(O.sigmas(2, 5.0), [1.0, 5 / 6, 0.0], rtol=0, atol=1e-15)


def test_sigmas_endpoints_monotone_and_shift1_linear():
    g = golden()["defaults"]
    s = O.sigmas(g["num_steps"], g["shift"])
    assert len(s) == g["num_steps"] + 1 and s[0] == 1.0 and s[-1] == 0.0
    assert np.all(np.diff(s) < 0)
    np.testing.assert_allclose(O.sigmas(10, 1.0), np.linspace(1, 0, 11), atol=1e-15)
    # the shift only warps time: s recovered by the inverse map is the uniform grid
    s_back = s / (g["shift"] - (g["shift"] - 1) * s)
    np.testing.assert_allclose(s_back, np.linspace(1, 0, g["num_steps"] + 1), atol=1e-14)


def test_slg_window_first_step_full_cfg():
    # The default window (0.01 to 1.0) makes the unconditional pass skip block 22 on every step but the
    # first, which runs at full CFG; a window starting at 0.0 skips it from step 0 on (SGLang cookbook
    # for MOSS-Image, section 3).
    g = golden()["defaults"]
    N = g["num_steps"]
    active = [i for i in range(N) if O.slg_active(i, N, g["slg_start"], g["slg_stop"])]
    assert active == list(range(1, N))
    assert [i for i in range(N) if O.slg_active(i, N, 0.0, 1.0)] == list(range(N))
    assert [O.slg_active(i, 2) for i in range(2)] == [False, True]


# ------------------------------------------------------------------------------------------------
# A12: guidance and Euler
# ------------------------------------------------------------------------------------------------

def test_cfg_identities():
    rng = np.random.default_rng(2)
    vc, vu = rng.standard_normal(100), rng.standard_normal(100)
    np.testing.assert_array_equal(O.cfg_combine(vc, vu, 1.0), vc)
    np.testing.assert_array_equal(O.cfg_combine(vc, vc, 4.5), vc)
    np.testing.assert_allclose(O.cfg_combine(vc, vu, 3.0), 3 * vc - 2 * vu, atol=1e-14)
    with pytest.raises(ValueError):
        O.cfg_combine(vc, vu, 0.5)


def test_euler_constant_velocity_telescopes():
    sig = O.sigmas(50, 5.0)
    rng = np.random.default_rng(3)
    x0, v = rng.standard_normal(64), rng.standard_normal(64)
    x = x0.copy()
    for i in range(50):
        x = O.euler_step(x, v, sig[i], sig[i + 1])
    np.testing.assert_allclose(x, x0 - v, atol=1e-12)


def test_euler_point_mass_field_lands_on_target():
    # v(x, sigma) = (x - x*)/sigma gives x_{i+1} - x* = (x_i - x*) sigma_{i+1}/sigma_i -> x_N = x*.
    sig = O.sigmas(50, 5.0)
    rng = np.random.default_rng(4)
    xs, x = rng.standard_normal(64), rng.standard_normal(64)
    x_mid = None
    for i in range(50):
        x = O.euler_step(x, (x - xs) / sig[i], sig[i], sig[i + 1])
        if i == 24:
            x_mid = x.copy()
    np.testing.assert_allclose(x, xs, atol=1e-12)


# ------------------------------------------------------------------------------------------------
# A2: time features and modulation
# ------------------------------------------------------------------------------------------------

def test_time_features_hand_values():
    cfg = O.Config()
    e0 = O.time_features(0.0, cfg)
    np.testing.assert_array_equal(e0, [1.0] * 128 + [0.0] * 128)
    e = O.time_features(0.5, cfg)           # t = 1000 * 0.5 = 500
    assert e[0] == pytest.approx(math.cos(500.0), abs=1e-12)
    assert e[128] == pytest.approx(math.sin(500.0), abs=1e-12)
    # k = 64 -> f = 10^4^(-1/2) = 0.01 -> angle 5
    assert e[64] == pytest.approx(math.cos(5.0), abs=1e-12)
    assert e[192] == pytest.approx(math.sin(5.0), abs=1e-12)


def test_modulation_chunk_order_scalar_bruteforce():
    cfg = O.Config(num_layers=2, hidden=8, temb_dim=256)
    rng = np.random.default_rng(5)
    W = {"t_w1": rng.standard_normal((256, 256)) * 0.05, "t_w2": rng.standard_normal((256, 256)) * 0.05,
         "mod_w": [rng.standard_normal((48, 256)) for _ in range(2)], "final_mod_w": rng.standard_normal((16, 256))}
    sigma = 0.3
    m, mf = O.modulation(sigma, W, cfg)
    # scalar re-derivation
    t = 1000.0 * sigma
    e = [math.cos(t * math.exp(-math.log(1e4) * k / 128)) for k in range(128)] + \
        [math.sin(t * math.exp(-math.log(1e4) * k / 128)) for k in range(128)]
    sl = lambda z: z / (1 + math.exp(-z))
    a1 = [sl(sum(W["t_w1"][i][j] * e[j] for j in range(256))) for i in range(256)]
    temb = [sum(W["t_w2"][i][j] * a1[j] for j in range(256)) for i in range(256)]
    u = [sl(z) for z in temb]
    for l in range(2):
        for chunk in range(6):
            for dd in range(8):
                row = chunk * 8 + dd
                ref = sum(W["mod_w"][l][row][j] * u[j] for j in range(256))
                assert m[l, chunk, dd] == pytest.approx(ref, rel=1e-10, abs=1e-12)
    assert mf[1, 3] == pytest.approx(sum(W["final_mod_w"][8 + 3][j] * u[j] for j in range(256)), rel=1e-10)


# ------------------------------------------------------------------------------------------------
# A3 / A11: patchify
# ------------------------------------------------------------------------------------------------

def test_patchify_hand_element_and_inverse():
    lat = np.zeros((32, 6, 8))
    lat[3, 5, 2] = 1.0          # grid (r, c) = (2, 1), (dy, dx) = (1, 0) -> n = 2*4 + 1, j = 3*4 + 2
    tok = O.patchify(lat)
    assert tok.shape == (12, 128)
    assert tok[9, 14] == 1.0 and tok.sum() == 1.0
    rng = np.random.default_rng(6)
    lat = rng.standard_normal((32, 6, 8))
    np.testing.assert_array_equal(O.unpatchify(O.patchify(lat), 32, 6, 8), lat)


def test_token_count_at_1024():
    g = golden()["architecture"]
    side = 1024 // g["vae_downsample"]                       # latent side 128
    assert (side // g["patch"]) ** 2 == g["image_tokens_at_1024"]
    assert g["vae_downsample"] * g["patch"] == g["pixels_per_token_side"]


# ------------------------------------------------------------------------------------------------
# A4 / A8: LayerNorm modulation
# ------------------------------------------------------------------------------------------------

def test_layernorm_against_statistics_module():
    rng = np.random.default_rng(7)
    row = rng.standard_normal(3072) * 3 + 1.5
    mu, var = statistics.fmean(row), statistics.pvariance(row)
    ref = [(v - mu) / math.sqrt(var + 1e-6) for v in row]
    np.testing.assert_allclose(O.layernorm(row[None], 1e-6)[0], ref, atol=1e-12)


def test_ln_modulate_special_rows():
    D = 64
    rng = np.random.default_rng(8)
    shift, scale = rng.standard_normal(D), rng.standard_normal(D)
    np.testing.assert_allclose(O.ln_modulate(np.full((1, D), 2.5), shift, scale, 1e-6)[0], shift, atol=1e-12)
    np.testing.assert_allclose(O.ln_modulate(np.zeros((1, D)), shift, scale, 1e-6)[0], shift, atol=1e-12)
    a = 3.0
    row = np.array([a, -a] * (D // 2))
    n = a / math.sqrt(a * a + 1e-6)
    ref = np.array([n, -n] * (D // 2)) * (1 + scale) + shift
    np.testing.assert_allclose(O.ln_modulate(row[None], shift, scale, 1e-6)[0], ref, atol=1e-12)


# ------------------------------------------------------------------------------------------------
# RoPE
# ------------------------------------------------------------------------------------------------

def test_rope_hand_angles():
    a = O.rope_angles(1, 0, 128, 1e4)
    assert a.shape == (64,) and a[0] == 1.0 and a[32] == 0.0
    assert O.rope_angles(2, 0, 128, 1e4)[16] == pytest.approx(0.02, rel=1e-14)   # 2 * 1e4^(-1/2)
    assert O.rope_angles(0, 3, 128, 1e4)[32 + 8] == pytest.approx(0.3, rel=1e-14)  # 3 * 1e4^(-1/4)


def test_rope_rows_rotates_right_halves():
    d = 128
    x = np.zeros((3, 2 * d))
    x[:, 0] = 1.0            # head 0, dim 0 (row half)
    x[:, 64] = 1.0           # head 0, dim 64 (column half)
    x[:, d + 65] = 1.0       # head 1, dim 65 (column half, odd element)
    # sequence: 1 text row, then image tokens at (0,0) and (0,1) on a 2-wide grid
    y = O.rope_rows(x, text_len=1, grid_w=2, head_dim=d, theta=1e4)
    np.testing.assert_array_equal(y[0], x[0])                 # text row untouched
    np.testing.assert_array_equal(y[1], x[1])                 # position (0,0) is the identity
    c, s = math.cos(1.0), math.sin(1.0)
    assert y[2, 0] == 1.0 and y[2, 1] == 0.0                  # row position 0: dims 0,1 fixed
    assert y[2, 64] == pytest.approx(c) and y[2, 65] == pytest.approx(s)
    assert y[2, d + 64] == pytest.approx(-s) and y[2, d + 65] == pytest.approx(c)


def test_rope_preserves_norm_and_relative_positions():
    rng = np.random.default_rng(9)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    ang = lambda r, c: O.rope_angles(r, c, 128, 1e4)
    qr = O.apply_rope(q, ang(5, 7))
    assert np.linalg.norm(qr) == pytest.approx(np.linalg.norm(q), rel=1e-13)
    s1 = O.apply_rope(q, ang(5, 7)) @ O.apply_rope(k, ang(2, 30))
    s2 = O.apply_rope(q, ang(5 + 11, 7 + 4)) @ O.apply_rope(k, ang(2 + 11, 30 + 4))
    assert s1 == pytest.approx(s2, rel=1e-10)
    s3 = O.apply_rope(q, ang(5, 8)) @ O.apply_rope(k, ang(2, 30))
    assert abs(s3 - s1) > 1e-6


# ------------------------------------------------------------------------------------------------
# A6: attention
# ------------------------------------------------------------------------------------------------

def _attn_bruteforce(q, k, v, H, d):
    Sq, Sk = len(q), len(k)
    out = [[0.0] * (H * d) for _ in range(Sq)]
    for h in range(H):
        base = h * d
        for i in range(Sq):
            sc = [sum(q[i][base + t] * k[j][base + t] for t in range(d)) / math.sqrt(d) for j in range(Sk)]
            mx = max(sc)
            w = [math.exp(s - mx) for s in sc]
            z = sum(w)
            for t in range(d):
                out[i][base + t] = sum(w[j] * v[j][base + t] for j in range(Sk)) / z
    return np.array(out)


@pytest.mark.parametrize("S,H", [(1, 1), (7, 2), (12, 1)])
def test_attention_vs_scalar_bruteforce(S, H):
    rng = np.random.default_rng(10 + S)
    q, k, v = (rng.standard_normal((S, H * 128)) for _ in range(3))
    np.testing.assert_allclose(O.attention(q, k, v, H, 128), _attn_bruteforce(q.tolist(), k.tolist(), v.tolist(), H, 128),
                               rtol=1e-10, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(11)
    v = rng.standard_normal((1, 256))
    np.testing.assert_allclose(O.attention(rng.standard_normal((3, 256)), rng.standard_normal((1, 256)), v, 2, 128),
                               np.repeat(v, 3, axis=0), atol=1e-14)
    k = np.repeat(rng.standard_normal((1, 128)), 5, axis=0)
    v = rng.standard_normal((5, 128))
    np.testing.assert_allclose(O.attention(rng.standard_normal((2, 128)), k, v, 1, 128),
                               np.repeat(v.mean(0, keepdims=True), 2, axis=0), atol=1e-13)
    # hand 3:1 split: scores ln 3 and 0 after the 1/sqrt(128) scale
    q = np.zeros((1, 128)); q[0, 0] = math.sqrt(128) * math.log(3.0)
    k = np.zeros((2, 128)); k[0, 0] = 1.0
    v = rng.standard_normal((2, 128))
    np.testing.assert_allclose(O.attention(q, k, v, 1, 128)[0], 0.75 * v[0] + 0.25 * v[1], atol=1e-13)


# ------------------------------------------------------------------------------------------------
# A4..A10: one block, against a scalar brute force
# ------------------------------------------------------------------------------------------------

def _block_bruteforce(x, m, Wqkv, Wo, Wgu, Wd, T, gw, D, H, d, F, eps, theta):
    S = len(x)
    sl = lambda z: z / (1 + math.exp(-z))

    def ln_mod(rowv, sh, sc):
        mu = sum(rowv) / D
        var = sum((a - mu) ** 2 for a in rowv) / D
        return [(rowv[i] - mu) / math.sqrt(var + eps) * (1 + sc[i]) + sh[i] for i in range(D)]

    def lin(vec, Wm, rows, cols):
        return [sum(Wm[o][i] * vec[i] for i in range(cols)) for o in range(rows)]

    def rope(vec, s):
        if s < T:
            return vec
        pr, pc = divmod(s - T, gw)
        out = list(vec)
        for h in range(H):
            for i in range(0, d, 2):
                half, pair = divmod(i, d // 2)
                pos = pr if half == 0 else pc
                kk = pair // 2
                phi = pos * theta ** (-kk / (d // 4))
                a, b = vec[h * d + i], vec[h * d + i + 1]
                out[h * d + i] = a * math.cos(phi) - b * math.sin(phi)
                out[h * d + i + 1] = a * math.sin(phi) + b * math.cos(phi)
        return out

    sh1, sc1, g1, sh2, sc2, g2 = [list(c) for c in m]
    A = [ln_mod(x[s], sh1, sc1) for s in range(S)]
    QKV = [lin(A[s], Wqkv, 3 * D, D) for s in range(S)]
    Q = [rope(QKV[s][:D], s) for s in range(S)]
    K = [rope(QKV[s][D:2 * D], s) for s in range(S)]
    V = [QKV[s][2 * D:] for s in range(S)]
    Oh = _attn_bruteforce(Q, K, V, H, d).tolist()
    x1 = []
    for s in range(S):
        ao = lin(Oh[s], Wo, D, D)
        x1.append([x[s][i] + g1[i] * ao[i] for i in range(D)])
    x2 = []
    for s in range(S):
        a2 = ln_mod(x1[s], sh2, sc2)
        gu = lin(a2, Wgu, 2 * F, D)
        hf = [sl(gu[j]) * gu[F + j] for j in range(F)]
        fo = lin(hf, Wd, D, F)
        x2.append([x1[s][i] + g2[i] * fo[i] for i in range(D)])
    return np.array(x2)


def test_block_vs_scalar_bruteforce():
    H, d, F = 2, 128, 32
    D = H * d
    cfg = O.Config(num_layers=1, hidden=D, num_heads=H, head_dim=d, ffn_hidden=F)
    rng = np.random.default_rng(12)
    T, gw = 2, 2
    S = T + 4                                   # 2x2 image grid
    x = rng.standard_normal((S, D))
    m = rng.standard_normal((6, D)) * 0.5
    W = {"qkv_w": [rng.standard_normal((3 * D, D)) * 0.06], "out_w": [rng.standard_normal((D, D)) * 0.06],
         "gate_up_w": [rng.standard_normal((2 * F, D)) * 0.06], "down_w": [rng.standard_normal((D, F)) * 0.06]}
    got = O.block(x, m, W, 0, cfg, T, gw)
    ref = _block_bruteforce(x.tolist(), m.tolist(), W["qkv_w"][0].tolist(), W["out_w"][0].tolist(),
                            W["gate_up_w"][0].tolist(), W["down_w"][0].tolist(), T, gw, D, H, d, F, 1e-6, 1e4)
    np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-10)
    # computing a subset of rows gives the same rows
    sub = O.block(x, m, W, 0, cfg, T, gw, rows=[1, 4])
    np.testing.assert_allclose(sub, got[[1, 4]], rtol=1e-12, atol=1e-13)


def test_block_zero_gates_is_identity_and_mirror_rounds_residual():
    H, d, F = 1, 128, 64
    D = H * d
    cfg = O.Config(num_layers=1, hidden=D, num_heads=H, head_dim=d, ffn_hidden=F)
    rng = np.random.default_rng(13)
    x = O.bf16_round(rng.standard_normal((5, D)))
    m = rng.standard_normal((6, D))
    m[2] = 0.0
    m[5] = 0.0
    W = {"qkv_w": [rng.standard_normal((3 * D, D)) * 0.05], "out_w": [rng.standard_normal((D, D)) * 0.05],
         "gate_up_w": [rng.standard_normal((2 * F, D)) * 0.05], "down_w": [rng.standard_normal((D, F)) * 0.05]}
    np.testing.assert_array_equal(O.block(x, m, W, 0, cfg, 1, 2, mirror=True), x)
    m[2] = 0.3
    taps = {}
    y = O.block(x, m, W, 0, cfg, 1, 2, mirror=True, taps=taps)
    np.testing.assert_array_equal(O.bf16_round(y), y)
    np.testing.assert_allclose(taps["x1"], O.bf16_round(x + m[2] * taps["attn_out"]), atol=0)


# ------------------------------------------------------------------------------------------------
# forward and sampling step
# ------------------------------------------------------------------------------------------------

def _tiny_cfg():
    return O.Config(num_layers=2, hidden=128, num_heads=1, head_dim=128, ffn_hidden=64)


def _tiny_weights(cfg, rng, gate_zero=False):
    D, F, E, P = cfg.hidden, cfg.ffn_hidden, cfg.temb_dim, cfg.patch_dim
    W = {"t_w1": rng.standard_normal((E, 256)) * 0.05, "t_w2": rng.standard_normal((E, E)) * 0.05,
         "x_embed_w": rng.standard_normal((D, P)) * 0.05,
         "mod_w": [rng.standard_normal((6 * D, E)) for _ in range(cfg.num_layers)],
         "qkv_w": [rng.standard_normal((3 * D, D)) * 0.05 for _ in range(cfg.num_layers)],
         "out_w": [rng.standard_normal((D, D)) * 0.05 for _ in range(cfg.num_layers)],
         "gate_up_w": [rng.standard_normal((2 * F, D)) * 0.05 for _ in range(cfg.num_layers)],
         "down_w": [rng.standard_normal((D, F)) * 0.05 for _ in range(cfg.num_layers)],
         "final_mod_w": rng.standard_normal((2 * D, E)), "final_w": rng.standard_normal((P, D)) * 0.05}
    if gate_zero:
        for l in range(cfg.num_layers):
            W["mod_w"][l][2 * D:3 * D] = 0.0
            W["mod_w"][l][5 * D:6 * D] = 0.0
    return W


def test_forward_with_all_gates_zero_is_embed_then_final_bruteforce():
    cfg = _tiny_cfg()
    rng = np.random.default_rng(14)
    W = _tiny_weights(cfg, rng, gate_zero=True)
    C, h, w, T, D = 32, 4, 4, 3, cfg.hidden
    lat = rng.standard_normal((1, C, h, w))
    txt = rng.standard_normal((1, T, D))
    v = O.forward(lat, txt, [0.7], W, cfg)
    # scalar brute force of: patch -> embed -> (blocks are identities) -> LN-mod final -> W_f -> place
    _, mf = O.modulation(0.7, W, cfg)
    ref = np.zeros((C, h, w))
    for r in range(h // 2):
        for c in range(w // 2):
            feat = [lat[0, ch, 2 * r + dy, 2 * c + dx] for ch in range(C) for dy in range(2) for dx in range(2)]
            z = [sum(W["x_embed_w"][o][j] * feat[j] for j in range(128)) for o in range(D)]
            mu = sum(z) / D
            var = sum((a - mu) ** 2 for a in z) / D
            a = [(z[i] - mu) / math.sqrt(var + 1e-6) * (1 + mf[1][i]) + mf[0][i] for i in range(D)]
            y = [sum(W["final_w"][o][i] * a[i] for i in range(D)) for o in range(128)]
            for ch in range(C):
                for dy in range(2):
                    for dx in range(2):
                        ref[ch, 2 * r + dy, 2 * c + dx] = y[ch * 4 + dy * 2 + dx]
    np.testing.assert_allclose(v[0], ref, rtol=1e-10, atol=1e-12)


def test_skip_equals_zeroed_gate_rows_bitwise():
    cfg = _tiny_cfg()
    rng = np.random.default_rng(15)
    W = _tiny_weights(cfg, rng)
    lat = O.bf16_round(rng.standard_normal((1, 32, 4, 4)))
    txt = rng.standard_normal((1, 3, cfg.hidden))
    v_skip = O.forward(lat, txt, [0.4], W, cfg, skip=[{1}], mirror=True)
    W0 = {k: (list(v) if isinstance(v, list) else v) for k, v in W.items()}
    mw = W["mod_w"][1].copy()
    mw[2 * cfg.hidden:3 * cfg.hidden] = 0.0
    mw[5 * cfg.hidden:] = 0.0
    W0["mod_w"] = [W["mod_w"][0], mw]
    np.testing.assert_array_equal(O.forward(lat, txt, [0.4], W0, cfg, mirror=True), v_skip)
    assert not np.array_equal(O.forward(lat, txt, [0.4], W, cfg, mirror=True), v_skip)


def test_sample_step_guidance_paths():
    cfg = _tiny_cfg()
    rng = np.random.default_rng(16)
    W = _tiny_weights(cfg, rng)
    x = rng.standard_normal((1, 32, 4, 4))
    tc = rng.standard_normal((1, 3, cfg.hidden))
    tu = np.zeros_like(tc)
    sig = O.sigmas(2, 5.0)
    # cfg = 1: no negative pass, x1 = x + dsigma * v_c
    vel = []
    x1 = O.sample_step(x, tc, None, W, cfg, 0, sig, cfg_scale=1.0, velocities=vel)
    assert vel[0][1] is None
    np.testing.assert_array_equal(x1, x + (sig[1] - sig[0]) * O.forward(x, tc, [sig[0]], W, cfg))
    # step 0 is outside the default window: the skip list does not matter there
    a = O.sample_step(x, tc, tu, W, cfg, 0, sig, 3.0, (1,))
    b = O.sample_step(x, tc, tu, W, cfg, 0, sig, 3.0, ())
    np.testing.assert_array_equal(a, b)
    # step 1 is inside: skipping block 1 changes the result; [] is ordinary CFG
    vel = []
    a = O.sample_step(x, tc, tu, W, cfg, 1, sig, 3.0, (1,), velocities=vel)
    vel2 = []
    b = O.sample_step(x, tc, tu, W, cfg, 1, sig, 3.0, (), velocities=vel2)
    assert not np.allclose(a, b)
    np.testing.assert_array_equal(vel[0][0], vel2[0][0])     # the cond pass never skips
    v_ref = vel2[0][1] + 3.0 * (vel2[0][0] - vel2[0][1])
    np.testing.assert_allclose(b, x + (sig[2] - sig[1]) * v_ref, atol=1e-14)


def test_cfg_truncation_boundary_table():
    # CFG truncation X leaves the negative branch out of the last (1 - X) of the steps (MossInfer
    # guide, lossy accelerators); steps are numbered from 0, X = 1 (the default) is off, and CFG 1 runs
    # no negative branch at all.
    runs = lambda X, N, cfg=3.0: [i for i in range(N) if O.negative_pass_runs(i, N, cfg, X)]
    assert runs(1.0, 50) == list(range(50))
    assert runs(0.0, 50) == []
    assert runs(0.8, 50) == list(range(40))
    assert runs(0.5, 3) == [0, 1]           # 1.5: step 1 still runs, step 2 does not
    assert runs(0.5, 2) == [0]
    assert runs(1.0, 50, cfg=1.0) == []


def test_guidance_combine_hand_values():
    one, zero, quarter = np.ones(3), np.zeros(3), np.full(3, 0.25)
    # v_u + cfg (v_c - v_u) + slg (v_c - v_s) = 0 + 3*1 + 2*0.75
    np.testing.assert_array_equal(O.guidance_combine(one, zero, quarter, 3.0, 2.0), np.full(3, 4.5))
    # no negative branch: v_c + slg (v_c - v_s) = 1 + 2*0.75
    np.testing.assert_array_equal(O.guidance_combine(one, None, quarter, 3.0, 2.0), np.full(3, 2.5))
    # no third prediction: the two-pass combine, and v_c alone without a negative branch
    np.testing.assert_array_equal(O.guidance_combine(one, zero, None, 3.0, 2.0), np.full(3, 3.0))
    np.testing.assert_array_equal(O.guidance_combine(one, None, None, 3.0, 2.0), one)
    rng = np.random.default_rng(21)
    vc, vu, vs = rng.standard_normal((3, 50))
    # v_s = v_c adds nothing, bitwise; the term is linear in slg_scale
    np.testing.assert_array_equal(O.guidance_combine(vc, vu, vc, 3.0, 5.0), O.cfg_combine(vc, vu, 3.0))
    f = lambda g: O.guidance_combine(vc, vu, vs, 3.0, g)
    np.testing.assert_allclose(f(2.5) - f(0.0), (f(1.0) - f(0.0)) + (f(1.5) - f(0.0)), atol=1e-13)


def test_three_pass_slg_and_truncation_paths():
    cfg = _tiny_cfg()
    rng = np.random.default_rng(22)
    W = _tiny_weights(cfg, rng)
    x = rng.standard_normal((1, 32, 4, 4))
    tc = rng.standard_normal((1, 3, cfg.hidden))
    tu = np.zeros_like(tc)
    sig = O.sigmas(2, 5.0)
    two = O.sample_step(x, tc, tu, W, cfg, 1, sig, 3.0, (1,))
    # step 1 is inside the default window: the third row is the conditional forward with block 1
    # skipped, i.e. with block 1's gate rows zeroed (an independent route to the same prediction)
    vel = []
    three = O.sample_step(x, tc, tu, W, cfg, 1, sig, 3.0, (1,), velocities=vel, slg_scale=2.0)
    v_c, v_u, v_s = vel[0]
    W0 = {k: (list(v) if isinstance(v, list) else v) for k, v in W.items()}
    mw = W["mod_w"][1].copy()
    mw[2 * cfg.hidden:3 * cfg.hidden] = 0.0
    mw[5 * cfg.hidden:] = 0.0
    W0["mod_w"] = [W["mod_w"][0], mw]
    np.testing.assert_array_equal(v_s, O.forward(x, tc, [sig[1]], W0, cfg))
    np.testing.assert_array_equal(v_c, O.forward(x, tc, [sig[1]], W, cfg))
    assert not np.allclose(three, two)
    dv = (three - two) / (sig[2] - sig[1])
    np.testing.assert_allclose(dv, 2.0 * (v_c - v_s), atol=1e-10)
    # the same step without the term: slg 0, an empty skip list, or a step outside the window
    np.testing.assert_array_equal(O.sample_step(x, tc, tu, W, cfg, 1, sig, 3.0, (1,), slg_scale=0.0), two)
    np.testing.assert_array_equal(O.sample_step(x, tc, tu, W, cfg, 1, sig, 3.0, (), slg_scale=2.0),
                                  O.sample_step(x, tc, tu, W, cfg, 1, sig, 3.0, ()))
    np.testing.assert_array_equal(O.sample_step(x, tc, tu, W, cfg, 0, sig, 3.0, (1,), slg_scale=2.0),
                                  O.sample_step(x, tc, tu, W, cfg, 0, sig, 3.0, (1,)))
    # truncation at X = 0.5 of 2 steps: step 1 runs without the negative branch, i.e. as at CFG 1
    vel = []
    tr = O.sample_step(x, tc, tu, W, cfg, 1, sig, 3.0, (1,), velocities=vel, cfg_truncation=0.5)
    assert vel[0][1] is None and vel[0][2] is None
    np.testing.assert_array_equal(tr, O.sample_step(x, tc, None, W, cfg, 1, sig, 1.0, (1,)))
    np.testing.assert_array_equal(O.sample_step(x, tc, tu, W, cfg, 0, sig, 3.0, (1,), cfg_truncation=0.5),
                                  O.sample_step(x, tc, tu, W, cfg, 0, sig, 3.0, (1,)))
    # truncated three-pass step: v_c + slg (v_c - v_s)
    vel = []
    trs = O.sample_step(x, tc, tu, W, cfg, 1, sig, 3.0, (1,), velocities=vel, slg_scale=2.0, cfg_truncation=0.5)
    assert vel[0][1] is None
    np.testing.assert_allclose((trs - x) / (sig[2] - sig[1]), 3.0 * v_c - 2.0 * v_s, atol=1e-10)


def _refiner_weights(cfg, rng, text_dim, zero_branches=False):
    D, F = cfg.hidden, cfg.ffn_hidden
    L = 2
    W = {"text_proj_w": rng.standard_normal((D, text_dim)) * 0.05,
         "refiner_qkv_w": [rng.standard_normal((3 * D, D)) * 0.05 for _ in range(L)],
         "refiner_out_w": [rng.standard_normal((D, D)) * 0.05 for _ in range(L)],
         "refiner_gate_up_w": [rng.standard_normal((2 * F, D)) * 0.05 for _ in range(L)],
         "refiner_down_w": [rng.standard_normal((D, F)) * 0.05 for _ in range(L)]}
    if zero_branches:
        W["refiner_out_w"] = [np.zeros((D, D)) for _ in range(L)]
        W["refiner_down_w"] = [np.zeros((D, F)) for _ in range(L)]
    return W


def test_text_refine_projection_bruteforce():
    # with zero output projections in both blocks every branch adds 0, so the refiner is the bare
    # projection; checked against a scalar loop (no bias), with and without the bf16 storage points
    cfg = _tiny_cfg()
    rng = np.random.default_rng(31)
    E = 48
    W = _refiner_weights(cfg, rng, E, zero_branches=True)
    enc = rng.standard_normal((5, E))
    ref = np.zeros((5, cfg.hidden))
    for t in range(5):
        for o in range(cfg.hidden):
            acc = 0.0
            for i in range(E):
                acc += enc[t, i] * W["text_proj_w"][o, i]
            ref[t, o] = acc
    np.testing.assert_allclose(O.text_refine(enc, W, cfg), ref, rtol=1e-12, atol=1e-12)
    got = O.text_refine(enc, W, cfg, mirror=True)
    np.testing.assert_array_equal(got, O.bf16_round(O.bf16_round(enc) @ W["text_proj_w"].T))


def test_text_refine_permutation_equivariant():
    # no positional rotation and no mask on text rows: permuting the prompt's rows permutes the output
    cfg = _tiny_cfg()
    rng = np.random.default_rng(32)
    W = _refiner_weights(cfg, rng, 40)
    enc = rng.standard_normal((7, 40))
    perm = rng.permutation(7)
    a = O.text_refine(enc, W, cfg)
    b = O.text_refine(enc[perm], W, cfg)
    np.testing.assert_allclose(b, a[perm], rtol=1e-10, atol=1e-12)
    assert not np.allclose(a, O.text_refine(enc[:, ::-1].copy(), W, cfg))
    # equal rows stay equal (each row attends to the same key set with the same scores)
    enc2 = enc.copy()
    enc2[3] = enc2[1]
    c = O.text_refine(enc2, W, cfg)
    np.testing.assert_allclose(c[3], c[1], rtol=1e-12, atol=1e-12)


def test_text_refine_blocks_are_unmodulated_joint_blocks():
    # one refiner block equals the generic joint block with shift = scale = 0 and gate = 1, and a
    # block whose gate is 1 is not the identity (the branch outputs are added at full weight)
    cfg = _tiny_cfg()
    rng = np.random.default_rng(33)
    W = _refiner_weights(cfg, rng, 32)
    W1 = dict(W)
    for k in ("refiner_qkv_w", "refiner_out_w", "refiner_gate_up_w", "refiner_down_w"):
        W1[k] = W[k][:1]
    enc = rng.standard_normal((6, 32))
    x0 = enc @ W["text_proj_w"].T
    # scalar brute force of LN without modulation on row 0
    row = x0[0]
    mu = sum(row) / len(row)
    var = sum((v - mu) ** 2 for v in row) / len(row)
    np.testing.assert_allclose(O.ln_modulate(x0, np.zeros(cfg.hidden), np.zeros(cfg.hidden), cfg.norm_eps)[0],
                               (row - mu) / math.sqrt(var + cfg.norm_eps), rtol=1e-12)
    taps = {}
    m = np.zeros((6, cfg.hidden))
    m[2] = m[5] = 1.0
    Wb = {"qkv_w": W["refiner_qkv_w"], "out_w": W["refiner_out_w"], "gate_up_w": W["refiner_gate_up_w"],
          "down_w": W["refiner_down_w"]}
    x1 = O.block(x0, m, Wb, 0, cfg, 6, 1, taps=taps)
    np.testing.assert_allclose(x1, x0 + taps["attn_out"] + taps["ffn_out"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.text_refine(enc, W1, cfg), x1, rtol=1e-12, atol=1e-12)


def test_first_block_change_hand_values():
    r_prev = np.array([[1.0, -2.0], [0.5, 0.5]])
    r = np.array([[1.5, -2.0], [0.5, 0.0]])
    assert O.first_block_change(r, r_prev) == (0.5 + 0.5) / 4.0
    assert O.first_block_change(r_prev, r_prev) == 0.0


def _cache_run(W, cfg, x, tc, tu, sig, threshold, skip=()):
    cache = O.StepCache()
    xs, xu = [], []
    xa, xb = x.copy(), x.copy()
    for i in range(len(sig) - 1):
        xa = O.sample_step_cached(xa, tc, tu, W, cfg, i, sig, cache, threshold, 3.0, skip)
        xb = O.sample_step(xb, tc, tu, W, cfg, i, sig, 3.0, skip)
        xs.append(xa.copy()), xu.append(xb.copy())
    return cache, xs, xu


def test_step_cache_threshold_zero_is_the_plain_step():
    cfg = _tiny_cfg()
    rng = np.random.default_rng(41)
    W = _tiny_weights(cfg, rng)
    x = rng.standard_normal((1, 32, 4, 4))
    tc, tu = rng.standard_normal((1, 3, cfg.hidden)), np.zeros((1, 3, cfg.hidden))
    sig = O.sigmas(3, 5.0)
    cache, xs, xu = _cache_run(W, cfg, x, tc, tu, sig, 0.0)
    for a, b in zip(xs, xu):
        np.testing.assert_array_equal(a, b)
    assert (cache.full_calls, cache.reused_calls) == (3, 0)
    assert np.isfinite(cache.last_change) and cache.last_change > 0


def test_step_cache_reuse_composes_block0_and_the_cached_rest():
    # with the gates of every block after block 0 zeroed, blocks 1.. are identities: the cached rest
    # is 0 and a reused call must give the full call's result bit for bit; with a huge threshold every
    # call after the first reuses, except where the row plan changes (the negative pass starts skipping
    # block 1 at step 1 of 3, which restarts the cache)
    cfg = _tiny_cfg()
    rng = np.random.default_rng(42)
    W = _tiny_weights(cfg, rng)
    for l in range(1, cfg.num_layers):
        W["mod_w"][l][2 * cfg.hidden:3 * cfg.hidden] = 0.0
        W["mod_w"][l][5 * cfg.hidden:] = 0.0
    x = rng.standard_normal((1, 32, 4, 4))
    tc, tu = rng.standard_normal((1, 3, cfg.hidden)), np.zeros((1, 3, cfg.hidden))
    sig = O.sigmas(3, 5.0)
    cache, xs, xu = _cache_run(W, cfg, x, tc, tu, sig, 1e9)
    for a, b in zip(xs, xu):
        np.testing.assert_array_equal(a, b)
    assert (cache.full_calls, cache.reused_calls) == (1, 2)
    cache, xs, xu = _cache_run(W, cfg, x, tc, tu, sig, 1e9, skip=(1,))
    assert (cache.full_calls, cache.reused_calls) == (2, 1)
    for a, b in zip(xs, xu):
        np.testing.assert_array_equal(a, b)
    # with live blocks a reused call differs from the full one (the cache is lossy)
    W2 = _tiny_weights(cfg, np.random.default_rng(42))
    cache, xs, xu = _cache_run(W2, cfg, x, tc, tu, sig, 1e9)
    assert cache.reused_calls == 2 and not np.array_equal(xs[2], xu[2])
    np.testing.assert_array_equal(xs[0], xu[0])


def _e4m3_table():
    # every finite E4M3 value from the bit layout: S EEEE MMM, bias 7, E = 0 subnormal, S 1111 111 NaN
    vals = []
    for code in range(256):
        s_, e, m = code >> 7, (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            continue
        v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        vals.append((-v if s_ else v, m))
    return vals


def test_e4m3_round_bruteforce_over_all_codes():
    table = _e4m3_table()
    assert max(v for v, _ in table) == golden()["fp8_e4m3"]["max_finite"] == O.E4M3_MAX
    assert min(v for v, _ in table if v > 0) == golden()["fp8_e4m3"]["min_subnormal"]
    rng = np.random.default_rng(60)
    xs = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.uniform(-4, 3, 3000),
                         [v + d for v, _ in table for d in (0.0,)],          # every code exactly
                         [0.5 * (a + b) for (a, _), (b, _) in zip(sorted(table), sorted(table)[1:])]])  # every tie
    got = O.e4m3_round(xs)
    for x, g in zip(xs, got):
        if abs(x) >= O.E4M3_MAX:
            assert g == math.copysign(O.E4M3_MAX, x)
            continue
        best = min(table, key=lambda vm: (abs(vm[0] - x), vm[1] & 1))   # nearest, ties to even mantissa
        assert g == best[0] or (g == 0 and best[0] == 0), (x, g, best)


def test_mx_quantize_hand_blocks_and_bounds():
    # amax 3 -> scale exponent floor(log2 3) - 8 = -7; codes 1*2^7 = 128, 3*2^7 = 384 (both exact)
    x = np.zeros((1, 64))
    x[0, 0], x[0, 1] = 1.0, 3.0
    x[0, 32] = 500.0          # second block: exponent 8 - 8 = 0, 500 saturates to 448
    q, ex = O.mx_quantize(x)
    assert ex.tolist() == [[-7, 0]]
    assert (q[0, 0], q[0, 1], q[0, 32]) == (128.0, 384.0, 448.0)
    np.testing.assert_array_equal(O.mx_dequantize(np.zeros((2, 32))), 0.0)
    assert O.mx_quantize(np.zeros((1, 32)))[1].tolist() == [[-127]]
    # values of the form e4m3 * 2^k with a shared block exponent come back exactly
    rng = np.random.default_rng(61)
    codes = np.array([v for v, _ in _e4m3_table() if abs(v) >= 1.0])
    blk = rng.choice(codes, (4, 32)) * 2.0 ** -5
    blk[:, 0] = 256.0 * 2.0 ** -5                        # fixes each block's amax binade
    np.testing.assert_array_equal(O.mx_dequantize(blk), blk)
    # error bound: half a unit of the element's binade (3 mantissa bits), or of 2^(scale-9) below normals,
    # except where the scaled value exceeds 448 (the scale exponent floor(log2 amax) - 8 lets a block's
    # largest elements reach [448, 512)) and saturates
    x = rng.standard_normal((8, 256)) * 10.0 ** rng.uniform(-3, 3, (8, 1))
    d = O.mx_dequantize(x)
    _, ex = O.mx_quantize(x)
    scale = np.repeat(np.ldexp(1.0, ex), 32, axis=1)
    _, E = np.frexp(np.abs(x))
    unit = np.maximum(np.ldexp(1.0, E - 1 - 3), scale * 2.0 ** -9)
    sat = np.abs(x) >= O.E4M3_MAX * scale
    assert np.all(np.abs(d - x)[~sat] <= 0.5 * unit[~sat])
    np.testing.assert_array_equal(np.abs(d[sat]), (O.E4M3_MAX * scale)[sat])
    assert sat.any()


def test_mxfp8_projection_is_the_product_of_quantized_operands():
    # the FP8 tier's projection multiplies the MXFP8 values of both operands (quantized along the
    # reduction axis): on operands that already are MXFP8 values it is the plain product, exactly; and
    # a whole block stays within a few percent of the bf16 block's update
    cfg = _tiny_cfg()
    cfg8 = O.Config(**{**cfg.__dict__, "gemm_precision": "mxfp8"})
    rng = np.random.default_rng(62)
    a = O.mx_dequantize(rng.standard_normal((5, 64)))
    w = O.mx_dequantize(rng.standard_normal((7, 64)) * 0.05)
    np.testing.assert_array_equal(O.projection(a, w, cfg8), a @ w.T)
    a2 = rng.standard_normal((5, 64))
    np.testing.assert_array_equal(O.projection(a2, w, cfg8), O.mx_dequantize(a2) @ w.T)
    W = _tiny_weights(cfg, rng)
    x = rng.standard_normal((6, cfg.hidden))
    m, _ = O.modulation(0.4, W, cfg)
    b16 = O.block(x, m[0], W, 0, cfg, 2, 2)
    b8 = O.block(x, m[0], W, 0, cfg8, 2, 2)
    rel = np.linalg.norm(b8 - b16) / np.linalg.norm(b16 - x)
    assert 1e-4 < rel < 0.2          # 3 mantissa bits: about 2-3 % per operand, compounded


# ------------------------------------------------------------------------------------------------
# dimension pins (the SwiGLU / shape readings against the pages' printed sizes)
# ------------------------------------------------------------------------------------------------

def test_page_dimensions():
    g = golden()
    a = g["architecture"]
    cfg = O.Config()
    assert (cfg.num_layers, cfg.hidden, cfg.num_heads, cfg.head_dim, cfg.ffn_hidden, cfg.latent_channels,
            cfg.patch) == (a["num_layers"], a["hidden"], a["num_heads"], a["head_dim"], a["ffn_hidden"],
                           a["latent_channels"], a["patch"])
    assert cfg.num_heads * cfg.head_dim == cfg.hidden
    # q is a D x D projection: 42 * 3072^2 * 2 bytes ~ 0.74 GiB
    q_gib = cfg.num_layers * cfg.hidden ** 2 * 2 / 2 ** 30
    assert abs(q_gib - g["q_projection_memory"]["total_gib_about"]) < 0.005
    # SwiGLU blocks + modulation: ~5B parameters, ~10 GB in bf16
    D, F = cfg.hidden, cfg.ffn_hidden
    per_block = 4 * D * D + 3 * D * F + 6 * D * cfg.temb_dim
    params = cfg.num_layers * per_block + D * cfg.patch_dim + cfg.patch_dim * D + 2 * D * cfg.temb_dim
    assert round(params / 1e9) == a["dit_params_billion"]
    assert round(params * 2 / 1e9) == a["dit_bf16_gb_about"]
    # a two-matrix GELU FFN of 8192 would give ~3.9B: the SwiGLU reading is the one that reaches 5B
    assert round(cfg.num_layers * (4 * D * D + 2 * D * F) / 1e9) != a["dit_params_billion"]


# ------------------------------------------------------------------------------------------------
# FP8 tier: 8-bit attention (INT8 Q K^T, FP8 P V)
# ------------------------------------------------------------------------------------------------

def test_int8_codes_by_hand():
    # amax 1: 0.5 * 127 = 63.5 -> 64 (tie to even), 0.25 * 127 = 31.75 -> 32, the amax element -> -127
    q = np.array([[0.5, -1.0, 0.25, 0.0], [0.0, 0.0, 0.0, 0.0], [3.0, 1.5, -0.75, 0.1015625]])
    codes, amax = O.q8_quantize_q(q)
    assert codes[0].tolist() == [64.0, -127.0, 32.0, 0.0]
    assert codes[1].tolist() == [0.0, 0.0, 0.0, 0.0] and amax[1] == 0.0
    # amax 3: 1.5 * 127 / 3 = 63.5 -> 64; -0.75 * 127 / 3 = -31.75 -> -32; 0.1015625 * 127 / 3 = 4.2995.. -> 4
    assert codes[2].tolist() == [127.0, 64.0, -32.0, 4.0] and amax[2] == 3.0
    assert np.abs(codes).max() <= 127


def test_q8_key_blocks_and_v_channels():
    rng = np.random.default_rng(70)
    k = rng.standard_normal((100, 8))
    k[64:] *= 100.0                                    # the second block is 100x larger
    codes, amax = O.q8_quantize_k(k)
    assert amax.shape == (2,)
    assert amax[0] == np.abs(k[:64].astype(np.float32)).max() and amax[1] == np.abs(k[64:].astype(np.float32)).max()
    assert np.abs(codes[:64]).max() == 127 and np.abs(codes[64:]).max() == 127   # each block uses the full range
    err = np.abs(codes * np.repeat(amax, [64, 36])[:, None] / 127 - k)
    assert np.all(err[:64] <= 0.5 * amax[0] / 127 * (1 + 1e-6)) and np.all(err[64:] <= 0.5 * amax[1] / 127 * (1 + 1e-6))
    v = rng.standard_normal((50, 4))
    vc, va = O.fp8_quantize_v(v)
    assert np.all(np.abs(vc).max(axis=0) == O.E4M3_MAX)                            # each channel's amax -> 448
    np.testing.assert_array_equal(vc, O.e4m3_round(vc))                            # valid E4M3 values
    rel = np.abs(vc * va / O.E4M3_MAX - v) / np.abs(v)
    assert np.all(rel[np.abs(v) > va / 64] <= 2.0 ** -4 * (1 + 1e-6))             # half an E4M3 unit (3 bits)


def test_q8_attention_exact_probabilities_is_softmax_of_dequantized_operands():
    # with the probability rounding switched off, the online block algorithm must reproduce the exact
    # softmax attention (the pinned oracle above) of the dequantized q, k, v; Sk = 150 leaves a ragged block
    rng = np.random.default_rng(71)
    H, d, Sq, Sk = 2, 16, 7, 150
    q = rng.standard_normal((Sq, H * d)) * 2.0
    k = rng.standard_normal((Sk, H * d)) * 2.0
    v = rng.standard_normal((Sk, H * d))
    got = O.attention_q8(q, k, v, H, d, quantize_p=False)
    deq = lambda c, a: c * a / 127.0
    qd, kd, vd = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for h in range(H):
        sl = slice(h * d, (h + 1) * d)
        c, a = O.q8_quantize_q(q[:, sl]); qd[:, sl] = deq(c, a[:, None])
        c, a = O.q8_quantize_k(k[:, sl]); kd[:, sl] = deq(c, np.repeat(a, [64, 64, 22])[:, None])
        c, a = O.fp8_quantize_v(v[:, sl]); vd[:, sl] = c * a[None, :] / O.E4M3_MAX
    np.testing.assert_allclose(got, O.attention(qd, kd, vd, H, d), rtol=1e-12, atol=1e-12)


def test_q8_attention_convex_weights_and_selection():
    rng = np.random.default_rng(72)
    H, d = 1, 16
    q = rng.standard_normal((5, d))
    k = rng.standard_normal((130, d))
    vrow = O.bf16_round(rng.standard_normal(d))        # bf16 inputs, as the GPU gets them
    v = np.tile(vrow, (130, 1))                        # V constant over keys: amax = |v| -> codes +-448, exact
    np.testing.assert_allclose(O.attention_q8(q, k, v, H, d), np.tile(vrow, (5, 1)), rtol=1e-12)
    np.testing.assert_allclose(O.attention_q8(q, k[:1], v[:1], H, d), np.tile(vrow, (5, 1)), rtol=1e-12)
    # one key far above the rest: its probability is 1, the others round to 0 in E4M3 -> its V row
    k2 = rng.standard_normal((70, d)) * 0.01
    k2[37] = q[0] * 40.0
    v2 = rng.standard_normal((70, d))
    vc, va = O.fp8_quantize_v(v2)
    np.testing.assert_allclose(O.attention_q8(q[:1], k2, v2, H, d)[0], vc[37] * va / O.E4M3_MAX, rtol=1e-12)


def test_q8_attention_is_close_to_exact():
    rng = np.random.default_rng(73)
    H, d, S = 2, 128, 200
    q, k, v = (rng.standard_normal((S, H * d)) for _ in range(3))
    exact = O.attention(q, k, v, H, d)
    got = O.attention_q8(q, k, v, H, d)
    rel = np.linalg.norm(got - exact) / np.linalg.norm(exact)
    assert 1e-4 < rel < 0.05, rel


def test_block_with_q8_attention_uses_attention_q8():
    # the block's attention tap under attention_mode "q8" is attention_q8 of the block's own q, k, v
    cfg = _tiny_cfg()
    cfgq = O.Config(**{**cfg.__dict__, "attention_mode": "q8"})
    rng = np.random.default_rng(74)
    W = _tiny_weights(cfg, rng)
    x = rng.standard_normal((6, cfg.hidden))
    m, _ = O.modulation(0.4, W, cfg)
    taps = {}
    bq = O.block(x, m[0], W, 0, cfgq, 2, 2, taps=taps)
    np.testing.assert_array_equal(taps["o"], O.attention_q8(taps["q"], taps["k"], taps["v"], cfg.num_heads, cfg.head_dim))
    b16 = O.block(x, m[0], W, 0, cfg, 2, 2)
    rel = np.linalg.norm(bq - b16) / np.linalg.norm(b16 - x)
    assert 0 < rel < 0.1


def test_q8_attention_reference_max_moves_only_by_more_than_a_factor_two():
    # one query, keys in three blocks whose maxima rise by 0.5, then 1.5 units of log2: the reference
    # max stays at block 0's through block 1 (so block 1's top probability is 2^0.5, coded on the 224
    # scale) and moves at block 2; the result must equal a hand computation of that schedule
    d = 128
    q = np.zeros((1, d)); q[0, 0] = 1.0
    k = np.zeros((192, d))
    ln2 = math.log(2.0)
    tops = [0.0, 0.5, 2.0]                               # block maxima in log2 units (of the scaled score)
    for t, top in enumerate(tops):
        k[64 * t, 0] = top * ln2 * math.sqrt(d)          # score = q.k / sqrt(d) = top * ln 2
    v = np.zeros((192, d)); v[:, 1] = np.arange(192) + 1.0
    got = O.attention_q8(q, k, v, 1, d)
    # rebuild with the same quantizers and the expected schedule of reference maxima
    qc, qa = O.q8_quantize_q(q)
    kc, ka = O.q8_quantize_k(k)
    vc, va = O.fp8_quantize_v(v)
    vh = vc * va / O.E4M3_MAX
    s_all = [(qc @ kc[64 * t:64 * t + 64].T)[0] * qa[0] / 127 * ka[t] / 127 / math.sqrt(d) for t in range(3)]
    m_sched = [s_all[0].max(), s_all[0].max(), s_all[2].max()]   # no move at block 1 (0.5 < 1), a move at block 2
    o = np.zeros(d); l = 0.0; m_prev = None
    for t in range(3):
        a = 1.0 if m_prev is None or m_prev == m_sched[t] else math.exp(m_prev - m_sched[t])
        p = O.e4m3_round(np.exp(s_all[t] - m_sched[t]) * O.Q8_P_SCALE) / O.Q8_P_SCALE
        o = o * a + p @ vh[64 * t:64 * t + 64]
        l = l * a + p.sum()
        m_prev = m_sched[t]
    np.testing.assert_allclose(got[0], o / l, rtol=1e-12)
    assert np.exp(s_all[1] - m_sched[1]).max() > 1.0         # block 1 really had a probability above 1
