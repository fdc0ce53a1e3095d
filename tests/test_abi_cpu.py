"""C-ABI checks that need no GPU: the library loads and exports every symbol the headers declare,
struct layouts agree with the C compiler's, defaults equal the pages' values, the host-only schedule
matches the oracle, and every validation error path returns its status and message."""
import ctypes as C
import json
import os
import re
import subprocess

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
dt = pytest.importorskip("diffusion_transformer_text_amd")


def golden():
    with open(os.path.join(ROOT, "tests", "golden", "page_constants.json")) as f:
        return json.load(f)


def declared_functions():
    names = set()
    for h in ("moss_dit.h", "moss_dit_ops.h"):
        txt = open(os.path.join(ROOT, "include", h)).read()
        txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
        names |= set(re.findall(r"\b(moss_[a-z0-9_]+)\s*\(", txt))
    return names


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 20
    assert names == set(dt.EXPORTED)
    lib = C.CDLL(dt.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version():
    assert dt.moss_dit_abi_version() == dt.ABI_VERSION == 1
    assert dt.moss_status_string(0) == "ok"
    assert dt.moss_status_string(5) == "ABI mismatch"


def test_struct_layouts_match_c_compiler(tmp_path):
    src = tmp_path / "sz.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "moss_dit_ops.h"\n'
                   'int main(void){printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(moss_dit_config), '
                   'sizeof(moss_dit_weights), sizeof(moss_forward_args), sizeof(moss_step_args), sizeof(moss_block_taps), '
                   'offsetof(moss_step_args, cfg_scale), offsetof(moss_step_args, n_skip), offsetof(moss_forward_args, sigma), '
                   'offsetof(moss_dit_weights, q_norm_w), offsetof(moss_dit_weights, final_mod_w));}\n')
    exe = tmp_path / "sz"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [C.sizeof(dt.moss_dit_config), C.sizeof(dt.moss_dit_weights), C.sizeof(dt.moss_forward_args),
            C.sizeof(dt.moss_step_args), C.sizeof(dt.moss_block_taps), dt.moss_step_args.cfg_scale.offset,
            dt.moss_step_args.n_skip.offset, dt.moss_forward_args.sigma.offset, dt.moss_dit_weights.q_norm_w.offset,
            dt.moss_dit_weights.final_mod_w.offset]
    assert got == want


def test_config_defaults_are_the_pages():
    a = golden()["architecture"]
    c = dt.moss_dit_config_init()
    assert (c.num_layers, c.hidden, c.num_heads, c.head_dim, c.ffn_hidden, c.latent_channels, c.patch) == \
        (a["num_layers"], a["hidden"], a["num_heads"], a["head_dim"], a["ffn_hidden"], a["latent_channels"], a["patch"])
    o = O.Config()
    assert (c.temb_dim, c.rope_theta, c.norm_eps, c.flow_multiplier) == (o.temb_dim, o.rope_theta,
                                                                          np.float32(o.norm_eps), o.flow_multiplier)
    # the refiner: two text-only blocks ("Architecture and specs"); the state width is a reading
    assert c.refiner_layers == a["refiner_blocks"] == o.refiner_layers and c.text_dim == o.text_dim
    assert c.gemm_precision == 0 and o.gemm_precision == "bf16"    # the reference tier is bf16
    assert c.attention_mode == 0 and o.attention_mode == "exact"  # and runs exact attention


def test_step_defaults_are_the_pages():
    g = golden()["defaults"]
    s = dt.moss_step_args_init()
    assert s.num_steps == g["num_steps"] and s.step == 0
    assert s.cfg_scale == g["cfg_scale"]
    assert s.slg_start == np.float32(g["slg_start"]) and s.slg_stop == g["slg_stop"]
    assert [s.uncond_skip_layers[i] for i in range(s.n_skip)] == g["uncond_skip_layers"]
    assert (s.latent_h * 8, s.latent_w * 8) == (g["height"], g["width"])
    # the guidance variants are off by default: two-pass recipe, no CFG truncation
    assert s.slg_scale == 0.0 and s.cfg_truncation == 1.0
    assert s.step_cache == 0 and s.step_cache_threshold == 0.0      # the step cache is off by default


@pytest.mark.parametrize("N,shift", [(50, 5.0), (2, 5.0), (7, 1.0), (1000, 3.0)])
def test_sigmas_match_oracle(N, shift):
    got = dt.moss_sigmas(N, shift)
    ref = O.sigmas(N, shift)
    assert got[0] == 1.0 and got[-1] == 0.0
    np.testing.assert_array_equal(got, ref.astype(np.float32))


def test_sigmas_rejects_bad_input():
    with pytest.raises(dt.MossError):
        dt.moss_sigmas(0, 5.0)


def _valid_step(cfg):
    a = dt.moss_step_args_init()
    a.x, a.text_cond, a.text_uncond = 16, 32, 48          # never dereferenced by host validation
    sig = np.ascontiguousarray(O.sigmas(50, 5.0).astype(np.float32))
    a.sigmas = sig.ctypes.data_as(C.POINTER(C.c_float))
    return a, sig


def test_validate_step_accepts_defaults_and_2048():
    cfg = dt.moss_dit_config_init()
    a, keep = _valid_step(cfg)
    assert dt.moss_validate_step_args(cfg, a) == (0, "ok")
    a.latent_h = a.latent_w = 256                            # 2048^2 = 4.19 MP
    a.text_len = 4096
    assert dt.moss_validate_step_args(cfg, a)[0] == 0


@pytest.mark.parametrize("field,value,status,needle", [
    ("latent_h", 127, 1, "multiple of 16 px"),
    ("latent_w", 0, 1, "multiple of 16 px"),
    ("latent_w", 514, 1, "4096 px"),
    ("text_len", 0, 1, "text_len"),
    ("text_len", 4097, 1, "text_len"),
    ("cfg_scale", 0.5, 1, "cfg_scale"),
    ("step", 50, 1, "step"),
    ("num_steps", 0, 1, "num_steps"),
    ("struct_size", 8, 5, "struct_size"),
    ("slg_scale", -0.5, 1, "slg_scale"),
    ("slg_scale", float("inf"), 1, "slg_scale"),
    ("cfg_truncation", 1.5, 1, "cfg_truncation"),
    ("cfg_truncation", -0.1, 1, "cfg_truncation"),
    ("cfg_truncation", float("nan"), 1, "cfg_truncation"),
    ("step_cache", 2, 1, "step_cache"),
    ("step_cache_threshold", float("nan"), 1, "step_cache"),
])
def test_validate_step_errors(field, value, status, needle):
    cfg = dt.moss_dit_config_init()
    a, keep = _valid_step(cfg)
    setattr(a, field, value)
    st, msg = dt.moss_validate_step_args(cfg, a)
    assert st == status and needle in msg


def test_validate_step_pixel_cap_and_skip_range():
    cfg = dt.moss_dit_config_init()
    lim = golden()["limits"]
    a, keep = _valid_step(cfg)
    a.latent_h = a.latent_w = 258                            # 2064^2 = 4.26 MP > 4.2 MP
    st, msg = dt.moss_validate_step_args(cfg, a)
    assert st == 1 and "4.2" in msg
    assert 2064 ** 2 > lim["max_megapixels"] * 1e6 > 2048 ** 2
    a, keep = _valid_step(cfg)
    bad = (C.c_int32 * 1)(lim["skip_layer_max"] + 1)
    a.uncond_skip_layers = C.cast(bad, C.POINTER(C.c_int32))
    st, msg = dt.moss_validate_step_args(cfg, a)
    assert st == 1 and "41" in msg
    ok = (C.c_int32 * 3)(22, 24, 26)
    a.uncond_skip_layers = C.cast(ok, C.POINTER(C.c_int32))
    a.n_skip = 3
    assert dt.moss_validate_step_args(cfg, a)[0] == 0


def test_validate_step_null_pointers_and_cfg1():
    cfg = dt.moss_dit_config_init()
    a, keep = _valid_step(cfg)
    a.text_uncond = None
    assert dt.moss_validate_step_args(cfg, a)[0] == 1        # cfg 3 needs the negative text
    a.cfg_scale = 1.0
    assert dt.moss_validate_step_args(cfg, a)[0] == 0        # cfg 1 runs no negative pass
    a.x = None
    assert dt.moss_validate_step_args(cfg, a)[0] == 1


def test_validate_unsupported_config():
    for kw in ({"head_dim": 64}, {"hidden": 3000}, {"ffn_hidden": 8200}, {"qk_norm": 1}, {"num_layers": 65},
               {"text_dim": 100}, {"text_dim": 32}, {"refiner_layers": 9}):
        cfg = dt.moss_dit_config_init(**kw)
        a, keep = _valid_step(cfg)
        st, msg = dt.moss_validate_step_args(cfg, a)
        assert st == 2, kw


def test_validate_fp8_tier_config():
    """gemm_precision: 0 or 1; the MXFP8 tier needs ffn_hidden % 256 == 0 (a whole k-tile group)."""
    for kw, want in (({"gemm_precision": 1}, 0), ({"gemm_precision": 2}, 1), ({"gemm_precision": -1}, 1),
                     ({"gemm_precision": 1, "ffn_hidden": 8192 + 64}, 2), ({"gemm_precision": 0, "ffn_hidden": 8192 + 64}, 0)):
        cfg = dt.moss_dit_config_init(**kw)
        a, keep = _valid_step(cfg)
        assert dt.moss_validate_step_args(cfg, a)[0] == want, kw


def test_validate_attention_mode():
    for kw, want in (({"attention_mode": 1}, 0), ({"attention_mode": 2}, 1), ({"attention_mode": -1}, 1),
                     ({"attention_mode": 1, "gemm_precision": 1}, 0)):
        cfg = dt.moss_dit_config_init(**kw)
        a, keep = _valid_step(cfg)
        assert dt.moss_validate_step_args(cfg, a)[0] == want, kw


def test_validate_forward_args():
    cfg = dt.moss_dit_config_init()
    a = dt.moss_forward_args_init()
    a.batch, a.latent_h, a.latent_w, a.text_len = 2, 128, 128, 256
    a.latents, a.text, a.velocity = 16, 32, 48
    sig = (C.c_float * 2)(0.5, 0.5)
    a.sigma = C.cast(sig, C.POINTER(C.c_float))
    mask = (C.c_uint64 * 2)(0, 1 << 22)
    a.skip_mask = C.cast(mask, C.POINTER(C.c_uint64))
    assert dt.moss_validate_forward_args(cfg, a)[0] == 0
    mask[1] = 1 << 42
    assert dt.moss_validate_forward_args(cfg, a)[0] == 1
    mask[1] = 0
    sig[0] = 1.5
    assert dt.moss_validate_forward_args(cfg, a)[0] == 1
    sig[0] = 0.5
    a.batch = 9
    assert dt.moss_validate_forward_args(cfg, a)[0] == 1


def test_handleless_errors_set_thread_message():
    h = C.c_void_p()
    st = dt._lib.moss_dit_create(None, None, 0, None, C.byref(h))
    assert st == 1 and not h
    assert "config" in dt.moss_dit_last_error()
    assert dt._lib.moss_cfg_euler(None, None, None, 4, 3.0, 1.0, 0.5, None) == 1
    assert "moss_cfg_euler" in dt.moss_dit_last_error()


# Placeholder device addresses (256-byte aligned, never dereferenced: every case below is refused on the
# host before any device work).
_P = 0x100000


@pytest.mark.parametrize("name,args,needle", [
    # exact attention (and its no-allocation twin): empty batch, empty sequence, no heads, more text
    # rows than rows, NULL operands, image rows that are not whole rows of the RoPE grid
    ("moss_attention", (_P, _P, 0, 128, 2, 0, 1, 0, None), "batch, seq and heads >= 1"),
    ("moss_attention", (_P, _P, 1, 0, 2, 0, 1, 0, None), "batch, seq and heads >= 1"),
    ("moss_attention", (_P, _P, 1, 128, 0, 0, 1, 0, None), "batch, seq and heads >= 1"),
    ("moss_attention", (_P, _P, 1, 128, 2, 129, 1, 0, None), "text_len <= seq"),
    ("moss_attention", (None, _P, 1, 128, 2, 0, 1, 0, None), "need qkv and out"),
    ("moss_attention", (_P, None, 1, 128, 2, 0, 1, 0, None), "need qkv and out"),
    ("moss_attention", (_P, _P, 1, 100, 2, 10, 7, 1, None), "grid"),
    ("moss_attention_noalloc", (_P, _P, 1, 0, 2, 0, 1, 0, None), "batch, seq and heads >= 1"),
    ("moss_attention_noalloc", (_P, _P, 1, 100, 2, 10, 7, 1, None), "grid"),
    # 8-bit attention: empty shapes, a workspace one byte short or off its 256-byte alignment
    ("moss_attention_q8", (_P, _P, 0, 128, 2, _P, 1 << 30, None), "bad arguments"),
    ("moss_attention_q8", (_P, _P, 1, 128, 2, None, 1 << 30, None), "bad arguments"),
    ("moss_attention_q8", (_P, _P, 1, 128, 2, _P, "short", None), "workspace"),
    ("moss_attention_q8", (_P, _P, 1, 128, 2, _P + 16, "full", None), "workspace"),
    # bf16 GEMM: empty M, N off the 128-wide tiles, K off the 64-deep k-tiles, NULL output
    ("moss_gemm_bf16", (_P, _P, _P, 0, 128, 64, None), "M, N, K >= 1"),
    ("moss_gemm_bf16", (_P, _P, _P, 16, 100, 64, None), "N % 128"),
    ("moss_gemm_bf16", (_P, _P, _P, 16, 128, 48, None), "K % 64"),
    ("moss_gemm_bf16", (_P, _P, None, 16, 128, 64, None), "non-NULL"),
    # MXFP8 quantizer: no rows, K off the 256-element groups, scale rows fewer than rows, misaligned x
    ("moss_mx_quantize", (_P, 0, 256, _P, _P, 1, None), "rows >= 1"),
    ("moss_mx_quantize", (_P, 4, 192, _P, _P, 4, None), "K % 256"),
    ("moss_mx_quantize", (_P, 4, 256, _P, _P, 3, None), "ld_scale >= rows"),
    ("moss_mx_quantize", (_P + 8, 4, 256, _P, _P, 4, None), "16-byte aligned"),
    # MXFP8 GEMM: empty M, N off 256, scale-word strides too short or off 256
    ("moss_gemm_mxfp8", (_P, _P, 256, _P, _P, 256, _P, 0, 256, 256, None), "M, N, K >= 1"),
    ("moss_gemm_mxfp8", (_P, _P, 256, _P, _P, 256, _P, 16, 200, 256, None), "N % 256"),
    ("moss_gemm_mxfp8", (_P, _P, 256, _P, _P, 256, _P, 300, 256, 256, None), "lds_a >= M rounded up"),
    ("moss_gemm_mxfp8", (_P, _P, 512, _P, _P, 128, _P, 300, 256, 256, None), "lds_w >= N"),
    ("moss_gemm_mxfp8", (_P, _P, 300, _P, _P, 256, _P, 16, 256, 256, None), "multiples of 256"),
])
def test_ops_refuse_bad_arguments_on_the_host(name, args, needle):
    """The standalone kernel entry points refuse what their declarations rule out -- empty and ragged
    sizes, NULL pointers, short or misaligned workspaces -- with MOSS_ERR_INVALID_ARGUMENT and a message
    naming the rule, before any device work (so this runs without a GPU)."""
    if name == "moss_attention_q8":
        ws = int(dt._lib.moss_attention_q8_workspace(1, 128, 2))
        assert ws > 0
        args = tuple(ws - 1 if a == "short" else ws if a == "full" else a for a in args)
    st = getattr(dt._lib, name)(*args)
    assert st == 1, (name, args, st)
    msg = dt.moss_dit_last_error()
    assert name in msg and needle in msg, msg


def test_q8_workspace_of_empty_shapes_is_zero():
    for b, s, h in [(0, 128, 2), (1, 0, 2), (1, 128, 0), (-1, 128, 2)]:
        assert dt._lib.moss_attention_q8_workspace(b, s, h) == 0
    assert dt._lib.moss_attention_q8_workspace(1, 128, 2) > 0
