"""A pytest plugin that plants ONE named mistake in the CPU oracle, to show that the oracle's pins
(tests/test_oracle_pins.py) catch it. Loaded only by tests/test_oracle_mutations.py, in a child
pytest run (``-p tests.oracle_mutants``, mistake named by MOSS_ORACLE_MUTANT); nothing else imports it.
Each mistake replaces one oracle function, in both the module and the package namespace, by a wrong
variant built around the original."""
import math
import os

import numpy as np

import oracle
import oracle.moss_oracle as M


def _swap_final(orig):
    return lambda x_img, m_f, W, cfg, mirror=False: orig(x_img, m_f[::-1], W, cfg, mirror)


def _swiglu_swap(orig):
    def block(x, m, W, l, cfg, *a, **k):
        F = cfg.ffn_hidden
        gu = W["gate_up_w"][l]
        W2 = dict(W)
        W2["gate_up_w"] = list(W["gate_up_w"])
        W2["gate_up_w"][l] = np.concatenate([gu[F:], gu[:F]], axis=0)
        return orig(x, m, W2, l, cfg, *a, **k)
    return block


def _ddof(orig):
    def layernorm(x, eps):
        mu = x.mean(axis=-1, keepdims=True)
        var = ((x - mu) ** 2).sum(axis=-1, keepdims=True) / (x.shape[-1] - 1)
        return (x - mu) / np.sqrt(var + eps)
    return layernorm


def _patch_order(orig):
    def patchify(latent, p=2):
        out = orig(latent, p)
        n, cpp = out.shape
        return out.reshape(n, cpp // (p * p), p, p).transpose(0, 1, 3, 2).reshape(n, cpp)
    return patchify


def _shift_formula(orig):
    def sigmas(num_steps, shift=5.0):
        s = orig(num_steps, 1.0)                    # the linear grid
        return s / (shift - (shift - 1.0) * s)
    return sigmas


def _sincos(orig):
    def time_features(sigma, cfg):
        e = orig(sigma, cfg)
        h = e.shape[0] // 2
        return np.concatenate([e[h:], e[:h]])
    return time_features


def _cfg(orig):
    return lambda v_cond, v_uncond, cfg_scale: (v_cond if v_uncond is None
                                                 else v_cond + cfg_scale * (v_cond - v_uncond))


MUTANTS = {
    # name: (function name, wrapper around the original)
    "rope_sign": ("apply_rope", lambda orig: (lambda v, angles: orig(v, -angles))),
    "attention_scale": ("attention", lambda orig: (lambda q, k, v, H, d: orig(q / math.sqrt(d), k, v, H, d))),
    "swapped_gates": ("block", lambda orig: (lambda x, m, *a, **k: orig(x, m[[0, 1, 5, 3, 4, 2]], *a, **k))),
    "missing_one_plus": ("ln_modulate", lambda orig: (lambda x, shift, scale, eps: orig(x, shift, scale - 1.0, eps))),
    "rope_halves": ("rope_angles", lambda orig: (lambda pr, pc, d, theta: orig(pc, pr, d, theta))),
    "patch_order": ("patchify", _patch_order),
    "shift_formula": ("sigmas", _shift_formula),
    "swiglu_operands": ("block", _swiglu_swap),
    "variance_ddof": ("layernorm", _ddof),
    "reversed_v": ("attention", lambda orig: (lambda q, k, v, H, d: orig(q, k, v[::-1], H, d))),
    "sincos_order": ("time_features", _sincos),
    "cfg_formula": ("cfg_combine", _cfg),
    "exclusive_window": ("slg_active", lambda orig: (
        lambda step, n, slg_start=0.01, slg_stop=1.0: slg_start < step / n < slg_stop)),
    "final_shift_scale": ("final_layer", _swap_final),
}

_name = os.environ.get("MOSS_ORACLE_MUTANT", "none")
if _name != "none":
    fn, wrap = MUTANTS[_name]
    bad = wrap(getattr(M, fn))
    setattr(M, fn, bad)
    if hasattr(oracle, fn):
        setattr(oracle, fn, bad)
