"""The step cache (First-Block Cache, opt-in and lossy) on the GPU, tiny model with the x50 modulation
(block updates survive the bf16 residual), 3 Euler steps, CFG 3:

* threshold 0 never reuses: every step equals the plain step bit for bit;
* with the gates of blocks 1.. zeroed those blocks are identities, the cached rest is exactly 0 and a
  reused call gives the full call's bits;
* a huge threshold reuses every call after the first unless the row plan changes (the negative pass
  starting to skip block 1 at step 1 restarts the cache); each step against the oracle's cached step
  from the same input; the measured change against the oracle's.
"""
import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_util import REL_L2_BF16, log, oracle_cfg, rel_l2

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
dt = pytest.importorskip("diffusion_transformer_text_amd")
from tests.test_gpu_model import model, tiny_cfg  # noqa: E402


def _run(m, inp, sig, n, skip, **kw):
    tc = torch.from_numpy(inp.text_cond).cuda()
    tu = torch.from_numpy(inp.text_uncond).cuda()
    x = torch.from_numpy(inp.latents.copy()).cuda()
    xs = []
    for i in range(n):
        m.moss_sample_step(x, tc, tu, sig, i, cfg_scale=3.0, uncond_skip_layers=skip, **kw)
        torch.cuda.synchronize()
        xs.append(x.cpu().numpy().copy())
    return xs


def test_step_cache_threshold_zero_and_identity_blocks_bitwise():
    m, w, inp, W, ocfg, dw = model(50.0)
    sig = dt.moss_sigmas(3, 5.0)
    plain = _run(m, inp, sig, 3, [1])
    cached = _run(m, inp, sig, 3, [1], step_cache=True, step_cache_threshold=1e-30)
    for a, b in zip(plain, cached):
        np.testing.assert_array_equal(a, b)
    full, reused, change = m.moss_step_cache_stats()
    log(f"threshold ~0: full {full}, reused {reused}, last change {change:.3e}")
    assert (full, reused) == (3, 0) and change > 0
    # blocks 1.. as identities: reused calls are exact
    D = ocfg.hidden
    dw2 = dict(dw)
    dw2["mod_w"] = [dw["mod_w"][0]]
    for l in range(1, ocfg.num_layers):
        t = dw["mod_w"][l].clone()
        t[2 * D:3 * D] = 0
        t[5 * D:] = 0
        dw2["mod_w"].append(t)
    m2 = dt.MossDiT(tiny_cfg(), dw2)
    plain = _run(m2, inp, sig, 3, [])
    cached = _run(m2, inp, sig, 3, [], step_cache=True, step_cache_threshold=1e9)
    assert m2.moss_step_cache_stats()[:2] == (1, 2)
    for a, b in zip(plain, cached):
        np.testing.assert_array_equal(a, b)
    m2.close()


@pytest.mark.parametrize("skip,expect", [((), (1, 2)), ((1,), (2, 1))])
def test_step_cache_reuse_vs_oracle(skip, expect):
    m, w, inp, W, ocfg, _ = model(50.0)
    sig = dt.moss_sigmas(3, 5.0)
    xs = _run(m, inp, sig, 3, list(skip), step_cache=True, step_cache_threshold=1e9)
    full, reused, change = m.moss_step_cache_stats()
    assert (full, reused) == expect
    # the oracle runs the same cached sampling; each step is compared from the same input x_i
    f = lambda a: np.asarray(a, dtype=np.float64)
    cache = O.StepCache()
    x_prev = f(inp.latents)
    plain = _run(m, inp, sig, 3, list(skip))
    for i in range(3):
        ref = O.sample_step_cached(x_prev, f(inp.text_cond), f(inp.text_uncond), W, ocfg, i, f(sig), cache, 1e9, 3.0,
                                   skip, mirror=True)
        e = rel_l2(xs[i] - x_prev, ref - x_prev)
        log(f"skip {skip} step {i}: update rel-L2 {e:.2e}; reused-vs-plain differ: {not np.array_equal(xs[i], plain[i])}")
        assert e <= REL_L2_BF16
        x_prev = xs[i].astype(np.float64)
    assert (cache.full_calls, cache.reused_calls) == expect
    log(f"last change: GPU {change:.4e}, oracle {cache.last_change:.4e}")
    assert abs(change - cache.last_change) <= 0.1 * abs(cache.last_change)
