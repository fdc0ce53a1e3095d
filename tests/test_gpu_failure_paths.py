"""Failure paths of the C ABI on the GPU, forced from the host (no kernel faults or hangs):

* allocation failure (MOSS_DIT_FAIL_ALLOC=1 makes every device allocation of the library fail):
  moss_dit_create returns MOSS_ERR_OUT_OF_MEMORY and leaves nothing behind; a handle whose workspace
  allocation fails returns MOSS_ERR_OUT_OF_MEMORY from the call and stays usable -- the next call,
  with allocation working again, gives the same bits as a fresh handle;
* device error (MOSS_DIT_FAIL_LAUNCH=n reports the n-th checked HIP call of the thread as a failed
  launch; the launch itself ran normally): the call returns MOSS_ERR_DEVICE, and every later call on
  that handle returns MOSS_ERR_DEVICE until it is destroyed, as the MossInfer integration guide's C-API
  rules have a caller free the engine after a device error; a new handle works.

Tiny model: 2 blocks, hidden 256, 2 heads x 128, FFN 704, 16x16 latent + 32 text tokens, seed 0."""
import os

import numpy as np
import pytest

import synth
from tests.gpu_util import dev_weights, log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
dt = pytest.importorskip("diffusion_transformer_text_amd")


def _tiny():
    w, inp = synth.tiny_workload(mod_scale=50.0)
    s = synth.TINY
    cfg = dt.moss_dit_config_init(num_layers=s.num_layers, hidden=s.hidden, num_heads=s.num_heads,
                                  ffn_hidden=s.ffn_hidden)
    return cfg, dev_weights(w, torch), inp


def _forward(m, inp):
    lat = torch.from_numpy(np.concatenate([inp.latents, inp.latents])).cuda()
    txt = torch.from_numpy(np.concatenate([inp.text_cond, inp.text_uncond])).cuda()
    vel = torch.full_like(lat, float("nan"))
    m.moss_dit_forward(lat, txt, [0.6, 0.6], vel, skip_mask=[0, 1 << 1])
    torch.cuda.synchronize()
    return vel.cpu().numpy()


class _env:
    def __init__(self, name, value):
        self.name, self.value = name, value

    def __enter__(self):
        os.environ[self.name] = self.value

    def __exit__(self, *a):
        os.environ.pop(self.name, None)


def test_allocation_failure_create_and_workspace():
    cfg, dw, inp = _tiny()
    log("MOSS_DIT_FAIL_ALLOC: create")
    with _env("MOSS_DIT_FAIL_ALLOC", "1"):
        with pytest.raises(dt.MossError) as ei:
            dt.MossDiT(cfg, dw)
    assert ei.value.status == dt.MOSS_ERR_OUT_OF_MEMORY
    assert "allocation" in str(ei.value)
    ref_model = dt.MossDiT(cfg, dw)           # allocation works again
    ref = _forward(ref_model, inp)
    assert np.isfinite(ref).all()
    ref_model.close()
    log("MOSS_DIT_FAIL_ALLOC: workspace of a live handle")
    m = dt.MossDiT(cfg, dw)
    with _env("MOSS_DIT_FAIL_ALLOC", "1"):
        with pytest.raises(dt.MossError) as ei:
            _forward(m, inp)                   # the first call allocates the workspace
    assert ei.value.status == dt.MOSS_ERR_OUT_OF_MEMORY
    assert "workspace" in m.last_error()
    got = _forward(m, inp)                     # the handle stays usable
    np.testing.assert_array_equal(got, ref)
    m.close()


@pytest.mark.parametrize("n", [1, 7, 20])   # a tiny forward makes 21 checked HIP calls
def test_injected_device_error_kills_the_handle(n):
    cfg, dw, inp = _tiny()
    m = dt.MossDiT(cfg, dw)
    ref = _forward(m, inp)
    log(f"MOSS_DIT_FAIL_LAUNCH={n}")
    with _env("MOSS_DIT_FAIL_LAUNCH", str(n)):
        with pytest.raises(dt.MossError) as ei:
            _forward(m, inp)
    assert ei.value.status == dt.MOSS_ERR_DEVICE
    torch.cuda.synchronize()                  # what was enqueued before the failure completes normally
    # dead until destroyed: forward, sampling step and modulation all refuse
    with pytest.raises(dt.MossError) as ei:
        _forward(m, inp)
    assert ei.value.status == dt.MOSS_ERR_DEVICE and "destroy" in m.last_error()
    x = torch.from_numpy(inp.latents.copy()).cuda()
    with pytest.raises(dt.MossError) as ei:
        m.moss_sample_step(x, torch.from_numpy(inp.text_cond).cuda(), torch.from_numpy(inp.text_uncond).cuda(),
                           dt.moss_sigmas(2, 5.0), 0, uncond_skip_layers=[1])
    assert ei.value.status == dt.MOSS_ERR_DEVICE
    mod = torch.empty((1, m.mod_stride), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dt.MossError) as ei:
        m.moss_dit_modulation([0.5], mod)
    assert ei.value.status == dt.MOSS_ERR_DEVICE
    m.close()
    m2 = dt.MossDiT(cfg, dw)                   # a new handle works and gives the same bits
    np.testing.assert_array_equal(_forward(m2, inp), ref)
    m2.close()
