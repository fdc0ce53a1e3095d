// Host-only planning of the MOSS-Image DiT library (see host_plan.h). No HIP: built into the library by
// hipcc and, on its own, by the CPU tests under the address and undefined-behaviour sanitizers.
//
// Validation messages are written for the end user and name the rule that failed (the convention of
// the MossInfer integration guide's C API); the limits are the pages': sides a multiple of 16 px, at
// most 4096 px per side and 4.2 MP, prompts of at most 4096 tokens (MossInfer integration guide,
// per-image settings), CFG >= 1 (InvokeAI guide "MOSS-Image", "Generation settings"), skip layers
// among the model's blocks ("Skip layers").
#include "host_plan.h"

#include "moss_dit_ops.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

namespace moss {

std::string fmt(const char* f, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, f);
  vsnprintf(buf, sizeof buf, f, ap);
  va_end(ap);
  return buf;
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

void rope_table_host(float theta, float* out) {
  const int Q = kHeadDim / 4;
  for (int pos = 0; pos < kRopeMaxPos; ++pos)
    for (int k = 0; k < Q; ++k) {
      const double ang = (double)pos * std::pow((double)theta, -(double)k / Q);
      out[pos * Q + k] = (float)std::cos(ang);
      out[kRopeMaxPos * Q + pos * Q + k] = (float)std::sin(ang);
    }
}

void copy_msg(const std::string& m, char* msg, int32_t len) {
  if (msg && len > 0) {
    strncpy(msg, m.c_str(), (size_t)len - 1);
    msg[len - 1] = 0;
  }
}

std::string& thread_error() {
  thread_local std::string e;
  return e;
}

int check_config(const moss_dit_config* c, std::string& msg) {
  if (!c) {
    msg = "config is NULL";
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  if (c->struct_size != sizeof(moss_dit_config)) {
    msg = fmt("moss_dit_config.struct_size %u, this library expects %zu (fill it with moss_dit_config_init)",
              c->struct_size, sizeof(moss_dit_config));
    return MOSS_ERR_ABI_MISMATCH;
  }
  if (c->num_layers < 1 || c->hidden < 1 || c->num_heads < 1 || c->head_dim < 1 || c->ffn_hidden < 1 ||
      c->latent_channels < 1 || c->patch < 1 || c->temb_dim < 1 || !(c->norm_eps > 0.f) ||
      !(c->rope_theta > 1.f) || !std::isfinite(c->flow_multiplier)) {
    msg = "config values must be positive";
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  if (c->head_dim != kHeadDim || c->hidden != c->num_heads * c->head_dim || c->hidden % 256 != 0 ||
      c->hidden > 4096 || c->ffn_hidden % 64 != 0 || c->temb_dim != kSinusoidDim || c->patch != 2 ||
      c->num_layers > 64 || c->qk_norm != 0 || c->latent_channels * 4 % 128 != 0) {
    msg = fmt("unsupported configuration (need head_dim 128, hidden = heads*128, hidden %% 256 == 0 and <= 4096, "
              "ffn %% 64 == 0, temb 256, patch 2, channels*4 %% 128 == 0, <= 64 layers, no qk_norm)");
    return MOSS_ERR_NOT_SUPPORTED;
  }
  if (c->text_dim < 64 || c->text_dim > 16384 || c->text_dim % 64 != 0 || c->refiner_layers < 0 ||
      c->refiner_layers > 8) {
    msg = fmt("unsupported text refiner configuration (need text_dim %% 64 == 0 in [64, 16384], 0..8 refiner layers; "
              "got %d, %d)", c->text_dim, c->refiner_layers);
    return MOSS_ERR_NOT_SUPPORTED;
  }
  if (c->gemm_precision != 0 && c->gemm_precision != 1) {
    msg = fmt("gemm_precision must be 0 (bf16) or 1 (MXFP8), got %d", c->gemm_precision);
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  if (c->attention_mode != 0 && c->attention_mode != 1) {
    msg = fmt("attention_mode must be 0 (exact) or 1 (8-bit), got %d", c->attention_mode);
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  if (c->gemm_precision == 1 && c->ffn_hidden % 256 != 0) {
    msg = fmt("the MXFP8 tier needs ffn_hidden %% 256 == 0 (got %d)", c->ffn_hidden);
    return MOSS_ERR_NOT_SUPPORTED;
  }
  return MOSS_OK;
}

int check_latent(int32_t lh, int32_t lw, std::string& msg) {
  if (lh <= 0 || lw <= 0 || lh % 2 || lw % 2) {
    msg = fmt("latent height and width must be positive and even, i.e. image sides a multiple of 16 px (got %dx%d)", lh, lw);
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  if (lh > kMaxLatentSide || lw > kMaxLatentSide) {
    msg = fmt("latent sides above %d (4096 px) are not supported (got %dx%d)", kMaxLatentSide, lh, lw);
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  if (64.0 * lh * lw > kMaxPixels) {
    msg = fmt("images above 4.2 MP are not supported (latent %dx%d)", lh, lw);
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  return MOSS_OK;
}

int check_text_len(int32_t t, std::string& msg) {
  if (t < 1 || t > kMaxTextLen) {
    msg = fmt("text_len %d out of range [1, %d]", t, kMaxTextLen);
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  return MOSS_OK;
}

int validate_forward(const moss_dit_config* c, const moss_forward_args* a, std::string& msg) {
  int s = check_config(c, msg);
  if (s) return s;
  if (!a) {
    msg = "args is NULL";
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  if (a->struct_size != sizeof(moss_forward_args)) {
    msg = fmt("moss_forward_args.struct_size %u, this library expects %zu", a->struct_size, sizeof(moss_forward_args));
    return MOSS_ERR_ABI_MISMATCH;
  }
  if (a->batch < 1 || a->batch > kMaxBatch) {
    msg = fmt("batch %d out of range [1, %d]", a->batch, kMaxBatch);
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  if ((s = check_latent(a->latent_h, a->latent_w, msg))) return s;
  if ((s = check_text_len(a->text_len, msg))) return s;
  if (!a->latents || !a->text || !a->sigma || !a->velocity) {
    msg = "latents, text, sigma and velocity must not be NULL";
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  for (int b = 0; b < a->batch; ++b) {
    if (!(a->sigma[b] >= 0.f && a->sigma[b] <= 1.f)) {
      msg = fmt("sigma[%d] = %g outside [0, 1]", b, (double)a->sigma[b]);
      return MOSS_ERR_INVALID_ARGUMENT;
    }
    if (a->skip_mask && c->num_layers < 64 && (a->skip_mask[b] >> c->num_layers)) {
      msg = fmt("skip_mask[%d] names a block >= num_layers (%d)", b, c->num_layers);
      return MOSS_ERR_INVALID_ARGUMENT;
    }
  }
  return MOSS_OK;
}

int validate_step(const moss_dit_config* c, const moss_step_args* a, std::string& msg) {
  int s = check_config(c, msg);
  if (s) return s;
  if (!a) {
    msg = "args is NULL";
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  if (a->struct_size != sizeof(moss_step_args)) {
    msg = fmt("moss_step_args.struct_size %u, this library expects %zu", a->struct_size, sizeof(moss_step_args));
    return MOSS_ERR_ABI_MISMATCH;
  }
  if ((s = check_latent(a->latent_h, a->latent_w, msg))) return s;
  if ((s = check_text_len(a->text_len, msg))) return s;
  if (a->num_steps < 1) {
    msg = "num_steps must be at least 1";
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  if (a->step < 0 || a->step >= a->num_steps) {
    msg = fmt("step %d out of range [0, %d)", a->step, a->num_steps);
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  if (!std::isfinite(a->cfg_scale) || a->cfg_scale < 1.f) {
    msg = fmt("cfg_scale must be finite and >= 1 (1 = no guidance), got %g", (double)a->cfg_scale);
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  if (!std::isfinite(a->slg_start) || !std::isfinite(a->slg_stop)) {
    msg = "slg_start and slg_stop must be finite";
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  if (!std::isfinite(a->slg_scale) || a->slg_scale < 0.f) {
    msg = "slg_scale must be finite and >= 0";
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  if (!std::isfinite(a->cfg_truncation) || a->cfg_truncation < 0.f || a->cfg_truncation > 1.f) {
    msg = "cfg_truncation must be in [0, 1] (1 = off)";
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  if ((a->step_cache != 0 && a->step_cache != 1) || !std::isfinite(a->step_cache_threshold)) {
    msg = "step_cache must be 0 (off) or 1 (First-Block Cache) and step_cache_threshold finite";
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  if (!a->x || !a->text_cond || !a->sigmas) {
    msg = "x, text_cond and sigmas must not be NULL";
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  if (a->cfg_scale > 1.f && !a->text_uncond) {
    msg = "text_uncond must not be NULL when cfg_scale > 1";
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  if (a->n_skip < 0 || a->n_skip > c->num_layers || (a->n_skip > 0 && !a->uncond_skip_layers)) {
    msg = fmt("n_skip %d invalid", a->n_skip);
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  for (int i = 0; i < a->n_skip; ++i) {
    const int l = a->uncond_skip_layers[i];
    if (l < 0 || l >= c->num_layers) {
      msg = fmt("uncond_skip_layers[%d] = %d is not a block index in [0, %d]", i, l, c->num_layers - 1);
      return MOSS_ERR_INVALID_ARGUMENT;
    }
  }
  for (int i = 0; i <= a->num_steps; ++i) {
    if (!std::isfinite(a->sigmas[i])) {
      msg = fmt("sigmas[%d] is not finite", i);
      return MOSS_ERR_INVALID_ARGUMENT;
    }
  }
  return MOSS_OK;
}


int check_attention_args(const void* qkv, const void* out, int32_t batch, int32_t seq, int32_t heads,
                         int32_t text_len, int32_t grid_w, int32_t rope, std::string& msg) {
  if (!qkv || !out || batch < 1 || seq < 1 || heads < 1 || text_len < 0 || text_len > seq) {
    msg = "bad arguments (need qkv and out, batch, seq and heads >= 1, 0 <= text_len <= seq)";
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  const int n_img = seq - text_len;
  if (rope && (grid_w < 1 || n_img % grid_w != 0 || grid_w > kRopeMaxPos || n_img / grid_w > kRopeMaxPos)) {
    msg = "image rows must fill a grid of width grid_w (<= 256 per side)";
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  if (2L * seq * 3 * heads * kHeadDim > 0x7fffffffL) {
    msg = "one sample's qkv rows must stay below 2 GiB";
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  return MOSS_OK;
}

StepPlan step_plan(const moss_step_args* a) {
  // The skip-layer window is on the progress step/num_steps, inclusive at both ends; the negative
  // branch runs for cfg > 1 until step cfg_truncation * num_steps; the third row runs inside the
  // window when slg_scale > 0 and there is a layer to skip.
  StepPlan p{};
  const double prog = (double)a->step / (double)a->num_steps;
  const bool window = (double)a->slg_start <= prog && prog <= (double)a->slg_stop;
  uint64_t mask = 0;
  if (window)
    for (int i = 0; i < a->n_skip; ++i) mask |= 1ULL << a->uncond_skip_layers[i];
  p.neg = a->cfg_scale > 1.f && (double)a->step < (double)a->cfg_truncation * (double)a->num_steps;
  p.third = a->slg_scale > 0.f && mask != 0;
  p.rows = 1 + (p.neg ? 1 : 0) + (p.third ? 1 : 0);
  for (int r = 0; r < p.rows; ++r) p.skip[r] = r == 0 ? 0 : mask;
  return p;
}

AttnSplitPlan attention_split_plan(int B, int S, int H, long slots) {
  AttnSplitPlan sp{};
  const long total = (long)((S + kAttnBQ - 1) / kAttnBQ) * H * B;
  const int ntiles = (S + kAttnBKV - 1) / kAttnBKV;
  sp.n_full = (int)total;
  sp.n_split = 0;
  sp.parts = 1;
  // whole rounds stay unsplit; a last round holding at most half the slots is split into parts
  if (slots > 0 && total > slots) {
    const long rem = total % slots;
    const int parts = rem > 0 ? (int)std::min<long>(std::min<long>(slots / rem, ntiles / 2), 8) : 1;
    if (rem > 0 && rem * 2 <= slots && parts >= 2) {
      sp.n_full = (int)(total - rem);
      sp.n_split = (int)rem;
      sp.parts = parts;
    }
  }
  return sp;
}

size_t attention_split_bytes(int B, int S, int H, long slots) {
  const AttnSplitPlan sp = attention_split_plan(B, S, H, slots);
  const size_t rows = (size_t)sp.n_split * sp.parts * kAttnBQ;
  return rows == 0 ? 0 : rows * kHeadDim * 4 + rows * 2 * 4 + 256;
}

size_t attention_q8_bytes(int B, int S, int H) {
  const size_t nblk = (size_t)(S + kAttnBKV - 1) / kAttnBKV, M = (size_t)B * S, DM = (size_t)H * kHeadDim;
  return align_up(M * DM) * 2 + align_up((size_t)B * H * kHeadDim * nblk * kAttnBKV) + align_up(M * H * 4) +
         align_up((size_t)B * H * nblk * 4) + align_up((size_t)B * H * kHeadDim * 4) +
         align_up((size_t)B * H * nblk * kHeadDim * 4);
}

WsLayout ws_layout(const moss_dit_config& k, int B, int S, int N, long lat_elems, long attn_slots) {
  const size_t D = k.hidden, F = k.ffn_hidden, P = (size_t)k.latent_channels * 4;
  const size_t M = (size_t)B * S;
  const size_t mod_rows = (size_t)k.num_layers * 6 * D + 2 * D;
  WsLayout t;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t p = off;
    off += align_up(bytes);
    return p;
  };
  t.x = take(M * D * 2);
  t.a = take(M * D * 2);
  t.qkv = take(M * 3 * D * 2);
  t.o = take(M * D * 2);
  t.h = take(M * F * 2);
  t.tokens = take((size_t)B * N * P * 2);
  t.mod = take((size_t)B * mod_rows * 2);
  t.u = take((size_t)B * k.temb_dim * 4);
  t.vel = take((size_t)B * lat_elems * 4);         // one velocity per row of the batch
  t.q8 = t.s8 = t.q8h = t.s8h = kNoRegion;
  t.lds8 = (long)((M + 255) / 256 * 256);
  if (k.gemm_precision == 1) {
    const size_t Kmax = std::max(D, F);
    t.q8 = take(M * Kmax);
    t.s8 = take(Kmax / 128 * (size_t)t.lds8 * 4);
    t.q8h = take(M * F);
    t.s8h = take(F / 128 * (size_t)t.lds8 * 4);
  }
  t.attn_split_bytes = attention_split_bytes(B, S, k.num_heads, attn_slots);
  t.attn_split = t.attn_split_bytes ? take(t.attn_split_bytes) : kNoRegion;
  t.attn8_bytes = 0;
  t.attn8 = kNoRegion;
  if (k.attention_mode == 1) {
    t.attn8_bytes = attention_q8_bytes(B, S, k.num_heads);
    t.attn8 = take(t.attn8_bytes);
  }
  t.total = off;
  return t;
}

}  // namespace moss

// =============================================================================================
// exported host-only functions of the C ABI (moss_dit.h, moss_dit_ops.h)
// =============================================================================================
using namespace moss;

extern "C" {

int moss_dit_abi_version(void) { return MOSS_DIT_ABI_VERSION; }

const char* moss_status_string(int s) {
  switch (s) {
    case MOSS_OK: return "ok";
    case MOSS_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOSS_ERR_NOT_SUPPORTED: return "not supported";
    case MOSS_ERR_OUT_OF_MEMORY: return "out of device memory";
    case MOSS_ERR_DEVICE: return "device error";
    case MOSS_ERR_ABI_MISMATCH: return "ABI mismatch";
    default: return "unknown status";
  }
}


void moss_dit_config_init(moss_dit_config* c, uint32_t size) {
  if (!c) return;
  moss_dit_config d;
  d.struct_size = size;
  d.num_layers = 42;
  d.hidden = 3072;
  d.num_heads = 24;
  d.head_dim = 128;
  d.ffn_hidden = 8192;
  d.latent_channels = 32;
  d.patch = 2;
  d.temb_dim = 256;
  d.qk_norm = 0;
  d.rope_theta = 1.0e4f;
  d.norm_eps = 1.0e-6f;
  d.flow_multiplier = 1000.f;
  d.text_dim = 4096;
  d.refiner_layers = 2;
  d.gemm_precision = 0;
  d.attention_mode = 0;
  memcpy(c, &d, size < sizeof d ? size : sizeof d);
}

void moss_dit_weights_init(moss_dit_weights* w, uint32_t size) {
  if (!w) return;
  moss_dit_weights d;
  memset(&d, 0, sizeof d);
  d.struct_size = size;
  memcpy(w, &d, size < sizeof d ? size : sizeof d);
}

void moss_forward_args_init(moss_forward_args* a, uint32_t size) {
  if (!a) return;
  moss_forward_args d;
  memset(&d, 0, sizeof d);
  d.struct_size = size;
  d.batch = 1;
  d.latent_h = d.latent_w = 128;
  d.text_len = 256;
  memcpy(a, &d, size < sizeof d ? size : sizeof d);
}

static const int32_t kDefaultSkip[1] = {22};

void moss_step_args_init(moss_step_args* a, uint32_t size) {
  if (!a) return;
  moss_step_args d;
  memset(&d, 0, sizeof d);
  d.struct_size = size;
  d.latent_h = d.latent_w = 128;
  d.text_len = 256;
  d.num_steps = 50;
  d.step = 0;
  d.cfg_scale = 3.0f;
  d.slg_start = 0.01f;
  d.slg_stop = 1.0f;
  d.uncond_skip_layers = kDefaultSkip;
  d.n_skip = 1;
  d.slg_scale = 0.0f;
  d.cfg_truncation = 1.0f;
  d.step_cache = 0;
  d.step_cache_threshold = 0.0f;
  memcpy(a, &d, size < sizeof d ? size : sizeof d);
}

void moss_block_taps_init(moss_block_taps* t, uint32_t size) {
  if (!t) return;
  moss_block_taps d;
  memset(&d, 0, sizeof d);
  d.struct_size = size;
  memcpy(t, &d, size < sizeof d ? size : sizeof d);
}

int moss_sigmas(int32_t num_steps, float shift, float* sigmas) {
  if (num_steps < 1 || !sigmas || !(shift > 0.f) || !std::isfinite(shift)) {
    thread_error() = "num_steps must be >= 1, shift > 0 and sigmas non-NULL";
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  for (int i = 0; i <= num_steps; ++i) {
    const double s = (double)(num_steps - i) / (double)num_steps;
    sigmas[i] = (float)((double)shift * s / (1.0 + ((double)shift - 1.0) * s));
  }
  return MOSS_OK;
}

int moss_validate_forward_args(const moss_dit_config* cfg, const moss_forward_args* a, char* msg, int32_t msg_len) {
  std::string m;
  const int s = validate_forward(cfg, a, m);
  copy_msg(s ? m : std::string("ok"), msg, msg_len);
  return s;
}

int moss_validate_step_args(const moss_dit_config* cfg, const moss_step_args* a, char* msg, int32_t msg_len) {
  std::string m;
  const int s = validate_step(cfg, a, m);
  copy_msg(s ? m : std::string("ok"), msg, msg_len);
  return s;
}

}  // extern "C"
