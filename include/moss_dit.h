/* moss_dit.h -- C ABI of the MI355X (gfx950) MOSS-Image DiT denoising step.
 *
 * What the library computes (pages cited by title and section):
 *   - one forward pass of the single-stream diffusion transformer: 42 joint blocks, hidden 3072,
 *     24 heads of 128, FFN 8192, over the joint sequence [text tokens | 2x2-patch image tokens]
 *     ("MOSS-Image: specs, settings, VRAM and text rendering tested", table "Architecture and specs");
 *   - one denoising step: a conditional and an unconditional pass (the unconditional one skipping
 *     the blocks in uncond_skip_layers inside the slg_start..slg_stop window), the FP32 CFG combine
 *     and the flow-matching Euler update with shift 5 ("MOSS-Image" SGLang cookbook, section
 *     "3. Guidance and precision"; InvokeAI user guide "MOSS-Image", sections "Generation settings"
 *     and "Skip layers").
 * The text encoder and the VAE are not part of the library: the caller passes text states of width
 * `hidden` (standing in for the text refiner's output) and latents of `latent_channels` channels.
 *
 * Conventions (modelled on the C API rules of the MossInfer integration guide):
 *   - Each struct is prepared by its *_init(&s, sizeof s) call, and only then are its fields set.
 *     A struct_size other than this header's size makes the call return MOSS_ERR_ABI_MISMATCH.
 *   - Device pointers are HIP device memory of the device current at moss_dit_create, allocated and
 *     owned by the caller (e.g. torch tensors); the library only borrows them for the call. The
 *     handle owns a copy of the weights and its workspace.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Compute calls validate all
 *     arguments on the host first (no device work on error), then enqueue on the stream and return;
 *     device-side faults surface at the caller's next synchronisation.
 *   - Every function returns a moss_status. After MOSS_ERR_DEVICE the handle is dead: every later
 *     call on it returns MOSS_ERR_DEVICE; destroy it.
 *   - One call at a time per handle. Different handles may be used from different threads.
 *   - Layouts are row-major; bf16 tensors are 16-bit bfloat16 bit patterns.
 */
#ifndef MOSS_DIT_H
#define MOSS_DIT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOSS_DIT_ABI_VERSION 1

typedef enum {
  MOSS_OK = 0,
  MOSS_ERR_INVALID_ARGUMENT = 1, /* a value or pointer the call does not accept; message says which */
  MOSS_ERR_NOT_SUPPORTED = 2,    /* a configuration the kernels do not implement */
  MOSS_ERR_OUT_OF_MEMORY = 3,    /* device allocation failed; the handle stays usable */
  MOSS_ERR_DEVICE = 4,           /* a HIP runtime error; the handle is dead */
  MOSS_ERR_ABI_MISMATCH = 5      /* struct_size differs from this header's */
} moss_status;

typedef struct moss_dit moss_dit; /* opaque handle */

/* Returns MOSS_DIT_ABI_VERSION of the built library; refuse to run when it differs. */
int moss_dit_abi_version(void);
/* Static English text of a status code. */
const char* moss_status_string(int status);
/* Message of the last failed call on h, or of the calling thread's last failed call that had no
 * handle (h == NULL). Valid until the next call on the same handle / thread. Never NULL. */
const char* moss_dit_last_error(const moss_dit* h);

/* ---------------------------------------------------------------------------------------------
 * Model configuration. Defaults (moss_dit_config_init) are MOSS-Image's: 42 layers, hidden 3072,
 * 24 heads of 128, FFN 8192, 32 latent channels, 2x2 patches ("Architecture and specs"), and the
 * readings where the pages are silent: time-embedding width 256, RoPE theta 1e4, LayerNorm eps 1e-6,
 * flow multiplier 1000 (t = 1000 * sigma), no QK-norm; for the text refiner (a projection and two
 * blocks over the text rows alone, applied to the text encoder's last hidden states, "Architecture and
 * specs"):
 * encoder state width 4096 and 2 refiner blocks.
 * Supported: head_dim == 128, hidden == num_heads * 128, hidden % 256 == 0, hidden <= 4096,
 * ffn_hidden % 64 == 0, temb_dim == 256, patch == 2, 1 <= num_layers <= 64, qk_norm == 0,
 * text_dim % 64 == 0 and 64 <= text_dim <= 16384, 0 <= refiner_layers <= 8;
 * anything else -> MOSS_ERR_NOT_SUPPORTED.
 * gemm_precision = 1 selects the FP8 tier (lossy: the pages' "high/turbo" tiers run FP8 GEMMs, MossInfer
 * integration guide "Quality tier", Qwen-Image 2.1 cookbook "Online FP8"): the four projections of
 * every joint block (DiT and text refiner) quantize both operands to OCP MXFP8 -- E4M3 with one
 * power-of-two scale per 32 elements along the reduction axis, weights once at creation, activations
 * on the fly -- and run on the scaled FP8 matrix cores with fp32 accumulation; everything else stays
 * as in the bf16 tier. Needs ffn_hidden % 256 == 0. The pages' tiers use channel- or tensor-wise
 * scales; the block format is the one gfx950's FP8 matrix instruction applies in hardware.
 * attention_mode = 1 runs every joint block's attention in 8 bits, the pages' q8_fp8 mode (MossInfer
 * integration guide, "Quality tier": the faster tiers pair their GEMMs with 8-bit attention); the
 * arithmetic is the one moss_attention_q8 (moss_dit_ops.h) states. Independent of gemm_precision. */
typedef struct {
  uint32_t struct_size;
  int32_t num_layers, hidden, num_heads, head_dim, ffn_hidden, latent_channels, patch, temb_dim, qk_norm;
  float rope_theta, norm_eps, flow_multiplier;
  int32_t text_dim;                /* width of the text encoder's states (input of the text refiner)   */
  int32_t refiner_layers;          /* text-only blocks after the text projection                       */
  int32_t gemm_precision;          /* block projections: 0 = bf16 (default), 1 = MXFP8 (lossy FP8 tier) */
  int32_t attention_mode;          /* 0 = exact (default), 1 = 8-bit (q8_fp8: INT8 Q K^T, FP8 P V; lossy) */
} moss_dit_config;
void moss_dit_config_init(moss_dit_config* c, uint32_t size);

/* ---------------------------------------------------------------------------------------------
 * Weights: bf16, every linear [out_features, in_features] row-major, no biases. The library copies
 * (and re-lays out) them at moss_dit_create; the caller may free its copy afterwards.
 * Per-block arrays hold num_layers pointers. */
typedef struct {
  uint32_t struct_size;
  const void* t_w1;                /* [temb, 256]   time MLP layer 1 (on the sinusoidal features)      */
  const void* t_w2;                /* [temb, temb]  time MLP layer 2                                   */
  const void* x_embed_w;           /* [hidden, C*p*p] patch embedding                                  */
  const void* const* mod_w;        /* L x [6*hidden, temb]: (shift1, scale1, gate1, shift2, scale2, gate2) */
  const void* const* qkv_w;        /* L x [3*hidden, hidden]: rows [q | k | v], head h at rows h*128.. */
  const void* const* out_w;        /* L x [hidden, hidden]                                             */
  const void* const* gate_up_w;    /* L x [2*ffn, hidden]: rows [gate | up]                             */
  const void* const* down_w;       /* L x [hidden, ffn]                                                */
  /* Per-head RMSNorm weights of q and k (L x [head_dim]) for a model with QK-norm. The pages mention a
   * Q/K normalization only for another single-stream DiT (Qwen-Image 2.1 cookbook, "Lossless Q/K
   * normalization"); MOSS-Image is read as having none, so qk_norm must be 0 and these are ignored
   * (leave them NULL). The fields keep the struct's layout stable for a later QK-norm build. */
  const void* const* q_norm_w;
  const void* const* k_norm_w;
  const void* final_mod_w;         /* [2*hidden, temb]: (shift_f, scale_f)                              */
  const void* final_w;             /* [C*p*p, hidden] output projection                                */
  /* Text refiner (optional: text_proj_w == NULL leaves it out and moss_text_refine returns
   * MOSS_ERR_NOT_SUPPORTED). The refiner blocks have the joint blocks' layout and widths. */
  const void* text_proj_w;                 /* [hidden, text_dim]                                      */
  const void* const* refiner_qkv_w;        /* refiner_layers x [3*hidden, hidden]                     */
  const void* const* refiner_out_w;        /* refiner_layers x [hidden, hidden]                       */
  const void* const* refiner_gate_up_w;    /* refiner_layers x [2*ffn, hidden]: rows [gate | up]      */
  const void* const* refiner_down_w;       /* refiner_layers x [hidden, ffn]                          */
} moss_dit_weights;
void moss_dit_weights_init(moss_dit_weights* w, uint32_t size);

/* Validates the config, allocates the weight copy on the current device, copies and re-lays out the
 * weights (weights_on_device != 0: device pointers, else host pointers), builds the RoPE tables.
 * Enqueues on `stream` and synchronises it before returning. *out = NULL on failure. */
int moss_dit_create(const moss_dit_config* cfg, const moss_dit_weights* w, int weights_on_device,
                    void* stream, moss_dit** out);
/* Frees everything the handle owns (synchronises the device first). NULL is a no-op. */
void moss_dit_destroy(moss_dit* h);

/* ---------------------------------------------------------------------------------------------
 * One DiT forward pass on a batch of independent samples. */
typedef struct {
  uint32_t struct_size;
  int32_t batch;                 /* 1 .. 8                                                            */
  int32_t latent_h, latent_w;    /* latent size (8x downsampled pixels): even, <= 512 per side,      *
                                  * 64*h*w <= 4.2e6 pixels                                           */
  int32_t text_len;              /* 1 .. 4096                                                         */
  const float* latents;          /* device fp32 [B, C, latent_h, latent_w]                            */
  const float* text;             /* device fp32 [B, text_len, hidden]                                 */
  const float* sigma;            /* host fp32 [B], in [0, 1]                                          */
  const uint64_t* skip_mask;     /* host [B]: bit l set = sample b skips block l; NULL = none          */
  float* velocity;               /* device fp32 [B, C, latent_h, latent_w] (output)                   */
  void* residual_dump;           /* optional device bf16 [num_layers + 1, B, text_len + N, hidden]:   *
                                  * the residual stream after the embedding and after each block      *
                                  * (a skipped block repeats its input); NULL = not written           */
} moss_forward_args;
void moss_forward_args_init(moss_forward_args* a, uint32_t size);
int moss_dit_forward(moss_dit* h, const moss_forward_args* a, void* stream);
/* Host-only check of forward arguments (no GPU needed). msg (may be NULL) receives the reason. */
int moss_validate_forward_args(const moss_dit_config* cfg, const moss_forward_args* a, char* msg, int32_t msg_len);

/* ---------------------------------------------------------------------------------------------
 * Text refiner: out = refine(enc), run once per prompt before the denoising loop; `out` is what
 * moss_dit_forward / moss_sample_step take as text states: a projection followed by two blocks over
 * the text rows alone, applied to the text encoder's last hidden states ("MOSS-Image: specs, settings,
 * VRAM and text rendering tested", "Architecture and specs"). Readings (the pages say no more): the projection has no bias;
 * the text-only blocks are joint blocks of the same widths run on the text rows alone, without
 * timestep modulation (unmodulated LayerNorm, gates 1: they depend on the prompt only) and without
 * RoPE. bf16 storage as in the DiT; the result is written as fp32 (exact bf16 values).
 *   enc: device fp32 [batch, text_len, text_dim], 16-byte aligned; out: device fp32
 *   [batch, text_len, hidden]. 1 <= batch <= 8, 1 <= text_len <= 4096. Samples are independent.
 * Returns MOSS_ERR_NOT_SUPPORTED when the handle was created without refiner weights. */
int moss_text_refine(moss_dit* h, int32_t batch, int32_t text_len, const float* enc, float* out, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Sigma schedule of the flow-matching Euler sampler with flow shift `shift` (5 by default: "MOSS-Image"
 * SGLang cookbook, "3. Guidance and precision"; "MOSS-Image: specs, settings, VRAM and text rendering
 * tested", "Recommended settings": 50 steps, flow-matching Euler, shift 5). The pages name the shift
 * but print no formula; the reading is the usual shifted flow-matching time grid:
 *   sigmas[i] = shift*s/(1 + (shift-1)*s), s = (num_steps - i)/num_steps, i = 0..num_steps
 * (computed in double, stored fp32; sigmas[0] = 1, sigmas[num_steps] = 0). Host only.
 * Errors: MOSS_ERR_INVALID_ARGUMENT for num_steps < 1, shift <= 0 or not finite, sigmas == NULL. */
int moss_sigmas(int32_t num_steps, float shift, float* sigmas /* host [num_steps + 1] */);

/* ---------------------------------------------------------------------------------------------
 * One denoising step of one image: x_{step+1} = x_step + (sigma_{step+1} - sigma_step) * v.
 *   - The conditional pass always runs: v_c.
 *   - The negative (unconditional) pass runs when cfg_scale > 1 and step < cfg_truncation *
 *     num_steps, skipping uncond_skip_layers when slg_start <= step/num_steps <= slg_stop
 *     ("MOSS-Image" SGLang cookbook, "3. Guidance and precision"; CFG truncation leaves the negative
 *     branch out of the last (1 - X) of the steps: MossInfer integration guide, feature table "Lossy
 *     accelerators").
 *     Then v = v_u + cfg_scale * (v_c - v_u), else v = v_c.
 *   - Three-pass skip-layer guidance (slg_scale > 0; the cookbook's "adds a skipped conditional
 *     prediction"): inside the same window, a third pass runs the conditional input skipping the
 *     same uncond_skip_layers, v_s, and v += slg_scale * (v_c - v_s). The pages give no formula; this
 *     is the skip-layer guidance form. slg_scale = 0 (default) is the two-pass recipe.
 *   - Step cache (step_cache = 1, off by default; lossy: it changes the image): the First-Block Cache
 *     of the MossInfer integration guide ("Lossy accelerators"): as long as block 0's output moves
 *     less than step_cache_threshold between calls (<= 0: 0.02, the base model's default), blocks 1..
 *     are taken from the last call that ran them. Readings: the change is sum|r - r_prev| / sum|r_prev| with r = the
 *     residual stream after block 0 minus the one before it (all rows of the call) and r_prev the same
 *     at the last full call; a reused call takes the stream after the last block as bf16(x after block
 *     0 + the difference of those two streams at the last full call). A call whose rows (batch, shapes,
 *     per-row skip sets) differ from the cached call's, and every step 0, runs in full and restarts
 *     the cache. The cache lives in the handle; reading the change synchronises `stream` once per call.
 * All guidance arithmetic is fp32. */
typedef struct {
  uint32_t struct_size;
  int32_t latent_h, latent_w, text_len, num_steps, step;
  float* x;                          /* device fp32 [1, C, latent_h, latent_w], updated in place      */
  const float* text_cond;            /* device fp32 [1, text_len, hidden]                             */
  const float* text_uncond;          /* device fp32 [1, text_len, hidden]; NULL allowed iff cfg == 1   */
  const float* sigmas;               /* host fp32 [num_steps + 1] (e.g. from moss_sigmas)              */
  float cfg_scale;                   /* >= 1                                                          */
  float slg_start, slg_stop;
  const int32_t* uncond_skip_layers; /* host [n_skip], each in [0, num_layers)                       */
  int32_t n_skip;
  float slg_scale;                   /* >= 0; > 0 runs the third (skipped conditional) pass           */
  float cfg_truncation;              /* in [0, 1]; 1 = off                                            */
  int32_t step_cache;                /* 0 = off, 1 = First-Block Cache                                */
  float step_cache_threshold;        /* <= 0: 0.02                                                    */
} moss_step_args;
/* Defaults: cfg 3, slg_start 0.01, slg_stop 1.0, uncond_skip_layers = {22}, num_steps 50, step 0,
 * slg_scale 0 (two-pass), cfg_truncation 1 (off), step_cache 0 (off), step_cache_threshold 0. */
void moss_step_args_init(moss_step_args* a, uint32_t size);
int moss_sample_step(moss_dit* h, const moss_step_args* a, void* stream);
/* Step-cache counters of the current sampling run (reset at step 0): calls that ran every block,
 * calls that reused blocks 1.., and the last measured change (NaN before the first comparison).
 * Host only; any output pointer may be NULL. */
int moss_step_cache_stats(const moss_dit* h, int32_t* full_calls, int32_t* reused_calls, float* last_change);
/* Host-only check of step arguments (no GPU needed). msg (may be NULL) receives the reason. */
int moss_validate_step_args(const moss_dit_config* cfg, const moss_step_args* a, char* msg, int32_t msg_len);

/* ---------------------------------------------------------------------------------------------
 * The fused FP32 guidance + Euler kernel on its own: x[i] += (sigma_next - sigma) * v[i] with
 * v = v_uncond + cfg*(v_cond - v_uncond), or v = v_cond when v_uncond == NULL (requires cfg == 1).
 * Guidance and scheduler arithmetic are FP32 ("MOSS-Image" SGLang cookbook, "3. Guidance and
 * precision"); the combine is the ordinary linear one (Qwen-Image 2.1 cookbook, "5. Runtime features",
 * for a sibling single-stream DiT); CFG 1 turns guidance off (InvokeAI guide "MOSS-Image", "Generation
 * settings"). The Euler update of a flow-matching velocity moves x along v by the sigma step.
 * All pointers device fp32 [n], 16-byte aligned, owned by the caller; x is updated in place.
 * Errors (host-side, nothing enqueued): MOSS_ERR_INVALID_ARGUMENT for NULL v_cond / x, n < 0, cfg < 1
 * or not finite, v_uncond == NULL with cfg != 1, misaligned pointers; MOSS_ERR_DEVICE when the launch
 * fails. */
int moss_cfg_euler(const float* v_cond, const float* v_uncond, float* x, int64_t n, float cfg,
                   float sigma, float sigma_next, void* stream);

/* The same with the three-pass skip-layer guidance term: v as above (v_uncond == NULL: no negative
 * branch, any cfg >= 1 is then unused), plus slg * (v_cond - v_skip) when v_skip != NULL (slg finite).
 * This is the combine moss_sample_step runs. All pointers device fp32 [n], 16-byte aligned. */
int moss_guidance_euler(const float* v_cond, const float* v_uncond, const float* v_skip, float* x, int64_t n,
                        float cfg, float slg, float sigma, float sigma_next, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOSS_DIT_H */
