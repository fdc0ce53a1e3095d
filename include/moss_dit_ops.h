/* moss_dit_ops.h -- kernel-level entry points of the MOSS-Image DiT library.
 *
 * These expose the pieces of one forward pass on their own, for parity checks of each step against
 * an independent implementation and for per-kernel measurement. They follow the conventions of
 * moss_dit.h (status codes, borrowed device pointers, enqueue on `stream`, host-side validation).
 */
#ifndef MOSS_DIT_OPS_H
#define MOSS_DIT_OPS_H

#include <stdint.h>
#include "moss_dit.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Per-block modulation ("MOSS-Image" InvokeAI guide, "Transformer formats", names the time-embedding
 * and modulation layers): u = SiLU(W_t2 SiLU(W_t1 e(sigma))), then for every block
 * (shift1, scale1, gate1, shift2, scale2, gate2) = W_mod,l u and for the final layer
 * (shift_f, scale_f) = W_fmod u.
 * sigma: host fp32 [B]. mod: device bf16 [B, num_layers*6*hidden + 2*hidden] (block l's six chunks
 * at l*6*hidden, the final pair at num_layers*6*hidden). */
int moss_dit_modulation(moss_dit* h, const float* sigma, int32_t batch, void* mod, void* stream);

/* Optional outputs of moss_dit_block (device pointers, NULL = not written), rows = B*S:
 *   a      bf16 [rows, D]   LN1-modulated input of the qkv projection
 *   qkv    bf16 [rows, 3D]  q | k | v, q and k rotated on image rows
 *   o      bf16 [rows, D]   attention output
 *   attn   fp32 [rows, D]   o W_o^T (branch output before the gated add)
 *   x1     bf16 [rows, D]   residual after the attention branch
 *   a2     bf16 [rows, D]   LN2-modulated input of the FFN
 *   h      bf16 [rows, F]   SiLU(a2 W_g^T) * (a2 W_u^T)
 *   ffn    fp32 [rows, D]   h W_down^T (branch output before the gated add)
 * In the FP8 tier (gemm_precision 1) the kernels that produce a projection's input write its MXFP8
 * codes themselves and skip the bf16 copy; when taps is given, every such input is written in bf16
 * and quantized by the separate MXFP8 quantizer instead -- the same bits, so taps do not change the
 * block's result. */
typedef struct {
  uint32_t struct_size;
  void *a, *qkv, *o, *attn, *x1, *a2, *h, *ffn;
} moss_block_taps;
void moss_block_taps_init(moss_block_taps* t, uint32_t size);

/* One joint block `layer` of the handle's weights on a residual stream x (device bf16 [B, S, D],
 * updated in place), S = text_len + grid_h*grid_w, the first text_len rows of each sample being
 * text. mod: device bf16 [B, mod_stride] laid out as moss_dit_modulation writes it. */
int moss_dit_block(moss_dit* h, int32_t layer, void* x, int32_t batch, int32_t text_len, int32_t grid_h,
                   int32_t grid_w, const void* mod, int64_t mod_stride, const moss_block_taps* taps,
                   void* stream);

/* Exact attention at head_dim 128 on packed qkv (device bf16 [B, S, 3*H*128], q | k | v), out device
 * bf16 [B, S, H*128]. rope != 0: q and k of the image rows (sequence index >= text_len, grid of width
 * grid_w) are first turned by the axial rotary embedding (theta 1e4) -- in place, qkv is modified.
 * When the query tiles leave the last round of workgroups on the chip partly empty, the leftover tiles
 * are split along the keys and merged; their partial results go to a temporary device allocation,
 * and the call then synchronizes `stream` before returning (a test and measurement entry; the model
 * path keeps that scratch in its handle's workspace). */
int moss_attention(void* qkv, void* out, int32_t batch, int32_t seq, int32_t heads, int32_t text_len,
                   int32_t grid_w, int32_t rope, void* stream);

/* moss_attention for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same arguments, kernels and results (bit for
 * bit), but no allocation and no synchronisation. The split tail's partial results go to a static
 * device array of MOSS_ATTENTION_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends, and the
 * RoPE table to a second static array; the first call on each device sets them up (their device
 * addresses, and a synchronous host-to-device copy of the table), so make that first call outside
 * graph capture. Every call on one GPU shares that GPU's scratch: calls that overlap on one GPU
 * (different streams, or different threads) race; serialise them. Returns MOSS_ERR_INVALID_ARGUMENT
 * for the arguments moss_attention refuses and when a shape's split needs more scratch than the array
 * holds (only possible on a chip with more than 256 compute units), MOSS_ERR_DEVICE when the set-up or
 * a launch fails. */
#define MOSS_ATTENTION_NOALLOC_SCRATCH_BYTES (33L << 20)
int moss_attention_noalloc(void* qkv, void* out, int32_t batch, int32_t seq, int32_t heads, int32_t text_len,
                           int32_t grid_w, int32_t rope, void* stream);

/* 8-bit attention (the FP8 tier's attention: the pages' q8_fp8 mode -- 8-bit Q and K, FP8 P V; MossInfer
 * integration guide, "Quality tier" and its attention modes). Reading (the pages give no formula): Q
 * symmetric INT8 per token and head (scale amax/127), K symmetric INT8 per block of 64 consecutive keys
 * and head, V FP8 E4M3 per channel (scale amax/448); exact integer Q K^T, fp32 online softmax over
 * the 64-key blocks whose reference max per query moves to a block's max only when that exceeds it by
 * more than a factor 2 in probability, each probability (<= 2) rounded to E4M3 on the scale 224, the
 * normaliser summing the same rounded probabilities; fp32 accumulation.
 *   qkv: device bf16 [B, S, 3*H*128] (q | k | v, q and k already rotated where wanted), 16-byte
 *   aligned; out: device bf16 [B, S, H*128]. ws: device scratch of moss_attention_q8_workspace(B, S, H)
 *   bytes, 256-byte aligned, owned by the caller; it receives the codes and scales (contents undefined
 *   afterwards). One sample's qkv and the V^T copy must stay below 2 GiB. */
int64_t moss_attention_q8_workspace(int32_t batch, int32_t seq, int32_t heads);
int moss_attention_q8(const void* qkv, void* out, int32_t batch, int32_t seq, int32_t heads, void* ws,
                      int64_t ws_bytes, void* stream);

/* bf16 GEMM out = A W^T with an fp32 output (device A bf16 [M, K], W bf16 [N, K], out fp32 [M, N]);
 * M, N, K >= 1, K % 64 == 0, N % 128 == 0; other values return MOSS_ERR_INVALID_ARGUMENT before any device work. */
int moss_gemm_bf16(const void* A, const void* W, float* out, int32_t M, int32_t N, int32_t K, void* stream);

/* Per-kernel-class timing with HIP events recorded on the call's stream around every launch of the
 * handle's compute calls. Off by default; while on, each launch is bracketed by two events (a few
 * microseconds of host overhead per launch, no change to any result). Classes, in order:
 *   0 modulation (time MLP + modulation GEMV)   1 embed (text cast, patchify, patch GEMM)
 *   2 LayerNorm-modulation (LN1 and LN2)          3 qkv GEMM + RoPE
 *   4 attention                                  5 out GEMM + gated residual
 *   6 gate/up GEMM + SiLU*mul                    7 down GEMM + gated residual
 *   8 final layer (LN-mod + output GEMM)         9 CFG + Euler */
#define MOSS_PROF_CLASSES 10
/* FP8 tier ("MOSS-Image" SGLang cookbook, "3. Guidance and precision", and the MossInfer integration
 * guide, "Quality tier": lossy FP8 GEMM tiers; the Qwen-Image 2.1 cookbook, "Online FP8", quantizes
 * weights and activations on the fly). Format: OCP microscaling MXFP8 -- E4M3 codes and one E8M0
 * (power-of-two) scale per 32 consecutive elements of the reduction axis, scale exponent
 * floor(log2(block amax)) - 8, elements rounded to nearest even and saturated at +-448, an all-zero
 * block taking exponent -127. The pages' FP8 tiers use channel- or tensor-wise scales on their
 * hardware; the block format is what gfx950's scaled FP8 MFMA applies natively.
 *
 * Scale storage ("scale words"): uint32 words, word (2g + h) * ld + r holding in byte q (low byte
 * first) the biased exponent (exponent + 127) of block 8g + 2q + h of row r, for g < K / 256, h < 2,
 * q < 4: K / 128 * ld words in all.
 *
 * Quantize x (device bf16 [rows, K], 16-byte aligned) to codes (device uint8 [rows, K], E4M3 bytes,
 * 16-byte aligned) and scale words (device, ld_scale >= rows). K % 256 == 0, rows >= 1. */
int moss_mx_quantize(const void* x, int32_t rows, int32_t K, void* codes, void* scales, int64_t ld_scale,
                     void* stream);

/* MXFP8 GEMM with an fp32 output: out[m, n] = sum_k a(m, k) w(n, k), a and w the MXFP8 values of A
 * (codes [M, K], scale words with ld = lds_a) and W (codes [N, K], scale words with ld = lds_w), fp32
 * accumulation. M, N, K >= 1, N % 256 == 0, K % 256 == 0, lds_a >= M rounded up to 256 (the scale
 * words of rows M .. that bound are read, their products discarded), lds_w >= N, both multiples of
 * 256; other values return MOSS_ERR_INVALID_ARGUMENT before any device work. */
int moss_gemm_mxfp8(const void* A, const void* A_scales, int64_t lds_a, const void* W, const void* W_scales,
                    int64_t lds_w, float* out, int32_t M, int32_t N, int32_t K, void* stream);

int moss_dit_profile_enable(moss_dit* h, int32_t enable);
/* Synchronises the device, writes the summed milliseconds and the launch count of each class since
 * the last read (host arrays of MOSS_PROF_CLASSES), and resets the counters. */
int moss_dit_profile_read(moss_dit* h, double* ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* MOSS_DIT_OPS_H */
