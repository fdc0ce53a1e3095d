// Host-side launchers of the MOSS-Image DiT kernels (internal to the library; not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host_plan.h"

namespace moss {

// ---------------------------------------------------------------------------------------------
// bf16 MFMA GEMM: out[m, n] = epilogue(sum_k A[m, k] * W[n, k]); A [M, K] and W [N, K] row-major.
// ---------------------------------------------------------------------------------------------
enum Epilogue {
  EPI_BF16 = 0,         // out bf16 [m, n] (rows remapped by seg/seg_stride/seg_off)
  EPI_QKV_ROPE = 1,     // out bf16; columns < rope_cols of image rows get the axial rotary turn
  EPI_GATED_RES = 2,    // out bf16 residual in place: x = bf16(x + gate[b, n] * acc)
  EPI_SWIGLU = 3,       // W holds [gate | up] interleaved in 32-row groups; out h = bf16(SiLU(g) * u)
  EPI_F32 = 4,          // out fp32 [m, n]
  EPI_F32_UNPATCH = 5,  // out fp32 velocity [B, C, lat_h, lat_w]: m = image token, n = c*4 + dy*2 + dx
  EPI_SWIGLU_MX = 6,    // as EPI_SWIGLU, h written as MXFP8: codes to out (bytes, ldo), scale words to out_scale
};

struct GemmArgs {
  const uint16_t* A;
  const uint16_t* W;
  int M, N, K;
  long lda, ldw;
  void* out;
  long ldo;
  // EPI_BF16 row remap: out_row = (m / seg) * seg_stride + seg_off + m % seg
  int seg, seg_stride, seg_off;
  // EPI_GATED_RES: gate[(m / rows_per_sample) * gate_stride + n]
  const uint16_t* gate;
  int rows_per_sample;
  long gate_stride;
  // EPI_QKV_ROPE: sequence S = T text rows + image rows on a grid of width grid_w
  const float* rope_cos;
  const float* rope_sin;
  int S, T, grid_w, rope_cols;
  // EPI_F32_UNPATCH
  int C, lat_h, lat_w, n_img;
  // MXFP8 operands (launch_gemm_mxfp8): A and W hold E4M3 codes (bytes; lda / ldw in bytes); their E8M0
  // scales are 32-bit words, word (2g + h) * ld + r holding in byte q the scale of 32-element block
  // 8g + 2q + h of row r (ld = lds_a, lds_w in words; lds_a >= M rounded up to 256, lds_w >= N)
  const uint8_t* A_scale;
  const uint8_t* W_scale;
  long lds_a, lds_w;
  // EPI_SWIGLU_MX: scale words of h (ld = lds_out >= M)
  uint8_t* out_scale;
  long lds_out;
};

// Picks a tile shape for (M, N) and launches. Returns hipSuccess or the launch error.
hipError_t launch_gemm(const GemmArgs& a, int epi, hipStream_t stream);
// Compute units of the current device (cached per device).
int device_cu_count();
// The same product with MXFP8 operands (needs N % 256 == 0 and K % 256 == 0); same epilogues.
hipError_t launch_gemm_mxfp8(const GemmArgs& a, int epi, hipStream_t stream);
// Interleave W_gate_up [2F, D] = [gate rows | up rows] into 32-row groups [g0 | u0 | g1 | u1 | ...].
hipError_t launch_interleave_gate_up(const uint16_t* src, uint16_t* dst, int F, int D, hipStream_t stream);

// ---------------------------------------------------------------------------------------------
// LayerNorm + modulation: out[r] = bf16(LN(x[in_row(r)]) * (1 + scale[b]) + shift[b])
// ---------------------------------------------------------------------------------------------
struct LnModArgs {
  const uint16_t* x;
  uint16_t* out;
  int rows, D;
  int seg, seg_stride, seg_off;   // in_row = (r / seg) * seg_stride + seg_off + r % seg
  int rows_per_sample;            // b = r / rows_per_sample
  const uint16_t* shift;          // shift[b * mod_stride + i]
  const uint16_t* scale;
  long mod_stride;
  float eps;
  // optional MXFP8 copy of the output (the FP8 tier's GEMM operand): codes q8 [rows, D] and scale words
  // (GemmArgs::A_scale layout, ld = lds8) of the bf16-rounded output; out may then be nullptr
  uint8_t* q8;
  uint8_t* s8;
  long lds8;
};
hipError_t launch_ln_mod(const LnModArgs& a, hipStream_t stream);

// ---------------------------------------------------------------------------------------------
// Exact attention over qkv [B*S, 3*H*128] (q | k | v, head h at columns h*128), out o [B*S, H*128].
// ---------------------------------------------------------------------------------------------
struct AttnArgs {
  const uint16_t* qkv;
  uint16_t* out;
  int B, S, H;
  long ld_qkv, ld_out;
  float scale_log2;   // log2(e) / sqrt(d)
  // Optional MXFP8 output (the FP8 tier's out-projection input): when q8 is set, row r = b S + token is
  // written as the E4M3 codes of its bf16-rounded values, q8[r * H * 128 + col], with one E8M0 scale
  // byte per 32 columns in the scale words s8 (ld = lds8 >= B S) -- what the separate quantizer would
  // write; out is then not written. Needs H * 128 % 256 == 0.
  uint8_t* q8 = nullptr;
  uint8_t* s8 = nullptr;
  long lds8 = 0;
};
// ws (optional, attention_split_workspace bytes): when the query tiles leave the last round of
// workgroups on the chip partly empty, those leftover tiles are split along the keys into parts that
// run side by side, and a merge kernel combines the parts (no ws: no split).
hipError_t launch_attention(const AttnArgs& a, hipStream_t stream, void* ws = nullptr, size_t ws_bytes = 0);
size_t attention_split_workspace(int B, int S, int H);

// 8-bit attention (the FP8 tier's attention): qkv as above (q and k already rotated). The workspace
// (attention_q8_workspace bytes, 256-byte aligned) receives the INT8 Q and K, the FP8 V^T and their
// scales. Two quantization passes, then the attention.
struct AttnQ8Args {
  const uint16_t* qkv;
  uint16_t* out;
  int B, S, H;
  long ld_qkv, ld_out;
  float scale_log2;
  int nblk;                 // 64-key blocks per sequence
  int8_t* q8;               // [B*S][H*128] INT8
  int8_t* k8;               // [B*S][H*128] INT8
  uint8_t* vt8;             // [B][H][128][nblk*64] E4M3, keys permuted within each block
  float* qa;                // [B*S][H] per-token amax of q
  float* ka;                // [B][H][nblk] per-block amax of k
  float* va;                // [B][H][128] per-channel amax of v
  float* vpart;             // [B][H][nblk][128] per-block channel maxima of v
  uint8_t* out8;            // optional MXFP8 output (AttnArgs::q8 / s8 / lds8)
  uint8_t* out8_scale;
  long lds8;
};
size_t attention_q8_workspace(int B, int S, int H);
hipError_t launch_attention_q8(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t stream);

// In-place axial rotary turn of the q and k columns of the image rows of qkv (standalone attention).
hipError_t launch_rope_inplace(uint16_t* qkv, int B, int S, int T, int grid_w, int H, long ld,
                               const float* cos_t, const float* sin_t, hipStream_t stream);

// ---------------------------------------------------------------------------------------------
// Timestep embedding + modulation
// ---------------------------------------------------------------------------------------------
// u[b, :] = bf16(SiLU(bf16(W_t2 bf16(SiLU(W_t1 e(sigma_b)))))) stored as fp32, e(sigma) sinusoidal.
struct SigmaBatch {
  float s[kMaxBatch];
};
hipError_t launch_time_mlp(SigmaBatch sigma, int B, const uint16_t* t_w1, const uint16_t* t_w2,
                           int temb, float flow_multiplier, float* u_out, hipStream_t stream);
// m[b, r] = bf16(sum_j W[r, j] * u[b, j]) for r < rows (all modulation rows of every block + final).
hipError_t launch_mod_gemv(const uint16_t* W, int rows, int temb, const float* u, int B,
                           uint16_t* m_out, long m_stride, hipStream_t stream);

// ---------------------------------------------------------------------------------------------
// Embedding inputs, guidance
// ---------------------------------------------------------------------------------------------
struct PtrBatch {
  const float* p[kMaxBatch];
};
// tokens[b*N + n, ch*4 + dy*2 + dx] = bf16(latent_b[ch, 2r+dy, 2c+dx]), n = r*(w/2) + c
hipError_t launch_patchify(PtrBatch latents, int B, int C, int h, int w, uint16_t* tokens, hipStream_t stream);
// x[b*S + t, :] = bf16(text_b[t, :]) for t < T
hipError_t launch_text_cast(PtrBatch text, int B, int T, int D, int S, uint16_t* x, hipStream_t stream);
// x = x + (sigma_next - sigma) * (v_u + cfg * (v_c - v_u)); v_u == nullptr means v = v_c.
hipError_t launch_cfg_euler(const float* v_c, const float* v_u, float* x, long n, float cfg, float sigma,
                            float sigma_next, hipStream_t stream);
// As above plus slg * (v_c - v_s) when v_s != nullptr (the skipped conditional prediction).
hipError_t launch_guidance_euler(const float* v_c, const float* v_u, const float* v_s, float* x, long n, float cfg,
                                 float slg, float sigma, float sigma_next, hipStream_t stream);
// MXFP8 quantization (OCP MX: E4M3 codes, one E8M0 scale per 32 elements along K; K % 256 == 0):
// x bf16 [rows, K] (row stride ldx) -> q [rows, K] bytes and the scale words of GemmArgs::A_scale with
// ld = lds >= rows.
hipError_t launch_mx_quant(const uint16_t* x, long ldx, int rows, int K, uint8_t* q, uint8_t* s, long lds,
                           hipStream_t stream);
// Step cache (First-Block Cache): r_cur = x1 - x0 (fp32); with r_prev also sums[0] = sum|r_cur - r_prev|
// and sums[1] = sum|r_prev| (fixed-order reduction through `partial`, 2 * 1024 floats).
hipError_t launch_fbc_change(const uint16_t* x1, const uint16_t* x0, const float* r_prev, float* r_cur, long n,
                             float* partial, float* sums, hipStream_t stream);
// rest = xl - x1 (fp32)
hipError_t launch_fbc_rest(const uint16_t* xl, const uint16_t* x1, float* rest, long n, hipStream_t stream);
// x = bf16(x + rest)
hipError_t launch_fbc_apply(uint16_t* x, const float* rest, long n, hipStream_t stream);
constexpr int kFbcPartials = 1024;
// dst = float(src) for n bf16 values (src 8-byte, dst 16-byte aligned).
hipError_t launch_bf16_to_f32(const uint16_t* src, float* dst, long n, hipStream_t stream);

}  // namespace moss
