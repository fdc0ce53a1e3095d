// Host-only planning of the MOSS-Image DiT library: argument validation, the row plan of one sampling
// step, the attention work split and the workspace layout. Plain C++ with no HIP dependency, so it is
// also built on its own (with the address and undefined-behaviour sanitizers) by the CPU tests.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "moss_dit.h"

namespace moss {

constexpr int kMaxBatch = 8;        // samples per forward call
constexpr int kRopeMaxPos = 256;    // grid side limit: 4096 px / 16 px per token
constexpr int kHeadDim = 128;
constexpr int kMaxLatentSide = 512; // 4096 px / 8
constexpr double kMaxPixels = 4.2e6;
constexpr int kMaxTextLen = 4096;
constexpr int kSinusoidDim = 256;
constexpr int kAttnBQ = 128;        // queries per attention workgroup
constexpr int kAttnBKV = 64;        // keys per attention tile

std::string fmt(const char* f, ...);
size_t align_up(size_t x);          // next multiple of 256
// message of the calling thread's last failed call that had no handle (moss_dit_last_error(NULL))
std::string& thread_error();
// copies m into msg[0 .. len) (truncated, NUL-terminated); msg may be NULL
void copy_msg(const std::string& m, char* msg, int32_t len);

// ---- the axial RoPE table: cos and sin of pos * theta^(-k/32) for pos < kRopeMaxPos, k < 32, computed
// in double and rounded to fp32; out[0 .. T) = cos, out[T .. 2T) = sin with T = kRopeMaxPos * 32 ----
constexpr int kRopeTableFloats = 2 * kRopeMaxPos * (kHeadDim / 4);
void rope_table_host(float theta, float* out);

// ---- validation: status code (moss_status) and a user-facing message ----
int check_config(const moss_dit_config* c, std::string& msg);
int check_latent(int32_t lh, int32_t lw, std::string& msg);
int check_text_len(int32_t t, std::string& msg);
int validate_forward(const moss_dit_config* c, const moss_forward_args* a, std::string& msg);
int validate_step(const moss_dit_config* c, const moss_step_args* a, std::string& msg);

// arguments of the standalone exact attention (moss_attention and its no-allocation variant)
int check_attention_args(const void* qkv, const void* out, int32_t batch, int32_t seq, int32_t heads,
                         int32_t text_len, int32_t grid_w, int32_t rope, std::string& msg);

// ---- the rows of one sampling step's batch: [cond | negative (uncond) | cond skipping layers] ----
struct StepPlan {
  int rows;              // 1 .. 3
  bool neg, third;       // negative pass; third (skipped conditional) pass
  uint64_t skip[3];      // per-row skip mask
};
// a must have passed validate_step.
StepPlan step_plan(const moss_step_args* a);

// ---- exact attention's work split: workgroups [0, n_full) take whole query tiles; each of the
// n_split leftover tiles is split along its key tiles into `parts` workgroups (partial results are
// merged afterwards). slots = workgroups resident on the chip at once (two per compute unit). ----
struct AttnSplitPlan {
  int n_full, n_split, parts;
};
AttnSplitPlan attention_split_plan(int B, int S, int H, long slots);
// bytes of the partial results of that split (0 = nothing is split)
size_t attention_split_bytes(int B, int S, int H, long slots);
// bytes of the 8-bit attention's workspace (quantized q, k, v^T and their scales)
size_t attention_q8_bytes(int B, int S, int H);

// ---- workspace layout of one call: byte offsets of each region from the workspace base ----
struct WsLayout {
  size_t x, a, qkv, o, h, tokens, mod, u, vel;   // bf16 activations; fp32 u, vel
  size_t q8, s8, q8h, s8h;                        // FP8 tier (SIZE_MAX when absent)
  size_t attn_split, attn8;                       // exact attention split / 8-bit attention (SIZE_MAX when absent)
  size_t attn_split_bytes, attn8_bytes;
  long lds8;                                      // scale-word row stride of the FP8 tier
  size_t total;                                   // bytes of the whole workspace
};
constexpr size_t kNoRegion = (size_t)-1;
// B rows of S tokens (N image tokens each), lat_elems latent elements per row.
WsLayout ws_layout(const moss_dit_config& k, int B, int S, int N, long lat_elems, long attn_slots);

}  // namespace moss
