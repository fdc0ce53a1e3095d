// Shared device helpers of the MOSS-Image DiT kernels (gfx950 / CDNA4).
//
// Storage convention: bf16 tensors live in memory as uint16_t bit patterns; arithmetic is fp32.
// Every fp32 -> bf16 conversion rounds to nearest, ties to even (the bf16 DiT of the pages keeps
// weights and activations in bf16 while latents, guidance and the scheduler stay fp32:
// "MOSS-Image" SGLang cookbook, section "Guidance and precision").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moss {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 with gfx950's v_cvt_pk_bf16_f32 (round to nearest even under the default mode).
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  const floatx2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return (uint16_t)(pack2_bf16(f, 0.f) & 0xffffu); }

// Round an fp32 value to the nearest bf16 and return it as fp32.
__device__ __forceinline__ float round_bf16(float f) { return __uint_as_float(pack2_bf16(f, 0.f) << 16); }

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane i's bytes land at
// lds_window + 16 * i, where lds_window must be the same for the whole wave. Completion is tracked
// by vmcnt like any global load.
__device__ __forceinline__ void load_lds_16(const void* gptr, void* lds_window) {
  __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void*)lds_window, 16, 0, 0);
}

// Buffer resource over `bytes` bytes from `base` (raw: stride 0, 32-bit dwords). A buffer access whose
// per-lane offset reaches `bytes` returns zeros instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Buffer -> LDS copy of 16 bytes per lane (buffer_load_dwordx4 ... lds): lane i's bytes, read at byte
// offset `voffset` of the resource, land at lds_window + 16 * i (lds_window uniform over the wave).
__device__ __forceinline__ void buf_load_lds_16(__amdgpu_buffer_rsrc_t r, void* lds_window, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_window, 16, voffset, 0, 0, 0);
}

// Barrier that publishes direct-to-LDS copies: wait until this wave's vector-memory loads (the LDS
// copies included) have completed (s_waitcnt vmcnt(0); expcnt and lgkmcnt left at their maxima), then
// synchronise the workgroup. After it every wave's copies issued before the barrier are visible.
__device__ __forceinline__ void lds_copy_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
}

// ---- OCP MX FP8 (E4M3 elements, one E8M0 scale per 32 elements along the reduction axis) ----
// Scale exponent floor(log2(amax)) - 8 (8 = E4M3's largest exponent), read from the fp32 exponent
// field (exact for bf16 values), clamped to [-127, 127]; an all-zero block takes -127.
__device__ __forceinline__ int mx_exponent(float amax) {
  int ex = -127;
  if (amax > 0.f) {
    const int biased = (int)((__float_as_uint(amax) >> 23) & 0xff);
    ex = (biased == 0 ? -127 : biased - 127) - 8;
    ex = max(-127, min(127, ex));
  }
  return ex;
}
// 2^-ex, exact (ex <= 119 for finite bf16 amax)
__device__ __forceinline__ float mx_inv_scale(int ex) { return __uint_as_float((uint32_t)(127 - ex) << 23); }
// Four values -> four E4M3 codes, byte i = value i: x * inv clamped to the largest finite E4M3 value
// first (the hardware conversion rounds to nearest even but turns values past the range into NaN).
__device__ __forceinline__ uint32_t mx_pack4(float a, float b, float c, float d, float inv) {
  const float a0 = fminf(fmaxf(a * inv, -448.f), 448.f), a1 = fminf(fmaxf(b * inv, -448.f), 448.f);
  const float a2 = fminf(fmaxf(c * inv, -448.f), 448.f), a3 = fminf(fmaxf(d * inv, -448.f), 448.f);
  // The first conversion writes bytes 0-1 and keeps bytes 2-3 of its third operand, which the second
  // conversion then overwrites: a0's own bits serve as that operand, so the result is written in place
  // of a dead register instead of a zero materialised first.
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, __float_as_int(a0), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, w, true);
  return (uint32_t)w;
}
// Byte offset of the scale of 32-element block kb of row r in the scale-word layout (word
// (2g + h) * ld + r holds in byte q the scale of block 8g + 2q + h).
__device__ __forceinline__ long mx_scale_byte(int kb, long r, long ld) {
  return ((long)(2 * (kb >> 3) + (kb & 1)) * ld + r) * 4 + ((kb >> 1) & 3);
}

// Combination with lane l ^ 32 in one VALU instruction: gfx950's v_permlane32_swap, given the same
// register twice, returns x of lane (l & 31) and x of lane (l & 31) + 32 (checked on the hardware with
// an in-bounds probe). Unlike __shfl_xor (ds_bpermute) it does not go through LDS, so waiting for it
// does not also wait for the wave's outstanding LDS reads.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ int max_xor32(int x) {
  const auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return max((int)r[0], (int)r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max(a, b, c) for operands that are never NaN (scores, -inf for masked keys), as IEEE maximum
// (v_maximum3_f32 on gfx950). fmaxf must quiet signalling NaNs, so on values the compiler cannot
// prove canonical (MFMA results) it first runs a v_max x, x per operand; maximum propagates NaNs
// instead and needs no such step. (Not inline asm: the compiler then would not insert the wait
// states that a VALU read of an MFMA result needs.)
__device__ __forceinline__ float max3_f32(float a, float b, float c) {
  return __builtin_elementwise_maximum(a, __builtin_elementwise_maximum(b, c));
}

// One 32-element MX block held by the lane pair (l, l ^ 32) in the MFMA output layout: this lane's
// 16 values v[g][e] sit at block positions 8 g + 4 h + e (h = lane / 32), the partner's at the other
// 16. Rounds them to bf16, writes this lane's four code words at codes + 8 g + 4 h and, from the h == 0
// lane, the scale byte (biased exponent) at *scale -- the bytes the separate MXFP8 quantizer writes
// for the same bf16 values. Both lanes of the pair must execute it.
__device__ __forceinline__ void mx_store_pair_block(const float (&v)[4][4], int h, uint8_t* codes, uint8_t* scale) {
  float r[4][4];
  float amax = 0.f;
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[g][e] = round_bf16(v[g][e]);
      amax = fmaxf(amax, fabsf(r[g][e]));
    }
  amax = max_xor32(amax);
  const int ex = mx_exponent(amax);
  const float inv = mx_inv_scale(ex);
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *reinterpret_cast<uint32_t*>(codes + 8 * g + 4 * h) = mx_pack4(r[g][0], r[g][1], r[g][2], r[g][3], inv);
  if (h == 0) *scale = (uint8_t)(ex + 127);
}

// Wave-wide (64 lanes) sum.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace moss
