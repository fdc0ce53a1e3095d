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

// Wave-wide (64 lanes) sum.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace moss
