// FP8 tier: OCP microscaling (MX) FP8 operands for the block projections (gfx950).
//
// The pages run lossy FP8 tiers with channel-wise or tensor-wise scales on NVIDIA parts (Qwen-Image 2.1
// cookbook, "Online FP8"; MossInfer integration guide, "Quality tier"). gfx950's FP8 matrix instruction
// (v_mfma_scale_f32_32x32x64_f8f6f4) applies one power-of-two (E8M0) scale per 32 elements of the
// reduction axis in hardware, so this tier uses that block format, OCP MX FP8 (E4M3 elements, blocks
// of 32, scale exponent floor(log2(amax)) - 8).
//
// Layouts: codes [rows, K] bytes, row-major. Scales: E8M0 bytes (exponent + 127) packed four to a
// 32-bit word in the order the FP8 GEMM consumes them: word (2g + h) * ld + r holds in byte q the scale
// of block 8g + 2q + h of row r (g < K / 256, h < 2, q < 4; ld >= rows), i.e. the scales of block h of
// the four 64-element k-tiles 4g .. 4g + 3.
#include "common.h"
#include "kernels.h"

namespace moss {
namespace {

// One 32-element block per lane: workgroup = 64 rows x 4 blocks, lane (i, j) = row r0 + i, block
// kb0 + j. Reads 64 bytes of bf16 per lane (4 x 16 B), writes 32 code bytes (2 x 16 B) and one scale
// byte (the 64 lanes of a wave write 64 consecutive scale bytes of one block row).
__global__ __launch_bounds__(256) void mx_quant_kernel(const uint16_t* __restrict__ x, long ldx, int rows, int K,
                                                       uint8_t* __restrict__ q, uint8_t* __restrict__ s, long lds) {
  const int i = threadIdx.x & 63, j = threadIdx.x >> 6;
  const int r = blockIdx.x * 64 + i;
  const int kb = blockIdx.y * 4 + j;
  if (r >= rows || kb * 32 >= K) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + (long)r * ldx + kb * 32);
  uint4 w[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) w[c] = src[c];
  float v[32];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t u[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      v[8 * c + 2 * h] = __uint_as_float(u[h] << 16);
      v[8 * c + 2 * h + 1] = __uint_as_float(u[h] & 0xffff0000u);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(v[e]));
  const int ex = mx_exponent(amax);
  const float inv = mx_inv_scale(ex);
  uint32_t packed[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) packed[e] = mx_pack4(v[4 * e], v[4 * e + 1], v[4 * e + 2], v[4 * e + 3], inv);
  uint4* dst = reinterpret_cast<uint4*>(q + (long)r * K + kb * 32);
  dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  s[mx_scale_byte(kb, r, lds)] = (uint8_t)(ex + 127);
}

}  // namespace

hipError_t launch_mx_quant(const uint16_t* x, long ldx, int rows, int K, uint8_t* q, uint8_t* s, long lds,
                           hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (K % 256 != 0 || ldx % 8 != 0 || lds < rows || (reinterpret_cast<uintptr_t>(x) & 15) ||
      (reinterpret_cast<uintptr_t>(q) & 15))
    return hipErrorInvalidValue;
  dim3 grid((rows + 63) / 64, (K / 32 + 3) / 4);
  hipLaunchKernelGGL(mx_quant_kernel, grid, dim3(256), 0, stream, x, ldx, rows, K, q, s, lds);
  return hipGetLastError();
}

}  // namespace moss
