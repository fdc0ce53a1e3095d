// Affine-free LayerNorm fused with the adaLN modulation: out = bf16(LN(x) * (1 + scale) + shift).
//
// The fusion of LayerNorm with the "* (1 + scale)" modulation is the one the Qwen-Image 2.1 cookbook
// describes for its single-stream DiT ("Lossless LayerNorm modulation"); MOSS-Image's joint blocks
// take (shift, scale) from the per-block modulation layer. One wave normalises one row: the row is
// read once from HBM into registers (8-byte loads, 512 contiguous bytes per wave instruction), mean
// and then the centred variance are reduced across the wave in fp32, and the modulated row is
// written once. The kernel is HBM-bound: 2 * D bytes read + 2 * D bytes written per row.
#include "common.h"
#include "kernels.h"

namespace moss {
namespace {

constexpr int kMaxChunks = 16;   // D <= 16 * 256

__global__ __launch_bounds__(256) void ln_mod_kernel(LnModArgs p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave;
  if (r >= p.rows) return;
  const int nch = p.D >> 8;
  const long in_row = (long)(r / p.seg) * p.seg_stride + p.seg_off + r % p.seg;
  const uint16_t* xr = p.x + in_row * p.D;

  float v[kMaxChunks][4];
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    if (c < nch) {
      const uint2 u = *reinterpret_cast<const uint2*>(xr + (c * 64 + lane) * 4);
      v[c][0] = __uint_as_float(u.x << 16);
      v[c][1] = __uint_as_float(u.x & 0xffff0000u);
      v[c][2] = __uint_as_float(u.y << 16);
      v[c][3] = __uint_as_float(u.y & 0xffff0000u);
      s += (v[c][0] + v[c][1]) + (v[c][2] + v[c][3]);
    }
  }
  const float inv_d = 1.0f / (float)p.D;
  const float mean = wave_sum(s) * inv_d;
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    if (c < nch) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float d = v[c][e] - mean;
        q += d * d;
      }
    }
  }
  const float var = wave_sum(q) * inv_d;
  const float rstd = 1.0f / sqrtf(var + p.eps);

  const long b = r / p.rows_per_sample;
  const uint16_t* sh = p.shift + b * p.mod_stride;
  const uint16_t* sc = p.scale + b * p.mod_stride;
  uint16_t* o = p.out + (long)r * p.D;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    if (c < nch) {
      const int i0 = (c * 64 + lane) * 4;
      const uint2 su = *reinterpret_cast<const uint2*>(sh + i0);
      const uint2 cu = *reinterpret_cast<const uint2*>(sc + i0);
      const float shv[4] = {__uint_as_float(su.x << 16), __uint_as_float(su.x & 0xffff0000u),
                            __uint_as_float(su.y << 16), __uint_as_float(su.y & 0xffff0000u)};
      const float scv[4] = {__uint_as_float(cu.x << 16), __uint_as_float(cu.x & 0xffff0000u),
                            __uint_as_float(cu.y << 16), __uint_as_float(cu.y & 0xffff0000u)};
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = (v[c][e] - mean) * rstd * (1.0f + scv[e]) + shv[e];
      uint2 w;
      w.x = pack2_bf16(y[0], y[1]);
      w.y = pack2_bf16(y[2], y[3]);
      *reinterpret_cast<uint2*>(o + i0) = w;
    }
  }
}

}  // namespace

hipError_t launch_ln_mod(const LnModArgs& a, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  if (a.D % 256 != 0 || a.D > kMaxChunks * 256 || a.seg <= 0 || a.rows_per_sample <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ln_mod_kernel, dim3((a.rows + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moss
