// Small HBM- or latency-bound kernels of the denoising step: timestep embedding and modulation,
// patchify and text cast, and the fused FP32 guidance + Euler update.
#include "common.h"
#include "kernels.h"

namespace moss {
namespace {

// Time MLP for one sample per workgroup. Sinusoidal features of t = flow_multiplier * sigma
// (cos half, then sin half, frequencies exp(-ln(1e4) k / 128)), then u = SiLU(W_t2 SiLU(W_t1 e)).
// Each stored intermediate is rounded to bf16, as a bf16 model holds it between layers. The angle
// and the trigonometric functions are evaluated in fp64: t reaches 1000 and fp32 would lose the
// phase to ~1e-4.
__global__ void time_mlp_kernel(SigmaBatch sigma, const uint16_t* __restrict__ w1,
                                const uint16_t* __restrict__ w2, int E, float flow_multiplier,
                                float* __restrict__ u_out) {
  __shared__ float e[256];
  __shared__ float a1[1024];
  const int b = blockIdx.x, t = threadIdx.x;
  const double tt = (double)flow_multiplier * (double)sigma.s[b];
  if (t < 128) {
    const double f = exp(-log(1.0e4) * (double)t / 128.0);
    e[t] = round_bf16((float)cos(tt * f));
    e[t + 128] = round_bf16((float)sin(tt * f));
  }
  __syncthreads();
  if (t < E) {
    const uint16_t* row = w1 + (long)t * 256;
    float acc = 0.f;
    for (int j = 0; j < 256; ++j) acc += bf16_to_f32(row[j]) * e[j];
    a1[t] = round_bf16(silu_f32(acc));
  }
  __syncthreads();
  if (t < E) {
    const uint16_t* row = w2 + (long)t * E;
    float acc = 0.f;
    for (int j = 0; j < E; ++j) acc += bf16_to_f32(row[j]) * a1[j];
    const float temb = round_bf16(acc);
    u_out[(long)b * E + t] = round_bf16(silu_f32(temb));
  }
}

// m[b, r] = bf16(W[r, :] . u[b, :]) for temb = 256: 32 lanes per row (16 bytes each), two rows per
// wave instruction, grid-stride over row pairs. Reads every modulation weight once per call.
__global__ __launch_bounds__(256) void mod_gemv_kernel(const uint16_t* __restrict__ W, int rows,
                                                       const float* __restrict__ u, int B,
                                                       uint16_t* __restrict__ m, long m_stride) {
  __shared__ float us[kMaxBatch * 256];
  for (int i = threadIdx.x; i < B * 256; i += blockDim.x) us[i] = u[i];
  __syncthreads();
  const int lane = threadIdx.x & 63, half = lane >> 5, sl = lane & 31;
  const int wave_global = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * 4;
  for (int pr = wave_global; pr * 2 < rows; pr += nwaves) {
    const int row = pr * 2 + half;
    const bool ok = row < rows;
    uint4 wv = make_uint4(0, 0, 0, 0);
    if (ok) wv = *reinterpret_cast<const uint4*>(W + (long)row * 256 + sl * 8);
    const uint32_t wr[4] = {wv.x, wv.y, wv.z, wv.w};
    float wf[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wf[2 * j] = __uint_as_float(wr[j] << 16);
      wf[2 * j + 1] = __uint_as_float(wr[j] & 0xffff0000u);
    }
    for (int b = 0; b < B; ++b) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += wf[j] * us[b * 256 + sl * 8 + j];
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
      if (ok && sl == 0) m[(long)b * m_stride + row] = f32_to_bf16(acc);
    }
  }
}

__global__ void patchify_kernel(PtrBatch lat, int B, int C, int h, int w, uint16_t* __restrict__ tokens) {
  const int P = C * 4;
  const int gw = w / 2, N = (h / 2) * gw;
  const long total = (long)B * N * P;
  for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += (long)gridDim.x * blockDim.x) {
    const int j = (int)(idx % P);
    const long row = idx / P;
    const int b = (int)(row / N), n = (int)(row % N);
    const int r = n / gw, c = n % gw;
    const int ch = j >> 2, dy = (j >> 1) & 1, dx = j & 1;
    tokens[idx] = f32_to_bf16(lat.p[b][((long)ch * h + 2 * r + dy) * w + 2 * c + dx]);
  }
}

__global__ void text_cast_kernel(PtrBatch text, int B, int T, int D, int S, uint16_t* __restrict__ x) {
  const long per = (long)T * D / 4;
  const long total = (long)B * per;
  for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += (long)gridDim.x * blockDim.x) {
    const int b = (int)(idx / per);
    const long e = (idx % per) * 4;
    const long t = e / D, i = e % D;
    const float4 v = *reinterpret_cast<const float4*>(text.p[b] + e);
    uint2 o;
    o.x = pack2_bf16(v.x, v.y);
    o.y = pack2_bf16(v.z, v.w);
    *reinterpret_cast<uint2*>(x + ((long)b * S + t) * D + i) = o;
  }
}

// Fused FP32 classifier-free guidance and flow-matching Euler step ("MOSS-Image" SGLang cookbook,
// "Guidance and precision": CFG arithmetic and scheduler updates in FP32).
// Guided velocity and Euler update, all fp32: v = v_c, or v_u + cfg (v_c - v_u) when the negative
// branch ran (vu != nullptr); plus slg (v_c - v_s) when the skipped conditional prediction ran
// (vs != nullptr); then x += dt v. With vs == v_c the extra term is exactly zero.
__global__ void guidance_euler_kernel(const float* __restrict__ vc, const float* __restrict__ vu,
                                      const float* __restrict__ vs, float* __restrict__ x, long n, float cfg,
                                      float slg, float dt) {
  const long n4 = n / 4;
  const long stride = (long)gridDim.x * blockDim.x;
  const long t0 = (long)blockIdx.x * blockDim.x + threadIdx.x;
  for (long i = t0; i < n4; i += stride) {
    const float4 c = reinterpret_cast<const float4*>(vc)[i];
    float4 xv = reinterpret_cast<float4*>(x)[i];
    float4 v = c;
    if (vu != nullptr) {
      const float4 u = reinterpret_cast<const float4*>(vu)[i];
      v.x = u.x + cfg * (c.x - u.x);
      v.y = u.y + cfg * (c.y - u.y);
      v.z = u.z + cfg * (c.z - u.z);
      v.w = u.w + cfg * (c.w - u.w);
    }
    if (vs != nullptr) {
      const float4 k = reinterpret_cast<const float4*>(vs)[i];
      v.x = v.x + slg * (c.x - k.x);
      v.y = v.y + slg * (c.y - k.y);
      v.z = v.z + slg * (c.z - k.z);
      v.w = v.w + slg * (c.w - k.w);
    }
    xv.x = xv.x + dt * v.x;
    xv.y = xv.y + dt * v.y;
    xv.z = xv.z + dt * v.z;
    xv.w = xv.w + dt * v.w;
    reinterpret_cast<float4*>(x)[i] = xv;
  }
  for (long i = n4 * 4 + t0; i < n; i += stride) {
    float v = vc[i];
    if (vu != nullptr) v = vu[i] + cfg * (vc[i] - vu[i]);
    if (vs != nullptr) v = v + slg * (vc[i] - vs[i]);
    x[i] = x[i] + dt * v;
  }
}

// ---- step cache (First-Block Cache) ----
constexpr int kFbcBlocks = 1024;   // partial sums of the change measure: one pair per workgroup

// r_cur = float(x1) - float(x0) (block 0's residual); with r_prev, partial sums of |r_cur - r_prev|
// and |r_prev| per workgroup (written, not accumulated: a fixed-order reduction follows).
__global__ __launch_bounds__(256) void fbc_residual_kernel(const uint16_t* __restrict__ x1, const uint16_t* __restrict__ x0,
                                                           const float* __restrict__ r_prev, float* __restrict__ r_cur,
                                                           long n, float* __restrict__ partial) {
  float d = 0.f, a = 0.f;
  const long stride = (long)gridDim.x * blockDim.x;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float r = bf16_to_f32(x1[i]) - bf16_to_f32(x0[i]);
    r_cur[i] = r;
    if (r_prev != nullptr) {
      d += fabsf(r - r_prev[i]);
      a += fabsf(r_prev[i]);
    }
  }
  if (r_prev == nullptr) return;
  __shared__ float sd[4], sa[4];
  d = wave_sum(d);
  a = wave_sum(a);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    sd[wave] = d;
    sa[wave] = a;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    partial[2 * blockIdx.x] = (sd[0] + sd[1]) + (sd[2] + sd[3]);
    partial[2 * blockIdx.x + 1] = (sa[0] + sa[1]) + (sa[2] + sa[3]);
  }
}

// sums[0..1] = the workgroup partials added in a fixed order (one workgroup of 256 lanes)
__global__ __launch_bounds__(256) void fbc_sum_kernel(const float* __restrict__ partial, int nparts,
                                                      float* __restrict__ sums) {
  float d = 0.f, a = 0.f;
  for (int i = threadIdx.x; i < nparts; i += 256) {
    d += partial[2 * i];
    a += partial[2 * i + 1];
  }
  __shared__ float sd[4], sa[4];
  d = wave_sum(d);
  a = wave_sum(a);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    sd[wave] = d;
    sa[wave] = a;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    sums[0] = (sd[0] + sd[1]) + (sd[2] + sd[3]);
    sums[1] = (sa[0] + sa[1]) + (sa[2] + sa[3]);
  }
}

// rest = float(xL) - float(x1): what blocks 1.. added at a full call
__global__ void fbc_rest_kernel(const uint16_t* __restrict__ xl, const uint16_t* __restrict__ x1,
                                float* __restrict__ rest, long n) {
  const long stride = (long)gridDim.x * blockDim.x;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    rest[i] = bf16_to_f32(xl[i]) - bf16_to_f32(x1[i]);
}

// x = bf16(float(x) + rest): a reused call's stream after the last block
__global__ void fbc_apply_kernel(uint16_t* __restrict__ x, const float* __restrict__ rest, long n) {
  const long stride = (long)gridDim.x * blockDim.x;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    x[i] = f32_to_bf16(bf16_to_f32(x[i]) + rest[i]);
}

// fp32 copy of a bf16 tensor (exact), 4 elements per lane.
__global__ void bf16_to_f32_kernel(const uint16_t* __restrict__ src, float* __restrict__ dst, long n) {
  const long stride = (long)gridDim.x * blockDim.x;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n / 4; i += stride) {
    const uint2 u = reinterpret_cast<const uint2*>(src)[i];
    reinterpret_cast<float4*>(dst)[i] = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                                                    __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  }
  for (long i = (n / 4) * 4 + (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = bf16_to_f32(src[i]);
}

}  // namespace

hipError_t launch_time_mlp(SigmaBatch sigma, int B, const uint16_t* t_w1, const uint16_t* t_w2,
                           int temb, float flow_multiplier, float* u_out, hipStream_t stream) {
  if (temb > 1024 || temb < 1) return hipErrorInvalidValue;
  const int threads = temb < 128 ? 128 : ((temb + 63) / 64) * 64;
  hipLaunchKernelGGL(time_mlp_kernel, dim3(B), dim3(threads), 0, stream, sigma, t_w1, t_w2, temb,
                     flow_multiplier, u_out);
  return hipGetLastError();
}

hipError_t launch_mod_gemv(const uint16_t* W, int rows, int temb, const float* u, int B, uint16_t* m_out,
                           long m_stride, hipStream_t stream) {
  if (temb != 256 || B > kMaxBatch) return hipErrorInvalidValue;
  const int pairs = (rows + 1) / 2;
  int grid = (pairs + 3) / 4;
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(mod_gemv_kernel, dim3(grid), dim3(256), 0, stream, W, rows, u, B, m_out, m_stride);
  return hipGetLastError();
}

hipError_t launch_patchify(PtrBatch latents, int B, int C, int h, int w, uint16_t* tokens, hipStream_t stream) {
  const long total = (long)B * (h / 2) * (w / 2) * C * 4;
  int grid = (int)((total + 255) / 256);
  if (grid > 8192) grid = 8192;
  hipLaunchKernelGGL(patchify_kernel, dim3(grid), dim3(256), 0, stream, latents, B, C, h, w, tokens);
  return hipGetLastError();
}

hipError_t launch_text_cast(PtrBatch text, int B, int T, int D, int S, uint16_t* x, hipStream_t stream) {
  if (D % 4 != 0) return hipErrorInvalidValue;
  const long total = (long)B * T * D / 4;
  int grid = (int)((total + 255) / 256);
  if (grid > 8192) grid = 8192;
  hipLaunchKernelGGL(text_cast_kernel, dim3(grid), dim3(256), 0, stream, text, B, T, D, S, x);
  return hipGetLastError();
}

hipError_t launch_guidance_euler(const float* v_c, const float* v_u, const float* v_s, float* x, long n, float cfg,
                                 float slg, float sigma, float sigma_next, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if ((reinterpret_cast<uintptr_t>(v_c) | reinterpret_cast<uintptr_t>(v_u) | reinterpret_cast<uintptr_t>(v_s) |
       reinterpret_cast<uintptr_t>(x)) & 15)
    return hipErrorInvalidValue;
  long grid = (n / 4 + 255) / 256;
  if (grid < 1) grid = 1;
  if (grid > 2048) grid = 2048;
  hipLaunchKernelGGL(guidance_euler_kernel, dim3((unsigned)grid), dim3(256), 0, stream, v_c, v_u, v_s, x, n, cfg,
                     slg, sigma_next - sigma);
  return hipGetLastError();
}

hipError_t launch_cfg_euler(const float* v_c, const float* v_u, float* x, long n, float cfg, float sigma,
                            float sigma_next, hipStream_t stream) {
  return launch_guidance_euler(v_c, v_u, nullptr, x, n, cfg, 0.f, sigma, sigma_next, stream);
}

hipError_t launch_bf16_to_f32(const uint16_t* src, float* dst, long n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if ((reinterpret_cast<uintptr_t>(src) & 7) || (reinterpret_cast<uintptr_t>(dst) & 15)) return hipErrorInvalidValue;
  long grid = (n / 4 + 255) / 256;
  if (grid < 1) grid = 1;
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(bf16_to_f32_kernel, dim3((unsigned)grid), dim3(256), 0, stream, src, dst, n);
  return hipGetLastError();
}

hipError_t launch_fbc_change(const uint16_t* x1, const uint16_t* x0, const float* r_prev, float* r_cur, long n,
                             float* partial, float* sums, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fbc_residual_kernel, dim3(kFbcBlocks), dim3(256), 0, stream, x1, x0, r_prev, r_cur, n, partial);
  if (r_prev != nullptr) hipLaunchKernelGGL(fbc_sum_kernel, dim3(1), dim3(256), 0, stream, partial, kFbcBlocks, sums);
  return hipGetLastError();
}

hipError_t launch_fbc_rest(const uint16_t* xl, const uint16_t* x1, float* rest, long n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fbc_rest_kernel, dim3(2048), dim3(256), 0, stream, xl, x1, rest, n);
  return hipGetLastError();
}

hipError_t launch_fbc_apply(uint16_t* x, const float* rest, long n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fbc_apply_kernel, dim3(2048), dim3(256), 0, stream, x, rest, n);
  return hipGetLastError();
}

}  // namespace moss
