// Affine-free LayerNorm fused with the adaLN modulation: out = bf16(LN(x) * (1 + scale) + shift).
//
// The fusion of LayerNorm with the "* (1 + scale)" modulation is the one the Qwen-Image 2.1 cookbook
// describes for its single-stream DiT ("Lossless LayerNorm modulation"); MOSS-Image's joint blocks
// take (shift, scale) from the per-block modulation layer. One wave normalises one row: the row is
// read once from HBM into registers (16-byte loads, 1 KB contiguous per wave instruction, when the
// width allows), mean and then the centred variance are reduced across the wave in fp32, and the
// modulated row is written once. The kernel is HBM-bound: 2 * D bytes read + 2 * D bytes written per row.
#include <utility>

#include "common.h"
#include "kernels.h"

namespace moss {
namespace {

constexpr int kMaxElems = 64;   // elements per lane: D <= 64 * 64

// E elements per lane per chunk (E = 8: 16-byte loads, D % 512 == 0; E = 4: 8-byte loads), NCH chunks
// (D = 64 E NCH, a compile-time count so the row stays in exactly 3 NCH E / 2 registers). The
// modulation rows (shift, scale; served from L2) are requested together with the activation row, so
// their latency overlaps the row's HBM read instead of following the two reductions. The row is kept
// as packed bf16 and unpacked in each pass (two VALU per pair) to keep occupancy up.
template <int E, int NCH>
__global__ __launch_bounds__(256) void ln_mod_kernel(LnModArgs p) {
  typedef uint32_t words __attribute__((ext_vector_type(E / 2)));
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave;
  if (r >= p.rows) return;
  constexpr int D = 64 * E * NCH;
  const long in_row = (long)(r / p.seg) * p.seg_stride + p.seg_off + r % p.seg;
  const uint16_t* xr = p.x + in_row * D;
  const long b = r / p.rows_per_sample;
  const uint16_t* sh = p.shift + b * p.mod_stride;
  const uint16_t* sc = p.scale + b * p.mod_stride;

  words xw[NCH], sw[NCH], cw[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int i0 = (c * 64 + lane) * E;
    xw[c] = *reinterpret_cast<const words*>(xr + i0);
    sw[c] = *reinterpret_cast<const words*>(sh + i0);
    cw[c] = *reinterpret_cast<const words*>(sc + i0);
  }
  auto lo = [](uint32_t w) { return __uint_as_float(w << 16); };
  auto hi = [](uint32_t w) { return __uint_as_float(w & 0xffff0000u); };
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int h = 0; h < E / 2; ++h) s += lo(xw[c][h]) + hi(xw[c][h]);
  constexpr float inv_d = 1.0f / (float)D;
  const float mean = wave_sum(s) * inv_d;
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int h = 0; h < E / 2; ++h) {
      const float d0 = lo(xw[c][h]) - mean, d1 = hi(xw[c][h]) - mean;
      q += d0 * d0 + d1 * d1;
    }
  const float var = wave_sum(q) * inv_d;
  const float rstd = 1.0f / sqrtf(var + p.eps);

#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    words w;
#pragma unroll
    for (int h = 0; h < E / 2; ++h) {
      const float y0 = (lo(xw[c][h]) - mean) * rstd * (1.0f + lo(cw[c][h])) + lo(sw[c][h]);
      const float y1 = (hi(xw[c][h]) - mean) * rstd * (1.0f + hi(cw[c][h])) + hi(sw[c][h]);
      w[h] = pack2_bf16(y0, y1);
    }
    const int i0 = (c * 64 + lane) * E;
    if (p.out) *reinterpret_cast<words*>(p.out + (long)r * D + i0) = w;
    if (p.q8) {
      // MXFP8 of the bf16 output: a 32-element block spans 32 / E neighbouring lanes
      float amax = 0.f;
#pragma unroll
      for (int h = 0; h < E / 2; ++h) amax = fmaxf(amax, fmaxf(fabsf(lo(w[h])), fabsf(hi(w[h]))));
#pragma unroll
      for (int o = 1; o < 32 / E; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
      const int ex = mx_exponent(amax);
      const float inv = mx_inv_scale(ex);
      uint32_t codes[E / 4];
#pragma unroll
      for (int u = 0; u < E / 4; ++u)
        codes[u] = mx_pack4(lo(w[2 * u]), hi(w[2 * u]), lo(w[2 * u + 1]), hi(w[2 * u + 1]), inv);
      uint8_t* qd = p.q8 + (long)r * D + i0;
      if constexpr (E == 8) *reinterpret_cast<uint2*>(qd) = make_uint2(codes[0], codes[1]);
      else *reinterpret_cast<uint32_t*>(qd) = codes[0];
      if ((lane & (32 / E - 1)) == 0) p.s8[mx_scale_byte(i0 / 32, r, p.lds8)] = (uint8_t)(ex + 127);
    }
  }
}

template <int E, int NCH>
void launch_ln_n(const LnModArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((ln_mod_kernel<E, NCH>), dim3((a.rows + 3) / 4), dim3(256), 0, stream, a);
}

template <int E, int... N>
bool launch_ln_any(const LnModArgs& a, hipStream_t stream, std::integer_sequence<int, N...>) {
  const int nch = a.D / (64 * E);
  bool done = false;
  ((nch == N + 1 ? (launch_ln_n<E, N + 1>(a, stream), done = true) : false), ...);
  return done;
}

}  // namespace

hipError_t launch_ln_mod(const LnModArgs& a, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  if (a.D % 256 != 0 || a.D > kMaxElems * 64 || a.seg <= 0 || a.rows_per_sample <= 0) return hipErrorInvalidValue;
  if ((!a.out && !a.q8) || (a.q8 && (!a.s8 || a.lds8 < a.rows))) return hipErrorInvalidValue;
  const bool ok = (a.D % 512 == 0) ? launch_ln_any<8>(a, stream, std::make_integer_sequence<int, kMaxElems / 8>{})
                                   : launch_ln_any<4>(a, stream, std::make_integer_sequence<int, kMaxElems / 4>{});
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace moss
