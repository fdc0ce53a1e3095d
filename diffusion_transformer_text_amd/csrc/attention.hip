// Exact flash-style softmax attention for the joint [text | image] sequence, head_dim 128 (gfx950).
//
// MOSS-Image's single-stream blocks attend jointly over text and image tokens with no mask
// ("MOSS-Image: specs, settings, VRAM and text rendering tested", "Architecture and specs"); the
// reference quality tier of the MossInfer integration guide runs exact attention. This kernel
// computes softmax(Q K^T / sqrt(d)) V exactly in the online (running max / running sum) form, so the
// S x S score matrix never reaches HBM.
//
// One workgroup = 4 waves = 128 queries of one (sample, head); each wave owns 32 queries. Per
// iteration a tile of 64 keys is staged in LDS (double-buffered): K as [key][d] and V transposed as
// [d][key]. Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 so that lane l
// holds 32 scores of ONE query (l % 32): the row max and row sum are in-lane reductions plus one
// exchange with lane l ^ 32. The output is also computed transposed, O^T = V^T P^T, which leaves the
// lane's own query in its accumulator columns: the online-softmax rescale is a per-lane multiply and
// P feeds the second MFMA straight from the score registers (no LDS round trip for P).
#include "common.h"
#include "kernels.h"

namespace moss {
namespace {

constexpr int D = kHeadDim;   // 128
constexpr int BQ = 128;
constexpr int BKV = 64;

// K tile: [64 keys][128 d], 16-byte chunk c of row `key` at chunk c ^ (key & 7).
__device__ __forceinline__ int k_off(int key, int chunk) { return key * D + ((chunk ^ (key & 7)) << 3); }

// V^T tile: [128 d][64 keys], 8-byte unit u (4 keys) of row d at unit u ^ f(d). f makes both the
// transposed writes (16 rows d = 8c + e at once) and the fragment reads (16 consecutive rows) hit
// distinct banks.
__device__ __forceinline__ int vt_f(int d) { return (d & 15) ^ ((d >> 3) & 15); }
__device__ __forceinline__ int vt_off(int d, int key) { return d * BKV + ((((key >> 2) ^ vt_f(d)) & 15) << 2) + (key & 3); }

__global__ __launch_bounds__(256, 2) void attention_kernel(AttnArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][BKV * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][D * BKV];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 31, fh = lane >> 5;
  const int q0 = blockIdx.x * BQ, h = blockIdx.y, b = blockIdx.z;
  const int S = p.S;
  const int DM = p.H * D;
  const uint16_t* base = p.qkv + (long)b * S * p.ld_qkv;
  const uint16_t* Qg = base + h * D;
  const uint16_t* Kg = base + DM + h * D;
  const uint16_t* Vg = base + 2 * DM + h * D;

  // Q fragments (MFMA B operand of S^T = K Q^T): query q, d = 16 ds + 8 fh + [0, 8)
  const int my_q = q0 + wave * 32 + fr;
  const int q_ld = min(my_q, S - 1);
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds)
    qf[ds] = *reinterpret_cast<const bf16x8*>(Qg + (long)q_ld * p.ld_qkv + 16 * ds + 8 * fh);

  // K/V staging assignment. K: item = tid + 256 j -> key = item >> 4, chunk = item & 15.
  // V: item = tid + 256 j -> key pair = item >> 4 (keys 2 pair, 2 pair + 1), d chunk = item & 15.
  const int it_c = tid & 15, it_r = tid >> 4;
  uint4 rk[4], rv[4];
  auto load_kv = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = min(k0 + it_r + 16 * j, S - 1);
      rk[j] = *reinterpret_cast<const uint4*>(Kg + (long)key * p.ld_qkv + it_c * 8);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int pair = it_r + 16 * j;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int key = min(k0 + 2 * pair + kk, S - 1);
        rv[2 * j + kk] = *reinterpret_cast<const uint4*>(Vg + (long)key * p.ld_qkv + it_c * 8);
      }
    }
  };
  auto store_kv = [&](int stage) {
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4*>(&sK[stage][k_off(it_r + 16 * j, it_c)]) = rk[j];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int pair = it_r + 16 * j;
      const uint32_t* a = reinterpret_cast<const uint32_t*>(&rv[2 * j]);
      const uint32_t* c = reinterpret_cast<const uint32_t*>(&rv[2 * j + 1]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // d = 8 it_c + 2w and 2w + 1: pack (key 2pair, key 2pair+1) per d
        const uint32_t lo = (a[w] & 0xffffu) | (c[w] << 16);
        const uint32_t hi = (a[w] >> 16) | (c[w] & 0xffff0000u);
        const int d0 = 8 * it_c + 2 * w;
        *reinterpret_cast<uint32_t*>(&sV[stage][vt_off(d0, 2 * pair)]) = lo;
        *reinterpret_cast<uint32_t*>(&sV[stage][vt_off(d0 + 1, 2 * pair)]) = hi;
      }
    }
  };

  floatx16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c = p.scale_log2;

  const int ntiles = (S + BKV - 1) / BKV;
  load_kv(0);
  store_kv(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    const int k0 = t * BKV;
    if (t + 1 < ntiles) load_kv(k0 + BKV);

    // ---- S^T = K Q^T for 2 blocks of 32 keys ----
    floatx16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&sK[cur][k_off(32 * kb + fr, 2 * ds + fh)]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ds], s[kb], 0, 0, 0);
      }
    }
    // mask keys past the end of the sequence (last tile only)
    if (k0 + BKV > S) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = k0 + 32 * kb + 8 * (e >> 2) + 4 * fh + (e & 3);
          if (key >= S) s[kb][e] = -INFINITY;
        }
    }
    // ---- online softmax (one query per lane, shared with lane ^ 32) ----
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f((m_run - m_new) * c);
    const float mc = m_new * c;
    float lsum = 0.f;
    bf16x8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pv[j] = exp2f(s[kb][8 * hs + j] * c - mc);
          lsum += pv[j];
        }
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = pack2_bf16(pv[2 * j], pv[2 * j + 1]);
        pf[kb][hs] = *reinterpret_cast<bf16x8*>(w);
      }
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[i][e] *= alpha;

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int d = 32 * db + fr;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          const int key_a = 32 * kb + 16 * hs + 4 * fh;
          const uint2 va = *reinterpret_cast<const uint2*>(&sV[cur][vt_off(d, key_a)]);
          const uint2 vb = *reinterpret_cast<const uint2*>(&sV[cur][vt_off(d, key_a + 8)]);
          uint32_t w[4] = {va.x, va.y, vb.x, vb.y};
          const bf16x8 vf = *reinterpret_cast<bf16x8*>(w);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kb][hs], o[db], 0, 0, 0);
        }
      }
    }
    if (t + 1 < ntiles) store_kv(cur ^ 1);
    __syncthreads();
  }

  // ---- normalise and store: lane holds query my_q, d = 32 db + 8 g + 4 fh + [0, 4) ----
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  if (my_q < S) {
    uint16_t* orow = p.out + ((long)b * S + my_q) * p.ld_out + h * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * fh;
        uint2 w;
        w.x = pack2_bf16(o[db][4 * g] * inv, o[db][4 * g + 1] * inv);
        w.y = pack2_bf16(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d) = w;
      }
  }
}

__global__ void rope_inplace_kernel(uint16_t* qkv, int B, int S, int T, int grid_w, int H, long ld,
                                    const float* cos_t, const float* sin_t) {
  // one thread per (row, rotary pair) over the q and k columns of the image rows
  const int pairs = 2 * H * D / 2;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long n_img = S - T;
  if (idx >= (long)B * n_img * pairs) return;
  const int pi = (int)(idx % pairs);
  const long rr = idx / pairs;
  const int b = (int)(rr / n_img), ni = (int)(rr % n_img);
  const int col = 2 * pi;
  const int dim = col & (D - 1);
  const int pos = (dim < D / 2) ? ni / grid_w : ni % grid_w;
  const int k = (dim & (D / 2 - 1)) >> 1;
  uint16_t* x = qkv + ((long)b * S + T + ni) * ld + col;
  const float a = bf16_to_f32(x[0]), c2 = bf16_to_f32(x[1]);
  const float cs = cos_t[pos * (D / 4) + k], sn = sin_t[pos * (D / 4) + k];
  x[0] = f32_to_bf16(a * cs - c2 * sn);
  x[1] = f32_to_bf16(a * sn + c2 * cs);
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream) {
  if (a.S <= 0 || a.B <= 0) return hipSuccess;
  if (a.ld_qkv % 8 != 0 || a.ld_out % 4 != 0) return hipErrorInvalidValue;
  dim3 grid((a.S + BQ - 1) / BQ, a.H, a.B);
  hipLaunchKernelGGL(attention_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_rope_inplace(uint16_t* qkv, int B, int S, int T, int grid_w, int H, long ld,
                               const float* cos_t, const float* sin_t, hipStream_t stream) {
  const long total = (long)B * (S - T) * H * D;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(rope_inplace_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     qkv, B, S, T, grid_w, H, ld, cos_t, sin_t);
  return hipGetLastError();
}

}  // namespace moss
