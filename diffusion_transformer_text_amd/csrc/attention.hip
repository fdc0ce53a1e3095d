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

typedef short v4i16 __attribute__((ext_vector_type(4)));

// LDS tiles, both [64 keys][128 d] bf16 (256-byte rows of 16 chunks of 16 bytes):
//   K: chunk c of row `key` sits at chunk c ^ (key & 15) -> the 16 consecutive rows of one 16-lane
//      phase of a ds_read_b128 at the same logical chunk hit 16 distinct bank groups (a 256-byte row
//      spans all 64 banks, so only the chunk index decides the bank);
//   V: chunk c of row `key` sits at chunk c ^ (4 (key & 3)) -> a transpose read (4 rows x 32 bytes per
//      16-lane group, two groups per 256-byte bank phase) hits distinct 16-byte slots; the earlier
//      c ^ 2 (key & 3) measured 33 % of LDS cycles as bank conflicts (32-lane phases for the b64 read).
// Both tiles are filled by direct global -> LDS loads (1 KB per wave instruction = 4 rows); the
// swizzle is realised by the choice of source chunk.

// gfx950 transpose read (ds_read_b64_tr_b16): within each 16-lane group, lane i receives element
// (i % 4) of the 8-byte pieces addressed by lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12.
__device__ __forceinline__ v4i16 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p);
}

__global__ __launch_bounds__(256, 2) void attention_kernel(AttnArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][BKV * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][BKV * D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 31, fh = lane >> 5;
  // Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2). Remap the linear
  // id so that XCD x runs a contiguous range of (sample, head) pairs with all their query tiles:
  // the ~2 heads resident on an XCD at a time share their K/V in that XCD's L2.
  const int nq = (p.S + BQ - 1) / BQ;
  const int total = nq * p.H * p.B;
  int lin = blockIdx.x;
  if ((total & 7) == 0) lin = (lin & 7) * (total >> 3) + (lin >> 3);
  const int bh = lin / nq;
  const int q0 = (lin - bh * nq) * BQ, h = bh % p.H, b = bh / p.H;
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

  // ---- direct-load assignment: wave w fills windows 4w..4w+3 of each tile (rows 16w .. 16w+15) ----
  const int win_r = lane >> 4, win_pc = lane & 15;
  const int k_lc = win_pc ^ win_r;                  // ^ 4 (window & 3) per window below
  const int v_lc = win_pc ^ (4 * win_r);
  // per-lane source offsets of this wave's windows, relative to the tile's first key row
  int k_src[4], v_src[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int w = wave * 4 + j;                    // window: rows 4w .. 4w+3
    const int row = 4 * w + win_r;
    k_src[j] = (int)(row * p.ld_qkv) + 8 * (k_lc ^ (4 * (w & 3)));
    v_src[j] = (int)(row * p.ld_qkv) + 8 * v_lc;
  }
  auto issue_tile = [&](int k0, int stage) {
    if (k0 + BKV <= S) {
      const uint16_t* kt = Kg + (long)k0 * p.ld_qkv;
      const uint16_t* vt = Vg + (long)k0 * p.ld_qkv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        load_lds_16(kt + k_src[j], &sK[stage][(wave * 4 + j) * 512]);
        load_lds_16(vt + v_src[j], &sV[stage][(wave * 4 + j) * 512]);
      }
    } else {
      // ragged last tile: rows past the sequence re-read its last row (their scores are masked)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int w = wave * 4 + j;
        const long key = min(k0 + 4 * w + win_r, S - 1);
        load_lds_16(Kg + key * p.ld_qkv + 8 * (k_lc ^ (4 * (w & 3))), &sK[stage][w * 512]);
        load_lds_16(Vg + key * p.ld_qkv + 8 * v_lc, &sV[stage][w * 512]);
      }
    }
  };

  // ---- per-lane LDS read offsets (elements), loop-invariant ----
  int k_ofs[D / 16];
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds) k_ofs[ds] = fr * D + (((2 * ds + fh) ^ (fr & 15)) << 3);
  const int g = lane >> 4, j16 = lane & 15;
  int v_ofs[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int lc = 4 * db + 2 * (g & 1) + ((j16 & 3) >> 1);
    v_ofs[db] = ((j16 >> 2) + 4 * (g >> 1)) * D + ((lc ^ (4 * (j16 >> 2))) << 3) + 4 * (j16 & 1);
  }

  floatx16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c = p.scale_log2;

  const int ntiles = (S + BKV - 1) / BKV;
  issue_tile(0, 0);
  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    const int k0 = t * BKV;
    __syncthreads();                  // tile t has landed; the other stage is free again
    if (t + 1 < ntiles) issue_tile(k0 + BKV, cur ^ 1);
    const uint16_t* tK = sK[cur];
    const uint16_t* tV = sV[cur];

    // ---- S^T = K Q^T for 2 blocks of 32 keys ----
    floatx16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(tK + kb * 32 * D + k_ofs[ds]);
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
    // The running max is only moved when a score exceeds it by more than 2^8 in the exp2 domain:
    // with a stale max the probabilities stay below 256 (exact in fp32, same relative precision in
    // bf16), the final normalisation divides by the sum taken against the same max, so the result
    // is unchanged while the O rescale (64 multiplies per lane) runs only a few times per row.
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = (kb == 0 ? 2 : 0); e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (__any((mx - m_run) * c > 8.0f)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[i][e] *= alpha;
      m_run = m_new;
    }
    const float mc = m_run * c;
    float lsum = 0.f;
    bf16x8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pv[j] = __builtin_amdgcn_exp2f(s[kb][8 * hs + j] * c - mc);
          lsum += pv[j];
        }
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = pack2_bf16(pv[2 * j], pv[2 * j + 1]);
        pf[kb][hs] = *reinterpret_cast<bf16x8*>(w);
      }
    }
    l_run += lsum;

    // ---- O^T += V^T P^T: the V^T fragment (d = 32 db + fr, keys 32 kb + 16 hs + 4 fh + {0..3, 8..11})
    //      comes from two transpose reads of the row-major V tile ----
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          const uint16_t* vp = tV + v_ofs[db] + (32 * kb + 16 * hs) * D;
          const v4i16 lo = lds_read_tr16(vp);
          const v4i16 hi = lds_read_tr16(vp + 8 * D);
          const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kb][hs], o[db], 0, 0, 0);
        }
      }
    }
  }

  // ---- normalise and store: lane holds query my_q, d = 32 db + 8 g + 4 fh + [0, 4) ----
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  if (my_q < S) {
    uint16_t* orow = p.out + ((long)b * S + my_q) * p.ld_out + h * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int d = 32 * db + 8 * gg + 4 * fh;
        uint2 w;
        w.x = pack2_bf16(o[db][4 * gg] * inv, o[db][4 * gg + 1] * inv);
        w.y = pack2_bf16(o[db][4 * gg + 2] * inv, o[db][4 * gg + 3] * inv);
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
  const long wgs = (long)((a.S + BQ - 1) / BQ) * a.H * a.B;
  if (wgs > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attention_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, a);
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
