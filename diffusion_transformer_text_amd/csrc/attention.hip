// Exact flash-style softmax attention for the joint [text | image] sequence, head_dim 128 (gfx950).
//
// MOSS-Image's single-stream blocks attend jointly over text and image tokens with no mask
// ("MOSS-Image: specs, settings, VRAM and text rendering tested", "Architecture and specs"); the
// reference quality tier of the MossInfer integration guide runs exact attention. This kernel
// computes softmax(Q K^T / sqrt(d)) V exactly in the online (running max / running sum) form, so the
// S x S score matrix never reaches HBM.
//
// One workgroup = 4 waves = 128 queries of one (sample, head); each wave owns 32 queries. Per
// iteration a tile of 64 keys of K and of V is staged in LDS (double-buffered), both row-major
// [key][d]; the V^T fragments come from gfx950's transpose LDS read. Scores are computed transposed,
// S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 so that lane l holds 32 scores of ONE query (l % 32): the
// row max and row sum are in-lane reductions plus one exchange with lane l ^ 32. The output is also
// computed transposed, O^T = V^T P^T, which leaves the lane's own query in its accumulator columns:
// the online-softmax rescale is a per-lane multiply and P feeds the second MFMA straight from
// registers (no LDS round trip for P). Scores become exp2-domain offsets x = s c - m c as soon as they
// exist, so the probabilities are exp2(x).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moss {
namespace {

constexpr int D = kHeadDim;   // 128
constexpr int BQ = kAttnBQ;   // 128
constexpr int BKV = kAttnBKV; // 64

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// Row sum of the probabilities as the P V product sees them: the two bf16 values of a packed pair are
// added into the fp32 sum by one v_dot2 against (1, 1), half the VALU issues of adding the fp32 values
// one by one. Numerator and normaliser then weight each value row by the same rounded probability.
__device__ __forceinline__ float add_pair_bf16(float acc, uint32_t w) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
}

// Work split of one launch: workgroups [0, n_full) each take a whole query tile (all keys); each of the
// n_split leftover tiles (tile index n_full + j) is split along its key tiles into `parts` workgroups
// that write unnormalised partial results (o, running max, sum) for merge_kernel.
struct AttnSplit {
  int n_full, n_split, parts;
  float* part_o;     // [n_split * parts][BQ queries][128]
  float* part_ml;    // [n_split * parts][BQ queries][2]: running max in the exp2 domain (m c), sum
};

__global__ __launch_bounds__(256, 2) void attention_kernel(AttnArgs p, AttnSplit sp) {
  // Two LDS stages each for K and V, as four separate arrays: every access below names a fixed array
  // (the tile loop is unrolled by two), so the compiler can tell a read of one stage from the
  // direct loads still landing in another and waits for those loads only at the next barrier.
  __shared__ __attribute__((aligned(16))) uint16_t sK0[BKV * D];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[BKV * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[BKV * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV1[BKV * D];

  // the wave index, read once into a scalar register so that per-wave addresses (the LDS windows of
  // the direct loads) are scalar arithmetic instead of a v_readfirstlane per copy
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 31, fh = lane >> 5;
  // Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2). Remap the linear
  // id so that XCD x runs a contiguous range of (sample, head) pairs with all their query tiles:
  // the ~2 heads resident on an XCD at a time share their K/V in that XCD's L2.
  const int nq = (p.S + BQ - 1) / BQ;
  const int S = p.S;
  const int ntiles = (S + BKV - 1) / BKV;
  int lin = blockIdx.x;
  int t_begin = 0, t_end = ntiles, part_slot = -1;
  if (lin < sp.n_full) {
    if ((sp.n_full & 7) == 0) lin = (lin & 7) * (sp.n_full >> 3) + (lin >> 3);
  } else {
    const int j = lin - sp.n_full, part = j % sp.parts;
    part_slot = j;
    lin = sp.n_full + j / sp.parts;
    t_begin = part * ntiles / sp.parts;
    t_end = (part + 1) * ntiles / sp.parts;
  }
  const int bh = lin / nq;
  const int q0 = (lin - bh * nq) * BQ, h = bh % p.H, b = bh / p.H;
  const int DM = p.H * D;
  const uint16_t* base = p.qkv + (long)b * S * p.ld_qkv;
  const uint16_t* Qg = base + h * D;

  // Q fragments (MFMA B operand of S^T = K Q^T): query q, d = 16 ds + 8 fh + [0, 8)
  const int my_q = q0 + wave * 32 + fr;
  const int q_ld = min(my_q, S - 1);
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds)
    qf[ds] = *reinterpret_cast<const bf16x8*>(Qg + (long)q_ld * p.ld_qkv + 16 * ds + 8 * fh);

  // ---- direct-load assignment: wave w fills windows 4w..4w+3 of each tile (rows 16w .. 16w+15) ----
  // A tile is read through a buffer resource over the sample's rows from the tile's first key on, so
  // rows past the end of the sequence (ragged last tile) come back as zeros from the hardware range
  // check: their scores are masked and their probabilities are zero.
  const int win_r = lane >> 4, win_pc = lane & 15;
  const int k_lc = win_pc ^ win_r;                  // ^ 4 (window & 3) per window below
  const int v_lc = win_pc ^ (4 * win_r);
  // per-lane byte offsets of this wave's windows, relative to the tile's first key row
  int k_vo[4], v_vo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int w = wave * 4 + j;                    // window: rows 4w .. 4w+3
    const int row = 4 * w + win_r;
    k_vo[j] = 2 * (row * p.ld_qkv + DM + h * D + 8 * (k_lc ^ (4 * (w & 3))));
    v_vo[j] = 2 * (row * p.ld_qkv + 2 * DM + h * D + 8 * v_lc);
  }
  auto tile_rsrc = [&](int t) {
    const int k0 = t * BKV;
    return make_rsrc(base + (long)k0 * p.ld_qkv, 2 * (S - k0) * p.ld_qkv);
  };
  auto issue_k = [&](int t, uint16_t* dst) {
    const auto r = tile_rsrc(t);
#pragma unroll
    for (int j = 0; j < 4; ++j) buf_load_lds_16(r, dst + (wave * 4 + j) * 512, k_vo[j]);
  };
  auto issue_v = [&](int t, uint16_t* dst) {
    const auto r = tile_rsrc(t);
#pragma unroll
    for (int j = 0; j < 4; ++j) buf_load_lds_16(r, dst + (wave * 4 + j) * 512, v_vo[j]);
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
  // running max in the exp2 domain (m c, m the largest score seen when it last moved) and running sum of
  // the bf16 probabilities
  float mc_run = 0.f, l_run = 0.f;
  const float c = p.scale_log2;

  // S^T = K Q^T for the 64 keys of one LDS tile (2 blocks of 32 keys)
  auto scores = [&](const uint16_t* tK, floatx16 (&sc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[kb][e] = 0.f;
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(tK + kb * 32 * D + k_ofs[ds]);
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ds], sc[kb], 0, 0, 0);
      }
    }
  };
  // row max of one tile's values: in-lane over 32 values, then with lane ^ 32 (same query)
  auto rowmax = [&](const floatx16 (&sc)[2]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; e += 2) mx = max3_f32(mx, sc[kb][e], sc[kb][e + 1]);
    return max_xor32(mx);
  };
  // keys of tile t past the end of the sequence (only the last tile has any) get -inf
  auto mask_tail = [&](floatx16 (&sc)[2], int t) {
    const int k0 = t * BKV;
    if (k0 + BKV <= S) return;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + 32 * kb + 8 * (e >> 2) + 4 * fh + (e & 3);
        if (key >= S) sc[kb][e] = -INFINITY;
      }
  };
  // A tile's scores are turned into x = s c - m c (one fma each) as soon as they exist, and its
  // probabilities are exp2(x). The running max only moves when a tile's largest x exceeds 8 (2^8 in
  // the probabilities): with a stale max the probabilities stay below 256 (exact in fp32, the same
  // relative precision in bf16), and the final normalisation divides by the sum taken against the same
  // max, so the result is unchanged while the O rescale (64 multiplies per lane) runs only a few times
  // per row. A move by d rescales O and the sum by 2^-d and shifts the tile's x by -d.
  auto maybe_shift = [&](float mx, floatx16 (&x)[2]) {
    if (__any(mx > 8.0f)) {
      const float d = mx > 8.0f ? mx : 0.f;
      const float alpha = __builtin_amdgcn_exp2f(-d);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[i][e] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) x[kb][e] -= d;
      mc_run += d;
    }
  };
  // P = exp2(x) as bf16 MFMA operands, and the running row sum of those bf16 values
  auto probs = [&](const floatx16 (&x)[2], bf16x8 (&pf)[2][2]) {
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) pv[j] = __builtin_amdgcn_exp2f(x[kb][8 * hs + j]);
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          w[j] = pack2_bf16(pv[2 * j], pv[2 * j + 1]);
          lsum = add_pair_bf16(lsum, w[j]);
        }
        pf[kb][hs] = __builtin_bit_cast(bf16x8, w);
      }
    }
    l_run += lsum;
  };
  // O^T += V^T P^T: the V^T fragment (d = 32 db + fr, keys 32 kb + 16 hs + 4 fh + {0..3, 8..11})
  // comes from two transpose reads of the row-major V tile
  auto pv_update = [&](const uint16_t* tV, const bf16x8 (&pf)[2][2]) {
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
  };

  // ---- software pipeline: K runs one tile ahead of V. In iteration t the MFMAs of S(t+1) are
  // interleaved with the softmax VALU work of tile t, and the MFMAs of P(t) V(t) with the row max of
  // S(t+1). Stages: K(t) lives in sK[t & 1], V(t) in sV[t & 1]. Iteration t reads K(t+1) and V(t)
  // and refills the two stages read one iteration earlier: K(t+2) -> sK[t & 1], V(t+1) -> sV[(t+1) & 1]. ----
  // key tiles [t_begin, t_end) of this workgroup (all of them unless it holds one part of a split tile)
  issue_k(t_begin, sK0);
  issue_v(t_begin, sV0);
  if (t_begin + 1 < t_end) issue_k(t_begin + 1, sK1);
  lds_copy_barrier();
  floatx16 s_cur[2];
  scores(sK0, s_cur);
  mask_tail(s_cur, t_begin);         // a first tile that is also the last one: mask before the first max
  mc_run = rowmax(s_cur) * c;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) s_cur[kb][e] = s_cur[kb][e] * c - mc_run;
  float mx_cur = 0.f;                // the first tile's x are relative to its own max
  // s_cur holds x(t) on entry; S(t+1) is written to s_next and turned into x(t+1) there (the unrolled
  // pair swaps the two)
  auto iteration = [&](int t, uint16_t* kFree, const uint16_t* kNext, uint16_t* vFree, const uint16_t* vCur,
                       floatx16 (&s_cur)[2], floatx16 (&s_next)[2]) {
    lds_copy_barrier();              // K(t+1) and V(t) have landed; kFree and vFree are no longer read
    if (t + 2 < t_end) issue_k(t + 2, kFree);
    issue_v(t + 1, vFree);
    maybe_shift(mx_cur, s_cur);
    // region A: S(t+1) on the matrix core while the VALU turns x(t) into probabilities. Step i issues
    // one MFMA (accumulators alternate so consecutive MFMAs are independent), the LDS read of the K
    // fragment four steps ahead, and the exp2/pack/sum of two scores; sched_barrier keeps that order.
    bf16x8 pf[2][2];
    {
      const uint16_t* tK = kNext;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s_next[kb][e] = 0.f;
      bf16x8 kf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        kf[i] = *reinterpret_cast<const bf16x8*>(tK + (i & 1) * 32 * D + k_ofs[i >> 1]);
      float lsum = 0.f;
      u32x4 w[4];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s_next[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i & 3], qf[i >> 1], s_next[i & 1], 0, 0, 0);
        if (i + 4 < 16)
          kf[i & 3] = *reinterpret_cast<const bf16x8*>(tK + (i & 1) * 32 * D + k_ofs[(i + 4) >> 1]);
        const float p0 = __builtin_amdgcn_exp2f(s_cur[i >> 3][2 * (i & 7)]);
        const float p1 = __builtin_amdgcn_exp2f(s_cur[i >> 3][2 * (i & 7) + 1]);
        w[i >> 2][i & 3] = pack2_bf16(p0, p1);
        lsum = add_pair_bf16(lsum, w[i >> 2][i & 3]);
        __builtin_amdgcn_sched_barrier(0);
      }
      l_run += lsum;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) pf[kb][hs] = __builtin_bit_cast(bf16x8, w[2 * kb + hs]);
    }
    // region B: P(t) V(t) on the matrix core while the VALU turns S(t+1) into x(t+1) and finds its row
    // max. Step i (16 per tile: 4 d-blocks x 2 key blocks x 2 halves) is one MFMA into o[i & 3], the
    // two transpose reads of the V fragment two steps ahead, and the fma and max of two scores.
    float mx_next;
    {
      const uint16_t* tV = vCur;
      auto vfrag = [&](int i) {
        const int db = i & 3, hs = (i >> 2) & 1, kb = i >> 3;
        const uint16_t* vp = tV + v_ofs[db] + (32 * kb + 16 * hs) * D;
        const v4i16 lo = lds_read_tr16(vp);
        const v4i16 hi = lds_read_tr16(vp + 8 * D);
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      constexpr int VA = 2;          // V fragments are read VA steps ahead of their MFMA
      bf16x8 vf[VA + 1];
#pragma unroll
      for (int j = 0; j < VA; ++j) vf[j] = vfrag(j);
      float mx = -INFINITY;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i + VA < 16) vf[(i + VA) % (VA + 1)] = vfrag(i + VA);
        o[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i % (VA + 1)], pf[i >> 3][(i >> 2) & 1], o[i & 3], 0, 0, 0);
        s_next[i >> 3][(2 * i) & 15] = s_next[i >> 3][(2 * i) & 15] * c - mc_run;
        s_next[i >> 3][(2 * i + 1) & 15] = s_next[i >> 3][(2 * i + 1) & 15] * c - mc_run;
        mx = max3_f32(mx, s_next[i >> 3][(2 * i) & 15], s_next[i >> 3][(2 * i + 1) & 15]);
        asm volatile("" : "+v"(mx));   // no instruction: keeps the chain from being rebuilt as a tree after the loop
        __builtin_amdgcn_sched_barrier(0);
      }
      mx_next = fmaxf(mx, __shfl_xor(mx, 32, 64));   // (the VALU exchange here costs a spill)
    }
    mx_cur = mx_next;
  };
  floatx16 s_alt[2];
  int t = t_begin;
  for (; t + 2 < t_end; t += 2) {
    iteration(t, sK0, sK1, sV1, sV0, s_cur, s_alt);
    iteration(t + 1, sK1, sK0, sV0, sV1, s_alt, s_cur);
  }
  if (t + 1 < t_end) {
    iteration(t, sK0, sK1, sV1, sV0, s_cur, s_alt);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s_cur[kb] = s_alt[kb];
  }
  // ---- last tile: mask keys past the sequence, then the same softmax and P V ----
  {
    const int t = t_end - 1;
    const int k0 = t * BKV;
    lds_copy_barrier();              // V(t) has landed
    if (k0 + BKV > S) {              // x of the keys past the sequence: -inf, and the max without them
      mask_tail(s_cur, t);
      mx_cur = rowmax(s_cur);
    }
    maybe_shift(mx_cur, s_cur);
    bf16x8 pf[2][2];
    probs(s_cur, pf);
    pv_update(((t - t_begin) & 1) ? sV1 : sV0, pf);
  }

  const float l_tot = sum_xor32(l_run);
  if (part_slot >= 0) {
    // one part of a split tile: the unnormalised output and the (max in the exp2 domain, sum) pair it
    // is relative to
    const long qrow = (long)part_slot * BQ + wave * 32 + fr;
    float* po = sp.part_o + qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
        *reinterpret_cast<float4*>(po + 32 * db + 8 * gg + 4 * fh) =
            make_float4(o[db][4 * gg], o[db][4 * gg + 1], o[db][4 * gg + 2], o[db][4 * gg + 3]);
    if (fh == 0) *reinterpret_cast<float2*>(sp.part_ml + 2 * qrow) = make_float2(mc_run, l_tot);
    return;
  }
  // ---- normalise and store: lane holds query my_q, d = 32 db + 8 g + 4 fh + [0, 4) ----
  const float inv = 1.0f / l_tot;
  if (my_q < S && p.q8) {                 // MXFP8 codes (both lanes of a query take this branch)
    const long row = (long)b * S + my_q;
    uint8_t* crow = p.q8 + row * DM + h * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      float v[4][4];
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[gg][e] = o[db][4 * gg + e] * inv;
      mx_store_pair_block(v, fh, crow + 32 * db, p.s8 + mx_scale_byte((h * D + 32 * db) / 32, row, p.lds8));
    }
  } else if (my_q < S) {
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

// Combines the parts of the split tiles: workgroup x covers 16 queries of split tile x / 8; thread
// (query qi = tid / 16, dims [8 (tid % 16), +8)), so the 16 threads of a query read its 512-byte
// partial rows contiguously. Each part stores its running max in the exp2 domain (mc_p = m_p c):
// out = sum_p o_p 2^(mc_p - mc) / sum_p l_p 2^(mc_p - mc), mc = max_p mc_p.
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs p, AttnSplit sp) {
  constexpr int QPW = 16;                                // queries per workgroup
  const int j = blockIdx.x / (BQ / QPW);
  const int qi = (blockIdx.x % (BQ / QPW)) * QPW + (threadIdx.x >> 4), d0 = (threadIdx.x & 15) * 8;
  const int nq = (p.S + BQ - 1) / BQ;
  const int idx = sp.n_full + j;
  const int bh = idx / nq;
  const int q0 = (idx - bh * nq) * BQ, h = bh % p.H, b = bh / p.H;
  const int q = q0 + qi;
  if (q >= p.S) return;
  float m = -INFINITY;
  for (int pt = 0; pt < sp.parts; ++pt) m = fmaxf(m, sp.part_ml[2 * ((long)(j * sp.parts + pt) * BQ + qi)]);
  float acc[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) acc[d] = 0.f;
  float l = 0.f;
  for (int pt = 0; pt < sp.parts; ++pt) {
    const long row = (long)(j * sp.parts + pt) * BQ + qi;
    const float2 ml = *reinterpret_cast<const float2*>(sp.part_ml + 2 * row);
    const float f = __builtin_amdgcn_exp2f(ml.x - m);
    l += ml.y * f;
    const float4* po = reinterpret_cast<const float4*>(sp.part_o + row * D + d0);
    const float4 v0 = po[0], v1 = po[1];
    acc[0] += v0.x * f;
    acc[1] += v0.y * f;
    acc[2] += v0.z * f;
    acc[3] += v0.w * f;
    acc[4] += v1.x * f;
    acc[5] += v1.y * f;
    acc[6] += v1.z * f;
    acc[7] += v1.w * f;
  }
  const float inv = 1.0f / l;
  const long row = (long)b * p.S + q;
  if (p.q8) {
    // MXFP8 codes: a 32-column block is 4 threads (consecutive lanes, the same query)
    float r[8];
    float amax = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      r[d] = round_bf16(acc[d] * inv);
      amax = fmaxf(amax, fabsf(r[d]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    const int ex = mx_exponent(amax);
    const float sc = mx_inv_scale(ex);
    *reinterpret_cast<uint2*>(p.q8 + row * (p.H * D) + h * D + d0) =
        make_uint2(mx_pack4(r[0], r[1], r[2], r[3], sc), mx_pack4(r[4], r[5], r[6], r[7], sc));
    if ((threadIdx.x & 3) == 0) p.s8[mx_scale_byte((h * D + d0) / 32, row, p.lds8)] = (uint8_t)(ex + 127);
    return;
  }
  uint2* orow = reinterpret_cast<uint2*>(p.out + row * p.ld_out + h * D + d0);   // 8-byte aligned
  orow[0] = make_uint2(pack2_bf16(acc[0] * inv, acc[1] * inv), pack2_bf16(acc[2] * inv, acc[3] * inv));
  orow[1] = make_uint2(pack2_bf16(acc[4] * inv, acc[5] * inv), pack2_bf16(acc[6] * inv, acc[7] * inv));
}

// The split plan (host_plan.cpp): `slots` workgroups fit on the chip at once (two per CU).
AttnSplit split_plan(int B, int S, int H) {
  const AttnSplitPlan pl = attention_split_plan(B, S, H, 2L * device_cu_count());
  AttnSplit sp{};
  sp.n_full = pl.n_full;
  sp.n_split = pl.n_split;
  sp.parts = pl.parts;
  return sp;
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

// Compute units of the current device (cached per device).
int device_cu_count() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

size_t attention_split_workspace(int B, int S, int H) {
  return attention_split_bytes(B, S, H, 2L * device_cu_count());
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream, void* ws, size_t ws_bytes) {
  if (a.S <= 0 || a.B <= 0) return hipSuccess;
  if (a.ld_qkv % 8 != 0 || a.ld_out % 4 != 0) return hipErrorInvalidValue;
  if (a.q8 && (!a.s8 || (a.H * D) % 256 != 0 || a.lds8 < (long)a.B * a.S)) return hipErrorInvalidValue;
  const long wgs = (long)((a.S + BQ - 1) / BQ) * a.H * a.B;
  if (wgs > 0x7fffffffL) return hipErrorInvalidValue;
  if (2L * a.S * a.ld_qkv > 0x7fffffffL) return hipErrorInvalidValue;   // 32-bit buffer offsets per sample
  AttnSplit sp = split_plan(a.B, a.S, a.H);
  const size_t rows = (size_t)sp.n_split * sp.parts * BQ;
  if (rows == 0 || !ws || ws_bytes < attention_split_workspace(a.B, a.S, a.H)) {
    sp.n_full = (int)wgs;                    // no workspace (or nothing to split): whole tiles only
    sp.n_split = 0;
    sp.parts = 1;
  } else {
    char* base = static_cast<char*>(ws);
    base += (256 - (reinterpret_cast<uintptr_t>(base) & 255)) & 255;
    sp.part_o = reinterpret_cast<float*>(base);
    sp.part_ml = reinterpret_cast<float*>(base + rows * D * 4);
  }
  const long grid = (long)sp.n_full + (long)sp.n_split * sp.parts;
  hipLaunchKernelGGL(attention_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a, sp);
  if (sp.n_split > 0)
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)sp.n_split * (BQ / 16)), dim3(256), 0, stream, a, sp);
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
