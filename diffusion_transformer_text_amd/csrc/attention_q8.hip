// 8-bit attention for the FP8 tier (gfx950): Q K^T on INT8 codes with v_mfma_i32_32x32x32_i8 and
// P V on FP8 E4M3 codes with v_mfma_scale_f32_32x32x64_f8f6f4, fp32 softmax in between.
//
// The pages' faster quality tiers run one of four 8-bit attention modes (q8_fp8: 8-bit Q and K, FP8
// P V) instead of exact attention (MossInfer integration guide, "Quality tier" and the attention
// modes of its feature table) without printing their arithmetic. Reading: Q symmetric INT8 per token
// and head (scale amax / 127), K symmetric INT8 per block of 64 consecutive keys and head, V FP8 E4M3
// per channel (scale amax / 448); integer dot products are exact, the softmax runs online over the
// 64-key blocks, each query's reference max moving to a block's max only when that is more than one
// log2 unit above it (so the rare moves are the only rescales and every probability stays <= 2), the
// probabilities are rounded to E4M3 on the scale 224, and the normaliser sums the same rounded
// probabilities, so the output is a convex combination of the dequantized V rows. Codes are decided in fp32: x * 127 and x * 448 are exact for
// bf16 inputs, followed by one correctly rounded division.
//
// Two passes quantize the (roped) bf16 qkv of a layer: q8k8_quant_kernel writes the INT8 Q and K and
// each key block's V channel maxima; vt8_quant_kernel reduces those maxima and writes V transposed
// per head ([128 dims][keys], FP8), with the keys of every 64-key block permuted into the order in
// which the P operand of the P V MFMA holds them, so the V^T fragment of a lane is 32 contiguous bytes.
//
// The attention kernel keeps the bf16 kernel's transposed form (S^T = K Q^T, O^T = V^T P^T: lane l
// holds the scores and the output of query l % 32) with 8 KB K and V^T tiles, half of the bf16 ones.
#include <climits>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moss {
namespace {

constexpr int D = kHeadDim;   // 128
constexpr int KB = 64;        // keys per block / tile
constexpr float kE4M3Max = 448.f;
constexpr float kLog2PScale = 7.807354922057604f;   // log2 224: probabilities <= 2 code to <= 448
constexpr int kMaxKeyBlocks = 512;   // 32768 keys

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ int int8_code(float x, float amax) {
  // rint(x * 127 / amax), x * 127 exact, one correctly rounded division; amax == 0 -> 0
  return amax > 0.f ? (int)__builtin_rintf(__fdiv_rn(x * 127.f, amax)) : 0;
}

// Position of key kk (0..63) of a block in the permuted V^T row: the P operand of lane (query, h)
// holds, in byte b, the probability of key 32 (b >> 4) + 8 ((b & 15) >> 2) + 4 h + (b & 3), so key
// 32 kb + 8 j + 4 h + i goes to position 32 h + 16 kb + 4 j + i.
__device__ __forceinline__ int vt_pos(int kk) {
  const int kb = kk >> 5, j = (kk >> 3) & 3, h = (kk >> 2) & 1, i = kk & 3;
  return 32 * h + 16 * kb + 4 * j + i;
}

// grid (key blocks, H, B), 256 threads: thread (row r = tid / 4, quarter c = tid % 4) owns dims
// [32c, 32c + 32) of sequence row k0 + r of head h.
__global__ __launch_bounds__(256) void q8k8_quant_kernel(AttnQ8Args p) {
  __shared__ float s_red[4];
  __shared__ float s_vmax[KB][D + 1];
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, r = tid >> 2, c = tid & 3, lane = tid & 63, wave = tid >> 6;
  const int S = p.S, DM = p.H * D;
  const int row = blk * KB + r;
  const bool valid = row < S;
  const long grow = (long)b * S + row;
  float q[32], k[32], v[32];
  if (valid) {
    const uint4* src = reinterpret_cast<const uint4*>(p.qkv + grow * p.ld_qkv + h * D + 32 * c);
#pragma unroll
    for (int part = 0; part < 3; ++part) {
      const uint4* sp = src + part * (DM / 8);
      float* dst = part == 0 ? q : (part == 1 ? k : v);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint4 w = sp[u];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dst[8 * u + 2 * e] = bf16_lo(ws[e]);
          dst[8 * u + 2 * e + 1] = bf16_hi(ws[e]);
        }
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) q[e] = k[e] = v[e] = 0.f;
  }
  // Q: per row, reduce over the 4 threads of the row
  float qa = 0.f, ka = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    qa = fmaxf(qa, fabsf(q[e]));
    ka = fmaxf(ka, fabsf(k[e]));
    s_vmax[r][32 * c + e] = fabsf(v[e]);
  }
  qa = fmaxf(qa, __shfl_xor(qa, 1, 64));
  qa = fmaxf(qa, __shfl_xor(qa, 2, 64));
  // K: the whole block
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ka = fmaxf(ka, __shfl_xor(ka, o, 64));
  if (lane == 0) s_red[wave] = ka;
  __syncthreads();
  ka = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  if (valid) {
    uint32_t qw[8], kw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      uint32_t a = 0, bb = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a |= (uint32_t)(int8_code(q[4 * u + e], qa) & 0xff) << (8 * e);
        bb |= (uint32_t)(int8_code(k[4 * u + e], ka) & 0xff) << (8 * e);
      }
      qw[u] = a;
      kw[u] = bb;
    }
    uint4* qd = reinterpret_cast<uint4*>(p.q8 + grow * DM + h * D + 32 * c);
    uint4* kd = reinterpret_cast<uint4*>(p.k8 + grow * DM + h * D + 32 * c);
    qd[0] = make_uint4(qw[0], qw[1], qw[2], qw[3]);
    qd[1] = make_uint4(qw[4], qw[5], qw[6], qw[7]);
    kd[0] = make_uint4(kw[0], kw[1], kw[2], kw[3]);
    kd[1] = make_uint4(kw[4], kw[5], kw[6], kw[7]);
    if (c == 0) p.qa[grow * p.H + h] = qa;
  }
  const long bh = (long)b * p.H + h;
  if (tid == 0) p.ka[bh * p.nblk + blk] = ka;
  // V: this block's channel maxima
  if (tid < D) {
    float m = 0.f;
    for (int rr = 0; rr < KB; ++rr) m = fmaxf(m, s_vmax[rr][tid]);
    p.vpart[(bh * p.nblk + blk) * D + tid] = m;
  }
}

// grid (H, B), 1024 threads: V's channel maxima over all key blocks. Thread (group g = tid / 128,
// dim d = tid % 128) reduces key blocks g, g + 8, ... (independent loads, several in flight), then
// the 8 groups combine through LDS.
__global__ __launch_bounds__(1024) void va_reduce_kernel(AttnQ8Args p) {
  __shared__ float s_m[8][D];
  const long bh = (long)blockIdx.y * p.H + blockIdx.x;
  const int d = threadIdx.x & (D - 1), g = threadIdx.x >> 7;
  const float* src = p.vpart + bh * p.nblk * D + d;
  float m = 0.f;
#pragma unroll 4
  for (int t = g; t < p.nblk; t += 8) m = fmaxf(m, src[(long)t * D]);
  s_m[g][d] = m;
  __syncthreads();
  if (g == 0) {
#pragma unroll
    for (int j = 1; j < 8; ++j) m = fmaxf(m, s_m[j][d]);
    p.va[bh * D + d] = m;
  }
}

// grid (key blocks, H, B), 256 threads: this block's 64 keys of V as E4M3 codes, transposed and
// permuted: vt8[(b H + h) D + d][blk 64 + vt_pos(key)].
__global__ __launch_bounds__(256) void vt8_quant_kernel(AttnQ8Args p) {
  __shared__ float s_va[D];
  __shared__ __attribute__((aligned(16))) uint8_t s_t[D][KB];
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, r = tid >> 2, c = tid & 3;
  const int S = p.S, DM = p.H * D;
  const long bh = (long)b * p.H + h;
  if (tid < D) s_va[tid] = p.va[bh * D + tid];
  __syncthreads();
  const int row = blk * KB + r;
  float v[32];
  if (row < S) {
    const uint4* src = reinterpret_cast<const uint4*>(p.qkv + ((long)b * S + row) * p.ld_qkv + 2 * DM + h * D + 32 * c);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint4 w = src[u];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * u + 2 * e] = bf16_lo(ws[e]);
        v[8 * u + 2 * e + 1] = bf16_hi(ws[e]);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) v[e] = 0.f;
  }
  const int pos = vt_pos(r);
#pragma unroll
  for (int e = 0; e < 32; e += 2) {
    const int d = 32 * c + e;
    const float a0 = s_va[d] > 0.f ? __fdiv_rn(v[e] * kE4M3Max, s_va[d]) : 0.f;
    const float a1 = s_va[d + 1] > 0.f ? __fdiv_rn(v[e + 1] * kE4M3Max, s_va[d + 1]) : 0.f;
    const int w = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, __float_as_int(a0), false);   // bytes 2-3 unused
    s_t[d][pos] = (uint8_t)(w & 0xff);
    s_t[d + 1][pos] = (uint8_t)((w >> 8) & 0xff);
  }
  __syncthreads();
  // 128 rows x 64 bytes out: thread t writes 16 bytes of row t / 4 twice (rows t / 4 and 64 + t / 4)
  const long rowlen = (long)p.nblk * KB;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int d = half * 64 + (tid >> 2), q4 = tid & 3;
    const uint4 w = *reinterpret_cast<const uint4*>(&s_t[d][16 * q4]);
    *reinterpret_cast<uint4*>(p.vt8 + (bh * D + d) * rowlen + (long)blk * KB + 16 * q4) = w;
  }
}

// LDS tiles: K [64 keys][128 B] with 16-byte chunk c of row r at chunk c ^ ((r >> 1) & 7) (the 16 rows
// of a ds_read_b128 phase land on 16 distinct (row parity, chunk) slots of a 256-byte bank line);
// V^T [128 dims][64 B] with chunk c of row d at c ^ ((d >> 2) & 3) (4 rows per bank line).
__device__ __forceinline__ int k_swz(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }
__device__ __forceinline__ int v_swz(int d, int c) { return d * 64 + ((c ^ ((d >> 2) & 3)) << 4); }

template <int N>
__device__ __forceinline__ void copy_barrier_n() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0070 | N);   // this wave's copies older than the N newest have landed
  asm volatile("s_barrier" ::: "memory");
}

__global__ __launch_bounds__(256, 2) void attention_q8_kernel(AttnQ8Args p) {
  constexpr int BQ = 128;
  // four stages of a K tile and a V^T tile (16 KB each), as separate arrays named statically
  __shared__ __attribute__((aligned(16))) uint8_t st0[2 * KB * D];
  __shared__ __attribute__((aligned(16))) uint8_t st1[2 * KB * D];
  __shared__ __attribute__((aligned(16))) uint8_t st2[2 * KB * D];
  __shared__ __attribute__((aligned(16))) uint8_t st3[2 * KB * D];
  __shared__ float s_ka[kMaxKeyBlocks];

  // the wave index in a scalar register: per-wave addresses (LDS windows of the direct loads) stay scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 31, fh = lane >> 5;
  const int nq = (p.S + BQ - 1) / BQ;
  const int total = nq * p.H * p.B;
  int lin = blockIdx.x;
  if ((total & 7) == 0) lin = (lin & 7) * (total >> 3) + (lin >> 3);   // XCD-contiguous (sample, head) runs
  const int bhl = lin / nq;
  const int q0 = (lin - bhl * nq) * BQ, h = bhl % p.H, b = bhl / p.H;
  const int S = p.S, DM = p.H * D;
  const long bh = (long)b * p.H + h;

  // Q fragment (MFMA B operand of S^T = K Q^T): query my_q, dims [32 ds + 16 fh, +16)
  const int my_q = q0 + wave * 32 + fr;
  const int q_ld = min(my_q, S - 1);
  v4i qf[D / 32];
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds)
    qf[ds] = *reinterpret_cast<const v4i*>(p.q8 + ((long)b * S + q_ld) * DM + h * D + 32 * ds + 16 * fh);
  const float qscale = p.qa[((long)b * S + q_ld) * p.H + h] * (1.0f / 127.f) * p.scale_log2;

  // direct loads: K tile = 8 windows of 8 rows x 128 B, V^T tile = 8 windows of 16 rows x 64 B; wave w
  // fills windows 2w, 2w + 1 of each. K rows past the sequence come back as zeros (range check).
  const long rowlen = (long)p.nblk * KB;
  int k_vo[2], v_vo[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int w = 2 * wave + j;
    const int kr = 8 * w + (lane >> 3), kc = (lane & 7) ^ ((kr >> 1) & 7);
    k_vo[j] = kr * DM + h * D + 16 * kc;
    const int vd = 16 * w + (lane >> 2), vc = (lane & 3) ^ ((vd >> 2) & 3);
    v_vo[j] = (int)((bh * D + vd) * rowlen) + 16 * vc;   // the tile's key offset is added per tile
  }
  const __amdgpu_buffer_rsrc_t rV = make_rsrc(p.vt8, (int)((long)p.B * p.H * D * rowlen));
  const __amdgpu_buffer_rsrc_t rK = make_rsrc(p.k8 + (long)b * S * DM, S * DM);
  const int ntiles = p.nblk;
  // copies of tiles past the last one (the look-ahead of the last steps) get offsets beyond their
  // buffers: the range check returns zeros without touching memory, so every step issues the same
  // number of copies and the waits below stay exact; such a tile's keys are all masked
  auto issue = [&](int t, uint8_t* st) __attribute__((always_inline)) {
    const bool live = t < ntiles;
    const uint32_t ko = live ? (uint32_t)(t * KB * DM) : 0x80000000u;   // both buffers are < 2^31 bytes
    const uint32_t vo = live ? (uint32_t)(t * KB) : 0x80000000u;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      buf_load_lds_16(rK, st + (2 * wave + j) * 1024, (int)(ko + (uint32_t)k_vo[j]));
      buf_load_lds_16(rV, st + KB * D + (2 * wave + j) * 1024, (int)(vo + (uint32_t)v_vo[j]));
    }
  };

  floatx16 o[D / 32];
  floatx16 o_l;   // sum of the rounded probabilities (ones x P^T), the same in every register
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    o_l[e] = 0.f;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) o[i][e] = 0.f;
  }
  float m_run = -INFINITY;
  constexpr int kBiasI = 0x4B400000;          // the float 1.5 * 2^23
  constexpr float kBiasF = 12582912.0f;
  const v16i bias = {kBiasI, kBiasI, kBiasI, kBiasI, kBiasI, kBiasI, kBiasI, kBiasI,
                     kBiasI, kBiasI, kBiasI, kBiasI, kBiasI, kBiasI, kBiasI, kBiasI};
  const v8i ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                    0x38383838, 0x38383838, 0x38383838, 0x38383838};   // E4M3 1.0

  // tile t from stage st; MASK: keys past the sequence get score -inf (only the last tile has any)
  auto tile = [&](auto mask_c, int t, const uint8_t* st) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_c)::value;
    const uint8_t* tK = st;
    const uint8_t* tV = st + KB * D;
    // S^T = K Q^T on INT8 codes: 2 key blocks x 4 dim slices of 32
    // The accumulators start at kBiasI (the first MFMA of each chain reads the constant registers
    // `bias` as its C operand), so each ends as kBiasI + s for the integer score s; |s| <= 128^2 128 =
    // 2^21 for any INT8 codes keeps that in the binade [2^23, 2^24), where its bit pattern read as a
    // float is exactly 1.5 * 2^23 + s: no int-to-float conversion per score.
    v16i si[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int ds = 0; ds < D / 32; ++ds) {
        const v4i kf = *reinterpret_cast<const v4i*>(tK + k_swz(32 * kb + fr, 2 * ds + fh));
        si[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qf[ds], ds == 0 ? bias : si[kb], 0, 0, 0);
      }
    }
    // scores in the exp2 domain are s * f (f >= 0, so the largest code gives the largest score); keys
    // past the sequence are masked (the biased scores are positive, so 0 stands below every key)
    const float f = qscale * s_ka[min(t, ntiles - 1)] * (1.0f / 127.f);
    const int k0 = t * KB;
    int mi = 0;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const bool dead = MASK && k0 + 32 * kb + 8 * (e >> 2) + 4 * fh + (e & 3) >= S;
        mi = max(mi, dead ? 0 : si[kb][e]);
      }
    mi = max_xor32(mi);
    const float mx = (float)(mi - kBiasI) * f;   // a wholly masked tile never moves the reference (tile 0 has a key)
    // lazy reference max: a query's reference moves to the tile's max only when that is more than one
    // log2 unit above it, so every probability stays <= 2; a move rescales that query's sums
    const bool move = mx - m_run > 1.0f;
    if (__any(move)) {
      const float alpha = move ? __builtin_amdgcn_exp2f(m_run - mx) : 1.0f;   // exp2(-inf) = 0 at the start
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        o_l[e] *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) o[i][e] *= alpha;
      }
      m_run = move ? mx : m_run;
    }
    // P <= 2 as E4M3 codes of 224 p = exp2(s - m_run + log2 224) <= 448: byte b of the operand = key
    // 32 (b >> 4) + 8 ((b & 15) >> 2) + 4 fh + (b & 3)
    // exp2 argument s f - m_b = (1.5 * 2^23 + s) f + c0 with c0 = -(1.5 * 2^23 f + m_b) rounded once per
    // tile: one fma per score, off the exact argument by at most half an ulp of c0 (<= 0.75 f + 2^-24
    // |m_b| log2 units; f is about 1e-4 for unit-variance q and k, 2e-3 for scores spread over +-60)
    const float m_b = m_run - kLog2PScale;
    const float c0 = __builtin_fmaf(-kBiasF, f, -m_b);
    v8i pf;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int kb = u >> 2, e0 = 4 * (u & 3);
      float a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = __builtin_fmaf(__int_as_float(si[kb][e0 + i]), f, c0);
        if (MASK && k0 + 32 * kb + 8 * (e0 >> 2) + 4 * fh + i >= S) a[i] = -INFINITY;
      }
      // bytes 2-3 of the first conversion's third operand are overwritten by the second: the first
      // probability's own register serves, so no zero is materialised per word
      const float p0 = __builtin_amdgcn_exp2f(a[0]);
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(p0, __builtin_amdgcn_exp2f(a[1]), __float_as_int(p0), false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_exp2f(a[2]), __builtin_amdgcn_exp2f(a[3]), w, true);
      pf[u] = w;
    }
    // O^T += V^T P^T on E4M3 codes (scale bytes 127 = 2^0): V^T fragment = 32 contiguous bytes of
    // row d = 32 db + fr at positions [32 fh, 32 fh + 32)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int d = 32 * db + fr;
      const v4i lo = *reinterpret_cast<const v4i*>(tV + v_swz(d, 2 * fh));
      const v4i hi = *reinterpret_cast<const v4i*>(tV + v_swz(d, 2 * fh + 1));
      const v8i vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf, o[db], 0, 0, 0, 127, 0, 127);
    }
    o_l = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pf, o_l, 0, 0, 0, 127, 0, 127);
  };

  // Four stages, three tiles in flight: step t waits for tile t (the copies of tiles t+1 and t+2, four
  // per wave each, may still run), then refills tile t-1's stage with tile t+3 (every wave finished
  // reading it before this barrier) and computes tile t. The loop runs whole groups of four steps,
  // unrolled so every LDS access names a fixed array; the steps past the last tile only see masked keys.
  // each key block's K scale, in LDS (a global load here would be a vector load, and waiting for it
  // would also wait for the tile copies issued before it)
  for (int i = tid; i < ntiles; i += 256) s_ka[i] = p.ka[bh * ntiles + i];
  issue(0, st0);
  issue(1, st1);
  issue(2, st2);
  // Whole groups of four interior tiles, then one last group with masking: it holds the last tile
  // (keys past the sequence masked) and up to three steps past it, whose keys are all masked (zero
  // probabilities, zero V): no branch inside the steps, so the compiler keeps its waits exact.
  auto group = [&](auto mask_c, int t) __attribute__((always_inline)) {
    copy_barrier_n<8>();
    issue(t + 3, st3);
    tile(mask_c, t, st0);
    copy_barrier_n<8>();
    issue(t + 4, st0);
    tile(mask_c, t + 1, st1);
    copy_barrier_n<8>();
    issue(t + 5, st1);
    tile(mask_c, t + 2, st2);
    copy_barrier_n<8>();
    issue(t + 6, st2);
    tile(mask_c, t + 3, st3);
  };
  int t = 0;
  for (; t + 4 < ntiles; t += 4) group(std::false_type{}, t);
  group(std::true_type{}, t);
  __builtin_amdgcn_s_waitcnt(0x0F70);       // the look-ahead copies land before the LDS is released

  // out = O / l, with V's channel scale: lane holds query my_q, d = 32 db + 8 g + 4 fh + [0, 4)
  if (my_q < S && p.out8) {               // MXFP8 codes (both lanes of a query take this branch)
    const float inv = 1.0f / (kE4M3Max * o_l[0]);
    const long row = (long)b * S + my_q;
    uint8_t* crow = p.out8 + row * DM + h * D;
    const float* va = p.va + bh * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      float v[4][4];
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const float4 sv = *reinterpret_cast<const float4*>(va + 32 * db + 8 * gg + 4 * fh);
        v[gg][0] = o[db][4 * gg] * sv.x * inv;
        v[gg][1] = o[db][4 * gg + 1] * sv.y * inv;
        v[gg][2] = o[db][4 * gg + 2] * sv.z * inv;
        v[gg][3] = o[db][4 * gg + 3] * sv.w * inv;
      }
      mx_store_pair_block(v, fh, crow + 32 * db, p.out8_scale + mx_scale_byte((h * D + 32 * db) / 32, row, p.lds8));
    }
  } else if (my_q < S) {
    const float inv = 1.0f / (kE4M3Max * o_l[0]);
    uint16_t* orow = p.out + ((long)b * S + my_q) * p.ld_out + h * D;
    const float* va = p.va + bh * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int d = 32 * db + 8 * gg + 4 * fh;
        const float4 sv = *reinterpret_cast<const float4*>(va + d);
        uint2 w;
        w.x = pack2_bf16(o[db][4 * gg] * sv.x * inv, o[db][4 * gg + 1] * sv.y * inv);
        w.y = pack2_bf16(o[db][4 * gg + 2] * sv.z * inv, o[db][4 * gg + 3] * sv.w * inv);
        *reinterpret_cast<uint2*>(orow + d) = w;
      }
  }
}

}  // namespace

size_t attention_q8_workspace(int B, int S, int H) {
  static_assert(KB == kAttnBKV && D == kHeadDim, "the workspace size assumes 64-key blocks of 128 dims");
  return attention_q8_bytes(B, S, H);
}

hipError_t launch_attention_q8(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (a.S <= 0 || a.B <= 0) return hipSuccess;
  if (a.ld_qkv % 8 != 0 || a.ld_out % 4 != 0 || !ws || ws_bytes < attention_q8_workspace(a.B, a.S, a.H) ||
      (reinterpret_cast<uintptr_t>(ws) & 255))
    return hipErrorInvalidValue;
  const long nblk = (a.S + KB - 1) / KB;
  const long DM = (long)a.H * D;
  if (nblk > kMaxKeyBlocks) return hipErrorInvalidValue;
  if (a.q8 && (!a.s8 || DM % 256 != 0 || a.lds8 < (long)a.B * a.S)) return hipErrorInvalidValue;
  // 32-bit buffer offsets: K codes per sample and all of V^T
  if ((long)a.S * DM > 0x7fffffffL || (long)a.B * a.H * D * nblk * KB > 0x7fffffffL) return hipErrorInvalidValue;
  AttnQ8Args p;
  p.qkv = a.qkv;
  p.out = a.out;
  p.B = a.B;
  p.S = a.S;
  p.H = a.H;
  p.ld_qkv = a.ld_qkv;
  p.ld_out = a.ld_out;
  p.scale_log2 = a.scale_log2;
  p.nblk = (int)nblk;
  p.out8 = a.q8;
  p.out8_scale = a.s8;
  p.lds8 = a.lds8;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  char* c = static_cast<char*>(ws);
  const size_t M = (size_t)a.B * a.S;
  p.q8 = (int8_t*)c;
  c += al(M * DM);
  p.k8 = (int8_t*)c;
  c += al(M * DM);
  p.vt8 = (uint8_t*)c;
  c += al((size_t)a.B * a.H * D * nblk * KB);
  p.qa = (float*)c;
  c += al(M * a.H * 4);
  p.ka = (float*)c;
  c += al((size_t)a.B * a.H * nblk * 4);
  p.va = (float*)c;
  c += al((size_t)a.B * a.H * D * 4);
  p.vpart = (float*)c;
  const dim3 qgrid((unsigned)nblk, (unsigned)a.H, (unsigned)a.B);
  hipLaunchKernelGGL(q8k8_quant_kernel, qgrid, dim3(256), 0, stream, p);
  hipLaunchKernelGGL(va_reduce_kernel, dim3((unsigned)a.H, (unsigned)a.B), dim3(1024), 0, stream, p);
  hipLaunchKernelGGL(vt8_quant_kernel, qgrid, dim3(256), 0, stream, p);
  const long wgs = (long)((a.S + 127) / 128) * a.H * a.B;
  hipLaunchKernelGGL(attention_q8_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace moss
