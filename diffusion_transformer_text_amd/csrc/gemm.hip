// bf16 MFMA GEMM with fused epilogues for the DiT projections (gfx950).
//
// The projections of a joint block are plain bf16 GEMMs with fp32 accumulation (MossInfer
// integration guide, "Quality tier": the reference tier runs the DiT's bf16 GEMMs). Their
// elementwise tails are fused into the GEMM epilogue, as the Qwen-Image 2.1 cookbook does with
// separate kernels ("Lossless RoPE fusion", "Lossless MLP and residual fusion"): the rotary turn of
// q/k, the gated residual add and the SiLU-multiply of the SwiGLU FFN.
//
// Tiling: a workgroup of WAVES_M x WAVES_N waves computes a BM (tokens) x BN (features) tile, BK = 64,
// with both operands staged through a double-buffered, XOR-swizzled LDS tile. Each wave issues
// v_mfma_f32_32x32x16_bf16 with the WEIGHT fragment as the MFMA A operand and the activation
// fragment as the B operand, so the accumulator of lane l holds token (l % 32) and, per group of
// four registers, four consecutive output features: the epilogue stores 8-byte runs and finds the
// rotary pair (2k, 2k+1) and the gate/up pair in its own registers.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moss {
namespace {

constexpr int BK = 64;
constexpr int kGroupM = 8;   // tile rows per L2 group

template <int BM, int BN, int WAVES_M, int WAVES_N>
struct Tile {
  static constexpr int NW = WAVES_M * WAVES_N;          // waves per workgroup
  static constexpr int THREADS = 64 * NW;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;   // wave tile
  static constexpr int TM = WM / 32, TN = WN / 32;      // 32x32 MFMA blocks per wave
  static constexpr int STAGE = (BM + BN) * BK;          // elements per LDS stage
  static_assert(WN % 64 == 0, "a wave's features must hold whole 64-row gate/up groups");
  static_assert((BM / 8) % NW == 0 && (BN / 8) % NW == 0, "1 KB load windows must split evenly");
};

// Element offset of 16-byte chunk c of row r in a [rows][BK] bf16 LDS tile. A fragment load reads
// one chunk from each of 32 consecutive rows; gfx950 serves ds_read_b128 in phases of 16 lanes over
// 64 four-byte banks (256 bytes), i.e. two 128-byte rows per bank line. XOR-ing the chunk index
// with (r & 7) ^ ((r >> 3) & 1) puts the 16 rows of a phase on 16 distinct (row parity, chunk)
// slots; a plain (r & 7) leaves rows r and r + 8 on the same banks (measured: every read 2-way
// conflicted, SQ_LDS_BANK_CONFLICT = half of SQ_LDS_IDX_ACTIVE).
__device__ __forceinline__ int swz_key(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ swz_key(r)) << 3); }

// Maps the linear workgroup id to a (tile_m, tile_n) pair. Workgroups are dispatched round-robin
// over the 8 XCDs; the remap gives each XCD a contiguous run of tiles, and within the run tiles go
// in groups of kGroupM tile rows so the workgroups resident on one XCD share A rows and W columns
// in that XCD's L2.
__device__ __forceinline__ void tile_coords(int nM, int nN, int& tm, int& tn) {
  const int nt = gridDim.x;
  int lin = blockIdx.x;
  if ((nt & 7) == 0) lin = (lin & 7) * (nt >> 3) + (lin >> 3);
  const int per_group = kGroupM * nN;
  const int group = lin / per_group;
  const int first_m = group * kGroupM;
  const int gsize = min(nM - first_m, kGroupM);
  const int in_group = lin - group * per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// ---- epilogue: acc[i][j][4g + e] = C[token m, feature n + e] ----
template <class T, int EPI>
__device__ __forceinline__ void store_tile(const GemmArgs& p, floatx16 (&acc)[T::TM][T::TN], int m0, int n0, int wm,
                                           int wn, int fr, int fh) {
#pragma unroll
  for (int i = 0; i < T::TM; ++i) {
    const int m = m0 + wm * T::WM + i * 32 + fr;
    if (m >= p.M) continue;
    if constexpr (EPI == EPI_SWIGLU) {
      // feature blocks (2q, 2q+1) of this wave are the gate and up rows of the same 32 h-columns
      uint16_t* out = static_cast<uint16_t*>(p.out);
#pragma unroll
      for (int q = 0; q < T::TN / 2; ++q) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int hc = (n0 + wn * T::WN) / 2 + q * 32 + 8 * g + 4 * fh;
          float h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = silu_f32(acc[i][2 * q][4 * g + e]) * acc[i][2 * q + 1][4 * g + e];
          uint2 v;
          v.x = pack2_bf16(h[0], h[1]);
          v.y = pack2_bf16(h[2], h[3]);
          *reinterpret_cast<uint2*>(out + (long)m * p.ldo + hc) = v;
        }
      }
    } else if constexpr (EPI == EPI_SWIGLU_MX) {
      // the same 32 h-columns per q are one MX block: 16 values here, 16 in lane ^ 32 (same token);
      // codes of the bf16-rounded h, as the separate quantizer would write them
      uint8_t* out = static_cast<uint8_t*>(p.out);
#pragma unroll
      for (int q = 0; q < T::TN / 2; ++q) {
        float h[4][4];
        float amax = 0.f;
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            h[g][e] = round_bf16(silu_f32(acc[i][2 * q][4 * g + e]) * acc[i][2 * q + 1][4 * g + e]);
            amax = fmaxf(amax, fabsf(h[g][e]));
          }
        amax = max_xor32(amax);
        const int ex = mx_exponent(amax);
        const float inv = mx_inv_scale(ex);
        const int hb = (n0 + wn * T::WN) / 2 + q * 32;
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<uint32_t*>(out + (long)m * p.ldo + hb + 8 * g + 4 * fh) =
              mx_pack4(h[g][0], h[g][1], h[g][2], h[g][3], inv);
        if (fh == 0) p.out_scale[mx_scale_byte(hb / 32, m, p.lds_out)] = (uint8_t)(ex + 127);
      }
    } else {
#pragma unroll
      for (int j = 0; j < T::TN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * T::WN + j * 32 + 8 * g + 4 * fh;
          float c[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) c[e] = acc[i][j][4 * g + e];
          if constexpr (EPI == EPI_BF16) {
            const long orow = (long)(m / p.seg) * p.seg_stride + p.seg_off + m % p.seg;
            uint2 v;
            v.x = pack2_bf16(c[0], c[1]);
            v.y = pack2_bf16(c[2], c[3]);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + orow * p.ldo + n) = v;
          } else if constexpr (EPI == EPI_QKV_ROPE) {
#pragma unroll
            for (int e = 0; e < 4; ++e) c[e] = round_bf16(c[e]);
            const int t = m % p.S;
            if (n < p.rope_cols && t >= p.T) {
              const int ni = t - p.T;
              const int dim = n & (kHeadDim - 1);
              const int pos = (dim < kHeadDim / 2) ? ni / p.grid_w : ni % p.grid_w;
              const int k0 = (dim & (kHeadDim / 2 - 1)) >> 1;
#pragma unroll
              for (int pr = 0; pr < 2; ++pr) {
                const float cs = p.rope_cos[pos * (kHeadDim / 4) + k0 + pr];
                const float sn = p.rope_sin[pos * (kHeadDim / 4) + k0 + pr];
                const float a = c[2 * pr], b = c[2 * pr + 1];
                c[2 * pr] = a * cs - b * sn;
                c[2 * pr + 1] = a * sn + b * cs;
              }
            }
            uint2 v;
            v.x = pack2_bf16(c[0], c[1]);
            v.y = pack2_bf16(c[2], c[3]);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + (long)m * p.ldo + n) = v;
          } else if constexpr (EPI == EPI_GATED_RES) {
            uint16_t* xo = static_cast<uint16_t*>(p.out) + (long)m * p.ldo + n;
            const uint2 xv = *reinterpret_cast<const uint2*>(xo);
            const uint2 gv = *reinterpret_cast<const uint2*>(p.gate + (long)(m / p.rows_per_sample) * p.gate_stride + n);
            const float x0 = __uint_as_float(xv.x << 16), x1 = __uint_as_float(xv.x & 0xffff0000u);
            const float x2 = __uint_as_float(xv.y << 16), x3 = __uint_as_float(xv.y & 0xffff0000u);
            const float g0 = __uint_as_float(gv.x << 16), g1 = __uint_as_float(gv.x & 0xffff0000u);
            const float g2 = __uint_as_float(gv.y << 16), g3 = __uint_as_float(gv.y & 0xffff0000u);
            uint2 v;
            v.x = pack2_bf16(x0 + g0 * c[0], x1 + g1 * c[1]);
            v.y = pack2_bf16(x2 + g2 * c[2], x3 + g3 * c[3]);
            *reinterpret_cast<uint2*>(xo) = v;
          } else if constexpr (EPI == EPI_F32) {
            *reinterpret_cast<float4*>(static_cast<float*>(p.out) + (long)m * p.ldo + n) =
                make_float4(c[0], c[1], c[2], c[3]);
          } else if constexpr (EPI == EPI_F32_UNPATCH) {
            const int b = m / p.n_img, ni = m % p.n_img;
            const int gw = p.lat_w / 2;
            const int y = 2 * (ni / gw), x = 2 * (ni % gw);
            const int ch = n >> 2;
            float* v = static_cast<float*>(p.out) + (((long)b * p.C + ch) * p.lat_h + y) * p.lat_w + x;
            *reinterpret_cast<float2*>(v) = make_float2(c[0], c[1]);
            *reinterpret_cast<float2*>(v + p.lat_w) = make_float2(c[2], c[3]);
          }
        }
      }
    }
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int EPI>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, 1) void gemm_bf16_kernel(GemmArgs p) {
  using T = Tile<BM, BN, WAVES_M, WAVES_N>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * T::STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int nN = p.N / BN, nM = (p.M + BM - 1) / BM;
  int tm, tn;
  tile_coords(nM, nN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // ---- global -> LDS, without staging registers: global_load_lds_dwordx4 writes lane i's 16 bytes
  // to (LDS base + 16 i), so one instruction fills a 1 KB window = 8 rows of 128 bytes. The XOR
  // swizzle is realised by the choice of source: window lane i stores physical chunk i % 8 of row
  // i / 8, which holds logical chunk (i % 8) ^ swz_key(row).
  constexpr int A_WIN = BM / 8, W_WIN = BN / 8;          // 1 KB windows per tile
  constexpr int A_PER_WAVE = A_WIN / T::NW, W_PER_WAVE = W_WIN / T::NW;
  // window rows are 8 w + lane / 8 with w = wave + NW j (NW even), so the row's swizzle key is
  // (lane / 8) ^ (wave & 1) for every window of this wave
  const int win_row = lane >> 3, win_chunk = (lane & 7) ^ win_row ^ (wave & 1);
  uint32_t a_off[A_PER_WAVE], w_off[W_PER_WAVE];
#pragma unroll
  for (int j = 0; j < A_PER_WAVE; ++j) {
    const int r = min(m0 + (wave + T::NW * j) * 8 + win_row, p.M - 1);
    a_off[j] = (uint32_t)(r * p.lda + win_chunk * 8);
  }
#pragma unroll
  for (int j = 0; j < W_PER_WAVE; ++j) {
    const int r = n0 + (wave + T::NW * j) * 8 + win_row;
    w_off[j] = (uint32_t)(r * p.ldw + win_chunk * 8);
  }
  // loads of one tile are spread over the four k16 slices of the previous tile's MFMA work, so the
  // wave never waits behind its own queue of memory instructions before starting to compute
  constexpr int LOADS = A_PER_WAVE + W_PER_WAVE;
  constexpr int LOADS_PER_SLICE = (LOADS + BK / 16 - 1) / (BK / 16);
  auto issue_part = [&](int kt, int stage, int part) {
    const int k0 = kt * BK;
    uint16_t* sA = lds + stage * T::STAGE;
    uint16_t* sW = sA + BM * BK;
#pragma unroll
    for (int q = 0; q < LOADS_PER_SLICE; ++q) {
      const int j = part * LOADS_PER_SLICE + q;
      if (j < A_PER_WAVE) {
        load_lds_16(p.A + a_off[j] + k0, sA + (wave + T::NW * j) * 512);
      } else if (j < LOADS) {
        const int jw = j - A_PER_WAVE;
        load_lds_16(p.W + w_off[jw] + k0, sW + (wave + T::NW * jw) * 512);
      }
    }
  };

  floatx16 acc[T::TM][T::TN];
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int fr = lane & 31, fh = lane >> 5;
  // fragment rows of this lane: wave and block offsets are multiples of 32, so swz_key(row) =
  // swz_key(fr) and the swizzle term is a per-lane constant
  const int a_row0 = wm * T::WM + fr, w_row0 = wn * T::WN + fr;
  const int KT = p.K / BK;
  bf16x8 fa[2][T::TM], fw[2][T::TN];
  auto load_frags = [&](const uint16_t* sA, const uint16_t* sW, int s, int buf) {
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
      fa[buf][i] = *reinterpret_cast<const bf16x8*>(sA + swz(a_row0 + i * 32, 2 * s + fh));
#pragma unroll
    for (int j = 0; j < T::TN; ++j)
      fw[buf][j] = *reinterpret_cast<const bf16x8*>(sW + swz(w_row0 + j * 32, 2 * s + fh));
  };

#pragma unroll
  for (int part = 0; part < BK / 16; ++part) issue_part(0, 0, part);
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    lds_copy_barrier();                 // tile kt has landed in LDS; stage cur ^ 1 is free again
    const bool more = kt + 1 < KT;
    const uint16_t* sA = lds + cur * T::STAGE;
    const uint16_t* sW = sA + BM * BK;
    load_frags(sA, sW, 0, 0);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      // the next slice's fragment reads are issued before this slice's MFMAs and kept there: the
      // LDS latency then hides behind TM * TN matrix instructions instead of stalling the wave
      if (s + 1 < BK / 16) load_frags(sA, sW, s + 1, (s + 1) & 1);
      if (more) issue_part(kt + 1, cur ^ 1, s);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[s & 1][j], fa[s & 1][i], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  store_tile<T, EPI>(p, acc, m0, n0, wm, wn, fr, fh);
}

// ---------------------------------------------------------------------------------------------
// Big projections: BK = 32 and four LDS stages (the same 128 KB as two stages of BK = 64), so a
// k-tile's global -> LDS copies are issued three k-tiles before it is used. The stages are four
// separate LDS arrays and the k loop is unrolled by four, so every LDS access names a fixed array:
// the compiler then sees that reading one stage does not alias the copies still landing in the others
// and does not wait for them. The wait for a k-tile is explicit (s_waitcnt vmcnt(N) with N = the
// copies issued after that k-tile), followed by a barrier.
// LDS rows are 32 bf16 (64 bytes, four 16-byte chunks); chunk c of row r is stored at chunk
// c ^ ((r >> 2) & 3): the 16 rows a ds_read_b128 phase reads then cover 16 distinct (bank quarter,
// chunk) slots (conflict-free), and a 1 KB copy window holds 16 whole rows.
constexpr int BK2 = 32;
__device__ __forceinline__ int swz2(int r, int c) { return r * BK2 + ((c ^ ((r >> 2) & 3)) << 3); }

// Workgroup barrier of the pipeline: s_waitcnt vmcnt(N) lgkmcnt(0), then s_barrier. vmcnt(N)
// leaves only the N newest copies in flight (the main loop issues no other vector-memory
// instruction, and they complete in order), lgkmcnt(0) finishes this wave's LDS reads (so a stage
// may be refilled after the barrier). The barrier is written as asm with a memory clobber on
// purpose: __syncthreads() carries a workgroup fence, and the compiler treats the pending copies as
// LDS writes under that fence and waits for all of them (vmcnt(0)), which would drain the pipeline.
// The clobber keeps the compiler from moving memory accesses across the barrier.
template <int N>
__device__ __forceinline__ void copy_barrier() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0070 | N);
  asm volatile("s_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------------------------
// Ping-pong GEMM for the big projections: a 256 x 256 tile, BK = 32 k-tiles in four LDS stages, eight
// waves in two groups of four (waves 0-3 and 4-7; wave w runs on SIMD w % 4, so every SIMD holds one
// wave of each group). Group g owns rows [128 g, 128 g + 128) of the tile, each of its waves 128 rows x
// 64 features (4 x 2 accumulator blocks of 32 x 32). The groups alternate, half a k-tile apart, between
// a COMPUTE phase -- the 16 MFMAs of one k-tile on fragments already in registers, with no memory
// instruction in between, at raised wave priority -- and a MEMORY phase -- this wave's four global ->
// LDS copies three k-tiles ahead and the twelve fragment reads of its next k-tile. While one wave of a
// SIMD computes, the other loads, so the matrix pipe always has a wave with its operands ready; a
// workgroup barrier separates consecutive phases.
//
// Phases (k-tile t, KT k-tiles): phase 2t: group 0 computes t, group 1 loads t; phase 2t + 1: group 1
// computes t, group 0 loads t + 1 (group 0 loads k-tile 0 in phase -1). Each memory phase for k-tile t
// issues the copies of k-tile t + 3 into the stage of k-tile t - 1, which both groups finished reading
// before the previous barrier. Every wave issues 4 copies per memory phase (copies past the last
// k-tile point beyond the buffer: the range check writes zeros to a stage no longer read), so before
// every barrier `vmcnt(8)` leaves exactly the two newest k-tiles' copies in flight and k-tile t + 1 is
// in LDS, from every wave, by the start of the phase that first reads it.
//
// Measured against the same tile computed by eight waves that each interleave copies, fragment reads
// and MFMAs (one barrier per k-tile; bit-identical results): 5-7 % faster on the four projections.
// Under this load the chip is power-limited: the ping-pong raises the matrix pipe's busy fraction to
// about 0.67 while the clock falls to about 1.7 GHz (rocprofv3 GRBM_GUI_ACTIVE over the kernel), a
// register-only MFMA loop with random operands runs at about 1.77 GHz; two k-tiles per phase (half the
// barriers) and splitting the fragment reads between the two phases were slower or equal.
template <int EPI>
__global__ __launch_bounds__(512, 1) void gemm_bf16_pp_kernel(GemmArgs p) {
  constexpr int BM = 256, BN = 256;
  using T = Tile<BM, BN, 2, 4>;                           // wave tile 128 x 64: TM = 4, TN = 2
  constexpr int SZ = (BM + BN) * BK2;                     // elements per stage: A rows, then W rows
  __shared__ __attribute__((aligned(16))) uint16_t st0[SZ];
  __shared__ __attribute__((aligned(16))) uint16_t st1[SZ];
  __shared__ __attribute__((aligned(16))) uint16_t st2[SZ];
  __shared__ __attribute__((aligned(16))) uint16_t st3[SZ];

  // the wave index in a scalar register: per-wave addresses (LDS windows of the direct loads) stay scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;               // wm = the wave's group
  const int nN = p.N / BN, nM = (p.M + BM - 1) / BM;
  int tm, tn;
  tile_coords(nM, nN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // copy windows: 16 rows x 64 bytes; lane i writes LDS bytes 16 i (row i / 4, physical chunk i % 4)
  // and so reads logical chunk (i % 4) ^ ((row >> 2) & 3) = (i % 4) ^ ((i >> 4) & 3) of its row
  constexpr int A_PER_WAVE = BM / 16 / T::NW, W_PER_WAVE = BN / 16 / T::NW;   // 2 + 2 copy windows
  constexpr int LOADS = A_PER_WAVE + W_PER_WAVE;
  static_assert(LOADS == 4, "the vmcnt counts below assume four copies per wave per k-tile");
  const int win_row = lane >> 2, win_chunk = (lane & 3) ^ ((lane >> 4) & 3);
  uint32_t a_off[A_PER_WAVE], w_off[W_PER_WAVE];
#pragma unroll
  for (int j = 0; j < A_PER_WAVE; ++j) {
    const int r = min(m0 + (wave + T::NW * j) * 16 + win_row, p.M - 1);
    a_off[j] = (uint32_t)(r * p.lda + win_chunk * 8);
  }
#pragma unroll
  for (int j = 0; j < W_PER_WAVE; ++j) {
    const int r = n0 + (wave + T::NW * j) * 16 + win_row;
    w_off[j] = (uint32_t)(r * p.ldw + win_chunk * 8);
  }
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A, (int)(2L * p.M * p.lda));
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(p.W, (int)(2L * p.N * p.ldw));
  const int KT = p.K / BK2;                               // a multiple of 4 (checked at launch)
  auto issue = [&](int kt, uint16_t* st) {
    const bool real = kt < KT;
    const int k0 = kt * BK2;
#pragma unroll
    for (int j = 0; j < A_PER_WAVE; ++j)
      buf_load_lds_16(rA, st + (wave + T::NW * j) * 512, real ? 2 * (int)(a_off[j] + k0) : 0x7ffffff0);
#pragma unroll
    for (int j = 0; j < W_PER_WAVE; ++j)
      buf_load_lds_16(rW, st + BM * BK2 + (wave + T::NW * j) * 512, real ? 2 * (int)(w_off[j] + k0) : 0x7ffffff0);
  };

  floatx16 acc[T::TM][T::TN];
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int fr = lane & 31, fh = lane >> 5;
  const int a_row0 = wm * T::WM + fr, w_row0 = wn * T::WN + fr;
  bf16x8 fa[2][T::TM], fw[2][T::TN];                      // [k16 slice][block] of the next k-tile
  // memory phase: copies of k-tile `kt_issue` into `fill`, then the fragments of the k-tile in `cur`
  auto mem = [&](const uint16_t* cur, int kt_issue, uint16_t* fill) {
    issue(kt_issue, fill);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int i = 0; i < T::TM; ++i)
        fa[s][i] = *reinterpret_cast<const bf16x8*>(cur + swz2(a_row0 + i * 32, 2 * s + fh));
#pragma unroll
      for (int j = 0; j < T::TN; ++j)
        fw[s][j] = *reinterpret_cast<const bf16x8*>(cur + BM * BK2 + swz2(w_row0 + j * 32, 2 * s + fh));
    }
  };
  auto compute = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[s][j], fa[s][i], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto bar = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    copy_barrier<2 * LOADS>();
    __builtin_amdgcn_sched_barrier(0);
  };

  issue(0, st0);
  issue(1, st1);
  issue(2, st2);
  bar();                                                  // k-tile 0 has landed (phase -1 starts)
  if (wm == 0) {
    mem(st0, 3, st3);                                     // phase -1: load k-tile 0
    bar();
    for (int t = 0; t < KT; t += 4) {                     // k-tiles t .. t + 3 (stages 0 .. 3)
      compute();                                          // phase 2t
      bar();
      mem(st1, t + 4, st0);                               // phase 2t + 1: load t + 1, copy t + 4
      bar();
      compute();
      bar();
      mem(st2, t + 5, st1);
      bar();
      compute();
      bar();
      mem(st3, t + 6, st2);
      bar();
      compute();                                          // k-tile t + 3
      bar();
      if (t + 4 < KT) {
        mem(st0, t + 7, st3);
        bar();
      }
    }
  } else {
    bar();                                                // phase -1: nothing to do
    for (int t = 0; t < KT; t += 4) {
      mem(st0, t + 3, st3);                               // phase 2t: load t, copy t + 3
      bar();
      compute();                                          // phase 2t + 1
      bar();
      mem(st1, t + 4, st0);
      bar();
      compute();
      bar();
      mem(st2, t + 5, st1);
      bar();
      compute();
      bar();
      mem(st3, t + 6, st2);
      bar();
      compute();                                          // k-tile t + 3
      if (t + 4 < KT) bar();
    }
  }
  // the look-ahead copies (zeros into unused stages) land before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(0x0F70);                     // vmcnt(0)
  store_tile<T, EPI>(p, acc, m0, n0, wm, wn, fr, fh);
}

// ---------------------------------------------------------------------------------------------
// MXFP8 GEMM (the FP8 tier). One v_mfma_scale_f32_32x32x64_f8f6f4 consumes a k-tile of 64 E4M3 codes:
// lane (row r = lane % 32, half h = lane / 32) supplies bytes 0..15 = K [16h, 16h + 16) and bytes
// 16..31 = K [32 + 16h, 48 + 16h) of row r, i.e. 16-byte chunks h and 2 + h of the row's 64 bytes,
// and the E8M0 scale of 32-element block h of row r (measured on the hardware with an in-bounds probe).
//
// A k-tile row is 64 bytes, so a 256 x 256 tile stages 32 KB per k-tile; four stages are in LDS.
//
// Scales do not go through LDS: a lane loads its own scale words straight into VGPRs. Scales are
// stored as 32-bit words, word (2g + h) * ld + r holding in byte q the scale of block 8g + 2q + h of
// row r, so one word covers the four k-tiles 4g .. 4g + 3 and k-tile 4g + q picks byte q with the
// MFMA's scale byte select. A lane's words for group g + 1 are loaded during group g.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ int swzb(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }

// copy_barrier for vmcnt up to 63 (the count's high bits sit in bits 15:14 of the immediate)
template <int N>
__device__ __forceinline__ void copy_barrier64() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0070 | (N & 15) | ((N >> 4) << 14));
  asm volatile("s_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------------------------
// Ping-pong MXFP8 GEMM: the bf16 ping-pong kernel's schedule on MXFP8 operands. A 64-element FP8 k-tile
// is a 64-byte row, exactly the bf16 kernel's BK = 32 k-tile, so the four 32 KB stages, the copy
// windows, the swizzle and the phase structure are the same; one k-tile is 4 x 2 scaled MFMAs per wave
// (32 x 32 x 64, 64 cycles each: the same 512 matrix-core cycles per compute phase as 16 bf16 MFMAs),
// its fragments 12 ds_read_b128 (two 16-byte halves per operand). The scale words of a group of four
// k-tiles (byte q of a word = k-tile 4g + q, the MFMA's opsel) are per-lane global loads: each wave
// loads the next group's six words in the memory phase of the group's second k-tile, so the barriers
// whose window of the two most recent memory phases holds them wait with vmcnt(8 + 6) instead of
// vmcnt(8) and every k-tile copy is still in LDS, from every wave, before its first reader; the words
// are complete two phases before the trip that copies them into use.
//
// Measured against the previous schedule (four waves, one per SIMD, 128 x 128 each with the
// accumulators in AGPRs, every MFMA followed by one copy, scale load or fragment half; bit-identical
// fp32 results on random MXFP8 operands at M = 8704): out -5.6 %, gate/up -5.5 %, qkv -1.0 %, down
// +0.3 %, -3.1 % over a block's four projections.
template <int EPI>
__global__ __launch_bounds__(512, 1) void gemm_mxfp8_pp_kernel(GemmArgs p) {
  constexpr int BM = 256, BN = 256;
  using T = Tile<BM, BN, 2, 4>;                           // wave tile 128 x 64: TM = 4, TN = 2
  typedef int int8v __attribute__((ext_vector_type(8)));
  typedef int int4v __attribute__((ext_vector_type(4)));
  constexpr int SZ = (BM + BN) * 64;                      // bytes per stage: A rows, then W rows
  __shared__ __attribute__((aligned(16))) uint8_t st0[SZ];
  __shared__ __attribute__((aligned(16))) uint8_t st1[SZ];
  __shared__ __attribute__((aligned(16))) uint8_t st2[SZ];
  __shared__ __attribute__((aligned(16))) uint8_t st3[SZ];

  // the wave index in a scalar register: per-wave addresses (LDS windows of the direct loads) stay scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;               // wm = the wave's group
  const int nN = p.N / BN, nM = (p.M + BM - 1) / BM;
  int tm, tn;
  tile_coords(nM, nN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  constexpr int A_PER_WAVE = BM / 16 / T::NW, W_PER_WAVE = BN / 16 / T::NW;   // 2 + 2 copy windows
  constexpr int LOADS = A_PER_WAVE + W_PER_WAVE;
  constexpr int NSC = T::TM + T::TN;                      // scale words per lane and group
  static_assert(LOADS == 4 && NSC == 6, "the vmcnt counts below assume four copies and six scale words");
  const int win_row = lane >> 2, win_chunk = (lane & 3) ^ ((lane >> 4) & 3);
  uint32_t a_off[A_PER_WAVE], w_off[W_PER_WAVE];
#pragma unroll
  for (int j = 0; j < A_PER_WAVE; ++j) {
    const int r = min(m0 + (wave + T::NW * j) * 16 + win_row, p.M - 1);
    a_off[j] = (uint32_t)(r * p.lda + win_chunk * 16);
  }
#pragma unroll
  for (int j = 0; j < W_PER_WAVE; ++j) {
    const int r = n0 + (wave + T::NW * j) * 16 + win_row;
    w_off[j] = (uint32_t)(r * p.ldw + win_chunk * 16);
  }
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A, (int)((long)p.M * p.lda));
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(p.W, (int)((long)p.N * p.ldw));
  const int KT = p.K / 64;                                // a multiple of 4 (K % 256 == 0)
  auto issue = [&](int kt, uint8_t* st) {
    const bool real = kt < KT;
    const int k0 = kt * 64;
#pragma unroll
    for (int j = 0; j < A_PER_WAVE; ++j)
      buf_load_lds_16(rA, st + (wave + T::NW * j) * 1024, real ? (int)(a_off[j] + k0) : 0x7ffffff0);
#pragma unroll
    for (int j = 0; j < W_PER_WAVE; ++j)
      buf_load_lds_16(rW, st + BM * 64 + (wave + T::NW * j) * 1024, real ? (int)(w_off[j] + k0) : 0x7ffffff0);
  };

  const int fr = lane & 31, fh = lane >> 5;
  const int a_row0 = wm * T::WM + fr, w_row0 = wn * T::WN + fr;
  const int G = p.K / 256;                                // k-tile groups
  const __amdgpu_buffer_rsrc_t rSA = make_rsrc(p.A_scale, (int)(8L * G * p.lds_a));
  const __amdgpu_buffer_rsrc_t rSW = make_rsrc(p.W_scale, (int)(8L * G * p.lds_w));
  const int sa_off = (fh * (int)p.lds_a + m0 + a_row0) * 4, sw_off = (fh * (int)p.lds_w + n0 + w_row0) * 4;
  uint32_t sa[T::TM], sw[T::TN], sa_n[T::TM], sw_n[T::TN];
  // group g's words; group G's are past the range: zeros, never used
  auto load_scales = [&](int g) {
    const int ga = sa_off + g * 8 * (int)p.lds_a, gw = sw_off + g * 8 * (int)p.lds_w;
#pragma unroll
    for (int i = 0; i < T::TM; ++i) sa_n[i] = __builtin_amdgcn_raw_buffer_load_b32(rSA, ga + 128 * i, 0, 0);
#pragma unroll
    for (int j = 0; j < T::TN; ++j) sw_n[j] = __builtin_amdgcn_raw_buffer_load_b32(rSW, gw + 128 * j, 0, 0);
  };

  floatx16 acc[T::TM][T::TN];
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  int8v fa[T::TM], fw[T::TN];                             // the fragments of the next k-tile
  auto frag = [](const uint8_t* st, int r, int h) {
    const int4v lo = *reinterpret_cast<const int4v*>(st + swzb(r, h));
    const int4v hi = *reinterpret_cast<const int4v*>(st + swzb(r, 2 + h));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // memory phase: copies of k-tile `kt_issue` into `fill`, then the fragments of the k-tile in `cur`
  // (and, with SC, the next group's scale words)
  auto mem = [&](auto sc_c, const uint8_t* cur, int kt_issue, uint8_t* fill, int g_next) {
    issue(kt_issue, fill);
    if constexpr (decltype(sc_c)::value) load_scales(g_next);
#pragma unroll
    for (int i = 0; i < T::TM; ++i) fa[i] = frag(cur, a_row0 + i * 32, fh);
#pragma unroll
    for (int j = 0; j < T::TN; ++j) fw[j] = frag(cur + BM * 64, w_row0 + j * 32, fh);
  };
  // compute phase of k-tile 4g + Q
  auto compute = [&](auto q_c) {
    constexpr int Q = decltype(q_c)::value;
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
      for (int j = 0; j < T::TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw[j], fa[i], acc[i][j], 0, 0, Q, (int)sw[j], Q,
                                                                    (int)sa[i]);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // N = this wave's vector-memory operations of its two most recent memory phases
  auto bar = [&](auto n_c) {
    __builtin_amdgcn_sched_barrier(0);
    copy_barrier64<decltype(n_c)::value>();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto use_scales = [&]() {
#pragma unroll
    for (int i = 0; i < T::TM; ++i) sa[i] = sa_n[i];
#pragma unroll
    for (int j = 0; j < T::TN; ++j) sw[j] = sw_n[j];
  };
  using N8 = std::integral_constant<int, 2 * LOADS>;
  using N14 = std::integral_constant<int, 2 * LOADS + NSC>;
  using Q0 = std::integral_constant<int, 0>;
  using Q1 = std::integral_constant<int, 1>;
  using Q2 = std::integral_constant<int, 2>;
  using Q3 = std::integral_constant<int, 3>;
  using SC = std::true_type;
  using NS = std::false_type;

  load_scales(0);                                         // before the copies: complete at the first barrier
  issue(0, st0);
  issue(1, st1);
  issue(2, st2);
  bar(N8{});                                              // group 0's words and k-tile 0 have landed
  if (wm == 0) {
    mem(NS{}, st0, 3, st3, 0);                            // phase -1: load k-tile 0
    bar(N8{});
    for (int t = 0; t < KT; t += 4) {                     // k-tiles t .. t + 3 (stages 0 .. 3)
      use_scales();
      compute(Q0{});                                      // phase 2t
      bar(N8{});
      mem(SC{}, st1, t + 4, st0, t / 4 + 1);              // phase 2t + 1: load t + 1, copy t + 4, next words
      bar(N14{});
      compute(Q1{});
      bar(N14{});
      mem(NS{}, st2, t + 5, st1, 0);
      bar(N14{});
      compute(Q2{});
      bar(N14{});
      mem(NS{}, st3, t + 6, st2, 0);
      bar(N8{});
      compute(Q3{});                                      // k-tile t + 3
      bar(N8{});
      if (t + 4 < KT) {
        mem(NS{}, st0, t + 7, st3, 0);
        bar(N8{});
      }
    }
  } else {
    bar(N8{});                                            // phase -1: nothing to do
    for (int t = 0; t < KT; t += 4) {
      use_scales();
      mem(NS{}, st0, t + 3, st3, 0);                      // phase 2t: load t, copy t + 3
      bar(N8{});
      compute(Q0{});                                      // phase 2t + 1
      bar(N8{});
      mem(SC{}, st1, t + 4, st0, t / 4 + 1);
      bar(N14{});
      compute(Q1{});
      bar(N14{});
      mem(NS{}, st2, t + 5, st1, 0);
      bar(N14{});
      compute(Q2{});
      bar(N14{});
      mem(NS{}, st3, t + 6, st2, 0);
      bar(N8{});
      compute(Q3{});                                      // k-tile t + 3
      if (t + 4 < KT) bar(N8{});
    }
  }
  // the look-ahead copies (zeros into unused stages) land before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(0x0F70);                     // vmcnt(0)
  store_tile<T, EPI>(p, acc, m0, n0, wm, wn, fr, fh);
}

template <int BM, int BN, int WAVES_M, int WAVES_N>
hipError_t launch_tile(const GemmArgs& a, int epi, hipStream_t stream) {
  const int nM = (a.M + BM - 1) / BM, nN = a.N / BN;
  dim3 grid(nM * nN), block(64 * WAVES_M * WAVES_N);
#define MOSS_GEMM_LAUNCH(E) \
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WAVES_M, WAVES_N, E>), grid, block, 0, stream, a)
  switch (epi) {
    case EPI_BF16: MOSS_GEMM_LAUNCH(EPI_BF16); break;
    case EPI_QKV_ROPE: MOSS_GEMM_LAUNCH(EPI_QKV_ROPE); break;
    case EPI_GATED_RES: MOSS_GEMM_LAUNCH(EPI_GATED_RES); break;
    case EPI_SWIGLU: MOSS_GEMM_LAUNCH(EPI_SWIGLU); break;
    case EPI_F32: MOSS_GEMM_LAUNCH(EPI_F32); break;
    case EPI_F32_UNPATCH:
      // the output projection has N = C*4 = 128: only the 128-wide tile is ever used for it
      if constexpr (BN == 128) {
        MOSS_GEMM_LAUNCH(EPI_F32_UNPATCH);
        break;
      } else {
        return hipErrorInvalidValue;
      }
    default: return hipErrorInvalidValue;
  }
#undef MOSS_GEMM_LAUNCH
  return hipGetLastError();
}

__global__ void interleave_gate_up_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, int F, int D) {
  const long row = blockIdx.x;               // destination row
  const int grp = (int)(row / 64), w = (int)(row % 64);
  const long srow = (w < 32) ? (long)grp * 32 + w : (long)F + (long)grp * 32 + (w - 32);
  const uint4* s = reinterpret_cast<const uint4*>(src + srow * D);
  uint4* d = reinterpret_cast<uint4*>(dst + row * D);
  for (int i = threadIdx.x; i < D / 8; i += blockDim.x) d[i] = s[i];
}

}  // namespace

static hipError_t launch_tile_pp(const GemmArgs& a, int epi, hipStream_t stream) {
  const int nM = (a.M + 255) / 256, nN = a.N / 256;
  dim3 grid(nM * nN), block(512);
#define MOSS_GEMM_LAUNCH(E) hipLaunchKernelGGL((gemm_bf16_pp_kernel<E>), grid, block, 0, stream, a)
  switch (epi) {
    case EPI_BF16: MOSS_GEMM_LAUNCH(EPI_BF16); break;
    case EPI_QKV_ROPE: MOSS_GEMM_LAUNCH(EPI_QKV_ROPE); break;
    case EPI_GATED_RES: MOSS_GEMM_LAUNCH(EPI_GATED_RES); break;
    case EPI_SWIGLU: MOSS_GEMM_LAUNCH(EPI_SWIGLU); break;
    case EPI_F32: MOSS_GEMM_LAUNCH(EPI_F32); break;
    default: return hipErrorInvalidValue;
  }
#undef MOSS_GEMM_LAUNCH
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, int epi, hipStream_t stream) {
  if (a.M <= 0) return hipSuccess;
  if (a.K % BK != 0 || a.lda % 8 != 0 || a.ldw % 8 != 0) return hipErrorInvalidValue;
  if ((long)a.M * a.lda >= (1L << 31) || (long)a.N * a.ldw >= (1L << 31)) return hipErrorInvalidValue;
  // SwiGLU pairs feature blocks inside a wave: the wave's feature width must hold whole 64-row groups.
  const bool big_n = (a.N % 256 == 0);
  const long tiles256 = (long)((a.M + 255) / 256) * (a.N / 256);
  const bool fits32 = 2L * a.M * a.lda < (1L << 31) && 2L * a.N * a.ldw < (1L << 31);   // buffer byte offsets
  // 256 x 256 tiles from half a round of the chip on: one batch-1 out / down projection (204 tiles)
  // runs 25-30 % faster on them than as 816 tiles of 128 x 128 (measured)
  if (big_n && epi != EPI_F32_UNPATCH && a.M > 1024 && tiles256 >= 128) {
    if (fits32 && a.K % (4 * BK2) == 0) return launch_tile_pp(a, epi, stream);
    return launch_tile<256, 256, 2, 4>(a, epi, stream);
  }
  if (a.N % 128 == 0) return launch_tile<128, 128, 2, 2>(a, epi, stream);
  return hipErrorInvalidValue;
}

static hipError_t launch_mxfp8_pp(const GemmArgs& a, int epi, hipStream_t stream) {
  const int nM = (a.M + 255) / 256, nN = a.N / 256;
  dim3 grid(nM * nN), block(512);
#define MOSS_GEMM_LAUNCH(E) hipLaunchKernelGGL((gemm_mxfp8_pp_kernel<E>), grid, block, 0, stream, a)
  switch (epi) {
    case EPI_BF16: MOSS_GEMM_LAUNCH(EPI_BF16); break;
    case EPI_QKV_ROPE: MOSS_GEMM_LAUNCH(EPI_QKV_ROPE); break;
    case EPI_GATED_RES: MOSS_GEMM_LAUNCH(EPI_GATED_RES); break;
    case EPI_SWIGLU: MOSS_GEMM_LAUNCH(EPI_SWIGLU); break;
    case EPI_SWIGLU_MX: MOSS_GEMM_LAUNCH(EPI_SWIGLU_MX); break;
    case EPI_F32: MOSS_GEMM_LAUNCH(EPI_F32); break;
    default: return hipErrorInvalidValue;
  }
#undef MOSS_GEMM_LAUNCH
  return hipGetLastError();
}

hipError_t launch_gemm_mxfp8(const GemmArgs& a, int epi, hipStream_t stream) {
  if (a.M <= 0) return hipSuccess;
  if ((reinterpret_cast<uintptr_t>(a.A) & 15) || (reinterpret_cast<uintptr_t>(a.W) & 15) ||
      (reinterpret_cast<uintptr_t>(a.A_scale) & 3) || (reinterpret_cast<uintptr_t>(a.W_scale) & 3))
    return hipErrorInvalidValue;
  if (a.N % 256 != 0 || a.K % 256 != 0 || a.lda % 16 != 0 || a.ldw % 16 != 0 || !a.A_scale || !a.W_scale ||
      a.lds_a % 256 != 0 || a.lds_a < (a.M + 255) / 256 * 256 || a.lds_w % 256 != 0 || a.lds_w < a.N)
    return hipErrorInvalidValue;
  if ((long)a.M * a.lda >= (1L << 31) || (long)a.N * a.ldw >= (1L << 31) ||
      2L * a.K * a.lds_a / 64 >= (1L << 31) || 2L * a.K * a.lds_w / 64 >= (1L << 31))
    return hipErrorInvalidValue;                          // buffer byte offsets must fit 31 bits
  if (epi == EPI_SWIGLU_MX && (!a.out_scale || a.lds_out < a.M || a.ldo % 4 != 0)) return hipErrorInvalidValue;
  return launch_mxfp8_pp(a, epi, stream);
}

hipError_t launch_interleave_gate_up(const uint16_t* src, uint16_t* dst, int F, int D, hipStream_t stream) {
  if (F % 32 != 0 || D % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(interleave_gate_up_kernel, dim3(2 * F), dim3(256), 0, stream, src, dst, F, D);
  return hipGetLastError();
}

}  // namespace moss
