// Host-only checks of the library's argument validation, sampling-step row plan and workspace layout,
// built with g++ under -fsanitize=address,undefined together with csrc/host_plan.cpp (no GPU, no HIP).
//
// 1. Validation on edge-case and randomised arguments: every call returns a status and a message
//    without touching memory it does not own (the sanitizers abort otherwise).
// 2. For every accepted sampling step over a grid of shapes and guidance settings, and for every
//    accepted forward batch: the workspace layout of the call's row count holds what the kernels of
//    that call write -- sizes written out here from the kernels' outputs (the residual stream, LN
//    output, qkv, attention output, SwiGLU output, patch tokens, modulation, time features, one fp32
//    velocity per row, the FP8 tier's codes and scale words, attention scratch), not from the layout
//    code -- with every region inside the workspace and no two regions overlapping. A workspace whose
//    velocity region held fewer rows than the step runs is the kind of bug this catches.
// Prints "ok <cases>" and exits 0, or prints the failures and exits 1.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "host_plan.h"
#include "moss_dit_ops.h"

using namespace moss;

static long g_fail = 0, g_cases = 0;
#define CHECK(cond, ...)                                        \
  do {                                                          \
    if (!(cond)) {                                              \
      if (++g_fail <= 20) {                                     \
        std::printf("FAIL %s:%d: ", __FILE__, __LINE__);        \
        std::printf(__VA_ARGS__);                               \
        std::printf("\n");                                      \
      }                                                         \
    }                                                           \
  } while (0)

struct Region {
  const char* name;
  size_t off, need;
};

// The regions one call writes, with their sizes from the kernels' outputs.
static void check_layout(const moss_dit_config& k, int B, int S, int N, long lat, long slots) {
  ++g_cases;
  const WsLayout L = ws_layout(k, B, S, N, lat, slots);
  const size_t M = (size_t)B * S, D = k.hidden, F = k.ffn_hidden, P = (size_t)k.latent_channels * 4;
  const size_t mod_rows = (size_t)k.num_layers * 6 * D + 2 * D;
  std::vector<Region> r = {
      {"x (residual, bf16 [M, D])", L.x, M * D * 2},
      {"a (LN output, bf16 [M, D])", L.a, M * D * 2},
      {"qkv (bf16 [M, 3D])", L.qkv, M * 3 * D * 2},
      {"o (attention output, bf16 [M, D])", L.o, M * D * 2},
      {"h (SwiGLU output, bf16 [M, F])", L.h, M * F * 2},
      {"tokens (patches, bf16 [B N, C p p])", L.tokens, (size_t)B * N * P * 2},
      {"mod (bf16 [B, mod_rows])", L.mod, (size_t)B * mod_rows * 2},
      {"u (time features, fp32 [B, temb])", L.u, (size_t)B * k.temb_dim * 4},
      {"vel (fp32 [B, C, h, w], one per row)", L.vel, (size_t)B * lat * 4},
  };
  if (k.gemm_precision == 1) {
    const size_t Kmax = D > F ? D : F, ld = (M + 255) / 256 * 256;
    CHECK(L.lds8 >= (long)M && L.lds8 % 256 == 0, "lds8 %ld for M %zu", L.lds8, M);
    r.push_back({"q8 (codes [M, max(D, F)])", L.q8, M * Kmax});
    r.push_back({"s8 (scale words)", L.s8, Kmax / 128 * ld * 4});
    r.push_back({"q8h (codes of h [M, F])", L.q8h, M * F});
    r.push_back({"s8h (scale words of h)", L.s8h, F / 128 * ld * 4});
  }
  const AttnSplitPlan sp = attention_split_plan(B, S, k.num_heads, slots);
  const size_t split_rows = (size_t)sp.n_split * sp.parts * kAttnBQ;
  CHECK((long)sp.n_full + (long)sp.n_split == (long)((S + kAttnBQ - 1) / kAttnBQ) * k.num_heads * B,
        "split plan loses query tiles (B %d S %d)", B, S);
  CHECK(sp.n_split == 0 || (sp.parts >= 2 && (long)sp.n_split * sp.parts <= slots), "split plan oversubscribes");
  if (split_rows) r.push_back({"attention split partials", L.attn_split, split_rows * (kHeadDim + 2) * 4});
  if (k.attention_mode == 1) {
    const size_t nblk = (S + 63) / 64, H = k.num_heads;
    // q and k codes, V^T codes, per-token q scale, per-block k scale, per-channel v scale, block maxima
    const size_t need = M * H * 128 * 2 + (size_t)B * H * 128 * nblk * 64 + M * H * 4 + (size_t)B * H * nblk * 4 +
                        (size_t)B * H * 128 * 4 + (size_t)B * H * nblk * 128 * 4;
    r.push_back({"8-bit attention workspace", L.attn8, need});
  }
  for (size_t i = 0; i < r.size(); ++i) {
    CHECK(r[i].off != kNoRegion, "%s missing (B %d S %d)", r[i].name, B, S);
    if (r[i].off == kNoRegion) continue;
    CHECK(r[i].off % 256 == 0, "%s misaligned", r[i].name);
    CHECK(r[i].off + r[i].need <= L.total, "%s ends past the workspace (B %d S %d N %d: %zu + %zu > %zu)", r[i].name,
          B, S, N, r[i].off, r[i].need, L.total);
    for (size_t j = 0; j < i; ++j) {
      if (r[j].off == kNoRegion) continue;
      const bool disjoint = r[i].off + r[i].need <= r[j].off || r[j].off + r[j].need <= r[i].off;
      CHECK(disjoint, "%s overlaps %s (B %d S %d)", r[i].name, r[j].name, B, S);
    }
  }
}

static moss_dit_config cfg_with(int precision, int attention_mode) {
  moss_dit_config c;
  moss_dit_config_init(&c, sizeof c);
  c.gemm_precision = precision;
  c.attention_mode = attention_mode;
  return c;
}

int main() {
  std::mt19937_64 rng(12345);
  // ---- 1. validation fuzz ----
  {
    const moss_dit_config base = cfg_with(0, 0);
    std::vector<float> sig(2049, 0.5f);
    int32_t skips[70];
    for (int i = 0; i < 70; ++i) skips[i] = i - 3;
    char msg[96];
    for (int it = 0; it < 20000; ++it) {
      moss_dit_config c = base;
      if (rng() % 8 == 0) c.hidden = (int)(rng() % 9000) - 100;
      if (rng() % 8 == 0) c.num_layers = (int)(rng() % 80) - 5;
      if (rng() % 16 == 0) c.struct_size = (uint32_t)(rng() % 200);
      if (rng() % 16 == 0) c.qk_norm = 1;
      moss_step_args a;
      moss_step_args_init(&a, sizeof a);
      float x = 0.f, t = 0.f;
      a.x = &x;
      a.text_cond = &t;
      a.text_uncond = (rng() % 4) ? &t : nullptr;
      a.latent_h = (int)(rng() % 1200) - 100;
      a.latent_w = (int)(rng() % 1200) - 100;
      a.text_len = (int)(rng() % 5000) - 10;
      a.num_steps = (int)(rng() % 2060) - 10;
      a.step = (int)(rng() % 2100) - 10;
      a.cfg_scale = (float)((double)(rng() % 1000) / 100.0 - 1.0);
      a.slg_scale = (rng() % 4 == 0) ? -1.f : (float)(rng() % 5);
      a.cfg_truncation = (float)((double)(rng() % 300) / 200.0 - 0.2);
      a.sigmas = (a.num_steps >= 0 && a.num_steps < 2048) ? sig.data() : nullptr;
      a.n_skip = (int)(rng() % 80) - 5;
      a.uncond_skip_layers = (a.n_skip >= 0 && a.n_skip <= 67) ? skips + (rng() % 3) : nullptr;
      if (rng() % 32 == 0) a.struct_size = 4;
      const int st = moss_validate_step_args(&c, &a, msg, (int32_t)(rng() % sizeof msg));
      CHECK(st >= 0 && st <= 5, "status %d", st);
      if (st == 0) {
        const StepPlan p = step_plan(&a);
        CHECK(p.rows >= 1 && p.rows <= 3, "rows %d", p.rows);
        CHECK(!(p.neg && a.text_uncond == nullptr), "negative pass without negative text");
      }
      moss_forward_args f;
      moss_forward_args_init(&f, sizeof f);
      uint64_t masks[9];
      float sg[9];
      for (int i = 0; i < 9; ++i) {
        masks[i] = rng() % 4 == 0 ? rng() : 0;
        sg[i] = (float)((double)(rng() % 300) / 200.0 - 0.2);
      }
      f.batch = (int)(rng() % 12) - 2;
      f.latent_h = a.latent_h;
      f.latent_w = a.latent_w;
      f.text_len = a.text_len;
      f.latents = &x;
      f.text = &t;
      f.velocity = &x;
      f.sigma = (f.batch >= 0 && f.batch <= 9) ? sg : nullptr;
      f.skip_mask = (rng() % 2 && f.batch >= 0 && f.batch <= 9) ? masks : nullptr;
      const int fs = moss_validate_forward_args(&c, &f, nullptr, 0);
      CHECK(fs >= 0 && fs <= 5, "status %d", fs);
      ++g_cases;
    }
    CHECK(moss_validate_step_args(nullptr, nullptr, msg, sizeof msg) != 0, "NULL config accepted");
  }

  // ---- 2. layouts of every accepted step and forward ----
  const int sides[] = {2, 16, 30, 64, 96, 128, 130, 192, 256, 320, 352, 384, 402, 512};
  const int texts[] = {1, 7, 64, 256, 1000, 4096};
  const long slot_counts[] = {2 * 256, 2 * 304, 2 * 80, 64};
  int32_t skip22[2] = {22, 3};
  std::vector<float> sig(51);
  moss_sigmas(50, 5.f, sig.data());
  for (int prec = 0; prec <= 1; ++prec)
    for (int am = 0; am <= 1; ++am) {
      const moss_dit_config c = cfg_with(prec, am);
      for (int lh : sides)
        for (int lw : sides)
          for (int T : texts) {
            moss_step_args a;
            moss_step_args_init(&a, sizeof a);
            float x = 0.f, t = 0.f;
            a.x = &x;
            a.text_cond = a.text_uncond = &t;
            a.sigmas = sig.data();
            a.latent_h = lh;
            a.latent_w = lw;
            a.text_len = T;
            a.uncond_skip_layers = skip22;
            const float cfgs[] = {1.f, 3.f};
            const float slgs[] = {0.f, 2.5f};
            const float truncs[] = {1.f, 0.5f};
            const int steps[] = {0, 1, 30};
            const int nskips[] = {0, 1, 2};
            for (float cf : cfgs)
              for (float sl : slgs)
                for (float tr : truncs)
                  for (int stp : steps)
                    for (int ns : nskips) {
                      a.cfg_scale = cf;
                      a.slg_scale = sl;
                      a.cfg_truncation = tr;
                      a.step = stp;
                      a.n_skip = ns;
                      std::string m;
                      if (validate_step(&c, &a, m) != 0) continue;
                      const StepPlan p = step_plan(&a);
                      const int N = (lh / 2) * (lw / 2), S = T + N;
                      const long lat = 32L * lh * lw;
                      const long slots = slot_counts[(lh + lw + T) % 4];
                      check_layout(c, p.rows, S, N, lat, slots);
                    }
            // forwards of 1..8 samples at this shape
            for (int B = 1; B <= kMaxBatch; ++B) {
              moss_forward_args f;
              moss_forward_args_init(&f, sizeof f);
              float sg[kMaxBatch];
              for (int i = 0; i < kMaxBatch; ++i) sg[i] = 0.5f;
              f.batch = B;
              f.latent_h = lh;
              f.latent_w = lw;
              f.text_len = T;
              f.latents = f.text = &x;
              f.velocity = &x;
              f.sigma = sg;
              std::string m;
              if (validate_forward(&c, &f, m) != 0) continue;
              const int N = (lh / 2) * (lw / 2);
              check_layout(c, B, T + N, N, 32L * lh * lw, slot_counts[B % 4]);
            }
          }
    }
  if (g_fail) {
    std::printf("%ld failures in %ld cases\n", g_fail, g_cases);
    return 1;
  }
  std::printf("ok %ld\n", g_cases);
  return 0;
}
