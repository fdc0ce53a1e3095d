"""CPU oracle of the MOSS-Image DiT denoising step -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this package. It is independent of the HIP path: it imports nothing from
``diffusion_transformer_text_amd`` and shares no kernels, tables, constants or helpers with it.

Parity status of each function (pins in tests/test_oracle_pins.py):
  bf16_round, from_bf16_bits  pinned: torch's bfloat16 cast (a library routine), hand bit patterns
  sigmas, slg_active          pinned: closed-form hand fractions, endpoints, "first step at full CFG"
  time_features               pinned: hand values (sigma 0, t = 500 at k = 0 and k = 64)
  modulation                  pinned: zero weights, chunk order via scalar brute force
  patchify, unpatchify        pinned: hand-placed elements, mutual inverse, 4,096 tokens at 1024^2
  layernorm, ln_modulate      pinned: statistics.pstdev (library), constant and +-a rows
  rope_angles, apply_rope,    pinned: hand angles (1 rad, 0.02 rad), norm preservation, identity at
  rope_rows                   (0, 0), relative-position invariance, row/column halves
  attention                   pinned: scalar brute force, S = 1 -> V, equal keys -> mean(V), a
                              hand 3:1 softmax split that fixes the 1/sqrt(d) scale
  block                       pinned: scalar brute-force block on a tiny shape, gate = 0 identity,
                              taps consistency
  embed, final_layer,         pinned: all-gates-zero forward equals embed -> final closed form,
  forward                     skip == zeroed gate rows (bitwise), per-sample independence
  cfg_combine, euler_step,    pinned: CFG identities, telescoping under constant v, point-mass field
  sample_step                 lands exactly on x*, cfg = 1 runs no negative pass
  text_refine                 pinned: projection vs a scalar brute force (blocks made identities by
                              zero branch weights), permutation equivariance (no RoPE, no mask on
                              text rows), equal rows stay equal
  first_block_change,         pinned: hand values of the change measure; threshold 0 gives the plain
  forward_cached,             forward/step bit for bit; with blocks 1.. made identities (zero gates)
  sample_step_cached          a reused call equals the full call bit for bit; step 0 and a new row
                              plan restart the cache
  e4m3_round, mx_quantize,    pinned: E4M3 rounding against a brute force over all 256 codes decoded
  mx_dequantize               from the bit layout (ties to even, saturation); hand MX blocks (scale
                              exponent, saturation, zero block); exact round trip of representable
                              values; the per-element error bound
  negative_pass_runs          pinned: hand table of the truncation boundary (X * steps, steps from 0)
  guidance_combine            pinned: hand values of each term, v_s = v_c leaves the two-pass result,
                              linearity in slg_scale
  sample_step (three-pass,    pinned: the third row equals the conditional forward with the skipped
  truncation)                 blocks' gate rows zeroed (bitwise); slg 0 / empty skip list / outside
                              the window give the two-pass step bitwise; a truncated step equals the
                              CFG-1 step bitwise
  int8_codes, q8_quantize_q,  pinned: hand codes (half-even ties, the amax row at +-127, zero rows),
  q8_quantize_k,              per-block amax of K blocks of different magnitude, E4M3 codes of V
  fp8_quantize_v              channels (amax channel at +-448)
  attention_q8                pinned: with exact probabilities it equals the exact softmax of the
                              dequantized operands (the pinned attention above), ragged last block;
                              V constant over keys and a single key give V exactly (convex weights);
                              a dominant key selects its V row; within a few percent of the exact
                              attention on random inputs; the lazy reference max against a hand
                              schedule of three blocks (no move at +0.5 log2, a move at +1.5)
"""
from .moss_oracle import *  # noqa: F401,F403
from .moss_oracle import (Config, attention, bf16_round, block, cfg_combine, embed, euler_step,  # noqa
                          final_layer, forward, from_bf16_bits, guidance_combine, layernorm, ln_modulate,
                          modulation, negative_pass_runs, text_refine, StepCache,
                          first_block_change, forward_cached, sample_step_cached,
                          e4m3_round, mx_quantize, mx_dequantize, E4M3_MAX, projection,
                          attention_q8, q8_quantize_q, q8_quantize_k, fp8_quantize_v, int8_codes,
                          Q8_KEY_BLOCK, Q8_P_SCALE,
                          patchify, rope_angles, apply_rope, rope_rows, sample_step, sigmas, silu,
                          slg_active, time_features, unpatchify, weights_to_f64)
