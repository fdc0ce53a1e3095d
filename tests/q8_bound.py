"""The 8-bit attention's error bound against exact softmax attention on its quantized operands, shared by
the GPU test (tests/test_gpu_attention_q8.py) and its CPU pins (tests/test_q8_bound_cpu.py). Test
infrastructure: calls the oracle's quantizers only."""
import numpy as np

import oracle as O


def exact_on_quantized(q, k, v):
    """Exact softmax attention (fp64) on the reading's dequantized operands -- q INT8 per token, k INT8
    per 64-key block, v E4M3 per channel -- and the per-element bound of a kernel that rounds every
    probability p_i to E4M3 on the 224 scale and divides by the sum of the rounded values. With
    p~_i = p_i + d_i: o - o_ref = sum_i d_i (v_i - o_ref) / sum_i p~_i. E4M3 has 3 fraction bits, so
    |d_i| <= 2^-4 p_i for normal codes and <= d0 = 2^-10 / 224 (half the smallest subnormal step) below;
    the row's largest probability is at least 1 against any reference max at most the row max, so
    sum p >= 1 and sum p~ >= sum p (1 - 2^-4 - e - S d0). Hence
        |o_d - o_ref,d| <= sum_i ((2^-4 + e) w_i + d0) |v_i,d - o_ref,d| / (1 - 2^-4 - e - S d0)
    with w the exact softmax weights; e covers the fp32 score and exp2 arithmetic: 1e-4, plus the error
    of the kernel's exp2 argument, which it takes from the INT8 accumulator read as the float
    1.5 * 2^23 + s (s the integer score) times the score unit f, shifted by a per-tile constant rounded
    once: at most 2^-24 (1.5 * 2^23 f + |m|) log2 units, m the reference (at most the largest score
    plus log2 224 away from 0), so a relative error of ln 2 times that in each probability."""
    S = k.shape[0]
    qc, qa = O.q8_quantize_q(q)
    kc, ka = O.q8_quantize_k(k)
    vc, va = O.fp8_quantize_v(v)
    qh = qc * (qa / 127.0)[:, None]
    kh = kc * np.repeat(ka / 127.0, O.Q8_KEY_BLOCK)[:S, None]
    vh = vc * (va / O.E4M3_MAX)[None, :]
    sc = qh @ kh.T / np.sqrt(128.0)
    log2e = 1.0 / np.log(2.0)
    f_max = qa.max() * ka.max() / 127.0 ** 2 / np.sqrt(128.0) * log2e
    m_max = np.abs(sc).max() * log2e + np.log2(O.Q8_P_SCALE) + 1.0
    e = 1e-4 + np.log(2.0) * 2.0 ** -24 * (1.5 * 2.0 ** 23 * f_max + m_max)
    sc -= sc.max(axis=1, keepdims=True)
    w = np.exp(sc)
    w /= w.sum(axis=1, keepdims=True)
    o = w @ vh
    d0 = 2.0 ** -10 / O.Q8_P_SCALE
    den = 1.0 - 2.0 ** -4 - e - S * d0
    bound = np.empty_like(o)
    for r in range(o.shape[0]):                    # per query row: [S, 128] at a time
        dev = np.abs(vh - o[r][None, :])
        bound[r] = (((2.0 ** -4 + e) * w[r][:, None] + d0) * dev).sum(axis=0) / den
    return o, bound
