"""Decode-attention parity cases and the tolerance that holds
kivi_cache_attend to the oracle's exact attention (OracleCache.attend_exact).

The kernel and the oracle compute the same function (include/kivi.h,
kivi_cache_attend: quantized tokens enter as code * scale + zero, never
rounded to 16 bits); what separates them is fp32 rounding only.  With
e = 2^-24 (fp32), u the unit roundoff of the output type (2^-11 fp16,
2^-8 bf16), L = 2^bits - 1, and per (bh, query head j, token t, channel d):

 * score error.  The kernel forms sum_d q_d K_td as
   sum_d (q_d scale_d) code_td + sum_d q_d zero_d (matrix cores or vector
   units) or as sum_d q_d RN(RN(code scale) + zero); in both, every term is
   bounded by T_t = sum_d |q_d| (code_td |scale_d| + |zero_d|) (by
   sum_d |q_d| |K_td| for exact ring tokens), and the rounding of the
   products, the hi + lo f16 split (2^-22 relative), a sum of at most 2D + 1
   terms and the bias sum make
       eps_t <= (2D + 24) e T_t + D L 2^-37 P_g
   where P_g = max_d |q_d scale_gd| of the token's key group bounds the
   absolute error of an operand part that falls below f16's normal range
   (2^-24 of the power-of-two scaled operand, which is < 2^14);
 * weight error.  The weight of token t, exp(s_t - M) with
   s_t = sm * score, carries a relative error of at most
       eta_t = sm eps_t + e (|s_t| + 4 (M - s_t)) + 2^-19
   (the fp32 product with sm, the subtraction of the chunk maximum, the
   log2(e) scaling inside exp for the token and for its chunk in the merge,
   and the exp instructions themselves); the same rounded weights feed the
   numerator and the denominator, so to first order the output moves by
       sum_t p_t eta_t |V_td - o_d|;
 * value sums.  Every partial sum of the numerator is a sum of at most
   256 + n_chunks + 40 terms (two f16 parts per token in the matrix-core
   sums of a chunk, the zero-point and ring sums, the merge), each bounded by
   W_td = code_td |vscale_t| + |vzero_t| (|V_td| for ring tokens):
       (296 + n_chunks) e sum_t p_t W_td,
   plus the f16 split's absolute part, n_chunks L 2^-30 vsmax (vsmax the
   largest value scale of the bh);
 * the denominator, a sum of positive terms of depth < n_chunks + 160:
   (n_chunks + 160) e |o_d|;
 * the output: one division and the rounding to the 16-bit type,
   u |o_d| + the half spacing of 16-bit subnormals.
The bound is twice the sum of the first-order terms, plus the output
rounding.  tests/test_attend_bound.py checks on the CPU that planted bugs in
the oracle (a dropped key group, another group's params, no zero points,
sm_scale * 1.01, dropped ring tokens, codes ignored) exceed it in every
case below.
"""
import numpy as np

FP16, BF16 = 0, 1
E32 = 2.0 ** -24

CASES = [
    # (BH, D, R, G_k, G_v, bits, dtype, n_q, appends)
    (4, 128, 32, 32, 32, 2, FP16, 3, [300]),
    (3, 64, 32, 32, 32, 2, FP16, 4, [200, 1, 1, 57]),
    (2, 128, 16, 16, 128, 4, BF16, 7, [129, 64, 2]),
    (5, 128, 32, 32, 32, 2, FP16, 1, [20]),          # nothing quantized yet
    (2, 64, 0, 8, 8, 8, BF16, 2, [256]),             # everything quantized
    (3, 128, 5, 32, 64, 1, FP16, 8, [1000, 3]),
    (2, 128, 32, 32, 32, 2, FP16, 4, [1]),           # a single token
    # chunks of 128 fully quantized tokens take the matrix-core kernel
    (3, 128, 32, 16, 16, 4, BF16, 6, [700]),
    (2, 64, 32, 32, 64, 2, FP16, 2, [500, 9]),
    (2, 64, 16, 16, 32, 2, BF16, 3, [290]),
    (1, 128, 0, 32, 128, 2, FP16, 5, [512]),         # every chunk full
    (2, 64, 32, 32, 32, 4, FP16, 4, [400]),          # 4-bit value code pairs, D = 64
    (2, 128, 32, 32, 32, 1, BF16, 2, [600]),         # 1-bit value code pairs
]

# a 2059-token prompt in prefill chunks of 2048 plus 40 one-token decode
# appends, GQA with 4 query heads per KV head: 17 chunks merged
LONG_CASE = (8, 128, 32, 32, 32, 2, FP16, 4,
             [2048, 11] + [1] * 40)


def case_id(c):
    return "x".join(map(str, c[:8])) + "_" + (
        "-".join(map(str, c[8])) if len(c[8]) <= 6 else f"{len(c[8])}appends")


def tokens(seed, BH, n, D, dtype, scale=1.0):
    """Seeded 16-bit tokens [BH, n, D] with a few large channels (keys and
    values of the decode-attention cases)."""
    r = np.random.default_rng(seed)
    x = (r.standard_normal((BH, n, D)) * scale).astype(np.float32)
    x[:, :, r.choice(D, size=max(1, D // 32), replace=False)] *= 8.0
    if dtype == FP16:
        return x.astype(np.float16).view(np.uint16)
    import torch
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16)
    return t.numpy().view(np.uint16)


def case_inputs(case, seeds=(41, 42, 43)):
    """Keys and values of every append, and the queries, of one case."""
    BH, D, R, Gk, Gv, bits, dtype, n_q, appends = case
    S_max = sum(appends) + 8
    k = tokens(seeds[0], BH, S_max, D, dtype)
    v = tokens(seeds[1], BH, S_max, D, dtype)
    q = tokens(seeds[2], BH, n_q, D, dtype, scale=0.5)
    return k, v, q, S_max


def oracle_cache(O, case, k, v, S_max):
    BH, D, R, Gk, Gv, bits, dtype, n_q, appends = case
    oc = O.cache(BH, D, S_max, R, Gk, Gv, bits, dtype)
    t = 0
    for n in appends:
        oc.append(np.ascontiguousarray(k[:, t:t + n]),
                  np.ascontiguousarray(v[:, t:t + n]))
        t += n
    return oc


def unit_roundoff(dtype):
    return 2.0 ** -11 if dtype == FP16 else 2.0 ** -8


def subnormal_half_spacing(dtype):
    return 2.0 ** -25 if dtype == FP16 else 2.0 ** -134


def attend_bound(O, oc, q, sm):
    """Per-element bound [BH, n_q, D] on |kivi_cache_attend -
    oc.attend_exact(q, sm)| (the derivation is in the module docstring);
    returns (bound, exact output)."""
    c = oc.c
    dt, BH, D, Q, T = c.dtype, c.BH, c.D, c.Q, c.T
    Gk, Gv, bits = c.G_k, c.G_v, c.bits
    L = 2 ** bits - 1
    sm32 = float(np.float32(sm))
    Kx = oc.reconstructed("K")
    Vx = oc.reconstructed("V")
    qf = O.widen(np.ascontiguousarray(q), dt).astype(np.float64)
    aq = np.abs(qf)
    s = sm32 * np.einsum("bjd,btd->bjt", qf, Kx)
    M = s.max(axis=2, keepdims=True)
    w = np.exp(s - M)
    p = w / w.sum(axis=2, keepdims=True)
    o = np.einsum("bjt,btd->bjd", p, Vx)
    n_chunks = (T + 127) // 128

    # score error per (bh, j, t)
    Tk = np.einsum("bjd,btd->bjt", aq, np.abs(Kx))       # ring tokens
    Psplit = np.zeros_like(Tk)
    if Q:
        kc = O.unpack(np.ascontiguousarray(oc.k_codes[:, :Q]), D, bits)
        ks = np.abs(oc.k_scale[:, :Q // Gk].astype(np.float64))
        kz = np.abs(oc.k_zero[:, :Q // Gk].astype(np.float64))
        term = (kc.astype(np.float64) * np.repeat(ks, Gk, axis=1)
                + np.repeat(kz, Gk, axis=1))
        Tk[:, :, :Q] = np.einsum("bjd,btd->bjt", aq, term)
        Pg = (aq[:, :, None, :] * ks[:, None, :, :]).max(axis=3)
        Psplit[:, :, :Q] = np.repeat(Pg, Gk, axis=2)
    eps = (2 * D + 24) * E32 * Tk + D * L * 2.0 ** -37 * Psplit
    eta = sm32 * eps + E32 * (np.abs(s) + 4 * (M - s)) + 2.0 ** -19
    dev = np.abs(Vx[:, None, :, :] - o[:, :, None, :])
    b_w = np.einsum("bjt,bjtd->bjd", p * eta, dev)

    # value sums
    Wv = np.abs(Vx)
    vsmax = np.zeros((BH, 1, 1))
    if Q:
        vc = O.unpack(np.ascontiguousarray(oc.v_codes[:, :Q]), D, bits)
        vs = np.abs(oc.v_scale[:, :Q].astype(np.float64))
        vz = np.abs(oc.v_zero[:, :Q].astype(np.float64))
        Wv[:, :Q] = (vc.astype(np.float64) * np.repeat(vs, Gv, axis=2)[:, :, :D]
                     + np.repeat(vz, Gv, axis=2)[:, :, :D])
        vsmax = vs.max(axis=(1, 2))[:, None, None]
    b_v = (296 + n_chunks) * E32 * np.einsum("bjt,btd->bjd", p, Wv)
    b_split = n_chunks * L * 2.0 ** -30 * vsmax
    b_l = (n_chunks + 160) * E32 * np.abs(o)
    bound = (2.0 * (b_w + b_v + b_split + b_l)
             + unit_roundoff(dt) * np.abs(o) + subnormal_half_spacing(dt))
    return bound, o
