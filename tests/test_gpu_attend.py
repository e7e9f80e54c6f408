"""GPU parity of decode attention over the residual-window cache
(kivi_cache_attend, reading the packed store) against the oracle's float64
attention over the dequantized cache (oracle.OracleCache.attend).

Tolerance, derived from the arithmetic (u = 2^-11 for fp16, 2^-8 for bf16,
e = 2^-24 for fp32):
 * keys: the kernel forms a score of a quantized token as
   sum_d (q_d scale_d) code_d + sum_d q_d zero_d in fp32, never rounding the
   key to the 16-bit type as the oracle's dequantized cache does; the score
   moves by at most
       ds_t = sm * (u * sum_d |q_d| |k_td| + e (D + 4) sum_d |q_d| (|k_td| + 2 |z_td|))
   (|code * scale| <= |k| + |z|, an fp32 sum of D + 2 terms), and the
   softmax weights then move by at most 2 max_t ds_t in total variation,
   which moves the output by that times max |V|;
 * values: likewise summed as sum_t (p_t scale_t) code_t + sum_t p_t zero_t in
   fp32 without the 16-bit rounding: at most u max|V| from the rounding, plus
   e n_acc (max|V| + 2 max|z_v|) for fp32 sums of depth at most
   n_acc = 128 + chunks + 8 (tokens of a chunk, the chunk merge, the shuffle
   tree);
 * the result is rounded once to the 16-bit type (u |o|), and 2^-20 max|V|
   covers the fp32 exponentials;
 * the matrix-core kernel feeds q * scale and p * vscale to f16 operands as
   hi + lo after a power-of-two scaling bounded by qmax * smax (vmax for
   values): relative error 2^-22 (inside the terms above) plus, where lo
   falls below f16's normal range, an absolute 2^-38 of the bound per
   operand: at most sm 2^-34 D qmax smax on a score and 2^-34 T vmax on
   the output.
The test bound is the sum of these terms, the first two times 1.25, per
element, with the maxima taken per (bh, query head)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle                                              # noqa: E402
from gpu_util import FP16, BF16, host, say                 # noqa: E402


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_quantization_kivi_amd as K
    return K


@pytest.fixture(scope="module")
def O():
    return oracle.default()


def _tokens(seed, BH, n, D, dtype, scale=1.0):
    r = np.random.default_rng(seed)
    x = (r.standard_normal((BH, n, D)) * scale).astype(np.float32)
    x[:, :, r.choice(D, size=max(1, D // 32), replace=False)] *= 8.0
    if dtype == FP16:
        return x.astype(np.float16).view(np.uint16)
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16)
    return t.numpy().view(np.uint16)


def _dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16))
    return t.view(torch.float16 if dtype == FP16 else torch.bfloat16).cuda()


def _widen(O, x, dtype):
    return O.widen(np.ascontiguousarray(x), dtype).astype(np.float64)


def _bound(O, oc, q, sm, ref, dtype):
    u = 2.0 ** -11 if dtype == FP16 else 2.0 ** -8
    e = 2.0 ** -24
    Kf = _widen(O, oc.dequantized("K"), dtype)
    Vf = _widen(O, oc.dequantized("V"), dtype)
    qf = _widen(O, q, dtype)
    BH, T, D = Kf.shape
    Q, G_k = oc.Q, oc.c.G_k
    zk = np.zeros((BH, T, D))
    zk[:, :Q] = np.repeat(oc.k_zero[:, :Q // G_k].astype(np.float64), G_k, axis=1)
    aq = np.abs(qf)
    ds = sm * (u * np.einsum("bjd,btd->bjt", aq, np.abs(Kf))
               + e * (D + 4) * np.einsum("bjd,btd->bjt", aq, np.abs(Kf) + 2 * np.abs(zk)))
    vmax = np.abs(Vf).max(axis=(1, 2))[:, None, None]
    zv = np.abs(oc.v_zero[:, :Q].astype(np.float64))
    zvmax = (zv.max(axis=(1, 2)) if Q else np.zeros(BH))[:, None, None]
    n_acc = 128 + (T + 127) // 128 + 8
    if Q:
        skmax = np.abs(oc.k_scale[:, :Q // G_k]).max(axis=(1, 2))[:, None]
        svmax = np.abs(oc.v_scale[:, :Q]).max(axis=(1, 2))[:, None, None]
    else:
        skmax = np.zeros((BH, 1))
        svmax = np.zeros((BH, 1, 1))
    ds = ds + sm * 2.0 ** -34 * D * aq.max(axis=2)[:, :, None] * skmax[:, :, None]
    vterm = u * vmax + e * n_acc * (vmax + 2 * zvmax) + 2.0 ** -34 * T * svmax
    return (1.25 * (2.0 * ds.max(axis=2)[:, :, None] * vmax + vterm)
            + u * np.abs(ref) + 2.0 ** -20 * vmax)


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


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(
    map(str, c[:8])) + "_" + "-".join(map(str, c[8])))
def test_attend_matches_oracle(K, O, case):
    BH, D, R, Gk, Gv, bits, dtype, n_q, appends = case
    tdt = torch.float16 if dtype == FP16 else torch.bfloat16
    S_max = sum(appends) + 8
    c = K.KiviCache(BH, D, S_max, R, Gk, Gv, bits, tdt)
    oc = O.cache(BH, D, S_max, R, Gk, Gv, bits, dtype)
    t = 0
    k = _tokens(41, BH, S_max, D, dtype)
    v = _tokens(42, BH, S_max, D, dtype)
    for n in appends:
        kn, vn = np.ascontiguousarray(k[:, t:t + n]), np.ascontiguousarray(v[:, t:t + n])
        c.append(_dev(kn, dtype), _dev(vn, dtype))
        oc.append(kn, vn)
        t += n
    q = _tokens(43, BH, n_q, D, dtype, scale=0.5)
    sm = 1.0 / np.sqrt(D)
    say(f"[attend {case[:8]} T={c.T} Q={c.Q}]")
    out = c.attend(_dev(q, dtype), sm)
    torch.cuda.synchronize()
    got = _widen(O, host(out.view(torch.int16)).view(np.uint16), dtype)
    ref = oc.attend(q, sm)
    bound = _bound(O, oc, q, sm, ref, dtype)
    err = np.abs(got - ref)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert (err <= bound).all(), (case[:8], worst, got[worst], ref[worst],
                                  bound[worst])


def test_attend_long_context_chunks(K, O):
    """Prompt of 2059 tokens (prefill chunks of 2048) plus 40 decode tokens,
    GQA with 4 query heads per KV head: 17 chunks of 128 tokens merged."""
    BH, D, n_q = 8, 128, 4
    S_max = 2099
    c = K.KiviCache(BH, D, S_max, 32, 32, 32, 2, torch.float16)
    oc = O.cache(BH, D, S_max, 32, 32, 32, 2, FP16)
    k = _tokens(51, BH, S_max, D, FP16)
    v = _tokens(52, BH, S_max, D, FP16)
    for a, b in ((0, 2048), (2048, 2059)):
        c.append(_dev(k[:, a:b], FP16), _dev(v[:, a:b], FP16))
        oc.append(np.ascontiguousarray(k[:, a:b]), np.ascontiguousarray(v[:, a:b]))
    for s in range(2059, S_max):
        c.append(_dev(k[:, s:s + 1], FP16), _dev(v[:, s:s + 1], FP16))
        oc.append(np.ascontiguousarray(k[:, s:s + 1]), np.ascontiguousarray(v[:, s:s + 1]))
    q = _tokens(53, BH, n_q, D, FP16, scale=0.5)
    sm = 1.0 / np.sqrt(D)
    out = c.attend(_dev(q, FP16), sm)
    torch.cuda.synchronize()
    got = _widen(O, host(out.view(torch.int16)).view(np.uint16), FP16)
    ref = oc.attend(q, sm)
    assert (np.abs(got - ref) <= _bound(O, oc, q, sm, ref, FP16)).all()


def test_attend_rejects(K):
    c = K.KiviCache(2, 256, 64, 8, 8, 8, 2, torch.float16)  # D = 256
    x = torch.zeros((2, 4, 256), dtype=torch.float16, device="cuda")
    c.append(x, x)
    with pytest.raises(K.KiviError):
        c.attend(torch.zeros((2, 1, 256), dtype=torch.float16, device="cuda"), 1.0)
    c2 = K.KiviCache(2, 64, 64, 8, 8, 8, 2, torch.float16)
    with pytest.raises(K.KiviError):                      # T = 0
        c2.attend(torch.zeros((2, 1, 64), dtype=torch.float16, device="cuda"), 1.0)
    y = torch.zeros((2, 4, 64), dtype=torch.float16, device="cuda")
    c2.append(y, y)
    with pytest.raises(K.KiviError):                      # n_q = 9
        c2.attend(torch.zeros((2, 9, 64), dtype=torch.float16, device="cuda"), 1.0)
