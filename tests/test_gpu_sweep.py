"""Seeded random sweeps on the GPU, each case against the oracle bit for bit.

- Flush entry points: every compute call (quantize, dequantize, fused,
  recon-only; keys and values) on random shapes, bit widths, group sizes,
  dtypes and value distributions. These reach the fast kernels and the
  generic fallbacks alike.
- K+V calls: each equals the two single calls on its tensors.
- Residual-window cache: random append sequences; after every append the
  store and the ring must equal the oracle scheduler's.
- Decode attention over random caches: within the derived bound of the
  oracle's exact attention (tests/attend_bound.py).
- KIVI-Sink and per-token mixed precision on random prompts: scores, lists,
  codes, params and reconstructions bit for bit.

The cases come from a fixed seed; the test ids name each case's
parameters."""
import zlib

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle                                               # noqa: E402
from gpu_util import FP16, host, say, to_dev                # noqa: E402
from test_gpu_cache import _compare as cache_compare       # noqa: E402
from test_gpu_parity import compare, run_all                # noqa: E402


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_quantization_kivi_amd as K
    return K


@pytest.fixture(scope="module")
def O():
    return oracle.default()


DISTS = ["normal", "outliers", "uniform", "constant_rows", "token_scales",
         "small_ints", "zeros_mixed"]


def values(seed, BH, S, D, dtype, dist):
    """A seeded [BH, S, D] tensor of 16-bit patterns of one of DISTS."""
    r = np.random.default_rng(seed)
    if dist == "normal":
        x = r.standard_normal((BH, S, D))
    elif dist == "outliers":
        x = r.standard_normal((BH, S, D))
        ch = r.choice(D, size=max(1, D // 16), replace=False)
        x[:, :, ch] *= 40.0
    elif dist == "uniform":
        x = r.uniform(-3.0, 5.0, (BH, S, D))
    elif dist == "constant_rows":         # runs of equal tokens: constant key groups
        base = r.standard_normal((BH, 1, D))
        x = np.repeat(base, S, axis=1)
        x[:, ::7] = r.standard_normal((BH, x[:, ::7].shape[1], D))
    elif dist == "token_scales":          # magnitudes from 1e-3 to 1e3 by token
        x = r.standard_normal((BH, S, D)) * 10.0 ** r.uniform(-3, 3, (BH, S, 1))
    elif dist == "small_ints":            # values on a small integer grid
        x = r.integers(-3, 4, (BH, S, D)).astype(np.float64)
    else:                                 # exact zeros (both signs) among values
        x = r.standard_normal((BH, S, D))
        x[r.random((BH, S, D)) < 0.4] = 0.0
        x[r.random((BH, S, D)) < 0.1] = -0.0
    x = x.astype(np.float32)
    if dtype == FP16:
        return x.astype(np.float16).view(np.uint16)
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16)
    return t.numpy().view(np.uint16)


def flush_cases(n=120, seed=2024):
    r = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        BH = int(r.integers(1, 7))
        S = int(r.choice([1, 2, 7, 31, 32, 33, 64, 95, 128, 200, 257, 400]))
        D = int(r.choice([8, 16, 24, 40, 64, 96, 128, 200, 256, 520]))
        dtype = int(r.integers(0, 2))
        bits = int(r.choice([1, 2, 4, 8]))
        gk = int(r.choice([1, 2, 3, 5, 8, 13, 16, 17, 24, 31, 32, 33, 64]))
        gv = int(r.choice([1, 3, 4, 8, 16, 24, 32, 64, 128, 256, D]))
        dist = DISTS[int(r.integers(0, len(DISTS)))]
        cases.append((BH, S, D, dtype, bits, gk, gv, dist))
    return cases


def case_id(c):
    return "x".join(map(str, c))


def _seed(case):
    """A seed from the case's parameters, the same in every process."""
    return zlib.crc32(repr(case).encode()) & 0x7FFFFFFF


@pytest.mark.parametrize("case", flush_cases(), ids=case_id)
def test_flush_sweep(K, O, case):
    BH, S, D, dtype, bits, gk, gv, dist = case
    x = values(_seed(case), BH, S, D, dtype, dist)
    tag = "sweep " + case_id(case)
    got = run_all(K, to_dev(x, dtype), dtype, bits, gk, gv, tag)
    compare(O, got, x, dtype, bits, gk, gv, tag)


def kv_cases(n=32, seed=77):
    r = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        BH = int(r.choice([1, 3, 32, 224, 600]))
        S = int(r.choice([1, 16, 32, 40, 64]))
        D = int(r.choice([64, 128, 256]))
        dtype = int(r.integers(0, 2))
        bits = int(r.choice([1, 2, 4, 8]))
        gk = int(r.choice([8, 17, 24, 32, 48]))
        gv = int(r.choice([16, 32, 64, 96, 128]))
        cases.append((BH, S, D, dtype, bits, gk, gv))
    return cases


def _same_bits(a, b, what):
    """Two device tensors hold the same bytes."""
    assert a.shape == b.shape, (what, a.shape, b.shape)
    assert np.array_equal(host(a.contiguous().view(torch.uint8)),
                          host(b.contiguous().view(torch.uint8))), what


@pytest.mark.parametrize("case", kv_cases(), ids=case_id)
def test_kv_calls_sweep(K, case):
    """kivi_quant_kv, kivi_quant_dequant_kv and kivi_dequant_kv (one launch
    or two, by their rule) against the single calls on each tensor."""
    BH, S, D, dtype, bits, gk, gv = case
    seed = _seed(case)
    k = to_dev(values(seed, BH, S, D, dtype, "outliers"), dtype)
    v = to_dev(values(seed + 1, BH, S, D, dtype, "normal"), dtype)
    say(f"[kv sweep {case_id(case)}]")
    qk = K.kivi_quant_keys(k, bits, gk)
    qv = K.kivi_quant_values(v, bits, gv)
    kq, vq = K.kivi_quant_kv(k, v, bits, gk, gv)
    fk = K.kivi_quant_dequant_keys(k, bits, gk)
    fv = K.kivi_quant_dequant_values(v, bits, gv)
    fkr, fvr, fkq, fvq = K.kivi_quant_dequant_kv(k, v, bits, gk, gv)
    dk = K.kivi_dequant_keys(*qk, bits, gk, out_dtype=k.dtype)
    dv = K.kivi_dequant_values(*qv, bits, gv, out_dtype=v.dtype)
    dkr, dvr = K.kivi_dequant_kv(qk, qv, bits, gk, gv, out_dtype=k.dtype)
    torch.cuda.synchronize()
    for name, a, b in zip(["key codes", "key scale", "key zero"], qk, kq):
        _same_bits(a, b, "quant_kv " + name)
    for name, a, b in zip(["value codes", "value scale", "value zero"], qv, vq):
        _same_bits(a, b, "quant_kv " + name)
    _same_bits(fk[0], fkr, "quant_dequant_kv key recon")
    _same_bits(fv[0], fvr, "quant_dequant_kv value recon")
    for name, a, b in zip(["key codes", "key scale", "key zero"], fk[1:], fkq):
        _same_bits(a, b, "quant_dequant_kv " + name)
    for name, a, b in zip(["value codes", "value scale", "value zero"], fv[1:], fvq):
        _same_bits(a, b, "quant_dequant_kv " + name)
    _same_bits(dk, dkr, "dequant_kv keys")
    _same_bits(dv, dvr, "dequant_kv values")


def cache_cases(n=36, seed=5):
    r = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        BH = int(r.choice([1, 2, 5, 9]))
        D = int(r.choice([16, 64, 128]))
        R = int(r.choice([0, 1, 5, 16, 32, 40]))
        gk = int(r.choice([8, 16, 32]))
        gv = int(r.choice([8, 16, 32, 64, D]))
        bits = int(r.choice([1, 2, 4, 8]))
        dtype = int(r.integers(0, 2))
        sizes = [int(s) for s in r.choice([1, 1, 1, 2, 7, 31, 32, 33, 100, 250],
                                          size=int(r.integers(3, 12)))]
        cases.append((BH, D, R, gk, gv, bits, dtype, tuple(sizes)))
    return cases


@pytest.mark.parametrize("case", cache_cases(),
                         ids=lambda c: case_id(c[:7]) + "_" + "-".join(map(str, c[7])))
def test_cache_sweep(K, O, case):
    BH, D, R, gk, gv, bits, dtype, sizes = case
    S_max = sum(sizes) + 3
    x = values(_seed(case), BH, S_max, D, dtype, "outliers")
    y = values(_seed(case) + 1, BH, S_max, D, dtype, "normal")
    tdt = torch.float16 if dtype == FP16 else torch.bfloat16
    c = K.KiviCache(BH, D, S_max, R, gk, gv, bits, tdt)
    o = O.cache(BH, D, S_max, R, gk, gv, bits, dtype)
    t = 0
    for i, n in enumerate(sizes):
        kx = np.ascontiguousarray(x[:, t:t + n])
        vy = np.ascontiguousarray(y[:, t:t + n])
        c.append(to_dev(kx, dtype), to_dev(vy, dtype))
        o.append(kx, vy)
        torch.cuda.synchronize()
        cache_compare(c, o, f"cache sweep append {i} (n={n}, T={t + n})")
        t += n


def attend_cases(n=40, seed=11):
    r = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        BH = int(r.integers(1, 7))
        D = int(r.choice([64, 128]))
        R = int(r.choice([0, 3, 8, 32, 40]))
        gk = int(r.choice([8, 16, 32]))
        gv = int(r.choice([8, 16, 32, 64, D]))
        bits = int(r.choice([1, 2, 4, 8]))
        if D * bits < 128:                 # kivi_cache_attend's rule
            bits = 2 if D == 64 else bits
        dtype = int(r.integers(0, 2))
        n_q = int(r.integers(1, 9))
        sizes = tuple(int(s) for s in r.choice([1, 1, 2, 9, 31, 64, 127, 128, 129, 300],
                                               size=int(r.integers(1, 6))))
        cases.append((BH, D, R, gk, gv, bits, dtype, n_q, sizes))
    return cases


@pytest.mark.parametrize("case", attend_cases(),
                         ids=lambda c: case_id(c[:8]) + "_" + "-".join(map(str, c[8])))
def test_attend_sweep(K, O, case):
    """kivi_cache_attend on random caches (both chunk kernels: G_k = 8 and
    8-bit codes take the token-per-thread one) within the derived bound of
    the oracle's exact attention."""
    from attend_bound import attend_bound, oracle_cache
    BH, D, R, gk, gv, bits, dtype, n_q, sizes = case
    S_max = sum(sizes) + 8
    seed = _seed(case)
    k = values(seed, BH, S_max, D, dtype, "outliers")
    v = values(seed + 1, BH, S_max, D, dtype, "normal")
    q = values(seed + 2, BH, n_q, D, dtype, "normal")   # 16-bit patterns
    tdt = torch.float16 if dtype == FP16 else torch.bfloat16
    c = K.KiviCache(BH, D, S_max, R, gk, gv, bits, tdt)
    t = 0
    for n in sizes:
        c.append(to_dev(np.ascontiguousarray(k[:, t:t + n]), dtype),
                 to_dev(np.ascontiguousarray(v[:, t:t + n]), dtype))
        t += n
    oc = oracle_cache(O, (BH, D, R, gk, gv, bits, dtype, n_q, list(sizes)), k, v, S_max)
    assert (c.T, c.Q) == (oc.T, oc.Q)
    sm = float(np.float32(1.0 / np.sqrt(D)))
    say(f"[attend sweep {case_id(case[:8])} T={c.T} Q={c.Q}]")
    out = c.attend(to_dev(q, dtype), sm)
    torch.cuda.synchronize()
    got = O.widen(host(out.view(torch.int16)).view(np.uint16), dtype).astype(np.float64)
    bound, ref = attend_bound(O, oc, q, sm)
    err = np.abs(got - ref)
    assert (err <= bound).all(), float((err / bound).max())


def sink_cases(n=24, seed=13):
    r = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        B = int(r.integers(1, 4))
        H = int(r.integers(1, 5))
        S = int(r.choice([1, 5, 31, 64, 100, 257, 600]))
        D = int(r.choice([8, 16, 64, 128, 256]))   # a power of two (the selection's rule)
        n_sink = int(min(S, r.choice([0, 1, 3, 5, 16, 64])))
        bits = int(r.choice([1, 2, 4, 8]))
        G = int(r.choice([1, 3, 8, 16, 31, 32]))
        dtype = int(r.integers(0, 2))
        dist = DISTS[int(r.integers(0, len(DISTS)))]
        cases.append((B, H, S, D, n_sink, bits, G, dtype, dist))
    return cases


@pytest.mark.parametrize("case", sink_cases(), ids=case_id)
def test_sink_sweep(K, O, case):
    """KIVI-Sink on random prompts: scores, lists, the sink-masked key
    quantization (codes, params, reconstruction) and the gathered rows, bit
    for bit against the oracle."""
    from gpu_util import (assert_codes_equal, assert_f32_bits_equal,
                          assert_recon_equal, bits16)
    B, H, S, D, n_sink, bits, G, dtype, dist = case
    x = values(_seed(case), B * H, S, D, dtype, dist)
    xd = to_dev(x, dtype)
    say(f"[sink sweep {case_id(case)}]")
    idx_d, score_d = K.kivi_sink_select(xd, n_sink, H=H)
    recon, codes, scale, zero = K.kivi_quant_keys_sink(xd, idx_d, bits, G, H=H,
                                                       with_recon=True)
    kept = K.kivi_sink_gather(xd, idx_d, H=H)
    torch.cuda.synchronize()
    want_s = O.sink_scores(x, dtype, H)
    assert np.array_equal(host(score_d).view(np.uint32), want_s.view(np.uint32)), "scores"
    idx = host(idx_d)
    assert np.array_equal(idx, O.sink_select(want_s, n_sink)), "sink lists"
    wc, ws, wz = O.quant_keys_sink(x, dtype, H, bits, G, idx)
    assert_codes_equal(host(codes), wc, "codes")
    assert_f32_bits_equal(host(scale), ws, "scale")
    assert_f32_bits_equal(host(zero), wz, "zero")
    assert_recon_equal(bits16(recon), O.sink_recon(x, dtype, H, bits, G, idx), "recon")
    assert np.array_equal(bits16(kept), O.sink_gather(x, H, idx)), "gathered rows"


def mixed_cases(n=24, seed=17):
    r = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        B = int(r.integers(1, 4))
        H = int(r.integers(1, 4))
        S = int(r.choice([1, 7, 40, 128, 300, 1000]))
        D = int(r.choice([8, 32, 64, 128, 256]))
        n_hi = int(r.integers(0, S + 1))
        hi_bits, lo_bits = [int(b) for b in r.choice([[4, 2], [8, 4], [2, 1], [4, 1]])]
        Gk = int(r.choice([1, 5, 8, 16, 32]))
        Gv = int(r.choice([8, 16, 32, 64, D]))
        dtype = int(r.integers(0, 2))
        dist = DISTS[int(r.integers(0, len(DISTS)))]
        cases.append((B, H, S, D, n_hi, hi_bits, lo_bits, Gk, Gv, dtype, dist))
    return cases


@pytest.mark.parametrize("case", mixed_cases(), ids=case_id)
def test_mixed_sweep(K, O, case):
    """Per-token mixed precision on random prompts: the key-norm partition
    and both sets' listed-row quantization and dequantization, bit for bit
    against the oracle."""
    from gpu_util import (TORCH_DT, assert_codes_equal, assert_f32_bits_equal,
                          assert_recon_equal, bits16, to_dev_raw)
    B, H, S, D, n_hi, hb, lb, Gk, Gv, dtype, dist = case
    seed = _seed(case)
    k = values(seed, B * H, S, D, dtype, dist)
    v = values(seed + 1, B * H, S, D, dtype, "normal")
    kd, vd = to_dev(k, dtype), to_dev(v, dtype)
    say(f"[mixed sweep {case_id(case)}]")
    score = K.kivi_key_scores(kd, H=H)
    hi, lo = K.kivi_partition_top(score, n_hi)
    torch.cuda.synchronize()
    want_s = O.sink_scores(k, dtype, H)
    ehi, elo = O.partition_top(want_s, n_hi)
    assert np.array_equal(host(hi), ehi) and np.array_equal(host(lo), elo), "partition"
    for pos, bits in ((ehi, hb), (elo, lb)):
        if pos.shape[1] == 0:
            continue
        pd = to_dev_raw(np.ascontiguousarray(pos))
        for keys, x, xd, G in ((True, k, kd, Gk), (False, v, vd, Gv)):
            q = K.kivi_quant_keys_rows if keys else K.kivi_quant_values_rows
            dq = K.kivi_dequant_keys_rows if keys else K.kivi_dequant_values_rows
            codes, scale, zero = q(xd, pd, bits, G, H=H)
            out = torch.zeros((B * H, S, D), dtype=TORCH_DT[dtype], device="cuda")
            dq(codes, scale, zero, pd, out, bits, G, H=H)
            torch.cuda.synchronize()
            oq = O.quant_keys_rows if keys else O.quant_values_rows
            odq = O.dequant_keys_rows if keys else O.dequant_values_rows
            wc, ws, wz = oq(x, dtype, H, bits, G, pos)
            tag = f"bits={bits} keys={keys}"
            assert_codes_equal(host(codes), wc, "codes " + tag)
            assert_f32_bits_equal(host(scale), ws, "scale " + tag)
            assert_f32_bits_equal(host(zero), wz, "zero " + tag)
            assert_recon_equal(bits16(out), odq(wc, ws, wz, x.shape, H, bits, G, pos, dtype),
                               "recon " + tag)
