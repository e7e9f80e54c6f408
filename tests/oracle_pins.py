"""Pins that tie the KIVI oracle to something other than itself.

Each `pin_*` function takes an oracle object (oracle.Oracle) and raises
AssertionError when the oracle disagrees with what the VeloxQuant-MLX pages
or the mathematics fix:

  - hand-worked groups and packing bytes (tests/golden/worked_examples.json,
    each case with its citation and derivation);
  - exhaustive / boundary checks of the 16-bit conversions against numpy
    (fp16) and torch on the CPU (bf16);
  - exact rational arithmetic: the fp32 division is a correctly rounded
    quotient (not a reciprocal product), the code is the nearest grid point;
  - invariants: code range, min -> code 0, max -> top code, reconstruction
    error within scale/2, constant groups, grid-exact round trips,
    determinism;
  - equivalences: a ragged group equals the pages' edge-replicate padding;
    per-channel keys equal per-token values of the transposed tensor;
  - the residual-window cache: the pages' flush counts (prompts of 559,
    2059, 8209 tokens flush 512, 2016, 8160; 240 decode tokens make 7
    flushes), the window invariant, and group-by-group flushing equal to
    quantizing the flushed prefix at once;
  - KIVI-Sink: the key-norm score re-derived bit-exactly with numpy and
    3-4-5 rows, selection equal to numpy's stable argsort, a hand-worked
    spike group, brute-force masked group params and codes, n_sink = 0
    equal to plain KIVI, and the pages' claims on planted-sink data (sinks
    bit-exact, lower MSE than plain KIVI and than keeping the first n);
  - per-token mixed precision: the partition equals numpy's stable argsort,
    listed rows equal numpy-gathered tensors through the plain quantizers,
    and the page's evidence (cosine above 0.995 at 4 bits and 0.8 at 2,
    all-hi beats all-lo, mixed in between in error and bytes);
  - the pages' statistic: 2-bit reconstruction cosine about 0.93 on
    unit-norm Gaussian keys (KIVI release post, "Honest limitations"; PyPI
    page, KIVI section), 4-bit above 0.995 (PyPI page, ZipCache section).

tests/test_oracle_pins.py runs them on the real oracle;
tests/test_oracle_mutants.py runs them on broken copies and requires each
copy to fail at least one.
"""
import json
import os
from fractions import Fraction

import numpy as np

from exact import F, bits32, from_bits32, rn32, round_half_even

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
FP16, BF16 = 0, 1


def golden():
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        return json.load(f)


def _expect_f32(case, key):
    if key + "_bits" in case:
        return from_bits32(int(case[key + "_bits"], 16))
    return np.float32(case[key])


def _f16_bits(vals):
    return np.asarray(vals, np.float32).astype(np.float16).view(np.uint16)


# --------------------------------------------------------------------------
# 16-bit conversions
# --------------------------------------------------------------------------

def pin_fp16_widen_exhaustive(o):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.widen(h, FP16)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _narrow_probe_set(rng, widen_of_all):
    """fp32 values around every representable 16-bit value: the values, the
    midpoints between neighbours and one fp32 ulp either side of each."""
    finite = widen_of_all[np.isfinite(widen_of_all)].astype(np.float64)
    finite = np.unique(finite)
    mids = (finite[:-1] + finite[1:]) / 2.0
    pts = np.concatenate([finite, mids]).astype(np.float32)
    pts = pts[np.isfinite(pts)]
    up = np.nextafter(pts, np.float32(np.inf))
    dn = np.nextafter(pts, np.float32(-np.inf))
    rnd = rng.integers(0, 2**32, size=400_000, dtype=np.uint64)
    rnd = rnd.astype(np.uint32).view(np.float32)
    rnd = rnd[~np.isnan(rnd)]
    return np.concatenate([pts, up, dn, rnd,
                           np.array([np.inf, -np.inf, 65504, 65519.996,
                                     65520, -65520, 1e-8, 2.0**-25,
                                     2.0**-24, 3 * 2.0**-26], np.float32)])


def pin_fp16_narrow_rne(o):
    rng = np.random.default_rng(11)
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    probes = _narrow_probe_set(rng, h.view(np.float16).astype(np.float32))
    got = o.narrow(probes, FP16)
    with np.errstate(over="ignore"):
        ref = probes.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref), int(np.sum(got != ref))


def pin_bf16_widen_narrow(o):
    import torch
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.widen(h, BF16)
    ref = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).float()
    ref = ref.numpy()
    nan = np.isnan(ref)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    rng = np.random.default_rng(12)
    probes = _narrow_probe_set(rng, ref)
    probes = probes[np.abs(probes) < 3.0e38]
    got = o.narrow(probes, BF16)
    refn = torch.from_numpy(probes).to(torch.bfloat16).view(torch.int16)
    refn = refn.numpy().view(np.uint16)
    assert np.array_equal(got, refn), int(np.sum(got != refn))


# --------------------------------------------------------------------------
# Worked examples from the golden file
# --------------------------------------------------------------------------

def pin_worked_groups(o):
    for case in golden()["groups"]:
        vals = np.asarray(case["values"], np.float32)
        bits = case["bits"]
        sc, z = o.group_params(vals, bits)
        name = case["name"]
        assert bits32(z) == bits32(_expect_f32(case, "zero")), name
        assert bits32(sc) == bits32(_expect_f32(case, "scale")), name
        codes = [o.code(v, sc, z, bits) for v in vals]
        assert codes == case["codes"], (name, codes)
        if "recon" in case:
            rec = [float(o.recon(c, sc, z)) for c in codes]
            assert rec == case["recon"], (name, rec)
        # the same group through the tensor path, as one value row
        x = _f16_bits(vals)[None, None, :]
        if np.array_equal(x.view(np.float16).astype(np.float32)[0, 0], vals) \
                and (vals.size * bits) % 8 == 0:
            c2, s2, z2 = o.quant_values_unpacked(x, FP16, bits, vals.size)
            assert c2[0, 0].tolist() == case["codes"], name
            assert bits32(s2[0, 0, 0]) == bits32(sc), name


def pin_recon_two_roundings(o):
    c = golden()["recon_two_roundings"]
    sc = from_bits32(int(c["scale_bits"], 16))
    z = np.float32(c["zero"])
    r = o.recon(c["code"], sc, z)
    assert bits32(r) == int(c["recon_f32_bits"], 16)
    # through dequant to fp16: one value row of 4 codes (2-bit), code 3 first
    packed = np.array([[[0x03]]], np.uint8)
    out = o.dequant_values(packed, np.array([[[sc]]], np.float32),
                           np.array([[[z]]], np.float32), (1, 1, 4), 2, 4,
                           FP16)
    assert int(out[0, 0, 0]) == int(c["recon_fp16_bits"], 16)
    assert int(out[0, 0, 0]) != int(c["fma_recon_fp16_bits"], 16)
    out_k = o.dequant_keys(packed, np.full((1, 1, 4), sc, np.float32),
                           np.full((1, 1, 4), z, np.float32), (1, 1, 4), 2, 1,
                           FP16)
    assert int(out_k[0, 0, 0]) == int(c["recon_fp16_bits"], 16)


def pin_packing_golden(o):
    for case in golden()["packing"]["cases"]:
        bits = case["bits"]
        codes = np.asarray(case["codes"], np.uint8)[None, :]
        want = [int(b, 16) for b in case["bytes"]]
        got = o.pack(codes, bits)[0].tolist()
        assert got == want, (case, got)
        back = o.unpack(np.asarray(want, np.uint8)[None, :], codes.shape[1],
                        bits)
        assert np.array_equal(back, codes), case


def pin_pack_roundtrip_lsb_first(o):
    rng = np.random.default_rng(3)
    for bits in (1, 2, 4, 8):
        D = 64
        codes = rng.integers(0, 2**bits, size=(5, 7, D), dtype=np.uint8)
        packed = o.pack(codes, bits)
        assert packed.shape == (5, 7, D * bits // 8)
        assert np.array_equal(o.unpack(packed, D, bits), codes)
        # the rule itself: code i of byte j sits at bits [i*bits, (i+1)*bits)
        per = 8 // bits
        for i in range(per):
            field = (packed.astype(np.uint32) >> (i * bits)) & ((1 << bits) - 1)
            assert np.array_equal(field, codes[..., i::per])


# --------------------------------------------------------------------------
# Exact arithmetic
# --------------------------------------------------------------------------

def pin_clip(o):
    """The chain's clip step (KIVI Metal-kernel post, 'What we're actually
    optimizing'): an element outside [zero, zero + (2^b - 1) * scale] is
    clipped to the end codes.  Inside a group it never binds, so it is
    pinned through the element call."""
    for bits in (1, 2, 4, 8):
        top = 2**bits - 1
        assert o.code(top + 5.0, 1.0, 0.0, bits) == top
        assert o.code(top + 0.75, 1.0, 0.0, bits) == top
        assert o.code(-3.0, 1.0, 0.0, bits) == 0
        assert o.code(-0.75, 0.5, 0.0, bits) == 0
        assert o.code(top * 0.5, 0.5, 0.0, bits) == top


def pin_params_exact(o):
    """zero = min exactly; scale = RN32(RN32(max - min) / (2^b - 1))."""
    rng = np.random.default_rng(5)
    for trial in range(300):
        n = int(rng.integers(1, 70))
        bits = int(rng.choice([1, 2, 4, 8]))
        v = (rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 3))
        v = v.astype(np.float16).astype(np.float32)
        sc, z = o.group_params(v, bits)
        mn, mx = v.min(), v.max()
        want_z = np.float32(0.0) if mn == 0 else mn
        assert bits32(z) == bits32(want_z)
        rng_ = rn32(F(mx) - F(mn if mn != 0 else 0.0))
        want_s = rn32(F(rng_) / (2**bits - 1))
        assert bits32(sc) == bits32(want_s), (v, bits)


def pin_divide_not_reciprocal(o):
    """Cases where a*RN(1/scale) would round to another code than RN(a/scale):
    the oracle must give the correctly rounded quotient's code."""
    rng = np.random.default_rng(17)
    found = 0
    for _ in range(200_000):
        s = np.float32(rng.uniform(0.01, 100.0))
        y = rn32(Fraction(1) / F(s))
        k = int(rng.integers(0, 3))
        a = np.float32((k + 0.5) * float(s))
        for a_try in (a, np.nextafter(a, np.float32(0)),
                      np.nextafter(a, np.float32(np.inf))):
            t_div = rn32(F(a_try) / F(s))
            t_rcp = rn32(F(a_try) * F(y))
            c_div = round_half_even(F(t_div))
            if round_half_even(F(t_rcp)) != c_div:
                assert o.code(a_try, s, 0.0, 2) == min(max(c_div, 0), 3)
                found += 1
        if found >= 20:
            break
    assert found >= 20


def pin_nearest_code_bruteforce(o):
    """Brute force over every code: the chosen code is the grid point nearest
    to x (exact rationals), except within a relative 2^-20 of a midpoint,
    where either neighbour is acceptable."""
    rng = np.random.default_rng(23)
    for trial in range(400):
        bits = int(rng.choice([1, 2, 4, 8]))
        n = int(rng.integers(2, 40))
        v = rng.standard_normal(n) * 10.0 ** rng.uniform(-2, 2)
        v = v.astype(np.float16).astype(np.float32)
        sc, z = o.group_params(v, bits)
        if sc == 0:
            continue
        for x in v:
            c = o.code(x, sc, z, bits)
            dists = [abs(F(x) - F(z) - j * F(sc)) for j in range(2**bits)]
            best = min(dists)
            second = sorted(dists)[1]
            if second - best > Fraction(1, 2**20) * (abs(F(x) - F(z)) + F(sc)):
                assert dists[c] == best, (x, c, dists.index(best))
            else:
                assert dists[c] in (best, second)


# --------------------------------------------------------------------------
# Invariants on tensors
# --------------------------------------------------------------------------

def _rand_tensor(rng, BH, S, D, dtype, outliers=True):
    x = rng.standard_normal((BH, S, D)).astype(np.float32)
    if outliers:
        ch = rng.choice(D, size=max(1, D // 32), replace=False)
        x[:, :, ch] *= 20.0
    if dtype == FP16:
        return x.astype(np.float16).view(np.uint16)
    u = x.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _out_ulp(vals, dtype):
    a = np.abs(vals).astype(np.float64)
    if dtype == FP16:
        e = np.floor(np.log2(np.maximum(a, 2.0**-14)))
        return 2.0 ** (e - 10)
    e = np.floor(np.log2(np.maximum(a, 2.0**-126)))
    return 2.0 ** (e - 7)


def _check_quant_invariants(o, x, dtype, bits, gk, gv):
    BH, S, D = x.shape
    f = o.widen(x, dtype).astype(np.float64)
    maxc = 2**bits - 1
    for kind in ("keys", "values"):
        if kind == "keys":
            codes, sc, z = o.quant_keys_unpacked(x, dtype, bits, gk)
            gidx = np.arange(S) // gk
            scx = sc[:, gidx, :].astype(np.float64)
            zx = z[:, gidx, :].astype(np.float64)
            packed, sc2, z2 = o.quant_keys(x, dtype, bits, gk)
            rec = o.dequant_keys(packed, sc2, z2, x.shape, bits, gk, dtype)
        else:
            codes, sc, z = o.quant_values_unpacked(x, dtype, bits, gv)
            gidx = np.arange(D) // gv
            scx = sc[:, :, gidx].astype(np.float64)
            zx = z[:, :, gidx].astype(np.float64)
            packed, sc2, z2 = o.quant_values(x, dtype, bits, gv)
            rec = o.dequant_values(packed, sc2, z2, x.shape, bits, gv, dtype)
        assert np.array_equal(sc, sc2) and np.array_equal(z, z2)
        assert np.array_equal(o.unpack(packed, D, bits), codes)
        assert codes.max() <= maxc
        # zero is the group min; every element is >= zero
        assert np.all(f >= zx)
        # reconstruction within half a step plus rounding slack
        r = o.widen(rec, dtype).astype(np.float64)
        slack = (np.abs(f) + np.abs(zx) + maxc * scx) * 2.0**-22 \
            + _out_ulp(r, dtype)
        err = np.abs(r - f)
        assert np.all(err <= scx / 2 + slack), float((err - scx / 2).max())
        # group min -> code 0, group max -> top code (when the range > 0)
        if kind == "keys":
            for bh in range(BH):
                for g in range(sc.shape[1]):
                    blk = f[bh, g * gk:(g + 1) * gk, :]
                    cb = codes[bh, g * gk:(g + 1) * gk, :]
                    am = blk.argmin(0)
                    ax = blk.argmax(0)
                    d = np.arange(D)
                    assert np.all(cb[am, d] == 0)
                    pos = sc[bh, g] > 0
                    assert np.all(cb[ax, d][pos] == maxc)
        else:
            for j in range(sc.shape[2]):
                blk = f[:, :, j * gv:(j + 1) * gv]
                cb = codes[:, :, j * gv:(j + 1) * gv]
                am = blk.argmin(2)[..., None]
                ax = blk.argmax(2)[..., None]
                assert np.all(np.take_along_axis(cb, am, 2) == 0)
                pos = sc[:, :, j] > 0
                assert np.all(np.take_along_axis(cb, ax, 2)[..., 0][pos]
                              == maxc)


def pin_tensor_invariants(o):
    rng = np.random.default_rng(29)
    for (BH, S, D, dtype, bits, gk, gv) in [
            (2, 64, 64, FP16, 2, 32, 32),
            (3, 70, 48, FP16, 2, 32, 32),     # ragged S and D groups
            (2, 40, 128, BF16, 4, 32, 128),
            (2, 33, 16, FP16, 1, 16, 8),
            (1, 50, 24, BF16, 8, 7, 5),
            (2, 96, 64, FP16, 4, 64, 64)]:
        x = _rand_tensor(rng, BH, S, D, dtype)
        _check_quant_invariants(o, x, dtype, bits, gk, gv)


def pin_constant_groups(o):
    rng = np.random.default_rng(31)
    for dtype in (FP16, BF16):
        x = _rand_tensor(rng, 2, 64, 64, dtype)
        cval = _f16_bits([0.75])[0] if dtype == FP16 else np.uint16(0x3F40)
        x[1, 32:64, 5] = cval             # constant key group
        x[0, 10, 32:64] = cval            # constant value group
        for kind in ("keys", "values"):
            if kind == "keys":
                packed, sc, z = o.quant_keys(x, dtype, 2, 32)
                codes = o.unpack(packed, 64, 2)
                assert sc[1, 1, 5] == 0
                assert bits32(z[1, 1, 5]) == bits32(np.float32(0.75))
                assert np.all(codes[1, 32:64, 5] == 0)
                rec = o.dequant_keys(packed, sc, z, x.shape, 2, 32, dtype)
                assert np.all(rec[1, 32:64, 5] == cval)
            else:
                packed, sc, z = o.quant_values(x, dtype, 2, 32)
                codes = o.unpack(packed, 64, 2)
                assert sc[0, 10, 1] == 0
                assert bits32(z[0, 10, 1]) == bits32(np.float32(0.75))
                assert np.all(codes[0, 10, 32:64] == 0)
                rec = o.dequant_values(packed, sc, z, x.shape, 2, 32, dtype)
                assert np.all(rec[0, 10, 32:64] == cval)


def pin_ragged_equals_edge_padding(o):
    """KIVI Metal-kernel post, 'Three ways to be off by one bit', item 3: a
    ragged last group behaves as if padded with copies of its edge element."""
    rng = np.random.default_rng(37)
    for dtype in (FP16, BF16):
        x = _rand_tensor(rng, 2, 70, 48, dtype)      # S=70: last key group 6
        G = 32
        xp = np.concatenate([x, np.repeat(x[:, -1:, :], 96 - 70, axis=1)], 1)
        c1, s1, z1 = o.quant_keys_unpacked(x, dtype, 2, G)
        c2, s2, z2 = o.quant_keys_unpacked(xp, dtype, 2, G)
        assert np.array_equal(s1, s2) and np.array_equal(z1, z2)
        assert np.array_equal(c1, c2[:, :70, :])
        # D=48 with G=32: last value group has 16 channels
        xv = np.concatenate([x, np.repeat(x[:, :, -1:], 64 - 48, axis=2)], 2)
        c1, s1, z1 = o.quant_values_unpacked(x, dtype, 2, G)
        c2, s2, z2 = o.quant_values_unpacked(xv, dtype, 2, G)
        assert np.array_equal(s1, s2) and np.array_equal(z1, z2)
        assert np.array_equal(c1, c2[:, :, :48])


def pin_keys_equal_values_of_transpose(o):
    """Per-channel keys grouped over tokens are per-token values of the
    transposed tensor grouped over channels (KIVI Metal-kernel post, 'The
    layout problem that shapes everything')."""
    rng = np.random.default_rng(41)
    x = _rand_tensor(rng, 3, 64, 40, FP16)
    xt = np.ascontiguousarray(x.transpose(0, 2, 1))
    for G in (32, 8, 5):
        ck, sk, zk = o.quant_keys_unpacked(x, FP16, 2, G)
        cv, sv, zv = o.quant_values_unpacked(xt, FP16, 2, G)
        assert np.array_equal(ck, cv.transpose(0, 2, 1))
        assert np.array_equal(sk, sv.transpose(0, 2, 1))
        assert np.array_equal(zk, zv.transpose(0, 2, 1))


def pin_grid_exact_roundtrip(o):
    """Elements already on a group's grid reconstruct bit-exactly."""
    rng = np.random.default_rng(43)
    for bits in (1, 2, 4):
        maxc = 2**bits - 1
        z0 = np.float32(-2.0)
        step = np.float32(0.125)
        codes = rng.integers(0, maxc + 1, size=(2, 32, 64))
        codes[:, 0, :] = 0
        codes[:, 1, :] = maxc           # every key group spans the full range
        f = (z0 + codes.astype(np.float32) * step).astype(np.float32)
        x = f.astype(np.float16).view(np.uint16)
        packed, sc, z = o.quant_keys(x, FP16, bits, 32)
        assert np.all(sc == step) and np.all(z == z0)
        assert np.array_equal(o.unpack(packed, 64, bits), codes)
        rec = o.dequant_keys(packed, sc, z, x.shape, bits, 32, FP16)
        assert np.array_equal(rec, x)


def pin_determinism(o):
    rng = np.random.default_rng(47)
    x = _rand_tensor(rng, 2, 64, 64, BF16)
    a = o.quant_keys(x, BF16, 2, 32)
    b = o.quant_keys(x, BF16, 2, 32)
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def pin_invalid_args(o):
    x = np.zeros((1, 4, 6), np.uint16)
    for bits, G in ((3, 2), (2, 0)):
        try:
            o.quant_keys(x, FP16, bits, G)
        except ValueError:
            pass
        else:
            raise AssertionError("accepted bits=%d group=%d" % (bits, G))
    try:   # D*bits not a multiple of 8
        o.quant_values(np.zeros((1, 4, 6), np.uint16), FP16, 1, 2)
    except ValueError:
        pass
    else:
        raise AssertionError("accepted D*bits % 8 != 0")


# --------------------------------------------------------------------------
# The pages' statistic
# --------------------------------------------------------------------------

def _cosine_unit_norm_keys(o, bits, n_tok=4096, D=128, seed=53):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((n_tok, D))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    x = k.astype(np.float16).view(np.uint16)[None]
    packed, sc, z = o.quant_keys(x, FP16, bits, 32)
    rec = o.dequant_keys(packed, sc, z, x.shape, bits, 32, FP16)
    r = rec[0].view(np.float16).astype(np.float64)
    xf = x[0].view(np.float16).astype(np.float64)
    cos = (r * xf).sum(1) / (np.linalg.norm(r, axis=1)
                             * np.linalg.norm(xf, axis=1))
    return float(cos.mean())


def pin_cosine_statistics(o):
    c2 = _cosine_unit_norm_keys(o, 2)
    assert 0.92 <= c2 <= 0.94, c2        # the pages give about 0.93
    c4 = _cosine_unit_norm_keys(o, 4)
    assert c4 > 0.995, c4                # pages: 4-bit "> 0.995"


# --------------------------------------------------------------------------
# The residual-window cache (flush scheduling)
# --------------------------------------------------------------------------

def _tokens(seed, BH, n, D):
    r = np.random.default_rng(seed)
    return (r.standard_normal((BH, n, D)) * 2).astype(np.float16).view(
        np.uint16)


def pin_cache_flush_counts_from_pages(o):
    """KIVI blog post on the fused Metal kernels, "The full end-to-end
    record", Generation 1: with residual_length = group = 32, prompts of
    559, 2059 and 8209 tokens flush 512, 2016 and 8160 tokens per layer.
    The same counts whether the prompt arrives at once, in prefill chunks of
    2048 tokens (the chunking the post names) or token by token."""
    for prompt, flushed in ((559, 512), (2059, 2016), (8209, 8160)):
        x = _tokens(prompt, 1, prompt, 8)
        for chunk in (prompt, 2048, 1):
            c = o.cache(1, 8, 8320, 32, 32, 32, 2, FP16)
            for a in range(0, prompt, chunk):
                c.append(x[:, a:a + chunk], x[:, a:a + chunk])
            assert (c.T, c.Q) == (prompt, flushed), (prompt, chunk, c.Q)


def pin_cache_decode_flush_cadence(o):
    """Same post, "Four benchmarks that lied", Lie #2: 240 decode tokens
    after a 2k prompt make 7 flushes (R = G = 32; the 2059-token prompt of
    Generation 1)."""
    c = o.cache(1, 8, 2400, 32, 32, 32, 2, FP16)
    x = _tokens(7, 1, 2059 + 240, 8)
    c.append(x[:, :2059], x[:, :2059])
    events = 0
    for t in range(2059, 2059 + 240):
        q = c.Q
        c.append(x[:, t:t + 1], x[:, t:t + 1])
        assert c.Q in (q, q + 32)
        events += c.Q != q
    assert events == 7, events


def pin_cache_window_invariant(o):
    """After every append the unquantized tail holds the R most recent
    tokens and fewer than R + G in all: Q is a multiple of G, and
    R <= T - Q < R + G once T >= R + G (before that nothing is flushed);
    with R = 0 every whole group is flushed at once."""
    for R, G in ((32, 32), (0, 8), (5, 16), (40, 32)):
        c = o.cache(2, 16, 600, R, G, 16, 4, BF16)
        rng = np.random.default_rng(R + G)
        x = _tokens(3, 2, 600, 16)
        t = 0
        while t < 560:
            n = min(int(rng.choice([1, 1, 2, 7, 31, 64])), 600 - t)
            c.append(x[:, t:t + n], x[:, t:t + n])
            t += n
            assert c.T == t and c.Q % G == 0
            if t < R + G:
                assert c.Q == 0, (R, G, t, c.Q)
            else:
                assert R <= t - c.Q < R + G, (R, G, t, c.Q)


def pin_cache_equals_prefix_quantization(o):
    """Flushing group by group as tokens age out is the same as quantizing
    the whole flushed prefix at once (key groups are aligned at token 0 and
    independent; values are per token): codes and params of tokens [0, Q)
    equal the plain quantizers on the history prefix, untouched storage past
    Q stays zero, and the history holds every appended token."""
    for dtype, bits, Gk, Gv, R in ((FP16, 2, 32, 32, 32), (BF16, 4, 16, 64, 7),
                                   (FP16, 1, 8, 8, 0)):
        BH, D, S_max = 3, 64, 300
        c = o.cache(BH, D, S_max, R, Gk, Gv, bits, dtype)
        x = _tokens(11 + bits, BH, S_max, D)
        y = _tokens(12 + bits, BH, S_max, D)
        t = 0
        for n in (1, 5, 40, 1, 1, 70, 33, 2, 90, 3):
            c.append(x[:, t:t + n], y[:, t:t + n])
            t += n
        Q = c.Q
        assert Q > 0 and np.array_equal(c.k[:, :t], x[:, :t]) \
            and np.array_equal(c.v[:, :t], y[:, :t])
        ck, sk, zk = o.quant_keys(np.ascontiguousarray(x[:, :Q]), dtype, bits,
                                  Gk)
        cv, sv, zv = o.quant_values(np.ascontiguousarray(y[:, :Q]), dtype,
                                    bits, Gv)
        assert np.array_equal(c.k_codes[:, :Q], ck)
        assert np.array_equal(c.k_scale[:, :Q // Gk].view(np.uint32),
                              sk.view(np.uint32))
        assert np.array_equal(c.k_zero[:, :Q // Gk].view(np.uint32),
                              zk.view(np.uint32))
        assert np.array_equal(c.v_codes[:, :Q], cv)
        assert np.array_equal(c.v_scale[:, :Q].view(np.uint32),
                              sv.view(np.uint32))
        assert np.array_equal(c.v_zero[:, :Q].view(np.uint32),
                              zv.view(np.uint32))
        assert not c.k_codes[:, Q:].any() and not c.v_codes[:, Q:].any()
        assert not c.k_scale[:, Q // Gk:].any() and not c.v_scale[:, Q:].any()


def pin_cache_rejects_overflow(o):
    """An append past S_max is refused and leaves the cache unchanged."""
    c = o.cache(1, 8, 64, 8, 8, 8, 2, FP16)
    x = _tokens(1, 1, 70, 8)
    c.append(x[:, :60], x[:, :60])
    T, Q = c.T, c.Q
    try:
        c.append(x[:, 60:70], x[:, 60:70])
    except ValueError:
        pass
    else:
        raise AssertionError("append past S_max accepted")
    assert (c.T, c.Q) == (T, Q)


# --------------------------------------------------------------------------
# Decode attention over the cache (reading the compressed store)
# --------------------------------------------------------------------------

def _sdpa_f64(q, k, v, sm_scale):
    """torch's scaled_dot_product_attention on the CPU in float64 (a library
    routine independent of the oracle's own softmax)."""
    import torch
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, None], torch.from_numpy(k)[:, None],
        torch.from_numpy(v)[:, None], scale=float(sm_scale))
    return out[:, 0].numpy()


def pin_attend_matches_library_sdpa(o):
    """KIVI blog post on the fused Metal kernels, "So why does the kernel
    ship?": attention that reads the packed codes must equal attention over
    the dequantized cache.  The oracle's attend() against torch's SDPA
    (float64, CPU) on the K, V that the plain dequantizers give for tokens
    [0, Q) and the exact tokens [Q, T); with several query heads per KV
    head, and with nothing quantized yet (T < R + G)."""
    for T, R in ((300, 32), (40, 32)):
        c = o.cache(3, 64, 320, R, 32, 32, 2, FP16)
        k, v = _tokens(21, 3, T, 64), _tokens(22, 3, T, 64)
        c.append(k, v)
        q = _tokens(23, 3, 4, 64)
        sm = 1.0 / 8.0
        got = c.attend(q, sm)
        K = o.widen(c.dequantized("K"), FP16).astype(np.float64)
        V = o.widen(c.dequantized("V"), FP16).astype(np.float64)
        Qf = o.widen(q, FP16).astype(np.float64)
        ref = _sdpa_f64(Qf, K, V, sm)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), (T, R)
        # the quantized part really is the dequantized store ...
        Qn = c.Q
        deq = o.dequant_keys(c.k_codes[:, :Qn], c.k_scale[:, :Qn // 32],
                             c.k_zero[:, :Qn // 32], (3, Qn, 64), 2, 32, FP16)
        assert np.array_equal(c.dequantized("K")[:, :Qn], deq)
        # ... and the rest the exact tokens
        assert np.array_equal(c.dequantized("V")[:, Qn:], v[:, Qn:T])


def pin_attend_closed_forms(o):
    """q = 0 gives equal weights, so the output is the mean of the V rows;
    a single cached token gives that token's V; the output is a convex
    combination of V rows (within their per-channel min and max)."""
    c = o.cache(2, 32, 64, 4, 8, 8, 4, BF16)
    k, v = _tokens(31, 2, 50, 32), _tokens(32, 2, 50, 32)
    c.append(k, v)
    V = o.widen(c.dequantized("V"), BF16).astype(np.float64)
    zero_q = np.zeros((2, 3, 32), np.uint16)
    got = c.attend(zero_q, 0.2)
    assert np.allclose(got, V.mean(axis=1)[:, None, :].repeat(3, 1),
                       rtol=1e-12, atol=1e-12)
    q = _tokens(33, 2, 3, 32)
    got = c.attend(q, 0.2)
    assert (got <= V.max(axis=1)[:, None, :] + 1e-12).all()
    assert (got >= V.min(axis=1)[:, None, :] - 1e-12).all()
    one = o.cache(1, 32, 8, 4, 8, 8, 2, FP16)
    one.append(k[:1, :1], v[:1, :1])
    got = one.attend(q[:1], 0.2)
    vf = o.widen(v[:1, :1], FP16).astype(np.float64)
    assert np.allclose(got, vf.repeat(3, 1), rtol=0, atol=0)


def _grid_tokens(rng, BH, n, D, bits, G, keys):
    """fp16 tokens [BH, n, D] that lie on their quantization groups' grids:
    every key group (G tokens of one channel; keys=True) or value group
    (G channels of one token) has its own zero (a multiple of 1/4 in
    [-4, 4)) and power-of-two step (1/4 .. 1/32), and holds both code 0
    and code 2^bits - 1, so the quantizer must return exactly that zero and
    step and the element's own code."""
    maxc = 2 ** bits - 1
    codes = rng.integers(0, maxc + 1, size=(BH, n, D))
    if keys:
        ng = (n + G - 1) // G
        codes[:, 0::G, :] = 0
        codes[:, 1::G, :] = maxc
        zero = rng.integers(-16, 16, size=(BH, ng, D)) * 0.25
        step = 2.0 ** -rng.integers(2, 6, size=(BH, ng, D)).astype(float)
        zero = np.repeat(zero, G, axis=1)[:, :n]
        step = np.repeat(step, G, axis=1)[:, :n]
    else:
        ng = (D + G - 1) // G
        codes[:, :, 0::G] = 0
        codes[:, :, 1::G] = maxc
        zero = rng.integers(-16, 16, size=(BH, n, ng)) * 0.25
        step = 2.0 ** -rng.integers(2, 6, size=(BH, n, ng)).astype(float)
        zero = np.repeat(zero, G, axis=2)[:, :, :D]
        step = np.repeat(step, G, axis=2)[:, :, :D]
    f = zero + codes * step
    x = f.astype(np.float16)
    assert np.array_equal(x.astype(np.float64), f)     # exact in fp16
    return x.view(np.uint16)


def pin_attend_exact_reconstruction(o):
    """kivi_cache_attend's contract reconstructs a quantized token as
    code * scale + zero of its own group, never rounded to 16 bits.  On
    tokens that lie on their groups' grids (each group with its own zero and
    step) that reconstruction must give back the stored tokens exactly, so
    the oracle's reconstructed() picks each token's codes and each group's
    params; and on random tokens, rounded to fp16, it is within one ulp of
    the plain dequantizers' output (which round once from fp32) and equal
    to it almost everywhere."""
    rng = np.random.default_rng(61)
    BH, D, T = 2, 64, 300
    for bits, Gk, Gv in ((2, 32, 32), (4, 16, 64), (2, 8, 16)):
        kg = _grid_tokens(rng, BH, T, D, bits, Gk, keys=True)
        vg = _grid_tokens(rng, BH, T, D, bits, Gv, keys=False)
        c = o.cache(BH, D, T, 32, Gk, Gv, bits, FP16)
        c.append(kg, vg)
        assert c.Q > 0
        for which, x in (("K", kg), ("V", vg)):
            want = o.widen(x[:, :c.T], FP16).astype(np.float64)
            assert np.array_equal(c.reconstructed(which), want), (bits, which)
        q = _tokens(62, BH, 3, D)
        got = c.attend_exact(q, 0.125)
        ref = _sdpa_f64(o.widen(q, FP16).astype(np.float64),
                        o.widen(kg, FP16).astype(np.float64),
                        o.widen(vg, FP16).astype(np.float64), 0.125)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    c = o.cache(3, 64, 320, 32, 32, 32, 2, FP16)
    c.append(_tokens(63, 3, 300, 64), _tokens(64, 3, 300, 64))
    for which in ("K", "V"):
        r16 = c.reconstructed(which).astype(np.float16).view(np.uint16)
        d = c.dequantized(which)
        ia = np.where(r16 & 0x8000, 0x8000 - (r16 & 0x7FFF), 0x8000 + r16)
        ib = np.where(d & 0x8000, 0x8000 - (d & 0x7FFF), 0x8000 + d)
        diff = np.abs(ia.astype(np.int64) - ib)
        assert diff.max() <= 1 and (diff == 0).mean() > 0.99, which


def pin_attend_exact_matches_library_sdpa(o):
    """attend_exact() against torch's SDPA (float64, CPU) over
    reconstructed() keys and values, with sm_scale rounded to fp32 as the
    call receives it; bf16 and fp16, with and without quantized tokens."""
    for dtype, T, R, bits, Gk, Gv in ((FP16, 300, 32, 2, 32, 32),
                                      (BF16, 200, 5, 4, 16, 64),
                                      (BF16, 40, 32, 2, 32, 32)):
        c = o.cache(2, 64, 320, R, Gk, Gv, bits, dtype)
        c.append(_tokens(71, 2, T, 64), _tokens(72, 2, T, 64))
        q = _tokens(73, 2, 4, 64)
        sm = 1.0 / np.sqrt(3.0)
        got = c.attend_exact(q, sm)
        ref = _sdpa_f64(o.widen(q, dtype).astype(np.float64),
                        c.reconstructed("K"), c.reconstructed("V"),
                        float(np.float32(sm)))
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), (dtype, T)
        assert float(np.float32(sm)) != sm     # the fp32 rounding is real


# --------------------------------------------------------------------------
# KIVI-Sink (PyPI page of VeloxQuant-MLX 0.24.1, section "KVSink-adapted
# sink protection")
# --------------------------------------------------------------------------

def _sink_scores_numpy(o, k, dtype, H):
    """The score written out with numpy: per head the squares accumulated in
    channel order with one rounding per step, the fp32 square root, the
    head-order sum and one division by H.  x*x is exact in float64 and a
    float64 sum or square root rounded again to float32 equals the single
    float32 rounding (53 >= 2*24 + 2), so this is bit-exact."""
    f = o.widen(k, dtype).astype(np.float64)
    BH, S, D = f.shape
    ss = np.zeros((BH, S), np.float32)
    for d in range(D):
        ss = (f[:, :, d] * f[:, :, d] + ss.astype(np.float64)).astype(np.float32)
    norm = np.sqrt(ss.astype(np.float64)).astype(np.float32).reshape(BH // H, H, S)
    total = np.zeros((BH // H, S), np.float32)
    for h in range(H):
        total = total + norm[:, h]
    return total / np.float32(H)


def _planted_sinks(seed, B, H, S, D, positions, factor=30.0, dtype=FP16):
    """Keys N(0,1) whose sink positions (per sequence) carry keys `factor`
    times larger in every head."""
    r = np.random.default_rng(seed)
    x = r.standard_normal((B, H, S, D)).astype(np.float32)
    for b in range(B):
        x[b, :, positions[b]] *= factor
    x = x.reshape(B * H, S, D)
    if dtype == FP16:
        return x.astype(np.float16).view(np.uint16)
    u = x.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def pin_sink_scores(o):
    """The score is the mean over heads of the key's L2 norm: Pythagorean
    rows give exact norms (3-4-5: heads of norm 5 and 10 average to 7.5),
    and on random fp16 / bf16 keys the oracle equals the numpy
    re-derivation bit for bit."""
    rows = np.zeros((2, 1, 8), np.float32)      # B = 1, H = 2, S = 1, D = 8
    rows[0, 0, :2] = (3.0, 4.0)
    rows[1, 0, 5:7] = (6.0, 8.0)
    got = o.sink_scores(_f16_bits(rows), FP16, 2)
    assert got.shape == (1, 1) and got[0, 0] == np.float32(7.5), got
    r = np.random.default_rng(71)
    for dtype in (FP16, BF16):
        k = _rand_tensor(r, 6, 37, 24, dtype)
        for H in (1, 3):
            got = o.sink_scores(k, dtype, H)
            exp = _sink_scores_numpy(o, k, dtype, H)
            assert np.array_equal(got.view(np.uint32), exp.view(np.uint32)), (dtype, H)
            # and close to the float64 definition
            f = o.widen(k, dtype).astype(np.float64).reshape(6 // H, H, 37, 24)
            ref = np.sqrt((f * f).sum(axis=3)).mean(axis=1)
            assert np.allclose(got, ref, rtol=2.0**-24 * (24 + H + 4), atol=0)


def pin_sink_select(o):
    """Selection equals numpy's stable descending argsort (the lower position
    first among equal scores): random scores, planted ties, n_sink = 0 and
    n_sink = S."""
    r = np.random.default_rng(72)
    sc = r.random((3, 50)).astype(np.float32)
    sc[1, [4, 9, 30]] = np.float32(2.0)         # a three-way tie at the top
    sc[2, 10:20] = np.float32(0.5)              # a run of ties in the middle
    for n in (0, 1, 3, 7, 50):
        got = o.sink_select(sc, n)
        exp = np.argsort(-sc, axis=1, kind="stable")[:, :n].astype(np.int32)
        assert np.array_equal(got, exp), n
    assert np.array_equal(o.sink_select(sc, 3)[1], [4, 9, 30])
    try:
        o.sink_select(sc, 51)
    except ValueError:
        pass
    else:
        raise AssertionError("n_sink > S accepted")


def pin_sink_worked_group(o):
    """A spike among small keys (one channel, a group of four tokens
    [0, 1, 0.5, 100], 2 bits).  Plain KIVI: scale 100/3, codes [0, 0, 0, 3],
    so every neighbour reconstructs to 0.  With the spike as a sink: zero 0,
    scale RN(1/3) = 0x3EAAAAAB, codes [0, 3, 2, 0] (0.5 / RN(1/3) rounds to
    1.5 in fp32, then to the even 2), reconstruction [0, 1, 0.6666667] and
    the spike itself bit-exact."""
    x = _f16_bits(np.array([0.0, 1.0, 0.5, 100.0], np.float32).reshape(1, 4, 1)
                  .repeat(8, axis=2))
    idx = np.array([[3]], np.int32)
    codes, sc, z = o.quant_keys_sink_unpacked(x, FP16, 1, 2, 4, idx)
    assert codes[0, :, 0].tolist() == [0, 3, 2, 0], codes[0, :, 0]
    assert sc[0, 0, 0].view(np.uint32) == 0x3EAAAAAB and z[0, 0, 0] == 0.0
    plain, psc, _ = o.quant_keys_unpacked(x, FP16, 2, 4)
    assert plain[0, :, 0].tolist() == [0, 0, 0, 3]
    assert psc[0, 0, 0] == np.float32(100.0) / np.float32(3.0)
    rec = o.widen(o.sink_recon(x, FP16, 1, 2, 4, idx), FP16)[0, :, 0]
    assert rec.tolist() == [0.0, 1.0, float(np.float16(np.float32(2) * np.float32(1 / 3))), 100.0]


def pin_sink_quant_bruteforce(o):
    """Keys with sinks on ragged shapes against numpy float32: each group's
    zero and scale are numpy's min, max and (max - min) / (2^b - 1) over the
    group's non-sink tokens (+0 for a zero min or max), codes are
    rint((x - zero) / scale) clipped (0 when scale is 0) and a sink's code is
    0; a group of sinks only has scale 0 and zero 0.  Sink lists name each
    sequence's own tokens (H = 2 heads per sequence)."""
    r = np.random.default_rng(73)
    B, H, S, D, G, bits = 2, 2, 19, 8, 4, 2
    x = _rand_tensor(r, B * H, S, D, FP16)
    idx = np.array([[0, 1, 2, 3, 9, 18], [17, 5, 6, 40, -1, 6]], np.int32)
    codes, sc, z = o.quant_keys_sink_unpacked(x, FP16, H, bits, G, idx)
    f = o.widen(x, FP16)
    L = np.float32(2**bits - 1)
    for bh in range(B * H):
        sinks = set(int(s) for s in idx[bh // H])
        for g in range((S + G - 1) // G):
            toks = [s for s in range(g * G, min(g * G + G, S))]
            keep = [s for s in toks if s not in sinks]
            for d in range(D):
                if keep:
                    v = f[bh, keep, d]
                    mn, mx = np.float32(v.min()) + np.float32(0), np.float32(v.max()) + np.float32(0)
                    es, ez = np.float32(mx - mn) / L, mn
                else:
                    es, ez = np.float32(0), np.float32(0)
                assert sc[bh, g, d].view(np.uint32) == es.view(np.uint32), (bh, g, d)
                assert z[bh, g, d].view(np.uint32) == ez.view(np.uint32), (bh, g, d)
                for s in toks:
                    if s in sinks or es == 0:
                        e = 0
                    else:
                        t = np.float32(np.float32(f[bh, s, d] - ez) / es)
                        e = int(min(max(np.rint(t), 0), 2**bits - 1))
                    assert codes[bh, s, d] == e, (bh, s, d, codes[bh, s, d], e)
    # the second sequence's group 1 is tokens 4..7 with sinks 5 and 6; its
    # first group has none; the first sequence's group 0 is all sinks
    assert (sc[:2, 0] == 0).all() and (z[:2, 0] == 0).all()


def pin_sink_zero_is_plain_kivi(o):
    """With no sinks the variant is plain KIVI bit for bit (PyPI page,
    KVSink section: n_sink_tokens = 0 reproduces plain KIVI)."""
    r = np.random.default_rng(74)
    for dtype, bits, G in ((FP16, 2, 32), (BF16, 4, 8)):
        x = _rand_tensor(r, 4, 70, 16, dtype)
        got = o.quant_keys_sink(x, dtype, 2, bits, G, np.zeros((2, 0), np.int32))
        exp = o.quant_keys(x, dtype, bits, G)
        for a, b in zip(got, exp):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def pin_sink_claims(o):
    """The pages' evidence for the variant on planted-sink data: sinks come
    back bit-exact while the others are quantized; the sink-protected MSE is
    below plain KIVI's at the same bit width; and with sinks away from the
    front, dynamic selection beats keeping the first n tokens at the same
    fp16 budget.  Also gather then restore is the identity on sink rows."""
    B, H, S, D, n = 2, 4, 256, 32, 4
    pos = [np.array([40, 97, 150, 201]), np.array([3, 64, 130, 250])]
    x = _planted_sinks(75, B, H, S, D, pos)
    idx = o.sink_select(o.sink_scores(x, FP16, H), n)
    for b in range(B):
        assert sorted(idx[b].tolist()) == sorted(pos[b].tolist()), idx[b]
    f = o.widen(x, FP16).astype(np.float64)

    def mse(rec):
        return float(((o.widen(rec, FP16) - f) ** 2).mean())

    rec = o.sink_recon(x, FP16, H, 2, 32, idx)
    for bh in range(B * H):
        assert np.array_equal(rec[bh, idx[bh // H]], x[bh, idx[bh // H]])
    plain_codes, psc, pz = o.quant_keys(x, FP16, 2, 32)
    plain = o.dequant_keys(plain_codes, psc, pz, x.shape, 2, 32, FP16)
    first = np.tile(np.arange(n, dtype=np.int32), (B, 1))
    front = o.sink_recon(x, FP16, H, 2, 32, first)
    assert mse(rec) < 0.5 * mse(plain), (mse(rec), mse(plain))
    assert mse(rec) < mse(front), (mse(rec), mse(front))
    assert not np.array_equal(rec, x)
    # gather / restore
    xs = o.sink_gather(x, H, idx)
    for bh in range(B * H):
        assert np.array_equal(xs[bh], x[bh, idx[bh // H]])
    back = o.sink_restore(xs, H, idx, np.zeros_like(x))
    mask = np.zeros(x.shape[:2], bool)
    for bh in range(B * H):
        mask[bh, idx[bh // H]] = True
    assert np.array_equal(back[mask], x[mask]) and not back[~mask].any()
    # positions outside [0, S) leave their rows alone (the input sits in a
    # larger buffer, so a row read past the end stays inside it)
    big = np.concatenate([x, np.ones((1, S, D), np.uint16)])
    odd_g = np.array([[S, int(idx[0, 0])], [-1, S]], np.int32)
    xs2 = o.sink_gather(big[:B * H], H, odd_g)
    assert not xs2[:, 0].any() and not xs2[H:, 1].any()
    for bh in range(H):
        assert np.array_equal(xs2[bh, 1], x[bh, idx[0, 0]])
    odd = np.array([[-1, S], [S + 5, -7]], np.int32)     # nothing in range
    assert not o.sink_restore(np.ones((B * H, 2, D), np.uint16), H, odd,
                              np.zeros_like(x)).any()


# --------------------------------------------------------------------------
# Per-token mixed precision (PyPI page of VeloxQuant-MLX 0.24.1, section
# "ZipCache-adapted -- saliency-adaptive per-token mixed precision")
# --------------------------------------------------------------------------

def pin_mixed_partition(o):
    """The hi set is the first n_hi positions in the order (score
    descending, position ascending), i.e. numpy's stable descending argsort;
    both lists ascending and together a permutation of the positions; ties,
    n_hi = 0 and n_hi = S included."""
    r = np.random.default_rng(81)
    sc = r.random((3, 90)).astype(np.float32)
    sc[1, 10:40] = np.float32(0.7)               # a long run of ties
    sc[2] = np.float32(0.25)                      # everything tied
    for n in (0, 1, 17, 45, 89, 90):
        hi, lo = o.partition_top(sc, n)
        exp = np.sort(np.argsort(-sc, axis=1, kind="stable")[:, :n], axis=1)
        assert np.array_equal(hi, exp), n
        for b in range(3):
            assert np.array_equal(np.sort(np.concatenate([hi[b], lo[b]])),
                                  np.arange(90))
            assert (np.diff(lo[b]) > 0).all()
    assert o.partition_top(sc, 5)[0][2].tolist() == [0, 1, 2, 3, 4]


def pin_mixed_rows_are_gathered_tensors(o):
    """Quantizing listed rows equals quantizing the tensor numpy gathers
    (x[bh, pos[bh // H]]) with the plain quantizers; listing every position
    is plain KIVI; the row dequantizers write exactly the listed rows, each
    equal to the plain dequant of the gathered tensor."""
    r = np.random.default_rng(82)
    B, H, S, D = 2, 3, 61, 24
    x = _rand_tensor(r, B * H, S, D, FP16)
    pos = np.sort(np.stack([r.choice(S, 23, replace=False) for _ in range(B)]),
                  axis=1).astype(np.int32)
    g = np.stack([x[bh, pos[bh // H]] for bh in range(B * H)])
    for keys, bits, G in ((True, 4, 8), (False, 2, 8), (True, 2, 32), (False, 4, 16)):
        q = o.quant_keys_rows if keys else o.quant_values_rows
        pq = o.quant_keys if keys else o.quant_values
        got = q(x, FP16, H, bits, G, pos)
        exp = pq(g, FP16, bits, G)
        for a, b in zip(got, exp):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (keys, bits, G)
        allpos = np.tile(np.arange(S, dtype=np.int32), (B, 1))
        for a, b in zip(q(x, FP16, H, bits, G, allpos), pq(x, FP16, bits, G)):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
        dq = o.dequant_keys_rows if keys else o.dequant_values_rows
        pdq = o.dequant_keys if keys else o.dequant_values
        base = np.full(x.shape, 0x7777, np.uint16)
        out = dq(*got, x.shape, H, bits, G, pos, FP16, base)
        rec = pdq(*exp, g.shape, bits, G, FP16)
        want = base.copy()
        for bh in range(B * H):
            want[bh, pos[bh // H]] = rec[bh]
        assert np.array_equal(out, want), (keys, bits, G)
    bad = pos.copy()
    bad[1, 3] = S
    try:
        o.quant_keys_rows(x, FP16, H, 2, 8, bad)
    except ValueError:
        pass
    else:
        raise AssertionError("position outside [0, S) accepted")


def pin_mixed_claims(o):
    """The page's evidence for the variant: the saliency mask is the top
    fraction by key norm; 4-bit per-channel quantization of unit-norm
    Gaussian keys has cosine > 0.995 and 2-bit > 0.8; hi_fraction 1 beats
    hi_fraction 0; mixed bits sit between all-lo and all-hi in error and in
    bytes (compressed <= fp16, mixed >= all-lo), with average bits in
    [lo_bits, hi_bits]."""
    r = np.random.default_rng(83)
    B, H, S, D, G = 2, 2, 320, 64, 32
    f = r.standard_normal((B * H, S, D)).astype(np.float32)
    f /= np.linalg.norm(f, axis=2, keepdims=True)
    f *= r.uniform(0.5, 3.0, size=(B, 1, S, 1)).repeat(H, 1).reshape(B * H, S, 1).astype(np.float32)
    x = f.astype(np.float16).view(np.uint16)
    fx = o.widen(x, FP16).astype(np.float64)
    norms = np.sqrt((fx ** 2).sum(axis=2)).reshape(B, H, S).mean(axis=1)
    n_hi = int(0.2 * S)
    hi, lo = o.partition_top(o.sink_scores(x, FP16, H), n_hi)
    for b in range(B):
        assert np.array_equal(hi[b], np.sort(np.argsort(-norms[b])[:n_hi]))

    def err(rec):
        e = o.widen(rec, FP16).astype(np.float64) - fx
        return float((e ** 2).mean())

    def cos(rec):
        y = o.widen(rec, FP16).astype(np.float64)
        return float(((y * fx).sum(2) / np.linalg.norm(y, axis=2)
                      / np.linalg.norm(fx, axis=2)).mean())

    # the page's cosines are for unit-norm Gaussian keys
    u = (f / np.linalg.norm(f, axis=2, keepdims=True)).astype(np.float16).view(np.uint16)
    fu = o.widen(u, FP16).astype(np.float64)

    def cos_u(rec):
        y = o.widen(rec, FP16).astype(np.float64)
        return float(((y * fu).sum(2) / np.linalg.norm(y, axis=2)
                      / np.linalg.norm(fu, axis=2)).mean())

    c4 = cos_u(o.mixed_recon(u, FP16, H, S, 4, 2, G, True))
    c2 = cos_u(o.mixed_recon(u, FP16, H, 0, 4, 2, G, True))
    assert c4 > 0.995 and c2 > 0.8, (c4, c2)
    rec4 = o.mixed_recon(x, FP16, H, S, 4, 2, G, True)        # all hi
    rec2 = o.mixed_recon(x, FP16, H, 0, 4, 2, G, True)        # all lo
    mix = o.mixed_recon(x, FP16, H, n_hi, 4, 2, G, True)
    assert err(rec4) < err(mix) < err(rec2)
    assert cos(rec4) > cos(mix) > cos(rec2)
    # plain KIVI at one width is the mixed variant with an empty other set
    pc, psc, pz = o.quant_keys(x, FP16, 4, G)
    assert np.array_equal(rec4, o.dequant_keys(pc, psc, pz, x.shape, 4, G, FP16))

    def nbytes(n, bits):
        if n == 0:
            return 0
        c, sc, z = o.quant_keys_rows(x, FP16, H, bits, G, np.tile(
            np.arange(n, dtype=np.int32), (B, 1)))
        return c.nbytes + sc.nbytes + z.nbytes

    mixed = nbytes(n_hi, 4) + nbytes(S - n_hi, 2)
    assert nbytes(S, 2) <= mixed <= nbytes(S, 4) <= x.nbytes
    avg = (n_hi * 4 + (S - n_hi) * 2) / S
    assert 2 <= avg <= 4


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
