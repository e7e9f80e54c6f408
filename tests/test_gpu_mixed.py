"""GPU parity of per-token mixed precision (kivi_partition_top,
kivi_quant_{keys,values}_rows, kivi_dequant_{keys,values}_rows) against the
oracle: bit-exact position lists, codes, fp32 params and reconstructions.

Small cases cover ties, n_hi = 0 and S, sequence lengths that are not a
multiple of the partition's block, ragged key groups of a set, bits 1 to 8
and every value-group form; the full-size prompt (14 x 8 KV heads x 32768
tokens, 20% at 4 bits) runs in the benchmark's launch shape and is compared
on sampled key groups and value rows."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle                                              # noqa: E402
import workloads as W                                      # noqa: E402
from gpu_util import (FP16, BF16, TORCH_DT, assert_codes_equal,   # noqa: E402
                      assert_f32_bits_equal, assert_recon_equal, bits16,
                      by_blocks, host, say, to_dev, to_dev_raw)


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_quantization_kivi_amd as K
    return K


@pytest.fixture(scope="module")
def O():
    return oracle.default()


def _x(seed, BH, S, D, dtype):
    r = np.random.default_rng(seed)
    x = r.standard_normal((BH, S, D)).astype(np.float32)
    x *= r.uniform(0.3, 3.0, size=(BH, S, 1)).astype(np.float32)
    x[:, :, r.choice(D, size=max(1, D // 32), replace=False)] *= 10.0
    if dtype == FP16:
        return x.astype(np.float16).view(np.uint16)
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16)
    return t.numpy().view(np.uint16)


def _ix(a):
    return torch.from_numpy(np.asarray(a, np.int64))


PART_CASES = [(3, 90, 17), (2, 5000, 1000), (1, 40000, 8000), (4, 1024, 0),
              (2, 777, 777), (2, 1025, 1), (3, 3000, 2999)]


@pytest.mark.parametrize("case", PART_CASES, ids=lambda c: "x".join(map(str, c)))
def test_partition_matches_oracle(K, O, case):
    B, S, n = case
    say(f"[partition {case}]")
    r = np.random.default_rng(91)
    sc = r.random((B, S)).astype(np.float32)
    sc[0, : S // 3] = np.float32(0.5)               # a long run of ties
    if B > 1:
        sc[1] = np.round(sc[1] * 8) / 8              # few distinct values
    sc[-1, S // 2] = np.float32(-0.0)
    sc[-1, S // 3] = np.float32(0.0)
    hi, lo = K.kivi_partition_top(to_dev_raw(sc), n)
    torch.cuda.synchronize()
    ehi, elo = O.partition_top(sc, n)
    assert np.array_equal(host(hi), ehi)
    assert np.array_equal(host(lo), elo)


ROW_CASES = [
    # (B, H, S, D, n, bits, G_k, G_v, dtype)
    (2, 4, 300, 128, 61, 4, 32, 32, FP16),
    (2, 4, 300, 128, 239, 2, 32, 32, FP16),
    (3, 2, 70, 64, 19, 1, 8, 8, BF16),
    (1, 3, 100, 256, 100, 8, 5, 16, FP16),
    (2, 1, 50, 32, 33, 2, 16, 64, BF16),
    (1, 2, 40, 8, 7, 4, 1, 8, FP16),
    # whole key groups only: every wave of the key dequantizer stages its
    # codes through LDS (2, 1 and 4 bits; 4, 8 and 2 groups per wave)
    (2, 4, 300, 128, 256, 2, 32, 32, FP16),
    (2, 2, 200, 64, 128, 1, 16, 16, BF16),
    (1, 2, 300, 256, 64, 4, 32, 64, FP16),
]


@pytest.mark.parametrize("case", ROW_CASES, ids=lambda c: "x".join(map(str, c)))
def test_rows_match_oracle(K, O, case):
    B, H, S, D, n, bits, Gk, Gv, dtype = case
    say(f"[rows {case}]")
    x = _x(92, B * H, S, D, dtype)
    r = np.random.default_rng(93)
    pos = np.sort(np.stack([r.choice(S, n, replace=False) for _ in range(B)]),
                  axis=1).astype(np.int32)
    xd, pd = to_dev(x, dtype), to_dev_raw(pos)
    for keys, G in ((True, Gk), (False, Gv)):
        q = K.kivi_quant_keys_rows if keys else K.kivi_quant_values_rows
        dq = K.kivi_dequant_keys_rows if keys else K.kivi_dequant_values_rows
        codes, scale, zero = q(xd, pd, bits, G, H=H)
        out = torch.full((B * H, S, D), 0.0, dtype=TORCH_DT[dtype], device="cuda")
        dq(codes, scale, zero, pd, out, bits, G, H=H)
        torch.cuda.synchronize()
        oq = O.quant_keys_rows if keys else O.quant_values_rows
        odq = O.dequant_keys_rows if keys else O.dequant_values_rows
        wc, ws, wz = oq(x, dtype, H, bits, G, pos)
        assert_codes_equal(host(codes), wc, f"codes keys={keys}")
        assert_f32_bits_equal(host(scale), ws, f"scale keys={keys}")
        assert_f32_bits_equal(host(zero), wz, f"zero keys={keys}")
        want = odq(wc, ws, wz, x.shape, H, bits, G, pos, dtype)
        assert_recon_equal(bits16(out), want, f"recon keys={keys}")


def test_mixed_end_to_end(K, O):
    """Scores, partition, both sets quantized and dequantized back into one
    tensor: equal to the oracle's mixed reconstruction, keys and values."""
    B, H, S, D, n_hi = 2, 4, 500, 128, 100
    k = _x(94, B * H, S, D, FP16)
    v = _x(95, B * H, S, D, FP16)
    kd, vd = to_dev(k, FP16), to_dev(v, FP16)
    score = K.kivi_key_scores(kd, H=H)
    hi, lo = K.kivi_partition_top(score, n_hi)
    outs = []
    for x, keys in ((kd, True), (vd, False)):
        out = torch.zeros_like(x)
        for pos, bits in ((hi, 4), (lo, 2)):
            q = K.kivi_quant_keys_rows if keys else K.kivi_quant_values_rows
            dq = K.kivi_dequant_keys_rows if keys else K.kivi_dequant_values_rows
            c, s, z = q(x, pos, bits, 32, H=H)
            dq(c, s, z, pos, out, bits, 32, H=H)
        outs.append(out)
    torch.cuda.synchronize()
    assert_recon_equal(bits16(outs[0]), O.mixed_recon(k, FP16, H, n_hi, 4, 2, 32, True), "keys")
    assert_recon_equal(bits16(outs[1]), O.mixed_recon(v, FP16, H, n_hi, 4, 2, 32, k), "values")


@pytest.mark.timeout(900)
def test_mixed_full_size(K, O):
    """The benchmark's step on the benchmark's prompt, compared in full:
    every score, both position lists, the codes and params of every key
    group and value row of both sets (keys from K, values from V), and the
    key and value tensors both sets' dequantizers wrote back, against the
    oracle run over blocks of sequences on a thread pool."""
    mw = W.MIXED_WORKLOADS["mixed-prefill"]
    w = mw.tokens()
    B, H, S, D, n_hi = mw.B, mw.H, mw.S, mw.D, mw.n_hi
    say(f"[mixed full size {mw.name}] generating")
    k = W.gen_tensor(w, "K")
    v = W.gen_tensor(w, "V")
    kd, vd = to_dev(k, w.dtype), to_dev(v, w.dtype)
    score = K.kivi_key_scores(kd, H=H)
    hi, lo = K.kivi_partition_top(score, n_hi)
    sets = []
    k_out, v_out = torch.zeros_like(kd), torch.zeros_like(vd)
    for name, pos, bits in (("hi", hi, mw.hi_bits), ("lo", lo, mw.lo_bits)):
        kq = K.kivi_quant_keys_rows(kd, pos, bits, mw.group_k, H=H)
        vq = K.kivi_quant_values_rows(vd, pos, bits, mw.group_v, H=H)
        K.kivi_dequant_keys_rows(*kq, pos, k_out, bits, mw.group_k, H=H)
        K.kivi_dequant_values_rows(*vq, pos, v_out, bits, mw.group_v, H=H)
        sets.append((name, host(pos), bits, [host(t) for t in kq],
                     [host(t) for t in vq]))
    torch.cuda.synchronize()
    sc, k_out, v_out = host(score), bits16(k_out), bits16(v_out)
    del kd, vd
    torch.cuda.empty_cache()
    say(f"[mixed full size] oracle over all {B} sequences")

    def rows(a, b):
        return slice(a * H, b * H)

    want_sc = np.concatenate(by_blocks(B, lambda a, b: O.sink_scores(
        np.ascontiguousarray(k[rows(a, b)]), w.dtype, H)))
    assert_f32_bits_equal(sc, want_sc, "scores")
    ehi, elo = O.partition_top(want_sc, n_hi)
    assert np.array_equal(sets[0][1], ehi) and np.array_equal(sets[1][1], elo)

    def block(a, b):
        r = rows(a, b)
        ks, vs_ = np.ascontiguousarray(k[r]), np.ascontiguousarray(v[r])
        kr = vr = None
        for name, pos, bits, (kc, kscale, kz), (vc, vscale, vz) in sets:
            pb = np.ascontiguousarray(pos[a:b])
            tag = f"{name} seq[{a}:{b}]"
            wc, ws, wz = O.quant_keys_rows(ks, w.dtype, H, bits, mw.group_k, pb)
            assert_codes_equal(kc[r], wc, f"{tag} key codes")
            assert_f32_bits_equal(kscale[r], ws, f"{tag} key scale")
            assert_f32_bits_equal(kz[r], wz, f"{tag} key zero")
            kr = O.dequant_keys_rows(wc, ws, wz, ks.shape, H, bits,
                                     mw.group_k, pb, w.dtype, kr)
            wc, ws, wz = O.quant_values_rows(vs_, w.dtype, H, bits,
                                             mw.group_v, pb)
            assert_codes_equal(vc[r], wc, f"{tag} value codes")
            assert_f32_bits_equal(vscale[r], ws, f"{tag} value scale")
            assert_f32_bits_equal(vz[r], wz, f"{tag} value zero")
            vr = O.dequant_values_rows(wc, ws, wz, vs_.shape, H, bits,
                                       mw.group_v, pb, w.dtype, vr)
        assert_recon_equal(k_out[r], kr, f"key recon seq[{a}:{b}]")
        assert_recon_equal(v_out[r], vr, f"value recon seq[{a}:{b}]")

    by_blocks(B, block)
    say("[mixed full size] every score, list, group, row and recon equal")
