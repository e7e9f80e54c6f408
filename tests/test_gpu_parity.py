"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Codes (packed bytes) and fp32 scale/zero must be bit-exact; reconstructions
are compared bit-exactly as well (the stated bar is one ulp of the output
type, the path computes the same IEEE operations as the oracle).  Every
workload is compared in full: the full-size ones run on the GPU at their
real shape, in the same launch configuration the benchmark times, and the
oracle covers every (bh) slice, in contiguous blocks on a thread pool.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle                                              # noqa: E402
import workloads as W                                      # noqa: E402
from gpu_util import (FP16, BF16, assert_codes_equal,      # noqa: E402
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


# --------------------------------------------------------------------------
# one tensor, every entry point
# --------------------------------------------------------------------------

def run_all(K, x_dev, dtype, bits, gk, gv, tag):
    """All six compute entry points on one device tensor; returns host
    copies keyed by name."""
    out = {}
    say(f"[{tag}] quant keys/values bits={bits} gk={gk} gv={gv}")
    ck, sk, zk = K.kivi_quant_keys(x_dev, bits, gk)
    cv, sv, zv = K.kivi_quant_values(x_dev, bits, gv)
    say(f"[{tag}] dequant")
    odt = x_dev.dtype
    rk = K.kivi_dequant_keys(ck, sk, zk, bits, gk, out_dtype=odt)
    rv = K.kivi_dequant_values(cv, sv, zv, bits, gv, out_dtype=odt)
    say(f"[{tag}] fused")
    fk, fck, fsk, fzk = K.kivi_quant_dequant_keys(x_dev, bits, gk)
    fv, fcv, fsv, fzv = K.kivi_quant_dequant_values(x_dev, bits, gv)
    fk2 = K.kivi_quant_dequant_keys(x_dev, bits, gk, with_codes=False)
    fv2 = K.kivi_quant_dequant_values(x_dev, bits, gv, with_codes=False)
    torch.cuda.synchronize()
    say(f"[{tag}] done")
    for name, t in dict(ck=ck, sk=sk, zk=zk, cv=cv, sv=sv, zv=zv, fck=fck,
                        fsk=fsk, fzk=fzk, fcv=fcv, fsv=fsv,
                        fzv=fzv).items():
        out[name] = host(t)
    for name, t in dict(rk=rk, rv=rv, fk=fk, fv=fv, fk2=fk2,
                        fv2=fv2).items():
        out[name] = bits16(t)
    return out


def compare(O, got, x, dtype, bits, gk, gv, tag, sel=None):
    """Compare GPU results (optionally the slices `sel` of them) with the
    oracle on the host tensor x (already restricted to those slices)."""
    if sel is None:
        sel = slice(None)
    ck, sk, zk = O.quant_keys(x, dtype, bits, gk)
    cv, sv, zv = O.quant_values(x, dtype, bits, gv)
    rk = O.dequant_keys(ck, sk, zk, x.shape, bits, gk, dtype)
    rv = O.dequant_values(cv, sv, zv, x.shape, bits, gv, dtype)
    assert_codes_equal(got["ck"][sel], ck, f"{tag} key codes")
    assert_f32_bits_equal(got["sk"][sel], sk, f"{tag} key scale")
    assert_f32_bits_equal(got["zk"][sel], zk, f"{tag} key zero")
    assert_codes_equal(got["cv"][sel], cv, f"{tag} value codes")
    assert_f32_bits_equal(got["sv"][sel], sv, f"{tag} value scale")
    assert_f32_bits_equal(got["zv"][sel], zv, f"{tag} value zero")
    assert_recon_equal(got["rk"][sel], rk, f"{tag} key dequant")
    assert_recon_equal(got["rv"][sel], rv, f"{tag} value dequant")
    assert_codes_equal(got["fck"][sel], ck, f"{tag} fused key codes")
    assert_f32_bits_equal(got["fsk"][sel], sk, f"{tag} fused key scale")
    assert_f32_bits_equal(got["fzk"][sel], zk, f"{tag} fused key zero")
    assert_codes_equal(got["fcv"][sel], cv, f"{tag} fused value codes")
    assert_f32_bits_equal(got["fsv"][sel], sv, f"{tag} fused value scale")
    assert_f32_bits_equal(got["fzv"][sel], zv, f"{tag} fused value zero")
    assert_recon_equal(got["fk"][sel], rk, f"{tag} fused key recon")
    assert_recon_equal(got["fv"][sel], rv, f"{tag} fused value recon")
    assert_recon_equal(got["fk2"][sel], rk, f"{tag} recon-only key")
    assert_recon_equal(got["fv2"][sel], rv, f"{tag} recon-only value")


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_workload_full(K, O, name):
    w = W.WORKLOADS[name]
    for tensor in ("K", "V"):
        x = W.gen_tensor(w, tensor)
        tag = f"{name}/{tensor}"
        got = run_all(K, to_dev(x, w.dtype), w.dtype, w.bits, w.group_k,
                      w.group_v, tag)
        compare(O, got, x, w.dtype, w.bits, w.group_k, w.group_v, tag)


def test_tiny_constant_groups_hit(K, O):
    """The tiny workload's planted constant groups come out as scale 0,
    code 0, recon == zero."""
    w = W.WORKLOADS["tiny"]
    k = W.gen_tensor(w, "K")
    v = W.gen_tensor(w, "V")
    ck, sk, zk = K.kivi_quant_keys(to_dev(k, FP16), 2, 32)
    cv, sv, zv = K.kivi_quant_values(to_dev(v, FP16), 2, 32)
    sk, zk, sv, zv = host(sk), host(zk), host(sv), host(zv)
    assert sk[1, 1, 5] == 0 and zk[1, 1, 5] == np.float32(0.75)
    assert sv[2, 10, 1] == 0 and zv[2, 10, 1] == np.float32(-1.25)
    assert np.all(O.unpack(host(ck), 64, 2)[1, 32:64, 5] == 0)
    assert np.all(O.unpack(host(cv), 64, 2)[2, 10, 32:64] == 0)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("tensor", ["K", "V"])
@pytest.mark.parametrize("name", ["prefill", "serve", "roundtrip"])
def test_workload_full_size(K, O, name, tensor):
    """Every element of the large workloads: the GPU results of all six
    entry points on one full-size tensor against the oracle on every (bh)
    slice."""
    w = W.WORKLOADS[name]
    tag = f"{name}/{tensor}"
    say(f"[{tag}] generating {w.BH}x{w.S}x{w.D}")
    x = W.gen_tensor(w, tensor)
    got = run_all(K, to_dev(x, w.dtype), w.dtype, w.bits, w.group_k,
                  w.group_v, tag)
    torch.cuda.empty_cache()
    say(f"[{tag}] oracle over all {w.BH} slices")

    def block(a, b):
        compare(O, {n: g[a:b] for n, g in got.items()},
                np.ascontiguousarray(x[a:b]), w.dtype, w.bits, w.group_k,
                w.group_v, f"{tag} bh[{a}:{b}]")

    by_blocks(w.BH, block)
    say(f"[{tag}] all {w.BH} slices equal")


# --------------------------------------------------------------------------
# directed cases: ragged groups, other bits/groups, generic fallbacks,
# constant and signed-zero groups, extreme magnitudes
# --------------------------------------------------------------------------

def _rand(seed, BH, S, D, dtype, scale=1.0, outliers=True):
    r = np.random.default_rng(seed)
    x = (r.standard_normal((BH, S, D)) * scale).astype(np.float32)
    if outliers and D >= 8:
        ch = r.choice(D, size=max(1, D // 16), replace=False)
        x[:, :, ch] *= 20.0
    if dtype == FP16:
        return x.astype(np.float16).view(np.uint16)
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16)
    return t.numpy().view(np.uint16)


DIRECTED = [
    # (BH, S, D, dtype, bits, gk, gv)
    (3, 70, 48, FP16, 2, 32, 32),      # ragged S and D groups
    (2, 70, 48, BF16, 4, 32, 32),
    (2, 64, 40, FP16, 2, 16, 16),      # D8 = 5, two-lane value groups
    (2, 33, 64, FP16, 1, 8, 8),        # bits 1, GMAX 8
    (2, 50, 64, BF16, 8, 5, 64),       # bits 8, ragged small key group
    (2, 48, 128, FP16, 4, 16, 128),    # GMAX 16, whole-row value group
    (2, 96, 128, FP16, 2, 64, 24),     # generic keys (G > 32), generic values
    (2, 40, 12, FP16, 2, 32, 4),       # D % 8 != 0: generic everything
    (1, 37, 20, BF16, 2, 3, 5),        # generic, groups straddle code bytes
    (2, 32, 512, FP16, 2, 32, 256),    # 64 lanes per row, cross-row reduce
    (1, 32, 512, BF16, 2, 32, 512),
    (2, 16, 1024, FP16, 2, 32, 32),    # 32 lanes per row, in-lane groups
    (1, 1, 8, FP16, 2, 32, 8),         # one token
    (3, 64, 128, FP16, 2, 256, 512),   # group larger than S / D
    (2, 16, 1024, BF16, 4, 32, 1024),  # 32-lane value groups (cross-row)
    (1, 8, 2048, FP16, 2, 16, 2048),   # 64-lane value groups
    (2, 24, 96, FP16, 2, 32, 64),      # 3 lanes per row padded to 4
    (2, 24, 2056, FP16, 2, 32, 32),    # D > 2048: generic values
]


@pytest.mark.parametrize("case", DIRECTED, ids=lambda c: "x".join(map(str, c)))
def test_directed(K, O, case):
    BH, S, D, dtype, bits, gk, gv = case
    x = _rand(hash(case) % (2**31), BH, S, D, dtype)
    tag = "directed " + "x".join(map(str, case))
    got = run_all(K, to_dev(x, dtype), dtype, bits, gk, gv, tag)
    compare(O, got, x, dtype, bits, gk, gv, tag)


# The key quantizer splits each (bh, token group, 8-channel chunk) item
# over 4 lanes below 65536 items (the decode-time flush) and over 2 lanes
# above it, when D/8 allows (a power of two up to 16, resp. 32); other
# shapes take one lane per item.  The key dequantizer splits items over 4
# lanes below 65536 items and uses one lane per item above.  Each shape runs
# once with the BH given and once with BH raised past the threshold.
KEY_PATHS = [
    # (BH, S, D, dtype, bits, gk)
    (2, 33, 64, FP16, 1, 8),      # ragged: the last group has one token
    (2, 50, 64, BF16, 8, 5),      # group 5 over 4 lanes of 2 tokens
    (2, 48, 128, FP16, 4, 16),
    (1, 1, 8, FP16, 2, 32),       # one token, D8 = 1
    (3, 70, 32, BF16, 2, 32),     # ragged 32-token group
    (2, 64, 16, FP16, 4, 32),
    (2, 64, 256, FP16, 2, 32),    # D8 = 32: one lane (small), two (large)
    (2, 64, 512, BF16, 4, 32),    # D8 = 64: one lane per item, staged codes
    (2, 96, 64, FP16, 2, 48),     # group > 32: generic quantizer, direct dequant
    # D = 128 with codes of at most 4 bits: a tile's codes go through LDS
    # and out as 16-byte pieces of its code block; ragged last groups
    (3, 70, 128, BF16, 2, 32),    # last group of 6 tokens
    (2, 45, 128, FP16, 1, 32),    # 1-bit rows of 16 bytes
    (2, 41, 128, BF16, 4, 8),     # GMAX 8, last group of one token
    (2, 50, 128, FP16, 2, 16),    # GMAX 16, last group of 2 tokens
]
KEY_SPLIT_BELOW = 65536


def _key_path_bh(S, D, gk, split):
    if split:
        return None
    items = ((S + gk - 1) // gk) * (D // 8)
    return -(-KEY_SPLIT_BELOW // items)


@pytest.mark.parametrize("split", [True, False], ids=["small", "large"])
@pytest.mark.parametrize("case", KEY_PATHS,
                         ids=lambda c: "x".join(map(str, c)))
def test_key_kernel_paths(K, O, case, split):
    BH, S, D, dtype, bits, gk = case
    BH = _key_path_bh(S, D, gk, split) or BH
    tag = f"keys {'small' if split else 'large'} BH={BH} " + \
        "x".join(map(str, case[1:]))
    x = _rand(hash(case) % (2**31), BH, S, D, dtype)
    xd = to_dev(x, dtype)
    say(f"[{tag}] quant / fused / dequant")
    ck, sk, zk = K.kivi_quant_keys(xd, bits, gk)
    rk = K.kivi_dequant_keys(ck, sk, zk, bits, gk, out_dtype=xd.dtype)
    fk, fck, fsk, fzk = K.kivi_quant_dequant_keys(xd, bits, gk)
    fk2 = K.kivi_quant_dequant_keys(xd, bits, gk, with_codes=False)
    torch.cuda.synchronize()
    eck, esk, ezk = O.quant_keys(x, dtype, bits, gk)
    erk = O.dequant_keys(eck, esk, ezk, x.shape, bits, gk, dtype)
    for got, exp, what in ((ck, eck, "codes"), (fck, eck, "fused codes")):
        assert_codes_equal(host(got), exp, f"{tag} {what}")
    for got, exp, what in ((sk, esk, "scale"), (zk, ezk, "zero"),
                           (fsk, esk, "fused scale"),
                           (fzk, ezk, "fused zero")):
        assert_f32_bits_equal(host(got), exp, f"{tag} {what}")
    for got, what in ((rk, "dequant"), (fk, "fused recon"),
                      (fk2, "recon-only")):
        assert_recon_equal(bits16(got), erk, f"{tag} {what}")


def test_constant_and_signed_zero_groups(K, O):
    for dtype in (FP16, BF16):
        x = _rand(5, 2, 64, 64, dtype)
        one = np.float32(1.5)
        cst = one.astype(np.float16).view(np.uint16) if dtype == FP16 \
            else np.uint16(0x3FC0)
        x[0, 0:32, 3] = cst                 # constant key group
        x[1, 7, 8:16] = cst                 # constant value group (G=8)
        x[1, 32:64, 9] = 0x8000             # -0 key group
        x[1, 32:48, 10] = 0x8000            # mixed +-0 key group
        x[1, 48:64, 10] = 0x0000
        x[0, 5, 16:24] = 0x8000             # -0 value group
        x[0, 6, 24:32] = np.array([0, 0x8000] * 4, np.uint16)
        tag = f"zeros dtype={dtype}"
        got = run_all(K, to_dev(x, dtype), dtype, 2, 32, 8, tag)
        compare(O, got, x, dtype, 2, 32, 8, tag)


def test_all_zero_tensor(K, O):
    x = np.zeros((2, 64, 64), np.uint16)
    got = run_all(K, to_dev(x, FP16), FP16, 2, 32, 32, "all zero")
    compare(O, got, x, FP16, 2, 32, 32, "all zero")


@pytest.mark.parametrize("mag", [1e-38, 1e-30, 1e30, 3e38])
def test_bf16_extreme_magnitudes(K, O, mag):
    """bf16 groups with tiny or huge scales take the exact-division path;
    results must still match (3e38 keeps max - min finite by using one
    sign)."""
    r = np.random.default_rng(int(np.log10(mag) + 100))
    f = np.abs(r.standard_normal((2, 64, 64))).astype(np.float32)
    f = (f / f.max() * mag).astype(np.float32)
    if mag < 1e38:
        f[:, ::3] *= -1
    x = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy()
    x = x.view(np.uint16)
    tag = f"bf16 magnitude {mag}"
    got = run_all(K, to_dev(x, BF16), BF16, 2, 32, 32, tag)
    compare(O, got, x, BF16, 2, 32, 32, tag)


def test_fp16_subnormal_and_max_values(K, O):
    r = np.random.default_rng(9)
    x = r.integers(0, 0x400, size=(2, 64, 64)).astype(np.uint16)   # subnormal
    x[:, ::2] |= 0x8000
    x[0, :, 0:8] = 0x7BFF                      # 65504
    x[0, :32, 8:16] = 0xFBFF                   # -65504
    got = run_all(K, to_dev(x, FP16), FP16, 4, 32, 32, "fp16 extremes")
    compare(O, got, x, FP16, 4, 32, 32, "fp16 extremes")


def test_empty_tensors(K):
    for shape in ((0, 64, 64), (2, 0, 64), (2, 64, 0)):
        x = torch.zeros(shape, dtype=torch.float16, device="cuda")
        c, s, z = K.kivi_quant_keys(x, 2, 32)
        c2, s2, z2 = K.kivi_quant_values(x, 2, 32)
        r = K.kivi_quant_dequant_keys(x, 2, 32, with_codes=False)
        assert c.numel() == 0 or shape[1] == 0 or shape[2] == 0
        assert r.shape == x.shape
    torch.cuda.synchronize()


def test_deterministic_and_stream(K):
    w = W.WORKLOADS["decode"]
    x = to_dev(W.gen_tensor(w, "K"), w.dtype)
    a = [host(t) for t in K.kivi_quant_keys(x, 2, 32)]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = [host(t) for t in K.kivi_quant_keys(x, 2, 32)]
        s.synchronize()
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))
    # stream= given as a torch stream and as its raw handle
    s2 = torch.cuda.Stream()
    for st in (s2, s2.cuda_stream):
        out = K.kivi_quant_keys(x, 2, 32, stream=st)
        s2.synchronize()
        for u, v in zip(a, [host(t) for t in out]):
            assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


@pytest.mark.parametrize("shape", [(224, 32, 128), (512, 256, 128)],
                         ids=["small", "large"])
def test_graph_capture_replays(K, shape):
    """Every compute entry point captured in one HIP graph (as the benchmark
    replays a launch-bound step): three replays, each after eager work that
    scribbles over the outputs and a synchronisation, must reproduce the
    eager results bit for bit."""
    BH, S, D = shape
    bits, g = 2, 32
    x = to_dev(_rand(11, BH, S, D, FP16), FP16)
    ck, sk, zk = K.kivi_quant_keys(x, bits, g)
    cv, sv, zv = K.kivi_quant_values(x, bits, g)
    rk = K.kivi_dequant_keys(ck, sk, zk, bits, g, out_dtype=x.dtype)
    rv = K.kivi_dequant_values(cv, sv, zv, bits, g, out_dtype=x.dtype)
    fk = K.kivi_quant_dequant_keys(x, bits, g)
    fv = K.kivi_quant_dequant_values(x, bits, g)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (ck, sk, zk, cv, sv, zv, rk, rv, *fk, *fv)]
    outs = [torch.empty_like(t) for t in eager]
    (gck, gsk, gzk, gcv, gsv, gzv, grk, grv,
     gfk, gfck, gfsk, gfzk, gfv, gfcv, gfsv, gfzv) = outs
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=cap):
        K.kivi_quant_keys(x, bits, g, gck, gsk, gzk)
        K.kivi_quant_values(x, bits, g, gcv, gsv, gzv)
        K.kivi_dequant_keys(eager[0], eager[1], eager[2], bits, g,
                            out_dtype=x.dtype, out=grk)
        K.kivi_dequant_values(eager[3], eager[4], eager[5], bits, g,
                              out_dtype=x.dtype, out=grv)
        K.kivi_quant_dequant_keys(x, bits, g, True, gfk, gfck, gfsk, gfzk)
        K.kivi_quant_dequant_values(x, bits, g, True, gfv, gfcv, gfsv, gfzv)
    for rep in range(3):
        say(f"[graph {shape}] replay {rep}")
        for t in outs:                     # eager work between replays
            t.view(torch.uint8).fill_(0xA5 + rep)
        K.kivi_quant_keys(x, bits, g)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, eager)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), \
                f"replay {rep}, output {i}"


def test_more_than_2_31_elements(K, O):
    """A [520, 32768, 128] fp16 tensor (2.2e9 elements, 4.4 GB): 64-bit
    offsets throughout.  Built by tiling 8 seeded slices; the oracle checks
    slices past the 2^31-element mark."""
    BH, S, D = 520, 32768, 128
    w = W.WORKLOADS["prefill"]
    base = W.gen_tensor(w, "K", range(8))
    say(f"[max size] uploading {BH}x{S}x{D}")
    x = torch.empty((BH, S, D), dtype=torch.float16, device="cuda")
    bd = to_dev(base, FP16)
    for i in range(0, BH, 8):
        n = min(8, BH - i)
        x[i:i + n] = bd[:n]
    del bd
    sel = [511, 519]                       # elements beyond 2^31
    for kind in ("keys", "values"):
        say(f"[max size] {kind}")
        if kind == "keys":
            c, s_, z = K.kivi_quant_keys(x, 2, 32)
        else:
            c, s_, z = K.kivi_quant_values(x, 2, 32)
        torch.cuda.synchronize()
        xs = base[[b % 8 for b in sel]]
        if kind == "keys":
            oc, os_, oz = O.quant_keys(xs, FP16, 2, 32)
        else:
            oc, os_, oz = O.quant_values(xs, FP16, 2, 32)
        assert_codes_equal(host(c[sel]), oc, f"max size {kind} codes")
        assert_f32_bits_equal(host(s_[sel]), os_, f"max size {kind} scale")
        assert_f32_bits_equal(host(z[sel]), oz, f"max size {kind} zero")
        if kind == "keys":
            r = K.kivi_dequant_keys(c, s_, z, 2, 32, out_dtype=torch.float16)
            want = O.dequant_keys(oc, os_, oz, xs.shape, 2, 32, FP16)
        else:
            r = K.kivi_dequant_values(c, s_, z, 2, 32, out_dtype=torch.float16)
            want = O.dequant_values(oc, os_, oz, xs.shape, 2, 32, FP16)
        assert_recon_equal(bits16(r[sel]), want, f"max size {kind} dequant")
        del c, s_, z, r
        torch.cuda.empty_cache()


def test_keys_just_under_4_gib(K, O):
    """A [511, 32768, 128] fp16 tensor (4 286 578 688 bytes, just under
    2^32): the dense key quantizer forms its row addresses as 32-bit byte
    offsets here.  The two topmost slices (offsets within 16 MB of 2^32)
    are checked against the oracle, quantize-only and fused."""
    BH, S, D = 511, 32768, 128
    assert BH * S * D * 2 < 2 ** 32 and (BH + 1) * S * D * 2 > 2 ** 32 - 2 ** 23
    w = W.WORKLOADS["prefill"]
    base = W.gen_tensor(w, "K", range(8))
    say(f"[4 GiB] uploading {BH}x{S}x{D}")
    x = torch.empty((BH, S, D), dtype=torch.float16, device="cuda")
    bd = to_dev(base, FP16)
    for i in range(0, BH, 8):
        n = min(8, BH - i)
        x[i:i + n] = bd[:n]
    del bd
    sel = [509, 510]
    xs = base[[b % 8 for b in sel]]
    oc, os_, oz = O.quant_keys(xs, FP16, 2, 32)
    want = O.dequant_keys(oc, os_, oz, xs.shape, 2, 32, FP16)
    say("[4 GiB] quant keys")
    c, s_, z = K.kivi_quant_keys(x, 2, 32)
    torch.cuda.synchronize()
    assert_codes_equal(host(c[sel]), oc, "4 GiB key codes")
    assert_f32_bits_equal(host(s_[sel]), os_, "4 GiB key scale")
    assert_f32_bits_equal(host(z[sel]), oz, "4 GiB key zero")
    del c, s_, z
    say("[4 GiB] fused keys")
    r, c, s_, z = K.kivi_quant_dequant_keys(x, 2, 32)
    torch.cuda.synchronize()
    assert_codes_equal(host(c[sel]), oc, "4 GiB fused key codes")
    assert_recon_equal(bits16(r[sel]), want, "4 GiB fused key recon")
    del r, c, s_, z, x
    torch.cuda.empty_cache()


def test_selftest_division(K):
    """The exact-division shortcuts hold on this GPU for every significand
    at every exponent the kernels use them."""
    assert K.kivi_selftest_division() == 0


def test_time_next_launch(K):
    """kivi_time_next_launch times exactly the next kernel: a positive
    duration no longer than the events around the whole call, and the pair
    is disarmed after one launch."""
    w = W.WORKLOADS["decode"]
    x = to_dev(W.gen_tensor(w, "K"), w.dtype)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    o1, o2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for e in (a, b):
        e.record()
    torch.cuda.synchronize()
    o1.record()
    K.kivi_time_next_launch(a, b)
    K.kivi_quant_keys(x, 2, 32)
    o2.record()
    K.kivi_quant_keys(x, 2, 32)          # not timed: the pair was consumed
    torch.cuda.synchronize()
    dt = a.elapsed_time(b)
    assert 0.0 < dt <= o1.elapsed_time(o2)
