"""GPU parity of the residual-window cache (kivi_cache_append) against the
oracle's token-by-token scheduler (oracle.OracleCache).

After every append the counters T and Q must match, the compressed store
(codes and fp32 params of tokens [0, Q)) must be bit-identical, storage past
Q must be untouched, and the ring must hold tokens [Q, T) exactly (token s in
slot s % ring)."""
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


def _tokens(seed, BH, n, D, dtype):
    r = np.random.default_rng(seed)
    x = (r.standard_normal((BH, n, D)) * 1.5).astype(np.float32)
    if D >= 16:
        x[:, :, r.choice(D, size=D // 16, replace=False)] *= 12.0
    if dtype == FP16:
        return x.astype(np.float16).view(np.uint16)
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16)
    return t.numpy().view(np.uint16)


def _dev(x, dtype):
    t = torch.from_numpy(x.view(np.int16))
    return t.view(torch.float16 if dtype == FP16 else torch.bfloat16).cuda()


def _compare(c, o, tag):
    assert (c.T, c.Q) == (o.T, o.Q), (tag, c.T, c.Q, o.T, o.Q)
    Q, T = o.Q, o.T
    G = c.c.G_k
    kc, vc = host(c.k_codes), host(c.v_codes)
    assert np.array_equal(kc[:, :Q], o.k_codes[:, :Q]), tag + " key codes"
    assert np.array_equal(vc[:, :Q], o.v_codes[:, :Q]), tag + " value codes"
    assert not kc[:, Q:].any() and not vc[:, Q:].any(), tag + " past Q"
    for got, exp, what in ((c.k_scale, o.k_scale, "key scale"),
                           (c.k_zero, o.k_zero, "key zero")):
        g = host(got)
        assert np.array_equal(g[:, :Q // G].view(np.uint32),
                              exp[:, :Q // G].view(np.uint32)), tag + what
        assert not g[:, Q // G:].any(), tag + what + " past Q"
    for got, exp, what in ((c.v_scale, o.v_scale, "value scale"),
                           (c.v_zero, o.v_zero, "value zero")):
        g = host(got)
        assert np.array_equal(g[:, :Q].view(np.uint32),
                              exp[:, :Q].view(np.uint32)), tag + what
        assert not g[:, Q:].any(), tag + what + " past Q"
    ring = c.c.ring
    slots = np.arange(Q, T) % ring
    for got, hist, what in ((c.k_ring, o.k, "key ring"),
                            (c.v_ring, o.v, "value ring")):
        r = host(got.view(torch.int16)).view(np.uint16)
        assert np.array_equal(r[:, slots], hist[:, Q:T]), tag + " " + what


CONFIGS = [
    # (BH, D, S_max, R, G_k, G_v, bits, dtype, append sizes)
    (4, 128, 400, 32, 32, 32, 2, FP16, [1, 3, 40, 1, 1, 100, 31, 33, 1, 64]),
    (3, 64, 300, 7, 16, 64, 4, BF16, [5, 1, 17, 64, 2, 2, 90, 1, 1, 1]),
    (2, 256, 200, 0, 8, 8, 8, FP16, [1, 1, 7, 9, 40, 3, 60, 1]),
    (5, 8, 160, 40, 32, 8, 1, BF16, [2, 80, 1, 1, 30, 41]),
    (2, 32, 300, 5, 32, 256, 2, FP16, [37, 1, 64, 2, 100]),
    (3, 16, 200, 3, 5, 16, 4, FP16, [1, 2, 3, 50, 4, 7]),
    (2, 64, 256, 32, 24, 64, 4, BF16, [1, 50, 1, 1, 30, 70, 2]),  # K+V flush in one launch
]


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: "x".join(
    map(str, c[:8])))
def test_cache_appends_match_oracle(K, O, cfg):
    BH, D, S_max, R, Gk, Gv, bits, dtype, sizes = cfg
    tdt = torch.float16 if dtype == FP16 else torch.bfloat16
    c = K.KiviCache(BH, D, S_max, R, Gk, Gv, bits, tdt)
    o = O.cache(BH, D, S_max, R, Gk, Gv, bits, dtype)
    total = sum(sizes)
    k = _tokens(1 + bits, BH, total, D, dtype)
    v = _tokens(2 + bits, BH, total, D, dtype)
    t = 0
    for i, n in enumerate(sizes):
        tag = f"[cache {cfg[:8]} append {i} n={n} T={t}]"
        say(tag)
        kn = np.ascontiguousarray(k[:, t:t + n])
        vn = np.ascontiguousarray(v[:, t:t + n])
        c.append(_dev(kn, dtype), _dev(vn, dtype))
        o.append(kn, vn)
        torch.cuda.synchronize()
        t += n
        _compare(c, o, tag)


@pytest.mark.parametrize("BH", [224, 512])
def test_cache_prefill_chunks_then_decode(K, O, BH):
    """A 2059-token prompt in prefill chunks of 2048, then 240 decode
    tokens (R = G = 32, D = 128; 28 layers x 8 KV heads, or 512 heads):
    2016 tokens flushed by the prompt, 7 decode flushes, everything
    bit-identical to the oracle.  The prompt flush of 224 heads (225792 key
    items) runs K and V in one launch; that of 512 heads (516096) takes the
    two launches and the two-lane key kernel."""
    D, R, G = 128, 32, 32
    S_max = 2059 + 240
    c = K.KiviCache(BH, D, S_max, R, G, G, 2, torch.float16)
    o = O.cache(BH, D, S_max, R, G, G, 2, FP16)
    k = _tokens(5, BH, S_max, D, FP16)
    v = _tokens(6, BH, S_max, D, FP16)
    for a in (0, 2048):
        b = min(a + 2048, 2059)
        say(f"[cache prefill BH={BH} chunk {a}:{b}]")
        kn, vn = np.ascontiguousarray(k[:, a:b]), np.ascontiguousarray(v[:, a:b])
        c.append(_dev(kn, FP16), _dev(vn, FP16))
        o.append(kn, vn)
    torch.cuda.synchronize()
    assert c.Q == 2016
    _compare(c, o, "[after prompt]")
    flushes = 0
    for t in range(2059, S_max):
        q = c.Q
        kn, vn = np.ascontiguousarray(k[:, t:t + 1]), np.ascontiguousarray(v[:, t:t + 1])
        c.append(_dev(kn, FP16), _dev(vn, FP16))
        o.append(kn, vn)
        flushes += c.Q != q
    torch.cuda.synchronize()
    assert flushes == 7
    _compare(c, o, "[after decode]")


def test_cache_rejects_overflow_and_keeps_state(K):
    c = K.KiviCache(2, 64, 64, 8, 8, 8, 2, torch.float16)
    x = torch.zeros((2, 60, 64), dtype=torch.float16, device="cuda")
    c.append(x, x)
    T, Q = c.T, c.Q
    y = torch.zeros((2, 10, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(K.KiviError) as e:
        c.append(y, y)
    assert e.value.status == 2 and (c.T, c.Q) == (T, Q)
