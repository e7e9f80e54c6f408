"""kivi_cache_attend_noalloc, the entry point for callers that cannot
allocate: through the C ABI, on two calls in a row (the second over a
smaller cache), its output must equal kivi_cache_attend's bit for bit, and
both must sit within the attention tolerance of the oracle."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle                                              # noqa: E402
from attend_bound import (attend_bound, case_id,           # noqa: E402
                          case_inputs, oracle_cache)
from gpu_util import FP16, host, say                       # noqa: E402


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_quantization_kivi_amd as K
    return K


def _dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16))
    return t.view(torch.float16 if dtype == FP16 else torch.bfloat16).cuda()


def _cache(K, case):
    BH, D, R, Gk, Gv, bits, dtype, n_q, appends = case
    k, v, q, S_max = case_inputs(case)
    c = K.KiviCache(BH, D, S_max, R, Gk, Gv, bits,
                    torch.float16 if dtype == FP16 else torch.bfloat16)
    t = 0
    for n in appends:
        c.append(_dev(k[:, t:t + n], dtype), _dev(v[:, t:t + n], dtype))
        t += n
    return c, k, v, q, S_max


# the first call over the larger cache (the attend-decode shape: 224 KV
# heads x 3 query heads, 2059 tokens, 17 chunks), the second over a
# smaller one (fewer heads, fewer chunks, bf16, 4-bit codes)
CALLS = [
    (224, 128, 32, 32, 32, 2, FP16, 3, [2048, 11]),
    (3, 128, 32, 16, 16, 4, 1, 6, [700]),
]


def test_noalloc_matches_attend_twice(K):
    O = oracle.default()
    for i, case in enumerate(CALLS):
        c, k, v, q, S_max = _cache(K, case)
        qd = _dev(q, case[6])
        sm = 1.0 / np.sqrt(case[1])
        need = c.attend_work_bytes(case[7])
        assert 0 < need <= K.ATTEND_SCRATCH_BYTES
        say(f"[no-alloc call {i}: {case_id(case)} T={c.T} Q={c.Q} "
            f"workspace {need} bytes]")
        ref = c.attend(qd, sm)
        out = torch.full_like(qd, float("nan"))
        c.attend_noalloc(qd, sm, out)
        torch.cuda.synchronize()
        a = host(out.view(torch.int16))
        b = host(ref.view(torch.int16))
        assert np.array_equal(a, b), f"call {i}: differs from kivi_cache_attend"
        oc = oracle_cache(O, case, k, v, S_max)
        bound, want = attend_bound(O, oc, q, sm)
        got = O.widen(a.view(np.uint16), case[6]).astype(np.float64)
        assert (np.abs(got - want) <= bound).all(), f"call {i}: outside bound"


def test_noalloc_rejects_too_large_a_workspace(K):
    """A cache whose workspace exceeds the library's buffer is refused
    (KIVI_ERR_SCRATCH) before anything is launched."""
    BH, D, n_q = 2048, 128, 8
    c = K.KiviCache(BH, D, 600, 32, 32, 32, 2, torch.float16)
    x = torch.zeros((BH, 600, D), dtype=torch.float16, device="cuda")
    c.append(x, x)
    assert c.attend_work_bytes(n_q) > K.ATTEND_SCRATCH_BYTES
    q = torch.zeros((BH, n_q, D), dtype=torch.float16, device="cuda")
    with pytest.raises(K.KiviError) as e:
        c.attend_noalloc(q, 0.1, torch.empty_like(q))
    assert e.value.status == 8
