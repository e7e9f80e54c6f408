"""The decode-attention tolerance can fail (CPU only).

Each planted bug below is a plausible mistake of an attention kernel over
the packed cache, planted in the oracle (a mutated copy of the oracle
cache's store or counters, evaluated by OracleCache.attend_exact).  For
every parity case of tests/test_gpu_attend.py where the bug changes
anything, its output must leave the bound of tests/attend_bound.py
somewhere; and the exact oracle itself must sit inside its own bound."""
import copy

import numpy as np
import pytest

import oracle
from attend_bound import (CASES, LONG_CASE, attend_bound, case_id,
                          case_inputs, oracle_cache)


@pytest.fixture(scope="module")
def O():
    return oracle.default()


def _mutant(oc, Q=None, T=None, **arrays):
    """A copy of the oracle cache with some arrays replaced and, if given,
    new counters (attend_exact reads nothing else)."""
    m = copy.copy(oc)
    c = oc.c
    m.c = oracle._RefCache(c.BH, c.D, c.S_max, c.R, c.G_k, c.G_v, c.bits,
                           c.dtype, 0, 0, 0, 0, 0, 0, 0, 0,
                           c.T if T is None else T, c.Q if Q is None else Q)
    for k, v in arrays.items():
        setattr(m, k, v)
    return m


def _drop_tokens(oc, a, b, keys_group=None):
    """Tokens [a, b) removed from the cache (codes, value params, history);
    keys_group: the key group [a, b) is, whose params go too."""
    def cut(x):
        return np.ascontiguousarray(np.concatenate([x[:, :a], x[:, b:]], 1))
    g = keys_group
    return _mutant(
        oc, Q=oc.Q - (b - a), T=oc.T - (b - a),
        k=cut(oc.k), v=cut(oc.v), k_codes=cut(oc.k_codes),
        v_codes=cut(oc.v_codes), v_scale=cut(oc.v_scale),
        v_zero=cut(oc.v_zero),
        k_scale=np.ascontiguousarray(np.concatenate(
            [oc.k_scale[:, :g], oc.k_scale[:, g + 1:]], 1)),
        k_zero=np.ascontiguousarray(np.concatenate(
            [oc.k_zero[:, :g], oc.k_zero[:, g + 1:]], 1)))


def _roll(x, n):
    """x with its first n entries along axis 1 rotated by one (entry i takes
    entry i - 1's value; entry 0 the last one's)."""
    y = x.copy()
    y[:, :n] = np.roll(x[:, :n], 1, axis=1)
    return y


def _zeroed(x, n):
    y = x.copy()
    y[:, :n] = 0
    return y


def planted_bugs(oc):
    """{name: (mutated cache or None if the bug changes nothing here,
    sm factor)}"""
    c = oc.c
    Q, T, Gk = oc.Q, oc.T, c.G_k
    ng = Q // Gk
    bugs = {}
    g = ng // 2
    bugs["drop one key group"] = (
        _drop_tokens(oc, g * Gk, (g + 1) * Gk, keys_group=g)
        if ng >= 1 and T > Gk else None, 1.0)
    bugs["previous key group's params"] = (
        _mutant(oc, k_scale=_roll(oc.k_scale, ng), k_zero=_roll(oc.k_zero, ng))
        if ng >= 2 else None, 1.0)
    bugs["previous token's value params"] = (
        _mutant(oc, v_scale=_roll(oc.v_scale, Q), v_zero=_roll(oc.v_zero, Q))
        if Q >= 2 else None, 1.0)
    bugs["no key zero point"] = (
        _mutant(oc, k_zero=_zeroed(oc.k_zero, ng)) if Q else None, 1.0)
    bugs["no value zero point"] = (
        _mutant(oc, v_zero=_zeroed(oc.v_zero, Q)) if Q else None, 1.0)
    bugs["sm_scale * 1.01"] = (oc if T >= 2 else None, 1.01)
    bugs["ring tokens dropped"] = (
        _mutant(oc, T=Q) if Q and T > Q else None, 1.0)
    bugs["codes ignored"] = (
        _mutant(oc, k_codes=_zeroed(oc.k_codes, Q),
                v_codes=_zeroed(oc.v_codes, Q)) if Q else None, 1.0)
    return bugs


ALL_CASES = CASES + [LONG_CASE]


@pytest.mark.parametrize("case", ALL_CASES, ids=case_id)
def test_planted_bugs_exceed_bound(O, case):
    k, v, q, S_max = case_inputs(case)
    oc = oracle_cache(O, case, k, v, S_max)
    sm = 1.0 / np.sqrt(case[1])
    bound, ref = attend_bound(O, oc, q, sm)
    assert np.allclose(ref, oc.attend_exact(q, sm), rtol=1e-13, atol=1e-13)
    caught, missed = [], []
    for name, (mut, f) in planted_bugs(oc).items():
        if mut is None:
            continue
        got = mut.attend_exact(q, sm * f)
        ratio = float((np.abs(got - ref) / bound).max())
        (caught if ratio > 1.0 else missed).append((name, round(ratio, 2)))
    assert not missed, (case_id(case), missed)
    assert caught or oc.T == 1       # one exact token: no bug above applies


def test_every_bug_applies_to_most_cases(O):
    """Each planted bug is live in all but the cases that lack what it
    breaks: no quantized token (2 cases), no ring token (2), a single
    token (1), whose weight is 1 whatever the scores."""
    live = {}
    for case in ALL_CASES:
        k, v, q, S_max = case_inputs(case)
        oc = oracle_cache(O, case, k, v, S_max)
        for name, (mut, _) in planted_bugs(oc).items():
            live[name] = live.get(name, 0) + (mut is not None)
    assert all(n >= len(ALL_CASES) - 4 for n in live.values()), live


def test_bound_is_small_against_the_output(O):
    """The bound is a small fraction of the output: its median is under
    1/16 of the median |output| in every case (0.05-3.6% here; the bound it
    replaces, which covered the 16-bit rounding of the reconstruction, was
    15-50 times the output in the bf16 cases)."""
    for case in ALL_CASES:
        k, v, q, S_max = case_inputs(case)
        oc = oracle_cache(O, case, k, v, S_max)
        bound, ref = attend_bound(O, oc, q, 1.0 / np.sqrt(case[1]))
        assert np.median(bound) < np.median(np.abs(ref)) / 16, (
            case_id(case), np.median(bound), np.median(np.abs(ref)))
