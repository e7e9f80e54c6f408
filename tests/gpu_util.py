"""Helpers for the GPU parity tests: moving uint16 bit patterns between numpy
and torch device tensors, and comparing GPU outputs with the oracle's."""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

FP16, BF16 = 0, 1
TORCH_DT = {FP16: torch.float16, BF16: torch.bfloat16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def by_blocks(n, fn, threads=None):
    """fn(a, b) over contiguous blocks [a, b) that cover range(n), on a
    thread pool of up to 16 threads (the oracle's C calls release the GIL,
    so blocks of slices run in parallel); returns the results in order and
    re-raises the first failure."""
    threads = max(1, min(threads or min(16, os.cpu_count() or 1), n))
    cuts = np.linspace(0, n, threads + 1).astype(int)
    with ThreadPoolExecutor(max_workers=threads) as ex:
        futs = [ex.submit(fn, int(a), int(b))
                for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
        return [f.result() for f in futs]


def to_dev(bits16, dtype, device="cuda"):
    t = torch.from_numpy(np.ascontiguousarray(bits16).view(np.int16))
    return t.view(TORCH_DT[dtype]).to(device)


def to_dev_raw(arr, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def bits16(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def host(t):
    return t.detach().cpu().numpy()


def assert_codes_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
    assert bad.size == 0, (f"{what}: {bad.size} code bytes differ; first at "
                           f"flat {bad[0]}: got {got.reshape(-1)[bad[0]]:#04x}"
                           f" want {want.reshape(-1)[bad[0]]:#04x}")


def assert_f32_bits_equal(got, want, what):
    g = np.ascontiguousarray(got, dtype=np.float32).view(np.uint32)
    w = np.ascontiguousarray(want, dtype=np.float32).view(np.uint32)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    bad = np.flatnonzero(g.reshape(-1) != w.reshape(-1))
    assert bad.size == 0, (
        f"{what}: {bad.size} fp32 values differ; first at flat {bad[0]}: got "
        f"{g.reshape(-1)[bad[0]]:#010x} want {w.reshape(-1)[bad[0]]:#010x}")


def ulp_distance16(a, b):
    """Distance in units in the last place between 16-bit float patterns of
    the same format (sign-magnitude mapped to a monotone integer line)."""
    a = a.astype(np.int32)
    b = b.astype(np.int32)
    ia = np.where(a & 0x8000, 0x8000 - (a & 0x7FFF), 0x8000 + a)
    ib = np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + b)
    return np.abs(ia - ib)


def assert_recon_equal(got, want, what, max_ulp=0):
    """Reconstructions: 0 ulp of the output type (max_ulp 0), which is bit
    for bit except that +0 and -0, the same value, compare equal."""
    got = np.asarray(got, np.uint16)
    want = np.asarray(want, np.uint16)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    d = ulp_distance16(got, want)
    zero_pair = ((got & 0x7FFF) == 0) & ((want & 0x7FFF) == 0)
    d = np.where(zero_pair, 0, d)
    worst = int(d.max()) if d.size else 0
    n_bad = int((d > max_ulp).sum())
    assert n_bad == 0, f"{what}: {n_bad} elements beyond {max_ulp} ulp (max {worst})"
