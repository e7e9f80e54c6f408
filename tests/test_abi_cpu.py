"""The C ABI on the CPU: the library loads, exports every declared symbol,
and rejects invalid arguments before touching the GPU (no compute calls)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kivi.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kivi_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def K():
    import kv_cache_quantization_kivi_amd as K
    return K


def test_header_declares_the_abi():
    names = declared_functions()
    for n in ("kivi_quant_keys", "kivi_quant_values", "kivi_dequant_keys",
              "kivi_dequant_values", "kivi_quant_dequant_keys",
              "kivi_quant_dequant_values", "kivi_codes_bytes",
              "kivi_key_param_count", "kivi_value_param_count",
              "kivi_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(K):
    lib = ctypes.CDLL(K.library_path())
    for n in declared_functions():
        assert hasattr(lib, n), n
    # the python binding carries the same names
    for n in declared_functions():
        assert hasattr(K, n), n


def test_size_helpers(K):
    assert K.kivi_codes_bytes(224, 32, 128, 2) == 224 * 32 * 32
    assert K.kivi_codes_bytes(4, 70, 48, 4) == 4 * 70 * 24
    assert K.kivi_key_param_count(112, 32768, 128, 32) == 112 * 1024 * 128
    assert K.kivi_key_param_count(3, 70, 48, 32) == 3 * 3 * 48
    assert K.kivi_value_param_count(128, 8192, 128, 128) == 128 * 8192
    assert K.kivi_value_param_count(3, 70, 48, 32) == 3 * 70 * 2
    assert K.kivi_codes_bytes(1, 1, 6, 1) == -1        # D*bits % 8 != 0
    assert K.kivi_codes_bytes(1, 1, 8, 3) == -1        # bits
    assert K.kivi_key_param_count(1, 1, 8, 0) == -1    # group
    assert K.kivi_codes_bytes(-1, 1, 8, 2) == -1
    assert K.kivi_codes_bytes(1 << 40, 1 << 20, 1 << 10, 2) == -1  # overflow
    assert K.kivi_codes_bytes(0, 5, 8, 2) == 0


def test_status_strings(K):
    for s in range(9):
        assert K.kivi_status_string(s)
    assert K.kivi_status_string(0) == "ok"


def _raw_quant(K, name, x=0x1000, dt=0, BH=2, S=64, D=64, bits=2, G=32,
               codes=0x2000, scale=0x3000, zero=0x4000):
    fn = getattr(K.raw(), name)
    return fn(ctypes.c_void_p(x), dt, BH, S, D, bits, G, ctypes.c_void_p(codes),
              ctypes.c_void_p(scale), ctypes.c_void_p(zero), None)


@pytest.mark.parametrize("name", ["kivi_quant_keys", "kivi_quant_values"])
def test_quant_argument_errors(K, name):
    # Every call below fails validation before any HIP call: the fake
    # pointers are never dereferenced.
    assert _raw_quant(K, name, bits=3) == 3
    assert _raw_quant(K, name, bits=0) == 3
    assert _raw_quant(K, name, G=0) == 4
    assert _raw_quant(K, name, G=-5) == 4
    assert _raw_quant(K, name, D=6, bits=1) == 2      # D*bits % 8
    assert _raw_quant(K, name, BH=-1) == 2
    assert _raw_quant(K, name, BH=1 << 40, S=1 << 20, D=1 << 8) == 2
    assert _raw_quant(K, name, dt=2) == 5
    assert _raw_quant(K, name, x=0) == 1
    assert _raw_quant(K, name, codes=0) == 1
    assert _raw_quant(K, name, scale=0) == 1
    assert _raw_quant(K, name, zero=0) == 1
    assert _raw_quant(K, name, x=0x1008) == 6          # misaligned
    assert _raw_quant(K, name, zero=0x4004) == 6
    # empty tensors are valid no-ops, even with NULL pointers
    assert _raw_quant(K, name, BH=0, x=0, codes=0, scale=0, zero=0) == 0
    assert _raw_quant(K, name, S=0, x=0, codes=0, scale=0, zero=0) == 0


@pytest.mark.parametrize("name", ["kivi_quant_dequant_keys",
                                  "kivi_quant_dequant_values"])
def test_fused_argument_errors(K, name):
    fn = getattr(K.raw(), name)
    P = ctypes.c_void_p
    # recon is required
    assert fn(P(0x1000), 0, 2, 64, 64, 2, 32, P(0x2000), P(0x3000), P(0x4000),
              None, None) == 1
    # codes/scale/zero: all or none
    assert fn(P(0x1000), 0, 2, 64, 64, 2, 32, P(0x2000), None, P(0x4000),
              P(0x5000), None) == 1
    assert fn(P(0x1000), 0, 2, 64, 64, 2, 32, None, None, None, P(0x5008),
              None) == 6
    assert fn(P(0x1000), 0, 2, 64, 64, 3, 32, None, None, None, P(0x5000),
              None) == 3


@pytest.mark.parametrize("name", ["kivi_dequant_keys", "kivi_dequant_values"])
def test_dequant_argument_errors(K, name):
    fn = getattr(K.raw(), name)
    P = ctypes.c_void_p

    def call(codes=0x1000, scale=0x2000, zero=0x3000, BH=2, S=64, D=64,
             bits=2, G=32, dt=0, out=0x4000):
        return fn(P(codes), P(scale), P(zero), BH, S, D, bits, G, dt, P(out),
                  None)
    assert call(bits=5) == 3
    assert call(G=0) == 4
    assert call(D=4, bits=1) == 2
    assert call(dt=7) == 5
    assert call(out=0) == 1
    assert call(codes=0) == 1
    assert call(scale=0x2002) == 6
    assert call(S=0, codes=0, scale=0, zero=0, out=0) == 0


def test_binding_rejects_bad_tensors(K):
    import torch
    x = torch.zeros(2, 8, 8, dtype=torch.float32)
    with pytest.raises(TypeError):
        K.kivi_quant_keys(x)
    y = torch.zeros(2, 8, 16, dtype=torch.float16)[:, :, :8]
    with pytest.raises(ValueError):
        K.kivi_quant_keys(y)


def test_missing_library_fails_loudly_but_build_module_imports(tmp_path):
    """From a checkout where libkivi.so is not built, the package and its
    `build` submodule import (so the build can run), and the first call
    raises ImportError naming the missing library: there is no fallback."""
    import shutil
    import subprocess
    import sys
    pkg = os.path.join(ROOT, "kv_cache_quantization_kivi_amd")
    dst = tmp_path / "kv_cache_quantization_kivi_amd"
    shutil.copytree(pkg, dst, ignore=shutil.ignore_patterns(
        "*.so", "_build", "__pycache__"))
    code = (
        "import kv_cache_quantization_kivi_amd.build as b\n"
        "import kv_cache_quantization_kivi_amd as K\n"
        "assert callable(b.build)\n"
        "try:\n"
        "    K.kivi_codes_bytes(1, 1, 8, 2)\n"
        "except ImportError as e:\n"
        "    assert 'libkivi.so' in str(e)\n"
        "    print('loud')\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=tmp_path,
                         capture_output=True, text=True, timeout=120,
                         env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "loud"


def test_cache_append_rejects_before_any_launch(K):
    """kivi_cache_append validates the whole struct and its arguments first:
    every case below returns its status without a HIP call (fake aligned
    pointers) and leaves the counters as they were; a valid append that
    flushes nothing and copies nothing (n = 0) returns OK."""
    C = K._Cache
    L = K.raw()
    L.kivi_cache_append.argtypes = [ctypes.POINTER(C), ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_void_p]
    L.kivi_cache_append.restype = ctypes.c_int

    def cache(**kw):
        f = dict(BH=2, D=128, S_max=256, R=32, G_k=32, G_v=32, ring=64,
                 bits=2, dtype=0, k_ring=0x10000, v_ring=0x20000,
                 k_codes=0x30000, v_codes=0x40000, k_scale=0x50000,
                 k_zero=0x60000, v_scale=0x70000, v_zero=0x80000, T=0, Q=0)
        f.update(kw)
        return C(*[f[name] for name, _ in C._fields_])

    def call(c, n=1, k=0x90000, v=0xA0000):
        T, Q = c.T, c.Q
        st = L.kivi_cache_append(ctypes.byref(c), k, v, n, None)
        assert (c.T, c.Q) == (T, Q) or st == 0
        return st

    OK, NULL, SHAPE, BITS, GROUP, DTYPE, ALIGN = 0, 1, 2, 3, 4, 5, 6
    assert L.kivi_cache_append(None, 0x90000, 0xA0000, 1, None) == NULL
    assert call(cache(), n=0) == OK
    assert call(cache(bits=3)) == BITS
    assert call(cache(G_k=0)) == GROUP
    assert call(cache(G_k=33, ring=66)) == GROUP
    assert call(cache(G_v=24)) == GROUP
    assert call(cache(G_v=96)) == GROUP             # not 32 * 2^k
    assert call(cache(G_v=64), n=0) == OK
    assert call(cache(dtype=2)) == DTYPE
    assert call(cache(D=96)) == SHAPE
    assert call(cache(D=512)) == SHAPE
    assert call(cache(ring=48)) == SHAPE            # not a multiple of G_k
    assert call(cache(ring=32)) == SHAPE            # < R + G_k
    assert call(cache(R=-1)) == SHAPE
    assert call(cache(S_max=1 << 31)) == SHAPE
    assert call(cache(BH=1 << 20, S_max=1 << 20)) == SHAPE   # 32-bit lanes
    assert call(cache(T=10, Q=32)) == SHAPE         # Q > T
    assert call(cache(T=40, Q=8)) == SHAPE          # Q not group-aligned
    assert call(cache(T=100, Q=0)) == SHAPE         # T - Q >= ring
    assert call(cache(T=250, Q=224), n=7) == SHAPE  # past S_max
    assert call(cache(k_codes=0)) == NULL
    assert call(cache(), k=0) == NULL
    assert call(cache(v_zero=0x80004)) == ALIGN
    assert call(cache(), v=0xA0008) == ALIGN


def test_attend_noalloc_rejects_before_any_launch(K):
    """kivi_cache_attend_noalloc checks the struct, the pointers and the
    workspace size against the library's fixed buffer before any HIP call
    (fake aligned pointers): too large a workspace is KIVI_ERR_SCRATCH."""
    C = K._Cache
    L = K.raw()
    L.kivi_cache_attend_noalloc.argtypes = [
        ctypes.POINTER(C), ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
        ctypes.c_void_p, ctypes.c_void_p]
    L.kivi_cache_attend_noalloc.restype = ctypes.c_int

    def cache(**kw):
        f = dict(BH=224, D=128, S_max=40000, R=32, G_k=32, G_v=32, ring=64,
                 bits=2, dtype=0, k_ring=0x10000, v_ring=0x20000,
                 k_codes=0x30000, v_codes=0x40000, k_scale=0x50000,
                 k_zero=0x60000, v_scale=0x70000, v_zero=0x80000, T=2059,
                 Q=2016)
        f.update(kw)
        return C(*[f[name] for name, _ in C._fields_])

    def call(c, n_q=3, q=0x90000, out=0xA0000):
        return L.kivi_cache_attend_noalloc(ctypes.byref(c), q, n_q, 0.1, out,
                                           None)

    NULL, SHAPE, GROUP, ALIGN, SCRATCH = 1, 2, 4, 6, 8
    assert L.kivi_cache_attend_noalloc(None, 0x90000, 1, 0.1, 0xA0000,
                                       None) == NULL
    assert call(cache(), q=0) == NULL
    assert call(cache(), out=0) == NULL
    assert call(cache(), out=0xA0008) == ALIGN
    assert call(cache(), n_q=9) == SHAPE
    assert call(cache(T=0, Q=0)) == SHAPE
    assert call(cache(G_k=16, ring=64, D=256)) == SHAPE
    # workspace = BH * chunks * n_q * (D + 4) * 4 bytes
    big = cache(T=32000, Q=31968)
    need = 224 * ((32000 + 127) // 128) * 3 * 132 * 4
    assert need > K.ATTEND_SCRATCH_BYTES
    assert call(big) == SCRATCH
    assert K.kivi_status_string(SCRATCH).startswith("the call needs more")


def test_sink_entry_points_reject_before_any_launch(K):
    """KIVI-Sink argument rules (include/kivi.h): every call below fails
    validation, so the fake pointers are never dereferenced."""
    L = K.raw()
    P = ctypes.c_void_p
    k, sc, idx, out = P(0x1000), P(0x2000), P(0x3000), P(0x4000)

    def select(B=2, H=4, S=64, D=128, n=5, dt=0, k=k, sc=sc, idx=idx):
        return L.kivi_sink_select(k, dt, B, H, S, D, n, sc, idx, None)

    assert select(n=65, S=100) == 2        # n_sink > 64
    assert select(n=9, S=8) == 2           # n_sink > S
    assert select(n=-1) == 2
    assert select(D=48) == 2               # not a power of two in [8, 256]
    assert select(D=512) == 2
    assert select(B=0) == 2 and select(H=0) == 2 and select(S=0) == 2
    assert select(B=1 << 20, S=1 << 12, H=1, D=8) == 2   # B*S >= 2^31
    assert select(dt=2) == 5
    assert select(k=None) == 1 and select(sc=None) == 1
    assert select(idx=None) == 1 and select(n=0, idx=None, k=P(0x1001)) == 6
    assert select(k=P(0x1008)) == 6                     # k not 16-byte aligned
    assert select(sc=P(0x2002)) == 6

    def qks(bits=2, G=32, D=128, n=5, codes=P(0x5000), scale=P(0x6000),
            zero=P(0x7000), recon=None, idx=idx, S=64):
        return L.kivi_quant_keys_sink(k, 0, 2, 4, S, D, bits, G, idx, n,
                                      codes, scale, zero, recon, None)

    assert qks(bits=3) == 3
    assert qks(G=0) == 4 and qks(G=33) == 4
    assert qks(D=12) == 2
    assert qks(codes=None) == 1                          # partial q outputs
    assert qks(codes=None, scale=None, zero=None) == 1   # no output at all
    assert qks(idx=None) == 1
    assert qks(recon=P(0x8004)) == 6
    assert qks(n=70, S=100) == 2

    for name in ("kivi_sink_gather", "kivi_sink_restore"):
        fn = getattr(L, name)
        assert fn(k, 2, 4, 64, 12, idx, 5, out, None) == 2      # D % 8
        assert fn(k, 2, 4, 64, 128, idx, 65, out, None) == 2
        assert fn(k, 2, 4, 64, 128, None, 5, out, None) == 1
        assert fn(k, 2, 4, 64, 128, idx, 5, P(0x4008), None) == 6
        assert fn(None, 2, 4, 64, 128, idx, 0, None, None) == 0  # nothing to do


def test_mixed_precision_entry_points_reject_before_any_launch(K):
    """Listed-set rules (include/kivi.h); fake pointers, never dereferenced."""
    L = K.raw()
    P = ctypes.c_void_p
    x, pos, c, s, z = P(0x1000), P(0x2000), P(0x3000), P(0x4000), P(0x5000)
    part = L.kivi_partition_top
    assert part(s, 2, 100, 101, pos, pos, None) == 2          # n_hi > S
    assert part(s, 2, 100, -1, pos, pos, None) == 2
    assert part(s, 0, 100, 5, pos, pos, None) == 2
    assert part(None, 2, 100, 5, pos, pos, None) == 1
    assert part(s, 2, 100, 5, None, pos, None) == 1
    assert part(s, 2, 100, 100, None, pos, None) == 1          # all hi needs pos_hi
    assert part(s, 2, 100, 5, pos, P(0x2002), None) == 6

    for name, keys in (("kivi_quant_keys_rows", True),
                       ("kivi_quant_values_rows", False)):
        fn = getattr(L, name)

        def q(bits=2, G=32, D=128, n=40, S=64, dt=0, x=x, pos=pos, codes=c):
            return fn(x, dt, 2, 4, S, D, bits, G, pos, n, codes, s, z, None)

        assert q(bits=3) == 3
        assert q(G=0) == 4
        assert q(G=48) == 4 and q(G=96) == 4                    # not 32 * 2^k
        if keys:
            assert q(G=33) == 4 and q(G=5) != 4
        else:
            assert q(G=5) == 4 and q(G=64) != 4
        assert q(D=48) == 2 and q(D=512) == 2
        assert q(n=65) == 2 and q(n=-1) == 2
        assert q(dt=3) == 5
        assert q(x=None) == 1 and q(pos=None) == 1 and q(codes=None) == 1
        assert q(x=P(0x1004)) == 6 and q(pos=P(0x2001)) == 6
        assert q(n=0, x=None) == 0                              # nothing to do
        if keys:        # 2^30 one-token groups of 128 channels: too many lanes
            assert fn(x, 0, 1, 1, 1 << 30, 128, 2, 1, pos, (1 << 30) - 1,
                      c, s, z, None) == 2

    for name in ("kivi_dequant_keys_rows", "kivi_dequant_values_rows"):
        fn = getattr(L, name)
        assert fn(c, s, z, 2, 4, 64, 128, 2, 32, pos, 65, 0, x, None) == 2
        assert fn(c, s, z, 2, 4, 64, 128, 2, 32, pos, 40, 0, None, None) == 1
        assert fn(c, s, z, 2, 4, 64, 128, 2, 32, pos, 40, 0, P(0x1008), None) == 6
        assert fn(c, s, z, 2, 4, 64, 128, 2, 32, pos, 40, 7, x, None) == 5
        if name == "kivi_dequant_keys_rows":
            assert fn(c, s, z, 1, 1, 1 << 30, 128, 2, 1, pos, (1 << 30) - 1, 0,
                      x, None) == 2


def test_kv_entry_points_reject_before_any_launch(K):
    """K+V rules (include/kivi.h): each half by the single call's rules,
    codes for both tensors or neither; fake pointers, never dereferenced."""
    L = K.raw()
    P = ctypes.c_void_p
    k, v = P(0x1000), P(0x2000)
    kc, ks, kz, vc, vs, vz = (P(0x10000 * i) for i in range(3, 9))
    kr, vr = P(0x90000), P(0xa0000)

    def q(bits=2, gk=32, gv=32, dt=0, D=128, **kw):
        a = dict(k=k, v=v, kc=kc, ks=ks, kz=kz, vc=vc, vs=vs, vz=vz)
        a.update(kw)
        return L.kivi_quant_kv(a["k"], a["v"], dt, 4, 32, D, bits, gk, gv,
                               a["kc"], a["ks"], a["kz"], a["vc"], a["vs"],
                               a["vz"], None)

    assert q(bits=3) == 3
    assert q(gk=0) == 4 and q(gv=0) == 4
    assert q(D=13) == 2                       # D * bits % 8
    assert q(dt=5) == 5
    assert q(k=None) == 1 and q(vz=None) == 1
    assert q(v=P(0x2008)) == 6 and q(kc=P(0x30004)) == 6
    assert L.kivi_quant_kv(k, v, 0, 0, 32, 128, 2, 32, 32, *([None] * 6),
                           None) == 0         # empty: nothing to do

    def f(**kw):
        a = dict(kc=kc, ks=ks, kz=kz, vc=vc, vs=vs, vz=vz, kr=kr, vr=vr)
        a.update(kw)
        return L.kivi_quant_dequant_kv(k, v, 0, 4, 32, 128, 2, 32, 32, a["kc"],
                                       a["ks"], a["kz"], a["vc"], a["vs"],
                                       a["vz"], a["kr"], a["vr"], None)

    assert f(kr=None) == 1 and f(vr=None) == 1
    assert f(ks=None) == 1                    # a partial set of outputs
    assert f(kc=None, ks=None, kz=None) == 1  # codes for one tensor only
    assert f(vr=P(0xa0002)) == 6

    def d(bits=2, gk=32, gv=32, odt=0, **kw):
        a = dict(kc=kc, ks=ks, kz=kz, vc=vc, vs=vs, vz=vz, kr=kr, vr=vr)
        a.update(kw)
        return L.kivi_dequant_kv(a["kc"], a["ks"], a["kz"], a["vc"], a["vs"],
                                 a["vz"], 4, 32, 128, bits, gk, gv, odt,
                                 a["kr"], a["vr"], None)

    assert d(bits=5) == 3 and d(gv=0) == 4 and d(odt=2) == 5
    assert d(vr=None) == 1 and d(kz=None) == 1
    assert d(vs=P(0x70004)) == 6
