"""KIVI reference oracle: TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It wraps the plain C oracle (kivi_oracle.c) with ctypes
and numpy; it shares no code with the GPU library and the product path never
calls it.  All tensors are numpy arrays; 16-bit floats travel as uint16 bit
patterns (dtype 0 = fp16, 1 = bf16).

`Oracle(path)` wraps any build of kivi_oracle.c (the mutation tests load
deliberately broken copies); the module-level functions use the default
build at oracle/libkivi_oracle.so.
"""
import ctypes
import os

import numpy as np

from .build_oracle import LIB, build

FP16 = 0
BF16 = 1


def n_groups(n, g):
    return (n + g - 1) // g if g > 0 else 0


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    def __init__(self, path=LIB):
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        F = ctypes.c_float
        L.kivi_ref_half_to_float.argtypes = [ctypes.c_uint16]
        L.kivi_ref_half_to_float.restype = F
        L.kivi_ref_float_to_half.argtypes = [F]
        L.kivi_ref_float_to_half.restype = ctypes.c_uint16
        L.kivi_ref_bf16_to_float.argtypes = [ctypes.c_uint16]
        L.kivi_ref_bf16_to_float.restype = F
        L.kivi_ref_float_to_bf16.argtypes = [F]
        L.kivi_ref_float_to_bf16.restype = ctypes.c_uint16
        L.kivi_ref_widen_array.argtypes = [P, I64, I, P]
        L.kivi_ref_narrow_array.argtypes = [P, I64, I, P]
        L.kivi_ref_group_params.argtypes = [P, I64, I, P, P]
        L.kivi_ref_code.argtypes = [F, F, F, I]
        L.kivi_ref_recon.argtypes = [I, F, F]
        L.kivi_ref_recon.restype = F
        for name in ("kivi_ref_quant_keys_unpacked",
                     "kivi_ref_quant_values_unpacked",
                     "kivi_ref_quant_keys", "kivi_ref_quant_values"):
            getattr(L, name).argtypes = [P, I, I64, I64, I64, I, I64, P, P, P]
        L.kivi_ref_pack.argtypes = [P, I64, I64, I, P]
        L.kivi_ref_unpack.argtypes = [P, I64, I64, I, P]
        for name in ("kivi_ref_dequant_keys", "kivi_ref_dequant_values"):
            getattr(L, name).argtypes = [P, P, P, I64, I64, I64, I, I64, I, P]
        L.kivi_ref_sink_scores.argtypes = [P, I, I64, I64, I64, I64, P]
        L.kivi_ref_sink_select.argtypes = [P, I64, I64, I64, P]
        for name in ("kivi_ref_quant_keys_sink_unpacked",
                     "kivi_ref_quant_keys_sink"):
            getattr(L, name).argtypes = [P, I, I64, I64, I64, I64, I, I64, P,
                                         I64, P, P, P]
        L.kivi_ref_sink_gather.argtypes = [P, I64, I64, I64, I64, P, I64, P]
        L.kivi_ref_sink_restore.argtypes = [P, I64, I64, I64, I64, P, I64, P]
        L.kivi_ref_partition_top.argtypes = [P, I64, I64, I64, P, P]
        for name in ("kivi_ref_quant_keys_rows", "kivi_ref_quant_values_rows"):
            getattr(L, name).argtypes = [P, I, I64, I64, I64, I64, I, I64, P,
                                         I64, P, P, P]
        for name in ("kivi_ref_dequant_keys_rows",
                     "kivi_ref_dequant_values_rows"):
            getattr(L, name).argtypes = [P, P, P, I64, I64, I64, I64, I, I64,
                                         P, I64, I, P]
        self.L = L
        self.path = path

    @staticmethod
    def _check(st, what):
        if st != 0:
            raise ValueError(f"oracle {what}: bad arguments")

    # conversions ------------------------------------------------------------
    def widen(self, bits16, dtype):
        a = np.ascontiguousarray(bits16, dtype=np.uint16)
        out = np.zeros(a.shape, np.float32)
        self._check(self.L.kivi_ref_widen_array(_ptr(a), a.size, dtype,
                                                _ptr(out)), "widen")
        return out

    def narrow(self, f32, dtype):
        a = np.ascontiguousarray(f32, dtype=np.float32)
        out = np.zeros(a.shape, np.uint16)
        self._check(self.L.kivi_ref_narrow_array(_ptr(a), a.size, dtype,
                                                 _ptr(out)), "narrow")
        return out

    # one group / one element -----------------------------------------------
    def group_params(self, vals, bits):
        v = np.ascontiguousarray(vals, dtype=np.float32)
        sc = np.zeros(1, np.float32)
        z = np.zeros(1, np.float32)
        self._check(self.L.kivi_ref_group_params(_ptr(v), v.size, bits,
                                                 _ptr(sc), _ptr(z)),
                    "group_params")
        return sc[0], z[0]

    def code(self, f, scale, zero, bits):
        return self.L.kivi_ref_code(float(f), float(scale), float(zero), bits)

    def recon(self, c, scale, zero):
        return np.float32(self.L.kivi_ref_recon(int(c), float(scale),
                                                float(zero)))

    # tensors ----------------------------------------------------------------
    def _quant(self, name, x, dtype, bits, group, packed, key_params):
        x = np.ascontiguousarray(x, dtype=np.uint16)
        BH, S, D = x.shape
        if key_params:
            pshape = (BH, n_groups(S, group), D)
        else:
            pshape = (BH, S, n_groups(D, group))
        sc = np.zeros(pshape, np.float32)
        z = np.zeros(pshape, np.float32)
        if packed:
            if (D * bits) % 8:
                raise ValueError("D*bits must be a multiple of 8")
            codes = np.zeros((BH, S, D * bits // 8), np.uint8)
        else:
            codes = np.zeros((BH, S, D), np.uint8)
        self._check(getattr(self.L, name)(_ptr(x), dtype, BH, S, D, bits,
                                          group, _ptr(codes), _ptr(sc),
                                          _ptr(z)), name)
        return codes, sc, z

    def quant_keys(self, x, dtype, bits, group):
        """-> (packed [BH,S,D*bits/8] u8, scale [BH,NG,D], zero [BH,NG,D])"""
        return self._quant("kivi_ref_quant_keys", x, dtype, bits, group,
                           True, True)

    def quant_values(self, x, dtype, bits, group):
        """-> (packed [BH,S,D*bits/8] u8, scale [BH,S,NGD], zero [BH,S,NGD])"""
        return self._quant("kivi_ref_quant_values", x, dtype, bits, group,
                           True, False)

    def quant_keys_unpacked(self, x, dtype, bits, group):
        return self._quant("kivi_ref_quant_keys_unpacked", x, dtype, bits,
                           group, False, True)

    def quant_values_unpacked(self, x, dtype, bits, group):
        return self._quant("kivi_ref_quant_values_unpacked", x, dtype, bits,
                           group, False, False)

    def pack(self, codes, bits):
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        D = codes.shape[-1]
        rows = codes.size // D if D else 0
        out = np.zeros(codes.shape[:-1] + (D * bits // 8,), np.uint8)
        self._check(self.L.kivi_ref_pack(_ptr(codes), rows, D, bits,
                                         _ptr(out)), "pack")
        return out

    def unpack(self, packed, D, bits):
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        rb = D * bits // 8
        rows = packed.size // rb if rb else 0
        out = np.zeros(packed.shape[:-1] + (D,), np.uint8)
        self._check(self.L.kivi_ref_unpack(_ptr(packed), rows, D, bits,
                                           _ptr(out)), "unpack")
        return out

    def _dequant(self, name, packed, scale, zero, shape, bits, group,
                 out_dtype):
        BH, S, D = shape
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        scale = np.ascontiguousarray(scale, dtype=np.float32)
        zero = np.ascontiguousarray(zero, dtype=np.float32)
        out = np.zeros((BH, S, D), np.uint16)
        self._check(getattr(self.L, name)(_ptr(packed), _ptr(scale),
                                          _ptr(zero), BH, S, D, bits, group,
                                          out_dtype, _ptr(out)), name)
        return out

    def dequant_keys(self, packed, scale, zero, shape, bits, group,
                     out_dtype):
        return self._dequant("kivi_ref_dequant_keys", packed, scale, zero,
                             shape, bits, group, out_dtype)

    def dequant_values(self, packed, scale, zero, shape, bits, group,
                       out_dtype):
        return self._dequant("kivi_ref_dequant_values", packed, scale, zero,
                             shape, bits, group, out_dtype)

    # KIVI-Sink --------------------------------------------------------------
    def sink_scores(self, k, dtype, H):
        """k [B*H, S, D] -> float32 [B, S]: mean over heads of key L2 norms."""
        k = np.ascontiguousarray(k, dtype=np.uint16)
        BH, S, D = k.shape
        out = np.zeros((BH // H, S), np.float32)
        self._check(self.L.kivi_ref_sink_scores(_ptr(k), dtype, BH // H, H, S,
                                                D, _ptr(out)), "sink_scores")
        return out

    def sink_select(self, score, n_sink):
        """score [B, S] -> int32 [B, n_sink], highest first."""
        score = np.ascontiguousarray(score, dtype=np.float32)
        B, S = score.shape
        idx = np.zeros((B, n_sink), np.int32)
        self._check(self.L.kivi_ref_sink_select(_ptr(score), B, S, n_sink,
                                                _ptr(idx)), "sink_select")
        return idx

    def _quant_sink(self, name, x, dtype, H, bits, group, idx, packed):
        x = np.ascontiguousarray(x, dtype=np.uint16)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        BH, S, D = x.shape
        n_sink = idx.shape[1] if idx.ndim == 2 else 0
        sc = np.zeros((BH, n_groups(S, group), D), np.float32)
        z = np.zeros_like(sc)
        codes = np.zeros((BH, S, D * bits // 8 if packed else D), np.uint8)
        self._check(getattr(self.L, name)(_ptr(x), dtype, BH // H, H, S, D,
                                          bits, group, _ptr(idx), n_sink,
                                          _ptr(codes), _ptr(sc), _ptr(z)), name)
        return codes, sc, z

    def quant_keys_sink(self, x, dtype, H, bits, group, idx):
        """-> (packed codes, scale [BH,NG,D], zero [BH,NG,D]); idx [B, n_sink]"""
        return self._quant_sink("kivi_ref_quant_keys_sink", x, dtype, H, bits,
                                group, idx, True)

    def quant_keys_sink_unpacked(self, x, dtype, H, bits, group, idx):
        return self._quant_sink("kivi_ref_quant_keys_sink_unpacked", x, dtype,
                                H, bits, group, idx, False)

    def sink_gather(self, x, H, idx):
        """x [B*H, S, D] -> [B*H, n_sink, D] rows of the sinks."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        BH, S, D = x.shape
        out = np.zeros((BH, idx.shape[1], D), np.uint16)
        self._check(self.L.kivi_ref_sink_gather(_ptr(x), BH // H, H, S, D,
                                                _ptr(idx), idx.shape[1],
                                                _ptr(out)), "sink_gather")
        return out

    def sink_restore(self, x_sink, H, idx, out):
        """Copy the sink rows back into out [B*H, S, D]; returns a new array."""
        x_sink = np.ascontiguousarray(x_sink, dtype=np.uint16)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        out = np.array(out, dtype=np.uint16, copy=True, order="C")
        BH, S, D = out.shape
        self._check(self.L.kivi_ref_sink_restore(_ptr(x_sink), BH // H, H, S,
                                                 D, _ptr(idx), idx.shape[1],
                                                 _ptr(out)), "sink_restore")
        return out

    def sink_recon(self, x, dtype, H, bits, group, idx):
        """Plain-KIVI-with-sinks reconstruction of keys x: quantize with the
        sinks left out of calibration, dequantize, put the sink rows back."""
        BH, S, D = x.shape
        codes, sc, z = self.quant_keys_sink(x, dtype, H, bits, group, idx)
        deq = self.dequant_keys(codes, sc, z, (BH, S, D), bits, group, dtype)
        return self.sink_restore(self.sink_gather(x, H, idx), H, idx, deq)

    # per-token mixed precision -------------------------------------------
    def partition_top(self, score, n_hi):
        """score [B, S] -> (pos_hi [B, n_hi], pos_lo [B, S - n_hi]), int32,
        each ascending."""
        score = np.ascontiguousarray(score, dtype=np.float32)
        B, S = score.shape
        hi = np.zeros((B, n_hi), np.int32)
        lo = np.zeros((B, S - n_hi), np.int32)
        self._check(self.L.kivi_ref_partition_top(_ptr(score), B, S, n_hi,
                                                  _ptr(hi), _ptr(lo)),
                    "partition_top")
        return hi, lo

    def _quant_rows(self, name, x, dtype, H, bits, group, pos, keys):
        x = np.ascontiguousarray(x, dtype=np.uint16)
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        BH, S, D = x.shape
        n = pos.shape[1]
        pshape = (BH, n_groups(n, group), D) if keys else (BH, n, n_groups(D, group))
        sc = np.zeros(pshape, np.float32)
        z = np.zeros(pshape, np.float32)
        codes = np.zeros((BH, n, D * bits // 8), np.uint8)
        self._check(getattr(self.L, name)(_ptr(x), dtype, BH // H, H, S, D,
                                          bits, group, _ptr(pos), n,
                                          _ptr(codes), _ptr(sc), _ptr(z)), name)
        return codes, sc, z

    def quant_keys_rows(self, x, dtype, H, bits, group, pos):
        return self._quant_rows("kivi_ref_quant_keys_rows", x, dtype, H, bits,
                                group, pos, True)

    def quant_values_rows(self, x, dtype, H, bits, group, pos):
        return self._quant_rows("kivi_ref_quant_values_rows", x, dtype, H,
                                bits, group, pos, False)

    def _dequant_rows(self, name, codes, scale, zero, shape, H, bits, group,
                      pos, out_dtype, out):
        BH, S, D = shape
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        out = (np.zeros(shape, np.uint16) if out is None
               else np.array(out, dtype=np.uint16, copy=True, order="C"))
        args = [np.ascontiguousarray(a) for a in (codes, scale, zero)]
        self._check(getattr(self.L, name)(_ptr(args[0]), _ptr(args[1]),
                                          _ptr(args[2]), BH // H, H, S, D,
                                          bits, group, _ptr(pos), pos.shape[1],
                                          out_dtype, _ptr(out)), name)
        return out

    def dequant_keys_rows(self, codes, scale, zero, shape, H, bits, group,
                          pos, out_dtype, out=None):
        return self._dequant_rows("kivi_ref_dequant_keys_rows", codes, scale,
                                  zero, shape, H, bits, group, pos, out_dtype,
                                  out)

    def dequant_values_rows(self, codes, scale, zero, shape, H, bits, group,
                            pos, out_dtype, out=None):
        return self._dequant_rows("kivi_ref_dequant_values_rows", codes, scale,
                                  zero, shape, H, bits, group, pos, out_dtype,
                                  out)

    def mixed_recon(self, x, dtype, H, n_hi, hi_bits, lo_bits, group, keys):
        """The mixed-precision reconstruction of keys (keys=True, per-channel
        groups over each set's tokens) or values: the n_hi highest key-norm
        tokens of each sequence at hi_bits, the rest at lo_bits.  The ranking
        always comes from the keys, so for values pass the keys as `keys`."""
        kx = x if keys is True else keys
        hi, lo = self.partition_top(self.sink_scores(kx, dtype, H), n_hi)
        out = np.zeros(x.shape, np.uint16)
        q = self.quant_keys_rows if keys is True else self.quant_values_rows
        dq = self.dequant_keys_rows if keys is True else self.dequant_values_rows
        for pos, bits in ((hi, hi_bits), (lo, lo_bits)):
            if pos.shape[1] == 0:
                continue
            c, sc, z = q(x, dtype, H, bits, group, pos)
            out = dq(c, sc, z, x.shape, H, bits, group, pos, dtype, out)
        return out

    def cache(self, BH, D, S_max, R, G_k, G_v, bits, dtype):
        """A residual-window cache (kivi_ref_cache) over numpy arrays."""
        return OracleCache(self, BH, D, S_max, R, G_k, G_v, bits, dtype)


class _RefCache(ctypes.Structure):
    _fields_ = [("BH", ctypes.c_int64), ("D", ctypes.c_int64),
                ("S_max", ctypes.c_int64), ("R", ctypes.c_int64),
                ("G_k", ctypes.c_int64), ("G_v", ctypes.c_int64),
                ("bits", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("k_zero", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("v_zero", ctypes.c_void_p),
                ("T", ctypes.c_int64), ("Q", ctypes.c_int64)]


class OracleCache:
    """kivi_ref_cache with its arrays held here: append(k_new, v_new) with
    [BH, n, D] uint16 patterns; T, Q; the compressed store and the history
    as numpy arrays (k_codes, k_scale, ..., k, v)."""

    def __init__(self, oracle, BH, D, S_max, R, G_k, G_v, bits, dtype):
        self.o = oracle
        NG = n_groups(S_max, G_k)
        NGD = n_groups(D, G_v)
        rb = D * bits // 8
        self.k = np.zeros((BH, S_max, D), np.uint16)
        self.v = np.zeros((BH, S_max, D), np.uint16)
        self.k_codes = np.zeros((BH, S_max, rb), np.uint8)
        self.v_codes = np.zeros((BH, S_max, rb), np.uint8)
        self.k_scale = np.zeros((BH, NG, D), np.float32)
        self.k_zero = np.zeros((BH, NG, D), np.float32)
        self.v_scale = np.zeros((BH, S_max, NGD), np.float32)
        self.v_zero = np.zeros((BH, S_max, NGD), np.float32)
        self.c = _RefCache(BH, D, S_max, R, G_k, G_v, bits, dtype,
                           *[a.ctypes.data for a in (
                               self.k, self.v, self.k_codes, self.v_codes,
                               self.k_scale, self.k_zero, self.v_scale,
                               self.v_zero)], 0, 0)
        oracle.L.kivi_ref_cache_append.argtypes = [
            ctypes.POINTER(_RefCache), ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64]

    @property
    def T(self):
        return self.c.T

    @property
    def Q(self):
        return self.c.Q

    def dequantized(self, which):
        """The cache as the pages' attention sees it: tokens [0, Q)
        dequantized (to the cache's 16-bit type, exactly as the dequantizers
        produce them) followed by the exact tokens [Q, T); [BH, T, D] uint16
        patterns."""
        c = self.c
        Q, T = c.Q, c.T
        if which == "K":
            deq = self.o.dequant_keys(
                np.ascontiguousarray(self.k_codes[:, :Q]),
                np.ascontiguousarray(self.k_scale[:, :Q // c.G_k]),
                np.ascontiguousarray(self.k_zero[:, :Q // c.G_k]),
                (c.BH, Q, c.D), c.bits, c.G_k, c.dtype)
            tail = self.k[:, Q:T]
        else:
            deq = self.o.dequant_values(
                np.ascontiguousarray(self.v_codes[:, :Q]),
                np.ascontiguousarray(self.v_scale[:, :Q]),
                np.ascontiguousarray(self.v_zero[:, :Q]),
                (c.BH, Q, c.D), c.bits, c.G_v, c.dtype)
            tail = self.v[:, Q:T]
        return np.concatenate([deq, tail], axis=1)

    def reconstructed(self, which):
        """The cache as attention over the packed store reads it (the
        contract of kivi_cache_attend): tokens [0, Q) as code * scale + zero
        with their group's params, evaluated in float64 (the product is
        exact, the sum rounded once at 2^-53) and never rounded to fp32 or
        to the 16-bit type, followed by the exact tokens [Q, T) widened;
        float64 [BH, T, D]."""
        c = self.c
        Q, T, D = c.Q, c.T, c.D
        if which == "K":
            codes = self.o.unpack(np.ascontiguousarray(self.k_codes[:, :Q]),
                                  D, c.bits)
            sc = np.repeat(self.k_scale[:, :Q // c.G_k], c.G_k, axis=1)
            z = np.repeat(self.k_zero[:, :Q // c.G_k], c.G_k, axis=1)
            hist = self.k
        else:
            codes = self.o.unpack(np.ascontiguousarray(self.v_codes[:, :Q]),
                                  D, c.bits)
            sc = np.repeat(self.v_scale[:, :Q], c.G_v, axis=2)[:, :, :D]
            z = np.repeat(self.v_zero[:, :Q], c.G_v, axis=2)[:, :, :D]
            hist = self.v
        rec = (codes.astype(np.float64) * sc.astype(np.float64)
               + z.astype(np.float64))
        tail = self.o.widen(np.ascontiguousarray(hist[:, Q:T]),
                            c.dtype).astype(np.float64)
        return np.concatenate([rec, tail], axis=1)

    @staticmethod
    def _softmax_attend(qf, Kf, Vf, sm_scale):
        """softmax_t(sm_scale * q . K_t) V_t in float64 for every (bh, query
        head); qf [BH, n_q, D], Kf and Vf [BH, T, D]."""
        s = np.einsum("bjd,btd->bjt", qf, Kf) * float(sm_scale)
        s -= s.max(axis=2, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=2, keepdims=True)
        return np.einsum("bjt,btd->bjd", p, Vf)

    def attend(self, q, sm_scale):
        """Decode attention of q [BH, n_q, D] (16-bit patterns; n_q query
        heads share each KV head) over all T cached tokens, in float64:
        softmax(sm_scale * q K^T) V with K, V from dequantized(), the
        reading in which the pages' fetch hands attention a dequantized
        16-bit cache.  Returns float64 [BH, n_q, D]."""
        dt = self.c.dtype
        Kf = self.o.widen(self.dequantized("K"), dt).astype(np.float64)
        Vf = self.o.widen(self.dequantized("V"), dt).astype(np.float64)
        qf = self.o.widen(np.ascontiguousarray(q), dt).astype(np.float64)
        return self._softmax_attend(qf, Kf, Vf, sm_scale)

    def attend_exact(self, q, sm_scale):
        """Decode attention as kivi_cache_attend defines it: as attend(),
        but over reconstructed() (quantized tokens never rounded to 16 bits)
        and with sm_scale taken as the fp32 value the call receives.
        Returns float64 [BH, n_q, D]."""
        dt = self.c.dtype
        qf = self.o.widen(np.ascontiguousarray(q), dt).astype(np.float64)
        sm = float(np.float32(sm_scale))
        return self._softmax_attend(qf, self.reconstructed("K"),
                                    self.reconstructed("V"), sm)

    def append(self, k_new, v_new):
        k_new = np.ascontiguousarray(k_new, dtype=np.uint16)
        v_new = np.ascontiguousarray(v_new, dtype=np.uint16)
        n = k_new.shape[1] if k_new.ndim == 3 else 0
        self.o._check(self.o.L.kivi_ref_cache_append(
            ctypes.byref(self.c), _ptr(k_new), _ptr(v_new), n),
            "cache_append")


_default = None


def default():
    global _default
    if _default is None:
        if not os.path.exists(LIB):
            build()
        _default = Oracle(LIB)
    return _default


def __getattr__(name):
    # module-level access to the default oracle's methods
    if name.startswith("_"):
        raise AttributeError(name)
    return getattr(default(), name)
