"""KIVI KV-cache flush for MI355X: Python binding of libkivi.so.

Argument marshalling only: every step of quantization and dequantization
runs in the HIP kernels behind the C ABI declared in include/kivi.h.  Torch
tensors supply device memory and the current HIP stream (every call also
takes stream=, a torch.cuda.Stream or a raw handle); outputs that are
not passed in are allocated with torch on the input's device.  Importing
this package works without the library (so that its `build` submodule can
run from a clean checkout), but the first call of any function below fails
loudly with ImportError if the library has not been built: there is no
fallback of any kind.

Functions (same names as the C ABI):
    kivi_quant_keys(k, bits, group)      -> (codes, scale, zero)
    kivi_quant_values(v, bits, group)    -> (codes, scale, zero)
    kivi_dequant_keys(codes, scale, zero, bits, group, out_dtype) -> out
    kivi_dequant_values(codes, scale, zero, bits, group, out_dtype) -> out
    kivi_quant_dequant_keys(k, bits, group, with_codes=True)
        -> (recon, codes, scale, zero) or recon when with_codes=False
    kivi_quant_dequant_values(...)       likewise
    kivi_codes_bytes, kivi_key_param_count, kivi_value_param_count,
    kivi_status_string
    KiviCache(BH, D, S_max, R, G_k, G_v, bits, dtype), kivi_cache_append
        the residual-window cache (recent tokens kept exact, whole key
        groups flushed into packed storage as they age out), and
        kivi_cache_attend, decode attention reading the packed store
    kivi_sink_select, kivi_quant_keys_sink, kivi_sink_gather,
    kivi_sink_restore
        KIVI-Sink: the highest key-norm tokens kept in 16-bit form and left
        out of the key groups' min/max
    kivi_key_scores, kivi_partition_top, kivi_quant_{keys,values}_rows,
    kivi_dequant_{keys,values}_rows
        per-token mixed precision: the highest key-norm tokens at hi_bits,
        the rest at lo_bits, each set quantized as its own tensor
Tensors are [BH, S, D] (or [B, H, S, D], flattened to BH = B*H), contiguous,
float16 or bfloat16; codes are uint8 [..., S, D*bits/8]; key params are
float32 [..., ceil(S/group), D]; value params float32 [..., S, ceil(D/group)].
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkivi.so")
# kivi_cache_attend_noalloc's per-device workspace (include/kivi.h)
ATTEND_SCRATCH_BYTES = 32 << 20

KIVI_FP16 = 0
KIVI_BF16 = 1

STATUS = {
    0: "KIVI_OK", 1: "KIVI_ERR_NULL", 2: "KIVI_ERR_SHAPE", 3: "KIVI_ERR_BITS",
    4: "KIVI_ERR_GROUP", 5: "KIVI_ERR_DTYPE", 6: "KIVI_ERR_ALIGN",
    7: "KIVI_ERR_LAUNCH", 8: "KIVI_ERR_SCRATCH",
}


class KiviError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} "
                         f"({_lib().kivi_status_string(status).decode()})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m "
            "kv_cache_quantization_kivi_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    quant = [P, I, I64, I64, I64, I, I64, P, P, P, P]
    L.kivi_quant_keys.argtypes = quant
    L.kivi_quant_values.argtypes = quant
    fused = [P, I, I64, I64, I64, I, I64, P, P, P, P, P]
    L.kivi_quant_dequant_keys.argtypes = fused
    L.kivi_quant_dequant_values.argtypes = fused
    dq = [P, P, P, I64, I64, I64, I, I64, I, P, P]
    L.kivi_dequant_keys.argtypes = dq
    L.kivi_dequant_values.argtypes = dq
    L.kivi_quant_kv.argtypes = [P, P, I, I64, I64, I64, I, I64, I64] + [P] * 7
    L.kivi_quant_dequant_kv.argtypes = [P, P, I, I64, I64, I64, I, I64, I64] + [P] * 9
    L.kivi_dequant_kv.argtypes = [P] * 6 + [I64, I64, I64, I, I64, I64, I, P, P, P]
    for name in ("kivi_quant_keys", "kivi_quant_values",
                 "kivi_quant_dequant_keys", "kivi_quant_dequant_values",
                 "kivi_dequant_keys", "kivi_dequant_values", "kivi_quant_kv",
                 "kivi_quant_dequant_kv", "kivi_dequant_kv"):
        getattr(L, name).restype = I
    L.kivi_time_next_launch.argtypes = [P, P]
    L.kivi_time_next_launch.restype = None
    L.kivi_selftest_division.argtypes = [P, P]
    L.kivi_selftest_division.restype = I
    L.kivi_codes_bytes.argtypes = [I64, I64, I64, I]
    L.kivi_codes_bytes.restype = I64
    L.kivi_key_param_count.argtypes = [I64, I64, I64, I64]
    L.kivi_key_param_count.restype = I64
    L.kivi_value_param_count.argtypes = [I64, I64, I64, I64]
    L.kivi_value_param_count.restype = I64
    L.kivi_sink_select.argtypes = [P, I, I64, I64, I64, I64, I64, P, P, P]
    L.kivi_quant_keys_sink.argtypes = [P, I, I64, I64, I64, I64, I, I64, P,
                                       I64, P, P, P, P, P]
    copy = [P, I64, I64, I64, I64, P, I64, P, P]
    L.kivi_sink_gather.argtypes = copy
    L.kivi_sink_restore.argtypes = copy
    for name in ("kivi_sink_select", "kivi_quant_keys_sink",
                 "kivi_sink_gather", "kivi_sink_restore"):
        getattr(L, name).restype = I
    L.kivi_partition_top.argtypes = [P, I64, I64, I64, P, P, P]
    qrows = [P, I, I64, I64, I64, I64, I, I64, P, I64, P, P, P, P]
    L.kivi_quant_keys_rows.argtypes = qrows
    L.kivi_quant_values_rows.argtypes = qrows
    drows = [P, P, P, I64, I64, I64, I64, I, I64, P, I64, I, P, P]
    L.kivi_dequant_keys_rows.argtypes = drows
    L.kivi_dequant_values_rows.argtypes = drows
    for name in ("kivi_partition_top", "kivi_quant_keys_rows",
                 "kivi_quant_values_rows", "kivi_dequant_keys_rows",
                 "kivi_dequant_values_rows"):
        getattr(L, name).restype = I
    L.kivi_status_string.argtypes = [I]
    L.kivi_status_string.restype = ctypes.c_char_p
    C = ctypes.POINTER(_Cache)
    L.kivi_cache_append.argtypes = [C, P, P, I64, P]
    L.kivi_cache_append.restype = I
    L.kivi_cache_attend.argtypes = [C, P, I64, ctypes.c_float, P, P, I64, P]
    L.kivi_cache_attend.restype = I
    L.kivi_cache_attend_noalloc.argtypes = [C, P, I64, ctypes.c_float, P, P]
    L.kivi_cache_attend_noalloc.restype = I
    L.kivi_cache_attend_work_bytes.argtypes = [C, I64]
    L.kivi_cache_attend_work_bytes.restype = I64
    L.kivi_launch_count.argtypes = []
    L.kivi_launch_count.restype = I64
    return L


_C = None


def _lib():
    """The loaded libkivi.so (loaded on first use; ImportError if absent)."""
    global _C
    if _C is None:
        _C = _load()
    return _C


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------

def _dtype_code(dt):
    if dt == torch.float16:
        return KIVI_FP16
    if dt == torch.bfloat16:
        return KIVI_BF16
    raise TypeError(f"KIVI tensors are float16 or bfloat16, got {dt}")


def _torch_dtype(code):
    return torch.float16 if code == KIVI_FP16 else torch.bfloat16


def _bsd(x):
    """Leading dims flattened into BH; returns (BH, S, D, lead_shape)."""
    if x.dim() < 2:
        raise ValueError("expected a [..., S, D] tensor")
    if not x.is_contiguous():
        raise ValueError("KIVI tensors must be contiguous")
    S, D = x.shape[-2], x.shape[-1]
    lead = tuple(x.shape[:-2])
    BH = 1
    for n in lead:
        BH *= n
    return BH, S, D, lead


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


# torch's current stream as a raw handle, without building a Stream object
# (a few microseconds per call, which a one-token cache append notices)
_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(device, stream):
    """The stream as an int handle: `stream` if given (a torch.cuda.Stream
    or a raw hipStream_t handle), else torch's current stream on `device`."""
    if stream is not None:
        return int(getattr(stream, "cuda_stream", stream))
    if _RAW_STREAM is not None:
        idx = device.index
        return _RAW_STREAM(idx if idx is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(device).cuda_stream


def _stream(device, stream):
    return ctypes.c_void_p(_stream_handle(device, stream))


def _check(st, what):
    if st != 0:
        raise KiviError(st, what)


def _ngroups(n, g):
    return (n + g - 1) // g


def _alloc_quant(x, keys, bits, group, codes, scale, zero):
    BH, S, D, lead = _bsd(x)
    if codes is None:
        codes = torch.empty(lead + (S, D * bits // 8), dtype=torch.uint8,
                            device=x.device)
    pshape = lead + ((_ngroups(S, group), D) if keys
                     else (S, _ngroups(D, group)))
    if scale is None:
        scale = torch.empty(pshape, dtype=torch.float32, device=x.device)
    if zero is None:
        zero = torch.empty(pshape, dtype=torch.float32, device=x.device)
    return codes, scale, zero


# --------------------------------------------------------------------------
# the C ABI, tensor level
# --------------------------------------------------------------------------

def _quant(name, keys, x, bits, group, codes, scale, zero, stream):
    BH, S, D, _ = _bsd(x)
    if group < 1:
        _check(4, name)
    codes, scale, zero = _alloc_quant(x, keys, bits, group, codes, scale, zero)
    st = getattr(_lib(), name)(_ptr(x), _dtype_code(x.dtype), BH, S, D, bits,
                           group, _ptr(codes), _ptr(scale), _ptr(zero),
                           _stream(x.device, stream))
    _check(st, name)
    return codes, scale, zero


def kivi_quant_keys(k, bits=2, group=32, codes=None, scale=None, zero=None,
                    stream=None):
    """Per-channel key quantization -> (codes, scale, zero)."""
    return _quant("kivi_quant_keys", True, k, bits, group, codes, scale, zero,
                  stream)


def kivi_quant_values(v, bits=2, group=32, codes=None, scale=None, zero=None,
                      stream=None):
    """Per-token value quantization -> (codes, scale, zero)."""
    return _quant("kivi_quant_values", False, v, bits, group, codes, scale,
                  zero, stream)


def _fused(name, keys, x, bits, group, with_codes, recon, codes, scale, zero,
           stream):
    BH, S, D, _ = _bsd(x)
    if group < 1:
        _check(4, name)
    if recon is None:
        recon = torch.empty_like(x)
    if with_codes:
        codes, scale, zero = _alloc_quant(x, keys, bits, group, codes, scale,
                                          zero)
    else:
        codes = scale = zero = None
    st = getattr(_lib(), name)(_ptr(x), _dtype_code(x.dtype), BH, S, D, bits,
                           group, _ptr(codes), _ptr(scale), _ptr(zero),
                           _ptr(recon), _stream(x.device, stream))
    _check(st, name)
    return (recon, codes, scale, zero) if with_codes else recon


def kivi_quant_dequant_keys(k, bits=2, group=32, with_codes=True, recon=None,
                            codes=None, scale=None, zero=None, stream=None):
    """Fused key quantize -> dequantize in one pass."""
    return _fused("kivi_quant_dequant_keys", True, k, bits, group, with_codes,
                  recon, codes, scale, zero, stream)


def kivi_quant_dequant_values(v, bits=2, group=32, with_codes=True,
                              recon=None, codes=None, scale=None, zero=None,
                              stream=None):
    """Fused value quantize -> dequantize in one pass."""
    return _fused("kivi_quant_dequant_values", False, v, bits, group,
                  with_codes, recon, codes, scale, zero, stream)


def _dequant(name, keys, codes, scale, zero, bits, group, out_dtype, out,
             stream):
    if codes.dim() < 2 or not codes.is_contiguous():
        raise ValueError("codes must be a contiguous [..., S, D*bits/8] tensor")
    lead = tuple(codes.shape[:-2])
    S = codes.shape[-2]
    D = codes.shape[-1] * 8 // bits if bits in (1, 2, 4, 8) else 0
    BH = 1
    for n in lead:
        BH *= n
    if out is None:
        out = torch.empty(lead + (S, D), dtype=out_dtype, device=codes.device)
    st = getattr(_lib(), name)(_ptr(codes), _ptr(scale), _ptr(zero), BH, S, D,
                           bits, group, _dtype_code(out.dtype), _ptr(out),
                           _stream(codes.device, stream))
    _check(st, name)
    return out


def kivi_dequant_keys(codes, scale, zero, bits=2, group=32,
                      out_dtype=torch.float16, out=None, stream=None):
    """Key dequantization -> [..., S, D] of out_dtype."""
    return _dequant("kivi_dequant_keys", True, codes, scale, zero, bits,
                    group, out_dtype, out, stream)


def kivi_dequant_values(codes, scale, zero, bits=2, group=32,
                        out_dtype=torch.float16, out=None, stream=None):
    """Value dequantization -> [..., S, D] of out_dtype."""
    return _dequant("kivi_dequant_values", False, codes, scale, zero, bits,
                    group, out_dtype, out, stream)


def _same_kv(k, v):
    if k.shape != v.shape or k.dtype != v.dtype:
        raise ValueError("keys and values must share shape and dtype")


def kivi_quant_kv(k, v, bits=2, group_k=32, group_v=32, k_out=None,
                  v_out=None, stream=None):
    """Keys and values of one flush in one call (one launch for small
    flushes) -> ((k_codes, k_scale, k_zero), (v_codes, v_scale, v_zero)).
    k_out / v_out: optional preallocated (codes, scale, zero) triples."""
    _same_kv(k, v)
    BH, S, D, _ = _bsd(k)
    if group_k < 1 or group_v < 1:
        _check(4, "kivi_quant_kv")
    kq = _alloc_quant(k, True, bits, group_k, *(k_out or (None,) * 3))
    vq = _alloc_quant(v, False, bits, group_v, *(v_out or (None,) * 3))
    st = _lib().kivi_quant_kv(_ptr(k), _ptr(v), _dtype_code(k.dtype), BH, S, D,
                              bits, group_k, group_v, *map(_ptr, kq),
                              *map(_ptr, vq), _stream(k.device, stream))
    _check(st, "kivi_quant_kv")
    return kq, vq


def kivi_quant_dequant_kv(k, v, bits=2, group_k=32, group_v=32,
                          with_codes=True, k_recon=None, v_recon=None,
                          k_out=None, v_out=None, stream=None):
    """Fused quantize -> dequantize of keys and values in one call ->
    (k_recon, v_recon[, (k codes, scale, zero), (v codes, scale, zero)])."""
    _same_kv(k, v)
    BH, S, D, _ = _bsd(k)
    if group_k < 1 or group_v < 1:
        _check(4, "kivi_quant_dequant_kv")
    k_recon = torch.empty_like(k) if k_recon is None else k_recon
    v_recon = torch.empty_like(v) if v_recon is None else v_recon
    if with_codes:
        kq = _alloc_quant(k, True, bits, group_k, *(k_out or (None,) * 3))
        vq = _alloc_quant(v, False, bits, group_v, *(v_out or (None,) * 3))
    else:
        kq = vq = (None, None, None)
    st = _lib().kivi_quant_dequant_kv(
        _ptr(k), _ptr(v), _dtype_code(k.dtype), BH, S, D, bits, group_k,
        group_v, *map(_ptr, kq), *map(_ptr, vq), _ptr(k_recon), _ptr(v_recon),
        _stream(k.device, stream))
    _check(st, "kivi_quant_dequant_kv")
    return (k_recon, v_recon, kq, vq) if with_codes else (k_recon, v_recon)


def kivi_dequant_kv(kq, vq, bits=2, group_k=32, group_v=32,
                    out_dtype=torch.float16, k_out=None, v_out=None,
                    stream=None):
    """Keys and values dequantized in one call from (codes, scale, zero)
    triples -> (k, v) of out_dtype."""
    kc, vc = kq[0], vq[0]
    if kc.shape != vc.shape or kc.dim() < 2 or not kc.is_contiguous() \
            or not vc.is_contiguous():
        raise ValueError("codes must be contiguous [..., S, D*bits/8] tensors "
                         "of one shape")
    lead = tuple(kc.shape[:-2])
    S = kc.shape[-2]
    D = kc.shape[-1] * 8 // bits if bits in (1, 2, 4, 8) else 0
    BH = 1
    for n in lead:
        BH *= n
    if k_out is None:
        k_out = torch.empty(lead + (S, D), dtype=out_dtype, device=kc.device)
    if v_out is None:
        v_out = torch.empty(lead + (S, D), dtype=out_dtype, device=kc.device)
    st = _lib().kivi_dequant_kv(*map(_ptr, kq), *map(_ptr, vq), BH, S, D, bits,
                                group_k, group_v, _dtype_code(k_out.dtype),
                                _ptr(k_out), _ptr(v_out),
                                _stream(kc.device, stream))
    _check(st, "kivi_dequant_kv")
    return k_out, v_out


# --------------------------------------------------------------------------
# KIVI-Sink
# --------------------------------------------------------------------------

def _bhsd(x, H):
    """(B, H, S, D) of a [B, H, S, D] tensor, or of [..., S, D] with the
    given H heads per sequence (the flattened rows must be B*H)."""
    BH, S, D, lead = _bsd(x)
    if x.dim() == 4 and H is None:
        H = x.shape[1]
    if H is None or H < 1 or BH % H:
        raise ValueError(f"cannot split {BH} rows into sequences of H={H} heads")
    return BH // H, H, S, D


def _idx_arg(idx):
    if idx.dtype != torch.int32 or idx.dim() != 2 or not idx.is_contiguous():
        raise ValueError("sink lists are contiguous int32 [B, n_sink] tensors")
    return idx.shape[1]


def kivi_sink_select(k, n_sink, H=None, score=None, idx=None, stream=None):
    """Per-sequence sinks of keys [B, H, S, D] -> (idx int32 [B, n_sink],
    score float32 [B, S]): the n_sink highest mean key L2 norms, highest
    first."""
    B, H, S, D = _bhsd(k, H)
    if score is None:
        score = torch.empty((B, S), dtype=torch.float32, device=k.device)
    if idx is None:
        idx = torch.empty((B, max(n_sink, 0)), dtype=torch.int32, device=k.device)
    st = _lib().kivi_sink_select(_ptr(k), _dtype_code(k.dtype), B, H, S, D,
                                 n_sink, _ptr(score), _ptr(idx),
                                 _stream(k.device, stream))
    _check(st, "kivi_sink_select")
    return idx, score


def kivi_quant_keys_sink(k, idx, bits=2, group=32, H=None, with_codes=True,
                         with_recon=False, codes=None, scale=None, zero=None,
                         recon=None, stream=None):
    """Per-channel key quantization with the sinks idx [B, n_sink] left out
    of every group's min/max.  Returns (codes, scale, zero), with the
    reconstruction first when with_recon, or the reconstruction alone when
    not with_codes."""
    B, H, S, D = _bhsd(k, H)
    n_sink = _idx_arg(idx)
    if group < 1:
        _check(4, "kivi_quant_keys_sink")
    if not with_codes:
        with_recon = True
    if with_recon and recon is None:
        recon = torch.empty_like(k)
    if with_codes:
        codes, scale, zero = _alloc_quant(k, True, bits, group, codes, scale,
                                          zero)
    else:
        codes = scale = zero = None
    st = _lib().kivi_quant_keys_sink(
        _ptr(k), _dtype_code(k.dtype), B, H, S, D, bits, group, _ptr(idx),
        n_sink, _ptr(codes), _ptr(scale), _ptr(zero),
        _ptr(recon) if with_recon else None, _stream(k.device, stream))
    _check(st, "kivi_quant_keys_sink")
    if not with_codes:
        return recon
    return (recon, codes, scale, zero) if with_recon else (codes, scale, zero)


def kivi_sink_gather(x, idx, H=None, out=None, stream=None):
    """The sinks' rows of x [B, H, S, D] -> [B, H, n_sink, D]."""
    B, H, S, D = _bhsd(x, H)
    n_sink = _idx_arg(idx)
    if out is None:
        out = torch.empty(tuple(x.shape[:-2]) + (n_sink, D), dtype=x.dtype,
                          device=x.device)
    st = _lib().kivi_sink_gather(_ptr(x), B, H, S, D, _ptr(idx), n_sink,
                                 _ptr(out), _stream(x.device, stream))
    _check(st, "kivi_sink_gather")
    return out


def kivi_sink_restore(x_sink, idx, out, H=None, stream=None):
    """Write the sink rows x_sink [B, H, n_sink, D] back into out
    [B, H, S, D] (in place); returns out."""
    B, H, S, D = _bhsd(out, H)
    n_sink = _idx_arg(idx)
    st = _lib().kivi_sink_restore(_ptr(x_sink), B, H, S, D, _ptr(idx), n_sink,
                                  _ptr(out), _stream(out.device, stream))
    _check(st, "kivi_sink_restore")
    return out


# --------------------------------------------------------------------------
# per-token mixed precision
# --------------------------------------------------------------------------

def kivi_key_scores(k, H=None, score=None, stream=None):
    """Mean key L2 norm over the heads of each sequence, float32 [B, S]
    (kivi_sink_select with n_sink = 0)."""
    B, H, S, D = _bhsd(k, H)
    _, score = kivi_sink_select(k, 0, H=H, score=score, stream=stream)
    return score


def kivi_partition_top(score, n_hi, pos_hi=None, pos_lo=None, stream=None):
    """score float32 [B, S] -> (pos_hi int32 [B, n_hi], pos_lo [B, S - n_hi]):
    the n_hi highest scores' positions and the rest, each ascending."""
    if score.dtype != torch.float32 or score.dim() != 2 or not score.is_contiguous():
        raise ValueError("score must be a contiguous float32 [B, S] tensor")
    B, S = score.shape
    if pos_hi is None:
        pos_hi = torch.empty((B, max(n_hi, 0)), dtype=torch.int32, device=score.device)
    if pos_lo is None:
        pos_lo = torch.empty((B, max(S - n_hi, 0)), dtype=torch.int32,
                             device=score.device)
    st = _lib().kivi_partition_top(_ptr(score), B, S, n_hi, _ptr(pos_hi),
                                   _ptr(pos_lo), _stream(score.device, stream))
    _check(st, "kivi_partition_top")
    return pos_hi, pos_lo


def _quant_rows(name, keys, x, pos, bits, group, H, codes, scale, zero,
                stream):
    B, H, S, D = _bhsd(x, H)
    n = _idx_arg(pos)
    lead = (B, H) if x.dim() == 4 else (B * H,)
    if codes is None:
        codes = torch.empty(lead + (n, D * bits // 8), dtype=torch.uint8,
                            device=x.device)
    pshape = lead + ((_ngroups(n, max(group, 1)), D) if keys
                     else (n, _ngroups(D, max(group, 1))))
    if scale is None:
        scale = torch.empty(pshape, dtype=torch.float32, device=x.device)
    if zero is None:
        zero = torch.empty(pshape, dtype=torch.float32, device=x.device)
    st = getattr(_lib(), name)(_ptr(x), _dtype_code(x.dtype), B, H, S, D, bits,
                               group, _ptr(pos), n, _ptr(codes), _ptr(scale),
                               _ptr(zero), _stream(x.device, stream))
    _check(st, name)
    return codes, scale, zero


def kivi_quant_keys_rows(k, pos, bits=2, group=32, H=None, codes=None,
                         scale=None, zero=None, stream=None):
    """Per-channel key quantization of the listed tokens pos [B, n] as one
    tensor -> (codes [.., n, D*bits/8], scale, zero [.., ceil(n/group), D])."""
    return _quant_rows("kivi_quant_keys_rows", True, k, pos, bits, group, H,
                       codes, scale, zero, stream)


def kivi_quant_values_rows(v, pos, bits=2, group=32, H=None, codes=None,
                           scale=None, zero=None, stream=None):
    """Per-token value quantization of the listed tokens -> (codes, scale,
    zero [.., n, ceil(D/group)])."""
    return _quant_rows("kivi_quant_values_rows", False, v, pos, bits, group, H,
                       codes, scale, zero, stream)


def _dequant_rows(name, codes, scale, zero, pos, out, bits, group, H, stream):
    B, H, S, D = _bhsd(out, H)
    n = _idx_arg(pos)
    st = getattr(_lib(), name)(_ptr(codes), _ptr(scale), _ptr(zero), B, H, S,
                               D, bits, group, _ptr(pos), n,
                               _dtype_code(out.dtype), _ptr(out),
                               _stream(out.device, stream))
    _check(st, name)
    return out


def kivi_dequant_keys_rows(codes, scale, zero, pos, out, bits=2, group=32,
                           H=None, stream=None):
    """Dequantize a listed key set into its rows of out [B, H, S, D]."""
    return _dequant_rows("kivi_dequant_keys_rows", codes, scale, zero, pos,
                         out, bits, group, H, stream)


def kivi_dequant_values_rows(codes, scale, zero, pos, out, bits=2, group=32,
                             H=None, stream=None):
    """Dequantize a listed value set into its rows of out [B, H, S, D]."""
    return _dequant_rows("kivi_dequant_values_rows", codes, scale, zero, pos,
                         out, bits, group, H, stream)


class _Cache(ctypes.Structure):
    _fields_ = [("BH", ctypes.c_int64), ("D", ctypes.c_int64),
                ("S_max", ctypes.c_int64), ("R", ctypes.c_int64),
                ("G_k", ctypes.c_int64), ("G_v", ctypes.c_int64),
                ("ring", ctypes.c_int64), ("bits", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("k_ring", ctypes.c_void_p),
                ("v_ring", ctypes.c_void_p), ("k_codes", ctypes.c_void_p),
                ("v_codes", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("k_zero", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("v_zero", ctypes.c_void_p), ("T", ctypes.c_int64),
                ("Q", ctypes.c_int64)]


class KiviCache:
    """A residual-window KIVI cache (kivi_cache / kivi_cache_append): the
    device buffers are torch tensors held here, the counters live in the C
    struct.  append(k_new, v_new) takes [BH, n, D] (or [..., n, D]) tensors
    of the cache's dtype on its device and enqueues on the current stream.
    Attributes: k_ring, v_ring [BH, ring, D]; k_codes, v_codes
    [BH, S_max, D*bits/8]; k_scale, k_zero [BH, ceil(S_max/G_k), D];
    v_scale, v_zero [BH, S_max, ceil(D/G_v)]; T, Q."""

    def __init__(self, BH, D, S_max, R=32, G_k=32, G_v=32, bits=2,
                 dtype=torch.float16, device="cuda", ring=None):
        if ring is None:
            ring = ((R + G_k) + G_k - 1) // G_k * G_k
        dev = torch.device(device)
        rb = D * bits // 8
        self.k_ring = torch.empty((BH, ring, D), dtype=dtype, device=dev)
        self.v_ring = torch.empty((BH, ring, D), dtype=dtype, device=dev)
        self.k_codes = torch.zeros((BH, S_max, rb), dtype=torch.uint8,
                                   device=dev)
        self.v_codes = torch.zeros((BH, S_max, rb), dtype=torch.uint8,
                                   device=dev)
        ng = _ngroups(S_max, G_k) if G_k > 0 else 0
        ngd = _ngroups(D, G_v) if G_v > 0 else 0
        f32 = dict(dtype=torch.float32, device=dev)
        self.k_scale = torch.zeros((BH, ng, D), **f32)
        self.k_zero = torch.zeros((BH, ng, D), **f32)
        self.v_scale = torch.zeros((BH, S_max, ngd), **f32)
        self.v_zero = torch.zeros((BH, S_max, ngd), **f32)
        self.dtype = dtype
        self.c = _Cache(BH, D, S_max, R, G_k, G_v, ring, bits,
                        _dtype_code(dtype), *[t.data_ptr() for t in (
                            self.k_ring, self.v_ring, self.k_codes,
                            self.v_codes, self.k_scale, self.k_zero,
                            self.v_scale, self.v_zero)], 0, 0)
        self._cref = ctypes.byref(self.c)      # reused by every call

    @property
    def T(self):
        return self.c.T

    @property
    def Q(self):
        return self.c.Q

    def append(self, k_new, v_new, stream=None):
        """Append n tokens of every bh and flush what ages out."""
        for t in (k_new, v_new):
            if t.dtype != self.dtype or not t.is_contiguous():
                raise ValueError("k_new, v_new: contiguous tensors of the "
                                 "cache's dtype")
        n = k_new.shape[-2]
        if v_new.shape != k_new.shape:
            raise ValueError("k_new and v_new differ in shape")
        # every argument type is declared, so plain ints marshal directly
        st = _lib().kivi_cache_append(self._cref, k_new.data_ptr(),
                                      v_new.data_ptr(), n,
                                      _stream_handle(k_new.device, stream))
        if st != 0:
            raise KiviError(st, "kivi_cache_append")

    def attend(self, q, sm_scale, out=None, work=None, stream=None):
        """Decode attention of q [BH, n_q, D] (the cache's dtype) over the
        cache's T tokens, reading the packed store (kivi_cache_attend);
        returns out [BH, n_q, D].  `work` (uint8 device tensor) is allocated
        if not given."""
        if q.dtype != self.dtype or not q.is_contiguous():
            raise ValueError("q: a contiguous tensor of the cache's dtype")
        n_q = q.shape[-2]
        L = _lib()
        if out is None:
            out = torch.empty_like(q)
        if work is None:
            nb = L.kivi_cache_attend_work_bytes(self._cref, n_q)
            work = torch.empty(max(nb, 16), dtype=torch.uint8,
                               device=q.device)
        st = L.kivi_cache_attend(self._cref, q.data_ptr(), n_q,
                                 float(sm_scale), out.data_ptr(),
                                 work.data_ptr(), work.numel(),
                                 _stream_handle(q.device, stream))
        _check(st, "kivi_cache_attend")
        return out

    def attend_noalloc(self, q, sm_scale, out, stream=None):
        """As attend(), through kivi_cache_attend_noalloc: the workspace is
        the library's own per-device buffer and nothing is allocated (out
        must be given)."""
        if q.dtype != self.dtype or not q.is_contiguous():
            raise ValueError("q: a contiguous tensor of the cache's dtype")
        if out is None or out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out: a tensor shaped and typed like q")
        L = _lib()
        st = L.kivi_cache_attend_noalloc(self._cref, q.data_ptr(),
                                         q.shape[-2], float(sm_scale),
                                         out.data_ptr(),
                                         _stream_handle(q.device, stream))
        _check(st, "kivi_cache_attend_noalloc")
        return out

    def attend_work_bytes(self, n_q):
        return _lib().kivi_cache_attend_work_bytes(self._cref, n_q)


def kivi_cache_attend(cache, q, sm_scale, out=None, work=None, stream=None):
    """C-ABI name: decode attention over a KiviCache."""
    return cache.attend(q, sm_scale, out, work, stream)


def kivi_cache_attend_noalloc(cache, q, sm_scale, out, stream=None):
    """C-ABI name: decode attention over a KiviCache with the library's own
    workspace (allocates nothing)."""
    return cache.attend_noalloc(q, sm_scale, out, stream)


def kivi_cache_attend_work_bytes(cache, n_q):
    return cache.attend_work_bytes(n_q)


def kivi_cache_append(cache, k_new, v_new, stream=None):
    """C-ABI name: append to a KiviCache."""
    cache.append(k_new, v_new, stream)


def kivi_time_next_launch(start, stop):
    """Arm a pair of recorded torch.cuda.Event objects (or raw hipEvent_t
    handles) to time the next kernel this thread launches through the
    library; None disarms."""
    def h(e):
        if e is None:
            return None
        return ctypes.c_void_p(e.cuda_event if hasattr(e, "cuda_event")
                               else int(e))
    _lib().kivi_time_next_launch(h(start), h(stop))


def kivi_launch_count():
    """Kernel launches the library has made in this process (a launch
    recorded into a graph counts once)."""
    L = _lib()
    return int(L.kivi_launch_count())


def kivi_selftest_division(device="cuda", stream=None):
    """Number of mismatches of the kernels' exact division shortcuts
    against IEEE division on this GPU (0 is required)."""
    dev = torch.device(device)
    cnt = torch.zeros(1, dtype=torch.int64, device=dev)
    st = _lib().kivi_selftest_division(_ptr(cnt), _stream(dev, stream))
    _check(st, "kivi_selftest_division")
    return int(cnt.item())


def kivi_codes_bytes(BH, S, D, bits):
    return _lib().kivi_codes_bytes(BH, S, D, bits)


def kivi_key_param_count(BH, S, D, group):
    return _lib().kivi_key_param_count(BH, S, D, group)


def kivi_value_param_count(BH, S, D, group):
    return _lib().kivi_value_param_count(BH, S, D, group)


def kivi_status_string(status):
    return _lib().kivi_status_string(status).decode()


def library_path():
    return LIB_PATH


def raw():
    """The ctypes handle of libkivi.so (pointer-level calls)."""
    return _lib()
