"""Seeded synthetic KV-cache inputs for the KIVI flush.

Holds none of the quantizer's arithmetic: it only draws keys and values with
the shapes and value distributions of the workloads the VeloxQuant-MLX pages
measure (KIVI blog post on the fused Metal kernels: flushes of 32 decode
tokens and 2048-token prefill chunks over 28 layers x 8 KV heads x 128;
release post for KIVI 0.8.0: Llama-3.2-3B, Qwen2.5-7B, Mistral-7B KV
geometry; keys carry a few channels of consistently large magnitude, values
are flatter).  Both the GPU path and the oracle are fed from here.

Every tensor is drawn one (bh) slice at a time from numpy's PCG64 seeded with
(config seed, tensor id, bh, pool index), so any slice can be regenerated on
its own; fp16 casts use numpy (round to nearest even), bf16 casts use torch
on the CPU (round to nearest even).  Tensors are returned as uint16 bit
patterns [BH, S, D].
"""
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

FP16 = 0
BF16 = 1

_TENSOR_ID = {"K": 1, "V": 2}


@dataclass(frozen=True)
class Workload:
    name: str
    BH: int
    S: int
    D: int
    dtype: int        # FP16 or BF16
    bits: int
    group_k: int      # tokens per key group (per-channel quantization)
    group_v: int      # channels per value group (per-token quantization)
    seed: int
    key_kind: str     # recipe for K
    value_kind: str   # recipe for V
    desc: str
    heads: int = 1    # KV heads per sequence (rows b*heads .. of BH)
    n_planted: int = 0   # planted high-norm key tokens per sequence

    @property
    def elems(self):
        return self.BH * self.S * self.D


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny", 4, 64, 64, FP16, 2, 32, 32, 1, "tiny", "tiny",
                 "tiny 2-bit flush, K/V fp16 [4,64,64], one constant group "
                 "per tensor"),
        Workload("decode", 224, 32, 128, FP16, 2, 32, 32, 2, "outlier15",
                 "normal",
                 "decode-time flush, 28 layers x 8 KV heads, 32 residual "
                 "tokens, D=128, fp16, 2-bit"),
        Workload("prefill", 112, 32768, 128, FP16, 2, 32, 32, 3, "prefill",
                 "normal05",
                 "prefill quantize, 28 layers x 4 KV heads, S=32768, D=128, "
                 "fp16, 2-bit"),
        Workload("serve", 128, 8192, 128, BF16, 4, 32, 128, 4, "prefill",
                 "student_t4",
                 "batched serving flush, 16 x 8 KV heads, S=8192, D=128, "
                 "bf16, 4-bit, value group = whole head"),
        Workload("roundtrip", 256, 4096, 128, FP16, 2, 32, 32, 5, "outlier15",
                 "normal",
                 "quantize + dequantize round trip, 32 x 8 KV heads, S=4096, "
                 "D=128, fp16, 2-bit"),
    ]
}


@dataclass(frozen=True)
class CacheWorkload:
    """A residual-window cache workload: a step appends `appends` blocks of
    `n` tokens to a cache that starts the step holding T0 tokens (the
    counters are reset before every step)."""
    name: str
    BH: int
    D: int
    dtype: int
    bits: int
    group_k: int
    group_v: int
    R: int
    T0: int
    n: int
    appends: int
    seed: int
    key_kind: str
    value_kind: str
    desc: str

    def tokens(self):
        """The Workload that draws this step's new tokens ([BH, n*appends,
        D] of the same recipes)."""
        return Workload(self.name, self.BH, self.n * self.appends, self.D,
                        self.dtype, self.bits, self.group_k, self.group_v,
                        self.seed, self.key_kind, self.value_kind, self.desc)


CACHE_WORKLOADS = {
    w.name: w for w in [
        CacheWorkload("cache-prefill", 112, 128, FP16, 2, 32, 32, 32, 0, 2048,
                      1, 6, "prefill", "normal05",
                      "prefill chunk of 2048 tokens into an empty residual-"
                      "window cache (R = 32): flush 2016 tokens, keep 32; "
                      "28 layers x 4 KV heads, D=128, fp16, 2-bit"),
        CacheWorkload("cache-decode", 224, 128, FP16, 2, 32, 32, 32, 2059, 1,
                      32, 7, "outlier15", "normal",
                      "32 decode tokens appended one at a time after a "
                      "2059-token prompt (R = 32): one flush of 32 tokens; "
                      "28 layers x 8 KV heads, D=128, fp16, 2-bit"),
    ]
}


@dataclass(frozen=True)
class AttendWorkload:
    """Decode attention over a cache holding T tokens (R of them exact):
    n_q query heads per KV head, one decode position each."""
    name: str
    BH: int
    D: int
    dtype: int
    bits: int
    group_k: int
    group_v: int
    R: int
    T: int
    n_q: int
    seed: int
    key_kind: str
    value_kind: str
    desc: str

    def tokens(self):
        return Workload(self.name, self.BH, self.T, self.D, self.dtype,
                        self.bits, self.group_k, self.group_v, self.seed,
                        self.key_kind, self.value_kind, self.desc)


ATTEND_WORKLOADS = {
    w.name: w for w in [
        AttendWorkload("attend-decode", 224, 128, FP16, 2, 32, 32, 32, 2059,
                       3, 8, "outlier15", "normal",
                       "decode attention of 3 query heads per KV head over "
                       "a 2059-token KIVI cache (2016 tokens packed, 43 "
                       "exact), 28 layers x 8 KV heads, D=128, fp16, 2-bit"),
    ]
}


@dataclass(frozen=True)
class SinkWorkload:
    """KIVI-Sink over a prompt: B sequences of H KV heads ([B*H, S, D]),
    keys with n_planted tokens per sequence whose rows (in every head) are
    scaled up, so that they stand out by key norm the way attention sinks
    do; n_sink tokens per sequence are selected and kept."""
    name: str
    B: int
    H: int
    S: int
    D: int
    dtype: int
    bits: int
    group_k: int
    group_v: int
    n_sink: int
    seed: int
    key_kind: str
    value_kind: str
    desc: str

    def tokens(self):
        return Workload(self.name, self.B * self.H, self.S, self.D, self.dtype,
                        self.bits, self.group_k, self.group_v, self.seed,
                        self.key_kind, self.value_kind, self.desc,
                        heads=self.H, n_planted=self.n_sink)


SINK_WORKLOADS = {
    w.name: w for w in [
        SinkWorkload("sink-prefill", 14, 8, 32768, 128, FP16, 2, 32, 32, 5, 9,
                     "prefill", "normal05",
                     "KIVI-Sink over a 32768-token prompt: 14 layers x 8 KV "
                     "heads, D=128, fp16, 2-bit, 5 sinks per layer (token 0 "
                     "and 4 seeded positions carry 6x keys)"),
    ]
}

@dataclass(frozen=True)
class MixedWorkload:
    """Per-token mixed precision over a prompt: B sequences of H KV heads
    ([B*H, S, D]); the floor(hi_fraction * S) tokens of highest key norm
    per sequence at hi_bits, the rest at lo_bits."""
    name: str
    B: int
    H: int
    S: int
    D: int
    dtype: int
    hi_bits: int
    lo_bits: int
    group_k: int
    group_v: int
    hi_fraction: float
    seed: int
    key_kind: str
    value_kind: str
    desc: str

    @property
    def n_hi(self):
        return int(self.hi_fraction * self.S)

    def tokens(self):
        return Workload(self.name, self.B * self.H, self.S, self.D, self.dtype,
                        self.lo_bits, self.group_k, self.group_v, self.seed,
                        self.key_kind, self.value_kind, self.desc,
                        heads=self.H)


MIXED_WORKLOADS = {
    w.name: w for w in [
        MixedWorkload("mixed-prefill", 14, 8, 32768, 128, FP16, 4, 2, 32, 32,
                      0.2, 10, "prefill", "normal05",
                      "per-token mixed precision over a 32768-token prompt: "
                      "14 layers x 8 KV heads, D=128, fp16; the 20% of tokens "
                      "with the highest key norm at 4 bits, the rest at 2 "
                      "bits, groups of 32"),
    ]
}

PLANT_FACTOR = 6.0


def planted_positions(w, b):
    """The planted high-norm tokens of sequence b: token 0 and n_planted - 1
    further distinct positions drawn from (seed, b)."""
    r = np.random.default_rng([w.seed, 11, b])
    rest = r.choice(np.arange(1, w.S), size=w.n_planted - 1, replace=False)
    return np.sort(np.concatenate([[0], rest])).astype(np.int64)


def _rng(w, tensor, bh, pool):
    return np.random.default_rng([w.seed, _TENSOR_ID[tensor], bh, pool])


def _to_bits(f32, dtype):
    if dtype == FP16:
        return f32.astype(np.float16).view(np.uint16)
    import torch
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _tiny_key_channels(w, pool):
    r = np.random.default_rng([w.seed, 99, pool])
    return r.choice(w.D, size=4, replace=False)


def slice_f32(w, tensor, bh, pool=0):
    """fp32 draw of one [S, D] slice before the cast to the tensor dtype."""
    r = _rng(w, tensor, bh, pool)
    S, D = w.S, w.D
    kind = w.key_kind if tensor == "K" else w.value_kind
    if kind == "tiny":
        x = r.standard_normal((S, D), dtype=np.float32)
        if tensor == "K":
            x[:, _tiny_key_channels(w, pool)] *= np.float32(20.0)
            if bh == 1:   # one constant key group: channel 5, tokens 32..63
                x[32:64, 5] = np.float32(0.75)
        elif bh == 2:     # one constant value group: token 10, channels 32..63
            x[10, 32:64] = np.float32(-1.25)
        return x
    if kind == "normal":
        return r.standard_normal((S, D), dtype=np.float32)
    if kind == "normal05":
        return r.standard_normal((S, D), dtype=np.float32) * np.float32(0.5)
    if kind == "outlier15":
        x = r.standard_normal((S, D), dtype=np.float32)
        ch = r.choice(D, size=4, replace=False)
        x[:, ch] *= np.float32(15.0)
        return x
    if kind == "prefill":
        # ~3% of channels scaled by U(10, 30), every channel shifted by a
        # per-channel mean offset U(-2, 2).
        n_out = max(1, int(round(0.03 * D)))
        ch = r.choice(D, size=n_out, replace=False)
        f = np.ones(D, np.float32)
        f[ch] = r.uniform(10.0, 30.0, size=n_out).astype(np.float32)
        off = r.uniform(-2.0, 2.0, size=D).astype(np.float32)
        z = r.standard_normal((S, D), dtype=np.float32)
        return z * f[None, :] + off[None, :]
    if kind == "student_t4":
        return r.standard_t(4.0, size=(S, D)).astype(np.float32)
    raise ValueError(kind)


def gen_slice(w, tensor, bh, pool=0):
    """uint16 bit patterns of one [S, D] slice."""
    x = slice_f32(w, tensor, bh, pool)
    if tensor == "K" and w.n_planted > 0:
        x[planted_positions(w, bh // w.heads)] *= np.float32(PLANT_FACTOR)
    return _to_bits(x, w.dtype)


def gen_tensor(w, tensor, bhs=None, pool=0, threads=None):
    """uint16 [len(bhs), S, D]; bhs defaults to every slice.  Slices are
    independent draws, so they are generated on a thread pool."""
    if bhs is None:
        bhs = range(w.BH)
    bhs = list(bhs)
    out = np.empty((len(bhs), w.S, w.D), np.uint16)

    def one(i):
        out[i] = gen_slice(w, tensor, bhs[i], pool)

    n = threads or min(16, os.cpu_count() or 1)
    if n <= 1 or len(bhs) <= 2:
        for i in range(len(bhs)):
            one(i)
    else:
        with ThreadPoolExecutor(max_workers=n) as ex:
            list(ex.map(one, range(len(bhs))))
    return out


def sample_bhs(w, n, seed=0):
    """A deterministic spread of n slice indices: first, last and random."""
    if w.BH <= n:
        return list(range(w.BH))
    r = np.random.default_rng([w.seed, 7, seed])
    mid = r.choice(np.arange(1, w.BH - 1), size=n - 2, replace=False)
    return sorted({0, w.BH - 1, *mid.tolist()})
