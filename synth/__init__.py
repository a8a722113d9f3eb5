"""Seeded synthetic inputs for the decode step (weights, cached K/V, tokens, positions).

This module draws numbers only; it holds none of the decode arithmetic.  The
oracle and the HIP path both read the arrays it returns, so they see the same
stored values.  The stream definition (SplitMix64 counters + Box-Muller) is in
``synth.c``.

Tensor ids follow one fixed enumeration so that any tensor can be redrawn on
its own:

* 0: token embedding table
* 1 + 64*l + j for layer l: j = 0 attn_norm, 1 wq, 2 wk, 3 wv, 4 wo,
  5 ffn_norm, 6 router, 8 + 3*e + {0 gate, 1 up, 2 down} for expert e
* 1 + 64*L: output norm, 2 + 64*L: output (LM head) matrix
* 2**20 + {0 tokens, 1 positions}
* 2**21 + 2*(slot*L + l) + {0 K, 1 V}: cached K/V of one slot and layer,
  laid out [pos][kv_head][head_dim]
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_SRC = os.path.join(_HERE, "synth.c")

F32, BF16, I8, Q8_0, Q4_0 = 0, 1, 2, 3, 4
Q8_BLOCK, Q8_BLOCK_BYTES, Q4_BLOCK_BYTES = 32, 34, 18
DTYPE_NAMES = {F32: "f32", BF16: "bf16", I8: "i8"}

TID_EMBD = 0
TID_TOKENS = 1 << 20
TID_POSITIONS = (1 << 20) + 1
TID_KV = 1 << 21

J_ATTN_NORM, J_WQ, J_WK, J_WV, J_WO, J_FFN_NORM, J_ROUTER = 0, 1, 2, 3, 4, 5, 6
J_BQ, J_BK, J_BV = 40, 41, 42
W_STD = 0.02
GAIN_STD = 0.1
BIAS_STD = 0.5


def build(force: bool = False) -> str:
    """Compile libsynth.so with gcc (host code only)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.synth_normal.argtypes = [u64, u64, u64, u64, dbl, dbl, ctypes.c_int, vp, ctypes.c_int]
        L.synth_normal.restype = None
        L.synth_int8_rows.argtypes = [u64, u64, u64, u64, dbl, vp, vp, ctypes.c_int]
        L.synth_int8_rows.restype = None
        L.synth_q8_0_rows.argtypes = [u64, u64, u64, u64, dbl, vp, ctypes.c_int]
        L.synth_q8_0_rows.restype = None
        L.synth_q4_0_rows.argtypes = [u64, u64, u64, u64, dbl, vp, ctypes.c_int]
        L.synth_q4_0_rows.restype = None
        L.synth_uniform_int.argtypes = [u64, u64, u64, i64, i64, vp]
        L.synth_uniform_int.restype = None
        L.synth_distinct_int.argtypes = [u64, u64, u64, i64, i64, vp]
        L.synth_distinct_int.restype = ctypes.c_int
        L.synth_draw_u64.argtypes = [u64, u64]
        L.synth_draw_u64.restype = u64
        _lib = L
    return _lib


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal(seed, tid, n, mean=0.0, std=1.0, dtype=F32, start=0, threads=None, out=None):
    """Elements start..start+n-1 of normal stream `tid`, stored as fp32 or bf16 bits (uint16)."""
    npdt = np.float32 if dtype == F32 else np.uint16
    if out is None:
        out = np.empty(n, dtype=npdt)
    assert out.dtype == npdt and out.size == n and out.flags.c_contiguous
    lib().synth_normal(seed, tid, start, n, mean, std, dtype, out.ctypes.data,
                       threads or default_threads())
    return out


def int8_rows(seed, tid, rows, cols, std=W_STD, threads=None):
    """INT8 symmetric per-row quantisation of a bf16 N(0, std) draw: (q [rows, cols], scale [rows])."""
    q = np.empty((rows, cols), dtype=np.int8)
    s = np.empty(rows, dtype=np.float32)
    lib().synth_int8_rows(seed, tid, rows, cols, std, q.ctypes.data, s.ctypes.data,
                          threads or default_threads())
    return q, s


def q8_0_rows(seed, tid, rows, cols, std=W_STD, threads=None):
    """Q8_0 rows quantised from an fp32 N(0, std) draw: uint8 [rows][cols / 32 * 34]."""
    assert cols % Q8_BLOCK == 0
    out = np.empty((rows, cols // Q8_BLOCK * Q8_BLOCK_BYTES), dtype=np.uint8)
    lib().synth_q8_0_rows(seed, tid, rows, cols, std, out.ctypes.data, threads or default_threads())
    return out


def q4_0_rows(seed, tid, rows, cols, std=W_STD, threads=None):
    """Q4_0 rows quantised from an fp32 N(0, std) draw: uint8 [rows][cols / 32 * 18]."""
    assert cols % Q8_BLOCK == 0
    out = np.empty((rows, cols // Q8_BLOCK * Q4_BLOCK_BYTES), dtype=np.uint8)
    lib().synth_q4_0_rows(seed, tid, rows, cols, std, out.ctypes.data, threads or default_threads())
    return out


def uniform_int(seed, tid, n, lo, hi):
    out = np.empty(n, dtype=np.int32)
    lib().synth_uniform_int(seed, tid, n, lo, hi, out.ctypes.data)
    return out


def distinct_int(seed, tid, n, lo, hi):
    out = np.empty(n, dtype=np.int32)
    rc = lib().synth_distinct_int(seed, tid, n, lo, hi, out.ctypes.data)
    if rc != 0:
        raise ValueError("range too small for %d distinct values" % n)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 values (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------- workloads


@dataclass
class Workload:
    """A model shape, its storage dtypes and the decode workload run on it."""

    name: str
    n_layer: int
    n_embd: int
    n_head: int
    n_kv_head: int
    head_dim: int
    n_ff: int
    n_vocab: int
    rope_theta: float = 10000.0
    rms_norm_eps: float = 1e-5
    sliding_window: int = 0
    n_expert: int = 0
    n_expert_used: int = 0
    w_dtype: int = F32
    kv_dtype: int = F32
    act_dtype: int = F32
    rope_neox: bool = False      # half-split RoPE pairs (i, i + d/2)
    qkv_bias: bool = False       # q, k, v projections carry fp32 biases
    seed: int = 1
    slots: int = 1
    steps: int = 8
    prompt_len: int = 0          # tokens fed one at a time from position 0 before decoding
    prefill: int = 0             # batch-1: K/V positions 0..prefill-1 filled with N(0,1)
    pos_range: tuple = ()        # batched: slot positions drawn from [lo, hi]
    distinct_pos: bool = False
    extra: dict = field(default_factory=dict)

    @property
    def embd_dtype(self) -> int:
        return F32 if self.w_dtype == F32 else BF16

    @property
    def router_dtype(self) -> int:
        return F32 if self.w_dtype == F32 else BF16

    @property
    def n_experts_stored(self) -> int:
        return max(1, self.n_expert)

    def tid_layer(self, l: int, j: int) -> int:
        return 1 + 64 * l + j

    def tid_expert(self, l: int, e: int, which: int) -> int:
        return 1 + 64 * l + 8 + 3 * e + which

    @property
    def tid_out_norm(self) -> int:
        return 1 + 64 * self.n_layer

    @property
    def tid_out(self) -> int:
        return 2 + 64 * self.n_layer

    def tid_kv(self, slot: int, l: int, which: int) -> int:
        return TID_KV + 2 * (slot * self.n_layer + l) + which

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    # positions at which each slot starts decoding
    def start_positions(self) -> np.ndarray:
        if self.slots == 1 and not self.pos_range:
            return np.array([self.prefill], dtype=np.int32)
        lo, hi = self.pos_range
        if self.distinct_pos:
            return distinct_int(self.seed, TID_POSITIONS, self.slots, lo, hi)
        return uniform_int(self.seed, TID_POSITIONS, self.slots, lo, hi)

    def first_tokens(self, n=None) -> np.ndarray:
        n = self.slots if n is None else n
        return uniform_int(self.seed, TID_TOKENS, n, 0, self.n_vocab - 1)

    def prompt_tokens(self) -> np.ndarray:
        return uniform_int(self.seed, TID_TOKENS, self.prompt_len, 0, self.n_vocab - 1)

    def kv_window_start(self, pos: int) -> int:
        """First cached position that the step at `pos` can attend to."""
        if self.sliding_window > 0:
            return max(0, pos - self.sliding_window + 1)
        return 0

    def kv_prefill(self, slot: int, l: int, p0: int, n: int, threads=None):
        """Cached K and V of positions p0..p0+n-1: arrays [n][n_kv_head][head_dim] in kv dtype
        (fp32 for a Q4 cache, whose set_kv quantises as an append does)."""
        per = self.n_kv_head * self.head_dim
        dt = F32 if self.kv_dtype == Q4_0 else self.kv_dtype
        k = normal(self.seed, self.tid_kv(slot, l, 0), n * per, 0.0, 1.0, dt, start=p0 * per, threads=threads)
        v = normal(self.seed, self.tid_kv(slot, l, 1), n * per, 0.0, 1.0, dt, start=p0 * per, threads=threads)
        shp = (n, self.n_kv_head, self.head_dim)
        return k.reshape(shp), v.reshape(shp)


def q8_0_blocks(w: np.ndarray) -> np.ndarray:
    """Quantise fp32 rows [rows][cols] (cols a multiple of 32) into Q8_0 blocks as
    a checkpoint would store them: per block of 32, d = max|w| / 127 as fp16,
    codes round(w / d); 34 bytes per block (d little-endian, then the codes)."""
    rows, cols = w.shape
    b = w.reshape(rows, cols // Q8_BLOCK, Q8_BLOCK).astype(np.float64)
    d = (np.abs(b).max(axis=2) / 127.0).astype(np.float16)
    df = d.astype(np.float64)[..., None]
    q = np.where(df > 0, np.rint(b / np.where(df > 0, df, 1.0)), 0.0)
    q = np.clip(q, -127, 127).astype(np.int8)
    out = np.empty((rows, cols // Q8_BLOCK, Q8_BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = d.view(np.uint8).reshape(rows, cols // Q8_BLOCK, 2)
    out[:, :, 2:] = q.view(np.uint8)
    return out.reshape(rows, cols // Q8_BLOCK * Q8_BLOCK_BYTES)


def _matrix(wl: Workload, tid: int, rows: int, cols: int, threads=None):
    if wl.w_dtype == I8:
        q, s = int8_rows(wl.seed, tid, rows, cols, W_STD, threads)
        return q, s
    if wl.w_dtype == Q8_0:
        return q8_0_rows(wl.seed, tid, rows, cols, W_STD, threads), None
    if wl.w_dtype == Q4_0:
        return q4_0_rows(wl.seed, tid, rows, cols, W_STD, threads), None
    m = normal(wl.seed, tid, rows * cols, 0.0, W_STD, wl.w_dtype, threads=threads)
    return m.reshape(rows, cols), None


def _gain(wl: Workload, tid: int, n: int, threads=None):
    return normal(wl.seed, tid, n, 1.0, GAIN_STD, F32, threads=threads)


def make_layer(wl: Workload, l: int, threads=None) -> dict:
    """Weights of one layer as host arrays (matrices row-major [out][in])."""
    E, H, Hk, d, F = wl.n_embd, wl.n_head, wl.n_kv_head, wl.head_dim, wl.n_ff
    out = {
        "attn_norm": _gain(wl, wl.tid_layer(l, J_ATTN_NORM), E, threads),
        "ffn_norm": _gain(wl, wl.tid_layer(l, J_FFN_NORM), E, threads),
    }
    for name, j, rows, cols in (("wq", J_WQ, H * d, E), ("wk", J_WK, Hk * d, E),
                                ("wv", J_WV, Hk * d, E), ("wo", J_WO, E, H * d)):
        m, s = _matrix(wl, wl.tid_layer(l, j), rows, cols, threads)
        out[name] = m
        out["s_" + name[1:]] = s
    for name, j, rows in (("b_q", J_BQ, H * d), ("b_k", J_BK, Hk * d), ("b_v", J_BV, Hk * d)):
        out[name] = (normal(wl.seed, wl.tid_layer(l, j), rows, 0.0, BIAS_STD, F32, threads=threads)
                     if wl.qkv_bias else None)
    gates, ups, downs, sg, su, sd = [], [], [], [], [], []
    for e in range(wl.n_experts_stored):
        m, s = _matrix(wl, wl.tid_expert(l, e, 0), F, E, threads)
        gates.append(m)
        sg.append(s)
        m, s = _matrix(wl, wl.tid_expert(l, e, 1), F, E, threads)
        ups.append(m)
        su.append(s)
        m, s = _matrix(wl, wl.tid_expert(l, e, 2), E, F, threads)
        downs.append(m)
        sd.append(s)
    out["w_gate"], out["w_up"], out["w_down"] = gates, ups, downs
    out["s_gate"], out["s_up"], out["s_down"] = sg, su, sd
    if wl.n_expert > 0:
        r = normal(wl.seed, wl.tid_layer(l, J_ROUTER), wl.n_expert * E, 0.0, W_STD,
                   wl.router_dtype, threads=threads)
        out["w_router"] = r.reshape(wl.n_expert, E)
    else:
        out["w_router"] = None
    return out


def make_weights(wl: Workload, threads=None, layers=None) -> dict:
    """All weights of a workload as host arrays.

    `layers` may be an iterable of layer indices to draw (others are None),
    which lets a caller stream layers without holding the whole model.
    """
    E, V = wl.n_embd, wl.n_vocab
    w = {}
    w["tok_embd"] = normal(wl.seed, TID_EMBD, V * E, 0.0, W_STD, wl.embd_dtype,
                           threads=threads).reshape(V, E)
    w["out_norm"] = _gain(wl, wl.tid_out_norm, E, threads)
    m, s = _matrix(wl, wl.tid_out, V, E, threads)
    w["w_out"], w["s_out"] = m, s
    want = range(wl.n_layer) if layers is None else set(layers)
    w["layers"] = [make_layer(wl, l, threads) if l in want else None for l in range(wl.n_layer)]
    return w


# --------------------------------------------------------------------------- named workloads

def tiny_fp32() -> Workload:
    """Tiny Llama-style model, fp32 end to end; 4-token prompt then 128 greedy steps."""
    return Workload("tiny-fp32", n_layer=2, n_embd=256, n_head=8, n_kv_head=2, head_dim=32,
                    n_ff=688, n_vocab=1024, rope_theta=10000.0, w_dtype=F32, kv_dtype=F32,
                    act_dtype=F32, seed=1, prompt_len=4, steps=128)


def llama3_8b_bf16() -> Workload:
    """Llama-3-8B shape, bf16 weights and KV, fp32 activations; KV prefilled to 2048."""
    return Workload("llama3-8b-bf16", n_layer=32, n_embd=4096, n_head=32, n_kv_head=8,
                    head_dim=128, n_ff=14336, n_vocab=128256, rope_theta=500000.0,
                    w_dtype=BF16, kv_dtype=BF16, act_dtype=F32, seed=2, prefill=2048, steps=256)


def llama3_8b_int8() -> Workload:
    """Llama-3-8B shape, INT8 per-row weights, bf16 activations and KV; KV context 8192."""
    return llama3_8b_bf16().with_(name="llama3-8b-int8", w_dtype=I8, act_dtype=BF16, seed=3,
                                  prefill=8192, steps=256)


def mistral_7b_slots() -> Workload:
    """Mistral-7B shape, bf16, window 4096; 8 slots at distinct positions in [1024, 16384]."""
    return Workload("mistral-7b-8slots", n_layer=32, n_embd=4096, n_head=32, n_kv_head=8,
                    head_dim=128, n_ff=14336, n_vocab=32000, rope_theta=10000.0,
                    sliding_window=4096, w_dtype=BF16, kv_dtype=BF16, act_dtype=BF16, seed=4,
                    slots=8, pos_range=(1024, 16384), distinct_pos=True, steps=128)


def mixtral_8x7b_slots() -> Workload:
    """Mixtral-8x7B shape, bf16, top-2 of 8 experts; 16 slots at positions in [512, 4096]."""
    return Workload("mixtral-8x7b-16slots", n_layer=32, n_embd=4096, n_head=32, n_kv_head=8,
                    head_dim=128, n_ff=14336, n_vocab=32000, rope_theta=10000.0, n_expert=8,
                    n_expert_used=2, w_dtype=BF16, kv_dtype=BF16, act_dtype=BF16, seed=5,
                    slots=16, pos_range=(512, 4096), steps=64)


def llama3_8b_q8_0() -> Workload:
    """Llama-3-8B shape, Q8_0 block-quantised weights, bf16 activations and KV; KV from 2048."""
    return llama3_8b_bf16().with_(name="llama3-8b-q8_0", w_dtype=Q8_0, act_dtype=BF16, seed=6)


def llama3_8b_q4_0() -> Workload:
    """Llama-3-8B shape, Q4_0 block-quantised weights, bf16 activations and KV; KV from 2048."""
    return llama3_8b_bf16().with_(name="llama3-8b-q4_0", w_dtype=Q4_0, act_dtype=BF16, seed=7)


def llama3_8b_kv_long(kv_dtype: int) -> Workload:
    """Llama-3-8B shape, Q4_0 weights, batch 1 from position 32768, with a bf16 or Q4 KV cache."""
    return llama3_8b_q4_0().with_(name="llama3-8b-q4_0-kv%s-32k" % ("q4" if kv_dtype == Q4_0 else "bf16"),
                                  kv_dtype=kv_dtype, prefill=32768)


WORKLOADS = {
    "tiny-fp32": tiny_fp32,
    "llama3-8b-bf16": llama3_8b_bf16,
    "llama3-8b-int8": llama3_8b_int8,
    "mistral-7b-8slots": mistral_7b_slots,
    "mixtral-8x7b-16slots": mixtral_8x7b_slots,
    "llama3-8b-q8_0": llama3_8b_q8_0,
    "llama3-8b-q4_0": llama3_8b_q4_0,
    "llama3-8b-q4_0-kvbf16-32k": lambda: llama3_8b_kv_long(BF16),
    "llama3-8b-q4_0-kvq4-32k": lambda: llama3_8b_kv_long(Q4_0),
}
