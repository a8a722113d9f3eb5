"""Python handle on the fp64 CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc -O2 and OpenMP (host code only)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


class Config(ctypes.Structure):
    _fields_ = [
        ("n_layer", ctypes.c_int32), ("n_embd", ctypes.c_int32), ("n_head", ctypes.c_int32),
        ("n_kv_head", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("n_ff", ctypes.c_int32),
        ("n_vocab", ctypes.c_int32), ("n_expert", ctypes.c_int32),
        ("n_expert_used", ctypes.c_int32), ("sliding_window", ctypes.c_int32),
        ("rope_theta", ctypes.c_double), ("rms_norm_eps", ctypes.c_double),
        ("w_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
        ("rope_neox", ctypes.c_int32),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        vp, i32, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        P = ctypes.POINTER
        L.orc_layer_stride.argtypes = [P(Config)]
        L.orc_layer_stride.restype = i32
        L.orc_round_bf16.argtypes = [dbl]
        L.orc_round_bf16.restype = dbl
        L.orc_rmsnorm.argtypes = [vp, vp, i32, dbl, vp]
        L.orc_rmsnorm.restype = None
        L.orc_rope.argtypes = [vp, i32, i32, dbl]
        L.orc_rope.restype = None
        L.orc_rope_neox.argtypes = [vp, i32, i32, dbl]
        L.orc_rope_neox.restype = None
        L.orc_half_to_double.argtypes = [ctypes.c_uint16]
        L.orc_half_to_double.restype = dbl
        L.orc_q4_kv_round.argtypes = [vp, i32, vp]
        L.orc_q4_kv_round.restype = None
        L.orc_matvec.argtypes = [vp, i32, vp, i32, i32, vp, vp]
        L.orc_matvec.restype = None
        L.orc_attend.argtypes = [vp, vp, vp, i32, i32, vp]
        L.orc_attend.restype = None
        L.orc_attention.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
        L.orc_attention.restype = None
        L.orc_silu.argtypes = [dbl]
        L.orc_silu.restype = dbl
        L.orc_moe_route.argtypes = [vp, i32, i32, vp, vp]
        L.orc_moe_route.restype = dbl
        L.orc_argmax.argtypes = [vp, i32]
        L.orc_argmax.restype = i32
        L.orc_state_new.argtypes = [P(Config), i32]
        L.orc_state_new.restype = vp
        L.orc_state_free.argtypes = [vp]
        L.orc_state_free.restype = None
        L.orc_state_set_pos.argtypes = [vp, i32]
        L.orc_state_set_pos.restype = None
        L.orc_state_pos.argtypes = [vp]
        L.orc_state_pos.restype = i32
        L.orc_state_set_kv.argtypes = [vp, i32, i32, i32, vp, vp]
        L.orc_state_set_kv.restype = i32
        L.orc_step.argtypes = [P(Config), vp, vp, i32, vp, i32, vp, vp]
        L.orc_step.restype = i32
        L.orc_step_ex.argtypes = [P(Config), vp, vp, i32, vp, i32, vp, vp, vp, ctypes.c_uint64]
        L.orc_step_ex.restype = i32
        L.orc_embed.argtypes = [P(Config), vp, i32, vp]
        L.orc_embed.restype = i32
        L.orc_layer.argtypes = [P(Config), vp, vp, i32, i32, vp, vp, i32, i32, vp]
        L.orc_layer.restype = dbl
        L.orc_head.argtypes = [P(Config), vp, vp, vp, i32]
        L.orc_head.restype = i32
        L.orc_round_store.argtypes = [dbl, i32]
        L.orc_round_store.restype = dbl
        L.orc_set_perturbation.argtypes = [dbl, ctypes.c_uint64]
        L.orc_set_perturbation.restype = None
        L.orc_moe_route_swapped.argtypes = [vp, i32, i32, vp, vp]
        L.orc_moe_route_swapped.restype = dbl
        L.orc_full_recompute.argtypes = [P(Config), vp, vp, i32, vp, i32]
        L.orc_full_recompute.restype = i32
        L.orc_max_threads.argtypes = []
        L.orc_max_threads.restype = i32
        _lib = L
    return _lib


def _ptr(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags.c_contiguous
    return a.ctypes.data


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


# ----------------------------------------------------------------- building blocks

def rmsnorm(x, g, eps):
    x = _f64(x)
    g = np.ascontiguousarray(g, dtype=np.float32)
    y = np.empty_like(x)
    lib().orc_rmsnorm(_ptr(x), _ptr(g), x.size, eps, _ptr(y))
    return y


def rope(u, pos, theta):
    """RoPE of one head vector u [d] at position pos."""
    u = _f64(u).copy()
    lib().orc_rope(_ptr(u), u.size, pos, theta)
    return u


def half_to_double(bits):
    return lib().orc_half_to_double(int(bits))


def q4_kv_round(u):
    """A head vector as a Q4 KV cache stores it (blocks of 32 dims)."""
    u = _f64(u).copy()
    out = np.empty_like(u)
    lib().orc_q4_kv_round(_ptr(u), u.size, _ptr(out))
    return out


def matvec(W, dt, s, rows, cols, x):
    """y = W x through the oracle's mat-vec (W in storage type dt; s: int8 row scales)."""
    W = np.ascontiguousarray(W)
    x = _f64(x)
    y = np.empty(rows)
    sp = None if s is None else np.ascontiguousarray(s, dtype=np.float32)
    lib().orc_matvec(_ptr(W), dt, _ptr(sp), rows, cols, _ptr(x), _ptr(y))
    return y


def rope_neox(u, pos, theta):
    """Half-split (NeoX) RoPE of one head vector u [d] at position pos."""
    u = _f64(u).copy()
    lib().orc_rope_neox(_ptr(u), u.size, pos, theta)
    return u


def attend(q, K, V):
    q, K, V = _f64(q), _f64(K), _f64(V)
    o = np.empty(q.size)
    lib().orc_attend(_ptr(q), _ptr(K), _ptr(V), K.shape[0], q.size, _ptr(o))
    return o


def attention(q, K, V, pos, window=0):
    """q [H][d]; K, V [Hk][T][d]; keys max(0,pos-W+1)..pos. Returns o [H][d]."""
    q, K, V = _f64(q), _f64(K), _f64(V)
    H, d = q.shape
    Hk, T, _ = K.shape
    o = np.empty((H, d))
    lib().orc_attention(_ptr(q), _ptr(K), _ptr(V), H, Hk, d, T, pos, window, _ptr(o))
    return o


def silu(z):
    return lib().orc_silu(float(z))


def moe_route(r, k):
    r = _f64(r)
    ids = np.empty(k, dtype=np.int32)
    w = np.empty(k)
    gap = lib().orc_moe_route(_ptr(r), r.size, k, _ptr(ids), _ptr(w))
    return ids, w, gap


def argmax(logits):
    logits = _f64(logits)
    return lib().orc_argmax(_ptr(logits), logits.size)


def round_store(v, dt):
    """v as the oracle stores a value of type dt (fp32, or bf16 through fp32)."""
    return lib().orc_round_store(float(v), int(dt))


def set_perturbation(eps, seed=1):
    """Sensitivity probe: multiply every value about to be stored as bf16 by
    (1 + eps*u), u uniform in [-1, 1); eps = 0 turns it off."""
    lib().orc_set_perturbation(float(eps), int(seed))


def moe_route_swapped(r, k):
    """Top-k routing with the (k+1)-th expert in the k-th one's place."""
    r = _f64(r)
    ids = np.zeros(k, dtype=np.int32)
    w = np.zeros(k)
    gap = lib().orc_moe_route_swapped(_ptr(r), r.size, k, _ptr(ids), _ptr(w))
    return ids, w, gap


def round_bf16(v):
    return lib().orc_round_bf16(float(v))


# ----------------------------------------------------------------- model


def config_of(wl) -> Config:
    return Config(wl.n_layer, wl.n_embd, wl.n_head, wl.n_kv_head, wl.head_dim, wl.n_ff,
                  wl.n_vocab, wl.n_expert, wl.n_expert_used, wl.sliding_window,
                  float(wl.rope_theta), float(wl.rms_norm_eps), wl.w_dtype, wl.kv_dtype,
                  wl.act_dtype, int(wl.rope_neox))


class Model:
    """Oracle view of a weight set drawn by ``synth.make_weights``."""

    def __init__(self, wl, weights):
        self.wl = wl
        self.cfg = config_of(wl)
        self.w = weights
        stride = lib().orc_layer_stride(ctypes.byref(self.cfg))
        n = 4 + wl.n_layer * stride
        tab = (ctypes.c_void_p * n)()
        tab[0] = _ptr(weights["tok_embd"])
        tab[1] = _ptr(weights["out_norm"])
        tab[2] = _ptr(weights["w_out"])
        tab[3] = _ptr(weights["s_out"])
        for l, L in enumerate(weights["layers"]):
            if L is None:
                raise ValueError("oracle needs every layer's weights")
            b = 4 + l * stride
            tab[b + 0] = _ptr(L["attn_norm"])
            tab[b + 1] = _ptr(L["ffn_norm"])
            for i, name in enumerate(("wq", "wk", "wv", "wo")):
                tab[b + 2 + i] = _ptr(L[name])
                tab[b + 6 + i] = _ptr(L["s_" + name[1:]])
            tab[b + 10] = _ptr(L["w_router"])
            for i, name in enumerate(("b_q", "b_k", "b_v")):
                tab[b + 11 + i] = _ptr(L.get(name))
            for e in range(len(L["w_gate"])):
                eb = b + 16 + 6 * e
                tab[eb + 0] = _ptr(L["w_gate"][e])
                tab[eb + 1] = _ptr(L["w_up"][e])
                tab[eb + 2] = _ptr(L["w_down"][e])
                tab[eb + 3] = _ptr(L["s_gate"][e])
                tab[eb + 4] = _ptr(L["s_up"][e])
                tab[eb + 5] = _ptr(L["s_down"][e])
        self.tab = tab

    def new_state(self, max_ctx):
        return State(self, max_ctx)

    def embed(self, token):
        """The token's embedding row (fp64 [E])."""
        x = np.empty(self.wl.n_embd)
        if lib().orc_embed(ctypes.byref(self.cfg), self.tab, int(token), _ptr(x)) != 0:
            raise ValueError("token out of range")
        return x

    def head(self, x, threads=1):
        """Logits (fp64 [V]) and greedy id of a final residual x [E]."""
        x = _f64(x)
        logits = np.empty(self.wl.n_vocab)
        am = lib().orc_head(ctypes.byref(self.cfg), self.tab, _ptr(x), _ptr(logits), threads)
        return logits, am

    def full_recompute(self, tokens, threads=1):
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        logits = np.empty(self.wl.n_vocab)
        am = lib().orc_full_recompute(ctypes.byref(self.cfg), self.tab, _ptr(tokens), tokens.size,
                                      _ptr(logits), threads)
        return logits, am


class State:
    def __init__(self, model: Model, max_ctx: int):
        self.model = model
        self.h = lib().orc_state_new(ctypes.byref(model.cfg), max_ctx)
        if not self.h:
            raise MemoryError("oracle state allocation failed")

    def __del__(self):
        h = getattr(self, "h", None)
        if h and _lib is not None:
            _lib.orc_state_free(h)
            self.h = None

    @property
    def pos(self):
        return lib().orc_state_pos(self.h)

    @pos.setter
    def pos(self, p):
        lib().orc_state_set_pos(self.h, int(p))

    def set_kv(self, layer, pos0, k, v):
        k = np.ascontiguousarray(k)
        v = np.ascontiguousarray(v)
        rc = lib().orc_state_set_kv(self.h, layer, pos0, k.shape[0], _ptr(k), _ptr(v))
        if rc != 0:
            raise ValueError("set_kv out of range")

    def layer(self, l, pos, x, threads=1, swap=False, want_route=False):
        """Layer l applied to x [E] at position pos: the output residual (fp64 [E]),
        with the layer's k, v appended to this state's cache at pos (pos not
        moved); with want_route also the chosen experts and the router gap."""
        x = _f64(x)
        out = np.empty_like(x)
        ids = np.zeros(max(1, self.model.wl.n_expert_used), dtype=np.int32)
        gap = lib().orc_layer(ctypes.byref(self.model.cfg), self.model.tab, self.h, int(l), int(pos), _ptr(x),
                              _ptr(out), threads, int(bool(swap)), _ptr(ids))
        if gap < -1e300:
            raise ValueError("bad layer or position")
        return (out, ids, gap) if want_route else out

    def step(self, token, threads=1, want_route=False, swap_mask=0, want_gaps=False):
        """One decode step. Returns (logits float64 [V], argmax id[, route ids, route gap]
        [, per-layer router gaps]).  Bit l of swap_mask routes layer l to the
        (k+1)-th expert in place of the k-th."""
        wl = self.model.wl
        logits = np.empty(wl.n_vocab)
        ids = None
        gap = ctypes.c_double(0.0)
        gaps = np.zeros(wl.n_layer) if want_gaps else None
        if want_route:
            ids = np.zeros((wl.n_layer, max(1, wl.n_expert_used)), dtype=np.int32)
        am = lib().orc_step_ex(ctypes.byref(self.model.cfg), self.model.tab, self.h, int(token),
                               _ptr(logits), threads, _ptr(ids), _ptr(gaps), ctypes.byref(gap),
                               int(swap_mask))
        if am < -1:
            raise ValueError("oracle step failed (%d)" % am)
        out = (logits, am)
        if want_route:
            out = out + (ids, gap.value)
        if want_gaps:
            out = out + (gaps,)
        return out
