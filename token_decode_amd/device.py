"""Device plumbing for the C ABI: torch owns the device buffers and streams.

Nothing here computes any part of the decode step; it uploads host arrays,
allocates the caller-owned buffers the library asks for and forwards pointers.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _capi as C


def _stream_ptr(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def upload(arr, device="cuda"):
    """Host numpy array -> device tensor holding the same bytes (bf16 bits as int16)."""
    if arr is None:
        return None
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def make_config(n_layer, n_embd, n_head, n_kv_head, head_dim, n_ff, n_vocab, *, n_ctx=2048,
                n_expert=0, n_expert_used=0, sliding_window=0, max_batch=1, rope_theta=10000.0,
                rms_norm_eps=1e-5, w_dtype=C.PN_BF16, kv_dtype=C.PN_BF16, act_dtype=C.PN_F32,
                rope_neox=False, qkv_bias=False, prefill_chunk=0):
    cfg = C.pn_config()
    C.lib().pn_config_default(ctypes.byref(cfg))
    for k, v in dict(n_layer=n_layer, n_embd=n_embd, n_head=n_head, n_kv_head=n_kv_head,
                     head_dim=head_dim, n_ff=n_ff, n_vocab=n_vocab, n_ctx=n_ctx, n_expert=n_expert,
                     n_expert_used=n_expert_used, sliding_window=sliding_window,
                     max_batch=max_batch, rope_theta=rope_theta, rms_norm_eps=rms_norm_eps,
                     w_dtype=w_dtype, kv_dtype=kv_dtype, act_dtype=act_dtype,
                     rope_neox=int(rope_neox), qkv_bias=int(qkv_bias),
                     prefill_chunk=prefill_chunk).items():
        setattr(cfg, k, v)
    return cfg


def _aligned(buf):
    p = buf.data_ptr()
    return (p + 255) & ~255


class DeviceModel:
    """A model in a torch-allocated device buffer, built layer by layer from host arrays.

    `weights` uses the key names of pn_layer_weights / pn_weights: tok_embd,
    out_norm, w_out, s_out and `layers`, a list of dicts with attn_norm,
    ffn_norm, wq, wk, wv, wo, w_gate, w_up, w_down (lists over experts),
    w_router, the int8 scales s_q, s_k, s_v, s_o, s_gate, s_up, s_down and
    the biases b_q, b_k, b_v.  A fused checkpoint may give `wqkv` ([q; k; v]
    rows) instead of wq, wk, wv and, for a dense FFN, `w_gate_up` ([gate; up]
    rows) instead of w_gate, w_up: the library is handed pointers into it.
    """

    def __init__(self, cfg, weights, stream=None, device="cuda"):
        self.cfg = cfg
        L = C.lib()
        nbytes = L.pn_model_bytes(ctypes.byref(cfg))
        if nbytes == 0:
            C.check(L.pn_config_check(ctypes.byref(cfg)))
        self.nbytes = nbytes
        self.buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        h = ctypes.c_void_p()
        C.check(L.pn_model_init(ctypes.byref(cfg), ctypes.c_void_p(_aligned(self.buf)), nbytes,
                                ctypes.byref(h)))
        self.h = h
        self._L = L
        s = stream if stream is not None else torch.cuda.current_stream()
        sp = _stream_ptr(s)
        g = [upload(weights["tok_embd"], device), upload(weights["out_norm"], device),
             upload(weights["w_out"], device), upload(weights.get("s_out"), device)]
        C.check(L.pn_model_load_globals(h, *[_ptr(t) for t in g], sp))
        s.synchronize()
        del g
        for l, W in enumerate(weights["layers"]):
            t = {k: upload(W[k], device) for k in ("attn_norm", "ffn_norm", "wq", "wk", "wv", "wo",
                                                   "s_q", "s_k", "s_v", "s_o", "w_router",
                                                   "b_q", "b_k", "b_v") if W.get(k) is not None}
            for k in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down"):
                v = W.get(k)
                t[k] = None if (v is None or v[0] is None) else upload(np.stack(v), device)
            ptrs = {k: _ptr(t.get(k)) for k, _ in C.pn_layer_weights._fields_}
            # fused checkpoints: pointers into one device copy of [q; k; v] / [gate; up]
            if W.get("wqkv") is not None:
                t["wqkv"] = upload(W["wqkv"], device)
                row = t["wqkv"].element_size() * cfg.n_embd
                base = t["wqkv"].data_ptr()
                hq, hk = cfg.n_head * cfg.head_dim, cfg.n_kv_head * cfg.head_dim
                ptrs["wq"], ptrs["wk"] = ctypes.c_void_p(base), ctypes.c_void_p(base + hq * row)
                ptrs["wv"] = ctypes.c_void_p(base + (hq + hk) * row)
            if W.get("w_gate_up") is not None:  # dense FFN: [2F][E]
                t["w_gate_up"] = upload(W["w_gate_up"], device)
                base = t["w_gate_up"].data_ptr()
                ptrs["w_gate"] = ctypes.c_void_p(base)
                ptrs["w_up"] = ctypes.c_void_p(base + cfg.n_ff * cfg.n_embd * t["w_gate_up"].element_size())
            lw = C.pn_layer_weights(**ptrs)
            C.check(L.pn_model_load_layer(h, l, ctypes.byref(lw), sp))
            s.synchronize()
            del t

    def __del__(self):
        # the library handle is held by the object: module globals may already
        # be gone when this runs at interpreter exit
        h, L = getattr(self, "h", None), getattr(self, "_L", None)
        if h is not None and h.value and L is not None:
            L.pn_model_free(h)
            self.h = None

    def set_option(self, option, value):
        C.check(C.lib().pn_model_set_option(self.h, option, value))

    def profile_begin(self, kernel):
        C.check(C.lib().pn_profile_begin(self.h, kernel))

    def profile_replay(self, kernel, reps, stream=None):
        """Enqueue reps copies of the last launch of a kernel class (for timing)."""
        C.check(C.lib().pn_profile_replay(self.h, kernel, reps, _stream_ptr(stream)))

    def profile_end(self, stream=None):
        ms = ctypes.c_double()
        n = ctypes.c_int64()
        C.check(C.lib().pn_profile_end(self.h, _stream_ptr(stream), ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value


class DevicePool:
    """A shared pool of K/V pages for pooled states, in a torch-allocated device buffer."""

    def __init__(self, model: DeviceModel, n_pages: int, device="cuda"):
        L = C.lib()
        self.model = model
        nbytes = L.pn_pool_bytes(model.h, n_pages)
        if nbytes == 0:
            raise C.PNError(C.PN_ERANGE, "invalid pool size %d pages" % n_pages)
        self.buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        h = ctypes.c_void_p()
        C.check(L.pn_pool_new(model.h, n_pages, ctypes.c_void_p(_aligned(self.buf)), nbytes, ctypes.byref(h)))
        self.h = h
        self._L = L

    @property
    def free_pages(self):
        return self._L.pn_pool_free_pages(self.h)

    def __del__(self):
        h, L = getattr(self, "h", None), getattr(self, "_L", None)
        if h is not None and h.value and L is not None:
            L.pn_pool_free(h)
            self.h = None


class DeviceState:
    """A decode state (paged KV cache + position) in a torch-allocated device
    buffer; with `pool`, its K/V pages come from that shared pool."""

    def __init__(self, model: DeviceModel, max_ctx: int, stream=None, device="cuda", pool: DevicePool = None):
        L = C.lib()
        self.model = model
        self.pool = pool  # the pool outlives its states
        nbytes = L.pn_state_bytes_pooled(model.h, max_ctx) if pool else L.pn_state_bytes(model.h, max_ctx)
        if nbytes == 0:
            raise C.PNError(C.PN_EINVAL, "invalid state capacity %d" % max_ctx)
        self.buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        h = ctypes.c_void_p()
        if pool:
            C.check(L.pn_state_new_pooled(model.h, pool.h, max_ctx, ctypes.c_void_p(_aligned(self.buf)), nbytes,
                                          _stream_ptr(stream), ctypes.byref(h)))
        else:
            C.check(L.pn_state_new(model.h, max_ctx, ctypes.c_void_p(_aligned(self.buf)), nbytes,
                                   _stream_ptr(stream), ctypes.byref(h)))
        self.h = h
        self._L = L

    def free(self):
        """Release the state now (a pooled state's pages go back to its pool)."""
        h, L = getattr(self, "h", None), getattr(self, "_L", None)
        if h is not None and h.value and L is not None:
            L.pn_state_free(h)
        self.h = None

    def __del__(self):
        self.free()

    @property
    def pos(self):
        return C.lib().pn_state_pos(self.h)

    @pos.setter
    def pos(self, p):
        self.set_pos(p)

    def set_pos(self, p, stream=None):
        C.check(C.lib().pn_state_set_pos(self.h, int(p), _stream_ptr(stream)))

    @property
    def n_pages(self):
        return C.lib().pn_state_pages(self.h)

    def set_kv(self, layer, pos0, k, v, stream=None):
        """Cached K/V of positions pos0.. from host or device arrays [n][n_kv_head][head_dim]."""
        kt = k if isinstance(k, torch.Tensor) else upload(k)
        vt = v if isinstance(v, torch.Tensor) else upload(v)
        C.check(C.lib().pn_state_set_kv(self.h, layer, pos0, kt.shape[0], _ptr(kt), _ptr(vt),
                                        _stream_ptr(stream)))
        (stream or torch.cuda.current_stream()).synchronize()

    def set_page_table(self, pages, stream=None):
        arr = (ctypes.c_int32 * len(pages))(*[int(p) for p in pages])
        C.check(C.lib().pn_state_set_page_table(self.h, arr, len(pages), _stream_ptr(stream)))

    def reset(self, stream=None):
        C.check(C.lib().pn_state_reset(self.h, _stream_ptr(stream)))

    def check_flags(self, stream=None):
        f = ctypes.c_int32()
        C.check(C.lib().pn_state_check(self.h, _stream_ptr(stream), ctypes.byref(f)))
        return f.value


def forward_step(model, state, token_dev, logits_dev=None, argmax_dev=None, stream=None):
    C.check(C.lib().pn_forward_step(model.h, state.h, _ptr(token_dev), _ptr(logits_dev),
                                    _ptr(argmax_dev), _stream_ptr(stream)))


def forward_batch(model, states, tokens_dev, logits_dev=None, argmax_dev=None, stream=None):
    arr = (ctypes.c_void_p * len(states))(*[s.h.value for s in states])
    C.check(C.lib().pn_forward_batch(model.h, arr, len(states), _ptr(tokens_dev), _ptr(logits_dev),
                                     _ptr(argmax_dev), _stream_ptr(stream)))


def prefill(model, state, tokens_dev, logits_dev=None, argmax_dev=None, stream=None):
    """Feed tokens_dev [n] to the state at consecutive positions (chunks of max_batch, or of
    prefill_chunk rows on the wide path)."""
    C.check(C.lib().pn_prefill(model.h, state.h, _ptr(tokens_dev), int(tokens_dev.numel()), _ptr(logits_dev),
                               _ptr(argmax_dev), _stream_ptr(stream)))


def sample(model, logits_dev, params, u_dev, ids_dev, recent_dev=None, stream=None):
    """Sample one token per row of logits_dev [n][n_vocab] into ids_dev [n].
    params: a list of n dicts (temperature, repeat_penalty, top_k, top_p);
    u_dev [n] fp32 uniform draws; recent_dev [n][n_recent] int32 or None."""
    n = len(params)
    arr = (C.pn_sampling_params * n)()
    for i, p in enumerate(params):
        arr[i].temperature = p.get("temperature", 1.0)
        arr[i].repeat_penalty = p.get("repeat_penalty", 1.0)
        arr[i].top_k = p.get("top_k", 40)
        arr[i].top_p = p.get("top_p", 1.0)
    n_recent = 0 if recent_dev is None else int(recent_dev.shape[-1])
    C.check(C.lib().pn_sample(model.h, _ptr(logits_dev), n, arr, _ptr(recent_dev), n_recent, _ptr(u_dev),
                              _ptr(ids_dev), _stream_ptr(stream)))
