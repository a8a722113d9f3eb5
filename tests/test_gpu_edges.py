"""GPU edge cases of the attention window and of the model-building boundary.

- A window of one key (W = 1): the step attends to its own new key only, so
  the attention output is exactly that key's value ("Engine Architecture",
  section "Config Parsing": sliding_window bounds the keys a step attends to),
  and nothing of the cache or the position reaches the logits.  The GPU's
  logits at any position, over any cache, must then equal its logits at
  position 0 of a fresh state bit for bit, and the oracle's within tolerance.
  At position 0 the single key's softmax weight is exactly 1, so this also
  checks, on the GPU, that attending to one key returns its value unchanged.
- Windows whose first or last key sits on a 64-key page boundary, against the
  oracle (a window that is exactly one page, one that starts a key past a
  page start, one that ends on a page's last key).
- pn_model_create (one call, from a pn_weights struct of device pointers)
  builds the same model as pn_model_init + load_globals + load_layer: the
  logits are bitwise equal.
- Scores that jump by far more than the matrix-core attention's lazy-max
  threshold (2^8 in the softmax weights) from one page to the next, in one
  split and across splits, so the running maximum moves and the output is
  rescaled, against the oracle.
"""
import ctypes

import numpy as np
import pytest

import synth

from harness import Pair, compare_step, log

pytestmark = pytest.mark.gpu


def small(name, **kw):
    base = dict(n_layer=2, n_embd=200, n_head=6, n_kv_head=2, head_dim=32, n_ff=300, n_vocab=1000,
                rope_theta=10000.0, seed=151)
    base.update(kw)
    return synth.Workload(name, **base)


def _one_step(pair, ds, token):
    import torch
    from token_decode_amd import device as dv
    tok = torch.tensor([token], dtype=torch.int32, device="cuda")
    lg = torch.empty(pair.wl.n_vocab, dtype=torch.float32, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    dv.forward_step(pair.dm, ds, tok, lg, am)
    return lg.cpu().numpy(), int(am.item())


@pytest.mark.parametrize("wl", [
    small("w1-f32", w_dtype=synth.F32, kv_dtype=synth.F32, act_dtype=synth.F32, sliding_window=1),
    small("w1-bf16", w_dtype=synth.BF16, kv_dtype=synth.BF16, act_dtype=synth.BF16, sliding_window=1, seed=152),
    small("w1-bf16-d128-g4", n_head=8, n_kv_head=2, head_dim=128, w_dtype=synth.BF16, kv_dtype=synth.BF16,
          act_dtype=synth.F32, sliding_window=1, seed=153),
], ids=lambda w: w.name)
def test_window_of_one_key(wl):
    from token_decode_amd import device as dv
    p = Pair(wl)
    token = int(synth.uniform_int(wl.seed, 5, 1, 0, wl.n_vocab - 1)[0])
    ds0 = dv.DeviceState(p.dm, 8)
    ref, ref_id = _one_step(p, ds0, token)
    # the oracle at position 0
    ost = p.om.new_state(8)
    ol, oa = ost.step(token)
    compare_step(wl, ref, ol, ref_id, oa, "pos 0:")
    # a filled cache at positions inside a page, at a page's last key and at a
    # page's first key: each step attends to its own key only
    for pos in (700, 767, 768, 64 * 40 - 1):
        ds = dv.DeviceState(p.dm, pos + 2)
        os_ = p.om.new_state(pos + 2)
        for l in range(wl.n_layer):  # 300 cached keys below pos, none of them in the window
            k, v = wl.kv_prefill(1, l, pos - 300, 300)
            ds.set_kv(l, pos - 300, k, v)
            os_.set_kv(l, pos - 300, k, v)
        ds.pos = os_.pos = pos
        g, gid = _one_step(p, ds, token)
        assert g.tobytes() == ref.tobytes() and gid == ref_id, "pos %d differs from pos 0" % pos
        ol, oa = os_.step(token)
        compare_step(wl, g, ol, gid, oa, "pos %d:" % pos)
    log("  %s: logits at positions 700, 767, 768, 2559 equal position 0 bit for bit" % wl.name)


@pytest.mark.parametrize("window,pos", [
    (64, 127),   # window = keys 64..127: exactly one page
    (64, 128),   # keys 65..128: a page less its first key, then one key
    (128, 191),  # keys 64..191: two whole pages
    (65, 191),   # keys 127..191: the last key of a page, then a whole page
    (100, 255),  # ends on a page's last key
])
def test_window_on_page_boundaries(window, pos):
    wl = small("page-edge-w%d" % window, w_dtype=synth.BF16, kv_dtype=synth.BF16, act_dtype=synth.F32,
               sliding_window=window, seed=154)
    p = Pair(wl)
    ds, os_ = p.states(0, pos, pos + 4)
    token = int(synth.uniform_int(wl.seed, 6, 1, 0, wl.n_vocab - 1)[0])
    for i in range(3):  # pos, pos + 1, pos + 2
        g, gid = _one_step(p, ds, token)
        ol, oa = os_.step(token)
        rel, _ = compare_step(wl, g, ol, gid, oa, "window %d, pos %d:" % (window, pos + i))
        token = oa
    log("  window %d from pos %d: ok (last rel L2 %.2e)" % (window, pos, rel))


def test_model_create_equals_init_and_load():
    import torch
    from token_decode_amd import _capi as C
    from token_decode_amd import device as dv
    wl = small("create-bf16", w_dtype=synth.I8, kv_dtype=synth.BF16, act_dtype=synth.BF16, qkv_bias=True, seed=155)
    p = Pair(wl)
    W = p.W
    keep = []

    def up(a):
        if a is None:
            return None
        t = dv.upload(a)
        keep.append(t)
        return t.data_ptr()

    layers = (C.pn_layer_weights * wl.n_layer)()
    for l, Lw in enumerate(W["layers"]):
        for name in ("attn_norm", "ffn_norm", "wq", "wk", "wv", "wo", "s_q", "s_k", "s_v", "s_o", "b_q", "b_k", "b_v"):
            setattr(layers[l], name, up(Lw.get(name)))
        for name in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down"):
            setattr(layers[l], name, up(np.stack(Lw[name])))
    w = C.pn_weights(up(W["tok_embd"]), up(W["out_norm"]), up(W["w_out"]), up(W.get("s_out")), layers)
    L = C.lib()
    need = L.pn_model_bytes(ctypes.byref(p.cfg))
    buf = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    base = (buf.data_ptr() + 255) & ~255
    h = ctypes.c_void_p()
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    C.check(L.pn_model_create(ctypes.byref(p.cfg), ctypes.byref(w), ctypes.c_void_p(base), need, sp, ctypes.byref(h)))
    torch.cuda.synchronize()
    del keep[:]  # the sources may go once the packing has completed

    class Created:
        pass
    cm = Created()
    cm.h = h
    try:
        toks = [int(t) for t in synth.uniform_int(wl.seed, 7, 6, 0, wl.n_vocab - 1)]
        sa, sb = dv.DeviceState(p.dm, 16), dv.DeviceState(p.dm, 16)
        sb_h = ctypes.c_void_p()
        sbuf = torch.empty(L.pn_state_bytes(h, 16) + 256, dtype=torch.uint8, device="cuda")
        C.check(L.pn_state_new(h, 16, ctypes.c_void_p((sbuf.data_ptr() + 255) & ~255), L.pn_state_bytes(h, 16), sp,
                               ctypes.byref(sb_h)))
        tok = torch.zeros(1, dtype=torch.int32, device="cuda")
        la = torch.empty(wl.n_vocab, dtype=torch.float32, device="cuda")
        lb = torch.empty_like(la)
        aa = torch.empty(1, dtype=torch.int32, device="cuda")
        ab = torch.empty_like(aa)
        for t in toks:
            tok.fill_(t)
            dv.forward_step(p.dm, sa, tok, la, aa)
            C.check(L.pn_forward_step(h, sb_h, ctypes.c_void_p(tok.data_ptr()), ctypes.c_void_p(lb.data_ptr()),
                                      ctypes.c_void_p(ab.data_ptr()), sp))
            assert la.cpu().numpy().tobytes() == lb.cpu().numpy().tobytes()
            assert int(aa.item()) == int(ab.item())
        L.pn_state_free(sb_h)
    finally:
        L.pn_model_free(h)
    log("  pn_model_create: 6 steps bitwise equal to the init + load path")


def _pow2_scale_bf16(bits, factor):
    """bf16 bits times a power of two (exact)."""
    f = (bits.astype(np.uint32) << 16).view(np.float32) * np.float32(factor)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("kps,act", [(0, synth.F32), (4096, synth.F32), (4096, synth.BF16)])
def test_attention_running_max_moves(kps, act):
    """K rows of pages 3..5 scaled by 2^3 and of pages 6..10 by 2^6: each group's
    scores dwarf the earlier ones', so a wave walking the pages in one split
    (keys per split 4096) moves its running max twice and rescales its output;
    with automatic splits (one page each) the merge weighs them instead."""
    from token_decode_amd import _capi as C
    wl = small("max-jump-kps%d" % kps, n_head=8, n_kv_head=2, head_dim=128, w_dtype=synth.BF16,
               kv_dtype=synth.BF16, act_dtype=act, seed=156)
    p = Pair(wl)
    if kps:
        p.dm.set_option(C.PN_OPT_ATTN_KEYS_PER_SPLIT, kps)
    from token_decode_amd import device as dv
    pos = 11 * 64 - 5
    ds = dv.DeviceState(p.dm, pos + 4)
    os_ = p.om.new_state(pos + 4)
    for l in range(wl.n_layer):
        k, v = wl.kv_prefill(0, l, 0, pos)
        k = k.copy()
        k[3 * 64:6 * 64] = _pow2_scale_bf16(k[3 * 64:6 * 64], 8.0)
        k[6 * 64:] = _pow2_scale_bf16(k[6 * 64:], 64.0)
        ds.set_kv(l, 0, k, v)
        os_.set_kv(l, 0, k, v)
    ds.pos = os_.pos = pos
    token = int(synth.uniform_int(wl.seed, 8, 1, 0, wl.n_vocab - 1)[0])
    for i in range(3):
        g, gid = _one_step(p, ds, token)
        ol, oa = os_.step(token)
        rel, _ = compare_step(wl, g, ol, gid, oa, "kps %d, pos %d:" % (kps, pos + i))
        token = oa
    log("  running max moved between pages (keys per split %s): ok (last rel L2 %.2e)" % (kps or "auto", rel))
