"""The C ABI on the host: every declared symbol is exported, the config defaults
are the pages', and invalid arguments are rejected before any device work."""
import ctypes
import json
import os
import re

import pytest

import token_decode_amd as td
from token_decode_amd import _capi as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "pn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pn_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    lib = C.lib()
    names = declared_functions()
    assert len(names) >= 25
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(C.EXPORTS)


def test_config_defaults_match_pages():
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "config_defaults.json")))
    cfg = C.pn_config()
    C.lib().pn_config_default(ctypes.byref(cfg))
    d = gold["defaults"]
    assert cfg.n_ctx == d["n_ctx"]
    assert cfg.rope_theta == pytest.approx(d["rope_theta"])
    assert cfg.rms_norm_eps == pytest.approx(d["rms_norm_eps"], rel=1e-6)
    assert cfg.sliding_window == d["sliding_window"]


def good_cfg(**kw):
    from token_decode_amd import device as dv
    base = dict(n_layer=2, n_embd=256, n_head=8, n_kv_head=2, head_dim=32, n_ff=688, n_vocab=1024,
                w_dtype=C.PN_F32, kv_dtype=C.PN_F32, act_dtype=C.PN_F32)
    base.update(kw)
    return dv.make_config(**base)


def test_flag_fields_are_zero_or_one():
    cfg = good_cfg()
    cfg.rope_neox = 2
    assert C.lib().pn_config_check(ctypes.byref(cfg)) == C.PN_EINVAL
    cfg.rope_neox, cfg.qkv_bias = 0, -1
    assert C.lib().pn_config_check(ctypes.byref(cfg)) == C.PN_EINVAL


@pytest.mark.parametrize("kw,code", [
    (dict(n_head=6, n_kv_head=4), C.PN_EINVAL),
    (dict(head_dim=48), C.PN_EUNSUPPORTED),
    (dict(n_head=16, n_kv_head=1), C.PN_EUNSUPPORTED),
    (dict(n_layer=0), C.PN_EINVAL),
    (dict(w_dtype=C.PN_I8, act_dtype=C.PN_F32), C.PN_EUNSUPPORTED),
    (dict(kv_dtype=C.PN_I8), C.PN_EINVAL),
    (dict(max_batch=17), C.PN_EINVAL),
    (dict(w_dtype=C.PN_BF16, act_dtype=C.PN_F32, max_batch=6), C.PN_EUNSUPPORTED),
    (dict(n_expert=4, n_expert_used=5), C.PN_EINVAL),
    (dict(sliding_window=-1), C.PN_EINVAL),
    (dict(rope_theta=0.0), C.PN_EINVAL),
    (dict(n_embd=252), C.PN_EUNSUPPORTED),
    (dict(w_dtype=C.PN_Q8_0, act_dtype=C.PN_F32), C.PN_EUNSUPPORTED),
    (dict(w_dtype=C.PN_Q4_0, act_dtype=C.PN_BF16, n_ff=680), C.PN_EINVAL),  # rows of whole 32-blocks
    (dict(w_dtype=C.PN_Q4_0, act_dtype=C.PN_BF16, n_embd=264), C.PN_EINVAL),
    (dict(w_dtype=5), C.PN_EINVAL),
    (dict(kv_dtype=C.PN_Q8_0), C.PN_EINVAL),
    (dict(kv_dtype=C.PN_Q4_0, rope_neox=True), C.PN_EUNSUPPORTED),
    (dict(prefill_chunk=-1), C.PN_EINVAL),
    (dict(prefill_chunk=257), C.PN_EINVAL),
    (dict(prefill_chunk=64, n_expert=8, n_expert_used=2), C.PN_EUNSUPPORTED),  # fp32 weights
    (dict(prefill_chunk=64, kv_dtype=C.PN_Q4_0), C.PN_EUNSUPPORTED),
])
def test_bad_configs_rejected(kw, code):
    cfg = good_cfg(**kw)
    assert C.lib().pn_config_check(ctypes.byref(cfg)) == code
    assert C.lib().pn_last_error()
    assert C.lib().pn_model_bytes(ctypes.byref(cfg)) == 0


def test_good_configs_and_sizes():
    L = C.lib()
    for kw in (dict(), dict(w_dtype=C.PN_BF16, kv_dtype=C.PN_BF16, act_dtype=C.PN_F32, max_batch=5),
               dict(w_dtype=C.PN_I8, kv_dtype=C.PN_BF16, act_dtype=C.PN_BF16, max_batch=16),
               dict(n_expert=8, n_expert_used=2, w_dtype=C.PN_BF16, act_dtype=C.PN_BF16),
               dict(n_kv_head=0),
               dict(w_dtype=C.PN_Q8_0, act_dtype=C.PN_BF16, n_ff=672),
               dict(w_dtype=C.PN_Q4_0, act_dtype=C.PN_BF16, n_ff=672, kv_dtype=C.PN_Q4_0),
               dict(rope_neox=True, qkv_bias=True),
               dict(prefill_chunk=256, w_dtype=C.PN_BF16, act_dtype=C.PN_F32, kv_dtype=C.PN_F32),
               dict(prefill_chunk=64, w_dtype=C.PN_I8, act_dtype=C.PN_BF16, kv_dtype=C.PN_BF16),
               dict(prefill_chunk=64, w_dtype=C.PN_Q8_0, act_dtype=C.PN_BF16, n_ff=672),
               dict(prefill_chunk=64, w_dtype=C.PN_Q4_0, act_dtype=C.PN_BF16, n_ff=672),
               dict(prefill_chunk=128, n_expert=8, n_expert_used=2, w_dtype=C.PN_BF16, act_dtype=C.PN_BF16,
                    kv_dtype=C.PN_BF16)):
        cfg = good_cfg(**kw)
        assert L.pn_config_check(ctypes.byref(cfg)) == 0, L.pn_last_error()
        assert L.pn_model_bytes(ctypes.byref(cfg)) > 0


def test_block_formats_and_q4_cache_sizes():
    """Llama-3-8B shape: Q8_0 / Q4_0 packed weights take 34 / 18 bytes per 32 weights (codes
    plus fp16 scales); a Q4 KV cache takes 9/16 byte per element, 9/32 of a bf16 one."""
    L = C.lib()
    shape = dict(n_layer=32, n_embd=4096, n_head=32, n_kv_head=8, head_dim=128, n_ff=14336, n_vocab=128256,
                 act_dtype=C.PN_BF16)
    params = 32 * (4096 * 6144 + 4096 * 4096 + 3 * 4096 * 14336) + 128256 * 4096
    embd = 128256 * 4096 * 2
    for wt, per32 in ((C.PN_Q8_0, 34), (C.PN_Q4_0, 18)):
        n = L.pn_model_bytes(ctypes.byref(good_cfg(w_dtype=wt, kv_dtype=C.PN_BF16, **shape)))
        assert params * per32 / 32 + embd <= n < (params * per32 / 32 + embd) * 1.01
    sizes = {}
    for kvt in (C.PN_BF16, C.PN_Q4_0):
        cfg = good_cfg(w_dtype=C.PN_Q4_0, kv_dtype=kvt, **shape)
        need = L.pn_model_bytes(ctypes.byref(cfg))
        h = ctypes.c_void_p()
        assert L.pn_model_init(ctypes.byref(cfg), ctypes.c_void_p(1 << 20), need, ctypes.byref(h)) == 0
        try:
            sizes[kvt] = (L.pn_state_bytes(h, 32768), L.pn_pool_bytes(h, 1))
        finally:
            L.pn_model_free(h)
    kv_bf16 = 2 * 32 * 32768 * 8 * 128 * 2
    assert sizes[C.PN_BF16][1] * 9 == sizes[C.PN_Q4_0][1] * 32  # a page: 9/32 of the bf16 bytes
    assert sizes[C.PN_BF16][0] - sizes[C.PN_Q4_0][0] == kv_bf16 * 23 // 32


def test_model_bytes_cover_packed_weights():
    """Llama-3-8B shape in bf16: the packed weights alone are 16.06e9 bytes."""
    cfg = good_cfg(n_layer=32, n_embd=4096, n_head=32, n_kv_head=8, head_dim=128, n_ff=14336,
                   n_vocab=128256, w_dtype=C.PN_BF16, kv_dtype=C.PN_BF16)
    n = C.lib().pn_model_bytes(ctypes.byref(cfg))
    params = 32 * (4096 * 6144 + 4096 * 4096 + 3 * 4096 * 14336) + 2 * 128256 * 4096
    assert 2 * params <= n < 2 * params * 1.01


def test_init_rejects_bad_buffers_without_device_work():
    L = C.lib()
    cfg = good_cfg()
    need = L.pn_model_bytes(ctypes.byref(cfg))
    h = ctypes.c_void_p()
    assert L.pn_model_init(ctypes.byref(cfg), None, need, ctypes.byref(h)) == C.PN_EINVAL
    assert L.pn_model_init(ctypes.byref(cfg), ctypes.c_void_p(1 << 20), need - 1, ctypes.byref(h)) == C.PN_ERANGE
    assert L.pn_model_init(ctypes.byref(cfg), ctypes.c_void_p((1 << 20) + 8), need, ctypes.byref(h)) == C.PN_EINVAL
    # a layout on a fake (never dereferenced) address: sizing queries need no device
    assert L.pn_model_init(ctypes.byref(cfg), ctypes.c_void_p(1 << 20), need, ctypes.byref(h)) == 0
    try:
        assert L.pn_state_bytes(h, 132) > 0
        assert L.pn_state_bytes(h, -1) == 0
        assert L.pn_state_bytes(h, 2_000_000_000) == 0  # one layer's K pool past 2 GiB
        st = ctypes.c_void_p()
        assert L.pn_state_new(h, 64, None, 1 << 20, None, ctypes.byref(st)) == C.PN_EINVAL
        assert L.pn_state_new(h, 64, ctypes.c_void_p(1 << 21), 16, None, ctypes.byref(st)) == C.PN_ERANGE
        arr = (ctypes.c_void_p * 1)(None)
        assert L.pn_forward_batch(h, arr, 1, ctypes.c_void_p(1 << 22), None, None, None) == C.PN_EINVAL
        assert L.pn_forward_batch(h, arr, 2, ctypes.c_void_p(1 << 22), None, None, None) == C.PN_EINVAL
        assert L.pn_model_set_option(h, C.PN_OPT_ATTN_KEYS_PER_SPLIT, 100) == C.PN_EINVAL
        assert L.pn_model_set_option(h, C.PN_OPT_ATTN_KEYS_PER_SPLIT, 512) == 0
        assert L.pn_model_set_option(h, C.PN_OPT_ATTN_KERNEL, 3) == C.PN_EINVAL
        assert L.pn_model_set_option(h, C.PN_OPT_ATTN_KERNEL, 2) == 0
        assert L.pn_model_set_option(h, C.PN_OPT_ATTN_COMBINE, 2) == C.PN_EINVAL
        assert L.pn_model_set_option(h, C.PN_OPT_ATTN_COMBINE, 1) == 0
        assert L.pn_model_set_option(h, C.PN_OPT_ATTN_COMBINE, 0) == 0
        assert L.pn_model_set_option(h, C.PN_OPT_ATTN_WAVES, 16) == C.PN_EINVAL
        assert L.pn_model_set_option(h, C.PN_OPT_ATTN_WAVES, 8) == 0
        assert L.pn_model_set_option(h, C.PN_OPT_ATTN_WAVES, 0) == 0
        assert L.pn_model_set_option(h, C.PN_OPT_GEMM_PROLOGUE, 2) == C.PN_EINVAL
        assert L.pn_model_set_option(h, C.PN_OPT_GEMM_PROLOGUE, 1) == 0
        assert L.pn_model_set_option(h, C.PN_OPT_GEMM_PROLOGUE, 0) == 0
        assert L.pn_profile_begin(h, 99) == C.PN_EINVAL
        # shared page pool: sizing, creation and argument checks enqueue nothing
        page = L.pn_pool_bytes(h, 1)
        assert page > 0 and L.pn_pool_bytes(h, 10) == 10 * page
        assert L.pn_pool_bytes(h, 0) == 0 and L.pn_pool_bytes(None, 4) == 0
        assert L.pn_pool_bytes(h, 1 << 30) == 0  # one layer's K pages past 2 GiB
        pool = ctypes.c_void_p()
        assert L.pn_pool_new(h, 10, ctypes.c_void_p(1 << 24), 10 * page - 1, ctypes.byref(pool)) == C.PN_ERANGE
        assert L.pn_pool_new(h, 10, ctypes.c_void_p((1 << 24) + 64), 10 * page, ctypes.byref(pool)) == C.PN_EINVAL
        assert L.pn_pool_new(h, 0, ctypes.c_void_p(1 << 24), 10 * page, ctypes.byref(pool)) == C.PN_EINVAL
        assert L.pn_pool_new(h, 10, ctypes.c_void_p(1 << 24), 10 * page, ctypes.byref(pool)) == 0
        try:
            assert L.pn_pool_free_pages(pool) == 10 and L.pn_pool_free_pages(None) == -1
            sb = L.pn_state_bytes_pooled(h, 132)
            assert 0 < sb < L.pn_state_bytes(h, 132)
            assert L.pn_state_bytes_pooled(h, 2_000_000_000) > 0  # K/V live in the pool
            assert L.pn_state_new_pooled(h, None, 64, ctypes.c_void_p(1 << 21), sb, None, ctypes.byref(st)) == C.PN_EINVAL
            assert L.pn_state_new_pooled(h, pool, 132, ctypes.c_void_p(1 << 21), sb - 1, None,
                                         ctypes.byref(st)) == C.PN_ERANGE
        finally:
            L.pn_pool_free(pool)
        # sampling: every argument is checked on the host before anything is enqueued
        sp = (C.pn_sampling_params * 2)()
        for i in range(2):
            sp[i].temperature, sp[i].repeat_penalty, sp[i].top_k, sp[i].top_p = 1.0, 1.0, 40, 0.9
        dv_ = ctypes.c_void_p(1 << 22)
        assert L.pn_sample(h, dv_, 0, sp, None, 0, dv_, dv_, None) == C.PN_EINVAL
        assert L.pn_sample(h, None, 1, sp, None, 0, dv_, dv_, None) == C.PN_EINVAL
        assert L.pn_sample(h, dv_, 1, sp, None, 2000, dv_, dv_, None) == C.PN_EINVAL
        assert L.pn_sample(h, dv_, 1, sp, None, 8, dv_, dv_, None) == C.PN_EINVAL  # recent NULL
        sp[0].top_k = 0
        assert L.pn_sample(h, dv_, 1, sp, None, 0, dv_, dv_, None) == C.PN_EUNSUPPORTED
        sp[0].top_k = 5000
        assert L.pn_sample(h, dv_, 1, sp, None, 0, dv_, dv_, None) == C.PN_EUNSUPPORTED
        sp[0].top_k, sp[0].repeat_penalty = 40, 0.0
        assert L.pn_sample(h, dv_, 1, sp, None, 0, dv_, dv_, None) == C.PN_EINVAL
        sp[0].repeat_penalty, sp[0].temperature = 1.0, float("nan")
        assert L.pn_sample(h, dv_, 1, sp, None, 0, dv_, dv_, None) == C.PN_EINVAL
        assert L.pn_profile_replay(h, C.PN_K_GATEUP, 4, None) == C.PN_EINVAL  # nothing recorded yet
        assert L.pn_profile_replay(h, 99, 4, None) == C.PN_EINVAL
        lw = C.pn_layer_weights()
        assert L.pn_model_load_layer(h, 0, ctypes.byref(lw), None) == C.PN_EINVAL
        assert L.pn_model_load_layer(h, 5, ctypes.byref(lw), None) == C.PN_EINVAL
    finally:
        L.pn_model_free(h)


def test_package_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(C, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(C, "_lib", None)
    with pytest.raises(ImportError):
        C.lib()


def test_wide_prefill_buffers_in_model_bytes():
    """The wide path's row buffers are part of pn_model_bytes: larger chunks take more."""
    L = C.lib()
    sizes = []
    for chunk in (0, 32, 128):
        cfg = good_cfg(prefill_chunk=chunk, w_dtype=C.PN_BF16, act_dtype=C.PN_F32)
        sizes.append(L.pn_model_bytes(ctypes.byref(cfg)))
    assert 0 < sizes[0] < sizes[1] < sizes[2]


def test_model_create_checks_every_layer_before_any_device_work():
    """pn_model_create validates the pointers of every layer before it enqueues
    anything: a NULL in the last layer fails with PN_EINVAL and names that layer.
    (On this host there is no device, so any enqueue would fail as PN_EHIP.)"""
    L = C.lib()
    cfg = good_cfg(n_layer=4)
    need = L.pn_model_bytes(ctypes.byref(cfg))
    fake = ctypes.c_void_p(1 << 20)
    layers = (C.pn_layer_weights * 4)()
    for l in range(4):
        for name, _ in C.pn_layer_weights._fields_:
            if name in ("w_router", "s_q", "s_k", "s_v", "s_o", "s_gate", "s_up", "s_down", "b_q", "b_k", "b_v"):
                continue
            setattr(layers[l], name, fake.value)
    layers[3].wo = None
    w = C.pn_weights(fake.value, fake.value, fake.value, None, layers)
    h = ctypes.c_void_p()
    assert L.pn_model_create(ctypes.byref(cfg), ctypes.byref(w), fake, need, None, ctypes.byref(h)) == C.PN_EINVAL
    assert b"layer 3" in L.pn_last_error()
    assert not h.value
    w.w_out = None
    assert L.pn_model_create(ctypes.byref(cfg), ctypes.byref(w), fake, need, None, ctypes.byref(h)) == C.PN_EINVAL
    assert b"global" in L.pn_last_error()


def test_route_log_and_stream_read_arguments():
    L = C.lib()
    fake = ctypes.c_void_p(1 << 20)
    for kw, ok in ((dict(), False), (dict(n_expert=4, n_expert_used=2), True)):
        cfg = good_cfg(**kw)
        need = L.pn_model_bytes(ctypes.byref(cfg))
        h = ctypes.c_void_p()
        assert L.pn_model_init(ctypes.byref(cfg), fake, need, ctypes.byref(h)) == 0
        try:
            rc = L.pn_model_route_log(h, ctypes.c_void_p(1 << 22), 4)
            assert rc == (0 if ok else C.PN_EINVAL)
            if ok:
                assert L.pn_model_route_log(h, ctypes.c_void_p(1 << 22), 0) == C.PN_EINVAL
                assert L.pn_model_route_log(h, None, 0) == 0  # off
        finally:
            L.pn_model_free(h)
    assert L.pn_model_route_log(None, None, 0) == C.PN_EINVAL
    assert L.pn_stream_read(None, 1024, fake, None) == C.PN_EINVAL
    assert L.pn_stream_read(fake, 1000, fake, None) == C.PN_EINVAL
    assert L.pn_stream_read(ctypes.c_void_p((1 << 20) + 4), 1024, fake, None) == C.PN_EINVAL


def test_sample_noalloc_rejects_sizes_past_its_array():
    """pn_sample_noalloc's bounds are checked on the host, before any device work."""
    L = C.lib()
    sp = (C.pn_sampling_params * 1)()
    sp[0].temperature, sp[0].repeat_penalty, sp[0].top_k, sp[0].top_p = 1.0, 1.0, 40, 0.9
    d = ctypes.c_void_p(1 << 22)
    assert L.pn_sample_noalloc(d, 0, 1000, sp, None, 0, d, d, None) == C.PN_EINVAL
    assert L.pn_sample_noalloc(d, 17, 1000, sp, None, 0, d, d, None) == C.PN_EINVAL
    assert L.pn_sample_noalloc(d, 1, 0, sp, None, 0, d, d, None) == C.PN_EINVAL
    assert L.pn_sample_noalloc(d, 1, 262145, sp, None, 0, d, d, None) == C.PN_EINVAL
    assert L.pn_sample_noalloc(None, 1, 1000, sp, None, 0, d, d, None) == C.PN_EINVAL
    assert L.pn_sample_noalloc(d, 1, 262145, sp, None, 0, d, d, None) == C.PN_EINVAL
    assert b"262144" in L.pn_last_error()
