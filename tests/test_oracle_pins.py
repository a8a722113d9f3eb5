"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test checks one building block (or the whole step) against a closed form,
an invariant, a brute-force or library computation (torch CPU routines in
float64), or a special case that reduces to the textbook form.  Each was chosen
so that a plausible slip (a dropped term, a wrong sign or index, a transposed
operand, an off-by-one window) fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth

rng = np.random.default_rng(1234)


# ----------------------------------------------------------------------------- RMSNorm

def test_rmsnorm_constant_vector_closed_form():
    E, c, eps = 96, 0.37, 1e-5
    g = (1.0 + 0.1 * rng.standard_normal(E)).astype(np.float32)
    y = oracle.rmsnorm(np.full(E, c), g, eps)
    want = c / math.sqrt(c * c + eps) * g.astype(np.float64)
    np.testing.assert_allclose(y, want, rtol=1e-15, atol=0)


def test_rmsnorm_unit_rms_and_scale_invariance():
    E = 257
    x = rng.standard_normal(E) * 3.0
    ones = np.ones(E, dtype=np.float32)
    y = oracle.rmsnorm(x, ones, 0.0)
    assert abs(np.sum(y * y) - E) < 1e-9 * E
    np.testing.assert_allclose(oracle.rmsnorm(x * 1000.0, ones, 0.0), y, rtol=1e-13)


def test_rmsnorm_matches_torch_rms_norm():
    E, eps = 512, 1e-5
    x = rng.standard_normal(E)
    g = (1.0 + 0.1 * rng.standard_normal(E)).astype(np.float32)
    ref = F.rms_norm(torch.tensor(x), (E,), weight=torch.tensor(g.astype(np.float64)), eps=eps)
    np.testing.assert_allclose(oracle.rmsnorm(x, g, eps), ref.numpy(), rtol=1e-13)


# ----------------------------------------------------------------------------- RoPE

def _rope_complex(u, pos, theta):
    """RoPE written as a complex product of adjacent pairs (torch.polar)."""
    d = u.size
    freqs = 1.0 / (theta ** (torch.arange(0, d, 2, dtype=torch.float64) / d))
    rot = torch.polar(torch.ones(d // 2, dtype=torch.float64), pos * freqs)
    z = torch.view_as_complex(torch.tensor(u).reshape(d // 2, 2).contiguous())
    return torch.view_as_real(z * rot).reshape(d).numpy()


@pytest.mark.parametrize("d,theta", [(32, 1e4), (128, 5e5), (64, 1e4)])
def test_rope_matches_complex_rotation(d, theta):
    for pos in (0, 1, 7, 2048, 16511):
        u = rng.standard_normal(d)
        np.testing.assert_allclose(oracle.rope(u, pos, theta), _rope_complex(u, pos, theta),
                                   rtol=0, atol=1e-12)


def _rope_half_split_complex(u, pos, theta):
    """NeoX RoPE as a complex product: z_i = u_i + 1j * u_{i+d/2} (numpy complex)."""
    d = u.size
    h = d // 2
    freqs = theta ** (-np.arange(0, d, 2, dtype=np.float64) / d)
    z = (u[:h] + 1j * u[h:]) * np.exp(1j * pos * freqs)
    return np.concatenate([z.real, z.imag])


@pytest.mark.parametrize("d,theta", [(32, 1e4), (128, 1e6), (64, 1e4)])
def test_rope_neox_matches_half_split_complex_rotation(d, theta):
    for pos in (0, 1, 9, 4096, 30001):
        u = rng.standard_normal(d)
        # the angle pos * w carries pos * ulp(w) of difference between the two ways of computing w
        np.testing.assert_allclose(oracle.rope_neox(u, pos, theta), _rope_half_split_complex(u, pos, theta),
                                   rtol=0, atol=2e-11)


def test_rope_neox_pairs_and_relative_position():
    d, h = 64, 32
    u = rng.standard_normal(d)
    np.testing.assert_array_equal(oracle.rope_neox(u, 0, 1e4), u)
    r = oracle.rope_neox(u, 777, 1e4)
    np.testing.assert_allclose(r[:h] ** 2 + r[h:] ** 2, u[:h] ** 2 + u[h:] ** 2, rtol=1e-12)
    assert not np.allclose(r, oracle.rope(u, 777, 1e4))  # not the adjacent-pair form
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for m, n, delta in [(5, 2, 100), (300, 17, 4000)]:
        a = oracle.rope_neox(q, m, 1e4) @ oracle.rope_neox(k, n, 1e4)
        b = oracle.rope_neox(q, m + delta, 1e4) @ oracle.rope_neox(k, n + delta, 1e4)
        assert abs(a - b) < 1e-9


def test_rope_identity_at_zero_and_pair_norms():
    d = 64
    u = rng.standard_normal(d)
    np.testing.assert_array_equal(oracle.rope(u, 0, 1e4), u)
    r = oracle.rope(u, 1234, 1e4)
    np.testing.assert_allclose(np.hypot(r[0::2], r[1::2]), np.hypot(u[0::2], u[1::2]), rtol=1e-14)


def test_rope_theta_dependence():
    d, p = 128, 37
    e0 = np.zeros(d)
    e0[0::2] = 1.0  # every pair starts at angle 0
    for theta in (1e4, 5e5):
        r = oracle.rope(e0, p, theta)
        ang = np.arctan2(r[1::2], r[0::2])
        # pair 0 turns by exactly p radians whatever theta is
        assert abs(math.remainder(ang[0] - p, 2 * math.pi)) < 1e-12
        # the last pair turns by p * theta^(-(d-2)/d)
        want = p * theta ** (-(d - 2) / d)
        assert abs(math.remainder(ang[-1] - want, 2 * math.pi)) < 1e-12
    # changing theta changes only pairs i > 0
    a, b = oracle.rope(e0, p, 1e4), oracle.rope(e0, p, 5e5)
    np.testing.assert_array_equal(a[:2], b[:2])
    assert np.all(np.abs(a[2:] - b[2:]).reshape(-1, 2).max(axis=1) > 0)


def test_rope_relative_position():
    d = 32
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for m, n, delta in ((5, 2, 11), (100, 0, 3), (7, 7, 1000)):
        a = oracle.rope(q, m, 1e4) @ oracle.rope(k, n, 1e4)
        b = oracle.rope(q, m + delta, 1e4) @ oracle.rope(k, n + delta, 1e4)
        assert abs(a - b) < 1e-11 * (1 + abs(a))


# ----------------------------------------------------------------------------- attention

def _sdpa(q, K, V, pos, window):
    """torch scaled_dot_product_attention (float64) with GQA and an explicit boolean mask."""
    H, d = q.shape
    Hk, T, _ = K.shape
    t = torch.arange(T)
    lo = max(0, pos - window + 1) if window > 0 else 0
    mask = (t >= lo) & (t <= pos)
    out = F.scaled_dot_product_attention(
        torch.tensor(q)[None, :, None, :], torch.tensor(K)[None], torch.tensor(V)[None],
        attn_mask=mask[None, None, None, :], enable_gqa=True)
    return out[0, :, 0, :].numpy()


@pytest.mark.parametrize("H,Hk,d,T", [(8, 2, 32, 40), (4, 4, 16, 30), (6, 1, 8, 25), (32, 8, 128, 70)])
def test_attention_matches_sdpa(H, Hk, d, T):
    q = rng.standard_normal((H, d))
    K = rng.standard_normal((Hk, T, d))
    V = rng.standard_normal((Hk, T, d))
    for pos in (0, 1, T // 2, T - 1):
        for W in (0, 1, 3, 8, T + 5):
            np.testing.assert_allclose(oracle.attention(q, K, V, pos, W), _sdpa(q, K, V, pos, W),
                                       rtol=1e-12, atol=1e-12)


def test_window_bruteforce_small_contexts():
    H, Hk, d = 4, 2, 8
    for p in range(0, 25):
        T = p + 1
        q = rng.standard_normal((H, d))
        K = rng.standard_normal((Hk, T, d))
        V = rng.standard_normal((Hk, T, d))
        full = oracle.attention(q, K, V, p, 0)
        for W in (1, 2, 3, 5, 8):
            got = oracle.attention(q, K, V, p, W)
            np.testing.assert_allclose(got, _sdpa(q, K, V, p, W), rtol=1e-12, atol=1e-13)
            if W >= p + 1:
                np.testing.assert_array_equal(got, full)
            if W == 1:  # a one-key window returns the newest value exactly
                np.testing.assert_array_equal(got, V[np.arange(H) // (H // Hk), p])


def test_attention_special_cases():
    d, T = 16, 9
    q = rng.standard_normal(d)
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d))
    # one key: the output is that value exactly
    np.testing.assert_array_equal(oracle.attend(q, K[:1], V[:1]), V[0])
    # equal scores: the mean of the values
    np.testing.assert_allclose(oracle.attend(q, np.zeros((T, d)), V), V.mean(axis=0), rtol=1e-14)
    # shifting every score by the same amount changes nothing
    u = rng.standard_normal(d)
    np.testing.assert_allclose(oracle.attend(q, K + u, V), oracle.attend(q, K, V), rtol=1e-12)


def test_gqa_equals_mha_with_repeated_kv():
    H, Hk, d, T = 8, 2, 16, 12
    q = rng.standard_normal((H, d))
    K = rng.standard_normal((Hk, T, d))
    V = rng.standard_normal((Hk, T, d))
    rep = H // Hk
    Kr, Vr = np.repeat(K, rep, axis=0), np.repeat(V, rep, axis=0)
    for pos, W in ((11, 0), (6, 3)):
        np.testing.assert_array_equal(oracle.attention(q, K, V, pos, W),
                                      oracle.attention(q, Kr, Vr, pos, W))


# ----------------------------------------------------------------------------- FFN pieces

def test_silu_matches_torch():
    for z in (-30.0, -2.5, -1e-3, 0.0, 0.7, 4.0, 50.0):
        assert abs(oracle.silu(z) - F.silu(torch.tensor(z, dtype=torch.float64)).item()) < 1e-15


def test_moe_route_weights():
    for _ in range(20):
        r = rng.standard_normal(8) * 2
        ids, w, gap = oracle.moe_route(r, 2)
        assert abs(w.sum() - 1.0) < 1e-14
        want = torch.softmax(torch.tensor(r[ids]), 0).numpy()
        np.testing.assert_allclose(w, want, rtol=1e-13)
        order = np.argsort(-r.astype(np.float32), kind="stable")
        np.testing.assert_array_equal(ids, order[:2])
        assert gap >= 0
    # ties go to the lower index
    ids, w, gap = oracle.moe_route(np.array([0.5, 1.0, 1.0, 1.0, 0.2]), 2)
    assert list(ids) == [1, 2] and gap == 0.0
    np.testing.assert_allclose(w, [0.5, 0.5])


def test_argmax_lowest_index_on_ties():
    x = rng.standard_normal(1000)
    x[[17, 400, 999]] = 9.0
    assert oracle.argmax(x) == 17
    y = rng.standard_normal(5000)
    assert oracle.argmax(y) == int(np.argmax(y.astype(np.float32)))
    # values equal in fp32 but not in fp64 are a tie
    z = np.zeros(10)
    z[3], z[6] = 1.0, 1.0 + 1e-12
    assert oracle.argmax(z) == 3


def test_round_bf16_matches_torch():
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    mine = np.array([oracle.round_bf16(float(a)) for a in v])
    ref = torch.tensor(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(mine, ref)


# ----------------------------------------------------------------------------- Q8_0 weights

def test_half_to_double_matches_numpy_float16():
    bits = np.concatenate([np.arange(0, 0x7C00, 37), [0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF]]).astype(np.uint16)
    bits = np.concatenate([bits, bits | 0x8000])
    want = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(b) for b in bits])
    np.testing.assert_array_equal(got, want)
    assert oracle.half_to_double(0x7C00) == np.inf and np.isnan(oracle.half_to_double(0x7E00))


def _q8_block(d, codes):
    return np.concatenate([np.array([d], np.float16).view(np.uint8),
                           np.asarray(codes, np.int8).view(np.uint8)])


def test_q8_0_matvec_closed_form():
    # two rows of two blocks: d = 0.5 and 2^-20 (an fp16 subnormal scale); then -0.25 and 3
    c = np.arange(-16, 16)
    W = np.stack([np.concatenate([_q8_block(0.5, c), _q8_block(2.0 ** -20, c[::-1])]),
                  np.concatenate([_q8_block(-0.25, np.full(32, 127)), _q8_block(3.0, np.full(32, -128))])])
    x = np.concatenate([np.ones(32), np.full(32, 2.0)])
    y = oracle.matvec(W, synth.Q8_0, None, 2, 64, x)
    want0 = 0.5 * c.sum() + 2.0 * 2.0 ** -20 * c[::-1].sum()
    want1 = -0.25 * 127 * 32 + 2.0 * 3.0 * (-128) * 32
    np.testing.assert_array_equal(y, [want0, want1])
    # one-hot x reads single weights: d * q at block b, index i
    for col in (0, 31, 32, 47, 63):
        e = np.zeros(64)
        e[col] = 1.0
        d = (0.5, 2.0 ** -20)[col // 32]
        q = (c, c[::-1])[col // 32][col % 32]
        assert oracle.matvec(W, synth.Q8_0, None, 2, 64, e)[0] == d * q


def test_q8_0_matvec_matches_numpy_dequantisation():
    w = rng.standard_normal((24, 160)).astype(np.float32) * 0.05
    blocks = synth.q8_0_blocks(w)
    b = blocks.reshape(24, 5, 34)
    deq = (b[:, :, 0:2].copy().view(np.float16).astype(np.float64)
           * b[:, :, 2:].copy().view(np.int8).astype(np.float64)).reshape(24, 160)
    assert np.abs(deq - w).max() <= np.abs(w).max() / 127  # a faithful quantisation of w
    x = rng.standard_normal(160)
    np.testing.assert_allclose(oracle.matvec(blocks, synth.Q8_0, None, 24, 160, x), deq @ x, rtol=1e-13)


def _q4_block(d, codes):
    codes = np.asarray(codes, np.uint8)
    return np.concatenate([np.array([d], np.float16).view(np.uint8), codes[:16] | (codes[16:] << 4)])


def test_q4_0_matvec_closed_form():
    c = np.arange(32) % 16  # codes 0..15, 0..15: weights d * (-8..7)
    W = np.stack([np.concatenate([_q4_block(0.5, c), _q4_block(-2.0 ** -18, c[::-1])])])
    x = np.concatenate([np.ones(32), np.full(32, 3.0)])
    y = oracle.matvec(W, synth.Q4_0, None, 1, 64, x)
    want = 0.5 * (c - 8).sum() + 3.0 * -(2.0 ** -18) * (c[::-1] - 8).sum()
    np.testing.assert_array_equal(y, [want])
    for col in (0, 5, 15, 16, 31, 32, 48, 63):  # low nibbles hold codes 0..15, high ones 16..31
        e = np.zeros(64)
        e[col] = 1.0
        d = (0.5, -(2.0 ** -18))[col // 32]
        code = (c, c[::-1])[col // 32][col % 32]
        assert oracle.matvec(W, synth.Q4_0, None, 1, 64, e)[0] == d * (int(code) - 8)


def test_q4_0_rows_are_a_faithful_quantisation():
    q = synth.q4_0_rows(3, 9, 24, 160)
    b = q.reshape(24, 5, 18)
    d = b[:, :, 0:2].copy().view(np.float16).astype(np.float64)
    codes = np.concatenate([b[:, :, 2:] & 15, b[:, :, 2:] >> 4], axis=2).astype(np.float64)
    deq = (d * (codes - 8)).reshape(24, 160)
    w = synth.normal(3, 9, 24 * 160, 0.0, synth.W_STD, synth.F32).reshape(24, 160).astype(np.float64)
    amax = np.abs(w.reshape(24, 5, 32)).max(axis=2)
    # half a step (d = amax / 8) everywhere, a whole step where +8 steps clip to code 15
    assert np.all(np.abs(deq - w).reshape(24, 5, 32).max(axis=2) <= amax / 8 * 1.01)
    x = rng.standard_normal(160)
    np.testing.assert_allclose(oracle.matvec(q, synth.Q4_0, None, 24, 160, x), deq @ x, rtol=1e-13)


# ----------------------------------------------------------------------------- Q4 KV cache

def test_q4_kv_round_worked_examples():
    z = [0.0] * 24
    # m = -4: d = 0.5; 0.25 / 0.5 = 0.5 rounds to even (0), 0.75 / 0.5 = 1.5 to 2, -0.5 to -0
    got = oracle.q4_kv_round(np.array([-4, 1, 2, 3.5, 0, 0.25, 0.75, -0.25] + z))
    np.testing.assert_array_equal(got[:8], [-4, 1, 2, 3.5, 0, 0, 1, 0])
    # m = +4: d = -0.5; -4 would be code 16 and clips to 15: -0.5 * 7 = -3.5
    got = oracle.q4_kv_round(np.array([4, -4, 1] + [0.0] * 29))
    np.testing.assert_array_equal(got[:3], [4, -3.5, 1])
    # equal magnitudes: the first is m (3 -> d = -0.375, so -3 clips to -2.625)
    got = oracle.q4_kv_round(np.array([3, -3] + [0.0] * 30))
    np.testing.assert_array_equal(got[:2], [3, -2.625])
    # d is an fp16: m = 1 + 2^-12 gives d = -0.125 exactly, so m itself comes back as 1
    got = oracle.q4_kv_round(np.array([1 + 2.0 ** -12] + [0.0] * 31))
    assert got[0] == 1.0
    # an all-zero block stays zero; blocks are independent
    got = oracle.q4_kv_round(np.array([0.0] * 32 + [8.0] + [0.0] * 31))
    np.testing.assert_array_equal(got[:32], 0.0)
    assert got[32] == 8.0


def test_q4_kv_round_values_are_scaled_codes():
    for trial in range(20):
        u = rng.standard_normal(128) * (10.0 ** rng.uniform(-3, 2))
        got = oracle.q4_kv_round(u)
        for b in range(4):
            blk, g = u[32 * b: 32 * b + 32], got[32 * b: 32 * b + 32]
            m = blk[np.argmax(np.abs(blk.astype(np.float32)))]
            d = float(np.float16(np.float32(m) / np.float32(-8.0)))
            codes = g / d + 8
            np.testing.assert_array_equal(codes, np.rint(codes))
            assert codes.min() >= 0 and codes.max() <= 15
            ok = codes != 15  # away from the clipped end every value is within half a step
            assert np.all(np.abs(g - blk)[ok] <= abs(d) / 2 * (1 + 1e-6))


# ----------------------------------------------------------------------------- whole model

def _torch_forward(wl, W, tokens, kv_out=None):
    """The same model built from torch library routines (float64), full causal recompute.
    With `kv_out` (a list), each layer appends (k, v): every position's cached k
    (after RoPE) and v, [n][Hk][d], in the form a cache of the workload's KV type
    is written with (fp32 values, bf16 bits, or fp32 values before Q4 blocks)."""
    E, H, Hk, d = wl.n_embd, wl.n_head, wl.n_kv_head, wl.head_dim

    def mat(m, s=None):
        if m.dtype == np.uint8 and wl.w_dtype == synth.Q8_0:  # fp16 scale, 32 int8 codes
            b = m.reshape(m.shape[0], -1, 34)
            d = b[:, :, 0:2].copy().view(np.float16).astype(np.float64)
            q = b[:, :, 2:].copy().view(np.int8).astype(np.float64)
            return torch.tensor((d * q).reshape(m.shape[0], -1))
        if m.dtype == np.uint8:  # Q4_0: fp16 scale, codes 0..15 in nibbles (i low, i + 16 high)
            b = m.reshape(m.shape[0], -1, 18)
            d = b[:, :, 0:2].copy().view(np.float16).astype(np.float64)
            codes = np.concatenate([b[:, :, 2:] & 15, b[:, :, 2:] >> 4], axis=2).astype(np.float64)
            return torch.tensor((d * (codes - 8)).reshape(m.shape[0], -1))
        if m.dtype == np.uint16:
            a = torch.tensor(synth.bf16_to_f32(m).astype(np.float64))
        elif m.dtype == np.int8:
            a = torch.tensor(m.astype(np.float64)) * torch.tensor(s.astype(np.float64))[:, None]
        else:
            a = torch.tensor(m.astype(np.float64))
        return a

    def act(t):
        if wl.act_dtype == synth.BF16:
            return t.to(torch.bfloat16).to(torch.float64)
        return t.to(torch.float32).to(torch.float64)

    def kvr(t):
        if wl.kv_dtype == synth.BF16:
            return t.to(torch.bfloat16).to(torch.float64)
        if wl.kv_dtype == synth.Q4_0:  # per head vector, blocks of 32: fp16 scale, 4-bit codes
            f = t.to(torch.float32).numpy().reshape(-1, 32)
            m = f[np.arange(len(f)), np.argmax(np.abs(f), axis=1)]
            dd = (m / np.float32(-8.0)).astype(np.float16).astype(np.float32)[:, None]
            with np.errstate(divide="ignore", invalid="ignore"):
                c = np.where(dd != 0, np.clip(np.rint(f / np.where(dd != 0, dd, 1)) + 8, 0, 15), 8)
            return torch.tensor((dd.astype(np.float64) * (c - 8)).reshape(t.shape))
        return t.to(torch.float32).to(torch.float64)

    n = len(tokens)
    x = mat(W["tok_embd"])[torch.tensor(np.asarray(tokens, dtype=np.int64))]
    pos = torch.arange(n, dtype=torch.float64)
    freqs = 1.0 / (wl.rope_theta ** (torch.arange(0, d, 2, dtype=torch.float64) / d))
    rot = torch.polar(torch.ones(n, d // 2, dtype=torch.float64), pos[:, None] * freqs[None])

    def rope(t):  # t [n, heads, d]
        if wl.rope_neox:  # half-split pairs (i, i + d/2): rotate_half form
            c, s_ = rot.real[:, None, :].repeat(1, 1, 2), rot.imag[:, None, :].repeat(1, 1, 2)
            half = torch.cat([-t[..., d // 2:], t[..., :d // 2]], dim=-1)
            return t * c + half * s_
        z = torch.view_as_complex(t.reshape(n, t.shape[1], d // 2, 2).contiguous())
        return torch.view_as_real(z * rot[:, None, :]).reshape(t.shape)

    def bias(name):
        b = L.get(name)
        return 0.0 if b is None else torch.tensor(b.astype(np.float64))

    tpos = torch.arange(n)
    mask = tpos[None, :] <= tpos[:, None]
    if wl.sliding_window > 0:
        mask &= tpos[None, :] > tpos[:, None] - wl.sliding_window
    for L in W["layers"]:
        g = torch.tensor(L["attn_norm"].astype(np.float64))
        xn = act(F.rms_norm(x, (E,), weight=g, eps=wl.rms_norm_eps))
        q = rope((xn @ mat(L["wq"], L["s_q"]).T + bias("b_q")).reshape(n, H, d))
        k_raw = rope((xn @ mat(L["wk"], L["s_k"]).T + bias("b_k")).reshape(n, Hk, d))
        v_raw = (xn @ mat(L["wv"], L["s_v"]).T + bias("b_v")).reshape(n, Hk, d)
        k, v = kvr(k_raw), kvr(v_raw)
        if kv_out is not None:
            if wl.kv_dtype == synth.BF16:
                kv_out.append(tuple(t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
                                    for t in (k_raw, v_raw)))
            else:
                kv_out.append(tuple(t.to(torch.float32).numpy().copy() for t in (k_raw, v_raw)))
        o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None],
                                           v.transpose(0, 1)[None], attn_mask=mask[None, None],
                                           enable_gqa=True)[0].transpose(0, 1).reshape(n, H * d)
        x = x + act(o) @ mat(L["wo"], L["s_o"]).T
        g2 = torch.tensor(L["ffn_norm"].astype(np.float64))
        xn2 = act(F.rms_norm(x, (E,), weight=g2, eps=wl.rms_norm_eps))
        if wl.n_expert == 0:
            h = act(F.silu(xn2 @ mat(L["w_gate"][0], L["s_gate"][0]).T)
                    * (xn2 @ mat(L["w_up"][0], L["s_up"][0]).T))
            x = x + h @ mat(L["w_down"][0], L["s_down"][0]).T
        else:
            r = xn2 @ mat(L["w_router"]).T
            top = torch.topk(r, wl.n_expert_used, dim=-1)
            wts = torch.softmax(top.values, dim=-1)
            out = torch.zeros_like(x)
            for t in range(n):
                for a in range(wl.n_expert_used):
                    e = int(top.indices[t, a])
                    h = act(F.silu(xn2[t] @ mat(L["w_gate"][e], L["s_gate"][e]).T)
                            * (xn2[t] @ mat(L["w_up"][e], L["s_up"][e]).T))
                    out[t] += wts[t, a] * (h @ mat(L["w_down"][e], L["s_down"][e]).T)
            x = x + out
    xf = act(F.rms_norm(x[-1], (E,), weight=torch.tensor(W["out_norm"].astype(np.float64)),
                        eps=wl.rms_norm_eps))
    return (xf @ mat(W["w_out"], W["s_out"]).T).numpy()


SMALL = [
    synth.tiny_fp32().with_(name="small-dense-f32", n_layer=2),
    synth.tiny_fp32().with_(name="small-window-bf16", w_dtype=synth.BF16, kv_dtype=synth.BF16,
                            act_dtype=synth.BF16, sliding_window=3, seed=11),
    synth.tiny_fp32().with_(name="small-int8", w_dtype=synth.I8, kv_dtype=synth.BF16,
                            act_dtype=synth.BF16, seed=12, n_head=4, n_kv_head=4, head_dim=64),
    synth.tiny_fp32().with_(name="small-moe", n_expert=4, n_expert_used=2, seed=13, n_ff=96),
    synth.tiny_fp32().with_(name="small-neox-bias-f32", rope_neox=True, qkv_bias=True, seed=14),
    synth.tiny_fp32().with_(name="small-neox-bias-bf16-window", rope_neox=True, qkv_bias=True, w_dtype=synth.BF16,
                            kv_dtype=synth.BF16, act_dtype=synth.BF16, sliding_window=4, seed=15),
    synth.tiny_fp32().with_(name="small-bias-int8", qkv_bias=True, w_dtype=synth.I8, kv_dtype=synth.BF16,
                            act_dtype=synth.BF16, seed=16),
    synth.tiny_fp32().with_(name="small-neox-moe", rope_neox=True, n_expert=4, n_expert_used=2, seed=17, n_ff=96),
    synth.tiny_fp32().with_(name="small-q8_0", w_dtype=synth.Q8_0, kv_dtype=synth.BF16, act_dtype=synth.BF16,
                            seed=18, n_ff=672),
    synth.tiny_fp32().with_(name="small-q8_0-moe-neox-bias", w_dtype=synth.Q8_0, kv_dtype=synth.F32,
                            act_dtype=synth.BF16, n_expert=4, n_expert_used=2, n_ff=96, rope_neox=True,
                            qkv_bias=True, seed=19),
    synth.tiny_fp32().with_(name="small-q4_0", w_dtype=synth.Q4_0, kv_dtype=synth.BF16, act_dtype=synth.BF16,
                            seed=20, n_ff=672),
    synth.tiny_fp32().with_(name="small-q4kv-window", kv_dtype=synth.Q4_0, sliding_window=5, seed=22),
    synth.tiny_fp32().with_(name="small-q4kv-bf16-moe", w_dtype=synth.BF16, kv_dtype=synth.Q4_0,
                            act_dtype=synth.BF16, n_expert=4, n_expert_used=2, n_ff=96, seed=23),
    synth.tiny_fp32().with_(name="small-q4_0-moe-window", w_dtype=synth.Q4_0, kv_dtype=synth.BF16,
                            act_dtype=synth.BF16, n_expert=4, n_expert_used=2, n_ff=96, sliding_window=5, seed=21),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_whole_model_matches_torch_composition(wl):
    W = synth.make_weights(wl)
    m = oracle.Model(wl, W)
    tokens = list(synth.uniform_int(wl.seed, 99, 9, 0, wl.n_vocab - 1))
    ref = _torch_forward(wl, W, tokens)
    lf, _ = m.full_recompute(tokens)
    rel = np.linalg.norm(lf - ref) / np.linalg.norm(ref)
    assert rel < 1e-12, rel
    st = m.new_state(16)
    for t in tokens:
        li, _ = st.step(int(t))
    np.testing.assert_array_equal(li, lf)


def test_incremental_equals_full_recompute_tiny_fp32():
    """The KV-cache bookkeeping: every cached step equals a from-scratch causal forward."""
    wl = synth.tiny_fp32()
    m = oracle.Model(wl, synth.make_weights(wl))
    st = m.new_state(wl.prompt_len + wl.steps)
    seq = [int(t) for t in wl.prompt_tokens()]
    for i, t in enumerate(seq):
        li, am = st.step(t)
    for s in range(wl.steps):
        seq.append(am)
        li, am = st.step(am)
        if s % 4 == 0 or s == wl.steps - 1:
            lf, af = m.full_recompute(seq)
            rel = np.linalg.norm(li - lf) / np.linalg.norm(lf)
            assert rel <= 1e-12 and am == af, (s, rel)
    assert st.pos == wl.prompt_len + wl.steps


def test_single_expert_equals_dense():
    dense = synth.tiny_fp32().with_(n_layer=1, seed=21)
    moe = dense.with_(n_expert=1, n_expert_used=1)
    Wd = synth.make_weights(dense)
    Wm = synth.make_weights(moe)
    # the router of a one-expert model changes nothing: the expert weight is 1
    for k in ("w_gate", "w_up", "w_down"):
        np.testing.assert_array_equal(Wd["layers"][0][k][0], Wm["layers"][0][k][0])
    toks = [3, 99, 500, 7]
    ld, _ = oracle.Model(dense, Wd).full_recompute(toks)
    lm, _ = oracle.Model(moe, Wm).full_recompute(toks)
    np.testing.assert_allclose(lm, ld, rtol=1e-14, atol=1e-15)


def test_identical_experts_equal_dense():
    dense = synth.tiny_fp32().with_(n_layer=1, seed=22)
    moe = dense.with_(n_expert=4, n_expert_used=2)
    Wd = synth.make_weights(dense)
    Wm = synth.make_weights(moe)
    for k in ("w_gate", "w_up", "w_down"):
        Wm["layers"][0][k] = [Wd["layers"][0][k][0]] * 4
    for k in ("tok_embd", "out_norm", "w_out"):
        Wm[k] = Wd[k]
    for k in ("attn_norm", "ffn_norm", "wq", "wk", "wv", "wo"):
        Wm["layers"][0][k] = Wd["layers"][0][k]
    toks = [1, 2, 3]
    ld, _ = oracle.Model(dense, Wd).full_recompute(toks)
    lm, _ = oracle.Model(moe, Wm).full_recompute(toks)
    np.testing.assert_allclose(lm, ld, rtol=1e-13, atol=1e-14)


def test_state_errors():
    wl = synth.tiny_fp32().with_(n_layer=1)
    m = oracle.Model(wl, synth.make_weights(wl))
    st = m.new_state(2)
    st.step(1)
    st.step(2)
    with pytest.raises(ValueError):
        st.step(3)  # pos 2 is past max_ctx
    st2 = m.new_state(4)
    with pytest.raises(ValueError):
        st2.step(wl.n_vocab)  # token id out of range
