"""GPU parity of chunked prefill (pn_prefill) against the oracle's one step per
prompt token: every row's logits and greedy id, then ordinary decode steps on
the resulting cache (which checks every appended K/V)."""
import pytest

import synth

from harness import Pair, compare_step, log, oracle_threads

pytestmark = pytest.mark.gpu


def ragged(name, **kw):
    base = dict(n_layer=2, n_embd=200, n_head=6, n_kv_head=2, head_dim=32, n_ff=300, n_vocab=1000,
                rope_theta=10000.0, seed=81)
    base.update(kw)
    return synth.Workload(name, **base)


def run_prefill(p, start, prompt, n_decode, tol=None):
    import torch
    from token_decode_amd import device as dv
    wl = p.wl
    ds, os_ = p.states(0, start, start + len(prompt) + n_decode + 1)
    toks = torch.tensor([int(t) for t in prompt], dtype=torch.int32, device="cuda")
    logits = torch.empty(len(prompt), wl.n_vocab, dtype=torch.float32, device="cuda")
    am = torch.empty(len(prompt), dtype=torch.int32, device="cuda")
    dv.prefill(p.dm, ds, toks, logits, am)
    assert ds.pos == start + len(prompt)
    g, ga = logits.cpu().numpy(), am.cpu().numpy()
    worst, near, nxt = 0.0, 0, None
    th = oracle_threads()
    for t, tok in enumerate(prompt):
        ol, oa = os_.step(int(tok), th)
        if t % 32 == 31:
            log("    (oracle at prompt row %d)" % t)
        rel, nt = compare_step(wl, g[t], ol, int(ga[t]), oa, "prompt row %d:" % t, tol)
        worst, near, nxt = max(worst, rel), near + int(nt), oa
    # decode on from the prefilled cache
    tok = torch.tensor([nxt], dtype=torch.int32, device="cuda")
    lg1 = torch.empty(wl.n_vocab, dtype=torch.float32, device="cuda")
    a1 = torch.empty(1, dtype=torch.int32, device="cuda")
    for i in range(n_decode):
        dv.forward_step(p.dm, ds, tok, lg1, a1)
        ol, oa = os_.step(int(tok.item()), th)
        rel, nt = compare_step(wl, lg1.cpu().numpy(), ol, int(a1.item()), oa, "decode step %d:" % i, tol)
        worst, near = max(worst, rel), near + int(nt)
        tok.fill_(oa)
    return worst, near


def test_prefill_tiny_fp32_from_zero():
    wl = synth.tiny_fp32()
    p = Pair(wl, max_batch=16)
    prompt = list(synth.uniform_int(wl.seed, 91, 37, 0, wl.n_vocab - 1))
    worst, near = run_prefill(p, 0, prompt, 5)
    log("  tiny fp32, 37 prompt tokens in chunks of 16: worst rel L2 %.2e, near %d" % (worst, near))
    assert near == 0


def test_prefill_window_on_existing_cache():
    """Chunks of 16 over a 300-token cache with a 40-token window: rows of one
    chunk see each other's keys and drop the ones that leave the window."""
    wl = ragged("prefill-bf16-window", w_dtype=synth.BF16, kv_dtype=synth.BF16, act_dtype=synth.BF16,
                sliding_window=40)
    p = Pair(wl, max_batch=16)
    prompt = list(synth.uniform_int(wl.seed, 92, 50, 0, wl.n_vocab - 1))
    worst, near = run_prefill(p, 300, prompt, 3)
    log("  bf16 window 40, 50 tokens from 300: worst rel L2 %.2e, near %d" % (worst, near))


def test_prefill_fp32_activations_chunks_of_five():
    wl = ragged("prefill-actf32", w_dtype=synth.BF16, kv_dtype=synth.BF16, act_dtype=synth.F32, seed=82)
    p = Pair(wl, max_batch=5)
    prompt = list(synth.uniform_int(wl.seed, 93, 12, 0, wl.n_vocab - 1))
    worst, near = run_prefill(p, 63, prompt, 2)
    log("  bf16 weights, fp32 activations, 12 tokens from 63: worst rel L2 %.2e" % worst)


def test_prefill_moe():
    wl = ragged("prefill-moe", n_expert=4, n_expert_used=2, w_dtype=synth.BF16, kv_dtype=synth.BF16,
                act_dtype=synth.BF16, seed=83, n_ff=128)
    p = Pair(wl, max_batch=7)
    prompt = list(synth.uniform_int(wl.seed, 94, 10, 0, wl.n_vocab - 1))
    worst, near = run_prefill(p, 5, prompt, 2)
    log("  MoE, 10 tokens from 5: worst rel L2 %.2e" % worst)


def test_prefill_range_error():
    import torch
    from token_decode_amd import _capi as C
    from token_decode_amd import device as dv
    wl = synth.tiny_fp32()
    p = Pair(wl, max_batch=4)
    ds = dv.DeviceState(p.dm, 20)
    ds.pos = 15
    with pytest.raises(C.PNError) as e:
        dv.prefill(p.dm, ds, torch.zeros(6, dtype=torch.int32, device="cuda"))
    assert e.value.code == C.PN_ERANGE
    assert ds.pos == 15


# ---- the wide path (prefill_chunk > 0): each chunk through every projection
# as one matrix product, K split over work-groups, fp32 partial sums added in
# split order

def test_wide_fp32_activations_three_chunks():
    """fp32 activations (three bf16 pieces per value), chunks of 64 rows:
    64 + 64 + 22 prompt tokens from position 0, then decode on the cache."""
    wl = ragged("wide-actf32", w_dtype=synth.BF16, kv_dtype=synth.BF16, act_dtype=synth.F32, seed=84)
    p = Pair(wl, max_batch=1, prefill_chunk=64)
    prompt = list(synth.uniform_int(wl.seed, 95, 150, 0, wl.n_vocab - 1))
    worst, near = run_prefill(p, 0, prompt, 3)
    log("  wide, fp32 activations, 150 tokens in chunks of 64: worst rel L2 %.2e, near %d" % (worst, near))


def test_wide_window_bias_neox_on_existing_cache():
    """bf16 activations, fp32 cache, q/k/v biases, NeoX RoPE and a 40-token
    window narrower than the 48-row chunks, from a cache written up to 200."""
    wl = ragged("wide-bf16-window", w_dtype=synth.BF16, kv_dtype=synth.F32, act_dtype=synth.BF16,
                sliding_window=40, rope_neox=True, qkv_bias=True, seed=85)
    p = Pair(wl, max_batch=2, prefill_chunk=48)
    prompt = list(synth.uniform_int(wl.seed, 96, 100, 0, wl.n_vocab - 1))
    worst, near = run_prefill(p, 200, prompt, 3)
    log("  wide, window 40, bias + NeoX, 100 tokens from 200: worst rel L2 %.2e, near %d" % (worst, near))


def test_wide_outputs_optional_and_pooled():
    """A pooled, windowed state: the prompt in chunks of 32 with only the
    argmax asked for, then with no output (the LM head is skipped), then
    decode steps that read every appended K/V; the pooled twin of a private
    state prefilled the decode-kernel way gives the same decode logits to
    within the wide path's summation order."""
    import numpy as np
    import torch
    from token_decode_amd import device as dv
    wl = ragged("wide-pooled", w_dtype=synth.BF16, kv_dtype=synth.BF16, act_dtype=synth.BF16,
                sliding_window=70, seed=86)
    p = Pair(wl, max_batch=1, prefill_chunk=32)
    pool = dv.DevicePool(p.dm, 6)
    ds = dv.DeviceState(p.dm, 600, pool=pool)
    os_ = p.om.new_state(600)
    prompt = [int(t) for t in synth.uniform_int(wl.seed, 97, 140, 0, wl.n_vocab - 1)]
    from harness import compare_step
    am = torch.empty(90, dtype=torch.int32, device="cuda")
    dv.prefill(p.dm, ds, torch.tensor(prompt[:90], dtype=torch.int32, device="cuda"), None, am)
    got = am.cpu().numpy()
    # a private twin takes the same chunks with the logits asked for: the ids
    # without logits must be its ids bit for bit, and its logits and ids are
    # held to the oracle by the parity rule
    twin = dv.DeviceState(p.dm, 600)
    tl = torch.empty(90, wl.n_vocab, dtype=torch.float32, device="cuda")
    ta = torch.empty(90, dtype=torch.int32, device="cuda")
    dv.prefill(p.dm, twin, torch.tensor(prompt[:90], dtype=torch.int32, device="cuda"), tl, ta)
    np.testing.assert_array_equal(got, ta.cpu().numpy())
    tg = tl.cpu().numpy()
    for t in range(90):
        ol, oa = os_.step(prompt[t])
        compare_step(wl, tg[t], ol, int(got[t]), oa, "row %d:" % t)
    twin.free()
    dv.prefill(p.dm, ds, torch.tensor(prompt[90:], dtype=torch.int32, device="cuda"))
    for t in prompt[90:]:
        ol, oa = os_.step(t)
    assert ds.pos == 140 and pool.free_pages >= 0
    tok = torch.tensor([oa], dtype=torch.int32, device="cuda")
    lg = torch.empty(wl.n_vocab, dtype=torch.float32, device="cuda")
    a1 = torch.empty(1, dtype=torch.int32, device="cuda")
    worst = 0.0
    for i in range(4):
        dv.forward_step(p.dm, ds, tok, lg, a1)
        ol, oa = os_.step(int(tok.item()))
        rel, _ = compare_step(wl, lg.cpu().numpy(), ol, int(a1.item()), oa, "decode step %d:" % i)
        worst = max(worst, rel)
        tok.fill_(oa)
    log("  wide, pooled window 70, argmax-only then no output: decode after worst rel L2 %.2e" % worst)


def test_wide_llama3_shape():
    """Llama-3-8B layer shape (2 layers, full 128256 vocabulary): 40 prompt
    tokens in chunks of 32 (32 + 8 rows) after a 100-token cache."""
    wl = synth.WORKLOADS["llama3-8b-bf16"]().with_(name="wide-llama3-2l", n_layer=2, seed=87)
    p = Pair(wl, max_batch=1, prefill_chunk=32)
    prompt = list(synth.uniform_int(wl.seed, 98, 40, 0, wl.n_vocab - 1))
    worst, near = run_prefill(p, 100, prompt, 1)
    log("  wide, Llama-3-8B shape, 40 tokens from 100: worst rel L2 %.2e, near %d" % (worst, near))


def test_wide_tiled_attention_window():
    """A bf16 cache on the matrix cores with four query heads per KV head: the
    256-row chunk's attention runs four rows per work-group, each of its 16
    columns with its own 40-key window (windows that start mid-tile, pages
    that end mid-tile, 16-key groups that hold none of a column's keys), after
    a cache written up to 120; the 44-row tail runs one row per work-group."""
    wl = ragged("wide-tiled-window", n_head=8, n_kv_head=2, w_dtype=synth.BF16, kv_dtype=synth.BF16,
                act_dtype=synth.F32, sliding_window=40, seed=95)
    p = Pair(wl, max_batch=1, prefill_chunk=256)
    prompt = list(synth.uniform_int(wl.seed, 106, 300, 0, wl.n_vocab - 1))
    worst, near = run_prefill(p, 120, prompt, 2)
    log("  wide, 4 rows per attention work-group, window 40, 300 tokens from 120: worst rel L2 %.2e, near %d"
        % (worst, near))


def test_wide_one_row_then_full_chunk():
    """Chunks of 256 rows: a 1-row prefill (one row tile, clamped loads), then
    300 tokens (a full 256-row chunk over two row groups, then 44 rows)."""
    wl = ragged("wide-256", w_dtype=synth.BF16, kv_dtype=synth.BF16, act_dtype=synth.F32, seed=88)
    p = Pair(wl, max_batch=1, prefill_chunk=256)
    prompt = list(synth.uniform_int(wl.seed, 99, 301, 0, wl.n_vocab - 1))
    import torch
    from token_decode_amd import device as dv
    ds, os_ = p.states(0, 0, 400)
    worst = 0.0
    for part in (prompt[:1], prompt[1:]):
        toks = torch.tensor(part, dtype=torch.int32, device="cuda")
        lg = torch.empty(len(part), wl.n_vocab, dtype=torch.float32, device="cuda")
        am = torch.empty(len(part), dtype=torch.int32, device="cuda")
        dv.prefill(p.dm, ds, toks, lg, am)
        g, ga = lg.cpu().numpy(), am.cpu().numpy()
        for t, tok in enumerate(part):
            ol, oa = os_.step(int(tok))
            from harness import compare_step
            rel, _ = compare_step(wl, g[t], ol, int(ga[t]), oa, "row %d:" % t)
            worst = max(worst, rel)
    assert ds.pos == 301
    log("  wide, 1 row then 256 + 44 rows: worst rel L2 %.2e" % worst)


def test_wide_bad_token_sets_the_flag():
    """An id outside the vocabulary reads row 0 of the embedding and sets the
    state's token flag, as on the decode path; the flag clears on reading."""
    import torch
    from token_decode_amd import device as dv
    wl = ragged("wide-badtok", w_dtype=synth.BF16, kv_dtype=synth.BF16, act_dtype=synth.BF16, seed=89)
    p = Pair(wl, max_batch=1, prefill_chunk=32)
    ds = dv.DeviceState(p.dm, 100)
    toks = torch.tensor([3, 5, wl.n_vocab, 7], dtype=torch.int32, device="cuda")
    am = torch.empty(4, dtype=torch.int32, device="cuda")
    lg = torch.empty(4, wl.n_vocab, dtype=torch.float32, device="cuda")
    dv.prefill(p.dm, ds, toks, lg, am)
    assert ds.check_flags() & 1
    assert ds.check_flags() == 0
    assert ds.pos == 4
    # the same chunk with token 0 in its place gives the same logits bit for bit
    d0 = dv.DeviceState(p.dm, 100)
    lg0 = torch.empty(4, wl.n_vocab, dtype=torch.float32, device="cuda")
    dv.prefill(p.dm, d0, torch.tensor([3, 5, 0, 7], dtype=torch.int32, device="cuda"), lg0, None)
    assert d0.check_flags() == 0
    assert lg.cpu().numpy().tobytes() == lg0.cpu().numpy().tobytes()


def test_wide_int8_weights():
    """INT8 weights (per-row scales, f16 matrix-core steps over the widened
    codes, the scale applied to each output row) with bf16 activations, chunks
    of 64 over 150 tokens from a cache written up to 40."""
    wl = ragged("wide-int8", w_dtype=synth.I8, kv_dtype=synth.BF16, act_dtype=synth.BF16, seed=90)
    p = Pair(wl, max_batch=1, prefill_chunk=64)
    prompt = list(synth.uniform_int(wl.seed, 100, 150, 0, wl.n_vocab - 1))
    worst, near = run_prefill(p, 40, prompt, 2)
    log("  wide, int8 weights, 150 tokens from 40: worst rel L2 %.2e, near %d" % (worst, near))


def test_wide_int8_llama3_shape():
    """Llama-3-8B layer shape with INT8 weights (2 layers, full vocabulary),
    32 prompt tokens in one chunk after a 60-token cache."""
    wl = synth.WORKLOADS["llama3-8b-int8"]().with_(name="wide-llama3-int8-2l", n_layer=2, seed=91)
    p = Pair(wl, max_batch=1, prefill_chunk=32)
    prompt = list(synth.uniform_int(wl.seed, 101, 32, 0, wl.n_vocab - 1))
    worst, near = run_prefill(p, 60, prompt, 1)
    log("  wide, Llama-3-8B int8, 32 tokens from 60: worst rel L2 %.2e, near %d" % (worst, near))


def test_wide_q8_0_weights():
    """Q8_0 weights (an fp16 scale per 32-weight block: each block's matrix-core
    step from zero, scaled and added in fp32) with bf16 activations, chunks of
    64 over 150 tokens from a cache written up to 40; n_embd 224 leaves the
    last 64-wide k tile half past K.  The small products run in work-groups of
    8 weight tiles."""
    wl = ragged("wide-q8_0", w_dtype=synth.Q8_0, kv_dtype=synth.BF16, act_dtype=synth.BF16, n_embd=224,
                n_ff=320, seed=93)
    p = Pair(wl, max_batch=1, prefill_chunk=64)
    prompt = list(synth.uniform_int(wl.seed, 103, 150, 0, wl.n_vocab - 1))
    worst, near = run_prefill(p, 40, prompt, 2)
    log("  wide, Q8_0 weights, 150 tokens from 40: worst rel L2 %.2e, near %d" % (worst, near))


def test_wide_q8_0_llama3_shape():
    """Llama-3-8B layer shape with Q8_0 weights (2 layers, full vocabulary):
    40 prompt tokens in chunks of 32 after a 30-token cache.  At 32 rows the
    planner runs QKV and gate/up in work-groups of 14 weight tiles (QKV's 384
    tiles leave the last group ragged), O and down in groups of 8 and the LM
    head in groups of 16, all but the LM head with K split over work-groups."""
    wl = synth.WORKLOADS["llama3-8b-q8_0"]().with_(name="wide-llama3-q8_0-2l", n_layer=2, seed=94)
    p = Pair(wl, max_batch=1, prefill_chunk=32)
    prompt = list(synth.uniform_int(wl.seed, 104, 40, 0, wl.n_vocab - 1))
    worst, near = run_prefill(p, 30, prompt, 1)
    log("  wide, Llama-3-8B Q8_0, 40 tokens from 30: worst rel L2 %.2e, near %d" % (worst, near))


def test_wide_q4_0_weights():
    """Q4_0 weights (4-bit codes in 128-wide tiles, four 32-weight blocks each:
    every block's matrix-core step from zero, scaled and added in fp32) with
    bf16 activations, chunks of 64 over 150 tokens from a cache written up to
    40; n_embd 224 and n_ff 320 leave the last 128-wide k tile partly past K."""
    wl = ragged("wide-q4_0", w_dtype=synth.Q4_0, kv_dtype=synth.BF16, act_dtype=synth.BF16, n_embd=224,
                n_ff=320, seed=96)
    p = Pair(wl, max_batch=1, prefill_chunk=64)
    prompt = list(synth.uniform_int(wl.seed, 107, 150, 0, wl.n_vocab - 1))
    worst, near = run_prefill(p, 40, prompt, 2)
    log("  wide, Q4_0 weights, 150 tokens from 40: worst rel L2 %.2e, near %d" % (worst, near))


def test_wide_q4_0_llama3_shape():
    """Llama-3-8B layer shape with Q4_0 weights (2 layers, full vocabulary): a
    256-row chunk (14-tile groups for gate/up, the tiled attention) and a
    44-row tail after a 30-token cache."""
    wl = synth.WORKLOADS["llama3-8b-q4_0"]().with_(name="wide-llama3-q4_0-2l", n_layer=2, seed=97)
    p = Pair(wl, max_batch=1, prefill_chunk=256)
    prompt = list(synth.uniform_int(wl.seed, 108, 300, 0, wl.n_vocab - 1))
    worst, near = run_prefill(p, 30, prompt, 1)
    log("  wide, Llama-3-8B Q4_0, 300 tokens from 30: worst rel L2 %.2e, near %d" % (worst, near))


def test_wide_mistral_shape_full_chunk():
    """Mistral-7B layer shape (2 layers, bf16 activations, window 4096): a full
    256-row chunk, then 44 rows.  At 256 rows the planner runs QKV (ragged
    last group) and gate/up in work-groups of 14 weight tiles, O in groups of
    8 and down and the LM head in groups of 16; the 44-row tail takes narrower
    groups with more K splits."""
    wl = synth.mistral_7b_slots().with_(name="wide-mistral-2l", n_layer=2, slots=1, seed=92)
    p = Pair(wl, max_batch=1, prefill_chunk=256)
    prompt = list(synth.uniform_int(wl.seed, 102, 300, 0, wl.n_vocab - 1))
    worst, near = run_prefill(p, 0, prompt, 1)
    log("  wide, Mistral-7B shape, 300 tokens in chunks of 256: worst rel L2 %.2e, near %d" % (worst, near))


ROUTE_TOL = 1e-2  # router k-th / (k+1)-th gaps below this admit the swapped branch


def run_prefill_moe(p, start, prompt, n_decode):
    """run_prefill for an MoE model: every row is checked by the routing-branch
    rule (a routing near tie may take the other expert; the oracle runs both
    branches and the row must match one), and the oracle continues in the
    branch the GPU took."""
    import torch
    from harness import moe_step_branches
    from token_decode_amd import device as dv
    wl = p.wl
    ds, os_ = p.states(0, start, start + len(prompt) + n_decode + 1)
    toks = torch.tensor([int(t) for t in prompt], dtype=torch.int32, device="cuda")
    logits = torch.empty(len(prompt), wl.n_vocab, dtype=torch.float32, device="cuda")
    am = torch.empty(len(prompt), dtype=torch.int32, device="cuda")
    dv.prefill(p.dm, ds, toks, logits, am)
    assert ds.pos == start + len(prompt)
    g, ga = logits.cpu().numpy(), am.cpu().numpy()
    worst, near, swaps, nxt = 0.0, 0, 0, None
    th = oracle_threads()
    for t, tok in enumerate(prompt):
        rel, nt, mask, oa = moe_step_branches(wl, os_, int(tok), g[t], int(ga[t]), ROUTE_TOL, th)
        worst, near, swaps, nxt = max(worst, rel), near + int(nt), swaps + int(mask != 0), oa
    tok = torch.tensor([nxt], dtype=torch.int32, device="cuda")
    lg1 = torch.empty(wl.n_vocab, dtype=torch.float32, device="cuda")
    a1 = torch.empty(1, dtype=torch.int32, device="cuda")
    for i in range(n_decode):
        dv.forward_step(p.dm, ds, tok, lg1, a1)
        rel, nt, mask, oa = moe_step_branches(wl, os_, int(tok.item()), lg1.cpu().numpy(), int(a1.item()),
                                              ROUTE_TOL, th)
        worst, near, swaps = max(worst, rel), near + int(nt), swaps + int(mask != 0)
        tok.fill_(oa)
    return worst, near, swaps


@pytest.mark.parametrize("dt", [synth.BF16, synth.I8], ids=["bf16", "int8"])
def test_wide_moe_weights(dt):
    """Experts on the wide path: 4 experts, top-2, a ragged model (n_embd 200,
    n_ff 300) after a 5-token cache, 70 tokens in chunks of 32 (32 + 32 + 6):
    every row routed, packed by expert, each expert's gate/up and down over its
    rows, the weighted sum; every row against the oracle, then decode steps."""
    wl = ragged("wide-moe-%d" % dt, n_expert=4, n_expert_used=2, w_dtype=dt, kv_dtype=synth.BF16,
                act_dtype=synth.BF16, seed=110 + dt)
    p = Pair(wl, max_batch=1, prefill_chunk=32)
    prompt = list(synth.uniform_int(wl.seed, 111, 70, 0, wl.n_vocab - 1))
    worst, near, swaps = run_prefill_moe(p, 5, prompt, 2)
    log("  wide MoE (%d), 70 tokens from 5: worst rel L2 %.2e, near %d, routing swaps %d" % (dt, worst, near, swaps))


def test_wide_moe_every_row_to_every_expert():
    """2 experts, top-2: every row goes to both, so each expert takes all 256
    rows of a full chunk (two 128-row groups of the grouped product), then a
    44-row tail; top-1 of 3 experts after it (weights of exactly 1)."""
    for ne, nu, seed in ((2, 2, 120), (3, 1, 121)):
        wl = ragged("wide-moe-e%d-k%d" % (ne, nu), n_expert=ne, n_expert_used=nu, w_dtype=synth.BF16,
                    kv_dtype=synth.BF16, act_dtype=synth.F32, seed=seed)
        p = Pair(wl, max_batch=1, prefill_chunk=256)
        prompt = list(synth.uniform_int(wl.seed, 122, 300, 0, wl.n_vocab - 1))
        worst, near, swaps = run_prefill_moe(p, 0, prompt, 1)
        log("  wide MoE %d experts top-%d, 300 tokens: worst rel L2 %.2e, near %d, swaps %d"
            % (ne, nu, worst, near, swaps))


def test_wide_moe_mixtral_shape():
    """Mixtral-8x7B layer shape (2 layers, 8 experts of n_ff 14336, top-2,
    bf16): 80 tokens in chunks of 64 after a 10-token cache."""
    wl = synth.mixtral_8x7b_slots().with_(name="wide-mixtral-2l", n_layer=2, slots=1, seed=123)
    p = Pair(wl, max_batch=1, prefill_chunk=64)
    prompt = list(synth.uniform_int(wl.seed, 124, 80, 0, wl.n_vocab - 1))
    worst, near, swaps = run_prefill_moe(p, 10, prompt, 1)
    log("  wide, Mixtral-8x7B shape, 80 tokens from 10: worst rel L2 %.2e, near %d, swaps %d"
        % (worst, near, swaps))
