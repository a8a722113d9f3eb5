"""GPU parity of Q8_0 block-quantised weights (per row, blocks of 32 weights
with one fp16 scale and int8 codes) against the oracle, which dequantises each
weight as d * q in fp64 before the product.

The GPU widens the codes to f16 exactly, runs one matrix-core step per block
and adds d times that block's partial sum in fp32, so only fp32 summation
order separates it from the oracle; the shapes make K a whole number of
32-wide blocks but not of the 64-wide tiles (half-empty last tiles), with
several tiles, ragged row counts and several attention splits."""
import pytest

import synth

from harness import Pair, log, run_batch, run_single

pytestmark = pytest.mark.gpu


def q8(name, **kw):
    base = dict(n_layer=2, n_embd=224, n_head=6, n_kv_head=2, head_dim=32, n_ff=288, n_vocab=1000,
                rope_theta=10000.0, w_dtype=synth.Q8_0, kv_dtype=synth.BF16, act_dtype=synth.BF16, seed=71)
    base.update(kw)
    return synth.Workload(name, **base)


def test_q8_from_position_zero():
    wl = q8("q8-from-zero", seed=72, prompt_len=4)
    p = Pair(wl)
    worst, near, n = run_single(p, 0, wl.prompt_tokens(), 24)
    log("  Q8_0 from position 0: %d steps, worst rel L2 %.2e, near %d" % (n, worst, near))


SINGLE = [
    q8("q8-ragged"),
    q8("q8-fp32-cache-d128", n_head=4, n_kv_head=2, head_dim=128, kv_dtype=synth.F32, seed=73, n_ff=352),
    q8("q8-neox-bias-window", rope_neox=True, qkv_bias=True, sliding_window=300, seed=74),
    q8("q8-d64-g8", n_head=8, n_kv_head=1, head_dim=64, seed=75, n_embd=256, n_ff=704),
]


@pytest.mark.parametrize("wl", SINGLE, ids=lambda w: w.name)
def test_q8_single_on_prefilled_cache(wl):
    p = Pair(wl)
    toks = synth.uniform_int(wl.seed, 1 << 20, 2, 0, wl.n_vocab - 1)
    worst, near, n = run_single(p, 700, toks, 4)
    log("  %s: worst rel L2 %.2e near %d" % (wl.name, worst, near))


def test_q8_batched_window():
    wl = q8("q8-batch-window", sliding_window=200, seed=76)
    p = Pair(wl, max_batch=5)
    worst, near = run_batch(p, [3, 64, 129, 450, 1000], 3)
    log("  Q8_0, 5 slots: worst rel L2 %.2e near %d" % (worst, near))


def test_q8_batched_16_slots():
    wl = q8("q8-batch16", seed=77)
    p = Pair(wl, max_batch=16)
    worst, near = run_batch(p, [int(x) for x in synth.uniform_int(wl.seed, 5, 16, 0, 600)], 2)
    log("  Q8_0, 16 slots: worst rel L2 %.2e near %d" % (worst, near))


def test_q8_moe_batched():
    wl = q8("q8-moe", n_expert=4, n_expert_used=2, n_ff=96, seed=78)
    p = Pair(wl, max_batch=6)
    worst, near = run_batch(p, [5, 70, 200, 260, 511, 9], 3)
    log("  Q8_0 MoE: worst rel L2 %.2e near %d" % (worst, near))


def test_q8_prefill():
    import torch
    from token_decode_amd import device as dv
    from harness import compare_step
    wl = q8("q8-prefill", seed=79)
    p = Pair(wl, max_batch=8)
    ds, os_ = p.states(0, 40, 200)
    prompt = [int(t) for t in synth.uniform_int(wl.seed, 96, 21, 0, wl.n_vocab - 1)]
    logits = torch.empty(len(prompt), wl.n_vocab, dtype=torch.float32, device="cuda")
    am = torch.empty(len(prompt), dtype=torch.int32, device="cuda")
    dv.prefill(p.dm, ds, torch.tensor(prompt, dtype=torch.int32, device="cuda"), logits, am)
    g, ga = logits.cpu().numpy(), am.cpu().numpy()
    worst = 0.0
    for t, tok in enumerate(prompt):
        ol, oa = os_.step(tok)
        rel, _ = compare_step(wl, g[t], ol, int(ga[t]), oa, "prompt row %d:" % t)
        worst = max(worst, rel)
    log("  Q8_0 prefill of 21 tokens in chunks of 8: worst rel L2 %.2e" % worst)
