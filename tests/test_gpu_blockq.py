"""GPU parity of block-quantised weights (per row, blocks of 32 weights with
one fp16 scale: Q8_0 with int8 codes, Q4_0 with 4-bit codes) against the
oracle, which dequantises each weight (d * q, d * (code - 8)) in fp64 before
the product.

The GPU widens the codes to f16 exactly, runs one matrix-core step per block
and adds d times that block's partial sum in fp32, so only fp32 summation
order separates it from the oracle; the shapes make K a whole number of
32-wide blocks but not of the 64-wide tiles (half-empty last tiles), with
several tiles, ragged row counts and several attention splits.  Every case
runs for both formats."""
import pytest

import synth

from harness import Pair, log, run_batch, run_single

pytestmark = pytest.mark.gpu


FORMATS = [synth.Q8_0, synth.Q4_0]
FMT_IDS = ["q8_0", "q4_0"]


def q8(name, dt=synth.Q8_0, **kw):
    base = dict(n_layer=2, n_embd=224, n_head=6, n_kv_head=2, head_dim=32, n_ff=288, n_vocab=1000,
                rope_theta=10000.0, w_dtype=dt, kv_dtype=synth.BF16, act_dtype=synth.BF16, seed=71)
    base.update(kw)
    return synth.Workload("%s-%s" % (name, FMT_IDS[FORMATS.index(dt)]), **base)


fmt = pytest.mark.parametrize("dt", FORMATS, ids=FMT_IDS)


@fmt
def test_blockq_from_position_zero(dt):
    wl = q8("from-zero", dt, seed=72, prompt_len=4)
    p = Pair(wl)
    worst, near, n = run_single(p, 0, wl.prompt_tokens(), 24)
    log("  %s from position 0: %d steps, worst rel L2 %.2e, near %d" % (wl.name, n, worst, near))


SINGLE = [
    q8(name, dt, **kw) for dt in FORMATS for name, kw in (
        ("ragged", {}),
        ("fp32-cache-d128", dict(n_head=4, n_kv_head=2, head_dim=128, kv_dtype=synth.F32, seed=73, n_ff=352)),
        ("neox-bias-window", dict(rope_neox=True, qkv_bias=True, sliding_window=300, seed=74)),
        ("d64-g8", dict(n_head=8, n_kv_head=1, head_dim=64, seed=75, n_embd=256, n_ff=704)),
    )
]


@pytest.mark.parametrize("wl", SINGLE, ids=lambda w: w.name)
def test_blockq_single_on_prefilled_cache(wl):
    p = Pair(wl)
    toks = synth.uniform_int(wl.seed, 1 << 20, 2, 0, wl.n_vocab - 1)
    worst, near, n = run_single(p, 700, toks, 4)
    log("  %s: worst rel L2 %.2e near %d" % (wl.name, worst, near))


@fmt
def test_blockq_batched_window(dt):
    wl = q8("batch-window", dt, sliding_window=200, seed=76)
    p = Pair(wl, max_batch=5)
    worst, near = run_batch(p, [3, 64, 129, 450, 1000], 3)
    log("  %s, 5 slots: worst rel L2 %.2e near %d" % (wl.name, worst, near))


@fmt
def test_blockq_batched_16_slots(dt):
    wl = q8("batch16", dt, seed=77)
    p = Pair(wl, max_batch=16)
    worst, near = run_batch(p, [int(x) for x in synth.uniform_int(wl.seed, 5, 16, 0, 600)], 2)
    log("  %s, 16 slots: worst rel L2 %.2e near %d" % (wl.name, worst, near))


@fmt
def test_blockq_moe_batched(dt):
    wl = q8("moe", dt, n_expert=4, n_expert_used=2, n_ff=96, seed=78)
    p = Pair(wl, max_batch=6)
    worst, near = run_batch(p, [5, 70, 200, 260, 511, 9], 3)
    log("  %s: worst rel L2 %.2e near %d" % (wl.name, worst, near))


@fmt
def test_blockq_prefill(dt):
    import torch
    from token_decode_amd import device as dv
    from harness import compare_step
    wl = q8("prefill", dt, seed=79)
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
    log("  %s: 21 tokens in chunks of 8: worst rel L2 %.2e" % (wl.name, worst))
