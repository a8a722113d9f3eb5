"""GPU parity of the Q4 KV cache (each cached k and v head vector as 32-dim
blocks of an fp16 scale and 4-bit codes) against the oracle, which quantises
every appended vector by the same rule with its decisions on fp32 values.

The GPU's fp32 k and v differ from the oracle's fp64 ones by rounding, so a
code can land on the other side of a rounding boundary now and then, moving one
cached value by a quantisation step; the logits are held to the 2e-2 bound of
the low-precision workloads.  Cases cover the three head sizes (one lane's
quarter of a key is a whole block, half a block or a quarter), a window,
batched slots, MoE, chunked prefill, the fp32 rows of set_kv, and a shared page
pool (whose pages are 9/32 of a bf16 page)."""
import numpy as np
import pytest

import synth

from harness import Pair, compare_step, log, run_batch, run_single

pytestmark = pytest.mark.gpu


def q4kv(name, **kw):
    base = dict(n_layer=2, n_embd=200, n_head=6, n_kv_head=2, head_dim=32, n_ff=300, n_vocab=1000,
                rope_theta=10000.0, w_dtype=synth.BF16, kv_dtype=synth.Q4_0, act_dtype=synth.BF16, seed=101)
    base.update(kw)
    return synth.Workload(name, **base)


def test_q4kv_tiny_from_zero():
    wl = synth.tiny_fp32().with_(name="tiny-q4kv", kv_dtype=synth.Q4_0, seed=102)
    p = Pair(wl)
    worst, near, n = run_single(p, 0, wl.prompt_tokens(), 40)
    log("  fp32 weights, Q4 cache from position 0: %d steps, worst rel L2 %.2e, near %d" % (n, worst, near))


CASES = [
    q4kv("q4kv-d32"),
    q4kv("q4kv-d64-g8-window", n_head=8, n_kv_head=1, head_dim=64, sliding_window=300, seed=103),
    q4kv("q4kv-d128-actf32", n_head=4, n_kv_head=2, head_dim=128, act_dtype=synth.F32, seed=104, n_ff=520),
    q4kv("q4kv-int8-d128", n_head=4, n_kv_head=2, head_dim=128, w_dtype=synth.I8, seed=105, n_ff=520),
]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_q4kv_single_on_prefilled_cache(wl):
    """700 positions written with set_kv (fp32 rows, quantised on the device), then 6 steps."""
    p = Pair(wl)
    toks = synth.uniform_int(wl.seed, 1 << 20, 2, 0, wl.n_vocab - 1)
    worst, near, n = run_single(p, 700, toks, 4)
    log("  %s: worst rel L2 %.2e near %d" % (wl.name, worst, near))


def test_q4kv_batched_window():
    wl = q4kv("q4kv-batch", sliding_window=200, seed=106, head_dim=64, n_head=4, n_kv_head=2)
    p = Pair(wl, max_batch=5)
    worst, near = run_batch(p, [3, 64, 129, 450, 1000], 3)
    log("  Q4 cache, 5 slots: worst rel L2 %.2e near %d" % (worst, near))


def test_q4kv_moe_batched():
    wl = q4kv("q4kv-moe", n_expert=4, n_expert_used=2, n_ff=128, seed=107)
    p = Pair(wl, max_batch=4)
    worst, near = run_batch(p, [5, 70, 200, 511], 3)
    log("  Q4 cache MoE: worst rel L2 %.2e near %d" % (worst, near))


def test_q4kv_prefill():
    import torch
    from token_decode_amd import device as dv
    wl = q4kv("q4kv-prefill", seed=108, head_dim=128, n_head=4, n_kv_head=2)
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
    log("  Q4 cache prefill, 21 tokens in chunks of 8: worst rel L2 %.2e" % worst)


def test_q4kv_pool_matches_private():
    """Pooled Q4-cache states run the same kernels as private ones: equal bit for bit."""
    import torch
    from token_decode_amd import device as dv
    wl = q4kv("q4kv-pool", sliding_window=100, seed=109)
    p = Pair(wl, max_batch=3)
    pool = dv.DevicePool(p.dm, 12)
    pooled = [dv.DeviceState(p.dm, 1000, pool=pool) for _ in range(3)]
    private = [dv.DeviceState(p.dm, 1000) for _ in range(3)]
    rng = np.random.default_rng(7)
    for t in range(150):
        toks = torch.tensor([int(x) for x in rng.integers(0, wl.n_vocab, 3)], dtype=torch.int32, device="cuda")
        outs = []
        for side in (pooled, private):
            lg = torch.empty(3, wl.n_vocab, dtype=torch.float32, device="cuda")
            dv.forward_batch(p.dm, side, toks, lg)
            outs.append(lg.cpu().numpy())
        np.testing.assert_array_equal(outs[0], outs[1])
    assert pool.free_pages >= 12 - 3 * (100 // 64 + 2)
    log("  Q4 cache, 3 pooled states x 150 steps: equal to private bit for bit")
