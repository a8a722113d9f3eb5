"""GPU parity: the HIP path against the fp64 oracle on the same seeded inputs.

Every case runs the GPU on the oracle's greedy trajectory (the GPU is fed the
oracle's tokens) and compares every step's logits (relative L2 within 1e-4 for
fp32 models, 2e-2 for bf16 / int8) and greedy ids (equal, or a near tie that
the oracle's top-two gap cannot resolve).  Shapes are chosen to span several
tiles with ragged tails: dimensions that are not multiples of the tile widths,
several attention splits and partial KV pages.
"""
import pytest

import synth

from harness import Pair, log, run_batch, run_single

pytestmark = pytest.mark.gpu


def ragged(name, **kw):
    base = dict(n_layer=2, n_embd=200, n_head=6, n_kv_head=2, head_dim=32, n_ff=300, n_vocab=1000,
                rope_theta=10000.0, seed=31)
    base.update(kw)
    return synth.Workload(name, **base)


def test_tiny_fp32_full_run():
    """The tiny fp32 model: a 4-token prompt then 128 greedy steps (positions 0..131)."""
    wl = synth.tiny_fp32()
    p = Pair(wl)
    worst, near, n = run_single(p, 0, wl.prompt_tokens(), wl.steps)
    log("  tiny-fp32: %d steps, worst rel L2 %.2e, near ties %d" % (n, worst, near))
    assert near == 0


CASES = [
    ragged("ragged-f32", w_dtype=synth.F32, kv_dtype=synth.F32, act_dtype=synth.F32),
    ragged("ragged-bf16-actf32-window", w_dtype=synth.BF16, kv_dtype=synth.BF16,
           act_dtype=synth.F32, sliding_window=300, seed=32),
    ragged("ragged-bf16-d64-g8", n_head=8, n_kv_head=1, head_dim=64, w_dtype=synth.BF16,
           kv_dtype=synth.BF16, act_dtype=synth.BF16, seed=33),
    ragged("ragged-int8-d128", n_head=4, n_kv_head=2, head_dim=128, w_dtype=synth.I8,
           kv_dtype=synth.BF16, act_dtype=synth.BF16, seed=34, n_ff=520),
    ragged("ragged-f32-kvbf16-mha", n_head=4, n_kv_head=4, w_dtype=synth.F32, kv_dtype=synth.BF16,
           act_dtype=synth.BF16, seed=35),
]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_ragged_single(wl):
    """Batch 1 with 700 cached positions (several attention splits), then 6 steps."""
    p = Pair(wl)
    toks = synth.uniform_int(wl.seed, 1 << 20, 2, 0, wl.n_vocab - 1)
    worst, near, n = run_single(p, 700, toks, 4)
    log("  %s: worst rel L2 %.2e near %d" % (wl.name, worst, near))


def test_tiny_from_position_zero_bf16():
    wl = synth.tiny_fp32().with_(name="tiny-bf16", w_dtype=synth.BF16, kv_dtype=synth.BF16,
                                 act_dtype=synth.BF16, seed=41)
    p = Pair(wl)
    worst, near, n = run_single(p, 0, wl.prompt_tokens(), 20)
    log("  tiny-bf16: worst rel L2 %.2e near %d" % (worst, near))


def test_batched_slots_window():
    """Five slots at different positions (one inside the first page) with a window."""
    wl = ragged("batch-bf16-window", w_dtype=synth.BF16, kv_dtype=synth.BF16, act_dtype=synth.BF16,
                sliding_window=200, seed=42)
    p = Pair(wl, max_batch=5)
    worst, near = run_batch(p, [3, 64, 129, 450, 1000], 3)
    log("  batch: worst rel L2 %.2e near %d" % (worst, near))


def test_batched_fp32_activations():
    wl = ragged("batch-bf16-actf32", w_dtype=synth.BF16, kv_dtype=synth.BF16, act_dtype=synth.F32,
                seed=43)
    p = Pair(wl, max_batch=5)
    worst, near = run_batch(p, [0, 17, 300, 301, 999], 3)
    log("  batch f32 act: worst rel L2 %.2e near %d" % (worst, near))


def test_moe_small_batched():
    wl = ragged("moe-small", n_expert=6, n_expert_used=2, w_dtype=synth.BF16, kv_dtype=synth.BF16,
                act_dtype=synth.BF16, seed=44, n_ff=160)
    p = Pair(wl, max_batch=7)
    worst, near = run_batch(p, [5, 70, 200, 260, 511, 600, 10], 3)
    log("  moe: worst rel L2 %.2e near %d" % (worst, near))


def test_moe_many_experts():
    """Twelve experts, top-3: the router's waves take experts w, w + 4 and w + 8
    (the last pass loads its weights inside the loop), and routing picks three."""
    wl = ragged("moe-e12", n_expert=12, n_expert_used=3, w_dtype=synth.BF16, kv_dtype=synth.BF16,
                act_dtype=synth.BF16, seed=46, n_ff=96)
    p = Pair(wl, max_batch=4)
    worst, near = run_batch(p, [3, 90, 257, 400], 3)
    log("  moe 12 experts: worst rel L2 %.2e near %d" % (worst, near))


def test_moe_single_fp32():
    wl = ragged("moe-f32", n_expert=4, n_expert_used=2, w_dtype=synth.F32, kv_dtype=synth.F32,
                act_dtype=synth.F32, seed=45, n_ff=96)
    p = Pair(wl)
    worst, near, n = run_single(p, 100, [7, 8], 6)
    log("  moe f32: worst rel L2 %.2e near %d" % (worst, near))


@pytest.mark.parametrize("kps", [64, 192, 320, 1024])
def test_attention_split_sizes(kps):
    """Keys per attention split (one chunk, several chunks, the whole 1001-key
    window in one split) change the result only by fp32 rounding: every split
    size matches the oracle, with fp32 (at 1e-4) and bf16 caches."""
    from token_decode_amd import _capi as C
    for kv in (synth.F32, synth.BF16):
        wl = ragged("split-%d-kv%d" % (kps, kv), w_dtype=synth.F32, kv_dtype=kv,
                    act_dtype=synth.F32, seed=46)
        p = Pair(wl)
        p.dm.set_option(C.PN_OPT_ATTN_KEYS_PER_SPLIT, kps)
        worst, near, n = run_single(p, 999, [11, 12], 2)
        log("  kps %d kv %d: worst rel L2 %.2e near %d" % (kps, kv, worst, near))


@pytest.mark.parametrize("start", [40, 200, 700, 2100])
def test_split_combine_in_o_prologue(start):
    """Batch 1 over a bf16 cache with at most 4 query heads per KV head takes
    at most 8 attention splits (8-wave work-groups) and combines them in the O
    projection's prologue: from one page (one split, whose output the prologue
    reads as is) to 34 pages (8 splits of 4 or 5 pages), with head_dim 128 and
    fp32 activations, head_dim 64 and bf16 activations; then with 64 keys per
    split the 700- and 2100-key windows need more than 8 splits and go through
    the merge launch instead, and with the combine switched off the 8-wave
    attention work-groups feed the merge launch.  Every step against the
    oracle."""
    from token_decode_amd import _capi as C
    for kps, combine, waves in ((0, 0, 0), (64, 0, 0), (0, 1, 8)):
        if (kps or combine) and start < 700:
            continue
        for i, (H, Hk, d, act) in enumerate(((8, 2, 128, synth.F32), (6, 3, 64, synth.BF16))):
            wl = ragged("combine-%d-%d-kps%d-c%d" % (start, d, kps, combine), n_head=H, n_kv_head=Hk,
                        head_dim=d, w_dtype=synth.BF16, kv_dtype=synth.BF16, act_dtype=act, seed=60 + i)
            p = Pair(wl)
            p.dm.set_option(C.PN_OPT_ATTN_KEYS_PER_SPLIT, kps)
            p.dm.set_option(C.PN_OPT_ATTN_COMBINE, combine)
            p.dm.set_option(C.PN_OPT_ATTN_WAVES, waves)
            worst, near, n = run_single(p, start, [5, 6], 2, max_ctx=start + 8)
            log("  %s: worst rel L2 %.2e near %d" % (wl.name, worst, near))


@pytest.mark.parametrize("kind", [1, 2], ids=["vector", "matrix"])
@pytest.mark.parametrize("kps", [0, 64, 256])
def test_attention_kernels_bf16_cache(kind, kps):
    """Both attention kernels over a bf16 cache (vector units, matrix cores),
    automatic and fixed split sizes: batch 1 with a window and head_dim 64 /
    128, and five batched slots, against the oracle."""
    from token_decode_amd import _capi as C
    wl = ragged("attn-kind%d-kps%d" % (kind, kps), n_head=8, n_kv_head=2, head_dim=64, w_dtype=synth.BF16,
                kv_dtype=synth.BF16, act_dtype=synth.F32, sliding_window=333, seed=47)
    p = Pair(wl)
    p.dm.set_option(C.PN_OPT_ATTN_KERNEL, kind)
    p.dm.set_option(C.PN_OPT_ATTN_KEYS_PER_SPLIT, kps)
    worst, near, n = run_single(p, 700, [21, 22], 2)
    log("  kind %d kps %d d64 window: worst rel L2 %.2e near %d" % (kind, kps, worst, near))
    wl = ragged("attn-kind%d-kps%d-b" % (kind, kps), n_head=4, n_kv_head=2, head_dim=128, w_dtype=synth.BF16,
                kv_dtype=synth.BF16, act_dtype=synth.BF16, seed=49)
    p = Pair(wl, max_batch=5)
    p.dm.set_option(C.PN_OPT_ATTN_KERNEL, kind)
    p.dm.set_option(C.PN_OPT_ATTN_KEYS_PER_SPLIT, kps)
    worst, near = run_batch(p, [0, 15, 63, 64, 900], 2)
    log("  kind %d kps %d d128 batch: worst rel L2 %.2e near %d" % (kind, kps, worst, near))


@pytest.mark.parametrize("heads", [(6, 2, 32), (6, 1, 64), (3, 1, 128)], ids=["g3-d32", "g6-d64", "g3-d128"])
def test_attention_group_sizes(heads):
    """Query heads per KV head of 3 and 6 (the matrix-core tile's unused
    columns) and head_dim 32, over a bf16 cache with a window, batch 1 and
    three batched slots."""
    H, Hk, d = heads
    wl = ragged("attn-g%d-d%d" % (H // Hk, d), n_head=H, n_kv_head=Hk, head_dim=d, w_dtype=synth.BF16,
                kv_dtype=synth.BF16, act_dtype=synth.F32, sliding_window=250, seed=50 + H + d)
    p = Pair(wl, max_batch=3)
    worst, near, n = run_single(p, 600, [31, 32], 2)
    log("  %s single: worst rel L2 %.2e near %d" % (wl.name, worst, near))
    worst, near = run_batch(p, [1, 249, 777], 2)
    log("  %s batch: worst rel L2 %.2e near %d" % (wl.name, worst, near))


def test_batched_16_slots_large_lds():
    """16 slots with n_embd 2048: several GEMM variants stage more than 64 KiB of
    A in LDS in the same step (each needs its own launch attribute)."""
    wl = ragged("batch16-e2048", n_embd=2048, n_head=16, n_kv_head=4, head_dim=128, n_ff=600,
                w_dtype=synth.BF16, kv_dtype=synth.BF16, act_dtype=synth.BF16, seed=48)
    p = Pair(wl, max_batch=16)
    starts = [int(s) for s in synth.uniform_int(48, 99, 16, 0, 400)]
    worst, near = run_batch(p, starts, 2)
    log("  batch 16: worst rel L2 %.2e near %d" % (worst, near))
