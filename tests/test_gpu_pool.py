"""Shared page pool (pooled states): continuous batching with sequences that
join and leave, sliding-window page recycling, prefill and set_kv into pooled
states, pool exhaustion and the state lifecycle.

A pooled state computes what a private state computes: both run the same
kernels on the same values, only the page table differs, so every test drives
a private twin through the same calls in the same batches and requires the
logits to be equal bit for bit (the private path itself is held to the oracle
by the parity tests); one test also holds a pooled trajectory to the oracle."""
import numpy as np
import pytest

import synth

from harness import Pair, compare_step, log

pytestmark = pytest.mark.gpu

PAGE = 64


def wl_window(window=100, **kw):
    base = dict(n_layer=2, n_embd=200, n_head=6, n_kv_head=2, head_dim=32, n_ff=300, n_vocab=1000,
                rope_theta=10000.0, w_dtype=synth.BF16, kv_dtype=synth.BF16, act_dtype=synth.BF16,
                sliding_window=window, seed=91)
    base.update(kw)
    return synth.Workload("pool-window%d" % window, **base)


class Twins:
    """Pooled states and private twins of one model, stepped in the same batches."""

    def __init__(self, pair, n_pages, max_ctx):
        from token_decode_amd import device as dv
        self.p = pair
        self.pool = dv.DevicePool(pair.dm, n_pages)
        self.max_ctx = max_ctx
        self.pooled, self.private = {}, {}

    def join(self, key, pos=0):
        from token_decode_amd import device as dv
        self.pooled[key] = dv.DeviceState(self.p.dm, self.max_ctx, pool=self.pool)
        self.private[key] = dv.DeviceState(self.p.dm, self.max_ctx)
        if pos:
            self.pooled[key].pos = pos
            self.private[key].pos = pos

    def leave(self, key):
        self.pooled.pop(key).free()
        self.private.pop(key).free()

    def step(self, keys, toks):
        """One batched step of `keys` on both sides; returns the pooled logits."""
        import torch
        from token_decode_amd import device as dv
        n, V = len(keys), self.p.wl.n_vocab
        tok = torch.tensor(toks, dtype=torch.int32, device="cuda")
        out = []
        for side in (self.pooled, self.private):
            lg = torch.empty(n, V, dtype=torch.float32, device="cuda")
            am = torch.empty(n, dtype=torch.int32, device="cuda")
            dv.forward_batch(self.p.dm, [side[k] for k in keys], tok, lg, am)
            out.append((lg.cpu().numpy(), am.cpu().numpy()))
        (a, ia), (b, ib) = out
        np.testing.assert_array_equal(a, b)
        np.testing.assert_array_equal(ia, ib)
        for k in keys:
            assert self.pooled[k].pos == self.private[k].pos
        return a, ia


def test_continuous_batching_with_window_recycling():
    """Six sequences over 260 steps: they join and leave between steps (up to
    four at once, in changing order), each windowed state holds at most
    window/64 + 2 pages, and a sequence that joins later reuses pages that
    others gave back (zeroed on the way)."""
    wl = wl_window(100)
    p = Pair(wl, max_batch=4)
    tw = Twins(p, n_pages=4 * 4, max_ctx=2000)
    rng = np.random.default_rng(3)
    sched = {0: (0, 260), 1: (0, 120), 2: (10, 260), 3: (60, 200), 4: (125, 260), 5: (205, 260)}
    live = []
    for t in range(260):
        for k, (a, b) in sched.items():
            if t == a:
                tw.join(k)
                live.append(k)
            if t == b and k in live:
                tw.leave(k)
                live.remove(k)
        keys = [int(k) for k in rng.permutation(live)]
        toks = [int(x) for x in rng.integers(0, wl.n_vocab, len(keys))]
        tw.step(keys, toks)
        held = 16 - tw.pool.free_pages
        assert held <= len(live) * (100 // PAGE + 2), (t, held, len(live))
    for k in list(live):
        tw.leave(k)
    assert tw.pool.free_pages == 16
    log("  6 sequences, 260 steps, 16-page pool: pooled == private bit for bit")


def test_pooled_trajectory_matches_oracle():
    """One pooled sequence against the oracle over 200 positions with a
    70-position window (pages recycled as it goes)."""
    import torch
    from token_decode_amd import device as dv
    wl = wl_window(70, seed=92)
    p = Pair(wl, max_batch=1)
    pool = dv.DevicePool(p.dm, 3)
    ds = dv.DeviceState(p.dm, 400, pool=pool)
    os_ = p.om.new_state(400)
    toks = synth.uniform_int(wl.seed, 95, 200, 0, wl.n_vocab - 1)
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    lg = torch.empty(wl.n_vocab, dtype=torch.float32, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    worst = 0.0
    for i, t in enumerate(toks):
        tok.fill_(int(t))
        dv.forward_step(p.dm, ds, tok, lg, am)
        ol, oa = os_.step(int(t))
        rel, _ = compare_step(wl, lg.cpu().numpy(), ol, int(am.item()), oa, "step %d:" % i)
        worst = max(worst, rel)
    assert pool.free_pages >= 0
    log("  pooled, window 70, 200 steps on a 3-page pool: worst rel L2 %.2e" % worst)


def test_exhaustion_leaves_states_unchanged():
    wl = wl_window(0, seed=93)  # no window: pages are only freed by reset / free
    p = Pair(wl, max_batch=2)
    tw = Twins(p, n_pages=3, max_ctx=1000)
    tw.join("a")
    tw.join("b")
    rng = np.random.default_rng(4)
    for t in range(PAGE):  # one page each
        tw.step(["a", "b"], [int(x) for x in rng.integers(0, wl.n_vocab, 2)])
    for t in range(PAGE):
        tw.step(["a"], [int(rng.integers(0, wl.n_vocab))])
    assert tw.pool.free_pages == 0
    from token_decode_amd import _capi as C
    from token_decode_amd import device as dv
    import torch
    tok = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(C.PNError) as e:  # both need a page; none is left
        dv.forward_batch(p.dm, [tw.pooled["b"], tw.pooled["a"]], tok)
    assert e.value.code == C.PN_ERANGE
    assert tw.pooled["a"].pos == 2 * PAGE and tw.pooled["b"].pos == PAGE and tw.pool.free_pages == 0
    with pytest.raises(C.PNError) as e:
        dv.prefill(p.dm, tw.pooled["a"], tok)
    assert e.value.code == C.PN_ERANGE and tw.pooled["a"].pos == 2 * PAGE
    tw.pooled["b"].reset()  # b's page goes back; the private twin is reset too
    tw.private["b"].reset()
    assert tw.pool.free_pages == 1
    tw.step(["a"], [5])  # now a gets it, and results are still those of the private twin
    tw.step(["a"], [6])
    assert tw.pool.free_pages == 0
    tw.leave("a")
    assert tw.pool.free_pages == 3


def test_prefill_set_kv_and_rewind():
    """set_kv and prefill into pooled states, set_pos jumps forward (unwritten
    positions read as zeros, on reused pages too) and back within the window;
    a rewind below recycled pages is refused."""
    import torch
    from token_decode_amd import _capi as C
    from token_decode_amd import device as dv
    wl = wl_window(100, seed=94)
    p = Pair(wl, max_batch=8)
    tw = Twins(p, n_pages=12, max_ctx=3000)
    # dirty every page of the pool first, then give them back
    tw.join("dirty")
    for side in (tw.pooled["dirty"],):
        for l in range(wl.n_layer):
            k, v = wl.kv_prefill(7, l, 0, 12 * PAGE)
            # 12 pages of positions, window or not: set_kv takes a page for each
            side.set_kv(l, 0, k, v)
    assert tw.pool.free_pages == 0
    tw.leave("dirty")
    assert tw.pool.free_pages == 12
    # resume from a cache written with set_kv (positions 150..299), as the parity tests do
    tw.join("s")
    for l in range(wl.n_layer):
        k, v = wl.kv_prefill(1, l, 150, 150)
        tw.pooled["s"].set_kv(l, 150, k, v)
        tw.private["s"].set_kv(l, 150, k, v)
    tw.pooled["s"].pos = 300
    tw.private["s"].pos = 300
    rng = np.random.default_rng(5)
    for t in range(30):
        tw.step(["s"], [int(rng.integers(0, wl.n_vocab))])
    # a prompt in chunks of 8 on both sides
    prompt = torch.tensor(rng.integers(0, wl.n_vocab, 45), dtype=torch.int32, device="cuda")
    outs = []
    for st in (tw.pooled["s"], tw.private["s"]):
        lg = torch.empty(45, wl.n_vocab, dtype=torch.float32, device="cuda")
        dv.prefill(p.dm, st, prompt, lg)
        outs.append(lg.cpu().numpy())
    np.testing.assert_array_equal(outs[0], outs[1])
    assert tw.pooled["s"].pos == 375
    # rewind inside the kept pages (the window of 360 starts at 261, page 4), then go on
    tw.pooled["s"].pos = 360
    tw.private["s"].pos = 360
    for t in range(5):
        tw.step(["s"], [int(rng.integers(0, wl.n_vocab))])
    # a rewind whose window reaches recycled pages is refused, pos unchanged
    with pytest.raises(C.PNError) as e:
        tw.pooled["s"].pos = 100
    assert e.value.code == C.PN_ERANGE and tw.pooled["s"].pos == 365
    with pytest.raises(C.PNError) as e:
        k, v = wl.kv_prefill(1, 0, 0, 10)
        tw.pooled["s"].set_kv(0, 0, k, v)
    assert e.value.code == C.PN_ERANGE
    # a jump forward over unwritten positions on a fresh pooled state (reused,
    # dirty pages): they read as zeros, as on the private twin
    tw.join("j", pos=0)
    tw.pooled["j"].pos = 130
    tw.private["j"].pos = 130
    for t in range(3):
        tw.step(["s", "j"], [int(x) for x in rng.integers(0, wl.n_vocab, 2)])
    with pytest.raises(C.PNError) as e:
        tw.pooled["j"].set_page_table(list(range(tw.pooled["j"].n_pages)))
    assert e.value.code == C.PN_EUNSUPPORTED
    log("  set_kv, prefill, rewind and jump on pooled states: equal to private bit for bit")


def test_fp32_cache_pool():
    """fp32 K/V rows and columns through the pool (no window: pages accumulate)."""
    wl = synth.tiny_fp32()
    p = Pair(wl, max_batch=3)
    tw = Twins(p, n_pages=12, max_ctx=500)
    rng = np.random.default_rng(6)
    for k in range(3):
        tw.join(k, pos=int(rng.integers(0, 100)))
    for t in range(90):
        keys = [k for k in range(3) if (t + k) % 4]
        tw.step(keys, [int(x) for x in rng.integers(0, wl.n_vocab, len(keys))])
    log("  fp32 cache, 3 sequences: pooled == private, %d pages free" % tw.pool.free_pages)
