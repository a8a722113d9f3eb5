"""GPU invariants of the batch, paging and state bookkeeping, checked on the HIP
path against itself (the oracle is not needed for these):

- a batched step equals each slot stepped alone;
- a permuted page table gives bit-identical results to the identity table;
- repeating the same steps from the same state is bitwise reproducible;
- an out-of-range token id sets the state's error flag and is read as row 0;
- greedy feedback on the device (the next token read from the previous step's
  argmax buffer) follows the same trajectory as feeding the ids from the host.
"""
import numpy as np
import pytest

import synth

from harness import LOW_TOL, Pair, compare_step, log

pytestmark = pytest.mark.gpu


def small(name, **kw):
    base = dict(n_layer=2, n_embd=200, n_head=6, n_kv_head=2, head_dim=32, n_ff=300, n_vocab=1000,
                rope_theta=10000.0, seed=61)
    base.update(kw)
    return synth.Workload(name, **base)


F32_WL = small("inv-f32", w_dtype=synth.F32, kv_dtype=synth.F32, act_dtype=synth.F32)
BF16_WL = small("inv-bf16-window", w_dtype=synth.BF16, kv_dtype=synth.BF16, act_dtype=synth.BF16,
                sliding_window=150, seed=62)


def _fill(pair, ds, slot, start):
    wl = pair.wl
    lo = wl.kv_window_start(start) if start > 0 else 0
    for l in range(wl.n_layer):
        if start > lo:
            k, v = wl.kv_prefill(slot, l, lo, start - lo)
            ds.set_kv(l, lo, k, v)
    ds.pos = start


def _state(pair, slot, start, max_ctx, pages=None):
    from token_decode_amd import device as dv
    ds = dv.DeviceState(pair.dm, max_ctx)
    if pages is not None:
        ds.set_page_table(pages)
    _fill(pair, ds, slot, start)
    return ds


def _steps_single(pair, ds, toks):
    """Step one state through toks; returns (logits [n][V], ids [n])."""
    import torch
    from token_decode_amd import device as dv
    wl = pair.wl
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    logits = torch.empty(wl.n_vocab, dtype=torch.float32, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    out_l, out_i = [], []
    for t in toks:
        tok.fill_(int(t))
        dv.forward_step(pair.dm, ds, tok, logits, am)
        out_l.append(logits.cpu().numpy().copy())
        out_i.append(int(am.item()))
    return np.stack(out_l), np.array(out_i)


def _steps_batch(pair, dss, toks):
    """toks [steps][n]; returns (logits [steps][n][V], ids [steps][n])."""
    import torch
    from token_decode_amd import device as dv
    wl = pair.wl
    n = len(dss)
    tok = torch.zeros(n, dtype=torch.int32, device="cuda")
    logits = torch.empty(n, wl.n_vocab, dtype=torch.float32, device="cuda")
    am = torch.empty(n, dtype=torch.int32, device="cuda")
    out_l, out_i = [], []
    for row in toks:
        tok.copy_(torch.tensor([int(t) for t in row], dtype=torch.int32))
        dv.forward_batch(pair.dm, dss, tok, logits, am)
        out_l.append(logits.cpu().numpy().copy())
        out_i.append(am.cpu().numpy().copy())
    return np.stack(out_l), np.stack(out_i)


@pytest.mark.parametrize("wl", [F32_WL, BF16_WL], ids=lambda w: w.name)
def test_batch_equals_single(wl):
    """Five slots stepped together equal the same slots stepped one at a time:
    fp32 within 1e-5 relative L2 with equal ids; bf16 activations within the
    bf16 tolerance (the batched and single GEMMs add in different orders, which
    can flip bf16 roundings), ids equal unless the top-two gap is a near tie."""
    starts = [0, 31, 64, 200, 401]
    n_steps = 3
    p = Pair(wl, max_batch=len(starts))
    toks = synth.uniform_int(wl.seed, 77, n_steps * len(starts), 0, wl.n_vocab - 1)
    toks = toks.reshape(n_steps, len(starts))
    max_ctx = max(starts) + n_steps + 1
    dss = [_state(p, i, s, max_ctx) for i, s in enumerate(starts)]
    bl, bi = _steps_batch(p, dss, toks)
    tol = 1e-5 if wl.act_dtype == synth.F32 else LOW_TOL
    worst = 0.0
    for i, s in enumerate(starts):
        ds = _state(p, i, s, max_ctx)
        sl, si = _steps_single(p, ds, toks[:, i])
        for t in range(n_steps):
            rel, _ = compare_step(wl, bl[t, i], sl[t].astype(np.float64), int(bi[t, i]), int(si[t]),
                                  "slot %d step %d:" % (i, t), tol)
            worst = max(worst, rel)
    log("  %s: batch vs single worst rel L2 %.2e" % (wl.name, worst))


@pytest.mark.parametrize("wl", [F32_WL, BF16_WL], ids=lambda w: w.name)
def test_permuted_page_table_bitwise(wl):
    """A state whose logical pages map to a seeded permutation of the physical
    pages gives bit-identical logits to one with the identity table."""
    start, n_steps = 450, 3
    p = Pair(wl)
    max_ctx = start + n_steps + 1
    toks = synth.uniform_int(wl.seed, 78, n_steps, 0, wl.n_vocab - 1)
    a = _state(p, 0, start, max_ctx)
    n = a.n_pages
    perm = np.random.default_rng(7).permutation(n)
    assert n > 2 and not np.array_equal(perm, np.arange(n))
    b = _state(p, 0, start, max_ctx, pages=perm)
    la, ia = _steps_single(p, a, toks)
    lb, ib = _steps_single(p, b, toks)
    np.testing.assert_array_equal(ia, ib)
    assert la.tobytes() == lb.tobytes(), "permuted page table changed the logits"
    log("  %s: %d pages permuted, logits bit-identical" % (wl.name, n))


def test_repeat_runs_bitwise():
    """The same batched steps from the same cached state, run twice (the cache
    refilled in between, positions rewound), give bit-identical logits and ids."""
    wl = BF16_WL
    starts = [5, 130, 260, 777]
    n_steps = 3
    p = Pair(wl, max_batch=len(starts))
    toks = synth.uniform_int(wl.seed, 79, n_steps * len(starts), 0, wl.n_vocab - 1)
    toks = toks.reshape(n_steps, len(starts))
    max_ctx = max(starts) + n_steps + 1
    dss = [_state(p, i, s, max_ctx) for i, s in enumerate(starts)]
    l1, i1 = _steps_batch(p, dss, toks)
    for i, (ds, s) in enumerate(zip(dss, starts)):
        ds.reset()
        _fill(p, ds, i, s)
    l2, i2 = _steps_batch(p, dss, toks)
    np.testing.assert_array_equal(i1, i2)
    assert l1.tobytes() == l2.tobytes(), "repeated steps differ"


def test_bad_token_sets_flag():
    """A token id >= n_vocab sets bit 0 of the state's flags and embeds row 0:
    its logits equal those of token 0 bit for bit.  Reading clears the flags."""
    wl = F32_WL
    p = Pair(wl)
    a = _state(p, 0, 40, 48)
    b = _state(p, 0, 40, 48)
    la, _ = _steps_single(p, a, [0])
    assert a.check_flags() == 0
    lb, _ = _steps_single(p, b, [wl.n_vocab + 5])
    assert b.check_flags() & 1
    assert b.check_flags() == 0
    assert la.tobytes() == lb.tobytes()


def test_device_greedy_feedback():
    """Feeding each step the previous step's argmax buffer on the device follows
    the trajectory of feeding the same ids from the host, bit for bit."""
    import torch
    from token_decode_amd import device as dv
    wl = F32_WL
    p = Pair(wl)
    n_steps = 12
    a = _state(p, 0, 100, 100 + n_steps + 1)
    b = _state(p, 0, 100, 100 + n_steps + 1)
    am = torch.full((1,), 17, dtype=torch.int32, device="cuda")
    logits = torch.empty(wl.n_vocab, dtype=torch.float32, device="cuda")
    dev_ids, dev_l = [], []
    for _ in range(n_steps):
        dv.forward_step(p.dm, a, am, logits, am)
        dev_ids.append(int(am.item()))
        dev_l.append(logits.cpu().numpy().copy())
    host_toks = [17] + dev_ids[:-1]
    hl, hi = _steps_single(p, b, host_toks)
    np.testing.assert_array_equal(np.array(dev_ids), hi)
    assert np.stack(dev_l).tobytes() == hl.tobytes()


@pytest.mark.parametrize("act", [synth.BF16, synth.F32], ids=["bf16-act", "f32-act"])
def test_o_prologue_per_wave_bitwise(act):
    """The O projection's input conversion done per wave over every slot (the
    automatic choice for 2 to 8 slots in 16-wave work-groups) gives the same
    logits, bit for bit, as the work-group converting it together.  bf16
    weights, 16-wave O groups, 8 slots (5 with fp32 activations, three bf16
    pieces each), from ragged positions."""
    from token_decode_amd import _capi as C
    wl = small("inv-oprologue-" + ("bf16" if act == synth.BF16 else "f32"), n_head=8, n_kv_head=2, head_dim=64,
               n_embd=512, n_ff=640, w_dtype=synth.BF16, kv_dtype=synth.BF16, act_dtype=act, seed=63)
    starts = [3, 70, 129, 200, 257, 64, 1, 333][:8 if act == synth.BF16 else 5]
    n_steps = 3
    p = Pair(wl, max_batch=len(starts))
    p.dm.set_option(C.PN_OPT_WAVES_O, 16)
    toks = synth.uniform_int(wl.seed, 79, n_steps * len(starts), 0, wl.n_vocab - 1).reshape(n_steps, len(starts))
    max_ctx = max(starts) + n_steps + 1
    out = []
    for mode in (0, 1):
        p.dm.set_option(C.PN_OPT_GEMM_PROLOGUE, mode)
        dss = [_state(p, i, s, max_ctx) for i, s in enumerate(starts)]
        out.append(_steps_batch(p, dss, toks))
    np.testing.assert_array_equal(out[0][1], out[1][1])
    assert out[0][0].tobytes() == out[1][0].tobytes(), "the per-wave O prologue changed the logits"
    log("  %s: %d slots, %d steps, per-wave and shared O prologues bit-identical" % (wl.name, len(starts), n_steps))
