"""Shared helpers of the GPU parity tests: drive the HIP path and the oracle on
the same seeded inputs and compare them."""
from __future__ import annotations

import os
import time

import numpy as np

import oracle
import synth

FP32_TOL = 1e-4   # relative L2 of fp32 logits
LOW_TOL = 2e-2    # relative L2 of bf16 / int8 logits


def tol_of(wl):
    return FP32_TOL if (wl.w_dtype == synth.F32 and wl.act_dtype == synth.F32
                        and wl.kv_dtype == synth.F32) else LOW_TOL


def oracle_threads():
    return max(1, min(16, os.cpu_count() or 1))


def log(msg):
    print(msg, flush=True)


def device_config(wl, max_batch=1, prefill_chunk=0):
    from token_decode_amd import device as dv
    return dv.make_config(wl.n_layer, wl.n_embd, wl.n_head, wl.n_kv_head, wl.head_dim, wl.n_ff,
                          wl.n_vocab, n_expert=wl.n_expert, n_expert_used=wl.n_expert_used,
                          sliding_window=wl.sliding_window, max_batch=max_batch,
                          rope_theta=wl.rope_theta, rms_norm_eps=wl.rms_norm_eps,
                          w_dtype=wl.w_dtype, kv_dtype=wl.kv_dtype, act_dtype=wl.act_dtype,
                          rope_neox=wl.rope_neox, qkv_bias=wl.qkv_bias, prefill_chunk=prefill_chunk)


def check_step(wl, g_logits, o_logits, g_id, o_id, tol=None):
    """The parity rule without asserting: (ok, relative L2, near tie, message).
    Relative L2 within the workload's tolerance (or `tol`); ids equal unless the
    oracle's top-two gap is within 8x the observed error (a near tie, either id
    valid)."""
    tol = tol_of(wl) if tol is None else tol
    g = np.asarray(g_logits, dtype=np.float64)
    rel = float(np.linalg.norm(g - o_logits) / np.linalg.norm(o_logits))
    if not rel <= tol:
        return False, rel, False, "relative L2 %.3g > %.1g" % (rel, tol)
    near = False
    if g_id != o_id:
        err = float(np.max(np.abs(g - o_logits)))
        gap = float(np.float32(o_logits[o_id]) - np.float32(o_logits[g_id]))
        near = gap <= 8 * err
        if not near:
            return False, rel, False, "id %d vs oracle %d (gap %.3g, max err %.3g)" % (g_id, o_id, gap, err)
    return True, rel, near, ""


def compare_step(wl, g_logits, o_logits, g_id, o_id, what="", tol=None):
    """Assert the parity rule of check_step; returns (relative L2, near tie)."""
    ok, rel, near, msg = check_step(wl, g_logits, o_logits, g_id, o_id, tol)
    assert ok, "%s %s" % (what, msg)
    return rel, near


MAX_TIE_LAYERS = 4  # routing near ties enumerated per slot-step (2^4 branches at most)


def moe_step_branches(wl, ost, token, g_logits, g_id, route_tol, threads, tol=None):
    """One oracle MoE step checked against the GPU's row, with routing near ties.

    The oracle steps once, recording each layer's router gap between the k-th
    and (k+1)-th expert logits (compared in fp32).  Where a gap is below
    `route_tol`, the GPU's router, whose input carries the bf16 rounding noise
    of the layers before, may validly pick the (k+1)-th expert instead, and
    everything after that layer differs.  So the oracle also runs every
    combination of those swaps (the position is rewound and the step redone;
    each step rewrites every layer's K/V at that position), and the GPU must
    match one branch by the parity rule.  The oracle's state ends in the
    matching branch, so later steps continue from the cache the GPU holds.
    Returns (relative L2, near tie, swap mask of the matching branch, that
    branch's greedy id); no value comes from the GPU except the row being
    checked."""
    p = ost.pos
    ol, oa, _, _, gaps = ost.step(token, threads=threads, want_route=True, want_gaps=True)
    ok, rel, near, msg = check_step(wl, g_logits, ol, g_id, oa, tol)
    if ok:
        return rel, near, 0, oa
    ties = [l for l in range(wl.n_layer) if gaps[l] < route_tol]
    assert ties, msg + " (no routing near tie: gaps >= %.1g)" % route_tol
    assert len(ties) <= MAX_TIE_LAYERS, "%d routing near ties: %s" % (len(ties), ties)
    tried = ["base: " + msg]
    for sub in range(1, 1 << len(ties)):
        mask = sum(1 << ties[i] for i in range(len(ties)) if (sub >> i) & 1)
        ost.pos = p
        bl, ba = ost.step(token, threads=threads, swap_mask=mask)
        ok, rel, near, msg = check_step(wl, g_logits, bl, g_id, ba, tol)
        if ok:
            return rel, near, mask, ba
        tried.append("swap %s: %s" % ([l for l in ties if (mask >> l) & 1], msg))
    raise AssertionError("no routing branch matches (near-tie layers %s, gaps %s): %s"
                         % (ties, [float("%.2e" % gaps[l]) for l in ties], "; ".join(tried)))


class Pair:
    """A device model and the oracle over the same seeded weights."""

    def __init__(self, wl, max_batch=1, weights=None, prefill_chunk=0):
        from token_decode_amd import device as dv
        t = time.time()
        self.wl = wl
        self.W = weights if weights is not None else synth.make_weights(wl)
        self.om = oracle.Model(wl, self.W)
        self.cfg = device_config(wl, max_batch, prefill_chunk)
        self.dm = dv.DeviceModel(self.cfg, self.W)
        log("  [%s] weights ready in %.1fs" % (wl.name, time.time() - t))

    def states(self, slot, start_pos, max_ctx):
        """A device state and an oracle state for `slot`, K/V filled below start_pos."""
        from token_decode_amd import device as dv
        wl = self.wl
        ds = dv.DeviceState(self.dm, max_ctx)
        os_ = self.om.new_state(max_ctx)
        lo = wl.kv_window_start(start_pos) if start_pos > 0 else 0
        if start_pos > 0:
            for l in range(wl.n_layer):
                k, v = wl.kv_prefill(slot, l, lo, start_pos - lo)
                ds.set_kv(l, lo, k, v)
                os_.set_kv(l, lo, k, v)
        ds.pos = start_pos
        os_.pos = start_pos
        return ds, os_


def run_single(pair, start_pos, tokens_in, n_decode, max_ctx=None, threads=None, tol=None):
    """Feed tokens_in, then n_decode greedy steps of the oracle; the GPU is fed the
    oracle's tokens.  Returns (max rel L2, near-tie count, steps)."""
    import torch
    from token_decode_amd import device as dv
    wl = pair.wl
    threads = threads or oracle_threads()
    total = len(tokens_in) + n_decode
    max_ctx = max_ctx or (start_pos + total + 1)
    ds, ost = pair.states(0, start_pos, max_ctx)
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    logits = torch.empty(wl.n_vocab, dtype=torch.float32, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    seq = list(int(t) for t in tokens_in)
    worst, near = 0.0, 0
    for i in range(total):
        t = seq[i]
        tok.fill_(t)
        dv.forward_step(pair.dm, ds, tok, logits, am)
        ol, oa = ost.step(t, threads=threads)
        g = logits.cpu().numpy()
        rel, nt = compare_step(wl, g, ol, int(am.item()), oa, "step %d:" % i, tol)
        log("    step %d: rel L2 %.2e" % (i, rel))
        worst = max(worst, rel)
        near += int(nt)
        if i >= len(tokens_in) - 1 and len(seq) < total:
            seq.append(oa)
    assert ds.pos == start_pos + total
    return worst, near, total


def run_batch(pair, starts, n_steps, max_ctx=None, threads=None, slots=None, tol=None, route_tol=None,
              stats=None):
    """Batched steps: slot i starts at starts[i]; the GPU is fed each slot's oracle
    trajectory.  Returns (max rel L2, near-tie count).

    With `route_tol` (MoE), each slot-step goes through moe_step_branches: where
    a layer's router gap is below it, the oracle's swapped-expert branches are
    also valid results and the GPU must match one of them; `stats` (a dict)
    receives the counts of slot-steps matched on the oracle's own routing
    ("base") and on a swapped branch ("swapped")."""
    import torch
    from token_decode_amd import device as dv
    wl = pair.wl
    threads = threads or oracle_threads()
    n = len(starts)
    slots = slots if slots is not None else list(range(n))
    pairs = [pair.states(slots[i], int(starts[i]), max_ctx or int(starts[i]) + n_steps + 1)
             for i in range(n)]
    dss = [p[0] for p in pairs]
    oss = [p[1] for p in pairs]
    toks = [int(t) for t in synth.uniform_int(wl.seed, (1 << 20) + 7, n, 0, wl.n_vocab - 1)]
    tok = torch.zeros(n, dtype=torch.int32, device="cuda")
    logits = torch.empty(n, wl.n_vocab, dtype=torch.float32, device="cuda")
    am = torch.empty(n, dtype=torch.int32, device="cuda")
    worst, near = 0.0, 0
    for step in range(n_steps):
        tok.copy_(torch.tensor(toks, dtype=torch.int32))
        dv.forward_batch(pair.dm, dss, tok, logits, am)
        g = logits.cpu().numpy()
        ga = am.cpu().numpy()
        for i in range(n):
            what = "step %d slot %d:" % (step, i)
            if route_tol is None:
                ol, oa = oss[i].step(toks[i], threads=threads)
                rel, nt = compare_step(wl, g[i], ol, int(ga[i]), oa, what, tol)
            else:
                try:
                    rel, nt, mask, oa = moe_step_branches(wl, oss[i], toks[i], g[i], int(ga[i]), route_tol,
                                                      threads, tol)
                except AssertionError as e:
                    raise AssertionError("%s %s" % (what, e))
                if mask:
                    log("    %s matched the routing branch with layers %s swapped"
                        % (what, [l for l in range(wl.n_layer) if (mask >> l) & 1]))
                if stats is not None:
                    key = "swapped" if mask else "base"
                    stats[key] = stats.get(key, 0) + 1
            worst = max(worst, rel)
            near += int(nt)
            toks[i] = oa
    return worst, near
