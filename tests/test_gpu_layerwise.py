"""Full-depth parity, one layer at a time.

A layer is a function of its input residual x, the cache and the position
("Core Engine API", section "pn_model struct": the forward maps a token and a
state to logits; "Core Engine API", section "Scratch (arena) estimation": the
per-layer intermediates are computed from x).  End to end, 32 layers of bf16
activations amplify the few bf16 roundings that fp32 arithmetic decides
differently from the fp64 oracle to a ~2% logit difference (the end-to-end
full-depth cases in test_gpu_fullsize.py measure it, and
tests/test_oracle_state_pins.py shows the oracle alone moving that much under
fp32-sized perturbations).  Layer by layer there is no amplification: the
device records the residual entering every layer (pn_model_trace), the oracle
recomputes each layer from the device's own input at the same position (its
cache fed the same way, so it holds what the device's holds), and every
layer's update of the residual must agree within LAYER_TOL; the LM head on the
device's final residual is then held to the step's own tolerance and id rule.
LAYER_TOL is the benchmark spec's bound for bf16 / INT8 logits applied to each
layer's update: within one layer a single bf16 rounding flip of a normed
input moves every gate/up output by ~1e-4 relative, which flips hundreds of
the hidden values' roundings in turn, so a layer's update legitimately moves
by up to ~3e-3 (measured worst: 1.9e-3 Llama-3-8B INT8, 3.2e-3 Mistral-7B,
2.8e-3 Mixtral); a wrong index, term or routing moves it by O(1).
The embedding row must match bit for bit.  For MoE, where a layer's router
gap between the k-th and (k+1)-th experts is below ROUTE_TOL, the layer may
also match the oracle's branch with those experts swapped.
"""
import ctypes
import time

import numpy as np
import pytest

import synth

from harness import Pair, compare_step, log, oracle_threads

pytestmark = pytest.mark.gpu

LAYER_TOL = 2e-2  # relative L2 of one layer's update of the residual stream
ROUTE_TOL = 1e-2


def _layerwise(wl, steps=2):
    import torch
    from token_decode_amd import _capi as C
    from token_decode_amd import device as dv
    t = time.time()
    p = Pair(wl, max_batch=wl.slots)
    B, L, E = wl.slots, wl.n_layer, wl.n_embd
    starts = [int(s) for s in wl.start_positions()]
    pairs = [p.states(i, starts[i], starts[i] + steps + 1) for i in range(B)]
    dss, oss = [q[0] for q in pairs], [q[1] for q in pairs]
    log("  [%s] ready in %.1fs" % (wl.name, time.time() - t))
    trace = torch.zeros((L + 1, B, E), dtype=torch.float32, device="cuda")
    C.check(C.lib().pn_model_trace(p.dm.h, ctypes.c_void_p(trace.data_ptr())))
    threads = oracle_threads()
    toks = [int(x) for x in wl.first_tokens()]
    tok = torch.zeros(B, dtype=torch.int32, device="cuda")
    logits = torch.empty(B, wl.n_vocab, dtype=torch.float32, device="cuda")
    am = torch.empty(B, dtype=torch.int32, device="cuda")
    worst_layer, worst_head, swaps = 0.0, 0.0, 0
    try:
        for step in range(steps):
            tok.copy_(torch.tensor(toks, dtype=torch.int32))
            if B == 1:
                dv.forward_step(p.dm, dss[0], tok, logits, am)
            else:
                dv.forward_batch(p.dm, dss, tok, logits, am)
            xs = trace.cpu().numpy()
            g, ga = logits.cpu().numpy(), am.cpu().numpy()
            for i in range(B):
                pos = oss[i].pos
                x0 = p.om.embed(toks[i])
                assert np.array_equal(xs[0, i].astype(np.float64), x0), "step %d slot %d: embedding" % (step, i)
                for l in range(L):
                    xin = xs[l, i].astype(np.float64)
                    dg = xs[l + 1, i].astype(np.float64) - xin
                    out, _, gap = oss[i].layer(l, pos, xin, threads=threads, want_route=True)
                    do = out - xin
                    rel = float(np.linalg.norm(dg - do) / np.linalg.norm(do))
                    if rel > LAYER_TOL and wl.n_expert > 0 and gap < ROUTE_TOL:
                        out = oss[i].layer(l, pos, xin, threads=threads, swap=True)
                        do = out - xin
                        rel = float(np.linalg.norm(dg - do) / np.linalg.norm(do))
                        swaps += 1
                        log("    step %d slot %d layer %d: matched the swapped routing branch (gap %.2e)"
                            % (step, i, l, gap))
                    assert rel <= LAYER_TOL, "step %d slot %d layer %d: update relative L2 %.3g > %.1g" % (
                        step, i, l, rel, LAYER_TOL)
                    worst_layer = max(worst_layer, rel)
                ol, oa = p.om.head(xs[L, i], threads=threads)
                rel, _ = compare_step(wl, g[i], ol, int(ga[i]), oa, "step %d slot %d head:" % (step, i))
                worst_head = max(worst_head, rel)
                oss[i].pos = pos + 1
                toks[i] = oa
            log("    step %d: worst layer update %.2e, worst head %.2e" % (step, worst_layer, worst_head))
    finally:
        C.check(C.lib().pn_model_trace(p.dm.h, None))
    log("  %s: %d layers x %d slots x %d steps, worst layer update rel L2 %.2e, worst logits %.2e, "
        "routing swaps %d" % (wl.name, L, B, steps, worst_layer, worst_head, swaps))


def test_layerwise_llama3_8b_int8_full():
    """Llama-3-8B INT8 weights, bf16 activations and cache, all 32 layers, from position 8192."""
    _layerwise(synth.llama3_8b_int8())


def test_layerwise_mistral_7b_8slots_full():
    """Mistral-7B shape, window 4096, 8 slots, all 32 layers."""
    _layerwise(synth.mistral_7b_slots())


def test_layerwise_mixtral_8x7b_16slots_full():
    """Mixtral-8x7B shape, 8 experts top-2, 16 slots, all 32 layers (93 GB of weights)."""
    _layerwise(synth.mixtral_8x7b_slots())
