"""GPU parity of the layout variants that share the Llama forward through
config flags: q/k/v projection biases (Qwen2) and the NeoX half-split RoPE
(Phi-3), against the oracle, in every storage type; and fused QKV / gate+up
checkpoints, which must load into the same packed model as separate ones.

The NeoX rotation is realised by storing each head's q and k rows in
rotation-pair order (the attention's dot products are order-free); the cached
k is then in that order too, so resuming from K/V written with set_kv also
checks the reordering of the caller's k rows."""
import numpy as np
import pytest

import synth

from harness import Pair, log, run_batch, run_single

pytestmark = pytest.mark.gpu


def ragged(name, **kw):
    base = dict(n_layer=2, n_embd=200, n_head=6, n_kv_head=2, head_dim=32, n_ff=300, n_vocab=1000,
                rope_theta=10000.0, seed=61)
    base.update(kw)
    return synth.Workload(name, **base)


def test_neox_bias_tiny_fp32_from_zero():
    wl = synth.tiny_fp32().with_(name="tiny-neox-bias", rope_neox=True, qkv_bias=True, seed=62)
    p = Pair(wl)
    worst, near, n = run_single(p, 0, wl.prompt_tokens(), 40)
    log("  tiny fp32 NeoX + bias: %d steps, worst rel L2 %.2e, near %d" % (n, worst, near))
    assert near == 0


SINGLE = [
    ragged("neox-f32", rope_neox=True, w_dtype=synth.F32, kv_dtype=synth.F32, act_dtype=synth.F32),
    ragged("bias-f32", qkv_bias=True, w_dtype=synth.F32, kv_dtype=synth.F32, act_dtype=synth.F32, seed=63),
    ragged("neox-bias-bf16-actf32-window", rope_neox=True, qkv_bias=True, w_dtype=synth.BF16,
           kv_dtype=synth.BF16, act_dtype=synth.F32, sliding_window=300, seed=64),
    ragged("neox-bias-int8-d128", rope_neox=True, qkv_bias=True, n_head=4, n_kv_head=2, head_dim=128,
           w_dtype=synth.I8, kv_dtype=synth.BF16, act_dtype=synth.BF16, seed=65, n_ff=520),
    ragged("neox-bf16-d64-g8", rope_neox=True, n_head=8, n_kv_head=1, head_dim=64, w_dtype=synth.BF16,
           kv_dtype=synth.BF16, act_dtype=synth.BF16, seed=66),
]


@pytest.mark.parametrize("wl", SINGLE, ids=lambda w: w.name)
def test_variant_single_on_prefilled_cache(wl):
    """700 positions written with set_kv (several attention splits), then 6 steps."""
    p = Pair(wl)
    toks = synth.uniform_int(wl.seed, 1 << 20, 2, 0, wl.n_vocab - 1)
    worst, near, n = run_single(p, 700, toks, 4)
    log("  %s: worst rel L2 %.2e near %d" % (wl.name, worst, near))


def test_variant_batched_window():
    wl = ragged("neox-bias-batch", rope_neox=True, qkv_bias=True, w_dtype=synth.BF16, kv_dtype=synth.BF16,
                act_dtype=synth.BF16, sliding_window=200, seed=67)
    p = Pair(wl, max_batch=5)
    worst, near = run_batch(p, [3, 64, 129, 450, 1000], 3)
    log("  NeoX + bias, 5 slots: worst rel L2 %.2e near %d" % (worst, near))


def test_variant_moe_batched():
    wl = ragged("neox-bias-moe", rope_neox=True, qkv_bias=True, n_expert=4, n_expert_used=2, w_dtype=synth.BF16,
                kv_dtype=synth.BF16, act_dtype=synth.BF16, seed=68, n_ff=128)
    p = Pair(wl, max_batch=4)
    worst, near = run_batch(p, [5, 70, 200, 511], 3)
    log("  NeoX + bias MoE: worst rel L2 %.2e near %d" % (worst, near))


@pytest.mark.parametrize("dt", [synth.BF16, synth.I8])
def test_fused_checkpoints_load_the_same_model(dt):
    """[q; k; v] and [gate; up] in one buffer each: the same logits, bit for bit."""
    import torch
    from token_decode_amd import device as dv
    from harness import device_config
    wl = ragged("fused-%d" % dt, rope_neox=True, qkv_bias=True, w_dtype=dt, kv_dtype=synth.BF16,
                act_dtype=synth.BF16, seed=69)
    W = synth.make_weights(wl)
    Wf = dict(W)
    Wf["layers"] = []
    for L in W["layers"]:
        Lf = dict(L)
        Lf["wqkv"] = np.concatenate([L["wq"], L["wk"], L["wv"]])
        Lf["w_gate_up"] = np.concatenate([L["w_gate"][0], L["w_up"][0]])
        for k in ("wq", "wk", "wv"):
            Lf[k] = None
        Lf["w_gate"], Lf["w_up"] = [None], [None]
        Wf["layers"].append(Lf)
    cfg = device_config(wl)
    outs = []
    for weights in (W, Wf):
        dm = dv.DeviceModel(cfg, weights)
        st = dv.DeviceState(dm, 64)
        lg = torch.empty(wl.n_vocab, dtype=torch.float32, device="cuda")
        rows = []
        for t in (5, 17, 900, 3):
            dv.forward_step(dm, st, torch.tensor([t], dtype=torch.int32, device="cuda"), lg)
            rows.append(lg.cpu().numpy().copy())
        outs.append(np.stack(rows))
    np.testing.assert_array_equal(outs[0], outs[1])
