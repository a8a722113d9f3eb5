"""GPU parity of on-device sampling (pn_sample) against the reference sampler.

The ranking decisions (which tokens form the top-k, their canonical order)
are taken on the same fp32 values on both sides and must agree exactly.  The
draw compares u times a prefix total with fp64 prefix sums of exp() values,
which the GPU computes in fp32 and the oracle in fp64: a draw is accepted when
the GPU's token is the oracle's, or when u lies within 1e-5 (relative to the
prefix total) of the boundary between the two tokens' intervals, where either
token is a correct result at fp32 precision; such near ties are counted and
must stay rare.
"""
import numpy as np
import pytest

import synth
from oracle import sampling as S

from harness import device_config, log

pytestmark = pytest.mark.gpu

V = 128256
SLOTS = 4


@pytest.fixture(scope="module")
def model():
    from token_decode_amd import device as dv
    wl = synth.Workload("sampler-host", n_layer=1, n_embd=64, n_head=2, n_kv_head=1, head_dim=32, n_ff=64,
                        n_vocab=V, rope_theta=10000.0, w_dtype=synth.BF16, kv_dtype=synth.BF16,
                        act_dtype=synth.BF16, seed=71)
    return dv.DeviceModel(device_config(wl, max_batch=SLOTS), synth.make_weights(wl))


def run(model, rows, params, us, recent=None):
    import torch
    from token_decode_amd import device as dv
    n = len(params)
    lg = torch.from_numpy(np.ascontiguousarray(np.stack(rows).astype(np.float32))).cuda()
    u = torch.tensor(us, dtype=torch.float32, device="cuda")
    ids = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    rc = None if recent is None else torch.from_numpy(np.ascontiguousarray(recent, dtype=np.int32)).cuda()
    dv.sample(model, lg, params, u, ids, rc)
    return ids.cpu().numpy()


def check(row, p, u, got, recent=(), tol=1e-5):
    """True when exact, 'near' for an accepted near tie; raises otherwise."""
    want, ids, cum, tot = S.sample(row, p["temperature"], p.get("top_k", 40), p.get("top_p", 1.0),
                                   p.get("repeat_penalty", 1.0), recent, u, detail=True)
    if got == want:
        return True
    pos = np.nonzero(ids == got)[0]
    assert len(pos) == 1, "token %d outside the oracle's prefix (want %d)" % (got, want)
    j, jw = int(pos[0]), int(np.nonzero(ids == want)[0][0])
    assert abs(j - jw) == 1, "token %d at %d, oracle %d at %d" % (got, j, want, jw)
    boundary = cum[min(j, jw)]
    assert abs(u * tot - boundary) <= tol * tot, "u*W %.9g vs boundary %.9g" % (u * tot, boundary)
    return "near"


def test_greedy_ties_and_nan(model):
    rng = np.random.default_rng(1)
    rows = []
    for b in range(SLOTS):
        r = rng.standard_normal(V).astype(np.float32)
        m = float(r.max()) + 1.0
        r[[5 + b, 9000 + b, V - 1]] = m  # three equal maxima: the lowest index wins
        if b == 1:
            r[3] = np.nan
        rows.append(r)
    got = run(model, rows, [dict(temperature=0.0)] * SLOTS, [0.9] * SLOTS)
    np.testing.assert_array_equal(got, [5 + b for b in range(SLOTS)])


def test_top1_with_penalty(model):
    rng = np.random.default_rng(2)
    rows = [rng.standard_normal(V).astype(np.float32) for _ in range(SLOTS)]
    recent = np.full((SLOTS, 16), -1, np.int32)
    for b in range(SLOTS):
        top = np.argsort(-rows[b])[:8]
        recent[b, :8] = top  # penalise the 8 highest: the 9th ranks first unless a penalty is mild
        recent[b, 8] = top[0]  # a repeat counts once
    params = [dict(temperature=0.8, top_k=1, repeat_penalty=r) for r in (1.0, 1.3, 2.0, 5.0)]
    got = run(model, rows, params, [0.5] * SLOTS, recent)
    for b in range(SLOTS):
        want = S.sample(rows[b], 0.8, 1, repeat_penalty=params[b]["repeat_penalty"], recent=recent[b])
        assert got[b] == want


@pytest.mark.parametrize("temp,k,p", [(1.0, 40, 1.0), (0.7, 1000, 0.9), (1.5, 4096, 0.95), (1.0, 4096, 0.5),
                                      (2.0, 7, 0.3)])
def test_draws_match_oracle(model, temp, k, p):
    rng = np.random.default_rng(int(temp * 10) + k)
    rows = [(rng.standard_normal(V) * 2).astype(np.float32) for _ in range(SLOTS)]
    recent = rng.integers(-1, V, size=(SLOTS, 64)).astype(np.int32)
    params = [dict(temperature=temp, top_k=k, top_p=p, repeat_penalty=1.1)] * SLOTS
    near = exact = 0
    for i in range(16):
        us = [float((i * SLOTS + b + 0.5) / (16 * SLOTS)) for b in range(SLOTS)]
        got = run(model, rows, params, us, recent)
        for b in range(SLOTS):
            r = check(rows[b], params[b], us[b], int(got[b]), recent[b])
            near += r == "near"
            exact += r is True
    log("  T %.1f k %d p %.2f: %d exact, %d near ties" % (temp, k, p, exact, near))
    assert near <= 2


def test_equal_logits_take_lowest_indices(model):
    """128256 equal values: the top 4096 are tokens 0..4095 in index order."""
    rows = [np.full(V, 0.25, np.float32) for _ in range(SLOTS)]
    us = [0.0, 0.3, 0.71, 0.999]
    got = run(model, rows, [dict(temperature=1.0, top_k=4096)] * SLOTS, us)
    for b in range(SLOTS):
        assert got[b] == int(us[b] * 4096)  # equal weights: a uniform pick over 0..4095
        assert got[b] == S.sample(rows[b], 1.0, 4096, u=us[b])


def test_near_equal_logits_refine(model):
    """Values spread over a few fp32 ulps (most keys share their top 24 bits):
    the histogram narrows over all three key levels."""
    rng = np.random.default_rng(5)
    base = np.float32(1.5)
    rows = []
    for _ in range(SLOTS):
        r = np.full(V, base, np.float32)
        steps = rng.integers(0, 200, size=V)
        r = np.nextafter(r, np.float32(2.0))
        r = (base + steps.astype(np.float32) * (r[0] - base)).astype(np.float32)
        rows.append(r)
    params = [dict(temperature=1.0, top_k=k, top_p=1.0) for k in (1, 100, 2000, 4096)]
    us = [0.5, 0.25, 0.8, 0.1]
    got = run(model, rows, params, us)
    for b in range(SLOTS):
        check(rows[b], params[b], us[b], int(got[b]))


def test_mixed_rows(model):
    rng = np.random.default_rng(6)
    rows = [(rng.standard_normal(V) * s).astype(np.float32) for s in (0.5, 1.0, 3.0, 8.0)]
    params = [dict(temperature=0.0), dict(temperature=1.0, top_k=50, top_p=0.9),
              dict(temperature=0.3, top_k=4096, top_p=0.99, repeat_penalty=1.5), dict(temperature=5.0, top_k=2)]
    recent = rng.integers(0, V, size=(SLOTS, 1024)).astype(np.int32)
    us = [0.4, 0.77, 0.05, 0.5]
    got = run(model, rows, params, us, recent)
    for b in range(SLOTS):
        check(rows[b], params[b], us[b], int(got[b]), recent[b])


def test_sampled_decode_loop():
    """Decode with sampling on the device: each step's sampled id is the next
    step's token (no host round trip).  Every step's draw is checked against
    the reference sampler applied to the GPU's own logits with the same u."""
    import torch
    from token_decode_amd import device as dv
    wl = synth.tiny_fp32()
    dm = dv.DeviceModel(device_config(wl), synth.make_weights(wl))
    st = dv.DeviceState(dm, 64)
    n = 40
    us = np.random.default_rng(8).random(n).astype(np.float32)
    u_dev = torch.from_numpy(us).cuda()
    tok = torch.tensor([int(wl.prompt_tokens()[0])], dtype=torch.int32, device="cuda")
    logits = torch.empty(wl.n_vocab, dtype=torch.float32, device="cuda")
    params = [dict(temperature=0.9, top_k=50, top_p=0.9, repeat_penalty=1.2)]
    recent = torch.full((1, 8), -1, dtype=torch.int32, device="cuda")
    hist, near = [int(tok.item())], 0
    for i in range(n):
        dv.forward_step(dm, st, tok, logits, None)
        recent[0, i % 8] = tok[0]  # the window holds the last 8 tokens fed
        dv.sample(dm, logits.view(1, -1), params, u_dev[i:i + 1], tok, recent)
        g = logits.cpu().numpy()
        r = check(g, params[0], float(us[i]), int(tok.item()), recent.cpu().numpy()[0])
        near += r == "near"
        hist.append(int(tok.item()))
    log("  sampled trajectory %s..., near ties %d" % (hist[:12], near))
    assert near <= 1
    assert st.pos == n


def test_vocab_past_one_pass():
    """A vocabulary of 262147 tokens: each key / gather work-group loops over
    more than one pass of its share, and the last share is ragged."""
    from token_decode_amd import device as dv
    Vb = 262147
    wl = synth.Workload("sampler-wide", n_layer=1, n_embd=64, n_head=2, n_kv_head=1, head_dim=32, n_ff=64,
                        n_vocab=Vb, rope_theta=10000.0, w_dtype=synth.BF16, kv_dtype=synth.BF16,
                        act_dtype=synth.BF16, seed=72)
    dm = dv.DeviceModel(device_config(wl, max_batch=3), synth.make_weights(wl))
    rng = np.random.default_rng(9)
    rows = [(rng.standard_normal(Vb) * s).astype(np.float32) for s in (1.0, 2.0, 4.0)]
    rows[2][Vb - 1] = 40.0  # the last token (in the ragged tail) dominates this row
    params = [dict(temperature=0.8, top_k=40, top_p=0.95, repeat_penalty=1.1),
              dict(temperature=1.0, top_k=4096, top_p=1.0), dict(temperature=0.0)]
    recent = rng.integers(0, Vb, size=(3, 64)).astype(np.int32)
    us = [0.3, 0.9, 0.5]
    got = run(dm, rows, params, us, recent)
    for b in range(3):
        check(rows[b], params[b], us[b], int(got[b]), recent[b])
    assert got[2] == Vb - 1


def test_graph_replays(model):
    """pn_sample captured in a HIP graph and replayed with new logits and draws
    in the captured buffers: every replay matches the reference sampler and the
    eager call (the histogram scratch is cleared by a kernel, so replays start
    from zero without a memset)."""
    import torch
    from token_decode_amd import device as dv
    rng = np.random.default_rng(10)
    params = [dict(temperature=0.9, top_k=50, top_p=0.9), dict(temperature=1.2, top_k=1000, top_p=0.97)]
    n = len(params)
    lg = torch.zeros(n, V, dtype=torch.float32, device="cuda")
    u = torch.zeros(n, dtype=torch.float32, device="cuda")
    ids = torch.zeros(n, dtype=torch.int32, device="cuda")
    dv.sample(model, lg, params, u, ids)  # eager warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dv.sample(model, lg, params, u, ids)
    for rep in range(4):
        rows = [(rng.standard_normal(V) * (1.0 + rep)).astype(np.float32) for _ in range(n)]
        us = [float(x) for x in rng.random(n)]
        lg.copy_(torch.from_numpy(np.stack(rows)))
        u.copy_(torch.tensor(us, dtype=torch.float32))
        g.replay()
        torch.cuda.synchronize()
        got = ids.cpu().numpy().copy()
        eager = run(model, rows, params, us)  # eager work between the replays
        np.testing.assert_array_equal(got, eager)
        for b in range(n):
            check(rows[b], params[b], us[b], int(got[b]))
    log("  4 graph replays of pn_sample: equal to the eager calls and to the reference sampler")
