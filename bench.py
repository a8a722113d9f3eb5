"""Decode throughput of the HIP path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--cpu-seconds S]

A step is one whole decode step (embedding, every layer, LM head and greedy
argmax) for every sequence of the workload, with the previous step's argmax
fed back on the device.  Inputs are seeded synthetic weights and K/V of the
workload's shape, resident in HBM before the timed region starts.

By default the line covers both halves of the metric: batch 1 on the
Llama-3-8B bf16 workload (the headline `value`), and 8 slots on the
Mistral-7B workload (the `slots8` record, same fields).  Each carries its
tokens/s, achieved HBM GB/s against the 8 TB/s peak and against a measured
streaming-read ceiling, the roofline of its dominant kernel (gate/up:
algorithmic bytes over its average launch time, from HIP events around
replays of the timed steps' launches on the launch stream; HBM traffic from
the committed counter summary while the GEMM sources are unchanged), per
kernel-class times, and the fp64 CPU oracle timed on a bounded sample of the
same workload (all host threads of the GPU's share, and one thread).

`--workload NAME` times one workload alone (any of synth.WORKLOADS, including
the Mixtral MoE one, whose bytes per step count the experts each step's
routing actually touched, read from the library's routing log).

The headline also reports, outside the timed steps, the time of one
on-device sampling call (pn_sample) and the throughput of a 512-token prompt
prefilled on the wide path (pn_prefill in chunks of 256 rows).

--calibrate-copy runs only a 1 GiB device copy, the reference for scaling the
HBM byte counters; --print-source-hash prints the hash the counter summary is
tied to.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
HEADLINE = "llama3-8b-bf16"
SLOTS8 = "mistral-7b-8slots"

# chunked prefill, timed next to the decode step: rows per wide chunk and prompt length
PREFILL_CHUNK = 256
PREFILL_TOKENS = 512


def wide_ok(wl):
    """Whether the workload can take the wide prefill path (bf16, int8, Q8_0 or Q4_0 weights,
    fp32 or bf16 cache; dense or experts)."""
    import synth
    return (wl.w_dtype in (synth.BF16, synth.I8, synth.Q8_0, synth.Q4_0) and
            wl.kv_dtype in (synth.F32, synth.BF16))


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _elem_sizes(wl):
    sw = {0: 4, 1: 2, 2: 1, 3: 34 / 32, 4: 18 / 32}[wl.w_dtype]  # Q8_0 / Q4_0: codes + fp16 scale per 32
    skv = {0: 4, 1: 2, 4: 9 / 16}[wl.kv_dtype]  # Q4 cache: codes and a 2-byte scale per 32 dims
    se = 4 if wl.w_dtype == 0 else 2
    return sw, skv, se


def algorithmic_bytes(wl, positions, experts_touched=None):
    """Bytes one step must move: every weight matrix read once, the cached K/V of
    each sequence's window read once, the new k/v written, the logits written and
    one embedding row per sequence read.  Activations and scratch (KB-scale,
    cache-resident) are not counted.  For an MoE model, `experts_touched[l]` is
    the number of distinct experts that layer l's routing chose for at least one
    row of the step: only those experts' FFN weights are read."""
    E, H, Hk, d, F, V, L = (wl.n_embd, wl.n_head, wl.n_kv_head, wl.head_dim, wl.n_ff,
                            wl.n_vocab, wl.n_layer)
    sw, skv, se = _elem_sizes(wl)
    attn_layer = (H * d * E + 2 * Hk * d * E + E * H * d) * sw
    ffn_expert = 3 * E * F * sw
    scale_rows_attn = H * d + 2 * Hk * d + E
    scale_rows_ffn = 2 * F + E
    i8 = 4 if wl.w_dtype == 2 else 0
    if wl.n_expert > 0:
        assert experts_touched is not None and len(experts_touched) == L
        ffn = sum(int(n) * (ffn_expert + scale_rows_ffn * i8) for n in experts_touched)
        router = L * wl.n_expert * E * se
    else:
        ffn = L * (ffn_expert + scale_rows_ffn * i8)
        router = 0
    weights = L * (attn_layer + scale_rows_attn * i8) + ffn + router + V * E * sw + V * i8 + (2 * L + 1) * E * 4
    kv = 0
    for p in (int(q) for q in positions):
        keys = min(p + 1, wl.sliding_window) if wl.sliding_window > 0 else p + 1
        kv += L * 2 * Hk * d * skv * (keys + 1)  # read the window, write the new k, v
    out = len(positions) * (4 * V + E * se)
    return weights + kv + out


def gemm_bytes(wl, kind):
    """Algorithmic bytes of one launch of a GEMM kernel class (weights + scales)."""
    E, H, Hk, d, F, V = wl.n_embd, wl.n_head, wl.n_kv_head, wl.head_dim, wl.n_ff, wl.n_vocab
    sw = _elem_sizes(wl)[0]
    sc = 4 if wl.w_dtype == 2 else 0
    rows, cols = {"qkv": ((H + 2 * Hk) * d, E), "o": (E, H * d), "gateup": (2 * F, E),
                  "down": (E, F), "lmhead": (V, E)}[kind]
    return rows * cols * sw + rows * sc


def cpu_facts():
    """The host the oracle baseline runs on: CPU model, logical CPUs, and the
    threads this process may use (its affinity; the oracle uses at most 16,
    the host share of one GPU)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": os.cpu_count() or 1, "affinity": aff,
            "threads": max(1, min(16, aff))}


def stream_ceiling(nbytes=4 << 30, reps=10):
    """GB/s of the library's plain streaming read (pn_stream_read) over a 4 GiB
    buffer: the read ceiling the step's HBM rates are set against."""
    import torch
    from token_decode_amd import _capi as C
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    L = C.lib()
    for _ in range(3):
        C.check(L.pn_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()), sp))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        C.check(L.pn_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()), sp))
    e1.record(stream)
    torch.cuda.synchronize()
    gbs = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf
    torch.cuda.empty_cache()
    log("streaming read ceiling: %.1f GB/s (%.1f%% of 8 TB/s)" % (gbs, 100 * gbs / HBM_PEAK_GBS))
    return round(gbs, 1)


def run_workload(name, steps, warmup, cpu_seconds, ceiling, extras=False):
    """Draw, pack, prefill and time one workload; returns its record."""
    import torch

    import synth
    from token_decode_amd import _capi as C
    from token_decode_amd import device as dv

    wl = synth.WORKLOADS[name]()
    moe = wl.n_expert > 0
    torch.cuda.set_device(0)
    t0 = time.time()
    W = synth.make_weights(wl)
    log("[%s] weights drawn in %.1fs" % (name, time.time() - t0))
    cfg = dv.make_config(wl.n_layer, wl.n_embd, wl.n_head, wl.n_kv_head, wl.head_dim, wl.n_ff,
                         wl.n_vocab, n_expert=wl.n_expert, n_expert_used=wl.n_expert_used,
                         sliding_window=wl.sliding_window, max_batch=wl.slots,
                         rope_theta=wl.rope_theta, rms_norm_eps=wl.rms_norm_eps,
                         w_dtype=wl.w_dtype, kv_dtype=wl.kv_dtype, act_dtype=wl.act_dtype,
                         prefill_chunk=PREFILL_CHUNK if (extras and wide_ok(wl)) else 0)
    t0 = time.time()
    model = dv.DeviceModel(cfg, W)
    log("[%s] model packed in %.1fs (%.2f GB)" % (name, time.time() - t0, model.nbytes / 1e9))

    B = wl.slots
    starts = [int(p) for p in wl.start_positions()]
    total_steps = warmup + steps
    states = []
    t0 = time.time()
    for b in range(B):
        st = dv.DeviceState(model, starts[b] + total_steps + 16)  # + the MoE roofline's untimed steps
        lo = wl.kv_window_start(starts[b]) if starts[b] > 0 else 0
        for l in range(wl.n_layer):
            k, v = wl.kv_prefill(b, l, lo, starts[b] - lo)
            st.set_kv(l, lo, k, v)
        st.pos = starts[b]
        states.append(st)
    log("[%s] KV prefilled in %.1fs" % (name, time.time() - t0))

    stream = torch.cuda.current_stream()
    ids = torch.tensor([int(t) for t in wl.first_tokens()], dtype=torch.int32, device="cuda")
    logits = torch.empty(B, wl.n_vocab, dtype=torch.float32, device="cuda")

    def step():
        if B == 1:
            dv.forward_step(model, states[0], ids, logits, ids)
        else:
            dv.forward_batch(model, states, ids, logits, ids)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    route_log = None
    if moe:
        # the routing of every timed step, written by the router kernels themselves
        route_log = torch.full((steps, wl.n_layer, B, wl.n_expert_used), -1, dtype=torch.int32, device="cuda")
        C.check(C.lib().pn_model_route_log(model.h, ctypes.c_void_p(route_log.data_ptr()), steps))
    pos_timed = [st.pos for st in states]
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    ms_step = ms / steps
    tok_s = B * steps / (ms / 1e3)
    touched = None
    if moe:
        C.check(C.lib().pn_model_route_log(model.h, None, 0))
        rl = route_log.cpu().numpy()
        assert (rl >= 0).all() and (rl < wl.n_expert).all(), "routing log incomplete"
        touched = [[len(np.unique(rl[i, l])) for l in range(wl.n_layer)] for i in range(steps)]
    step_bytes = float(np.mean([algorithmic_bytes(wl, [p + i for p in pos_timed],
                                                  touched[i] if touched else None) for i in range(steps)]))
    gbs = step_bytes / (ms_step / 1e3) / 1e9
    log("[%s] step %.3f ms, %.1f tok/s, %.1f GB/s (%.1f%% of 8 TB/s)" % (name, ms_step, tok_s, gbs,
                                                                        100 * gbs / HBM_PEAK_GBS))

    # per-kernel-class timing: HIP events on the launch stream around back-to-back
    # replays of the class's launches in the last timed step (every layer's, in
    # order, with the step's arguments)
    kinds = {"qkv": C.PN_K_QKV, "attn": C.PN_K_ATTN, "o": C.PN_K_O, "lmhead": C.PN_K_LMHEAD}
    if not moe:
        kinds.update({"gateup": C.PN_K_GATEUP, "down": C.PN_K_DOWN})
    per_kernel = {}
    for kname, k in kinds.items():
        reps = 64 if kname == "lmhead" else 8 * wl.n_layer
        model.profile_replay(k, 2, stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        model.profile_replay(k, reps, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        per_kernel[kname] = {"avg_us": round(1e3 * e0.elapsed_time(e1) / reps, 3), "replays": reps}
    for kname in ("qkv", "o", "gateup", "down", "lmhead"):
        if kname in per_kernel:
            bb = gemm_bytes(wl, kname)
            per_kernel[kname]["GBps"] = round(bb / (per_kernel[kname]["avg_us"] * 1e-6) / 1e9, 1)
    log("[%s] per kernel: %s" % (name, json.dumps(per_kernel)))

    rec = {
        "workload": wl.name,
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "dtype": {0: "f32", 1: "bf16", 2: "int8", 3: "q8_0", 4: "q4_0"}[wl.w_dtype] + "-weights/" +
                 {0: "f32", 1: "bf16"}[wl.act_dtype] + "-act",
        "config": {"workload": wl.name, "n_layer": wl.n_layer, "n_embd": wl.n_embd,
                   "n_head": wl.n_head, "n_kv_head": wl.n_kv_head, "n_ff": wl.n_ff,
                   "n_vocab": wl.n_vocab, "n_expert": wl.n_expert, "n_expert_used": wl.n_expert_used,
                   "slots": B, "start_positions": starts[:16], "window": wl.sliding_window},
        "hbm": {"bytes_per_step": int(step_bytes), "GBps": round(gbs, 1),
                "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                "stream_ceiling_GBps": ceiling,
                "frac_of_ceiling": round(gbs / ceiling, 4) if ceiling else None},
        "kernels": per_kernel,
    }
    if moe:
        tt = np.array(touched)
        rec["hbm"]["experts_touched_per_layer_mean"] = round(float(tt.mean()), 3)
    if not moe:
        dom = "gateup"
        dom_bytes = gemm_bytes(wl, dom)
        dom_us = per_kernel[dom]["avg_us"]
        achieved = dom_bytes / (dom_us * 1e-6) / 1e9
        rec["roofline"] = {"kernel": "gate/up GEMM + SwiGLU", "bound": "hbm", "achieved": round(achieved, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                           "traffic": measured_traffic(wl.name), "bytes_per_launch": dom_bytes,
                           "avg_launch_us": round(dom_us, 3)}
    else:
        # the expert GEMMs of a layer read the touched experts' weights; timed as
        # one class with pn_profile over a few untimed steps
        rec["roofline"] = moe_roofline(model, wl, step, stream)

    if extras:
        rec["sampling"] = time_sampling(model, wl, logits, stream)
        rec["prefill"] = time_prefill(model, wl, stream) if wide_ok(wl) else None
    if cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline(wl, W, starts, cpu_seconds, one_thread=extras)
    for st in states:
        st.free()
    del states, model, W
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def moe_roofline(model, wl, step, stream, n_steps=4):
    """Expert gate/up and down launches of a few untimed steps, timed with the
    library's per-launch events (pn_profile_begin/end), against the bytes of the
    experts those launches read (from the routing log of the same steps)."""
    import torch
    from token_decode_amd import _capi as C
    sw = _elem_sizes(wl)[0]
    out = {}
    for kname, k, mats in (("moe_gateup", C.PN_K_MOE_GATEUP, 2), ("moe_down", C.PN_K_MOE_DOWN, 1)):
        log_t = torch.full((n_steps, wl.n_layer, wl.slots, wl.n_expert_used), -1, dtype=torch.int32, device="cuda")
        C.check(C.lib().pn_model_route_log(model.h, ctypes.c_void_p(log_t.data_ptr()), n_steps))
        model.profile_begin(k)
        for _ in range(n_steps):
            step()
        ms, n = model.profile_end(stream)
        C.check(C.lib().pn_model_route_log(model.h, None, 0))
        rl = log_t.cpu().numpy()
        touched = sum(len(np.unique(rl[i, l])) for i in range(n_steps) for l in range(wl.n_layer))
        nbytes = touched * mats * wl.n_ff * wl.n_embd * sw
        out[kname] = (nbytes, ms, n, touched)
    gu_bytes, ms_gu, n_gu, touched = out["moe_gateup"]
    dn_bytes, ms_dn, n_dn, _ = out["moe_down"]
    achieved = gu_bytes / (ms_gu * 1e-3) / 1e9
    return {"kernel": "expert gate/up GEMM + SwiGLU", "bound": "hbm", "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
            "bytes_per_launch": int(gu_bytes / max(1, n_gu)), "avg_launch_us": round(1e3 * ms_gu / max(1, n_gu), 3),
            "expert_down_GBps": round(dn_bytes / (ms_dn * 1e-3) / 1e9, 1),
            "experts_touched_per_layer": round(touched / (n_steps * wl.n_layer), 3)}


def time_sampling(model, wl, logits, stream):
    """One on-device sampling call (pn_sample) over every slot's row, for the record."""
    import torch
    from token_decode_amd import device as dv
    B = wl.slots
    sp = [dict(temperature=0.8, top_k=40, top_p=0.95, repeat_penalty=1.1)] * B
    u_dev = torch.full((B,), 0.5, dtype=torch.float32, device="cuda")
    s_ids = torch.empty(B, dtype=torch.int32, device="cuda")
    s_recent = torch.zeros((B, 64), dtype=torch.int32, device="cuda")
    for _ in range(4):
        dv.sample(model, logits, sp, u_dev, s_ids, s_recent, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(64):
        dv.sample(model, logits, sp, u_dev, s_ids, s_recent, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    return {"us_per_call": round(1e3 * e0.elapsed_time(e1) / 64, 2), "rows": B, "vocab": wl.n_vocab,
            "params": "temperature 0.8, top_k 40, top_p 0.95, repeat_penalty 1.1 over 64 recent tokens"}


def time_prefill(model, wl, stream):
    """Chunked prefill on the wide path (pn_prefill), for the record: a 512-token
    prompt from position 0 into a fresh state, greedy ids only."""
    import torch

    import synth
    from token_decode_amd import device as dv
    n_p = PREFILL_TOKENS
    pst = dv.DeviceState(model, n_p + 8)
    ptok = torch.from_numpy(synth.uniform_int(wl.seed, 99, n_p, 0, wl.n_vocab - 1).astype("int32")).cuda()
    pam = torch.empty(n_p, dtype=torch.int32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    runs = []
    for i in range(3):
        pst.pos = 0
        e0.record(stream)
        dv.prefill(model, pst, ptok, None, pam, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        if i:
            runs.append(e0.elapsed_time(e1))
    p_ms = sum(runs) / len(runs)
    pieces = 3 if wl.act_dtype == synth.F32 else 1
    # multiply-adds per token: attention projections, the FFN of each expert a token is routed
    # to (one for a dense model), the LM head
    ffn_per_token = 3 * wl.n_embd * wl.n_ff * (wl.n_expert_used if wl.n_expert > 0 else 1)
    mm = wl.n_layer * (wl.n_embd * (wl.n_head + 2 * wl.n_kv_head) * wl.head_dim +
                       wl.n_head * wl.head_dim * wl.n_embd + ffn_per_token) + wl.n_vocab * wl.n_embd
    pst.free()
    log("[%s] prefill: %d tokens in %.2f ms = %.0f tokens/s" % (wl.name, n_p, p_ms, n_p / p_ms * 1e3))
    return {"tokens_per_s": round(n_p / p_ms * 1e3, 1), "tokens": n_p, "chunk": PREFILL_CHUNK,
            "ms": round(p_ms, 3), "matrix_core_tflops": round(2.0 * mm * n_p * pieces / (p_ms * 1e-3) / 1e12, 1),
            "bf16_pieces_per_input": pieces}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default=None,
                    help="time this workload alone (default: %s, then %s as the slots8 record)" % (HEADLINE, SLOTS8))
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="rough budget of each CPU-oracle baseline sample (0 = skip)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (the scale of the HBM byte counters)")
    ap.add_argument("--print-source-hash", action="store_true",
                    help="print the hash of the GEMM sources the counter summary is tied to")
    args = ap.parse_args()
    if args.print_source_hash:
        print(kernel_source_hash())
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        calibrate_copy()
        return
    torch.cuda.set_device(0)
    ceiling = stream_ceiling()
    cpu = cpu_facts()
    log("host: %s, nproc %d, affinity %d" % (cpu["cpu_model"], cpu["nproc"], cpu["affinity"]))

    if args.workload:
        head = run_workload(args.workload, args.steps, args.warmup, args.cpu_seconds, ceiling, extras=True)
        slots8 = None
    else:
        head = run_workload(HEADLINE, args.steps, args.warmup, args.cpu_seconds, ceiling, extras=True)
        slots8 = run_workload(SLOTS8, args.steps, args.warmup, args.cpu_seconds, ceiling)
    B = head["config"]["slots"]
    rec = {
        "metric": "decode tokens/sec at batch 1 and 8 slots; achieved HBM GB/s vs peak",
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) cached K/V)",
        "config": dict(head["config"], batch=B),
        "hbm": head["hbm"],
        "roofline": head["roofline"],
        "kernels": head["kernels"],
        "sampling": head.get("sampling"),
        "prefill": head.get("prefill"),
        "cpu_baseline": head.get("cpu_baseline"),
        "host": cpu,
    }
    if slots8 is not None:
        rec["slots8"] = slots8
    print(json.dumps(rec), flush=True)


GEMM_SOURCES = ("token_decode_amd/csrc/pn_kernels.hpp", "token_decode_amd/csrc/pn_gemm.hip")
COUNTERS = os.path.join(ROOT, "profiles", "gateup_llama3-8b-bf16_counters.md")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per gate/up launch from the committed counter summary (FETCH_SIZE
    + WRITE_SIZE, each scaled by the same counter on a copy of known size), or
    None when the summary is missing, is for another workload, or was taken on
    GEMM sources that have changed since."""
    try:
        with open(COUNTERS) as fh:
            kv = dict(l.strip("- \n").split(": ", 1) for l in fh if l.startswith("- ") and ": " in l)
    except OSError:
        return None
    if kv.get("workload") != workload or kv.get("kernel sources sha256/16") != kernel_source_hash():
        return None
    try:
        return int(kv["traffic bytes per launch"])
    except (KeyError, ValueError):
        return None


def calibrate_copy(nbytes=1 << 30, reps=5):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps}), flush=True)


def cpu_baseline(wl, W, starts, budget_s, one_thread=False):
    """The fp64 oracle on the host cores: a bounded sample of decode steps of the
    same workload.  Batch 1: sequence 0 from its start position, steps until the
    budget; batched: whole batched steps (every slot one oracle step), at most 4.
    With one_thread, also one step on a single thread."""
    import oracle
    facts = cpu_facts()
    threads = facts["threads"]
    om = oracle.Model(wl, W)
    B = len(starts)
    sts = []
    for b in range(B):
        p0 = starts[b]
        st = om.new_state(p0 + 64)
        lo = wl.kv_window_start(p0) if p0 > 0 else 0
        for l in range(wl.n_layer):
            k, v = wl.kv_prefill(b, l, lo, p0 - lo)
            st.set_kv(l, lo, k, v)
        st.pos = p0
        sts.append(st)
    toks = [int(t) for t in wl.first_tokens()]
    times = []
    t_start = time.time()
    cap = 32 if B == 1 else 4
    while len(times) < 2 or (time.time() - t_start < budget_s and len(times) < cap):
        t = time.time()
        for b in range(B):
            _, toks[b] = sts[b].step(toks[b], threads=threads)
        times.append(time.time() - t)
    med = float(np.median(times))
    log("[%s] cpu oracle: %d %s, median %.3f s on %d threads" % (wl.name, len(times),
                                                                   "steps" if B == 1 else "batched steps", med,
                                                                   threads))
    out = {"value": round(B / med, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": "%d %s of %s (%s), median time per step; fp64, %d threads" % (
               len(times), "decode steps" if B == 1 else "batched steps (every slot one oracle step)",
               wl.name, "sequence 0 from position %d" % starts[0] if B == 1 else "%d slots" % B, threads),
           "cpu_model": facts["cpu_model"], "nproc": facts["nproc"],
           "GBps": round(algorithmic_bytes(wl, starts) / med / 1e9, 2) if wl.n_expert == 0 else None}
    if one_thread:
        t = time.time()
        _, _ = sts[0].step(toks[0], threads=1)
        t1 = time.time() - t
        out["one_thread"] = {"value": round(1.0 / t1, 4), "unit": "tokens/s", "sample": "1 decode step, 1 thread"}
        log("[%s] cpu oracle, 1 thread: %.2f s per step" % (wl.name, t1))
    return out


if __name__ == "__main__":
    main()
