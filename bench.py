"""Decode throughput of the HIP path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--cpu-seconds S]

A step is one whole decode step (embedding, every layer, LM head and greedy
argmax) for every sequence of the workload, with the previous step's argmax
fed back on the device.  Inputs are seeded synthetic weights and K/V of the
workload's shape, resident in HBM before the timed region starts.  Prints one
JSON line with the throughput, the roofline of the dominant kernel (gate/up:
algorithmic bytes over its average launch time, from HIP events around
replays of the timed steps' launches; HBM traffic from the committed counter
summary while the GEMM sources are unchanged) and the fp64 CPU oracle timed
on a bounded sample of the same workload.

The line also reports, outside the timed steps, the time of one on-device
sampling call (pn_sample) over the step's logits and the throughput of a
512-token prompt prefilled on the wide path (pn_prefill in chunks of 256 rows).

--calibrate-copy runs only a 1 GiB device copy, the reference for scaling the
HBM byte counters; --print-source-hash prints the hash the counter summary is
tied to.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


# chunked prefill, timed next to the decode step: rows per wide chunk and prompt length
PREFILL_CHUNK = 256
PREFILL_TOKENS = 512


def wide_ok(wl):
    """Whether the workload can take the wide prefill path (bf16 or int8 weights, dense, fp32 or bf16 cache)."""
    import synth
    return wl.w_dtype in (synth.BF16, synth.I8) and wl.n_expert == 0 and wl.kv_dtype in (synth.F32, synth.BF16)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(wl, positions):
    """Bytes one step must move: every weight matrix read once, the cached K/V of
    each sequence's window read once, the new k/v written, the logits written and
    one embedding row per sequence read.  Activations and scratch (KB-scale,
    cache-resident) are not counted.  Dense models only."""
    E, H, Hk, d, F, V, L = (wl.n_embd, wl.n_head, wl.n_kv_head, wl.head_dim, wl.n_ff,
                            wl.n_vocab, wl.n_layer)
    # Q8_0 / Q4_0: 34 / 18 bytes per 32 weights (codes + fp16 scale)
    sw = {0: 4, 1: 2, 2: 1, 3: 34 / 32, 4: 18 / 32}[wl.w_dtype]
    skv = {0: 4, 1: 2, 4: 9 / 16}[wl.kv_dtype]  # Q4 cache: codes and a 2-byte scale per 32 dims
    se = 4 if wl.w_dtype == 0 else 2
    per_layer_w = (H * d * E + 2 * Hk * d * E + E * H * d + 3 * E * F) * sw
    rows_layer = H * d + 2 * Hk * d + E + 2 * F + E
    scales = (rows_layer * L + V) * 4 if wl.w_dtype == 2 else 0
    weights = L * per_layer_w + V * E * sw + scales + (2 * L + 1) * E * 4
    kv = 0
    for p in positions:
        keys = min(p + 1, wl.sliding_window) if wl.sliding_window > 0 else p + 1
        kv += L * 2 * Hk * d * skv * (keys + 1)  # read the window, write the new k, v
    out = len(positions) * (4 * V + E * se)
    return weights + kv + out


def gemm_bytes(wl, kind):
    """Algorithmic bytes of one launch of a GEMM kernel class (weights + scales)."""
    E, H, Hk, d, F, V = wl.n_embd, wl.n_head, wl.n_kv_head, wl.head_dim, wl.n_ff, wl.n_vocab
    sw = {0: 4, 1: 2, 2: 1, 3: 34 / 32, 4: 18 / 32}[wl.w_dtype]
    sc = 4 if wl.w_dtype == 2 else 0
    rows, cols = {"qkv": ((H + 2 * Hk) * d, E), "o": (E, H * d), "gateup": (2 * F, E),
                  "down": (E, F), "lmhead": (V, E)}[kind]
    return rows * cols * sw + rows * sc


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="llama3-8b-bf16")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="rough budget of the CPU-oracle baseline sample (0 = skip)")
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

    import synth
    from token_decode_amd import _capi as C
    from token_decode_amd import device as dv

    wl = synth.WORKLOADS[args.workload]()
    if wl.n_expert > 0:
        raise SystemExit("bench.py times dense workloads")
    torch.cuda.set_device(0)
    dev = torch.cuda.current_device()
    t0 = time.time()
    W = synth.make_weights(wl)
    log("weights drawn in %.1fs" % (time.time() - t0))
    cfg = dv.make_config(wl.n_layer, wl.n_embd, wl.n_head, wl.n_kv_head, wl.head_dim, wl.n_ff,
                         wl.n_vocab, n_expert=wl.n_expert, n_expert_used=wl.n_expert_used,
                         sliding_window=wl.sliding_window, max_batch=wl.slots,
                         rope_theta=wl.rope_theta, rms_norm_eps=wl.rms_norm_eps,
                         w_dtype=wl.w_dtype, kv_dtype=wl.kv_dtype, act_dtype=wl.act_dtype,
                         prefill_chunk=PREFILL_CHUNK if wide_ok(wl) else 0)
    t0 = time.time()
    model = dv.DeviceModel(cfg, W)
    log("model packed in %.1fs (%.2f GB)" % (time.time() - t0, model.nbytes / 1e9))

    B = wl.slots
    starts = [int(p) for p in wl.start_positions()]
    total_steps = args.warmup + args.steps
    states = []
    t0 = time.time()
    for b in range(B):
        st = dv.DeviceState(model, starts[b] + total_steps + 1)
        lo = wl.kv_window_start(starts[b]) if starts[b] > 0 else 0
        for l in range(wl.n_layer):
            k, v = wl.kv_prefill(b, l, lo, starts[b] - lo)
            st.set_kv(l, lo, k, v)
        st.pos = starts[b]
        states.append(st)
    log("KV prefilled in %.1fs" % (time.time() - t0))

    stream = torch.cuda.current_stream()
    ids = torch.tensor([int(t) for t in wl.first_tokens()], dtype=torch.int32, device="cuda")
    logits = torch.empty(B, wl.n_vocab, dtype=torch.float32, device="cuda")

    def step():
        if B == 1:
            dv.forward_step(model, states[0], ids, logits, ids)
        else:
            dv.forward_batch(model, states, ids, logits, ids)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    pos_timed = [st.pos for st in states]
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    ms_step = ms / args.steps
    tok_s = B * args.steps / (ms / 1e3)
    step_bytes = np.mean([algorithmic_bytes(wl, [p + i for p in pos_timed])
                          for i in range(args.steps)])
    gbs = step_bytes / (ms_step / 1e3) / 1e9
    log("step %.3f ms, %.1f tok/s, %.1f GB/s (%.1f%% of 8 TB/s)" % (ms_step, tok_s, gbs,
                                                                   100 * gbs / HBM_PEAK_GBS))

    # per-kernel-class timing: HIP events on the launch stream around back-to-back
    # replays of the class's launches in the last timed step (every layer's, in
    # order, with the step's arguments)
    kinds = {"qkv": C.PN_K_QKV, "attn": C.PN_K_ATTN, "o": C.PN_K_O, "gateup": C.PN_K_GATEUP,
             "down": C.PN_K_DOWN, "lmhead": C.PN_K_LMHEAD}
    per_kernel = {}
    for name, k in kinds.items():
        reps = 64 if name == "lmhead" else 8 * wl.n_layer
        model.profile_replay(k, 2, stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        model.profile_replay(k, reps, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        per_kernel[name] = {"avg_us": round(1e3 * e0.elapsed_time(e1) / reps, 3), "replays": reps}
    # on-device sampling of the step's logits (pn_sample), for the record: one
    # call per step over every slot's row
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
    sample_us = round(1e3 * e0.elapsed_time(e1) / 64, 2)
    # chunked prefill on the wide path (pn_prefill), for the record: a
    # 512-token prompt from position 0 into a fresh state, greedy ids only
    prefill = None
    if wide_ok(wl):
        n_p = PREFILL_TOKENS
        pst = dv.DeviceState(model, n_p + 8)
        ptok = torch.from_numpy(synth.uniform_int(wl.seed, 99, n_p, 0, wl.n_vocab - 1).astype("int32")).cuda()
        pam = torch.empty(n_p, dtype=torch.int32, device="cuda")
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
        mm = wl.n_layer * (wl.n_embd * (wl.n_head + 2 * wl.n_kv_head) * wl.head_dim +
                           wl.n_head * wl.head_dim * wl.n_embd + 3 * wl.n_embd * wl.n_ff) + wl.n_vocab * wl.n_embd
        prefill = {"tokens_per_s": round(n_p / p_ms * 1e3, 1), "tokens": n_p, "chunk": PREFILL_CHUNK,
                   "ms": round(p_ms, 3),
                   "matrix_core_tflops": round(2.0 * mm * n_p * pieces / (p_ms * 1e-3) / 1e12, 1),
                   "bf16_pieces_per_input": pieces}
        pst.free()
        log("prefill: %d tokens in %.2f ms = %.0f tokens/s" % (n_p, p_ms, n_p / p_ms * 1e3))
    dom = "gateup"
    dom_bytes = gemm_bytes(wl, dom)
    dom_us = per_kernel[dom]["avg_us"]
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    for name in ("qkv", "o", "gateup", "down", "lmhead"):
        bb = gemm_bytes(wl, name)
        per_kernel[name]["GBps"] = round(bb / (per_kernel[name]["avg_us"] * 1e-6) / 1e9, 1)
    log("per kernel: " + json.dumps(per_kernel))
    traffic = measured_traffic(wl.name)

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(wl, W, starts, args.cpu_seconds)

    rec = {
        "metric": "decode tokens/sec (batch %d); achieved HBM GB/s vs peak" % B,
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {0: "f32", 1: "bf16", 2: "int8", 3: "q8_0", 4: "q4_0"}[wl.w_dtype] + "-weights/" +
                 {0: "f32", 1: "bf16"}[wl.act_dtype] + "-act",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) cached K/V)",
        "config": {"workload": wl.name, "n_layer": wl.n_layer, "n_embd": wl.n_embd,
                   "n_head": wl.n_head, "n_kv_head": wl.n_kv_head, "n_ff": wl.n_ff,
                   "n_vocab": wl.n_vocab, "slots": B, "start_positions": starts[:16],
                   "window": wl.sliding_window},
        "hbm": {"bytes_per_step": int(step_bytes), "GBps": round(gbs, 1),
                "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)},
        "roofline": {"kernel": "gate/up GEMM + SwiGLU", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_us, 3)},
        "kernels": per_kernel,
        "sampling": {"us_per_call": sample_us, "rows": B, "vocab": wl.n_vocab,
                     "params": "temperature 0.8, top_k 40, top_p 0.95, repeat_penalty 1.1 over 64 recent tokens"},
        "prefill": prefill,
        "cpu_baseline": cpu,
    }
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


def cpu_baseline(wl, W, starts, budget_s):
    """The fp64 oracle on the host cores: a bounded sample of decode steps of the
    same workload (first sequence, from its start position)."""
    import oracle
    threads = max(1, min(16, os.cpu_count() or 1))
    om = oracle.Model(wl, W)
    p0 = starts[0]
    st = om.new_state(p0 + 64)
    lo = wl.kv_window_start(p0) if p0 > 0 else 0
    for l in range(wl.n_layer):
        k, v = wl.kv_prefill(0, l, lo, p0 - lo)
        st.set_kv(l, lo, k, v)
    st.pos = p0
    tok = int(wl.first_tokens()[0])
    times = []
    t_start = time.time()
    while len(times) < 2 or (time.time() - t_start < budget_s and len(times) < 32):
        t = time.time()
        _, tok = st.step(tok, threads=threads)
        times.append(time.time() - t)
    med = float(np.median(times))
    log("cpu oracle: %d steps, median %.3f s/step on %d threads" % (len(times), med, threads))
    return {"value": round(1.0 / med, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d decode steps of %s (sequence 0 from position %d), median step time"
                      % (len(times), wl.name, p0)}


if __name__ == "__main__":
    main()
