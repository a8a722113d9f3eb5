"""Reference token sampler: the pages' sampling steps, applied one after the
other, on the CPU ("Engine Architecture", section "Sampling": temperature,
repetition penalty, top-k, top-p, softmax, multinomial draw).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does.

Readings where the pages leave a step open (each also taken by the HIP
sampler):
- temperature <= 0 is greedy decoding: the argmax of the raw logits (lowest
  index among equal maxima); no other step applies;
- the logits are divided by the temperature in fp32, then every distinct
  token of the recent window is penalised in fp32: z / r if z > 0, else z * r;
  -0 counts as +0 and NaN as -inf;
- the tokens are ranked by z, highest first, equal z by lower index (the
  canonical order); top-k keeps the first k of that order;
- probabilities are exp(z - z_max) over the kept tokens, in fp64 (a token
  whose z equals z_max weighs 1, so all -inf rows draw evenly);
- top-p keeps the shortest prefix of the canonical order whose cumulative
  probability exceeds p times the kept total (p >= 1: all kept tokens);
- the draw takes a uniform u in [0, 1) as an input and returns the first
  token of the prefix whose cumulative probability exceeds u times the
  prefix total.
The ranking decisions are taken on the fp32 values of z, as the GPU takes
them; only the probability sums are fp64.
"""
from __future__ import annotations

import numpy as np


def transformed(logits, temperature, repeat_penalty=1.0, recent=()):
    """z in fp32: logits / temperature, then the repetition penalty on the
    distinct tokens of `recent` (entries < 0 are empty)."""
    z = np.asarray(logits, dtype=np.float32) / np.float32(temperature)
    r = np.float32(repeat_penalty)
    for t in sorted({int(t) for t in recent if int(t) >= 0 and int(t) < len(z)}):
        z[t] = z[t] / r if z[t] > 0 else z[t] * r
    z = np.where(np.isnan(z), np.float32(-np.inf), z).astype(np.float32)
    z[z == 0] = np.float32(0.0)  # -0 -> +0
    return z


def canonical_order(z):
    """Token ids by z descending, equal z by index ascending."""
    idx = np.arange(len(z))
    return np.lexsort((idx, -z.astype(np.float64)))


def sample(logits, temperature, top_k, top_p=1.0, repeat_penalty=1.0, recent=(), u=0.0, detail=False):
    """One sampled token id; with detail, also (ids of the top-p prefix in
    canonical order, their cumulative probabilities, the prefix total)."""
    logits = np.asarray(logits, dtype=np.float32)
    if temperature <= 0:
        lg = np.where(np.isnan(logits), -np.inf, logits)
        tok = int(np.argmax(lg))  # first maximum
        return (tok, np.array([tok]), np.array([1.0]), 1.0) if detail else tok
    z = transformed(logits, temperature, repeat_penalty, recent)
    order = canonical_order(z)[:max(1, int(top_k))]
    zk = z[order].astype(np.float64)
    with np.errstate(invalid="ignore"):
        w = np.where(zk == zk[0], 1.0, np.exp(zk - zk[0]))  # (all -inf: equal weights)
    cum = np.cumsum(w)
    if top_p < 1.0:
        n_p = int(np.argmax(cum > top_p * cum[-1])) + 1 if np.any(cum > top_p * cum[-1]) else len(cum)
    else:
        n_p = len(cum)
    cum_p = cum[:n_p]
    r = u * cum_p[-1]
    hit = np.nonzero(cum_p > r)[0]
    j = int(hit[0]) if len(hit) else n_p - 1
    tok = int(order[j])
    return (tok, order[:n_p], cum_p, float(cum_p[-1])) if detail else tok
