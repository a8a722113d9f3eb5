"""pn_sample_noalloc, the sampler for callers that cannot allocate (its scratch
is a file-scope device array), against pn_sample (scratch in the model
buffer): the same ids on the same logits, parameters and draws, over two
calls in a row, the second with fewer rows and a smaller vocabulary."""
import ctypes

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _params(n, rng):
    from token_decode_amd import _capi as C
    arr = (C.pn_sampling_params * n)()
    kinds = [(0.0, 1.0, 40, 1.0), (0.8, 1.1, 40, 0.95), (1.0, 1.0, 1, 1.0), (1.3, 1.0, 4096, 1.0),
             (0.7, 1.3, 200, 0.5), (1.0, 1.0, 1000, 0.99)]
    for i in range(n):
        t, r, k, p = kinds[i % len(kinds)]
        arr[i].temperature, arr[i].repeat_penalty, arr[i].top_k, arr[i].top_p = t, r, k, p
    return arr


def _case(n, V, seed):
    """A model of vocabulary V (its scratch serves pn_sample) and n rows of logits."""
    import torch
    from token_decode_amd import device as dv
    wl = synth.tiny_fp32().with_(name="noalloc-%d" % V, n_layer=1, n_vocab=V, seed=seed)
    cfg = dv.make_config(wl.n_layer, wl.n_embd, wl.n_head, wl.n_kv_head, wl.head_dim, wl.n_ff, V,
                         max_batch=16, w_dtype=synth.F32, kv_dtype=synth.F32, act_dtype=synth.F32)
    model = dv.DeviceModel(cfg, synth.make_weights(wl))
    rng = np.random.default_rng(seed)
    logits = torch.from_numpy((rng.standard_normal((n, V)) * 3).astype(np.float32)).cuda()
    logits[0, 7] = logits[0].max() + 1  # a clear greedy winner in row 0
    u = torch.from_numpy(rng.random(n).astype(np.float32)).cuda()
    recent = torch.from_numpy(rng.integers(-5, V + 5, (n, 32)).astype(np.int32)).cuda()
    return model, logits, u, recent, _params(n, rng)


def test_noalloc_sampler_matches_model_sampler():
    import torch
    from token_decode_amd import _capi as C
    L = C.lib()
    f = L.pn_sample_noalloc
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for n, V, seed in ((12, 50000, 1), (3, 1000, 2)):  # the second call: fewer rows, smaller vocabulary
        model, logits, u, recent, params = _case(n, V, seed)
        ids_a = torch.full((n,), -1, dtype=torch.int32, device="cuda")
        ids_b = torch.full((n,), -2, dtype=torch.int32, device="cuda")
        C.check(L.pn_sample(model.h, ctypes.c_void_p(logits.data_ptr()), n, params,
                            ctypes.c_void_p(recent.data_ptr()), 32, ctypes.c_void_p(u.data_ptr()),
                            ctypes.c_void_p(ids_a.data_ptr()), sp))
        C.check(f(ctypes.c_void_p(logits.data_ptr()), n, V, params, ctypes.c_void_p(recent.data_ptr()), 32,
                  ctypes.c_void_p(u.data_ptr()), ctypes.c_void_p(ids_b.data_ptr()), sp))
        torch.cuda.synchronize()
        a, b = ids_a.cpu().numpy(), ids_b.cpu().numpy()
        assert (a >= 0).all() and (a < V).all()
        np.testing.assert_array_equal(a, b)
        assert a[0] == 7
    # sizes past the array's maximum are refused before anything is enqueued
    assert f(ctypes.c_void_p(logits.data_ptr()), 17, V, params, None, 0, ctypes.c_void_p(u.data_ptr()),
             ctypes.c_void_p(ids_b.data_ptr()), sp) == C.PN_EINVAL
    assert f(ctypes.c_void_p(logits.data_ptr()), 1, 262145, params, None, 0, ctypes.c_void_p(u.data_ptr()),
             ctypes.c_void_p(ids_b.data_ptr()), sp) == C.PN_EINVAL
