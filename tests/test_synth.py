"""The seeded input generator: determinism, addressability, distributions, INT8 rule."""
import numpy as np

import synth


def test_stream_is_splitmix64_element():
    # element c of the stream is mix(key + (c+1)*gamma) with key = mix(seed + gamma)
    M = (1 << 64) - 1

    def mix(z):
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M
        return z ^ (z >> 31)

    g = 0x9E3779B97F4A7C15
    for seed in (0, 1, 5, 123456789):
        key = mix((seed + g) & M)
        for c in (0, 1, 2, 1 << 41, (7 << 41) + 99):
            assert synth.lib().synth_draw_u64(seed, c) == mix((key + (c + 1) * g) & M)


def test_normal_deterministic_and_addressable():
    a = synth.normal(7, 3, 10001, 0.0, 1.0, synth.F32)
    b = synth.normal(7, 3, 10001, 0.0, 1.0, synth.F32, threads=1)
    np.testing.assert_array_equal(a, b)
    part = synth.normal(7, 3, 777, 0.0, 1.0, synth.F32, start=4321)
    np.testing.assert_array_equal(part, a[4321:4321 + 777])
    c = synth.normal(8, 3, 10001, 0.0, 1.0, synth.F32)
    assert not np.array_equal(a, c)
    d = synth.normal(7, 4, 10001, 0.0, 1.0, synth.F32)
    assert not np.array_equal(a, d)


def test_normal_moments():
    x = synth.normal(1, 11, 1 << 20, 0.0, 0.02, synth.F32).astype(np.float64)
    assert abs(x.mean()) < 0.02 * 5 / 1024
    assert abs(x.std() / 0.02 - 1) < 0.005
    # fourth standardized moment of a normal is 3
    assert abs(((x / x.std()) ** 4).mean() - 3.0) < 0.05
    g = synth.normal(1, 12, 1 << 18, 1.0, 0.1, synth.F32).astype(np.float64)
    assert abs(g.mean() - 1.0) < 0.002 and abs(g.std() - 0.1) < 0.002


def test_bf16_storage_is_rounded_fp32_draw():
    f = synth.normal(3, 5, 50000, 0.0, 0.02, synth.F32)
    h = synth.normal(3, 5, 50000, 0.0, 0.02, synth.BF16)
    hv = synth.bf16_to_f32(h).astype(np.float64)
    # within half a bf16 ulp of the (fp32) draw
    ulp = np.exp2(np.floor(np.log2(np.abs(f.astype(np.float64)))) - 7)
    assert np.all(np.abs(hv - f) <= ulp / 2 * (1 + 1e-6))


def test_int8_rows_rule():
    rows, cols = 64, 300
    q, s = synth.int8_rows(2, 9, rows, cols, 0.02)
    w = synth.bf16_to_f32(synth.normal(2, 9, rows * cols, 0.0, 0.02, synth.BF16)).reshape(rows, cols)
    amax = np.abs(w).max(axis=1)
    np.testing.assert_array_equal(s, (amax / np.float32(127.0)).astype(np.float32))
    err = np.abs(w.astype(np.float64) - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) / 2 * (1 + 1e-6))
    assert np.all(np.abs(q).max(axis=1) == 127)
    assert q.min() >= -127 and q.max() <= 127


def test_integer_draws():
    t = synth.uniform_int(4, 1 << 20, 5000, 0, 31999)
    assert t.min() >= 0 and t.max() <= 31999 and len(np.unique(t)) > 4000
    p = synth.distinct_int(4, (1 << 20) + 1, 8, 1024, 16384)
    assert len(set(p.tolist())) == 8 and p.min() >= 1024 and p.max() <= 16384
    p2 = synth.distinct_int(9, 77, 6, 0, 5)
    assert sorted(p2.tolist()) == list(range(6))


def test_workload_positions_and_kv():
    wl = synth.mistral_7b_slots()
    pos = wl.start_positions()
    assert len(set(pos.tolist())) == 8 and pos.min() >= 1024 and pos.max() <= 16384
    wl5 = synth.mixtral_8x7b_slots()
    p5 = wl5.start_positions()
    assert p5.size == 16 and p5.min() >= 512 and p5.max() <= 4096
    small = synth.tiny_fp32().with_(kv_dtype=synth.BF16)
    k, v = small.kv_prefill(0, 1, 5, 3)
    kk, vv = small.kv_prefill(0, 1, 0, 8)
    np.testing.assert_array_equal(k, kk[5:8])
    np.testing.assert_array_equal(v, vv[5:8])
    assert not np.array_equal(k, v)
