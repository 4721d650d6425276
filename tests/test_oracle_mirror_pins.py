"""CPU pins of the oracle's exact attention over the fp32 mirror cache.

Page: 9-3 "q8 KV 精度对照实验" -- §1 (the exact baseline: scores of the raw
fp32 q and K, max-subtracted softmax, weighted raw V) and the closing note of
§3 (the write path also keeps every new K/V row in a float cache, so the
quantized and the exact attention coexist).  Each test checks the oracle
against something other than itself: closed forms, a pure-Python brute force
on tiny inputs, and invariants of the blocked layout.  No GPU needed.
"""
import math

import numpy as np
import pytest

import oracle
import workloads

SCALE = workloads.softmax_scale(128)


def f32bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


def mirror(k, v, lens, kv_bs=32, seed=0, spare=2):
    table, nb = workloads.block_table(np.asarray(lens, np.int32), kv_bs, seed, spare_blocks=spare)
    return oracle.build_mirror(k, v, lens, table, nb, kv_bs)


def brute(q, k, v, scale):
    """Attention of one query over rows k, v, written with Python floats and
    math.exp only (independent of the C oracle)."""
    s = [scale * math.fsum(float(a) * float(b) for a, b in zip(q, kr)) for kr in k]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    tot = math.fsum(w)
    return np.array([math.fsum(wi * float(vr[i]) for wi, vr in zip(w, v)) / tot for i in range(len(v[0]))])


def test_seq_len_one_returns_v_row_bitwise():
    # One token: weight 1, sum 1, so the output is that token's fp32 V row.
    rng = np.random.default_rng(31)
    k = rng.standard_normal((2, 1, 2, 128)).astype(np.float32)
    v = rng.standard_normal((2, 1, 2, 128)).astype(np.float32)
    q = rng.standard_normal((2, 4, 128)).astype(np.float32)
    out = oracle.decode_attn_f32(mirror(k, v, np.array([1, 1], np.int32)), q, 4, SCALE)
    for b in range(2):
        for h in range(4):
            np.testing.assert_array_equal(f32bits(out[b, h]), f32bits(v[b, 0, h // 2]))


def test_zero_query_gives_mean_of_values():
    # q = 0: every score is 0, every weight 1: the plain mean of the V rows.
    rng = np.random.default_rng(32)
    n = 91
    k = rng.standard_normal((1, n, 1, 128)).astype(np.float32)
    v = rng.standard_normal((1, n, 1, 128)).astype(np.float32)
    out = oracle.decode_attn_f32(mirror(k, v, np.array([n], np.int32)), np.zeros((1, 1, 128), np.float32), 1,
                                 SCALE)
    want = v[0, :, 0].astype(np.float64).mean(0)
    np.testing.assert_allclose(out[0, 0], want, rtol=2e-7, atol=1e-8)


def test_two_keys_closed_form():
    # Scale chosen so that the two scores differ by exactly ln 3: weights 3/4, 1/4.
    rng = np.random.default_rng(33)
    q = rng.standard_normal((1, 1, 128)).astype(np.float32)
    k = rng.standard_normal((1, 2, 1, 128)).astype(np.float32)
    v = rng.standard_normal((1, 2, 1, 128)).astype(np.float32)
    d = k[0, :, 0].astype(np.float64) @ q[0, 0].astype(np.float64)
    scale = np.float32(math.log(3.0) / (d[0] - d[1]))
    out = oracle.decode_attn_f32(mirror(k, v, np.array([2], np.int32)), q, 1, scale)
    # the oracle uses the fp32 scale; recompute the weights with that exact scale
    r = math.exp(float(scale) * (d[0] - d[1]))
    want = (r * v[0, 0, 0].astype(np.float64) + v[0, 1, 0]) / (r + 1.0)
    assert abs(r - 3.0) < 1e-6
    np.testing.assert_allclose(out[0, 0], want, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("n", [1, 2, 5, 13])
def test_brute_force_tiny(n):
    # Pure-Python attention on tiny inputs, with heavy-tailed values and a
    # large score spread.
    rng = np.random.default_rng(34 + n)
    k = (rng.standard_t(3, (1, n, 1, 128)) * 3).astype(np.float32)
    v = (rng.standard_t(3, (1, n, 1, 128)) * 3).astype(np.float32)
    q = rng.standard_normal((1, 1, 128)).astype(np.float32)
    out = oracle.decode_attn_f32(mirror(k, v, np.array([n], np.int32), kv_bs=8), q, 1, SCALE)
    want = brute(q[0, 0], k[0, :, 0], v[0, :, 0], float(SCALE))
    np.testing.assert_allclose(out[0, 0], want, rtol=1e-6, atol=1e-6 * np.abs(want).max())


def test_one_dominant_key():
    # Every other score more than 104 below the maximum: exp underflows even
    # in double relative terms far below fp32 resolution -> that token's V row.
    rng = np.random.default_rng(35)
    n = 40
    q = np.ones((1, 1, 128), np.float32)
    k = (rng.standard_normal((1, n, 1, 128)) * 0.01).astype(np.float32)
    k[0, 23, 0] = 30.0
    v = rng.standard_normal((1, n, 1, 128)).astype(np.float32)
    out = oracle.decode_attn_f32(mirror(k, v, np.array([n], np.int32)), q, 1, SCALE)
    np.testing.assert_array_equal(f32bits(out[0, 0]), f32bits(v[0, 23, 0]))


def test_convexity_and_gqa_reduction():
    # Head h of nq = nkv * G equals the dense attention over KV head h / G;
    # every output component lies within the V rows' range.
    rng = np.random.default_rng(36)
    lens = np.array([70, 33, 1, 0, 129], np.int32)
    nkv, nq = 2, 8
    k = (rng.standard_normal((5, 129, nkv, 128)) * 2).astype(np.float32)
    v = rng.standard_normal((5, 129, nkv, 128)).astype(np.float32)
    q = rng.standard_normal((5, nq, 128)).astype(np.float32)
    out = oracle.decode_attn_f32(mirror(k, v, lens, seed=3), q, nq, SCALE)
    for b in range(5):
        n = int(lens[b])
        for h in range(nq):
            if n == 0:
                assert np.all(out[b, h] == 0)
                continue
            kh = h // (nq // nkv)
            want = oracle.attend_dense(q[b, h].astype(np.float64), k[b, :n, kh].astype(np.float64),
                                       v[b, :n, kh].astype(np.float64), float(SCALE)).astype(np.float32)
            np.testing.assert_array_equal(out[b, h], want)
            assert np.all(out[b, h] >= v[b, :n, kh].min(0) - 1e-6)
            assert np.all(out[b, h] <= v[b, :n, kh].max(0) + 1e-6)


def test_placement_invariance_kv_bs_and_rows():
    # Block placement and block size change nothing (same values, same order);
    # the row-list form returns the same rows.
    rng = np.random.default_rng(37)
    lens = np.array([200, 65, 9], np.int32)
    k = rng.standard_normal((3, 200, 2, 128)).astype(np.float32)
    v = rng.standard_normal((3, 200, 2, 128)).astype(np.float32)
    q = rng.standard_normal((3, 4, 128)).astype(np.float32)
    outs = [oracle.decode_attn_f32(mirror(k, v, lens, kv_bs=bs, seed=sd, spare=5), q, 4, SCALE)
            for bs, sd in ((32, 1), (32, 2), (8, 3), (64, 4))]
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])
    rows = oracle.decode_attn_f32(mirror(k, v, lens), q, 4, SCALE, rows_bh=[0, 5, 11, 7])
    np.testing.assert_array_equal(rows, outs[0].reshape(12, 128)[[0, 5, 11, 7]])


def test_bad_block_id_is_reported():
    rng = np.random.default_rng(38)
    k = rng.standard_normal((1, 40, 1, 128)).astype(np.float32)
    v = rng.standard_normal((1, 40, 1, 128)).astype(np.float32)
    m = mirror(k, v, np.array([40], np.int32))
    m.block_table[0, 1] = m.num_blocks   # out of range
    with pytest.raises(ValueError):
        oracle.decode_attn_f32(m, np.ones((1, 1, 128), np.float32), 1, SCALE)


def test_precision_gap_against_the_q8_path():
    # "9-3" §3: the exact and the q8 attention differ by quantization alone.
    # Here the q8 path's inputs are the oracle's quantized rows; the exact path
    # gets the same q and the raw rows.  At N(0,1), L = 256, the gap stays
    # below the step-sized bound the page argues for (half the mean K step
    # plus the Q quantization of a 32-block max/127), and above zero.
    rng = np.random.default_rng(39)
    n = 256
    k = rng.standard_normal((1, n, 1, 128)).astype(np.float32)
    v = rng.standard_normal((1, n, 1, 128)).astype(np.float32)
    q = rng.standard_normal((1, 1, 128)).astype(np.float32)
    lens = np.array([n], np.int32)
    table, nb = workloads.block_table(lens, 32, 0)
    exact = oracle.decode_attn_f32(oracle.build_mirror(k, v, lens, table, nb, 32), q, 1, SCALE)
    quant = oracle.decode_attn(oracle.build_cache(k, v, lens, table, nb, 32), q, 1, SCALE)
    gap = np.abs(exact - quant).max()
    _, dv = oracle.quantize_kv(v[0, :, 0])
    assert 0 < gap < float(dv.mean())
