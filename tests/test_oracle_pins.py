"""CPU pins of the oracle: each test checks the oracle against something other
than itself -- values the pages print, closed forms, invariants the pages or
mathematics fix, brute force on tiny inputs.  No GPU needed.

Pages: 9-2 "flash_attn_single_q_q8_neon -- 单 q 单遍扫全 KV" (§2 segments 1-3,
§3, §4); 9-3 "q8 KV 精度对照实验" (§1-§4); 10-1 "why long context must be
sparse" (§1).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
INV127 = np.float32(1.0) / np.float32(127.0)
SCALE = workloads.softmax_scale(128)


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f32bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


# ------------------------------------------------------------------ constants
def test_constants_bit_patterns():
    # fl(1/127) and fl(1/sqrt(128)) as fp32 bit patterns.
    assert int(f32bits(INV127)) == 0x3C010204
    assert int(f32bits(SCALE)) == 0x3DB504F3
    # 127 * fl(1/127) is exactly 1 in fp32: the worked cases rely on it.
    assert np.float32(127.0) * INV127 == np.float32(1.0)


# ---------------------------------------------------------- P1: K/V quantizer
def test_kv_quantizer_worked_cases():
    g = golden("quantizer_cases.json")
    row = np.full(128, g["fill_value_rest"], np.float32)
    row[: len(g["kv_row_prefix"])] = g["kv_row_prefix"]
    codes, step = oracle.quantize_kv(row)
    want = np.full(128, g["fill_code_kv"], np.int8)
    want[: len(g["kv_codes_prefix"])] = g["kv_codes_prefix"]
    np.testing.assert_array_equal(codes, want)
    assert step == np.float32(g["kv_step"])


@pytest.mark.parametrize("dist", ["normal", "student", "uniform"])
def test_kv_quantizer_invariants(dist):
    rng = np.random.default_rng(7)
    n = 4096
    if dist == "normal":
        x = rng.standard_normal((n, 128)).astype(np.float32)
    elif dist == "student":
        x = (3 * rng.standard_t(3, (n, 128))).astype(np.float32)
    else:
        x = rng.uniform(-5, 5, (n, 128)).astype(np.float32)
    codes, step = oracle.quantize_kv(x)
    a = np.abs(x).max(1)
    # |code| <= 127, and the max-abs element maps to +-127 (9-3 §2 clamp to [-127, 127]).
    assert np.abs(codes.astype(np.int32)).max() <= 127
    arg = np.abs(x).argmax(1)
    assert np.all(np.abs(codes[np.arange(n), arg].astype(np.int32)) == 127)
    # code has the sign of x (or is 0)
    assert np.all(codes.astype(np.int32) * np.sign(x) >= 0)
    # stored step is max-abs/127 to within two fp32 roundings (9-3 §2: scale = max_abs/127;
    # fl(1/127) is itself rounded, then the product)
    rel = np.abs(step.astype(np.float64) - a.astype(np.float64) / 127.0) / (a.astype(np.float64) / 127.0)
    assert rel.max() <= 2 * 2.0 ** -24
    # and exactly max-abs * fl(1/127): the step the 9-2 kernel applies on read is the
    # stored per-token value times KVQ_INV (9-2 §2 segment 2), the same product.
    np.testing.assert_array_equal(f32bits(step), f32bits(a * INV127))
    # dequantization error at most half a step (9-3 §3: each dequantized value is off by <= half a step),
    # up to the fp32 roundings: x*r and x/d differ by at most 4 roundings of a value <= 127.
    err = np.abs(x.astype(np.float64) - oracle.dequantize(codes, step))
    assert np.all(err <= step.astype(np.float64)[:, None] * (0.5 + 127 * 4 * 2.0 ** -24))


def test_kv_quantizer_power_of_two_equivariance():
    # Scaling a row by 2^k changes no code and multiplies the step by exactly 2^k
    # (every fp32 step of the rule commutes with exact binary scaling).
    rng = np.random.default_rng(11)
    x = rng.standard_normal((2048, 128)).astype(np.float32)
    c0, d0 = oracle.quantize_kv(x)
    for k in (-5, -2, 2, 5):
        c1, d1 = oracle.quantize_kv(x * np.float32(2.0 ** k))
        np.testing.assert_array_equal(c1, c0)
        np.testing.assert_array_equal(f32bits(d1), f32bits(d0 * np.float32(2.0 ** k)))


def test_kv_quantizer_guard_boundary():
    # The guard is strict: max-abs == 1e-6f is quantized normally, the next float
    # below it is replaced by 1 (step = fl(1/127), codes of tiny values = 0).
    t = np.float32(1e-6)
    below = np.nextafter(t, np.float32(0))
    row = np.full(128, t * np.float32(0.5), np.float32)
    row[3] = t
    c, d = oracle.quantize_kv(row)
    assert c[3] == 127 and d == t * INV127
    assert np.all(c[np.arange(128) != 3] == 64)  # 0.5 * 127 = 63.5 -> 64 (half away from zero)
    row2 = np.full(128, below * np.float32(0.5), np.float32)
    row2[5] = -below
    c2, d2 = oracle.quantize_kv(row2)
    assert d2 == INV127
    assert np.all(c2 == 0)
    # all-zero row
    c3, d3 = oracle.quantize_kv(np.zeros(128, np.float32))
    assert d3 == INV127 and np.all(c3 == 0)


def test_kv_quantizer_row_independence():
    # One scale per (token, head) row (9-3 §4: the head's 128 dims share one scale):
    # changing one row leaves every other row's codes and step unchanged.
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    c0, d0 = oracle.quantize_kv(x)
    x2 = x.copy()
    x2[17] *= 40
    c1, d1 = oracle.quantize_kv(x2)
    mask = np.arange(64) != 17
    np.testing.assert_array_equal(c1[mask], c0[mask])
    np.testing.assert_array_equal(d1[mask], d0[mask])


def test_kv_quantizer_x3_amplitude():
    # 9-3 §4: scaling K/V by 3 scales the step by ~3 and leaves the relative error
    # about the same -- at the quantizer, codes change only at near-ties.
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4096, 128)).astype(np.float32)
    c0, d0 = oracle.quantize_kv(x)
    c3, d3 = oracle.quantize_kv(x * np.float32(3))
    assert np.mean(c3 != c0) < 1e-4
    np.testing.assert_allclose(d3, 3 * d0, rtol=3e-7)


# ------------------------------------------------------------ P1: Q quantizer
def test_q_quantizer_worked_cases():
    g = golden("quantizer_cases.json")
    blk = np.full(32, g["fill_value_rest"], np.float32)
    blk[: len(g["q_block_prefix"])] = g["q_block_prefix"]
    q = np.tile(blk, 4)
    codes, qsc = oracle.quantize_q(q)
    want = np.full(32, g["fill_code_q"], np.int8)
    want[: len(g["q_codes_prefix"])] = g["q_codes_prefix"]
    np.testing.assert_array_equal(codes, np.tile(want, 4))
    np.testing.assert_array_equal(qsc, np.full(4, g["q_scale"], np.float32))


def test_q_quantizer_invariants():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((4096, 128)).astype(np.float32)
    q[::7, 32:64] *= 1e-8        # some blocks fall under the guard
    codes, qsc = oracle.quantize_q(q)
    blocks = q.reshape(4096, 4, 32).astype(np.float64)
    m = np.abs(blocks).max(2)
    guarded = m < 1e-6
    m_eff = np.where(guarded, 1.0, m)
    # block scale = m * fl(1/127) exactly
    np.testing.assert_array_equal(qsc, (m_eff.astype(np.float32) * INV127))
    c = codes.reshape(4096, 4, 32).astype(np.int32)
    assert c.min() >= -127 and c.max() <= 127          # -128 is unreachable
    # truncation toward zero: |code| <= |q| * 127/m and the error is below one step
    r = np.float32(127.0) / m_eff.astype(np.float32)
    y = (blocks.astype(np.float32) * r[..., None]).astype(np.float64)
    assert np.all(np.abs(c) <= np.abs(y))
    assert np.all(np.abs(y - c) < 1.0)
    assert np.all(c * np.sign(blocks) >= 0)
    # guarded blocks of tiny values give all-zero codes
    assert np.all(c[guarded] == 0)
    # truncation leaves the block max at 126 in a sizeable fraction of blocks
    top = np.abs(c).max(2)[~guarded]
    assert set(np.unique(top)) <= {126, 127}
    assert 0.02 < np.mean(top == 126) < 0.4


def test_q_quantizer_block_independence():
    rng = np.random.default_rng(4)
    q = rng.standard_normal(128).astype(np.float32)
    c0, s0 = oracle.quantize_q(q)
    q2 = q.copy()
    q2[40] = 50.0
    c1, s1 = oracle.quantize_q(q2)
    for blk in (0, 2, 3):
        np.testing.assert_array_equal(c1[32 * blk:32 * blk + 32], c0[32 * blk:32 * blk + 32])
        assert s1[blk] == s0[blk]
    assert s1[1] != s0[1]


# ------------------------------------------------------------------ P2: partials
def test_partials_exhaustive_products():
    # Every int8 x int8 product, placed alone in a block, is returned exactly.
    vals = np.arange(-128, 128, dtype=np.int32)
    for a in vals:
        cq = np.zeros(128, np.int8)
        ck = np.zeros(128, np.int8)
        # four products per call: block j holds (a, b_j)
        for j in range(0, 256, 4):
            bs = vals[j:j + 4]
            cq[[0, 32, 64, 96]] = a
            ck[[0, 32, 64, 96]] = bs
            p = oracle.block_partials(cq, ck)
            np.testing.assert_array_equal(p, a * bs)


def test_partials_extremes_and_bruteforce():
    one = np.ones(128, np.int8)
    assert list(oracle.block_partials(one * 127, one * 127)) == [32 * 127 * 127] * 4
    assert list(oracle.block_partials(one * -128, one * 127)) == [-32 * 128 * 127] * 4
    assert list(oracle.block_partials(one * -128, one * -128)) == [32 * 128 * 128] * 4
    rng = np.random.default_rng(1)
    for _ in range(200):
        cq = rng.integers(-128, 128, 128).astype(np.int8)
        ck = rng.integers(-127, 128, 128).astype(np.int8)
        want = [sum(int(cq[i]) * int(ck[i]) for i in range(32 * b, 32 * b + 32)) for b in range(4)]
        assert list(oracle.block_partials(cq, ck)) == want


# ----------------------------------------------------------- attention pins
def _rand_case(rng, n, hd, pattern="random"):
    q = rng.standard_normal(hd).astype(np.float32)
    k = rng.standard_normal((n, hd)).astype(np.float32)
    v = rng.standard_normal((n, hd)).astype(np.float32)
    if pattern == "equal":
        k[:] = k[0]
    elif pattern in ("increasing", "decreasing"):
        # keys along q with strictly monotone projections
        base = q / np.linalg.norm(q)
        steps = np.arange(n, dtype=np.float32) * np.float32(0.05)
        if pattern == "decreasing":
            steps = steps[::-1]
        k = (np.outer(steps, base) + 0.001 * k).astype(np.float32)
    return q, k, v


def _q8_parts(q, k, v):
    cq, qsc = oracle.quantize_q(q)
    ck, ks = oracle.quantize_kv(k)
    cv, vs = oracle.quantize_kv(v)
    return cq, qsc, ck, ks, cv, vs


def _three_pass(cq, qsc, ck, ks, cv, vs, scale):
    return oracle.attend_dense(oracle.dequantize_q(cq, qsc), oracle.dequantize(ck, ks),
                               oracle.dequantize(cv, vs), scale)


def _close(a, b, rtol=2e-5, atol=1e-6):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.max(np.abs(a - b)) <= rtol * np.max(np.abs(b)) + atol


def test_single_pass_equals_three_pass():
    # 9-2 §3: the single pass with online rescale is functionally the same as
    # computing all scores first.  fp32 single pass vs double three pass.
    rng = np.random.default_rng(2024)
    cases = 0
    for it in range(1500):
        hd = (32, 64, 128)[it % 3]
        n = int(rng.integers(1, 301))
        pattern = ("random", "equal", "increasing", "decreasing")[it % 4]
        q, k, v = _rand_case(rng, n, hd, pattern)
        if it % 5 == 0:
            k *= np.float32(rng.uniform(0.2, 6.0))
        parts = _q8_parts(q, k, v)
        out1, trace = oracle.single_pass(*parts, SCALE)
        out3 = _three_pass(*parts, SCALE)
        assert _close(out1, out3), (it, n, hd, pattern)
        cases += 1
    assert cases == 1500


def test_running_max_monotone_and_loop_count():
    # 9-2 §4: the loop runs exactly seq_len times and M never decreases; it ends
    # at the largest score.
    rng = np.random.default_rng(8)
    for pattern in ("random", "equal", "increasing", "decreasing"):
        q, k, v = _rand_case(rng, 257, 128, pattern)
        cq, qsc, ck, ks, cv, vs = _q8_parts(q, k, v)
        _, trace = oracle.single_pass(cq, qsc, ck, ks, cv, vs, SCALE)
        assert trace.shape == (257,)
        assert np.all(np.diff(trace) >= 0)
        qh = oracle.dequantize_q(cq, qsc)
        s = SCALE * (oracle.dequantize(ck, ks) @ qh)
        assert abs(trace[-1] - s.max()) <= 1e-5 * max(1.0, abs(s.max()))
        if pattern == "increasing":
            assert np.all(np.diff(trace) > 0)
        if pattern == "decreasing":
            assert np.all(trace == trace[0])


def _cache_from_dense(k, v, lens, kv_bs=32, seed=0, spare=3):
    table, nblocks = workloads.block_table(lens, kv_bs, seed, spare_blocks=spare)
    return oracle.build_cache(k, v, lens, table, nblocks, kv_bs)


def test_seq_len_one_returns_dequantized_v_bitwise():
    # With one token, w = 1 and S = 1, so the output is the dequantized V row.
    rng = np.random.default_rng(12)
    k = rng.standard_normal((1, 1, 2, 128)).astype(np.float32)
    v = rng.standard_normal((1, 1, 2, 128)).astype(np.float32)
    q = rng.standard_normal((1, 4, 128)).astype(np.float32)
    cache = _cache_from_dense(k, v, np.array([1], np.int32))
    out = oracle.decode_attn(cache, q, 4, SCALE)
    cv, dv = oracle.quantize_kv(v[0, 0])
    for h in range(4):
        want = (cv[h // 2].astype(np.float32) * dv[h // 2]).astype(np.float32)
        np.testing.assert_array_equal(f32bits(out[0, h]), f32bits(want))


def test_zero_query_gives_mean_of_values():
    # q = 0: every block is guarded, all codes are 0, every score is 0, so every
    # weight is 1 and the output is the plain mean of the dequantized V rows.
    rng = np.random.default_rng(13)
    n = 77
    k = rng.standard_normal((1, n, 1, 128)).astype(np.float32)
    v = rng.standard_normal((1, n, 1, 128)).astype(np.float32)
    cache = _cache_from_dense(k, v, np.array([n], np.int32))
    out = oracle.decode_attn(cache, np.zeros((1, 1, 128), np.float32), 1, SCALE)
    cv, dv = oracle.quantize_kv(v[0, :, 0])
    want = oracle.dequantize(cv, dv).mean(0)
    np.testing.assert_allclose(out[0, 0], want, rtol=1e-6, atol=1e-7)


def test_two_keys_closed_form():
    # Two keys whose scores differ by exactly ln 3: weights 3/4 and 1/4.
    rng = np.random.default_rng(14)
    q = rng.standard_normal(128).astype(np.float32)
    k = rng.standard_normal((2, 128)).astype(np.float32)
    v = rng.standard_normal((2, 128)).astype(np.float32)
    cq, qsc, ck, ks, cv, vs = _q8_parts(q, k, v)
    qh = oracle.dequantize_q(cq, qsc)
    dots = oracle.dequantize(ck, ks) @ qh
    scale = math.log(3.0) / (dots[0] - dots[1])
    out = oracle.attend_dense(qh, oracle.dequantize(ck, ks), oracle.dequantize(cv, vs), scale)
    vh = oracle.dequantize(cv, vs)
    np.testing.assert_allclose(out, 0.75 * vh[0] + 0.25 * vh[1], rtol=1e-12, atol=1e-14)


def test_one_dominant_key():
    # Scores more than 104 below the maximum underflow fp32 exp: the output is
    # the dominant key's dequantized V row.
    rng = np.random.default_rng(15)
    n = 50
    q = np.ones((1, 1, 128), np.float32)
    k = (rng.standard_normal((1, n, 1, 128)) * 0.01).astype(np.float32)
    k[0, 17, 0] = 100.0               # s ~ 100*128/sqrt(128)*... far above the rest
    v = rng.standard_normal((1, n, 1, 128)).astype(np.float32)
    cache = _cache_from_dense(k, v, np.array([n], np.int32))
    out = oracle.decode_attn(cache, q, 1, SCALE)
    cv, dv = oracle.quantize_kv(v[0, 17, 0])
    np.testing.assert_allclose(out[0, 0], oracle.dequantize(cv, dv), rtol=1e-7, atol=0)


def test_convexity():
    # Softmax weights are a convex combination: every output component lies
    # between the smallest and largest dequantized V component.
    rng = np.random.default_rng(16)
    for n in (3, 40, 300):
        k = (rng.standard_normal((1, n, 2, 128)) * 3).astype(np.float32)
        v = rng.standard_normal((1, n, 2, 128)).astype(np.float32)
        q = rng.standard_normal((1, 2, 128)).astype(np.float32)
        cache = _cache_from_dense(k, v, np.array([n], np.int32))
        out = oracle.decode_attn(cache, q, 2, SCALE)
        for h in range(2):
            cv, dv = oracle.quantize_kv(v[0, :, h])
            vh = oracle.dequantize(cv, dv)
            assert np.all(out[0, h] >= vh.min(0) - 1e-6) and np.all(out[0, h] <= vh.max(0) + 1e-6)


def test_gqa_reduction_and_blocked_walk():
    # Head h of an nq = nkv * G run equals a one-head attention over KV head h / G,
    # computed here from dense dequantized rows (no block table involved).
    rng = np.random.default_rng(17)
    lens = np.array([70, 33, 1, 0, 128], np.int32)
    nkv, nq = 2, 8
    k = rng.standard_normal((5, 128, nkv, 128)).astype(np.float32)
    v = rng.standard_normal((5, 128, nkv, 128)).astype(np.float32)
    q = rng.standard_normal((5, nq, 128)).astype(np.float32)
    cache = _cache_from_dense(k, v, lens, kv_bs=32, seed=5)
    out = oracle.decode_attn(cache, q, nq, SCALE)
    for b in range(5):
        n = int(lens[b])
        for h in range(nq):
            if n == 0:
                assert np.all(out[b, h] == 0)
                continue
            kh = h // (nq // nkv)
            cq, qsc = oracle.quantize_q(q[b, h])
            ck, ks = oracle.quantize_kv(k[b, :n, kh])
            cv, vs = oracle.quantize_kv(v[b, :n, kh])
            want = _three_pass(cq, qsc, ck, ks, cv, vs, SCALE).astype(np.float32)
            np.testing.assert_array_equal(out[b, h], want)


def test_placement_invariance_and_kv_bs():
    # Where the blocks sit in the pool, and the block size, do not change the
    # result (exact: the same values are visited in the same order).
    rng = np.random.default_rng(18)
    lens = np.array([200, 65, 9], np.int32)
    k = rng.standard_normal((3, 200, 2, 128)).astype(np.float32)
    v = rng.standard_normal((3, 200, 2, 128)).astype(np.float32)
    q = rng.standard_normal((3, 4, 128)).astype(np.float32)
    outs = []
    for kv_bs, seed in ((32, 1), (32, 2), (8, 3), (64, 4), (16, 5)):
        cache = _cache_from_dense(k, v, lens, kv_bs=kv_bs, seed=seed, spare=7)
        outs.append(oracle.decode_attn(cache, q, 4, SCALE))
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])
    rows = oracle.decode_attn_rows(_cache_from_dense(k, v, lens), q, 4, SCALE, [0, 5, 11, 7])
    np.testing.assert_array_equal(rows, outs[0].reshape(12, 128)[[0, 5, 11, 7]])


def test_bad_block_id_and_length_are_reported():
    rng = np.random.default_rng(19)
    k = rng.standard_normal((1, 40, 1, 128)).astype(np.float32)
    cache = _cache_from_dense(k, k, np.array([40], np.int32))
    q = rng.standard_normal((1, 1, 128)).astype(np.float32)
    cache.block_table[0, 1] = cache.num_blocks + 3
    with pytest.raises(ValueError):
        oracle.decode_attn(cache, q, 1, SCALE)
    cache2 = _cache_from_dense(k, k, np.array([40], np.int32))
    cache2.seq_lens[0] = 10_000
    with pytest.raises(ValueError):
        oracle.decode_attn(cache2, q, 1, SCALE)


def test_qk_partials_over_cache():
    rng = np.random.default_rng(20)
    lens = np.array([45, 3], np.int32)
    k = rng.standard_normal((2, 45, 2, 128)).astype(np.float32)
    q = rng.standard_normal((2, 4, 128)).astype(np.float32)
    cache = _cache_from_dense(k, k, lens, seed=9)
    p = oracle.qk_partials(cache, q, 4, 48)
    assert p.shape == (2, 4, 48, 4)
    for b in range(2):
        for h in range(4):
            cq, _ = oracle.quantize_q(q[b, h])
            ck, _ = oracle.quantize_kv(k[b, : lens[b], h // 2])
            want = (cq.astype(np.int64)[None, :] * ck.astype(np.int64)).reshape(lens[b], 4, 32).sum(2)
            np.testing.assert_array_equal(p[b, h, : lens[b]], want)
            assert np.all(p[b, h, lens[b]:] == 0)


# --------------------------------------------------------- P12: pages' gap
def _gap_experiment(seed, quantizer, amp=1.0):
    """9-3 §1: the same attention over fp32 K/V and over quantized-then-
    dequantized K/V (Q stays fp32), L = 256, hd = 128, K/V ~ N(0, 1)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(128).astype(np.float32)
    k = (amp * rng.standard_normal((256, 128))).astype(np.float32)
    v = (amp * rng.standard_normal((256, 128))).astype(np.float32)
    out_f = oracle.attend_dense(q, k, v, SCALE)
    kq = quantizer(k)
    vq = quantizer(v)
    out_q = oracle.attend_dense(q, kq[0], vq[0], SCALE)
    d = np.abs(out_q - out_f)
    return d.max(), d.mean(), kq[1].mean(), out_f, out_q


def _oracle_rule(x):
    c, s = oracle.quantize_kv(x)
    return oracle.dequantize(c, s), s


def _biased_rule(x):
    # Diagnostic only (never used by the library or the oracle): "+0.5 then
    # truncate toward zero", a common C idiom that is biased for negative values.
    a = np.abs(x).max(1, keepdims=True)
    r = np.float32(127.0) / a
    c = np.clip(np.trunc(x * r + np.float32(0.5)), -127, 127)
    step = (a * INV127)[:, 0]
    return c.astype(np.float64) * step[:, None], step


def test_pages_gap_unbiased_rule():
    g = golden("pages_q8_gap.json")
    stats = np.array([_gap_experiment(s, _oracle_rule)[:3] for s in range(60)])
    mx, mean, step = np.median(stats, 0)
    # The rule as read gives a gap at or below the pages' printed figures ...
    assert mx <= g["max_abs_diff"] and mean <= g["mean_abs_diff"]
    # ... of the size half a step predicts for independent rounding errors
    # averaged by the softmax: well under half a step, far above zero.
    assert 0.5e-3 < mx < 0.5 * step
    assert 0.2e-3 < mean < 0.25 * step
    # the N(0,1) max of 128 values is ~2.8, so the step is ~0.022
    assert 0.019 < step < 0.025


def test_pages_gap_pattern_matches_biased_rounding():
    # The pages' numbers (all four printed differences positive, mean gap about
    # half the average step) are what a biased rounding produces.
    g = golden("pages_q8_gap.json")
    stats = [_gap_experiment(s, _biased_rule) for s in range(30)]
    mean_gap = np.median([s[1] for s in stats])
    avg_step = np.median([s[2] for s in stats])
    pages_ratio = g["mean_abs_diff"] / g["avg_k_step"]
    assert abs(mean_gap / avg_step - pages_ratio) < 0.1
    pos = np.mean([np.all((s[4] - s[3])[:4] > 0) for s in stats])
    assert pos > 0.9
    printed = np.array(g["out_q8_first4"]) - np.array(g["out_fp32_first4"])
    assert np.all(printed > 0)


def test_x3_amplitude_relative_gap():
    # 9-3 §4: with K/V amplitude x3 the relative error stays about the same
    # (the scale follows the rows); scores also grow x3, so the softmax sharpens.
    r1, r3 = [], []
    for s in range(40):
        for amp, acc in ((1.0, r1), (3.0, r3)):
            mx, _, _, out_f, _ = _gap_experiment(1000 + s, _oracle_rule, amp)
            acc.append(mx / np.abs(out_f).max())
    ratio = np.median(r3) / np.median(r1)
    assert 0.5 <= ratio <= 3.0


# --------------------------------------------------------------- P14: bytes
def test_bytes_per_token_layer():
    g = golden("pages_structure.json")
    assert workloads.kv_bytes_per_token(8, 128) == g["kv_bytes_per_token_layer"]["value"]
    # versus an f16 cache of the same shape (2 x 8 x 128 x 2 bytes)
    assert round(2112 / (2 * 8 * 128 * 2), 2) == g["q8_vs_f16_bandwidth_ratio"]["value"]
    # one layer at 8K: about 17 MB
    assert abs(8192 * 2112 / 1e6 - g["one_layer_full_scan_at_8k_MB"]["value"]) < 1.0
