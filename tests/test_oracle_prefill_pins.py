"""CPU pins of the oracle's batched prefill attention over the q8 cache.

Page: "why long context must be sparse" (10-1) -- §1 (a prefill batch of nb
new tokens scores against the whole history, O(nb x n)) and §2 (the exact
batched prefill path beside the block-sparse one).  The readings the oracle
takes where the page is silent (the new tokens are the last positions of the
cache; causal masking inside the batch; each query row quantized like the
decode query) are pinned here against closed forms, a pure-Python brute
force, an independent numpy recomputation and invariants.
"""
import math

import numpy as np
import pytest

import oracle
import workloads

SCALE = workloads.softmax_scale(128)


def cache_of(k, v, lens, kv_bs=32, seed=0):
    table, nb = workloads.block_table(np.asarray(lens, np.int32), kv_bs, seed, spare_blocks=2)
    return oracle.build_cache(k, v, np.asarray(lens, np.int32), table, nb, kv_bs)


def kv(rng, batch, n, nkv, dist="normal"):
    if dist == "t":
        return [(rng.standard_t(3, (batch, n, nkv, 128)) * 3).astype(np.float32) for _ in range(2)]
    return [rng.standard_normal((batch, n, nkv, 128)).astype(np.float32) for _ in range(2)]


def causal_numpy(q_row, k_rows, v_rows, p):
    """Attention of one query over positions 0..p, from the pinned quantizers
    and numpy float64 (not the oracle's attention code)."""
    cq, qsc = oracle.quantize_q(q_row)
    ck, ks = oracle.quantize_kv(k_rows[:p + 1])
    cv, vs = oracle.quantize_kv(v_rows[:p + 1])
    qh = oracle.dequantize_q(cq, qsc)
    kh, vh = oracle.dequantize(ck, ks), oracle.dequantize(cv, vs)
    s = float(SCALE) * (kh @ qh)
    w = np.exp(s - s.max())
    return (w @ vh) / w.sum()


def test_first_row_of_a_fresh_prompt_is_the_first_v_row():
    # Position 0 sees only itself: weight 1, so the output is its dequantized
    # V row, bit for bit.
    rng = np.random.default_rng(70)
    n = 37
    k, v = kv(rng, 1, n, 2)
    q = rng.standard_normal((n, 4, 128)).astype(np.float32)
    out = oracle.prefill_attn(cache_of(k, v, [n]), q, [0, n], 4, SCALE)
    cv, vs = oracle.quantize_kv(v[0, 0])
    for h in range(4):
        want = (cv[h // 2].astype(np.float64) * np.float64(vs[h // 2])).astype(np.float32)
        np.testing.assert_array_equal(out[0, h], want)


@pytest.mark.parametrize("n,nb", [(1, 1), (5, 5), (9, 4), (12, 1)])
def test_brute_force_tiny(n, nb):
    # Pure Python (math.exp, math.fsum) over the dequantized values, causal.
    rng = np.random.default_rng(71 + n + nb)
    k, v = kv(rng, 1, n, 1, dist="t")
    q = rng.standard_normal((nb, 2, 128)).astype(np.float32)
    out = oracle.prefill_attn(cache_of(k, v, [n], kv_bs=8), q, [0, nb], 2, SCALE)
    ck, ks = oracle.quantize_kv(k[0, :, 0])
    cv, vs = oracle.quantize_kv(v[0, :, 0])
    for r in range(nb):
        p = n - nb + r
        for h in range(2):
            cq, qsc = oracle.quantize_q(q[r, h])
            qh = [float(cq[i]) * float(qsc[i // 32]) for i in range(128)]
            s = [float(SCALE) * math.fsum(qh[i] * float(ck[t, i]) * float(ks[t]) for i in range(128))
                 for t in range(p + 1)]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            tot = math.fsum(w)
            want = [math.fsum(w[t] * float(cv[t, i]) * float(vs[t]) for t in range(p + 1)) / tot
                    for i in range(128)]
            np.testing.assert_allclose(out[r, h], want, rtol=1e-6, atol=1e-6 * max(abs(x) for x in want))


def test_causality():
    # Row at position p is unchanged by anything at positions > p (K, V) and
    # by the other query rows.
    rng = np.random.default_rng(72)
    n, nb = 300, 40
    k, v = kv(rng, 1, n, 2)
    q = rng.standard_normal((nb, 4, 128)).astype(np.float32)
    base = oracle.prefill_attn(cache_of(k, v, [n]), q, [0, nb], 4, SCALE)
    r = 17
    p = n - nb + r
    k2, v2, q2 = k.copy(), v.copy(), q.copy()
    k2[0, p + 1:] = rng.standard_normal(k2[0, p + 1:].shape) * 5
    v2[0, p + 1:] = rng.standard_normal(v2[0, p + 1:].shape) * 5
    q2[r + 1:] = 0
    q2[:r] *= -2
    out = oracle.prefill_attn(cache_of(k2, v2, [n]), q2, [0, nb], 4, SCALE)
    np.testing.assert_array_equal(out[r], base[r])
    assert not np.array_equal(out[r + 1], base[r + 1])


def test_last_row_is_the_decode_step():
    # The last new token sees the whole cache: the decode attention.
    rng = np.random.default_rng(73)
    lens = [90, 33, 500]
    k, v = kv(rng, 3, 500, 2)
    nbs = [7, 33, 1]
    qs = np.concatenate([[0], np.cumsum(nbs)]).astype(np.int32)
    q = rng.standard_normal((int(qs[-1]), 8, 128)).astype(np.float32)
    c = cache_of(k, v, lens, seed=5)
    out = oracle.prefill_attn(c, q, qs, 8, SCALE)
    dec = oracle.decode_attn(c, q[qs[1:] - 1], 8, SCALE)
    np.testing.assert_array_equal(out[qs[1:] - 1], dec)


def test_zero_query_gives_prefix_means():
    rng = np.random.default_rng(74)
    n, nb = 64, 10
    k, v = kv(rng, 1, n, 1)
    out = oracle.prefill_attn(cache_of(k, v, [n]), np.zeros((nb, 1, 128), np.float32), [0, nb], 1, SCALE)
    cv, vs = oracle.quantize_kv(v[0, :, 0])
    vh = oracle.dequantize(cv, vs)
    for r in range(nb):
        p = n - nb + r
        np.testing.assert_allclose(out[r, 0], vh[:p + 1].mean(0), rtol=2e-7, atol=1e-8)


def test_chunked_prefill_equals_one_batch():
    # Prefilling 50 tokens at once or as 30 + 20 (the second chunk after the
    # first is in the cache) gives the same rows, bit for bit.
    rng = np.random.default_rng(75)
    h0, nb1, nb2 = 100, 30, 20
    n = h0 + nb1 + nb2
    k, v = kv(rng, 1, n, 2)
    q = rng.standard_normal((nb1 + nb2, 4, 128)).astype(np.float32)
    whole = oracle.prefill_attn(cache_of(k, v, [n]), q, [0, nb1 + nb2], 4, SCALE)
    a = oracle.prefill_attn(cache_of(k[:, :h0 + nb1], v[:, :h0 + nb1], [h0 + nb1]), q[:nb1], [0, nb1], 4, SCALE)
    b = oracle.prefill_attn(cache_of(k, v, [n]), q[nb1:], [0, nb2], 4, SCALE)
    np.testing.assert_array_equal(np.concatenate([a, b]), whole)


def test_ragged_batch_gqa_against_numpy():
    rng = np.random.default_rng(76)
    lens = [40, 1, 129, 77]
    nbs = [40, 1, 16, 0]
    k, v = kv(rng, 4, 129, 2, dist="t")
    qs = np.concatenate([[0], np.cumsum(nbs)]).astype(np.int32)
    q = rng.standard_normal((int(qs[-1]), 8, 128)).astype(np.float32)
    out = oracle.prefill_attn(cache_of(k, v, lens, kv_bs=16, seed=3), q, qs, 8, SCALE)
    for b in range(4):
        for r in range(int(qs[b]), int(qs[b + 1])):
            p = lens[b] - nbs[b] + (r - int(qs[b]))
            for h in range(8):
                want = causal_numpy(q[r, h], k[b, :, h // 4], v[b, :, h // 4], p)
                np.testing.assert_allclose(out[r, h], want, rtol=1e-6, atol=1e-6 * np.abs(want).max())


def test_bad_q_start_is_reported():
    rng = np.random.default_rng(77)
    k, v = kv(rng, 2, 20, 1)
    c = cache_of(k, v, [20, 5])
    q = np.ones((12, 1, 128), np.float32)
    with pytest.raises(ValueError):   # 6 new tokens in a 5-token sequence
        oracle.prefill_attn(c, q[:12], [0, 6, 12], 1, SCALE)
    with pytest.raises(ValueError):   # decreasing
        oracle.prefill_attn(c, q[:4], [0, 5, 4], 1, SCALE)
