"""CPU pins of the oracle's block-sparse decode.

Page: "why long context must be sparse" (10-1) -- §1: cut the history into
32-token blocks, find the most relevant k blocks with a cheap probe, run
exact attention over the chosen blocks only; §2: k = 32 blocks per head,
32 positions per block, 8 probe samples per block ("max-dot fusion"), the
sparse path only for sequences longer than two blocks.  The readings the
oracle takes where the page defers to a missing one (probe rows 0, 4, ..., 28;
importance = the block's largest probe score; per query head; ties to the
lower block index) are pinned here against an independent numpy
re-derivation, closed forms and designed cases.
"""
import numpy as np
import pytest

import oracle
import workloads

SCALE = workloads.softmax_scale(128)
LOG2E_SC = np.float32(float(SCALE) * 1.4426950408889634)


def cache_of(k, v, lens, kv_bs=32, seed=0):
    table, nb = workloads.block_table(np.asarray(lens, np.int32), kv_bs, seed, spare_blocks=2)
    return oracle.build_cache(k, v, np.asarray(lens, np.int32), table, nb, kv_bs)


def probe_scores_np(q_row, k_rows):
    """Block scores of one query head over its K rows [n, 128], re-derived with
    numpy float32 arithmetic in the kernel's order (the oracle's C code is not
    used)."""
    cq, qsc = oracle.quantize_q(q_row)
    ck, ks = oracle.quantize_kv(k_rows)
    n = k_rows.shape[0]
    nb = (n + 31) // 32
    out = np.full(nb, -np.inf, np.float32)
    for j in range(nb):
        for r in range(0, 32, 4):
            t = 32 * j + r
            if t >= n:
                break
            p = [int(np.dot(cq[32 * b:32 * b + 32].astype(np.int64), ck[t, 32 * b:32 * b + 32].astype(np.int64)))
                 for b in range(4)]
            x = [np.float32(p[b]) * np.float32(qsc[b]) for b in range(4)]
            y = np.float32(np.float32(x[0] + x[1]) + np.float32(x[3] + x[2]))
            s = np.float32(y * np.float32(np.float32(ks[t]) * LOG2E_SC))
            out[j] = max(out[j], s)
    return out


def topk_np(scores, k):
    order = sorted(range(len(scores)), key=lambda j: (-float(scores[j]), j))
    return sorted(order[:k])


def dense_over(q_row, k_rows, v_rows, blocks, n):
    cq, qsc = oracle.quantize_q(q_row)
    ck, ks = oracle.quantize_kv(k_rows[:n])
    cv, vs = oracle.quantize_kv(v_rows[:n])
    idx = np.concatenate([np.arange(32 * j, min(32 * j + 32, n)) for j in blocks])
    kh = oracle.dequantize(ck[idx], ks[idx])
    vh = oracle.dequantize(cv[idx], vs[idx])
    return oracle.attend_dense(oracle.dequantize_q(cq, qsc), kh, vh, float(SCALE)).astype(np.float32)


@pytest.mark.parametrize("n,topk", [(300, 4), (1000, 32), (2049, 7), (4059, 32)])
def test_selection_and_output_match_independent_rederivation(n, topk):
    rng = np.random.default_rng(n + topk)
    nkv, nq = 2, 4
    k = rng.standard_normal((1, n, nkv, 128)).astype(np.float32)
    v = rng.standard_normal((1, n, nkv, 128)).astype(np.float32)
    q = rng.standard_normal((1, nq, 128)).astype(np.float32)
    out, sel = oracle.decode_attn_sparse(cache_of(k, v, [n], seed=n), q, nq, SCALE, topk)
    for h in range(nq):
        kh = h // (nq // nkv)
        want_sel = topk_np(probe_scores_np(q[0, h], k[0, :, kh]), topk)
        got_sel = [int(j) for j in sel[0, h] if j >= 0]
        assert got_sel == want_sel
        np.testing.assert_array_equal(out[0, h], dense_over(q[0, h], k[0, :, kh], v[0, :, kh], want_sel, n))


@pytest.mark.parametrize("n,topk", [(1, 32), (64, 2), (1024, 32), (700, 200)])
def test_few_blocks_is_exact_attention(n, topk):
    # At most two blocks' worth of tokens, or at most k blocks: every block
    # is kept, and the result is the exact q8 attention bit for bit.
    rng = np.random.default_rng(7 * n + topk)
    k = rng.standard_normal((1, n, 2, 128)).astype(np.float32)
    v = rng.standard_normal((1, n, 2, 128)).astype(np.float32)
    q = rng.standard_normal((1, 4, 128)).astype(np.float32)
    c = cache_of(k, v, [n], kv_bs=16, seed=3)
    out, sel = oracle.decode_attn_sparse(c, q, 4, SCALE, topk)
    np.testing.assert_array_equal(out, oracle.decode_attn(c, q, 4, SCALE))
    nb = (n + 31) // 32
    assert np.all(sel[0, :, :nb] == np.arange(nb)) and np.all(sel[0, :, nb:] == -1)


def test_gate_at_two_blocks():
    # With the smallest k (2), 64 tokens (2 blocks) keep both blocks and 65
    # tokens (3 blocks) are sparse: two of the three kept.
    rng = np.random.default_rng(11)
    k = rng.standard_normal((1, 65, 1, 128)).astype(np.float32)
    v = rng.standard_normal((1, 65, 1, 128)).astype(np.float32)
    q = rng.standard_normal((1, 1, 128)).astype(np.float32)
    _, sel = oracle.decode_attn_sparse(cache_of(k, v, [65]), q, 1, SCALE, 2)
    assert (sel[0, 0] >= 0).sum() == 2
    _, sel = oracle.decode_attn_sparse(cache_of(k[:, :64], v[:, :64], [64]), q, 1, SCALE, 2)
    assert list(sel[0, 0]) == [0, 1]


def test_probe_rows_are_every_fourth_row():
    # A key aligned with q at a probe row (row 8 of block 5) makes its block a
    # top block; a stronger key at a non-probe row (row 9 of block 7) is
    # invisible to the probe, so block 7 is not among the k = 2 kept -- until
    # the same key moves to a probe row.
    rng = np.random.default_rng(12)
    n = 32 * 12
    k = (rng.standard_normal((1, n, 1, 128)) * 0.1).astype(np.float32)
    v = rng.standard_normal((1, n, 1, 128)).astype(np.float32)
    q = rng.standard_normal((1, 1, 128)).astype(np.float32)
    k[0, 32 * 5 + 8, 0] = q[0, 0] * 3
    k[0, 32 * 7 + 9, 0] = q[0, 0] * 6
    _, sel = oracle.decode_attn_sparse(cache_of(k, v, [n]), q, 1, SCALE, 2)
    assert 5 in sel[0, 0] and 7 not in sel[0, 0]
    k[0, 32 * 7 + 8, 0] = q[0, 0] * 6          # now at a probe row
    _, sel = oracle.decode_attn_sparse(cache_of(k, v, [n]), q, 1, SCALE, 2)
    assert list(sel[0, 0]) == [5, 7]


def test_ties_go_to_lower_blocks():
    # q = 0: every probe score is 0; the k lowest block indices are kept.
    rng = np.random.default_rng(13)
    n = 32 * 40 + 5
    k = rng.standard_normal((1, n, 1, 128)).astype(np.float32)
    v = rng.standard_normal((1, n, 1, 128)).astype(np.float32)
    _, sel = oracle.decode_attn_sparse(cache_of(k, v, [n]), np.zeros((1, 1, 128), np.float32), 1, SCALE, 6)
    assert list(sel[0, 0]) == [0, 1, 2, 3, 4, 5]


def test_per_query_head_selection_and_gqa():
    # Two query heads of one KV head may keep different blocks; each head's
    # output is the single-head run with that head's query.
    rng = np.random.default_rng(14)
    n = 32 * 30
    k = rng.standard_normal((1, n, 1, 128)).astype(np.float32)
    v = rng.standard_normal((1, n, 1, 128)).astype(np.float32)
    q = rng.standard_normal((1, 2, 128)).astype(np.float32)
    c = cache_of(k, v, [n])
    out, sel = oracle.decode_attn_sparse(c, q, 2, SCALE, 5)
    assert not np.array_equal(sel[0, 0], sel[0, 1])
    for h in range(2):
        o1, s1 = oracle.decode_attn_sparse(c, q[:, h:h + 1], 1, SCALE, 5)
        np.testing.assert_array_equal(o1[0, 0], out[0, h])
        np.testing.assert_array_equal(s1[0, 0], sel[0, h])


def test_zero_length_and_bad_block():
    rng = np.random.default_rng(15)
    k = rng.standard_normal((2, 100, 1, 128)).astype(np.float32)
    v = rng.standard_normal((2, 100, 1, 128)).astype(np.float32)
    c = cache_of(k, v, [0, 100])
    out, sel = oracle.decode_attn_sparse(c, np.ones((2, 1, 128), np.float32), 1, SCALE, 2)
    assert np.all(out[0] == 0) and np.all(sel[0] == -1)
    c.block_table[1, 2] = c.num_blocks
    with pytest.raises(ValueError):
        oracle.decode_attn_sparse(c, np.ones((2, 1, 128), np.float32), 1, SCALE, 2)


def test_probe_scores_bitwise():
    # The probe score is a decision input: it must follow the fp32 formula
    # step for step (numpy re-derivation, bit for bit, on many rows).
    rng = np.random.default_rng(16)
    n, nkv, nq = 32 * 20 + 9, 2, 4
    k = (rng.standard_t(3, (1, n, nkv, 128)) * 2).astype(np.float32)
    v = rng.standard_normal((1, n, nkv, 128)).astype(np.float32)
    q = rng.standard_normal((1, nq, 128)).astype(np.float32)
    got = oracle.sparse_scores(cache_of(k, v, [n], kv_bs=8, seed=4), q, nq, SCALE)
    for h in range(nq):
        want = probe_scores_np(q[0, h], k[0, :, h // 2])
        np.testing.assert_array_equal(got[0, h].view(np.uint32), want.view(np.uint32))
