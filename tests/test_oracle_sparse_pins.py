"""CPU pins of the oracle's block-sparse decode.

Page: "why long context must be sparse" (10-1) -- §1: cut the history into
32-token blocks, find the most relevant k blocks with a cheap probe, run
exact attention over the chosen blocks only; §2: k = 32 blocks per head,
32 positions per block, 8 probe samples per block ("max-dot fusion"), the
sparse path only for sequences longer than two blocks.  The score of a probe
row is the q8 attention score of "9-2 flash_attn_single_q_q8_neon" §2
segment 2: s = (sum over 32-blocks of P_b * qscale_b) * kscale * scale.

The readings the oracle takes where the page defers to a missing one (probe
rows 0, 4, ..., 28; importance = the block's largest probe score; per query
head; ties to the lower block index) are pinned here against things other
than the oracle's own arithmetic: exact rational brute force, a closed form
on a structured input, exact power-of-two and sign equivariance, designed
blocks (a dominant probe row, a strong key off the probe rows), exact
ranking, and pure-Python attention over the kept tokens.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

SCALE = workloads.softmax_scale(128)
U53 = 2.0 ** -53


def cache_of(k, v, lens, kv_bs=32, seed=0):
    table, nb = workloads.block_table(np.asarray(lens, np.int32), kv_bs, seed, spare_blocks=2)
    return oracle.build_cache(k, v, np.asarray(lens, np.int32), table, nb, kv_bs)


def exact_row_score(cq, qsc, ck_row, ks_row):
    """The page's score of one key row in exact rational arithmetic (Python
    integers for the block sums, Fractions of the fp32 scales)."""
    s = Fraction(0)
    for b in range(4):
        p = sum(int(cq[i]) * int(ck_row[i]) for i in range(32 * b, 32 * b + 32))
        s += p * Fraction(float(qsc[b]))
    return s * Fraction(float(ks_row)) * Fraction(float(SCALE))


def exact_importance(q_row, k_rows):
    """Per block: (exact max over probe rows 0, 4, ..., 28 of the exact score,
    the absolute-term magnitude of that row), quantizing with the oracle's
    quantizers (pinned on their own in test_oracle_pins.py)."""
    cq, qsc = oracle.quantize_q(q_row)
    ck, ks = oracle.quantize_kv(k_rows)
    n = k_rows.shape[0]
    out = []
    for j in range((n + 31) // 32):
        best = None
        for t in range(32 * j, min(32 * j + 32, n), 4):
            s = exact_row_score(cq, qsc, ck[t], ks[t])
            if best is None or s > best:
                best = s
        out.append(best)
    return out


def ranked(scores, k):
    """Top k by (score descending, index ascending), returned ascending."""
    order = sorted(range(len(scores)), key=lambda j: (-scores[j], j))
    return sorted(order[:k])


def brute_attention(q_row, k_rows, v_rows, tokens):
    """Pure-Python attention over the given tokens: dequantized q, K, V
    (code times scale), scores, max-subtracted exp weights (math.exp), sums
    with math.fsum."""
    cq, qsc = oracle.quantize_q(q_row)
    ck, ks = oracle.quantize_kv(k_rows)
    cv, vs = oracle.quantize_kv(v_rows)
    qh = [float(cq[i]) * float(qsc[i // 32]) for i in range(128)]
    s = []
    for t in tokens:
        kh = [float(ck[t, i]) * float(ks[t]) for i in range(128)]
        s.append(float(SCALE) * math.fsum(a * b for a, b in zip(qh, kh)))
    m = max(s)
    w = [math.exp(x - m) for x in s]
    tot = math.fsum(w)
    return np.array([math.fsum(w[u] * float(cv[t, i]) * float(vs[t]) for u, t in enumerate(tokens)) / tot
                     for i in range(128)])


# ---------------------------------------------------------------- the score --
@pytest.mark.parametrize("dist", ["normal", "student"])
def test_importance_is_the_exact_page_score_within_double_rounding(dist):
    # Exact rational brute force of every block's importance on heavy and
    # light tails, three query heads, GQA 2 (kv head = h // 2), kv_bs 8.
    rng = np.random.default_rng(31 if dist == "normal" else 32)
    n, nkv, nq = 32 * 6 + 13, 2, 4
    if dist == "normal":
        k = rng.standard_normal((1, n, nkv, 128)).astype(np.float32)
    else:
        k = (3 * rng.standard_t(3, (1, n, nkv, 128))).astype(np.float32)
    v = rng.standard_normal((1, n, nkv, 128)).astype(np.float32)
    q = rng.standard_normal((1, nq, 128)).astype(np.float32)
    got, mag = oracle.sparse_scores(cache_of(k, v, [n], kv_bs=8, seed=5), q, nq, SCALE)
    for h in range(nq):
        want = exact_importance(q[0, h], k[0, :, h // 2])
        for j, e in enumerate(want):
            err = abs(Fraction(float(got[0, h, j])) - e)
            # one rounding per block term, three in the sum, two in the products
            assert err <= Fraction(8 * U53) * Fraction(float(mag[0, h, j])), (h, j)
            assert mag[0, h, j] >= abs(float(e)) * (1 - 1e-12)
        assert np.all(np.isneginf(got[0, h, len(want):]))


def test_importance_closed_form_on_a_constant_block():
    # q = 1 everywhere: every query code is 127 with step fl(1/127).  K rows
    # of one block all 2: codes 127, step fl(2 * fl(1/127)) = 2 fl(1/127).
    # So P_b = 32 * 127 * 127 and the score is
    #   scale * 2 fl(1/127) * 4 * 32 * 127^2 * fl(1/127),
    # with fl(1/127) = 0x3C010204 and scale = fl(1/sqrt(128)) = 0x3DB504F3.
    inv127 = Fraction(float(np.array(0x3C010204, np.uint32).view(np.float32)))
    scale = Fraction(float(np.array(0x3DB504F3, np.uint32).view(np.float32)))
    assert float(scale) == float(SCALE)
    want = scale * 2 * inv127 * 4 * 32 * 127 * 127 * inv127
    k = np.full((1, 96, 1, 128), 2.0, np.float32)
    k[0, 32:] = np.random.default_rng(3).standard_normal((64, 1, 128)).astype(np.float32) * 0.01
    v = np.zeros_like(k)
    got, _ = oracle.sparse_scores(cache_of(k, v, [96]), np.ones((1, 1, 128), np.float32), 1, SCALE)
    assert abs(Fraction(float(got[0, 0, 0])) - want) <= want * Fraction(4 * U53)
    assert got[0, 0, 0] > got[0, 0, 1] and got[0, 0, 0] > got[0, 0, 2]


def test_importance_power_of_two_and_sign_equivariance():
    # Quantizer codes are unchanged by a power-of-two scale and the steps scale
    # exactly (pinned in test_oracle_pins.py), so every score scales by the
    # same power of two bit for bit; truncation toward zero is odd, so -q
    # negates every row score, and a block holding a single probe row (the
    # last one, 1 token) negates its importance.
    rng = np.random.default_rng(33)
    n = 32 * 5 + 1
    k = rng.standard_normal((1, n, 1, 128)).astype(np.float32)
    v = rng.standard_normal((1, n, 1, 128)).astype(np.float32)
    q = rng.standard_normal((1, 1, 128)).astype(np.float32)
    base, _ = oracle.sparse_scores(cache_of(k, v, [n]), q, 1, SCALE)
    k4, _ = oracle.sparse_scores(cache_of(4 * k, v, [n]), q, 1, SCALE)
    q8_, _ = oracle.sparse_scores(cache_of(k, v, [n]), np.float32(0.125) * q, 1, SCALE)
    neg, _ = oracle.sparse_scores(cache_of(k, v, [n]), -q, 1, SCALE)
    np.testing.assert_array_equal(k4, 4 * base)
    np.testing.assert_array_equal(q8_, 0.125 * base)
    assert neg[0, 0, 5] == -base[0, 0, 5]
    # and a multi-row block's importance under -q is minus its smallest row score
    rows = [exact_row_score(*oracle.quantize_q(q[0, 0]), *[a[t] for a in oracle.quantize_kv(k[0, :, 0])])
            for t in range(64, 96, 4)]
    assert abs(Fraction(float(neg[0, 0, 2])) + min(rows)) <= abs(min(rows)) * Fraction(8 * U53) + Fraction(1, 10 ** 30)


def test_dominant_probe_row_sets_the_block_and_is_kept():
    # Blocks 3 and 9 each hold one key aligned with q at a probe row (rows 12
    # and 28); their importance is that row's exact score, and they are the
    # two blocks kept at k = 2.
    rng = np.random.default_rng(34)
    n = 32 * 14
    k = (rng.standard_normal((1, n, 1, 128)) * 0.05).astype(np.float32)
    v = rng.standard_normal((1, n, 1, 128)).astype(np.float32)
    q = rng.standard_normal((1, 1, 128)).astype(np.float32)
    k[0, 32 * 3 + 12, 0] = 2 * q[0, 0]
    k[0, 32 * 9 + 28, 0] = 3 * q[0, 0]
    c = cache_of(k, v, [n])
    got, _ = oracle.sparse_scores(c, q, 1, SCALE)
    cq, qsc = oracle.quantize_q(q[0, 0])
    ck, ks = oracle.quantize_kv(k[0, :, 0])
    for j, t in ((3, 32 * 3 + 12), (9, 32 * 9 + 28)):
        e = exact_row_score(cq, qsc, ck[t], ks[t])
        assert abs(Fraction(float(got[0, 0, j])) - e) <= abs(e) * Fraction(8 * U53)
    _, sel = oracle.decode_attn_sparse(c, q, 1, SCALE, 2)
    assert list(sel[0, 0]) == [3, 9]


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


# ------------------------------------------------------ selection and output --
@pytest.mark.parametrize("n,topk", [(300, 4), (1000, 6), (2049, 7)])
def test_selection_is_the_exact_ranking_and_output_the_brute_force(n, topk):
    # The kept set equals the top k of the exact rational importances (ties to
    # the lower index); the output equals pure-Python attention over the
    # kept tokens.
    rng = np.random.default_rng(n + topk)
    nkv, nq = 2, 4
    k = rng.standard_normal((1, n, nkv, 128)).astype(np.float32)
    v = rng.standard_normal((1, n, nkv, 128)).astype(np.float32)
    q = rng.standard_normal((1, nq, 128)).astype(np.float32)
    out, sel = oracle.decode_attn_sparse(cache_of(k, v, [n], seed=n), q, nq, SCALE, topk)
    for h in range(nq):
        kh = h // (nq // nkv)
        imp = exact_importance(q[0, h], k[0, :, kh])
        want_sel = ranked(imp, topk)
        # the data has a clear margin at the cut, so double rounding cannot reorder it
        kth = sorted(imp, reverse=True)[topk - 1]
        nxt = sorted(imp, reverse=True)[topk]
        assert kth - nxt > abs(kth) * Fraction(1, 10 ** 9)
        got_sel = [int(j) for j in sel[0, h] if j >= 0]
        assert got_sel == want_sel
        tokens = [t for j in want_sel for t in range(32 * j, min(32 * j + 32, n))]
        ref = brute_attention(q[0, h], k[0, :, kh], v[0, :, kh], tokens)
        np.testing.assert_allclose(out[0, h], ref, rtol=1e-6, atol=1e-7)


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


# --------------------------------------------- attention over a given block set --
def test_block_set_attention_against_repacked_cache_and_brute_force():
    # Attention over blocks {1, 4, 6 (the partial last one)} of a 32 * 6 + 9
    # token sequence equals (a) the decode attention of a sequence holding
    # exactly those tokens in that order, bit for bit, and (b) pure-Python
    # attention over them; all blocks equals the full decode bit for bit.
    rng = np.random.default_rng(35)
    n, nkv, nq = 32 * 6 + 9, 2, 4
    k = (2 * rng.standard_t(3, (1, n, nkv, 128))).astype(np.float32)
    v = rng.standard_normal((1, n, nkv, 128)).astype(np.float32)
    q = rng.standard_normal((1, nq, 128)).astype(np.float32)
    c = cache_of(k, v, [n], kv_bs=16, seed=6)
    blocks = [1, 4, 6]
    sel = np.full((1, nq, 8), -1, np.int32)
    sel[0, :, :3] = blocks
    got = oracle.decode_attn_blocks(c, q, nq, SCALE, sel)
    tokens = [t for j in blocks for t in range(32 * j, min(32 * j + 32, n))]
    packed = cache_of(k[:, tokens], v[:, tokens], [len(tokens)], kv_bs=32, seed=9)
    np.testing.assert_array_equal(got, oracle.decode_attn(packed, q, nq, SCALE))
    for h in range(nq):
        ref = brute_attention(q[0, h], k[0, :, h // 2], v[0, :, h // 2], tokens)
        np.testing.assert_allclose(got[0, h], ref, rtol=1e-6, atol=1e-7)
    every = np.tile(np.arange(7, dtype=np.int32), (1, nq, 1))
    np.testing.assert_array_equal(oracle.decode_attn_blocks(c, q, nq, SCALE, every), oracle.decode_attn(c, q, nq, SCALE))
    # per-head block lists; an empty list gives zeros; an index past the end is refused
    sel2 = np.full((1, nq, 2), -1, np.int32)
    sel2[0, 0] = [0, 2]
    sel2[0, 1] = [5, -1]
    got2 = oracle.decode_attn_blocks(c, q, nq, SCALE, sel2)
    assert np.all(got2[0, 2:] == 0)
    t1 = list(range(160, 192))
    np.testing.assert_allclose(got2[0, 1], brute_attention(q[0, 1], k[0, :, 0], v[0, :, 0], t1), rtol=1e-6, atol=1e-7)
    sel2[0, 3, 0] = 7
    with pytest.raises(ValueError):
        oracle.decode_attn_blocks(c, q, nq, SCALE, sel2)
