"""GPU parity of the batched prefill attention ("why long context must be
sparse" §1-§2) against the oracle, through the C ABI.

Each query row must satisfy max |gpu - oracle| <= 2e-5 * max |oracle| + 1e-6
per (row, head); the oracle's prefill is pinned on the CPU.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import DeviceCache, assert_rows_close, dense_kv, q8, say, torch

pytestmark = pytest.mark.gpu
SCALE = float(workloads.softmax_scale(128))


def _run(dc, q, q_start, nq, max_new=None):
    t, m = torch(), q8()
    qs = np.asarray(q_start, np.int32)
    if max_new is None:
        max_new = int(max(1, np.diff(qs).max())) if qs.size > 1 else 1
    out = t.full((q.shape[0], nq, 128), float("nan"), dtype=t.float32, device="cuda")
    m.prefill_attn(dc.layer, dc.batch, nq, t.from_numpy(qs).cuda(), max_new, t.from_numpy(q).cuda(), SCALE, out,
                   dev_status=dc.status)
    return out.cpu().numpy()


def _case(lens, nbs, nq, nkv, kv_bs, seed, dist="normal"):
    lens = np.asarray(lens, np.int32)
    k, v = dense_kv(lens, nkv, seed=seed, dist=dist)
    dc = DeviceCache(lens, nkv, kv_bs, seed=seed)
    dc.append_dense(k, v)
    qs = np.concatenate([[0], np.cumsum(nbs)]).astype(np.int32)
    q = np.random.default_rng([seed, 9]).standard_normal((int(qs[-1]), nq, 128)).astype(np.float32)
    got = _run(dc, q, qs, nq)
    assert dc.status_word() == 0
    want = oracle.prefill_attn(dc.host(), q, qs, nq, SCALE)
    return assert_rows_close(got, want, f"prefill nq={nq} nkv={nkv} kv_bs={kv_bs}"), dc, q, qs, got


@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("kv_bs", [8, 16, 32, 64, 256])
def test_prefill_fresh_prompts(group, kv_bs):
    # the whole prompt is new: row 0 sees only itself, the last row everything
    say(f"[prefill] fresh prompts group={group} kv_bs={kv_bs}")
    lens = [1, 17, 64, 100, 257]
    w, *_ = _case(lens, lens, 2 * group, 2, kv_bs, seed=800 + 10 * group + kv_bs)
    say(f"  worst err/tol {w:.3f}")


@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_prefill_after_history(group):
    say(f"[prefill] chunks after a history group={group}")
    lens = [300, 1000, 65, 33, 40]
    nbs = [7, 64, 65, 1, 0]
    w, *_ = _case(lens, nbs, 2 * group, 2, 32, seed=820 + group)
    say(f"  worst err/tol {w:.3f}")


def test_one_new_token_is_the_decode_step():
    say("[prefill] one new token per sequence vs the GPU decode")
    lens = [5, 129, 2000]
    w, dc, q, qs, got = _case(lens, [1, 1, 1], 16, 8, 32, seed=830)
    dec = dc.decode(q, 16, SCALE).cpu().numpy()
    assert_rows_close(got, dec, "prefill of one token vs decode")
    say(f"  worst err/tol {w:.3f}")


def test_prefill_heavy_tails_8b_shape():
    say("[prefill] 8B shape, student-t x3")
    lens = [700, 1500]
    w, *_ = _case(lens, [700, 300], 32, 8, 32, seed=840, dist="student3x3")
    say(f"  worst err/tol {w:.3f}")


def test_bad_q_start_is_reported():
    # 50 new rows claimed for a 40-token sequence: flagged, its rows zero;
    # the other sequence is computed normally
    say("[prefill] bad q_start")
    lens = np.array([40, 90], np.int32)
    k, v = dense_kv(lens, 2, seed=850)
    dc = DeviceCache(lens, 2, 32, seed=850)
    dc.append_dense(k, v)
    qs = np.array([0, 50, 60], np.int32)
    q = np.random.default_rng(851).standard_normal((60, 4, 128)).astype(np.float32)
    got = _run(dc, q, qs, 4, max_new=50)
    assert dc.status_word() & 0x1
    assert np.all(got[:50] == 0)
    ok = oracle.prefill_attn(dc.host(), q[50:], [0, 0, 10], 4, SCALE)
    assert_rows_close(got[50:], ok, "the good sequence")


@pytest.mark.parametrize("kv_bs", [8, 16, 32, 64])
def test_prefill_bad_block_is_left_out(kv_bs):
    # an out-of-range id in the middle of sequence 0's table: reported, and
    # every row attends to its visible tokens without that block's.  Attention
    # does not depend on the order of its tokens, so the reference for a row
    # at position p is the oracle's decode over a table with the block removed
    # and the length reduced by the block's tokens at or before p.
    say(f"[prefill] bad block id, kv_bs={kv_bs}")
    nq, nkv = 4, 2
    lens = np.array([200, 150], np.int32)
    nbs = np.array([200, 50], np.int32)
    k, v = dense_kv(lens, nkv, seed=880 + kv_bs)
    dc = DeviceCache(lens, nkv, kv_bs, seed=880 + kv_bs)
    dc.append_dense(k, v)
    bi = 96 // kv_bs   # the block holding token 96
    dc.table_t[0, bi] = dc.num_blocks + 7
    qs = np.concatenate([[0], np.cumsum(nbs)]).astype(np.int32)
    q = np.random.default_rng(881 + kv_bs).standard_normal((int(qs[-1]), nq, 128)).astype(np.float32)
    got = _run(dc, q, qs, nq)
    assert dc.status_word() & q8().DEV_BAD_BLOCK_ID
    h = dc.host()
    tables, ns = [], []
    for b in range(2):
        for i in range(int(nbs[b])):
            p = int(lens[b] - nbs[b] + i)
            row = h.block_table[b].copy()
            n = p + 1
            if b == 0:
                row = np.concatenate([np.delete(row, bi), row[:1]])
                n -= min(max(p + 1 - bi * kv_bs, 0), kv_bs)
            tables.append(row)
            ns.append(n)
    view = oracle.Cache(h.k_codes, h.v_codes, h.k_step, h.v_step, np.stack(tables).astype(np.int32),
                        np.array(ns, np.int32), nkv, 128)
    want = oracle.decode_attn(view, q, nq, SCALE)
    w = assert_rows_close(got, want, f"prefill with a bad block, kv_bs={kv_bs}")
    say(f"  worst err/tol {w:.3f}")


def test_prefill_2b_prompt_4059_sampled():
    # the pages' longest prefill prompt (n = 4059) on the 2B shape, 28 layers'
    # worth of one layer; checked on sampled rows: row p of the prefill is the
    # decode attention over the first p + 1 tokens (an oracle identity pinned
    # on the CPU), so a cache view with seq_len = p + 1 per sample gives it
    say("[prefill] 2B shape, 4059-token prompt, sampled rows")
    n, nq, nkv = 4059, 16, 8
    lens = np.array([n], np.int32)
    k, v = dense_kv(lens, nkv, seed=860)
    dc = DeviceCache(lens, nkv, 32, seed=860)
    dc.append_dense(k, v)
    q = np.random.default_rng(861).standard_normal((n, nq, 128)).astype(np.float32)
    got = _run(dc, q, [0, n], nq)
    assert dc.status_word() == 0
    h = dc.host()
    pos = np.unique(np.concatenate([[0, 1, 15, 16, 17, 31, 32, n - 2, n - 1],
                                    np.random.default_rng(862).integers(0, n, 40)]))
    view = oracle.Cache(h.k_codes, h.v_codes, h.k_step, h.v_step, np.repeat(h.block_table, pos.size, axis=0),
                        (pos + 1).astype(np.int32), nkv, 128)
    want = oracle.decode_attn(view, q[pos], nq, SCALE)
    w = assert_rows_close(got[pos], want, "sampled prefill rows")
    say(f"  {pos.size} positions, worst err/tol {w:.3f}")


def test_prefill_graph_replays_match_eager():
    # append of the new tokens + prefill captured in one HIP graph; every
    # replay (with eager work and synchronizations between them) must equal
    # the eager result bit for bit
    say("[prefill] graph capture / replay")
    t, m = torch(), q8()
    lens = np.array([600, 97, 1200], np.int32)
    nbs = np.array([600, 33, 100], np.int32)
    k, v = dense_kv(lens, 8, seed=870)
    dc = DeviceCache(lens, 8, 32, seed=870)
    dc.append_dense(k, v)   # history and the new tokens' first values
    qs = t.from_numpy(np.concatenate([[0], np.cumsum(nbs)]).astype(np.int32)).cuda()
    total = int(nbs.sum())
    seq = t.from_numpy(np.repeat(np.arange(3, dtype=np.int32), nbs)).cuda()
    pos = t.from_numpy(np.concatenate([np.arange(n - c, n, dtype=np.int32) for n, c in zip(lens, nbs)])).cuda()
    g_ = t.Generator(device="cuda")
    g_.manual_seed(871)
    kn = t.randn((total, 8, 128), generator=g_, device="cuda")
    vn = t.randn((total, 8, 128), generator=g_, device="cuda")
    q = t.randn((total, 16, 128), generator=g_, device="cuda")
    out = t.empty((total, 16, 128), dtype=t.float32, device="cuda")

    def body():
        m.kv_append(dc.layer, dc.batch, seq, pos, kn, vn, dev_status=dc.status)
        m.prefill_attn(dc.layer, dc.batch, 16, qs, int(nbs.max()), q, SCALE, out, dev_status=dc.status)

    body()
    t.cuda.synchronize()
    eager = out.clone()
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        body()
    t.cuda.current_stream().wait_stream(side)
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        body()
    for i in range(4):
        out.fill_(float("nan"))
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        assert t.equal(out, eager), f"replay {i}"
    assert dc.status_word() == 0
    # and the result is the oracle's
    want = oracle.prefill_attn(dc.host(), q.cpu().numpy(), qs.cpu().numpy(), 16, SCALE)
    assert_rows_close(eager.cpu().numpy(), want, "prefill after graph replays")
