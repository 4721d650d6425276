"""GPU parity of the block-sparse decode ("why long context must be sparse"
§1-§2) against the oracle, through the C ABI.

The kept blocks are a decision the GPU takes on fp32 scores; they are judged
against the oracle's importances (the page's score of each probe row, in
double): every kept block must score at least every dropped one within the
fp32 evaluation bound, exact ties going to the lower block
(gpu_cases.check_sparse_selection).  The outputs must satisfy max |gpu -
oracle| <= 2e-5 * max |oracle| + 1e-6 per (b, h) row against the oracle's
attention over the blocks the GPU kept.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import (SPARSE_EPS_U, DeviceCache, dense_kv, q8, run_sparse_and_check, say, torch)

pytestmark = pytest.mark.gpu
SCALE = float(workloads.softmax_scale(128))
EDGE_LENS = [0, 1, 31, 32, 33, 64, 65, 100, 255, 256, 257, 700, 1024, 1025, 2049]


def _sparse_case(lens, nq, nkv, kv_bs, topk, seed, dist="normal", q=None):
    lens = np.asarray(lens, np.int32)
    k, v = dense_kv(lens, nkv, seed=seed, dist=dist)
    if q is None:
        q = np.random.default_rng([seed, 7]).standard_normal((len(lens), nq, 128)).astype(np.float32)
    dc = DeviceCache(lens, nkv, kv_bs, seed=seed)
    dc.append_dense(k, v)
    worst, band = run_sparse_and_check(dc, q, nq, SCALE, topk)
    say(f"  rows decided inside the fp32 band: {band}")
    return worst


@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("kv_bs", [8, 32, 64])
def test_sparse_edges(group, kv_bs):
    say(f"[sparse] edges group={group} kv_bs={kv_bs}")
    w = _sparse_case(EDGE_LENS, 2 * group, 2, kv_bs, topk=4, seed=400 + 10 * group + kv_bs)
    say(f"  worst err/tol {w:.3f}")


@pytest.mark.parametrize("topk", [2, 7, 32, 64])
def test_sparse_topk_2b_shape(topk):
    say(f"[sparse] 2B shape topk={topk}")
    lens = np.array([4059, 2046, 506, 3000, 65, 8192], np.int32)
    w = _sparse_case(lens, 16, 8, 32, topk=topk, seed=500 + topk)
    say(f"  worst err/tol {w:.3f}")


def test_sparse_heavy_tails_8b_shape():
    say("[sparse] 8B shape, student-t x3")
    lens = np.array([1, 64, 65, 1500, 4096, 3333], np.int32)
    w = _sparse_case(lens, 32, 8, 32, topk=32, seed=501, dist="student3x3")
    say(f"  worst err/tol {w:.3f}")


def test_sparse_long_sequence():
    say("[sparse] one 20K-token sequence")
    w = _sparse_case([20000], 8, 2, 32, topk=32, seed=502)
    say(f"  worst err/tol {w:.3f}")


def test_sparse_ties_keep_lowest_blocks():
    # q = 0: every probe score is 0, the k lowest blocks are kept
    say("[sparse] all-equal scores")
    lens = np.array([1000, 333], np.int32)
    _sparse_case(lens, 4, 2, 32, topk=5, seed=503, q=np.zeros((2, 4, 128), np.float32))


def test_sparse_graph_replays_match_eager():
    t = torch()
    m = q8()
    say("[sparse] graph capture / replay")
    lens = np.array([3000, 65, 1, 1200], np.int32)
    k, v = dense_kv(lens, 8, seed=504)
    dc = DeviceCache(lens, 8, 32, seed=504)
    dc.append_dense(k, v)
    q = t.from_numpy(np.random.default_rng(504).standard_normal((4, 16, 128)).astype(np.float32)).cuda()
    ws = t.empty(m.decode_attn_sparse_workspace_bytes(dc.layer, dc.batch, 16, 8), dtype=t.uint8, device="cuda")
    out = t.empty((4, 16, 128), dtype=t.float32, device="cuda")

    def body():
        m.decode_attn_sparse(dc.layer, dc.batch, 16, q, SCALE, out, ws, topk=8, dev_status=dc.status)

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
        ws.fill_(0xAB)
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        assert t.equal(out, eager), f"replay {i}"
    assert dc.status_word() == 0


@pytest.mark.parametrize("group,kv_bs", [(1, 32), (2, 8), (4, 32), (8, 16)])
def test_sparse_probe_scores_within_fp32_bound(group, kv_bs):
    # White-box: the probe's block scores sit at the start of the workspace,
    # [batch * nq][max_nb] fp32 (max_nb = ceil(max_seq_len / 32)), in the log2
    # domain (times fl(scale * log2 e) / scale).  Wherever a sequence has more
    # than k blocks they must lie within the fp32 evaluation bound of the
    # oracle's double importances.
    say(f"[sparse] probe scores group={group} kv_bs={kv_bs}")
    t, m = torch(), q8()
    nkv, nq, topk = 2, 2 * group, 4
    lens = np.array([1500, 97, 5, 4096, 700], np.int32)
    k, v = dense_kv(lens, nkv, seed=600 + group, dist="student3x3")
    q = np.random.default_rng([600 + group, 7]).standard_normal((len(lens), nq, 128)).astype(np.float32)
    dc = DeviceCache(lens, nkv, kv_bs, seed=600 + group)
    dc.append_dense(k, v)
    want, mag = oracle.sparse_scores(dc.host(), q, nq, SCALE)
    out = t.empty((len(lens), nq, 128), dtype=t.float32, device="cuda")
    ws = t.empty(m.decode_attn_sparse_workspace_bytes(dc.layer, dc.batch, nq, topk), dtype=t.uint8, device="cuda")
    ws.fill_(0xCD)
    m.decode_attn_sparse(dc.layer, dc.batch, nq, t.from_numpy(q).cuda(), SCALE, out, ws, topk=topk,
                         dev_status=dc.status)
    assert dc.status_word() == 0
    max_nb = want.shape[-1]
    got = ws[:len(lens) * nq * max_nb * 4].cpu().numpy().view(np.float32).reshape(len(lens), nq, max_nb)
    sigma = float(np.float32(float(np.float32(SCALE)) * 1.4426950408889634)) / float(np.float32(SCALE))
    checked = 0
    for b, n in enumerate(lens):
        nb = (int(n) + 31) // 32
        if nb <= topk:
            continue
        err = np.abs(got[b, :, :nb].astype(np.float64) / sigma - want[b, :, :nb])
        bound = SPARSE_EPS_U * mag[b, :, :nb] + 1e-300
        assert np.all(err <= bound), f"sequence {b}: worst err/bound {(err / bound).max():.3f}"
        checked += nq * nb
    assert checked > 0
