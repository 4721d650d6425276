"""GPU parity of the fp32 mirror path ("9-3 q8 KV 精度对照实验": §3 closing
note, the float cache the write path keeps beside the q8 one; §1, the exact
attention over it) against the oracle, through the C ABI.

The mirror must hold the appended rows bit for bit; the exact decode must
match the oracle's double-precision attention over the same fp32 rows within
max |gpu - oracle| <= 2e-5 * max |oracle| + 1e-6 per (b, h) row.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import DeviceCache, assert_rows_close, dense_kv, q8, say, torch

pytestmark = pytest.mark.gpu
SCALE = float(workloads.softmax_scale(128))
EDGE_LENS = [0, 1, 2, 7, 8, 9, 31, 32, 33, 63, 64, 65, 100, 255, 256, 257, 700]


@pytest.mark.parametrize("kv_bs", [8, 32])
def test_append_fills_mirror_bit_exact(kv_bs):
    # Every appended row lands unchanged at its (block, row) slot; the q8
    # codes are still written; slots no token occupies keep their contents.
    say(f"[mirror] append kv_bs={kv_bs}")
    lens = np.array([1, 33, 200, 0, 95], np.int32)
    k, v = dense_kv(lens, 4, seed=200 + kv_bs, dist="student3x3")
    dc = DeviceCache(lens, 4, kv_bs, seed=200 + kv_bs, mirror=True)
    dc.append_dense(k, v)
    assert dc.status_word() == 0
    kf = dc.layer.k_f32.cpu().numpy().reshape(dc.num_blocks * kv_bs, 4, 128)
    vf = dc.layer.v_f32.cpu().numpy().reshape(dc.num_blocks * kv_bs, 4, 128)
    used = np.zeros(dc.num_blocks * kv_bs, bool)
    for b, n in enumerate(lens):
        t = np.arange(n)
        slot = dc.table[b, t // kv_bs] * kv_bs + t % kv_bs
        used[slot] = True
        np.testing.assert_array_equal(kf[slot].view(np.uint32), k[b, :n].view(np.uint32))
        np.testing.assert_array_equal(vf[slot].view(np.uint32), v[b, :n].view(np.uint32))
    assert np.all(np.isnan(kf[~used])) and np.all(np.isnan(vf[~used]))
    # the q8 side of the same append is unchanged by the mirror
    ref = DeviceCache(lens, 4, kv_bs, seed=200 + kv_bs)
    ref.append_dense(k, v)
    t = torch()
    assert t.equal(ref.layer.k_codes.cpu()[used.reshape(dc.num_blocks, kv_bs)],
                   dc.layer.k_codes.cpu()[used.reshape(dc.num_blocks, kv_bs)])


def _f32_case(lens, nq, nkv, kv_bs, seed, nparts_list, dist="normal"):
    lens = np.asarray(lens, np.int32)
    k, v = dense_kv(lens, nkv, seed=seed, dist=dist)
    q = np.random.default_rng([seed, 6]).standard_normal((len(lens), nq, 128)).astype(np.float32)
    dc = DeviceCache(lens, nkv, kv_bs, seed=seed, mirror=True)
    dc.append_dense(k, v)
    want = oracle.decode_attn_f32(oracle.build_mirror(k, v, lens, dc.table, dc.num_blocks, kv_bs), q, nq, SCALE)
    worst = 0.0
    for nparts in nparts_list:
        got = dc.decode_f32(q, nq, SCALE, nparts=nparts).cpu().numpy()
        assert dc.status_word() == 0
        worst = max(worst, assert_rows_close(got, want, f"f32 nparts={nparts}"))
        for b in np.nonzero(lens == 0)[0]:
            assert np.all(got[b] == 0)
    return worst


def test_f32_single_head_256():
    say("[mirror] decode single head 256")
    say(f"  worst err/tol {_f32_case([256], 1, 1, 32, 2001, [0, 1, 3, 8]):.3f}")


@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("kv_bs", [8, 32, 64])
def test_f32_ragged_edges(group, kv_bs):
    say(f"[mirror] ragged edges group={group} kv_bs={kv_bs}")
    w = _f32_case(EDGE_LENS, 2 * group, 2, kv_bs, seed=300 + group * 10 + kv_bs, nparts_list=[0, 1, 7, 1000])
    say(f"  worst err/tol {w:.3f}")


def test_f32_2b_shape_heavy_tails():
    say("[mirror] 2B shape, student-t x3, ragged")
    lens = np.array([4059, 1, 2046, 65, 506, 3000], np.int32)
    w = _f32_case(lens, 16, 8, 32, seed=2002, nparts_list=[0, 5], dist="student3x3")
    say(f"  worst err/tol {w:.3f}")


def test_f32_seq_len_one_is_v_row_bitwise():
    say("[mirror] seq_len 1")
    lens = np.array([1, 1, 1], np.int32)
    k, v = dense_kv(lens, 2, seed=2003)
    q = np.random.default_rng(2003).standard_normal((3, 8, 128)).astype(np.float32)
    dc = DeviceCache(lens, 2, 32, seed=2003, mirror=True)
    dc.append_dense(k, v)
    got = dc.decode_f32(q, 8, SCALE).cpu().numpy()
    for b in range(3):
        for h in range(8):
            np.testing.assert_array_equal(got[b, h].view(np.uint32), v[b, 0, h // 4].view(np.uint32))


def test_f32_without_mirror_is_rejected():
    t = torch()
    m = q8()
    dc = DeviceCache(np.array([40], np.int32), 2, 32, seed=2004)
    q = t.zeros((1, 4, 128), dtype=t.float32, device="cuda")
    out = t.empty_like(q)
    ws = t.empty(m.decode_attn_workspace_bytes(dc.layer, dc.batch, 4, 0), dtype=t.uint8, device="cuda")
    with pytest.raises(m.Q8Error):
        m.decode_attn_f32(dc.layer, dc.batch, 4, q, SCALE, out, ws)


def test_f32_graph_replays_match_eager():
    t = torch()
    m = q8()
    say("[mirror] graph capture / replay")
    lens = np.array([700, 65, 1, 300], np.int32)
    k, v = dense_kv(lens, 8, seed=2005)
    dc = DeviceCache(lens, 8, 32, seed=2005, mirror=True)
    dc.append_dense(k, v)
    rng = np.random.default_rng(2005)
    q = t.from_numpy(rng.standard_normal((4, 16, 128)).astype(np.float32)).cuda()
    kn = t.from_numpy(rng.standard_normal((4, 8, 128)).astype(np.float32)).cuda()
    vn = t.from_numpy(rng.standard_normal((4, 8, 128)).astype(np.float32)).cuda()
    seqs = t.arange(4, dtype=t.int32, device="cuda")
    pos = (dc.lens_t - 1).to(t.int32)
    ws = t.empty(m.decode_attn_workspace_bytes(dc.layer, dc.batch, 16, 0), dtype=t.uint8, device="cuda")
    out = t.empty((4, 16, 128), dtype=t.float32, device="cuda")

    def body():
        m.kv_append(dc.layer, dc.batch, seqs, pos, kn, vn, dev_status=dc.status)
        m.decode_attn_f32(dc.layer, dc.batch, 16, q, SCALE, out, ws, dev_status=dc.status)

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


def test_f32_phase_entry_points_equal_one_call():
    t = torch()
    m = q8()
    say("[mirror] f32 partial + merge == f32 decode")
    lens = np.array([1000, 70, 3], np.int32)
    k, v = dense_kv(lens, 8, seed=2006)
    q = t.from_numpy(np.random.default_rng(2006).standard_normal((3, 16, 128)).astype(np.float32)).cuda()
    dc = DeviceCache(lens, 8, 32, seed=2006, mirror=True)
    dc.append_dense(k, v)
    one = dc.decode_f32(q, 16, SCALE, nparts=9)
    ws = t.empty(m.decode_attn_workspace_bytes(dc.layer, dc.batch, 16, 9), dtype=t.uint8, device="cuda")
    out = t.empty_like(one)
    m.decode_attn_f32_partial(dc.layer, dc.batch, 16, q, SCALE, out, ws, nparts=9)
    m.decode_attn_merge(dc.layer, dc.batch, 16, q, SCALE, out, ws, nparts=9)
    assert t.equal(out, one)
