"""GPU tests of the batch-invariant cut (q8_batch.flags = Q8_BATCH_INVARIANT),
through the C ABI.

Every sequence is cut into chunks counted from its own start (128 positions,
256 from 4096 positions on, 512 from 16384 on), each chunk leaves its own
partial state, and the chunk states of a sequence are combined in chunk order
by a merge whose shape is fixed.  So a
sequence's output bits may depend on nothing but its own length, K, V and q:
the same sequence decoded alone, inside a larger batch, in another order, with
another partition count or with its blocks elsewhere in the pool gives the
same bits.  The outputs are also checked against the oracle (within the
tolerance), and the fused step, the fp32 mirror, the no-alloc step and graph
replay against their counterparts bit for bit.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import DeviceCache, assert_rows_close, dense_kv, q8, say, torch

pytestmark = pytest.mark.gpu
SCALE = float(workloads.softmax_scale(128))
# one chunk, exactly one chunk, one chunk and a token, many chunks, empty, single token
LENS = np.array([3000, 40, 1700, 1, 640, 2100, 0, 9000, 256, 257, 512, 33], np.int32)


def _bits(x):
    t = torch()
    return x.view(t.int32) if x.dtype == t.float32 else x.view(t.uint8)


def _invariant(dc):
    return q8().make_batch(dc.table_t, dc.lens_t, dc.max_seq_len, invariant=True)


def _cache(lens, nkv, kv_bs, k, v, seed, spare=2, mirror=False, upto=None):
    dc = DeviceCache(lens, nkv, kv_bs, seed=seed, spare=spare, mirror=mirror)
    if upto is not None:
        full = dc.lens
        dc.lens = np.maximum(full - 1, 0)
        dc.append_dense(k, v)
        dc.lens = full
    else:
        dc.append_dense(k, v)
    return dc


def _decode(dc, q, nq, nparts=0, f32=False):
    t, m = torch(), q8()
    b = _invariant(dc)
    qd = t.from_numpy(np.ascontiguousarray(q, np.float32)).cuda()
    out = t.full((b.batch, nq, 128), float("nan"), dtype=t.float32, device="cuda")
    ws = t.empty(m.decode_attn_workspace_bytes(dc.layer, b, nq, nparts), dtype=t.uint8, device="cuda")
    (m.decode_attn_f32 if f32 else m.decode_attn)(dc.layer, b, nq, qd, SCALE, out, ws, nparts=nparts,
                                                    dev_status=dc.status)
    assert dc.status_word() == 0
    return out


@pytest.mark.parametrize("group,kv_bs", [(2, 32), (4, 32), (1, 8), (8, 16), (4, 256)])
def test_bits_do_not_depend_on_the_rest_of_the_batch(group, kv_bs):
    nkv = 2
    nq = nkv * group
    say(f"[invariant] group={group} kv_bs={kv_bs}")
    k, v = dense_kv(LENS, nkv, seed=2000 + group)
    q = np.random.default_rng(2001).standard_normal((LENS.size, nq, 128)).astype(np.float32)
    full_dc = _cache(LENS, nkv, kv_bs, k, v, seed=3)
    full = _decode(full_dc, q, nq)
    # other partition counts, and other placements of the blocks
    for nparts in (1, 7, 300):
        assert t_equal(_decode(full_dc, q, nq, nparts=nparts), full), nparts
    moved = _cache(LENS, nkv, kv_bs, k, v, seed=11, spare=9)
    assert t_equal(_decode(moved, q, nq), full)
    # sub-batches, alone and reordered
    for idx in ([0], [7], [3], [8, 9, 10], [5, 4, 3, 2, 1, 0], [11, 7, 1, 9], list(range(LENS.size))[::-1]):
        idx = np.array(idx)
        dc = _cache(LENS[idx], nkv, kv_bs, k[idx], v[idx], seed=5 + len(idx))
        got = _decode(dc, q[idx], nq)
        assert t_equal(got, full[torch().from_numpy(idx).cuda()]), idx.tolist()


def t_equal(a, b):
    return bool(torch().equal(_bits(a), _bits(b)))


@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("kv_bs", [8, 32, 256])
def test_invariant_decode_against_the_oracle(group, kv_bs):
    nkv = 2
    nq = nkv * group
    say(f"[invariant] oracle group={group} kv_bs={kv_bs}")
    k, v = dense_kv(LENS, nkv, seed=2100 + group + kv_bs)
    q = np.random.default_rng(2101).standard_normal((LENS.size, nq, 128)).astype(np.float32)
    dc = _cache(LENS, nkv, kv_bs, k, v, seed=13)
    got = _decode(dc, q, nq).cpu().numpy()
    want = oracle.decode_attn(dc.host(), q, nq, SCALE)
    worst = assert_rows_close(got, want, "invariant")
    assert np.all(got[LENS == 0] == 0)
    say(f"  worst err/tol {worst:.3f}")


def test_invariant_2b_shape_with_heavy_tails():
    say("[invariant] 2B shape, student-t x3 with near-zero rows")
    lens = np.array([4059, 506, 2046, 1, 8192, 777], np.int32)
    k, v = dense_kv(lens, 8, seed=2200, dist="student3x3")
    q = np.random.default_rng(2201).standard_normal((lens.size, 16, 128)).astype(np.float32)
    dc = _cache(lens, 8, 32, k, v, seed=17)
    got = _decode(dc, q, 16).cpu().numpy()
    assert_rows_close(got, oracle.decode_attn(dc.host(), q, 16, SCALE), "2B invariant")


@pytest.mark.parametrize("group,kv_bs", [(2, 32), (4, 32), (1, 8)])
def test_invariant_step_equals_append_then_decode(group, kv_bs):
    # the fused append of the range that walks each sequence's last chunk:
    # every cache byte and output bit as q8_kv_append followed by the decode
    t, m = torch(), q8()
    nkv = 2
    nq = nkv * group
    say(f"[invariant] step group={group} kv_bs={kv_bs}")
    lens = LENS[LENS > 0]
    k, v = dense_kv(lens, nkv, seed=2300 + group)
    q = np.random.default_rng(2301).standard_normal((lens.size, nq, 128)).astype(np.float32)
    a = _cache(lens, nkv, kv_bs, k, v, seed=19, upto="last")
    b = _cache(lens, nkv, kv_bs, k, v, seed=19, upto="last")
    k_new = t.from_numpy(np.ascontiguousarray(np.stack([k[i, n - 1] for i, n in enumerate(lens)]))).cuda()
    v_new = t.from_numpy(np.ascontiguousarray(np.stack([v[i, n - 1] for i, n in enumerate(lens)]))).cuda()
    m.kv_append(b.layer, b.batch, t.arange(lens.size, dtype=t.int32, device="cuda"),
                (b.lens_t - 1).to(t.int32), k_new, v_new, dev_status=b.status)
    want = _decode(b, q, nq)
    ba = _invariant(a)
    qd = t.from_numpy(q).cuda()
    got = t.full_like(want, float("nan"))
    ws = t.empty(m.decode_attn_workspace_bytes(a.layer, ba, nq, 0), dtype=t.uint8, device="cuda")
    m.decode_step(a.layer, ba, nq, k_new, v_new, qd, SCALE, got, ws, dev_status=a.status)
    assert a.status_word() == 0 and b.status_word() == 0
    for name in ("k_codes", "v_codes", "k_scale", "v_scale"):
        assert t.equal(_bits(getattr(a.layer, name)), _bits(getattr(b.layer, name))), name
    assert t_equal(got, want)
    # and the no-alloc step gives the same bits (fresh twin cache)
    c = _cache(lens, nkv, kv_bs, k, v, seed=19, upto="last")
    got_s = t.full_like(want, float("nan"))
    m.decode_step_static(c.layer, _invariant(c), nq, k_new, v_new, qd, SCALE, got_s, dev_status=c.status)
    assert c.status_word() == 0
    assert t_equal(got_s, want)


def test_invariant_f32_mirror():
    say("[invariant] fp32 mirror")
    k, v = dense_kv(LENS, 4, seed=2400)
    q = np.random.default_rng(2401).standard_normal((LENS.size, 8, 128)).astype(np.float32)
    full_dc = _cache(LENS, 4, 32, k, v, seed=23, mirror=True)
    full = _decode(full_dc, q, 8, f32=True)
    assert_rows_close(full.cpu().numpy(), oracle.decode_attn_f32(full_dc.host_mirror(), q, 8, SCALE), "f32")
    idx = np.array([7, 0, 5])
    dc = _cache(LENS[idx], 4, 32, k[idx], v[idx], seed=29, mirror=True)
    assert t_equal(_decode(dc, q[idx], 8, f32=True), full[torch().from_numpy(idx).cuda()])
    assert t_equal(_decode(full_dc, q, 8, nparts=5, f32=True), full)


def test_invariant_graph_replays_match_eager():
    t, m = torch(), q8()
    say("[invariant] graph capture")
    k, v = dense_kv(LENS, 8, seed=2500)
    dc = _cache(LENS, 8, 32, k, v, seed=31)
    b = _invariant(dc)
    q = t.from_numpy(np.random.default_rng(2501).standard_normal((LENS.size, 16, 128)).astype(np.float32)).cuda()
    out = t.empty((LENS.size, 16, 128), dtype=t.float32, device="cuda")
    ws = t.empty(m.decode_attn_workspace_bytes(dc.layer, b, 16, 0), dtype=t.uint8, device="cuda")

    def step():
        m.decode_attn(dc.layer, b, 16, q, SCALE, out, ws, dev_status=dc.status)

    step()
    t.cuda.synchronize()
    eager = out.clone()
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        step()
    t.cuda.current_stream().wait_stream(side)
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        step()
    for i in range(3):
        out.fill_(float("nan"))
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        assert t_equal(out, eager), f"replay {i}"
    assert dc.status_word() == 0


@pytest.mark.parametrize("lens", [[4064, 4096, 4097, 300], [16352, 16384, 17000, 300]])
def test_long_sequences_use_longer_chunks_and_stay_invariant(lens):
    # either side of each doubling of the chunk length (127 / 128 / 129 tiles:
    # 128 -> 256 positions; 511 / 512 / 532 tiles: 256 -> 512 positions): the
    # chunk length follows the sequence's own length only
    say(f"[invariant] chunk length thresholds {lens}")
    lens = np.array(lens, np.int32)
    k, v = dense_kv(lens, 2, seed=2600)
    q = np.random.default_rng(2601).standard_normal((lens.size, 4, 128)).astype(np.float32)
    dc = _cache(lens, 2, 32, k, v, seed=37)
    full = _decode(dc, q, 4)
    assert_rows_close(full.cpu().numpy(), oracle.decode_attn(dc.host(), q, 4, SCALE), "long chunks")
    for idx in ([0], [1], [2, 3], [3, 2, 1, 0]):
        idx = np.array(idx)
        sub = _cache(lens[idx], 2, 32, k[idx], v[idx], seed=41 + len(idx))
        assert t_equal(_decode(sub, q[idx], 4), full[torch().from_numpy(idx).cuda()]), idx.tolist()
    assert t_equal(_decode(dc, q, 4, nparts=3), full)
