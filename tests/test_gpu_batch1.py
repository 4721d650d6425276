"""GPU tests of a batch of one sequence, through the C ABI.

With one sequence the automatic cut gives every range one 32-token tile (up
to one range per resident workgroup slot), so nearly every result goes
through the (M, S, acc) records and the merge kernel; a sequence of one tile
is finished in place.  The results are checked against the oracle within the
tolerance over lengths from one token to several hundred tiles, every group
size and block size, and bit for bit where the method fixes them (one token:
the dequantized V row).  The fused step, the fp32 mirror, a step plan, the
no-alloc step and graph replay must each equal their counterpart bit for
bit, since the same kernels run on the same data.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import DeviceCache, assert_rows_close, dense_kv, q8, say, torch

pytestmark = pytest.mark.gpu
SCALE = float(workloads.softmax_scale(128))
# 1 to 282 tiles: in place, a few ranges, many ranges
BATCH1_LENS = [1, 2, 33, 100, 257, 512, 513, 3000, 9000]


def _bits(x):
    t = torch()
    return x.view(t.int32) if x.dtype == t.float32 else x.view(t.uint8)


def _filled(n, nkv, kv_bs, seed, mirror=False, upto=None):
    lens = np.array([n], np.int32)
    k, v = dense_kv(lens, nkv, seed=seed)
    dc = DeviceCache(lens, nkv, kv_bs, seed=seed, mirror=mirror)
    if upto is None:
        dc.append_dense(k, v)
    else:
        dc.lens = np.minimum(lens, upto)
        dc.append_dense(k, v)
        dc.lens = lens
    return dc, k, v


def _q(nq, seed):
    return np.random.default_rng([seed, 5]).standard_normal((1, nq, 128)).astype(np.float32)


def test_a_batch_of_one_is_cut_into_one_tile_per_range():
    # fewer tiles than resident workgroup slots: one range per tile
    m = q8()
    for n in (1, 32, 33, 512, 3000):
        dc, _, _ = _filled(n, 2, 32, seed=5, upto=0)
        assert m.decode_attn_auto_parts(dc.layer, dc.batch, 4) == (n + 31) // 32, n


@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("kv_bs", [8, 32, 256])
def test_batch1_decode_against_the_oracle(group, kv_bs):
    nkv = 2
    nq = nkv * group
    worst = 0.0
    for n in BATCH1_LENS:
        say(f"[batch1] group={group} kv_bs={kv_bs} n={n}")
        seed = 1200 + 10 * group + kv_bs + n
        dc, _, _ = _filled(n, nkv, kv_bs, seed)
        q = _q(nq, seed)
        got = dc.decode(q, nq, SCALE).cpu().numpy()
        assert dc.status_word() == 0
        want = oracle.decode_attn(dc.host(), q, nq, SCALE)
        worst = max(worst, assert_rows_close(got, want, f"n={n}"))
    say(f"  worst err/tol {worst:.3f}")


def test_batch1_many_kv_heads_and_student_t():
    # 12 KV heads (two workgroups per range), heavy-tailed x3 values with
    # near-zero rows, the 2B and 8B group sizes
    for nkv, group, n, dist in ((12, 2, 3000, "student3x3"), (8, 4, 2047, "student3x3"), (8, 2, 4059, "normal")):
        say(f"[batch1] nkv={nkv} group={group} n={n} {dist}")
        lens = np.array([n], np.int32)
        k, v = dense_kv(lens, nkv, seed=n, dist=dist)
        dc = DeviceCache(lens, nkv, 32, seed=n)
        dc.append_dense(k, v)
        q = _q(nkv * group, n)
        got = dc.decode(q, nkv * group, SCALE).cpu().numpy()
        assert dc.status_word() == 0
        assert_rows_close(got, oracle.decode_attn(dc.host(), q, nkv * group, SCALE), f"nkv={nkv}")


@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_batch1_seq_len_one_is_dequantized_v_bitwise(group):
    # one token: one range finishes it in place with w = 1 and S = 1, so the
    # output is float(code) * step bit for bit
    nkv = 2
    dc, k, v = _filled(1, nkv, 32, seed=77 + group)
    got = dc.decode(_q(nkv * group, 77), nkv * group, SCALE).cpu().numpy()
    for h in range(nkv * group):
        cv, dv = oracle.quantize_kv(v[0, 0, h // group])
        want = (cv.astype(np.float32) * dv).astype(np.float32)
        np.testing.assert_array_equal(got[0, h].view(np.uint32), want.view(np.uint32))


def test_batch1_empty_sequence_gives_zero_rows():
    t = torch()
    lens = np.array([0], np.int32)
    dc = DeviceCache(lens, 2, 32, seed=3)
    out = dc.decode(_q(4, 3), 4, SCALE)
    assert dc.status_word() == 0
    assert bool((out == 0).all())


@pytest.mark.parametrize("group,kv_bs", [(1, 8), (2, 32), (4, 32), (4, 8), (8, 16)])
def test_batch1_step_equals_append_then_decode(group, kv_bs):
    # the fused append of the range that holds the last tile: every cache
    # byte and output bit as q8_kv_append followed by q8_decode_attn
    t, m = torch(), q8()
    nkv = 2
    nq = nkv * group
    for n in (1, 2, 33, 512, 513, 3000):
        say(f"[batch1] step group={group} kv_bs={kv_bs} n={n}")
        seed = 1300 + group + kv_bs + n
        a, k, v = _filled(n, nkv, kv_bs, seed, upto=n - 1)
        b, _, _ = _filled(n, nkv, kv_bs, seed, upto=n - 1)
        k_new = t.from_numpy(np.ascontiguousarray(k[:, n - 1])).cuda()
        v_new = t.from_numpy(np.ascontiguousarray(v[:, n - 1])).cuda()
        q = t.from_numpy(_q(nq, seed)).cuda()
        m.kv_append(b.layer, b.batch, t.zeros(1, dtype=t.int32, device="cuda"),
                    t.full((1,), n - 1, dtype=t.int32, device="cuda"), k_new, v_new, dev_status=b.status)
        want = b.decode(q, nq, SCALE)
        got = t.full((1, nq, 128), float("nan"), dtype=t.float32, device="cuda")
        ws = t.empty(m.decode_attn_workspace_bytes(a.layer, a.batch, nq, 0), dtype=t.uint8, device="cuda")
        m.decode_step(a.layer, a.batch, nq, k_new, v_new, q, SCALE, got, ws, dev_status=a.status)
        assert a.status_word() == 0 and b.status_word() == 0
        for name in ("k_codes", "v_codes", "k_scale", "v_scale"):
            assert t.equal(_bits(getattr(a.layer, name)), _bits(getattr(b.layer, name))), name
        assert t.equal(_bits(got), _bits(want)), f"n={n}"
        if n == 3000:
            assert_rows_close(got.cpu().numpy(), oracle.decode_attn(a.host(), q.cpu().numpy(), nq, SCALE), "step")


@pytest.mark.parametrize("group", [1, 2, 4])
def test_batch1_f32_mirror_against_the_oracle(group):
    nkv = 2
    nq = nkv * group
    for n in (1, 100, 513, 3000):
        say(f"[batch1] f32 group={group} n={n}")
        dc, _, _ = _filled(n, nkv, 32, seed=1400 + n + group, mirror=True)
        q = _q(nq, n)
        got = dc.decode_f32(q, nq, SCALE).cpu().numpy()
        assert dc.status_word() == 0
        assert_rows_close(got, oracle.decode_attn_f32(dc.host_mirror(), q, nq, SCALE), f"n={n}")


def _plan_for(dc, nq, nparts=0):
    t, m = torch(), q8()
    plan = t.empty(m.decode_plan_bytes(dc.layer, dc.batch, nq, nparts), dtype=t.uint8, device="cuda")
    plan.fill_(0xA5)
    m.decode_plan(dc.layer, dc.batch, nq, plan, nparts=nparts, dev_status=dc.status)
    return dc.batch.with_plan(plan)


def test_batch1_with_a_plan_equals_without_and_a_foreign_plan_is_refused():
    t, m = torch(), q8()
    for n in (300, 3000):
        say(f"[batch1] planned n={n}")
        dc, _, _ = _filled(n, 8, 32, seed=1500 + n)
        q = t.from_numpy(_q(16, n)).cuda()
        ref = dc.decode(q, 16, SCALE)
        ws = t.empty(m.decode_attn_workspace_bytes(dc.layer, dc.batch, 16, 0), dtype=t.uint8, device="cuda")
        got = t.full_like(ref, float("nan"))
        m.decode_attn(dc.layer, _plan_for(dc, 16), 16, q, SCALE, got, ws, dev_status=dc.status)
        assert dc.status_word() == 0
        assert t.equal(_bits(got), _bits(ref))
    # a plan cut for another partition count: refused on the device, nothing
    # written -- by the partial kernel and by the merge (which reads the
    # plan's prefix only when the plan's header matches the call)
    foreign = _plan_for(dc, 16, nparts=5)
    assert dc.status_word() == 0
    out = t.full((1, 16, 128), 123.0, dtype=t.float32, device="cuda")
    m.decode_attn(dc.layer, foreign, 16, q, SCALE, out, ws, dev_status=dc.status)
    assert dc.status_word() & m.DEV_BAD_PLAN
    assert bool((out == 123.0).all())


def test_batch1_static_step_equals_step():
    t, m = torch(), q8()
    for n in (257, 9000):
        say(f"[batch1] static step n={n}")
        a, k, v = _filled(n, 8, 32, seed=1600 + n, upto=n - 1)
        b, _, _ = _filled(n, 8, 32, seed=1600 + n, upto=n - 1)
        k_new = t.from_numpy(np.ascontiguousarray(k[:, n - 1])).cuda()
        v_new = t.from_numpy(np.ascontiguousarray(v[:, n - 1])).cuda()
        q = t.from_numpy(_q(32, n)).cuda()
        out_a = t.full((1, 32, 128), float("nan"), dtype=t.float32, device="cuda")
        out_b = out_a.clone()
        ws = t.empty(m.decode_attn_workspace_bytes(a.layer, a.batch, 32, 0), dtype=t.uint8, device="cuda")
        m.decode_step(a.layer, a.batch, 32, k_new, v_new, q, SCALE, out_a, ws, dev_status=a.status)
        m.decode_step_static(b.layer, b.batch, 32, k_new, v_new, q, SCALE, out_b, dev_status=b.status)
        assert a.status_word() == 0 and b.status_word() == 0
        assert t.equal(_bits(out_a), _bits(out_b))
        for name in ("k_codes", "v_codes", "k_scale", "v_scale"):
            assert t.equal(_bits(getattr(a.layer, name)), _bits(getattr(b.layer, name))), name


def test_batch1_graph_replays_match_eager():
    # a captured batch-1 decode over two layers: every replay equals the
    # eager result
    t, m = torch(), q8()
    say("[batch1] graph capture")
    layers = [_filled(n, 8, 32, seed=1700 + n)[0] for n in (400, 5000)]
    q = t.from_numpy(_q(16, 1700)).cuda()
    outs = [t.empty((1, 16, 128), dtype=t.float32, device="cuda") for _ in layers]
    wss = [t.empty(m.decode_attn_workspace_bytes(dc.layer, dc.batch, 16, 0), dtype=t.uint8, device="cuda")
           for dc in layers]

    def step():
        for dc, o, ws in zip(layers, outs, wss):
            m.decode_attn(dc.layer, dc.batch, 16, q, SCALE, o, ws, dev_status=dc.status)

    step()
    t.cuda.synchronize()
    eager = [o.clone() for o in outs]
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        step()
    t.cuda.current_stream().wait_stream(side)
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        step()
    for i in range(3):
        for o in outs:
            o.fill_(float("nan"))
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert t.equal(_bits(o), _bits(e)), f"replay {i}"
    assert all(dc.status_word() == 0 for dc in layers)
