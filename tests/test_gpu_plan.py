"""The step plan (q8_decode_plan, q8_batch.plan) on the GPU, through the C ABI.

A decode call that reads a plan walks the same pieces as one that makes the
cut itself, so its outputs -- and, for q8_decode_step, every cache byte it
writes -- must equal the unplanned call's bit for bit; the unplanned calls
are checked against the oracle elsewhere, and one case here is checked
against the oracle directly.  A plan made for another partition count is
detected on the device.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import DeviceCache, assert_rows_close, dense_kv, q8, say, torch

pytestmark = pytest.mark.gpu
SCALE = float(workloads.softmax_scale(128))
EDGE = [0, 1, 2, 7, 8, 9, 31, 32, 33, 63, 64, 65, 100, 255, 256, 257, 700, 0]


def _bits(x):
    t = torch()
    return x.view(t.int32) if x.dtype == t.float32 else x


def _planned(dc, nq, nparts):
    t, m = torch(), q8()
    plan = t.empty(m.decode_plan_bytes(dc.layer, dc.batch, nq, nparts), dtype=t.uint8, device="cuda")
    plan.fill_(0xA5)
    m.decode_plan(dc.layer, dc.batch, nq, plan, nparts=nparts, dev_status=dc.status)
    return dc.batch.with_plan(plan)


def _inputs(lens, nq, nkv, seed):
    t = torch()
    rng = np.random.default_rng([seed, 3])
    q = t.from_numpy(rng.standard_normal((len(lens), nq, 128)).astype(np.float32)).cuda()
    kn = t.from_numpy(rng.standard_normal((len(lens), nkv, 128)).astype(np.float32)).cuda()
    vn = t.from_numpy(rng.standard_normal((len(lens), nkv, 128)).astype(np.float32)).cuda()
    return q, kn, vn


def _cache(lens, nkv, kv_bs, seed, mirror=False, full=False):
    """A cache holding every position but each sequence's last (the one a
    decode step appends), or every position with full=True."""
    lens = np.asarray(lens, np.int32)
    k, v = dense_kv(lens, nkv, seed=seed)
    dc = DeviceCache(lens, nkv, kv_bs, seed=seed, mirror=mirror)
    dc.lens = lens if full else np.maximum(lens - 1, 0)
    dc.append_dense(k, v)
    dc.lens = lens
    return dc, k, v


@pytest.mark.parametrize("group,kv_bs", [(1, 32), (2, 8), (2, 32), (4, 16), (4, 32), (4, 256), (8, 64)])
@pytest.mark.parametrize("nparts", [0, 1, 7, 300])
def test_planned_decode_equals_unplanned_bitwise(group, kv_bs, nparts):
    t, m = torch(), q8()
    nkv = 2
    nq = nkv * group
    say(f"[plan] decode group={group} kv_bs={kv_bs} nparts={nparts}")
    dc, _, _ = _cache(EDGE, nkv, kv_bs, seed=810 + group + kv_bs)
    q, _, _ = _inputs(EDGE, nq, nkv, 811)
    ws = t.empty(m.decode_attn_workspace_bytes(dc.layer, dc.batch, nq, nparts), dtype=t.uint8, device="cuda")
    ref = t.full((len(EDGE), nq, 128), float("nan"), dtype=t.float32, device="cuda")
    m.decode_attn(dc.layer, dc.batch, nq, q, SCALE, ref, ws, nparts=nparts, dev_status=dc.status)
    pb = _planned(dc, nq, nparts)
    got = t.full_like(ref, float("nan"))
    ws.fill_(0x5A)
    m.decode_attn(dc.layer, pb, nq, q, SCALE, got, ws, nparts=nparts, dev_status=dc.status)
    assert dc.status_word() == 0
    assert t.equal(_bits(got), _bits(ref))


@pytest.mark.parametrize("group,kv_bs,nkv", [(2, 32, 8), (4, 32, 8), (1, 8, 12), (8, 16, 2)])
@pytest.mark.parametrize("nparts", [0, 3, 65])
def test_planned_step_equals_unplanned_bitwise(group, kv_bs, nkv, nparts):
    # the fused append reads its block ids from the plan: every cache byte and
    # output bit as the unplanned step (twin caches, same placement and junk)
    t, m = torch(), q8()
    nq = nkv * group
    say(f"[plan] step group={group} kv_bs={kv_bs} nkv={nkv} nparts={nparts}")
    seed = 820 + group + kv_bs + nkv
    a, _, _ = _cache(EDGE, nkv, kv_bs, seed)
    b, _, _ = _cache(EDGE, nkv, kv_bs, seed)
    q, kn, vn = _inputs(EDGE, nq, nkv, seed)
    ws = t.empty(m.decode_attn_workspace_bytes(a.layer, a.batch, nq, nparts), dtype=t.uint8, device="cuda")
    out_a = t.full((len(EDGE), nq, 128), float("nan"), dtype=t.float32, device="cuda")
    out_b = out_a.clone()
    m.decode_step(a.layer, a.batch, nq, kn, vn, q, SCALE, out_a, ws, nparts=nparts, dev_status=a.status)
    pb = _planned(b, nq, nparts)
    m.decode_step(b.layer, pb, nq, kn, vn, q, SCALE, out_b, ws, nparts=nparts, dev_status=b.status)
    assert a.status_word() == 0 and b.status_word() == 0
    assert t.equal(_bits(out_a), _bits(out_b))
    for name in ("k_codes", "v_codes", "k_scale", "v_scale"):
        assert t.equal(_bits(getattr(a.layer, name)), _bits(getattr(b.layer, name))), name


def test_planned_ragged_batch_against_the_oracle_and_many_sequences():
    # 131 sequences with empty ones at the edges of 64-entry groups, the
    # 2B shape, automatic and wide cuts; planned against unplanned bit for
    # bit and the automatic one against the oracle
    t, m = torch(), q8()
    say("[plan] 131 sequences, 2B shape")
    rng = np.random.default_rng(830)
    lens = rng.integers(1, 3000, 131).astype(np.int32)
    lens[[0, 63, 64, 127, 128, 130]] = 0
    dc, k, v = _cache(lens, 8, 32, 830, full=True)
    q, kn, vn = _inputs(lens, 16, 8, 830)
    for nparts in (0, 5000):
        ws = t.empty(m.decode_attn_workspace_bytes(dc.layer, dc.batch, 16, nparts), dtype=t.uint8, device="cuda")
        ref = t.empty((len(lens), 16, 128), dtype=t.float32, device="cuda")
        m.decode_attn(dc.layer, dc.batch, 16, q, SCALE, ref, ws, nparts=nparts, dev_status=dc.status)
        got = t.full_like(ref, float("nan"))
        m.decode_attn(dc.layer, _planned(dc, 16, nparts), 16, q, SCALE, got, ws, nparts=nparts,
                      dev_status=dc.status)
        assert dc.status_word() == 0
        assert t.equal(_bits(got), _bits(ref)), nparts
    want = oracle.decode_attn(dc.host(), q.cpu().numpy(), 16, SCALE)
    worst = assert_rows_close(got.cpu().numpy(), want, "planned 131 sequences")
    say(f"  worst err/tol {worst:.3f}")


def test_planned_f32_mirror_and_static_step():
    t, m = torch(), q8()
    say("[plan] fp32 mirror decode and the no-alloc step")
    lens = np.array([300, 0, 65, 1, 2049, 31], np.int32)
    dc, _, _ = _cache(lens, 8, 32, 840, mirror=True)
    q, kn, vn = _inputs(lens, 32, 8, 840)
    ws = t.empty(m.decode_attn_workspace_bytes(dc.layer, dc.batch, 32, 0), dtype=t.uint8, device="cuda")
    ref = t.empty((len(lens), 32, 128), dtype=t.float32, device="cuda")
    m.decode_attn_f32(dc.layer, dc.batch, 32, q, SCALE, ref, ws, dev_status=dc.status)
    pb = _planned(dc, 32, 0)
    got = t.full_like(ref, float("nan"))
    m.decode_attn_f32(dc.layer, pb, 32, q, SCALE, got, ws, dev_status=dc.status)
    assert t.equal(_bits(got), _bits(ref))
    a, _, _ = _cache(lens, 8, 32, 841)
    b, _, _ = _cache(lens, 8, 32, 841)
    out_a = t.empty((len(lens), 32, 128), dtype=t.float32, device="cuda")
    out_b = t.full_like(out_a, float("nan"))
    m.decode_step_static(a.layer, a.batch, 32, kn, vn, q, SCALE, out_a, dev_status=a.status)
    m.decode_step_static(b.layer, _planned(b, 32, 0), 32, kn, vn, q, SCALE, out_b, dev_status=b.status)
    assert dc.status_word() == 0 and a.status_word() == 0 and b.status_word() == 0
    assert t.equal(_bits(out_a), _bits(out_b))


def test_plan_for_another_partition_count_is_refused():
    t, m = torch(), q8()
    say("[plan] mismatched plan")
    lens = np.array([300, 65, 1000], np.int32)
    dc, _, _ = _cache(lens, 2, 32, 850)
    q, _, _ = _inputs(lens, 4, 2, 850)
    pb = _planned(dc, 4, 7)
    assert dc.status_word() == 0
    out = t.full((3, 4, 128), 123.0, dtype=t.float32, device="cuda")
    ws = t.empty(m.decode_attn_workspace_bytes(dc.layer, dc.batch, 4, 8), dtype=t.uint8, device="cuda")
    m.decode_attn_partial(dc.layer, pb, 4, q, SCALE, out, ws, nparts=8, dev_status=dc.status)
    assert dc.status_word() & m.DEV_BAD_PLAN
    assert bool((out == 123.0).all())   # nothing written


def test_planned_step_graph_replays_match_eager():
    # one captured decode step over two layers with a plan made inside the
    # graph: every replay equals the eager planned step
    t, m = torch(), q8()
    say("[plan] graph capture: plan + two layers")
    lens = np.array([700, 1, 65, 2049, 0, 300], np.int32)
    layers = [_cache(lens, 8, 32, 860 + i)[0] for i in range(2)]
    q, kn, vn = _inputs(lens, 16, 8, 860)
    dc0 = layers[0]
    plan = t.empty(m.decode_plan_bytes(dc0.layer, dc0.batch, 16, 0), dtype=t.uint8, device="cuda")
    ws = t.empty(m.decode_attn_workspace_bytes(dc0.layer, dc0.batch, 16, 0), dtype=t.uint8, device="cuda")
    outs = [t.empty((len(lens), 16, 128), dtype=t.float32, device="cuda") for _ in layers]
    pb = dc0.batch.with_plan(plan)

    def step():
        m.decode_plan(dc0.layer, dc0.batch, 16, plan, dev_status=dc0.status)
        for dc, o in zip(layers, outs):
            m.decode_attn(dc.layer, pb, 16, q, SCALE, o, ws, dev_status=dc0.status)

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
        plan.fill_(0)
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert t.equal(_bits(o), _bits(e)), f"replay {i}"
    assert dc0.status_word() == 0
