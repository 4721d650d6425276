"""q8_decode_step_static (the decode step for callers that cannot allocate)
against q8_decode_step, through the C ABI: two calls in a row on twin caches,
the second on a smaller batch, outputs and every cache byte identical; a plan
larger than the library's scratch is refused before anything runs."""
import numpy as np
import pytest

import workloads
from gpu_cases import DeviceCache, dense_kv, q8, say, torch

pytestmark = pytest.mark.gpu
SCALE = float(workloads.softmax_scale(128))


def _twins(lens, nq, nkv, kv_bs, seed):
    """Two identical caches (same placement, same junk in unused rows)
    holding every position but each sequence's last."""
    lens = np.asarray(lens, np.int32)
    k, v = dense_kv(lens, nkv, seed=seed)
    hist = np.maximum(lens - 1, 0)
    a = DeviceCache(lens, nkv, kv_bs, seed=seed)
    b = DeviceCache(lens, nkv, kv_bs, seed=seed)
    for dc in (a, b):
        dc.lens = hist
        dc.append_dense(k, v)
        dc.lens = lens
    rng = np.random.default_rng([seed, 9])
    t = torch()
    k_new = t.from_numpy(rng.standard_normal((len(lens), nkv, 128)).astype(np.float32)).cuda()
    v_new = t.from_numpy(rng.standard_normal((len(lens), nkv, 128)).astype(np.float32)).cuda()
    q = t.from_numpy(rng.standard_normal((len(lens), nq, 128)).astype(np.float32)).cuda()
    return a, b, k_new, v_new, q


def _compare(lens, nq, nkv, kv_bs, seed, nparts):
    t, m = torch(), q8()
    a, b, k_new, v_new, q = _twins(lens, nq, nkv, kv_bs, seed)
    out_a = t.full((len(lens), nq, 128), float("nan"), dtype=t.float32, device="cuda")
    out_b = out_a.clone()
    ws = t.empty(m.decode_attn_workspace_bytes(a.layer, a.batch, nq, nparts), dtype=t.uint8, device="cuda")
    m.decode_step(a.layer, a.batch, nq, k_new, v_new, q, SCALE, out_a, ws, nparts=nparts, dev_status=a.status)
    m.decode_step_static(b.layer, b.batch, nq, k_new, v_new, q, SCALE, out_b, nparts=nparts, dev_status=b.status)
    assert a.status_word() == 0 and b.status_word() == 0
    assert t.equal(out_a, out_b), "outputs differ"
    for name in ("k_codes", "v_codes", "k_scale", "v_scale"):
        # bit patterns: rows no token occupies hold NaN scales on purpose
        x, y = getattr(a.layer, name), getattr(b.layer, name)
        if x.dtype == t.float32:
            x, y = x.view(t.int32), y.view(t.int32)
        assert t.equal(x, y), name


def test_static_step_equals_workspace_step_twice_then_smaller():
    # first a large batch (the 8B shape, many ranges), then a smaller one: the
    # second call reads none of what the first left in the scratch
    say("[static] 8B shape, 40 sequences, then 2B shape, 5 sequences")
    lens1 = np.random.default_rng(1).integers(1, 3000, 40).astype(np.int32)
    lens1[:4] = [1, 33, 64, 0]
    _compare(lens1, 32, 8, 32, seed=71, nparts=0)
    _compare([700, 1, 65, 0, 2049], 16, 8, 32, seed=72, nparts=0)
    _compare([700, 1, 65, 0, 2049], 16, 8, 8, seed=73, nparts=7)


def test_static_step_refuses_a_plan_larger_than_its_scratch():
    t, m = torch(), q8()
    say("[static] plan larger than the scratch")
    lens = np.full(8, 4096, np.int32)
    dc = DeviceCache(lens, 8, 32, seed=74)
    nq = 64
    nparts = 1024
    need = m.decode_attn_workspace_bytes(dc.layer, dc.batch, nq, nparts)
    assert need > m.decode_step_static_scratch_bytes()
    x = t.zeros((8, 8, 128), dtype=t.float32, device="cuda")
    q = t.zeros((8, nq, 128), dtype=t.float32, device="cuda")
    out = t.zeros((8, nq, 128), dtype=t.float32, device="cuda")
    with pytest.raises(m.Q8Error) as e:
        m.decode_step_static(dc.layer, dc.batch, nq, x, x, q, SCALE, out, nparts=nparts, dev_status=dc.status)
    assert e.value.status == m.Q8_EWORKSPACE
