"""GPU tests of q8_decode_step: the append of each sequence's newest token
fused into the decode's partial kernel must equal q8_kv_append followed by
q8_decode_attn -- every cache byte (codes, steps, fp32 mirror) and every
output bit for bit (the same quantizer and the same attention kernels run on
the same data)."""
import numpy as np
import pytest

import workloads
from gpu_cases import DeviceCache, dense_kv, q8, say, torch

pytestmark = pytest.mark.gpu
SCALE = float(workloads.softmax_scale(128))
LENS = [1, 2, 31, 32, 33, 64, 65, 100, 257, 1000, 2049]


def _pair(lens, nkv, kv_bs, seed, mirror=False):
    """Two identical caches (same placement, same junk in unused rows) holding
    every position but the last of each sequence."""
    t = torch()
    lens = np.asarray(lens, np.int32)
    k, v = dense_kv(lens, nkv, seed=seed)
    caches = []
    for _ in range(2):
        dc = DeviceCache(lens, nkv, kv_bs, seed=seed, mirror=mirror)
        seqs = np.concatenate([np.full(n - 1, b, np.int32) for b, n in enumerate(lens) if n > 1])
        poss = np.concatenate([np.arange(n - 1, dtype=np.int32) for n in lens if n > 1])
        kh = np.concatenate([k[b, :n - 1] for b, n in enumerate(lens) if n > 1])
        vh = np.concatenate([v[b, :n - 1] for b, n in enumerate(lens) if n > 1])
        q8().kv_append(dc.layer, dc.batch, t.from_numpy(seqs).cuda(), t.from_numpy(poss).cuda(),
                       t.from_numpy(np.ascontiguousarray(kh)).cuda(), t.from_numpy(np.ascontiguousarray(vh)).cuda(),
                       dev_status=dc.status)
        caches.append(dc)
    k_new = np.ascontiguousarray(np.stack([k[b, n - 1] for b, n in enumerate(lens)]))
    v_new = np.ascontiguousarray(np.stack([v[b, n - 1] for b, n in enumerate(lens)]))
    return caches, t.from_numpy(k_new).cuda(), t.from_numpy(v_new).cuda()


def _separate(dc, k_new, v_new, q, nq, nparts):
    t, m = torch(), q8()
    B = dc.batch.batch
    m.kv_append(dc.layer, dc.batch, t.arange(B, dtype=t.int32, device="cuda"), (dc.lens_t - 1).to(t.int32), k_new,
                v_new, dev_status=dc.status)
    return dc.decode(q, nq, SCALE, nparts=nparts)


def _fused(dc, k_new, v_new, q, nq, nparts):
    t, m = torch(), q8()
    out = t.full((dc.batch.batch, nq, 128), float("nan"), dtype=t.float32, device="cuda")
    ws = t.empty(m.decode_attn_workspace_bytes(dc.layer, dc.batch, nq, nparts), dtype=t.uint8, device="cuda")
    m.decode_step(dc.layer, dc.batch, nq, k_new, v_new, q, SCALE, out, ws, nparts=nparts, dev_status=dc.status)
    return out


def _same_cache(a, b, mirror=False):
    names = ["k_codes", "v_codes", "k_scale", "v_scale"] + (["k_f32", "v_f32"] if mirror else [])
    t = torch()
    for nm in names:
        x, y = getattr(a.layer, nm), getattr(b.layer, nm)
        assert t.equal(x.view(t.uint8) if x.dtype == t.int8 else x.view(t.int32),
                       y.view(t.uint8) if y.dtype == t.int8 else y.view(t.int32)), nm


@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("kv_bs", [8, 32, 64])
def test_step_equals_append_then_decode(group, kv_bs):
    say(f"[step] group={group} kv_bs={kv_bs}")
    t = torch()
    nkv, nq = 2, 2 * group
    (a, b), k_new, v_new = _pair(LENS, nkv, kv_bs, seed=950 + group + kv_bs)
    q = t.from_numpy(np.random.default_rng(951).standard_normal((len(LENS), nq, 128)).astype(np.float32)).cuda()
    for nparts in (0, 1, 7):
        want = _separate(b, k_new, v_new, q, nq, nparts)
        got = _fused(a, k_new, v_new, q, nq, nparts)
        assert a.status_word() == 0 and b.status_word() == 0
        _same_cache(a, b)
        assert t.equal(got, want), f"nparts={nparts}"


def test_step_wide_batch():
    # 131 sequences (more than one 64-entry step of the range lookups), short
    # and tile-edge lengths around the step edges
    say("[step] 131 sequences")
    t = torch()
    lens = np.random.default_rng(78).integers(1, 300, 131).astype(np.int32)
    lens[[62, 63, 64, 65, 127, 128, 130]] = [1, 32, 33, 31, 1, 64, 2]
    nkv, nq = 2, 4
    (a, b), k_new, v_new = _pair(lens, nkv, 32, seed=978)
    q = t.from_numpy(np.random.default_rng(979).standard_normal((len(lens), nq, 128)).astype(np.float32)).cuda()
    for nparts in (0, 3, 65, 300):
        want = _separate(b, k_new, v_new, q, nq, nparts)
        got = _fused(a, k_new, v_new, q, nq, nparts)
        assert a.status_word() == 0 and b.status_word() == 0
        _same_cache(a, b)
        assert t.equal(got, want), f"nparts={nparts}"


def test_step_with_mirror_and_8b_shape():
    say("[step] 8B shape with the fp32 mirror")
    t = torch()
    (a, b), k_new, v_new = _pair(LENS, 8, 32, seed=960, mirror=True)
    q = t.from_numpy(np.random.default_rng(961).standard_normal((len(LENS), 32, 128)).astype(np.float32)).cuda()
    want = _separate(b, k_new, v_new, q, 32, 0)
    got = _fused(a, k_new, v_new, q, 32, 0)
    _same_cache(a, b, mirror=True)
    assert t.equal(got, want)


def test_step_bad_block_id_is_reported_and_skipped():
    # the block that would hold sequence 1's new token is out of range: flagged,
    # its row not written (as q8_kv_append); the other sequences are appended
    say("[step] bad block id at the new position")
    t = torch()
    lens = [40, 70, 9]
    (a, b), k_new, v_new = _pair(lens, 2, 32, seed=970)
    for dc in (a, b):
        dc.table_t[1, (70 - 1) // 32] = dc.num_blocks + 3
    q = t.from_numpy(np.random.default_rng(971).standard_normal((3, 4, 128)).astype(np.float32)).cuda()
    _separate(b, k_new, v_new, q, 4, 0)
    _fused(a, k_new, v_new, q, 4, 0)
    assert a.status_word() & 0x2 and b.status_word() & 0x2
    _same_cache(a, b)


def test_step_graph_replays():
    say("[step] graph capture / replay")
    t, m = torch(), q8()
    (a, b), k_new, v_new = _pair(LENS, 8, 32, seed=980)
    q = t.from_numpy(np.random.default_rng(981).standard_normal((len(LENS), 16, 128)).astype(np.float32)).cuda()
    out = t.empty((len(LENS), 16, 128), dtype=t.float32, device="cuda")
    ws = t.empty(m.decode_attn_workspace_bytes(a.layer, a.batch, 16, 0), dtype=t.uint8, device="cuda")

    def body():
        m.decode_step(a.layer, a.batch, 16, k_new, v_new, q, SCALE, out, ws, dev_status=a.status)

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
    want = _separate(b, k_new, v_new, q, 16, 0)
    assert t.equal(eager, want)
    _same_cache(a, b)
    assert a.status_word() == 0
