"""GPU parity at the full sizes of the batched workloads, in the launch
configuration bench.py times (automatic partition count), on sampled rows.

The caches are filled through q8_kv_append from GPU-drawn K/V with each
workload's value distribution; the oracle then reads the codes and steps back
and computes the sampled (sequence, query head) rows one by one.  Rows must
satisfy max |gpu - oracle| <= 2e-5 * max |oracle| + 1e-6.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import DeviceCache, assert_rows_close, q8, say, torch

pytestmark = pytest.mark.gpu
SCALE = float(workloads.softmax_scale(128))
CHUNK = 1 << 16   # tokens appended per call


def _filled(w, seed, mirror=False):
    """One layer of workload w on the GPU, every position appended."""
    t, m = torch(), q8()
    lens = workloads.seq_lens(w)
    dc = DeviceCache(lens, w.nkv, w.kv_bs, seed=seed, garbage=False, mirror=mirror)
    seqs = np.concatenate([np.full(n, b, np.int32) for b, n in enumerate(lens)])
    poss = np.concatenate([np.arange(n, dtype=np.int32) for n in lens])
    gen = t.Generator(device="cuda")
    gen.manual_seed(seed)
    for c0 in range(0, seqs.size, CHUNK):
        c1 = min(seqs.size, c0 + CHUNK)
        k = workloads.kv_pool_torch(w, c1 - c0, gen, "cuda")
        v = workloads.kv_pool_torch(w, c1 - c0, gen, "cuda")
        m.kv_append(dc.layer, dc.batch, t.from_numpy(seqs[c0:c1]).cuda(), t.from_numpy(poss[c0:c1]).cuda(), k, v,
                    dev_status=dc.status)
    q = t.randn((w.batch, w.nq, 128), generator=gen, device="cuda")
    assert dc.status_word() == 0
    return dc, lens, q


def _sample_seqs(lens, k, seed):
    order = np.argsort(lens)
    pick = {int(order[0]), int(order[-1])}
    rng = np.random.default_rng(seed)
    while len(pick) < min(k, lens.size):
        pick.add(int(rng.integers(0, lens.size)))
    return sorted(pick)


@pytest.mark.parametrize("name,nseq", [("qwen2b_b64_ragged", 6), ("qwen8b_b32_n32k", 3), ("qwen8b_b1_n128k", 1),
                                       ("qwen8b_b128_stress", 10)])
def test_decode_full_size_sampled(name, nseq):
    w = workloads.WORKLOADS[name]
    say(f"[full size] {name}: batch {w.batch}, {w.nq}/{w.nkv} heads, {w.lens}")
    dc, lens, q = _filled(w, seed=900 + len(name))
    out = dc.decode(q, w.nq, SCALE, nparts=0).cpu().numpy()   # automatic partitions, as bench.py
    assert dc.status_word() == 0
    seqs = _sample_seqs(lens, nseq, 901)
    if name == "qwen8b_b128_stress":
        # also the forced short lengths
        seqs = sorted(set(seqs) | {int(b) for b in np.nonzero(lens <= 65)[0][:8]})
    rows = np.array([b * w.nq + h for b in seqs for h in range(w.nq)], np.int64)
    want = oracle.decode_attn_rows(dc.host(), q.cpu().numpy(), w.nq, SCALE, rows)
    worst = assert_rows_close(out.reshape(-1, 128)[rows], want, name)
    say(f"  {rows.size} rows of sequences {seqs} (lengths {lens[seqs].tolist()}), worst err/tol {worst:.3f}")


@pytest.mark.parametrize("name,nseq", [("qwen2b_b64_ragged", 6), ("qwen8b_b128_stress", 10)])
def test_decode_step_full_size_sampled(name, nseq):
    # the call bench.py times: q8_decode_step (the newest token of every
    # sequence appended inside the decode kernel), automatic partitions
    w = workloads.WORKLOADS[name]
    say(f"[full size] decode step {name}: batch {w.batch}, {w.nq}/{w.nkv} heads, {w.lens}")
    t, m = torch(), q8()
    lens = workloads.seq_lens(w)
    dc = DeviceCache(lens, w.nkv, w.kv_bs, seed=930, garbage=False)
    hist = np.maximum(lens - 1, 0)
    seqs = np.concatenate([np.full(n, b, np.int32) for b, n in enumerate(hist)])
    poss = np.concatenate([np.arange(n, dtype=np.int32) for n in hist])
    gen = t.Generator(device="cuda")
    gen.manual_seed(931)
    for c0 in range(0, seqs.size, CHUNK):
        c1 = min(seqs.size, c0 + CHUNK)
        k = workloads.kv_pool_torch(w, c1 - c0, gen, "cuda")
        v = workloads.kv_pool_torch(w, c1 - c0, gen, "cuda")
        m.kv_append(dc.layer, dc.batch, t.from_numpy(seqs[c0:c1]).cuda(), t.from_numpy(poss[c0:c1]).cuda(), k, v,
                    dev_status=dc.status)
    k_new = workloads.kv_pool_torch(w, w.batch, gen, "cuda").reshape(w.batch, w.nkv, 128).contiguous()
    v_new = workloads.kv_pool_torch(w, w.batch, gen, "cuda").reshape(w.batch, w.nkv, 128).contiguous()
    q = t.randn((w.batch, w.nq, 128), generator=gen, device="cuda")
    out = t.full((w.batch, w.nq, 128), float("nan"), dtype=t.float32, device="cuda")
    ws = t.empty(m.decode_attn_workspace_bytes(dc.layer, dc.batch, w.nq, 0), dtype=t.uint8, device="cuda")
    m.decode_step(dc.layer, dc.batch, w.nq, k_new, v_new, q, SCALE, out, ws, nparts=0, dev_status=dc.status)
    assert dc.status_word() == 0
    host = dc.host()
    # every appended row: codes and steps bit-exact
    live = np.nonzero(lens > 0)[0]
    pos = lens[live] - 1
    slots = dc.table[live, pos // w.kv_bs] * w.kv_bs + pos % w.kv_bs
    ck, dk = oracle.quantize_kv(k_new.cpu().numpy()[live])
    cv, dv = oracle.quantize_kv(v_new.cpu().numpy()[live])
    np.testing.assert_array_equal(host.k_codes.reshape(-1, w.nkv, 128)[slots], ck)
    np.testing.assert_array_equal(host.v_codes.reshape(-1, w.nkv, 128)[slots], cv)
    np.testing.assert_array_equal(host.k_step.reshape(-1, w.nkv)[slots].view(np.uint32), dk.view(np.uint32))
    np.testing.assert_array_equal(host.v_step.reshape(-1, w.nkv)[slots].view(np.uint32), dv.view(np.uint32))
    # sampled output rows within tolerance of the oracle over the whole cache
    seqs_s = _sample_seqs(lens, nseq, 932)
    if name == "qwen8b_b128_stress":
        seqs_s = sorted(set(seqs_s) | {int(b) for b in np.nonzero(lens <= 65)[0][:8]})
    rows = np.array([b * w.nq + h for b in seqs_s for h in range(w.nq)], np.int64)
    want = oracle.decode_attn_rows(host, q.cpu().numpy(), w.nq, SCALE, rows)
    worst = assert_rows_close(out.cpu().numpy().reshape(-1, 128)[rows], want, name)
    say(f"  {live.size} appended rows exact; {rows.size} rows of sequences {seqs_s}, worst err/tol {worst:.3f}")


def test_sparse_full_size_ragged():
    # every (sequence, query head) of the ragged 2B batch: kept blocks exact,
    # outputs within tolerance
    w = workloads.WORKLOADS["qwen2b_b64_ragged"]
    say("[full size] block-sparse decode, qwen2b_b64_ragged, k = 32")
    t, m = torch(), q8()
    dc, lens, q = _filled(w, seed=910)
    out = t.empty((w.batch, w.nq, 128), dtype=t.float32, device="cuda")
    sel = t.empty((w.batch, w.nq, 32), dtype=t.int32, device="cuda")
    ws = t.empty(m.decode_attn_sparse_workspace_bytes(dc.layer, dc.batch, w.nq, 32), dtype=t.uint8, device="cuda")
    m.decode_attn_sparse(dc.layer, dc.batch, w.nq, q, SCALE, out, ws, topk=32, selected=sel, dev_status=dc.status)
    assert dc.status_word() == 0
    want, want_sel = oracle.decode_attn_sparse(dc.host(), q.cpu().numpy(), w.nq, SCALE, 32)
    np.testing.assert_array_equal(sel.cpu().numpy(), want_sel)
    worst = assert_rows_close(out.cpu().numpy(), want, "sparse full size")
    say(f"  {w.batch * w.nq} rows, worst err/tol {worst:.3f}")


def test_f32_mirror_full_size_ragged():
    w = workloads.WORKLOADS["qwen2b_b64_ragged"]
    say("[full size] exact fp32 decode over the mirror, qwen2b_b64_ragged")
    dc, lens, q = _filled(w, seed=920, mirror=True)
    out = dc.decode_f32(q, w.nq, SCALE, nparts=0).cpu().numpy()
    assert dc.status_word() == 0
    seqs = _sample_seqs(lens, 6, 921)
    rows = np.array([b * w.nq + h for b in seqs for h in range(w.nq)], np.int64)
    want = oracle.decode_attn_f32(dc.host_mirror(), q.cpu().numpy(), w.nq, SCALE, rows_bh=rows)
    worst = assert_rows_close(out.reshape(-1, 128)[rows], want, "f32 full size")
    say(f"  {rows.size} rows, worst err/tol {worst:.3f}")


def test_decode_wide_cut_long_sequence():
    """One 1M-token sequence (32768 tiles, one KV head) cut into 65536
    ranges: nparts * tiles = 2^31, so the range bounds take the 64-bit
    division in the partial and the merge kernels, and half of the ranges are
    empty.  The automatic cut (32-bit division) is checked beside it."""
    t, m = torch(), q8()
    n = 1 << 20
    lens = np.array([n], np.int32)
    say(f"[wide cut] one sequence of {n} tokens, 1/1 heads, kv_bs 32")
    dc = DeviceCache(lens, 1, 32, seed=951, garbage=False)
    gen = t.Generator(device="cuda")
    gen.manual_seed(951)
    seqs = t.zeros(CHUNK, dtype=t.int32, device="cuda")
    for c0 in range(0, n, CHUNK):
        pos = t.arange(c0, c0 + CHUNK, dtype=t.int32, device="cuda")
        k = t.randn((CHUNK, 1, 128), generator=gen, device="cuda")
        v = t.randn((CHUNK, 1, 128), generator=gen, device="cuda")
        m.kv_append(dc.layer, dc.batch, seqs, pos, k, v, dev_status=dc.status)
    q = t.randn((1, 1, 128), generator=gen, device="cuda")
    assert dc.status_word() == 0
    want = oracle.decode_attn_rows(dc.host(), q.cpu().numpy(), 1, SCALE, np.array([0], np.int64))
    for nparts in (65536, 0):
        out = dc.decode(q, 1, SCALE, nparts=nparts).cpu().numpy()
        assert dc.status_word() == 0
        worst = assert_rows_close(out.reshape(-1, 128), want, f"1M tokens, nparts {nparts}")
        say(f"  nparts {nparts}: worst err/tol {worst:.3f}")
