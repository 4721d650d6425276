"""GPU parity at the full sizes of the batched workloads, in the launch
configuration bench.py times (q8_decode_step, automatic partition count).

Every history row is appended through q8_kv_append from K/V drawn on the GPU
with the workload's value distribution (the stress batch includes rows at
both sides of the 1e-6 guard); after every chunk, the codes and steps of
every appended row are checked bit for bit against the oracle's quantizer of
the same fp32 rows.  The decode step then appends each sequence's newest
token (also checked bit for bit) and attends; the oracle reads the whole
cache back and computes EVERY (sequence, query head) row, each within
max |gpu - oracle| <= 2e-5 * max |oracle| + 1e-6.  q8_decode_attn over the
same cache afterwards must give the step's output bit for bit.

Layers: the ragged 2B batch on two independently drawn layers (standing for
its first and last), the other workloads on one.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import DeviceCache, assert_rows_close, q8, run_sparse_and_check, say, torch

pytestmark = pytest.mark.gpu
SCALE = float(workloads.softmax_scale(128))
CHUNK = 1 << 16   # tokens appended per call


def _check_rows(dc, slots, k, v, what):
    """Codes and steps at cache rows `slots` (block * kv_bs + row) against the
    oracle's quantizer of the fp32 rows k, v [T, nkv, 128] (torch, GPU)."""
    t = torch()
    L = dc.layer
    st = t.from_numpy(slots).cuda()
    blk, row = st // dc.kv_bs, st % dc.kv_bs
    got_kc = L.k_codes.view(-1, dc.nkv, 128)[st].cpu().numpy()
    got_vc = L.v_codes.view(-1, dc.nkv, 128)[st].cpu().numpy()
    got_ks = L.k_scale[blk, :, row].cpu().numpy()
    got_vs = L.v_scale[blk, :, row].cpu().numpy()
    ck, dk = oracle.quantize_kv(k.cpu().numpy())
    cv, dv = oracle.quantize_kv(v.cpu().numpy())
    np.testing.assert_array_equal(got_kc, ck, err_msg=f"{what}: K codes")
    np.testing.assert_array_equal(got_vc, cv, err_msg=f"{what}: V codes")
    np.testing.assert_array_equal(got_ks.view(np.uint32), dk.view(np.uint32), err_msg=f"{what}: K steps")
    np.testing.assert_array_equal(got_vs.view(np.uint32), dv.view(np.uint32), err_msg=f"{what}: V steps")


def _guard_hits(k):
    m = k.abs().amax(-1)
    return int((m == np.float32(1e-6)).sum()), int((m == float(np.nextafter(np.float32(1e-6), np.float32(0)))).sum())


def _filled(w, seed, hist=None):
    """One layer of workload w on the GPU: positions [0, hist[b]) of every
    sequence appended (default: all but the last), every row bit-checked.
    Returns (cache, lens, generator, guard-row counts)."""
    t, m = torch(), q8()
    lens = workloads.seq_lens(w)
    hist = np.maximum(lens - 1, 0) if hist is None else hist
    dc = DeviceCache(lens, w.nkv, w.kv_bs, seed=seed, garbage=False)
    seqs = np.concatenate([np.full(n, b, np.int32) for b, n in enumerate(hist)])
    poss = np.concatenate([np.arange(n, dtype=np.int32) for n in hist])
    slots = dc.table[seqs, poss // w.kv_bs].astype(np.int64) * w.kv_bs + poss % w.kv_bs
    gen = t.Generator(device="cuda")
    gen.manual_seed(seed)
    hits = np.zeros(2, np.int64)
    for c0 in range(0, seqs.size, CHUNK):
        c1 = min(seqs.size, c0 + CHUNK)
        k = workloads.kv_pool_torch(w, c1 - c0, gen, "cuda")
        v = workloads.kv_pool_torch(w, c1 - c0, gen, "cuda")
        m.kv_append(dc.layer, dc.batch, t.from_numpy(seqs[c0:c1]).cuda(), t.from_numpy(poss[c0:c1]).cuda(), k, v,
                    dev_status=dc.status)
        t.cuda.synchronize()
        _check_rows(dc, slots[c0:c1], k, v, f"{w.name} history tokens {c0}..{c1}")
        hits += np.array(_guard_hits(k)) + np.array(_guard_hits(v))
    assert dc.status_word() == 0
    return dc, lens, gen, hits


def _step_and_check(w, dc, lens, gen, what):
    """q8_decode_step (automatic partitions) appending every sequence's newest
    token, then every appended row bit-checked and every output row against
    the oracle; q8_decode_attn afterwards gives the same bits."""
    t, m = torch(), q8()
    k_new = workloads.kv_pool_torch(w, w.batch, gen, "cuda").reshape(w.batch, w.nkv, 128).contiguous()
    v_new = workloads.kv_pool_torch(w, w.batch, gen, "cuda").reshape(w.batch, w.nkv, 128).contiguous()
    q = t.randn((w.batch, w.nq, 128), generator=gen, device="cuda")
    out = t.full((w.batch, w.nq, 128), float("nan"), dtype=t.float32, device="cuda")
    ws = t.empty(m.decode_attn_workspace_bytes(dc.layer, dc.batch, w.nq, 0), dtype=t.uint8, device="cuda")
    m.decode_step(dc.layer, dc.batch, w.nq, k_new, v_new, q, SCALE, out, ws, nparts=0, dev_status=dc.status)
    assert dc.status_word() == 0
    live = np.nonzero(lens > 0)[0]
    pos = lens[live] - 1
    slots = dc.table[live, pos // w.kv_bs].astype(np.int64) * w.kv_bs + pos % w.kv_bs
    _check_rows(dc, slots, k_new[live], v_new[live], f"{what}: appended tokens")
    again = dc.decode(q, w.nq, SCALE, nparts=0)
    assert dc.status_word() == 0
    assert t.equal(again, out), f"{what}: q8_decode_attn differs from q8_decode_step"
    say(f"  step done; oracle over all {w.batch * w.nq} rows ...")
    want = oracle.decode_attn(dc.host(), q.cpu().numpy(), w.nq, SCALE)
    worst = assert_rows_close(out.cpu().numpy(), want, what)
    zero = np.nonzero(lens == 0)[0]
    assert np.all(out.cpu().numpy()[zero] == 0)
    return worst


@pytest.mark.parametrize("name,layer_seeds", [("qwen2b_b64_ragged", (900, 927)), ("qwen8b_b32_n32k", (940,)),
                                              ("qwen8b_b1_n128k", (950,)), ("qwen8b_b128_stress", (960,))])
def test_decode_step_full_size_every_row(name, layer_seeds):
    w = workloads.WORKLOADS[name]
    for seed in layer_seeds:
        say(f"[full size] {name} (layer seed {seed}): batch {w.batch}, {w.nq}/{w.nkv} heads, {w.lens}")
        dc, lens, gen, hits = _filled(w, seed)
        say(f"  {int(np.maximum(lens - 1, 0).sum())} history tokens appended, codes and steps exact "
            f"(guard rows at 1e-6 / below: {hits.tolist()})")
        if w.dist != "normal":
            assert hits[0] > 0 and hits[1] > 0
        worst = _step_and_check(w, dc, lens, gen, f"{name} seed {seed}")
        say(f"  every row within tolerance, worst err/tol {worst:.3f}")
        del dc
        torch().cuda.empty_cache()


def test_sparse_full_size_ragged():
    # every (sequence, query head) of the ragged 2B batch: the kept blocks
    # valid against the oracle's exact importances, outputs within tolerance
    # of the oracle's attention over them
    w = workloads.WORKLOADS["qwen2b_b64_ragged"]
    say("[full size] block-sparse decode, qwen2b_b64_ragged, k = 32")
    t = torch()
    lens = workloads.seq_lens(w)
    dc, lens, gen, _ = _filled(w, seed=910, hist=lens)
    q = t.randn((w.batch, w.nq, 128), generator=gen, device="cuda")
    worst, band = run_sparse_and_check(dc, q, w.nq, SCALE, 32, "full size")
    say(f"  {w.batch * w.nq} rows, worst err/tol {worst:.3f}, rows decided inside the fp32 band: {band}")


def test_f32_mirror_full_size_ragged():
    w = workloads.WORKLOADS["qwen2b_b64_ragged"]
    say("[full size] exact fp32 decode over the mirror, qwen2b_b64_ragged, every row")
    t, m = torch(), q8()
    lens = workloads.seq_lens(w)
    dc = DeviceCache(lens, w.nkv, w.kv_bs, seed=920, garbage=False, mirror=True)
    seqs = np.concatenate([np.full(n, b, np.int32) for b, n in enumerate(lens)])
    poss = np.concatenate([np.arange(n, dtype=np.int32) for n in lens])
    gen = t.Generator(device="cuda")
    gen.manual_seed(920)
    for c0 in range(0, seqs.size, CHUNK):
        c1 = min(seqs.size, c0 + CHUNK)
        k = workloads.kv_pool_torch(w, c1 - c0, gen, "cuda")
        v = workloads.kv_pool_torch(w, c1 - c0, gen, "cuda")
        m.kv_append(dc.layer, dc.batch, t.from_numpy(seqs[c0:c1]).cuda(), t.from_numpy(poss[c0:c1]).cuda(), k, v,
                    dev_status=dc.status)
    q = t.randn((w.batch, w.nq, 128), generator=gen, device="cuda")
    out = dc.decode_f32(q, w.nq, SCALE, nparts=0).cpu().numpy()
    assert dc.status_word() == 0
    want = oracle.decode_attn_f32(dc.host_mirror(), q.cpu().numpy(), w.nq, SCALE)
    worst = assert_rows_close(out, want, "f32 full size")
    say(f"  {w.batch * w.nq} rows, worst err/tol {worst:.3f}")


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
