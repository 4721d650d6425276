"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Integer and byte results (codes, scales, Q codes, int32
block sums) must be bit-identical; fp32 outputs must satisfy, per (b, h) row,
max |gpu - oracle| <= 2e-5 * max |oracle| + 1e-6.

Sizes here run the oracle in seconds while spanning several tiles, partial
blocks and ragged tails; the full-size workloads are in test_gpu_fullsize.py.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import (DeviceCache, assert_rows_close, dense_kv, expected_codes, q8, say, torch)

pytestmark = pytest.mark.gpu
SCALE = float(workloads.softmax_scale(128))
EDGE_LENS = [0, 1, 2, 7, 8, 9, 31, 32, 33, 63, 64, 65, 100, 255, 256, 257, 700]


# ------------------------------------------------------------- append (a1)
@pytest.mark.parametrize("kv_bs", [8, 16, 32, 64])
@pytest.mark.parametrize("dist", ["normal", "student3x3"])
def test_append_codes_and_scales_bit_exact(kv_bs, dist):
    say(f"[append] kv_bs={kv_bs} dist={dist}")
    lens = np.array([1, 33, 200, 64, 0, 95], np.int32)
    k, v = dense_kv(lens, 8, seed=kv_bs, dist=dist)
    if dist == "normal":
        # hand rows: exact ties (max-abs 127 -> r = 1), zero row, both sides of the guard
        k[1, 0, 0, :] = 0.25
        k[1, 0, 0, :6] = [127.0, -127.0, 2.5, -2.5, 0.5, -0.5]
        k[1, 1, 3, :] = 0.0
        k[1, 2, 5, :] = np.float32(1e-6) * 0.5
        k[1, 2, 5, 7] = np.float32(1e-6)
        k[1, 3, 6, :] = np.nextafter(np.float32(1e-6), np.float32(0))
    dc = DeviceCache(lens, 8, kv_bs, seed=3)
    dc.append_dense(k, v)
    assert dc.status_word() == 0
    host = dc.host()
    slots, ck, cv, dk, dv = expected_codes(dc, k, v)
    got_k = host.k_codes.reshape(-1, 8, 128)[slots]
    got_v = host.v_codes.reshape(-1, 8, 128)[slots]
    np.testing.assert_array_equal(got_k, ck)
    np.testing.assert_array_equal(got_v, cv)
    np.testing.assert_array_equal(host.k_step.reshape(-1, 8)[slots].view(np.uint32), dk.view(np.uint32))
    np.testing.assert_array_equal(host.v_step.reshape(-1, 8)[slots].view(np.uint32), dv.view(np.uint32))


# rows = tokens x KV heads picks the heads per append wave: < 16384 rows one,
# then two, four, and eight from 65536 rows; 12 and 3 KV heads leave part of
# the last group of eight empty
@pytest.mark.parametrize("nkv,lens", [(8, [1000, 1048]), (8, [4096]), (12, [3000, 2999, 1]), (3, [24000])],
                         ids=["h2", "h4", "h8-nkv12", "h8-nkv3"])
def test_append_heads_per_wave_bit_exact(nkv, lens):
    say(f"[append] nkv={nkv} tokens={sum(lens)}")
    lens = np.array(lens, np.int32)
    k, v = dense_kv(lens, nkv, seed=int(lens.sum()) + nkv, dist="student3x3")
    dc = DeviceCache(lens, nkv, 32, seed=5)
    dc.append_dense(k, v)
    assert dc.status_word() == 0
    host = dc.host()
    slots, ck, cv, dk, dv = expected_codes(dc, k, v)
    np.testing.assert_array_equal(host.k_codes.reshape(-1, nkv, 128)[slots], ck)
    np.testing.assert_array_equal(host.v_codes.reshape(-1, nkv, 128)[slots], cv)
    np.testing.assert_array_equal(host.k_step.reshape(-1, nkv)[slots].view(np.uint32), dk.view(np.uint32))
    np.testing.assert_array_equal(host.v_step.reshape(-1, nkv)[slots].view(np.uint32), dv.view(np.uint32))


def test_append_one_token_per_step_matches_bulk():
    # decode-style appends (one token per sequence per call at seq_lens - 1)
    # leave exactly the bytes a bulk append leaves.
    t = torch()
    say("[append] stepwise vs bulk")
    lens = np.array([40, 17, 64], np.int32)
    k, v = dense_kv(lens, 2, seed=5)
    bulk = DeviceCache(lens, 2, 16, seed=9, garbage=False)
    bulk.layer.k_codes.zero_(); bulk.layer.v_codes.zero_(); bulk.layer.k_scale.zero_(); bulk.layer.v_scale.zero_()
    bulk.append_dense(k, v)
    step = DeviceCache(lens, 2, 16, seed=9, garbage=False)
    step.layer.k_codes.zero_(); step.layer.v_codes.zero_(); step.layer.k_scale.zero_(); step.layer.v_scale.zero_()
    m = q8()
    for pos in range(int(lens.max())):
        live = np.nonzero(lens > pos)[0].astype(np.int32)
        m.kv_append(step.layer, step.batch, t.from_numpy(live).cuda(),
                    t.from_numpy(np.full(live.size, pos, np.int32)).cuda(),
                    t.from_numpy(np.ascontiguousarray(k[live, pos])).cuda(),
                    t.from_numpy(np.ascontiguousarray(v[live, pos])).cuda(), dev_status=step.status)
    assert step.status_word() == 0
    for name in ("k_codes", "v_codes", "k_scale", "v_scale"):
        assert t.equal(getattr(step.layer, name), getattr(bulk.layer, name)), name


# ------------------------------------------------------- Q quantizer (a2)
@pytest.mark.parametrize("path,rows", [(0, 1000), (1, 1000), (1, 1001), (1, 1003)])
def test_quantize_q_bit_exact(path, rows):
    # both of the decode's device routines: two lanes per 32-block (path 0)
    # and one lane per 32-block in the matrix-core A layout (path 1, four
    # rows per wave; 1001 and 1003 rows end in a partial group)
    t = torch()
    say(f"[quantize_q] path {path}, {rows} rows")
    rng = np.random.default_rng(21)
    q = rng.standard_normal((rows, 128)).astype(np.float32)
    q[::5, 32:64] *= 1e-8                     # guarded blocks
    q[3] = 0.0
    q[7, :] = 0.25
    q[7, :12] = [127.0, -126.9, 2.5, -2.5, 0.99, -0.99, 126.99, -127.0, 64.7, -64.7, 0.0, 1.0]
    q[11] = (3 * rng.standard_t(3, 128)).astype(np.float32)
    q[13, :32] = np.float32(1e-6)             # both sides of the 1e-6 guard
    q[13, 32:64] = np.nextafter(np.float32(1e-6), np.float32(0))
    qd = t.from_numpy(q).cuda()
    codes = t.full((rows + 4, 128), 99, dtype=t.int8, device="cuda")
    qsc = t.full((rows + 4, 4), -1.0, dtype=t.float32, device="cuda")
    q8().quantize_q(qd, codes, qsc, path=path)
    want_c, want_s = oracle.quantize_q(q)
    np.testing.assert_array_equal(codes[:rows].cpu().numpy(), want_c)
    np.testing.assert_array_equal(qsc[:rows].cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    assert bool((codes[rows:] == 99).all()) and bool((qsc[rows:] == -1.0).all())   # nothing past the rows


# ------------------------------------------------------ int32 partials (a4)
@pytest.mark.parametrize("nq,nkv,kv_bs", [(1, 1, 32), (16, 8, 32), (32, 8, 8), (8, 1, 64),
                                          (32, 8, 32), (32, 8, 64), (32, 8, 256), (8, 2, 16), (8, 2, 32)])
def test_qk_block_partials_bit_exact(nq, nkv, kv_bs):
    # The decode's own routine for the shape: at four query heads per KV head
    # with kv_bs >= 32 the matrix-core path (one-lane-per-block query codes,
    # v_mfma_i32_16x16x64_i8), else sdot4; codes, scales and every partial
    # bit-exact, partials past a sequence's end 0.
    t = torch()
    say(f"[partials] nq={nq} nkv={nkv} kv_bs={kv_bs}")
    lens = np.array([70, 1, 0, 33, 128, 5, 300], np.int32)
    k, v = dense_kv(lens, nkv, seed=nq + kv_bs, dist="student3x3" if nq == 32 else "normal")
    rng = np.random.default_rng(nq + kv_bs)
    q = rng.standard_normal((len(lens), nq, 128)).astype(np.float32)
    q[1, 0, 32:64] = np.float32(1e-6)
    q[1, 0, 64:96] = 0.0
    dc = DeviceCache(lens, nkv, kv_bs, seed=4)
    dc.append_dense(k, v)
    out = t.full((len(lens), nq, dc.max_seq_len, 4), -7, dtype=t.int32, device="cuda")
    qc = t.full((len(lens), nq, 128), 99, dtype=t.int8, device="cuda")
    qs = t.full((len(lens), nq, 4), -1.0, dtype=t.float32, device="cuda")
    q8().qk_block_partials(dc.layer, dc.batch, nq, t.from_numpy(q).cuda(), out, qcodes=qc, qscale=qs,
                           dev_status=dc.status)
    assert dc.status_word() == 0
    ref_cache = oracle.build_cache(k, v, lens, dc.table, dc.num_blocks, kv_bs)
    want = oracle.qk_partials(ref_cache, q, nq, dc.max_seq_len)
    np.testing.assert_array_equal(out.cpu().numpy(), want)
    want_c, want_s = oracle.quantize_q(q)
    np.testing.assert_array_equal(qc.cpu().numpy(), want_c)
    np.testing.assert_array_equal(qs.cpu().numpy().view(np.uint32), want_s.view(np.uint32))


# ----------------------------------------------------------- decode (a3-a9)
def _decode_case(lens, nq, nkv, kv_bs, seed, nparts_list, dist="normal"):
    lens = np.asarray(lens, np.int32)
    k, v = dense_kv(lens, nkv, seed=seed, dist=dist)
    rng = np.random.default_rng([seed, 5])
    q = rng.standard_normal((len(lens), nq, 128)).astype(np.float32)
    dc = DeviceCache(lens, nkv, kv_bs, seed=seed)
    dc.append_dense(k, v)
    ref_cache = oracle.build_cache(k, v, lens, dc.table, dc.num_blocks, kv_bs)
    want = oracle.decode_attn(ref_cache, q, nq, SCALE)
    worst = 0.0
    for nparts in nparts_list:
        got = dc.decode(q, nq, SCALE, nparts=nparts).cpu().numpy()
        assert dc.status_word() == 0
        worst = max(worst, assert_rows_close(got, want, f"nparts={nparts}"))
        for b in np.nonzero(lens == 0)[0]:
            assert np.all(got[b] == 0)
    return worst


def test_single_head_256():
    # one sequence, one head, L = 256, N(0, 1), kv_bs 32 (the pages' 9-3 setting)
    say("[decode] single head 256")
    w = _decode_case([256], 1, 1, 32, seed=1001, nparts_list=[0, 1, 3, 8])
    say(f"  worst err/tol {w:.3f}")


@pytest.mark.parametrize("n", [506, 2046, 4059])
def test_qwen2b_batch1(n):
    say(f"[decode] 2B shape batch 1 n={n}")
    w = _decode_case([n], 16, 8, 32, seed=1002 + n, nparts_list=[0, 1, 5])
    say(f"  worst err/tol {w:.3f}")


@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("kv_bs", [8, 16, 32, 64, 256])
def test_ragged_edges(group, kv_bs):
    say(f"[decode] ragged edges group={group} kv_bs={kv_bs}")
    nkv = 2
    w = _decode_case(EDGE_LENS, nkv * group, nkv, kv_bs, seed=group * 100 + kv_bs,
                     nparts_list=[0, 1, 2, 7, 50, 1000])
    say(f"  worst err/tol {w:.3f}")


# more than 64 sequences, with empty ones at the edges of the 64-entry steps
# of the range lookups (and at both ends of the batch)
WIDE_LENS = [0 if b in (0, 62, 63, 64, 65, 127, 128, 130) else int(x)
             for b, x in enumerate(np.random.default_rng(77).integers(1, 300, 131))]


@pytest.mark.parametrize("kv_bs", [8, 32])
def test_wide_batch_with_empty_sequences(kv_bs):
    say(f"[decode] 131 sequences, 8 empty, kv_bs={kv_bs}")
    w = _decode_case(WIDE_LENS, 4, 2, kv_bs, seed=77 + kv_bs, nparts_list=[0, 1, 3, 64, 65, 300, 5000])
    say(f"  worst err/tol {w:.3f}")


def test_heavy_tails_and_guard_rows():
    say("[decode] student-t x3 with near-zero rows")
    lens = np.array([1, 2, 31, 32, 33, 63, 64, 65, 500, 1500, 3000], np.int32)
    w = _decode_case(lens, 32, 8, 32, seed=1006, nparts_list=[0, 9], dist="student3x3")
    say(f"  worst err/tol {w:.3f}")


@pytest.mark.parametrize("nq,nkv", [(24, 12), (20, 10), (40, 10)])
def test_many_kv_heads(nq, nkv):
    # more KV heads than one workgroup takes: at G = 2 workgroups of 4 waves
    # (12 heads: three per range; 10 heads: three, two waves of the last one
    # idle), at G = 4 of up to 8 (10 heads: two workgroups of 5 waves)
    say(f"[decode] nq={nq} nkv={nkv}")
    w = _decode_case([300, 45, 1], nq, nkv, 32, seed=nq + nkv, nparts_list=[0, 4])
    say(f"  worst err/tol {w:.3f}")


def test_seq_len_one_is_dequantized_v_bitwise():
    # w = 1, S = 1: the output is float(code) * step, bit for bit.
    say("[decode] seq_len 1")
    lens = np.ones(5, np.int32)
    k, v = dense_kv(lens, 4, seed=31)
    q = np.random.default_rng(31).standard_normal((5, 16, 128)).astype(np.float32)
    dc = DeviceCache(lens, 4, 32, seed=31)
    dc.append_dense(k, v)
    got = dc.decode(q, 16, SCALE).cpu().numpy()
    for b in range(5):
        for h in range(16):
            cv, dv = oracle.quantize_kv(v[b, 0, h // 4])
            want = (cv.astype(np.float32) * dv).astype(np.float32)
            np.testing.assert_array_equal(got[b, h].view(np.uint32), want.view(np.uint32))


def test_placement_invariance_and_reproducibility():
    # Where blocks sit in the pool does not change a single bit; the same call
    # twice gives the same bits; another partition count stays within tolerance.
    t = torch()
    say("[decode] placement / reproducibility")
    lens = np.array([900, 33, 257, 1, 640], np.int32)
    k, v = dense_kv(lens, 8, seed=41)
    q = np.random.default_rng(41).standard_normal((5, 32, 128)).astype(np.float32)
    outs = []
    for seed in (1, 2):
        dc = DeviceCache(lens, 8, 32, seed=seed, spare=11)
        dc.append_dense(k, v)
        outs.append(dc.decode(q, 32, SCALE, nparts=6).cpu().numpy())
        again = dc.decode(q, 32, SCALE, nparts=6).cpu().numpy()
        np.testing.assert_array_equal(again.view(np.uint32), outs[-1].view(np.uint32))
    np.testing.assert_array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    other = dc.decode(q, 32, SCALE, nparts=1).cpu().numpy()
    assert_rows_close(other, outs[0], "nparts 1 vs 6")


def test_batch_composition_changes_bits_only_within_tolerance():
    # The cut runs over the whole batch, so other sequences move the places
    # where a long sequence is cut: its output may change in the last bits,
    # never beyond the tolerance.  Sub-batch and super-batch against the batch.
    say("[decode] batch composition")
    lens = np.array([3000, 40, 1700, 1, 640, 2100], np.int32)
    k, v = dense_kv(lens, 8, seed=43)
    q = np.random.default_rng(43).standard_normal((lens.size, 16, 128)).astype(np.float32)

    def run(idx):
        dc = DeviceCache(lens[idx], 8, 32, seed=7)
        dc.append_dense(k[idx], v[idx])
        out = dc.decode(q[idx], 16, SCALE, nparts=12).cpu().numpy()
        assert dc.status_word() == 0
        return out

    full = run(np.arange(lens.size))
    for idx in (np.array([0, 2, 5]), np.array([2]), np.array([5, 4, 3, 2, 1, 0])):
        part = run(idx)
        assert_rows_close(part, full[idx], f"sequences {idx.tolist()}")


def test_zero_query_gives_mean_of_values():
    say("[decode] q = 0")
    lens = np.array([77, 300], np.int32)
    k, v = dense_kv(lens, 2, seed=51)
    dc = DeviceCache(lens, 2, 32, seed=51)
    dc.append_dense(k, v)
    got = dc.decode(np.zeros((2, 4, 128), np.float32), 4, SCALE).cpu().numpy()
    for b, n in enumerate(lens):
        for h in range(4):
            cv, dv = oracle.quantize_kv(v[b, :n, h // 2])
            want = oracle.dequantize(cv, dv).mean(0)
            assert_rows_close(got[b, h], want, "mean")


# ------------------------------------------------------- device-side errors
def test_device_detected_errors_are_reported():
    t = torch()
    say("[status] bad block id / bad length / bad token")
    lens = np.array([64, 40], np.int32)
    k, v = dense_kv(lens, 2, seed=61)
    q = np.random.default_rng(61).standard_normal((2, 4, 128)).astype(np.float32)
    dc = DeviceCache(lens, 2, 32, seed=61)
    dc.append_dense(k, v)
    assert dc.status_word() == 0
    # an out-of-range block id in sequence 1: reported, the block is skipped
    dc.table_t[1, 1] = dc.num_blocks + 5
    out = dc.decode(q, 4, SCALE).cpu().numpy()
    assert dc.status_word() & q8().DEV_BAD_BLOCK_ID
    assert np.all(np.isfinite(out))
    # a length beyond max_seq_len: reported, the row reads as empty
    dc.table_t[1, 1] = int(dc.table[1, 1])
    dc.status.zero_()
    dc.lens_t[0] = dc.max_seq_len + 1
    out = dc.decode(q, 4, SCALE).cpu().numpy()
    assert dc.status_word() & q8().DEV_BAD_SEQ_LEN
    assert np.all(out[0] == 0)
    # an append at a position outside its sequence: reported, nothing written
    dc.lens_t[0] = 64
    dc.status.zero_()
    before = dc.layer.k_codes.clone()
    q8().kv_append(dc.layer, dc.batch, t.tensor([1], dtype=t.int32, device="cuda"),
                   t.tensor([40], dtype=t.int32, device="cuda"),
                   t.zeros((1, 2, 128), device="cuda"), t.zeros((1, 2, 128), device="cuda"),
                   dev_status=dc.status)
    assert dc.status_word() & q8().DEV_BAD_TOKEN
    assert t.equal(before, dc.layer.k_codes)


def test_phase_entry_points_equal_one_call():
    t = torch()
    say("[decode] partial + merge == decode")
    lens = np.array([1000, 70, 3], np.int32)
    k, v = dense_kv(lens, 8, seed=71)
    q = t.from_numpy(np.random.default_rng(71).standard_normal((3, 16, 128)).astype(np.float32)).cuda()
    dc = DeviceCache(lens, 8, 32, seed=71)
    dc.append_dense(k, v)
    one = dc.decode(q, 16, SCALE, nparts=9)
    m = q8()
    ws = t.empty(m.decode_attn_workspace_bytes(dc.layer, dc.batch, 16, 9), dtype=t.uint8, device="cuda")
    out = t.empty_like(one)
    m.decode_attn_partial(dc.layer, dc.batch, 16, q, SCALE, out, ws, nparts=9)
    m.decode_attn_merge(dc.layer, dc.batch, 16, q, SCALE, out, ws, nparts=9)
    assert t.equal(out, one)


def test_graph_replays_match_eager():
    # The append + decode sequence captured in one HIP graph and replayed
    # several times, with eager work and synchronizations in between, gives
    # the eager bits every time (no memset nodes are involved).
    t = torch()
    say("[graph] capture / replay")
    lens = np.array([700, 65, 1, 300], np.int32)
    k, v = dense_kv(lens, 8, seed=81)
    dc = DeviceCache(lens, 8, 32, seed=81)
    dc.append_dense(k, v)
    m = q8()
    rng = np.random.default_rng(81)
    q = t.from_numpy(rng.standard_normal((4, 16, 128)).astype(np.float32)).cuda()
    kn = t.from_numpy(rng.standard_normal((4, 8, 128)).astype(np.float32)).cuda()
    vn = t.from_numpy(rng.standard_normal((4, 8, 128)).astype(np.float32)).cuda()
    seqs = t.arange(4, dtype=t.int32, device="cuda")
    pos = (dc.lens_t - 1).to(t.int32)
    ws = t.empty(m.decode_attn_workspace_bytes(dc.layer, dc.batch, 16, 0), dtype=t.uint8, device="cuda")
    out = t.empty((4, 16, 128), dtype=t.float32, device="cuda")

    def body():
        m.kv_append(dc.layer, dc.batch, seqs, pos, kn, vn, dev_status=dc.status)
        m.decode_attn(dc.layer, dc.batch, 16, q, SCALE, out, ws, dev_status=dc.status)

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
        ws.fill_(0xAB)                      # eager work touching the workspace in between
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        assert t.equal(out, eager), f"replay {i}"
    assert dc.status_word() == 0
