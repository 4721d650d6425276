"""Helpers for the GPU tests: put seeded inputs through the library's C ABI
and read results back.  Inputs come from ``workloads``; expected values come
only from ``oracle``."""
from __future__ import annotations

import numpy as np

import oracle
import workloads

TOL_REL = 2e-5
TOL_ABS = 1e-6


def torch():
    import torch as t
    return t


def q8():
    import decode_attention_int8_kv_amd as m
    m.lib()
    return m


def say(*a):
    print(*a, flush=True)


class DeviceCache:
    """One layer on the GPU plus its batch metadata."""

    def __init__(self, lens, nkv, kv_bs, seed, spare=2, device="cuda", garbage=True, mirror=False):
        t = torch()
        m = q8()
        self.lens = np.asarray(lens, np.int32)
        self.nkv, self.kv_bs = nkv, kv_bs
        self.table, self.num_blocks = workloads.block_table(self.lens, kv_bs, seed, spare_blocks=spare)
        self.layer = m.alloc_layer(self.num_blocks, kv_bs, nkv, device, mirror=mirror)
        if garbage:
            # rows no token occupies hold junk codes and NaN scales: masking must ignore them
            g = t.Generator(device=device)
            g.manual_seed(seed)
            self.layer.k_codes.copy_(t.randint(-128, 128, self.layer.k_codes.shape, generator=g, device=device,
                                               dtype=t.int8))
            self.layer.v_codes.copy_(t.randint(-128, 128, self.layer.v_codes.shape, generator=g, device=device,
                                               dtype=t.int8))
            self.layer.k_scale.fill_(float("nan"))
            self.layer.v_scale.fill_(float("nan"))
            if mirror:
                self.layer.k_f32.fill_(float("nan"))
                self.layer.v_f32.fill_(float("nan"))
        self.table_t = t.from_numpy(self.table).to(device)
        self.lens_t = t.from_numpy(self.lens).to(device)
        self.max_seq_len = int(max(1, self.lens.max()))
        self.batch = m.make_batch(self.table_t, self.lens_t, self.max_seq_len)
        self.status = t.zeros(1, dtype=t.int32, device=device)

    def append_dense(self, k, v, t0=0):
        """Append tokens [t0, len_b) of every sequence from dense fp32 host
        arrays k, v [batch, >= len, nkv, hd] through q8_kv_append."""
        t = torch()
        seqs, poss, ks, vs = [], [], [], []
        for b, n in enumerate(self.lens):
            if n <= t0:
                continue
            seqs.append(np.full(n - t0, b, np.int32))
            poss.append(np.arange(t0, n, dtype=np.int32))
            ks.append(k[b, t0:n])
            vs.append(v[b, t0:n])
        if not seqs:
            return
        dev = self.layer.k_codes.device
        q8().kv_append(self.layer, self.batch,
                       t.from_numpy(np.concatenate(seqs)).to(dev), t.from_numpy(np.concatenate(poss)).to(dev),
                       t.from_numpy(np.ascontiguousarray(np.concatenate(ks), np.float32)).to(dev),
                       t.from_numpy(np.ascontiguousarray(np.concatenate(vs), np.float32)).to(dev),
                       dev_status=self.status)

    def host(self):
        """The cache as an oracle.Cache (codes and steps copied back)."""
        L = self.layer
        # the library stores scales [block][kv head][row]; the oracle takes [block][row][kv head]
        ks = np.ascontiguousarray(L.k_scale.cpu().numpy().transpose(0, 2, 1))
        vs = np.ascontiguousarray(L.v_scale.cpu().numpy().transpose(0, 2, 1))
        return oracle.Cache(L.k_codes.cpu().numpy(), L.v_codes.cpu().numpy(), ks, vs,
                            self.table, self.lens, self.nkv, 128)

    def host_mirror(self):
        """The fp32 mirror as an oracle.MirrorCache (copied back)."""
        L = self.layer
        return oracle.MirrorCache(L.k_f32.cpu().numpy(), L.v_f32.cpu().numpy(), self.table, self.lens,
                                  self.nkv, 128)

    def decode_f32(self, q, nq, scale, nparts=0, out=None):
        t = torch()
        m = q8()
        dev = self.layer.k_codes.device
        qd = q if isinstance(q, t.Tensor) else t.from_numpy(np.ascontiguousarray(q, np.float32)).to(dev)
        if out is None:
            out = t.full((self.batch.batch, nq, 128), float("nan"), dtype=t.float32, device=dev)
        nbytes = m.decode_attn_workspace_bytes(self.layer, self.batch, nq, nparts)
        ws = t.empty(nbytes, dtype=t.uint8, device=dev)
        m.decode_attn_f32(self.layer, self.batch, nq, qd, scale, out, ws, nparts=nparts, dev_status=self.status)
        return out

    def decode(self, q, nq, scale, nparts=0, out=None):
        t = torch()
        m = q8()
        dev = self.layer.k_codes.device
        qd = q if isinstance(q, t.Tensor) else t.from_numpy(np.ascontiguousarray(q, np.float32)).to(dev)
        if out is None:
            out = t.full((self.batch.batch, nq, 128), float("nan"), dtype=t.float32, device=dev)
        nbytes = m.decode_attn_workspace_bytes(self.layer, self.batch, nq, nparts)
        ws = t.empty(nbytes, dtype=t.uint8, device=dev)
        m.decode_attn(self.layer, self.batch, nq, qd, scale, out, ws, nparts=nparts, dev_status=self.status)
        return out

    def status_word(self):
        torch().cuda.synchronize()
        return int(self.status.item())


def dense_kv(lens, nkv, seed, dist="normal", hd=128):
    rng = np.random.default_rng([seed, 77])
    max_len = int(max(1, np.max(lens)))
    shape = (len(lens), max_len, nkv, hd)
    if dist == "normal":
        return (rng.standard_normal(shape, dtype=np.float32), rng.standard_normal(shape, dtype=np.float32))
    w = workloads.Workload("t", nkv, nkv, len(lens), 1, ("fixed", max_len), "student3x3", seed)
    k, v = workloads.kv_host(w, np.asarray(lens, np.int32))
    return k, v


def expected_codes(dc: DeviceCache, k, v):
    """Oracle codes/steps of every appended token, gathered at its cache slot."""
    rows_k, rows_v, steps_k, steps_v, slots = [], [], [], [], []
    for b, n in enumerate(dc.lens):
        if n == 0:
            continue
        ck, dk = oracle.quantize_kv(k[b, :n])
        cv, dv = oracle.quantize_kv(v[b, :n])
        t = np.arange(n)
        slots.append(dc.table[b, t // dc.kv_bs] * dc.kv_bs + t % dc.kv_bs)
        rows_k.append(ck), rows_v.append(cv), steps_k.append(dk), steps_v.append(dv)
    return (np.concatenate(slots), np.concatenate(rows_k), np.concatenate(rows_v),
            np.concatenate(steps_k), np.concatenate(steps_v))


def row_errors(got, want):
    """Per (b, h) row: max |got - want| and the allowed tolerance."""
    got = np.asarray(got, np.float64).reshape(-1, 128)
    want = np.asarray(want, np.float64).reshape(-1, 128)
    err = np.abs(got - want).max(1)
    tol = TOL_REL * np.abs(want).max(1) + TOL_ABS
    return err, tol


def assert_rows_close(got, want, what=""):
    err, tol = row_errors(got, want)
    bad = np.nonzero(~(err <= tol))[0]
    assert bad.size == 0, (f"{what}: {bad.size} rows out of tolerance; worst row {bad[np.argmax(err[bad] / tol[bad])]} "
                           f"err {err[bad].max():.3e} tol {tol[bad].min():.3e}")
    return float((err / tol).max()) if err.size else 0.0


# ------------------------------------------------------- block-sparse decisions
# The GPU evaluates each probe row's score s = (sum_b P_b * qscale_b) *
# kscale * scale in fp32, scaled by the positive constant fl(scale * log2 e) /
# scale common to every block (the block ranking is unchanged by it): the
# four block terms x_b = fl(P_b * qscale_b) (P_b exact), two pairwise sums and
# their sum, then one product with fl(kscale * sc).  Each block term passes
# through at most three roundings on its way into the sum and the result
# through two more, so |gpu / const - s| <= ~5 u * sum_b |x_b| * kscale *
# scale with u = 2^-24; a block's importance (a max over probe rows) moves
# by at most the largest such bound over its rows.  SPARSE_EPS_U = 8 gives
# margin over 5.
SPARSE_EPS_U = 8 * 2.0 ** -24


def check_sparse_selection(sel, scores, mags, lens, topk):
    """The GPU's kept blocks sel [batch, nq, topk] (ascending, -1 after the
    last) against the oracle's exact importances (scores, mags from
    oracle.sparse_scores): for every (b, h) with more than topk blocks,
    exactly topk distinct blocks of the sequence are kept, every kept block's
    importance plus its bound is at least every dropped block's importance
    minus its bound, and no dropped block ties exactly with a kept block of
    higher index; otherwise every block is kept.  Returns the number of rows
    whose kept set differs from the exact top-k (decisions inside the fp32
    rounding band)."""
    sel = np.asarray(sel)
    batch, nq, _ = sel.shape
    inside_band = 0
    for b in range(batch):
        n = int(lens[b])
        nb = (n + 31) // 32
        for h in range(nq):
            row = [int(x) for x in sel[b, h]]
            k = sum(1 for x in row if x >= 0)
            assert all(x >= 0 for x in row[:k]) and all(x == -1 for x in row[k:]), (b, h, row)
            kept = row[:k]
            if nb <= topk:
                assert kept == list(range(nb)), (b, h, kept)
                continue
            assert k == topk and kept == sorted(set(kept)) and 0 <= kept[0] and kept[-1] < nb, (b, h, kept)
            d = scores[b, h, :nb]
            e = SPARSE_EPS_U * mags[b, h, :nb] + 1e-300
            mask = np.zeros(nb, bool)
            mask[kept] = True
            lo = np.min(d[mask] + e[mask])
            hi = np.max(d[~mask] - e[~mask])
            assert lo >= hi, f"(b {b}, h {h}): kept block scored {lo} below dropped {hi}"
            for i in np.nonzero(~mask)[0]:
                assert not np.any(mask[i + 1:] & (d[i + 1:] == d[i])), f"(b {b}, h {h}): tie not to block {i}"
            exact = sorted(sorted(range(nb), key=lambda j: (-d[j], j))[:topk])
            inside_band += kept != exact
    return inside_band


def run_sparse_and_check(dc, q, nq, scale, topk, what=""):
    """Block-sparse decode on the GPU cache dc (q: host [batch, nq, 128]
    fp32), checked against the oracle over the codes read back: the kept
    blocks by check_sparse_selection, the outputs within the decode
    tolerance of the oracle's attention over the GPU's kept blocks.  Returns
    (worst err/tol, rows decided inside the rounding band)."""
    t = torch()
    m = q8()
    batch = len(dc.lens)
    qd = q if isinstance(q, t.Tensor) else t.from_numpy(np.ascontiguousarray(q, np.float32)).cuda()
    qh = qd.cpu().numpy()
    out = t.full((batch, nq, 128), float("nan"), dtype=t.float32, device="cuda")
    sel = t.full((batch, nq, topk), -7, dtype=t.int32, device="cuda")
    ws = t.empty(m.decode_attn_sparse_workspace_bytes(dc.layer, dc.batch, nq, topk), dtype=t.uint8, device="cuda")
    ws.fill_(0xCD)
    m.decode_attn_sparse(dc.layer, dc.batch, nq, qd, scale, out, ws, topk=topk, selected=sel, dev_status=dc.status)
    assert dc.status_word() == 0
    host = dc.host()
    got_sel = sel.cpu().numpy()
    scores, mags = oracle.sparse_scores(host, qh, nq, scale)
    band = check_sparse_selection(got_sel, scores, mags, dc.lens, topk)
    want = oracle.decode_attn_blocks(host, qh, nq, scale, got_sel)
    worst = assert_rows_close(out.cpu().numpy(), want, f"sparse topk={topk} {what}")
    return worst, band
