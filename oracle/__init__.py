"""CPU oracle for q8 single-query decode attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never links, loads or
calls it, and this package imports nothing from the library: the two share no
code.  The arithmetic lives in ``q8kv_oracle.c`` (plain C, built with gcc,
``-ffp-contract=off``, no fast-math); this module only marshals numpy arrays.

Pages the oracle follows (cited by title and section):
  * 9-2 "flash_attn_single_q_q8_neon -- 单 q 单遍扫全 KV": §2 segment 1 (Q
    quantizer), §2 segment 2 (blocked KV walk, per-32-block int partials,
    online softmax), §2 segment 3 (final division), §3 (single pass is
    functionally the same as storing every score first), §4 (observables).
  * 9-3 "q8 KV 精度对照实验": §1 (the reference attention), §2 (per-(token,
    head) K/V quantizer), §3 (printed fp32-KV vs q8-KV gap, and the fp32
    mirror cache of its closing note).
  * 10-1 "why long context must be sparse": §1-§2 (block-sparse decode; the
    batched prefill over the cache).

Every oracle function is pinned by a CPU test against facts fixed by the
pages or by mathematics (closed forms, invariants, brute force); none is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q8kv_oracle.c")
# Q8KV_ORACLE_LIB names another build of the same source (a sanitizer build,
# for instance); by default the library is built next to the source.
_LIB_PATH = os.environ.get("Q8KV_ORACLE_LIB") or os.path.join(_HERE, "liboracle_q8kv.so")
_lib = None

HEAD_BLOCK = 32  # Q block length (9-2 §2 segment 1)


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle_q8kv.so``."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, I64, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    lib.orc_quantize_kv_rows.argtypes = [P, I64, I, P, P]
    lib.orc_quantize_q_rows.argtypes = [P, I64, I, P, P]
    lib.orc_block_partials.argtypes = [P, P, I, P]
    lib.orc_block_partials.restype = I
    lib.orc_attend_dense.argtypes = [P, P, P, I64, I, ctypes.c_double, P]
    lib.orc_decode_attn.argtypes = [I, I, I, I, I, P, I, P, I, P, P, P, P, P, F, P, I]
    lib.orc_decode_attn.restype = I
    lib.orc_decode_attn_rows.argtypes = [I, I, I, I, P, I, P, I, P, P, P, P, P, F, P, I, P, I]
    lib.orc_decode_attn_rows.restype = I
    lib.orc_qk_partials.argtypes = [I, I, I, I, I, P, I, P, I, I, P, P, P]
    lib.orc_qk_partials.restype = I
    lib.orc_single_pass.argtypes = [P, P, P, P, P, P, I64, I, F, P, P]
    lib.orc_decode_attn_f32.argtypes = [I, I, I, I, I, P, I, P, I, P, P, P, F, P, I, P, I]
    lib.orc_decode_attn_f32.restype = I
    lib.orc_decode_attn_sparse.argtypes = [I, I, I, I, I, P, I, P, I, P, P, P, P, P, F, I, P, P, I]
    lib.orc_decode_attn_sparse.restype = I
    lib.orc_sparse_scores.argtypes = [I, I, I, I, I, P, I, P, I, P, P, P, F, I, P, P]
    lib.orc_sparse_scores.restype = I
    lib.orc_decode_attn_blocks.argtypes = [I, I, I, I, I, P, I, P, I, P, P, P, P, P, F, P, I, P, I]
    lib.orc_decode_attn_blocks.restype = I
    lib.orc_prefill_attn.argtypes = [I, I, I, I, I, P, I, P, I, P, P, P, P, P, I, P, F, P, I]
    lib.orc_prefill_attn.restype = I
    lib.orc_num_threads_available.restype = I
    _lib = lib
    return lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def threads_available() -> int:
    return int(_load().orc_num_threads_available())


# --------------------------------------------------------------- quantizers --
def quantize_kv(x: np.ndarray):
    """Per-row K/V quantizer (9-3 §2).  x: [..., hd] fp32 -> (codes int8 [..., hd],
    step fp32 [...]) where step = max-abs * fl(1/127) is the stored scale."""
    x = _c(x, np.float32)
    hd = x.shape[-1]
    rows = x.size // hd
    codes = np.empty(x.shape, np.int8)
    steps = np.empty(x.shape[:-1], np.float32)
    _load().orc_quantize_kv_rows(_p(x), rows, hd, _p(codes), _p(steps))
    return codes, steps


def quantize_q(q: np.ndarray):
    """Q block quantizer (9-2 §2 segment 1).  q: [..., hd] fp32 -> (codes int8
    [..., hd], qsc fp32 [..., hd/32])."""
    q = _c(q, np.float32)
    hd = q.shape[-1]
    assert hd % HEAD_BLOCK == 0
    rows = q.size // hd
    codes = np.empty(q.shape, np.int8)
    qsc = np.empty(q.shape[:-1] + (hd // HEAD_BLOCK,), np.float32)
    _load().orc_quantize_q_rows(_p(q), rows, hd, _p(codes), _p(qsc))
    return codes, qsc


def block_partials(cq: np.ndarray, ck: np.ndarray) -> np.ndarray:
    """Exact int32 block sums (9-2 §2 segment 2).  cq, ck: [hd] int8."""
    cq = _c(cq, np.int8)
    ck = _c(ck, np.int8)
    hd = cq.shape[-1]
    out = np.empty(hd // HEAD_BLOCK, np.int32)
    if _load().orc_block_partials(_p(cq), _p(ck), hd, _p(out)):
        raise OverflowError("block sum does not fit int32")
    return out


def dequantize(codes: np.ndarray, step: np.ndarray) -> np.ndarray:
    """Exact dequantization in double: code * step (row-wise step)."""
    return codes.astype(np.float64) * np.asarray(step, np.float64)[..., None]


def dequantize_q(codes: np.ndarray, qsc: np.ndarray) -> np.ndarray:
    """Exact dequantization of a block-quantized query in double."""
    hd = codes.shape[-1]
    return codes.astype(np.float64) * np.repeat(np.asarray(qsc, np.float64), HEAD_BLOCK, axis=-1)[..., :hd]


# ---------------------------------------------------------------- attention --
def attend_dense(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Three-pass attention in double (9-3 §1).  q [hd], k/v [n, hd] -> [hd] float64."""
    q = _c(q, np.float64)
    k = _c(k, np.float64)
    v = _c(v, np.float64)
    hd = q.shape[-1]
    n = k.shape[0] if k.ndim == 2 else 0
    out = np.empty(hd, np.float64)
    _load().orc_attend_dense(_p(q), _p(k), _p(v), n, hd, float(scale), _p(out))
    return out


def single_pass(cq, qsc, ck, ks, cv, vs, scale: float):
    """Page-literal fp32 single pass (9-2 §2 segments 2-3).  Returns (out fp32
    [hd], running max after each token fp32 [n])."""
    cq = _c(cq, np.int8)
    qsc = _c(qsc, np.float32)
    ck = _c(ck, np.int8)
    ks = _c(ks, np.float32)
    cv = _c(cv, np.int8)
    vs = _c(vs, np.float32)
    n, hd = ck.shape
    out = np.empty(hd, np.float32)
    trace = np.empty(max(n, 1), np.float32)
    _load().orc_single_pass(_p(cq), _p(qsc), _p(ck), _p(ks), _p(cv), _p(vs), n, hd,
                            float(np.float32(scale)), _p(out), _p(trace))
    return out, trace[:n]


class Cache:
    """Host copy of one layer's blocked q8 cache plus batch metadata.

    k_codes/v_codes: [num_blocks, kv_bs, nkv*hd] int8
    k_step/v_step:   [num_blocks, kv_bs, nkv] fp32
    block_table:     [batch, max_blocks_per_seq] int32; seq_lens: [batch] int32
    """

    def __init__(self, k_codes, v_codes, k_step, v_step, block_table, seq_lens, nkv, hd):
        self.k_codes = _c(k_codes, np.int8)
        self.v_codes = _c(v_codes, np.int8)
        self.k_step = _c(k_step, np.float32)
        self.v_step = _c(v_step, np.float32)
        self.block_table = _c(block_table, np.int32)
        self.seq_lens = _c(seq_lens, np.int32)
        self.nkv, self.hd = int(nkv), int(hd)
        self.num_blocks, self.kv_bs = self.k_codes.shape[0], self.k_codes.shape[1]
        self.batch, self.max_blocks_per_seq = self.block_table.shape


def decode_attn(cache: Cache, q: np.ndarray, nq: int, scale: float, nthreads: int = 0) -> np.ndarray:
    """Decode attention for every (b, h).  q: [batch, nq, hd] -> [batch, nq, hd] fp32."""
    q = _c(q, np.float32)
    out = np.empty(q.shape, np.float32)
    nthreads = nthreads or threads_available()
    rc = _load().orc_decode_attn(cache.batch, nq, cache.nkv, cache.hd, cache.kv_bs,
                                 _p(cache.block_table), cache.max_blocks_per_seq,
                                 _p(cache.seq_lens), cache.num_blocks,
                                 _p(cache.k_codes), _p(cache.v_codes),
                                 _p(cache.k_step), _p(cache.v_step),
                                 _p(q), float(np.float32(scale)), _p(out), nthreads)
    if rc:
        raise ValueError("oracle: bad sequence length or block id")
    return out


def decode_attn_rows(cache: Cache, q: np.ndarray, nq: int, scale: float, rows_bh, nthreads: int = 0):
    """Decode attention for selected rows (b * nq + h) only -> [len(rows), hd] fp32."""
    q = _c(q, np.float32)
    rows = _c(np.asarray(rows_bh), np.int64)
    out = np.empty((rows.size, cache.hd), np.float32)
    nthreads = nthreads or threads_available()
    rc = _load().orc_decode_attn_rows(nq, cache.nkv, cache.hd, cache.kv_bs,
                                      _p(cache.block_table), cache.max_blocks_per_seq,
                                      _p(cache.seq_lens), cache.num_blocks,
                                      _p(cache.k_codes), _p(cache.v_codes),
                                      _p(cache.k_step), _p(cache.v_step),
                                      _p(q), float(np.float32(scale)), _p(rows), rows.size,
                                      _p(out), nthreads)
    if rc:
        raise ValueError("oracle: bad sequence length or block id")
    return out


def qk_partials(cache: Cache, q: np.ndarray, nq: int, max_seq_len: int) -> np.ndarray:
    """int32 block partials [batch, nq, max_seq_len, hd/32] over the cache."""
    q = _c(q, np.float32)
    nblk = cache.hd // HEAD_BLOCK
    out = np.empty((cache.batch, nq, max_seq_len, nblk), np.int32)
    rc = _load().orc_qk_partials(cache.batch, nq, cache.nkv, cache.hd, cache.kv_bs,
                                 _p(cache.block_table), cache.max_blocks_per_seq,
                                 _p(cache.seq_lens), cache.num_blocks, max_seq_len,
                                 _p(cache.k_codes), _p(q), _p(out))
    if rc < 0:
        raise ValueError("oracle: bad sequence length or block id")
    if rc > 0:
        raise OverflowError("block sum does not fit int32")
    return out


def build_cache(k: np.ndarray, v: np.ndarray, seq_lens, block_table, num_blocks: int, kv_bs: int) -> Cache:
    """Quantize dense fp32 K/V ([batch, max_len, nkv, hd]) with the oracle's own
    quantizer and scatter them into a blocked cache through ``block_table``.
    Rows of the cache that no token occupies are left as zero codes / zero step."""
    batch, _, nkv, hd = k.shape
    kc = np.zeros((num_blocks, kv_bs, nkv * hd), np.int8)
    vc = np.zeros_like(kc)
    ks = np.zeros((num_blocks, kv_bs, nkv), np.float32)
    vs = np.zeros_like(ks)
    for b in range(batch):
        n = int(seq_lens[b])
        if n == 0:
            continue
        ck, dk = quantize_kv(k[b, :n])
        cv, dv = quantize_kv(v[b, :n])
        t = np.arange(n)
        blk = np.asarray(block_table)[b, t // kv_bs]
        row = t % kv_bs
        kc[blk, row] = ck.reshape(n, nkv * hd)
        vc[blk, row] = cv.reshape(n, nkv * hd)
        ks[blk, row] = dk
        vs[blk, row] = dv
    return Cache(kc, vc, ks, vs, block_table, seq_lens, nkv, hd)


class MirrorCache:
    """Host copy of one layer's fp32 mirror cache ("9-3" §3 closing note: the
    write path also stores every new K/V row in a float cache) plus batch
    metadata.

    k_f32/v_f32: [num_blocks, kv_bs, nkv*hd] fp32 (the code layout, fp32 elements)
    block_table: [batch, max_blocks_per_seq] int32; seq_lens: [batch] int32
    """

    def __init__(self, k_f32, v_f32, block_table, seq_lens, nkv, hd):
        self.k_f32 = _c(k_f32, np.float32)
        self.v_f32 = _c(v_f32, np.float32)
        self.block_table = _c(block_table, np.int32)
        self.seq_lens = _c(seq_lens, np.int32)
        self.nkv, self.hd = int(nkv), int(hd)
        self.num_blocks, self.kv_bs = self.k_f32.shape[0], self.k_f32.shape[1]
        self.batch, self.max_blocks_per_seq = self.block_table.shape


def decode_attn_f32(cache: MirrorCache, q: np.ndarray, nq: int, scale: float, rows_bh=None,
                    nthreads: int = 0) -> np.ndarray:
    """Exact decode attention over the fp32 mirror ("9-3" §1: scores of the
    raw fp32 q and K, max-subtracted softmax, weighted raw V; three passes in
    double).  Every (b, h) -> [batch, nq, hd], or the rows b * nq + h listed in
    rows_bh -> [len(rows_bh), hd]."""
    q = _c(q, np.float32)
    nthreads = nthreads or threads_available()
    if rows_bh is None:
        out = np.empty((cache.batch, nq, cache.hd), np.float32)
        rows_p, n_rows = None, cache.batch * nq
    else:
        rows = _c(np.asarray(rows_bh), np.int64)
        out = np.empty((rows.size, cache.hd), np.float32)
        rows_p, n_rows = _p(rows), rows.size
    rc = _load().orc_decode_attn_f32(cache.batch, nq, cache.nkv, cache.hd, cache.kv_bs,
                                     _p(cache.block_table), cache.max_blocks_per_seq,
                                     _p(cache.seq_lens), cache.num_blocks,
                                     _p(cache.k_f32), _p(cache.v_f32),
                                     _p(q), float(np.float32(scale)), rows_p, n_rows, _p(out), nthreads)
    if rc:
        raise ValueError("oracle: bad sequence length or block id")
    return out


def build_mirror(k: np.ndarray, v: np.ndarray, seq_lens, block_table, num_blocks: int, kv_bs: int) -> MirrorCache:
    """Scatter dense fp32 K/V ([batch, max_len, nkv, hd]) into a blocked fp32
    mirror through ``block_table``; rows no token occupies stay zero."""
    batch, _, nkv, hd = k.shape
    kf = np.zeros((num_blocks, kv_bs, nkv * hd), np.float32)
    vf = np.zeros_like(kf)
    for b in range(batch):
        n = int(seq_lens[b])
        if n == 0:
            continue
        t = np.arange(n)
        blk = np.asarray(block_table)[b, t // kv_bs]
        row = t % kv_bs
        kf[blk, row] = k[b, :n].reshape(n, nkv * hd)
        vf[blk, row] = v[b, :n].reshape(n, nkv * hd)
    return MirrorCache(kf, vf, block_table, seq_lens, nkv, hd)


SPARSE_BLOCK = 32     # positions per sparse block ("10-1" §2 defaults)
SPARSE_PROBES = 8     # probe samples per block


def decode_attn_sparse(cache: Cache, q: np.ndarray, nq: int, scale: float, topk: int = 32, nthreads: int = 0):
    """Block-sparse decode ("10-1" §1-§2): per (b, h) the top-k 32-token blocks
    by importance (``sparse_scores``, ranked exactly in double, ties to the
    lower block), then exact attention over their tokens.  Returns
    (out [batch, nq, hd] fp32, selected [batch, nq, topk] int32 block indices
    ascending, -1 after the last)."""
    if topk < 2:
        raise ValueError("topk must be at least 2 (two blocks are always kept below the sparse gate)")
    q = _c(q, np.float32)
    out = np.empty(q.shape, np.float32)
    sel = np.empty((cache.batch, nq, topk), np.int32)
    nthreads = nthreads or threads_available()
    rc = _load().orc_decode_attn_sparse(cache.batch, nq, cache.nkv, cache.hd, cache.kv_bs,
                                        _p(cache.block_table), cache.max_blocks_per_seq,
                                        _p(cache.seq_lens), cache.num_blocks,
                                        _p(cache.k_codes), _p(cache.v_codes),
                                        _p(cache.k_step), _p(cache.v_step),
                                        _p(q), float(np.float32(scale)), int(topk), _p(out), _p(sel), nthreads)
    if rc:
        raise ValueError("oracle: bad sequence length or block id")
    return out, sel


def prefill_attn(cache: Cache, q: np.ndarray, q_start, nq: int, scale: float, nthreads: int = 0) -> np.ndarray:
    """Batched prefill attention ("10-1" §1-§2, readings in the C source):
    the q_start[b + 1] - q_start[b] new tokens of sequence b are the last
    positions of its cache; query row r sits at position seq_lens[b] - nb +
    (r - q_start[b]) and attends causally to positions 0..p.  q: [total_q,
    nq, hd] fp32 -> the same shape."""
    q = _c(q, np.float32)
    qs = _c(np.asarray(q_start), np.int32)
    if qs.shape != (cache.batch + 1,) or q.shape[0] != int(qs[-1]):
        raise ValueError("q_start must be [batch + 1] with q_start[batch] = number of query rows")
    out = np.zeros(q.shape, np.float32)
    nthreads = nthreads or threads_available()
    rc = _load().orc_prefill_attn(cache.batch, nq, cache.nkv, cache.hd, cache.kv_bs,
                                  _p(cache.block_table), cache.max_blocks_per_seq,
                                  _p(cache.seq_lens), cache.num_blocks,
                                  _p(cache.k_codes), _p(cache.v_codes),
                                  _p(cache.k_step), _p(cache.v_step),
                                  _p(qs), int(q.shape[0]), _p(q), float(np.float32(scale)), _p(out), nthreads)
    if rc:
        raise ValueError("oracle: bad q_start, sequence length or block id")
    return out


def sparse_scores(cache: Cache, q: np.ndarray, nq: int, scale: float):
    """Importance of every 32-token block of every (b, h) ("10-1" §1-§2,
    readings in the C source): the largest over the block's probe rows 0, 4,
    ..., 28 of the page's q8 score s = (sum_b P_b * qscale_b) * kscale * scale
    ("9-2" §2 segment 2), in double.  Returns (scores [batch, nq, max blocks]
    float64, -inf past a sequence's last block; mags, the same shape: the
    largest over the block's probe rows of the same expression with every
    block term taken by absolute value, 0 past the end)."""
    q = _c(q, np.float32)
    max_nb = max(1, (int(cache.seq_lens.max()) + SPARSE_BLOCK - 1) // SPARSE_BLOCK)
    out = np.empty((cache.batch, nq, max_nb), np.float64)
    mag = np.empty((cache.batch, nq, max_nb), np.float64)
    rc = _load().orc_sparse_scores(cache.batch, nq, cache.nkv, cache.hd, cache.kv_bs,
                                   _p(cache.block_table), cache.max_blocks_per_seq,
                                   _p(cache.seq_lens), cache.num_blocks,
                                   _p(cache.k_codes), _p(cache.k_step),
                                   _p(q), float(np.float32(scale)), max_nb, _p(out), _p(mag))
    if rc:
        raise ValueError("oracle: bad sequence length or block id")
    return out, mag


def decode_attn_blocks(cache: Cache, q: np.ndarray, nq: int, scale: float, sel, nthreads: int = 0) -> np.ndarray:
    """Attention (O4-O7) of every (b, h) over the tokens of a given set of
    32-token blocks: sel [batch, nq, width] int32 block indices, ended by the
    first negative entry (the block order given is the summation order).
    q: [batch, nq, hd] -> [batch, nq, hd] fp32."""
    q = _c(q, np.float32)
    sel = _c(np.asarray(sel), np.int32)
    if sel.ndim != 3 or sel.shape[:2] != (cache.batch, nq):
        raise ValueError("sel must be [batch, nq, width]")
    out = np.empty(q.shape, np.float32)
    nthreads = nthreads or threads_available()
    rc = _load().orc_decode_attn_blocks(cache.batch, nq, cache.nkv, cache.hd, cache.kv_bs,
                                        _p(cache.block_table), cache.max_blocks_per_seq,
                                        _p(cache.seq_lens), cache.num_blocks,
                                        _p(cache.k_codes), _p(cache.v_codes),
                                        _p(cache.k_step), _p(cache.v_step),
                                        _p(q), float(np.float32(scale)), _p(sel), sel.shape[2], _p(out), nthreads)
    if rc:
        raise ValueError("oracle: bad sequence length, block index or block id")
    return out
