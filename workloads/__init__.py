"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds input recipes only -- shapes, lengths, value distributions,
block-table placement -- and none of the method's arithmetic (no quantization,
no attention).  Both the HIP path and the CPU oracle are fed from here.

The workloads stand in for the Qwen3-VL decode steps the pages measure
(Qwen3-VL-2B: 16 query heads / 8 KV heads; Qwen3-VL-8B: 32 / 8; head_dim 128;
kv_bs 32).  No dataset or checkpoint is involved: every value is drawn from a
seeded generator.
"""
from __future__ import annotations

import dataclasses

import numpy as np

HEAD_DIM = 128
KV_BS = 32
CHUNK_TOKENS = 2048  # bulk K/V are generated per (layer, sequence, chunk of this many tokens)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    nq: int
    nkv: int
    batch: int
    layers: int
    lens: tuple          # ("fixed", n) | ("uniform", lo, hi) | ("uniform_forced", lo, hi, forced)
    dist: str            # "normal" | "student3x3"
    seed: int
    append_per_step: int = 1   # tokens appended per sequence per decode step
    head_dim: int = HEAD_DIM
    kv_bs: int = KV_BS

    @property
    def group(self) -> int:
        return self.nq // self.nkv


# The five workloads (the second one is three context lengths).
WORKLOADS = {
    "single_head_256": Workload("single_head_256", 1, 1, 1, 1, ("fixed", 256), "normal", 1001),
    "qwen2b_b1_n506": Workload("qwen2b_b1_n506", 16, 8, 1, 28, ("fixed", 506), "normal", 1002),
    "qwen2b_b1_n2046": Workload("qwen2b_b1_n2046", 16, 8, 1, 28, ("fixed", 2046), "normal", 1002),
    "qwen2b_b1_n4059": Workload("qwen2b_b1_n4059", 16, 8, 1, 28, ("fixed", 4059), "normal", 1002),
    "qwen2b_b64_ragged": Workload("qwen2b_b64_ragged", 16, 8, 64, 28, ("uniform", 512, 8192), "normal", 1003),
    "qwen8b_b32_n32k": Workload("qwen8b_b32_n32k", 32, 8, 32, 36, ("fixed", 32768), "normal", 1004),
    "qwen8b_b1_n128k": Workload("qwen8b_b1_n128k", 32, 8, 1, 36, ("fixed", 131072), "normal", 1005),
    "qwen8b_b128_stress": Workload("qwen8b_b128_stress", 32, 8, 128, 36,
                                   ("uniform_forced", 1, 4096, (1, 2, 31, 32, 33, 63, 64, 65)),
                                   "student3x3", 1006),
    # batched prefill: append_per_step new tokens per sequence are the queries
    # (the last positions of each sequence).  The pages' prefill table runs
    # whole prompts of 506 / 2046 / 4059 tokens on the 2B model.
    "qwen2b_prefill_n4059": Workload("qwen2b_prefill_n4059", 16, 8, 1, 28, ("fixed", 4059), "normal", 1007,
                                     append_per_step=4059),
    "qwen2b_prefill_b8_c512": Workload("qwen2b_prefill_b8_c512", 16, 8, 8, 28, ("fixed", 4096), "normal", 1008,
                                       append_per_step=512),
}


def seq_lens(w: Workload) -> np.ndarray:
    """Context lengths (tokens visible to attention, including this step's append)."""
    rng = np.random.default_rng([w.seed, 1])
    kind = w.lens[0]
    if kind == "fixed":
        return np.full(w.batch, w.lens[1], np.int32)
    lo, hi = w.lens[1], w.lens[2]
    n = rng.integers(lo, hi + 1, size=w.batch).astype(np.int32)
    if kind == "uniform_forced":
        forced = np.asarray(w.lens[3], np.int32)
        n[: forced.size] = forced
        rng.shuffle(n)
    return n


def block_table(lens: np.ndarray, kv_bs: int, seed, spare_blocks: int = 0):
    """Scatter every sequence's logical blocks over a shared physical pool in a
    random order.  Returns (table [batch, max_blocks] int32, num_blocks).
    Unused table slots hold -1."""
    rng = np.random.default_rng([seed, 2])
    nblk = [(int(n) + kv_bs - 1) // kv_bs for n in lens]
    max_blocks = max(1, max(nblk) if len(nblk) else 1)
    total = sum(nblk) + spare_blocks
    perm = rng.permutation(max(total, 1)).astype(np.int32)
    table = np.full((len(lens), max_blocks), -1, np.int32)
    pos = 0
    for b, k in enumerate(nblk):
        table[b, :k] = perm[pos:pos + k]
        pos += k
    return table, max(total, 1)


def query(w: Workload, step: int = 0, layer: int = 0) -> np.ndarray:
    """q ~ N(0, 1), [batch, nq, head_dim] fp32."""
    rng = np.random.default_rng([w.seed, 3, layer, step])
    return rng.standard_normal((w.batch, w.nq, w.head_dim), dtype=np.float32)


def _student3x3_np(rng, shape):
    """3 * t(nu=3): z / sqrt(chi2_3 / 3), times 3."""
    z = rng.standard_normal(shape)
    chi2 = (rng.standard_normal((3,) + tuple(shape)) ** 2).sum(0)
    return 3.0 * z / np.sqrt(chi2 / 3.0)


def inject_small_rows_np(x: np.ndarray, rng) -> np.ndarray:
    """Stress rows ([..., head_dim] fp32, rows are (token, head)): 1% of rows
    scaled by 1e-7, 0.2% exactly zero, and a few rows whose max-abs is exactly
    1e-6 or the float just below it (the two sides of the 1e-6 guard)."""
    rows = x.reshape(-1, x.shape[-1])
    r = rows.shape[0]
    u = rng.random(r)
    rows[u < 0.01] *= np.float32(1e-7)
    rows[(u >= 0.01) & (u < 0.012)] = 0.0
    targets = (np.float32(1e-6), np.nextafter(np.float32(1e-6), np.float32(0)))
    picks = rng.choice(r, size=min(r, 4), replace=False) if r >= 4 else np.arange(r)
    for i, idx in enumerate(picks):
        t = targets[i % 2]
        row = rows[idx].astype(np.float64)
        amax = np.abs(row).max()
        row = row * (float(t) / amax) if amax > 0 else np.full_like(row, float(t) * 0.5)
        j = int(np.abs(row).argmax())
        out = np.clip(row.astype(np.float32), -t, t)
        out[j] = t if row[j] >= 0 else -t
        rows[idx] = out
    return x


def kv_host(w: Workload, lens: np.ndarray, layer: int = 0):
    """Dense fp32 K and V, [batch, max_len, nkv, head_dim], drawn on the host
    (numpy) -- for the small workloads the oracle checks in full."""
    max_len = int(max(1, lens.max() if lens.size else 1))
    shape = (w.batch, max_len, w.nkv, w.head_dim)
    out = []
    for which in (0, 1):
        rng = np.random.default_rng([w.seed, 4, layer, which])
        if w.dist == "normal":
            x = rng.standard_normal(shape, dtype=np.float32)
        else:
            x = _student3x3_np(rng, shape).astype(np.float32)
            x = inject_small_rows_np(x, rng)
        out.append(x)
    return out[0], out[1]


# ------------------------------------------------------------ torch (device) --
GUARD_ROWS_PER_DRAW = 4   # rows per torch draw pinned to the two sides of the 1e-6 guard


def _guard_rows_torch(x, gen):
    """In GUARD_ROWS_PER_DRAW rows of x ([..., head_dim] fp32, rows are
    (token, head)) picked with generator `gen`: rescale the row so that its
    max-abs is exactly 1e-6 (even picks) or the float just below it (odd
    picks) -- the two sides of the 1e-6 guard."""
    import torch
    rows = x.view(-1, x.shape[-1])
    if rows.shape[0] == 0:
        return x
    idx = torch.randint(0, rows.shape[0], (GUARD_ROWS_PER_DRAW,), generator=gen, device=x.device)
    two = torch.tensor([1e-6, float(np.nextafter(np.float32(1e-6), np.float32(0)))], dtype=torch.float32,
                       device=x.device)
    t = two[torch.arange(GUARD_ROWS_PER_DRAW, device=x.device) % 2][:, None]      # fp32 targets
    sel = rows[idx].double()
    amax = sel.abs().amax(-1, keepdim=True)
    scaled = torch.where(amax > 0, sel * (t.double() / torch.where(amax > 0, amax, 1.0)), 0.5 * t.double())
    out = torch.maximum(torch.minimum(scaled.float(), t), -t)
    j = scaled.abs().argmax(-1, keepdim=True)
    sign = torch.where(scaled.gather(1, j) >= 0, 1.0, -1.0).float()
    out.scatter_(1, j, sign * t)          # one element exactly +-target: max-abs == target
    rows[idx] = out
    return x


def _student3x3_torch(shape, gen, device):
    """3 * t(nu=3) (z / sqrt(chi2_3 / 3), times 3) with the stress rows: 1% of
    rows scaled by 1e-7, 0.2% exactly zero, and guard-boundary rows."""
    import torch
    z = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    e = torch.randn((3,) + tuple(shape), generator=gen, device=device, dtype=torch.float32)
    x = 3.0 * z / torch.sqrt((e * e).sum(0) / 3.0)
    u = torch.rand(shape[:-1], generator=gen, device=device)
    x = torch.where((u < 0.01)[..., None], x * 1e-7, x)
    x = torch.where(((u >= 0.01) & (u < 0.012))[..., None], torch.zeros_like(x), x)
    return _guard_rows_torch(x.contiguous(), gen)


def kv_chunk_torch(w: Workload, layer: int, b: int, chunk: int, which: int, device):
    """One chunk of CHUNK_TOKENS tokens of K (which=0) or V (which=1) for
    sequence b, [CHUNK_TOKENS, nkv, head_dim] fp32, drawn with torch's
    generator on ``device``.  The same key on the same device type always
    gives the same values, so a sampled row can be regenerated for the oracle."""
    import torch
    key = ((w.seed * 1000003 + layer) * 1000003 + b) * 1000003 + chunk * 2 + which
    g = torch.Generator(device=device)
    g.manual_seed(key % (2 ** 63))
    shape = (CHUNK_TOKENS, w.nkv, w.head_dim)
    if w.dist == "normal":
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return _student3x3_torch(shape, g, device)


def kv_pool_torch(w: Workload, n: int, gen, device):
    """n rows [n, nkv, head_dim] fp32 with the workload's value distribution,
    drawn from torch generator ``gen`` (bench.py appends cache history from
    such a pool at random offsets)."""
    import torch
    shape = (n, w.nkv, w.head_dim)
    if w.dist == "normal":
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return _student3x3_torch(shape, gen, device)


def kv_range_torch(w: Workload, layer: int, b: int, t0: int, t1: int, which: int, device):
    """Tokens [t0, t1) of sequence b, assembled from their chunks."""
    import torch
    parts = []
    c0, c1 = t0 // CHUNK_TOKENS, (t1 - 1) // CHUNK_TOKENS
    for c in range(c0, c1 + 1):
        x = kv_chunk_torch(w, layer, b, c, which, device)
        lo = max(t0, c * CHUNK_TOKENS) - c * CHUNK_TOKENS
        hi = min(t1, (c + 1) * CHUNK_TOKENS) - c * CHUNK_TOKENS
        parts.append(x[lo:hi])
    return torch.cat(parts, 0)


def softmax_scale(head_dim: int = HEAD_DIM) -> np.float32:
    """1/sqrt(head_dim) as fp32, the caller-supplied softmax scale."""
    return np.float32(1.0) / np.sqrt(np.float32(head_dim))


def kv_bytes_per_token(nkv: int, head_dim: int = HEAD_DIM) -> int:
    """Bytes one token adds to one layer of the q8 cache: int8 K and V codes plus
    one fp32 K and one fp32 V scale per KV head."""
    return nkv * (2 * head_dim + 2 * 4)


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


__all__ = ["Workload", "WORKLOADS", "seq_lens", "block_table", "query", "kv_host",
           "kv_chunk_torch", "kv_range_torch", "softmax_scale", "kv_bytes_per_token",
           "inject_small_rows_np", "ceil_div", "HEAD_DIM", "KV_BS", "CHUNK_TOKENS"]
