"""Python binding of libq8kv: q8 single-query decode attention for MI355X.

Argument marshalling only.  Every step of the path runs in the library's HIP
kernels (include/q8kv.h declares the C ABI); torch tensors are used only as
device memory and ``torch.cuda.current_stream()`` as the stream.  There is no
CPU or PyTorch fallback: if ``libq8kv.so`` is missing, importing the library
handle raises.

Entry points (same names as the C ABI, without the ``q8_`` prefix):
  kv_append, decode_attn, decode_attn_partial, decode_attn_merge,
  decode_attn_workspace_bytes, decode_attn_auto_parts, decode_step,
  decode_step_partial, decode_attn_f32, decode_attn_f32_partial,
  decode_attn_sparse, decode_attn_sparse_workspace_bytes, prefill_attn, issue_probe,
  quantize_q, qk_block_partials, abi_version, status_string, last_error.

Every entry point checks the tensors it passes on (dtype, contiguity, size,
one GPU device) and raises ValueError before anything is enqueued; the C ABI
itself only sees pointers and cannot.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq8kv.so")

Q8_OK, Q8_EINVAL, Q8_EUNSUPPORTED, Q8_EWORKSPACE, Q8_EHIP = 0, -1, -2, -3, -4
DEV_BAD_PLAN = 0x8
BATCH_INVARIANT = 0x1           # q8_batch.flags: Q8_BATCH_INVARIANT
ABI_VERSION = 7                 # the q8_batch / entry-point layout these bindings marshal
QPATH_VALU, QPATH_MFMA = 0, 1   # q8_quantize_q: two lanes or one lane per 32-block
DEV_BAD_SEQ_LEN, DEV_BAD_BLOCK_ID, DEV_BAD_TOKEN = 0x1, 0x2, 0x4
HEAD_DIM = 128


class Q8Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        lib = _load()
        text = lib.q8_status_string(status).decode()
        detail = lib.q8_last_error().decode() if status == Q8_EHIP else ""
        super().__init__(f"{where}: {text} ({status}) {detail}".strip())


class _Layer(ctypes.Structure):
    _fields_ = [("nkv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("kv_bs", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("k_f32", ctypes.c_void_p), ("v_f32", ctypes.c_void_p)]


class _Batch(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32), ("block_table", ctypes.c_void_p),
                ("seq_lens", ctypes.c_void_p), ("plan", ctypes.c_void_p), ("flags", ctypes.c_int32)]


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libq8kv.so not built ({LIB_PATH}); run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    LP, BP = ctypes.POINTER(_Layer), ctypes.POINTER(_Batch)
    lib.q8_kv_append.argtypes = [LP, BP, I32, P, P, P, P, P, P]
    lib.q8_kv_append.restype = I32
    lib.q8_decode_attn_auto_parts.argtypes = [LP, BP, I32]
    lib.q8_decode_attn_auto_parts.restype = I32
    lib.q8_decode_attn_workspace_bytes.argtypes = [LP, BP, I32, I32]
    lib.q8_decode_attn_workspace_bytes.restype = SZ
    lib.q8_decode_plan_bytes.argtypes = [LP, BP, I32, I32]
    lib.q8_decode_plan_bytes.restype = SZ
    lib.q8_decode_plan.argtypes = [LP, BP, I32, I32, P, SZ, P, P]
    lib.q8_decode_plan.restype = I32
    for name in ("q8_decode_attn", "q8_decode_attn_partial", "q8_decode_attn_merge", "q8_decode_attn_f32",
                 "q8_decode_attn_f32_partial"):
        fn = getattr(lib, name)
        fn.argtypes = [LP, BP, I32, P, F, P, I32, P, SZ, P, P]
        fn.restype = I32
    lib.q8_decode_attn_sparse_workspace_bytes.argtypes = [LP, BP, I32, I32]
    lib.q8_decode_attn_sparse_workspace_bytes.restype = SZ
    lib.q8_decode_attn_sparse.argtypes = [LP, BP, I32, P, F, P, I32, P, P, SZ, P, P]
    lib.q8_decode_attn_sparse.restype = I32
    for fn in (lib.q8_decode_step, lib.q8_decode_step_partial):
        fn.argtypes = [LP, BP, I32, P, P, P, F, P, I32, P, SZ, P, P]
        fn.restype = I32
    lib.q8_decode_step_static.argtypes = [LP, BP, I32, P, P, P, F, P, I32, P, P]
    lib.q8_decode_step_static.restype = I32
    lib.q8_decode_step_static_scratch_bytes.argtypes = []
    lib.q8_decode_step_static_scratch_bytes.restype = SZ
    lib.q8_prefill_attn.argtypes = [LP, BP, I32, P, I32, I32, P, F, P, P, P]
    lib.q8_prefill_attn.restype = I32
    lib.q8_quantize_q.argtypes = [P, I32, I32, I32, P, P, P]
    lib.q8_quantize_q.restype = I32
    lib.q8_qk_block_partials.argtypes = [LP, BP, I32, P, P, P, P, P, P]
    lib.q8_qk_block_partials.restype = I32
    lib.q8_stream_read.argtypes = [P, SZ, I32, I32, P, P]
    lib.q8_stream_read.restype = I32
    lib.q8_status_string.argtypes = [I32]
    lib.q8_status_string.restype = ctypes.c_char_p
    lib.q8_last_error.restype = ctypes.c_char_p
    lib.q8_abi_version.restype = I32
    if lib.q8_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH}: ABI {lib.q8_abi_version()}, these bindings need {ABI_VERSION}; rebuild it")
    _lib = lib
    return lib


def lib():
    """The loaded ctypes handle of libq8kv.so (raises ImportError if absent)."""
    return _load()


# ------------------------------------------------------------------ plumbing --
def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != Q8_OK:
        raise Q8Error(status, where)


# Argument checks of the Python entry points.  The C ABI sees only pointers
# and sizes, so it cannot tell an int64 table from an int32 one or a short
# buffer from a long one; a wrong dtype, a strided view or an undersized
# tensor would become an out-of-bounds device access.  Every tensor an entry
# point hands to the library is checked here first (ValueError otherwise):
# dtype, contiguity and size of each, then that all sit on one GPU.
class _Args:
    def __init__(self):
        self.tensors = []

    def need(self, t, name: str, dtype, min_numel: int, exact: bool = False):
        """t: a contiguous tensor of `dtype` with at least (exactly, if
        `exact`) `min_numel` elements; None is passed over."""
        import torch
        if t is None:
            return self
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name}: expected a torch tensor, got {type(t).__name__} "
                             "(raw pointers go through lib() directly)")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: must be contiguous")
        n = t.numel()
        if (exact and n != min_numel) or n < min_numel:
            raise ValueError(f"{name}: {n} elements, expected {'' if exact else 'at least '}{min_numel}")
        self.tensors.append((name, t))
        return self

    def layer(self, layer: "KVLayer"):
        import torch
        if (layer.k_f32 is None) != (layer.v_f32 is None):
            raise ValueError("layer.k_f32 and layer.v_f32: both or neither")
        row = layer.nkv_heads * layer.head_dim
        rows = layer.num_blocks * layer.kv_bs
        self.need(layer.k_codes, "layer.k_codes", torch.int8, rows * row, exact=True)
        self.need(layer.v_codes, "layer.v_codes", torch.int8, rows * row, exact=True)
        self.need(layer.k_scale, "layer.k_scale", torch.float32, rows * layer.nkv_heads, exact=True)
        self.need(layer.v_scale, "layer.v_scale", torch.float32, rows * layer.nkv_heads, exact=True)
        self.need(layer.k_f32, "layer.k_f32", torch.float32, rows * row, exact=True)
        self.need(layer.v_f32, "layer.v_f32", torch.float32, rows * row, exact=True)
        return self

    def batch(self, batch: "Batch"):
        import torch
        self.need(batch.block_table, "batch.block_table", torch.int32, batch.batch * batch.max_blocks_per_seq,
                  exact=True)
        self.need(batch.seq_lens, "batch.seq_lens", torch.int32, batch.batch, exact=True)
        if batch.plan is not None:
            if not isinstance(batch.plan, torch.Tensor):
                raise ValueError("batch.plan: expected a torch tensor")
            self.need(batch.plan, "batch.plan", batch.plan.dtype, 0)
        return self

    def done(self):
        """All tensors on one GPU; returns the workspace-independent device."""
        dev = None
        for name, t in self.tensors:
            if not t.is_cuda:
                raise ValueError(f"{name}: must be on a GPU (is on {t.device})")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"{name}: on {t.device}, the other arguments are on {dev}")
        return dev


def _nbytes(workspace) -> int:
    return workspace.numel() * workspace.element_size()


@dataclasses.dataclass
class KVLayer:
    """One layer's blocked q8 pool (torch tensors on the GPU, or raw pointers).

    k_codes/v_codes: int8 [num_blocks, kv_bs, nkv_heads * head_dim]
    k_scale/v_scale: fp32 [num_blocks, nkv_heads, kv_bs]
    k_f32/v_f32:     fp32 [num_blocks, kv_bs, nkv_heads * head_dim] mirror, or None
    """
    k_codes: object
    v_codes: object
    k_scale: object
    v_scale: object
    nkv_heads: int
    kv_bs: int
    num_blocks: int
    head_dim: int = HEAD_DIM
    k_f32: object = None
    v_f32: object = None

    def c(self) -> _Layer:
        return _Layer(self.nkv_heads, self.head_dim, self.kv_bs, self.num_blocks,
                      _ptr(self.k_codes), _ptr(self.v_codes), _ptr(self.k_scale), _ptr(self.v_scale),
                      _ptr(self.k_f32), _ptr(self.v_f32))


@dataclasses.dataclass
class Batch:
    """Per-step batch metadata: block_table int32 [batch, max_blocks_per_seq],
    seq_lens int32 [batch] (device tensors), host-side max_seq_len, an
    optional step plan (a device tensor filled by decode_plan), and whether
    the decode calls cut it batch-invariantly (Q8_BATCH_INVARIANT: a
    sequence's bits independent of the rest of the batch; no plan)."""
    block_table: object
    seq_lens: object
    batch: int
    max_blocks_per_seq: int
    max_seq_len: int
    plan: object = None
    invariant: bool = False

    def c(self) -> _Batch:
        return _Batch(self.batch, self.max_blocks_per_seq, self.max_seq_len,
                      _ptr(self.block_table), _ptr(self.seq_lens), _ptr(self.plan),
                      BATCH_INVARIANT if self.invariant else 0)

    def with_plan(self, plan) -> "Batch":
        """The same batch with a step plan (or None)."""
        return dataclasses.replace(self, plan=plan)


def alloc_layer(num_blocks: int, kv_bs: int, nkv_heads: int, device="cuda", head_dim: int = HEAD_DIM,
                mirror: bool = False) -> KVLayer:
    """Allocate an uninitialised pool with torch (device memory only); with
    mirror=True also the fp32 mirror that q8_kv_append fills and
    q8_decode_attn_f32 reads."""
    import torch
    kc = torch.empty((num_blocks, kv_bs, nkv_heads * head_dim), dtype=torch.int8, device=device)
    vc = torch.empty_like(kc)
    ks = torch.empty((num_blocks, nkv_heads, kv_bs), dtype=torch.float32, device=device)
    vs = torch.empty_like(ks)
    kf = vf = None
    if mirror:
        kf = torch.empty((num_blocks, kv_bs, nkv_heads * head_dim), dtype=torch.float32, device=device)
        vf = torch.empty_like(kf)
    return KVLayer(kc, vc, ks, vs, nkv_heads, kv_bs, num_blocks, head_dim, kf, vf)


def make_batch(block_table, seq_lens, max_seq_len: int, invariant: bool = False) -> Batch:
    """Batch from block_table int32 [batch, max_blocks_per_seq] and seq_lens
    int32 [batch] (contiguous GPU tensors on one device); invariant=True asks
    the decode calls for the batch-invariant cut."""
    import torch
    if not isinstance(block_table, torch.Tensor) or block_table.dim() != 2:
        raise ValueError("block_table: expected a 2-D torch tensor [batch, max_blocks_per_seq]")
    b, mb = int(block_table.shape[0]), int(block_table.shape[1])
    (_Args().need(block_table, "block_table", torch.int32, b * mb, exact=True)
            .need(seq_lens, "seq_lens", torch.int32, b, exact=True).done())
    return Batch(block_table, seq_lens, b, mb, int(max_seq_len), invariant=bool(invariant))


# ------------------------------------------------------------- entry points --
def _common(layer, batch, dev_status):
    import torch
    return _Args().layer(layer).batch(batch).need(dev_status, "dev_status", torch.int32, 1)


def _q_out(args, batch, nq_heads, q, out, head_dim=HEAD_DIM):
    import torch
    n = batch.batch * nq_heads * head_dim
    return args.need(q, "q", torch.float32, n).need(out, "out", torch.float32, n)


def kv_append(layer: KVLayer, batch: Batch, tok_seq, tok_pos, k_new, v_new, dev_status=None, stream=None):
    """q8_kv_append: quantize k_new/v_new [n_tokens, nkv, 128] fp32 into the
    cache at (tok_seq, tok_pos) (int32 [n_tokens])."""
    import torch
    if not isinstance(tok_seq, torch.Tensor):
        raise ValueError("tok_seq: expected a torch tensor")
    n = int(tok_seq.numel())
    row = layer.nkv_heads * layer.head_dim
    (_common(layer, batch, dev_status).need(tok_seq, "tok_seq", torch.int32, n, exact=True)
        .need(tok_pos, "tok_pos", torch.int32, n, exact=True)
        .need(k_new, "k_new", torch.float32, n * row).need(v_new, "v_new", torch.float32, n * row).done())
    st = _load().q8_kv_append(ctypes.byref(layer.c()), ctypes.byref(batch.c()), n, _ptr(tok_seq),
                              _ptr(tok_pos), _ptr(k_new), _ptr(v_new), _ptr(dev_status), _stream(stream))
    _check(st, "q8_kv_append")


def decode_plan_bytes(layer: KVLayer, batch: Batch, nq_heads: int, nparts: int = 0) -> int:
    return int(_load().q8_decode_plan_bytes(ctypes.byref(layer.c()), ctypes.byref(batch.c()), nq_heads, nparts))


def decode_plan(layer: KVLayer, batch: Batch, nq_heads: int, plan, nparts: int = 0, dev_status=None, stream=None):
    """q8_decode_plan: fill `plan` (a GPU tensor of at least decode_plan_bytes
    bytes) with the step's cut; use it through batch.with_plan(plan) in every
    layer's decode call of the step."""
    _common(layer, batch.with_plan(None), dev_status).need(plan, "plan", None, 0).done()
    st = _load().q8_decode_plan(ctypes.byref(layer.c()), ctypes.byref(batch.with_plan(None).c()), nq_heads,
                                int(nparts), _ptr(plan), _nbytes(plan), _ptr(dev_status), _stream(stream))
    _check(st, "q8_decode_plan")


def decode_attn_auto_parts(layer: KVLayer, batch: Batch, nq_heads: int) -> int:
    return int(_load().q8_decode_attn_auto_parts(ctypes.byref(layer.c()), ctypes.byref(batch.c()), nq_heads))


def decode_attn_workspace_bytes(layer: KVLayer, batch: Batch, nq_heads: int, nparts: int = 0) -> int:
    return int(_load().q8_decode_attn_workspace_bytes(ctypes.byref(layer.c()), ctypes.byref(batch.c()),
                                                      nq_heads, nparts))


def _decode(name, layer, batch, nq_heads, q, scale, out, workspace, nparts, dev_status, stream):
    args = _q_out(_common(layer, batch, dev_status), batch, nq_heads, q, out, layer.head_dim)
    args.need(workspace, "workspace", None, 0).done()
    fn = getattr(_load(), name)
    st = fn(ctypes.byref(layer.c()), ctypes.byref(batch.c()), nq_heads, _ptr(q), float(scale), _ptr(out),
            nparts, _ptr(workspace), _nbytes(workspace), _ptr(dev_status), _stream(stream))
    _check(st, name)


def decode_attn(layer, batch, nq_heads, q, scale, out, workspace, nparts=0, dev_status=None, stream=None):
    """q8_decode_attn: out [batch, nq, 128] fp32 from q [batch, nq, 128] fp32."""
    _decode("q8_decode_attn", layer, batch, nq_heads, q, scale, out, workspace, nparts, dev_status, stream)


def decode_attn_f32(layer, batch, nq_heads, q, scale, out, workspace, nparts=0, dev_status=None, stream=None):
    """q8_decode_attn_f32: exact attention over the layer's fp32 mirror."""
    _decode("q8_decode_attn_f32", layer, batch, nq_heads, q, scale, out, workspace, nparts, dev_status, stream)


def decode_attn_f32_partial(layer, batch, nq_heads, q, scale, out, workspace, nparts=0, dev_status=None,
                            stream=None):
    _decode("q8_decode_attn_f32_partial", layer, batch, nq_heads, q, scale, out, workspace, nparts, dev_status,
            stream)


def decode_attn_partial(layer, batch, nq_heads, q, scale, out, workspace, nparts=0, dev_status=None, stream=None):
    _decode("q8_decode_attn_partial", layer, batch, nq_heads, q, scale, out, workspace, nparts, dev_status, stream)


def decode_attn_merge(layer, batch, nq_heads, q, scale, out, workspace, nparts=0, dev_status=None, stream=None):
    _decode("q8_decode_attn_merge", layer, batch, nq_heads, q, scale, out, workspace, nparts, dev_status, stream)


def decode_attn_sparse_workspace_bytes(layer, batch, nq_heads: int, topk: int = 32) -> int:
    return int(_load().q8_decode_attn_sparse_workspace_bytes(ctypes.byref(layer.c()), ctypes.byref(batch.c()),
                                                             nq_heads, topk))


def decode_attn_sparse(layer, batch, nq_heads, q, scale, out, workspace, topk=32, selected=None, dev_status=None,
                       stream=None):
    """q8_decode_attn_sparse: top-k 32-token blocks per query head by probe,
    exact q8 attention over them.  selected: optional int32 [batch, nq, topk]."""
    import torch
    args = _q_out(_common(layer, batch, dev_status), batch, nq_heads, q, out, layer.head_dim)
    (args.need(selected, "selected", torch.int32, batch.batch * nq_heads * int(topk))
         .need(workspace, "workspace", None, 0).done())
    st = _load().q8_decode_attn_sparse(ctypes.byref(layer.c()), ctypes.byref(batch.c()), nq_heads, _ptr(q),
                                       float(scale), _ptr(out), int(topk), _ptr(selected), _ptr(workspace),
                                       _nbytes(workspace), _ptr(dev_status), _stream(stream))
    _check(st, "q8_decode_attn_sparse")


def _step(name, layer, batch, nq_heads, k_new, v_new, q, scale, out, workspace, nparts, dev_status, stream):
    import torch
    row = layer.nkv_heads * layer.head_dim
    args = _q_out(_common(layer, batch, dev_status), batch, nq_heads, q, out, layer.head_dim)
    (args.need(k_new, "k_new", torch.float32, batch.batch * row)
         .need(v_new, "v_new", torch.float32, batch.batch * row)
         .need(workspace, "workspace", None, 0).done())
    st = getattr(_load(), name)(ctypes.byref(layer.c()), ctypes.byref(batch.c()), nq_heads, _ptr(k_new),
                                _ptr(v_new), _ptr(q), float(scale), _ptr(out), int(nparts), _ptr(workspace),
                                _nbytes(workspace), _ptr(dev_status), _stream(stream))
    _check(st, name)


def decode_step(layer, batch, nq_heads, k_new, v_new, q, scale, out, workspace, nparts=0, dev_status=None,
                stream=None):
    """q8_decode_step: append the token at position seq_lens[b] - 1 of every
    sequence (k_new, v_new [batch, nkv, 128] fp32) and decode, in one call."""
    _step("q8_decode_step", layer, batch, nq_heads, k_new, v_new, q, scale, out, workspace, nparts, dev_status,
          stream)


def decode_step_partial(layer, batch, nq_heads, k_new, v_new, q, scale, out, workspace, nparts=0,
                        dev_status=None, stream=None):
    """q8_decode_step_partial: the step's append + cache walk; decode_attn_merge
    with the same arguments completes it."""
    _step("q8_decode_step_partial", layer, batch, nq_heads, k_new, v_new, q, scale, out, workspace, nparts,
          dev_status, stream)


def decode_step_static(layer, batch, nq_heads, k_new, v_new, q, scale, out, nparts=0, dev_status=None,
                       stream=None):
    """q8_decode_step_static: q8_decode_step without a workspace (the
    library's own device scratch; nothing allocated)."""
    import torch
    row = layer.nkv_heads * layer.head_dim
    args = _q_out(_common(layer, batch, dev_status), batch, nq_heads, q, out, layer.head_dim)
    (args.need(k_new, "k_new", torch.float32, batch.batch * row)
         .need(v_new, "v_new", torch.float32, batch.batch * row).done())
    st = _load().q8_decode_step_static(ctypes.byref(layer.c()), ctypes.byref(batch.c()), nq_heads, _ptr(k_new),
                                       _ptr(v_new), _ptr(q), float(scale), _ptr(out), int(nparts),
                                       _ptr(dev_status), _stream(stream))
    _check(st, "q8_decode_step_static")


def decode_step_static_scratch_bytes() -> int:
    return int(_load().q8_decode_step_static_scratch_bytes())


def prefill_attn(layer, batch, nq_heads, q_start, max_new, q, scale, out, dev_status=None, stream=None):
    """q8_prefill_attn: causal attention of the new tokens' queries (the last
    q_start[b + 1] - q_start[b] positions of each sequence's cache) over the
    q8 cache.  q_start: device int32 [batch + 1]; q, out: [total_q, nq, 128]."""
    import torch
    if not isinstance(q, torch.Tensor) or q.dim() < 1:
        raise ValueError("q: expected a torch tensor [total_q, nq, 128]")
    total_q = int(q.shape[0])
    n = total_q * nq_heads * layer.head_dim
    (_common(layer, batch, dev_status).need(q_start, "q_start", torch.int32, batch.batch + 1, exact=True)
        .need(q, "q", torch.float32, n, exact=True).need(out, "out", torch.float32, n).done())
    st = _load().q8_prefill_attn(ctypes.byref(layer.c()), ctypes.byref(batch.c()), nq_heads, _ptr(q_start),
                                 total_q, int(max_new), _ptr(q), float(scale), _ptr(out), _ptr(dev_status),
                                 _stream(stream))
    _check(st, "q8_prefill_attn")


def quantize_q(q, codes, qscale, path=QPATH_VALU, stream=None):
    """q8_quantize_q test hook: q [rows, 128] fp32 -> codes int8 [rows, 128],
    qscale fp32 [rows, 4], by the decode's two-lanes-per-block routine
    (path=QPATH_VALU) or its one-lane-per-block matrix-core one (QPATH_MFMA)."""
    import torch
    if not isinstance(q, torch.Tensor) or q.dim() < 1:
        raise ValueError("q: expected a torch tensor [rows, 128]")
    rows = int(q.shape[0])
    (_Args().need(q, "q", torch.float32, rows * HEAD_DIM, exact=True)
        .need(codes, "codes", torch.int8, rows * HEAD_DIM)
        .need(qscale, "qscale", torch.float32, rows * (HEAD_DIM // 32)).done())
    st = _load().q8_quantize_q(_ptr(q), rows, HEAD_DIM, int(path), _ptr(codes), _ptr(qscale), _stream(stream))
    _check(st, "q8_quantize_q")


def qk_block_partials(layer, batch, nq_heads, q, partials, qcodes=None, qscale=None, dev_status=None, stream=None):
    """q8_qk_block_partials test hook: partials int32 [batch, nq, max_seq_len, 4]
    and, optionally, the query codes int8 [batch, nq, 128] and scales fp32
    [batch, nq, 4] they were formed with, by the decode's routine for the
    shape."""
    import torch
    nblk = layer.head_dim // 32
    if (qcodes is None) != (qscale is None):
        raise ValueError("qcodes and qscale: both or neither")
    (_common(layer, batch, dev_status).need(q, "q", torch.float32, batch.batch * nq_heads * layer.head_dim)
        .need(partials, "partials", torch.int32, batch.batch * nq_heads * batch.max_seq_len * nblk)
        .need(qcodes, "qcodes", torch.int8, batch.batch * nq_heads * layer.head_dim)
        .need(qscale, "qscale", torch.float32, batch.batch * nq_heads * nblk).done())
    st = _load().q8_qk_block_partials(ctypes.byref(layer.c()), ctypes.byref(batch.c()), nq_heads, _ptr(q),
                                      _ptr(partials), _ptr(qcodes), _ptr(qscale), _ptr(dev_status),
                                      _stream(stream))
    _check(st, "q8_qk_block_partials")


def stream_read(buf, workgroups: int, nontemporal: bool, sink, stream=None):
    """q8_stream_read measurement hook: read every byte of buf (a contiguous
    GPU tensor, size a multiple of 16 bytes) once; sink: int32 GPU tensor."""
    import torch
    if not isinstance(buf, torch.Tensor):
        raise ValueError("buf: expected a torch tensor")
    _Args().need(buf, "buf", buf.dtype, 0).need(sink, "sink", torch.int32, 1).done()
    st = _load().q8_stream_read(_ptr(buf), _nbytes(buf), int(workgroups), int(bool(nontemporal)), _ptr(sink),
                                _stream(stream))
    _check(st, "q8_stream_read")


def issue_probe(out, mode: int, valu_iters: int, mfma_iters: int, workgroups: int, stream=None):
    """q8_issue_probe measurement hook (VALU and matrix-core issue on one CU);
    out: fp32 GPU scratch tensor of at least workgroups * 1024 elements."""
    import torch
    lib = _load()
    if not getattr(lib, "_issue_probe_typed", False):
        lib.q8_issue_probe.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_void_p]
        lib.q8_issue_probe.restype = ctypes.c_int32
        lib._issue_probe_typed = True
    _Args().need(out, "out", torch.float32, int(workgroups) * 1024).done()
    st = lib.q8_issue_probe(_ptr(out), int(mode), int(valu_iters), int(mfma_iters), int(workgroups), _stream(stream))
    _check(st, "q8_issue_probe")


def abi_version() -> int:
    return int(_load().q8_abi_version())


def status_string(status: int) -> str:
    return _load().q8_status_string(status).decode()


def last_error() -> str:
    return _load().q8_last_error().decode()
