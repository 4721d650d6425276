"""CPU tests of the C ABI: the library loads without a GPU, exports every
function include/q8kv.h declares, and rejects bad arguments on the host
before anything is enqueued.  No test here launches a kernel."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q8kv.h")


@pytest.fixture(scope="module")
def q8():
    import decode_attention_int8_kv_amd as m
    if not os.path.exists(m.LIB_PATH):
        from decode_attention_int8_kv_amd import build
        build.build()
    m._load()
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q8_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("q8_kv_append", "q8_decode_attn", "q8_decode_attn_partial", "q8_decode_attn_merge",
                 "q8_decode_attn_workspace_bytes", "q8_decode_attn_auto_parts", "q8_quantize_q",
                 "q8_qk_block_partials", "q8_status_string", "q8_last_error", "q8_abi_version",
                 "q8_decode_attn_f32", "q8_decode_attn_sparse", "q8_prefill_attn", "q8_decode_step"):
        assert want in names


def test_library_exports_every_declared_symbol(q8):
    lib = ctypes.CDLL(q8.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(q8):
    assert q8.abi_version() == 7 == q8.ABI_VERSION
    assert q8.status_string(0) == "ok"
    assert q8.status_string(-3).startswith("workspace")
    assert q8.last_error() == ""


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def layer(q8, **kw):
    d = dict(k_codes=FAKE, v_codes=FAKE, k_scale=FAKE, v_scale=FAKE, nkv_heads=8, kv_bs=32, num_blocks=100)
    d.update(kw)
    return q8.KVLayer(**d)


def batch(q8, **kw):
    d = dict(block_table=FAKE, seq_lens=FAKE, batch=4, max_blocks_per_seq=10, max_seq_len=300)
    d.update(kw)
    return q8.Batch(**d)


def call_append(q8, L, B, n=1, **ptrs):
    p = dict(tok_seq=FAKE, tok_pos=FAKE, k_new=FAKE, v_new=FAKE)
    p.update(ptrs)
    return q8.lib().q8_kv_append(ctypes.byref(L.c()), ctypes.byref(B.c()), n, p["tok_seq"], p["tok_pos"],
                                 p["k_new"], p["v_new"], None, None)


def call_decode(q8, L, B, nq=16, ws=FAKE, ws_bytes=1 << 30, q=FAKE, out=FAKE, nparts=4):
    return q8.lib().q8_decode_attn(ctypes.byref(L.c()), ctypes.byref(B.c()), nq, q, 0.088, out, nparts,
                                   ws, ws_bytes, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), -2), (dict(kv_bs=24), -2), (dict(kv_bs=4), -2), (dict(kv_bs=2048), -2),
    (dict(nkv_heads=0), -2), (dict(nkv_heads=17), -2), (dict(num_blocks=0), -1),
    (dict(k_codes=0), -1), (dict(v_codes=FAKE + 8), -1), (dict(k_scale=FAKE + 2), -1),
])
def test_layer_validation(q8, kw, status):
    assert call_append(q8, layer(q8, **kw), batch(q8)) == status
    assert call_decode(q8, layer(q8, **kw), batch(q8)) == status


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), -1), (dict(batch=5000), -2), (dict(max_blocks_per_seq=0), -1),
    (dict(max_seq_len=-1), -1), (dict(max_seq_len=321), -1), (dict(block_table=0), -1),
    (dict(seq_lens=FAKE + 1), -1),
])
def test_batch_validation(q8, kw, status):
    assert call_append(q8, layer(q8), batch(q8, **kw)) == status
    assert call_decode(q8, layer(q8), batch(q8, **kw)) == status


def test_append_argument_validation(q8):
    L, B = layer(q8), batch(q8)
    assert call_append(q8, L, B, n=0) == 0            # no-op, nothing enqueued
    assert call_append(q8, L, B, n=-1) == -1
    assert call_append(q8, L, B, tok_seq=0) == -1
    assert call_append(q8, L, B, k_new=FAKE + 4) == -1  # 16-byte alignment


def call_decode_f32(q8, L, B, nq=16, ws=FAKE, ws_bytes=1 << 30, q=FAKE, out=FAKE, nparts=4):
    return q8.lib().q8_decode_attn_f32(ctypes.byref(L.c()), ctypes.byref(B.c()), nq, q, 0.088, out, nparts,
                                       ws, ws_bytes, None, None)


def test_mirror_validation(q8):
    B = batch(q8)
    # the fp32 mirror is all or nothing, 16-byte aligned
    assert call_append(q8, layer(q8, k_f32=FAKE), B) == -1
    assert call_append(q8, layer(q8, v_f32=FAKE), B) == -1
    assert call_append(q8, layer(q8, k_f32=FAKE + 4, v_f32=FAKE), B) == -1
    assert call_decode(q8, layer(q8, k_f32=FAKE, v_f32=FAKE + 8), B) == -1
    # exact decode needs the mirror; otherwise it validates like q8_decode_attn
    assert call_decode_f32(q8, layer(q8), B) == -1
    L = layer(q8, k_f32=FAKE, v_f32=FAKE)
    assert call_decode_f32(q8, L, B, nq=24) == -2
    assert call_decode_f32(q8, L, B, ws=0) == -3
    assert call_decode_f32(q8, L, B, ws_bytes=q8.decode_attn_workspace_bytes(L, B, 16, 4) - 1) == -3


def test_decode_argument_validation(q8):
    L, B = layer(q8), batch(q8)
    assert call_decode(q8, L, B, nq=12) == -1           # nq % nkv != 0
    assert call_decode(q8, L, B, nq=24) == -2           # group 3
    assert call_decode(q8, L, B, nq=128) == -2          # group 16
    assert call_decode(q8, L, B, q=0) == -1
    assert call_decode(q8, L, B, out=FAKE + 4) == -1
    assert call_decode(q8, L, B, nparts=-1) == -1
    assert call_decode(q8, L, B, ws=0) == -3
    assert call_decode(q8, L, B, ws=FAKE + 64) == -3    # 256-byte alignment
    need = q8.decode_attn_workspace_bytes(L, B, 16, 4)
    assert need > 0
    assert call_decode(q8, L, B, ws_bytes=need - 1) == -3


def test_workspace_size_grows_with_parts_and_heads(q8):
    L, B = layer(q8), batch(q8)
    a = q8.decode_attn_workspace_bytes(L, B, 16, 4)
    b = q8.decode_attn_workspace_bytes(L, B, 16, 8)
    c = q8.decode_attn_workspace_bytes(L, B, 32, 8)
    assert 0 < a < b < c
    # every range can leave two cut pieces of (M, S, acc[128]) per query head
    assert b - a >= 4 * 2 * 16 * (128 + 2) * 4
    assert q8.decode_attn_workspace_bytes(L, B, 12, 4) == 0


def test_hook_validation(q8):
    lib = q8.lib()
    assert lib.q8_quantize_q(FAKE, 4, 64, 0, FAKE, FAKE, None) == -2
    assert lib.q8_quantize_q(FAKE, -1, 128, 0, FAKE, FAKE, None) == -1
    assert lib.q8_quantize_q(FAKE, 0, 128, 0, FAKE, FAKE, None) == 0
    assert lib.q8_quantize_q(FAKE + 4, 1, 128, 0, FAKE, FAKE, None) == -1
    assert lib.q8_quantize_q(FAKE, 1, 128, 2, FAKE, FAKE, None) == -1      # unknown path
    assert lib.q8_quantize_q(FAKE, 1, 128, -1, FAKE, FAKE, None) == -1
    L, B = layer(q8), batch(q8)

    def partials(nq=16, q=FAKE, p=FAKE, qc=None, qs=None):
        return lib.q8_qk_block_partials(ctypes.byref(L.c()), ctypes.byref(B.c()), nq, q, p, qc, qs, None, None)

    assert partials(nq=12) == -1
    assert partials(p=0) == -1
    assert partials(p=FAKE + 4) == -1          # the partials are written 16 bytes at a time
    assert partials(qc=FAKE) == -1             # codes and scales: both or neither
    assert partials(qs=FAKE) == -1
    assert partials(qc=FAKE + 8, qs=FAKE) == -1


def test_stream_read_validation(q8):
    lib = q8.lib()
    assert lib.q8_stream_read(FAKE, 0, 256, 1, FAKE, None) == 0          # nothing to read
    assert lib.q8_stream_read(FAKE, 100, 256, 1, FAKE, None) == -1       # not a multiple of 16
    assert lib.q8_stream_read(FAKE + 8, 1024, 256, 1, FAKE, None) == -1  # misaligned buffer
    assert lib.q8_stream_read(FAKE, 1024, 0, 1, FAKE, None) == -1
    assert lib.q8_stream_read(FAKE, 1024, 70000, 1, FAKE, None) == -1
    assert lib.q8_stream_read(FAKE, 1024, 256, 2, FAKE, None) == -1
    assert lib.q8_stream_read(FAKE, 1024, 256, 1, None, None) == -1


def test_issue_probe_validation(q8):
    lib = q8.lib()
    f = lib.q8_issue_probe
    f.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    assert f(None, 0, 16, 16, 256, None) == -1       # no buffer
    assert f(FAKE + 2, 0, 16, 16, 256, None) == -1   # misaligned
    assert f(FAKE, 5, 16, 16, 256, None) == -1       # unknown mode
    assert f(FAKE, -1, 16, 16, 256, None) == -1
    assert f(FAKE, 0, 0, 16, 256, None) == -1        # iteration counts
    assert f(FAKE, 0, 16, (1 << 20) + 1, 256, None) == -1
    assert f(FAKE, 0, 16, 16, 0, None) == -1         # workgroups
    assert f(FAKE, 0, 16, 16, 65537, None) == -1


def test_binding_refuses_to_run_without_library(tmp_path, monkeypatch):
    import decode_attention_int8_kv_amd as m
    monkeypatch.setattr(m, "_lib", None)
    monkeypatch.setattr(m, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        m.lib()


def call_sparse(q8, L, B, nq=16, topk=32, ws=FAKE, ws_bytes=1 << 30, q=FAKE, out=FAKE, sel=None):
    return q8.lib().q8_decode_attn_sparse(ctypes.byref(L.c()), ctypes.byref(B.c()), nq, q, 0.088, out, topk, sel,
                                          ws, ws_bytes, None, None)


def test_sparse_validation(q8):
    L, B = layer(q8), batch(q8)
    assert call_sparse(q8, L, B, topk=1) == -1
    assert call_sparse(q8, L, B, topk=65) == -1
    assert call_sparse(q8, L, B, nq=24) == -2
    assert call_sparse(q8, L, B, q=FAKE + 4) == -1
    assert call_sparse(q8, L, B, sel=FAKE + 2) == -1
    assert call_sparse(q8, L, B, ws=0) == -3
    need = q8.decode_attn_sparse_workspace_bytes(L, B, 16, 32)
    # one fp32 score per (sequence, query head, 32-token block)
    assert need >= 4 * 16 * ((300 + 31) // 32) * 4
    assert call_sparse(q8, L, B, ws_bytes=need - 1) == -3
    assert q8.decode_attn_sparse_workspace_bytes(L, B, 16, 1) == 0


def call_prefill(q8, L, B, nq=16, q_start=FAKE, total_q=64, max_new=32, q=FAKE, out=FAKE):
    return q8.lib().q8_prefill_attn(ctypes.byref(L.c()), ctypes.byref(B.c()), nq, q_start, total_q, max_new, q,
                                    0.088, out, None, None)


def test_prefill_validation(q8):
    L, B = layer(q8), batch(q8)
    assert call_prefill(q8, L, B, nq=24) == -2
    assert call_prefill(q8, L, B, nq=0) == -1
    assert call_prefill(q8, L, B, q_start=0) == -1
    assert call_prefill(q8, L, B, q_start=FAKE + 2) == -1
    assert call_prefill(q8, L, B, total_q=-1) == -1
    assert call_prefill(q8, L, B, max_new=-1) == -1
    assert call_prefill(q8, L, B, max_new=301) == -1     # above max_seq_len
    assert call_prefill(q8, L, B, q=FAKE + 8) == -1
    assert call_prefill(q8, L, B, out=0) == -1
    assert call_prefill(q8, L, B, total_q=0) == 0        # nothing to do, nothing enqueued
    assert call_prefill(q8, L, B, max_new=0) == 0
    assert call_prefill(q8, layer(q8, kv_bs=24), B) == -2


def call_step(q8, L, B, nq=16, k_new=FAKE, v_new=FAKE, q=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 30, status=None):
    return q8.lib().q8_decode_step(ctypes.byref(L.c()), ctypes.byref(B.c()), nq, k_new, v_new, q, 0.088, out, 0,
                                   ws, ws_bytes, status, None)


def test_decode_step_validation(q8):
    L, B = layer(q8), batch(q8)
    assert call_step(q8, L, B, nq=24) == -2
    assert call_step(q8, L, B, k_new=0) == -1
    assert call_step(q8, L, B, v_new=0) == -1
    assert call_step(q8, L, B, k_new=FAKE + 4) == -1
    assert call_step(q8, L, B, v_new=FAKE + 2) == -1
    assert call_step(q8, L, B, q=FAKE + 4) == -1
    assert call_step(q8, L, B, status=FAKE + 2) == -1
    assert call_step(q8, L, B, ws=0) == -3
    assert call_step(q8, L, B, ws_bytes=q8.decode_attn_workspace_bytes(L, B, 16, 0) - 1) == -3


# ------------------------------------------------- Python binding argument checks
def _cpu_layer(q8, **over):
    import torch
    nb, bs, nkv = 4, 32, 2
    d = dict(k_codes=torch.zeros((nb, bs, nkv * 128), dtype=torch.int8),
             v_codes=torch.zeros((nb, bs, nkv * 128), dtype=torch.int8),
             k_scale=torch.zeros((nb, nkv, bs)), v_scale=torch.zeros((nb, nkv, bs)),
             nkv_heads=nkv, kv_bs=bs, num_blocks=nb)
    d.update(over)
    return q8.KVLayer(**d)


def test_binding_rejects_wrong_tensors_before_any_call(q8):
    # The checks run before the library is called; CPU tensors reach the
    # dtype, contiguity and size checks (the device check comes last).
    import torch
    with pytest.raises(ValueError, match="dtype"):
        q8.make_batch(torch.zeros((2, 3), dtype=torch.int64), torch.zeros(2, dtype=torch.int32), 10)
    with pytest.raises(ValueError, match="dtype"):
        q8.make_batch(torch.zeros((2, 3), dtype=torch.int32), torch.zeros(2, dtype=torch.int64), 10)
    with pytest.raises(ValueError, match="contiguous"):
        q8.make_batch(torch.zeros((3, 2), dtype=torch.int32).t(), torch.zeros(2, dtype=torch.int32), 10)
    with pytest.raises(ValueError, match="elements"):
        q8.make_batch(torch.zeros((2, 3), dtype=torch.int32), torch.zeros(3, dtype=torch.int32), 10)
    with pytest.raises(ValueError, match="GPU"):
        q8.make_batch(torch.zeros((2, 3), dtype=torch.int32), torch.zeros(2, dtype=torch.int32), 10)
    # layer tensors: wrong dtype, wrong size
    B = q8.Batch(torch.zeros((2, 3), dtype=torch.int32), torch.zeros(2, dtype=torch.int32), 2, 3, 10)
    q = torch.zeros((2, 4, 128))
    out = torch.zeros((2, 4, 128))
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="layer.k_codes: dtype"):
        q8.decode_attn(_cpu_layer(q8, k_codes=torch.zeros((4, 32, 256))), B, 4, q, 0.1, out, ws)
    with pytest.raises(ValueError, match="layer.v_scale: .*elements"):
        q8.decode_attn(_cpu_layer(q8, v_scale=torch.zeros((4, 2, 16))), B, 4, q, 0.1, out, ws)
    with pytest.raises(ValueError, match="torch tensor"):
        q8.decode_attn(_cpu_layer(q8, k_codes=FAKE), B, 4, q, 0.1, out, ws)
    # q / out: half precision, strided, too small
    L = _cpu_layer(q8)
    with pytest.raises(ValueError, match="GPU"):
        q8.decode_attn(L, B, 4, q, 0.1, out, ws)      # everything right but on the CPU
    with pytest.raises(ValueError, match="q: dtype"):
        q8.decode_attn(L, B, 4, q.half(), 0.1, out, ws)
    with pytest.raises(ValueError, match="out: must be contiguous"):
        q8.decode_attn(L, B, 4, q, 0.1, torch.zeros((2, 128, 4)).transpose(1, 2), ws)
    with pytest.raises(ValueError, match="out: .*elements"):
        q8.decode_attn(L, B, 4, q, 0.1, out[:1], ws)
    with pytest.raises(ValueError, match="dev_status: dtype"):
        q8.decode_attn(L, B, 4, q, 0.1, out, ws, dev_status=torch.zeros(1, dtype=torch.int64))
    # append: int64 token indices, short K rows
    seq = torch.zeros(3, dtype=torch.int32)
    kn = torch.zeros((3, 2, 128))
    with pytest.raises(ValueError, match="tok_pos: dtype"):
        q8.kv_append(L, B, seq, seq.long(), kn, kn)
    with pytest.raises(ValueError, match="v_new: .*elements"):
        q8.kv_append(L, B, seq, seq, kn, kn[:2])
    # decode step: short new rows; sparse: short selection; prefill: q_start size
    with pytest.raises(ValueError, match="k_new: .*elements"):
        q8.decode_step(L, B, 4, kn[:1], kn, q, 0.1, out, ws)
    with pytest.raises(ValueError, match="selected: .*elements"):
        q8.decode_attn_sparse(L, B, 4, q, 0.1, out, ws, topk=8, selected=torch.zeros(8, dtype=torch.int32))
    with pytest.raises(ValueError, match="q_start: .*elements"):
        q8.prefill_attn(L, B, 4, torch.zeros(2, dtype=torch.int32), 1, q, 0.1, out)
    with pytest.raises(ValueError, match="partials: .*elements"):
        q8.qk_block_partials(L, B, 4, q, torch.zeros(10, dtype=torch.int32))


def test_batch_flags_and_the_invariant_cut(q8):
    L = layer(q8)
    lib = q8.lib()
    # unknown flag bits are refused; the invariant flag is accepted
    bad = batch(q8)
    c = bad.c()
    c.flags = 0x2
    assert lib.q8_decode_attn(ctypes.byref(L.c()), ctypes.byref(c), 16, FAKE, 0.088, FAKE, 4, FAKE, 1 << 30,
                              None, None) == -1
    inv = batch(q8, invariant=True)
    assert inv.c().flags == q8.BATCH_INVARIANT
    # an invariant batch carries no step plan and cannot be planned
    assert call_decode(q8, L, batch(q8, invariant=True, plan=FAKE)) == -1
    assert lib.q8_decode_plan_bytes(ctypes.byref(L.c()), ctypes.byref(inv.c()), 16, 0) == 0
    assert lib.q8_decode_plan(ctypes.byref(L.c()), ctypes.byref(inv.c()), 16, 0, FAKE, 1 << 20, None, None) == -1
    # one record per chunk per sequence and query head, for any partition count
    for nparts in (0, 1, 4, 1000):
        need = q8.decode_attn_workspace_bytes(L, inv, 16, nparts)
        chunks = 4 * ((300 + 127) // 128)
        assert need >= chunks * 16 * (128 + 2) * 4
        assert call_decode(q8, L, inv, ws_bytes=need - 1, nparts=nparts) == -3


def _invariant_chunks(n):
    # the header's rule: chunks of 128 positions, 256 from 4096 positions on,
    # 512 from 16384 on (the last chunk shorter)
    tiles = (n + 31) // 32
    length = 512 if n >= 16384 else 256 if n >= 4096 else 128
    return (tiles * 32 + length - 1) // length if tiles else 0


@pytest.mark.parametrize("max_seq_len", [1, 127, 128, 4064, 4095, 4096, 4097, 8191, 16352, 16383, 16384,
                                         40000, 1 << 20])
def test_invariant_workspace_holds_the_most_chunks_a_length_has(q8, max_seq_len):
    # the workspace's record count is the largest chunk count of any length up
    # to max_seq_len (at the top of a band of the rule, just below a doubling
    # of the chunk length, a shorter sequence can have more chunks)
    most = max(_invariant_chunks(n) for n in range(0, max_seq_len + 1, 1 if max_seq_len < 70000 else 32))
    if max_seq_len >= 70000:
        most = max(most, _invariant_chunks(max_seq_len))
    inv = batch(q8, invariant=True, max_seq_len=max_seq_len, max_blocks_per_seq=(max_seq_len + 31) // 32)
    need = q8.decode_attn_workspace_bytes(layer(q8), inv, 16, 0)
    payload = 4 * max(most, 1) * 16 * (128 + 2) * 4
    assert payload <= need <= payload + 2 * 256 + 4 * 5
