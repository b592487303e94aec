"""The C ABI on the CPU: the library loads, exports every symbol include/gale.h declares,
the host packer round-trips, and argument validation rejects bad calls before any
GPU work (no compute call reaches the GPU here)."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import quantized_expert_gemv_amd as q
from quantized_expert_gemv_amd import binding as B
from synth import gen_matrix, config_seed

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    txt = open(os.path.join(ROOT, "include", "gale.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(gale_[a-z0-9_]+)\s*\(", txt)))


def test_exports_every_declared_symbol():
    L = q.lib()
    names = header_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(q.exported_symbols())


def test_status_strings():
    L = q.lib()
    for code in range(0, -10, -1):
        assert L.gale_status_str(code).decode() != "unknown status"


def test_packed_sizes_closed_form():
    s = q.packed_sizes(2048, 4096, 2048 * 41)
    assert s["format_bytes"] == 1_393_664
    s2 = q.packed_sizes(4096, 2048, 4096 * 20)
    assert s2["format_bytes"] == 1_392_640
    with pytest.raises(q.GaleError):
        q.packed_sizes(2048, 4000, 0)


@pytest.mark.parametrize("rows,cols", [(16, 1024), (48, 2048), (64, 4096)])
def test_host_pack_roundtrip(rows, cols):
    m = gen_matrix(config_seed(7), (rows, cols), rows, cols)
    ds, dsc = q.pack_host(rows, cols, m.signs, m.block_scales)
    assert not torch.equal(ds, m.signs)                 # the layout really permutes
    cs, csc = q.unpack_host(rows, cols, ds, dsc)
    assert torch.equal(cs, m.signs) and torch.equal(csc, m.block_scales)


def _fp4_operand_column(g, j, i):
    # column inside a 128-column block of nibble i of dword j held by lane group g of a
    # 16x16x128 fp4 MFMA B operand (measured on gfx950 with one-hot operands)
    return 64 * (g & 1) + 16 * (g >> 1) + 32 * (j >> 1) + 8 * (j & 1) + i


def test_fp4_operand_order_is_a_bijection():
    cols = sorted(_fp4_operand_column(g, j, i) for g in range(4) for j in range(4) for i in range(8))
    assert cols == list(range(128))


def test_host_pack_plane_structure():
    # bit (4 i + d % 4) of word 4 (d // 4) + j of lane 16 g + n % 16 is column
    # 128 d + kh(g, j, i) of row n: a single canonical bit must land exactly there
    rows, cols = 16, 1024
    expect = {}
    for g in range(4):
        for j in range(4):
            for i in range(8):
                expect[_fp4_operand_column(g, j, i)] = (g, j, i)
    for (n, k) in [(0, 0), (5, 130), (15, 1023), (3, 4 * 9 + 2 + 128 * 6), (9, 128 * 3 + 77)]:
        s = torch.zeros(rows, cols // 32, dtype=torch.int32)
        s[n, k // 32] = np.int32(np.uint32(1 << (k % 32)).view(np.int32))
        ds, _ = q.pack_host(rows, cols, s, torch.zeros(rows, cols // 128, dtype=torch.int16))
        nz = torch.nonzero(ds.view(-1)).flatten()
        assert nz.numel() == 1
        w = int(nz[0])
        word = int(ds.view(-1)[w].item()) & 0xFFFFFFFF
        d = (k % 1024) // 128
        g, j, i = expect[k % 128]
        lane = 16 * g + n % 16
        assert w == ((0 * 2 + d // 4) * 64 + lane) * 4 + j
        assert word == 1 << (4 * i + d % 4)


def test_check_canonical_rejects_bad_csr():
    rp = np.array([0, 2, 3] + [3] * 14, dtype=np.int32)
    good = np.array([1, 5, 7], dtype=np.uint16)
    q.check_canonical(16, 1024, rp, good)
    for bad in (np.array([5, 1, 7], dtype=np.uint16), np.array([1, 1, 7], dtype=np.uint16),
                np.array([1, 5, 1024], dtype=np.uint16)):
        with pytest.raises(q.GaleError) as e:
            q.check_canonical(16, 1024, rp, bad)
        assert e.value.status == -7
    with pytest.raises(q.GaleError):
        q.check_canonical(16, 1024, np.array([0, 2, 1] + [3] * 14, dtype=np.int32), good)


def _call(name, *args):
    return getattr(q.lib(), name)(*args)


def test_validation_before_any_gpu_work():
    # invalid arguments return their specific code without enqueueing (no GPU needed)
    F = 0x1000  # a fake non-null, 256-aligned pointer value; never dereferenced on these paths
    assert _call("gale_expert_gemv", 2048, 4000, F, 1, F, 1, 0, 1, F, 1, F, 1 << 30, 0, None) == -2
    assert _call("gale_expert_gemv", 2040, 4096, F, 1, F, 1, 0, 1, F, 1, F, 1 << 30, 0, None) == -2
    assert _call("gale_expert_gemv", 2048, 4096, None, 1, F, 1, 0, 1, F, 1, F, 1 << 30, 0, None) == -1
    assert _call("gale_expert_gemv", 2048, 4096, F, 1, F, 7, 0, 1, F, 1, F, 1 << 30, 0, None) == -3
    assert _call("gale_expert_gemv", 2048, 4096, F, 1, F + 2, 1, 0, 1, F, 1, F, 1 << 30, 0, None) == -4
    assert _call("gale_expert_gemv", 2048, 4096, F, 1, F, 1, 0, 1, F, 1, F, 16, 0, None) == -5
    assert _call("gale_expert_gemv", 2048, 4096, F, 0, F, 1, 0, 1, F, 1, F, 1 << 30, 0, None) == -2
    assert _call("gale_fwht1024", F, F, 1, 1000, 1, 1, None) == -2
    assert _call("gale_fwht1024", F, F, 1, 1024, 1, 2, None) == -3        # in place needs equal dtypes
    assert _call("gale_expert_ffn", 4096, 2048, F, 1, F, 0, 1, F, F, 16, None) == -5
    assert _call("gale_moe_layer_fwd", 4096, 2048, F, 256, F, 9, F, 1, F, None, None, F, 1 << 30, 0, None) == -2
    assert _call("gale_moe_layer_fwd", 4096, 2048, F, 600, F, 6, F, 1, F, None, None, F, 1 << 30, 0, None) == -2
    assert _call("gale_moe_layer_fwd", 4096, 2048, F, 256, F, 6, F, 65, F, None, None, F, 1 << 30,
                 B.GALE_PATH_DECODE, None) == -2
    assert _call("gale_moe_layer_fwd", 4096, 2048, F, 256, F, 6, F, 1, F, None, None, F, 16, 0, None) == -5
    # hidden above GALE_MAX_HIDDEN (the w1/w3 workgroup would exceed 1024 threads)
    assert _call("gale_expert_ffn", 9216, 2048, F, 1, F, 0, 1, F, F, 1 << 30, None) == -2
    assert _call("gale_moe_layer_fwd", 9216, 2048, F, 256, F, 6, F, 1, F, None, None, F, 1 << 30, 0, None) == -2
    assert "above" in q.lib().gale_last_error().decode()
    # routing variants: a selection bias and fixed experts exclude each other; alignment
    assert _call("gale_moe_layer_fwd_routed", 4096, 2048, F, 256, F, F, F, 6, F, 1, F, None, None, F, 1 << 30, 0,
                 None) == -2
    assert _call("gale_moe_layer_fwd_routed", 4096, 2048, F, 256, F, F + 2, None, 6, F, 1, F, None, None, F,
                 1 << 30, 0, None) == -4
    assert _call("gale_moe_layer_fwd_routed", 4096, 2048, F, 256, F, None, F + 1, 6, F, 1, F, None, None, F,
                 1 << 30, 0, None) == -4
    assert _call("gale_route_topk", F, 4, 256, 9, F, F, None, None, None, 0, None) == -2
    assert _call("gale_route_topk", F, 4, 256, 6, F, F, F, None, None, 0, None) == -1
    assert _call("gale_route_topk", F, 100, 256, 6, F, F, F, F, None, 0, None) == -5
    assert "workspace" in q.lib().gale_last_error().decode()


def test_workspace_sizes_monotone():
    a = q.gemv_workspace_bytes(2048, 4096, 1, 1, 0)
    b = q.gemv_workspace_bytes(2048, 4096, 8, 1, 0)
    c = q.gemv_workspace_bytes(2048, 4096, 8, 1, 1)
    assert b > a and c == a and a % 256 == 0
    assert q.moe_workspace_bytes(32, 256, 6, 4096, 2048) > q.moe_workspace_bytes(1, 256, 6, 4096, 2048)


def test_descriptor_refuses_null_sections():
    # an empty torch slice has a NULL data pointer; the kernels read every outlier
    # section in whole 16-byte chunks, so a descriptor must never carry one
    z = torch.zeros(16, dtype=torch.uint8)
    ok = q.PackedMatrix(16, 1024, torch.zeros(512, dtype=torch.int32), torch.zeros(128, dtype=torch.int16),
                        torch.zeros(16, dtype=torch.int16), torch.zeros(17, dtype=torch.int32),
                        z.view(torch.int16), z, nnz=0)
    d = ok.descriptor()
    assert d.out_cols and d.out_vals
    bad = q.PackedMatrix(16, 1024, torch.zeros(512, dtype=torch.int32), torch.zeros(128, dtype=torch.int16),
                         torch.zeros(16, dtype=torch.int16), torch.zeros(17, dtype=torch.int32),
                         z.view(torch.int16)[:0], z[:0])
    with pytest.raises(ValueError):
        bad.descriptor()
    assert B._padded16(torch.zeros(0, dtype=torch.int16)).numel() == 16
    assert B._padded16(torch.zeros(9, dtype=torch.int16)).numel() == 32


def test_decode_stack_validation_before_gpu_work():
    """gale_moe_decode_stack rejects bad requests on the host, before anything is enqueued."""
    L = q.lib()
    ws_bytes = q.decode_stack_workspace_bytes(4096, 2048, 6)
    assert ws_bytes >= q.GALE_SYNC_BYTES + 4 * 2048 * 6
    assert q.decode_stack_workspace_bytes(4096, 2048, 9) == 0
    fake = 1 << 40                      # never dereferenced: every call below fails validation
    assert L.gale_moe_decode_stack(4096, 2048, 256, 6, 0, fake, fake, ws_bytes, 0, None) == -2      # no layers
    assert L.gale_moe_decode_stack(4096, 2048, 256, 6, 2, None, fake, ws_bytes, 0, None) == -1      # NULL table
    assert L.gale_moe_decode_stack(4096, 2048, 256, 6, 2, fake, fake, ws_bytes - 1, 0, None) == -5  # workspace
    assert L.gale_moe_decode_stack(4096, 2048, 256, 6, 2, fake, fake + 8, ws_bytes, 0, None) == -4  # alignment
    assert L.gale_moe_decode_stack(8192, 2048, 256, 6, 2, fake, fake, 1 << 30, 0, None) == -6       # shape
    assert L.gale_moe_decode_stack(4096, 2048, 256, 9, 2, fake, fake, 1 << 30, 0, None) == -2      # top_k
    assert L.gale_sync_init(None, None) == -1
    assert L.gale_sync_init(fake + 8, None) == -4


def test_read_stream_validation_before_gpu_work():
    """The streaming-read diagnostic refuses bad arguments on the host."""
    L = q.lib()
    fake = 1 << 40                      # never dereferenced: every call below fails validation
    assert L.gale_read_stream(None, 1024, fake, 4, None) == -1
    assert L.gale_read_stream(fake, 1024, None, 4, None) == -1
    assert L.gale_read_stream(fake, 1000, fake, 4, None) == -2      # not a multiple of 16
    assert L.gale_read_stream(fake, 0, fake, 4, None) == -2
    assert L.gale_read_stream(fake, 1024, fake, 0, None) == -2
    assert L.gale_read_stream(fake + 8, 1024, fake, 4, None) == -4  # alignment


def test_empty_inputs_refused_before_gpu_work():
    """No tokens, matrices or experts: refused on the host with GALE_ERR_SHAPE."""
    L = q.lib()
    fake = 1 << 40                      # never dereferenced: every call below fails validation
    # gale_expert_gemv(rows, cols, table, n_mat, x, x_dtype, x_shared, n_tok, y, y_dtype, ws, ws_bytes, flags, stream)
    assert L.gale_expert_gemv(2048, 4096, fake, 0, fake, 0, 0, 1, fake, 0, fake, 1 << 30, 0, None) == -2
    assert L.gale_expert_gemv(2048, 4096, fake, 1, fake, 0, 0, 0, fake, 0, fake, 1 << 30, 0, None) == -2
    # gale_expert_ffn(hidden, inter, table, n_exp, x, x_shared, n_tok, y, ws, ws_bytes, stream)
    assert L.gale_expert_ffn(4096, 2048, fake, 0, fake, 0, 1, fake, fake, 1 << 30, None) == -2
    assert L.gale_expert_ffn(4096, 2048, fake, 1, fake, 0, 0, fake, fake, 1 << 30, None) == -2
    # gale_moe_layer_fwd(hidden, inter, table, n_experts, logits, top_k, x, n_tok, y, idx, w, ws, ws_bytes, flags, stream)
    assert L.gale_moe_layer_fwd(4096, 2048, fake, 256, fake, 6, fake, 0, fake, None, None, fake, 1 << 30, 0, None) == -2
    assert L.gale_moe_layer_fwd(4096, 2048, fake, 0, fake, 6, fake, 1, fake, None, None, fake, 1 << 30, 0, None) == -2
