"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before touching a device.

Every call below passes an explicit partition count, so no device query runs, and
each one fails a host check; nothing is ever enqueued.
"""
import ctypes
import math
import os
import subprocess

import pytest

import mla_latent_kv_16_amd as mla
from mla_latent_kv_16_amd import _binding as bnd

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
FAKE = 0x10000  # 16-byte aligned host address; never dereferenced by the host checks


def test_library_exports_every_header_function():
    names = mla.header_functions()
    assert names == sorted([
        "mla_absorb_q", "mla_project_o",
        "mla_decode", "mla_decode_auto_partitions", "mla_decode_combine", "mla_decode_e4m3",
        "mla_decode_nope", "mla_decode_noalloc", "mla_decode_splitkv_nope",
        "mla_decode_single_pass", "mla_decode_single_pass_e4m3", "mla_decode_splitkv",
        "mla_decode_splitkv_e4m3", "mla_decode_splitkv_placement",
        "mla_decode_splitkv_timeline", "mla_decode_tree",
        "mla_decode_tree_e4m3",
        "mla_decode_varlen", "mla_decode_workspace_bytes", "mla_decode_workspace_size",
        "mla_kv_append", "mla_kv_append_e4m3", "mla_prefill_with_prefix",
        "mla_prefill_workspace_bytes", "mla_read_error_flags", "mla_status_string"])
    L = mla.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", mla.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(names) <= exported


def test_peaks_library_exports_its_header():
    """libmla_peaks.so (measurement support) exports every function mla_peaks.h declares
    and rejects bad arguments on the host (nothing is launched)."""
    from mla_latent_kv_16_amd import peaks
    hdr = os.path.join(os.path.dirname(mla.LIB_PATH), "..", "include", "mla_peaks.h")
    names = bnd.header_functions(hdr)
    assert names == sorted(["mla_peak_stream_read", "mla_peak_dma_stream",
                            "mla_peak_dma_stream_bytes", "mla_peak_mfma_bf16",
                            "mla_peak_mfma_bf16_flops"])
    out = subprocess.run(["nm", "-D", "--defined-only", peaks.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(names) <= exported
    L = peaks.lib()
    assert L.mla_peak_stream_read(None, 1 << 20, FAKE, 8, None) == -1
    assert L.mla_peak_stream_read(FAKE + 4, 1 << 20, FAKE, 8, None) == -1
    assert L.mla_peak_dma_stream(FAKE, 1000, FAKE, 8, None) == -1  # under one block each
    assert L.mla_peak_mfma_bf16(0, FAKE, 8, None) == -1
    assert L.mla_peak_dma_stream_bytes(36864 * 10 + 5, 3) == 36864 * 9
    assert L.mla_peak_mfma_bf16_flops(10, 2) == 2 * 4 * 10 * 4 * 32768


@pytest.mark.parametrize("header", ["mla.h", "mla_peaks.h"])
def test_header_compiles_as_c(header):
    hdr = os.path.join(os.path.dirname(mla.LIB_PATH), "..", "include", header)
    src = f'#include "{os.path.abspath(hdr)}"\nint main(void) {{ return 0; }}\n'
    res = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-x", "c", "-", "-o", "/dev/null"],
                         input=src, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_status_strings():
    for s in (OK, INVALID, UNSUPPORTED, WORKSPACE, -4, -5):
        assert mla.status_string(s)
    assert "DEVICE_CHECK" in mla.status_string(-5)
    assert "unknown" in mla.status_string(12345)


@pytest.mark.parametrize("fn", ["mla_decode_workspace_bytes", "mla_prefill_workspace_bytes"])
@pytest.mark.parametrize("args", [(0, 4, 16, 10), (2, 0, 16, 10), (2, 4, 0, 10), (2, 4, 16, 0),
                                  (1025, 1, 16, 4), (1, 1 << 20, 32, 4)])
def test_workspace_bytes_is_zero_for_rejected_sizes(fn, args):
    """Sizes the compute calls would reject give 0 (checked before any device query)."""
    assert getattr(mla.lib(), fn)(*args) == 0


@pytest.mark.parametrize("shape", [(4, 4, 16, 1025), (1, 4096, 16, 1088), (64, 1, 128, 512),
                                   (1, 1, 16, 4)])
def test_workspace_bytes_matches_workspace_size_for_the_automatic_count(shape):
    """Both plain-value sizes equal mla_decode_workspace_size with num_partitions = 0;
    where no device can be queried (a host without a GPU) all three report failure."""
    out = ctypes.c_size_t(0)
    st = mla.lib().mla_decode_workspace_size(*shape, 0, ctypes.byref(out))
    dec = mla.lib().mla_decode_workspace_bytes(*shape)
    pre = mla.lib().mla_prefill_workspace_bytes(*shape)
    if st == OK:
        assert dec == pre == out.value > 0
    else:
        assert st == -4 and dec == pre == 0


def _counters(B, n_mt):
    """Single-pass arrival + merged-row counters: 2 B n_mt words, in 256-byte units."""
    return ((2 * B * n_mt * 4 + 255) // 256) * 256


def test_workspace_size_explicit_partitions():
    # one partition: header only; split: header, counters, then (B + G) slots of
    # min(M, 64) rows x (512 + 1) floats
    assert mla.workspace_size(4, 4, 16, 1025, 1) == 256
    n = mla.workspace_size(4, 4, 16, 1025, 256)
    slots, rows = (4 + 256) * 1, 64
    assert n == 256 + _counters(4, 1) + slots * rows * 512 * 4 + \
        (((slots * rows * 4) + 255) // 256) * 256
    # M = 256 rows -> 4 M-tiles of 64 rows
    n2 = mla.workspace_size(16, 16, 16, 3200, 64)
    slots2 = (16 + 64) * 4
    assert n2 == 256 + _counters(16, 4) + slots2 * 64 * 512 * 4 + \
        (((slots2 * 64 * 4) + 255) // 256) * 256
    # M smaller than a tile: slots hold only M rows
    n3 = mla.workspace_size(1, 1, 5, 4, 3)
    assert n3 == 256 + _counters(1, 1) + 4 * 5 * 512 * 4 + 256
    # many M-tiles: the counters span several 256-byte units
    n4 = mla.workspace_size(64, 4, 128, 100, 2)
    slots4 = (64 + 2) * 8
    assert _counters(64, 8) == 4096
    assert n4 == 256 + 4096 + slots4 * 64 * 512 * 4 + (((slots4 * 64 * 4) + 255) // 256) * 256


@pytest.mark.parametrize("args,code", [
    (dict(B=0), INVALID), (dict(Sq=0), INVALID), (dict(H=0), INVALID),
    (dict(max_pages=0), INVALID), (dict(B=1025), UNSUPPORTED), (dict(parts=-1), INVALID),
])
def test_workspace_size_rejects(args, code):
    a = dict(B=2, Sq=2, H=2, max_pages=4, parts=3)
    a.update(args)
    out = ctypes.c_size_t(0)
    st = mla.lib().mla_decode_workspace_size(a["B"], a["Sq"], a["H"], a["max_pages"], a["parts"],
                                             ctypes.byref(out))
    assert st == code


def _call(name="mla_decode", **over):
    a = dict(q_nope=FAKE, q_rope=FAKE, kv_pool=FAKE, num_pages=8, page_size=64,
             block_table=FAKE, max_pages=4, seq_lens=FAKE, B=1, Sq=1, H=16, scale=0.07,
             causal=1, parts=2, O=FAKE, lse=FAKE, ws=FAKE, ws_bytes=1 << 30, stream=None,
             kv_scale=0.015625)
    a.update(over)
    fn = getattr(mla.lib(), name)
    # the E4M3 entry points take the pool's scale right after the pool
    pool = ((a["kv_pool"], a["kv_scale"]) if name.endswith("_e4m3") else (a["kv_pool"],))
    return fn(a["q_nope"], a["q_rope"], *pool, a["num_pages"], a["page_size"],
              a["block_table"], a["max_pages"], a["seq_lens"], a["B"], a["Sq"], a["H"],
              a["scale"], a["causal"], a["parts"], a["O"], a["lse"], a["ws"], a["ws_bytes"],
              a["stream"])


COMPUTE_ENTRY_POINTS = ["mla_decode", "mla_decode_splitkv", "mla_prefill_with_prefix",
                        "mla_decode_single_pass", "mla_decode_e4m3", "mla_decode_splitkv_e4m3",
                        "mla_decode_single_pass_e4m3"]


@pytest.mark.parametrize("name", COMPUTE_ENTRY_POINTS)
@pytest.mark.parametrize("over,code", [
    (dict(q_nope=None), INVALID), (dict(q_rope=None), INVALID), (dict(kv_pool=None), INVALID),
    (dict(block_table=None), INVALID), (dict(seq_lens=None), INVALID), (dict(O=None), INVALID),
    (dict(lse=None), INVALID), (dict(q_nope=FAKE + 8), INVALID), (dict(kv_pool=FAKE + 2), INVALID),
    (dict(O=FAKE + 4), INVALID), (dict(seq_lens=FAKE + 2), INVALID),
    (dict(page_size=32), UNSUPPORTED), (dict(page_size=128), UNSUPPORTED),
    (dict(num_pages=0), INVALID), (dict(scale=math.nan), INVALID), (dict(scale=math.inf), INVALID),
    (dict(causal=2), INVALID), (dict(B=0), INVALID), (dict(Sq=0), INVALID), (dict(H=-1), INVALID),
    (dict(max_pages=0), INVALID), (dict(B=4096), UNSUPPORTED), (dict(parts=-3), INVALID),
    (dict(ws=None), WORKSPACE), (dict(ws=FAKE + 4), WORKSPACE), (dict(ws_bytes=100), WORKSPACE),
    (dict(ws_bytes=255, parts=1), WORKSPACE),
])
def test_compute_entry_points_reject_on_host(name, over, code):
    assert _call(name, **over) == code


@pytest.mark.parametrize("name", ["mla_decode_e4m3", "mla_decode_splitkv_e4m3",
                                  "mla_decode_single_pass_e4m3"])
@pytest.mark.parametrize("kv_scale", [0.0, -1.0, math.nan, math.inf, -math.inf])
def test_e4m3_entry_points_reject_bad_scale(name, kv_scale):
    assert _call(name, kv_scale=kv_scale) == INVALID


def _tree_call(name="mla_decode_tree", **over):
    a = dict(q_nope=FAKE, q_rope=FAKE, kv_pool=FAKE, num_pages=8, page_size=64,
             block_table=FAKE, max_pages=4, seq_lens=FAKE, tree=FAKE, B=1, Sq=4, H=16,
             scale=0.07, parts=2, O=FAKE, lse=FAKE, ws=FAKE, ws_bytes=1 << 30, stream=None,
             kv_scale=0.015625)
    a.update(over)
    pool = ((a["kv_pool"], a["kv_scale"]) if name.endswith("_e4m3") else (a["kv_pool"],))
    return getattr(mla.lib(), name)(
        a["q_nope"], a["q_rope"], *pool, a["num_pages"], a["page_size"], a["block_table"],
        a["max_pages"], a["seq_lens"], a["tree"], a["B"], a["Sq"], a["H"], a["scale"], a["parts"],
        a["O"], a["lse"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("name", ["mla_decode_tree", "mla_decode_tree_e4m3"])
@pytest.mark.parametrize("over,code", [
    (dict(tree=None), INVALID), (dict(tree=FAKE + 4), INVALID), (dict(Sq=65), UNSUPPORTED),
    (dict(Sq=0), INVALID), (dict(q_nope=None), INVALID), (dict(page_size=32), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(scale=math.nan), INVALID),
])
def test_tree_entry_points_reject_on_host(name, over, code):
    assert _tree_call(name, **over) == code


def test_varlen_rejects_on_host():
    L = mla.lib()
    args = [FAKE, FAKE, FAKE, 8, 64, FAKE, 4, FAKE]
    rest = [1, 4, 16, 0.07, 2, FAKE, FAKE, FAKE, 1 << 30, None]
    assert L.mla_decode_varlen(*args, None, *rest) == INVALID
    assert L.mla_decode_varlen(*args, FAKE + 2, *rest) == INVALID
    assert L.mla_decode_varlen(*args, FAKE, 1, 4, 16, 0.07, 2, FAKE, FAKE, None, 1 << 30,
                               None) == WORKSPACE


@pytest.mark.parametrize("over,code", [
    (dict(new=None), INVALID), (dict(pool=None), INVALID), (dict(new=FAKE + 8), INVALID),
    (dict(pool=FAKE + 2), INVALID), (dict(bt=FAKE + 2), INVALID), (dict(page=32), UNSUPPORTED),
    (dict(B=0), INVALID), (dict(Sq=0), INVALID), (dict(ws=None), WORKSPACE),
    (dict(ws_bytes=128), WORKSPACE), (dict(scale=0.0), INVALID), (dict(scale=math.inf), INVALID),
])
def test_kv_append_rejects_on_host(over, code):
    a = dict(new=FAKE, pool=FAKE, bt=FAKE, sl=FAKE, page=64, B=2, Sq=4, ws=FAKE, ws_bytes=256,
             scale=0.015625)
    a.update(over)
    L = mla.lib()
    common = (a["page"], a["bt"], 8, a["sl"], a["B"], a["Sq"], a["ws"], a["ws_bytes"], None)
    if "scale" not in over:
        assert L.mla_kv_append(a["new"], a["pool"], 16, *common) == code
    assert L.mla_kv_append_e4m3(a["new"], a["pool"], a["scale"], 16, *common) == code


@pytest.mark.parametrize("name", ["mla_absorb_q", "mla_project_o"])
@pytest.mark.parametrize("args,code", [
    ((None, FAKE, FAKE, 1, 1, 1), INVALID), ((FAKE, None, FAKE, 1, 1, 1), INVALID),
    ((FAKE, FAKE, None, 1, 1, 1), INVALID), ((FAKE + 8, FAKE, FAKE, 1, 1, 1), INVALID),
    ((FAKE, FAKE, FAKE, 0, 1, 1), INVALID), ((FAKE, FAKE, FAKE, 1, 0, 1), INVALID),
    ((FAKE, FAKE, FAKE, 1, 1, 0), INVALID), ((FAKE, FAKE, FAKE, 1, 1, 70000), UNSUPPORTED),
])
def test_gemms_reject_on_host(name, args, code):
    assert getattr(mla.lib(), name)(*args, None) == code


def test_tree_e4m3_rejects_bad_scale():
    assert _tree_call("mla_decode_tree_e4m3", kv_scale=0.0) == INVALID


def test_workspace_one_byte_short_is_rejected():
    # (a call that passes every host check would enqueue kernels on these fake
    # pointers, so none is made here)
    need = mla.workspace_size(1, 1, 16, 4, 2)
    assert _call(ws_bytes=need - 1) == WORKSPACE


def test_combine_rejects_on_host():
    L = mla.lib()
    f = L.mla_decode_combine
    assert f(None, 4, 1, 1, 16, 2, FAKE, FAKE, FAKE, 1 << 20, None) == INVALID
    assert f(FAKE, 4, 1, 1, 16, 2, None, FAKE, FAKE, 1 << 20, None) == INVALID
    assert f(FAKE, 4, 1, 1, 16, 2, FAKE + 4, FAKE, FAKE, 1 << 20, None) == INVALID
    assert f(FAKE, 4, 0, 1, 16, 2, FAKE, FAKE, FAKE, 1 << 20, None) == INVALID
    assert f(FAKE, 4, 1, 1, 16, 2, FAKE, FAKE, None, 1 << 20, None) == WORKSPACE
    assert f(FAKE, 4, 1, 1, 16, 2, FAKE, FAKE, FAKE, 10, None) == WORKSPACE


def test_placement_record_rejects_on_host():
    """The placement record needs 3 int32 per split-KV workgroup (G x M-tiles), and an
    aligned, non-null buffer; any shortfall is refused before anything is enqueued."""
    f = mla.lib().mla_decode_splitkv_placement

    def call(trace, n, B=4, Sq=16, H=16, parts=8):
        return f(FAKE, FAKE, FAKE, 64, 64, FAKE, 16, FAKE, B, Sq, H, 0.07, 1, parts, FAKE, FAKE,
                 FAKE, 1 << 30, trace, n, None)
    # Sq * H = 256 folded rows: 4 M-tiles of 64, so 8 partitions run 32 workgroups
    assert call(FAKE, 3 * 32 - 1) == INVALID
    assert call(None, 3 * 32) == INVALID
    assert call(FAKE + 2, 3 * 32) == INVALID
    assert call(FAKE, 3 * 32, parts=-1) == INVALID
    assert call(FAKE, 3 * 32, B=0) == INVALID
    assert call(FAKE, 3 * 8 - 1, Sq=4, parts=8) == INVALID  # one M-tile: 8 workgroups


def test_timeline_records_reject_on_host():
    """The timeline needs the placement record (3 int32 per split-KV workgroup) and 5
    int64 per workgroup in an 8-byte-aligned buffer; any shortfall is refused before
    anything is enqueued."""
    f = mla.lib().mla_decode_splitkv_timeline

    def call(trace, n, times, m, parts=8):
        return f(FAKE, FAKE, FAKE, 64, 64, FAKE, 16, FAKE, 4, 16, 16, 0.07, 1, parts, FAKE, FAKE,
                 FAKE, 1 << 30, trace, n, times, m, None)
    # 4 M-tiles x 8 partitions = 32 workgroups
    assert call(FAKE, 3 * 32 - 1, FAKE, 5 * 32) == INVALID
    assert call(FAKE, 3 * 32, FAKE, 5 * 32 - 1) == INVALID
    assert call(FAKE, 3 * 32, None, 5 * 32) == INVALID
    assert call(FAKE, 3 * 32, FAKE + 4, 5 * 32) == INVALID
    assert call(None, 3 * 32, FAKE, 5 * 32) == INVALID
    assert call(FAKE, 3 * 32, FAKE, 5 * 32, parts=-1) == INVALID


def test_read_error_flags_rejects_null():
    out = ctypes.c_uint32(0)
    assert mla.lib().mla_read_error_flags(None, None, ctypes.byref(out)) == INVALID
    assert mla.lib().mla_read_error_flags(FAKE, None, None) == INVALID


def test_binding_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(bnd, "_lib", None)
    monkeypatch.setattr(bnd, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="missing"):
        bnd.lib()
