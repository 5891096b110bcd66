"""ctypes binding of libmla.so: argument marshalling only.

Every step of the computation runs in the library's HIP kernels; this module turns
torch tensors into device pointers, picks the current HIP stream, and maps status
codes to exceptions.  It never computes attention itself and has no CPU fallback:
if the library is missing it raises.
"""
from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "mla.h")

MLA_OK = 0
MLA_ERR_INVALID_ARG = -1
MLA_ERR_UNSUPPORTED = -2
MLA_ERR_WORKSPACE = -3
MLA_ERR_HIP = -4
MLA_ERR_DEVICE_CHECK = -5
MLA_FLAG_BAD_SEQ_LEN = 1
MLA_FLAG_BAD_PAGE_ID = 2
PAGE_SIZE = 64
NOPE_DIM = 512
ROPE_DIM = 64

_lib = None

_vp = ctypes.c_void_p
_i32 = ctypes.c_int
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_sz = ctypes.c_size_t

_COMPUTE_ARGS = [_vp, _vp, _vp, _i64, _i32, _vp, _i32, _vp, _i32, _i32, _i32, _f32, _i32, _i32,
                 _vp, _vp, _vp, _sz, _vp]
_COMPUTE_ARGS_E4M3 = [_vp, _vp, _vp, _f32, _i64, _i32, _vp, _i32, _vp, _i32, _i32, _i32, _f32,
                      _i32, _i32, _vp, _vp, _vp, _sz, _vp]
_SIGNATURES = {
    "mla_status_string": ([_i32], ctypes.c_char_p),
    "mla_decode_auto_partitions": ([_i32, _i32, _i32, _i32, ctypes.POINTER(_i32)], _i32),
    "mla_decode_workspace_size": ([_i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz)], _i32),
    "mla_decode_workspace_bytes": ([_i32, _i32, _i32, _i32], _sz),
    "mla_prefill_workspace_bytes": ([_i32, _i32, _i32, _i32], _sz),
    "mla_decode": (_COMPUTE_ARGS, _i32),
    "mla_decode_splitkv": (_COMPUTE_ARGS, _i32),
    "mla_prefill_with_prefix": (_COMPUTE_ARGS, _i32),
    "mla_decode_e4m3": (_COMPUTE_ARGS_E4M3, _i32),
    "mla_decode_single_pass": (_COMPUTE_ARGS, _i32),
    "mla_decode_noalloc": (_COMPUTE_ARGS[:16] + [_vp], _i32),
    "mla_kv_append": ([_vp, _vp, _i64, _i32, _vp, _i32, _vp, _i32, _i32, _vp, _sz, _vp], _i32),
    "mla_kv_append_e4m3": ([_vp, _vp, _f32, _i64, _i32, _vp, _i32, _vp, _i32, _i32, _vp, _sz,
                            _vp], _i32),
    "mla_decode_nope": ([_vp, _vp, _i64, _i32, _vp, _i32, _vp, _i32, _i32, _i32, _f32, _i32,
                         _i32, _vp, _vp, _vp, _sz, _vp], _i32),
    "mla_decode_splitkv_nope": ([_vp, _vp, _i64, _i32, _vp, _i32, _vp, _i32, _i32, _i32, _f32,
                                 _i32, _i32, _vp, _vp, _vp, _sz, _vp], _i32),
    "mla_absorb_q": ([_vp, _vp, _vp, _i32, _i32, _i32, _vp], _i32),
    "mla_project_o": ([_vp, _vp, _vp, _i32, _i32, _i32, _vp], _i32),
    "mla_decode_varlen": ([_vp, _vp, _vp, _i64, _i32, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _f32,
                           _i32, _vp, _vp, _vp, _sz, _vp], _i32),
    "mla_decode_tree": ([_vp, _vp, _vp, _i64, _i32, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _f32,
                         _i32, _vp, _vp, _vp, _sz, _vp], _i32),
    "mla_decode_tree_e4m3": ([_vp, _vp, _vp, _f32, _i64, _i32, _vp, _i32, _vp, _vp, _i32, _i32,
                              _i32, _f32, _i32, _vp, _vp, _vp, _sz, _vp], _i32),
    "mla_decode_single_pass_e4m3": (_COMPUTE_ARGS_E4M3, _i32),
    "mla_decode_splitkv_e4m3": (_COMPUTE_ARGS_E4M3, _i32),
    "mla_decode_combine": ([_vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp], _i32),
    "mla_decode_splitkv_placement": (_COMPUTE_ARGS[:-1] + [_vp, _i64, _vp], _i32),
    "mla_decode_splitkv_timeline": (_COMPUTE_ARGS[:-1] + [_vp, _i64, _vp, _i64, _vp], _i32),
    "mla_read_error_flags": ([_vp, _vp, ctypes.POINTER(ctypes.c_uint32)], _i32),
}


class MLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def header_functions(path: str = HEADER_PATH):
    """Names of the functions include/mla.h declares."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def lib():
    """Loads libmla.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m mla_latent_kv_16_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().mla_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != MLA_OK:
        raise MLAError(status, where)


def auto_partitions(B: int, Sq: int, H: int, max_pages_per_seq: int) -> int:
    out = _i32(0)
    _check(lib().mla_decode_auto_partitions(B, Sq, H, max_pages_per_seq, ctypes.byref(out)),
           "mla_decode_auto_partitions")
    return out.value


def workspace_size(B: int, Sq: int, H: int, max_pages_per_seq: int, num_partitions: int = 0) -> int:
    out = _sz(0)
    _check(lib().mla_decode_workspace_size(B, Sq, H, max_pages_per_seq, num_partitions,
                                           ctypes.byref(out)), "mla_decode_workspace_size")
    return out.value


def workspace_bytes(B: int, Sq: int, H: int, max_pages_per_seq: int, prefill: bool = False) -> int:
    """Workspace bytes for the automatic partition count (0 = sizes rejected)."""
    fn = lib().mla_prefill_workspace_bytes if prefill else lib().mla_decode_workspace_bytes
    return int(fn(B, Sq, H, max_pages_per_seq))


def _torch():
    import torch
    return torch


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _expect(t, name, dtypes, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def new_workspace(B, Sq, H, max_pages_per_seq, num_partitions=0, device=None):
    """Zero-filled workspace of the size the library asks for."""
    torch = _torch()
    n = workspace_size(B, Sq, H, max_pages_per_seq, num_partitions)
    return torch.zeros(n, dtype=torch.uint8, device=device or "cuda")


def _prep(q_nope, q_rope, kv_pool, block_table, seq_lens, out, lse, workspace, num_partitions,
          e4m3=False, nope=False):
    """Checks shapes, dtypes and placement; allocates missing outputs and workspace.
    nope: 512-wide pool rows and no q_rope (q_rope is then ignored)."""
    torch = _torch()
    bf = (torch.bfloat16, torch.int16)
    if q_nope.dim() != 4:
        raise ValueError("q_nope must be [B, Sq, H, 512]")
    B, Sq, H, D = q_nope.shape
    if D != NOPE_DIM:
        raise ValueError("q_nope last dim must be 512")
    _expect(q_nope, "q_nope", bf)
    if not nope:
        _expect(q_rope, "q_rope", bf, (B, Sq, H, ROPE_DIM))
    width = NOPE_DIM if nope else NOPE_DIM + ROPE_DIM
    if kv_pool.dim() != 3 or kv_pool.shape[1] != PAGE_SIZE or kv_pool.shape[2] != width:
        raise ValueError(f"kv_pool must be [num_pages, 64, {width}]")
    _expect(kv_pool, "kv_pool", (torch.uint8,) if e4m3 else bf)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages_per_seq]")
    _expect(block_table, "block_table", (torch.int32,))
    _expect(seq_lens, "seq_lens", (torch.int32,), (B,))
    dev = q_nope.device
    if out is None:
        out = torch.empty((B, Sq, H, NOPE_DIM), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, Sq, H), dtype=torch.float32, device=dev)
    _expect(out, "out", (torch.float32,), (B, Sq, H, NOPE_DIM))
    _expect(lse, "lse", (torch.float32,), (B, Sq, H))
    maxp = block_table.shape[1]
    if workspace is None:
        workspace = new_workspace(B, Sq, H, maxp, num_partitions, device=dev)
    _expect(workspace, "workspace", (torch.uint8,))
    return B, Sq, H, maxp, out, lse, workspace


def _compute(fn_name, q_nope, q_rope, kv_pool, block_table, seq_lens, softmax_scale, causal,
             num_partitions, out, lse, workspace, stream):
    B, Sq, H, maxp, out, lse, workspace = _prep(q_nope, q_rope, kv_pool, block_table, seq_lens,
                                                out, lse, workspace, num_partitions)
    fn = getattr(lib(), fn_name)
    st = fn(_ptr(q_nope), _ptr(q_rope), _ptr(kv_pool), kv_pool.shape[0], PAGE_SIZE,
            _ptr(block_table), maxp, _ptr(seq_lens), B, Sq, H, float(softmax_scale),
            1 if causal else 0, int(num_partitions), _ptr(out), _ptr(lse), _ptr(workspace),
            workspace.numel(), _stream_handle(stream))
    _check(st, fn_name)
    return out, lse


def _compute_e4m3(fn_name, q_nope, q_rope, kv_pool, kv_scale, block_table, seq_lens,
                  softmax_scale, causal, num_partitions, out, lse, workspace, stream):
    B, Sq, H, maxp, out, lse, workspace = _prep(q_nope, q_rope, kv_pool, block_table, seq_lens,
                                                out, lse, workspace, num_partitions, e4m3=True)
    fn = getattr(lib(), fn_name)
    st = fn(_ptr(q_nope), _ptr(q_rope), _ptr(kv_pool), float(kv_scale), kv_pool.shape[0],
            PAGE_SIZE, _ptr(block_table), maxp, _ptr(seq_lens), B, Sq, H, float(softmax_scale),
            1 if causal else 0, int(num_partitions), _ptr(out), _ptr(lse), _ptr(workspace),
            workspace.numel(), _stream_handle(stream))
    _check(st, fn_name)
    return out, lse


def decode_e4m3(q_nope, q_rope, kv_pool, kv_scale, block_table, seq_lens, softmax_scale,
                causal=True, num_partitions=0, out=None, lse=None, workspace=None, stream=None):
    """mla_decode_e4m3: decode over an E4M3 pool (uint8 [P, 64, 576]) with a per-tensor
    scale.  Returns (O fp32 [B,Sq,H,512], lse fp32 [B,Sq,H])."""
    return _compute_e4m3("mla_decode_e4m3", q_nope, q_rope, kv_pool, kv_scale, block_table,
                         seq_lens, softmax_scale, causal, num_partitions, out, lse, workspace,
                         stream)


def decode_splitkv_e4m3(q_nope, q_rope, kv_pool, kv_scale, block_table, seq_lens,
                        softmax_scale, causal=True, num_partitions=0, out=None, lse=None,
                        workspace=None, stream=None):
    """mla_decode_splitkv_e4m3: the split-KV pass alone over an E4M3 pool."""
    return _compute_e4m3("mla_decode_splitkv_e4m3", q_nope, q_rope, kv_pool, kv_scale,
                         block_table, seq_lens, softmax_scale, causal, num_partitions, out, lse,
                         workspace, stream)


def decode_single_pass_e4m3(q_nope, q_rope, kv_pool, kv_scale, block_table, seq_lens,
                            softmax_scale, causal=True, num_partitions=0, out=None, lse=None,
                            workspace=None, stream=None):
    """mla_decode_single_pass_e4m3: the E4M3-pool decode in one launch."""
    return _compute_e4m3("mla_decode_single_pass_e4m3", q_nope, q_rope, kv_pool, kv_scale,
                         block_table, seq_lens, softmax_scale, causal, num_partitions, out, lse,
                         workspace, stream)


def decode(q_nope, q_rope, kv_pool, block_table, seq_lens, softmax_scale, causal=True,
           num_partitions=0, out=None, lse=None, workspace=None, stream=None):
    """mla_decode: split-KV pass + combine pass.  Returns (O fp32 [B,Sq,H,512], lse fp32 [B,Sq,H])."""
    return _compute("mla_decode", q_nope, q_rope, kv_pool, block_table, seq_lens, softmax_scale,
                    causal, num_partitions, out, lse, workspace, stream)


def decode_noalloc(q_nope, q_rope, kv_pool, block_table, seq_lens, softmax_scale, causal=True,
                   num_partitions=0, out=None, lse=None, stream=None):
    """mla_decode_noalloc: the decode with its workspace in the library's own static
    device array (no workspace argument, nothing allocated by the library)."""
    torch = _torch()
    B, Sq, H, _ = q_nope.shape
    ws = torch.empty(256, dtype=torch.uint8, device=q_nope.device)  # validation only
    B, Sq, H, maxp, out, lse, _ = _prep(q_nope, q_rope, kv_pool, block_table, seq_lens, out, lse,
                                        ws, 1)
    st = lib().mla_decode_noalloc(_ptr(q_nope), _ptr(q_rope), _ptr(kv_pool), kv_pool.shape[0],
                                  PAGE_SIZE, _ptr(block_table), maxp, _ptr(seq_lens), B, Sq, H,
                                  float(softmax_scale), 1 if causal else 0, int(num_partitions),
                                  _ptr(out), _ptr(lse), _stream_handle(stream))
    _check(st, "mla_decode_noalloc")
    return out, lse


def decode_single_pass(q_nope, q_rope, kv_pool, block_table, seq_lens, softmax_scale,
                       causal=True, num_partitions=0, out=None, lse=None, workspace=None,
                       stream=None):
    """mla_decode_single_pass: the same decode in one launch (merging workgroups appended
    to the split-KV grid)."""
    return _compute("mla_decode_single_pass", q_nope, q_rope, kv_pool, block_table, seq_lens,
                    softmax_scale, causal, num_partitions, out, lse, workspace, stream)


def _tree_mask_arg(tree_mask, B, Sq):
    torch = _torch()
    if tree_mask.dtype not in (torch.int64, torch.uint64) or tuple(tree_mask.shape) != (B, Sq):
        raise ValueError("tree_mask must be int64/uint64 [B, Sq] (ancestor bits)")
    if not tree_mask.is_contiguous() or not tree_mask.is_cuda:
        raise ValueError("tree_mask must be a contiguous device tensor")
    return _ptr(tree_mask)


def decode_tree(q_nope, q_rope, kv_pool, block_table, seq_lens, tree_mask, softmax_scale,
                num_partitions=0, out=None, lse=None, workspace=None, stream=None,
                kv_scale=None):
    """mla_decode_tree (bf16 pool) or mla_decode_tree_e4m3 (uint8 pool with kv_scale):
    decode of a draft tree, tree_mask int64 [B, Sq] ancestor bits (Sq <= 64)."""
    e4m3 = kv_scale is not None
    B, Sq, H, maxp, out, lse, workspace = _prep(q_nope, q_rope, kv_pool, block_table, seq_lens,
                                                out, lse, workspace, num_partitions, e4m3=e4m3)
    tm = _tree_mask_arg(tree_mask, B, Sq)
    L = lib()
    pool = (_ptr(kv_pool), float(kv_scale)) if e4m3 else (_ptr(kv_pool),)
    name = "mla_decode_tree_e4m3" if e4m3 else "mla_decode_tree"
    st = getattr(L, name)(_ptr(q_nope), _ptr(q_rope), *pool, kv_pool.shape[0], PAGE_SIZE,
                          _ptr(block_table), maxp, _ptr(seq_lens), tm, B, Sq, H,
                          float(softmax_scale), int(num_partitions), _ptr(out), _ptr(lse),
                          _ptr(workspace), workspace.numel(), _stream_handle(stream))
    _check(st, name)
    return out, lse


def decode_nope(q_nope, kv_pool, block_table, seq_lens, softmax_scale, causal=True,
                num_partitions=0, out=None, lse=None, workspace=None, stream=None):
    """mla_decode_nope: NoPE-MLA decode, kv_pool bf16 [P, 64, 512], no q_rope."""
    B, Sq, H, maxp, out, lse, workspace = _prep(q_nope, None, kv_pool, block_table, seq_lens,
                                                out, lse, workspace, num_partitions, nope=True)
    st = lib().mla_decode_nope(_ptr(q_nope), _ptr(kv_pool), kv_pool.shape[0], PAGE_SIZE,
                               _ptr(block_table), maxp, _ptr(seq_lens), B, Sq, H,
                               float(softmax_scale), 1 if causal else 0, int(num_partitions),
                               _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                               _stream_handle(stream))
    _check(st, "mla_decode_nope")
    return out, lse


def absorb_q(q_heads, w_uk_t, out=None, stream=None):
    """mla_absorb_q: q_heads bf16 [B, Sq, H, 128], w_uk_t bf16 [H, 512, 128] ->
    q_lat bf16 [B, Sq, H, 512] (the absorbed query mla_decode takes)."""
    call, out = bound_absorb_q(q_heads, w_uk_t, out, stream)
    call()
    return out


def bound_absorb_q(q_heads, w_uk_t, out=None, stream=None):
    """absorb_q checked and marshalled once: returns (callable, out)."""
    torch = _torch()
    bf = (torch.bfloat16, torch.int16)
    if q_heads.dim() != 4 or q_heads.shape[3] != 128:
        raise ValueError("q_heads must be [B, Sq, H, 128]")
    B, Sq, H = q_heads.shape[:3]
    _expect(q_heads, "q_heads", bf)
    _expect(w_uk_t, "w_uk_t", bf, (H, 512, 128))
    if out is None:
        out = torch.empty((B, Sq, H, 512), dtype=q_heads.dtype, device=q_heads.device)
    _expect(out, "out", bf, (B, Sq, H, 512))
    fn, args = lib().mla_absorb_q, (_ptr(q_heads), _ptr(w_uk_t), _ptr(out), B, Sq, H,
                                    _stream_handle(stream))

    def call(_keep=(q_heads, w_uk_t, out)):
        _check(fn(*args), "mla_absorb_q")
    return call, out


def project_o(O, w_uv, out=None, stream=None):
    """mla_project_o: O fp32 [B, Sq, H, 512], w_uv bf16 [H, 128, 512] ->
    fp32 [B, Sq, H, 128]."""
    call, out = bound_project_o(O, w_uv, out, stream)
    call()
    return out


def bound_project_o(O, w_uv, out=None, stream=None):
    """project_o checked and marshalled once: returns (callable, out)."""
    torch = _torch()
    if O.dim() != 4 or O.shape[3] != 512:
        raise ValueError("O must be [B, Sq, H, 512]")
    B, Sq, H = O.shape[:3]
    _expect(O, "O", (torch.float32,))
    _expect(w_uv, "w_uv", (torch.bfloat16, torch.int16), (H, 128, 512))
    if out is None:
        out = torch.empty((B, Sq, H, 128), dtype=torch.float32, device=O.device)
    _expect(out, "out", (torch.float32,), (B, Sq, H, 128))
    fn, args = lib().mla_project_o, (_ptr(O), _ptr(w_uv), _ptr(out), B, Sq, H,
                                     _stream_handle(stream))

    def call(_keep=(O, w_uv, out)):
        _check(fn(*args), "mla_project_o")
    return call, out


def decode_varlen(q_nope, q_rope, kv_pool, block_table, seq_lens, q_lens, softmax_scale,
                  num_partitions=0, out=None, lse=None, workspace=None, stream=None):
    """mla_decode_varlen: request b verifies q_lens[b] (int32 [B], device) of the Sq
    query slots; padding slots come back as O = 0, LSE = -inf."""
    torch = _torch()
    B, Sq, H, maxp, out, lse, workspace = _prep(q_nope, q_rope, kv_pool, block_table, seq_lens,
                                                out, lse, workspace, num_partitions)
    if q_lens.dtype != torch.int32 or tuple(q_lens.shape) != (B,) or not q_lens.is_cuda:
        raise ValueError("q_lens must be an int32 [B] device tensor")
    st = lib().mla_decode_varlen(_ptr(q_nope), _ptr(q_rope), _ptr(kv_pool), kv_pool.shape[0],
                                 PAGE_SIZE, _ptr(block_table), maxp, _ptr(seq_lens),
                                 _ptr(q_lens), B, Sq, H, float(softmax_scale),
                                 int(num_partitions), _ptr(out), _ptr(lse), _ptr(workspace),
                                 workspace.numel(), _stream_handle(stream))
    _check(st, "mla_decode_varlen")
    return out, lse


def kv_append(kv_new, kv_pool, block_table, seq_lens, workspace, kv_scale=None, stream=None):
    """mla_kv_append (bf16 pool) or mla_kv_append_e4m3 (uint8 pool, with kv_scale):
    kv_new bf16 [B, Sq, 576] becomes each request's last Sq logical rows."""
    bound_kv_append(kv_new, kv_pool, block_table, seq_lens, workspace, kv_scale, stream)()
    return kv_pool


def bound_kv_append(kv_new, kv_pool, block_table, seq_lens, workspace, kv_scale=None,
                    stream=None):
    """kv_append with its arguments checked and marshalled once: returns a callable
    that makes the single foreign call (for loops that repeat the same write)."""
    torch = _torch()
    e4m3 = kv_scale is not None
    if kv_new.dim() != 3 or kv_new.shape[2] != 576 or kv_new.dtype not in (torch.bfloat16,
                                                                              torch.int16):
        raise ValueError("kv_new must be bf16 [B, Sq, 576]")
    if kv_pool.dim() != 3 or tuple(kv_pool.shape[1:]) != (PAGE_SIZE, 576):
        raise ValueError("kv_pool must be [num_pages, 64, 576] (rows of the width kv_new has)")
    want = torch.uint8 if e4m3 else (torch.bfloat16, torch.int16)
    if (kv_pool.dtype != want) if e4m3 else (kv_pool.dtype not in want):
        raise ValueError("kv_pool dtype does not match the pool format")
    for name, t in (("kv_new", kv_new), ("kv_pool", kv_pool), ("block_table", block_table),
                    ("seq_lens", seq_lens), ("workspace", workspace)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    B, Sq = kv_new.shape[:2]
    L = lib()
    pool = (_ptr(kv_pool), float(kv_scale)) if e4m3 else (_ptr(kv_pool),)
    name = "mla_kv_append_e4m3" if e4m3 else "mla_kv_append"
    fn = getattr(L, name)
    args = (_ptr(kv_new), *pool, kv_pool.shape[0], PAGE_SIZE, _ptr(block_table),
            block_table.shape[1], _ptr(seq_lens), B, Sq, _ptr(workspace), workspace.numel(),
            _stream_handle(stream))
    keep = (kv_new, kv_pool, block_table, seq_lens, workspace)

    def call(_keep=keep):
        _check(fn(*args), name)
    return call


def decode_splitkv(q_nope, q_rope, kv_pool, block_table, seq_lens, softmax_scale, causal=True,
                   num_partitions=0, out=None, lse=None, workspace=None, stream=None):
    """mla_decode_splitkv: the split-KV pass alone."""
    return _compute("mla_decode_splitkv", q_nope, q_rope, kv_pool, block_table, seq_lens,
                    softmax_scale, causal, num_partitions, out, lse, workspace, stream)


def decode_splitkv_placement(q_nope, q_rope, kv_pool, block_table, seq_lens, softmax_scale,
                             causal=True, num_partitions=0, out=None, lse=None, workspace=None,
                             stream=None):
    """mla_decode_splitkv_placement: the split-KV pass plus, per split-KV workgroup in
    launch order, the (XCC id, KV partition, M-tile) it ran with, as an int32 [n, 3]
    device tensor."""
    torch = _torch()
    B, Sq, H, maxp, out, lse, workspace = _prep(q_nope, q_rope, kv_pool, block_table, seq_lens,
                                                out, lse, workspace, num_partitions)
    G = int(num_partitions) or auto_partitions(B, Sq, H, maxp)
    n_wg = G * ((Sq * H + 63) // 64)
    trace = torch.full((n_wg, 3), -1, dtype=torch.int32, device=q_nope.device)
    st = lib().mla_decode_splitkv_placement(
        _ptr(q_nope), _ptr(q_rope), _ptr(kv_pool), kv_pool.shape[0], PAGE_SIZE,
        _ptr(block_table), maxp, _ptr(seq_lens), B, Sq, H, float(softmax_scale),
        1 if causal else 0, int(num_partitions), _ptr(out), _ptr(lse), _ptr(workspace),
        workspace.numel(), _ptr(trace), trace.numel(), _stream_handle(stream))
    _check(st, "mla_decode_splitkv_placement")
    return out, lse, trace


def decode_splitkv_timeline(q_nope, q_rope, kv_pool, block_table, seq_lens, softmax_scale,
                            causal=True, num_partitions=0, out=None, lse=None, workspace=None,
                            stream=None):
    """mla_decode_splitkv_timeline: the split-KV pass plus, per split-KV workgroup in
    launch order, the (XCC id, KV partition, M-tile) it ran with (int32 [n, 3]) and five
    ticks of the 100 MHz constant clock (int64 [n, 5]: start, page prefix built, first
    block in LDS, walk over, stores complete; 0 where not reached)."""
    torch = _torch()
    B, Sq, H, maxp, out, lse, workspace = _prep(q_nope, q_rope, kv_pool, block_table, seq_lens,
                                                out, lse, workspace, num_partitions)
    G = int(num_partitions) or auto_partitions(B, Sq, H, maxp)
    n_wg = G * ((Sq * H + 63) // 64)
    trace = torch.full((n_wg, 3), -1, dtype=torch.int32, device=q_nope.device)
    ticks = torch.zeros((n_wg, 5), dtype=torch.int64, device=q_nope.device)
    st = lib().mla_decode_splitkv_timeline(
        _ptr(q_nope), _ptr(q_rope), _ptr(kv_pool), kv_pool.shape[0], PAGE_SIZE,
        _ptr(block_table), maxp, _ptr(seq_lens), B, Sq, H, float(softmax_scale),
        1 if causal else 0, int(num_partitions), _ptr(out), _ptr(lse), _ptr(workspace),
        workspace.numel(), _ptr(trace), trace.numel(), _ptr(ticks), ticks.numel(),
        _stream_handle(stream))
    _check(st, "mla_decode_splitkv_timeline")
    return out, lse, trace, ticks


def decode_combine(seq_lens, max_pages_per_seq, Sq, H, out, lse, workspace, num_partitions=0,
                   stream=None):
    """mla_decode_combine: the log-sum-exp merge of the split-KV partials."""
    B = seq_lens.shape[0]
    st = lib().mla_decode_combine(_ptr(seq_lens), max_pages_per_seq, B, Sq, H,
                                  int(num_partitions), _ptr(out), _ptr(lse), _ptr(workspace),
                                  workspace.numel(), _stream_handle(stream))
    _check(st, "mla_decode_combine")
    return out, lse


def prefill_with_prefix(q_nope, q_rope, kv_pool, block_table, seq_lens, softmax_scale,
                        causal=True, num_partitions=0, out=None, lse=None, workspace=None,
                        stream=None):
    """mla_prefill_with_prefix: a chunk of Sq new tokens over its cached prefix."""
    return _compute("mla_prefill_with_prefix", q_nope, q_rope, kv_pool, block_table, seq_lens,
                    softmax_scale, causal, num_partitions, out, lse, workspace, stream)


def read_error_flags(workspace, stream=None) -> int:
    """Synchronises the stream and returns (and clears) the kernels' data-fault flags."""
    out = ctypes.c_uint32(0)
    _check(lib().mla_read_error_flags(_ptr(workspace), _stream_handle(stream), ctypes.byref(out)),
           "mla_read_error_flags")
    return out.value


class BoundDecode:
    """Decode call with its arguments validated and marshalled once.

    For loops that launch the same shapes repeatedly (benchmarks, serving steps):
    each call is a single foreign-function call into the library.  The tensors are
    kept alive by this object.
    """

    def __init__(self, q_nope, q_rope, kv_pool, block_table, seq_lens, softmax_scale, causal=True,
                 num_partitions=0, out=None, lse=None, workspace=None, stream=None,
                 kv_scale=None, nope=False):
        e4m3 = kv_scale is not None  # an E4M3 pool comes with its scale
        B, Sq, H, maxp, out, lse, workspace = _prep(q_nope, q_rope, kv_pool, block_table,
                                                    seq_lens, out, lse, workspace, num_partitions,
                                                    e4m3=e4m3, nope=nope)
        self.tensors = (q_nope, q_rope, kv_pool, block_table, seq_lens, out, lse, workspace)
        self.out, self.lse, self.workspace = out, lse, workspace
        self.num_partitions = int(num_partitions) or auto_partitions(B, Sq, H, maxp)
        pool_args = ((_ptr(kv_pool), float(kv_scale)) if e4m3 else (_ptr(kv_pool),))
        q_args = (_ptr(q_nope),) if nope else (_ptr(q_nope), _ptr(q_rope))
        self._args = (*q_args, *pool_args, kv_pool.shape[0], PAGE_SIZE,
                      _ptr(block_table), maxp, _ptr(seq_lens), B, Sq, H, float(softmax_scale),
                      1 if causal else 0, self.num_partitions, _ptr(out), _ptr(lse),
                      _ptr(workspace), workspace.numel(), _stream_handle(stream))
        self._cargs = (_ptr(seq_lens), maxp, B, Sq, H, self.num_partitions, _ptr(out), _ptr(lse),
                       _ptr(workspace), workspace.numel(), _stream_handle(stream))
        L = lib()
        if nope:
            self._decode, self._split = L.mla_decode_nope, L.mla_decode_splitkv_nope
            self._single = None
        elif e4m3:
            self._decode, self._split = L.mla_decode_e4m3, L.mla_decode_splitkv_e4m3
            self._single = L.mla_decode_single_pass_e4m3
        else:
            self._decode, self._split = L.mla_decode, L.mla_decode_splitkv
            self._single = L.mla_decode_single_pass
        self._combine = L.mla_decode_combine

    def __call__(self):
        _check(self._decode(*self._args), "mla_decode")

    def single_pass(self):
        if self._single is None:
            raise ValueError("no single-pass entry point for NoPE pools")
        _check(self._single(*self._args), "mla_decode_single_pass")

    def splitkv(self):
        _check(self._split(*self._args), "mla_decode_splitkv")

    def combine(self):
        _check(self._combine(*self._cargs), "mla_decode_combine")
