"""ctypes binding of libverify_attn.so (argument marshalling only).

Every step of the verify path runs in the library's HIP kernels; this module
turns torch tensors into the pointers, strides and scalars the C ABI of
``include/verify_attn.h`` takes.  PyTorch provides device memory and the
current stream, nothing else.  If the library is missing the functions raise:
there is no CPU or PyTorch fallback.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libverify_attn.so")

VA_OK, VA_EINVAL, VA_EUNSUPPORTED, VA_EWORKSPACE, VA_EHIP = 0, 1, 2, 3, 4
VA_KV_BF16, VA_KV_FP8_E4M3FN = 0, 1

EXPORTED = (
    "verify_attn_build_block_table",
    "verify_attn_fwd",
    "verify_attn_combine",
    "verify_attn_can_handle",
    "verify_attn_num_splits",
    "verify_attn_workspace_bytes",
    "verify_attn_strerror",
    "verify_attn_abi_version",
    "verify_attn_translate_slots",
)


class VerifyAttnArgs(ctypes.Structure):
    """Mirror of ``verify_attn_args`` (include/verify_attn.h), field for field."""

    _fields_ = [
        ("struct_size", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("draft_len", ctypes.c_int32),
        ("hq", ctypes.c_int32),
        ("hkv", ctypes.c_int32),
        ("qk_dim", ctypes.c_int32),
        ("v_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("sm_scale", ctypes.c_float),
        ("window_left", ctypes.c_int32),
        ("max_prefix_len", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("q_stride_row", ctypes.c_int64),
        ("q_stride_head", ctypes.c_int64),
        ("k_cache", ctypes.c_void_p),
        ("k_stride_slot", ctypes.c_int64),
        ("k_stride_head", ctypes.c_int64),
        ("v_cache", ctypes.c_void_p),
        ("v_stride_slot", ctypes.c_int64),
        ("v_stride_head", ctypes.c_int64),
        ("block_table", ctypes.c_void_p),
        ("max_pages_per_seq", ctypes.c_int32),
        ("prefix_lens", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_int64),
        ("out", ctypes.c_void_p),
        ("o_stride_row", ctypes.c_int64),
        ("o_stride_head", ctypes.c_int64),
        ("lse", ctypes.c_void_p),
        # version 2 extensions
        ("qo_indptr", ctypes.c_void_p),
        ("draft_slots", ctypes.c_void_p),
        ("tree_mask", ctypes.c_void_p),
        ("sinks", ctypes.c_void_p),
        ("logit_cap", ctypes.c_float),
    ]


# size of the version 1 layout (every field before qo_indptr)
V1_SIZE = VerifyAttnArgs.qo_indptr.offset


class VerifyAttnError(RuntimeError):
    def __init__(self, func: str, status: int, text: str):
        super().__init__(f"{func} failed with status {status} ({text})")
        self.status = status


_lib = None


def load(path: Optional[str] = None):
    """Load the library once (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(
            f"{p} is missing: build it with `python -m speculative_decoding_verify_02_amd.build`")
    lib = ctypes.CDLL(p)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    args_p = ctypes.POINTER(VerifyAttnArgs)
    lib.verify_attn_build_block_table.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp]
    lib.verify_attn_build_block_table.restype = ctypes.c_int
    for name in ("verify_attn_fwd", "verify_attn_combine"):
        getattr(lib, name).argtypes = [args_p, vp]
        getattr(lib, name).restype = ctypes.c_int
    lib.verify_attn_can_handle.argtypes = [args_p]
    lib.verify_attn_can_handle.restype = ctypes.c_int
    lib.verify_attn_num_splits.argtypes = [args_p]
    lib.verify_attn_num_splits.restype = i32
    lib.verify_attn_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.verify_attn_workspace_bytes.restype = i64
    lib.verify_attn_strerror.argtypes = [ctypes.c_int]
    lib.verify_attn_strerror.restype = ctypes.c_char_p
    lib.verify_attn_abi_version.argtypes = []
    lib.verify_attn_abi_version.restype = i32
    lib.verify_attn_translate_slots.argtypes = [vp, i64, vp, i64, vp, vp]
    lib.verify_attn_translate_slots.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def strerror(status: int) -> str:
    return load().verify_attn_strerror(status).decode()


def _check(func: str, status: int) -> None:
    if status != VA_OK:
        raise VerifyAttnError(func, status, strerror(status))


def _stream_ptr(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


# ---------------------------------------------------------------------------
# a1: block table
# ---------------------------------------------------------------------------

def verify_attn_build_block_table(kv_indptr, kv_indices, page_size: int, max_pages_per_seq: int,
                                  block_table=None, kv_lens=None, stream=None, check=True):
    """Scatter token-level slots into a [B, max_pages] int32 page table (on the GPU).

    ``kv_indptr`` [B+1] and ``kv_indices`` int32 CUDA tensors.  Allocates the outputs
    when not given.  Returns (block_table, kv_lens) or the raw status if check=False."""
    import torch
    batch = kv_indptr.numel() - 1
    dev = kv_indptr.device
    if block_table is None:
        block_table = torch.empty((batch, max_pages_per_seq), dtype=torch.int32, device=dev)
    if kv_lens is None:
        kv_lens = torch.empty((batch,), dtype=torch.int32, device=dev)
    st = load().verify_attn_build_block_table(
        _ptr(kv_indptr), _ptr(kv_indices), batch, page_size, max_pages_per_seq,
        _ptr(block_table), _ptr(kv_lens), _stream_ptr(stream))
    if not check:
        return st
    _check("verify_attn_build_block_table", st)
    return block_table, kv_lens


# ---------------------------------------------------------------------------
# a2-a7: forward + combine
# ---------------------------------------------------------------------------

@dataclass
class VerifyCall:
    """A ready-to-launch call: the ctypes args plus the tensors they point into
    (kept alive here so the pointers stay valid)."""

    args: VerifyAttnArgs
    tensors: dict


def make_args(*, q, k_cache, v_cache, block_table, prefix_lens, draft_len: int, page_size: int,
              sm_scale: float, max_prefix_len: int, out, workspace, lse=None,
              kv_dtype: int = VA_KV_BF16, k_scale: float = 1.0, v_scale: float = 1.0,
              window_left: int = -1, num_splits: int = 0, v_dim: Optional[int] = None,
              qk_dim: Optional[int] = None, qo_indptr=None, draft_slots=None, tree_mask=None,
              sinks=None, logit_cap: float = 0.0) -> VerifyCall:
    """Build verify_attn_args from torch tensors.

    q [B*D, Hq, qk_dim] bf16; k_cache [num_slots, Hkv, >= qk_dim] and v_cache
    [num_slots, Hkv, >= v_dim] (bf16, or uint8 holding e4m3fn codes) - v_cache may be
    k_cache itself (MLA alias, give v_dim); block_table [B, max_pages] int32;
    prefix_lens [B] int32; out [B*D, Hq, v_dim] bf16; workspace a float32 tensor of
    at least workspace_bytes() (or None while sizing it: see set_workspace); lse
    [B*D, Hq] float32 or None.  Extensions (include/verify_attn.h, version 2):
    qo_indptr [B+1] int32 (ragged rows; q/out/lse then have qo_indptr[B] rows),
    draft_slots [B, D] int32 with tree_mask [B, D, D] uint8 (tree verify), sinks
    [Hq] float32, logit_cap."""
    qk_dim = q.shape[-1] if qk_dim is None else qk_dim
    v_dim = out.shape[-1] if v_dim is None else v_dim
    a = VerifyAttnArgs()
    a.struct_size = ctypes.sizeof(VerifyAttnArgs)
    a.batch = prefix_lens.numel()
    a.draft_len = draft_len
    a.hq = q.shape[1]
    a.hkv = k_cache.shape[1]
    a.qk_dim = qk_dim
    a.v_dim = v_dim
    a.page_size = page_size
    a.kv_dtype = kv_dtype
    a.k_scale = k_scale
    a.v_scale = v_scale
    a.sm_scale = sm_scale
    a.window_left = window_left
    a.max_prefix_len = max_prefix_len
    a.num_splits = num_splits
    a.q = _ptr(q)
    a.q_stride_row, a.q_stride_head = q.stride(0), q.stride(1)
    a.k_cache = _ptr(k_cache)
    a.k_stride_slot, a.k_stride_head = k_cache.stride(0), k_cache.stride(1)
    a.v_cache = _ptr(v_cache)
    a.v_stride_slot, a.v_stride_head = v_cache.stride(0), v_cache.stride(1)
    a.block_table = _ptr(block_table)
    a.max_pages_per_seq = block_table.shape[1]
    a.prefix_lens = _ptr(prefix_lens)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.out = _ptr(out)
    a.o_stride_row, a.o_stride_head = out.stride(0), out.stride(1)
    a.lse = _ptr(lse)
    a.qo_indptr = _ptr(qo_indptr)
    a.draft_slots = _ptr(draft_slots)
    a.tree_mask = _ptr(tree_mask)
    a.sinks = _ptr(sinks)
    a.logit_cap = float(logit_cap)
    return VerifyCall(a, dict(q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                              prefix_lens=prefix_lens, out=out, workspace=workspace, lse=lse,
                              qo_indptr=qo_indptr, draft_slots=draft_slots, tree_mask=tree_mask,
                              sinks=sinks))


def verify_attn_fwd(call: VerifyCall, stream=None, check=True) -> int:
    st = load().verify_attn_fwd(ctypes.byref(call.args), _stream_ptr(stream))
    if check:
        _check("verify_attn_fwd", st)
    return st


def verify_attn_combine(call: VerifyCall, stream=None, check=True) -> int:
    st = load().verify_attn_combine(ctypes.byref(call.args), _stream_ptr(stream))
    if check:
        _check("verify_attn_combine", st)
    return st


def verify_attn_can_handle(call: VerifyCall) -> int:
    return load().verify_attn_can_handle(ctypes.byref(call.args))


def verify_attn_num_splits(call: VerifyCall) -> int:
    """The heuristic's split count for these arguments (host only; -1 if rejected)."""
    return load().verify_attn_num_splits(ctypes.byref(call.args))


def set_workspace(call: VerifyCall, workspace) -> None:
    """Point an existing call at a (new) workspace tensor."""
    call.args.workspace = _ptr(workspace)
    call.args.workspace_bytes = workspace.numel() * workspace.element_size()
    call.tensors["workspace"] = workspace


def verify_attn_translate_slots(slots, full_to_swa, out=None, stream=None, check=True):
    """out[i] = full_to_swa[slots[i]] on the GPU (int32 tensors); returns out."""
    import torch
    if out is None:
        out = torch.empty_like(slots)
    st = load().verify_attn_translate_slots(_ptr(slots), slots.numel(), _ptr(full_to_swa),
                                            full_to_swa.numel(), _ptr(out), _stream_ptr(stream))
    if not check:
        return st
    _check("verify_attn_translate_slots", st)
    return out


def verify_attn_workspace_bytes(batch, hkv, hq, draft_len, v_dim, num_splits) -> int:
    return load().verify_attn_workspace_bytes(batch, hkv, hq, draft_len, v_dim, num_splits)
