"""ctypes binding of libverify_attn.so (argument marshalling only).

Every step of the verify path runs in the library's HIP kernels; this module
turns torch tensors into the pointers, strides and scalars the C ABI of
``include/verify_attn.h`` takes.  PyTorch provides device memory and the
current stream, nothing else.  If the library is missing the functions raise:
there is no CPU or PyTorch fallback.  An optional host-side validator (off by
default, ``set_debug_validation``) checks the device data the kernels trust
before a launch.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; VERIFY_ATTN_LIB names another build of the same sources (the
# host-sanitizer build the CPU tests load, for instance)
LIB_PATH = os.environ.get("VERIFY_ATTN_LIB") or os.path.join(PKG, "libverify_attn.so")

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
    "verify_attn_fwd_combine_noalloc",
)

# bytes of the static per-device array verify_attn_fwd_combine_noalloc uses
STATIC_SCRATCH_BYTES = 64 << 20


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


class VerifyAttnInputError(ValueError):
    """A precondition of include/verify_attn.h that the kernels trust is broken (raised by
    the optional host-side validator before anything is launched)."""


# Host-side debug validation of the device inputs the kernels trust (page ids inside the
# pool, consecutive slots within a page, block-table width, row offsets).  Off by
# default: it copies those tensors to the host and synchronises.  A bad page id is a GPU
# memory fault, not a status code (the unified-attention page splits HSA memory-access
# faults out as their own fix), so a caller can switch this on while integrating.
_debug_validate = os.environ.get("VERIFY_ATTN_DEBUG_VALIDATE", "0") == "1"


def set_debug_validation(on: bool) -> None:
    """Switch the host-side validator for build_block_table / fwd / combine on or off."""
    global _debug_validate
    _debug_validate = bool(on)


def debug_validation() -> bool:
    return _debug_validate


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
    for name in ("verify_attn_fwd", "verify_attn_combine", "verify_attn_fwd_combine_noalloc"):
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

def _host(t):
    import numpy as np
    return None if t is None else np.asarray(t.detach().cpu().numpy())


def validate_block_table_inputs(kv_indptr, kv_indices, page_size: int, max_pages_per_seq: int,
                                num_slots: Optional[int] = None) -> None:
    """Host check of verify_attn_build_block_table's preconditions (NumPy arrays or
    tensors): kv_indptr starts at 0 and never decreases, kv_indices holds its entries,
    every slot lies in the pool, each sequence starts at offset 0 of a page and the
    slots of one page are consecutive (true at topk = 1, the page-size page's review),
    and no sequence needs more pages than the table is wide.  Raises
    VerifyAttnInputError naming the first violation."""
    import numpy as np
    ind = np.asarray(_host(kv_indptr) if hasattr(kv_indptr, "cpu") else kv_indptr, dtype=np.int64)
    idx = np.asarray(_host(kv_indices) if hasattr(kv_indices, "cpu") else kv_indices,
                     dtype=np.int64)
    if ind.ndim != 1 or ind.size < 1:
        raise VerifyAttnInputError("kv_indptr must be a 1-D array of batch + 1 entries")
    if ind[0] != 0:
        raise VerifyAttnInputError(f"kv_indptr[0] = {ind[0]}, must be 0")
    n = np.diff(ind)
    if (n < 0).any():
        b = int(np.argmax(n < 0))
        raise VerifyAttnInputError(f"kv_indptr decreases at sequence {b}")
    if ind[-1] > idx.size:
        raise VerifyAttnInputError(f"kv_indptr[B] = {ind[-1]} exceeds the {idx.size} kv_indices")
    used = idx[:ind[-1]]
    if used.size and (used.min() < 0 or (num_slots is not None and used.max() >= num_slots)):
        raise VerifyAttnInputError(f"a slot in kv_indices lies outside the pool of {num_slots} slots")
    pages = -(-n // page_size)
    if pages.size and pages.max() > max_pages_per_seq:
        b = int(np.argmax(pages))
        raise VerifyAttnInputError(f"sequence {b} needs {pages[b]} pages, the table has "
                                   f"{max_pages_per_seq} columns")
    for b in range(n.size):
        s = idx[ind[b]:ind[b + 1]]
        t = np.arange(s.size)
        if (s % page_size != t % page_size).any():
            raise VerifyAttnInputError(f"sequence {b}: a token's slot is not at its offset in a "
                                       f"page (sequences start at offset 0 of a page)")
        first = s[t - t % page_size]
        if (s != first + t % page_size).any():
            raise VerifyAttnInputError(f"sequence {b}: the slots of one page are not consecutive")


def validate_call(call: "VerifyCall", kv_indptr=None) -> None:
    """Host check of the device data verify_attn_fwd and verify_attn_combine trust: prefix
    lengths >= 0, ragged row offsets (from 0, non-decreasing, at most draft_len rows per
    sequence, within q), block-table columns enough for every sequence's keys, page ids
    of those columns inside the K and V pools, tree-verify draft slots inside the pools,
    and (when the token-level kv_indptr the table came from is given) that sequence b
    holds L_b + n_b tokens (L_b at tree verify).  Raises VerifyAttnInputError."""
    import numpy as np
    a, t = call.args, call.tensors
    B, D, P = a.batch, a.draft_len, a.page_size
    if B == 0:
        return
    L = np.asarray(_host(t["prefix_lens"]), dtype=np.int64).reshape(-1)
    if L.size != B:
        raise VerifyAttnInputError(f"prefix_lens has {L.size} entries for batch {B}")
    if (L < 0).any():
        raise VerifyAttnInputError(f"prefix_lens[{int(np.argmax(L < 0))}] is negative")
    q_rows = t["q"].shape[0]
    if t.get("qo_indptr") is not None:
        qo = np.asarray(_host(t["qo_indptr"]), dtype=np.int64).reshape(-1)
        if qo.size != B + 1 or qo[0] != 0:
            raise VerifyAttnInputError("qo_indptr must hold batch + 1 offsets starting at 0")
        nr = np.diff(qo)
        if (nr < 0).any() or (nr > D).any():
            raise VerifyAttnInputError("qo_indptr must not decrease and gives at most draft_len "
                                       "rows per sequence")
        if qo[-1] > q_rows:
            raise VerifyAttnInputError(f"qo_indptr[B] = {qo[-1]} exceeds the {q_rows} rows of q")
    else:
        nr = np.full(B, D, dtype=np.int64)
        if B * D > q_rows:
            raise VerifyAttnInputError(f"q has {q_rows} rows, batch x draft_len = {B * D}")
    tree = t.get("draft_slots") is not None
    keys = L if tree else L + nr
    keys = np.where(nr > 0, keys, 0)   # a sequence without rows reads nothing
    bt = np.asarray(_host(t["block_table"]), dtype=np.int64)
    if bt.ndim != 2 or bt.shape[0] < B or bt.shape[1] != a.max_pages_per_seq:
        raise VerifyAttnInputError("block_table must be [batch, max_pages_per_seq]")
    pages = -(-keys // P)
    if pages.max() > a.max_pages_per_seq:
        b = int(np.argmax(pages))
        raise VerifyAttnInputError(f"sequence {b} needs {pages[b]} pages, the table has "
                                   f"{a.max_pages_per_seq} columns")
    k_slots = t["k_cache"].shape[0]
    v_slots = t["v_cache"].shape[0]
    pool_pages = min(k_slots, v_slots) // P
    for b in range(B):
        ids = bt[b, :pages[b]]
        if ids.size and (ids.min() < 0 or ids.max() >= pool_pages):
            raise VerifyAttnInputError(f"sequence {b}: a page id in the block table lies outside "
                                       f"the pool of {pool_pages} pages")
    if tree:
        ds = np.asarray(_host(t["draft_slots"]), dtype=np.int64)
        if ds.size < B * D or ds[:B * D].min() < 0 or ds[:B * D].max() >= min(k_slots, v_slots):
            raise VerifyAttnInputError("draft_slots must hold [batch, draft_len] slots inside the pool")
    if kv_indptr is not None:
        ind = np.asarray(_host(kv_indptr) if hasattr(kv_indptr, "cpu") else kv_indptr,
                         dtype=np.int64).reshape(-1)
        if ind.size != B + 1:
            raise VerifyAttnInputError(f"kv_indptr has {ind.size} entries for batch {B}")
        bad = (nr > 0) & (np.diff(ind) != keys)
        if bad.any():
            b = int(np.argmax(bad))
            raise VerifyAttnInputError(f"sequence {b}: kv_indptr gives {int(ind[b + 1] - ind[b])} "
                                       f"tokens, prefix_lens and the draft rows give {keys[b]}")


def verify_attn_build_block_table(kv_indptr, kv_indices, page_size: int, max_pages_per_seq: int,
                                  block_table=None, kv_lens=None, stream=None, check=True):
    """Scatter token-level slots into a [B, max_pages] int32 page table (on the GPU).

    ``kv_indptr`` [B+1] and ``kv_indices`` int32 CUDA tensors.  Allocates the outputs
    when not given.  Returns (block_table, kv_lens) or the raw status if check=False.
    With debug validation on, the inputs are checked on the host first."""
    import torch
    if _debug_validate:
        validate_block_table_inputs(kv_indptr, kv_indices, page_size, max_pages_per_seq)
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
    if _debug_validate:
        validate_call(call)
    st = load().verify_attn_fwd(ctypes.byref(call.args), _stream_ptr(stream))
    if check:
        _check("verify_attn_fwd", st)
    return st


def verify_attn_combine(call: VerifyCall, stream=None, check=True) -> int:
    if _debug_validate:
        validate_call(call)
    st = load().verify_attn_combine(ctypes.byref(call.args), _stream_ptr(stream))
    if check:
        _check("verify_attn_combine", st)
    return st


def verify_attn_fwd_combine_noalloc(call: VerifyCall, stream=None, check=True) -> int:
    """fwd + combine with the library's static per-device scratch instead of the call's
    workspace (for callers that cannot allocate); calls overlapping on one GPU race."""
    if _debug_validate:
        validate_call(call)
    st = load().verify_attn_fwd_combine_noalloc(ctypes.byref(call.args), _stream_ptr(stream))
    if check:
        _check("verify_attn_fwd_combine_noalloc", st)
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
