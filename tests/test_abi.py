"""The C ABI on the CPU: the library loads, exports every declared symbol, and its
host-only gate returns the documented statuses without launching anything.

No call here reaches a kernel launch: every argument set is rejected before the
launch, or batch = 0 (nothing to launch), or the call is host-only."""

import ctypes
import os
import re

import pytest

from speculative_decoding_verify_02_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # 16-byte aligned non-null address; never dereferenced by these calls


def header_functions():
    text = open(os.path.join(ROOT, "include", "verify_attn.h")).read()
    return sorted(set(re.findall(r"\b(verify_attn_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = B.load()
    declared = header_functions()
    assert set(declared) == set(B.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.verify_attn_abi_version() == 2


def fake_args(**kw):
    a = B.VerifyAttnArgs()
    a.struct_size = ctypes.sizeof(B.VerifyAttnArgs)
    a.batch, a.draft_len, a.hq, a.hkv = 2, 4, 8, 2
    a.qk_dim = a.v_dim = 128
    a.page_size = 16
    a.kv_dtype = B.VA_KV_BF16
    a.k_scale = a.v_scale = 1.0
    a.sm_scale = 0.088
    a.window_left = -1
    a.max_prefix_len = 1000
    a.num_splits = 4
    a.q = a.k_cache = a.v_cache = a.block_table = a.prefix_lens = a.workspace = a.out = FAKE
    a.q_stride_row, a.q_stride_head = 8 * 128, 128
    a.k_stride_slot, a.k_stride_head = 2 * 128, 128
    a.v_stride_slot, a.v_stride_head = 2 * 128, 128
    a.max_pages_per_seq = 70
    a.workspace_bytes = 0
    a.o_stride_row, a.o_stride_head = 8 * 128, 128
    a.lse = None
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def can_handle(**kw):
    return B.load().verify_attn_can_handle(ctypes.byref(fake_args(**kw)))


def fwd(**kw):
    return B.load().verify_attn_fwd(ctypes.byref(fake_args(**kw)), None)


def combine(**kw):
    return B.load().verify_attn_combine(ctypes.byref(fake_args(**kw)), None)


def test_gate_accepts_supported_shapes():
    assert can_handle() == B.VA_OK
    assert can_handle(qk_dim=256, v_dim=256, k_stride_head=256, v_stride_head=256,
                      k_stride_slot=512, v_stride_slot=512) == B.VA_OK
    assert can_handle(qk_dim=256, v_dim=256) == B.VA_EINVAL       # rows overlap
    assert can_handle(qk_dim=576, v_dim=512, hq=16, hkv=1, kv_dtype=B.VA_KV_FP8_E4M3FN,
                      k_scale=0.05, v_scale=0.05, k_stride_slot=576, k_stride_head=576,
                      v_stride_slot=576, v_stride_head=576) == B.VA_OK
    assert can_handle(page_size=1) == B.VA_OK and can_handle(page_size=1024) == B.VA_OK
    assert can_handle(window_left=0) == B.VA_OK and can_handle(draft_len=8) == B.VA_OK
    assert can_handle(num_splits=0) == B.VA_OK          # heuristic, host only


@pytest.mark.parametrize("kw,status", [
    (dict(struct_size=8), B.VA_EINVAL),
    (dict(q=None), B.VA_EINVAL),
    (dict(k_cache=None), B.VA_EINVAL),
    (dict(workspace=None), B.VA_EINVAL),
    (dict(out=None), B.VA_EINVAL),
    (dict(block_table=None), B.VA_EINVAL),
    (dict(prefix_lens=None), B.VA_EINVAL),
    (dict(hq=7), B.VA_EINVAL),                          # hq % hkv != 0
    (dict(batch=-1), B.VA_EINVAL),
    (dict(draft_len=0), B.VA_EINVAL),
    (dict(window_left=-2), B.VA_EINVAL),
    (dict(q=FAKE + 2), B.VA_EINVAL),                    # misaligned rows
    (dict(k_stride_slot=2 * 128 + 4), B.VA_EINVAL),
    (dict(sm_scale=float("nan")), B.VA_EINVAL),
    (dict(k_scale=0.5), B.VA_EINVAL),                   # scales must be 1 for bf16
    (dict(kv_dtype=7), B.VA_EINVAL),
    (dict(struct_size=B.V1_SIZE + 4), B.VA_EINVAL),     # neither layout
    (dict(draft_slots=FAKE), B.VA_EINVAL),              # a tree needs its mask
    (dict(tree_mask=FAKE), B.VA_EINVAL),
    (dict(logit_cap=-1.0), B.VA_EINVAL),
    (dict(logit_cap=float("inf")), B.VA_EINVAL),
    (dict(draft_slots=FAKE, tree_mask=FAKE, window_left=8), B.VA_EUNSUPPORTED),
    (dict(draft_slots=FAKE, tree_mask=FAKE, qo_indptr=FAKE), B.VA_EUNSUPPORTED),
    (dict(draft_len=9), B.VA_EUNSUPPORTED),
    (dict(qk_dim=64, v_dim=64), B.VA_EUNSUPPORTED),
    (dict(qk_dim=128, v_dim=256), B.VA_EUNSUPPORTED),
    (dict(page_size=3), B.VA_EUNSUPPORTED),
    (dict(page_size=2048), B.VA_EUNSUPPORTED),
    (dict(hq=64, hkv=1, draft_len=4), B.VA_EUNSUPPORTED),   # 256 rows per KV head
    (dict(k_stride_slot=1 << 31), B.VA_EUNSUPPORTED),       # 4 GiB slot rows (bf16)
    (dict(v_stride_slot=1 << 31), B.VA_EUNSUPPORTED),
    # the combine's grid takes batch and hkv as dimensions of at most 65535
    (dict(batch=65536), B.VA_EUNSUPPORTED),
    (dict(hq=65536, hkv=65536), B.VA_EUNSUPPORTED),
    (dict(batch=65536, num_splits=1), B.VA_EUNSUPPORTED),
])
def test_gate_rejects(kw, status):
    assert can_handle(**kw) == status
    assert fwd(**kw) == status          # nothing launched: rejected before the launch
    assert combine(**kw) == status


def test_largest_grid_dimensions_accepted():
    assert can_handle(batch=65535) == B.VA_OK
    assert can_handle(hq=65535, hkv=65535, draft_len=1) == B.VA_OK
    lib = B.load()
    assert lib.verify_attn_num_splits(ctypes.byref(fake_args(batch=65536))) == -1
    assert lib.verify_attn_num_splits(ctypes.byref(fake_args(batch=65535))) >= 1


def test_fp8_latent_head_with_separate_v_cache_is_served():
    # fp8 576/512 with a V cache that is not a view of the K rows is a valid request
    # (served by the generic kernel, not the one that reads V from the K rows)
    mla = dict(qk_dim=576, v_dim=512, hq=16, hkv=1, kv_dtype=B.VA_KV_FP8_E4M3FN, k_scale=0.05,
               v_scale=0.05, k_stride_slot=576, k_stride_head=576)
    assert can_handle(**mla, v_stride_slot=576, v_stride_head=576) == B.VA_OK
    assert can_handle(**mla, v_cache=FAKE + 0x100000, v_stride_slot=512, v_stride_head=512) == B.VA_OK


def noalloc(**kw):
    return B.load().verify_attn_fwd_combine_noalloc(ctypes.byref(fake_args(**kw)), None)


def test_noalloc_rejects_before_any_launch():
    # the same argument checks as fwd; the caller's workspace fields are ignored
    assert noalloc(q=None) == B.VA_EINVAL
    assert noalloc(draft_len=9) == B.VA_EUNSUPPORTED
    assert noalloc(batch=0, workspace=None, workspace_bytes=0) == B.VA_OK
    # partials beyond the static array: an explicit slot count that does not fit, and a
    # batch for which not even one slot per sequence fits (2000 x 2 x 16 rows x 513 x 4 B)
    per_slot = B.verify_attn_workspace_bytes(2, 2, 8, 4, 128, 1) - 2 * 4
    fit = (B.STATIC_SCRATCH_BYTES - 8) // per_slot
    assert noalloc(num_splits=fit + 1) == B.VA_EWORKSPACE
    assert noalloc(batch=2000, qk_dim=576, v_dim=512, hq=16, hkv=1, kv_dtype=B.VA_KV_FP8_E4M3FN,
                   k_scale=0.05, v_scale=0.05, k_stride_slot=576, k_stride_head=576,
                   v_stride_slot=576, v_stride_head=576, num_splits=0) == B.VA_EWORKSPACE


def test_workspace_checked_before_launch():
    need = B.verify_attn_workspace_bytes(2, 2, 8, 4, 128, 4)
    assert need == (2 * 2 * 4 * 16 * 129 + 2) * 4     # partials + one piece count per sequence
    assert fwd(workspace_bytes=need - 1) == B.VA_EWORKSPACE
    assert combine(workspace_bytes=need - 1) == B.VA_EWORKSPACE


def test_empty_batch_launches_nothing():
    kw = dict(batch=0, q=None, k_cache=None, v_cache=None, block_table=None, prefix_lens=None,
              workspace=None, out=None, workspace_bytes=0)
    assert fwd(**kw) == B.VA_OK and combine(**kw) == B.VA_OK
    lib = B.load()
    assert lib.verify_attn_build_block_table(None, None, 0, 4, 1, None, None, None) == B.VA_OK


def test_block_table_arguments():
    lib = B.load()
    assert lib.verify_attn_build_block_table(FAKE, FAKE, -1, 4, 4, FAKE, None, None) == B.VA_EINVAL
    assert lib.verify_attn_build_block_table(FAKE, FAKE, 2, 4, 0, FAKE, None, None) == B.VA_EINVAL
    assert lib.verify_attn_build_block_table(FAKE, FAKE, 2, 6, 4, FAKE, None, None) == B.VA_EUNSUPPORTED
    assert lib.verify_attn_build_block_table(None, FAKE, 2, 4, 4, FAKE, None, None) == B.VA_EINVAL


def test_host_helpers():
    assert B.verify_attn_workspace_bytes(1, 1, 1, 1, 128, 0) == -1
    assert B.verify_attn_workspace_bytes(1, 2, 3, 1, 128, 1) == -1     # hq % hkv
    lib = B.load()
    for kw in [dict(), dict(max_prefix_len=0), dict(batch=0, max_prefix_len=70000),
               dict(qk_dim=576, v_dim=512, hq=16, hkv=1, kv_dtype=B.VA_KV_FP8_E4M3FN,
                    k_scale=0.05, v_scale=0.05, k_stride_slot=576, k_stride_head=576,
                    v_stride_slot=576, v_stride_head=576),
               dict(num_splits=3)]:
        s = lib.verify_attn_num_splits(ctypes.byref(fake_args(**kw)))
        assert s >= 1, kw
    # host-only sizing query: pointers may still be unset
    assert lib.verify_attn_num_splits(ctypes.byref(fake_args(workspace=None, q=None, out=None))) >= 1
    assert lib.verify_attn_num_splits(ctypes.byref(fake_args(max_prefix_len=-5))) == -1
    assert lib.verify_attn_num_splits(ctypes.byref(fake_args(hq=7))) == -1
    for st in range(6):
        assert isinstance(B.strerror(st), str)


def test_version1_layout_still_accepted():
    # a caller built against the version 1 header passes the shorter struct size;
    # the extension fields then read as off, whatever lies past its struct
    a = fake_args(struct_size=B.V1_SIZE, draft_slots=FAKE, logit_cap=-5.0)
    assert B.load().verify_attn_can_handle(ctypes.byref(a)) == B.VA_OK
    assert B.load().verify_attn_num_splits(ctypes.byref(a)) >= 1


def test_extensions_accepted():
    assert can_handle(qo_indptr=FAKE) == B.VA_OK
    assert can_handle(draft_slots=FAKE, tree_mask=FAKE) == B.VA_OK
    assert can_handle(sinks=FAKE, logit_cap=30.0) == B.VA_OK


def test_translate_slots_arguments():
    lib = B.load()
    assert lib.verify_attn_translate_slots(None, 0, None, 1, None, None) == B.VA_OK
    assert lib.verify_attn_translate_slots(FAKE, -1, FAKE, 1, FAKE, None) == B.VA_EINVAL
    assert lib.verify_attn_translate_slots(FAKE, 4, FAKE, 0, FAKE, None) == B.VA_EINVAL
    assert lib.verify_attn_translate_slots(None, 4, FAKE, 8, FAKE, None) == B.VA_EINVAL
    assert lib.verify_attn_translate_slots(FAKE, 4, FAKE, 8, None, None) == B.VA_EINVAL
