"""The binding's host-side debug validator (CPU): each precondition the kernels trust
(include/verify_attn.h) is fed a violation and must raise before anything is launched.

The tensors here live on the CPU, so a call that got past the validator would hand
host pointers to the library; every violating call below raises first, and the valid
ones only run the validator functions themselves."""

import numpy as np
import pytest
import torch

from speculative_decoding_verify_02_amd import binding as B
from speculative_decoding_verify_02_amd import workloads as W


def problem(**kw):
    base = dict(name="validator", batch=3, prefix_lens=[5, 40, 17], hq=4, hkv=2, qk_dim=128,
                page_size=4, seed=5)
    base.update(kw)
    return W.make_problem(**base)


def table(p):
    import oracle
    return oracle.run_block_table(p)[0]


def cpu_call(p, bt=None, **over):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    q = t(p.q.view(np.int16)).view(torch.bfloat16)
    k = t(p.k_cache.view(np.int16)).view(torch.bfloat16)
    v = k if p.v_cache is None else t(p.v_cache.view(np.int16)).view(torch.bfloat16)
    bt = t(table(p) if bt is None else bt).to(torch.int32)
    kw = dict(q=q, k_cache=k, v_cache=v, block_table=bt,
              prefix_lens=t(p.prefix_lens.astype(np.int32)), draft_len=p.draft_len,
              page_size=p.page_size, sm_scale=p.sm_scale, max_prefix_len=p.max_prefix_len,
              out=torch.empty((p.rows, p.hq, p.v_dim), dtype=torch.bfloat16), workspace=None,
              qo_indptr=None if p.qo_indptr is None else t(p.qo_indptr),
              draft_slots=None if p.draft_slots is None else t(p.draft_slots),
              tree_mask=None if p.tree_mask is None else t(p.tree_mask))
    kw.update(over)
    return B.make_args(**kw)


@pytest.fixture
def validating():
    B.set_debug_validation(True)
    yield
    B.set_debug_validation(False)


def test_off_by_default():
    assert not B.debug_validation()


def test_valid_inputs_pass():
    for kw in (dict(), dict(page_size=1), dict(page_size=16), dict(ragged=True),
               dict(tree=True), dict(prefix_lens=[0, 0, 3])):
        p = problem(**kw)
        B.validate_block_table_inputs(p.kv_indptr, p.kv_indices, p.page_size,
                                      p.max_pages_per_seq, num_slots=p.num_slots)
        B.validate_call(cpu_call(p), kv_indptr=p.kv_indptr)


def bt_violation(p, mutate):
    ind, idx = p.kv_indptr.copy(), p.kv_indices.copy()
    mutate(ind, idx)
    return ind, idx


@pytest.mark.parametrize("what", ["indptr0", "decreasing", "short_indices", "slot_range",
                                  "page_offset", "non_consecutive", "table_width"])
def test_block_table_violations_raise_before_launch(validating, what):
    p = problem()
    ind, idx, mp, ns = p.kv_indptr.copy(), p.kv_indices.copy(), p.max_pages_per_seq, p.num_slots
    P = p.page_size
    if what == "indptr0":
        ind = ind + 1
    elif what == "decreasing":
        ind[2] = ind[1] - 1
    elif what == "short_indices":
        idx = idx[:-1]
    elif what == "slot_range":
        idx[3] = ns
    elif what == "page_offset":
        s = ind[1]
        idx[s:s + P] = idx[s:s + P] + 1          # sequence 1 starts at offset 1 of its page
    elif what == "non_consecutive":
        s = ind[1]
        idx[s + 1], idx[s + 2] = idx[s + 2], idx[s + 1]
    elif what == "table_width":
        mp = 2
    with pytest.raises(B.VerifyAttnInputError):
        B.validate_block_table_inputs(ind, idx, P, mp, num_slots=ns)
    # through the binding: the validator raises before the library is called
    with pytest.raises(B.VerifyAttnInputError):
        B.verify_attn_build_block_table(torch.from_numpy(ind.astype(np.int32)),
                                        torch.from_numpy(idx.astype(np.int32)), P, mp,
                                        block_table=torch.zeros((3, max(mp, 1)), dtype=torch.int32),
                                        kv_lens=torch.zeros(3, dtype=torch.int32))


@pytest.mark.parametrize("what", ["negative_len", "table_narrow", "page_outside_pool",
                                  "page_negative", "indptr_mismatch", "qo_start",
                                  "qo_too_many_rows", "qo_beyond_q", "draft_slot_outside"])
def test_forward_violations_raise_before_launch(validating, what):
    kw = {}
    if what.startswith("qo"):
        kw = dict(ragged=True)
    if what == "draft_slot_outside":
        kw = dict(tree=True)
    p = problem(**kw)
    bt = table(p)
    over = {}
    ind = p.kv_indptr
    if what == "negative_len":
        L = p.prefix_lens.copy()
        L[1] = -1
        over["prefix_lens"] = torch.from_numpy(L)
    elif what == "table_narrow":
        bt = bt[:, :3].copy()
    elif what == "page_outside_pool":
        bt[2, 1] = p.num_pages
    elif what == "page_negative":
        bt[0, 0] = -1
    elif what == "indptr_mismatch":
        ind = ind.copy()
        ind[2:] += 1
    elif what == "qo_start":
        qo = p.qo_indptr.copy()
        qo[0] = 1
        over["qo_indptr"] = torch.from_numpy(qo)
    elif what == "qo_too_many_rows":
        qo = p.qo_indptr.copy()
        qo[1:] += p.draft_len + 1
        over["qo_indptr"] = torch.from_numpy(qo)
    elif what == "qo_beyond_q":
        qo = p.qo_indptr.copy()
        qo[-1] += 1
        over["qo_indptr"] = torch.from_numpy(qo)
    elif what == "draft_slot_outside":
        ds = p.draft_slots.copy()
        ds[1, 2] = p.num_slots
        over["draft_slots"] = torch.from_numpy(ds)
    call = cpu_call(p, bt=bt, **over)
    if what == "indptr_mismatch":
        with pytest.raises(B.VerifyAttnInputError):
            B.validate_call(call, kv_indptr=ind)
        return
    with pytest.raises(B.VerifyAttnInputError):
        B.validate_call(call)
    with pytest.raises(B.VerifyAttnInputError):
        B.verify_attn_fwd(call)
    with pytest.raises(B.VerifyAttnInputError):
        B.verify_attn_combine(call)
