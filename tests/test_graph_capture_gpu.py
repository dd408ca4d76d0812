"""HIP-graph capture of the whole step (block table + split-KV pass + combine) on fixed
buffers, replayed with new device lengths, page lists and KV contents.

Every launch decision of the library reads host scalars only, and its workspace is sized
once for the largest batch, so one captured graph serves every later call of the same
batch whose lengths stay within the captured bounds (the split-KV page's can_handle()
gate reads no tensor values; its review keys scratch on a stable max batch and fixed
addresses).  Each replay is checked against the oracle and, bit for bit, against the
same calls run eagerly on the same buffers; eager work and synchronisations sit
between the replays.
"""

import numpy as np
import pytest

from speculative_decoding_verify_02_amd import workloads as W

from test_verify_attn_gpu import DIMS, LSE_TOL, O_TOL, oracle_run

pytestmark = pytest.mark.gpu

# (prefix lengths) per replay; the pool and batch stay fixed
LENGTH_SETS = [[500, 1200, 30, 2000], [2047, 0, 777, 64], [1, 1900, 1900, 333]]
NUM_PAGES = 600
PAGE = 16


def _dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.cuda()


@pytest.mark.parametrize("dims", [0, 1, 2])
def test_graph_replay_with_new_lengths(dims):
    import torch
    from speculative_decoding_verify_02_amd import binding as B
    import oracle

    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    d = DIMS[dims]
    hq, hkv = (16, 1) if d["qk_dim"] == 576 else (8, 2)
    probs = [W.make_problem(name="graph", batch=4, prefix_lens=ls, hq=hq, hkv=hkv,
                            page_size=PAGE, num_pages=NUM_PAGES, seed=1200 + 10 * dims + i,
                            v_mean=1.0, **d)
             for i, ls in enumerate(LENGTH_SETS)]
    p0 = probs[0]
    print(f"[case] graph dims={dims} hq={hq} hkv={hkv} dk={p0.qk_dim}", flush=True)
    max_L = max(int(p.prefix_lens.max()) for p in probs)
    max_pages = -(-(max_L + p0.draft_len) // PAGE)
    max_tokens = max(int(p.kv_indptr[-1]) for p in probs)
    kvdt = None if p0.kv_dtype == W.KV_FP8_E4M3FN else "bf16"

    # fixed buffers, filled from the first problem
    q = _dev(p0.q, "bf16")
    k = _dev(p0.k_cache, kvdt)
    v = k if p0.v_cache is None else _dev(p0.v_cache, kvdt)
    indptr = _dev(p0.kv_indptr.astype(np.int32))
    indices = torch.zeros(max_tokens, dtype=torch.int32, device="cuda")
    indices[:p0.kv_indices.size] = _dev(p0.kv_indices.astype(np.int32))
    lens = _dev(p0.prefix_lens.astype(np.int32))
    bt = torch.empty((p0.batch, max_pages), dtype=torch.int32, device="cuda")
    kv_lens = torch.empty(p0.batch, dtype=torch.int32, device="cuda")
    out = torch.empty((p0.rows, hq, p0.v_dim), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((p0.rows, hq), dtype=torch.float32, device="cuda")
    call = B.make_args(q=q, k_cache=k, v_cache=v, block_table=bt, prefix_lens=lens,
                       draft_len=p0.draft_len, page_size=PAGE, sm_scale=p0.sm_scale,
                       max_prefix_len=max_L, out=out, workspace=None, lse=lse,
                       kv_dtype=p0.kv_dtype, k_scale=p0.k_scale, v_scale=p0.v_scale,
                       qk_dim=p0.qk_dim, v_dim=p0.v_dim)
    splits = B.verify_attn_num_splits(call)
    assert splits >= 1
    ws = torch.empty(B.verify_attn_workspace_bytes(p0.batch, hkv, hq, p0.draft_len, p0.v_dim,
                                                   splits) // 4, dtype=torch.float32, device="cuda")
    B.set_workspace(call, ws)
    call.args.num_splits = splits

    def step():
        B.verify_attn_build_block_table(indptr, indices, PAGE, max_pages, bt, kv_lens)
        B.verify_attn_fwd(call)
        B.verify_attn_combine(call)

    # warm up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(2):
        for p in probs:
            # new inputs into the captured buffers (eager work between replays)
            q.copy_(_dev(p.q, "bf16"))
            k.copy_(_dev(p.k_cache, kvdt))
            if p.v_cache is not None:
                v.copy_(_dev(p.v_cache, kvdt))
            indptr.copy_(_dev(p.kv_indptr.astype(np.int32)))
            indices.zero_()
            indices[:p.kv_indices.size] = _dev(p.kv_indices.astype(np.int32))
            lens.copy_(_dev(p.prefix_lens.astype(np.int32)))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            O_g = out.float().cpu().numpy().astype(np.float64)
            L_g = lse.cpu().numpy().astype(np.float64)
            bt_g = bt.cpu().numpy()
            out.fill_(float("nan"))
            lse.fill_(float("nan"))
            step()                                   # the same calls, eagerly
            torch.cuda.synchronize()
            assert np.array_equal(out.float().cpu().numpy().astype(np.float64), O_g)
            assert np.array_equal(lse.cpu().numpy().astype(np.float64), L_g)
            bt_ref, _ = oracle.block_table(p.kv_indptr, p.kv_indices, PAGE, max_pages)
            assert np.array_equal(bt_g, bt_ref)
            O_ref, L_ref = oracle_run(p)
            tol = O_TOL[p.kv_dtype]
            ok_o, err_o, _ = oracle.allclose_report(O_g, O_ref, tol, tol)
            ok_l, err_l, _ = oracle.allclose_report(L_g, L_ref, LSE_TOL, LSE_TOL)
            print(f"   replay {rep} lens={list(p.prefix_lens)} max|dO|={err_o:.2e} "
                  f"max|dLSE|={err_l:.2e}", flush=True)
            assert ok_o and ok_l
