"""The allocation-free entry point (verify_attn_fwd_combine_noalloc) against the
workspace entry points (verify_attn_fwd + verify_attn_combine) through the C ABI: two
calls in a row on one device, the second with a smaller input (the static array keeps
the first call's contents), each equal bit for bit to the workspace path at the same
slot count and within the parity tolerances of the oracle at the slot count the array
allows."""

import numpy as np
import pytest

from speculative_decoding_verify_02_amd import workloads as W

from test_verify_attn_gpu import LSE_TOL, O_TOL, describe, oracle_run

pytestmark = pytest.mark.gpu


def _outputs(dp):
    import torch
    torch.cuda.synchronize()
    return (dp.out.float().cpu().numpy().astype(np.float64),
            dp.lse.cpu().numpy().astype(np.float64))


def test_noalloc_two_calls_second_smaller():
    import torch
    import oracle
    from speculative_decoding_verify_02_amd import binding as B
    from speculative_decoding_verify_02_amd.runner import DeviceProblem

    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    # the MLA share first (its heuristic slot count, 9, needs 72 MiB of partials: the
    # entry point lowers it to the 7 the 64 MiB array holds), then a small GQA problem
    cases = [W.make_config(4, v_mean=1.0),
             W.make_problem(name="noalloc-small", batch=3, prefix_lens=[40, 900, 5], hq=8,
                            hkv=2, qk_dim=128, page_size=16, seed=1300, v_mean=1.0)]
    for p in cases:
        print(describe(p, entry="noalloc"), flush=True)
        dp = DeviceProblem(p)
        heur = dp.splits
        per_slot = B.verify_attn_workspace_bytes(p.batch, p.hkv, p.hq, p.draft_len, p.v_dim, 1) \
            - 4 * p.batch
        fit = (B.STATIC_SCRATCH_BYTES - 4 * p.batch) // per_slot
        used = min(heur, fit)
        # workspace path at the slot count the static array allows
        dp_ref = DeviceProblem(p, num_splits=used)
        dp_ref.step()
        O_ws, L_ws = _outputs(dp_ref)
        # the allocation-free path: explicit slot count (bit for bit) ...
        call = dp_ref.calls[0]
        dp_ref.out.fill_(float("nan"))
        dp_ref.lse.fill_(float("nan"))
        assert B.verify_attn_fwd_combine_noalloc(call) == B.VA_OK
        O_na, L_na = _outputs(dp_ref)
        assert np.array_equal(O_na, O_ws) and np.array_equal(L_na, L_ws)
        # ... and the heuristic's count (lowered to what fits when needed)
        call.args.num_splits = 0
        dp_ref.out.fill_(float("nan"))
        dp_ref.lse.fill_(float("nan"))
        assert B.verify_attn_fwd_combine_noalloc(call) == B.VA_OK
        O_h, L_h = _outputs(dp_ref)
        assert np.array_equal(O_h, O_ws) and np.array_equal(L_h, L_ws)
        O_ref, L_ref = oracle_run(p)
        tol = O_TOL[p.kv_dtype]
        ok_o, err_o, _ = oracle.allclose_report(O_h, O_ref, tol, tol)
        ok_l, err_l, _ = oracle.allclose_report(L_h, L_ref, LSE_TOL, LSE_TOL)
        print(f"   slots heuristic {heur} static {used}: max|dO|={err_o:.2e} "
              f"max|dLSE|={err_l:.2e}", flush=True)
        assert ok_o and ok_l
        # an explicit slot count beyond the array is refused, nothing launched
        call.args.num_splits = fit + 1
        assert B.verify_attn_fwd_combine_noalloc(call, check=False) == B.VA_EWORKSPACE
        del dp, dp_ref
