"""The library through its C ABI from a plain C program (tests/c_abi/verify_c_caller.c,
compiled with the host C compiler against include/verify_attn.h and the HIP runtime's
C API): the host-only calls on the CPU, and one verify call on the GPU compared with
the oracle on the same inputs (drawn by tests/c_abi/inputs.py from the same seeded
stream the C program draws)."""

import os
import subprocess

import numpy as np
import pytest

import oracle
from c_abi import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_caller_host_calls(tmp_path):
    from speculative_decoding_verify_02_amd import binding
    from speculative_decoding_verify_02_amd import build as build_mod
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("library not built")
    try:
        exe = build_mod.build_c_caller(str(tmp_path / "verify_c_caller"))
    except RuntimeError as e:
        pytest.skip(f"cannot build the C caller: {e}")
    res = subprocess.run([exe, "abi"], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    got = dict(line.split("=", 1) for line in res.stdout.split())
    rows = (inputs.HQ // inputs.HKV) * inputs.D
    assert got == {
        "abi_version": "2",
        "strerror_ok": "ok",
        # partial outputs and LSEs of 4 slots, then one piece count per sequence
        "workspace_bytes_s4": str((inputs.B * inputs.HKV * 4 * rows * (inputs.DIM + 1) + inputs.B) * 4),
        "workspace_bytes_bad": "-1",        # hq not a multiple of hkv
        "can_handle": str(binding.VA_OK),
        "num_splits_positive": "1",
        "can_handle_draft9": str(binding.VA_EUNSUPPORTED),
        "can_handle_dim96": str(binding.VA_EUNSUPPORTED),
        "can_handle_null_q": str(binding.VA_EINVAL),
        "fwd_small_workspace": str(binding.VA_EWORKSPACE),
    }


def _read_inputs(path, p):
    raw = np.fromfile(path, dtype=np.uint8)
    parts, off = [], 0
    for name, dt in (("kv_indices", np.int32), ("q", np.uint16), ("k_cache", np.uint16),
                     ("v_cache", np.uint16)):
        nbytes = p[name].size * np.dtype(dt).itemsize
        parts.append(raw[off:off + nbytes].view(dt))
        off += nbytes
    assert off == raw.size
    return parts


def test_c_caller_draws_the_same_inputs(tmp_path):
    # the C program's generator against this module's, value for value
    from speculative_decoding_verify_02_amd import binding
    from speculative_decoding_verify_02_amd import build as build_mod
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("library not built")
    try:
        exe = build_mod.build_c_caller(str(tmp_path / "verify_c_caller"))
    except RuntimeError as e:
        pytest.skip(f"cannot build the C caller: {e}")
    path = str(tmp_path / "inputs.bin")
    res = subprocess.run([exe, "inputs", path], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    p = inputs.problem()
    idx, q, k, v = _read_inputs(path, p)
    assert np.array_equal(idx, p["kv_indices"])
    assert np.array_equal(q, p["q"].ravel())
    assert np.array_equal(k, p["k_cache"].ravel()) and np.array_equal(v, p["v_cache"].ravel())


@pytest.mark.gpu
def test_c_caller_matches_oracle(tmp_path):
    from speculative_decoding_verify_02_amd import build as build_mod
    exe = build_mod.C_CALLER_PATH
    if not os.path.exists(exe):
        pytest.fail(f"{exe} is missing: build it first (__graft_entry__.build())")
    out_file = str(tmp_path / "result.bin")
    print("[case] C caller: B 3, L 0/17/100, D 4, hq 8, hkv 2, d 128, P 4, bf16", flush=True)
    res = subprocess.run([exe, "run", out_file], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    p = inputs.problem()
    B, D, HQ, DIM = inputs.B, inputs.D, inputs.HQ, inputs.DIM
    raw = np.fromfile(out_file, dtype=np.uint8)
    head = raw[:12].view(np.int32)
    assert list(head[:2]) == [B, p["max_pages"]] and head[2] >= 1
    off = 12
    nbt = B * p["max_pages"]
    bt = raw[off:off + 4 * nbt].view(np.int32).reshape(B, -1)
    off += 4 * nbt
    lens = raw[off:off + 4 * B].view(np.int32)
    off += 4 * B
    out = raw[off:off + 2 * B * D * HQ * DIM].view(np.uint16).reshape(B * D, HQ, DIM)
    off += 2 * B * D * HQ * DIM
    lse = raw[off:off + 4 * B * D * HQ].view(np.float32).reshape(B * D, HQ)
    assert off + 4 * B * D * HQ == raw.size

    bt_ref, lens_ref = oracle.block_table(p["kv_indptr"], p["kv_indices"], inputs.PAGE,
                                          p["max_pages"])
    assert np.array_equal(bt, bt_ref) and np.array_equal(lens, lens_ref)
    O_ref, LSE_ref = oracle.verify_attention(
        q=p["q"], k_cache=p["k_cache"], v_cache=p["v_cache"], kv_indptr=p["kv_indptr"],
        kv_indices=p["kv_indices"], prefix_lens=p["prefix_lens"], draft_len=D, hq=HQ,
        hkv=inputs.HKV, qk_dim=DIM, v_dim=DIM, sm_scale=1.0 / np.sqrt(np.float32(DIM)))
    O = oracle.bf16_to_f64(out)
    ok_o, err_o, _ = oracle.allclose_report(O, O_ref, 1e-2, 1e-2)
    ok_l, err_l, _ = oracle.allclose_report(lse.astype(np.float64), LSE_ref, 1e-3, 1e-3)
    print(f"   max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
    assert ok_o and ok_l
