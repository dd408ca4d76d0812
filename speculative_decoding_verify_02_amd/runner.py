"""Device-side driver: upload a host Problem once, then run the verify path.

One step = block-table scatter + split-KV pass + combine, all in the library's
HIP kernels on the current torch stream.  Buffers are allocated once (sized
for the problem) and reused, so a step allocates nothing.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from . import binding
from .workloads import KV_FP8_E4M3FN, Problem


def _to_dev(a: np.ndarray, device, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(device)


class DeviceProblem:
    """A Problem resident in HBM plus its output, workspace and block-table buffers."""

    def __init__(self, p: Problem, device="cuda", num_splits: Optional[int] = None,
                 kv_copies: int = 1):
        import torch

        self.p = p
        self.device = torch.device(device)
        dt = None if p.kv_dtype == KV_FP8_E4M3FN else "bf16"
        self.q = _to_dev(p.q, device, "bf16")
        k0 = _to_dev(p.k_cache, device, dt)
        # optional extra copies of the KV pool so consecutive steps read cold memory
        self.k_copies = [k0] + [k0.clone() for _ in range(kv_copies - 1)]
        if p.v_cache is None:
            self.v_copies = list(self.k_copies)
        else:
            v0 = _to_dev(p.v_cache, device, dt)
            self.v_copies = [v0] + [v0.clone() for _ in range(kv_copies - 1)]
        self.kv_indptr = _to_dev(p.kv_indptr.astype(np.int32), device)
        self.kv_indices = _to_dev(p.kv_indices.astype(np.int32), device)
        self.prefix_lens = _to_dev(p.prefix_lens.astype(np.int32), device)
        self.max_pages = p.max_pages_per_seq
        self.block_table = torch.empty((p.batch, self.max_pages), dtype=torch.int32,
                                       device=device)
        self.kv_lens = torch.empty((p.batch,), dtype=torch.int32, device=device)
        self.out = torch.empty((p.rows, p.hq, p.v_dim), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((p.rows, p.hq), dtype=torch.float32, device=device)
        opt = lambda a: None if a is None else _to_dev(np.ascontiguousarray(a), device)
        self.qo_indptr = opt(None if p.qo_indptr is None else p.qo_indptr.astype(np.int32))
        self.draft_slots = opt(None if p.draft_slots is None else p.draft_slots.astype(np.int32))
        self.tree_mask = opt(None if p.tree_mask is None else p.tree_mask.astype(np.uint8))
        self.sinks = opt(None if p.sinks is None else p.sinks.astype(np.float32))
        ns = p.num_splits if num_splits is None else num_splits
        self.workspace = None
        self.calls = [self._make_call(c) for c in range(kv_copies)]
        self.splits = ns if ns > 0 else binding.verify_attn_num_splits(self.calls[0])
        if self.splits < 1:
            raise ValueError(f"arguments rejected (status for {p.name})")
        ws = binding.verify_attn_workspace_bytes(p.batch, p.hkv, p.hq, p.draft_len, p.v_dim,
                                                 self.splits)
        self.workspace = torch.empty((max(ws, 4) + 3) // 4, dtype=torch.float32, device=device)
        for c in self.calls:
            c.args.num_splits = self.splits
            binding.set_workspace(c, self.workspace)

    def _make_call(self, copy: int) -> binding.VerifyCall:
        p = self.p
        return binding.make_args(
            q=self.q, k_cache=self.k_copies[copy], v_cache=self.v_copies[copy],
            block_table=self.block_table, prefix_lens=self.prefix_lens,
            draft_len=p.draft_len, page_size=p.page_size, sm_scale=p.sm_scale,
            max_prefix_len=p.max_prefix_len, out=self.out, workspace=self.workspace,
            lse=self.lse, kv_dtype=p.kv_dtype, k_scale=p.k_scale, v_scale=p.v_scale,
            window_left=p.window_left, num_splits=0, qk_dim=p.qk_dim, v_dim=p.v_dim,
            qo_indptr=self.qo_indptr, draft_slots=self.draft_slots, tree_mask=self.tree_mask,
            sinks=self.sinks, logit_cap=p.logit_cap)

    def build_block_table(self, stream=None):
        binding.verify_attn_build_block_table(self.kv_indptr, self.kv_indices, self.p.page_size,
                                              self.max_pages, self.block_table, self.kv_lens,
                                              stream=stream)

    def step(self, copy: int = 0, stream=None):
        """a1-a7 once: block table, split-KV pass, combine."""
        self.build_block_table(stream)
        binding.verify_attn_fwd(self.calls[copy], stream)
        binding.verify_attn_combine(self.calls[copy], stream)

    def results(self):
        """(block_table, kv_lens, out as float64 numpy, lse as float64 numpy)."""
        import torch
        torch.cuda.synchronize(self.device)
        return (self.block_table.cpu().numpy(), self.kv_lens.cpu().numpy(),
                self.out.float().cpu().numpy().astype(np.float64),
                self.lse.cpu().numpy().astype(np.float64))
