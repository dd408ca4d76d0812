"""Seeded synthetic inputs for EAGLE target-verify attention (topk = 1).

This module only *draws* inputs: prefix lengths, a paged KV pool with a
shuffled page table, and bf16 / fp8-e4m3fn encoded q, k, v.  It holds none of
the attention arithmetic, so both the fp64 CPU oracle and the HIP path can be
fed from it without sharing any computation.

Layouts follow the paged-cache views of the pages' unified-attention call
(PR #23146, "Code Review" excerpt: ``k_cache.view(-1, page_size, H_kv, d)``,
``o.view(-1, H_q, v_head_dim)``):

* ``q``        [B*D, H_q, qk_dim]  bf16 bits (uint16); row ``b*D + i`` is draft i of sequence b
* ``k_cache``  [num_slots, H_kv, k_row]  bf16 bits (uint16) or e4m3fn bytes (uint8)
* ``v_cache``  [num_slots, H_kv, v_dim]  same dtype; ``None`` when V aliases the
  first ``v_dim`` columns of the K row (the MLA latent layout)
* ``kv_indptr`` int32 [B+1], ``kv_indices`` int32 [sum(L_b + D)]: the token-level
  slot list of each sequence, prefix tokens first, then its D draft tokens
  (PR #23146, "Code Review": ``kv_indptr, kv_indices = spec_info.kv_indptr, ...``).
  Within a page the slots are consecutive, which is what makes a page table valid
  at topk = 1 (PR #5168, reviewer note that all tokens in the page table are
  consecutive when top k = 1).

Recipe (seed = 1000 + config index unless given).  ``SeedSequence(seed)`` spawns
four children: child 0 draws the prefix lengths (integers, both ends inclusive)
and then the page permutation; child 1 draws q; children 2 and 3 draw the K and
V pools.  Normal values are float64 N(0,1) draws made in chunks of 2^22 values,
chunk c from its own PCG64 stream (the c-th spawn of the tensor's child), so
chunks can be drawn in parallel; they are rounded to bf16 with
round-to-nearest-even, or stored as ``e4m3fn(x / scale)`` with RNE and
saturation to +-448.  Only pages some sequence owns are drawn (in page-id
order); the rest of the pool is zero, or NaN bit patterns in poison mode.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

KV_BF16 = 0
KV_FP8_E4M3FN = 1

# bit patterns used to poison memory that must never be read
BF16_NAN_BITS = 0x7FC0
E4M3FN_NAN_BITS = 0x7F


@dataclasses.dataclass
class Problem:
    """One verify-attention call's inputs, all on the host."""

    name: str
    batch: int
    draft_len: int
    hq: int
    hkv: int
    qk_dim: int
    v_dim: int
    page_size: int
    kv_dtype: int                 # KV_BF16 or KV_FP8_E4M3FN
    k_scale: float
    v_scale: float
    sm_scale: float
    window_left: int              # -1: no window
    num_splits: int               # 0: library heuristic
    prefix_lens: np.ndarray       # int32 [B]
    kv_indptr: np.ndarray         # int32 [B+1]
    kv_indices: np.ndarray        # int32 [sum n_b]
    page_ids: list                # per sequence: int64 array of its page ids (in order)
    num_pages: int                # pool size in pages
    q: np.ndarray                 # uint16 [rows, Hq, qk_dim]
    k_cache: np.ndarray           # uint16 / uint8 [num_slots, Hkv, k_row]
    v_cache: Optional[np.ndarray]  # same dtype [num_slots, Hkv, v_dim] or None (alias of K)
    seed: int = 0
    # optional extensions (None / 0 = target verify at topk = 1)
    qo_indptr: Optional[np.ndarray] = None    # int32 [B+1]: ragged draft rows per sequence
    draft_slots: Optional[np.ndarray] = None  # int32 [B, D]: tree verify, slot of draft key j
    tree_mask: Optional[np.ndarray] = None    # uint8 [B, D, D]: row i sees draft key j
    sinks: Optional[np.ndarray] = None        # float32 [Hq]: sink logit per q head
    logit_cap: float = 0.0                    # > 0: scores s -> cap * tanh(s / cap)

    @property
    def rows(self) -> int:
        """Query rows: B*D, or qo_indptr[B] with ragged rows."""
        return int(self.qo_indptr[-1]) if self.qo_indptr is not None else self.batch * self.draft_len

    @property
    def v_aliases_k(self) -> bool:
        return self.v_cache is None

    @property
    def num_slots(self) -> int:
        return self.num_pages * self.page_size

    @property
    def max_prefix_len(self) -> int:
        return int(self.prefix_lens.max()) if self.batch else 0

    @property
    def max_pages_per_seq(self) -> int:
        if self.batch == 0:
            return 1
        return max(1, -(-(self.max_prefix_len + self.draft_len) // self.page_size))

    @property
    def elem_bytes(self) -> int:
        return 1 if self.kv_dtype == KV_FP8_E4M3FN else 2

    def v_view(self) -> np.ndarray:
        """The V cache as an array [num_slots, Hkv, v_dim] (a view when V aliases K)."""
        if self.v_cache is None:
            return self.k_cache[:, :, : self.v_dim]
        return self.v_cache


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """float -> bf16 bit patterns with round-to-nearest-even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u >> np.uint32(16)).astype(np.uint16)


def _e4m3fn_bytes(x: np.ndarray) -> np.ndarray:
    """float -> OCP e4m3fn bytes, RNE with saturation to +-448 (torch's conversion)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).clamp_(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


_CHUNK = 1 << 22


def _normal_encoded(seq: np.random.SeedSequence, n: int, kv_dtype: int,
                    scale: float, col_mean: Optional[np.ndarray] = None) -> np.ndarray:
    """n N(0,1) values, encoded; chunk c of 2^22 values comes from spawn c of ``seq``.

    ``col_mean`` (length w) is added to value i as col_mean[i % w]: the values are
    rows of w columns and column c gets mean col_mean[c]."""
    from concurrent.futures import ThreadPoolExecutor

    out = np.empty(n, dtype=np.uint8 if kv_dtype == KV_FP8_E4M3FN else np.uint16)
    nchunks = -(-n // _CHUNK)
    kids = seq.spawn(nchunks)

    def draw(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        x = np.random.default_rng(kids[c]).standard_normal(hi - lo)
        if col_mean is not None:
            x += col_mean[np.arange(lo, hi) % len(col_mean)]
        if kv_dtype == KV_FP8_E4M3FN:
            out[lo:hi] = _e4m3fn_bytes(x / scale)
        else:
            out[lo:hi] = _bf16_bits(x)

    if nchunks <= 1:
        for c in range(nchunks):
            draw(c)
    else:
        import os
        workers = max(1, min(16, len(os.sched_getaffinity(0)), nchunks))
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(draw, range(nchunks)))
    return out


def make_problem(*, name: str = "custom", batch: int, prefix_lens=None,
                 prefix_range: Optional[Sequence[int]] = None, draft_len: int = 4,
                 hq: int, hkv: int, qk_dim: int, v_dim: Optional[int] = None,
                 page_size: int = 1, kv_dtype: int = KV_BF16, kv_scale: float = 1.0,
                 v_aliases_k: bool = False, sm_scale: Optional[float] = None,
                 window_left: int = -1, num_splits: int = 0,
                 num_pages: Optional[int] = None, pool_factor: float = 1.25,
                 seed: int = 0, poison: bool = False, shuffle_pages: bool = True,
                 draft_counts=None, ragged: bool = False, tree: bool = False,
                 sinks: bool = False, logit_cap: float = 0.0, v_mean: float = 0.0) -> Problem:
    """Draw one problem.

    ``prefix_lens``: explicit list, or ``prefix_range=(lo, hi)`` for
    uniform integers in [lo, hi].  ``num_pages`` fixes the pool size, else
    ``ceil(pool_factor * total pages)``.  With ``poison`` the pool's page 0 is
    reserved and every slot no sequence owns (including the unused tail of a
    sequence's last page) holds NaN bit patterns.  ``shuffle_pages=False`` hands
    out pages in pool order (each sequence's pages contiguous), the layout a
    fresh allocator would produce.

    Extensions (each drawn from its own child stream, so the base arrays do not
    change): ``ragged`` (or explicit ``draft_counts``) gives sequence b n_b draft
    rows, uniform in [1, D], laid out by ``qo_indptr``; ``tree`` keeps the token
    list to the prefix and puts the D draft keys of each sequence at scattered
    slots of extra pages, with a random tree (each draft's parent is an earlier
    draft or the prefix) whose ancestor-or-self relation is ``tree_mask``;
    ``sinks`` draws one N(0, 1) sink logit per q head; ``logit_cap`` is passed on.

    ``v_mean`` gives V column c the mean v_mean * cos(0.37 c + 0.5) (for V aliasing
    K: the first v_dim columns of the K rows), so outputs are of order v_mean instead
    of shrinking with the number of keys.
    """
    v_dim = qk_dim if v_dim is None else v_dim
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(qk_dim)
    kids = np.random.SeedSequence(seed).spawn(7)
    rng = np.random.default_rng(kids[0])
    if tree and (ragged or draft_counts is not None or window_left >= 0):
        raise ValueError("tree verify takes uniform rows and no window")

    # 1. prefix lengths
    if prefix_lens is not None:
        lens = np.asarray(prefix_lens, dtype=np.int64).reshape(batch)
    elif prefix_range is not None:
        lens = rng.integers(prefix_range[0], prefix_range[1] + 1, size=batch).astype(np.int64)
    else:
        raise ValueError("give prefix_lens or prefix_range")
    if draft_counts is not None:
        nq = np.asarray(draft_counts, dtype=np.int64).reshape(batch)
    elif ragged:
        nq = np.random.default_rng(kids[4]).integers(1, draft_len + 1, size=batch).astype(np.int64)
    else:
        nq = np.full(batch, draft_len, dtype=np.int64)
    # explicit counts may hold 0 (a sequence with no rows owns no keys this call);
    # random ragged counts are in [1, draft_len]
    if (ragged or draft_counts is not None) and ((nq < 0).any() or (nq > draft_len).any()):
        raise ValueError("draft counts must be in [0, draft_len]")
    # token list: prefix then the sequence's draft tokens (tree: prefix only)
    n_tok = lens if tree else lens + nq
    n_pages = -(-n_tok // page_size)
    d_pages = -(-draft_len // page_size) if tree else 0   # tree: pages holding draft keys
    total_pages = int(n_pages.sum()) + batch * d_pages

    # 2. page permutation: each sequence's pages, in order, from a shuffled pool
    reserved = 1 if poison else 0
    if num_pages is None:
        num_pages = max(int(math.ceil(pool_factor * total_pages)), total_pages) + reserved
    if num_pages - reserved < total_pages:
        raise ValueError("pool too small")
    if shuffle_pages:
        perm = rng.permutation(num_pages - reserved)[:total_pages] + reserved
    else:
        perm = np.arange(total_pages) + reserved
    page_ids = []
    indptr = np.zeros(batch + 1, dtype=np.int64)
    indices = np.empty(int(n_tok.sum()), dtype=np.int64)
    off = 0
    for b in range(batch):
        pg = perm[off: off + n_pages[b]].astype(np.int64)
        off += n_pages[b]
        page_ids.append(pg)
        t = np.arange(n_tok[b], dtype=np.int64)
        indices[indptr[b]: indptr[b] + n_tok[b]] = pg[t // page_size] * page_size + t % page_size
        indptr[b + 1] = indptr[b] + n_tok[b]
    draft_slots = tree_mask = None
    if tree:
        trng = np.random.default_rng(kids[5])
        dpg = perm[off: off + batch * d_pages].astype(np.int64)
        cand = (dpg[:, None] * page_size + np.arange(page_size)[None, :]).reshape(-1)
        draft_slots = trng.permutation(cand)[: batch * draft_len].reshape(batch, draft_len)
        tree_mask = np.zeros((batch, draft_len, draft_len), dtype=np.uint8)
        for b in range(batch):
            parent = [-1] + [int(trng.integers(-1, j)) for j in range(1, draft_len)]
            for i in range(draft_len):
                a = i
                while a >= 0:          # ancestors and self
                    tree_mask[b, i, a] = 1
                    a = parent[a]

    # 3-5. q, then the owned pages of the K and V pools (in page-id order)
    num_slots = num_pages * page_size
    n_rows = int(nq.sum())
    q = _normal_encoded(kids[1], n_rows * hq * qk_dim, KV_BF16, 1.0)
    q = q.reshape(n_rows, hq, qk_dim)
    owned_pages = np.sort(perm)

    def pool(seq, width, v_cols):
        per_page = page_size * hkv * width
        dt = np.uint8 if kv_dtype == KV_FP8_E4M3FN else np.uint16
        arr = np.zeros((num_pages, per_page), dtype=dt)
        mean = None
        if v_mean and v_cols:
            mean = np.zeros(width)
            mean[:v_cols] = v_mean * np.cos(0.37 * np.arange(v_cols) + 0.5)
        arr[owned_pages] = _normal_encoded(seq, total_pages * per_page, kv_dtype,
                                           kv_scale, mean).reshape(total_pages, per_page)
        return arr.reshape(num_slots, hkv, width)

    k = pool(kids[2], qk_dim, v_dim if v_aliases_k else 0)
    v = None if v_aliases_k else pool(kids[3], v_dim, v_dim)

    if poison:
        owned = np.zeros(num_slots, dtype=bool)
        owned[indices] = True
        if draft_slots is not None:
            owned[draft_slots.reshape(-1)] = True
        nan = E4M3FN_NAN_BITS if kv_dtype == KV_FP8_E4M3FN else BF16_NAN_BITS
        k[~owned] = nan
        if v is not None:
            v[~owned] = nan

    return Problem(
        name=name, batch=batch, draft_len=draft_len, hq=hq, hkv=hkv, qk_dim=qk_dim,
        v_dim=v_dim, page_size=page_size, kv_dtype=kv_dtype,
        k_scale=float(kv_scale) if kv_dtype == KV_FP8_E4M3FN else 1.0,
        v_scale=float(kv_scale) if kv_dtype == KV_FP8_E4M3FN else 1.0,
        sm_scale=float(sm_scale), window_left=int(window_left), num_splits=int(num_splits),
        prefix_lens=lens.astype(np.int32), kv_indptr=indptr.astype(np.int32),
        kv_indices=indices.astype(np.int32), page_ids=page_ids, num_pages=int(num_pages),
        q=q, k_cache=k, v_cache=v, seed=seed,
        qo_indptr=(np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
                   if (ragged or draft_counts is not None) else None),
        draft_slots=None if draft_slots is None else draft_slots.astype(np.int32),
        tree_mask=tree_mask,
        sinks=(np.random.default_rng(kids[6]).standard_normal(hq).astype(np.float32)
               if sinks else None),
        logit_cap=float(logit_cap))


# The five workloads.  Shapes follow the pages' serving settings: 4 draft tokens at
# topk = 1 (PR #5168 benchmark server flags), page sizes 1/4/16/64, head dims 128 and
# 256 (PR #27382 accuracy tests), GQA, and an MLA latent head whose V is the first 512
# columns of the 576-wide K row (PR #23146 review: qk_head_dim may differ from v_head_dim).
CONFIG_NAMES = (
    "tiny-verify",
    "llama8b-verify",
    "long-context-batch",
    "sliding-window-gqa",
    "mla-fp8-share",
)


def config_kwargs(idx: int) -> dict:
    if idx == 0:
        return dict(batch=1, prefix_lens=[256], draft_len=4, hq=8, hkv=2, qk_dim=128,
                    page_size=1, num_pages=260, num_splits=4)
    if idx == 1:
        return dict(batch=4, prefix_lens=[2048] * 4, draft_len=4, hq=32, hkv=8, qk_dim=128,
                    page_size=4, num_pages=4096)
    if idx == 2:
        return dict(batch=32, prefix_range=(4096, 32768), draft_len=4, hq=32, hkv=8,
                    qk_dim=128, page_size=16)
    if idx == 3:
        return dict(batch=16, prefix_range=(16384, 65536), draft_len=4, hq=32, hkv=4,
                    qk_dim=256, v_dim=256, page_size=64, window_left=4096)
    if idx == 4:
        return dict(batch=64, prefix_range=(1024, 8192), draft_len=4, hq=16, hkv=1,
                    qk_dim=576, v_dim=512, v_aliases_k=True, kv_dtype=KV_FP8_E4M3FN,
                    kv_scale=0.05, page_size=64, sm_scale=1.0 / math.sqrt(192.0))
    raise ValueError(f"no config {idx}")


def make_config(idx: int, seed: Optional[int] = None, **overrides) -> Problem:
    kw = config_kwargs(idx)
    kw.update(overrides)
    return make_problem(name=CONFIG_NAMES[idx], seed=1000 + idx if seed is None else seed, **kw)


def visible_token_count(prefix_len: int, draft_len: int, window_left: int) -> int:
    """Keys that at least one of a sequence's D draft rows may see.

    Row i (absolute position L+i) sees keys t <= L+i, and with a left window W only
    t >= L+i-W (flash-attention ``window_size=(W, -1)``); the union over rows is
    [max(0, L-W), L+D).
    """
    lo = 0 if window_left < 0 else max(0, prefix_len - window_left)
    return prefix_len + draft_len - lo


def algorithmic_kv_bytes(p: Problem) -> int:
    """KV bytes a verify call must read: every visible token once per KV head.

    K and V rows count separately unless V aliases K, in which case the K row
    (qk_dim wide) already holds V.  Excludes q, the output, indices, partials and
    page-rounding over-fetch.
    """
    per_tok = p.hkv * (p.qk_dim + (0 if p.v_aliases_k else p.v_dim)) * p.elem_bytes
    return int(sum(visible_token_count(int(L), n, p.window_left)
                   for L, n in zip(p.prefix_lens, draft_rows(p)))) * per_tok


def algorithmic_flops(p: Problem) -> int:
    """Matrix flops of a verify call: every query row against every key its sequence
    shows any row (the visible keys above), 2 (qk_dim + v_dim) flops per (row, key):
    one multiply-add per element of QK^T and of PV.  Excludes the softmax and the
    masked-out products inside partly visible tiles."""
    per_row_key = 2 * (p.qk_dim + p.v_dim)
    return int(sum(visible_token_count(int(L), n, p.window_left) * n * p.hq
                   for L, n in zip(p.prefix_lens, draft_rows(p)))) * per_row_key


def draft_rows(p: Problem):
    """Draft rows (and draft keys) of each sequence: D, or qo_indptr's counts."""
    if p.qo_indptr is None:
        return [p.draft_len] * p.batch
    return [int(p.qo_indptr[b + 1] - p.qo_indptr[b]) for b in range(p.batch)]
