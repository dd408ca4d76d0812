"""Plain fp64 CPU oracle for EAGLE target-verify attention at topk = 1.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline leg use this module; the library never does.  It shares no code with
the HIP path: it reads the same input arrays and nothing else.

What it computes
----------------
At topk = 1 the draft tree is a single chain, so target verification is plain
causal attention of each sequence's D draft-token queries over that sequence's
prefix followed by the draft tokens themselves (PR #27382, "Modifications":
topk = 1 reduces the EAGLE tree to pure causal; PR #23146 calls the unified
kernel with ``causal=True``).  The split-KV method of PR #27382 ("Motivation":
split the prefix across programs and merge partials with a log-sum-exp; its
combine stage adds the causal draft-draft block) is an exact rewrite of that
softmax, so the oracle writes out the plain definition:

  for draft row i of sequence b (absolute position p = L_b + i) and q head h,
  with KV head g = h // (H_q / H_kv):
      visible keys  t in [0, p]            (and t >= p - W with a left window W)
      s_t  = sm_scale * k_scale * <q, K_t>            (fp64)
      O    = sum_t softmax(s)_t * v_scale * V_t
      LSE  = log(sum_t exp(s_t))                      (natural log of scaled scores)

Readings taken where the pages are silent (each is listed with its status):
  1. Draft K/V sit in the paged cache after the prefix, under the same token
     list (the verify call passes only the cache to the kernel).
  2. Causal alignment is bottom-right: draft i sees the whole prefix and drafts
     0..i.  Pinned by full causal attention over the concatenated sequence.
  3. Sliding window follows flash-attention ``window_size=(W, -1)``: keep
     p - W <= t <= p.  Parity unpinned by the pages (a documented convention).
  4. GQA: q head h uses KV head h // G (contiguous groups).  The pages say
     nothing; it matches ``repeat_interleave`` / torch's ``enable_gqa``.
  5. LSE uses the natural log of the scaled scores.
  6. fp8 is OCP e4m3fn; the dequantised value is code * scale.
  7. MLA: V is the first v_dim columns of the K row.
  8. Block-table padding is page id 0 (parity unpinned by the pages: convention).

Extensions beyond topk = 1 (the split-KV page lists them as what its fast path
leaves to the fallback in "Modifications": sinks, logit cap, ragged extend;
PR #12128's review builds draft-extend ``cu_seqlens_q`` from ``accept_length``;
PR #5168 leaves topk > 1 to a later change; PR #23146's page-table code translates
full-pool slots to a sliding-window pool):
  9. Ragged rows (draft-extend): sequence b owns the query rows
     qo_indptr[b] .. qo_indptr[b+1]-1, n_b of them, the last n_b tokens of its KV
     (positions L_b .. L_b + n_b - 1); row i sees keys t <= L_b + i as above.
 10. Tree verify (topk > 1): the prefix is paged as before, but draft key j of
     sequence b lives at an arbitrary slot draft_slots[b, j], and row i sees draft
     key j iff tree_mask[b, i, j] is set (instead of j <= i).  No window.
 11. Attention sinks: one extra logit sinks[h] per q head joins the softmax
     denominator with a zero value vector (so LSE includes it).
 12. Logit cap: scaled scores s become cap * tanh(s / cap) before the softmax
     (cap > 0; sinks are not capped).
 13. Sliding-window pool: full-pool slot s maps to full_to_swa[s] in the window
     pool; the window pool's block table is built from the mapped slots.
"""

from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np


# ---------------------------------------------------------------------------
# element decoding (exact)
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64: a bf16 is the top half of a float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):          # NaN payloads widen to NaN
        return b.view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP fp8 e4m3fn bytes -> float64, from the format's bit definition.

    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
    holds subnormals m/8 * 2^-6; S.1111.111 is NaN; there are no infinities.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * mag
    out[(e == 0xF) & (c & 0x7 == 0x7)] = np.nan
    return out


def decode_kv(raw: np.ndarray, kv_dtype: int) -> np.ndarray:
    """Cache elements -> float64.  kv_dtype 0 = bf16 bits, 1 = e4m3fn bytes."""
    return e4m3fn_to_f64(raw) if kv_dtype == 1 else bf16_to_f64(raw)


# ---------------------------------------------------------------------------
# a1: block table from the token-level slot list
# ---------------------------------------------------------------------------

def block_table(kv_indptr: np.ndarray, kv_indices: np.ndarray, page_size: int,
                max_pages: int) -> Tuple[np.ndarray, np.ndarray]:
    """Token-level ragged slots -> [B, max_pages] page ids (+ per-sequence KV length).

    At topk = 1 a sequence's slots are consecutive inside each page (PR #5168),
    so the page holding token t is the slot of the page's first token divided by
    the page size (PR #23146 builds the same 2-D table from the spec-decode
    indices).  Entries past a sequence's last page are 0.  kv_lens[b] is the
    sequence's KV length from kv_indptr (PR #23146, seqused_k commit).
    """
    B = len(kv_indptr) - 1
    bt = np.zeros((B, max_pages), dtype=np.int64)
    lens = np.zeros(B, dtype=np.int64)
    for b in range(B):
        start, end = int(kv_indptr[b]), int(kv_indptr[b + 1])
        n = end - start
        lens[b] = n
        npages = -(-n // page_size)
        for pg in range(npages):
            bt[b, pg] = int(kv_indices[start + pg * page_size]) // page_size
    return bt, lens


# ---------------------------------------------------------------------------
# a3-a7 as one plain definition
# ---------------------------------------------------------------------------

def visible_keys(prefix_len: int, i: int, window_left: int) -> np.ndarray:
    """Key positions draft row i may attend: bottom-right causal, optional left window."""
    p = prefix_len + i
    lo = 0 if window_left < 0 else max(0, p - window_left)
    return np.arange(lo, p + 1, dtype=np.int64)


def _sequence_kv(b, kv_indptr, kv_indices, k_cache, v_cache, qk_dim, v_dim, kv_dtype,
                 k_scale, v_scale):
    """Gather sequence b's K and V rows (all heads) by the token-level slot list."""
    start, end = int(kv_indptr[b]), int(kv_indptr[b + 1])
    slots = np.asarray(kv_indices[start:end], dtype=np.int64)
    K = decode_kv(k_cache[slots, :, :qk_dim], kv_dtype) * k_scale   # [n, Hkv, dk]
    V = decode_kv(v_cache[slots, :, :v_dim], kv_dtype) * v_scale    # [n, Hkv, dv]
    return K, V


def attend(q_row: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float,
           logit_cap: float = 0.0, sink: Optional[float] = None):
    """softmax(s) V and the natural-log LSE for one query row (fp64), s = sm_scale * K q.

    With ``logit_cap`` > 0 the scores are s -> cap * tanh(s / cap) first (reading 12);
    a ``sink`` logit joins the denominator with a zero value vector (reading 11)."""
    s = sm_scale * (K @ q_row) if K.shape[0] else np.zeros(0)
    if logit_cap > 0:
        s = logit_cap * np.tanh(s / logit_cap)
    allx = s if sink is None else np.append(s, float(sink))
    if allx.size == 0 or np.all(allx == -math.inf):
        return np.zeros(V.shape[1]), -math.inf
    m = allx.max()
    w = np.exp(s - m)
    z = np.exp(allx - m).sum()
    return (w @ V) / z, m + math.log(z)


def translate_slots(kv_indices: np.ndarray, full_to_swa: np.ndarray) -> np.ndarray:
    """Full-pool slots -> sliding-window-pool slots through the pool's map (reading 13)."""
    return np.asarray(full_to_swa, dtype=np.int64)[np.asarray(kv_indices, dtype=np.int64)]


def verify_attention(q, k_cache, v_cache, kv_indptr, kv_indices, prefix_lens, draft_len,
                     hq, hkv, qk_dim, v_dim, sm_scale, window_left=-1, kv_dtype=0,
                     k_scale=1.0, v_scale=1.0, rows: Optional[Sequence[int]] = None,
                     qo_indptr=None, draft_slots=None, tree_mask=None, sinks=None,
                     logit_cap: float = 0.0):
    """The verify output O [rows, Hq, v_dim] and LSE [rows, Hq], in float64.

    ``q`` holds bf16 bits [rows, Hq, qk_dim] (rows = B*D, or qo_indptr[B] with
    ragged rows); the caches hold raw elements [num_slots, Hkv, row]; ``v_cache``
    may be ``k_cache`` itself when V is the first v_dim columns of the K row.
    ``rows`` optionally restricts the work to the given query rows (others stay
    NaN) so large problems can be sampled.  ``qo_indptr``, ``draft_slots`` with
    ``tree_mask``, ``sinks`` and ``logit_cap`` select readings 9-12.
    """
    B = len(prefix_lens)
    G = hq // hkv
    tree = draft_slots is not None
    if qo_indptr is None:
        qo = np.arange(B + 1, dtype=np.int64) * draft_len
    else:
        qo = np.asarray(qo_indptr, dtype=np.int64)
    R = int(qo[B])
    O = np.full((R, hq, v_dim), np.nan)
    LSE = np.full((R, hq), np.nan)
    wanted = None if rows is None else set(int(r) for r in rows)
    for b in range(B):
        rows_b = list(range(int(qo[b]), int(qo[b + 1])))
        if wanted is not None and not wanted.intersection(rows_b):
            continue
        K, V = _sequence_kv(b, kv_indptr, kv_indices, k_cache, v_cache, qk_dim, v_dim,
                            kv_dtype, k_scale, v_scale)
        L = int(prefix_lens[b])
        if tree:
            ds = np.asarray(draft_slots[b], dtype=np.int64)
            Kd = decode_kv(k_cache[ds, :, :qk_dim], kv_dtype) * k_scale
            Vd = decode_kv(v_cache[ds, :, :v_dim], kv_dtype) * v_scale
        for i, r in enumerate(rows_b):
            if wanted is not None and r not in wanted:
                continue
            if tree:
                sel = np.nonzero(np.asarray(tree_mask[b, i]) != 0)[0]
                Kr = np.concatenate([K[:L], Kd[sel]], axis=0)
                Vr = np.concatenate([V[:L], Vd[sel]], axis=0)
            else:
                vis = visible_keys(L, i, window_left)
                Kr, Vr = K[vis], V[vis]
            for h in range(hq):
                g = h // G
                qf = bf16_to_f64(q[r, h, :qk_dim])
                sink = None if sinks is None else float(sinks[h])
                O[r, h], LSE[r, h] = attend(qf, Kr[:, g], Vr[:, g], sm_scale, logit_cap, sink)
    return O, LSE


# ---------------------------------------------------------------------------
# the split route: partial (O, LSE) per key chunk, merged by log-sum-exp
# ---------------------------------------------------------------------------

def lse_merge(parts: List[Tuple[np.ndarray, float]]):
    """Merge softmax partials (O_c normalised within chunk c, LSE_c).

    O = sum_c e^{LSE_c - M} O_c / sum_c e^{LSE_c - M}, LSE = M + log sum_c e^{LSE_c - M},
    M = max_c LSE_c; chunks with LSE = -inf carry weight 0 (PR #27382: partials
    merged via log-sum-exp).
    """
    lses = np.array([p[1] for p in parts], dtype=np.float64)
    M = lses.max() if len(lses) else -math.inf
    if M == -math.inf:
        return np.zeros_like(parts[0][0]) if parts else None, -math.inf
    w = np.exp(lses - M)
    num = sum(wc * oc for wc, (oc, _) in zip(w, parts))
    z = w.sum()
    return num / z, M + math.log(z)


def verify_attention_split(q, k_cache, v_cache, kv_indptr, kv_indices, prefix_lens,
                           draft_len, hq, hkv, qk_dim, v_dim, sm_scale, window_left=-1,
                           kv_dtype=0, k_scale=1.0, v_scale=1.0, num_splits=1):
    """Split-KV route: the prefix keys of each sequence are cut into ``num_splits``
    contiguous chunks, the draft keys form one more chunk (the draft-draft block),
    each chunk is attended separately and the partials are merged with ``lse_merge``.
    Must equal ``verify_attention`` up to rounding."""
    B = len(prefix_lens)
    G = hq // hkv
    O = np.zeros((B * draft_len, hq, v_dim))
    LSE = np.zeros((B * draft_len, hq))
    for b in range(B):
        K, V = _sequence_kv(b, kv_indptr, kv_indices, k_cache, v_cache, qk_dim, v_dim,
                            kv_dtype, k_scale, v_scale)
        L = int(prefix_lens[b])
        bounds = np.linspace(0, L, num_splits + 1).round().astype(np.int64)
        for i in range(draft_len):
            r = b * draft_len + i
            vis = visible_keys(L, i, window_left)
            chunks = [vis[(vis >= bounds[c]) & (vis < bounds[c + 1])] for c in range(num_splits)]
            chunks.append(vis[vis >= L])
            for h in range(hq):
                g = h // G
                qf = bf16_to_f64(q[r, h, :qk_dim])
                parts = [attend(qf, K[c, g], V[c, g], sm_scale) for c in chunks]
                O[r, h], LSE[r, h] = lse_merge(parts)
    return O, LSE


# ---------------------------------------------------------------------------
# convenience wrappers taking an object with the input fields
# ---------------------------------------------------------------------------

def problem_fields(p):
    """verify_attention's base keyword arguments from an object carrying the inputs."""
    v_cache = p.k_cache if p.v_cache is None else p.v_cache
    return dict(q=p.q, k_cache=p.k_cache, v_cache=v_cache, kv_indptr=p.kv_indptr,
                kv_indices=p.kv_indices, prefix_lens=p.prefix_lens, draft_len=p.draft_len,
                hq=p.hq, hkv=p.hkv, qk_dim=p.qk_dim, v_dim=p.v_dim, sm_scale=p.sm_scale,
                window_left=p.window_left, kv_dtype=p.kv_dtype, k_scale=p.k_scale,
                v_scale=p.v_scale)


def _ext_fields(p):
    return dict(qo_indptr=getattr(p, "qo_indptr", None),
                draft_slots=getattr(p, "draft_slots", None),
                tree_mask=getattr(p, "tree_mask", None), sinks=getattr(p, "sinks", None),
                logit_cap=float(getattr(p, "logit_cap", 0.0) or 0.0))


def run(p, rows=None):
    """verify_attention on an object carrying the input arrays and scalars."""
    return verify_attention(**problem_fields(p), **_ext_fields(p), rows=rows)


def run_split(p, num_splits):
    return verify_attention_split(**problem_fields(p), num_splits=num_splits)


def run_block_table(p, max_pages=None):
    mp = p.max_pages_per_seq if max_pages is None else max_pages
    return block_table(p.kv_indptr, p.kv_indices, p.page_size, mp)


# ---------------------------------------------------------------------------
# comparison helper used by the parity tests
# ---------------------------------------------------------------------------

def allclose_report(got: np.ndarray, ref: np.ndarray, atol: float, rtol: float):
    """numpy-allclose style check |got - ref| <= atol + rtol * |ref| (NaN in ref skipped).

    Returns (ok, max_abs_err, worst_excess) where worst_excess is the largest
    |got-ref| - (atol + rtol|ref|) (<= 0 when ok)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = ~np.isnan(ref)
    if not m.any():
        return True, 0.0, -math.inf
    d = np.abs(got[m] - ref[m])
    bad = np.isnan(got[m])
    excess = d - (atol + rtol * np.abs(ref[m]))
    excess[bad] = math.inf
    return bool((excess <= 0).all()), float(np.nanmax(np.where(bad, math.inf, d))), float(excess.max())
