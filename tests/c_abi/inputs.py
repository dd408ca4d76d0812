"""The C caller's inputs, drawn in Python from the same splitmix64 stream (Steele, Lea
and Flood's published generator, seed 12345) in the same order as
tests/c_abi/verify_c_caller.c: page shuffle, q, k_cache, v_cache.  Values are uniform
in [-1, 1) from the top 24 bits of each draw, rounded to bf16 (nearest even).  This
module generates inputs only; it computes nothing of the verify method."""

import numpy as np

B, D, HQ, HKV, DIM, PAGE, POOL_PAGES = 3, 4, 8, 2, 128, 4, 40
PREFIX = [0, 17, 100]
_MASK = (1 << 64) - 1


class SplitMix64:
    def __init__(self, seed: int):
        self.state = seed & _MASK

    def next(self) -> int:
        self.state = (self.state + 0x9E3779B97F4A7C15) & _MASK
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK
        return z ^ (z >> 31)


def _bf16_draws(gen: SplitMix64, n: int) -> np.ndarray:
    top = np.array([gen.next() >> 40 for _ in range(n)], dtype=np.float64)
    x = (top / 16777216.0).astype(np.float32) * np.float32(2.0) - np.float32(1.0)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def problem():
    """dict of the host arrays and scalars the C caller uploads."""
    gen = SplitMix64(12345)
    n = [L + D for L in PREFIX]
    pages = [(x + PAGE - 1) // PAGE for x in n]
    perm = list(range(POOL_PAGES))
    for i in range(POOL_PAGES - 1, 0, -1):
        j = gen.next() % (i + 1)
        perm[i], perm[j] = perm[j], perm[i]
    indptr = [0]
    indices = []
    p0 = 0
    for b in range(B):
        indices += [perm[p0 + t // PAGE] * PAGE + t % PAGE for t in range(n[b])]
        indptr.append(indptr[-1] + n[b])
        p0 += pages[b]
    slots = POOL_PAGES * PAGE
    q = _bf16_draws(gen, B * D * HQ * DIM).reshape(B * D, HQ, DIM)
    k = _bf16_draws(gen, slots * HKV * DIM).reshape(slots, HKV, DIM)
    v = _bf16_draws(gen, slots * HKV * DIM).reshape(slots, HKV, DIM)
    return dict(q=q, k_cache=k, v_cache=v, kv_indptr=np.array(indptr, dtype=np.int32),
                kv_indices=np.array(indices, dtype=np.int32),
                prefix_lens=np.array(PREFIX, dtype=np.int32), max_pages=max(pages))
