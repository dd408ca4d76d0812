/*
 * verify_attn.h - EAGLE target-verify attention at topk = 1 on MI355X (gfx950).
 *
 * What the library computes
 *   Each of B sequences has a prefix of L_b tokens and D draft tokens whose K/V
 *   already sit in a paged KV cache right after the prefix.  Draft row i of
 *   sequence b (absolute position p = L_b + i) attends, per query head h, to the
 *   keys t in [0, p] of its own sequence (bottom-right causal; at topk = 1 the
 *   draft tree is a single chain so no custom mask is needed - PR #27382
 *   "[AMD][Perf] Split-KV flash-decode attention for EAGLE target-verify",
 *   section "Modifications"), optionally limited to t >= p - W by a left sliding
 *   window in flash-attention's window_size=(W, -1) convention (PR #23146,
 *   "Code Review" on the target-verify unified-attention call).
 *
 *   The work is split as on PR #27382 ("Motivation", "Modifications"): a
 *   split-KV (flash-decode) pass writes one partial output and log-sum-exp per
 *   piece of a sequence's keys (verify_attn_fwd), then a combine merges the
 *   partials by log-sum-exp (verify_attn_combine).  Here the pass also covers
 *   the small causal draft-draft block: the D draft keys are the last keys of a
 *   sequence and the per-row causal bound t <= p masks them, so the combine is a
 *   pure merge.  The paged cache is addressed through a 2-D block table built
 *   from the token-level kv_indptr/kv_indices lists
 *   (verify_attn_build_block_table; PR #23146 builds the same table with scatter
 *   kernels, and PR #5168 notes that at topk = 1 the tokens of a page are
 *   consecutive, which is what makes the table valid).
 *
 * Conventions for every entry point
 *   - Pointers named in a verify_attn_args or passed to build_block_table are
 *     DEVICE pointers; the caller allocates and owns all memory.  The library
 *     never allocates, frees or synchronises, and keeps no pointer after a call.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *     void*, NULL = the default stream).
 *   - Every launch decision depends only on host scalars, never on device data,
 *     so calls are safe to record into a HIP graph (workspace addresses stay fixed).
 *   - Calls return a status; on any status other than VA_OK nothing was launched.
 *     Device data that breaks a stated precondition (page ids outside the pool,
 *     a block table too narrow) is NOT detected and may fault the GPU (the Python
 *     binding has an optional host-side validator for integration and debugging).
 *   - Indices are int32; byte offsets are computed in 64 bits.
 */
#ifndef VERIFY_ATTN_H
#define VERIFY_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define VA_OK 0           /* success                                                   */
#define VA_EINVAL 1       /* null pointer, negative size, bad stride or alignment      */
#define VA_EUNSUPPORTED 2 /* valid request this library does not serve: caller falls back
                             (the static-shape gate of PR #27382, "Modifications")      */
#define VA_EWORKSPACE 3   /* workspace smaller than verify_attn_workspace_bytes()       */
#define VA_EHIP 4         /* the HIP runtime reported an error on launch                */

/* KV cache element types */
#define VA_KV_BF16 0          /* bfloat16                                               */
#define VA_KV_FP8_E4M3FN 1    /* OCP fp8 e4m3fn; value = code * k_scale (or v_scale)    */

/*
 * Arguments of verify_attn_fwd / verify_attn_combine / verify_attn_can_handle.
 * Plain C struct passed by pointer; struct_size must be sizeof(verify_attn_args)
 * or VERIFY_ATTN_ARGS_V1_SIZE.
 * All strides are in ELEMENTS of the pointed-to type; the innermost dimension of
 * every tensor is contiguous.  q and out are indexed by query row r = b*D + i
 * (the uniform-draft qo_indptr of PR #23146).
 */
typedef struct verify_attn_args {
    int32_t struct_size;

    /* problem shape */
    int32_t batch;          /* B >= 0                                                   */
    int32_t draft_len;      /* D, 1..8                                                  */
    int32_t hq, hkv;        /* query / KV heads; hq % hkv == 0, G = hq / hkv            */
    int32_t qk_dim, v_dim;  /* (128,128), (256,256) or (576,512); v_dim may differ from
                               qk_dim (PR #23146 review on the output view)              */
    int32_t page_size;      /* P: a power of two, 1..1024                               */
    int32_t kv_dtype;       /* VA_KV_BF16 or VA_KV_FP8_E4M3FN (q is always bf16)        */
    float k_scale, v_scale; /* dequantisation multipliers of the fp8 cache (PR #27382
                               "Modifications"); must be 1.0 for bf16                    */
    float sm_scale;         /* softmax scale applied to q.k                             */
    int32_t window_left;    /* -1: no window; W >= 0: keep keys t >= p - W              */
    int32_t max_prefix_len; /* host-side upper bound of prefix_lens[b]; sizes the grid.
                               A larger device value stays correct but runs slower.     */
    int32_t num_splits;     /* S, partial slots per (sequence, KV head): 0 = library
                               heuristic (CU count); else >= 1.  The keys of all
                               sequences are cut into equal ranges, one per
                               workgroup, and S bounds how many ranges one sequence
                               may span (1 = one workgroup per sequence).           */

    /* q: [B*D, hq, qk_dim] bf16, any finite values                                     */
    const void* q;
    int64_t q_stride_row, q_stride_head;
    /* K cache: row of token slot s, KV head g at k_cache + s*k_stride_slot +
       g*k_stride_head, qk_dim elements; slot s = page*P + offset (the
       [-1, P, hkv, d] paged view of PR #23146).  A slot stride of 4 GiB or more
       (in bytes) is VA_EUNSUPPORTED: kernels form slot * stride as one 32 x 32-bit
       product.                                                                         */
    const void* k_cache;
    int64_t k_stride_slot, k_stride_head;
    /* V cache, same addressing, v_dim elements.  May equal k_cache with the same
       strides (MLA: V is the first v_dim columns of the K row); fp8 576/512 calls
       whose V is that view take the latent-head kernel, others the generic one.       */
    const void* v_cache;
    int64_t v_stride_slot, v_stride_head;
    /* [B, max_pages_per_seq] int32 page ids, from verify_attn_build_block_table       */
    const int32_t* block_table;
    int32_t max_pages_per_seq;
    /* [B] int32 prefix lengths L_b (the KV length of sequence b is L_b + D)           */
    const int32_t* prefix_lens;

    /* fp32 workspace of at least verify_attn_workspace_bytes() bytes, written by
       verify_attn_fwd and read by verify_attn_combine                                  */
    float* workspace;
    int64_t workspace_bytes;

    /* out: [B*D, hq, v_dim] bf16 (round to nearest even)                               */
    void* out;
    int64_t o_stride_row, o_stride_head;
    /* lse: [B*D, hq] fp32 contiguous natural-log LSE of the scaled scores, or NULL     */
    float* lse;

    /* ---- version 2: optional extensions.  A caller passing struct_size =
       VERIFY_ATTN_ARGS_V1_SIZE (the layout up to here) gets none of them; with
       sizeof(verify_attn_args), NULL / 0 turns each off. ----                          */
    /* Ragged draft rows (draft-extend: rows = accept_length + 1 per sequence, the
       cu_seqlens_q of PR #12128's draft-extend replay metadata, "Code Review"): [B+1] int32 device,
       non-decreasing from 0; sequence b owns q/out/lse rows qo_indptr[b] ..
       qo_indptr[b+1]-1, n_b <= draft_len of them, at positions L_b .. L_b+n_b-1
       (its KV holds L_b + n_b tokens).  NULL: n_b = draft_len, row b*D + i.      */
    const int32_t* qo_indptr;
    /* Tree verify (topk > 1, left to a later change by PR #5168): draft key j of
       sequence b sits at slot draft_slots[b*D + j] ([B, D] int32 device) instead of
       after the prefix in the block table, and row i sees it iff
       tree_mask[(b*D + i)*D + j] != 0 ([B, D, D] uint8 device).  The block table
       then only needs the prefix.  Requires window_left = -1 and qo_indptr = NULL. */
    const int32_t* draft_slots;
    const uint8_t* tree_mask;
    /* Attention sinks: [hq] fp32 device, one extra logit per q head (natural-log
       units of the scaled scores) in every row's softmax denominator with a zero
       value; lse includes it.  NULL: none.                                         */
    const float* sinks;
    /* Logit cap: > 0 replaces each scaled score s by cap * tanh(s / cap) (sinks are
       not capped); 0: off.                                                         */
    float logit_cap;
} verify_attn_args;

/* Size of the version 1 layout (every field before qo_indptr). */
#define VERIFY_ATTN_ARGS_V1_SIZE ((int32_t)offsetof(verify_attn_args, qo_indptr))

/*
 * Block-table scatter (PR #23146 page-table scatter kernels; validity at topk = 1
 * from PR #5168).  For sequence b with n_b = kv_indptr[b+1] - kv_indptr[b] tokens:
 *     block_table[b*max_pages_per_seq + p] = kv_indices[kv_indptr[b] + p*P] / P
 * for p < ceil(n_b / P), and 0 for the remaining columns.  kv_lens (optional,
 * NULL to skip) receives n_b, the per-sequence KV length that PR #23146 derives
 * from kv_indptr.
 *   kv_indptr  [batch+1] int32 device, non-decreasing, kv_indptr[0] = 0
 *   kv_indices [kv_indptr[batch]] int32 device token slots; within a sequence the
 *              slots of one page are consecutive and each sequence starts at
 *              offset 0 of its first page
 *   block_table [batch, max_pages_per_seq] int32 device, written
 *   kv_lens    [batch] int32 device or NULL
 * Precondition: max_pages_per_seq >= ceil(n_b / P) (pages past the width are dropped).
 * Errors: VA_EINVAL for null pointers with batch > 0, batch < 0, max_pages < 1;
 *         VA_EUNSUPPORTED when page_size is not a power of two in 1..1024.
 */
int verify_attn_build_block_table(const int32_t* kv_indptr, const int32_t* kv_indices,
                                  int32_t batch, int32_t page_size, int32_t max_pages_per_seq,
                                  int32_t* block_table, int32_t* kv_lens, void* stream);

/*
 * Split-KV pass (PR #27382 stage 1).  Sequence b owns the keys [lo_b, L_b + D):
 * its attended prefix (lo_b = max(0, L_b - W) with a window, else 0) and its D
 * draft keys.  The keys of all sequences, laid end to end, are cut into equal
 * ranges of about T / (workgroups) keys (at least ceil(max len / (S - 1))); a
 * range is split at sequence ends into pieces, and each piece is gathered through
 * the block table and attended by all G*D query rows of each KV head, row i
 * seeing keys p - W <= t <= p (p = L_b + i).  Piece k of sequence b writes its
 * partial output (normalised within the piece, times v_scale) and LSE to slot k
 * of the workspace, and the number of pieces of b is recorded there too.  The
 * ranges are derived on the device from prefix_lens; only host scalars size the
 * grid, and a sequence never spans more than S slots.
 * Errors: VA_EINVAL / VA_EUNSUPPORTED / VA_EWORKSPACE as for can_handle plus a
 * workspace check; VA_EHIP if the launch fails.
 */
int verify_attn_fwd(const verify_attn_args* args, void* stream);

/*
 * Combine (PR #27382 stage 2): per query row, the partials of the sequence's
 * pieces are merged by log-sum-exp into out (bf16) and lse (fp32, optional).  A
 * piece in which the row sees no key carries LSE = -inf and weight 0; every row
 * sees at least its own draft key.  Must follow verify_attn_fwd with the same
 * args on the same stream.
 */
int verify_attn_combine(const verify_attn_args* args, void* stream);

/*
 * Host-only gate (PR #27382's can_handle(): reads no device memory, so it is safe
 * during graph capture).  Returns VA_OK when fwd/combine serve these arguments,
 * else the status they would return (VA_EINVAL or VA_EUNSUPPORTED).  Does not
 * check the workspace size.
 */
int verify_attn_can_handle(const verify_attn_args* args);

/*
 * Split slots per (sequence, KV head) that the heuristic picks for these arguments
 * on the current device: how many programs the long shared prefix may be spread
 * over (PR #27382, "Motivation": split the prefix across parallel programs), from
 * the compute-unit count and the kernel the arguments select; args->num_splits is
 * ignored.  It takes the whole argument struct rather than a list of scalars because
 * the choice depends on every field the gate reads (KV dtype, qk_dim and v_dim, the
 * window, GQA ratio and draft length pick the kernel, and the kernel sets the tile
 * and per-piece cost).  Size the workspace with it once for the largest batch and
 * keep it (PR #27382 review: scratch keyed on a stable max batch).  Host only,
 * reads no device memory: the pointers may still be unset.  Returns >= 1, or -1
 * when the arguments are rejected (the status verify_attn_can_handle would give).
 */
int32_t verify_attn_num_splits(const verify_attn_args* args);

/*
 * Workspace bytes needed for num_splits partial slots (>= 1):
 *   (batch * hkv * num_splits * (hq/hkv * draft_len) * (v_dim + 1) + batch) * 4
 * (partial outputs, partial LSEs, one int32 piece count per sequence).
 * Host only.  Returns -1 on invalid input.  Size it once for the largest batch
 * and reuse it (PR #27382 review: scratch keyed on a stable max batch, fixed
 * addresses for graph replay).
 */
int64_t verify_attn_workspace_bytes(int32_t batch, int32_t hkv, int32_t hq, int32_t draft_len,
                                    int32_t v_dim, int32_t num_splits);

/*
 * Sliding-window pool slots (the unified-attention page's
 * translate_loc_from_full_to_swa before the page-table transform): for i < n,
 *     out[i] = full_to_swa[in[i]]
 * so layers with a separate sliding-window KV pool can build their block table
 * (verify_attn_build_block_table on `out`) from the full pool's token list.
 *   in          [n] int32 device full-pool slots, each in [0, map_len)
 *   full_to_swa [map_len] int32 device map
 *   out         [n] int32 device, written (may not alias in)
 * Errors: VA_EINVAL for n < 0, map_len < 1 or null pointers with n > 0.  Values of
 * `in` outside [0, map_len) are a precondition violation (not detected).
 */
int verify_attn_translate_slots(const int32_t* in, int64_t n, const int32_t* full_to_swa,
                                int64_t map_len, int32_t* out, void* stream);

/*
 * verify_attn_fwd followed by verify_attn_combine, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the partials live in a static per-device array of
 * VERIFY_ATTN_STATIC_SCRATCH_BYTES bytes (64 MiB) that the library's code object
 * holds on each device it runs on until the process ends, instead of in the caller's
 * workspace.  args->workspace and args->workspace_bytes are ignored.  The call makes
 * no allocation (no hipMalloc, no allocating library routine).
 *   num_splits = 0: the heuristic's slot count, lowered to the most the array holds;
 *   num_splits > 0: that count, or VA_EWORKSPACE when its partials
 *   (verify_attn_workspace_bytes) exceed the array.  VA_EWORKSPACE also when not even
 *   one slot per sequence fits.  Other errors as for verify_attn_fwd; VA_EHIP if the
 *   array's device address cannot be obtained.
 * Nothing in the array needs clearing between calls (the combine reads only what the
 * split-KV pass of the same call wrote), but every call on one device shares that
 * device's array: calls that overlap on one GPU (other streams, other threads) race
 * and must be serialised by the caller.
 */
#define VERIFY_ATTN_STATIC_SCRATCH_BYTES ((int64_t)64 << 20)
int verify_attn_fwd_combine_noalloc(const verify_attn_args* args, void* stream);

/* Text for a status code (static storage). */
const char* verify_attn_strerror(int status);

/* ABI version: bumps when verify_attn_args changes layout.  This header is version 2. */
int32_t verify_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VERIFY_ATTN_H */
