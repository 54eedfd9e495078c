/*
 * rr.h -- C ABI of the RRAttention sparse-prefill library (librr.so, gfx950).
 *
 * The method (RRAttention, arXiv 2602.05853): a per-head round-robin sample of
 * one query per stride of S tokens is scored against stride-pooled keys, a
 * causal stride-level softmax is pooled into B x B block scores, an adaptive
 * Top-tau rule keeps the smallest set of key blocks per query block-row whose
 * probability mass reaches tau, and causal attention runs on the kept blocks
 * only (RRAttention summary page, "Summary" and "Key points"; abstract; the
 * Top-tau rule follows the find_blocks definition on the XAttention review
 * page, "threshold block selection").
 *
 * Conventions for every entry point
 *  - Tensor pointers are DEVICE pointers to contiguous memory, batch 1.
 *    Q and O are [L][Hq][d]; K and V are [L][Hkv][d]; bf16 travels as its
 *    16-bit pattern (uint16_t).  Query head h reads kv-head h / (Hq/Hkv).
 *  - nb = ceil(L / B) key/query blocks; ns = L / S strides.
 *  - Supported shapes: d in {64, 128}; B in {64, 128}; S a power of two with
 *    S <= B; L % S == 0 (L % B may be nonzero: the last block is short);
 *    Hq % Hkv == 0; Hq <= 1024; nb <= 4096.
 *  - The caller owns every buffer (inputs, outputs and workspace).  The
 *    library never allocates, frees or synchronises; all work is enqueued on
 *    `stream` (a hipStream_t passed as void*, NULL = the null stream) and the
 *    call returns as soon as it is enqueued.  Nothing outside the given
 *    buffers is written.  Results are ready when the stream reaches them.
 *    Only kernels are enqueued (no memset, copy or host callback), so a call
 *    may be captured into a HIP graph and replayed on the same buffers.
 *  - Errors: argument checks run on the host before any launch and return a
 *    nonzero rr_status with no work enqueued; RR_E_HIP reports a failed
 *    launch (outputs are then undefined).  The library keeps no state and
 *    may be called from several host threads at once (on distinct buffers).
 */
#ifndef RR_H
#define RR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RR_OK = 0,
    RR_E_NULL = 1,        /* a required pointer is NULL */
    RR_E_SHAPE = 2,       /* non-positive size, Hq % Hkv, B % S or L % S nonzero, S > B */
    RR_E_TAU = 3,         /* tau is NaN or outside (0, 1] */
    RR_E_WORKSPACE = 4,   /* ws_bytes below the required workspace size */
    RR_E_UNSUPPORTED = 5, /* d, B or S outside the compiled instantiations, nb or Hq too large */
    RR_E_HIP = 6          /* a HIP launch failed */
} rr_status;

typedef enum {
    RR_OUT_BF16 = 0, /* O stored as bf16 (round to nearest even from fp32) */
    RR_OUT_F32 = 1   /* O stored as fp32 */
} rr_out_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char *rr_status_str(int status);

/* ABI version of this header (incremented on incompatible change). */
int rr_abi_version(void);

/*
 * rr_workspace_bytes -- one workspace size for a shape: the largest amount of
 * device workspace any entry point of this header needs for (L, Hq, Hkv, d,
 * B, S) (rr_estimate, rr_sparse_attn, rr_prefill, rr_xattn_estimate,
 * rr_estimate_materialized and rr_rescue_estimate), so that one caller-owned
 * buffer of this size serves every call on that shape.  0 if the shape is
 * invalid or unsupported (the same checks as the calls themselves).
 */
size_t rr_workspace_bytes(int L, int Hq, int Hkv, int d, int B, int S);

/*
 * Per-call workspace sizes in bytes (0 if the shape is invalid), each <=
 * rr_workspace_bytes.  The prefill size is large enough for each of the
 * three stage calls as well.
 */
size_t rr_estimate_workspace_bytes(int L, int Hq, int Hkv, int d, int B, int S);
size_t rr_sparse_attn_workspace_bytes(int L, int Hq, int Hkv, int d, int B);
size_t rr_prefill_workspace_bytes(int L, int Hq, int Hkv, int d, int B, int S);

/*
 * rr_estimate -- block scores of the round-robin estimate.
 * Per stride j and kv-head g the pooled key is the mean of the stride's S
 * keys ("scores are pooled per stride", RRAttention summary page, Summary).
 * Query head h scores token i*S + (h mod S) of every stride i (the offset
 * rotates from head to head, same passage) against pooled keys j <= i with
 * scale 1/sqrt(d); each such row is normalised by a softmax over j <= i
 * (stride-level softmax, Key points), and the probabilities are summed over
 * B x B blocks (stride-level aggregation, abstract).
 *   block_scores  out, fp32 [Hq][nb][nb]; entry (h, I, J) for J <= I, zero
 *                 for J > I.  Block-row I sums to the number of strides in
 *                 block I (B/S, fewer for a short last block).
 *   ws, ws_bytes  device workspace, >= rr_estimate_workspace_bytes(...).
 */
int rr_estimate(const uint16_t *Q, const uint16_t *K, int L, int Hq, int Hkv, int d, int B,
                int S, float *block_scores, void *ws, size_t ws_bytes, void *stream);

/*
 * rr_estimate_materialized -- the same block scores as rr_estimate, computed
 * by writing every stride score to memory and pooling it in a second pass
 * (the stride-level scoring, then the stride-level softmax and aggregation,
 * as separate steps: RRAttention summary page, Summary and Key points).  It
 * moves far more bytes than rr_estimate (at L = 128K, 32 heads, S = 8 the
 * scores alone are 17.2 GB, written once and read once) and exists to
 * expose the stride scores and to measure that design; rr_estimate keeps
 * only per-(row, block) statistics and is faster.
 *   stride_scores out, fp32, rr_stride_scores_count(...) floats.  For head h
 *                 and block-row I, row a (stride i = I*(B/S) + a) of that
 *                 block-row holds the scores of strides j = 0 .. (I+1)*(B/S)-1
 *                 at h*C*P + C*C*I*(I+1)/2 + a*(I+1)*C + j, where C = B/S and
 *                 P = C*nb*(nb+1)/2: s = (1/sqrt(d)) * log2(e) * Q[iS + (h mod
 *                 S)][h] . Kbar[j][g] (base-2 logits), -inf for j > i.  Rows
 *                 a past a short last block are not written.
 *   block_scores  out, fp32 [Hq][nb][nb], as for rr_estimate (agrees with it
 *                 to fp32 rounding of the sums).
 *   ws, ws_bytes  device workspace, >= rr_estimate_materialized_workspace_bytes.
 * Supported: B/S >= 4 (S <= B/4), else RR_E_UNSUPPORTED; other shape rules as
 * for rr_estimate.
 */
long long rr_stride_scores_count(int L, int Hq, int Hkv, int d, int B, int S);
size_t rr_estimate_materialized_workspace_bytes(int L, int Hq, int Hkv, int d, int B, int S);
int rr_estimate_materialized(const uint16_t *Q, const uint16_t *K, int L, int Hq, int Hkv, int d,
                             int B, int S, float *stride_scores, float *block_scores, void *ws,
                             size_t ws_bytes, void *stream);

/*
 * rr_select -- adaptive Top-tau per (query head, query block-row).
 * For block-row I of head h with W = sum_{J<=I} A[h][I][J]: order the blocks
 * by (score descending, block index ascending) and keep the shortest prefix
 * whose cumulative score is >= tau * W (find_blocks, XAttention review page,
 * threshold block selection); tau = 1 keeps every causal block.  Sums run in
 * fp32.
 *   block_scores  in, fp32 [Hq][nb][nb] (as written by rr_estimate).  The
 *                 rule is defined for finite scores >= 0, which is what the
 *                 estimators write; an entry J <= I that is negative, NaN or
 *                 infinite is read as 0 (zero mass, ordered by J among the
 *                 other zeros), so such input cannot break the ordering.
 *   counts        out, int32 [Hq][nb]: number of kept blocks (>= 1).
 *   block_idx     out, int32 [Hq][nb][nb]: kept key-block indices of row
 *                 (h, I) in ascending order in its first counts[h][I]
 *                 entries, -1 in the rest.
 */
int rr_select(const float *block_scores, int Hq, int L, int B, float tau, int32_t *counts,
              int32_t *block_idx, void *stream);

/*
 * rr_sparse_attn -- causal block-sparse attention with GQA over a compacted
 * block list (attention computed only on the kept blocks, abstract).
 * For token t in block I = t / B and head h the keys are the n <= t whose
 * block n / B is listed in block_idx[h][I][0 .. counts[h][I]); softmax of
 * (1/sqrt(d)) Q[t][h] . K[n][g] over them, applied to V[n][g].
 * Lists are read as rr_select writes them: ascending, in range J <= I.  Any
 * other list is accepted too: an entry out of range or repeated is ignored,
 * and the listed blocks are taken in ascending order whatever their order in
 * the list (the output is then bitwise that of the sorted list).  A row whose
 * list holds no valid block gets O = 0.
 *   O         out, [L][Hq][d] in o_dtype (rr_out_dtype).
 *   ws        device workspace, >= rr_sparse_attn_workspace_bytes(...).
 */
int rr_sparse_attn(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int L, int Hq,
                   int Hkv, int d, int B, const int32_t *counts, const int32_t *block_idx,
                   void *O, int o_dtype, void *ws, size_t ws_bytes, void *stream);

/*
 * rr_prefill -- the whole path: rr_estimate, rr_select and rr_sparse_attn on
 * one stream, with the block scores kept in the workspace.
 *   counts, block_idx  out, as for rr_select (the mask that was applied).
 *   ws                 device workspace, >= rr_prefill_workspace_bytes(...).
 */
int rr_prefill(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int L, int Hq, int Hkv,
               int d, int B, int S, float tau, void *O, int o_dtype, int32_t *counts,
               int32_t *block_idx, void *ws, size_t ws_bytes, void *stream);

/*
 * rr_prefill_noalloc -- rr_prefill for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same checks, kernels and results as rr_prefill, with
 * the workspace taken from a device array the library owns instead of from
 * the caller.  It allocates nothing and frees nothing.
 *   Arguments as for rr_prefill, minus ws / ws_bytes.
 *   Size limit: shapes whose rr_prefill_workspace_bytes(...) exceeds
 *   rr_noalloc_scratch_bytes() (64 MiB; e.g. L = 16384 at 32/8 heads, d = 128,
 *   B = 128, S = 8 fits, L = 32768 does not) return RR_E_WORKSPACE.
 *   `stream` must belong to the current device (else RR_E_UNSUPPORTED).
 * Every GPU the library runs on holds one 64 MiB array until the process
 * ends; its device address is looked up on the first call made on that
 * device.  All calls on one GPU share that array: calls that overlap on one
 * GPU (on different streams, or from several host threads) race and give
 * undefined results; calls ordered on one stream are safe.
 */
size_t rr_noalloc_scratch_bytes(void);
int rr_prefill_noalloc(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int L, int Hq,
                       int Hkv, int d, int B, int S, float tau, void *O, int o_dtype,
                       int32_t *counts, int32_t *block_idx, void *stream);

/*
 * rr_xattn_estimate -- XAttention's antidiagonal block scores (XAttention
 * review page, "importance prediction" and "threshold block selection"
 * steps 1-2), the estimator the RRAttention pages compare against, on the
 * same softmax pooling so that rr_select and rr_sparse_attn consume it
 * unchanged.  Inside each S x S sub-block (i, j) of the attention map the
 * antidiagonal logits are summed: x[h][i][j] = (1/sqrt(d)) * sum_{t<S}
 * Q[iS+t][h] . K[jS+S-1-t][g]; each stride row i is normalised by a softmax
 * over j <= i and the probabilities are summed over B x B blocks.
 *   average       0: the antidiagonal sum as the page states it; nonzero:
 *                 the sum divided by S (mean logit, so the softmax keeps the
 *                 temperature of single tokens), an alternative reading.
 *   block_scores  out, fp32 [Hq][nb][nb], as for rr_estimate.
 *   ws, ws_bytes  device workspace, >= rr_estimate_workspace_bytes(...).
 * Supported: B/S in {8, 16, 32} (S = 4, 8, 16 at B = 128), else
 * RR_E_UNSUPPORTED; other shape rules as for rr_estimate.
 */
int rr_xattn_estimate(const uint16_t *Q, const uint16_t *K, int L, int Hq, int Hkv, int d, int B,
                      int S, int average, float *block_scores, void *ws, size_t ws_bytes,
                      void *stream);

/*
 * rr_rescue_estimate -- block scores of an RBS-style rescue branch (RBS-
 * Attention page, abstract and method summary: a block centroid can hide one
 * highly relevant key, so a second branch built on the maximum key-block
 * radius flags blocks at risk; the branches are thresholded independently and
 * their masks combined).  The page gives no formula; the reading taken here:
 *   u[h][I][J] = (1/sqrt(d)) * (qc . kc_J + ||qc|| * r_J),   J <= I,
 * with qc the mean query of block I (head h), kc_J the mean key of block J
 * (kv-head g), r_J = max over the keys of block J of ||K[n] - kc_J||: the
 * largest logit qc can reach against a key of block J.  block_scores[h][I]
 * is the softmax of u over J <= I (rows sum to 1, zeros for J > I), so
 * rr_select keeps blocks with the branch's own tau and rr_merge_masks ORs
 * the result into another mask.  A short last block uses its own tokens.
 *   ws, ws_bytes  device workspace, >= rr_rescue_workspace_bytes(...).
 * Shapes: d in {64, 128}, B in {64, 128}, nb <= 4096 (no stride here).
 */
size_t rr_rescue_workspace_bytes(int L, int Hq, int Hkv, int d, int B);
int rr_rescue_estimate(const uint16_t *Q, const uint16_t *K, int L, int Hq, int Hkv, int d, int B,
                       float *block_scores, void *ws, size_t ws_bytes, void *stream);

/*
 * rr_merge_masks -- union of two kept-block masks given as lists (the
 * combined mask of two selection branches, RBS-Attention page).  Per (h, I)
 * the output lists every block J (0 <= J <= I) that either input lists, in
 * ascending order with -1 after counts[h][I] (the layout of rr_select).
 * Input entries past their count, out of range or repeated are ignored.
 * Outputs must not alias the inputs.
 */
int rr_merge_masks(const int32_t *counts_a, const int32_t *block_idx_a, const int32_t *counts_b,
                   const int32_t *block_idx_b, int Hq, int L, int B, int32_t *counts,
                   int32_t *block_idx, void *stream);

/*
 * rr_mask_quality -- how well a kept-block mask matches a reference mask and
 * how much block mass it keeps (precision and F1 of the selected blocks,
 * RRAttention summary page, Key points).  The intended reference is the
 * Top-tau selection on the exact attention mass of every block: rr_estimate
 * with S = 1 samples every token and pools nothing, so its block scores are
 * the exact causal softmax mass of each B x B block; rr_select on them with
 * the same tau gives the reference mask.
 * Per (head h, block-row I), over distinct listed blocks J with 0 <= J <= I
 * (entries past the count, out of range or repeated are ignored):
 *   kept  = blocks of the tested mask, ref = blocks of the reference mask,
 *   both  = blocks in both,
 *   share = sum of mass[h][I][J] over the tested mask's blocks
 *           / sum of mass[h][I][J] over all J <= I (0 if that sum is 0).
 *   counts, block_idx          in, the tested mask (layout of rr_select).
 *   ref_counts, ref_block_idx  in, the reference mask (same layout).
 *   mass                       in, fp32 [Hq][nb][nb] block mass (J <= I read).
 *   rows                       out, fp32 [Hq][nb][4]: kept, ref, both, share.
 *   totals                     out, fp64 [5]: sums of kept, ref, both and
 *                              share over all rows, then the minimum share.
 *                              Summed in a fixed order (reproducible).
 * Precision = both / kept, recall = both / ref, F1 = 2 both / (kept + ref).
 */
int rr_mask_quality(const int32_t *counts, const int32_t *block_idx, const int32_t *ref_counts,
                    const int32_t *ref_block_idx, const float *mass, int Hq, int L, int B,
                    float *rows, double *totals, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RR_H */
