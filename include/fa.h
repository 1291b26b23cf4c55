/*
 * fa.h -- C ABI of the MI355X (gfx950) exact causal attention library
 *         (FlashAttention-2 forward and backward).
 *
 * The operations are the ones the CS336 Assignment 2 handout states in
 * section 4.2 "FlashAttention-2" (videobook.pages.dev, Stanford-CS336 A2):
 *
 *   forward   (Eq. 4-6, Eq. 12, Algorithm 1)
 *       S = Q K^T * scale,  P = softmax_row(S)  (causal: key j allowed iff j <= i),
 *       O = P V,            L_i = log sum_j exp(S_ij)   (natural log, scaled scores)
 *   backward  (Eq. 13-19, Algorithm 2)
 *       D_i = rowsum(O o dO)_i,  P_ij = exp(S_ij - L_i),
 *       dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),
 *       dQ = dS K * scale,  dK = dS^T Q * scale
 *
 * Layout.  Every matrix argument (q, k, v, o, dout, dq, dk, dv) is one
 * contiguous row-major block [B][H][S][D] of `dtype` elements in device
 * memory (heads folded into the batch, as in the handout's launch grid
 * (T_q, batch)); lse and delta are contiguous [B][H][S] fp32.  Queries and
 * keys share the length S and both start at position 0, except in the
 * key-set calls (fa_fwd_partial, fa_bwd_partial), which take the two lengths
 * and the queries' offset from key 0 separately.
 *
 * Ownership.  The caller allocates every buffer (including the backward
 * workspace); the library never allocates, frees, copies to or from the
 * host, or synchronises.  (The one device memory it holds itself is the
 * fixed scratch array of fa_bwd_noalloc, part of its code object.)  Outputs
 * are fully overwritten; inputs must not alias outputs.  All pointers must
 * be device pointers aligned to 16 bytes.
 *
 * Streams and errors.  All work is enqueued on `stream` (0 = the null
 * stream).  Argument errors are returned synchronously, before anything is
 * enqueued.  Faults inside a kernel surface at the caller's next stream
 * synchronisation.  Launch shapes depend on the compute-unit count of the
 * stream's device, read once per device and cached.  The library is
 * thread-safe, except that fa_bwd_noalloc calls on one GPU share its scratch.
 *
 * Supported shapes.  D in {16, 32, 64, 80, 96, 128}; dtype FA_F32 or FA_BF16
 * (bf16 storage, bf16 matrix-core products with fp32 accumulation; the
 * softmax statistics, L and D are fp32).  scale must be finite and > 0.
 * B*H*S*D must fit in 63 bits; S <= 2^30 (tile positions stay within int).
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP's stream handle (identical to the typedef in hip_runtime_api.h). */
typedef struct ihipStream_t *hipStream_t;

/* Element type codes, passed to the entry points as an int `dtype`: any other
 * value returns FA_EUNSUPPORTED. */
typedef enum { FA_F32 = 0, FA_BF16 = 1 } fa_dtype;

/* Status codes: 0 = success; negative = error, and nothing was enqueued. */
enum {
    FA_OK = 0,
    FA_EINVAL = -1,       /* null pointer, B/H/S <= 0, causal not 0/1, scale <= 0 or not finite, size overflow */
    FA_EUNSUPPORTED = -2, /* D or dtype not built */
    FA_EALIGN = -3,       /* a pointer is not 16-byte aligned */
    FA_EWORKSPACE = -4,   /* workspace below B*H*S fp32 values (see fa_bwd) */
    FA_EHIP = -5,         /* the HIP runtime failed: no device visible for the stream,
                             a device query failed, or a launch was refused */
    FA_ESCRATCH = -6      /* fa_bwd_noalloc: B*H*S beyond its fixed device scratch */
};

/*
 * Forward pass (handout section 4.2.2, Algorithm 1; Eq. 4-6 and 12).
 *   q, k, v : [B][H][S][D] inputs          o   : [B][H][S][D] output
 *   lse     : [B][H][S] fp32 output, L_i = ln sum_{j allowed} exp(scale * q_i . k_j)
 *   causal  : 1 = key j is used by query i only when j <= i; 0 = all keys.
 * Tiles of keys that lie wholly above the diagonal are never visited.
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int H, int S, int D, float scale, int causal, int dtype,
           hipStream_t stream);

/*
 * Bytes of device workspace fa_fwd_ws can use for these sizes: 0 when it runs
 * as fa_fwd; otherwise n*B*H*S*(D+1) fp32 partial values (two regions, each
 * rounded up to 256 bytes; at most 256 MiB), for problems with few query
 * tiles per compute unit, whose longest tiles would walk many keys alone
 * (the size is that of causal = 1, which splits most; a non-causal call may
 * take fewer chunks).  The compute-unit count is the current device's (256, that of one
 * MI355X, when no device is visible).  Returns 0 for invalid sizes too.
 */
size_t fa_fwd_workspace_size(int B, int H, int S, int D, int dtype);

/*
 * fa_fwd with a caller workspace (same arguments, results and errors, plus
 * the workspace).  When the keys of a problem are worth splitting, it cuts
 * them into n chunks of whole 64-key tiles that run side by side as
 * fa_fwd_partial does, then merges the chunks' (O, L) exactly as fa_merge
 * does (the page "[Attention]FlashAttention/Ring-Attention/混合序列并行的统一原理",
 * sections "online softmax" and "online attention"; handout section 4.2.2 for
 * the forward itself).  The result
 * equals fa_fwd's up to the order of fp32 sums; it is deterministic.
 *   workspace : device memory of fa_fwd_workspace_size() bytes, 16-byte
 *               aligned, or NULL (then, or with fewer bytes than one split
 *               needs, it runs as fa_fwd; with fewer than the full size it
 *               takes as many chunks as fit).  Contents on entry do not
 *               matter; calls sharing a workspace must be ordered on one
 *               stream.
 */
int fa_fwd_ws(const void *q, const void *k, const void *v, void *o, float *lse, void *workspace,
              size_t workspace_bytes, int B, int H, int S, int D, float scale, int causal, int dtype,
              hipStream_t stream);

/*
 * Backward preprocessing (handout Algorithm 2, its first step, and the text
 * before Eq. 13): delta_i = sum_d o_id * dout_id, accumulated in fp32 from
 * the stored forward output o.
 *   o, dout : [B][H][S][D] inputs          delta : [B][H][S] fp32 output
 */
int fa_bwd_preprocess(const void *o, const void *dout, float *delta,
                      int B, int H, int S, int D, int dtype, hipStream_t stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes: B*H*S fp32 values
 * (rounded up to 256 bytes), where fa_bwd keeps lse in base 2 (L * log2 e)
 * so that recomputing P = 2^(S * scale * log2 e - L * log2 e) costs no
 * multiply per probability.  For problems with too few key tiles to fill
 * the GPU (S > 256 for bf16, S > 64 for fp32; the chunk count follows the
 * number of dK/dV workgroups per compute unit, S, D and the mask, as
 * fa_get_plan reports it), fa_bwd can instead cut each pass into n chunks
 * (n <= 8, 64-row multiples) that run side by side and sum their fp32
 * partial dQ, dK, dV in a fixed order (still bit-reproducible): the size
 * returned then adds 3*n*B*H*S*D fp32 values (at most 256 MiB).  The size
 * is that of the causal problem, which never takes fewer chunks than the
 * same problem without the mask.  The compute-unit count is the current
 * device's (that of one MI355X, 256, when no device is visible).
 * Returns 0 for invalid sizes; fa_bwd reports those.
 */
size_t fa_bwd_workspace_size(int B, int H, int S, int D, int dtype);

/*
 * Backward pass (handout section 4.2.3, Algorithm 2; Eq. 13-19), with the
 * probabilities recomputed from lse:
 *   q, k, v, dout : [B][H][S][D] inputs    lse, delta : [B][H][S] fp32 inputs
 *   dq, dk, dv    : [B][H][S][D] outputs
 *   workspace     : device scratch of fa_bwd_workspace_size() bytes,
 *                   16-byte aligned (FA_EINVAL if NULL).  Its contents on
 *                   entry do not matter and are overwritten.  Calls that
 *                   share one workspace must be ordered on one stream.  A
 *                   smaller workspace of at least B*H*S fp32 (rounded up to
 *                   256 bytes) is accepted too: the split backward then
 *                   takes only as many chunks as it holds partials for, and
 *                   none below two (equal results up to the order of fp32
 *                   sums, slower on few-head problems); below that,
 *                   FA_EWORKSPACE.
 * `scale` and `causal` must be the values the forward pass used.
 */
int fa_bwd(const void *q, const void *k, const void *v, const void *dout,
           const float *lse, const float *delta, void *dq, void *dk, void *dv,
           void *workspace, size_t workspace_bytes,
           int B, int H, int S, int D, float scale, int causal, int dtype,
           hipStream_t stream);

/*
 * Forward pass over shifted and/or split keys, producing partial results to
 * merge (the ring-attention page "[Attention]FlashAttention/Ring-Attention/
 * 混合序列并行的统一原理", sections "online softmax" and "online attention":
 * attention over a key set can be split along the keys and the parts merged
 * exactly).
 *   q          : [B][H][Sq][D] queries; query i sits q_offset positions after
 *                key 0 of this call (causal: key j is allowed iff j <= i + q_offset).
 *   k, v       : [B][H][Sk][D] keys and values.
 *   n_split    : the keys are cut into n_split chunks of
 *                chunk = 64 * ceil(Sk / (64 * n_split)) rows (the last one
 *                shorter or empty); chunk s holds keys [s*chunk, min((s+1)*chunk, Sk)).
 *   o_parts    : [n_split][B][H][Sq][D] fp32 output: for every chunk, the
 *                attention of each query over that chunk's allowed keys
 *                (normalised within the chunk).
 *   lse_parts  : [n_split][B][H][Sq] fp32 output: the chunk's
 *                L_i = ln sum_{j in chunk, allowed} exp(scale * q_i . k_j).
 *   A row that allows no key of a chunk gets O = 0 and L = -inf there.
 * With q_offset = 0, Sq = Sk and n_split = 1 this is fa_fwd with fp32 output.
 * Constraints as fa_fwd, plus 1 <= Sq, Sk <= 2^29, 1 <= n_split <= 65535 and
 * n_split*B*H*Sq*D within 63 bits.
 */
int fa_fwd_partial(const void *q, const void *k, const void *v, float *o_parts, float *lse_parts,
                   int B, int H, int Sq, int Sk, int D, float scale, int causal, int q_offset,
                   int n_split, int dtype, hipStream_t stream);

/*
 * Merge n_parts results over disjoint key sets of the same queries (the same
 * page, section "online attention": each part's output is rescaled by its
 * share of the common softmax denominator).  With M = max_r L_r:
 *   w_r = exp(L_r - M),  O = sum_r w_r O_r / sum_r w_r,  L = M + ln sum_r w_r;
 * a row empty in every part (all L_r = -inf) gives O = 0, L = -inf.
 *   o_parts   : [n_parts][B][H][S][D] fp32     lse_parts : [n_parts][B][H][S] fp32
 *   o         : [B][H][S][D] output in `dtype` lse       : [B][H][S] fp32 output
 * Parts are combined in a fixed order, so results are reproducible.
 * Constraints: n_parts >= 1 (and n_parts*B*H*S*D within 63 bits); D and
 * dtype as fa_fwd.
 */
int fa_merge(const float *o_parts, const float *lse_parts, int n_parts, void *o, float *lse,
             int B, int H, int S, int D, int dtype, hipStream_t stream);

/*
 * Gradient contributions of one key set, for attention split over keys (the
 * backward counterpart of fa_fwd_partial).  With the statistics L and Delta of
 * the whole attention, P_ij = exp(scale * q_i . k_j - L_i) (handout Eq. 14),
 * and each of dQ, dK, dV (Eq. 15-19) is a sum over keys or over queries, so
 * disjoint key sets contribute independently: this call adds
 *   dQ_i += scale * sum_{j in set} dS_ij k_j,   dK_j = scale * sum_i dS_ij q_i,
 *   dV_j = sum_i P_ij dO_i,   dS_ij = P_ij (dO_i . v_j - Delta_i),
 * over the allowed pairs (causal: j <= i + q_offset).
 *   q, dout         : [B][H][Sq][D] queries and output gradient.
 *   k, v            : [B][H][Sk][D] this key set.
 *   lse, delta      : [B][H][Sq] fp32 L (from fa_merge of every set, or fa_fwd)
 *                     and Delta (fa_bwd_preprocess of the final O and dout).
 *                     A row with L = -inf must allow no key of this set (as
 *                     it does when L covers every set); it contributes nothing.
 *   dq_acc          : [B][H][Sq][D] fp32 output.
 *   dk_acc, dv_acc  : [B][H][Sk][D] fp32 outputs.
 *   accumulate      : 0 = overwrite the outputs, 1 = add to them.
 * Outputs are fp32 for either input dtype so that contributions add without
 * intermediate rounding.  With q_offset = 0, Sq = Sk and accumulate = 0 this
 * is fa_bwd with fp32 outputs.  Constraints as fa_fwd_partial.
 */
int fa_bwd_partial(const void *q, const void *k, const void *v, const void *dout,
                   const float *lse, const float *delta, float *dq_acc, float *dk_acc,
                   float *dv_acc, int accumulate, int B, int H, int Sq, int Sk, int D,
                   float scale, int causal, int q_offset, int dtype, hipStream_t stream);

/*
 * fa_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  It computes what fa_bwd computes, with the same
 * arguments minus the workspace, and allocates nothing: its scratch is a
 * fixed 64 MiB array in device memory that the library holds on every GPU it
 * runs on until the process ends.  It holds the base-2 lse (B*H*S fp32), so
 * B*H*S must be at most 16777216 (FA_ESCRATCH otherwise), and the split
 * backward's partials when they fit beside it (fewer chunks than fa_bwd with
 * a full workspace may take; results equal up to the order of fp32 sums).
 * Every call on one GPU uses that GPU's one array: calls that may overlap on
 * a GPU (different streams, different threads) race and must be ordered by
 * the caller.  No call depends on what an earlier call left in it.
 */
int fa_bwd_noalloc(const void *q, const void *k, const void *v, const void *dout,
                   const float *lse, const float *delta, void *dq, void *dk, void *dv,
                   int B, int H, int S, int D, float scale, int causal, int dtype,
                   hipStream_t stream);

/*
 * The tile configuration fa_fwd and fa_bwd choose for a problem (handout,
 * leaderboard problem: the tile sizes are tuned to the shape), for a device
 * with num_cu compute units (num_cu <= 0: the current device's; FA_EHIP if
 * none is visible).  Launches use the count of the device they run on.
 */
typedef struct {
    int num_cu;             /* compute units the plan was made for */
    int fwd_block_queries;  /* queries per forward workgroup: 128, 256 or 512 */
    int fwd_key_groups;     /* 2: two wave groups split the key tiles and merge; else 1 */
    int fwd_key_tile;       /* keys per LDS tile of the forward */
    int fwd_band;           /* forward workgroup order: 0 = consecutive workgroups take
                               consecutive heads; b > 0 = each of the 8 XCDs takes every
                               8th head, in bands of b query tiles per head (B*H a
                               multiple of 8) */
    int bwd_chunks;         /* chunks of the causal split backward (1: not split), with
                               a workspace of fa_bwd_workspace_size() bytes; without
                               the mask fa_bwd may take fewer */
    int bwd_chunk_rows;     /* rows per chunk (S when not split) */
} fa_plan;

int fa_get_plan(int B, int H, int S, int D, int dtype, int num_cu, fa_plan *plan);

/* Static, human-readable text for a status code. */
const char *fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
