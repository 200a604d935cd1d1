/*
 * fa.h -- C ABI of the MI355X (gfx950) FlashAttention-2 library: the
 * forward pass (fa_fwd, fa_fwd_ws; fa_fwd_varlen and fa_fwd_varlen_ws for
 * variable-length batches, fa_fwd_masked and fa_fwd_masked_ws for
 * local-window + global-token masks, fa_fwd_fp8
 * and fa_fwd_fp8_ws for FP8 inputs) and its
 * backward pass (fa_bwd, fa_bwd_varlen, fa_bwd_masked).
 *
 * The operation (page "FlashAttention-2实现与优化：高效注意力机制详解",
 * §3.1 PyTorch forward and §3.2 Triton forward; page
 * "解释FlashAttention的显存优化原理" §一.2 tiling): for every batch b, head h
 * and query row i,
 *
 *     s_ij = scale * <q_i, k_j>          for the keys j visible to row i
 *     O_i  = sum_j softmax_j(s_i.) v_j
 *     L_i  = ln sum_j exp(s_ij)          (the per-row logsumexp, m + ln l)
 *
 * computed tile by tile with an online softmax, so the Nq x Nk score matrix
 * never exists in device memory.  With causal != 0, key j is visible to row
 * i iff j <= i (indices from 0 in both sequences, the masking rule of the
 * same page, §4.3); otherwise every key j < Nk is visible.
 *
 * Layout.  q is [B,H,Nq,D], k and v are [B,H,Nk,D], o is [B,H,Nq,D] and lse
 * is [B,H,Nq]; all contiguous, row-major, in device memory.  Element types:
 *
 *   dtype           q, k, v   o      lse   contraction
 *   FA_F32          fp32      fp32   fp32  fp32 products, fp32 sums
 *   FA_BF16         bf16      bf16   fp32  bf16 products, fp32 sums
 *   FA_BF16_OF32    bf16      fp32   fp32  as FA_BF16, O kept in fp32
 *   FA_F16          fp16      fp16   fp32  fp16 products, fp32 sums
 *   FA_F16_OF32     fp16      fp32   fp32  as FA_F16, O kept in fp32
 *
 * With 16-bit inputs the softmax, its statistics and the O accumulator are
 * fp32; the probabilities are rounded to the input type before they
 * multiply V, as in the Triton forward of the same page (§3.2, §4.2).  O is
 * rounded to its storage type once, at the end.
 *
 * Ownership.  Every pointer belongs to the caller.  The library allocates,
 * frees and synchronises nothing; it only enqueues work on `stream`.
 *
 * Thread safety.  Calls may be made concurrently from any host thread.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage types of (q, k, v ; o).  lse is always fp32. */
enum fa_dtype {
    FA_F32 = 0,
    FA_BF16 = 1,
    FA_BF16_OF32 = 2,
    FA_F16 = 3,
    FA_F16_OF32 = 4
};

/* Status codes.  Validation errors are reported before any device work is
 * enqueued, so on a non-zero return nothing has been written. */
enum fa_status {
    FA_OK = 0,
    FA_ERR_NULLPTR = 1,  /* q, k, v, o or lse is NULL                        */
    FA_ERR_SHAPE = 2,    /* B, H, Nq or Nk < 1, or a size overflows          */
    FA_ERR_HEAD_DIM = 3, /* D not in {16, 32, 64, 128}                       */
    FA_ERR_DTYPE = 4,    /* dtype is not one of enum fa_dtype                */
    FA_ERR_SCALE = 5,    /* scale is NaN or infinite                          */
    FA_ERR_ALIGN = 6,    /* q, k, v or o not 16-byte aligned, lse not 4-byte */
    FA_ERR_HIP = 7,      /* the HIP runtime refused the launch               */
    FA_ERR_OVERLAP = 8,  /* o, lse or workspace overlaps an input or another
                            output                                           */
    FA_ERR_WORKSPACE = 9 /* workspace NULL or smaller than the call needs     */
};

/*
 * fa_fwd -- enqueue one attention forward pass on `stream`.
 *
 *   q          device pointer, [B,H,Nq,D] of the dtype's input type
 *   k, v       device pointers, [B,H,Nk,D] of the input type
 *   o          device pointer, [B,H,Nq,D] of the dtype's output type (written)
 *   lse        device pointer, [B,H,Nq] fp32, natural-log logsumexp (written)
 *   B, H       batch size and number of heads (>= 1)
 *   Nq, Nk     query and key sequence lengths (>= 1; need not be equal, need
 *              not be multiples of any tile size)
 *   D          head dimension: 16, 32, 64 or 128
 *   scale      multiplier of q.k (the pages use 1/sqrt(D)); any finite value
 *   causal     0: all keys visible; non-zero: key j visible to row i iff j<=i
 *   dtype      one of enum fa_dtype
 *   stream     a hipStream_t (NULL = the default stream)
 *
 * Returns FA_OK once the work is enqueued (asynchronous, like any launch:
 * results are valid after the stream is synchronised), a validation error
 * (nothing enqueued), or FA_ERR_HIP with the runtime's message available
 * from fa_last_hip_error().  o and lse must not overlap q, k, v or each
 * other (checked on the host: FA_ERR_OVERLAP).  Each (batch, head) slice is
 * addressed with 32-bit byte offsets, so (Nq + 256) * D * 4 and
 * (Nk + 64) * D * 4 must stay below 2^31 (FA_ERR_SHAPE otherwise), as must
 * B*H*ceil(Nq/128).
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
           float scale, int causal, int dtype, void *stream);

/*
 * fa_fwd_workspace_size -- device scratch bytes that fa_fwd_ws needs for
 * this problem on the current device (written to *bytes; 0 when fa_fwd_ws
 * takes the same path as fa_fwd: 16-bit inputs with at least four query
 * tiles of 128 rows per compute unit, or fp32 inputs with at least one per
 * compute unit, where one workgroup per tile already keeps every unit
 * busy, or a single 64-key tile per query tile).
 *
 * One workgroup per query tile leaves compute units idle when tiles are
 * few or, under the causal mask, of very unequal length.  fa_fwd_ws instead
 * lays all the work out as one sequence of (query tile, 64-key tile) units
 * and gives each compute unit an equal contiguous share of it (a stream-K
 * schedule, with query tiles in zigzag order so that every share mixes
 * short and long causal rows).  A query tile cut between two shares keeps
 * one partial (running max, sum, O) per share in the workspace, and a
 * second kernel combines them with the rescaling that the online softmax
 * applies when it folds one key block into the running statistics (page
 * "FlashAttention-2实现与优化：高效注意力机制详解" §3.1, the incremental
 * update of (m, l, o_acc)).  Cutting the work along the sequence is the
 * sequence parallelism of page "FlashAttention技术演进全景图" §3.2.  The size
 * is 2 * G * R * (D + 4) * 4 bytes, G = min(compute units, 256, units of work),
 * R the rows of a query tile in this schedule (256, or 128 at D = 128
 * when there are fewer 256-row tiles than compute units and the work per
 * compute unit is under 64 tiles of 128 x 64, or, non-causal, at most one
 * 128-row tile per compute unit).
 *
 * fp32 inputs take a simpler split: each 128-row query tile's keys are cut
 * into n <= 4 chunks of KC 64-key tiles (KC the smallest length that keeps
 * the workgroups within one per compute unit), each chunk run by its own
 * workgroup and the chunks combined by a second kernel as above.  The size
 * is then T * n * 128 * (D + 4) * 4 bytes for T query tiles.
 *
 * Returns FA_OK, FA_ERR_NULLPTR (bytes NULL), FA_ERR_SHAPE, FA_ERR_HEAD_DIM,
 * FA_ERR_DTYPE or FA_ERR_HIP (device query failed).
 */
int fa_fwd_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                          int64_t D, int causal, int dtype, size_t *bytes);

/*
 * fa_fwd_ws -- fa_fwd with caller-owned device scratch.
 *
 * Arguments as fa_fwd, plus
 *   workspace        device pointer, 16-byte aligned, or NULL when
 *                    fa_fwd_workspace_size reports 0 bytes (then the call
 *                    is fa_fwd)
 *   workspace_bytes  its size in bytes
 *
 * Computes the same O and lse as fa_fwd up to fp32 rounding order (the
 * parts are combined in a different order).  The workspace is overwritten
 * and holds nothing of use afterwards; two calls that share one workspace
 * must be ordered (the same stream).  Returns fa_fwd's codes, and
 * FA_ERR_WORKSPACE when the plan needs scratch and `workspace` is NULL or
 * smaller than fa_fwd_workspace_size reports; FA_ERR_ALIGN and
 * FA_ERR_OVERLAP also cover the workspace.
 */
int fa_fwd_ws(const void *q, const void *k, const void *v, void *o, float *lse,
              int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
              float scale, int causal, int dtype, void *workspace,
              size_t workspace_bytes, void *stream);

/*
 * fa_fwd_noalloc -- fa_fwd_ws without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Arguments, results and errors as fa_fwd_ws; the stream-K schedule's
 * partial results go to a scratch array inside the library, one copy per
 * device (FA_NOALLOC_SCRATCH_BYTES, held until the process ends; its
 * address is looked up on the first call on each device).  A plan that
 * needs more scratch than that returns FA_ERR_WORKSPACE (on devices of up
 * to 256 compute units no plan does).  The call enqueues the same kernels
 * as fa_fwd_ws and allocates, frees and synchronises nothing.  Every call
 * on one device shares that device's scratch: calls that may run at the
 * same time on one device (different streams, or graphs replayed
 * concurrently) race and must be ordered by the caller.  Nothing in the
 * scratch needs to start at zero (every slot a combine reads was written
 * by the same call).
 */
#define FA_NOALLOC_SCRATCH_BYTES (72u * 1024u * 1024u)
int fa_fwd_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                   int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                   float scale, int causal, int dtype, void *stream);

/*
 * fa_fwd_varlen -- the forward pass over a variable-length batch (page
 * "FlashAttention-2实现与优化：高效注意力机制详解" §7, ragged input sequences).
 *
 *   q          device pointer, [H, Tq, D] of the dtype's input type: S
 *              sequences packed along the token axis, sequence s at rows
 *              cu_seqlens_q[s] .. cu_seqlens_q[s+1] - 1 of every head
 *   k, v       device pointers, [H, Tk, D]; sequence s at rows
 *              cu_seqlens_k[s] .. cu_seqlens_k[s+1] - 1
 *   o          device pointer, [H, Tq, D] of the dtype's output type (written)
 *   lse        device pointer, [H, Tq] fp32 (written)
 *   cu_seqlens_q, cu_seqlens_k
 *              device pointers to S + 1 int32 offsets each, starting at 0,
 *              non-decreasing, ending at Tq / Tk
 *   S, H       number of sequences (>= 1) and heads (>= 1)
 *   Tq, Tk     total query rows (>= 1) and key rows (>= 0)
 *   max_seqlen_q  an upper bound of every query length.  A sequence longer
 *              than it is computed up to the end of the query tile that
 *              holds row max_seqlen_q - 1 (128 or 256 rows); its rows past
 *              that tile get O = NaN and lse = NaN, so no row is left
 *              unwritten
 *   D, scale, causal   as fa_fwd; the causal rule applies within each
 *              sequence: key j of a sequence is visible to its row i iff
 *              j <= i (indices from the sequence's first row)
 *   dtype      FA_BF16, FA_BF16_OF32, FA_F16 or FA_F16_OF32 (FA_F32 is not
 *              supported here: FA_ERR_DTYPE)
 *
 * Each sequence attends only to its own keys; its rows get exactly what
 * fa_fwd computes for that sequence alone.  A sequence with queries and no
 * keys gets O = 0 and lse = -inf.  The offsets live in device memory and
 * are read by the kernel, which clamps them to [0, Tq] / [0, Tk]: offsets
 * that break the rules above give wrong rows but never an access outside
 * the tensors.  Validation, ownership and error codes as fa_fwd (the
 * offsets need 4-byte alignment).
 */
int fa_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                  const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                  int64_t S, int64_t H, int64_t Tq, int64_t Tk,
                  int64_t max_seqlen_q, int64_t D, float scale, int causal,
                  int dtype, void *stream);

/*
 * fa_fwd_varlen_workspace_size -- device scratch bytes that fa_fwd_varlen_ws
 * needs for this problem on the current device (written to *bytes; 0 when
 * no query tile is split, and then fa_fwd_varlen_ws is fa_fwd_varlen).
 *
 * Arguments as fa_fwd_varlen, plus max_seqlen_k (>= 0), an estimate of the
 * longest key length; 0 asks for no split.  Two schedules split work over
 * the keys (sequence parallelism, page "FlashAttention技术演进全景图"
 * §3.2), and a second kernel combines the partial results with the
 * online-softmax rescaling of page
 * "FlashAttention-2实现与优化：高效注意力机制详解" §3.1:
 *   - at most 512 (head, sequence) pairs (H * S <= 512): a stream
 *     schedule.  G = min(compute units, 256) workgroups each take an equal
 *     share of the call's (query tile, 64-key tile) units, counted from the
 *     offsets in device memory, so the work is balanced whatever the
 *     lengths; a query tile cut between two workgroups is combined by the
 *     second kernel.  Workspace: 2 G partial tiles of 128 or 256 rows by
 *     (D + 4) fp32, rounded up to 256 bytes, and 12 G bytes for the cuts.
 *   - more pairs: a tile whose key range is longer than the call's share
 *     per compute unit (bounded with max_seqlen_q and max_seqlen_k) is cut
 *     into at most 16 chunks, each run by its own workgroup.
 * Returns FA_OK, or the shape / head-dim / dtype errors of fa_fwd_varlen,
 * FA_ERR_NULLPTR (bytes NULL) or FA_ERR_HIP.
 */
int fa_fwd_varlen_workspace_size(int64_t S, int64_t H, int64_t Tq, int64_t Tk,
                                 int64_t max_seqlen_q, int64_t max_seqlen_k,
                                 int64_t D, int causal, int dtype, size_t *bytes);

/*
 * fa_fwd_varlen_ws -- fa_fwd_varlen with work split over the keys and
 * caller-owned device scratch.
 *
 * Arguments as fa_fwd_varlen, plus
 *   max_seqlen_k     as for fa_fwd_varlen_workspace_size; with max_seqlen_q
 *                    it steers the schedule only (which one, the tile
 *                    height, the chunk sizes): every key is seen whatever
 *                    the real lengths
 *   workspace        device pointer, 16-byte aligned, of at least the bytes
 *                    fa_fwd_varlen_workspace_size reports for the same
 *                    arguments, or NULL when it reports 0
 *   workspace_bytes  its size in bytes
 *
 * Results as fa_fwd_varlen up to the order of the fp32 summation (split
 * tiles add their chunks' partial sums in a different order), with one
 * difference under the stream schedule (H * S <= 512): it walks the offsets
 * themselves, so the rows of a sequence longer than max_seqlen_q are all
 * computed instead of set to NaN.  Calls that share a workspace must be
 * ordered on one stream.  Errors as fa_fwd_varlen, plus FA_ERR_WORKSPACE
 * (workspace NULL or too small), FA_ERR_ALIGN and FA_ERR_OVERLAP for the
 * workspace.
 */
int fa_fwd_varlen_ws(const void *q, const void *k, const void *v, void *o,
                     float *lse, const int32_t *cu_seqlens_q,
                     const int32_t *cu_seqlens_k, int64_t S, int64_t H, int64_t Tq,
                     int64_t Tk, int64_t max_seqlen_q, int64_t max_seqlen_k,
                     int64_t D, float scale, int causal, int dtype,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * fa_fwd_masked -- the forward pass under a local-window + global-token
 * mask (page "FlashAttention-2实现与优化：高效注意力机制详解" §7, sparse
 * attention combining local windows and global tokens; the pages give no
 * definition, so this library reads it as): key j (< Nk) is visible to
 * query i iff
 *
 *     (causal ? 0 <= i - j < window : |i - j| < window)
 *  or (j < nglobal || i < nglobal) && (!causal || j <= i)
 *
 * and each row is the softmax over its visible keys: O_i and L_i as fa_fwd
 * computes them over that key set.  A row with no visible key (only when
 * Nq > Nk) gets O = 0 and lse = -inf.  With window >= max(Nq, Nk) and
 * nglobal = 0 this is fa_fwd's operation.
 *
 *   q, k, v, o, lse, B, H, Nq, Nk, scale, causal   as fa_fwd
 *   D          16, 32, 64 or 128
 *   window     >= 1 (window 1 leaves the diagonal)
 *   nglobal    >= 0: the first nglobal queries and keys are global tokens
 *   dtype      FA_BF16, FA_BF16_OF32, FA_F16 or FA_F16_OF32 (FA_F32:
 *              FA_ERR_DTYPE)
 *
 * It runs fa_fwd's pipelined kernel, one workgroup per 256-row query tile,
 * over that tile's 64-key tiles that hold a visible pair: the global
 * tokens' tiles, then the band's.  Scores of hidden pairs inside those tiles
 * are masked, so the work is proportional to the visible pairs, rounded up
 * to whole tiles.  Status codes as fa_fwd; window < 1 or nglobal < 0 is
 * FA_ERR_SHAPE.
 */
int fa_fwd_masked(const void *q, const void *k, const void *v, void *o, float *lse,
                  int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                  float scale, int causal, int64_t window, int64_t nglobal,
                  int dtype, void *stream);

/*
 * fa_fwd_masked_workspace_size -- device scratch bytes that let
 * fa_fwd_masked_ws split long tiles (written to *bytes; 0 when nothing is
 * split).  Without the causal rule a 256-row tile that holds a global
 * query sees every key, far more than a band tile: the first
 * ceil(min(nglobal, Nq) / 256) tiles of every (batch, head) are cut into
 * P parts along the keys (each about a band tile's key range, at least 32
 * key tiles of 64), each leaving 256 x (D + 4) fp32 values; the size is
 * B * H * ceil(min(nglobal, Nq) / 256) * P * 256 * (D + 4) * 4 bytes.
 * The query needs no device.  Returns FA_OK, FA_ERR_NULLPTR, FA_ERR_SHAPE
 * (also window < 1 or nglobal < 0), FA_ERR_HEAD_DIM or FA_ERR_DTYPE.
 */
int fa_fwd_masked_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                 int64_t D, int causal, int64_t window,
                                 int64_t nglobal, int dtype, size_t *bytes);

/*
 * fa_fwd_masked_ws -- fa_fwd_masked with a caller-owned workspace (device
 * memory, 16-byte aligned, overlapping no other argument; NULL or fewer
 * than fa_fwd_masked_workspace_size bytes: the long tiles run whole, as in
 * fa_fwd_masked).  The split parts' partial results are combined by a
 * second kernel in part order (deterministic; the same results as the
 * unsplit call within the rounding of that combination).  Calls that share
 * a workspace must not overlap.  Arguments and status codes otherwise as
 * fa_fwd_masked (FA_ERR_ALIGN, FA_ERR_OVERLAP for the workspace).
 */
int fa_fwd_masked_ws(const void *q, const void *k, const void *v, void *o,
                     float *lse, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                     int64_t D, float scale, int causal, int64_t window,
                     int64_t nglobal, int dtype, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * fa_fwd_fp8 -- the forward pass with FP8 inputs (page "FlashAttention技术
 * 演进全景图" §5.3 names FP8 support; the pages give no rules, so this
 * library reads it as): q, k, v hold OCP e4m3 values (one byte each,
 * [B,H,N,D] contiguous) and the real inputs are those values times the
 * per-tensor factors descale_q, descale_k, descale_v.  The result is fa_fwd's
 * O and lse for the real inputs; O is bf16 (out_f32 = 0) or fp32 (out_f32 !=
 * 0).  The score products run on FP8 MFMAs with fp32 sums (exact products);
 * P.V runs in bf16 (V's e4m3 values widen exactly; P is rounded to bf16 as
 * on the 16-bit path).  D must be 64 or 128.  Other arguments, ownership and
 * status codes as fa_fwd (FA_ERR_SCALE also when a factor, or their product
 * with scale, is not finite).
 */
int fa_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse,
               int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, float scale,
               float descale_q, float descale_k, float descale_v, int causal,
               int out_f32, void *stream);

/*
 * fa_fwd_fp8_workspace_size -- device scratch bytes that fa_fwd_fp8_ws
 * needs (written to *bytes): V widened to bf16 (B*H*Nk*D*2 bytes, rounded
 * up to 256), plus, when the shape takes the stream-K schedule of fa_fwd_ws
 * (same rule as for bf16 inputs), that schedule's partials.  Returns FA_OK,
 * FA_ERR_NULLPTR (bytes NULL), FA_ERR_SHAPE, FA_ERR_HEAD_DIM (D not 64 or
 * 128) or FA_ERR_HIP.
 */
int fa_fwd_fp8_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                              int64_t D, int causal, int out_f32, size_t *bytes);

/*
 * fa_fwd_fp8_ws -- fa_fwd_fp8 on the pipelined kernel of fa_fwd_ws, with
 * caller-owned device scratch (FP8 support, page "FlashAttention技术演进全景图"
 * §5.3; the work split of §3.2 there).  The score products K.Q^T run on the
 * FP8 MFMA (e4m3 operands, fp32 sums: exact products) with q and k read as
 * stored; V's e4m3 values are first widened exactly to bf16 into the
 * workspace by a separate kernel, and P.V runs on the bf16 MFMA with P
 * rounded to bf16 as on the 16-bit path; descale_v multiplies O in fp32 at
 * the normalisation.  Arguments, results and errors as fa_fwd_fp8, plus
 *   workspace        device pointer, 16-byte aligned, of at least the bytes
 *                    fa_fwd_fp8_workspace_size reports for the same shape
 *   workspace_bytes  its size in bytes
 * and FA_ERR_WORKSPACE (workspace NULL or too small), FA_ERR_ALIGN and
 * FA_ERR_OVERLAP for the workspace.  Calls that share a workspace must be
 * ordered on one stream.
 */
int fa_fwd_fp8_ws(const void *q, const void *k, const void *v, void *o, float *lse,
                  int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, float scale,
                  float descale_q, float descale_k, float descale_v, int causal,
                  int out_f32, void *workspace, size_t workspace_bytes, void *stream);

/*
 * fa_bwd_workspace_size -- device scratch bytes for fa_bwd (written to
 * *bytes): B * H * Nq * 4, one fp32 row term per query row; at D = 64 and
 * 128, when a stream-K schedule may run (fewer than two 128-row query tiles,
 * or 128-key tiles, per compute unit), that rounded up to 256 bytes plus the
 * larger of the two schedules' partial sums: for dQ two slots of 128 x D
 * fp32 per chunk, for dK/dV two slots of 2 x 128 x D fp32 per chunk, at most
 * 256 chunks (the figure covers every device of up to 256 compute units).
 * fa_bwd needs only the row terms; with less than this size it runs one
 * workgroup per tile instead of the stream schedule (same results within
 * fp32 rounding of the sums' order).  The query needs no device.
 *
 * Returns FA_OK, FA_ERR_NULLPTR (bytes NULL), FA_ERR_SHAPE, FA_ERR_HEAD_DIM
 * or FA_ERR_DTYPE, with the rules of fa_bwd.
 */
int fa_bwd_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                          int64_t D, int causal, int dtype, size_t *bytes);

/*
 * fa_bwd -- enqueue the backward pass of fa_fwd on `stream`: the gradients
 * dq, dk, dv of sum(dout * O) for the upstream gradient dout of O.
 *
 * The pages describe the backward pass as recomputing the attention
 * probabilities block by block from the saved logsumexp instead of storing
 * them (page "解释FlashAttention的显存优化原理" §一.2(2); page
 * "FlashAttention-2实现与优化：高效注意力机制详解" §3.1 saves q, k, v, o and L
 * for it, §7 lists it as the next step).  With P_ij = exp(scale <q_i, k_j>
 * - L_i) over the visible pairs (the forward's mask rule):
 *
 *     dv_j = sum_i P_ij dout_i
 *     dS_ij = P_ij (<dout_i, v_j> - <dout_i, o_i>)
 *     dq_i = scale sum_j dS_ij k_j,     dk_j = scale sum_i dS_ij q_i
 *
 *   q, k, v    the forward's inputs, [B,H,Nq,D] / [B,H,Nk,D], 16-bit
 *   o          the forward's output O, [B,H,Nq,D], same 16-bit type
 *   lse        the forward's L, [B,H,Nq] fp32
 *   dout       upstream gradient of O, [B,H,Nq,D], same 16-bit type
 *   dq         [B,H,Nq,D] (written); dk, dv [B,H,Nk,D] (written)
 *   B .. causal  as fa_fwd; D must be 16, 32, 64 or 128
 *   dtype      FA_BF16 / FA_F16: every tensor in that type (gradients
 *              rounded once, at the end); FA_BF16_OF32 / FA_F16_OF32: the
 *              same inputs, gradients stored in fp32.  FA_F32 is not
 *              supported here (FA_ERR_DTYPE).
 *   workspace  device pointer, 16-byte aligned, at least B * H * Nq * 4
 *              bytes; fa_bwd_workspace_size bytes let the stream-K
 *              schedules run (overwritten, as far as the call uses it)
 *   stream     a hipStream_t (NULL = the default stream)
 *
 * Products are formed from 16-bit operands with fp32 accumulation; P and dS
 * are rounded to the input type before they multiply dout, q and k.  Every
 * gradient element is written by exactly one workgroup, with plain stores
 * (a tile split by a stream-K schedule leaves fp32 partial sums in the
 * workspace, added in a fixed order by a second kernel): results are
 * deterministic.  Returns FA_OK once enqueued, a validation
 * error (nothing enqueued: FA_ERR_NULLPTR, FA_ERR_SHAPE, FA_ERR_HEAD_DIM,
 * FA_ERR_DTYPE, FA_ERR_SCALE, FA_ERR_ALIGN, FA_ERR_WORKSPACE, or
 * FA_ERR_OVERLAP when dq, dk, dv or the workspace overlap an input or each
 * other), or FA_ERR_HIP.  The library allocates nothing.
 */
int fa_bwd(const void *q, const void *k, const void *v, const void *o,
           const float *lse, const void *dout, void *dq, void *dk, void *dv,
           int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
           float scale, int causal, int dtype, void *workspace,
           size_t workspace_bytes, void *stream);

/*
 * fa_bwd_masked_workspace_size -- device scratch bytes for fa_bwd_masked
 * with this rule (written to *bytes): B * H * Nq * 4 (the row terms, as
 * fa_bwd_workspace_size); at D = 64 and 128 with nglobal > 0, when tiles
 * that hold global tokens meet many more tiles than a band tile does, that
 * rounded up to 256 bytes plus the larger of two part areas: dK/dV (D = 64,
 * and D = 128 under the causal rule), B * H * ceil(min(nglobal, Nk) / 128)
 * * P slots of 2 x 128 x D fp32 for the 128-key tiles that hold global
 * keys; dQ (without the causal rule), B * H * ceil(min(nglobal, Nq) / 128)
 * * P' slots of 128 x D fp32 for the 128-row tiles that hold global
 * queries.  P and P' are the numbers of parts each such tile's walk is cut
 * into (each part about a band tile's walk, at least 32 tiles of 64).
 * The query needs no device.  Returns FA_OK, FA_ERR_NULLPTR,
 * FA_ERR_SHAPE (also window < 1 or nglobal < 0), FA_ERR_HEAD_DIM or
 * FA_ERR_DTYPE.
 */
int fa_bwd_masked_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                 int64_t D, int causal, int64_t window,
                                 int64_t nglobal, int dtype, size_t *bytes);

/*
 * fa_bwd_masked -- fa_bwd under the local-window + global-token mask of
 * fa_fwd_masked (same window, nglobal and causal rule; o and lse from
 * fa_fwd_masked): the gradients of its O over the visible pairs.  Rows
 * without a visible key get dq = 0; keys no row sees get dk = dv = 0.
 * Query and key blocks without a visible pair are skipped.  The workspace
 * needs the row terms (B * H * Nq * 4 bytes); with
 * fa_bwd_masked_workspace_size bytes the tiles that hold global tokens are
 * cut into parts that run in parallel and whose fp32 partial sums are
 * added in part order (deterministic; with less they run whole, the same
 * results within the rounding of the sums' order).  Arguments, dtypes,
 * head dims and status codes as fa_bwd; window < 1 or nglobal < 0 is
 * FA_ERR_SHAPE.
 */
int fa_bwd_masked(const void *q, const void *k, const void *v, const void *o,
                  const float *lse, const void *dout, void *dq, void *dk, void *dv,
                  int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                  float scale, int causal, int64_t window, int64_t nglobal,
                  int dtype, void *workspace, size_t workspace_bytes, void *stream);

/*
 * fa_bwd_varlen -- fa_bwd over a variable-length batch laid out as for
 * fa_fwd_varlen: q, o, dout, dq [H, Tq, D]; k, v, dk, dv [H, Tk, D]; lse
 * [H, Tq]; sequence s at rows cu_seqlens_q[s] .. cu_seqlens_q[s+1] - 1 (keys
 * cu_seqlens_k[s] .. cu_seqlens_k[s+1] - 1), offsets in device memory
 * (S + 1 int32 each, 0 .. Tq / Tk, non-decreasing; the kernels clamp them
 * to the tensors).  max_seqlen_q and max_seqlen_k bound every sequence's
 * query and key count: a longer sequence is computed up to the end of the
 * 64-row tile that holds row max_seqlen_q - 1 (key max(max_seqlen_k, 1) - 1),
 * and its dq rows (dk and dv rows) past that tile are set to NaN, so no row
 * is left unwritten.  Each sequence's gradients are exactly fa_bwd's for that
 * sequence alone; keys that no query sees get dk = dv = 0, queries without
 * keys get dq = 0.  The workspace needs H * Tq * 4 bytes (the row terms of
 * fa_bwd_workspace_size for B = 1, Nq = Tq).  Other arguments,
 * dtypes, head dims and status codes as fa_bwd (the offsets need 4-byte
 * alignment).
 */
int fa_bwd_varlen(const void *q, const void *k, const void *v, const void *o,
                  const float *lse, const void *dout, void *dq, void *dk, void *dv,
                  const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                  int64_t S, int64_t H, int64_t Tq, int64_t Tk,
                  int64_t max_seqlen_q, int64_t max_seqlen_k, int64_t D,
                  float scale, int causal, int dtype, void *workspace,
                  size_t workspace_bytes, void *stream);

/* Static description of a status code; never NULL. */
const char *fa_status_str(int status);

/* Text of the last FA_ERR_HIP raised on the calling thread ("" if none). */
const char *fa_last_hip_error(void);

/* Library version, as major*10000 + minor*100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
