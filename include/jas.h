/*
 * jas.h -- fixed-order, batch-invariant row softmax for AMD Instinct MI355X
 * (gfx950): forward, backward, optional per-head sink, and a fused attention
 * forward built on the same softmax.
 *
 * What the library computes (the pages it follows):
 *   - RL-Kernel PR #453, "[WS1][kernels] Add fixed-order joint-attention
 *     softmax for Qwen-Image", Summary: the softmax that sits between the
 *     QK GEMM and the AV GEMM of joint attention, taken along the key
 *     dimension of each row of scores; each row is split into fixed
 *     256-key tiles processed left to right, each tile reduces its max and
 *     its sum of exponentials with one fixed tree, the per-tile states are
 *     merged in tile order, all intermediates are FP32 and the only rounding
 *     to the tensor dtype happens at the write.  Backward: delta is the same
 *     fixed-order sum of P*dP, then dScores = P*(dP - delta).
 *   - ROCm TransformerEngine PR #678, "Add softmax sink (learnable
 *     off-by-one) support for the ROCm/CK fused attention backend", title and
 *     Description: an optional learnable logit per head adds one term to the
 *     softmax denominator; backward produces its gradient d_sink per head.
 *     The sink buffer holds one value per head and is indexed by head only.
 *   - RL-Kernel PR #240, "Batch-invariant attention (standard softmax --
 *     cuda version)", Fixed Reduction Contract and Path Status: the reduction
 *     tree's shape depends on nothing but the tile (not on batch size, row
 *     position, launch geometry or grid), fully masked rows are handled, the
 *     row's log-sum-exp is a second output, and FP16 is a dtype beside
 *     BF16.
 *
 * Exact arithmetic of one row of N keys, T = ceil(N/256) tiles (every
 * operation binary32, round to nearest-even, no fused multiply-add):
 *   kend  = the row's visible key prefix: N, cut by JAS_FLAG_CAUSAL to
 *           q + (N - q_rows) + 1 (a key is visible to query q when
 *           key <= keys - q_rows + q; RL-Kernel PR #240, Prefill / Decode)
 *           and by JAS_FLAG_KEY_LEN to key_len[b], clamped to [0, N]
 *   x_j   = float(s_j) (+ mask_j, one rounding, when JAS_FLAG_MASK) for
 *           j < kend; -inf for j >= kend (those scores are never read)
 *   m_t   = max over tile t (positions past N count as -inf)
 *   e_j   = exp_(x_j - m_t), exp_(y) = 2^fl(y*log2e), 0 when that exponent
 *           is below -126 (or y is -inf); 0 in a tile whose max is -inf
 *   l_t   = balanced pairwise tree sum of the tile's 256 e values in key
 *           order (positions past N count as 0)
 *   (M,L) = (-inf,0) merged with (m_t,l_t) for t = 0..T-1 in order, then
 *           with (sigma_h, 1) when JAS_FLAG_SINK; merging (m,l) into (M,L):
 *           Mn = max(M,m), L = fl(L*exp_(M-Mn)) + fl(l*exp_(m-Mn)), a -inf
 *           side contributes 0, and an all -inf state stays (-inf, 0)
 *   invL  = 1/L (0 when L is 0)
 *   P_j   = round_to_dtype(e_j * fl(exp_(m_t - M) * invL))
 *   p_sink= fl(exp_(sigma_h - M) * invL)      (0 when sigma_h is -inf)
 *   lse   = fl(M + fl(log2_(L) * ln2)) with the hardware base-2 logarithm
 *           and ln2 the binary32 nearest to ln 2; -inf when L is 0.  Within
 *           4e-6 * max(1, |lse|) of M + ln(L) rounded once.
 * Backward on the stored P (P_j taken as +0 without being read for
 * j >= kend):
 *   d_t   = balanced tree sum of fl(P_j*dP_j) over tile t; delta = d_0, then
 *           delta = fl(delta + d_t) for t = 1..T-1
 *   dS_j  = round_to_dtype(P_j * fl(dP_j - delta))
 *   d_sink[h] = the rows of head h in (batch, query) order, in chunks of 256
 *           rows (the last padded with +0), each chunk summed with the same
 *           balanced tree over -fl(p_sink_r*delta_r), chunk sums added left
 *           to right from the first; d_sink is overwritten, never accumulated.
 * round_to_dtype is round to nearest-even into bf16 or binary16 (subnormals
 * kept, overflow to infinity), the identity for binary32.  The exponential
 * is the hardware base-2 exponential; everything else is exact IEEE
 * arithmetic, so results do not depend on batch size, a row's
 * position, launch geometry or grid size.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are device pointers owned by the caller.  The library
 *     never allocates, frees or synchronizes; all work is enqueued on
 *     `stream` (a void * holding a hipStream_t, so this header needs no HIP
 *     include; NULL is the null stream) and the call returns
 *     without waiting for it.
 *   - Validation is done entirely on the host before any HIP call; on any
 *     error nothing is enqueued and the status says why.  JAS_ERR_HIP means
 *     the HIP runtime refused a launch (hipGetLastError is read after each
 *     launch); for jas_bwd with a sink the row kernel may then already be
 *     enqueued while the d_sink reduction is not.
 *   - Rows: rows = batch*heads*q_rows, row r = (b*heads + h)*q_rows + q,
 *     row r starts at element r*ld of scores / probs / dprobs / dscores.
 *   - An empty call (rows == 0) reads nothing; its row tensors (scores,
 *     probs, dprobs, dscores, mask, sink, p_sink, lse, workspace) may be
 *     NULL.
 *     jas_bwd with JAS_FLAG_SINK still writes d_sink[h] = +0 for every head.
 *   - Element pointers must be aligned to their element size; any further
 *     alignment only selects the faster 16-byte load path (same results).
 *   - The library is stateless: concurrent calls on different streams are
 *     fine.
 */
#ifndef JAS_H_
#define JAS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest supported row length (keys per row).  Rows of up to 16,384 keys
 * are held in registers for one pass over HBM; longer rows are streamed
 * (RL-Kernel PR #453, Summary: rows are processed tile by tile, left to
 * right): the tile states of the whole row are kept on chip, the last
 * segment stays in registers and the one before it in LDS, and the other
 * segments are read a second time to write the outputs, with the same
 * arithmetic and so the same bits. */
#define JAS_MAX_KEYS 262144

/* Element type of scores, probs, dprobs and dscores.  mask, sink, p_sink,
   lse, d_sink and the workspace are always binary32. */
typedef enum { JAS_DTYPE_F32 = 0, JAS_DTYPE_BF16 = 1, JAS_DTYPE_F16 = 2 } jas_dtype_t;

/* Flags: the only predicates for "has a mask", "has a sink", "causal",
 * "has per-batch key lengths" and "writes the row log-sum-exp".  CAUSAL and
 * KEY_LEN exclude a suffix of each row: excluded keys behave exactly as keys
 * whose score is -inf, and whole 256-key tiles past the visible prefix are
 * not read (forward: scores; backward: P, which the forward wrote as +0
 * there).  LSE applies to the forward only (the backward ignores it). */
enum {
  JAS_FLAG_MASK = 1u << 0,
  JAS_FLAG_SINK = 1u << 1,
  JAS_FLAG_CAUSAL = 1u << 2,
  JAS_FLAG_KEY_LEN = 1u << 3,
  JAS_FLAG_LSE = 1u << 4
};

typedef enum {
  JAS_OK = 0,
  JAS_ERR_NULL_POINTER = 1, /* desc, a tensor, or the operand of a set flag is NULL */
  JAS_ERR_BAD_SHAPE = 2,    /* negative dim, keys < 1, ld < keys, negative mask stride, size overflow */
  JAS_ERR_BAD_DTYPE = 3,    /* dtype is not a jas_dtype_t */
  JAS_ERR_BAD_FLAGS = 4,    /* unknown flag bit, or a pointer given for a flag that is not set */
  JAS_ERR_ALIASING = 5,     /* an output overlaps another buffer (beyond the allowed in-place pairs) */
  JAS_ERR_WORKSPACE = 6,    /* workspace NULL or smaller than jas_bwd_workspace_bytes */
  JAS_ERR_UNSUPPORTED = 7,  /* keys > JAS_MAX_KEYS, or a launch override that cannot hold the row */
  JAS_ERR_HIP = 8,          /* the HIP runtime refused a launch */
  JAS_ERR_ALIGNMENT = 9,    /* a pointer is not aligned to its element size */
  JAS_ERR_SCRATCH = 10      /* jas_bwd_noalloc with a sink: rows > JAS_NOALLOC_MAX_ROWS */
} jas_status_t;

/* Problem description, shared by forward and backward. */
typedef struct {
  int64_t batch, heads, q_rows, keys; /* >= 0, keys >= 1; a zero batch/heads/q_rows is an empty call */
  int64_t ld;                         /* elements between consecutive rows, ld >= keys */
  int32_t dtype;                      /* jas_dtype_t */
  uint32_t flags;                     /* JAS_FLAG_* */
  int64_t mask_stride_b;              /* mask element (b,h,q,k) is at     */
  int64_t mask_stride_h;              /*   mask[b*msb + h*msh + q*msq + k] */
  int64_t mask_stride_q;              /* strides >= 0; 0 broadcasts        */
} jas_desc_t;

/* Launch geometry override (for invariance tests and tuning).  Every valid
 * geometry gives bit-identical results.  Zero fields take the library
 * default.  waves_per_row in {1,2,4}: wavefronts sharing one row;
 * chunks_per_lane: 16-byte chunks of the row each lane keeps in registers
 * (one of the compiled sizes; waves_per_row*chunks_per_lane chunks of 64
 * lanes must cover the row); rows_per_block: rows per workgroup, with
 * waves_per_row*rows_per_block <= 4; max_blocks: grid size cap (the
 * workgroups then loop over the rows).  streaming = 1 runs the streaming
 * kernels for rows of any length (they always run for rows over 16,384
 * keys): 4 waves and 1 row per workgroup, chunks_per_lane per segment in
 * {4, 8} for 16-bit types, {8, 16} for fp32.  mask_in_registers (forward
 * only): 1 keeps each wave's share of the mask row in registers from one of
 * its workgroup's rows to the next, reloading it only when the row's mask
 * row (or visible length) changes; it needs a 16-bit dtype, a mask,
 * waves_per_row 2 (taken when waves_per_row is 0) and chunks_per_lane at
 * most 5 (rows that are not whole aligned 16-byte chunks then run the
 * element-wise forward on the same grid), and defaults to rows_per_block 1
 * and half as many workgroups as rows.  2 turns it off.  0 takes the
 * default: on when no other field is set, the mask is broadcast over
 * queries (mask_stride_q 0), there is no causal flag, the rows are whole
 * 16-byte chunks, the default geometry qualifies and there are at least
 * 16,384 rows.  In the plan jas_launch_plan returns it reads 1 when used
 * and 0 otherwise. */
typedef struct {
  int32_t waves_per_row;
  int32_t chunks_per_lane;
  int32_t rows_per_block;
  int32_t max_blocks;
  int32_t streaming;
  int32_t mask_in_registers;
} jas_launch_t;

/* Forward.
 *   scores [rows, ld] (dtype)  read.   probs [rows, ld] (dtype) written,
 *   keys columns per row; probs == scores (in place) is allowed, any other
 *   overlap of probs with an input is JAS_ERR_ALIASING.
 *   mask   binary32, required iff JAS_FLAG_MASK (see jas_desc_t strides).
 *   key_len int32 [batch] device array, required iff JAS_FLAG_KEY_LEN:
 *          keys at or past key_len[b] are excluded (values are clamped to
 *          [0, keys] in the kernels).
 *   sink   binary32 [heads], required iff JAS_FLAG_SINK.
 *   p_sink binary32 [rows] written, required iff JAS_FLAG_SINK; the sink's
 *          own probability, which jas_bwd reads.
 *   lse    binary32 [rows] written, required iff JAS_FLAG_LSE: the row's
 *          log-sum-exp (the sink's term included), -inf for a row with
 *          nothing to sum.
 * (Definition: RL-Kernel PR #453, Summary, fixed-order online softmax;
 *  sink: TransformerEngine PR #678, Description; lse: RL-Kernel PR #240,
 *  Fixed Reduction Contract, Softmax and LSE.) */
jas_status_t jas_fwd(const jas_desc_t *desc, const void *scores, const float *mask,
                     const int32_t *key_len, const float *sink, void *probs, float *p_sink,
                     float *lse, void *stream);

/* jas_fwd with an explicit launch geometry (NULL = default). */
jas_status_t jas_fwd_ex(const jas_desc_t *desc, const void *scores, const float *mask,
                        const int32_t *key_len, const float *sink, void *probs, float *p_sink,
                        float *lse, const jas_launch_t *launch, void *stream);

/* Bytes of device workspace jas_bwd needs: 4*rows rounded up to 256 when
 * JAS_FLAG_SINK is set, else 0.  The workspace holds each row's share
 * -fl(p_sink*delta) of d_sink, which the d_sink kernel then reduces per head
 * in a fixed order without atomics.  Depends on the shape and flags only,
 * never on pointers, so a sizing call and the jas_bwd call that uses the
 * workspace always agree on whether there is a sink (ROCm TransformerEngine
 * PR #678, review of the backward's workspace-size query: the sizing pass
 * and the execution pass must take the has-sink decision from the same
 * predicate, never from whether the sink pointer is NULL, or the workspace
 * is under-allocated).  Returns 0 for a NULL or invalid desc. */
size_t jas_bwd_workspace_bytes(const jas_desc_t *desc);

/* Backward on the stored probabilities.
 *   probs, dprobs [rows, ld] (dtype) read.  dscores [rows, ld] written;
 *   JAS_FLAG_LSE is ignored here;
 *   dscores may equal probs or dprobs (in place), any other overlap is
 *   JAS_ERR_ALIASING.  JAS_FLAG_MASK and the mask strides are ignored:
 *   masked keys already have P = 0.  With JAS_FLAG_CAUSAL / JAS_FLAG_KEY_LEN
 *   (key_len as for the forward) P is not read on excluded keys and taken
 *   as +0; dprobs is read on every key, so dS keeps its signed zeros.
 *   p_sink  binary32 [rows] read, required iff JAS_FLAG_SINK.
 *   d_sink  binary32 [heads] written (overwritten, not accumulated),
 *           required iff JAS_FLAG_SINK.
 *   workspace, workspace_bytes: device scratch of at least
 *           jas_bwd_workspace_bytes(desc) bytes (binary32 aligned), used
 *           only with a sink; its contents on entry do not matter.
 * (Definition: RL-Kernel PR #453, Summary, fixed-order backward; d_sink:
 *  TransformerEngine PR #678, reduced here in a fixed order without
 *  atomics.) */
jas_status_t jas_bwd(const jas_desc_t *desc, const void *probs, const void *dprobs,
                     const int32_t *key_len, const float *p_sink, void *dscores, float *d_sink,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Rows jas_bwd_noalloc takes with a sink: its per-row d_sink shares live in
 * a static device array of this many floats (4 MiB per GPU). */
#define JAS_NOALLOC_MAX_ROWS 1048576

/* jas_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments without the workspace, the same kernels and the same
 * bits.  With JAS_FLAG_SINK the per-row d_sink shares go to a static device
 * array of the library (JAS_NOALLOC_MAX_ROWS floats, one copy on each GPU
 * the library runs on, held until the process ends); a call with more rows
 * returns JAS_ERR_SCRATCH and enqueues nothing.  The call itself calls no
 * allocating routine.  The array's device address is looked up on the first
 * call on each device (the device of `stream`).  All calls on one GPU share
 * the array and every call rewrites the part it uses before reading it, so
 * its contents on entry never matter; calls that overlap on one GPU (on
 * concurrent streams) race and must be ordered by the caller.  Without a
 * sink it is jas_bwd without a workspace. */
jas_status_t jas_bwd_noalloc(const jas_desc_t *desc, const void *probs, const void *dprobs,
                             const int32_t *key_len, const float *p_sink, void *dscores,
                             float *d_sink, void *stream);

/* jas_bwd with an explicit launch geometry (NULL = default). */
jas_status_t jas_bwd_ex(const jas_desc_t *desc, const void *probs, const void *dprobs,
                        const int32_t *key_len, const float *p_sink, void *dscores,
                        float *d_sink, void *workspace, size_t workspace_bytes,
                        const jas_launch_t *launch, void *stream);

/* The row-kernel geometry jas_fwd_ex (backward = 0) or jas_bwd_ex
 * (backward = 1) would launch for this descriptor and override (NULL =
 * default): waves_per_row, chunks_per_lane, rows_per_block, max_blocks = the
 * grid size, streaming = 1 for the streaming kernels.  Host only: reads no
 * device memory and enqueues nothing.  Returns the status those calls give
 * for the shape and override (before any pointer check); *plan is all zeros
 * on an error and for zero rows (no row kernel runs).  JAS_ERR_NULL_POINTER
 * for a NULL plan, JAS_ERR_BAD_FLAGS for backward outside {0, 1}.  Every
 * geometry gives the same bits (RL-Kernel PR #453, Summary: batch-invariant
 * order). */
jas_status_t jas_launch_plan(const jas_desc_t *desc, int backward, const jas_launch_t *launch,
                             jas_launch_t *plan);

/* ------------------------------------------------------------------------
 * Fused attention forward: scores = scale * Q K^T on the matrix cores, the
 * row softmax above on those binary32 scores (bit for bit what jas_fwd
 * computes from them), P rounded once to the tensor dtype, out = P V.
 * (RL-Kernel PR #453, Summary: the softmax sits between the QK GEMM and the
 * AV GEMM; RL-Kernel PR #240, Fixed Reduction Contract: one writer per
 * score and per output element, a fixed accumulation order, no split of the
 * key range; its Path Status: MHA, MQA and GQA head layouts, causal and
 * padding masks.)
 *
 * Arithmetic: dot_j is the head-dimension sum of q_d*k_jd accumulated by
 * v_mfma_f32_16x16x32 (bf16 / fp16 inputs, exact products, binary32
 * accumulation in the instruction's fixed internal order, 32 dims per step
 * in ascending steps); s_j = fl(scale * dot_j); the softmax of jas_fwd on
 * s (mask, causal, key lengths, sink, lse exactly as there); P_j rounded to
 * the dtype; out_d = the key sum of P_j*v_jd accumulated the same way, 32
 * keys per step in ascending steps, rounded once to the dtype.  The scores
 * differ from a sequential binary32 dot product only in summation order.
 * ------------------------------------------------------------------------ */

/* Longest key range of the fused attention (keys per row). */
#define JAS_ATTN_MAX_KEYS 16384

/* Extra flags of jas_attn_fwd: also write P (dtype) / the scores (binary32),
 * [batch, heads, q_len, kv_len] each.  Meant for checking and for a backward
 * that needs P; they cost a full write of the matrix. */
enum { JAS_FLAG_PROBS = 1u << 5, JAS_FLAG_SCORES = 1u << 6 };

typedef struct {
  int64_t batch, heads, kv_heads;  /* heads a multiple of kv_heads; query head h reads
                                      key/value head h / (heads / kv_heads) */
  int64_t q_len, kv_len;           /* queries and keys per (batch, head); kv_len >= 1 */
  int64_t head_dim;                /* 64 or 128 */
  int32_t dtype;                   /* JAS_DTYPE_BF16 or JAS_DTYPE_F16 */
  uint32_t flags;                  /* MASK, SINK, CAUSAL, KEY_LEN, LSE, PROBS, SCORES */
  float scale;                     /* score scale, e.g. 1/sqrt(head_dim) */
  int64_t mask_stride_b, mask_stride_h, mask_stride_q; /* as in jas_desc_t */
} jas_attn_desc_t;

/* Fused attention forward.
 *   q [batch, heads, q_len, head_dim], k and v [batch, kv_heads, kv_len,
 *   head_dim], contiguous, dtype; 16-byte aligned.
 *   out [batch, heads, q_len, head_dim] written (dtype).
 *   mask, key_len, sink: as for jas_fwd (mask element (b, h, q, key)).
 *   lse, p_sink: binary32 [batch*heads*q_len], required iff JAS_FLAG_LSE /
 *   JAS_FLAG_SINK.  probs / scores: required iff JAS_FLAG_PROBS /
 *   JAS_FLAG_SCORES.
 * Outputs must not overlap each other or the inputs.  No workspace: V is
 * read in place (the PV operands come from gfx950's transposed LDS reads).
 */
jas_status_t jas_attn_fwd(const jas_attn_desc_t *desc, const void *q, const void *k,
                          const void *v, const float *mask, const int32_t *key_len,
                          const float *sink, void *out, float *lse, float *p_sink, void *probs,
                          float *scores, void *stream);

/* jas_attn_fwd with an explicit number of 16-query blocks per wavefront,
 * query_blocks: 1, 2, or 0 for the library's choice.  Two blocks share every
 * K and V operand read between two products.  The library runs 1 block,
 * whatever was asked, when the mask varies by query (mask_stride_q != 0) or
 * when two blocks' tile maxima would take the workgroup's LDS past 64 KB
 * (more than 14,336 keys at head_dim 128).  Its own choice (0) is 2
 * without JAS_FLAG_PROBS / JAS_FLAG_SCORES when
 * batch*heads*ceil(q_len/128) >= 512, else 1.  Each query is computed by
 * the same operations in the same order either way, so the outputs are
 * identical for 0, 1 and 2 (RL-Kernel PR #240, Fixed Reduction Contract:
 * results independent of the launch).  JAS_ERR_BAD_FLAGS for any other
 * value; otherwise as jas_attn_fwd. */
jas_status_t jas_attn_fwd_ex(const jas_attn_desc_t *desc, const void *q, const void *k,
                             const void *v, const float *mask, const int32_t *key_len,
                             const float *sink, void *out, float *lse, float *p_sink, void *probs,
                             float *scores, int query_blocks, void *stream);

/* Static text for a status code (never NULL; "unknown status" for a value
 * outside jas_status_t).  Every entry point reports a refused call through
 * its status instead of reaching the GPU with it: a flag whose pointer is
 * NULL is JAS_ERR_NULL_POINTER before any launch (ROCm TransformerEngine
 * PR #678, review of the sink pointer under has_sink: once the flag is set
 * the pointer is a hard requirement, and a NULL one must be a clear error,
 * not a GPU fault or a silent no-op), and the launch status is read after
 * every launch and returned as JAS_ERR_HIP (RL-Kernel PR #240, review of
 * the launch wrappers: a launch without an error check lets a bad launch
 * surface later at an unrelated call). */
const char *jas_status_str(jas_status_t status);

/* Static fingerprint of the arithmetic contract: tile size, tree, merge
 * order, accumulator precision, exponential, rounding, target
 * (RL-Kernel PR #453, Summary: the trace records reduction order,
 * accumulator precision and a kernel fingerprint). */
const char *jas_contract(void);

#ifdef __cplusplus
}
#endif

#endif /* JAS_H_ */
