/*
 * fa_varlen.h -- C ABI of the MI355X (gfx950) varlen attention backward.
 *
 * Operation: the backward pass of scaled-dot-product attention over
 * variable-length sequences packed in TND layout, as defined on the CANN
 * ops-transformer page "FlashAttention梯度V2"
 * (aclnnFlashAttentionUnpaddingScoreGradV2), section 计算公式 (formulas):
 *
 *     forward    S = Mask(scale * Q K^T, atten_mask)
 *                P = Dropout(Softmax(S), keepProb),   Y = P V
 *     backward   dV = P^T dY
 *                dQ = scale * dS K
 *                dK = scale * dS^T Q
 *
 * with the softmax Jacobian step dP = dY V^T, dS = Ps o (dP o Z/kp - D),
 * D_i = sum_d dY_i,d Y_i,d, where Ps is the pre-dropout softmax rebuilt from
 * the forward statistics, Ps = exp(S - max) / sum, and Z the keep bits.
 *
 * Argument list and error classes follow the page's 函数原型 (prototypes),
 * 参数说明 (parameter table) and 返回值 (return codes) sections, collapsed
 * into one call: there is no separate workspace query, the library keeps its
 * own workspace (see fa_varlen_bwd) or, in fa_varlen_bwd_noalloc, a fixed one.
 *
 * Ownership: the caller owns every tensor, both cu_seqlens arrays and the
 * stream.  Tensor and statistics pointers are DEVICE pointers; cu_seqlens
 * arrays are HOST arrays, read before the call returns.  dq, dk, dv are fully
 * overwritten (never accumulated): a query row that sees no key gets dq = 0,
 * a key that no query sees gets dk = dv = 0.
 *
 * Errors are detected before any device work is enqueued; on a non-OK
 * status nothing has been launched and fa_last_error() describes the cause.
 * On FA_OK the work is enqueued asynchronously on `stream`.
 *
 * Determinism (the page's constraints section makes a deterministic mode
 * opt-in): every entry point here is deterministic.  No kernel uses atomics,
 * each output row has one owner and a fixed summation order, so repeated
 * calls on the same inputs give bitwise identical results.
 */
#ifndef FA_VARLEN_H
#define FA_VARLEN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of the page's tensor table (FLOAT32, FLOAT16, BFLOAT16). */
typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype_t;

/* A TND tensor view: element [t, n, d] lives at
 * data + (t * stride_t + n * stride_h + d) * sizeof(element).
 * Strides are in elements; the innermost (d) stride must be 1.  Non-contiguous
 * token and head strides are accepted, as the page's tensor table allows. */
typedef struct {
    void*   data;       /* device pointer */
    int32_t dtype;      /* fa_dtype_t */
    int64_t tokens;     /* T */
    int64_t heads;      /* N */
    int64_t head_dim;   /* D */
    int64_t stride_t;
    int64_t stride_h;
} fa_tensor_t;

/* Sequence boundaries: a HOST array of batch + 1 int64 prefix sums with
 * cu[0] = 0 and cu[batch] = T (the page's actualSeqQLen / actualSeqKvLen). */
typedef struct {
    const int64_t* cu;
    int64_t        batch;
} fa_seqlens_t;

/* An explicit attention mask (the page's attenMaskOptional: parameter table, atten_mask in the
 * formulas section): DEVICE uint8 (or bool) elements, nonzero = the pair takes no part.
 * Element (b, n, i, j) -- sequence b, query head n, sequence-relative query i and key j -- is
 * data[b * stride_b + n * stride_n + i * stride_q + j].  The page's shapes map to
 *   [B, N, Sq, Skv]  stride_b = N*Sq*Skv, stride_n = Sq*Skv, stride_q = Skv
 *   [B, 1, Sq, Skv]  stride_n = 0;   [1, 1, Sq, Skv] and [Sq, Skv]: stride_b = stride_n = 0.
 * rows >= every Lq_b and cols >= every Lkv_b (Sq, Skv); stride_q >= cols; strides >= 0.  Only
 * elements with i < Lq_b and j < Lkv_b are read.  A pair is admitted when the window of
 * atten_mode admits it and its mask element is 0 (with FA_MASK_NONE the mask alone decides). */
typedef struct {
    const uint8_t* data;
    int64_t        stride_b;
    int64_t        stride_n;
    int64_t        stride_q;
    int64_t        rows;
    int64_t        cols;
} fa_mask_t;

/* Status codes.  FA_ERR_NULLPTR and FA_ERR_INVALID mirror the page's
 * ACLNN_ERR_PARAM_NULLPTR (161001) and ACLNN_ERR_PARAM_INVALID (161002). */
enum {
    FA_OK = 0,
    FA_ERR_NULLPTR = 1,      /* a required pointer is null */
    FA_ERR_INVALID = 2,      /* a value outside the page's constraints */
    FA_ERR_UNSUPPORTED = 3,  /* allowed by the page, not built here */
    FA_ERR_RUNTIME = 4       /* a HIP runtime failure */
};

/* Mask modes.  The page's atten_mask marks excluded positions with 1; here the
 * excluded set is generated from the mode.  With off_b = Lkv_b - Lq_b:
 *   FA_MASK_NONE    every key of the sequence is admitted;
 *   FA_MASK_CAUSAL  key j is admitted for query i iff j <= i + off_b
 *                   (lower-triangular, aligned to the bottom-right corner);
 *   FA_MASK_BAND    iff i + off_b - pre_tokens <= j <= i + off_b + next_tokens
 *                   (the preTokens/nextTokens sliding window). */
enum { FA_MASK_NONE = 0, FA_MASK_CAUSAL = 1, FA_MASK_BAND = 2 };

/*
 * fa_varlen_bwd -- dQ, dK, dV of varlen attention.
 *
 * q                 [Tq, N, Dk] input.
 * dy, y             [Tq, N, Dv] inputs (y is the forward output attentionIn).
 * k, v              [Tkv, Nkv, Dk] and [Tkv, Nkv, Dv] inputs.  Nkv divides N
 *                   (grouped heads, constraints section of the page): query
 *                   head n reads key/value head n / (N / Nkv), and dk, dv of
 *                   a shared head hold the sum over the query heads that read
 *                   it.  Dv <= Dk (parameter table: V's head dim may be the
 *                   smaller one).
 * softmax_max/sum   [N, Tq, 8] contiguous fp32 device arrays: the forward's
 *                   row max and row sum of exp, replicated over the last
 *                   axis (element 0 is read).  Rows with no admitted key are
 *                   never read.
 * cu_seqlens_q/kv   HOST prefix sums, equal batch counts (1..2048).
 * atten_mode        FA_MASK_*; pre_tokens/next_tokens are read only in
 *                   FA_MASK_BAND.
 * keep_prob         in (0, 1].  Below 1, drop_mask must be given.
 * drop_mask         DEVICE uint8 bit stream, least significant bit first:
 *                   for each sequence b in order, a row-major
 *                   [N, Lq_b, Lkv_b] block of keep bits with no padding
 *                   (bit 1 keeps; kept values are scaled by 1/keep_prob).
 *                   Not read when keep_prob == 1 (may be NULL).
 * scale             the page's scaleValue (replaces 1/sqrt(d)).
 * head_num          N; must equal q->heads.
 * dq, dk, dv        outputs, same dtype and shapes as q, k, v.
 * stream            hipStream_t (NULL = the null stream).
 *
 * Supported: all tensors one dtype (FA_F32, FA_F16 or FA_BF16); head dims
 * (Dk, Dv) in {(128, 128), (128, 64), (64, 64)}.  Other head dims the page
 * allows return FA_ERR_UNSUPPORTED.
 * Tq == 0 returns FA_OK with nothing launched.
 *
 * Library memory: the work lists (which tiles each workgroup visits) are built on the host once
 * per sequence layout (cu_seqlens, mask mode and window, heads, dtype path), uploaded with an
 * asynchronous copy on `stream` from pinned staging memory, and never modified afterwards; the
 * host does not wait for the device, also when the layout changes.  Up to 64 layouts stay cached
 * per device; an evicted list's memory is reused only after its last uses have completed.  The
 * row statistics (8 bytes per query token and head) live in a buffer per stream, so calls on
 * different streams may overlap.  A stream's buffer grows when a call needs more (the host then
 * waits for that stream once).  fa_release() frees everything.
 *
 * Graph capture: a call made while `stream` is being captured allocates and uploads nothing.  It
 * needs a cached list for its layout and a large enough row-statistics buffer on that stream,
 * i.e. one earlier uncaptured call with the same layout and at least as many tokens on the same
 * stream; otherwise it returns FA_ERR_UNSUPPORTED.  The list and the buffer it records are then
 * kept for the graph until fa_release(): later calls, with any layout, never modify or reuse
 * them, so the graph can be replayed at any time.  Replays of one graph must not overlap each
 * other (they share that buffer).
 */
int fa_varlen_bwd(const fa_tensor_t* q, const fa_tensor_t* k, const fa_tensor_t* v,
                  const fa_tensor_t* dy, const fa_tensor_t* y,
                  const float* softmax_max, const float* softmax_sum,
                  const fa_seqlens_t* cu_seqlens_q, const fa_seqlens_t* cu_seqlens_kv,
                  int32_t atten_mode, int64_t pre_tokens, int64_t next_tokens,
                  double keep_prob, const uint8_t* drop_mask,
                  double scale, int64_t head_num,
                  const fa_tensor_t* dq, const fa_tensor_t* dk, const fa_tensor_t* dv,
                  void* stream);

/*
 * fa_varlen_bwd_masked -- fa_varlen_bwd with an explicit attention mask (the page's
 * attenMaskOptional, parameter table): every argument as for fa_varlen_bwd, plus atten_mask
 * (a fa_mask_t, see above; NULL = none, which is exactly fa_varlen_bwd).
 * Additional status codes: FA_ERR_NULLPTR when atten_mask->data is NULL; FA_ERR_INVALID when
 * rows / cols do not cover every sequence, a stride is negative or stride_q < cols;
 * FA_ERR_UNSUPPORTED when one (sequence, head) block spans 2^31 bytes or more.
 */
int fa_varlen_bwd_masked(const fa_tensor_t* q, const fa_tensor_t* k, const fa_tensor_t* v,
                         const fa_tensor_t* dy, const fa_tensor_t* y,
                         const float* softmax_max, const float* softmax_sum,
                         const fa_seqlens_t* cu_seqlens_q, const fa_seqlens_t* cu_seqlens_kv,
                         int32_t atten_mode, int64_t pre_tokens, int64_t next_tokens,
                         double keep_prob, const uint8_t* drop_mask, const fa_mask_t* atten_mask,
                         double scale, int64_t head_num,
                         const fa_tensor_t* dq, const fa_tensor_t* dk, const fa_tensor_t* dv,
                         void* stream);

/*
 * fa_varlen_bwd_noalloc -- fa_varlen_bwd for callers that cannot allocate device memory (code
 * that must not call hipMalloc: tight serving loops, harnesses that forbid allocation, stream
 * capture).  Arguments, results, kernels and status codes are those of fa_varlen_bwd.
 *
 * Instead of library allocations it uses one fixed device array per GPU (50 MiB, held from
 * the first call until the process ends): 48 MiB for the row statistics, i.e. at most
 * 6,291,456 query token-heads (Tq * N), and 2 MiB for the work lists.  Larger inputs return
 * FA_ERR_UNSUPPORTED before any device work.  It calls no allocating routine.
 *
 * Every call on a GPU shares that array: calls that overlap in time on one GPU (on different
 * streams, or with fa_varlen_bwd_noalloc calls from other threads) race and give wrong
 * results.  When the sequence layout differs from the previous call's on that GPU, the new work
 * list is copied into the array and the host waits for `stream` to finish; a call with the same
 * layout only enqueues kernels (it can then also be recorded into a HIP graph; a layout change
 * while `stream` is being captured returns FA_ERR_UNSUPPORTED).
 */
int fa_varlen_bwd_noalloc(const fa_tensor_t* q, const fa_tensor_t* k, const fa_tensor_t* v,
                          const fa_tensor_t* dy, const fa_tensor_t* y,
                          const float* softmax_max, const float* softmax_sum,
                          const fa_seqlens_t* cu_seqlens_q, const fa_seqlens_t* cu_seqlens_kv,
                          int32_t atten_mode, int64_t pre_tokens, int64_t next_tokens,
                          double keep_prob, const uint8_t* drop_mask,
                          double scale, int64_t head_num,
                          const fa_tensor_t* dq, const fa_tensor_t* dk, const fa_tensor_t* dv,
                          void* stream);

/* Thread-local description of the last non-OK status (empty string if none). */
const char* fa_last_error(void);

/* Frees the library's cached work lists, staging memory and row-statistics
 * buffers, including those kept for captured graphs (synchronises every device
 * first; graphs that recorded calls must not be replayed afterwards).  The next
 * call re-allocates what it needs.  The fixed array of fa_varlen_bwd_noalloc is
 * not affected. */
void fa_release(void);

/* One work item: a block of rows of one sequence that a workgroup keeps
 * resident (keys, or queries), and the range of tiles of the other side that
 * hold at least one admitted (query, key) pair with it. */
typedef struct {
    int32_t q_start;     /* first token of the sequence in q/dy/y/dq */
    int32_t kv_start;    /* first token of the sequence in k/v/dk/dv */
    int32_t len_q;       /* Lq_b */
    int32_t len_kv;      /* Lkv_b */
    int32_t block;       /* resident block index: rows [block*block_rows, +block_rows) */
    int32_t tile_begin;  /* first walked tile (rows tile*tile_rows ...) with an admitted pair */
    int32_t tile_end;    /* one past the last; == tile_begin: the block sees nothing */
    int32_t seq;         /* sequence index b */
    int64_t drop_base;   /* bit index of element (0, 0) of head 0 of this sequence */
} fa_work_item_t;

/* Item kinds of fa_varlen_worklist. */
enum {
    FA_ITEMS_KEY_BLOCKS = 0,   /* resident key blocks walking query tiles (dK, dV) */
    FA_ITEMS_QUERY_BLOCKS = 1  /* resident query blocks walking key tiles (dQ) */
};

/*
 * fa_varlen_worklist -- a host-side work list the backward launches over
 * (exposed for inspection and testing; no device work).
 *
 * kind FA_ITEMS_KEY_BLOCKS: one item per block of block_rows keys of every
 * sequence with Lkv_b > 0; its tile range covers exactly the query tiles of
 * tile_rows rows that hold an admitted pair with a key of the block.
 * kind FA_ITEMS_QUERY_BLOCKS: one item per block of block_rows queries of
 * every sequence with Lq_b > 0; its range covers exactly the key tiles of
 * tile_rows rows that hold a key admitted by some query of the block.
 * Blocks with an empty range are kept so their outputs are written as zeros.
 * Items are ordered sequence by sequence (sequences whose longest range is
 * longest first, ties by sequence index), and longest range first within a
 * sequence.
 *
 * items: HOST array of capacity entries, may be NULL to only count.
 * Returns the number of items (>= 0), or -FA_ERR_* on invalid input.
 */
int64_t fa_varlen_worklist(const fa_seqlens_t* cu_seqlens_q, const fa_seqlens_t* cu_seqlens_kv,
                           int32_t atten_mode, int64_t pre_tokens, int64_t next_tokens,
                           int64_t heads, int32_t kind, int32_t block_rows, int32_t tile_rows,
                           fa_work_item_t* items, int64_t capacity);

/*
 * Kernel timing (instrumentation for benchmarks).  While enabled, every
 * fa_varlen_bwd / fa_varlen_fwd call records a pair of HIP events around each
 * of its kernels on the call's stream: index 0 the separate row pass (fp32 inputs
 * only; for bf16 / fp16 the dQ kernel does it), 1 the dK/dV kernel, 2 (unused),
 * 3 the dQ kernel, 4 the forward.
 */
void fa_profile_enable(int on);

/* Waits for the recorded events, writes the summed milliseconds and launch
 * counts per kernel index into ms[] / launches[] (capacity entries each, may be
 * NULL) and clears the record.  Returns the number of kernel indices (5), or
 * -FA_ERR_RUNTIME if an event could not be read. */
int fa_profile_read(double* ms, int64_t* launches, int capacity);

/*
 * Varlen forward: the operator whose outputs the backward consumes ("FlashAttention梯度V2"
 * page, 功能说明 and 计算公式 sections: the forward definition the gradient formulas refer to).
 *   S = scale * Q K^T with the mask of atten_mode / pre_tokens / next_tokens (as in
 *   fa_varlen_bwd), P = softmax of S over the admitted keys of each row, Y = (P o Z / keep_prob) V.
 * Arguments q, k, v, cu_seqlens_*, atten_mode, pre_tokens, next_tokens, keep_prob, drop_mask,
 * scale, head_num and stream mean what they mean for fa_varlen_bwd.  Outputs (caller-owned
 * device memory): y, a TND view with q's tokens and heads and v's head_dim, in q's dtype;
 * softmax_max and softmax_sum, [N, Tq, 8] fp32 (16-byte aligned), each row holding the row's
 * max of the admitted scaled scores and its sum of exp(S - max), repeated 8 times.  A row with
 * no admitted key gets max -inf, sum 0 and a zero Y row.  The statistics are those of the
 * softmax before dropout, which is what fa_varlen_bwd expects.
 * Returns the status codes of fa_varlen_bwd.  Asynchronous on stream; its work lists follow
 * the rules of fa_varlen_bwd (it has no row statistics).
 */
int fa_varlen_fwd(const fa_tensor_t* q, const fa_tensor_t* k, const fa_tensor_t* v,
                  const fa_seqlens_t* cu_seqlens_q, const fa_seqlens_t* cu_seqlens_kv,
                  int32_t atten_mode, int64_t pre_tokens, int64_t next_tokens, double keep_prob,
                  const uint8_t* drop_mask, double scale, int64_t head_num, const fa_tensor_t* y,
                  float* softmax_max, float* softmax_sum, void* stream);

/* fa_varlen_fwd with an explicit attention mask (NULL = none): the forward counterpart of
 * fa_varlen_bwd_masked, with the same mask rules and status codes.  A row whose keys are all
 * excluded gets max -inf, sum 0 and a zero Y row. */
int fa_varlen_fwd_masked(const fa_tensor_t* q, const fa_tensor_t* k, const fa_tensor_t* v,
                         const fa_seqlens_t* cu_seqlens_q, const fa_seqlens_t* cu_seqlens_kv,
                         int32_t atten_mode, int64_t pre_tokens, int64_t next_tokens, double keep_prob,
                         const uint8_t* drop_mask, const fa_mask_t* atten_mask, double scale,
                         int64_t head_num, const fa_tensor_t* y, float* softmax_max, float* softmax_sum,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_VARLEN_H */
