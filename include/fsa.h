/*
 * fsa.h -- C ABI of libfsa: top-k selected block-sparse flash attention
 * (prefill forward) and top-k gathered paged-KV decode for AMD MI355X
 * (gfx950).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor arguments are DEVICE pointers into memory the caller owns and
 *   keeps alive until the enqueued work has finished.  The library never
 *   allocates, frees or synchronises; it enqueues kernels on `stream`
 *   (a hipStream_t passed as void*, NULL = the default stream) and returns.
 *   FSA_SUCCESS therefore means "validated and enqueued".
 * - bf16 tensors are IEEE bfloat16 bit patterns, row-major, innermost
 *   dimension contiguous, with exactly the shapes given below (no strides).
 * - Argument errors (null pointer, bad size, unsupported shape, workspace too
 *   small) are detected on the host before anything is enqueued and before
 *   any device memory is written.
 * - Index CONTENTS never produce an error or a fault.  Block ids, token
 *   positions and page ids that point outside the valid range are skipped,
 *   and a repeated id counts once (the lists are sets).  A query row that
 *   ends up with no visible key gets O = 0 and LSE = -inf.
 * - softmax_scale <= 0 selects the default 1/sqrt(head_dim).
 * - max_seqlen_q / max_seqlen_k larger than total_q / total_k are read as
 *   total_q / total_k (no sequence is longer than its tensor).  A call whose
 *   kernels would need more than 2^22 workgroups in one launch returns
 *   FSA_ERROR_NOT_SUPPORTED before launching anything (the query-centric
 *   prefill, for instance, launches batch * ceil(max_seqlen_q / T) *
 *   num_heads_kv * splits of them, T >= 1 tokens per workgroup).
 * - Calls are thread-safe.  Process-wide state: per-device records that a
 *   kernel's LDS limit has been raised (an idempotent runtime setting), the
 *   scratch array of fsa_topk_decode_noalloc, and the diagnostics of the
 *   kernels' bounded waits (fsa_set_wait_poll_limit, fsa_wait_timeouts).
 *
 * Semantics follow the pages this library is built from:
 * - GQA: query head h reads kv head h / (num_heads_q / num_heads_kv);
 *   num_heads_q must be a multiple of num_heads_kv (flash-attention-npu page,
 *   flash_attn_func docstring, MQA/GQA paragraph with the 6/2-head example).
 * - Causal masking is aligned to the bottom-right corner: row i of a sequence
 *   with S_q queries and S_k keys sees key j iff j <= i + S_k - S_q; an
 *   all-masked row outputs zeros (same docstring, causal paragraph and its
 *   2x5 / 5x2 examples).
 * - LSE is the natural-log logsumexp of the scaled scores of each row, stored
 *   fp32 with layout (num_heads_q, total_q) for the varlen prefill
 *   (flash_attn_varlen_func docstring, softmax_lse) and (batch, num_heads_q)
 *   for decode.
 * - Selected attention: each (query token, kv head) carries a list of topk
 *   key-block ids (blocks of block_size consecutive keys of its sequence);
 *   its G query heads attend to the keys of those blocks only (FSA page:
 *   NSA selected attention with block_size / topk; the Ascend SFA blog:
 *   gather the selected K/V rows, then ordinary attention, -1 = invalid).
 * - Top-k paged decode: the one query token of each sequence attends to the
 *   cache positions listed for its kv head (a set, like the block lists);
 *   position t of sequence b is row t % page_size of page
 *   block_table[b][t / page_size] of the paged cache, and positions at or
 *   past cache_seqlens[b] are skipped (FSA page, main features: top-k gather
 *   KV-cache decoding and paged attention; flash-attention-npu page,
 *   flash_attn_with_kvcache docstring: k_cache / v_cache
 *   [num_blocks, page_block_size, nheads_k, headdim], block_table,
 *   cache_seqlens).
 */
#ifndef FSA_H_
#define FSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FSA_ABI_VERSION 2

typedef enum {
    FSA_SUCCESS = 0,
    FSA_ERROR_INVALID_VALUE = 1,  /* null pointer, negative or inconsistent size */
    FSA_ERROR_NOT_SUPPORTED = 2,  /* shape outside what the kernels are built for */
    FSA_ERROR_WORKSPACE = 3,      /* workspace missing or smaller than required */
    FSA_ERROR_LAUNCH = 4          /* a kernel launch was rejected by the HIP runtime */
} fsa_status_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* fsa_status_string(fsa_status_t status);

/* FSA_ABI_VERSION of the built library. */
int32_t fsa_abi_version(void);

/*
 * Diagnostics of the bounded waits inside the prefill, window and backward
 * kernels.  Their producer and consumer waves hand K/V blocks over through
 * LDS flags; every wait polls a bounded number of times, so an error in that
 * hand-over can never hang the GPU.  A wave whose wait runs out gives up:
 * it goes on with whatever LDS holds (its results are then wrong; every
 * access stays in bounds), adds one to a counter in device memory of the
 * current device, makes each of its later waits a single poll and tells the
 * other waves of its workgroup, which stop waiting within ~1024 polls.
 *
 * fsa_wait_timeouts: *count = that counter (0 after correct runs); a nonzero
 *   reset clears it.  Synchronous (a device-to-host copy on the null stream);
 *   FSA_ERROR_INVALID_VALUE for a NULL count, FSA_ERROR_LAUNCH if the copy
 *   fails.
 * fsa_set_wait_poll_limit: the number of polls a wait makes before it gives
 *   up, for calls enqueued afterwards by any thread; 0 restores the default
 *   (2^22, about half a second; a wait normally ends within ~1e3 polls).  A
 *   tiny limit makes waits give up on purpose, which exercises this path
 *   without any out-of-bounds access.  FSA_ERROR_INVALID_VALUE if negative.
 */
fsa_status_t fsa_wait_timeouts(uint32_t* count, int32_t reset);
fsa_status_t fsa_set_wait_poll_limit(int32_t polls);

/*
 * Bytes of device workspace fsa_selected_attn_fwd needs for these arguments
 * (0 when no workspace is needed).  num_splits = 0 prices the automatic
 * choice.  Returns 0 as well for arguments fsa_selected_attn_fwd would reject.
 * The block-centric schedule (below) needs about
 * total_q * num_heads_q * topk * (2 * head_dim + 4) bytes of partials plus
 * the inverted index.
 */
size_t fsa_selected_attn_fwd_workspace_size(int32_t batch, int64_t total_q,
                                             int32_t max_seqlen_q, int32_t max_seqlen_k,
                                             int32_t num_heads_q, int32_t num_heads_kv,
                                             int32_t head_dim, int32_t block_size,
                                             int32_t topk, int32_t num_splits);

/*
 * Selected block-sparse attention forward (prefill), varlen layout.
 *
 *   q        bf16 [total_q, num_heads_q, head_dim]
 *   k, v     bf16 [total_k, num_heads_kv, head_dim]
 *   blk_idx  int32 [total_q, num_heads_kv, topk]: key-block ids of the token's
 *            sequence, block b = keys [b*block_size, (b+1)*block_size); any
 *            order; -1 (or any id outside [0, ceil(S_k/block_size))) = unused
 *   cu_seqlens_q, cu_seqlens_k  int32 [batch + 1] prefix sums of the per-
 *            sequence lengths (they may be the same pointer); must be non-
 *            decreasing with cu_seqlens_q[batch] <= total_q and
 *            cu_seqlens_k[batch] <= total_k (rows past those are not touched)
 *   max_seqlen_q  >= every S_q; max_seqlen_k >= every S_k
 *   head_dim 64 or 128; block_size 64; 1 <= topk <= 64;
 *   num_heads_q / num_heads_kv <= 224
 *   causal   nonzero: bottom-right causal mask; zero: no mask
 *   num_splits  selects the schedule.
 *            -1: block-centric (the FSA page's loop swap: the lists are
 *            inverted on the GPU, each key block is computed once against the
 *            dense 16-row tiles of the query rows that selected it, and the
 *            per-(token, block) partials are merged by logsumexp; needs
 *            workspace); num_heads_q / num_heads_kv <= 16, else
 *            FSA_ERROR_NOT_SUPPORTED.
 *            n >= 1: query-centric (a workgroup per tile of query tokens
 *            streams the union of their blocks) with every tile's selected-
 *            block set split into n parts computed by separate workgroups and
 *            merged by logsumexp (needs workspace when n > 1); at most 16.
 *            0: automatic -- block-centric when num_heads_q / num_heads_kv
 *            <= 2, else query-centric with an automatic split count.
 *   workspace, workspace_bytes  device scratch of at least
 *            fsa_selected_attn_fwd_workspace_size(...) bytes (may be NULL when
 *            that size is 0); contents on entry are ignored
 *   out      bf16 [total_q, num_heads_q, head_dim]
 *   lse      fp32 [num_heads_q, total_q], or NULL to skip it
 */
fsa_status_t fsa_selected_attn_fwd(const void* q, const void* k, const void* v,
                                   const int32_t* blk_idx, const int32_t* cu_seqlens_q,
                                   const int32_t* cu_seqlens_k, int32_t batch, int64_t total_q,
                                   int64_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                   int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                   int32_t block_size, int32_t topk, float softmax_scale,
                                   int32_t causal, int32_t num_splits, void* workspace,
                                   size_t workspace_bytes, void* out, float* lse, void* stream);

/*
 * Backward of fsa_selected_attn_fwd (the training use of selected attention
 * on the FSA page): the gradients of sum(dout * out) with respect to q, k and
 * v, for the same lists, causal flag and scale as the forward call.
 *
 *   q, k, v, blk_idx, cu_seqlens_q/k, batch, total_q, total_k, max_seqlen_q,
 *            max_seqlen_k, head counts, head_dim, block_size, topk,
 *            softmax_scale, causal: as in fsa_selected_attn_fwd (head groups
 *            num_heads_q / num_heads_kv <= 32)
 *   out      bf16 [total_q, num_heads_q, head_dim]: the forward's output
 *   lse      fp32 [num_heads_q, total_q]: the forward's LSE
 *   dout     bf16 [total_q, num_heads_q, head_dim]: gradient of the output
 *   workspace at least fsa_selected_attn_bwd_workspace_size(...) bytes,
 *            256-byte aligned
 *   dq       bf16 [total_q, num_heads_q, head_dim]
 *   dk, dv   bf16 [total_k, num_heads_kv, head_dim]; keys no row sees get 0
 * Rows with no visible key get dq = 0.  dk and dv are summed in an order that
 * can change between calls, so they may differ in the last bits run to run.
 */
size_t fsa_selected_attn_bwd_workspace_size(int32_t batch, int64_t total_q, int64_t total_k,
                                            int32_t max_seqlen_q, int32_t max_seqlen_k,
                                            int32_t num_heads_q, int32_t num_heads_kv,
                                            int32_t head_dim, int32_t block_size, int32_t topk);

fsa_status_t fsa_selected_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                                   const float* lse, const void* dout, const int32_t* blk_idx,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                   int32_t batch, int64_t total_q, int64_t total_k,
                                   int32_t max_seqlen_q, int32_t max_seqlen_k,
                                   int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                   int32_t block_size, int32_t topk, float softmax_scale,
                                   int32_t causal, void* workspace, size_t workspace_bytes,
                                   void* dq, void* dk, void* dv, void* stream);

/*
 * Local (sliding-window) attention forward, dense within the window, varlen
 * layout.  Row i of a sequence with S_q queries and S_k keys attends to every
 * key j of its sequence with
 *     i + S_k - S_q - window_left <= j <= i + S_k - S_q + window_right
 * (window_size = (left, right) of the flash_attn_func docstring on the
 * flash-attention-npu page; -1 leaves that side unlimited, so (-1, 0) is
 * causal attention, FlashAttention tutorial page section 4.3, and (-1, -1) is
 * full attention).  The FSA page's sliding-window branch with window w is
 * (w - 1, 0).  A row with no key in its window gets O = 0 and LSE = -inf.
 *
 *   q, k, v, cu_seqlens_q, cu_seqlens_k, batch, total_q, total_k,
 *   max_seqlen_q, max_seqlen_k, head dims and groups, softmax_scale,
 *   num_splits, workspace, out, lse: as in fsa_selected_attn_fwd (no block
 *   lists); window_left, window_right >= -1
 */
size_t fsa_sliding_window_fwd_workspace_size(int32_t batch, int64_t total_q,
                                             int32_t max_seqlen_q, int32_t num_heads_q,
                                             int32_t num_heads_kv, int32_t head_dim,
                                             int32_t num_splits);

fsa_status_t fsa_sliding_window_fwd(const void* q, const void* k, const void* v,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                    int32_t batch, int64_t total_q, int64_t total_k,
                                    int32_t max_seqlen_q, int32_t max_seqlen_k,
                                    int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                    int32_t window_left, int32_t window_right,
                                    float softmax_scale, int32_t num_splits, void* workspace,
                                    size_t workspace_bytes, void* out, float* lse, void* stream);

/*
 * Bytes of device workspace fsa_topk_decode needs: the split partials, so 0
 * when the lists are not split (num_splits = 1, or an automatic choice of 1).
 * num_splits = 0 prices the automatic choice.  Returns 0 as well for
 * arguments fsa_topk_decode rejects.
 */
size_t fsa_topk_decode_workspace_size(int32_t batch, int32_t num_heads_q, int32_t num_heads_kv,
                                      int32_t head_dim, int32_t topk, int32_t num_splits);

/* The split count fsa_topk_decode uses for num_splits = 0 (0 for arguments
 * it rejects). */
int32_t fsa_topk_decode_auto_splits(int32_t batch, int32_t num_heads_q, int32_t num_heads_kv,
                                    int32_t topk);

/*
 * Top-k gathered decode over a paged KV cache: one query token per sequence
 * attends to the cache positions listed for its kv head.
 *
 * Defining passages: the flash-sparse-attn page's feature list (main
 * features: top-k gather KV-cache decoding, paged attention, split-KV for
 * decode load balance) and its decode example (a [batch, heads, head_dim]
 * query against the cache); the flash-attention-npu page's
 * flash_attn_with_kvcache docstring for the paged layout (k_cache / v_cache
 * [num_blocks, page_block_size, nheads_k, headdim] with block_table
 * [batch, max_num_blocks_per_seq]), cache_seqlens, softmax_scale, num_splits
 * and the (batch, nheads) softmax_lse; the Ascend SFA blog for the -1
 * invalid index and gather-then-attend.  The list is read as a set of
 * positions (a selection), like the prefill's block lists.
 *
 *   q          bf16 [batch, num_heads_q, head_dim]
 *   k_cache, v_cache  bf16 [num_pages, page_size, num_heads_kv, head_dim]
 *   tok_idx    int32 [batch, num_heads_kv, topk]: logical cache positions,
 *              any order; entries outside [0, cache_seqlens[b]) are skipped,
 *              repeats count once
 *   block_table int32 [batch, max_pages_per_seq]: position t of sequence b is
 *              row t % page_size of page block_table[b][t / page_size]; a
 *              position whose page slot is >= max_pages_per_seq or whose page
 *              id is outside [0, num_pages) is skipped
 *   cache_seqlens int32 [batch]
 *   head_dim 64 or 128; 1 <= topk <= 8192; num_heads_q / num_heads_kv <= 16;
 *   num_pages * page_size < 2^31
 *   num_splits 0 = automatic (fsa_topk_decode_auto_splits), else 1..64: each
 *              (sequence, kv head) list is cut into that many parts whose
 *              partial results are merged by logsumexp
 *   workspace  at least fsa_topk_decode_workspace_size(...) bytes, 256-byte
 *              aligned; may be NULL when that size is 0
 *   out        bf16 [batch, num_heads_q, head_dim]
 *   lse        fp32 [batch, num_heads_q], or NULL
 * The query sits after every cache position, so the bottom-right causal rule
 * leaves every listed position t < cache_seqlens[b] visible.  The waves of a
 * workgroup take batches of the list as they free up, so the fp32 summation
 * order can change between calls: out may differ in the last bit run to run.
 */
fsa_status_t fsa_topk_decode(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* tok_idx, const int32_t* block_table,
                             const int32_t* cache_seqlens, int32_t batch, int32_t num_heads_q,
                             int32_t num_heads_kv, int32_t head_dim, int32_t page_size,
                             int32_t max_pages_per_seq, int32_t num_pages, int32_t topk,
                             float softmax_scale, int32_t num_splits, void* workspace,
                             size_t workspace_bytes, void* out, float* lse, void* stream);

/*
 * fsa_topk_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without workspace / workspace_bytes, the same kernels
 * and the same results.  The split partials (its only scratch) go to a
 * library-owned device array of FSA_NOALLOC_SCRATCH_BYTES per GPU, created
 * with the library's code object on that GPU and held until the process
 * ends; the call allocates and frees nothing.  It uses the array of the
 * calling thread's current device, so `stream` must belong to that device.
 * Nothing in the array needs clearing: every call overwrites the partials it
 * reads.  Calls that overlap in time on one GPU (other streams, other
 * threads) share the array and race.  A call whose partials would exceed
 * the array (fsa_topk_decode_workspace_size(...) > FSA_NOALLOC_SCRATCH_BYTES)
 * returns FSA_ERROR_WORKSPACE; other errors are those of fsa_topk_decode,
 * plus FSA_ERROR_LAUNCH if the array's address cannot be obtained.
 */
#define FSA_NOALLOC_SCRATCH_BYTES (32u << 20)
fsa_status_t fsa_topk_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* tok_idx, const int32_t* block_table,
                                     const int32_t* cache_seqlens, int32_t batch,
                                     int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                     int32_t page_size, int32_t max_pages_per_seq,
                                     int32_t num_pages, int32_t topk, float softmax_scale,
                                     int32_t num_splits, void* out, float* lse, void* stream);

/*
 * Top-k gathered decode over an FP8 paged KV cache: fsa_topk_decode with K
 * and V stored as FP8 E4M3 bytes (the torch.float8_e4m3fn format the
 * FlashAttention tutorial page lists; the flash-sparse-attn page's fused-quant
 * decode) and dequantisation factors as in the FP8 path of the
 * flash-attention-npu page's v3 docstrings (k_descale, v_descale).
 *
 *   k_cache, v_cache  uint8 [num_pages, page_size, num_heads_kv, head_dim]:
 *              the byte x of sequence b, kv head g stands for
 *              e4m3(x) * k_descale[b * num_heads_kv + g] (V: v_descale);
 *              16-byte aligned
 *   k_descale, v_descale  fp32 [batch, num_heads_kv] device arrays, or NULL
 *              for a factor of 1
 * All other arguments, the limits, the workspace
 * (fsa_topk_decode_workspace_size with the same arguments) and the error
 * behaviour are those of fsa_topk_decode; q, out and lse stay bf16 / fp32.
 * The two NaN codes (S.1111.111) are not meaningful cache contents: the
 * outputs of a list that reaches one are unspecified.
 */
fsa_status_t fsa_topk_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                                 const float* k_descale, const float* v_descale,
                                 const int32_t* tok_idx, const int32_t* block_table,
                                 const int32_t* cache_seqlens, int32_t batch, int32_t num_heads_q,
                                 int32_t num_heads_kv, int32_t head_dim, int32_t page_size,
                                 int32_t max_pages_per_seq, int32_t num_pages, int32_t topk,
                                 float softmax_scale, int32_t num_splits, void* workspace,
                                 size_t workspace_bytes, void* out, float* lse, void* stream);

/*
 * Block-index producer: the lists fsa_selected_attn_fwd reads, from a
 * compressed view of the keys (FSA page, quick start: kernel_size 32,
 * kernel_stride 16, block_size 64, topk, init_blocks 1, local_blocks 2; the
 * page gives the parameters, the steps below are the reading this library
 * takes):
 *   1. window j of a sequence covers keys [16j, 16j + 32) (windows that fit
 *      in the sequence); its summary c_j is the mean of those keys per kv
 *      head, rounded to bf16;
 *   2. row (token i, q head h) sees window j when 16j + 31 <= i + S_k - S_q
 *      (the whole window in its causal past); p_j = softmax of
 *      softmax_scale * <q, c_j> over the visible windows;
 *   3. block b (keys [64b, 64b + 64)) scores the probability mass of its keys,
 *      each window's p_j spread evenly over its 32 keys, summed over the q
 *      heads of the kv head's group;
 *   4. with qb = floor((i + S_k - S_q) / 64): blocks 0 .. init_blocks-1 (those
 *      <= qb), then the local blocks qb, qb-1, ... (local_blocks of them,
 *      >= 0, not yet listed), then the blocks in [init_blocks, qb -
 *      local_blocks + 1) of highest score (ties to the smaller id), in
 *      decreasing score order; -1 pads.  A row with qb < 0 gets all -1.
 *
 *   q        bf16 [total_q, num_heads_q, head_dim], 16-byte aligned
 *   k        bf16 [total_k, num_heads_kv, head_dim], 16-byte aligned
 *   cu_seqlens_q/k, batch, total_q/k, max_seqlen_q/k, head counts, head_dim
 *            (64 or 128), softmax_scale (<= 0: 1/sqrt(head_dim)): as in
 *            fsa_selected_attn_fwd; max_seqlen_k must bound every S_k
 *   kernel_size, kernel_stride, block_size  32, 16, 64 (others:
 *            FSA_ERROR_NOT_SUPPORTED)
 *   topk     1..64; init_blocks, local_blocks >= 0
 *            (num_heads_q / num_heads_kv <= 128; max_seqlen_k <= 2^20, so
 *            that a tile's block-importance table fits 64 KiB of LDS)
 *   workspace at least fsa_block_select_workspace_size(...) bytes (the
 *            compressed keys), 16-byte aligned; may be NULL when that is 0
 *   blk_idx  int32 [total_q, num_heads_kv, topk], written
 * Scores are accumulated in fp32 in an order that can vary between calls, so
 * blocks whose scores tie to rounding may swap places.
 */
size_t fsa_block_select_workspace_size(int32_t batch, int32_t max_seqlen_k, int32_t num_heads_kv,
                                       int32_t head_dim, int32_t kernel_size, int32_t kernel_stride);
fsa_status_t fsa_block_select(const void* q, const void* k, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, int32_t batch, int64_t total_q,
                              int64_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                              int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                              int32_t kernel_size, int32_t kernel_stride, int32_t block_size,
                              int32_t topk, int32_t init_blocks, int32_t local_blocks,
                              float softmax_scale, void* workspace, size_t workspace_bytes,
                              int32_t* blk_idx, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FSA_H_ */
