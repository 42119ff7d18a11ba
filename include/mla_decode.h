/*
 * mla_decode.h - C ABI of the MI355X (gfx950) MLA decode library
 * (libmla_decode.so).
 *
 * Operation.  Multi-head latent attention decode in absorbed form over a
 * paged latent KV cache.  Every cached token is ONE 576-wide vector shared by
 * all heads: a 512-wide latent c (kv_lora_rank) followed by a 64-wide rope
 * part r.  The pages size the split-KV partial as kv_lora_rank + 1 floats
 * (vLLM PR #46819 digest, "Key code excerpt") and fix the DeepSeek-R1 head
 * dims at 128 no-rope + 64 rope, so the default softmax scale is 1/sqrt(192)
 * (vLLM PR #41778 digest, "Risks and impact" item 4).  For query row
 * (b, t, h) and each visible token j:
 *
 *     s_j = softmax_scale * ( <q_nope[b,t,h,:], c_j> + <q_pe[b,t,h,:], r_j> )
 *     out[b,t,h,:] = sum_j softmax(s)_j * c_j          (latent space, 512 wide)
 *     lse[b,t,h]   = ln sum_j exp(s_j)                  (natural log)
 *
 * Visible tokens.  Dense calls: q_len = T draft tokens per sequence
 * (multi-token prediction, vLLM PR #41778 digest, "Motivation"); seq_lens[b]
 * counts the cache INCLUDING the T draft tokens, and draft token t sees
 * positions 0 .. seq_lens[b] - T + t (causal inside the draft).  Sparse
 * calls: token t of sequence b sees the positions listed in
 * topk_indices[b, t, 0..K) (index_topk per query token, vLLM PR #47327
 * digest, "Key code excerpt"); entries outside [0, seq_lens[b]) - the -1
 * padding included - are skipped, duplicates count as listed, and no
 * causal mask is added.  A row with no visible token gets out = 0 and
 * lse = -inf.
 *
 * Paging.  Position j of sequence b lives in page block_table[b, j / 64],
 * slot j % 64, of kv_cache [num_blocks, 64, 576] (row-major, 576 contiguous).
 * Only block_size = 64 is supported.
 *
 * Split-KV.  A call may cut each sequence's tokens into up to num_kv_splits
 * page-aligned pieces, write one fp32 partial per (b, row, piece) into the
 * caller's workspace [B, T*H, splits, 513] (512 normalized outputs, then the
 * piece's lse) and merge them by log-sum-exp in a second kernel, as in the
 * two-stage Triton MLA decode (vLLM PR #46819 digest, "Implementation"
 * items 1-3).  With one split the first kernel writes out and lse itself
 * and the workspace is not touched.
 *   A dense call with more than one split whose batch (at most 1024
 * sequences) is smaller than the number of pieces one round of resident
 * workgroups holds is cut by the actual lengths, on the device: every
 * sequence of n pages becomes k = max(1, ceil(n / c)) pieces of floor(n / k)
 * or ceil(n / k) pages, with one piece length c for the batch: the smallest
 * that keeps the batch within that number of pieces, and at least
 * ceil(longest / splits) pages.  A long
 * sequence of a mixed batch thus gets more pieces than a short one, and all
 * pieces are about equally long.  Slots past a sequence's k-th get lse =
 * -inf and no outputs.  The two-round plan of mla_num_kv_splits (two
 * splits, batch of one to two rounds of pieces) cuts the same way for two
 * rounds and numbers the pieces longest first.  Other calls cut fixed chunks of
 * ceil(ceil(max_seq_len / 64) / splits) pages.  Either way the merged result
 * is the same attention; rounding differs with the cut.
 *   Single launch (tokenspeed's in-kernel merge, vLLM PR #41778 digest,
 * "Implementation" item 1): with the environment variable
 * MLA_SINGLE_LAUNCH=1, a call whose units all fit the device at once (one
 * round of workgroups, at most 64 splits) runs as one kernel: the units of
 * each (sequence, row block) meet at two 8-byte words after the partials
 * and merge the block's rows themselves, with the same arithmetic and
 * result bits as the merge kernel.  The words carry the call's number and
 * need no clearing; they are left at zero counts, so graph replays work.
 * On MI355X it measures slower than the two launches (the units share no
 * L2, so their meeting costs device-scope round trips), so it is off by
 * default.
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is DEVICE memory owned by the caller, contiguous,
 *    row-major, on the current HIP device.  The library allocates nothing
 *    and keeps no state between calls beyond two caches: the compute-unit
 *    count of each device and the resident workgroups per compute unit of
 *    each kernel variant, both asked of the runtime once (256 and the LDS
 *    model are assumed where no device can be asked).  Plans follow the
 *    device's count, so a partitioned MI355X gets a plan for its share.
 *  - Calls enqueue on `stream` (a hipStream_t; NULL = the null stream) and
 *    return without synchronizing; they are safe to capture in a HIP graph.
 *  - Scales are read on every call and never cached (the pages record a
 *    bug where cached scales kept profiling-time values: vLLM PR #41778
 *    digest, "Review highlights").
 *  - q_len is uniform across the batch; non-uniform batches are not
 *    representable (the same review flags an unsafe fallback for them).
 *  - Errors the host can see are returned BEFORE any launch, and nothing is
 *    enqueued: bad dims, T outside [1, 8], block_size != 64, a NULL required
 *    pointer, num_kv_splits outside [0, MLA_MAX_KV_SPLITS], a softmax_scale
 *    (or fp8 q_scale / kv_scale) that is not positive and finite, a
 *    workspace smaller than mla_workspace_size().  A split may cover at most 1024
 *    pages (dense) or 1024 top-k entries (sparse); an explicit num_kv_splits
 *    that violates this returns MLA_ERR_UNSUPPORTED (the library's own choice
 *    never does).  A failed launch returns MLA_ERR_HIP.
 *  - Device data is not validated on the host.  In the kernels, seq_lens are
 *    clamped to [0, max_blocks_per_seq * 64], and block-table slots past a
 *    sequence's last page are never read.  A page number outside
 *    [0, num_blocks) is never dereferenced: in dense calls (and the MHA
 *    route) its tokens read as zero vectors, which still take part in the
 *    softmax with score 0; in sparse calls an index whose page is outside
 *    that range is skipped, as an index outside [0, seq_lens[b]) is.  seq_lens[b] must not exceed
 *    max_seq_len (the host bound that sizes the splits); tokens beyond
 *    num_kv_splits chunks of the bound (beyond the bound itself, when the
 *    device cuts the pieces) are not attended.
 *  - out and lse may not alias any input or the workspace.
 *
 * Two-stage use.  A decode call with out = NULL and lse = NULL stops after
 * the first stage: it writes the split partials into the workspace and
 * launches nothing else (this needs an explicit num_kv_splits >= 2).
 * mla_merge_partials() then runs the second stage on such a workspace.  The
 * stages can thus be timed, overlapped or fed with partials from elsewhere
 * (for instance chunks of a sequence held on other GPUs), while the one-call
 * form stays the common path.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = 1,
  MLA_ERR_UNSUPPORTED = 2,
  MLA_ERR_WORKSPACE_TOO_SMALL = 3,
  MLA_ERR_HIP = 4,
  MLA_ERR_SCRATCH_LIMIT = 5   /* mla_decode_fp8_noalloc: partials exceed its static buffer */
} mla_status_t;

/* Output element type of `out`. */
enum { MLA_OUT_BF16 = 0, MLA_OUT_F32 = 1 };

#define MLA_KV_LORA_RANK 512
#define MLA_ROPE_DIM 64
#define MLA_TOKEN_DIM 576
#define MLA_BLOCK_SIZE 64
#define MLA_MAX_Q_LEN 8
#define MLA_MAX_KV_SPLITS 256
#define MLA_MHA_MAX_Q_LEN 65536   /* mla_dense_mha only: query tokens per sequence */

/* Static text for a status code (never NULL).  A convenience of this library,
 * not an operation of the pages. */
const char* mla_status_string(mla_status_t status);

/*
 * Split count (partial slots per sequence) the library picks for a call when
 * num_kv_splits = 0.  The pages' Triton decode derives its split count from
 * max_seq_len and the SM count, in one function shared by the workspace
 * reservation and the kernel launch so that the two cannot drift (vLLM PR
 * #46819 digest, "Implementation" item 1 and "Key code excerpt"); here the
 * same function serves mla_workspace_size and the decode calls, and it is
 * costed for the device's compute units instead of a fixed work-per-split
 * rule.  Work units are (sequence, row block, split).  Each
 * candidate row-block width and split count is costed, for sequences of
 * max_seq_len, as the bytes it moves (the KV once per row block, plus the
 * fp32 partials written and read back when split) divided by how fully its
 * units occupy the chip's workgroup slots; the cheapest wins.  A dense call
 * whose pieces are cut by the actual lengths (see Split-KV above) then gets
 * twice that many slots (at most one per page), so that long sequences of a
 * mixed batch can take more pieces.  A dense call that the costing gives one
 * split, with at least four row blocks per sequence and a batch that fills
 * one round of workgroup slots but not two (at most 64 sequences), gets 2:
 * its sequences are cut into pieces for two rounds, dispatched longest piece
 * first.  Passing the returned count explicitly gives the same launch.  Deterministic in its arguments; topk = 0 means a
 * dense call, otherwise a sparse call with that K.  kv_fp8 (nonzero for the
 * fp8 calls) is an argument the pages' rule does not have: the fp8 kernels
 * hold the same tile in half the LDS, and their residency, which the
 * costing uses, differs.  Returns 0 on invalid arguments.
 */
int mla_num_kv_splits(int batch, int q_len, int num_heads, int max_seq_len, int topk,
                      int kv_fp8);

/*
 * Waves per workgroup (1, 2 or 4; each wave owns 32 query rows) that a call
 * with these arguments launches.  Follows from the shape alone, whatever
 * num_kv_splits is; lets tests and tuning tell which kernel variant a shape
 * runs.  A query of this library's plan, not an operation of the pages.
 * Returns 0 on invalid arguments.
 */
int mla_launch_waves(int batch, int q_len, int num_heads, int max_seq_len, int topk, int kv_fp8);

/*
 * Workspace bytes a call needs: batch * q_len * num_heads * splits * 513 * 4,
 * the fp32 partials of kv_lora_rank + 1 floats per (row, split) that the
 * pages' Triton decode reserves ahead of time as [B, H, splits, 513]
 * (vLLM PR #46819 digest, "Implementation" item 2 and "Key code excerpt";
 * tokenspeed sizes its preallocated workspace with the same 513-float rows,
 * vLLM PR #41778 digest, "Implementation" item 1), or 0 when the call runs
 * with one split; with the single launch (below)
 * rounded up to 16 and followed by 16 bytes per (sequence, row block).  num_kv_splits = 0 means the
 * heuristic choice above.  Returns 0 for invalid arguments as well; pass the
 * same arguments to the decode call.
 */
size_t mla_workspace_size(int batch, int q_len, int num_heads, int max_seq_len, int topk,
                          int kv_fp8, int num_kv_splits);

/*
 * Dense bf16 decode.
 *   q_nope      [B, T, H, 512] bf16   absorbed no-rope query
 *   q_pe        [B, T, H, 64]  bf16   rope query
 *   kv_cache    [num_blocks, 64, 576] bf16
 *   block_table [B, max_blocks_per_seq] int32
 *   seq_lens    [B] int32, tokens in the cache per sequence (draft included)
 *   max_seq_len host upper bound of seq_lens (sizes the splits)
 *   out         [B, T, H, 512] in out_dtype (MLA_OUT_BF16 or MLA_OUT_F32), or
 *               NULL together with lse for the first stage only (see above)
 *   lse         [B, T, H] fp32, or NULL
 *   workspace   >= mla_workspace_size(B, T, H, max_seq_len, 0, 0, num_kv_splits)
 *               bytes (may be NULL when that size is 0); contents on entry
 *               are ignored and left undefined on return
 *   num_kv_splits 0 = library choice, else 1 .. MLA_MAX_KV_SPLITS
 */
mla_status_t mla_decode(const void* q_nope, const void* q_pe, const void* kv_cache,
                        const int32_t* block_table, const int32_t* seq_lens, int batch,
                        int q_len, int num_heads, int num_blocks, int block_size,
                        int max_blocks_per_seq, int max_seq_len, float softmax_scale,
                        void* out, int out_dtype, float* lse, void* workspace,
                        size_t workspace_bytes, int num_kv_splits, void* stream);

/*
 * Dense fp8 decode.  q_nope, q_pe and kv_cache hold OCP e4m3fn bytes with
 * one per-tensor dequant scale each: the query value is byte * q_scale (one
 * scale for q_nope and q_pe together) and the cache value byte * kv_scale
 * (fp8 decode with dequant scales, vLLM PR #41778 digest, "Implementation"
 * item 1).  Logits use softmax_scale * q_scale * kv_scale; the output is the
 * dequantized latent average, i.e. it carries kv_scale.  Inside, both
 * products run on fp8 MFMA; the softmax probabilities are scaled by 2^8
 * before their e4m3 rounding so they stay in the format's normal range.
 * Work units planned at most 16384 tokens long also multiply V by the e4m3
 * residual of the probabilities (about 2^-8 per weight).  Longer units
 * skip that product while their weight is spread over many tokens: a row
 * whose bound of sum w^2 (w its normalized weights) exceeds 2^-7 gets the
 * residual product of its heaviest 64-token tile added, or, when that tile
 * alone does not bring it under the bound, its unit reruns with the
 * residual product throughout.  One launch per stage either way.  Other
 * arguments as mla_decode;
 * workspace sized with kv_fp8 = 1.
 */
mla_status_t mla_decode_fp8(const void* q_nope, const void* q_pe, const void* kv_cache,
                            const int32_t* block_table, const int32_t* seq_lens, int batch,
                            int q_len, int num_heads, int num_blocks, int block_size,
                            int max_blocks_per_seq, int max_seq_len, float softmax_scale,
                            float q_scale, float kv_scale, void* out, int out_dtype, float* lse,
                            void* workspace, size_t workspace_bytes, int num_kv_splits,
                            void* stream);

/*
 * mla_decode_fp8 for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same arguments without workspace / workspace_bytes, the same plan,
 * kernels and results.  The split partials go to a static device buffer of
 * 64 MiB that the library holds on each GPU it runs on until the process
 * ends; its address is looked up once per device, on the first call made
 * with that device current.  The call allocates nothing.
 *   A call whose partials (mla_workspace_size(B, T, H, max_seq_len, 0, 1,
 * num_kv_splits) bytes) exceed 64 MiB returns MLA_ERR_SCRATCH_LIMIT before
 * anything is enqueued; pass a smaller num_kv_splits to fit.  Every call on
 * one GPU shares that GPU's buffer, so calls that overlap on one GPU (on
 * different streams, or from different threads without ordering) race and
 * give undefined results.  Nothing in the buffer has to start at a given
 * value: each call writes every partial it later reads.
 */
mla_status_t mla_decode_fp8_noalloc(const void* q_nope, const void* q_pe, const void* kv_cache,
                                    const int32_t* block_table, const int32_t* seq_lens, int batch,
                                    int q_len, int num_heads, int num_blocks, int block_size,
                                    int max_blocks_per_seq, int max_seq_len, float softmax_scale,
                                    float q_scale, float kv_scale, void* out, int out_dtype, float* lse,
                                    int num_kv_splits, void* stream);

/*
 * Dense un-absorbed multi-head attention over the paged latent cache: the
 * route the pages take for sparse-MLA batches whose sequences all fit in
 * top-k (then every position is in the top-k list, so the attention is
 * dense), when the query count passes a threshold (vLLM PR #47327
 * digest, "Summary" and "Implementation" item 2).  Each head h expands the cached
 * latents with its own up-projections (DeepSeek-R1 dims: 128 no-rope + 64
 * rope for keys, 128 for values; vLLM PR #41778 digest, "Risks and impact"
 * item 4):
 *     k[h,j] = [ W_UK[h] c_j ; r_j ]  (192)     v[h,j] = W_UV[h] c_j  (128)
 *     out[b,t,h,:] = sum_j softmax_j(softmax_scale * <q[b,t,h], k[h,j]>) v[h,j]
 *     lse[b,t,h]   = ln sum_j exp(softmax_scale * <q[b,t,h], k[h,j]>)
 * over positions j = 0 .. seq_lens[b] - q_len + t (causal, as in the
 * decode calls; with q_len = seq_lens[b] this is a whole prefill).  It pays
 * off over the absorbed form when many query tokens share a sequence's
 * expansion, and costs far more than it at decode sizes.
 *   q_nope   [B, T, H, 128] bf16   un-absorbed no-rope query
 *   q_pe     [B, T, H, 64]  bf16   rope query
 *   kv_cache, block_table, seq_lens, block_size, max_seq_len as mla_decode
 *   w_uk, w_uv [H, 128, 512] bf16  W_UK[h][d][k], W_UV[h][d][k]
 *   out      [B, T, H, 128] in out_dtype; lse [B, T, H] fp32 or NULL
 *   workspace >= mla_dense_mha_workspace_size(B, H, max_seq_len) bytes
 *             (the expanded K and V, bf16, each sequence padded to a multiple
 *             of 128 tokens); contents on entry ignored
 * The expanded keys and values are rounded to bf16 (the model's activation
 * type; the pages leave it open), products accumulate in fp32, and the
 * softmax weights enter the value product as bf16.
 * q_len is 1 .. MLA_MHA_MAX_Q_LEN; softmax_scale must be positive and finite.
 * Rows that see no token get 0 and -inf.
 * Two kernels on `stream` (expansion, then attention); no allocation.
 */
size_t mla_dense_mha_workspace_size(int batch, int num_heads, int max_seq_len);
mla_status_t mla_dense_mha(const void* q_nope, const void* q_pe, const void* kv_cache,
                           const int32_t* block_table, const int32_t* seq_lens, const void* w_uk,
                           const void* w_uv, int batch, int q_len, int num_heads, int num_blocks,
                           int block_size, int max_blocks_per_seq, int max_seq_len,
                           float softmax_scale, void* out, int out_dtype, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Top-k sparse bf16 decode.  topk_indices [B, T, K] int32 lists, per query
 * token, the cache positions it attends (shared by all heads); see
 * "Visible tokens" above.  K >= 1.  Workspace sized with topk = K.  Other
 * arguments as mla_decode.
 */
mla_status_t mla_sparse_decode(const void* q_nope, const void* q_pe, const void* kv_cache,
                               const int32_t* block_table, const int32_t* seq_lens,
                               const int32_t* topk_indices, int topk, int batch, int q_len,
                               int num_heads, int num_blocks, int block_size,
                               int max_blocks_per_seq, int max_seq_len, float softmax_scale,
                               void* out, int out_dtype, float* lse, void* workspace,
                               size_t workspace_bytes, int num_kv_splits, void* stream);

/*
 * Top-k sparse fp8 decode: the token lists of mla_sparse_decode over the
 * e4m3fn cache and query of mla_decode_fp8, with the same per-tensor
 * q_scale and kv_scale (index_topk per query token, vLLM PR #47327 digest,
 * "Key code excerpt"; fp8 dequant scales, vLLM PR #41778 digest,
 * "Implementation" item 1).  A gathered token row is 576 bytes.  Every work
 * unit holds at most 1024 indices, so the softmax weights always get the
 * second (residual) fp8 product that carries them to about 2^-8.  Workspace
 * sized with topk = K and kv_fp8 = 1; other arguments as mla_sparse_decode.
 */
mla_status_t mla_sparse_decode_fp8(const void* q_nope, const void* q_pe, const void* kv_cache,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   const int32_t* topk_indices, int topk, int batch, int q_len,
                                   int num_heads, int num_blocks, int block_size,
                                   int max_blocks_per_seq, int max_seq_len, float softmax_scale,
                                   float q_scale, float kv_scale, void* out, int out_dtype,
                                   float* lse, void* workspace, size_t workspace_bytes,
                                   int num_kv_splits, void* stream);

/*
 * Second stage alone: log-sum-exp merge of split partials.
 *   workspace  [rows, num_kv_splits, 513] fp32, as a decode call writes it
 *              (rows = B * T * H; per (row, split): 512 normalized outputs
 *              then the split's lse, -inf for a split that saw no token)
 *   out        [rows, 512] in out_dtype; lse [rows] fp32 or NULL
 * out = sum_s exp(lse_s - lse) * O_s with lse = ln sum_s exp(lse_s), the
 * merge of the two-stage Triton MLA decode (vLLM PR #46819 digest,
 * "Implementation" items 1-3); rows whose splits are all empty get 0 and
 * -inf.  The outputs of a split whose weight exp(lse_s - lse) is zero (an
 * empty one above all) are not read, so they may hold anything.
 * num_kv_splits in [1, MLA_MAX_KV_SPLITS].
 */
mla_status_t mla_merge_partials(const float* workspace, int64_t rows, int num_kv_splits, void* out,
                                int out_dtype, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
