/*
 * libmla -- Multi-head Latent Attention decode over a paged latent KV cache,
 * for AMD MI355X (gfx950).
 *
 * What is computed.  For each request b (cached length L_b), each of its s_q
 * new query tokens i and each of h_q query heads h, one attention row:
 *     score_j = softmax_scale * <q[b,i,h,0:576], K_j[0:576]>,  j < n(b,i)
 *     lse     = ln sum_j exp(score_j)
 *     out     = sum_j exp(score_j - lse) * K_j[0:512]
 * Every head shares the same cached latent row K_j per token: the MQA-style
 * sharing of one KV stream that MLA uses, with a 512-dim compressed latent
 * plus a 64-dim decoupled RoPE part (Novita AI FlashMLA page, section
 * "Was ist MLA?", MHA/MQA/GQA/MLA comparison table).  The value is the first
 * 512 dims of the same row.  n(b,i) = L_b without causal masking; with causal
 * masking row i is the (s_q-1-i)-th newest token and sees L_b - (s_q-1-i)
 * keys.  A row that sees no key gets out = 0, lse = -inf.
 *
 * Cache layouts (both paged in blocks of 64 tokens: DeepSeek launch
 * announcement on the 8bitnewsroom FlashMLA page; aivengo.media feature list):
 *   bf16: [num_pages][64][576] bf16, 1152 bytes per token.
 *   fp8 : [num_pages][64][656] bytes, one 656-byte record per token
 *         (DeepSeek KB page, "Key Contributions": 656 vs 1152 bytes per
 *         token, RoPE slice kept in BF16): bytes [0,512) OCP E4M3FN codes of
 *         latent dims 0..511; [512,528) four little-endian fp32 scales, one per
 *         128-dim tile (value = code * scale); [528,656) 64 bf16 RoPE dims.
 * block_table[b * block_table_stride + j] is the physical page holding
 * tokens [64 j, 64 j + 64) of request b.  Only entries j < ceil(L_b / 64) are
 * read; cache slots at or beyond L_b are never read.
 *
 * Conventions.
 *   - Pointers are device pointers unless a name ends in _host.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every device
 *     call only enqueues work on it and returns; nothing synchronises.
 *   - The caller owns every buffer.  The library allocates and frees nothing
 *     and keeps no state besides a per-device cache of the CU count (and the
 *     fixed scratch array of mla_decode_fwd_noalloc, with its per-device
 *     address).
 *   - Tensors are dense and row-major:
 *       q     bf16  [batch][s_q][h_q][576]
 *       out   bf16  [batch][s_q][h_q][512]
 *       lse   fp32  [batch][s_q][h_q]      (natural log)
 *       seqlens int32 [batch]; block_table int32 [batch][block_table_stride]
 *   - Shapes supported: s_q in {1, 2, 4}; h_q in {16, 32, 64, 128}; one shared
 *     KV head; d_qk 576, d_v 512, page 64.  Others: MLA_ERR_UNSUPPORTED.
 *   - Argument errors that the host can see are reported before any HIP call.
 *     Device-resident contents (page ids inside [0, num_pages), lengths that
 *     fit the block table, sparse list entries) are the caller's contract and
 *     are not checked by the decode calls; mla_check_block_table and
 *     mla_check_sparse_indices (end of this header) check them on demand.
 *   - Every device call only launches kernels (no memsets, copies or
 *     allocations), so a decode step can be captured in a HIP graph.
 *
 * Entry points: planning (mla_get_metadata, mla_get_metadata_host), decode
 * (mla_decode_fwd, mla_decode_fwd_fp8, and its halves mla_decode_attn and
 * mla_decode_combine; mla_decode_fwd_noalloc, which allocates nothing and
 * needs no workspace), sparse decode over token lists (mla_decode_sparse),
 * the cache writer (mla_kv_cache_write, mla_kv_cache_write_fp8), device-side
 * input checks, and size / default queries.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, bad stride */
    MLA_ERR_UNSUPPORTED = -2, /* shape outside the supported set */
    MLA_ERR_WORKSPACE = -3,   /* workspace smaller than mla_workspace_bytes */
    MLA_ERR_HIP = -4          /* a HIP runtime call or launch failed */
} mla_status;

#define MLA_D_QK 576
#define MLA_D_V 512
#define MLA_PAGE 64
#define MLA_FP8_RECORD 656
#define MLA_META_INTS 8
/* Largest batch (requests; for mla_decode_sparse: batch * s_q lists) and
 * largest num_parts any call accepts; beyond them MLA_ERR_UNSUPPORTED. */
#define MLA_MAX_BATCH 16384
#define MLA_MAX_PARTS 16384

/* Static string for a status code.  Thread-safe; never NULL. */
const char *mla_status_string(int status);

/* Number of int32 in the plan buffer `meta` for num_parts parts. */
size_t mla_metadata_ints(int num_parts);

/* Bytes of split workspace needed by mla_decode_* for these sizes (the upper
 * bound over every plan with num_parts parts: at most batch + num_parts
 * request segments, each holding s_q*h_q rows of 512 fp32 + 1 fp32 lse). */
size_t mla_workspace_bytes(int batch, int s_q, int h_q, int num_parts);

/* Overhead, in page units, that the planner charges per request segment:
 * 1 + (s_q * h_q) / 64. */
int mla_plan_overhead(int s_q, int h_q);

/* Plan size suited to the kernels on `device` (a multiple of 8 derived from
 * the CU count: one work-group per CU); < 0 on error (status code).  Needs a
 * visible GPU.  mla_default_num_parts is for the bf16 dense decode;
 * mla_default_num_parts_ex gives the size for a cache format (kv_format 0 =
 * bf16, 1 = FP8 records) and for sparse decode (sparse = 1; s_q is then
 * ignored: the plan covers one-token problems), whose kernels may run a part
 * on a different number of work-groups.  Any num_parts gives the same result;
 * these sizes fill the GPU in one round.
 *
 * mla_default_num_parts_for also takes the batch and the longest request
 * (max_seqlen tokens; the block table's width times 64 will do) and returns
 * the size this library measures fastest: for 128 query rows per request
 * (s_q * h_q = 128) over a bf16 cache with at least 48 pages per part at one
 * part per CU, one part per CU (the CU count rounded up to a multiple of 8);
 * otherwise mla_default_num_parts_ex's size.
 *
 * Which kernel a dense decode runs follows from the plan: 128-row requests
 * over a bf16 cache run on the 128-row kernel (one work-group per part) when
 * num_parts >= the device's CU count, and on the 64-row kernel (two
 * work-groups per part) otherwise.  Both give the same result within the
 * tolerance. */
int mla_default_num_parts(int device, int s_q, int h_q);
int mla_default_num_parts_ex(int device, int s_q, int h_q, int kv_format, int sparse);
int mla_default_num_parts_for(int device, int batch, int max_seqlen, int s_q, int h_q,
                              int kv_format, int sparse);

/*
 * Split-KV plan.  Cuts the batch's pages into num_parts contiguous pieces of
 * equal cost so that every CU gets the same amount of work however the
 * lengths vary (the launch announcement quoted on the 8bitnewsroom FlashMLA
 * page says the kernel targets variable-length batches; the cut rule is this
 * library's).  Definition: request b has n_b = ceil(L_b/64) pages; requests
 * with pages are laid end to end on a cost line, each taking
 * c = mla_plan_overhead(s_q, h_q) units then one unit per page, total T.
 * With P = min(num_parts, T), the page at cost position x goes to part
 * floor(x * P / T).
 *   seqlens    int32 [batch] (device); lengths >= 0 with T < 2^31 (the
 *              plan counts cost units in int32; the lengths are device data,
 *              so this is the caller's contract, as are the table contents)
 *   meta       int32 [num_parts][8] (device, written): for a part with pages
 *              {b_first, j_first, b_last, j_last, split_first, 0, 0, 0} --
 *              it runs from page j_first of request b_first to page j_last of
 *              b_last inclusive; split_first is its rank among the parts that
 *              touch b_first.  A part without pages has b_first = -1.
 *   split_base int32 [batch + 1] (device, written): prefix sum of the number
 *              of parts touching each request; request b owns workspace split
 *              slots [split_base[b], split_base[b+1]).
 * One small kernel on `stream`; no host synchronisation.
 */
mla_status mla_get_metadata(const int32_t *seqlens, int batch, int s_q, int h_q, int num_parts,
                            int32_t *meta, int32_t *split_base, void *stream);

/* The same plan computed on the host from host arrays (no GPU needed). */
mla_status mla_get_metadata_host(const int32_t *seqlens_host, int batch, int s_q, int h_q,
                                 int num_parts, int32_t *meta_host, int32_t *split_base_host);

/*
 * bf16-cache decode: attention kernel plus, for requests the plan split, the
 * LSE merge of their partial results (mla_decode_attn then mla_decode_combine).
 *   q           bf16 [batch][s_q][h_q][576]
 *   kcache      bf16 [num_pages][64][576]
 *   block_table int32 [batch][block_table_stride]
 *   seqlens     int32 [batch]
 *   softmax_scale  multiplies the full 576-dim dot product; finite and > 0
 *   causal      0 or 1 (only matters for s_q > 1)
 *   meta, split_base, num_parts   a plan from mla_get_metadata for the same
 *               seqlens, s_q, h_q
 *   workspace   >= mla_workspace_bytes(batch, s_q, h_q, num_parts) bytes,
 *               256-byte aligned; scratch owned by the caller
 *   out         bf16 [batch][s_q][h_q][512];  lse  fp32 [batch][s_q][h_q]
 */
mla_status mla_decode_fwd(const void *q, const void *kcache, int64_t num_pages,
                          const int32_t *block_table, int block_table_stride,
                          const int32_t *seqlens, int batch, int s_q, int h_q,
                          float softmax_scale, int causal, const int32_t *meta,
                          const int32_t *split_base, int num_parts, void *workspace,
                          size_t workspace_bytes, void *out, float *lse, void *stream);

/* FP8-cache decode: as mla_decode_fwd with kcache_fp8 = uint8
 * [num_pages][64][656] records (E4M3FN codes dequantised in the kernel). */
mla_status mla_decode_fwd_fp8(const void *q, const void *kcache_fp8, int64_t num_pages,
                              const int32_t *block_table, int block_table_stride,
                              const int32_t *seqlens, int batch, int s_q, int h_q,
                              float softmax_scale, int causal, const int32_t *meta,
                              const int32_t *split_base, int num_parts, void *workspace,
                              size_t workspace_bytes, void *out, float *lse, void *stream);

/*
 * First half of mla_decode_fwd{,_fp8}: the attention kernel alone.  Writes
 * out/lse for requests the plan did not split and partial results
 * (normalised fp32 output + lse per split slot) into the workspace for the
 * others.  kv_format: 0 = bf16 cache, 1 = fp8 records.  Arguments as above.
 */
mla_status mla_decode_attn(const void *q, const void *kcache, int kv_format, int64_t num_pages,
                           const int32_t *block_table, int block_table_stride,
                           const int32_t *seqlens, int batch, int s_q, int h_q,
                           float softmax_scale, int causal, const int32_t *meta,
                           const int32_t *split_base, int num_parts, void *workspace,
                           size_t workspace_bytes, void *out, float *lse, void *stream);

/*
 * Second half: for every request with two or more split slots, merges the
 * slots' partial results by their log-sum-exp (merged lse = ln sum_s
 * exp(lse_s); out = sum_s exp(lse_s - lse) * o_s) and writes out/lse.
 * Requests with no pages get out = 0, lse = -inf.  Requests with one slot
 * are left as mla_decode_attn wrote them.  Workspace layout: o fp32
 * [batch + num_parts][s_q*h_q][512], then lse fp32 [batch + num_parts][s_q*h_q].
 */
mla_status mla_decode_combine(const int32_t *split_base, int batch, int s_q, int h_q,
                              int num_parts, const void *workspace, size_t workspace_bytes,
                              void *out, float *lse, void *stream);

/*
 * Allocation-free decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): mla_decode_fwd / mla_decode_fwd_fp8 (kv_format 0 / 1) with the
 * plan made inside the call (mla_default_num_parts_for parts, with max_seqlen
 * = 64 * block_table_stride) and the plan and the split workspace held in the
 * library's own scratch, a fixed device array of MLA_NOALLOC_SCRATCH_BYTES per
 * GPU, held from the library's first use on that GPU until the process ends.
 * The call allocates and frees nothing; the caller passes inputs and outputs
 * as for mla_decode_fwd.  Problems whose plan and workspace need more than
 * the scratch (mla_noalloc_scratch_need returns the need on the current
 * device for the larger plan the call may make, 0 for bad arguments) get
 * MLA_ERR_WORKSPACE before any launch.  Every call on one GPU shares that
 * GPU's scratch: calls that overlap in time on one GPU (different streams,
 * or threads) race and must be serialised by the caller.  Nothing in the
 * scratch needs clearing between calls (every value read is written by the
 * same call).  Three kernels on `stream` (plan, attention, merge).
 */
#define MLA_NOALLOC_SCRATCH_BYTES (128u << 20)
size_t mla_noalloc_scratch_need(int batch, int s_q, int h_q, int kv_format);
mla_status mla_decode_fwd_noalloc(const void *q, const void *kcache, int kv_format,
                                  int64_t num_pages, const int32_t *block_table,
                                  int block_table_stride, const int32_t *seqlens, int batch,
                                  int s_q, int h_q, float softmax_scale, int causal, void *out,
                                  float *lse, void *stream);

/*
 * Sparse decode: query token i of request b attends only to the cached tokens
 * its list names (DeepSeek KB page, "Key Contributions": the FP8 cache serves
 * a sparse decode kernel; the list comes from an indexer the pages do not
 * describe).
 *   indices  int32 [batch][s_q][topk]: token positions within request b; the
 *            list of (b, i) ends at its first negative entry (pad short lists
 *            with -1).  A position listed twice counts twice.  Positions must
 *            lie inside the request's cached length (caller's contract, like
 *            block-table contents).
 * Every head h of (b, i) attends over the listed keys (no causal mask: the
 * list decides); a token whose list is empty gets out = 0, lse = -inf.
 * The call plans num_parts parts over batch * s_q one-token problems of
 * their list lengths, decodes them and merges the splits: one pass over the
 * listed tokens per query token instead of the whole cache.  The decode
 * reads each listed row (bf16) or record (FP8) in place, through per-list
 * token ids (page * 64 + slot, int32: needs num_pages * 64 < 2^31, else
 * MLA_ERR_UNSUPPORTED).  Entries at or past the first negative one are
 * never dereferenced.
 *   kv_format 0 = bf16 cache, 1 = FP8 records; q, out, lse as for decode.
 *   batch * s_q <= 16384; topk >= 1 and batch * s_q * 64 * ceil(topk / 64)
 *   < 2^31 (list positions are counted in int32; the size query returns 0
 *   beyond it); num_parts as for mla_get_metadata
 *   (mla_default_num_parts_ex(device, 1, h_q, kv_format, 1) suits).
 *   workspace >= mla_sparse_workspace_bytes(...) bytes, 256-byte aligned.
 */
size_t mla_sparse_workspace_bytes(int batch, int s_q, int h_q, int topk, int kv_format,
                                  int num_parts);
mla_status mla_decode_sparse(const void *q, const void *kcache, int kv_format, int64_t num_pages,
                             const int32_t *block_table, int block_table_stride,
                             const int32_t *indices, int topk, int batch, int s_q, int h_q,
                             float softmax_scale, int num_parts, void *workspace,
                             size_t workspace_bytes, void *out, float *lse, void *stream);

/*
 * Cache writer: stores the rows of the newest n_new tokens of every request
 * in the paged cache.  Row i of request b (k_new[b][i]: 576 bf16 values, 512
 * latent then 64 RoPE) is the token at position L_b - n_new + i (seqlens count
 * the new tokens, as for decode; rows at negative positions are skipped): page
 * block_table[b * block_table_stride + pos / 64], slot pos % 64.
 *   k_new       bf16 [batch][n_new][576] (device)
 *   kcache      mla_kv_cache_write: bf16 [num_pages][64][576], the row is
 *               copied.  mla_kv_cache_write_fp8: [num_pages][64][656] records
 *               (layout above); per 128-dim latent tile scale = amax / 448 in
 *               fp32 (448 is E4M3FN's largest finite value; an all-zero tile
 *               gets scale 0 and zero codes) and code = E4M3FN
 *               round-to-nearest-even of x / scale (fp32 division, clipped to
 *               +-448); the RoPE dims are copied.  The pages give the record
 *               layout (DeepSeek KB page, "Key Contributions") but not the
 *               quantiser; this is its plain reading.
 *   n_new >= 1; batch * n_new < 2^31.  A decode step appends s_q rows per
 *   request; a prefill passes whole sequences right-aligned in n_new rows.
 * Nothing else in the cache is written.  One kernel on `stream`; rows of
 * different requests must not map to the same slot.
 */
mla_status mla_kv_cache_write(const void *k_new, int batch, int n_new,
                              const int32_t *block_table, int block_table_stride,
                              const int32_t *seqlens, void *kcache, int64_t num_pages,
                              void *stream);
mla_status mla_kv_cache_write_fp8(const void *k_new, int batch, int n_new,
                                  const int32_t *block_table, int block_table_stride,
                                  const int32_t *seqlens, void *kcache_fp8, int64_t num_pages,
                                  void *stream);

/*
 * Device-side checks of the caller's device data.  The decode, sparse and
 * writer calls take block-table contents, lengths and list entries on trust
 * (like any paged-attention kernel); these calls verify them on the device,
 * reading only table entries inside the table, so they are safe on the very
 * inputs they reject.  Each writes result (device, 2 x uint64, 8-byte
 * aligned) on `stream`; read it after synchronising:
 *   result[0]  number of bad requests (mla_check_block_table) or bad lists
 *              (mla_check_sparse_indices); 0 if all is well
 *   result[1]  smallest (request_or_list << 32) | where over the bad ones,
 *              ~0 if none.  where = first bad logical page (a table entry
 *              outside [0, num_pages)), first bad list position (its page
 *              is past the table's width or its entry is outside the pool),
 *              or 0xFFFFFFFF for a length that is negative or needs more
 *              than block_table_stride pages.  A list is b * s_q + i.
 * mla_check_block_table covers pages 0 .. ceil(L_b / 64) - 1 of each request;
 * mla_check_sparse_indices covers entries before each list's first negative
 * one.  Two kernels on `stream`; graph-capturable; argument errors as for
 * the decode calls.
 */
mla_status mla_check_block_table(const int32_t *seqlens, int batch, const int32_t *block_table,
                                 int block_table_stride, int64_t num_pages, uint64_t *result,
                                 void *stream);
mla_status mla_check_sparse_indices(const int32_t *block_table, int block_table_stride,
                                    int64_t num_pages, const int32_t *indices, int topk,
                                    int batch, int s_q, uint64_t *result, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
