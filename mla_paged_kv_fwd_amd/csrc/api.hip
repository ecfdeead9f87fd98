// libmla C ABI: argument validation and launches.  Every host-visible error is
// reported before the first HIP call.
#include <math.h>

#include <atomic>

#include "../../include/mla.h"
#include "common.h"

namespace mla {
hipError_t launch_plan(const int32_t *seqlens, int batch, int c, int num_parts, int32_t *meta,
                       int32_t *split_base, hipStream_t stream);
void plan_host(const int32_t *seqlens, int batch, int c, int num_parts, int32_t *meta,
               int32_t *split_base);
hipError_t launch_decode(const DecodeArgs &a, bool fp8, hipStream_t stream);
int decode_rows_per_group();
hipError_t launch_decode_rows64(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_decode_rows64_fp8(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_decode_rows128(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_kv_write(const uint16_t *k_new, int batch, int n_new, const int32_t *block_table,
                           int64_t bt_stride, const int32_t *seqlens, void *cache, bool fp8,
                           hipStream_t stream);
hipError_t launch_sparse_ids(const int32_t *indices, const int32_t *block_table,
                             int64_t bt_stride, int rows, int s_q, int topk, int tok_per,
                             int32_t *lens, int32_t *ids, hipStream_t stream);
hipError_t launch_check_block_table(const int32_t *seqlens, int batch, const int32_t *block_table,
                                    int64_t bt_stride, int64_t num_pages,
                                    unsigned long long *result, hipStream_t stream);
hipError_t launch_check_sparse(const int32_t *block_table, int64_t bt_stride, int64_t num_pages,
                               const int32_t *indices, int rows, int s_q, int topk,
                               unsigned long long *result, hipStream_t stream);
hipError_t launch_combine(const int32_t *split_base, int batch, int M, const float *o_part,
                          const float *lse_part, uint16_t *out, float *lse, hipStream_t stream);
}  // namespace mla

namespace mla {
// Scratch of the allocation-free decode (see scratch_address below).
__device__ __align__(256) unsigned char scratch[(size_t)MLA_NOALLOC_SCRATCH_BYTES];
}  // namespace mla

static_assert(MLA_D_QK == mla::kDQk && MLA_D_V == mla::kDV && MLA_PAGE == mla::kPage &&
                  MLA_FP8_RECORD == mla::kTokBytesFp8 && MLA_META_INTS == mla::kMetaInts &&
                  MLA_MAX_BATCH == mla::kMaxBatch && MLA_MAX_PARTS == mla::kMaxParts,
              "header and kernels disagree");

namespace {

// Kernel choice.  64 query rows per work-group with specialised score /
// value waves when a request has at least 32 rows (32 rows leave half the
// group as padding: the problem is memory-bound and reads each page once
// instead of twice); 16 rows per work-group otherwise.  128-row requests over
// a bf16 cache (dense decode) run on the 128-row kernel instead when the plan
// has at least one part per CU: it runs a part on one work-group (the 64-row
// kernel on two), so such plans fill the chip with it, and it is the faster
// kernel when the parts are long (it halves the LDS traffic per row; with
// short parts its larger fixed cost per segment loses).
// mla_default_num_parts_for plans one part per CU exactly when the parts are
// long.  With 256 or 512 rows the 64-row kernel is as fast or faster (a
// part's row groups share its half-pages through L2, and with half the parts
// per CU fewer requests are split, so fewer partial results are written and
// merged).
bool use_rows128(int M, int kv_format, int token_list, int num_parts, int cus) {
    return M == 128 && kv_format == 0 && !token_list && num_parts >= cus;
}
bool use_rows64(int M) { return M >= 32; }
int rows64_groups(int M) { return (M + 63) / 64; }  // M = 32 pads one group
// work-groups per part of the 64- and 16-row kernels
int groups_per_part(int M, int token_list) {
    (void)token_list;  // token lists run on the same kernels as dense decode
    if (use_rows64(M)) return rows64_groups(M);
    return M / 16;
}
// Pages per part from which a 128-row plan with one part per CU beats the
// 64-row kernel's plan (measured: 32 pages per part lose or tie, 64 win).
constexpr int kRows128MinPagesPerPart = 48;

// CUs of each device, queried once (0: not yet)
int g_cu_count[64];
// CU count of `device`, or a status code (< 0)
int cu_count(int device) {
    if (device < 0 || device >= 64) return MLA_ERR_INVALID_ARG;
    if (g_cu_count[device] <= 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
            cus <= 0)
            return MLA_ERR_HIP;
        g_cu_count[device] = cus;
    }
    return g_cu_count[device];
}

bool shape_supported(int s_q, int h_q) {
    return (s_q == 1 || s_q == 2 || s_q == 4) && (h_q == 16 || h_q == 32 || h_q == 64 || h_q == 128);
}

mla_status check_plan_args(int batch, int s_q, int h_q, int num_parts) {
    if (batch <= 0 || num_parts <= 0 || s_q <= 0 || h_q <= 0) return MLA_ERR_INVALID_ARG;
    if (batch > mla::kMaxBatch || num_parts > mla::kMaxParts) return MLA_ERR_UNSUPPORTED;
    if (!shape_supported(s_q, h_q)) return MLA_ERR_UNSUPPORTED;
    return MLA_OK;
}

size_t workspace_bytes(int batch, int s_q, int h_q, int num_parts) {
    const size_t slots = (size_t)batch + (size_t)num_parts;
    const size_t rows = (size_t)s_q * h_q;
    return slots * rows * (mla::kDV + 1) * sizeof(float);
}

mla_status decode_attn_impl(const void *q, const void *kcache, int kv_format, int64_t num_pages,
                            const int32_t *block_table, int block_table_stride,
                            const int32_t *seqlens, int batch, int s_q, int h_q,
                            float softmax_scale, int causal, const int32_t *meta,
                            const int32_t *split_base, int num_parts, void *workspace,
                            size_t ws_bytes, void *out, float *lse, void *stream,
                            int token_list = 0) {
    if (!q || !kcache || !block_table || !seqlens || !meta || !split_base || !out || !lse)
        return MLA_ERR_INVALID_ARG;
    if (kv_format != 0 && kv_format != 1) return MLA_ERR_INVALID_ARG;
    if (num_pages <= 0 || block_table_stride < 1) return MLA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return MLA_ERR_INVALID_ARG;
    if (!isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_INVALID_ARG;
    mla_status st = check_plan_args(batch, s_q, h_q, num_parts);
    if (st != MLA_OK) return st;
    if (!workspace) return MLA_ERR_WORKSPACE;
    if (ws_bytes < workspace_bytes(batch, s_q, h_q, num_parts)) return MLA_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255) != 0) return MLA_ERR_WORKSPACE;

    mla::DecodeArgs a;
    const int M = s_q * h_q;
    const size_t slots = (size_t)batch + num_parts;
    a.q = (const uint16_t *)q;
    a.kv = (const unsigned char *)kcache;
    a.block_table = block_table;
    a.seqlens = seqlens;
    a.meta = meta;
    a.split_base = split_base;
    a.o_part = (float *)workspace;
    a.lse_part = (float *)workspace + slots * M * mla::kDV;
    a.out = (uint16_t *)out;
    a.lse = lse;
    a.bt_stride = block_table_stride;
    a.batch = batch;
    a.s_q = s_q;
    a.h_q = h_q;
    a.M = M;
    a.num_parts = num_parts;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    a.causal = causal;
    a.token_list = token_list;
    hipError_t e;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
    const int cus = cu_count(dev);
    if (cus < 0) return (mla_status)cus;
    // token lists run on the 64-row kernels, or on the 16-row kernel for M = 16
    if (use_rows128(M, kv_format, token_list, num_parts, cus)) {
        a.row_groups = M / 128;
        e = mla::launch_decode_rows128(a, (hipStream_t)stream);
    } else if (use_rows64(M)) {
        a.row_groups = rows64_groups(M);
        e = kv_format == 1 ? mla::launch_decode_rows64_fp8(a, (hipStream_t)stream)
                           : mla::launch_decode_rows64(a, (hipStream_t)stream);
    } else {
        a.row_groups = M / mla::decode_rows_per_group();
        e = mla::launch_decode(a, kv_format == 1, (hipStream_t)stream);
    }
    return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status combine_impl(const int32_t *split_base, int batch, int s_q, int h_q, int num_parts,
                        const void *workspace, size_t ws_bytes, void *out, float *lse,
                        void *stream) {
    if (!split_base || !out || !lse) return MLA_ERR_INVALID_ARG;
    mla_status st = check_plan_args(batch, s_q, h_q, num_parts);
    if (st != MLA_OK) return st;
    if (!workspace || ws_bytes < workspace_bytes(batch, s_q, h_q, num_parts))
        return MLA_ERR_WORKSPACE;
    const int M = s_q * h_q;
    const size_t slots = (size_t)batch + num_parts;
    const float *o_part = (const float *)workspace;
    const float *lse_part = o_part + slots * M * mla::kDV;
    hipError_t e = mla::launch_combine(split_base, batch, M, o_part, lse_part, (uint16_t *)out,
                                       lse, (hipStream_t)stream);
    return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status kv_write_impl(const void *k_new, int batch, int n_new, const int32_t *block_table,
                         int block_table_stride, const int32_t *seqlens, void *kcache,
                         int64_t num_pages, bool fp8, void *stream) {
    if (!k_new || !block_table || !seqlens || !kcache) return MLA_ERR_INVALID_ARG;
    if (batch <= 0 || n_new <= 0 || block_table_stride < 1 || num_pages <= 0)
        return MLA_ERR_INVALID_ARG;
    if (batch > mla::kMaxBatch || (int64_t)batch * n_new > 0x7FFFFFFFLL) return MLA_ERR_UNSUPPORTED;
    hipError_t e = mla::launch_kv_write((const uint16_t *)k_new, batch, n_new, block_table,
                                        block_table_stride, seqlens, kcache, fp8,
                                        (hipStream_t)stream);
    return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

// Sparse decode workspace: the token ids [rows][64 * pages], the list
// lengths, the plan, then the decode workspace of the one-token problems.
struct SparseLayout {
    size_t ids, lens, meta, split_base, decode_ws, decode_ws_bytes, total;
};

SparseLayout sparse_layout(int batch, int s_q, int h_q, int topk, int kv_format, int num_parts) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t rows = (size_t)batch * s_q, pages = (size_t)(topk + mla::kPage - 1) / mla::kPage;
    (void)kv_format;  // the records are read in place: the layout is the same for both
    SparseLayout L;
    size_t off = 0;
    L.ids = off;
    off += up(rows * pages * mla::kPage * 4);
    L.lens = off;
    off += up(rows * 4);
    L.meta = off;
    off += up((size_t)num_parts * mla::kMetaInts * 4);
    L.split_base = off;
    off += up((rows + 1) * 4);
    L.decode_ws = off;
    L.decode_ws_bytes = workspace_bytes((int)rows, 1, h_q, num_parts);
    off += up(L.decode_ws_bytes);
    L.total = off;
    return L;
}

mla_status decode_sparse_impl(const void *q, const void *kcache, int kv_format, int64_t num_pages,
                              const int32_t *block_table, int block_table_stride,
                              const int32_t *indices, int topk, int batch, int s_q, int h_q,
                              float softmax_scale, int num_parts, void *workspace, size_t ws_bytes,
                              void *out, float *lse, void *stream) {
    if (!q || !kcache || !block_table || !indices || !out || !lse) return MLA_ERR_INVALID_ARG;
    if (kv_format != 0 && kv_format != 1) return MLA_ERR_INVALID_ARG;
    if (num_pages <= 0 || block_table_stride < 1 || topk < 1) return MLA_ERR_INVALID_ARG;
    if (!isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_INVALID_ARG;
    if (batch <= 0 || s_q <= 0 || h_q <= 0 || num_parts <= 0) return MLA_ERR_INVALID_ARG;
    if (!shape_supported(s_q, h_q)) return MLA_ERR_UNSUPPORTED;
    const int rows = batch * s_q;
    mla_status st = check_plan_args(rows, 1, h_q, num_parts);
    if (st != MLA_OK) return st;
    const SparseLayout L = sparse_layout(batch, s_q, h_q, topk, kv_format, num_parts);
    if (!workspace || ws_bytes < L.total || ((uintptr_t)workspace & 255) != 0)
        return MLA_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    unsigned char *ws = (unsigned char *)workspace;
    const int pages_per = (int)(((int64_t)topk + mla::kPage - 1) / mla::kPage);
    // the plan and the id lists count list positions in int32
    if ((int64_t)rows * pages_per * mla::kPage > 0x7FFFFFFFLL) return MLA_ERR_UNSUPPORTED;
    // token ids are int32: page * 64 + slot must stay below 2^31
    if (num_pages > 0x7FFFFFFFLL / mla::kPage) return MLA_ERR_UNSUPPORTED;
    int32_t *lens = (int32_t *)(ws + L.lens), *ids = (int32_t *)(ws + L.ids);
    int32_t *meta = (int32_t *)(ws + L.meta), *split_base = (int32_t *)(ws + L.split_base);
    hipError_t e = mla::launch_sparse_ids(indices, block_table, block_table_stride, rows, s_q,
                                          topk, pages_per * mla::kPage, lens, ids, s);
    if (e == hipSuccess)
        // no overhead units: full lists are equally long, and a list split over
        // two parts pays its fixed cost in both, so equal page shares balance
        // the parts (with c units per list, one half got c pages fewer)
        e = mla::launch_plan(lens, rows, 0, num_parts, meta, split_base, s);
    if (e != hipSuccess) return MLA_ERR_HIP;
    // the one-token problems: q, out and lse keep their memory layout
    st = decode_attn_impl(q, kcache, kv_format, num_pages, ids, pages_per * mla::kPage, lens, rows,
                          1, h_q, softmax_scale, 0, meta, split_base, num_parts, ws + L.decode_ws,
                          L.decode_ws_bytes, out, lse, stream, 1);
    if (st != MLA_OK) return st;
    return combine_impl(split_base, rows, 1, h_q, num_parts, ws + L.decode_ws, L.decode_ws_bytes,
                        out, lse, stream);
}


// Scratch of the allocation-free decode (mla_decode_fwd_noalloc): the plan and
// the split workspace of one call, in a file-scope device array that every
// GPU the library runs on holds until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is a stand-in, not a
// device address): each device's address comes from hipGetSymbolAddress,
// taken once per device with that device current.
constexpr size_t kNoallocScratch = (size_t)MLA_NOALLOC_SCRATCH_BYTES;
std::atomic<unsigned char *> g_scratch_dev[64];

mla_status scratch_address(unsigned char **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MLA_ERR_HIP;
    unsigned char *p = g_scratch_dev[dev].load(std::memory_order_acquire);
    if (!p) {
        void *addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(mla::scratch)) != hipSuccess || !addr)
            return MLA_ERR_HIP;
        p = (unsigned char *)addr;
        g_scratch_dev[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return MLA_OK;
}

}  // namespace

extern "C" {

const char *mla_status_string(int status) {
    switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported shape";
    case MLA_ERR_WORKSPACE:
        return "workspace missing, too small or misaligned (or, for the allocation-free "
               "decode, the problem needs more than its fixed scratch)";
    case MLA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

size_t mla_metadata_ints(int num_parts) {
    return num_parts > 0 ? (size_t)num_parts * mla::kMetaInts : 0;
}

size_t mla_workspace_bytes(int batch, int s_q, int h_q, int num_parts) {
    if (batch <= 0 || s_q <= 0 || h_q <= 0 || num_parts <= 0) return 0;
    return workspace_bytes(batch, s_q, h_q, num_parts);
}

int mla_plan_overhead(int s_q, int h_q) { return mla::plan_overhead(s_q, h_q); }

int mla_default_num_parts_ex(int device, int s_q, int h_q, int kv_format, int sparse) {
    if (!shape_supported(s_q, h_q)) return MLA_ERR_UNSUPPORTED;
    if ((kv_format != 0 && kv_format != 1) || (sparse != 0 && sparse != 1)) return MLA_ERR_INVALID_ARG;
    const int cus = cu_count(device);
    if (cus < 0) return cus;
    // one work-group per CU, all in one round: a part spans as many
    // work-groups as the kernel that runs it has row groups (sparse decode
    // plans one-token problems of h_q rows)
    const int M = sparse ? h_q : s_q * h_q;
    int parts = cus / groups_per_part(M, sparse);
    parts = parts < 8 ? 8 : parts;
    return (parts + 7) / 8 * 8;
}

int mla_default_num_parts_for(int device, int batch, int max_seqlen, int s_q, int h_q, int kv_format,
                              int sparse) {
    const int parts = mla_default_num_parts_ex(device, s_q, h_q, kv_format, sparse);
    if (parts < 0) return parts;
    if (batch < 0 || max_seqlen < 0) return MLA_ERR_INVALID_ARG;
    const int cus = cu_count(device);
    if (cus < 0) return cus;
    // 128-row requests over a bf16 cache with long parts: one part per CU,
    // which runs them on the 128-row kernel
    const int64_t pages = (int64_t)batch * (((int64_t)max_seqlen + mla::kPage - 1) / mla::kPage);
    const int one_per_cu = (cus + 7) / 8 * 8;
    if (!sparse && kv_format == 0 && s_q * h_q == 128 &&
        pages >= (int64_t)kRows128MinPagesPerPart * one_per_cu)
        return one_per_cu;
    return parts;
}

int mla_default_num_parts(int device, int s_q, int h_q) {
    return mla_default_num_parts_ex(device, s_q, h_q, 0, 0);
}

mla_status mla_get_metadata(const int32_t *seqlens, int batch, int s_q, int h_q, int num_parts,
                            int32_t *meta, int32_t *split_base, void *stream) {
    if (!seqlens || !meta || !split_base) return MLA_ERR_INVALID_ARG;
    mla_status st = check_plan_args(batch, s_q, h_q, num_parts);
    if (st != MLA_OK) return st;
    hipError_t e = mla::launch_plan(seqlens, batch, mla::plan_overhead(s_q, h_q), num_parts, meta,
                                    split_base, (hipStream_t)stream);
    return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_get_metadata_host(const int32_t *seqlens_host, int batch, int s_q, int h_q,
                                 int num_parts, int32_t *meta_host, int32_t *split_base_host) {
    if (!seqlens_host || !meta_host || !split_base_host) return MLA_ERR_INVALID_ARG;
    mla_status st = check_plan_args(batch, s_q, h_q, num_parts);
    if (st != MLA_OK) return st;
    mla::plan_host(seqlens_host, batch, mla::plan_overhead(s_q, h_q), num_parts, meta_host,
                   split_base_host);
    return MLA_OK;
}

mla_status mla_decode_attn(const void *q, const void *kcache, int kv_format, int64_t num_pages,
                           const int32_t *block_table, int block_table_stride,
                           const int32_t *seqlens, int batch, int s_q, int h_q,
                           float softmax_scale, int causal, const int32_t *meta,
                           const int32_t *split_base, int num_parts, void *workspace,
                           size_t workspace_bytes_, void *out, float *lse, void *stream) {
    return decode_attn_impl(q, kcache, kv_format, num_pages, block_table, block_table_stride,
                            seqlens, batch, s_q, h_q, softmax_scale, causal, meta, split_base,
                            num_parts, workspace, workspace_bytes_, out, lse, stream);
}

mla_status mla_decode_combine(const int32_t *split_base, int batch, int s_q, int h_q,
                              int num_parts, const void *workspace, size_t workspace_bytes_,
                              void *out, float *lse, void *stream) {
    return combine_impl(split_base, batch, s_q, h_q, num_parts, workspace, workspace_bytes_, out,
                        lse, stream);
}

static mla_status decode_fwd(const void *q, const void *kcache, int kv_format, int64_t num_pages,
                             const int32_t *block_table, int block_table_stride,
                             const int32_t *seqlens, int batch, int s_q, int h_q,
                             float softmax_scale, int causal, const int32_t *meta,
                             const int32_t *split_base, int num_parts, void *workspace,
                             size_t ws_bytes, void *out, float *lse, void *stream) {
    mla_status st = decode_attn_impl(q, kcache, kv_format, num_pages, block_table,
                                     block_table_stride, seqlens, batch, s_q, h_q, softmax_scale,
                                     causal, meta, split_base, num_parts, workspace, ws_bytes, out,
                                     lse, stream);
    if (st != MLA_OK) return st;
    return combine_impl(split_base, batch, s_q, h_q, num_parts, workspace, ws_bytes, out, lse,
                        stream);
}

mla_status mla_decode_fwd(const void *q, const void *kcache, int64_t num_pages,
                          const int32_t *block_table, int block_table_stride,
                          const int32_t *seqlens, int batch, int s_q, int h_q,
                          float softmax_scale, int causal, const int32_t *meta,
                          const int32_t *split_base, int num_parts, void *workspace,
                          size_t workspace_bytes_, void *out, float *lse, void *stream) {
    return decode_fwd(q, kcache, 0, num_pages, block_table, block_table_stride, seqlens, batch,
                      s_q, h_q, softmax_scale, causal, meta, split_base, num_parts, workspace,
                      workspace_bytes_, out, lse, stream);
}

mla_status mla_decode_fwd_fp8(const void *q, const void *kcache_fp8, int64_t num_pages,
                              const int32_t *block_table, int block_table_stride,
                              const int32_t *seqlens, int batch, int s_q, int h_q,
                              float softmax_scale, int causal, const int32_t *meta,
                              const int32_t *split_base, int num_parts, void *workspace,
                              size_t workspace_bytes_, void *out, float *lse, void *stream) {
    return decode_fwd(q, kcache_fp8, 1, num_pages, block_table, block_table_stride, seqlens, batch,
                      s_q, h_q, softmax_scale, causal, meta, split_base, num_parts, workspace,
                      workspace_bytes_, out, lse, stream);
}

size_t mla_noalloc_scratch_need(int batch, int s_q, int h_q, int kv_format) {
    if (batch <= 0 || s_q <= 0 || h_q <= 0 || (kv_format != 0 && kv_format != 1)) return 0;
    if (!shape_supported(s_q, h_q) || batch > mla::kMaxBatch) return 0;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    // the larger of the plans the call may make (one part per CU for
    // 128-row requests with long contexts)
    int parts = mla_default_num_parts_ex(dev, s_q, h_q, kv_format, 0);
    if (parts <= 0) return 0;
    if (s_q * h_q == 128 && kv_format == 0) {
        const int cus = cu_count(dev);
        if (cus <= 0) return 0;
        const int one_per_cu = (cus + 7) / 8 * 8;
        parts = parts > one_per_cu ? parts : one_per_cu;
    }
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    return up((size_t)parts * mla::kMetaInts * 4) + up(((size_t)batch + 1) * 4) +
           workspace_bytes(batch, s_q, h_q, parts);
}

mla_status mla_decode_fwd_noalloc(const void *q, const void *kcache, int kv_format,
                                  int64_t num_pages, const int32_t *block_table,
                                  int block_table_stride, const int32_t *seqlens, int batch,
                                  int s_q, int h_q, float softmax_scale, int causal, void *out,
                                  float *lse, void *stream) {
    // host-visible argument errors first, as for the other decode calls
    if (!q || !kcache || !block_table || !seqlens || !out || !lse) return MLA_ERR_INVALID_ARG;
    if (kv_format != 0 && kv_format != 1) return MLA_ERR_INVALID_ARG;
    if (num_pages <= 0 || block_table_stride < 1) return MLA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return MLA_ERR_INVALID_ARG;
    if (!isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_INVALID_ARG;
    if (batch <= 0 || s_q <= 0 || h_q <= 0) return MLA_ERR_INVALID_ARG;
    if (batch > mla::kMaxBatch || !shape_supported(s_q, h_q)) return MLA_ERR_UNSUPPORTED;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
    // plan size from the longest request the table can hold
    const int64_t max_len = (int64_t)block_table_stride * mla::kPage;
    const int parts = mla_default_num_parts_for(dev, batch, max_len < INT32_MAX ? (int)max_len : INT32_MAX,
                                                s_q, h_q, kv_format, 0);
    if (parts <= 0) return parts < 0 ? (mla_status)parts : MLA_ERR_HIP;
    // scratch layout: meta, split_base, then the split workspace (256-byte aligned)
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t meta_off = 0, sb_off = up((size_t)parts * mla::kMetaInts * 4);
    const size_t ws_off = sb_off + up(((size_t)batch + 1) * 4);
    const size_t ws_bytes = workspace_bytes(batch, s_q, h_q, parts);
    if (ws_off + ws_bytes > kNoallocScratch) return MLA_ERR_WORKSPACE;
    unsigned char *base = nullptr;
    mla_status st = scratch_address(&base);
    if (st != MLA_OK) return st;
    int32_t *meta = (int32_t *)(base + meta_off), *split_base = (int32_t *)(base + sb_off);
    hipError_t e = mla::launch_plan(seqlens, batch, mla::plan_overhead(s_q, h_q), parts, meta,
                                    split_base, (hipStream_t)stream);
    if (e != hipSuccess) return MLA_ERR_HIP;
    return decode_fwd(q, kcache, kv_format, num_pages, block_table, block_table_stride, seqlens,
                      batch, s_q, h_q, softmax_scale, causal, meta, split_base, parts,
                      base + ws_off, ws_bytes, out, lse, stream);
}

size_t mla_sparse_workspace_bytes(int batch, int s_q, int h_q, int topk, int kv_format,
                                  int num_parts) {
    if (batch <= 0 || s_q <= 0 || h_q <= 0 || topk <= 0 || num_parts <= 0) return 0;
    if (kv_format != 0 && kv_format != 1) return 0;
    if ((int64_t)batch * s_q * (((int64_t)topk + mla::kPage - 1) / mla::kPage) * mla::kPage >
        0x7FFFFFFFLL)
        return 0;  // beyond what mla_decode_sparse accepts
    return sparse_layout(batch, s_q, h_q, topk, kv_format, num_parts).total;
}

mla_status mla_decode_sparse(const void *q, const void *kcache, int kv_format, int64_t num_pages,
                             const int32_t *block_table, int block_table_stride,
                             const int32_t *indices, int topk, int batch, int s_q, int h_q,
                             float softmax_scale, int num_parts, void *workspace,
                             size_t workspace_bytes_, void *out, float *lse, void *stream) {
    return decode_sparse_impl(q, kcache, kv_format, num_pages, block_table, block_table_stride,
                              indices, topk, batch, s_q, h_q, softmax_scale, num_parts, workspace,
                              workspace_bytes_, out, lse, stream);
}

mla_status mla_kv_cache_write(const void *k_new, int batch, int n_new,
                              const int32_t *block_table, int block_table_stride,
                              const int32_t *seqlens, void *kcache, int64_t num_pages,
                              void *stream) {
    return kv_write_impl(k_new, batch, n_new, block_table, block_table_stride, seqlens, kcache,
                         num_pages, false, stream);
}

mla_status mla_kv_cache_write_fp8(const void *k_new, int batch, int n_new,
                                  const int32_t *block_table, int block_table_stride,
                                  const int32_t *seqlens, void *kcache_fp8, int64_t num_pages,
                                  void *stream) {
    return kv_write_impl(k_new, batch, n_new, block_table, block_table_stride, seqlens,
                         kcache_fp8, num_pages, true, stream);
}

mla_status mla_check_block_table(const int32_t *seqlens, int batch, const int32_t *block_table,
                                 int block_table_stride, int64_t num_pages, uint64_t *result,
                                 void *stream) {
    if (!seqlens || !block_table || !result) return MLA_ERR_INVALID_ARG;
    if (batch <= 0 || block_table_stride < 1 || num_pages <= 0) return MLA_ERR_INVALID_ARG;
    if (batch > mla::kMaxBatch) return MLA_ERR_UNSUPPORTED;
    hipError_t e = mla::launch_check_block_table(seqlens, batch, block_table, block_table_stride,
                                                 num_pages, (unsigned long long *)result,
                                                 (hipStream_t)stream);
    return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_check_sparse_indices(const int32_t *block_table, int block_table_stride,
                                    int64_t num_pages, const int32_t *indices, int topk,
                                    int batch, int s_q, uint64_t *result, void *stream) {
    if (!block_table || !indices || !result) return MLA_ERR_INVALID_ARG;
    if (batch <= 0 || s_q <= 0 || topk < 1 || block_table_stride < 1 || num_pages <= 0)
        return MLA_ERR_INVALID_ARG;
    if ((int64_t)batch * s_q > mla::kMaxBatch) return MLA_ERR_UNSUPPORTED;
    hipError_t e = mla::launch_check_sparse(block_table, block_table_stride, num_pages, indices,
                                            batch * s_q, s_q, topk, (unsigned long long *)result,
                                            (hipStream_t)stream);
    return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"
