// Pieces shared by the 64-row decode kernels (bf16 and FP8 caches): the
// work-group shape, request segments of a split part, the softmax restart
// threshold and the output epilogue.
#pragma once

#include "common.h"
#include "device_util.h"

namespace mla {
namespace rows64 {

constexpr int kThreads = 256;   // 4 waves: 2 score waves, 2 value waves
constexpr int kRowsWG = 64;     // query rows per work-group
constexpr int kHalf = 32;       // tokens per step (half a page)
constexpr int kRing = 4;        // half-pages resident in LDS
// Reference headroom (log2 units) before a segment restarts.  Weights up to
// 2^64 stay exact in bf16's exponent range and their sums over any sequence
// stay far below fp32's, so a large headroom only makes restarts rarer.
constexpr float kGrowLog2 = 64.f;
constexpr int kXStride = kDV + 4;  // padded row stride of the output stage

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Both halves' maximum for lanes l and l ^ 32.
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int N>
__device__ __forceinline__ void wait_own_dma(bool more) {
    if (more) wait_vmcnt<N>(); else wait_vmcnt<0>();
}

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// One request segment of a part: pages j0..j1 of request b.
struct Segment {
    int b, L, npages, j0, rank, nsplit, H;  // H = number of 32-token steps
    const int32_t *bt;
    // last valid token (0..31) of half-page t of the segment
    __device__ __forceinline__ int tok_last(int t) const {
        const int first = (j0 + (t >> 1)) * kPage + (t & 1) * kHalf;
        const int last = L - 1 - first;
        return last < kHalf - 1 ? last : kHalf - 1;
    }
};

// Calls f(seg) for every non-empty request segment of a part, in order.
template <class F>
__device__ __forceinline__ void for_each_segment(const int32_t *mrow, const int32_t *seqlens,
                                                 const int32_t *split_base,
                                                 const int32_t *block_table, int64_t bt_stride,
                                                 F &&f) {
    const int b_first = mrow[0], j_first = mrow[1], b_last = mrow[2], j_last = mrow[3];
    for (int b = b_first; b <= b_last; ++b) {
        Segment sg;
        sg.b = b;
        sg.L = seqlens[b];
        if (sg.L <= 0) continue;
        sg.npages = (sg.L + kPage - 1) / kPage;
        sg.j0 = (b == b_first) ? j_first : 0;
        const int j1 = (b == b_last) ? j_last : sg.npages - 1;
        sg.rank = (b == b_first) ? mrow[4] : 0;
        sg.nsplit = split_base[b + 1] - split_base[b];
        sg.bt = block_table + (int64_t)b * bt_stride;
        // the last page may hold a single half
        const int tok_end = (j1 == sg.npages - 1) ? sg.L : (j1 + 1) * kPage;
        sg.H = (tok_end - sg.j0 * kPage + kHalf - 1) / kHalf;
        f(sg);
    }
}

// Token-list mode (sparse decode).  A "request" is then one query token's
// list of cache token ids (physical page * 64 + slot, in list order), and the
// block-table argument holds these lists, bt_stride ids apart: half-page u of
// a segment covers list positions 64 j0 + 32 u .. + 31.  The score waves copy
// the ids of a half-page into LDS slot u % kRing before the value waves issue
// its loads, which then address each token's row by its id.
__device__ __forceinline__ const int32_t *list_ids(const Segment &sg, int u) {
    return sg.bt + sg.j0 * kPage + u * kHalf;
}

// Ids of half-pages 0, 1, 2 (those the value waves load before the first
// step's barrier) into their LDS slots; lanes 0..31 of a score wave.
__device__ __forceinline__ void stage_first_ids(lds_i32 *ids, const Segment &sg, int l32, int h) {
    if (h == 0) {
#pragma unroll
        for (int u = 0; u < 3; ++u)
            if (u < sg.H) ids[u * kHalf + l32] = list_ids(sg, u)[l32];
    }
}

// All 256 threads: the staged [64][kXStride] fp32 output -> out (bf16) or the
// segment's split slot (fp32), four threads per row, coalesced.  Rows at or
// past M (padding of a 32-row problem) are not written.
__device__ __forceinline__ void write_rows(const DecodeArgs &a, const Segment &sg,
                                           const int32_t *split_base, const float *X,
                                           const float *row_sum, int row0, int tid) {
    // 16 threads per row, four rounds of 16 rows; thread j of a row takes
    // dims 4 j + 64 k (k = 0..7), so the 16 lanes of an LDS pass read 64
    // consecutive floats of one row (no bank conflicts) and write 256
    // consecutive bytes of it
    const int j = tid & 15;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const int r = 16 * rr + (tid >> 4);
        const int orow = row0 + r;
        if (orow >= a.M) continue;
        const float *xr = X + r * kXStride + 4 * j;
        const float lsum = row_sum[r];
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        if (sg.nsplit == 1) {
            uint16_t *dst = a.out + ((int64_t)sg.b * a.M + orow) * kDV + 4 * j;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const f32x4 u = *(const f32x4 *)(xr + 64 * k) * inv;
                *(u32x2 *)(dst + 64 * k) = (u32x2){pack_bf16(u[0], u[1]), pack_bf16(u[2], u[3])};
            }
        } else {
            float *dst = a.o_part + ((int64_t)(split_base[sg.b] + sg.rank) * a.M + orow) * kDV + 4 * j;
#pragma unroll
            for (int k = 0; k < 8; ++k) *(f32x4 *)(dst + 64 * k) = *(const f32x4 *)(xr + 64 * k) * inv;
        }
    }
}

// Stage O^T (unnormalised fp32, 2 row tiles x 8 dim tiles of 32x32) of the
// value wave owning dims d0 .. d0 + 255 in LDS as [row][dim].  Lane holds,
// for row tile r, row 32 r + lane % 32 and dims d0 + 32 dt + 8 (i / 4) +
// 4 (lane / 32) + (i % 4).  Plain stores straight from the accumulators.
__device__ __forceinline__ void stage_output(float *X, const f32x16 (&o)[2][8], int d0, int lane) {
    const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        float *xrow = X + (32 * r + l32) * kXStride + d0 + 4 * h;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const f32x16 &acc = o[r][dt];
                *(f32x4 *)(xrow + 32 * dt + 8 * qd) =
                    (f32x4){acc[4 * qd], acc[4 * qd + 1], acc[4 * qd + 2], acc[4 * qd + 3]};
            }
    }
}

// Zeroes the accumulators with MFMAs (0 x 0 + 0), so they are born in the
// accumulator registers; plain zero stores get hoisted into 256 VGPRs of
// constants by the compiler.  Each tile gets its own zero operand from an asm
// statement: identical MFMAs would be merged into one whose result is then
// copied into the other tiles.
__device__ __forceinline__ void zero_acc(f32x16 (&o)[2][8]) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            u32x4 zw;
            asm volatile("v_mov_b32 %0, 0\n\tv_mov_b32 %1, 0\n\tv_mov_b32 %2, 0\n\tv_mov_b32 %3, 0"
                         : "=v"(zw[0]), "=v"(zw[1]), "=v"(zw[2]), "=v"(zw[3]));
            const bf16x8 zf = __builtin_bit_cast(bf16x8, zw);
            o[r][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(zf, zf, (f32x16){}, 0, 0, 0);
        }
}

}  // namespace rows64
}  // namespace mla
