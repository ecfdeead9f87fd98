// MLA decode attention for 128 query rows per work-group (s_q * h_q >= 128)
// over a bf16 cache: gfx950 kernel in which every wave owns its rows outright.
//
// A work-group (4 waves, one per SIMD) owns one split-KV part and one group of
// 128 query rows.  Wave w owns rows 32 w .. 32 w + 31 of the group: their Q^T
// operand (144 VGPRs), their O^T accumulator over all 512 value dims (256
// AGPRs) and their softmax state.  For each 32-token half-page every wave
//   - computes S^T (32 tokens x 32 rows) = K . Q^T on 32x32x16 bf16 MFMAs;
//   - takes the softmax of its rows in registers.  The S^T accumulator layout
//     (lane = row, 16 tokens per lane) is the layout of the P^T operand of the
//     value MFMA once the V reads take the tokens in the matching order, so P
//     is only rounded to bf16 in place and never leaves the wave;
//   - accumulates O^T (512 dims x 32 rows) += V^T . P^T, V^T read from LDS
//     with transposing reads;
//   - issues its quarter of the direct-to-LDS loads of half-page t + 3 (one
//     group of eight tokens, nine 1 KB loads).
// Every half-page brought into LDS serves 128 rows, twice as many as in the
// 64-row kernel (whose score and value waves each leave half of the register
// file unused), so each CU moves half as many bytes per FLOP.
//
// Half-pages use the layout of halfpage_bf16.h in a 4-deep LDS ring: in step t
// the waves read half-page t, and half-pages t + 1 .. t + 3 are in flight.  One
// work-group barrier per step.  The softmax reference and restart scheme are
// those of the 64-row kernels: a fixed exponent reference per row for a pass
// over a request segment, and a work-group restart of the segment when a
// row's running max passes it by more than kGrowLog2.
#include <math.h>

#include "common.h"
#include "device_util.h"
#include "halfpage_bf16.h"
#include "rows64.h"

namespace mla {

namespace {

using namespace rows64;

constexpr int kRows = 128;                       // query rows per work-group
constexpr int kHalfBytes = halfpage::kBytes;     // 36864
constexpr int kDmaPerWave = halfpage::kBlocksPerGroup;  // 9 loads per wave per step
constexpr int kAhead = 3;                        // half-pages in flight beyond the current one
constexpr int kFlagOff = kRing * kHalfBytes;     // restart flags [2 parities][4 waves]
constexpr int kStatOff = kFlagOff + 64;          // final row sums [128]
constexpr int kLdsBytes = kStatOff + kRows * 4;
static_assert(kAhead == kRing - 1, "the slot of half-page t + kAhead is the one half-page t - 1 used");
static_assert(64 * kXStride * 4 <= kRing * kHalfBytes, "output stage fits over the ring");

// Wave w's loads of half-page t of a segment: token group w, lines 0..8.
struct GroupDma {
    const unsigned char *src;
    unsigned dst;  // LDS byte address of the group's first 1 KB block
    __device__ __forceinline__ void issue(int lam) const {
        dma16(src + 128 * lam, __builtin_amdgcn_readfirstlane(dst + lam * 1024));
    }
};

// Page of half-page t of a segment.
__device__ __forceinline__ int page_of(const Segment &sg, int t) { return sg.bt[sg.j0 + (t >> 1)]; }

__device__ __forceinline__ GroupDma group_dma(const Segment &sg, const unsigned char *kv, int t,
                                              int64_t phys, int w, int lane, unsigned ring0) {
    const int j = sg.j0 + (t >> 1);
    const int tok_last = (j == sg.npages - 1) ? (sg.L - 1 - j * kPage) : (kPage - 1);
    GroupDma d;
    d.src = halfpage::dma_row(kv, phys, (t & 1) * kHalf, tok_last, w, lane);
    d.dst = ring0 + (t % kRing) * kHalfBytes + halfpage::kBlocksPerGroup * w * 1024;
    return d;
}

__device__ __forceinline__ void issue_group(const Segment &sg, const unsigned char *kv, int t,
                                            int w, int lane, unsigned ring0) {
    const GroupDma d = group_dma(sg, kv, t, page_of(sg, t), w, lane, ring0);
#pragma unroll
    for (int lam = 0; lam < kDmaPerWave; ++lam) d.issue(lam);
}

// Wait until this wave's loads of half-page t have landed; the loads of the
// later half-pages t + 1 .. min(t + 2, H - 1) may stay in flight.
__device__ __forceinline__ void wait_group(int t, int H) {
    if (t + 2 < H) wait_vmcnt<2 * kDmaPerWave>();
    else if (t + 1 < H) wait_vmcnt<kDmaPerWave>();
    else wait_vmcnt<0>();
}

// Any of the four waves' restart flags at f[0..3] (one 16-byte LDS read).
__device__ __forceinline__ int flags_any(volatile __attribute__((address_space(3))) int *f) {
    const u32x4 v = *(volatile __attribute__((address_space(3))) u32x4 *)f;
    return (int)(v[0] | v[1] | v[2] | v[3]);
}

// Zeroes the accumulators with MFMAs (0 x 0 + 0), so they are born in the
// accumulator registers.
__device__ __forceinline__ void zero_acc16(f32x16 (&o)[16]) {
    u32x4 zw;
    asm volatile("v_mov_b32 %0, 0\n\tv_mov_b32 %1, 0\n\tv_mov_b32 %2, 0\n\tv_mov_b32 %3, 0"
                 : "=v"(zw[0]), "=v"(zw[1]), "=v"(zw[2]), "=v"(zw[3]));
    const bf16x8 zf = __builtin_bit_cast(bf16x8, zw);
#pragma unroll
    for (int dt = 0; dt < 16; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(zf, zf, (f32x16){}, 0, 0, 0);
}

// Stage a wave's O^T (unnormalised fp32, 16 dim tiles of 32 dims x 32 rows) in
// LDS as rows r0 .. r0 + 31 of [64][kXStride].  Lane holds row r0 + lane % 32
// and, in tile dt, dims 32 dt + 8 (i / 4) + 4 (lane / 32) + (i % 4).
__device__ __forceinline__ void stage_rows32(float *X, const f32x16 (&o)[16], int r0, int lane) {
    float *xrow = X + (r0 + (lane & 31)) * kXStride + 4 * (lane >> 5);
#pragma unroll
    for (int dt = 0; dt < 16; ++dt)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
            *(f32x4 *)(xrow + 32 * dt + 8 * qd) =
                (f32x4){o[dt][4 * qd], o[dt][4 * qd + 1], o[dt][4 * qd + 2], o[dt][4 * qd + 3]};
}

__global__ __launch_bounds__(kThreads, 1) void decode_rows128_kernel(
    const DecodeArgs a, const uint16_t *__restrict__ q, const unsigned char *__restrict__ kv,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seqlens,
    const int32_t *__restrict__ meta, const int32_t *__restrict__ split_base) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[kLdsBytes];
    lds_u8 *smem = (lds_u8 *)smem_raw;
    const int tid = threadIdx.x, lane = tid & 63;
    // wave index as a scalar (uniform branches and LDS offsets)
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h = lane >> 5;

    // blockIdx -> (part, row group), row groups of a part on one XCD
    const int lin = blockIdx.x;
    const int rest = lin >> 3;
    const int rg = rest % a.row_groups;
    const int part = (rest / a.row_groups) * 8 + (lin & 7);
    if (part >= a.num_parts) return;
    const int32_t *mrow = meta + part * kMetaInts;
    if (mrow[0] < 0) return;

    const unsigned ring0 = lds_addr(smem);
    volatile __attribute__((address_space(3))) int *flag_lds =
        (volatile __attribute__((address_space(3))) int *)(smem + kFlagOff);
    float *stat_lds = (float *)(smem_raw + kStatOff);
    float *X = (float *)smem_raw;  // output stage [64][kXStride], over the ring
    const int row0 = rg * kRows;
    const int row = row0 + 32 * w + l32;
    const int qi = row / a.h_q;
    const float c = a.scale_log2;  // > 0
    const float grow = kGrowLog2 / c;
    int kofs[4];
    halfpage::k_offsets(kofs, l32, h);
    int vofs[2][2];
    halfpage::v_offsets(vofs, lane, 0);

    for_each_segment(mrow, seqlens, split_base, block_table, a.bt_stride, [&](const Segment &sg) {
        int n_visible = a.causal ? sg.L - (a.s_q - 1 - qi) : sg.L;
        n_visible = n_visible > 0 ? n_visible : 0;
        const int n_visible_all = a.causal ? sg.L - (a.s_q - 1) : sg.L;  // every row sees these
        // Q^T operand for 32x32x16: lane holds dims 16 ks + 8 h .. +8 of its row
        bf16x8 qf[kDQk / 16];
        const uint16_t *qrow = q + ((int64_t)sg.b * a.M + row) * kDQk + 8 * h;
#pragma unroll
        for (int ks = 0; ks < kDQk / 16; ++ks) qf[ks] = *(const bf16x8 *)(qrow + 16 * ks);
#pragma unroll
        for (int ks = 0; ks < kDQk / 16; ++ks) asm volatile("" : : "v"(qf[ks]));
        for (int t = 0; t < kAhead && t < sg.H; ++t) issue_group(sg, kv, t, w, lane, ring0);

        f32x16 o[16];
        // Exponent reference per row (raw score units), fixed for a pass over
        // the segment; rows that have not seen a key yet adopt their first max
        // freely (their accumulators are zero).
        float m_seen = -INFINITY, m, lsum;
        bool again;
        do {  // one pass over the segment; repeated only after a restart
            m = m_seen;
            lsum = 0.f;
            again = false;
            zero_acc16(o);
            // Restart flags by step parity: in step t wave w writes slot
            // 4 (t % 2) + w, and every wave reads slot (t + 1) % 2 (written in
            // step t - 1) after the step's barrier, so no flag is read in the
            // step that writes it.
            if (lane == 0) {
                flag_lds[w] = 0;
                flag_lds[4 + w] = 0;
            }
            // page of the next half-page to load, looked up one step ahead
            int page_next = kAhead < sg.H ? page_of(sg, kAhead) : 0;
            for (int t = 0; t <= sg.H; ++t) {
                // half-page t + 3 goes to the slot half-page t - 1 used (every
                // wave is past it once this step's barrier is passed)
                const bool more = t + kAhead < sg.H;
                GroupDma dma;
                if (more) dma = group_dma(sg, kv, t + kAhead, page_next, w, lane, ring0);
                if (t + kAhead + 1 < sg.H) page_next = page_of(sg, t + kAhead + 1);
                if (t < sg.H) wait_group(t, sg.H);
                __syncthreads();
                // restart flags of step t - 1: one 16-byte read of the four
                // waves' flags
                if (__builtin_amdgcn_readfirstlane(flags_any(flag_lds + 4 * ((t + 1) & 1)))) {
                    again = true;  // restart with the larger references
                    break;
                }
                if (t == sg.H) break;
                const lds_u8 *S = smem + (t % kRing) * kHalfBytes;

                // ---- S^T = K . Q^T
                f32x16 sacc = {};
                constexpr int kPre = 8;  // K fragments in flight ahead of the MFMAs
                bf16x8 kf[kPre];
#pragma unroll
                for (int ks = 0; ks < kPre; ++ks) kf[ks] = halfpage::read_k(S, kofs, ks);
#pragma unroll
                for (int ks = 0; ks < kDQk / 16; ++ks) {
                    const bf16x8 cur = kf[ks % kPre];
                    const int kn = ks + kPre;
                    if (kn < kDQk / 16) kf[ks % kPre] = halfpage::read_k(S, kofs, kn);
                    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[ks], sacc, 0, 0, 0);
                }
                // keep kPre K reads in flight: one read after each MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, kPre, 0);
#pragma unroll
                for (int ks = 0; ks < kDQk / 16 - kPre; ++ks) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, kPre, 0);

                // ---- softmax of this wave's rows; lane holds tokens
                // 8 (i / 4) + 4 h + (i % 4) of the half-page for its row
                const int tok0 = sg.j0 * kPage + t * kHalf;
                float x[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) x[i] = sacc[i];
                if (tok0 + kHalf > n_visible_all) {  // the causal edge or the segment's end
                    const int tok_base = tok0 + 4 * h;
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        x[i] = (tok_base + 8 * (i >> 2) + (i & 3) < n_visible) ? x[i] : -INFINITY;
                }
                float mloc = x[0];
#pragma unroll
                for (int i = 1; i < 16; ++i) mloc = fmaxf(mloc, x[i]);
                mloc = max_xor32(mloc);
                m_seen = fmaxf(m_seen, mloc);
                if (m == -INFINITY) m = mloc;  // first keys of this row
                const bool overflow = mloc > m + grow;
                flag_lds[4 * (t & 1) + w] = __builtin_amdgcn_ballot_w64(overflow) != 0;
                const float mc = (m == -INFINITY) ? 0.f : m * c;
                float psum = 0.f;
                unsigned pk[8];
#pragma unroll
                for (int i = 0; i < 16; i += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], c, -mc));
                    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i + 1], c, -mc));
                    psum += p0 + p1;
                    pk[i >> 1] = pack_bf16(p0, p1);
                }
                lsum += psum;
                // P^T operand of k-step kk = tokens 16 kk .. 16 kk + 15
                const bf16x8 pf[2] = {__builtin_bit_cast(bf16x8, (u32x4){pk[0], pk[1], pk[2], pk[3]}),
                                      __builtin_bit_cast(bf16x8, (u32x4){pk[4], pk[5], pk[6], pk[7]})};

                // ---- O^T += V^T . P^T; the wave's loads of half-page t + 3
                // go out between the MFMAs
                constexpr int kVPre = 8;  // V fragments in flight ahead of the MFMAs
                bf16x8 vf[kVPre];
#pragma unroll
                for (int n = 0; n < kVPre; ++n) vf[n] = halfpage::read_v(S, vofs, n >> 4, n & 15);
#pragma unroll
                for (int n = 0; n < 32; ++n) {
                    const bf16x8 cur = vf[n % kVPre];
                    const int nn = n + kVPre;
                    if (nn < 32) vf[n % kVPre] = halfpage::read_v(S, vofs, nn >> 4, nn & 15);
                    o[n & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, pf[n >> 4], o[n & 15], 0, 0, 0);
                    if (more && n % 3 == 1 && n / 3 < kDmaPerWave) dma.issue(n / 3);
                }
            }
            if (again) {
                wait_vmcnt<0>();
                __syncthreads();  // every wave has left the pass; the ring is idle
                for (int t = 0; t < kAhead && t < sg.H; ++t) issue_group(sg, kv, t, w, lane, ring0);
            }
        } while (again);

        lsum += __shfl_xor(lsum, 32);
        if (h == 0) {
            stat_lds[32 * w + l32] = lsum;
            const float lse_val = lsum > 0.f ? (m * c + log2f(lsum)) * 0.69314718055994530942f : -INFINITY;
            if (sg.nsplit == 1)
                a.lse[(int64_t)sg.b * a.M + row] = lse_val;
            else
                a.lse_part[(int64_t)(split_base[sg.b] + sg.rank) * a.M + row] = lse_val;
        }
        // Output in two slabs of 64 rows through the idle ring: waves 0, 1
        // first, then waves 2, 3.
#pragma unroll
        for (int slab = 0; slab < 2; ++slab) {
            __syncthreads();  // ring (or the previous slab) free, row sums visible
            if ((w >> 1) == slab) stage_rows32(X, o, 32 * (w & 1), lane);
            __syncthreads();  // slab staged
            write_rows(a, sg, split_base, X, stat_lds + 64 * slab, row0 + 64 * slab, tid);
        }
        __syncthreads();  // LDS free for the next segment
    });
}

}  // namespace

hipError_t launch_decode_rows128(const DecodeArgs &a, hipStream_t stream) {
    const int groups8 = (a.num_parts + 7) / 8;
    const dim3 grid(groups8 * 8 * a.row_groups), block(kThreads);
    hipLaunchKernelGGL(decode_rows128_kernel, grid, block, 0, stream, a, a.q, a.kv, a.block_table,
                       a.seqlens, a.meta, a.split_base);
    return hipGetLastError();
}

}  // namespace mla
