// MLA decode attention for many query rows per request (s_q * h_q >= 32; 32
// rows run as one 64-row group with padding rows): gfx950 kernel with specialised waves.
//
// A work-group (4 waves, one per SIMD) owns one split-KV part and one group of
// 64 query rows.  It walks the part's pages in 32-token half-pages:
//   - waves 0, 1 ("score waves") each hold 32 query rows of Q in registers and
//     compute S^T (32 tokens x 32 rows) = K . Q^T on 32x32x16 bf16 MFMAs, then
//     the online softmax of their rows, and hand P (bf16) to the value waves
//     through LDS;
//   - waves 2, 3 ("value waves") each own 256 of the 512 output dims for all
//     64 rows and accumulate O^T (dims x rows) += V^T . P^T, one half-page
//     behind the score waves.  They also issue every direct-to-LDS load, so
//     the score waves never stall on the memory pipeline.
// Half-pages stream HBM -> LDS with direct-to-LDS loads into a 4-deep ring:
// during step t the score waves read half-page t, the value waves half-page
// t-1, and half-pages t+1, t+2 are in flight.  One work-group barrier per step.
//
// The half-page LDS layout and the operand addressing are in halfpage_bf16.h.
//
// Token-list mode (sparse decode, kList): each "request" is one query token's
// list of cache token ids; the score waves stage the ids of half-page t + 3 in
// LDS during step t, and the value waves load each listed row straight from
// its page, so the listed rows are read once, from the cache itself.
#include <math.h>

#include "common.h"
#include "device_util.h"
#include "halfpage_bf16.h"
#include "rows64.h"

namespace mla {

namespace {

using namespace rows64;

constexpr int kHalfBytes = halfpage::kBytes;  // 36864
constexpr int kDmaPerWave = kHalfBytes / 1024 / 2;  // 18 direct-to-LDS loads per value wave per step
constexpr int kPOff = kRing * kHalfBytes;         // P hand-off: 2 x (2 row tiles x 2 k-steps x 1 KB)
constexpr int kPBytes = 4096;
constexpr int kFlagOff = kPOff + 2 * kPBytes;     // restart flags of the two score waves
constexpr int kStatOff = kFlagOff + 64;           // final (m, l) per row
constexpr int kIdsOff = kStatOff + 2 * kRowsWG * 4;  // token-list mode: ids of kRing half-pages
constexpr int kLdsBytes = kIdsOff + kRing * kHalf * 4;

// Value wave v's share of a half-page: the 18 one-KB blocks (G, lam) with
// G = 2 v + g2, each one 128-byte line (lam = 0..8) of eight tokens.
struct HalfDma {
    const unsigned char *src[2];  // per g2
    unsigned dst;                 // LDS byte address of the half-page slot
    __device__ __forceinline__ void issue(int v, int k) const {  // k = 9 g2 + lam
        const int g2 = k / 9, lam = k % 9;
        dma16(src[g2] + 128 * lam, __builtin_amdgcn_readfirstlane(dst + (9 * (2 * v + g2) + lam) * 1024));
    }
};

// Value wave v's direct-to-LDS loads of half-page t of a segment: from its
// page, or (token-list mode) from the rows whose ids sit in LDS slot t % kRing.
template <bool kList>
__device__ __forceinline__ HalfDma half_dma(const Segment &sg, const unsigned char *kv, int t, int v,
                                            int lane, unsigned ring0, const lds_i32 *ids) {
    HalfDma d;
    if constexpr (kList) {
        const lds_i32 *id = ids + (t % kRing) * kHalf;
        const int tok_last = sg.tok_last(t);
        d.src[0] = halfpage::dma_row_ids(kv, id, tok_last, 2 * v, lane);
        d.src[1] = halfpage::dma_row_ids(kv, id, tok_last, 2 * v + 1, lane);
    } else {
        const int j = sg.j0 + (t >> 1);
        const int tok_last = (j == sg.npages - 1) ? (sg.L - 1 - j * kPage) : (kPage - 1);
        const int64_t phys = sg.bt[j];
        d.src[0] = halfpage::dma_row(kv, phys, (t & 1) * kHalf, tok_last, 2 * v, lane);
        d.src[1] = halfpage::dma_row(kv, phys, (t & 1) * kHalf, tok_last, 2 * v + 1, lane);
    }
    d.dst = ring0 + (t % kRing) * kHalfBytes;
    return d;
}

template <bool kList>
__device__ __forceinline__ void issue_step(const Segment &sg, const unsigned char *kv, int t, int v,
                                           int lane, unsigned ring0, const lds_i32 *ids) {
    const HalfDma d = half_dma<kList>(sg, kv, t, v, lane, ring0, ids);
#pragma unroll
    for (int k = 0; k < kDmaPerWave; ++k) d.issue(v, k);
}

template <bool kList>
__global__ __launch_bounds__(kThreads, 1) void decode_rows64_kernel(
    const DecodeArgs a, const uint16_t *__restrict__ q, const unsigned char *__restrict__ kv,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seqlens,
    const int32_t *__restrict__ meta, const int32_t *__restrict__ split_base) {
    // The read-only tables arrive as separate restrict-qualified arguments so
    // that their uniform reads compile to scalar loads.
    __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[kLdsBytes];
    lds_u8 *smem = (lds_u8 *)smem_raw;
    const int tid = threadIdx.x, lane = tid & 63;
    // wave index as a scalar: the role branches below hold barriers and must be
    // compiled as uniform branches
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
    lds_i32 *ids_lds = (lds_i32 *)(smem + kIdsOff);
    float *X = (float *)smem_raw;  // output stage [64][kXStride], over the ring
    const int row0 = rg * kRowsWG;

    if (w < 2) {
        // ================= score waves: rows row0 + 32 w + (lane % 32)
        // rows past M (M = 32 pads one 64-row group) repeat the last row's
        // query and visibility; their results are not written
        const int row = row0 + 32 * w + l32;
        const int row_q = row < a.M ? row : a.M - 1;
        const int qi = row_q / a.h_q;
        const float c = a.scale_log2;  // > 0
        const float grow = kGrowLog2 / c;
        int kofs[4];  // K operand of k-step ks for this lane
        halfpage::k_offsets(kofs, l32, h);
        for_each_segment(mrow, seqlens, split_base, block_table, a.bt_stride, [&](const Segment &sg) {
            if constexpr (kList) {
                stage_first_ids(ids_lds, sg, l32, h);
                __syncthreads();  // the value waves load half-pages 0 .. 2
            }
            int n_visible = a.causal ? sg.L - (a.s_q - 1 - qi) : sg.L;
            n_visible = n_visible > 0 ? n_visible : 0;
            const int n_visible_all = a.causal ? sg.L - (a.s_q - 1) : sg.L;  // every row sees these
            // Q^T operand for 32x32x16: lane holds dims 16 ks + 8 h .. +8 of its row
            bf16x8 qf[kDQk / 16];
            const uint16_t *qrow = q + ((int64_t)sg.b * a.M + row_q) * kDQk + 8 * h;
#pragma unroll
            for (int ks = 0; ks < kDQk / 16; ++ks) qf[ks] = *(const bf16x8 *)(qrow + 16 * ks);
#pragma unroll
            for (int ks = 0; ks < kDQk / 16; ++ks) asm volatile("" : : "v"(qf[ks]));
            // Exponent reference per row (raw score units).  It is fixed for a
            // pass over the segment, so the value waves never rescale their
            // accumulators: a row whose running max exceeds it by more than
            // kGrowLog2 (after scaling) makes the whole work-group restart the
            // segment with the larger reference (rows that have not seen a key
            // yet adopt their first max freely, their accumulators being zero).
            // lsum: sum of the fp32 weights (for the lse); wsum: sum of the
            // weights as rounded to bf16 for the value product, which
            // normalises the output (the effective weights then sum to 1, so
            // a row dominated by one key returns that key's value exactly)
            float m_seen = -INFINITY, m, lsum, wsum;
            bool again;
            do {  // one pass over the segment; repeated only after a restart
                m = m_seen;
                lsum = 0.f;
                wsum = 0.f;
                again = false;
                // Restart flags by step parity: in step t a score wave writes slot
                // t % 2, and every wave reads slot (t + 1) % 2 (written in step
                // t - 1) right after the step's barrier, so no flag is read in
                // the step that writes it.
                if (lane == 0) {
                    flag_lds[w] = 0;
                    flag_lds[2 + w] = 0;
                }
                for (int t = 0; t <= sg.H; ++t) {
                    __syncthreads();
                    // restart flags: read now, acted on after this step's MFMAs
                    // (the value waves act on them at once; work done here in
                    // the meantime is discarded)
                    const int fr = 2 * ((t + 1) & 1);
                    int f0 = flag_lds[fr], f1 = flag_lds[fr + 1];
                    if (t == sg.H) {
                        again = __builtin_amdgcn_readfirstlane(f0 | f1) != 0;
                        break;
                    }
                    // token-list mode: ids of half-page t + 3, into LDS at the
                    // end of this step (the value waves issue its loads in
                    // step t + 1)
                    const bool stage = kList && t + 3 < sg.H;
                    int id_next = 0;
                    if (stage) id_next = list_ids(sg, t + 3)[l32];
                    const lds_u8 *S = smem + (t % kRing) * kHalfBytes;
                    f32x16 sacc = {};
                    constexpr int kPre = 8;  // K fragments in flight ahead of the MFMAs
                    bf16x8 kf[kPre];
#pragma unroll
                    for (int ks = 0; ks < kPre; ++ks)
                        kf[ks] = halfpage::read_k(S, kofs, ks);
#pragma unroll
                    for (int ks = 0; ks < kDQk / 16; ++ks) {
                        const bf16x8 cur = kf[ks % kPre];
                        const int kn = ks + kPre;
                        if (kn < kDQk / 16)
                            kf[ks % kPre] = halfpage::read_k(S, kofs, kn);
                        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[ks], sacc, 0, 0, 0);
                    }
                    // keep kPre K reads in flight: kPre reads, then one MFMA per read
                    __builtin_amdgcn_sched_group_barrier(0x100, kPre, 0);
#pragma unroll
                    for (int ks = 0; ks < kDQk / 16 - kPre; ++ks) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, kPre, 0);
                    asm volatile("" : "+v"(f0), "+v"(f1));  // keeps the flag test behind the MFMAs
                    if (__builtin_amdgcn_readfirstlane(f0 | f1)) {  // restart with the larger reference
                        again = true;
                        break;
                    }
                    // lane holds tokens 8 (i/4) + 4 h + (i%4) of the half-page for its row
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
                    flag_lds[2 * (t & 1) + w] = __builtin_amdgcn_ballot_w64(overflow) != 0;  // same value from every lane
                    const float mc = (m == -INFINITY) ? 0.f : m * c;
                    float psum = 0.f, rsum = 0.f;
                    unsigned pk[8];
#pragma unroll
                    for (int i = 0; i < 16; i += 2) {
                        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], c, -mc));
                        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i + 1], c, -mc));
                        psum += p0 + p1;
                        pk[i >> 1] = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){p0, p1}, bf16x2));
                        rsum = add_bf16_pair(pk[i >> 1], rsum);
                    }
                    lsum += psum;
                    wsum += rsum;
                    // P^T operand blocks: (row tile w, k-step kk) -> 1 KB at P + (2 w + kk) KB
                    lds_u8 *P = smem + kPOff + (t & 1) * kPBytes;
                    *(u32x4 __attribute__((address_space(3))) *)(P + (2 * w + 0) * 1024 + lane * 16) =
                        (u32x4){pk[0], pk[1], pk[2], pk[3]};
                    *(u32x4 __attribute__((address_space(3))) *)(P + (2 * w + 1) * 1024 + lane * 16) =
                        (u32x4){pk[4], pk[5], pk[6], pk[7]};
                    if (stage && h == 0) ids_lds[((t + 3) % kRing) * kHalf + l32] = id_next;
                }
                if (again) {
                    if constexpr (kList) stage_first_ids(ids_lds, sg, l32, h);
                    wait_vmcnt<0>();
                    __syncthreads();
                }
            } while (again);
            lsum += __shfl_xor(lsum, 32);
            wsum += __shfl_xor(wsum, 32);
            if (h == 0) {
                stat_lds[kRowsWG + 32 * w + l32] = wsum;
                const float lse_val =
                    lsum > 0.f ? (m * c + log2f(lsum)) * 0.69314718055994530942f : -INFINITY;
                if (row >= a.M) {
                } else if (sg.nsplit == 1) {
                    a.lse[(int64_t)sg.b * a.M + row] = lse_val;
                } else {
                    a.lse_part[(int64_t)(split_base[sg.b] + sg.rank) * a.M + row] = lse_val;
                }
            }
            __syncthreads();  // stats visible to the value waves
            __syncthreads();  // value waves have staged the output
            write_rows(a, sg, split_base, X, stat_lds + kRowsWG, row0, tid);
            __syncthreads();  // LDS free for the next segment
        });
    } else {
        // ================= value waves: dims d0 .. d0 + 255 for all 64 rows
        const int v = w - 2, d0 = v * 256;
        int vofs[2][2];  // transposed V reads of this wave's 256 dims
        halfpage::v_offsets(vofs, lane, 4 * v);
        for_each_segment(mrow, seqlens, split_base, block_table, a.bt_stride, [&](const Segment &sg) {
            if constexpr (kList) __syncthreads();  // ids of half-pages 0 .. 2 staged
            issue_step<kList>(sg, kv, 0, v, lane, ring0, ids_lds);
            if (sg.H > 1) issue_step<kList>(sg, kv, 1, v, lane, ring0, ids_lds);
            f32x16 o[2][8];
            bool again;
            do {  // one pass over the segment; repeated only after a restart
                zero_acc(o);
                again = false;
                for (int t = 0; t <= sg.H; ++t) {
                    wait_own_dma<kDmaPerWave>(t + 1 < sg.H);
                    __syncthreads();
                    const int fr = 2 * ((t + 1) & 1);
                    if (__builtin_amdgcn_readfirstlane(flag_lds[fr] | flag_lds[fr + 1])) {  // the score waves restart the segment
                        again = true;
                        break;
                    }
                    const bool more = t + 2 < sg.H;
                    if (t == 0) {
                        if (more) issue_step<kList>(sg, kv, t + 2, v, lane, ring0, ids_lds);
                        continue;
                    }
                    // Half-page t + 2 goes to the slot half-page t - 2 used; its
                    // loads are spread over this step's MFMAs (one per MFMA
                    // pair) so that no load waits for the memory pipeline.
                    const int tp = t - 1;  // half-page processed this step
                    const lds_u8 *V = smem + (tp % kRing) * kHalfBytes;
                    const lds_u8 *P = smem + kPOff + (tp & 1) * kPBytes;
                    HalfDma dma;
                    if (more) dma = half_dma<kList>(sg, kv, t + 2, v, lane, ring0, ids_lds);
                    auto read_v = [&](int kk, int dt) { return halfpage::read_v(V, vofs, kk, dt); };
                    auto read_p = [&](int blk) {
                        return *(const bf16x8 __attribute__((address_space(3))) *)(P + blk * 1024 + lane * 16);
                    };
                    // k-step 0: all its operands first; k-step 1's operands are
                    // read between k-step 0's MFMAs, one DMA after each MFMA pair
                    bf16x8 v0[8], v1[8];
                    const bf16x8 p00 = read_p(0), p01 = read_p(2);
#pragma unroll
                    for (int dt = 0; dt < 8; ++dt) v0[dt] = read_v(0, dt);
                    const bf16x8 p10 = read_p(1), p11 = read_p(3);
#pragma unroll
                    for (int dt = 0; dt < 8; ++dt) {
                        o[0][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0[dt], p00, o[0][dt], 0, 0, 0);
                        o[1][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0[dt], p01, o[1][dt], 0, 0, 0);
                        v1[dt] = read_v(1, dt);
                        if (more) dma.issue(v, dt);
                    }
#pragma unroll
                    for (int dt = 0; dt < 8; ++dt) {
                        o[0][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1[dt], p10, o[0][dt], 0, 0, 0);
                        o[1][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1[dt], p11, o[1][dt], 0, 0, 0);
                        if (more) dma.issue(v, 8 + dt);
                    }
                    if (more) {
#pragma unroll
                        for (int k = 16; k < kDmaPerWave; ++k) dma.issue(v, k);
                    }
                }
                if (again) {
                    wait_vmcnt<0>();
                    __syncthreads();
                    issue_step<kList>(sg, kv, 0, v, lane, ring0, ids_lds);
                    if (sg.H > 1) issue_step<kList>(sg, kv, 1, v, lane, ring0, ids_lds);
                }
            } while (again);
            __syncthreads();  // score waves' final stats visible
            stage_output(X, o, d0, lane);  // the ring is free
            __syncthreads();  // staged output complete
            write_rows(a, sg, split_base, X, stat_lds + kRowsWG, row0, tid);
            __syncthreads();  // LDS free for the next segment
        });
    }
}

}  // namespace

hipError_t launch_decode_rows64(const DecodeArgs &a, hipStream_t stream) {
    const int groups8 = (a.num_parts + 7) / 8;
    const dim3 grid(groups8 * 8 * a.row_groups), block(kThreads);
    if (a.token_list)
        hipLaunchKernelGGL(decode_rows64_kernel<true>, grid, block, 0, stream, a, a.q, a.kv,
                           a.block_table, a.seqlens, a.meta, a.split_base);
    else
        hipLaunchKernelGGL(decode_rows64_kernel<false>, grid, block, 0, stream, a, a.q, a.kv,
                           a.block_table, a.seqlens, a.meta, a.split_base);
    return hipGetLastError();
}

}  // namespace mla
