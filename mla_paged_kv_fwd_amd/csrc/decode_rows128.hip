// MLA decode attention for 128 or more query rows per request (s_q * h_q in
// {128, 256, 512}), bf16 cache: gfx950 kernel, 128 query rows per work-group.
//
// A work-group of 4 waves (one per SIMD) owns one split-KV part and one group
// of 128 query rows, and walks the part in 32-token steps (half-pages).  Every
// wave does the same two jobs:
//   - scores: it holds Q for 32 of the rows in registers and computes
//     S^T (32 tokens x 32 rows) = K . Q^T on 32x32x16 bf16 MFMAs, then the
//     online softmax of those rows; the bf16 weights P go to LDS;
//   - values: it owns 128 of the 512 output dims for all 128 rows and
//     accumulates O^T (128 dims x 128 rows, 256 accumulator registers)
//     += V^T . P^T over the previous step's weights of every row.
// So each cached value element is read from LDS once per work-group, and a
// half-page brought into LDS serves all 128 rows.  Within a step a wave runs
// the QK MFMAs of step t, then the PV MFMAs of step t - 1 with the softmax of
// step t issued between them, so the matrix unit keeps working while the
// softmax runs.  One work-group barrier per step.
//
// LDS ring: seven 16-token units of 18 KB.  Unit u (tokens 16 u .. 16 u + 15
// of the segment) sits in slot u % 7.  In step t the QK reads units 2t, 2t+1,
// the PV reads 2t-2, 2t-1, and the loads of units 2t+3 and 2t+4 are issued
// (waves 0, 1 and 2, 3 respectively; each wave one group of 8 tokens of its
// unit), into the slots units 2t-4 and 2t-3 left at the step's barrier.
// Unit layout: token tau (0..15), 16-byte chunk c (0..71) of its 1152-byte
// row sits at byte 1024 (9 (tau / 8) + c / 8) + 128 (tau % 8) +
// 16 ((c % 8) ^ swz(tau)), swz(tau) = 4 bit1(tau) + 2 bit2(tau) + bit3(tau):
// each direct-to-LDS load reads eight whole 128-byte lines, and the K reads
// (ds_read_b128) and transposed V reads (ds_read_b64_tr_b16) are free of bank
// conflicts (the same layout as a token group of the 64-row kernel's
// half-page).
//
// Softmax reference and restarts as in the 64-row kernels: a row's exponent
// reference is fixed for a pass over a request segment, so no accumulator is
// ever rescaled; a row whose running max passes it by more than kGrowLog2
// (log2 units) raises a flag and the work-group re-runs the segment with the
// larger reference.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "device_util.h"
#include "rows64.h"

namespace mla {

namespace {

using rows64::f32x16;
using rows64::kGrowLog2;
using rows64::kXStride;
using rows64::Segment;

constexpr int kThreads = 256;
constexpr int kRowsWG = 128;
constexpr int kStepTok = 32;
constexpr int kUnitBytes = 16 * kTokBytesBf16;  // 18432
constexpr int kUnits = 7;
constexpr int kPOff = kUnits * kUnitBytes;      // 129024
constexpr int kPBytes = 8192;                   // P^T: 4 row tiles x 2 k-steps x 1 KB
constexpr int kFlagOff = kPOff + 2 * kPBytes;   // 145408: restart flags [2][4]
constexpr int kStatOff = kFlagOff + 64;         // row weight sums [128]
constexpr int kLdsBytes = kStatOff + kRowsWG * 4;
static_assert(64 * kXStride * 4 <= kFlagOff, "the output stage fits over the ring and P");

__device__ __forceinline__ int swz(int tau) {
    return 4 * ((tau >> 1) & 1) + 2 * ((tau >> 2) & 1) + ((tau >> 3) & 1);
}

__device__ __forceinline__ unsigned unit_slot(int u) { return (unsigned)(u % kUnits) * kUnitBytes; }

// Register classes: the PV MFMAs are builtins, whose accumulators the
// compiler keeps in the 256 accumulator registers (O^T), and the QK MFMAs are
// asm with the score accumulator S^T in VGPRs beside Q^T.  The QK asm is
// volatile, which keeps the K fragment reads where the source puts them, a
// fixed distance ahead of their MFMAs.  A dependent chain on one accumulator
// needs no wait states between its MFMAs; the first MFMA of a chain adds to
// an inline zero, so no VALU-written accumulator is read; qk_done() covers
// the MFMA-write to VALU-read distance before the scores are read (the
// compiler does not see inside the asm).
__device__ __forceinline__ void qk_first(f32x16 &s, const bf16x8 &k, const bf16x8 &qv) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(k), "v"(qv));
}
__device__ __forceinline__ void qk_next(f32x16 &s, const bf16x8 &k, const bf16x8 &qv) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(k), "v"(qv));
}
__device__ __forceinline__ void qk_done(f32x16 &s) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s));
}
// Direct-to-LDS load without a memory clobber: the LDS slot it fills is read
// only after the step barrier that follows the wait for it (both of which
// order every memory access), so the K and V reads of the current step may
// move across it.
__device__ __forceinline__ void dma16_nc(const void *g, unsigned lds_byte_addr) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(lds_byte_addr) : "m0");
}

// Source of lane `lane`'s part of the loads of token group g (0, 1) of unit u
// of a segment: token 8 g + lane / 8 of the unit (clamped to the segment's
// last token), and within each 128-byte line the chunk whose swizzled slot is
// lane % 8.  Line lam of the group is at +128 lam and lands in the unit's
// 1 KB block 9 g + lam.
__device__ __forceinline__ const unsigned char *unit_src(const Segment &sg, const unsigned char *kv,
                                                         int u, int g, int lane) {
    const int a = lane >> 3, b = lane & 7;
    const int tau = 8 * g + a;
    const int j = sg.j0 + (u >> 2);
    const int tok_last = (j == sg.npages - 1) ? (sg.L - 1 - j * kPage) : (kPage - 1);
    int t = 16 * (u & 3) + tau;
    t = t < tok_last ? t : tok_last;
    const int64_t phys = sg.bt[j];
    return kv + (phys * kPage + t) * kTokBytesBf16 + 16 * (b ^ swz(tau));
}

// The 9 direct-to-LDS loads of token group g of unit u.
__device__ __forceinline__ void issue_group(const unsigned char *src, unsigned ring0, int u, int g) {
    const unsigned dst = ring0 + unit_slot(u) + 9216 * g;
#pragma unroll
    for (int lam = 0; lam < 9; ++lam)
        dma16_nc(src + 128 * lam, __builtin_amdgcn_readfirstlane(dst + 1024 * lam));
}

// Zeroes the accumulators with MFMAs (0 x 0 + 0), so they are born in the
// accumulator registers.  Each tile gets its own zero operand from an asm
// statement: identical MFMAs would be merged into one whose result is then
// copied into the other tiles.
__device__ __forceinline__ void zero_acc16(f32x16 (&o)[4][4]) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            u32x4 zw;
            asm volatile("v_mov_b32 %0, 0\n\tv_mov_b32 %1, 0\n\tv_mov_b32 %2, 0\n\tv_mov_b32 %3, 0"
                         : "=v"(zw[0]), "=v"(zw[1]), "=v"(zw[2]), "=v"(zw[3]));
            o[r][d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, zw),
                                                               __builtin_bit_cast(bf16x8, zw),
                                                               (f32x16){}, 0, 0, 0);
        }
}

__global__ __launch_bounds__(kThreads, 1) void decode_rows128_kernel(
    const DecodeArgs a, const uint16_t *__restrict__ q, const unsigned char *__restrict__ kv,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seqlens,
    const int32_t *__restrict__ meta, const int32_t *__restrict__ split_base) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[kLdsBytes];
    lds_u8 *smem = (lds_u8 *)smem_raw;
    const int tid = threadIdx.x, lane = tid & 63;
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
    float *X = (float *)smem_raw;  // output stage [64][kXStride], over the ring and P
    const int row0 = rg * kRowsWG;

    // scores: rows row0 + 32 w + l32
    const int row = row0 + 32 * w + l32;
    const int qi = row / a.h_q;
    const float c = a.scale_log2;  // > 0
    const float grow = kGrowLog2 / c;
    // K operand of k-step ks (A: lane = token l32 of the step, 8 dims
    // 16 ks + 8 h ..): byte kofs[ks % 4] + 1024 (ks / 4) of the token's unit
    int kofs[4];
    {
        const int tau = l32 & 15, y = h ^ swz(tau);
#pragma unroll
        for (int k3 = 0; k3 < 4; ++k3)
            kofs[k3] = 9216 * (tau >> 3) + 128 * (tau & 7) + 16 * ((2 * k3) ^ y);
    }
    // values: dims 128 w .. 128 w + 127 = lines 2 w, 2 w + 1 of a row.
    // Transposed V reads, 32x32x16 A operand of k-step kk (the 16 tokens of
    // unit 2 (t-1) + kk), dim tile dt (32 dims): 16-lane group gq = lane / 16
    // covers dims 32 dt + 16 (gq & 1) + (lane % 16); its lanes point at token
    // 8 sel + 4 (gq >> 1) + (lane % 16) / 4 of the unit, 8 bytes at dim
    // offset 4 (lane % 4), for sel = 0 (first read) and 1 (second read).  The
    // token order inside a k-step matches the S^T accumulator layout of the
    // 32x32 MFMA (lane = row, register i = token 8 (i / 4) + 4 (lane / 32) +
    // i % 4), so P^T blocks written straight from that accumulator are the B
    // operand.  Byte offset in the unit: vofs[sel][dt & 1] + 1024 (dt / 2).
    int vofs[2][2];
    {
        const int gq = lane >> 4, i16 = lane & 15;
        const int ta = 4 * (gq >> 1) + (i16 >> 2);
        const int y2 = 2 * (gq & 1) + ((i16 & 3) >> 1);
#pragma unroll
        for (int sel = 0; sel < 2; ++sel)
#pragma unroll
            for (int d1 = 0; d1 < 2; ++d1)
                vofs[sel][d1] = 9216 * sel + 1024 * (2 * w) + 128 * ta +
                                16 * ((4 * d1) ^ y2 ^ swz(8 * sel + ta)) + 8 * (i16 & 1);
    }
    // this wave's loads in step t: token group w & 1 of unit 2 t + 3 + (w >> 1)
    const int g_load = w & 1, u_off = 3 + (w >> 1);

    rows64::for_each_segment(mrow, seqlens, split_base, block_table, a.bt_stride, [&](const Segment &sg) {
        const int last_unit = 2 * sg.H - 1;
        int n_visible = a.causal ? sg.L - (a.s_q - 1 - qi) : sg.L;
        n_visible = n_visible > 0 ? n_visible : 0;
        const int n_visible_all = a.causal ? sg.L - (a.s_q - 1) : sg.L;  // every row sees these
        // Q^T operand for 32x32x16: lane holds dims 16 ks + 8 h .. +8 of its row
        bf16x8 qf[kDQk / 16];
        {
            const uint16_t *qrow = q + ((int64_t)sg.b * a.M + row) * kDQk + 8 * h;
#pragma unroll
            for (int ks = 0; ks < kDQk / 16; ++ks) qf[ks] = *(const bf16x8 *)(qrow + 16 * ks);
        }
        // Loads of unit u, group g_load.  Units past the segment's last one
        // re-read the last one (from L2) into their slot, which no step reads:
        // every step issues the same loads, so the step code has no branches.
        auto unit_load_src = [&](int u) {
            return unit_src(sg, kv, u < last_unit ? u : last_unit, g_load, lane);
        };
        float m_seen = -INFINITY, m, lsum, wsum;
        f32x16 o[4][4];
        bool again;
        // One step: wait for the units this step reads, barrier, restart
        // check, then QK(t) (kQK) and PV(t-1) with the softmax of step t
        // (kPV).  Returns true when the work-group must restart the segment.
        auto step = [&](int t, auto qk_tag, auto pv_tag) -> bool {
            constexpr bool kQK = decltype(qk_tag)::value, kPV = decltype(pv_tag)::value;
            // own loads of units <= 2t+1 complete: waves 0, 1 issued unit 2t+1
            // last (step t-1); waves 2, 3 issued 2t (step t-2), then 2t+2
            if (w < 2) wait_vmcnt<0>(); else wait_vmcnt<9>();
            __syncthreads();
            // restart flags of step t - 1 (one 16-byte read), acted on after
            // this step's QK MFMAs are issued; work done here in the meantime
            // is discarded
            const u32x4 fl = *(const u32x4 __attribute__((address_space(3))) *)(smem + kFlagOff + 16 * ((t + 1) & 1));
            f32x16 sacc;
            if constexpr (kQK) {
                // ---------------- QK(t), with this step's loads between the MFMAs
                const lds_u8 *S = smem + (l32 < 16 ? unit_slot(2 * t) : unit_slot(2 * t + 1));
                const int u_ld = 2 * t + u_off;
                const unsigned char *src = unit_load_src(u_ld);
                const unsigned dst = ring0 + unit_slot(u_ld) + 9216 * g_load;
                auto read_k = [&](int ks) {
                    return *(const bf16x8 __attribute__((address_space(3))) *)(S + kofs[ks & 3] + 1024 * (ks >> 2));
                };
                // K fragments kPre k-steps ahead of their MFMAs; this step's
                // loads after every fourth MFMA from the first one on (issued
                // in one burst they stall the wave longer)
                constexpr int kPre = 4;
                bf16x8 kf[kDQk / 16];
#pragma unroll
                for (int ks = 0; ks < kPre; ++ks) kf[ks] = read_k(ks);
#pragma unroll
                for (int ks = 0; ks < kDQk / 16; ++ks) {
                    if (ks + kPre < kDQk / 16) kf[ks + kPre] = read_k(ks + kPre);
                    if (ks == 0) qk_first(sacc, kf[ks], qf[ks]); else qk_next(sacc, kf[ks], qf[ks]);
                    if ((ks & 3) == 0)
                        dma16_nc(src + 128 * (ks >> 2), __builtin_amdgcn_readfirstlane(dst + 1024 * (ks >> 2)));
                }
                qk_done(sacc);
            }
            if (__builtin_amdgcn_readfirstlane(fl[0] | fl[1] | fl[2] | fl[3])) return true;
            float x[16];
            if constexpr (kQK) {
#pragma unroll
                for (int i = 0; i < 16; ++i) x[i] = sacc[i];
                const int tok0 = sg.j0 * kPage + t * kStepTok;
                if (tok0 + kStepTok > n_visible_all) {  // the causal edge or the segment's end
                    const int tok_base = tok0 + 4 * h;
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        x[i] = (tok_base + 8 * (i >> 2) + (i & 3) < n_visible) ? x[i] : -INFINITY;
                }
            }
            if constexpr (kPV) {
                // ---------------- PV(t-1)
                const int tp = t - 1;
                const lds_u8 *V0 = smem + unit_slot(2 * tp), *V1 = smem + unit_slot(2 * tp + 1);
                const lds_u8 *P = smem + kPOff + (tp & 1) * kPBytes + lane * 16;
                auto read_v = [&](int kk, int dt) {
                    const lds_u8 *V = (kk ? V1 : V0) + 1024 * (dt >> 1);
                    const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (i16x4 __attribute__((address_space(3))) *)(V + vofs[0][dt & 1]));
                    const i16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (i16x4 __attribute__((address_space(3))) *)(V + vofs[1][dt & 1]));
                    const i16x8 v8 = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
                    return __builtin_bit_cast(bf16x8, v8);
                };
                auto read_p = [&](int kk, int rt) {
                    return *(const bf16x8 __attribute__((address_space(3))) *)(P + (2 * rt + kk) * 1024);
                };
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    bf16x8 pf[4];
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt) pf[rt] = read_p(kk, rt);
                    bf16x8 vf[4];
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) vf[dt] = read_v(kk, dt);
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                        for (int rt = 0; rt < 4; ++rt)
                            o[rt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[dt], pf[rt], o[rt][dt], 0, 0, 0);
                }
            }
            if constexpr (kQK) {
                // ---------------- softmax of step t: lane holds tokens
                // 8 (i/4) + 4 h + (i%4) of the step for its row
                float mloc = x[0];
#pragma unroll
                for (int i = 1; i < 16; ++i) mloc = fmaxf(mloc, x[i]);
                mloc = rows64::max_xor32(mloc);
                m_seen = fmaxf(m_seen, mloc);
                if (m == -INFINITY) m = mloc;  // first keys of this row
                const int ovf = mloc > m + grow;
                const float mc = (m == -INFINITY) ? 0.f : m * c;
                float psum = 0.f, rsum = 0.f;
                unsigned pk[8];
#pragma unroll
                for (int i = 0; i < 16; i += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], c, -mc));
                    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i + 1], c, -mc));
                    psum += p0 + p1;
                    pk[i >> 1] = rows64::pack_bf16(p0, p1);
                    rsum = add_bf16_pair(pk[i >> 1], rsum);
                }
                lsum += psum;
                wsum += rsum;
                // P^T operand blocks: (row tile w, k-step kk) -> 1 KB at P + (2 w + kk) KB
                lds_u8 *Pw = smem + kPOff + (t & 1) * kPBytes + (2 * w) * 1024 + lane * 16;
                *(u32x4 __attribute__((address_space(3))) *)(Pw) = (u32x4){pk[0], pk[1], pk[2], pk[3]};
                *(u32x4 __attribute__((address_space(3))) *)(Pw + 1024) = (u32x4){pk[4], pk[5], pk[6], pk[7]};
                const int any = __builtin_amdgcn_ballot_w64(ovf) != 0;
                if (lane == 0) flag_lds[4 * (t & 1) + w] = any;
            }
            if constexpr (kQK && kPV) {
                // the softmax's VALU work between the PV MFMAs: each k-step's
                // operand reads, then its 16 MFMAs with three VALU
                // instructions after each
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 12, 1);
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                        __builtin_amdgcn_sched_group_barrier(0x002, 3, 1);
                    }
                }
            }
            return false;
        };
        using yes = std::integral_constant<bool, true>;
        using no = std::integral_constant<bool, false>;
        do {  // one pass over the segment; repeated only after a restart
            m = m_seen;
            lsum = 0.f;
            wsum = 0.f;
            // Restart flags by step parity: in step t wave w writes slot
            // [t % 2][w]; every wave reads slot (t + 1) % 2 (written in step
            // t - 1) right after the step's barrier.
            if (lane == 0) {
                flag_lds[w] = 0;
                flag_lds[4 + w] = 0;
            }
            // the loads of "steps -2 and -1": units 0, 1, 2 (waves 2, 3 load
            // unit 0, then every wave its unit of step -1)
            if (w >= 2) issue_group(unit_load_src(0), ring0, 0, g_load);
            issue_group(unit_load_src(u_off - 2), ring0, u_off - 2, g_load);
            // Q arrives together with the first units; marking it used here
            // also keeps its loads out of the step loop
#pragma unroll
            for (int ks = 0; ks < kDQk / 16; ++ks) asm volatile("" : : "v"(qf[ks]));
            again = step(0, yes{}, no{});
            zero_acc16(o);  // here rather than earlier: O then stays in the loop's registers
            for (int t = 1; t < sg.H && !again; ++t) again = step(t, yes{}, yes{});
            if (!again) again = step(sg.H, no{}, yes{});
            wait_vmcnt<0>();  // the loads past the last unit
            __syncthreads();
        } while (again);
        // ---------------- epilogue: lse, weight sums, output
        lsum += __shfl_xor(lsum, 32);
        wsum += __shfl_xor(wsum, 32);
        if (h == 0) {
            stat_lds[32 * w + l32] = wsum;
            const float lse_val =
                lsum > 0.f ? (m * c + log2f(lsum)) * 0.69314718055994530942f : -INFINITY;
            if (sg.nsplit == 1)
                a.lse[(int64_t)sg.b * a.M + row] = lse_val;
            else
                a.lse_part[(int64_t)(split_base[sg.b] + sg.rank) * a.M + row] = lse_val;
        }
        __syncthreads();  // weight sums visible
#pragma unroll
        for (int hr = 0; hr < 2; ++hr) {
            // stage rows 64 hr .. 64 hr + 63 (row tiles 2 hr, 2 hr + 1) of this
            // wave's 128 dims: lane holds row 32 r + l32 and dims 128 w + 32 dt +
            // 8 (i / 4) + 4 h + (i % 4)
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2) {
                float *xrow = X + (32 * r2 + l32) * kXStride + 128 * w + 4 * h;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int qd = 0; qd < 4; ++qd) {
                        const f32x16 &acc = o[2 * hr + r2][dt];
                        *(f32x4 *)(xrow + 32 * dt + 8 * qd) =
                            (f32x4){acc[4 * qd], acc[4 * qd + 1], acc[4 * qd + 2], acc[4 * qd + 3]};
                    }
            }
            __syncthreads();
            rows64::write_rows(a, sg, split_base, X, stat_lds + 64 * hr, row0 + 64 * hr, tid);
            __syncthreads();
        }
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
