// MLA decode attention over an FP8 latent cache for many query rows per
// request (s_q * h_q >= 32, 32 rows padded to one 64-row group): gfx950 kernel with specialised waves.
//
// Cache record (656 bytes per token): 512 OCP E4M3FN codes of the latent
// dims, four little-endian fp32 scales (one per 128-dim tile), 64 bf16 RoPE
// dims.  The dequantised key is code * scale[dim / 128].
//
// Work split as in the bf16 64-row kernel: a work-group of 4 waves owns one
// split part and 64 query rows, walking the part in 32-token half-pages;
// waves 0, 1 score 32 rows each, waves 2, 3 accumulate 256 output dims each
// for all 64 rows, one half-page behind, and issue all loads.
//
// Dequantisation happens in registers, exactly:
//   - K fragments (16 codes of one token, two k-steps) are read with
//     ds_read_b128 and turned into bf16 with v_cvt_scalef32_pk_bf16_fp8 at
//     scale 1 (every E4M3FN value is a bf16 value); QK^T keeps one
//     accumulator per 128-dim tile plus one for the RoPE dims, and the
//     token's tile scales weight the tile accumulators afterwards, in fp32;
//   - a V fragment (one dim of 8 tokens) comes from ds_read_b64_tr_b8; each
//     code is widened to fp32, multiplied by its token's tile scale and
//     rounded once to bf16 (P stays the plain bf16 softmax weight, as in the
//     bf16 kernel, so the largest weight of a row is exact and a row that
//     sees one key returns that key's dequantised value).  The conversion
//     instruction's own scale operand cannot stand in for the multiply: it
//     applies only the scale's power of two.
//
// A half-page (32 records, 20992 bytes) lands in LDS as the plain memory
// image, 21 direct-to-LDS loads of 1 KB each; records past the segment's last
// token are replaced by that token's record.  The 656-byte record stride
// (164 dwords, 36 mod 64 banks) needs no swizzle: the 16-byte K reads (16
// lanes, so 16 tokens, per pass) hit distinct banks.  Tokens 16 apart share
// banks, so 8-byte reads, served 32 lanes per pass, must not mix them: MFMA
// row m of a 16-token k-step holds token tok_of_row(m) = 8 m3 + 4 m1 + 2 m0
// + m2 (m = 8 m3 + 4 m2 + 2 m1 + m0), in the K reads, the score scales and
// mask, and the V reads and scales alike, so the two 32-lane passes of a
// transposed V read cover the even and then the odd tokens of a k-step,
// whose 8-byte pieces sit on disjoint banks.
//
// Token-list mode (sparse decode, kList): each "request" is one query token's
// list of cache token ids; the score waves stage the ids of half-page t + 3 in
// LDS during step t, and each direct-to-LDS load takes its record from the
// cache page the id names, so the listed records are read once, in place.
#include <math.h>

#include "common.h"
#include "device_util.h"
#include "rows64.h"

namespace mla {

namespace {

using namespace rows64;

constexpr int kHalfFp8 = kHalf * kTokBytesFp8;         // 20992
constexpr int kDmaFp8 = (kHalfFp8 + 1023) / 1024;      // 21 one-KB loads per half-page
constexpr int kDmaWave = (kDmaFp8 + 1) / 2;            // 11 per value wave: blocks 0..10 and 10..20
constexpr int kSlot = kDmaFp8 * 1024;                  // 21504 (the last load is half padding)
constexpr int kChunks = kTokBytesFp8 / 16;             // 41 sixteen-byte chunks per record
constexpr int kPOff = kRing * kSlot;                   // 86016
constexpr int kPBytes = 4096;                          // P^T: 2 row tiles x 2 k-steps x 1 KB
constexpr int kXBytes = kRowsWG * kXStride * 4;        // output stage, over ring and P
constexpr int kFlagOff = (kPOff + 2 * kPBytes) > kXBytes ? (kPOff + 2 * kPBytes) : kXBytes;
constexpr int kStatOff = kFlagOff + 64;
constexpr int kIdsOff = kStatOff + 2 * kRowsWG * 4;  // token-list mode: ids of kRing half-pages
constexpr int kLdsBytes = kIdsOff + kRing * kHalf * 4;

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) f32x2 lds_f32x2;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// 8 E4M3FN codes (little-endian in two dwords) -> 8 bf16, exactly.
__device__ __forceinline__ bf16x8 codes_to_bf16(unsigned lo, unsigned hi) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    return (bf16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Score-wave MFMAs.  The score waves keep Q^T in the accumulator registers,
// which they do not otherwise use (the value waves hold O^T there), and their
// five score accumulators in VGPRs, where the tile scales are applied without
// copies; this leaves VGPRs for reading every tile scale of a step before its
// MFMAs.  Written as asm, since the compiler would give the MFMA builtins of
// this kernel accumulator-register destinations.  The K operand is written by
// VALU conversions two wait states before an MFMA may read it (s_nop 1); a
// dependent chain on one accumulator needs none between its MFMAs; the first
// MFMA of a chain adds to an inline zero; score_done() covers the MFMA-write
// to VALU-read distance before the scores are read.
__device__ __forceinline__ void score_first(f32x16 &s, const bf16x8 &k, const bf16x8 &qa) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(k), "a"(qa));
}
__device__ __forceinline__ void score_next(f32x16 &s, const bf16x8 &k, const bf16x8 &qa) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(k), "a"(qa));
}
__device__ __forceinline__ void score_done(f32x16 (&s)[5]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0]), "+v"(s[1]), "+v"(s[2]), "+v"(s[3]), "+v"(s[4]));
}

// Blocks of value wave v: 0 .. 10 (v = 0) or 10 .. 20 (v = 1).  Both waves
// load block 10 (the same bytes to the same place), which keeps their code
// identical.
__device__ __forceinline__ int first_block(int v) { return v ? kDmaFp8 - kDmaWave : 0; }

// Token of MFMA row m (0..31) of a half-page: within each 16-token k-step,
// bits (m3 m2 m1 m0) -> 8 m3 + 4 m1 + 2 m0 + m2.
__device__ __forceinline__ int tok_of_row(int m) {
    return (m & 16) + 8 * ((m >> 3) & 1) + 4 * ((m >> 1) & 1) + 2 * (m & 1) + ((m >> 2) & 1);
}

// Value wave v's direct-to-LDS loads of a half-page: its k-th load is 1 KB
// block i = first_block(v) + k, bytes [1024 i, 1024 i + 1024) of the 32
// records; lane l takes chunk 64 i + l, i.e. chunk c = 64 i + l - 41 tau of
// record tau = (64 i + l) / 41, moved to the same chunk of record tl (the
// half-page's last valid record) when tau lies past it.
//
// Paged mode: record tau is at hp + 656 tau, so a load is a uniform base plus
// this lane's byte offset, which depends on (v, k, tl) alone: computed once
// for full half-pages (tl = 31) and once per segment for its last one.
__device__ __forceinline__ unsigned half_offset(int v, int k, int lane, int tl) {
    int ch = 64 * (first_block(v) + k) + lane;
    const int tau = ch / kChunks;
    if (tau > tl) ch = kChunks * tl + (ch - kChunks * tau);
    return 16u * (unsigned)ch;
}

// Direct-to-LDS load of this lane's 16 bytes at base + off, base uniform.
// Memory is not named as clobbered, so LDS reads may move across it: the
// slot a load fills is read by no wave before the step barrier that follows
// the load's wait.
__device__ __forceinline__ void dma16_s(const unsigned char *base, unsigned off, unsigned lds) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "s"(lds) : "m0");
}

// Paged-mode loads of one half-page into one ring slot.
struct HalfDmaFp8 {
    const unsigned char *base;  // first record of the half-page
    unsigned dst;               // LDS byte address of the slot
    bool last;                  // the segment's last half-page
    __device__ __forceinline__ void issue(int v, int k, const unsigned (&fo)[kDmaWave],
                                          const unsigned (&lo)[kDmaWave]) const {
        const unsigned lds = __builtin_amdgcn_readfirstlane(dst + 1024 * (first_block(v) + k));
        dma16_s(base, last ? lo[k] : fo[k], lds);
    }
};

// Loads for the ring slot of half-page t.  Past the segment's end (t >= H)
// they repeat its last half-page into a slot that no wave reads again in
// this segment, so that every step issues the same loads without a branch.
__device__ __forceinline__ HalfDmaFp8 half_dma(const Segment &sg, const unsigned char *kv, int t,
                                               unsigned ring0) {
    const int src = t < sg.H ? t : sg.H - 1;
    HalfDmaFp8 d;
    d.dst = ring0 + (t % kRing) * kSlot;
    d.last = src == sg.H - 1;
    const int j = sg.j0 + (src >> 1);
    d.base = kv + ((int64_t)sg.bt[j] * kPage + (src & 1) * kHalf) * kTokBytesFp8;
    return d;
}

// Token-list mode loads of half-page t (< H) into its ring slot: record tau
// is at kv + 656 id[tau], id[k] keeping this lane's id for load k.
struct ListDma {
    const unsigned char *kv;
    unsigned dst;
    int id[kDmaWave];
    __device__ __forceinline__ void issue(int i0, int k, int lane) const {
        const int ch = 64 * (i0 + k) + lane;
        const int tau = ch / kChunks;
        dma16(kv + (int64_t)id[k] * kTokBytesFp8 + 16 * (ch - kChunks * tau),
              __builtin_amdgcn_readfirstlane(dst + 1024 * (i0 + k)));
    }
};

__device__ __forceinline__ ListDma list_dma(const Segment &sg, const unsigned char *kv, int t, int v,
                                            int lane, unsigned ring0, const lds_i32 *ids) {
    ListDma d;
    d.kv = kv;
    d.dst = ring0 + (t % kRing) * kSlot;
    const int tl = sg.tok_last(t);
    const lds_i32 *id = ids + (t % kRing) * kHalf;
#pragma unroll
    for (int k = 0; k < kDmaWave; ++k) {
        const int tau = (64 * (first_block(v) + k) + lane) / kChunks;
        d.id[k] = id[tau < tl ? tau : tl];
    }
    return d;
}

__device__ __forceinline__ void list_issue_step(const Segment &sg, const unsigned char *kv, int t, int v,
                                                int lane, unsigned ring0, const lds_i32 *ids) {
    const ListDma d = list_dma(sg, kv, t, v, lane, ring0, ids);
#pragma unroll
    for (int k = 0; k < kDmaWave; ++k) d.issue(first_block(v), k, lane);
}

template <bool kList>
__global__ __launch_bounds__(kThreads, 1) void decode_rows64_fp8_kernel(
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
    lds_i32 *ids_lds = (lds_i32 *)(smem + kIdsOff);
    float *X = (float *)smem_raw;  // output stage [64][kXStride]
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
        const int krec = kTokBytesFp8 * tok_of_row(l32);  // this lane's K token record in a slot
        for_each_segment(mrow, seqlens, split_base, block_table, a.bt_stride, [&](const Segment &sg) {
            if constexpr (kList) {
                stage_first_ids(ids_lds, sg, l32, h);
                __syncthreads();  // the value waves load half-pages 0 .. 2
            }
            int n_visible = a.causal ? sg.L - (a.s_q - 1 - qi) : sg.L;
            n_visible = n_visible > 0 ? n_visible : 0;
            const int n_visible_all = a.causal ? sg.L - (a.s_q - 1) : sg.L;
            // Q^T operand for 32x32x16 (loaded into VGPRs, then moved to the
            // accumulator registers).  Latent k-steps 2 pp + e (pp < 16, e < 2)
            // give lane half h dims 32 pp + 16 h + 8 e .. +8, so that one
            // 16-byte read of 16 codes per lane feeds both k-steps of a pair
            // (K reads below); RoPE k-steps 32 + r give it dims 512 + 16 r + 8 h.
            bf16x8 qf[kDQk / 16];
            const uint16_t *qrow = q + ((int64_t)sg.b * a.M + row_q) * kDQk;
            bf16x8 qv[kDQk / 16];
#pragma unroll
            for (int ks = 0; ks < kDQk / 16; ++ks)
                qv[ks] = *(const bf16x8 *)(qrow + (ks < kDV / 16 ? 32 * (ks >> 1) + 16 * h + 8 * (ks & 1)
                                                                 : 16 * ks + 8 * h));
#pragma unroll
            for (int ks = 0; ks < kDQk / 16; ++ks) asm volatile("; q to agprs" : "=a"(qf[ks]) : "0"(qv[ks]));
            // lsum: sum of the fp32 weights (for the lse); wsum: sum of the
            // weights as rounded to bf16 for the value product, which
            // normalises the output
            float m_seen = -INFINITY, m, lsum, wsum;
            bool again;
            do {  // one pass over the segment; repeated only after a restart
                m = m_seen;
                lsum = 0.f;
                wsum = 0.f;
                again = false;
                bool ovf = false;
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
                    const lds_u8 *S = smem + (t % kRing) * kSlot;
                    // lane holds tokens 8 (i/4) + 2 (i%4) + h of the half-page for
                    // its row; a token's four tile scales are the 16 bytes at byte
                    // 512 of its record: all sixteen read now, used after the MFMAs
                    f32x4 sc[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        sc[i] = *(const lds_f32x4 *)(S + kTokBytesFp8 * (8 * (i >> 2) + 2 * (i & 3) + h) + kFp8ScalesAt);
                    // S^T (32 tokens x 32 rows) per 128-dim tile and for the RoPE dims
                    f32x16 acc[5];
                    // K codes of k-steps 2 pp, 2 pp + 1: the 16 codes at dims
                    // 32 pp + 16 h of this lane's token, one 16-byte read,
                    // kPairs pairs in flight ahead of their MFMAs; the fences
                    // pin that order.  A 16-lane group of the read covers 16
                    // tokens, whose records start 36 banks apart (mod 64):
                    // every lane of the group hits its own 4 banks.
                    constexpr int kPairs = 4;
                    auto read_pair = [&](int pp) {
                        return *(const lds_u32x4 *)(S + krec + 32 * pp + 16 * h);
                    };
                    bf16x8 kr[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        kr[r] = *(const lds_bf16x8 *)(S + krec + kFp8RopeAt + 32 * r + 16 * h);
                    u32x4 kc[kPairs];
#pragma unroll
                    for (int pp = 0; pp < kPairs; ++pp) kc[pp] = read_pair(pp);
#pragma unroll
                    for (int pp = 0; pp < 16; ++pp) {
                        __builtin_amdgcn_sched_barrier(0);
                        const u32x4 cur = kc[pp % kPairs];
                        if (pp + kPairs < 16) kc[pp % kPairs] = read_pair(pp + kPairs);
                        f32x16 &at = acc[pp >> 2];
                        if ((pp & 3) == 0) score_first(at, codes_to_bf16(cur[0], cur[1]), qf[2 * pp]);
                        else score_next(at, codes_to_bf16(cur[0], cur[1]), qf[2 * pp]);
                        score_next(at, codes_to_bf16(cur[2], cur[3]), qf[2 * pp + 1]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    score_first(acc[4], kr[0], qf[32]);
#pragma unroll
                    for (int r = 1; r < 4; ++r) score_next(acc[4], kr[r], qf[32 + r]);
                    score_done(acc);
                    asm volatile("" : "+v"(f0), "+v"(f1));  // the flag test stays behind the MFMAs
                    if (__builtin_amdgcn_readfirstlane(f0 | f1)) {
                        again = true;
                        break;
                    }
                    // per score: x = RoPE + s0 t0 + s1 t1 + s2 t2 + s3 t3, one fma at
                    // a time in that order
                    float x[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        float v = __builtin_fmaf(sc[i][0], acc[0][i], acc[4][i]);
                        v = __builtin_fmaf(sc[i][1], acc[1][i], v);
                        v = __builtin_fmaf(sc[i][2], acc[2][i], v);
                        x[i] = __builtin_fmaf(sc[i][3], acc[3][i], v);
                    }
                    const int tok0 = sg.j0 * kPage + t * kHalf;
                    if (tok0 + kHalf > n_visible_all) {  // the causal edge or the segment's end
                        const int tok_base = tok0 + h;
#pragma unroll
                        for (int i = 0; i < 16; ++i)
                            x[i] = (tok_base + 8 * (i >> 2) + 2 * (i & 3) < n_visible) ? x[i] : -INFINITY;
                    }
                    float mloc = x[0];
#pragma unroll
                    for (int i = 1; i < 16; ++i) mloc = fmaxf(mloc, x[i]);
                    mloc = max_xor32(mloc);
                    m_seen = fmaxf(m_seen, mloc);
                    if (m == -INFINITY) m = mloc;  // first keys of this row
                    ovf |= mloc > m + grow;
                    flag_lds[2 * (t & 1) + w] = __builtin_amdgcn_ballot_w64(ovf) != 0;  // same value from every lane
                    const float mc = (m == -INFINITY) ? 0.f : m * c;
                    float p[16], psum = 0.f;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], c, -mc));
                        psum += p[i];
                    }
                    lsum += psum;
                    // P^T operand blocks: (row tile w, k-step kk) -> 1 KB at P + (2 w + kk) KB
                    lds_u8 *P = smem + kPOff + (t & 1) * kPBytes + (2 * w) * 1024 + lane * 16;
                    float rsum = 0.f;
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        const int i0 = 8 * kk;
                        const u32x4 pw = {pack_bf16(p[i0], p[i0 + 1]), pack_bf16(p[i0 + 2], p[i0 + 3]),
                                          pack_bf16(p[i0 + 4], p[i0 + 5]), pack_bf16(p[i0 + 6], p[i0 + 7])};
#pragma unroll
                        for (int e = 0; e < 4; ++e) rsum = add_bf16_pair(pw[e], rsum);
                        *(lds_u32x4 *)(P + kk * 1024) = pw;
                    }
                    wsum += rsum;
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
        // ================= value waves: dims d0 .. d0 + 255 (tiles 2 v, 2 v + 1), all 64 rows
        if constexpr (kList) {
            const int v = w - 2, d0 = v * 256;
            // Transposed V reads (ds_read_b64_tr_b8), 32x32x16 A operand of
            // k-step kk, dim tile dt.  The k order must match P^T, which keeps the
            // score accumulator's order: lane half h = lane / 32 holds rows
            // 4 h + 0..3 and 8 + 4 h + 0..3 of the 16-token k-step, which are
            // tokens h + 0, 2, 4, 6 and 8 + h + 0, 2, 4, 6 (tok_of_row).  16-lane
            // group g = lane / 16 covers dims d0 + 32 dt + 16 (g & 1) + (lane % 16);
            // its lanes 2 r, 2 r + 1 point at the r-th of those 8 tokens, 8 codes
            // at dim offset 8 (lane % 2).
            const int g = lane >> 4, i16 = lane & 15, vr = i16 >> 1;
            const int vtok = tok_of_row(4 * (g >> 1) + (vr & 3) + 8 * (vr >> 2));
            const int vrec = kTokBytesFp8 * vtok + d0 + 16 * (g & 1) + 8 * (i16 & 1);
            // scales of tiles 2 v, 2 v + 1 of this lane's first token (lane / 32)
            const int vsc = kTokBytesFp8 * (lane >> 5) + kFp8ScalesAt + 8 * v;
            for_each_segment(mrow, seqlens, split_base, block_table, a.bt_stride, [&](const Segment &sg) {
                if constexpr (kList) __syncthreads();  // ids of half-pages 0 .. 2 staged
                list_issue_step(sg, kv, 0, v, lane, ring0, ids_lds);
                if (sg.H > 1) list_issue_step(sg, kv, 1, v, lane, ring0, ids_lds);
                f32x16 o[2][8];
                bool again;
                do {  // one pass over the segment; repeated only after a restart
                    zero_acc(o);
                    again = false;
                    for (int t = 0; t <= sg.H; ++t) {
                        wait_own_dma<kDmaWave>(t + 1 < sg.H);
                        __syncthreads();
                        const int fr = 2 * ((t + 1) & 1);
                        if (__builtin_amdgcn_readfirstlane(flag_lds[fr] | flag_lds[fr + 1])) {
                            again = true;  // the score waves restart the segment
                            break;
                        }
                        const bool more = t + 2 < sg.H;
                        if (t == 0) {
                            if (more) list_issue_step(sg, kv, t + 2, v, lane, ring0, ids_lds);
                            continue;
                        }
                        // half-page t + 2 goes to the slot half-page t - 2 used; its
                        // loads are spread over this step's MFMAs (one after each
                        // MFMA pair)
                        ListDma dma;
                        if (more) dma = list_dma(sg, kv, t + 2, v, lane, ring0, ids_lds);
                        const int i0 = first_block(v);
                        const int tp = t - 1;  // half-page processed this step
                        const lds_u8 *V = smem + (tp % kRing) * kSlot + vrec;
                        const lds_u8 *Vs = smem + (tp % kRing) * kSlot + vsc;
                        const lds_u8 *P = smem + kPOff + (tp & 1) * kPBytes + lane * 16;
                        // scales of this lane's 8 tokens of k-step kk (tile 2 v and 2 v + 1)
                        auto read_scales = [&](int kk, f32x2 (&sc)[8]) {
    #pragma unroll
                            for (int j = 0; j < 8; ++j)
                                sc[j] = *(const lds_f32x2 *)(Vs + kTokBytesFp8 * (16 * kk + 2 * (j & 3) + 8 * (j >> 2)));
                        };
                        // V^T fragment: one dim of the 8 tokens, each code times its
                        // token's scale of tile 2 v + (dt / 4), rounded to bf16
                        auto read_v = [&](int kk, int dt, const f32x2 (&sc)[8]) {
                            const i32x2 cv = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                                (lds_i32x2 *)(V + kTokBytesFp8 * 16 * kk + 32 * dt));
                            const int ti = dt >> 2;
                            const f32x2 a0 = __builtin_amdgcn_cvt_pk_f32_fp8((unsigned)cv[0], false);
                            const f32x2 a1 = __builtin_amdgcn_cvt_pk_f32_fp8((unsigned)cv[0], true);
                            const f32x2 a2 = __builtin_amdgcn_cvt_pk_f32_fp8((unsigned)cv[1], false);
                            const f32x2 a3 = __builtin_amdgcn_cvt_pk_f32_fp8((unsigned)cv[1], true);
                            return __builtin_bit_cast(bf16x8, (u32x4){
                                pack_bf16(a0[0] * sc[0][ti], a0[1] * sc[1][ti]), pack_bf16(a1[0] * sc[2][ti], a1[1] * sc[3][ti]),
                                pack_bf16(a2[0] * sc[4][ti], a2[1] * sc[5][ti]), pack_bf16(a3[0] * sc[6][ti], a3[1] * sc[7][ti])});
                        };
                        auto read_p = [&](int r, int kk) {
                            return *(const lds_bf16x8 *)(P + (2 * r + kk) * 1024);
                        };
                        // k-step 0's operands first; k-step 1's are read between
                        // k-step 0's MFMAs
                        f32x2 sc0[8], sc1[8];
                        read_scales(0, sc0);
                        bf16x8 v0[8], v1[8];
                        const bf16x8 p00 = read_p(0, 0), p10 = read_p(1, 0);
    #pragma unroll
                        for (int dt = 0; dt < 8; ++dt) v0[dt] = read_v(0, dt, sc0);
                        read_scales(1, sc1);
                        const bf16x8 p01 = read_p(0, 1), p11 = read_p(1, 1);
    #pragma unroll
                        for (int dt = 0; dt < 8; ++dt) {
                            o[0][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0[dt], p00, o[0][dt], 0, 0, 0);
                            o[1][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0[dt], p10, o[1][dt], 0, 0, 0);
                            v1[dt] = read_v(1, dt, sc1);
                            if (more) dma.issue(i0, dt, lane);
                        }
    #pragma unroll
                        for (int dt = 0; dt < 8; ++dt) {
                            o[0][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1[dt], p01, o[0][dt], 0, 0, 0);
                            o[1][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1[dt], p11, o[1][dt], 0, 0, 0);
                            if (more && dt < kDmaWave - 8) dma.issue(i0, 8 + dt, lane);
                        }
                    }
                    if (again) {
                        wait_vmcnt<0>();
                        __syncthreads();
                        list_issue_step(sg, kv, 0, v, lane, ring0, ids_lds);
                        if (sg.H > 1) list_issue_step(sg, kv, 1, v, lane, ring0, ids_lds);
                    }
                } while (again);
                __syncthreads();  // score waves' final stats visible
                stage_output(X, o, d0, lane);
                __syncthreads();  // staged output complete
                write_rows(a, sg, split_base, X, stat_lds + kRowsWG, row0, tid);
                __syncthreads();  // LDS free for the next segment
            });
        } else {
            const int v = w - 2, d0 = v * 256;
            // Transposed V reads (ds_read_b64_tr_b8), 32x32x16 A operand of
            // k-step kk, dim tile dt.  The k order must match P^T, which keeps the
            // score accumulator's order: lane half h = lane / 32 holds rows
            // 4 h + 0..3 and 8 + 4 h + 0..3 of the 16-token k-step, which are
            // tokens h + 0, 2, 4, 6 and 8 + h + 0, 2, 4, 6 (tok_of_row).  16-lane
            // group g = lane / 16 covers dims d0 + 32 dt + 16 (g & 1) + (lane % 16);
            // its lanes 2 r, 2 r + 1 point at the r-th of those 8 tokens, 8 codes
            // at dim offset 8 (lane % 2).
            const int g = lane >> 4, i16 = lane & 15, vr = i16 >> 1;
            const int vtok = tok_of_row(4 * (g >> 1) + (vr & 3) + 8 * (vr >> 2));
            const int vrec = kTokBytesFp8 * vtok + d0 + 16 * (g & 1) + 8 * (i16 & 1);
            // scales of tiles 2 v, 2 v + 1 of this lane's first token (lane / 32)
            const int vsc = kTokBytesFp8 * (lane >> 5) + kFp8ScalesAt + 8 * v;
            unsigned fo[kDmaWave];  // offsets of the loads of a full half-page
    #pragma unroll
            for (int k = 0; k < kDmaWave; ++k) fo[k] = half_offset(v, k, lane, kHalf - 1);
            for_each_segment(mrow, seqlens, split_base, block_table, a.bt_stride, [&](const Segment &sg) {
                unsigned lo[kDmaWave];  // offsets of the loads of the segment's last half-page
                const int tl_end = sg.tok_last(sg.H - 1);
    #pragma unroll
                for (int k = 0; k < kDmaWave; ++k) lo[k] = half_offset(v, k, lane, tl_end);
                auto issue_all = [&](int t) {
                    const HalfDmaFp8 d = half_dma(sg, kv, t, ring0);
    #pragma unroll
                    for (int k = 0; k < kDmaWave; ++k) d.issue(v, k, fo, lo);
                };
                if constexpr (kList) __syncthreads();  // ids of half-pages 0 .. 2 staged
                issue_all(0);
                issue_all(1);
                f32x16 o[2][8];
                // k-step 0's V^T operands of the half-page the next step
                // processes, dequantised one step ahead
                bf16x8 vn[8];
                // scales of this lane's 8 tokens of k-step kk of half-page u (tiles 2 v, 2 v + 1)
                auto read_scales = [&](int u, int kk, f32x2 (&sc)[8]) {
                    const lds_u8 *Vs = smem + (u % kRing) * kSlot + vsc;
    #pragma unroll
                    for (int j = 0; j < 8; ++j)
                        sc[j] = *(const lds_f32x2 *)(Vs + kTokBytesFp8 * (16 * kk + 2 * (j & 3) + 8 * (j >> 2)));
                };
                // V^T fragment of half-page u: one dim of the 8 tokens (codes), then
                // each code times its token's scale of tile 2 v + (dt / 4), rounded
                // to bf16
                auto read_codes = [&](int u, int kk, int dt) {
                    return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (lds_i32x2 *)(smem + (u % kRing) * kSlot + vrec + kTokBytesFp8 * 16 * kk + 32 * dt));
                };
                auto dequant = [&](const i32x2 cv, int dt, const f32x2 (&sc)[8]) {
                    const int ti = dt >> 2;
                    const f32x2 a0 = __builtin_amdgcn_cvt_pk_f32_fp8((unsigned)cv[0], false);
                    const f32x2 a1 = __builtin_amdgcn_cvt_pk_f32_fp8((unsigned)cv[0], true);
                    const f32x2 a2 = __builtin_amdgcn_cvt_pk_f32_fp8((unsigned)cv[1], false);
                    const f32x2 a3 = __builtin_amdgcn_cvt_pk_f32_fp8((unsigned)cv[1], true);
                    return __builtin_bit_cast(bf16x8, (u32x4){
                        pack_bf16(a0[0] * sc[0][ti], a0[1] * sc[1][ti]), pack_bf16(a1[0] * sc[2][ti], a1[1] * sc[3][ti]),
                        pack_bf16(a2[0] * sc[4][ti], a2[1] * sc[5][ti]), pack_bf16(a3[0] * sc[6][ti], a3[1] * sc[7][ti])});
                };
                // step t >= 1: O += V^T P^T over half-page t - 1, the loads of
                // half-page t + 2 (repeats past the end) and the reads ahead for
                // step t + 1 (unused after the last step)
                auto body = [&](int t) {
                    const int tp = t - 1;
                    const HalfDmaFp8 dma = half_dma(sg, kv, t + 2, ring0);
                    const lds_u8 *P = smem + kPOff + (tp & 1) * kPBytes + lane * 16;
                    auto read_p = [&](int r, int kk) { return *(const lds_bf16x8 *)(P + (2 * r + kk) * 1024); };
                    f32x2 sc[8];
                    read_scales(tp, 1, sc);
                    const bf16x8 p00 = read_p(0, 0), p10 = read_p(1, 0), p01 = read_p(0, 1), p11 = read_p(1, 1);
                    bf16x8 v1[8];
                    i32x2 raw[8];
                    raw[0] = read_codes(tp, 1, 0);
                    raw[1] = read_codes(tp, 1, 1);
    #pragma unroll
                    for (int dt = 0; dt < 8; ++dt) {
                        o[0][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vn[dt], p00, o[0][dt], 0, 0, 0);
                        o[1][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vn[dt], p10, o[1][dt], 0, 0, 0);
                        if (dt + 2 < 8) raw[dt + 2] = read_codes(tp, 1, dt + 2);
                        v1[dt] = dequant(raw[dt], dt, sc);
                        dma.issue(v, dt, fo, lo);
                    }
                    read_scales(t, 0, sc);
                    raw[0] = read_codes(t, 0, 0);
                    raw[1] = read_codes(t, 0, 1);
    #pragma unroll
                    for (int dt = 0; dt < 8; ++dt) {
                        o[0][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1[dt], p01, o[0][dt], 0, 0, 0);
                        o[1][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1[dt], p11, o[1][dt], 0, 0, 0);
                        if (dt + 2 < 8) raw[dt + 2] = read_codes(t, 0, dt + 2);
                        vn[dt] = dequant(raw[dt], dt, sc);
                        if (dt < kDmaWave - 8) dma.issue(v, 8 + dt, fo, lo);
                    }
                };
                bool again;
                do {  // one pass over the segment; repeated only after a restart
                    zero_acc(o);
                    again = false;
                    for (int t = 0; t <= sg.H; ++t) {
                        // every wave's loads of half-page t are done (those of t + 1
                        // may be in flight) and the flags of step t - 1 are visible
                        wait_vmcnt<kDmaWave>();
                        __syncthreads();
                        const int fr = 2 * ((t + 1) & 1);
                        if (__builtin_amdgcn_readfirstlane(flag_lds[fr] | flag_lds[fr + 1])) {
                            again = true;  // the score waves restart the segment
                            break;
                        }
                        if (t == 0) {
                            issue_all(2);
                            f32x2 sc[8];
                            read_scales(0, 0, sc);
    #pragma unroll
                            for (int dt = 0; dt < 8; ++dt) vn[dt] = dequant(read_codes(0, 0, dt), dt, sc);
                            continue;
                        }
                        body(t);
                    }
                    if (again) {
                        wait_vmcnt<0>();
                        __syncthreads();
                        issue_all(0);
                        issue_all(1);
                    }
                } while (again);
                wait_vmcnt<0>();  // the repeated loads past the segment's end have landed
                __syncthreads();  // score waves' final stats visible
                stage_output(X, o, d0, lane);
                __syncthreads();  // staged output complete
                write_rows(a, sg, split_base, X, stat_lds + kRowsWG, row0, tid);
                __syncthreads();  // LDS free for the next segment
            });
        }
    }
}

}  // namespace

hipError_t launch_decode_rows64_fp8(const DecodeArgs &a, hipStream_t stream) {
    const int groups8 = (a.num_parts + 7) / 8;
    const dim3 grid(groups8 * 8 * a.row_groups), block(kThreads);
    if (a.token_list)
        hipLaunchKernelGGL(decode_rows64_fp8_kernel<true>, grid, block, 0, stream, a, a.q, a.kv,
                           a.block_table, a.seqlens, a.meta, a.split_base);
    else
        hipLaunchKernelGGL(decode_rows64_fp8_kernel<false>, grid, block, 0, stream, a, a.q, a.kv,
                           a.block_table, a.seqlens, a.meta, a.split_base);
    return hipGetLastError();
}

}  // namespace mla
