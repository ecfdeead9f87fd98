// MLA decode attention over a paged latent KV cache: gfx950 kernels.
//
// Work decomposition ("row-group" kernel).  A work-group of 4 waves owns one
// split-KV part (a contiguous run of pages, possibly spanning requests) and
// one group of 16 query rows.  Each wave owns a 16-token slice of every page
// of the part and keeps its own online-softmax state (row max, row sum and a
// 16-row x 512-dim output accumulator), so the page loop needs no barrier: a
// wave streams its slices HBM -> LDS with direct-to-LDS loads (double
// buffered), runs S^T = K Q^T and O^T += V^T P^T on MFMA, and only at the end
// of a request segment do the 4 waves merge their states through LDS.
//
// Everything is computed transposed (tokens / dims on the MFMA row axis,
// query rows on the column axis) so that the score accumulator of
// S^T = K Q^T lands exactly in the register layout the PV product needs for
// its P^T operand, and every lane's softmax statistics belong to one query
// row (lane % 16).
//
// LDS slice layout ("chunk-major", swizzled): 16-byte chunk c of token t of a
// slice sits in slot c * 16 + (t ^ 4 * (c & 1)).  The K operand of QK^T is
// then one 1 KB ds_read_b128 block per wave, and the V^T operand of PV a
// ds_read_b64_tr_b16 (4 tokens x 16 dims transposed per 16-lane group); the
// XOR keeps both free of bank conflicts.
#include <math.h>

#include "common.h"
#include "device_util.h"

namespace mla {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 16;                       // query rows per work-group
constexpr int kSlice = 16;                      // tokens per wave per page
constexpr int kSliceBf16 = kSlice * kTokBytesBf16;  // 18432 B
constexpr int kSliceFp8 = 11 * 1024;            // 656 chunks used, 704 slots
constexpr int kLoadsBf16 = kSliceBf16 / 1024;   // 18 direct-to-LDS loads per slice
constexpr int kLoadsFp8 = 11;
constexpr int kXStride = kDV + 4;               // padded row stride of the merge buffer

// Issue the direct-to-LDS loads of this wave's slice of page `phys`.
// Tokens beyond `tok_last` (the last valid token of the page) are loaded from
// `tok_last` instead, so a slot past the sequence end holds finite data and is
// never read from outside the sequence.
template <bool FP8>
__device__ __forceinline__ void issue_slice(const unsigned char *kv, int64_t phys, int tok_last,
                                            int w, int lane, unsigned lds_dst) {
    const int lr = lane & 15, lg = lane >> 4;
    if constexpr (!FP8) {
        // block s = chunks 4 s + lg of the slice's tokens; the swizzle puts
        // token lr ^ 4 (lg & 1) in this lane's slot
        int t = kSlice * w + (lr ^ (4 * (lg & 1)));
        t = t < tok_last ? t : tok_last;
        const unsigned char *src = kv + (phys * kPage + t) * kTokBytesBf16 + lg * 16;
#pragma unroll
        for (int s = 0; s < kLoadsBf16; ++s)
            dma16(src + s * 64, __builtin_amdgcn_readfirstlane(lds_dst + s * 1024));
    } else {
        int t = kSlice * w + lr;  // FP8 slices are not swizzled
        t = t < tok_last ? t : tok_last;
        const unsigned char *rec = kv + (phys * kPage + t) * kTokBytesFp8;
#pragma unroll
        for (int s = 0; s < kLoadsFp8; ++s) {
            int cidx = 4 * s + lg;
            cidx = cidx < 40 ? cidx : 40;  // slots past chunk 40 are padding
            dma16(rec + cidx * 16, __builtin_amdgcn_readfirstlane(lds_dst + s * 1024));
        }
    }
}

// slot of chunk c of token t in a swizzled bf16 slice
__device__ __forceinline__ int slot16(int c, int t) { return c * 16 + (t ^ (4 * (c & 1))); }

// FP8 slice (chunk-major, 41 chunks x 16 tokens) -> bf16 slice (72 x 16).
// The latent codes are converted exactly (every E4M3FN value is a bf16
// value); their per-128-dim scales are applied after the MFMAs instead (to
// the per-tile partial scores, and to P for the value product), so the fp32
// scale is never rounded into the operands.  The RoPE chunks are copied.
// Also returns the scales of the lane's 4 tokens (4*lg + i): tsc[i][tile].
__device__ __forceinline__ void dequant_slice(const lds_u8 *f8, lds_u8 *bf, int lane, f32x4 *tsc) {
    const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int c = lg + 4 * k;  // fp8 chunk (16 codes of latent dims 16c .. 16c+15)
        const u32x4 codes = *(const u32x4 __attribute__((address_space(3))) *)(f8 + (c * 16 + lr) * 16);
        // two codes -> two bf16 per instruction (scale 1: exact), low byte
        // pair first, so each packed word keeps the codes' order
        unsigned packed[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            packed[2 * q] = __builtin_bit_cast(
                unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[q], 1.0f, false));
            packed[2 * q + 1] = __builtin_bit_cast(
                unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[q], 1.0f, true));
        }
        *(u32x4 __attribute__((address_space(3))) *)(bf + slot16(2 * c, lr) * 16) =
            (u32x4){packed[0], packed[1], packed[2], packed[3]};
        *(u32x4 __attribute__((address_space(3))) *)(bf + slot16(2 * c + 1, lr) * 16) =
            (u32x4){packed[4], packed[5], packed[6], packed[7]};
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int r = 33 + lg + 4 * k;  // RoPE chunk in the record
        const u32x4 v = *(const u32x4 __attribute__((address_space(3))) *)(f8 + (r * 16 + lr) * 16);
        *(u32x4 __attribute__((address_space(3))) *)(bf + slot16(64 + r - 33, lr) * 16) = v;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        tsc[i] = *(const f32x4 __attribute__((address_space(3))) *)(f8 + (32 * 16 + 4 * lg + i) * 16);
    // No wait here: the bf16 slice is read back only by this wave, whose LDS
    // operations execute in order, so its reads see these writes.
}

constexpr float kRescaleLog2 = 8.f;

typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

struct RowState {
    f32x4 o[kDV / 16];  // O^T tiles: lane holds dims 16*dt + 4*(lane/16) + i of row lane%16
    float m;            // running max of scaled scores (log2 domain)
    float lsum;         // this lane's share of the running sum (for the lse)
    float wsum;         // the same sum over the weights as the value product used
                        // them (bf16-rounded for a bf16 cache); normalises the output
};

// Scores, online softmax and PV for one 16-token slice held in LDS (bf16,
// chunk-major).  tok0 = sequence index of the slice's first token.
template <bool FP8>
__device__ __forceinline__ void attend_slice(const lds_u8 *S, const bf16x8 *qf, RowState &st,
                                             int lane, int tok0, int n_visible, float scale_log2,
                                             const f32x4 *tsc) {
    const int lr = lane & 15, lg = lane >> 4;
    const int kl = lane ^ (4 * (lg & 1));  // slot of (chunk 4 ks + lg, token lr) in block ks
    // S^T (16 tokens x 16 rows) = K (16 x 576) . Q^T (576 x 16).  bf16 cache:
    // two accumulation chains.  FP8 cache: one chain per 128-dim scale tile
    // plus one for the RoPE dims, combined with the token scales afterwards.
    float sc[4];
    if constexpr (!FP8) {
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kDQk / 32; ks += 2) {
            const bf16x8 k0 = *(const bf16x8 __attribute__((address_space(3))) *)(S + (ks * 64 + kl) * 16);
            const bf16x8 k1 = *(const bf16x8 __attribute__((address_space(3))) *)(S + ((ks + 1) * 64 + kl) * 16);
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[ks], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[ks + 1], s1, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = s0[i] + s1[i];
    } else {
        f32x4 acc[5];
#pragma unroll
        for (int t = 0; t < 5; ++t) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kDQk / 32; ++ks) {
            const bf16x8 kf = *(const bf16x8 __attribute__((address_space(3))) *)(S + (ks * 64 + kl) * 16);
            const int t = ks < 16 ? ks / 4 : 4;
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], acc[t], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sc[i] = acc[4][i] + tsc[i][0] * acc[0][i] + tsc[i][1] * acc[1][i] +
                    tsc[i][2] * acc[2][i] + tsc[i][3] * acc[3][i];
    }
    // lane holds tokens tok0 + 4*lg + i (i < 4) of query row lr
    float x[4];
    float mloc = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tok = tok0 + 4 * lg + i;
        x[i] = (tok < n_visible) ? sc[i] * scale_log2 : -INFINITY;
        mloc = fmaxf(mloc, x[i]);
    }
    mloc = wave_max16(mloc);
    // Lazy rescaling: the exponent reference m only moves when a row's max
    // grows by more than kRescaleLog2 (so p <= 2^kRescaleLog2); the final
    // result is the same for any reference.  A row with no visible key yet
    // (m = -inf) takes the new max without touching its all-zero accumulator.
    const bool fresh = (st.m == -INFINITY);
    const bool grow = mloc > st.m + kRescaleLog2;
    const float m_new = grow ? mloc : st.m;
    const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = grow ? __builtin_amdgcn_exp2f(st.m - m_ref) : 1.f;
    float psum = 0.f, p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(x[i] - m_ref);
        psum += p[i];
    }
    st.lsum = st.lsum * alpha + psum;
    st.m = m_new;
    if (__builtin_amdgcn_ballot_w64(grow && !fresh) != 0) {
#pragma unroll
        for (int dt = 0; dt < kDV / 16; ++dt) st.o[dt] *= alpha;
    }
    // P^T operand (tokens 4*lg + i of row lr).  FP8 cache: one copy per
    // 128-dim value tile with that tile's token scales folded in.
    constexpr int kTiles = FP8 ? 4 : 1;
    i16x4 pf[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            pf[t][i] = (short)f32_to_bf16_bits(FP8 ? p[i] * tsc[i][t] : p[i]);
    }
    // the output's normaliser: the weights as the value product uses them
    // (FP8: each 128-dim value tile has its own scaled copy of P, so no single
    // rounded sum matches them and the fp32 sum is used)
    if constexpr (FP8) {
        st.wsum = st.wsum * alpha + psum;
    } else {
        const auto pw = __builtin_bit_cast(u32x2_t, pf[0]);
        st.wsum = st.wsum * alpha + add_bf16_pair(pw[1], add_bf16_pair(pw[0], 0.f));
    }
    // O^T (512 dims x 16 rows) += V^T (512 x 16 tokens) . P^T (16 tokens x 16 rows)
    const int vp = (lr >> 1) & 1;  // chunk parity of this lane's V reads
    const lds_u8 *vt = S + (vp * 16 + 4 * (lg ^ vp) + (lr >> 2)) * 16 + 8 * (lr & 1);
#pragma unroll
    for (int dt = 0; dt < kDV / 16; ++dt) {
        const i16x4 vf = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (i16x4 __attribute__((address_space(3))) *)(vt + dt * 2 * 16 * 16));
        st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, pf[FP8 ? dt / 8 : 0], st.o[dt], 0, 0, 0);
    }
}

template <bool FP8>
__global__ __launch_bounds__(kThreads, 1) void decode_rowgroup_kernel(
    const DecodeArgs a, const uint16_t *__restrict__ q, const unsigned char *__restrict__ kv,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seqlens,
    const int32_t *__restrict__ meta, const int32_t *__restrict__ split_base) {
    // The read-only tables arrive as separate restrict-qualified arguments so
    // that their uniform reads compile to scalar loads.
    constexpr int kWaveLds = FP8 ? (2 * kSliceFp8 + kSliceBf16) : (2 * kSliceBf16);
    static_assert(4 * (kWaves * kRows * kXStride + 3 * kWaves * kRows) <= kWaves * kWaveLds,
                  "the merge buffers fit in the slice buffers");
    __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[kWaves * kWaveLds];
    lds_u8 *smem = (lds_u8 *)smem_raw;

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;

    // blockIdx -> (part, row group): the row groups of a part sit on one XCD
    // (blockIdx % 8) in consecutive dispatch slots so they share its L2.
    const int lin = blockIdx.x;
    const int rest = lin >> 3;
    const int rg = rest % a.row_groups;
    const int part = (rest / a.row_groups) * 8 + (lin & 7);
    if (part >= a.num_parts) return;
    const int32_t *mrow = meta + part * kMetaInts;
    const int b_first = mrow[0];
    if (b_first < 0) return;
    const int j_first = mrow[1], b_last = mrow[2], j_last = mrow[3], split_first = mrow[4];

    lds_u8 *wbase = smem + w * kWaveLds;
    const unsigned buf_addr[2] = {lds_addr(wbase), lds_addr(wbase + (FP8 ? kSliceFp8 : kSliceBf16))};
    lds_u8 *bf_slice = wbase + 2 * kSliceFp8;  // FP8 only: dequantised slice

    const int row0 = rg * kRows;
    const int row = row0 + lr;
    const int qi = row / a.h_q;

    for (int b = b_first; b <= b_last; ++b) {
        const int L = seqlens[b];
        const int npages = (L + kPage - 1) / kPage;
        if (L <= 0) continue;
        const int j0 = (b == b_first) ? j_first : 0;
        const int j1 = (b == b_last) ? j_last : npages - 1;
        const int rank = (b == b_first) ? split_first : 0;
        const int nsplit = split_base[b + 1] - split_base[b];
        int n_visible = a.causal ? L - (a.s_q - 1 - qi) : L;
        n_visible = n_visible > 0 ? n_visible : 0;
        const int32_t *bt = block_table + (int64_t)b * a.bt_stride;

        auto tok_last_of = [&](int j) { return (j == npages - 1) ? (L - 1 - j * kPage) : (kPage - 1); };
        issue_slice<FP8>(kv, bt[j0], tok_last_of(j0), w, lane, buf_addr[0]);

        // Q^T operand: lane holds dims 32*ks + 8*lg .. +8 of query row `row`
        bf16x8 qf[kDQk / 32];
        const uint16_t *qrow = q + ((int64_t)b * a.M + row) * kDQk + 8 * lg;
#pragma unroll
        for (int ks = 0; ks < kDQk / 32; ++ks) qf[ks] = *(const bf16x8 *)(qrow + 32 * ks);
        // Make the compiler retire the Q loads here (together with the first
        // slice, which was issued before them), not inside the page loop.
#pragma unroll
        for (int ks = 0; ks < kDQk / 32; ++ks) asm volatile("" : : "v"(qf[ks]));

        RowState st;
#pragma unroll
        for (int dt = 0; dt < kDV / 16; ++dt) st.o[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
        st.m = -INFINITY;
        st.lsum = 0.f;
        st.wsum = 0.f;

        int phys_ahead = (j0 < j1) ? bt[j0 + 1] : 0;
        for (int j = j0; j <= j1; ++j) {
            const int cur = (j - j0) & 1;
            if (j < j1) {
                issue_slice<FP8>(kv, phys_ahead, tok_last_of(j + 1), w, lane, buf_addr[cur ^ 1]);
                phys_ahead = (j + 2 <= j1) ? bt[j + 2] : 0;
                wait_vmcnt<FP8 ? kLoadsFp8 : kLoadsBf16>();
            } else {
                wait_vmcnt<0>();
            }
            const lds_u8 *S = wbase + cur * (FP8 ? kSliceFp8 : kSliceBf16);
            f32x4 tsc[4];
            if constexpr (FP8) {
                dequant_slice(S, bf_slice, lane, tsc);
                S = bf_slice;
            }
            attend_slice<FP8>(S, qf, st, lane, j * kPage + kSlice * w, n_visible, a.scale_log2, tsc);
        }

        // ---- merge the 4 waves' states and write the result
        st.lsum = wave_sum16(st.lsum);
        st.wsum = wave_sum16(st.wsum);
        __syncthreads();  // every wave is done reading its slices
        float *X = (float *)smem_raw;                 // [4][16][kXStride]
        float *Mw = X + kWaves * kRows * kXStride;     // [4][16]
        float *Lw = Mw + kWaves * kRows;               // [4][16]
        float *Rw = Lw + kWaves * kRows;               // [4][16]
#pragma unroll
        for (int dt = 0; dt < kDV / 16; ++dt)
            *(f32x4 *)(X + (w * kRows + lr) * kXStride + 16 * dt + 4 * lg) = st.o[dt];
        if (lg == 0) {
            Mw[w * kRows + lr] = st.m;
            Lw[w * kRows + lr] = st.lsum;
            Rw[w * kRows + lr] = st.wsum;
        }
        __syncthreads();
        {
            const int r = tid >> 4, d0 = (tid & 15) * 32;
            float mw[kWaves], mf = -INFINITY;
#pragma unroll
            for (int v = 0; v < kWaves; ++v) {
                mw[v] = Mw[v * kRows + r];
                mf = fmaxf(mf, mw[v]);
            }
            float aw[kWaves], lf = 0.f, rf = 0.f;
#pragma unroll
            for (int v = 0; v < kWaves; ++v) {
                aw[v] = (mw[v] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw[v] - mf);
                lf += aw[v] * Lw[v * kRows + r];
                rf += aw[v] * Rw[v * kRows + r];
            }
            const float inv = rf > 0.f ? 1.f / rf : 0.f;
            const float lse_val = lf > 0.f ? (mf + log2f(lf)) * 0.69314718055994530942f : -INFINITY;
            const int orow = row0 + r;
            if (nsplit == 1) {
                uint16_t *dst = a.out + ((int64_t)b * a.M + orow) * kDV + d0;
#pragma unroll
                for (int d = 0; d < 32; d += 8) {
                    unsigned pk[4];
#pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        float v0 = 0.f, v1 = 0.f;
#pragma unroll
                        for (int v = 0; v < kWaves; ++v) {
                            v0 += aw[v] * X[(v * kRows + r) * kXStride + d0 + d + e];
                            v1 += aw[v] * X[(v * kRows + r) * kXStride + d0 + d + e + 1];
                        }
                        pk[e / 2] = (unsigned)f32_to_bf16_bits(v0 * inv) |
                                    ((unsigned)f32_to_bf16_bits(v1 * inv) << 16);
                    }
                    *(u32x4 *)(dst + d) = (u32x4){pk[0], pk[1], pk[2], pk[3]};
                }
                if ((tid & 15) == 0) a.lse[(int64_t)b * a.M + orow] = lse_val;
            } else {
                const int slot = split_base[b] + rank;
                float *dst = a.o_part + ((int64_t)slot * a.M + orow) * kDV + d0;
#pragma unroll
                for (int d = 0; d < 32; d += 4) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int v = 0; v < kWaves; ++v)
                        acc += aw[v] * *(const f32x4 *)(X + (v * kRows + r) * kXStride + d0 + d);
                    *(f32x4 *)(dst + d) = acc * inv;
                }
                if ((tid & 15) == 0) a.lse_part[(int64_t)slot * a.M + orow] = lse_val;
            }
        }
        __syncthreads();  // LDS is reused by the next segment
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, bool fp8, hipStream_t stream) {
    const int groups8 = (a.num_parts + 7) / 8;
    const dim3 grid(groups8 * 8 * a.row_groups), block(kThreads);
    if (fp8)
        hipLaunchKernelGGL(decode_rowgroup_kernel<true>, grid, block, 0, stream, a, a.q, a.kv,
                           a.block_table, a.seqlens, a.meta, a.split_base);
    else
        hipLaunchKernelGGL(decode_rowgroup_kernel<false>, grid, block, 0, stream, a, a.q, a.kv,
                           a.block_table, a.seqlens, a.meta, a.split_base);
    return hipGetLastError();
}

int decode_rows_per_group() { return kRows; }

}  // namespace mla
