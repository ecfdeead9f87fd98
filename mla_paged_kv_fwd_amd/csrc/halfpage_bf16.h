// LDS layout of one 32-token half-page of a bf16 cache as the 64-row bf16
// decode kernel holds it, with the lane addressing of its direct-to-LDS loads
// and of the MFMA operand reads.
//
// A half-page is 36 KB: 2304 slots of 16 bytes.  Token tau (0..31), 16-byte
// chunk c (0..71) of its 1152-byte row sits in slot
//   64 * (9 * (tau / 8) + c / 8) + 8 * (tau % 8) + ((c % 8) ^ swz(tau)),
//   swz(tau) = 4 * bit1(tau) + 2 * bit2(tau) + bit3(tau).
// Each 1 KB block (token group G = tau / 8, line lam = c / 8) holds one
// 128-byte line of eight consecutive tokens, so a direct-to-LDS load reads
// eight whole cache lines; the XOR keeps the K operand reads (ds_read_b128,
// 16 lanes per LDS cycle) and the transposed V operand reads
// (ds_read_b64_tr_b16, 16 or 32 lanes per cycle) free of bank conflicts.
#pragma once

#include "common.h"
#include "device_util.h"

namespace mla {
namespace halfpage {

constexpr int kTokens = 32;
constexpr int kBytes = kTokens * kTokBytesBf16;  // 36864
constexpr int kBlocksPerGroup = 9;               // 128-byte lines per 1152-byte row

// XOR term of the layout for token tau (bits 1, 2, 3 of tau).
__device__ __forceinline__ int swz(int tau) {
    return 4 * ((tau >> 1) & 1) + 2 * ((tau >> 2) & 1) + ((tau >> 3) & 1);
}

// Source row of the direct-to-LDS loads of token group G (tokens 8 G .. 8 G + 7
// of the half-page starting at page token tok0): lane l covers token
// 8 G + l / 8 (tokens past tok_last re-read tok_last) and, within each
// 128-byte line, the chunk whose swizzled slot is l % 8.  Line lam of the group
// is at +128 lam and lands in the half-page's 1 KB block 9 G + lam.
__device__ __forceinline__ const unsigned char *dma_row(const unsigned char *kv, int64_t phys,
                                                        int tok0, int tok_last, int G, int lane) {
    const int a = lane >> 3, b = lane & 7;
    const int tau = 8 * G + a;
    int t = tok0 + tau;
    t = t < tok_last ? t : tok_last;
    return kv + (phys * kPage + t) * kTokBytesBf16 + 16 * (b ^ swz(tau));
}

// The same loads when the half-page's tokens are listed by cache token id
// (ids[tau] = page * 64 + slot of token tau of the half-page, in LDS).
__device__ __forceinline__ const unsigned char *dma_row_ids(const unsigned char *kv,
                                                            const lds_i32 *ids, int tok_last,
                                                            int G, int lane) {
    const int a = lane >> 3, b = lane & 7;
    const int tau = 8 * G + a;
    const int t = tau < tok_last ? tau : tok_last;
    return kv + (int64_t)ids[t] * kTokBytesBf16 + 16 * (b ^ swz(tau));
}

// K operand of 32x32x16 k-step ks (A operand: lane = token l32, 8 dims
// 16 ks + 8 h .. + 8): byte offset kofs[ks % 4] + 1024 (ks / 4).
__device__ __forceinline__ void k_offsets(int (&kofs)[4], int l32, int h) {
    const int tau = l32, y = h ^ swz(tau);
#pragma unroll
    for (int k3 = 0; k3 < 4; ++k3)
        kofs[k3] = 9216 * (tau >> 3) + 128 * (tau & 7) + 16 * ((2 * k3) ^ y);
}

// Transposed V reads (ds_read_b64_tr_b16), 32x32x16 A operand of k-step kk
// (tokens 16 kk .. 16 kk + 15), dim tile dt (32 dims): 16-lane group
// g = lane / 16 covers dims 32 dt + 16 (g & 1) + (lane % 16) of the line
// range starting at line0; its lanes point at token
// 16 kk + 8 sel + 4 (g >> 1) + (lane % 16) / 4, 8 bytes at dim offset
// 4 (lane % 4), for sel = 0 (first read) and 1 (second read).  The token
// order inside a k-step matches the S^T accumulator layout of the 32x32
// MFMA (lane = row, register i = token 8 (i / 4) + 4 (lane / 32) + i % 4),
// so P^T from that accumulator is the B operand without any shuffle.
// Byte offset: vofs[sel][dt & 1] + 18432 kk + 1024 (dt / 2).
__device__ __forceinline__ void v_offsets(int (&vofs)[2][2], int lane, int line0) {
    const int g = lane >> 4, i16 = lane & 15;
    const int ta = 4 * (g >> 1) + (i16 >> 2);  // token within its group of 8
    const int y2 = 2 * (g & 1) + ((i16 & 3) >> 1);
#pragma unroll
    for (int sel = 0; sel < 2; ++sel)
#pragma unroll
        for (int d1 = 0; d1 < 2; ++d1)
            vofs[sel][d1] = 9216 * sel + 1024 * line0 + 128 * ta +
                            16 * ((4 * d1) ^ y2 ^ swz(8 * sel + ta)) + 8 * (i16 & 1);
}

__device__ __forceinline__ bf16x8 read_k(const lds_u8 *S, const int (&kofs)[4], int ks) {
    return *(const bf16x8 __attribute__((address_space(3))) *)(S + kofs[ks & 3] + 1024 * (ks >> 2));
}

__device__ __forceinline__ bf16x8 read_v(const lds_u8 *V, const int (&vofs)[2][2], int kk, int dt) {
    const int off = 18432 * kk + 1024 * (dt >> 1);
    const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (i16x4 __attribute__((address_space(3))) *)(V + vofs[0][dt & 1] + off));
    const i16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (i16x4 __attribute__((address_space(3))) *)(V + vofs[1][dt & 1] + off));
    const i16x8 v8 = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
    return __builtin_bit_cast(bf16x8, v8);
}

}  // namespace halfpage
}  // namespace mla
