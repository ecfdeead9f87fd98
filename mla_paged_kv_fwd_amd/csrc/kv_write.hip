// Cache writer: stores the newest rows of every request into the paged latent
// cache, as bf16 rows or as 656-byte FP8 records (gfx950).
//
// One wave per row (576 bf16 values: 512 latent + 64 RoPE), four rows of one
// request per work-group (grid: row quads x requests), so the row, its
// position and its record address are wave-uniform scalars.  Row i of request
// b is the token at position L_b - n_new + i, in page block_table[b][pos / 64],
// slot pos % 64.
//
// FP8 record (DeepSeek KB page, "Key Contributions": 656 bytes per token, RoPE
// kept in BF16): bytes [0, 512) E4M3FN codes of the latent dims, [512, 528)
// one fp32 scale per 128-dim tile, [528, 656) the RoPE dims as bf16.  Each
// lane holds 8 latent dims (16 lanes per tile); the tile's absolute maximum
// is reduced across its 16 lanes and mapped to 448, E4M3FN's largest finite
// value: scale = amax / 448 in fp32, code = round-to-nearest-even of
// clip(x / scale, +-448), both divisions correctly rounded; an all-zero tile
// gets scale 0 and zero codes.
//
// x / scale: one correctly rounded reciprocal y = RN(1 / scale) per lane, then
// q0 = RN(x y) and two correction steps q' = RN(q + (x - q scale) y), the
// residual exact by FMA.  The first step brings q within one ulp of x / scale;
// from there one step gives the correctly rounded quotient (Markstein's
// theorem, e.g. Muller et al., Handbook of Floating-Point Arithmetic, on
// division with a fused multiply-add).  The theorem needs residuals that do
// not underflow; tiles whose amax is below 2^-60 take the plain division
// instead.  The quotient takes x's sign at the end, so -0 stays -0.
#include "common.h"

namespace mla {

namespace {

constexpr int kRowsPerBlock = 4;
constexpr float kE4m3Max = 448.f;

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xFFFF0000u); }

// Four fp32 values (already inside +-448) -> four E4M3FN codes, nearest even.
__device__ __forceinline__ unsigned e4m3x4(float a, float b, float c, float d) {
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
    return (unsigned)v;
}

__device__ __forceinline__ float clip448(float x) { return fminf(fmaxf(x, -kE4m3Max), kE4m3Max); }

template <bool FP8>
__global__ __launch_bounds__(64 * kRowsPerBlock) void kv_write_kernel(
    const uint16_t *__restrict__ k_new, int n_new, const int32_t *__restrict__ block_table,
    int64_t bt_stride, const int32_t *__restrict__ seqlens, unsigned char *__restrict__ cache) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.y;
    const int i = blockIdx.x * kRowsPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (i >= n_new) return;
    const int pos = seqlens[b] - n_new + i;
    if (pos < 0) return;
    const int64_t phys = block_table[(int64_t)b * bt_stride + pos / kPage];
    const int64_t tok = phys * kPage + pos % kPage;
    const unsigned char *src = (const unsigned char *)(k_new + ((int64_t)b * n_new + i) * kDQk);

    // latent dims 8 lane .. 8 lane + 7; lanes 0..7 also carry RoPE dims
    // 512 + 8 lane .. + 7
    const u32x4 lat = *(const u32x4 *)(src + 16 * lane);
    u32x4 rope = {};
    if (lane < 8) rope = *(const u32x4 *)(src + 2 * kDV + 16 * lane);

    if constexpr (!FP8) {
        unsigned char *dst = cache + tok * kTokBytesBf16;
        *(u32x4 *)(dst + 16 * lane) = lat;
        if (lane < 8) *(u32x4 *)(dst + 2 * kDV + 16 * lane) = rope;
    } else {
        unsigned char *dst = cache + tok * kTokBytesFp8;
        float x[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[2 * k] = bf16_lo(lat[k]);
            x[2 * k + 1] = bf16_hi(lat[k]);
        }
        float amax = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(x[k]));
        // the tile's 16 lanes are lanes 16 t .. 16 t + 15
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
        const float scale = amax / kE4m3Max;
        u32x2 codes = {0u, 0u};
        if (scale > 0.f) {
            float y[8];
            if (amax >= 0x1p-60f) {
                const float rs = 1.f / scale;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    float q = x[k] * rs;
                    q = __builtin_fmaf(__builtin_fmaf(-q, scale, x[k]), rs, q);
                    q = __builtin_fmaf(__builtin_fmaf(-q, scale, x[k]), rs, q);
                    // the corrections turn -0 into +0; the quotient has x's sign
                    y[k] = clip448(__builtin_copysignf(q, x[k]));
                }
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k) y[k] = clip448(x[k] / scale);
            }
            codes[0] = e4m3x4(y[0], y[1], y[2], y[3]);
            codes[1] = e4m3x4(y[4], y[5], y[6], y[7]);
        }
        *(u32x2 *)(dst + 8 * lane) = codes;
        if ((lane & 15) == 0) *(float *)(dst + kFp8ScalesAt + 4 * (lane >> 4)) = scale;
        if (lane < 8) *(u32x4 *)(dst + kFp8RopeAt + 16 * lane) = rope;
    }
}

}  // namespace

hipError_t launch_kv_write(const uint16_t *k_new, int batch, int n_new, const int32_t *block_table,
                           int64_t bt_stride, const int32_t *seqlens, void *cache, bool fp8,
                           hipStream_t stream) {
    const dim3 grid((unsigned)((n_new + kRowsPerBlock - 1) / kRowsPerBlock), (unsigned)batch);
    const dim3 block(64 * kRowsPerBlock);
    if (fp8)
        hipLaunchKernelGGL(kv_write_kernel<true>, grid, block, 0, stream, k_new, n_new,
                           block_table, bt_stride, seqlens, (unsigned char *)cache);
    else
        hipLaunchKernelGGL(kv_write_kernel<false>, grid, block, 0, stream, k_new, n_new,
                           block_table, bt_stride, seqlens, (unsigned char *)cache);
    return hipGetLastError();
}

}  // namespace mla
