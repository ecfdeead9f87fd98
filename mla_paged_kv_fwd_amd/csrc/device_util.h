// Device helpers shared by the decode kernels (gfx950).
#pragma once

#include "common.h"

namespace mla {

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) int lds_i32;

__device__ __forceinline__ unsigned lds_addr(const lds_u8 *p) { return (unsigned)(uintptr_t)p; }

// One 16-byte-per-lane load from global memory straight into LDS.  LDS
// destination = m0 + 16 * lane.  Issued from inline asm so that the compiler
// does not serialise LDS reads behind outstanding prefetches; completion is
// tracked explicitly with vmcnt waits.
__device__ __forceinline__ void dma16(const void *g, unsigned lds_byte_addr) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(lds_byte_addr)
                 : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

__device__ __forceinline__ float wave_max16(float v) {  // across lanes l, l^16, l^32, l^48
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}
__device__ __forceinline__ float wave_sum16(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

// acc + the two bf16 values packed in w (one v_dot2c_f32_bf16 against 1, 1).
__device__ __forceinline__ float add_bf16_pair(unsigned w, float acc) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), one, acc, false);
}

__device__ __forceinline__ unsigned short f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(unsigned short, (__bf16)f);
}


}  // namespace mla
