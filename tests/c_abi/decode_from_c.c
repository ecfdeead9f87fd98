/*
 * A plain C consumer of libmla: builds a small paged problem on the host,
 * plans and decodes it through the C ABI only (include/mla.h and the HIP
 * runtime, no torch), and writes inputs and outputs as raw little-endian
 * files for a test to check against the oracle.
 *
 * usage: decode_from_c <out_dir> <fp8: 0 or 1>
 * files: q.bin (bf16 bits), cache.bin (bf16 bits or 656-byte records),
 *        bt.bin, seqlens.bin (int32), out.bin (bf16 bits), lse.bin (fp32),
 *        shape.txt ("batch s_q h_q pages width")
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mla.h"

#define CHECK_HIP(x)                                                                  \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));           \
            exit(2);                                                                  \
        }                                                                             \
    } while (0)
#define CHECK_MLA(x)                                                                  \
    do {                                                                              \
        int s_ = (int)(x);                                                            \
        if (s_ != MLA_OK) {                                                           \
            fprintf(stderr, "%s failed: %s\n", #x, mla_status_string(s_));           \
            exit(3);                                                                  \
        }                                                                             \
    } while (0)

static uint32_t rng_state = 0x9E3779B9u;
static float next_uniform(void) { /* xorshift32 -> [-1, 1) */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 17;
    rng_state ^= rng_state << 5;
    return (float)(rng_state >> 8) / 8388608.0f - 1.0f;
}

static uint16_t to_bf16(float f) { /* round to nearest even */
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static void write_file(const char *dir, const char *name, const void *p, size_t n) {
    char path[1024];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(p, 1, n, f) != n) {
        fprintf(stderr, "cannot write %s\n", path);
        exit(4);
    }
    fclose(f);
}

int main(int argc, char **argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s <out_dir> <fp8>\n", argv[0]);
        return 1;
    }
    const char *dir = argv[1];
    const int fp8 = atoi(argv[2]) != 0;
    const int batch = 3, s_q = 2, h_q = 64, M = s_q * h_q;
    const int seqlens[3] = {37, 700, 64};
    int width = 0, pages = 0;
    for (int b = 0; b < batch; ++b) {
        const int n = (seqlens[b] + MLA_PAGE - 1) / MLA_PAGE;
        pages += n;
        width = n > width ? n : width;
    }
    const size_t tok = fp8 ? MLA_FP8_RECORD : 2 * MLA_D_QK;
    const size_t q_bytes = (size_t)batch * M * MLA_D_QK * 2;
    const size_t c_bytes = (size_t)pages * MLA_PAGE * tok;
    uint16_t *q = malloc(q_bytes);
    unsigned char *cache = malloc(c_bytes);
    int32_t *bt = malloc(sizeof(int32_t) * batch * width);
    for (size_t i = 0; i < q_bytes / 2; ++i) q[i] = to_bf16(next_uniform());
    for (size_t t = 0; t < (size_t)pages * MLA_PAGE; ++t) {
        unsigned char *rec = cache + t * tok;
        if (!fp8) {
            for (int d = 0; d < MLA_D_QK; ++d) ((uint16_t *)rec)[d] = to_bf16(next_uniform());
        } else {
            /* codes 0x00..0x7E with random signs, four positive tile scales,
               bf16 RoPE dims: any such record is a valid FP8 record */
            for (int d = 0; d < 512; ++d) {
                unsigned c = (unsigned)((next_uniform() + 1.0f) * 63.0f);
                rec[d] = (unsigned char)((c > 0x7E ? 0x7E : c) | (next_uniform() < 0 ? 0x80 : 0));
            }
            for (int k = 0; k < 4; ++k) {
                const float s = 0.002f * (1.0f + k + next_uniform() * 0.5f);
                memcpy(rec + 512 + 4 * k, &s, 4);
            }
            for (int d = 0; d < 64; ++d) ((uint16_t *)(rec + 528))[d] = to_bf16(next_uniform());
        }
    }
    /* pages handed out in reverse order; unused entries -1 */
    int next_page = pages - 1;
    for (int b = 0; b < batch; ++b)
        for (int j = 0; j < width; ++j)
            bt[b * width + j] = j < (seqlens[b] + MLA_PAGE - 1) / MLA_PAGE ? next_page-- : -1;

    void *d_q, *d_cache, *d_bt, *d_sl, *d_meta, *d_sb, *d_ws, *d_out, *d_lse;
    const int parts = mla_default_num_parts(0, s_q, h_q);
    if (parts <= 0) {
        fprintf(stderr, "mla_default_num_parts: %d\n", parts);
        return 3;
    }
    const size_t ws_bytes = mla_workspace_bytes(batch, s_q, h_q, parts);
    CHECK_HIP(hipMalloc(&d_q, q_bytes));
    CHECK_HIP(hipMalloc(&d_cache, c_bytes));
    CHECK_HIP(hipMalloc(&d_bt, sizeof(int32_t) * batch * width));
    CHECK_HIP(hipMalloc(&d_sl, sizeof seqlens));
    CHECK_HIP(hipMalloc(&d_meta, sizeof(int32_t) * mla_metadata_ints(parts)));
    CHECK_HIP(hipMalloc(&d_sb, sizeof(int32_t) * (batch + 1)));
    CHECK_HIP(hipMalloc(&d_ws, ws_bytes));
    CHECK_HIP(hipMalloc(&d_out, (size_t)batch * M * MLA_D_V * 2));
    CHECK_HIP(hipMalloc(&d_lse, (size_t)batch * M * 4));
    CHECK_HIP(hipMemcpy(d_q, q, q_bytes, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_cache, cache, c_bytes, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_bt, bt, sizeof(int32_t) * batch * width, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_sl, seqlens, sizeof seqlens, hipMemcpyHostToDevice));

    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));
    const float scale = 1.0f / sqrtf((float)MLA_D_QK);
    CHECK_MLA(mla_get_metadata(d_sl, batch, s_q, h_q, parts, d_meta, d_sb, stream));
    if (fp8)
        CHECK_MLA(mla_decode_fwd_fp8(d_q, d_cache, pages, d_bt, width, d_sl, batch, s_q, h_q, scale,
                                     1, d_meta, d_sb, parts, d_ws, ws_bytes, d_out, d_lse,
                                     stream));
    else
        CHECK_MLA(mla_decode_fwd(d_q, d_cache, pages, d_bt, width, d_sl, batch, s_q, h_q, scale, 1,
                                 d_meta, d_sb, parts, d_ws, ws_bytes, d_out, d_lse, stream));
    CHECK_HIP(hipStreamSynchronize(stream));

    uint16_t *out = malloc((size_t)batch * M * MLA_D_V * 2);
    float *lse = malloc((size_t)batch * M * 4);
    CHECK_HIP(hipMemcpy(out, d_out, (size_t)batch * M * MLA_D_V * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(lse, d_lse, (size_t)batch * M * 4, hipMemcpyDeviceToHost));

    write_file(dir, "q.bin", q, q_bytes);
    write_file(dir, "cache.bin", cache, c_bytes);
    write_file(dir, "bt.bin", bt, sizeof(int32_t) * batch * width);
    write_file(dir, "seqlens.bin", seqlens, sizeof seqlens);
    write_file(dir, "out.bin", out, (size_t)batch * M * MLA_D_V * 2);
    write_file(dir, "lse.bin", lse, (size_t)batch * M * 4);
    char shape[128];
    const int n = snprintf(shape, sizeof shape, "%d %d %d %d %d\n", batch, s_q, h_q, pages, width);
    write_file(dir, "shape.txt", shape, (size_t)n);
    printf("decode_from_c: batch %d s_q %d h_q %d pages %d fp8 %d ok\n", batch, s_q, h_q, pages, fp8);
    return 0;
}
