/*
 * A plain C (C99) caller of libsq: device memory from the HIP runtime's C API,
 * no Python, no C++.  One pool of two slots x three heads (4-bit, FP16 pivot,
 * FP32 state), d = 128.  Checks closed forms of the step through the C ABI:
 *   - alpha = 1, beta = 1, k = e_m: row m of the state becomes v (write into
 *     a row of the gated delta rule), other rows keep their values;
 *   - the readout o = S'^T q with q = e_m is v for the FP32 head;
 *   - sq_check_slots flags a repeated slot;
 *   - with scale_slot_stride = H every slot has its own factors: a 4-bit
 *     state stored with step 1/4 in slot 1 and 1/8 in slot 0 loads back as
 *     rne(x / step) * step of its own slot;
 *   - a NaN stored sets the pool's sticky flag (code 0 is stored), which
 *     sq_pool_last_device_error reads and clears.
 * Exit status 0 on success; prints the failing check otherwise.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../include/sq.h"

#define D 128
#define H 3
#define SLOTS 2

#define CHECK(cond, msg)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            fprintf(stderr, "abi_smoke: %s\n", msg);      \
            return 1;                                     \
        }                                                 \
    } while (0)

int main(void)
{
    const uint8_t bits[H] = {4, 16, 32};
    uint64_t nbytes = sq_pool_bytes(SLOTS, H, D, D, bits);
    CHECK(nbytes == (uint64_t)SLOTS * (8192 + 32768 + 65536), "pool size");

    float *h_r = malloc(sizeof(float) * H * D), *h_c = malloc(sizeof(float) * H * D);
    float *h_S = malloc(sizeof(float) * SLOTS * H * D * D), *h_out = malloc(sizeof(float) * SLOTS * H * D * D);
    for (int i = 0; i < H * D; i++) {
        h_r[i] = 1.0f;
        h_c[i] = 0.125f; /* 4-bit step 1/8: codes -7..7 cover [-0.875, 0.875] */
    }
    for (long i = 0; i < (long)SLOTS * H * D * D; i++) h_S[i] = (float)((i * 37 % 15) - 7) * 0.125f;

    void *state, *r, *c, *S, *out, *q, *k, *v, *alpha, *beta, *o, *ids, *flag;
    CHECK(hipMalloc(&state, nbytes) == hipSuccess, "hipMalloc state");
    CHECK(hipMalloc(&r, sizeof(float) * H * D) == hipSuccess, "hipMalloc r");
    CHECK(hipMalloc(&c, sizeof(float) * H * D) == hipSuccess, "hipMalloc c");
    CHECK(hipMalloc(&S, sizeof(float) * SLOTS * H * D * D) == hipSuccess, "hipMalloc S");
    CHECK(hipMalloc(&out, sizeof(float) * SLOTS * H * D * D) == hipSuccess, "hipMalloc out");
    CHECK(hipMalloc(&q, sizeof(float) * SLOTS * H * D) == hipSuccess, "hipMalloc q");
    CHECK(hipMalloc(&k, sizeof(float) * SLOTS * H * D) == hipSuccess, "hipMalloc k");
    CHECK(hipMalloc(&v, sizeof(float) * SLOTS * H * D) == hipSuccess, "hipMalloc v");
    CHECK(hipMalloc(&alpha, sizeof(float) * SLOTS * H) == hipSuccess, "hipMalloc alpha");
    CHECK(hipMalloc(&beta, sizeof(float) * SLOTS * H) == hipSuccess, "hipMalloc beta");
    CHECK(hipMalloc(&o, sizeof(float) * SLOTS * H * D) == hipSuccess, "hipMalloc o");
    CHECK(hipMalloc(&ids, sizeof(int32_t) * 3) == hipSuccess, "hipMalloc ids");
    CHECK(hipMalloc(&flag, sizeof(int32_t)) == hipSuccess, "hipMalloc flag");

    hipMemcpy(r, h_r, sizeof(float) * H * D, hipMemcpyHostToDevice);
    hipMemcpy(c, h_c, sizeof(float) * H * D, hipMemcpyHostToDevice);
    hipMemcpy(S, h_S, sizeof(float) * SLOTS * H * D * D, hipMemcpyHostToDevice);

    sq_pool_desc desc;
    memset(&desc, 0, sizeof(desc));
    desc.n_slots = SLOTS;
    desc.n_heads = H;
    desc.d_k = D;
    desc.d_v = D;
    desc.head_bits = bits;
    desc.row_scale = (const float *)r;
    desc.col_scale = (const float *)c;
    desc.state = state;
    desc.state_bytes = nbytes;
    sq_pool *pool = NULL;
    CHECK(sq_pool_alloc(&desc, &pool) == SQ_OK && pool, "sq_pool_alloc");

    const int32_t h_ids[3] = {1, 0, 1};
    hipMemcpy(ids, h_ids, sizeof(h_ids), hipMemcpyHostToDevice);
    CHECK(sq_pool_store(pool, (const int32_t *)ids, SLOTS, (const float *)S, NULL) == SQ_OK, "store");

    /* one step: k = e_m, q = e_m, alpha = beta = 1, v_j = (j % 13 - 6) / 8 */
    const int m = 37;
    float *h_q = calloc((size_t)SLOTS * H * D, sizeof(float)), *h_v = malloc(sizeof(float) * SLOTS * H * D);
    float h_ab[SLOTS * H];
    for (int n = 0; n < SLOTS * H; n++) {
        h_q[n * D + m] = 1.0f;
        h_ab[n] = 1.0f;
        for (int j = 0; j < D; j++) h_v[n * D + j] = (float)(j % 13 - 6) * 0.125f;
    }
    hipMemcpy(q, h_q, sizeof(float) * SLOTS * H * D, hipMemcpyHostToDevice);
    hipMemcpy(k, h_q, sizeof(float) * SLOTS * H * D, hipMemcpyHostToDevice);
    hipMemcpy(v, h_v, sizeof(float) * SLOTS * H * D, hipMemcpyHostToDevice);
    hipMemcpy(alpha, h_ab, sizeof(h_ab), hipMemcpyHostToDevice);
    hipMemcpy(beta, h_ab, sizeof(h_ab), hipMemcpyHostToDevice);
    CHECK(sq_decode_step(pool, (const int32_t *)ids, SLOTS, q, k, v, SQ_F32, (const float *)alpha,
                         (const float *)beta, (float *)o, NULL) == SQ_OK, "decode step");
    CHECK(sq_pool_load(pool, (const int32_t *)ids, SLOTS, (float *)out, NULL) == SQ_OK, "load");
    CHECK(hipDeviceSynchronize() == hipSuccess, "synchronize");
    hipMemcpy(h_out, out, sizeof(float) * SLOTS * H * D * D, hipMemcpyDeviceToHost);
    float *h_o = malloc(sizeof(float) * SLOTS * H * D);
    hipMemcpy(h_o, o, sizeof(float) * SLOTS * H * D, hipMemcpyDeviceToHost);

    for (int n = 0; n < SLOTS; n++)
        for (int h = 0; h < H; h++) {
            const float *before = h_S + ((long)n * H + h) * D * D;
            const float *after = h_out + ((long)n * H + h) * D * D;
            for (int i = 0; i < D; i++)
                for (int j = 0; j < D; j++) {
                    const float want = (i == m) ? h_v[(n * H + h) * D + j] : before[i * D + j];
                    if (after[i * D + j] != want) {
                        fprintf(stderr, "abi_smoke: state (%d, %d) element (%d, %d): %g, want %g\n",
                                n, h, i, j, after[i * D + j], want);
                        return 1;
                    }
                }
            for (int j = 0; j < D; j++)
                CHECK(fabsf(h_o[(n * H + h) * D + j] - h_v[(n * H + h) * D + j]) <= 1e-6f, "readout o = v");
        }

    /* a repeated slot is flagged */
    CHECK(sq_check_slots(pool, (const int32_t *)ids, 3, (int32_t *)flag, NULL) == SQ_OK, "check call");
    int32_t h_flag = -1;
    hipMemcpy(&h_flag, flag, sizeof(h_flag), hipMemcpyDeviceToHost);
    CHECK(h_flag == 2, "repeated slot flagged");
    CHECK(sq_check_slots(pool, (const int32_t *)ids, 2, (int32_t *)flag, NULL) == SQ_OK, "check call");
    hipMemcpy(&h_flag, flag, sizeof(h_flag), hipMemcpyDeviceToHost);
    CHECK(h_flag == 0, "valid batch");

    CHECK(sq_decode_step(pool, (const int32_t *)ids, SLOTS, q, k, v, 7, (const float *)alpha,
                         (const float *)beta, NULL, NULL) == SQ_ERR_INVALID, "bad dtype rejected");
    CHECK(sq_pool_last_device_error(pool, NULL) == SQ_OK, "no non-finite value met");
    sq_pool_free(pool);

    /* per-slot factors: vector p * H + h holds the factors of slot p, head h */
    float *h_r2 = malloc(sizeof(float) * SLOTS * H * D), *h_c2 = malloc(sizeof(float) * SLOTS * H * D);
    for (int p = 0; p < SLOTS; p++)
        for (int i = 0; i < H * D; i++) {
            h_r2[p * H * D + i] = 1.0f;
            h_c2[p * H * D + i] = p == 1 ? 0.25f : 0.125f;
        }
    void *r2, *c2, *state2, *ids2;
    CHECK(hipMalloc(&r2, sizeof(float) * SLOTS * H * D) == hipSuccess, "hipMalloc r2");
    CHECK(hipMalloc(&c2, sizeof(float) * SLOTS * H * D) == hipSuccess, "hipMalloc c2");
    CHECK(hipMalloc(&state2, nbytes) == hipSuccess, "hipMalloc state2");
    CHECK(hipMalloc(&ids2, sizeof(int32_t) * SLOTS) == hipSuccess, "hipMalloc ids2");
    hipMemcpy(r2, h_r2, sizeof(float) * SLOTS * H * D, hipMemcpyHostToDevice);
    hipMemcpy(c2, h_c2, sizeof(float) * SLOTS * H * D, hipMemcpyHostToDevice);
    const int32_t h_ids2[SLOTS] = {0, 1};
    hipMemcpy(ids2, h_ids2, sizeof(h_ids2), hipMemcpyHostToDevice);
    desc.row_scale = (const float *)r2;
    desc.col_scale = (const float *)c2;
    desc.scale_slot_stride = H;
    desc.state = state2;
    sq_pool *pool2 = NULL;
    CHECK(sq_pool_alloc(&desc, &pool2) == SQ_OK && pool2, "sq_pool_alloc with a slot stride");
    desc.scale_slot_stride = H - 1;
    sq_pool *bad = NULL;
    CHECK(sq_pool_alloc(&desc, &bad) == SQ_ERR_INVALID && !bad, "slot stride below n_heads rejected");
    CHECK(sq_pool_store(pool2, (const int32_t *)ids2, SLOTS, (const float *)S, NULL) == SQ_OK, "store 2");
    CHECK(sq_pool_load(pool2, (const int32_t *)ids2, SLOTS, (float *)out, NULL) == SQ_OK, "load 2");
    CHECK(hipDeviceSynchronize() == hipSuccess, "synchronize 2");
    hipMemcpy(h_out, out, sizeof(float) * SLOTS * H * D * D, hipMemcpyDeviceToHost);
    for (int n = 0; n < SLOTS; n++)
        for (int h = 0; h < H; h++)
            for (long e = 0; e < (long)D * D; e++) {
                const float x = h_S[((long)n * H + h) * D * D + e];
                const float step = n == 1 ? 0.25f : 0.125f;
                const float want = h == 0 ? nearbyintf(x / step) * step : x; /* |x / step| <= 7 */
                if (h_out[((long)n * H + h) * D * D + e] != want) {
                    fprintf(stderr, "abi_smoke: slot %d head %d element %ld: %g, want %g\n", n, h, e,
                            h_out[((long)n * H + h) * D * D + e], want);
                    return 1;
                }
            }
    CHECK(sq_pool_last_device_error(pool2, NULL) == SQ_OK, "finite store leaves the flag clear");

    /* a NaN stored: code 0, and the flag is set until read */
    h_S[5] = NAN;
    hipMemcpy(S, h_S, sizeof(float) * D * D, hipMemcpyHostToDevice);
    CHECK(sq_pool_store(pool2, (const int32_t *)ids2, 1, (const float *)S, NULL) == SQ_OK, "store NaN");
    CHECK(sq_pool_last_device_error(pool2, NULL) == SQ_ERR_DEVICE, "NaN sets the flag");
    CHECK(sq_pool_last_device_error(pool2, NULL) == SQ_OK, "the flag is cleared once read");
    CHECK(sq_pool_load(pool2, (const int32_t *)ids2, 1, (float *)out, NULL) == SQ_OK, "load 3");
    CHECK(hipDeviceSynchronize() == hipSuccess, "synchronize 3");
    hipMemcpy(h_out, out, sizeof(float) * D * D, hipMemcpyDeviceToHost);
    CHECK(h_out[5] == 0.0f && h_out[4] == h_S[4], "a NaN stores code 0");
    sq_pool_free(pool2);
    printf("abi_smoke ok\n");
    return 0;
}
