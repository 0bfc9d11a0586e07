/*
 * scan_from_c.c -- libmamba_scan called from plain C: no Python, no PyTorch.
 *
 * Runs a forward selective scan over a short batch (fp32, an L that is not a whole number of
 * 16-byte vectors) and one decode step continuing from its final state, then writes the inputs
 * and results to a binary file so that they can be checked elsewhere:
 *
 *     scan_from_c OUT_FILE
 *
 * OUT_FILE: int32 Bt, Dn, N, L, then float32 arrays in this order: u, delta, z (Bt, Dn, L);
 * A (Dn, N); B, C (Bt, N, L); D, delta_bias (Dn); out (Bt, Dn, L); last_state (Bt, Dn, N);
 * x1, dt1, z1 (Bt, Dn); B1, C1 (Bt, N); state after the decode step (Bt, Dn, N); out1 (Bt, Dn).
 * Exit status 0 on success; every library call's status is checked, and one deliberately
 * invalid call must be rejected before touching the device.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "mamba_scan.h"

enum { BT = 2, DN = 64, NS = 16, LEN = 37 };

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

/* uniform in [lo, hi) from a 64-bit linear congruential generator (Knuth's MMIX constants) */
static float uniform(float lo, float hi) {
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return lo + (hi - lo) * (float)((rng_state >> 40) * (1.0 / 16777216.0));
}

static mss_tensor_t desc(void* data, int ndim, int64_t s0, int64_t s1, int64_t s2) {
    mss_tensor_t t;
    int64_t shape[4] = {s0, s1, s2, 1};
    t.data = data;
    t.dtype = MSS_F32;
    t.ndim = ndim;
    for (int i = 0; i < 4; ++i) t.shape[i] = i < ndim ? shape[i] : 1;
    t.stride[ndim - 1] = 1;
    for (int i = ndim - 2; i >= 0; --i) t.stride[i] = t.stride[i + 1] * t.shape[i + 1];
    for (int i = ndim; i < 4; ++i) t.stride[i] = 1;
    return t;
}

#define HIP_CHECK(call)                                                          \
    do {                                                                         \
        hipError_t e_ = (call);                                                  \
        if (e_ != hipSuccess) {                                                  \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));    \
            return 1;                                                            \
        }                                                                        \
    } while (0)

#define MSS_CHECK(call)                                                          \
    do {                                                                         \
        int s_ = (call);                                                         \
        if (s_ != MSS_OK) {                                                      \
            fprintf(stderr, "%s failed: %s\n", #call, mss_status_string(s_));    \
            return 1;                                                            \
        }                                                                        \
    } while (0)

struct buf {
    const char* name;
    size_t n;
    float* host;
    float* dev;
};

int main(int argc, char** argv) {
    if (argc != 2) {
        fprintf(stderr, "usage: %s OUT_FILE\n", argv[0]);
        return 2;
    }
    const size_t nx = (size_t)BT * DN * LEN, nbc = (size_t)BT * NS * LEN, ns = (size_t)BT * DN * NS;
    struct buf b[] = {
        {"u", nx, 0, 0},      {"delta", nx, 0, 0},   {"z", nx, 0, 0},      {"A", DN * NS, 0, 0},
        {"B", nbc, 0, 0},     {"C", nbc, 0, 0},      {"D", DN, 0, 0},      {"bias", DN, 0, 0},
        {"out", nx, 0, 0},    {"last", ns, 0, 0},    {"x1", BT * DN, 0, 0}, {"dt1", BT * DN, 0, 0},
        {"z1", BT * DN, 0, 0}, {"B1", BT * NS, 0, 0}, {"C1", BT * NS, 0, 0}, {"state", ns, 0, 0},
        {"out1", BT * DN, 0, 0}};
    enum { I_U, I_DELTA, I_Z, I_A, I_B, I_C, I_D, I_BIAS, I_OUT, I_LAST, I_X1, I_DT1, I_Z1, I_B1, I_C1, I_STATE, I_OUT1, NBUF };
    for (int i = 0; i < NBUF; ++i) {
        b[i].host = (float*)calloc(b[i].n, sizeof(float));
        if (!b[i].host) return 1;
        HIP_CHECK(hipMalloc((void**)&b[i].dev, b[i].n * sizeof(float)));
    }
    /* inputs: u, delta, z, B, C in [-1, 1); A = -(n + 1) scaled per channel (not the power
       form); D in [0.5, 1.5); delta_bias in [-4, -1) */
    for (int i = 0; i < NBUF; ++i) {
        if (i == I_OUT || i == I_LAST || i == I_STATE || i == I_OUT1) continue;
        for (size_t k = 0; k < b[i].n; ++k) b[i].host[k] = uniform(-1.0f, 1.0f);
    }
    for (int d = 0; d < DN; ++d) {
        const float scale = uniform(0.5f, 1.5f);
        for (int n = 0; n < NS; ++n) b[I_A].host[d * NS + n] = -(float)(n + 1) * scale;
        b[I_D].host[d] = uniform(0.5f, 1.5f);
        b[I_BIAS].host[d] = uniform(-4.0f, -1.0f);
    }
    for (int i = 0; i < NBUF; ++i)
        HIP_CHECK(hipMemcpy(b[i].dev, b[i].host, b[i].n * sizeof(float), hipMemcpyHostToDevice));

    mss_tensor_t u = desc(b[I_U].dev, 3, BT, DN, LEN), delta = desc(b[I_DELTA].dev, 3, BT, DN, LEN);
    mss_tensor_t z = desc(b[I_Z].dev, 3, BT, DN, LEN), Am = desc(b[I_A].dev, 2, DN, NS, 1);
    mss_tensor_t Bm = desc(b[I_B].dev, 3, BT, NS, LEN), Cm = desc(b[I_C].dev, 3, BT, NS, LEN);
    mss_tensor_t Dv = desc(b[I_D].dev, 1, DN, 1, 1), bias = desc(b[I_BIAS].dev, 1, DN, 1, 1);
    mss_tensor_t out = desc(b[I_OUT].dev, 3, BT, DN, LEN), last = desc(b[I_LAST].dev, 3, BT, DN, NS);

    /* an invalid call (no u) is rejected before any device work */
    if (mss_selective_scan_fwd(NULL, &delta, &Am, &Bm, &Cm, &Dv, &z, &bias, 1, &out, &last, NULL) !=
        MSS_ERR_NULL_ARG) {
        fprintf(stderr, "a call without u was not rejected\n");
        return 1;
    }
    MSS_CHECK(mss_selective_scan_fwd(&u, &delta, &Am, &Bm, &Cm, &Dv, &z, &bias, 1, &out, &last, NULL));

    /* one decode token continuing from the final state (copied, so both can be written out) */
    HIP_CHECK(hipMemcpy(b[I_STATE].dev, b[I_LAST].dev, ns * sizeof(float), hipMemcpyDeviceToDevice));
    mss_tensor_t state = desc(b[I_STATE].dev, 3, BT, DN, NS);
    mss_tensor_t x1 = desc(b[I_X1].dev, 2, BT, DN, 1), dt1 = desc(b[I_DT1].dev, 2, BT, DN, 1);
    mss_tensor_t z1 = desc(b[I_Z1].dev, 2, BT, DN, 1), out1 = desc(b[I_OUT1].dev, 2, BT, DN, 1);
    mss_tensor_t B1 = desc(b[I_B1].dev, 2, BT, NS, 1), C1 = desc(b[I_C1].dev, 2, BT, NS, 1);
    MSS_CHECK(mss_selective_state_update(&state, &x1, &dt1, &Am, &B1, &C1, &Dv, &z1, &bias, &out1, NULL));
    HIP_CHECK(hipDeviceSynchronize());

    for (int i = 0; i < NBUF; ++i)
        HIP_CHECK(hipMemcpy(b[i].host, b[i].dev, b[i].n * sizeof(float), hipMemcpyDeviceToHost));
    FILE* f = fopen(argv[1], "wb");
    if (!f) return 1;
    const int32_t dims[4] = {BT, DN, NS, LEN};
    int ok = fwrite(dims, sizeof(dims), 1, f) == 1;
    for (int i = 0; i < NBUF; ++i) ok = ok && fwrite(b[i].host, sizeof(float), b[i].n, f) == b[i].n;
    ok = (fclose(f) == 0) && ok;
    for (int i = 0; i < NBUF; ++i) {
        free(b[i].host);
        HIP_CHECK(hipFree(b[i].dev));
    }
    printf("libmamba_scan %d: scan %dx%dx%d and one decode step done\n", mss_version(), BT, DN, LEN);
    return ok ? 0 : 1;
}
