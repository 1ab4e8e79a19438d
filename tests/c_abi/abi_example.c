/*
 * abi_example.c -- a plain C caller of libmi355norm.so (no Python, no torch):
 * reads an fp32 matrix from a file, runs ln_fwd, rms_fwd and ln_bwd on the
 * device through the C ABI of include/mi355norm.h, and writes the results
 * to a file for the test that compares them with the oracle.
 *
 * usage: abi_example <in.bin> <out.bin>
 *   in.bin : int64 M, int64 N, then fp32 x[M*N], gamma[N], beta[N], dy[M*N]
 *   out.bin: fp32 y_ln[M*N], mean[M], rstd_ln[M], y_rms[M*N], rstd_rms[M],
 *            dx[M*N], dgamma[N], dbeta[N]
 * Exit status 0 on success; any library status or HIP error is printed and
 * ends the program with status 1.
 */
#include <stdio.h>
#include <stdlib.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "mi355norm.h"

#define HIP_CHECK(call)                                                           \
    do {                                                                          \
        hipError_t e_ = (call);                                                   \
        if (e_ != hipSuccess) {                                                   \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));     \
            return 1;                                                             \
        }                                                                         \
    } while (0)

#define NORM_CHECK(call)                                                          \
    do {                                                                          \
        int s_ = (call);                                                          \
        if (s_ != NORM_OK) {                                                      \
            fprintf(stderr, "%s: %s [%s]\n", #call, norm_status_str(s_), norm_last_error()); \
            return 1;                                                             \
        }                                                                         \
    } while (0)

static void* dev_copy(const void* host, size_t bytes) {
    void* d = NULL;
    if (hipMalloc(&d, bytes) != hipSuccess) return NULL;
    if (host && hipMemcpy(d, host, bytes, hipMemcpyHostToDevice) != hipSuccess) return NULL;
    return d;
}

int main(int argc, char** argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s in.bin out.bin\n", argv[0]);
        return 1;
    }
    FILE* f = fopen(argv[1], "rb");
    if (!f) return 1;
    int64_t MN[2];
    if (fread(MN, sizeof MN, 1, f) != 1) return 1;
    const int64_t M = MN[0], N = MN[1];
    const size_t mat = (size_t)(M * N), row = (size_t)N;
    float* h = (float*)malloc(sizeof(float) * (2 * mat + 2 * row));
    if (!h || fread(h, sizeof(float), 2 * mat + 2 * row, f) != 2 * mat + 2 * row) return 1;
    fclose(f);
    const float *x = h, *gamma = h + mat, *beta = h + mat + row, *dy = h + mat + 2 * row;

    hipStream_t stream;
    HIP_CHECK(hipStreamCreate(&stream));
    void* dx_in = dev_copy(x, sizeof(float) * mat);
    void* dg = dev_copy(gamma, sizeof(float) * row);
    void* db = dev_copy(beta, sizeof(float) * row);
    void* ddy = dev_copy(dy, sizeof(float) * mat);
    void* dy_ln = dev_copy(NULL, sizeof(float) * mat);
    void* dy_rms = dev_copy(NULL, sizeof(float) * mat);
    void* ddx = dev_copy(NULL, sizeof(float) * mat);
    float* dmean = (float*)dev_copy(NULL, sizeof(float) * M);
    float* drstd = (float*)dev_copy(NULL, sizeof(float) * M);
    float* drstd2 = (float*)dev_copy(NULL, sizeof(float) * M);
    float* ddg = (float*)dev_copy(NULL, sizeof(float) * row);
    float* ddb = (float*)dev_copy(NULL, sizeof(float) * row);
    if (!dx_in || !dg || !db || !ddy || !dy_ln || !dy_rms || !ddx || !dmean || !drstd || !drstd2 || !ddg || !ddb) {
        fprintf(stderr, "hipMalloc / hipMemcpy failed\n");
        return 1;
    }

    NORM_CHECK(ln_fwd(dx_in, dg, db, dy_ln, dmean, drstd, M, N, 1e-5f, NORM_F32, stream));
    NORM_CHECK(rms_fwd(dx_in, dg, NULL, dy_rms, NULL, drstd2, M, N, 1e-6f, NORM_F32, stream));
    NORM_CHECK(ln_bwd(ddy, dx_in, dg, dmean, drstd, ddx, ddg, ddb, M, N, NORM_F32, stream));
    /* a rejected call leaves everything untouched and says why */
    if (rms_fwd(dx_in, dg, db, dy_rms, NULL, drstd2, M, N, 1e-6f, NORM_F32, stream) != NORM_ERR_BAD_ARG) {
        fprintf(stderr, "rms_fwd with a beta was not rejected\n");
        return 1;
    }
    HIP_CHECK(hipStreamSynchronize(stream));

    float* out = (float*)malloc(sizeof(float) * (3 * mat + 3 * (size_t)M + 2 * row));
    if (!out) return 1;
    float* p = out;
    HIP_CHECK(hipMemcpy(p, dy_ln, sizeof(float) * mat, hipMemcpyDeviceToHost)); p += mat;
    HIP_CHECK(hipMemcpy(p, dmean, sizeof(float) * M, hipMemcpyDeviceToHost)); p += M;
    HIP_CHECK(hipMemcpy(p, drstd, sizeof(float) * M, hipMemcpyDeviceToHost)); p += M;
    HIP_CHECK(hipMemcpy(p, dy_rms, sizeof(float) * mat, hipMemcpyDeviceToHost)); p += mat;
    HIP_CHECK(hipMemcpy(p, drstd2, sizeof(float) * M, hipMemcpyDeviceToHost)); p += M;
    HIP_CHECK(hipMemcpy(p, ddx, sizeof(float) * mat, hipMemcpyDeviceToHost)); p += mat;
    HIP_CHECK(hipMemcpy(p, ddg, sizeof(float) * row, hipMemcpyDeviceToHost)); p += row;
    HIP_CHECK(hipMemcpy(p, ddb, sizeof(float) * row, hipMemcpyDeviceToHost)); p += row;
    FILE* o = fopen(argv[2], "wb");
    if (!o || fwrite(out, sizeof(float), (size_t)(p - out), o) != (size_t)(p - out)) return 1;
    fclose(o);
    hipFree(dx_in); hipFree(dg); hipFree(db); hipFree(ddy); hipFree(dy_ln); hipFree(dy_rms); hipFree(ddx);
    hipFree(dmean); hipFree(drstd); hipFree(drstd2); hipFree(ddg); hipFree(ddb);
    HIP_CHECK(hipStreamDestroy(stream));
    free(h);
    free(out);
    printf("abi_example: M=%lld N=%lld ok\n", (long long)M, (long long)N);
    return 0;
}
