/*
 * A caller of libany4.so through its C ABI alone: no Python, no torch.
 * Test infrastructure (tests/test_gpu_zz_c_caller.py runs it and checks its output
 * against the CPU oracle).
 *
 * Usage: abi_demo IN OUT
 *   IN:  int64 M, N, K, g; uint8 idx[N][K]; uint16 lut[N][16];
 *        uint16 alpha[N][K/g]; uint16 beta[N][K/g]; uint16 x[M][K]
 *   OUT: uint16 w[N][K] (any4_dequant of any4_pack(idx)); uint16 y[M][N]
 *        (any4_gemm on a stream of its own)
 * It also checks that a shape the library rejects comes back as
 * ANY4_E_SHAPE with nothing launched.  Exit status 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "any4.h"

#define HIP_CHECK(e)                                                            \
    do {                                                                        \
        hipError_t err_ = (e);                                                  \
        if (err_ != hipSuccess) {                                               \
            fprintf(stderr, "%s:%d %s\n", __FILE__, __LINE__, hipGetErrorString(err_)); \
            return 2;                                                           \
        }                                                                       \
    } while (0)

#define ANY4_CHECK(e)                                                           \
    do {                                                                        \
        any4_status st_ = (e);                                                  \
        if (st_ != ANY4_OK) {                                                   \
            fprintf(stderr, "%s:%d %s\n", __FILE__, __LINE__, any4_status_string(st_)); \
            return 3;                                                           \
        }                                                                       \
    } while (0)

static int read_all(FILE* f, void* p, size_t n)
{
    return fread(p, 1, n, f) == n ? 0 : 1;
}

int main(int argc, char** argv)
{
    if (argc != 3) {
        fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
        return 1;
    }
    FILE* in = fopen(argv[1], "rb");
    if (!in)
        return 1;
    int64_t hdr[4];
    if (read_all(in, hdr, sizeof hdr))
        return 1;
    const int64_t M = hdr[0], N = hdr[1], K = hdr[2], g = hdr[3], G = K / g;
    const size_t n_idx = (size_t)N * K, n_lut = (size_t)N * 16, n_ab = (size_t)N * G,
                 n_x = (size_t)M * K, n_y = (size_t)M * N;
    uint8_t* idx = malloc(n_idx);
    uint16_t* lut = malloc(2 * n_lut);
    uint16_t* alpha = malloc(2 * n_ab);
    uint16_t* beta = malloc(2 * n_ab);
    uint16_t* x = malloc(2 * n_x);
    uint16_t* w = malloc(2 * n_idx);
    uint16_t* y = malloc(2 * n_y);
    if (!idx || !lut || !alpha || !beta || !x || !w || !y)
        return 1;
    if (read_all(in, idx, n_idx) || read_all(in, lut, 2 * n_lut) ||
        read_all(in, alpha, 2 * n_ab) || read_all(in, beta, 2 * n_ab) || read_all(in, x, 2 * n_x))
        return 1;
    fclose(in);

    const size_t n_packed = any4_packed_bytes(N, K);
    void *d_idx, *d_packed, *d_lut, *d_alpha, *d_beta, *d_x, *d_w, *d_y;
    HIP_CHECK(hipMalloc(&d_idx, n_idx));
    HIP_CHECK(hipMalloc(&d_packed, n_packed));
    HIP_CHECK(hipMalloc(&d_lut, 2 * n_lut));
    HIP_CHECK(hipMalloc(&d_alpha, 2 * n_ab));
    HIP_CHECK(hipMalloc(&d_beta, 2 * n_ab));
    HIP_CHECK(hipMalloc(&d_x, 2 * n_x));
    HIP_CHECK(hipMalloc(&d_w, 2 * n_idx));
    HIP_CHECK(hipMalloc(&d_y, 2 * n_y));
    HIP_CHECK(hipMemcpy(d_idx, idx, n_idx, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(d_lut, lut, 2 * n_lut, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(d_alpha, alpha, 2 * n_ab, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(d_beta, beta, 2 * n_ab, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(d_x, x, 2 * n_x, hipMemcpyHostToDevice));

    hipStream_t s;
    HIP_CHECK(hipStreamCreate(&s));
    const size_t ws = any4_gemm_workspace_size(M, N, K, g);
    if (ws != 0) {
        fprintf(stderr, "unexpected workspace size %zu\n", ws);
        return 4;
    }
    ANY4_CHECK(any4_pack(d_idx, d_packed, N, K, s));
    ANY4_CHECK(any4_dequant(d_packed, d_lut, d_alpha, d_beta, d_w, N, K, g, s));
    ANY4_CHECK(any4_gemm(d_x, d_packed, d_lut, d_alpha, d_beta, d_y, M, N, K, g, NULL, 0, s));
    /* rejected before any launch: K not a multiple of 128 */
    if (any4_gemm(d_x, d_packed, d_lut, d_alpha, d_beta, d_y, M, N, 100, g, NULL, 0, s) !=
        ANY4_E_SHAPE) {
        fprintf(stderr, "K = 100 was not rejected\n");
        return 5;
    }
    HIP_CHECK(hipStreamSynchronize(s));
    HIP_CHECK(hipMemcpy(w, d_w, 2 * n_idx, hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(y, d_y, 2 * n_y, hipMemcpyDeviceToHost));
    HIP_CHECK(hipStreamDestroy(s));
    hipFree(d_idx);
    hipFree(d_packed);
    hipFree(d_lut);
    hipFree(d_alpha);
    hipFree(d_beta);
    hipFree(d_x);
    hipFree(d_w);
    hipFree(d_y);

    FILE* out = fopen(argv[2], "wb");
    if (!out || fwrite(w, 2, n_idx, out) != n_idx || fwrite(y, 2, n_y, out) != n_y)
        return 1;
    fclose(out);
    free(idx);
    free(lut);
    free(alpha);
    free(beta);
    free(x);
    free(w);
    free(y);
    printf("abi_demo ok: M=%lld N=%lld K=%lld g=%lld\n", (long long)M, (long long)N, (long long)K,
           (long long)g);
    return 0;
}
