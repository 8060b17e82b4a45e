// abi_roundtrip -- drives libqgemm.so through include/qgemm.h alone (no
// Python, no torch): device buffers from hipMalloc, qg_pack, then
// qg_gemm_int4 or qg_gemm_int2 with the workspace qg_gemm_ws_bytes asks for.
// Test infrastructure for the C ABI; the GPU test compares what it writes
// with the oracle.
//
// usage: abi_roundtrip IN OUT
//   IN : int32 K, N, M, bits; float W[K][N]; uint16 X[M][K] (FP16 bits)
//   OUT: uint32 codes[N][K*bits/32]; uint16 scales[N][K/128]; uint16 zeros[N][K/128];
//        uint16 Y[M][N] (FP16 bits)
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "qgemm.h"

#define HIP_OK(x)                                                                     \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
            return 2;                                                                 \
        }                                                                             \
    } while (0)
#define QG_OK_(x)                                                                           \
    do {                                                                                    \
        int s_ = (x);                                                                       \
        if (s_ != QG_OK) {                                                                  \
            fprintf(stderr, "%s:%d: status %d: %s\n", __FILE__, __LINE__, s_, qg_last_error()); \
            return 3;                                                                       \
        }                                                                                   \
    } while (0)

static bool read_all(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n; }

int main(int argc, char** argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
        return 1;
    }
    FILE* in = fopen(argv[1], "rb");
    if (!in) return 1;
    int32_t hdr[4];
    if (!read_all(in, hdr, sizeof hdr)) return 1;
    const int32_t K = hdr[0], N = hdr[1], M = hdr[2], bits = hdr[3];
    if (K <= 0 || N <= 0 || M <= 0 || K % 128 || N % 8 || (bits != 4 && bits != 2)) return 1;
    std::vector<float> W((size_t)K * N);
    std::vector<uint16_t> X((size_t)M * K);
    if (!read_all(in, W.data(), W.size() * 4) || !read_all(in, X.data(), X.size() * 2)) return 1;
    fclose(in);

    const size_t ncodes = (size_t)N * K * bits / 32, nsz = (size_t)N * (K / 128);
    float* dW;
    uint32_t* dcodes;
    qg_half *dscales, *dzeros, *dX, *dY;
    HIP_OK(hipMalloc((void**)&dW, W.size() * 4));
    HIP_OK(hipMalloc((void**)&dcodes, ncodes * 4));
    HIP_OK(hipMalloc((void**)&dscales, nsz * 2));
    HIP_OK(hipMalloc((void**)&dzeros, nsz * 2));
    HIP_OK(hipMalloc((void**)&dX, X.size() * 2));
    HIP_OK(hipMalloc((void**)&dY, (size_t)M * N * 2));
    HIP_OK(hipMemcpy(dW, W.data(), W.size() * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dX, X.data(), X.size() * 2, hipMemcpyHostToDevice));

    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    QG_OK_(qg_pack(dW, N, K, N, bits, 128, dcodes, dscales, dzeros, s));
    const qg_weight w = {bits, K, N, 128, dcodes, dscales, dzeros};
    const size_t ws_bytes = qg_gemm_ws_bytes(&w, M);
    void* ws = nullptr;
    if (ws_bytes) HIP_OK(hipMalloc(&ws, ws_bytes));
    if (bits == 4)
        QG_OK_(qg_gemm_int4(dX, K, &w, dY, N, M, ws, ws_bytes, s));
    else
        QG_OK_(qg_gemm_int2(dX, K, &w, dY, N, M, ws, ws_bytes, s));
    HIP_OK(hipStreamSynchronize(s));

    std::vector<uint32_t> codes(ncodes);
    std::vector<uint16_t> scales(nsz), zeros(nsz), Y((size_t)M * N);
    HIP_OK(hipMemcpy(codes.data(), dcodes, ncodes * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(scales.data(), dscales, nsz * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(zeros.data(), dzeros, nsz * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(Y.data(), dY, Y.size() * 2, hipMemcpyDeviceToHost));
    FILE* out = fopen(argv[2], "wb");
    if (!out) return 1;
    fwrite(codes.data(), 4, codes.size(), out);
    fwrite(scales.data(), 2, nsz, out);
    fwrite(zeros.data(), 2, nsz, out);
    fwrite(Y.data(), 2, Y.size(), out);
    fclose(out);

    qg_release_cache();
    (void)hipStreamDestroy(s);
    if (ws) (void)hipFree(ws);
    (void)hipFree(dW);
    (void)hipFree(dcodes);
    (void)hipFree(dscales);
    (void)hipFree(dzeros);
    (void)hipFree(dX);
    (void)hipFree(dY);
    return 0;
}
