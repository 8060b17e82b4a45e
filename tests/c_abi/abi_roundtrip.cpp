// abi_roundtrip -- drives libqgemm.so through include/qgemm.h alone (no
// Python, no torch): device buffers from hipMalloc, qg_pack, then
// qg_gemm_int4 or qg_gemm_int2 with the workspace qg_gemm_ws_bytes asks for;
// or, with --loop, a whole block: qg_pack of the four projections (INT4),
// qg_requant_4to2 of each when bits == 2, and qg_loop_range with the scratch
// qg_loop_scratch_bytes asks for.  Test infrastructure for the C ABI; the GPU
// test compares what it writes with the oracle.
//
// usage: abi_roundtrip IN OUT
//   IN : int32 K, N, M, bits; float W[K][N]; uint16 X[M][K] (FP16 bits)
//   OUT: uint32 codes[N][K*bits/32]; uint16 scales[N][K/128]; uint16 zeros[N][K/128];
//        uint16 Y[M][N] (FP16 bits)
// usage: abi_roundtrip --loop IN OUT
//   IN : int32 D, F, M, bits, L0, L1; float Wqkv[D][3D], Wout[D][D], Wup[D][F],
//        Wdown[F][D]; float h[M][D]
//   OUT: float h[M][D] after iterations [L0, L1)
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

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

// Device allocations of the loop mode, freed together at exit.
struct DeviceBuffers {
    std::vector<void*> p;
    ~DeviceBuffers() {
        for (void* q : p) (void)hipFree(q);
    }
    template <class T>
    hipError_t alloc(T** out, size_t bytes) {
        hipError_t e = hipMalloc((void**)out, bytes);
        if (e == hipSuccess) p.push_back(*out);
        return e;
    }
};

static int run_loop(const char* in_path, const char* out_path) {
    FILE* in = fopen(in_path, "rb");
    if (!in) return 1;
    int32_t hdr[6];
    if (!read_all(in, hdr, sizeof hdr)) return 1;
    const int32_t D = hdr[0], F = hdr[1], M = hdr[2], bits = hdr[3], L0 = hdr[4], L1 = hdr[5];
    if (D <= 0 || F <= 0 || M <= 0 || D % 128 || F % 128 || (bits != 4 && bits != 2) || L0 < 0 ||
        L1 < L0)
        return 1;
    const int32_t shape[4][2] = {{D, 3 * D}, {D, D}, {D, F}, {F, D}};  // qkv, out, up, down
    std::vector<float> W[4];
    for (int i = 0; i < 4; ++i) {
        W[i].resize((size_t)shape[i][0] * shape[i][1]);
        if (!read_all(in, W[i].data(), W[i].size() * 4)) return 1;
    }
    std::vector<float> h((size_t)M * D);
    if (!read_all(in, h.data(), h.size() * 4)) return 1;
    fclose(in);

    DeviceBuffers dev;
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    qg_weight w[4];
    for (int i = 0; i < 4; ++i) {
        const int32_t K = shape[i][0], N = shape[i][1];
        const size_t nsz = (size_t)N * (K / 128);
        float* dW;
        uint32_t* codes;
        qg_half *scales, *zeros;
        HIP_OK(dev.alloc(&dW, W[i].size() * 4));
        HIP_OK(dev.alloc(&codes, (size_t)N * K / 8 * 4));
        HIP_OK(dev.alloc(&scales, nsz * 2));
        HIP_OK(dev.alloc(&zeros, nsz * 2));
        HIP_OK(hipMemcpy(dW, W[i].data(), W[i].size() * 4, hipMemcpyHostToDevice));
        QG_OK_(qg_pack(dW, N, K, N, 4, 128, codes, scales, zeros, s));
        w[i] = {4, K, N, 128, codes, scales, zeros};
        if (bits == 2) {
            // the tier switch in place, INT2 rows kept at the INT4 row stride
            // (K/8 words): the pages' in-place form, through the ldc field
            const qg_weight w2 = {2, K, N, 128, codes, scales, zeros, (int64_t)K / 8};
            QG_OK_(qg_requant_4to2(&w[i], &w2, s));
            w[i] = w2;
        }
    }
    qg_block blk;
    memset(&blk, 0, sizeof blk);  // gate.codes == NULL: the four-projection block
    blk.D = D;
    blk.F = F;
    blk.qkv = w[0];
    blk.out = w[1];
    blk.up = w[2];
    blk.down = w[3];
    const size_t scratch_bytes = qg_loop_scratch_bytes(&blk, M);
    void* scratch;
    float* dh;
    HIP_OK(dev.alloc(&scratch, scratch_bytes));
    HIP_OK(dev.alloc(&dh, h.size() * 4));
    HIP_OK(hipMemcpy(dh, h.data(), h.size() * 4, hipMemcpyHostToDevice));
    QG_OK_(qg_loop_range(&blk, dh, M, L0, L1, scratch, scratch_bytes, s));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(h.data(), dh, h.size() * 4, hipMemcpyDeviceToHost));
    FILE* out = fopen(out_path, "wb");
    if (!out) return 1;
    fwrite(h.data(), 4, h.size(), out);
    fclose(out);
    qg_release_cache();
    (void)hipStreamDestroy(s);
    return 0;
}

int main(int argc, char** argv) {
    if (argc == 4 && strcmp(argv[1], "--loop") == 0) return run_loop(argv[2], argv[3]);
    if (argc != 3) {
        fprintf(stderr, "usage: %s [--loop] IN OUT\n", argv[0]);
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
