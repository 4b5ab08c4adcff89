// A C++ caller of libfp8fg that uses nothing but include/fp8fg.h and the HIP runtime: no Python, no torch.
// It allocates its own device buffers (the library allocates nothing), runs one training-step Linear on a
// small shape - X [256, 512] and W [384, 512] quantized in one launch (X in both tilings), dY [256, 384]
// quantized in both tilings, Fprop (BF16 out), Dgrad (FP32 out), Wgrad (FP32 out), all with FP32 scales, on
// one stream - and writes every code, scale and output to one binary file, in that order. The inputs come
// from a fixed integer generator whose bf16 bit patterns tests/test_gpu_c_consumer.py reproduces.
//
// usage: c_consumer <output file>      exit status 0 on success; a failed call prints its status and exits 1
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "fp8fg.h"

namespace {

constexpr int64_t M = 256, N = 384, K = 512;   // tokens, output channels, input channels

// bf16 bit patterns: a 64-bit LCG (Knuth's MMIX constants), sign from bit 63, a biased exponent in
// [e0, e0 + 8) from bits 40..42, the 7 mantissa bits from bits 33..39
std::vector<uint16_t> bf16_inputs(uint64_t seed, int64_t count, int e0) {
    std::vector<uint16_t> v(count);
    uint64_t s = seed;
    for (int64_t i = 0; i < count; i++) {
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        const uint32_t sign = (uint32_t)(s >> 63);
        const uint32_t exp = (uint32_t)e0 + (uint32_t)((s >> 40) & 7);
        const uint32_t man = (uint32_t)((s >> 33) & 0x7F);
        v[i] = (uint16_t)((sign << 15) | (exp << 7) | man);
    }
    return v;
}

#define HIP_OK(x)                                                                             \
    do {                                                                                      \
        hipError_t e_ = (x);                                                                  \
        if (e_ != hipSuccess) {                                                               \
            std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            std::exit(1);                                                                     \
        }                                                                                     \
    } while (0)

void fg_ok(fg_status st, const char* what) {
    if (st != FG_OK) {
        std::fprintf(stderr, "%s: %s (HIP error %d)\n", what, fg_status_string(st), fg_last_hip_error());
        std::exit(1);
    }
}

template <class T>
T* dev_alloc(int64_t count) {
    void* p = nullptr;
    HIP_OK(hipMalloc(&p, (size_t)count * sizeof(T)));
    return static_cast<T*>(p);
}

template <class T>
void dump(FILE* f, const T* d, int64_t count) {
    std::vector<T> h(count);
    HIP_OK(hipMemcpy(h.data(), d, (size_t)count * sizeof(T), hipMemcpyDeviceToHost));
    if (std::fwrite(h.data(), sizeof(T), (size_t)count, f) != (size_t)count) {
        std::fprintf(stderr, "short write\n");
        std::exit(1);
    }
}

}  // namespace

int main(int argc, char** argv) {
    if (argc != 2) {
        std::fprintf(stderr, "usage: %s <output file>\n", argv[0]);
        return 2;
    }
    const std::vector<uint16_t> hx = bf16_inputs(1, M * K, 120);    // |x| in [2^-7, 2)
    const std::vector<uint16_t> hw = bf16_inputs(2, N * K, 115);    // |w| in [2^-12, 2^-3)
    const std::vector<uint16_t> hdy = bf16_inputs(3, M * N, 110);   // |dy| in [2^-17, 2^-8)

    uint16_t* x = dev_alloc<uint16_t>(M * K);
    uint16_t* w = dev_alloc<uint16_t>(N * K);
    uint16_t* dy = dev_alloc<uint16_t>(M * N);
    HIP_OK(hipMemcpy(x, hx.data(), hx.size() * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(w, hw.data(), hw.size() * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dy, hdy.data(), hdy.size() * 2, hipMemcpyHostToDevice));

    uint8_t* xq = dev_alloc<uint8_t>(M * K);            // X, 1x128 tiles along the channels
    float* sx = dev_alloc<float>(K / 128 * M);
    uint8_t* xtq = dev_alloc<uint8_t>(K * M);           // X^T, 1x128 tiles along the tokens
    float* sxt = dev_alloc<float>(M / 128 * K);
    uint8_t* wq = dev_alloc<uint8_t>(N * K);
    float* sw = dev_alloc<float>(N / 128 * (K / 128));
    uint8_t* dyq = dev_alloc<uint8_t>(M * N);
    float* sdy = dev_alloc<float>(N / 128 * M);
    uint8_t* dytq = dev_alloc<uint8_t>(N * M);
    float* sdyt = dev_alloc<float>(M / 128 * N);
    uint16_t* y = dev_alloc<uint16_t>(M * N);           // BF16
    float* dx = dev_alloc<float>(M * K);
    float* dw = dev_alloc<float>(N * K);

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    fg_ok(fg_quantize_fprop_operands(x, M, K, w, N, K, K, FG_SCALE_FP32, xq, sx, xtq, sxt, wq, sw, stream),
          "fg_quantize_fprop_operands");
    fg_ok(fg_fp8_gemm_fprop(xq, sx, wq, sw, M, N, K, y, FG_OUT_BF16, FG_SCALE_FP32, stream), "fg_fp8_gemm_fprop");
    fg_ok(fg_quantize_act_1x128_both(dy, M, N, N, FG_SCALE_FP32, dyq, sdy, dytq, sdyt, stream),
          "fg_quantize_act_1x128_both");
    fg_ok(fg_fp8_gemm_dgrad(dyq, sdy, wq, sw, M, N, K, dx, FG_OUT_F32, FG_SCALE_FP32, stream), "fg_fp8_gemm_dgrad");
    fg_ok(fg_fp8_gemm_wgrad(dytq, sdyt, xtq, sxt, M, N, K, dw, 0, FG_SCALE_FP32, stream), "fg_fp8_gemm_wgrad");
    // a rejected call launches nothing and says why: Fprop with K not a multiple of 128
    if (fg_fp8_gemm_fprop(xq, sx, wq, sw, M, N, K - 1, y, FG_OUT_BF16, FG_SCALE_FP32, stream) !=
        FG_ERR_UNSUPPORTED_SHAPE) {
        std::fprintf(stderr, "K %% 128 != 0 was not rejected\n");
        return 1;
    }
    HIP_OK(hipStreamSynchronize(stream));

    FILE* f = std::fopen(argv[1], "wb");
    if (!f) {
        std::fprintf(stderr, "cannot open %s\n", argv[1]);
        return 1;
    }
    dump(f, xq, M * K);
    dump(f, sx, K / 128 * M);
    dump(f, xtq, K * M);
    dump(f, sxt, M / 128 * K);
    dump(f, wq, N * K);
    dump(f, sw, N / 128 * (K / 128));
    dump(f, dyq, M * N);
    dump(f, sdy, N / 128 * M);
    dump(f, dytq, N * M);
    dump(f, sdyt, M / 128 * N);
    dump(f, y, M * N);
    dump(f, dx, M * K);
    dump(f, dw, N * K);
    std::fclose(f);

    for (void* p : {(void*)x, (void*)w, (void*)dy, (void*)xq, (void*)sx, (void*)xtq, (void*)sxt, (void*)wq, (void*)sw,
                    (void*)dyq, (void*)sdy, (void*)dytq, (void*)sdyt, (void*)y, (void*)dx, (void*)dw})
        HIP_OK(hipFree(p));
    HIP_OK(hipStreamDestroy(stream));
    std::printf("c_consumer done\n");
    return 0;
}
