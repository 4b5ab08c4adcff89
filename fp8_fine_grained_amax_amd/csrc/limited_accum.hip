// Fprop without promotion, accumulating in a register of limited precision: the accuracy study.
//
// "5 Ways You can get More Deepseek While Spending Less" and the why-be.why-be.co.kr page report a
// maximum relative error of nearly 2% at a contraction length of 4096 when an FP8 GEMM accumulates inside
// the tensor core with its limited accumulation width, and remove it by promoting partial sums to FP32
// every 128 elements. This kernel emulates the unpromoted accumulation on gfx950 for comparison with the
// product's promoted GEMMs: every 32-element chunk of the contraction is one v_mfma_f32_16x16x32_fp8_fp8
// (the chunk sum of decoded code products), scaled by the chunk's tile and block scales, and added to an
// FP32 accumulator that is truncated to `bits` explicit mantissa bits after every addition. It is written
// for clarity, not speed: one wave per 16x16 output tile, operands straight from global memory.
#include "common.h"

namespace {

__global__ __launch_bounds__(64) void fg_fprop_limited_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ sx,
                                                              const uint8_t* __restrict__ wq, const float* __restrict__ sw,
                                                              int64_t M, int64_t N, int64_t K, int bits,
                                                              float* __restrict__ y) {
    const int lane = threadIdx.x;
    const int64_t n_tiles = (N + 15) / 16;
    const int64_t m0 = (int64_t)(blockIdx.x / n_tiles) * 16, n0 = (int64_t)(blockIdx.x % n_tiles) * 16;
    // operand rows held by this lane: x row m (lane % 16), w row n (lane % 16); K bytes 8*(lane/16) .. +7 of
    // each 32-element chunk. Rows past the end re-read the last row (their outputs are not stored).
    const int64_t ma = m0 + (lane & 15) < M ? m0 + (lane & 15) : M - 1;
    const int64_t nb = n0 + (lane & 15) < N ? n0 + (lane & 15) : N - 1;
    const int koff = 8 * (lane >> 4);
    // output: row m = m0 + lane % 16, columns n = n0 + 4 * (lane / 16) + r
    const int64_t m = m0 + (lane & 15);
    const int64_t mo = m < M ? m : M - 1;
    const uint32_t keep = bits >= 23 ? 0xFFFFFFFFu : ~((1u << (23 - bits)) - 1u);
    const int64_t kblocks = K / FG_GROUP;
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    for (int64_t k0 = 0; k0 < K; k0 += 32) {
        const int64_t kb = k0 / FG_GROUP;
        const long a = *reinterpret_cast<const long*>(xq + ma * K + k0 + koff);
        const long b = *reinterpret_cast<const long*>(wq + nb * K + k0 + koff);
        // first operand: the w rows (output columns), second: the x rows (output rows)
        const v4f p = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(b, a, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        const float s = sx[kb * M + mo] * sw[(n0 / FG_GROUP) * kblocks + kb];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const float t = acc[r] + p[r] * s;
            acc[r] = __uint_as_float(__float_as_uint(t) & keep);
        }
    }
    if (m < M) {
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int64_t n = n0 + 4 * (lane >> 4) + r;
            if (n < N) y[m * N + n] = acc[r];
        }
    }
}

}  // namespace

hipError_t fg_launch_fprop_limited(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw, int64_t M,
                                   int64_t N, int64_t K, int bits, float* y, hipStream_t stream) {
    const int64_t tiles = ((M + 15) / 16) * ((N + 15) / 16);
    hipLaunchKernelGGL(fg_fprop_limited_kernel, dim3((unsigned)tiles), dim3(64), 0, stream, xq, sx, wq, sw, M, N, K,
                       bits, y);
    return hipGetLastError();
}
