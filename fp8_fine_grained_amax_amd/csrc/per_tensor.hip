// Per-tensor E4M3 scaling, the prior practice the fine-grained tiles are measured against.
//
// "5 Ways You can get More Deepseek While Spending Less" describes the usual FP8 recipe: one scale for a
// whole tensor, chosen so that the tensor's max-abs lands on the largest FP8 value, and notes how badly
// activation outliers then hurt every other value. "Three Fast Methods To Study Deepseek" describes
// delayed quantization: the scale comes from a history of max-abs values of earlier iterations, so the
// current tensor is quantized in one pass, and values above the history's maximum saturate.
//
// Both are one kernel here: the scale is derived on the device from a max-abs history array (one entry:
// the current tensor's max-abs from fg_amax_kernel, i.e. the current per-tensor scaling with two reads
// of the input; several entries: delayed scaling with one read). The codes use the same scale rule and
// quotient forms as the 1x128 quantizers, with saturation at +-448. The scale is broadcast into the
// 1x128 activation or 128x128 weight scale layout, so the block-scaled GEMMs consume these codes as
// they are. The kernel can fold the tensor's own max-abs into a history slot on the way.
#include "common.h"
#include "host_util.h"

namespace {

constexpr int kUnroll = 4;          // 16-byte loads in flight per lane
constexpr uint32_t kBf16MaxBits = 0x7F7F0000u;

// Largest |entry| of the history, rounded up to a bf16 value (and at most the largest finite bf16), as
// bf16 bits; 0 for an empty history. Every lane of the calling wave gets the result.
__device__ __forceinline__ uint32_t hist_amax_bf16_bits(const float* __restrict__ hist, int64_t n) {
    uint32_t m = 0;
    for (int64_t i = threadIdx.x & 63; i < n; i += 64) {
        const uint32_t a = __float_as_uint(hist[i]) & 0x7FFFFFFFu;
        m = a > m ? a : m;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const uint32_t t = (uint32_t)__shfl_xor((int)m, o);
        m = t > m ? t : m;
    }
    if (m & 0xFFFFu) m = (m & 0xFFFF0000u) + 0x10000u;
    m = m > kBf16MaxBits ? kBf16MaxBits : m;
    return m >> 16;
}

// x / s handed to the E4M3 conversion, saturated: any quotient outside [-448, 448] (including the
// overflowed and NaN intermediates of inputs far above the history's max-abs) becomes +-448 with x's
// sign. Within the max-abs the quotient forms are the correctly rounded quotient (see common.h); above
// it the exact quotient exceeds 448 unless s is a power of two, where every form is exact.
template <int MODE>
__device__ __forceinline__ float quot_sat(float x, const fg_divisor& d) {
    const float q = fg_quot_arg<MODE>(x, d);
    return __builtin_fabsf(q) <= 448.0f ? q : __builtin_copysignf(448.0f, x);
}

template <int MODE>
__device__ __forceinline__ uint2 quant8_sat(uint4 v, const fg_divisor& d) {
    auto pk = [&](uint32_t w0, uint32_t w1) {
        uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(quot_sat<MODE>(fg_bf16_lo(w0), d),
                                                               quot_sat<MODE>(fg_bf16_hi(w0), d), 0, false);
        return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(quot_sat<MODE>(fg_bf16_lo(w1), d),
                                                         quot_sat<MODE>(fg_bf16_hi(w1), d), (int)c, true);
    };
    return make_uint2(pk(v.x, v.y), pk(v.z, v.w));
}

// One pass over x [rows][cols] (cols % 8 == 0). Workgroup b owns a contiguous band of rows and sweeps it
// as one flat run of 16 B chunks, kUnroll loads in flight per lane. Returns this lane's max-abs (bf16
// bits); with QUANT it also writes the codes.
constexpr int kThreads = 1024;

template <bool QUANT, int MODE>
__device__ __forceinline__ uint32_t sweep(const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
                                          const fg_divisor& d, uint8_t* __restrict__ q) {
    const uint32_t cpr = (uint32_t)(cols / 8);                     // chunks per row
    const int64_t r0 = (int64_t)blockIdx.x * rows / gridDim.x;
    const int64_t r1 = (int64_t)(blockIdx.x + 1) * rows / gridDim.x;
    const uint32_t n = (uint32_t)(r1 - r0) * cpr;                  // host-checked to fit
    uint32_t m = 0;
    for (uint32_t i0 = threadIdx.x; i0 < n; i0 += kThreads * kUnroll) {
        uint4 v[kUnroll];
        int64_t off[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const uint32_t i = i0 + kThreads * u;
            const uint32_t rr = i / cpr, c = i - rr * cpr;
            off[u] = (r0 + rr) * ld + (int64_t)c * 8;
            v[u] = i < n ? *reinterpret_cast<const uint4*>(x + off[u]) : make_uint4(0, 0, 0, 0);
            if constexpr (QUANT) off[u] = (r0 + rr) * cols + (int64_t)c * 8;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            m = fg_pk_max_u16(m, fg_pk_max_u16(fg_pk_max_u16(v[u].x & 0x7FFF7FFFu, v[u].y & 0x7FFF7FFFu),
                                               fg_pk_max_u16(v[u].z & 0x7FFF7FFFu, v[u].w & 0x7FFF7FFFu)));
            if constexpr (QUANT) {
                if (i0 + kThreads * u < n) *reinterpret_cast<uint2*>(q + off[u]) = quant8_sat<MODE>(v[u], d);
            }
        }
    }
    return fg_max_halves(m);
}

// Max over the workgroup, then at most one atomic max per workgroup into *out (the fp32 bits of the
// bf16 max-abs: non-negative floats order like their bit patterns). The value at *out only grows, so a
// workgroup whose max is already covered by what it reads there skips its atomic: a stale read can only
// be smaller than the true value and costs an unneeded atomic, never a lost one.
__device__ __forceinline__ void fold_amax(uint32_t m, uint32_t* out) {
    __shared__ uint32_t wmax[kThreads / 64];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const uint32_t t = (uint32_t)__shfl_xor((int)m, o);
        m = t > m ? t : m;
    }
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t b = wmax[0];
        for (int w = 1; w < kThreads / 64; w++) b = wmax[w] > b ? wmax[w] : b;
        b <<= 16;
        if (b > __hip_atomic_load(out, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(out, b);
    }
}

__global__ __launch_bounds__(kThreads) void fg_amax_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                           int64_t ld, uint32_t* amax) {
    const fg_divisor d{1.0f, 1.0f};
    fold_amax(sweep<false, FG_Q_POW2>(x, rows, cols, ld, d, nullptr), amax);
}

__global__ __launch_bounds__(kThreads) void fg_quant_per_tensor_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                                       int64_t cols, int64_t ld,
                                                                       const float* __restrict__ hist, int64_t n_hist,
                                                                       int pow2, int64_t n_scales,
                                                                       uint8_t* __restrict__ q,
                                                                       float* __restrict__ scales, uint32_t* amax_out) {
    const uint32_t ab = hist_amax_bf16_bits(hist, n_hist);
    const float s = fg_scale_from_amax_bits(ab, pow2);
    const fg_divisor d = fg_make_divisor(s, pow2);
    // the broadcast scale array, flat and coalesced
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n_scales; i += (int64_t)gridDim.x * kThreads)
        scales[i] = s;
    uint32_t m;
    if (pow2)
        m = sweep<true, FG_Q_POW2>(x, rows, cols, ld, d, q);
    else if (!fg_divisor_tiny(d))
        m = sweep<true, FG_Q_FAST>(x, rows, cols, ld, d, q);
    else
        m = sweep<true, FG_Q_TINY>(x, rows, cols, ld, fg_divisor_shifted(d), q);
    if (amax_out) fold_amax(m, amax_out);
}

// One workgroup of 1024 lanes per compute unit (fewer for short tensors): 64 KB of loads in flight per
// CU, and at most one max-abs atomic per CU.
unsigned grid_rows(int64_t rows) {
    const int cus = fg_device_cus();
    return (unsigned)(rows < cus ? rows : cus);
}

}  // namespace

hipError_t fg_launch_amax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, float* amax, hipStream_t stream) {
    hipLaunchKernelGGL(fg_amax_kernel, dim3(grid_rows(rows)), dim3(kThreads), 0, stream, x, rows, cols, ld,
                       reinterpret_cast<uint32_t*>(amax));
    return hipGetLastError();
}

hipError_t fg_launch_quant_per_tensor(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, const float* hist,
                                      int64_t n_hist, int pow2, int64_t n_scales, uint8_t* q, float* scales,
                                      float* amax_out, hipStream_t stream) {
    hipLaunchKernelGGL(fg_quant_per_tensor_kernel, dim3(grid_rows(rows)), dim3(kThreads), 0, stream, x, rows, cols, ld,
                       hist, n_hist, pow2, n_scales, q, scales, reinterpret_cast<uint32_t*>(amax_out));
    return hipGetLastError();
}
