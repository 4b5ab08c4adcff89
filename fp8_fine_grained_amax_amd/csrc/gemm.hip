// Block-scaled FP8 (OCP E4M3) GEMMs for gfx950 with per-128-K FP32 promotion.
//
//   C[m][n] = sum_b  sA(m, b) * sB(n, b) * P_b(m, n),   P_b = sum_{k in block b} A[m][k] * B[n][k]
//
// One 128-deep K step is exactly one v_mfma_scale_f32_16x16x128_f8f6f4 (neutral E8M0 scales): the matrix
// core forms the block partial P_b of a 16x16 output tile from zero, and the VALU folds it into the FP32
// accumulators with one FMA per element: acc = fma(P_b, sA*sB, acc). This is the promotion of partial
// sums into FP32 registers every 128 elements of K (the "128 elements, equal to four WGMMAs" interval in
// "5 Ways You can get More Deepseek While Spending Less"), with the dequantization folded into the same
// step (per-group scaling along the inner dimension, same page). On the pages' H800 the promotion ran on
// CUDA cores while a second warpgroup kept the tensor cores busy (untitled gnrental.net page); here the
// MFMA of one 16x16 tile runs while the VALU promotes the previous one, inside each wave.
//
// Workgroup tile 256 x 256 x 128, 8 waves (2 x 4), wave tile 128 (M) x 64 (N): 32 MFMAs and 128 FP32
// accumulator VGPRs per wave per K step. Operand tiles go HBM -> LDS with global_load_lds_dwordx4 (no
// register staging), double-buffered (2 x 64 KB). LDS rows are 16 B-chunk XOR-swizzled so the fragment
// reads are conflict-free. The MFMA is issued with the B-role fragment first, so each lane ends up with
// one output row m and four consecutive output columns n (8 B bf16 / 16 B fp32 stores).
//
// Variants:
//   B_TRANS   B is stored [K][N] (the weight W[N_contr][K_out] read by Dgrad): the tile lands in LDS as
//             [128 contraction rows][256 B] and fragments are read with ds_read_b64_tr_b8, the transposed
//             LDS read (the capability the gnrental.net page asks future hardware for).
//   SB_BLOCK  sB = sw[n/128][b]           (Fprop / grouped: 128x128 weight blocks)
//   SB_BLOCK_T sB = sw[b][n/128]          (Dgrad: the same blocks, read along the other axis)
//   SB_ROW    sB = sb[b][n]               (Wgrad: 1x128 tiles along tokens on both operands)
//   GROUPED   rows split into per-group segments given by device offsets, B and sB per group.
#include "common.h"

namespace {

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int NTHREADS = 512;
constexpr int WAVE_M = 128, WAVE_N = 64;
constexpr int MSUB = WAVE_M / 16, NSUB = WAVE_N / 16;   // 8 x 4 MFMA tiles per wave
constexpr int STAGE_A = BM * BK;                        // 32 KB
constexpr int STAGE_B = BN * BK;                        // 32 KB
constexpr int STAGE = STAGE_A + STAGE_B + 2048;         // + A and B scale slices
constexpr int LDS_BYTES = 2 * STAGE;                    // 132 KB

enum { SB_BLOCK = 0, SB_BLOCK_T = 1, SB_ROW = 2 };

struct GemmParams {
    const uint8_t* a;       // A-role codes [rows][K], row stride K
    const float* sa;        // [K/128][sa_ld]
    int64_t sa_ld;          // rows of the activation-scale layout (M, or T for grouped)
    const uint8_t* b;       // NT: [N][K]; B_TRANS: [K][N]
    const float* sb;
    int64_t M, N, K;
    void* out;              // [M][N]
    int out_bf16;
    int accumulate;
    const int32_t* offsets; // grouped: [G+1]
    int G;
    int64_t b_group_stride; // elements between consecutive groups' B
    int64_t sb_group_stride;
};

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
    return (uint32_t)__builtin_bit_cast(unsigned short, (__bf16)f);
}

template <bool B_TRANS, int SBK, bool GROUPED>
__global__ __launch_bounds__(NTHREADS, 1) void fg_gemm_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int64_t N = p.N, K = p.K;
    const int64_t lda = K;
    const bool vec_ok = (N & 3) == 0;       // rows of the output are 16 B (fp32) / 8 B (bf16) aligned
    const int nkb = (int)(K / BK);

    // ---------------- tile assignment ----------------
    int64_t m0, m_end, n0;
    const uint8_t* Bp = p.b;
    const float* SBp = p.sb;
    const int n_tiles = (int)((N + BN - 1) / BN);
    if constexpr (GROUPED) {
        const int id_m = blockIdx.x / n_tiles;
        const int nt = blockIdx.x % n_tiles;
        int g = 0, cum = 0;
        int64_t seg0 = 0, seg1 = 0;
        for (; g < p.G; g++) {
            seg0 = p.offsets[g];
            seg1 = p.offsets[g + 1];
            int mt_g = (int)((seg1 - seg0 + BM - 1) / BM);
            if (id_m < cum + mt_g) break;
            cum += mt_g;
        }
        if (g >= p.G) return;                       // grid is sized for the worst case
        m0 = seg0 + (int64_t)(id_m - cum) * BM;
        m_end = seg1;
        n0 = (int64_t)nt * BN;
        Bp += (int64_t)g * p.b_group_stride;
        SBp += (int64_t)g * p.sb_group_stride;
    } else {
        const int m_tiles = (int)((p.M + BM - 1) / BM);
        const int total = m_tiles * n_tiles;
        int id = blockIdx.x;
        // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a contiguous range of
        // logical tiles so the tiles it runs at the same time share A and B panels in its own L2.
        if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);
        // groups of 8 M tiles: tiles in flight together form a compact block of the output
        const int GM = 8;
        const int group = id / (GM * n_tiles);
        const int first_m = group * GM;
        const int gsz = min(m_tiles - first_m, GM);
        const int within = id - group * GM * n_tiles;
        const int mt = first_m + within % gsz;
        const int nt = within / gsz;
        m0 = (int64_t)mt * BM;
        m_end = p.M;
        n0 = (int64_t)nt * BN;
    }

    // LDS stage st: [A 32 KB][B 32 KB][A scales 1 KB][B scales 1 KB (per-row B scales only)]
    auto stA = [&](int st) { return smem + st * STAGE; };
    auto stB = [&](int st) { return smem + st * STAGE + STAGE_A; };
    auto stSA = [&](int st) { return reinterpret_cast<float*>(smem + st * STAGE + STAGE_A + STAGE_B); };
    auto stSB = [&](int st) { return reinterpret_cast<float*>(smem + st * STAGE + STAGE_A + STAGE_B + 1024); };

    // ---------------- global -> LDS load plan (per thread, fixed over K) ----------------
    // Offsets are relative to wave-uniform tile bases (SGPRs) and fit in 32 bits (rows < 256 per tile).
    // A: wave w loads rows [32w, 32w+32) of the 256-row tile, 8 rows (1 KB) per instruction; lane l
    // lands at LDS row l/8, physical 16 B chunk l%8, and fetches logical chunk (l%8) ^ (row%8).
    const uint8_t* a_tile = p.a + m0 * lda;
    uint32_t a_off[4];
#pragma unroll
    for (int t = 0; t < 4; t++) {
        const int row = wave * 32 + t * 8 + (lane >> 3);
        const int lch = (lane & 7) ^ (row & 7);
        int64_t gr = m0 + row;
        gr = gr < m_end ? gr : m_end - 1;
        a_off[t] = (uint32_t)((gr - m0) * lda + lch * 16);
    }
    const uint8_t* b_tile;
    uint32_t b_off[4];
    if constexpr (!B_TRANS) {
        b_tile = Bp + n0 * K;
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const int row = wave * 32 + t * 8 + (lane >> 3);
            const int lch = (lane & 7) ^ (row & 7);
            int64_t gr = n0 + row;
            gr = gr < N ? gr : N - 1;
            b_off[t] = (uint32_t)((gr - n0) * K + lch * 16);
        }
    } else {
        // B^T tile: 128 contraction rows x 256 B (output columns); wave w loads rows [16w, 16w+16),
        // 4 rows per instruction; lane l lands at row l/16, physical chunk l%16 = logical ^ (row%16).
        b_tile = Bp;
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const int row = wave * 16 + t * 4 + (lane >> 4);
            const int lch = (lane & 15) ^ (row & 15);
            int64_t gc = n0 + lch * 16;
            gc = gc < N ? gc : N - 16;
            b_off[t] = (uint32_t)((int64_t)row * N + gc);
        }
    }
    // Scales of one K step: the tile's 256 A rows (waves 0-3, one float per lane) and, for per-row B
    // scales, the tile's 256 B rows (waves 4-7); rows past the end re-read the last valid row.
    int64_t sc_row;
    if (wave < 4) {
        sc_row = m0 + wave * 64 + lane;
        sc_row = sc_row < p.sa_ld ? sc_row : p.sa_ld - 1;
    } else {
        sc_row = n0 + (wave - 4) * 64 + lane;
        sc_row = sc_row < N ? sc_row : N - 1;
    }

    auto issue_loads = [&](int kb, int st) {
        const uint8_t* a_k = a_tile + (int64_t)kb * BK;
#pragma unroll
        for (int t = 0; t < 4; t++)
            __builtin_amdgcn_global_load_lds(FG_GLOBAL(a_k + a_off[t]), FG_LDS(stA(st) + (wave * 32 + t * 8) * BK),
                                             16, 0, 0);
        if constexpr (!B_TRANS) {
            const uint8_t* b_k = b_tile + (int64_t)kb * BK;
#pragma unroll
            for (int t = 0; t < 4; t++)
                __builtin_amdgcn_global_load_lds(FG_GLOBAL(b_k + b_off[t]),
                                                 FG_LDS(stB(st) + (wave * 32 + t * 8) * BK), 16, 0, 0);
        } else {
            const uint8_t* b_k = b_tile + (int64_t)kb * BK * N;
#pragma unroll
            for (int t = 0; t < 4; t++)
                __builtin_amdgcn_global_load_lds(FG_GLOBAL(b_k + b_off[t]),
                                                 FG_LDS(stB(st) + (wave * 16 + t * 4) * 256), 16, 0, 0);
        }
        if (wave < 4) {
            __builtin_amdgcn_global_load_lds(FG_GLOBAL(p.sa + (int64_t)kb * p.sa_ld + sc_row),
                                             FG_LDS(stSA(st) + wave * 64), 4, 0, 0);
        } else if constexpr (SBK == SB_ROW) {
            __builtin_amdgcn_global_load_lds(FG_GLOBAL(SBp + (int64_t)kb * N + sc_row),
                                             FG_LDS(stSB(st) + (wave - 4) * 64), 4, 0, 0);
        }
    };

    // ---------------- scale addressing ----------------
    const int lrow = lane & 15;        // output row (m) within a 16x16 tile held by this lane
    const int lcol4 = (lane >> 4) * 4; // first of the 4 output columns (n) held by this lane
    const int64_t wave_n0 = n0 + wn * WAVE_N;
    const int64_t nblocks = (N + 127) / 128;
    int64_t nblk = wave_n0 / 128;
    nblk = nblk < nblocks ? nblk : nblocks - 1;
    auto block_scale = [&](int kb) -> float {
        if constexpr (SBK == SB_BLOCK) return SBp[nblk * nkb + kb];
        if constexpr (SBK == SB_BLOCK_T) return SBp[(int64_t)kb * nblocks + nblk];
        return 1.0f;
    };

    // ---------------- accumulators ----------------
    v4f acc[MSUB][NSUB];
#pragma unroll
    for (int i = 0; i < MSUB; i++)
#pragma unroll
        for (int j = 0; j < NSUB; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    if (p.accumulate) {
        const float* o = reinterpret_cast<const float*>(p.out);
#pragma unroll
        for (int i = 0; i < MSUB; i++) {
            const int64_t m = m0 + wm * WAVE_M + i * 16 + lrow;
#pragma unroll
            for (int j = 0; j < NSUB; j++) {
                const int64_t n = wave_n0 + j * 16 + lcol4;
                if (m < m_end) {
                    if (vec_ok && n + 3 < N) {
                        float4 v = *reinterpret_cast<const float4*>(o + m * N + n);
                        acc[i][j] = v4f{v.x, v.y, v.z, v.w};
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; r++)
                            if (n + r < N) acc[i][j][r] = o[m * N + n + r];
                    }
                }
            }
        }
    }

    // ---------------- main loop ----------------
    if (nkb > 0) issue_loads(0, 0);
    const int g16 = lane >> 4;
    for (int kb = 0; kb < nkb; kb++) {
        const int st = kb & 1;
        const float sb_blk = block_scale(kb);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (kb + 1 < nkb) issue_loads(kb + 1, st ^ 1);
        const uint8_t* sAs = stA(st);
        const uint8_t* sBs = stB(st);
        const float* sSA = stSA(st);
        // B-role fragments for the wave's 4 N tiles
        v8i bf[NSUB];
#pragma unroll
        for (int j = 0; j < NSUB; j++) {
            if constexpr (!B_TRANS) {
                const int row = wn * WAVE_N + j * 16 + lrow;
                const uint8_t* base = sBs + row * BK;
                const v4i lo = *reinterpret_cast<const v4i*>(base + (((2 * g16) ^ (row & 7)) << 4));
                const v4i hi = *reinterpret_cast<const v4i*>(base + (((2 * g16 + 1) ^ (row & 7)) << 4));
                bf[j] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            } else {
                v2i part[4];
#pragma unroll
                for (int h = 0; h < 4; h++) {
                    const int crow = 32 * g16 + 8 * h + (lrow >> 1);
                    const int col = wn * WAVE_N + j * 16 + 8 * (lrow & 1);
                    const int off = crow * 256 + ((((col >> 4) ^ (crow & 15))) << 4) + (col & 15);
                    part[h] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (__attribute__((address_space(3))) v2i*)(sBs + off));
                }
                bf[j] = v8i{part[0].x, part[0].y, part[1].x, part[1].y, part[2].x, part[2].y, part[3].x, part[3].y};
            }
        }
        float4 sbr[NSUB];
        if constexpr (SBK == SB_ROW) {
            const float* sSB = stSB(st);
#pragma unroll
            for (int j = 0; j < NSUB; j++) sbr[j] = *reinterpret_cast<const float4*>(sSB + wn * WAVE_N + j * 16 + lcol4);
        }
#pragma unroll
        for (int i = 0; i < MSUB; i++) {
            const int row = wm * WAVE_M + i * 16 + lrow;
            const uint8_t* base = sAs + row * BK;
            const v4i lo = *reinterpret_cast<const v4i*>(base + (((2 * g16) ^ (row & 7)) << 4));
            const v4i hi = *reinterpret_cast<const v4i*>(base + (((2 * g16 + 1) ^ (row & 7)) << 4));
            const v8i af = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            const float sa_i = sSA[row];
            const float s_i = sa_i * sb_blk;
#pragma unroll
            for (int j = 0; j < NSUB; j++) {
                const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    bf[j], af, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
                if constexpr (SBK != SB_ROW) {
#pragma unroll
                    for (int r = 0; r < 4; r++) acc[i][j][r] = __builtin_fmaf(part[r], s_i, acc[i][j][r]);
                } else {
                    const float sb4[4] = {sbr[j].x, sbr[j].y, sbr[j].z, sbr[j].w};
#pragma unroll
                    for (int r = 0; r < 4; r++) acc[i][j][r] = __builtin_fmaf(part[r], sa_i * sb4[r], acc[i][j][r]);
                }
            }
        }
    }

    // ---------------- epilogue ----------------
#pragma unroll
    for (int i = 0; i < MSUB; i++) {
        const int64_t m = m0 + wm * WAVE_M + i * 16 + lrow;
        if (m >= m_end) continue;
#pragma unroll
        for (int j = 0; j < NSUB; j++) {
            const int64_t n = wave_n0 + j * 16 + lcol4;
            if (p.out_bf16) {
                uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + m * N + n;
                if (vec_ok && n + 3 < N) {
                    uint2 v;
                    v.x = bf16_rne_bits(acc[i][j][0]) | (bf16_rne_bits(acc[i][j][1]) << 16);
                    v.y = bf16_rne_bits(acc[i][j][2]) | (bf16_rne_bits(acc[i][j][3]) << 16);
                    *reinterpret_cast<uint2*>(o) = v;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; r++)
                        if (n + r < N) o[r] = (uint16_t)bf16_rne_bits(acc[i][j][r]);
                }
            } else {
                float* o = reinterpret_cast<float*>(p.out) + m * N + n;
                if (vec_ok && n + 3 < N) {
                    *reinterpret_cast<float4*>(o) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; r++)
                        if (n + r < N) o[r] = acc[i][j][r];
                }
            }
        }
    }
}

template <bool B_TRANS, int SBK, bool GROUPED>
hipError_t launch(const GemmParams& p, unsigned grid, hipStream_t stream) {
    auto kern = fg_gemm_kernel<B_TRANS, SBK, GROUPED>;
    static bool attr_set = false;   // benign race: setting the attribute twice is harmless
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NTHREADS), LDS_BYTES, stream, p);
    return hipGetLastError();
}

unsigned tiles_2d(int64_t M, int64_t N) {
    return (unsigned)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
}

}  // namespace

hipError_t fg_launch_gemm_fprop(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw, int64_t M,
                                int64_t N, int64_t K, void* y, int out_bf16, hipStream_t stream) {
    GemmParams p{};
    p.a = xq; p.sa = sx; p.sa_ld = M; p.b = wq; p.sb = sw;
    p.M = M; p.N = N; p.K = K; p.out = y; p.out_bf16 = out_bf16;
    return launch<false, SB_BLOCK, false>(p, tiles_2d(M, N), stream);
}

hipError_t fg_launch_gemm_dgrad(const uint8_t* dyq, const float* sdy, const uint8_t* wq, const float* sw, int64_t M,
                                int64_t N, int64_t K, void* dx, int out_bf16, hipStream_t stream) {
    // dX[M][K] = dY[M][N] . W[N][K]: A-role = dY (contraction N), B-role = W read transposed.
    GemmParams p{};
    p.a = dyq; p.sa = sdy; p.sa_ld = M; p.b = wq; p.sb = sw;
    p.M = M; p.N = K; p.K = N; p.out = dx; p.out_bf16 = out_bf16;
    return launch<true, SB_BLOCK_T, false>(p, tiles_2d(M, K), stream);
}

hipError_t fg_launch_gemm_wgrad(const uint8_t* dytq, const float* sdyt, const uint8_t* xtq, const float* sxt,
                                int64_t M, int64_t N, int64_t K, float* dw, int accumulate, hipStream_t stream) {
    // dW[N][K] = dYt[N][M] . Xt[K][M]^T: A-role = dYt (rows N), B-role = Xt (rows K), contraction M.
    GemmParams p{};
    p.a = dytq; p.sa = sdyt; p.sa_ld = N; p.b = xtq; p.sb = sxt;
    p.M = N; p.N = K; p.K = M; p.out = dw; p.out_bf16 = 0; p.accumulate = accumulate;
    return launch<false, SB_ROW, false>(p, tiles_2d(N, K), stream);
}

hipError_t fg_launch_gemm_grouped(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw,
                                  const int32_t* offsets, int32_t G, int64_t T, int64_t N, int64_t K, void* y,
                                  int out_bf16, hipStream_t stream) {
    GemmParams p{};
    p.a = xq; p.sa = sx; p.sa_ld = T; p.b = wq; p.sb = sw;
    p.M = T; p.N = N; p.K = K; p.out = y; p.out_bf16 = out_bf16;
    p.offsets = offsets; p.G = G;
    p.b_group_stride = N * K;
    p.sb_group_stride = ((N + 127) / 128) * (K / 128);
    const int64_t n_tiles = (N + BN - 1) / BN;
    const int64_t m_tiles_max = (T + BM - 1) / BM + G;
    return launch<false, SB_BLOCK, true>(p, (unsigned)(m_tiles_max * n_tiles), stream);
}
