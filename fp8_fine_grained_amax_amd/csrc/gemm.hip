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
// Workgroup tile 256 (M) x 192 (N) x 128 (K), 12 waves of 64 x 64 (3 waves per SIMD): 16 MFMAs and 64 FP32
// accumulator VGPRs per wave per K step, so each wave stays under the 168-VGPR budget of 3 waves per SIMD
// and the SIMD hides MFMA and LDS latency by switching between waves. Operand tiles go HBM -> LDS with
// global_load_lds_dwordx4 (no register staging), double-buffered (2 x 58 KB). LDS rows are 16 B-chunk
// swizzled so the fragment reads are bank-conflict-free. The MFMA is issued with the B-role fragment
// first, so each lane ends up with one output row m and four consecutive output columns n (8 B bf16 /
// 16 B fp32 stores). The DeepSeek-V3 dense-MLP Fprop (4096 x 18432) is exactly 1536 tiles: 6 full rounds
// of 256 CUs.
//
// Variants:
//   B_TRANS   B is stored [K][N] (the weight W[N_contr][K_out] read by Dgrad): the tile lands in LDS as
//             [128 contraction rows][192 B] and fragments are read with ds_read_b64_tr_b8, the transposed
//             LDS read (the capability the gnrental.net page asks future hardware for).
//   SB_BLOCK  sB = sw[n/128][b]           (Fprop / grouped: 128x128 weight blocks)
//   SB_BLOCK_T sB = sw[b][n/128]          (Dgrad: the same blocks, read along the other axis)
//   SB_ROW    sB = sb[b][n]               (Wgrad: 1x128 tiles along tokens on both operands)
//   GROUPED   rows split into per-group segments given by device offsets, B and sB per group.
#include "common.h"

namespace {

// Workgroup tile 256 (M) x 192 (N) x 128 (K), 12 waves in a 4 x 3 grid, wave tile 64 x 64.
constexpr int BM = 256, BN = 192, BK = 128;
constexpr int NWAVES = 12;
constexpr int NTHREADS = NWAVES * 64;
constexpr int WAVE_M = 64, WAVE_N = 64;
constexpr int WAVES_N = BN / WAVE_N;                    // 3
constexpr int MSUB = WAVE_M / 16, NSUB = WAVE_N / 16;   // 4 x 4 MFMA tiles per wave
constexpr int STAGE_A = BM * BK;                        // 32 KB
constexpr int STAGE_B = BN * BK;                        // 24 KB (NT: [192][128 B]; transposed: [128][192 B])
constexpr int STAGE = STAGE_A + STAGE_B + 2048;         // + A and B scale slices (1 KB each)
constexpr int LDS_BYTES = 2 * STAGE;                    // 116 KB, double-buffered

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

// LDS swizzles. gfx950 serves a ds_read_b128 16 lanes (256 B, all 64 banks) at a time, and the 8 rows
// one direct-load instruction writes as 128 B per row. For a [rows][128 B] tile the 16 B chunk c of row r
// is stored at c ^ swz128(r): rows r..r+15 read at one logical chunk land on 16 distinct (row parity,
// chunk) bank groups.
__device__ __forceinline__ int swz128(int r) { return (r & 7) ^ ((r >> 3) & 1); }
// Transposed B tile [128 contraction rows][192 B]: chunk c of row r is stored at c ^ swzT(r) (only the
// low two bits move, so chunks stay inside their aligned group of four, i.e. inside the 12-chunk row).
// ds_read_b64_tr_b8 serves 32 lanes at a time: rows r..r+7 and r+32..r+39, two 8 B halves of one logical
// chunk each; with the 192 B row stride these hit 32 distinct 8 B slots of the 256 B bank window.
__device__ __forceinline__ int swzT(int r) { return ((r >> 2) & 1) | (((r >> 5) & 1) << 1); }

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
    return (uint32_t)__builtin_bit_cast(unsigned short, (__bf16)f);
}

// One 16x128 E4M3 MFMA operand from a swizzled [rows][128 B] LDS tile whose first row is a multiple of
// 16: lane l holds row l%16 and bytes [32 g, 32 g + 32) of its 128-byte K slice, g = l/16; `lo_off` and
// `hi_off` are the lane's byte offsets of the two 16 B halves (row and swizzle folded in).
__device__ __forceinline__ v8i frag_at(const uint8_t* tile16, int lo_off, int hi_off) {
    const v4i lo = *reinterpret_cast<const v4i*>(tile16 + lo_off);
    const v4i hi = *reinterpret_cast<const v4i*>(tile16 + hi_off);
    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// E8M0 code of an fp32 power of two in [2^-127, 2^127]: its biased exponent field.
__device__ __forceinline__ int e8m0_of(float s) { return (int)(__float_as_uint(s) >> 23) & 0xFF; }

template <bool B_TRANS, int SBK, bool GROUPED, bool POW2>
__global__ __launch_bounds__(NTHREADS, 1) void fg_gemm_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int64_t N = p.N, K = p.K;
    const int64_t lda = K;
    const bool vec_ok = (N & 3) == 0;       // output rows are 16 B (fp32) / 8 B (bf16) aligned
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

    // LDS stage st: [A 32 KB][B 24 KB][A scales 1 KB][B scales 1 KB (per-row B scales only)]
    auto stA = [&](int st) { return smem + st * STAGE; };
    auto stB = [&](int st) { return smem + st * STAGE + STAGE_A; };
    auto stSA = [&](int st) { return reinterpret_cast<float*>(smem + st * STAGE + STAGE_A + STAGE_B); };
    auto stSB = [&](int st) { return reinterpret_cast<float*>(smem + st * STAGE + STAGE_A + STAGE_B + 1024); };

    // ---------------- global -> LDS load plan (per thread, fixed over K) ----------------
    // Each global_load_lds_dwordx4 instruction fills 1 KB of LDS: lane l lands at byte 16 l of it.
    // A: 32 instructions of 8 rows (instruction t: rows 8t .. 8t+7); wave w issues t = w, w+12, w+24.
    // Lane l lands at row 8t + l/8, physical chunk l%8, and fetches logical chunk (l%8) ^ swz128(row).
    // Offsets are relative to wave-uniform tile bases (SGPRs) and fit in 32 bits.
    const uint8_t* a_tile = p.a + m0 * lda;
    uint32_t a_off[3];
#pragma unroll
    for (int u = 0; u < 3; u++) {
        const int t = wave + NWAVES * u;
        const int row = (t * 8 + (lane >> 3)) & (BM - 1);
        const int lch = (lane & 7) ^ swz128(row);
        int64_t gr = m0 + row;
        gr = gr < m_end ? gr : m_end - 1;
        a_off[u] = (uint32_t)((gr - m0) * lda + lch * 16);
    }
    const int a_count = wave + NWAVES * 2 < BM / 8 ? 3 : 2;
    // B (NT): 24 instructions of 8 rows, wave w issues t = w, w+12.
    // B (transposed): [128][192 B] = 24 instructions of 1 KB; flat 16 B slot f = 64 t + l is row f/12,
    // physical chunk f%12, holding logical chunk (f%12) ^ swzT(row) (output columns 16 * logical ..).
    const uint8_t* b_tile;
    uint32_t b_off[2];
    if constexpr (!B_TRANS) {
        b_tile = Bp + n0 * K;
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int t = wave + NWAVES * u;
            const int row = t * 8 + (lane >> 3);
            const int lch = (lane & 7) ^ swz128(row);
            int64_t gr = n0 + row;
            gr = gr < N ? gr : N - 1;
            b_off[u] = (uint32_t)((gr - n0) * K + lch * 16);
        }
    } else {
        b_tile = Bp;
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int f = (wave + NWAVES * u) * 64 + lane;
            const int row = f / 12, pch = f % 12;
            const int lch = pch ^ swzT(row);
            int64_t gc = n0 + lch * 16;
            gc = gc < N ? gc : N - 16;
            b_off[u] = (uint32_t)((int64_t)row * N + gc);
        }
    }
    // Scales of one K step: the tile's 256 A rows (waves 0-3, one float per lane) and, for per-row B
    // scales, the tile's 192 B rows (waves 4-6); rows past the end re-read the last valid row.
    int64_t sc_row = 0;
    if (wave < 4) {
        sc_row = m0 + wave * 64 + lane;
        sc_row = sc_row < p.sa_ld ? sc_row : p.sa_ld - 1;
    } else if (wave < 7) {
        sc_row = n0 + (wave - 4) * 64 + lane;
        sc_row = sc_row < N ? sc_row : N - 1;
    }

    // Staging loads of one K step: every wave issues exactly six (3 A + 2 B + 1 scale slice), branch-free,
    // in four pieces spread over the step's four M-tile MFMA groups: a burst of all of them right after
    // the barrier stalls the issuing waves in the memory pipeline before their MFMAs. Waves 8-11 own only
    // two A instructions and waves 7-11 no scale slice: they re-issue one of their own loads (same source,
    // same LDS bytes), which is harmless.
    const int a_u2 = a_count == 3 ? 2 : 0;
    const int sc_wave = wave < 7 ? wave : (wave - 7) & 3;
    if (wave >= 7) {
        int64_t r = m0 + sc_wave * 64 + lane;
        sc_row = r < p.sa_ld ? r : p.sa_ld - 1;
    }
    auto issue_piece = [&](int kb, int st, int piece) {
        const uint8_t* a_k = a_tile + (int64_t)kb * BK;
        const uint8_t* b_k = B_TRANS ? b_tile + (int64_t)kb * BK * N : b_tile + (int64_t)kb * BK;
        if (piece == 0) {
            __builtin_amdgcn_global_load_lds(FG_GLOBAL(a_k + a_off[0]), FG_LDS(stA(st) + wave * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(FG_GLOBAL(a_k + a_off[1]), FG_LDS(stA(st) + (wave + NWAVES) * 1024), 16, 0,
                                             0);
        } else if (piece == 1) {
            __builtin_amdgcn_global_load_lds(FG_GLOBAL(a_k + a_off[a_u2]), FG_LDS(stA(st) + (wave + NWAVES * a_u2) * 1024),
                                             16, 0, 0);
            __builtin_amdgcn_global_load_lds(FG_GLOBAL(b_k + b_off[0]), FG_LDS(stB(st) + wave * 1024), 16, 0, 0);
        } else if (piece == 2) {
            __builtin_amdgcn_global_load_lds(FG_GLOBAL(b_k + b_off[1]), FG_LDS(stB(st) + (wave + NWAVES) * 1024), 16, 0,
                                             0);
        } else {
            const bool rowb = SBK == SB_ROW && sc_wave >= 4;
            const float* src = rowb ? SBp + (int64_t)kb * N + sc_row : p.sa + (int64_t)kb * p.sa_ld + sc_row;
            float* dst = rowb ? stSB(st) + (sc_wave - 4) * 64 : stSA(st) + (sc_wave & 3) * 64;
            if (!(SBK == SB_ROW) && sc_wave >= 4) {             // no per-row B scales: re-load an A slice
                src = p.sa + (int64_t)kb * p.sa_ld + (m0 + (sc_wave & 3) * 64 + lane < p.sa_ld
                                                          ? m0 + (sc_wave & 3) * 64 + lane : p.sa_ld - 1);
                dst = stSA(st) + (sc_wave & 3) * 64;
            }
            __builtin_amdgcn_global_load_lds(FG_GLOBAL(src), FG_LDS(dst), 4, 0, 0);
        }
    };
    auto issue_loads = [&](int kb, int st) {
#pragma unroll
        for (int piece = 0; piece < 4; piece++) issue_piece(kb, st, piece);
    };

    // ---------------- scale addressing ----------------
    const int lrow = lane & 15;        // output row (m) within a 16x16 tile held by this lane
    const int lcol4 = (lane >> 4) * 4; // first of the 4 output columns (n) held by this lane
    const int64_t wave_n0 = n0 + wn * WAVE_N;
    const int64_t nblocks = (N + 127) / 128;
    int64_t nblk = wave_n0 / 128;                 // a 64-column wave tile never straddles a 128-block
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

    // Per-lane LDS offsets of the MFMA operand reads. The swizzle depends only on the row modulo 16 and
    // every fragment starts on a multiple of 16 rows, so one lane offset plus an immediate per fragment
    // addresses all of them.
    const int g16 = lane >> 4;
    const int frag_lo = lrow * BK + (((2 * g16) ^ swz128(lrow)) << 4);
    const int frag_hi = lrow * BK + (((2 * g16 + 1) ^ swz128(lrow)) << 4);
    // Transposed B reads: lane l of group g reads contraction row 32 g + 8 h + (l%16)/2, the 8 B half
    // l%2 of the 16-column chunk of its output columns; chunk c of row r is stored at c ^ swzT(r).
    int tr_off[4], tr_z[4];
#pragma unroll
    for (int h = 0; h < 4; h++) {
        const int crow = 32 * g16 + 8 * h + (lrow >> 1);
        tr_off[h] = crow * 192 + 8 * (lrow & 1);
        tr_z[h] = swzT(crow);
    }

    // ---------------- main loop ----------------
    // The 128x128 block scale of step kb+1 is fetched with that step's tile loads, so the wait at the top
    // of each step covers it and no step waits on a scale load of its own.
    float sb_next = 1.0f;
    if (nkb > 0) {
        issue_loads(0, 0);
        sb_next = block_scale(0);
    }
    for (int kb = 0; kb < nkb; kb++) {
        const int st = kb & 1;
        const float sb_blk = sb_next;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        // next step's stage (on the last step: a harmless reload of this step's data into the idle buffer,
        // which keeps the step body branch-free)
        const int kb1 = kb + 1 < nkb ? kb + 1 : kb;
        sb_next = block_scale(kb1);
        const uint8_t* sAs = stA(st);
        const uint8_t* sBs = stB(st);
        const float* sSA = stSA(st);
        // B-role fragments for the wave's 4 N tiles, held for the whole K step
        v8i bf[NSUB];
#pragma unroll
        for (int j = 0; j < NSUB; j++) {
            if constexpr (!B_TRANS) {
                bf[j] = frag_at(sBs + (wn * WAVE_N + j * 16) * BK, frag_lo, frag_hi);
            } else {
                const int chunk = wn * 4 + j;
                v2i part[4];
#pragma unroll
                for (int h = 0; h < 4; h++)
                    part[h] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (__attribute__((address_space(3))) v2i*)(sBs + tr_off[h] + ((chunk ^ tr_z[h]) << 4)));
                bf[j] = v8i{part[0].x, part[0].y, part[1].x, part[1].y, part[2].x, part[2].y, part[3].x, part[3].y};
            }
        }
        float4 sbr[NSUB];
        if constexpr (SBK == SB_ROW && !POW2) {
            const float* sSB = stSB(st);
#pragma unroll
            for (int j = 0; j < NSUB; j++) sbr[j] = *reinterpret_cast<const float4*>(sSB + wn * WAVE_N + j * 16 + lcol4);
        }
        const uint8_t* sA_w = sAs + wm * WAVE_M * BK;
        const float* sSA_w = sSA + wm * WAVE_M + lrow;
        if constexpr (POW2) {
            // Power-of-two scales: the matrix core applies them itself. Per lane l the E8M0 scale operand
            // of a 16x128 fragment scales row l%16 (all four 32-element K sub-blocks of the lane carry the
            // same scale), so the A-role operand takes the row scale of output row m and the B-role
            // operand the block scale (or, with per-row B scales, the scale of output column n); the MFMA
            // adds 2^(ea+eb) * P_b straight into the FP32 accumulator, with no VALU promotion.
            int eb[NSUB];
#pragma unroll
            for (int j = 0; j < NSUB; j++)
                eb[j] = SBK == SB_ROW ? e8m0_of(stSB(st)[wn * WAVE_N + j * 16 + lrow]) : e8m0_of(sb_blk);
#pragma unroll
            for (int i = 0; i < MSUB; i++) {
                issue_piece(kb1, st ^ 1, i);
                const v8i af = frag_at(sA_w + i * 16 * BK, frag_lo, frag_hi);
                const int ea = e8m0_of(sSA_w[i * 16]);
#pragma unroll
                for (int j = 0; j < NSUB; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af, acc[i][j], 0, 0, 0, eb[j], 0,
                                                                                ea);
            }
        } else {
            // VALU promotion, software-pipelined by one MFMA: the FMAs that fold tile (i, j) into the FP32
            // accumulators are issued after the MFMA of the next tile, so no FMA waits on the MFMA right
            // before it (a VALU read of an MFMA result is not interlocked; the wait states would stall the
            // wave). The scheduling groups pin the order: MFMA, then the previous tile's 4 FMAs.
            v4f prev = v4f{0.f, 0.f, 0.f, 0.f};
            float s_prev[4] = {0.f, 0.f, 0.f, 0.f};
            int ip = -1, jp = -1;
            float sa_v[MSUB];
#pragma unroll
            for (int i = 0; i < MSUB; i++) sa_v[i] = sSA_w[i * 16];
#pragma unroll
            for (int i = 0; i < MSUB; i++) {
                issue_piece(kb1, st ^ 1, i);
                const v8i af = frag_at(sA_w + i * 16 * BK, frag_lo, frag_hi);
#pragma unroll
                for (int j = 0; j < NSUB; j++) {
                    const v4f cur = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        bf[j], af, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
                    if (ip >= 0) {
#pragma unroll
                        for (int r = 0; r < 4; r++) acc[ip][jp][r] = __builtin_fmaf(prev[r], s_prev[r], acc[ip][jp][r]);
                    }
                    prev = cur;
                    ip = i;
                    jp = j;
                    if constexpr (SBK != SB_ROW) {
                        const float s_ij = sa_v[i] * sb_blk;
                        s_prev[0] = s_prev[1] = s_prev[2] = s_prev[3] = s_ij;
                    } else {
                        s_prev[0] = sa_v[i] * sbr[j].x;
                        s_prev[1] = sa_v[i] * sbr[j].y;
                        s_prev[2] = sa_v[i] * sbr[j].z;
                        s_prev[3] = sa_v[i] * sbr[j].w;
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < 4; r++) acc[ip][jp][r] = __builtin_fmaf(prev[r], s_prev[r], acc[ip][jp][r]);
        }
    }

    __builtin_amdgcn_s_waitcnt(0);          // the last step's (redundant) staging loads
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

template <bool B_TRANS, int SBK, bool GROUPED, bool POW2>
hipError_t launch_one(const GemmParams& p, unsigned grid, hipStream_t stream) {
    auto kern = fg_gemm_kernel<B_TRANS, SBK, GROUPED, POW2>;
    static bool attr_set = false;   // benign race: setting the attribute twice is harmless
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NTHREADS), LDS_BYTES, stream, p);
    return hipGetLastError();
}

template <bool B_TRANS, int SBK, bool GROUPED>
hipError_t launch(const GemmParams& p, unsigned grid, int pow2, hipStream_t stream) {
    return pow2 ? launch_one<B_TRANS, SBK, GROUPED, true>(p, grid, stream)
                : launch_one<B_TRANS, SBK, GROUPED, false>(p, grid, stream);
}

unsigned tiles_2d(int64_t M, int64_t N) {
    return (unsigned)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
}

}  // namespace

hipError_t fg_launch_gemm_fprop(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw, int64_t M,
                                int64_t N, int64_t K, void* y, int out_bf16, int pow2, hipStream_t stream) {
    GemmParams p{};
    p.a = xq; p.sa = sx; p.sa_ld = M; p.b = wq; p.sb = sw;
    p.M = M; p.N = N; p.K = K; p.out = y; p.out_bf16 = out_bf16;
    return launch<false, SB_BLOCK, false>(p, tiles_2d(M, N), pow2, stream);
}

hipError_t fg_launch_gemm_dgrad(const uint8_t* dyq, const float* sdy, const uint8_t* wq, const float* sw, int64_t M,
                                int64_t N, int64_t K, void* dx, int out_bf16, int pow2, hipStream_t stream) {
    // dX[M][K] = dY[M][N] . W[N][K]: A-role = dY (contraction N), B-role = W read transposed.
    GemmParams p{};
    p.a = dyq; p.sa = sdy; p.sa_ld = M; p.b = wq; p.sb = sw;
    p.M = M; p.N = K; p.K = N; p.out = dx; p.out_bf16 = out_bf16;
    return launch<true, SB_BLOCK_T, false>(p, tiles_2d(M, K), pow2, stream);
}

hipError_t fg_launch_gemm_wgrad(const uint8_t* dytq, const float* sdyt, const uint8_t* xtq, const float* sxt,
                                int64_t M, int64_t N, int64_t K, float* dw, int accumulate, int pow2, hipStream_t stream) {
    // dW[N][K] = dYt[N][M] . Xt[K][M]^T: A-role = dYt (rows N), B-role = Xt (rows K), contraction M.
    GemmParams p{};
    p.a = dytq; p.sa = sdyt; p.sa_ld = N; p.b = xtq; p.sb = sxt;
    p.M = N; p.N = K; p.K = M; p.out = dw; p.out_bf16 = 0; p.accumulate = accumulate;
    return launch<false, SB_ROW, false>(p, tiles_2d(N, K), pow2, stream);
}

hipError_t fg_launch_gemm_grouped(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw,
                                  const int32_t* offsets, int32_t G, int64_t T, int64_t N, int64_t K, void* y,
                                  int out_bf16, int pow2, hipStream_t stream) {
    GemmParams p{};
    p.a = xq; p.sa = sx; p.sa_ld = T; p.b = wq; p.sb = sw;
    p.M = T; p.N = N; p.K = K; p.out = y; p.out_bf16 = out_bf16;
    p.offsets = offsets; p.G = G;
    p.b_group_stride = N * K;
    p.sb_group_stride = ((N + 127) / 128) * (K / 128);
    const int64_t n_tiles = (N + BN - 1) / BN;
    const int64_t m_tiles_max = (T + BM - 1) / BM + G;
    return launch<false, SB_BLOCK, true>(p, (unsigned)(m_tiles_max * n_tiles), pow2, stream);
}
