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
// MFMAs of one row of 16x16 tiles run while the VALU promotes the previous row, inside each wave.
// With power-of-two scales the MFMA's own E8M0 scale operands apply them and the partial goes straight
// into the FP32 accumulator.
//
// Two workgroup shapes, chosen per launch (the one whose tiles fill the 256 CUs in the fewest rounds of
// equal work):
//   256 x 192 x 128, 12 waves (4 x 3) of 64 x 64: 3 waves per SIMD, 64 accumulator VGPRs per wave;
//   256 x 256 x 128,  8 waves (2 x 4) of 128 x 64: 2 waves per SIMD, 128 accumulator VGPRs per wave; a
//                     wave reads 25% fewer LDS bytes per MFMA, which also lowers the LDS power that
//                     competes with the matrix cores for the chip's clock.
// Operand tiles go HBM -> LDS with buffer_load_dwordx4 ... lds (no register staging), double-buffered. The
// next K step's loads are issued in pieces ahead of the current step's first MFMA rows. LDS rows are 16 B-chunk
// swizzled so fragment reads are bank-conflict-free. The MFMA is issued with the B-role fragment first, so
// each lane ends up with one output row m and four consecutive output columns n. The 256 x 256 shape
// re-lays each wave's finished tile in LDS and stores it in full rows (a compute unit streams 16-row x
// 64-byte stores at a third of the rate of full-row ones); the 256 x 192 shape and tiles that run past N
// store straight from that layout (8 B bf16 / 16 B fp32 per lane).
//
// Variants:
//   B_TRANS   B is stored [K][N] (the weight W[N_contr][K_out] read by Dgrad): the tile lands in LDS as
//             [128 contraction rows][BN bytes] and fragments are read with ds_read_b64_tr_b8, the
//             transposed LDS read (the capability the gnrental.net page asks future hardware for).
//   SB_BLOCK  sB = sw[n/128][b]           (Fprop / grouped: 128x128 weight blocks)
//   SB_BLOCK_T sB = sw[b][n/128]          (Dgrad: the same blocks, read along the other axis)
//   SB_ROW    sB = sb[b][n]               (Wgrad: 1x128 tiles along tokens on both operands)
//   GRP_ROWS  rows split into per-group segments given by device offsets, B and sB per group (grouped
//             Fprop, grouped Dgrad of the MoE experts).
//   GRP_K     the contraction split into per-group token segments given by device offsets (multiples of
//             128), one output matrix per group (grouped Wgrad of the MoE experts).
#include <stdlib.h>
#include <string.h>

#include "common.h"
#include "host_util.h"

namespace {

constexpr int BK = 128;

template <int WAVES_M_, int WAVES_N_, int WAVE_M_, int WAVE_N_>
struct TileCfg {
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int WAVE_M = WAVE_M_, WAVE_N = WAVE_N_;
    static constexpr int NW = WAVES_M * WAVES_N;
    static constexpr int NTHREADS = NW * 64;
    static constexpr int BM = WAVES_M * WAVE_M, BN = WAVES_N * WAVE_N;
    static constexpr int MSUB = WAVE_M / 16, NSUB = WAVE_N / 16;
    static constexpr int STAGE_A = BM * BK;
    static constexpr int STAGE_B = BN * BK;             // NT: [BN][128 B]; transposed: [128][BN B]
    static constexpr int SCALES_A = BM * 4, SCALES_B = BN * 4;
    static constexpr int STAGE = STAGE_A + STAGE_B + SCALES_A + SCALES_B;
    static constexpr int LDS_BYTES = 2 * STAGE;
    // direct-to-LDS 16-byte load instructions per stage (1 KB each) and per wave
    static constexpr int LA = STAGE_A / 1024, LB = STAGE_B / 1024;
    static constexpr int UA = (LA + NW - 1) / NW, UB = (LB + NW - 1) / NW;
    static constexpr int SLICES_A = BM / 64, SLICES_B = BN / 64;   // 64-float scale slices
    static constexpr int LOADS_PER_WAVE = UA + UB + 1;
    static_assert(SLICES_A + SLICES_B <= NW, "one scale slice per wave");
    static_assert(BN % 16 == 0 && BN <= 256, "transposed B rows hold at most 16 chunks");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};
using Cfg12 = TileCfg<4, 3, 64, 64>;   // 256 x 192
using Cfg8 = TileCfg<2, 4, 128, 64>;   // 256 x 256

enum { SB_BLOCK = 0, SB_BLOCK_T = 1, SB_ROW = 2 };
enum { GRP_NONE = 0, GRP_ROWS = 1, GRP_K = 2 };
enum { EPI_STORE = 0, EPI_QUANT = 1 };

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
    int64_t out_group_stride; // GRP_K: elements between consecutive groups' outputs
    uint8_t* q_out;           // EPI_QUANT: E4M3 codes of the BF16 output [M][N]
    float* s_out;             // EPI_QUANT: their 1x128 scales [N/128][M]
    int q_pow2;               // EPI_QUANT: power-of-2 output scales
};

// LDS swizzles. gfx950 serves a ds_read_b128 16 lanes (256 B, all 64 banks) at a time, and the 8 rows
// one direct-load instruction writes as 128 B per row. For a [rows][128 B] tile the 16 B chunk c of row r
// is stored at c ^ swz128(r): rows r..r+15 read at one logical chunk land on 16 distinct (row parity,
// chunk) bank groups.
__device__ __forceinline__ int swz128(int r) { return (r & 7) ^ ((r >> 3) & 1); }
// Transposed B tile [128 contraction rows][BN B]. ds_read_b64_tr_b8 serves 32 lanes at a time: rows
// r..r+7 and r+32..r+39 (r a multiple of 8), 16 B of one logical chunk each. With a 192 B row stride the
// rows already spread over the bank window and moving the two low chunk bits suffices; with a 256 B stride
// every row starts at bank 0, so the chunk is XORed with all 16 distinct values (r & 7) | ((r >> 5 & 1) << 3).
template <int BN>
__device__ __forceinline__ int swzT(int r) {
    if constexpr (BN == 256) return (r & 7) | (((r >> 5) & 1) << 3);
    return ((r >> 2) & 1) | (((r >> 5) & 1) << 1);
}

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

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup b runs on XCD b % 8, each XCD with its
// own L2). Map workgroup b of a grid of `total` to a logical tile id so that every XCD holds one contiguous
// range of ids: XCD x gets ids [x * (total / 8) + min(x, total % 8), ...), one per workgroup it runs.
__device__ __forceinline__ int xcd_remap(int b, int total) {
    const int x = b & 7, local = b >> 3;
    const int base = total >> 3, extra = total & 7;
    return x * base + (x < extra ? x : extra) + local;
}

// Raw buffer descriptor over [base, base + 2^32 - 1): stride 0, no swizzle; the range check never
// triggers for the 32-bit offsets the kernels use (the host bounds the sizes so they stay below 2^32).
// The base is wave-uniform by construction; taking it through readfirstlane states so, and the descriptor
// then lives in SGPRs without a per-lane loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t fg_buffer_rsrc(const void* base) {
    const uint64_t u = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    void* b = (void*)(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(b, (short)0, (int)0xFFFFFFFFu, 0x00020000);
}

// 16-byte direct-to-LDS buffer load (lane l lands at byte 16 l of the LDS destination). The call is
// compiled in the device pass only: the host pass checks this builtin's size operand against its own
// target, rejects 16 without a diagnostic and then drops every kernel that uses it from the host object.
__device__ __forceinline__ void fg_buffer_load_lds16(__amdgpu_buffer_rsrc_t rs, void* lds, uint32_t voffset) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, FG_LDS(lds), 16, voffset, 0, 0, 0);
#endif
}

template <bool B>
struct fg_bool {
    static constexpr bool value = B;
};

// A device-resident group offset clamped into [lo, hi].
__device__ __forceinline__ int64_t fg_clamp_offset(int32_t v, int64_t lo, int64_t hi) {
    const int64_t x = v;
    return x < lo ? lo : (x > hi ? hi : x);
}

// E8M0 code of an fp32 power of two in [2^-126, 2^127]: its biased exponent field. `bad` collects the bits
// that a power-of-two scale never has (sign and mantissa), so a power-of-2 launch handed other scales can
// poison its outputs instead of silently dropping the mantissas.
__device__ __forceinline__ int e8m0_of(float s, uint32_t& bad) {
    const uint32_t u = __float_as_uint(s);
    bad |= u & 0x807FFFFFu;
    return (int)(u >> 23) & 0xFF;
}

// STREAM: the output tile is stored past the caches (chosen per launch, see launch()); a compile-time
// choice because the compiler folds a run-time choice between an ordinary and a non-temporal store of the
// same value into one ordinary store.
template <class C, bool B_TRANS, int SBK, int GROUP, bool POW2, int EPI = EPI_STORE, bool STREAM = false>
__global__ __launch_bounds__(C::NTHREADS, 1) void fg_gemm_kernel(GemmParams p) {
    constexpr int BM = C::BM, BN = C::BN, NW = C::NW, MSUB = C::MSUB, NSUB = C::NSUB;
    constexpr int WAVE_M = C::WAVE_M, WAVE_N = C::WAVE_N;
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int64_t N = p.N, K = p.K;
    const int64_t lda = K;
    const bool vec_ok = (N & 3) == 0;       // output rows are 16 B (fp32) / 8 B (bf16) aligned
    const int nkb_all = (int)(K / BK);      // 128-blocks of the whole contraction (block-scale layout)
    int nkb = nkb_all;                      // K steps of this tile

    // ---------------- tile assignment ----------------
    int64_t m0, m_end, n0;
    const uint8_t* Ap = p.a;
    const uint8_t* Bp = p.b;
    const float* SAp = p.sa;
    const float* SBp = p.sb;
    void* outp = p.out;
    const int n_tiles = (int)((N + BN - 1) / BN);
    if constexpr (GROUP == GRP_K) {
        // tile id = g * (tiles per group) + local tile; the group's token segment [off[g], off[g+1]) is the
        // contraction, a whole number of 128-blocks
        const int m_tiles = (int)((p.M + BM - 1) / BM);
        const int tpg = m_tiles * n_tiles;
        // consecutive workgroups (different XCDs) share a group: the groups' contraction lengths differ
        // widely, and keeping one group on one XCD would leave that XCD with the longest tiles
        const int g = blockIdx.x / tpg;
        const int local = blockIdx.x % tpg;
        // offsets outside [0, T] are clamped into it and a decreasing pair is an empty group, so malformed
        // offsets give wrong sums but never an access outside the operands
        const int64_t seg0 = fg_clamp_offset(p.offsets[g], 0, K);
        const int64_t seg1 = fg_clamp_offset(p.offsets[g + 1], seg0, K);
        const int64_t kb0 = seg0 / BK;
        nkb = (int)((seg1 - seg0) / BK);
        const int mt = local % m_tiles, nt = local / m_tiles;
        m0 = (int64_t)mt * BM;
        m_end = p.M;
        n0 = (int64_t)nt * BN;
        Ap += kb0 * BK;
        Bp += kb0 * BK;
        SAp += kb0 * p.sa_ld;
        SBp += kb0 * N;
        outp = reinterpret_cast<float*>(p.out) + (int64_t)g * p.out_group_stride;
    } else if constexpr (GROUP == GRP_ROWS) {
        // Grouped Fprop: rows of N tiles are dealt to the XCDs in turn (row k to XCD k % 8), so an XCD keeps
        // an M tile's N tiles together and the trailing no-op ids of the worst-case grid (a multiple of 8
        // rows) spread over all XCDs; 3-4% faster on the MoE up-projection. (Bands of 4 rows walked column by
        // column, so that the tiles an XCD runs at once form a 4 x 8 block, halve the MoE down-projection's
        // HBM-side traffic but make it 6% slower, and leave the up-projection unchanged.) Grouped Dgrad keeps
        // the launch order, which deals an M tile's N tiles over the XCDs: each XCD then reuses its share of
        // the transposed weight panel across M tiles (2-3% faster there than dealing whole rows, 3% faster
        // than bands of 4 rows).
        int id = (int)blockIdx.x;
        if constexpr (!B_TRANS) {
            const int b = id, x = b & 7, j = b >> 3;
            id = ((j / n_tiles) * 8 + x) * n_tiles + j % n_tiles;
        }
        const int id_m = id / n_tiles;
        const int nt = id % n_tiles;
        int g = 0, cum = 0;
        int64_t seg0 = 0, seg1 = 0;
        for (; g < p.G; g++) {
            // clamped into [0, T] as in the grouped Wgrad: malformed offsets stay inside the operands
            seg0 = fg_clamp_offset(p.offsets[g], 0, p.M);
            seg1 = fg_clamp_offset(p.offsets[g + 1], seg0, p.M);
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
        // each XCD runs a contiguous range of logical tiles, so the tiles it runs at the same time share A
        // and B panels in its own L2
        const int id = xcd_remap((int)blockIdx.x, total);
        // groups of GM M tiles: tiles in flight together on an XCD form a compact block of the output (4 x 8
        // tiles of 256x192 and 8 x 4 tiles of 256x256 are the near-square blocks; both measured best)
        const int GM = C::NW == 12 ? 4 : 8;
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

    // LDS stage st: [A][B][A scales (BM floats)][B scales (BN floats, per-row B scales only)]
    auto stA = [&](int st) { return smem + st * C::STAGE; };
    auto stB = [&](int st) { return smem + st * C::STAGE + C::STAGE_A; };
    auto stSA = [&](int st) { return reinterpret_cast<float*>(smem + st * C::STAGE + C::STAGE_A + C::STAGE_B); };
    auto stSB = [&](int st) {
        return reinterpret_cast<float*>(smem + st * C::STAGE + C::STAGE_A + C::STAGE_B + C::SCALES_A);
    };

    // ---------------- global -> LDS load plan (per thread, fixed over K) ----------------
    // Each direct-to-LDS 16-byte load instruction fills 1 KB of LDS: lane l lands at byte 16 l of it.
    // A: LA instructions of 8 rows (instruction t: rows 8t .. 8t+7); wave w issues t = w + NW u. A wave
    // with fewer instructions than UA re-issues its previous one (same source, same LDS bytes: harmless),
    // which keeps every wave's issue sequence identical and branch-free.
    // Lane l lands at row 8t + l/8, physical chunk l%8, and fetches logical chunk (l%8) ^ swz128(row).
    // Offsets are relative to wave-uniform tile bases (SGPRs) and fit in 32 bits.
    const uint8_t* a_tile = Ap + m0 * lda;
    uint32_t a_off[C::UA];
    int a_t[C::UA];
#pragma unroll
    for (int u = 0; u < C::UA; u++) {
        int t = wave + NW * u;
        t = t < C::LA ? t : t - NW;
        a_t[u] = t;
        const int row = t * 8 + (lane >> 3);
        const int lch = (lane & 7) ^ swz128(row);
        int64_t gr = m0 + row;
        gr = gr < m_end ? gr : m_end - 1;
        a_off[u] = (uint32_t)((gr - m0) * lda + lch * 16);
    }
    // B (NT): LB instructions of 8 rows. B (transposed): [128][BN B], LB instructions of 1 KB; flat 16 B
    // slot f = 64 t + l is row f / (BN/16), physical chunk f % (BN/16), holding logical chunk
    // pch ^ swzT(row) (output columns 16 * logical ..).
    const uint8_t* b_tile;
    uint32_t b_off[C::UB];
    int b_t[C::UB];
#pragma unroll
    for (int u = 0; u < C::UB; u++) {
        int t = wave + NW * u;
        t = t < C::LB ? t : t - NW;
        b_t[u] = t;
    }
    if constexpr (!B_TRANS) {
        b_tile = Bp + n0 * K;
#pragma unroll
        for (int u = 0; u < C::UB; u++) {
            const int row = b_t[u] * 8 + (lane >> 3);
            const int lch = (lane & 7) ^ swz128(row);
            int64_t gr = n0 + row;
            gr = gr < N ? gr : N - 1;
            b_off[u] = (uint32_t)((gr - n0) * K + lch * 16);
        }
    } else {
        b_tile = Bp;
        constexpr int CPR = BN / 16;          // 16 B chunks per transposed row
#pragma unroll
        for (int u = 0; u < C::UB; u++) {
            const int f = b_t[u] * 64 + lane;
            const int row = f / CPR, pch = f % CPR;
            const int lch = pch ^ swzT<BN>(row);
            int64_t gc = n0 + lch * 16;
            gc = gc < N ? gc : N - 16;
            b_off[u] = (uint32_t)((int64_t)row * N + gc);
        }
    }
    // Scales of one K step: slice s (64 floats) of the tile's BM A rows (s < SLICES_A) or, for per-row B
    // scales, of its BN B rows. Wave w loads slice w; waves past the last slice re-load an A slice. Rows
    // past the end re-read the last valid row.
    const int n_slices = SBK == SB_ROW ? C::SLICES_A + C::SLICES_B : C::SLICES_A;
    const int sc_slice = wave < n_slices ? wave : wave % C::SLICES_A;
    const bool sc_is_b = SBK == SB_ROW && sc_slice >= C::SLICES_A;
    int64_t sc_row;
    if (sc_is_b) {
        sc_row = n0 + (sc_slice - C::SLICES_A) * 64 + lane;
        sc_row = sc_row < N ? sc_row : N - 1;
    } else {
        sc_row = m0 + sc_slice * 64 + lane;
        sc_row = sc_row < p.sa_ld ? sc_row : p.sa_ld - 1;
    }
    const int sc_dst = sc_is_b ? C::SCALES_A + (sc_slice - C::SLICES_A) * 256 : sc_slice * 256;

    // Load q of the wave's LOADS_PER_WAVE for K step kb into stage st: A instructions, then B, then the
    // scale slice. `issue_piece(kb, st, i)` issues the i-th of MSUB near-equal pieces of that sequence.
    // Buffer-descriptor form of the direct-to-LDS loads: a wave-uniform base (rebuilt per K step in SGPRs)
    // plus the lane's 32-bit offset. Unlike the global form, which the compiler must treat as a pending
    // LDS access of unknown order, it leaves the LDS fragment reads countable one by one, so a wait for
    // one fragment does not also wait for the fragments read ahead of it.
    const uint32_t sc_off = (uint32_t)(sc_row * 4);
    auto issue_load = [&](int kb, int st, int q) {
        if (q < C::UA) {
            const auto rs = fg_buffer_rsrc(a_tile + (int64_t)kb * BK);
            fg_buffer_load_lds16(rs, stA(st) + a_t[q] * 1024, a_off[q]);
        } else if (q < C::UA + C::UB) {
            const int u = q - C::UA;
            const auto rs = fg_buffer_rsrc(B_TRANS ? b_tile + (int64_t)kb * BK * N : b_tile + (int64_t)kb * BK);
            fg_buffer_load_lds16(rs, stB(st) + b_t[u] * 1024, b_off[u]);
        } else {
            const auto rs = fg_buffer_rsrc(sc_is_b ? SBp + (int64_t)kb * N : SAp + (int64_t)kb * p.sa_ld);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, FG_LDS(reinterpret_cast<uint8_t*>(stSA(st)) + sc_dst), 4, sc_off,
                                                     0, 0, 0);
        }
    };

    // Pieces go out ahead of the first F MFMA rows of the step (loads issued early have longer to land;
    // loads spread out disturb the MFMA stream less). Measured per kernel on the dense-MLP and MoE GEMMs
    // (same box, each against its neighbours): 256x192: F = 2. 256x256: the FP32-scale Fprop, whose
    // interleaved promotion keeps the VALU busy between MFMAs, F = 4 (2-4% faster than 3, dense and
    // grouped) and the FP32-scale grouped Dgrad (1% faster); the other 128x128-block kernels F = 3; the
    // FP32-scale Wgrad spreads them over every row but the last (the loads must be out before the step's
    // hand-over barrier), the power-of-2 Wgrad F = 3 (5% faster than spreading).
    constexpr int F = C::NW == 12 ? 2
                    : SBK == SB_ROW ? (POW2 ? 3 : MSUB - 1)
                    : (!POW2 && (!B_TRANS || GROUP == GRP_ROWS)) ? 4 : 3;
    static_assert(F <= MSUB - 1, "the next stage's loads are all issued before the last row's hand-over barrier");
    // A wave raises its priority while it issues a row of MFMAs, so the SIMD keeps the matrix core fed
    // ahead of the other waves' loads and LDS reads (measured inside the training step: Fprop 2-3% faster,
    // Dgrad 3-5%, Wgrad unchanged).
    constexpr int MFMA_PRIO = 3;
    auto issue_piece = [&](int kb, int st, int piece) {
        if (piece < F) {
#pragma unroll
            for (int q = piece * C::LOADS_PER_WAVE / F; q < (piece + 1) * C::LOADS_PER_WAVE / F; q++)
                issue_load(kb, st, q);
        }
    };

    // ---------------- scale addressing ----------------
    const int lrow = lane & 15;        // output row (m) within a 16x16 tile held by this lane
    const int lcol4 = (lane >> 4) * 4; // first of the 4 output columns (n) held by this lane
    const int64_t wave_n0 = n0 + wn * WAVE_N;
    const int64_t nblocks = (N + 127) / 128;
    int64_t nblk = wave_n0 / 128;                 // a 64-column wave tile never straddles a 128-block
    nblk = nblk < nblocks ? nblk : nblocks - 1;
    auto block_scale = [&](int kb) -> float {
        if constexpr (SBK == SB_BLOCK) return SBp[nblk * nkb_all + kb];
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
        const float* o = reinterpret_cast<const float*>(outp);
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
        tr_off[h] = crow * BN + 8 * (lrow & 1);
        tr_z[h] = swzT<BN>(crow);
    }

    // ---------------- main loop ----------------
    // Step kb computes from stage kb & 1 while the loads of step kb+1 fill the other stage. The barrier that
    // hands the next stage over sits just before each step's last row of MFMAs: every read of the current
    // stage is done by then (the last row's A fragment is already in registers), and the next step's B
    // fragments and first A fragment are read while that last row issues, so no step starts with every
    // wave of the SIMD waiting on LDS. The 128x128 block scale of step kb+1 is fetched one step ahead.
    float sb_next = 1.0f;
    uint32_t bad_scale = 0;                 // power-of-2 mode: sign or mantissa bits seen in any scale
    // Two A register sets fit wherever the promotion leaves 8 registers free; the FP32-scale Wgrad (per-row
    // B scales, two scale products per element) reads each row's fragment just before it.
    constexpr bool AF_AHEAD = POW2 || SBK != SB_ROW;
    v8i bf[NSUB];                           // B-role fragments of the wave's NSUB N tiles, one K step
    float4 sbr[NSUB];                       // per-row B scales (FP32 mode) of the lane's 4 output columns
    int ebr[NSUB];                          // per-row B scales (power-of-2 mode) as E8M0, column lrow
    v8i af_next;                            // the next row's A fragment and A-row scale
    float sa_next = 0.f;
    auto read_b = [&](int st, int j) {
        const uint8_t* sBs = stB(st);
        if constexpr (!B_TRANS) {
            bf[j] = frag_at(sBs + (wn * WAVE_N + j * 16) * BK, frag_lo, frag_hi);
        } else {
            const int chunk = wn * (WAVE_N / 16) + j;
            v2i part[4];
#pragma unroll
            for (int h = 0; h < 4; h++)
                part[h] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) v2i*)(sBs + tr_off[h] + ((chunk ^ tr_z[h]) << 4)));
            bf[j] = v8i{part[0].x, part[0].y, part[1].x, part[1].y, part[2].x, part[2].y, part[3].x, part[3].y};
        }
        if constexpr (SBK == SB_ROW) {
            if constexpr (POW2) ebr[j] = e8m0_of(stSB(st)[wn * WAVE_N + j * 16 + lrow], bad_scale);
            else sbr[j] = *reinterpret_cast<const float4*>(stSB(st) + wn * WAVE_N + j * 16 + lcol4);
        }
    };
    auto read_a0 = [&](int st) {
        af_next = frag_at(stA(st) + wm * WAVE_M * BK, frag_lo, frag_hi);
        sa_next = stSA(st)[wm * WAVE_M + lrow];
    };
    if (nkb > 0) {
#pragma unroll
        for (int q = 0; q < C::LOADS_PER_WAVE; q++) issue_load(0, 0, q);
        sb_next = block_scale(0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        read_a0(0);
#pragma unroll
        for (int j = 0; j < NSUB; j++) read_b(0, j);
    }
    // One K step; MORE: a next step exists (every step but the last), a compile-time flag so that no
    // register set is kept alive across the loop's back edge for a path that leaves the loop.
    auto step = [&](int kb, auto more_tag) {
        constexpr bool more = decltype(more_tag)::value;
        const int st = kb & 1;
        const float sb_blk = sb_next;
        if (more) sb_next = block_scale(kb + 1);
        const uint8_t* sA_w = stA(st) + wm * WAVE_M * BK;
        const float* sSA_w = stSA(st) + wm * WAVE_M + lrow;
        // Row i's A fragment and A-row scale (the scale is read with the fragment, so waiting for one never
        // waits for reads issued after it). The last row's is in registers before the hand-over barrier.
        auto next_af = [&](int i, float& sa) -> v8i {
            if constexpr (AF_AHEAD) {
                const v8i af = af_next;
                sa = sa_next;
                if (i + 1 < MSUB) {
                    af_next = frag_at(sA_w + (i + 1) * 16 * BK, frag_lo, frag_hi);
                    sa_next = sSA_w[(i + 1) * 16];
                }
                return af;
            } else {
                sa = i == 0 ? sa_next : sSA_w[i * 16];
                return i == 0 ? af_next : frag_at(sA_w + i * 16 * BK, frag_lo, frag_hi);
            }
        };
        // Before the last row: wait for this wave's loads of the next stage, then for every wave's.
        // The scheduling fences keep the compiler from moving MFMAs of the earlier rows past the barrier
        // (which would shorten the time the next stage's loads have to land).
        auto hand_over = [&](int i) {
            if (more && i == MSUB - 1) {
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (AF_AHEAD) read_a0(st ^ 1);
            }
        };
        // After the last row's MFMA j has issued, its B fragment register takes the next step's.
        auto after_mfma = [&](int i, int j) {
            if (more && i == MSUB - 1) {
                read_b(st ^ 1, j);
                if constexpr (!AF_AHEAD)
                    if (j == NSUB - 1) read_a0(st ^ 1);
            }
        };
        auto load_piece = [&](int i) {
            if (more) issue_piece(kb + 1, st ^ 1, i);
        };
        if constexpr (POW2) {
            // Power-of-two scales: the matrix core applies them itself. Per lane l the E8M0 scale operand
            // of a 16x128 fragment scales row l%16 (all four 32-element K sub-blocks of the lane carry the
            // same scale), so the A-role operand takes the row scale of output row m and the B-role
            // operand the block scale (or, with per-row B scales, the scale of output column n); the MFMA
            // adds 2^(ea+eb) * P_b straight into the FP32 accumulator, with no VALU promotion.
            const int eb_blk = SBK == SB_ROW ? 0 : e8m0_of(sb_blk, bad_scale);
#pragma unroll
            for (int i = 0; i < MSUB; i++) {
                load_piece(i);
                float sa_i;
                const v8i af = next_af(i, sa_i);
                const int ea = e8m0_of(sa_i, bad_scale);
                hand_over(i);
                if constexpr (MFMA_PRIO) __builtin_amdgcn_s_setprio(MFMA_PRIO);
#pragma unroll
                for (int j = 0; j < NSUB; j++) {
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        bf[j], af, acc[i][j], 0, 0, 0, SBK == SB_ROW ? ebr[j] : eb_blk, 0, ea);
                    after_mfma(i, j);
                }
                if constexpr (MFMA_PRIO) __builtin_amdgcn_s_setprio(0);
            }
        } else {
            // VALU promotion, software-pipelined so that no FMA reads the result of the MFMA issued just
            // before it (a VALU read of an MFMA result waits for the whole MFMA). With registers to spare
            // (8-wave shape, one scale per lane) the FMAs that fold row i-1 into the FP32 accumulators go
            // with the MFMAs of row i, four after each MFMA, so that the wave's own VALU work runs while its
            // MFMAs execute; the wave keeps its raised priority through the FMAs (measured 2-3% faster on
            // the FP32-scale Fprop and Dgrad than issuing the row's MFMAs first and its FMAs after); otherwise
            // the FMAs of each tile follow the next tile's MFMA.
            constexpr bool ROW_PIPE = C::NW == 8 && SBK != SB_ROW;
            if constexpr (ROW_PIPE) {
                v4f prev[NSUB], cur[NSUB];
                float sa_prev = 0.f;
#pragma unroll
                for (int i = 0; i <= MSUB; i++) {
                    float sa_i = 0.f;
                    if (i < MSUB) {
                        load_piece(i);
                        const v8i af = next_af(i, sa_i);
                        hand_over(i);
                        if constexpr (MFMA_PRIO) __builtin_amdgcn_s_setprio(MFMA_PRIO);
#pragma unroll
                        for (int j = 0; j < NSUB; j++) {
                            cur[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af, v4f{0.f, 0.f, 0.f, 0.f},
                                                                                     0, 0, 0, 127, 0, 127);
                            after_mfma(i, j);
                        }
                    }
                    if (i > 0) {
                        const float s = sa_prev * sb_blk;
#pragma unroll
                        for (int j = 0; j < NSUB; j++)
#pragma unroll
                            for (int r = 0; r < 4; r++) acc[i - 1][j][r] = __builtin_fmaf(prev[j][r], s, acc[i - 1][j][r]);
                    }
                    // the interleave (not in the hand-over row, whose MFMAs sit behind scheduling fences)
                    if (i > 0 && i < MSUB - 1) {
#pragma unroll
                        for (int j = 0; j < NSUB; j++) {
                            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // four VALU operations
                        }
                    }
                    if (i < MSUB) {
                        if constexpr (MFMA_PRIO) __builtin_amdgcn_s_setprio(0);
                    }
#pragma unroll
                    for (int j = 0; j < NSUB; j++) prev[j] = cur[j];
                    sa_prev = sa_i;
                }
            } else {
                // Tile-lagged promotion: the FMAs issued after MFMA t fold tile t - LAG, whose result is long
                // complete. Per-row B scales (two scale products per element) take the deeper lag where the
                // registers allow it (8-wave shape); measured 3-4% faster on Wgrad than folding tile t - 1,
                // and neutral on the 256x192 Fprop. The 12-wave shape's Wgrad (168 VGPRs per wave) folds
                // tile t - 1: one more pending tile there spills registers to scratch.
                constexpr int LAG = SBK != SB_ROW ? 2 : C::NW == 8 ? 3 : 1;
                v4f pend[LAG];
                float pend_s[LAG][4];
                int pend_i[LAG], pend_j[LAG];
#pragma unroll
                for (int l = 0; l < LAG; l++) pend_i[l] = -1;
#pragma unroll
                for (int i = 0; i < MSUB; i++) {
                    load_piece(i);
                    float sa_i;
                    const v8i af = next_af(i, sa_i);
                    hand_over(i);
#pragma unroll
                    for (int j = 0; j < NSUB; j++) {
                        const v4f cur = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            bf[j], af, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
                        constexpr int O = LAG - 1;    // the oldest pending tile
                        if (pend_i[O] >= 0) {
#pragma unroll
                            for (int r = 0; r < 4; r++)
                                acc[pend_i[O]][pend_j[O]][r] =
                                    __builtin_fmaf(pend[O][r], pend_s[O][r], acc[pend_i[O]][pend_j[O]][r]);
                        }
#pragma unroll
                        for (int l = O; l > 0; l--) {
                            pend[l] = pend[l - 1];
                            pend_i[l] = pend_i[l - 1];
                            pend_j[l] = pend_j[l - 1];
#pragma unroll
                            for (int r = 0; r < 4; r++) pend_s[l][r] = pend_s[l - 1][r];
                        }
                        pend[0] = cur;
                        pend_i[0] = i;
                        pend_j[0] = j;
                        if constexpr (SBK != SB_ROW) {
                            const float s_ij = sa_i * sb_blk;
                            pend_s[0][0] = pend_s[0][1] = pend_s[0][2] = pend_s[0][3] = s_ij;
                        } else {
                            pend_s[0][0] = sa_i * sbr[j].x;
                            pend_s[0][1] = sa_i * sbr[j].y;
                            pend_s[0][2] = sa_i * sbr[j].z;
                            pend_s[0][3] = sa_i * sbr[j].w;
                        }
                        after_mfma(i, j);
                    }
                }
#pragma unroll
                for (int l = LAG - 1; l >= 0; l--)
#pragma unroll
                    for (int r = 0; r < 4; r++)
                        acc[pend_i[l]][pend_j[l]][r] = __builtin_fmaf(pend[l][r], pend_s[l][r], acc[pend_i[l]][pend_j[l]][r]);
            }
        }
    };
    for (int kb = 0; kb + 1 < nkb; kb++) step(kb, fg_bool<true>{});
    if (nkb > 0) step(nkb - 1, fg_bool<false>{});

    __builtin_amdgcn_s_waitcnt(0);
    if constexpr (POW2) {
        // A scale that is not a positive power of two was applied without its mantissa: the wave's whole
        // output tile becomes NaN, so the misuse shows instead of giving plausible wrong sums.
        if (__builtin_amdgcn_ballot_w64(bad_scale != 0) != 0) {
#pragma unroll
            for (int i = 0; i < MSUB; i++)
#pragma unroll
                for (int j = 0; j < NSUB; j++) acc[i][j] = v4f{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                                                               __builtin_nanf("")};
        }
    }
    // ---------------- epilogue ----------------
    if constexpr (EPI == EPI_QUANT) {
        // The BF16 output, quantized 1x128 along its columns exactly as fg_quantize_act_1x128 would quantize
        // it (same max-abs, scale and quotient), without writing or re-reading the BF16 values. A 128-column
        // group is two neighbouring 64-column wave tiles: each wave reduces its half of every row over the 4
        // lanes holding it, and the pair exchange halves through LDS (the stages are idle by now).
        static_assert(WAVE_N == 64 && BN % 128 == 0, "a 128-column group is a pair of 64-column wave tiles");
        __syncthreads();                         // every wave's staging loads and LDS reads are done
        uint32_t* rmax = reinterpret_cast<uint32_t*>(smem);   // [WAVES_N][BM] max |bf16| bits per row half
        uint2 hb[MSUB][NSUB];                    // the lane's 4 BF16 values of each 16x16 tile, packed
#pragma unroll
        for (int i = 0; i < MSUB; i++) {
            uint32_t mx = 0;
#pragma unroll
            for (int j = 0; j < NSUB; j++) {
                hb[i][j].x = bf16_rne_bits(acc[i][j][0]) | (bf16_rne_bits(acc[i][j][1]) << 16);
                hb[i][j].y = bf16_rne_bits(acc[i][j][2]) | (bf16_rne_bits(acc[i][j][3]) << 16);
                mx = fg_pk_max_u16(mx, fg_pk_max_u16(hb[i][j].x & 0x7FFF7FFFu, hb[i][j].y & 0x7FFF7FFFu));
            }
            mx = fg_max_halves(mx);
            uint32_t o = (uint32_t)__shfl_xor((int)mx, 16);  // the 4 lanes holding a row: lane + 16 k
            mx = o > mx ? o : mx;
            o = (uint32_t)__shfl_xor((int)mx, 32);
            mx = o > mx ? o : mx;
            if (lane < 16) rmax[wn * BM + wm * WAVE_M + i * 16 + lrow] = mx;
        }
        __syncthreads();
        // With the whole 256-column tile inside the output (uniform over the workgroup), the codes go
        // through an LDS copy of the tile ([BM][BN B], 16-byte chunk c of row r at c ^ (r % 16)) and every
        // wave stores BM / NW full rows, 4 rows x 256 B per instruction, instead of 16 rows x 16 B from the
        // MFMA layout.
        const bool staged = n0 + BN <= N;
        uint8_t* ctile = smem + C::WAVES_N * BM * 4;
#pragma unroll
        for (int i = 0; i < MSUB; i++) {
            const int row = wm * WAVE_M + i * 16 + lrow;
            const uint32_t a0 = rmax[wn * BM + row], a1 = rmax[(wn ^ 1) * BM + row];
            const float sc = fg_scale_from_amax_bits(a0 > a1 ? a0 : a1, p.q_pow2);
            fg_divisor d = fg_make_divisor(sc, p.q_pow2);
            // the quotient form, as in the standalone quantizer: exact product for pow2 scales, else the
            // corrected quotient, moved up by 2^64 for the rows whose scale is below 2^-100
            const int mode = p.q_pow2 ? FG_Q_POW2
                           : (__builtin_amdgcn_ballot_w64(fg_divisor_tiny(d)) != 0 && fg_divisor_tiny(d)) ? FG_Q_TINY
                                                                                                       : FG_Q_FAST;
            if (mode == FG_Q_TINY) d = fg_divisor_shifted(d);
            const int64_t m = m0 + row;
            const bool row_ok = m < m_end;
#pragma unroll
            for (int j = 0; j < NSUB; j++) {
                const uint32_t lo = hb[i][j].x, hi = hb[i][j].y;
                uint32_t c;
                if (mode == FG_Q_POW2) {
                    c = fg_cvt2q<FG_Q_POW2, false>(fg_bf16_lo(lo), fg_bf16_hi(lo), d, 0);
                    c = fg_cvt2q<FG_Q_POW2, true>(fg_bf16_lo(hi), fg_bf16_hi(hi), d, c);
                } else if (mode == FG_Q_FAST) {
                    c = fg_cvt2q<FG_Q_FAST, false>(fg_bf16_lo(lo), fg_bf16_hi(lo), d, 0);
                    c = fg_cvt2q<FG_Q_FAST, true>(fg_bf16_lo(hi), fg_bf16_hi(hi), d, c);
                } else {
                    c = fg_cvt2q<FG_Q_TINY, false>(fg_bf16_lo(lo), fg_bf16_hi(lo), d, 0);
                    c = fg_cvt2q<FG_Q_TINY, true>(fg_bf16_lo(hi), fg_bf16_hi(hi), d, c);
                }
                const int64_t n = wave_n0 + j * 16 + lcol4;
                if (staged) {
                    const int ch = (wn * (WAVE_N / 16) + j) ^ lrow;
                    *reinterpret_cast<uint32_t*>(ctile + row * BN + ch * 16 + lcol4) = c;
                } else if (row_ok && n < N) {
                    *reinterpret_cast<uint32_t*>(p.q_out + m * N + n) = c;
                }
            }
            if ((wn & 1) == 0 && lane < 16 && row_ok && wave_n0 < N) p.s_out[(wave_n0 >> 7) * p.M + m] = sc;
        }
        if (staged) {
            static_assert(BN == 256 && BM % (4 * NW) == 0, "staged code rows: 16 lanes x 16 B per row");
            __syncthreads();
#pragma unroll
            for (int k = 0; k < BM / (4 * NW); k++) {
                const int r = wave * (BM / NW) + 4 * k + (lane >> 4);
                const int ch = lane & 15;
                const uint4 v = *reinterpret_cast<const uint4*>(ctile + r * BN + ((ch ^ (r & 15)) << 4));
                const int64_t m = m0 + r;
                if (m < m_end) *reinterpret_cast<uint4*>(p.q_out + m * N + n0 + ch * 16) = v;
            }
        }
        return;
    }
    if constexpr (NW == 8 && WAVE_M == 128 && WAVE_N == 64 && C::LDS_BYTES >= NW * 64 * 256) {
        // FP32 output through LDS. In the MFMA layout one 16-byte store per lane writes 16 rows x 64 B, and
        // a compute unit streams such stores at about a third of the rate of stores that write 4 rows x
        // 256 B. Each wave re-lays half of its 128x64 tile (64 rows x 256 B) in a private 16 KB LDS region
        // (16-byte chunk c of row r at c ^ (r % 16): conflict-free for the writes, whose 16 lanes share a
        // chunk and span 16 rows, and for the reads, whose 16 lanes share a row) and stores it 4 rows x
        // 256 B at a time. The values are only moved. The condition is uniform over the workgroup, so every
        // wave reaches the barrier that frees the stages (the last K step's fragment reads are then done).
        // BF16 output: the wave's whole tile (128 rows x 128 B) fits its region; the MFMA layout's 8-byte
        // stores write 16 rows x 32 B, the staged ones 8 full 128 B rows (16-byte chunk c of row r at
        // c ^ ((r / 2) % 8): rows r, r + 1 share a 256 B bank window, so 16 rows of one chunk, or two rows
        // of 8 chunks, cover its 16 chunk slots once).
        if (p.out_bf16 && (N & 7) == 0) {
            __syncthreads();
            if (wave_n0 + WAVE_N <= N) {
                uint8_t* reg = smem + wave * (128 * 128);
                uint16_t* o = reinterpret_cast<uint16_t*>(outp);
#pragma unroll
                for (int i = 0; i < MSUB; i++)
#pragma unroll
                    for (int j = 0; j < NSUB; j++) {
                        const int r = i * 16 + lrow;
                        const int c = (2 * j + (lane >> 5)) ^ ((r >> 1) & 7);
                        uint2 v;
                        v.x = bf16_rne_bits(acc[i][j][0]) | (bf16_rne_bits(acc[i][j][1]) << 16);
                        v.y = bf16_rne_bits(acc[i][j][2]) | (bf16_rne_bits(acc[i][j][3]) << 16);
                        *reinterpret_cast<uint2*>(reg + r * 128 + c * 16 + ((lane >> 4) & 1) * 8) = v;
                    }
#pragma unroll
                for (int k = 0; k < 16; k++) {
                    const int r = 8 * k + (lane >> 3);
                    const int c = lane & 7;
                    const uint4 v = *reinterpret_cast<const uint4*>(reg + r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
                    const int64_t m = m0 + wm * WAVE_M + r;
                    if (m < m_end) {
                        if constexpr (STREAM)   // an output too large to stay cached (see launch())
                            __builtin_nontemporal_store(__builtin_bit_cast(v4i, v), reinterpret_cast<v4i*>(o + m * N + wave_n0 + c * 8));
                        else
                            *reinterpret_cast<uint4*>(o + m * N + wave_n0 + c * 8) = v;
                    }
                }
                return;
            }
        } else if (!p.out_bf16 && vec_ok) {
            __syncthreads();
            if (wave_n0 + WAVE_N <= N) {
                uint8_t* reg = smem + wave * (64 * 256);
                float* o = reinterpret_cast<float*>(outp);
#pragma unroll
                for (int h = 0; h < 2; h++) {
#pragma unroll
                    for (int i = 0; i < 4; i++)
#pragma unroll
                        for (int j = 0; j < NSUB; j++) {
                            const int r = i * 16 + lrow;
                            const int c = (j * 4 + (lane >> 4)) ^ lrow;
                            *reinterpret_cast<v4f*>(reg + r * 256 + c * 16) = acc[h * 4 + i][j];
                        }
#pragma unroll
                    for (int k = 0; k < 16; k++) {
                        const int r = 4 * k + (lane >> 4);
                        const int c = lane & 15;
                        const v4f v = *reinterpret_cast<const v4f*>(reg + r * 256 + ((c ^ (r & 15)) << 4));
                        const int64_t m = m0 + wm * WAVE_M + h * 64 + r;
                        if (m < m_end) {
                            // Streamed past the caches: weight gradients (they go to the optimizer, not
                            // to the next kernel) and outputs too large to stay cached (see launch()).
                            if constexpr (SBK == SB_ROW || STREAM)
                                __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(o + m * N + wave_n0 + c * 4));
                            else
                                *reinterpret_cast<float4*>(o + m * N + wave_n0 + c * 4) = make_float4(v[0], v[1], v[2], v[3]);
                        }
                    }
                }
                return;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < MSUB; i++) {
        const int64_t m = m0 + wm * WAVE_M + i * 16 + lrow;
        if (m >= m_end) continue;
#pragma unroll
        for (int j = 0; j < NSUB; j++) {
            const int64_t n = wave_n0 + j * 16 + lcol4;
            if (p.out_bf16) {
                uint16_t* o = reinterpret_cast<uint16_t*>(outp) + m * N + n;
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
                float* o = reinterpret_cast<float*>(outp) + m * N + n;
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

// ---------------------------------------------------------------------------------------------------------
// Fprop on 256 x 288 x 128 workgroup tiles: 8 waves (4 x 2) of 64 x 144.
//
// The 256 x 256 shape runs one workgroup per CU, so a GEMM takes whole rounds of 256 tiles. The
// DeepSeek-V3-like dense-MLP Fprop (N = 18432) is 4.5 such rounds, and its half-filled last round costs
// nearly as much as a full one; 288 = 18432 / 64 covers the same output in exactly 4 rounds of tiles with
// 12.5% more work each. A 144-column wave tile has 9 B fragments per K step, more than the registers left
// beside its 144 accumulators can hold, so the operand roles of fg_gemm_kernel are swapped: a wave keeps
// its four 16-row A fragments in registers for the whole K step and streams the nine 16-column B
// fragments, each read one strip ahead of its MFMAs. Every output element still takes one scaled MFMA per
// 128-K block and the same promotion (fma(P_b, RN(sA * sB), acc) with FP32 scales, the E8M0 operands
// with power-of-2 scales) in the same block order, so the results equal the other shapes' bit for bit.
// A 144-column wave tile can straddle two 128 x 128 weight blocks: each 16-column strip takes the scale of
// the block it lies in.
struct WideCfg {
    static constexpr int WAVES_M = 4, WAVES_N = 2, WAVE_M = 64, WAVE_N = 144;
    static constexpr int NW = WAVES_M * WAVES_N, NTHREADS = NW * 64;
    static constexpr int BM = WAVES_M * WAVE_M, BN = WAVES_N * WAVE_N;       // 256 x 288
    static constexpr int MSUB = WAVE_M / 16, NSUB = WAVE_N / 16;             // 4 x 9 MFMA tiles per wave
    static constexpr int STAGE_A = BM * BK, STAGE_B = BN * BK, SCALES_A = BM * 4;
    static constexpr int STAGE = STAGE_A + STAGE_B + SCALES_A;
    static constexpr int LA = STAGE_A / 1024, LB = STAGE_B / 1024;
    static constexpr int UA = (LA + NW - 1) / NW, UB = (LB + NW - 1) / NW;
    static constexpr int SLICES_A = BM / 64;
    static constexpr int LOADS_PER_WAVE = UA + UB + 1;
    // epilogue: a wave re-lays 64 rows of BF16 (or 32 rows of FP32) of its tile in a private LDS region
    static constexpr int OUT_REGION = 64 * WAVE_N * 2;
    static constexpr int LDS_BYTES = 2 * STAGE > NW * OUT_REGION ? 2 * STAGE : NW * OUT_REGION;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    static_assert(STAGE % 1024 == 0, "stages start on 1 KB boundaries");
    static_assert(SLICES_A <= NW, "one scale slice per wave");
};

template <bool POW2, bool STREAM>
__global__ __launch_bounds__(WideCfg::NTHREADS, 1) void fg_gemm_wide_kernel(GemmParams p) {
    using C = WideCfg;
    constexpr int BM = C::BM, BN = C::BN, NW = C::NW, MSUB = C::MSUB, NSUB = C::NSUB;
    constexpr int WAVE_M = C::WAVE_M, WAVE_N = C::WAVE_N;
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int nkb = (int)(K / BK);

    // Tile order of fg_gemm_kernel's dense GEMMs: XCD-contiguous ranges of tile ids, walked in groups of 8
    // M tiles, so the tiles an XCD runs at once share A and B panels in its L2.
    const int n_tiles = (int)((N + BN - 1) / BN);
    const int m_tiles = (int)((M + BM - 1) / BM);
    const int id = xcd_remap((int)blockIdx.x, m_tiles * n_tiles);
    constexpr int GM = 8;
    const int group = id / (GM * n_tiles);
    const int first_m = group * GM;
    const int gsz = min(m_tiles - first_m, GM);
    const int within = id - group * GM * n_tiles;
    const int64_t m0 = (int64_t)(first_m + within % gsz) * BM;
    const int64_t n0 = (int64_t)(within / gsz) * BN;

    // LDS stage st: [A: BM rows x 128 B][B: BN rows x 128 B][A scales: BM floats]
    auto stA = [&](int st) { return smem + st * C::STAGE; };
    auto stB = [&](int st) { return smem + st * C::STAGE + C::STAGE_A; };
    auto stSA = [&](int st) { return reinterpret_cast<float*>(smem + st * C::STAGE + C::STAGE_A + C::STAGE_B); };

    // Global -> LDS load plan, as in fg_gemm_kernel: 1 KB (8 rows of 128 B) per direct-to-LDS instruction,
    // instruction t of a wave = wave + NW u (a wave short of instructions re-issues its previous one), lane l
    // at row 8t + l/8 fetching logical 16 B chunk (l % 8) ^ swz128(row); rows past the end re-read the last.
    const uint8_t* a_tile = p.a + m0 * K;
    const uint8_t* b_tile = p.b + n0 * K;
    uint32_t a_off[C::UA], b_off[C::UB];
    int a_t[C::UA], b_t[C::UB];
#pragma unroll
    for (int u = 0; u < C::UA; u++) {
        int t = wave + NW * u;
        t = t < C::LA ? t : t - NW;
        a_t[u] = t;
        const int row = t * 8 + (lane >> 3);
        int64_t gr = m0 + row;
        gr = gr < M ? gr : M - 1;
        a_off[u] = (uint32_t)((gr - m0) * K + (((lane & 7) ^ swz128(row)) << 4));
    }
#pragma unroll
    for (int u = 0; u < C::UB; u++) {
        int t = wave + NW * u;
        t = t < C::LB ? t : t - NW;
        b_t[u] = t;
        const int row = t * 8 + (lane >> 3);
        int64_t gr = n0 + row;
        gr = gr < N ? gr : N - 1;
        b_off[u] = (uint32_t)((gr - n0) * K + (((lane & 7) ^ swz128(row)) << 4));
    }
    // A-row scales of one K step: wave w loads 64-float slice w % SLICES_A of the tile's BM rows
    const int sc_slice = wave % C::SLICES_A;
    int64_t sc_row = m0 + sc_slice * 64 + lane;
    sc_row = sc_row < p.sa_ld ? sc_row : p.sa_ld - 1;
    const uint32_t sc_off = (uint32_t)(sc_row * 4);
    const int sc_dst = sc_slice * 256;
    auto issue_load = [&](int kb, int st, int q) {
        if (q < C::UA) {
            const auto rs = fg_buffer_rsrc(a_tile + (int64_t)kb * BK);
            fg_buffer_load_lds16(rs, stA(st) + a_t[q] * 1024, a_off[q]);
        } else if (q < C::UA + C::UB) {
            const int u = q - C::UA;
            const auto rs = fg_buffer_rsrc(b_tile + (int64_t)kb * BK);
            fg_buffer_load_lds16(rs, stB(st) + b_t[u] * 1024, b_off[u]);
        } else {
            const auto rs = fg_buffer_rsrc(p.sa + (int64_t)kb * p.sa_ld);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, FG_LDS(reinterpret_cast<uint8_t*>(stSA(st)) + sc_dst), 4, sc_off,
                                                     0, 0, 0);
        }
    };
    // The next step's loads go out in F pieces ahead of the first F strips of MFMAs (all before the last
    // strip's hand-over barrier). F = 5 measured best with either scale mode on the dense-MLP Fprop (1-2%
    // faster than 3 or 4 pieces, 3-9% faster than 6 to 8).
    constexpr int F = 5;
    static_assert(F <= NSUB - 1, "the next stage's loads are all issued before the hand-over barrier");
    auto issue_piece = [&](int kb, int st, int piece) {
#pragma unroll
        for (int q = piece * C::LOADS_PER_WAVE / F; q < (piece + 1) * C::LOADS_PER_WAVE / F; q++) issue_load(kb, st, q);
    };

    // Weight block scales: the wave's 144 columns [wave_n0, wave_n0 + 144) lie in blocks blk0 and blk1 =
    // blk0 + 1 (wave_n0 is a multiple of 16, so at most two blocks); strip j lies in blk0 iff 16 j < split.
    const int lrow = lane & 15;
    const int lcol4 = (lane >> 4) * 4;
    const int64_t wave_n0 = n0 + wn * WAVE_N;
    const int64_t nblocks = (N + 127) / 128;
    int64_t blk0 = wave_n0 / 128;
    blk0 = blk0 < nblocks ? blk0 : nblocks - 1;
    const int64_t blk1 = blk0 + 1 < nblocks ? blk0 + 1 : nblocks - 1;
    const int split = 128 - (int)(wave_n0 & 127);
    const float* sb_row0 = p.sb + blk0 * nkb;
    const float* sb_row1 = p.sb + blk1 * nkb;

    v4f acc[MSUB][NSUB];
#pragma unroll
    for (int i = 0; i < MSUB; i++)
#pragma unroll
        for (int j = 0; j < NSUB; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int g16 = lane >> 4;
    const int frag_lo = lrow * BK + (((2 * g16) ^ swz128(lrow)) << 4);
    const int frag_hi = lrow * BK + (((2 * g16 + 1) ^ swz128(lrow)) << 4);

    // ---------------- main loop ----------------
    // Step kb computes from stage kb & 1 while the loads of step kb + 1 fill the other stage. The barrier
    // that hands the next stage over sits before the last strip of MFMAs: that strip's B fragment is already
    // in registers, and the next step's A fragments are read after the MFMAs that last use each register.
    v8i af[MSUB];                     // A fragments of the step, one per 16-row strip
    float sa[MSUB];                   // their row scales (row lrow of each strip)
    v8i bnext;                        // the next strip's B fragment
    float sb0_next = 1.f, sb1_next = 1.f;
    uint32_t bad_scale = 0;           // power-of-2 mode: sign or mantissa bits seen in any scale
    auto read_a = [&](int st, int i) {
        af[i] = frag_at(stA(st) + (wm * WAVE_M + i * 16) * BK, frag_lo, frag_hi);
        sa[i] = stSA(st)[wm * WAVE_M + i * 16 + lrow];
    };
    auto read_b = [&](int st, int j) -> v8i { return frag_at(stB(st) + (wn * WAVE_N + j * 16) * BK, frag_lo, frag_hi); };
    if (nkb > 0) {
#pragma unroll
        for (int q = 0; q < C::LOADS_PER_WAVE; q++) issue_load(0, 0, q);
        sb0_next = sb_row0[0];
        sb1_next = sb_row1[0];
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < MSUB; i++) read_a(0, i);
        bnext = read_b(0, 0);
    }
    // FP32 scales: the wave raises its priority while a strip of MFMAs issues, as in fg_gemm_kernel.
    // Power-of-2 scales keep the default priority (measured on the dense-MLP Fprop: 2% faster there, 2%
    // slower with FP32 scales).
    constexpr int MFMA_PRIO = POW2 ? 0 : 3;
    auto step = [&](int kb, auto more_tag) {
        constexpr bool more = decltype(more_tag)::value;
        const int st = kb & 1;
        const float sb0 = sb0_next, sb1 = sb1_next;
        if (more) {
            sb0_next = sb_row0[kb + 1];
            sb1_next = sb_row1[kb + 1];
        }
        int ea[MSUB];
        int eb0 = 0, eb1 = 0;
        if constexpr (POW2) {
#pragma unroll
            for (int i = 0; i < MSUB; i++) ea[i] = e8m0_of(sa[i], bad_scale);
            eb0 = e8m0_of(sb0, bad_scale);
            eb1 = e8m0_of(sb1, bad_scale);
        }
        // FP32 scales: tile-lagged promotion, the FMAs issued after MFMA t folding tile t - 4 (a VALU read of
        // an MFMA result waits for the whole MFMA). Measured on the dense-MLP Fprop against lags of 2 and 3
        // and against interleave hints (one MFMA, five VALU operations): 3-5% faster than a lag of 2, and the
        // only one faster than the 256 x 256 shape; the pending tiles fill the register file to its 256.
        constexpr int LAG = 4;
        v4f pend[LAG];
        float pend_s[LAG];
        int pend_i[LAG], pend_j[LAG];
#pragma unroll
        for (int l = 0; l < LAG; l++) pend_i[l] = -1;
#pragma unroll
        for (int j = 0; j < NSUB; j++) {
            if (more && j < F) issue_piece(kb + 1, st ^ 1, j);
            const v8i bcur = bnext;
            if (j + 1 < NSUB) bnext = read_b(st, j + 1);
            constexpr int LAST = NSUB - 1;
            if (more && j == LAST) {
                // every read of this stage is done and this wave's next-stage loads have landed; then every
                // wave's (the fences keep earlier MFMAs from moving past the barrier)
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                __builtin_amdgcn_sched_barrier(0);
            }
            const bool in0 = 16 * j < split;
            if constexpr (MFMA_PRIO) __builtin_amdgcn_s_setprio(MFMA_PRIO);
#pragma unroll
            for (int i = 0; i < MSUB; i++) {
                if constexpr (POW2) {
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bcur, af[i], acc[i][j], 0, 0, 0,
                                                                                in0 ? eb0 : eb1, 0, ea[i]);
                } else {
                    const v4f cur = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bcur, af[i], v4f{0.f, 0.f, 0.f, 0.f},
                                                                                     0, 0, 0, 127, 0, 127);
                    constexpr int O = LAG - 1;
                    if (pend_i[O] >= 0) {
#pragma unroll
                        for (int r = 0; r < 4; r++)
                            acc[pend_i[O]][pend_j[O]][r] = __builtin_fmaf(pend[O][r], pend_s[O], acc[pend_i[O]][pend_j[O]][r]);
                    }
#pragma unroll
                    for (int l = O; l > 0; l--) {
                        pend[l] = pend[l - 1];
                        pend_s[l] = pend_s[l - 1];
                        pend_i[l] = pend_i[l - 1];
                        pend_j[l] = pend_j[l - 1];
                    }
                    pend[0] = cur;
                    pend_s[0] = sa[i] * (in0 ? sb0 : sb1);
                    pend_i[0] = i;
                    pend_j[0] = j;
                }
                if (more && j == LAST) read_a(st ^ 1, i);
            }
            if constexpr (MFMA_PRIO) __builtin_amdgcn_s_setprio(0);
            if (more && j == LAST) bnext = read_b(st ^ 1, 0);
        }
        if constexpr (!POW2) {
#pragma unroll
            for (int l = LAG - 1; l >= 0; l--)
#pragma unroll
                for (int r = 0; r < 4; r++)
                    acc[pend_i[l]][pend_j[l]][r] = __builtin_fmaf(pend[l][r], pend_s[l], acc[pend_i[l]][pend_j[l]][r]);
        }
    };
    for (int kb = 0; kb + 1 < nkb; kb++) step(kb, fg_bool<true>{});
    if (nkb > 0) step(nkb - 1, fg_bool<false>{});

    __builtin_amdgcn_s_waitcnt(0);
    if constexpr (POW2) {
        // a scale that is not a positive power of two: the wave's whole output tile becomes NaN
        if (__builtin_amdgcn_ballot_w64(bad_scale != 0) != 0) {
#pragma unroll
            for (int i = 0; i < MSUB; i++)
#pragma unroll
                for (int j = 0; j < NSUB; j++) acc[i][j] = v4f{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                                                               __builtin_nanf("")};
        }
    }

    // ---------------- epilogue ----------------
    // A wave whose 144 columns lie inside the output re-lays its tile in a private LDS region (64 rows of
    // 288 B for BF16; FP32 in two halves of 32 rows of 576 B) and stores it as contiguous 16-byte chunks:
    // the region is dense, so chunk f of it is row f / (chunks per row), and one store instruction writes
    // whole 288 B or 576 B row segments instead of 16 rows x 32 B (BF16) or 16 rows x 64 B (FP32) from the
    // MFMA layout. The values are only moved. The condition of the barrier is uniform over the workgroup.
    const bool bf16 = p.out_bf16 != 0;
    if (bf16 ? (N & 7) == 0 : (N & 3) == 0) {
        __syncthreads();                    // the stages are free: every wave's last fragment reads are done
        if (wave_n0 + WAVE_N <= N) {
            uint8_t* reg = smem + wave * C::OUT_REGION;
            const int64_t mw = m0 + wm * WAVE_M;
            if (bf16) {
                constexpr int RB = WAVE_N * 2, CPR = RB / 16;          // 288 B, 18 chunks per row
                uint16_t* o = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
                for (int i = 0; i < MSUB; i++)
#pragma unroll
                    for (int j = 0; j < NSUB; j++) {
                        uint2 v;
                        v.x = bf16_rne_bits(acc[i][j][0]) | (bf16_rne_bits(acc[i][j][1]) << 16);
                        v.y = bf16_rne_bits(acc[i][j][2]) | (bf16_rne_bits(acc[i][j][3]) << 16);
                        *reinterpret_cast<uint2*>(reg + (i * 16 + lrow) * RB + (j * 16 + lcol4) * 2) = v;
                    }
#pragma unroll
                for (int k = 0; k < 64 * CPR / 64; k++) {
                    const int f = 64 * k + lane;
                    const int r = f / CPR, c = f % CPR;
                    const uint4 v = *reinterpret_cast<const uint4*>(reg + 16 * f);
                    const int64_t m = mw + r;
                    if (m < M) {
                        if constexpr (STREAM)   // an output too large to stay cached (see launch())
                            __builtin_nontemporal_store(__builtin_bit_cast(v4i, v), reinterpret_cast<v4i*>(o + m * N + wave_n0 + c * 8));
                        else
                            *reinterpret_cast<uint4*>(o + m * N + wave_n0 + c * 8) = v;
                    }
                }
            } else {
                constexpr int RB = WAVE_N * 4, CPR = RB / 16;          // 576 B, 36 chunks per row
                float* o = reinterpret_cast<float*>(p.out);
#pragma unroll
                for (int h = 0; h < 2; h++) {
#pragma unroll
                    for (int i = 0; i < 2; i++)
#pragma unroll
                        for (int j = 0; j < NSUB; j++)
                            *reinterpret_cast<v4f*>(reg + (i * 16 + lrow) * RB + (j * 16 + lcol4) * 4) = acc[2 * h + i][j];
#pragma unroll
                    for (int k = 0; k < 32 * CPR / 64; k++) {
                        const int f = 64 * k + lane;
                        const int r = f / CPR, c = f % CPR;
                        const v4f v = *reinterpret_cast<const v4f*>(reg + 16 * f);
                        const int64_t m = mw + 32 * h + r;
                        if (m < M) {
                            if constexpr (STREAM)
                                __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(o + m * N + wave_n0 + c * 4));
                            else
                                *reinterpret_cast<float4*>(o + m * N + wave_n0 + c * 4) = make_float4(v[0], v[1], v[2], v[3]);
                        }
                    }
                }
            }
            return;
        }
    }
    // Straight from the MFMA layout (a wave tile that runs past N, or unaligned output rows): lane l holds
    // row lrow and columns lcol4 .. lcol4 + 3 of every 16 x 16 tile.
    const bool vec_ok = (N & 3) == 0;
#pragma unroll
    for (int i = 0; i < MSUB; i++) {
        const int64_t m = m0 + wm * WAVE_M + i * 16 + lrow;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < NSUB; j++) {
            const int64_t n = wave_n0 + j * 16 + lcol4;
            if (bf16) {
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

template <class C, bool B_TRANS, int SBK, int GROUP, bool POW2, int EPI = EPI_STORE, bool STREAM = false>
hipError_t launch_one(const GemmParams& p, unsigned grid, hipStream_t stream) {
    auto kern = fg_gemm_kernel<C, B_TRANS, SBK, GROUP, POW2, EPI, STREAM>;
    static std::atomic<uint64_t> lds_limit_set{0};
    const hipError_t e = fg_set_lds_limit_once((const void*)kern, C::LDS_BYTES, lds_limit_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(C::NTHREADS), C::LDS_BYTES, stream, p);
    return hipGetLastError();
}

template <class C>
unsigned grid_for(const GemmParams& p, int group) {
    const int64_t n_tiles = (p.N + C::BN - 1) / C::BN;
    const int64_t m_tiles = (p.M + C::BM - 1) / C::BM;
    // worst case, a multiple of 8 rows of tiles (the host bounds it below 2^31 workgroups)
    if (group == GRP_ROWS) return (unsigned)(((m_tiles + p.G + 7) / 8) * 8 * n_tiles);
    if (group == GRP_K) return (unsigned)(m_tiles * n_tiles * p.G);
    return (unsigned)(m_tiles * n_tiles);
}

// Workgroup shape for one launch: the one with the smaller estimated time, counting full rounds of tiles
// over the compute units, a tile's work (BM * BN) and the measured per-tile rate of the 8-wave shape
// relative to the 12-wave one: 21% more MFMA throughput per CU (measured at the dense-MLP Fprop shape,
// where the two shapes need 4.5 and 6 rounds, inside the whole training step: 542 against 580 us with FP32
// scales, 488 against 553 us with power-of-2 scales). FG_GEMM_TILE=256x192 or 256x256 in the environment
// forces a shape (tuning and tests).
bool use_cfg8(const GemmParams& p, int grouped) {
    const char* force = getenv("FG_GEMM_TILE");
    if (force && strcmp(force, "256x256") == 0) return true;
    if (force && strcmp(force, "256x192") == 0) return false;
    const int64_t cus = fg_device_cus();
    const int64_t r12 = (grid_for<Cfg12>(p, grouped) + cus - 1) / cus;
    const int64_t r8 = (grid_for<Cfg8>(p, grouped) + cus - 1) / cus;
    return (double)r8 * Cfg8::BM * Cfg8::BN / 1.21 < (double)r12 * Cfg12::BM * Cfg12::BN;
}

// An output at least as large as the 256 MB Infinity Cache cannot stay there for the next kernel: its
// stores go past the caches instead of filling them with dirty lines that the next kernels would pay to
// write back, and that would evict the operands this kernel re-reads. Measured with back-to-back launches of
// the MoE share (same box, outputs bit-identical): grouped Dgrad (1.9 GB of FP32 dX) 1159 -> 1046 us,
// down-projection (940 MB of BF16) 1015 -> 973 us, up-projection (268 MB) 953 -> 945 us. The dense-MLP Fprop
// and Dgrad outputs (151 and 117 MB) keep ordinary stores: the next layer reads them, from the cache if
// still there.
constexpr int64_t kStreamOutBytes = 256ll << 20;

template <bool B_TRANS, int SBK, int GROUP>
hipError_t launch(const GemmParams& p, int pow2, hipStream_t stream) {
    if (use_cfg8(p, GROUP)) {
        if constexpr (SBK != SB_ROW) {   // weight gradients are always streamed
            const int64_t out_bytes = p.M * p.N * (p.out_bf16 ? 2 : 4);
            if (out_bytes >= kStreamOutBytes) {
                const unsigned grid = grid_for<Cfg8>(p, GROUP);
                return pow2 ? launch_one<Cfg8, B_TRANS, SBK, GROUP, true, EPI_STORE, true>(p, grid, stream)
                            : launch_one<Cfg8, B_TRANS, SBK, GROUP, false, EPI_STORE, true>(p, grid, stream);
            }
        }
        const unsigned grid = grid_for<Cfg8>(p, GROUP);
        return pow2 ? launch_one<Cfg8, B_TRANS, SBK, GROUP, true>(p, grid, stream)
                    : launch_one<Cfg8, B_TRANS, SBK, GROUP, false>(p, grid, stream);
    }
    const unsigned grid = grid_for<Cfg12>(p, GROUP);
    return pow2 ? launch_one<Cfg12, B_TRANS, SBK, GROUP, true>(p, grid, stream)
                : launch_one<Cfg12, B_TRANS, SBK, GROUP, false>(p, grid, stream);
}

// Fprop on 256 x 288 tiles (fg_gemm_wide_kernel) when they need fewer tile-work units than the 8-wave
// 256 x 256 shape: rounds of tiles over the CUs times the tile's area, as in use_cfg8. At the dense-MLP
// Fprop (M = 4096, N = 18432) that is 4 rounds of 256 x 288 against 4.5 (counted as 5) of 256 x 256.
// FG_GEMM_TILE=256x288 forces it; FG_GEMM_TILE=256x192 or 256x256 rules it out. Its B operand offsets
// reach 287 K, so contractions with 288 K >= 2^32 keep the other shapes.
bool use_wide(const GemmParams& p) {
    if ((int64_t)WideCfg::BN * p.K >= (1ll << 32)) return false;
    const char* force = getenv("FG_GEMM_TILE");
    if (force && strcmp(force, "256x288") == 0) return true;
    if (force && (strcmp(force, "256x256") == 0 || strcmp(force, "256x192") == 0)) return false;
    if (!use_cfg8(p, GRP_NONE)) return false;
    const int64_t cus = fg_device_cus();
    const int64_t m_tiles = (p.M + 255) / 256;
    const int64_t rw = (m_tiles * ((p.N + WideCfg::BN - 1) / WideCfg::BN) + cus - 1) / cus;
    const int64_t r8 = (m_tiles * ((p.N + Cfg8::BN - 1) / Cfg8::BN) + cus - 1) / cus;
    return rw * WideCfg::BN < r8 * Cfg8::BN;
}

template <bool POW2, bool STREAM>
hipError_t launch_wide(const GemmParams& p, unsigned grid, hipStream_t stream) {
    auto kern = fg_gemm_wide_kernel<POW2, STREAM>;
    static std::atomic<uint64_t> lds_limit_set{0};
    const hipError_t e = fg_set_lds_limit_once((const void*)kern, WideCfg::LDS_BYTES, lds_limit_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(WideCfg::NTHREADS), WideCfg::LDS_BYTES, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t fg_launch_gemm_fprop(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw, int64_t M,
                                int64_t N, int64_t K, void* y, int out_bf16, int pow2, hipStream_t stream) {
    GemmParams p{};
    p.a = xq; p.sa = sx; p.sa_ld = M; p.b = wq; p.sb = sw;
    p.M = M; p.N = N; p.K = K; p.out = y; p.out_bf16 = out_bf16;
    if (use_wide(p)) {
        const unsigned grid = (unsigned)(((M + WideCfg::BM - 1) / WideCfg::BM) * ((N + WideCfg::BN - 1) / WideCfg::BN));
        const bool stream_out = M * N * (out_bf16 ? 2 : 4) >= kStreamOutBytes;
        if (stream_out)
            return pow2 ? launch_wide<true, true>(p, grid, stream) : launch_wide<false, true>(p, grid, stream);
        return pow2 ? launch_wide<true, false>(p, grid, stream) : launch_wide<false, false>(p, grid, stream);
    }
    return launch<false, SB_BLOCK, GRP_NONE>(p, pow2, stream);
}

hipError_t fg_launch_gemm_dgrad(const uint8_t* dyq, const float* sdy, const uint8_t* wq, const float* sw, int64_t M,
                                int64_t N, int64_t K, void* dx, int out_bf16, int pow2, hipStream_t stream) {
    // dX[M][K] = dY[M][N] . W[N][K]: A-role = dY (contraction N), B-role = W read transposed.
    GemmParams p{};
    p.a = dyq; p.sa = sdy; p.sa_ld = M; p.b = wq; p.sb = sw;
    p.M = M; p.N = K; p.K = N; p.out = dx; p.out_bf16 = out_bf16;
    return launch<true, SB_BLOCK_T, GRP_NONE>(p, pow2, stream);
}

hipError_t fg_launch_gemm_wgrad(const uint8_t* dytq, const float* sdyt, const uint8_t* xtq, const float* sxt,
                                int64_t M, int64_t N, int64_t K, float* dw, int accumulate, int pow2, hipStream_t stream) {
    // dW[N][K] = dYt[N][M] . Xt[K][M]^T: A-role = dYt (rows N), B-role = Xt (rows K), contraction M.
    GemmParams p{};
    p.a = dytq; p.sa = sdyt; p.sa_ld = N; p.b = xtq; p.sb = sxt;
    p.M = N; p.N = K; p.K = M; p.out = dw; p.out_bf16 = 0; p.accumulate = accumulate;
    return launch<false, SB_ROW, GRP_NONE>(p, pow2, stream);
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
    return launch<false, SB_BLOCK, GRP_ROWS>(p, pow2, stream);
}

hipError_t fg_launch_gemm_grouped_dgrad(const uint8_t* dyq, const float* sdy, const uint8_t* wq, const float* sw,
                                        const int32_t* offsets, int32_t G, int64_t T, int64_t N, int64_t K, void* dx,
                                        int out_bf16, int pow2, hipStream_t stream) {
    // per group g: dX[rows of g][K] = dY[rows of g][N] . W[g][N][K] (A-role dY, B-role W[g] read transposed)
    GemmParams p{};
    p.a = dyq; p.sa = sdy; p.sa_ld = T; p.b = wq; p.sb = sw;
    p.M = T; p.N = K; p.K = N; p.out = dx; p.out_bf16 = out_bf16;
    p.offsets = offsets; p.G = G;
    p.b_group_stride = N * K;
    p.sb_group_stride = (N / 128) * ((K + 127) / 128);
    return launch<true, SB_BLOCK_T, GRP_ROWS>(p, pow2, stream);
}

hipError_t fg_launch_gemm_grouped_wgrad(const uint8_t* dytq, const float* sdyt, const uint8_t* xtq, const float* sxt,
                                        const int32_t* offsets, int32_t G, int64_t T, int64_t N, int64_t K, float* dw,
                                        int accumulate, int pow2, hipStream_t stream) {
    // per group g: dW[g][N][K] (+)= dYt[N][tokens of g] . Xt[K][tokens of g]^T
    GemmParams p{};
    p.a = dytq; p.sa = sdyt; p.sa_ld = N; p.b = xtq; p.sb = sxt;
    p.M = N; p.N = K; p.K = T; p.out = dw; p.out_bf16 = 0; p.accumulate = accumulate;
    p.offsets = offsets; p.G = G;
    p.out_group_stride = N * K;
    return launch<false, SB_ROW, GRP_K>(p, pow2, stream);
}

hipError_t fg_launch_gemm_fprop_quant(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw, int64_t M,
                                      int64_t N, int64_t K, uint8_t* yq, float* sy, int pow2, int out_pow2,
                                      hipStream_t stream) {
    GemmParams p{};
    p.a = xq; p.sa = sx; p.sa_ld = M; p.b = wq; p.sb = sw;
    p.M = M; p.N = N; p.K = K; p.out = nullptr; p.out_bf16 = 1;
    p.q_out = yq; p.s_out = sy; p.q_pow2 = out_pow2;
    const unsigned grid = grid_for<Cfg8>(p, GRP_NONE);
    return pow2 ? launch_one<Cfg8, false, SB_BLOCK, GRP_NONE, true, EPI_QUANT>(p, grid, stream)
                : launch_one<Cfg8, false, SB_BLOCK, GRP_NONE, false, EPI_QUANT>(p, grid, stream);
}
