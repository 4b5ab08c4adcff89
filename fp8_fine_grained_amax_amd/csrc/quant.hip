// Online E4M3 quantization kernels for gfx950: 1x128 activation tiles (along columns, or along the token
// dimension with a transposed write) and 128x128 weight blocks.
//
// Each kernel reads the bf16 input from HBM exactly once, finds the group's max-abs on chip, derives the
// fp32 scale and writes E4M3 codes plus the scale. The operation is HBM-bound (2 B read + 1 B written
// per element, + 4 B per group), so the kernels are built around wide coalesced accesses, several
// 16-byte loads in flight per lane, and reductions that stay in registers (DPP) or a tiny LDS array.
//
// Sources: the fine-grained scaling (1x128 tiles for activations, 128x128 blocks for weights) is Figure 7
// (a) as quoted on the pages "Three Fast Methods To Study Deepseek" and the untitled cameseeing.com and
// why-be.why-be.co.kr pages; the online max-abs per tile/block and the online quantization are from the
// cameseeing.com page's passage next to that figure; the alignment of the max-abs to the largest FP8
// value from "5 Ways You can get More Deepseek While Spending Less" (paragraph on per-group scaling);
// power-of-2 scales from the opening paragraph of that page.
#include "common.h"

// ------------------------------------------------------------------------------------------------
// 1x128 tiles along columns.
// One 1x128 bf16 tile is 256 B = 16 lanes x 16 B, i.e. exactly one DPP row, so the tile max-abs is four
// DPP steps with no LDS. A 256-thread workgroup covers 16 rows of one 128-column group per unrolled
// slot, and the 16 scales of a slot are one contiguous 64 B write in the MN-major scale layout
// [cols/128][rows]. Workgroups are numbered column group first: the ones in flight together read whole
// row segments of the same rows, which streams from HBM at the rate of a plain copy.
// ------------------------------------------------------------------------------------------------
template <int UNROLL>
__global__ __launch_bounds__(256) void fg_quant_act_cols_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                                int64_t ld, int64_t groups, int pow2,
                                                                uint8_t* __restrict__ q, int64_t ldq,
                                                                float* __restrict__ scales) {
    const int lane16 = threadIdx.x & 15;
    const int slot = threadIdx.x >> 4;
    const uint32_t bid = blockIdx.x, ng = (uint32_t)groups;
    const int64_t g = bid % ng;
    const int64_t r_base = (int64_t)(bid / ng) * (16 * UNROLL) + slot;

    uint4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; u++) {
        int64_t r = r_base + 16 * u;
        if (r < rows)
            v[u] = *reinterpret_cast<const uint4*>(x + r * ld + g * FG_GROUP + lane16 * 8);
        else
            v[u] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; u++) {
        int64_t r = r_base + 16 * u;
        uint32_t m = fg_pk_max_u16(fg_pk_max_u16(v[u].x & 0x7FFF7FFFu, v[u].y & 0x7FFF7FFFu),
                                   fg_pk_max_u16(v[u].z & 0x7FFF7FFFu, v[u].w & 0x7FFF7FFFu));
        m = fg_max_halves(fg_row16_max_pk(m));
        const float s = fg_scale_from_amax_bits(m, pow2);
        const uint2 codes = fg_quant8_any(v[u], fg_make_divisor(s, pow2), pow2);
        if (r < rows) {
            *reinterpret_cast<uint2*>(q + r * ldq + g * FG_GROUP + lane16 * 8) = codes;
            if (lane16 == 0) scales[g * rows + r] = s;
        }
    }
}

// ------------------------------------------------------------------------------------------------
// 1x128 tiles along rows (token dimension), codes written transposed.
// A 256-thread workgroup owns 128 rows x 64 columns. Thread t reads rows 4*(t/8)+i (i = 0..3) of the
// 8-column chunk t%8 (16 B per row, coalesced 128 B per row across 8 lanes). Column max-abs: 4 rows in
// registers, then across the 8 lanes sharing a chunk with lane shuffles, then across the 4 waves in LDS.
// Codes of one column and 4 consecutive rows pack into one dword (two cvt_pk per dword), go to an LDS
// transpose buffer [64 cols][128 rows], and leave as 16 B stores: 128 contiguous bytes per column.
// Workgroups are numbered row block first, so the ones in flight together extend the same output
// columns: their 128 B pieces form contiguous runs of the transposed codes.
//
// FROM_CODES: the input is not bf16 but FP8 codes cached in 1x128 tiles along the columns (codes
// [rows][cols], row scales [cols/128][rows]). Each element is dequantized to the bf16 activation it
// stands for, bf16(RN_f32(code * row scale)), and that tensor is quantized along the tokens exactly as a
// bf16 input would be: the read, dequantize, transpose and re-quantize step of the backward pass.
// ------------------------------------------------------------------------------------------------
// Eight E4M3 codes (8 B) times their row's scale, rounded to fp32 and then to bf16: eight bf16 values.
__device__ __forceinline__ uint32_t fg_dequant2_bf16(float lo, float hi, float s) {
    return (uint32_t)__builtin_bit_cast(unsigned short, (__bf16)(lo * s)) |
           ((uint32_t)__builtin_bit_cast(unsigned short, (__bf16)(hi * s)) << 16);
}
__device__ __forceinline__ uint4 fg_dequant8_bf16(uint2 c, float s) {
    // exact E4M3 -> fp32 decode of bytes 0-1 (false) or 2-3 (true) of a dword
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.x, false), b = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.x, true);
    const auto e = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.y, false), f = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.y, true);
    return make_uint4(fg_dequant2_bf16(a[0], a[1], s), fg_dequant2_bf16(b[0], b[1], s),
                      fg_dequant2_bf16(e[0], e[1], s), fg_dequant2_bf16(f[0], f[1], s));
}

template <bool FROM_CODES>
__global__ __launch_bounds__(256) void fg_quant_act_rows_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                                int64_t cols, int64_t ld, int pow2,
                                                                uint8_t* __restrict__ q, float* __restrict__ scales,
                                                                const uint8_t* __restrict__ q_in,
                                                                const float* __restrict__ s_in) {
    __shared__ uint32_t colmax[4][32];          // [wave][column pair], packed u16 max-abs
    __shared__ float col_s[64], col_r[64];      // per-column scale and reciprocal
    __shared__ int any_tiny;
    __shared__ uint4 codes_t[64 * 8];           // [column][16 B piece], pieces swizzled per column

    const int t = threadIdx.x;
    const int chunk = t & 7;                    // 8-column chunk within the 64-column tile
    const int rgrp = t >> 3;                    // rows 4*rgrp .. 4*rgrp+3 within the 128-row tile
    const int64_t r0 = (int64_t)blockIdx.x * FG_GROUP;
    const int64_t c0 = (int64_t)blockIdx.y * 64;
    const int64_t col = c0 + chunk * 8;
    const bool col_ok = col < cols;

    uint4 v[4];
    if constexpr (FROM_CODES) {
        // the 64-column tile lies inside one 128-column group: one row scale per row
        const float4 sr = col_ok ? *reinterpret_cast<const float4*>(s_in + (col / FG_GROUP) * rows + r0 + 4 * rgrp)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint2 c = col_ok ? *reinterpret_cast<const uint2*>(q_in + (r0 + 4 * rgrp + i) * cols + col)
                                   : make_uint2(0, 0);
            v[i] = fg_dequant8_bf16(c, (&sr.x)[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            if (col_ok)
                v[i] = *reinterpret_cast<const uint4*>(x + (r0 + 4 * rgrp + i) * ld + col);
            else
                v[i] = make_uint4(0, 0, 0, 0);
        }
    }
    // packed max-abs per column pair over this thread's 4 rows
    uint32_t m[4];
#pragma unroll
    for (int p = 0; p < 4; p++) {
        uint32_t a = (&v[0].x)[p] & 0x7FFF7FFFu, b = (&v[1].x)[p] & 0x7FFF7FFFu;
        uint32_t c = (&v[2].x)[p] & 0x7FFF7FFFu, d = (&v[3].x)[p] & 0x7FFF7FFFu;
        m[p] = fg_pk_max_u16(fg_pk_max_u16(a, b), fg_pk_max_u16(c, d));
    }
    // across the 8 lanes of a wave that share this chunk (lane bits 3..5)
#pragma unroll
    for (int p = 0; p < 4; p++) {
        m[p] = fg_pk_max_u16(m[p], (uint32_t)__shfl_xor((int)m[p], 8));
        m[p] = fg_pk_max_u16(m[p], (uint32_t)__shfl_xor((int)m[p], 16));
        m[p] = fg_pk_max_u16(m[p], (uint32_t)__shfl_xor((int)m[p], 32));
    }
    const int wave = t >> 6;
    if ((t & 63) < 8) {
#pragma unroll
        for (int p = 0; p < 4; p++) colmax[wave][chunk * 4 + p] = m[p];
    }
    __syncthreads();
    // One scale and reciprocal per column, computed once (wave 0, lane = column) and shared through LDS;
    // the tile's 64 scales leave as one contiguous 256 B write.
    if (wave == 0) {
        const int c = t, pair = c >> 1;
        const uint32_t mp = fg_pk_max_u16(fg_pk_max_u16(colmax[0][pair], colmax[1][pair]),
                                          fg_pk_max_u16(colmax[2][pair], colmax[3][pair]));
        const float s = fg_scale_from_amax_bits((c & 1) ? mp >> 16 : mp & 0xFFFFu, pow2);
        const fg_divisor d = fg_make_divisor(s, pow2);
        col_s[c] = d.s;
        col_r[c] = d.r;
        const uint64_t tiny = __builtin_amdgcn_ballot_w64(fg_divisor_tiny(d));
        if (c == 0) any_tiny = tiny != 0;
        if (c0 + c < cols) scales[(int64_t)blockIdx.x * cols + c0 + c] = s;
    }
    __syncthreads();
    // codes: dword j holds column chunk*8+j, rows 4*rgrp .. 4*rgrp+3 (byte i = row i)
    uint32_t* ct = reinterpret_cast<uint32_t*>(codes_t);
    const int mode = pow2 ? FG_Q_POW2 : (any_tiny ? FG_Q_TINY : FG_Q_FAST);
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const int c = chunk * 8 + j;
        fg_divisor d{col_s[c], col_r[c]};
        float f[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            uint32_t w = (&v[i].x)[j >> 1];
            f[i] = (j & 1) ? fg_bf16_hi(w) : fg_bf16_lo(w);
        }
        uint32_t dw;
        if (mode == FG_Q_POW2) {
            dw = fg_cvt2q<FG_Q_POW2, true>(f[2], f[3], d, fg_cvt2q<FG_Q_POW2, false>(f[0], f[1], d, 0));
        } else if (mode == FG_Q_FAST || !fg_divisor_tiny(d)) {
            dw = fg_cvt2q<FG_Q_FAST, true>(f[2], f[3], d, fg_cvt2q<FG_Q_FAST, false>(f[0], f[1], d, 0));
        } else {
            d = fg_divisor_shifted(d);
            dw = fg_cvt2q<FG_Q_TINY, true>(f[2], f[3], d, fg_cvt2q<FG_Q_TINY, false>(f[0], f[1], d, 0));
        }
        // dword rgrp of column c; the 16 B piece index (rgrp >> 2) is XOR-swizzled by (c >> 3) & 3
        const int piece = (rgrp >> 2) ^ ((c >> 3) & 3) * 2;
        ct[c * 32 + piece * 4 + (rgrp & 3)] = dw;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const int id = t + 256 * h;             // 512 pieces: column id/8, logical piece id%8
        const int c = id >> 3, p = id & 7;
        const int64_t gc = c0 + c;
        if (gc < cols) {
            uint4 val = codes_t[c * 8 + (p ^ (((c >> 3) & 3) * 2))];
            *reinterpret_cast<uint4*>(q + gc * rows + r0 + 16 * p) = val;
        }
    }
}

// ------------------------------------------------------------------------------------------------
// 128x128 weight blocks. One 256-thread workgroup per block: thread t holds rows t/16 + 16 i (i = 0..7)
// of the 16 B chunk t%16, so each 16-lane group reads one full 256 B block row. The block max-abs is a
// register max, a DPP row max, two lane shuffles and a 4-entry LDS exchange; the block is read once.
// ------------------------------------------------------------------------------------------------
// Block (bk, bn): input columns 128 bk.., rows 128 bn...
__device__ __forceinline__ void fg_quant_w_block(const uint16_t* __restrict__ w, int64_t n, int64_t ld, int64_t kblocks,
                                                 int pow2, uint8_t* __restrict__ q, int64_t ldq,
                                                 float* __restrict__ scales, int64_t bk, int64_t bn) {
    __shared__ uint32_t wmax[4];
    const int t = threadIdx.x;
    const int chunk = t & 15;
    const int rsub = t >> 4;
    const int64_t r0 = bn * FG_GROUP;
    const int64_t c0 = bk * FG_GROUP + chunk * 8;

    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        int64_t r = r0 + rsub + 16 * i;
        if (r < n)
            v[i] = *reinterpret_cast<const uint4*>(w + r * ld + c0);
        else
            v[i] = make_uint4(0, 0, 0, 0);
    }
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; i++)
        m = fg_pk_max_u16(m, fg_pk_max_u16(fg_pk_max_u16(v[i].x & 0x7FFF7FFFu, v[i].y & 0x7FFF7FFFu),
                                           fg_pk_max_u16(v[i].z & 0x7FFF7FFFu, v[i].w & 0x7FFF7FFFu)));
    m = fg_row16_max_pk(m);
    m = fg_pk_max_u16(m, (uint32_t)__shfl_xor((int)m, 16));
    m = fg_pk_max_u16(m, (uint32_t)__shfl_xor((int)m, 32));
    if ((t & 63) == 0) wmax[t >> 6] = fg_max_halves(m);
    __syncthreads();
    uint32_t a = wmax[0] > wmax[1] ? wmax[0] : wmax[1];
    uint32_t b = wmax[2] > wmax[3] ? wmax[2] : wmax[3];
    const float s = fg_scale_from_amax_bits(a > b ? a : b, pow2);
    if (t == 0) scales[bn * kblocks + bk] = s;
    const fg_divisor d = fg_make_divisor(s, pow2);
#pragma unroll
    for (int i = 0; i < 8; i++) {
        int64_t r = r0 + rsub + 16 * i;
        const uint2 codes = fg_quant8_any(v[i], d, pow2);
        if (r < n) *reinterpret_cast<uint2*>(q + r * ldq + c0) = codes;
    }
}

__global__ __launch_bounds__(256) void fg_quant_w_kernel(const uint16_t* __restrict__ w, int64_t n, int64_t ld,
                                                         int64_t kblocks, int pow2, uint8_t* __restrict__ q,
                                                         int64_t ldq, float* __restrict__ scales) {
    fg_quant_w_block(w, n, ld, kblocks, pow2, q, ldq, scales, blockIdx.x, blockIdx.y);
}

// ------------------------------------------------------------------------------------------------
// Both 1x128 tilings from one read: the codes and scales of FG_ALONG_COLS (tiles along the channels, as
// the Fprop/Dgrad operand) and of FG_ALONG_ROWS (tiles along the tokens, transposed, as the Wgrad
// operand). A 256-thread workgroup owns a 128 x 128 block: thread t holds rows 8*(t/16)+i (i = 0..7) of
// the 8-column chunk t%16, so the 16 lanes of a DPP row hold one full 128-column row (row max-abs by DPP)
// and the lanes sharing a chunk hold one column (column max-abs by lane shuffles and a 4-wave LDS
// exchange). Row-tile codes leave directly (128 contiguous bytes per row); column-tile codes go through
// an LDS transpose buffer [128 columns][128 rows] whose 16 B pieces are XOR-swizzled by column.
// The bf16 block is read once instead of twice.
// ------------------------------------------------------------------------------------------------
// Block (br, bc): rows 128 br.., columns 128 bc...
__device__ __forceinline__ void fg_quant_act_both_block(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                        int64_t ld, int pow2, uint8_t* __restrict__ qc,
                                                        float* __restrict__ sc, uint8_t* __restrict__ qr,
                                                        float* __restrict__ sr, int64_t br, int64_t bc) {
    __shared__ uint32_t colmax[4][64];          // [wave][column pair], packed u16 max-abs
    __shared__ float col_s[128], col_r[128];    // per-column scale and reciprocal
    __shared__ int tiny_w[2];                   // per wave of the column-scale step: a scale below 2^-100
    __shared__ uint4 codes_t[128 * 8];          // [column][16 B piece], pieces swizzled per column

    const int t = threadIdx.x;
    const int chunk = t & 15;                   // 8-column chunk within the 128-column block
    const int rgrp = t >> 4;                    // rows 8*rgrp .. 8*rgrp+7 within the 128-row block
    const int wave = t >> 6;
    const int64_t r0 = br * FG_GROUP;
    const int64_t c0 = bc * FG_GROUP;
    const int64_t g = bc;                       // column group of the row tiles

    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = *reinterpret_cast<const uint4*>(x + (r0 + 8 * rgrp + i) * ld + c0 + chunk * 8);

    // column max-abs (packed pairs): 8 rows in registers, the 4 lanes of a wave sharing the chunk, 4 waves
    uint32_t m[4];
#pragma unroll
    for (int p = 0; p < 4; p++) {
        m[p] = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) m[p] = fg_pk_max_u16(m[p], (&v[i].x)[p] & 0x7FFF7FFFu);
        m[p] = fg_pk_max_u16(m[p], (uint32_t)__shfl_xor((int)m[p], 16));
        m[p] = fg_pk_max_u16(m[p], (uint32_t)__shfl_xor((int)m[p], 32));
    }
    if ((t & 63) < 16) {
#pragma unroll
        for (int p = 0; p < 4; p++) colmax[wave][chunk * 4 + p] = m[p];
    }

    // row tiles: max-abs over the 16 lanes of the DPP row, codes straight out
    float s_row[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        uint32_t mr = fg_pk_max_u16(fg_pk_max_u16(v[i].x & 0x7FFF7FFFu, v[i].y & 0x7FFF7FFFu),
                                    fg_pk_max_u16(v[i].z & 0x7FFF7FFFu, v[i].w & 0x7FFF7FFFu));
        mr = fg_max_halves(fg_row16_max_pk(mr));
        s_row[i] = fg_scale_from_amax_bits(mr, pow2);
        const uint2 codes = fg_quant8_any(v[i], fg_make_divisor(s_row[i], pow2), pow2);
        *reinterpret_cast<uint2*>(qc + (r0 + 8 * rgrp + i) * cols + c0 + chunk * 8) = codes;
    }
    // lane `chunk` < 8 of each DPP row writes the scale of row 8*rgrp + chunk: 32 contiguous bytes
#pragma unroll
    for (int i = 0; i < 8; i++)
        if (chunk == i) sc[g * rows + r0 + 8 * rgrp + i] = s_row[i];

    __syncthreads();
    // column tiles: one scale and reciprocal per column, shared through LDS
    if (t < 128) {
        const int c = t, pair = c >> 1;
        const uint32_t mp = fg_pk_max_u16(fg_pk_max_u16(colmax[0][pair], colmax[1][pair]),
                                          fg_pk_max_u16(colmax[2][pair], colmax[3][pair]));
        const float s = fg_scale_from_amax_bits((c & 1) ? mp >> 16 : mp & 0xFFFFu, pow2);
        const fg_divisor d = fg_make_divisor(s, pow2);
        col_s[c] = d.s;
        col_r[c] = d.r;
        const uint64_t tiny = __builtin_amdgcn_ballot_w64(fg_divisor_tiny(d));
        if ((c & 63) == 0) tiny_w[c >> 6] = tiny != 0;
        sr[br * cols + c0 + c] = s;
    }
    __syncthreads();
    const int mode = pow2 ? FG_Q_POW2 : ((tiny_w[0] | tiny_w[1]) ? FG_Q_TINY : FG_Q_FAST);
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const int c = chunk * 8 + j;
        fg_divisor d{col_s[c], col_r[c]};
        float f[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t w = (&v[i].x)[j >> 1];
            f[i] = (j & 1) ? fg_bf16_hi(w) : fg_bf16_lo(w);
        }
        uint32_t d0, d1;
        if (mode == FG_Q_POW2) {
            d0 = fg_cvt2q<FG_Q_POW2, true>(f[2], f[3], d, fg_cvt2q<FG_Q_POW2, false>(f[0], f[1], d, 0));
            d1 = fg_cvt2q<FG_Q_POW2, true>(f[6], f[7], d, fg_cvt2q<FG_Q_POW2, false>(f[4], f[5], d, 0));
        } else if (mode == FG_Q_FAST || !fg_divisor_tiny(d)) {
            d0 = fg_cvt2q<FG_Q_FAST, true>(f[2], f[3], d, fg_cvt2q<FG_Q_FAST, false>(f[0], f[1], d, 0));
            d1 = fg_cvt2q<FG_Q_FAST, true>(f[6], f[7], d, fg_cvt2q<FG_Q_FAST, false>(f[4], f[5], d, 0));
        } else {
            d = fg_divisor_shifted(d);
            d0 = fg_cvt2q<FG_Q_TINY, true>(f[2], f[3], d, fg_cvt2q<FG_Q_TINY, false>(f[0], f[1], d, 0));
            d1 = fg_cvt2q<FG_Q_TINY, true>(f[6], f[7], d, fg_cvt2q<FG_Q_TINY, false>(f[4], f[5], d, 0));
        }
        // rows 8*rgrp .. +7 of column c: the 8 B half (rgrp & 1) of 16 B piece rgrp >> 1, swizzled
        const int piece = (rgrp >> 1) ^ (chunk & 7);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(codes_t) + c * 128 + piece * 16 + (rgrp & 1) * 8) =
            make_uint2(d0, d1);
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 4; h++) {
        const int id = t + 256 * h;             // 1024 pieces: column id/8, logical piece id%8
        const int c = id >> 3, p = id & 7;
        const uint4 val = codes_t[c * 8 + (p ^ ((c >> 3) & 7))];
        *reinterpret_cast<uint4*>(qr + (c0 + c) * rows + r0 + 16 * p) = val;
    }
}

__global__ __launch_bounds__(256) void fg_quant_act_both_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                                int64_t cols, int64_t ld, int pow2,
                                                                uint8_t* __restrict__ qc, float* __restrict__ sc,
                                                                uint8_t* __restrict__ qr, float* __restrict__ sr) {
    fg_quant_act_both_block(x, rows, cols, ld, pow2, qc, sc, qr, sr, blockIdx.x, blockIdx.y);
}

// ------------------------------------------------------------------------------------------------
// The Linear operator's two forward operands in one launch: X in both 1x128 tilings and W in 128x128
// blocks. Workgroups [0, xb) are X blocks (row block fastest, as in fg_quant_act_both_kernel), the rest W
// blocks (column block fastest, as in fg_quant_w_kernel). One launch streams X and W back to back, so the
// ramp-up and drain of a launch are paid once for both tensors instead of once each, and the X part no
// longer runs as a launch too short to reach full HBM bandwidth on its own.
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fg_quant_x_both_w_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                                int64_t cols, int64_t ldx, uint8_t* __restrict__ qc,
                                                                float* __restrict__ sc, uint8_t* __restrict__ qr,
                                                                float* __restrict__ sr, const uint16_t* __restrict__ w,
                                                                int64_t n, int64_t ldw, uint8_t* __restrict__ qw,
                                                                float* __restrict__ sw, int pow2) {
    const int64_t id = blockIdx.x;
    const int64_t xrb = rows / FG_GROUP, xb = xrb * (cols / FG_GROUP);
    if (id < xb) {
        fg_quant_act_both_block(x, rows, cols, ldx, pow2, qc, sc, qr, sr, id % xrb, id / xrb);
    } else {
        const int64_t kb = cols / FG_GROUP, wid = id - xb;
        fg_quant_w_block(w, n, ldw, kb, pow2, qw, cols, sw, wid % kb, wid / kb);
    }
}

// ------------------------------------------------------------------------------------------------
// Host launchers (arguments already validated by the C-ABI layer).
// ------------------------------------------------------------------------------------------------
constexpr int kActColsUnroll = 2;

hipError_t fg_launch_quant_act_cols(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int pow2,
                                    uint8_t* q, float* scales, hipStream_t stream) {
    const int64_t groups = cols / FG_GROUP;
    const int64_t row_blocks = (rows + 16 * kActColsUnroll - 1) / (16 * kActColsUnroll);
    hipLaunchKernelGGL(fg_quant_act_cols_kernel<kActColsUnroll>, dim3((unsigned)(groups * row_blocks)), dim3(256), 0,
                       stream, x, rows, ld, groups, pow2, q, cols, scales);
    return hipGetLastError();
}

hipError_t fg_launch_quant_act_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int pow2,
                                    uint8_t* q, float* scales, hipStream_t stream) {
    dim3 grid((unsigned)(rows / FG_GROUP), (unsigned)((cols + 63) / 64));
    hipLaunchKernelGGL(fg_quant_act_rows_kernel<false>, grid, dim3(256), 0, stream, x, rows, cols, ld, pow2, q, scales,
                       nullptr, nullptr);
    return hipGetLastError();
}

hipError_t fg_launch_requant_rows(const uint8_t* q_in, const float* s_in, int64_t rows, int64_t cols, int pow2,
                                  uint8_t* q, float* scales, hipStream_t stream) {
    dim3 grid((unsigned)(rows / FG_GROUP), (unsigned)(cols / 64));
    hipLaunchKernelGGL(fg_quant_act_rows_kernel<true>, grid, dim3(256), 0, stream, nullptr, rows, cols, cols, pow2, q,
                       scales, q_in, s_in);
    return hipGetLastError();
}

hipError_t fg_launch_quant_w(const uint16_t* w, int64_t n, int64_t k, int64_t ld, int pow2, uint8_t* q,
                             float* scales, hipStream_t stream) {
    dim3 grid((unsigned)(k / FG_GROUP), (unsigned)((n + FG_GROUP - 1) / FG_GROUP));
    hipLaunchKernelGGL(fg_quant_w_kernel, grid, dim3(256), 0, stream, w, n, ld, k / FG_GROUP, pow2, q, k, scales);
    return hipGetLastError();
}

hipError_t fg_launch_quant_act_both(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int pow2,
                                    uint8_t* qc, float* sc, uint8_t* qr, float* sr, hipStream_t stream) {
    dim3 grid((unsigned)(rows / FG_GROUP), (unsigned)(cols / FG_GROUP));
    hipLaunchKernelGGL(fg_quant_act_both_kernel, grid, dim3(256), 0, stream, x, rows, cols, ld, pow2, qc, sc, qr, sr);
    return hipGetLastError();
}

hipError_t fg_launch_quant_x_both_w(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* qc, float* sc,
                                    uint8_t* qr, float* sr, const uint16_t* w, int64_t n, int64_t ldw, uint8_t* qw,
                                    float* sw, int pow2, hipStream_t stream) {
    const int64_t blocks = (rows / FG_GROUP) * (cols / FG_GROUP) + ((n + FG_GROUP - 1) / FG_GROUP) * (cols / FG_GROUP);
    hipLaunchKernelGGL(fg_quant_x_both_w_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, rows, cols, ldx, qc, sc,
                       qr, sr, w, n, ldw, qw, sw, pow2);
    return hipGetLastError();
}
