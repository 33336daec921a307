// tile_math.h -- wave-level helpers shared by the bf16 / head_dim 128 decode
// kernels (attn_fast.hip, attn_prefix.hip): MFMA operand types, 16-lane row
// reductions, wave scans and the tile constants.
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTok = 16;              // tokens per tile
constexpr int kHd = 128;              // head_dim of this path
constexpr float kLazyRescale = 8.0f;  // log2 units the running max may trail the tile max

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// All-reduce within each 16-lane row (row_ror 8, 4, 2, 1).
__device__ __forceinline__ float row_max16(float v) {
    v = fmaxf(v, dpp_f<0x128>(v));
    v = fmaxf(v, dpp_f<0x124>(v));
    v = fmaxf(v, dpp_f<0x122>(v));
    v = fmaxf(v, dpp_f<0x121>(v));
    return v;
}
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp_f<0x128>(v);
    v += dpp_f<0x124>(v);
    v += dpp_f<0x122>(v);
    v += dpp_f<0x121>(v);
    return v;
}

// Pairwise combines across 16-lane rows without LDS, by the gfx950 lane-swap
// moves.  v_permlane16_swap given two copies of v returns (rows 0,0,2,2 of v;
// rows 1,1,3,3 of v), so combining the two gives every lane l the pair
// {v[l], v[l ^ 16]}; v_permlane32_swap does the same for the two halves,
// {v[l], v[l ^ 32]}.  Both lanes of a pair combine the same two values in
// the same order, so they agree bit for bit.
__device__ __forceinline__ float sum_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// DPP move of an int where lanes without a source, and lanes of rows outside
// ROW_MASK, read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i0(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, true);
}

// Inclusive prefix sum over the 64 lanes, all in DPP moves (no LDS permutes):
// a Hillis-Steele scan inside every 16-lane row (shifts by 1, 2, 4, 8), then
// the running totals carried across rows -- lane 15 of rows 0 and 2 into rows
// 1 and 3, then lane 31 into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan_int(int v) {
    v += dpp_i0<0x111, 0xF>(v);  // row_shr:1
    v += dpp_i0<0x112, 0xF>(v);  // row_shr:2
    v += dpp_i0<0x114, 0xF>(v);  // row_shr:4
    v += dpp_i0<0x118, 0xF>(v);  // row_shr:8
    v += dpp_i0<0x142, 0xA>(v);  // row_bcast:15
    v += dpp_i0<0x143, 0xC>(v);  // row_bcast:31
    return v;
}

// Sum over the 64 lanes (wave-uniform result).
__device__ __forceinline__ int wave_sum_int(int v) { return __builtin_amdgcn_readlane(wave_incl_scan_int(v), 63); }

// floor(num / den) for 0 <= num < 2^53 and 0 < den < 2^53: the correctly
// rounded double quotient is within one of it, and one step corrects it.
__device__ __forceinline__ int64_t div_floor(int64_t num, int64_t den) {
    int64_t q = (int64_t)((double)num / (double)den);
    if (q * den > num) {
        --q;
    } else if ((q + 1) * den <= num) {
        ++q;
    }
    return q;
}

// The fast kernel's split of Nt tiles over W waves.  Waves w = x * W8 + j
// (j < W8) run on XCD x (workgroups are dealt to the eight XCDs in turn), and
// a wave's share is wt(x) * wh(j) in 4096ths of an equal share: wt(x) = b on
// odd x, 128 - b on even x, and wh(j) = 64 + d for the first half of the
// XCD's waves in dispatch order (j < W8 / 2: with two waves per SIMD, the
// first wave of every SIMD), 64 - d for the second half.  S(w), the shares of
// the waves before w, is 64 W8 base(x) + wt(x) * (the wh of the XCD's waves
// before w), with base(x) the wt of one wave of each XCD before x; S(W) =
// 4096 W, and wave w takes tiles [floor(Nt S(w) / 4096 W), floor(Nt S(w + 1)
// / 4096 W)).  W8 = 0 is the equal split floor(Nt w / W).
constexpr int kFirstHalfShare = 20;  // d above, in 64ths
struct Split {
    int64_t Nt;
    int W;
    int W8;
    int b;
    int d;
    __device__ __forceinline__ int wt(int x) const { return (x & 1) ? b : 128 - b; }
    __device__ __forceinline__ int64_t base(int x) const {
        return (int64_t)(x >> 1) * 128 + ((x & 1) ? 128 - b : 0);
    }
    // wh summed over the first j waves of an XCD
    __device__ __forceinline__ int64_t halves(int j) const {
        const int H = W8 / 2;
        return j < H ? (int64_t)j * (64 + d) : (int64_t)H * (64 + d) + (int64_t)(j - H) * (64 - d);
    }
    __device__ __forceinline__ int64_t S(int w) const {
        if (W8 == 0) return 4096ll * w;
        const int x = w / W8;
        return 64ll * W8 * base(x) + (int64_t)wt(x) * halves(w - x * W8);
    }
    // First tile of wave w (w = W gives Nt).
    __device__ __forceinline__ int64_t start(int w) const { return div_floor(Nt * S(w), 4096ll * W); }
    // The wave whose tiles include tile t: the last w with start(w) <= t, i.e.
    // with S(w) <= T = floor(((t + 1) 4096 W - 1) / Nt).
    __device__ __forceinline__ int wave_of(int64_t t) const {
        const int64_t T = div_floor((t + 1) * 4096ll * W - 1, Nt);
        if (W8 == 0) return (int)min<int64_t>(W - 1, T / 4096);
        int x = 7;
        while (x > 0 && 64ll * W8 * base(x) > T) --x;
        const int64_t R = T - 64ll * W8 * base(x);  // shares into XCD x
        const int H = W8 / 2;
        const int64_t first = (int64_t)wt(x) * H * (64 + d);
        const int64_t j = R < first ? R / ((int64_t)wt(x) * (64 + d)) : H + (R - first) / ((int64_t)wt(x) * (64 - d));
        return x * W8 + (int)min<int64_t>(W8 - 1, j);
    }
};

// The split for W of the grid's waves.  The weighted shares apply when W is
// the whole grid, the grid is a whole number of waves per XCD, and the
// smallest share is still at least one tile (Nt * min(b, 128 - b) * (64 - d)
// >= 4096 W): every wave below W then owns a tile, so the waves that touch a
// unit are consecutive and each leaves a partial result.  The halves apply
// with the XCD shares (launches of two waves per SIMD) when every XCD has an
// even number of waves.
__device__ __forceinline__ Split make_split(int64_t Nt, int W, int grid_waves, int balance) {
    const int lo = balance < 128 - balance ? balance : 128 - balance;
    const int W8 = grid_waves / 8;
    const int d = W8 % 2 == 0 ? kFirstHalfShare : 0;
    const bool per_xcd = W == grid_waves && grid_waves % 8 == 0 && balance != 64 && balance > 0 &&
                         balance < 128 && Nt * lo * (64 - d) >= 4096ll * W;
    return Split{Nt, W, per_xcd ? W8 : 0, per_xcd ? balance : 64, per_xcd ? d : 0};
}

__device__ __forceinline__ int tiles_of(int ctx, int table_tokens) {
    return (ctx < 0 || ctx > table_tokens) ? 0 : (ctx + kTok - 1) / kTok;
}

// Tiles of tokens [start, ctx) of a sequence; 0 when the pair is not valid
// (start outside [0, ctx] or not a whole number of tiles, ctx past the table).
__device__ __forceinline__ int tiles_from(int ctx, int start, int table_tokens) {
    return (start < 0 || start > ctx || ctx > table_tokens || (start & (kTok - 1)) != 0)
               ? 0
               : (ctx - start + kTok - 1) / kTok;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// 2^x with the hardware instruction alone (no denormal-range fix-up: softmax
// weights below 2^-126 flush to zero, far below the fp32 accumulation error).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace
}  // namespace pkv
