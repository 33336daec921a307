// attn_fast.hip -- paged decode attention for bf16 caches with head_dim 128
// (block sizes 16, 32, 64; query-group sizes 1, 2, 4, 8) on gfx950.
//
// Work decomposition.  The unit of work is a tile: 16 consecutive logical
// tokens of one (sequence, KV head).  All tiles are laid end to end in the
// order (sequence, KV head, tile) and the grid's W waves each take an equal
// contiguous run of them (W = the waves the device keeps resident), so the
// load is balanced whatever the length mix: a long sequence spreads over many
// waves, many short ones share a wave.  Each wave finds its first tile from
// the context lengths alone (two passes of a wave-wide prefix sum), so no host
// synchronisation or planning kernel is needed.
//
// Per tile (4 KiB of K and 4 KiB of V for one KV head):
//   * scores: the G query rows of the KV head (zero-padded to 16) times the 16
//     key rows, as four v_mfma_f32_16x16x32_bf16 (A = q, B = K^T).  Each lane
//     loads its B fragment straight from HBM: token (lane % 16), 8 consecutive
//     dims per MFMA, so one load instruction reads 64 contiguous bytes of each
//     of the 16 rows.  Lane t < 16 (t < 32 for G = 8) ends up with the scores
//     of token t for four query heads.
//   * online softmax in log2 units: the tile max per head is a 16-lane DPP
//     reduction; the running max only moves when the tile max exceeds it by
//     more than 8 (so exp2 stays <= 256 and the rescale of the accumulator is
//     rare); p = exp2(s - m) with tail tokens masked by select.
//   * P.V on the vector ALUs in fp32: lane l owns dims 8*(l%16) .. +7 of tokens
//     4*i + l/16 (i = 0..3), i.e. each V load instruction reads 1 KiB
//     contiguous; the weights p travel through 512 bytes of LDS.
// When the wave leaves a (sequence, KV head) it folds the four lane groups,
// then either normalises and writes the output row (it saw every tile of the
// unit) or stores (m, l, acc) as a partial result; the wave that saw the
// unit's first tile also records where the unit's partials start and how many
// there are.  combine_fast_kernel merges the partials with log-sum-exp.
//
// Block-table entries are fetched 64 at a time into a lane-indexed window and
// picked out with readlane; the next tile's K, V and (on a unit change) q are
// requested before the current tile is computed.
#include <math.h>

#include <map>
#include <mutex>
#include <utility>

#include "device_common.h"
#include "launch.h"

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

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

__device__ __forceinline__ int wave_incl_scan_int(int v, int lane) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int t = __shfl_up(v, d, kWave);
        if (lane >= d) v += t;
    }
    return v;
}

__device__ __forceinline__ int tiles_of(int ctx, int table_tokens) {
    return (ctx < 0 || ctx > table_tokens) ? 0 : (ctx + kTok - 1) / kTok;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

struct Cursor {
    int i;             // sequence
    int g;             // KV head
    int b;             // tile within the (sequence, KV head) unit
    int n;             // tiles of the unit
    int ctx;           // tokens of the sequence
    int64_t seq_base;  // global index of the sequence's first tile
};

}  // namespace

template <int BS, int G>
__global__ __launch_bounds__(64) void decode_fast_kernel(const DecodeArgs a, float qscale) {
    static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
    static_assert(BS % kTok == 0, "block size");
    constexpr int ROWS = (G + 3) / 4;  // 16-lane rows that hold scores
    const int lane = threadIdx.x;
    const int nwaves = gridDim.x;
    const int bid = blockIdx.x;
    // Consecutive runs of tiles go to one XCD (workgroups are dealt to the 8
    // XCDs round-robin), so sequences sharing prefix blocks meet in one L2.
    const int w = (nwaves % 8 == 0) ? (bid % 8) * (nwaves / 8) + bid / 8 : bid;

    const int S = a.num_seqs;
    const int Hkv = a.num_kv_heads;
    const int Hq = a.num_q_heads;
    const int maxB = a.max_blocks_per_seq;
    const int table_tokens = maxB * BS;
    const int32_t* __restrict__ ctxp = a.context_lens;

    // ---- 1. total tiles
    int total = 0;
    for (int base = 0; base < S; base += kWave * 8) {
        int s = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int i = base + lane * 8 + k;
            if (i < S) s += tiles_of(ctxp[i], table_tokens);
        }
        total += wave_sum_int(s);
    }
    const int64_t Nt = (int64_t)total * Hkv;
    if (Nt == 0) return;
    const int W = (int)(Nt < nwaves ? Nt : nwaves);
    if (w >= W) return;
    const int64_t c0 = (int64_t)w * Nt / W;
    const int64_t c1 = (int64_t)(w + 1) * Nt / W;

    // ---- 2. the sequence holding tile c0
    int i0 = -1;
    int64_t base0 = 0;
    {
        int64_t acc = 0;
        for (int base = 0; base < S; base += kWave * 8) {
            int nv[8];
            int s = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = base + lane * 8 + k;
                nv[k] = i < S ? tiles_of(ctxp[i], table_tokens) : 0;
                s += nv[k];
            }
            const int incl = wave_incl_scan_int(s, lane);
            const int64_t chunk = (int64_t)read_lane(incl, kWave - 1) * Hkv;
            if (c0 < acc + chunk) {
                const unsigned long long mask = __ballot(acc + (int64_t)incl * Hkv > c0);
                const int L = __ffsll(mask) - 1;
                int64_t b0 = acc + (int64_t)read_lane(incl - s, L) * Hkv;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int n = read_lane(nv[k], L);
                    if (i0 < 0) {
                        if (c0 < b0 + (int64_t)n * Hkv) {
                            i0 = base + L * 8 + k;
                            base0 = b0;
                        } else {
                            b0 += (int64_t)n * Hkv;
                        }
                    }
                }
                break;
            }
            acc += chunk;
        }
    }

    if (i0 < 0) return;  // unreachable when the two passes agree; keeps every index below in range

    const uint16_t* __restrict__ qbase = static_cast<const uint16_t*>(a.q);
    const uint16_t* __restrict__ kbase = static_cast<const uint16_t*>(a.k_cache);
    const uint16_t* __restrict__ vbase = static_cast<const uint16_t*>(a.v_cache);
    const int32_t* __restrict__ bt = a.block_tables;

    Cursor P;
    P.i = i0;
    P.ctx = ctxp[i0];
    P.n = tiles_of(P.ctx, table_tokens);
    P.seq_base = base0;
    {
        const int64_t off = c0 - base0;
        P.g = (int)(off / P.n);
        P.b = (int)(off % P.n);
    }

    // block-table window: lane k holds entry win_b0 + k of sequence win_i
    int win = -1, win_i = -1, win_b0 = 0;

    const int r16 = lane & 15;  // MFMA column (token) / V column group
    const int grp = lane >> 4;  // MFMA k-group / V token phase

    auto load_q = [&](const Cursor& c, uint4 (&qf)[4]) {
        if (r16 < G) {
            const uint4* src = reinterpret_cast<const uint4*>(
                qbase + ((int64_t)c.i * Hq + (int64_t)c.g * G + r16) * kHd + grp * 8);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) qf[kk] = src[kk * 4];
        } else {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) qf[kk] = make_uint4(0, 0, 0, 0);
        }
    };

    // Issue the loads of tile c; returns its valid rows and whether its block id was bad.
    auto fetch = [&](const Cursor& c, uint4 (&kf)[4], uint4 (&vf)[4], int& valid, bool& badt) {
        const int tok0 = c.b * kTok;
        const int blk = tok0 / BS;
        if (c.i != win_i || blk < win_b0 || blk >= win_b0 + kWave) {
            win_i = c.i;
            win_b0 = blk;
            const int e = blk + lane;
            win = e < maxB ? bt[(int64_t)c.i * maxB + e] : -1;
        }
        int phys = read_lane(win, blk - win_b0);
        badt = (unsigned)phys >= (unsigned)a.num_blocks;
        if (badt) phys = 0;
        valid = min(kTok, c.ctx - tok0);
        const int64_t tile = (((int64_t)phys * Hkv + c.g) * BS + (tok0 % BS)) * kHd;
        const uint4* kp = reinterpret_cast<const uint4*>(kbase + tile + r16 * kHd) + grp;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) kf[kk] = kp[kk * 4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int row = min(4 * ii + grp, valid - 1);
            vf[ii] = reinterpret_cast<const uint4*>(vbase + tile + row * kHd)[r16];
        }
    };

    auto advance = [&](Cursor& c) {
        if (++c.b == c.n) {
            c.b = 0;
            if (++c.g == Hkv) {
                c.g = 0;
                c.seq_base += (int64_t)Hkv * c.n;
                do {
                    ++c.i;
                    c.ctx = ctxp[c.i];
                    c.n = tiles_of(c.ctx, table_tokens);
                } while (c.n == 0);
            }
        }
    };

    __shared__ float4 p_lds[16 * ROWS];

    uint4 qc[4], qn[4], kc[4], vc[4], kn[4], vn[4];
    int valid_n;
    bool bad_n;
    load_q(P, qn);
    fetch(P, kn, vn, valid_n, bad_n);

    float acc[G][8];
    float m[4], l[4];
    bool bad = false, from_start = false;

    for (int64_t t = c0; t < c1; ++t) {
        const Cursor C = P;
        const int valid = valid_n;
        const bool bad_t = bad_n;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            kc[k] = kn[k];
            vc[k] = vn[k];
        }
        const bool first = (t == c0) || (C.b == 0);
        if (first) {
#pragma unroll
            for (int k = 0; k < 4; ++k) qc[k] = qn[k];
        }
        if (t + 1 < c1) {  // request the next tile before computing this one
            advance(P);
            if (P.b == 0) load_q(P, qn);
            fetch(P, kn, vn, valid_n, bad_n);
        }
        if (first) {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                m[r] = -INFINITY;
                l[r] = 0.f;
            }
            bad = false;
            from_start = (C.b == 0);
        }
        bad = bad || bad_t;

        // scores of the 16 tokens for the (padded) query rows
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qc[kk]), as_bf16x8(kc[kk]), sc, 0, 0, 0);

        const bool tok_ok = r16 < valid;
        float s[4], tm[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            s[r] = tok_ok ? sc[r] * qscale : -INFINITY;
            tm[r] = row_max16(s[r]);
        }
        bool need = false;
#pragma unroll
        for (int r = 0; r < 4; ++r) need = need || (tm[r] > m[r] + kLazyRescale);
        if (__any(need && lane < 16 * ROWS)) {
            float alpha[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float mn = tm[r] > m[r] + kLazyRescale ? tm[r] : m[r];
                alpha[r] = exp2f(m[r] - mn);
                m[r] = mn;
                l[r] *= alpha[r];
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float ah = read_lane(alpha[h & 3], 16 * (h >> 2));
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] *= ah;
            }
        }
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p[r] = exp2f(s[r] - m[r]);
            l[r] += p[r];
        }
        if (lane < 16 * ROWS) p_lds[lane] = make_float4(p[0], p[1], p[2], p[3]);
        __syncthreads();

#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int trow = 4 * ii + grp;
            float pw[8];
            const float4 p0 = p_lds[trow];
            pw[0] = p0.x; pw[1] = p0.y; pw[2] = p0.z; pw[3] = p0.w;
            if (G == 8) {
                const float4 p1 = p_lds[16 + trow];
                pw[4] = p1.x; pw[5] = p1.y; pw[6] = p1.z; pw[7] = p1.w;
            }
            const uint4 u = vc[ii];
            float vv[8];
            vv[0] = bf16_lo(u.x); vv[1] = bf16_hi(u.x);
            vv[2] = bf16_lo(u.y); vv[3] = bf16_hi(u.y);
            vv[4] = bf16_lo(u.z); vv[5] = bf16_hi(u.z);
            vv[6] = bf16_lo(u.w); vv[7] = bf16_hi(u.w);
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pw[h], vv[e], acc[h][e]);
        }
        __syncthreads();

        const bool unit_end = (C.b == C.n - 1);
        if (unit_end || t + 1 == c1) {
            // fold the four token phases: every lane group then holds the full sums
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    acc[h][e] += __shfl_xor(acc[h][e], 16, kWave);
                    acc[h][e] += __shfl_xor(acc[h][e], 32, kWave);
                }
            float lsum[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) lsum[r] = row_sum16(l[r]);
            const int u = C.i * Hkv + C.g;
            const bool complete = from_start && unit_end;
            if (complete) {
                if (lane < 16) {
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        const float lh = read_lane(lsum[h & 3], 16 * (h >> 2));
                        const float inv = 1.f / lh;
                        float* o = a.out + ((int64_t)C.i * Hq + (int64_t)C.g * G + h) * kHd + 8 * lane;
                        float4 o0, o1;
                        o0.x = acc[h][0] * inv; o0.y = acc[h][1] * inv; o0.z = acc[h][2] * inv; o0.w = acc[h][3] * inv;
                        o1.x = acc[h][4] * inv; o1.y = acc[h][5] * inv; o1.z = acc[h][6] * inv; o1.w = acc[h][7] * inv;
                        if (bad) o0 = o1 = make_float4(NAN, NAN, NAN, NAN);
                        reinterpret_cast<float4*>(o)[0] = o0;
                        reinterpret_cast<float4*>(o)[1] = o1;
                    }
                }
            } else {
                const int64_t slot = (int64_t)u + w;
                if (lane < 16) {
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        float* pa = a.ws_acc + (slot * G + h) * kHd + 8 * lane;
                        reinterpret_cast<float4*>(pa)[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
                        reinterpret_cast<float4*>(pa)[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
                    }
                }
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float lh = read_lane(lsum[h & 3], 16 * (h >> 2));
                    const float mh = read_lane(m[h & 3], 16 * (h >> 2));
                    if (lane == 0) a.ws_ml[slot * G + h] = make_float2(mh, bad ? NAN : lh);
                }
            }
            if (from_start && lane == 0) {
                const int64_t last_tile = C.seq_base + (int64_t)C.g * C.n + C.n - 1;
                const int64_t w_last = ((last_tile + 1) * W - 1) / Nt;
                a.ws_rec[u] = make_int2(u + w, (int)(w_last - w + 1));
            }
        }
    }
}

// One wave per (sequence, query head) row: merge the partial results of the
// row's unit; rows finished by the partition kernel (one partial) are left
// alone.  Empty sequences get zeros, out-of-range lengths NaN.
template <int G>
__global__ __launch_bounds__(64) void combine_fast_kernel(const DecodeArgs a, int table_tokens) {
    const int lane = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int i = (int)(row / a.num_q_heads);
    const int h = (int)(row % a.num_q_heads);
    const int g = h / G, hh = h % G;
    const int ctx = a.context_lens[i];
    float* out = a.out + row * kHd + 2 * lane;
    if (ctx < 0 || ctx > table_tokens) {
        out[0] = NAN;
        out[1] = NAN;
        return;
    }
    if (ctx == 0) {
        out[0] = 0.f;
        out[1] = 0.f;
        return;
    }
    const int2 rec = a.ws_rec[(int64_t)i * a.num_kv_heads + g];
    const int np = rec.y;
    if (np == 1) return;
    const int64_t slots = (int64_t)a.num_seqs * a.num_kv_heads + kMaxGridWaves;
    if (np < 1 || rec.x < 0 || (int64_t)rec.x + np > slots) {  // never written: refuse to read
        out[0] = NAN;
        out[1] = NAN;
        return;
    }
    const float2* ml = a.ws_ml + (int64_t)rec.x * G + hh;
    float M = -INFINITY;
    for (int p = lane; p < np; p += kWave) M = fmaxf(M, ml[(int64_t)p * G].x);
    M = wave_max(M);
    float L = 0.f;
    for (int p = lane; p < np; p += kWave) {
        const float2 v = ml[(int64_t)p * G];
        L += exp2f(v.x - M) * v.y;
    }
    L = wave_sum(L);
    float o0 = 0.f, o1 = 0.f;
    const float* acc = a.ws_acc + ((int64_t)rec.x * G + hh) * kHd + 2 * lane;
    for (int p = 0; p < np; ++p) {
        const float wgt = exp2f(ml[(int64_t)p * G].x - M);
        const float2 v = *reinterpret_cast<const float2*>(acc + (int64_t)p * G * kHd);
        o0 = fmaf(wgt, v.x, o0);
        o1 = fmaf(wgt, v.y, o1);
    }
    out[0] = o0 / L;
    out[1] = o1 / L;
}

namespace {

// Resident waves of one kernel on the current device (cached).
int resident_waves(const void* kernel) {
    static std::mutex mu;
    static std::map<std::pair<int, const void*>, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    auto key = std::make_pair(dev, kernel);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kWave, 0) != hipSuccess) return 0;
    int waves = cus * (per_cu > 0 ? per_cu : 1);
    waves = waves / 8 * 8;
    if (waves < 8) waves = 8;
    if (waves > kMaxGridWaves) waves = kMaxGridWaves;
    cache[key] = waves;
    return waves;
}

template <int BS, int G>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
    const void* k = reinterpret_cast<const void*>(&decode_fast_kernel<BS, G>);
    int waves = a.grid_waves > 0 ? a.grid_waves : resident_waves(k);
    if (waves <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_fast_kernel<BS, G>), dim3(waves), dim3(kWave), 0, stream, a, a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_combine_fast(a, stream);
}

template <int BS>
hipError_t by_group(const DecodeArgs& a, hipStream_t stream) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_t<BS, 1>(a, stream);
        case 2: return launch_t<BS, 2>(a, stream);
        case 4: return launch_t<BS, 4>(a, stream);
        case 8: return launch_t<BS, 8>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool fast_supports(int32_t dtype, int32_t head_dim, int32_t block_size, int32_t group) {
    const bool g_ok = group == 1 || group == 2 || group == 4 || group == 8;
    const bool b_ok = block_size == 16 || block_size == 32 || block_size == 64;
    return dtype == 1 && head_dim == kHd && b_ok && g_ok;
}

hipError_t launch_decode_fast(const DecodeArgs& a, hipStream_t stream) {
    switch (a.block_size) {
        case 16: return by_group<16>(a, stream);
        case 32: return by_group<32>(a, stream);
        case 64: return by_group<64>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_combine_fast(const DecodeArgs& a, hipStream_t stream) {
    const int64_t rows = (int64_t)a.num_seqs * a.num_q_heads;
    if (rows == 0) return hipSuccess;
    const int table_tokens = a.max_blocks_per_seq * a.block_size;
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: hipLaunchKernelGGL(combine_fast_kernel<1>, dim3((unsigned)rows), dim3(kWave), 0, stream, a, table_tokens); break;
        case 2: hipLaunchKernelGGL(combine_fast_kernel<2>, dim3((unsigned)rows), dim3(kWave), 0, stream, a, table_tokens); break;
        case 4: hipLaunchKernelGGL(combine_fast_kernel<4>, dim3((unsigned)rows), dim3(kWave), 0, stream, a, table_tokens); break;
        case 8: hipLaunchKernelGGL(combine_fast_kernel<8>, dim3((unsigned)rows), dim3(kWave), 0, stream, a, table_tokens); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pkv
