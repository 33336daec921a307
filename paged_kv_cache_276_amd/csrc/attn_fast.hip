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
//   * online softmax in log2 units: the running max only moves when a score
//     exceeds it by more than 8 (so exp2 stays <= 256); a ballot detects that
//     case, and only then is the tile max reduced along the 16-lane row (DPP)
//     and the accumulator rescaled; p = exp2(s - m), tail tokens masked by
//     select.
//   * P.V on the vector ALUs in fp32: lane l owns dims 8*(l%16) .. +7 of tokens
//     4*i + l/16 (i = 0..3), i.e. each V load instruction reads 1 KiB
//     contiguous; the weights p travel through 512 bytes of LDS.
// When the wave leaves a (sequence, KV head) it folds the four lane groups,
// then either normalises and writes the output rows (it saw every tile of the
// unit) or stores (m, l, acc) as a partial result at slot unit + wave; the
// wave that saw the unit's first tile records the unit's first slot and
// partial count.  merge_fast_kernel then merges the partials with log-sum-exp
// in slot order and writes the rows of sequences without tiles.
//
// Block-table entries are fetched 64 at a time into a lane-indexed window and
// picked out with readlane.  Tile buffers form a ring: the loads of tiles
// t + 1 and t + 2 (t + 1 only, for G = 8) are in flight while tile t is
// computed.
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

// Wait for every outstanding vector-memory load (vmcnt 0; expcnt and lgkmcnt
// left at their maxima).  Placed at the end of the rare branches that load
// (block-table refill, a unit's q) so the common path's waits count only the
// tile loads and the next tile stays in flight.
__device__ __forceinline__ void drain_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// 2^x with the hardware instruction alone (no denormal-range fix-up: softmax
// weights below 2^-126 flush to zero, far below the fp32 accumulation error).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

struct Cursor {
    int i;             // sequence
    int g;             // KV head
    int b;             // tile within the (sequence, KV head) unit
    int n;             // tiles of the unit
    int ctx;           // tokens of the sequence
    int64_t seq_base;  // global index of the sequence's first tile
};

struct TileLoad {
    uint4 k[4];  // MFMA B fragments of the 16 key rows
    uint4 v[4];  // value rows 4*i + lane/16, dims 8*(lane%16) .. +7
    Cursor c;    // which tile
    int valid;   // tokens of the tile inside the sequence
    bool bad;    // the block-table entry was outside the pool
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

    // Issue the K and V loads of the tile under cursor c.
    auto issue = [&](const Cursor& c, TileLoad& T) {
        T.c = c;
        const int tok0 = c.b * kTok;
        const int blk = tok0 / BS;
        if (c.i != win_i || blk < win_b0 || blk >= win_b0 + kWave) {
            win_i = c.i;
            win_b0 = blk;
            const int e = blk + lane;
            win = e < maxB ? bt[(int64_t)c.i * maxB + e] : -1;
            drain_vmem();
        }
        int phys = read_lane(win, blk - win_b0);
        T.bad = (unsigned)phys >= (unsigned)a.num_blocks;
        if (T.bad) phys = 0;
        T.valid = min(kTok, c.ctx - tok0);
        // The tile's base address is wave-uniform: keep it in scalar registers
        // and give the loads 32-bit lane offsets.
        const int64_t tile = (((int64_t)phys * Hkv + c.g) * BS + (tok0 % BS)) * kHd;
        const uint32_t tlo = __builtin_amdgcn_readfirstlane((uint32_t)tile);
        const uint32_t thi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)tile >> 32));
        const int64_t tile_s = (int64_t)(((uint64_t)thi << 32) | tlo);
        const uint16_t* kt = kbase + tile_s;
        const uint16_t* vt = vbase + tile_s;
        const uint32_t koff = (uint32_t)(r16 * kHd + grp * 8);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) T.k[kk] = *reinterpret_cast<const uint4*>(kt + koff + kk * 32);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const uint32_t voff = (uint32_t)min(4 * ii + grp, T.valid - 1) * (uint32_t)kHd + (uint32_t)r16 * 8u;
            T.v[ii] = *reinterpret_cast<const uint4*>(vt + voff);
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
                drain_vmem();
            }
        }
    };

    __shared__ float4 p_lds[16 * ROWS];

    uint4 qc[4];
    float acc[G][8];
    float m[4], l[4];
    bool bad = false, from_start = false;

    // Leave the current unit: write its output (the wave saw every tile of it)
    // or a partial result at slot unit + wave; the wave that saw the unit's
    // first tile records where the unit's partials start and how many there
    // are (waves from the one holding its first tile to the one holding its
    // last), for the merge kernel.
    auto finish_unit = [&](const Cursor& C, bool unit_end) {
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
        const int64_t u = (int64_t)C.i * Hkv + C.g;
        if (from_start && unit_end) {
            if (lane < 16) {
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float inv = bad ? NAN : 1.f / read_lane(lsum[h & 3], 16 * (h >> 2));
                    float4* o = reinterpret_cast<float4*>(
                        a.out + ((int64_t)C.i * Hq + (int64_t)C.g * G + h) * kHd + 8 * lane);
                    o[0] = make_float4(acc[h][0] * inv, acc[h][1] * inv, acc[h][2] * inv, acc[h][3] * inv);
                    o[1] = make_float4(acc[h][4] * inv, acc[h][5] * inv, acc[h][6] * inv, acc[h][7] * inv);
                }
            }
            if (lane == 0) a.ws_rec[u] = make_int2((int)(u + w), 1);
            return;
        }
        const int64_t slot = u + w;
        if (lane < 16) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float4* pa = reinterpret_cast<float4*>(a.ws_acc + (slot * G + h) * kHd + 8 * lane);
                pa[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
                pa[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float lh = read_lane(lsum[h & 3], 16 * (h >> 2));
            const float mh = read_lane(m[h & 3], 16 * (h >> 2));
            if (lane == h) a.ws_ml[slot * G + h] = make_float2(mh, bad ? NAN : lh);
        }
        if (from_start && lane == 0) {
            const int64_t last_tile = C.seq_base + (int64_t)C.g * C.n + C.n - 1;
            const int64_t w_last = ((last_tile + 1) * W - 1) / Nt;
            a.ws_rec[u] = make_int2((int)slot, (int)(w_last - w + 1));
        }
    };

    // Entering a tile: at a unit's first tile (or the chunk's first) load the
    // unit's q and reset the running state.  Called before the next tile's
    // loads are issued, so its drain waits only for data this tile needs.
    auto begin = [&](int64_t t, const TileLoad& T) {
        const Cursor& C = T.c;
        if (t == c0 || C.b == 0) {
            const uint4* src = reinterpret_cast<const uint4*>(
                qbase + ((int64_t)C.i * Hq + (int64_t)C.g * G + (r16 < G ? r16 : 0)) * kHd + grp * 8);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) qc[kk] = r16 < G ? src[kk * 4] : make_uint4(0, 0, 0, 0);
            drain_vmem();
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
    };

    // One tile: scores by MFMA, online softmax, P.V into the accumulator.
    auto step = [&](int64_t t, const TileLoad& T) {
        const Cursor& C = T.c;
        bad = bad || T.bad;

        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qc[kk]), as_bf16x8(T.k[kk]), sc, 0, 0, 0);

        const bool tok_ok = r16 < T.valid;
        float s[4];
        bool need = false;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            s[r] = tok_ok ? sc[r] * qscale : -INFINITY;
            need = need || (s[r] > m[r] + kLazyRescale);
        }
        // The running max moves only when some score passes it by more than
        // the threshold (always on a unit's first tile, rarely after); only
        // then is the tile max reduced along the row and the state rescaled.
        if (__any(need && lane < 16 * ROWS)) {
            float alpha[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float tm = row_max16(s[r]);
                const float mn = tm > m[r] + kLazyRescale ? tm : m[r];
                alpha[r] = fast_exp2(m[r] - mn);
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
            p[r] = fast_exp2(s[r] - m[r]);
            l[r] += p[r];
        }
        // The weights move from the score layout to the P.V layout through LDS.
        // One wave per workgroup: LDS operations of a wave complete in order,
        // the fences only keep the compiler from moving them.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        if (lane < 16 * ROWS) p_lds[lane] = make_float4(p[0], p[1], p[2], p[3]);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();

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
            const uint4 u = T.v[ii];
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
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();

        const bool unit_end = (C.b == C.n - 1);
        if (unit_end || t + 1 == c1) finish_unit(C, unit_end);
    };

    // Tile buffers in a ring: while tile t is computed, the next tiles are in
    // flight (two of them for G <= 4; for G = 8 the wider accumulator leaves
    // room for one).  Every phase issues exactly one tile's loads (past the
    // end of the run it requests the tile issued last again, which the cache
    // holds), so all paths issue the same loads in the same order and each
    // wait counts exactly the loads it needs.
    if constexpr (G <= 4) {
        auto phase = [&](int64_t tt, TileLoad& cur, TileLoad& ahead) {
            if (tt < c1) begin(tt, cur);
            if (tt + 2 < c1) advance(P);
            issue(P, ahead);  // tile tt + 2
            if (tt < c1) step(tt, cur);
        };
        TileLoad X0, X1, X2;
        issue(P, X0);
        if (c0 + 1 < c1) advance(P);
        issue(P, X1);
        for (int64_t t = c0; t < c1; t += 3) {
            phase(t, X0, X2);
            phase(t + 1, X1, X0);
            phase(t + 2, X2, X1);
        }
    } else {
        auto phase = [&](int64_t tt, TileLoad& cur, TileLoad& ahead) {
            if (tt < c1) begin(tt, cur);
            if (tt + 1 < c1) advance(P);
            issue(P, ahead);  // tile tt + 1
            if (tt < c1) step(tt, cur);
        };
        TileLoad X0, X1;
        issue(P, X0);
        for (int64_t t = c0; t < c1; t += 2) {
            phase(t, X0, X1);
            phase(t + 1, X1, X0);
        }
    }
}

// Merge kernel: one workgroup per (sequence, KV head) unit, one wave per query
// head of the group.  Units the partition kernel finished (one partial) are
// left alone; otherwise head h gets M = max_p m_p, L = sum_p 2^(m_p - M) l_p
// and out = sum_p 2^(m_p - M) acc_p / L over the unit's partials in slot
// order.  Sequences without tiles get zero rows (empty) or NaN rows (length
// outside the table).  Lanes own two output columns each.
template <int G>
__global__ __launch_bounds__(64 * G) void merge_fast_kernel(const DecodeArgs a, int table_tokens) {
    const int lane = threadIdx.x & (kWave - 1);
    const int h = threadIdx.x / kWave;
    const int64_t u = blockIdx.x;
    const int i = (int)(u / a.num_kv_heads);
    const int g = (int)(u % a.num_kv_heads);
    const int ctx = a.context_lens[i];
    float2* out = reinterpret_cast<float2*>(
        a.out + ((int64_t)i * a.num_q_heads + (int64_t)g * G + h) * kHd + 2 * lane);
    if (tiles_of(ctx, table_tokens) == 0) {
        const float v = ctx == 0 ? 0.f : NAN;
        *out = make_float2(v, v);
        return;
    }
    const int2 rec = a.ws_rec[u];
    const int np = rec.y;
    if (np == 1) return;
    const int64_t slots = (int64_t)a.num_seqs * a.num_kv_heads + kMaxGridWaves;
    if (np < 1 || rec.x < 0 || (int64_t)rec.x + np > slots) {  // never written: refuse to read
        *out = make_float2(NAN, NAN);
        return;
    }
    const float2* ml = a.ws_ml + (int64_t)rec.x * G + h;
    float M = -INFINITY;
    for (int p = lane; p < np; p += kWave) M = fmaxf(M, ml[(int64_t)p * G].x);
    M = wave_max(M);
    float L = 0.f;
    for (int p = lane; p < np; p += kWave) {
        const float2 v = ml[(int64_t)p * G];
        L += exp2f(v.x - M) * v.y;
    }
    L = wave_sum(L);
    const float* acc = a.ws_acc + ((int64_t)rec.x * G + h) * kHd + 2 * lane;
    const int64_t pstride = (int64_t)G * kHd;
    float o0 = 0.f, o1 = 0.f;
    int p = 0;
    for (; p + 4 <= np; p += 4) {  // four partials' loads in flight at once
        float2 v[4], mlv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[k] = *reinterpret_cast<const float2*>(acc + (p + k) * pstride);
            mlv[k] = ml[(int64_t)(p + k) * G];
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float wgt = exp2f(mlv[k].x - M);
            o0 = fmaf(wgt, v[k].x, o0);
            o1 = fmaf(wgt, v[k].y, o1);
        }
    }
    for (; p < np; ++p) {
        const float2 v = *reinterpret_cast<const float2*>(acc + p * pstride);
        const float wgt = exp2f(ml[(int64_t)p * G].x - M);
        o0 = fmaf(wgt, v.x, o0);
        o1 = fmaf(wgt, v.y, o1);
    }
    *out = make_float2(o0 / L, o1 / L);
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
    const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads;
    hipLaunchKernelGGL((merge_fast_kernel<G>), dim3((unsigned)units), dim3(kWave * G), 0, stream, a,
                       a.max_blocks_per_seq * BS);
    return hipGetLastError();
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

}  // namespace pkv
