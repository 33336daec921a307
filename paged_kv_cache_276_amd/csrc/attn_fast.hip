// attn_fast.hip -- paged decode attention for bf16 caches with head_dim 128
// (block sizes 8, 16, 32, 64; query-group sizes 1, 2, 4, 8) on gfx950.
//
// Work decomposition.  The unit of work is a tile: 16 consecutive logical
// tokens of one (sequence, KV head).  All tiles are laid end to end in the
// order (sequence, KV head, tile) and the grid's W waves each take one
// contiguous run of them (W = the waves the device keeps resident, or half of
// them for few long units: see launch_t), so the
// load is balanced whatever the length mix: a long sequence spreads over many
// waves, many short ones share a wave.  The runs are equal, or weighted by the
// wave's XCD (odd XCDs read more slowly) and by its half of the XCD's waves
// (the first wave of every SIMD drains faster; Split in tile_math.h).  Each wave
// finds its first tile from the context lengths alone (two passes of a
// wave-wide prefix sum), so no host synchronisation or planning kernel is
// needed.
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
// then stages either the normalised output rows (it saw every tile of the
// unit) or (m, l, acc) as a partial result for slot unit + wave in LDS; the
// stage is stored when the wave's run ends.  The wave that saw the unit's
// first tile records the unit's first slot and partial count.
// merge_fast_kernel then merges the partials with log-sum-exp in slot order
// and writes the rows of sequences without tiles.
//
// Set-up per segment (up to 128 tiles and 8 pieces of units): one walk over
// the segment's units writes a record per tile to LDS (element offset of the
// tile in the pools, valid rows, first/last/bad flags) with all block-table
// entries and q rows fetched by the lanes at once; the tile loop then reads
// one LDS record per tile.  Two tile buffers alternate: the loads of tile
// t + 1 are in flight while tile t is computed.
#include <math.h>

#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "device_common.h"
#include "launch.h"
#include "pagedkv.h"
#include "tile_math.h"

namespace pkv {

namespace {

struct Cursor {
    int i;             // sequence
    int start;         // first token of the sequence this kernel covers (0 without a shared prefix)
    int g;             // KV head
    int b;             // tile within the (sequence, KV head) unit
    int n;             // tiles of the unit
    int ctx;           // tokens of the sequence
    int64_t seq_base;  // global index of the sequence's first tile
};

struct TileLoad {
    uint4 k[4];      // MFMA B fragments of the 16 key rows
    uint4 v[4];      // value rows 4*i + lane/16, dims 8*(lane%16) .. +7
    uint32_t flags;  // valid rows | run << 8 | kFirst | kLast | kBad (the tile's record)
};

// Loads marked non-temporal: K and V rows are read once per call, and
// streaming them past the caches' replacement keeps the read rate up
// (16-byte pieces for the decode kernel, 4-byte ones for the multi-query
// kernels' LDS-staged tiles; the shared-prefix pass measured no gain).  The
// decode kernel streams V always and K when its units are few and long (see
// launch_t): with many units, K read with ordinary loads measured faster, and
// it keeps blocks that several sequences share in the caches.  The multi-query
// chunk kernel reads K with ordinary loads too (121.6 against 126.9 us on
// 64-token chunks of 16 x 4k); the split-run kernel streams both (121.2
// against 124.4 us on 4 new tokens x 64 sequences).
__device__ __forceinline__ uint4 load_plain(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint4 load_stream(const uint16_t* p) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t load_stream(const uint32_t* p) { return __builtin_nontemporal_load(p); }

// Device-coherent 64-bit load (another workgroup, maybe on another XCD, stored
// the value with a device-scope store in this launch).
__device__ __forceinline__ uint64_t load_agent(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kSegTiles = 128;  // tiles per segment (two per lane in the set-up)
constexpr uint32_t kFirst = 1u << 16;  // tile 0 of its unit
constexpr uint32_t kLast = 1u << 17;   // last tile of its unit
constexpr uint32_t kBad = 1u << 18;    // block-table entry outside the pool

}  // namespace

// START: every sequence i covers tokens [seq_start[i], ctx) only (the tokens
// before are a shared prefix handled by decode_prefix_kernel), and no unit is
// finished here: all of them leave partial results for the merge.
// KSTREAM: K rows read with non-temporal loads too (V rows always are).
template <int BS, int G, bool START, bool KSTREAM>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_fast_kernel(const DecodeArgs a,
                                                                                                  float qscale) {
    static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
    static_assert(BS == 8 || BS % kTok == 0, "block size");
    constexpr bool kSplit = BS < kTok;  // block size 8: a tile's rows 8..15 sit in the next block
    constexpr int ROWS = (G + 3) / 4;       // 16-lane rows that hold scores
    constexpr int kQv = (G * kHd * 2 + 1023) / 1024;  // 16-byte loads per lane for a unit's q rows
    constexpr int kSegRuns = G == 8 ? 4 : 8;          // runs (pieces of units) per segment
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

    // ---- 1. total tiles.  The lengths of the first 512 sequences stay in
    // registers (as tile counts) and in LDS, so for batches up to that size
    // the search below and the unit walk read no more global memory.
    __shared__ int ctx_lds[kWave * 8];
    __shared__ int start_lds[START ? kWave * 8 : 1];
    const bool lens_in_lds = S <= kWave * 8;
    const int32_t* __restrict__ startp = a.seq_start;
    auto tiles_at = [&](int c, int st) { return START ? tiles_from(c, st, table_tokens) : tiles_of(c, table_tokens); };
    int nv0[8];
    int s0 = 0;
    int total = 0;
    for (int base = 0; base < S; base += kWave * 8) {
        // All eight loads are issued before the first is used (the index is
        // clamped into range, the value masked after), so the pass costs one
        // memory round trip.
        int cv[8], sv[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int i = min(base + lane * 8 + k, S - 1);
            cv[k] = ctxp[i];
            sv[k] = START ? startp[i] : 0;
        }
        int s = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int i = base + lane * 8 + k;
            const int c = i < S ? cv[k] : 0;
            const int st = (START && i < S) ? sv[k] : 0;
            const int n = tiles_at(c, st);
            if (base == 0) {
                nv0[k] = n;
                ctx_lds[lane * 8 + k] = c;
                if (START) start_lds[lane * 8 + k] = st;
            }
            s += n;
        }
        if (base == 0) s0 = s;
        total += wave_sum_int(s);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int64_t Nt = (int64_t)total * Hkv;
    if (Nt == 0) return;
    const int W = (int)(Nt < nwaves ? Nt : nwaves);
    if (w >= W) return;
    const Split sp = make_split(Nt, W, nwaves, a.xcd_balance);
    const int64_t c0 = sp.start(w);
    const int64_t c1 = sp.start(w + 1);

    // ---- 2. the sequence holding tile c0
    int i0 = -1;
    int64_t base0 = 0;
    {
        int64_t acc = 0;
        for (int base = 0; base < S; base += kWave * 8) {
            int nv[8];
            int s = 0;
            if (base == 0) {
#pragma unroll
                for (int k = 0; k < 8; ++k) nv[k] = nv0[k];
                s = s0;
            } else {
                int cv[8], sv[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int i = min(base + lane * 8 + k, S - 1);
                    cv[k] = ctxp[i];
                    sv[k] = START ? startp[i] : 0;
                }
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int i = base + lane * 8 + k;
                    nv[k] = i < S ? tiles_at(cv[k], sv[k]) : 0;
                    s += nv[k];
                }
            }
            const int incl = wave_incl_scan_int(s);
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
    // Length of sequence i (wave-uniform i).
    auto len_of = [&](int i) -> int {
        return lens_in_lds ? __builtin_amdgcn_readfirstlane(ctx_lds[i]) : ctxp[i];
    };
    auto start_of = [&](int i) -> int {
        if (!START) return 0;
        return lens_in_lds ? __builtin_amdgcn_readfirstlane(start_lds[i]) : startp[i];
    };
    if (i0 < 0) return;  // unreachable when the two passes agree; keeps every index below in range

    const uint16_t* __restrict__ qbase = static_cast<const uint16_t*>(a.q);
    const uint16_t* __restrict__ kbase = static_cast<const uint16_t*>(a.k_cache);
    const uint16_t* __restrict__ vbase = static_cast<const uint16_t*>(a.v_cache);
    const int32_t* __restrict__ bt = a.block_tables;

    // Cursor at the next tile still to be placed in a segment.
    Cursor P;
    P.i = i0;
    P.ctx = len_of(i0);
    P.start = start_of(i0);
    P.n = tiles_at(P.ctx, P.start);
    P.seq_base = base0;
    {
        const int off = (int)(c0 - base0);  // < P.n * Hkv
        P.g = off / P.n;
        P.b = off - P.g * P.n;
    }

    const int r16 = lane & 15;  // MFMA column (token) / V column group
    const int grp = lane >> 4;  // MFMA k-group / V token phase

    // Issue the K and V loads of a tile from its record (element offset of
    // its 16 K/V rows in the pools, flags, second block of a split tile).
    // The tile's base address is wave-uniform: it goes to scalar registers,
    // the loads take 32-bit lane offsets.
    auto issue_rec = [&](const uint4 rv, TileLoad& T) {
        const uint32_t tlo = __builtin_amdgcn_readfirstlane(rv.x);
        const uint32_t thi = __builtin_amdgcn_readfirstlane(rv.y);
        T.flags = __builtin_amdgcn_readfirstlane(rv.z);
        const int64_t tile_s = (int64_t)(((uint64_t)thi << 32) | tlo);
        const int valid = (int)(T.flags & 0xffu);
        const uint16_t* kt = kbase + tile_s;
        const uint16_t* vt = vbase + tile_s;
        const uint32_t koff = (uint32_t)(r16 * kHd + grp * 8);
        if constexpr (kSplit) {
            // Rows BS.. of the tile live in the second block: they take
            // `diff` more elements than rows of the first block would.
            const int64_t tile2 = (int64_t)__builtin_amdgcn_readfirstlane(rv.w) * (BS * kHd);
            const int64_t diff = tile2 - (tile_s + (int64_t)BS * kHd);
            const int64_t kx = r16 >= BS ? diff : 0;
#pragma unroll
            for (int kq = 0; kq < 4; ++kq) T.k[kq] = KSTREAM ? load_stream(kt + koff + kq * 32 + kx) : load_plain(kt + koff + kq * 32 + kx);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int vr = min(4 * ii + grp, valid - 1);
                const int64_t voff = (int64_t)vr * kHd + r16 * 8 + (vr >= BS ? diff : 0);
                T.v[ii] = load_stream(vt + voff);
            }
        } else {
#pragma unroll
            for (int kq = 0; kq < 4; ++kq) T.k[kq] = KSTREAM ? load_stream(kt + koff + kq * 32) : load_plain(kt + koff + kq * 32);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const uint32_t voff = (uint32_t)min(4 * ii + grp, valid - 1) * (uint32_t)kHd + (uint32_t)r16 * 8u;
                T.v[ii] = load_stream(vt + voff);
            }
        }
    };

    // Each segment's first tile is issued before the segment's set-up (walk,
    // table entries, q rows), so that its latency overlaps the set-up; its
    // record is built from the cursor, exactly as the set-up builds it.  Every
    // segment enters the tile loop the same way, with that tile's loads
    // issued before the set-up's own loads, which keeps the loop's load waits
    // exact.
    auto issue_first = [&](const Cursor& C, TileLoad& T) {
        const int tok0 = C.start + C.b * kTok;
        const int64_t row = (int64_t)C.i * maxB + tok0 / BS;
        const int phys = bt[row];
        bool badp = (unsigned)phys >= (unsigned)a.num_blocks;
        const int ph = badp ? 0 : phys;
        uint32_t second = 0u;
        if constexpr (kSplit) {
            int ph2 = ph;
            if (tok0 + BS < C.ctx) {
                const int phys2 = bt[row + 1];
                const bool bad2 = (unsigned)phys2 >= (unsigned)a.num_blocks;
                badp = badp || bad2;
                ph2 = bad2 ? 0 : phys2;
            }
            second = (uint32_t)((int64_t)ph2 * Hkv + C.g);
        }
        const int64_t off = (((int64_t)ph * Hkv + C.g) * BS + (tok0 % BS)) * kHd;
        const uint32_t flags = (uint32_t)min(kTok, C.ctx - tok0) | (C.b == 0 ? kFirst : 0u) |
                               (C.b == C.n - 1 ? kLast : 0u) | (badp ? kBad : 0u);
        issue_rec(make_uint4((uint32_t)off, (uint32_t)((uint64_t)off >> 32), flags, second), T);
    };
    TileLoad X0, X1;

    // Per-segment tables in LDS (one wave per workgroup):
    //   rec[k]   tile k: element offset of its 16 K/V rows in the pools (x, y),
    //            valid rows | run << 8 | flags (z)
    //   qrow[r]  the G query rows of run r's (sequence, KV head), as stored in q
    //   run[r]   run r's sequence, KV head, tile count of the unit, first tile
    //            within the unit; seq_base, first segment slot, sequence length
    __shared__ uint4 rec_lds[kSegTiles];
    __shared__ uint4 q_lds[kSegRuns][kQv * kWave];
    __shared__ int4 run_lds[kSegRuns][2];
    __shared__ float4 p_lds[16 * ROWS];

    uint4 qc[4];
    float acc[G][8];
    float m[4], l[4];
    bool bad = false, from_start = false;
    int ui = 0, ug = 0, un = 1;  // unit being accumulated
    int useq_base = 0;           // global index of its sequence's first tile
    int ustart = 0;              // first token of its sequence covered here

    // Leave the current unit: its output (the wave saw every tile of it) or a
    // partial result for slot unit + wave; the wave that saw the unit's first
    // tile also records where the unit's partials start and how many there
    // are (waves from the one holding its first tile to the one holding its
    // last), for the merge kernel.  Results are staged in LDS and stored
    // together when the wave's run of tiles ends: a global store issued in
    // the middle of the run would hold back every load issued after it (the
    // memory counter retires in order), and under full read traffic a store
    // takes as long to be acknowledged as a tile takes to arrive.  A full
    // stage is flushed early.
    // Stage depth: what fits next to the other tables in 20 KB of LDS per
    // workgroup (eight workgroups per CU).
    constexpr int kStage = START ? (G == 1 ? 10 : G == 2 ? 5 : G == 4 ? 2 : 1)
                                 : (G == 1 ? 12 : G == 2 ? 6 : G == 4 ? 3 : 1);
    __shared__ float4 stage_acc[kStage][G * 32];  // result rows as stored: head h, dims 4f .. 4f + 3 at h * 32 + f
    __shared__ float2 stage_ml[kStage][G];        // partials: (m, l) per head
    __shared__ int4 stage_meta[kStage];           // partial?, unit, slot, record count (0: no record)
    int nstage = 0;                               // wave-uniform

    // Store the staged results: each one's G rows are G * 128 contiguous
    // floats of out (a finished unit) or of the partial slots; all 64 lanes
    // move 16 bytes per store.
    auto flush = [&]() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (int r = 0; r < nstage; ++r) {
            const int4 md = stage_meta[r];
            const bool part = __builtin_amdgcn_readfirstlane(md.x) != 0;
            const int64_t su = __builtin_amdgcn_readfirstlane(md.y);
            const int64_t sslot = __builtin_amdgcn_readfirstlane(md.z);
            const int rcount = __builtin_amdgcn_readfirstlane(md.w);
            float4* dst = reinterpret_cast<float4*>(part ? a.ws_acc + sslot * G * kHd : a.out + su * G * kHd);
#pragma unroll
            for (int f = lane; f < G * 32; f += kWave) dst[f] = stage_acc[r][f];
            if (part && lane < G) a.ws_ml[sslot * G + lane] = stage_ml[r][lane];
            if (rcount != 0 && lane == 0) a.ws_rec[su] = make_int2((int)sslot, rcount);
        }
        nstage = 0;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    auto finish_unit = [&](bool unit_end) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                acc[h][e] = sum_xor32(sum_xor16(acc[h][e]));
            }
        float lsum[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) lsum[r] = row_sum16(l[r]);
        const int64_t u = (int64_t)ui * Hkv + ug;
        const int64_t slot = u + w;
        const bool whole = from_start && unit_end && !(START && ustart != 0);
        if (nstage == kStage) flush();
        const int r = nstage;
        if (whole) {  // normalise in place (the accumulator is reset at the next unit)
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float inv = bad ? NAN : 1.f / read_lane(lsum[h & 3], 16 * (h >> 2));
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] *= inv;
            }
        }
        if (lane < 16) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                stage_acc[r][h * 32 + 2 * lane] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
                stage_acc[r][h * 32 + 2 * lane + 1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
            }
        }
        int rcount = whole ? 1 : 0;
        if (!whole) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float lh = read_lane(lsum[h & 3], 16 * (h >> 2));
                const float mh = read_lane(m[h & 3], 16 * (h >> 2));
                if (lane == h) stage_ml[r][h] = make_float2(mh, bad ? NAN : lh);
            }
            if (from_start) {
                const int64_t last_tile = (int64_t)useq_base + (int64_t)ug * un + un - 1;
                const int64_t w_last = sp.wave_of(last_tile);
                rcount = (int)(w_last - w + 1);
            }
        }
        if (lane == 0) stage_meta[r] = make_int4(whole ? 0 : 1, (int)u, (int)slot, rcount);
        nstage = r + 1;
    };

    for (int64_t seg0 = c0; seg0 < c1;) {
        issue_first(P, X0);  // the cursor is at the segment's first tile
        __builtin_amdgcn_sched_barrier(0);
        // ---- segment set-up: walk up to kSegRuns runs (pieces of units) and
        // kSegTiles tiles, then request every block-table entry and q row of
        // the segment at once and park them in LDS.
        const int room = (int)min((int64_t)kSegTiles, c1 - seg0);
        int nruns = 0, k = 0;
        while (k < room && nruns < kSegRuns) {  // wave-uniform walk
            const int len = min(P.n - P.b, room - k);
            if (lane == 0) {
                run_lds[nruns][0] = make_int4(P.i, P.g, P.n, P.b);
                run_lds[nruns][1] = make_int4((int)P.seq_base, P.start, k, P.ctx);
            }
            k += len;
            ++nruns;
            P.b += len;
            if (P.b == P.n && seg0 + k < c1) {  // next unit (more tiles follow)
                P.b = 0;
                if (++P.g == Hkv) {
                    P.g = 0;
                    P.seq_base += (int64_t)Hkv * P.n;
                    do {
                        ++P.i;
                        P.ctx = len_of(P.i);
                        P.start = start_of(P.i);
                        P.n = tiles_at(P.ctx, P.start);
                    } while (P.n == 0);
                }
            }
        }
        const int seg_len = k;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // q rows: run r's G rows are G * 256 contiguous bytes of q; lane l moves
        // bytes [16 l, 16 l + 16) of every 1 KiB piece.
        uint4 qv[kSegRuns][kQv];
#pragma unroll
        for (int r = 0; r < kSegRuns; ++r) {
            if (r < nruns) {
                const int4 d = run_lds[r][0];
                const uint4* qsrc = reinterpret_cast<const uint4*>(
                    qbase + ((int64_t)d.x * Hq + (int64_t)d.y * G) * kHd);
#pragma unroll
                for (int v = 0; v < kQv; ++v) {
                    const int idx = v * kWave + lane;
                    qv[r][v] = idx < G * kHd / 8 ? qsrc[idx] : make_uint4(0, 0, 0, 0);
                }
            }
        }
        // tile records: lane j covers tiles j and j + 64 of the segment
        int phys[2], phys2[2], trun[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int j = lane + kWave * half;
            int r = 0;
            for (int q = 1; q < nruns; ++q)
                if (j >= run_lds[q][1].z) r = q;
            trun[half] = r;
            const int4 d = run_lds[r][0];
            const int4 e = run_lds[r][1];
            const int b = d.w + (j - e.z);
            const int tok0 = e.y + b * kTok;
            phys[half] = j < seg_len ? bt[(int64_t)d.x * maxB + tok0 / BS] : 0;
            // The second block of a split tile is looked up only when its half
            // of the tile holds tokens (the entry past them may be unused).
            phys2[half] = (kSplit && j < seg_len && tok0 + BS < e.w) ? bt[(int64_t)d.x * maxB + tok0 / BS + 1] : 0;
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int j = lane + kWave * half;
            if (j < seg_len) {
                const int r = trun[half];
                const int4 d = run_lds[r][0];
                const int4 e = run_lds[r][1];
                const int b = d.w + (j - e.z);
                const int tok0 = e.y + b * kTok;
                bool badp = (unsigned)phys[half] >= (unsigned)a.num_blocks;
                const int ph = badp ? 0 : phys[half];
                const int64_t off = (((int64_t)ph * Hkv + d.y) * BS + (tok0 % BS)) * kHd;
                // Split tile: (second block * Hkv + KV head) of rows 8..15; the
                // first block again when that half holds no tokens, so that its
                // (masked) key rows are still read from inside the pool.
                uint32_t second = 0u;
                if constexpr (kSplit) {
                    int ph2 = ph;
                    if (tok0 + BS < e.w) {
                        const bool bad2 = (unsigned)phys2[half] >= (unsigned)a.num_blocks;
                        badp = badp || bad2;
                        ph2 = bad2 ? 0 : phys2[half];
                    }
                    second = (uint32_t)((int64_t)ph2 * Hkv + d.y);
                }
                const uint32_t flags = (uint32_t)min(kTok, e.w - tok0) | ((uint32_t)r << 8) |
                                       (b == 0 ? kFirst : 0u) | (b == d.z - 1 ? kLast : 0u) | (badp ? kBad : 0u);
                rec_lds[j] = make_uint4((uint32_t)off, (uint32_t)((uint64_t)off >> 32), flags, second);
            }
        }
#pragma unroll
        for (int r = 0; r < kSegRuns; ++r)
            if (r < nruns)
#pragma unroll
                for (int v = 0; v < kQv; ++v) q_lds[r][v * kWave + lane] = qv[r][v];
        // Every load of the set-up (and the first tile's, issued before it)
        // is complete here, on every path into the tile loop, so the loop's
        // waits count only its own tiles.
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- the segment's tiles
        // Issue the K and V loads of segment tile kk.  The tile's base address
        // is wave-uniform: it goes to scalar registers, the loads take 32-bit
        // lane offsets.
        auto issue = [&](int kk, TileLoad& T) { issue_rec(rec_lds[kk], T); };

        // Entering a tile: at a unit's first tile (or the chunk's first) take
        // the unit's q from LDS and reset the running state.
        auto begin = [&](int64_t t, const TileLoad& T) {
            if (t == c0 || (T.flags & kFirst)) {
                const int r = (int)((T.flags >> 8) & 0xffu);
                const int4 r0 = run_lds[r][0];
                const int4 r1 = run_lds[r][1];
                ui = __builtin_amdgcn_readfirstlane(r0.x);
                ug = __builtin_amdgcn_readfirstlane(r0.y);
                un = __builtin_amdgcn_readfirstlane(r0.z);
                useq_base = __builtin_amdgcn_readfirstlane(r1.x);
                ustart = __builtin_amdgcn_readfirstlane(r1.y);
                const uint16_t* qrow = reinterpret_cast<const uint16_t*>(&q_lds[r][0]);
#pragma unroll
                for (int kq = 0; kq < 4; ++kq) {
                    const uint4 v = *reinterpret_cast<const uint4*>(qrow + (r16 < G ? r16 : 0) * kHd + kq * 32 + grp * 8);
                    qc[kq] = r16 < G ? v : make_uint4(0, 0, 0, 0);
                }
#pragma unroll
                for (int h = 0; h < G; ++h)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
#pragma unroll
                for (int r2 = 0; r2 < 4; ++r2) {
                    m[r2] = -INFINITY;
                    l[r2] = 0.f;
                }
                bad = false;
                from_start = (T.flags & kFirst) != 0;
            }
        };

        // One tile: scores by MFMA, online softmax, P.V into the accumulator.
        auto step = [&](int64_t t, const TileLoad& T) {
            bad = bad || (T.flags & kBad);
            f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kq = 0; kq < 4; ++kq)
                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qc[kq]), as_bf16x8(T.k[kq]), sc, 0, 0, 0);

            const bool tok_ok = r16 < (int)(T.flags & 0xffu);
            float s[4];
            bool need = false;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                s[r] = tok_ok ? sc[r] * qscale : -INFINITY;
                need = need || (s[r] > m[r] + kLazyRescale);
            }
            // The running max moves only when some score passes it by more
            // than the threshold (always on a unit's first tile, rarely
            // after); only then is the tile max reduced along the row and the
            // state rescaled.
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
            // The weights move from the score layout to the P.V layout through
            // LDS.  One wave per workgroup: LDS operations of a wave complete
            // in order, the fences only keep the compiler from moving them.
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

            const bool unit_end = (T.flags & kLast) != 0;
            if (unit_end || t + 1 == c1) finish_unit(unit_end);
        };

        // Two tile buffers: while tile kk is computed, the loads of tile kk + 1
        // are in flight.  (A third buffer, two tiles ahead, measured no faster:
        // the chip's read queues are already full with one tile ahead per
        // wave.)  Every phase issues exactly one tile's loads (past the end of
        // the segment it requests its last tile again, which the cache holds),
        // so all paths issue the same loads in the same order and each wait
        // counts exactly the loads it needs.  The scheduling barriers keep
        // every tile's loads in issue order: if the compiler interleaves the
        // loads of two tiles, the wait counts it derives at the loop head have
        // to cover both, and the pipeline drains.
        auto phase = [&](int kk, TileLoad& cur, TileLoad& ahead) {
            if (kk < seg_len) begin(seg0 + kk, cur);
            __builtin_amdgcn_sched_barrier(0);
            issue(min(kk + 1, seg_len - 1), ahead);
            __builtin_amdgcn_sched_barrier(0);
            if (kk < seg_len) step(seg0 + kk, cur);
        };
        for (int kk = 0; kk < seg_len; kk += 2) {
            phase(kk, X0, X1);
            phase(kk + 1, X1, X0);
        }
        seg0 += seg_len;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
    flush();
}

// Merge kernel: one workgroup per (sequence, KV head) unit, one wave per query
// head of the group.  Units the partition kernel finished (one partial) are
// left alone; otherwise head h gets M = max_p m_p, L = sum_p 2^(m_p - M) l_p
// and out = sum_p 2^(m_p - M) acc_p / L over the unit's partials in slot
// order.  Sequences without tiles get zero rows (empty) or NaN rows (length
// outside the table).  Lanes own two output columns each.
// PREFIX: the unit also has the chunk partials of its group's shared prefix
// (tokens [0, seq_start[i]), from decode_prefix_kernel); they come first in
// the merge order, then the unit's own partials, and the partition kernel
// finished none of these units itself.
template <int G, bool PREFIX>
__global__ __launch_bounds__(64 * G) void merge_fast_kernel(const DecodeArgs a, int table_tokens) {
    constexpr int kFew = 8;  // partial counts handled with all loads in one round
    const int lane = threadIdx.x & (kWave - 1);
    const int h = threadIdx.x / kWave;
    const int64_t u = blockIdx.x;
    const int i = (int)(u / a.num_kv_heads);
    const int g = (int)(u % a.num_kv_heads);
    // The record is read together with the length (it is garbage, and unused,
    // when the sequence has no tiles here).
    const int ctx = a.context_lens[i];
    const int st = PREFIX ? a.seq_start[i] : 0;
    const int2 rec = a.ws_rec[u];
    float2* out = reinterpret_cast<float2*>(
        a.out + ((int64_t)i * a.num_q_heads + (int64_t)g * G + h) * kHd + 2 * lane);
    const bool valid = st >= 0 && st <= ctx && ctx <= table_tokens && (st & (kTok - 1)) == 0;
    const int ns = PREFIX ? tiles_from(ctx, st, table_tokens) : tiles_of(ctx, table_tokens);
    const int npc = (PREFIX && st > 0) ? (st / kTok + a.prefix_chunk_tiles - 1) / a.prefix_chunk_tiles : 0;
    if (!valid || npc > (PREFIX ? a.prefix_max_chunks : 0)) {
        *out = make_float2(NAN, NAN);
        return;
    }
    if (ns == 0 && npc == 0) {  // empty sequence
        *out = make_float2(0.f, 0.f);
        return;
    }
    const int nps = ns > 0 ? rec.y : 0;
    if (npc == 0 && nps == 1) return;  // finished by the partition kernel
    const int64_t slots = (int64_t)a.num_seqs * a.num_kv_heads + kMaxGridWaves;
    if (ns > 0 && (nps < 1 || rec.x < 0 || (int64_t)rec.x + nps > slots)) {  // never written: refuse to read
        *out = make_float2(NAN, NAN);
        return;
    }
    const int np = npc + nps;
    const int64_t prow = u * (PREFIX ? a.prefix_max_chunks : 0);
    // Partial p: prefix chunk p, then the unit's slots in order.
    auto ml_of = [&](int p) -> float2 {
        if (PREFIX && p < npc) return a.ws_pml[(prow + p) * G + h];
        return a.ws_ml[((int64_t)rec.x + p - npc) * G + h];
    };
    auto acc_of = [&](int p) -> float2 {
        const float* base = (PREFIX && p < npc) ? a.ws_pacc + ((prow + p) * G + h) * kHd
                                                : a.ws_acc + (((int64_t)rec.x + p - npc) * G + h) * kHd;
        return *reinterpret_cast<const float2*>(base + 2 * lane);
    };
    if (np <= kFew) {
        // lane p < np holds partial p's (m, l); every lane loads its two
        // columns of all partials at once.
        const float2 mlv = lane < np ? ml_of(lane) : make_float2(-INFINITY, 0.f);
        float2 v[kFew];
#pragma unroll
        for (int p = 0; p < kFew; ++p) v[p] = p < np ? acc_of(p) : make_float2(0.f, 0.f);
        const float M = wave_max(mlv.x);
        const float wgt = lane < np ? exp2f(mlv.x - M) : 0.f;
        const float L = wave_sum(wgt * mlv.y);
        float o0 = 0.f, o1 = 0.f;
#pragma unroll
        for (int p = 0; p < kFew; ++p) {
            const float wp = read_lane(wgt, p);
            o0 = fmaf(wp, v[p].x, o0);
            o1 = fmaf(wp, v[p].y, o1);
        }
        *out = make_float2(o0 / L, o1 / L);
        return;
    }
    float M = -INFINITY;
    for (int p = lane; p < np; p += kWave) M = fmaxf(M, ml_of(p).x);
    M = wave_max(M);
    float L = 0.f;
    for (int p = lane; p < np; p += kWave) {
        const float2 v = ml_of(p);
        L += exp2f(v.x - M) * v.y;
    }
    L = wave_sum(L);
    float o0 = 0.f, o1 = 0.f;
    int p = 0;
    for (; p + 4 <= np; p += 4) {  // four partials' loads in flight at once
        float2 v[4], mlv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[k] = acc_of(p + k);
            mlv[k] = ml_of(p + k);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float wgt = exp2f(mlv[k].x - M);
            o0 = fmaf(wgt, v[k].x, o0);
            o1 = fmaf(wgt, v[k].y, o1);
        }
    }
    for (; p < np; ++p) {
        const float2 v = acc_of(p);
        const float wgt = exp2f(ml_of(p).x - M);
        o0 = fmaf(wgt, v.x, o0);
        o1 = fmaf(wgt, v.y, o1);
    }
    *out = make_float2(o0 / L, o1 / L);
}

// Shared-prefix chunk partials.  Workgroup (group k, KV head g, chunk c) has
// four waves.  The group's prefix, tokens [0, P) named by the first member's
// block table, is read once per workgroup: every 16-token tile of the chunk is
// loaded into LDS by all 256 threads (kPrefixAhead tiles in flight), K as
// stored and V transposed (dims x tokens).  The group's query rows -- member
// m's heads g*G .. g*G+G-1 as rows m*G .. m*G+G-1, at most 64 -- are dealt 16
// per wave, so the matrix cores see no padding unless the group is small:
//   * S^T = K Q^T by four v_mfma_f32_16x16x32_bf16 (A = the 16 key rows, B =
//     the wave's 16 query rows), which leaves lane l the scores of row l % 16
//     for tokens 4 (l / 16) .. + 3;
//   * online softmax per row in log2 units (lazy max as in decode_fast_kernel;
//     the row's four lane groups agree on its max);
//   * P V by v_mfma_f32_16x16x16bf16_1k: the scores' layout is already the A
//     operand; P is split into a bf16 high part and a bf16 remainder (two
//     MFMAs each), so every product is exact and the sums are fp32; B = V^T
//     from LDS; the accumulator holds 16 rows x 128 dims in 32 registers.
// Each row's (m, l, acc) for chunk c goes to its member's partial slot.
constexpr int kPrefixWaves = 4;
constexpr int kPrefixThreads = kPrefixWaves * 64;
constexpr int kPrefixAhead = 6;           // tiles in flight per workgroup
constexpr int kPrefixChunkTilesMax = 64;  // LDS table size
constexpr int kMultiChunkTilesMax = 128;  // LDS table size of the multi-query chunk kernel
constexpr int kKRow = kHd * 2 + 16;       // padded LDS row of a K tile (bytes): conflict-free fragment reads
// LDS row of the transposed V tile: one dim, 16 tokens (32 bytes), padded to
// 40 bytes.  Rows 10 banks apart put the 16 rows that one P.V operand read
// touches on 16 different bank pairs (conflict-free), and the tile's writes --
// each lane its own dim row -- at most two to a bank; unpadded 32-byte rows
// measured 75% of LDS cycles in bank conflicts.
constexpr int kVtRow = kTok * 2 + 8;
// Byte offset of chunk c (tokens 4c .. 4c + 3) of transposed-V row (dim) d.
// In rows 16 .. 31 of every 32 the chunks are swapped pairwise: the lanes that
// write rows 2 vj and 2 vj + 16 then fall on different banks, while the 16
// rows one operand read covers all share the swap, so that read stays
// conflict-free.
__device__ __forceinline__ int vt_off(int d, int c) { return d * kVtRow + 8 * (c ^ ((d >> 4) & 1)); }
static_assert(kPrefixGroupMax * 8 <= 16 * kPrefixWaves, "rows of a full group at G = 8 fit the waves");

typedef short s16x4 __attribute__((ext_vector_type(4)));


template <int BS, int G>
__global__ __launch_bounds__(kPrefixThreads) void decode_prefix_kernel(const DecodeArgs a, float qscale) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wv = tid / kWave;
    const int k = blockIdx.x, g = blockIdx.y, c = blockIdx.z;
    const int S = a.num_seqs, Hkv = a.num_kv_heads, Hq = a.num_q_heads;
    const int maxB = a.max_blocks_per_seq;
    const int table_tokens = maxB * BS;
    const int CT = a.prefix_chunk_tiles;

    const int first = a.groups[2 * k];
    const int count = a.groups[2 * k + 1];
    if (first < 0 || count < 1 || count > kPrefixGroupMax || first > S - count) return;  // uniform
    const int P = a.seq_start[first];
    const bool p_ok = P > 0 && P % BS == 0 && P <= table_tokens;
    const int nt_total = p_ok ? P / kTok : 0;
    const int t0 = c * CT;
    const int t1 = min(t0 + CT, nt_total);
    const int ntile = max(t1 - t0, 0);
    const int rows = count * G;
    // Row groups of 16; a group with fewer than four gives each row group
    // D = 4 / (row groups) waves, which split its 128 dims (every wave works).
    const int nrg = (rows + 15) / 16;
    const int D = nrg == 1 ? 4 : nrg == 2 ? 2 : 1;
    const int rg = wv / D, dq = wv % D;
    const bool computes = rg < nrg;  // wave-uniform

    __shared__ uint2 toff_lds[kPrefixChunkTilesMax];  // element offset of each tile (lo, hi)
    __shared__ int tbad_lds[kPrefixChunkTilesMax];
    __shared__ __attribute__((aligned(16))) unsigned char k_lds[2][kTok * kKRow];
    __shared__ __attribute__((aligned(16))) unsigned char vt_lds[2][kHd * kVtRow];

    const int32_t* __restrict__ bt = a.block_tables;
    if (tid < ntile) {
        const int tok0 = (t0 + tid) * kTok;
        const int phys = bt[(int64_t)first * maxB + tok0 / BS];
        const bool badp = (unsigned)phys >= (unsigned)a.num_blocks;
        const int64_t off = (((int64_t)(badp ? 0 : phys) * Hkv + g) * BS + tok0 % BS) * kHd;
        toff_lds[tid] = make_uint2((uint32_t)off, (uint32_t)((uint64_t)off >> 32));
        tbad_lds[tid] = badp;
    }
    // The wave's query rows as the B operand of S^T = K Q^T (rows past the group are zero).
    const int r16 = lane & 15;
    const int grp = lane >> 4;
    uint4 qc[4];
    {
        const int r = 16 * rg + r16;
        const bool real = r < rows;
        const int mi = first + (real ? r / G : 0);
        const uint16_t* qrow =
            static_cast<const uint16_t*>(a.q) + ((int64_t)mi * Hq + (int64_t)g * G + (real ? r % G : 0)) * kHd;
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) {
            const uint4 v = *reinterpret_cast<const uint4*>(qrow + kq * 32 + grp * 8);
            qc[kq] = real ? v : make_uint4(0, 0, 0, 0);
        }
    }
    __syncthreads();

    // Thread tid takes dims 2j, 2j+1 (j = tid % 64) of tokens 4 (tid / 64) .. + 3
    // of both K and V: eight 4-byte loads, each 256 contiguous bytes per wave.
    // Every thread issues the same loads, so the waits for the tiles
    // kPrefixAhead ahead stay exact.  K is stored as it is (padded rows), V
    // transposed.
    const uint32_t* __restrict__ k32 = static_cast<const uint32_t*>(a.k_cache);
    const uint32_t* __restrict__ v32 = static_cast<const uint32_t*>(a.v_cache);
    const int vtg = tid >> 6, vj = tid & 63;
    struct TileKV {
        uint4 k, v;
    };
    auto load_tile = [&](int j) -> TileKV {
        const uint2 o = toff_lds[j];
        const int64_t off = (int64_t)(((uint64_t)o.y << 32) | o.x) / 2 + (int64_t)(4 * vtg) * (kHd / 2) + vj;
        TileKV t;
        t.k = make_uint4(k32[off], k32[off + kHd / 2], k32[off + 2 * (kHd / 2)], k32[off + 3 * (kHd / 2)]);
        t.v = make_uint4(v32[off], v32[off + kHd / 2], v32[off + 2 * (kHd / 2)], v32[off + 3 * (kHd / 2)]);
        return t;
    };
    auto store_tile = [&](int buf, const TileKV& t) {
        unsigned char* kb = &k_lds[buf][(4 * vtg) * kKRow + 4 * vj];
        *reinterpret_cast<uint32_t*>(kb) = t.k.x;
        *reinterpret_cast<uint32_t*>(kb + kKRow) = t.k.y;
        *reinterpret_cast<uint32_t*>(kb + 2 * kKRow) = t.k.z;
        *reinterpret_cast<uint32_t*>(kb + 3 * kKRow) = t.k.w;
        const uint4 v = t.v;
        const uint2 even = make_uint2((v.x & 0xffffu) | (v.y << 16), (v.z & 0xffffu) | (v.w << 16));
        const uint2 odd = make_uint2((v.x >> 16) | (v.y & 0xffff0000u), (v.z >> 16) | (v.w & 0xffff0000u));
        *reinterpret_cast<uint2*>(&vt_lds[buf][vt_off(2 * vj, vtg)]) = even;
        *reinterpret_cast<uint2*>(&vt_lds[buf][vt_off(2 * vj + 1, vtg)]) = odd;
    };

    auto run = [&](auto d_tag) {
    constexpr int JB = (kHd / 16) / decltype(d_tag)::value;  // 16-dim blocks of this wave: dims 16 (jb0 + jj) + r16
    const int jb0 = dq * JB;
    f32x4 acc[JB];  // rows 4 grp .. + 3 of the wave's row group
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) acc[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY;  // running max of row r16 (the same in its four lane groups)
    float l = 0.f;        // this lane's part of row r16's softmax denominator
    bool bad = false;     // a block-table entry outside the pool

    auto step = [&](int buf, int j) {
        bad = bad || tbad_lds[j] != 0;
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) {
            const uint4 kf = *reinterpret_cast<const uint4*>(&k_lds[buf][r16 * kKRow + kq * 64 + grp * 16]);
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf), as_bf16x8(qc[kq]), sc, 0, 0, 0);
        }
        float s[4];
        bool need = false;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            s[r] = sc[r] * qscale;
            need = need || (s[r] > m + kLazyRescale);
        }
        if (__any(need)) {
            float tm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
            tm = max_xor32(max_xor16(tm));
            const float mn = tm > m + kLazyRescale ? tm : m;
            const float alpha = fast_exp2(m - mn);
            m = mn;
            l *= alpha;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ar = __shfl(alpha, 4 * grp + r, kWave);
#pragma unroll
                for (int jj = 0; jj < JB; ++jj) acc[jj][r] *= ar;
            }
        }
        s16x4 phi, plo;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float pr = fast_exp2(s[r] - m);
            l += pr;
            const uint32_t hb = __float_as_uint(pr) & 0xffff0000u;
            phi[r] = (short)(hb >> 16);
            plo[r] = (short)(__float_as_uint(pr - __uint_as_float(hb)) >> 16);
        }
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
            const uint2 vb = *reinterpret_cast<const uint2*>(&vt_lds[buf][vt_off(16 * (jb0 + jj) + r16, grp)]);
            const s16x4 vv = __builtin_bit_cast(s16x4, vb);
            acc[jj] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, vv, acc[jj], 0, 0, 0);
            acc[jj] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, vv, acc[jj], 0, 0, 0);
        }
    };

    // Loads past the last tile fetch the last tile again (unused), so every
    // iteration issues the same loads.
    TileKV R[kPrefixAhead];
    if (ntile > 0) {
#pragma unroll
        for (int q = 0; q < kPrefixAhead; ++q) R[q] = load_tile(min(q, ntile - 1));
    }
    // Full groups of kPrefixAhead tiles (no branch around the loads), then the
    // remaining tiles, whose loads were issued by the last group.
    int j0 = 0;
    for (; j0 + kPrefixAhead <= ntile; j0 += kPrefixAhead) {
#pragma unroll
        for (int q = 0; q < kPrefixAhead; ++q) {
            const int j = j0 + q;
            store_tile(j & 1, R[q]);
            R[q] = load_tile(min(j + kPrefixAhead, ntile - 1));
            __syncthreads();
            if (computes) step(j & 1, j);
        }
    }
#pragma unroll
    for (int q = 0; q < kPrefixAhead - 1; ++q) {
        const int j = j0 + q;
        if (j < ntile) {  // uniform
            store_tile(j & 1, R[q]);
            __syncthreads();
            if (computes) step(j & 1, j);
        }
    }

    if (!computes) return;
    const float lt = sum_xor32(sum_xor16(l));
    // Row r of the wave is member r / G, head r % G.  A member writes chunk c
    // when its own prefix has that chunk; its rows are NaN when its prefix
    // disagrees with the group's or does not fit its sequence.
    auto row_state = [&](int r, int64_t& prow, bool& rbad) -> bool {
        if (r >= rows) return false;
        const int mi = first + r / G;
        const int st = a.seq_start[mi];
        const int npc = st > 0 ? (st / kTok + CT - 1) / CT : 0;
        if (c >= npc) return false;
        const int ctx = a.context_lens[mi];
        rbad = bad || !(p_ok && st == P && ctx >= P && ctx <= table_tokens);
        prow = ((int64_t)mi * Hkv + g) * a.prefix_max_chunks + c;
        return true;
    };
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const int r = 16 * rg + 4 * grp + rr;
        int64_t prow;
        bool rbad;
        if (row_state(r, prow, rbad)) {
#pragma unroll
            for (int jj = 0; jj < JB; ++jj) a.ws_pacc[(prow * G + r % G) * kHd + 16 * (jb0 + jj) + r16] = acc[jj][rr];
        }
    }
    if (lane < 16 && dq == 0) {
        const int r = 16 * rg + lane;
        int64_t prow;
        bool rbad;
        if (row_state(r, prow, rbad)) a.ws_pml[prow * G + r % G] = make_float2(m, rbad ? NAN : lt);
    }
    };
    if (D == 4)
        run(std::integral_constant<int, 4>{});
    else if (D == 2)
        run(std::integral_constant<int, 2>{});
    else
        run(std::integral_constant<int, 1>{});
}

// Several new tokens per sequence, causal.  Workgroup (sequence i, KV head g
// and block of 16 * NRG query rows, chunk c of the sequence's tiles) has the
// tile pipeline of decode_prefix_kernel: each 16-token tile of the chunk is
// read once into LDS, by all of the workgroup's threads, for all of its rows.
// The rows are dealt in groups of 16: one group per wave when NRG is 1 or 4,
// two per wave when NRG is 16 (8 waves), so that each K and V fragment read
// from LDS feeds two matrix products.  NRG is 1 when a sequence's rows fit one
// group (speculative decoding: no wave only loads, and the small workgroups
// all fit on the chip at once), else 4 or 16 (up to 256 rows per tile read).
// Tiles are computed in pairs, so that P.V runs on the 32-deep matrix
// instruction (v_mfma_f32_16x16x32_bf16: twice the work of the 16-deep one in
// the same cycles); an odd last tile is paired with a masked one.  Row r of a
// block is new token r / G (position ctx - q_len + r / G) and head r % G; a
// row sees the tokens up to its own position (the others are masked in the
// scores).  Each row leaves the chunk's (m, l, acc) for multi_merge_kernel.
template <int NRG>
struct MultiShape {
    static constexpr int RG = NRG == 16 ? 2 : 1;  // row groups per wave
    static constexpr int MW = NRG / RG;           // waves per workgroup
};

// The end of a chunk workgroup of the multi-query kernels.  Without MERGED each
// row leaves the chunk's (m, l, acc) in its partial slot for multi_merge_kernel.
// With MERGED the last workgroup of a (sequence, KV head, row block) to finish
// its chunk merges all of the unit's chunks (arrival counters in the
// workspace's counter region, zero between calls) and writes the output rows.
template <int G, int RG, bool MERGED>
__device__ __forceinline__ void multi_finish(const DecodeArgs& a, const f32x4 (&acc)[RG][kHd / 16], const float (&m)[RG],
                                             const float (&l)[RG], bool bad, bool computes, int i, int g, int rb, int c,
                                             int q0, int rows, int wrow0, int nt_total, int tid) {
    const int lane = tid & (kWave - 1);
    const int r16 = lane & 15;
    const int grp = lane >> 4;
    const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
    const int rbs = a.multi_row_blocks;
    const int CT = a.prefix_chunk_tiles;
    const int MC = a.prefix_max_chunks;
    const int nch = (nt_total + CT - 1) / CT;  // chunks of this sequence
    float lt[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) lt[rg] = computes ? sum_xor32(sum_xor16(l[rg])) : 0.f;
    // Partial slot of row r (new token r / G, head r % G) for chunk cc.
    auto prow_of = [&](int r, int cc) -> int64_t { return ((int64_t)(q0 + r / G) * Hq + (int64_t)g * G + r % G) * MC + cc; };
    if constexpr (!MERGED) {
        if (!computes) return;
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int r = wrow0 + 16 * rg + 4 * grp + rr;
                if (r < rows) {
                    const int64_t pr = prow_of(r, c);
#pragma unroll
                    for (int jb = 0; jb < kHd / 16; ++jb) a.ws_pacc[pr * kHd + 16 * jb + r16] = acc[rg][jb][rr];
                }
            }
            const int row = wrow0 + 16 * rg + lane;
            if (lane < 16 && row < rows) a.ws_pml[prow_of(row, c)] = make_float2(m[rg], bad ? NAN : lt[rg]);
        }
        return;
    } else {
        // Rows of the acc layout (rows 4 grp + rr of each group) take the softmax state of
        // the lane that holds their scores (lane 4 grp + rr).
        float mr[RG][4], lr[RG][4];
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                mr[rg][rr] = __shfl(m[rg], 4 * grp + rr, kWave);
                lr[rg][rr] = bad ? NAN : __shfl(lt[rg], 4 * grp + rr, kWave);
            }
        __shared__ int last_lds;
        if (nch > 1) {
            // Store this chunk's partial past the L2s (another workgroup, maybe on another
            // XCD, may merge it), make it complete, then count the arrival.
            if (computes) {
#pragma unroll
                for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int r = wrow0 + 16 * rg + 4 * grp + rr;
                        if (r < rows) {
                            const int64_t pr = prow_of(r, c);
#pragma unroll
                            for (int jb = 0; jb < kHd / 16; ++jb)
                                __hip_atomic_store(&a.ws_pacc[pr * kHd + 16 * jb + r16], acc[rg][jb][rr], __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
                        }
                    }
                    const int row = wrow0 + 16 * rg + lane;
                    if (lane < 16 && row < rows) {
                        const float2 v = make_float2(m[rg], bad ? NAN : lt[rg]);
                        __hip_atomic_store(reinterpret_cast<uint64_t*>(a.ws_pml) + prow_of(row, c),
                                           __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (tid == 0) {
                const int64_t unit = ((int64_t)i * Hkv + g) * rbs + rb;
                const uint32_t old = __builtin_amdgcn_atomic_inc32(a.ws_cnt + unit, (uint32_t)(nch - 1), __ATOMIC_RELAXED, "agent");
                last_lds = old == (uint32_t)(nch - 1);
            }
            __syncthreads();
            if (!last_lds) return;  // uniform: a later workgroup merges
        }
        if (!computes) return;
        // The last workgroup (or the only chunk): out = sum_c 2^(m_c - M) acc_c / sum_c
        // 2^(m_c - M) l_c over the chunks in order, its own from registers.  Chunks a
        // row cannot see carry m = -inf and weigh nothing.  The loads of one chunk for
        // all of the lane's rows are issued together.
        int64_t prw[RG][4];
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int r = wrow0 + 16 * rg + 4 * grp + rr;
                prw[rg][rr] = prow_of(r < rows ? r : wrow0, 0);
            }
        const uint64_t* ml64 = reinterpret_cast<const uint64_t*>(a.ws_pml);
        float M[RG][4];
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) M[rg][rr] = mr[rg][rr];
        for (int cc = 0; cc < nch; ++cc) {
            if (cc == c) continue;  // uniform
            float mc[RG][4];
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) mc[rg][rr] = __uint_as_float((uint32_t)load_agent(ml64 + prw[rg][rr] + cc));
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) M[rg][rr] = fmaxf(M[rg][rr], mc[rg][rr]);
        }
        // one row group at a time (fewer live registers), the chunks in order
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            float L[4], o[4][kHd / 16];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                L[rr] = 0.f;
#pragma unroll
                for (int jb = 0; jb < kHd / 16; ++jb) o[rr][jb] = 0.f;
            }
            for (int cc = 0; cc < nch; ++cc) {
                const bool own = cc == c;  // uniform
                float mc[4], lc[4], v[4][kHd / 16];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    if (own) {
                        mc[rr] = mr[rg][rr];
                        lc[rr] = lr[rg][rr];
#pragma unroll
                        for (int jb = 0; jb < kHd / 16; ++jb) v[rr][jb] = acc[rg][jb][rr];
                    } else {
                        const int64_t pr = prw[rg][rr] + cc;
                        const uint64_t mlv = load_agent(ml64 + pr);
                        mc[rr] = __uint_as_float((uint32_t)mlv);
                        lc[rr] = __uint_as_float((uint32_t)(mlv >> 32));
#pragma unroll
                        for (int jb = 0; jb < kHd / 16; ++jb)
                            v[rr][jb] = __hip_atomic_load(&a.ws_pacc[pr * kHd + 16 * jb + r16], __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    if (mc[rr] == -INFINITY) continue;
                    const float wgt = exp2f(mc[rr] - M[rg][rr]);
                    L[rr] = fmaf(wgt, lc[rr], L[rr]);
#pragma unroll
                    for (int jb = 0; jb < kHd / 16; ++jb) o[rr][jb] = fmaf(wgt, v[rr][jb], o[rr][jb]);
                }
            }
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int r = wrow0 + 16 * rg + 4 * grp + rr;
                if (r < rows) {
                    float* orow = a.out + ((int64_t)(q0 + r / G) * Hq + (int64_t)g * G + r % G) * kHd;
#pragma unroll
                    for (int jb = 0; jb < kHd / 16; ++jb) orow[16 * jb + r16] = o[rr][jb] / L[rr];
                }
            }
        }
    }
}

// MERGED: the last workgroup of a (sequence, KV head, row block) to finish its
// chunk merges all of the unit's chunks (arrival counters in the workspace's
// counter region, zero between calls) and writes the output rows; without it
// multi_merge_kernel merges the chunk partials.
template <int BS, int G, int NRG, bool MERGED>
__global__ __launch_bounds__(64 * MultiShape<NRG>::MW) __attribute__((amdgpu_waves_per_eu(NRG == 1 ? 1 : 2))) void multi_query_kernel(
    const DecodeArgs a, float qscale) {
    constexpr int RG = MultiShape<NRG>::RG;
    constexpr int MW = MultiShape<NRG>::MW;
    constexpr int T = 64 * MW;        // threads
    constexpr int TPI = 1024 / T;     // tokens of one dword column each thread moves per tile
    constexpr int kAhead = MW == 1 ? 2 : 4;  // tiles in flight, whole pairs (32 / 8 / 4 load registers per tile)
    static_assert(NRG == 1 || NRG == 4 || NRG == 16, "row groups per workgroup");
    static_assert(kAhead % 2 == 0, "tiles are loaded and computed in pairs");
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wv = tid / kWave;
    const int i = blockIdx.x;
    const int rbs = a.multi_row_blocks;
    const int g = blockIdx.y / rbs, rb = blockIdx.y % rbs;
    const int c = blockIdx.z;
    const int Hkv = a.num_kv_heads, Hq = a.num_q_heads;
    const int maxB = a.max_blocks_per_seq;
    const int table_tokens = maxB * BS;
    const int CT = a.prefix_chunk_tiles;

    const int q0 = a.cu_q[i], q1 = a.cu_q[i + 1];
    const int ql = q1 - q0;
    const int ctx = a.context_lens[i];
    // Sequences without rows to write, sequences whose rows are NaN (written by
    // chunk 0 here when merging in-kernel, else by the merge kernel), and blocks
    // with no rows or tiles (uniform).
    if (q0 < 0 || q1 > a.total_q || ql < 1) return;
    if (ql > a.max_q_len || ctx < ql || ctx > table_tokens) {
        if (MERGED && c == 0) {
            const int nrow = min(ql, a.max_q_len) * G;
            for (int r = 16 * NRG * rb; r < min(nrow, 16 * NRG * (rb + 1)); ++r) {
                float* o = a.out + ((int64_t)(q0 + r / G) * Hq + (int64_t)g * G + r % G) * kHd;
                for (int x = tid; x < kHd; x += 64 * MultiShape<NRG>::MW) o[x] = NAN;
            }
        }
        return;
    }
    const int rows = ql * G;
    const int row0 = 16 * NRG * rb;  // first row of this workgroup
    if (row0 >= rows) return;
    const int nt_total = (ctx + kTok - 1) / kTok;
    const int t0 = c * CT;
    const int t1 = min(t0 + CT, nt_total);
    const int ntile = t1 - t0;
    if (ntile <= 0) return;
    const int wrow0 = row0 + 16 * RG * wv;  // first row of this wave
    const bool computes = wrow0 < rows;

    // Tile j of the chunk sits in LDS buffer j % 4: two pairs, the one being
    // computed and the one being stored.
    __shared__ uint2 toff_lds[kMultiChunkTilesMax];
    __shared__ int tbad_lds[kMultiChunkTilesMax];
    __shared__ __attribute__((aligned(16))) unsigned char k_lds[4][kTok * kKRow];
    __shared__ __attribute__((aligned(16))) unsigned char vt_lds[4][kHd * kVtRow];

    const int32_t* __restrict__ bt = a.block_tables;
    for (int t = tid; t < ntile; t += T) {  // ntile <= kMultiChunkTilesMax (the plan's chunk limit)
        const int tok0 = (t0 + t) * kTok;
        const int phys = bt[(int64_t)i * maxB + tok0 / BS];
        const bool badp = (unsigned)phys >= (unsigned)a.num_blocks;
        // dword offset of the tile's 16 rows in the pools (two bf16 per dword)
        const int64_t off = (((int64_t)(badp ? 0 : phys) * Hkv + g) * BS + tok0 % BS) * (kHd / 2);
        toff_lds[t] = make_uint2((uint32_t)off, (uint32_t)((uint64_t)off >> 32));
        tbad_lds[t] = badp;
    }
    // This lane's row in each of the wave's groups (for the scores and the
    // softmax state): new token jq, head row % G.
    const int r16 = lane & 15;
    const int grp = lane >> 4;
    int pos_lim[RG];  // last token the row sees; -1 for a padding row
    // the smallest of them over the wave's rows (-1 if the wave has a padding row)
    const int pos_min = wrow0 + 16 * RG <= rows ? ctx - ql + wrow0 / G : -1;
    uint4 qc[RG][4];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        const int row = wrow0 + 16 * rg + r16;
        const bool real = row < rows;
        const int jq = real ? row / G : 0;
        pos_lim[rg] = real ? ctx - ql + jq : -1;
        const uint16_t* qrow =
            static_cast<const uint16_t*>(a.q) + ((int64_t)(q0 + jq) * Hq + (int64_t)g * G + (real ? row % G : 0)) * kHd;
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) {
            const uint4 v = *reinterpret_cast<const uint4*>(qrow + kq * 32 + grp * 8);
            qc[rg][kq] = real ? v : make_uint4(0, 0, 0, 0);
        }
    }
    __syncthreads();

    // Tile loads: thread (tg, vj) moves dword column vj (dims 2 vj, 2 vj + 1)
    // of tokens tg * TPI .. + TPI - 1, of K and of V; each load instruction
    // reads 256 contiguous bytes of one row.
    const uint32_t* __restrict__ k32 = static_cast<const uint32_t*>(a.k_cache);
    const uint32_t* __restrict__ v32 = static_cast<const uint32_t*>(a.v_cache);
    const int tg = tid >> 6, vj = tid & 63;
    struct TileKV {
        uint32_t k[TPI], v[TPI];
    };
    // The tile's base is wave-uniform (scalar registers); lanes add 32-bit offsets.
    const uint32_t lane_off = (uint32_t)(TPI * tg) * (kHd / 2) + (uint32_t)vj;
    auto load_tile = [&](int j, TileKV& t) {
        const uint2 o = toff_lds[j];
        const uint64_t tile = ((uint64_t)__builtin_amdgcn_readfirstlane(o.y) << 32) | __builtin_amdgcn_readfirstlane(o.x);
        const uint32_t* kt = k32 + tile;
        const uint32_t* vt = v32 + tile;
#pragma unroll
        for (int k = 0; k < TPI; ++k) t.k[k] = kt[lane_off + k * (kHd / 2)];  // K with ordinary loads: measured faster here
#pragma unroll
        for (int k = 0; k < TPI; ++k) t.v[k] = load_stream(vt + lane_off + k * (kHd / 2));
    };
    // K rows go to LDS as stored (padded rows); V goes transposed (one row
    // per dim, 16 tokens).  Value rows past the end of the context (the tail
    // of the last tile), and all of a tile past the chunk's end (the masked
    // partner of an odd last tile), are stored as zeros: their weights are
    // zero, and 0 * (whatever the slot holds, NaN included) must not reach
    // the sums.  Key rows there only give scores that the mask replaces.
    auto store_tile = [&](int buf, const TileKV& t, int j) {
        unsigned char* kb = &k_lds[buf][(TPI * tg) * kKRow + 4 * vj];
#pragma unroll
        for (int k = 0; k < TPI; ++k) *reinterpret_cast<uint32_t*>(kb + k * kKRow) = t.k[k];
        const int tokb = (t0 + j) * kTok + TPI * tg;
        const int vend = j < ntile ? ctx : 0;
        uint32_t v[TPI];
#pragma unroll
        for (int k = 0; k < TPI; ++k) v[k] = tokb + k < vend ? t.v[k] : 0u;
        unsigned char* vb = &vt_lds[buf][0];
        if constexpr (TPI == 1) {  // token tg: chunk tg / 4, position tg % 4
            *reinterpret_cast<uint16_t*>(vb + vt_off(2 * vj, tg >> 2) + 2 * (tg & 3)) = (uint16_t)(v[0] & 0xffffu);
            *reinterpret_cast<uint16_t*>(vb + vt_off(2 * vj + 1, tg >> 2) + 2 * (tg & 3)) = (uint16_t)(v[0] >> 16);
        } else if constexpr (TPI == 2) {  // tokens 2 tg, 2 tg + 1: chunk tg / 2, positions 2 (tg % 2) ..
            const uint32_t even = (v[0] & 0xffffu) | (v[1] << 16);
            const uint32_t odd = (v[0] >> 16) | (v[1] & 0xffff0000u);
            *reinterpret_cast<uint32_t*>(vb + vt_off(2 * vj, tg >> 1) + 4 * (tg & 1)) = even;
            *reinterpret_cast<uint32_t*>(vb + vt_off(2 * vj + 1, tg >> 1) + 4 * (tg & 1)) = odd;
        } else {
#pragma unroll
            for (int k = 0; k < TPI; k += 4) {
                const int ch = (TPI * tg + k) >> 2;
                const uint2 even = make_uint2((v[k] & 0xffffu) | (v[k + 1] << 16), (v[k + 2] & 0xffffu) | (v[k + 3] << 16));
                const uint2 odd = make_uint2((v[k] >> 16) | (v[k + 1] & 0xffff0000u), (v[k + 2] >> 16) | (v[k + 3] & 0xffff0000u));
                *reinterpret_cast<uint2*>(vb + vt_off(2 * vj, ch)) = even;
                *reinterpret_cast<uint2*>(vb + vt_off(2 * vj + 1, ch)) = odd;
            }
        }
    };

    f32x4 acc[RG][kHd / 16];
    float m[RG], l[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
        for (int jb = 0; jb < kHd / 16; ++jb) acc[rg][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[rg] = -INFINITY;
        l[rg] = 0.f;
    }
    bool bad = false;

    // Tiles j (even) and j + 1: S^T of each by four 16x16x32 MFMAs per row
    // group, the online softmax over the lane's eight scores, then P.V as one
    // 32-deep product per 16 dims.  In that product the lane's eight k values
    // are tokens 4 grp .. 4 grp + 3 of tile j, then the same tokens of tile
    // j + 1 -- in P (its scores) and in V (chunk grp of both transposed tiles)
    // alike.
    auto step = [&](int j) {
        const int ba = j & 3, bb = (j + 1) & 3;
        const bool has_b = j + 1 < ntile;  // uniform
        // Every row of the wave sees both tiles whole: no causal selects (uniform).
        const bool full = has_b && (t0 + j + 2) * kTok - 1 <= pos_min;
        bad |= (tbad_lds[j] | (has_b ? tbad_lds[j + 1] : 0)) != 0;
        f32x4 sa[RG], sb[RG];
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) sa[rg] = sb[rg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) {
            const uint4 ka = *reinterpret_cast<const uint4*>(&k_lds[ba][r16 * kKRow + kq * 64 + grp * 16]);
            const uint4 kb = *reinterpret_cast<const uint4*>(&k_lds[bb][r16 * kKRow + kq * 64 + grp * 16]);
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                sa[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka), as_bf16x8(qc[rg][kq]), sa[rg], 0, 0, 0);
                sb[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kb), as_bf16x8(qc[rg][kq]), sb[rg], 0, 0, 0);
            }
        }
        uint4 phi[RG], plo[RG];
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            // Token r of tile j (of tile j + 1) is visible when r <= lim_a
            // (lim_b): the causal limit, with padding rows and a missing
            // second tile seeing nothing.
            const int lim_a = pos_lim[rg] - ((t0 + j) * kTok + 4 * grp);
            const int lim_b = has_b ? lim_a - kTok : -1;
            float s[8];
            if (full) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    s[r] = sa[rg][r] * qscale;
                    s[4 + r] = sb[rg][r] * qscale;
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    s[r] = r <= lim_a ? sa[rg][r] * qscale : -INFINITY;
                    s[4 + r] = r <= lim_b ? sb[rg][r] * qscale : -INFINITY;
                }
            }
            const float smax =
                fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
            if (__any(smax > m[rg] + kLazyRescale)) {
                const float tm = max_xor32(max_xor16(smax));
                const float mn = tm > m[rg] + kLazyRescale ? tm : m[rg];
                const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m[rg] - mn);
                m[rg] = mn;
                l[rg] *= alpha;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float ar = __shfl(alpha, 4 * grp + r, kWave);
#pragma unroll
                    for (int jb = 0; jb < kHd / 16; ++jb) acc[rg][jb][r] *= ar;
                }
            }
            // m stays -inf only while the row has seen no token: then every
            // score is -inf and every weight 0.
            const float mref = m[rg] == -INFINITY ? 0.f : m[rg];
            // p = hi + lo, both bf16: each product with V is exact, the sums fp32.
            // (p rounded to bf16 alone measured up to 1.6x the tolerance on short
            // contexts, where few weights carry the output.)
            uint32_t hi[8], lo[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const float pr = fast_exp2(s[r] - mref);
                l[rg] += pr;
                const uint32_t hb = __float_as_uint(pr) & 0xffff0000u;
                hi[r] = hb >> 16;
                lo[r] = __float_as_uint(pr - __uint_as_float(hb)) >> 16;
            }
            phi[rg] = make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16));
            plo[rg] = make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16));
        }
#pragma unroll
        for (int jb = 0; jb < kHd / 16; ++jb) {
            const uint2 va = *reinterpret_cast<const uint2*>(&vt_lds[ba][vt_off(16 * jb + r16, grp)]);
            const uint2 vb = *reinterpret_cast<const uint2*>(&vt_lds[bb][vt_off(16 * jb + r16, grp)]);
            const bf16x8 vv = as_bf16x8(make_uint4(va.x, va.y, vb.x, vb.y));
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                acc[rg][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(phi[rg]), vv, acc[rg][jb], 0, 0, 0);
                acc[rg][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(plo[rg]), vv, acc[rg][jb], 0, 0, 0);
            }
        }
    };

    // kAhead tiles in flight, loaded and computed in pairs: every pair step
    // stores its two tiles, issues the loads of the pair kAhead tiles ahead
    // (clamped to the last tile, so every path issues the same loads and each
    // wait counts exactly the loads it needs), then computes.  A pair's
    // buffers are rewritten two pair steps later, after the barrier that
    // every wave passes only once its step on them is done.  The loop runs in
    // whole groups of kAhead tiles; a tail finishes the remaining pairs.
    const int ntile2 = ntile + (ntile & 1);  // tiles rounded up to whole pairs
    TileKV R[kAhead];
#pragma unroll
    for (int q = 0; q < kAhead; ++q) load_tile(min(q, ntile - 1), R[q]);
    int j0 = 0;
    for (; j0 + kAhead <= ntile2; j0 += kAhead) {
#pragma unroll
        for (int q = 0; q < kAhead; q += 2) {
            const int j = j0 + q;
            store_tile(j & 3, R[q], j);
            store_tile((j + 1) & 3, R[q + 1], j + 1);
            load_tile(min(j + kAhead, ntile - 1), R[q]);
            load_tile(min(j + 1 + kAhead, ntile - 1), R[q + 1]);
            __syncthreads();
            if (computes) step(j);
        }
    }
#pragma unroll
    for (int q = 0; q + 2 < kAhead; q += 2) {
        const int j = j0 + q;
        if (j < ntile2) {  // uniform
            store_tile(j & 3, R[q], j);
            store_tile((j + 1) & 3, R[q + 1], j + 1);
            __syncthreads();
            if (computes) step(j);
        }
    }

    multi_finish<G, RG, MERGED>(a, acc, m, l, bad, computes, i, g, rb, c, q0, rows, wrow0, nt_total, tid);
}

// LDS row of a transposed V pair: one dim, 16 tokens of each of the pair's two
// tiles (64 bytes), padded to 80.  Chunk c of a row holds tokens 4c .. 4c + 3
// of the first tile, then the same tokens of the second: the eight k values
// one lane feeds to the 32-deep P.V product, read as one 16-byte piece.  Rows
// 20 banks apart put the 16 rows of one read (dims 16 jb .. 16 jb + 15) on 16
// different 4-bank groups.  The chunks are permuted by bits 4-5 of the row,
// which one read never spans, so that a tile's stores (each lane its own dim
// row, 8 bytes) fall at most two lanes to a bank.
constexpr int kVpRow = 80;
__device__ __forceinline__ int vp_off(int d, int c) { return d * kVpRow + 16 * (c ^ ((d >> 4) & 3)); }

// max(a, b, c) in one instruction.  Scores come from matrix products, never
// signalling NaNs, so the quieting that fmaxf adds before each compare is not
// needed here.
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// The chunk kernel with the scores one pair ahead: the same workgroups, row
// groups, causal limits and results as multi_query_kernel (NRG 4 or 16), but
// each step computes S of pair p + 1 while it turns the scores of pair p into
// weights and multiplies them into V, so that the matrix products of one part
// run while the vector ALU works on the other.  K and V of a pair are staged
// separately: K two pairs ahead of the scores, V one pair ahead of P.V, each
// in a two-pair LDS ring, with one barrier per step.  A step stores K of pair
// p + 2 and V of pair p + 1 (loaded two steps before) and issues the loads of
// K of pair p + 4 and V of pair p + 3.  The score scale is folded into the
// exponent (p = 2^(s * qscale - m) as one fma) and the running max is taken
// on the raw scores, so the host passes a finite, non-zero qscale: its sign
// is moved onto q (negating bf16 is exact).
template <int BS, int G, int NRG, bool MERGED>
__global__ __launch_bounds__(64 * MultiShape<NRG>::MW) __attribute__((amdgpu_waves_per_eu(2))) void multi_pipe_kernel(
    const DecodeArgs a, float qscale) {
    constexpr int RG = MultiShape<NRG>::RG;
    constexpr int MW = MultiShape<NRG>::MW;
    constexpr int T = 64 * MW;             // threads
    constexpr int TPP = 2 * kTok * 64 / T;  // tokens of one dword column each thread moves per pair
    static_assert(NRG == 4 || NRG == 16, "row groups per workgroup");
    static_assert(TPP % 4 == 0 && TPP <= kTok, "each thread moves whole 4-token chunks of one tile");
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: scalar tile and row arithmetic
    const int i = blockIdx.x;
    const int rbs = a.multi_row_blocks;
    const int g = blockIdx.y / rbs, rb = blockIdx.y % rbs;
    const int c = blockIdx.z;
    const int Hkv = a.num_kv_heads, Hq = a.num_q_heads;
    const int maxB = a.max_blocks_per_seq;
    const int table_tokens = maxB * BS;
    const int CT = a.prefix_chunk_tiles;

    const int q0 = a.cu_q[i], q1 = a.cu_q[i + 1];
    const int ql = q1 - q0;
    const int ctx = a.context_lens[i];
    if (q0 < 0 || q1 > a.total_q || ql < 1) return;
    if (ql > a.max_q_len || ctx < ql || ctx > table_tokens) {
        if (MERGED && c == 0) {
            const int nrow = min(ql, a.max_q_len) * G;
            for (int r = 16 * NRG * rb; r < min(nrow, 16 * NRG * (rb + 1)); ++r) {
                float* o = a.out + ((int64_t)(q0 + r / G) * Hq + (int64_t)g * G + r % G) * kHd;
                for (int x = tid; x < kHd; x += T) o[x] = NAN;
            }
        }
        return;
    }
    const int rows = ql * G;
    const int row0 = 16 * NRG * rb;
    if (row0 >= rows) return;
    const int nt_total = (ctx + kTok - 1) / kTok;
    const int t0 = c * CT;
    const int t1 = min(t0 + CT, nt_total);
    const int ntile = t1 - t0;
    if (ntile <= 0) return;
    const int np = (ntile + 1) / 2;  // pairs; an odd last tile is paired with a masked one
    const int wrow0 = row0 + 16 * RG * wv;
    const bool computes = wrow0 < rows;

    __shared__ uint2 toff_lds[kMultiChunkTilesMax];
    __shared__ __attribute__((aligned(16))) unsigned char k_lds[4][kTok * kKRow];  // pair p: buffers 2 (p % 2), + 1
    __shared__ __attribute__((aligned(16))) unsigned char vp_lds[2][kHd * kVpRow];  // pair p: buffer p % 2

    const int32_t* __restrict__ bt = a.block_tables;
    int badp_any = 0;
    for (int t = tid; t < ntile; t += T) {  // ntile <= kMultiChunkTilesMax (the plan's chunk limit)
        const int tok0 = (t0 + t) * kTok;
        const int phys = bt[(int64_t)i * maxB + tok0 / BS];
        const bool badp = (unsigned)phys >= (unsigned)a.num_blocks;
        const int64_t off = (((int64_t)(badp ? 0 : phys) * Hkv + g) * BS + tok0 % BS) * (kHd / 2);
        toff_lds[t] = make_uint2((uint32_t)off, (uint32_t)((uint64_t)off >> 32));
        badp_any |= badp;
    }
    const int r16 = lane & 15;
    const int grp = lane >> 4;
    int pos_lim[RG];
    const int pos_min = wrow0 + 16 * RG <= rows ? ctx - ql + wrow0 / G : -1;
    const uint32_t qsign = qscale < 0.f ? 0x80008000u : 0u;
    const float qs = fabsf(qscale);
    uint4 qc[RG][4];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        const int row = wrow0 + 16 * rg + r16;
        const bool real = row < rows;
        const int jq = real ? row / G : 0;
        pos_lim[rg] = real ? ctx - ql + jq : -1;
        const uint16_t* qrow =
            static_cast<const uint16_t*>(a.q) + ((int64_t)(q0 + jq) * Hq + (int64_t)g * G + (real ? row % G : 0)) * kHd;
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) {
            const uint4 v = *reinterpret_cast<const uint4*>(qrow + kq * 32 + grp * 8);
            qc[rg][kq] = real ? make_uint4(v.x ^ qsign, v.y ^ qsign, v.z ^ qsign, v.w ^ qsign) : make_uint4(0, 0, 0, 0);
        }
    }
    const bool bad = __syncthreads_or(badp_any) != 0;

    // Wave wv moves tokens ptok .. ptok + TPP - 1 of tile ptile of each pair:
    // each load instruction reads 256 contiguous bytes of one row.
    const uint32_t* __restrict__ k32 = static_cast<const uint32_t*>(a.k_cache);
    const uint32_t* __restrict__ v32 = static_cast<const uint32_t*>(a.v_cache);
    const int vj = tid & 63;
    const int ptile = (TPP * wv) / kTok;
    const int ptok = (TPP * wv) % kTok;
    const uint32_t lane_off = (uint32_t)ptok * (kHd / 2) + (uint32_t)vj;
    struct Cols {
        uint32_t x[TPP];
    };
    // Tile indices past the chunk are clamped to its last tile: every path
    // issues the same loads, and the data is never used unmasked.
    auto tile_base = [&](int p) -> uint64_t {
        const uint2 o = toff_lds[min(2 * p + ptile, ntile - 1)];
        return ((uint64_t)__builtin_amdgcn_readfirstlane(o.y) << 32) | __builtin_amdgcn_readfirstlane(o.x);
    };
    auto load_k = [&](int p, Cols& t) {
        const uint32_t* kt = k32 + tile_base(p);
#pragma unroll
        for (int k = 0; k < TPP; ++k) t.x[k] = kt[lane_off + k * (kHd / 2)];
    };
    auto load_v = [&](int p, Cols& t) {
        const uint32_t* vt = v32 + tile_base(p);
#pragma unroll
        for (int k = 0; k < TPP; ++k) t.x[k] = load_stream(vt + lane_off + k * (kHd / 2));
    };
    auto store_k = [&](int p, const Cols& t) {
        unsigned char* kb = &k_lds[2 * (p & 1) + ptile][ptok * kKRow + 4 * vj];
#pragma unroll
        for (int k = 0; k < TPP; ++k) *reinterpret_cast<uint32_t*>(kb + k * kKRow) = t.x[k];
    };
    // Value rows past the context (the tail of the last tile) and all of a
    // tile past the chunk are stored as zeros: their weights are zero, and
    // 0 * (whatever the slot holds, NaN included) must not reach the sums.
    auto store_v = [&](int p, const Cols& t) {
        const int j = 2 * p + ptile;
        const int tok = (t0 + j) * kTok + ptok;
        const int vend = j < ntile ? ctx : 0;
        uint32_t v[TPP];
#pragma unroll
        for (int k = 0; k < TPP; ++k) v[k] = t.x[k];
        if (tok + TPP > vend) {  // uniform: only the last pair
#pragma unroll
            for (int k = 0; k < TPP; ++k) v[k] = tok + k < vend ? v[k] : 0u;
        }
        unsigned char* vb = &vp_lds[p & 1][8 * ptile];
#pragma unroll
        for (int q4 = 0; q4 < TPP / 4; ++q4) {
            const int ch = ptok / 4 + q4;
            const uint32_t* w = v + 4 * q4;
            const uint2 even = make_uint2(__builtin_amdgcn_perm(w[1], w[0], 0x05040100u), __builtin_amdgcn_perm(w[3], w[2], 0x05040100u));
            const uint2 odd = make_uint2(__builtin_amdgcn_perm(w[1], w[0], 0x07060302u), __builtin_amdgcn_perm(w[3], w[2], 0x07060302u));
            *reinterpret_cast<uint2*>(vb + vp_off(2 * vj, ch)) = even;
            *reinterpret_cast<uint2*>(vb + vp_off(2 * vj + 1, ch)) = odd;
        }
    };
    // S^T of pair p for every row group: four 16x16x32 MFMAs per tile.
    auto scores = [&](int p, f32x4 (&s)[RG][2]) {
        const unsigned char* ka = &k_lds[2 * (p & 1)][r16 * kKRow + grp * 16];
        const unsigned char* kb = &k_lds[2 * (p & 1) + 1][r16 * kKRow + grp * 16];
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) s[rg][0] = s[rg][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) {
            const uint4 fa = *reinterpret_cast<const uint4*>(ka + kq * 64);
            const uint4 fb = *reinterpret_cast<const uint4*>(kb + kq * 64);
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                s[rg][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(fa), as_bf16x8(qc[rg][kq]), s[rg][0], 0, 0, 0);
                s[rg][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(fb), as_bf16x8(qc[rg][kq]), s[rg][1], 0, 0, 0);
            }
        }
    };

    f32x4 acc[RG][kHd / 16];
    float m[RG], l[RG], thr[RG], nm[RG];  // running max (scaled), sum, max + lazy margin, -max (0 while -inf)
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
        for (int jb = 0; jb < kHd / 16; ++jb) acc[rg][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[rg] = -INFINITY;
        thr[rg] = -INFINITY;
        nm[rg] = 0.f;
        l[rg] = 0.f;
    }

    // Prologue: K of pairs 0 and 1 and V of pair 0 stored, the ring filled
    // with K of pairs 2, 3 and V of pairs 1, 2, and S of pair 0.
    Cols KR[2], VR[2];
    {
        Cols k0, k1, v0;
        load_k(0, k0);
        load_k(1, k1);
        load_v(0, v0);
        load_k(2, KR[0]);
        load_k(3, KR[1]);
        load_v(1, VR[0]);
        load_v(2, VR[1]);
        store_k(0, k0);
        store_k(1, k1);
        store_v(0, v0);
    }
    __syncthreads();
    f32x4 SA[RG][2], SB[RG][2];
    if (computes) scores(0, SA);

    // Step p: S holds the raw scores of pair p; Sn gets those of pair p + 1.
    // MASK applies the causal limits to S first: tokens a row cannot see, and
    // all of a missing second tile, score -inf.  Each loop below runs one
    // kind, so that no step holds a branch between its matrix products and
    // the vector work they are meant to overlap.
    auto step = [&](auto mask_tag, int p, Cols& kr, Cols& vr, f32x4 (&S)[RG][2], f32x4 (&Sn)[RG][2]) {
        constexpr bool MASK = decltype(mask_tag)::value;
        __syncthreads();  // K of pair p + 1 and V of pair p stored; pair p - 1's buffers free
        store_k(p + 2, kr);
        store_v(p + 1, vr);
        load_k(p + 4, kr);
        load_v(p + 3, vr);
        if (!computes) return;
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            if constexpr (MASK) {
                // token r of the first (second) tile is visible when r <= lim_a (lim_b)
                const int j = 2 * p;
                const int lim_a = pos_lim[rg] - ((t0 + j) * kTok + 4 * grp);
                const int lim_b = j + 1 < ntile ? lim_a - kTok : -1;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    S[rg][0][r] = r <= lim_a ? S[rg][0][r] : -INFINITY;
                    S[rg][1][r] = r <= lim_b ? S[rg][1][r] : -INFINITY;
                }
            }
            const float sm = max3f(max3f(S[rg][0][0], S[rg][0][1], S[rg][0][2]), max3f(S[rg][0][3], S[rg][1][0], S[rg][1][1]),
                                   max3f(S[rg][1][2], S[rg][1][3], S[rg][1][3]));
            if (__any(sm * qs > thr[rg])) {
                const float tm = max_xor32(max_xor16(sm)) * qs;
                const float mn = tm > thr[rg] ? tm : m[rg];
                const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m[rg] - mn);
                m[rg] = mn;
                thr[rg] = mn + kLazyRescale;
                nm[rg] = mn == -INFINITY ? 0.f : -mn;
                l[rg] *= alpha;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float ar = __shfl(alpha, 4 * grp + r, kWave);
#pragma unroll
                    for (int jb = 0; jb < kHd / 16; ++jb) acc[rg][jb][r] *= ar;
                }
            }
        }
        // S of the next pair, then the weights of this one and P.V.
        scores(p + 1, Sn);
        const unsigned char* vb = &vp_lds[p & 1][0];
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            // p = hi + lo, both bf16 (hi the top half of p's bits, lo the rest
            // rounded down): each product with V is exact, the sums fp32.
            uint32_t hi[4], lo[4];
            float pw[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) pw[r] = fast_exp2(fmaf(S[rg][r >> 2][r & 3], qs, nm[rg]));
            l[rg] += ((pw[0] + pw[1]) + (pw[2] + pw[3])) + ((pw[4] + pw[5]) + (pw[6] + pw[7]));
#pragma unroll
            for (int r = 0; r < 8; r += 2) {
                const float r0 = pw[r] - __uint_as_float(__float_as_uint(pw[r]) & 0xffff0000u);
                const float r1 = pw[r + 1] - __uint_as_float(__float_as_uint(pw[r + 1]) & 0xffff0000u);
                hi[r / 2] = __builtin_amdgcn_perm(__float_as_uint(pw[r + 1]), __float_as_uint(pw[r]), 0x07060302u);
                lo[r / 2] = __builtin_amdgcn_perm(__float_as_uint(r1), __float_as_uint(r0), 0x07060302u);
            }
            const uint4 phi = make_uint4(hi[0], hi[1], hi[2], hi[3]);
            const uint4 plo = make_uint4(lo[0], lo[1], lo[2], lo[3]);
#pragma unroll
            for (int jb = 0; jb < kHd / 16; ++jb) {
                const uint4 vv = *reinterpret_cast<const uint4*>(vb + vp_off(16 * jb + r16, grp));
                acc[rg][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(phi), as_bf16x8(vv), acc[rg][jb], 0, 0, 0);
                acc[rg][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(plo), as_bf16x8(vv), acc[rg][jb], 0, 0, 0);
            }
        }
    };
    // Pairs every row of the wave sees whole (both tiles, no causal limit),
    // rounded down to even: those steps skip the masks.  Every wave still
    // runs np steps, one barrier each.
    const int span = pos_min < 0 ? 0 : max(0, min((pos_min + 1) / kTok - t0, ntile));  // tiles seen whole by every row
    const int pf = computes ? (span / 2) & ~1 : 0;
    int p = 0;
    for (; p + 2 <= pf; p += 2) {
        step(std::false_type{}, p, KR[0], VR[0], SA, SB);
        step(std::false_type{}, p + 1, KR[1], VR[1], SB, SA);
    }
    for (; p + 2 <= np; p += 2) {
        step(std::true_type{}, p, KR[0], VR[0], SA, SB);
        step(std::true_type{}, p + 1, KR[1], VR[1], SB, SA);
    }
    if (p < np) step(std::true_type{}, p, KR[0], VR[0], SA, SB);

    multi_finish<G, RG, MERGED>(a, acc, m, l, bad, computes, i, g, rb, c, q0, rows, wrow0, nt_total, tid);
}

// Merge of the chunk partials of one new token's G heads (wave h = head g*G+h,
// lanes own two columns): out = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c
// over the sequence's chunks in order (chunks past a token's position carry
// m = -inf and weigh nothing).  Invalid sequence descriptions give NaN rows.
template <int G>
__global__ __launch_bounds__(64 * G) void multi_merge_kernel(const DecodeArgs a, int table_tokens) {
    const int lane = threadIdx.x & (kWave - 1);
    const int h = threadIdx.x / kWave;
    const int i = blockIdx.x, j = blockIdx.y, g = blockIdx.z;
    const int q0 = a.cu_q[i], q1 = a.cu_q[i + 1];
    const int ql = q1 - q0;
    if (q0 < 0 || q1 > a.total_q || ql < 1 || j >= ql) return;  // no row to write
    const int ctx = a.context_lens[i];
    const int64_t orow = (int64_t)(q0 + j) * a.num_q_heads + (int64_t)g * G + h;
    float2* out = reinterpret_cast<float2*>(a.out + orow * kHd + 2 * lane);
    const int CT = a.prefix_chunk_tiles;
    const int nch = ctx >= 1 ? ((ctx + kTok - 1) / kTok + CT - 1) / CT : 0;
    if (ql > a.max_q_len || ctx < ql || ctx > table_tokens || nch > a.prefix_max_chunks) {
        *out = make_float2(NAN, NAN);
        return;
    }
    const int64_t base = orow * a.prefix_max_chunks;
    constexpr int kFew = 8;
    if (nch <= kFew) {
        // Lane p < nch holds chunk p's (m, l); every lane loads its two
        // columns of all chunks at once.  Chunks the row cannot see (m = -inf)
        // weigh nothing, whatever their l and acc hold.
        const float2 mlv = lane < nch ? a.ws_pml[base + lane] : make_float2(-INFINITY, 0.f);
        float2 v[kFew];
#pragma unroll
        for (int p = 0; p < kFew; ++p)
            v[p] = p < nch ? *reinterpret_cast<const float2*>(a.ws_pacc + (base + p) * kHd + 2 * lane) : make_float2(0.f, 0.f);
        const float M = read_lane(row_max16(mlv.x), 0);
        const bool seen = lane < nch && mlv.x != -INFINITY;
        const float wgt = seen ? exp2f(mlv.x - M) : 0.f;
        const float L = read_lane(row_sum16(seen ? wgt * mlv.y : 0.f), 0);
        float o0 = 0.f, o1 = 0.f;
#pragma unroll
        for (int p = 0; p < kFew; ++p) {
            const float wp = read_lane(wgt, p);
            if (wp != 0.f) {  // uniform
                o0 = fmaf(wp, v[p].x, o0);
                o1 = fmaf(wp, v[p].y, o1);
            }
        }
        *out = make_float2(o0 / L, o1 / L);
        return;
    }
    float M = -INFINITY;
    for (int p = lane; p < nch; p += kWave) M = fmaxf(M, a.ws_pml[base + p].x);
    M = wave_max(M);
    float L = 0.f;
    for (int p = lane; p < nch; p += kWave) {
        const float2 v = a.ws_pml[base + p];
        L += v.x == -INFINITY ? 0.f : exp2f(v.x - M) * v.y;
    }
    L = wave_sum(L);
    float o0 = 0.f, o1 = 0.f;
    for (int p = 0; p < nch; ++p) {
        const float mp = a.ws_pml[base + p].x;
        if (mp == -INFINITY) continue;  // uniform
        const float wgt = exp2f(mp - M);
        const float2 v = *reinterpret_cast<const float2*>(a.ws_pacc + (base + p) * kHd + 2 * lane);
        o0 = fmaf(wgt, v.x, o0);
        o1 = fmaf(wgt, v.y, o1);
    }
    *out = make_float2(o0 / L, o1 / L);
}

// Several new tokens per sequence with all of a KV head's rows in one 16-row
// block (q_len * G <= 16: the verification of a few drafted tokens), and decode
// of the shapes decode_fast_kernel does not hold (one row per head: 16 query
// heads per KV head, head dims 64 and 256).  The
// tiles of all (sequence, KV head) units are laid end to end, as in
// decode_fast_kernel, and split into equal runs over the resident waves, so a
// wave's share does not depend on the length mix.  A wave walks its run in
// pieces of one unit each; a piece goes through LDS in segments of up to
// kPrefixChunkTilesMax tiles with the tile pipeline of multi_query_kernel (K as
// stored, V transposed, q.K and P.V on the matrix cores).  At the end of a
// piece the wave writes the unit's output rows (it saw all of the unit's tiles)
// or each row's (m, l, acc) to partial slot unit + wave; the wave holding the
// unit's first tile records the first slot and the number of partials (waves
// from it to the one holding the unit's last tile) for multi_sk_merge_kernel.
// HD: the head dim (128 on the multi-query path; 64 and 256 for decode).
// DEC: decode, one query row per sequence (row i of sequence i; cu_q unused).
// KNT: K rows read with non-temporal loads (V rows always are).
template <int BS, int G, int HD, bool DEC, bool KNT = true>
__global__ __launch_bounds__(64) void multi_sk_kernel(const DecodeArgs a, float qscale) {
    static_assert(HD == 64 || HD == 128 || HD == 256, "head dim");
    // Tile loads: a token row of K or V is HD / 2 dwords.  Lane l moves dword
    // column(s) l % NCL (+ 64) of TPL tokens, tokens TPL (l / NCL) .. + TPL - 1:
    // each load instruction reads whole rows (HD = 64: two 128-byte rows).
    // Decode at HD = 128 loads 16-byte pieces instead (lane l: dims 8 (l % 16)
    // .. + 7 of tokens 4 (l / 16) .. + 3, four whole rows per instruction, a
    // quarter of the load instructions): 128/8 heads over 64 sequences of
    // U[128, 4096] 101.0 against 102.5 us, same box, alternating.
    constexpr int NC = HD / 2;                // dword columns of a row
    constexpr int NCL = NC < kWave ? NC : kWave;
    constexpr int CPL = NC / NCL;             // columns per lane: 1, or 2 at HD = 256
    constexpr int TPL = kTok * NCL / kWave;   // tokens per lane: 16, or 8 at HD = 64
    constexpr int KROW = HD * 2 + 16;         // padded LDS row of a K tile (bytes)
    // tiles in flight (2 CPL TPL load registers each; 3 measured 3% faster than 2 at HD = 128)
    constexpr int kAhead = HD == 256 ? 2 : 3;
    constexpr int kSegMax = kPrefixChunkTilesMax;
    const int lane = threadIdx.x;
    const int nwaves = gridDim.x;
    const int bid = blockIdx.x;
    const int w = (nwaves % 8 == 0) ? (bid % 8) * (nwaves / 8) + bid / 8 : bid;
    const int S = a.num_seqs, Hkv = a.num_kv_heads, Hq = a.num_q_heads;
    const int maxB = a.max_blocks_per_seq;
    const int table_tokens = maxB * BS;

    // Tiles of sequence i < S; none for a description the merge reports as NaN
    // rows or leaves unwritten.
    auto seq_tiles = [&](int i) -> int {
        const int q0 = DEC ? i : a.cu_q[i], q1 = DEC ? i + 1 : a.cu_q[i + 1], ctx = a.context_lens[i];
        const int64_t ql = (int64_t)q1 - q0;
        const bool ok = q0 >= 0 && q1 <= a.total_q && ql >= 1 && ql <= a.max_q_len && ctx >= ql && ctx <= table_tokens;
        return ok ? (ctx + kTok - 1) / kTok : 0;
    };

    // ---- total tiles, one sequence per lane and round
    int total = 0;
    for (int base = 0; base < S; base += kWave) {
        const int i = base + lane;
        const int n = seq_tiles(min(i, S - 1));
        total += wave_sum_int(i < S ? n : 0);
    }
    const int64_t Nt = (int64_t)total * Hkv;
    if (Nt == 0) return;
    const int W = (int)min<int64_t>(Nt, nwaves);
    if (w >= W) return;
    const Split sp = make_split(Nt, W, nwaves, 64);  // equal runs, every wave at least one tile
    const int64_t c0 = sp.start(w), c1 = sp.start(w + 1);

    // ---- the sequence holding tile c0, and its first tile's global index
    int i = -1;
    int64_t seq_base = 0;
    {
        int64_t acc = 0;
        for (int base = 0; base < S; base += kWave) {
            const int il = base + lane;
            const int nl = seq_tiles(min(il, S - 1));
            const int n = il < S ? nl : 0;
            const int incl = wave_incl_scan_int(n);
            const int64_t chunk = (int64_t)read_lane(incl, kWave - 1) * Hkv;
            if (c0 < acc + chunk) {
                const int L = __ffsll(__ballot(acc + (int64_t)incl * Hkv > c0)) - 1;
                i = base + L;
                seq_base = acc + (int64_t)read_lane(incl - n, L) * Hkv;
                break;
            }
            acc += chunk;
        }
    }
    if (i < 0) return;  // unreachable when the two passes agree
    int n = seq_tiles(i);
    int g, b;
    {
        const int64_t off = c0 - seq_base;  // < n * Hkv
        g = (int)(off / n);
        b = (int)(off - (int64_t)g * n);
    }

    __shared__ uint2 toff_lds[kSegMax];
    __shared__ int tbad_lds[kSegMax];
    __shared__ __attribute__((aligned(16))) unsigned char k_lds[2][kTok * KROW];
    __shared__ __attribute__((aligned(16))) unsigned char vt_lds[2][HD * kVtRow];

    const int32_t* __restrict__ bt = a.block_tables;
    const uint32_t* __restrict__ k32 = static_cast<const uint32_t*>(a.k_cache);
    const uint32_t* __restrict__ v32 = static_cast<const uint32_t*>(a.v_cache);
    const int r16 = lane & 15;  // this lane's row (scores, softmax state) / output column
    const int grp = lane >> 4;
    const int lcol = lane % NCL, ltok = (lane / NCL) * TPL;  // this lane's first column and token
    struct TileKV {
        uint32_t k[CPL][TPL], v[CPL][TPL];
    };

    for (int64_t t = c0; t < c1;) {
        const int len = (int)min<int64_t>((int64_t)(n - b), c1 - t);  // tiles of this piece
        const int q0 = DEC ? i : a.cu_q[i];
        const int ql = DEC ? 1 : a.cu_q[i + 1] - q0;
        const int ctx = a.context_lens[i];
        const int rows = ql * G;
        const bool real = r16 < rows;
        const int jq = real ? r16 / G : 0;
        const int pos = ctx - ql + jq;  // last token row r16 sees
        uint4 qc[HD / 32];
        {
            const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                                   ((int64_t)(q0 + jq) * Hq + (int64_t)g * G + (real ? r16 % G : 0)) * HD;
#pragma unroll
            for (int kq = 0; kq < HD / 32; ++kq) {
                const uint4 v = *reinterpret_cast<const uint4*>(qrow + kq * 32 + grp * 8);
                qc[kq] = real ? v : make_uint4(0, 0, 0, 0);
            }
        }
        f32x4 acc[HD / 16];
#pragma unroll
        for (int jb = 0; jb < HD / 16; ++jb) acc[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m = -INFINITY;
        float l = 0.f;
        bool bad = false;

        for (int t0 = b; t0 < b + len; t0 += kSegMax) {  // tiles t0 .. t0 + ntile - 1 of the unit
            const int ntile = min(kSegMax, b + len - t0);
            if (lane < ntile) {
                const int tok0 = (t0 + lane) * kTok;
                const int phys = bt[(int64_t)i * maxB + tok0 / BS];
                const bool badp = (unsigned)phys >= (unsigned)a.num_blocks;
                const int64_t off = (((int64_t)(badp ? 0 : phys) * Hkv + g) * BS + tok0 % BS) * HD;
                toff_lds[lane] = make_uint2((uint32_t)off, (uint32_t)((uint64_t)off >> 32));
                tbad_lds[lane] = badp;
            }
            __syncthreads();

            auto load_k = [](const uint32_t* p) -> uint32_t {
                if constexpr (KNT) return load_stream(p);
                else return *p;
            };
            auto load_tile = [&](int j, TileKV& tk) {
                const uint2 o = toff_lds[j];
                if constexpr (HD == kHd && DEC) {
                    // lane l: 16 bytes (dims 8 (l % 16) .. + 7) of tokens 4 (l / 16) .. + 3,
                    // one token per load: each load instruction reads 4 whole rows
                    const int64_t off = (int64_t)(((uint64_t)o.y << 32) | o.x) + (lane >> 4) * 4 * kHd + (lane & 15) * 8;
                    const uint16_t* k16 = static_cast<const uint16_t*>(a.k_cache);
                    const uint16_t* v16 = static_cast<const uint16_t*>(a.v_cache);
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint4 x = KNT ? load_stream(k16 + off + k * kHd) : *reinterpret_cast<const uint4*>(k16 + off + k * kHd);
                        tk.k[0][4 * k] = x.x; tk.k[0][4 * k + 1] = x.y; tk.k[0][4 * k + 2] = x.z; tk.k[0][4 * k + 3] = x.w;
                    }
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint4 x = load_stream(v16 + off + k * kHd);
                        tk.v[0][4 * k] = x.x; tk.v[0][4 * k + 1] = x.y; tk.v[0][4 * k + 2] = x.z; tk.v[0][4 * k + 3] = x.w;
                    }
                } else if constexpr (HD == kHd) {  // lane l: column l of all 16 tokens
                    const int64_t off = (int64_t)(((uint64_t)o.y << 32) | o.x) / 2 + lane;
#pragma unroll
                    for (int k = 0; k < kTok; ++k) tk.k[0][k] = load_k(k32 + off + k * (kHd / 2));
#pragma unroll
                    for (int k = 0; k < kTok; ++k) tk.v[0][k] = load_stream(v32 + off + k * (kHd / 2));
                } else {
                    const int64_t off = (int64_t)(((uint64_t)o.y << 32) | o.x) / 2 + (int64_t)ltok * NC + lcol;
#pragma unroll
                    for (int c = 0; c < CPL; ++c)
#pragma unroll
                        for (int k = 0; k < TPL; ++k) tk.k[c][k] = load_k(k32 + off + k * NC + c * kWave);
#pragma unroll
                    for (int c = 0; c < CPL; ++c)
#pragma unroll
                        for (int k = 0; k < TPL; ++k) tk.v[c][k] = load_stream(v32 + off + k * NC + c * kWave);
                }
            };
            // K rows as stored (padded rows); V transposed, its rows past the
            // context stored as zeros (0 * whatever the slot holds must not
            // reach the sums; the key rows there only give masked scores).
            auto store_tile = [&](int buf, const TileKV& tk, int j) {
                if constexpr (HD == kHd && DEC) {  // tokens 4 tg .. + 3, dims 8 c .. + 7 of this lane
                    const int tg = lane >> 4, c = lane & 15;
                    unsigned char* kb = &k_lds[buf][4 * tg * KROW + 16 * c];
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        *reinterpret_cast<uint4*>(kb + k * KROW) =
                            make_uint4(tk.k[0][4 * k], tk.k[0][4 * k + 1], tk.k[0][4 * k + 2], tk.k[0][4 * k + 3]);
                    const int tokb = (t0 + j) * kTok + 4 * tg;
                    uint32_t v[kTok];  // v[4 k + q]: dims 8 c + 2 q, + 1 of token 4 tg + k
#pragma unroll
                    for (int k = 0; k < 4; ++k)
#pragma unroll
                        for (int q = 0; q < 4; ++q) v[4 * k + q] = tokb + k < ctx ? tk.v[0][4 * k + q] : 0u;
                    unsigned char* vb = &vt_lds[buf][0];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t t0v = v[q], t1v = v[4 + q], t2v = v[8 + q], t3v = v[12 + q];
                        const uint2 even = make_uint2((t0v & 0xffffu) | (t1v << 16), (t2v & 0xffffu) | (t3v << 16));
                        const uint2 odd = make_uint2((t0v >> 16) | (t1v & 0xffff0000u), (t2v >> 16) | (t3v & 0xffff0000u));
                        *reinterpret_cast<uint2*>(vb + vt_off(8 * c + 2 * q, tg)) = even;
                        *reinterpret_cast<uint2*>(vb + vt_off(8 * c + 2 * q + 1, tg)) = odd;
                    }
                    return;
                } else if constexpr (HD == kHd) {  // lane l: column l of all 16 tokens
                    unsigned char* kb = &k_lds[buf][4 * lane];
#pragma unroll
                    for (int k = 0; k < kTok; ++k) *reinterpret_cast<uint32_t*>(kb + k * KROW) = tk.k[0][k];
                    const int tokb = (t0 + j) * kTok;
                    uint32_t v[kTok];
#pragma unroll
                    for (int k = 0; k < kTok; ++k) v[k] = tokb + k < ctx ? tk.v[0][k] : 0u;
                    unsigned char* vb = &vt_lds[buf][0];
#pragma unroll
                    for (int k = 0; k < kTok; k += 4) {
                        const uint2 even = make_uint2((v[k] & 0xffffu) | (v[k + 1] << 16), (v[k + 2] & 0xffffu) | (v[k + 3] << 16));
                        const uint2 odd = make_uint2((v[k] >> 16) | (v[k + 1] & 0xffff0000u), (v[k + 2] >> 16) | (v[k + 3] & 0xffff0000u));
                        *reinterpret_cast<uint2*>(vb + vt_off(2 * lane, k >> 2)) = even;
                        *reinterpret_cast<uint2*>(vb + vt_off(2 * lane + 1, k >> 2)) = odd;
                    }
                    return;
                }
                const int tokb = (t0 + j) * kTok + ltok;
                unsigned char* vb = &vt_lds[buf][0];
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const int col = lcol + c * kWave;
                    unsigned char* kb = &k_lds[buf][ltok * KROW + 4 * col];
#pragma unroll
                    for (int k = 0; k < TPL; ++k) *reinterpret_cast<uint32_t*>(kb + k * KROW) = tk.k[c][k];
                    uint32_t v[TPL];
#pragma unroll
                    for (int k = 0; k < TPL; ++k) v[k] = tokb + k < ctx ? tk.v[c][k] : 0u;
#pragma unroll
                    for (int k = 0; k < TPL; k += 4) {
                        const uint2 even = make_uint2((v[k] & 0xffffu) | (v[k + 1] << 16), (v[k + 2] & 0xffffu) | (v[k + 3] << 16));
                        const uint2 odd = make_uint2((v[k] >> 16) | (v[k + 1] & 0xffff0000u), (v[k + 2] >> 16) | (v[k + 3] & 0xffff0000u));
                        *reinterpret_cast<uint2*>(vb + vt_off(2 * col, (ltok + k) >> 2)) = even;
                        *reinterpret_cast<uint2*>(vb + vt_off(2 * col + 1, (ltok + k) >> 2)) = odd;
                    }
                }
            };
            auto step = [&](int buf, int j) {
                bad = bad || tbad_lds[j] != 0;
                f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kq = 0; kq < HD / 32; ++kq) {
                    const uint4 kf = *reinterpret_cast<const uint4*>(&k_lds[buf][r16 * KROW + kq * 64 + grp * 16]);
                    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf), as_bf16x8(qc[kq]), sc, 0, 0, 0);
                }
                const int tok = (t0 + j) * kTok + 4 * grp;
                float s[4];
                bool vis[4];
                bool need = false;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    vis[r] = real && tok + r <= pos;
                    s[r] = vis[r] ? sc[r] * qscale : -INFINITY;
                    need = need || (vis[r] && s[r] > m + kLazyRescale);
                }
                if (__any(need)) {
                    float tm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
                    tm = max_xor32(max_xor16(tm));
                    const float mn = tm > m + kLazyRescale ? tm : m;
                    const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m - mn);
                    m = mn;
                    l *= alpha;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float ar = __shfl(alpha, 4 * grp + r, kWave);
#pragma unroll
                        for (int jb = 0; jb < HD / 16; ++jb) acc[jb][r] *= ar;
                    }
                }
                s16x4 phi, plo;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float pr = vis[r] ? fast_exp2(s[r] - m) : 0.f;
                    l += pr;
                    const uint32_t hb = __float_as_uint(pr) & 0xffff0000u;
                    phi[r] = (short)(hb >> 16);
                    plo[r] = (short)(__float_as_uint(pr - __uint_as_float(hb)) >> 16);
                }
#pragma unroll
                for (int jb = 0; jb < HD / 16; ++jb) {
                    const uint2 vb = *reinterpret_cast<const uint2*>(&vt_lds[buf][vt_off(16 * jb + r16, grp)]);
                    const s16x4 vv = __builtin_bit_cast(s16x4, vb);
                    acc[jb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, vv, acc[jb], 0, 0, 0);
                    acc[jb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, vv, acc[jb], 0, 0, 0);
                }
            };

            // The pipeline of multi_query_kernel: every step issues one tile's
            // loads (clamped to the segment's last tile), whole groups of
            // kAhead, then the last kAhead - 1 tiles.
            TileKV R[kAhead];
#pragma unroll
            for (int q = 0; q < kAhead; ++q) load_tile(min(q, ntile - 1), R[q]);
            int j0 = 0;
            for (; j0 + kAhead <= ntile; j0 += kAhead) {
#pragma unroll
                for (int q = 0; q < kAhead; ++q) {
                    const int j = j0 + q;
                    store_tile(j & 1, R[q], j);
                    load_tile(min(j + kAhead, ntile - 1), R[q]);
                    __syncthreads();
                    step(j & 1, j);
                }
            }
#pragma unroll
            for (int q = 0; q < kAhead - 1; ++q) {
                const int j = j0 + q;
                if (j < ntile) {  // uniform
                    store_tile(j & 1, R[q], j);
                    __syncthreads();
                    step(j & 1, j);
                }
            }
            __syncthreads();  // the next segment rewrites the tables and tiles
        }

        // ---- end of the piece: lane (r16, grp) holds rows 4 grp .. 4 grp + 3,
        // column r16 of every 16-dim block; row r's l is in lane r.
        const float lt = sum_xor32(sum_xor16(l));
        const int64_t u = (int64_t)i * Hkv + g;
        const int64_t slot = u + w;
        const bool whole = b == 0 && len == n;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int r = 4 * grp + rr;
            const float lr = __shfl(lt, r, kWave);
            if (r < rows) {
                if (whole) {
                    float* o = a.out + ((int64_t)(q0 + r / G) * Hq + (int64_t)g * G + r % G) * HD;
                    const float inv = bad ? NAN : 1.f / lr;
#pragma unroll
                    for (int jb = 0; jb < HD / 16; ++jb) o[16 * jb + r16] = acc[jb][rr] * inv;
                } else {
                    float* o = a.ws_acc + (slot * 16 + r) * HD;
#pragma unroll
                    for (int jb = 0; jb < HD / 16; ++jb) o[16 * jb + r16] = acc[jb][rr];
                }
            }
        }
        if (!whole && lane < 16 && real) a.ws_ml[slot * 16 + r16] = make_float2(m, bad ? NAN : lt);
        if (b == 0 && lane == 0) {
            const int64_t last_tile = seq_base + (int64_t)g * n + n - 1;
            const int rcount = whole ? 1 : (int)(sp.wave_of(last_tile) - w + 1);
            a.ws_rec[u] = make_int2((int)slot, rcount);
        }

        // ---- next piece
        t += len;
        b += len;
        if (b == n && t < c1) {
            b = 0;
            if (++g == Hkv) {
                g = 0;
                seq_base += (int64_t)Hkv * n;
                do {
                    ++i;
                } while (i < S && seq_tiles(i) == 0);
                if (i >= S) return;  // unreachable when the two passes agree
                n = seq_tiles(i);
            }
        }
    }
}

// Merge for multi_sk_kernel: one workgroup per (sequence, new token j, KV
// head g), one wave per query head h of the group, lanes owning HD / 64
// adjacent columns.  Units the tile kernel finished (one partial) are left
// alone; otherwise row r = j * G + h of the unit gets out = sum_p 2^(m_p - M)
// acc_p / sum_p 2^(m_p - M) l_p over the unit's partial slots in order (a
// partial whose tiles all lie past the row's position has m = -inf and weighs
// nothing).  Invalid sequence descriptions give NaN rows; without cu_q (decode:
// one row per sequence) an empty sequence gives a zero row.
// N adjacent floats (N = 1, 2, 4) at an address aligned to 4 N bytes, in one access.
template <int N>
__device__ __forceinline__ void load_cols(const float* p, float (&v)[N]) {
    if constexpr (N == 4) {
        const float4 t = *reinterpret_cast<const float4*>(p);
        v[0] = t.x, v[1] = t.y, v[2] = t.z, v[3] = t.w;
    } else if constexpr (N == 2) {
        const float2 t = *reinterpret_cast<const float2*>(p);
        v[0] = t.x, v[1] = t.y;
    } else {
        v[0] = *p;
    }
}
template <int N>
__device__ __forceinline__ void store_cols(float* p, const float (&v)[N]) {
    if constexpr (N == 4) {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    } else if constexpr (N == 2) {
        *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
    } else {
        *p = v[0];
    }
}

template <int G, int HD, bool DEC>
__global__ __launch_bounds__(64 * G) void multi_sk_merge_kernel(const DecodeArgs a, int table_tokens) {
    constexpr int kFew = 8;
    constexpr int VPL = HD / kWave;  // columns per lane
    const int lane = threadIdx.x & (kWave - 1);
    const int h = threadIdx.x / kWave;
    const int i = blockIdx.x, j = blockIdx.y, g = blockIdx.z;
    const int q0 = DEC ? i : a.cu_q[i], q1 = DEC ? i + 1 : a.cu_q[i + 1];
    const int ctx = a.context_lens[i];
    const int64_t u = (int64_t)i * a.num_kv_heads + g;
    const int2 rec = a.ws_rec[u];  // garbage, and unused, for an invalid sequence
    const int64_t ql = (int64_t)q1 - q0;
    if (q0 < 0 || q1 > a.total_q || ql < 1 || j >= ql) return;  // no row to write
    float* out = a.out + ((int64_t)(q0 + j) * a.num_q_heads + (int64_t)g * G + h) * HD + VPL * lane;
    auto put = [&](const float (&o)[VPL]) { store_cols<VPL>(out, o); };
    auto fill = [&](float x) {
        float o[VPL];
#pragma unroll
        for (int e = 0; e < VPL; ++e) o[e] = x;
        put(o);
    };
    if (DEC && ctx == 0) {  // decode of an empty sequence
        fill(0.f);
        return;
    }
    if (ql > a.max_q_len || ctx < ql || ctx > table_tokens) {
        fill(NAN);
        return;
    }
    if (rec.y == 1) return;  // finished by the tile kernel
    const int64_t slots = (int64_t)a.num_seqs * a.num_kv_heads + kMaxGridWaves;
    if (rec.y < 1 || rec.x < 0 || (int64_t)rec.x + rec.y > slots) {  // never written: refuse to read
        fill(NAN);
        return;
    }
    const int np = rec.y;
    const int r = j * G + h;  // < max_q_len * G <= 16
    auto ml_of = [&](int p) -> float2 { return a.ws_ml[((int64_t)rec.x + p) * 16 + r]; };
    auto acc_of = [&](int p, float (&v)[VPL]) {
        load_cols<VPL>(a.ws_acc + (((int64_t)rec.x + p) * 16 + r) * HD + VPL * lane, v);
    };
    float o[VPL];
#pragma unroll
    for (int e = 0; e < VPL; ++e) o[e] = 0.f;
    if (np <= kFew) {
        const float2 mlv = lane < np ? ml_of(lane) : make_float2(-INFINITY, 0.f);
        float v[kFew][VPL];
#pragma unroll
        for (int p = 0; p < kFew; ++p) {
            if (p < np) {
                acc_of(p, v[p]);
            } else {
#pragma unroll
                for (int e = 0; e < VPL; ++e) v[p][e] = 0.f;
            }
        }
        const float M = wave_max(mlv.x);
        const float wgt = lane < np ? exp2f(mlv.x - M) : 0.f;
        const float L = wave_sum(wgt * mlv.y);
#pragma unroll
        for (int p = 0; p < kFew; ++p) {
            const float wp = read_lane(wgt, p);
#pragma unroll
            for (int e = 0; e < VPL; ++e) o[e] = fmaf(wp, v[p][e], o[e]);
        }
#pragma unroll
        for (int e = 0; e < VPL; ++e) o[e] /= L;
        put(o);
        return;
    }
    float M = -INFINITY;
    for (int p = lane; p < np; p += kWave) M = fmaxf(M, ml_of(p).x);
    M = wave_max(M);
    float L = 0.f;
    for (int p = lane; p < np; p += kWave) {
        const float2 v = ml_of(p);
        L += exp2f(v.x - M) * v.y;
    }
    L = wave_sum(L);
    int p = 0;
    for (; p + 4 <= np; p += 4) {  // four partials' loads in flight at once
        float v[4][VPL];
        float2 mlv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            acc_of(p + k, v[k]);
            mlv[k] = ml_of(p + k);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float wgt = exp2f(mlv[k].x - M);
#pragma unroll
            for (int e = 0; e < VPL; ++e) o[e] = fmaf(wgt, v[k][e], o[e]);
        }
    }
    for (; p < np; ++p) {
        float v[VPL];
        acc_of(p, v);
        const float wgt = exp2f(ml_of(p).x - M);
#pragma unroll
        for (int e = 0; e < VPL; ++e) o[e] = fmaf(wgt, v[e], o[e]);
    }
#pragma unroll
    for (int e = 0; e < VPL; ++e) o[e] /= L;
    put(o);
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
hipError_t launch_prefix_chunks(const DecodeArgs& a, hipStream_t stream) {
    if (a.num_groups == 0 || a.prefix_max_chunks == 0) return hipSuccess;
    const dim3 grid((unsigned)a.num_groups, (unsigned)a.num_kv_heads, (unsigned)a.prefix_max_chunks);
    hipLaunchKernelGGL((decode_prefix_kernel<BS, G>), grid, dim3(kPrefixThreads), 0, stream, a,
                       a.scale * kLog2e);
    return hipGetLastError();
}

template <int BS, int G>
hipError_t launch_multi_t(const DecodeArgs& a, hipStream_t stream) {
    const dim3 mgrid((unsigned)a.num_seqs, (unsigned)a.max_q_len, (unsigned)a.num_kv_heads);
    if (a.multi_split_runs) {
        const void* k = reinterpret_cast<const void*>(&multi_sk_kernel<BS, G, kHd, false>);
        const int waves = a.grid_waves > 0 ? a.grid_waves : resident_waves(k);
        if (waves <= 0) return hipErrorInvalidValue;
        hipLaunchKernelGGL((multi_sk_kernel<BS, G, kHd, false>), dim3(waves), dim3(kWave), 0, stream, a, a.scale * kLog2e);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((multi_sk_merge_kernel<G, kHd, false>), mgrid, dim3(kWave * G), 0, stream, a, a.max_blocks_per_seq * BS);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)a.num_seqs, (unsigned)(a.num_kv_heads * a.multi_row_blocks), (unsigned)a.prefix_max_chunks);
    // The chunks are merged in the kernel while the arrival counters of all (sequence,
    // KV head, row block) units fit the workspace's counter region.
    const bool merged = (int64_t)a.num_seqs * a.num_kv_heads * a.multi_row_blocks <= kCounterUnits;
    const float qs = a.scale * kLog2e;
    // The pipelined kernel folds the scale into the exponent: a finite, non-zero one.
    const bool pipe = a.multi_waves != 1 && isfinite(qs) && qs != 0.f;
    switch (a.multi_waves * 4 + (pipe ? 2 : 0) + (merged ? 1 : 0)) {
        case 4: hipLaunchKernelGGL((multi_query_kernel<BS, G, 1, false>), grid, dim3(64), 0, stream, a, qs); break;
        case 5: hipLaunchKernelGGL((multi_query_kernel<BS, G, 1, true>), grid, dim3(64), 0, stream, a, qs); break;
        case 16: hipLaunchKernelGGL((multi_query_kernel<BS, G, 4, false>), grid, dim3(256), 0, stream, a, qs); break;
        case 17: hipLaunchKernelGGL((multi_query_kernel<BS, G, 4, true>), grid, dim3(256), 0, stream, a, qs); break;
        case 18: hipLaunchKernelGGL((multi_pipe_kernel<BS, G, 4, false>), grid, dim3(256), 0, stream, a, qs); break;
        case 19: hipLaunchKernelGGL((multi_pipe_kernel<BS, G, 4, true>), grid, dim3(256), 0, stream, a, qs); break;
        case 64: hipLaunchKernelGGL((multi_query_kernel<BS, G, 16, false>), grid, dim3(64 * MultiShape<16>::MW), 0, stream, a, qs); break;
        case 65: hipLaunchKernelGGL((multi_query_kernel<BS, G, 16, true>), grid, dim3(64 * MultiShape<16>::MW), 0, stream, a, qs); break;
        case 66: hipLaunchKernelGGL((multi_pipe_kernel<BS, G, 16, false>), grid, dim3(64 * MultiShape<16>::MW), 0, stream, a, qs); break;
        case 67: hipLaunchKernelGGL((multi_pipe_kernel<BS, G, 16, true>), grid, dim3(64 * MultiShape<16>::MW), 0, stream, a, qs); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || merged) return e;
    hipLaunchKernelGGL((multi_merge_kernel<G>), mgrid, dim3(kWave * G), 0, stream, a, a.max_blocks_per_seq * BS);
    return hipGetLastError();
}

// Decode on the split-run kernel of the multi-query path, with one query row
// per sequence (DEC: row i is sequence i's), whose G rows are the G heads, then its merge:
// the shapes decode_fast_kernel does not hold (16 query heads per KV head, head
// dims 64 and 256).  Its partial slots (16 rows each, after one record per
// unit) are the fast workspace of these shapes.
template <int BS, int G, int HD>
hipError_t launch_decode_split(const DecodeArgs& a, hipStream_t stream) {
    DecodeArgs b = a;
    b.cu_q = nullptr;
    b.total_q = a.num_seqs;
    b.max_q_len = 1;
    const void* k = reinterpret_cast<const void*>(&multi_sk_kernel<BS, G, HD, true>);
    const int resident = resident_waves(k);
    const int waves = a.grid_waves > 0 ? a.grid_waves : resident;
    if (waves <= 0) return hipErrorInvalidValue;
    // K rows streamed as in decode_fast_kernel when the units are few (at most a
    // sixteenth as many as resident waves), and always at head dim 256; else
    // ordinary loads.  Same box, alternating (streamed against ordinary): 64
    // sequences of U[128, 4096] at 128/8 heads 108.5-109.3 against 102.1-102.2
    // us, at 32/2 38.1 against 36.5, at 32/8 heads of 64 dims 54.7 against 52.5,
    // at 32/8 heads of 256 dims 186.7 against 194.5; 8 x 32k at 128/8 175.1
    // against 177.9; 256 lognormal lengths at 128/8 337.7 against 339.8.
    const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads;
    const bool knt = HD == 256 || units * 16 <= resident;
    if (knt) {
        hipLaunchKernelGGL((multi_sk_kernel<BS, G, HD, true, true>), dim3(waves), dim3(kWave), 0, stream, b,
                           b.scale * kLog2e);
    } else {
        hipLaunchKernelGGL((multi_sk_kernel<BS, G, HD, true, false>), dim3(waves), dim3(kWave), 0, stream, b,
                           b.scale * kLog2e);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 mgrid((unsigned)a.num_seqs, 1u, (unsigned)a.num_kv_heads);
    hipLaunchKernelGGL((multi_sk_merge_kernel<G, HD, true>), mgrid, dim3(kWave * G), 0, stream, b, a.max_blocks_per_seq * BS);
    e = hipGetLastError();
    if (e == hipSuccess) last_launch() = LaunchInfo{PKV_KERNEL_FAST, waves, 64, kTok, knt ? 1 : 0};
    return e;
}

template <int BS>
hipError_t multi_by_group(const DecodeArgs& a, hipStream_t stream) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_multi_t<BS, 1>(a, stream);
        case 2: return launch_multi_t<BS, 2>(a, stream);
        case 4: return launch_multi_t<BS, 4>(a, stream);
        case 8: return launch_multi_t<BS, 8>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int BS, int G, bool PREFIX>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
    if constexpr (PREFIX) {
        const hipError_t e = launch_prefix_chunks<BS, G>(a, stream);
        if (e != hipSuccess) return e;
    }
    const void* k = reinterpret_cast<const void*>(&decode_fast_kernel<BS, G, PREFIX, true>);
    const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads;
    const int resident = resident_waves(k);
    // K rows streamed (non-temporal) when each unit spans many waves (at most a
    // sixteenth as many units as resident waves), and in the prefix path's suffix
    // pass; else K is read with ordinary loads.  Same box, alternating: 8 x 32k
    // 166.4 us streamed against 171.2; 256 sequences of lognormal lengths 271.5
    // against 276.3, 64 of U[128, 4096] 85.0 against 89.4, and the plain path on
    // 32 x 8 sequences sharing 2048-token prefixes 302.6 against 368.
    const bool k_stream = PREFIX || units * 16 <= resident;
    int waves = a.grid_waves;
    bool one_per_simd = false;
    if (waves <= 0) {
        // The resident waves (two per SIMD), or one per SIMD when there are at most a
        // quarter as many (sequence, KV head) units: long units then span half as many
        // waves and leave half as many partials.  Measured on one box: 8 x 32k 194.5 ->
        // 190.2 us and 64 sequences of U[128, 4096] 103.2 -> 101.3 us with one per SIMD;
        // 256 sequences (2,048 units) 294.9 against 295.6 us with two.
        waves = resident;
        if (waves >= 16 && units * 4 <= waves) {
            waves = waves / 2 / 8 * 8;
            one_per_simd = true;
        }
    }
    if (waves <= 0) return hipErrorInvalidValue;
    // The library's XCD shares: with two waves per SIMD, odd XCDs drain more slowly
    // (PKV_XCD_BALANCE_DEFAULT); with one per SIMD, equal shares measured best (8 x 32k:
    // 187.5 us against 188.7 at 60/64 and 189.0 at 62/64; 64 sequences: a tie), and so
    // they did for the prefix path's suffix pass, whose runs are short (32 x 8 samples
    // past 2048-token prefixes: call 113.3-113.8 us against 117.4-117.5).
    DecodeArgs b = a;
    if (b.xcd_balance == 0) b.xcd_balance = (one_per_simd || PREFIX) ? 64 : PKV_XCD_BALANCE_DEFAULT;
    if (k_stream) {
        hipLaunchKernelGGL((decode_fast_kernel<BS, G, PREFIX, true>), dim3(waves), dim3(kWave), 0, stream, b,
                           b.scale * kLog2e);
    } else if constexpr (!PREFIX) {
        hipLaunchKernelGGL((decode_fast_kernel<BS, G, PREFIX, false>), dim3(waves), dim3(kWave), 0, stream, b,
                           b.scale * kLog2e);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((merge_fast_kernel<G, PREFIX>), dim3((unsigned)units), dim3(kWave * G), 0, stream, a,
                       a.max_blocks_per_seq * BS);
    e = hipGetLastError();
    if (e == hipSuccess) last_launch() = LaunchInfo{PKV_KERNEL_FAST, waves, b.xcd_balance, kTok, k_stream ? 1 : 0};
    return e;
}

template <int BS, bool PREFIX>
hipError_t by_group(const DecodeArgs& a, hipStream_t stream) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_t<BS, 1, PREFIX>(a, stream);
        case 2: return launch_t<BS, 2, PREFIX>(a, stream);
        case 4: return launch_t<BS, 4, PREFIX>(a, stream);
        case 8: return launch_t<BS, 8, PREFIX>(a, stream);
        case 16:
            if constexpr (!PREFIX && BS >= kTok) return launch_decode_split<BS, 16, kHd>(a, stream);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool fast_supports(int32_t dtype, int32_t head_dim, int32_t block_size, int32_t group) {
    // 16 query heads per KV head and head dims 64 and 256 run on the multi-query
    // split-run kernel, which reads whole 16-token tiles of one block
    const bool g_ok = group == 1 || group == 2 || group == 4 || group == 8 || group == 16;
    const bool b_ok = block_size == 8 || block_size == 16 || block_size == 32 || block_size == 64;
    const bool split = group == 16 || head_dim != kHd;
    const bool d_ok = head_dim == 64 || head_dim == kHd || head_dim == 256;
    return dtype == 1 && d_ok && b_ok && g_ok && (!split || block_size >= kTok);
}

// Decode of head dims 64 and 256 (any group size of the fast family).
template <int BS, int HD>
hipError_t split_by_group(const DecodeArgs& a, hipStream_t stream) {
    if constexpr (BS < kTok) {
        return hipErrorInvalidValue;
    } else {
        switch (a.num_q_heads / a.num_kv_heads) {
            case 1: return launch_decode_split<BS, 1, HD>(a, stream);
            case 2: return launch_decode_split<BS, 2, HD>(a, stream);
            case 4: return launch_decode_split<BS, 4, HD>(a, stream);
            case 8: return launch_decode_split<BS, 8, HD>(a, stream);
            case 16: return launch_decode_split<BS, 16, HD>(a, stream);
            default: return hipErrorInvalidValue;
        }
    }
}

template <int BS>
hipError_t fast_by_dim(const DecodeArgs& a, hipStream_t stream) {
    switch (a.head_dim) {
        case 64: return split_by_group<BS, 64>(a, stream);
        case kHd: return by_group<BS, false>(a, stream);
        case 256: return split_by_group<BS, 256>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_fast(const DecodeArgs& a, hipStream_t stream) {
    switch (a.block_size) {
        case 8: return fast_by_dim<8>(a, stream);
        case 16: return fast_by_dim<16>(a, stream);
        case 32: return fast_by_dim<32>(a, stream);
        case 64: return fast_by_dim<64>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_multi(const DecodeArgs& a, hipStream_t stream) {
    if (a.num_seqs == 0 || a.total_q == 0) return hipSuccess;
    switch (a.block_size) {
        case 16: return multi_by_group<16>(a, stream);
        case 32: return multi_by_group<32>(a, stream);
        case 64: return multi_by_group<64>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_prefix(const DecodeArgs& a, hipStream_t stream) {
    switch (a.block_size) {
        case 16: return by_group<16, true>(a, stream);
        case 32: return by_group<32, true>(a, stream);
        case 64: return by_group<64, true>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
