// attn_generic.hip -- split-K partition kernel of paged decode attention for
// every supported shape (fp32 or bf16, head_dim 64/128/256, any block size
// that is a power of two, query-group size 1/2/4/8/16).
//
// Work unit: one workgroup of one wave per (sequence, KV head, partition of
// part_tokens logical tokens).  The G query heads that share the KV head are
// handled together, so each K/V byte is read once for all of them.
//
// Per 64-token tile (logical positions t0 .. t0+63 of the partition):
//   * lane l owns token j = t0 + l: it looks up the physical block of j in the
//     block table (block_tables[seq][j / block_size]) and computes the G scores
//     q_h . K[j] with q pre-multiplied by scale * log2(e) (scores in log2 units);
//   * online softmax: tile max by wave reduction, running max m, rescale of the
//     denominator l and of the accumulator by exp2(m_old - m_new);
//   * P.V: lanes own head_dim/64 output columns each; the tile's tokens are
//     walked in logical order, each token's weight and physical block taken
//     from its lane by readlane, its V row read coalesced across the wave,
//     16 or 32 rows' loads issued before the first is used.
// A sequence that fits in one partition is normalised and written to `out`
// directly; otherwise (m, l, acc) go to the workspace for the combine kernel.
// Summation order depends only on logical positions, never on placement.
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace pkv {

template <typename E, int D, int G>
__global__ __launch_bounds__(64) void decode_generic_kernel(const DecodeArgs a, int block_shift,
                                                            float qscale) {
    using T = typename E::storage;
    constexpr int VPL = D / kWave;             // output columns per lane
    constexpr int CH = Chunk16<E>::kElems;     // elements per 16-byte chunk
    const int lane = threadIdx.x;
    const int64_t wg = blockIdx.x;
    const int part = (int)(wg % a.max_parts);
    const int64_t rest = wg / a.max_parts;
    const int g = (int)(rest % a.num_kv_heads);
    const int seq = (int)(rest / a.num_kv_heads);

    const int table_tokens = a.max_blocks_per_seq << block_shift;
    const SeqSpan sp = seq_span(a.context_lens[seq], table_tokens, a.part_tokens);
    if (part >= sp.nparts) return;
    const int start = part * a.part_tokens;
    const int end = min(sp.ctx, start + a.part_tokens);

    __shared__ float q_s[G][D];
    const T* qp = static_cast<const T*>(a.q) + ((int64_t)seq * a.num_q_heads + (int64_t)g * G) * D;
    for (int i = lane; i < G * D; i += kWave) q_s[i / D][i % D] = widen(qp[i]) * qscale;
    __syncthreads();

    float m[G], l[G], acc[G][VPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < VPL; ++e) acc[h][e] = 0.f;
    }
    bool bad = sp.bad;

    const int32_t* bt = a.block_tables + (int64_t)seq * a.max_blocks_per_seq;
    const int64_t head_stride = (int64_t)D << block_shift;
    const int64_t block_stride = head_stride * a.num_kv_heads;
    const T* kbase = static_cast<const T*>(a.k_cache) + g * head_stride;
    const T* vbase = static_cast<const T*>(a.v_cache) + g * head_stride;
    const int bmask = (1 << block_shift) - 1;

    for (int t0 = start; t0 < end; t0 += kWave) {
        const int j = t0 + lane;
        const bool valid = j < end;
        int blk = valid ? bt[j >> block_shift] : 0;
        if ((unsigned)blk >= (unsigned)a.num_blocks) {
            bad = bad || valid;
            blk = 0;
        }
        float s[G];
#pragma unroll
        for (int h = 0; h < G; ++h) s[h] = 0.f;
        if (valid) {
            const T* kr = kbase + (int64_t)blk * block_stride + (int64_t)(j & bmask) * D;
            // K chunks in flight: 8 (4 measured 5% slower on bf16 d = 128), 4 where
            // the row has only 8 chunks (bf16 d = 64: 8 spilled at G >= 8).
            constexpr int KU = D / CH >= 16 ? 8 : 4;
#pragma unroll KU
            for (int x = 0; x < D; x += CH) {
                float kf[CH];
                Chunk16<E>::load(kr + x, kf);
#pragma unroll
                for (int h = 0; h < G; ++h)
#pragma unroll
                    for (int e = 0; e < CH; ++e) s[h] = fmaf(q_s[h][x + e], kf[e], s[h]);
            }
        }
        float p[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mt = wave_max(valid ? s[h] : -INFINITY);
            const float mn = fmaxf(m[h], mt);
            const float alpha = exp2f(m[h] - mn);
            p[h] = valid ? exp2f(s[h] - mn) : 0.f;
            l[h] = l[h] * alpha + p[h];
#pragma unroll
            for (int e = 0; e < VPL; ++e) acc[h][e] *= alpha;
            m[h] = mn;
        }
        // The tile's V rows, U at a time: all of a group's loads are issued
        // before its first use (one row at a time left the wave waiting on
        // every load: 2.4-2.6x slower).
        const int ntok = min(kWave, end - t0);
        constexpr int U = VPL >= 4 ? 16 : 32;
        auto v_row = [&](int t) -> const T* {
            return vbase + (int64_t)read_lane(blk, t) * block_stride + (int64_t)((t0 + t) & bmask) * D + lane * VPL;
        };
        int t = 0;
        for (; t + U <= ntok; t += U) {
            float vf[U][VPL];
#pragma unroll
            for (int u = 0; u < U; ++u) load_small<E, VPL>(v_row(t + u), vf[u]);
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float pt = read_lane(p[h], t + u);
#pragma unroll
                    for (int e = 0; e < VPL; ++e) acc[h][e] = fmaf(pt, vf[u][e], acc[h][e]);
                }
            }
        }
        for (; t < ntok; ++t) {
            float vf[VPL];
            load_small<E, VPL>(v_row(t), vf);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float pt = read_lane(p[h], t);
#pragma unroll
                for (int e = 0; e < VPL; ++e) acc[h][e] = fmaf(pt, vf[e], acc[h][e]);
            }
        }
    }

    bad = __any(bad);
#pragma unroll
    for (int h = 0; h < G; ++h) l[h] = wave_sum(l[h]);

    const int64_t row0 = (int64_t)seq * a.num_q_heads + (int64_t)g * G;
    if (sp.nparts == 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float* o = a.out + (row0 + h) * D + lane * VPL;
#pragma unroll
            for (int e = 0; e < VPL; ++e) o[e] = bad ? NAN : (sp.ctx == 0 ? 0.f : acc[h][e] / l[h]);
        }
    } else {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float* w = a.ws_acc + ((row0 + h) * a.max_parts + part) * D + lane * VPL;
#pragma unroll
            for (int e = 0; e < VPL; ++e) w[e] = acc[h][e];
            if (lane == 0) a.ws_ml[(row0 + h) * a.max_parts + part] = make_float2(m[h], bad ? NAN : l[h]);
        }
    }
}

namespace {

template <typename E, int D, int G>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
    const int block_shift = __builtin_ctz((unsigned)a.block_size);
    const int64_t grid = (int64_t)a.max_parts * a.num_kv_heads * a.num_seqs;
    hipLaunchKernelGGL((decode_generic_kernel<E, D, G>), dim3((unsigned)grid), dim3(kWave), 0, stream,
                       a, block_shift, a.scale * kLog2e);
    return hipGetLastError();
}

template <typename E, int D>
hipError_t by_group(const DecodeArgs& a, hipStream_t stream) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_t<E, D, 1>(a, stream);
        case 2: return launch_t<E, D, 2>(a, stream);
        case 4: return launch_t<E, D, 4>(a, stream);
        case 8: return launch_t<E, D, 8>(a, stream);
        case 16: return launch_t<E, D, 16>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename E>
hipError_t by_dim(const DecodeArgs& a, hipStream_t stream) {
    switch (a.head_dim) {
        case 64: return by_group<E, 64>(a, stream);
        case 128: return by_group<E, 128>(a, stream);
        case 256: return by_group<E, 256>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool generic_supports(int32_t dtype, int32_t head_dim, int32_t group) {
    const bool d_ok = head_dim == 64 || head_dim == 128 || head_dim == 256;
    const bool g_ok = group == 1 || group == 2 || group == 4 || group == 8 || group == 16;
    return (dtype == 0 || dtype == 1) && d_ok && g_ok;
}

hipError_t launch_decode_generic(const DecodeArgs& a, hipStream_t stream) {
    return a.dtype == 0 ? by_dim<F32>(a, stream) : by_dim<BF16>(a, stream);
}

}  // namespace pkv
