// attn_combine.hip -- log-sum-exp merge of split-K partitions.
//
// Partition p of a (sequence, query head) row left m_p (max score, log2
// units), l_p = sum_j 2^(s_j - m_p) and acc_p = sum_j 2^(s_j - m_p) v_j.  With
// M = max_p m_p and w_p = 2^(m_p - M):
//     out = sum_p w_p acc_p / sum_p w_p l_p,
// which equals the softmax-weighted sum over all tokens of the row exactly in
// real arithmetic.  One wave per row; lanes own head_dim/64 columns.  Rows of
// sequences that fit in one partition were finished by the partition kernel
// and are skipped.  The merge order is fixed (partition order), so results do
// not depend on scheduling.
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace pkv {

template <int D>
__global__ __launch_bounds__(64) void combine_kernel(const DecodeArgs a, int table_tokens) {
    constexpr int VPL = D / kWave;
    const int lane = threadIdx.x;
    const int64_t row = blockIdx.x;  // seq * num_q_heads + head
    const int seq = (int)(row / a.num_q_heads);
    const SeqSpan sp = seq_span(a.context_lens[seq], table_tokens, a.part_tokens);
    if (sp.nparts <= 1) return;
    const float2* ml = a.ws_ml + row * a.max_parts;

    float M = -INFINITY;
    for (int p = lane; p < sp.nparts; p += kWave) M = fmaxf(M, ml[p].x);
    M = wave_max(M);
    float L = 0.f;
    for (int p = lane; p < sp.nparts; p += kWave) {
        const float2 v = ml[p];
        L += exp2f(v.x - M) * v.y;
    }
    L = wave_sum(L);

    float o[VPL];
#pragma unroll
    for (int e = 0; e < VPL; ++e) o[e] = 0.f;
    const float* acc = a.ws_acc + row * a.max_parts * D + lane * VPL;
    for (int p = 0; p < sp.nparts; ++p) {
        const float w = exp2f(ml[p].x - M);
#pragma unroll
        for (int e = 0; e < VPL; ++e) o[e] = fmaf(w, acc[(int64_t)p * D + e], o[e]);
    }
    float* out = a.out + row * D + lane * VPL;
#pragma unroll
    for (int e = 0; e < VPL; ++e) out[e] = o[e] / L;
}

hipError_t launch_combine(const DecodeArgs& a, hipStream_t stream) {
    const int table_tokens = a.max_blocks_per_seq * a.block_size;
    const int64_t rows = (int64_t)a.num_seqs * a.num_q_heads;
    if (rows == 0) return hipSuccess;
    switch (a.head_dim) {
        case 64:
            hipLaunchKernelGGL(combine_kernel<64>, dim3((unsigned)rows), dim3(kWave), 0, stream, a, table_tokens);
            break;
        case 128:
            hipLaunchKernelGGL(combine_kernel<128>, dim3((unsigned)rows), dim3(kWave), 0, stream, a, table_tokens);
            break;
        case 256:
            hipLaunchKernelGGL(combine_kernel<256>, dim3((unsigned)rows), dim3(kWave), 0, stream, a, table_tokens);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pkv
