// lse_merge.hip -- exact merge of partial attention results.
//
// "vLLM DCP and PCP: Decode and Prefill Context Parallelism", Deep Dive 6,
// "Deriving the partial and global outputs": with l = max_i L_i and
// a_i = exp(L_i - l), the exact output is O = sum_i a_i o_i / sum_i a_i and
// its LSE is L = l + log sum_i a_i.  ("Breaking the Long-Sequence Inference
// Bottleneck ...", section 3: correct_attn after the output exchange.)
//
// HBM-bound: every partial element is read once, every output written once.
// A row is handled by Dv/4 threads, each owning one float4 column slice, so
// loads of one part are fully coalesced; the n LSEs of a row are re-read by
// each of its threads from cache.
#include <math.h>

#include "internal.hpp"

namespace cpattn {

template <bool kBf16Out>
__global__ void __launch_bounds__(256) merge_kernel(MergeDesc m, int32_t tpr, int32_t rpb) {
    const int32_t sub = threadIdx.x / tpr;
    const int32_t lane = threadIdx.x - sub * tpr;
    const int64_t row = (int64_t)blockIdx.x * rpb + sub;
    if (sub >= rpb || row >= m.rows) return;
    const float *lp = m.part_lse + row * m.l_row_stride;
    float lmax = -INFINITY;
    bool any_nan = false;
    for (int32_t i = 0; i < m.n_parts; ++i) {
        float L = lp[i * m.l_part_stride];
        any_nan |= (L != L);
        lmax = fmaxf(lmax, L);
    }
    float asum = 0.f;
    if (!any_nan && lmax != -INFINITY)
        for (int32_t i = 0; i < m.n_parts; ++i) {
            float L = lp[i * m.l_part_stride];
            if (L != -INFINITY) asum += expf(L - lmax);
        }
    const int32_t n4 = m.Dv / 4;
    const float inv = any_nan ? NAN : (asum > 0.f ? 1.f / asum : 0.f);
    for (int32_t c = lane; c < n4; c += tpr) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        if (!any_nan && lmax != -INFINITY) {
            for (int32_t i = 0; i < m.n_parts; ++i) {
                float L = lp[i * m.l_part_stride];
                if (L == -INFINITY) continue;  // empty part: weight 0, output not read
                float a = expf(L - lmax);
                const float4 o = *reinterpret_cast<const float4 *>(
                    m.part_out + i * m.o_part_stride + row * m.o_row_stride + 4 * (int64_t)c);
                acc.x += a * o.x;
                acc.y += a * o.y;
                acc.z += a * o.z;
                acc.w += a * o.w;
            }
        }
        acc.x *= inv;
        acc.y *= inv;
        acc.z *= inv;
        acc.w *= inv;
        if (kBf16Out) {
            uint2 pk;
            pk.x = pack_bf16x2(acc.x, acc.y);
            pk.y = pack_bf16x2(acc.z, acc.w);
            reinterpret_cast<uint2 *>(m.out)[row * n4 + c] = pk;
        } else {
            reinterpret_cast<float4 *>(m.out)[row * n4 + c] = acc;
        }
    }
    if (m.lse_out && lane == 0)
        m.lse_out[row] = any_nan ? NAN : (lmax == -INFINITY ? -INFINITY : lmax + logf(asum));
}

cp_status launch_merge(const MergeDesc &m, hipStream_t stream) {
    if (m.rows == 0) return CP_OK;
    int32_t n4 = m.Dv / 4;
    int32_t tpr = n4 < 256 ? n4 : 256;
    int32_t rpb = 256 / tpr;
    int64_t blocks = ceil_div(m.rows, rpb);
    if (blocks > 0x7fffffff) return fail(CP_E_UNSUPPORTED, "merge: too many rows");
    if (m.out_dt == CP_BF16)
        hipLaunchKernelGGL(merge_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, m, tpr,
                           rpb);
    else
        hipLaunchKernelGGL(merge_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, m,
                           tpr, rpb);
    return check_launch("lse merge");
}

}  // namespace cpattn

using namespace cpattn;

extern "C" cp_status cp_lse_merge(int32_t n_parts, int64_t rows, int32_t Dv, const float *part_out,
                                  const float *part_lse, void *out, cp_dtype out_dt, float *lse_out,
                                  hipStream_t stream) {
    clear_error();
    if (n_parts < 1 || rows < 0 || Dv < 1)
        return fail(CP_E_INVALID, "cp_lse_merge: n_parts=%d rows=%lld Dv=%d", n_parts,
                    (long long)rows, Dv);
    if (Dv % 4 != 0) return fail(CP_E_UNSUPPORTED, "cp_lse_merge: Dv=%d not a multiple of 4", Dv);
    if (out_dt != CP_F32 && out_dt != CP_BF16)
        return fail(CP_E_UNSUPPORTED, "cp_lse_merge: output dtype must be F32 or BF16");
    if (rows == 0) return CP_OK;
    if (!part_out || !part_lse || !out) return fail(CP_E_INVALID, "cp_lse_merge: NULL pointer");
    if (!aligned16(part_out) || !aligned16(out))
        return fail(CP_E_INVALID, "cp_lse_merge: part_out/out must be 16-byte aligned");
    MergeDesc m;
    m.n_parts = n_parts;
    m.rows = rows;
    m.Dv = Dv;
    m.part_out = part_out;
    m.part_lse = part_lse;
    m.o_part_stride = rows * Dv;
    m.o_row_stride = Dv;
    m.l_part_stride = rows;
    m.l_row_stride = 1;
    m.out = out;
    m.out_dt = out_dt;
    m.lse_out = lse_out;
    return launch_merge(m, stream);
}
