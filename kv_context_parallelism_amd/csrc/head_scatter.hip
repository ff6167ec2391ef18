// head_scatter.hip -- the per-rank kernels on either side of the output
// exchanges that leave each rank with a slice of the heads.
//
// "vLLM DCP and PCP: Decode and Prefill Context Parallelism", Deep Dive 6:
//   * AG+RS (and AG+AR): the ranks all-gather their LSEs; each then knows the
//     global L = log sum_i exp(L_i) of every row, scales its own normalised
//     output by exp(L_i - L), and a reduce-scatter (all-reduce) over heads
//     adds the corrected outputs.  cp_lse_correct is that scaling.
//   * all-to-all: each rank packs every partial output row together with its
//     fp32 LSE into one send buffer, laid out by destination head partition;
//     one all-to-all delivers to rank d the N partials of heads
//     d*H/N .. (d+1)*H/N - 1, which it merges exactly.  cp_a2a_pack is the
//     packing; cp_lse_merge_packed the merge over the received buffer (the
//     same merge kernels as cp_lse_merge, with the packed strides).
//
// All of it is HBM-bound streaming: each element is read once and written once;
// the correction and the packing write with non-temporal stores (their output
// is not read again by the same kernel; the pack went from 9.8 to 8.2 us per
// call at the MLA decode shape).
#include <math.h>

#include "internal.hpp"

namespace cpattn {

namespace {

constexpr int kThreads = 256;

// AG+RS correction.  A group of kS lanes owns a row: lane j reads LSEs
// j, j + kS, ... of the row, the group reduces max and sum of exp(L_i - max)
// with butterfly shuffles (xor masks below kS stay inside the group), and the
// lanes then scale float4 columns j, j + kS, ... of the rank's output.
template <int kS>
__global__ void __launch_bounds__(kThreads) correct_kernel(int32_t n, int64_t rows, int32_t n4,
                                                           int32_t rank, const float *__restrict__ po,
                                                           const float *__restrict__ pl,
                                                           float *__restrict__ co,
                                                           float *__restrict__ lse_out) {
    constexpr int kRowsPerBlock = kThreads / kS;
    const int lane_g = threadIdx.x % kS;
    for (int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kS; row < rows;
         row += (int64_t)gridDim.x * kRowsPerBlock) {
        float lmax = -INFINITY;
        int nan = 0;
        for (int i = lane_g; i < n; i += kS) {
            const float L = pl[(int64_t)i * rows + row];
            nan |= (L != L);
            lmax = fmaxf(lmax, L);
        }
#pragma unroll
        for (int x = kS / 2; x >= 1; x >>= 1) {
            lmax = fmaxf(lmax, shfl_xor(lmax, x));
            nan |= shfl_xor(nan, x);
        }
        float asum = 0.f;
        if (lmax != -INFINITY && !nan)
            for (int i = lane_g; i < n; i += kS) {
                const float L = pl[(int64_t)i * rows + row];
                asum += L == -INFINITY ? 0.f : expf(L - lmax);
            }
#pragma unroll
        for (int x = kS / 2; x >= 1; x >>= 1) asum += shfl_xor(asum, x);
        const float Li = pl[(int64_t)rank * rows + row];
        // exp(L_i - L) = exp(L_i - max) / sum_j exp(L_j - max)
        float f = 0.f;
        if (nan) f = NAN;
        else if (Li != -INFINITY) f = expf(Li - lmax) / asum;
        const float4 *src = reinterpret_cast<const float4 *>(po) + row * n4;
        float4 *dst = reinterpret_cast<float4 *>(co) + row * n4;
        for (int c = lane_g; c < n4; c += kS) {
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (f != 0.f) {  // an empty part's output is never read
                v = src[c];
                v.x *= f;
                v.y *= f;
                v.z *= f;
                v.w *= f;
            }
            store16_stream(dst + c, __builtin_bit_cast(u32x4, v));
        }
        if (lse_out && lane_g == 0)
            lse_out[row] = nan ? NAN : (lmax == -INFINITY ? -INFINITY : lmax + logf(asum));
    }
}

// All-to-all packing.  One thread per float4 of the send buffer
// [N][B][hs][n4 + 1]: packed row (d, b, j) takes output row (b, d*hs + j);
// its last float4 is (LSE, 0, 0, 0).
__global__ void __launch_bounds__(kThreads) pack_kernel(int64_t total4, int32_t B, int32_t H,
                                                        int32_t hs, int32_t n4,
                                                        const float *__restrict__ out,
                                                        const float *__restrict__ lse,
                                                        float *__restrict__ buf) {
    const int32_t w4 = n4 + 1;
    for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < total4;
         q += (int64_t)gridDim.x * kThreads) {
        const int64_t prow = q / w4;
        const int32_t c = (int32_t)(q - prow * w4);
        const int64_t per_dest = (int64_t)B * hs;
        const int32_t d = (int32_t)(prow / per_dest);
        const int64_t rem = prow - d * per_dest;
        const int32_t b = (int32_t)(rem / hs);
        const int32_t j = (int32_t)(rem - (int64_t)b * hs);
        const int64_t src_row = (int64_t)b * H + (int64_t)d * hs + j;
        float4 v;
        if (c < n4) v = reinterpret_cast<const float4 *>(out)[src_row * n4 + c];
        else v = make_float4(lse[src_row], 0.f, 0.f, 0.f);
        store16_stream(reinterpret_cast<float4 *>(buf) + q, __builtin_bit_cast(u32x4, v));
    }
}

unsigned grid_for(int64_t units, int64_t per_block) {
    const int64_t need = (units + per_block - 1) / per_block;
    const int64_t cap = (int64_t)device_cus() * 16;
    return (unsigned)(need < cap ? need : cap);
}

}  // namespace

}  // namespace cpattn

using namespace cpattn;

extern "C" cp_status cp_lse_correct(int32_t n_parts, int64_t rows, int32_t Dv, int32_t rank,
                                    const float *part_out_i, const float *part_lse,
                                    float *corrected, float *lse_out, hipStream_t stream) {
    clear_error();
    if (n_parts < 1 || rows < 0 || Dv < 1 || rank < 0 || rank >= n_parts)
        return fail(CP_E_INVALID, "cp_lse_correct: n_parts=%d rows=%lld Dv=%d rank=%d", n_parts,
                    (long long)rows, Dv, rank);
    if (Dv % 4 != 0) return fail(CP_E_UNSUPPORTED, "cp_lse_correct: Dv=%d not a multiple of 4", Dv);
    if (rows == 0) return CP_OK;
    if (!part_out_i || !part_lse || !corrected)
        return fail(CP_E_INVALID, "cp_lse_correct: NULL pointer");
    if (!aligned16(part_out_i) || !aligned16(corrected))
        return fail(CP_E_INVALID, "cp_lse_correct: part_out_i/corrected must be 16-byte aligned");
    const int32_t n4 = Dv / 4;
    // lanes per row: the float4 columns rounded up to a power of two, 8 .. 64
    int S = 8;
    while (S < n4 && S < 64) S *= 2;
    const unsigned grid = grid_for(rows, kThreads / S);
    switch (S) {
    case 8:
        hipLaunchKernelGGL(correct_kernel<8>, dim3(grid), dim3(kThreads), 0, stream, n_parts, rows,
                           n4, rank, part_out_i, part_lse, corrected, lse_out);
        break;
    case 16:
        hipLaunchKernelGGL(correct_kernel<16>, dim3(grid), dim3(kThreads), 0, stream, n_parts, rows,
                           n4, rank, part_out_i, part_lse, corrected, lse_out);
        break;
    case 32:
        hipLaunchKernelGGL(correct_kernel<32>, dim3(grid), dim3(kThreads), 0, stream, n_parts, rows,
                           n4, rank, part_out_i, part_lse, corrected, lse_out);
        break;
    default:
        hipLaunchKernelGGL(correct_kernel<64>, dim3(grid), dim3(kThreads), 0, stream, n_parts, rows,
                           n4, rank, part_out_i, part_lse, corrected, lse_out);
        break;
    }
    return check_launch("cp_lse_correct");
}

extern "C" cp_status cp_a2a_pack(int32_t B, int32_t H, int32_t Dv, int32_t N, const float *out,
                                 const float *lse, float *buf, hipStream_t stream) {
    clear_error();
    if (B < 0 || H < 1 || Dv < 1 || N < 1 || H % N != 0)
        return fail(CP_E_INVALID, "cp_a2a_pack: B=%d H=%d Dv=%d N=%d (H must be a multiple of N)",
                    B, H, Dv, N);
    if (Dv % 4 != 0) return fail(CP_E_UNSUPPORTED, "cp_a2a_pack: Dv=%d not a multiple of 4", Dv);
    if (B == 0) return CP_OK;
    if (!out || !lse || !buf) return fail(CP_E_INVALID, "cp_a2a_pack: NULL pointer");
    if (!aligned16(out) || !aligned16(buf))
        return fail(CP_E_INVALID, "cp_a2a_pack: out/buf must be 16-byte aligned");
    const int64_t total4 = (int64_t)B * H * (Dv / 4 + 1);
    hipLaunchKernelGGL(pack_kernel, dim3(grid_for(total4, kThreads)), dim3(kThreads), 0, stream,
                       total4, B, H, H / N, Dv / 4, out, lse, buf);
    return check_launch("cp_a2a_pack");
}

extern "C" cp_status cp_lse_merge_packed(int32_t n_parts, int64_t rows, int32_t Dv,
                                         const float *packed, int64_t part_stride, void *out,
                                         cp_dtype out_dt, float *lse_out, hipStream_t stream) {
    clear_error();
    if (n_parts < 1 || rows < 0 || Dv < 1)
        return fail(CP_E_INVALID, "cp_lse_merge_packed: n_parts=%d rows=%lld Dv=%d", n_parts,
                    (long long)rows, Dv);
    if (Dv % 4 != 0)
        return fail(CP_E_UNSUPPORTED, "cp_lse_merge_packed: Dv=%d not a multiple of 4", Dv);
    if (out_dt != CP_F32 && out_dt != CP_BF16)
        return fail(CP_E_UNSUPPORTED, "cp_lse_merge_packed: output dtype must be F32 or BF16");
    const int64_t row_w = (int64_t)Dv + 4;
    if (part_stride < rows * row_w || part_stride % 4 != 0)
        return fail(CP_E_INVALID,
                    "cp_lse_merge_packed: part_stride=%lld must be a multiple of 4 and >= %lld",
                    (long long)part_stride, (long long)(rows * row_w));
    if (rows == 0) return CP_OK;
    if (!packed || !out) return fail(CP_E_INVALID, "cp_lse_merge_packed: NULL pointer");
    if (!aligned16(packed) || !aligned16(out))
        return fail(CP_E_INVALID, "cp_lse_merge_packed: packed/out must be 16-byte aligned");
    MergeDesc m;
    m.n_parts = n_parts;
    m.rows = rows;
    m.Dv = Dv;
    m.part_out = packed;
    m.part_lse = packed + Dv;
    m.o_part_stride = part_stride;
    m.o_row_stride = row_w;
    m.l_part_stride = part_stride;
    m.l_row_stride = row_w;
    m.out = out;
    m.out_dt = out_dt;
    m.lse_out = lse_out;
    return launch_merge(m, stream);
}
