// lse_merge.hip -- exact merge of partial attention results.
//
// "vLLM DCP and PCP: Decode and Prefill Context Parallelism", Deep Dive 6,
// "Deriving the partial and global outputs": with l = max_i L_i and
// a_i = exp(L_i - l), the exact output is O = sum_i a_i o_i / sum_i a_i and
// its LSE is L = l + log sum_i a_i.  ("Breaking the Long-Sequence Inference
// Bottleneck ...", section 3: correct_attn after the output exchange.)
//
// HBM-bound: every partial element is read once, every output written once.
// Two kernels:
//   * rows of up to 256 columns with up to kLaneParts parts (every merge of
//     the decode and prefill paths): a group of S lanes (S = the float4
//     columns, rounded up to a power of two, at most 64) owns a row; each lane
//     reads the row's few LSEs itself (the group's lanes read the same
//     addresses), keeps max, weights and their sum in registers, and
//     accumulates its float4 columns over the parts -- no LDS, no barrier,
//     and all of a lane's part loads in flight together.  A grid-stride loop
//     over row groups keeps every wave busy;
//   * otherwise one 256-thread workgroup per output row: the row's LSEs are
//     reduced (max, then sum of weights) across the block, then thread
//     (column c, group gi) accumulates float4 column c over the parts gi,
//     gi+G, ..., and the G group sums are added in LDS.
#include <math.h>

#include "internal.hpp"

namespace cpattn {

namespace {

constexpr int kThreads = 256;
constexpr int kCachedWeights = 2048;  // weights kept in LDS; beyond that, recomputed
constexpr int kLaneParts = 64;        // parts per row above which the block kernel is used
constexpr int kLaneCols = 4;          // float4 columns per lane (Dv <= 64 * 4 * 4)

// Rows of the merge: parts, LSE and output base of row r (plain or segmented).
// The output base is an element offset into part_out (fp32 or bf16 elements).
struct RowParts {
    const float *lp;
    int64_t oe;
    int32_t n;
};
__device__ __forceinline__ RowParts row_parts(const MergeDesc &m, int64_t row) {
    RowParts rp;
    rp.lp = m.part_lse + row * m.l_row_stride;
    rp.oe = row * m.o_row_stride;
    rp.n = m.n_parts;
    if (m.seg) {  // parts of this row live at slots first .. first+count-1
        const int64_t grp = row / m.rows_per_seg, sub = row % m.rows_per_seg;
        const int64_t first = m.seg[2 * grp];
        rp.n = m.seg[2 * grp + 1];
        rp.lp = m.part_lse + first * m.l_part_stride + sub * m.l_row_stride;
        rp.oe = first * m.o_part_stride + sub * m.o_row_stride;
    }
    return rp;
}

// Four consecutive partial-output elements from element offset e (a multiple
// of 4): one 16-byte fp32 load, or one 8-byte load of bf16 values widened
// exactly.  The element type is a template flag, so that a batch's loads
// are one straight run of instructions.
template <bool kBf16In>
__device__ __forceinline__ float4 load_part4(const MergeDesc &m, int64_t e) {
    if constexpr (kBf16In) {
        const u32x2 w = *reinterpret_cast<const u32x2 *>(
            reinterpret_cast<const uint16_t *>(m.part_out) + e);
        return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                           __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
    }
    return *reinterpret_cast<const float4 *>(m.part_out + e);
}

// Lane-parallel merge: lane j of a kS-lane group owns float4 columns
// j, j + kS, ... (kCols of them) of its row.  One pass over the parts, eight
// at a time: the batch's LSEs and output columns are loaded together (no
// dependent round trip from an LSE to its output), then the running maximum
// is raised to the batch's and the earlier sums are rescaled by
// exp(old max - new max) -- a no-op for rows of at most eight parts.
//
// kWpr > 1 (rows of many parts): kWpr lane groups of one workgroup share a row,
// group w taking the batches of parts w*8 .., (w+kWpr)*8 .., each with its
// own maximum, weight sum and columns; the groups' states are then rescaled
// to the largest maximum and added through LDS (the same exact rescaling as
// between batches), so a row's dependent load rounds drop kWpr-fold.
template <bool kBf16Out, int kS, int kCols, bool kBf16In, int kWpr>
__global__ void __launch_bounds__(kThreads) merge_lanes_kernel(MergeDesc m) {
    constexpr int kRowsPerBlock = kThreads / kS / kWpr;
    constexpr int kBatch = 8;
    static_assert(kWpr == 1 || kRowsPerBlock == 1, "groups share a row only one row per block");
    const int lane_g = threadIdx.x % kS;
    const int sub = kWpr > 1 ? (int)(threadIdx.x / kS) : 0;
    const int n4 = m.Dv / 4;
    __shared__ float s_m[kWpr], s_s[kWpr];
    __shared__ int s_nan[kWpr];
    __shared__ float4 s_acc[kWpr > 1 ? kWpr : 1][kCols][kS];
    for (int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (kWpr > 1 ? 0 : threadIdx.x / kS);
         row < m.rows; row += (int64_t)gridDim.x * kRowsPerBlock) {
        const RowParts rp = row_parts(m, row);
        float lmax = -INFINITY;
        bool nan = false;
        float asum = 0.f;
        float4 acc[kCols];
#pragma unroll
        for (int cc = 0; cc < kCols; ++cc) acc[cc] = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int i0 = sub * kBatch; i0 < rp.n; i0 += kBatch * kWpr) {
            float L[kBatch];
            float4 o[kBatch][kCols];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                L[j] = i0 + j < rp.n ? rp.lp[(int64_t)(i0 + j) * m.l_part_stride] : -INFINITY;
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                if constexpr (kBf16In) {
                    // Unconditional loads from clamped (valid) addresses, then a
                    // select: a load under a condition would be widened inside
                    // its branch and wait there, one load at a time.
                    const int jj = i0 + j < rp.n ? i0 + j : rp.n - 1;
                    const int64_t oe = rp.oe + (int64_t)jj * m.o_part_stride;
#pragma unroll
                    for (int cc = 0; cc < kCols; ++cc) {
                        const int c = lane_g + cc * kS;
                        const float4 v = load_part4<true>(m, oe + 4 * (c < n4 ? c : n4 - 1));
                        o[j][cc] = i0 + j < rp.n && c < n4 ? v : make_float4(0.f, 0.f, 0.f, 0.f);
                    }
                } else {
                    const int64_t oe = rp.oe + (int64_t)(i0 + j) * m.o_part_stride;
#pragma unroll
                    for (int cc = 0; cc < kCols; ++cc) {
                        const int c = lane_g + cc * kS;
                        o[j][cc] = i0 + j < rp.n && c < n4 ? load_part4<false>(m, oe + 4 * c)
                                                            : make_float4(0.f, 0.f, 0.f, 0.f);
                    }
                }
            }
            float bmax = lmax;
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                nan |= (L[j] != L[j]);
                bmax = fmaxf(bmax, L[j]);
            }
            // every part so far is empty: nothing to add (with bf16 parts the
            // batch falls through instead, adding zeros, so that its loads are
            // not moved below this test and issued after the LSEs arrive)
            if (!kBf16In && bmax == -INFINITY) continue;
            if (bmax != lmax) {               // rescale the earlier sums to the new maximum
                const float sc = lmax == -INFINITY ? 0.f : expf(lmax - bmax);
                asum *= sc;
#pragma unroll
                for (int cc = 0; cc < kCols; ++cc) {
                    acc[cc].x *= sc;
                    acc[cc].y *= sc;
                    acc[cc].z *= sc;
                    acc[cc].w *= sc;
                }
                lmax = bmax;
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const float a = L[j] == -INFINITY ? 0.f : expf(L[j] - lmax);
                asum += a;
#pragma unroll
                for (int cc = 0; cc < kCols; ++cc) {
                    // an empty part's output is loaded but never used
                    const float4 v = a > 0.f ? o[j][cc] : make_float4(0.f, 0.f, 0.f, 0.f);
                    acc[cc].x += a * v.x;
                    acc[cc].y += a * v.y;
                    acc[cc].z += a * v.z;
                    acc[cc].w += a * v.w;
                }
            }
        }
        if constexpr (kWpr > 1) {  // add the groups' states in group 0
            if (lane_g == 0) {
                s_m[sub] = lmax;
                s_s[sub] = asum;
                s_nan[sub] = nan;
            }
#pragma unroll
            for (int cc = 0; cc < kCols; ++cc) s_acc[sub][cc][lane_g] = acc[cc];
            __syncthreads();
            if (sub == 0) {
                float M = -INFINITY;
                for (int w = 0; w < kWpr; ++w) {
                    M = fmaxf(M, s_m[w]);
                    nan |= s_nan[w] != 0;
                }
                asum = 0.f;
#pragma unroll
                for (int cc = 0; cc < kCols; ++cc) acc[cc] = make_float4(0.f, 0.f, 0.f, 0.f);
                for (int w = 0; w < kWpr; ++w) {
                    const float sc = s_m[w] == -INFINITY ? 0.f : expf(s_m[w] - M);
                    asum += s_s[w] * sc;
#pragma unroll
                    for (int cc = 0; cc < kCols; ++cc) {
                        const float4 v = s_acc[w][cc][lane_g];
                        acc[cc].x += sc * v.x;
                        acc[cc].y += sc * v.y;
                        acc[cc].z += sc * v.z;
                        acc[cc].w += sc * v.w;
                    }
                }
                lmax = M;
            }
        }
        const bool empty = lmax == -INFINITY;
        const float inv = nan ? NAN : (!empty && asum > 0.f ? 1.f / asum : 0.f);
#pragma unroll
        for (int cc = 0; cc < kCols; ++cc) {
            const int c = lane_g + cc * kS;
            if (c >= n4 || sub != 0) break;
            float4 v = empty && !nan ? make_float4(0.f, 0.f, 0.f, 0.f) : acc[cc];
            v.x *= inv;
            v.y *= inv;
            v.z *= inv;
            v.w *= inv;
            if (kBf16Out) {
                u32x2 pk;
                pk.x = pack_bf16x2(v.x, v.y);
                pk.y = pack_bf16x2(v.z, v.w);
                reinterpret_cast<u32x2 *>(m.out)[merge_out_row(m, row) * n4 + c] = pk;
            } else {
                reinterpret_cast<float4 *>(m.out)[merge_out_row(m, row) * n4 + c] = v;
            }
        }
        if (m.lse_out && lane_g == 0 && sub == 0)
            m.lse_out[merge_out_row(m, row)] = nan ? NAN : (empty ? -INFINITY : lmax + logf(asum));
        if constexpr (kWpr > 1) __syncthreads();  // LDS free for the next row
    }
}

__device__ __forceinline__ float block_reduce(float v, bool is_max, float *s_red) {
    for (int x = 32; x >= 1; x >>= 1) {
        const float o = __shfl_xor(v, x, 64);
        v = is_max ? fmaxf(v, o) : v + o;
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();
    if (lane == 0) s_red[wave] = v;
    __syncthreads();
    v = s_red[0];
    for (int i = 1; i < kThreads / 64; ++i) v = is_max ? fmaxf(v, s_red[i]) : v + s_red[i];
    return v;
}

template <bool kBf16Out, bool kBf16In>
__global__ void __launch_bounds__(kThreads) merge_rows_kernel(MergeDesc m) {
    __shared__ float s_w[kCachedWeights];
    __shared__ float s_red[kThreads / 64];
    __shared__ float4 s_acc[kThreads];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    const RowParts rp = row_parts(m, row);
    const float *lp = rp.lp;
    m.n_parts = rp.n;

    // 1. l = max_i L_i (NaN anywhere poisons the row)
    float lmax = -INFINITY;
    int nan = 0;
    for (int i = tid; i < m.n_parts; i += kThreads) {
        const float L = lp[(int64_t)i * m.l_part_stride];
        nan |= (L != L);
        lmax = fmaxf(lmax, L);
    }
    lmax = block_reduce(lmax, true, s_red);
    nan = __syncthreads_or(nan);
    // 2. a_i = exp(L_i - l), their sum
    float asum = 0.f;
    const bool empty = (lmax == -INFINITY) || nan;
    if (!empty)
        for (int i = tid; i < m.n_parts; i += kThreads) {
            const float L = lp[(int64_t)i * m.l_part_stride];
            const float a = (L == -INFINITY) ? 0.f : expf(L - lmax);
            if (i < kCachedWeights) s_w[i] = a;
            asum += a;
        }
    asum = block_reduce(asum, false, s_red);  // includes a barrier: s_w is visible

    // 3. weighted column sums, parts spread over G thread groups
    const int n4 = m.Dv / 4;
    const int cols = n4 < kThreads ? n4 : kThreads;
    const int G = kThreads / cols;
    const int c0 = tid % cols, gi = tid / cols;
    const float inv = nan ? NAN : (asum > 0.f ? 1.f / asum : 0.f);
    for (int cb = 0; cb < n4; cb += cols) {
        const int c = cb + c0;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        if (!empty && gi < G && c < n4) {
            const int64_t oc = rp.oe + 4 * (int64_t)c;
            for (int i = gi; i < m.n_parts; i += G) {
                float a;
                if (i < kCachedWeights) {
                    a = s_w[i];
                } else {
                    const float L = lp[(int64_t)i * m.l_part_stride];
                    a = (L == -INFINITY) ? 0.f : expf(L - lmax);
                }
                if (a > 0.f) {  // an empty part's output is never read
                    const float4 o = load_part4<kBf16In>(m, oc + (int64_t)i * m.o_part_stride);
                    acc.x += a * o.x;
                    acc.y += a * o.y;
                    acc.z += a * o.z;
                    acc.w += a * o.w;
                }
            }
        }
        s_acc[tid] = acc;
        __syncthreads();
        if (gi == 0 && c < n4) {
            for (int g2 = 1; g2 < G; ++g2) {
                const float4 o = s_acc[g2 * cols + c0];
                acc.x += o.x;
                acc.y += o.y;
                acc.z += o.z;
                acc.w += o.w;
            }
            acc.x *= inv;
            acc.y *= inv;
            acc.z *= inv;
            acc.w *= inv;
            if (kBf16Out) {
                u32x2 pk;
                pk.x = pack_bf16x2(acc.x, acc.y);
                pk.y = pack_bf16x2(acc.z, acc.w);
                reinterpret_cast<u32x2 *>(m.out)[merge_out_row(m, row) * n4 + c] = pk;
            } else {
                reinterpret_cast<float4 *>(m.out)[merge_out_row(m, row) * n4 + c] = acc;
            }
        }
        __syncthreads();
    }
    if (m.lse_out && tid == 0)
        m.lse_out[merge_out_row(m, row)] = nan ? NAN : (lmax == -INFINITY ? -INFINITY : lmax + logf(asum));
}

}  // namespace

int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <bool kBf16Out, bool kBf16In, int kS, int kCols, int kWpr = 1>
void launch_lanes(const MergeDesc &m, hipStream_t stream) {
    constexpr int kRowsPerBlock = kThreads / kS / kWpr;
    const int64_t need = (m.rows + kRowsPerBlock - 1) / kRowsPerBlock;
    const int64_t cap = (int64_t)device_cus() * 16;  // resident blocks, with margin
    const unsigned grid = (unsigned)(need < cap ? need : cap);
    hipLaunchKernelGGL((merge_lanes_kernel<kBf16Out, kS, kCols, kBf16In, kWpr>), dim3(grid), dim3(kThreads), 0,
                       stream, m);
}

// float4 columns -> (lanes per row, columns per lane).  Returns false (the
// caller then uses the block kernel) when the rows are too wide, or -- for a
// plain merge -- too few to keep enough column loads in flight on every CU
// (lanes times columns per lane: a row of 128 float4 columns in 64 lanes
// counts twice).  A split combine (segment table) always takes it: its rows
// have a few parts each, which one batch of loads covers, and that beats the
// block kernel's dependent passes even on 1,024 rows (GQA decode combine).
template <bool kBf16Out, bool kBf16In>
bool launch_lanes_for(const MergeDesc &m, hipStream_t stream) {
    const int n4 = m.Dv / 4;
    int S = 1;
    while (S < n4 && S < 64) S *= 2;
    const int cols = (n4 + S - 1) / S;
    if (!m.seg && m.rows * S * cols < (int64_t)device_cus() * 512) return false;
    if (n4 <= 1) launch_lanes<kBf16Out, kBf16In, 1, 1>(m, stream);
    else if (n4 <= 2) launch_lanes<kBf16Out, kBf16In, 2, 1>(m, stream);
    else if (n4 <= 4) launch_lanes<kBf16Out, kBf16In, 4, 1>(m, stream);
    else if (n4 <= 8) launch_lanes<kBf16Out, kBf16In, 8, 1>(m, stream);
    else if (n4 <= 16) launch_lanes<kBf16Out, kBf16In, 16, 1>(m, stream);
    else if (n4 <= 32) launch_lanes<kBf16Out, kBf16In, 32, 1>(m, stream);
    else if (n4 <= 64) launch_lanes<kBf16Out, kBf16In, 64, 1>(m, stream);
    else if (n4 <= 128 && m.parts_hint >= 16) launch_lanes<kBf16Out, kBf16In, 64, 2, 4>(m, stream);
    else if (n4 <= 128) launch_lanes<kBf16Out, kBf16In, 64, 2>(m, stream);
    else if (n4 <= 64 * kLaneCols) launch_lanes<kBf16Out, kBf16In, 64, kLaneCols>(m, stream);
    else return false;
    return true;
}

cp_status launch_merge(const MergeDesc &m, hipStream_t stream) {
    if (m.rows == 0) return CP_OK;
    if (m.rows > 0x7fffffff) return fail(CP_E_UNSUPPORTED, "merge: too many rows");
    // Many rows of up to 64 * kLaneCols float4 columns with few parts take
    // the lane-parallel kernel (a segment table's counts are a few per row by
    // construction of the decode schedules).
    if (m.seg || m.n_parts <= kLaneParts) {
        const bool ok = m.part_bf16 ? (m.out_dt == CP_BF16 ? launch_lanes_for<true, true>(m, stream)
                                                           : launch_lanes_for<false, true>(m, stream))
                                    : (m.out_dt == CP_BF16 ? launch_lanes_for<true, false>(m, stream)
                                                           : launch_lanes_for<false, false>(m, stream));
        if (ok) return check_launch("lse merge");
    }
    const dim3 g((unsigned)m.rows), b(kThreads);
    if (m.part_bf16) {
        if (m.out_dt == CP_BF16) hipLaunchKernelGGL((merge_rows_kernel<true, true>), g, b, 0, stream, m);
        else hipLaunchKernelGGL((merge_rows_kernel<false, true>), g, b, 0, stream, m);
    } else {
        if (m.out_dt == CP_BF16) hipLaunchKernelGGL((merge_rows_kernel<true, false>), g, b, 0, stream, m);
        else hipLaunchKernelGGL((merge_rows_kernel<false, false>), g, b, 0, stream, m);
    }
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
