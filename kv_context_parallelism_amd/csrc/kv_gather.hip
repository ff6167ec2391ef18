// kv_gather.hip -- the inverse of the interleaved KV placement: N DCP shards'
// paged caches -> one contiguous, token-major window of every request's KV.
//
// What it computes: "Breaking the Long-Sequence Inference Bottleneck ...",
// section 3, "MLA path": the gathered KV of all ranks is reorganised into each
// request's own order before attention; section 2 gives the placement it
// inverts (owner rank floor(t / I) mod N, local index
// floor(t / (N I)) I + t mod I on that rank, then the rank's block table).
//
// HBM-bound copy: every cache byte of the window is read once and every
// output byte written once.  A workgroup takes 32 window rows of one request:
// its first 32 threads resolve each row's shard and cache row (the index math
// is done once per token, not per byte) into LDS; then each wave copies whole
// token rows, lane l moving 16-byte chunks l, l + 64, ... of the row, so the
// loads of a (token, head) row are contiguous and the stores of a token row
// are contiguous.  For rows of up to 128 chunks a wave issues the loads of
// all its 8 tokens before the first store.  The output is written with
// non-temporal stores (it is not read again by this kernel; streaming it past
// the caches took the call from 116 to 90 us on the prefix workload).
#include "internal.hpp"

namespace cpattn {

namespace {

constexpr int kTok = 32;      // window rows per workgroup
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

struct GatherParams {
    const gbyte *kc[CP_MAX_SHARDS];
    const gbyte *vc[CP_MAX_SHARDS];
    cint32 *bt[CP_MAX_SHARDS];
    int64_t nb[CP_MAX_SHARDS];
    cint32 *seq_len;
    int32_t N, I, bs, bt_stride, Hkv, t0, W;
    int32_t row_chunks;   // 16-byte chunks of one (token, head) row: D * elem / 16
    int32_t chunks_log2;  // log2(row_chunks) when Hkv > 1
    int64_t row_bytes;    // bytes of one (token, head) row
    uint8_t *ko, *vo;
};

// Row state in LDS: >= 0 cache row (units of one (token, head) row) of head 0;
// kZero past the request's length; kBad for a block id or local block index
// out of range.
constexpr int64_t kZero = -1, kBad = -2;

__global__ void __launch_bounds__(kThreads) gather_kernel(GatherParams p) {
    __shared__ int64_t s_row[kTok];
    __shared__ int32_t s_shard[kTok];
    const int b = blockIdx.y;
    const int i0 = blockIdx.x * kTok;
    const int tid = threadIdx.x;
    if (tid < kTok) {
        const int i = i0 + tid;
        int64_t row = kZero;
        int r = 0;
        const int64_t L = p.seq_len[b];
        if (i < p.W) {
            const int64_t t = (int64_t)p.t0 + i;
            if (t < L) {
                r = (int)((t / p.I) % p.N);
                const int64_t l = (t / ((int64_t)p.N * p.I)) * p.I + t % p.I;
                const int64_t blk = l / p.bs;
                row = kBad;
                if (blk < p.bt_stride) {
                    const int32_t phys = p.bt[r][(int64_t)b * p.bt_stride + blk];
                    if (phys >= 0 && (int64_t)phys < p.nb[r])
                        row = (int64_t)phys * p.Hkv * p.bs + l % p.bs;  // head h adds h * bs
                }
            }
        }
        s_row[tid] = row;
        s_shard[tid] = r;
    }
    __syncthreads();

    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int per_tok = p.Hkv * p.row_chunks;  // 16-byte chunks of a token row (one tensor)
    const int nrows = min(kTok, p.W - i0);
    // chunk c of a token row: head c / row_chunks, chunk c % row_chunks of that head
    auto src_off = [&](int64_t row, int c) -> int64_t {
        const int h = p.Hkv > 1 ? c >> p.chunks_log2 : 0;
        const int cc = p.Hkv > 1 ? c & (p.row_chunks - 1) : c;
        return (row + (int64_t)h * p.bs) * p.row_bytes + cc * 16;
    };
    if (per_tok <= 2 * 64) {
        // Token rows of up to 128 chunks: each wave moves kBatch tokens at a
        // time, all their loads issued before the first store.
        constexpr int kBatch = kTok / kWaves;
        u32x4 kx[kBatch][2], vx[kBatch][2];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int j = wave + u * kWaves;
            if (j >= nrows) break;
            const int64_t row = __builtin_amdgcn_readfirstlane(s_row[j]);
            const int r = __builtin_amdgcn_readfirstlane(s_shard[j]);
            const u32x4 fill = row == kBad ? u32x4{~0u, ~0u, ~0u, ~0u} : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int c = lane + 64 * h2;
                kx[u][h2] = fill;
                vx[u][h2] = fill;
                if (c < per_tok && row >= 0) {
                    const int64_t so = src_off(row, c);
                    kx[u][h2] = load16(p.kc[r] + so);
                    if (p.vo) vx[u][h2] = load16(p.vc[r] + so);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int j = wave + u * kWaves;
            if (j >= nrows) break;
            const int64_t out_off = ((int64_t)b * p.W + i0 + j) * per_tok * 16;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int c = lane + 64 * h2;
                if (c < per_tok) {
                    store16_stream(p.ko + out_off + c * 16, kx[u][h2]);
                    if (p.vo) store16_stream(p.vo + out_off + c * 16, vx[u][h2]);
                }
            }
        }
        return;
    }
    for (int j = wave; j < nrows; j += kWaves) {
        const int64_t row = __builtin_amdgcn_readfirstlane(s_row[j]);  // uniform per token
        const int r = __builtin_amdgcn_readfirstlane(s_shard[j]);
        const int64_t out_off = ((int64_t)b * p.W + i0 + j) * per_tok * 16;
        const u32x4 fill = row == kBad ? u32x4{~0u, ~0u, ~0u, ~0u} : u32x4{0u, 0u, 0u, 0u};
        for (int c = lane; c < per_tok; c += 64) {
            if (row >= 0) {
                const int64_t src = src_off(row, c);
                const u32x4 kx = load16(p.kc[r] + src);
                if (p.vo) {
                    const u32x4 vx = load16(p.vc[r] + src);
                    store16_stream(p.vo + out_off + c * 16, vx);
                }
                store16_stream(p.ko + out_off + c * 16, kx);
            } else {
                store16_stream(p.ko + out_off + c * 16, fill);
                if (p.vo) store16_stream(p.vo + out_off + c * 16, fill);
            }
        }
    }
}

bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

}  // namespace

}  // namespace cpattn

using namespace cpattn;

extern "C" cp_status cp_kv_gather(const cp_kv_gather_args *a, hipStream_t stream) {
    clear_error();
    if (!a) return fail(CP_E_INVALID, "cp_kv_gather: NULL args");
    if (a->N < 1 || a->N > CP_MAX_SHARDS || a->I < 1 || a->bs < 1 || a->B < 0 || a->Hkv < 1 ||
        a->D < 1 || a->bt_stride < 1 || a->t0 < 0 || a->W < 0)
        return fail(CP_E_INVALID, "kv gather: N=%d I=%d bs=%d B=%d Hkv=%d D=%d bt_stride=%d t0=%d W=%d",
                    a->N, a->I, a->bs, a->B, a->Hkv, a->D, a->bt_stride, a->t0, a->W);
    const int eb = elem_bytes(a->dt);
    if (eb == 0) return fail(CP_E_INVALID, "kv gather: unknown dtype %d", (int)a->dt);
    const int64_t row_bytes = (int64_t)a->D * eb;
    if (row_bytes % 16 != 0)
        return fail(CP_E_UNSUPPORTED, "kv gather: a row of %d elements is not a multiple of 16 bytes",
                    a->D);
    const int64_t row_chunks = row_bytes / 16;
    if (a->Hkv > 1 && (!pow2(a->Hkv) || !pow2(row_chunks)))
        return fail(CP_E_UNSUPPORTED,
                    "kv gather: with Hkv=%d > 1, Hkv and D*elem/16=%lld must be powers of two", a->Hkv,
                    (long long)row_chunks);
    if ((int64_t)a->Hkv * row_chunks > (1 << 20))
        return fail(CP_E_UNSUPPORTED, "kv gather: token rows of %lld bytes",
                    (long long)(a->Hkv * row_bytes));
    if ((a->v_caches == nullptr) != (a->v_out == nullptr))
        return fail(CP_E_INVALID, "kv gather: v_caches and v_out must both be given or both NULL");
    if (a->B == 0 || a->W == 0) return CP_OK;
    if (!a->k_caches || !a->block_tables || !a->num_blocks || !a->seq_len || !a->k_out)
        return fail(CP_E_INVALID, "kv gather: NULL pointer");
    if (!aligned16(a->k_out) || (a->v_out && !aligned16(a->v_out)))
        return fail(CP_E_INVALID, "kv gather: outputs must be 16-byte aligned");
    GatherParams p{};
    for (int r = 0; r < a->N; ++r) {
        if (!a->k_caches[r] || !a->block_tables[r] || (a->v_caches && !a->v_caches[r]))
            return fail(CP_E_INVALID, "kv gather: NULL pointer for shard %d", r);
        if (!aligned16(a->k_caches[r]) || (a->v_caches && !aligned16(a->v_caches[r])))
            return fail(CP_E_INVALID, "kv gather: shard %d caches must be 16-byte aligned", r);
        if (a->num_blocks[r] < 0) return fail(CP_E_INVALID, "kv gather: num_blocks[%d] < 0", r);
        p.kc[r] = to_global(a->k_caches[r]);
        p.vc[r] = a->v_caches ? to_global(a->v_caches[r]) : nullptr;
        p.bt[r] = to_const(a->block_tables[r]);
        p.nb[r] = a->num_blocks[r];
    }
    p.seq_len = to_const(a->seq_len);
    p.N = a->N;
    p.I = a->I;
    p.bs = a->bs;
    p.bt_stride = a->bt_stride;
    p.Hkv = a->Hkv;
    p.t0 = a->t0;
    p.W = a->W;
    p.row_chunks = (int32_t)row_chunks;
    int lg = 0;
    while ((int64_t(1) << lg) < row_chunks) ++lg;
    p.chunks_log2 = lg;
    p.row_bytes = row_bytes;
    p.ko = static_cast<uint8_t *>(a->k_out);
    p.vo = static_cast<uint8_t *>(a->v_out);
    const int64_t gx = ((int64_t)a->W + kTok - 1) / kTok;
    if (gx > 0x7fffffff || a->B > 65535)
        return fail(CP_E_UNSUPPORTED, "kv gather: grid of %lld x %d workgroups", (long long)gx, a->B);
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)gx, (unsigned)a->B), dim3(kThreads), 0, stream, p);
    return check_launch("cp_kv_gather");
}
