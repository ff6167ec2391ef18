// slot_map.hip -- interleaved KV ownership, local lengths, slot mapping and the
// paged cache write.
//
// "Breaking the Long-Sequence Inference Bottleneck: A Deep Dive into vLLM's
// Distributed Context Parallelism Architecture", section 2 ("Interleave Size"
// rank formula; "Diagram: Actual mapping of the Block Table and Slot
// Mapping": tokens another rank owns map to -1 and are skipped), and
// "vLLM DCP and PCP: Decode and Prefill Context Parallelism", Deep Dive 5
// (virtual blocks, local sequence lengths).
//
// All three kernels are integer index math plus a bitwise copy: HBM-bound,
// one thread per token (index kernels) or per 16-byte chunk (copy).
#include "internal.hpp"

namespace cpattn {

// Tokens rank r owns among positions [0, L): complete rounds of N*I positions
// give I each; the partial round gives r its share of the remainder.
__device__ __forceinline__ int32_t local_len_of(int64_t L, int32_t r, int32_t N, int32_t I) {
    if (L <= 0) return 0;
    int64_t round = (int64_t)N * I;
    int64_t full = L / round, rem = L % round;
    int64_t part = rem - (int64_t)r * I;
    part = part < 0 ? 0 : (part > I ? I : part);
    return (int32_t)(full * I + part);
}

__global__ void local_lens_kernel(int32_t B, const int32_t *__restrict__ seq_lens, int32_t rank,
                                  int32_t N, int32_t I, int32_t *__restrict__ out) {
    int32_t b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) out[b] = local_len_of(seq_lens[b], rank, N, I);
}

// Slot of token (request b, position t) on `rank`, or a sentinel: not this
// rank's position (-1), or an invalid request, position or local block (-2).
__device__ __forceinline__ int64_t slot_of(int32_t b, int32_t t, const int32_t *__restrict__ block_table,
                                           int32_t B, int32_t bt_stride, int32_t max_blocks,
                                           int32_t rank, int32_t N, int32_t I, int32_t bs) {
    if (b < 0 || b >= B || t < 0) return CP_SLOT_INVALID;
    const int32_t group = t / I;         // interleave group of the position
    if (group % N != rank) return CP_SLOT_NOT_MINE;  // owner = floor(t / I) mod N
    const int32_t l = (group / N) * I + (t - group * I);  // l <= t, fits in 32 bits
    const int32_t blk = l / bs;
    if (blk >= max_blocks) return CP_SLOT_INVALID;
    return (int64_t)block_table[(int64_t)b * bt_stride + blk] * bs + (l - blk * bs);
}

__global__ void slot_map_kernel(int32_t T, const int32_t *__restrict__ req,
                                const int32_t *__restrict__ pos,
                                const int32_t *__restrict__ block_table, int32_t B,
                                int32_t bt_stride, int32_t max_blocks, int32_t rank, int32_t N,
                                int32_t I, int32_t bs, int64_t *__restrict__ slot_out) {
    int32_t j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= T) return;
    slot_out[j] = slot_of(req[j], pos[j], block_table, B, bt_stride, max_blocks, rank, N, I, bs);
}

__global__ void cache_write_kernel(int32_t T, const int64_t *__restrict__ slot,
                                   const u32x4 *__restrict__ k, const u32x4 *__restrict__ v,
                                   uint32_t n_heads, uint32_t row_chunks,
                                   u32x4 *__restrict__ k_cache, u32x4 *__restrict__ v_cache,
                                   int64_t num_slots, int32_t bs, int32_t bs_log2) {
    const uint32_t per_tok = n_heads * row_chunks;
    const uint32_t idx = blockIdx.x * blockDim.x + threadIdx.x;
    const uint32_t j = idx / per_tok;
    if (j >= (uint32_t)T) return;
    const uint32_t c = idx - j * per_tok;
    // the row chunk is loaded together with the slot (one round trip)
    const int64_t src = (int64_t)j * per_tok + c;
    const u32x4 kx = k[src];
    const u32x4 vx = v ? v[src] : u32x4{0u, 0u, 0u, 0u};
    const int64_t s = slot[j];
    if (s < 0 || s >= num_slots) return;
    const uint32_t h = c / row_chunks;
    const uint32_t cc = c - h * row_chunks;
    int64_t blk, off;
    if (bs_log2 >= 0) {
        blk = s >> bs_log2;
        off = s & (bs - 1);
    } else {
        blk = s / bs;
        off = s - blk * bs;
    }
    const int64_t dst = ((blk * n_heads + h) * bs + off) * row_chunks + cc;
    k_cache[dst] = kx;
    if (v) v_cache[dst] = vx;
}


// Both steps in one launch: thread (token j, 16-byte chunk c) computes the
// token's slot itself (a few integer operations), the chunk-0 thread stores it
// when slot_out is given, and every thread copies its chunk like
// cache_write_kernel.
__global__ void slot_map_write_kernel(int32_t T, const int32_t *__restrict__ req,
                                      const int32_t *__restrict__ pos,
                                      const int32_t *__restrict__ block_table, int32_t B,
                                      int32_t bt_stride, int32_t max_blocks, int32_t rank,
                                      int32_t N, int32_t I, int32_t bs, int64_t *__restrict__ slot_out,
                                      const u32x4 *__restrict__ k, const u32x4 *__restrict__ v,
                                      uint32_t n_heads, uint32_t row_chunks,
                                      u32x4 *__restrict__ k_cache, u32x4 *__restrict__ v_cache,
                                      int64_t num_slots, int32_t bs_log2) {
    const uint32_t per_tok = n_heads * row_chunks;
    const uint32_t idx = blockIdx.x * blockDim.x + threadIdx.x;
    const uint32_t j = idx / per_tok;
    if (j >= (uint32_t)T) return;
    const uint32_t c = idx - j * per_tok;
    // the row chunk does not depend on the slot: load it first, so that its
    // latency overlaps the slot's (position, then block table) loads
    const int64_t src = (int64_t)j * per_tok + c;
    const u32x4 kx = k[src];
    const u32x4 vx = v ? v[src] : u32x4{0u, 0u, 0u, 0u};
    // request and position in one round trip (not the position after the
    // request's range check)
    int32_t rq = req[j], ps = pos[j];
    asm volatile("" : "+v"(rq), "+v"(ps));
    const int64_t s = slot_of(rq, ps, block_table, B, bt_stride, max_blocks, rank, N, I, bs);
    if (c == 0 && slot_out) slot_out[j] = s;
    if (s < 0 || s >= num_slots) return;
    const uint32_t h = c / row_chunks;
    const uint32_t cc = c - h * row_chunks;
    int64_t blk, off;
    if (bs_log2 >= 0) {
        blk = s >> bs_log2;
        off = s & (bs - 1);
    } else {
        blk = s / bs;
        off = s - blk * bs;
    }
    const int64_t dst = ((blk * n_heads + h) * bs + off) * row_chunks + cc;
    k_cache[dst] = kx;
    if (v) v_cache[dst] = vx;
}
}  // namespace cpattn

using namespace cpattn;

extern "C" cp_status cp_local_seq_lens(int32_t B, const int32_t *seq_lens, int32_t rank, int32_t N,
                                       int32_t I, int32_t *local_lens, hipStream_t stream) {
    clear_error();
    if (B < 0 || N < 1 || I < 1 || rank < 0 || rank >= N)
        return fail(CP_E_INVALID, "cp_local_seq_lens: B=%d N=%d I=%d rank=%d", B, N, I, rank);
    if (B == 0) return CP_OK;
    if (!seq_lens || !local_lens) return fail(CP_E_INVALID, "cp_local_seq_lens: NULL pointer");
    hipLaunchKernelGGL(local_lens_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, B, seq_lens,
                       rank, N, I, local_lens);
    return check_launch("cp_local_seq_lens");
}

extern "C" cp_status cp_slot_map(int32_t T, const int32_t *req, const int32_t *pos,
                                 const int32_t *block_table, int32_t B, int32_t bt_stride,
                                 int32_t max_blocks, int32_t rank, int32_t N, int32_t I,
                                 int32_t bs, int64_t *slot_out, hipStream_t stream) {
    clear_error();
    if (T < 0 || B < 1 || N < 1 || I < 1 || bs < 1 || rank < 0 || rank >= N || max_blocks < 1 ||
        max_blocks > bt_stride)
        return fail(CP_E_INVALID,
                    "cp_slot_map: T=%d B=%d N=%d I=%d bs=%d rank=%d max_blocks=%d bt_stride=%d", T,
                    B, N, I, bs, rank, max_blocks, bt_stride);
    if (T == 0) return CP_OK;
    if (!req || !pos || !block_table || !slot_out)
        return fail(CP_E_INVALID, "cp_slot_map: NULL pointer");
    hipLaunchKernelGGL(slot_map_kernel, dim3((T + 255) / 256), dim3(256), 0, stream, T, req, pos,
                       block_table, B, bt_stride, max_blocks, rank, N, I, bs, slot_out);
    return check_launch("cp_slot_map");
}

extern "C" cp_status cp_cache_write(int64_t T, const int64_t *slot, const void *k, const void *v,
                                    int32_t n_kv_heads, int32_t row_dim, cp_dtype dt, void *k_cache,
                                    void *v_cache, int64_t num_blocks, int32_t bs,
                                    hipStream_t stream) {
    clear_error();
    int eb = elem_bytes(dt);
    if (T < 0 || n_kv_heads < 1 || row_dim < 1 || num_blocks < 0 || bs < 1 || eb == 0)
        return fail(CP_E_INVALID, "cp_cache_write: T=%lld heads=%d row_dim=%d num_blocks=%lld bs=%d",
                    (long long)T, n_kv_heads, row_dim, (long long)num_blocks, bs);
    if ((v == nullptr) != (v_cache == nullptr))
        return fail(CP_E_INVALID, "cp_cache_write: give both v and v_cache, or neither");
    if (((int64_t)row_dim * eb) % 16 != 0)
        return fail(CP_E_UNSUPPORTED, "cp_cache_write: row of %d bytes is not a multiple of 16",
                    row_dim * eb);
    if (T == 0) return CP_OK;
    if (!slot || !k || !k_cache) return fail(CP_E_INVALID, "cp_cache_write: NULL pointer");
    if (!aligned16(k) || !aligned16(k_cache) || (v && (!aligned16(v) || !aligned16(v_cache))))
        return fail(CP_E_INVALID, "cp_cache_write: data pointers must be 16-byte aligned");
    const int32_t row_chunks = (int32_t)(((int64_t)row_dim * eb) / 16);
    const int64_t per_tok = (int64_t)n_kv_heads * row_chunks;
    if (per_tok > (1 << 20)) return fail(CP_E_UNSUPPORTED, "cp_cache_write: rows too wide");
    int bs_log2 = -1;
    if ((bs & (bs - 1)) == 0)
        for (bs_log2 = 0; (1 << bs_log2) < bs; ++bs_log2) {
        }
    // launches of < 2^31 chunks each
    const int64_t tok_per_launch = ((int64_t)1 << 30) / per_tok;
    for (int64_t t0 = 0; t0 < T; t0 += tok_per_launch) {
        const int32_t tn = (int32_t)(T - t0 < tok_per_launch ? T - t0 : tok_per_launch);
        const int64_t total = (int64_t)tn * per_tok;
        const u32x4 *kp = (const u32x4 *)k + t0 * per_tok;
        const u32x4 *vp = v ? (const u32x4 *)v + t0 * per_tok : nullptr;
        hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0,
                           stream, tn, slot + t0, kp, vp, (uint32_t)n_kv_heads,
                           (uint32_t)row_chunks, (u32x4 *)k_cache, (u32x4 *)v_cache,
                           num_blocks * bs, bs, bs_log2);
    }
    return check_launch("cp_cache_write");
}

extern "C" cp_status cp_slot_map_cache_write(int32_t T, const int32_t *req, const int32_t *pos,
                                             const int32_t *block_table, int32_t B,
                                             int32_t bt_stride, int32_t max_blocks, int32_t rank,
                                             int32_t N, int32_t I, int32_t bs, int64_t *slot_out,
                                             const void *k, const void *v, int32_t n_kv_heads,
                                             int32_t row_dim, cp_dtype dt, void *k_cache,
                                             void *v_cache, int64_t num_blocks, hipStream_t stream) {
    clear_error();
    const int eb = elem_bytes(dt);
    if (T < 0 || B < 1 || N < 1 || I < 1 || bs < 1 || rank < 0 || rank >= N || max_blocks < 1 ||
        max_blocks > bt_stride || n_kv_heads < 1 || row_dim < 1 || num_blocks < 0 || eb == 0)
        return fail(CP_E_INVALID,
                    "cp_slot_map_cache_write: T=%d B=%d N=%d I=%d bs=%d rank=%d max_blocks=%d "
                    "bt_stride=%d heads=%d row_dim=%d num_blocks=%lld",
                    T, B, N, I, bs, rank, max_blocks, bt_stride, n_kv_heads, row_dim,
                    (long long)num_blocks);
    if ((v == nullptr) != (v_cache == nullptr))
        return fail(CP_E_INVALID, "cp_slot_map_cache_write: give both v and v_cache, or neither");
    if (((int64_t)row_dim * eb) % 16 != 0)
        return fail(CP_E_UNSUPPORTED,
                    "cp_slot_map_cache_write: row of %d bytes is not a multiple of 16", row_dim * eb);
    if (T == 0) return CP_OK;
    if (!req || !pos || !block_table || !k || !k_cache)
        return fail(CP_E_INVALID, "cp_slot_map_cache_write: NULL pointer");
    if (!aligned16(k) || !aligned16(k_cache) || (v && (!aligned16(v) || !aligned16(v_cache))))
        return fail(CP_E_INVALID, "cp_slot_map_cache_write: data pointers must be 16-byte aligned");
    const int32_t row_chunks = (int32_t)(((int64_t)row_dim * eb) / 16);
    const int64_t per_tok = (int64_t)n_kv_heads * row_chunks;
    if (per_tok > (1 << 20)) return fail(CP_E_UNSUPPORTED, "cp_slot_map_cache_write: rows too wide");
    int bs_log2 = -1;
    if ((bs & (bs - 1)) == 0)
        for (bs_log2 = 0; (1 << bs_log2) < bs; ++bs_log2) {
        }
    // launches of < 2^31 chunks each
    const int64_t tok_per_launch = ((int64_t)1 << 30) / per_tok;
    for (int64_t t0 = 0; t0 < T; t0 += tok_per_launch) {
        const int32_t tn = (int32_t)(T - t0 < tok_per_launch ? T - t0 : tok_per_launch);
        const int64_t total = (int64_t)tn * per_tok;
        const u32x4 *kp = (const u32x4 *)k + t0 * per_tok;
        const u32x4 *vp = v ? (const u32x4 *)v + t0 * per_tok : nullptr;
        hipLaunchKernelGGL(slot_map_write_kernel, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0,
                           stream, tn, req + t0, pos + t0, block_table, B, bt_stride, max_blocks,
                           rank, N, I, bs, slot_out ? slot_out + t0 : nullptr, kp, vp,
                           (uint32_t)n_kv_heads, (uint32_t)row_chunks, (u32x4 *)k_cache,
                           (u32x4 *)v_cache, num_blocks * bs, bs_log2);
    }
    return check_launch("cp_slot_map_cache_write");
}
