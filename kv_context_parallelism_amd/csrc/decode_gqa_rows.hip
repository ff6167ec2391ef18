// decode_gqa_rows.hip -- GQA decode partial for 256-byte KV rows (bf16 head
// dim 128, fp32 head dim 64): row-layout waves over a balanced flat schedule.
//
// What it computes: "vLLM DCP and PCP: Decode and Prefill Context
// Parallelism", Deep Dive 6, "Deriving the partial and global outputs" --
// every rank applies the same query to its own KV shard and returns the
// shard-normalised output o_i and L_i = log sum_j exp(s_j).
//
// Work distribution.  The (request, KV head, 32-token chunk) space is laid
// out flat, request-major.  Exactly W waves are launched (four per CU, all
// resident at once) and wave w takes the contiguous chunk range
// [w*R/W, (w+1)*R/W) of the R chunks, so every wave streams the same number of
// KV bytes whatever the mix of context lengths.  A wave whose range crosses
// from one (request, KV head) into the next writes one partial per piece to
// slot  w + (request * Hkv + head).  At most R waves are scheduled, so each
// owns at least one chunk and the waves covering one (request, head) are
// consecutive: its partials occupy consecutive slots, and workgroup 0 records
// (first slot, count) per (request, head) for the exact LSE merge that follows.
//
// Wave layout.  Lane = (token row R = lane / 16, 16-byte chunk c = lane % 16).
// One load instruction reads 4 consecutive tokens' full rows (1 KB,
// contiguous): K for the scores, V for the weighted sum use the same layout.
// Partial dot products of the 4 tokens x G query heads are summed over the 16
// lanes of a row by an in-register reduce-scatter (DPP), leaving one finished
// score per lane (G = 4), so the online softmax does one exp per lane per 16
// tokens.  Probabilities are regrouped per row through a small LDS buffer; the
// V product uses packed bf16 dot2 over token pairs (fp32 accumulate).
// Loads are software-pipelined: the next tile's K is requested after this
// tile's scores, its V after this tile's V product.
//
// Multi-token queries (a separate instantiation): the G rows per KV head are
// q_len tokens x Hq/Hkv heads, and each row sees the shard's keys up to its
// token's position; tiles past the first token's limit mask per row.
#include <math.h>

#include <type_traits>

#include "internal.hpp"

namespace cpattn {

namespace {

constexpr int kWaves = 4;       // waves per workgroup
constexpr int kTile = 32;       // tokens per tile = per scheduling chunk
constexpr int kNG = kTile / 16; // 16-token groups per tile
constexpr int kMaxB = 8192;     // requests handled by the in-LDS prefix sum
// Register bound for the compiler: at least 2 workgroups per CU.
constexpr int kMinWgPerCu = 2;
// Workgroups the schedule spreads the work over, per CU.  One (a wave per
// SIMD) measured faster than filling the CU with the 2-3 that fit: each
// (request, KV head) is split into fewer partials for the combine, and the
// four waves' loads in flight already keep HBM busy.
constexpr int kSchedWgPerCu = 1;

struct RowParams {
    const gbyte *q, *kc, *vc;
    cint32 *bt, *len;
    int32_t B, Hq, Hkv, bs_log2, bt_stride;
    int64_t num_blocks;
    float qk_scale;   // softmax scale * log2(e)
    int32_t W;        // waves launched
    float *ws_o;      // [slots][G][D]
    float *ws_l;      // [slots][G]
    int32_t *seg;     // [B*Hkv][2]: first slot, count
    // Multi-token queries: the kernel's G = Tg x Greal rows per KV head are
    // query token t0 + t (the request's position seq_len - T + t0 + t) of
    // head g Greal + h, row t Greal + h, for the launch's Tg tokens t0 ..
    // t0 + Tg - 1 of the request's T.  A token sees the shard's keys at
    // positions <= its own (seq_len == nullptr: T = 1, no limit).
    const int32_t *seq_len;
    int32_t T, t0, Greal;
    int32_t dcp_rank, dcp_size, dcp_I;
};

// Positions below x held by DCP rank r of N with interleave I ("Breaking the
// Long-Sequence Inference Bottleneck ...", section 2: the owner of position t
// is floor(t / I) mod N): whole rounds of N I positions give I each, the
// partial round the overlap of [0, x mod N I) with [r I, r I + I).  A shard's
// local keys are its positions in increasing order, so this is also the
// number of local keys a query at position x - 1 may see.
__device__ __forceinline__ int32_t owned_below(int32_t x, int32_t r, int32_t N, int32_t I) {
    if (x <= 0) return 0;
    const int32_t round = N * I;
    const int32_t q = x / round, rem = x - q * round;
    return q * I + min(max(rem - r * I, 0), I);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int CTRL, int BANKS = 0xF>
__device__ __forceinline__ float dpp(float old, float v) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, 0xF, BANKS, false));
}

// Value of lane (lane ^ M) within a row of 16 lanes.
template <int M>
__device__ __forceinline__ float xor_row(float v) {
    if constexpr (M == 1) return dpp<0xB1>(0.f, v);          // quad_perm [1,0,3,2]
    else if constexpr (M == 2) return dpp<0x4E>(0.f, v);     // quad_perm [2,3,0,1]
    else if constexpr (M == 8) return dpp<0x128>(0.f, v);    // row_ror:8
    else {                                                   // M == 4
        float t = dpp<0x104, 0x5>(0.f, v);                   // row_shl:4 into lanes 0-3, 8-11
        return dpp<0x114, 0xA>(t, v);                        // row_shr:4 into lanes 4-7, 12-15
    }
}

// Broadcast the value of quad position Q to all four lanes of each quad.
template <int Q>
__device__ __forceinline__ float quad_bcast(float v) {
    return dpp<Q * 0x55>(0.f, v);
}

// One reduce-scatter step over lane mask M: n values -> n/2, the lanes with the
// M bit set keeping the upper half.  With n == 1 the last value is summed.
template <int M, int N>
__device__ __forceinline__ void rs_step(float *v, bool up) {
    if constexpr (N >= 2) {
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            const float keep = up ? v[i + N / 2] : v[i];
            const float give = up ? v[i] : v[i + N / 2];
            v[i] = keep + xor_row<M>(give);
        }
    } else {
        v[0] += xor_row<M>(v[0]);
    }
}

// Sum NV values over the 16 lanes of a row.  Afterwards lane c holds
//   NV >= 16: the sums of values c*(NV/16) + k, k < NV/16, in v[k];
//   NV <  16: the sum of value c / (16/NV) in v[0].
template <int NV>
__device__ __forceinline__ void row_reduce_scatter(float *v, int c) {
    rs_step<8, NV>(v, c & 8);
    rs_step<4, (NV >= 2 ? NV / 2 : 1)>(v, c & 4);
    rs_step<2, (NV >= 4 ? NV / 4 : 1)>(v, c & 2);
    rs_step<1, (NV >= 8 ? NV / 8 : 1)>(v, c & 1);
}

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint16_t bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// smallest wave index whose range contains chunk c: the w with
// floor(w*R/W) <= c < floor((w+1)*R/W)
__device__ __forceinline__ int64_t owner_of(int64_t c, int64_t R, int64_t W) {
    return ((c + 1) * W - 1) / R;
}

template <int EB, int G, int MINWG, bool kMtp>
__global__ void __launch_bounds__(64 * kWaves, MINWG) gqa_rows_kernel(RowParams p) {
    constexpr bool kBf16 = (EB == 2);
    constexpr int D = 256 / EB;                 // 128 bf16 or 64 fp32
    constexpr int EPC = 16 / EB;                // elements per 16-byte chunk
    constexpr int NV = 4 * G;                   // partial sums per lane per 16-token group
    constexpr int NF = NV >= 16 ? NV / 16 : 1;  // finished scores per lane per group
    constexpr int REP = NV >= 16 ? 1 : 16 / NV; // lanes sharing one finished score
    constexpr int PW = kBf16 ? 4 * kNG * 2 * G : 4 * kNG * 4 * G;  // LDS words per wave

    __shared__ int32_t s_pref[kMaxB + 1];
    __shared__ uint32_t s_p[kWaves][PW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int R = lane >> 4, c = lane & 15, qp = c & 3;
    const int64_t cap = (int64_t)p.bt_stride << p.bs_log2;
    const int bs = 1 << p.bs_log2;

    // ---- chunks per request and their prefix sum (every workgroup) ----
    // a request with an invalid length is given one chunk, processed as NaN
    auto chunks_of = [&](int32_t L) -> int32_t {
        if (L < 0 || (int64_t)L > cap) return 1;
        return (L + kTile - 1) / kTile;
    };
    // Below 64 requests every wave scans the chunk counts by itself (lane l
    // holds request l's exclusive prefix, lane B the total): no LDS, no
    // barrier, and a chunk's request is one ballot.  More requests take the
    // workgroup-wide scan into LDS and a binary search.
    const bool wave_pref = p.B < 64;
    int32_t prefv = 0;
    if (wave_pref) {
        const int32_t cnt = lane < p.B ? chunks_of(p.len[lane]) : 0;
        int32_t incl = cnt;
#pragma unroll
        for (int x = 1; x < 64; x <<= 1) {
            const int32_t o = __shfl_up(incl, x, 64);
            if (lane >= x) incl += o;
        }
        prefv = incl - cnt;
        if (blockIdx.x == 0) {  // workgroup 0 publishes the segment table from LDS below
            if (tid <= p.B) s_pref[tid] = prefv;
            __syncthreads();
        }
    } else {
        const int per = (p.B + 64 * kWaves - 1) / (64 * kWaves);
        const int b0 = tid * per;
        int32_t run = 0;
        for (int i = 0; i < per && b0 + i < p.B; ++i) run += chunks_of(p.len[b0 + i]);
        // block-wide exclusive scan of the per-thread totals
        int32_t incl = run;
#pragma unroll
        for (int x = 1; x < 64; x <<= 1) {
            const int32_t o = __shfl_up(incl, x, 64);
            if (lane >= x) incl += o;
        }
        __shared__ int32_t s_wsum[kWaves];
        if (lane == 63) s_wsum[tid >> 6] = incl;
        __syncthreads();
        int32_t base = 0;
        for (int i = 0; i < (tid >> 6); ++i) base += s_wsum[i];
        int32_t acc = base + incl - run;
        for (int i = 0; i < per && b0 + i < p.B; ++i) {
            s_pref[b0 + i] = acc;
            acc += chunks_of(p.len[b0 + i]);
        }
        if (tid == 64 * kWaves - 1) s_pref[p.B] = base + incl;
        __syncthreads();
    }
    // Waves actually scheduled: never more than there are chunks, so every
    // scheduled wave owns at least one chunk and the waves covering one
    // (request, head) are consecutive -- which makes its partial slots consecutive.
    // values read back from LDS are the same in every lane: keep them scalar
    auto pref = [&](int i) -> int32_t {
        return wave_pref ? __builtin_amdgcn_readlane(prefv, i) : __builtin_amdgcn_readfirstlane(s_pref[i]);
    };
    const int64_t R_tot = (int64_t)p.Hkv * pref(p.B);
    const int64_t W = R_tot < p.W ? R_tot : p.W;

    // ---- workgroup 0 publishes (first slot, count) of every (request, head) ----
    if (blockIdx.x == 0) {
        for (int bg = tid; bg < p.B * p.Hkv; bg += 64 * kWaves) {
            const int b = bg / p.Hkv, g = bg - b * p.Hkv;
            const int64_t n = s_pref[b + 1] - s_pref[b];
            int32_t first = 0, count = 0;
            if (n > 0) {
                const int64_t F = (int64_t)p.Hkv * s_pref[b] + g * n;
                const int64_t o0 = owner_of(F, R_tot, W), o1 = owner_of(F + n - 1, R_tot, W);
                first = (int32_t)(o0 + bg);
                count = (int32_t)(o1 - o0 + 1);
            }
            p.seg[2 * bg] = first;
            p.seg[2 * bg + 1] = count;
        }
    }

    const int64_t w = (int64_t)blockIdx.x * kWaves + wave;
    if (w >= W || R_tot == 0) return;
    int64_t cc = w * R_tot / W;
    const int64_t hi = (w + 1) * R_tot / W;
    const u32x4 zero4 = {0u, 0u, 0u, 0u};

    while (cc < hi) {
        // ---- locate chunk cc: request b, KV head g, chunk k of (b, g) ----
        int lo_b = 0, hi_b = p.B;  // largest b with Hkv * pref[b] <= cc
        if (wave_pref) {  // the prefixes rise with b: count the lanes b < B at or below cc
            const uint64_t m = __ballot(lane < p.B && (int64_t)p.Hkv * prefv <= cc);
            lo_b = __popcll(m) - 1;
        } else {
            while (hi_b - lo_b > 1) {
                const int mid = (lo_b + hi_b) >> 1;
                if ((int64_t)p.Hkv * pref(mid) <= cc) lo_b = mid;
                else hi_b = mid;
            }
        }
        const int b = __builtin_amdgcn_readfirstlane(lo_b);
        const int32_t pb = pref(b);
        const int32_t n = pref(b + 1) - pb;
        if (n == 0) {  // only reachable through empty requests sharing a prefix value
            // (the search returns the last b with that prefix, which has n > 0)
            break;
        }
        const int64_t rem = cc - (int64_t)p.Hkv * pb;
        const int g = (int)(rem / n);
        const int32_t k = (int32_t)(rem - (int64_t)g * n);
        const int32_t nseg = (int32_t)min<int64_t>(hi - cc, n - k);
        const int32_t Lraw = p.len[b];
        bool bad = Lraw < 0 || (int64_t)Lraw > cap;
        const int32_t L = bad ? 0 : Lraw;
        const int32_t s0 = k * kTile;
        const int32_t s1 = min(s0 + nseg * kTile, L);
        const int64_t slot = w + (int64_t)b * p.Hkv + g;
        cint32 *bt_row = p.bt + (int64_t)b * p.bt_stride;
        // Key limits: row hh (query token hh / Greal) sees local keys below
        // lim[k2] of this piece; min_lim is the first token's, the smallest.
        int32_t qpos0 = 0;  // position of the launch's query token 0 (token t0 of the request)
        if constexpr (kMtp) {
            const int32_t first = p.seq_len[b] - p.T;  // position of the request's first query token
            bad |= first < 0;
            qpos0 = first + p.t0;
        }
        auto causal_lim = [&](int t) -> int32_t {
            if constexpr (!kMtp) return s1;
            return min(s1, owned_below(qpos0 + t + 1, p.dcp_rank, p.dcp_size, p.dcp_I));
        };
        const int32_t min_lim = causal_lim(0);
        int32_t lim[NF];
#pragma unroll
        for (int k2 = 0; k2 < NF; ++k2) {
            const int hh = NV >= 16 ? qp * NF + k2 : (qp / REP) % G;
            lim[k2] = causal_lim(hh / p.Greal);
        }

        // First cache row (head g) of the 16-token group at local index lb.  The
        // block id is a uniform (scalar) load, so waiting for it never waits for
        // the K/V vector loads in flight.  Groups past the segment's end map to
        // the group one tile earlier (the tile this wave is reading now, whose
        // lines are still in its L2) or, for the segment's first tile, to its
        // first group, so every address stays inside the cache and the
        // unconditional prefetch past the end fetches nothing new from HBM.
        auto group_row = [&](int32_t lb) -> int64_t {
            const int32_t gsel = lb < s1 ? lb : (lb - kTile >= s0 ? lb - kTile : s0);
            int32_t phys = bt_row[gsel >> p.bs_log2];
            const bool ok = phys >= 0 && (int64_t)phys < p.num_blocks;
            bad |= !ok;
            phys = ok ? phys : 0;
            return ((int64_t)phys * p.Hkv + g) * bs + (gsel & (bs - 1));
        };
        auto load_tile = [&](const gbyte *base, const int64_t (&rows)[kNG], u32x4 (&reg)[kNG][4]) {
#pragma unroll
            for (int gi = 0; gi < kNG; ++gi) {
                const gbyte *gp = base + rows[gi] * 256 + lane * 16;
#pragma unroll
                for (int j = 0; j < 4; ++j) reg[gi][j] = load16(gp + j * 1024);
            }
        };
        int64_t rows_cur[kNG], rows_next[kNG];

        float m[NF], lpart[NF], acc[G][EPC];
#pragma unroll
        for (int k2 = 0; k2 < NF; ++k2) {
            m[k2] = -INFINITY;
            lpart[k2] = 0.f;
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[hh][e] = 0.f;

        // Prologue: the first tile's K and V, then the query chunk c of the G
        // heads (lane-private), all in flight together; then wait for all of
        // them, so that the loop is entered with nothing in flight and the
        // waits inside, set by its back edge (K then V of the next tile in
        // flight), stay exact.  The query's latency overlaps the tile's.
        u32x4 kreg[kNG][4], vreg[kNG][4];
        if (s1 > s0) {
#pragma unroll
            for (int gi = 0; gi < kNG; ++gi) rows_cur[gi] = group_row(s0 + gi * 16);
            load_tile(p.kc, rows_cur, kreg);
            load_tile(p.vc, rows_cur, vreg);
        }
        u32x4 qraw[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const int t = hh / p.Greal, h = hh - t * p.Greal;
            qraw[hh] = load16(p.q + (((int64_t)b * p.T + p.t0 + t) * p.Hq + g * p.Greal + h) * 256 + c * 16);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        float qf[kBf16 ? 1 : G][4];
        if constexpr (!kBf16) {
#pragma unroll
            for (int hh = 0; hh < G; ++hh)
#pragma unroll
                for (int e = 0; e < 4; ++e) qf[hh][e] = __uint_as_float(qraw[hh][e]) * p.qk_scale;
        }
        // One tile.  kTail: the segment's last tile is partial -- scores of
        // tokens past the end become -inf and their V rows (which may hold NaN
        // poison) are zeroed right before the V product.  Full tiles carry no
        // masking at all, so no wait on the V loads is forced before the scores.
        auto tile = [&](int32_t tb, auto tail_tag) {
            constexpr bool kTail = decltype(tail_tag)::value;
            const int32_t tn = tb + kTile;
            // keys of this tile past some row's limit (multi-token queries)
            const bool mask = kTail || (kMtp && tn > min_lim);
            // Block ids of the next tile, early: they are needed after the scores.
            // Full tiles always prefetch (past the segment's end the rows clamp to
            // the current tile and the reads hit the cache): a conditional
            // prefetch would make the compiler copy the live V registers, which
            // forces a wait on every load in flight.
            if constexpr (!kTail) {
#pragma unroll
                for (int gi = 0; gi < kNG; ++gi) rows_next[gi] = group_row(tn + gi * 16);
            }

            // ---- scores: partial dots, then reduce-scatter over the row ----
            float sc[kNG][NF];
#pragma unroll
            for (int gi = 0; gi < kNG; ++gi) {
                float v[NV];
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int hh = 0; hh < G; ++hh) {
                        float a = 0.f;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if constexpr (kBf16)
                                a = dot2_bf16(kreg[gi][j][e], qraw[hh][e], a);
                            else
                                a = fmaf(__uint_as_float(kreg[gi][j][e]), qf[hh][e], a);
                        }
                        v[j * G + hh] = a;
                    }
                row_reduce_scatter<NV>(v, c);
                // this lane's scores belong to token (c >> 2) of its row
                const int32_t tok = tb + gi * 16 + (c >> 2) * 4 + R;
#pragma unroll
                for (int k2 = 0; k2 < NF; ++k2) {
                    const bool ok = !mask || tok < lim[k2];
                    sc[gi][k2] = ok ? (kBf16 ? v[k2] * p.qk_scale : v[k2]) : -INFINITY;
                }
            }
            if constexpr (!kTail) load_tile(p.kc, rows_next, kreg);

            // ---- online softmax: max over the lanes holding the same head ----
            float alpha[NF];
#pragma unroll
            for (int k2 = 0; k2 < NF; ++k2) {
                float mt = sc[0][k2];
#pragma unroll
                for (int gi = 1; gi < kNG; ++gi) mt = fmaxf(mt, sc[gi][k2]);
                mt = fmaxf(mt, xor_row<4>(mt));
                mt = fmaxf(mt, xor_row<8>(mt));
                mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
                mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
                const float mn = fmaxf(m[k2], mt);
                // a row with no visible key yet (multi-token queries) keeps
                // m = -inf: no rescale, and its masked scores give 0
                const float mref = kMtp && mn == -INFINITY ? 0.f : mn;
                alpha[k2] = kMtp && mn == -INFINITY ? 1.f : fast_exp2(m[k2] - mn);
                m[k2] = mn;
                float ps = 0.f;
#pragma unroll
                for (int gi = 0; gi < kNG; ++gi) {
                    sc[gi][k2] = fast_exp2(sc[gi][k2] - mref);
                    ps += sc[gi][k2];
                }
                lpart[k2] = lpart[k2] * alpha[k2] + ps;
            }
            // rescale the accumulators of every head by that head's alpha
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                float ah;
                if constexpr (NV >= 16) {
                    // head hh is value hh % NF of quad position hh / NF
                    const float src = alpha[hh % NF];
                    const int q = hh / NF;
                    ah = q == 0 ? quad_bcast<0>(src)
                                : (q == 1 ? quad_bcast<1>(src)
                                          : (q == 2 ? quad_bcast<2>(src) : quad_bcast<3>(src)));
                } else {
                    // head hh is held by quad position hh * (4 / G)
                    const int q = hh * (4 / G);
                    ah = q == 0 ? quad_bcast<0>(alpha[0])
                                : (q == 1 ? quad_bcast<1>(alpha[0])
                                          : (q == 2 ? quad_bcast<2>(alpha[0])
                                                    : quad_bcast<3>(alpha[0])));
                }
#pragma unroll
                for (int e = 0; e < EPC; ++e) acc[hh][e] *= ah;
            }

            // ---- probabilities of the row's tokens to every lane of the row ----
            wave_sync();
            if ((c & (REP - 1)) == 0) {
                const int tok = c >> 2;
#pragma unroll
                for (int gi = 0; gi < kNG; ++gi)
#pragma unroll
                    for (int k2 = 0; k2 < NF; ++k2) {
                        const int hh = NV >= 16 ? qp * NF + k2 : (qp / REP) % G;
                        if constexpr (kBf16) {
                            const int idx = (((R * kNG + gi) * 2 + (tok >> 1)) * G + hh) * 2 + (tok & 1);
                            reinterpret_cast<uint16_t *>(s_p[wave])[idx] = bf16_bits(sc[gi][k2]);
                        } else {
                            const int idx = ((R * kNG + gi) * 4 + tok) * G + hh;
                            reinterpret_cast<float *>(s_p[wave])[idx] = sc[gi][k2];
                        }
                    }
            }
            wave_sync();

            if constexpr (kTail) {
#pragma unroll
                for (int gi = 0; gi < kNG; ++gi)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (tb + gi * 16 + j * 4 + R >= s1) vreg[gi][j] = zero4;
            }

            // ---- V product ----
#pragma unroll
            for (int gi = 0; gi < kNG; ++gi) {
                if constexpr (kBf16) {
#pragma unroll
                    for (int pi = 0; pi < 2; ++pi) {
                        uint32_t pw[G];
#pragma unroll
                        for (int hh = 0; hh < G; ++hh)
                            pw[hh] = s_p[wave][((R * kNG + gi) * 2 + pi) * G + hh];
                        const u32x4 v0 = vreg[gi][2 * pi], v1 = vreg[gi][2 * pi + 1];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t lo = __builtin_amdgcn_perm(v1[e], v0[e], 0x05040100u);
                            const uint32_t hi2 = __builtin_amdgcn_perm(v1[e], v0[e], 0x07060302u);
#pragma unroll
                            for (int hh = 0; hh < G; ++hh) {
                                acc[hh][2 * e] = dot2_bf16(lo, pw[hh], acc[hh][2 * e]);
                                acc[hh][2 * e + 1] = dot2_bf16(hi2, pw[hh], acc[hh][2 * e + 1]);
                            }
                        }
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float pv[G];
#pragma unroll
                        for (int hh = 0; hh < G; ++hh)
                            pv[hh] = reinterpret_cast<const float *>(
                                s_p[wave])[((R * kNG + gi) * 4 + j) * G + hh];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float vv = __uint_as_float(vreg[gi][j][e]);
#pragma unroll
                            for (int hh = 0; hh < G; ++hh) acc[hh][e] = fmaf(pv[hh], vv, acc[hh][e]);
                        }
                    }
                }
            }
            if constexpr (!kTail) {
                load_tile(p.vc, rows_next, vreg);
#pragma unroll
                for (int gi = 0; gi < kNG; ++gi) rows_cur[gi] = rows_next[gi];
            }
        };
        int32_t tb = s0;
        for (; tb + kTile <= s1; tb += kTile) tile(tb, std::false_type{});
        if (tb < s1) tile(tb, std::true_type{});

        // ---- finish the segment: full sums, normalise, write the partial ----
        bad = __ballot(bad) != 0;
        float lsum[NF];
#pragma unroll
        for (int k2 = 0; k2 < NF; ++k2) {
            float t = lpart[k2];
            t += xor_row<4>(t);
            t += xor_row<8>(t);
            t += __shfl_xor(t, 16, 64);
            t += __shfl_xor(t, 32, 64);
            lsum[k2] = t;
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                acc[hh][e] += __shfl_xor(acc[hh][e], 16, 64);
                acc[hh][e] += __shfl_xor(acc[hh][e], 32, 64);
            }
        float *o_dst = p.ws_o + slot * G * D;
        float *l_dst = p.ws_l + slot * G;
        const bool empty = !(s1 > s0);  // bad request: nothing was read
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            float lh;
            if constexpr (NV >= 16) {
                const float src = lsum[hh % NF];
                const int q = hh / NF;
                lh = q == 0 ? quad_bcast<0>(src)
                            : (q == 1 ? quad_bcast<1>(src)
                                      : (q == 2 ? quad_bcast<2>(src) : quad_bcast<3>(src)));
            } else {
                const int q = hh * (4 / G);
                lh = q == 0 ? quad_bcast<0>(lsum[0])
                            : (q == 1 ? quad_bcast<1>(lsum[0])
                                      : (q == 2 ? quad_bcast<2>(lsum[0]) : quad_bcast<3>(lsum[0])));
            }
            if (R == 0) {
                // a row without any visible key of this piece: 0 and LSE -inf
                const float inv = bad ? NAN : (empty || !(lh > 0.f) ? 0.f : 1.f / lh);
                float *dst = o_dst + hh * D + c * EPC;
#pragma unroll
                for (int e = 0; e < EPC; e += 4)
                    *reinterpret_cast<float4 *>(dst + e) =
                        make_float4(acc[hh][e] * inv, acc[hh][e + 1] * inv, acc[hh][e + 2] * inv,
                                    acc[hh][e + 3] * inv);
            }
        }
        if (R == 0 && c < 4 && (c & (REP - 1)) == 0) {
#pragma unroll
            for (int k2 = 0; k2 < NF; ++k2) {
                const int hh = NV >= 16 ? c * NF + k2 : c / REP;
                l_dst[hh] = bad ? NAN
                                : (empty || !(lsum[k2] > 0.f) ? -INFINITY
                                                              : (m[k2] + fast_log2(lsum[k2])) * kLn2);
            }
        }
        cc += nseg;
    }
}

template <int EB, int G>
cp_status launch_rows(const RowParams &p, hipStream_t stream) {
    const int64_t blocks = ceil_div(p.W, kWaves);
    if (p.seq_len)
        hipLaunchKernelGGL((gqa_rows_kernel<EB, G, kMinWgPerCu, true>), dim3((unsigned)blocks),
                           dim3(64 * kWaves), 0, stream, p);
    else
        hipLaunchKernelGGL((gqa_rows_kernel<EB, G, kMinWgPerCu, false>), dim3((unsigned)blocks),
                           dim3(64 * kWaves), 0, stream, p);
    return check_launch("cp_decode_attn_partial_gqa");
}

}  // namespace

bool gqa_rows_supported(const cp_gqa_args &a, int T) {
    const int G = a.Hkv > 0 ? a.Hq / a.Hkv * T : 0;
    const bool row256 = (a.dt == CP_BF16 && a.D == 128) || (a.dt == CP_F32 && a.D == 64);
    return row256 && (G == 1 || G == 2 || G == 4 || G == 8) && a.B <= kMaxB;
}

int gqa_mtp_group_tokens(const cp_gqa_args &a, int T) {
    const int Greal = a.Hkv > 0 ? a.Hq / a.Hkv : 0;
    if (Greal < 1 || Greal > 8 || (Greal & (Greal - 1)) || T < 1) return 0;
    int tg = T < 8 / Greal ? T : 8 / Greal;
    while (tg & (tg - 1)) tg &= tg - 1;  // the kernel takes 1, 2, 4 or 8 rows per KV head
    return tg;
}

int gqa_rows_waves(const cp_gqa_args &a, int T, bool mtp) {
    (void)a;
    (void)T;
    (void)mtp;
    return device_cus() * kSchedWgPerCu * kWaves;
}

cp_status gqa_rows_launch(const cp_gqa_args &a, int bs_log2, float *ws_o, float *ws_l,
                          int32_t *seg, int32_t W, const GqaMtp &mtp, hipStream_t stream) {
    RowParams p;
    p.q = to_global(a.q);
    p.kc = to_global(a.k_cache);
    p.vc = to_global(a.v_cache);
    p.bt = to_const(a.block_table);
    p.len = to_const(a.local_len);
    p.B = a.B;
    p.Hq = a.Hq;
    p.Hkv = a.Hkv;
    p.bs_log2 = bs_log2;
    p.bt_stride = a.bt_stride;
    p.num_blocks = a.num_blocks;
    p.qk_scale = a.scale * kLog2e;
    p.W = W;
    p.ws_o = ws_o;
    p.ws_l = ws_l;
    p.seg = seg;
    p.seq_len = mtp.seq_len;
    p.T = mtp.T;
    p.t0 = mtp.t0;
    p.Greal = a.Hq / a.Hkv;
    p.dcp_rank = mtp.dcp_rank;
    p.dcp_size = mtp.dcp_size;
    p.dcp_I = mtp.dcp_I;
    const int G = a.Hq / a.Hkv * (mtp.Tg > 0 ? mtp.Tg : mtp.T);  // rows per KV head
    if (a.dt == CP_BF16) {
        switch (G) {
        case 1: return launch_rows<2, 1>(p, stream);
        case 2: return launch_rows<2, 2>(p, stream);
        case 4: return launch_rows<2, 4>(p, stream);
        case 8: return launch_rows<2, 8>(p, stream);
        }
    } else {
        switch (G) {
        case 1: return launch_rows<4, 1>(p, stream);
        case 2: return launch_rows<4, 2>(p, stream);
        case 4: return launch_rows<4, 4>(p, stream);
        case 8: return launch_rows<4, 8>(p, stream);
        }
    }
    return fail(CP_E_UNSUPPORTED, "gqa decode: group size %d", G);
}

}  // namespace cpattn
