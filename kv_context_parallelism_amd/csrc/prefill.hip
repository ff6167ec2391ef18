// prefill.hip -- PCP load-balanced causal prefill attention on gfx950 matrix
// cores: rank r's two pieces of the new chunk against either the chunk's own
// keys (causal) or one DCP shard of the cached prefix (no mask).
//
// What it computes:
//   "Breaking the Long-Sequence Inference Bottleneck ...", section 4,
//   "Head-tail concatenation strategy" and "Minimal state progression": the
//   chunk is cut into 2N equal pieces and rank r computes pieces r and
//   2N-1-r; attention is causal (a token sees itself and earlier positions).
//   Section 5, "AllGather Q path": full queries against a partial (DCP shard)
//   KV give a partial result, merged exactly with the others afterwards.
//   "vLLM DCP and PCP: Decode and Prefill Context Parallelism", Deep Dive 6:
//   partial output and LSE per key set.
//
// Design:
//   * workgroup = G waves (the query heads of one KV head) x 32 query rows of
//     one piece; every 64-key K/V tile staged in LDS serves all G heads;
//   * K/V tiles go from HBM straight into a double-buffered, row-padded LDS
//     ring (global_load_lds); scores S^T = K Q^T on v_mfma_f32_16x16x32_bf16
//     with the wave's queries held in registers; the score tile is already in
//     the A-operand layout of the value product; V is read by the transposing
//     LDS read ds_read_b64_tr_b16;
//   * online softmax in the exp2 domain; causal masking only on the diagonal
//     tile (key position <= query position), tiles past the diagonal are never
//     visited;
//   * blockIdx % Hkv is the KV head, so the workgroups reading one head's keys
//     share an XCD (and its L2); query blocks are issued longest-first.
#include <math.h>

#include "internal.hpp"

namespace cpattn {

namespace {

constexpr int kD = 128;
constexpr int kBM = 32;                  // query rows per workgroup
constexpr int kBN = 64;                  // keys per tile
constexpr int kRowB = kD * 2 + 16;       // padded LDS row (272 B)
constexpr int kTileB = kBN * kRowB;      // one K or V tile in LDS
constexpr int kMaxWaves = 8;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T *)(p))

struct PrefillParams {
    const gbyte *q;
    const gbyte *k, *v;           // dense: [C][Hkv][D]
    const gbyte *kc, *vc;         // paged: [nblk][Hkv][bs][D]
    cint32 *bt;
    int32_t local_len, bs_log2;
    int64_t num_blocks;
    int32_t C, pcp_rank, pcp_size, Hq, Hkv, G;
    float qk_scale;               // scale * log2(e)
    int32_t nqb;                  // query blocks per piece
    float *out, *lse;
};

__device__ __forceinline__ f32x4_t mfma16(const u32x4_t &a, const u32x4_t &b, const f32x4_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, static_cast<__bf16>(lo)) |
           ((uint32_t)__builtin_bit_cast(uint16_t, static_cast<__bf16>(hi)) << 16);
}

template <bool kPaged>
__global__ void __launch_bounds__(64 * kMaxWaves) prefill_kernel(PrefillParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t s_k[2][kTileB];
    __shared__ __attribute__((aligned(16))) uint8_t s_v[2][kTileB];

    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int nwaves = nthr >> 6;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G4 = lane >> 4, j16 = lane & 15;

    // ---- work item: KV head innermost (one XCD per head), longest first ----
    const int g = blockIdx.x % p.Hkv;
    const int f = blockIdx.x / p.Hkv;               // 0 .. 2*nqb-1
    const int piece_slot = f < p.nqb ? 1 : 0;       // tail piece first
    const int qb = p.nqb - 1 - (f % p.nqb);         // last rows first
    const int npieces = 2 * p.pcp_size;
    const int piece = piece_slot == 0 ? p.pcp_rank : npieces - 1 - p.pcp_rank;
    const int c = p.C / npieces;                    // rows per piece
    const int i0 = piece * c + qb * kBM;            // first query row (chunk index)
    const int h = g * p.G + wave;                   // this wave's query head

    // keys visible to the block: causal -> [0, i0 + 32); paged shard -> [0, local_len)
    const int32_t kend = kPaged ? p.local_len : min(i0 + kBM, p.C);
    const int bs = 1 << p.bs_log2;

    // ---- queries as the B operand: Q[i0 + 16 mb + j16][h][32 ks + 8 G4 .. +8] ----
    u32x4_t qb_reg[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int row = i0 + 16 * mb + j16;
        gbyte *qrow = p.q + ((int64_t)row * p.Hq + h) * (kD * 2) + G4 * 16;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qb_reg[mb][ks] = load16(qrow + ks * 64);
    }

    // ---- tile staging: 64 key rows of K and V straight into LDS ----
    bool bad = false;
    auto key_row = [&](int32_t t, const gbyte *dense, const gbyte *paged) -> const gbyte * {
        if constexpr (kPaged) {
            int32_t phys = p.bt[t >> p.bs_log2];
            const bool ok = phys >= 0 && (int64_t)phys < p.num_blocks;
            bad |= !ok;
            phys = ok ? phys : 0;
            return paged + (((int64_t)phys * p.Hkv + g) * bs + (t & (bs - 1))) * (kD * 2);
        } else {
            return dense + ((int64_t)t * p.Hkv + g) * (kD * 2);
        }
    };
    auto stage_issue = [&](int32_t j0, int buf) {
        constexpr int kPer = kRowB / 16;              // 17 LDS chunks per row (16 data + pad)
        constexpr int kSlots = (kBN * kPer + 63) / 64;
        for (int sl = wave; sl < 2 * kSlots; sl += nwaves) {
            const bool isv = sl >= kSlots;
            const int s2 = isv ? sl - kSlots : sl;
            const int cidx = s2 * 64 + lane;
            const int tt = cidx / kPer, ch = cidx - tt * kPer;
            // the row's physical block is uniform per 16 keys: read it once per row group
            const bool ok = tt < kBN && ch < 16 && j0 + tt < kend;
            if (ok) {
                const gbyte *src = key_row(j0 + tt, isv ? p.v : p.k, isv ? p.vc : p.kc) + ch * 16;
                uint8_t *dst = (isv ? s_v[buf] : s_k[buf]) + s2 * 1024;
                __builtin_amdgcn_global_load_lds((const CP_GLOBAL void *)src,
                                                 (__attribute__((address_space(3))) void *)dst, 16,
                                                 0, 0);
            }
        }
    };
    // rows past the visible range are zeroed (probability 0 must not meet NaN bits)
    auto stage_zero_tail = [&](int32_t j0, int buf) {
        if (j0 + kBN <= kend) return;
        const u32x4_t z = {0u, 0u, 0u, 0u};
        for (int cidx = tid; cidx < kBN * 16; cidx += nthr) {
            const int tt = cidx >> 4, ch = cidx & 15;
            if (j0 + tt >= kend) {
                *reinterpret_cast<u32x4_t *>(s_k[buf] + tt * kRowB + ch * 16) = z;
                *reinterpret_cast<u32x4_t *>(s_v[buf] + tt * kRowB + ch * 16) = z;
            }
        }
    };

    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
    f32x4_t o[2][8];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int db = 0; db < 8; ++db) o[mb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    int buf = 0;
    if (kend > 0) stage_issue(0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (kend > 0 && kBN > kend) {
        stage_zero_tail(0, 0);
        __syncthreads();
    }
    for (int32_t j0 = 0; j0 < kend; j0 += kBN) {
        const int32_t jn = j0 + kBN;
        const bool has_next = jn < kend;
        if (has_next) stage_issue(jn, buf ^ 1);
        const uint8_t *tk = s_k[buf];
        const uint8_t *tv = s_v[buf];

        // ---- scores S^T[key][row]: 4 key blocks x 2 row blocks ----
        f32x4_t sc[2][4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const uint8_t *arow = tk + (kb * 16 + j16) * kRowB + G4 * 16;
            u32x4_t a[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) a[ks] = *reinterpret_cast<const u32x4_t *>(arow + ks * 64);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) acc = mfma16(a[ks], qb_reg[mb][ks], acc);
                sc[mb][kb] = acc;
            }
        }
        // lane holds keys j0 + 16 kb + 4 G4 + e for query row i0 + 16 mb + j16
        const bool diag = !kPaged && (j0 + kBN - 1 > i0);  // some key may follow some row
        float alpha[2];
        u32x4_t pa[2][2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int qrow = i0 + 16 * mb + j16;
            float mt = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int key = j0 + 16 * kb + 4 * G4 + e;
                    float s = sc[mb][kb][e] * p.qk_scale;
                    if (key >= kend || (diag && key > qrow)) s = -INFINITY;
                    sc[mb][kb][e] = s;
                    mt = fmaxf(mt, s);
                }
            mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
            mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
            const float mn = fmaxf(m_run[mb], mt);
            // a row with no visible key yet keeps m = -inf: use 0 as the shift
            const float ms = mn == -INFINITY ? 0.f : mn;
            alpha[mb] = fast_exp2(m_run[mb] - ms);
            m_run[mb] = mn;
            float ps = 0.f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sc[mb][kb][e] = fast_exp2(sc[mb][kb][e] - ms);
                    ps += sc[mb][kb][e];
                }
            l_run[mb] = l_run[mb] * alpha[mb] + ps;
            // P as A operand for 32-key steps: k = 8 G4 + e <-> key blocks (2s, 2s+1)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                pa[mb][s2][0] = pack2_bf16(sc[mb][2 * s2][0], sc[mb][2 * s2][1]);
                pa[mb][s2][1] = pack2_bf16(sc[mb][2 * s2][2], sc[mb][2 * s2][3]);
                pa[mb][s2][2] = pack2_bf16(sc[mb][2 * s2 + 1][0], sc[mb][2 * s2 + 1][1]);
                pa[mb][s2][3] = pack2_bf16(sc[mb][2 * s2 + 1][2], sc[mb][2 * s2 + 1][3]);
            }
        }
        // rescale output rows 16 mb + 4 G4 + e
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            float ar[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) ar[e] = __shfl(alpha[mb], G4 * 4 + e, 64);
#pragma unroll
            for (int db = 0; db < 8; ++db)
#pragma unroll
                for (int e = 0; e < 4; ++e) o[mb][db][e] *= ar[e];
        }
        // ---- values: O[row][d] += P[row][key] V[key][d] ----
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const uint8_t *vrow0 = tv + (32 * s2 + 4 * G4 + (j16 >> 2)) * kRowB + (j16 & 3) * 8;
            const uint8_t *vrow1 = vrow0 + 16 * kRowB;
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                const i16x4_t t0 =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4_t, vrow0 + db * 32));
                const i16x4_t t1 =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4_t, vrow1 + db * 32));
                u32x4_t vb;
                vb[0] = (uint32_t)(uint16_t)t0[0] | ((uint32_t)(uint16_t)t0[1] << 16);
                vb[1] = (uint32_t)(uint16_t)t0[2] | ((uint32_t)(uint16_t)t0[3] << 16);
                vb[2] = (uint32_t)(uint16_t)t1[0] | ((uint32_t)(uint16_t)t1[1] << 16);
                vb[3] = (uint32_t)(uint16_t)t1[2] | ((uint32_t)(uint16_t)t1[3] << 16);
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) o[mb][db] = mfma16(pa[mb][s2], vb, o[mb][db]);
            }
        }

        __builtin_amdgcn_s_waitcnt(0x0F70);  // the next tile has landed
        __syncthreads();
        if (has_next && jn + kBN > kend) {
            stage_zero_tail(jn, buf ^ 1);
            __syncthreads();
        }
        buf ^= 1;
    }

    // ---- finish: normalise and write rows of this piece ----
    bad = __syncthreads_or(bad);
    const int local0 = qb * kBM;  // row within the piece
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        float lt = l_run[mb];
        lt += __shfl_xor(lt, 16, 64);
        lt += __shfl_xor(lt, 32, 64);
        float inv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float le = __shfl(lt, G4 * 4 + e, 64);
            inv[e] = bad ? NAN : (le > 0.f ? 1.f / le : 0.f);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = local0 + 16 * mb + 4 * G4 + e;
            float *dst = p.out + (((int64_t)piece_slot * c + r) * p.Hq + h) * kD;
#pragma unroll
            for (int db = 0; db < 8; ++db) dst[db * 16 + j16] = o[mb][db][e] * inv[e];
        }
        if (lane < 16) {
            const int r = local0 + 16 * mb + lane;
            p.lse[((int64_t)piece_slot * c + r) * p.Hq + h] =
                bad ? NAN : (m_run[mb] == -INFINITY ? -INFINITY
                                                    : (m_run[mb] + fast_log2(lt)) * kLn2);
        }
    }
}

int log2_exact(int32_t x) {
    if (x <= 0 || (x & (x - 1))) return -1;
    int l = 0;
    while ((1 << l) < x) ++l;
    return l;
}

}  // namespace

}  // namespace cpattn

using namespace cpattn;

extern "C" cp_status pcp_prefill_attn_causal(const cp_prefill_args *a, void *ws, size_t ws_bytes,
                                             hipStream_t stream) {
    (void)ws;
    (void)ws_bytes;
    clear_error();
    if (!a) return fail(CP_E_INVALID, "pcp_prefill_attn_causal: NULL args");
    if (a->C < 0 || a->P < 0 || a->pcp_size < 1 || a->pcp_rank < 0 || a->pcp_rank >= a->pcp_size ||
        a->Hq < 1 || a->Hkv < 1 || a->D < 1)
        return fail(CP_E_INVALID, "prefill: C=%d P=%d rank=%d size=%d Hq=%d Hkv=%d D=%d", a->C, a->P,
                    a->pcp_rank, a->pcp_size, a->Hq, a->Hkv, a->D);
    if (a->C % (2 * a->pcp_size) != 0)
        return fail(CP_E_INVALID, "prefill: chunk length %d is not a multiple of 2 x %d", a->C,
                    a->pcp_size);
    if (a->Hq % a->Hkv != 0) return fail(CP_E_INVALID, "prefill: Hq %% Hkv != 0");
    const int G = a->Hq / a->Hkv;
    if (a->D != kD) return fail(CP_E_UNSUPPORTED, "prefill: head dim %d (128 supported)", a->D);
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(CP_E_UNSUPPORTED, "prefill: Hq/Hkv = %d not in {1, 2, 4, 8}", G);
    const int rows = a->C / (2 * a->pcp_size);
    if (rows % kBM != 0)
        return fail(CP_E_UNSUPPORTED, "prefill: piece of %d rows is not a multiple of %d", rows,
                    kBM);
    if (a->kv_source != CP_KV_DENSE && a->kv_source != CP_KV_PAGED)
        return fail(CP_E_INVALID, "prefill: kv_source %d", a->kv_source);
    if (!(a->scale == a->scale)) return fail(CP_E_INVALID, "prefill: scale is NaN");
    if (a->C == 0) return CP_OK;
    if (!a->q || !a->out || !a->lse) return fail(CP_E_INVALID, "prefill: NULL pointer");
    PrefillParams p{};
    p.q = to_global(a->q);
    int bs_log2 = 4;
    if (a->kv_source == CP_KV_DENSE) {
        if (!a->k || !a->v) return fail(CP_E_INVALID, "prefill: dense source needs k and v");
        if (!aligned16(a->k) || !aligned16(a->v))
            return fail(CP_E_INVALID, "prefill: k/v must be 16-byte aligned");
        p.k = to_global(a->k);
        p.v = to_global(a->v);
    } else {
        if (!a->k_cache || !a->v_cache || !a->block_table)
            return fail(CP_E_INVALID, "prefill: paged source needs caches and a block table");
        if (a->local_len < 0 || (int64_t)a->local_len > (int64_t)a->bt_stride * a->bs)
            return fail(CP_E_INVALID, "prefill: local_len %d beyond the block table", a->local_len);
        bs_log2 = log2_exact(a->bs);
        if (bs_log2 < 4)
            return fail(CP_E_UNSUPPORTED, "prefill: block size %d must be a power of two >= 16",
                        a->bs);
        if (!aligned16(a->k_cache) || !aligned16(a->v_cache))
            return fail(CP_E_INVALID, "prefill: caches must be 16-byte aligned");
        p.kc = to_global(a->k_cache);
        p.vc = to_global(a->v_cache);
        p.bt = to_const(a->block_table);
        p.local_len = a->local_len;
        p.num_blocks = a->num_blocks;
    }
    p.bs_log2 = bs_log2;
    p.C = a->C;
    p.pcp_rank = a->pcp_rank;
    p.pcp_size = a->pcp_size;
    p.Hq = a->Hq;
    p.Hkv = a->Hkv;
    p.G = G;
    p.qk_scale = a->scale * kLog2e;
    p.nqb = rows / kBM;
    p.out = a->out;
    p.lse = a->lse;
    const int64_t blocks = (int64_t)2 * p.nqb * a->Hkv;
    if (blocks > 0x7fffffff) return fail(CP_E_UNSUPPORTED, "prefill: too many query blocks");
    const int threads = 64 * G;
    if (a->kv_source == CP_KV_PAGED)
        hipLaunchKernelGGL(prefill_kernel<true>, dim3((unsigned)blocks), dim3(threads), 0, stream, p);
    else
        hipLaunchKernelGGL(prefill_kernel<false>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                           p);
    return check_launch("pcp_prefill_attn_causal");
}
