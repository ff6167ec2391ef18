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
//   * workgroup = R x G waves: the G query heads of one KV head times R blocks
//     of 32 query rows of one piece (R G = 8 where the piece allows: one
//     workgroup per CU, two waves per SIMD); every 64-key K/V tile staged in
//     LDS serves all R G waves, so the copy work per MFMA flop falls as 1 / R;
//   * K/V tiles go from HBM straight into a ring of kStages LDS buffers
//     (global_load_lds issued from asm and waited for with explicit vmcnt
//     counts, so the copies of the next tiles overlap the compute of this
//     one); the block ids of a tile are read once, by scalar loads;
//   * LDS rows are unpadded (256 bytes) with the 16-byte chunks of row t
//     XOR-swizzled by t % 16: the row-major score-operand reads and the
//     transposing value reads are both free of bank conflicts;
//   * scores S^T = K Q^T on v_mfma_f32_16x16x32_bf16 with the wave's queries
//     held in registers (each K read feeds both 16-row blocks, eight
//     independent accumulation chains interleaved); the score tile is already
//     in the A-operand layout of the value product; V is read by the
//     transposing LDS read ds_read_b64_tr_b16; LDS operands are requested
//     three steps ahead of their MFMA;
//   * online softmax in the exp2 domain with a lazily raised reference
//     maximum (rescale only past 2^8); causal masking only on tiles that
//     straddle a wave's diagonal (key position <= query position); a wave
//     skips the tiles past its own diagonal (the workgroup stages up to the
//     diagonal of its last row block); keys past the visible range reuse the
//     last visible row (finite data) and get probability 0;
//   * blockIdx % Hkv is the KV head, so the workgroups reading one head's keys
//     share an XCD (and its L2); query blocks are issued longest-first.
#include <math.h>

#include "internal.hpp"

namespace cpattn {

namespace {

constexpr int kD = 128;
constexpr int kBM = 32;                  // query rows per workgroup
constexpr int kBN = 64;                  // keys per tile
constexpr int kRowB = kD * 2;            // LDS row (256 B = 16 chunks)
constexpr int kTileB = kBN * kRowB;      // one K or V tile in LDS (16 KB)
constexpr int kSlots = 2 * kTileB / 1024;  // 64-lane copies per K+V tile pair (32)
constexpr int kMaxWaves = 8;
constexpr float kLazy = 8.f;
#ifndef PF_STAGES
#define PF_STAGES 2
#endif
constexpr int kStages = PF_STAGES;      // LDS ring of K/V tile pairs (32 KB each)
static_assert(kStages >= 2 && kStages * 2 * kTileB <= 160 * 1024, "ring fits the LDS");

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) const uint8_t lds_u8;

struct PrefillParams {
    const gbyte *q;
    const gbyte *k, *v;           // dense: [C][Hkv][D]
    const gbyte *kc, *vc;         // paged: [nblk][Hkv][bs][D]
    cint32 *bt;
    int32_t local_len, bs_log2;
    int64_t num_blocks;
    int32_t C, pcp_rank, pcp_size, Hq, Hkv, G;
    float qk_scale;               // scale * log2(e)
    int32_t nqb;                  // workgroup query blocks (R x 32 rows) per piece
    int32_t R, G_log2;            // row blocks per workgroup; log2 G
    float *out, *lse;
};

__device__ __forceinline__ f32x4_t mfma16(const u32x4_t &a, const u32x4_t &b, const f32x4_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// The lane id, recomputed where it is used: keeps per-lane addresses from
// being hoisted out of the tile loop and held in registers.
__device__ __forceinline__ int lane_id_here() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// One 64-lane HBM -> LDS copy: lane i moves 16 bytes from `src` to LDS byte
// lds + 16 i (`lds` wave-uniform).  Issued from asm so that the compiler's
// wait insertion does not tie the LDS reads of the tile being consumed to it;
// readers wait explicitly (vmcnt + barrier).  M0 is written here and read by
// nothing the compiler emits in this file.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(gbyte *src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds), "v"(src)
                 : "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Wait until at most n (wave-uniform, >= 0) of this wave's copies are
// outstanding, rounded down to a listed count (waiting for more is safe).
__device__ __forceinline__ void wait_copies_at_most(int n) {
    if (n >= 48) vm_wait<48>();
    else if (n >= 32) vm_wait<32>();
    else if (n >= 24) vm_wait<24>();
    else if (n >= 16) vm_wait<16>();
    else if (n >= 12) vm_wait<12>();
    else if (n >= 8) vm_wait<8>();
    else if (n >= 4) vm_wait<4>();
    else vm_wait<0>();
}

template <bool kPaged>
__global__ void __launch_bounds__(64 * kMaxWaves) prefill_kernel(PrefillParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t s_kv[kStages][2 * kTileB];  // [buf][K tile | V tile]

    const int tid = threadIdx.x;
    const int nwaves = blockDim.x >> 6;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hw = wave & (p.G - 1), rb = wave >> p.G_log2;  // head in the group, row block
    const int G4 = lane >> 4, j16 = lane & 15;

    // ---- work item: KV head innermost (one XCD per head), longest first ----
    const int g = blockIdx.x % p.Hkv;
    const int f = blockIdx.x / p.Hkv;               // 0 .. 2*nqb-1
    const int piece_slot = f < p.nqb ? 1 : 0;       // tail piece first
    const int qb = p.nqb - 1 - (f % p.nqb);         // last rows first
    const int npieces = 2 * p.pcp_size;
    const int piece = piece_slot == 0 ? p.pcp_rank : npieces - 1 - p.pcp_rank;
    const int c = p.C / npieces;                    // rows per piece
    const int i0 = piece * c + qb * kBM * p.R;      // first query row of the workgroup
    const int i0w = i0 + kBM * rb;                  // first query row of this wave
    const int h = g * p.G + hw;                     // this wave's query head

    // keys staged for the workgroup (causal: [0, i0 + 32 R); paged shard:
    // [0, local_len)) and keys visible to this wave's rows
    const int32_t kend = kPaged ? p.local_len : min(i0 + kBM * p.R, p.C);
    const int32_t kend_w = kPaged ? p.local_len : min(i0w + kBM, p.C);
    const int bs = 1 << p.bs_log2;

    // ---- queries as the B operand: Q[i0w + 16 mb + j16][h][32 ks + 8 G4 .. +8] ----
    u32x4_t qb_reg[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int row = i0w + 16 * mb + j16;
        gbyte *qrow = p.q + ((int64_t)row * p.Hq + h) * (kD * 2) + G4 * 16;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qb_reg[mb][ks] = load16(qrow + ks * 64);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): queries in registers before any copy

    // ---- tile staging: 64 key rows of K and V straight into LDS ----
    bool bad = false;
    const uint32_t kv_lds = (uint32_t)(uintptr_t)(lds_u8 *)(&s_kv[0][0]);
    auto stage_issue = [&](int32_t j0, int buf) {
        // base row of each 16-key group of the tile (uniform: scalar loads)
        int64_t base[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int32_t t = min(j0 + 16 * q4, kend - 1);
            if constexpr (kPaged) {
                int32_t phys = p.bt[t >> p.bs_log2];
                const bool ok = phys >= 0 && (int64_t)phys < p.num_blocks;
                bad |= !ok;
                phys = ok ? phys : 0;
                base[q4] = ((int64_t)phys * p.Hkv + g) * bs + (t & (bs - 1) & ~15);
            } else {
                base[q4] = (int64_t)(t & ~15) * p.Hkv + g;  // row index in units of D
            }
        }
        const uint32_t dst = kv_lds + (uint32_t)(buf * 2 * kTileB);
        const int ln = lane_id_here();
        const int l16 = ln >> 4, pos = ln & 15;
        if (j0 + kBN <= kend) {
            // full tile: copy sl holds rows 4 (sl % 16) .. +3, all in the 16-key
            // group q4 = (sl % 16) / 4; the per-lane part of the address is
            // row r16 = 4 (sl % 4) + lane / 16 of the group and chunk
            // (lane % 16) ^ r16 of that row
            constexpr int64_t kRow = kD * 2;
            const int64_t rstride = kPaged ? kRow : (int64_t)p.Hkv * kRow;
            for (int sl = wave; sl < kSlots; sl += nwaves) {
                const bool isv = sl >= kSlots / 2;
                const int s2 = sl & (kSlots / 2 - 1);
                const int q4 = s2 >> 2;
                const int64_t b4 = q4 == 0 ? base[0] : q4 == 1 ? base[1] : q4 == 2 ? base[2] : base[3];
                const gbyte *gbase =
                    (kPaged ? (isv ? p.vc : p.kc) : (isv ? p.v : p.k)) + b4 * kRow;  // uniform
                const int r16 = 4 * (s2 & 3) + l16;
                const uint32_t off = (uint32_t)(r16 * rstride) + (uint32_t)((pos ^ r16) * 16);
                dma16(gbase + off, __builtin_amdgcn_readfirstlane(dst + sl * 1024));
            }
        } else {
            for (int sl = wave; sl < kSlots; sl += nwaves) {
                const bool isv = sl >= kSlots / 2;
                const int tt = (sl & (kSlots / 2 - 1)) * 4 + l16;  // key row in the tile
                // clamp past the visible range to the last visible key (probability 0)
                const int tc = min(tt, kend - 1 - j0);
                const int q4 = tc >> 4, r16 = tc & 15;
                const int64_t b4 =
                    q4 == 0 ? base[0] : q4 == 1 ? base[1] : q4 == 2 ? base[2] : base[3];
                const int64_t row = kPaged ? b4 + r16 : b4 + (int64_t)r16 * p.Hkv;
                const gbyte *src = (kPaged ? (isv ? p.vc : p.kc) : (isv ? p.v : p.k)) +
                                   row * (kD * 2) + ((pos ^ (tt & 15)) * 16);
                dma16(src, __builtin_amdgcn_readfirstlane(dst + sl * 1024));
            }
        }
    };

    float m_ref[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
    f32x4_t o[2][8];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int db = 0; db < 8; ++db) o[mb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    constexpr int kPre = 3;
    const int ntile = kend > 0 ? (kend + kBN - 1) / kBN : 0;
    const int ntile_w = kend_w > 0 ? (kend_w + kBN - 1) / kBN : 0;  // a prefix of the tiles
    const int per_tile = kSlots / nwaves;  // this wave's copies per tile (nwaves divides 32)
#pragma unroll
    for (int j = 0; j < kStages - 1; ++j)
        if (j < ntile) stage_issue(j * kBN, j);
    for (int32_t it = 0; it < ntile; ++it) {
        // tile it has landed (own copies; later tiles may still be in flight) ...
        wait_copies_at_most(min(kStages - 2, ntile - 1 - it) * per_tile);
        __syncthreads();  // ... for every wave; the buffer of tile it - 1 is free again
        if (it + kStages - 1 < ntile) stage_issue((it + kStages - 1) * kBN, (it + kStages - 1) % kStages);
        if (it >= ntile_w) continue;  // past this wave's diagonal (uniform)
        const int32_t j0 = it * kBN;
        const int buf = it % kStages;
        lds_u8 *tk = (lds_u8 *)(&s_kv[buf][0]);
        lds_u8 *tv = tk + kTileB;

        // per-lane addresses (fresh lane id per tile).  Score operand of key
        // block kb, k-step ks: row 16 kb + j, chunk 4 ks + G; since rows
        // 16 kb + j share the swizzle j, ks only flips the chunk bits 2..3.
        // Value operand of column block db, key step s2: rows 32 s2 + 4 G + j / 4
        // (and + 16), chunk 2 db + (j % 4) / 2, byte 8 (j % 2).
        lds_u8 *ap[4], *vp[2];
        {
            const int ln = lane_id_here();
            const int G = ln >> 4, j = ln & 15;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) ap[ks] = tk + j * kRowB + 16 * ((4 * ks + G) ^ j);
            const int vr = 4 * G + (j >> 2);
            vp[0] = tv + vr * kRowB + 8 * (j & 1);
            vp[1] = tv + (vr + 16) * kRowB + 8 * (j & 1);
        }
        const int vr_sw = (4 * G4 + (j16 >> 2)) & 15;  // swizzle of both value rows
        auto read_a = [&](int i) -> u32x4_t {  // step i: ks = i / 4, kb = i % 4
            const int ks = i >> 2, kb = i & 3;
            return *(__attribute__((address_space(3))) const u32x4_t *)(ap[ks] + kb * 16 * kRowB);
        };
        auto read_v = [&](int i) -> u32x4_t {  // step i: s2 = i / 8, db = i % 8
            const int s2 = i >> 3, db = i & 7;
            const int chunk = (2 * db + ((j16 & 3) >> 1)) ^ vr_sw;
            lds_u8 *va0 = vp[0] + s2 * 32 * kRowB + chunk * 16;
            lds_u8 *va1 = vp[1] + s2 * 32 * kRowB + chunk * 16;
            const i16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4_t *)(va0));
            const i16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4_t *)(va1));
            const u32x2_t w0 = __builtin_bit_cast(u32x2_t, t0), w1 = __builtin_bit_cast(u32x2_t, t1);
            return u32x4_t{w0[0], w0[1], w1[0], w1[1]};
        };

        // ---- scores S^T[key][row]: 4 key blocks x 2 row blocks, k-step outer ----
        // (raw dot products; the scale is applied inside the exponent below)
        f32x4_t sc[2][4];
        {
            u32x4_t abuf[kPre];
#pragma unroll
            for (int i = 0; i < kPre; ++i) abuf[i] = read_a(i);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const u32x4_t a = abuf[i % kPre];
                if (i + kPre < 16) abuf[i % kPre] = read_a(i + kPre);
                const int ks = i >> 2, kb = i & 3;
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
                    sc[mb][kb] = mfma16(a, qb_reg[mb][ks],
                                        ks == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : sc[mb][kb]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // lane holds keys j0 + 16 kb + 4 G4 + e for query row i0 + 16 mb + j16.
        // Only tiles that reach past the visible keys or straddle the diagonal
        // need a mask (a uniform test).
        const bool diag = !kPaged && (j0 + kBN - 1 > i0w);  // some key may follow some row
        if (diag || j0 + kBN > kend_w) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                const int lim = min(kend_w, diag ? i0w + 16 * mb + j16 + 1 : kend_w) - j0 - 4 * G4;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (16 * kb + e >= lim) sc[mb][kb][e] = -INFINITY;
            }
        }
        u32x4_t pa[2][2];
        bool need = false;
        float mt[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            float m = fmaxf(sc[mb][0][0], sc[mb][0][1]);
            m = fmaxf(m, fmaxf(sc[mb][0][2], sc[mb][0][3]));
#pragma unroll
            for (int kb = 1; kb < 4; ++kb) {
                m = fmaxf(m, fmaxf(sc[mb][kb][0], sc[mb][kb][1]));  // v_max3
                m = fmaxf(m, fmaxf(sc[mb][kb][2], sc[mb][kb][3]));
            }
            m = fmaxf(m, __shfl_xor(m, 16, 64));
            m = fmaxf(m, __shfl_xor(m, 32, 64));
            mt[mb] = m * p.qk_scale;  // the scale is positive: max commutes with it
            need |= mt[mb] > m_ref[mb] + kLazy;
        }
        if (__any(need)) {
            // raise the reference maximum of the rows that need it and rescale
            // their partial sums and output rows 16 mb + 4 G4 + e
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                const float mn = mt[mb] > m_ref[mb] + kLazy ? mt[mb] : m_ref[mb];
                const float alpha = m_ref[mb] == -INFINITY ? 0.f : fast_exp2(m_ref[mb] - mn);
                m_ref[mb] = mn;
                l_run[mb] *= alpha;
                float ar[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) ar[e] = __shfl(alpha, G4 * 4 + e, 64);
#pragma unroll
                for (int db = 0; db < 8; ++db)
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[mb][db][e] *= ar[e];
            }
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            // p = 2^(s * scale - m_ref); a row with no visible key yet keeps the
            // reference at -inf and shifts by 0
            const float ms = m_ref[mb] == -INFINITY ? 0.f : m_ref[mb];
            // (the denominator is summed in fp32: the LSE needs more than the
            // bf16 precision of the weights)
            float ps = 0.f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sc[mb][kb][e] = fast_exp2(fmaf(sc[mb][kb][e], p.qk_scale, -ms));
                    ps += sc[mb][kb][e];
                }
            l_run[mb] += ps;
            // P as A operand for 32-key steps: k = 8 G4 + e <-> key blocks (2s, 2s+1)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                pa[mb][s2][0] = pack_bf16x2(sc[mb][2 * s2][0], sc[mb][2 * s2][1]);
                pa[mb][s2][1] = pack_bf16x2(sc[mb][2 * s2][2], sc[mb][2 * s2][3]);
                pa[mb][s2][2] = pack_bf16x2(sc[mb][2 * s2 + 1][0], sc[mb][2 * s2 + 1][1]);
                pa[mb][s2][3] = pack_bf16x2(sc[mb][2 * s2 + 1][2], sc[mb][2 * s2 + 1][3]);
            }
        }
        // ---- values: O[row][d] += P[row][key] V[key][d] ----
        {
            u32x4_t vbuf[kPre];
#pragma unroll
            for (int i = 0; i < kPre; ++i) vbuf[i] = read_v(i);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const u32x4_t vb = vbuf[i % kPre];
                if (i + kPre < 16) vbuf[i % kPre] = read_v(i + kPre);
                const int s2 = i >> 3, db = i & 7;
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) o[mb][db] = mfma16(pa[mb][s2], vb, o[mb][db]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // ---- finish: normalise and write rows of this piece ----
    bad = __syncthreads_or(bad);
    const int local0 = (qb * p.R + rb) * kBM;  // row within the piece
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
                bad ? NAN : (m_ref[mb] == -INFINITY || !(lt > 0.f)
                                 ? -INFINITY
                                 : (m_ref[mb] + fast_log2(lt)) * kLn2);
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
    if (!(a->scale > 0.f) || !(a->scale < INFINITY))
        return fail(CP_E_INVALID, "prefill: the softmax scale must be positive and finite");
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
    // R row blocks per workgroup: eight waves where the piece's row blocks divide
    int R = 8 / G;
    while (R > 1 && (rows / kBM) % R != 0) R /= 2;
    int G_log2 = 0;
    while ((1 << G_log2) < G) ++G_log2;
    p.R = R;
    p.G_log2 = G_log2;
    p.nqb = rows / (kBM * R);
    p.out = a->out;
    p.lse = a->lse;
    const int64_t blocks = (int64_t)2 * p.nqb * a->Hkv;
    if (blocks > 0x7fffffff) return fail(CP_E_UNSUPPORTED, "prefill: too many query blocks");
    const int threads = 64 * G * R;
    if (a->kv_source == CP_KV_PAGED)
        hipLaunchKernelGGL(prefill_kernel<true>, dim3((unsigned)blocks), dim3(threads), 0, stream, p);
    else
        hipLaunchKernelGGL(prefill_kernel<false>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                           p);
    return check_launch("pcp_prefill_attn_causal");
}
