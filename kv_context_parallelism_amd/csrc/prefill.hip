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
//     XOR-swizzled by swz(t % 16), which swaps the two 2-bit halves of t % 16:
//     the row-major score-operand reads (32 rows, one chunk) and the
//     transposing value reads (4 rows, 4 chunks per 32 lanes) are both free of
//     bank conflicts (measured; the plain t % 16 swizzle leaves the value
//     reads with a 2-way conflict);
//   * scores S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (M = 32 keys, N = the
//     wave's 32 query rows, held in registers): two 32-key blocks per tile,
//     two independent accumulation chains interleaved; the score tile is
//     already in the A-operand layout of the value product (the key order
//     inside each 16-key step is permuted identically on both operands);
//     V is read by the transposing LDS read ds_read_b64_tr_b16; LDS operands
//     are requested three steps ahead of their MFMA.  (The 32 x 32 shape
//     does twice the work per instruction of the 16 x 16 one in 1.6 times
//     its issue time on this chip);
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
constexpr float kLazyW = 256.f;  // 2^kLazy
// A wave reads tile it's K and tile it - 1's V in iteration it, while the
// copies of tiles it + 1 .. it + kPf are in flight: a ring of kPf + 2 K/V tile
// pairs (32 KB each).
constexpr int kPf = 2;
constexpr int kStages = kPf + 2;
static_assert(kStages * 2 * kTileB <= 160 * 1024, "ring fits the LDS");
static_assert((kStages & (kStages - 1)) == 0, "ring index by mask");

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
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
    // causal paged source (a DCP shard holding prefix and chunk keys): the
    // chunk's row i sits at position P + i; the shard is rank dcp_rank of
    // dcp_size with interleave dcp_I
    int32_t dcp_causal, P, dcp_rank, dcp_size, dcp_I;
};

// Positions below x owned by DCP rank s of N with interleave I ("Breaking the
// Long-Sequence Inference Bottleneck ...", section 2: owner floor(t / I) mod N):
// whole rounds of N I positions give I each, the partial round the overlap of
// [0, x mod N I) with [s I, s I + I).
__device__ __forceinline__ int32_t owned_below(int32_t x, int32_t s, int32_t N, int32_t I) {
    const int32_t round = N * I;
    const int32_t q = x / round, rem = x - q * round;
    return q * I + min(max(rem - s * I, 0), I);
}

// D (32 x 32) += A (32 x 16) B (16 x 32); lane l holds A[l % 32][8 (l / 32) + e],
// B[8 (l / 32) + e][l % 32] (e = 0 .. 7) and D[acc_row(e, l / 32)][l % 32]
// (e = 0 .. 15).
__device__ __forceinline__ f32x16_t mfma32(const u32x4_t &a, const u32x4_t &b, const f32x16_t &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ constexpr int acc_row(int e, int hf) { return 8 * (e >> 2) + 4 * hf + (e & 3); }

// Chunk c of tile row t sits at chunk position c ^ swz(t % 16).
__device__ __forceinline__ int swz(int t16) { return ((t16 & 3) << 2) | ((t16 >> 2) & 3); }

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

// The same copy from base + off, with base wave-uniform (an SGPR pair) and off
// a per-lane 32-bit byte offset: the address is formed by the instruction.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_s(gbyte *base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds), "v"(off), "s"(base)
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
    const int hf = lane >> 5, r32 = lane & 31;

    // ---- work item: KV head innermost (one XCD per head), longest first ----
    const int g = blockIdx.x % p.Hkv;
    const int f = blockIdx.x / p.Hkv;               // 0 .. 2*nqb-1
    const int piece_slot = f < p.nqb ? 1 : 0;       // tail piece first
    const int qb = p.nqb - 1 - (f % p.nqb);         // last rows first
    const int npieces = 2 * p.pcp_size;
    const int piece = piece_slot == 0 ? p.pcp_rank : npieces - 1 - p.pcp_rank;
    const int c = p.C / npieces;                    // rows per piece
    const int pe = piece * c + c;                   // end of the piece (exclusive)
    const int i0 = piece * c + qb * kBM * p.R;      // first query row of the workgroup
    const int i0w = i0 + kBM * rb;                  // first query row of this wave
    const int h = g * p.G + hw;                     // this wave's query head
    // A piece need not be a multiple of 32 rows: the last row block of a piece
    // is partial, and a wave whose rows all lie past the piece's end (i0w >= pe)
    // computes nothing but still stages its share of every tile.  Rows past the
    // end read the piece's last row (in bounds) and are never written.
    const bool wave_rows = i0w < pe;

    // keys staged for the workgroup (causal: [0, i0 + 32 R); paged shard:
    // [0, local_len)) and keys visible to this wave's rows
    // Key limits.  Dense (causal): row i sees chunk keys [0, i].  Paged prefix
    // shard: every row sees all local_len keys.  Causal paged shard: the row at
    // position P + i sees the shard's keys below owned_below(P + i + 1).
    auto row_keys = [&](int32_t i) -> int32_t {  // keys visible to chunk row i (< C)
        if (!kPaged) return i + 1;
        if (!p.dcp_causal) return p.local_len;
        return min(p.local_len, owned_below(p.P + i + 1, p.dcp_rank, p.dcp_size, p.dcp_I));
    };
    const int32_t kend = row_keys(min(i0 + kBM * p.R, pe) - 1);   // staged for the workgroup
    const int32_t kend_w = wave_rows ? row_keys(min(i0w + kBM, pe) - 1) : 0;  // wave's last row
    const int32_t kfirst_w = row_keys(min(i0w, pe - 1));          // this wave's first row
    const int32_t klim_r = row_keys(min(i0w + r32, pe - 1));      // this lane's row
    const int bs = 1 << p.bs_log2;

    // ---- queries as the B operand: lane l holds Q[i0w + l % 32][h][16 ks + 8 (l / 32) .. +8] ----
    u32x4_t qb_reg[8];
    {
        gbyte *qrow = p.q + ((int64_t)min(i0w + r32, pe - 1) * p.Hq + h) * (kD * 2) + hf * 16;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qb_reg[ks] = load16(qrow + ks * 32);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): queries in registers before any copy

    // ---- tile staging: 64 key rows of K and V straight into LDS ----
    bool bad = false;
    const uint32_t kv_lds = (uint32_t)(uintptr_t)(lds_u8 *)(&s_kv[0][0]);
    // A tile's copy is split in two: its block ids (scalar loads, looked up
    // before the barrier that their latency then overlaps) and its per-wave
    // copies, which a deeper ring spreads over the wave's MFMA steps (a burst
    // of copies from every wave fills the vector-memory queue and stalls all
    // of them).  Copy k of this wave is slot sl = wave + k * nwaves.
    struct TileSrc {
        int64_t base[4];  // base row of each 16-key group of the tile
    };
    auto stage_rows = [&](int32_t j0) -> TileSrc {
        TileSrc ts;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int32_t t = min(j0 + 16 * q4, kend - 1);
            if constexpr (kPaged) {
                int32_t phys = p.bt[t >> p.bs_log2];
                const bool ok = phys >= 0 && (int64_t)phys < p.num_blocks;
                bad |= !ok;
                phys = ok ? phys : 0;
                ts.base[q4] = ((int64_t)phys * p.Hkv + g) * bs + (t & (bs - 1) & ~15);
            } else {
                ts.base[q4] = (int64_t)(t & ~15) * p.Hkv + g;  // row index in units of D
            }
        }
        return ts;
    };
    auto stage_copy = [&](int32_t j0, int buf, const TileSrc &ts, int k) {
        const int sl = wave + k * nwaves;
        const uint32_t dst = kv_lds + (uint32_t)(buf * 2 * kTileB);
        const int ln = lane_id_here();
        const int l16 = ln >> 4, pos = ln & 15;
        const bool isv = sl >= kSlots / 2;
        const int s2 = sl & (kSlots / 2 - 1);
        if (j0 + kBN <= kend) {
            // full tile: copy sl holds rows 4 (sl % 16) .. +3, all in the 16-key
            // group q4 = (sl % 16) / 4; the per-lane part of the address is
            // row r16 = 4 (sl % 4) + lane / 16 of the group and chunk
            // (lane % 16) ^ swz(r16) of that row
            constexpr int64_t kRow = kD * 2;
            const int64_t rstride = kPaged ? kRow : (int64_t)p.Hkv * kRow;
            const int q4 = s2 >> 2;
            const int64_t b4 = q4 == 0 ? ts.base[0] : q4 == 1 ? ts.base[1] : q4 == 2 ? ts.base[2] : ts.base[3];
            const gbyte *gbase = (kPaged ? (isv ? p.vc : p.kc) : (isv ? p.v : p.k)) + b4 * kRow;  // uniform
            const int r16 = 4 * (s2 & 3) + l16;
            const uint32_t off = (uint32_t)(r16 * rstride) + (uint32_t)((pos ^ swz(r16)) * 16);
            dma16(gbase + off, __builtin_amdgcn_readfirstlane(dst + sl * 1024));
        } else {
            const int tt = s2 * 4 + l16;  // key row in the tile
            // clamp past the visible range to the last visible key (probability 0)
            const int tc = min(tt, kend - 1 - j0);
            const int q4 = tc >> 4, r16 = tc & 15;
            const int64_t b4 = q4 == 0 ? ts.base[0] : q4 == 1 ? ts.base[1] : q4 == 2 ? ts.base[2] : ts.base[3];
            const int64_t row = kPaged ? b4 + r16 : b4 + (int64_t)r16 * p.Hkv;
            const gbyte *src = (kPaged ? (isv ? p.vc : p.kc) : (isv ? p.v : p.k)) + row * (kD * 2) +
                               ((pos ^ swz(tt & 15)) * 16);
            dma16(src, __builtin_amdgcn_readfirstlane(dst + sl * 1024));
        }
    };

    // online-softmax state of query row i0w + l % 32 (the same in both lane halves)
    float m_ref = -INFINITY, l_run = 0.f;
    f32x16_t o[4];  // O[row acc_row(e, l / 32)][32 db + l % 32]
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] = 0.f;

    constexpr int kPre = 3;  // LDS operands requested ahead of their MFMA
    const int ntile = kend > 0 ? (kend + kBN - 1) / kBN : 0;
    const int ntile_w = kend_w > 0 ? (kend_w + kBN - 1) / kBN : 0;  // a prefix of the tiles
    const int per_tile = kSlots / nwaves;  // this wave's copies per tile (nwaves divides 32)
#pragma unroll
    for (int j = 0; j < kPf; ++j) {
        if (j < ntile) {
            const TileSrc ts = stage_rows(j * kBN);
            for (int k = 0; k < per_tile; ++k) stage_copy(j * kBN, j, ts, k);
        }
    }
    // Spread copies (eight waves, full tiles, a ring of three or more): wave w
    // copies slots w, w + 8 (K) and w + 16, w + 24 (V), i.e. key rows
    // 16 qa + 4 (w % 4) .. +3 and 16 qb + 4 (w % 4) .. +3 of K and of V, with
    // qa = w / 4 and qb = 2 + w / 4: two block ids and one per-lane offset.
    const bool spread_ok = nwaves == 8;
    const int qa = wave >> 2, qb2 = 2 + (wave >> 2);
    const uint32_t off8 = [&]() {
        const int ln = lane_id_here();
        const int r16 = 4 * (wave & 3) + (ln >> 4);
        const int64_t rstride = kPaged ? (int64_t)kD * 2 : (int64_t)p.Hkv * kD * 2;
        return (uint32_t)(r16 * rstride) + (uint32_t)(((ln & 15) ^ swz(r16)) * 16);
    }();
    // Base row of the 16-key group at key t, in 32-bit arithmetic (the host
    // checks that every row index of the source fits in 31 bits); one unsigned
    // compare rejects negative and too large block ids.
    auto group_row = [&](int32_t t) -> uint32_t {
        if constexpr (kPaged) {
            uint32_t phys = (uint32_t)p.bt[t >> p.bs_log2];
            const bool ok = phys < (uint32_t)p.num_blocks;
            bad |= !ok;
            phys = ok ? phys : 0u;
            return ((phys * (uint32_t)p.Hkv + (uint32_t)g) << p.bs_log2) + (uint32_t)(t & (bs - 1) & ~15);
        } else {
            return (uint32_t)(t & ~15) * (uint32_t)p.Hkv + (uint32_t)g;
        }
    };
    // Ping-pong.  Iteration it is one MFMA block -- the value product of tile
    // it - 1, then the scores of tile it -- and the softmax of tile it (VALU).
    // The first wave of each SIMD (waves 0-3) runs the block and then the
    // softmax; the second (waves 4-7) holds its scores over the barrier and
    // runs the softmax of tile it - 1 first.  After every barrier one wave of
    // a SIMD is thus in its VALU phase while the other issues MFMAs.
    const bool pong = (wave >> 2) & 1;
    f32x16_t sc[2];   // scores S^T[key][row] of the last scored tile (raw dot products)
    u32x4_t pa[4];    // its probabilities as the A operand of the value product
    // online softmax of tile t (scores in sc) -> pa; rescales o when the
    // reference maximum is raised
    auto softmax = [&](int32_t t) {
        const int32_t j0 = t * kBN;
        // lane holds keys j0 + 32 kb + acc_row(e, hf) for query row i0w + l % 32.
        // Only tiles that reach past the visible keys or straddle the diagonal
        // need a mask (a uniform test).
        if (j0 + kBN > kfirst_w) {  // some key of the tile is past some row's limit
            const int lim = klim_r - j0 - 4 * hf;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (32 * kb + acc_row(e, 0) >= lim) sc[kb][e] = -INFINITY;
        }
        // P as the A operand of 16-key step kk: elements 8 (kk % 2) .. +7 of
        // key block kk / 2, in order.  p = 2^(s * scale - m_ref); a row with no
        // visible key yet keeps the reference at -inf and shifts by 0.  (The
        // denominator is summed in fp32: the LSE needs more than the bf16
        // precision of the weights.)
        float ps = 0.f;
        auto weights = [&]() {
            const float ms = m_ref == -INFINITY ? 0.f : m_ref;
            ps = 0.f;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x0 = fast_exp2(fmaf(sc[kk >> 1][8 * (kk & 1) + 2 * i], p.qk_scale, -ms));
                    const float x1 = fast_exp2(fmaf(sc[kk >> 1][8 * (kk & 1) + 2 * i + 1], p.qk_scale, -ms));
                    ps += x0;
                    ps += x1;
                    pa[kk][i] = pack_bf16x2(x0, x1);
                }
        };
        // The weights are taken against the current reference first, without
        // the tile's maximum: a lane whose weights sum to at most 2^kLazy has
        // none above 2^kLazy, which is all the lazy reference asks for.  Where
        // a weight may be larger (or overflowed, or is NaN), or a row with a
        // visible key in the tile has no reference yet, the tile's maximum is
        // taken, the reference raised where it must be, and the weights taken
        // again (a uniform branch; rare after a row's first tile).
        weights();
        if (__any(!(ps <= kLazyW) || (m_ref == -INFINITY && klim_r > j0))) {
            float m = sc[0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = (kb == 0 ? 1 : 0); e < 16; ++e) m = fmaxf(m, sc[kb][e]);
            m = fmaxf(m, __shfl_xor(m, 32, 64));
            const float mt = m * p.qk_scale;  // the scale is positive: max commutes with it
            const bool need = mt > m_ref + kLazy;
            if (__any(need)) {
                // raise the reference maximum of the rows that need it and rescale
                // their partial sums and output rows acc_row(e, hf)
                const float mn = need ? mt : m_ref;
                const float alpha = m_ref == -INFINITY ? 0.f : fast_exp2(m_ref - mn);
                m_ref = mn;
                l_run *= alpha;
                float ar[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) ar[e] = __shfl(alpha, acc_row(e, hf), 64);
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int e = 0; e < 16; ++e) o[db][e] *= ar[e];
            }
            weights();
        }
        l_run += ps;
    };

    // Per-lane LDS byte offsets inside a tile, computed once.  Score operand of
    // key block kb, k-step ks: row 32 kb + l % 32, chunk 2 ks + l / 32 (the key
    // block is a constant offset: rows r and r + 32 share the swizzle).  Value
    // operand of column block db, 16-key step kk: in the 16-lane group of
    // column half g = (l / 16) % 2, lane j reads row 16 kk + 4 (l / 32) + j / 4
    // and the same + 8, chunk 4 db + 2 g + (j % 4) / 2, byte 8 (j % 2) (kk is a
    // constant offset).  The swizzle mixes the lane bits into the chunk
    // position, so each k-step and each (column block, row half) has its own
    // offset.
    uint32_t aoff[8], voff[2][4];
    {
        const int r = lane & 31, h2 = lane >> 5;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) aoff[ks] = r * kRowB + 16 * ((2 * ks + h2) ^ swz(r & 15));
        const int g2 = (lane >> 4) & 1, j = lane & 15;
        const int row0 = 4 * h2 + (j >> 2), cg = 2 * g2 + ((j & 3) >> 1);
#pragma unroll
        for (int hr = 0; hr < 2; ++hr)
#pragma unroll
            for (int db = 0; db < 4; ++db)
                voff[hr][db] = (row0 + 8 * hr) * kRowB + 16 * ((4 * db + cg) ^ swz(row0 + 8 * hr)) + 8 * (j & 1);
    }
    const gbyte *ksrc = kPaged ? p.kc : p.k, *vsrc = kPaged ? p.vc : p.v;
    for (int32_t it = 0; it <= ntile; ++it) {  // it == ntile: the last value product only
        const bool pre = it + kPf < ntile;
        const int32_t jn = (it + kPf) * kBN;
        const int bn = (it + kPf) & (kStages - 1);
        const bool spread = spread_ok && pre && jn + kBN <= kend;
        uint32_t ra = 0, rb2 = 0;
        if (spread) {  // scalar loads before the barrier that their latency then overlaps
            ra = group_row(jn + 16 * qa);
            rb2 = group_row(jn + 16 * qb2);
        }
        // tile it has landed (own copies; later tiles may still be in flight) ...
        static_assert(kPf == 2, "the eight-wave wait below leaves one tile in flight");
        if (nwaves == 8) {  // four copies per wave and tile
            if (it + 1 < ntile) vm_wait<4>();
            else vm_wait<0>();
        } else {
            wait_copies_at_most(min(kPf - 1, ntile - 1 - it) * per_tile);
        }
        __syncthreads();  // ... for every wave; the buffer of tile it - 2 is free again
        // the block ids are needed from here on: wait for them now, while no
        // LDS read is in flight (the two share a wait counter)
        asm volatile("" ::"s"(ra), "s"(rb2));
        const uint32_t dstn = kv_lds + (uint32_t)(bn * 2 * kTileB) + (uint32_t)(wave * 1024);
        // sources of this wave's four copies of tile it + kPf: K then V of its
        // two 16-key groups
        const gbyte *csrc[4] = {ksrc + ((uint64_t)ra << 8), ksrc + ((uint64_t)rb2 << 8),
                                vsrc + ((uint64_t)ra << 8), vsrc + ((uint64_t)rb2 << 8)};
        // copy k of tile it + kPf goes after MFMA step 8 k + 7 of this block
        auto side = [&](int step) {
            if ((step & 7) != 7 || !spread) return;
            const int k = step >> 3;
            dma16_s(csrc[k], off8, dstn + (uint32_t)(k * 8 * 1024));
        };
        if (pre && !spread) {
            const TileSrc ts = stage_rows(jn);
            for (int k = 0; k < per_tile; ++k) stage_copy(jn, bn, ts, k);
        }
        const bool do_pv = it >= 1 && it - 1 < ntile_w;   // value product of tile it - 1
        const bool do_s = it < ntile_w;                  // scores of tile it
        if (!do_pv && !do_s) {  // past this wave's diagonal (uniform): copies only
#pragma unroll
            for (int st = 0; st < 32; ++st) side(st);
            continue;
        }
        if (pong && do_pv) softmax(it - 1);

        // ---- values of tile it - 1: O[row][d] += P[row][key] V[key][d], 4 column blocks x 4 key steps ----
        if (do_pv) {
            lds_u8 *tv = (lds_u8 *)(&s_kv[(it - 1) % kStages][0]) + kTileB;
            lds_u8 *vp[2][4];
#pragma unroll
            for (int hr = 0; hr < 2; ++hr)
#pragma unroll
                for (int db = 0; db < 4; ++db) vp[hr][db] = tv + voff[hr][db];
            auto read_v = [&](int i) -> u32x4_t {  // step i: kk = i / 4, db = i % 4
                const int kk = i >> 2, db = i & 3;
                lds_u8 *va0 = vp[0][db] + kk * 16 * kRowB;
                lds_u8 *va1 = vp[1][db] + kk * 16 * kRowB;
                const i16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4_t *)(va0));
                const i16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4_t *)(va1));
                const u32x2_t w0 = __builtin_bit_cast(u32x2_t, t0), w1 = __builtin_bit_cast(u32x2_t, t1);
                return u32x4_t{w0[0], w0[1], w1[0], w1[1]};
            };
            u32x4_t vbuf[kPre];
#pragma unroll
            for (int i = 0; i < kPre; ++i) vbuf[i] = read_v(i);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const u32x4_t vb = vbuf[i % kPre];
                if (i + kPre < 16) vbuf[i % kPre] = read_v(i + kPre);
                const int kk = i >> 2, db = i & 3;
                o[db] = mfma32(pa[kk], vb, o[db]);
                __builtin_amdgcn_sched_barrier(0);
                side(i);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int st = 0; st < 16; ++st) side(st);
        }
        // ---- scores of tile it: 2 key blocks x 8 k-steps, key blocks interleaved ----
        // (raw dot products; the scale is applied inside the exponent)
        if (do_s) {
            lds_u8 *tk = (lds_u8 *)(&s_kv[it % kStages][0]);
            lds_u8 *ap[8];
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) ap[ks] = tk + aoff[ks];
            auto read_a = [&](int i) -> u32x4_t {  // step i: ks = i / 2, kb = i % 2
                const int ks = i >> 1, kb = i & 1;
                return *(__attribute__((address_space(3))) const u32x4_t *)(ap[ks] + kb * 32 * kRowB);
            };
            u32x4_t abuf[kPre];
#pragma unroll
            for (int i = 0; i < kPre; ++i) abuf[i] = read_a(i);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const u32x4_t a = abuf[i % kPre];
                if (i + kPre < 16) abuf[i % kPre] = read_a(i + kPre);
                const int ks = i >> 1, kb = i & 1;
                f32x16_t zero;
#pragma unroll
                for (int e = 0; e < 16; ++e) zero[e] = 0.f;
                sc[kb] = mfma32(a, qb_reg[ks], ks == 0 ? zero : sc[kb]);
                __builtin_amdgcn_sched_barrier(0);
                side(16 + i);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (!pong) softmax(it);
        } else {
#pragma unroll
            for (int st = 16; st < 32; ++st) side(st);
        }
    }

    // ---- finish: normalise and write rows of this piece ----
    bad = __syncthreads_or(bad);
    const int local0 = (qb * p.R + rb) * kBM;  // row within the piece
    const float lt = l_run + __shfl_xor(l_run, 32, 64);  // full sum of row l % 32
    const float inv_r = bad ? NAN : (lt > 0.f ? 1.f / lt : 0.f);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const float iv = __shfl(inv_r, acc_row(e, hf), 64);
        const int r = local0 + acc_row(e, hf);
        float *dst = p.out + (((int64_t)piece_slot * c + r) * p.Hq + h) * kD + r32;
        if (r < c) {
#pragma unroll
            for (int db = 0; db < 4; ++db) dst[db * 32] = o[db][e] * iv;
        }
    }
    if (lane < 32 && local0 + lane < c) {
        const int r = local0 + lane;
        p.lse[((int64_t)piece_slot * c + r) * p.Hq + h] =
            bad ? NAN : (m_ref == -INFINITY || !(lt > 0.f) ? -INFINITY : (m_ref + fast_log2(lt)) * kLn2);
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
    const int nrb = (rows + kBM - 1) / kBM;  // 32-row blocks per piece (the last may be partial)
    if (a->kv_source != CP_KV_DENSE && a->kv_source != CP_KV_PAGED &&
        a->kv_source != CP_KV_PAGED_CAUSAL)
        return fail(CP_E_INVALID, "prefill: kv_source %d", a->kv_source);
    const bool dcp_causal = a->kv_source == CP_KV_PAGED_CAUSAL;
    if (dcp_causal) {
        if (a->dcp_size < 1 || a->dcp_rank < 0 || a->dcp_rank >= a->dcp_size ||
            a->dcp_interleave < 1 || (int64_t)a->dcp_size * a->dcp_interleave > (1 << 30) ||
            (int64_t)a->P + a->C > 0x7ffffffe)
            return fail(CP_E_INVALID, "prefill: dcp rank %d of %d, interleave %d, P + C = %lld",
                        a->dcp_rank, a->dcp_size, a->dcp_interleave, (long long)a->P + a->C);
        // the last chunk position P + C - 1 sees every shard key below P + C
        const int64_t round = (int64_t)a->dcp_size * a->dcp_interleave, x = (int64_t)a->P + a->C;
        const int64_t rem = x % round - (int64_t)a->dcp_rank * a->dcp_interleave;
        const int64_t need = x / round * a->dcp_interleave +
                             (rem < 0 ? 0 : (rem > a->dcp_interleave ? a->dcp_interleave : rem));
        if (a->local_len < need)
            return fail(CP_E_INVALID,
                        "prefill: the shard holds %d keys, positions below P + C need %lld",
                        a->local_len, (long long)need);
    }
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
        if ((int64_t)a->C * a->Hkv >= ((int64_t)1 << 31))
            return fail(CP_E_UNSUPPORTED, "prefill: %d x %d K/V rows exceed 2^31", a->C, a->Hkv);
        p.k = to_global(a->k);
        p.v = to_global(a->v);
    } else {  // CP_KV_PAGED or CP_KV_PAGED_CAUSAL
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
        if (a->num_blocks < 0 || a->num_blocks * a->Hkv * a->bs >= ((int64_t)1 << 31))
            return fail(CP_E_UNSUPPORTED, "prefill: %lld blocks x %d heads x %d rows exceed 2^31",
                        (long long)a->num_blocks, a->Hkv, a->bs);
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
    while (R > 1 && nrb % R != 0) R /= 2;
    // at least two waves: a lone wave would keep two tiles' 32 copies each in
    // flight, past the 63 outstanding loads its counter can track (the second
    // wave of a one-block piece has no rows and only stages)
    if (G * R < 2) R = 2;
    int G_log2 = 0;
    while ((1 << G_log2) < G) ++G_log2;
    p.R = R;
    p.G_log2 = G_log2;
    p.nqb = (nrb + R - 1) / R;
    p.out = a->out;
    p.lse = a->lse;
    p.dcp_causal = dcp_causal ? 1 : 0;
    p.P = a->P;
    p.dcp_rank = dcp_causal ? a->dcp_rank : 0;
    p.dcp_size = dcp_causal ? a->dcp_size : 1;
    p.dcp_I = dcp_causal ? a->dcp_interleave : 1;
    const int64_t blocks = (int64_t)2 * p.nqb * a->Hkv;
    if (blocks > 0x7fffffff) return fail(CP_E_UNSUPPORTED, "prefill: too many query blocks");
    const int threads = 64 * G * R;
    if (a->kv_source != CP_KV_DENSE)
        hipLaunchKernelGGL(prefill_kernel<true>, dim3((unsigned)blocks), dim3(threads), 0, stream, p);
    else
        hipLaunchKernelGGL(prefill_kernel<false>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                           p);
    return check_launch("pcp_prefill_attn_causal");
}
