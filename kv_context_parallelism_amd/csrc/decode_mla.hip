// decode_mla.hip -- absorbed multi-head latent attention (MLA) decode partial
// over one DCP shard of a paged latent cache, on gfx950 matrix cores.
//
// What it computes: "vLLM DCP and PCP: Decode and Prefill Context
// Parallelism", Deep Dive 6, "Deriving the partial and global outputs" (local
// scores, local LSE, shard-normalised output), for the latent layout of
// "Breaking the Long-Sequence Inference Bottleneck ...", section 3, "MLA path":
// one compressed KV row per token shared by every query head (KV head = 1).
// Keys are the whole latent row (Dk = 576: 512 latent + 64 rope), values its
// first Dv = 512 columns.
//
// Design (a dense contraction: up to 128 heads x 576 against every cached row):
//   * one workgroup = 8 waves (two per SIMD); every latent tile staged in LDS
//     feeds all 128 heads.  Scores are split by heads: wave w computes the
//     scores and the softmax of query heads 16w .. 16w+15 (its queries stay in
//     registers for the segment).  The value product is split by columns:
//     wave w accumulates O[h][64 w .. 64 w + 63] for every head h, so each
//     value column is read from LDS by one wave only.  The probabilities pass
//     between the two through LDS, together with each head's rescale factor.
//     bf16: one barrier per tile -- after it, a wave runs the value product of
//     the previous tile (its probabilities in one of two LDS buffers), then
//     the scores of this tile (into the other buffer); fp8: a second barrier
//     per tile between the scores and the value product of the same tile.  The accumulators (128 x 64 fp32 outputs,
//     16 x 32 scores) and the queries fit a wave's 256 VGPRs; the file is
//     compiled with MFMA results in VGPRs so that rescales update them in place;
//   * 32-token latent tiles go HBM -> LDS by global_load_lds (no registers)
//     into a ring of three: bf16 reads tiles it - 1 and it while tile it + 1
//     is in flight (the second probability buffer leaves no room for a
//     fourth); fp8 keeps two raw tiles in flight.
//     The copies are issued from inline asm and waited for with explicit
//     vmcnt counts, so the compiler does not serialise them against the LDS
//     reads of the tile being consumed;
//   * LDS rows are unpadded (1152 bytes) with the 16-byte chunks of row t
//     XOR-swizzled by (t / 2) % 8: both LDS read patterns below are free of
//     bank conflicts;
//   * scores S^T = C Q^T on v_mfma_f32_16x16x32_bf16 (A = latent rows from
//     LDS, B = the wave's 16 queries); the probabilities are stored per head
//     in the k order of the value product;
//   * values O = P V on v_mfma_f32_32x32x16_bf16, the V operand read by
//     ds_read_b64_tr_b16 (transposing LDS read), the P operand one 16-byte
//     LDS read per 32-head block;
//   * online softmax in the exp2 domain with a lazily updated reference
//     maximum: the output is rescaled only when a tile's maximum exceeds the
//     reference by more than 2^8, which keeps every probability <= 256 and the
//     result exact up to rounding while skipping almost all rescales;
//   * fp8 E4M3 latent lands in a raw ring and is widened to bf16 (exact) one
//     tile ahead of its use; the per-tensor scale is folded into the score
//     scale and the output;
//   * the balanced flat schedule of the GQA kernel: exactly the resident
//     workgroups, each taking an equal range of (request, 32-token tile)
//     space; partials go to slot workgroup + request and are merged exactly
//     afterwards.
#include <math.h>

#include <type_traits>

#include "internal.hpp"

namespace cpattn {

namespace {

constexpr int kDk = 576, kDv = 512;
constexpr int kT = 32;                  // tokens per tile / per scheduling chunk
constexpr int kRowB = kDk * 2;          // LDS row: 1152 bytes = 72 chunks of 16
constexpr int kRowC = kRowB / 16;
constexpr int kTileB = kT * kRowB;      // 36,864 bytes
constexpr int kKs = kDk / 32;           // 18 k-steps of the score MFMA
constexpr int kMaxB = 4096;
constexpr int kWaves = 8;               // 16 heads per wave, two waves per SIMD
constexpr int kHeadsWg = 16 * kWaves;   // 128
constexpr int kThreads = 64 * kWaves;
constexpr float kLazy = 8.f;            // rescale only past 2^8
constexpr int kPRow = 80;               // LDS row of one head's 32 probabilities (64 + 16 bytes)
constexpr int kVcW = kDv / kWaves;      // value columns of one wave in the value product (64)

// copies per tile: bf16 goes straight into the tile (36 copies of 64 chunks),
// fp8 into a raw ring (36 chunks per row, 18 copies)
constexpr int kBfSlots = kT * kRowC / 64;        // 36
constexpr int kRawSlots = kT * (kDk / 16) / 64;  // 18
static_assert(kT * kRowC % 64 == 0 && kT * (kDk / 16) % 64 == 0, "whole 64-chunk copies");
static_assert(kRowC % 8 == 0, "the chunk swizzle permutes aligned groups of 8");

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) const uint8_t lds_u8;

struct MlaParams {
    const gbyte *q, *kv;
    cint32 *bt, *len;
    int32_t B, H, bs_log2, bt_stride;
    int64_t num_blocks;
    float qk_scale;   // scale * kv_scale * log2(e)
    float v_scale;    // kv_scale (fp8) or 1
    int32_t W;        // tile ranges = workgroups launched
    float *ws_o;      // [slots][H][512]
    float *ws_l;      // [slots][H]
    int32_t *seg;     // [B][2]
};

__device__ __forceinline__ f32x4_t mfma16(const u32x4_t &a, const u32x4_t &b, const f32x4_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// D (32 x 32) += A (32 x 16) B (16 x 32); lane l holds A[l % 32][8 (l / 32) + e],
// B[8 (l / 32) + e][l % 32] (e = 0 .. 7) and D[8 (e / 4) + 4 (l / 32) + e % 4][l % 32]
// (e = 0 .. 15).
__device__ __forceinline__ f32x16_t mfma32(const u32x4_t &a, const u32x4_t &b, const f32x16_t &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ int64_t owner_of(int64_t c, int64_t R, int64_t W) {
    return ((c + 1) * W - 1) / R;
}

// Chunk c (16 bytes) of tile row t sits at chunk position c ^ swz(t) of the row.
__device__ __forceinline__ int swz(int t) { return (t >> 1) & 7; }

// The lane id, recomputed where it is used: keeps per-lane addresses from
// being hoisted out of the tile loop and held in registers.
__device__ __forceinline__ int lane_id_here() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// One 64-lane HBM -> LDS copy: lane i moves 16 bytes from `src` to LDS byte
// lds + 16 i.  `lds` must be wave-uniform.  Issued from asm so that the
// compiler's wait insertion does not tie later LDS reads to it; every reader
// waits explicitly (vm_wait + barrier) before touching the destination.
// (M0 is written here and read by nothing the compiler emits in this file.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(gbyte *src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds), "v"(src)
                 : "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]).  Issued as
// the builtin so that the compiler's own wait tracking sees it.
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Wave w issues the copies w, w + 4, ... of a tile: wait until at most one
// (or two) further tiles' worth of this wave's copies is outstanding.
template <int Slots>
__device__ __forceinline__ void wait_all_but_one_tile(bool one_in_flight, int wave) {
    constexpr int lo = Slots / kWaves, extra = Slots % kWaves;
    if (!one_in_flight) vm_wait<0>();
    else if (wave < extra) vm_wait<lo + 1>();
    else vm_wait<lo>();
}

template <int Slots>
__device__ __forceinline__ void wait_all_but_two_tiles(bool two, bool one, int wave) {
    constexpr int lo = Slots / kWaves, extra = Slots % kWaves;
    if (two) {
        if (wave < extra) vm_wait<2 * (lo + 1)>();
        else vm_wait<2 * lo>();
    } else {
        wait_all_but_one_tile<Slots>(one, wave);
    }
}

template <bool kFp8>
__global__ void __launch_bounds__(kThreads, 1) mla_kernel(MlaParams p) {
    constexpr int kBfBufs = kFp8 ? 2 : 3;
    constexpr int kRawBufs = kFp8 ? 3 : 1;
    __shared__ __attribute__((aligned(16))) uint8_t s_kv[kBfBufs][kTileB];
    __shared__ __attribute__((aligned(16))) uint8_t s_raw[kRawBufs][kFp8 ? kT * kDk : 16];
    __shared__ int32_t s_pref[kMaxB + 1];
    __shared__ int32_t s_wsum[kWaves];
    // probabilities of the tile, [head][32 tokens in value-product k order]
    // (rows padded to 80 bytes: the 16-byte reads of 16 rows hit distinct banks)
    // (bf16: two buffers, tile it's written while tile it - 1's are read)
    constexpr int kPBufs = kFp8 ? 1 : 2;
    __shared__ __attribute__((aligned(16))) uint8_t s_pp[kPBufs][kHeadsWg * kPRow];
    __shared__ __attribute__((aligned(16))) float s_alphap[kPBufs][kHeadsWg];  // rescale of each head's rows
    __shared__ __attribute__((aligned(16))) float s_linv[kHeadsWg];   // 1 / row sum at the end
    __shared__ __attribute__((aligned(8))) uint8_t s_flagp[kPBufs][kWaves];    // a head of wave w rescaled

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int range = blockIdx.x;
    const int h0 = wave * 16;
    const bool active = h0 < p.H;  // waves past H only help stage tiles
    const int64_t cap = (int64_t)p.bt_stride << p.bs_log2;
    const int bs = 1 << p.bs_log2;

    // ---- tiles per request and their prefix sum ----
    auto tiles_of = [&](int32_t L) -> int32_t {
        if (L < 0 || (int64_t)L > cap) return 1;  // invalid length: one NaN tile
        return (L + kT - 1) / kT;
    };
    {
        const int per = (p.B + kThreads - 1) / kThreads;
        const int b0 = tid * per;
        int32_t run = 0;
        for (int i = 0; i < per && b0 + i < p.B; ++i) run += tiles_of(p.len[b0 + i]);
        int32_t incl = run;
#pragma unroll
        for (int x = 1; x < 64; x <<= 1) {
            const int32_t o = __shfl_up(incl, x, 64);
            if (lane >= x) incl += o;
        }
        if (lane == 63) s_wsum[tid >> 6] = incl;
        __syncthreads();
        int32_t base = 0;
        for (int i = 0; i < (tid >> 6); ++i) base += s_wsum[i];
        int32_t acc = base + incl - run;
        for (int i = 0; i < per && b0 + i < p.B; ++i) {
            s_pref[b0 + i] = acc;
            acc += tiles_of(p.len[b0 + i]);
        }
        if (tid == kThreads - 1) s_pref[p.B] = base + incl;
        __syncthreads();
    }
    auto pref = [&](int i) -> int32_t { return __builtin_amdgcn_readfirstlane(s_pref[i]); };
    const int64_t R_tot = pref(p.B);
    const int64_t W = R_tot < p.W ? R_tot : p.W;

    if (blockIdx.x == 0) {
        for (int b = tid; b < p.B; b += kThreads) {
            const int64_t n = s_pref[b + 1] - s_pref[b];
            int32_t first = 0, count = 0;
            if (n > 0) {
                const int64_t F = s_pref[b];
                const int64_t o0 = owner_of(F, R_tot, W), o1 = owner_of(F + n - 1, R_tot, W);
                first = (int32_t)(o0 + b);
                count = (int32_t)(o1 - o0 + 1);
            }
            p.seg[2 * b] = first;
            p.seg[2 * b + 1] = count;
        }
    }
    if (range >= W || R_tot == 0) return;
    int64_t cc = (int64_t)range * R_tot / W;
    const int64_t hi = ((int64_t)range + 1) * R_tot / W;

    // LDS byte addresses of the buffers (wave-uniform)
    const uint32_t kv_lds = (uint32_t)(uintptr_t)(lds_u8 *)(&s_kv[0][0]);
    const uint32_t raw_lds = (uint32_t)(uintptr_t)(lds_u8 *)(&s_raw[0][0]);

    while (cc < hi) {
        int lo_b = 0, hi_b = p.B;
        while (hi_b - lo_b > 1) {
            const int mid = (lo_b + hi_b) >> 1;
            if (pref(mid) <= cc) lo_b = mid;
            else hi_b = mid;
        }
        const int b = __builtin_amdgcn_readfirstlane(lo_b);
        const int32_t pb = pref(b);
        const int32_t n = pref(b + 1) - pb;
        const int32_t k = (int32_t)(cc - pb);
        const int32_t nseg = (int32_t)min<int64_t>(hi - cc, n - k);
        const int32_t Lraw = p.len[b];
        bool bad = Lraw < 0 || (int64_t)Lraw > cap;
        const int32_t L = bad ? 0 : Lraw;
        const int32_t s0 = k * kT;
        const int32_t s1 = min(s0 + nseg * kT, L);
        const int32_t ntile = s1 > s0 ? (s1 - s0 + kT - 1) / kT : 0;
        const int64_t slot = range + b;
        cint32 *bt_row = p.bt + (int64_t)b * p.bt_stride;

        // ---- the wave's 16 queries as the B operand: Q[h0 + l % 16][32 ks + 8 (l / 16) .. +8] ----
        // (lanes of heads past H load head H - 1: their columns of the score and
        // output tiles are computed but never written)
        u32x4_t qb[kKs];
        {
            const int hq = min(h0 + (lane & 15), p.H - 1);
            gbyte *qrow = p.q + ((int64_t)b * p.H + hq) * (kDk * 2) + (lane >> 4) * 16;
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks) qb[ks] = load16(qrow + ks * 64);
        }
        vm_wait<0>();  // the queries are in registers before any tile copy is issued

        // ---- tile copies (all waves) ----
        // Cache rows of the tile's tokens: a 32-token tile spans at most two
        // blocks (bs >= 16).  Tokens past the segment's end reuse the row of its
        // last token (finite data; their probability is forced to 0).  Copy sl
        // fills destination chunks 64 sl .. 64 sl + 63 of the tile; the source
        // chunk of destination position p in row t is p ^ swz(t).
        // A tile's copies: the cache rows of its two 16-token halves (scalar
        // block-table loads), then this wave's copies, copy i being slot
        // sl = wave + 8 i.
        struct TileRows {
            int64_t r0, r1;  // cache rows of the tile's first token and of token 16
            int32_t nval;    // real tokens of the tile
            int32_t it;      // tile index (ring position)
        };
        auto tile_rows = [&](int32_t it) -> TileRows {
            const int32_t tb = s0 + it * kT;
            const int32_t nval = min(kT, s1 - tb);
            auto row_of = [&](int32_t tok) -> int64_t {
                int32_t phys = bt_row[tok >> p.bs_log2];
                const bool ok = phys >= 0 && (int64_t)phys < p.num_blocks;
                bad |= !ok;
                phys = ok ? phys : 0;
                return ((int64_t)phys << p.bs_log2) + (tok & (bs - 1));
            };
            TileRows tr;
            tr.r0 = row_of(tb);
            tr.r1 = row_of(tb + min(16, nval - 1));  // == r0 + 16 within one block
            tr.nval = nval;
            tr.it = it;
            return tr;
        };
        constexpr int kSlots = kFp8 ? kRawSlots : kBfSlots;
        constexpr int kCopies = (kSlots + kWaves - 1) / kWaves;  // per wave, at most
        auto issue_copy = [&](const TileRows &tr, int i) {
            const int sl = wave + kWaves * i;
            if (sl >= kSlots) return;
            const int64_t r0 = tr.r0, r1 = tr.r1;
            const int32_t nval = tr.nval;
            if constexpr (kFp8) {
                const uint32_t dst = raw_lds + (uint32_t)((tr.it % 3) * (kT * kDk));
                const int c = sl * 64 + lane_id_here();
                const int tt = min(c / (kDk / 16), nval - 1), ch = c % (kDk / 16);
                const int64_t row = (tt < 16 ? r0 : r1 - 16) + tt;
                dma16(p.kv + row * kDk + ch * 16, __builtin_amdgcn_readfirstlane(dst + sl * 1024));
            } else {
                const uint32_t dst = kv_lds + (uint32_t)((tr.it % 3) * kTileB);
                const int c = sl * 64 + lane_id_here();  // destination chunk in the tile
                const int t = c / kRowC, pos = c - t * kRowC;
                const int tt = min(t, nval - 1);
                const int64_t rbase = tt < 16 ? r0 : r1 - 16;
                dma16(p.kv + (rbase + tt) * kRowB + (pos ^ swz(t)) * 16,
                      __builtin_amdgcn_readfirstlane(dst + sl * 1024));
            }
        };
        // Cache rows of the tile's tokens: a 32-token tile spans at most two
        // blocks (bs >= 16).  Tokens past the segment's end reuse the row of its
        // last token (finite data; their probability is forced to 0).  Copy sl
        // fills destination chunks 64 sl .. 64 sl + 63 of the tile; the source
        // chunk of destination position p in row t is p ^ swz(t).
        auto issue_tile = [&](int32_t it) {
            const TileRows tr = tile_rows(it);
#pragma unroll
            for (int i = 0; i < kCopies; ++i) issue_copy(tr, i);
        };
        // fp8: widen raw tile `it` into bf16 buffer it % 2 (all threads)
        auto widen_tile = [&](int32_t it) {
            if constexpr (kFp8) {
                const uint8_t *raw = s_raw[it % 3];
                uint8_t *dst = s_kv[it % 2];
                for (int c = tid; c < kT * (kDk / 16); c += kThreads) {
                    const int tt = c / (kDk / 16), ch = c % (kDk / 16);
                    const u32x4_t x = *reinterpret_cast<const u32x4_t *>(raw + c * 16);
                    u32x4_t lo, hi2;
#pragma unroll
                    for (int wd = 0; wd < 4; ++wd) {
                        const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8(x[wd], false);
                        const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8(x[wd], true);
                        const uint32_t a = (__float_as_uint(f01[0]) >> 16) |
                                           (__float_as_uint(f01[1]) & 0xffff0000u);
                        const uint32_t b2 = (__float_as_uint(f23[0]) >> 16) |
                                            (__float_as_uint(f23[1]) & 0xffff0000u);
                        if (wd < 2) {
                            lo[2 * wd] = a;
                            lo[2 * wd + 1] = b2;
                        } else {
                            hi2[2 * (wd - 2)] = a;
                            hi2[2 * (wd - 2) + 1] = b2;
                        }
                    }
                    *reinterpret_cast<u32x4_t *>(dst + tt * kRowB + ((2 * ch) ^ swz(tt)) * 16) = lo;
                    *reinterpret_cast<u32x4_t *>(dst + tt * kRowB + ((2 * ch + 1) ^ swz(tt)) * 16) = hi2;
                }
            }
        };

        float m_ref = -INFINITY, l_run = 0.f;  // per head lane % 16 (same in all four groups)
        // The value product is split by columns: wave w accumulates
        // O[h][64 w .. 64 w + 63] for every head h, in 32 x 32 blocks
        // o[hb][cb] = O[32 hb + 8 (e / 4) + 4 (l / 32) + e % 4][64 w + 32 cb + l % 32].
        f32x16_t o[4][2];
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[hb][cb][e] = 0.f;
        // All four 32-head blocks are computed whatever H is: rows of heads
        // >= H (probabilities never written) are never stored.
        constexpr int nhb = 4;

        // Scores and softmax of the wave's 16 heads (active waves).  The
        // probabilities go to s_p in the k order of the value product; the
        // rescale factors of the wave's heads to s_alpha and whether any head
        // was rescaled to s_flag[wave].  The score product is pipelined by
        // hand, three LDS operands ahead, with a scheduling barrier per step.
        constexpr int kPre = 3;
        auto scores_softmax = [&](int32_t it, const uint8_t *tile, int pb) {
            uint8_t *s_p = s_pp[pb];
            float *s_alpha = s_alphap[pb];
            uint8_t *s_flag = s_flagp[pb];
            const int32_t tb = s0 + it * kT;
            // Per-lane addresses (16-lane group G = lane / 16, j = lane % 16),
            // recomputed per tile from a fresh lane id.  Score operand of half hf,
            // k-step ks: row 16 hf + j, chunk 4 ks + G.  Rows r and r + 16 share
            // swz(r), so the + 16 row halves are a constant offset; the swizzle
            // acts on the chunk's low 3 bits.
            lds_u8 *t3 = (lds_u8 *)(tile);
            lds_u8 *ap[2];
            {
                const int ln = lane_id_here();
                const int G = ln >> 4, j = ln & 15;
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2) ap[k2] = t3 + j * kRowB + 16 * ((4 * k2 + G) ^ swz(j));
            }
            auto read_a = [&](int i) -> u32x4_t {  // step i: half i % 2, k-step i / 2
                const int hf = i & 1, ks = i >> 1;
                return *(__attribute__((address_space(3))) const u32x4_t *)(
                    ap[ks & 1] + hf * 16 * kRowB + 128 * (ks >> 1));
            };

            // ---- scores S^T[t][h]: two 16-token halves x 18 k-steps, the halves
            // interleaved (two independent accumulation chains) ----
            f32x4_t sc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
            {
                constexpr int kSteps = 2 * kKs;
                u32x4_t abuf[kPre];
#pragma unroll
                for (int i = 0; i < kPre; ++i) abuf[i] = read_a(i);
#pragma unroll
                for (int i = 0; i < kSteps; ++i) {
                    const u32x4_t a = abuf[i % kPre];
                    if (i + kPre < kSteps) abuf[i % kPre] = read_a(i + kPre);
                    sc[i & 1] = mfma16(a, qb[i >> 1], sc[i & 1]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // lane holds head lane % 16, tokens tb + 16 hf + 4 G + e
            const int G = lane >> 4;
            const int lim = s1 - tb - 4 * G;  // token (hf, e) is real iff 16 hf + e < lim
            float mt = -INFINITY;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float sv = sc[hf][e] * p.qk_scale;
                    if (16 * hf + e >= lim) sv = -INFINITY;
                    sc[hf][e] = sv;
                    mt = fmaxf(mt, sv);
                }
            mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
            mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
            float alpha = 1.f;
            int resc = 0;
            if (it == 0) {
                m_ref = mt;
            } else if (__any(mt > m_ref + kLazy)) {
                const float mn = fmaxf(m_ref, mt);
                alpha = fast_exp2(m_ref - mn);
                m_ref = mn;
                l_run *= alpha;
                resc = 1;
            }
            float ps = 0.f;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sc[hf][e] = fast_exp2(sc[hf][e] - m_ref);
                    ps += sc[hf][e];
                }
            l_run += ps;
            // token 16 hf + 4 G + e sits at k position 16 hf + 8 (G % 2) + 4 (G / 2) + e
            {
                uint8_t *prow = s_p + (h0 + (lane & 15)) * kPRow + 2 * (8 * (G & 1) + 4 * (G >> 1));
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
                    *reinterpret_cast<u32x2_t *>(prow + 32 * hf) =
                        u32x2_t{pack_bf16x2(sc[hf][0], sc[hf][1]), pack_bf16x2(sc[hf][2], sc[hf][3])};
            }
            if (lane < 16) s_alpha[h0 + lane] = alpha;
            if (lane == 0) s_flag[wave] = (uint8_t)resc;
        };

        // Value product of the tile for this wave's 64 columns and every head:
        // O[h][c] += P[h][t] V[t][c] on 32 x 32 x 16 MFMAs, two 16-token k-steps.
        // V (B operand) is read by ds_read_b64_tr_b16: in the 16-lane group of
        // column half g = (l / 16) % 2, lane j reads rows 16 kk + 4 (l / 32) +
        // j / 4 and the same + 8, chunk 8 w + 4 cb + 2 g + (j % 4) / 2, byte
        // 8 (j % 2); the probabilities (A operand) are one 16-byte read per
        // (head block, k-step) from s_p, whose k order matches those rows.
        auto value_product = [&](const uint8_t *tile, int pb) {
            const uint8_t *s_p = s_pp[pb];
            const float *s_alpha = s_alphap[pb];
            const uint8_t *s_flag = s_flagp[pb];
            // rescale the rows of every head whose owner raised its reference maximum
            const uint64_t flags = *reinterpret_cast<const uint64_t *>(s_flag);
            if (flags != 0) {
                const int h2 = lane >> 5;
#pragma unroll
                for (int hb = 0; hb < 4; ++hb) {
                    if (hb >= nhb) break;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float4 a4 = *reinterpret_cast<const float4 *>(s_alpha + 32 * hb + 8 * q + 4 * h2);
#pragma unroll
                        for (int cb = 0; cb < 2; ++cb) {
                            o[hb][cb][4 * q + 0] *= a4.x;
                            o[hb][cb][4 * q + 1] *= a4.y;
                            o[hb][cb][4 * q + 2] *= a4.z;
                            o[hb][cb][4 * q + 3] *= a4.w;
                        }
                    }
                }
            }
            lds_u8 *t3 = (lds_u8 *)(tile);
            lds_u8 *vp[2][2];  // [cb][row half]
            lds_u8 *pp;
            {
                const int ln = lane_id_here();
                const int h2 = ln >> 5, g2 = (ln >> 4) & 1, j = ln & 15;
                const int row0 = 4 * h2 + (j >> 2), cg = 2 * g2 + ((j & 3) >> 1);
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                    for (int hr = 0; hr < 2; ++hr) {
                        const int r = row0 + 8 * hr;
                        vp[cb][hr] = t3 + r * kRowB + 16 * (8 * wave + ((4 * cb + cg) ^ swz(r))) + 8 * (j & 1);
                    }
                pp = (lds_u8 *)(s_p) + (ln & 31) * kPRow + 16 * h2;
            }
            auto read_v = [&](int cb, int kk) -> u32x4_t {  // rows + 16 kk share the swizzle
                const i16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4_t *)(vp[cb][0] + kk * 16 * kRowB));
                const i16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4_t *)(vp[cb][1] + kk * 16 * kRowB));
                const u32x2_t w0 = __builtin_bit_cast(u32x2_t, t0), w1 = __builtin_bit_cast(u32x2_t, t1);
                return u32x4_t{w0[0], w0[1], w1[0], w1[1]};
            };
            auto read_p = [&](int hb, int kk) -> u32x4_t {
                return *(__attribute__((address_space(3))) const u32x4_t *)(pp + hb * 32 * kPRow + 32 * kk);
            };
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const u32x4_t v0 = read_v(0, kk), v1 = read_v(1, kk);
                u32x4_t pn = read_p(0, kk);
#pragma unroll
                for (int hb = 0; hb < 4; ++hb) {
                    if (hb >= nhb) break;
                    const u32x4_t pa = pn;
                    if (hb + 1 < 4 && hb + 1 < nhb) pn = read_p(hb + 1, kk);
                    o[hb][0] = mfma32(pa, v0, o[hb][0]);
                    o[hb][1] = mfma32(pa, v1, o[hb][1]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        auto compute_tile = [&](int32_t it, const uint8_t *tile) {
            if (active) {
                scores_softmax(it, tile, 0);
            } else if (lane == 0) {
                s_flagp[0][wave] = 0;
            }
            __syncthreads();  // every head's probabilities and rescale factors are in LDS
            value_product(tile, 0);
        };

        if constexpr (kFp8) {
            // raw ring of 3, bf16 double buffer; tile it + 1 is widened while
            // tile it is consumed
            if (ntile > 0) issue_tile(0);
            if (ntile > 1) issue_tile(1);
            if (ntile > 2) issue_tile(2);
            wait_all_but_two_tiles<kRawSlots>(ntile > 2, ntile > 1, wave);
            __syncthreads();
            if (ntile > 0) widen_tile(0);
            for (int32_t it = 0; it < ntile; ++it) {
                // raw tile it + 1 has landed (tile it + 2 may still be in flight)
                wait_all_but_one_tile<kRawSlots>(it + 2 < ntile, wave);
                __syncthreads();  // widened tile it complete; buffers of it - 1 free
                if (it + 3 < ntile) issue_tile(it + 3);
                if (it + 1 < ntile) widen_tile(it + 1);
                compute_tile(it, s_kv[it % 2]);
            }
        } else {
            // one barrier per tile: iteration it runs the value product of
            // tile it - 1 (probabilities of buffer (it - 1) % 2) and then the
            // scores of tile it (into buffer it % 2); ring of 3, tile it + 1 in
            // flight
            if (ntile > 0) issue_tile(0);
            for (int32_t it = 0; it <= ntile; ++it) {
                vm_wait<0>();     // tile it has landed (own copies) ...
                __syncthreads();  // ... for every wave; tile it - 1's probabilities are in
                                  // LDS, and tile it - 2's buffer is free
                if (it + 1 < ntile) issue_tile(it + 1);
                if (it >= 1) value_product(s_kv[(it - 1) % 3], (it - 1) & 1);
                if (it < ntile) {
                    if (active) scores_softmax(it, s_kv[it % 3], it & 1);
                    else if (lane == 0) s_flagp[it & 1][wave] = 0;
                }
            }
        }

        // ---- finish: full softmax sums, normalise, write this segment's partial ----
        float lt = l_run;
        lt += __shfl_xor(lt, 16, 64);
        lt += __shfl_xor(lt, 32, 64);
        bad = __syncthreads_or(bad);  // also: every wave is done with the LDS ring
        const bool empty = ntile == 0;
        if (active) {
            const int ln = lane_id_here();
            if (ln < 16) {
                s_linv[h0 + ln] = bad ? NAN : (empty ? 0.f : p.v_scale / lt);
                if (h0 + ln < p.H)
                    p.ws_l[slot * p.H + h0 + ln] =
                        bad ? NAN : (empty ? -INFINITY : (m_ref + fast_log2(lt)) * kLn2);
            }
        }
        __syncthreads();  // every head's 1 / row sum is in LDS
        {
            const int ln = lane_id_here();
            const int h2 = ln >> 5;
            float *o_dst = p.ws_o + slot * p.H * kDv + kVcW * wave + (ln & 31);
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) {
                if (hb >= nhb) break;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 iv = *reinterpret_cast<const float4 *>(s_linv + 32 * hb + 8 * q + 4 * h2);
                    const float ivs[4] = {iv.x, iv.y, iv.z, iv.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int h = 32 * hb + 8 * q + 4 * h2 + r;
                        if (h < p.H) {
#pragma unroll
                            for (int cb = 0; cb < 2; ++cb)
                                o_dst[(int64_t)h * kDv + 32 * cb] = o[hb][cb][4 * q + r] * ivs[r];
                        }
                    }
                }
            }
        }
        cc += nseg;
    }
}

template <bool kFp8>
int resident_wgs(int threads) {
    static int cached[2][64] = {{0}};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int &c = cached[kFp8 ? 1 : 0][dev];
    if (c == 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &n, reinterpret_cast<const void *>(mla_kernel<kFp8>), threads, 0) != hipSuccess ||
            n < 1)
            n = 1;
        c = n;
    }
    return c;
}

int log2_exact(int32_t x) {
    if (x <= 0 || (x & (x - 1))) return -1;
    int l = 0;
    while ((1 << l) < x) ++l;
    return l;
}

}  // namespace

MlaPlan plan_mla(const cp_mla_args &a) {
    MlaPlan pl{};
    const bool fp8 = a.kv_dt == CP_FP8_E4M3FN;
    const int wgs = device_cus() * (fp8 ? resident_wgs<true>(kThreads) : resident_wgs<false>(kThreads));
    pl.split_tokens = kT;
    pl.nsplit = wgs;  // tile ranges = workgroups launched
    const size_t slots = (size_t)wgs + (size_t)(a.B > 0 ? a.B : 0);
    pl.ws_bytes = slots * (size_t)a.H * (kDv + 1) * sizeof(float) + (size_t)a.B * 2 * 4 + 512;
    return pl;
}

}  // namespace cpattn

using namespace cpattn;

extern "C" cp_status cp_decode_attn_partial_mla(const cp_mla_args *a, void *ws, size_t ws_bytes,
                                                hipStream_t stream) {
    clear_error();
    if (!a) return fail(CP_E_INVALID, "cp_decode_attn_partial_mla: NULL args");
    if (a->B < 0 || a->H < 1 || a->Dk < 1 || a->Dv < 1 || a->bs < 1 || a->bt_stride < 1 ||
        a->num_blocks < 0)
        return fail(CP_E_INVALID, "mla decode: B=%d H=%d Dk=%d Dv=%d bs=%d bt_stride=%d", a->B,
                    a->H, a->Dk, a->Dv, a->bs, a->bt_stride);
    if (a->Dk != kDk || a->Dv != kDv)
        return fail(CP_E_UNSUPPORTED, "mla decode: latent %d / value %d (576 / 512 supported)",
                    a->Dk, a->Dv);
    if (a->H % 16 != 0 || a->H > kHeadsWg)
        return fail(CP_E_UNSUPPORTED, "mla decode: H=%d (a multiple of 16 up to 128)", a->H);
    if (a->kv_dt != CP_BF16 && a->kv_dt != CP_FP8_E4M3FN)
        return fail(CP_E_UNSUPPORTED, "mla decode: latent dtype must be BF16 or FP8_E4M3FN");
    const int bs_log2 = log2_exact(a->bs);
    if (bs_log2 < 4)
        return fail(CP_E_UNSUPPORTED, "mla decode: block size %d must be a power of two >= 16",
                    a->bs);
    if (a->B > kMaxB) return fail(CP_E_UNSUPPORTED, "mla decode: B=%d > %d", a->B, kMaxB);
    if (!(a->scale == a->scale) || !(a->kv_scale == a->kv_scale))
        return fail(CP_E_INVALID, "mla decode: NaN scale");
    if (a->B == 0) return CP_OK;
    if (!a->q || !a->kv_cache || !a->block_table || !a->local_len || !a->out || !a->lse)
        return fail(CP_E_INVALID, "mla decode: NULL pointer");
    if (!aligned16(a->q) || !aligned16(a->kv_cache) || !aligned16(a->out))
        return fail(CP_E_INVALID, "mla decode: q, cache and out must be 16-byte aligned");
    const MlaPlan pl = plan_mla(*a);
    if (!ws || ws_bytes < pl.ws_bytes)
        return fail(CP_E_WORKSPACE, "mla decode: workspace of %zu bytes needed, %zu given",
                    pl.ws_bytes, ws_bytes);
    const bool fp8 = a->kv_dt == CP_FP8_E4M3FN;
    const size_t slots = (size_t)pl.nsplit + (size_t)a->B;
    float *ws_o = static_cast<float *>(ws);
    float *ws_l = ws_o + slots * a->H * kDv;
    int32_t *seg = reinterpret_cast<int32_t *>(
        (reinterpret_cast<uintptr_t>(ws_l + slots * a->H) + 255) & ~uintptr_t(255));

    MlaParams p;
    p.q = to_global(a->q);
    p.kv = to_global(a->kv_cache);
    p.bt = to_const(a->block_table);
    p.len = to_const(a->local_len);
    p.B = a->B;
    p.H = a->H;
    p.bs_log2 = bs_log2;
    p.bt_stride = a->bt_stride;
    p.num_blocks = a->num_blocks;
    const float kvs = fp8 ? a->kv_scale : 1.f;
    p.qk_scale = a->scale * kvs * kLog2e;
    p.v_scale = kvs;
    p.W = pl.nsplit;
    p.ws_o = ws_o;
    p.ws_l = ws_l;
    p.seg = seg;
    if (fp8)
        hipLaunchKernelGGL(mla_kernel<true>, dim3(pl.nsplit), dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(mla_kernel<false>, dim3(pl.nsplit), dim3(kThreads), 0, stream, p);
    cp_status st = check_launch("cp_decode_attn_partial_mla");
    if (st != CP_OK) return st;

    MergeDesc m;
    m.seg = seg;
    m.rows_per_seg = a->H;
    m.n_parts = 0;
    m.rows = (int64_t)a->B * a->H;
    m.Dv = kDv;
    m.part_out = ws_o;
    m.part_lse = ws_l;
    m.o_part_stride = (int64_t)a->H * kDv;
    m.o_row_stride = kDv;
    m.l_part_stride = a->H;
    m.l_row_stride = 1;
    m.out = a->out;
    m.out_dt = CP_F32;
    m.lse_out = a->lse;
    return launch_merge(m, stream);
}
