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
// Design (a dense contraction: up to 128 heads x 576 against every cached row;
// at one workgroup per CU both matrix products stream every operand from LDS,
// so the count of LDS instructions per 32-token tile sets the pace):
//   * one workgroup per CU = 4 waves, one per SIMD, each with the whole
//     512-entry register file.  Wave w computes the scores and the online
//     softmax of query heads 32 w .. 32 w + 31 (their queries stay in 144
//     VGPRs) and the value product of every head for output columns
//     128 w .. 128 w + 127 (O[128 heads][128 columns] in 256 AGPRs), so each
//     value column of a tile is read from LDS by one wave only.  The
//     probabilities and lazy-rescale factors pass between waves through a
//     double-buffered LDS exchange, ordered by the one barrier per tile;
//   * both products on v_mfma_f32_32x32x16_bf16: scores S[32 tokens][32 heads]
//     = C Q^T in one accumulation chain (A = latent rows from LDS, B = the
//     wave's queries), then O[32 heads][32 columns] += P V (A = the
//     probabilities of a 32-head block, in the A-operand layout of the score
//     accumulator; B = latent rows read by the transposing LDS read
//     ds_read_b64_tr_b16 and shared by the four head blocks, the token order
//     inside each 16-token step permuted identically on both operands);
//   * software pipeline, one barrier per tile: iteration it computes the
//     scores of tile it, then the value product of tile it - 1 with the
//     softmax of tile it cut into pieces between its MFMAs (a VALU
//     instruction issued while an MFMA runs costs ~6 cycles, an MFMA 32);
//   * online softmax in the exp2 domain with a lazily raised reference
//     maximum: O is rescaled only when a tile's maximum exceeds the reference
//     by more than 2^8 (rare; the rescale multiplies the AGPR accumulators in
//     place, between the value products of the two tiles), which keeps every
//     probability <= 256;
//   * the MFMAs are issued from asm so that each accumulator keeps its
//     register file; their latencies (results, operand reads) are handled
//     explicitly (mfma_drain, keep);
//   * staging: HBM -> LDS by global_load_lds (no registers), issued from asm
//     and waited for with explicit vmcnt counts, in a ring of 3 bf16 tiles:
//     tile it + 1's nine copies per wave are spread over the score MFMAs of
//     iteration it.  fp8 E4M3: one raw tile lands per iteration; each lane
//     widens the chunks it copied (exactly) into the bf16 ring one tile ahead
//     of use; the per-tensor scale is folded into the score scale and the
//     output;
//   * LDS tiles are stored as nine groups of 8 chunks (16 bytes each), each
//     group row-major over the 32 rows with 128-byte rows, the chunks of row t
//     XOR-swizzled (swz below): a wave's copy of one group of its 8 rows is 1 KB
//     of contiguous LDS, and the 16 rows of a score-operand read and the 4-row
//     blocks of the transposing value reads hit distinct banks;
//   * a balanced schedule: request b (n_b tiles) is cut into k_b equal tile
//     ranges with sum k_b <= CUs, one workgroup per range, all resident at
//     once; partials go to slot = workgroup (outputs in bf16, half the bytes
//     of the write here and of the read in the merge; LSEs in fp32) and are
//     merged exactly afterwards by a segment table.  Per-request tile counts are prefix-summed per
//     64-request chunk in LDS and resolved within a chunk by a wave scan.
#include <math.h>

#include <type_traits>

#include "internal.hpp"

// The asm below writes M0 (reserved for the compiler, which uses it for
// nothing in this file) and names it as clobbered.
#pragma clang diagnostic ignored "-Winline-asm"

namespace cpattn {

namespace {

constexpr int kDk = 576, kDv = 512;
constexpr int kT = 32;                   // tokens per tile / per scheduling chunk
constexpr int kRowB = kDk * 2;           // bf16 LDS row: 1152 bytes = 72 chunks of 16
constexpr int kRowC = kRowB / 16;
constexpr int kTileB = kT * kRowB;       // 36,864 bytes
// LDS tile layout: nine groups of 8 chunks; group g holds chunks 8 g .. 8 g + 7
// of all 32 rows, row-major with 128-byte rows (chunk c of row t at
// kGroupB * (c / 8) + 128 t + 16 ((c % 8) ^ swz(t))), so that the chunk group
// of any 8 consecutive rows is 1 KB of contiguous LDS: one 64-lane copy
constexpr int kGroupB = kT * 128;        // 4,096 bytes
constexpr int kRawRowB = kDk;            // fp8 row: 576 bytes = 36 chunks
constexpr int kRawRowC = kRawRowB / 16;
constexpr int kRawTileB = kT * kRawRowB; // 18,432 bytes
constexpr int kKs = kDk / 16;            // 36 k-steps of the score MFMA
constexpr int kWaves = 4;                // one per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kHW = 32;                  // query heads per wave
constexpr int kHeadsWg = kHW * kWaves;   // 128
constexpr int kMaxB = 4096;
constexpr int kChunkB = 64;              // requests per prefix-sum chunk
constexpr int kMaxChunks = kMaxB / kChunkB;
constexpr float kLazy = 8.f;             // rescale only past 2^8
constexpr float kLazyW = 256.f;          // 2^kLazy
constexpr int kTabTiles = 1024;          // tile rows held in LDS (longer segments load them)
// bf16: ring of 3 tiles, tile it + 1 copied while tiles it and it - 1 are
// read; wave w copies rows 8 w .. 8 w + 7 of every tile (nine 64-lane copies)
constexpr int kStagesBf = 3;
constexpr int kCopiesBf = 8 * kRowC / 64;  // 9
// fp8: one raw tile (18 copies, wave w taking w, w + 4, ...), widened into a
// ring of 3 bf16 tiles
constexpr int kStagesF8 = 3, kRawStages = 1;
// value product: wave w accumulates O[all 128 heads][128 w .. 128 w + 127] as
// 4 head blocks x 4 column blocks of 32 x 32
constexpr int kHb = kHeadsWg / 32, kCbW = kDv / 32 / kWaves;
constexpr int kRawSlots = kT * kRawRowC / 64;  // 18
static_assert(8 * kRowC % 64 == 0 && kT * kRawRowC % 64 == 0, "whole 64-chunk copies");
static_assert(kRowC % 8 == 0, "the chunk swizzle permutes aligned groups of 8");
static_assert(kStagesBf * kTileB + 17 * 1024 <= 150 * 1024 &&
                  kStagesF8 * kTileB + kRawStages * kRawTileB + 17 * 1024 <= 150 * 1024,
              "tile rings and the probability exchange fit the LDS");
static_assert(kHb == 4 && kCbW == 4, "four waves: 4 head blocks, 4 column blocks each");

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) const uint8_t lds_u8;
typedef __attribute__((address_space(3))) uint8_t lds_w8;

struct MlaParams {
    const gbyte *q, *kv;
    cint32 *bt, *len;
    int32_t B, H, bs_log2, bt_stride;
    int32_t num_blocks;  // the host checks num_blocks * bs < 2^31: cache rows are 32-bit
    int32_t cap;         // bt_stride * bs, clamped to 2^31 - 1 (the most tokens a table holds)
    float qk_scale;   // |scale| * kv_scale * log2(e)
    uint32_t q_sign;  // 0x80008000 when the scale is negative (queries negated), else 0
    float v_scale;    // kv_scale (fp8) or 1
    int32_t W;        // tile ranges = workgroups launched
    float *ws_o;      // [slots][H][512] bf16 (the split partials; fp32 LSEs beside them)
    float *ws_l;      // [slots][H]
    int32_t *seg;     // [B][2]
};

// D (32 x 32) += A (32 x 16) B (16 x 32); lane l holds A[l % 32][8 (l / 32) + e],
// B[8 (l / 32) + e][l % 32] (e = 0 .. 7) and D[8 (e / 4) + 4 (l / 32) + e % 4][l % 32]
// (e = 0 .. 15).
//
// Issued from asm so that each accumulator keeps the register file it is
// given: the score accumulators in VGPRs (the softmax reads them), the output
// accumulators in AGPRs (only MFMAs and the rescale touch them).  The compiler
// waits for the LDS reads feeding A and B (operand tracking) but does not see
// the MFMA's own latency: a VALU read of an accumulator written by these
// follows at least 19 wait states (mfma_drain), and the AGPR accumulators are
// read only after such a drain.  Dependent accumulations into the same
// registers need no wait states.
__device__ __forceinline__ void mfma32_v(f32x16_t &c, const u32x4_t &a, const u32x4_t &b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_v0(f32x16_t &c, const u32x4_t &a, const u32x4_t &b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_a(f32x16_t &c, const u32x4_t &a, const u32x4_t &b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
//
// The drain is fenced by scheduling barriers: without them the scheduler
// moves register arithmetic above the s_nops, where it reads an accumulator
// before the MFMA has written it, or takes one of the MFMA's destination
// registers for another value that the MFMA's write-back then overwrites.
__device__ __forceinline__ void mfma_drain() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}
// The compiler also does not know that an asm MFMA reads its A and B
// registers after issue: left to itself it reuses them for the very next VALU
// result.  keep(x) marks x as read at that point, so an operand stays
// allocated until the next MFMA has issued (by which time the previous one
// has read its operands) or until after mfma_drain().
__device__ __forceinline__ void keep(const u32x4_t &x) { asm volatile("" ::"v"(x)); }
// row of accumulator element e in lane half h
__device__ __forceinline__ constexpr int acc_row(int e, int h) { return 8 * (e >> 2) + 4 * h + (e & 3); }

// Chunk c (16 bytes) of tile row t sits at position c ^ swz(t) of its group of
// 8.  With u = (t / 2) % 8, swz = 4 (u % 2) + u / 2: over the rows of one parity
// it takes all 8 values (16 consecutive rows of one chunk -- score-operand reads,
// fp8 widening writes -- hit 16 distinct bank slots of 256 bytes, rows t and
// t + 1 being 128 bytes apart), and rows t, t + 2 with t % 4 < 2 land in
// opposite halves of the group (the 4-row x 4-chunk blocks of the transposing
// value reads are conflict-free too; (t / 2) % 8 alone gives them two-way
// conflicts).
__device__ __forceinline__ int swz(int t) {
    const int u = (t >> 1) & 7;
    return ((u & 1) << 2) | (u >> 1);
}

// max / sum of x over lanes l and l ^ 32 (v_permlane32_swap exchanges the
// upper half of its first operand with the lower half of its second: with x
// in both, the two results hold x[l % 32] and x[32 + l % 32] in every lane).
__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One 64-lane HBM -> LDS copy: lane i moves 16 bytes from `src` to LDS byte
// lds + 16 i.  `lds` must be wave-uniform.  Issued from asm so that the
// compiler's wait insertion does not tie later LDS reads to it; every reader
// waits explicitly (vm_wait + barrier) before touching the destination.
// (M0 is written here and read by nothing the compiler emits in this file.)
__device__ __forceinline__ void dma16(gbyte *src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds), "v"(src)
                 : "m0");
}
// The same from src + kOff to lds, with kOff as the instruction's immediate
// offset (so that the copies of one tile share one address register).  The
// immediate offset is added to the LDS address as well as to the global one,
// so M0 is set to lds - kOff.  dma16_group(i, ..) takes kOff = 128 i (i is a
// constant once the caller's loop is unrolled).
template <int kOff>
__device__ __forceinline__ void dma16_off(gbyte *src, uint32_t lds) {
    static_assert(kOff >= 0 && kOff < 4096, "global offset range");
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:%2"
                 :
                 : "s"(lds - (uint32_t)kOff), "v"(src), "i"(kOff)
                 : "m0");
}
__device__ __forceinline__ void dma16_group(int i, gbyte *src, uint32_t lds) {
    switch (i) {
        case 0: dma16_off<0>(src, lds); break;
        case 1: dma16_off<128>(src, lds); break;
        case 2: dma16_off<256>(src, lds); break;
        case 3: dma16_off<384>(src, lds); break;
        case 4: dma16_off<512>(src, lds); break;
        case 5: dma16_off<640>(src, lds); break;
        case 6: dma16_off<768>(src, lds); break;
        case 7: dma16_off<896>(src, lds); break;
        default: dma16_off<1024>(src, lds); break;
    }
}

// Multiply accumulator element e of one output block, held in an AGPR, by f
// (the rescale of the online softmax).  Written as AGPR-level asm so that the
// accumulators keep their AGPR home: with plain C++ the compiler moves all 256
// of them to VGPRs around the (rare) rescale and spills the queries.  The
// caller separates it from the MFMAs that wrote the accumulators.
__device__ __forceinline__ void scale_acc_agpr(f32x16_t &o, int e, float f) {
    float x = o[e];
    float t;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(x), "=&v"(t)
                 : "v"(f));
    o[e] = x;
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]).  Issued as
// the builtin so that the compiler's own wait tracking sees it.
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Inclusive prefix sum of x over the 64 lanes.
__device__ __forceinline__ int32_t wave_incl_scan(int32_t x, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t o = __shfl_up(x, d, 64);
        if (lane >= d) x += o;
    }
    return x;
}

template <bool kFp8>
__global__ void __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_kernel(MlaParams p) {
    // Iteration it reads tile it (scores) and tile it - 1 (value product), in
    // a ring of 3 bf16 tiles: tile it + 1 goes to the position of tile it - 2
    // (last read in iteration it - 1).  bf16: copied during iteration it.  fp8:
    // the raw tile it + 1 (copied during iteration it - 1) is widened at the
    // start of iteration it, then raw tile it + 2 is copied into the one raw
    // position (each lane widens and re-fills only the chunks it copies).
    constexpr int kStages = kFp8 ? kStagesF8 : kStagesBf;
    constexpr int kRaw = kFp8 ? kRawStages : 1;
    __shared__ __attribute__((aligned(16))) uint8_t s_kv[kStages][kTileB];
    __shared__ __attribute__((aligned(16))) uint8_t s_raw[kRaw][kFp8 ? kRawTileB : 16];
    __shared__ int32_t s_chunk[kMaxChunks];     // per 64-request chunk: tiles, then ranges
    __shared__ int32_t s_kc[kMaxChunks];        // per chunk: non-empty requests
    __shared__ int32_t s_ksum[kMaxChunks + 1];  // ranges of requests [0, 64 c)
    __shared__ int32_t s_rtot, s_bn;
    // cache rows of the segment's tiles (first token, token 16), filled once
    __shared__ __attribute__((aligned(8))) int32_t s_rows[kTabTiles][2];
    // probabilities of every wave's 32 heads for the value product of all
    // waves, [tile parity][wave][16-token step][lane] in the A-operand layout;
    // the lazy-rescale factors of those heads and a per-wave "rescaled" flag;
    // the softmax sums of every head for the final normalisation
    __shared__ __attribute__((aligned(16))) u32x4_t s_p[2][kWaves][2][64];
    __shared__ __attribute__((aligned(16))) float s_alpha[2][kWaves][32];
    __shared__ __attribute__((aligned(16))) int32_t s_aflag[2][kWaves];
    __shared__ __attribute__((aligned(16))) float s_lsum[kWaves][32];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h0 = wave * kHW;
    // The lane id passed through an empty asm: a fresh value at each use, so
    // that per-lane addresses derived from it are recomputed where they are
    // used instead of hoisted out of the tile loop into registers (no
    // instruction, where v_mbcnt would cost two).
    auto lane_now = [&]() -> int {
        int l = lane;
        asm volatile("" : "+v"(l));
        return l;
    };
    const int r32 = lane & 31, h2 = lane >> 5;
    const int32_t cap = p.cap;
    const int bs = 1 << p.bs_log2;
    const int nch = (p.B + kChunkB - 1) / kChunkB;

    // ---- the schedule: request b (n_b tiles) is cut into k_b equal tile ranges,
    // k_b = min(n_b, 1 + floor(n_b (C - Bn) / R)) with C workgroups per wave
    // (one per CU), Bn non-empty requests and R tiles in all, so that
    // sum k_b <= C: one workgroup per range, all of them resident at once,
    // each range at most R / (C - Bn) tiles (exactly R / C for equal lengths).
    // Workgroup g takes range g - K_b of the request b with K_b <= g < K_b + k_b
    // (K_b = sum of k over earlier requests) and writes partial slot g. ----
    auto tiles_of = [&](int b) -> int32_t {
        if (b >= p.B) return 0;
        const int32_t L = p.len[b];
        if (L < 0 || L > cap) return 1;  // invalid length: one NaN tile
        return (L + kT - 1) / kT;
    };
    for (int c = wave; c < nch; c += kWaves) {
        const int32_t n = tiles_of(c * kChunkB + lane);
        int32_t t = n, ne = n > 0;
#pragma unroll
        for (int x = 32; x >= 1; x >>= 1) {
            t += __shfl_xor(t, x, 64);
            ne += __shfl_xor(ne, x, 64);
        }
        if (lane == 0) {
            s_chunk[c] = t;
            s_kc[c] = ne;
        }
    }
    __syncthreads();
    if (tid < 64) {
        const int32_t incl = wave_incl_scan(tid < nch ? s_chunk[tid] : 0, lane);
        const int32_t ne = wave_incl_scan(tid < nch ? s_kc[tid] : 0, lane);
        if (tid == 63) {
            s_rtot = incl;
            s_bn = ne;
        }
    }
    __syncthreads();
    const int32_t R_tot = s_rtot;
    const int32_t Cq = max(p.W - s_bn, 0);
    auto ks_of = [&](int b) -> int32_t {
        const int32_t n = tiles_of(b);
        if (n == 0) return 0;
        return min(n, 1 + (int32_t)((int64_t)n * Cq / R_tot));
    };
    if (R_tot > 0) {
        for (int c = wave; c < nch; c += kWaves) {
            int32_t k = ks_of(c * kChunkB + lane);
#pragma unroll
            for (int x = 32; x >= 1; x >>= 1) k += __shfl_xor(k, x, 64);
            if (lane == 0) s_chunk[c] = k;
        }
    }
    __syncthreads();
    if (tid < 64) {
        const int32_t incl = wave_incl_scan(tid < nch && R_tot > 0 ? s_chunk[tid] : 0, lane);
        s_ksum[tid + 1] = incl;
        if (tid == 0) s_ksum[0] = 0;
    }
    __syncthreads();
    if (blockIdx.x == 0) {  // the split combine's segment table
        for (int c = wave; c < nch; c += kWaves) {
            const int b = c * kChunkB + lane;
            const int32_t k = R_tot > 0 ? ks_of(b) : 0;
            const int32_t incl = wave_incl_scan(k, lane);
            if (b < p.B) {
                p.seg[2 * b] = s_ksum[c] + incl - k;
                p.seg[2 * b + 1] = k;
            }
        }
    }
    const int32_t g = blockIdx.x;
    if (R_tot == 0 || g >= s_ksum[nch]) return;
    // the request of workgroup g: its chunk by binary search, its lane by a scan
    int lo = 0;
    {
        int hic = nch;
        while (hic - lo > 1) {
            const int mid = (lo + hic) >> 1;
            if (s_ksum[mid] <= g) lo = mid;
            else hic = mid;
        }
    }
    int b;
    int32_t kb, Kb;
    {
        const int32_t k = ks_of(lo * kChunkB + lane);
        const int32_t incl = wave_incl_scan(k, lane);
        const uint64_t m = __ballot(incl > g - s_ksum[lo]);
        const int first = __builtin_ffsll((long long)m) - 1;
        b = __builtin_amdgcn_readfirstlane(lo * kChunkB + first);
        kb = __builtin_amdgcn_readfirstlane(__shfl(k, first, 64));
        Kb = s_ksum[lo] + __builtin_amdgcn_readfirstlane(__shfl(incl, first, 64)) - kb;
    }
    const int32_t nreq = tiles_of(b), j = g - Kb;
    const int32_t k = (int32_t)((int64_t)j * nreq / kb);
    const int32_t nseg = (int32_t)((int64_t)(j + 1) * nreq / kb) - k;
    const int32_t Lraw = p.len[b];
    bool bad = Lraw < 0 || Lraw > cap;
    const int32_t L = bad ? 0 : Lraw;
    const int32_t s0 = k * kT;
    const int32_t s1 = min(s0 + nseg * kT, L);
    const int32_t ntile = s1 > s0 ? (s1 - s0 + kT - 1) / kT : 0;
    const int32_t slot = g;
    cint32 *bt_row = p.bt + (int64_t)b * p.bt_stride;

    // ---- per-lane LDS offsets ----
    // score operand, k-step ks: row r32, chunk 2 ks + h2, i.e. group ks / 4,
    // position 2 (ks % 4) + h2 within it (swizzled)
    const int ln = lane_now();  // (recomputed per segment, not carried across)
    uint32_t kofs[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        kofs[q] = (ln & 31) * 128 + 16 * ((2 * q + (ln >> 5)) ^ swz(ln & 31));
    // value operand of column block cb, 16-token step kk, row half hr: in the
    // 16-lane group of column half c = (l / 16) % 2, lane j reads row
    // 16 kk + 4 h2 + j / 4 + 8 hr, chunk 4 cb + 2 c + (j % 4) / 2, byte 8 (j % 2)
    // (the swizzle of those rows does not depend on kk)
    uint32_t vofs[2][2];
    {
        const int j = ln & 15, g2 = (ln >> 4) & 1, lh = ln >> 5;
        const int cg = 2 * g2 + ((j & 3) >> 1);
#pragma unroll
        for (int c1 = 0; c1 < 2; ++c1)
#pragma unroll
            for (int hr = 0; hr < 2; ++hr) {
                const int row = 4 * lh + (j >> 2) + 8 * hr;
                vofs[c1][hr] = row * 128 + 16 * ((4 * c1 + cg) ^ swz(row)) + 8 * (j & 1);
            }
    }
    // copy offsets.  bf16: copy i of wave w moves chunk group i of the wave's
    // rows 8 w .. 8 w + 7 (1 KB of LDS); lane l takes row 8 w + l / 8, LDS
    // position l % 8 of the group, i.e. source chunk 8 i + ((l % 8) ^ swz(row)):
    // source offset coff + 128 i from the wave's first row.
    // fp8: copy i of wave w is raw slot w + 4 i: lane l moves row l % 32, chunk
    // 2 (w + 4 i) + l / 32 of the raw tile (the raw ring is [slot][lane]).
    constexpr int kNc = kFp8 ? (kRawSlots + kWaves - 1) / kWaves : kCopiesBf;
    const int ncopy = kFp8 ? (wave < kRawSlots % kWaves ? kNc : kNc - 1) : kNc;  // this wave's
    const uint32_t ccol = (uint32_t)(16 * ((ln & 7) ^ swz(8 * wave + (ln >> 3))));

    const uint32_t kv_lds = (uint32_t)(uintptr_t)(lds_u8 *)(&s_kv[0][0]);
    const uint32_t raw_lds = (uint32_t)(uintptr_t)(lds_u8 *)(&s_raw[0][0]);

    // ---- the cache rows of every tile of the segment into LDS (the loop then
    // reads them with the LDS reads it waits for anyway; scalar loads in the
    // loop would force waits for every LDS read in flight) ----
    const bool tab = ntile <= kTabTiles;
    if (tab) {
        for (int32_t jt = tid; jt < ntile; jt += kThreads) {
            const int32_t tb = s0 + jt * kT;
            const int32_t nv = min(kT, s1 - tb);
            const int32_t t1 = tb + min(16, nv - 1);
            const int32_t ph0 = bt_row[tb >> p.bs_log2], ph1 = bt_row[t1 >> p.bs_log2];
            const bool ok0 = (uint32_t)ph0 < (uint32_t)p.num_blocks;
            const bool ok1 = (uint32_t)ph1 < (uint32_t)p.num_blocks;
            bad |= !(ok0 && ok1);
            s_rows[jt][0] = ((ok0 ? ph0 : 0) << p.bs_log2) + (tb & (bs - 1));
            s_rows[jt][1] = ((ok1 ? ph1 : 0) << p.bs_log2) + (t1 & (bs - 1));
        }
    }

    // ---- the wave's 32 queries as the score B operand:
    // Q[h0 + l % 32][16 ks + 8 (l / 32) .. +8] (heads past H load head H - 1;
    // their rows are computed and never written) ----
    u32x4_t qb[kKs];
    {
        const int hq = min(h0 + r32, p.H - 1);
        gbyte *qrow = p.q + ((int64_t)b * p.H + hq) * kRowB + h2 * 16;
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) {
            qb[ks] = load16(qrow + ks * 32);
            qb[ks] ^= p.q_sign;
        }
    }
    vm_wait<0>();     // the queries are in registers before any tile copy is issued
    __syncthreads();  // the row table is complete

    // ---- tile copies ----
    // Cache rows of tile j: a 32-token tile spans at most two blocks
    // (bs >= 16): r0 is the row of its first token, r1 that of token 16.
    // Tokens past the segment's end reuse the row of its last token (finite
    // data; their probability is forced to 0).
    struct TileSrc {
        int32_t r0, r1;  // cache rows (32-bit: num_blocks * bs < 2^31)
        int32_t nval;
    };
    auto tile_src = [&](int32_t j) -> TileSrc {
        const int32_t tb = s0 + j * kT;
        const int32_t nval = min(kT, s1 - tb);
        if (tab) {
            TileSrc ts;
            ts.r0 = __builtin_amdgcn_readfirstlane(s_rows[j][0]);
            ts.r1 = __builtin_amdgcn_readfirstlane(s_rows[j][1]);
            ts.nval = nval;
            return ts;
        }
        auto row_of = [&](int32_t tok) -> int32_t {
            const int32_t phys = bt_row[tok >> p.bs_log2];
            const bool ok = (uint32_t)phys < (uint32_t)p.num_blocks;
            bad |= !ok;
            return ((ok ? phys : 0) << p.bs_log2) + (tok & (bs - 1));
        };
        TileSrc ts;
        ts.r0 = row_of(tb);
        ts.r1 = row_of(tb + min(16, nval - 1));  // == r0 + 16 within one block
        ts.nval = nval;
        return ts;
    };
    // copy i of tile j (this wave's share) into its ring position
    auto issue_copy = [&](const TileSrc &ts, int32_t j, int i) {
        if constexpr (kFp8) {
            // raw slot sl: lane l moves row l % 32, chunk 2 sl + l / 32 of the tile
            if (i >= ncopy) return;
            const int sl = wave + kWaves * i;
            const uint32_t dst = raw_lds + (uint32_t)((j % kRaw) * kRawTileB + sl * 1024);
            const int l = lane_now();
            const int t = l & 31, pos = 2 * sl + (l >> 5);
            const int tt = min(t, ts.nval - 1);
            const int32_t row = tt < 16 ? ts.r0 + tt : ts.r1 - 16 + tt;
            dma16(p.kv + (int64_t)row * kRawRowB + 16 * pos, __builtin_amdgcn_readfirstlane(dst));
        } else {
            const uint32_t dst = kv_lds + (uint32_t)((j % kStagesBf) * kTileB + i * kGroupB +
                                                     8 * wave * 128);
            const int t = 8 * wave + (lane_now() >> 3);
            const int tt = min(t, ts.nval - 1);
            const int32_t row = tt < 16 ? ts.r0 + tt : ts.r1 - 16 + tt;
            dma16(p.kv + (int64_t)row * kRowB + ccol + 128 * i, __builtin_amdgcn_readfirstlane(dst));
        }
    };
    auto issue_tile = [&](int32_t j) {
        const TileSrc ts = tile_src(j);
#pragma unroll
        for (int i = 0; i < kNc; ++i) issue_copy(ts, j, i);
    };
    // fp8: widen the raw chunks this lane copied for tile j into bf16 ring
    // position j % 3 (exact: every E4M3 value is a bf16 value)
    auto widen_tile = [&](int32_t j) {
        if constexpr (kFp8) {
            lds_u8 *raw = (lds_u8 *)(&s_raw[j % kRaw][0]);
            lds_w8 *dst = (lds_w8 *)(&s_kv[j % kStages][0]);
            // every read first, then the conversions and writes (one LDS latency)
            // (lane l holds row l % 32 of chunk column 2 sl + l / 32: a 16-lane group
            // writes one chunk column of 16 rows, which hit distinct banks)
            u32x4_t xs[kNc];
#pragma unroll
            for (int i = 0; i < kNc; ++i) {
                if (i >= ncopy) break;
                const int sl = wave + kWaves * i;
                xs[i] = *(__attribute__((address_space(3))) const u32x4_t *)(raw + sl * 1024 +
                                                                               16 * lane_now());
            }
#pragma unroll
            for (int i = 0; i < kNc; ++i) {
                if (i >= ncopy) break;
                const int l = lane_now();
                const int t = l & 31, pos = 2 * (wave + kWaves * i) + (l >> 5);
                const u32x4_t x = xs[i];
                u32x4_t lo2, hi2;
#pragma unroll
                for (int wd = 0; wd < 4; ++wd) {
                    const uint32_t a = __builtin_bit_cast(
                        uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[wd], 1.f, false));
                    const uint32_t b2 = __builtin_bit_cast(
                        uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[wd], 1.f, true));
                    if (wd < 2) {
                        lo2[2 * wd] = a;
                        lo2[2 * wd + 1] = b2;
                    } else {
                        hi2[2 * (wd - 2)] = a;
                        hi2[2 * (wd - 2) + 1] = b2;
                    }
                }
                // bf16 chunks 2 pos and 2 pos + 1 of row t: group pos / 4,
                // positions 2 (pos % 4) and 2 (pos % 4) + 1 (swizzled)
                lds_w8 *row = dst + (pos >> 2) * kGroupB + t * 128;
                const int q2 = 2 * (pos & 3);
                *(__attribute__((address_space(3))) u32x4_t *)(row + 16 * (q2 ^ swz(t))) = lo2;
                *(__attribute__((address_space(3))) u32x4_t *)(row + 16 * ((q2 + 1) ^ swz(t))) = hi2;
            }
        }
    };
    // wait until this wave's copies of all but the newest `pend` tiles landed
    auto wait_copies = [&](int pend) {
        if constexpr (kFp8) {
            if (pend <= 0) vm_wait<0>();
            else if (pend == 1) {
                if (ncopy == kNc) vm_wait<kNc>();
                else vm_wait<kNc - 1>();
            } else {
                if (ncopy == kNc) vm_wait<2 * kNc>();
                else vm_wait<2 * (kNc - 1)>();
            }
        } else {
            if (pend <= 0) vm_wait<0>();
            else if (pend == 1) vm_wait<kCopiesBf>();
            else vm_wait<2 * kCopiesBf>();
        }
    };

    // ---- online-softmax state of head h0 + l % 32 (the same in both halves) ----
    float m_ref = -INFINITY, l_run = 0.f;
    // O[32 hb + acc_row(e, h2)][128 w + 32 cb + l % 32] in o[4 hb + cb]
    f32x16_t o[kHb * kCbW];
#pragma unroll
    for (int x = 0; x < kHb * kCbW; ++x)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[x][e] = 0.f;

    // Operand reads address a tile through per-lane base registers made opaque
    // to the compiler, so that every read of the tile is base + an immediate
    // offset (otherwise the ring index is folded into one hoisted address
    // register per read, which the register file cannot hold).
    auto tile_ptr = [&](int32_t j) -> uint32_t {
        return kv_lds + (uint32_t)(j % kStages) * (uint32_t)kTileB;
    };
    auto opaque = [](uint32_t x) {
        asm volatile("" : "+v"(x));
        return x;
    };
    struct KBase { uint32_t a[4]; };
    struct VBase { uint32_t a[2][2]; };
    auto k_base = [&](uint32_t t) {
        KBase kb;
#pragma unroll
        for (int q = 0; q < 4; ++q) kb.a[q] = opaque(t + kofs[q]);
        return kb;
    };
    // this wave's value columns 128 w .. 128 w + 127 are chunk groups 2 w, 2 w + 1
    auto v_base = [&](uint32_t t) {
        VBase vb;
#pragma unroll
        for (int c1 = 0; c1 < 2; ++c1)
#pragma unroll
            for (int hr = 0; hr < 2; ++hr)
                vb.a[c1][hr] = opaque(t + (uint32_t)(2 * wave * kGroupB) + vofs[c1][hr]);
        return vb;
    };
    auto read_k = [&](const KBase &kb, int ks) -> u32x4_t {
        return *(__attribute__((address_space(3))) const u32x4_t *)(
            (lds_u8 *)(uintptr_t)kb.a[ks & 3] + kGroupB * (ks >> 2));
    };
    // B operand of 16-token step kk, column block cb of this wave
    auto read_v = [&](const VBase &vb, int kk, int cb) -> u32x4_t {
        const int off = kk * 16 * 128 + kGroupB * (cb >> 1);
        const i16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_t *)((lds_u8 *)(uintptr_t)vb.a[cb & 1][0] + off));
        const i16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_t *)((lds_u8 *)(uintptr_t)vb.a[cb & 1][1] + off));
        const u32x2_t w0 = __builtin_bit_cast(u32x2_t, t0), w1 = __builtin_bit_cast(u32x2_t, t1);
        return u32x4_t{w0[0], w0[1], w1[0], w1[1]};
    };

    // ---- prologue ----
    if constexpr (kFp8) {
        // raw tile 0 landed and widened, raw tile 1 in flight
        if (ntile > 0) {
            issue_tile(0);
            wait_copies(0);
            widen_tile(0);
        }
        if (ntile > 1) issue_tile(1);
    } else {
        if (ntile > 0) issue_tile(0);
    }

    // O[hb][cb] += P[hb][kk] V[kk][cb] over tile t (probabilities of parity
    // buffer pb), 32 MFMAs, each value operand feeding the four head blocks;
    // side(i) after MFMA i
    // The first operands (probabilities of step 0, the first two value
    // operands) are read by vp_begin, which the caller issues early.
    struct VpOps {
        VBase tv;
        uint32_t pp;  // this lane's probabilities in parity buffer pb (entry [0][0])
        u32x4_t pa[kHb][2];
        u32x4_t vq[3];
    };
    // probabilities of head block hb, 16-token step kk: an immediate offset from op.pp
    auto read_p = [&](const VpOps &op, int hb, int kk) -> u32x4_t {
        return *(__attribute__((address_space(3))) const u32x4_t *)(
            (lds_u8 *)(uintptr_t)op.pp + (hb * 2 + kk) * 64 * 16);
    };
    auto vp_begin = [&](uint32_t t, int pb, VpOps &op) {
        op.tv = v_base(t);
        op.pp = opaque((uint32_t)(uintptr_t)(lds_u8 *)(&s_p[pb][0][0][0]) + 16u * (uint32_t)lane);
#pragma unroll
        for (int hb = 0; hb < kHb; ++hb) op.pa[hb][0] = read_p(op, hb, 0);
        op.vq[0] = read_v(op.tv, 0, 0);
        op.vq[1] = read_v(op.tv, 0, 1);
    };
    auto value_product = [&](VpOps &op, int pb, auto side) {
        const VBase &tv = op.tv;
        auto &pa = op.pa;
        auto &vq = op.vq;  // value operands two column groups ahead
        u32x4_t vb_prev;
#pragma unroll
        for (int j = 0; j < 2 * kCbW; ++j) {  // (kk, cb) = (j / 4, j % 4)
            const u32x4_t vb = vq[j % 3];
            if (j + 2 < 2 * kCbW) vq[(j + 2) % 3] = read_v(tv, (j + 2) >> 2, (j + 2) & 3);
            if (j == 0)
#pragma unroll
                for (int hb = 0; hb < kHb; ++hb) pa[hb][1] = read_p(op, hb, 1);
#pragma unroll
            for (int hb = 0; hb < kHb; ++hb) {
                mfma32_a(o[4 * hb + (j & 3)], pa[hb][j >> 2], vb);
                __builtin_amdgcn_sched_barrier(0);
                if (hb == 0 && j > 0) keep(vb_prev);
                if (hb == 0 && j == kCbW)
#pragma unroll
                    for (int h = 0; h < kHb; ++h) keep(pa[h][0]);
                side(4 * j + hb);
                __builtin_amdgcn_sched_barrier(0);
            }
            vb_prev = vb;
        }
        mfma_drain();
        keep(vb_prev);
#pragma unroll
        for (int h = 0; h < kHb; ++h) keep(pa[h][1]);
        __builtin_amdgcn_sched_barrier(0);
    };

    // A reference raised by the softmax of tile it (any wave) rescales those
    // heads' rows of O after the value product of tile it - 1 and before that
    // of tile it: in the next iteration (or before the last value product),
    // with the factors of parity buffer pb.  flags: the four waves' flags of
    // that buffer, read early (the LDS latency is then hidden).
    auto read_flags = [&](int pb) -> u32x4_t {
        return *(__attribute__((address_space(3))) const u32x4_t *)(&s_aflag[pb][0]);
    };
    auto rescale_pending = [&](const u32x4_t &flags, int pb) {
        const int32_t f0 = __builtin_amdgcn_readfirstlane(flags[0]);
        const int32_t f1 = __builtin_amdgcn_readfirstlane(flags[1]);
        const int32_t f2 = __builtin_amdgcn_readfirstlane(flags[2]);
        const int32_t f3 = __builtin_amdgcn_readfirstlane(flags[3]);
        if (f0 | f1 | f2 | f3) {  // rare: rows whose reference maximum rose by more than 2^8
            __builtin_amdgcn_sched_barrier(0);
            mfma_drain();  // the value-product MFMAs issued last write the AGPRs read below
            __builtin_amdgcn_sched_barrier(0);
            const int hh = 4 * (lane_now() >> 5);
#pragma unroll
            for (int hb = 0; hb < kHb; ++hb) {
                const int32_t fl = hb == 0 ? f0 : hb == 1 ? f1 : hb == 2 ? f2 : f3;
                if (!fl) continue;
#pragma unroll
                for (int q = 0; q < 4; ++q) {  // rows 8 q + hh .. + 3: elements 4 q .. 4 q + 3
                    const f32x4_t al = *(__attribute__((address_space(3))) const f32x4_t *)(
                        &s_alpha[pb][hb][8 * q + hh]);
#pragma unroll
                    for (int cb = 0; cb < kCbW; ++cb) {
                        scale_acc_agpr(o[4 * hb + cb], 4 * q + 0, al.x);
                        scale_acc_agpr(o[4 * hb + cb], 4 * q + 1, al.y);
                        scale_acc_agpr(o[4 * hb + cb], 4 * q + 2, al.z);
                        scale_acc_agpr(o[4 * hb + cb], 4 * q + 3, al.w);
                    }
                }
            }
        }
    };

    // bf16: the cache rows of tile it + 1, read one iteration ahead
    i32x2_t rows_next{};
    if (!kFp8 && tab && ntile > 1)
        rows_next = *(__attribute__((address_space(3))) const i32x2_t *)(&s_rows[1][0]);

    // ---- tiles: the scores of tile it, then the value product of tile it - 1
    // with the softmax of tile it woven between its MFMAs ----
    // (the first tile is peeled: it has no value product of a previous tile)
    auto iteration = [&](const int32_t it, auto first_tag) {
        constexpr bool kFirst = decltype(first_tag)::value;
        // tile it landed (bf16: this wave's copies; fp8: widened in iteration
        // it - 1), and the probabilities of tile it - 1 are written ...
        if constexpr (!kFp8) wait_copies(0);
        __syncthreads();  // ... by every wave; tile it - 2's position is free
        bool copy_now = false;
        TileSrc nsrc{};
        if (!kFp8 && it + 1 < ntile) {
            if (tab) {
                nsrc.r0 = __builtin_amdgcn_readfirstlane(rows_next[0]);
                nsrc.r1 = __builtin_amdgcn_readfirstlane(rows_next[1]);
                nsrc.nval = min(kT, s1 - (s0 + (it + 1) * kT));
            } else {
                nsrc = tile_src(it + 1);
            }
            copy_now = true;
        }
        // the rows of tile it + 2, read now for the next iteration
        if (!kFp8 && tab && it + 2 < ntile)
            rows_next = *(__attribute__((address_space(3))) const i32x2_t *)(&s_rows[it + 2][0]);
        if constexpr (kFp8) {
            // raw tile it + 1 (landed: the only copy in flight) -> bf16 position
            // (it + 1) % 3; then raw tile it + 2 into the raw position
            if (it + 1 < ntile) {
                wait_copies(0);
                widen_tile(it + 1);
            }
            if (it + 2 < ntile) issue_tile(it + 2);
        }
        // bf16 copy i of tile it + 1 follows score MFMA kAt[i]
        // (lane l copies row t = 8 w + l / 8 of the tile; in a partial tile
        // rows past its end repeat its last row)
        gbyte *csrc = nullptr;
        if (!kFp8 && copy_now) {
            const int t = 8 * wave + (lane_now() >> 3);
            const int tt = min(t, nsrc.nval - 1);
            const int32_t row = tt < 16 ? nsrc.r0 + tt : nsrc.r1 - 16 + tt;
            uint64_t a = (uint64_t)(uintptr_t)(p.kv + (int64_t)row * kRowB + ccol);
            asm volatile("" : "+v"(a));
            csrc = (gbyte *)(uintptr_t)a;
        }
        const uint32_t cdst = kv_lds + (uint32_t)(((it + 1) % kStagesBf) * kTileB + 8 * wave * 128);
        auto copy_at = [&](int m) {
            if constexpr (!kFp8) {
                constexpr int kAt[kCopiesBf] = {0, 3, 6, 9, 12, 15, 18, 21, 24};
#pragma unroll
                for (int i = 0; i < kCopiesBf; ++i)
                    if (m == kAt[i] && copy_now) dma16_group(i, csrc, cdst + i * kGroupB);
            }
        };
        u32x4_t flags{};
        if constexpr (!kFirst) flags = read_flags((it - 1) & 1);
        const KBase tile = k_base(tile_ptr(it));

        // ---- scores S[token][head] of tile it: 36 k-steps accumulated in one
        // chain (a dependent MFMA issues back to back with its predecessor) ----
        f32x16_t sc;
        VpOps vop;  // the value product's first operands, read during the last score MFMAs
        {
            constexpr int kPre = 4;
            u32x4_t abuf[kPre];
#pragma unroll
            for (int i = 0; i < kPre; ++i) abuf[i] = read_k(tile, i);
            u32x4_t a_prev;
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks) {
                const u32x4_t a = abuf[ks % kPre];
                if (ks + kPre < kKs) abuf[ks % kPre] = read_k(tile, ks + kPre);
                if (ks == 0) mfma32_v0(sc, a, qb[ks]);
                else mfma32_v(sc, a, qb[ks]);
                __builtin_amdgcn_sched_barrier(0);
                if (ks > 0) keep(a_prev);
                copy_at(ks);
                if constexpr (!kFirst)
                    if (ks == kKs - 4) vp_begin(tile_ptr(it - 1), (it - 1) & 1, vop);
                __builtin_amdgcn_sched_barrier(0);
                a_prev = a;
            }
            mfma_drain();
            keep(a_prev);
        }

        // ---- softmax of tile it (mask past the segment's end, tile maximum,
        // lazy reference, probabilities) for this wave's 32 heads, woven into
        // the value product of tile it - 1; the probabilities and the
        // rescale factors go to the parity-(it % 2) exchange buffers ----
        const int32_t nval = min(kT, s1 - (s0 + it * kT));
        float alpha = 1.f;
        bool resc = false;
        // The steps below are cut so that each fits the shadow of one MFMA
        // (a VALU instruction issued while an MFMA runs costs about 6 cycles,
        // an exp2 about 10; an MFMA takes 32).
        float mt = 0.f;
        auto soft_mask = [&]() {
            if (nval < kT) {  // token acc_row(e, h2) = acc_row(e, 0) + 4 h2 is real iff < nval
                const int lim = nval - 4 * (lane_now() >> 5);
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (acc_row(e, 0) >= lim) sc[e] = -INFINITY;
            }
        };
        auto soft_max_lo = [&]() {  // the lane's maximum of elements 0 .. 8
            mt = fmaxf(fmaxf(sc[0], sc[1]), sc[2]);
            mt = fmaxf(fmaxf(mt, sc[3]), sc[4]);
            mt = fmaxf(fmaxf(mt, sc[5]), sc[6]);
            mt = fmaxf(fmaxf(mt, sc[7]), sc[8]);
        };
        auto soft_max_hi = [&]() {  // ... and of 9 .. 15
            mt = fmaxf(fmaxf(mt, sc[9]), sc[10]);
            mt = fmaxf(fmaxf(mt, sc[11]), sc[12]);
            mt = fmaxf(fmaxf(mt, sc[13]), sc[14]);
            mt = fmaxf(mt, sc[15]);
        };
        auto soft_halves = [&]() {  // the tile maximum of the head (both lane halves)
            mt = halves_max(mt) * p.qk_scale;  // the scale is >= 0: the maximum commutes
        };
        auto soft_ref = [&]() {  // the lazy reference
            if constexpr (kFirst) {
                m_ref = mt;
            } else {
                const bool need = mt > m_ref + kLazy;
                resc = __any(need);
                alpha = need ? fast_exp2(m_ref - mt) : 1.f;
                m_ref = need ? mt : m_ref;
            }
        };
        // probabilities as the A operand of the value product: Pn[kk] holds
        // elements 8 kk .. 8 kk + 7 (the token order of 16-token step kk);
        // ps sums them in fp32 (before the bf16 rounding)
        u32x4_t Pn[2];
        float ps = 0.f, pe0 = 0.f, pe1 = 0.f;
        auto soft_exp = [&](int e2) {  // elements 2 e2, 2 e2 + 1
            pe0 = fast_exp2(fmaf(sc[2 * e2], p.qk_scale, -m_ref));
            pe1 = fast_exp2(fmaf(sc[2 * e2 + 1], p.qk_scale, -m_ref));
        };
        auto soft_pack = [&](int e2) {  // ... as one bf16 pair
            Pn[e2 >> 2][e2 & 3] = pack_bf16x2(pe0, pe1);
            ps += pe0 + pe1;
        };
        // Past the first tile the weights are taken against the current
        // reference without the tile's maximum: a lane whose weights sum to at
        // most 2^kLazy has none above 2^kLazy, which is all the lazy reference
        // asks for.  Where a weight may be larger (or overflowed, or is NaN)
        // the maximum is taken, the reference raised where it must be, and the
        // weights taken again (a uniform branch; rare once the reference has
        // settled).
        auto soft_check = [&]() {
            if (__any(!(ps <= kLazyW))) {
                soft_max_lo();
                soft_max_hi();
                soft_halves();
                soft_ref();
                ps = 0.f;
#pragma unroll
                for (int e2 = 0; e2 < 8; ++e2) {
                    soft_exp(e2);
                    soft_pack(e2);
                }
            }
        };
        auto publish_p = [&]() {
            const int ln2 = lane_now();
            s_p[it & 1][wave][0][ln2] = Pn[0];
            s_p[it & 1][wave][1][ln2] = Pn[1];
        };
        auto publish_alpha = [&]() {
            const int ln2 = lane_now();
            if (ln2 < 32) s_alpha[it & 1][wave][ln2] = alpha;
            if (ln2 == 0) s_aflag[it & 1][wave] = resc ? 1 : 0;
        };
        if constexpr (!kFirst) {
            rescale_pending(flags, (it - 1) & 1);
            // the softmax steps after MFMAs 1 .. 30 of the value product
            value_product(vop, (it - 1) & 1, [&](int i) {
                if (i == 1) soft_mask();
                // pair k: exponentials after MFMA kSlot[2 k], packing after kSlot[2 k + 1]
                constexpr int kSlot[16] = {2, 3, 5, 6, 8, 9, 11, 12, 14, 15, 17, 18, 20, 21, 23, 24};
#pragma unroll
                for (int k2 = 0; k2 < 8; ++k2) {
                    if (i == kSlot[2 * k2]) soft_exp(k2);
                    if (i == kSlot[2 * k2 + 1]) soft_pack(k2);
                }
                if (i == 26) soft_check();
                if (i == 29) publish_p();
                if (i == 30) publish_alpha();
            });
        } else {
            soft_mask();
            soft_max_lo();
            soft_max_hi();
            soft_halves();
            soft_ref();
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) {
                soft_exp(e2);
                soft_pack(e2);
            }
            publish_p();
            publish_alpha();
        }
        l_run = l_run * alpha + ps;
    };
    if (ntile > 0) iteration(0, std::true_type{});
    for (int32_t it = 1; it < ntile; ++it) iteration(it, std::false_type{});
    // ---- value product of the last tile ----
    if (ntile > 0) {
        __syncthreads();  // every wave's probabilities of the last tile are written
        rescale_pending(read_flags((ntile - 1) & 1), (ntile - 1) & 1);
        VpOps op;
        vp_begin(tile_ptr(ntile - 1), (ntile - 1) & 1, op);
        value_product(op, (ntile - 1) & 1, [&](int) {});
        __builtin_amdgcn_sched_barrier(0);
        mfma_drain();
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---- finish: full softmax sums of every head, normalise, write this
    // segment's partial (the wave's columns of every head; the LSE of its own
    // heads) ----
    const float lt = halves_sum(l_run);
    if (h2 == 0) s_lsum[wave][r32] = lt;
    bad = __syncthreads_or(bad);
    const bool empty = ntile == 0;
    if (h2 == 0 && h0 + r32 < p.H)
        p.ws_l[(int64_t)slot * p.H + h0 + r32] =
            bad ? NAN : (empty ? -INFINITY : (m_ref + fast_log2(lt)) * kLn2);
    // bf16 partials, written as whole dwords: lanes 2k and 2k+1 hold columns
    // 2k and 2k+1 of a head's column block; they swap one value so that the
    // even lane stores the pair of block cb and the odd lane that of block cb+1.
    const bool odd = (r32 & 1) != 0;
    uint32_t *o_dst = reinterpret_cast<uint32_t *>(p.ws_o) +
                      ((int64_t)slot * p.H * kDv + 128 * wave + (r32 & ~1)) / 2;
#pragma unroll
    for (int hb = 0; hb < kHb; ++hb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {  // rows 32 hb + 8 q + 4 h2 + (0 .. 3): elements 4 q + (0 .. 3)
            const f32x4_t ls = *(__attribute__((address_space(3))) const f32x4_t *)(
                &s_lsum[hb][8 * q + 4 * h2]);
            const float lv[4] = {ls.x, ls.y, ls.z, ls.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int e = 4 * q + r;
                const int head = 32 * hb + acc_row(e, h2);
                const float iv = bad ? NAN : (empty ? 0.f : p.v_scale / lv[r]);
#pragma unroll
                for (int cb = 0; cb < kCbW; cb += 2) {
                    const float A = o[4 * hb + cb][e] * iv, B = o[4 * hb + cb + 1][e] * iv;
                    const float y = __int_as_float(__builtin_amdgcn_mov_dpp(
                        __float_as_int(odd ? A : B), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
                    if (head < p.H)
                        o_dst[((int64_t)head * kDv + 32 * (cb + (odd ? 1 : 0))) / 2] =
                            odd ? pack_bf16x2(y, B) : pack_bf16x2(A, y);
                }
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

MlaPlan plan_mla(const cp_mla_args &a) {
    MlaPlan pl{};
    const int wgs = device_cus();  // one workgroup per CU (its four waves hold every register)
    pl.split_tokens = kT;
    pl.nsplit = wgs;  // tile ranges = workgroups launched
    const size_t slots = (size_t)wgs + (size_t)(a.B > 0 ? a.B : 0);
    pl.ws_bytes = slots * (size_t)a.H * (kDv * sizeof(uint16_t) + sizeof(float)) + (size_t)a.B * 2 * 4 + 512;
    return pl;
}

}  // namespace cpattn

using namespace cpattn;

extern "C" cp_status cp_decode_attn_partial_mla(const cp_mla_args *a, void *ws, size_t ws_bytes,
                                                hipStream_t stream) {
    clear_error();
    if (!a) return fail(CP_E_INVALID, "cp_decode_attn_partial_mla: NULL args");
    if (a->B < 0 || a->H < 1 || a->Dk < 1 || a->Dv < 1 || a->bs < 1 || a->bt_stride < 1 ||
        a->num_blocks < 1)
        return fail(CP_E_INVALID,
                    "mla decode: B=%d H=%d Dk=%d Dv=%d bs=%d bt_stride=%d num_blocks=%lld", a->B,
                    a->H, a->Dk, a->Dv, a->bs, a->bt_stride, (long long)a->num_blocks);
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
    const bool fp8 = a->kv_dt == CP_FP8_E4M3FN;
    const float kvs = fp8 ? a->kv_scale : 1.f;
    if (!isfinite(a->scale) || !isfinite(kvs) || !(kvs > 0.f))
        return fail(CP_E_INVALID, "mla decode: scale %g and kv_scale %g must be finite (kv_scale > 0)",
                    (double)a->scale, (double)kvs);
    if (a->B == 0) return CP_OK;
    if (!a->q || !a->kv_cache || !a->block_table || !a->local_len || !a->out || !a->lse)
        return fail(CP_E_INVALID, "mla decode: NULL pointer");
    if (!aligned16(a->q) || !aligned16(a->kv_cache) || !aligned16(a->out))
        return fail(CP_E_INVALID, "mla decode: q, cache and out must be 16-byte aligned");
    const MlaPlan pl = plan_mla(*a);
    if (!ws || ws_bytes < pl.ws_bytes)
        return fail(CP_E_WORKSPACE, "mla decode: workspace of %zu bytes needed, %zu given",
                    pl.ws_bytes, ws_bytes);
    const size_t slots = (size_t)pl.nsplit + (size_t)a->B;
    float *ws_o = static_cast<float *>(ws);
    float *ws_l = ws_o + slots * a->H * kDv / 2;  // after the bf16 partial outputs
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
    if (a->num_blocks * a->bs >= ((int64_t)1 << 31))
        return fail(CP_E_UNSUPPORTED, "mla decode: %lld blocks x %d rows exceed 2^31 cache rows",
                    (long long)a->num_blocks, a->bs);
    p.num_blocks = (int32_t)a->num_blocks;
    const int64_t cap = (int64_t)a->bt_stride << bs_log2;
    if ((int64_t)a->B * ((cap + kT - 1) / kT) >= ((int64_t)1 << 31))
        return fail(CP_E_UNSUPPORTED, "mla decode: %d requests x %lld tokens of table exceed 2^31 tiles",
                    a->B, (long long)cap);
    p.cap = (int32_t)cap;
    // a negative scale negates the queries instead (exact), so that the
    // kernel's scale is >= 0 and commutes with the maximum
    p.qk_scale = fabsf(a->scale) * kvs * kLog2e;
    p.q_sign = a->scale < 0.f ? 0x80008000u : 0u;
    p.v_scale = kvs;
    p.W = pl.nsplit;
    p.ws_o = ws_o;
    p.ws_l = ws_l;
    p.seg = seg;
    // one workgroup per tile range: at most W = #CUs ranges, or one per non-empty
    // request when there are more requests than CUs (ranges past the last exit)
    const unsigned grid = (unsigned)(pl.nsplit + a->B);
    if (fp8)
        hipLaunchKernelGGL(mla_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(mla_kernel<false>, dim3(grid), dim3(kThreads), 0, stream, p);
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
    m.part_bf16 = true;
    m.parts_hint = (int32_t)(pl.nsplit / (a->B > 0 ? a->B : 1));  // tile ranges per request, lengths alike
    m.o_part_stride = (int64_t)a->H * kDv;
    m.o_row_stride = kDv;
    m.l_part_stride = a->H;
    m.l_row_stride = 1;
    m.out = a->out;
    m.out_dt = CP_F32;
    m.lse_out = a->lse;
    return launch_merge(m, stream);
}
