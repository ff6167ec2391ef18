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
// Design (a dense contraction: 128 heads x 576 against every cached row):
//   * one workgroup = H/16 waves, wave w owns query heads 16w .. 16w+15;
//     all waves share each 32-token latent tile, staged once from HBM into a
//     double-buffered LDS ring (rows padded to 1168 B: conflict-free reads);
//   * scores S^T = C Q^T on v_mfma_f32_16x16x32_bf16 (A = latent rows from
//     LDS, B = the wave's 16 queries, kept in registers for the segment);
//   * online softmax in the exp2 domain; the score tile comes out of the MFMA
//     already in the A-operand layout of the value product (token order is
//     permuted identically on both operands, so no register shuffle);
//   * values O = P V on the same MFMA with the V operand read straight from the
//     row-major tile by ds_read_b64_tr_b16 (transposing LDS read), 16 value
//     columns per instruction; the 16 x 512 fp32 output tile stays in registers;
//   * fp8 E4M3 latent is widened to bf16 while being staged (exact), the
//     per-tensor scale folded into the score scale and the output;
//   * the same balanced flat schedule as the GQA kernel: exactly the resident
//     workgroups, each taking an equal range of (request, 32-token tile) space;
//     partials to slot wg + request, merged exactly afterwards.
#include <math.h>

#include <type_traits>

#include "internal.hpp"

namespace cpattn {

namespace {

constexpr int kDk = 576, kDv = 512;
constexpr int kT = 32;                  // tokens per tile / per scheduling chunk
constexpr int kRowB = kDk * 2 + 16;     // LDS row stride in bytes (bf16 + pad)
constexpr int kKs = kDk / 32;           // 18 k-steps of the score MFMA
constexpr int kVb = kDv / 16;           // 32 value-column blocks
constexpr int kMaxB = 4096;
constexpr int kMaxWaves = 8;            // 128 heads

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T *)(p))

struct MlaParams {
    const gbyte *q, *kv;
    cint32 *bt, *len;
    int32_t B, H, bs_log2, bt_stride;
    int64_t num_blocks;
    float qk_scale;   // scale * kv_scale * log2(e)
    float v_scale;    // kv_scale (fp8) or 1
    int32_t W;        // workgroups launched
    float *ws_o;      // [slots][H][512]
    float *ws_l;      // [slots][H]
    int32_t *seg;     // [B][2]
};

__device__ __forceinline__ f32x4_t mfma16(const u32x4_t &a, const u32x4_t &b, const f32x4_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, static_cast<__bf16>(lo)) |
           ((uint32_t)__builtin_bit_cast(uint16_t, static_cast<__bf16>(hi)) << 16);
}

__device__ __forceinline__ int64_t owner_of(int64_t c, int64_t R, int64_t W) {
    return ((c + 1) * W - 1) / R;
}

template <bool kFp8>
__global__ void __launch_bounds__(64 * kMaxWaves, 1) mla_kernel(MlaParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t s_kv[2][kT * kRowB];
    // fp8 only: raw rows as loaded (size 1 otherwise)
    __shared__ __attribute__((aligned(16))) uint8_t s_raw[2][kFp8 ? kT * kDk : 16];
    __shared__ int32_t s_pref[kMaxB + 1];
    __shared__ int32_t s_wsum[kMaxWaves];

    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G4 = lane >> 4, j16 = lane & 15;
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
        const int per = (p.B + nthr - 1) / nthr;
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
        if (tid == nthr - 1) s_pref[p.B] = base + incl;
        __syncthreads();
    }
    auto pref = [&](int i) -> int32_t { return __builtin_amdgcn_readfirstlane(s_pref[i]); };
    const int64_t R_tot = pref(p.B);
    const int64_t W = R_tot < p.W ? R_tot : p.W;

    if (blockIdx.x == 0) {
        for (int b = tid; b < p.B; b += nthr) {
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
    const int64_t wg = blockIdx.x;
    if (wg >= W || R_tot == 0) return;
    int64_t cc = wg * R_tot / W;
    const int64_t hi = (wg + 1) * R_tot / W;

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
        const int64_t slot = wg + b;
        cint32 *bt_row = p.bt + (int64_t)b * p.bt_stride;

        // ---- the wave's 16 queries as the B operand: Q[h0+j16][32ks + 8 G4 .. +8] ----
        u32x4_t qb[kKs];
        if (active) {
            gbyte *qrow = p.q + ((int64_t)b * p.H + h0 + j16) * (kDk * 2) + G4 * 16;
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks) qb[ks] = load16(qrow + ks * 64);
        }

        // ---- staging of one tile (all threads): latent rows -> bf16 rows in LDS ----
        // block ids of the tile's tokens (bs >= 16: at most two blocks per tile)
        auto tile_blocks = [&](int32_t tb, int64_t &r0, int64_t &r1) {
            const int32_t lb0 = tb, lb1 = tb + 16;
            auto row_of = [&](int32_t lb) -> int64_t {
                const int32_t gsel = lb < s1 ? lb : s0;
                int32_t phys = bt_row[gsel >> p.bs_log2];
                const bool ok = phys >= 0 && (int64_t)phys < p.num_blocks;
                bad |= !ok;
                phys = ok ? phys : 0;
                return ((int64_t)phys << p.bs_log2) + (gsel & (bs - 1));
            };
            r0 = row_of(lb0);
            r1 = row_of(lb1);
        };
        // Tiles reach LDS without passing through registers: each lane of a
        // global_load_lds_dwordx4 moves 16 bytes to LDS address base + 16 * lane,
        // so lane (slot, lane) fetches the source chunk that belongs at LDS chunk
        // c = 64 * slot + lane of the destination region.
        //   bf16: the destination is the padded tile itself (73 chunks per row,
        //         the 73rd is padding and not loaded);
        //   fp8:  raw rows (36 chunks each) land in a staging ring and are
        //         widened to bf16 after the tile has arrived.
        auto stage_issue = [&](int32_t tb, int buf) {
            int64_t r0, r1;
            tile_blocks(tb, r0, r1);
            constexpr int kPer = kFp8 ? kDk / 16 : kRowB / 16;   // chunks per destination row
            constexpr int kSlots = (kT * kPer + 63) / 64;        // 64-chunk load instructions
            uint8_t *base = kFp8 ? s_raw[buf] : s_kv[buf];
#pragma unroll
            for (int i = 0; i < (kSlots + kMaxWaves - 1) / kMaxWaves; ++i) {
                const int sl = wave + kMaxWaves * i;
                if (sl >= kSlots) break;
                const int c = sl * 64 + lane;
                const int tt = c / kPer, ch = c - tt * kPer;
                const bool ok = tt < kT && (kFp8 || ch < kDk * 2 / 16) && tb + tt < s1;
                if (ok) {
                    const int64_t row = tt < 16 ? r0 + tt : r1 + (tt - 16);
                    __builtin_amdgcn_global_load_lds(
                        (const CP_GLOBAL void *)(p.kv + row * (kFp8 ? kDk : kDk * 2) + ch * 16),
                        (__attribute__((address_space(3))) void *)(base + sl * 1024), 16, 0, 0);
                }
            }
        };
        // After the tile's loads have landed (vmcnt(0) + barrier): fp8 rows are
        // widened into the bf16 tile; rows past the segment's end are zeroed (their
        // probability is 0, and the V product must not see stale NaN bits).
        auto stage_finish = [&](int32_t tb, int buf) {
            uint8_t *dst = s_kv[buf];
            if constexpr (kFp8) {
                const uint8_t *raw = s_raw[buf];
                for (int c = tid; c < kT * (kDk / 16); c += nthr) {
                    const int tt = c / (kDk / 16), ch = c - tt * (kDk / 16);
                    u32x4_t lo = {0u, 0u, 0u, 0u}, hi2 = {0u, 0u, 0u, 0u};
                    if (tb + tt < s1) {
                        const u32x4_t x = *reinterpret_cast<const u32x4_t *>(raw + c * 16);
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
                    }
                    *reinterpret_cast<u32x4_t *>(dst + tt * kRowB + ch * 32) = lo;
                    *reinterpret_cast<u32x4_t *>(dst + tt * kRowB + ch * 32 + 16) = hi2;
                }
            } else if (tb + kT > s1) {
                const u32x4_t z = {0u, 0u, 0u, 0u};
                for (int c = tid; c < kT * (kDk * 2 / 16); c += nthr) {
                    const int tt = c / (kDk * 2 / 16), ch = c - tt * (kDk * 2 / 16);
                    if (tb + tt >= s1) *reinterpret_cast<u32x4_t *>(dst + tt * kRowB + ch * 16) = z;
                }
            }
        };

        float m_run = -INFINITY, l_run = 0.f;  // stats of head h0 + j16 (same in all 4 groups)
        f32x4_t o[kVb];
#pragma unroll
        for (int vb = 0; vb < kVb; ++vb) o[vb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        int buf = 0;
        if (s1 > s0) stage_issue(s0, 0);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the tile has landed in LDS
        __syncthreads();
        if (s1 > s0) stage_finish(s0, 0);
        if (kFp8 || s0 + kT > s1) __syncthreads();
        for (int32_t tb = s0; tb < s1; tb += kT) {
            const int32_t tn = tb + kT;
            const bool has_next = tn < s1;  // uniform across the workgroup
            // the next tile streams into the other buffer while this one is used
            if (has_next) stage_issue(tn, buf ^ 1);
            const uint8_t *tile = s_kv[buf];
            if (active) {
            // ---- scores S^T[t][h]: two 16-token halves ----
            f32x4_t sc[2];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
                const uint8_t *arow = tile + (hf * 16 + j16) * kRowB + G4 * 16;
#pragma unroll
                for (int ks = 0; ks < kKs; ++ks) {
                    const u32x4_t a = *reinterpret_cast<const u32x4_t *>(arow + ks * 64);
                    acc = mfma16(a, qb[ks], acc);
                }
                sc[hf] = acc;
            }
            // lane holds tokens tb + 16 hf + 4 G4 + e of head h0 + j16
            float mt = -INFINITY;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float s = sc[hf][e] * p.qk_scale;
                    if (tb + hf * 16 + G4 * 4 + e >= s1) s = -INFINITY;
                    sc[hf][e] = s;
                    mt = fmaxf(mt, s);
                }
            mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
            mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
            const float mn = fmaxf(m_run, mt);
            const float alpha = fast_exp2(m_run - mn);
            m_run = mn;
            float ps = 0.f;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sc[hf][e] = fast_exp2(sc[hf][e] - mn);
                    ps += sc[hf][e];
                }
            l_run = l_run * alpha + ps;  // partial over this lane's tokens
            // P as the A operand: k = 8 G4 + e <-> tokens 4 G4 + e (e < 4), 16 + 4 G4 + e - 4
            u32x4_t pa;
            pa[0] = pack2_bf16(sc[0][0], sc[0][1]);
            pa[1] = pack2_bf16(sc[0][2], sc[0][3]);
            pa[2] = pack2_bf16(sc[1][0], sc[1][1]);
            pa[3] = pack2_bf16(sc[1][2], sc[1][3]);
            // rescale the output rows (heads 4 G4 + e) by their alpha
            float ar[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) ar[e] = __shfl(alpha, G4 * 4 + e, 64);
#pragma unroll
            for (int vb = 0; vb < kVb; ++vb)
#pragma unroll
                for (int e = 0; e < 4; ++e) o[vb][e] *= ar[e];

            // ---- values: O[h][v] += P[h][t] V[t][v], 16 columns per MFMA ----
            const uint8_t *vrow0 = tile + (4 * G4 + (j16 >> 2)) * kRowB + (j16 & 3) * 8;
            const uint8_t *vrow1 = vrow0 + 16 * kRowB;
#pragma unroll
            for (int vb = 0; vb < kVb; ++vb) {
                const i16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    LDS_PTR(i16x4_t, vrow0 + vb * 32));
                const i16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    LDS_PTR(i16x4_t, vrow1 + vb * 32));
                u32x4_t vbop;
                vbop[0] = (uint32_t)(uint16_t)t0[0] | ((uint32_t)(uint16_t)t0[1] << 16);
                vbop[1] = (uint32_t)(uint16_t)t0[2] | ((uint32_t)(uint16_t)t0[3] << 16);
                vbop[2] = (uint32_t)(uint16_t)t1[0] | ((uint32_t)(uint16_t)t1[1] << 16);
                vbop[3] = (uint32_t)(uint16_t)t1[2] | ((uint32_t)(uint16_t)t1[3] << 16);
                o[vb] = mfma16(pa, vbop, o[vb]);
            }
            }  // active

            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): next tile landed
            __syncthreads();                     // and nobody reads this buffer any more
            if (has_next) {
                stage_finish(tn, buf ^ 1);
                if (kFp8 || tn + kT > s1) __syncthreads();
            }
            buf ^= 1;
        }

        // ---- finish: full softmax sums, normalise, write this segment's partial ----
        float lt = l_run;
        lt += __shfl_xor(lt, 16, 64);
        lt += __shfl_xor(lt, 32, 64);
        bad = __syncthreads_or(bad);
        const bool empty = !(s1 > s0);
        float inv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float le = __shfl(lt, G4 * 4 + e, 64);
            inv[e] = bad ? NAN : (empty ? 0.f : p.v_scale / le);
        }
        float *o_dst = p.ws_o + (slot * p.H + h0) * kDv;
        if (active)
#pragma unroll
            for (int vb = 0; vb < kVb; ++vb)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o_dst[(G4 * 4 + e) * kDv + vb * 16 + j16] = o[vb][e] * inv[e];
        if (active && lane < 16)
            p.ws_l[slot * p.H + h0 + lane] =
                bad ? NAN : (empty ? -INFINITY : (m_run + fast_log2(lt)) * kLn2);
        cc += nseg;
        __syncthreads();  // the LDS ring is reused by the next segment
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
    const int threads = 64 * kMaxWaves;
    const int wgs = device_cus() * (fp8 ? resident_wgs<true>(threads) : resident_wgs<false>(threads));
    pl.split_tokens = kT;
    pl.nsplit = wgs;  // workgroups launched
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
    if (a->H % 16 != 0 || a->H > 16 * kMaxWaves)
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
    const int threads = 64 * kMaxWaves;
    if (fp8)
        hipLaunchKernelGGL(mla_kernel<true>, dim3(pl.nsplit), dim3(threads), 0, stream, p);
    else
        hipLaunchKernelGGL(mla_kernel<false>, dim3(pl.nsplit), dim3(threads), 0, stream, p);
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
