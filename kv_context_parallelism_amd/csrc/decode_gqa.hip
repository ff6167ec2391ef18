// decode_gqa.hip -- rank-local GQA decode attention over one paged KV shard,
// returning the partial output o_i and its LSE L_i.
//
// "vLLM DCP and PCP: Decode and Prefill Context Parallelism", Deep Dive 6,
// "Deriving the partial and global outputs": every DCP rank applies the same
// query to its own KV shard, s_j = q.k_j / sqrt(d), L_i = log sum exp s_j,
// o_i = sum exp(s_j) v_j / exp(L_i).  "Breaking the Long-Sequence Inference
// Bottleneck ...", section 3, GQA path step 2: the expanded query heads of a
// KV head attend to the local KV shard.
//
// Design (gfx950, wave64, no MFMA: 4 FLOP per KV byte is far below the VALU
// ridge, so the kernel is HBM-bound and the job is to stream KV at full rate):
//   * one wave per work item = (request, KV head, split of S local tokens);
//     split-K partials are merged exactly by the shared LSE-merge kernel;
//   * the KV head's G query heads are processed together, so each K/V byte
//     is read from HBM once;
//   * tiles of TILE tokens; K rows are read 64 contiguous bytes per lane
//     quad (4 lanes = one token, each lane a quarter of the row) with 128-bit
//     loads; dot products use packed bf16 dot2 (fp32 accumulate) and a
//     two-step DPP quad reduction;
//   * online softmax in the exp2 domain with wave-wide max shuffles; the
//     running max is shared by the whole wave so accumulators never need a
//     cross-lane rescale;
//   * probabilities go through a per-wave LDS buffer into the PV layout, where
//     16 lanes cover one V row (fully coalesced 1 KB per load instruction) and
//     bf16 PV uses dot2 over token pairs (probabilities rounded to bf16);
//   * the block table is read with uniform (scalar) loads once per 16-token
//     group: with bs a power of two >= 16 every load instruction's tokens sit
//     in one physical block.
#include <math.h>

#include "internal.hpp"

namespace cpattn {

namespace {

constexpr int kWaves = 4;
constexpr int kMaxSplitBlocks = 64;  // block ids staged per work item (split <= 64 blocks)

struct GqaParams {
    const gbyte *q, *kc, *vc;
    const int32_t *bt, *len;
    int32_t B, Hq, Hkv, bs_log2, bt_stride;
    int64_t num_blocks;
    float qk_scale;  // softmax scale * log2(e)
    int32_t split_tokens, nsplit;
    float *out, *lse;  // [B][Hq][nsplit][D] and [B][Hq][nsplit]
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 4 lanes of a quad (DPP quad_perm [1,0,3,2] then [2,3,0,1]).
__device__ __forceinline__ float quad_sum(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    return v;
}

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t w(const u32x4 &v, int i) { return v[i]; }

template <int EB, int D, int G, int TILE>
struct GqaTraits {
    static constexpr int ROWB = D * EB;        // bytes of one token's row
    static constexpr int CH = ROWB / 16;       // 16-byte chunks per row
    static constexpr int EPC = 16 / EB;        // elements per chunk
    static constexpr int NCQ = CH / 4;         // chunks per lane in the QK layout
    static constexpr int RG = 64 / CH;         // token rows per wave in the PV layout
    static constexpr int NPASS = TILE / 16;    // QK passes (16 tokens each) per tile
    static constexpr int TPL = TILE / RG;      // tokens per lane per tile in the PV layout
    static constexpr int PWORDS = EB == 2 ? (TILE / 2) * G : TILE * G;
    static_assert(CH == 8 || CH == 16 || CH == 32, "row must be 128, 256 or 512 bytes");
    static_assert(TILE % 16 == 0 && TILE % (2 * RG) == 0, "tile shape");
    static_assert(16 % RG == 0, "one PV load instruction must stay inside a 16-token group");
};

template <int EB, int D, int G, int TILE, int MIN_WG_PER_CU>
__global__ void __launch_bounds__(64 * kWaves, MIN_WG_PER_CU) gqa_decode_kernel(GqaParams p) {
    using Tr = GqaTraits<EB, D, G, TILE>;
    constexpr int ROWB = Tr::ROWB, CH = Tr::CH, EPC = Tr::EPC, NCQ = Tr::NCQ, RG = Tr::RG;
    constexpr int NPASS = Tr::NPASS, TPL = Tr::TPL;
    constexpr bool kBf16 = (EB == 2);
    __shared__ uint32_t s_p[kWaves][Tr::PWORDS];
    __shared__ int32_t s_bt[kWaves][kMaxSplitBlocks];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t item = (int64_t)blockIdx.x * kWaves + wave;
    if (item >= (int64_t)p.B * p.Hkv * p.nsplit) return;
    const int split = (int)(item % p.nsplit);
    const int64_t bg = item / p.nsplit;
    const int g = (int)(bg % p.Hkv);
    const int b = (int)(bg / p.Hkv);
    const int bs = 1 << p.bs_log2;
    const int64_t cap = (int64_t)p.bt_stride << p.bs_log2;

    int32_t L = p.len[b];
    bool bad = (L < 0) || ((int64_t)L > cap);
    L = L < 0 ? 0 : ((int64_t)L > cap ? (int32_t)cap : L);
    const int32_t s0 = split * p.split_tokens;
    const int32_t s1 = min(s0 + p.split_tokens, L);
    const int h0 = g * G;
    const int64_t o_hstride = (int64_t)p.nsplit * D;
    float *o_dst = p.out + (((int64_t)b * p.Hq + h0) * p.nsplit + split) * D;
    float *l_dst = p.lse + ((int64_t)b * p.Hq + h0) * p.nsplit + split;
    const int32_t *bt_row = p.bt + (int64_t)b * p.bt_stride;

    if (s0 >= L) {  // nothing local in this split: o = 0, L = -inf (NaN if metadata is bad)
        for (int i = lane; i < G * D; i += 64) o_dst[(i / D) * o_hstride + i % D] = bad ? NAN : 0.f;
        if (lane < G) l_dst[lane * p.nsplit] = bad ? NAN : -INFINITY;
        return;
    }

    // ---- query registers (QK layout: lane = (token tp, quarter qd)) ----
    const int qd = lane & 3, tp = lane >> 2;
    u32x4 qraw[G][NCQ];
    float qf[kBf16 ? 1 : G][kBf16 ? 1 : NCQ][4];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int j = 0; j < NCQ; ++j) {
            const u32x4 v = load16(p.q + ((int64_t)b * p.Hq + h0 + hh) * ROWB + (j * 4 + qd) * 16);
            if constexpr (kBf16) {
                qraw[hh][j] = v;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) qf[hh][j][e] = __uint_as_float(w(v, e)) * p.qk_scale;
            }
        }

    // ---- PV layout: lane = (row R, chunk c) ----
    const int R = lane / CH, c = lane % CH;
    float m[G], lsum[G], acc[G][EPC];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        m[hh] = -INFINITY;
        lsum[hh] = 0.f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[hh][e] = 0.f;
    }
    const u32x4 zero4 = {0u, 0u, 0u, 0u};

    // ---- this split's physical block ids, staged once in LDS ----
    const int32_t blk0 = s0 >> p.bs_log2;
    const int32_t nblk = ((s1 - 1) >> p.bs_log2) - blk0 + 1;
    for (int i = lane; i < nblk; i += 64) {
        int32_t phys = bt_row[blk0 + i];
        const bool ok = phys >= 0 && (int64_t)phys < p.num_blocks;
        bad |= !ok;
        s_bt[wave][i] = ok ? phys : 0;
    }
    bad = __ballot(bad) != 0;
    wave_sync();

    // First cache row (head g) of the 16-token group starting at local index lb.
    // Groups past the split's end map to the split's first group, so every
    // address formed below stays inside the cache.
    auto group_row = [&](int32_t lb) -> int64_t {
        const int32_t gsel = lb < s1 ? lb : s0;
        const int32_t phys =
            __builtin_amdgcn_readfirstlane(s_bt[wave][(gsel >> p.bs_log2) - blk0]);
        return ((int64_t)phys * p.Hkv + g) * bs + (gsel & (bs - 1));
    };
    // K of tile tb in the QK layout.  Rows of tokens past the split's end lie in
    // an allocated block of this split; their scores are replaced by -inf.
    auto load_k = [&](int32_t tb, u32x4 (&kreg)[NPASS][NCQ]) {
#pragma unroll
        for (int pp = 0; pp < NPASS; ++pp) {
            const gbyte *rowp = p.kc + (group_row(tb + pp * 16) + tp) * ROWB;
#pragma unroll
            for (int j = 0; j < NCQ; ++j) kreg[pp][j] = load16(rowp + (j * 4 + qd) * 16);
        }
    };
    // V of tile tb in the PV layout; zero_tail() clears rows past the split's
    // end (their probability is 0, but the row may hold NaN poison).
    auto load_v = [&](int32_t tb, u32x4 (&vreg)[TPL]) {
        constexpr int NG = TILE / 16;
        int64_t grow[NG];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) grow[gi] = group_row(tb + gi * 16);
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const gbyte *rowp = p.vc + (grow[(i * RG) / 16] + ((i * RG) & 15) + R) * ROWB;
            vreg[i] = load16(rowp + c * 16);
        }
    };
    auto zero_tail = [&](int32_t tb, u32x4 (&vreg)[TPL]) {
#pragma unroll
        for (int i = 0; i < TPL; ++i)
            if (tb + i * RG + R >= s1) vreg[i] = zero4;
    };

    // Staggered pipeline: K of the next tile is requested right after this
    // tile's scores are formed (overlapping softmax and PV), V of the next tile
    // right after this tile's PV (overlapping the next scores).
    u32x4 kreg[NPASS][NCQ];
    u32x4 vreg[TPL];
    load_k(s0, kreg);
    load_v(s0, vreg);
    for (int32_t tb = s0; tb < s1; tb += TILE) {
        const int32_t tn = tb + TILE;
        if (tn > s1) zero_tail(tb, vreg);  // only the split's last tile can be partial
        bool kval[NPASS];
#pragma unroll
        for (int pp = 0; pp < NPASS; ++pp) kval[pp] = (tb + pp * 16 + tp) < s1;

        // ---- scores (log2 domain) ----
        float s[NPASS][G];
#pragma unroll
        for (int pp = 0; pp < NPASS; ++pp)
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                float a = 0.f;
#pragma unroll
                for (int j = 0; j < NCQ; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if constexpr (kBf16)
                            a = dot2_bf16(w(kreg[pp][j], e), w(qraw[hh][j], e), a);
                        else
                            a = fmaf(__uint_as_float(w(kreg[pp][j], e)), qf[hh][j][e], a);
                    }
                a = quad_sum(a);
                if constexpr (kBf16) a *= p.qk_scale;
                s[pp][hh] = kval[pp] ? a : -INFINITY;
            }

        if (tn < s1) load_k(tn, kreg);

        // ---- online softmax: wave-wide running max per head ----
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            float mt = s[0][hh];
#pragma unroll
            for (int pp = 1; pp < NPASS; ++pp) mt = fmaxf(mt, s[pp][hh]);
            mt = fmaxf(mt, shfl_xor(mt, 4));
            mt = fmaxf(mt, shfl_xor(mt, 8));
            mt = fmaxf(mt, shfl_xor(mt, 16));
            mt = fmaxf(mt, shfl_xor(mt, 32));
            const float mn = fmaxf(m[hh], mt);
            const float alpha = fast_exp2(m[hh] - mn);
            m[hh] = mn;
            float ps = 0.f;
#pragma unroll
            for (int pp = 0; pp < NPASS; ++pp) {
                s[pp][hh] = fast_exp2(s[pp][hh] - mn);
                ps += s[pp][hh];
            }
            lsum[hh] = lsum[hh] * alpha + ps;
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[hh][e] *= alpha;
        }

        // ---- probabilities to the PV layout through LDS ----
        wave_sync();  // the previous tile's reads of s_p are complete
#pragma unroll
        for (int pp = 0; pp < NPASS; ++pp) {
            const int tk = pp * 16 + tp;
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                if ((hh & 3) != qd) continue;  // one writer per (token, head)
                if constexpr (kBf16) {
                    const int i = tk / RG, rr = tk % RG;
                    const int pair = (i >> 1) * RG + rr;
                    reinterpret_cast<uint16_t *>(s_p[wave])[(pair * G + hh) * 2 + (i & 1)] =
                        (uint16_t)f32_to_bf16_bits(s[pp][hh]);
                } else {
                    reinterpret_cast<float *>(s_p[wave])[tk * G + hh] = s[pp][hh];
                }
            }
        }
        wave_sync();

        // ---- PV ----
        if constexpr (kBf16) {
#pragma unroll
            for (int pi = 0; pi < TPL / 2; ++pi) {
                const int pair = pi * RG + R;
                uint32_t pw[G];
#pragma unroll
                for (int hh = 0; hh < G; ++hh) pw[hh] = s_p[wave][pair * G + hh];
                const u32x4 v0 = vreg[2 * pi], v1 = vreg[2 * pi + 1];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // (token t0, token t1) pairs of columns 2e and 2e+1 of the chunk
                    const uint32_t lo = __builtin_amdgcn_perm(w(v1, e), w(v0, e), 0x05040100u);
                    const uint32_t hi = __builtin_amdgcn_perm(w(v1, e), w(v0, e), 0x07060302u);
#pragma unroll
                    for (int hh = 0; hh < G; ++hh) {
                        acc[hh][2 * e] = dot2_bf16(lo, pw[hh], acc[hh][2 * e]);
                        acc[hh][2 * e + 1] = dot2_bf16(hi, pw[hh], acc[hh][2 * e + 1]);
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                const int t = i * RG + R;
                float pv[G];
#pragma unroll
                for (int hh = 0; hh < G; ++hh)
                    pv[hh] = reinterpret_cast<const float *>(s_p[wave])[t * G + hh];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float vv = __uint_as_float(w(vreg[i], e));
#pragma unroll
                    for (int hh = 0; hh < G; ++hh) acc[hh][e] = fmaf(pv[hh], vv, acc[hh][e]);
                }
            }
        }
        if (tn < s1) load_v(tn, vreg);
    }

    // ---- finish: sum the per-lane pieces, normalise, write o_i and L_i ----
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        float t = lsum[hh];
        t += shfl_xor(t, 4);
        t += shfl_xor(t, 8);
        t += shfl_xor(t, 16);
        t += shfl_xor(t, 32);
        lsum[hh] = t;
#pragma unroll
        for (int e = 0; e < EPC; ++e)
#pragma unroll
            for (int x = CH; x < 64; x <<= 1) acc[hh][e] += shfl_xor(acc[hh][e], x);
    }
    if (lane < CH) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const float inv = bad ? NAN : 1.f / lsum[hh];
            float *dst = o_dst + hh * o_hstride + c * EPC;
#pragma unroll
            for (int e = 0; e < EPC; e += 4)
                *reinterpret_cast<float4 *>(dst + e) =
                    make_float4(acc[hh][e] * inv, acc[hh][e + 1] * inv, acc[hh][e + 2] * inv,
                                acc[hh][e + 3] * inv);
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
            l_dst[hh * p.nsplit] = bad ? NAN : (m[hh] + fast_log2(lsum[hh])) * kLn2;
    }
}

constexpr int kTile = 32;

template <int EB, int D, int G>
cp_status launch_gqa(const GqaParams &p, int64_t items, hipStream_t stream) {
    constexpr int QREGS = G * (D * EB / 16 / 4) * 4;
    if constexpr (QREGS > 128) {
        return fail(CP_E_UNSUPPORTED, "gqa decode: group %d x head dim %d in %s is too wide", G, D,
                    EB == 4 ? "fp32" : "bf16");
    } else {
        const int64_t blocks = ceil_div(items, kWaves);
        if (blocks > 0x7fffffff) return fail(CP_E_UNSUPPORTED, "gqa decode: too many work items");
        // Two workgroups (8 waves) per CU when the tile's registers fit in 256
        // VGPRs, else one (wider groups / fp32 rows) to avoid spills.
        using Tr = GqaTraits<EB, D, G, kTile>;
        constexpr int kEst = QREGS + Tr::NPASS * Tr::NCQ * 4 + Tr::TPL * 4 + G * Tr::EPC + 40;
        constexpr int kMinWg = kEst <= 200 ? 2 : 1;
        hipLaunchKernelGGL((gqa_decode_kernel<EB, D, G, kTile, kMinWg>), dim3((unsigned)blocks),
                           dim3(64 * kWaves), 0, stream, p);
        return check_launch("cp_decode_attn_partial_gqa");
    }
}

template <int EB, int D>
cp_status dispatch_g(int G, const GqaParams &p, int64_t items, hipStream_t s) {
    switch (G) {
    case 1: return launch_gqa<EB, D, 1>(p, items, s);
    case 2: return launch_gqa<EB, D, 2>(p, items, s);
    case 4: return launch_gqa<EB, D, 4>(p, items, s);
    case 8: return launch_gqa<EB, D, 8>(p, items, s);
    }
    return fail(CP_E_UNSUPPORTED, "gqa decode: Hq/Hkv = %d not in {1, 2, 4, 8}", G);
}

int log2_exact(int32_t x) {
    if (x <= 0 || (x & (x - 1))) return -1;
    int l = 0;
    while ((1 << l) < x) ++l;
    return l;
}

}  // namespace

// Row-layout kernel: one partial slot per launched wave plus one per
// (request, KV head) boundary, then a (first, count) table.  T query tokens
// per request give T x Hq/Hkv rows per KV head.
static GqaPlan plan_rows(const cp_gqa_args &a, int T, bool mtp) {
    GqaPlan pl{};
    const int G = a.Hq / a.Hkv * T;
    pl.rows = true;
    pl.waves = gqa_rows_waves(a, T, mtp);
    const size_t slots = (size_t)pl.waves + (size_t)(a.B > 0 ? a.B : 0) * a.Hkv;
    pl.ws_bytes = slots * G * (a.D + 1) * sizeof(float) + (size_t)(a.B > 0 ? a.B : 0) * a.Hkv * 2 * 4 + 512;
    return pl;
}

// Multi-token decode: the request's q_len tokens in launches of Tg tokens
// (Tg Hq/Hkv rows of at most 8 per KV head, the row kernel's widest form),
// one after the other on the stream; the workspace holds one launch's
// partials and is reused.
GqaPlan plan_gqa_mtp(const cp_gqa_mtp_args &m) {
    const cp_gqa_args &a = m.base;
    if (a.Hkv < 1 || a.Hq % a.Hkv != 0 || m.q_len < 1) return GqaPlan{};
    const int Tg = gqa_mtp_group_tokens(a, m.q_len);
    if (Tg < 1 || !gqa_rows_supported(a, Tg)) return GqaPlan{};
    return plan_rows(a, Tg, true);
}

GqaPlan plan_gqa(const cp_gqa_args &a) {
    if (gqa_rows_supported(a)) return plan_rows(a, 1, false);
    GqaPlan pl{};
    // General kernel: split the capacity of each (request, KV head) into work
    // items of S tokens so that about 8K items exist; the hardware dispatcher
    // then balances the tail at the granularity of one item.  S is a power of
    // two in [64, 512] and at most 64 blocks (the LDS staging of block ids).
    const int64_t cap = (int64_t)a.bt_stride * a.bs;
    const int64_t heads = (int64_t)a.B * (a.Hkv > 0 ? a.Hkv : 1);
    int64_t S = 512;
    while (S > 64 && heads * ceil_div(cap, S) < 8192) S /= 2;
    while (S > 64 && S / (a.bs > 0 ? a.bs : 1) > kMaxSplitBlocks) S /= 2;
    pl.split_tokens = (int32_t)S;
    pl.nsplit = (int32_t)(cap > 0 ? ceil_div(cap, S) : 1);
    pl.ws_bytes = pl.nsplit > 1 ? (size_t)a.B * a.Hq * pl.nsplit * (a.D + 1) * sizeof(float) + 256
                                : 0;
    return pl;
}

}  // namespace cpattn

using namespace cpattn;

namespace cpattn {

// Host checks shared by the single- and multi-token entries (CP_OK or the error).
cp_status validate_gqa(const cp_gqa_args *a) {
    if (a->B < 0 || a->Hq < 1 || a->Hkv < 1 || a->D < 1 || a->bs < 1 || a->bt_stride < 1 ||
        a->num_blocks < 0)
        return fail(CP_E_INVALID, "gqa decode: B=%d Hq=%d Hkv=%d D=%d bs=%d bt_stride=%d", a->B,
                    a->Hq, a->Hkv, a->D, a->bs, a->bt_stride);
    if (a->Hq % a->Hkv != 0)
        return fail(CP_E_INVALID, "gqa decode: Hq=%d not a multiple of Hkv=%d", a->Hq, a->Hkv);
    if (a->dt != CP_F32 && a->dt != CP_BF16)
        return fail(CP_E_UNSUPPORTED, "gqa decode: dtype must be F32 or BF16");
    if (a->D != 64 && a->D != 128) return fail(CP_E_UNSUPPORTED, "gqa decode: D=%d", a->D);
    const int bs_log2 = log2_exact(a->bs);
    if (bs_log2 < 4)
        return fail(CP_E_UNSUPPORTED, "gqa decode: block size %d must be a power of two >= 16",
                    a->bs);
    if (!(a->scale == a->scale)) return fail(CP_E_INVALID, "gqa decode: scale is NaN");
    if (a->B == 0) return CP_OK;
    if (!a->q || !a->k_cache || !a->v_cache || !a->block_table || !a->local_len || !a->out ||
        !a->lse)
        return fail(CP_E_INVALID, "gqa decode: NULL pointer");
    if (!aligned16(a->q) || !aligned16(a->k_cache) || !aligned16(a->v_cache) ||
        !aligned16(a->out))
        return fail(CP_E_INVALID, "gqa decode: q, caches and out must be 16-byte aligned");
    return CP_OK;
}

namespace {

// The row-layout kernel and its split combine: Tg x Hq/Hkv rows per KV head
// (tokens t0 .. t0 + Tg - 1 of T), merged into out [B][T][Hq][D] and
// lse [B][T][Hq].
cp_status run_rows(const cp_gqa_args *a, int bs_log2, void *ws, const GqaPlan &pl,
                   const GqaMtp &mtp, hipStream_t stream) {
    const int T = mtp.Tg > 0 ? mtp.Tg : mtp.T;
    const int G = a->Hq / a->Hkv * T;
    const size_t slots = (size_t)pl.waves + (size_t)a->B * a->Hkv;
    float *ws_o = static_cast<float *>(ws);
    float *ws_l = ws_o + slots * G * a->D;
    int32_t *seg = reinterpret_cast<int32_t *>(
        (reinterpret_cast<uintptr_t>(ws_l + slots * G) + 255) & ~uintptr_t(255));
    cp_status st = gqa_rows_launch(*a, bs_log2, ws_o, ws_l, seg, pl.waves, mtp, stream);
    if (st != CP_OK) return st;
    MergeDesc m;
    m.seg = seg;
    m.rows_per_seg = G;
    m.n_parts = 0;
    m.rows = (int64_t)a->B * a->Hq * T;
    m.Dv = a->D;
    m.part_out = ws_o;
    m.part_lse = ws_l;
    m.o_part_stride = (int64_t)G * a->D;
    m.o_row_stride = a->D;
    m.l_part_stride = G;
    m.l_row_stride = 1;
    m.out = a->out;
    m.out_dt = CP_F32;
    m.lse_out = a->lse;
    m.remap_T = T;
    m.remap_G = a->Hq / a->Hkv;
    m.remap_Hkv = a->Hkv;
    m.remap_Tfull = mtp.T;
    m.remap_t0 = mtp.t0;
    return launch_merge(m, stream);
}

}  // namespace
}  // namespace cpattn

extern "C" cp_status cp_decode_attn_partial_gqa_mtp(const cp_gqa_mtp_args *m, void *ws,
                                                    size_t ws_bytes, hipStream_t stream) {
    clear_error();
    if (!m) return fail(CP_E_INVALID, "cp_decode_attn_partial_gqa_mtp: NULL args");
    const cp_gqa_args *a = &m->base;
    cp_status st = validate_gqa(a);
    if (st != CP_OK || a->B == 0) return st;
    if (m->q_len < 1 || m->dcp_size < 1 || m->dcp_rank < 0 || m->dcp_rank >= m->dcp_size ||
        m->interleave < 1 || (int64_t)m->dcp_size * m->interleave > (1 << 30))
        return fail(CP_E_INVALID, "gqa mtp decode: q_len=%d dcp rank %d of %d, interleave %d",
                    m->q_len, m->dcp_rank, m->dcp_size, m->interleave);
    if (!m->seq_len) return fail(CP_E_INVALID, "gqa mtp decode: NULL seq_len");
    const int tg_max = gqa_mtp_group_tokens(*a, m->q_len);
    if (tg_max < 1 || !gqa_rows_supported(*a, tg_max))
        return fail(CP_E_UNSUPPORTED,
                    "gqa mtp decode: Hq/Hkv = %d, D = %d (the row kernel takes groups of 1, 2, 4 "
                    "or 8 heads with 256-byte K/V rows)",
                    a->Hq / a->Hkv, a->D);
    const GqaPlan pl = plan_gqa_mtp(*m);
    if (!ws || ws_bytes < pl.ws_bytes)
        return fail(CP_E_WORKSPACE, "gqa mtp decode: workspace of %zu bytes needed, %zu given",
                    pl.ws_bytes, ws_bytes);
    GqaMtp mtp;
    mtp.T = m->q_len;
    mtp.seq_len = m->seq_len;
    mtp.dcp_rank = m->dcp_rank;
    mtp.dcp_size = m->dcp_size;
    mtp.dcp_I = m->interleave;
    // launches of tg_max tokens, then the largest power of two that the rest allows
    for (int t0 = 0; t0 < m->q_len;) {
        int tg = m->q_len - t0 < tg_max ? m->q_len - t0 : tg_max;
        while (tg & (tg - 1)) tg &= tg - 1;
        mtp.t0 = t0;
        mtp.Tg = tg;
        const cp_status st2 = run_rows(a, log2_exact(a->bs), ws, pl, mtp, stream);
        if (st2 != CP_OK) return st2;
        t0 += tg;
    }
    return CP_OK;
}

extern "C" cp_status cp_decode_attn_partial_gqa(const cp_gqa_args *a, void *ws, size_t ws_bytes,
                                                hipStream_t stream) {
    clear_error();
    if (!a) return fail(CP_E_INVALID, "cp_decode_attn_partial_gqa: NULL args");
    cp_status st0 = validate_gqa(a);
    if (st0 != CP_OK || a->B == 0) return st0;
    const int bs_log2 = log2_exact(a->bs);
    const GqaPlan pl = plan_gqa(*a);
    if (pl.ws_bytes > 0 && (!ws || ws_bytes < pl.ws_bytes))
        return fail(CP_E_WORKSPACE, "gqa decode: workspace of %zu bytes needed, %zu given",
                    pl.ws_bytes, ws_bytes);

    if (pl.rows) return run_rows(a, bs_log2, ws, pl, GqaMtp{}, stream);

    GqaParams p;
    p.q = to_global(a->q);
    p.kc = to_global(a->k_cache);
    p.vc = to_global(a->v_cache);
    p.bt = a->block_table;
    p.len = a->local_len;
    p.B = a->B;
    p.Hq = a->Hq;
    p.Hkv = a->Hkv;
    p.bs_log2 = bs_log2;
    p.bt_stride = a->bt_stride;
    p.num_blocks = a->num_blocks;
    p.qk_scale = a->scale * kLog2e;
    p.split_tokens = pl.split_tokens;
    p.nsplit = pl.nsplit;
    float *ws_o = static_cast<float *>(ws);
    float *ws_l = ws_o + (size_t)a->B * a->Hq * pl.nsplit * a->D;
    p.out = pl.nsplit > 1 ? ws_o : a->out;
    p.lse = pl.nsplit > 1 ? ws_l : a->lse;

    const int G = a->Hq / a->Hkv;
    const int64_t items = (int64_t)a->B * a->Hkv * pl.nsplit;
    cp_status st;
    if (a->dt == CP_BF16)
        st = a->D == 128 ? dispatch_g<2, 128>(G, p, items, stream)
                         : dispatch_g<2, 64>(G, p, items, stream);
    else
        st = a->D == 128 ? dispatch_g<4, 128>(G, p, items, stream)
                         : dispatch_g<4, 64>(G, p, items, stream);
    if (st != CP_OK || pl.nsplit == 1) return st;

    MergeDesc m;
    m.n_parts = pl.nsplit;
    m.rows = (int64_t)a->B * a->Hq;
    m.Dv = a->D;
    m.part_out = ws_o;
    m.part_lse = ws_l;
    m.o_part_stride = a->D;
    m.o_row_stride = (int64_t)pl.nsplit * a->D;
    m.l_part_stride = 1;
    m.l_row_stride = pl.nsplit;
    m.out = a->out;
    m.out_dt = CP_F32;
    m.lse_out = a->lse;
    return launch_merge(m, stream);
}
