// internal.hpp -- shared host/device helpers of libcpattn (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cpattn.h"

namespace cpattn {

// ---------------------------------------------------------------- host side

// Records a message for cp_last_error() (per host thread) and returns `st`.
cp_status fail(cp_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Returns CP_E_HIP with a message if the last launch on this thread failed.
cp_status check_launch(const char *what);

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int elem_bytes(cp_dtype dt) {
    switch (dt) {
    case CP_F32: return 4;
    case CP_BF16: return 2;
    case CP_FP8_E4M3FN: return 1;
    }
    return 0;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Split-K plans: how a decode call divides each request's local tokens.
struct GqaPlan {
    bool rows;             // balanced row-layout kernel (256-byte rows) or the general one
    int32_t split_tokens;  // general kernel: tokens per work item (multiple of 64)
    int32_t nsplit;        // general kernel: work items per (request, kv head)
    int32_t waves;         // row kernel: waves launched (one per resident slot)
    size_t ws_bytes;       // partial outputs + LSEs (+ segment table), 0 if none
};
GqaPlan plan_gqa(const cp_gqa_args &a);
// Host checks of a GQA decode call (CP_OK, or the error with its message set).
cp_status validate_gqa(const cp_gqa_args *a);
GqaPlan plan_gqa_mtp(const cp_gqa_mtp_args &m);

struct MlaPlan {
    int32_t split_tokens;
    int32_t nsplit;  // workgroups launched (partial slots besides the per-request ones)
    size_t ws_bytes;
};
MlaPlan plan_mla(const cp_mla_args &a);

// Exact LSE merge over strided partials (shared by cp_lse_merge and the
// split-K combine of the decode kernels).  Part i of row r:
//   out: part_out[i*o_part_stride + r*o_row_stride + d],
//   lse: part_lse[i*l_part_stride + r*l_row_stride].
// Output row r at out[r*Dv], lse_out[r] (lse_out may be null).
struct MergeDesc {
    // Optional per-row-group segment table: when seg != nullptr, row r belongs
    // to group r / rows_per_seg with (first slot, part count) at seg[2*group];
    // part i of row r then sits at slot first+i and the strides below apply to
    // slots: out at part_out[(first+i)*o_part_stride + (r % rows_per_seg)*o_row_stride],
    // LSE at part_lse[(first+i)*l_part_stride + (r % rows_per_seg)*l_row_stride].
    // A count of 0 gives an all-zero row with LSE -inf.
    const int32_t *seg = nullptr;
    int32_t rows_per_seg = 1;
    int32_t n_parts;
    int64_t rows;
    int32_t Dv;
    const float *part_out;  // fp32 partial outputs, or bf16 when part_bf16 (strides in elements)
    const float *part_lse;
    bool part_bf16 = false;
    int32_t parts_hint = 0;  // expected parts per row (segment tables): many parts share a row over waves
    int64_t o_part_stride, o_row_stride;
    int64_t l_part_stride, l_row_stride;
    void *out;
    cp_dtype out_dt;
    float *lse_out;
    // Output row of merge row r in multi-token decode: merge rows are
    // (request, KV head, token of the group, head in group), remap_T tokens
    // per group; outputs are [request][remap_Tfull][Hq] with the group's
    // tokens at remap_t0 .. (remap_Tfull 0: the group is every token).  See
    // merge_out_row.
    int32_t remap_T = 1, remap_G = 1, remap_Hkv = 1;
    int32_t remap_Tfull = 0, remap_t0 = 0;
};
cp_status launch_merge(const MergeDesc &m, hipStream_t stream);

__host__ __device__ inline int64_t merge_out_row(const MergeDesc &m, int64_t r) {
    const int64_t Tf = m.remap_Tfull > 0 ? m.remap_Tfull : m.remap_T;
    if (Tf <= 1) return r;
    const int64_t per = (int64_t)m.remap_T * m.remap_G;  // rows per (request, KV head)
    const int64_t seg = r / per, sub = r - seg * per;
    const int64_t b = seg / m.remap_Hkv, g = seg - b * m.remap_Hkv;
    const int64_t t = sub / m.remap_G, h = sub - t * m.remap_G;
    return (b * Tf + m.remap_t0 + t) * ((int64_t)m.remap_Hkv * m.remap_G) + g * m.remap_G + h;
}

// Compute units of the current device (cached per device).
int device_cus();

// Row-layout GQA decode kernel (256-byte KV rows), decode_gqa_rows.hip.
// T > 1: multi-token queries (the request's last T positions, causal on the
// shard's interleaved positions); T = 1 with seq_len == nullptr: single token.
struct GqaMtp {
    int32_t T = 1;
    const int32_t *seq_len = nullptr;
    int32_t dcp_rank = 0, dcp_size = 1, dcp_I = 1;
    // the tokens of one launch: t0 .. t0 + Tg - 1 of the T (Tg 0: all T)
    int32_t t0 = 0, Tg = 0;
};
bool gqa_rows_supported(const cp_gqa_args &a, int T = 1);
// tokens per launch of the multi-token entry: G = Tg Hq/Hkv rows must be 1, 2, 4 or 8
int gqa_mtp_group_tokens(const cp_gqa_args &a, int T);
int gqa_rows_waves(const cp_gqa_args &a, int T = 1, bool mtp = false);
cp_status gqa_rows_launch(const cp_gqa_args &a, int bs_log2, float *ws_o, float *ws_l,
                          int32_t *seg, int32_t W, const GqaMtp &mtp, hipStream_t stream);

// ---------------------------------------------------------------- device side

// Global-memory byte pointer: keeps loads on the global (not flat) path.
#define CP_GLOBAL __attribute__((address_space(1)))
typedef const uint8_t CP_GLOBAL gbyte;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

inline gbyte *to_global(const void *p) { return (gbyte *)(p); }

// Read-only metadata (block tables, lengths) read through the constant address
// space: uniform reads of it become scalar loads, which wait on their own
// counter instead of behind the KV vector loads in flight.
#define CP_CONST __attribute__((address_space(4)))
typedef const int32_t CP_CONST cint32;
inline cint32 *to_const(const int32_t *p) { return (cint32 *)(p); }

__device__ __forceinline__ u32x4 load16(gbyte *p) {
    return *reinterpret_cast<const CP_GLOBAL u32x4 *>(p);
}

// A 16-byte store of output that no later part of the same kernel reads:
// non-temporal, so that it streams to memory without allocating in the caches
// (for HBM-bound kernels that write as many bytes as they read this is worth
// ~20%: the KV gather went from 116 to 90 us per call).
__device__ __forceinline__ void store16_stream(void *p, const u32x4 &v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two floats to a bf16 pair (round to nearest even; lo in bits 0..15) in one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f32x2_cvt __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_cvt __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_cvt{lo, hi}, bf16x2_cvt));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
    return __shfl_xor(v, mask, 64);
}

}  // namespace cpattn
