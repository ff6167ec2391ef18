/*
 * cpattn.h -- C ABI of libcpattn: the single-GPU hot path of decode / prefill
 * context parallelism (DCP / PCP) for AMD Instinct MI355X (gfx950).
 *
 * Pages that define the operations (cited by title and section):
 *   [P1] "Breaking the Long-Sequence Inference Bottleneck: A Deep Dive into
 *        vLLM's Distributed Context Parallelism Architecture"
 *   [P3] "vLLM DCP and PCP: Decode and Prefill Context Parallelism"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every data pointer is a DEVICE pointer owned by the caller.  Arrays are
 *    dense and row-major in the shapes stated; base pointers of element data
 *    must be 16-byte aligned.  The library never allocates or frees device
 *    memory and keeps no state between calls besides its loaded kernels.
 *  - Calls are asynchronous on the given HIP stream and never synchronise.
 *    Argument errors are detected on the host before anything is launched;
 *    values that live in device memory (lengths, block ids, positions) are
 *    checked by the kernels, which never read or write out of bounds: the
 *    affected outputs are marked as stated per call (slot -2, NaN rows).
 *  - Return value: CP_OK, or an error code with a message available from
 *    cp_last_error() (per host thread).  No exception crosses the ABI.
 *  - LSE values are fp32 natural-log log-sum-exp.  A key set that is empty
 *    yields LSE = -inf and an all-zero output row.
 *  - Inputs are never written; outputs may not alias inputs.
 */
#ifndef CPATTN_H
#define CPATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CP_ABI_VERSION 1

typedef enum cp_status {
    CP_OK = 0,
    CP_E_INVALID = 1,     /* bad argument: shape, rank, size, null or misaligned pointer */
    CP_E_UNSUPPORTED = 2, /* valid, but this dtype / shape has no kernel */
    CP_E_WORKSPACE = 3,   /* workspace missing or smaller than cp_workspace_bytes() */
    CP_E_HIP = 4          /* a HIP launch error */
} cp_status;

typedef enum cp_dtype {
    CP_F32 = 0,
    CP_BF16 = 1,
    CP_FP8_E4M3FN = 2 /* OCP 8-bit E4M3, finite-only ("fn"), max 448 */
} cp_dtype;

/* Slot values produced by cp_slot_map besides real slots. */
#define CP_SLOT_NOT_MINE (-1) /* another rank owns the token: the cache write skips it */
#define CP_SLOT_INVALID (-2)  /* bad metadata (request id, position, block table too short) */

const char *cp_status_str(cp_status s);
const char *cp_last_error(void);
int cp_abi_version(void);

/* ------------------------------------------------------------------------
 * Ownership and paging
 * ------------------------------------------------------------------------ */

/* Local KV length of every request on one rank ([P3] Deep Dive 5,
 * get_dcp_local_seq_lens): the number of positions t in [0, seq_lens[b])
 * with floor(t / I) mod N == rank ([P1] section 2 rank formula).
 *   seq_lens  [B] int32, >= 0 (a negative length gives local length 0)
 *   local_lens[B] int32 output
 * Errors: CP_E_INVALID if B < 0, N < 1, I < 1, rank outside [0, N), or a
 * pointer is NULL while B > 0. */
cp_status cp_local_seq_lens(int32_t B, const int32_t *seq_lens, int32_t rank, int32_t N,
                            int32_t I, int32_t *local_lens, hipStream_t stream);

/* Slot mapping with interleaved ownership ([P1] section 2, "Interleave Size"
 * and "Diagram: Actual mapping of the Block Table and Slot Mapping";
 * [P3] Deep Dive 5).  For token j of request req[j] at position t = pos[j]:
 *   owner = floor(t / I) mod N;  owner != rank  ->  slot_out[j] = -1
 *   else  l = floor(t / (N*I)) * I + t mod I   (tokens this rank owns before t)
 *         slot_out[j] = block_table[req[j]*bt_stride + l / bs] * bs + l mod bs
 * With I dividing bs this is the pages' virtual block: block_size x N logical
 * positions fill one physical block on every rank.
 *   req, pos     [T] int32          block_table [B][bt_stride] int32
 *   slot_out     [T] int64 output   max_blocks: valid columns of block_table
 * slot_out[j] = -2 if req[j] is outside [0, B), t < 0, or l / bs >= max_blocks.
 * Block ids themselves are not range-checked here (cp_cache_write checks them).
 * Errors: CP_E_INVALID for T < 0, B < 1, N < 1, I < 1, bs < 1, rank outside
 * [0, N), max_blocks outside [1, bt_stride], or NULL pointers with T > 0. */
cp_status cp_slot_map(int32_t T, const int32_t *req, const int32_t *pos,
                      const int32_t *block_table, int32_t B, int32_t bt_stride,
                      int32_t max_blocks, int32_t rank, int32_t N, int32_t I, int32_t bs,
                      int64_t *slot_out, hipStream_t stream);

/* Paged KV-cache write ([P1] section 2: entries of -1 are skipped;
 * [P3] Deep Dive 4, do_kv_cache_update).  A bitwise copy of each token's rows
 * to its slot; the source rows are already in the cache's dtype.
 *   GQA: k, v       [T][n_kv_heads][row_dim]
 *        k_cache, v_cache [num_blocks][n_kv_heads][bs][row_dim]
 *   MLA (one latent row per token, used as both key and value): pass
 *        v = v_cache = NULL, n_kv_heads = 1: k [T][row_dim] -> k_cache
 *        [num_blocks][bs][row_dim].
 *   slot [T] int64 from cp_slot_map.
 * Tokens with slot < 0 or slot >= num_blocks * bs are skipped.
 * Errors: CP_E_INVALID for negative sizes, NULL pointers, only one of v /
 * v_cache given; CP_E_UNSUPPORTED if row_dim * elem_size is not a multiple of
 * 16 bytes. */
cp_status cp_cache_write(int64_t T, const int64_t *slot, const void *k, const void *v,
                         int32_t n_kv_heads, int32_t row_dim, cp_dtype dt, void *k_cache,
                         void *v_cache, int64_t num_blocks, int32_t bs, hipStream_t stream);

/* cp_slot_map followed by cp_cache_write in one launch (the same two steps of
 * [P1] section 2 and [P3] Deep Dive 4-5 for a step's new tokens): every token's
 * slot is computed as cp_slot_map computes it and its rows are copied as
 * cp_cache_write copies them; the results are identical to the two calls.
 * Arguments are those of the two calls; slot_out [T] int64 may be NULL (the
 * slots are then not stored).  Errors: those of both calls. */
cp_status cp_slot_map_cache_write(int32_t T, const int32_t *req, const int32_t *pos,
                                  const int32_t *block_table, int32_t B, int32_t bt_stride,
                                  int32_t max_blocks, int32_t rank, int32_t N, int32_t I,
                                  int32_t bs, int64_t *slot_out, const void *k, const void *v,
                                  int32_t n_kv_heads, int32_t row_dim, cp_dtype dt, void *k_cache,
                                  void *v_cache, int64_t num_blocks, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Rank-local decode attention: partial output + LSE
 * ([P3] Deep Dive 6, "Deriving the partial and global outputs": every rank
 * uses the same query against its own KV shard and returns o_i and L_i;
 * [P1] section 3, GQA path step 2 "Attention: local computation")
 * ------------------------------------------------------------------------ */

typedef struct cp_gqa_args {
    const void *q;              /* [B][Hq][D], dtype dt (the full query on every rank) */
    const void *k_cache;        /* [num_blocks][Hkv][bs][D], dtype dt */
    const void *v_cache;        /* [num_blocks][Hkv][bs][D], dtype dt */
    const int32_t *block_table; /* [B][bt_stride] physical block of local block j */
    const int32_t *local_len;   /* [B] tokens of request b held by this shard */
    int32_t B, Hq, Hkv, D;      /* query head h reads KV head floor(h*Hkv/Hq) */
    int32_t bs, bt_stride;      /* block size; block-table row stride (= capacity in blocks) */
    int64_t num_blocks;         /* blocks in the cache pool */
    float scale;                /* softmax scale (1/sqrt(D) on the pages) */
    cp_dtype dt;                /* CP_F32 or CP_BF16 for q and the caches */
    float *out;                 /* [B][Hq][D] fp32 output: o_i */
    float *lse;                 /* [B][Hq]    fp32 output: L_i */
} cp_gqa_args;

/* Exact attention of q[b,h] over the shard's local tokens 0..local_len[b]-1
 * of request b (the shard's local tokens are non-causal to the decode query:
 * they are all earlier positions or the query's own token).
 * Supported: D in {64, 128}; Hq/Hkv in {1, 2, 4, 8}; dt in {CP_F32, CP_BF16}.
 * A request whose local_len exceeds bt_stride*bs, or whose block table names a
 * block outside [0, num_blocks), gets NaN in all its output rows and LSEs.
 * Workspace: cp_workspace_bytes(CP_OP_DECODE_GQA, &args) bytes (split-K
 * partials); it need not be initialised.
 * Errors: CP_E_INVALID (sizes, Hq % Hkv, NULL pointers), CP_E_UNSUPPORTED,
 * CP_E_WORKSPACE. */
cp_status cp_decode_attn_partial_gqa(const cp_gqa_args *args, void *workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/* The same call without a caller workspace, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid allocation): the split-context partials go to a scratch array
 * the library holds on each device, of cp_noalloc_scratch_bytes() bytes
 * (16 MiB; the array stays allocated on every GPU the library has run on
 * until the process ends).  Results are those of cp_decode_attn_partial_gqa
 * with a workspace.  The call allocates nothing.  All calls on one device
 * share that device's array: calls that overlap in time on one device (other
 * streams, other host threads) race and must be serialised by the caller.
 * Errors: as cp_decode_attn_partial_gqa; CP_E_WORKSPACE if the call needs more
 * split-partial space than the scratch holds (cp_workspace_bytes(
 * CP_OP_DECODE_GQA, args) > cp_noalloc_scratch_bytes(), e.g. B x Hkv above
 * ~7,000 at Hq/Hkv = 4, D = 128); CP_E_HIP if the scratch address cannot be
 * looked up. */
cp_status cp_decode_attn_partial_gqa_noalloc(const cp_gqa_args *args, hipStream_t stream);
size_t cp_noalloc_scratch_bytes(void);

/* Multi-token decode queries (speculative decoding / MTP verification: [P1]
 * "Inapplicable scenarios and known limitations" and [P4] "Future Roadmap"
 * name the combination of DCP with MTP and speculative decoding).  Request b's
 * q_len query tokens are its last q_len positions, seq_len[b] - q_len + t for
 * t = 0 .. q_len-1, their K/V already written to the caches; token t attends
 * the keys at positions <= its own ("a token sees itself and earlier
 * positions", [P1] section 4).  On DCP rank dcp_rank of dcp_size (interleave
 * I) the shard holds local keys in increasing position order, so token t sees
 * the shard's first min(local_len[b], owned_below(seq_len[b] - q_len + t + 1))
 * keys, owned_below(x) = floor(x / (N I)) I + clamp(x mod N I - rank I, 0, I)
 * ([P1] section 2).  A token with no visible key on the shard gets o = 0 and
 * LSE -inf.
 *   base.q   [B][q_len][Hq][D], base.out [B][q_len][Hq][D] fp32,
 *   base.lse [B][q_len][Hq] fp32; other base fields as cp_gqa_args.
 * Supported: 256-byte K/V rows (bf16 D 128 or fp32 D 64), Hq/Hkv in
 * {1, 2, 4, 8}, any q_len >= 1.  The tokens are processed in launches of a
 * power of two tokens, at most 8 / (Hq/Hkv) (8 query rows per KV head), one after the other on
 * the stream; each launch reads the shard's K/V once, so q_len * Hq/Hkv above
 * 8 costs ceil(q_len * Hq/Hkv / 8) or more passes over the shard.
 * seq_len[b] < q_len gives NaN rows.
 * Workspace: cp_workspace_bytes(CP_OP_DECODE_GQA_MTP, &args) (one launch's
 * partials, reused by the next); need not be initialised.
 * Errors: as cp_decode_attn_partial_gqa, plus CP_E_INVALID for q_len < 1, a
 * rank outside [0, dcp_size), interleave < 1, NULL seq_len; CP_E_UNSUPPORTED
 * for other shapes. */
typedef struct cp_gqa_mtp_args {
    cp_gqa_args base;
    int32_t q_len;              /* query tokens per request */
    int32_t dcp_rank, dcp_size; /* this shard's rank and the DCP group size */
    int32_t interleave;         /* I: consecutive positions per rank */
    const int32_t *seq_len;     /* [B] global context length, including the q_len tokens */
} cp_gqa_mtp_args;

cp_status cp_decode_attn_partial_gqa_mtp(const cp_gqa_mtp_args *args, void *workspace,
                                         size_t workspace_bytes, hipStream_t stream);

typedef struct cp_mla_args {
    const void *q;              /* [B][H][Dk] bf16 absorbed queries */
    const void *kv_cache;       /* [num_blocks][bs][Dk], dtype kv_dt: latent rows */
    const int32_t *block_table; /* [B][bt_stride] */
    const int32_t *local_len;   /* [B] */
    int32_t B, H, Dk, Dv;       /* keys: all Dk columns; values: first Dv columns */
    int32_t bs, bt_stride;
    int64_t num_blocks;
    float scale;                /* softmax scale */
    cp_dtype kv_dt;             /* CP_BF16 or CP_FP8_E4M3FN */
    float kv_scale;             /* fp8: element value = decoded byte * kv_scale (ignored for bf16) */
    float *out;                 /* [B][H][Dv] fp32 */
    float *lse;                 /* [B][H] fp32 */
} cp_mla_args;

/* Absorbed multi-head latent attention on one DCP shard: one latent KV row
 * per token shared by all H query heads ([P1] section 3 "MLA path", KV head
 * effectively 1; [P3] Deep Dive 6: local attention then exact merge).
 * Supported: Dk = 576, Dv = 512, bs a power of two >= 16, H a multiple of 16 up to
 * 128, B up to 4096 (CP_E_UNSUPPORTED otherwise).
 * Bad lengths / block ids give NaN rows as for GQA.
 * Workspace: cp_workspace_bytes(CP_OP_DECODE_MLA, &args); need not be
 * initialised.  The context of a request is split over the GPU's compute
 * units; the split outputs are held there in bf16 (their LSEs in fp32) and
 * merged exactly into out/lse, so out carries the rounding of one bf16 store
 * (relative 2^-9) on top of the kernel's own.
 * Errors: as cp_decode_attn_partial_gqa, plus CP_E_INVALID for num_blocks < 1,
 * a scale that is not finite, or (fp8) a kv_scale that is not positive and
 * finite. */
cp_status cp_decode_attn_partial_mla(const cp_mla_args *args, void *workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Exact LSE merge ([P3] Deep Dive 6: l = max_i L_i, a_i = exp(L_i - l),
 * O = sum a_i o_i / sum a_i, L = l + log sum a_i; [P1] section 3,
 * correct_attn)
 * ------------------------------------------------------------------------ */

/*   part_out [n_parts][rows][Dv] fp32, part_lse [n_parts][rows] fp32
 *   out      [rows][Dv], dtype out_dt (CP_F32 or CP_BF16, round to nearest even)
 *   lse_out  [rows] fp32, may be NULL
 * Parts with LSE = -inf get weight 0 (their outputs are not read); a row
 * whose parts are all -inf gets out = 0, LSE = -inf.  A NaN LSE gives a NaN
 * row.  Supported: Dv a multiple of 4, n_parts >= 1.
 * Errors: CP_E_INVALID for n_parts < 1, rows < 0, Dv < 1, NULL pointers;
 * CP_E_UNSUPPORTED for Dv % 4 != 0 or out_dt not F32/BF16. */
cp_status cp_lse_merge(int32_t n_parts, int64_t rows, int32_t Dv, const float *part_out,
                       const float *part_lse, void *out, cp_dtype out_dt, float *lse_out,
                       hipStream_t stream);

/* ------------------------------------------------------------------------
 * Head-scattered exchange steps around the merge ([P3] Deep Dive 6: the
 * AG+RS path corrects every rank's output after the LSE all-gather and
 * reduce-scatters heads; the A2A path packs each partial output with its fp32
 * LSE into one buffer, exchanges head partitions with one all-to-all and
 * reduces them exactly).  The collectives themselves are not part of this
 * library; these are the per-rank kernels on either side of them.
 * ------------------------------------------------------------------------ */

/* AG+RS correction of one rank's partial: with L = log sum_i exp(L_i) over
 * the n_parts gathered LSEs of each row,
 *     corrected[r][d] = part_out_i[r][d] * exp(L_i[r] - L[r]),
 * so that summing the n_parts corrected outputs (the reduce-scatter) gives the
 * merged output.  part_out_i [rows][Dv] is rank `rank`'s partial, part_lse
 * [n_parts][rows] every rank's LSE.  lse_out [rows] (may be NULL) receives L.
 * A part with L_i = -inf gets factor 0 (its output is not read); a row whose
 * parts are all -inf gets zeros and L = -inf; a NaN LSE gives a NaN row.
 * Errors: as cp_lse_merge, plus CP_E_INVALID for rank outside [0, n_parts). */
cp_status cp_lse_correct(int32_t n_parts, int64_t rows, int32_t Dv, int32_t rank,
                         const float *part_out_i, const float *part_lse, float *corrected,
                         float *lse_out, hipStream_t stream);

/* A2A packing of one rank's partial: out [B][H][Dv] and lse [B][H] (fp32) go
 * to buf [N][B][H/N][Dv + 4] fp32, destination d getting heads
 * d*H/N .. (d+1)*H/N - 1; a packed row is the Dv outputs, the LSE, and three
 * zero floats (rows stay 16-byte aligned).  Requires H % N == 0, Dv % 4 == 0.
 * Errors: CP_E_INVALID (sizes, H % N, NULL or misaligned pointers),
 * CP_E_UNSUPPORTED (Dv % 4). */
cp_status cp_a2a_pack(int32_t B, int32_t H, int32_t Dv, int32_t N, const float *out,
                      const float *lse, float *buf, hipStream_t stream);

/* Exact merge of n_parts packed partials (after the all-to-all): part i of
 * row r is at packed[i * part_stride + r * (Dv + 4)] (Dv outputs, then the
 * LSE), part_stride >= rows * (Dv + 4) floats.  Same arithmetic and output
 * contract as cp_lse_merge.
 * Errors: as cp_lse_merge, plus CP_E_INVALID for a part_stride below
 * rows * (Dv + 4). */
cp_status cp_lse_merge_packed(int32_t n_parts, int64_t rows, int32_t Dv, const float *packed,
                              int64_t part_stride, void *out, cp_dtype out_dt, float *lse_out,
                              hipStream_t stream);

/* ------------------------------------------------------------------------
 * PCP load-balanced causal prefill ([P1] section 4 "Head-tail concatenation
 * strategy" and "Minimal state progression"; section 5 "AllGather Q path";
 * [P3] Deep Dive 3)
 * ------------------------------------------------------------------------ */

#define CP_KV_DENSE 0 /* new-chunk keys/values, contiguous, causal mask on positions */
#define CP_KV_PAGED 1 /* one DCP shard of the cached prefix, all positions visible */
#define CP_KV_PAGED_CAUSAL 2 /* one DCP shard holding prefix AND chunk keys (interleaved):
                                 each query sees the shard's keys at positions <= its own */

typedef struct cp_prefill_args {
    const void *q;          /* [C][Hq][D] bf16: the whole new chunk in position order */
    int32_t C;              /* new tokens, a multiple of 2*pcp_size */
    int32_t P;              /* cached prefix length: the chunk covers positions P..P+C-1 */
    int32_t pcp_rank, pcp_size;
    int32_t Hq, Hkv, D;
    float scale;
    int32_t kv_source;      /* CP_KV_DENSE or CP_KV_PAGED */
    /* CP_KV_DENSE: */
    const void *k, *v;      /* [C][Hkv][D] bf16, chunk keys/values in position order */
    /* CP_KV_PAGED: */
    const void *k_cache, *v_cache; /* [num_blocks][Hkv][bs][D] bf16 */
    const int32_t *block_table;    /* [bt_stride] blocks of this shard's prefix tokens */
    int32_t local_len;      /* prefix tokens held by the shard (host value) */
    int32_t bs, bt_stride;
    int64_t num_blocks;
    float *out;             /* [2][C/(2*pcp_size)][Hq][D] fp32: head piece, then tail piece */
    float *lse;             /* [2][C/(2*pcp_size)][Hq] fp32 */
    /* CP_KV_PAGED_CAUSAL (ignored otherwise): the shard's place in the DCP
     * group; its local key l sits at global position
     * floor(l/I)*dcp_size*I + dcp_rank*I + l mod I */
    int32_t dcp_rank, dcp_size, dcp_interleave;
} cp_prefill_args;

/* The chunk is cut into 2*pcp_size equal pieces; rank r computes the query
 * rows of pieces r and 2*pcp_size-1-r, in that order.  Query row i of the
 * chunk sits at global position P+i.
 *  - CP_KV_DENSE: keys are the chunk's own tokens at positions <= the
 *    query's (causal, "itself and preceding positions").
 *  - CP_KV_PAGED: keys are one DCP shard's prefix tokens (all before every
 *    chunk position, so no mask): the "Full Q + Partial KV" step of the
 *    AllGather-Q path; partials are then merged with cp_lse_merge.
 *  - CP_KV_PAGED_CAUSAL: keys are one DCP shard's tokens of prefix and chunk
 *    alike (the chunk's KV written interleaved like the prefix's, the DCP
 *    long-prefill of [P1] section 5 "AllGather Q path"): the query at
 *    position p sees the shard's keys at positions <= p, i.e. its first
 *    cnt(p + 1) local keys, cnt(x) being the positions below x the shard owns
 *    ([P1] section 2).  local_len bounds the keys (at least cnt(P + C));
 *    merging the dcp_size shards' partials gives the causal attention over
 *    prefix and chunk.
 * Supported: any C that is a multiple of 2*pcp_size (pieces of any length: the
 * pages' PCP2 example with C = 8 gives pieces of 2 rows); D = 128, Hq/Hkv in
 * {1, 2, 4, 8}, bf16; K/V sources of fewer than 2^31 rows of D (C x Hkv
 * dense, num_blocks x Hkv x bs paged); paged block sizes a power of two >= 16.
 * Workspace: none needed (cp_workspace_bytes returns 0).
 * Errors: CP_E_INVALID (C % (2*pcp_size), rank, sizes, pointers, a scale
 * that is not positive and finite; for CP_KV_PAGED_CAUSAL a dcp_rank outside
 * [0, dcp_size), dcp_interleave < 1 or local_len below cnt(P + C)),
 * CP_E_UNSUPPORTED. */
cp_status pcp_prefill_attn_causal(const cp_prefill_args *args, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * KV gather: the inverse of the interleaved placement ([P1] section 3, "MLA
 * path": after the all-gather, the KV of every rank is reorganised into each
 * request's contiguous order before attention; [P1] section 2 for the
 * ownership and local-index rules it inverts)
 * ------------------------------------------------------------------------ */

#define CP_MAX_SHARDS 16

typedef struct cp_kv_gather_args {
    int32_t N, I, bs;       /* DCP shards (1..CP_MAX_SHARDS), interleave size, block size */
    int32_t B;              /* requests */
    int32_t Hkv, D;         /* heads and elements of a cache row: GQA K/V (Hkv, D) or the
                               MLA latent (Hkv = 1, D = 576) */
    cp_dtype dt;            /* element type of the caches and the outputs */
    const void *const *k_caches;        /* HOST array [N] of device pointers: shard r's cache
                                           [num_blocks[r]][Hkv][bs][D] (latent: K only) */
    const void *const *v_caches;        /* HOST array [N] of device pointers, or NULL */
    const int32_t *const *block_tables; /* HOST array [N] of device pointers: shard r's
                                           [B][bt_stride] physical block of local block j */
    const int64_t *num_blocks;          /* HOST array [N]: blocks in shard r's pool */
    int32_t bt_stride;
    int32_t t0, W;          /* window of global positions t0 .. t0+W-1 of every request */
    const int32_t *seq_len; /* [B] device: global length L_b of request b */
    void *k_out;            /* [B][W][Hkv][D] device, type dt */
    void *v_out;            /* [B][W][Hkv][D] device; NULL iff v_caches is NULL */
} cp_kv_gather_args;

/* For every request b and window row i (global position t = t0 + i):
 *  - t < L_b: the row is copied bit for bit from the cache of the shard that
 *    owns t, r = floor(t/I) mod N, at local index
 *    l = floor(t/(N*I))*I + t mod I, i.e. cache slot
 *    block_tables[r][b][floor(l/bs)]*bs + l mod bs (the slot cp_slot_map
 *    gives t on rank r);
 *  - t >= L_b: the row is zero;
 *  - a local block index past bt_stride or a block id outside
 *    [0, num_blocks[r]): the row is filled with 0xFF bytes (NaN in every
 *    supported dtype).
 * The output is token-major, so a window of the cached prefix can feed
 * pcp_prefill_attn_causal's CP_KV_DENSE source.
 * Supported: D * elem_size a multiple of 16; for Hkv > 1 also Hkv and
 * D * elem_size / 16 powers of two.
 * Errors: CP_E_INVALID (N outside 1..CP_MAX_SHARDS, I, bs, B, W, t0 < 0,
 * NULL or misaligned pointers, v_out without v_caches or the reverse),
 * CP_E_UNSUPPORTED (row shape). */
cp_status cp_kv_gather(const cp_kv_gather_args *args, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Workspace sizing
 * ------------------------------------------------------------------------ */
#define CP_OP_DECODE_GQA 1
#define CP_OP_DECODE_MLA 2
#define CP_OP_PREFILL 3
#define CP_OP_DECODE_GQA_MTP 4

/* Bytes of device workspace the call with these arguments needs (0 if none);
 * args points to the op's argument struct.  Returns (size_t)-1 for an unknown
 * op or NULL args. */
size_t cp_workspace_bytes(int op, const void *args);

#ifdef __cplusplus
}
#endif

#endif /* CPATTN_H */
