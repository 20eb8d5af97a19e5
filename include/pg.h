/*
 * pg.h -- C ABI of the packed shared-prefix attention library (libpg.so).
 *
 * The operation: a batch holds groups; each group is one prompt prefix stored
 * once, followed by its response suffixes, all in one packed row of tokens
 * ("Preference Packing: Efficient Preference Optimization for LLMs", core idea
 * and technical framework). Prefix tokens attend causally within the prefix;
 * a suffix token attends to the whole prefix and causally to its own suffix,
 * never to a sibling suffix; position ids restart at the prefix length for
 * every suffix (verl "prefix_grouper_utils.py" page, section 1 and the
 * prefix-sharing diagram). Query blocks of all groups are scheduled as one
 * launch over a work list balanced by masked-area FLOPs ("PackInfer", abstract).
 *
 * Conventions for every entry point:
 *  - Packed token order: group 0 [prefix, suffix_1..suffix_n], group 1 [...],
 *    no padding. T = sum of all prefix and suffix lengths.
 *  - Device tensors are dense, row-major, caller-owned device pointers:
 *      Q, Q_out, O : [T, Hq, d]    K, K_out, V : [T, Hkv, d]
 *      lse         : [Hq, T] fp32  pos         : [T] int64
 *    Q/K/V/O share one dtype (pg_dtype). Query head h reads KV head
 *    h / (Hq / Hkv).
 *  - Calls that take a stream enqueue work on it and return without waiting;
 *    they never synchronise the device. Argument checks run before any launch.
 *  - Errors come back as pg_status; no exception crosses the ABI. The text of
 *    the last error of the calling thread is in pg_last_error().
 *  - T = 0 (or zero groups) is legal: the compute calls return PG_OK and
 *    launch nothing.
 */
#ifndef PG_H
#define PG_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pg_status {
  PG_OK = 0,
  PG_ERR_INVALID_ARG = -1, /* null pointer, negative length, bad head counts, overflow */
  PG_ERR_UNSUPPORTED = -2, /* head_dim or dtype this build has no kernel for           */
  PG_ERR_HIP = -3,         /* a HIP runtime call or kernel launch failed              */
  PG_ERR_OOM = -4,         /* host or device allocation failed                         */
  PG_ERR_STATE = -5        /* layout used on the device before pg_layout_upload        */
} pg_status;

typedef enum pg_dtype { PG_F32 = 0, PG_BF16 = 1 } pg_dtype;

/* Opaque packed layout: offsets, per-token descriptors, the key spans and the
 * FLOP-balanced work list. Immutable after it is built. */
typedef struct pg_layout pg_layout;

/* Summary of a built layout. */
typedef struct pg_layout_summary {
  int64_t total_tokens;    /* T                                                  */
  int32_t num_groups;      /* G                                                  */
  int32_t num_segments;    /* G + sum(suffix_counts): one prefix segment per group
                              plus one per suffix, zero-length ones included     */
  int32_t max_position;    /* largest position id (-1 when T = 0)                */
  int32_t num_items;       /* work items of the attention launch                 */
  int32_t num_spans;       /* key spans referenced by the work items             */
  int32_t block_tokens;    /* query tokens per work item (at most)               */
  int32_t heads_per_item;  /* query heads per work item                          */
  int32_t device_ready;    /* 1 once the device copy exists                      */
  int64_t useful_pairs;    /* allowed (query, key) pairs per query head; useful
                              FLOP of the attention = 4 * d * Hq * useful_pairs  */
  int64_t unpacked_pairs;  /* pairs of causal attention over every unpacked
                              prefix+suffix sequence (the work packing avoids)   */
  int64_t max_item_cost;   /* largest work item, in (query, key) pairs x heads   */
  int64_t max_xcd_cost;    /* largest per-XCD sum of item costs (balance check)  */
  int32_t num_kv_items;    /* work items of the backward dK/dV launch            */
  int32_t num_dec_items;   /* work items of the decode launch (padding included) */
  int64_t num_dec_refs;    /* entries of the decode merge lists                  */
  int32_t max_group_len;   /* longest group row (prefix + its responses): the
                              smallest max_len of the padded form                */
  int32_t reserved;        /* 0                                                  */
} pg_layout_summary;

/* One work item of the attention launch: query tokens [t0, t1) of one group,
 * query heads [hq0, hq0 + heads_per_item), keys from spans
 * [span0, span0 + nspan) of the span list, walked in ntiles tiles of 64 keys;
 * k0 and k1 repeat the first span, so a kernel can fetch its first tiles
 * without reading the span list. Items are stored in launch order: item p
 * runs on XCD p % 8; every item of one (group, KV head) sits on one XCD, and
 * each XCD's items are in cost-descending order per cluster. Items with
 * nspan == 0 are padding and do nothing. */
typedef struct pg_work_item {
  int32_t t0;
  int32_t t1;
  int32_t hq0;
  int32_t pe;     /* end of the group's prefix (absolute token index)       */
  int32_t span0;
  int32_t nspan;
  int32_t ntiles; /* sum over the spans of ceil(span length / 64)            */
  int32_t k0;     /* the first span, spans[span0]                            */
  int32_t k1;
  int32_t reserved;
  int64_t cost;   /* allowed (query, key) pairs of the item x its heads      */
} pg_work_item;

/* One work item of the backward dK/dV launch: keys [k0, k1) of KV head hk,
 * inside one segment (prompt or one response) of one group, at most 128 keys.
 * Every query that reads these keys lies in [k0, qend): qend is the group's end
 * for prompt keys and the response's end for response keys. Stored in launch
 * order like pg_work_item (XCD p % 8, clusters of one group and KV head on one
 * XCD); items with k0 == k1 are padding. */
typedef struct pg_kv_item {
  int32_t k0;
  int32_t k1;
  int32_t hk;
  int32_t qend;
  int64_t cost;   /* (query, key) pairs of the item x the r query heads      */
} pg_kv_item;

/* One work item of the decode launch (pg_attn_decode): cache rows [k0, k1) of
 * KV head hk inside one segment [seg0, seg1) of the layout -- a prompt
 * (resp = -1) or the segment of response `resp` at its capacity -- for the
 * query rows [row0, row0 + nrow), at most 32, where query row k * r + i is
 * query head hk * r + i of response k (r = Hq / Hkv). A prompt item carries
 * rows of the group's responses, a response item only rows of its own
 * response and stops, at run time, at that response's current length.
 * Launch order as pg_work_item (XCD p % 8); nrow == 0 marks padding. */
typedef struct pg_dec_item {
  int32_t k0;
  int32_t k1;
  int32_t hk;
  int32_t resp;
  int32_t seg0;
  int32_t seg1;
  int32_t row0;
  int32_t nrow;
} pg_dec_item;

/* A contiguous key range [k0, k1) inside one segment of one group. */
typedef struct pg_key_span {
  int32_t k0;
  int32_t k1;
} pg_key_span;

/*
 * pg_build_layout_host -- build the packed layout on the host only.
 *
 * Follows the grouping of "Preference Packing" (technical framework: store each
 * prompt once, then its responses) and the per-group prefix_len / suffix_lens
 * of the layout object on the verl page (sections 1-2).
 *
 *  num_groups      G >= 0
 *  prefix_lens     host int32 [G], each >= 0 (0: block-diagonal causal suffixes)
 *  suffix_counts   host int32 [G], each >= 0 (0: the group is its prefix alone)
 *  suffix_lens     host int32 [sum(suffix_counts)], each >= 0, group-major order;
 *                  zero-length suffixes occupy no tokens
 *  num_q_heads     Hq >= 1;  num_kv_heads Hkv >= 1 with Hq % Hkv == 0
 *  head_dim        d in {64, 128}
 *  rope_theta      > 0, base of the rotary frequencies used by pg_rope
 *  out             receives the new layout (caller frees with pg_layout_destroy)
 *
 * T must not exceed 2^30. Arrays are copied; the caller keeps ownership.
 * Returns PG_ERR_INVALID_ARG (bad argument), PG_ERR_UNSUPPORTED (head_dim),
 * PG_ERR_OOM. *out is set to NULL on error.
 */
pg_status pg_build_layout_host(int32_t num_groups, const int32_t* prefix_lens,
                               const int32_t* suffix_counts, const int32_t* suffix_lens,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               double rope_theta, pg_layout** out);

/*
 * pg_layout_upload -- copy the device part of a layout (per-token descriptors,
 * work list, key spans, rotary frequencies) to the current HIP device, enqueued
 * on `stream`. The image is written into pinned host memory and copied
 * asynchronously into a device buffer owned by the layout; both come from a
 * per-device cache of upload buffers that the library keeps until the process
 * ends. Never waits for the device. Calling it again is a no-op.
 * PG_ERR_HIP / PG_ERR_OOM on failure.
 *
 * Graph capture: when this call or any compute call with the layout is made
 * on a stream under capture, the layout's upload buffer is never reused,
 * even after pg_layout_destroy, so a captured graph stays valid for the life
 * of the process (the buffer is held that long).
 */
pg_status pg_layout_upload(pg_layout* layout, hipStream_t stream);

/*
 * pg_build_layout -- pg_build_layout_host followed by pg_layout_upload on
 * `stream`: the layout builder of the packed path (group offsets, prefix and
 * suffix spans, per-token descriptors and the work list of query blocks
 * balanced by masked-area FLOPs, after the load-balanced execution groups of
 * the "PackInfer" abstract).
 */
pg_status pg_build_layout(int32_t num_groups, const int32_t* prefix_lens,
                          const int32_t* suffix_counts, const int32_t* suffix_lens,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          double rope_theta, hipStream_t stream, pg_layout** out);

/* Fill *info. PG_ERR_INVALID_ARG on null. */
pg_status pg_layout_info(const pg_layout* layout, pg_layout_summary* info);

/* Host copies of the offsets: group_off [G+1] (first token of each group, then
 * T) and seg_off [num_segments+1] (first token of each segment, then T).
 * Either pointer may be NULL to skip it. */
pg_status pg_layout_copy_offsets(const pg_layout* layout, int32_t* group_off, int32_t* seg_off);

/* Host copies of the per-token descriptors, each [T] (any may be NULL):
 * g0 = first token of the token's group, pe = end of that group's prefix,
 * ss = first token of the token's own segment (g0 for prefix tokens). */
pg_status pg_layout_copy_tokens(const pg_layout* layout, int32_t* g0, int32_t* pe, int32_t* ss);

/* Host copies of the work list ([num_items], launch order) and of the key
 * spans ([num_spans]); either may be NULL. */
pg_status pg_layout_copy_work(const pg_layout* layout, pg_work_item* items, pg_key_span* spans);

/* Host copy of the backward dK/dV work list: items [num_kv_items]. */
pg_status pg_layout_copy_kv_work(const pg_layout* layout, pg_kv_item* items);

/* Host copy of the decode work list: items [num_dec_items] (launch order),
 * ref_off [N * Hkv + 1] and refs [num_dec_refs]: the items whose rows include
 * response k's query heads of KV head hk are refs[ref_off[k * Hkv + hk] ..
 * ref_off[k * Hkv + hk + 1]) (indices into items). Any pointer may be NULL. */
pg_status pg_layout_copy_decode_work(const pg_layout* layout, pg_dec_item* items,
                                     int32_t* ref_off, int32_t* refs);

/* Free the layout. Returns at once: its upload buffer goes back to the cache
 * and is reused only after the work already enqueued with this layout has
 * completed on every stream it was used on (an event is recorded after each
 * enqueue), so no pending call is cut short. A layout used on more than four
 * distinct streams makes this call wait for its device instead. A layout used
 * under graph capture keeps its buffer reserved (see pg_layout_upload), so
 * the graph may be replayed after this call. NULL is ignored. */
void pg_layout_destroy(pg_layout* layout);

/*
 * pg_position_ids -- int64 position id of every packed token, on the device.
 * verl page, section 1: a prefix token gets its index within the prefix; a
 * suffix token gets prefix_len + its index within its own suffix, so every
 * suffix restarts at prefix_len.
 *  pos   device int64 [T], written completely.
 * Needs an uploaded layout (PG_ERR_STATE otherwise).
 */
pg_status pg_position_ids(const pg_layout* layout, int64_t* pos, hipStream_t stream);

/*
 * pg_rope -- rotary embedding of Q and K at the given positions, one launch.
 * The pages fix only the positions (verl page, section 1); the rotation is the
 * rotate-half convention: for i < d/2, phi = pos * theta^(-2i/d) (computed in
 * fp64), (x_i, x_{i+d/2}) -> (x_i cos phi - x_{i+d/2} sin phi,
 *                             x_{i+d/2} cos phi + x_i sin phi),
 * arithmetic in fp64, result rounded once to the tensor dtype (nearest-even).
 * V is not touched.
 *  pos           device int64 [T], any values >= 0 (normally pg_position_ids)
 *  q_in, q_out   device [T, Hq, d];  k_in, k_out  device [T, Hkv, d]
 *                q_out may equal q_in and k_out may equal k_in (in place);
 *                other overlaps are not allowed. One pair may be NULL as a whole
 *                (q_in and q_out, or k_in and k_out): only the other is rotated
 *                (a decode step rotates the new token's K and Q separately).
 *  dtype         PG_F32 or PG_BF16
 */
pg_status pg_rope(const pg_layout* layout, const int64_t* pos, const void* q_in,
                  const void* k_in, void* q_out, void* k_out, pg_dtype dtype,
                  hipStream_t stream);

/*
 * pg_attn_fwd -- packed shared-prefix causal attention, forward.
 * For every token t and query head h: softmax over the allowed keys
 * K(t) = { j : j in t's group, j <= t, and j is a prefix token or in t's own
 * segment } of softmax_scale * <q[t,h], k[j,h/r]>, times v[j,h/r]; this equals
 * causal attention over the unpacked sequence prefix || own suffix
 * ("Preference Packing", core idea: prompt attention computed once and reused
 * by every response; verl page, prefix-sharing diagram).
 *  q, k, v   device inputs (layouts above), dtype `dtype`
 *  o         device [T, Hq, d] output in `dtype`, written completely
 *  lse       device fp32 [Hq, T]: ln(sum_j exp(softmax_scale * <q, k_j>)),
 *            written completely; may be NULL to skip it
 *  softmax_scale  finite, > 0
 * bf16 runs on the MFMA kernel (d = 128) with fp32 accumulation; fp32 and
 * bf16 with d = 64 run on a plain per-row kernel. Deterministic: every output
 * element is written by exactly one thread, no atomics.
 */
pg_status pg_attn_fwd(const pg_layout* layout, const void* q, const void* k, const void* v,
                      void* o, float* lse, pg_dtype dtype, float softmax_scale,
                      hipStream_t stream);


/*
 * pg_pack_rows -- build packed rows from right-padded per-prompt and
 * per-response rows: packed row t is row t - g0 of its group's prompt or row
 * t - (response start) of its response (verl prefix_grouper_utils.py page,
 * section 2: each prompt once, then its responses, right padding).
 *  prefix  [G, prefix_pad] rows (first prefix_lens[g] of group g used)
 *  suffix  [N, suffix_pad] rows, responses in group order (first suffix_lens[k] used)
 *  packed  [T] rows, written completely
 *  row_bytes  size of one row, a positive multiple of 4 (ids, hidden states,
 *             logits: any row type)
 * prefix_pad / suffix_pad must cover the longest prompt / response. Device
 * pointers; PG_ERR_INVALID_ARG on bad sizes or NULL where rows are needed.
 */
pg_status pg_pack_rows(const pg_layout* layout, const void* prefix, int32_t prefix_pad,
                       const void* suffix, int32_t suffix_pad, void* packed, int64_t row_bytes,
                       hipStream_t stream);

/*
 * pg_unpack_rows -- split packed rows back per prompt and per response, the
 * response part led by its group's last prompt row (verl page, section 3: the
 * output is split with the last prefix position included, whose logit
 * predicts the response's first token).
 *  prefix_out [G, prefix_pad] rows or NULL: row i of group g = packed row of
 *             prompt token i; zero past the prompt
 *  suffix_out [N, suffix_pad + 1] rows or NULL: row 0 = the group's last prompt
 *             row (zero for a group without prompt), row 1 + j = response
 *             token j; zero past the response
 * Both outputs are written completely. row_bytes as for pg_pack_rows.
 */
pg_status pg_unpack_rows(const pg_layout* layout, const void* packed, int64_t row_bytes,
                         void* prefix_out, int32_t prefix_pad, void* suffix_out,
                         int32_t suffix_pad, hipStream_t stream);

/*
 * pg_attn_bwd -- gradients of pg_attn_fwd's output O for an upstream gradient
 * dO: dQ, dK, dV. The derivative of the packed attention, by the chain rule:
 * with P the softmax of a row over its key set, dV = P^T dO, dS = P (dO V^T -
 * D) with D = rowsum(dO * O), dQ = scale dS K, dK = scale dS^T Q; KV heads sum
 * over their query heads. A prompt key is stored once, so its dK and dV collect
 * the gradient of every response of its group ("Preference Packing", core
 * idea: the prompt's attention is shared by all responses). lse carries no
 * gradient. Recomputes P from Q, K and the forward's lse.
 *  q, k, v     the forward's inputs (after RoPE)
 *  o, lse      the forward's outputs for the same inputs (lse fp32 [Hq, T])
 *  dout        dO [T, Hq, d]
 *  dq          [T, Hq, d], dk, dv [T, Hkv, d]: written completely (every row of
 *              dk/dv is written, zero where no query reads the key)
 *  delta       caller-owned device scratch of Hq * T floats; on return it holds
 *              D = rowsum(dO * O) of every (head, token) row, fp32 [Hq, T]
 * All tensors share dtype. bf16 with d = 128 runs the MFMA kernels (P and dS
 * enter the matrix cores rounded to bf16; dS is formed from P rounded to fp16,
 * 11 significant bits); fp32, and bf16 with d = 64, run a
 * reference-grade per-row path (one wave per query row, then one per key row,
 * fp32 arithmetic throughout; for correctness checks and small problems: it
 * reads every query row once per key that the row reads). dq, dk, dv must
 * not alias the inputs or each other. PG_ERR_UNSUPPORTED for another dtype.
 */
pg_status pg_attn_bwd(const pg_layout* layout, const void* q, const void* k, const void* v,
                      const void* o, const float* lse, const void* dout, void* dq, void* dk,
                      void* dv, float* delta, pg_dtype dtype, float softmax_scale,
                      hipStream_t stream);

/*
 * pg_decode_workspace_size -- bytes of device scratch pg_attn_decode needs on
 * this layout: one fp32 partial result (32 rows x (d + 2) floats) per decode
 * work item. 0 for a layout without responses.
 */
pg_status pg_decode_workspace_size(const pg_layout* layout, size_t* bytes);

/*
 * pg_attn_decode -- one decode step of shared-prefix attention over a
 * group-contiguous KV cache (PackInfer abstract: I/O-aware grouping co-locates
 * requests that share a prefix and keeps their KV cache group-contiguous as
 * generation proceeds, so a prompt's keys are read once per group per step).
 *
 * The cache is the layout's packed order with every response segment at its
 * capacity: build the layout with suffix_lens = the capacities. Response k's
 * first len_k = clamp(cur_lens[k], 0, capacity_k) rows are valid, the last of
 * them holding the token being decoded (its K and V already written). Its
 * query attends to the group's prompt rows and its own valid rows, never to a
 * sibling's.
 *  q          [N, Hq, d], the query of each response's newest token (N =
 *             sum(suffix_counts), responses in group order)
 *  k_cache, v_cache  [T, Hkv, d]
 *  cur_lens   device int32 [N]; read on the device, so a decode loop updates it
 *             without a host round trip
 *  o          [N, Hq, d], written completely (zero for an empty key set)
 *  lse        fp32 [Hq, N], natural log of the scaled scores' exp sum (-inf for
 *             an empty key set)
 *  workspace  device scratch of workspace_bytes >= pg_decode_workspace_size
 *             bytes (used by the bf16, d = 128 kernel; other dtypes and d = 64
 *             run one workgroup per output row and leave it untouched, and
 *             may pass NULL)
 * Device pointers; all tensors share dtype. Calls that share a workspace must
 * not overlap. PG_ERR_INVALID_ARG on NULL tensors, a short workspace or a bad
 * scale.
 */
pg_status pg_attn_decode(const pg_layout* layout, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* cur_lens, void* o, float* lse,
                         void* workspace, size_t workspace_bytes, pg_dtype dtype,
                         float softmax_scale, hipStream_t stream);

/* Size of the static device array pg_attn_decode_noalloc keeps its partial
 * results in (one copy per GPU, held until the process ends): 32 MiB, which
 * covers a decode step of up to 2016 work items at d = 128. */
#define PG_DECODE_SCRATCH_BYTES (32u << 20)

/*
 * pg_attn_decode_noalloc -- pg_attn_decode without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc). Same arguments,
 * results and errors as pg_attn_decode, bit-identical outputs (same kernels);
 * the bf16, d = 128 kernel keeps its partial results in a library-owned
 * static device array of PG_DECODE_SCRATCH_BYTES on the current GPU instead.
 * Allocates nothing: no hipMalloc, hipFree or allocating library call. The
 * array's device address is looked up on the first call on each GPU.
 * PG_ERR_INVALID_ARG (before any launch) when the layout's step needs more
 * than PG_DECODE_SCRATCH_BYTES (pg_decode_workspace_size tells); nothing in
 * the array needs to start at zero (every partial a step reads is written by
 * that step first). Every call on one GPU shares that GPU's array, which keeps
 * the last call's contents: calls that overlap on one GPU (other streams,
 * other threads, without ordering between them) race, and the caller must
 * order them.
 */
pg_status pg_attn_decode_noalloc(const pg_layout* layout, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* cur_lens, void* o, float* lse,
                                 pg_dtype dtype, float softmax_scale, hipStream_t stream);

/*
 * Right-padded compatibility form. The verl page (sections 1-2) keeps a batch
 * as [G, max_len]: row g is group g's packed row (prompt, then each response),
 * right-padded; its position ids start from zeros (section 1), so padding
 * keeps position 0, and its padding mask marks the real tokens. These calls
 * convert between that form and the packed rows every other call takes.
 * max_len must be >= max_group_len (pg_layout_info); PG_ERR_INVALID_ARG
 * otherwise, or for NULL outputs or a row_bytes that is not a positive
 * multiple of 4. Device pointers; outputs are written completely.
 */

/* pos: int64 [G, max_len], the padded form's position ids (padding 0);
 * mask: uint8 [G, max_len] or NULL, 1 on real tokens and 0 on padding. */
pg_status pg_position_ids_padded(const pg_layout* layout, int32_t max_len, int64_t* pos,
                                 uint8_t* mask, hipStream_t stream);

/* padded [G, max_len] rows of row_bytes <- packed [T] rows; padding rows zero. */
pg_status pg_pad_rows(const pg_layout* layout, const void* packed, int64_t row_bytes,
                      void* padded, int32_t max_len, hipStream_t stream);

/* packed [T] rows <- the real rows of padded [G, max_len] (padding not read). */
pg_status pg_unpad_rows(const pg_layout* layout, const void* padded, int32_t max_len,
                        int64_t row_bytes, void* packed, hipStream_t stream);

/* Static text for a status code. */
const char* pg_status_string(pg_status status);

/* Text of the last error raised on the calling thread ("" if none). */
const char* pg_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PG_H */
