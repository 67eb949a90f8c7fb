/* kda_attn.h - C ABI of packed-varlen causal GQA training attention with head
 * dimension 256 (forward and first-order backward) for MI355X (gfx950).
 *
 * flashinfer PR #7774, description and commit notes: dense GQA attention over
 * inputs packed by cu_seqlens, a causal mask aligned to the bottom right of
 * each segment so that query and key lengths may differ, BF16 inputs and
 * outputs with FP32 accumulation, the forward with the natural-log LSE, and a
 * backward whose dK / dV are FP32 sums over the query heads of each key head,
 * returned in one of three forms: BF16, FP32 window gradients, or added in
 * FP32 into caller-owned destinations through a row map (repeated
 * destination rows allowed). Per segment s with Lq queries and Lk keys, query
 * row i (0-based in the segment) of head h sees key j of key head
 * h / (Hq / Hkv) iff j <= i + (Lk - Lq):
 *
 *     lse_i = log sum_j exp(scale <q_i, k_j>),   o_i = sum_j exp(scale <q_i, k_j> - lse_i) v_j
 *
 * A row that sees no key gets o = 0 and lse = -inf, and no gradient.
 *
 * Conventions (as kda.h): DEVICE pointers, contiguous row-major, 16-byte
 * aligned. q, o, dO, dq [Tq, Hq, 256] bf16; k, v [Tk, Hkv, 256] bf16; lse
 * [Tq, Hq] fp32. cu_seqlens_q, cu_seqlens_k [num_seqs + 1] int32, read only
 * on the device (each starts at 0, is nondecreasing and ends at Tq / Tk; a
 * violating array gives unspecified values with every kernel in bounds). The
 * caller owns every buffer and the library allocates nothing. Arguments are
 * validated on the host before anything is enqueued; all work is enqueued on
 * `stream` and nothing blocks the host. No floating-point atomics: results
 * are bitwise reproducible run to run.
 */
#ifndef KDA_ATTN_H_
#define KDA_ATTN_H_

#include "kda.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int64_t Tq, Tk;     /* packed query and key tokens, >= 0 (at most 2^30 each) */
  int32_t num_seqs;   /* segments, >= 1 */
  int32_t Hq, Hkv;    /* query and key heads; Hq a multiple of Hkv */
  int32_t D;          /* head dimension; this build serves 256 */
  float scale;        /* softmax scale, finite and > 0; usually 1/sqrt(D) */
} kda_attn_problem;

/* Forms of the key and value gradients written by kda_attn_bwd. */
enum {
  KDA_ATTN_DKV_BF16 = 0,    /* dk, dv [Tk, Hkv, 256] bf16, overwritten */
  KDA_ATTN_DKV_F32 = 1,     /* dk, dv [Tk, Hkv, 256] fp32 window gradients, overwritten */
  KDA_ATTN_DKV_F32_ADD = 2  /* dk, dv [dkv_dst_rows, Hkv, 256] fp32 destinations: key j's
                               sums are added to row dkv_row_map[j] (a value outside
                               [0, dkv_dst_rows) drops the key); the keys that share a
                               row are summed in ascending key order and the total added
                               once; rows no key names are left as they were */
};

/* Workspace bytes of a call: stage 0 the forward, stage 1 the backward in
 * form BF16 or F32, stage 2 the backward in form F32_ADD (which needs room
 * for the fp32 window gradients and the sorted row map; dkv_dst_rows is read
 * only here). Covers the segments' block tables and, for the backward, the
 * per-row <dO, o> sums. 0 for an invalid problem or stage. */
size_t kda_attn_workspace_bytes(const kda_attn_problem* p, int stage, int64_t dkv_dst_rows);

/* Forward: o, and the natural-log lse unless lse is NULL (the backward needs
 * it). */
kda_status kda_attn_fwd(const kda_attn_problem* p, const void* q, const void* k, const void* v,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* o,
                        float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Backward of L = sum <o, dO> from the forward's o and lse: dq (bf16,
 * overwritten) and the key-head sums dk, dv in form dkv_form (see above;
 * dkv_row_map [Tk] int32 on the device and dkv_dst_rows >= 0 are read only in
 * form F32_ADD). */
kda_status kda_attn_bwd(const kda_attn_problem* p, const void* q, const void* k, const void* v,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, const void* o,
                        const float* lse, const void* dO, void* dq, void* dk, void* dv,
                        int dkv_form, const int32_t* dkv_row_map, int64_t dkv_dst_rows,
                        void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KDA_ATTN_H_ */
