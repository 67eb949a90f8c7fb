/* kda_state.h - C ABI of one rank's share of a packed sequence split over
 * ranks (MI355X, gfx950).
 *
 * flashinfer PR #7176, opening section: the context-parallel variant splits
 * the packed sequence over the ranks of a group and passes the recurrent
 * state between ranks through FP32 affine state summaries, the state leaving
 * a fragment being S_out = M S_in + B, carried across fragment boundaries by
 * a transfer walk; its backward mirrors this with the gradient of the state.
 * The exchange between ranks (an all-gather of (M, B) over RCCL) is the
 * caller's. What one GPU runs for fragment r:
 *
 *   forward   (M_r, B_r) = kda_state_summary(fragment r, saved): s_final =
 *             M_r s_init + B_r, the prep left in the saved set. After the
 *             exchange, S_init(r) = M_{r-1} S_init(r-1) + B_{r-1} by
 *             kda_state_apply (S_init(0) = 0, and 0 wherever a fragment
 *             starts with a new document); then kda_fwd_state(fragment r,
 *             s_init = S_init(r), saved, KDA_FWD_PREP_DONE).
 *   backward  B'_r = kda_state_grad_summary(fragment r, dO, saved): ds_init =
 *             M_r^T ds_final + B'_r. After the exchange, dS_final(r) =
 *             M_{r+1}^T dS_final(r+1) + B'_{r+1} by kda_state_apply with
 *             transpose = 1 (zero for the last rank, and wherever the next
 *             fragment starts with a new document); then kda_bwd_state(
 *             fragment r, ds_final = dS_final(r)).
 *
 * The summaries run the forward's prep (once per fragment when the saved set
 * carries it to the forward) and one state chain per (document, head, column
 * tile) of only the documents they need, storing nothing per chunk; the
 * gradient summary reuses the saving forward's operand panels.
 *
 * States are fp32 [H, 128, 128] row-major: element (h, k, v) is row k (key
 * channel), column v (value channel) of head h's state, at (h*128 + k)*128 + v.
 * Document 0 of the fragment enters with s_init; the state leaving the last
 * document is s_final (an empty last document leaves the state it enters
 * with). All pointers are DEVICE pointers, 16-byte aligned; the other
 * arguments and their conventions are those of kda_fwd / kda_bwd (kda.h),
 * and kda_fwd_state / kda_bwd_state take the workspace sizes of kda_fwd /
 * kda_bwd. Errors as for kda_fwd: arguments are validated on the host before
 * anything is enqueued.
 */
#ifndef KDA_STATE_H_
#define KDA_STATE_H_

#include "kda.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Flags of kda_fwd_state. */
enum {
  KDA_FWD_PREP_DONE = 1  /* the saved set already holds this fragment's prep, written by
                            kda_state_summary with the same problem and inputs: it is not
                            run again (needs saved; other inputs give unspecified values) */
};

/* kda_fwd with document 0 entering from s_init (NULL: zero) and the state
 * leaving the last document written to s_final (NULL: not written). The
 * saved set, when given, holds the states of this run (s_init included).
 * flags: 0 or KDA_FWD_PREP_DONE. */
kda_status kda_fwd_state(const kda_problem* p, const void* q, const void* k, const void* v,
                         const void* beta, const void* g_or_a, const float* A_log,
                         const float* dt_bias, const int32_t* cu_seqlens, const float* s_init,
                         void* o, float* s_final, void* saved, int flags, void* workspace,
                         size_t workspace_bytes, void* stream);

/* kda_bwd of L = sum <o, dO> + <s_final, ds_final>: s_init is the forward's
 * (read only by a replay, saved == NULL); ds_final (NULL: zero) is the
 * gradient with respect to s_final; ds_init (NULL: not written) receives the
 * gradient with respect to s_init. */
kda_status kda_bwd_state(const kda_problem* p, const void* q, const void* k, const void* v,
                         const void* beta, const void* g_or_a, const float* A_log,
                         const float* dt_bias, const int32_t* cu_seqlens, const float* s_init,
                         const void* dO, const float* ds_final, const void* saved, void* dq,
                         void* dk, void* dv, void* dbeta, void* dg_or_da, float* dA_log,
                         float* ddt_bias, float* ds_init, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Workspace bytes of kda_state_summary and kda_state_grad_summary (0 for an
 * invalid problem). */
size_t kda_state_summary_workspace_bytes(const kda_problem* p);

/* The fragment's affine state map s_final = M s_init + B, M and B fp32
 * [H,128,128] (either NULL: not written). M is the identity when the
 * fragment has no tokens and zero when it has more than one document (its
 * last document starts from zero); else the product of its chunks' maps,
 * run from the identity with V = 0. B is s_final from a zero s_init. Both in
 * fp32 with the forward's operand precision. saved (NULL: the prep stays in
 * the workspace) receives the prep in the layout of kda_fwd's saved set (of
 * kda_saved_bytes(p) bytes), for a following kda_fwd_state with
 * KDA_FWD_PREP_DONE; the workspace then needs only the chunk table. */
kda_status kda_state_summary(const kda_problem* p, const void* q, const void* k, const void* v,
                             const void* beta, const void* g_or_a, const float* A_log,
                             const float* dt_bias, const int32_t* cu_seqlens, float* M, float* B,
                             void* saved, void* workspace, size_t workspace_bytes,
                             void* stream);

/* dB [H,128,128] fp32: the gradient with respect to s_init of L = sum <o,
 * dO> with a zero gradient of s_final, which is ds_init of kda_bwd_state with
 * ds_final = NULL (it does not depend on s_init). saved is the set of a
 * saving kda_fwd / kda_fwd_state of the same fragment (its operand panels are
 * read), or NULL to rebuild them in the workspace. */
kda_status kda_state_grad_summary(const kda_problem* p, const void* q, const void* k,
                                  const void* v, const void* beta, const void* g_or_a,
                                  const float* A_log, const float* dt_bias,
                                  const int32_t* cu_seqlens, const void* dO, const void* saved,
                                  float* dB, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* y = M x + B (transpose = 0) or M^T x + B (transpose = 1) for H heads of
 * [128,128] states, B NULL meaning zero: the transfer step, on bf16x3 split
 * MFMA products with fp32 accumulation (PR #7176, opening section). y may
 * alias x or B. */
kda_status kda_state_apply(int32_t H, const float* M, int transpose, const float* B,
                           const float* x, float* y, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KDA_STATE_H_ */
