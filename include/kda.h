/* kda.h - C ABI of the MI355X (gfx950) chunked KDA training library.
 *
 * Kimi Delta Attention (KDA): per head h the state is S (dk x dv, fp32),
 * reset to zero at every packed document start, and for each token t
 *     S'  = Diag(exp(g_t)) S            (per-channel forget gate)
 *     u_t = v_t - S'^T k_t
 *     S   = S' + beta_t k_t u_t^T       (gated delta rule)
 *     o_t = scale * S^T q_t
 * The library computes this forward pass and the first-order backward of
 * L = sum <o, dO> in the chunked form (chunks of 64 tokens restarting at each
 * document start): gate cumsum, UT/WY triangular solve, intra-chunk products,
 * and an inter-chunk state scan (the per-chunk affine state map
 * S_out = M S_in + B).
 *
 * Sources: flashinfer PR #8909 "fix(cake_kda_det): gate-gradient accuracy of
 * the GLM intra stage", opening section (the deterministic single-device KDA
 * training package: gate form g or raw, Q/K L2 norm off or fused, backward
 * from the saved forward set or by replay with no saved set; bf16 q/k/v/beta,
 * fp32 gate, head dim 128; bitwise reproducible); flashinfer PR #7176
 * "perf(cake_kda): ... BF16x3 half-width transfer walk", opening section
 * (documents packed into one sequence; FP32 affine state summaries; BF16x3
 * split products); flashinfer PR #7774 "feat(cake_gqa_train)", description
 * and review (run-time lengths read only on the device, launch on the
 * caller's stream, rejection of head counts below one).
 *
 * Conventions
 *  - Every tensor pointer is a DEVICE pointer to contiguous row-major memory,
 *    16-byte aligned. T = packed tokens, H = heads, D = 128.
 *      q, k, v, o, dO, dq, dk, dv           [T, H, 128] bf16
 *      beta, dbeta                          [T, H]      bf16
 *      gate form g:   g, dg                 [T, H, 128] fp32 (log of the forget gate,
 *                                           g <= 0; a positive g gives unspecified
 *                                           values, with every kernel in bounds)
 *      gate form raw: a, da                 [T, H, 128] bf16
 *                     A_log, dA_log         [H]         fp32
 *                     dt_bias, ddt_bias     [H, 128]    fp32
 *      with g = -exp(A_log[h]) * softplus(a + dt_bias[h]).
 *      cu_seqlens                           [num_seqs+1] int32, cu[0] = 0,
 *                                           nondecreasing, cu[num_seqs] = T.
 *  - cu_seqlens is read only on the device; the host never synchronises. Its
 *    validity is a precondition (not checked): a violating array gives
 *    unspecified results but every kernel stays inside the buffers sized from
 *    T, H and num_seqs.
 *  - Ownership: the caller owns every buffer (inputs, outputs, the saved set
 *    and the workspace). The library allocates nothing and keeps no state
 *    between calls apart from its loaded code; calls are re-entrant. Calls
 *    that share a workspace or saved set must be ordered on one stream.
 *  - Outputs are overwritten, never accumulated. No output may overlap another
 *    output, an input, the saved set or the workspace: kda_bwd reads dv back
 *    after writing it (the per-chunk backward takes dR as the bf16 dv).
 *  - Errors: arguments are validated on the host before anything is
 *    enqueued; an invalid call returns a status and launches nothing. A
 *    launch failure returns KDA_ERR_DEVICE. kda_last_error() gives a
 *    thread-local message for the last failing call of the thread.
 *  - Stream: all work is enqueued on `stream` in order; nothing blocks the
 *    host. T == 0: kda_fwd launches nothing; kda_bwd in the raw gate form
 *    writes zeros to dA_log and ddt_bias (sums over no tokens) with one small
 *    fill kernel and launches nothing else.
 *  - Determinism: no floating-point atomics; results are bitwise identical
 *    run to run, and the replay backward is bitwise identical to the saved
 *    backward of the same inputs.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 1

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARGUMENT = 1,   /* bad scalar, null or misaligned pointer */
  KDA_ERR_UNSUPPORTED = 2,        /* a valid request this build does not serve: dk, dv != 128,
                                     H > 65535, or more than 2^29 (document, head) pairs */
  KDA_ERR_WORKSPACE_TOO_SMALL = 3,
  KDA_ERR_DEVICE = 4              /* a HIP call failed; see kda_last_error() */
} kda_status;

typedef enum { KDA_GATE_G = 0, KDA_GATE_RAW = 1 } kda_gate_form;

typedef struct {
  int64_t T;          /* packed tokens, >= 0 */
  int32_t H;          /* heads, >= 1 */
  int32_t num_seqs;   /* documents, >= 1 */
  int32_t dk, dv;     /* head dims; this build serves 128, 128 */
  int32_t gate;       /* kda_gate_form */
  int32_t l2norm;     /* 0: q, k used as given; 1: fused per-(token, head) L2 norm */
  float scale;        /* output scale, usually 1/sqrt(dk) */
  float l2_eps;       /* L2 norm: x * (sum x^2 + l2_eps)^(-1/2) */
} kda_problem;

/* Size in bytes of the saved forward set of a problem: what kda_fwd writes
 * when `saved` is non-NULL and what kda_bwd reads. Opaque to the caller;
 * reusable across calls of problems with the same T, H and num_seqs.
 * Defined by the saved backward path of the KDA training package (PR #8909,
 * opening section: the backward either uses the saved forward set or replays
 * the forward from a checkpoint). Returns 0 for an invalid problem. */
size_t kda_saved_bytes(const kda_problem* p);

/* Size in bytes of the scratch workspace a call needs. The caller allocates
 * it; a workspace may be reused by later calls ordered on the same stream
 * (workspace reuse across calls as in PR #7774's test list).
 *   backward = 0, replay = 0: kda_fwd with saved != NULL;
 *   backward = 0, replay = 1: kda_fwd with saved == NULL (the forward half of
 *                             a replay pair; it needs private room for the
 *                             per-chunk states);
 *   backward = 1, replay = 0: kda_bwd with saved != NULL;
 *   backward = 1, replay = 1: kda_bwd with saved == NULL.
 * Returns 0 for an invalid problem. */
size_t kda_workspace_bytes(const kda_problem* p, int backward, int replay);

/* Forward (PR #8909, opening section: the package's forward over the gate
 * forms g / raw and the optional fused Q/K L2 norm; PR #7176, opening
 * section: documents packed into one sequence, state reset at each document
 * start). Writes o, and the saved forward set when `saved` is non-NULL.
 * g_or_a is g (fp32) for KDA_GATE_G or a (bf16) for KDA_GATE_RAW; A_log and
 * dt_bias are read only for KDA_GATE_RAW (may be NULL otherwise).
 * workspace_bytes must be at least kda_workspace_bytes(p, 0, saved == NULL).
 * Errors: KDA_ERR_INVALID_ARGUMENT (bad scalar, NULL or misaligned pointer),
 * KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE_TOO_SMALL, all before any launch;
 * KDA_ERR_DEVICE if a launch fails. */
kda_status kda_fwd(const kda_problem* p, const void* q, const void* k, const void* v,
                   const void* beta, const void* g_or_a, const float* A_log,
                   const float* dt_bias, const int32_t* cu_seqlens, void* o, void* saved,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Backward of L = sum <o, dO> (PR #8909, opening section: the saved and
 * replay backward paths, and the gate gradients dg, dA_log and dt_bias that
 * its accuracy fix is about). With saved != NULL it reads the set written
 * by kda_fwd for the same inputs; with saved == NULL it first recomputes the
 * forward state from q, k, v, beta and the gate (replay; o is not written).
 * Writes dq, dk, dv, dbeta and, for KDA_GATE_G, dg_or_da = dg (fp32); for
 * KDA_GATE_RAW, dg_or_da = da (bf16), dA_log and ddt_bias. With the fused L2
 * norm, dq and dk are gradients with respect to the raw (unnormalised) q, k.
 * workspace_bytes must be at least kda_workspace_bytes(p, 1, saved == NULL).
 * Errors as for kda_fwd. */
kda_status kda_bwd(const kda_problem* p, const void* q, const void* k, const void* v,
                   const void* beta, const void* g_or_a, const float* A_log,
                   const float* dt_bias, const int32_t* cu_seqlens, const void* dO,
                   const void* saved, void* dq, void* dk, void* dv, void* dbeta,
                   void* dg_or_da, float* dA_log, float* ddt_bias, void* workspace,
                   size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): kda_fwd
 * with its workspace taken from a fixed scratch array that the library holds
 * on each GPU it runs on (KDA_NOALLOC_SCRATCH_BYTES per GPU, from module load
 * until the process ends) instead of a caller buffer. Inputs, o and the saved
 * set are the caller's, as for kda_fwd; results are identical to kda_fwd's.
 * It allocates nothing. A call whose workspace would exceed the scratch
 * (kda_workspace_bytes(p, 0, saved == NULL) > KDA_NOALLOC_SCRATCH_BYTES: a
 * forward without a saved set beyond a few hundred chunk-heads) returns
 * KDA_ERR_WORKSPACE_TOO_SMALL before any launch. Every call on one GPU uses
 * the same array: calls that overlap in time on one GPU (other streams,
 * other threads) race and must not be issued. */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)
kda_status kda_fwd_noalloc(const kda_problem* p, const void* q, const void* k, const void* v,
                           const void* beta, const void* g_or_a, const float* A_log,
                           const float* dt_bias, const int32_t* cu_seqlens, void* o,
                           void* saved, void* stream);

/* Instrumentation for callers that time the library's kernels (for example
 * with HIP events): when set, `hook` is called on the host immediately before
 * (end = 0) and after (end = 1) every kernel launch, with the kernel's name
 * and the stream it is enqueued on. Process-wide; set it while no other
 * thread is calling the library. NULL removes it. */
typedef void (*kda_launch_hook)(void* user, const char* kernel, int end, void* stream);
void kda_set_launch_hook(kda_launch_hook hook, void* user);

/* Error reporting (PR #7774's review: invalid requests such as a head count
 * below one are rejected with a clear validation error). */
const char* kda_status_string(kda_status s);
const char* kda_last_error(void);   /* thread-local; "" if none */
int kda_abi_version(void);          /* KDA_ABI_VERSION */

#ifdef __cplusplus
}
#endif
#endif /* KDA_H_ */
