/* kda_conv.h - C ABI of the width-4 causal conv1d + SiLU training op
 * (forward and backward) over packed documents, with a halo, for MI355X
 * (gfx950). It is the step of the KDA module forward in front of the state
 * passing: flashinfer PR #7176, measurement paragraph of the description (the
 * module forward is conv halo + conv + state passing) and the paragraph on the
 * family's other variants (the halo variant of the width-4 causal conv1d +
 * SiLU training backend). The pages print no formula; this library computes,
 * per channel c of a packed [T, D] input x with document starts s_d,
 *
 *     z[t, c] = b[c] + sum_{j=0..3} w[c, j] * xx(t - 3 + j, c),  y = z * sigmoid(z)
 *
 * where xx(u) = x[u] for u inside t's document; before the start of document
 * 0, the halo rows (the 3 tokens that precede x[0] in that document, oldest
 * first) when a halo is given; zero otherwise. w[c, 3] multiplies the current
 * token. The backward gives dx, dw, db and the halo's gradient dhalo (to be
 * added into the previous fragment's dx).
 *
 * Conventions (as kda.h): DEVICE pointers, contiguous row-major, 16-byte
 * aligned; x, y, dy, dx [T, D] bf16; halo, dhalo [3, D] bf16; w, dw [D, 4]
 * fp32; b, db [D] fp32; cu_seqlens [num_seqs + 1] int32, read only on the
 * device (cu[0] = 0, nondecreasing, cu[num_seqs] = T; a violating array gives
 * unspecified values with every kernel in bounds). The caller owns every
 * buffer; the library allocates nothing. Arguments are validated on the host
 * before anything is enqueued; all work is enqueued on `stream` and nothing
 * blocks the host. Outputs are overwritten. No floating-point atomics:
 * results are bitwise reproducible run to run.
 */
#ifndef KDA_CONV_H_
#define KDA_CONV_H_

#include "kda.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int64_t T;          /* packed tokens, >= 0 (at most 2^30) */
  int32_t D;          /* channels, a positive multiple of 8 */
  int32_t num_seqs;   /* documents, >= 1 */
  int32_t width;      /* conv width; this build serves 4 */
  int32_t has_bias;   /* 0: no b (and no db); 1: b [D] */
  int32_t has_halo;   /* 0: document 0 starts at x[0]; 1: halo [3, D] precedes it */
} kda_conv_problem;

/* Workspace bytes of a forward (backward = 0: none needed) or backward call
 * (backward = 1: fixed-order partial sums of dw and db). 0 for an invalid
 * problem. */
size_t kda_conv_workspace_bytes(const kda_conv_problem* p, int backward);

/* Forward: y = SiLU(causal conv of x with w, plus b). b and halo are read
 * when has_bias / has_halo (may be NULL otherwise). workspace may be NULL. */
kda_status kda_conv_silu_fwd(const kda_conv_problem* p, const void* x, const float* w,
                             const float* b, const void* halo, const int32_t* cu_seqlens,
                             void* y, void* workspace, size_t workspace_bytes, void* stream);

/* Backward of L = sum <y, dy>: dx (bf16), dw (fp32), db (fp32, when
 * has_bias), dhalo (bf16, when has_halo; its rows that see no token of
 * document 0 are zero). Needs kda_conv_workspace_bytes(p, 1) bytes. */
kda_status kda_conv_silu_bwd(const kda_conv_problem* p, const void* x, const float* w,
                             const float* b, const void* halo, const int32_t* cu_seqlens,
                             const void* dy, void* dx, float* dw, float* db, void* dhalo,
                             void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KDA_CONV_H_ */
