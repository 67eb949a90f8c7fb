// Internal interface between the host API (kda_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

// Records a printf-style message as the calling thread's kda_last_error()
// and returns s.
__attribute__((visibility("hidden"))) kda_status fail(kda_status s, const char* fmt, ...);

// Device-side chunk table built from cu_seqlens by the chunk-map kernel.
// Chunks are 64 tokens long and restart at every document start; chunk ids
// are assigned in document order. n_chunks_max = floor(T/64) + num_seqs is an
// upper bound on the number of chunks that the host can compute without
// reading cu_seqlens.
struct ChunkTable {
  int32_t* doc_c0;   // [N+1]: chunks of document d are [doc_c0[d], doc_c0[d+1])
  int32_t* tok;      // [n_chunks_max]: first token of the chunk
  int32_t* len;      // [n_chunks_max]: tokens in the chunk (1..64)
  // Segments: each document's chunks cut into runs of Dims::L chunks (one
  // segment per document when L = 0), numbered in document order. Segment s
  // of document d is its k-th, k = s - seg_doc0[d].
  int32_t* seg_doc0; // [N+1]: segments of document d are [seg_doc0[d], seg_doc0[d+1])
  int32_t* seg_doc;  // [n_segments_max]: document of segment s
};

// Per-chunk matrices and states (the saved forward set), all fp32. The gate
// cumsum G is not saved: the per-chunk backward rebuilds it from the gate input.
//
// S_in, R and U~ are stored per chunk-head in MFMA tile order: a 16 x 16 tile
// (row block rb, column block cb) is 256 contiguous floats at
// (rb * 8 + cb) * 256, and within it the element (4 (l / 16) + i, l % 16)
// sits at 4 l + i, i.e. each lane of the producing or consuming MFMA reads
// or writes its four values as one 16-byte vector. Rows past the chunk's end
// hold zeros.
struct SavedSet {
  float* S_in;   // [NC, H, 128 x 128] state before each chunk (tile order)
  float* Tm;     // [NC, H, 64, 64]  (I + Diag(beta) A_kk)^-1, zero above the diagonal
  float* Akk;    // [NC, H, 64, 64]  decayed k.k products, zero on and above the diagonal
  float* R;      // [NC, H, 64 x 128] V - (K*e^G) S_in (tile order)
  float* U;      // [NC, H, 64 x 128] U~ = Tb R (tile order)
  float* rq;     // [T, H]           L2 scalars (1 without the fused norm)
  float* rk;     // [T, H]
  void* panels;  // [NC, H, fwd_panel::ELEMS] bf16 operand panels (also the reverse scan's)
  float* Mseg;   // [NS, H, 128 x 128] homogeneous part of each segment's state map (L > 0)
};

// Segment-parallel scans (L > 0): the state map of a segment of chunks is
// affine, S_out = M S_in + B, and its reverse is dS_in = M^T dS_out + B'.
// fp32, tile order as SavedSet::S_in.
struct SegWork {
  float* M;      // [NS, H, 128 x 128] M of each segment (the saved set's Mseg)
  float* B;      // [NS, H, 128 x 128] B: the state after the segment from a zero state
  float* S0;     // [NS, H, 128 x 128] state entering each segment (forward walk)
  float* Brev;   // [NS, H, 128 x 128] B': dS at the segment start from a zero dS at its end
  float* D0;     // [NS, H, 128 x 128] dS at each segment's end (reverse walk)
  // Boundary states of the packed sequence, caller layout [H][128][128]
  // row-major (key row, value column), all nullable: the state entering
  // document 0, the state leaving the last document, the gradient with
  // respect to the latter, and the gradient with respect to the former.
  const float* s_init;
  float* s_final;
  const float* ds_final;
  float* ds_init;
  // The affine map of the whole sequence, s_final = M s_init + B (caller
  // layout, nullable): written by the forward scan in mode SCAN_MAP.
  float* map_M;
  float* map_B;
};
// Scan passes: per-chunk outputs from the walk's segment states, the segment
// summaries only, or (SCAN_MAP, whole documents, nothing per chunk stored)
// the summary of the whole sequence: forward map_M and map_B, reverse the
// gradient entering document 0 from a zero gradient leaving the sequence,
// written to ds_init.
enum : int { SCAN_FINISH = 0, SCAN_SUMMARY = 1, SCAN_MAP = 2 };

struct Dims {
  int64_t T;
  int H;
  int N;        // documents
  int NC;       // n_chunks_max
  int L;        // chunks per segment of the segment-parallel scans (0: whole documents)
  int NS;       // n_segments_max
  int raw;      // gate form raw
  int l2norm;
  float scale;
  float l2_eps;
};

struct Inputs {
  const void* q;
  const void* k;
  const void* v;
  const void* beta;
  const void* gate;   // g (fp32) or a (bf16)
  const float* A_log;
  const float* dt_bias;
  const int32_t* cu;
};

struct BwdOut {
  void* dq;
  void* dk;
  void* dv;
  void* dbeta;
  void* dgate;        // dg (fp32) or da (bf16)
  float* dA_log;
  float* ddt_bias;
};

struct BwdWork {
  float* dS;          // [NC, H, 128 x 128] gradient w.r.t. the state after each chunk (tile order)
  float* dU;          // [NC, H, 64 x 128] gradient w.r.t. U~ (tile order, as SavedSet::R)
  float* part_A;      // [NC, H]      raw form: per-chunk sum of dg*g
  float* part_dt;     // [NC, H, 128] raw form: per-chunk sum of dz
};

// Per chunk-head operand panels, written by the prep kernel as bf16 planes
// (hi = RNE(x), lo = RNE(x - hi)), row-major. The first CHAIN elements are
// what the sequential state scan needs; QD and AQ feed the output kernel; the
// reverse scan reads Ke^T, A_qk, Tb, Qd and -Kd transposed (LDS transpose
// loads), for which the lo planes of -Kd and Tb follow at the end (written only
// when a backward will use them). Offsets in bf16 elements.
namespace fwd_panel {
constexpr int KD = 0;                        // -Kd hi            [64][128]
constexpr int TB = KD + 64 * 128;            // Tb hi             [64][64]
constexpr int KE = TB + 64 * 64;             // Ke^T hi, lo       [2][128][64]
constexpr int GAM = KE + 2 * 128 * 64;       // e^(G_last), fp32  [128]
constexpr int CHAIN = GAM + 2 * 128;         // end of the scan's part
constexpr int QD = CHAIN;                    // scale Qd hi, lo   [2][64][128]
constexpr int AQ = QD + 2 * 64 * 128;        // scale A_qk hi, lo [2][64][64]
constexpr int KDL = AQ + 2 * 64 * 64;        // -Kd lo            [64][128]
constexpr int TBL = KDL + 64 * 128;          // Tb lo             [64][64]
constexpr int ELEMS = TBL + 64 * 64;         // 65792 bf16 elements per chunk-head
constexpr size_t BYTES = (size_t)ELEMS * 2;  // 131584, a multiple of 16
}  // namespace fwd_panel

// Blocks of `block` tokens per document (64: the chunks of the method).
hipError_t launch_chunk_map(const Dims& d, const int32_t* cu, const ChunkTable& ct,
                            hipStream_t s, int block = 64);
hipError_t launch_seg_map(const Dims& d, const ChunkTable& ct, hipStream_t s);
// H states of 128 x 128 (caller layout): FILL_ZERO, FILL_IDENTITY, or
// FILL_COPY of src (zero when src is null).
enum : int { FILL_ZERO = 0, FILL_IDENTITY = 1, FILL_COPY = 2 };
hipError_t launch_fill_states(int H, float* dst, const float* src, int mode, hipStream_t s);
// y = (M or M^T) x + B per head (B nullable), caller layout.
hipError_t launch_state_apply(int H, const float* M, int transpose, const float* B,
                              const float* x, float* y, hipStream_t s);
hipError_t launch_walk(const Dims& d, const ChunkTable& ct, const SegWork& sg, int reverse,
                       hipStream_t s);
hipError_t launch_fwd_prep(const Dims& d, const Inputs& in, const ChunkTable& ct,
                           const SavedSet& sv, int with_bwd, hipStream_t s);
hipError_t launch_fwd_scan(const Dims& d, const Inputs& in, const ChunkTable& ct,
                           const SavedSet& sv, const void* panels, int save_R,
                           const SegWork& sg, int mode, hipStream_t s);
hipError_t launch_fwd_out(const Dims& d, const ChunkTable& ct, const SavedSet& sv,
                          const void* panels, void* o, hipStream_t s);
hipError_t launch_bwd_scan(const Dims& d, const Inputs& in, const ChunkTable& ct,
                           const SavedSet& sv, const void* dO, void* dv,
                           const BwdWork& bw, const SegWork& sg, int mode, hipStream_t s);
hipError_t launch_bwd_intra(const Dims& d, const Inputs& in, const ChunkTable& ct,
                            const SavedSet& sv, const void* dO, const BwdOut& out,
                            const BwdWork& bw, hipStream_t s);
hipError_t launch_finalize(const Dims& d, const ChunkTable& ct, const BwdOut& out,
                           const BwdWork& bw, hipStream_t s);
// Raw form with T == 0: dA_log[H] and ddt_bias[H, 128] are sums over no tokens.
hipError_t launch_zero_params(const Dims& d, float* dA_log, float* ddt_bias, hipStream_t s);

}  // namespace kda
