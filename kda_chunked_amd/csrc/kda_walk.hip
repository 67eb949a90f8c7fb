// Transfer walks of the segment-parallel state scans.
//
// A document's chunks are cut into segments; the state map of a segment is
// affine, S_out = M S_in + B (flashinfer PR #7176, opening section: the
// FP32 affine state summaries and the transfer walk that carries the state
// across fragment boundaries as S_out = M * S_in + B, computed as a
// half-width BF16x3 split product with two workgroups per (segment, head),
// each covering half of the state's columns). Once every segment's M and B
// are known (forward scan, summary pass), the forward walk gives each
// segment's entering state; the reverse walk carries dS backwards through
// dS_in = M^T dS_out + B' (B' from the reverse scan's summary pass) and gives
// each segment's leaving dS. The finishing scan passes then run all segments
// in parallel.
//
// Products use the three-part split x = hi + mid + lo of each fp32 operand
// (hi = bf16(x), mid = bf16(x - hi), lo = bf16(x - hi - mid)) and the six
// terms down to order 2^-16 relative, lo*hi + mid*mid + hi*lo + mid*hi +
// hi*mid + hi*hi, added small first, with fp32 accumulation on the MFMA.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int WK_THREADS = 256;     // 4 waves, 16 state columns each
constexpr int WK_LD = HD + 8;       // rows of 272 bytes

struct WalkSmem {
  bf16 m[3][HD][WK_LD];             // M [r][c]: hi, mid, lo
  bf16 x[3][64][WK_LD];             // the half state, transposed [j][row]: hi, mid, lo
};

KDA_DEV void split3(float v, bf16& h, bf16& m, bf16& l) {
  h = f2bf(v);
  const float r1 = v - bf2f(h);
  m = f2bf(r1);
  l = f2bf(r1 - bf2f(m));
}

// M (128 x 128, tile order) of one segment and head into the three planes.
KDA_DEV void stage_m(WalkSmem& sm, const float* M) {
  for (int v = threadIdx.x; v < HD * HD / 4; v += WK_THREADS) {
    const int tile = v >> 6, ln = v & 63, rb = tile >> 3, cb = tile & 7;
    const f32x4 x = *reinterpret_cast<const f32x4*>(M + tile * 256 + 4 * ln);
    const int col = 16 * cb + (ln & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * rb + 4 * (ln >> 4) + i;
      split3(x[i], sm.m[0][row][col], sm.m[1][row][col], sm.m[2][row][col]);
    }
  }
}

// This wave's 16 columns of the half state (D layout, rows 16 m) into the
// transposed planes, rows 16 w .. 16 w + 15 of x.
KDA_DEV void stage_x(WalkSmem& sm, const f32x4 (&X)[8]) {
  const int l = lane_id(), w = wave_id();
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    bf16x4 h, md, lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16 a, b, c;
      split3(X[m][i], a, b, c);
      h[i] = a;
      md[i] = b;
      lo[i] = c;
    }
    const int j = 16 * w + (l & 15), c = 16 * m + 4 * (l >> 4);
    *reinterpret_cast<bf16x4*>(&sm.x[0][j][c]) = h;
    *reinterpret_cast<bf16x4*>(&sm.x[1][j][c]) = md;
    *reinterpret_cast<bf16x4*>(&sm.x[2][j][c]) = lo;
  }
}

// Rows 16 m + drow(i), column 16 cb + dcol() of head h's 128 x 128 state in
// the caller layout (row-major), as D-layout tiles; zero when x is null.
KDA_DEV void load_state(f32x4 (&X)[8], const float* x, int h, int cb) {
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      X[m][i] = x ? x[((int64_t)h * HD + 16 * m + drow(i)) * HD + 16 * cb + dcol()] : 0.f;
}

KDA_DEV void store_state(const f32x4 (&X)[8], float* x, int h, int cb) {
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) x[((int64_t)h * HD + 16 * m + drow(i)) * HD + 16 * cb + dcol()] = X[m][i];
}

// acc[m] += (M or M^T)[16 m .., :] X[:, this wave's columns], six split terms.
template <bool TRANS>
KDA_DEV void walk_product(const WalkSmem& sm, f32x4 (&acc)[8]) {
  const int w = wave_id();
#pragma unroll
  for (int k = 0; k < HD; k += 32) {
    bf16x8 b[3];
#pragma unroll
    for (int p = 0; p < 3; ++p) b[p] = frag(&sm.x[p][0][0], WK_LD, 16 * w, k);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      bf16x8 a[3];
#pragma unroll
      for (int p = 0; p < 3; ++p) a[p] = afrag<TRANS>(&sm.m[p][0][0], WK_LD, 16 * m, k);
      acc[m] = mfma16(a[2], b[0], acc[m]);
      acc[m] = mfma16(a[1], b[1], acc[m]);
      acc[m] = mfma16(a[0], b[2], acc[m]);
      acc[m] = mfma16(a[1], b[0], acc[m]);
      acc[m] = mfma16(a[0], b[1], acc[m]);
      acc[m] = mfma16(a[0], b[0], acc[m]);
    }
  }
}

// Block b: document and head (b >> 1), column half (b & 1). Documents with a
// single segment need no walk (their segment starts from zero and ends at
// the document end).
template <bool REV>
__global__ __launch_bounds__(WK_THREADS) void walk_kernel(Dims d, ChunkTable ct, SegWork sg) {
  __shared__ WalkSmem sm;
  const int half = blockIdx.x & 1, pair = blockIdx.x >> 1;
  const int doc = pair / d.H, h = pair % d.H;
  if (doc >= d.N) return;
  const int s0 = ld_const(ct.seg_doc0, doc), s1 = ld_const(ct.seg_doc0, doc + 1);
  if (s1 - s0 < 2) return;
  const int w = wave_id();
  const int cb = 4 * half + w;             // this wave's 16-column block of the state
  auto off = [&](int s) { return ((int64_t)s * d.H + h) * HD * HD; };
  f32x4 X[8];
  // the walk starts from zero, or from the caller's boundary state: the state
  // entering document 0 (forward) or the gradient leaving the last document
  const float* x0 = REV ? (doc == d.N - 1 ? sg.ds_final : nullptr) : (doc == 0 ? sg.s_init : nullptr);
  load_state(X, x0, h, cb);
  if (!REV) {
    // S entering segment s0 is zero (or s_init); S entering s + 1 = M_s S + B_s
    for (int s = s0; s < s1; ++s) {
      float* dst = sg.S0 + off(s);
#pragma unroll
      for (int m = 0; m < 8; ++m) *reinterpret_cast<f32x4*>(dst + tile_off(m, cb)) = X[m];
      if (s + 1 == s1) break;
      __syncthreads();                      // the previous step's reads of the planes are done
      stage_m(sm, sg.M + off(s));
      stage_x(sm, X);
#pragma unroll
      for (int m = 0; m < 8; ++m)
        X[m] = *reinterpret_cast<const f32x4*>(sg.B + off(s) + tile_off(m, cb));
      __syncthreads();
      walk_product<false>(sm, X);
    }
  } else {
    // dS leaving the last segment is zero (or ds_final); dS leaving s - 1 = M_s^T dS + B'_s
    for (int s = s1 - 1; s > s0; --s) {
      __syncthreads();
      stage_m(sm, sg.M + off(s));
      stage_x(sm, X);
#pragma unroll
      for (int m = 0; m < 8; ++m)
        X[m] = *reinterpret_cast<const f32x4*>(sg.Brev + off(s) + tile_off(m, cb));
      __syncthreads();
      walk_product<true>(sm, X);
      float* dst = sg.D0 + off(s - 1);
#pragma unroll
      for (int m = 0; m < 8; ++m) *reinterpret_cast<f32x4*>(dst + tile_off(m, cb)) = X[m];
    }
  }
}

// y = (M or M^T) x + B for the 128 x 128 states of H heads in the caller
// layout: the transfer step of a sequence split over ranks (flashinfer PR
// #7176, opening section: S_out = M S_in + B, and in the backward
// dS_in = M^T dS_out + B'), on the same six-term split products as the walks.
// Block b: head b >> 1, column half b & 1. Every block reads its columns of x
// and B before it writes those of y, so y may alias x or B.
template <bool TRANS>
__global__ __launch_bounds__(WK_THREADS) void state_apply_kernel(const float* M, const float* B,
                                                                 const float* x, float* y) {
  __shared__ WalkSmem sm;
  const int h = blockIdx.x >> 1, half = blockIdx.x & 1;
  const int cb = 4 * half + wave_id();
  for (int v = threadIdx.x; v < HD * HD / 4; v += WK_THREADS) {
    const int r = v >> 5, c4 = (v & 31) * 4;
    const f32x4 t = *reinterpret_cast<const f32x4*>(M + ((int64_t)h * HD + r) * HD + c4);
#pragma unroll
    for (int i = 0; i < 4; ++i) split3(t[i], sm.m[0][r][c4 + i], sm.m[1][r][c4 + i], sm.m[2][r][c4 + i]);
  }
  f32x4 X[8], acc[8];
  load_state(X, x, h, cb);
  load_state(acc, B, h, cb);
  stage_x(sm, X);
  __syncthreads();
  walk_product<TRANS>(sm, acc);
  store_state(acc, y, h, cb);
}

// Boundary-state fills: zero, identity, or a copy (zero from a null source).
__global__ __launch_bounds__(256) void fill_states_kernel(int64_t n, float* dst, const float* src,
                                                          int mode) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int r = (int)((e / HD) % HD), c = (int)(e % HD);
    dst[e] = mode == FILL_IDENTITY ? (r == c ? 1.f : 0.f) : (mode == FILL_COPY && src ? src[e] : 0.f);
  }
}

hipError_t launch_fill_states(int H, float* dst, const float* src, int mode, hipStream_t s) {
  const int64_t n = (int64_t)H * HD * HD;
  const int64_t b = (n + 255) / 256;
  hipLaunchKernelGGL(fill_states_kernel, dim3((unsigned)(b < 4096 ? b : 4096)), dim3(256), 0, s, n,
                     dst, src, mode);
  return hipGetLastError();
}

hipError_t launch_state_apply(int H, const float* M, int transpose, const float* B,
                              const float* x, float* y, hipStream_t s) {
  if (transpose)
    hipLaunchKernelGGL(state_apply_kernel<true>, dim3(2 * H), dim3(WK_THREADS), 0, s, M, B, x, y);
  else
    hipLaunchKernelGGL(state_apply_kernel<false>, dim3(2 * H), dim3(WK_THREADS), 0, s, M, B, x, y);
  return hipGetLastError();
}

hipError_t launch_walk(const Dims& d, const ChunkTable& ct, const SegWork& sg, int reverse,
                       hipStream_t s) {
  const dim3 grid(2 * d.N * d.H);
  if (reverse)
    hipLaunchKernelGGL(walk_kernel<true>, grid, dim3(WK_THREADS), 0, s, d, ct, sg);
  else
    hipLaunchKernelGGL(walk_kernel<false>, grid, dim3(WK_THREADS), 0, s, d, ct, sg);
  return hipGetLastError();
}

}  // namespace kda
