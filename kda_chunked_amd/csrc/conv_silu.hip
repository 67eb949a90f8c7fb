// Width-4 causal conv1d + SiLU over packed documents, with a halo: forward
// and backward (the conv step in front of the KDA state passing; flashinfer
// PR #7176, description: module forward = conv halo + conv + state passing,
// and the halo variant of the width-4 causal conv1d + SiLU training backend).
//
//   z[t, c] = b[c] + sum_j w[c, j] xx(t - 3 + j, c),   y = z sigmoid(z)
//   dz = dy (s + z s (1 - s)),  dx[u] = sum_j w[j] dz[u + 3 - j] (same document),
//   dw[c, j] = sum_t dz[t] xx(t - 3 + j),  db[c] = sum_t dz[t]
//
// The op streams a [T, D] bf16 tensor once each way, so it is bound by HBM:
// lanes own VEC consecutive channels (8 forward, 4 backward: one 16- or
// 8-byte vector) and a run of tokens, keep the 3-token window in registers,
// and a wave moves 64 VEC channels of each token row. A workgroup is 4 waves
// on the same 64 VEC channels and 4 consecutive 64-token runs; the backward adds its 4 runs' dw and db partials in LDS in a fixed
// order and a second kernel adds the workgroup rows in order, so the sums are
// the same bits every run.
#include "kda_conv.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace conv {

constexpr int W = 4;          // conv width
constexpr int VEC_FWD = 8;    // channels per lane, forward
constexpr int VEC_BWD = 4;    // channels per lane, backward (half the registers of 8:
                              // four waves per SIMD keep twice the loads in flight)
constexpr int CG = 64;        // lanes per wave: channel groups of a workgroup
constexpr int SUB = 4;        // waves per workgroup: token runs
constexpr int RUN = 64;       // tokens per run
constexpr int ROWS = SUB * RUN;
constexpr int NP = W + 1;     // partial sums per channel: dw[0..3], db

template <int V>
KDA_DEV void loadv(const bf16* p, float* v) {
  typedef __bf16 vec __attribute__((ext_vector_type(V)));
  const vec a = *reinterpret_cast<const vec*>(p);
#pragma unroll
  for (int i = 0; i < V; ++i) v[i] = bf2f(a[i]);
}

template <int V>
KDA_DEV void storev(bf16* p, const float* v) {
  typedef __bf16 vec __attribute__((ext_vector_type(V)));
  vec a;
#pragma unroll
  for (int i = 0; i < V; ++i) a[i] = f2bf(v[i]);
  *reinterpret_cast<vec*>(p) = a;
}

KDA_DEV float sigm(float z) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-z * LOG2E));
}

// Document of token t: the last d with cu[d] <= t (documents before it end
// at or before t).
KDA_DEV int doc_of(const int32_t* cu, int N, int64_t t) {
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// The lane's view of its run: taps, bias, document bounds and the window
// xx(t0 - 3), xx(t0 - 2), xx(t0 - 1).
template <int VEC>
struct Lane {
  float wk[W][VEC], bb[VEC];
  int d;
  int64_t s, e;
};

template <int VEC>
KDA_DEV void setup(Lane<VEC>& L, float (&xm)[3][VEC], int64_t T, int D, int N, const bf16* x,
                   const float* w, const float* b, const bf16* halo, const int32_t* cu, int c0,
                   int64_t t0) {
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    const f32x4 t4 = *reinterpret_cast<const f32x4*>(w + (int64_t)(c0 + i) * W);
#pragma unroll
    for (int j = 0; j < W; ++j) L.wk[j][i] = t4[j];
    L.bb[i] = b ? b[c0 + i] : 0.f;
  }
  L.d = doc_of(cu, N, t0);
  // bounds clamped into [0, T] so that no access leaves the buffers
  const int64_t s = cu[L.d], e = cu[L.d + 1];
  L.s = s < 0 ? 0 : (s > t0 ? t0 : s);
  L.e = e <= t0 ? t0 + 1 : (e > T ? T : e);
#pragma unroll
  for (int k = 1; k <= 3; ++k) {
    const int64_t u = t0 - k;
    float* v = xm[3 - k];
    if (u >= L.s) {
      loadv<VEC>(x + u * D + c0, v);
    } else if (L.d == 0 && halo) {
      loadv<VEC>(halo + (3 + (u - L.s)) * D + c0, v);
    } else {
#pragma unroll
      for (int i = 0; i < VEC; ++i) v[i] = 0.f;
    }
  }
}

// Moves to the document that contains t (t reached the current one's end).
template <int VEC>
KDA_DEV void next_doc(Lane<VEC>& L, int64_t T, int N, const int32_t* cu, int64_t t) {
  while (L.d + 1 < N && cu[L.d + 1] <= t) ++L.d;
  L.s = t;
  const int64_t e = cu[L.d + 1];
  L.e = e <= t ? t + 1 : (e > T ? T : e);
}

template <int VEC>
__global__ __launch_bounds__(CG * SUB) void conv_fwd_kernel(int64_t T, int D, int N,
                                                            const bf16* __restrict__ x,
                                                            const float* __restrict__ w,
                                                            const float* __restrict__ b,
                                                            const bf16* __restrict__ halo,
                                                            const int32_t* __restrict__ cu,
                                                            bf16* __restrict__ y) {
  const int lane = threadIdx.x & (CG - 1), sub = threadIdx.x / CG;
  const int c0 = (blockIdx.x * CG + lane) * VEC;
  const int64_t t0 = (int64_t)blockIdx.y * ROWS + sub * RUN;
  if (c0 >= D || t0 >= T) return;
  const int64_t t1 = t0 + RUN < T ? t0 + RUN : T;
  Lane<VEC> L;
  float xm[3][VEC];
  setup(L, xm, T, D, N, x, w, b, halo, cu, c0, t0);
  for (int64_t t = t0; t < t1; ++t) {
    if (t >= L.e) {
      next_doc(L, T, N, cu, t);
#pragma unroll
      for (int k = 0; k < 3; ++k)
#pragma unroll
        for (int i = 0; i < VEC; ++i) xm[k][i] = 0.f;
    }
    float xt[VEC], yv[VEC];
    loadv<VEC>(x + t * D + c0, xt);
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const float z = L.bb[i] + L.wk[0][i] * xm[0][i] + L.wk[1][i] * xm[1][i] +
                      L.wk[2][i] * xm[2][i] + L.wk[3][i] * xt[i];
      yv[i] = z * sigm(z);
      xm[0][i] = xm[1][i];
      xm[1][i] = xm[2][i];
      xm[2][i] = xt[i];
    }
    storev<VEC>(y + t * D + c0, yv);
  }
}

// Backward of one run: dz for the run's tokens and up to 3 tokens past it
// (they reach back into the run through dx); dx of the run's tokens; the
// run's dw and db partials; dhalo from the run that starts at token 0.
template <int VEC>
__global__ __launch_bounds__(CG * SUB) void conv_bwd_kernel(
    int64_t T, int D, int N, const bf16* __restrict__ x, const float* __restrict__ w,
    const float* __restrict__ b, const bf16* __restrict__ halo, const int32_t* __restrict__ cu,
    const bf16* __restrict__ dy, bf16* __restrict__ dx, bf16* __restrict__ dhalo,
    float* __restrict__ part) {
  __shared__ float red[SUB][NP][CG * VEC];
  // dhalo sums of the run that starts at token 0, in LDS rather than in 12
  // registers that every other run would hold too (each lane owns its slots)
  __shared__ float dhs[3][CG * VEC];
  const int lane = threadIdx.x & (CG - 1), sub = threadIdx.x / CG;
  const int c0 = (blockIdx.x * CG + lane) * VEC;
  const int64_t t0 = (int64_t)blockIdx.y * ROWS + sub * RUN;
  const bool on = c0 < D && t0 < T;
  float pw[W][VEC], pb[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    pb[i] = 0.f;
#pragma unroll
    for (int j = 0; j < W; ++j) pw[j][i] = 0.f;
  }
  if (on) {
    const int64_t t1 = t0 + RUN < T ? t0 + RUN : T;
    const int64_t tend = t1 + 3 < T ? t1 + 3 : T;
    Lane<VEC> L;
    float xm[3][VEC];
    setup(L, xm, T, D, N, x, w, b, halo, cu, c0, t0);
    const bool with_halo = halo && dhalo && t0 == 0;
    if (with_halo) {
#pragma unroll
      for (int k = 0; k < 3; ++k)
#pragma unroll
        for (int i = 0; i < VEC; ++i) dhs[k][lane * VEC + i] = 0.f;
    }
    // acc[k]: dx of token t - 3 + k while token t is processed
    float acc[4][VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k][i] = 0.f;
    }
    // dx of token u, complete: stored when it belongs to this run and document
    auto put = [&](int64_t u, const float* v) {
      if (u >= t0 && u < t1 && u >= L.s) storev<VEC>(dx + u * D + c0, v);
    };
    // x and dy rows requested two tokens ahead (rows past tend repeat the
    // last one): the row a token uses was requested two iterations earlier
    typedef __bf16 vec __attribute__((ext_vector_type(VEC)));
    auto row_x = [&](int64_t u) {
      return *reinterpret_cast<const vec*>(x + (u < tend ? u : tend - 1) * D + c0);
    };
    auto row_dy = [&](int64_t u) {
      return *reinterpret_cast<const vec*>(dy + (u < tend ? u : tend - 1) * D + c0);
    };
    vec cx = row_x(t0), cg = row_dy(t0), nx = row_x(t0 + 1), ng = row_dy(t0 + 1);
    for (int64_t t = t0; t < tend; ++t) {
      const vec fx = row_x(t + 2), fg = row_dy(t + 2);
      if (t >= L.e) {
        // the document ended: tokens t-3 .. t-1 receive nothing more
#pragma unroll
        for (int k = 0; k < 3; ++k) put(t - 3 + k, acc[k]);
        if (t >= t1) break;     // past the run, later documents do not matter
        next_doc(L, T, N, cu, t);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
#pragma unroll
          for (int k = 0; k < 3; ++k) xm[k][i] = acc[k][i] = 0.f;
          acc[3][i] = 0.f;
        }
      }
      float xt[VEC], gy[VEC], dz[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) xt[i] = bf2f(cx[i]), gy[i] = bf2f(cg[i]);
      cx = nx, cg = ng, nx = fx, ng = fg;
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        const float z = L.bb[i] + L.wk[0][i] * xm[0][i] + L.wk[1][i] * xm[1][i] +
                        L.wk[2][i] * xm[2][i] + L.wk[3][i] * xt[i];
        const float s = sigm(z);
        dz[i] = gy[i] * (s + z * s * (1.f - s));
      }
      if (t < t1) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          pw[0][i] += dz[i] * xm[0][i];
          pw[1][i] += dz[i] * xm[1][i];
          pw[2][i] += dz[i] * xm[2][i];
          pw[3][i] += dz[i] * xt[i];
          pb[i] += dz[i];
        }
      }
      // token t - 3 + j receives w[j] dz[t] (inside the document), or the
      // halo row 3 + (t - 3 + j) - s before document 0
#pragma unroll
      for (int j = 0; j < W; ++j) {
        const int64_t u = t - 3 + j;
        if (u >= L.s) {
#pragma unroll
          for (int i = 0; i < VEC; ++i) acc[j][i] += L.wk[j][i] * dz[i];
        } else if (with_halo && L.d == 0) {
          const int r = (int)(3 + (u - L.s));
#pragma unroll
          for (int i = 0; i < VEC; ++i) dhs[r][lane * VEC + i] += L.wk[j][i] * dz[i];
        }
      }
      put(t - 3, acc[0]);
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        acc[0][i] = acc[1][i];
        acc[1][i] = acc[2][i];
        acc[2][i] = acc[3][i];
        acc[3][i] = 0.f;
        xm[0][i] = xm[1][i];
        xm[1][i] = xm[2][i];
        xm[2][i] = xt[i];
      }
      if (t + 1 == tend && tend == T) {
        // the packed sequence ends: the last tokens receive nothing more
#pragma unroll
        for (int k = 0; k < 3; ++k) put(t - 2 + k, acc[k]);
      }
    }
    if (with_halo) {
#pragma unroll
      for (int k = 0; k < 3; ++k) storev<VEC>(dhalo + (int64_t)k * D + c0, &dhs[k][lane * VEC]);
    }
  }
  // the workgroup's 4 runs added in a fixed order
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
#pragma unroll
    for (int j = 0; j < W; ++j) red[sub][j][lane * VEC + i] = pw[j][i];
    red[sub][W][lane * VEC + i] = pb[i];
  }
  __syncthreads();
  // NP * CG * VEC sums over the 4 runs, spread over the 256 threads
  const int cbase = blockIdx.x * CG * VEC;
  for (int e = threadIdx.x; e < NP * CG * VEC; e += CG * SUB) {
    const int k = e / (CG * VEC), cc = e % (CG * VEC);
    if (cbase + cc < D) {
      const float v = (red[0][k][cc] + red[1][k][cc]) + (red[2][k][cc] + red[3][k][cc]);
      part[((int64_t)blockIdx.y * NP + k) * D + cbase + cc] = v;
    }
  }
}

// dw[c, j] and db[c]: the workgroup rows' partials added in row order.
__global__ __launch_bounds__(256) void conv_reduce_kernel(int rows, int D, const float* part,
                                                          float* dw, float* db) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= D) return;
  float s[NP] = {0.f, 0.f, 0.f, 0.f, 0.f};
  for (int r = 0; r < rows; ++r)
#pragma unroll
    for (int k = 0; k < NP; ++k) s[k] += part[((int64_t)r * NP + k) * D + c];
#pragma unroll
  for (int j = 0; j < W; ++j) dw[(int64_t)c * W + j] = s[j];
  if (db) db[c] = s[W];
}

// T == 0: every gradient that is a sum over tokens is zero.
__global__ __launch_bounds__(256) void conv_zero_kernel(int D, float* dw, float* db,
                                                        bf16* dhalo) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= D) return;
#pragma unroll
  for (int j = 0; j < W; ++j) dw[(int64_t)c * W + j] = 0.f;
  if (db) db[c] = 0.f;
  if (dhalo)
    for (int k = 0; k < 3; ++k) dhalo[(int64_t)k * D + c] = f2bf(0.f);
}

int part_rows(int64_t T) { return (int)((T + ROWS - 1) / ROWS); }

}  // namespace conv
}  // namespace kda

namespace {

using kda::fail;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

kda_status check(const kda_conv_problem* p) {
  if (!p) return fail(KDA_ERR_INVALID_ARGUMENT, "problem is NULL");
  if (p->T < 0 || p->T > ((int64_t)1 << 30))
    return fail(KDA_ERR_INVALID_ARGUMENT, "T = %lld outside [0, 2^30]", (long long)p->T);
  if (p->D < 8 || p->D % 8 != 0)
    return fail(KDA_ERR_INVALID_ARGUMENT, "D = %d: need a positive multiple of 8 channels", p->D);
  if (p->num_seqs < 1 || p->num_seqs > (1 << 24))
    return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs = %d outside [1, 2^24]", p->num_seqs);
  if (p->width != 4) return fail(KDA_ERR_UNSUPPORTED, "width = %d: this build serves 4", p->width);
  if ((p->has_bias != 0 && p->has_bias != 1) || (p->has_halo != 0 && p->has_halo != 1))
    return fail(KDA_ERR_INVALID_ARGUMENT, "has_bias and has_halo must be 0 or 1");
  if ((int64_t)p->T * p->D > ((int64_t)1 << 40))
    return fail(KDA_ERR_UNSUPPORTED, "T * D exceeds 2^40 elements");
  return KDA_OK;
}

#define REQ(ptr, name)                                                                  \
  do {                                                                                  \
    if (!(ptr)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is NULL", name);              \
    if (!aligned16(ptr)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name); \
  } while (0)

size_t bwd_ws(const kda_conv_problem* p) {
  return (size_t)kda::conv::part_rows(p->T) * kda::conv::NP * p->D * sizeof(float);
}

dim3 grid_of(const kda_conv_problem* p, int vec) {
  return dim3((p->D / vec + kda::conv::CG - 1) / kda::conv::CG,
              (unsigned)kda::conv::part_rows(p->T));
}

}  // namespace

extern "C" {

size_t kda_conv_workspace_bytes(const kda_conv_problem* p, int backward) {
  if (check(p) != KDA_OK) return 0;
  return backward ? bwd_ws(p) : 0;
}

kda_status kda_conv_silu_fwd(const kda_conv_problem* p, const void* x, const float* w,
                             const float* b, const void* halo, const int32_t* cu_seqlens,
                             void* y, void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  kda_status st = check(p);
  if (st != KDA_OK) return st;
  if (p->T == 0) return KDA_OK;
  REQ(x, "x");
  REQ(w, "w");
  REQ(cu_seqlens, "cu_seqlens");
  REQ(y, "y");
  if (p->has_bias) REQ(b, "b");
  if (p->has_halo) REQ(halo, "halo");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(kda::conv::conv_fwd_kernel<kda::conv::VEC_FWD>,
                     grid_of(p, kda::conv::VEC_FWD), dim3(kda::conv::CG * kda::conv::SUB),
                     0, hs, p->T, p->D, p->num_seqs, static_cast<const kda::bf16*>(x), w,
                     p->has_bias ? b : nullptr,
                     p->has_halo ? static_cast<const kda::bf16*>(halo) : nullptr, cu_seqlens,
                     static_cast<kda::bf16*>(y));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(KDA_ERR_DEVICE, "conv forward launch failed: %s", hipGetErrorString(e));
  return KDA_OK;
}

kda_status kda_conv_silu_bwd(const kda_conv_problem* p, const void* x, const float* w,
                             const float* b, const void* halo, const int32_t* cu_seqlens,
                             const void* dy, void* dx, float* dw, float* db, void* dhalo,
                             void* workspace, size_t workspace_bytes, void* stream) {
  kda_status st = check(p);
  if (st != KDA_OK) return st;
  REQ(dw, "dw");
  if (p->has_bias) REQ(db, "db");
  if (p->has_halo) REQ(dhalo, "dhalo");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  float* dbp = p->has_bias ? db : nullptr;
  kda::bf16* dh = p->has_halo ? static_cast<kda::bf16*>(dhalo) : nullptr;
  if (p->T == 0) {
    hipLaunchKernelGGL(kda::conv::conv_zero_kernel, dim3((p->D + 255) / 256), dim3(256), 0, hs,
                       p->D, dw, dbp, dh);
  } else {
    REQ(x, "x");
    REQ(w, "w");
    REQ(cu_seqlens, "cu_seqlens");
    REQ(dy, "dy");
    REQ(dx, "dx");
    if (p->has_bias) REQ(b, "b");
    if (p->has_halo) REQ(halo, "halo");
    REQ(workspace, "workspace");
    const size_t need = bwd_ws(p);
    if (workspace_bytes < need)
      return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu",
                  workspace_bytes, need);
    float* part = static_cast<float*>(workspace);
    hipLaunchKernelGGL(kda::conv::conv_bwd_kernel<kda::conv::VEC_BWD>,
                       grid_of(p, kda::conv::VEC_BWD),
                       dim3(kda::conv::CG * kda::conv::SUB), 0, hs, p->T, p->D, p->num_seqs,
                       static_cast<const kda::bf16*>(x), w, p->has_bias ? b : nullptr,
                       p->has_halo ? static_cast<const kda::bf16*>(halo) : nullptr, cu_seqlens,
                       static_cast<const kda::bf16*>(dy), static_cast<kda::bf16*>(dx), dh, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
      return fail(KDA_ERR_DEVICE, "conv backward launch failed: %s", hipGetErrorString(e));
    hipLaunchKernelGGL(kda::conv::conv_reduce_kernel, dim3((p->D + 255) / 256), dim3(256), 0, hs,
                       kda::conv::part_rows(p->T), p->D, part, dw, dbp);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(KDA_ERR_DEVICE, "conv backward launch failed: %s", hipGetErrorString(e));
  return KDA_OK;
}

}  // extern "C"
