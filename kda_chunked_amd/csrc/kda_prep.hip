// Chunk table and the per-chunk forward preparation of the KDA chunked form.
//
// Per (chunk, head), with G the chunk-local inclusive cumsum of the log gate g
// (the gated delta rule of flashinfer PR #8909's KDA training package, opening
// section; chunks restart at each packed document as in PR #7176, opening
// section):
//   A_kk[r,i] = sum_c k_r[c] k_i[c] e^(G_r[c] - G_i[c])   (i < r)
//   A_qk[r,i] = sum_c q_r[c] k_i[c] e^(G_r[c] - G_i[c])   (i <= r)
//   T = (I + Diag(beta) A_kk)^-1                          (UT/WY solve)
//
// Fast-decay safety. e^(G_r - G_i) is formed from two factors that never
// overflow: rows of block I (16 rows) use the reference rho_I = G at the row
// before the block, X_r = x_r e^(G_r - rho_I) <= 1 and, for columns i before
// the block, Y_i = k_i e^(rho_I - G_i) <= 1. For columns inside the block the
// second factor exceeds 1; it is used only when the block's own decay span is
// at most CALM_SPAN in every channel, otherwise that diagonal tile is summed
// element by element in fp32.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr float CALM_SPAN = 40.f;

#ifndef KDA_SPLIT_P1
#define KDA_SPLIT_P1 SPLIT_AB    // A_kk = X_k Y^T, A_qk = X_q Y^T
#endif

__global__ __launch_bounds__(256) void chunk_map_kernel(const int32_t* __restrict__ cu, int N,
                                                        int64_t T, int NC, ChunkTable ct) {
  __shared__ int32_t scan[256];
  const int t = threadIdx.x;
  int carry = 0;
  for (int base = 0; base < N; base += 256) {
    const int d = base + t;
    int a = 0, b = 0, cnt = 0;
    if (d < N) {
      int64_t ca = cu[d], cb = cu[d + 1];
      ca = ca < 0 ? 0 : (ca > T ? T : ca);
      cb = cb < ca ? ca : (cb > T ? T : cb);
      a = (int)ca;
      b = (int)cb;
      cnt = (b - a + CL - 1) / CL;
    }
    scan[t] = cnt;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int v = t >= off ? scan[t - off] : 0;
      __syncthreads();
      scan[t] += v;
      __syncthreads();
    }
    const int c0 = carry + scan[t] - cnt;
    const int total = scan[255];
    if (d < N) {
      ct.doc_c0[d] = min(c0, NC);
      for (int c = 0; c < cnt && c0 + c < NC; ++c) {
        const int tok = a + CL * c;
        ct.tok[c0 + c] = tok;
        ct.len[c0 + c] = min(CL, b - tok);
      }
    }
    carry += total;
    __syncthreads();
  }
  if (t == 0) ct.doc_c0[N] = min(carry, NC);
}

hipError_t launch_chunk_map(const Dims& d, const int32_t* cu, const ChunkTable& ct,
                            hipStream_t s) {
  hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(256), 0, s, cu, d.N, d.T, d.NC, ct);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The prep kernel: 512 threads (8 waves). Thread t owns row rA = t >> 3 and
// channels cA .. cA+15 (cA = 16 (t & 7)) of every 64 x 128 chunk quantity.
constexpr int NT_PREP = 512;
constexpr int GS_LD = HD + 1;     // fp32 row stride of G (scalar accesses only)
constexpr int XS_LD = HD + 8;     // bf16 row stride of the K = 128 panels
constexpr int F_LD = CL + 1;      // fp32 64 x 64 matrices

struct PrepSmem {
  float G[CL][GS_LD];
  float qtot[4][HD];
  float nrm[2][8][CL];
  float rq[CL], rk[CL], beta[CL];
  float rho[4][HD];
  int calm_blk[4];
  int calm_chunk;
  union {
    struct {                                   // single reference: Kd, Qd, Y = k^ e^-G
      bf16 xk_hi[CL][XS_LD], xk_lo[CL][XS_LD];
      bf16 xq_hi[CL][XS_LD], xq_lo[CL][XS_LD];
      bf16 y_hi[CL][XS_LD], y_lo[CL][XS_LD];
    } a;
    struct {                                   // one reference per 16-row block
      bf16 xk_hi[16][XS_LD], xk_lo[16][XS_LD];
      bf16 xq_hi[16][XS_LD], xq_lo[16][XS_LD];
      bf16 y_hi[CL][XS_LD], y_lo[CL][XS_LD];
      bf16 qs[CL][XS_LD], ks[CL][XS_LD];       // raw q, k for the exact diagonal sums
    } b;
    struct {
      float Tm[CL][F_LD];
      float Z[3][16][17];
    } s;
  } u;
  float Akk[CL][F_LD];
};

__global__ __launch_bounds__(NT_PREP) void fwd_prep_kernel(Dims d, Inputs in, ChunkTable ct,
                                                            float* __restrict__ G_out,
                                                            SavedSet sv) {
  __shared__ PrepSmem sm;
  const int ci = blockIdx.x, h = blockIdx.y;
  if (ci >= ct.doc_c0[d.N]) return;
  const int64_t t0 = ct.tok[ci];
  const int n = ct.len[ci];
  const int t = threadIdx.x, w = wave_id(), l = lane_id();
  const int H = d.H;
  const int64_t ch = (int64_t)ci * H + h;
  const bf16* q = reinterpret_cast<const bf16*>(in.q);
  const bf16* k = reinterpret_cast<const bf16*>(in.k);
  const bf16* beta = reinterpret_cast<const bf16*>(in.beta);
  const int rA = t >> 3, cA = 16 * (t & 7);
  const bool okA = rA < n;
  const int64_t baseA = ((t0 + (okA ? rA : n - 1)) * H + h) * HD + cA;

  // ---- 1. loads (all issued before use): q, k, gate of this thread's 16 elements
  bf16x8 q0 = *reinterpret_cast<const bf16x8*>(q + baseA);
  bf16x8 q1 = *reinterpret_cast<const bf16x8*>(q + baseA + 8);
  bf16x8 k0 = *reinterpret_cast<const bf16x8*>(k + baseA);
  bf16x8 k1 = *reinterpret_cast<const bf16x8*>(k + baseA + 8);
  float g[16];
  if (!d.raw) {
    const float* gp = reinterpret_cast<const float*>(in.gate) + baseA;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(gp + 4 * j);
#pragma unroll
      for (int u = 0; u < 4; ++u) g[4 * j + u] = x[u];
    }
  } else {
    const bf16* ap = reinterpret_cast<const bf16*>(in.gate) + baseA;
    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(ap);
    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(ap + 8);
    const float ea = __expf(in.A_log[h]);
#pragma unroll
    for (int j = 0; j < 16; ++j)
      g[j] = -ea * softplus(bf2f(j < 8 ? a0[j] : a1[j - 8]) + in.dt_bias[h * HD + cA + j]);
  }
  if (t < CL) sm.beta[t] = t < n ? bf2f(beta[(t0 + (t < n ? t : n - 1)) * H + h]) : 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) sm.G[rA][cA + j] = okA ? g[j] : 0.f;
  // L2 row sums: partial over this thread's 16 channels
  {
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float a = bf2f(j < 8 ? q0[j] : q1[j - 8]), b = bf2f(j < 8 ? k0[j] : k1[j - 8]);
      sq += a * a;
      sk += b * b;
    }
    sm.nrm[0][t & 7][rA] = sq;
    sm.nrm[1][t & 7][rA] = sk;
  }
  __syncthreads();

  // ---- 2. chunk-local cumsum of g: four threads per channel (16 rows each)
  {
    const int c = t & 127, qr = t >> 7;
    float run = 0.f;
    for (int r = 16 * qr; r < 16 * qr + 16; ++r) {
      run += sm.G[r][c];
      sm.G[r][c] = run;
    }
    sm.qtot[qr][c] = run;
    if (t < CL) {
      float a = 0.f, b = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        a += sm.nrm[0][j][t];
        b += sm.nrm[1][j][t];
      }
      const float rq = d.l2norm ? 1.f / sqrtf(a + d.l2_eps) : 1.f;
      const float rk = d.l2norm ? 1.f / sqrtf(b + d.l2_eps) : 1.f;
      sm.rq[t] = t < n ? rq : 0.f;
      sm.rk[t] = t < n ? rk : 0.f;
      if (t < n) {
        sv.rq[(t0 + t) * H + h] = rq;
        sv.rk[(t0 + t) * H + h] = rk;
      }
    }
    __syncthreads();
    float carry = 0.f;
    for (int j = 0; j < qr; ++j) carry += sm.qtot[j][c];
    if (qr > 0)
      for (int r = 16 * qr; r < 16 * qr + 16; ++r) sm.G[r][c] += carry;
  }
  if (t < 4) sm.calm_blk[t] = 1;
  if (t == 4) sm.calm_chunk = 1;
  __syncthreads();
  // this thread's G (rows >= n hold G[n-1] because their g is 0)
  float Gv[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) Gv[j] = sm.G[rA][cA + j];
  if (okA) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<f32x4*>(G_out + baseA + 4 * j) =
          f32x4{Gv[4 * j], Gv[4 * j + 1], Gv[4 * j + 2], Gv[4 * j + 3]};
  }
  if (t < HD) {
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      const float ref = I == 0 ? 0.f : sm.G[16 * I - 1][t];
      sm.rho[I][t] = ref;
      if (ref - sm.G[16 * I + 15][t] > CALM_SPAN) sm.calm_blk[I] = 0;
    }
    if (-sm.G[CL - 1][t] > CALM_SPAN) sm.calm_chunk = 0;
  }
  __syncthreads();

  const float rqA = sm.rq[rA], rkA = sm.rk[rA];
  float* Aqk_g = sv.Aqk + ch * CL * CL;
  const int rb = w & 3, isq = w >> 2;         // MFMA role: row block rb of A_kk (isq = 0) or A_qk
  if (sm.calm_chunk) {
    // ---- 3a. single reference at the chunk start: A = X Y^T with X = x^ e^G, Y = k^ e^-G
    const Panel XK{&sm.u.a.xk_hi[0][0], &sm.u.a.xk_lo[0][0], XS_LD};
    const Panel XQ{&sm.u.a.xq_hi[0][0], &sm.u.a.xq_lo[0][0], XS_LD};
    const Panel Y{&sm.u.a.y_hi[0][0], &sm.u.a.y_lo[0][0], XS_LD};
    float xk[16], xq[16], y[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float e1 = fexp(Gv[j]);
      const float kh = bf2f(j < 8 ? k0[j] : k1[j - 8]) * rkA;
      const float qh = bf2f(j < 8 ? q0[j] : q1[j - 8]) * rqA;
      xk[j] = kh * e1;
      xq[j] = qh * e1;
      y[j] = kh * fexp(-Gv[j]);
    }
    put8(XK, rA, cA, xk);
    put8(XK, rA, cA + 8, xk + 8);
    put8(XQ, rA, cA, xq);
    put8(XQ, rA, cA + 8, xq + 8);
    put8(Y, rA, cA, y);
    put8(Y, rA, cA + 8, y + 8);
    __syncthreads();
    f32x4 acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = zero4();
    mma_row<KDA_SPLIT_P1, 4>(acc, isq ? XQ : XK, 16 * rb, Y, 0, 0, HD);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int r = 16 * rb + drow(i4), i = 16 * nt + dcol();
        if (isq)
          Aqk_g[r * CL + i] = (i <= r) ? acc[nt][i4] : 0.f;
        else
          sm.Akk[r][i] = (i < r) ? acc[nt][i4] : 0.f;
      }
    __syncthreads();
  } else {
    // ---- 3b. one reference per 16-row block; exact sums for wide diagonal blocks
    const Panel XK{&sm.u.b.xk_hi[0][0], &sm.u.b.xk_lo[0][0], XS_LD};
    const Panel XQ{&sm.u.b.xq_hi[0][0], &sm.u.b.xq_lo[0][0], XS_LD};
    const Panel Y{&sm.u.b.y_hi[0][0], &sm.u.b.y_lo[0][0], XS_LD};
    *reinterpret_cast<bf16x8*>(&sm.u.b.qs[rA][cA]) = q0;
    *reinterpret_cast<bf16x8*>(&sm.u.b.qs[rA][cA + 8]) = q1;
    *reinterpret_cast<bf16x8*>(&sm.u.b.ks[rA][cA]) = k0;
    *reinterpret_cast<bf16x8*>(&sm.u.b.ks[rA][cA + 8]) = k1;
    for (int I = 0; I < 4; ++I) {
      const int calm = sm.calm_blk[I];
      const int bA = rA >> 4;
      float y[16];
      const bool on = bA < I || (bA == I && calm);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float kh = bf2f(j < 8 ? k0[j] : k1[j - 8]) * rkA;
        y[j] = on ? kh * fexp(sm.rho[I][cA + j] - Gv[j]) : 0.f;
      }
      put8(Y, rA, cA, y);
      put8(Y, rA, cA + 8, y + 8);
      if (bA == I) {
        float xk[16], xq[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float e1 = fexp(Gv[j] - sm.rho[I][cA + j]);
          xk[j] = bf2f(j < 8 ? k0[j] : k1[j - 8]) * rkA * e1;
          xq[j] = bf2f(j < 8 ? q0[j] : q1[j - 8]) * rqA * e1;
        }
        put8(XK, rA & 15, cA, xk);
        put8(XK, rA & 15, cA + 8, xk + 8);
        put8(XQ, rA & 15, cA, xq);
        put8(XQ, rA & 15, cA + 8, xq + 8);
      }
      __syncthreads();
      // tile-products (matrix, J) for J = 0..I, one per wave
      {
        const int J = w >> 1, pq = w & 1;
        if (J <= I) {
          f32x4 acc = zero4();
          if (J < I || calm) mma_k<KDA_SPLIT_P1, HD>(acc, pq ? XQ : XK, 0, Y, 16 * J);
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int r = 16 * I + drow(i4), i = 16 * J + dcol();
            if (pq)
              Aqk_g[r * CL + i] = (i <= r) ? acc[i4] : 0.f;
            else
              sm.Akk[r][i] = (i < r) ? acc[i4] : 0.f;
          }
        }
        // zero the strictly-upper tiles of A_qk and A_kk for this row block
        for (int e = t; e < 16 * (CL - 16 * (I + 1)); e += NT_PREP) {
          const int rl = e / (CL - 16 * (I + 1)), i = 16 * (I + 1) + e % (CL - 16 * (I + 1));
          Aqk_g[(16 * I + rl) * CL + i] = 0.f;
          sm.Akk[16 * I + rl][i] = 0.f;
        }
      }
      __syncthreads();
    }
    // exact fp32 sums on the diagonal tiles of blocks whose span is too wide
    for (int p = t; p < 4 * 256; p += NT_PREP) {
      const int I = p >> 8;
      if (sm.calm_blk[I]) continue;
      const int r = 16 * I + ((p >> 4) & 15), i = 16 * I + (p & 15);
      if (i > r) continue;
      float skk = 0.f, sqk = 0.f;
      for (int c = 0; c < HD; ++c) {
        const float e = fexp(sm.G[r][c] - sm.G[i][c]) * bf2f(sm.u.b.ks[i][c]);
        skk += bf2f(sm.u.b.ks[r][c]) * e;
        sqk += bf2f(sm.u.b.qs[r][c]) * e;
      }
      Aqk_g[r * CL + i] = sqk * sm.rq[r] * sm.rk[i];
      if (i < r) sm.Akk[r][i] = skk * sm.rk[r] * sm.rk[i];
    }
    __syncthreads();
  }

  // ---- 4. T = (I + Diag(beta) A_kk)^-1 by 16x16 blocks, fp32
  float (*Tm)[F_LD] = sm.u.s.Tm;
  for (int e = t; e < CL * F_LD; e += NT_PREP) (&Tm[0][0])[e] = 0.f;
  __syncthreads();
  if (w < 4 && l < 16) {
    // wave w inverts diagonal block w; lane = column j
    const int I = w, j = l;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s2 = (r == j) ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) s2 -= sm.beta[16 * I + r] * sm.Akk[16 * I + r][16 * I + i] * x[i];
      x[r] = s2;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Tm[16 * I + r][16 * I + j] = x[r];
  }
  __syncthreads();
  for (int dist = 1; dist < 4; ++dist) {
    // the (4 - dist) blocks of this distance in parallel, 256 threads each
    const int nb = 4 - dist;
    const int bsel = t >> 8, r = (t >> 4) & 15, j = t & 15;
    for (int J0 = 0; J0 < nb; J0 += 2) {
      const int J = J0 + bsel;
      const int I = J + dist;
      if (J < nb) {
        float z = 0.f;
        for (int m = 16 * J; m < 16 * I; ++m)
          z += sm.beta[16 * I + r] * sm.Akk[16 * I + r][m] * Tm[m][16 * J + j];
        sm.u.s.Z[bsel][r][j] = z;
      }
      __syncthreads();
      if (J < nb) {
        float s2 = 0.f;
        for (int m = 0; m < 16; ++m) s2 += Tm[16 * I + r][16 * I + m] * sm.u.s.Z[bsel][m][j];
        Tm[16 * I + r][16 * J + j] = -s2;
      }
      __syncthreads();
    }
  }
  float* Tg = sv.Tm + ch * CL * CL;
  float* Akk_g = sv.Akk + ch * CL * CL;
  {
    const int r = t >> 3, i8 = 8 * (t & 7);
    *reinterpret_cast<f32x4*>(Tg + r * CL + i8) = f32x4{Tm[r][i8], Tm[r][i8 + 1], Tm[r][i8 + 2], Tm[r][i8 + 3]};
    *reinterpret_cast<f32x4*>(Tg + r * CL + i8 + 4) =
        f32x4{Tm[r][i8 + 4], Tm[r][i8 + 5], Tm[r][i8 + 6], Tm[r][i8 + 7]};
    *reinterpret_cast<f32x4*>(Akk_g + r * CL + i8) =
        f32x4{sm.Akk[r][i8], sm.Akk[r][i8 + 1], sm.Akk[r][i8 + 2], sm.Akk[r][i8 + 3]};
    *reinterpret_cast<f32x4*>(Akk_g + r * CL + i8 + 4) =
        f32x4{sm.Akk[r][i8 + 4], sm.Akk[r][i8 + 5], sm.Akk[r][i8 + 6], sm.Akk[r][i8 + 7]};
  }
}

hipError_t launch_fwd_prep(const Dims& d, const Inputs& in, const ChunkTable& ct, float* G,
                           const SavedSet& sv, hipStream_t s) {
  hipLaunchKernelGGL(fwd_prep_kernel, dim3(d.NC, d.H), dim3(NT_PREP), 0, s, d, in, ct, G, sv);
  return hipGetLastError();
}

}  // namespace kda
