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
// Shared-memory layout of the prep kernel.
constexpr int GS_LD = HD + 4;     // fp32 row stride of G
constexpr int XS_LD = HD + 8;     // bf16 row stride of q, k and the K=128 panels
constexpr int AK_LD = CL + 4;     // fp32 row stride of 64x64 matrices

struct PrepSmem {
  float G[CL][GS_LD];
  bf16 qs[CL][XS_LD];
  bf16 ks[CL][XS_LD];
  float rq[CL], rk[CL], beta[CL];
  float rho[HD];
  float half_tot[HD];
  int calm[4];
  bf16 xk_hi[16][XS_LD], xk_lo[16][XS_LD];
  bf16 xq_hi[16][XS_LD], xq_lo[16][XS_LD];
  union {
    struct {
      bf16 y_hi[CL][XS_LD], y_lo[CL][XS_LD];
    } p;
    struct {
      float Tm[CL][AK_LD];
      float Z[16][17];
    } s;
  } u;
  float Akk[CL][AK_LD];
};

// Loads the chunk's gate, forms G = cumsum(g) in LDS (rows >= n hold G[n-1])
// and, when G_out is non-null, writes G for the chunk's tokens.
KDA_DEV void load_gate_cumsum(float (*Gs)[GS_LD], float* half_tot, const Dims& d, const Inputs& in,
                              int64_t t0, int n, int h, float* G_out) {
  const int t = threadIdx.x;
  for (int e = t; e < CL * HD; e += 256) {
    const int r = e / HD, c = e % HD;
    Gs[r][c] = r < n ? gate_value(in.gate, d.raw, in.A_log, in.dt_bias, t0 + r, h, d.H, c) : 0.f;
  }
  __syncthreads();
  // Two threads per channel: rows 0-31 and 32-63, then the upper half adds
  // the lower half's total (a fixed order, so every kernel that recomputes G
  // gets the same bits).
  const int c = t & (HD - 1), half = t >> 7;
  float run = 0.f;
  for (int r = 32 * half; r < 32 * half + 32; ++r) {
    run += Gs[r][c];
    Gs[r][c] = run;
  }
  if (half == 0) half_tot[c] = run;
  __syncthreads();
  if (half == 1) {
    const float base = half_tot[c];
    for (int r = 32; r < 64; ++r) Gs[r][c] += base;
  }
  __syncthreads();
  if (G_out) {
    for (int e = t; e < n * HD; e += 256) {
      const int r = e / HD, c2 = e % HD;
      G_out[((t0 + r) * d.H + h) * HD + c2] = Gs[r][c2];
    }
  }
}

__global__ __launch_bounds__(256) void fwd_prep_kernel(Dims d, Inputs in, ChunkTable ct,
                                                        float* __restrict__ G_out, SavedSet sv) {
  __shared__ PrepSmem sm;
  const int ci = blockIdx.x, h = blockIdx.y;
  if (ci >= ct.doc_c0[d.N]) return;
  const int64_t t0 = ct.tok[ci];
  const int n = ct.len[ci];
  const int t = threadIdx.x, w = wave_id(), l = lane_id();
  const int64_t ch = (int64_t)ci * d.H + h;
  const bf16* q = reinterpret_cast<const bf16*>(in.q);
  const bf16* k = reinterpret_cast<const bf16*>(in.k);
  const bf16* beta = reinterpret_cast<const bf16*>(in.beta);

  // 1. q, k rows (zero padded), beta, L2 scalars.
  for (int e = t; e < CL * (HD / 8); e += 256) {
    const int r = e / (HD / 8), c8 = (e % (HD / 8)) * 8;
    bf16x8 qv, kv;
    if (r < n) {
      qv = *reinterpret_cast<const bf16x8*>(q + ((t0 + r) * d.H + h) * HD + c8);
      kv = *reinterpret_cast<const bf16x8*>(k + ((t0 + r) * d.H + h) * HD + c8);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[i] = kv[i] = f2bf(0.f);
    }
    *reinterpret_cast<bf16x8*>(&sm.qs[r][c8]) = qv;
    *reinterpret_cast<bf16x8*>(&sm.ks[r][c8]) = kv;
  }
  for (int e = t; e < CL * AK_LD; e += 256) (&sm.Akk[0][0])[e] = 0.f;
  if (t < CL) sm.beta[t] = t < n ? bf2f(beta[(t0 + t) * d.H + h]) : 0.f;
  __syncthreads();
  {
    // four threads per row, 32 channels each
    const int r = t >> 2, part = t & 3;
    float sq = 0.f, sk = 0.f;
    for (int c = 32 * part; c < 32 * part + 32; ++c) {
      const float a = bf2f(sm.qs[r][c]), b = bf2f(sm.ks[r][c]);
      sq += a * a;
      sk += b * b;
    }
    sq += __shfl_xor(sq, 1);
    sk += __shfl_xor(sk, 1);
    sq += __shfl_xor(sq, 2);
    sk += __shfl_xor(sk, 2);
    if (part == 0) {
      const float a = d.l2norm ? 1.f / sqrtf(sq + d.l2_eps) : 1.f;
      const float b = d.l2norm ? 1.f / sqrtf(sk + d.l2_eps) : 1.f;
      sm.rq[r] = a;
      sm.rk[r] = b;
      if (r < n) {
        sv.rq[(t0 + r) * d.H + h] = a;
        sv.rk[(t0 + r) * d.H + h] = b;
      }
    }
  }

  // 2. Gate cumsum.
  load_gate_cumsum(sm.G, sm.half_tot, d, in, t0, n, h, G_out);

  // 3. Calm flags: decay span of each 16-row block, per channel.
  if (t < 4) sm.calm[t] = 1;
  __syncthreads();
  if (t < HD) {
    for (int I = 0; I < 4; ++I) {
      const float ref = I == 0 ? 0.f : sm.G[16 * I - 1][t];
      if (ref - sm.G[16 * I + 15][t] > CALM_SPAN) sm.calm[I] = 0;
    }
  }
  __syncthreads();

  const Panel XK{&sm.xk_hi[0][0], &sm.xk_lo[0][0], XS_LD};
  const Panel XQ{&sm.xq_hi[0][0], &sm.xq_lo[0][0], XS_LD};
  const Panel Y{&sm.u.p.y_hi[0][0], &sm.u.p.y_lo[0][0], XS_LD};
  float* Aqk_g = sv.Aqk + ch * CL * CL;

  // 4. Off-diagonal and calm diagonal tiles on MFMA, one row block at a time.
  for (int I = 0; I < 4; ++I) {
    if (t < HD) sm.rho[t] = I == 0 ? 0.f : sm.G[16 * I - 1][t];
    __syncthreads();
    const int calm = sm.calm[I];
    const int ny = 16 * I + 16;
    // X rows of block I (q and k), 8 channels per task.
    for (int e = t; e < 16 * (HD / 8); e += 256) {
      const int rl = e / (HD / 8), c8 = (e % (HD / 8)) * 8;
      const int r = 16 * I + rl;
      float xk[8], xq[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float f = fexp(sm.G[r][c8 + j] - sm.rho[c8 + j]);
        xk[j] = bf2f(sm.ks[r][c8 + j]) * sm.rk[r] * f;
        xq[j] = bf2f(sm.qs[r][c8 + j]) * sm.rq[r] * f;
      }
      put8(XK, rl, c8, xk);
      put8(XQ, rl, c8, xq);
    }
    // Y rows 0 .. 16I+15 (block I's own rows only when calm).
    for (int e = t; e < ny * (HD / 8); e += 256) {
      const int i = e / (HD / 8), c8 = (e % (HD / 8)) * 8;
      float y[8];
      const bool on = i < 16 * I || calm;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        y[j] = on ? bf2f(sm.ks[i][c8 + j]) * sm.rk[i] * fexp(sm.rho[c8 + j] - sm.G[i][c8 + j]) : 0.f;
      put8(Y, i, c8, y);
    }
    __syncthreads();
    // tile-products: (matrix, J) for J = 0..I; wave w takes every 4th.
    for (int p = w; p < 2 * (I + 1); p += 4) {
      const int J = p >> 1, isq = p & 1;
      if (J == I && !calm) continue;
      f32x4 acc = zero4();
      mma_k<SPLIT_AB, HD>(acc, isq ? XQ : XK, 0, Y, 16 * J);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int r = 16 * I + drow(i4), i = 16 * J + dcol();
        if (isq) {
          Aqk_g[r * CL + i] = (i <= r) ? acc[i4] : 0.f;
        } else {
          sm.Akk[r][i] = (i < r) ? acc[i4] : 0.f;
        }
      }
    }
    // zero the strictly-upper tiles of A_qk for this row block
    for (int e = t; e < 16 * (CL - ny); e += 256) {
      const int rl = e / (CL - ny), i = ny + e % (CL - ny);
      Aqk_g[(16 * I + rl) * CL + i] = 0.f;
    }
    __syncthreads();
  }

  // 5. Diagonal tiles of blocks whose decay span is too wide: exact fp32 sums,
  //    one (r, i) entry per task over the 4 x 256 entries of the diagonal tiles.
  for (int p = t; p < 4 * 256; p += 256) {
    const int I = p >> 8;
    if (sm.calm[I]) continue;
    const int r = 16 * I + ((p >> 4) & 15), i = 16 * I + (p & 15);
    if (i > r) {
      Aqk_g[r * CL + i] = 0.f;
      continue;
    }
    float skk = 0.f, sqk = 0.f;
    for (int c = 0; c < HD; ++c) {
      const float e = fexp(sm.G[r][c] - sm.G[i][c]) * bf2f(sm.ks[i][c]);
      skk += bf2f(sm.ks[r][c]) * e;
      sqk += bf2f(sm.qs[r][c]) * e;
    }
    Aqk_g[r * CL + i] = sqk * sm.rq[r] * sm.rk[i];
    if (i < r) sm.Akk[r][i] = skk * sm.rk[r] * sm.rk[i];
  }
  __syncthreads();

  // 6. T = (I + Diag(beta) A_kk)^-1 by 16x16 blocks, fp32.
  float (*Tm)[AK_LD] = sm.u.s.Tm;
  for (int e = t; e < CL * AK_LD; e += 256) (&Tm[0][0])[e] = 0.f;
  __syncthreads();
  if (l < 16) {
    // wave w inverts diagonal block w; lane = column j
    const int I = w, j = l;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = (r == j) ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) s -= sm.beta[16 * I + r] * sm.Akk[16 * I + r][16 * I + i] * x[i];
      x[r] = s;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Tm[16 * I + r][16 * I + j] = x[r];
  }
  __syncthreads();
  for (int dist = 1; dist < 4; ++dist) {
    for (int J = 0; J + dist < 4; ++J) {
      const int I = J + dist;
      const int r = t >> 4, j = t & 15;
      // Z = sum_{m in blocks J..I-1} X[I-row r][m] T[m][J-col j]
      float z = 0.f;
      for (int m = 16 * J; m < 16 * I; ++m)
        z += sm.beta[16 * I + r] * sm.Akk[16 * I + r][m] * Tm[m][16 * J + j];
      sm.u.s.Z[r][j] = z;
      __syncthreads();
      float s = 0.f;
      for (int m = 0; m < 16; ++m) s += Tm[16 * I + r][16 * I + m] * sm.u.s.Z[m][j];
      Tm[16 * I + r][16 * J + j] = -s;
      __syncthreads();
    }
  }
  float* Tg = sv.Tm + ch * CL * CL;
  float* Akk_g = sv.Akk + ch * CL * CL;
  for (int e = t; e < CL * CL; e += 256) {
    const int r = e / CL, i = e % CL;
    Tg[e] = Tm[r][i];
    Akk_g[e] = sm.Akk[r][i];
  }
}

hipError_t launch_fwd_prep(const Dims& d, const Inputs& in, const ChunkTable& ct, float* G,
                           const SavedSet& sv, hipStream_t s) {
  hipLaunchKernelGGL(fwd_prep_kernel, dim3(d.NC, d.H), dim3(256), 0, s, d, in, ct, G, sv);
  return hipGetLastError();
}

}  // namespace kda
