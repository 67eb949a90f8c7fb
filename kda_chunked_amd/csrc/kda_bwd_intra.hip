// Per-chunk backward of the KDA chunked form (the "GLM intra" stage of
// flashinfer PR #8909, opening section and commit notes) plus the parameter
// reduction of the raw gate.
//
// Given the saved state S_in, the state gradient dS_out and dU~ (both from the
// reverse scan), one workgroup per (chunk, head) forms
//   U~ = Tb R,  dR = Tb^T dU~                      (Tb = T Diag(beta))
//   dQd = scale dO S_in^T,  dKd = -dR S_in^T,  dKe = U~ dS_out^T
//   dA_qk = scale dO U~^T (i <= r),  dTb = dU~ R^T (i <= r)
//   dT = dTb Diag(beta),  dX = -T^T dT T^T (i < r),  dA_kk = Diag(beta) dX
//   dbeta_i = sum_r dTb[r,i] T[r,i] + sum_i' dX[i,i'] A_kk[i,i']
// then pushes dA_qk, dA_kk through the decayed products (same fast-decay-safe
// references as the forward), accumulates dq, dk and dG (the gradient of the
// chunk-local cumsum G) per element, and finishes with
//   dg_j = sum_{r >= j} dG_r   (reverse cumsum inside the chunk)
// and the chain rules of the fused L2 norm and of the raw gate
//   g = -exp(A_log) softplus(a + dt_bias).
// Each pair term of dG enters dG_r with + and dG_i with - from products on the
// same rounded operands (the diagonal pair rule of PR #8909's accuracy fix).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int K1_LD = HD + 8;
constexpr int K2_LD = CL + 8;
constexpr int X_LD = 32 + 8;
constexpr int GS_LD = HD + 4;
constexpr int AK_LD = CL + 4;
constexpr float CALM_SPAN_B = 40.f;

struct BwdIntraSmem {
  union {
    struct {
      bf16 tb_hi[CL][K2_LD], tb_lo[CL][K2_LD];     // Tb   [r][i]
      bf16 tbt_hi[CL][K2_LD], tbt_lo[CL][K2_LD];   // Tb^T [i][r]
      bf16 rt_hi[HD][K2_LD], rt_lo[HD][K2_LD];     // R^T  [j][i]
      bf16 dut_hi[HD][K2_LD], dut_lo[HD][K2_LD];   // dU~^T [j][r]
    } p1;
    struct {
      bf16 s_hi[HD][K1_LD], s_lo[HD][K1_LD];       // S_in [c][j], then dS_out [c][j]
      bf16 a_hi[CL][K1_LD], a_lo[CL][K1_LD];       // dR [r][j], then U~ [r][j]
      bf16 do_hi[CL][K1_LD];                       // dO [r][j]
    } p2;
    struct {
      bf16 du_hi[CL][K1_LD], du_lo[CL][K1_LD];     // dU~ [r][j]
      bf16 r_hi[CL][K1_LD], r_lo[CL][K1_LD];       // R [i][j]
    } p4;
    struct {
      float T[CL][AK_LD], Akk[CL][AK_LD], dT[CL][AK_LD], tmp[CL][AK_LD];
    } p5;
    struct {
      float G[CL][GS_LD];
      bf16 yt_hi[HD][K2_LD], yt_lo[HD][K2_LD];     // Y^T [c][i]
      bf16 xt_hi[HD][X_LD], xt_lo[HD][X_LD];       // [Xq ; Xk]^T [c][32]
      bf16 dq_hi[16][K2_LD], dq_lo[16][K2_LD];     // dA_qk rows of block I [r][i]
      bf16 dk_hi[16][K2_LD], dk_lo[16][K2_LD];     // dA_kk rows of block I
      bf16 dat_hi[CL][X_LD], dat_lo[CL][X_LD];     // [dA_qk^T | dA_kk^T] [i][32]
      float rho[HD];
    } p6;
    struct {
      float dG[CL][GS_LD];
      float red[HD];
    } p7;
  } u;
  float dAqk[CL][AK_LD];
  float dAkk[CL][AK_LD];
  float beta[CL], rq[CL], rk[CL], db[CL];
  float GL[HD], gam[HD], dGL[HD];
  float dGLw[4][HD];
  int calm[4];
};

__global__ __launch_bounds__(256) void bwd_intra_kernel(Dims d, Inputs in, ChunkTable ct,
                                                         const float* __restrict__ G,
                                                         SavedSet sv,
                                                         const bf16* __restrict__ dO,
                                                         BwdOut out, BwdWork bw) {
  __shared__ BwdIntraSmem sm;
  const int ci = blockIdx.x, h = blockIdx.y;
  if (ci >= ct.doc_c0[d.N]) return;
  const int64_t t0 = ct.tok[ci];
  const int n = ct.len[ci];
  const int t = threadIdx.x, w = wave_id(), l = lane_id();
  const int64_t ch = (int64_t)ci * d.H + h;
  const int H = d.H;
  const bf16* q = reinterpret_cast<const bf16*>(in.q);
  const bf16* k = reinterpret_cast<const bf16*>(in.k);
  const bf16* beta = reinterpret_cast<const bf16*>(in.beta);
  const float* Tg = sv.Tm + ch * CL * CL;
  const float* Akk_g = sv.Akk + ch * CL * CL;

  // element (r, c) of this lane's accumulators: r = 16w + drow(i), c = 16nt + dcol()
  f32x4 adq[8], adk[8], adG[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) adq[nt] = adk[nt] = adG[nt] = zero4();

  auto rowidx = [&](int r) -> int64_t { return (t0 + r) * H + h; };

  if (t < CL) {
    const bool ok = t < n;
    sm.beta[t] = ok ? bf2f(beta[rowidx(t)]) : 0.f;
    sm.rq[t] = ok ? sv.rq[rowidx(t)] : 0.f;
    sm.rk[t] = ok ? sv.rk[rowidx(t)] : 0.f;
  } else if (t < CL + HD) {
    const int c = t - CL;
    const float gl = G[rowidx(n - 1) * HD + c];
    sm.GL[c] = gl;
    sm.gam[c] = fexp(gl);
  }
  for (int e = t; e < CL * AK_LD; e += 256) {
    (&sm.dAqk[0][0])[e] = 0.f;
    (&sm.dAkk[0][0])[e] = 0.f;
  }
  __syncthreads();

  // ------------------------------------------------ P1: U~ = Tb R, dR = Tb^T dU~
  f32x4 U[8], dR[8];
  {
    const Panel TB{&sm.u.p1.tb_hi[0][0], &sm.u.p1.tb_lo[0][0], K2_LD};
    const Panel TBT{&sm.u.p1.tbt_hi[0][0], &sm.u.p1.tbt_lo[0][0], K2_LD};
    const Panel RT{&sm.u.p1.rt_hi[0][0], &sm.u.p1.rt_lo[0][0], K2_LD};
    const Panel DUT{&sm.u.p1.dut_hi[0][0], &sm.u.p1.dut_lo[0][0], K2_LD};
    for (int e = t; e < CL * (CL / 8); e += 256) {
      const int r = e >> 3, i8 = (e & 7) * 8;
      float tb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) tb[j] = Tg[r * CL + i8 + j] * sm.beta[i8 + j];
      put8(TB, r, i8, tb);
    }
    for (int e = t; e < CL * (CL / 8); e += 256) {
      const int i = e & (CL - 1), r8 = (e >> 6) * 8;
      float tb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) tb[j] = Tg[(r8 + j) * CL + i] * sm.beta[i];
      put8(TBT, i, r8, tb);
    }
    for (int e = t; e < HD * (CL / 8); e += 256) {
      const int j = e & (HD - 1), r8 = (e >> 7) * 8;
      float rv[8], du[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int r = r8 + jj;
        rv[jj] = r < n ? sv.R[rowidx(r) * HD + j] : 0.f;
        du[jj] = r < n ? bw.dU[rowidx(r) * HD + j] : 0.f;
      }
      put8(RT, j, r8, rv);
      put8(DUT, j, r8, du);
    }
    __syncthreads();
    const int kend = ((16 * w + 16 + 31) / 32) * 32;
    const int kbeg = (16 * w / 32) * 32;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      U[nt] = zero4();
      dR[nt] = zero4();
      mma<SPLIT_AB>(U[nt], TB, 16 * w, RT, 16 * nt, 0, kend);
      mma<SPLIT_AB>(dR[nt], TBT, 16 * w, DUT, 16 * nt, kbeg, CL);
    }
    __syncthreads();
  }

  // ------------------------------------------------ P2: dQd and dKd against S_in
  const Panel SP{&sm.u.p2.s_hi[0][0], &sm.u.p2.s_lo[0][0], K1_LD};
  const Panel AP{&sm.u.p2.a_hi[0][0], &sm.u.p2.a_lo[0][0], K1_LD};
  const Panel DOP{&sm.u.p2.do_hi[0][0], nullptr, K1_LD};
  {
    const float* Sg = sv.S_in + ch * HD * HD;
    for (int e = t; e < HD * (HD / 8); e += 256) {
      const int c = e >> 4, j8 = (e & 15) * 8;
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(Sg + c * HD + j8);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(Sg + c * HD + j8 + 4);
      const float x[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      put8(SP, c, j8, x);
    }
    for (int e = t; e < CL * (HD / 8); e += 256) {
      const int r = e >> 4, j8 = (e & 15) * 8;
      bf16x8 x;
      if (r < n) {
        x = *reinterpret_cast<const bf16x8*>(dO + rowidx(r) * HD + j8);
      } else {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) x[jj] = f2bf(0.f);
      }
      *reinterpret_cast<bf16x8*>(&sm.u.p2.do_hi[r][j8]) = x;
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) store_tile_n(dR[nt], AP, 16 * w, 16 * nt);
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      f32x4 a = zero4(), b = zero4();
      mma_k<SPLIT_B, HD>(a, DOP, 16 * w, SP, 16 * nt);
      mma_k<SPLIT_AB, HD>(b, AP, 16 * w, SP, 16 * nt);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + drow(i), c = 16 * nt + dcol();
        if (r < n) {
          const int64_t idx = rowidx(r) * HD + c;
          const float e1 = fexp(G[idx]);
          const float qh = bf2f(q[idx]) * sm.rq[r], kh = bf2f(k[idx]) * sm.rk[r];
          const float p = d.scale * a[i] * e1;
          const float p2 = -b[i] * e1;
          adq[nt][i] += p;
          adk[nt][i] += p2;
          adG[nt][i] += p * qh + p2 * kh;
        }
      }
    }
    __syncthreads();
  }

  // ------------------------------------------------ P3: dKe, dA_qk, dgamma
  {
    const float* dSg = bw.dS + ch * HD * HD;
    for (int e = t; e < HD * (HD / 8); e += 256) {
      const int c = e >> 4, j8 = (e & 15) * 8;
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(dSg + c * HD + j8);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(dSg + c * HD + j8 + 4);
      const float x[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      put8(SP, c, j8, x);
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) store_tile_n(U[nt], AP, 16 * w, 16 * nt);
    __syncthreads();
    float colp[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      f32x4 a = zero4();
      mma_k<SPLIT_AB, HD>(a, AP, 16 * w, SP, 16 * nt);
      colp[nt] = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + drow(i), c = 16 * nt + dcol();
        if (r < n) {
          const int64_t idx = rowidx(r) * HD + c;
          const float kh = bf2f(k[idx]) * sm.rk[r];
          const float p3 = a[i] * fexp(sm.GL[c] - G[idx]);
          adk[nt][i] += p3;
          adG[nt][i] -= p3 * kh;
          colp[nt] += p3 * kh;
        }
      }
    }
    // column sums of the Ke term -> dG at the chunk's last row
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      float s = colp[nt];
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      if (l < 16) sm.dGLw[w][16 * nt + l] = s;
    }
    // dA_qk = scale dO U~^T, lower triangle including the diagonal
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      f32x4 a = zero4();
      mma_k<SPLIT_B, HD>(a, DOP, 16 * w, AP, 16 * nt);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + drow(i), c = 16 * nt + dcol();
        sm.dAqk[r][c] = (c <= r) ? d.scale * a[i] : 0.f;
      }
    }
    __syncthreads();
    // dgamma[c] = sum_j dS_out[c][j] S_in[c][j]; dG_last += dgamma * gamma
    {
      const float* Sg = sv.S_in + ch * HD * HD;
      const int c = t >> 1, half = t & 1;
      float s = 0.f;
      for (int j = 64 * half; j < 64 * half + 64; ++j) s += dSg[c * HD + j] * Sg[c * HD + j];
      s += __shfl_xor(s, 1);
      if (half == 0)
        sm.dGL[c] = s * sm.gam[c] + ((sm.dGLw[0][c] + sm.dGLw[1][c]) + (sm.dGLw[2][c] + sm.dGLw[3][c]));
    }
    __syncthreads();
  }

  // ------------------------------------------------ P4: dTb = dU~ R^T
  f32x4 dTb[4];
  {
    const Panel DU{&sm.u.p4.du_hi[0][0], &sm.u.p4.du_lo[0][0], K1_LD};
    const Panel RP{&sm.u.p4.r_hi[0][0], &sm.u.p4.r_lo[0][0], K1_LD};
    for (int e = t; e < CL * (HD / 8); e += 256) {
      const int r = e >> 4, j8 = (e & 15) * 8;
      float a[8], b[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        a[jj] = r < n ? bw.dU[rowidx(r) * HD + j8 + jj] : 0.f;
        b[jj] = r < n ? sv.R[rowidx(r) * HD + j8 + jj] : 0.f;
      }
      put8(DU, r, j8, a);
      put8(RP, r, j8, b);
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      dTb[nt] = zero4();
      mma_k<SPLIT_AB, HD>(dTb[nt], DU, 16 * w, RP, 16 * nt);
    }
    __syncthreads();
  }

  // ------------------------------------------------ P5: WY / UT backward (fp32)
  {
    float (*Tm)[AK_LD] = sm.u.p5.T;
    float (*Ak)[AK_LD] = sm.u.p5.Akk;
    float (*dT)[AK_LD] = sm.u.p5.dT;
    float (*tmp)[AK_LD] = sm.u.p5.tmp;
    for (int e = t; e < CL * CL; e += 256) {
      const int r = e >> 6, i = e & 63;
      Tm[r][i] = Tg[e];
      Ak[r][i] = Akk_g[e];
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + drow(i), c = 16 * nt + dcol();
        dT[r][c] = (c <= r) ? dTb[nt][i] : 0.f;
      }
    __syncthreads();
    if (t < CL) {
      // dbeta from Tb = T Diag(beta): column sums, fixed order
      float s = 0.f;
      for (int r = t; r < CL; ++r) s += dT[r][t] * Tm[r][t];
      sm.db[t] = s;
    }
    __syncthreads();
    for (int e = t; e < CL * CL; e += 256) {
      const int r = e >> 6, m = e & 63;
      dT[r][m] *= sm.beta[m];
    }
    __syncthreads();
    // tmp = dT T^T : tmp[r][i] = sum_{m <= min(r, i)} dT[r][m] T[i][m]
    for (int e = t; e < CL * CL; e += 256) {
      const int r = e >> 6, i = e & 63;
      const int mmax = min(r, i);
      float s = 0.f;
      for (int m = 0; m <= mmax; ++m) s += dT[r][m] * Tm[i][m];
      tmp[r][i] = s;
    }
    __syncthreads();
    {
      // dX[r][i] = -sum_{m >= r} T[m][r] tmp[m][i]  (i < r); four threads per row
      const int r = t >> 2, part = t & 3;
      float dbr = 0.f;
      for (int i = 16 * part; i < 16 * part + 16; ++i) {
        if (i >= r) break;
        float s = 0.f;
        for (int m = r; m < CL; ++m) s += Tm[m][r] * tmp[m][i];
        const float dx = -s;
        sm.dAkk[r][i] = sm.beta[r] * dx;
        dbr += dx * Ak[r][i];
      }
      dbr += __shfl_xor(dbr, 1);
      dbr += __shfl_xor(dbr, 2);
      if (part == 0) sm.db[r] += dbr;
    }
    __syncthreads();
  }

  // ------------------------------------------------ P6: decayed-product backward
  {
    float (*Gs)[GS_LD] = sm.u.p6.G;
    for (int e = t; e < CL * HD; e += 256) {
      const int r = e >> 7, c = e & 127;
      Gs[r][c] = r < n ? G[rowidx(r) * HD + c] : sm.GL[c];
    }
    if (t < 4) sm.calm[t] = 1;
    __syncthreads();
    if (t < HD) {
      for (int I = 0; I < 4; ++I) {
        const float ref = I == 0 ? 0.f : Gs[16 * I - 1][t];
        if (ref - Gs[16 * I + 15][t] > CALM_SPAN_B) sm.calm[I] = 0;
      }
    }
    const Panel YT{&sm.u.p6.yt_hi[0][0], &sm.u.p6.yt_lo[0][0], K2_LD};
    const Panel XT{&sm.u.p6.xt_hi[0][0], &sm.u.p6.xt_lo[0][0], X_LD};
    const Panel DQ{&sm.u.p6.dq_hi[0][0], &sm.u.p6.dq_lo[0][0], K2_LD};
    const Panel DK{&sm.u.p6.dk_hi[0][0], &sm.u.p6.dk_lo[0][0], K2_LD};
    const Panel DAT{&sm.u.p6.dat_hi[0][0], &sm.u.p6.dat_lo[0][0], X_LD};
    float* rho = sm.u.p6.rho;
    for (int I = 0; I < 4; ++I) {
      __syncthreads();
      if (t < HD) rho[t] = I == 0 ? 0.f : Gs[16 * I - 1][t];
      __syncthreads();
      const int calm = sm.calm[I];
      const int ny = 16 * I + 16;           // columns i of this row block
      const int nyk = ((ny + 31) / 32) * 32;
      // Y^T [c][i] = k^_i e^(rho - G_i), zero for i >= ny and for block I when not calm
      for (int e = t; e < HD * (CL / 8); e += 256) {
        const int c = e & (HD - 1), i8 = (e >> 7) * 8;
        float y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = i8 + j;
          const bool on = i < 16 * I || (i < ny && calm);
          y[j] = (on && i < n) ? bf2f(k[rowidx(i) * HD + c]) * sm.rk[i] * fexp(rho[c] - Gs[i][c]) : 0.f;
        }
        put8(YT, c, i8, y);
      }
      // X^T [c][rr] (q) and [c][16 + rr] (k) for rows of block I
      for (int e = t; e < HD * 4; e += 256) {
        const int c = e & (HD - 1), part = e >> 7;   // part: 0,1 -> q rows 0-7, 8-15; 2,3 -> k
        const int isk = part >> 1, rr0 = (part & 1) * 8;
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = 16 * I + rr0 + j;
          float v = 0.f;
          if (r < n) {
            const int64_t idx = rowidx(r) * HD + c;
            v = isk ? bf2f(k[idx]) * sm.rk[r] : bf2f(q[idx]) * sm.rq[r];
            v *= fexp(Gs[r][c] - rho[c]);
          }
          x[j] = v;
        }
        put8(XT, c, 16 * isk + rr0, x);
      }
      // dA rows of block I, and [dA_qk^T | dA_kk^T]
      for (int e = t; e < 16 * (CL / 8); e += 256) {
        const int rr = e >> 3, i8 = (e & 7) * 8;
        put8(DQ, rr, i8, &sm.dAqk[16 * I + rr][i8]);
        put8(DK, rr, i8, &sm.dAkk[16 * I + rr][i8]);
      }
      for (int e = t; e < CL * 4; e += 256) {
        const int i = e & (CL - 1), part = e >> 6;
        const int isk = part >> 1, rr0 = (part & 1) * 8;
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = 16 * I + rr0 + j;
          x[j] = isk ? sm.dAkk[r][i] : sm.dAqk[r][i];
        }
        put8(DAT, i, 16 * isk + rr0, x);
      }
      __syncthreads();
      if (w == I) {
        // row side: rows of block I
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          f32x4 aq = zero4(), ak = zero4();
          mma<SPLIT_AB>(aq, DQ, 0, YT, 16 * nt, 0, nyk);
          mma<SPLIT_AB>(ak, DK, 0, YT, 16 * nt, 0, nyk);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * I + drow(i), c = 16 * nt + dcol();
            if (r < n) {
              const int64_t idx = rowidx(r) * HD + c;
              const float e1 = fexp(Gs[r][c] - rho[c]);
              const float qh = bf2f(q[idx]) * sm.rq[r], kh = bf2f(k[idx]) * sm.rk[r];
              const float dqa = aq[i] * e1, dka = ak[i] * e1;
              adq[nt][i] += dqa;
              adk[nt][i] += dka;
              adG[nt][i] += dqa * qh + dka * kh;
            }
          }
        }
      }
      if (w < I || (w == I && calm)) {
        // column side: columns i of block w from rows of block I
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          f32x4 a = zero4();
          mma_k<SPLIT_AB, 32>(a, DAT, 16 * w, XT, 16 * nt);
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int i = 16 * w + drow(i4), c = 16 * nt + dcol();
            if (i < n) {
              const float kh = bf2f(k[rowidx(i) * HD + c]) * sm.rk[i];
              const float dka = a[i4] * fexp(rho[c] - Gs[i][c]);
              adk[nt][i4] += dka;
              adG[nt][i4] -= dka * kh;
            }
          }
        }
      }
    }
    // Diagonal tiles of blocks whose decay span is too wide: element-wise fp32.
    if (!sm.calm[w]) {
      const int I = w;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int r = 16 * I + drow(i4), c = 16 * nt + dcol();
          if (r >= n) continue;
          const float qr = bf2f(q[rowidx(r) * HD + c]) * sm.rq[r];
          const float kr = bf2f(k[rowidx(r) * HD + c]) * sm.rk[r];
          float dq_s = 0.f, dk_s = 0.f, dG_s = 0.f;
          // as a row r: pairs (r, i), i <= r
          for (int i = 16 * I; i <= r; ++i) {
            const float kk = bf2f(k[rowidx(i) * HD + c]) * sm.rk[i] * fexp(Gs[r][c] - Gs[i][c]);
            const float a = sm.dAqk[r][i], b = sm.dAkk[r][i];
            dq_s += a * kk;
            dk_s += b * kk;
            dG_s += (a * qr + b * kr) * kk;
          }
          // as a column i = r: pairs (r2, r), r2 >= r
          for (int r2 = r; r2 < 16 * I + 16 && r2 < n; ++r2) {
            const float E = fexp(Gs[r2][c] - Gs[r][c]);
            const float q2 = bf2f(q[rowidx(r2) * HD + c]) * sm.rq[r2];
            const float k2 = bf2f(k[rowidx(r2) * HD + c]) * sm.rk[r2];
            const float s = (sm.dAqk[r2][r] * q2 + sm.dAkk[r2][r] * k2) * E;
            dk_s += s;
            dG_s -= s * kr;
          }
          adq[nt][i4] += dq_s;
          adk[nt][i4] += dk_s;
          adG[nt][i4] += dG_s;
        }
    }
    __syncthreads();
  }

  // ------------------------------------------------ P7: dg, L2 chain, outputs
  {
    float (*dG)[GS_LD] = sm.u.p7.dG;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + drow(i), c = 16 * nt + dcol();
        dG[r][c] = adG[nt][i] + (r == CL - 1 ? sm.dGL[c] : 0.f);
      }
    __syncthreads();
    if (t < HD) {
      const int c = t;
      float run = 0.f, pdt = 0.f, pA = 0.f;
      const float ea = d.raw ? __expf(in.A_log[h]) : 0.f;
      const float dtb = d.raw ? in.dt_bias[h * HD + c] : 0.f;
      for (int r = CL - 1; r >= 0; --r) {
        run += dG[r][c];
        if (r < n) {
          const int64_t idx = rowidx(r) * HD + c;
          if (d.raw) {
            const float z = bf2f(reinterpret_cast<const bf16*>(in.gate)[idx]) + dtb;
            const float dz = run * (-ea) * sigmoid(z);
            reinterpret_cast<bf16*>(out.dgate)[idx] = f2bf(dz);
            pdt += dz;
            pA += run * (-ea * softplus(z));
          } else {
            reinterpret_cast<float*>(out.dgate)[idx] = run;
          }
        }
      }
      if (d.raw) {
        bw.part_dt[ch * HD + c] = pdt;
        sm.u.p7.red[c] = pA;
      }
    }
    __syncthreads();
    if (d.raw && t == 0) {
      float s = 0.f;
      for (int c = 0; c < HD; ++c) s += sm.u.p7.red[c];
      bw.part_A[ch] = s;
    }
    // L2 chain and the bf16 outputs
    bf16* dq = reinterpret_cast<bf16*>(out.dq);
    bf16* dk = reinterpret_cast<bf16*>(out.dk);
    float pq[4] = {0.f, 0.f, 0.f, 0.f}, pk[4] = {0.f, 0.f, 0.f, 0.f};
    if (d.l2norm) {
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * w + drow(i), c = 16 * nt + dcol();
          if (r < n) {
            const int64_t idx = rowidx(r) * HD + c;
            pq[i] += bf2f(q[idx]) * sm.rq[r] * adq[nt][i];
            pk[i] += bf2f(k[idx]) * sm.rk[r] * adk[nt][i];
          }
        }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        for (int m = 1; m < 16; m <<= 1) {
          pq[i] += __shfl_xor(pq[i], m);
          pk[i] += __shfl_xor(pk[i], m);
        }
      }
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + drow(i), c = 16 * nt + dcol();
        if (r < n) {
          const int64_t idx = rowidx(r) * HD + c;
          float gq = adq[nt][i], gk = adk[nt][i];
          if (d.l2norm) {
            const float rq = sm.rq[r], rk = sm.rk[r];
            gq = rq * (gq - bf2f(q[idx]) * rq * pq[i]);
            gk = rk * (gk - bf2f(k[idx]) * rk * pk[i]);
          }
          dq[idx] = f2bf(gq);
          dk[idx] = f2bf(gk);
        }
      }
    if (t < n) reinterpret_cast<bf16*>(out.dbeta)[rowidx(t)] = f2bf(sm.db[t]);
  }
}

hipError_t launch_bwd_intra(const Dims& d, const Inputs& in, const ChunkTable& ct,
                            const float* G, const SavedSet& sv, const void* dO,
                            const BwdOut& out, const BwdWork& bw, hipStream_t s) {
  hipLaunchKernelGGL(bwd_intra_kernel, dim3(d.NC, d.H), dim3(256), 0, s, d, in, ct, G, sv,
                     reinterpret_cast<const bf16*>(dO), out, bw);
  return hipGetLastError();
}

// Raw gate: dA_log[h] = sum over chunks of sum_{t,c} dg g, ddt_bias[h][c] =
// sum over chunks of sum_t dz, both in chunk order (deterministic).
__global__ __launch_bounds__(128) void finalize_kernel(Dims d, ChunkTable ct, BwdOut out,
                                                        BwdWork bw) {
  const int h = blockIdx.x, c = threadIdx.x;
  const int nch = ct.doc_c0[d.N];
  float s = 0.f;
  for (int ci = 0; ci < nch; ++ci) s += bw.part_dt[((int64_t)ci * d.H + h) * HD + c];
  out.ddt_bias[h * HD + c] = s;
  if (c == 0) {
    float a = 0.f;
    for (int ci = 0; ci < nch; ++ci) a += bw.part_A[(int64_t)ci * d.H + h];
    out.dA_log[h] = a;
  }
}

hipError_t launch_finalize(const Dims& d, const ChunkTable& ct, const BwdOut& out,
                           const BwdWork& bw, hipStream_t s) {
  hipLaunchKernelGGL(finalize_kernel, dim3(d.H), dim3(HD), 0, s, d, ct, out, bw);
  return hipGetLastError();
}

}  // namespace kda
