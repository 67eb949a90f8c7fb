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
// then pushes dA_qk, dA_kk through the decayed products, accumulates dq, dk
// and dG (the gradient of the chunk-local cumsum G) per element, and finishes
// with dg_j = sum_{r >= j} dG_r (reverse cumsum inside the chunk) and the chain
// rules of the fused L2 norm and of the raw gate g = -exp(A_log) softplus(a +
// dt_bias). Each pair term of dG enters dG_r with + and dG_i with - from
// products of the same rounded operands (the diagonal pair rule of PR #8909's
// accuracy fix).
//
// Decayed products. When the chunk's total decay span is at most CALM_SPAN in
// every channel, one reference (the chunk start) serves every (r, i) pair:
// x_r e^(G_r - G_i) k_i = (x_r e^(G_r)) (k_i e^(-G_i)), all factors <= e^40.
// Otherwise each 16-row block I uses the reference rho_I = G before the block
// (both factors <= 1 for columns before the block) and a diagonal block whose
// own span is too wide is summed element by element in fp32.
//
// Work layout: 512 threads (8 waves). Wave w owns rows 16*(w&3).. of the
// chunk and channels 64*(w>>2).. of every 64 x 128 per-element quantity; the
// thread keeps its 16 elements' G, q^, k^ in registers, so epilogues read no
// memory.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int NTHR = 512;
constexpr int K1_LD = HD + 8;
constexpr int K2_LD = CL + 8;
constexpr int X_LD = 32 + 8;
constexpr int GS_LD = HD + 4;
constexpr int F_LD = CL + 1;        // fp32 64x64 matrices
constexpr float CALM_SPAN_B = 40.f;

// Split terms per product (SPLIT_A: first operand carries its lo part, ...).
#ifndef KDA_SPLIT_B1
#define KDA_SPLIT_B1 SPLIT_B     // U~ = Tb R, dR = Tb^T dU~
#endif
#ifndef KDA_SPLIT_B2
#define KDA_SPLIT_B2 SPLIT_B     // dKd = dR S_in^T
#endif
#ifndef KDA_SPLIT_B3
#define KDA_SPLIT_B3 SPLIT_B     // dQd = dO S_in^T (dO exact)
#endif
#ifndef KDA_SPLIT_B4
#define KDA_SPLIT_B4 SPLIT_AB    // dKe = U~ dS_out^T
#endif
#ifndef KDA_SPLIT_B5
#define KDA_SPLIT_B5 SPLIT_B     // dA_qk = dO U~^T (dO exact)
#endif
#ifndef KDA_SPLIT_B6
#define KDA_SPLIT_B6 SPLIT_AB    // dTb = dU~ R^T
#endif
#ifndef KDA_SPLIT_B7
#define KDA_SPLIT_B7 SPLIT_AB    // decayed-product backward: dA Y, dA^T X
#endif

struct BwdIntraSmem {
  union {
    struct {
      bf16 a_hi[CL][K2_LD], a_lo[CL][K2_LD];       // Tb [r][i], then Tb^T [i][r]
      bf16 b_hi[HD][K2_LD], b_lo[HD][K2_LD];       // R^T [j][i], then dU~^T [j][r]
    } p1;
    struct {
      bf16 s_hi[HD][K1_LD], s_lo[HD][K1_LD];       // S_in [c][j], then dS_out [c][j]
      bf16 a_hi[CL][K1_LD], a_lo[CL][K1_LD];       // dR [r][j], then U~ [r][j]
      bf16 do_hi[CL][K1_LD];                       // dO [r][j]
    } p2;
    struct {
      bf16 a_hi[CL][K1_LD], a_lo[CL][K1_LD];       // dU~ [r][j]
      bf16 b_hi[CL][K1_LD], b_lo[CL][K1_LD];       // R [i][j]
    } p4;
    struct {
      float dAqk[CL][F_LD], dAkk[CL][F_LD];        // shared with p6
      float T[CL][F_LD], dT[CL][F_LD], tmp[CL][F_LD];
    } p5;
    struct {
      float dAqk[CL][F_LD], dAkk[CL][F_LD];
      union {
        struct {                                   // single-reference path, part 1
          bf16 dq_hi[CL][K2_LD], dq_lo[CL][K2_LD]; // dA_qk [r][i]
          bf16 dk_hi[CL][K2_LD], dk_lo[CL][K2_LD]; // dA_kk [r][i]
          bf16 yt_hi[HD][K2_LD], yt_lo[HD][K2_LD]; // (k^ e^-G)^T [c][i]
        } a;
        struct {                                   // single-reference path, part 2
          bf16 dat_hi[CL][K1_LD], dat_lo[CL][K1_LD];   // [dA_qk^T | dA_kk^T] [i][128]
          bf16 xt_hi[HD][K1_LD], xt_lo[HD][K1_LD];     // [q^ e^G ; k^ e^G]^T [c][128]
        } b;
        struct {                                   // per-block path
          bf16 yt_hi[HD][K2_LD], yt_lo[HD][K2_LD];
          bf16 xt_hi[HD][X_LD], xt_lo[HD][X_LD];
          bf16 dq_hi[16][K2_LD], dq_lo[16][K2_LD];
          bf16 dk_hi[16][K2_LD], dk_lo[16][K2_LD];
          bf16 dat_hi[CL][X_LD], dat_lo[CL][X_LD];
          float Gb[16][HD], qb[16][HD], kb[16][HD];  // one diagonal block, fp32
        } g;
      } u;
    } p6;
    struct {
      float dG[CL][GS_LD];
      bf16 a[CL][HD];
      float tot[HD];
      float red[2][2][HD];
      float rowp[2][2][CL];
    } p7;
  } u;
  float beta[CL], rq[CL], rk[CL], db[CL];
  float GL[HD], gam[HD], dGL[HD];
  float Gref[5][HD];       // G before block I (I = 0..3) and G_last (I = 4)
  float dGLw[4][HD];
  int calm_blk[4];
  int calm_chunk;
};

__global__ __launch_bounds__(NTHR) void bwd_intra_kernel(Dims d, Inputs in, ChunkTable ct,
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
  const int rb = w & 3, chh = w >> 2;          // row block, channel half
  const int64_t ch = (int64_t)ci * d.H + h;
  const int H = d.H;
  const bf16* q = reinterpret_cast<const bf16*>(in.q);
  const bf16* k = reinterpret_cast<const bf16*>(in.k);
  const bf16* beta = reinterpret_cast<const bf16*>(in.beta);
  const float* Tg = sv.Tm + ch * CL * CL;
  const float* Akk_g = sv.Akk + ch * CL * CL;
  auto rowidx = [&](int r) -> int64_t { return (t0 + r) * H + h; };
  auto clampr = [&](int r) -> int { return r < n ? r : n - 1; };

  // ------------------------------------------------------------ P0: setup
  // this thread's elements: rows er(i) = 16 rb + drow(i), channels ec(nt) = 64 chh + 16 nt + dcol()
  float eG[4][4];
  bf16 eqb[4][4], ekb[4][4];       // raw q, k (bf16); q^ = q * rqr[i], zero on padded rows
  float rqr[4], rkr[4];
  {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r0 = 16 * rb + drow(i), r = clampr(r0);
      const float a = sv.rq[rowidx(r)], b = sv.rk[rowidx(r)];
      rqr[i] = r0 < n ? a : 0.f;
      rkr[i] = r0 < n ? b : 0.f;
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = clampr(16 * rb + drow(i));
        const int64_t idx = rowidx(r) * HD + 64 * chh + 16 * nt + dcol();
        eG[nt][i] = G[idx];
        eqb[nt][i] = q[idx];
        ekb[nt][i] = k[idx];
      }
  }
#define EQ(nt, i) (bf2f(eqb[nt][i]) * rqr[i])
#define EK(nt, i) (bf2f(ekb[nt][i]) * rkr[i])
  if (t < CL) {
    const int r = clampr(t);
    const bool ok = t < n;
    const float b = bf2f(beta[rowidx(r)]), a = sv.rq[rowidx(r)], c = sv.rk[rowidx(r)];
    sm.beta[t] = ok ? b : 0.f;
    sm.rq[t] = ok ? a : 0.f;
    sm.rk[t] = ok ? c : 0.f;
  }
  for (int e = t; e < 5 * HD; e += NTHR) {
    const int I = e >> 7, c = e & 127;
    const float v = I == 0 ? 0.f : G[rowidx(clampr(16 * I - 1)) * HD + c];
    sm.Gref[I][c] = v;
    if (I == 4) {
      sm.GL[c] = v;
      sm.gam[c] = fexp(v);
    }
  }
  if (t < 4) sm.calm_blk[t] = 1;
  if (t == 4) sm.calm_chunk = 1;
  __syncthreads();
  if (t < HD) {
    if (-sm.Gref[4][t] > CALM_SPAN_B) sm.calm_chunk = 0;
#pragma unroll
    for (int I = 0; I < 4; ++I)
      if (sm.Gref[I][t] - sm.Gref[I + 1][t] > CALM_SPAN_B) sm.calm_blk[I] = 0;
  }

  f32x4 adq[4], adk[4], adG[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) adq[nt] = adk[nt] = adG[nt] = zero4();

  // ------------------------------------------------------------ P1: U~ and dR
  f32x4 U[4], dR[4];
  {
    const Panel A{&sm.u.p1.a_hi[0][0], (KDA_SPLIT_B1 & SPLIT_A) ? &sm.u.p1.a_lo[0][0] : nullptr, K2_LD};
    const Panel B{&sm.u.p1.b_hi[0][0], &sm.u.p1.b_lo[0][0], K2_LD};
    // Tb [r][i]
    {
      const int r = t >> 3, i8 = (t & 7) * 8;
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(Tg + r * CL + i8);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(Tg + r * CL + i8 + 4);
      float x[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = a0[j] * sm.beta[i8 + j];
        x[j + 4] = a1[j] * sm.beta[i8 + 4 + j];
      }
      put8(A, r, i8, x);
    }
    // R^T [j][i]
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      const int e = t + NTHR * rep, j = e & 127, i8 = (e >> 7) * 8;
      float x[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int i = i8 + jj;
        const float v = sv.R[rowidx(clampr(i)) * HD + j];
        x[jj] = i < n ? v : 0.f;
      }
      put8(B, j, i8, x);
    }
    __syncthreads();
    const int kend = ((16 * rb + 16 + 31) / 32) * 32;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) U[nt] = zero4();
    mma_row<KDA_SPLIT_B1, 4>(U, A, 16 * rb, B, 64 * chh, 0, kend);
    __syncthreads();
    // Tb^T [i][r]
    {
      const int i = t & 63, r8 = (t >> 6) * 8;
      float x[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) x[jj] = Tg[(r8 + jj) * CL + i] * sm.beta[i];
      put8(A, i, r8, x);
    }
    // dU~^T [j][r]
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      const int e = t + NTHR * rep, j = e & 127, r8 = (e >> 7) * 8;
      float x[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int r = r8 + jj;
        const float v = bw.dU[rowidx(clampr(r)) * HD + j];
        x[jj] = r < n ? v : 0.f;
      }
      put8(B, j, r8, x);
    }
    __syncthreads();
    const int kbeg = (16 * rb / 32) * 32;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) dR[nt] = zero4();
    mma_row<KDA_SPLIT_B1, 4>(dR, A, 16 * rb, B, 64 * chh, kbeg, CL);
    __syncthreads();
  }

  // ------------------------------------------------------------ P2: dQd, dKd
  const Panel SP{&sm.u.p2.s_hi[0][0], &sm.u.p2.s_lo[0][0], K1_LD};
  const Panel AP{&sm.u.p2.a_hi[0][0], &sm.u.p2.a_lo[0][0], K1_LD};
  const Panel DOP{&sm.u.p2.do_hi[0][0], nullptr, K1_LD};
  auto load_state_panel = [&](const float* src) {
    // 128 x 128 fp32 -> split panel [c][j]; 8 float4 per thread, all issued first
    f32x4 v[8];
#pragma unroll
    for (int rep = 0; rep < 8; ++rep) {
      const int e = t + NTHR * rep, c = e >> 5, j4 = (e & 31) * 4;
      v[rep] = *reinterpret_cast<const f32x4*>(src + c * HD + j4);
    }
#pragma unroll
    for (int rep = 0; rep < 8; ++rep) {
      const int e = t + NTHR * rep, c = e >> 5, j4 = (e & 31) * 4;
      put4(SP, c, j4, v[rep]);
    }
  };
  {
    load_state_panel(sv.S_in + ch * HD * HD);
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      const int e = t + NTHR * rep, r = e >> 4, j8 = (e & 15) * 8;
      bf16x8 x = *reinterpret_cast<const bf16x8*>(dO + rowidx(clampr(r)) * HD + j8);
      if (r >= n) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) x[jj] = f2bf(0.f);
      }
      *reinterpret_cast<bf16x8*>(&sm.u.p2.do_hi[r][j8]) = x;
    }
    const Panel APd{AP.hi, (KDA_SPLIT_B2 & SPLIT_A) ? AP.lo : nullptr, K1_LD};
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) store_tile_n(dR[nt], APd, 16 * rb, 64 * chh + 16 * nt);
    __syncthreads();
    {
      f32x4 a[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) a[nt] = zero4();
      mma_row<KDA_SPLIT_B3, 4>(a, DOP, 16 * rb, SP, 64 * chh, 0, HD);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = d.scale * a[nt][i] * fexp(eG[nt][i]);
          adq[nt][i] += p;
          adG[nt][i] += p * EQ(nt, i);
        }
    }
    {
      f32x4 b[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) b[nt] = zero4();
      mma_row<KDA_SPLIT_B2, 4>(b, AP, 16 * rb, SP, 64 * chh, 0, HD);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p2 = -b[nt][i] * fexp(eG[nt][i]);
          adk[nt][i] += p2;
          adG[nt][i] += p2 * EK(nt, i);
        }
    }
    __syncthreads();
  }

  // ------------------------------------------------------------ P3: dKe, dA_qk, dgamma
  f32x4 dAq[2];
  {
    load_state_panel(bw.dS + ch * HD * HD);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) store_tile_n(U[nt], AP, 16 * rb, 64 * chh + 16 * nt);
    __syncthreads();
    f32x4 a[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) a[nt] = zero4();
    mma_row<KDA_SPLIT_B4, 4>(a, AP, 16 * rb, SP, 64 * chh, 0, HD);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int c = 64 * chh + 16 * nt + dcol();
      float colp = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p3 = a[nt][i] * fexp(sm.GL[c] - eG[nt][i]);
        adk[nt][i] += p3;
        adG[nt][i] -= p3 * EK(nt, i);
        colp += p3 * EK(nt, i);
      }
      colp += __shfl_xor(colp, 16);
      colp += __shfl_xor(colp, 32);
      if (l < 16) sm.dGLw[rb][c] = colp;
    }
    // dA_qk = scale dO U~^T: rows 16 rb, columns i in tiles 2 chh, 2 chh + 1
    dAq[0] = dAq[1] = zero4();
    mma_row<KDA_SPLIT_B5, 2>(dAq, DOP, 16 * rb, AP, 32 * chh, 0, HD);
    // dgamma[c] = sum_j dS_out[c][j] S_in[c][j]; four threads per channel
    {
      const int c = t >> 2, part = t & 3;
      const float* dSg = bw.dS + ch * HD * HD + c * HD + 32 * part;
      const float* Sg = sv.S_in + ch * HD * HD + c * HD + 32 * part;
      f32x4 xa[8], xb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        xa[j] = *reinterpret_cast<const f32x4*>(dSg + 4 * j);
        xb[j] = *reinterpret_cast<const f32x4*>(Sg + 4 * j);
      }
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) s += xa[j][0] * xb[j][0] + xa[j][1] * xb[j][1] + xa[j][2] * xb[j][2] + xa[j][3] * xb[j][3];
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      __syncthreads();
      if (part == 0)
        sm.dGL[c] = s * sm.gam[c] + ((sm.dGLw[0][c] + sm.dGLw[1][c]) + (sm.dGLw[2][c] + sm.dGLw[3][c]));
    }
    __syncthreads();
  }

  // ------------------------------------------------------------ P4: dTb = dU~ R^T
  f32x4 dTb[2];
  {
    const Panel DU{&sm.u.p4.a_hi[0][0], &sm.u.p4.a_lo[0][0], K1_LD};
    const Panel RP{&sm.u.p4.b_hi[0][0], &sm.u.p4.b_lo[0][0], K1_LD};
    f32x4 va[4], vb[4];
#pragma unroll
    for (int rep = 0; rep < 4; ++rep) {
      const int e = t + NTHR * rep, r = e >> 5, j4 = (e & 31) * 4;
      va[rep] = *reinterpret_cast<const f32x4*>(bw.dU + rowidx(clampr(r)) * HD + j4);
      vb[rep] = *reinterpret_cast<const f32x4*>(sv.R + rowidx(clampr(r)) * HD + j4);
    }
#pragma unroll
    for (int rep = 0; rep < 4; ++rep) {
      const int e = t + NTHR * rep, r = e >> 5, j4 = (e & 31) * 4;
      const f32x4 z = zero4();
      put4(DU, r, j4, r < n ? va[rep] : z);
      put4(RP, r, j4, r < n ? vb[rep] : z);
    }
    __syncthreads();
    dTb[0] = dTb[1] = zero4();
    mma_row<KDA_SPLIT_B6, 2>(dTb, DU, 16 * rb, RP, 32 * chh, 0, HD);
    __syncthreads();
  }

  // ------------------------------------------------------------ P5: WY / UT backward (fp32)
  {
    float (*dAqk)[F_LD] = sm.u.p5.dAqk;
    float (*dAkk)[F_LD] = sm.u.p5.dAkk;
    float (*Tm)[F_LD] = sm.u.p5.T;
    float (*dT)[F_LD] = sm.u.p5.dT;
    float (*tmp)[F_LD] = sm.u.p5.tmp;
    {
      f32x4 a0 = *reinterpret_cast<const f32x4*>(Tg + 8 * t);
      f32x4 a1 = *reinterpret_cast<const f32x4*>(Tg + 8 * t + 4);
      const int r = t >> 3, i8 = (t & 7) * 8;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        Tm[r][i8 + j] = a0[j];
        Tm[r][i8 + 4 + j] = a1[j];
      }
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rb + drow(i), c = 32 * chh + 16 * nt + dcol();
        dT[r][c] = (c <= r) ? dTb[nt][i] : 0.f;
        dAqk[r][c] = (c <= r) ? d.scale * dAq[nt][i] : 0.f;
      }
    __syncthreads();
    if (t < CL) {
      float s = 0.f;
      for (int r = t; r < CL; ++r) s += dT[r][t] * Tm[r][t];
      sm.db[t] = s;
    }
    __syncthreads();
#pragma unroll
    for (int rep = 0; rep < 8; ++rep) {
      const int e = t + NTHR * rep, r = e >> 6, m = e & 63;
      dT[r][m] *= sm.beta[m];
    }
    __syncthreads();
    // tmp = dT T^T : tmp[r][i] = sum_{m <= min(r, i)} dT[r][m] T[i][m]
#pragma unroll
    for (int rep = 0; rep < 8; ++rep) {
      const int e = t + NTHR * rep, r = e >> 6, i = e & 63;
      const int mmax = min(r, i);
      float s = 0.f;
      for (int m = 0; m <= mmax; ++m) s += dT[r][m] * Tm[i][m];
      tmp[r][i] = s;
    }
    __syncthreads();
    {
      // dX[r][i] = -sum_{m >= r} T[m][r] tmp[m][i] (i < r); eight threads per row
      const int r = t >> 3, part = t & 7;
      const f32x4 ak0 = *reinterpret_cast<const f32x4*>(Akk_g + r * CL + 8 * part);
      const f32x4 ak1 = *reinterpret_cast<const f32x4*>(Akk_g + r * CL + 8 * part + 4);
      float dbr = 0.f;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int i = 8 * part + jj;
        float dx = 0.f;
        if (i < r) {
          float s = 0.f;
          for (int m = r; m < CL; ++m) s += Tm[m][r] * tmp[m][i];
          dx = -s;
        }
        dAkk[r][i] = sm.beta[r] * dx;
        dbr += dx * (jj < 4 ? ak0[jj] : ak1[jj - 4]);
      }
      dbr += __shfl_xor(dbr, 1);
      dbr += __shfl_xor(dbr, 2);
      dbr += __shfl_xor(dbr, 4);
      __syncthreads();
      if (part == 0) sm.db[r] += dbr;
    }
    __syncthreads();
  }

  // ------------------------------------------------------------ P6: decayed-product backward
  {
    float (*dAqk)[F_LD] = sm.u.p6.dAqk;
    float (*dAkk)[F_LD] = sm.u.p6.dAkk;
    if (sm.calm_chunk) {
      // single reference at the chunk start
      const Panel DQ{&sm.u.p6.u.a.dq_hi[0][0], &sm.u.p6.u.a.dq_lo[0][0], K2_LD};
      const Panel DK{&sm.u.p6.u.a.dk_hi[0][0], &sm.u.p6.u.a.dk_lo[0][0], K2_LD};
      const Panel YT{&sm.u.p6.u.a.yt_hi[0][0], &sm.u.p6.u.a.yt_lo[0][0], K2_LD};
      {
        const int r = t >> 3, i8 = (t & 7) * 8;
        put8(DQ, r, i8, &dAqk[r][i8]);
        put8(DK, r, i8, &dAkk[r][i8]);
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        f32x4 y;
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = EK(nt, i) * fexp(-eG[nt][i]);
        put4(YT, 64 * chh + 16 * nt + dcol(), 16 * rb + 4 * (l >> 4), y);
      }
      __syncthreads();
      const int kend = ((16 * rb + 16 + 31) / 32) * 32;
      f32x4 aq[4], ak[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) aq[nt] = ak[nt] = zero4();
      mma_row<KDA_SPLIT_B7, 4>(aq, DQ, 16 * rb, YT, 64 * chh, 0, kend);
      mma_row<KDA_SPLIT_B7, 4>(ak, DK, 16 * rb, YT, 64 * chh, 0, kend);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e1 = fexp(eG[nt][i]);
          const float dqa = aq[nt][i] * e1, dka = ak[nt][i] * e1;
          adq[nt][i] += dqa;
          adk[nt][i] += dka;
          adG[nt][i] += dqa * EQ(nt, i) + dka * EK(nt, i);
        }
      __syncthreads();
      const Panel DAT{&sm.u.p6.u.b.dat_hi[0][0], &sm.u.p6.u.b.dat_lo[0][0], K1_LD};
      const Panel XT{&sm.u.p6.u.b.xt_hi[0][0], &sm.u.p6.u.b.xt_lo[0][0], K1_LD};
      {
        const int i = t & 63, part = t >> 6;           // part: 8 groups of 8 rows (qk 0-3, kk 4-7)
        const int r8 = (part & 3) * 16, isk = part >> 2;
        float x[8], y[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          x[jj] = isk ? dAkk[r8 + jj][i] : dAqk[r8 + jj][i];
          y[jj] = isk ? dAkk[r8 + 8 + jj][i] : dAqk[r8 + 8 + jj][i];
        }
        put8(DAT, i, 64 * isk + r8, x);
        put8(DAT, i, 64 * isk + r8 + 8, y);
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        f32x4 xq, xk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e1 = fexp(eG[nt][i]);
          xq[i] = EQ(nt, i) * e1;
          xk[i] = EK(nt, i) * e1;
        }
        const int c = 64 * chh + 16 * nt + dcol(), r0 = 16 * rb + 4 * (l >> 4);
        put4(XT, c, r0, xq);
        put4(XT, c, 64 + r0, xk);
      }
      __syncthreads();
      f32x4 ac[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) ac[nt] = zero4();
      const int kb = (16 * rb / 32) * 32;
      mma_row<KDA_SPLIT_B7, 4>(ac, DAT, 16 * rb, XT, 64 * chh, kb, CL);
      mma_row<KDA_SPLIT_B7, 4>(ac, DAT, 16 * rb, XT, 64 * chh, CL + kb, 2 * CL);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float dka = ac[nt][i] * fexp(-eG[nt][i]);
          adk[nt][i] += dka;
          adG[nt][i] -= dka * EK(nt, i);
        }
      __syncthreads();
    } else {
      // one reference per 16-row block
      const Panel YT{&sm.u.p6.u.g.yt_hi[0][0], &sm.u.p6.u.g.yt_lo[0][0], K2_LD};
      const Panel XT{&sm.u.p6.u.g.xt_hi[0][0], &sm.u.p6.u.g.xt_lo[0][0], X_LD};
      const Panel DQ{&sm.u.p6.u.g.dq_hi[0][0], &sm.u.p6.u.g.dq_lo[0][0], K2_LD};
      const Panel DK{&sm.u.p6.u.g.dk_hi[0][0], &sm.u.p6.u.g.dk_lo[0][0], K2_LD};
      const Panel DAT{&sm.u.p6.u.g.dat_hi[0][0], &sm.u.p6.u.g.dat_lo[0][0], X_LD};
      for (int I = 0; I < 4; ++I) {
        const int calm = sm.calm_blk[I];
        const int ny = 16 * I + 16;
        const int nyk = ((ny + 31) / 32) * 32;
        // Y^T [c][i]: rows of this thread's block, zero unless before block I
        // (or block I itself when its span is narrow)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int c = 64 * chh + 16 * nt + dcol();
          const float rho = sm.Gref[I][c];
          const bool on = rb < I || (rb == I && calm);
          f32x4 y;
#pragma unroll
          for (int i = 0; i < 4; ++i) y[i] = on ? EK(nt, i) * fexp(rho - eG[nt][i]) : 0.f;
          put4(YT, c, 16 * rb + 4 * (l >> 4), y);
          if (rb == I) {
            f32x4 xq, xk;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float e1 = fexp(eG[nt][i] - rho);
              xq[i] = EQ(nt, i) * e1;
              xk[i] = EK(nt, i) * e1;
            }
            put4(XT, c, 4 * (l >> 4), xq);
            put4(XT, c, 16 + 4 * (l >> 4), xk);
          }
        }
        if (t < 128) {
          const int rr = t >> 3, i8 = (t & 7) * 8;
          put8(DQ, rr, i8, &dAqk[16 * I + rr][i8]);
          put8(DK, rr, i8, &dAkk[16 * I + rr][i8]);
        } else if (t < 128 + 256) {
          const int e = t - 128, i = e & 63, part = e >> 6;   // 4 parts of 8
          const int isk = part >> 1, rr0 = (part & 1) * 8;
          float x[8];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj)
            x[jj] = isk ? dAkk[16 * I + rr0 + jj][i] : dAqk[16 * I + rr0 + jj][i];
          put8(DAT, i, 16 * isk + rr0, x);
        }
        __syncthreads();
        if (rb == I) {
          f32x4 aq[4], ak[4];
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) aq[nt] = ak[nt] = zero4();
          mma_row<KDA_SPLIT_B7, 4>(aq, DQ, 0, YT, 64 * chh, 0, nyk);
          mma_row<KDA_SPLIT_B7, 4>(ak, DK, 0, YT, 64 * chh, 0, nyk);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            const float rho = sm.Gref[I][64 * chh + 16 * nt + dcol()];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float e1 = fexp(eG[nt][i] - rho);
              const float dqa = aq[nt][i] * e1, dka = ak[nt][i] * e1;
              adq[nt][i] += dqa;
              adk[nt][i] += dka;
              adG[nt][i] += dqa * EQ(nt, i) + dka * EK(nt, i);
            }
          }
        }
        if (rb < I || (rb == I && calm)) {
          f32x4 ac[4];
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) ac[nt] = zero4();
          mma_row<KDA_SPLIT_B7, 4>(ac, DAT, 16 * rb, XT, 64 * chh, 0, 32);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            const float rho = sm.Gref[I][64 * chh + 16 * nt + dcol()];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float dka = ac[nt][i] * fexp(rho - eG[nt][i]);
              adk[nt][i] += dka;
              adG[nt][i] -= dka * EK(nt, i);
            }
          }
        }
        __syncthreads();
        if (!calm) {
          // exact fp32 sums for the pairs inside block I
          if (rb == I) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int rl = drow(i), c = 64 * chh + 16 * nt + dcol();
                sm.u.p6.u.g.Gb[rl][c] = eG[nt][i];
                sm.u.p6.u.g.qb[rl][c] = EQ(nt, i);
                sm.u.p6.u.g.kb[rl][c] = EK(nt, i);
              }
          }
          __syncthreads();
          if (rb == I) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int rl = drow(i), r = 16 * I + rl, c = 64 * chh + 16 * nt + dcol();
                const float gr = eG[nt][i], qr = EQ(nt, i), kr = EK(nt, i);
                float dq_s = 0.f, dk_s = 0.f, dG_s = 0.f;
                for (int il = 0; il <= rl; ++il) {
                  const float kk = sm.u.p6.u.g.kb[il][c] * fexp(gr - sm.u.p6.u.g.Gb[il][c]);
                  const float a = dAqk[r][16 * I + il], b = dAkk[r][16 * I + il];
                  dq_s += a * kk;
                  dk_s += b * kk;
                  dG_s += (a * qr + b * kr) * kk;
                }
                for (int r2 = rl; r2 < 16; ++r2) {
                  const float E = fexp(sm.u.p6.u.g.Gb[r2][c] - gr);
                  const float s = (dAqk[16 * I + r2][r] * sm.u.p6.u.g.qb[r2][c] +
                                   dAkk[16 * I + r2][r] * sm.u.p6.u.g.kb[r2][c]) * E;
                  dk_s += s;
                  dG_s -= s * kr;
                }
                adq[nt][i] += dq_s;
                adk[nt][i] += dk_s;
                adG[nt][i] += dG_s;
              }
          }
          __syncthreads();
        }
      }
    }
  }

  // ------------------------------------------------------------ P7: dg, L2 chain, outputs
  {
    float (*dG)[GS_LD] = sm.u.p7.dG;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rb + drow(i), c = 64 * chh + 16 * nt + dcol();
        dG[r][c] = adG[nt][i] + (r == CL - 1 ? sm.dGL[c] : 0.f);
      }
    const bf16* araw = reinterpret_cast<const bf16*>(in.gate);
    if (d.raw) {
#pragma unroll
      for (int rep = 0; rep < 2; ++rep) {
        const int e = t + NTHR * rep, r = e >> 4, c8 = (e & 15) * 8;
        *reinterpret_cast<bf16x8*>(&sm.u.p7.a[r][c8]) =
            *reinterpret_cast<const bf16x8*>(araw + rowidx(clampr(r)) * HD + c8);
      }
    }
    // L2 row dot products <x^, dx^> over the 128 channels
    float pq[4] = {0.f, 0.f, 0.f, 0.f}, pk[4] = {0.f, 0.f, 0.f, 0.f};
    if (d.l2norm) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pq[i] += EQ(nt, i) * adq[nt][i];
          pk[i] += EK(nt, i) * adk[nt][i];
        }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) {
          pq[i] += __shfl_xor(pq[i], m);
          pk[i] += __shfl_xor(pk[i], m);
        }
      if (dcol() == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sm.u.p7.rowp[0][chh][16 * rb + drow(i)] = pq[i];
          sm.u.p7.rowp[1][chh][16 * rb + drow(i)] = pk[i];
        }
      }
    }
    __syncthreads();
    // reverse cumsum within the chunk; two threads per channel (rows 32-63, 0-31)
    const int cc = t & 127, half = (t >> 7) & 1;
    const bool active = t < 256;
    if (active) {
      float run = 0.f;
      for (int r = 32 * half + 31; r >= 32 * half; --r) {
        run += dG[r][cc];
        dG[r][cc] = run;
      }
      if (half == 1) sm.u.p7.tot[cc] = run;
    }
    __syncthreads();
    float pdt = 0.f, pA = 0.f;
    if (active) {
      const float base = half == 0 ? sm.u.p7.tot[cc] : 0.f;
      const float ea = d.raw ? __expf(in.A_log[h]) : 0.f;
      const float dtb = d.raw ? in.dt_bias[h * HD + cc] : 0.f;
      for (int r = 32 * half; r < 32 * half + 32 && r < n; ++r) {
        const float dg = dG[r][cc] + base;
        const int64_t idx = rowidx(r) * HD + cc;
        if (d.raw) {
          const float z = bf2f(sm.u.p7.a[r][cc]) + dtb;
          const float dz = dg * (-ea) * sigmoid(z);
          reinterpret_cast<bf16*>(out.dgate)[idx] = f2bf(dz);
          pdt += dz;
          pA += dg * (-ea * softplus(z));
        } else {
          reinterpret_cast<float*>(out.dgate)[idx] = dg;
        }
      }
      sm.u.p7.red[0][half][cc] = pdt;
      sm.u.p7.red[1][half][cc] = pA;
    }
    __syncthreads();
    if (d.raw) {
      if (t < HD) bw.part_dt[ch * HD + t] = sm.u.p7.red[0][0][t] + sm.u.p7.red[0][1][t];
      if (t == HD) {
        float s = 0.f;
        for (int c2 = 0; c2 < HD; ++c2) s += sm.u.p7.red[1][0][c2] + sm.u.p7.red[1][1][c2];
        bw.part_A[ch] = s;
      }
    }
    // dq, dk (L2 chain) and dbeta
    bf16* dq = reinterpret_cast<bf16*>(out.dq);
    bf16* dk = reinterpret_cast<bf16*>(out.dk);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * rb + drow(i);
      float tq = 0.f, tk = 0.f;
      if (d.l2norm) {
        tq = sm.u.p7.rowp[0][0][r] + sm.u.p7.rowp[0][1][r];
        tk = sm.u.p7.rowp[1][0][r] + sm.u.p7.rowp[1][1][r];
      }
      if (r < n) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int64_t idx = rowidx(r) * HD + 64 * chh + 16 * nt + dcol();
          float gq = adq[nt][i], gk = adk[nt][i];
          if (d.l2norm) {
            gq = sm.rq[r] * (gq - EQ(nt, i) * tq);
            gk = sm.rk[r] * (gk - EK(nt, i) * tk);
          }
          dq[idx] = f2bf(gq);
          dk[idx] = f2bf(gk);
        }
      }
    }
    if (t < n) reinterpret_cast<bf16*>(out.dbeta)[rowidx(t)] = f2bf(sm.db[t]);
  }
}

#undef EQ
#undef EK

hipError_t launch_bwd_intra(const Dims& d, const Inputs& in, const ChunkTable& ct,
                            const float* G, const SavedSet& sv, const void* dO,
                            const BwdOut& out, const BwdWork& bw, hipStream_t s) {
  hipLaunchKernelGGL(bwd_intra_kernel, dim3(d.NC, d.H), dim3(NTHR), 0, s, d, in, ct, G, sv,
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
