// Packed-varlen causal GQA training attention, head dimension 256 (flashinfer
// PR #7774, description and commit notes: bottom-right causal alignment per
// segment, natural-log LSE, dK / dV as FP32 sums over each key head's query
// heads in three output forms, BF16 in and out with FP32 accumulation).
//
// Every product runs on v_mfma_f32_16x16x32_bf16 with fp32 accumulation. A
// workgroup is 4 waves over a 64-row block; a wave owns 16 rows.
//   forward:  per (query block, HPW query heads of one group), key blocks of
//             64 in order with an online softmax in base 2: S = Q K^T,
//             P = exp2(S scale log2 e - m), O += P V, then O / l and
//             lse = (m + log2 l) ln 2. The heads of a workgroup share each
//             staged K / V block and every operand fragment read from it.
//   delta:    Delta_i = <dO_i, o_i> per (row, head).
//   dq:       per (query block, query head): S, P from the lse, dP = dO V^T,
//             dS = P (dP - Delta), dq += dS K.
//   dk, dv:   per (key block, key head): for each query head of the group in
//             order and each query block that sees the keys, P^T and dS^T,
//             dv += P^T dO, dk += dS^T Q; the fixed order makes the sums over
//             the group's heads the same bits every run.
//   row map:  the fp32 window sums go to their destination rows through a
//             sort of (row, key) pairs, so that the keys sharing a row are
//             summed in ascending key order.
// P and dS enter their products as bf16. Rows past a block's end are loaded
// from the block's last row and masked out.
#include <cmath>
#include <utility>

#include "kda_attn.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace attn {

constexpr int AD = 256;           // head dimension
constexpr int BR = 64;            // rows of a query or key block
constexpr int A_LD = AD + 16;     // 544-byte rows of a staged block (conflict-free 16-byte reads)
constexpr float LOG2E_F = 1.4426950408889634f;
constexpr float LN2_F = 0.6931471805599453f;

struct Dims {
  int64_t Tq, Tk;
  int S, Hq, Hkv, grp;
  int NCq, NCk;                   // 64-query and 128-key blocks, upper bounds
  float scale;
};

// The segment of block ci: the last s with c0[s] <= ci (an empty segment
// shares its first block index with the next one).
KDA_DEV int seg_of(const int32_t* c0, int S, int ci) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (ld_const(c0, mid) <= ci) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Segment bounds, clamped into the packed tensors.
KDA_DEV void seg_bounds(const int32_t* cu, int s, int64_t T, int64_t& a, int64_t& n) {
  int64_t x = ld_const(cu, s), y = ld_const(cu, s + 1);
  x = x < 0 ? 0 : (x > T ? T : x);
  y = y < x ? x : (y > T ? T : y);
  a = x;
  n = y - x;
}

// Workgroup x of a (query block, HPW query heads) launch: key heads vary
// fastest, then the HPW-head slices of the group, then the query block, so
// that the XCDs (dealt workgroups round robin) each see few key heads and the
// heads of one query block start together.
template <int HPW>
KDA_DEV void qblock_heads(const Dims& a, int x, int& ci, int& h0) {
  const int slices = a.grp / HPW, g = x % a.Hkv, rest = x / a.Hkv;
  ci = rest / slices;
  h0 = g * a.grp + (rest % slices) * HPW;
}

KDA_DEV float row_max16(float v) {
  v = fmaxf(v, row_xor<1>(v));
  v = fmaxf(v, row_xor<3>(v));
  v = fmaxf(v, row_xor<7>(v));
  return fmaxf(v, row_xor<15>(v));
}

// ------------------------------------------------------------------ helpers
// 64 rows of one head of a [T, H, 256] bf16 tensor into a padded LDS block
// (rows of A_LD = 272 elements: 34 chunks of 16 bytes, the last two padding)
// by direct global-to-LDS loads, which use no registers. Wave instruction
// `ins` fills the 64 chunks (1 KiB) from chunk 64 ins on, lane L the one at
// 64 ins + L; a padding chunk gets a copy of its row's last chunk. NW waves
// share the 34 instructions. Rows from n on repeat row n - 1. The caller
// waits for the loads (vmcnt) and then for the other waves.
template <int NW>
KDA_DEV void dma_rows(bf16 (*blk)[A_LD], const bf16* src, int64_t row0, int n, int H, int h) {
  typedef __attribute__((address_space(1))) const void* gptr;
  typedef __attribute__((address_space(3))) void* lptr;
  constexpr int CPR = A_LD / 8, INS = BR * CPR / 64;    // 34 chunks per row, 34 instructions
  static_assert(BR * CPR % 64 == 0, "whole wave instructions");
  const int w = wave_id(), l = lane_id();
  bf16* base = &blk[0][0];
  // row addresses: the first row read (common to the workgroup) plus a 32-bit
  // byte offset per lane. With n <= 0 every row is row0 + n - 1 (the row
  // before the block), which then is that first row.
  const int64_t rfirst = n > 0 ? row0 : row0 + n - 1;
  const int nn = n > 0 ? n : 1;
  const char* src0 = reinterpret_cast<const char*>(src + (rfirst * H + h) * AD);
  const uint32_t rs = 2u * (uint32_t)H * AD;
#pragma unroll
  for (int j = 0; j < (INS + NW - 1) / NW; ++j) {
    const int ins = w + NW * j;
    if (ins < INS) {
      const int qc = 64 * ins + l, r = qc / CPR, c = qc - r * CPR;
      const int cc = c < AD / 8 ? c : AD / 8 - 1, rr = r < nn ? r : nn - 1;
      __builtin_amdgcn_global_load_lds((gptr)(src0 + ((uint32_t)rr * rs + 16u * (uint32_t)cc)),
                                       (lptr)(base + 512 * ins), 16, 0, 0);
    }
  }
}

// A thread's share of 64 rows of one head of a [T, H, 256] bf16 tensor when
// NW waves stage a block (2048 chunks of 16 bytes): requested into registers
// one block ahead of its use, so that the loads fly while the current block
// is computed. Rows from n on repeat row n - 1.
template <int NW>
KDA_DEV void pre_load(bf16x8 (&x)[32 / NW], const bf16* src, int64_t row0, int n, int H, int h) {
  // (as in dma_rows: the first row read is the base; n <= 0 reads row0 + n - 1)
  const int64_t rfirst = n > 0 ? row0 : row0 + n - 1;
  const int nn = n > 0 ? n : 1;
  const bf16x8* src0 = reinterpret_cast<const bf16x8*>(src + (rfirst * H + h) * AD);
  const uint32_t rs = 2u * (uint32_t)H * AD;
#pragma unroll
  for (int i = 0; i < 32 / NW; ++i) {
    const int u = threadIdx.x + 64 * NW * i, r = u >> 5, c = u & 31;
    const int rr = r < nn ? r : nn - 1;
    x[i] = ld_at(src0, (uint32_t)rr * rs + 16u * (uint32_t)c);
  }
}

template <int NW>
KDA_DEV void pre_store(bf16 (*blk)[A_LD], const bf16x8 (&x)[32 / NW]) {
#pragma unroll
  for (int i = 0; i < 32 / NW; ++i) {
    const int u = threadIdx.x + 64 * NW * i;
    *reinterpret_cast<bf16x8*>(&blk[u >> 5][8 * (u & 31)]) = x[i];
  }
}

// Wait for this wave's direct loads, then for every wave.
KDA_DEV void dma_join() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// A wave's 16 x 256 fp32 tiles (D layout) to bf16 rows of a [T, H, 256]
// tensor through rows 16 wr .. + 15 of an LDS block.
KDA_DEV void write_rows_bf16(bf16 (*stage)[A_LD], int wr, const f32x4 (&acc)[16], float mul,
                             bf16* dst, int64_t row0, int nvalid, int H, int h) {
  // (no valid row: row0 may lie past the tensor, and nothing is written; the
  // staging below is this wave's own)
  if (nvalid <= 0) return;
  const int l = lane_id();
#pragma unroll
  for (int dt = 0; dt < 16; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) stage[16 * wr + drow(i)][16 * dt + dcol()] = f2bf(acc[dt][i] * mul);
  __builtin_amdgcn_s_waitcnt(0xc07f);     // this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  bf16* dst0 = dst + (row0 * H + h) * AD;
  for (int u = l; u < 16 * AD / 8; u += 64) {
    const int r = u >> 5, c8 = (u & 31) * 8, row = 16 * wr + r;
    if (row < nvalid)
      *reinterpret_cast<bf16x8*>(dst0 + ((uint32_t)row * (uint32_t)H * AD + c8)) =
          *reinterpret_cast<const bf16x8*>(&stage[row][c8]);
  }
}

// ------------------------------------------------------------------ P panels
// A wave's P (or dS) block goes through LDS transposed, as [64][16]: the
// four D-layout values a lane holds for one column (rows 4 (l / 16) .. + 3)
// are one 8-byte store, and the MFMA A operand comes back through the
// transpose loads. Rows of the panel are the block's 64 columns.
constexpr int PT_LD = 16;

KDA_DEV void put_pt(bf16* pt, int nt, const f32x4& x) {
  bf16x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = f2bf(x[i]);
  *reinterpret_cast<bf16x4*>(pt + (16 * nt + dcol()) * PT_LD + 4 * (lane_id() >> 4)) = v;
}

// Slack of the running maximum, in log2 units: the stored maximum moves only
// when a row's new maximum exceeds it by more than this, so P stays below
// 2^8 and the O rescale is skipped whenever no row of the wave moved.
constexpr float M_SLACK = 8.f;

// ------------------------------------------------------------------ forward
// Workgroup: one 64-row query block of HPW query heads of one group, 4 waves
// per head (wave w: head h0 + w / 4, rows 16 (w % 4) .. + 15). The heads
// share every staged K / V block.
template <int HPW>
struct FwdSmem {
  bf16 k[BR][A_LD];
  bf16 v[BR][A_LD];
  bf16 pt[4 * HPW][BR * PT_LD];
};

template <int HPW>
__global__ __launch_bounds__(256 * HPW) __attribute__((amdgpu_waves_per_eu(2, 2))) void
attn_fwd_kernel(Dims a, ChunkTable qt, const int32_t* __restrict__ cuq,
                const int32_t* __restrict__ cuk, const bf16* __restrict__ q,
                const bf16* __restrict__ k, const bf16* __restrict__ v, bf16* __restrict__ o,
                float* __restrict__ lse) {
  __shared__ FwdSmem<HPW> sm;
  int ci, h0;
  qblock_heads<HPW>(a, blockIdx.x, ci, h0);
  if (ci >= ld_const(qt.doc_c0, a.S)) return;
  const int s = seg_of(qt.doc_c0, a.S, ci);
  // a segment's query blocks in reverse: the late ones see the most keys and
  // start first
  ci = ld_const(qt.doc_c0, s) + ld_const(qt.doc_c0, s + 1) - 1 - ci;
  int64_t qs, Lq, ks, Lk;
  seg_bounds(cuq, s, a.Tq, qs, Lq);
  seg_bounds(cuk, s, a.Tk, ks, Lk);
  const int64_t t0 = ld_const(qt.tok, ci);
  const int nq = ld_const(qt.len, ci);
  const int64_t i0 = t0 - qs, off = Lk - Lq;
  const int w = wave_id(), wr = w & 3, l = lane_id();
  const int h = h0 + (w >> 2), g = h / a.grp;
  const float c2 = a.scale * LOG2E_F;

  bf16x8 qf[8];
  {
    const int r = 16 * wr + (l & 15), rr = r < nq ? r : nq - 1;
    const bf16* src = q + ((t0 + rr) * a.Hq + h) * AD + 8 * (l >> 4);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(src + 32 * kk);
  }
  // m: stored row maximum (scaled, log2 units); ls: this lane's partial row
  // sum over its columns, reduced across the row once at the end
  float m[4], ls[4];
  f32x4 O[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) m[i] = -INFINITY, ls[i] = 0.f;
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) O[dt] = zero4();
  int64_t kend = i0 + nq + off;             // keys [0, kend) can be seen by the block
  kend = kend < 0 ? 0 : (kend > Lk ? Lk : kend);
  // eight waves prefetch the next K / V block into registers (32 each);
  // four load theirs directly into LDS and rely on a second workgroup
  constexpr int NW = 4 * HPW;
  bf16x8 pk[32 / NW], pv[32 / NW];
  if constexpr (HPW == 2) {
    if (kend > 0) {
      const int n0 = (int)(kend < BR ? kend : BR);
      pre_load<NW>(pk, k, ks, n0, a.Hkv, g);
      pre_load<NW>(pv, v, ks, n0, a.Hkv, g);
    }
  }
  for (int64_t kb0 = 0; kb0 < kend; kb0 += BR) {
    const int nk = (int)(kend - kb0 < BR ? kend - kb0 : BR);
    __syncthreads();                        // every wave is done with the previous block
    if constexpr (HPW == 2) {
      pre_store<NW>(sm.k, pk);
      pre_store<NW>(sm.v, pv);
      __syncthreads();
      if (kb0 + BR < kend) {
        const int64_t nb = kb0 + BR;
        const int n1 = (int)(kend - nb < BR ? kend - nb : BR);
        pre_load<NW>(pk, k, ks + nb, n1, a.Hkv, g);
        pre_load<NW>(pv, v, ks + nb, n1, a.Hkv, g);
      }
    } else {
      dma_rows<NW>(sm.k, k, ks + kb0, nk, a.Hkv, g);
      dma_rows<NW>(sm.v, v, ks + kb0, nk, a.Hkv, g);
      dma_join();
    }
    f32x4 S[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) S[nt] = zero4();
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        S[nt] = mfma16(qf[kk], frag(&sm.k[0][0], A_LD, 16 * nt, 32 * kk), S[nt]);
    // every row of the block sees every key of this key block
    const bool full = nk == BR && nq == BR && kb0 + BR - 1 <= i0 + off;
    if (!full) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * wr + drow(i), jl = 16 * nt + dcol();
          if (!(r < nq && jl < nk && kb0 + jl <= i0 + r + off)) S[nt][i] = -INFINITY;
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mx = fmaxf(fmaxf(S[0][i], S[1][i]), fmaxf(S[2][i], S[3][i]));
      mx = row_max16(mx) * c2;
      const bool up = mx > m[i] + M_SLACK;
      // O rows move only when one of the four rows i of the wave moved
      if (__builtin_amdgcn_ballot_w64(up)) {
        const float corr = up ? __builtin_amdgcn_exp2f(m[i] - mx) : 1.f;
        ls[i] *= corr;
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) O[dt][i] *= corr;
      }
      m[i] = up ? mx : m[i];
      const float sub = m[i] == -INFINITY ? 0.f : m[i];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[nt][i], c2, -sub));
        S[nt][i] = p;
        ls[i] += p;
      }
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) put_pt(sm.pt[w], nt, S[nt]);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 pa = fragT(sm.pt[w], PT_LD, 0, 32 * kk);
#pragma unroll
      for (int dt = 0; dt < 16; ++dt)
        O[dt] = mfma16(pa, fragT(&sm.v[0][0], A_LD, 16 * dt, 32 * kk), O[dt]);
    }
  }
  __syncthreads();                          // K and V are free: O leaves through them
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * wr + drow(i);
    const float tot = row_sum16(ls[i]);
    const bool seen = tot > 0.f;
    const float inv = seen ? 1.f / tot : 0.f;
    if (lse && dcol() == 0 && r < nq)
      lse[(t0 + r) * a.Hq + h] = seen ? (m[i] + __builtin_amdgcn_logf(tot)) * LN2_F : -INFINITY;
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) O[dt][i] *= inv;
  }
  write_rows_bf16((w >> 2) ? sm.v : sm.k, wr, O, 1.f, o, t0, nq, a.Hq, h);
}

// ------------------------------------------------------------------ delta
// Delta[row, h] = <dO, o> over the 256 channels: one wave per (row, head).
__global__ __launch_bounds__(256) void attn_delta_kernel(int64_t n, const bf16* __restrict__ o,
                                                        const bf16* __restrict__ dO,
                                                        float* __restrict__ delta) {
  const int l = lane_id();
  for (int64_t e = (int64_t)blockIdx.x * 4 + wave_id(); e < n; e += (int64_t)gridDim.x * 4) {
    const bf16x4 x = *reinterpret_cast<const bf16x4*>(o + e * AD + 4 * l);
    const bf16x4 y = *reinterpret_cast<const bf16x4*>(dO + e * AD + 4 * l);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) s += bf2f(x[i]) * bf2f(y[i]);
    s = row_sum16(s);
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    if (l == 0) delta[e] = s;
  }
}

// ------------------------------------------------------------------ dq
// Workgroup as in the forward: one query block of HPW heads of one group.
template <int HPW>
struct DqSmem {
  bf16 k[BR][A_LD];
  bf16 v[BR][A_LD];
  bf16 pt[4 * HPW][BR * PT_LD];
};

template <int HPW>
__global__ __launch_bounds__(256 * HPW) __attribute__((amdgpu_waves_per_eu(2, 2))) void
attn_dq_kernel(Dims a, ChunkTable qt, const int32_t* __restrict__ cuq,
               const int32_t* __restrict__ cuk, const bf16* __restrict__ q,
               const bf16* __restrict__ k, const bf16* __restrict__ v,
               const bf16* __restrict__ dO, const float* __restrict__ lse,
               const float* __restrict__ delta, bf16* __restrict__ dq) {
  __shared__ DqSmem<HPW> sm;
  int ci, h0;
  qblock_heads<HPW>(a, blockIdx.x, ci, h0);
  if (ci >= ld_const(qt.doc_c0, a.S)) return;
  const int s = seg_of(qt.doc_c0, a.S, ci);
  // a segment's query blocks in reverse: the late ones see the most keys and
  // start first
  ci = ld_const(qt.doc_c0, s) + ld_const(qt.doc_c0, s + 1) - 1 - ci;
  int64_t qs, Lq, ks, Lk;
  seg_bounds(cuq, s, a.Tq, qs, Lq);
  seg_bounds(cuk, s, a.Tk, ks, Lk);
  const int64_t t0 = ld_const(qt.tok, ci);
  const int nq = ld_const(qt.len, ci);
  const int64_t i0 = t0 - qs, off = Lk - Lq;
  const int w = wave_id(), wr = w & 3, l = lane_id();
  const int h = h0 + (w >> 2), g = h / a.grp;
  const float c2 = a.scale * LOG2E_F;

  bf16x8 qf[8], df[8];
  {
    const int r = 16 * wr + (l & 15), rr = r < nq ? r : nq - 1;
    const int64_t base = ((t0 + rr) * a.Hq + h) * AD + 8 * (l >> 4);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      qf[kk] = *reinterpret_cast<const bf16x8*>(q + base + 32 * kk);
      df[kk] = *reinterpret_cast<const bf16x8*>(dO + base + 32 * kk);
    }
  }
  float lb[4], dl[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * wr + drow(i), rr = r < nq ? r : nq - 1;
    lb[i] = lse[(t0 + rr) * a.Hq + h] * LOG2E_F;
    dl[i] = delta[(t0 + rr) * a.Hq + h];
  }
  f32x4 dQ[16];
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) dQ[dt] = zero4();
  int64_t kend = i0 + nq + off;
  kend = kend < 0 ? 0 : (kend > Lk ? Lk : kend);
  for (int64_t kb0 = 0; kb0 < kend; kb0 += BR) {
    const int nk = (int)(kend - kb0 < BR ? kend - kb0 : BR);
    __syncthreads();
    dma_rows<4 * HPW>(sm.k, k, ks + kb0, nk, a.Hkv, g);
    dma_rows<4 * HPW>(sm.v, v, ks + kb0, nk, a.Hkv, g);
    dma_join();
    f32x4 S[4], dP[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) S[nt] = dP[nt] = zero4();
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        S[nt] = mfma16(qf[kk], frag(&sm.k[0][0], A_LD, 16 * nt, 32 * kk), S[nt]);
        dP[nt] = mfma16(df[kk], frag(&sm.v[0][0], A_LD, 16 * nt, 32 * kk), dP[nt]);
      }
    const bool full = nk == BR && nq == BR && kb0 + BR - 1 <= i0 + off;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      f32x4 ds;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * wr + drow(i), jl = 16 * nt + dcol();
        const bool vis = full || (r < nq && jl < nk && kb0 + jl <= i0 + r + off);
        const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(S[nt][i], c2, -lb[i])) : 0.f;
        ds[i] = p * (dP[nt][i] - dl[i]);
      }
      put_pt(sm.pt[w], nt, ds);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 da = fragT(sm.pt[w], PT_LD, 0, 32 * kk);
#pragma unroll
      for (int dt = 0; dt < 16; ++dt)
        dQ[dt] = mfma16(da, fragT(&sm.k[0][0], A_LD, 16 * dt, 32 * kk), dQ[dt]);
    }
  }
  __syncthreads();
  write_rows_bf16((w >> 2) ? sm.v : sm.k, wr, dQ, a.scale, dq, t0, nq, a.Hq, h);
}

// ------------------------------------------------------------------ dk, dv
// Workgroup: one 128-key block (BK) of one key head, 8 waves of 16 keys that
// share each staged query block; the next item's q and dO are requested into
// registers while the current one is computed. K is the A operand of a
// wave's own keys and stays in registers; V (dk pass) is read from LDS. dv
// and dk are two launches of one kernel (WANT_DK false / true): holding both
// accumulators would leave no registers for a second wave per SIMD; the dk
// pass recomputes the S^T that the dv pass also forms.
constexpr int BK = 128;

struct KvSmem {
  union {
    struct {
      bf16 q[BR][A_LD];
      bf16 dO[BR][A_LD];
      bf16 pt[8][BR * PT_LD];       // P^T (dv pass) or dS^T (dk pass), stored [query][key]
    } in;
    float out[BR][AD + 4];          // fp32 results of four waves on their way out
  } u;
  bf16 vb[BK][A_LD];                // the block's V rows (dk pass: A operand of dP^T)
};

// F32: fp32 rows (window gradients, or the row-map form's staging), else bf16.
template <bool WANT_DK, bool F32>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_dkdv_kernel(
    Dims a, ChunkTable qt, ChunkTable kt, const int32_t* __restrict__ cuq,
    const int32_t* __restrict__ cuk, const bf16* __restrict__ q, const bf16* __restrict__ k,
    const bf16* __restrict__ v, const bf16* __restrict__ dO, const float* __restrict__ lse,
    const float* __restrict__ delta, void* __restrict__ out) {
  __shared__ KvSmem sm;
  // key heads vary fastest: neighbouring workgroups (which the dispatcher
  // deals round robin over the XCDs) take the same key block of every head,
  // so that each XCD sees the key heads congruent to it and the heavy early
  // blocks of a segment start together
  const int cj = blockIdx.x / a.Hkv, g = blockIdx.x % a.Hkv;
  if (cj >= ld_const(kt.doc_c0, a.S)) return;
  const int s = seg_of(kt.doc_c0, a.S, cj);
  int64_t qs, Lq, ks, Lk;
  seg_bounds(cuq, s, a.Tq, qs, Lq);
  seg_bounds(cuk, s, a.Tk, ks, Lk);
  const int64_t u0 = ld_const(kt.tok, cj);
  const int nk = ld_const(kt.len, cj);
  const int64_t j0 = u0 - ks, off = Lk - Lq;
  const int w = wave_id(), l = lane_id();
  const int jw = 16 * w;                // the wave's first key in the block
  const float c2 = a.scale * LOG2E_F;
  // query blocks of the segment that see some of these keys: i + off >= j0
  const int qc0 = ld_const(qt.doc_c0, s), qc1 = ld_const(qt.doc_c0, s + 1);
  int64_t ifirst = j0 - off;
  ifirst = ifirst < 0 ? 0 : ifirst;
  const int64_t qf64 = qc0 + ifirst / BR;
  const int qfirst = qf64 < qc1 ? (int)qf64 : qc1;

  bf16x8 kf[8];                       // A fragments of the wave's 16 keys
  {
    const int r = jw + (l & 15), rr = r < nk ? r : nk - 1;
    const int64_t base = ((u0 + rr) * a.Hkv + g) * AD + 8 * (l >> 4);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) kf[kk] = *reinterpret_cast<const bf16x8*>(k + base + 32 * kk);
  }
  if (WANT_DK) {
    // the block's V rows, 128 of them (rows past nk repeat the last key)
    dma_rows<8>(reinterpret_cast<bf16 (*)[A_LD]>(&sm.vb[0][0]), v, u0, nk, a.Hkv, g);
    dma_rows<8>(reinterpret_cast<bf16 (*)[A_LD]>(&sm.vb[BR][0]), v, u0 + BR, nk - BR, a.Hkv, g);
  }
  f32x4 acc[16];
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) acc[dt] = zero4();
  const int nqb = qc1 - qfirst, items = a.grp * nqb;
  // the (query head, query block) items in a fixed order, heads outer; each
  // item's q, dO, lse and Delta are requested one item ahead
  bf16x8 pq[4], pd[4];
  float plb[4], pdl[4];
  auto fetch = [&](int it) {
    const int h = g * a.grp + it / nqb, qc = qfirst + it % nqb;
    const int64_t t0 = ld_const(qt.tok, qc);
    const int nq = ld_const(qt.len, qc);
    pre_load<8>(pq, q, t0, nq, a.Hq, h);
    pre_load<8>(pd, dO, t0, nq, a.Hq, h);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int qcol = 16 * nt + dcol(), qq = qcol < nq ? qcol : nq - 1;
      const uint32_t o = 4u * (uint32_t)qq * (uint32_t)a.Hq;
      plb[nt] = ld_at(lse + t0 * a.Hq + h, o);
      pdl[nt] = WANT_DK ? ld_at(delta + t0 * a.Hq + h, o) : 0.f;
    }
  };
  if (items > 0) fetch(0);
  __builtin_amdgcn_s_waitcnt(0);      // the V rows (and the first item) have landed
  for (int it = 0; it < items; ++it) {
    const int qc = qfirst + it % nqb;
    const int64_t t0 = ld_const(qt.tok, qc);
    const int nq = ld_const(qt.len, qc);
    const int64_t i0 = t0 - qs;
    float lbq[4], dlq[4];             // lse log2 e and Delta of this lane's query columns
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) lbq[nt] = plb[nt] * LOG2E_F, dlq[nt] = pdl[nt];
    __syncthreads();                  // every wave is done with the previous item's panels
    pre_store<8>(sm.u.in.q, pq);
    pre_store<8>(sm.u.in.dO, pd);
    __syncthreads();
    if (it + 1 < items) fetch(it + 1);
    // a wave whose keys no query of this block sees skips the item
    if (jw >= nk || j0 + jw > i0 + nq - 1 + off) continue;
    f32x4 S[4], dP[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) S[nt] = dP[nt] = zero4();
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        S[nt] = mfma16(kf[kk], frag(&sm.u.in.q[0][0], A_LD, 16 * nt, 32 * kk), S[nt]);
        if (WANT_DK)
          dP[nt] = mfma16(frag(&sm.vb[0][0], A_LD, jw, 32 * kk),
                          frag(&sm.u.in.dO[0][0], A_LD, 16 * nt, 32 * kk), dP[nt]);
      }
    // S^T[key][query]: keys are rows jw + drow(i), queries columns 16 nt + dcol()
    const bool full = jw + 16 <= nk && nq == BR && j0 + jw + 15 <= i0 + off;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int qcol = 16 * nt + dcol();
      f32x4 x;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int jr = jw + drow(i);
        const bool vis = full || (jr < nk && qcol < nq && j0 + jr <= i0 + qcol + off);
        const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(S[nt][i], c2, -lbq[nt])) : 0.f;
        x[i] = WANT_DK ? p * (dP[nt][i] - dlq[nt]) : p;
      }
      put_pt(sm.u.in.pt[w], nt, x);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    // dv += P^T dO, or dk += dS^T Q
    const bf16* bpan = WANT_DK ? &sm.u.in.q[0][0] : &sm.u.in.dO[0][0];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 pa = fragT(sm.u.in.pt[w], PT_LD, 0, 32 * kk);
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) acc[dt] = mfma16(pa, fragT(bpan, A_LD, 16 * dt, 32 * kk), acc[dt]);
    }
  }
  __syncthreads();
  const float mul = WANT_DK ? a.scale : 1.f;
  if (!F32) {
    // waves 0-3 through the q block, 4-7 through the dO block
    write_rows_bf16(w < 4 ? sm.u.in.q : sm.u.in.dO, w & 3, acc, mul, reinterpret_cast<bf16*>(out),
                    u0 + 64 * (w >> 2), nk - 64 * (w >> 2), a.Hkv, g);
  } else {
    // the two halves of the block in turn through the fp32 rows
    for (int half = 0; half < 2; ++half) {
      if (half) __syncthreads();
      if ((w >> 2) == half)
#pragma unroll
        for (int dt = 0; dt < 16; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sm.u.out[16 * (w & 3) + drow(i)][16 * dt + dcol()] = acc[dt][i] * mul;
      __syncthreads();
      const int nv = nk - 64 * half;
      for (int e = threadIdx.x; e < BR * AD / 4; e += 512) {
        const int r = e >> 6, c4 = (e & 63) * 4;
        if (r < nv)
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) +
                                    ((u0 + 64 * half + r) * a.Hkv + g) * AD + c4) =
              *reinterpret_cast<const f32x4*>(&sm.u.out[r][c4]);
      }
    }
  }
}

// ------------------------------------------------------------------ row map
// Pairs (destination row, key) packed as row << 32 | key; a key whose row is
// outside [0, R) gets row R and sorts last. Keys are distinct, so the order
// is total and every sort gives the same sequence.
constexpr int SORT_TILE = 2048;

__global__ __launch_bounds__(256) void rowmap_keys_kernel(int64_t n, const int32_t* __restrict__ map,
                                                         int64_t R, uint64_t* __restrict__ out) {
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < n; j += (int64_t)gridDim.x * 256) {
    const int64_t r = map[j];
    const uint64_t rr = (r >= 0 && r < R) ? (uint64_t)r : (uint64_t)R;
    out[j] = rr << 32 | (uint64_t)j;
  }
}

// Bitonic sort of each tile of SORT_TILE pairs in LDS (the tail padded with
// the largest value and not written back).
__global__ __launch_bounds__(256) void rowmap_tile_sort_kernel(int64_t n, uint64_t* __restrict__ x) {
  __shared__ uint64_t t[SORT_TILE];
  const int64_t base = (int64_t)blockIdx.x * SORT_TILE;
  for (int i = threadIdx.x; i < SORT_TILE; i += 256)
    t[i] = base + i < n ? x[base + i] : ~(uint64_t)0;
  __syncthreads();
  for (int size = 2; size <= SORT_TILE; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < SORT_TILE / 2; i += 256) {
        const int lo = 2 * i - (i & (stride - 1)), hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint64_t a = t[lo], b = t[hi];
        if ((a > b) == up) t[lo] = b, t[hi] = a;
      }
      __syncthreads();
    }
  for (int i = threadIdx.x; i < SORT_TILE; i += 256)
    if (base + i < n) x[base + i] = t[i];
}

// One merge pass: sorted runs of `width` become runs of 2 width. Each element
// finds its place by counting the smaller elements of the other run.
__global__ __launch_bounds__(256) void rowmap_merge_kernel(int64_t n, int64_t width,
                                                          const uint64_t* __restrict__ x,
                                                          uint64_t* __restrict__ y) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int64_t pair0 = e / (2 * width) * (2 * width);
    const int64_t a0 = pair0, a1 = pair0 + width < n ? pair0 + width : n;
    const int64_t b0 = a1, b1 = pair0 + 2 * width < n ? pair0 + 2 * width : n;
    const uint64_t key = x[e];
    const bool inA = e < a1;
    int64_t lo = inA ? b0 : a0, hi = inA ? b1 : a1;     // first element >= key in the other run
    while (lo < hi) {
      const int64_t mid = (lo + hi) >> 1;
      if (x[mid] < key) lo = mid + 1;
      else hi = mid;
    }
    const int64_t pos = pair0 + (inA ? e - a0 : e - b0) + (lo - (inA ? b0 : a0));
    y[pos] = key;
  }
}

// Per run of one destination row in the sorted pairs: the window rows of its
// keys summed in key order, added once to the destination. A thread owns four
// channels of one key head.
__global__ __launch_bounds__(256) void rowmap_add_kernel(int64_t n, int64_t R, int Hkv,
                                                        const uint64_t* __restrict__ x,
                                                        const float* __restrict__ wk,
                                                        const float* __restrict__ wv,
                                                        float* __restrict__ dk,
                                                        float* __restrict__ dv) {
  const int64_t cols = (int64_t)Hkv * (AD / 4);
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n * cols;
       e += (int64_t)gridDim.x * 256) {
    const int64_t p = e / cols, c = e - p * cols;
    const int64_t r = (int64_t)(x[p] >> 32);
    if (r >= R || (p > 0 && (int64_t)(x[p - 1] >> 32) == r)) continue;
    f32x4 sk = zero4(), sv = zero4();
    for (int64_t u = p; u < n && (int64_t)(x[u] >> 32) == r; ++u) {
      const int64_t j = (int64_t)(x[u] & 0xffffffffu);
      sk += *reinterpret_cast<const f32x4*>(wk + j * cols * 4 + 4 * c);
      sv += *reinterpret_cast<const f32x4*>(wv + j * cols * 4 + 4 * c);
    }
    f32x4* pk = reinterpret_cast<f32x4*>(dk + r * cols * 4 + 4 * c);
    f32x4* pv = reinterpret_cast<f32x4*>(dv + r * cols * 4 + 4 * c);
    *pk = *pk + sk;
    *pv = *pv + sv;
  }
}

}  // namespace attn
}  // namespace kda

// ------------------------------------------------------------------ host
namespace {

using kda::fail;
namespace A = kda::attn;

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

constexpr int64_t MAX_BLOCKS = (int64_t)1 << 22;    // workgroups of a launch (x 512 threads < 2^32)

kda_status check(const kda_attn_problem* p) {
  if (!p) return fail(KDA_ERR_INVALID_ARGUMENT, "problem is NULL");
  if (p->Tq < 0 || p->Tk < 0 || p->Tq > ((int64_t)1 << 30) || p->Tk > ((int64_t)1 << 30))
    return fail(KDA_ERR_INVALID_ARGUMENT, "Tq = %lld, Tk = %lld outside [0, 2^30]",
                (long long)p->Tq, (long long)p->Tk);
  if (p->num_seqs < 1 || p->num_seqs > (1 << 24))
    return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs = %d outside [1, 2^24]", p->num_seqs);
  if (p->Hq < 1 || p->Hkv < 1)
    return fail(KDA_ERR_INVALID_ARGUMENT, "Hq = %d, Hkv = %d: need at least one head", p->Hq, p->Hkv);
  if (p->Hq % p->Hkv)
    return fail(KDA_ERR_INVALID_ARGUMENT, "Hq = %d is not a multiple of Hkv = %d", p->Hq, p->Hkv);
  if (p->Hq > 65535) return fail(KDA_ERR_UNSUPPORTED, "Hq = %d: more than 65535 heads", p->Hq);
  if (p->D != 256) return fail(KDA_ERR_UNSUPPORTED, "D = %d: this build serves 256", p->D);
  if (!(std::isfinite(p->scale) && p->scale > 0.f))
    return fail(KDA_ERR_INVALID_ARGUMENT, "scale must be finite and positive");
  if ((p->Tq / 64 + p->num_seqs) * (int64_t)p->Hq > MAX_BLOCKS ||
      (p->Tk / 128 + p->num_seqs) * (int64_t)p->Hkv > MAX_BLOCKS)
    return fail(KDA_ERR_UNSUPPORTED, "more than 2^22 workgroups (row blocks x heads)");
  return KDA_OK;
}

#define REQ(ptr, name)                                                                  \
  do {                                                                                  \
    if (!(ptr)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is NULL", name);              \
    if (!al16(ptr)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name); \
  } while (0)

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

struct Layout {
  A::Dims d;
  size_t q_tab, k_tab, delta, fwd_end, bwd_end;
  size_t win_k, win_v, keys0, keys1, map_end;
};

Layout layout_of(const kda_attn_problem* p) {
  Layout L;
  L.d.Tq = p->Tq;
  L.d.Tk = p->Tk;
  L.d.S = p->num_seqs;
  L.d.Hq = p->Hq;
  L.d.Hkv = p->Hkv;
  L.d.grp = p->Hq / p->Hkv;
  L.d.NCq = (int)(p->Tq / 64 + p->num_seqs);
  L.d.NCk = (int)(p->Tk / A::BK + p->num_seqs);
  L.d.scale = p->scale;
  auto tab = [&](int nc) { return up256(4 * (size_t)(p->num_seqs + 1)) + 2 * up256(4 * (size_t)nc); };
  L.q_tab = 0;
  L.k_tab = tab(L.d.NCq);
  L.fwd_end = L.k_tab;
  L.delta = L.k_tab + tab(L.d.NCk);
  L.bwd_end = L.delta + up256(4 * (size_t)p->Tq * p->Hq);
  const size_t win = up256(4 * (size_t)p->Tk * p->Hkv * A::AD);
  L.win_k = L.bwd_end;
  L.win_v = L.win_k + win;
  L.keys0 = L.win_v + win;
  L.keys1 = L.keys0 + up256(8 * (size_t)p->Tk);
  L.map_end = L.keys1 + up256(8 * (size_t)p->Tk);
  return L;
}

kda::ChunkTable table_at(char* base, int S, int nc) {
  kda::ChunkTable ct{};
  ct.doc_c0 = reinterpret_cast<int32_t*>(base);
  ct.tok = reinterpret_cast<int32_t*>(base + up256(4 * (size_t)(S + 1)));
  ct.len = reinterpret_cast<int32_t*>(base + up256(4 * (size_t)(S + 1)) + up256(4 * (size_t)nc));
  return ct;
}

kda::Dims map_dims(int64_t T, int S, int nc) {
  kda::Dims d{};
  d.T = T;
  d.N = S;
  d.NC = nc;
  return d;
}

unsigned grid_for(int64_t items) {
  const int64_t b = (items + 255) / 256;
  return (unsigned)(b < 1 ? 1 : (b > 65536 ? 65536 : b));
}

}  // namespace

extern "C" {

size_t kda_attn_workspace_bytes(const kda_attn_problem* p, int stage, int64_t dkv_dst_rows) {
  if (check(p) != KDA_OK) return 0;
  const Layout L = layout_of(p);
  switch (stage) {
    case 0: return L.fwd_end;
    case 1: return L.bwd_end;
    case 2: return (dkv_dst_rows >= 0 && dkv_dst_rows < ((int64_t)1 << 31)) ? L.map_end : 0;
    default: return 0;
  }
}

kda_status kda_attn_fwd(const kda_attn_problem* p, const void* q, const void* k, const void* v,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* o,
                        float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  kda_status st = check(p);
  if (st != KDA_OK) return st;
  if (p->Tq == 0) return KDA_OK;
  REQ(q, "q");
  REQ(cu_seqlens_q, "cu_seqlens_q");
  REQ(cu_seqlens_k, "cu_seqlens_k");
  REQ(o, "o");
  if (lse && !al16(lse)) return fail(KDA_ERR_INVALID_ARGUMENT, "lse is not 16-byte aligned");
  if (p->Tk > 0) {
    REQ(k, "k");
    REQ(v, "v");
  }
  REQ(workspace, "workspace");
  const Layout L = layout_of(p);
  if (workspace_bytes < L.fwd_end)
    return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes,
                L.fwd_end);
  char* ws = static_cast<char*>(workspace);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const kda::ChunkTable qt = table_at(ws + L.q_tab, p->num_seqs, L.d.NCq);
  hipError_t e = kda::launch_chunk_map(map_dims(p->Tq, p->num_seqs, L.d.NCq), cu_seqlens_q, qt, hs);
  if (e == hipSuccess) {
    const auto* qb = static_cast<const kda::bf16*>(q);
    const auto* kb = static_cast<const kda::bf16*>(k);
    const auto* vb = static_cast<const kda::bf16*>(v);
    auto* ob = static_cast<kda::bf16*>(o);
    if (L.d.grp % 2 == 0)
      hipLaunchKernelGGL(A::attn_fwd_kernel<2>, dim3(L.d.NCq * (p->Hq / 2)), dim3(512), 0, hs, L.d,
                         qt, cu_seqlens_q, cu_seqlens_k, qb, kb, vb, ob, lse);
    else
      hipLaunchKernelGGL(A::attn_fwd_kernel<1>, dim3(L.d.NCq * p->Hq), dim3(256), 0, hs, L.d, qt,
                         cu_seqlens_q, cu_seqlens_k, qb, kb, vb, ob, lse);
    e = hipGetLastError();
  }
  if (e != hipSuccess)
    return fail(KDA_ERR_DEVICE, "attention forward launch failed: %s", hipGetErrorString(e));
  return KDA_OK;
}

kda_status kda_attn_bwd(const kda_attn_problem* p, const void* q, const void* k, const void* v,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, const void* o,
                        const float* lse, const void* dO, void* dq, void* dk, void* dv,
                        int dkv_form, const int32_t* dkv_row_map, int64_t dkv_dst_rows,
                        void* workspace, size_t workspace_bytes, void* stream) {
  kda_status st = check(p);
  if (st != KDA_OK) return st;
  if (dkv_form != KDA_ATTN_DKV_BF16 && dkv_form != KDA_ATTN_DKV_F32 &&
      dkv_form != KDA_ATTN_DKV_F32_ADD)
    return fail(KDA_ERR_INVALID_ARGUMENT, "dkv_form = %d is not one of 0, 1, 2", dkv_form);
  const bool add = dkv_form == KDA_ATTN_DKV_F32_ADD;
  if (add && (dkv_dst_rows < 0 || dkv_dst_rows >= ((int64_t)1 << 31)))
    return fail(KDA_ERR_INVALID_ARGUMENT, "dkv_dst_rows = %lld outside [0, 2^31)",
                (long long)dkv_dst_rows);
  if (p->Tq == 0 && p->Tk == 0) return KDA_OK;
  REQ(cu_seqlens_q, "cu_seqlens_q");
  REQ(cu_seqlens_k, "cu_seqlens_k");
  if (p->Tq > 0) {
    REQ(q, "q");
    REQ(o, "o");
    REQ(lse, "lse");
    REQ(dO, "dO");
    REQ(dq, "dq");
  }
  const bool keys = p->Tk > 0 && (!add || dkv_dst_rows > 0);
  if (p->Tk > 0) {
    REQ(k, "k");
    REQ(v, "v");
  }
  if (keys) {
    REQ(dk, "dk");
    REQ(dv, "dv");
    if (add) REQ(dkv_row_map, "dkv_row_map");
  }
  REQ(workspace, "workspace");
  const Layout L = layout_of(p);
  const size_t need = add ? L.map_end : L.bwd_end;
  if (workspace_bytes < need)
    return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes,
                need);
  char* ws = static_cast<char*>(workspace);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const kda::ChunkTable qt = table_at(ws + L.q_tab, p->num_seqs, L.d.NCq);
  const kda::ChunkTable kt = table_at(ws + L.k_tab, p->num_seqs, L.d.NCk);
  float* delta = reinterpret_cast<float*>(ws + L.delta);
  const auto* qb = static_cast<const kda::bf16*>(q);
  const auto* kb = static_cast<const kda::bf16*>(k);
  const auto* vb = static_cast<const kda::bf16*>(v);
  const auto* dob = static_cast<const kda::bf16*>(dO);
  hipError_t e = kda::launch_chunk_map(map_dims(p->Tq, p->num_seqs, L.d.NCq), cu_seqlens_q, qt, hs);
  if (e == hipSuccess)
    e = kda::launch_chunk_map(map_dims(p->Tk, p->num_seqs, L.d.NCk), cu_seqlens_k, kt, hs, A::BK);
  if (e == hipSuccess && p->Tq > 0) {
    const int64_t rows = p->Tq * p->Hq;
    hipLaunchKernelGGL(A::attn_delta_kernel, dim3(grid_for(rows * 64)), dim3(256), 0, hs, rows,
                       static_cast<const kda::bf16*>(o), dob, delta);
    if (L.d.grp % 2 == 0)
      hipLaunchKernelGGL(A::attn_dq_kernel<2>, dim3(L.d.NCq * (p->Hq / 2)), dim3(512), 0, hs, L.d, qt,
                         cu_seqlens_q, cu_seqlens_k, qb, kb, vb, dob, lse, delta,
                         static_cast<kda::bf16*>(dq));
    else
      hipLaunchKernelGGL(A::attn_dq_kernel<1>, dim3(L.d.NCq * p->Hq), dim3(256), 0, hs, L.d, qt,
                         cu_seqlens_q, cu_seqlens_k, qb, kb, vb, dob, lse, delta,
                         static_cast<kda::bf16*>(dq));
    e = hipGetLastError();
  }
  if (e == hipSuccess && keys) {
    void* wk = add ? ws + L.win_k : dk;
    void* wv = add ? ws + L.win_v : dv;
    const dim3 grid((unsigned)((int64_t)L.d.NCk * p->Hkv));
    if (dkv_form == KDA_ATTN_DKV_BF16) {
      hipLaunchKernelGGL((A::attn_dkdv_kernel<false, false>), grid, dim3(512), 0, hs, L.d, qt, kt,
                         cu_seqlens_q, cu_seqlens_k, qb, kb, vb, dob, lse, delta, wv);
      hipLaunchKernelGGL((A::attn_dkdv_kernel<true, false>), grid, dim3(512), 0, hs, L.d, qt, kt,
                         cu_seqlens_q, cu_seqlens_k, qb, kb, vb, dob, lse, delta, wk);
    } else {
      hipLaunchKernelGGL((A::attn_dkdv_kernel<false, true>), grid, dim3(512), 0, hs, L.d, qt, kt,
                         cu_seqlens_q, cu_seqlens_k, qb, kb, vb, dob, lse, delta, wv);
      hipLaunchKernelGGL((A::attn_dkdv_kernel<true, true>), grid, dim3(512), 0, hs, L.d, qt, kt,
                         cu_seqlens_q, cu_seqlens_k, qb, kb, vb, dob, lse, delta, wk);
    }
    e = hipGetLastError();
    if (e == hipSuccess && add) {
      const int64_t n = p->Tk;
      auto* x0 = reinterpret_cast<uint64_t*>(ws + L.keys0);
      auto* x1 = reinterpret_cast<uint64_t*>(ws + L.keys1);
      hipLaunchKernelGGL(A::rowmap_keys_kernel, dim3(grid_for(n)), dim3(256), 0, hs, n, dkv_row_map,
                         dkv_dst_rows, x0);
      hipLaunchKernelGGL(A::rowmap_tile_sort_kernel,
                         dim3((unsigned)((n + A::SORT_TILE - 1) / A::SORT_TILE)), dim3(256), 0, hs,
                         n, x0);
      for (int64_t width = A::SORT_TILE; width < n; width *= 2) {
        hipLaunchKernelGGL(A::rowmap_merge_kernel, dim3(grid_for(n)), dim3(256), 0, hs, n, width,
                           x0, x1);
        std::swap(x0, x1);
      }
      hipLaunchKernelGGL(A::rowmap_add_kernel, dim3(grid_for(n * p->Hkv * (A::AD / 4))), dim3(256),
                         0, hs, n, dkv_dst_rows, p->Hkv, x0,
                         reinterpret_cast<const float*>(ws + L.win_k),
                         reinterpret_cast<const float*>(ws + L.win_v), static_cast<float*>(dk),
                         static_cast<float*>(dv));
      e = hipGetLastError();
    }
  }
  if (e != hipSuccess)
    return fail(KDA_ERR_DEVICE, "attention backward launch failed: %s", hipGetErrorString(e));
  return KDA_OK;
}

}  // extern "C"
