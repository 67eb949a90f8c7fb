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
// Fast-decay safety (g <= 0, so G falls along the chunk). e^(G_r - G_i) is
// formed from two factors that never overflow. A tile of rows in block I and
// columns in block J < I uses the reference rho = G at the end of block J:
// x_r e^(G_r - rho) <= 1 and k_i e^(rho - G_i) <= 1. A diagonal tile whose
// decay span (G before the block minus G at its last row) is at most SPAN_MAX
// in every channel uses the midpoint of that range as rho, so both factors lie
// within e^(+-SPAN_MAX/2) and their bf16 lo planes stay normal. A wider
// diagonal tile is summed in fp32 without exponentials of differences: down
// column i the factor e^(G_r - G_i) is the running product of the per-step
// decays e^(g_r), r = i+1 .. 15, which never exceeds 1 and underflows
// gracefully.
//
// A calm chunk (span at most SPAN_MAX in every channel) uses one reference
// for all of its tiles, rho = G_last / 2, so both factors lie within
// e^(+-SPAN_MAX/2): the k operand k^ e^(rho - G) is built once per row into an
// LDS panel and each wave builds its rows' x operands for half of the channels
// once, then runs every tile of its row block.
//
// Besides the saved fp32 matrices, the kernel writes the operand panels (-Kd,
// scale Qd, Ke^T, Tb, scale A_qk as bf16 hi/lo planes and e^(G_last)) that the
// two state scans and the output kernel stream; the lo planes of -Kd and Tb
// only when a backward will read them.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr float SPAN_MAX = 120.f;
constexpr int kPrepWorkgroups = 256;     // MI355X compute units

#ifndef KDA_SPLIT_P1
#define KDA_SPLIT_P1 SPLIT_AB    // A_kk = X_k Y^T, A_qk = X_q Y^T
#endif

__global__ __launch_bounds__(256) void chunk_map_kernel(const int32_t* __restrict__ cu, int N,
                                                        int64_t T, int NC, int cl, ChunkTable ct) {
  // documents are taken 256 at a time: a prefix sum of their chunk counts
  // gives each its first chunk, then every thread fills chunk entries c,
  // c + 256, ... of the batch, finding the document of entry c by a binary
  // search over the batch's inclusive chunk ends
  __shared__ int32_t scan[256], c_end[256], d_tok[256], d_end[256];
  const int t = threadIdx.x;
  int carry = 0;
  for (int base = 0; base < N; base += 256) {
    const int d = base + t;
    const int nb = min(256, N - base);
    int a = 0, b = 0, cnt = 0;
    if (d < N) {
      int64_t ca = cu[d], cb = cu[d + 1];
      ca = ca < 0 ? 0 : (ca > T ? T : ca);
      cb = cb < ca ? ca : (cb > T ? T : cb);
      a = (int)ca;
      b = (int)cb;
      cnt = (b - a + cl - 1) / cl;
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
    c_end[t] = carry + scan[t];
    d_tok[t] = a - cl * c0;       // first token of chunk c of this document: d_tok + cl c
    d_end[t] = b;
    if (d < N) ct.doc_c0[d] = min(c0, NC);
    __syncthreads();
    const int cstop = min(carry + total, NC);
    for (int c = carry + t; c < cstop; c += 256) {
      int lo = 0, hi = nb - 1;    // smallest document of the batch whose chunk end exceeds c
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (c_end[mid] > c) hi = mid;
        else lo = mid + 1;
      }
      const int tok = d_tok[lo] + cl * c;
      ct.tok[c] = tok;
      ct.len[c] = min(cl, d_end[lo] - tok);
    }
    carry += total;
    __syncthreads();
  }
  if (t == 0) ct.doc_c0[N] = min(carry, NC);
}

hipError_t launch_chunk_map(const Dims& d, const int32_t* cu, const ChunkTable& ct,
                            hipStream_t s, int block) {
  hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(256), 0, s, cu, d.N, d.T, d.NC, block, ct);
  return hipGetLastError();
}

// Segments: document d's chunks [doc_c0[d], doc_c0[d+1]) cut into runs of L
// chunks (one segment per document, empty or not, when L = 0). Documents are
// taken 256 at a time as in the chunk map: a prefix sum of their segment
// counts gives each its first segment, then segment entries are filled by a
// binary search over the batch's inclusive segment ends.
__global__ __launch_bounds__(256) void seg_map_kernel(int N, int L, int NS, ChunkTable ct) {
  __shared__ int32_t scan[256], s_end[256];
  const int t = threadIdx.x;
  int carry = 0;
  for (int base = 0; base < N; base += 256) {
    const int d = base + t;
    const int nb = min(256, N - base);
    int cnt = 0;
    if (d < N) {
      const int nch = max(0, ct.doc_c0[d + 1] - ct.doc_c0[d]);
      cnt = L > 0 ? (nch + L - 1) / L : 1;
    }
    scan[t] = cnt;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int v = t >= off ? scan[t - off] : 0;
      __syncthreads();
      scan[t] += v;
      __syncthreads();
    }
    const int total = scan[255];
    s_end[t] = carry + scan[t];
    if (d < N) ct.seg_doc0[d] = min(carry + scan[t] - cnt, NS);
    __syncthreads();
    const int sstop = min(carry + total, NS);
    for (int sg = carry + t; sg < sstop; sg += 256) {
      int lo = 0, hi = nb - 1;      // first document of the batch whose segment end exceeds sg
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_end[mid] > sg) hi = mid;
        else lo = mid + 1;
      }
      ct.seg_doc[sg] = base + lo;
    }
    carry += total;
    __syncthreads();
  }
  if (t == 0) ct.seg_doc0[N] = min(carry, NS);
}

hipError_t launch_seg_map(const Dims& d, const ChunkTable& ct, hipStream_t s) {
  hipLaunchKernelGGL(seg_map_kernel, dim3(1), dim3(256), 0, s, d.N, d.L, d.NS, ct);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The prep kernel: 512 threads (8 waves). For loads and the elementwise
// panels, thread t owns row rA = t >> 3 and channels cA .. cA+15 (cA = 16 (t & 7)).
constexpr int NT_PREP = 512;
constexpr int GP_LD = HD + 4;     // fp32 rows of G (16-byte aligned rows)
constexpr int XS_LD = HD + 8;     // bf16 rows of the raw q, k
constexpr int F_LD = CL + 1;      // fp32 64 x 64 matrices

struct __attribute__((aligned(16))) PrepSmem {
  float G[CL][GP_LD];
  bf16 qs[CL][XS_LD], ks[CL][XS_LD];   // raw q, k (rows >= n repeat row n - 1)
  float Akk[CL][F_LD], Aqk[CL][F_LD];
  float Tm[CL][F_LD];
  float Z[3][16][17];
  float Gref[5][HD];       // G before block I (I = 0..3) and G_last (I = 4)
  union {
    struct {
      float qtot[4][HD];   // cumsum carries of the row quarters
      float nrm[2][8][CL]; // L2 partial sums
    } s;
    float E[CL][HD];       // e^(g) per row and channel, once the above are dead
    bf16 Y[2][CL * HD];    // calm chunk: k^ e^(rho - G), hi and lo, rows of 16-byte
                           // chunks XOR-swizzled by row
  } u;
  float rq[CL], rk[CL], beta[CL];
  int wide[4];             // diagonal block I has a span > SPAN_MAX
  int notcalm;             // some channel's chunk span exceeds SPAN_MAX
};

// Element offset of (row, channel c) in a swizzled 64 x 128 bf16 plane: 16-byte
// chunk c / 8 of the row sits at position (c / 8) ^ (row & 15).
KDA_DEV int yswz(int row, int c) { return row * HD + ((((c >> 3) ^ (row & 15))) << 3) + (c & 7); }

// Off-diagonal tile (I, J), J < I, of the lower triangle of 16 x 16 blocks.
KDA_DEV void offdiag_tile(int item, int& I, int& J) {
  I = item < 1 ? 1 : item < 3 ? 2 : 3;
  J = item - I * (I - 1) / 2;
}

// The k and q fragments of one row share their factors e^(G - rho).
KDA_DEV void decayed_frag2(const PrepSmem& sm, float rk, float rq, int row, int c,
                           const float* ra, const float* rb, bf16x8& kh, bf16x8& kl,
                           bf16x8& qh, bf16x8& ql) {
  const f32x4 g0 = *reinterpret_cast<const f32x4*>(&sm.G[row][c]);
  const f32x4 g1 = *reinterpret_cast<const f32x4*>(&sm.G[row][c + 4]);
  const f32x4 a0 = *reinterpret_cast<const f32x4*>(ra + c);
  const f32x4 a1 = *reinterpret_cast<const f32x4*>(ra + c + 4);
  const f32x4 b0 = *reinterpret_cast<const f32x4*>(rb + c);
  const f32x4 b1 = *reinterpret_cast<const f32x4*>(rb + c + 4);
  const bf16x8 kv = *reinterpret_cast<const bf16x8*>(&sm.ks[row][c]);
  const bf16x8 qv = *reinterpret_cast<const bf16x8*>(&sm.qs[row][c]);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float gj = j < 4 ? g0[j] : g1[j - 4];
    const float rj = 0.5f * ((j < 4 ? a0[j] : a1[j - 4]) + (j < 4 ? b0[j] : b1[j - 4]));
    const float e = fexp(gj - rj);
    const float vk = bf2f(kv[j]) * rk * e, vq = bf2f(qv[j]) * rq * e;
    kh[j] = f2bf(vk);
    kl[j] = f2bf(vk - bf2f(kh[j]));
    qh[j] = f2bf(vq);
    ql[j] = f2bf(vq - bf2f(qh[j]));
  }
}

// One 8-channel MFMA fragment of x e^(+-(G - rho)) for row `row`, channels
// c .. c+7, split into hi and lo planes, with rho = (ra + rb) / 2 (exactly ra
// when ra == rb). sgn = +1: x e^(G - rho); -1: x e^(rho - G).
KDA_DEV void decayed_frag(const PrepSmem& sm, const bf16 (*x)[XS_LD], float rx, int row, int c,
                          const float* ra, const float* rb, float sgn, bf16x8& hi, bf16x8& lo) {
  const f32x4 g0 = *reinterpret_cast<const f32x4*>(&sm.G[row][c]);
  const f32x4 g1 = *reinterpret_cast<const f32x4*>(&sm.G[row][c + 4]);
  const f32x4 a0 = *reinterpret_cast<const f32x4*>(ra + c);
  const f32x4 a1 = *reinterpret_cast<const f32x4*>(ra + c + 4);
  const f32x4 b0 = *reinterpret_cast<const f32x4*>(rb + c);
  const f32x4 b1 = *reinterpret_cast<const f32x4*>(rb + c + 4);
  const bf16x8 xv = *reinterpret_cast<const bf16x8*>(&x[row][c]);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float gj = j < 4 ? g0[j] : g1[j - 4];
    const float rj = 0.5f * ((j < 4 ? a0[j] : a1[j - 4]) + (j < 4 ? b0[j] : b1[j - 4]));
    const float v = bf2f(xv[j]) * rx * fexp(sgn * (gj - rj));
    hi[j] = f2bf(v);
    lo[j] = f2bf(v - bf2f(hi[j]));
  }
}

// RAW: the gate input is the raw a (bf16) of g = -exp(A_log) softplus(a + dt_bias)
// rather than g itself (fp32); a template parameter so that neither form
// carries the other's registers through the chunk loop.
template <bool RAW>
__global__ __launch_bounds__(NT_PREP) void fwd_prep_kernel(Dims d, Inputs in, ChunkTable ct,
                                                            SavedSet sv, bf16* __restrict__ panels,
                                                            int with_lo) {
  __shared__ PrepSmem sm;
  const int h = blockIdx.y, nch = ld_const(ct.doc_c0, d.N);
  const int t = threadIdx.x, w = wave_id(), l = lane_id();
  const int H = d.H;
  const bf16* q = reinterpret_cast<const bf16*>(in.q);
  const bf16* k = reinterpret_cast<const bf16*>(in.k);
  const bf16* beta = reinterpret_cast<const bf16*>(in.beta);
  const int rA = t >> 3, cA = 16 * (t & 7);
  const int cG = t & 127, qG = t >> 7;

  // One chunk's raw inputs. Thread t: q, k of row rA, channels cA .. cA+15;
  // the gate of channel cG = t & 127, rows 16 qG .. 16 qG + 15; beta of row t.
  // The workgroup walks the chunks ci, ci + gridDim.x, ... of head h and loads
  // the next chunk's inputs while it works on the current one; the chunk
  // table entries are read one chunk earlier still, and the raw gate stays
  // bf16 until it is used, so that no wait follows the requests.
  bf16x8 q0, q1, k0, k1;
  float g[16], eg[16];
  bf16 ga[16];
  bf16 bt = f2bf(0.f);
  // Addresses: the chunk's first row is a base common to the workgroup; a
  // lane adds its row (clamped to the last one) times the row stride H * HD as
  // a 32-bit byte offset, so the 16 gate rows cost an add and a min each.
  auto load_raw = [&](int64_t u0, int un) {
    const int64_t cbase = (u0 * H + h) * HD;
    const uint32_t rs = (uint32_t)H * HD;     // elements from one row to the next
    const uint32_t oA = ((uint32_t)(rA < un ? rA : un - 1) * rs + cA) * 2u;
    q0 = ld_at(reinterpret_cast<const bf16x8*>(q + cbase), oA);
    q1 = ld_at(reinterpret_cast<const bf16x8*>(q + cbase), oA + 16u);
    k0 = ld_at(reinterpret_cast<const bf16x8*>(k + cbase), oA);
    k1 = ld_at(reinterpret_cast<const bf16x8*>(k + cbase), oA + 16u);
    const uint32_t o0 = 16u * qG * rs + cG, olast = (uint32_t)(un - 1) * rs + cG;
    if (!RAW) {
      const float* gp = reinterpret_cast<const float*>(in.gate) + cbase;
#pragma unroll
      for (int j = 0; j < 16; ++j) g[j] = ld_at(gp, 4u * min(o0 + j * rs, olast));
    } else {
      const bf16* ap = reinterpret_cast<const bf16*>(in.gate) + cbase;
#pragma unroll
      for (int j = 0; j < 16; ++j) ga[j] = ld_at(ap, 2u * min(o0 + j * rs, olast));
    }
    if (t < CL) bt = ld_at(beta + u0 * H + h, 2u * (uint32_t)(t < un ? t : un - 1) * (uint32_t)H);
  };
  int ci = blockIdx.x;
  if (ci >= nch) return;
  const int gx = gridDim.x;
  int64_t t0 = ld_const(ct.tok, ci);
  int n = ld_const(ct.len, ci);
  load_raw(t0, n);
  // raw gate parameters of this head and thread channel cG
  const float ea = RAW ? __expf(in.A_log[h]) : 0.f;
  const float dtb = RAW ? in.dt_bias[h * HD + cG] : 0.f;
  // table entry of the next chunk this workgroup takes (the last chunk when
  // there is none: its loads are then repeated, never used)
  int64_t nt0 = ld_const(ct.tok, min(ci + gx, nch - 1));
  int nn = ld_const(ct.len, min(ci + gx, nch - 1));
  // nothing is in flight when the loop is entered, so the waits counted at
  // its top follow the steady state (loads requested before the stores of
  // the previous chunk) and not the shorter entry path
  __builtin_amdgcn_s_waitcnt(0);
  for (;;) {
  // indices re-derived from an opaque copy of the thread id in every
  // iteration: otherwise the unrolled phases' LDS addresses are hoisted out of
  // the loop and held in registers across it
  int tt = threadIdx.x;
  asm volatile("" : "+v"(tt));
  const int t = tt, w = tt >> 6, l = tt & 63;
  const int rA = t >> 3, cA = 16 * (t & 7);
  const int cG = t & 127, qG = t >> 7;
  const int64_t ch = (int64_t)ci * H + h;

  // ---- 1. this chunk's raw inputs into LDS, L2 partial sums
  if (t < CL) sm.beta[t] = t < n ? bf2f(bt) : 0.f;
  *reinterpret_cast<bf16x8*>(&sm.qs[rA][cA]) = q0;
  *reinterpret_cast<bf16x8*>(&sm.qs[rA][cA + 8]) = q1;
  *reinterpret_cast<bf16x8*>(&sm.ks[rA][cA]) = k0;
  *reinterpret_cast<bf16x8*>(&sm.ks[rA][cA + 8]) = k1;
  // L2 row sums: partial over this thread's 16 channels
  {
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float a = bf2f(j < 8 ? q0[j] : q1[j - 8]), b = bf2f(j < 8 ? k0[j] : k1[j - 8]);
      sq += a * a;
      sk += b * b;
    }
    sm.u.s.nrm[0][t & 7][rA] = sq;
    sm.u.s.nrm[1][t & 7][rA] = sk;
  }
  // ---- 2. chunk-local cumsum of g in registers (16 rows per thread), then
  // the carry of the earlier row quarters
  {
    // no fused multiply-adds here: the per-chunk backward rebuilds G from the
    // gate input with the same operations and must round alike
#pragma clang fp contract(off)
    float run = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      float x = RAW ? bf2f(ga[j]) : g[j];
      if (RAW) x = -ea * softplus(x + dtb);
      x = (16 * qG + j < n) ? x : 0.f;
      run += x;
      g[j] = run;
      eg[j] = fexp(x);
    }
    sm.u.s.qtot[qG][cG] = run;
  }
  if (t < 4) sm.wide[t] = 0;
  if (t == 4) sm.notcalm = 0;
  __syncthreads();
  {
    float carry = 0.f;
    for (int j = 0; j < qG; ++j) carry += sm.u.s.qtot[j][cG];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = 16 * qG + j;
      const float Gx = g[j] + carry;
      sm.G[r][cG] = Gx;               // rows >= n hold G[n-1] (their g is 0)
    }
    // the chunk's span in this channel: 0 (before the first row) minus G_last
    if (qG == 3 && -(g[15] + carry) > SPAN_MAX) sm.notcalm = 1;
    if (t < CL) {
      float a = 0.f, b = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        a += sm.u.s.nrm[0][j][t];
        b += sm.u.s.nrm[1][j][t];
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
  }
  __syncthreads();
  // references: G before each 16-row block and G_last; the decay span of each
  // diagonal block; the per-step decays (qtot and nrm are dead now)
  if (t < HD) {
    sm.Gref[0][t] = 0.f;
#pragma unroll
    for (int I = 1; I <= 4; ++I) sm.Gref[I][t] = sm.G[16 * I - 1][t];
#pragma unroll
    for (int I = 0; I < 4; ++I)
      if ((I == 0 ? 0.f : sm.G[16 * I - 1][t]) - sm.G[16 * I + 15][t] > SPAN_MAX) sm.wide[I] = 1;
  }
  const bool calm = !sm.notcalm;
  if (!calm) {
#pragma unroll
    for (int j = 0; j < 16; ++j) sm.u.E[16 * qG + j][cG] = eg[j];
  } else {
    // Y = k^ e^(rho - G), rho = G_last / 2: thread t, row rA, channels cA .. cA + 15
    const float rkA = sm.rk[rA];
#pragma unroll
    for (int u2 = 0; u2 < 2; ++u2) {
      const int c = cA + 8 * u2;
      const bf16x8 kv = *reinterpret_cast<const bf16x8*>(&sm.ks[rA][c]);
      bf16x8 yh, yl;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float y = bf2f(kv[j]) * rkA * fexp(0.5f * sm.G[CL - 1][c + j] - sm.G[rA][c + j]);
        yh[j] = f2bf(y);
        yl[j] = f2bf(y - bf2f(yh[j]));
      }
      *reinterpret_cast<bf16x8*>(&sm.u.Y[0][yswz(rA, c)]) = yh;
      *reinterpret_cast<bf16x8*>(&sm.u.Y[1][yswz(rA, c)]) = yl;
    }
  }
  // (the strictly-upper 16 x 16 tiles of A_kk and A_qk are never written or
  // read: they leave as zeros)
  __syncthreads();

  // ---- 3. decayed products of A_kk and A_qk, as work items spread over the
  // 8 waves: each off-diagonal tile and each calm diagonal tile is one MFMA
  // product of bf16 hi/lo operands; each wide diagonal tile is two
  // running-product units (unit u: columns p and 15 - p, p = 4u .. 4u + 3).
  if (calm) {
    // One reference for the whole chunk: each wave takes one row block I and
    // channels 64 kh .. 64 kh + 63 of every tile (I, J <= I); its x operands
    // x^ e^(G - rho) are built once, the k operands come from the Y panel.
    // The two channel halves meet in LDS in a fixed order. Waves w and w + 4
    // share a SIMD: they take row blocks I and 3 - I, 5 tiles per SIMD.
    const int I = w < 4 ? (w & 1) : 3 - (w & 1), kh = (w >> 1) & 1, ra = 16 * I + (l & 15);
    const float rqa = sm.rq[ra], rka = sm.rk[ra];
    f32x4 akk[4], aqk[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) akk[J] = aqk[J] = zero4();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c = 64 * kh + 32 * ks + 8 * (l >> 4);
      bf16x8 xk_h, xk_l, xq_h, xq_l;
      {
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(&sm.G[ra][c]);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(&sm.G[ra][c + 4]);
        const f32x4 e0 = *reinterpret_cast<const f32x4*>(&sm.G[CL - 1][c]);
        const f32x4 e1 = *reinterpret_cast<const f32x4*>(&sm.G[CL - 1][c + 4]);
        const bf16x8 kv = *reinterpret_cast<const bf16x8*>(&sm.ks[ra][c]);
        const bf16x8 qv = *reinterpret_cast<const bf16x8*>(&sm.qs[ra][c]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float gj = j < 4 ? g0[j] : g1[j - 4];
          const float rj = 0.5f * (j < 4 ? e0[j] : e1[j - 4]);
          const float e = fexp(gj - rj);
          const float vk = bf2f(kv[j]) * rka * e, vq = bf2f(qv[j]) * rqa * e;
          xk_h[j] = f2bf(vk);
          xk_l[j] = f2bf(vk - bf2f(xk_h[j]));
          xq_h[j] = f2bf(vq);
          xq_l[j] = f2bf(vq - bf2f(xq_h[j]));
        }
      }
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        if (J <= I) {
          const int yo = yswz(16 * J + (l & 15), c);
          const bf16x8 y_h = *reinterpret_cast<const bf16x8*>(&sm.u.Y[0][yo]);
          const bf16x8 y_l = *reinterpret_cast<const bf16x8*>(&sm.u.Y[1][yo]);
          if (KDA_SPLIT_P1 & SPLIT_A) {
            akk[J] = mfma16(xk_l, y_h, akk[J]);
            aqk[J] = mfma16(xq_l, y_h, aqk[J]);
          }
          if (KDA_SPLIT_P1 & SPLIT_B) {
            akk[J] = mfma16(xk_h, y_l, akk[J]);
            aqk[J] = mfma16(xq_h, y_l, aqk[J]);
          }
          akk[J] = mfma16(xk_h, y_h, akk[J]);
          aqk[J] = mfma16(xq_h, y_h, aqk[J]);
        }
      }
    }
    // channels 0..63 (kh = 0) first, then kh = 1 adds channels 64..127 and masks
    if (kh == 0) {
#pragma unroll
      for (int J = 0; J < 4; ++J)
        if (J <= I) {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int r = 16 * I + drow(i4), i = 16 * J + dcol();
            sm.Akk[r][i] = akk[J][i4];
            sm.Aqk[r][i] = aqk[J][i4];
          }
        }
    }
    __syncthreads();
    if (kh == 1) {
#pragma unroll
      for (int J = 0; J < 4; ++J)
        if (J <= I) {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int r = 16 * I + drow(i4), i = 16 * J + dcol();
            const float vk = sm.Akk[r][i] + akk[J][i4], vq = sm.Aqk[r][i] + aqk[J][i4];
            sm.Akk[r][i] = (i < r) ? vk : 0.f;
            sm.Aqk[r][i] = (i <= r) ? vq : 0.f;
          }
        }
    }
  } else {
    int wide[4], n_wide = 0;
  #pragma unroll
    for (int I = 0; I < 4; ++I) {
      wide[I] = __builtin_amdgcn_readfirstlane(sm.wide[I]);
      n_wide += wide[I];
    }
    for (int item = w; item < 10 + n_wide; item += 8) {
      int I = 3, J, unit = -1;
      if (item < 6) {
        offdiag_tile(item, I, J);
      } else {
        int rem = item - 6;
        bool found = false;
  #pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int cnt = 1 + wide[b];
          if (!found && rem < cnt) {
            I = b;
            unit = wide[b] ? rem : -1;
            found = true;
          } else if (!found) {
            rem -= cnt;
          }
        }
        J = I;
      }
      if (unit < 0) {
        // rho: G at the end of block J (off-diagonal), else the midpoint of G
        // before block I and G at its last row
        const bool diag = I == J;
        const float* refa = diag ? sm.Gref[I] : sm.Gref[J + 1];
        const float* refb = sm.Gref[J + 1];
        const int ra = 16 * I + (l & 15), rbw = 16 * J + (l & 15);
        const float rqa = sm.rq[ra], rka = sm.rk[ra], rkb = sm.rk[rbw];
        f32x4 akk = zero4(), aqk = zero4();
  #pragma unroll
        for (int ks = 0; ks < HD / 32; ++ks) {
          const int c = 32 * ks + 8 * (l >> 4);
          bf16x8 xk_h, xk_l, xq_h, xq_l, y_h, y_l;
          decayed_frag2(sm, rka, rqa, ra, c, refa, refb, xk_h, xk_l, xq_h, xq_l);
          decayed_frag(sm, sm.ks, rkb, rbw, c, refa, refb, -1.f, y_h, y_l);
          if (KDA_SPLIT_P1 & SPLIT_A) {
            akk = mfma16(xk_l, y_h, akk);
            aqk = mfma16(xq_l, y_h, aqk);
          }
          if (KDA_SPLIT_P1 & SPLIT_B) {
            akk = mfma16(xk_h, y_l, akk);
            aqk = mfma16(xq_h, y_l, aqk);
          }
          akk = mfma16(xk_h, y_h, akk);
          aqk = mfma16(xq_h, y_h, aqk);
        }
  #pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int r = 16 * I + drow(i4), i = 16 * J + dcol();
          sm.Akk[r][i] = (i < r) ? akk[i4] : 0.f;
          sm.Aqk[r][i] = (i <= r) ? aqk[i4] : 0.f;
        }
      } else {
        // Lane (lg, cg): column pair p = 4 unit + lg, channels 8 cg .. + 7.
        // Step st walks column p for rows p .. 15 (st = 0 .. 15 - p), then
        // column 15 - p for rows 15 - p .. 15: 17 (r, i) pairs per lane group.
        const int lg = l >> 4, cg = l & 15, c = 8 * cg, b0 = 16 * I;
        const int p = 4 * unit + lg;
        auto pair_of = [&](int st, int& r, int& i) {
          const bool second = st > 15 - p;
          i = second ? 15 - p : p;
          r = second ? st - 1 : p + st;
        };
        float f[8] = {};    // k_i rk_i e^(G_r - G_i), channels c .. c+7
        // the starting values k_i rk_i of both columns, so that a step is
        // branch-free and the loads of later steps can be issued early
        float kpf[8], kzf[8];
        {
          const bf16x8 kp = *reinterpret_cast<const bf16x8*>(&sm.ks[b0 + p][c]);
          const bf16x8 kz = *reinterpret_cast<const bf16x8*>(&sm.ks[b0 + 15 - p][c]);
          const float rkp = sm.rk[b0 + p], rkz = sm.rk[b0 + 15 - p];
  #pragma unroll
          for (int j = 0; j < 8; ++j) {
            kpf[j] = bf2f(kp[j]) * rkp;
            kzf[j] = bf2f(kz[j]) * rkz;
          }
        }
        auto step = [&](int st, float& skk, float& sqk) {
          int r, i;
          pair_of(st, r, i);
          const bool restart = st == 16 - p;       // first row of column 15 - p
          // lanes cg >= 8 read their two halves in the other order, so that
          // each 16-byte read of the 16 lanes touches every bank once
          const int sw = (cg & 8) >> 1;
          const f32x4 ea = *reinterpret_cast<const f32x4*>(&sm.u.E[b0 + r][c + sw]);
          const f32x4 eb = *reinterpret_cast<const f32x4*>(&sm.u.E[b0 + r][c + 4 - sw]);
  #pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float ej = sw ? (j < 4 ? eb[j] : ea[j - 4]) : (j < 4 ? ea[j] : eb[j - 4]);
            const float fm = f[j] * ej;
            f[j] = st == 0 ? kpf[j] : restart ? kzf[j] : fm;
          }
          const bf16x8 kr = *reinterpret_cast<const bf16x8*>(&sm.ks[b0 + r][c]);
          const bf16x8 qr = *reinterpret_cast<const bf16x8*>(&sm.qs[b0 + r][c]);
          skk = sqk = 0.f;
  #pragma unroll
          for (int j = 0; j < 8; ++j) {
            skk += bf2f(kr[j]) * f[j];
            sqk += bf2f(qr[j]) * f[j];
          }
        };
        // the sums of step st (kind 0: A_kk, 1: A_qk), mirrored zero above the diagonal
        auto store = [&](int st, int kind, float v) {
          int r, i;
          pair_of(st, r, i);
          if (kind == 0) {
            sm.Akk[b0 + r][b0 + i] = r > i ? v * sm.rk[b0 + r] : 0.f;
            if (r > i) sm.Akk[b0 + i][b0 + r] = 0.f;
          } else {
            sm.Aqk[b0 + r][b0 + i] = v * sm.rq[b0 + r];
            if (r > i) sm.Aqk[b0 + i][b0 + r] = 0.f;
          }
        };
        // steps 0..15 in two groups of 8: the 16 sums of a group are reduced
        // over the 16 channel-group lanes (one DPP row), after which lane cg
        // holds the total of value cg (step cg / 2, kind cg % 2)
  #pragma unroll
        for (int gq = 0; gq < 2; ++gq) {
          float x[16];
  #pragma unroll
          for (int e = 0; e < 8; ++e) step(8 * gq + e, x[2 * e], x[2 * e + 1]);
          store(8 * gq + (cg >> 1), cg & 1, row_transpose_sum16(x, cg));
        }
        float skk, sqk;
        step(16, skk, sqk);
        skk = row_sum16(skk);
        sqk = row_sum16(sqk);
        if (cg == 0) {
          store(16, 0, skk);
          store(16, 1, sqk);
        }
      }
    }
  }
  __syncthreads();

  // the next chunk's raw inputs, in flight during the solve and the writes,
  // and the table entry of the chunk after it
  load_raw(nt0, nn);
  const int64_t nt0b = ld_const(ct.tok, min(ci + 2 * gx, nch - 1));
  const int nnb = ld_const(ct.len, min(ci + 2 * gx, nch - 1));

  // ---- 4. T = (I + Diag(beta) A_kk)^-1 by 16x16 blocks, fp32
  // (its strictly-upper 16 x 16 blocks are never written or read here: they
  // leave as zeros)
  float (*Tm)[F_LD] = sm.Tm;
  if (w < 4 && l < 16) {
    // wave w inverts diagonal block w by forward substitution, lane j taking
    // column j. Lane j first reads row j of the block of Diag(beta) A_kk into
    // registers; step r takes row r from lane r (readlane), so that no LDS
    // read waits inside the dependent chain.
    const int I = w, j = l;
    float brow[16];
    const float bj = sm.beta[16 * I + j];
#pragma unroll
    for (int i = 0; i < 16; ++i) brow[i] = bj * sm.Akk[16 * I + j][16 * I + i];
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s2 = (r == j) ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i)
        s2 -= __int_as_float(__builtin_amdgcn_readlane(__float_as_int(brow[i]), r)) * x[i];
      x[r] = s2;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Tm[16 * I + r][16 * I + j] = x[r];
  }
  __syncthreads();
  // Off-diagonal blocks by distance: T_IJ = -T_II sum_{m = J .. I-1} B_Im T_mJ
  // with B = Diag(beta) A_kk, one wave per block, on fp32 MFMA (exact
  // products, fp32 sums). Z = sum B_Im T_mJ passes through the wave's own LDS
  // rows to become the B operand of T_II Z.
#pragma unroll
  for (int dist = 1; dist < 4; ++dist) {
    if (w < 4 - dist) {
      const int J = w, I = J + dist, lr = l & 15, lk = l >> 4;
      const float bI = sm.beta[16 * I + lr];
      f32x4 z = zero4();
#pragma unroll
      for (int s4 = 0; s4 < 4 * dist; ++s4) {
        const int m = 16 * J + 4 * s4 + lk;
        z = __builtin_amdgcn_mfma_f32_16x16x4f32(bI * sm.Akk[16 * I + lr][m], Tm[m][16 * J + lr], z,
                                                 0, 0, 0);
      }
      float (*Zw)[17] = sm.Z[w];
#pragma unroll
      for (int i = 0; i < 4; ++i) Zw[4 * lk + i][lr] = z[i];
      f32x4 x = zero4();
#pragma unroll
      for (int kb = 0; kb < 16; kb += 4)
        x = __builtin_amdgcn_mfma_f32_16x16x4f32(Tm[16 * I + lr][16 * I + kb + lk], Zw[kb + lk][lr], x,
                                                 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) Tm[16 * I + 4 * lk + i][16 * J + lr] = -x[i];
    }
    __syncthreads();
  }

  // ---- 5. saved matrices (fp32) and the forward scan's operand panels
  float* Tg = sv.Tm + ch * CL * CL;
  float* Akk_g = sv.Akk + ch * CL * CL;
  bf16* P = panels ? panels + ch * (int64_t)fwd_panel::ELEMS : nullptr;
  {
    const int r = t >> 3, i8 = 8 * (t & 7);
    float tv[8], kv[8], qv[8];
    const bool upper = (i8 >> 4) > (r >> 4);    // a strictly-upper 16 x 16 block
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      tv[j] = upper ? 0.f : Tm[r][i8 + j];
      kv[j] = upper ? 0.f : sm.Akk[r][i8 + j];
      qv[j] = upper ? 0.f : sm.Aqk[r][i8 + j];
    }
    *reinterpret_cast<f32x4*>(Tg + r * CL + i8) = f32x4{tv[0], tv[1], tv[2], tv[3]};
    *reinterpret_cast<f32x4*>(Tg + r * CL + i8 + 4) = f32x4{tv[4], tv[5], tv[6], tv[7]};
    *reinterpret_cast<f32x4*>(Akk_g + r * CL + i8) = f32x4{kv[0], kv[1], kv[2], kv[3]};
    *reinterpret_cast<f32x4*>(Akk_g + r * CL + i8 + 4) = f32x4{kv[4], kv[5], kv[6], kv[7]};
    if (P) {
      bf16x8 tb, tl, ah, al;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float b = tv[j] * sm.beta[i8 + j];
        tb[j] = f2bf(b);
        tl[j] = f2bf(b - bf2f(tb[j]));
        const float a = qv[j] * d.scale;
        ah[j] = f2bf(a);
        al[j] = f2bf(a - bf2f(ah[j]));
      }
      *reinterpret_cast<bf16x8*>(P + fwd_panel::TB + r * CL + i8) = tb;
      if (with_lo) *reinterpret_cast<bf16x8*>(P + fwd_panel::TBL + r * CL + i8) = tl;
      *reinterpret_cast<bf16x8*>(P + fwd_panel::AQ + r * CL + i8) = ah;
      *reinterpret_cast<bf16x8*>(P + fwd_panel::AQ + CL * CL + r * CL + i8) = al;
    }
  }
  if (P) {
    // -Kd = -k^ e^G (hi) and scale Qd = scale q^ e^G (hi, lo): this thread's row
    const float rqA = sm.rq[rA], rkA = sm.rk[rA];
    bf16x8 kd[2], kl[2], qh[2], ql[2];
    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&sm.ks[rA][cA]);
    const bf16x8 kb = *reinterpret_cast<const bf16x8*>(&sm.ks[rA][cA + 8]);
    const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&sm.qs[rA][cA]);
    const bf16x8 qb = *reinterpret_cast<const bf16x8*>(&sm.qs[rA][cA + 8]);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float e1 = fexp(sm.G[rA][cA + j]);
      const float kx = -bf2f(j < 8 ? ka[j] : kb[j - 8]) * rkA * e1;
      const float qx = bf2f(j < 8 ? qa[j] : qb[j - 8]) * rqA * e1 * d.scale;
      const bf16 hk = f2bf(kx);
      kd[j >> 3][j & 7] = hk;
      kl[j >> 3][j & 7] = f2bf(kx - bf2f(hk));
      const bf16 hq = f2bf(qx);
      qh[j >> 3][j & 7] = hq;
      ql[j >> 3][j & 7] = f2bf(qx - bf2f(hq));
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      *reinterpret_cast<bf16x8*>(P + fwd_panel::KD + rA * HD + cA + 8 * u) = kd[u];
      if (with_lo) *reinterpret_cast<bf16x8*>(P + fwd_panel::KDL + rA * HD + cA + 8 * u) = kl[u];
      *reinterpret_cast<bf16x8*>(P + fwd_panel::QD + rA * HD + cA + 8 * u) = qh[u];
      *reinterpret_cast<bf16x8*>(P + fwd_panel::QD + CL * HD + rA * HD + cA + 8 * u) = ql[u];
    }
    // Ke^T [c][r] = k^_r e^(G_last - G_r): thread (c, rows 16 b .. 16 b + 15),
    // four consecutive threads per row c, so that a wave writes 16 whole
    // 128-byte rows of each plane
    const int c = t >> 2, b = t & 3;
    const float gl = sm.Gref[4][c];
    bf16x8 eh[2], el[2];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = 16 * b + j;
      const float x = bf2f(sm.ks[r][c]) * sm.rk[r] * fexp(gl - sm.G[r][c]);
      const bf16 hx = f2bf(x);
      eh[j >> 3][j & 7] = hx;
      el[j >> 3][j & 7] = f2bf(x - bf2f(hx));
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      *reinterpret_cast<bf16x8*>(P + fwd_panel::KE + c * CL + 16 * b + 8 * u) = eh[u];
      *reinterpret_cast<bf16x8*>(P + fwd_panel::KE + HD * CL + c * CL + 16 * b + 8 * u) = el[u];
    }
    if (t < HD) reinterpret_cast<float*>(P + fwd_panel::GAM)[t] = fexp(sm.Gref[4][t]);
  }
  ci += gx;
  if (ci >= nch) break;
  t0 = nt0;
  n = nn;
  nt0 = nt0b;
  nn = nnb;
  __syncthreads();     // the next chunk's first phase overwrites what was read above
  }
}

hipError_t launch_fwd_prep(const Dims& d, const Inputs& in, const ChunkTable& ct,
                           const SavedSet& sv, int with_bwd, hipStream_t s) {
  // about one workgroup per CU (the LDS allows one), each walking chunks of one head
  const int gx = std::max(1, std::min(d.NC, (kPrepWorkgroups + d.H - 1) / d.H));
  if (d.raw)
    hipLaunchKernelGGL(fwd_prep_kernel<true>, dim3(gx, d.H), dim3(NT_PREP), 0, s, d, in, ct, sv,
                       reinterpret_cast<bf16*>(sv.panels), with_bwd);
  else
    hipLaunchKernelGGL(fwd_prep_kernel<false>, dim3(gx, d.H), dim3(NT_PREP), 0, s, d, in, ct, sv,
                       reinterpret_cast<bf16*>(sv.panels), with_bwd);
  return hipGetLastError();
}

}  // namespace kda
