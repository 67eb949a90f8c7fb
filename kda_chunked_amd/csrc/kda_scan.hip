// Inter-chunk state scans of the KDA chunked form (forward and reverse).
//
// The state S (128 x 128 fp32 per head) is carried across the chunks of one
// packed document; each chunk applies the affine map S_out = M S_in + B of
// flashinfer PR #7176 (opening section), here in the factored form
//   R  = V - Kd S_in            Kd = k * e^G              (64 x 128)
//   U~ = Tb R                   Tb = T Diag(beta)          (64 x 64, lower)
//   O  = scale (Qd S_in + A_qk U~)                         (output rows)
//   S_out = Diag(e^G_last) S_in + Ke^T U~,   Ke = k * e^(G_last - G)
// and the reverse pass
//   dU~ = scale A_qk^T dO + Ke dS_out
//   dR  = Tb^T dU~                               (= dv)
//   dS_in = Diag(e^G_last) dS_out + scale Qd^T dO - Kd^T dR.
// State columns are independent, so each workgroup owns a 32-column tile of
// one (document, head) state (the column split of the half-width transfer
// walk on PR #7176, opening section) and walks the document's chunks in
// order; the 4 tiles of a head are mapped to one XCD so that they share the
// chunk operands through that XCD's L2.
//
// Pipelining: the raw inputs of the next chunk (q, k, v, T, A_qk, ...)
// are loaded into registers while the current chunk's products run, so the
// only memory latency on the sequential path is the first chunk's.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int NT_SCAN = 512;        // threads per scan workgroup (8 waves)
constexpr int VT = 32;              // state columns per workgroup
constexpr int NTILE = HD / VT;      // workgroups per (document, head)
constexpr int K1_LD = HD + 8;       // panels with K = 128
constexpr int K2_LD = CL + 8;       // panels with K = 64

// Split terms per product (SPLIT_A: first operand carries its lo part, ...).
#ifndef KDA_SPLIT_KS
#define KDA_SPLIT_KS SPLIT_NONE
#endif
#ifndef KDA_SPLIT_TR
#define KDA_SPLIT_TR SPLIT_B
#endif
#ifndef KDA_SPLIT_QS
#define KDA_SPLIT_QS SPLIT_AB
#endif
#ifndef KDA_SPLIT_AU
#define KDA_SPLIT_AU SPLIT_AB
#endif
#ifndef KDA_SPLIT_KU
#define KDA_SPLIT_KU SPLIT_AB
#endif
#ifndef KDA_SPLIT_BW
#define KDA_SPLIT_BW SPLIT_AB
#endif
constexpr int SPLIT_KS = KDA_SPLIT_KS;   // Kd S          (forward)
constexpr int SPLIT_TR = KDA_SPLIT_TR;   // Tb R          (forward)
constexpr int SPLIT_QS = KDA_SPLIT_QS;   // Qd S          (forward)
constexpr int SPLIT_AU = KDA_SPLIT_AU;   // A_qk U~       (forward)
constexpr int SPLIT_KU = KDA_SPLIT_KU;   // Ke^T U~       (forward)
constexpr int SPLIT_BW = KDA_SPLIT_BW;   // reverse-scan products with two computed operands

// blockIdx -> (pair = document * H + head, tile). Consecutive workgroups are
// dealt to the 8 XCDs round robin; the 4 tiles of a pair get ids 8 apart.
KDA_DEV bool scan_coords(int P, int& pair, int& tile) {
  const int b = blockIdx.x, x = b & 7, m = b >> 3;
  pair = (m / NTILE) * 8 + x;
  tile = m % NTILE;
  return pair < P;
}

static int scan_grid(int P) { return ((P + 7) / 8) * 8 * NTILE; }

KDA_DEV float bsel(bool ok, bf16 x) { return ok ? bf2f(x) : 0.f; }

// ------------------------------------------------------------------ forward
// The sequential state chain of one (document, head) and 32 state columns.
// Two compute waves, one per 16-column slice: each runs the whole chain of
// its slice by itself,
//   R = V - Kd S_in,  U~ = Tb R,  S_out = e^(G_last) * S_in + Ke^T U~,
// with the right operands of its products in registers (fragK*). Two copy
// waves (on the
// compute unit's other two SIMDs) bring the chunk's shared operands (-Kd, Tb,
// Ke^T, e^(G_last): the first fwd_panel::CHAIN elements of its panels) and
// its V rows global -> registers -> LDS (16-byte units): registers two chunks
// ahead, LDS one chunk ahead in the other of two buffers; the only barrier per
// chunk hands a buffer over.
// The compute waves thus never wait behind the copies at instruction issue.
// S_in, R (when saving for the backward) and U~ go to memory; the output
// O = Qd S_in + A_qk U~ is formed afterwards by fwd_out_kernel, in parallel
// over chunks.
constexpr int FS_THREADS = 128;                       // copy waves (and compute waves)
constexpr int FS_UNITS = fwd_panel::CHAIN / 8;          // 16-byte units: 3616
constexpr int FS_PER_THREAD = (FS_UNITS + FS_THREADS - 1) / FS_THREADS;   // 29
static_assert(fwd_panel::KD == 0 && fwd_panel::TB == 1024 * 8 && fwd_panel::KE == 1536 * 8 &&
                  fwd_panel::GAM == 3584 * 8 && FS_UNITS == 3616,
              "DMA map below assumes this panel layout");

// One chunk's shared operands in LDS, unpadded; 16-byte chunks of each row
// are XOR-swizzled so that 16 rows read at one K offset hit distinct banks.
struct __attribute__((aligned(16))) ChainBuf {
  bf16 kd[CL * HD];          // -Kd  [r][c], row 256 B, chunk ^= r & 15
  bf16 tb[CL * CL];          // Tb   [r][i], row 128 B, chunk ^= (r >> 1) & 7
  bf16 ke[2][HD * CL];       // Ke^T [c][r] hi, lo, as tb
  float gam[HD];
  bf16 v[CL * VT];           // V    [r][j] of the workgroup's 32 columns, row 64 B
};

KDA_DEV int swz256(int row, int kc) { return row * 128 + ((kc ^ (row & 15)) << 3); }
KDA_DEV int swz128(int row, int kc) { return row * 64 + ((kc ^ ((row >> 1) & 7)) << 3); }

// A fragment (16 rows from m0, K = 32 from k) of a swizzled panel.
KDA_DEV bf16x8 frag256(const bf16* p, int m0, int k) {
  const int l = lane_id(), row = m0 + (l & 15);
  return *reinterpret_cast<const bf16x8*>(p + swz256(row, (k >> 3) + (l >> 4)));
}
KDA_DEV bf16x8 frag128(const bf16* p, int m0, int k) {
  const int l = lane_id(), row = m0 + (l & 15);
  return *reinterpret_cast<const bf16x8*>(p + swz128(row, (k >> 3) + (l >> 4)));
}

// The chain's B operands stay in registers. A 32-row K block of a product is
// two D tiles of the right operand, and lane l holds rows 4 (l / 16) .. + 3 of
// each: taken as they are, lane group g supplies K slots 8 g .. 8 g + 7 =
// rows k + 4 g .. + 3 of the first tile and k + 16 + 4 g .. + 3 of the second.
// The A fragment is read in that K order (two 8-byte pieces per lane), so the
// products are the same sums, formed without an LDS round trip.
KDA_DEV bf16x8 cat44(const bf16x4& a, const bf16x4& b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
KDA_DEV bf16x8 fragK256(const bf16* p, int m0, int k) {
  const int l = lane_id(), row = m0 + (l & 15), c0 = k + 4 * (l >> 4), c1 = c0 + 16;
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(p + swz256(row, c0 >> 3) + (c0 & 7));
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(p + swz256(row, c1 >> 3) + (c1 & 7));
  return cat44(a, b);
}
KDA_DEV bf16x8 fragK128(const bf16* p, int m0, int k) {
  const int l = lane_id(), row = m0 + (l & 15), c0 = k + 4 * (l >> 4), c1 = c0 + 16;
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(p + swz128(row, c0 >> 3) + (c0 & 7));
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(p + swz128(row, c1 >> 3) + (c1 & 7));
  return cat44(a, b);
}
// B operand of the K block made of D tiles x0 (first 16 rows) and x1: hi
// planes, and the lo planes (x - hi) when wanted.
KDA_DEV bf16x8 bpair_hi(const f32x4& x0, const f32x4& x1) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = f2bf(x0[i]), r[4 + i] = f2bf(x1[i]);
  return r;
}
KDA_DEV void bpair(const f32x4& x0, const f32x4& x1, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = f2bf(x0[i]);
    hi[4 + i] = f2bf(x1[i]);
    lo[i] = f2bf(x0[i] - bf2f(hi[i]));
    lo[4 + i] = f2bf(x1[i] - bf2f(hi[4 + i]));
  }
}

// Source element (in the chunk's panels) of chain unit u = t + 128 k; the
// unit lands at byte 16 u of a ChainBuf.
KDA_DEV int chain_src(int k, int u) {
  if (k < 8) {
    const int row = u >> 4;
    return fwd_panel::KD + row * 128 + (((u & 15) ^ (row & 15)) << 3);
  }
  if (k < 12) {
    const int v = u - 1024, row = v >> 3;
    return fwd_panel::TB + row * 64 + (((v & 7) ^ ((row >> 1) & 7)) << 3);
  }
  if (k < 28) {
    const int v = u - 1536, pl = v >> 10, row = (v >> 3) & 127;
    return fwd_panel::KE + pl * (HD * CL) + row * 64 + (((v & 7) ^ ((row >> 1) & 7)) << 3);
  }
  return fwd_panel::GAM + (u - 3584) * 8;
}

// One chain is a segment of one head (a whole document when the scans are not
// segmented). MODE = SCAN_FINISH: the chain starts from the segment's entering
// state (zero at a document start, else the forward walk's) and stores the
// per-chunk S_in, R and U~. MODE = SCAN_SUMMARY (segments of documents with
// more than one segment): variant 0 starts from the identity with V = 0 and
// ends at the segment's M; variant 1 starts from zero and ends at its B.
template <int MODE>
__global__ __launch_bounds__(2 * FS_THREADS) void fwd_scan_kernel(Dims d, Inputs in, ChunkTable ct,
                                                               SavedSet sv,
                                                               const bf16* __restrict__ panels,
                                                               int save_R, SegWork sg) {
  __shared__ ChainBuf bufA;
  __shared__ ChainBuf bufB;
  int chain, tile;
  // summaries run two chains per segment: var 0 from the identity with V = 0
  // (ending at M), var 1 from zero (ending at B)
  constexpr bool TWO = MODE == SCAN_SUMMARY || MODE == SCAN_MAP;
  if (!scan_coords((TWO ? 2 : 1) * d.NS * d.H, chain, tile)) return;
  const int var = TWO ? chain & 1 : 0;
  const bool ident = TWO && var == 0;
  const int sh = TWO ? chain >> 1 : chain;
  const int seg = sh / d.H, h = sh % d.H;
  if (seg >= ld_const(ct.seg_doc0, d.N)) return;
  const int doc = ld_const(ct.seg_doc, seg);
  const int sfirst = ld_const(ct.seg_doc0, doc), slast = ld_const(ct.seg_doc0, doc + 1) - 1;
  if (MODE == SCAN_SUMMARY && sfirst == slast) return;
  // the map of a whole sequence: M from document 0 when it is the only one
  // (else M = 0, written by the host), B from the last document
  if (MODE == SCAN_MAP &&
      (var == 0 ? doc != 0 || d.N != 1 || !sg.map_M : doc != d.N - 1 || !sg.map_B))
    return;
  const int dc1 = ld_const(ct.doc_c0, doc + 1);
  const int c0 = ld_const(ct.doc_c0, doc) + (d.L > 0 ? d.L * (seg - sfirst) : 0);
  const int c1 = d.L > 0 ? min(dc1, c0 + d.L) : dc1;
  const int t = threadIdx.x, w = wave_id();
  const int jv = tile * VT + 16 * (w & 1);    // a compute wave's 16 state columns
  const int H = d.H;
  const bf16* v = reinterpret_cast<const bf16*>(in.v);

  // state slice: tile m holds rows 16 m .. 16 m + 15 (D layout)
  f32x4 S[8];
  const int64_t segoff = ((int64_t)seg * H + h) * HD * HD;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    if (MODE == SCAN_FINISH && seg != sfirst && w < 2) {
      S[m] = *reinterpret_cast<const f32x4*>(sg.S0 + segoff + tile_off(m, jv >> 4));
    } else if (MODE == SCAN_FINISH && doc == 0 && sg.s_init && w < 2) {
      // the caller's state entering document 0 (row-major [H][128][128])
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[m][i] = sg.s_init[((int64_t)h * HD + 16 * m + drow(i)) * HD + jv + dcol()];
    } else if (ident) {
#pragma unroll
      for (int i = 0; i < 4; ++i) S[m][i] = 16 * m + drow(i) == jv + dcol() ? 1.f : 0.f;
    } else {
      S[m] = zero4();
    }
  }
  // The chunks of a document are consecutive: first token and length follow
  // from the document's first token and end.
  int64_t tokA = 0, tEnd = 0;
  if (c0 < c1) {
    tokA = ld_const(ct.tok, c0);
    tEnd = (int64_t)ld_const(ct.tok, c1 - 1) + ld_const(ct.len, c1 - 1);
  }
  auto rows_in = [&](int cn, int64_t& t0, int& n) {
    t0 = tokA + (int64_t)CL * (cn - c0);
    const int64_t left = tEnd - t0;
    n = left < CL ? (int)left : CL;
  };
  auto panel_of = [&](int cn) { return panels + ((int64_t)cn * H + h) * fwd_panel::ELEMS; };

  auto step = [&](ChainBuf& cur, int ci) {
    int64_t t0;
    int n;
    rows_in(ci, t0, n);
    const int64_t ch = (int64_t)ci * H + h;
    __syncthreads();                   // `cur` has landed
    // R starts as V (D layout) through transpose loads of cur.v
    f32x4 R[4];
    {
      typedef short s16x4 __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
      const int l = lane_id(), sl = l & 15;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int r0 = 16 * rb + 4 * (l >> 4);
        const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(cur.v + (r0 + (sl >> 2)) * VT + 16 * w + 4 * (sl & 3)));
        const bf16x4 xb = __builtin_bit_cast(bf16x4, x);
        // the identity variant of a segment summary (and the map) takes V = 0
        const bool vz = ident;
#pragma unroll
        for (int i = 0; i < 4; ++i) R[rb][i] = r0 + i < n && !vz ? bf2f(xb[i]) : 0.f;
      }
    }
    // S_in to memory (streamed out, non-temporal: read only by later kernels)
    if (MODE == SCAN_FINISH) {
      float* Sg = sv.S_in + ch * HD * HD;
#pragma unroll
      for (int m = 0; m < 8; ++m)
        __builtin_nontemporal_store(S[m], reinterpret_cast<f32x4*>(Sg + tile_off(m, jv >> 4)));
    }
    // R = V - Kd S_in (the panel holds -Kd)
#pragma unroll
    for (int kb = 0; kb < HD / 32; ++kb) {
      const bf16x8 b = bpair_hi(S[2 * kb], S[2 * kb + 1]);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) R[rb] = mfma16(fragK256(cur.kd, 16 * rb, 32 * kb), b, R[rb]);
    }
    if (MODE == SCAN_FINISH && save_R) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        __builtin_nontemporal_store(
            R[rb], reinterpret_cast<f32x4*>(sv.R + ch * CL * HD + tile_off(rb, jv >> 4)));
    }
    // U~ = Tb R (Tb lower triangular: K up to the end of the row block)
    f32x4 U[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) U[rb] = zero4();
#pragma unroll
    for (int kb = 0; kb < CL / 32; ++kb) {
      bf16x8 bh, bl;
      bpair(R[2 * kb], R[2 * kb + 1], bh, bl);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        if (32 * kb < 16 * rb + 16) {
          const bf16x8 a = fragK128(cur.tb, 16 * rb, 32 * kb);
          U[rb] = mfma16(a, bl, U[rb]);
          U[rb] = mfma16(a, bh, U[rb]);
        }
      }
    }
    if (MODE == SCAN_FINISH) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        __builtin_nontemporal_store(
            U[rb], reinterpret_cast<f32x4*>(sv.U + ch * CL * HD + tile_off(rb, jv >> 4)));
    }
    // S_out = e^(G_last) * S_in + Ke^T U~
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[m][i] *= cur.gam[16 * m + drow(i)];
#pragma unroll
    for (int kb = 0; kb < CL / 32; ++kb) {
      bf16x8 bh, bl;
      bpair(U[2 * kb], U[2 * kb + 1], bh, bl);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const bf16x8 ah = fragK128(cur.ke[0], 16 * m, 32 * kb);
        const bf16x8 al = fragK128(cur.ke[1], 16 * m, 32 * kb);
        S[m] = mfma16(al, bh, S[m]);
        S[m] = mfma16(ah, bl, S[m]);
        S[m] = mfma16(ah, bh, S[m]);
      }
    }
  };

  if (w >= 2) {
    // copy waves
    const int tp = t - FS_THREADS;
    // Chunk cn + 1 is written from registers into the buffer freed at the
    // start of step cn, then chunk cn + 2 is requested into the registers:
    // each load has a whole step to arrive. V rows from n on repeat row n - 1
    // (masked when read); V unit u is row u / 4, columns j0 + 8 (u % 4).
    bf16x8 x[FS_PER_THREAD + 2];
    auto load = [&](int cn) {
      int64_t u0;
      int un;
      rows_in(cn, u0, un);
      const bf16* src = panel_of(cn);
#pragma unroll
      for (int k = 0; k < FS_PER_THREAD; ++k) {
        const int u = tp + FS_THREADS * k;
        if (k < FS_PER_THREAD - 1 || u < FS_UNITS)
          x[k] = *reinterpret_cast<const bf16x8*>(src + chain_src(k, u));
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int u = tp + FS_THREADS * k, r = u >> 2, rc = r < un ? r : un - 1;
        x[FS_PER_THREAD + k] =
            *reinterpret_cast<const bf16x8*>(v + ((u0 + rc) * H + h) * HD + tile * VT + 8 * (u & 3));
      }
    };
    auto store = [&](ChainBuf& dst) {
      char* base = reinterpret_cast<char*>(&dst);
#pragma unroll
      for (int k = 0; k < FS_PER_THREAD; ++k) {
        const int u = tp + FS_THREADS * k;
        if (k < FS_PER_THREAD - 1 || u < FS_UNITS)
          *reinterpret_cast<bf16x8*>(base + 16 * u) = x[k];
      }
#pragma unroll
      for (int k = 0; k < 2; ++k)
        *reinterpret_cast<bf16x8*>(reinterpret_cast<char*>(dst.v) + 16 * (tp + FS_THREADS * k)) =
            x[FS_PER_THREAD + k];
    };
    if (c0 < c1) {
      load(c0);
      store(bufA);
    }
    if (c0 + 1 < c1) load(c0 + 1);
    for (int ci = c0; ci < c1; ci += 2) {
      __syncthreads();
      if (ci + 1 < c1) {
        store(bufB);
        if (ci + 2 < c1) load(ci + 2);
        __syncthreads();
        if (ci + 2 < c1) {
          store(bufA);
          if (ci + 3 < c1) load(ci + 3);
        }
      }
    }
    return;
  }
  for (int ci = c0; ci < c1; ci += 2) {
    step(bufA, ci);
    if (ci + 1 < c1) step(bufB, ci + 1);
  }
  if (MODE == SCAN_SUMMARY) {
    float* dst = (var == 0 ? sg.M : sg.B) + segoff;
#pragma unroll
    for (int m = 0; m < 8; ++m) *reinterpret_cast<f32x4*>(dst + tile_off(m, jv >> 4)) = S[m];
  }
  // the state leaving the last document, or the sequence map's M or B, in
  // the caller layout
  float* leave = MODE == SCAN_MAP ? (var == 0 ? sg.map_M : sg.map_B)
               : MODE == SCAN_FINISH && doc == d.N - 1 && seg == slast ? sg.s_final : nullptr;
  if (leave) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        leave[((int64_t)h * HD + 16 * m + drow(i)) * HD + jv + dcol()] = S[m][i];
  }
}

hipError_t launch_fwd_scan(const Dims& d, const Inputs& in, const ChunkTable& ct,
                           const SavedSet& sv, const void* panels, int save_R,
                           const SegWork& sg, int mode, hipStream_t s) {
  const bf16* pn = reinterpret_cast<const bf16*>(panels);
  if (mode == SCAN_SUMMARY)
    hipLaunchKernelGGL(fwd_scan_kernel<SCAN_SUMMARY>, dim3(scan_grid(2 * d.NS * d.H)),
                       dim3(2 * FS_THREADS), 0, s, d, in, ct, sv, pn, save_R, sg);
  else if (mode == SCAN_MAP)
    hipLaunchKernelGGL(fwd_scan_kernel<SCAN_MAP>, dim3(scan_grid(2 * d.NS * d.H)),
                       dim3(2 * FS_THREADS), 0, s, d, in, ct, sv, pn, save_R, sg);
  else
    hipLaunchKernelGGL(fwd_scan_kernel<SCAN_FINISH>, dim3(scan_grid(d.NS * d.H)),
                       dim3(2 * FS_THREADS), 0, s, d, in, ct, sv, pn, save_R, sg);
  return hipGetLastError();
}

// O = scale (Qd S_in + A_qk U~) per (chunk, head), from the saved S_in and U~
// and the output panels (scale folded in). 8 waves: rows 16 (w & 3), columns
// 64 (w >> 2) .. + 63. A operands are read from memory as MFMA fragments; the
// B operands S_in^T and U~^T are split into LDS panels.
// Panel rows of 288 and 160 bytes: the 16-byte fragment reads of 16 rows then
// meet no bank conflict (272 and 144 bytes, the strides of the other kernels'
// panels, measured 2.3 % slower here).
constexpr int O1_LD = HD + 16, O2_LD = CL + 16;
struct __attribute__((aligned(16))) FwdOutSmem {
  bf16 s_hi[HD][O1_LD], s_lo[HD][O1_LD];     // S_in^T [j][c]
  bf16 u_hi[HD][O2_LD], u_lo[HD][O2_LD];     // U~^T   [j][i]
  bf16 ot[CL][O1_LD];                        // O [r][c] of the chunk, to rows of 16-byte stores
};

KDA_DEV bf16x8 gfrag(const bf16* p, int ld, int m0, int k) {
  const int l = lane_id();
  return *reinterpret_cast<const bf16x8*>(p + (m0 + (l & 15)) * ld + k + ((l >> 4) << 3));
}

// One workgroup walks the chunks ci, ci + gridDim.x, ... of head h and loads
// the next chunk's S_in, U~ tiles and Qd, A_qk fragments while it works on the
// current one.
constexpr int kOutWorkgroups = 256;     // about one per CU (the LDS allows one)

__global__ __launch_bounds__(512) void fwd_out_kernel(Dims d, ChunkTable ct,
                                                       SavedSet sv,
                                                       const bf16* __restrict__ panels,
                                                       bf16* __restrict__ o) {
  __shared__ FwdOutSmem sm;
  const int h = blockIdx.y, nch = ld_const(ct.doc_c0, d.N);
  const int H = d.H;
  const Panel SP{&sm.s_hi[0][0], &sm.s_lo[0][0], O1_LD};
  const Panel UP{&sm.u_hi[0][0], &sm.u_lo[0][0], O2_LD};
  const int w0 = wave_id(), rb0 = w0 & 3;
  f32x4 xs[8], xu[4];               // S_in tiles (c block w, all j blocks), U~ tiles (i blocks, j block w)
  bf16x8 fq[4][2], fa[2][2];        // scale Qd, scale A_qk fragments (hi, lo) of row block rb
  auto load_chunk = [&](int cn) {
    const int64_t cch = (int64_t)cn * H + h;
    const float* Sg = sv.S_in + cch * HD * HD;
    const float* Ug = sv.U + cch * CL * HD;
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) xs[jb] = *reinterpret_cast<const f32x4*>(Sg + tile_off(w0, jb));
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) xu[ib] = *reinterpret_cast<const f32x4*>(Ug + tile_off(ib, w0));
    const bf16* P = panels + cch * fwd_panel::ELEMS;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      fq[kk][0] = gfrag(P + fwd_panel::QD, HD, 16 * rb0, 32 * kk);
      fq[kk][1] = gfrag(P + fwd_panel::QD + CL * HD, HD, 16 * rb0, 32 * kk);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      fa[kk][0] = gfrag(P + fwd_panel::AQ, CL, 16 * rb0, 32 * kk);
      fa[kk][1] = gfrag(P + fwd_panel::AQ + CL * CL, CL, 16 * rb0, 32 * kk);
    }
  };
  int ci = blockIdx.x;
  if (ci >= nch) return;
  const int gx = gridDim.x;
  int64_t t0 = ld_const(ct.tok, ci);
  int n = ld_const(ct.len, ci);
  // O of a chunk leaves through sm.ot after the barrier that follows its
  // products: thread t writes row t / 8, columns 16 (t % 8) .. + 15
  auto store_o = [&](int64_t ot0, int on) {
    const int t = threadIdx.x, r = t >> 3, c = 16 * (t & 7);
    if (r < on) {
      bf16* dst = o + ((ot0 + r) * H + h) * HD + c;
      *reinterpret_cast<bf16x8*>(dst) = *reinterpret_cast<const bf16x8*>(&sm.ot[r][c]);
      *reinterpret_cast<bf16x8*>(dst + 8) = *reinterpret_cast<const bf16x8*>(&sm.ot[r][c + 8]);
    }
  };
  // S_in [c][j] -> S_in^T panel, U~ [i][j] -> U~^T panel, A fragments to the
  // registers the products read: the loaded values are consumed before the
  // loop closes, so that no load is still in flight across its back edge
  bf16x8 aq[4][2], aa[2][2];
  auto stage = [&]() {
    // indices from an opaque copy of the thread id, so that LDS addresses
    // are not hoisted out of the loop and held in registers
    int tt = threadIdx.x;
    asm volatile("" : "+v"(tt));
    const int w = tt >> 6;
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) store_tile_t(xs[jb], SP, 16 * w, 16 * jb);
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) store_tile_t(xu[ib], UP, 16 * ib, 16 * w);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) aq[kk][0] = fq[kk][0], aq[kk][1] = fq[kk][1];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) aa[kk][0] = fa[kk][0], aa[kk][1] = fa[kk][1];
  };
  load_chunk(ci);
  stage();
  __syncthreads();
  for (;;) {
    int tt = threadIdx.x;
    asm volatile("" : "+v"(tt));
    const int w = tt >> 6, rb = w & 3, chh = w >> 2;
    // the next chunk's operands and table entry, requested on every path
    // (the last chunk reloads itself)
    const int cn = min(ci + gx, nch - 1);
    const int64_t nt0 = ld_const(ct.tok, cn);
    const int nn = ld_const(ct.len, cn);
    load_chunk(cn);
    f32x4 acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = zero4();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 ah = aq[kk][0], al = aq[kk][1];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int n0 = 64 * chh + 16 * nt;
        const bf16x8 bh = frag(SP.hi, SP.ld, n0, 32 * kk), bl = frag(SP.lo, SP.ld, n0, 32 * kk);
        acc[nt] = mfma16(al, bh, acc[nt]);
        acc[nt] = mfma16(ah, bl, acc[nt]);
        acc[nt] = mfma16(ah, bh, acc[nt]);
      }
    }
    // A_qk is lower triangular: K up to the end of the row block
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      if (32 * kk < 16 * rb + 16) {
        const bf16x8 ah = aa[kk][0], al = aa[kk][1];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int n0 = 64 * chh + 16 * nt;
          const bf16x8 bh = frag(UP.hi, UP.ld, n0, 32 * kk), bl = frag(UP.lo, UP.ld, n0, 32 * kk);
          acc[nt] = mfma16(al, bh, acc[nt]);
          acc[nt] = mfma16(ah, bl, acc[nt]);
          acc[nt] = mfma16(ah, bh, acc[nt]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) sm.ot[16 * rb + drow(i)][64 * chh + 16 * nt + dcol()] = f2bf(acc[nt][i]);
    __syncthreads();   // the panels are free again and O is complete in sm.ot
    store_o(t0, n);
    if (ci + gx >= nch) break;
    stage();
    ci += gx;
    t0 = nt0;
    n = nn;
    __syncthreads();
  }
}

hipError_t launch_fwd_out(const Dims& d, const ChunkTable& ct, const SavedSet& sv,
                          const void* panels, void* o, hipStream_t s) {
  const int gx = std::max(1, std::min(d.NC, (kOutWorkgroups + d.H - 1) / d.H));
  hipLaunchKernelGGL(fwd_out_kernel, dim3(gx, d.H), dim3(512), 0, s, d, ct, sv,
                     reinterpret_cast<const bf16*>(panels), reinterpret_cast<bf16*>(o));
  return hipGetLastError();
}

// ------------------------------------------------------------------ reverse
// LDS of the reverse scan. The chunk's operands are the forward panels in
// their stored (row-major, natural) orientation; every product here needs
// them transposed (K along the stored rows), which the LDS transpose loads of
// fragT provide. Rows are padded to 72 or 144 elements so that those loads
// are free of bank conflicts. The panels arrive through 16-byte copies
// prefetched into registers one chunk ahead; scale Qd shares its LDS space
// with Ke^T and is staged once Ke^T has been consumed.
constexpr int QD_LD = HD + 16;       // 144: rows of 288 bytes
struct __attribute__((aligned(16))) BwdScanSmem {
  union {
    struct { bf16 hi[HD][K2_LD], lo[HD][K2_LD]; } ke;      // Ke^T         [c][r]
    struct { bf16 hi[CL][QD_LD], lo[CL][QD_LD]; } qd;      // scale*Qd     [r][c]
  } r1;
  bf16 kd_hi[CL][QD_LD], kd_lo[CL][QD_LD];                 // -Kd          [r][c]
  bf16 aq_hi[CL][K2_LD], aq_lo[CL][K2_LD];                 // scale*A_qk   [r][i]
  bf16 tb_hi[CL][K2_LD], tb_lo[CL][K2_LD];                 // Tb           [r][i]
  bf16 do_hi[VT][K2_LD];                                   // dO^T [j][r] (exact bf16)
  bf16 ds_hi[VT][K1_LD], ds_lo[VT][K1_LD];                 // dS^T [j][c]
  bf16 du_hi[VT][K2_LD], du_lo[VT][K2_LD];                 // dU~^T [j][r]
  bf16 dr_hi[VT][K2_LD], dr_lo[VT][K2_LD];                 // dR^T [j][r]
  float gam[HD];
};

// The operands as 8224 16-byte units u = t + 512 k, k = 0..16, read from the
// chunk's forward panels: k 0-3 Ke^T (hi, lo), 4-5 A_qk (hi, lo), 6 Tb hi,
// 7 Tb lo, 8-11 Qd (hi, lo; staged after Ke^T is consumed), 12-13 -Kd hi,
// 14-15 -Kd lo, 16 e^(G_last) (32 units).
constexpr int BP_UNITS = 8224;
constexpr int BP_PER_THREAD = (BP_UNITS + NT_SCAN - 1) / NT_SCAN;   // 17
static_assert(fwd_panel::KE + 2 * 128 * 64 == fwd_panel::GAM &&
                  fwd_panel::QD + 2 * 64 * 128 == fwd_panel::AQ,
              "staging map below assumes this panel layout");

// Panel offset (bf16 elements) of unit t + 512 k at t = 0.
KDA_DEV constexpr int bunit_src(int k) {
  return k < 4 ? fwd_panel::KE + 4096 * k
       : k < 6 ? fwd_panel::AQ + 4096 * (k - 4)
       : k == 6 ? fwd_panel::TB
       : k == 7 ? fwd_panel::TBL
       : k < 12 ? fwd_panel::QD + 4096 * (k - 8)
       : k < 14 ? fwd_panel::KD + 4096 * (k - 12)
       : k < 16 ? fwd_panel::KDL + 4096 * (k - 14)
       : fwd_panel::GAM;
}

// LDS destination of unit u = t + 512 k.
KDA_DEV void bstage_unit(BwdScanSmem& sm, int k, int t, const bf16x8& x) {
  const int v = t + NT_SCAN * (k < 4 ? k : k < 6 ? k - 4 : k < 8 ? 0 : k < 12 ? k - 8
                                     : k < 14 ? k - 12 : k < 16 ? k - 14 : 0);
  bf16* dst;
  if (k < 4) {                       // Ke^T [c][r] hi, lo
    dst = (v >> 10 ? &sm.r1.ke.lo[0][0] : &sm.r1.ke.hi[0][0]) + ((v >> 3) & 127) * K2_LD + ((v & 7) << 3);
  } else if (k < 6) {                // A_qk [r][i] hi, lo
    dst = (v >> 9 ? &sm.aq_lo[0][0] : &sm.aq_hi[0][0]) + ((v >> 3) & 63) * K2_LD + ((v & 7) << 3);
  } else if (k < 8) {                // Tb [r][i] hi (k = 6), lo (k = 7)
    dst = (k == 7 ? &sm.tb_lo[0][0] : &sm.tb_hi[0][0]) + (v >> 3) * K2_LD + ((v & 7) << 3);
  } else if (k < 12) {               // scale Qd [r][c] hi, lo (into the Ke^T space)
    dst = (v >> 10 ? &sm.r1.qd.lo[0][0] : &sm.r1.qd.hi[0][0]) + ((v >> 4) & 63) * QD_LD + ((v & 15) << 3);
  } else if (k < 16) {               // -Kd [r][c] hi (k = 12, 13), lo (k = 14, 15)
    dst = (k >= 14 ? &sm.kd_lo[0][0] : &sm.kd_hi[0][0]) + (v >> 4) * QD_LD + ((v & 15) << 3);
  } else {                           // e^(G_last), fp32 (32 units)
    *reinterpret_cast<bf16x8*>(&sm.gam[4 * t]) = x;
    return;
  }
  *reinterpret_cast<bf16x8*>(dst) = x;
}

// One chain is a segment of one head, walked from its last chunk to its
// first. MODE = SCAN_FINISH: dS starts from the segment's exit value (zero at a
// document end, else the reverse walk's) and the per-chunk dU~, dS_out and dv
// are stored. MODE = SCAN_SUMMARY (segments of documents with more than one
// segment): dS starts from zero and only the dS reached at the segment start
// (its B') is stored.
template <int MODE>
__global__ __launch_bounds__(NT_SCAN) void bwd_scan_kernel(Dims d, Inputs in, ChunkTable ct,
                                                            SavedSet sv,
                                                            const bf16* __restrict__ dO,
                                                            bf16* __restrict__ dv, BwdWork bw,
                                                            SegWork sg) {
  __shared__ BwdScanSmem sm;
  int chain, tile;
  if (!scan_coords(d.NS * d.H, chain, tile)) return;
  const int seg = chain / d.H, h = chain % d.H;
  if (seg >= ld_const(ct.seg_doc0, d.N)) return;
  const int doc = ld_const(ct.seg_doc, seg);
  const int sfirst = ld_const(ct.seg_doc0, doc), slast = ld_const(ct.seg_doc0, doc + 1) - 1;
  if (MODE == SCAN_SUMMARY && sfirst == slast) return;
  // the gradient summary of a whole sequence: document 0 only
  if (MODE == SCAN_MAP && doc != 0) return;
  const int dc1 = ld_const(ct.doc_c0, doc + 1);
  const int c0 = ld_const(ct.doc_c0, doc) + (d.L > 0 ? d.L * (seg - sfirst) : 0);
  const int c1 = d.L > 0 ? min(dc1, c0 + d.L) : dc1;
  const int64_t segoff = ((int64_t)seg * d.H + h) * HD * HD;
  const int t = threadIdx.x, w = wave_id();
  const int rb = w & 3, nw = w >> 2;
  const int j0 = tile * VT;
  const int H = d.H;
  const bf16* BP = reinterpret_cast<const bf16*>(sv.panels);

  const Panel KE{&sm.r1.ke.hi[0][0], &sm.r1.ke.lo[0][0], K2_LD};
  const Panel QD{&sm.r1.qd.hi[0][0], &sm.r1.qd.lo[0][0], QD_LD};
  const Panel KD{&sm.kd_hi[0][0], &sm.kd_lo[0][0], QD_LD};
  const Panel AQ{&sm.aq_hi[0][0], &sm.aq_lo[0][0], K2_LD};
  const Panel TB{&sm.tb_hi[0][0], &sm.tb_lo[0][0], K2_LD};
  const Panel DO{&sm.do_hi[0][0], nullptr, K2_LD};
  const Panel DS{&sm.ds_hi[0][0], &sm.ds_lo[0][0], K1_LD};
  const Panel DU{&sm.du_hi[0][0], &sm.du_lo[0][0], K2_LD};
  const Panel DR{&sm.dr_hi[0][0], &sm.dr_lo[0][0], K2_LD};

  // Each operand is staged into LDS in the phase before its first use, and
  // the next chunk's copy of it is requested right after staging, so the
  // memory requests of a chunk are spread over the four phases of the
  // previous one instead of queueing in one burst.
  bf16x8 pu[BP_PER_THREAD];
  bf16x4 pdo;          // dO, row rO, columns j0 + cO .. + 3
  const int rO = t >> 3, cO = 4 * (t & 7);
  // The chunks of a document are consecutive: first token and length follow
  // from the document's first token and end.
  int64_t tokA = 0, tEnd = 0;
  if (c0 < c1) {
    tokA = ld_const(ct.tok, c0);
    tEnd = (int64_t)ld_const(ct.tok, c1 - 1) + ld_const(ct.len, c1 - 1);
  }
  auto units = [&](int cn, int klo, int khi) {
    const bf16* src = BP + ((int64_t)cn * H + h) * fwd_panel::ELEMS + 8 * t;
#pragma unroll
    for (int k = 0; k < BP_PER_THREAD; ++k)
      if (k >= klo && k < khi && (k < BP_PER_THREAD - 1 || t < BP_UNITS - NT_SCAN * (BP_PER_THREAD - 1)))
        pu[k] = *reinterpret_cast<const bf16x8*>(src + bunit_src(k));
  };
  auto stage = [&](int klo, int khi) {
#pragma unroll
    for (int k = 0; k < BP_PER_THREAD; ++k)
      if (k >= klo && k < khi && (k < BP_PER_THREAD - 1 || t < BP_UNITS - NT_SCAN * (BP_PER_THREAD - 1)))
        bstage_unit(sm, k, t, pu[k]);
  };
  auto rows_in = [&](int cn, int64_t& t0, int& n) {
    t0 = tokA + (int64_t)CL * (cn - c0);
    const int64_t left = tEnd - t0;
    n = left < CL ? (int)left : CL;
  };
  auto load_dO = [&](int cn) {
    int64_t t0;
    int n;
    rows_in(cn, t0, n);
    const int rc = rO < n ? rO : n - 1;
    pdo = *reinterpret_cast<const bf16x4*>(dO + ((t0 + rc) * H + h) * HD + j0 + cO);
  };

  f32x4 dS[2];
  dS[0] = dS[1] = zero4();
  for (int e = t; e < VT * K1_LD; e += NT_SCAN) {
    (&sm.ds_hi[0][0])[e] = f2bf(0.f);
    (&sm.ds_lo[0][0])[e] = f2bf(0.f);
  }
  const bool tail_in = MODE == SCAN_FINISH && doc == d.N - 1 && seg == slast && sg.ds_final;
  if (MODE == SCAN_FINISH && (seg != slast || tail_in)) {
    // the dS leaving this segment (rows 16 w, this tile's columns): from the
    // reverse walk, or the caller's gradient of the state leaving the last
    // document (row-major [H][128][128])
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      if (seg != slast) {
        dS[nt] = *reinterpret_cast<const f32x4*>(sg.D0 + segoff + tile_off(w, (j0 >> 4) + nt));
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dS[nt][i] = sg.ds_final[((int64_t)h * HD + 16 * w + drow(i)) * HD + j0 + 16 * nt + dcol()];
      }
      store_tile_t(dS[nt], DS, 16 * w, 16 * nt);
    }
  }
  // issued in the order of one step's requests, so that the waits counted
  // for the first step are no stricter than for the later ones
  if (c0 < c1) {
    units(c1 - 1, 0, 6);
    load_dO(c1 - 1);
    units(c1 - 1, 6, 8);
    units(c1 - 1, 8, 12);
    units(c1 - 1, 12, BP_PER_THREAD);
  }

  for (int ci = c1 - 1; ci >= c0; --ci) {
    int64_t t0;
    int n;
    rows_in(ci, t0, n);
    // the next copies are requested on every path (the last chunk reloads
    // itself) so that the counted waits for them are the same on all paths
    const int cp = ci > c0 ? ci - 1 : ci;
    const int64_t ch = (int64_t)ci * H + h;
    // ---- A. Ke^T, A_qk, dO^T into LDS; their next copies requested
    stage(0, 6);
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.do_hi[cO + e][rO] = rO < n ? pdo[e] : f2bf(0.f);
    units(cp, 0, 6);
    load_dO(cp);
    __syncthreads();
    // ---- B. dU~ = scale A_qk^T dO + Ke dS_out   (tile rows 16 rb, cols 16 nw)
    {
      f32x4 dU = zero4();
      mma<SPLIT_A, true>(dU, AQ, 16 * rb, DO, 16 * nw, (16 * rb / 32) * 32, CL);
      mma_k<SPLIT_BW, HD, true>(dU, KE, 16 * rb, DS, 16 * nw);
      // dU~ and dS_out are streamed out (non-temporal): read only by the next kernel
      if (MODE == SCAN_FINISH)
        __builtin_nontemporal_store(
            dU, reinterpret_cast<f32x4*>(bw.dU + ch * CL * HD + tile_off(rb, (j0 >> 4) + nw)));
      store_tile_t(dU, DU, 16 * rb, 16 * nw);
    }
    stage(6, 8);                                   // Tb
    units(cp, 6, 8);
    __syncthreads();
    // ---- C. dR = Tb^T dU~ (= dv); scale Qd, -Kd, e^(G_last) into LDS
    {
      f32x4 acc = zero4();
      mma<SPLIT_BW, true>(acc, TB, 16 * rb, DU, 16 * nw, (16 * rb / 32) * 32, CL);
      store_tile_t(acc, DR, 16 * rb, 16 * nw);
    }
    stage(8, BP_PER_THREAD);
    units(cp, 8, 12);
    __syncthreads();
    // ---- D. dS_in = Diag(e^G_last) dS_out + scale Qd^T dO - Kd^T dR
    {
      // dv = bf16(dR): row rO, columns j0 + cO .. + 3, from the hi plane of dR^T
      if (MODE == SCAN_FINISH && rO < n) {
        bf16x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = sm.dr_hi[cO + e][rO];
        *reinterpret_cast<bf16x4*>(dv + ((t0 + rO) * H + h) * HD + j0 + cO) = x;
      }
      float* dSg = bw.dS + ch * HD * HD;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        if (MODE == SCAN_FINISH)
          __builtin_nontemporal_store(dS[nt],
                                      reinterpret_cast<f32x4*>(dSg + tile_off(w, (j0 >> 4) + nt)));
#pragma unroll
        for (int i = 0; i < 4; ++i) dS[nt][i] *= sm.gam[16 * w + drow(i)];
      }
      mma_row<SPLIT_A, 2, true>(dS, QD, 16 * w, DO, 0, 0, CL);
      mma_row<SPLIT_BW, 2, true>(dS, KD, 16 * w, DR, 0, 0, CL);
    }
    units(cp, 12, BP_PER_THREAD);
    // dS^T is read only in phase B: its panel is written before the barrier
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) store_tile_t(dS[nt], DS, 16 * w, 16 * nt);
    __syncthreads();
  }
  if (MODE == SCAN_SUMMARY) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
      *reinterpret_cast<f32x4*>(sg.Brev + segoff + tile_off(w, (j0 >> 4) + nt)) = dS[nt];
  }
  // the gradient with respect to the state entering document 0 (with a zero
  // gradient leaving the sequence: its B')
  if (MODE != SCAN_SUMMARY && doc == 0 && seg == sfirst && sg.ds_init) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sg.ds_init[((int64_t)h * HD + 16 * w + drow(i)) * HD + j0 + 16 * nt + dcol()] = dS[nt][i];
  }
}

hipError_t launch_bwd_scan(const Dims& d, const Inputs& in, const ChunkTable& ct,
                           const SavedSet& sv, const void* dO, void* dv,
                           const BwdWork& bw, const SegWork& sg, int mode, hipStream_t s) {
  const bf16* pdo = reinterpret_cast<const bf16*>(dO);
  bf16* pdv = reinterpret_cast<bf16*>(dv);
  if (mode == SCAN_SUMMARY)
    hipLaunchKernelGGL(bwd_scan_kernel<SCAN_SUMMARY>, dim3(scan_grid(d.NS * d.H)), dim3(NT_SCAN),
                       0, s, d, in, ct, sv, pdo, pdv, bw, sg);
  else if (mode == SCAN_MAP)      // the chains of document 0 are the first H
    hipLaunchKernelGGL(bwd_scan_kernel<SCAN_MAP>, dim3(scan_grid(d.H)), dim3(NT_SCAN), 0, s, d,
                       in, ct, sv, pdo, pdv, bw, sg);
  else
    hipLaunchKernelGGL(bwd_scan_kernel<SCAN_FINISH>, dim3(scan_grid(d.NS * d.H)), dim3(NT_SCAN),
                       0, s, d, in, ct, sv, pdo, pdv, bw, sg);
  return hipGetLastError();
}

}  // namespace kda
