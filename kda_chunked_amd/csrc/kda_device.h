// Device-side building blocks shared by the gfx950 KDA kernels.
//
// Matrix products run on the CDNA4 MFMA unit as v_mfma_f32_16x16x32_bf16
// (16x16 output tile, K step 32, fp32 accumulation). Operands that are not
// exact bf16 inputs are carried as an fp32 value split into two bf16 parts
// x = hi + lo (hi = RNE(x), lo = RNE(x - hi)); a product of two split operands
// is hi*hi + hi*lo + lo*hi (the BF16x3 split product named on flashinfer
// PR #7176, opening section), which keeps fp32-grade accuracy on bf16 MFMA.
//
// Lane layout of v_mfma_f32_16x16x32_bf16 (wave64, lane l):
//   A (16 x 32): lane l holds A[l % 16][8 * (l / 16) + 0..7]
//   B (32 x 16): lane l holds B[8 * (l / 16) + 0..7][l % 16]
//   D (16 x 16): lane l holds D[4 * (l / 16) + 0..3][l % 16]
// Operands are staged in LDS "panels": row-major bf16 tiles whose rows run
// along the product's K dimension (so one 16-byte read fills a fragment);
// a B operand is stored as its transpose (rows = N).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int CL = 64;    // chunk length (tokens)
constexpr int HD = 128;   // head dimension (dk = dv)
constexpr float LOG2E = 1.4426950408889634f;

#define KDA_DEV __device__ __forceinline__

KDA_DEV int lane_id() { return threadIdx.x & 63; }
KDA_DEV int wave_id() { return threadIdx.x >> 6; }

KDA_DEV f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

KDA_DEV f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

KDA_DEV float bf2f(bf16 x) { return (float)x; }
KDA_DEV bf16 f2bf(float x) { return (bf16)x; }  // round to nearest even

// exp(x) through the hardware base-2 exponential.
KDA_DEV float fexp(float x) { return __builtin_amdgcn_exp2f(x * LOG2E); }

// A global load at a 32-bit byte offset from a base pointer that is the same
// for every lane: the address is the base (scalar registers) plus the
// zero-extended offset, so a lane needs no 64-bit multiply for it. Offsets
// within one chunk's rows of a [T, H, 128] tensor stay below 2^32 bytes for
// every head count the library accepts (at most 65535).
template <class T>
KDA_DEV T ld_at(const T* base, uint32_t byte_off) {
  return *reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + byte_off);
}

// A read of data that no kernel in flight writes (the chunk table), through
// the constant address space: at a uniform index it becomes a scalar load,
// whose value lands in scalar registers without a wait on the vector memory
// counter (which would also wait for every vector load issued before it).
template <class T>
KDA_DEV T ld_const(const T* p, int i) {
  return ((const __attribute__((address_space(4))) T*)p)[i];
}

// An LDS operand panel: hi and lo bf16 planes, `ld` elements per row.
struct Panel {
  bf16* hi;
  bf16* lo;
  int ld;
};

// Which operands of a product carry their lo part.
enum : int { SPLIT_NONE = 0, SPLIT_A = 1, SPLIT_B = 2, SPLIT_AB = 3 };

KDA_DEV bf16x8 frag(const bf16* p, int ld, int row0, int k) {
  const int l = lane_id();
  return *reinterpret_cast<const bf16x8*>(p + (row0 + (l & 15)) * ld + k + ((l >> 4) << 3));
}

// The same fragment of A[m][k] from a panel that stores A transposed, as
// [k][m] (row k, ld elements per row), by two LDS transpose loads. Within each
// 16-lane group the load gives lane j the j-th column of the 4 x 16 block whose
// rows the group's lanes address: lane s (of 16) supplies row s / 4 and
// columns 4 (s % 4) .. + 3, so lane j receives rows 0..3 of column j. The
// panel must live in LDS with 8-byte aligned rows.
KDA_DEV bf16x8 fragT(const bf16* p, int ld, int m0, int k) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const int l = lane_id(), s = l & 15;
  const bf16* a = p + (k + 8 * (l >> 4) + (s >> 2)) * ld + m0 + 4 * (s & 3);
  const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a));
  const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 4 * ld));
  // whole-vector concatenation and one 16-byte bit cast (no per-element casts)
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// A operand fragment: K-contiguous panel (AT = false) or transposed panel.
template <bool AT>
KDA_DEV bf16x8 afrag(const bf16* p, int ld, int m0, int k) {
  return AT ? fragT(p, ld, m0, k) : frag(p, ld, m0, k);
}

// acc += A[m0:m0+16, k0:k1] * B[n0:n0+16, k0:k1]^T  (B K-contiguous; A too, or
// stored transposed when AT). Terms are added small-first: lo*hi, hi*lo, hi*hi.
template <int SPLIT, bool AT = false>
KDA_DEV void mma(f32x4& acc, const Panel& A, int m0, const Panel& B, int n0, int k0, int k1) {
  for (int k = k0; k < k1; k += 32) {
    const bf16x8 ah = afrag<AT>(A.hi, A.ld, m0, k);
    const bf16x8 bh = frag(B.hi, B.ld, n0, k);
    if (SPLIT & SPLIT_A) acc = mfma16(afrag<AT>(A.lo, A.ld, m0, k), bh, acc);
    if (SPLIT & SPLIT_B) acc = mfma16(ah, frag(B.lo, B.ld, n0, k), acc);
    acc = mfma16(ah, bh, acc);
  }
}

template <int SPLIT, int KLEN, bool AT = false>
KDA_DEV void mma_k(f32x4& acc, const Panel& A, int m0, const Panel& B, int n0) {
#pragma unroll
  for (int k = 0; k < KLEN; k += 32) {
    const bf16x8 ah = afrag<AT>(A.hi, A.ld, m0, k);
    const bf16x8 bh = frag(B.hi, B.ld, n0, k);
    if (SPLIT & SPLIT_A) acc = mfma16(afrag<AT>(A.lo, A.ld, m0, k), bh, acc);
    if (SPLIT & SPLIT_B) acc = mfma16(ah, frag(B.lo, B.ld, n0, k), acc);
    acc = mfma16(ah, bh, acc);
  }
}

// Register-blocked product over an MT x NT block of 16x16 tiles:
// acc[mt][nt] += A[m0 + 16 mt, k0:k1] * B[n0 + 16 nt, k0:k1]^T.
// Each fragment is read from LDS once per K step and reused across the block.
template <int SPLIT, int MT, int NT>
KDA_DEV void mma_blk(f32x4 (&acc)[MT][NT], const Panel& A, int m0, const Panel& B, int n0,
                     int k0, int k1) {
  for (int k = k0; k < k1; k += 32) {
    bf16x8 ah[MT], al[MT], bh[NT], bl[NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      ah[mt] = frag(A.hi, A.ld, m0 + 16 * mt, k);
      if (SPLIT & SPLIT_A) al[mt] = frag(A.lo, A.ld, m0 + 16 * mt, k);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      bh[nt] = frag(B.hi, B.ld, n0 + 16 * nt, k);
      if (SPLIT & SPLIT_B) bl[nt] = frag(B.lo, B.ld, n0 + 16 * nt, k);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (SPLIT & SPLIT_A) acc[mt][nt] = mfma16(al[mt], bh[nt], acc[mt][nt]);
        if (SPLIT & SPLIT_B) acc[mt][nt] = mfma16(ah[mt], bl[nt], acc[mt][nt]);
        acc[mt][nt] = mfma16(ah[mt], bh[nt], acc[mt][nt]);
      }
  }
}

// One row of tiles: acc[nt] += A[m0:m0+16] * B[n0 + 16 nt]^T. AT / BT: the
// panel stores its operand transposed, [k][m] / [k][n] (read by LDS transpose loads).
template <int SPLIT, int NT, bool AT = false, bool BT = false>
KDA_DEV void mma_row(f32x4 (&acc)[NT], const Panel& A, int m0, const Panel& B, int n0, int k0,
                     int k1) {
  for (int k = k0; k < k1; k += 32) {
    const bf16x8 ah = afrag<AT>(A.hi, A.ld, m0, k);
    bf16x8 al;
    if (SPLIT & SPLIT_A) al = afrag<AT>(A.lo, A.ld, m0, k);
    bf16x8 bh[NT], bl[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      bh[nt] = afrag<BT>(B.hi, B.ld, n0 + 16 * nt, k);
      if (SPLIT & SPLIT_B) bl[nt] = afrag<BT>(B.lo, B.ld, n0 + 16 * nt, k);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (SPLIT & SPLIT_A) acc[nt] = mfma16(al, bh[nt], acc[nt]);
      if (SPLIT & SPLIT_B) acc[nt] = mfma16(ah, bl[nt], acc[nt]);
      acc[nt] = mfma16(ah, bh[nt], acc[nt]);
    }
  }
}

// acc += A[m0:m0+16, k0:k0+16] * B[n0:n0+16, k0:k0+16]^T: a K = 16 product on
// the K = 32 instruction. Lanes 32..63 carry K = 16..31, which is zeroed (they
// read the same in-range elements as lanes 0..31, then drop them).
// With AT the A panel stores A transposed, [k][m] (LDS transpose loads; lanes
// 32..63 again address the rows of lanes 0..31).
template <int SPLIT, bool AT = false>
KDA_DEV void mma_k16(f32x4& acc, const Panel& A, int m0, const Panel& B, int n0, int k0) {
  const int l = lane_id();
  const bool on = l < 32;
  const int ko = k0 + ((l >> 4) & 1) * 8;
  const int ar = (m0 + (l & 15)) * A.ld + ko, br = (n0 + (l & 15)) * B.ld + ko;
  const bf16x8 z = {};
  auto aload = [&](const bf16* p) -> bf16x8 {
    if (!AT) return *reinterpret_cast<const bf16x8*>(p + ar);
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const int s = l & 15;
    const bf16* a = p + (k0 + 8 * ((l >> 4) & 1) + (s >> 2)) * A.ld + m0 + 4 * (s & 3);
    const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a));
    const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 4 * A.ld));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  const bf16x8 ah = on ? aload(A.hi) : z;
  const bf16x8 bh = on ? *reinterpret_cast<const bf16x8*>(B.hi + br) : z;
  if (SPLIT & SPLIT_A) {
    const bf16x8 al = on ? aload(A.lo) : z;
    acc = mfma16(al, bh, acc);
  }
  if (SPLIT & SPLIT_B) {
    const bf16x8 bl = on ? *reinterpret_cast<const bf16x8*>(B.lo + br) : z;
    acc = mfma16(ah, bl, acc);
  }
  acc = mfma16(ah, bh, acc);
}

// Split-store 8 consecutive fp32 values (16-byte aligned destination).
KDA_DEV void put8(const Panel& P, int row, int col, const float* x) {
  bf16x8 h, w;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = f2bf(x[i]);
    w[i] = f2bf(x[i] - bf2f(h[i]));
  }
  *reinterpret_cast<bf16x8*>(P.hi + row * P.ld + col) = h;
  if (P.lo) *reinterpret_cast<bf16x8*>(P.lo + row * P.ld + col) = w;
}

// D tile at (m0, n0) -> panel laid out [n][m] (the tile's rows become the
// panel's contiguous K axis): one 8-byte write per plane and lane.
KDA_DEV void store_tile_t(const f32x4& acc, const Panel& P, int m0, int n0) {
  const int l = lane_id();
  bf16x4 h, w;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = f2bf(acc[i]);
    w[i] = f2bf(acc[i] - bf2f(h[i]));
  }
  const int off = (n0 + (l & 15)) * P.ld + m0 + 4 * (l >> 4);
  *reinterpret_cast<bf16x4*>(P.hi + off) = h;
  if (P.lo) *reinterpret_cast<bf16x4*>(P.lo + off) = w;
}

// Split-store 4 consecutive fp32 values (8-byte aligned destination).
KDA_DEV void put4(const Panel& P, int row, int col, f32x4 x) {
  bf16x4 h, w;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = f2bf(x[i]);
    w[i] = f2bf(x[i] - bf2f(h[i]));
  }
  *reinterpret_cast<bf16x4*>(P.hi + row * P.ld + col) = h;
  if (P.lo) *reinterpret_cast<bf16x4*>(P.lo + row * P.ld + col) = w;
}

// Offset of this lane's 4 values of tile (rb, cb) in a tile-ordered matrix
// with 8 column blocks (128 columns): one 16-byte vector per lane.
KDA_DEV int tile_off(int rb, int cb) { return (rb * 8 + cb) * 256 + 4 * lane_id(); }

// Row / column of element i (0..3) of this lane's D tile.
KDA_DEV int drow(int i) { return 4 * (lane_id() >> 4) + i; }
KDA_DEV int dcol() { return lane_id() & 15; }

// Cross-lane exchange inside a 16-lane row by DPP (no LDS traffic): lane j
// receives the value of lane j ^ M for M = 1 (quad swap), 3 (quad reverse),
// 7 (half-row mirror) and 15 (row mirror).
template <int M>
KDA_DEV float row_xor(float v) {
  static_assert(M == 1 || M == 3 || M == 7 || M == 15, "row_xor mask");
  constexpr int ctrl = M == 1 ? 0xB1 : M == 3 ? 0x1B : M == 7 ? 0x141 : 0x140;
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), ctrl, 0xF, 0xF, true));
}

// Sum over the 16 lanes of a row (every lane gets the total).
KDA_DEV float row_sum16(float v) {
  v += row_xor<1>(v);
  v += row_xor<3>(v);
  v += row_xor<7>(v);
  return v + row_xor<15>(v);
}

template <int M, int HALF>
KDA_DEV void row_transpose_level(float* x, bool up) {
#pragma unroll
  for (int k = 0; k < HALF; ++k) {
    // opaque copies: a select between two array elements would otherwise be
    // folded into a dynamically indexed read of the whole array
    float lo = x[k], hi = x[HALF + k];
    asm("" : "+v"(lo), "+v"(hi));
    x[k] = (up ? hi : lo) + row_xor<M>(up ? lo : hi);
  }
}

// Transposing sum over a 16-lane row: each lane enters with 16 partial values
// x[0..15]; lane j (j = lane & 15) returns the row total of value j. Each
// level pairs lanes that differ in one more bit of j and halves the values a
// lane keeps (15 exchanges in all).
KDA_DEV float row_transpose_sum16(float* x, int j) {
  row_transpose_level<15, 8>(x, j & 8);
  row_transpose_level<7, 4>(x, j & 4);
  row_transpose_level<3, 2>(x, j & 2);
  row_transpose_level<1, 1>(x, j & 1);
  return x[0];
}

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e^-|x|), on the hardware
// base-2 exponential and logarithm. log1p(y) is taken as log(u) y / (u - 1)
// with u = 1 + y rounded (y itself when u rounds to 1): the rounding of u
// cancels between log(u) and u - 1, so small y (x far below zero) keeps its
// relative accuracy instead of losing it to 1 + y (D. Goldberg, "What every
// computer scientist should know about floating-point arithmetic", 1991).
KDA_DEV float softplus(float x) {
  const float y = __builtin_amdgcn_exp2f(-fabsf(x) * LOG2E);
  const float u = 1.f + y;
  const float l1p = u == 1.f ? y
                             : __builtin_amdgcn_logf(u) * 0.6931471805599453f *
                                   (y * __builtin_amdgcn_rcpf(u - 1.f));
  return fmaxf(x, 0.f) + l1p;
}
KDA_DEV float sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * LOG2E));
}

// The per-token log forget gate g for (token t, head h, channel c).
KDA_DEV float gate_value(const void* gate, int raw, const float* A_log, const float* dt_bias,
                         int64_t t, int h, int H, int c) {
  const int64_t idx = (t * H + h) * HD + c;
  if (!raw) return reinterpret_cast<const float*>(gate)[idx];
  const float a = bf2f(reinterpret_cast<const bf16*>(gate)[idx]);
  return -__expf(A_log[h]) * softplus(a + dt_bias[h * HD + c]);
}

}  // namespace kda
