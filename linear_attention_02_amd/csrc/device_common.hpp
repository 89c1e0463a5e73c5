// device_common.hpp -- register-fragment toolkit for the gfx950 linear
// attention kernels.
//
// Every kernel in this library is built from 16x16 MFMA tiles.  One wave64 is
// one independent worker; data moves between the operand and accumulator
// layouts in registers (the LDS only stages each wave's own input chunks),
// using two facts about CDNA MFMAs:
//
//   * accumulator ("C") layout of a 16x16 tile: lane l holds D[4g+r][n] for
//     r = 0..3, where n = l & 15 and g = l >> 4;
//   * operand layout of a 16-wide k slice: lane l holds A[n][4g+r] (A operand,
//     row n) or B[4g+r][n] (B operand, column n), r = 0..3.
//
// So an accumulator tile, rounded to the operand type, *is* an operand tile
// whose k index is the tile's row index -- the token-contracting products
// (A V and phi(K)^T V) consume accumulators of earlier products directly.
// Where a tile has to change orientation, multiplying it by an identity
// matrix on the MFMA pipe transposes it exactly (one non-zero product per
// output, accumulated in fp32).
//
// Feature and value columns are visited in the order pi(kt, g, r) below, so
// that a lane's global loads and stores are 16-byte vectors over 8 adjacent
// columns.  pi is a permutation of 0..63; every product contracts or indexes
// with the same pi on both sides, so results are in natural order in memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace linattn {

typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x2 __attribute__((__vector_size__(2 * sizeof(float))));

constexpr int kWave = 64;
constexpr int kD = 64;      // C = M = 64 features / value columns
constexpr int kChunk = 64;  // tokens per chunk (four 16-row tiles)

// Column visited by lane group g, register r, in k-tile (or column tile) kt.
__device__ __host__ inline constexpr int pi_col(int kt, int g, int r) {
  return 32 * (kt >> 1) + 8 * g + 4 * (kt & 1) + r;
}

__device__ inline f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------------------
// phi(x) = elu(x) + 1: x + 1 for x > 0, e^x otherwise ("Why Replace
// Attention?", §5.3).  Because e^x >= 1 + x for every x, phi(x) is the
// median of {x + 1, e^x, 1}: for x > 0, 1 < x + 1 <= e^x; for x <= 0,
// x + 1 <= e^x <= 1.  That is one v_med3_f32 instead of a compare and a
// select.  e^x is the device's exp2 of x * log2(e).
// ---------------------------------------------------------------------------
__device__ inline float phi(float x) { return __builtin_amdgcn_fmed3f(x + 1.f, __expf(x), 1.f); }

// ---------------------------------------------------------------------------
// The scale of one query row's phi(q).
//
// o_i is a ratio of two sums that are both linear in phi(q_i), so o_i does not
// change when phi(q_i) is multiplied by any positive constant ("Why Replace
// Attention?", §5.4: the weights are normalised per query).  A power of two
// changes no rounding, so it changes nothing at all unless the unscaled row
// would leave fp32's range: a row whose features are all far below zero has
// e^x underflow (at x < -87 in fp32), and a row with features near 1e19 or
// beyond overflows its products with phi(K).  Rows whose largest feature m
// lies in [kPhiQLow, kPhiQHigh] keep phi unchanged; the others are scaled so
// that their largest phi lies in [1, 2):
//   m > kPhiQHigh:  phi(x) * 2^-e with e = floor(log2(m + 1));
//   m < kPhiQLow:   e^x * 2^-e = 2^(x log2(e) - e) with e = floor(m log2(e)),
//                   evaluated as one exp2 so that nothing underflows first.
// ---------------------------------------------------------------------------
constexpr float kPhiQLow = -8.f;
constexpr float kPhiQHigh = 65535.f;
constexpr float kLog2e = 1.44269504088896340736f;

// phi(x) * 2^-(epos) when eneg == 0, else 2^(x log2(e) - eneg) (eneg < 0 is an
// integer; then every feature of the row is below kPhiQLow).
__device__ inline float phi_row_scaled(float x, float eneg, int epos) {
  const float p = eneg != 0.f ? __builtin_amdgcn_exp2f(x * kLog2e - eneg) : phi(x);
  return __builtin_amdgcn_ldexpf(p, -epos);
}

// The row scale (eneg, epos) from the row's largest raw feature m.
__device__ inline void phi_row_scale(float m, float &eneg, int &epos) {
  eneg = 0.f;
  epos = 0;
  if (m > kPhiQHigh) {
    epos = __builtin_amdgcn_frexp_expf(m + 1.f) - 1;  // m + 1 = f 2^(epos + 1), f in [0.5, 1)
  } else if (m < kPhiQLow) {
    eneg = floorf(m * kLog2e);
  }
}

// bf16 <-> fp32.  Widening is exact; narrowing is the hardware's
// round-to-nearest-even conversion of two values at once
// (v_cvt_pk_bf16_f32).
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ---------------------------------------------------------------------------
// Operand fragments: four consecutive-k values per lane for one 16-wide k
// slice.  Element type E is the MFMA operand type.
// ---------------------------------------------------------------------------
template <class E> struct Frag;

template <> struct Frag<__bf16> {
  // Element r lives in half (r & 1) of w[r >> 1].  A vector rather than an
  // array, so that fragments stored in arrays are always accessed as whole
  // values and stay in registers.
  u32x2 w;
};
template <> struct Frag<float> {
  float v[4];
};

template <class E> __device__ inline Frag<E> frag_zero();
template <> __device__ inline Frag<__bf16> frag_zero<__bf16>() { return {u32x2{0u, 0u}}; }
template <> __device__ inline Frag<float> frag_zero<float>() { return {{0.f, 0.f, 0.f, 0.f}}; }

// Accumulator (fp32) -> operand fragment.
template <class E> __device__ inline Frag<E> to_frag(f32x4 a);
template <> __device__ inline Frag<__bf16> to_frag<__bf16>(f32x4 a) {
  return {u32x2{pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3])}};
}
template <> __device__ inline Frag<float> to_frag<float>(f32x4 a) { return {{a[0], a[1], a[2], a[3]}}; }

// Constant B fragments: the identity (B[k][n] = [k == n]) and all-ones.
template <class E> __device__ inline Frag<E> frag_identity(int n16, int g);
template <> __device__ inline Frag<__bf16> frag_identity<__bf16>(int n16, int g) {
  const uint32_t one = 0x3f80u;
  const int d = n16 - 4 * g;  // the one register (if any) holding the 1
  Frag<__bf16> f;
  f.w[0] = (d == 0 ? one : 0u) | (d == 1 ? one << 16 : 0u);
  f.w[1] = (d == 2 ? one : 0u) | (d == 3 ? one << 16 : 0u);
  return f;
}
template <> __device__ inline Frag<float> frag_identity<float>(int n16, int g) {
  const int d = n16 - 4 * g;
  return {{d == 0 ? 1.f : 0.f, d == 1 ? 1.f : 0.f, d == 2 ? 1.f : 0.f, d == 3 ? 1.f : 0.f}};
}
template <class E> __device__ inline Frag<E> frag_ones();
template <> __device__ inline Frag<__bf16> frag_ones<__bf16>() { return {u32x2{0x3f803f80u, 0x3f803f80u}}; }
template <> __device__ inline Frag<float> frag_ones<float>() { return {{1.f, 1.f, 1.f, 1.f}}; }

// ---------------------------------------------------------------------------
// acc += A * B over a list of 16-wide k slices.
// bf16: pairs of slices go through one v_mfma_f32_16x16x32_bf16 (a lane's 8
// operand values are the two slices' 4 each; A and B use the same placement,
// so the contraction pairs matching k); a single slice goes through the same
// instruction with a zero slice as its partner, which adds nothing to any
// sum.  v_mfma_f32_16x16x16_bf16 is not used: on MI355X its results were
// measured to be read stale (in the last two accumulator registers) by a
// dependent 16x16x32 product three instructions later, and in a dQ tile read
// by vector instructions at the distances the compiler allows for the
// 16x16x32 form.  fp32: four v_mfma_f32_16x16x4_f32 per slice,
// register r of every lane in instruction r.
// ---------------------------------------------------------------------------
__device__ inline f32x4 mma2_bf16(f32x4 acc, const Frag<__bf16> &a0, const Frag<__bf16> &a1,
                                  const Frag<__bf16> &b0, const Frag<__bf16> &b1) {
  const u32x4 a = __builtin_shufflevector(a0.w, a1.w, 0, 1, 2, 3);
  const u32x4 b = __builtin_shufflevector(b0.w, b1.w, 0, 1, 2, 3);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc,
                                                 0, 0, 0);
}
__device__ inline f32x4 mma1_bf16(f32x4 acc, const Frag<__bf16> &a, const Frag<__bf16> &b) {
  const Frag<__bf16> zero = {u32x2{0u, 0u}};
  return mma2_bf16(acc, a, zero, b, zero);
}
__device__ inline f32x4 mma1_f32(f32x4 acc, const Frag<float> &a, const Frag<float> &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[0], b.v[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[1], b.v[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[2], b.v[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[3], b.v[3], acc, 0, 0, 0);
  return acc;
}

// One contraction step on a pair of 16-wide k slices (k0, k1):
//   acc += A[:, k0] B[k0, :] + A[:, k1] B[k1, :].
// bf16: a single v_mfma_f32_16x16x32_bf16.  fp32: eight v_mfma_f32_16x16x4_f32.
// Callers order their loops k-outer / tiles-inner, so consecutive MFMAs
// write different accumulators and issue back to back.
template <class E>
__device__ inline f32x4 mac2(f32x4 acc, const Frag<E> &a0, const Frag<E> &a1, const Frag<E> &b0,
                             const Frag<E> &b1);
template <>
__device__ inline f32x4 mac2<__bf16>(f32x4 acc, const Frag<__bf16> &a0, const Frag<__bf16> &a1,
                                     const Frag<__bf16> &b0, const Frag<__bf16> &b1) {
  return mma2_bf16(acc, a0, a1, b0, b1);
}
template <>
__device__ inline f32x4 mac2<float>(f32x4 acc, const Frag<float> &a0, const Frag<float> &a1, const Frag<float> &b0,
                                    const Frag<float> &b1) {
  return mma1_f32(mma1_f32(acc, a0, b0), a1, b1);
}
// Single k slice.
template <class E> __device__ inline f32x4 mac1(f32x4 acc, const Frag<E> &a, const Frag<E> &b);
template <> __device__ inline f32x4 mac1<__bf16>(f32x4 acc, const Frag<__bf16> &a, const Frag<__bf16> &b) {
  return mma1_bf16(acc, a, b);
}
template <> __device__ inline f32x4 mac1<float>(f32x4 acc, const Frag<float> &a, const Frag<float> &b) {
  return mma1_f32(acc, a, b);
}

// Re-orient a tile: the lane that holds row n of X across its registers
// (X[n][4g+r], operand layout) receives column n instead (X[4g+r][n],
// accumulator layout).  Computed as X * I on the MFMA pipe; exact, because
// each output has one non-zero product (inputs are finite).
template <class E>
__device__ inline f32x4 transpose_tile(const Frag<E> &x, const Frag<E> &ident) {
  return mac1<E>(zero4(), x, ident);
}

// ---------------------------------------------------------------------------
// fp32 row slabs.  A 16-row slab of a [rows][64] matrix is held so that lane
// (n, g) has row n's columns pi(kt, g, 0..3) for kt = 0..3: two 8-column
// runs, at columns 8g and 32 + 8g.  The forward kernels fill slabs from a
// chunk staged in LDS, the fp32 backward straight from global memory.
// ---------------------------------------------------------------------------
template <class E> struct Slab;  // raw (unconverted) data of one lane's row piece

template <> struct Slab<float> {
  f32x4 h[2][2];  // h[x][y] = 4 floats at columns 32x + 8g + 4y
};

template <class E> __device__ inline void slab_zero(Slab<E> &s);
template <> __device__ inline void slab_zero<float>(Slab<float> &s) {
  for (int x = 0; x < 2; ++x)
    for (int y = 0; y < 2; ++y) s.h[x][y] = zero4();
}

// row points at the first element of the lane's row.
template <class E> __device__ inline void slab_load(Slab<E> &s, const E *row, int g);
template <> __device__ inline void slab_load<float>(Slab<float> &s, const float *row, int g) {
  const f32x4 *p = reinterpret_cast<const f32x4 *>(row);
  s.h[0][0] = __builtin_nontemporal_load(p + 2 * g);
  s.h[0][1] = __builtin_nontemporal_load(p + 2 * g + 1);
  s.h[1][0] = __builtin_nontemporal_load(p + 8 + 2 * g);
  s.h[1][1] = __builtin_nontemporal_load(p + 8 + 2 * g + 1);
}

// Slab -> 4 operand fragments (kt = 0..3), optionally through phi.
template <class E> __device__ inline void slab_to_frags(const Slab<E> &s, Frag<E> f[4], bool apply_phi);

template <>
__device__ inline void slab_to_frags<float>(const Slab<float> &s, Frag<float> f[4], bool apply_phi) {
  for (int x = 0; x < 2; ++x)
    for (int y = 0; y < 2; ++y) {
      const f32x4 v = s.h[x][y];
      Frag<float> &d = f[2 * x + y];
#pragma unroll
      for (int r = 0; r < 4; ++r) d.v[r] = apply_phi ? phi(v[r]) : v[r];
    }
}

// Store 8 output values of one row at columns 32x + 8g (two transposed output
// tiles 2x and 2x+1, register r = column 32x + 8g + 4y + r).
template <class E> __device__ inline void store_row8(E *row, int g, int x, f32x4 lo, f32x4 hi);
template <>
__device__ inline void store_row8<float>(float *row, int g, int x, f32x4 lo, f32x4 hi) {
  f32x4 *p = reinterpret_cast<f32x4 *>(row) + 8 * x + 2 * g;
  __builtin_nontemporal_store(lo, p);
  __builtin_nontemporal_store(hi, p + 1);
}

}  // namespace linattn
