// backward_kernels.hpp -- gradients of elu(x)+1 linear attention for gfx950.
//
// The pages state that the gradients can themselves be written as forward and
// reverse cumulative sums, keeping training linear in time and memory
// ("[Paper Review] Transformers are RNNs", §3.5 "Gradient Computation";
// "Transformers Are RNNs: Linear Attention" knowledge note), without printing
// them.  By the chain rule through o_i = phi(q_i)^T S_i / phi(q_i)^T z_i, with
// g_i = dL/do_i and den_i = phi(q_i)^T z_i:
//   a_i = g_i / den_i,   b_i = -(g_i . o_i) / den_i,
//   dphi(q_i) = S_i a_i + b_i z_i                          (prefix state),
//   dphi(k_j) = R_j v_j + r_j,   dv_j = R_j^T phi(k_j)      (suffix state),
//   R_j = sum_{i : j in J(i)} phi(q_i) a_i^T,   r_j = sum_{i : j in J(i)} b_i phi(q_i),
//   dq = dphi(q) * phi'(q),  phi'(x) = min(e^x, 1)  (1 for x > 0, e^x otherwise).
// Regrouped over 64-token chunks like the forward, for the rows i and keys j of
// one chunk with the state of the earlier (S, z) or later (R, r) chunks:
//   D = tril(a V^T + b 1^T)            (D_ij = a_i . v_j + b_i, j <= i)
//   dphi(Q) = D phi(K) + a S^T + b z^T
//   dphi(K) = D^T phi(Q) + V R^T + 1 r^T
//   dV      = tril(phi(Q) phi(K)^T)^T a + phi(K) R
//   R += phi(Q)^T a,  r += phi(Q)^T b   (walking right to left).
// a is never rounded to the operand type: products take g (already exact in
// the input type) as the operand and apply 1/den_i to their fp32 results, or
// to phi(q_i) before its single rounding.
//
// Kernels, causal: the forward's segment totals and prefix scan give S, z at
// every segment start; a left-to-right walk recomputes o in fp32, writes dQ
// and the per-token pair (1/den_i, b_i); a totals pass over Q, dO and those
// pairs gives each segment's sum of phi(q) a^T and b phi(q); the scan run in
// reverse turns them into suffix states; a right-to-left walk writes dK, dV.
// With at most eight segments per head neither scan runs: each walk wave sums
// the totals records it needs itself, in the scan's order.
// Non-causal: S, z are the head's totals; one read pass writes dQ, the pairs
// and per-range partial sums of R, r; a scan totals those; a second read pass
// writes dK and dV.  All products are 16x16 MFMA tiles in the layouts of
// device_common.hpp.  Where a state is needed with its other index as the
// contraction index (S a^T contracts over value columns, the forward read
// over features), the walk transposes it once per chunk with identity
// products (exact: one non-zero term per output).
#pragma once

#include "forward_kernels.hpp"

namespace linattn {

struct BwdParams {
  const void *Q, *K, *V, *dO;
  void *dQ, *dK, *dV;
  long long N;        // tokens per head
  int heads;          // B * H
  int segments;       // causal walks: segments per head
  int seg_chunks;     // 64-token chunks per segment
  int ranges;         // non-causal reads: ranges per head
  int range_chunks;
  float *wsF;         // [heads][recF] records of (S, z)
  int recF;
  float *wsR;         // [heads][recR] records of (R, r)
  int recR;
  f32x2 *stats;       // [heads][stats_stride] pairs (1/den_i, b_i)
  long long stats_stride;
  int sum_in_walk;    // causal: wsF, wsR hold segment totals; each walk sums
                      // its own prefix (suffix) from them
  // Saved-forward backward (backward_saved_kernels.hpp).
  const void *O;      // the forward's output
  const float *rden;  // [heads][stats_stride] 1/den saved by the forward
  float *wsT;         // [heads][recT] records: totals at u + 1, then suffixes
  int recT;
  int walk_k;         // forward segments per walk segment
  int walk_segments;  // walk segments per head
  int rev_segments;   // reverse segments per head (the suffix state's anchors)
  int rev_chunks;     // chunks per reverse segment
  int rev_sum_in_walk;  // wsT holds totals (no suffix scan ran)
};

// Row tiles per chunk of the causal backward walks (32-token chunks): the
// walks hold two states' worth of operands, so the chunk is half the
// forward's to stay within the register file.
constexpr int kBwdTiles = 2;

__device__ inline float phi_prime(float x) { return fminf(__expf(x), 1.f); }

__device__ inline f32x4 frag_f32(const Frag<__bf16> &f) {
  return f32x4{bf16_lo(f.w[0]), bf16_hi(f.w[0]), bf16_lo(f.w[1]), bf16_hi(f.w[1])};
}
__device__ inline f32x4 frag_f32(const Frag<float> &f) { return f32x4{f.v[0], f.v[1], f.v[2], f.v[3]}; }

template <class E, int NT> __device__ inline void zero_rows(Frag<E> f[NT][4], int rows, int n16) {
#pragma unroll
  for (int it = 0; it < NT; ++it)
    if (16 * it + n16 >= rows)
#pragma unroll
      for (int c = 0; c < 4; ++c) f[it][c] = frag_zero<E>();
}
template <class E, int NT> __device__ inline void zero_tokens(Frag<E> f[NT][4], int rows, int g) {
#pragma unroll
  for (int it = 0; it < NT; ++it)
#pragma unroll
    for (int c = 0; c < 4; ++c) mask_tokens(f[it][c], 16 * it + 4 * g, rows);
}

// S^T as an A operand (rows = value column, k = feature: the forward read)
// -> S as an A operand (rows = feature, k = value column), per tile.
template <class E>
__device__ inline void transposed_state_operands(const StateOperands<E> &so, Frag<E> st[4][4], const Frag<E> &ident) {
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) st[ct][mt] = to_frag<E>(transpose_tile<E>(so.sa[ct][mt], ident));
}

// Row-layout fragments of NT row tiles of a [rows][64] fp32 matrix, straight
// from global memory (rows >= `rows` read as zero).
template <int NT>
__device__ inline void load_rows_f32(Frag<float> f[NT][4], const float *src, long long t0, int rows, int n16, int g) {
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    const int row = 16 * it + n16;
    Slab<float> s;
    if (row < rows) {
      slab_load<float>(s, src + (t0 + row) * kD, g);
    } else {
      slab_zero<float>(s);
    }
    slab_to_frags<float>(s, f[it], false);
  }
}

template <class E, int NT> __device__ inline void phi_all(Frag<E> f[NT][4]) {
#pragma unroll
  for (int it = 0; it < NT; ++it)
#pragma unroll
    for (int c = 0; c < 4; ++c) phi_frag<E>(f[it][c]);
}

// Per-token pairs (1/den, b) of a chunk staged in LDS behind the tensors:
// pair t of the chunk is f32x2 t of the region.  Fetched 16 bytes (two
// pairs) per lane.
template <int NT>
__device__ inline void stage_stats(u32x4 *region, const f32x2 *src, long long t0, int rows, int lane) {
  if (lane < 8 * NT && 2 * lane < rows)
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const u32x4 *>(src + t0) + lane, (lds_void *)region, 16, 0, 0);
}
// Pairs of the four tokens 16 it + 4 g + r (token layout): 1/den and b.
__device__ inline void stats_tok(const u32x4 *region, int it, int g, f32x4 &rd, f32x4 &b) {
  const f32x4 lo = __builtin_bit_cast(f32x4, region[8 * it + 2 * g]);
  const f32x4 hi = __builtin_bit_cast(f32x4, region[8 * it + 2 * g + 1]);
  rd = f32x4{lo[0], lo[2], hi[0], hi[2]};
  b = f32x4{lo[1], lo[3], hi[1], hi[3]};
}
// Pair of token 16 it + n (row layout).
__device__ inline f32x2 stats_row(const u32x4 *region, int it, int n16) {
  return reinterpret_cast<const f32x2 *>(region)[16 * it + n16];
}

// ---------------------------------------------------------------------------
// Left-to-right walk: dQ and the per-token pairs.
// ---------------------------------------------------------------------------
// Fragments of one chunk (NT row tiles):
//   qraw  Q, row layout, raw          kf  phi(K), row layout (keys >= rows zero)
//   kt    phi(K), token layout        vt  V, token layout (tokens >= rows zero)
//   vf    V, row layout (rows >= rows zero)    gf  dO, row layout
template <class E, int NT, bool kFull>
__device__ inline void bwd_f_chunk(State &st, const Frag<E> qraw[NT][4], const Frag<E> kf[NT][4],
                                   const Frag<E> kt[NT][4], const Frag<E> vt[NT][4], const Frag<E> vf[NT][4],
                                   const Frag<E> gf[NT][4], int rows, long long t0, E *dQh, f32x2 *stats_h, int n16,
                                   int g, const Frag<E> &ident) {
  StateOperands<E> so;
  state_operands<E>(st, so);  // S^T, z as A operands: the forward read
  Frag<E> sf[4][4];
  transposed_state_operands<E>(so, sf, ident);  // S as A operand: the S a^T term
  const Frag<E> ones = frag_ones<E>();
  float keep_rd = 0.f, keep_b = 0.f;
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    Frag<E> qf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      qf[c] = qraw[it][c];
      phi_frag<E>(qf[c]);
    }
    // Forward recomputation: num^T, den for the 16 tokens of row tile it.
    f32x4 nt[4] = {zero4(), zero4(), zero4(), zero4()};
    f32x4 dt = zero4();
    state_read<E>(so, qf, nt, dt);
    f32x4 at[NT];
#pragma unroll
    for (int jt = 0; jt <= it; ++jt) at[jt] = zero4();
#pragma unroll
    for (int kp = 0; kp < 2; ++kp)
#pragma unroll
      for (int jt = 0; jt <= it; ++jt)
        at[jt] = mac2<E>(at[jt], kf[jt][2 * kp], kf[jt][2 * kp + 1], qf[2 * kp], qf[2 * kp + 1]);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * g + r > n16) at[it][r] = 0.f;
    Frag<E> af[NT];
#pragma unroll
    for (int jt = 0; jt <= it; ++jt) af[jt] = to_frag<E>(at[jt]);
#pragma unroll
    for (int jp = 0; 2 * jp + 1 <= it; ++jp) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) nt[mt] = mac2<E>(nt[mt], vt[2 * jp][mt], vt[2 * jp + 1][mt], af[2 * jp], af[2 * jp + 1]);
      dt = mac2<E>(dt, ones, ones, af[2 * jp], af[2 * jp + 1]);
    }
    if ((it & 1) == 0) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) nt[mt] = mac1<E>(nt[mt], vt[it][mt], af[it]);
      dt = mac1<E>(dt, ones, af[it]);
    }
    // a = g / den, b = -(g . o) / den = -(g . num) / den^2 for token n.  a is
    // never rounded: the products below take g (exact in the input type) as
    // the operand and apply 1/den to their fp32 results, column by column.
    const float rd = __builtin_amdgcn_rcpf(dt[0]);
    float gn = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const f32x4 ga = frag_f32(gf[it][mt]);
#pragma unroll
      for (int r = 0; r < 4; ++r) gn += ga[r] * nt[mt][r];
    }
    gn += __shfl_xor(gn, 16);
    gn += __shfl_xor(gn, 32);
    const float b = -gn * rd * rd;
    // D^T (key j, query i) = (v_j . g_i) / den_i + b_i for j <= i.
    f32x4 dtt[NT];
#pragma unroll
    for (int jt = 0; jt <= it; ++jt) {
      f32x4 d = zero4();
      d = mac2<E>(d, vf[jt][0], vf[jt][1], gf[it][0], gf[it][1]);
      d = mac2<E>(d, vf[jt][2], vf[jt][3], gf[it][2], gf[it][3]);
      dtt[jt] = d * rd + b;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * g + r > n16) dtt[it][r] = 0.f;
    Frag<E> df[NT];
#pragma unroll
    for (int jt = 0; jt <= it; ++jt) df[jt] = to_frag<E>(dtt[jt]);
    // dphi(Q)^T = phi(K)^T D^T + (S g^T) / den + z b^T.
    f32x4 dq[4] = {zero4(), zero4(), zero4(), zero4()};
    f32x4 sg[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
    for (int jp = 0; 2 * jp + 1 <= it; ++jp)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) dq[ct] = mac2<E>(dq[ct], kt[2 * jp][ct], kt[2 * jp + 1][ct], df[2 * jp], df[2 * jp + 1]);
    if ((it & 1) == 0)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) dq[ct] = mac1<E>(dq[ct], kt[it][ct], df[it]);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      sg[ct] = mac2<E>(sg[ct], sf[ct][0], sf[ct][1], gf[it][0], gf[it][1]);
      sg[ct] = mac2<E>(sg[ct], sf[ct][2], sf[ct][3], gf[it][2], gf[it][3]);
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const f32x4 qv = frag_f32(qraw[it][ct]);
#pragma unroll
      for (int r = 0; r < 4; ++r) dq[ct][r] = (dq[ct][r] + sg[ct][r] * rd + st.z[ct][r] * b) * phi_prime(qv[r]);
    }
    store_tiles<E, kFull>(dQh, t0 + 16 * it, rows - 16 * it, dq, n16, g);
    if (g == it) {
      keep_rd = rd;
      keep_b = b;
    }
  }
  // Lane (n, g < NT) holds the pair of token 16 g + n: one store per chunk.
  if (g < NT && (kFull || 16 * g + n16 < rows)) stats_h[t0 + 16 * g + n16] = f32x2{keep_rd, keep_b};
  state_update<E, NT>(st, kt, vt);
}

template <int NT, bool kFull>
__device__ inline void bwd_f_chunk_lds(State &st, u32x4 *slot, const __bf16 *const src[4], long long t0,
                                       long long t_end, int rows, __bf16 *dQh, f32x2 *stats_h, int lane, int n16,
                                       int g, const Frag<__bf16> &ident) {
  typedef __bf16 E;
  constexpr int kT = 16 * NT;
  Frag<E> qraw[NT][4], kf[NT][4], vf[NT][4], gf[NT][4], vt[NT][4], kt[NT][4];
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    lds_row_frags<NT>(slot, 0, it, lane, qraw[it]);
    lds_row_frags<NT>(slot, 1, it, lane, kf[it]);
    lds_row_frags<NT>(slot, 2, it, lane, vf[it]);
    lds_row_frags<NT>(slot, 3, it, lane, gf[it]);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) vt[it][mt] = lds_tok_frag<NT>(slot, 2, it, mt, lane);
  }
  wait_lgkmcnt0();  // the slot is refilled only after every lane's read of it returned
  if (t0 + kT < t_end) stage_issue<4, NT>(slot, src, t0 + kT, (int)min<long long>(kT, t_end - t0 - kT), n16, g);
  phi_all<E, NT>(kf);
  if (!kFull) {
    zero_rows<E, NT>(kf, rows, n16);
    zero_rows<E, NT>(vf, rows, n16);
    zero_tokens<E, NT>(vt, rows, g);
  }
  row_to_tok<E, NT>(kf, kt, ident);
  bwd_f_chunk<E, NT, kFull>(st, qraw, kf, kt, vt, vf, gf, rows, t0, dQh, stats_h, n16, g, ident);
}

template <class E> __device__ inline void bwd_walk_f(const BwdParams &p) {
  const int worker = blockIdx.x;
  const int h = worker % p.heads;
  const int s = worker / p.heads;
  if (s >= p.segments) return;
  const int lane = threadIdx.x;
  const int n16 = lane & 15, g = lane >> 4;
  const long long base = (long long)h * p.N * kD;
  const E *Qh = reinterpret_cast<const E *>(p.Q) + base;
  const E *Kh = reinterpret_cast<const E *>(p.K) + base;
  const E *Vh = reinterpret_cast<const E *>(p.V) + base;
  const E *Gh = reinterpret_cast<const E *>(p.dO) + base;
  E *dQh = reinterpret_cast<E *>(p.dQ) + base;
  f32x2 *stats_h = p.stats + (long long)h * p.stats_stride;
  const long long t_begin = (long long)s * p.seg_chunks * kChunk;
  long long t_end = t_begin + (long long)p.seg_chunks * kChunk;
  if (t_end > p.N) t_end = p.N;
  const Frag<E> ident = frag_identity<E>(n16, g);
  constexpr int NT = kBwdTiles;
  constexpr int kT = 16 * NT;

  State st;
  if (p.recF > 0 && !p.sum_in_walk) {
    state_load_record(st, p.wsF + ((long long)h * p.recF + s) * kStateFloats, lane, g);
  } else {
    state_zero(st);
    if (p.recF > 0) state_add_records(st, p.wsF + (long long)h * p.recF * kStateFloats, s, kStateFloats, lane, g);
  }
  if constexpr (std::is_same<E, __bf16>::value) {
    __shared__ u32x4 slot[Slot<4, NT>::kVec];
    const __bf16 *src[4] = {Qh, Kh, Vh, Gh};
    if (t_begin < t_end) stage_issue<4, NT>(slot, src, t_begin, (int)min<long long>(kT, t_end - t_begin), n16, g);
    // The state's loads (and the first chunk's) land here, before the chunk
    // loop: left in flight, they would make the compiler wait for every
    // outstanding memory operation, earlier output stores included, at the
    // state's first use on every chunk.
    wait_vmcnt<0>();
    for (long long t0 = t_begin; t0 < t_end; t0 += kT) {
      const int rows = (int)min<long long>(kT, t_end - t0);
      // Outstanding: this chunk's loads, then the previous (full) chunk's
      // 2 NT dQ stores and one pair store; they retire in order.
      if (t0 == t_begin) {
        wait_vmcnt<0>();
      } else {
        wait_vmcnt<2 * NT + 1>();
      }
      if (rows == kT) {
        bwd_f_chunk_lds<NT, true>(st, slot, src, t0, t_end, rows, dQh, stats_h, lane, n16, g, ident);
      } else {
        bwd_f_chunk_lds<NT, false>(st, slot, src, t0, t_end, rows, dQh, stats_h, lane, n16, g, ident);
      }
    }
  } else {
    // The state's loads land here, before the chunk
    // loop: left in flight, they would make the compiler wait for every
    // outstanding memory operation, earlier output stores included, at the
    // state's first use on every chunk.
    wait_vmcnt<0>();
    for (long long t0 = t_begin; t0 < t_end; t0 += kT) {
      const int rows = (int)min<long long>(kT, t_end - t0);
      Frag<E> qraw[NT][4], kf[NT][4], vf[NT][4], gf[NT][4], vt[NT][4], kt[NT][4];
      load_rows_f32<NT>(qraw, Qh, t0, rows, n16, g);
      load_rows_f32<NT>(kf, Kh, t0, rows, n16, g);
      load_rows_f32<NT>(vf, Vh, t0, rows, n16, g);
      load_rows_f32<NT>(gf, Gh, t0, rows, n16, g);
      phi_all<E, NT>(kf);
      zero_rows<E, NT>(kf, rows, n16);
      row_to_tok<E, NT>(kf, kt, ident);
      row_to_tok<E, NT>(vf, vt, ident);
      bwd_f_chunk<E, NT, false>(st, qraw, kf, kt, vt, vf, gf, rows, t0, dQh, stats_h, n16, g, ident);
    }
  }
}

__global__ __launch_bounds__(64, 1) void bwd_walk_f_kernel_bf16(BwdParams p) { bwd_walk_f<__bf16>(p); }
__global__ __launch_bounds__(64, 1) void bwd_walk_f_kernel_f32(BwdParams p) { bwd_walk_f<float>(p); }

// ---------------------------------------------------------------------------
// Per-segment sums of phi(Q)^T a and phi(Q)^T b (the reverse pass's totals),
// for segments 1..P-1 (segment 0's sum is never needed by a suffix).
// ---------------------------------------------------------------------------
// acc += (phi(Q)/den)^T G and phi(Q)^T b over NT row tiles, from token-layout
// fragments of raw Q (qr) and dO (gt, tokens past the end zero) and the pairs
// in token layout (zero past the end).  phi(q) is computed in fp32 and
// rounded once, plain and scaled by 1/den; tokens past the end (1/den = 0)
// contribute nothing whatever their slot holds.
template <class E, int NT>
__device__ inline void reverse_sums(State &acc, const Frag<E> qr[NT][4], const Frag<E> gt[NT][4], const f32x4 rdt[NT],
                                    const f32x4 bt[NT]) {
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    Frag<E> qs[4], qp[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      f32x4 x = frag_f32(qr[it][c]);
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = rdt[it][r] != 0.f ? phi(x[r]) : 0.f;
      qp[c] = to_frag<E>(x);
      qs[c] = to_frag<E>(x * rdt[it]);
    }
    const Frag<E> bf = to_frag<E>(bt[it]);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc.S[ct][mt] = mac1<E>(acc.S[ct][mt], qs[ct], gt[it][mt]);
      acc.z[ct] = mac1<E>(acc.z[ct], qp[ct], bf);
    }
  }
}

template <class E, int kPolicy> __device__ inline void bwd_reverse_totals(const BwdParams &p) {
  const int worker = blockIdx.x;
  const int h = worker % p.heads;
  const int s = 1 + worker / p.heads;
  if (s >= p.segments) return;
  const int lane = threadIdx.x;
  const int n16 = lane & 15, g = lane >> 4;
  const long long base = (long long)h * p.N * kD;
  const E *Qh = reinterpret_cast<const E *>(p.Q) + base;
  const E *Gh = reinterpret_cast<const E *>(p.dO) + base;
  const f32x2 *stats_h = p.stats + (long long)h * p.stats_stride;
  const long long t_begin = (long long)s * p.seg_chunks * kChunk;
  long long t_end = t_begin + (long long)p.seg_chunks * kChunk;
  if (t_end > p.N) t_end = p.N;
  State acc;
  state_zero(acc);
  if constexpr (std::is_same<E, __bf16>::value) {
    constexpr int NT = 4;
    __shared__ u32x4 slot[Slot<2, NT>::kVec + 8 * NT];
    u32x4 *sreg = slot + Slot<2, NT>::kVec;
    const __bf16 *src[2] = {Qh, Gh};
    stage_issue<2, NT, kPolicy>(slot, src, t_begin, chunk_rows(t_begin, t_end), n16, g);
    stage_stats<NT>(sreg, stats_h, t_begin, chunk_rows(t_begin, t_end), lane);
    for (long long t0 = t_begin; t0 < t_end; t0 += kChunk) {
      const int rows = chunk_rows(t0, t_end);
      wait_vmcnt<0>();  // nothing is stored inside the loop
      Frag<E> qt[NT][4], gt[NT][4];
      f32x4 rdt[NT], bt[NT];
#pragma unroll
      for (int it = 0; it < NT; ++it) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          qt[it][c] = lds_tok_frag<NT>(slot, 0, it, c, lane);
          gt[it][c] = lds_tok_frag<NT>(slot, 1, it, c, lane);
        }
        stats_tok(sreg, it, g, rdt[it], bt[it]);
      }
      wait_lgkmcnt0();
      if (t0 + kChunk < t_end) {
        stage_issue<2, NT, kPolicy>(slot, src, t0 + kChunk, chunk_rows(t0 + kChunk, t_end), n16, g);
        stage_stats<NT>(sreg, stats_h, t0 + kChunk, chunk_rows(t0 + kChunk, t_end), lane);
      }
      if (rows < kChunk) {
        zero_tokens<E, NT>(gt, rows, g);
#pragma unroll
        for (int it = 0; it < NT; ++it)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * it + 4 * g + r >= rows) {
              rdt[it][r] = 0.f;
              bt[it][r] = 0.f;
            }
      }
      reverse_sums<E, NT>(acc, qt, gt, rdt, bt);
    }
  } else {
    constexpr int NT = 4;
    const Frag<E> ident = frag_identity<E>(n16, g);
    for (long long t0 = t_begin; t0 < t_end; t0 += kChunk) {
      const int rows = chunk_rows(t0, t_end);
      Frag<E> qf[NT][4], gf[NT][4], qt[NT][4], gt[NT][4];
      load_rows_f32<NT>(qf, Qh, t0, rows, n16, g);
      load_rows_f32<NT>(gf, Gh, t0, rows, n16, g);
      row_to_tok<E, NT>(qf, qt, ident);
      row_to_tok<E, NT>(gf, gt, ident);
      f32x4 rdt[NT], bt[NT];
#pragma unroll
      for (int it = 0; it < NT; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tok = 16 * it + 4 * g + r;
          const f32x2 pr = tok < rows ? stats_h[t0 + tok] : f32x2{0.f, 0.f};
          rdt[it][r] = pr[0];
          bt[it][r] = pr[1];
        }
      reverse_sums<E, NT>(acc, qt, gt, rdt, bt);
    }
  }
  state_store_record(acc, p.wsR + ((long long)h * p.recR + s) * kStateFloats, lane, n16, g);
}

template <int kPolicy>
__global__ __launch_bounds__(64, 1) void bwd_reverse_totals_kernel_bf16(BwdParams p) {
  bwd_reverse_totals<__bf16, kPolicy>(p);
}
__global__ __launch_bounds__(64, 1) void bwd_reverse_totals_kernel_f32(BwdParams p) {
  bwd_reverse_totals<float, kLoadDefault>(p);
}

// ---------------------------------------------------------------------------
// Right-to-left walk: dK and dV from the suffix state (R, r).
// ---------------------------------------------------------------------------
// Fragments: qraw Q and kraw K, row layout (rows >= rows of qraw zero); vf V
// row layout; gf dO row layout and gt dO token layout (rows >= rows zero);
// pair of token 16 it + n (sr) and of tokens 16 it + 4 g + r (rdt, bt), zero
// past the end.  a = g / den is never rounded: g (exact in the input type)
// is the operand and 1/den is applied in fp32, to D and W row by row and to
// phi(Q) before it is rounded for the state update.
template <class E, int NT, bool kFull>
__device__ inline void bwd_r_chunk(State &rs, const Frag<E> qraw[NT][4], const Frag<E> kf[NT][4],
                                   const Frag<E> kraw[NT][4], const Frag<E> vf[NT][4], const Frag<E> gf[NT][4],
                                   const Frag<E> gt[NT][4], const f32x2 sr[NT], const f32x4 rdt[NT],
                                   const f32x4 bt[NT], int rows, long long t0, E *dKh, E *dVh, int n16, int g,
                                   const Frag<E> &ident) {
  StateOperands<E> ro;
  state_operands<E>(rs, ro);  // R^T as A operand (rows = value column, k = feature)
  Frag<E> rf[4][4];
  transposed_state_operands<E>(ro, rf, ident);  // R as A operand (rows = feature, k = value column)
  Frag<E> qf[NT][4], qs[NT][4], qt[NT][4], qst[NT][4];
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    const bool valid = kFull || 16 * it + n16 < rows;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      f32x4 x = frag_f32(qraw[it][c]);
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = valid ? phi(x[r]) : 0.f;
      qf[it][c] = to_frag<E>(x);             // phi(q), row layout
      qs[it][c] = to_frag<E>(x * sr[it][0]);  // phi(q) / den, row layout
    }
  }
  row_to_tok<E, NT>(qf, qt, ident);
  row_to_tok<E, NT>(qs, qst, ident);
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) {
    f32x4 dk[4] = {zero4(), zero4(), zero4(), zero4()};
    f32x4 dv[4] = {zero4(), zero4(), zero4(), zero4()};
    auto state_terms = [&]() {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {  // R V^T
        dk[ct] = mac2<E>(dk[ct], rf[ct][0], rf[ct][1], vf[jt][0], vf[jt][1]);
        dk[ct] = mac2<E>(dk[ct], rf[ct][2], rf[ct][3], vf[jt][2], vf[jt][3]);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {  // R^T phi(K)^T
        dv[mt] = mac2<E>(dv[mt], ro.sa[0][mt], ro.sa[1][mt], kf[jt][0], kf[jt][1]);
        dv[mt] = mac2<E>(dv[mt], ro.sa[2][mt], ro.sa[3][mt], kf[jt][2], kf[jt][3]);
      }
    };
    // bf16: the state terms first, so that every accumulator chain runs its
    // 16x16x32 products before its 16x16x16 ones (device_common.hpp, mac1).
    // fp32 has one product size and keeps the order that spills least.
    constexpr bool kStateFirst = std::is_same<E, __bf16>::value;
    if constexpr (kStateFirst) state_terms();
#pragma unroll
    for (int it = jt; it < NT; ++it) {
      // Rows i = 16 it + 4 g + r, columns j = 16 jt + n, i >= j:
      // W' = phi(q_i) . phi(k_j) / den_i,  D = (g_i . v_j) / den_i + b_i.
      f32x4 w = zero4(), d = zero4();
      w = mac2<E>(w, qf[it][0], qf[it][1], kf[jt][0], kf[jt][1]);
      w = mac2<E>(w, qf[it][2], qf[it][3], kf[jt][2], kf[jt][3]);
      d = mac2<E>(d, gf[it][0], gf[it][1], vf[jt][0], vf[jt][1]);
      d = mac2<E>(d, gf[it][2], gf[it][3], vf[jt][2], vf[jt][3]);
      w = w * rdt[it];
      d = d * rdt[it] + bt[it];
      if (it == jt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * g + r < n16) {
            w[r] = 0.f;
            d[r] = 0.f;
          }
      const Frag<E> wf = to_frag<E>(w), dfr = to_frag<E>(d);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) dk[ct] = mac1<E>(dk[ct], qt[it][ct], dfr);  // phi(Q)^T D
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) dv[mt] = mac1<E>(dv[mt], gt[it][mt], wf);   // G^T W'
    }
    if constexpr (!kStateFirst) state_terms();
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const f32x4 kv = frag_f32(kraw[jt][ct]);
#pragma unroll
      for (int r = 0; r < 4; ++r) dk[ct][r] = (dk[ct][r] + rs.z[ct][r]) * phi_prime(kv[r]);
    }
    store_tiles<E, kFull>(dKh, t0 + 16 * jt, rows - 16 * jt, dk, n16, g);
    store_tiles<E, kFull>(dVh, t0 + 16 * jt, rows - 16 * jt, dv, n16, g);
  }
  // Move the suffix state past this chunk: R += (phi(Q)/den)^T G, r += phi(Q)^T b.
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    const Frag<E> bf = to_frag<E>(bt[it]);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) rs.S[ct][mt] = mac1<E>(rs.S[ct][mt], qst[it][ct], gt[it][mt]);
      rs.z[ct] = mac1<E>(rs.z[ct], qt[it][ct], bf);
    }
  }
}

template <int NT, bool kFull>
__device__ inline void bwd_r_chunk_lds(State &rs, u32x4 *slot, const __bf16 *const src[4], const f32x2 *stats_h,
                                       long long t0, long long t_next, int rows, __bf16 *dKh, __bf16 *dVh, int lane,
                                       int n16, int g, const Frag<__bf16> &ident) {
  typedef __bf16 E;
  constexpr int kT = 16 * NT;
  u32x4 *sreg = slot + Slot<4, NT>::kVec;
  Frag<E> qraw[NT][4], kf[NT][4], kraw[NT][4], vf[NT][4], gf[NT][4], gt[NT][4];
  f32x2 sr[NT];
  f32x4 rdt[NT], bt[NT];
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    lds_row_frags<NT>(slot, 0, it, lane, qraw[it]);
    lds_row_frags<NT>(slot, 1, it, lane, kraw[it]);
    lds_row_frags<NT>(slot, 2, it, lane, vf[it]);
    lds_row_frags<NT>(slot, 3, it, lane, gf[it]);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) gt[it][mt] = lds_tok_frag<NT>(slot, 3, it, mt, lane);
    sr[it] = stats_row(sreg, it, n16);
    stats_tok(sreg, it, g, rdt[it], bt[it]);
  }
  wait_lgkmcnt0();
  if (t_next >= 0) {
    stage_issue<4, NT>(slot, src, t_next, kT, n16, g);
    stage_stats<NT>(sreg, stats_h, t_next, kT, lane);
  }
#pragma unroll
  for (int it = 0; it < NT; ++it)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      kf[it][c] = kraw[it][c];
      phi_frag<E>(kf[it][c]);
    }
  if (!kFull) {
    zero_rows<E, NT>(qraw, rows, n16);
    zero_rows<E, NT>(gf, rows, n16);
    zero_tokens<E, NT>(gt, rows, g);
#pragma unroll
    for (int it = 0; it < NT; ++it) {
      if (16 * it + n16 >= rows) sr[it] = f32x2{0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (16 * it + 4 * g + r >= rows) {
          rdt[it][r] = 0.f;
          bt[it][r] = 0.f;
        }
    }
  }
  bwd_r_chunk<E, NT, kFull>(rs, qraw, kf, kraw, vf, gf, gt, sr, rdt, bt, rows, t0, dKh, dVh, n16, g, ident);
}

template <class E> __device__ inline void bwd_walk_r(const BwdParams &p) {
  const int worker = blockIdx.x;
  const int h = worker % p.heads;
  const int s = worker / p.heads;
  if (s >= p.segments) return;
  const int lane = threadIdx.x;
  const int n16 = lane & 15, g = lane >> 4;
  const long long base = (long long)h * p.N * kD;
  const E *Qh = reinterpret_cast<const E *>(p.Q) + base;
  const E *Kh = reinterpret_cast<const E *>(p.K) + base;
  const E *Vh = reinterpret_cast<const E *>(p.V) + base;
  const E *Gh = reinterpret_cast<const E *>(p.dO) + base;
  E *dKh = reinterpret_cast<E *>(p.dK) + base;
  E *dVh = reinterpret_cast<E *>(p.dV) + base;
  const f32x2 *stats_h = p.stats + (long long)h * p.stats_stride;
  const long long t_begin = (long long)s * p.seg_chunks * kChunk;
  long long t_end = t_begin + (long long)p.seg_chunks * kChunk;
  if (t_end > p.N) t_end = p.N;
  if (t_begin >= t_end) return;
  const Frag<E> ident = frag_identity<E>(n16, g);
  constexpr int NT = kBwdTiles;
  constexpr int kT = 16 * NT;
  const long long last = t_begin + ((t_end - 1 - t_begin) / kT) * kT;

  State rs;
  if (p.recR > 0 && !p.sum_in_walk) {
    state_load_record(rs, p.wsR + ((long long)h * p.recR + s) * kStateFloats, lane, g);
  } else {
    state_zero(rs);
    if (p.recR > 0)
      state_add_records(rs, p.wsR + ((long long)h * p.recR + p.segments - 1) * kStateFloats, p.segments - 1 - s,
                        -(long long)kStateFloats, lane, g);
  }
  if constexpr (std::is_same<E, __bf16>::value) {
    __shared__ u32x4 slot[Slot<4, NT>::kVec + 8 * NT];
    const __bf16 *src[4] = {Qh, Kh, Vh, Gh};
    stage_issue<4, NT>(slot, src, last, (int)(t_end - last), n16, g);
    stage_stats<NT>(slot + Slot<4, NT>::kVec, stats_h, last, (int)(t_end - last), lane);
    // The state's loads (and the first chunk's) land here, before the chunk
    // loop: left in flight, they would make the compiler wait for every
    // outstanding memory operation, earlier output stores included, at the
    // state's first use on every chunk.
    wait_vmcnt<0>();
    bool prev_full = false;
    for (long long t0 = last; t0 >= t_begin; t0 -= kT) {
      const int rows = (int)min<long long>(kT, t_end - t0);
      // Outstanding: this chunk's loads, then the previous chunk's 4 NT
      // stores.  Only a full previous chunk is known to have issued all of
      // them (the first chunk walked may be partial), so otherwise wait for
      // everything.
      if (prev_full) {
        wait_vmcnt<4 * NT>();
      } else {
        wait_vmcnt<0>();
      }
      const long long t_next = t0 - kT >= t_begin ? t0 - kT : -1;
      if (rows == kT) {
        bwd_r_chunk_lds<NT, true>(rs, slot, src, stats_h, t0, t_next, rows, dKh, dVh, lane, n16, g, ident);
      } else {
        bwd_r_chunk_lds<NT, false>(rs, slot, src, stats_h, t0, t_next, rows, dKh, dVh, lane, n16, g, ident);
      }
      prev_full = rows == kT;
    }
  } else {
    // The state's loads land here, before the chunk
    // loop: left in flight, they would make the compiler wait for every
    // outstanding memory operation, earlier output stores included, at the
    // state's first use on every chunk.
    wait_vmcnt<0>();
    for (long long t0 = last; t0 >= t_begin; t0 -= kT) {
      const int rows = (int)min<long long>(kT, t_end - t0);
      Frag<E> qraw[NT][4], kf[NT][4], kraw[NT][4], vf[NT][4], gf[NT][4], gt[NT][4];
      load_rows_f32<NT>(qraw, Qh, t0, rows, n16, g);
      load_rows_f32<NT>(kraw, Kh, t0, rows, n16, g);
      load_rows_f32<NT>(vf, Vh, t0, rows, n16, g);
      load_rows_f32<NT>(gf, Gh, t0, rows, n16, g);
#pragma unroll
      for (int it = 0; it < NT; ++it)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          kf[it][c] = kraw[it][c];
          phi_frag<E>(kf[it][c]);
        }
      row_to_tok<E, NT>(gf, gt, ident);
      f32x2 sr[NT];
      f32x4 rdt[NT], bt[NT];
#pragma unroll
      for (int it = 0; it < NT; ++it) {
        sr[it] = 16 * it + n16 < rows ? stats_h[t0 + 16 * it + n16] : f32x2{0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tok = 16 * it + 4 * g + r;
          const f32x2 pr = tok < rows ? stats_h[t0 + tok] : f32x2{0.f, 0.f};
          rdt[it][r] = pr[0];
          bt[it][r] = pr[1];
        }
      }
      bwd_r_chunk<E, NT, false>(rs, qraw, kf, kraw, vf, gf, gt, sr, rdt, bt, rows, t0, dKh, dVh, n16, g, ident);
    }
  }
}

__global__ __launch_bounds__(64, 1) void bwd_walk_r_kernel_bf16(BwdParams p) { bwd_walk_r<__bf16>(p); }
__global__ __launch_bounds__(64, 1) void bwd_walk_r_kernel_f32(BwdParams p) { bwd_walk_r<float>(p); }

// ---------------------------------------------------------------------------
// Non-causal: S, z are the head's totals (record `segments` of wsF).
// Pass A, per range of chunks: dQ = (S a^T + z b^T) * phi'(Q), the pairs, and
// the range's sums of phi(Q)^T a and phi(Q)^T b (record `range` of wsR).
// ---------------------------------------------------------------------------
template <class E, bool kFull>
__device__ inline void bwd_nc_a_tile(const StateOperands<E> &so, const Frag<E> sf[4][4], const State &st,
                                     State &acc, const Frag<E> qraw[4], const Frag<E> gf[4], int rows_left,
                                     long long row0, E *dQh, f32x2 *stats_h, int n16, int g, const Frag<E> &ident,
                                     float &keep_rd, float &keep_b, int it) {
  const bool valid = kFull || n16 < rows_left;
  // phi(q) in fp32 (zero past the end), rounded plain and scaled by 1/den.
  f32x4 pq[4];
  Frag<E> qf[4], gv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const f32x4 x = frag_f32(qraw[c]);
#pragma unroll
    for (int r = 0; r < 4; ++r) pq[c][r] = valid ? phi(x[r]) : 0.f;
    qf[c] = to_frag<E>(pq[c]);
    gv[c] = valid ? gf[c] : frag_zero<E>();
  }
  f32x4 nt[4] = {zero4(), zero4(), zero4(), zero4()};
  f32x4 dt = zero4();
  state_read<E>(so, qf, nt, dt);
  const float rd = valid ? __builtin_amdgcn_rcpf(dt[0]) : 0.f;
  float gn = 0.f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const f32x4 ga = frag_f32(gv[mt]);
#pragma unroll
    for (int r = 0; r < 4; ++r) gn += ga[r] * nt[mt][r];
  }
  gn += __shfl_xor(gn, 16);
  gn += __shfl_xor(gn, 32);
  const float b = -gn * rd * rd;
  // dphi(Q)^T = (S g^T) / den + z b^T; g is the operand, 1/den is applied in fp32.
  f32x4 dq[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    dq[ct] = mac2<E>(zero4(), sf[ct][0], sf[ct][1], gv[0], gv[1]);
    dq[ct] = mac2<E>(dq[ct], sf[ct][2], sf[ct][3], gv[2], gv[3]);
    const f32x4 qv = frag_f32(qraw[ct]);
#pragma unroll
    for (int r = 0; r < 4; ++r) dq[ct][r] = (dq[ct][r] * rd + st.z[ct][r] * b) * phi_prime(qv[r]);
  }
  store_tiles<E, kFull>(dQh, row0, rows_left, dq, n16, g);
  if (g == it) {
    keep_rd = rd;
    keep_b = b;
  }
  // The range's sums (phi(Q)/den)^T G and phi(Q)^T b contract over tokens;
  // the fragments above have the token as the row index, so they are
  // transposed by identity products (exact).
  Frag<E> qt[4], qst[4], gt[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    qt[c] = to_frag<E>(transpose_tile<E>(qf[c], ident));
    qst[c] = to_frag<E>(transpose_tile<E>(to_frag<E>(pq[c] * rd), ident));
    gt[c] = to_frag<E>(transpose_tile<E>(gv[c], ident));
  }
  const Frag<E> bk = to_frag<E>(transpose_tile<E>(to_frag<E>(f32x4{b, b, b, b}), ident));
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc.S[ct][mt] = mac1<E>(acc.S[ct][mt], qst[ct], gt[mt]);
    acc.z[ct] = mac1<E>(acc.z[ct], qt[ct], bk);
  }
}

template <class E> __device__ inline void bwd_nc_a(const BwdParams &p) {
  const int worker = blockIdx.x;
  const int h = worker % p.heads;
  const int s = worker / p.heads;
  if (s >= p.ranges) return;
  const int lane = threadIdx.x;
  const int n16 = lane & 15, g = lane >> 4;
  const long long base = (long long)h * p.N * kD;
  const E *Qh = reinterpret_cast<const E *>(p.Q) + base;
  const E *Gh = reinterpret_cast<const E *>(p.dO) + base;
  E *dQh = reinterpret_cast<E *>(p.dQ) + base;
  f32x2 *stats_h = p.stats + (long long)h * p.stats_stride;
  const long long t_begin = (long long)s * p.range_chunks * kChunk;
  long long t_end = t_begin + (long long)p.range_chunks * kChunk;
  if (t_end > p.N) t_end = p.N;
  const Frag<E> ident = frag_identity<E>(n16, g);

  State st;
  state_load_record(st, p.wsF + ((long long)h * p.recF + p.segments) * kStateFloats, lane, g);
  StateOperands<E> so;
  state_operands<E>(st, so);
  Frag<E> sf[4][4];
  transposed_state_operands<E>(so, sf, ident);
  State acc;
  state_zero(acc);
  if constexpr (std::is_same<E, __bf16>::value) {
    constexpr int NT = 4;
    __shared__ u32x4 slot[Slot<2, NT>::kVec];
    const __bf16 *src[2] = {Qh, Gh};
    if (t_begin < t_end) stage_issue<2, NT>(slot, src, t_begin, chunk_rows(t_begin, t_end), n16, g);
    for (long long t0 = t_begin; t0 < t_end; t0 += kChunk) {
      const int rows = chunk_rows(t0, t_end);
      // Outstanding: this chunk's loads, then the previous (full) chunk's
      // 2 NT dQ stores and one pair store.
      if (t0 == t_begin) {
        wait_vmcnt<0>();
      } else {
        wait_vmcnt<2 * NT + 1>();
      }
      Frag<E> qraw[NT][4], gf[NT][4];
#pragma unroll
      for (int it = 0; it < NT; ++it) {
        lds_row_frags<NT>(slot, 0, it, lane, qraw[it]);
        lds_row_frags<NT>(slot, 1, it, lane, gf[it]);
      }
      wait_lgkmcnt0();
      if (t0 + kChunk < t_end) stage_issue<2, NT>(slot, src, t0 + kChunk, chunk_rows(t0 + kChunk, t_end), n16, g);
      float keep_rd = 0.f, keep_b = 0.f;
      if (rows == kChunk) {
#pragma unroll
        for (int it = 0; it < NT; ++it)
          bwd_nc_a_tile<E, true>(so, sf, st, acc, qraw[it], gf[it], rows - 16 * it, t0 + 16 * it, dQh, stats_h, n16,
                                 g, ident, keep_rd, keep_b, it);
      } else {
#pragma unroll
        for (int it = 0; it < NT; ++it)
          bwd_nc_a_tile<E, false>(so, sf, st, acc, qraw[it], gf[it], rows - 16 * it, t0 + 16 * it, dQh, stats_h,
                                  n16, g, ident, keep_rd, keep_b, it);
      }
      if (16 * g + n16 < rows) stats_h[t0 + 16 * g + n16] = f32x2{keep_rd, keep_b};
    }
  } else {
    constexpr int NT = 4;
    for (long long t0 = t_begin; t0 < t_end; t0 += kChunk) {
      const int rows = chunk_rows(t0, t_end);
      Frag<E> qraw[NT][4], gf[NT][4];
      load_rows_f32<NT>(qraw, Qh, t0, rows, n16, g);
      load_rows_f32<NT>(gf, Gh, t0, rows, n16, g);
      float keep_rd = 0.f, keep_b = 0.f;
#pragma unroll
      for (int it = 0; it < NT; ++it)
        bwd_nc_a_tile<E, false>(so, sf, st, acc, qraw[it], gf[it], rows - 16 * it, t0 + 16 * it, dQh, stats_h, n16,
                                g, ident, keep_rd, keep_b, it);
      if (16 * g + n16 < rows) stats_h[t0 + 16 * g + n16] = f32x2{keep_rd, keep_b};
    }
  }
  state_store_record(acc, p.wsR + ((long long)h * p.recR + s) * kStateFloats, lane, n16, g);
}

__global__ __launch_bounds__(64, 1) void bwd_nc_a_kernel_bf16(BwdParams p) { bwd_nc_a<__bf16>(p); }
__global__ __launch_bounds__(64, 1) void bwd_nc_a_kernel_f32(BwdParams p) { bwd_nc_a<float>(p); }

// Pass B, per range: dK = (R V^T + r 1^T) * phi'(K), dV = R^T phi(K)^T with the
// head's totals R, r (record `ranges` of wsR).
template <class E, bool kFull>
__device__ inline void bwd_nc_b_tile(const StateOperands<E> &ro, const Frag<E> rf[4][4], const State &rs,
                                     const Frag<E> kraw[4], const Frag<E> vf[4], int rows_left, long long row0,
                                     E *dKh, E *dVh, int n16, int g) {
  Frag<E> kf[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    kf[c] = kraw[c];
    phi_frag<E>(kf[c]);
  }
  f32x4 dk[4], dv[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    dk[ct] = mac2<E>(zero4(), rf[ct][0], rf[ct][1], vf[0], vf[1]);
    dk[ct] = mac2<E>(dk[ct], rf[ct][2], rf[ct][3], vf[2], vf[3]);
    const f32x4 kv = frag_f32(kraw[ct]);
#pragma unroll
    for (int r = 0; r < 4; ++r) dk[ct][r] = (dk[ct][r] + rs.z[ct][r]) * phi_prime(kv[r]);
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    dv[mt] = mac2<E>(zero4(), ro.sa[0][mt], ro.sa[1][mt], kf[0], kf[1]);
    dv[mt] = mac2<E>(dv[mt], ro.sa[2][mt], ro.sa[3][mt], kf[2], kf[3]);
  }
  store_tiles<E, kFull>(dKh, row0, rows_left, dk, n16, g);
  store_tiles<E, kFull>(dVh, row0, rows_left, dv, n16, g);
}

template <class E> __device__ inline void bwd_nc_b(const BwdParams &p) {
  const int worker = blockIdx.x;
  const int h = worker % p.heads;
  const int s = worker / p.heads;
  if (s >= p.ranges) return;
  const int lane = threadIdx.x;
  const int n16 = lane & 15, g = lane >> 4;
  const long long base = (long long)h * p.N * kD;
  const E *Kh = reinterpret_cast<const E *>(p.K) + base;
  const E *Vh = reinterpret_cast<const E *>(p.V) + base;
  E *dKh = reinterpret_cast<E *>(p.dK) + base;
  E *dVh = reinterpret_cast<E *>(p.dV) + base;
  const long long t_begin = (long long)s * p.range_chunks * kChunk;
  long long t_end = t_begin + (long long)p.range_chunks * kChunk;
  if (t_end > p.N) t_end = p.N;
  const Frag<E> ident = frag_identity<E>(n16, g);

  State rs;
  state_load_record(rs, p.wsR + ((long long)h * p.recR + p.ranges) * kStateFloats, lane, g);
  StateOperands<E> ro;
  state_operands<E>(rs, ro);
  Frag<E> rf[4][4];
  transposed_state_operands<E>(ro, rf, ident);
  if constexpr (std::is_same<E, __bf16>::value) {
    constexpr int NT = 4;
    __shared__ u32x4 slot[Slot<2, NT>::kVec];
    const __bf16 *src[2] = {Kh, Vh};
    if (t_begin < t_end) stage_issue<2, NT>(slot, src, t_begin, chunk_rows(t_begin, t_end), n16, g);
    for (long long t0 = t_begin; t0 < t_end; t0 += kChunk) {
      const int rows = chunk_rows(t0, t_end);
      // Outstanding: this chunk's loads, then the previous (full) chunk's
      // 4 NT stores.
      if (t0 == t_begin) {
        wait_vmcnt<0>();
      } else {
        wait_vmcnt<4 * NT>();
      }
      Frag<E> kraw[NT][4], vf[NT][4];
#pragma unroll
      for (int it = 0; it < NT; ++it) {
        lds_row_frags<NT>(slot, 0, it, lane, kraw[it]);
        lds_row_frags<NT>(slot, 1, it, lane, vf[it]);
      }
      wait_lgkmcnt0();
      if (t0 + kChunk < t_end) stage_issue<2, NT>(slot, src, t0 + kChunk, chunk_rows(t0 + kChunk, t_end), n16, g);
      if (rows == kChunk) {
#pragma unroll
        for (int it = 0; it < NT; ++it)
          bwd_nc_b_tile<E, true>(ro, rf, rs, kraw[it], vf[it], rows - 16 * it, t0 + 16 * it, dKh, dVh, n16, g);
      } else {
#pragma unroll
        for (int it = 0; it < NT; ++it)
          bwd_nc_b_tile<E, false>(ro, rf, rs, kraw[it], vf[it], rows - 16 * it, t0 + 16 * it, dKh, dVh, n16, g);
      }
    }
  } else {
    constexpr int NT = 4;
    for (long long t0 = t_begin; t0 < t_end; t0 += kChunk) {
      const int rows = chunk_rows(t0, t_end);
      Frag<E> kraw[NT][4], vf[NT][4];
      load_rows_f32<NT>(kraw, Kh, t0, rows, n16, g);
      load_rows_f32<NT>(vf, Vh, t0, rows, n16, g);
#pragma unroll
      for (int it = 0; it < NT; ++it)
        bwd_nc_b_tile<E, false>(ro, rf, rs, kraw[it], vf[it], rows - 16 * it, t0 + 16 * it, dKh, dVh, n16, g);
    }
  }
}

__global__ __launch_bounds__(64, 1) void bwd_nc_b_kernel_bf16(BwdParams p) { bwd_nc_b<__bf16>(p); }
__global__ __launch_bounds__(64, 1) void bwd_nc_b_kernel_f32(BwdParams p) { bwd_nc_b<float>(p); }

template <class E> struct BwdKernels;
template <> struct BwdKernels<__bf16> {
  static constexpr auto walk_f = bwd_walk_f_kernel_bf16;
  static constexpr auto reverse_totals = bwd_reverse_totals_kernel_bf16<kLoadDefault>;
  static constexpr auto reverse_totals_streaming = bwd_reverse_totals_kernel_bf16<kLoadStreaming>;
  static constexpr auto walk_r = bwd_walk_r_kernel_bf16;
  static constexpr auto nc_a = bwd_nc_a_kernel_bf16;
  static constexpr auto nc_b = bwd_nc_b_kernel_bf16;
};
template <> struct BwdKernels<float> {
  static constexpr auto walk_f = bwd_walk_f_kernel_f32;
  static constexpr auto reverse_totals = bwd_reverse_totals_kernel_f32;
  static constexpr auto reverse_totals_streaming = bwd_reverse_totals_kernel_f32;
  static constexpr auto walk_r = bwd_walk_r_kernel_f32;
  static constexpr auto nc_a = bwd_nc_a_kernel_f32;
  static constexpr auto nc_b = bwd_nc_b_kernel_f32;
};

}  // namespace linattn
