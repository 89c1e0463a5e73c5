// forward_kernels.hpp -- chunked parallel forward of elu(x)+1 linear attention
// for gfx950.
//
// Math ("Why Replace Attention?", §6.2 and §7.1-§7.2): with phi = elu + 1,
//   causal:     o_i = phi(q_i)^T S_i / phi(q_i)^T z_i,  S_i = sum_{j<=i} phi(k_j) v_j^T,
//               z_i = sum_{j<=i} phi(k_j);
//   non-causal: the same with S, z summed over every token.
// Splitting the causal sums at chunk boundaries (64 tokens) gives, for the
// rows i of chunk c with the state S_prev, z_prev of all earlier tokens,
//   num_i = phi(q_i)^T S_prev + sum_{j in c, j<=i} (phi(q_i)^T phi(k_j)) v_j
//   den_i = phi(q_i)^T z_prev + sum_{j in c, j<=i}  phi(q_i)^T phi(k_j)
//   S_prev += phi(K_c)^T V_c,  z_prev += column sums of phi(K_c),
// which is the recurrence of §7.2 regrouped, so it reaches the same result up
// to rounding.  The chunk products are dense 64x64x64 contractions and run on
// MFMA; the state stays in fp32 MFMA accumulators for a whole segment.
//
// Parallel structure.  One wave64 is one worker and owns a (head, segment)
// pair: a run of whole chunks it walks left to right.  Sequence segments make
// the grid wide enough for few-head workloads; their starting states come
// from a two-pass scan (segment totals, then an exclusive prefix per head),
// the parallel-scan resolution of the left-to-right dependency ("Why Replace
// Attention?", §7.7).  No LDS and no inter-wave synchronisation: every wave
// is independent, data is exchanged only through the scan's workspace.
#pragma once

#include "device_common.hpp"

namespace linattn {

// One state record (S and z of one head at one segment boundary), fp32, in
// the registers' own order so a wave reads or writes it with 16-byte
// vectors:  S: [ct 4][mt 4][lane 64][r 4] = 4096 floats, where lane (n, g)
// register r of tile (ct, mt) is S[pi(ct,g,r)][pi(mt,n>>2,n&3)];
// z: [ct 4][g 4][r 4] = 64 floats, z[pi(ct,g,r)].
constexpr int kStateFloats = 4096 + 64;

enum InitMode : int { kInitZero = 0, kInitRecord = 1, kInitNatural = 2 };

struct FwdParams {
  const void *Q, *K, *V;
  void *O;
  long long N;         // tokens per head
  int heads;           // B * H
  int segments;        // segments per head (P)
  int seg_chunks;      // chunks per segment (the last one may be shorter)
  float *ws;           // [heads][records][kStateFloats]
  int records;         // records per head in ws
  int init;            // InitMode for the walk kernel
  const float *S0;     // natural order [heads][64][64] (kInitNatural / scan seed)
  const float *z0;     // [heads][64]
  float *S_out;        // natural order final state, written by the last segment
  float *z_out;
};

// ---------------------------------------------------------------------------
// Per-wave state: S (16 tiles) and z (4 tiles, every column equal).
// ---------------------------------------------------------------------------
struct State {
  f32x4 S[4][4];  // [ct][mt]
  f32x4 z[4];     // [ct]
};

__device__ inline void state_zero(State &st) {
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    st.z[a] = zero4();
#pragma unroll
    for (int b = 0; b < 4; ++b) st.S[a][b] = zero4();
  }
}

__device__ inline void state_load_record(State &st, const float *rec, int lane, int g) {
  const f32x4 *p = reinterpret_cast<const f32x4 *>(rec);
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) st.S[ct][mt] = p[(ct * 4 + mt) * 64 + lane];
    st.z[ct] = p[1024 + ct * 4 + g];
  }
}

__device__ inline void state_store_record(const State &st, float *rec, int lane, int n16, int g) {
  f32x4 *p = reinterpret_cast<f32x4 *>(rec);
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) p[(ct * 4 + mt) * 64 + lane] = st.S[ct][mt];
    if (n16 == 0) p[1024 + ct * 4 + g] = st.z[ct];
  }
}

__device__ inline void state_load_natural(State &st, const float *S, const float *z, int n16, int g) {
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = pi_col(ct, g, r);
      st.z[ct][r] = z[c];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) st.S[ct][mt][r] = S[c * 64 + pi_col(mt, n16 >> 2, n16 & 3)];
    }
  }
}

__device__ inline void state_store_natural(const State &st, float *S, float *z, int n16, int g) {
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = pi_col(ct, g, r);
      if (n16 == 0) z[c] = st.z[ct][r];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) S[c * 64 + pi_col(mt, n16 >> 2, n16 & 3)] = st.S[ct][mt][r];
    }
  }
}

// ---------------------------------------------------------------------------
// Raw chunk data of one wave: 4 slabs of 16 rows for each tensor.
// ---------------------------------------------------------------------------
template <class E> struct Chunk {
  Slab<E> q[4], k[4], v[4];
};

template <class E, bool kQ, bool kKV>
__device__ inline void chunk_load(Chunk<E> &d, const E *Qh, const E *Kh, const E *Vh, long long t0, int rows,
                                  int n16, int g) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = 16 * it + n16;
    if (row < rows) {
      const long long off = (t0 + row) * kD;
      if (kQ) slab_load<E>(d.q[it], Qh + off, g);
      if (kKV) {
        slab_load<E>(d.k[it], Kh + off, g);
        slab_load<E>(d.v[it], Vh + off, g);
      }
    } else {
      if (kQ) slab_zero<E>(d.q[it]);
      if (kKV) {
        slab_zero<E>(d.k[it]);
        slab_zero<E>(d.v[it]);
      }
    }
  }
}

// phi(K) fragments (zero for rows past the end, where phi(0) = 1 would
// otherwise leak into the sums) and V re-oriented for token contraction:
// vb[jt][mt] is the B operand with k = token 4g+r of tile jt and column n
// standing for value column pi(mt, n>>2, n&3).
template <class E>
__device__ inline void kv_frags(const Chunk<E> &d, int rows, int n16, const Frag<E> &ident, Frag<E> kf[4][4],
                                Frag<E> vb[4][4]) {
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    slab_to_frags<E>(d.k[jt], kf[jt], true);
    if (16 * jt + n16 >= rows) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) kf[jt][kt] = frag_zero<E>();
    }
    Frag<E> vr[4];
    slab_to_frags<E>(d.v[jt], vr, false);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) vb[jt][mt] = to_frag<E>(transpose_tile<E>(vr[mt], ident));
  }
}

// S += phi(K_c)^T V_c and z += column sums of phi(K_c) ("Why Replace
// Attention?", §7.2, applied to a chunk of tokens at once).
template <class E>
__device__ inline void state_update(State &st, const Frag<E> kf[4][4], const Frag<E> vb[4][4], const Frag<E> &ident) {
  Frag<E> kt_f[4][4];  // [jt][ct]: A operand, row n = feature pi(ct, n>>2, n&3), k = token of tile jt
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) kt_f[jt][ct] = to_frag<E>(transpose_tile<E>(kf[jt][ct], ident));
  const Frag<E> ones = frag_ones<E>();
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) st.S[ct][mt] = mma_k<E>(st.S[ct][mt], &kt_f[0][ct], 4, &vb[0][mt], 4, 4);
    st.z[ct] = mma_k<E>(st.z[ct], &kt_f[0][ct], 4, &ones, 0, 4);
  }
}

// Normalise a 16x64 block of outputs and write it: o = num / den, rounded to
// the output type, turned row-per-lane by an identity product and stored as
// two 16-byte vectors per lane.
template <class E>
__device__ inline void store_block(E *Oh, long long row0, int rows_left, const f32x4 num[4], f32x4 den, int n16,
                                   int g, const Frag<E> &ident) {
  f32x4 ot[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    f32x4 o;
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = num[mt][r] / den[r];
    ot[mt] = transpose_tile<E>(to_frag<E>(o), ident);
  }
  if (n16 < rows_left) {
    E *row = Oh + (row0 + n16) * kD;
    store_row8<E>(row, g, 0, ot[0], ot[1]);
    store_row8<E>(row, g, 1, ot[2], ot[3]);
  }
}

// ---------------------------------------------------------------------------
// Pass 1: per-segment totals of phi(K)^T V and phi(K).
// ---------------------------------------------------------------------------
template <class E>
__global__ __launch_bounds__(64, 1) void seg_totals_kernel(FwdParams p, int total_segments) {
  const int worker = blockIdx.x;
  const int h = worker % p.heads;
  const int s = worker / p.heads;
  if (s >= total_segments) return;
  const int lane = threadIdx.x;
  const int n16 = lane & 15, g = lane >> 4;
  const long long base = (long long)h * p.N * kD;
  const E *Kh = reinterpret_cast<const E *>(p.K) + base;
  const E *Vh = reinterpret_cast<const E *>(p.V) + base;
  const long long t_begin = (long long)s * p.seg_chunks * kChunk;
  long long t_end = t_begin + (long long)p.seg_chunks * kChunk;
  if (t_end > p.N) t_end = p.N;
  const Frag<E> ident = frag_identity<E>(n16, g);

  State st;
  state_zero(st);
  Chunk<E> cur, nxt;
  chunk_load<E, false, true>(cur, nullptr, Kh, Vh, t_begin, (int)min<long long>(kChunk, t_end - t_begin), n16, g);
  for (long long t0 = t_begin; t0 < t_end; t0 += kChunk) {
    const int rows = (int)min<long long>(kChunk, t_end - t0);
    const long long t1 = t0 + kChunk;
    if (t1 < t_end) chunk_load<E, false, true>(nxt, nullptr, Kh, Vh, t1, (int)min<long long>(kChunk, t_end - t1), n16, g);
    Frag<E> kf[4][4], vb[4][4];
    kv_frags<E>(cur, rows, n16, ident, kf, vb);
    state_update<E>(st, kf, vb, ident);
    cur = nxt;
  }
  float *rec = p.ws + ((long long)h * p.records + s) * kStateFloats;
  state_store_record(st, rec, lane, n16, g);
}

// ---------------------------------------------------------------------------
// Scan over segment records, one thread per (head, state element).
//   causal:     records 0..P-2 hold totals -> become exclusive prefixes seeded
//               with S0/z0 (or zero); record P-1 receives the prefix of the
//               last segment.
//   non-causal: record P receives the sum of records 0..P-1.
// The order of additions is fixed, so results are deterministic.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void scan_kernel(FwdParams p, int causal) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int h = (int)(idx / kStateFloats);
  const int e = (int)(idx % kStateFloats);
  if (h >= p.heads) return;
  float *recs = p.ws + (long long)h * p.records * kStateFloats + e;
  const int P = p.segments;
  if (causal) {
    float run = 0.f;
    if (p.S0 != nullptr) {
      if (e < 4096) {
        const int ct = e >> 10, mt = (e >> 8) & 3, lane = (e >> 2) & 63, r = e & 3;
        const int c = pi_col(ct, lane >> 4, r);
        const int m = pi_col(mt, (lane & 15) >> 2, lane & 3);
        run = p.S0[(long long)h * 4096 + c * 64 + m];
      } else {
        const int f = e - 4096;
        const int ct = f >> 4, g = (f >> 2) & 3, r = f & 3;
        run = p.z0[(long long)h * 64 + pi_col(ct, g, r)];
      }
    }
    for (int s = 0; s + 1 < P; ++s) {
      const float t = recs[(long long)s * kStateFloats];
      recs[(long long)s * kStateFloats] = run;
      run += t;
    }
    recs[(long long)(P - 1) * kStateFloats] = run;
  } else {
    float run = 0.f;
    for (int s = 0; s < P; ++s) run += recs[(long long)s * kStateFloats];
    recs[(long long)P * kStateFloats] = run;
  }
}

// ---------------------------------------------------------------------------
// Causal walk: outputs of one segment, starting from its prefix state.
// ---------------------------------------------------------------------------
template <class E>
__device__ inline void causal_chunk(State &st, const Chunk<E> &d, int rows, E *Oh, long long t0, int n16, int g,
                                    const Frag<E> &ident) {
  Frag<E> qf[4][4], kf[4][4], vb[4][4];
#pragma unroll
  for (int it = 0; it < 4; ++it) slab_to_frags<E>(d.q[it], qf[it], true);
  kv_frags<E>(d, rows, n16, ident, kf, vb);

  // The state before this chunk, as B operands for phi(Q) S and phi(Q) z.
  Frag<E> sb[4][4], zb[4];  // [kt][mt], [kt]
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) sb[kt][mt] = to_frag<E>(st.S[kt][mt]);
    zb[kt] = to_frag<E>(st.z[kt]);
  }
  const Frag<E> ones = frag_ones<E>();

#pragma unroll
  for (int it = 0; it < 4; ++it) {
    if (16 * it >= rows) break;
    f32x4 num[4], den = zero4();
    // Inter-chunk read: phi(Q) S_prev and phi(Q) z_prev.
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) num[mt] = mma_k<E>(zero4(), qf[it], 1, &sb[0][mt], 4, 4);
    den = mma_k<E>(den, qf[it], 1, zb, 1, 4);
    // Intra-chunk: A = tril(phi(Q) phi(K)^T) for key tiles jt <= it.  The
    // product phi(K) phi(Q)^T leaves lane (n, g) with A[i = n][j = 4g+r],
    // which is already the A operand of A V (k = key token).
    Frag<E> af[4];
#pragma unroll
    for (int jt = 0; jt <= it; ++jt) {
      f32x4 at = mma_k<E>(zero4(), kf[jt], 1, qf[it], 1, 4);
      if (jt == it) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * g + r > n16) at[r] = 0.f;  // inclusive mask j <= i ("Why Replace Attention?", §7.1)
      }
      af[jt] = to_frag<E>(at);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) num[mt] = mma_k<E>(num[mt], af, 1, &vb[0][mt], 4, it + 1);
    den = mma_k<E>(den, af, 1, &ones, 0, it + 1);
    store_block<E>(Oh, t0 + 16 * it, rows - 16 * it, num, den, n16, g, ident);
  }
  state_update<E>(st, kf, vb, ident);
}

template <class E>
__global__ __launch_bounds__(64, 1) void causal_walk_kernel(FwdParams p) {
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
  E *Oh = reinterpret_cast<E *>(p.O) + base;
  const long long t_begin = (long long)s * p.seg_chunks * kChunk;
  long long t_end = t_begin + (long long)p.seg_chunks * kChunk;
  if (t_end > p.N) t_end = p.N;
  const Frag<E> ident = frag_identity<E>(n16, g);

  State st;
  if (p.init == kInitRecord) {
    state_load_record(st, p.ws + ((long long)h * p.records + s) * kStateFloats, lane, g);
  } else if (p.init == kInitNatural) {
    state_load_natural(st, p.S0 + (long long)h * 4096, p.z0 + (long long)h * 64, n16, g);
  } else {
    state_zero(st);
  }

  Chunk<E> cur, nxt;
  if (t_begin < t_end)
    chunk_load<E, true, true>(cur, Qh, Kh, Vh, t_begin, (int)min<long long>(kChunk, t_end - t_begin), n16, g);
  for (long long t0 = t_begin; t0 < t_end; t0 += kChunk) {
    const int rows = (int)min<long long>(kChunk, t_end - t0);
    const long long t1 = t0 + kChunk;
    if (t1 < t_end) chunk_load<E, true, true>(nxt, Qh, Kh, Vh, t1, (int)min<long long>(kChunk, t_end - t1), n16, g);
    causal_chunk<E>(st, cur, rows, Oh, t0, n16, g, ident);
    cur = nxt;
  }
  if (p.S_out != nullptr && s == p.segments - 1)
    state_store_natural(st, p.S_out + (long long)h * 4096, p.z_out + (long long)h * 64, n16, g);
}

// ---------------------------------------------------------------------------
// Non-causal pass 2: o_i = phi(q_i)^T S / phi(q_i)^T z with the head's total
// S, z (record `segments` of the workspace) -- "Why Replace Attention?",
// §6.2 -- for one range of chunks per wave.
// ---------------------------------------------------------------------------
template <class E>
__global__ __launch_bounds__(64, 1) void noncausal_read_kernel(FwdParams p, int ranges, int range_chunks) {
  const int worker = blockIdx.x;
  const int h = worker % p.heads;
  const int s = worker / p.heads;
  if (s >= ranges) return;
  const int lane = threadIdx.x;
  const int n16 = lane & 15, g = lane >> 4;
  const long long base = (long long)h * p.N * kD;
  const E *Qh = reinterpret_cast<const E *>(p.Q) + base;
  E *Oh = reinterpret_cast<E *>(p.O) + base;
  const long long t_begin = (long long)s * range_chunks * kChunk;
  long long t_end = t_begin + (long long)range_chunks * kChunk;
  if (t_end > p.N) t_end = p.N;
  const Frag<E> ident = frag_identity<E>(n16, g);

  State st;
  state_load_record(st, p.ws + ((long long)h * p.records + p.segments) * kStateFloats, lane, g);
  Frag<E> sb[4][4], zb[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) sb[kt][mt] = to_frag<E>(st.S[kt][mt]);
    zb[kt] = to_frag<E>(st.z[kt]);
  }

  Chunk<E> cur, nxt;
  if (t_begin < t_end)
    chunk_load<E, true, false>(cur, Qh, nullptr, nullptr, t_begin, (int)min<long long>(kChunk, t_end - t_begin), n16, g);
  for (long long t0 = t_begin; t0 < t_end; t0 += kChunk) {
    const int rows = (int)min<long long>(kChunk, t_end - t0);
    const long long t1 = t0 + kChunk;
    if (t1 < t_end)
      chunk_load<E, true, false>(nxt, Qh, nullptr, nullptr, t1, (int)min<long long>(kChunk, t_end - t1), n16, g);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      if (16 * it >= rows) break;
      Frag<E> qf[4];
      slab_to_frags<E>(cur.q[it], qf, true);
      f32x4 num[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) num[mt] = mma_k<E>(zero4(), qf, 1, &sb[0][mt], 4, 4);
      const f32x4 den = mma_k<E>(zero4(), qf, 1, zb, 1, 4);
      store_block<E>(Oh, t0 + 16 * it, rows - 16 * it, num, den, n16, g, ident);
    }
    cur = nxt;
  }
}

}  // namespace linattn
