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

#include <type_traits>

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

// Walks the chunks [t_begin, t_end) of one head, calling body(chunk, t0, rows)
// for each.
__device__ inline int chunk_rows(long long t0, long long t_end) {
  return (int)(t_end - t0 < kChunk ? t_end - t0 : kChunk);
}

template <class E, bool kQ, bool kKV, class Body>
__device__ inline void stream_chunks(const E *Qh, const E *Kh, const E *Vh, long long t_begin, long long t_end,
                                     int n16, int g, Body &&body) {
  // Register path (fp32 storage): load a chunk, then compute it.  Latency is
  // hidden by the other waves of the compute unit rather than by prefetch,
  // which would need a second 192-register buffer.
  for (long long t0 = t_begin; t0 < t_end; t0 += kChunk) {
    Chunk<E> d;
    chunk_load<E, kQ, kKV>(d, Qh, Kh, Vh, t0, chunk_rows(t0, t_end), n16, g);
    body(d, t0, chunk_rows(t0, t_end));
  }
}

// ---------------------------------------------------------------------------
// bf16 chunk streaming through LDS.  The next chunk is fetched with
// global_load_lds_dwordx4 (HBM -> LDS without passing through VGPRs) into a
// wave-private staging slot while the current chunk is computed; at the top
// of each chunk the wave reads its slot back into registers.  Lane l's 16
// bytes of instruction i land at slot + 1024 * i + 16 * l, so every read is a
// conflict-free ds_read_b128 of the lane's own bytes.  No other wave touches
// the slot, so no barrier is needed -- only the wave's own wait counters.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

// Slot layout: [tensor][it 4][x 2][lane 64] x 16 B; tensors in the order
// they are loaded (Q first when present).
template <bool kQ, bool kKV> struct StageShape {
  static constexpr int kTensors = (kQ ? 1 : 0) + (kKV ? 2 : 0);
  static constexpr int kVec = kTensors * 8 * 64;  // 16-byte vectors per slot
  static constexpr int kLoadsPerChunk = kTensors * 8;
};

// s_waitcnt with only vmcnt set (expcnt, lgkmcnt left at "no wait").
template <int N> __device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <bool kQ, bool kKV>
__device__ inline void stage_issue(u32x4 *slot, const __bf16 *Qh, const __bf16 *Kh, const __bf16 *Vh, long long t0,
                                   int rows, int n16, int g) {
  const __bf16 *src[3] = {kQ ? Qh : Kh, kQ ? Kh : Vh, Vh};
#pragma unroll
  for (int tsr = 0; tsr < StageShape<kQ, kKV>::kTensors; ++tsr) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int row = 16 * it + n16;
      if (row < rows) {
        const u32x4 *gp = reinterpret_cast<const u32x4 *>(src[tsr] + (t0 + row) * kD);
#pragma unroll
        for (int x = 0; x < 2; ++x)
          __builtin_amdgcn_global_load_lds(gp + 4 * x + g, (lds_void *)(slot + ((tsr * 4 + it) * 2 + x) * 64), 16,
                                           0, 0);
      }
    }
  }
}

// Reads the slot back.  Rows past the end of the sequence (only in a
// partial last chunk) hold stale bytes: K and V rows are zeroed there, Q rows
// are left as they are because their outputs are never stored.
template <bool kQ, bool kKV>
__device__ inline void stage_read(const u32x4 *slot, Chunk<__bf16> &d, int rows, int lane, int n16) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    Slab<__bf16> *dst[3] = {kQ ? &d.q[it] : &d.k[it], kQ ? &d.k[it] : &d.v[it], &d.v[it]};
#pragma unroll
    for (int tsr = 0; tsr < StageShape<kQ, kKV>::kTensors; ++tsr)
#pragma unroll
      for (int x = 0; x < 2; ++x) dst[tsr]->h[x] = slot[((tsr * 4 + it) * 2 + x) * 64 + lane];
  }
  if (kKV && rows < kChunk) {  // uniform branch
#pragma unroll
    for (int it = 0; it < 4; ++it)
      if (16 * it + n16 >= rows) {
        slab_zero<__bf16>(d.k[it]);
        slab_zero<__bf16>(d.v[it]);
      }
  }
}

// kStores: vector-memory stores body() issues per full chunk (the outputs).
template <bool kQ, bool kKV, int kStores, class Body>
__device__ inline void stream_chunks_lds(u32x4 *slot, const __bf16 *Qh, const __bf16 *Kh, const __bf16 *Vh,
                                         long long t_begin, long long t_end, int lane, int n16, int g, Body &&body) {
  if (t_begin >= t_end) return;
  stage_issue<kQ, kKV>(slot, Qh, Kh, Vh, t_begin, chunk_rows(t_begin, t_end), n16, g);
  for (long long t0 = t_begin; t0 < t_end; t0 += kChunk) {
    const int rows = chunk_rows(t0, t_end);
    // Outstanding vector-memory operations: this chunk's loads, then the
    // previous chunk's kStores output stores (every chunk but the last is
    // full, so it issued all of them).  They retire in order, so waiting
    // down to kStores leaves only stores in flight.  The first chunk has no
    // stores behind its loads.
    if (t0 == t_begin) {
      wait_vmcnt<0>();
    } else {
      wait_vmcnt<kStores>();
    }
    Chunk<__bf16> d;
    stage_read<kQ, kKV>(slot, d, rows, lane, n16);
    // The slot is refilled only after every lane's read of it returned.
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
    const long long t1 = t0 + kChunk;
    if (t1 < t_end) stage_issue<kQ, kKV>(slot, Qh, Kh, Vh, t1, chunk_rows(t1, t_end), n16, g);
    body(d, t0, rows);
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
  for (int jp = 0; jp < 2; ++jp) {  // pairs of key tiles
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        st.S[ct][mt] = mac2<E>(st.S[ct][mt], kt_f[2 * jp][ct], kt_f[2 * jp + 1][ct], vb[2 * jp][mt], vb[2 * jp + 1][mt]);
      st.z[ct] = mac2<E>(st.z[ct], kt_f[2 * jp][ct], kt_f[2 * jp + 1][ct], ones, ones);
    }
  }
}

// Normalise a 16x64 block of outputs and write it: o = num / den, rounded to
// the output type, turned row-per-lane by an identity product and stored as
// two 16-byte vectors per lane.
template <class E>
__device__ inline void store_block(E *Oh, long long row0, int rows_left, const f32x4 num[4], f32x4 den, int n16,
                                   int g, const Frag<E> &ident) {
  f32x4 rden;
#pragma unroll
  for (int r = 0; r < 4; ++r) rden[r] = __builtin_amdgcn_rcpf(den[r]);
  f32x4 ot[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) ot[mt] = transpose_tile<E>(to_frag<E>(num[mt] * rden), ident);
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
  auto body = [&](const Chunk<E> &d, long long t0, int rows) {
    (void)t0;
    Frag<E> kf[4][4], vb[4][4];
    kv_frags<E>(d, rows, n16, ident, kf, vb);
    state_update<E>(st, kf, vb, ident);
  };
  if constexpr (std::is_same<E, __bf16>::value) {
    __shared__ u32x4 slot[StageShape<false, true>::kVec];
    stream_chunks_lds<false, true, 0>(slot, nullptr, Kh, Vh, t_begin, t_end, lane, n16, g, body);
  } else {
    stream_chunks<E, false, true>(nullptr, Kh, Vh, t_begin, t_end, n16, g, body);
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
    // The loads do not depend on the running sum: issue a batch of them,
    // then do the dependent stores, so each batch costs one memory latency.
    constexpr int kBatch = 32;
    for (int s0 = 0; s0 + 1 < P; s0 += kBatch) {
      float t[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (s0 + u + 1 < P) t[u] = recs[(long long)(s0 + u) * kStateFloats];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (s0 + u + 1 < P) {
          recs[(long long)(s0 + u) * kStateFloats] = run;
          run += t[u];
        }
    }
    recs[(long long)(P - 1) * kStateFloats] = run;
  } else {
    float run = 0.f;
    constexpr int kBatch = 32;
    for (int s0 = 0; s0 < P; s0 += kBatch) {
      float t[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) t[u] = s0 + u < P ? recs[(long long)(s0 + u) * kStateFloats] : 0.f;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) run += t[u];
    }
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

  // All four row tiles are computed even in a partial last chunk (rows past
  // the end read zeros and are not stored), keeping the loop branch-free.
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    f32x4 num[4] = {zero4(), zero4(), zero4(), zero4()};
    f32x4 den = zero4();
    // Inter-chunk read: phi(Q) S_prev and phi(Q) z_prev.
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        num[mt] = mac2<E>(num[mt], qf[it][2 * kp], qf[it][2 * kp + 1], sb[2 * kp][mt], sb[2 * kp + 1][mt]);
      den = mac2<E>(den, qf[it][2 * kp], qf[it][2 * kp + 1], zb[2 * kp], zb[2 * kp + 1]);
    }
    // Intra-chunk: A = tril(phi(Q) phi(K)^T) for key tiles jt <= it.  The
    // product phi(K) phi(Q)^T leaves lane (n, g) with A[i = n][j = 4g+r],
    // which is already the A operand of A V (k = key token).
    f32x4 at[4];
#pragma unroll
    for (int jt = 0; jt <= it; ++jt) at[jt] = zero4();
#pragma unroll
    for (int kp = 0; kp < 2; ++kp)
#pragma unroll
      for (int jt = 0; jt <= it; ++jt)
        at[jt] = mac2<E>(at[jt], kf[jt][2 * kp], kf[jt][2 * kp + 1], qf[it][2 * kp], qf[it][2 * kp + 1]);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * g + r > n16) at[it][r] = 0.f;  // inclusive mask j <= i ("Why Replace Attention?", §7.1)
    Frag<E> af[4];
#pragma unroll
    for (int jt = 0; jt <= it; ++jt) af[jt] = to_frag<E>(at[jt]);
#pragma unroll
    for (int jp = 0; 2 * jp + 1 <= it; ++jp) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) num[mt] = mac2<E>(num[mt], af[2 * jp], af[2 * jp + 1], vb[2 * jp][mt], vb[2 * jp + 1][mt]);
      den = mac2<E>(den, af[2 * jp], af[2 * jp + 1], ones, ones);
    }
    if ((it & 1) == 0) {  // odd number of key tiles: the diagonal one alone
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) num[mt] = mac1<E>(num[mt], af[it], vb[it][mt]);
      den = mac1<E>(den, af[it], ones);
    }
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

  auto body = [&](const Chunk<E> &d, long long t0, int rows) { causal_chunk<E>(st, d, rows, Oh, t0, n16, g, ident); };
  if constexpr (std::is_same<E, __bf16>::value) {
    __shared__ u32x4 slot[StageShape<true, true>::kVec];
    stream_chunks_lds<true, true, 8>(slot, Qh, Kh, Vh, t_begin, t_end, lane, n16, g, body);
  } else {
    stream_chunks<E, true, true>(Qh, Kh, Vh, t_begin, t_end, n16, g, body);
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

  auto body = [&](const Chunk<E> &d, long long t0, int rows) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      Frag<E> qf[4];
      slab_to_frags<E>(d.q[it], qf, true);
      f32x4 num[4] = {zero4(), zero4(), zero4(), zero4()};
      f32x4 den = zero4();
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          num[mt] = mac2<E>(num[mt], qf[2 * kp], qf[2 * kp + 1], sb[2 * kp][mt], sb[2 * kp + 1][mt]);
        den = mac2<E>(den, qf[2 * kp], qf[2 * kp + 1], zb[2 * kp], zb[2 * kp + 1]);
      }
      store_block<E>(Oh, t0 + 16 * it, rows - 16 * it, num, den, n16, g, ident);
    }
  };
  if constexpr (std::is_same<E, __bf16>::value) {
    __shared__ u32x4 slot[StageShape<true, false>::kVec];
    stream_chunks_lds<true, false, 8>(slot, Qh, nullptr, nullptr, t_begin, t_end, lane, n16, g, body);
  } else {
    stream_chunks<E, true, false>(Qh, nullptr, nullptr, t_begin, t_end, n16, g, body);
  }
}

}  // namespace linattn
