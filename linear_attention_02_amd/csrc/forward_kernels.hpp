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
// Products are laid out so that each result's accumulator tile is directly
// the operand of the next product (see device_common.hpp); outputs are
// computed transposed, o^T = S^T phi(Q)^T + V^T A^T, which leaves each lane
// with 8 adjacent output columns of one token (16-byte stores).
//
// Parallel structure.  One wave64 is one worker and owns a (head, segment)
// pair: a run of whole chunks it walks left to right.  Sequence segments make
// the grid wide enough for few-head workloads; their starting states come
// from a two-pass scan (segment totals, then an exclusive prefix per head),
// the parallel-scan resolution of the left-to-right dependency ("Why Replace
// Attention?", §7.7).  No inter-wave synchronisation: each wave's LDS is a
// private staging slot, and waves exchange data only through the workspace
// records, between kernel launches.
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

// kInitTotals: the workspace holds segment totals (no scan ran); the walk
// sums its own prefix from them, seeded with S0, z0 when given.
enum InitMode : int { kInitZero = 0, kInitRecord = 1, kInitNatural = 2, kInitTotals = 3 };

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
  const float *S0;     // natural order [heads][64][64] (kInitNatural, kInitTotals / scan seed)
  const float *z0;     // [heads][64]
  float *S_out;        // natural order final state, written by the last segment
  float *z_out;
  float *rden;         // [heads][rden_stride] 1/den per token (saving walk only)
  long long rden_stride;
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
// Fragments of one 64-token chunk, as the MFMA products consume them.
//   qf[it][kt]  phi(Q), row layout: lane (n, g) holds phi(Q)[16it+n][pi(kt,g,r)]
//   kf[jt][kt]  phi(K), row layout (A operand of phi(K) phi(Q)^T)
//   kt[jt][ct]  phi(K), token layout: lane (n, g) holds
//               phi(K)[16jt+4g+r][pi(ct,n>>2,n&3)] (A operand of phi(K)^T V)
//   vt[jt][mt]  V, token layout: lane (n, g) holds V[16jt+4g+r][pi(mt,n>>2,n&3)]
//               (B operand of phi(K)^T V, A operand of V^T A^T)
// Key rows past the end of the sequence are zero in kf, kt and vt.
// ---------------------------------------------------------------------------
__device__ inline int chunk_rows(long long t0, long long t_end) {
  return (int)(t_end - t0 < kChunk ? t_end - t0 : kChunk);
}

// Zero the registers of a token-layout fragment whose tokens are >= rows.
__device__ inline void mask_tokens(Frag<__bf16> &f, int tok0, int rows) {
  if (tok0 + 0 >= rows) f.w[0] &= 0xffff0000u;
  if (tok0 + 1 >= rows) f.w[0] &= 0x0000ffffu;
  if (tok0 + 2 >= rows) f.w[1] &= 0xffff0000u;
  if (tok0 + 3 >= rows) f.w[1] &= 0x0000ffffu;
}
__device__ inline void mask_tokens(Frag<float> &f, int tok0, int rows) {
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (tok0 + r >= rows) f.v[r] = 0.f;
}

template <class E> __device__ inline void phi_frag(Frag<E> &f);
template <> __device__ inline void phi_frag<__bf16>(Frag<__bf16> &f) {
  f.w[0] = pack_bf16(phi(bf16_lo(f.w[0])), phi(bf16_hi(f.w[0])));
  f.w[1] = pack_bf16(phi(bf16_lo(f.w[1])), phi(bf16_hi(f.w[1])));
}
template <> __device__ inline void phi_frag<float>(Frag<float> &f) {
#pragma unroll
  for (int r = 0; r < 4; ++r) f.v[r] = phi(f.v[r]);
}

// ---------------------------------------------------------------------------
// phi(Q) of one row tile, each query row scaled as phi_row_scale decides
// (device_common.hpp).  Lane (n, g) holds 16 of row n's features, so a lane's
// own maximum decides whether the row can need a scale; only then (rarely:
// never for inputs of moderate size) does the wave form each row's maximum
// across its four lanes.  Rows that need no scale get exactly phi.
// ---------------------------------------------------------------------------
__device__ inline float raw_elem(const Frag<__bf16> &f, int r) {
  const uint32_t w = f.w[r >> 1];
  return (r & 1) ? bf16_hi(w) : bf16_lo(w);
}
__device__ inline float raw_elem(const Frag<float> &f, int r) { return f.v[r]; }

template <class E> __device__ inline void phi_q_tile(Frag<E> f[4]) {
  float m = raw_elem(f[0], 0);
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) m = fmaxf(m, raw_elem(f[c], r));
  if (!__any(m > kPhiQHigh || m < kPhiQLow)) {
#pragma unroll
    for (int c = 0; c < 4; ++c) phi_frag<E>(f[c]);
    return;
  }
  // Row maximum over the lanes n, n + 16, n + 32, n + 48.
  m = fmaxf(m, __shfl_xor(m, 16, 64));
  m = fmaxf(m, __shfl_xor(m, 32, 64));
  float eneg;
  int epos;
  phi_row_scale(m, eneg, epos);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if constexpr (std::is_same<E, __bf16>::value) {
      f[c].w[0] = pack_bf16(phi_row_scaled(raw_elem(f[c], 0), eneg, epos), phi_row_scaled(raw_elem(f[c], 1), eneg, epos));
      f[c].w[1] = pack_bf16(phi_row_scaled(raw_elem(f[c], 2), eneg, epos), phi_row_scaled(raw_elem(f[c], 3), eneg, epos));
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) f[c].v[r] = phi_row_scaled(f[c].v[r], eneg, epos);
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 path: chunks staged in LDS.  The next chunk is fetched with
// global_load_lds_dwordx4 (HBM -> LDS without passing through VGPRs) into a
// wave-private slot while the current chunk is computed.  Each load
// instruction fetches 8 whole 128-byte rows: lane l loads row 8i + (l >> 3),
// 16-byte piece p = (l & 7) ^ (row & 7), and its bytes land at
// slot + 1024 i + 16 l.  So piece p of row R sits at 16-byte index
// 64 (R >> 3) + 8 (R & 7) + (p ^ (R & 7)); the XOR spreads the transpose
// reads below over the LDS banks.  No other wave touches the slot, so no
// barrier is needed -- only the wave's own wait counters.
//
// Row layout fragments: lane (n, g) reads pieces g and 4 + g of its row
// (ds_read_b128 each).  Token layout fragments come from ds_read_b64_tr_b16,
// which within each group of 16 lanes hands output lane i, register s,
// element i & 3 of the 8 bytes read by lane 4s + (i >> 2).  Lane (src, g)
// therefore reads row 16jt + 4g + (src >> 2), columns pi(mt, src & 3, 0..3),
// and lane (n, g) receives X[16jt + 4g + r][pi(mt, n >> 2, n & 3)], the token
// layout above.
// ---------------------------------------------------------------------------
__device__ inline int stage_index(int R, int p) { return 64 * (R >> 3) + 8 * (R & 7) + (p ^ (R & 7)); }

typedef __attribute__((address_space(3))) void lds_void;
typedef short i16x4_t __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

template <int kTensors, int NT = 4> struct Slot {
  static constexpr int kVec = kTensors * NT * 2 * 64;  // 16-byte vectors
  static constexpr int kLoads = kTensors * NT * 2;     // load instructions per chunk
};

// s_waitcnt with only vmcnt (resp. lgkmcnt) constrained.
template <int N> __device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ inline void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// Cache policy of the staging loads.  kLoadStreaming sets the non-temporal
// bit: measured on MI355X, a pass over data much larger than the 256 MB
// last-level cache reads faster with it, while data that fits is better left
// cacheable so that a following pass over the same tensors hits the cache.
constexpr int kLoadDefault = 0;
constexpr int kLoadStreaming = 2;

// Fetch rows [t0, t0 + rows) of the given tensors into the slot (chunks of
// NT row tiles of 16 tokens).
template <int kTensors, int NT = 4, int kPolicy = kLoadDefault>
__device__ inline void stage_issue(u32x4 *slot, const __bf16 *const src[kTensors], long long t0, int rows, int n16,
                                   int g) {
  const int lane = 16 * g + n16;
  const int sub = lane >> 3;                 // row within the instruction's 8
  const int piece = (lane & 7) ^ sub;        // (row & 7) == sub
#pragma unroll
  for (int tsr = 0; tsr < kTensors; ++tsr) {
#pragma unroll
    for (int i = 0; i < 2 * NT; ++i) {
      const int row = 8 * i + sub;
      if (row < rows)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const u32x4 *>(src[tsr] + (t0 + row) * kD) + piece,
                                         (lds_void *)(slot + (tsr * 2 * NT + i) * 64), 16, 0, kPolicy);
    }
  }
}

// Row layout fragments of tensor tsr, row tile it (raw, no phi).
template <int NT = 4>
__device__ inline void lds_row_frags(const u32x4 *slot, int tsr, int it, int lane, Frag<__bf16> f[4]) {
  const int R = 16 * it + (lane & 15), g = lane >> 4;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const u32x4 v = slot[tsr * 2 * NT * 64 + stage_index(R, 4 * x + g)];
    f[2 * x].w[0] = v[0];
    f[2 * x].w[1] = v[1];
    f[2 * x + 1].w[0] = v[2];
    f[2 * x + 1].w[1] = v[3];
  }
}

// Token layout fragment of tensor tsr, token tile jt, column tile mt (raw).
template <int NT = 4>
__device__ inline Frag<__bf16> lds_tok_frag(const u32x4 *slot, int tsr, int jt, int mt, int lane) {
  const int src = lane & 15, g = lane >> 4;
  const int R = 16 * jt + 4 * g + (src >> 2);
  const int byte = (tsr * 2 * NT * 64 + stage_index(R, 4 * (mt >> 1) + (src & 3))) * 16 + 8 * (mt & 1);
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4 *)(reinterpret_cast<__attribute__((address_space(3))) char *>((lds_void *)slot) + byte));
  Frag<__bf16> f;
  f.w[0] = (uint32_t)(uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
  f.w[1] = (uint32_t)(uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
  return f;
}

// As stage_issue, but every lane takes part in every load: rows at or past
// `rows` read row rows - 1 again.  A chunk then always costs exactly
// Slot<kTensors, NT>::kLoads load instructions, so a loop with several
// chunks in flight can count its outstanding loads exactly.  The slot's
// positions of rows past the end hold copies the caller masks or never stores.
template <int kTensors, int NT = 4, int kPolicy = kLoadDefault>
__device__ inline void stage_issue_counted(u32x4 *slot, const __bf16 *const src[kTensors], long long t0, int rows,
                                           int n16, int g) {
  const int lane = 16 * g + n16;
  const int sub = lane >> 3;
  const int piece = (lane & 7) ^ sub;
#pragma unroll
  for (int tsr = 0; tsr < kTensors; ++tsr) {
#pragma unroll
    for (int i = 0; i < 2 * NT; ++i) {
      const int row = min(8 * i + sub, rows - 1);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const u32x4 *>(src[tsr] + (t0 + row) * kD) + piece,
                                       (lds_void *)(slot + (tsr * 2 * NT + i) * 64), 16, 0, kPolicy);
    }
  }
}

// LDS reads issued from inline assembly, for loops that keep several chunks
// of LDS-DMA loads, or output stores, in flight.  Before an LDS read that
// follows LDS-DMA loads, the compiler may wait for every outstanding
// vector-memory operation (the newest DMA loads and the stores included),
// which would collapse such a pipeline to one chunk.  These reads are
// invisible to the compiler's wait counting, so the caller (1) has waited for
// the DMA loads of the chunk it reads itself, and (2) calls lds_reads_done,
// then passes every value read this way through after_lds_reads, before any
// use of it.
template <int NT = 4>
__device__ inline Frag<__bf16> lds_tok_frag_untracked(const u32x4 *slot, int tsr, int jt, int mt, int lane) {
  const int src = lane & 15, g = lane >> 4;
  const int R = 16 * jt + 4 * g + (src >> 2);
  const int byte = (tsr * 2 * NT * 64 + stage_index(R, 4 * (mt >> 1) + (src & 3))) * 16 + 8 * (mt & 1);
  const uint32_t addr = (uint32_t)(size_t)(lds_void *)slot + byte;
  Frag<__bf16> f;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(f.w) : "v"(addr));
  return f;
}

// lds_row_frags for bf16 (raw, no phi), read as lds_tok_frag_untracked is.
template <int NT = 4>
__device__ inline void lds_row_frags_untracked(const u32x4 *slot, int tsr, int it, int lane, Frag<__bf16> f[4]) {
  const int R = 16 * it + (lane & 15), g = lane >> 4;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const uint32_t addr = (uint32_t)(size_t)(lds_void *)slot + 16 * (tsr * 2 * NT * 64 + stage_index(R, 4 * x + g));
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
    f[2 * x].w = u32x2{v[0], v[1]};
    f[2 * x + 1].w = u32x2{v[2], v[3]};
  }
}

// Waits for every LDS read of this wave (lgkmcnt(0)).  The memory clobber
// keeps later LDS-DMA refills of the slot after it.
__device__ inline void lds_reads_done() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Makes each of the n fragments depend on the lds_reads_done before it, so
// that no use of them is scheduled ahead of that wait.
template <int n> __device__ inline void after_lds_reads(Frag<__bf16> *f) {
#pragma unroll
  for (int i = 0; i < n; ++i) asm volatile("" : "+v"(f[i].w));
}

// Walks the chunks [t_begin, t_end), the first one prefetched here.
// body(slot, t0, rows) runs on each chunk once its loads have landed: it reads
// the slot into registers, waits for lgkmcnt(0), issues the next chunk's loads
// into the same slot and then computes, so one chunk streams in while one is
// computed.  kStores is the number of vector-memory stores body() issues on a
// full chunk.
template <int kTensors, int kStores, int kPolicy, class Body>
__device__ inline void stream_lds(u32x4 *slot, const __bf16 *const src[kTensors], long long t_begin, long long t_end,
                                  int n16, int g, Body &&body) {
  if (t_begin >= t_end) return;
  stage_issue<kTensors, 4, kPolicy>(slot, src, t_begin, chunk_rows(t_begin, t_end), n16, g);
  for (long long t0 = t_begin; t0 < t_end; t0 += kChunk) {
    const int rows = chunk_rows(t0, t_end);
    // Outstanding vector-memory operations: this chunk's loads, then the
    // previous chunk's kStores stores (every chunk but the last is full).
    // They retire in order, so waiting down to kStores leaves only stores
    // in flight.  The first chunk has nothing behind its loads.
    if (t0 == t_begin) {
      wait_vmcnt<0>();
    } else {
      wait_vmcnt<kStores>();
    }
    body(slot, t0, rows);
  }
}

// ---------------------------------------------------------------------------
// fp32 path.
// ---------------------------------------------------------------------------
// fp32 chunks staged in LDS.  A row is 64 floats, sixteen 16-byte pieces;
// piece p of row r of a tensor's region sits at 16-byte unit
// 16 r + (p ^ (r & 15)), so that the sixteen rows a row-layout read touches
// at once fall on different banks.  One load instruction fetches four whole
// rows: lane l loads row 4i + (l >> 4), piece (l & 15) ^ (row & 15), and its
// bytes land at unit 64 i + l.
template <int kTensors, int NT>
__device__ inline void stage_issue_f32(u32x4 *slot, const float *const src[kTensors], long long t0, int rows,
                                       int lane) {
  const int sub = lane >> 4;
#pragma unroll
  for (int tsr = 0; tsr < kTensors; ++tsr) {
#pragma unroll
    for (int i = 0; i < 4 * NT; ++i) {
      const int row = 4 * i + sub;
      const int piece = (lane & 15) ^ (row & 15);
      if (row < rows)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const u32x4 *>(src[tsr] + (t0 + row) * kD) + piece,
                                         (lds_void *)(slot + (tsr * 16 * NT + 4 * i) * 16), 16, 0, kLoadDefault);
    }
  }
}

// The slab of row tile it of tensor tsr (rows past `rows` read as zero: the
// slot still holds an earlier chunk there, or nothing yet).
template <int NT>
__device__ inline void slab_from_lds_f32(Slab<float> &s, const u32x4 *slot, int tsr, int it, int rows, int n16,
                                         int g) {
  const int R = 16 * it + n16;
  if (R >= rows) {
    slab_zero<float>(s);
    return;
  }
  const u32x4 *row = slot + (tsr * 16 * NT + R) * 16;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) s.h[x][y] = __builtin_bit_cast(f32x4, row[(8 * x + 2 * g + y) ^ (R & 15)]);
}

// Row tiles per chunk of the fp32 walk: 32-token chunks, so that Q, K and V
// of one chunk (24 KB) stage in LDS like the bf16 walk's 64-token chunk.
constexpr int kWalkTilesF32 = 2;

// Token layout from row layout by an identity product (exact).
template <class E, int NT = 4>
__device__ inline void row_to_tok(const Frag<E> rowf[NT][4], Frag<E> tok[NT][4], const Frag<E> &ident) {
#pragma unroll
  for (int jt = 0; jt < NT; ++jt)
#pragma unroll
    for (int c = 0; c < 4; ++c) tok[jt][c] = to_frag<E>(transpose_tile<E>(rowf[jt][c], ident));
}

// ---------------------------------------------------------------------------
// Shared math.
// ---------------------------------------------------------------------------
// S += phi(K_c)^T V_c and z += column sums of phi(K_c) ("Why Replace
// Attention?", §7.2, applied to a chunk of tokens at once).
template <class E, int NT = 4>
__device__ inline void state_update(State &st, const Frag<E> kt[NT][4], const Frag<E> vt[NT][4]) {
  const Frag<E> ones = frag_ones<E>();
#pragma unroll
  for (int jp = 0; jp < NT / 2; ++jp) {  // pairs of token tiles
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        st.S[ct][mt] = mac2<E>(st.S[ct][mt], kt[2 * jp][ct], kt[2 * jp + 1][ct], vt[2 * jp][mt], vt[2 * jp + 1][mt]);
      st.z[ct] = mac2<E>(st.z[ct], kt[2 * jp][ct], kt[2 * jp + 1][ct], ones, ones);
    }
  }
}

// Operands of the state read: S as the A operand of S^T phi(Q)^T (row n =
// value column, k = feature) and z likewise (every row equal).
template <class E> struct StateOperands {
  Frag<E> sa[4][4];  // [kt][mt]
  Frag<E> za[4];     // [kt]
};
template <class E> __device__ inline void state_operands(const State &st, StateOperands<E> &so) {
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) so.sa[kt][mt] = to_frag<E>(st.S[kt][mt]);
    so.za[kt] = to_frag<E>(st.z[kt]);
  }
}

// num^T (4 tiles: value columns pi(mt, g, r), token n) and den for the 16
// tokens of row tile qf: the state read phi(Q) S and phi(Q) z.
template <class E>
__device__ inline void state_read(const StateOperands<E> &so, const Frag<E> qf[4], f32x4 nt[4], f32x4 &dt) {
  const Frag<E> q0 = qf[0], q1 = qf[1], q2 = qf[2], q3 = qf[3];
  const Frag<E> z0 = so.za[0], z1 = so.za[1], z2 = so.za[2], z3 = so.za[3];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) nt[mt] = mac2<E>(nt[mt], so.sa[0][mt], so.sa[1][mt], q0, q1);
  dt = mac2<E>(dt, z0, z1, q0, q1);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) nt[mt] = mac2<E>(nt[mt], so.sa[2][mt], so.sa[3][mt], q2, q3);
  dt = mac2<E>(dt, z2, z3, q2, q3);
}

// Store four accumulator tiles of 16 tokens: lane (n, g) holds token n's
// columns pi(mt, g, r) = 32x + 8g + 4y + r for mt = 2x + y, i.e. two runs of
// 8 adjacent columns.
//
// bf16: token n's 16 values are two 16-byte pieces (x = 0, 1) of its 128-byte
// row, one per lane group g.  Lanes n and n ^ 8 of each 16-lane row swap one
// piece (DPP row rotate by 8), after which one store instruction covers rows
// 0-7 of the tile and the other rows 8-15, each as whole 128-byte lines:
// lane n < 8 writes (row n, x = 0) then (row n + 8, x = 0); lane n >= 8 writes
// (row n - 8, x = 1) then (row n, x = 1).  Whole-line non-temporal writes
// reach memory without partial-line overhead.
template <class E, bool kFull>
__device__ inline void store_tiles(E *base, long long row0, int rows_left, const f32x4 a[4], int n16, int g) {
  if constexpr (std::is_same<E, __bf16>::value) {
    const u32x4 p0 = {pack_bf16(a[0][0], a[0][1]), pack_bf16(a[0][2], a[0][3]), pack_bf16(a[1][0], a[1][1]),
                      pack_bf16(a[1][2], a[1][3])};
    const u32x4 p1 = {pack_bf16(a[2][0], a[2][1]), pack_bf16(a[2][2], a[2][3]), pack_bf16(a[3][0], a[3][1]),
                      pack_bf16(a[3][2], a[3][3])};
    const bool low = n16 < 8;
    u32x4 send = low ? p1 : p0, recv;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      recv[i] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send[i], 0x128 /* row_ror:8 */, 0xf, 0xf, false);
    const u32x4 first = low ? p0 : recv, second = low ? recv : p1;
    const int r_first = n16 & 7, x = n16 >> 3;
    if (kFull || r_first < rows_left)
      __builtin_nontemporal_store(first, reinterpret_cast<u32x4 *>(base + (row0 + r_first) * kD) + 4 * x + g);
    if (kFull || r_first + 8 < rows_left)
      __builtin_nontemporal_store(second, reinterpret_cast<u32x4 *>(base + (row0 + r_first + 8) * kD) + 4 * x + g);
  } else {
    if (kFull || n16 < rows_left) {
      E *row = base + (row0 + n16) * kD;
      store_row8<E>(row, g, 0, a[0], a[1]);
      store_row8<E>(row, g, 1, a[2], a[3]);
    }
  }
}

// o = num / den for 16 tokens (num^T tiles nt, den in every register of dt),
// stored as above.
template <class E, bool kFull = false>
__device__ inline void store_rows(E *Oh, long long row0, int rows_left, const f32x4 nt[4], f32x4 dt, int n16, int g) {
  const float rd = __builtin_amdgcn_rcpf(dt[0]);
  const f32x4 a[4] = {nt[0] * rd, nt[1] * rd, nt[2] * rd, nt[3] * rd};
  store_tiles<E, kFull>(Oh, row0, rows_left, a, n16, g);
}

// ---------------------------------------------------------------------------
// Pass 1: per-segment totals of phi(K)^T V and phi(K).
// ---------------------------------------------------------------------------
// LDS staging of one totals wave: K and V of one 64-token chunk (bf16: 16 KB;
// fp32: 32 KB), as 16-byte vectors.
template <class E> struct TotalsSlot;
template <> struct TotalsSlot<__bf16> { static constexpr int kVec = Slot<2>::kVec; };
template <> struct TotalsSlot<float> { static constexpr int kVec = 2 * 16 * 4 * 16; };

// st = phi(K)^T V and the column sums of phi(K) over tokens [t_begin, t_end)
// of one head, streamed through the wave's slot.
template <class E, int kPolicy>
__device__ inline void range_totals(State &st, u32x4 *slot, const E *Kh, const E *Vh, long long t_begin,
                                    long long t_end, int lane) {
  const int n16 = lane & 15, g = lane >> 4;
  state_zero(st);
  if constexpr (std::is_same<E, __bf16>::value) {
    const __bf16 *src[2] = {Kh, Vh};
    stream_lds<2, 0, kPolicy>(slot, src, t_begin, t_end, n16, g, [&](const u32x4 *sl, long long t0, int rows) {
      Frag<E> kt[4][4], vt[4][4];
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          kt[jt][c] = lds_tok_frag(sl, 0, jt, c, lane);
          vt[jt][c] = lds_tok_frag(sl, 1, jt, c, lane);
        }
      wait_lgkmcnt0();
      if (t0 + kChunk < t_end)
        stage_issue<2, 4, kPolicy>(slot, src, t0 + kChunk, chunk_rows(t0 + kChunk, t_end), n16, g);
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int c = 0; c < 4; ++c) phi_frag<E>(kt[jt][c]);
      if (rows < kChunk) {
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            mask_tokens(kt[jt][c], 16 * jt + 4 * g, rows);
            mask_tokens(vt[jt][c], 16 * jt + 4 * g, rows);
          }
      }
      state_update<E>(st, kt, vt);
    });
  } else {
    // fp32: K and V of a 64-token chunk (32 KB) staged in LDS, the next
    // chunk's loads in flight while this one is computed.
    const Frag<E> ident = frag_identity<E>(n16, g);
    constexpr int NT = 4;
    const float *src[2] = {Kh, Vh};
    if (t_begin < t_end) stage_issue_f32<2, NT>(slot, src, t_begin, chunk_rows(t_begin, t_end), lane);
    for (long long t0 = t_begin; t0 < t_end; t0 += kChunk) {
      const int rows = chunk_rows(t0, t_end);
      wait_vmcnt<0>();  // no stores: everything outstanding is this chunk's loads
      Slab<float> d[2][NT];
#pragma unroll
      for (int jt = 0; jt < NT; ++jt)
#pragma unroll
        for (int tsr = 0; tsr < 2; ++tsr) slab_from_lds_f32<NT>(d[tsr][jt], slot, tsr, jt, rows, n16, g);
      wait_lgkmcnt0();
      if (t0 + kChunk < t_end) stage_issue_f32<2, NT>(slot, src, t0 + kChunk, chunk_rows(t0 + kChunk, t_end), lane);
      Frag<E> kf[4][4], vf[4][4], kt[4][4], vt[4][4];
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        slab_to_frags<E>(d[0][jt], kf[jt], true);
        if (16 * jt + n16 >= rows)
#pragma unroll
          for (int c = 0; c < 4; ++c) kf[jt][c] = frag_zero<E>();
        slab_to_frags<E>(d[1][jt], vf[jt], false);
      }
      row_to_tok<E>(kf, kt, ident);
      row_to_tok<E>(vf, vt, ident);
      state_update<E>(st, kt, vt);
    }
  }
}

template <class E, int kPolicy = kLoadDefault>
__global__ __launch_bounds__(64, 1) void seg_totals_kernel(FwdParams p, int total_segments) {
  const int worker = blockIdx.x;
  const int h = worker % p.heads;
  const int s = worker / p.heads;
  if (s >= total_segments) return;
  const int lane = threadIdx.x;
  const int n16 = lane & 15, g = lane >> 4;
  const long long base = (long long)h * p.N * kD;
  const long long t_begin = (long long)s * p.seg_chunks * kChunk;
  long long t_end = t_begin + (long long)p.seg_chunks * kChunk;
  if (t_end > p.N) t_end = p.N;
  __shared__ u32x4 slot[TotalsSlot<E>::kVec];
  State st;
  range_totals<E, kPolicy>(st, slot, reinterpret_cast<const E *>(p.K) + base, reinterpret_cast<const E *>(p.V) + base,
                           t_begin, t_end, lane);
  float *rec = p.ws + ((long long)h * p.records + s) * kStateFloats;
  state_store_record(st, rec, lane, n16, g);
}

// ---------------------------------------------------------------------------
// Non-causal pass 1 in workgroups: kGroupWaves waves of one head take
// consecutive segments, and their partial states meet in the LDS (the
// staging slots, free once the chunks are consumed), where they are added in
// wave order and written as one record per group.  The head's total is the
// sum of its `groups` records, in record order, which the read pass forms
// itself: no scan launch.
// ---------------------------------------------------------------------------
constexpr int kGroupWaves = 4;
constexpr int kStateVecs = kStateFloats / 4;

template <class E> struct GroupSlot {
  static constexpr int kVec = TotalsSlot<E>::kVec > kStateVecs ? TotalsSlot<E>::kVec : kStateVecs;
};

template <class E, int kPolicy = kLoadDefault>
__global__ __launch_bounds__(64 * kGroupWaves, 1) void group_totals_kernel(FwdParams p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n16 = lane & 15, g = lane >> 4;
  const int h = blockIdx.x % p.heads;
  const int grp = blockIdx.x / p.heads;
  const int s = grp * kGroupWaves + wave;
  __shared__ u32x4 slots[kGroupWaves][GroupSlot<E>::kVec];
  State st;
  if (s < p.segments) {
    const long long base = (long long)h * p.N * kD;
    const long long t_begin = (long long)s * p.seg_chunks * kChunk;
    long long t_end = t_begin + (long long)p.seg_chunks * kChunk;
    if (t_end > p.N) t_end = p.N;
    range_totals<E, kPolicy>(st, slots[wave], reinterpret_cast<const E *>(p.K) + base,
                             reinterpret_cast<const E *>(p.V) + base, t_begin, t_end, lane);
  } else {
    state_zero(st);
  }
  wait_vmcnt<0>();
  state_store_record(st, reinterpret_cast<float *>(slots[wave]), lane, n16, g);
  __syncthreads();
  f32x4 *rec = reinterpret_cast<f32x4 *>(p.ws + ((long long)h * p.records + grp) * kStateFloats);
  for (int v = threadIdx.x; v < kStateVecs; v += 64 * kGroupWaves) {
    f32x4 a = __builtin_bit_cast(f32x4, slots[0][v]);
#pragma unroll
    for (int w = 1; w < kGroupWaves; ++w) a += __builtin_bit_cast(f32x4, slots[w][v]);
    rec[v] = a;
  }
}

// ---------------------------------------------------------------------------
// Scan over segment records, one thread per (head, W consecutive state
// elements).
//   causal:     records 0..P-2 hold totals -> become exclusive prefixes seeded
//               with S0/z0 (or zero); record P-1 receives the prefix of the
//               last segment.
//   reverse:    the same over the records in the opposite order: records
//               P-1..1 hold totals and become exclusive suffix sums (sums over
//               the later segments); record 0 receives the suffix of segment 0.
//   non-causal: record P receives the sum of records 0..P-1.
// The loads do not depend on the running sum, so they are issued in batches
// (one memory latency per batch) before the dependent stores.  Every element
// is summed in record order, so results are deterministic and do not depend
// on W or the batch.  The host picks W = 4 (wide accesses) when that still
// gives a launch of at least 256 blocks, else W = 1, and a batch of eight for
// up to eight records (fewer registers, more resident waves).
// ---------------------------------------------------------------------------
constexpr int kScanBatchSmall = 8;
constexpr int kScanBatchLarge = 32;
static_assert(kStateFloats % 4 == 0, "state records split into whole vectors");

enum ScanMode : int { kScanTotal = 0, kScanPrefix = 1, kScanSuffix = 2 };

template <int W> struct ScanVecType;
template <> struct ScanVecType<1> { typedef float type; };
template <> struct ScanVecType<4> { typedef f32x4 type; };

// Element e of a head's record, from the natural-order S0, z0 (record layout:
// S tiles [ct][mt][lane][r], then z [ct][g][r]).
__device__ inline float scan_seed(const FwdParams &p, int h, int e) {
  if (e < 4096) {
    const int ct = e >> 10, mt = (e >> 8) & 3, lane = (e >> 2) & 63, r = e & 3;
    const int c = pi_col(ct, lane >> 4, r);
    const int m = pi_col(mt, (lane & 15) >> 2, lane & 3);
    return p.S0[(long long)h * 4096 + c * 64 + m];
  }
  const int f = e - 4096;
  const int ct = f >> 4, g = (f >> 2) & 3, r = f & 3;
  return p.z0[(long long)h * 64 + pi_col(ct, g, r)];
}

template <int W, int kBatch>
__global__ __launch_bounds__(256) void scan_kernel(FwdParams p, int mode) {
  typedef typename ScanVecType<W>::type V;
  constexpr int kThreads = kStateFloats / W;  // per head
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int h = (int)(idx / kThreads);
  const int e0 = (int)(idx % kThreads) * W;
  if (h >= p.heads) return;
  const int P = p.segments;
  // Logical record s lives at position s (prefix) or P - 1 - s (suffix).
  const long long step = (mode == kScanSuffix ? -(long long)kStateFloats : (long long)kStateFloats) / W;
  V *recs = reinterpret_cast<V *>(p.ws + (long long)h * p.records * kStateFloats + e0 +
                                  (mode == kScanSuffix ? (long long)(P - 1) * kStateFloats : 0));
  if (mode != kScanTotal) {
    V run = V{};
    if (mode == kScanPrefix && p.S0 != nullptr) {
      float *run_e = reinterpret_cast<float *>(&run);
#pragma unroll
      for (int r = 0; r < W; ++r) run_e[r] = scan_seed(p, h, e0 + r);
    }
    for (int s0 = 0; s0 + 1 < P; s0 += kBatch) {
      V t[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (s0 + u + 1 < P) t[u] = recs[(long long)(s0 + u) * step];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (s0 + u + 1 < P) {
          recs[(long long)(s0 + u) * step] = run;
          run += t[u];
        }
    }
    recs[(long long)(P - 1) * step] = run;
  } else {
    V run = V{};
    for (int s0 = 0; s0 < P; s0 += kBatch) {
      V t[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) t[u] = s0 + u < P ? recs[(long long)(s0 + u) * step] : V{};
#pragma unroll
      for (int u = 0; u < kBatch; ++u) run += t[u];
    }
    recs[(long long)P * step] = run;
  }
}

// ---------------------------------------------------------------------------
// The same scans for many records per head (few heads, very long sequences),
// where one thread per element would walk hundreds of records one batch after
// another.  A block covers kScanVecs four-element vectors of one head's
// records with kScanGroups groups of threads; group g owns a run of `per`
// consecutive records.  Each thread sums its run, the run totals meet in LDS,
// and each thread then writes its records' prefixes starting from the sum of
// the earlier runs.  Additions run in a fixed order (runs in record order,
// records in order within a run), so results are deterministic.
// ---------------------------------------------------------------------------
constexpr int kScanGroups = 32;
constexpr int kScanVecs = 256 / kScanGroups;
constexpr int kScanRunBatch = 32;  // records of a run loaded at once
constexpr int kScanBlocksPerHead = (kStateFloats / 4 + kScanVecs - 1) / kScanVecs;

__global__ __launch_bounds__(256) void scan_grouped_kernel(FwdParams p, int mode) {
  const long long hb = blockIdx.x;
  const int h = (int)(hb / kScanBlocksPerHead);
  const int vb = (int)(hb % kScanBlocksPerHead);
  const int grp = threadIdx.x / kScanVecs, lv = threadIdx.x % kScanVecs;
  const int e4 = vb * kScanVecs + lv;
  const bool active = e4 < kStateFloats / 4;
  const int P = p.segments;
  const int cnt = mode == kScanTotal ? P : P - 1;  // records summed
  const int per = (cnt + kScanGroups - 1) / kScanGroups;
  const int j0 = min(cnt, grp * per), j1 = min(cnt, j0 + per);
  // Logical record j lives at position j (prefix, total) or P - 1 - j (suffix).
  const long long step = (mode == kScanSuffix ? -(long long)kStateFloats : (long long)kStateFloats) / 4;
  f32x4 *recs = reinterpret_cast<f32x4 *>(p.ws + (long long)h * p.records * kStateFloats +
                                          (mode == kScanSuffix ? (long long)(P - 1) * kStateFloats : 0)) +
                e4;
  __shared__ f32x4 run_total[kScanGroups][kScanVecs];
  f32x4 t[kScanRunBatch];
  f32x4 local = f32x4{0.f, 0.f, 0.f, 0.f};
  if (active) {
    for (int b = j0; b < j1; b += kScanRunBatch) {
#pragma unroll
      for (int u = 0; u < kScanRunBatch; ++u)
        if (b + u < j1) t[u] = recs[(long long)(b + u) * step];
#pragma unroll
      for (int u = 0; u < kScanRunBatch; ++u)
        if (b + u < j1) local += t[u];
    }
  }
  run_total[grp][lv] = local;
  __syncthreads();
  if (!active) return;
  if (mode == kScanTotal) {
    if (grp == 0) {
      f32x4 run = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int g2 = 0; g2 < kScanGroups; ++g2) run += run_total[g2][lv];
      recs[(long long)P * step] = run;
    }
    return;
  }
  f32x4 run = f32x4{0.f, 0.f, 0.f, 0.f};
  if (mode == kScanPrefix && p.S0 != nullptr) {
#pragma unroll
    for (int r = 0; r < 4; ++r) run[r] = scan_seed(p, h, 4 * e4 + r);
  }
  for (int g2 = 0; g2 < grp; ++g2) run += run_total[g2][lv];
  // The run's records are read again unless they are all still held in t.
  const bool held = j1 - j0 <= kScanRunBatch;
  for (int b = j0; b < j1; b += kScanRunBatch) {
    if (!held) {
#pragma unroll
      for (int u = 0; u < kScanRunBatch; ++u)
        if (b + u < j1) t[u] = recs[(long long)(b + u) * step];
    }
#pragma unroll
    for (int u = 0; u < kScanRunBatch; ++u)
      if (b + u < j1) {
        recs[(long long)(b + u) * step] = run;
        run += t[u];
      }
  }
  if (j0 < j1 && j1 == cnt) recs[(long long)cnt * step] = run;
}

// ---------------------------------------------------------------------------
// Prefix of segment s summed by its own walk wave: st (the seed S0, z0 or
// zero) += totals records 0..s-1, in record order -- the same additions, in
// the same order, as the prefix scan, so the state is bit-identical (the
// backward's reverse walk sums the later segments' records the same way,
// last first, as the suffix scan does).  Used for few segments per head,
// where it costs less than a scan launch; two records are loaded before they
// are added.
// ---------------------------------------------------------------------------
constexpr int kSumInWalkMaxSegments = 8;

__device__ inline void state_add(State &st, const State &t) {
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    st.z[a] += t.z[a];
#pragma unroll
    for (int b = 0; b < 4; ++b) st.S[a][b] += t.S[a][b];
  }
}

// st += records first, first + stride, ... (count of them, in that order).
__device__ inline void state_add_records(State &st, const float *first, int count, long long stride, int lane,
                                         int g) {
  int j = 0;
  for (; j + 2 <= count; j += 2) {
    State a, b;
    state_load_record(a, first + j * stride, lane, g);
    state_load_record(b, first + (j + 1) * stride, lane, g);
    state_add(st, a);
    state_add(st, b);
  }
  if (j < count) {
    State a;
    state_load_record(a, first + j * stride, lane, g);
    state_add(st, a);
  }
}

// ---------------------------------------------------------------------------
// Causal walk: outputs of one segment, starting from its prefix state.
// ---------------------------------------------------------------------------
// kSave: also store 1/den_i to rdh[t0 + i] as the walk forms it, for the
// query row as scaled by phi_q_tile (a reader recovers the row's exponent
// from q_i with phi_row_scale); lanes g = 0 store each row tile's 16.
template <class E, int NT, bool kFull, bool kSave = false>
__device__ inline void causal_chunk(State &st, const Frag<E> qf[NT][4], const Frag<E> kf[NT][4],
                                    const Frag<E> kt[NT][4], const Frag<E> vt[NT][4], int rows, E *Oh, long long t0,
                                    int n16, int g, float *rdh = nullptr) {
  StateOperands<E> so;
  state_operands<E>(st, so);  // the state before this chunk (updated at the end)
  const Frag<E> ones = frag_ones<E>();
  // All row tiles are computed even in a partial last chunk (rows past the
  // end are not stored), keeping the tile loop branch-free.
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    f32x4 nt[4] = {zero4(), zero4(), zero4(), zero4()};
    f32x4 dt = zero4();
    // Inter-chunk read: phi(Q) S_prev and phi(Q) z_prev.
    state_read<E>(so, qf[it], nt, dt);
    // Intra-chunk: A^T = phi(K) phi(Q)^T for key tiles jt <= it; lane (n, g)
    // holds A[i = n][j = 4g+r], the B operand of V^T A^T (k = key token).
    f32x4 at[NT];
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
    Frag<E> af[NT];
#pragma unroll
    for (int jt = 0; jt <= it; ++jt) af[jt] = to_frag<E>(at[jt]);
#pragma unroll
    for (int jp = 0; 2 * jp + 1 <= it; ++jp) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) nt[mt] = mac2<E>(nt[mt], vt[2 * jp][mt], vt[2 * jp + 1][mt], af[2 * jp], af[2 * jp + 1]);
      dt = mac2<E>(dt, ones, ones, af[2 * jp], af[2 * jp + 1]);
    }
    if ((it & 1) == 0) {  // odd number of key tiles: the diagonal one alone
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) nt[mt] = mac1<E>(nt[mt], vt[it][mt], af[it]);
      dt = mac1<E>(dt, ones, af[it]);
    }
    store_rows<E, kFull>(Oh, t0 + 16 * it, rows - 16 * it, nt, dt, n16, g);
    // Every register of dt, in every lane group g, holds the denominator of
    // row n of this tile: the four groups store the same value (one store
    // instruction, no branch on g).
    if constexpr (kSave)
      if (kFull || 16 * it + n16 < rows) rdh[t0 + 16 * it + n16] = __builtin_amdgcn_rcpf(dt[0]);
  }
  state_update<E, NT>(st, kt, vt);
}

// bf16 chunk body: registers from the slot, refill the slot with the next
// chunk, then compute.  kFull: every row of the chunk is inside the sequence
// (all chunks but possibly a segment's last), so no masking is compiled in.
template <int NT, bool kFull, bool kSave = false>
__device__ inline void causal_chunk_lds(State &st, u32x4 *slot, const __bf16 *const src[3], long long t0,
                                        long long t_end, int rows, __bf16 *Oh, int lane, int n16, int g,
                                        const Frag<__bf16> &ident, float *rdh = nullptr) {
  typedef __bf16 E;
  constexpr int kT = 16 * NT;
  Frag<E> qf[NT][4], kf[NT][4], kt[NT][4], vt[NT][4];
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    lds_row_frags<NT>(slot, 0, it, lane, qf[it]);
    lds_row_frags<NT>(slot, 1, it, lane, kf[it]);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) vt[it][mt] = lds_tok_frag<NT>(slot, 2, it, mt, lane);
  }
  wait_lgkmcnt0();  // the slot is refilled only after every lane's read of it returned
  if (t0 + kT < t_end) stage_issue<3, NT>(slot, src, t0 + kT, (int)min<long long>(kT, t_end - t0 - kT), n16, g);
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    phi_q_tile<E>(qf[it]);
#pragma unroll
    for (int c = 0; c < 4; ++c) phi_frag<E>(kf[it][c]);
  }
  if (!kFull) {
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
      if (16 * jt + n16 >= rows)
#pragma unroll
        for (int c = 0; c < 4; ++c) kf[jt][c] = frag_zero<E>();
#pragma unroll
      for (int c = 0; c < 4; ++c) mask_tokens(vt[jt][c], 16 * jt + 4 * g, rows);
    }
  }
  row_to_tok<E, NT>(kf, kt, ident);
  causal_chunk<E, NT, kFull, kSave>(st, qf, kf, kt, vt, rows, Oh, t0, n16, g, rdh);
}

// Chunk body of the ring walk (LINATTN_WALK_RING): the chunk's slot is read
// with reads the compiler does not track (its loads have landed), and no
// refill is issued here.
template <int NT, bool kFull, bool kSave = false>
__device__ inline void causal_chunk_ring(State &st, const u32x4 *slot, long long t0, int rows, __bf16 *Oh, int lane,
                                         int n16, int g, const Frag<__bf16> &ident, float *rdh = nullptr) {
  typedef __bf16 E;
  Frag<E> qf[NT][4], kf[NT][4], kt[NT][4], vt[NT][4];
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    lds_row_frags_untracked<NT>(slot, 0, it, lane, qf[it]);
    lds_row_frags_untracked<NT>(slot, 1, it, lane, kf[it]);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) vt[it][mt] = lds_tok_frag_untracked<NT>(slot, 2, it, mt, lane);
  }
  lds_reads_done();
  after_lds_reads<4 * NT>(&qf[0][0]);
  after_lds_reads<4 * NT>(&kf[0][0]);
  after_lds_reads<4 * NT>(&vt[0][0]);
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    phi_q_tile<E>(qf[it]);
#pragma unroll
    for (int c = 0; c < 4; ++c) phi_frag<E>(kf[it][c]);
  }
  if (!kFull) {
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
      if (16 * jt + n16 >= rows)
#pragma unroll
        for (int c = 0; c < 4; ++c) kf[jt][c] = frag_zero<E>();
#pragma unroll
      for (int c = 0; c < 4; ++c) mask_tokens(vt[jt][c], 16 * jt + 4 * g, rows);
    }
  }
  row_to_tok<E, NT>(kf, kt, ident);
  causal_chunk<E, NT, kFull, kSave>(st, qf, kf, kt, vt, rows, Oh, t0, n16, g, rdh);
}

// s_waitcnt vmcnt(kLoads * later + kStores * stored) for later, stored in
// 0..2, known only at run time.
template <int kLoads, int kStores> __device__ inline void wait_ring(int later, int stored) {
  static_assert(2 * kLoads + 2 * kStores < 64, "vmcnt range");
  switch (3 * later + stored) {
  case 0: wait_vmcnt<0>(); break;
  case 1: wait_vmcnt<kStores>(); break;
  case 2: wait_vmcnt<2 * kStores>(); break;
  case 3: wait_vmcnt<kLoads>(); break;
  case 4: wait_vmcnt<kLoads + kStores>(); break;
  case 5: wait_vmcnt<kLoads + 2 * kStores>(); break;
  case 6: wait_vmcnt<2 * kLoads>(); break;
  case 7: wait_vmcnt<2 * kLoads + kStores>(); break;
  default: wait_vmcnt<2 * kLoads + 2 * kStores>(); break;
  }
}

// Row tiles per chunk of the bf16 walk: 4 (64-token chunks, the default) or
// 2 (32-token chunks, built with -DLINATTN_WALK_TILES_BF16=2).  The 32-token
// walk fits in 256 registers, so two waves share a SIMD; it was measured
// slower on MI355X (the walk is bound by memory traffic either way, and
// smaller chunks add per-chunk work), so 64 is the product default.
#ifndef LINATTN_WALK_TILES_BF16
#define LINATTN_WALK_TILES_BF16 4
#endif
constexpr int kWalkTilesBf16 = LINATTN_WALK_TILES_BF16;
static_assert(kWalkTilesBf16 == 2 || kWalkTilesBf16 == 4, "the bf16 walk takes 32- or 64-token chunks");
// LINATTN_WALK_RING=1 (with 32-token chunks): one wave per SIMD and a ring of
// three 12 KB slots, so that the next chunk's loads go out at the top of each
// chunk and two chunks are always in flight.
#ifndef LINATTN_WALK_RING
#define LINATTN_WALK_RING 0
#endif
constexpr bool kWalkRing = LINATTN_WALK_RING != 0;
static_assert(!kWalkRing || kWalkTilesBf16 == 2, "the ring walk takes 32-token chunks");
constexpr int kWalkWavesPerSimd = kWalkTilesBf16 == 2 && !kWalkRing ? 2 : 1;

template <class E, bool kSave = false>
__device__ inline void causal_walk(const FwdParams &p) {
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
  auto init_state = [&]() {
    if (p.init == kInitRecord) {
      state_load_record(st, p.ws + ((long long)h * p.records + s) * kStateFloats, lane, g);
    } else if (p.init == kInitNatural || (p.init == kInitTotals && p.S0 != nullptr)) {
      state_load_natural(st, p.S0 + (long long)h * 4096, p.z0 + (long long)h * 64, n16, g);
    } else {
      state_zero(st);
    }
    if (p.init == kInitTotals)
      state_add_records(st, p.ws + (long long)h * p.records * kStateFloats, s, kStateFloats, lane, g);
    // The state's loads land before the chunk loop (the first chunk waits
    // for everything outstanding anyway).  Left in flight, they would make
    // the compiler wait for all outstanding memory operations, the previous
    // chunk's output stores among them, at the state's first use on every
    // chunk.
    wait_vmcnt<0>();
  };

  if constexpr (std::is_same<E, __bf16>::value && kWalkRing) {
    constexpr int NT = kWalkTilesBf16;
    constexpr int kT = 16 * NT;
    constexpr int kRing = 3;
    // Per chunk: Slot::kLoads counted loads; per full chunk 2 NT output
    // stores and, when saving, NT 1/den stores.
    constexpr int kLoads = Slot<3, NT>::kLoads;
    constexpr int kStores = 2 * NT + (kSave ? NT : 0);
    __shared__ u32x4 ring[kRing][Slot<3, NT>::kVec];
    const __bf16 *src[3] = {Qh, Kh, Vh};
    float *rdh = kSave ? p.rden + (long long)h * p.rden_stride : nullptr;
    const int n = (int)((t_end - t_begin + kT - 1) / kT);
    auto issue = [&](int c) {
      const long long t0 = t_begin + (long long)c * kT;
      stage_issue_counted<3, NT>(ring[c % kRing], src, t0, (int)min<long long>(kT, t_end - t0), n16, g);
    };
    if (n > 0) issue(0);
    if (n > 1) issue(1);
    init_state();  // also waits for chunks 0 and 1
    for (int c = 0; c < n; ++c) {
      // Slot (c + 2) % 3 held chunk c - 1, read out (and waited for) in the
      // previous iteration.
      if (c + 2 < n) issue(c + 2);
      // Chunk c's loads were followed by those of the later chunks issued so
      // far (up to two) and by the stores of the chunks computed since (up to
      // two, all full); everything retires in order.
      wait_ring<kLoads, kStores>(min(2, n - 1 - c), min(c, 2));
      const long long t0 = t_begin + (long long)c * kT;
      const int rows = (int)min<long long>(kT, t_end - t0);
      if (rows == kT) {
        causal_chunk_ring<NT, true, kSave>(st, ring[c % kRing], t0, rows, Oh, lane, n16, g, ident, rdh);
      } else {
        causal_chunk_ring<NT, false, kSave>(st, ring[c % kRing], t0, rows, Oh, lane, n16, g, ident, rdh);
      }
    }
  } else if constexpr (std::is_same<E, __bf16>::value) {
    constexpr int NT = kWalkTilesBf16;
    constexpr int kT = 16 * NT;
    __shared__ u32x4 slot[Slot<3, NT>::kVec];
    const __bf16 *src[3] = {Qh, Kh, Vh};
    float *rdh = kSave ? p.rden + (long long)h * p.rden_stride : nullptr;
    // The first chunk's loads go out before the state's, so that their
    // latencies overlap.
    if (t_begin < t_end) stage_issue<3, NT>(slot, src, t_begin, (int)min<long long>(kT, t_end - t_begin), n16, g);
    init_state();
    for (long long t0 = t_begin; t0 < t_end; t0 += kT) {
      const int rows = (int)min<long long>(kT, t_end - t0);
      // Outstanding vector-memory operations: this chunk's loads, then the
      // previous chunk's 2*NT output stores (full chunk), and its NT 1/den
      // stores when saving.  They retire in order, so waiting down to that
      // count leaves only stores in flight.
      if (t0 == t_begin) {
        wait_vmcnt<0>();
      } else {
        wait_vmcnt<2 * NT + (kSave ? NT : 0)>();
      }
      if (rows == kT) {
        causal_chunk_lds<NT, true, kSave>(st, slot, src, t0, t_end, rows, Oh, lane, n16, g, ident, rdh);
      } else {
        causal_chunk_lds<NT, false, kSave>(st, slot, src, t0, t_end, rows, Oh, lane, n16, g, ident, rdh);
      }
    }
  } else {
    // fp32: 32-token chunks staged in LDS; the next chunk's loads are in
    // flight while this one is computed.
    constexpr int NT = kWalkTilesF32;
    constexpr int kT = 16 * NT;
    constexpr int kStores = 4 * NT;  // output stores of a full chunk
    __shared__ u32x4 slot[3 * 16 * NT * 16];
    const float *src[3] = {Qh, Kh, Vh};
    if (t_begin < t_end) stage_issue_f32<3, NT>(slot, src, t_begin, (int)min<long long>(kT, t_end - t_begin), lane);
    init_state();
    for (long long t0 = t_begin; t0 < t_end; t0 += kT) {
      const int rows = (int)min<long long>(kT, t_end - t0);
      // Outstanding: this chunk's loads, then the previous (full) chunk's
      // stores; they retire in order.
      if (t0 == t_begin) {
        wait_vmcnt<0>();
      } else {
        wait_vmcnt<kStores>();
      }
      Slab<float> d[3][NT];
#pragma unroll
      for (int it = 0; it < NT; ++it)
#pragma unroll
        for (int tsr = 0; tsr < 3; ++tsr) slab_from_lds_f32<NT>(d[tsr][it], slot, tsr, it, rows, n16, g);
      wait_lgkmcnt0();  // the slot is refilled only after every lane's read of it returned
      if (t0 + kT < t_end) stage_issue_f32<3, NT>(slot, src, t0 + kT, (int)min<long long>(kT, t_end - t0 - kT), lane);
      Frag<E> qf[NT][4], kf[NT][4], vf[NT][4], kt[NT][4], vt[NT][4];
#pragma unroll
      for (int it = 0; it < NT; ++it) {
        slab_to_frags<E>(d[0][it], qf[it], false);
        phi_q_tile<E>(qf[it]);
        slab_to_frags<E>(d[1][it], kf[it], true);
        if (16 * it + n16 >= rows)
#pragma unroll
          for (int c = 0; c < 4; ++c) kf[it][c] = frag_zero<E>();
        slab_to_frags<E>(d[2][it], vf[it], false);
      }
      row_to_tok<E, NT>(kf, kt, ident);
      row_to_tok<E, NT>(vf, vt, ident);
      causal_chunk<E, NT, false>(st, qf, kf, kt, vt, rows, Oh, t0, n16, g);
    }
  }
  if (p.S_out != nullptr && s == p.segments - 1)
    state_store_natural(st, p.S_out + (long long)h * 4096, p.z_out + (long long)h * 64, n16, g);
}

// One wave per SIMD: the walk keeps the state, one chunk's fragments and the
// products' accumulators in registers (about 480 of the 512).  With 32-token
// chunks it is held to 256 registers, two waves per SIMD.
__global__ __launch_bounds__(64, kWalkWavesPerSimd) void causal_walk_kernel_bf16(FwdParams p) {
  causal_walk<__bf16>(p);
}
// The same walk, also saving 1/den per token for the saved-forward backward.
__global__ __launch_bounds__(64, kWalkWavesPerSimd) void causal_walk_save_kernel_bf16(FwdParams p) {
  causal_walk<__bf16, true>(p);
}
__global__ __launch_bounds__(64, 1) void causal_walk_kernel_f32(FwdParams p) { causal_walk<float>(p); }
template <class E> struct WalkKernel;
template <> struct WalkKernel<__bf16> { static constexpr auto fn = causal_walk_kernel_bf16; };
template <> struct WalkKernel<float> { static constexpr auto fn = causal_walk_kernel_f32; };

// ---------------------------------------------------------------------------
// Non-causal pass 2: o_i = phi(q_i)^T S / phi(q_i)^T z with the head's total
// S, z -- "Why Replace Attention?", §6.2 -- in workgroups of kGroupWaves
// waves of one head, one range of chunks per wave.  The workgroup first sums
// the head's `groups` records (in record order; the first workgroup of each
// head also stores that total as record `groups`, for a backward that reuses
// it), each wave's first chunk of Q already on its way.
// ---------------------------------------------------------------------------
template <class E> struct ReadSlot;
template <> struct ReadSlot<__bf16> { static constexpr int kVec = Slot<1>::kVec; };
template <> struct ReadSlot<float> { static constexpr int kVec = 16 * 4 * 16; };

// tot = sum of the head's `groups` records, added in record order (16-byte
// vectors split over the workgroup's threads, at most kSumVecs each).  The
// loads do not depend on the running sums, so each thread issues those of
// kSumBatch records for all its vectors at once: a record sum costs one load
// round trip per kSumBatch records rather than one per record and vector.
constexpr int kSumThreads = 64 * kGroupWaves;
constexpr int kSumVecs = (kStateVecs + kSumThreads - 1) / kSumThreads;
constexpr int kSumBatch = 4;
__device__ inline void sum_group_records(u32x4 *tot, const FwdParams &p, int h, int groups, bool store_total) {
  const f32x4 *recs = reinterpret_cast<const f32x4 *>(p.ws + (long long)h * p.records * kStateFloats);
  f32x4 *total = reinterpret_cast<f32x4 *>(p.ws + ((long long)h * p.records + groups) * kStateFloats);
  f32x4 acc[kSumVecs];
#pragma unroll
  for (int i = 0; i < kSumVecs; ++i) {
    const int v = threadIdx.x + i * kSumThreads;
    acc[i] = v < kStateVecs ? recs[v] : zero4();
  }
  for (int j0 = 1; j0 < groups; j0 += kSumBatch) {
    f32x4 r[kSumBatch][kSumVecs];
#pragma unroll
    for (int b = 0; b < kSumBatch; ++b)
#pragma unroll
      for (int i = 0; i < kSumVecs; ++i) {
        const int v = threadIdx.x + i * kSumThreads;
        r[b][i] = j0 + b < groups && v < kStateVecs ? recs[(long long)(j0 + b) * kStateVecs + v] : zero4();
      }
#pragma unroll
    for (int b = 0; b < kSumBatch; ++b)
      if (j0 + b < groups)
#pragma unroll
        for (int i = 0; i < kSumVecs; ++i) acc[i] += r[b][i];
  }
#pragma unroll
  for (int i = 0; i < kSumVecs; ++i) {
    const int v = threadIdx.x + i * kSumThreads;
    if (v < kStateVecs) {
      tot[v] = __builtin_bit_cast(u32x4, acc[i]);
      if (store_total) total[v] = acc[i];
    }
  }
}

template <class E>
__global__ __launch_bounds__(64 * kGroupWaves, 1) void noncausal_read_kernel(FwdParams p, int groups, int ranges,
                                                                              int range_chunks) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n16 = lane & 15, g = lane >> 4;
  const int h = blockIdx.x % p.heads;
  const int rg = blockIdx.x / p.heads;
  const int s = rg * kGroupWaves + wave;
  const long long base = (long long)h * p.N * kD;
  const E *Qh = reinterpret_cast<const E *>(p.Q) + base;
  E *Oh = reinterpret_cast<E *>(p.O) + base;
  long long t_begin = (long long)s * range_chunks * kChunk;
  long long t_end = t_begin + (long long)range_chunks * kChunk;
  if (t_end > p.N) t_end = p.N;
  if (s >= ranges) t_begin = t_end = 0;  // no range: takes part in the sum only

  __shared__ u32x4 slots[kGroupWaves][ReadSlot<E>::kVec];
  __shared__ u32x4 tot[kStateVecs];
  u32x4 *slot = slots[wave];
  if constexpr (std::is_same<E, __bf16>::value) {
    const __bf16 *src[1] = {Qh};
    if (t_begin < t_end) stage_issue<1>(slot, src, t_begin, chunk_rows(t_begin, t_end), n16, g);
  } else {
    const float *src[1] = {Qh};
    if (t_begin < t_end) stage_issue_f32<1, 4>(slot, src, t_begin, chunk_rows(t_begin, t_end), lane);
  }
  sum_group_records(tot, p, h, groups, rg == 0);
  __syncthreads();
  if (t_begin >= t_end) return;

  State st;
  state_load_record(st, reinterpret_cast<const float *>(tot), lane, g);
  StateOperands<E> so;
  state_operands<E>(st, so);
  if constexpr (std::is_same<E, __bf16>::value) {
    const __bf16 *src[1] = {Qh};
    for (long long t0 = t_begin; t0 < t_end; t0 += kChunk) {
      const int rows = chunk_rows(t0, t_end);
      if (t0 == t_begin) {  // see stream_lds
        wait_vmcnt<0>();
      } else {
        wait_vmcnt<8>();
      }
      // Untracked reads: a compiler-visible LDS read here would also wait for
      // the previous chunk's output stores, a full store round trip per chunk.
      Frag<E> qf[4][4];
#pragma unroll
      for (int it = 0; it < 4; ++it) lds_row_frags_untracked(slot, 0, it, lane, qf[it]);
      lds_reads_done();  // the slot is refilled only after every lane's read of it returned
      after_lds_reads<16>(&qf[0][0]);
      if (t0 + kChunk < t_end) stage_issue<1>(slot, src, t0 + kChunk, chunk_rows(t0 + kChunk, t_end), n16, g);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        phi_q_tile<E>(qf[it]);
        f32x4 nt[4] = {zero4(), zero4(), zero4(), zero4()};
        f32x4 dt = zero4();
        state_read<E>(so, qf[it], nt, dt);
        store_rows<E>(Oh, t0 + 16 * it, rows - 16 * it, nt, dt, n16, g);
      }
    }
  } else {
    // fp32: Q of a 64-token chunk (16 KB) staged in LDS, the next chunk's
    // loads in flight while this one is computed.
    constexpr int NT = 4;
    constexpr int kStores = 4 * NT;  // output stores of a full chunk
    const float *src[1] = {Qh};
    for (long long t0 = t_begin; t0 < t_end; t0 += kChunk) {
      const int rows = chunk_rows(t0, t_end);
      if (t0 == t_begin) {  // see stream_lds
        wait_vmcnt<0>();
      } else {
        wait_vmcnt<kStores>();
      }
      Slab<float> d[NT];
#pragma unroll
      for (int it = 0; it < NT; ++it) slab_from_lds_f32<NT>(d[it], slot, 0, it, rows, n16, g);
      wait_lgkmcnt0();
      if (t0 + kChunk < t_end) stage_issue_f32<1, NT>(slot, src, t0 + kChunk, chunk_rows(t0 + kChunk, t_end), lane);
#pragma unroll
      for (int it = 0; it < NT; ++it) {
        Frag<E> qf[4];
        slab_to_frags<E>(d[it], qf, false);
        phi_q_tile<E>(qf);
        f32x4 nt[4] = {zero4(), zero4(), zero4(), zero4()};
        f32x4 dt = zero4();
        state_read<E>(so, qf, nt, dt);
        store_rows<E>(Oh, t0 + 16 * it, rows - 16 * it, nt, dt, n16, g);
      }
    }
  }
}

}  // namespace linattn
