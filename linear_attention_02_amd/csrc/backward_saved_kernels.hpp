// backward_saved_kernels.hpp -- the causal bf16 backward after a forward that
// saved 1/den_i, in one left-to-right pass over Q, K, V and dO.
//
// The gradients are those of backward_kernels.hpp ("[Paper Review]
// Transformers are RNNs", §3.5 "Gradient Computation": forward and reverse
// cumulative sums).  With the forward's output O and its saved 1/den_i, the
// per-token factors a_i = g_i / den_i and b_i = -(g_i . o_i) / den_i need no
// state, so the reverse sums can be formed before any walk:
//
//   1. saved totals: per reverse segment u (the forward's segments, a
//      one-segment plan split in two), T_u = sum_i (phi(q_i)/den_i)^T g_i and
//      t_u = sum_i phi(q_i) b_i over its tokens, plus the pairs
//      (1/den_i, b_i) for every token, from Q, dO, O and 1/den;
//   2. the suffix scan of those records: R, r exactly at every reverse
//      segment start (an anchor);
//   3. one walk per group of forward segments, left to right, in which three
//      waves share every staged chunk: one writes dQ from the prefix state
//      S, z (as the existing left-to-right walk), one dK and one dV from the
//      suffix state R, r.  The suffix state is taken exact at each anchor and
//      carried to the next by subtraction: each chunk's own terms are
//      subtracted before they are used.  The subtracted terms are built from
//      the same rounded operands as the totals (phi(q_i) rounded once to
//      bf16, then times 1/den_i rounded once; b_i rounded once; g_i exact),
//      so they cancel up to fp32 summation order: what remains at a token is
//      a few 2^-24 of the largest sum since its anchor.  Because 1/den_i
//      falls off like 1/i, the last anchor must not lie near the sequence
//      start (the planner's rule), or the tail's small true suffix would
//      drown in the rounding of the early tokens' large terms.
//
// A fourth wave of the workgroup moves and prepares data: it holds the next
// kLoaderDepth chunks of Q, K, V, dO and the pairs in registers (plain vector
// loads, so the compiler counts their waits), and for each chunk writes
// phi(Q), phi(K), V, dO and the pairs into one of two LDS slots, then meets
// the compute waves at one barrier per chunk.  phi is thus evaluated once per
// element instead of once per wave that reads it, and phi'(x) = min(phi(x), 1)
// (x + 1 > 1 for x > 0, e^x <= 1 otherwise) needs no second exponential.
// Every state is accumulated in the orientation its products read, so no
// wave transposes a state:
//   dQ wave: S^T tiles [mt][ct] (S as the A operand of S g^T);
//   dK wave: R^T tiles [mt][ct] (R as the A operand of R V^T), and r;
//   dV wave: R tiles [ct][mt] (R^T as the A operand of R^T phi(K)^T).
#pragma once

#include "backward_kernels.hpp"

namespace linattn {

// ---------------------------------------------------------------------------
// Transposed state records.  A record stores S tile (ct, mt) lane (n, g)
// register r = S[pi(ct,g,r)][pi(mt,n>>2,n&3)] (forward_kernels.hpp).  The
// transposed tile (mt, ct) holds, in lane (n, g) register r,
// S[pi(ct,n>>2,n&3)][pi(mt,g,r)]: the record's lane 16 (n>>2) + 4 g + r,
// register n & 3.  z is loaded as in state_load_record.
// ---------------------------------------------------------------------------
__device__ inline void state_load_record_t(State &st, const float *rec, int n16, int g) {
  const int lane_base = 16 * (n16 >> 2) + 4 * g;
  const int reg = n16 & 3;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) st.S[mt][ct][r] = rec[((ct * 4 + mt) * 64 + lane_base + r) * 4 + reg];
  const f32x4 *p = reinterpret_cast<const f32x4 *>(rec);
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) st.z[ct] = p[1024 + ct * 4 + g];
}

// st += records first, first + stride, ... (count of them, in that order),
// each loaded transposed.
__device__ inline void state_add_records_t(State &st, const float *first, int count, long long stride, int n16,
                                           int g) {
  for (int j = 0; j < count; ++j) {
    State a;
    state_load_record_t(a, first + j * stride, n16, g);
    state_add(st, a);
  }
}

// ---------------------------------------------------------------------------
// The rounded query operands shared by the saved totals and the walk.  From
// a token-layout fragment of phi(Q) (already rounded to bf16) and the
// tokens' 1/den (0 for tokens past the end): qp = phi(q) and
// qs = phi(q) * (sign / den) rounded once.  Tokens with 1/den = 0 give zero
// operands whatever their slot holds.  With sign = -1 the result is exactly
// the negation of sign = +1's (rounding to nearest even is symmetric), which
// is what lets the walk subtract exactly the terms the totals added.
// ---------------------------------------------------------------------------
__device__ inline void saved_q_operands(const Frag<__bf16> &phiq, f32x4 rd, float sign, Frag<__bf16> &qp,
                                        Frag<__bf16> &qs) {
  f32x4 x = frag_f32(phiq);
#pragma unroll
  for (int r = 0; r < 4; ++r) x[r] = rd[r] != 0.f ? x[r] : 0.f;
  qp = to_frag<__bf16>(x);
  qs = to_frag<__bf16>(x * (rd * sign));
}

// phi of the eight bf16 values in a 16-byte piece, rounded back to bf16.
__device__ inline u32x4 phi_piece(u32x4 v) {
  u32x4 o;
#pragma unroll
  for (int w = 0; w < 4; ++w) o[w] = pack_bf16(phi(bf16_lo(v[w])), phi(bf16_hi(v[w])));
  return o;
}

// phi'(x) = min(e^x, 1) from phi(x) itself.
__device__ inline float phi_prime_of_phi(float f) { return fminf(f, 1.f); }

// Row tiles per chunk of the saved-forward walk (32-token chunks) and chunks
// the loader holds in registers ahead of the one being computed.
constexpr int kSavedTiles = 2;
constexpr int kLoaderDepth = 3;
constexpr int kSavedSlotVec = Slot<4, kSavedTiles>::kVec + 8 * kSavedTiles;  // phi(Q), phi(K), V, dO, pairs
static_assert(kSavedTiles == 2, "the chunk bodies pair the two row tiles in their state updates");

// ---------------------------------------------------------------------------
// 1. Saved totals: one wave per reverse segment u of a head.  Writes the
//    pairs (1/den_i, b_i) of its tokens (padding tokens up to the chunk end
//    get zeros) and the record u + 1 of (T_u, t_u), in the State layout.
//    The forward saved 1/den for each query row as its walk scaled it; the
//    row's exponent is recovered here from q_i with the same rule.
// ---------------------------------------------------------------------------
template <int kPolicy> __device__ inline void bwd_saved_totals(const BwdParams &p) {
  typedef __bf16 E;
  constexpr int NT = 4;
  const int worker = blockIdx.x;
  const int h = worker % p.heads;
  const int u = worker / p.heads;
  if (u >= p.rev_segments) return;
  const int lane = threadIdx.x;
  const int n16 = lane & 15, g = lane >> 4;
  const long long base = (long long)h * p.N * kD;
  const E *Qh = reinterpret_cast<const E *>(p.Q) + base;
  const E *Gh = reinterpret_cast<const E *>(p.dO) + base;
  const E *Oh = reinterpret_cast<const E *>(p.O) + base;
  const float *rdh = p.rden + (long long)h * p.stats_stride;
  f32x2 *pairs_h = p.stats + (long long)h * p.stats_stride;
  const long long t_begin = (long long)u * p.rev_chunks * kChunk;
  long long t_end = t_begin + (long long)p.rev_chunks * kChunk;
  if (t_end > p.N) t_end = p.N;
  State acc;
  state_zero(acc);
  __shared__ u32x4 slot[Slot<3, NT>::kVec + 16];
  u32x4 *rreg = slot + Slot<3, NT>::kVec;  // the chunk's 64 saved 1/den
  const __bf16 *src[3] = {Qh, Gh, Oh};
  auto issue = [&](long long t0) {
    const int rows = chunk_rows(t0, t_end);
    stage_issue<3, NT, kPolicy>(slot, src, t0, rows, n16, g);
    if (lane < 16 && 4 * lane < rows)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const u32x4 *>(rdh + t0) + lane, (lds_void *)rreg, 16, 0,
                                       kPolicy);
  };
  if (t_begin < t_end) issue(t_begin);
  for (long long t0 = t_begin; t0 < t_end; t0 += kChunk) {
    const int rows = chunk_rows(t0, t_end);
    // Outstanding: this chunk's loads, then the previous chunk's pair store.
    if (t0 == t_begin) {
      wait_vmcnt<0>();
    } else {
      wait_vmcnt<1>();
    }
    Frag<E> qt[NT][4], gt[NT][4], qr[NT][4], gr[NT][4], orow[NT][4];
    float rd_row[NT];
#pragma unroll
    for (int it = 0; it < NT; ++it) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        qt[it][c] = lds_tok_frag<NT>(slot, 0, it, c, lane);
        gt[it][c] = lds_tok_frag<NT>(slot, 1, it, c, lane);
      }
      lds_row_frags<NT>(slot, 0, it, lane, qr[it]);
      lds_row_frags<NT>(slot, 1, it, lane, gr[it]);
      lds_row_frags<NT>(slot, 2, it, lane, orow[it]);
      rd_row[it] = reinterpret_cast<const float *>(rreg)[16 * it + n16];
    }
    wait_lgkmcnt0();
    if (t0 + kChunk < t_end) issue(t0 + kChunk);
    if (rows < kChunk) zero_tokens<E, NT>(gt, rows, g);
    // Token 16 it + n: its true 1/den (0 past the end) and
    // b = -(g . o) / den; lane (n, g) holds 16 of the token's columns.
    float b_row[NT];
#pragma unroll
    for (int it = 0; it < NT; ++it) {
      float m = raw_elem(qr[it][0], 0), go = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4 ga = frag_f32(gr[it][c]), oa = frag_f32(orow[it][c]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          m = fmaxf(m, raw_elem(qr[it][c], r));
          go += ga[r] * oa[r];
        }
      }
      m = fmaxf(m, __shfl_xor(m, 16, 64));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      go += __shfl_xor(go, 16, 64);
      go += __shfl_xor(go, 32, 64);
      float eneg;
      int epos;
      phi_row_scale(m, eneg, epos);
      const bool valid = 16 * it + n16 < rows;
      rd_row[it] = valid ? ldexpf(rd_row[it], -((int)eneg + epos)) : 0.f;
      b_row[it] = valid ? -go * rd_row[it] : 0.f;
    }
    // Pairs of tokens 16 g + n: one store for the chunk.
    float keep_rd = 0.f, keep_b = 0.f;
#pragma unroll
    for (int it = 0; it < NT; ++it)
      if (g == it) {
        keep_rd = rd_row[it];
        keep_b = b_row[it];
      }
    pairs_h[t0 + 16 * g + n16] = f32x2{keep_rd, keep_b};
    // Sums: T += (phi(Q)/den)^T G, t += phi(Q)^T b (token layout operands).
#pragma unroll
    for (int it = 0; it < NT; ++it) {
      f32x4 rdt, bt;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        rdt[r] = __shfl(rd_row[it], 4 * g + r, 64);
        bt[r] = __shfl(b_row[it], 4 * g + r, 64);
      }
      const Frag<E> bf = to_frag<E>(bt);
      Frag<E> qp[4], qs[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        Frag<E> phiq = qt[it][c];
        phi_frag<E>(phiq);
        saved_q_operands(phiq, rdt, 1.f, qp[c], qs[c]);
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc.S[ct][mt] = mac1<E>(acc.S[ct][mt], qs[ct], gt[it][mt]);
        acc.z[ct] = mac1<E>(acc.z[ct], qp[ct], bf);
      }
    }
  }
  state_store_record(acc, p.wsT + ((long long)h * p.recT + u + 1) * kStateFloats, lane, n16, g);
}

template <int kPolicy> __global__ __launch_bounds__(64, 1) void bwd_saved_totals_kernel(BwdParams p) {
  bwd_saved_totals<kPolicy>(p);
}

// ---------------------------------------------------------------------------
// 3. The walk.  Workgroup (h, s) covers walk segment s: forward segments
//    s k .. s k + k - 1 (k = p.walk_k).  Waves: 0 loader, 1 dQ, 2 dK, 3 dV.
// ---------------------------------------------------------------------------
// Every wave finishes its LDS accesses of the previous chunk before the
// barrier; the loader writes a slot only after the barrier that follows the
// compute waves' last read of it.
__device__ inline void saved_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

struct SavedSeg {
  long long t_begin, t_end;
  int chunks;  // 32-token chunks
};

__device__ inline SavedSeg saved_segment(const BwdParams &p, int s) {
  constexpr long long kT = 16 * kSavedTiles;
  SavedSeg sg;
  sg.t_begin = (long long)s * p.walk_k * p.seg_chunks * kChunk;
  sg.t_end = sg.t_begin + (long long)p.walk_k * p.seg_chunks * kChunk;
  if (sg.t_end > p.N) sg.t_end = p.N;
  sg.chunks = sg.t_begin < sg.t_end ? (int)((sg.t_end - sg.t_begin + kT - 1) / kT) : 0;
  return sg;
}

// One chunk in the loader's registers: lane l holds 16-byte piece (l & 7) of
// rows 8 i + (l >> 3) of Q, K, V and dO, and the pairs of tokens
// 2 (l & 15), 2 (l & 15) + 1.  Every load is issued unconditionally (rows
// past the end repeat the last row; the compute waves mask them), so the
// compiler's wait counts see a fixed 4 * 2 NT + 1 loads per chunk and can
// leave the later chunks in flight.
struct LoaderChunk {
  u32x4 v[4][2 * kSavedTiles];
  u32x4 pr;
};
constexpr int kLoaderLoads = 4 * 2 * kSavedTiles + 1;

__device__ inline void loader_fetch(LoaderChunk &L, const __bf16 *const src[4], const f32x2 *pairs_h, long long t0,
                                    int rows, int lane) {
  const int sub = lane >> 3, piece = lane & 7;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 2 * kSavedTiles; ++i) {
      const int row = min(8 * i + sub, rows - 1);
      L.v[t][i] = reinterpret_cast<const u32x4 *>(src[t] + (t0 + row) * kD)[piece];
    }
  // The pairs array holds every token of the chunk (padding tokens as zeros).
  L.pr = reinterpret_cast<const u32x4 *>(pairs_h + t0)[lane & 15];
}

// Writes a fetched chunk into a slot in the staging layout (stage_index):
// phi applied to Q and K.
__device__ inline void loader_store(const LoaderChunk &L, u32x4 *slot, int lane) {
  const int sub = lane >> 3, piece = lane & 7;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 2 * kSavedTiles; ++i)
      slot[(t * 2 * kSavedTiles + i) * 64 + 8 * sub + (piece ^ sub)] = t < 2 ? phi_piece(L.v[t][i]) : L.v[t][i];
  if (lane < 8 * kSavedTiles) slot[Slot<4, kSavedTiles>::kVec + lane] = L.pr;
}

__device__ inline void saved_loader(const BwdParams &p, u32x4 (*ring)[kSavedSlotVec], int h, const SavedSeg &sg,
                                    int lane) {
  constexpr int kT = 16 * kSavedTiles;
  const long long base = (long long)h * p.N * kD;
  const __bf16 *src[4] = {reinterpret_cast<const __bf16 *>(p.Q) + base, reinterpret_cast<const __bf16 *>(p.K) + base,
                          reinterpret_cast<const __bf16 *>(p.V) + base, reinterpret_cast<const __bf16 *>(p.dO) + base};
  const f32x2 *pairs_h = p.stats + (long long)h * p.stats_stride;
  // Chunks past the last one fetch the last one again (unused), keeping
  // every step's loads unconditional.
  auto fetch = [&](LoaderChunk &L, int c) {
    const long long t0 = sg.t_begin + (long long)min(c, sg.chunks - 1) * kT;
    loader_fetch(L, src, pairs_h, t0, (int)min<long long>(kT, sg.t_end - t0), lane);
  };
  // Chunk c: write it into slot c & 1 (its previous contents, chunk c - 2,
  // were last read before the barrier of chunk c - 1), refill the registers
  // with chunk c + kLoaderDepth, then the barrier that releases chunk c.
  auto step = [&](LoaderChunk &L, int c) {
    loader_store(L, ring[c & 1], lane);
    fetch(L, c + kLoaderDepth);
    saved_barrier();
  };
  static_assert(kLoaderDepth == 3, "the loop below holds three chunks");
  LoaderChunk L0, L1, L2;
  fetch(L0, 0);
  fetch(L1, 1);
  fetch(L2, 2);
  // Whole groups of three in a loop with one back edge (so the compiler's
  // wait counts carry over it), then the remaining one or two chunks.
  int c0 = 0;
  for (; c0 + 3 <= sg.chunks; c0 += 3) {
    step(L0, c0);
    step(L1, c0 + 1);
    step(L2, c0 + 2);
  }
  if (c0 < sg.chunks) step(L0, c0);
  if (c0 + 1 < sg.chunks) step(L1, c0 + 1);
}

// Lane (n, g) of a walk wave: 1/den and b of tokens 16 it + 4 g + r (token
// layout), tokens past the end zero.
template <bool kFull>
__device__ inline void saved_stats_tok(const u32x4 *sreg, int rows, int g, f32x4 rdt[kSavedTiles],
                                       f32x4 bt[kSavedTiles]) {
#pragma unroll
  for (int it = 0; it < kSavedTiles; ++it) {
    stats_tok(sreg, it, g, rdt[it], bt[it]);
    if (!kFull)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (16 * it + 4 * g + r >= rows) {
          rdt[it][r] = 0.f;
          bt[it][r] = 0.f;
        }
  }
}

// Slot tensors of the walk.
constexpr int kPhiQ = 0, kPhiK = 1, kVals = 2, kGrad = 3;

// dQ wave, one chunk: dphi(Q)^T = phi(K)^T D^T + (S G^T) / den + z b^T, then
// S^T += V^T phi(K), z += column sums of phi(K).
template <bool kFull>
__device__ inline void saved_dq_chunk(State &st, const u32x4 *slot, long long t0, int rows, __bf16 *dQh, int lane) {
  typedef __bf16 E;
  constexpr int NT = kSavedTiles;
  const int n16 = lane & 15, g = lane >> 4;
  const u32x4 *sreg = slot + Slot<4, NT>::kVec;
  Frag<E> qphi[NT][4], vf[NT][4], gf[NT][4], kt[NT][4], vt[NT][4];
  f32x2 sr[NT];
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    lds_row_frags<NT>(slot, kPhiQ, it, lane, qphi[it]);
    lds_row_frags<NT>(slot, kVals, it, lane, vf[it]);
    lds_row_frags<NT>(slot, kGrad, it, lane, gf[it]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      kt[it][c] = lds_tok_frag<NT>(slot, kPhiK, it, c, lane);
      vt[it][c] = lds_tok_frag<NT>(slot, kVals, it, c, lane);
    }
    sr[it] = stats_row(sreg, it, n16);
  }
  if (!kFull) {
    zero_tokens<E, NT>(kt, rows, g);
    zero_tokens<E, NT>(vt, rows, g);
  }
  Frag<E> sf[4][4];  // S as the A operand (row = feature, k = value column)
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) sf[ct][mt] = to_frag<E>(st.S[mt][ct]);
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    const float rd = sr[it][0], b = sr[it][1];
    // D^T (key j, query i) = (v_j . g_i) / den_i + b_i for j <= i.
    Frag<E> df[NT];
#pragma unroll
    for (int jt = 0; jt <= it; ++jt) {
      f32x4 d = zero4();
      d = mac2<E>(d, vf[jt][0], vf[jt][1], gf[it][0], gf[it][1]);
      d = mac2<E>(d, vf[jt][2], vf[jt][3], gf[it][2], gf[it][3]);
      d = d * rd + b;
      if (jt == it)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * g + r > n16) d[r] = 0.f;
      df[jt] = to_frag<E>(d);
    }
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
      const f32x4 pq = frag_f32(qphi[it][ct]);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        dq[ct][r] = (dq[ct][r] + sg[ct][r] * rd + st.z[ct][r] * b) * phi_prime_of_phi(pq[r]);
    }
    store_tiles<E, kFull>(dQh, t0 + 16 * it, rows - 16 * it, dq, n16, g);
  }
  // S^T += V^T phi(K) (tile [mt][ct]), z += phi(K)^T 1.
  const Frag<E> ones = frag_ones<E>();
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) st.S[mt][ct] = mac2<E>(st.S[mt][ct], vt[0][mt], vt[1][mt], kt[0][ct], kt[1][ct]);
    st.z[ct] = mac2<E>(st.z[ct], kt[0][ct], kt[1][ct], ones, ones);
  }
}

// dK wave, one chunk: first R^T -= G^T (phi(Q)/den), r -= phi(Q)^T b (the
// chunk's own terms), then dphi(K)^T = R V^T + r 1^T + phi(Q)^T D.
template <bool kFull>
__device__ inline void saved_dk_chunk(State &st, const u32x4 *slot, long long t0, int rows, __bf16 *dKh, int lane) {
  typedef __bf16 E;
  constexpr int NT = kSavedTiles;
  const int n16 = lane & 15, g = lane >> 4;
  const u32x4 *sreg = slot + Slot<4, NT>::kVec;
  Frag<E> qphit[NT][4], gf[NT][4], vf[NT][4], kphi[NT][4], gt[NT][4];
  f32x4 rdt[NT], bt[NT];
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    lds_row_frags<NT>(slot, kPhiK, it, lane, kphi[it]);
    lds_row_frags<NT>(slot, kVals, it, lane, vf[it]);
    lds_row_frags<NT>(slot, kGrad, it, lane, gf[it]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      qphit[it][c] = lds_tok_frag<NT>(slot, kPhiQ, it, c, lane);
      gt[it][c] = lds_tok_frag<NT>(slot, kGrad, it, c, lane);
    }
  }
  saved_stats_tok<kFull>(sreg, rows, g, rdt, bt);
  if (!kFull) {
    zero_rows<E, NT>(gf, rows, n16);
    zero_tokens<E, NT>(gt, rows, g);
  }
  Frag<E> qt[NT][4], qsn[NT][4];
#pragma unroll
  for (int it = 0; it < NT; ++it)
#pragma unroll
    for (int c = 0; c < 4; ++c) saved_q_operands(qphit[it][c], rdt[it], -1.f, qt[it][c], qsn[it][c]);
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) st.S[mt][ct] = mac2<E>(st.S[mt][ct], gt[0][mt], gt[1][mt], qsn[0][ct], qsn[1][ct]);
    st.z[ct] = mac2<E>(st.z[ct], qt[0][ct], qt[1][ct], to_frag<E>(-bt[0]), to_frag<E>(-bt[1]));
  }
  Frag<E> rf[4][4];  // R as the A operand (row = feature, k = value column)
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) rf[ct][mt] = to_frag<E>(st.S[mt][ct]);
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) {
    // R V^T first: each accumulator chain runs its 16x16x32 products before
    // its 16x16x16 ones (device_common.hpp, mac1).
    f32x4 dk[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      dk[ct] = mac2<E>(zero4(), rf[ct][0], rf[ct][1], vf[jt][0], vf[jt][1]);
      dk[ct] = mac2<E>(dk[ct], rf[ct][2], rf[ct][3], vf[jt][2], vf[jt][3]);
    }
#pragma unroll
    for (int it = jt; it < NT; ++it) {
      // D (query i = 16 it + 4 g + r, key j = 16 jt + n) = (g_i . v_j) / den_i + b_i, i >= j.
      f32x4 d = zero4();
      d = mac2<E>(d, gf[it][0], gf[it][1], vf[jt][0], vf[jt][1]);
      d = mac2<E>(d, gf[it][2], gf[it][3], vf[jt][2], vf[jt][3]);
      d = d * rdt[it] + bt[it];
      if (it == jt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * g + r < n16) d[r] = 0.f;
      const Frag<E> dfr = to_frag<E>(d);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) dk[ct] = mac1<E>(dk[ct], qt[it][ct], dfr);
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const f32x4 pk = frag_f32(kphi[jt][ct]);
#pragma unroll
      for (int r = 0; r < 4; ++r) dk[ct][r] = (dk[ct][r] + st.z[ct][r]) * phi_prime_of_phi(pk[r]);
    }
    store_tiles<E, kFull>(dKh, t0 + 16 * jt, rows - 16 * jt, dk, n16, g);
  }
}

// dV wave, one chunk: first R -= (phi(Q)/den)^T G, then
// dV^T = R^T phi(K)^T + G^T W' with W'_ij = phi(q_i) . phi(k_j) / den_i, i >= j.
template <bool kFull>
__device__ inline void saved_dv_chunk(State &st, const u32x4 *slot, long long t0, int rows, __bf16 *dVh, int lane) {
  typedef __bf16 E;
  constexpr int NT = kSavedTiles;
  const int n16 = lane & 15, g = lane >> 4;
  const u32x4 *sreg = slot + Slot<4, NT>::kVec;
  Frag<E> qf[NT][4], kf[NT][4], qphit[NT][4], gt[NT][4];
  f32x4 rdt[NT], bt[NT];
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    lds_row_frags<NT>(slot, kPhiQ, it, lane, qf[it]);
    lds_row_frags<NT>(slot, kPhiK, it, lane, kf[it]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      qphit[it][c] = lds_tok_frag<NT>(slot, kPhiQ, it, c, lane);
      gt[it][c] = lds_tok_frag<NT>(slot, kGrad, it, c, lane);
    }
  }
  saved_stats_tok<kFull>(sreg, rows, g, rdt, bt);
  if (!kFull) {
    zero_rows<E, NT>(qf, rows, n16);
    zero_tokens<E, NT>(gt, rows, g);
  }
  Frag<E> qsn[NT][4];
#pragma unroll
  for (int it = 0; it < NT; ++it)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      Frag<E> qp_unused;
      saved_q_operands(qphit[it][c], rdt[it], -1.f, qp_unused, qsn[it][c]);
    }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) st.S[ct][mt] = mac2<E>(st.S[ct][mt], qsn[0][ct], qsn[1][ct], gt[0][mt], gt[1][mt]);
  StateOperands<E> ro;  // R^T as the A operand (row = value column, k = feature)
  state_operands<E>(st, ro);
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) {
    // R^T phi(K)^T first, as in the dK wave.
    f32x4 dv[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      dv[mt] = mac2<E>(zero4(), ro.sa[0][mt], ro.sa[1][mt], kf[jt][0], kf[jt][1]);
      dv[mt] = mac2<E>(dv[mt], ro.sa[2][mt], ro.sa[3][mt], kf[jt][2], kf[jt][3]);
    }
#pragma unroll
    for (int it = jt; it < NT; ++it) {
      f32x4 w = zero4();
      w = mac2<E>(w, qf[it][0], qf[it][1], kf[jt][0], kf[jt][1]);
      w = mac2<E>(w, qf[it][2], qf[it][3], kf[jt][2], kf[jt][3]);
      w = w * rdt[it];
      if (it == jt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * g + r < n16) w[r] = 0.f;
      const Frag<E> wf = to_frag<E>(w);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) dv[mt] = mac1<E>(dv[mt], gt[it][mt], wf);
    }
    store_tiles<E, kFull>(dVh, t0 + 16 * jt, rows - 16 * jt, dv, n16, g);
  }
}

// The suffix state (R, r) from the start of reverse segment ur on: record ur
// after the suffix scan, or the sum of the totals records ur + 1 .. P, last
// first; transposed tiles for the dK wave.
__device__ inline void load_suffix(State &st, const BwdParams &p, int h, int ur, bool transposed, int lane, int n16,
                                   int g) {
  const float *recs = p.wsT + (long long)h * p.recT * kStateFloats;
  if (p.rev_sum_in_walk) {
    const float *last = recs + (long long)p.rev_segments * kStateFloats;
    const int count = p.rev_segments - ur;
    state_zero(st);
    if (transposed) {
      state_add_records_t(st, last, count, -(long long)kStateFloats, n16, g);
    } else {
      state_add_records(st, last, count, -(long long)kStateFloats, lane, g);
    }
  } else if (transposed) {
    state_load_record_t(st, recs + (long long)ur * kStateFloats, n16, g);
  } else {
    state_load_record(st, recs + (long long)ur * kStateFloats, lane, g);
  }
}

__global__ __launch_bounds__(256, 1) void bwd_saved_walk_kernel(BwdParams p) {
  constexpr int NT = kSavedTiles;
  constexpr int kT = 16 * NT;
  __shared__ u32x4 ring[2][kSavedSlotVec];
  const int worker = blockIdx.x;
  const int h = worker % p.heads;
  const int s = worker / p.heads;
  if (s >= p.walk_segments) return;
  const SavedSeg sg = saved_segment(p, s);
  if (sg.chunks == 0) return;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n16 = lane & 15, g = lane >> 4;
  if (wave == 0) {
    saved_loader(p, ring, h, sg, lane);
    return;
  }
  const long long base = (long long)h * p.N * kD;
  const int u0 = s * p.walk_k;  // first forward segment of this walk segment
  State st;
  if (wave == 1) {
    // Prefix (S, z) at the segment start, from the forward's records.
    state_zero(st);
    if (p.recF > 0) {
      if (p.sum_in_walk) {
        state_add_records_t(st, p.wsF + (long long)h * p.recF * kStateFloats, u0, kStateFloats, n16, g);
      } else {
        state_load_record_t(st, p.wsF + ((long long)h * p.recF + u0) * kStateFloats, n16, g);
      }
    }
  }
  // The suffix state starts exact at every reverse-segment start (walk
  // segments begin at one) and is carried by subtraction in between.
  const long long rev_tokens = (long long)p.rev_chunks * kChunk;
  if (wave != 1) load_suffix(st, p, h, (int)(sg.t_begin / rev_tokens), wave == 2, lane, n16, g);
  __bf16 *out = reinterpret_cast<__bf16 *>(wave == 1 ? p.dQ : wave == 2 ? p.dK : p.dV) + base;
  for (int c = 0; c < sg.chunks; ++c) {
    saved_barrier();
    const u32x4 *slot = ring[c & 1];
    const long long t0 = sg.t_begin + (long long)c * kT;
    const int rows = (int)min<long long>(kT, sg.t_end - t0);
    if (wave != 1 && c > 0 && t0 % rev_tokens == 0) load_suffix(st, p, h, (int)(t0 / rev_tokens), wave == 2, lane, n16, g);
    if (wave == 1) {
      if (rows == kT) {
        saved_dq_chunk<true>(st, slot, t0, rows, out, lane);
      } else {
        saved_dq_chunk<false>(st, slot, t0, rows, out, lane);
      }
    } else if (wave == 2) {
      if (rows == kT) {
        saved_dk_chunk<true>(st, slot, t0, rows, out, lane);
      } else {
        saved_dk_chunk<false>(st, slot, t0, rows, out, lane);
      }
    } else {
      if (rows == kT) {
        saved_dv_chunk<true>(st, slot, t0, rows, out, lane);
      } else {
        saved_dv_chunk<false>(st, slot, t0, rows, out, lane);
      }
    }
  }
}

}  // namespace linattn
