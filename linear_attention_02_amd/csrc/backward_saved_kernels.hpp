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

// phi'(x) = min(e^x, 1) from phi(x) >= 0 itself, as one clamp to [0, 1].
__device__ inline float phi_prime_of_phi(float f) { return __builtin_amdgcn_fmed3f(f, 0.f, 1.f); }

// Row tiles per chunk of the saved-forward walk (32-token chunks) and chunks
// the loader holds in registers ahead of the one being computed.
constexpr int kSavedTiles = 2;
constexpr int kLoaderDepth = 3;
// Slot of the walk: the tensors phi(Q), phi(K), V, dO and QSN = -phi(Q)/den
// (each rounded to bf16 as the saved totals round them), the pairs, the
// chunk's three D tiles in the dK waves' operand layout (written by the dQ
// waves, 64 lanes x 8 bytes each) and b by token in bf16 (written by loader
// 1, lane g's 16 bytes holding tokens 4 g .. 4 g + 3 of both row tiles).
constexpr int kPhiQ = 0, kPhiK = 1, kVals = 2, kGrad = 3, kQSN = 4, kSlotTensors = 5;
constexpr int kSavedPairsVec = Slot<kSlotTensors, kSavedTiles>::kVec;
constexpr int kSavedDVec = kSavedPairsVec + 8 * kSavedTiles;
constexpr int kSavedDTiles = kSavedTiles * (kSavedTiles + 1) / 2;
constexpr int kSavedBVec = kSavedDVec + 32 * kSavedDTiles;
constexpr int kSavedSlotVec = kSavedBVec + 4;
static_assert(kSavedTiles == 2, "the chunk bodies pair the two row tiles in their state updates");

// ---------------------------------------------------------------------------
// 1. Saved totals: one wave per reverse segment u of a head.  Writes the
//    pairs (1/den_i, b_i) of its tokens (padding tokens up to the chunk end
//    get zeros) and the record u + 1 of (T_u, t_u), in the State layout.
//    The forward saved 1/den for each query row as its walk scaled it; the
//    row's exponent is recovered here from q_i with the same rule.  (Measured
//    on the long-context workload, splitting a segment over 2 or 4 waves of
//    one workgroup whose partial sums meet in LDS was slower: 199 and 210 us
//    against 183 us.)
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
    // Outstanding: the previous chunk's pair store, then this chunk's loads
    // (issued after that store: the LDS reads below must wait for the loads,
    // and a store issued after them would be waited for as well).
    wait_vmcnt<0>();
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
    if (t0 + kChunk < t_end) issue(t0 + kChunk);
    // Sums: T += (phi(Q)/den)^T G, t += phi(Q)^T b (token layout operands),
    // two row tiles per product.
#pragma unroll
    for (int ip = 0; ip < NT / 2; ++ip) {
      Frag<E> bf[2], qp[2][4], qs[2][4];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int it = 2 * ip + x;
        f32x4 rdt, bt;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          rdt[r] = __shfl(rd_row[it], 4 * g + r, 64);
          bt[r] = __shfl(b_row[it], 4 * g + r, 64);
        }
        bf[x] = to_frag<E>(bt);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          Frag<E> phiq = qt[it][c];
          phi_frag<E>(phiq);
          saved_q_operands(phiq, rdt, 1.f, qp[x][c], qs[x][c]);
        }
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          acc.S[ct][mt] = mac2<E>(acc.S[ct][mt], qs[0][ct], qs[1][ct], gt[2 * ip][mt], gt[2 * ip + 1][mt]);
        acc.z[ct] = mac2<E>(acc.z[ct], qp[0][ct], qp[1][ct], bf[0], bf[1]);
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
//    s k .. s k + k - 1 (k = p.walk_k).  Eight waves, two per SIMD, two of
//    each role: loaders, dQ, dK and dV (the kernel maps waves to roles).  A
//    compute wave owns column half x of its output and of its state (the
//    other products are recomputed by both halves: the 16 x 16 D or W tiles
//    are cheap next to the state products); loader x moves half of the
//    tensors.
// ---------------------------------------------------------------------------
constexpr int kSavedWaves = 8;
// LDS slots in the ring: a loader fills chunk c + 2 while the compute waves
// read chunk c + 1 and compute chunk c.
constexpr int kSavedRing = 3;

// Every wave's LDS accesses issued before the barrier have completed when it
// passes it (the wait is also visible to the compiler's wait counting).  A
// loader writes a slot only after the barrier that follows the compute waves'
// last read of it.
__device__ inline void saved_barrier() {
  wait_lgkmcnt0();
  asm volatile("s_barrier" ::: "memory");
}

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

// One chunk of loader x's tensors in registers: tensor x (Q or K, phi is
// applied when it is stored) and tensor x + 2 (V or dO).  Lane l holds
// 16-byte piece (l & 7) of rows 8 i + (l >> 3); loader 0 also holds the pairs
// of those rows (for QS), loader 1 the pairs of tokens 2 (l & 15),
// 2 (l & 15) + 1.  Every load is issued
// unconditionally (rows past the end repeat the last row; the compute waves
// mask them), so the compiler's wait counts see a fixed number of loads per
// chunk and can leave the later chunks in flight.
struct LoaderChunk {
  u32x4 v[2][2 * kSavedTiles];
  u32x4 pr;
  f32x2 rowpr[2 * kSavedTiles];
};

template <int kHalf>
__device__ inline void loader_fetch(LoaderChunk &L, const __bf16 *const src[2], const f32x2 *pairs_h, long long t0,
                                    int rows, int lane) {
  const int sub = lane >> 3, piece = lane & 7;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 2 * kSavedTiles; ++i) {
      const int row = min(8 * i + sub, rows - 1);
      L.v[t][i] = reinterpret_cast<const u32x4 *>(src[t] + (t0 + row) * kD)[piece];
    }
  // The pairs array holds every token of the chunk (padding tokens as zeros).
  if constexpr (kHalf == 0) {
#pragma unroll
    for (int i = 0; i < 2 * kSavedTiles; ++i) L.rowpr[i] = pairs_h[t0 + 8 * i + sub];
  } else {
    L.pr = reinterpret_cast<const u32x4 *>(pairs_h + t0)[lane & 15];
  }
}

// QSN piece: the eight rounded phi(q) of a piece times minus the row's 1/den,
// rounded once (saved_q_operands with sign -1).
__device__ inline u32x4 qsn_piece(u32x4 phiq, float rd) {
  rd = -rd;
  u32x4 o;
#pragma unroll
  for (int w = 0; w < 4; ++w) o[w] = pack_bf16(bf16_lo(phiq[w]) * rd, bf16_hi(phiq[w]) * rd);
  return o;
}

// Writes a fetched chunk into a slot in the staging layout (stage_index).
template <int kHalf> __device__ inline void loader_store(const LoaderChunk &L, u32x4 *slot, int lane) {
  const int sub = lane >> 3, piece = lane & 7;
  auto at = [&](int tensor, int i) -> u32x4 & { return slot[(tensor * 2 * kSavedTiles + i) * 64 + 8 * sub + (piece ^ sub)]; };
#pragma unroll
  for (int i = 0; i < 2 * kSavedTiles; ++i) {
    const u32x4 ph = phi_piece(L.v[0][i]);
    at(kHalf, i) = ph;
    at(kHalf + 2, i) = L.v[1][i];
    if constexpr (kHalf == 0) at(kQSN, i) = qsn_piece(ph, L.rowpr[i][0]);
  }
  if constexpr (kHalf == 1) {
    if (lane < 8 * kSavedTiles) slot[kSavedPairsVec + lane] = L.pr;
    // b of tokens t = 2 l, 2 l + 1 (lane l < 16) at byte 16 g + 8 it + 2 r
    // of the b vector, t = 16 it + 4 g + r.
    if (lane < 16) {
      const int t = 2 * lane;
      const f32x4 pr = __builtin_bit_cast(f32x4, L.pr);
      reinterpret_cast<uint32_t *>(slot + kSavedBVec)[4 * ((t & 15) >> 2) + 2 * (t >> 4) + ((t & 3) >> 1)] =
          pack_bf16(pr[1], pr[3]);
    }
  }
}

template <int kHalf>
__device__ inline void saved_loader(const BwdParams &p, u32x4 (*ring)[kSavedSlotVec], int h, const SavedSeg &sg,
                                    int lane) {
  constexpr int kT = 16 * kSavedTiles;
  const long long base = (long long)h * p.N * kD;
  const __bf16 *src[2] = {reinterpret_cast<const __bf16 *>(kHalf == 0 ? p.Q : p.K) + base,
                          reinterpret_cast<const __bf16 *>(kHalf == 0 ? p.V : p.dO) + base};
  const f32x2 *pairs_h = p.stats + (long long)h * p.stats_stride;
  // Chunks past the last one fetch the last one again (unused), keeping
  // every step's loads unconditional.
  auto fetch = [&](LoaderChunk &L, int c) {
    const long long t0 = sg.t_begin + (long long)min(c, sg.chunks - 1) * kT;
    loader_fetch<kHalf>(L, src, pairs_h, t0, (int)min<long long>(kT, sg.t_end - t0), lane);
  };
  // Chunk c: write it into slot c mod 3 (its previous contents, chunk c - 3,
  // were read by the compute waves between the barriers of chunks c - 3 and
  // c - 1, and this wave has passed the latter), refill the registers with
  // chunk c + kLoaderDepth, then the barrier that releases chunk c.
  auto step = [&](LoaderChunk &L, int c) {
    loader_store<kHalf>(L, ring[c % kSavedRing], lane);
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
  saved_barrier();  // closing barrier (walk_chunks)
}

// A compute wave's half of a state.  dQ and dK waves hold transposed tiles
// [mt][x], tile (mt, ct = 2 hf + x) of S^T or R^T, and z or r of those
// feature columns; dV waves hold R tiles [ct][x], tile (ct, mt = 2 hf + x).
struct HalfState {
  f32x4 S[4][2];
  f32x4 z[2];
};

__device__ inline void half_zero(HalfState &st) {
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    st.z[x] = zero4();
#pragma unroll
    for (int a = 0; a < 4; ++a) st.S[a][x] = zero4();
  }
}

// Loads half hf of a record.  A record stores S tile (ct, mt) lane (n, g)
// register r = S[pi(ct,g,r)][pi(mt,n>>2,n&3)] (forward_kernels.hpp).  For dQ
// and dK it is loaded transposed, tiles (mt, ct) with ct = 2 hf + x: lane
// (n, g) register r takes S[pi(ct,n>>2,n&3)][pi(mt,g,r)], the record's lane
// 16 (n>>2) + 4 g + r, register n & 3, and z as state_load_record loads it.
// For dV it is loaded as stored, tiles mt = 2 hf + x, without z.
template <bool kTransposed> __device__ inline void half_load_record(HalfState &st, const float *rec, int hf, int lane) {
  const int n16 = lane & 15, g = lane >> 4;
  const f32x4 *p = reinterpret_cast<const f32x4 *>(rec);
  if constexpr (kTransposed) {
    const int lane_base = 16 * (n16 >> 2) + 4 * g, reg = n16 & 3;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int ct = 2 * hf + x;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) st.S[mt][x][r] = rec[((ct * 4 + mt) * 64 + lane_base + r) * 4 + reg];
      st.z[x] = p[1024 + ct * 4 + g];
    }
  } else {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      st.z[x] = zero4();
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) st.S[ct][x] = p[(ct * 4 + 2 * hf + x) * 64 + lane];
    }
  }
}

// st += half hf of a record, element by element (no second state is held).
template <bool kTransposed> __device__ inline void half_add_record(HalfState &st, const float *rec, int hf, int lane) {
  const int n16 = lane & 15, g = lane >> 4;
  const f32x4 *p = reinterpret_cast<const f32x4 *>(rec);
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    if constexpr (kTransposed) {
      const int ct = 2 * hf + x, lane_base = 16 * (n16 >> 2) + 4 * g, reg = n16 & 3;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) st.S[mt][x][r] += rec[((ct * 4 + mt) * 64 + lane_base + r) * 4 + reg];
      st.z[x] += p[1024 + ct * 4 + g];
    } else {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) st.S[ct][x] += p[(ct * 4 + 2 * hf + x) * 64 + lane];
    }
  }
}

// st = records first, first + stride, ... (count of them, added in that order).
template <bool kTransposed>
__device__ inline void half_sum_records(HalfState &st, const float *first, int count, long long stride, int hf,
                                        int lane) {
  half_zero(st);
#pragma unroll 1
  for (int j = 0; j < count; ++j) half_add_record<kTransposed>(st, first + j * stride, hf, lane);
}

// Row-layout fragments 2 x, 2 x + 1 of tensor tsr, row tile it.
template <int NT>
__device__ inline void lds_row_frag_pair(const u32x4 *slot, int tsr, int it, int x, int lane, Frag<__bf16> f[2]) {
  const int R = 16 * it + (lane & 15), g = lane >> 4;
  const u32x4 v = slot[tsr * 2 * NT * 64 + stage_index(R, 4 * x + g)];
  f[0].w[0] = v[0];
  f[0].w[1] = v[1];
  f[1].w[0] = v[2];
  f[1].w[1] = v[3];
}

// Stores output column tiles 2 x, 2 x + 1 of 16 rows (columns 32 x .. 32 x +
// 31): lane (n, g) holds row n, columns 32 x + 8 g .. 32 x + 8 g + 7.
template <bool kFull>
__device__ inline void store_half_tiles(__bf16 *base, long long row0, int rows_left, const f32x4 a[2], int x, int n16,
                                        int g) {
  const u32x4 v = {pack_bf16(a[0][0], a[0][1]), pack_bf16(a[0][2], a[0][3]), pack_bf16(a[1][0], a[1][1]),
                   pack_bf16(a[1][2], a[1][3])};
  if (kFull || n16 < rows_left)
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(base + (row0 + n16) * kD) + 4 * x + g);
}

// Lane (n, g) of a walk wave: 1/den and b of tokens 16 it + 4 g + r (token
// layout) from the two pair vectors stats_tok reads, tokens past the end zero.
template <bool kFull>
__device__ inline void saved_stats_tok(const u32x4 lo[kSavedTiles], const u32x4 hi[kSavedTiles], int rows, int g,
                                       f32x4 rdt[kSavedTiles], f32x4 bt[kSavedTiles]) {
#pragma unroll
  for (int it = 0; it < kSavedTiles; ++it) {
    const f32x4 l = __builtin_bit_cast(f32x4, lo[it]), h = __builtin_bit_cast(f32x4, hi[it]);
    rdt[it] = f32x4{l[0], l[2], h[0], h[2]};
    bt[it] = f32x4{l[1], l[3], h[1], h[3]};
    if (!kFull)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (16 * it + 4 * g + r >= rows) {
          rdt[it][r] = 0.f;
          bt[it][r] = 0.f;
        }
  }
}

// Each compute wave splits a chunk's LDS reads in two.  The "early" set, what
// the chunk's first products need, is read one chunk ahead: after the body
// of chunk c has started its first products, it issues the early reads of
// chunk c + 1 (published by the barrier at the top of its iteration).  The
// "late" set is read at the top of chunk c's own iteration and arrives while
// the first products run.  The ring keeps chunk c's slot intact until every
// wave has finished chunk c (a loader refills it only after the barrier of
// chunk c + 2).  sched_barrier keeps the compiler from moving the reads of
// chunk c + 1 ahead of the first products.
__device__ inline void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// dQ wave.  Early: V and dO rows and the pairs by row (the D^T tiles and
// S G^T).  Late: phi(K) tokens and phi(Q) rows of its features, V tokens.
struct DqEarly {
  Frag<__bf16> vf[kSavedTiles][4], gf[kSavedTiles][4];
  f32x2 sr[kSavedTiles];
};

__device__ inline void issue_dq_early(DqEarly &E, const u32x4 *slot, int lane) {
  constexpr int NT = kSavedTiles;
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    lds_row_frags<NT>(slot, kVals, it, lane, E.vf[it]);
    lds_row_frags<NT>(slot, kGrad, it, lane, E.gf[it]);
    E.sr[it] = stats_row(slot + kSavedPairsVec, it, lane & 15);
  }
}

// dQ wave, one chunk, feature columns ct = 2 hf + x:
// dphi(Q)^T = phi(K)^T D^T + (S G^T) / den + z b^T, then S^T += V^T phi(K),
// z += column sums of phi(K).  next: the slot of chunk c + 1, or null.
template <bool kFull>
__device__ inline void saved_dq_chunk(HalfState &st, const DqEarly &E, DqEarly &En, const u32x4 *slot,
                                      const u32x4 *next, long long t0, int rows, __bf16 *dQh, int hf, int lane) {
  typedef __bf16 E16;
  constexpr int NT = kSavedTiles;
  const int n16 = lane & 15, g = lane >> 4;
  Frag<E16> qphi[NT][2], kt[NT][2], vt[NT][4];
#pragma unroll
  for (int it = 0; it < NT; ++it) {
#pragma unroll
    for (int x = 0; x < 2; ++x) kt[it][x] = lds_tok_frag<NT>(slot, kPhiK, it, 2 * hf + x, lane);
    lds_row_frag_pair<NT>(slot, kPhiQ, it, hf, lane, qphi[it]);
#pragma unroll
    for (int c = 0; c < 4; ++c) vt[it][c] = lds_tok_frag<NT>(slot, kVals, it, c, lane);
  }
  // First products, from the early set: the D^T tiles and S G^T.
  Frag<E16> sf[2][4];  // S as the A operand (row = feature, k = value column)
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) sf[x][mt] = to_frag<E16>(st.S[mt][x]);
  // D^T (key j, query i) = (v_j . g_i) / den_i + b_i for j <= i; tile
  // (it, jt) at df[it * (it + 1) / 2 + jt].
  Frag<E16> df[NT * (NT + 1) / 2];
  f32x4 sg[NT][2];
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    const float rd = E.sr[it][0], b = E.sr[it][1];
#pragma unroll
    for (int jt = 0; jt <= it; ++jt) {
      f32x4 d = zero4();
      d = mac2<E16>(d, E.vf[jt][0], E.vf[jt][1], E.gf[it][0], E.gf[it][1]);
      d = mac2<E16>(d, E.vf[jt][2], E.vf[jt][3], E.gf[it][2], E.gf[it][3]);
      d = d * rd + b;
      if (jt == it)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * g + r > n16) d[r] = 0.f;
      df[it * (it + 1) / 2 + jt] = to_frag<E16>(d);
    }
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      sg[it][x] = mac2<E16>(zero4(), sf[x][0], sf[x][1], E.gf[it][0], E.gf[it][1]);
      sg[it][x] = mac2<E16>(sg[it][x], sf[x][2], sf[x][3], E.gf[it][2], E.gf[it][3]);
    }
  }
  // The dK waves' D tiles: D (query 4 g + r, key n) is the transpose of
  // D^T, taken exactly by a product with the identity (df as the A operand).
  // Wave hf = 0 writes tiles 0 and 2, wave 1 tile 1.
  {
    const Frag<E16> ident = frag_identity<E16>(n16, g);
    u32x2 *dout = reinterpret_cast<u32x2 *>(const_cast<u32x4 *>(slot) + kSavedDVec);
#pragma unroll
    for (int t = 0; t < NT * (NT + 1) / 2; ++t)
      if ((t & 1) == hf) dout[64 * t + lane] = to_frag<E16>(mac1<E16>(zero4(), df[t], ident)).w;
  }
  sched_fence();
  if (next) issue_dq_early(En, next, lane);
  sched_fence();
  if (!kFull)
#pragma unroll
    for (int it = 0; it < NT; ++it) {
#pragma unroll
      for (int x = 0; x < 2; ++x) mask_tokens(kt[it][x], 16 * it + 4 * g, rows);
#pragma unroll
      for (int c = 0; c < 4; ++c) mask_tokens(vt[it][c], 16 * it + 4 * g, rows);
    }
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    const float rd = E.sr[it][0], b = E.sr[it][1];
    const Frag<E16> *dft = df + it * (it + 1) / 2;
    f32x4 dq[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      dq[x] = zero4();
#pragma unroll
      for (int jp = 0; 2 * jp + 1 <= it; ++jp)
        dq[x] = mac2<E16>(dq[x], kt[2 * jp][x], kt[2 * jp + 1][x], dft[2 * jp], dft[2 * jp + 1]);
      if ((it & 1) == 0) dq[x] = mac1<E16>(dq[x], kt[it][x], dft[it]);
    }
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const f32x4 pq = frag_f32(qphi[it][x]);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        dq[x][r] = (dq[x][r] + sg[it][x][r] * rd + st.z[x][r] * b) * phi_prime_of_phi(pq[r]);
    }
    store_half_tiles<kFull>(dQh, t0 + 16 * it, rows - 16 * it, dq, hf, n16, g);
  }
  // S^T += V^T phi(K) (tiles [mt][x]), z += phi(K)^T 1.
  const Frag<E16> ones = frag_ones<E16>();
#pragma unroll
  for (int x = 0; x < 2; ++x) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) st.S[mt][x] = mac2<E16>(st.S[mt][x], vt[0][mt], vt[1][mt], kt[0][x], kt[1][x]);
    st.z[x] = mac2<E16>(st.z[x], kt[0][x], kt[1][x], ones, ones);
  }
}

// dK wave.  Early: dO tokens and -phi(Q)/den tokens of its features (the
// state update).  Late: phi(Q) tokens and phi(K) rows of its features, V and
// dO rows, the pairs by token.
struct DkEarly {
  Frag<__bf16> gt[kSavedTiles][4], qsn[kSavedTiles][2];
};

__device__ inline void issue_dk_early(DkEarly &E, const u32x4 *slot, int hf, int lane) {
  constexpr int NT = kSavedTiles;
#pragma unroll
  for (int it = 0; it < NT; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) E.gt[it][c] = lds_tok_frag<NT>(slot, kGrad, it, c, lane);
#pragma unroll
    for (int x = 0; x < 2; ++x) E.qsn[it][x] = lds_tok_frag<NT>(slot, kQSN, it, 2 * hf + x, lane);
  }
}

// dK wave, one chunk, feature columns ct = 2 hf + x: first R^T -= G^T
// (phi(Q)/den), r -= phi(Q)^T b (the chunk's own terms), then
// dphi(K)^T = R V^T + r 1^T + phi(Q)^T D.  The wave holds -r (negation is
// exact), so that the chunk's b terms are added as stored.
template <bool kFull>
__device__ inline void saved_dk_chunk(HalfState &st, DkEarly &E, DkEarly &En, const u32x4 *slot, const u32x4 *next,
                                      long long t0, int rows, __bf16 *dKh, int hf, int lane) {
  typedef __bf16 E16;
  constexpr int NT = kSavedTiles;
  const int n16 = lane & 15, g = lane >> 4;
  Frag<E16> qt[NT][2], kphi[NT][2], vf[NT][4], dfr[NT * (NT + 1) / 2];
#pragma unroll
  for (int it = 0; it < NT; ++it) {
#pragma unroll
    for (int x = 0; x < 2; ++x) qt[it][x] = lds_tok_frag<NT>(slot, kPhiQ, it, 2 * hf + x, lane);
    lds_row_frags<NT>(slot, kVals, it, lane, vf[it]);
    lds_row_frag_pair<NT>(slot, kPhiK, it, hf, lane, kphi[it]);
  }
  // D (query i = 16 it + 4 g + r, key j = 16 jt + n) = (g_i . v_j) / den_i + b_i
  // for i >= j, tile (it, jt) at dfr[it * (it + 1) / 2 + jt], from the dQ
  // waves; b by token.
#pragma unroll
  for (int t = 0; t < NT * (NT + 1) / 2; ++t) dfr[t].w = reinterpret_cast<const u32x2 *>(slot + kSavedDVec)[64 * t + lane];
  const u32x4 bv = slot[kSavedBVec + g];
  const Frag<E16> bt0 = {u32x2{bv[0], bv[1]}}, bt1 = {u32x2{bv[2], bv[3]}};
  if (!kFull) zero_tokens<E16, NT>(E.gt, rows, g);
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      st.S[mt][x] = mac2<E16>(st.S[mt][x], E.gt[0][mt], E.gt[1][mt], E.qsn[0][x], E.qsn[1][x]);
  sched_fence();
  if (next) issue_dk_early(En, next, hf, lane);
  sched_fence();
  static_assert(NT == 2, "the b vector holds two row tiles");
#pragma unroll
  for (int x = 0; x < 2; ++x) st.z[x] = mac2<E16>(st.z[x], qt[0][x], qt[1][x], bt0, bt1);
  Frag<E16> rf[2][4];  // R as the A operand (row = feature, k = value column)
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) rf[x][mt] = to_frag<E16>(st.S[mt][x]);
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) {
    f32x4 dk[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      dk[x] = mac2<E16>(zero4(), rf[x][0], rf[x][1], vf[jt][0], vf[jt][1]);
      dk[x] = mac2<E16>(dk[x], rf[x][2], rf[x][3], vf[jt][2], vf[jt][3]);
    }
    // Query tiles it >= jt: both in one 32-token product for jt = 0.
#pragma unroll
    for (int x = 0; x < 2; ++x)
      dk[x] = jt == 0 ? mac2<E16>(dk[x], qt[0][x], qt[1][x], dfr[0], dfr[1]) : mac1<E16>(dk[x], qt[1][x], dfr[2]);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const f32x4 pk = frag_f32(kphi[jt][x]);
#pragma unroll
      for (int r = 0; r < 4; ++r) dk[x][r] = (dk[x][r] - st.z[x][r]) * phi_prime_of_phi(pk[r]);
    }
    store_half_tiles<kFull>(dKh, t0 + 16 * jt, rows - 16 * jt, dk, hf, n16, g);
  }
}

// dV wave.  Early: -phi(Q)/den tokens and dO tokens of its value columns
// (the state update).  Late: the pairs by token, phi(Q) and phi(K) rows.
struct DvEarly {
  Frag<__bf16> qsn[kSavedTiles][4], gt[kSavedTiles][2];
};

__device__ inline void issue_dv_early(DvEarly &E, const u32x4 *slot, int hf, int lane) {
  constexpr int NT = kSavedTiles;
#pragma unroll
  for (int it = 0; it < NT; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) E.qsn[it][c] = lds_tok_frag<NT>(slot, kQSN, it, c, lane);
#pragma unroll
    for (int x = 0; x < 2; ++x) E.gt[it][x] = lds_tok_frag<NT>(slot, kGrad, it, 2 * hf + x, lane);
  }
}

// dV wave, one chunk, value columns mt = 2 hf + x: first R -= (phi(Q)/den)^T
// G, then dV^T = R^T phi(K)^T + G^T W' with
// W'_ij = phi(q_i) . phi(k_j) / den_i, i >= j.
template <bool kFull>
__device__ inline void saved_dv_chunk(HalfState &st, DvEarly &E, DvEarly &En, const u32x4 *slot, const u32x4 *next,
                                      long long t0, int rows, __bf16 *dVh, int hf, int lane) {
  typedef __bf16 E16;
  constexpr int NT = kSavedTiles;
  const int n16 = lane & 15, g = lane >> 4;
  Frag<E16> qf[NT][4], kf[NT][4];
  u32x4 slo[NT], shi[NT];
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    slo[it] = slot[kSavedPairsVec + 8 * it + 2 * g];
    shi[it] = slot[kSavedPairsVec + 8 * it + 2 * g + 1];
    lds_row_frags<NT>(slot, kPhiK, it, lane, kf[it]);
    lds_row_frags<NT>(slot, kPhiQ, it, lane, qf[it]);
  }
  if (!kFull)
#pragma unroll
    for (int it = 0; it < NT; ++it)
#pragma unroll
      for (int x = 0; x < 2; ++x) mask_tokens(E.gt[it][x], 16 * it + 4 * g, rows);
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int x = 0; x < 2; ++x)
      st.S[ct][x] = mac2<E16>(st.S[ct][x], E.qsn[0][ct], E.qsn[1][ct], E.gt[0][x], E.gt[1][x]);
  sched_fence();
  if (next) issue_dv_early(En, next, hf, lane);
  sched_fence();
  f32x4 rdt[NT], bt[NT];
  saved_stats_tok<kFull>(slo, shi, rows, g, rdt, bt);
  if (!kFull) zero_rows<E16, NT>(qf, rows, n16);
  // W' tiles first (phi(Q) rows and the pairs are then done with), tile
  // (it, jt) at wf[it * (it + 1) / 2 + jt].
  Frag<E16> wf[NT * (NT + 1) / 2];
#pragma unroll
  for (int it = 0; it < NT; ++it)
#pragma unroll
    for (int jt = 0; jt <= it; ++jt) {
      f32x4 w = zero4();
      w = mac2<E16>(w, qf[it][0], qf[it][1], kf[jt][0], kf[jt][1]);
      w = mac2<E16>(w, qf[it][2], qf[it][3], kf[jt][2], kf[jt][3]);
      w = w * rdt[it];
      if (it == jt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * g + r < n16) w[r] = 0.f;
      wf[it * (it + 1) / 2 + jt] = to_frag<E16>(w);
    }
  Frag<E16> ro[4][2];  // R^T as the A operand (row = value column, k = feature)
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int x = 0; x < 2; ++x) ro[ct][x] = to_frag<E16>(st.S[ct][x]);
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) {
    f32x4 dv[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      dv[x] = mac2<E16>(zero4(), ro[0][x], ro[1][x], kf[jt][0], kf[jt][1]);
      dv[x] = mac2<E16>(dv[x], ro[2][x], ro[3][x], kf[jt][2], kf[jt][3]);
    }
    // Query tiles it >= jt: both in one 32-token product for jt = 0.
#pragma unroll
    for (int x = 0; x < 2; ++x)
      dv[x] = jt == 0 ? mac2<E16>(dv[x], E.gt[0][x], E.gt[1][x], wf[0], wf[1]) : mac1<E16>(dv[x], E.gt[1][x], wf[2]);
    store_half_tiles<kFull>(dVh, t0 + 16 * jt, rows - 16 * jt, dv, hf, n16, g);
  }
}

// Half hf of the suffix state (R, -r) from the start of reverse segment ur
// on: record ur after the suffix scan, or the sum of the totals records
// ur + 1 .. P, last first; r negated (the dK wave's form; the dV wave has no
// r).
template <bool kTransposed>
__device__ inline void load_suffix(HalfState &st, const BwdParams &p, int h, int ur, int hf, int lane) {
  // The record addressing is derived here from an opaque copy of the lane
  // index, so the compiler recomputes it on this rare path instead of keeping
  // it in registers across the chunk loop.
  asm volatile("" : "+v"(lane));
  const float *recs = p.wsT + (long long)h * p.recT * kStateFloats;
  if (p.rev_sum_in_walk) {
    half_sum_records<kTransposed>(st, recs + (long long)p.rev_segments * kStateFloats, p.rev_segments - ur,
                                  -(long long)kStateFloats, hf, lane);
  } else {
    half_load_record<kTransposed>(st, recs + (long long)ur * kStateFloats, hf, lane);
  }
#pragma unroll
  for (int x = 0; x < 2; ++x) st.z[x] = -st.z[x];
  // The loads land here, on this rare path: otherwise the compiler, not
  // knowing which path a chunk took, waits for every outstanding memory
  // operation (the previous chunks' output stores included) before the
  // state's next use on every chunk.
  wait_vmcnt<0>();
}

// The compute waves' loop.  With kPrefetch, the barrier at the top of chunk
// c's iteration publishes chunk c + 1, and chunk(E, En, c, next) computes
// chunk c from its early set E and reads chunk c + 1's early set into En from
// slot next (null after the last chunk).  Without, the barrier publishes
// chunk c itself and its early set is read right after it.  Either way every
// wave passes the barriers of chunks 0 .. chunks - 1 in order, then one
// closing barrier (the loaders too).  The dK waves read chunk c's D tiles,
// which the dQ waves write while computing chunk c, after the barrier that
// follows it: that is barrier c + 1, and for the last chunk the closing one.
template <class Early, bool kPrefetch, class IssueEarly, class Chunk>
__device__ inline void walk_chunks(int chunks, const u32x4 (*ring)[kSavedSlotVec], IssueEarly &&issue_early,
                                   Chunk &&chunk) {
  if constexpr (kPrefetch) {
    Early e;
    saved_barrier();
    issue_early(e, ring[0]);
    for (int c = 0; c < chunks; ++c) {
      // Barrier c + 1: chunk c + 1 is in its slot, and the dQ waves have
      // written chunk c's D tiles, which the dK waves read in chunk(c).  The
      // last chunk's is the closing barrier, which every role passes.
      saved_barrier();
      const bool more = c + 1 < chunks;
      Early en;
      chunk(e, en, c, more ? ring[(c + 1) % kSavedRing] : nullptr);
      e = en;
    }
  } else {
    for (int c = 0; c < chunks; ++c) {
      Early e;
      saved_barrier();
      issue_early(e, ring[c % kSavedRing]);
      chunk(e, e, c, nullptr);
    }
    saved_barrier();  // closing: the last chunk's D tiles are written
  }
}

__global__ __launch_bounds__(64 * kSavedWaves, 1) void bwd_saved_walk_kernel(BwdParams p) {
  constexpr int NT = kSavedTiles;
  constexpr int kT = 16 * NT;
  __shared__ u32x4 ring[kSavedRing][kSavedSlotVec];
  const int worker = blockIdx.x;
  const int h = worker % p.heads;
  const int s = worker / p.heads;
  if (s >= p.walk_segments) return;
  const SavedSeg sg = saved_segment(p, s);
  if (sg.chunks == 0) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: kept in scalar registers
  const int lane = threadIdx.x & 63;
  // Waves w and w + 4 share a SIMD.  Pairing each loader with a dK wave and
  // each dQ wave with a dV wave balances the four SIMDs' arithmetic:
  // w 0, 1 loaders; 2, 3 dQ; 4, 5 dK; 6, 7 dV; hf = w & 1.
  const int hf = wave & 1;
  const int role = wave >> 1;
  if (role == 0) {
    if (hf == 0) {
      saved_loader<0>(p, ring, h, sg, lane);
    } else {
      saved_loader<1>(p, ring, h, sg, lane);
    }
    return;
  }
  const long long base = (long long)h * p.N * kD;
  const long long rev_tokens = (long long)p.rev_chunks * kChunk;
  HalfState st;
  auto chunk_t0 = [&](int c) { return sg.t_begin + (long long)c * kT; };
  auto chunk_rows = [&](int c) { return (int)min<long long>(kT, sg.t_end - chunk_t0(c)); };
  // The suffix state starts exact at every reverse-segment start (walk
  // segments begin at one) and is carried by subtraction in between: chunk
  // c is an anchor when its start is a multiple of rev_tokens.  The next
  // anchor is tracked as a chunk index, so no chunk divides.
  const int anchor_period = (int)(rev_tokens / kT);
  int next_anchor = anchor_period - (int)((sg.t_begin / kT) % anchor_period);
  int next_ur = (int)(sg.t_begin / rev_tokens) + 1;  // reverse segment starting at next_anchor
  auto anchor = [&](int c) {
    if (c != next_anchor) return false;
    next_anchor += anchor_period;
    return true;
  };
  if (role == 1) {
    // Prefix (S, z) at the segment start, from the forward's records.
    const int u0 = s * p.walk_k;  // first forward segment of this walk segment
    if (p.recF == 0) {
      half_zero(st);
    } else if (p.sum_in_walk) {
      half_sum_records<true>(st, p.wsF + (long long)h * p.recF * kStateFloats, u0, kStateFloats, hf, lane);
    } else {
      half_load_record<true>(st, p.wsF + ((long long)h * p.recF + u0) * kStateFloats, hf, lane);
    }
    wait_vmcnt<0>();
    __bf16 *out = reinterpret_cast<__bf16 *>(p.dQ) + base;
    walk_chunks<DqEarly, false>(
        sg.chunks, ring, [&](DqEarly &E, const u32x4 *slot) { issue_dq_early(E, slot, lane); },
        [&](DqEarly &E, DqEarly &En, int c, const u32x4 *next) {
          const u32x4 *slot = ring[c % kSavedRing];
          if (chunk_rows(c) == kT) {
            saved_dq_chunk<true>(st, E, En, slot, next, chunk_t0(c), kT, out, hf, lane);
          } else {
            saved_dq_chunk<false>(st, E, En, slot, next, chunk_t0(c), chunk_rows(c), out, hf, lane);
          }
        });
  } else if (role == 2) {
    load_suffix<true>(st, p, h, (int)(sg.t_begin / rev_tokens), hf, lane);
    __bf16 *out = reinterpret_cast<__bf16 *>(p.dK) + base;
    walk_chunks<DkEarly, true>(
        sg.chunks, ring, [&](DkEarly &E, const u32x4 *slot) { issue_dk_early(E, slot, hf, lane); },
        [&](DkEarly &E, DkEarly &En, int c, const u32x4 *next) {
          const u32x4 *slot = ring[c % kSavedRing];
          if (anchor(c)) load_suffix<true>(st, p, h, next_ur++, hf, lane);
          if (chunk_rows(c) == kT) {
            saved_dk_chunk<true>(st, E, En, slot, next, chunk_t0(c), kT, out, hf, lane);
          } else {
            saved_dk_chunk<false>(st, E, En, slot, next, chunk_t0(c), chunk_rows(c), out, hf, lane);
          }
        });
  } else {
    load_suffix<false>(st, p, h, (int)(sg.t_begin / rev_tokens), hf, lane);
    __bf16 *out = reinterpret_cast<__bf16 *>(p.dV) + base;
    walk_chunks<DvEarly, true>(
        sg.chunks, ring, [&](DvEarly &E, const u32x4 *slot) { issue_dv_early(E, slot, hf, lane); },
        [&](DvEarly &E, DvEarly &En, int c, const u32x4 *next) {
          const u32x4 *slot = ring[c % kSavedRing];
          if (anchor(c)) load_suffix<false>(st, p, h, next_ur++, hf, lane);
          if (chunk_rows(c) == kT) {
            saved_dv_chunk<true>(st, E, En, slot, next, chunk_t0(c), kT, out, hf, lane);
          } else {
            saved_dv_chunk<false>(st, E, En, slot, next, chunk_t0(c), chunk_rows(c), out, hf, lane);
          }
        });
  }
}

}  // namespace linattn
