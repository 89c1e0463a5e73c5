// validate.cpp -- host-side argument checks and the launch planner.
#include "validate.hpp"

#include <limits.h>

#include <algorithm>

namespace linattn {

namespace {

constexpr int kChunkTokens = 64;
constexpr size_t kStateBytes = (4096 + 64) * sizeof(float);
// Segments are at least this many chunks long while that still gives the
// device its target number of waves (a 16.6 KB record per segment is then
// small next to the segment's data).  When it does not -- few heads, short
// sequences, where a call is bound by the latency of each wave's serial
// chunks -- segments shrink down to one chunk, but to at most
// kMaxShortSegments per head, which keeps the prefix scan to one or two load
// batches.  Measured on MI355X for B1 H8, causal bf16: N = 512 forward
// 28.6 -> 14.2 us and forward + backward 109 -> 47 us; N = 8192 forward
// 35.4 -> 27.9 us with 64 segments (34.0 us with 128).
constexpr long long kMinSegmentChunks = 4;
constexpr long long kMaxShortSegments = 64;
// Workers (waves) aimed for per compute unit: one per SIMD (the walk kernel
// holds about 480 registers per lane).
constexpr long long kWavesPerCU = 4;


Check fail(linattn_status s, const std::string &msg) {
  Check c;
  c.status = s;
  c.message = msg;
  return c;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// a * b * c into *out without overflow of size_t; false on overflow.
bool mul3(size_t a, size_t b, size_t c, size_t *out) {
  if (a != 0 && b > SIZE_MAX / a) return false;
  size_t ab = a * b;
  if (ab != 0 && c > SIZE_MAX / ab) return false;
  *out = ab * c;
  return true;
}

}  // namespace

size_t dtype_bytes(linattn_dtype dt) {
  switch (dt) {
  case LINATTN_F32: return 4;
  case LINATTN_BF16: return 2;
  default: return 0;
  }
}

bool overlaps(const Buffer &a, const Buffer &b) {
  if (a.ptr == nullptr || b.ptr == nullptr || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.ptr), b0 = reinterpret_cast<uintptr_t>(b.ptr);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

Plan plan_forward(long long heads, long long N, int causal, int cus, int override_segments) {
  Plan p;
  p.heads = heads;
  p.chunks = ceil_div(N, kChunkTokens);
  if (heads <= 0 || N <= 0) return p;
  if (cus < 1) cus = 1;
  const long long target = kWavesPerCU * cus;
  long long segs;
  if (override_segments > 0) {
    segs = override_segments;
  } else {
    segs = ceil_div(target, heads);
    if (segs > p.chunks) segs = p.chunks;
    const long long long_cap = ceil_div(p.chunks, kMinSegmentChunks);
    if (segs > long_cap) segs = std::max(long_cap, std::min(segs, kMaxShortSegments));
  }
  if (segs > p.chunks) segs = p.chunks;
  if (segs < 1) segs = 1;
  if (segs > INT_MAX / 2) segs = INT_MAX / 2;
  if (segs > 1 && heads * segs > INT_MAX) segs = std::max(1LL, (long long)INT_MAX / heads);  // grid size
  long long seg_chunks = ceil_div(p.chunks, segs);
  segs = ceil_div(p.chunks, seg_chunks);  // no empty segment
  p.segments = (int)segs;
  p.seg_chunks = (int)seg_chunks;
  if (causal) {
    p.records = p.segments > 1 ? p.segments : 0;
  } else {
    // Segments are summed in workgroups of kPlanGroupWaves; one record per group,
    // then the head's total.
    p.groups = (int)ceil_div(p.segments, kPlanGroupWaves);
    p.records = p.groups + 1;
    long long ranges = ceil_div(target, heads);
    if (ranges > p.chunks) ranges = p.chunks;
    if (ranges < 1) ranges = 1;
    long long range_chunks = ceil_div(p.chunks, ranges);
    p.ranges = (int)ceil_div(p.chunks, range_chunks);
    p.range_chunks = (int)range_chunks;
    p.range_groups = (int)ceil_div(p.ranges, kPlanGroupWaves);
  }
  size_t bytes = 0;
  if (!mul3((size_t)heads, (size_t)p.records, kStateBytes, &bytes)) bytes = SIZE_MAX;
  p.workspace_bytes = bytes;
  return p;
}

namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace

BwdPlan plan_backward(long long heads, long long N, int causal, int cus, int override_segments) {
  BwdPlan b;
  b.fwd = plan_forward(heads, N, causal, cus, override_segments);
  if (heads <= 0 || N <= 0) return b;
  const Plan &p = b.fwd;
  b.recR = causal ? (p.segments > 1 ? p.segments : 0) : p.ranges + 1;
  b.stats_stride = ceil_div(N, kChunkTokens) * kChunkTokens;
  size_t f_bytes = p.workspace_bytes, r_bytes = 0, s_bytes = 0;
  if (f_bytes == SIZE_MAX || !mul3((size_t)heads, (size_t)b.recR, kStateBytes, &r_bytes) ||
      !mul3((size_t)heads, (size_t)b.stats_stride, 8, &s_bytes) || f_bytes > SIZE_MAX / 4 ||
      r_bytes > SIZE_MAX / 4 || s_bytes > SIZE_MAX / 4) {
    b.workspace_bytes = SIZE_MAX;
    return b;
  }
  b.off_r = align256(f_bytes);
  b.off_stats = align256(b.off_r + r_bytes);
  b.workspace_bytes = b.off_stats + s_bytes;
  return b;
}

TrainPlan plan_train(long long heads, long long N, int causal, int cus, int override_segments) {
  TrainPlan t;
  t.bwd = plan_backward(heads, N, causal, cus, override_segments);
  if (heads <= 0 || N <= 0) return t;
  const BwdPlan &b = t.bwd;
  if (b.workspace_bytes == SIZE_MAX) {
    t.workspace_bytes = SIZE_MAX;
    return t;
  }
  const long long P = b.fwd.segments;
  if (cus < 1) cus = 1;
  const long long per_head = std::max(1LL, ceil_div((long long)kTrainWalkGroupsPerCU * cus, heads));
  t.walk_k = (int)std::max(1LL, P / per_head);
  t.walk_segments = (int)ceil_div(P, t.walk_k);
  if (P == 1 && b.fwd.chunks >= kTrainSplitFrom) {
    t.rev_chunks = (int)ceil_div(b.fwd.chunks, 2);
    t.rev_segments = (int)ceil_div(b.fwd.chunks, t.rev_chunks);
  } else {
    t.rev_chunks = b.fwd.seg_chunks;
    t.rev_segments = (int)P;
  }
  t.recT = t.rev_segments + 1;
  size_t rden_bytes = 0, t_bytes = 0;
  if (!mul3((size_t)heads, (size_t)b.stats_stride, 4, &rden_bytes) ||
      !mul3((size_t)heads, (size_t)t.recT, kStateBytes, &t_bytes) || rden_bytes > SIZE_MAX / 4 ||
      t_bytes > SIZE_MAX / 4 || b.workspace_bytes > SIZE_MAX / 4) {
    t.workspace_bytes = SIZE_MAX;
    return t;
  }
  t.off_rden = align256(b.workspace_bytes);
  t.off_t = align256(t.off_rden + rden_bytes);
  t.workspace_bytes = t.off_t + t_bytes;
  return t;
}

Check check_backward(const void *Q, const void *K, const void *V, const void *dO, const void *dQ, const void *dK,
                     const void *dV, int B, int H, int N, int C, int M, linattn_dtype dt, const void *workspace,
                     size_t workspace_bytes, size_t workspace_needed) {
  const size_t eb = dtype_bytes(dt);
  if (eb == 0) return fail(LINATTN_ERR_DTYPE, "unknown element type");
  if (B < 0 || H < 0 || N < 0) return fail(LINATTN_ERR_SHAPE, "B, H and N must be non-negative");
  if (C != 64 || M != 64) return fail(LINATTN_ERR_SHAPE, "only C = M = 64 is supported");
  if ((long long)B * (long long)H > INT_MAX) return fail(LINATTN_ERR_SHAPE, "B * H exceeds INT_MAX");
  size_t elems = 0;
  if (!mul3((size_t)B * (size_t)H, (size_t)N, 64, &elems) || elems > SIZE_MAX / eb)
    return fail(LINATTN_ERR_SHAPE, "tensor size overflows");
  if (elems == 0) return Check();
  if (!Q || !K || !V || !dO || !dQ || !dK || !dV)
    return fail(LINATTN_ERR_NULL, "Q, K, V, dO, dQ, dK and dV must be non-NULL");
  for (const void *ptr : {Q, K, V, dO, dQ, dK, dV})
    if (!aligned16(ptr)) return fail(LINATTN_ERR_ALIGN, "Q, K, V, dO, dQ, dK and dV must be 16-byte aligned");
  const size_t bytes = elems * eb;
  const Buffer in[] = {{Q, bytes, "Q"}, {K, bytes, "K"}, {V, bytes, "V"}, {dO, bytes, "dO"}};
  const Buffer out[] = {{dQ, bytes, "dQ"}, {dK, bytes, "dK"}, {dV, bytes, "dV"}};
  for (const Buffer &o : out)
    for (const Buffer &i : in)
      if (overlaps(o, i)) return fail(LINATTN_ERR_ALIAS, std::string(o.name) + " overlaps " + i.name);
  if (overlaps(out[0], out[1]) || overlaps(out[0], out[2]) || overlaps(out[1], out[2]))
    return fail(LINATTN_ERR_ALIAS, "dQ, dK and dV must not overlap");
  if (workspace_needed > 0) {
    if (workspace_needed == SIZE_MAX) return fail(LINATTN_ERR_SHAPE, "workspace size overflows");
    if (workspace == nullptr || workspace_bytes < workspace_needed)
      return fail(LINATTN_ERR_WORKSPACE, "workspace needs " + std::to_string(workspace_needed) + " bytes, got " +
                                             std::to_string(workspace ? workspace_bytes : 0));
    if (!aligned16(workspace)) return fail(LINATTN_ERR_ALIGN, "workspace must be 16-byte aligned");
    const Buffer bw{workspace, workspace_needed, "workspace"};
    for (const Buffer &b : in)
      if (overlaps(bw, b)) return fail(LINATTN_ERR_ALIAS, std::string("workspace overlaps ") + b.name);
    for (const Buffer &b : out)
      if (overlaps(bw, b)) return fail(LINATTN_ERR_ALIAS, std::string("workspace overlaps ") + b.name);
  }
  return Check();
}

Check check_forward(const void *Q, const void *K, const void *V, const void *O, int B, int H, int N, int C, int M,
                    linattn_dtype dt, const void *workspace, size_t workspace_bytes, size_t workspace_needed) {
  const size_t eb = dtype_bytes(dt);
  if (eb == 0) return fail(LINATTN_ERR_DTYPE, "unknown element type");
  if (B < 0 || H < 0 || N < 0) return fail(LINATTN_ERR_SHAPE, "B, H and N must be non-negative");
  if (C != 64 || M != 64) return fail(LINATTN_ERR_SHAPE, "only C = M = 64 is supported");
  if ((long long)B * (long long)H > INT_MAX) return fail(LINATTN_ERR_SHAPE, "B * H exceeds INT_MAX");
  size_t elems = 0;
  if (!mul3((size_t)B * (size_t)H, (size_t)N, 64, &elems) || elems > SIZE_MAX / eb)
    return fail(LINATTN_ERR_SHAPE, "tensor size overflows");
  if (elems == 0) return Check();
  if (!Q || !K || !V || !O) return fail(LINATTN_ERR_NULL, "Q, K, V and O must be non-NULL");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O))
    return fail(LINATTN_ERR_ALIGN, "Q, K, V and O must be 16-byte aligned");
  const size_t bytes = elems * eb;
  const Buffer bq{Q, bytes, "Q"}, bk{K, bytes, "K"}, bv{V, bytes, "V"}, bo{O, bytes, "O"};
  if (overlaps(bo, bq) || overlaps(bo, bk) || overlaps(bo, bv))
    return fail(LINATTN_ERR_ALIAS, "O overlaps Q, K or V");
  if (workspace_needed > 0) {
    if (workspace_needed == SIZE_MAX) return fail(LINATTN_ERR_SHAPE, "workspace size overflows");
    if (workspace == nullptr || workspace_bytes < workspace_needed)
      return fail(LINATTN_ERR_WORKSPACE, "workspace needs " + std::to_string(workspace_needed) + " bytes, got " +
                                             std::to_string(workspace ? workspace_bytes : 0));
    if (!aligned16(workspace)) return fail(LINATTN_ERR_ALIGN, "workspace must be 16-byte aligned");
    const Buffer bw{workspace, workspace_needed, "workspace"};
    if (overlaps(bw, bq) || overlaps(bw, bk) || overlaps(bw, bv) || overlaps(bw, bo))
      return fail(LINATTN_ERR_ALIAS, "workspace overlaps Q, K, V or O");
  }
  return Check();
}

Check check_backward_train(const void *Q, const void *K, const void *V, const void *O, const void *dO,
                           const void *dQ, const void *dK, const void *dV, int B, int H, int N, int C, int M,
                           linattn_dtype dt, const void *workspace, size_t workspace_bytes, size_t workspace_needed) {
  const Check c = check_backward(Q, K, V, dO, dQ, dK, dV, B, H, N, C, M, dt, workspace, workspace_bytes,
                                 workspace_needed);
  if (!c.ok()) return c;
  const size_t bytes = (size_t)B * (size_t)H * (size_t)N * 64 * dtype_bytes(dt);
  if (bytes == 0) return Check();
  if (O == nullptr) return fail(LINATTN_ERR_NULL, "O must be non-NULL");
  if (!aligned16(O)) return fail(LINATTN_ERR_ALIGN, "O must be 16-byte aligned");
  const Buffer bo{O, bytes, "O"};
  const Buffer others[] = {{dQ, bytes, "dQ"}, {dK, bytes, "dK"}, {dV, bytes, "dV"},
                           {workspace, workspace_needed, "workspace"}};
  for (const Buffer &b : others)
    if (overlaps(bo, b)) return fail(LINATTN_ERR_ALIAS, std::string("O overlaps ") + b.name);
  return Check();
}

Check check_state_args(const float *S0, const float *z0, const float *S_out, const float *z_out, int B, int H,
                       const void *Q, const void *K, const void *V, const void *O, size_t qk_bytes,
                       size_t vo_bytes, const void *workspace, size_t workspace_bytes) {
  if ((S0 == nullptr) != (z0 == nullptr)) return fail(LINATTN_ERR_ARG, "give both S0 and z0, or neither");
  if ((S_out == nullptr) != (z_out == nullptr)) return fail(LINATTN_ERR_ARG, "give both S_out and z_out, or neither");
  const size_t heads = (size_t)B * (size_t)H;
  const size_t sb = heads * 4096 * sizeof(float), zb = heads * 64 * sizeof(float);
  if (heads == 0) return Check();
  for (const float *p : {S0, z0, S_out, z_out})
    if (p && !aligned16(p)) return fail(LINATTN_ERR_ALIGN, "state buffers must be 16-byte aligned");
  const Buffer s0{S0, sb, "S0"}, z0b{z0, zb, "z0"}, so{S_out, sb, "S_out"}, zo{z_out, zb, "z_out"};
  if (overlaps(s0, z0b) || overlaps(so, zo) || overlaps(s0, zo) || overlaps(so, z0b))
    return fail(LINATTN_ERR_ALIAS, "S and z buffers overlap");
  // S_out may be S0 itself (in-place), but not a partial overlap.
  if (overlaps(so, s0) && S_out != S0) return fail(LINATTN_ERR_ALIAS, "S_out partially overlaps S0");
  if (overlaps(zo, z0b) && z_out != z0) return fail(LINATTN_ERR_ALIAS, "z_out partially overlaps z0");
  const Buffer io[] = {{Q, qk_bytes, "Q"}, {K, qk_bytes, "K"}, {V, vo_bytes, "V"}, {O, vo_bytes, "O"},
                       {workspace, workspace_bytes, "workspace"}};
  for (const Buffer &b : io)
    for (const Buffer *s : {&s0, &z0b, &so, &zo})
      if (overlaps(*s, b)) return fail(LINATTN_ERR_ALIAS, std::string(s->name) + " overlaps " + b.name);
  return Check();
}

Check check_decode(const float *S, const float *z, const void *q, const void *k, const void *v, const float *o,
                   int BH, int C, int M, linattn_dtype dt, long long stride) {
  const size_t eb = dtype_bytes(dt);
  if (eb == 0) return fail(LINATTN_ERR_DTYPE, "unknown element type");
  if (BH < 0) return fail(LINATTN_ERR_SHAPE, "BH must be non-negative");
  if (C != 64 || M != 64) return fail(LINATTN_ERR_SHAPE, "only C = M = 64 is supported");
  if (stride < 64) return fail(LINATTN_ERR_SHAPE, "the row stride of q, k and v must be at least 64");
  if (stride > (long long)(SIZE_MAX / 16) / (BH > 0 ? BH : 1)) return fail(LINATTN_ERR_SHAPE, "stride overflows");
  if (BH == 0) return Check();
  if (!S || !z || !q || !k || !v || !o) return fail(LINATTN_ERR_NULL, "S, z, q, k, v and o must be non-NULL");
  if ((stride * (long long)eb) % 16 != 0) return fail(LINATTN_ERR_ALIGN, "the row stride must be a multiple of 16 bytes");
  for (const void *p : {(const void *)S, (const void *)z, q, k, v, (const void *)o})
    if (!aligned16(p)) return fail(LINATTN_ERR_ALIGN, "decode buffers must be 16-byte aligned");
  const size_t n = (size_t)BH;
  const Buffer bS{S, n * 4096 * 4, "S"}, bz{z, n * 64 * 4, "z"}, bo{o, n * 64 * 4, "o"};
  const size_t span = ((n - 1) * (size_t)stride + 64) * eb;  // first to last element of the rows
  const Buffer bq{q, span, "q"}, bk{k, span, "k"}, bv{v, span, "v"};
  if (overlaps(bS, bz) || overlaps(bo, bS) || overlaps(bo, bz))
    return fail(LINATTN_ERR_ALIAS, "S, z and o must not overlap");
  for (const Buffer *in : {&bq, &bk, &bv})
    for (const Buffer *st : {&bS, &bz, &bo})
      if (overlaps(*in, *st)) return fail(LINATTN_ERR_ALIAS, std::string(in->name) + " overlaps " + st->name);
  return Check();
}

}  // namespace linattn
