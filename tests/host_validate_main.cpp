// Host-only driver for validate.cpp: exercises the argument checks and the
// planner without HIP, so they can run under AddressSanitizer and UBSan.
#include <climits>
#include <cstdio>
#include <cstdlib>

#include "../linear_attention_02_amd/csrc/validate.hpp"

using namespace linattn;

static int failures = 0;

#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::printf("FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);   \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static const void *P(unsigned long v) { return reinterpret_cast<const void *>(v); }

int main() {
  // Planner.
  Plan p = plan_forward(16, 131072, 1, 256, 0);
  EXPECT(p.segments == 64 && p.seg_chunks == 32 && p.records == 64);
  EXPECT(p.workspace_bytes == (size_t)16 * 64 * 4160 * 4);
  p = plan_forward(128, 3072, 1, 256, 0);
  EXPECT(p.segments == 8 && p.seg_chunks == 6);
  p = plan_forward(64, 4096, 0, 256, 0);
  // Non-causal: 16 segments summed by 4 workgroups (one record each), then the total.
  EXPECT(p.segments == 16 && p.groups == 4 && p.records == 5 && p.ranges == 16 && p.range_chunks == 4 &&
         p.range_groups == 4);
  EXPECT(p.workspace_bytes == (size_t)64 * 5 * 4160 * 4);
  p = plan_forward(3, 64 * 10, 0, 256, 7);  // 7 segments: groups of 4 and 3
  EXPECT(p.segments == 5 || p.segments == 7);
  EXPECT(p.groups == (p.segments + 3) / 4 && p.records == p.groups + 1);
  // Few heads, short sequences: segments shorter than 4 chunks (down to one)
  // where longer ones would leave the device short of waves, at most 64.
  p = plan_forward(1, 65, 1, 256, 0);  // two chunks
  EXPECT(p.segments == 2 && p.seg_chunks == 1 && p.records == 2 && p.workspace_bytes == (size_t)2 * 4160 * 4);
  p = plan_forward(8, 512, 1, 256, 0);
  EXPECT(p.segments == 8 && p.seg_chunks == 1);
  p = plan_forward(8, 8192, 1, 256, 0);
  EXPECT(p.segments == 64 && p.seg_chunks == 2);
  p = plan_forward(8, 16384, 1, 256, 0);  // 4-chunk segments already fill the device
  EXPECT(p.segments == 64 && p.seg_chunks == 4);
  p = plan_forward(1, 1 << 20, 1, 256, 0);
  EXPECT(p.segments == 1024 && p.seg_chunks == 16);
  p = plan_forward(1, 64, 1, 256, 0);  // one chunk: one segment, no records
  EXPECT(p.segments == 1 && p.records == 0 && p.workspace_bytes == 0);
  p = plan_forward(1 << 24, 64 * 1000, 1, 256, 1000);  // override: the grid stays within INT_MAX waves
  EXPECT((long long)p.segments * (1 << 24) <= INT_MAX && p.segments >= 1);
  p = plan_forward(1, 64 * 10, 1, 256, 4);  // override
  EXPECT(p.segments == 4 && p.seg_chunks == 3);
  p = plan_forward(1, 64 * 10, 1, 256, 1000);  // override capped at the chunk count
  EXPECT(p.segments == 10 && p.seg_chunks == 1);
  p = plan_forward(0, 100, 1, 256, 0);
  EXPECT(p.workspace_bytes == 0);
  // Every planned segment is non-empty and the segments cover the sequence.
  for (long long N = 1; N < 5000; N += 97)
    for (int ovr = 0; ovr < 9; ++ovr) {
      Plan q = plan_forward(3, N, 1, 256, ovr);
      EXPECT((long long)(q.segments - 1) * q.seg_chunks < q.chunks);
      EXPECT((long long)q.segments * q.seg_chunks >= q.chunks);
    }

  // Forward checks.
  EXPECT(check_forward(P(0x10000), P(0x20000), P(0x30000), P(0x40000), 1, 1, 64, 64, 64, LINATTN_BF16, nullptr, 0,
                       0).ok());
  EXPECT(check_forward(nullptr, P(32), P(48), P(64), 1, 1, 64, 64, 64, LINATTN_BF16, nullptr, 0, 0).status ==
         LINATTN_ERR_NULL);
  EXPECT(check_forward(P(16), P(32), P(48), P(64), 1, 1, 64, 64, 32, LINATTN_BF16, nullptr, 0, 0).status ==
         LINATTN_ERR_SHAPE);
  EXPECT(check_forward(P(16), P(32), P(48), P(64), 1, 1, 64, 64, 64, (linattn_dtype)9, nullptr, 0, 0).status ==
         LINATTN_ERR_DTYPE);
  EXPECT(check_forward(P(0x10000), P(0x20000), P(0x30000), P(0x30010), 1, 1, 64, 64, 64, LINATTN_BF16, nullptr, 0,
                       0).status == LINATTN_ERR_ALIAS);
  EXPECT(check_forward(P(0x10000), P(0x20000), P(0x30000), P(0x40000), 1, 1, 64, 64, 64, LINATTN_BF16, nullptr, 0,
                       100).status == LINATTN_ERR_WORKSPACE);
  EXPECT(check_forward(P(0x10000), P(0x20000), P(0x30000), P(0x40000), 1, 1, 64, 64, 64, LINATTN_BF16, P(0x50000),
                       100, 100).ok());
  EXPECT(check_forward(P(16), P(32), P(48), P(64), 1 << 20, 1 << 20, 64, 64, 64, LINATTN_BF16, nullptr, 0, 0).status ==
         LINATTN_ERR_SHAPE);
  EXPECT(check_forward(P(16), P(32), P(48), P(64), 0x7fffffff, 0x7fffffff, 0x7fffffff, 64, 64, LINATTN_F32,
                       nullptr, 0, 0).status == LINATTN_ERR_SHAPE);

  // Decode checks.
  const float *S = (const float *)P(0x100000), *z = (const float *)P(0x200000), *o = (const float *)P(0x300000);
  EXPECT(check_decode(S, z, P(0x400000), P(0x500000), P(0x600000), o, 8, 64, 64, LINATTN_F32).ok());
  EXPECT(check_decode(S, S + 16, P(0x400000), P(0x500000), P(0x600000), o, 8, 64, 64, LINATTN_F32).status ==
         LINATTN_ERR_ALIAS);
  EXPECT(check_decode(S, z, P(0x400000), P(0x500000), P(0x600000), z, 8, 64, 64, LINATTN_F32).status ==
         LINATTN_ERR_ALIAS);

  // Strided decode: row stride, its alignment, and the span of strided rows.
  EXPECT(check_decode(S, z, P(0x400000), P(0x400080), P(0x400100), o, 8, 64, 64, LINATTN_BF16, 192).ok());
  EXPECT(check_decode(S, z, P(0x400000), P(0x400080), P(0x400100), o, 8, 64, 64, LINATTN_BF16, 32).status ==
         LINATTN_ERR_SHAPE);
  EXPECT(check_decode(S, z, P(0x400000), P(0x400080), P(0x400100), o, 8, 64, 64, LINATTN_BF16, 100).status ==
         LINATTN_ERR_ALIGN);
  // 8 heads x 192 bf16 = 3 KB of rows from q: o placed 2 KB after q overlaps them.
  EXPECT(check_decode(S, z, P(0x400000), P(0x400080), P(0x400100), (const float *)P(0x400800), 8, 64, 64,
                      LINATTN_BF16, 192).status == LINATTN_ERR_ALIAS);
  EXPECT(check_decode(S, z, P(0x400000), P(0x400080), P(0x400100), o, 8, 64, 64, LINATTN_BF16, 1LL << 62).status ==
         LINATTN_ERR_SHAPE);

  // Backward plan: two record sets and the per-token pairs, each 256-byte aligned.
  {
    BwdPlan b = plan_backward(16, 131072, 1, 256, 0);
    EXPECT(b.fwd.segments == 64 && b.recR == 64 && b.stats_stride == 131072);
    EXPECT(b.off_r % 256 == 0 && b.off_stats % 256 == 0 && b.off_r >= b.fwd.workspace_bytes);
    EXPECT(b.workspace_bytes == b.off_stats + (size_t)16 * 131072 * 8);
    b = plan_backward(4, 100, 1, 256, 0);  // ragged N: pairs padded to whole chunks
    EXPECT(b.stats_stride == 128);
    b = plan_backward(64, 4096, 0, 256, 0);  // non-causal: ranges + 1 reverse records
    EXPECT(b.recR == b.fwd.ranges + 1);
    b = plan_backward(1, 64, 1, 256, 0);  // one segment: no records, pairs only
    EXPECT(b.fwd.records == 0 && b.recR == 0 && b.workspace_bytes == b.off_stats + 64 * 8);
  }
  // Backward argument checks.
  EXPECT(check_backward(P(0x10000), P(0x20000), P(0x30000), P(0x40000), P(0x50000), P(0x60000), P(0x70000), 1, 1, 64,
                        64, 64, LINATTN_BF16, nullptr, 0, 0).ok());
  EXPECT(check_backward(P(0x10000), P(0x20000), P(0x30000), P(0x40000), P(0x50000), P(0x60000), P(0x50010), 1, 1, 64,
                        64, 64, LINATTN_BF16, nullptr, 0, 0).status == LINATTN_ERR_ALIAS);
  EXPECT(check_backward(P(0x10000), P(0x20000), P(0x30000), P(0x40000), P(0x40000), P(0x60000), P(0x70000), 1, 1, 64,
                        64, 64, LINATTN_BF16, nullptr, 0, 0).status == LINATTN_ERR_ALIAS);
  EXPECT(check_backward(P(0x10000), P(0x20000), P(0x30000), P(0x40000), P(0x50000), P(0x60000), P(0x70000), 1, 1, 64,
                        64, 64, LINATTN_BF16, P(0x80000), 99, 100).status == LINATTN_ERR_WORKSPACE);
  EXPECT(check_backward(P(0x10000), P(0x20000), P(0x30000), P(0x40000), P(0x50000), P(0x60000), P(0x70000), 1, 1, 64,
                        64, 64, LINATTN_BF16, P(0x61000), 4096, 4096).status == LINATTN_ERR_ALIAS);
  EXPECT(check_backward(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 8, 64, 64, 64,
                        LINATTN_BF16, nullptr, 0, 0).ok());

  // Overlap helper.
  EXPECT(overlaps({P(100), 10, "a"}, {P(109), 1, "b"}));
  EXPECT(!overlaps({P(100), 10, "a"}, {P(110), 1, "b"}));
  EXPECT(!overlaps({P(100), 0, "a"}, {P(100), 1, "b"}));

  if (failures == 0) std::printf("all host validation checks passed\n");
  return failures == 0 ? 0 : 1;
}
