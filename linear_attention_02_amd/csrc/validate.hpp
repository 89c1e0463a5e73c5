// validate.hpp -- argument checks and launch planning for liblinattn, in plain
// C++ with no HIP dependency, so the host logic can be built and tested
// without a GPU (and under host sanitizers).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "../../include/linattn.h"

namespace linattn {

struct Buffer {
  const void *ptr;
  size_t bytes;
  const char *name;
};

// Result of a check: status plus message for linattn_last_error().
struct Check {
  linattn_status status = LINATTN_OK;
  std::string message;
  bool ok() const { return status == LINATTN_OK; }
};

size_t dtype_bytes(linattn_dtype dt);  // 0 for an unknown type

// Launch plan for one forward call.
// Waves per workgroup of the non-causal kernels: one head's consecutive
// segments (ranges) share a workgroup.
constexpr int kPlanGroupWaves = 4;

struct Plan {
  long long heads = 0;      // B * H
  long long chunks = 0;     // ceil(N / 64)
  int segments = 1;         // sequence segments per head (scan units)
  int seg_chunks = 0;       // chunks per segment
  int records = 0;          // state records per head in the workspace
  int groups = 0;           // non-causal: totals workgroups per head (records 0..groups-1; the
                            // head's total is record `groups`)
  int ranges = 0;           // non-causal read ranges per head
  int range_chunks = 0;     // chunks per read range
  int range_groups = 0;     // non-causal read workgroups per head
  size_t workspace_bytes = 0;
};

// Plans a forward call.  `cus` is the device's compute-unit count, `override`
// a forced segment count (0 = automatic).
Plan plan_forward(long long heads, long long N, int causal, int cus, int override_segments);

Check check_forward(const void *Q, const void *K, const void *V, const void *O, int B, int H, int N, int C, int M,
                    linattn_dtype dt, const void *workspace, size_t workspace_bytes, size_t workspace_needed);

// Launch plan for one backward call: the forward plan's segments and ranges,
// plus the workspace layout [records of (S, z)] [records of (R, r)] [per-token
// pairs (1/den, b)], each region 256-byte aligned.
struct BwdPlan {
  Plan fwd;
  int recR = 0;                  // reverse-direction records per head
  long long stats_stride = 0;    // pairs per head (N rounded up to 64)
  size_t off_r = 0;              // byte offset of the reverse records
  size_t off_stats = 0;          // byte offset of the pairs
  size_t workspace_bytes = 0;
};

BwdPlan plan_backward(long long heads, long long N, int causal, int cus, int override_segments);

// Launch plan of the forward/backward pair that saves 1/den: the backward
// plan's layout, then [1/den per token] [suffix records], each region
// 256-byte aligned.  The saved-forward walk covers walk_k consecutive forward
// segments per workgroup, so that its segment starts are forward segment
// starts (where the forward's records give the prefix state).
constexpr int kTrainWalkGroupsPerCU = 1;

// The suffix state (R, r) of the saved-forward walk is carried by
// subtraction from an exact suffix sum at each reverse-segment start (an
// anchor).  The rounding left over at a token is about 2^-24 of the largest
// sum since its anchor, while the true suffix near the end of a sequence is a
// few tokens' terms, and 1/den_i falls off like 1/i; so the last reverse
// segment must not start near the beginning.  Reverse segments are the
// forward segments, except that a one-segment plan of kTrainSplitFrom chunks
// or more is split in two.
constexpr long long kTrainSplitFrom = 4;

struct TrainPlan {
  BwdPlan bwd;
  int walk_k = 1;            // forward segments per walk segment
  int walk_segments = 0;     // walk segments per head
  int rev_segments = 0;      // reverse segments per head (anchors of the suffix state)
  int rev_chunks = 0;        // chunks per reverse segment
  int recT = 0;              // suffix records per head (reverse segments + 1)
  size_t off_rden = 0;       // byte offset of 1/den (stats_stride floats per head)
  size_t off_t = 0;          // byte offset of the suffix records
  size_t workspace_bytes = 0;
};

TrainPlan plan_train(long long heads, long long N, int causal, int cus, int override_segments);

// Q, K, V, dO inputs and dQ, dK, dV outputs, all [B,H,N,64] in `dt`.
Check check_backward(const void *Q, const void *K, const void *V, const void *dO, const void *dQ, const void *dK,
                     const void *dV, int B, int H, int N, int C, int M, linattn_dtype dt, const void *workspace,
                     size_t workspace_bytes, size_t workspace_needed);

// check_backward plus the forward output O that linattn_backward_train reads:
// non-NULL, 16-byte aligned, the size of Q, and disjoint from dQ, dK, dV and
// the workspace.
Check check_backward_train(const void *Q, const void *K, const void *V, const void *O, const void *dO,
                           const void *dQ, const void *dK, const void *dV, int B, int H, int N, int C, int M,
                           linattn_dtype dt, const void *workspace, size_t workspace_bytes, size_t workspace_needed);

Check check_state_args(const float *S0, const float *z0, const float *S_out, const float *z_out, int B, int H,
                       const void *Q, const void *K, const void *V, const void *O, size_t qk_bytes,
                       size_t vo_bytes, const void *workspace, size_t workspace_bytes);

// q, k, v rows of consecutive heads are `stride` elements apart (>= 64).
Check check_decode(const float *S, const float *z, const void *q, const void *k, const void *v, const float *o,
                   int BH, int C, int M, linattn_dtype dt, long long stride = 64);

bool overlaps(const Buffer &a, const Buffer &b);

}  // namespace linattn
