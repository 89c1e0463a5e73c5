// api.hip -- the C ABI of liblinattn.so (declared in include/linattn.h).
//
// Host side only: validate arguments, plan the launch, enqueue kernels on the
// caller's stream.  All arithmetic runs in the kernels of forward_kernels.hpp,
// backward_kernels.hpp and decode_kernel.hpp.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/linattn.h"
#include "backward_kernels.hpp"
#include "backward_saved_kernels.hpp"
#include "decode_kernel.hpp"
#include "forward_kernels.hpp"
#include "validate.hpp"

using namespace linattn;

static_assert(kPlanGroupWaves == kGroupWaves, "planner and kernels agree on the workgroup size");

namespace {

thread_local char g_error[512] = {0};

linattn_status set_status(linattn_status s, const std::string &msg) {
  if (s == LINATTN_OK) {
    g_error[0] = 0;
  } else {
    std::snprintf(g_error, sizeof g_error, "%s: %s", linattn_status_string(s), msg.c_str());
  }
  return s;
}

linattn_status from_check(const Check &c) { return set_status(c.status, c.message); }

// --- device attribute cache -------------------------------------------------
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

int compute_units() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int v = g_cus[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  g_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

std::atomic<int> g_segment_override{0};

// --- kernel timer -----------------------------------------------------------
struct PendingEvent {
  std::string name;
  hipEvent_t start, stop;
};
std::mutex g_timer_mu;
std::atomic<bool> g_timer_on{false};
std::vector<PendingEvent> g_pending;
std::map<std::string, std::pair<double, long>> g_totals;

struct TimerScope {
  bool active = false;
  PendingEvent ev;
  hipStream_t stream;
  TimerScope(const char *name, hipStream_t s) : stream(s) {
    if (!g_timer_on.load(std::memory_order_relaxed)) return;
    ev.name = name;
    // No system-scope fence on recording: the events only timestamp the
    // stream, and a fence per kernel boundary would itself cost microseconds.
    if (hipEventCreateWithFlags(&ev.start, hipEventDisableSystemFence) != hipSuccess) return;
    if (hipEventCreateWithFlags(&ev.stop, hipEventDisableSystemFence) != hipSuccess) {
      (void)hipEventDestroy(ev.start);
      return;
    }
    active = hipEventRecord(ev.start, stream) == hipSuccess;
    if (!active) {
      (void)hipEventDestroy(ev.start);
      (void)hipEventDestroy(ev.stop);
    }
  }
  ~TimerScope() {
    if (!active) return;
    (void)hipEventRecord(ev.stop, stream);
    std::lock_guard<std::mutex> lk(g_timer_mu);
    g_pending.push_back(ev);
  }
};

linattn_status launch_error(const char *what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_status(LINATTN_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return LINATTN_OK;
}

const char *kname(const char *base, linattn_dtype dt) {
  static thread_local std::string s;
  s = std::string(base) + (dt == LINATTN_BF16 ? "_bf16" : "_f32");
  return s.c_str();
}

// A totals pass that reads more than the MI355X's 256 MB last-level cache
// holds uses the streaming load policy (kLoadStreaming); smaller ones keep the
// data cacheable for the walk that re-reads it.
constexpr size_t kLastLevelCacheBytes = size_t(256) << 20;

template <class E> using TotalsKernel = void (*)(FwdParams, int);
template <class E> TotalsKernel<E> totals_kernel(long long heads, long long N) {
  const size_t pass_bytes = (size_t)heads * (size_t)N * 2 * kD * sizeof(E);
  if (std::is_same<E, __bf16>::value && pass_bytes > kLastLevelCacheBytes) return seg_totals_kernel<E, kLoadStreaming>;
  return seg_totals_kernel<E, kLoadDefault>;
}

// One thread per (head, W state elements): W = 4 while that still launches
// 256 blocks or more, else 1; a batch of eight loads for up to eight records.
// kScanGroupedFrom records per head or more go to the grouped scan instead
// (128; a measurement build may set LINATTN_SCAN_GROUPED_FROM lower to compare
// the two forms on fewer records).
#ifndef LINATTN_SCAN_GROUPED_FROM
#define LINATTN_SCAN_GROUPED_FROM 128
#endif
constexpr int kScanGroupedFrom = LINATTN_SCAN_GROUPED_FROM;
static_assert(kScanGroupedFrom >= 1, "grouped scan threshold");

void launch_scan(const FwdParams &p, int mode, hipStream_t stream) {
  const int cnt = mode == kScanTotal ? p.segments : p.segments - 1;
  if (cnt >= kScanGroupedFrom && (long long)p.heads * kScanBlocksPerHead <= INT_MAX) {
    const unsigned blocks = (unsigned)((long long)p.heads * kScanBlocksPerHead);
    hipLaunchKernelGGL(scan_grouped_kernel, dim3(blocks), dim3(256), 0, stream, p, mode);
    return;
  }
  const long long blocks4 = ((long long)p.heads * (kStateFloats / 4) + 255) / 256;
  const long long blocks1 = ((long long)p.heads * kStateFloats + 255) / 256;
  const bool small = p.segments <= kScanBatchSmall;
  if (blocks4 >= 256) {
    const auto fn = small ? scan_kernel<4, kScanBatchSmall> : scan_kernel<4, kScanBatchLarge>;
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks4), dim3(256), 0, stream, p, mode);
  } else {
    const auto fn = small ? scan_kernel<1, kScanBatchSmall> : scan_kernel<1, kScanBatchLarge>;
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks1), dim3(256), 0, stream, p, mode);
  }
}

// Non-causal pass 1: one workgroup per kGroupWaves segments of a head.
template <class E> void launch_group_totals(const FwdParams &p, const Plan &plan, hipStream_t stream) {
  const size_t pass_bytes = (size_t)plan.heads * (size_t)p.N * 2 * kD * sizeof(E);
  const auto fn = std::is_same<E, __bf16>::value && pass_bytes > kLastLevelCacheBytes
                      ? group_totals_kernel<E, kLoadStreaming>
                      : group_totals_kernel<E, kLoadDefault>;
  hipLaunchKernelGGL(fn, dim3((unsigned)plan.heads * (unsigned)plan.groups), dim3(64 * kGroupWaves), 0, stream, p);
}

// Causal passes with at most this many segments per head skip the prefix
// (suffix) scan: each walk wave sums the totals records it needs.
bool sum_in_walk(int segments) { return segments <= kSumInWalkMaxSegments; }

template <class E>
linattn_status run_forward(const FwdParams &base, const Plan &plan, int causal, hipStream_t stream,
                           linattn_dtype dt) {
  FwdParams p = base;
  p.segments = plan.segments;
  p.seg_chunks = plan.seg_chunks;
  p.records = plan.records;
  const unsigned heads = (unsigned)plan.heads;
  if (causal) {
    if (plan.segments > 1) {
      {
        TimerScope t(kname("seg_totals", dt), stream);
        hipLaunchKernelGGL(totals_kernel<E>(plan.heads, p.N), dim3(heads * (unsigned)(plan.segments - 1)), dim3(64), 0,
                           stream,
                           p, plan.segments - 1);
      }
      if (launch_error("seg_totals") != LINATTN_OK) return LINATTN_ERR_HIP;
      // Summing in the walk, every wave reads S0, z0 at its start while the last
      // segment's wave writes S_out, z_out at its end: an in-place call
      // (S_out == S0) takes the scan, which reads S0, z0 in a launch of its own.
      const bool in_place = p.S0 != nullptr && (p.S_out == p.S0 || p.z_out == p.z0);
      if (sum_in_walk(plan.segments) && !in_place) {
        p.init = kInitTotals;
      } else {
        {
          TimerScope t("scan", stream);
          launch_scan(p, kScanPrefix, stream);
        }
        if (launch_error("scan") != LINATTN_OK) return LINATTN_ERR_HIP;
        p.init = kInitRecord;
      }
    } else {
      p.init = p.S0 != nullptr ? kInitNatural : kInitZero;
    }
    if (std::is_same<E, __bf16>::value && p.rden != nullptr) {
      TimerScope t("causal_walk_save_bf16", stream);
      hipLaunchKernelGGL(causal_walk_save_kernel_bf16, dim3(heads * (unsigned)plan.segments), dim3(64), 0, stream, p);
    } else {
      TimerScope t(kname("causal_walk", dt), stream);
      hipLaunchKernelGGL(WalkKernel<E>::fn, dim3(heads * (unsigned)plan.segments), dim3(64), 0, stream, p);
    }
    if (launch_error("causal_walk") != LINATTN_OK) return LINATTN_ERR_HIP;
  } else {
    {
      TimerScope t(kname("group_totals", dt), stream);
      launch_group_totals<E>(p, plan, stream);
    }
    if (launch_error("group_totals") != LINATTN_OK) return LINATTN_ERR_HIP;
    {
      TimerScope t(kname("noncausal_read", dt), stream);
      hipLaunchKernelGGL(noncausal_read_kernel<E>, dim3(heads * (unsigned)plan.range_groups), dim3(64 * kGroupWaves), 0,
                         stream, p, plan.groups, plan.ranges, plan.range_chunks);
    }
    if (launch_error("noncausal_read") != LINATTN_OK) return LINATTN_ERR_HIP;
  }
  return set_status(LINATTN_OK, "");
}

template <class E>
linattn_status run_backward(const BwdParams &base, const BwdPlan &bp, int causal, bool records_ready,
                            hipStream_t stream, linattn_dtype dt) {
  const Plan &plan = bp.fwd;
  BwdParams p = base;
  p.segments = plan.segments;
  p.seg_chunks = plan.seg_chunks;
  p.ranges = plan.ranges;
  p.range_chunks = plan.range_chunks;
  p.recF = plan.records;
  p.recR = bp.recR;
  // The forward's totals and scan kernels produce the (S, z) records.
  FwdParams f{};
  f.Q = p.Q;
  f.K = p.K;
  f.V = p.V;
  f.N = p.N;
  f.heads = p.heads;
  f.segments = plan.segments;
  f.seg_chunks = plan.seg_chunks;
  f.ws = p.wsF;
  f.records = plan.records;
  FwdParams r = f;  // the scan over the (R, r) records
  r.ws = p.wsR;
  r.records = bp.recR;
  const unsigned heads = (unsigned)plan.heads;
  const unsigned P = (unsigned)plan.segments;
  // The same choice as the forward's, whose records linattn_backward_after_forward reuses.
  p.sum_in_walk = causal && sum_in_walk(plan.segments) ? 1 : 0;
  if (causal) {
    if (P > 1 && !records_ready) {
      {
        TimerScope t(kname("seg_totals", dt), stream);
        hipLaunchKernelGGL(totals_kernel<E>(plan.heads, p.N), dim3(heads * (P - 1)), dim3(64), 0, stream, f, (int)P - 1);
      }
      if (launch_error("seg_totals") != LINATTN_OK) return LINATTN_ERR_HIP;
      if (!p.sum_in_walk) {
        {
          TimerScope t("scan", stream);
          launch_scan(f, kScanPrefix, stream);
        }
        if (launch_error("scan") != LINATTN_OK) return LINATTN_ERR_HIP;
      }
    }
    {
      TimerScope t(kname("bwd_walk_f", dt), stream);
      hipLaunchKernelGGL(BwdKernels<E>::walk_f, dim3(heads * P), dim3(64), 0, stream, p);
    }
    if (launch_error("bwd_walk_f") != LINATTN_OK) return LINATTN_ERR_HIP;
    if (P > 1) {
      {
        TimerScope t(kname("bwd_reverse_totals", dt), stream);
        const bool streaming = (size_t)plan.heads * (size_t)p.N * 2 * kD * sizeof(E) > kLastLevelCacheBytes;
        hipLaunchKernelGGL(streaming ? BwdKernels<E>::reverse_totals_streaming : BwdKernels<E>::reverse_totals,
                           dim3(heads * (P - 1)), dim3(64), 0, stream, p);
      }
      if (launch_error("bwd_reverse_totals") != LINATTN_OK) return LINATTN_ERR_HIP;
      if (!p.sum_in_walk) {
        {
          TimerScope t("scan", stream);
          launch_scan(r, kScanSuffix, stream);
        }
        if (launch_error("scan") != LINATTN_OK) return LINATTN_ERR_HIP;
      }
    }
    {
      TimerScope t(kname("bwd_walk_r", dt), stream);
      hipLaunchKernelGGL(BwdKernels<E>::walk_r, dim3(heads * P), dim3(64), 0, stream, p);
    }
    if (launch_error("bwd_walk_r") != LINATTN_OK) return LINATTN_ERR_HIP;
  } else {
    // The head's (S, z) total is record `groups` of wsF: written by the
    // forward's read pass, or here by a total scan over the group records.
    p.segments = plan.groups;
    if (!records_ready) {
      {
        TimerScope t(kname("group_totals", dt), stream);
        launch_group_totals<E>(f, plan, stream);
      }
      if (launch_error("group_totals") != LINATTN_OK) return LINATTN_ERR_HIP;
      FwdParams ft = f;
      ft.segments = plan.groups;
      {
        TimerScope t("scan", stream);
        launch_scan(ft, kScanTotal, stream);
      }
      if (launch_error("scan") != LINATTN_OK) return LINATTN_ERR_HIP;
    }
    {
      TimerScope t(kname("bwd_nc_a", dt), stream);
      hipLaunchKernelGGL(BwdKernels<E>::nc_a, dim3(heads * (unsigned)plan.ranges), dim3(64), 0, stream, p);
    }
    if (launch_error("bwd_nc_a") != LINATTN_OK) return LINATTN_ERR_HIP;
    r.segments = plan.ranges;
    {
      TimerScope t("scan", stream);
      launch_scan(r, kScanTotal, stream);
    }
    if (launch_error("scan") != LINATTN_OK) return LINATTN_ERR_HIP;
    {
      TimerScope t(kname("bwd_nc_b", dt), stream);
      hipLaunchKernelGGL(BwdKernels<E>::nc_b, dim3(heads * (unsigned)plan.ranges), dim3(64), 0, stream, p);
    }
    if (launch_error("bwd_nc_b") != LINATTN_OK) return LINATTN_ERR_HIP;
  }
  return set_status(LINATTN_OK, "");
}

// The bf16 causal backward after linattn_forward_train: saved totals, the
// suffix scan of their records (none with at most kSumInWalkMaxSegments
// segments: the walk sums them), then the one-pass walk.
linattn_status run_saved_backward(const BwdParams &base, const TrainPlan &tp, hipStream_t stream) {
  const Plan &plan = tp.bwd.fwd;
  BwdParams p = base;
  p.segments = plan.segments;
  p.seg_chunks = plan.seg_chunks;
  p.recF = plan.records;
  p.recT = tp.recT;
  p.walk_k = tp.walk_k;
  p.walk_segments = tp.walk_segments;
  p.rev_segments = tp.rev_segments;
  p.rev_chunks = tp.rev_chunks;
  p.sum_in_walk = sum_in_walk(plan.segments) ? 1 : 0;
  p.rev_sum_in_walk = sum_in_walk(tp.rev_segments) ? 1 : 0;
  const unsigned heads = (unsigned)plan.heads;
  {
    TimerScope t("bwd_saved_totals_bf16", stream);
    const bool streaming = (size_t)plan.heads * (size_t)p.N * 3 * kD * sizeof(__bf16) > kLastLevelCacheBytes;
    hipLaunchKernelGGL(streaming ? bwd_saved_totals_kernel<kLoadStreaming> : bwd_saved_totals_kernel<kLoadDefault>,
                       dim3(heads * (unsigned)tp.rev_segments), dim3(64), 0, stream, p);
  }
  if (launch_error("bwd_saved_totals") != LINATTN_OK) return LINATTN_ERR_HIP;
  if (!p.rev_sum_in_walk) {
    FwdParams t{};
    t.N = p.N;
    t.heads = p.heads;
    t.segments = tp.recT;
    t.records = tp.recT;
    t.ws = p.wsT;
    {
      TimerScope ts("scan", stream);
      launch_scan(t, kScanSuffix, stream);
    }
    if (launch_error("scan") != LINATTN_OK) return LINATTN_ERR_HIP;
  }
  {
    TimerScope t("bwd_saved_walk_bf16", stream);
    hipLaunchKernelGGL(bwd_saved_walk_kernel, dim3(heads * (unsigned)tp.walk_segments), dim3(64 * kSavedWaves), 0, stream,
                       p);
  }
  if (launch_error("bwd_saved_walk") != LINATTN_OK) return LINATTN_ERR_HIP;
  return set_status(LINATTN_OK, "");
}

linattn_status backward_impl(const void *Q, const void *K, const void *V, const void *dO, void *dQ, void *dK,
                             void *dV, int B, int H, int N, int C, int M, linattn_dtype dt, int causal,
                             bool records_ready, void *workspace, size_t workspace_bytes, void *stream) {
  const long long heads = (long long)B * (long long)H;
  BwdPlan bp;
  if (B >= 0 && H >= 0 && N >= 0)
    bp = plan_backward(heads, N, causal, (heads > 0 && N > 0) ? compute_units() : 1, g_segment_override.load());
  const Check c = check_backward(Q, K, V, dO, dQ, dK, dV, B, H, N, C, M, dt, workspace, workspace_bytes,
                                 (heads > 0 && N > 0) ? bp.workspace_bytes : 0);
  if (!c.ok()) return from_check(c);
  if (heads == 0 || N == 0) return set_status(LINATTN_OK, "");
  BwdParams p{};
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.dO = dO;
  p.dQ = dQ;
  p.dK = dK;
  p.dV = dV;
  p.N = N;
  p.heads = (int)heads;
  char *ws = reinterpret_cast<char *>(workspace);
  p.wsF = reinterpret_cast<float *>(ws);
  p.wsR = reinterpret_cast<float *>(ws + bp.off_r);
  p.stats = reinterpret_cast<f32x2 *>(ws + bp.off_stats);
  p.stats_stride = bp.stats_stride;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dt == LINATTN_BF16) return run_backward<__bf16>(p, bp, causal, records_ready, s, dt);
  return run_backward<float>(p, bp, causal, records_ready, s, dt);
}

linattn_status forward_train_impl(const void *Q, const void *K, const void *V, void *O, int B, int H, int N, int C,
                                  int M, linattn_dtype dt, int causal, void *workspace, size_t workspace_bytes,
                                  void *stream) {
  const long long heads = (long long)B * (long long)H;
  TrainPlan tp;
  if (B >= 0 && H >= 0 && N >= 0)
    tp = plan_train(heads, N, causal, (heads > 0 && N > 0) ? compute_units() : 1, g_segment_override.load());
  const Check c = check_forward(Q, K, V, O, B, H, N, C, M, dt, workspace, workspace_bytes,
                                (heads > 0 && N > 0) ? tp.workspace_bytes : 0);
  if (!c.ok()) return from_check(c);
  if (heads == 0 || N == 0) return set_status(LINATTN_OK, "");
  FwdParams p{};
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.O = O;
  p.N = N;
  p.heads = (int)heads;
  p.ws = reinterpret_cast<float *>(workspace);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dt == LINATTN_BF16) {
    if (causal) {
      p.rden = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + tp.off_rden);
      p.rden_stride = tp.bwd.stats_stride;
    }
    return run_forward<__bf16>(p, tp.bwd.fwd, causal, s, dt);
  }
  return run_forward<float>(p, tp.bwd.fwd, causal, s, dt);
}

linattn_status backward_train_impl(const void *Q, const void *K, const void *V, const void *O, const void *dO,
                                   void *dQ, void *dK, void *dV, int B, int H, int N, int C, int M, linattn_dtype dt,
                                   int causal, void *workspace, size_t workspace_bytes, void *stream) {
  const long long heads = (long long)B * (long long)H;
  TrainPlan tp;
  if (B >= 0 && H >= 0 && N >= 0)
    tp = plan_train(heads, N, causal, (heads > 0 && N > 0) ? compute_units() : 1, g_segment_override.load());
  const Check c = check_backward_train(Q, K, V, O, dO, dQ, dK, dV, B, H, N, C, M, dt, workspace, workspace_bytes,
                                       (heads > 0 && N > 0) ? tp.workspace_bytes : 0);
  if (!c.ok()) return from_check(c);
  if (heads == 0 || N == 0) return set_status(LINATTN_OK, "");
  BwdParams p{};
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.dO = dO;
  p.dQ = dQ;
  p.dK = dK;
  p.dV = dV;
  p.N = N;
  p.heads = (int)heads;
  char *ws = reinterpret_cast<char *>(workspace);
  p.wsF = reinterpret_cast<float *>(ws);
  p.wsR = reinterpret_cast<float *>(ws + tp.bwd.off_r);
  p.stats = reinterpret_cast<f32x2 *>(ws + tp.bwd.off_stats);
  p.stats_stride = tp.bwd.stats_stride;
  p.O = O;
  p.rden = reinterpret_cast<const float *>(ws + tp.off_rden);
  p.wsT = reinterpret_cast<float *>(ws + tp.off_t);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dt == LINATTN_BF16 && causal) return run_saved_backward(p, tp, s);
  // Other types and the non-causal form: the backward after a forward, on
  // the records the forward left at the same offsets.
  if (dt == LINATTN_BF16) return run_backward<__bf16>(p, tp.bwd, causal, true, s, dt);
  return run_backward<float>(p, tp.bwd, causal, true, s, dt);
}

// Writes S_out/z_out = S0/z0 (or zero) for every head: the N == 0 case of
// linattn_forward_state.
__global__ void state_copy_kernel(const float *S0, const float *z0, float *S_out, float *z_out, long long heads) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < heads * 4096) S_out[i] = S0 ? S0[i] : 0.f;
  if (i < heads * 64) z_out[i] = z0 ? z0[i] : 0.f;
}

}  // namespace

// ---------------------------------------------------------------------------
// Scratch of linattn_forward_noalloc: the forward's segment records live in
// this file-scope device array instead of a caller's workspace.  Every device
// the library runs on holds its own copy until the process ends.  In host code
// `scratch` names a host-side stand-in, not a device address: the device
// address of each device's copy comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is passed on.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[LINATTN_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

linattn_status scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_status(LINATTN_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return set_status(LINATTN_ERR_ARG, "device index beyond the library's table");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return set_status(LINATTN_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LINATTN_OK;
}

linattn_status forward_impl(const void *Q, const void *K, const void *V, void *O, int B, int H, int N, int C, int M,
                            linattn_dtype dt, int causal, const float *S0, const float *z0, float *S_out,
                            float *z_out, void *workspace, size_t workspace_bytes, void *stream) {
  const long long heads = (long long)B * (long long)H;
  Plan plan;
  if (B >= 0 && H >= 0 && N >= 0)
    plan = plan_forward(heads, N, causal, (heads > 0 && N > 0) ? compute_units() : 1, g_segment_override.load());
  const Check c = check_forward(Q, K, V, O, B, H, N, C, M, dt, workspace, workspace_bytes,
                                (heads > 0 && N > 0) ? plan.workspace_bytes : 0);
  if (!c.ok()) return from_check(c);
  const size_t eb = dtype_bytes(dt);
  const size_t tensor_bytes = (size_t)heads * (size_t)N * 64 * eb;
  const Check cs = check_state_args(S0, z0, S_out, z_out, B, H, Q, K, V, O, tensor_bytes, tensor_bytes, workspace,
                                    (heads > 0 && N > 0) ? plan.workspace_bytes : 0);
  if (!cs.ok()) return from_check(cs);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (heads == 0) return set_status(LINATTN_OK, "");
  if (N == 0) {
    if (S_out == nullptr) return set_status(LINATTN_OK, "");
    const long long n = heads * 4096;
    hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, S0, z0, S_out, z_out,
                       heads);
    if (launch_error("state_copy") != LINATTN_OK) return LINATTN_ERR_HIP;
    return set_status(LINATTN_OK, "");
  }
  FwdParams p{};
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.O = O;
  p.N = N;
  p.heads = (int)heads;
  p.ws = reinterpret_cast<float *>(workspace);
  p.S0 = S0;
  p.z0 = z0;
  p.S_out = S_out;
  p.z_out = z_out;
  if (dt == LINATTN_BF16) return run_forward<__bf16>(p, plan, causal, s, dt);
  return run_forward<float>(p, plan, causal, s, dt);
}

}  // namespace

extern "C" {

int linattn_version(void) { return 10000; }

const char *linattn_status_string(linattn_status s) {
  switch (s) {
  case LINATTN_OK: return "LINATTN_OK";
  case LINATTN_ERR_NULL: return "LINATTN_ERR_NULL";
  case LINATTN_ERR_SHAPE: return "LINATTN_ERR_SHAPE";
  case LINATTN_ERR_DTYPE: return "LINATTN_ERR_DTYPE";
  case LINATTN_ERR_ALIGN: return "LINATTN_ERR_ALIGN";
  case LINATTN_ERR_ALIAS: return "LINATTN_ERR_ALIAS";
  case LINATTN_ERR_WORKSPACE: return "LINATTN_ERR_WORKSPACE";
  case LINATTN_ERR_HIP: return "LINATTN_ERR_HIP";
  case LINATTN_ERR_ARG: return "LINATTN_ERR_ARG";
  }
  return "LINATTN_UNKNOWN_STATUS";
}

const char *linattn_last_error(void) { return g_error; }

size_t linattn_forward_workspace_bytes(int B, int H, int N, int C, int M, linattn_dtype dt, int causal) {
  if (B <= 0 || H <= 0 || N <= 0 || C != 64 || M != 64 || dtype_bytes(dt) == 0) return 0;
  const Plan p = plan_forward((long long)B * H, N, causal, compute_units(), g_segment_override.load());
  return p.workspace_bytes == SIZE_MAX ? 0 : p.workspace_bytes;
}

size_t linattn_forward_state_workspace_bytes(int B, int H, int N, int C, int M, linattn_dtype dt) {
  return linattn_forward_workspace_bytes(B, H, N, C, M, dt, 1);
}

linattn_status linattn_forward(const void *Q, const void *K, const void *V, void *O, int B, int H, int N, int C,
                               int M, linattn_dtype dt, int causal, void *workspace, size_t workspace_bytes,
                               void *stream) {
  try {
    return forward_impl(Q, K, V, O, B, H, N, C, M, dt, causal ? 1 : 0, nullptr, nullptr, nullptr, nullptr,
                        workspace, workspace_bytes, stream);
  } catch (...) {
    return set_status(LINATTN_ERR_ARG, "internal exception");
  }
}

linattn_status linattn_forward_state(const void *Q, const void *K, const void *V, void *O, int B, int H, int N,
                                     int C, int M, linattn_dtype dt, const float *S0, const float *z0, float *S_out,
                                     float *z_out, void *workspace, size_t workspace_bytes, void *stream) {
  try {
    return forward_impl(Q, K, V, O, B, H, N, C, M, dt, 1, S0, z0, S_out, z_out, workspace, workspace_bytes, stream);
  } catch (...) {
    return set_status(LINATTN_ERR_ARG, "internal exception");
  }
}

linattn_status linattn_forward_noalloc(const void *Q, const void *K, const void *V, void *O, int B, int H, int N,
                                       int C, int M, linattn_dtype dt, int causal, void *stream) {
  try {
    void *ws = nullptr;
    if (B > 0 && H > 0 && N > 0 && C == 64 && M == 64 && dtype_bytes(dt) != 0) {
      const Plan plan = plan_forward((long long)B * H, N, causal ? 1 : 0, compute_units(), g_segment_override.load());
      if (plan.workspace_bytes != SIZE_MAX && plan.workspace_bytes > (size_t)LINATTN_NOALLOC_SCRATCH_BYTES)
        return set_status(LINATTN_ERR_WORKSPACE, "this problem needs " + std::to_string(plan.workspace_bytes) +
                                                     " bytes of scratch; the static scratch holds " +
                                                     std::to_string((size_t)LINATTN_NOALLOC_SCRATCH_BYTES));
      if (plan.workspace_bytes > 0 && plan.workspace_bytes != SIZE_MAX) {
        const linattn_status st = scratch_address(&ws);
        if (st != LINATTN_OK) return st;
      }
    }
    return forward_impl(Q, K, V, O, B, H, N, C, M, dt, causal ? 1 : 0, nullptr, nullptr, nullptr, nullptr, ws,
                        ws ? (size_t)LINATTN_NOALLOC_SCRATCH_BYTES : 0, stream);
  } catch (...) {
    return set_status(LINATTN_ERR_ARG, "internal exception");
  }
}

size_t linattn_backward_workspace_bytes(int B, int H, int N, int C, int M, linattn_dtype dt, int causal) {
  if (B <= 0 || H <= 0 || N <= 0 || C != 64 || M != 64 || dtype_bytes(dt) == 0) return 0;
  const BwdPlan p = plan_backward((long long)B * H, N, causal, compute_units(), g_segment_override.load());
  return p.workspace_bytes == SIZE_MAX ? 0 : p.workspace_bytes;
}

linattn_status linattn_backward(const void *Q, const void *K, const void *V, const void *dO, void *dQ, void *dK,
                                void *dV, int B, int H, int N, int C, int M, linattn_dtype dt, int causal,
                                void *workspace, size_t workspace_bytes, void *stream) {
  try {
    return backward_impl(Q, K, V, dO, dQ, dK, dV, B, H, N, C, M, dt, causal ? 1 : 0, false, workspace,
                         workspace_bytes, stream);
  } catch (...) {
    return set_status(LINATTN_ERR_ARG, "internal exception");
  }
}

linattn_status linattn_backward_after_forward(const void *Q, const void *K, const void *V, const void *dO, void *dQ,
                                              void *dK, void *dV, int B, int H, int N, int C, int M,
                                              linattn_dtype dt, int causal, void *workspace, size_t workspace_bytes,
                                              void *stream) {
  try {
    return backward_impl(Q, K, V, dO, dQ, dK, dV, B, H, N, C, M, dt, causal ? 1 : 0, true, workspace,
                         workspace_bytes, stream);
  } catch (...) {
    return set_status(LINATTN_ERR_ARG, "internal exception");
  }
}

size_t linattn_train_workspace_bytes(int B, int H, int N, int C, int M, linattn_dtype dt, int causal) {
  if (B <= 0 || H <= 0 || N <= 0 || C != 64 || M != 64 || dtype_bytes(dt) == 0) return 0;
  const TrainPlan p = plan_train((long long)B * H, N, causal, compute_units(), g_segment_override.load());
  return p.workspace_bytes == SIZE_MAX ? 0 : p.workspace_bytes;
}

linattn_status linattn_forward_train(const void *Q, const void *K, const void *V, void *O, int B, int H, int N,
                                     int C, int M, linattn_dtype dt, int causal, void *workspace,
                                     size_t workspace_bytes, void *stream) {
  try {
    return forward_train_impl(Q, K, V, O, B, H, N, C, M, dt, causal ? 1 : 0, workspace, workspace_bytes, stream);
  } catch (...) {
    return set_status(LINATTN_ERR_ARG, "internal exception");
  }
}

linattn_status linattn_backward_train(const void *Q, const void *K, const void *V, const void *O, const void *dO,
                                      void *dQ, void *dK, void *dV, int B, int H, int N, int C, int M,
                                      linattn_dtype dt, int causal, void *workspace, size_t workspace_bytes,
                                      void *stream) {
  try {
    return backward_train_impl(Q, K, V, O, dO, dQ, dK, dV, B, H, N, C, M, dt, causal ? 1 : 0, workspace,
                               workspace_bytes, stream);
  } catch (...) {
    return set_status(LINATTN_ERR_ARG, "internal exception");
  }
}

}  // extern "C"

namespace {
linattn_status decode_impl(float *S, float *z, const void *q, const void *k, const void *v, float *o, int BH, int C,
                           int M, linattn_dtype dt, long long stride, void *stream) {
  const Check c = check_decode(S, z, q, k, v, o, BH, C, M, dt, stride);
  if (!c.ok()) return from_check(c);
  if (BH == 0) return set_status(LINATTN_OK, "");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const unsigned blocks = (unsigned)((BH + 3) / 4);
  {
    TimerScope t(kname("decode_step", dt), s);
    if (dt == LINATTN_BF16) {
      hipLaunchKernelGGL(decode_step_kernel<__bf16>, dim3(blocks), dim3(256), 0, s, S, z,
                         reinterpret_cast<const __bf16 *>(q), reinterpret_cast<const __bf16 *>(k),
                         reinterpret_cast<const __bf16 *>(v), o, BH, stride);
    } else {
      hipLaunchKernelGGL(decode_step_kernel<float>, dim3(blocks), dim3(256), 0, s, S, z,
                         reinterpret_cast<const float *>(q), reinterpret_cast<const float *>(k),
                         reinterpret_cast<const float *>(v), o, BH, stride);
    }
  }
  if (launch_error("decode_step") != LINATTN_OK) return LINATTN_ERR_HIP;
  return set_status(LINATTN_OK, "");
}
}  // namespace

extern "C" {

linattn_status linattn_decode_step(float *S, float *z, const void *q, const void *k, const void *v, float *o, int BH,
                                   int C, int M, linattn_dtype dt, void *stream) {
  try {
    return decode_impl(S, z, q, k, v, o, BH, C, M, dt, 64, stream);
  } catch (...) {
    return set_status(LINATTN_ERR_ARG, "internal exception");
  }
}

linattn_status linattn_decode_step_strided(float *S, float *z, const void *q, const void *k, const void *v, float *o,
                                           int BH, int C, int M, linattn_dtype dt, long long row_stride,
                                           void *stream) {
  try {
    return decode_impl(S, z, q, k, v, o, BH, C, M, dt, row_stride, stream);
  } catch (...) {
    return set_status(LINATTN_ERR_ARG, "internal exception");
  }
}

void linattn_timer_enable(int on) { g_timer_on.store(on != 0); }

void linattn_timer_reset(void) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  for (PendingEvent &e : g_pending) {
    (void)hipEventSynchronize(e.stop);
    (void)hipEventDestroy(e.start);
    (void)hipEventDestroy(e.stop);
  }
  g_pending.clear();
  g_totals.clear();
}

static void timer_drain_locked() {
  for (PendingEvent &e : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(e.stop) == hipSuccess && hipEventElapsedTime(&ms, e.start, e.stop) == hipSuccess) {
      auto &t = g_totals[e.name];
      t.first += ms;
      t.second += 1;
    }
    (void)hipEventDestroy(e.start);
    (void)hipEventDestroy(e.stop);
  }
  g_pending.clear();
}

int linattn_timer_read(const char *kernel, double *total_ms, long *launches) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  timer_drain_locked();
  if (kernel == nullptr) return -1;
  auto it = g_totals.find(kernel);
  if (it == g_totals.end()) return -1;
  if (total_ms) *total_ms = it->second.first;
  if (launches) *launches = it->second.second;
  return 0;
}

size_t linattn_timer_names(char *buf, size_t len) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  timer_drain_locked();
  std::string all;
  for (auto &kv : g_totals) {
    if (!all.empty()) all += ';';
    all += kv.first;
  }
  if (buf && len > 0) {
    const size_t n = all.size() < len - 1 ? all.size() : len - 1;
    std::memcpy(buf, all.data(), n);
    buf[n] = 0;
  }
  return all.size();
}

int linattn_set_segments(int segments_per_head) {
  return g_segment_override.exchange(segments_per_head > 0 ? segments_per_head : 0);
}

int linattn_plan_segments(int B, int H, int N, linattn_dtype dt, int causal) {
  (void)dt;
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  return plan_forward((long long)B * H, N, causal, compute_units(), g_segment_override.load()).segments;
}

}  // extern "C"
