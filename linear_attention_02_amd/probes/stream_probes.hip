// stream_probes.hip -- plain streaming kernels that measure what MI355X
// sustains for the memory access patterns of the attention kernels, so that
// their achieved bandwidth can be compared with a ceiling measured on the
// same device in the same run.  Not part of liblinattn.so; bench.py
// --probes loads libstreamprobes.so and times each probe with HIP events.
//
//   probe_read_lds     reads a buffer through LDS-DMA staging (16-byte
//                      pieces, one 16 KB chunk per wave per step, two chunks
//                      in flight), the way the totals and walk kernels
//                      stage their inputs; default or non-temporal policy.
//   probe_copy         16-byte loads and stores, one read to one write.
//   probe_write        16-byte stores only.
//   probe_mix31        three 16-byte reads to one write per element, the
//                      causal walk's read/write mix (Q, K, V in; O out).
//   probe_mix31_lds    the same mix in the causal walk's structure: 64-token
//                      chunks staged through LDS-DMA, one in flight per
//                      wave, four waves per CU, no arithmetic.
// probe_copy, probe_write and probe_mix31 take a cache policy (plain or
// non-temporal loads and stores) and a workgroup count, so that the caller
// can keep the best.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kChunkVec = 1024;  // 16 KB per chunk: 16 load instructions of 64 x 16 B
constexpr int kWaves = 1024;     // one wave per workgroup, four per CU on 256 CUs

template <int N> __device__ inline void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wave w reads chunks w, w + kWaves, ... of the buffer (`chunks` of 16 KB),
// two in flight, and folds one word per chunk into its result (so that the
// LDS contents are consumed).
template <int kPolicy>
__global__ __launch_bounds__(64) void read_lds_kernel(const u32x4 *src, long long chunks, uint32_t *out) {
  __shared__ u32x4 slot[2][kChunkVec];
  const int lane = threadIdx.x;
  auto issue = [&](long long c, int b) {
    const u32x4 *p = src + c * kChunkVec;
#pragma unroll
    for (int i = 0; i < kChunkVec / 64; ++i)
      __builtin_amdgcn_global_load_lds(p + i * 64 + lane, (lds_void *)(&slot[b][i * 64]), 16, 0, kPolicy);
  };
  uint32_t acc = 0;
  long long c = blockIdx.x;
  int b = 0;
  if (c < chunks) issue(c, 0);
  if (c + kWaves < chunks) issue(c + kWaves, 1);
  for (; c < chunks; c += kWaves, b ^= 1) {
    if (c + kWaves < chunks) {
      wait_vmcnt<kChunkVec / 64>();  // the older chunk has landed
    } else {
      wait_vmcnt<0>();
    }
    // One word of the chunk, read from inline assembly: a compiler-visible
    // LDS read after LDS-DMA loads would make it wait for the newer chunk too.
    const uint32_t addr = (uint32_t)(size_t)(lds_void *)&slot[b][lane];
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr));
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v) : : "memory");  // read before the refill
    acc ^= v;
    if (c + 2 * kWaves < chunks) issue(c + 2 * kWaves, b);
  }
  if (acc == 0x9e3779b9u) out[blockIdx.x] = acc;  // keeps the reads live
}

// The causal walk's memory structure without its arithmetic: one wave per
// workgroup and four per CU (the 40 KB of LDS each takes leaves room for no
// fifth), each wave streaming a contiguous range of 64-token chunks.  A chunk
// is 8 KB of each of three inputs, staged through LDS-DMA into one 24 KB
// slot; the wave waits for it, reads it into registers, issues the next
// chunk's loads into the same slot, and writes the chunk's 8 KB output (the
// XOR of the three inputs) with non-temporal stores.  One chunk is in flight
// per wave while the previous one is written, as in the walk.
constexpr int kStreamVec = 512;  // 8 KB of one input per chunk
__global__ __launch_bounds__(64) void mix31_lds_kernel(const u32x4 *a, const u32x4 *b, const u32x4 *c, u32x4 *d,
                                                       long long chunks) {
  __shared__ u32x4 slot[2560];  // 24 KB used, 40 KB held
  const int lane = threadIdx.x;
  const long long per = (chunks + gridDim.x - 1) / gridDim.x;
  const long long c0 = (long long)blockIdx.x * per;
  const long long c1 = c0 + per < chunks ? c0 + per : chunks;
  auto issue = [&](long long ch) {
    const u32x4 *src[3] = {a + ch * kStreamVec, b + ch * kStreamVec, c + ch * kStreamVec};
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
      for (int i = 0; i < kStreamVec / 64; ++i)
        __builtin_amdgcn_global_load_lds(src[s] + i * 64 + lane, (lds_void *)(&slot[s * kStreamVec + i * 64]), 16,
                                         0, 0);
  };
  if (c0 < c1) issue(c0);
  for (long long ch = c0; ch < c1; ++ch) {
    wait_vmcnt<0>();  // this chunk has landed (and the previous chunk's stores have gone out)
    u32x4 x[kStreamVec / 64];
#pragma unroll
    for (int i = 0; i < kStreamVec / 64; ++i) {
      const uint32_t base = (uint32_t)(size_t)(lds_void *)&slot[i * 64 + lane];
      u32x4 p, q, r;
      asm volatile("ds_read_b128 %0, %1" : "=v"(p) : "v"(base));
      asm volatile("ds_read_b128 %0, %1" : "=v"(q) : "v"(base + 16 * kStreamVec));
      asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(base + 32 * kStreamVec));
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(p), "+v"(q), "+v"(r) : : "memory");
      x[i] = p ^ q ^ r;
    }
    if (ch + 1 < c1) issue(ch + 1);  // the slot has been read
    u32x4 *out = d + ch * kStreamVec;
#pragma unroll
    for (int i = 0; i < kStreamVec / 64; ++i) __builtin_nontemporal_store(x[i], out + i * 64 + lane);
  }
}

// The element probes give each workgroup one contiguous range of the
// buffers (a grid-stride order, where neighbouring workgroups touch
// neighbouring addresses at once, streams about 20% slower here).  Each
// thread takes kUnroll elements 256 apart per step, all loads issued before
// the stores.  kPolicy bit 0: non-temporal loads; bit 1: non-temporal stores.
constexpr int kUnroll = 4;
constexpr int kMaxBlocks = 65536;

template <int kPolicy> __device__ inline u32x4 load16(const u32x4 *p) {
  if (kPolicy & 1) return __builtin_nontemporal_load(p);
  return *p;
}

template <int kPolicy> __device__ inline void store16(u32x4 v, u32x4 *p) {
  if (kPolicy & 2) {
    __builtin_nontemporal_store(v, p);
  } else {
    *p = v;
  }
}

// [begin, end) of this workgroup's range of n elements.
__device__ inline void block_range(long long n, long long &begin, long long &end) {
  const long long per = (n + gridDim.x - 1) / gridDim.x;
  begin = (long long)blockIdx.x * per;
  end = begin + per < n ? begin + per : n;
}

template <int kPolicy>
__global__ __launch_bounds__(256) void copy_kernel(const u32x4 *src, u32x4 *dst, long long n) {
  long long b0, e;
  block_range(n, b0, e);
  for (long long i = b0 + threadIdx.x; i < e; i += kUnroll * 256) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (i + u * 256 < e) v[u] = load16<kPolicy>(src + i + u * 256);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (i + u * 256 < e) store16<kPolicy>(v[u], dst + i + u * 256);
  }
}

template <int kPolicy> __global__ __launch_bounds__(256) void write_kernel(u32x4 *dst, long long n) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  long long b0, e;
  block_range(n, b0, e);
  for (long long i = b0 + threadIdx.x; i < e; i += kUnroll * 256)
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (i + u * 256 < e) store16<kPolicy>(z, dst + i + u * 256);
}

template <int kPolicy>
__global__ __launch_bounds__(256) void mix31_kernel(const u32x4 *a, const u32x4 *b, const u32x4 *c, u32x4 *d,
                                                    long long n) {
  long long b0, e;
  block_range(n, b0, e);
  for (long long i = b0 + threadIdx.x; i < e; i += kUnroll * 256) {
    u32x4 x[kUnroll], y[kUnroll], w[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (i + u * 256 < e) {
        x[u] = load16<kPolicy>(a + i + u * 256);
        y[u] = load16<kPolicy>(b + i + u * 256);
        w[u] = load16<kPolicy>(c + i + u * 256);
      }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (i + u * 256 < e) store16<kPolicy>(x[u] ^ y[u] ^ w[u], d + i + u * 256);
  }
}

}  // namespace

extern "C" {

// bytes: a multiple of 16 KB (read) or 16 B (others); buffers 16-byte
// aligned.  Returns 0, or -1 for an argument the probe cannot take, or the
// HIP error of the launch.
int probe_read_lds(const void *src, long long bytes, int streaming, uint32_t *scratch, void *stream) {
  if (src == nullptr || scratch == nullptr || bytes <= 0 || bytes % (16 * kChunkVec) != 0) return -1;
  const long long chunks = bytes / (16 * kChunkVec);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (streaming) {
    hipLaunchKernelGGL(read_lds_kernel<2>, dim3(kWaves), dim3(64), 0, s, reinterpret_cast<const u32x4 *>(src), chunks,
                       scratch);
  } else {
    hipLaunchKernelGGL(read_lds_kernel<0>, dim3(kWaves), dim3(64), 0, s, reinterpret_cast<const u32x4 *>(src), chunks,
                       scratch);
  }
  return (int)hipGetLastError();
}

// policy: bit 0 non-temporal loads, bit 1 non-temporal stores (the write
// probe uses bit 1 only).  blocks: workgroups of 256, 1..65536.
#define LINATTN_PROBE_POLICY_SWITCH(kernel, ...)                                                              \
  switch (policy) {                                                                                            \
  case 0: hipLaunchKernelGGL(kernel<0>, dim3(blocks), dim3(256), 0, s, __VA_ARGS__); break;                  \
  case 1: hipLaunchKernelGGL(kernel<1>, dim3(blocks), dim3(256), 0, s, __VA_ARGS__); break;                  \
  case 2: hipLaunchKernelGGL(kernel<2>, dim3(blocks), dim3(256), 0, s, __VA_ARGS__); break;                  \
  default: hipLaunchKernelGGL(kernel<3>, dim3(blocks), dim3(256), 0, s, __VA_ARGS__); break;                 \
  }

int probe_copy(const void *src, void *dst, long long bytes, int policy, int blocks, void *stream) {
  if (src == nullptr || dst == nullptr || bytes <= 0 || bytes % 16 != 0 || policy < 0 || policy > 3 || blocks < 1 ||
      blocks > kMaxBlocks)
    return -1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  LINATTN_PROBE_POLICY_SWITCH(copy_kernel, reinterpret_cast<const u32x4 *>(src), reinterpret_cast<u32x4 *>(dst),
                              bytes / 16)
  return (int)hipGetLastError();
}

int probe_write(void *dst, long long bytes, int policy, int blocks, void *stream) {
  if (dst == nullptr || bytes <= 0 || bytes % 16 != 0 || policy < 0 || policy > 3 || blocks < 1 ||
      blocks > kMaxBlocks)
    return -1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  LINATTN_PROBE_POLICY_SWITCH(write_kernel, reinterpret_cast<u32x4 *>(dst), bytes / 16)
  return (int)hipGetLastError();
}

// The walk-shaped 3:1 mix: each of a, b, c, d holds `bytes_each`, a
// multiple of 8 KB; `waves` one-wave workgroups, 1..65536.
int probe_mix31_lds(const void *a, const void *b, const void *c, void *d, long long bytes_each, int waves,
                    void *stream) {
  if (a == nullptr || b == nullptr || c == nullptr || d == nullptr || bytes_each <= 0 ||
      bytes_each % (16 * kStreamVec) != 0 || waves < 1 || waves > kMaxBlocks)
    return -1;
  hipLaunchKernelGGL(mix31_lds_kernel, dim3(waves), dim3(64), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const u32x4 *>(a), reinterpret_cast<const u32x4 *>(b),
                     reinterpret_cast<const u32x4 *>(c), reinterpret_cast<u32x4 *>(d),
                     bytes_each / (16 * kStreamVec));
  return (int)hipGetLastError();
}

// Each of a, b, c, d holds `bytes_each`.
int probe_mix31(const void *a, const void *b, const void *c, void *d, long long bytes_each, int policy, int blocks,
                void *stream) {
  if (a == nullptr || b == nullptr || c == nullptr || d == nullptr || bytes_each <= 0 || bytes_each % 16 != 0 ||
      policy < 0 || policy > 3 || blocks < 1 || blocks > kMaxBlocks)
    return -1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  LINATTN_PROBE_POLICY_SWITCH(mix31_kernel, reinterpret_cast<const u32x4 *>(a), reinterpret_cast<const u32x4 *>(b),
                              reinterpret_cast<const u32x4 *>(c), reinterpret_cast<u32x4 *>(d), bytes_each / 16)
  return (int)hipGetLastError();
}

}  // extern "C"
