// decode_kernel.hpp -- one recurrent decode step for many independent heads.
//
// Per head ("Why Replace Attention?", §7.2 steps 1-4; constant work per step,
// §7.4):  S += phi(k) v^T,  z += phi(k),  o = phi(q)^T S / phi(q)^T z,
// reading the state after the update.
//
// One wave64 owns one head; a 256-thread workgroup holds four heads.  The
// 64x64 fp32 state is 16 KB per head and is read and written once per step,
// so the step is bound by memory traffic (about 0.5 flop per byte).  Lane
// (m4, cq) = (l & 15, l >> 4) holds columns 4*m4..4*m4+3 of rows 16*cq..16*cq+15,
// so each 16-byte load or store instruction covers four whole 256-byte rows.
// The column sums phi(q)^T S are reduced across the four row groups with
// cross-lane shuffles; phi(q)^T z with a full-wave reduction.  The q, k and v
// vectors of consecutive heads are `stride` elements apart (64 when they are
// packed; larger when they are column slices of one projection output).
#pragma once

#include "device_common.hpp"

namespace linattn {

template <class E> __device__ inline float load_elem(const E *p, int i);
template <> __device__ inline float load_elem<float>(const float *p, int i) { return p[i]; }
template <> __device__ inline float load_elem<__bf16>(const __bf16 *p, int i) {
  return __uint_as_float((uint32_t)(reinterpret_cast<const uint16_t *>(p)[i]) << 16);
}

// Elements 16c .. 16c + 15 of a 64-element row as fp32, in 16-byte loads
// (four for fp32, two for bf16).  Rows are 16-byte aligned.
template <class E> __device__ inline void load16(const E *row, int c, float out[16]);
template <> __device__ inline void load16<float>(const float *row, int c, float out[16]) {
  const f32x4 *p = reinterpret_cast<const f32x4 *>(row) + 4 * c;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 x = p[i];
#pragma unroll
    for (int r = 0; r < 4; ++r) out[4 * i + r] = x[r];
  }
}
template <> __device__ inline void load16<__bf16>(const __bf16 *row, int c, float out[16]) {
  const u32x4 *p = reinterpret_cast<const u32x4 *>(row) + 2 * c;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const u32x4 x = p[i];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      out[8 * i + 2 * r] = bf16_lo(x[r]);
      out[8 * i + 2 * r + 1] = bf16_hi(x[r]);
    }
  }
}

// Elements 4c .. 4c + 3 (one 16-byte fp32 load, one 8-byte bf16 load).
template <class E> __device__ inline f32x4 load4(const E *row, int c);
template <> __device__ inline f32x4 load4<float>(const float *row, int c) {
  return reinterpret_cast<const f32x4 *>(row)[c];
}
template <> __device__ inline f32x4 load4<__bf16>(const __bf16 *row, int c) {
  const u32x2 x = reinterpret_cast<const u32x2 *>(row)[c];
  return f32x4{bf16_lo(x[0]), bf16_hi(x[0]), bf16_lo(x[1]), bf16_hi(x[1])};
}

template <class E>
__global__ __launch_bounds__(256) void decode_step_kernel(float *__restrict__ S, float *__restrict__ z,
                                                          const E *__restrict__ q, const E *__restrict__ k,
                                                          const E *__restrict__ v, float *__restrict__ o,
                                                          int heads, long long stride) {
  const int h = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (h >= heads) return;
  const int lane = threadIdx.x & 63;
  const int m4 = lane & 15, cq = lane >> 4;

  const E *qh = q + (long long)h * stride;
  const E *kh = k + (long long)h * stride;
  const E *vh = v + (long long)h * stride;
  float4 *Sh = reinterpret_cast<float4 *>(S + (long long)h * kD * kD);

  // q, k for this lane's 16 rows; v for its 4 columns.
  float qr[16], pk[16], pq[16];
  load16<E>(qh, cq, qr);
  load16<E>(kh, cq, pk);
  const f32x4 vv = load4<E>(vh, m4);
  const float v0 = vv[0], v1 = vv[1], v2 = vv[2], v3 = vv[3];
  // phi(q) scaled by the power of two phi_row_scale picks from the largest
  // of the 64 features (the same for the whole wave; o does not change).
  float qmax = qr[0];
#pragma unroll
  for (int rr = 1; rr < 16; ++rr) qmax = fmaxf(qmax, qr[rr]);
  qmax = fmaxf(qmax, __shfl_xor(qmax, 16, 64));
  qmax = fmaxf(qmax, __shfl_xor(qmax, 32, 64));
  float eneg;
  int epos;
  phi_row_scale(qmax, eneg, epos);
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    pk[rr] = phi(pk[rr]);
    pq[rr] = phi_row_scaled(qr[rr], eneg, epos);
  }

  // Rank-1 update S += phi(k) v^T, then the partial read phi(q)^T S.
  float4 s[16];
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) s[rr] = Sh[(16 * cq + rr) * 16 + m4];
  float n0 = 0.f, n1 = 0.f, n2 = 0.f, n3 = 0.f;
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    s[rr].x += pk[rr] * v0;
    s[rr].y += pk[rr] * v1;
    s[rr].z += pk[rr] * v2;
    s[rr].w += pk[rr] * v3;
    n0 += pq[rr] * s[rr].x;
    n1 += pq[rr] * s[rr].y;
    n2 += pq[rr] * s[rr].z;
    n3 += pq[rr] * s[rr].w;
  }
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) Sh[(16 * cq + rr) * 16 + m4] = s[rr];

  // z += phi(k): lane l owns z[l]; den = phi(q)^T z over the whole wave.
  float *zh = z + (long long)h * kD;
  const float zl = zh[lane] + phi(load_elem<E>(kh, lane));
  zh[lane] = zl;
  float den = phi_row_scaled(load_elem<E>(qh, lane), eneg, epos) * zl;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off, 64);

  // Sum the four row groups' partial columns.
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
    n0 += __shfl_xor(n0, off, 64);
    n1 += __shfl_xor(n1, off, 64);
    n2 += __shfl_xor(n2, off, 64);
    n3 += __shfl_xor(n3, off, 64);
  }
  if (cq == 0) {
    float4 r = make_float4(n0 / den, n1 / den, n2 / den, n3 / den);
    reinterpret_cast<float4 *>(o + (long long)h * kD)[m4] = r;
  }
}

}  // namespace linattn
