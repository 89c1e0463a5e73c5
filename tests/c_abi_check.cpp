// c_abi_check.cpp -- drives liblinattn.so through its C ABI alone (no Python,
// no PyTorch): device buffers from hipMalloc, inputs from a seeded host
// generator, results checked element by element against the fp64 oracle
// (oracle/liboracle.so, test infrastructure).  Exit status 0 when every case
// is within its bound, 1 otherwise.
//
// Cases: causal bf16 forward on a ragged length, non-causal fp32 forward,
// causal bf16 backward, and four fp32 decode steps on a head count that is not
// a multiple of the kernel's four heads per workgroup.  Error metric as in the
// Python tests: max |x - x_ref| / x_mag, with x_mag the oracle's magnitude
// companion; bounds 1e-4 for fp32 inputs, 2e-2 for bf16 inputs.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../include/linattn.h"

// The oracle's C entry points (oracle/oracle.c).
extern "C" {
int oracle_forward_recurrent(const void *Q, const void *K, const void *V, int dtype, long units, long N, long C,
                             long M, int causal, int absv, const double *S0, const double *z0, double *O,
                             double *S_out, double *z_out, int nthreads);
int oracle_decode_step(double *S, double *z, const void *q, const void *k, const void *v, int dtype, long units,
                       long C, long M, int absv, double *o, int nthreads);
int oracle_backward_recurrent(const void *Q, const void *K, const void *V, const void *G, int dtype, long units,
                              long N, long C, long M, int causal, int mode, double *dQ, double *dK, double *dV,
                              int nthreads);
}

namespace {

constexpr int kOracleF32 = 1, kOracleBf16 = 2;

// splitmix64 stream -> standard normal draws (Box-Muller).
struct Normal {
  uint64_t s;
  explicit Normal(uint64_t seed) : s(seed) {}
  uint64_t next() {
    uint64_t z = (s += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
  }
  double uniform() { return ((next() >> 11) + 0.5) * (1.0 / 9007199254740992.0); }
  float draw() { return (float)(std::sqrt(-2.0 * std::log(uniform())) * std::cos(6.283185307179586 * uniform())); }
};

uint16_t to_bf16(float x) {  // round to nearest even (finite inputs)
  uint32_t b;
  std::memcpy(&b, &x, 4);
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}
float from_bf16(uint16_t h) {
  const uint32_t b = (uint32_t)h << 16;
  float x;
  std::memcpy(&x, &b, 4);
  return x;
}

bool ok(hipError_t e, const char *what) {
  if (e != hipSuccess) std::printf("HIP error in %s: %s\n", what, hipGetErrorString(e));
  return e == hipSuccess;
}

// Device copy of a host array; freed by the caller.
template <class T> T *upload(const std::vector<T> &h) {
  T *d = nullptr;
  if (!ok(hipMalloc(&d, h.size() * sizeof(T) + 16), "hipMalloc")) return nullptr;
  if (!ok(hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice), "hipMemcpy")) return nullptr;
  return d;
}

double max_err(const std::vector<double> &got, const std::vector<double> &ref, const std::vector<double> &mag) {
  double e = 0.0;
  for (size_t i = 0; i < got.size(); ++i) {
    const double d = std::fabs(got[i] - ref[i]);
    if (mag[i] == 0.0) {
      if (d != 0.0) return INFINITY;
    } else if (d / mag[i] > e) {
      e = d / mag[i];
    }
  }
  return e;
}

bool report(const char *name, double err, double bound) {
  const bool pass = err <= bound;
  std::printf("%-44s err=%.3e bound=%.0e %s\n", name, err, bound, pass ? "PASS" : "FAIL");
  std::fflush(stdout);
  return pass;
}

// Inputs [units][N][64] as host floats and as the dtype's bytes.
struct Tensor {
  std::vector<float> f;
  std::vector<uint16_t> h;  // bf16 patterns (bf16 cases)
  bool bf16;
  const void *host() const { return bf16 ? (const void *)h.data() : (const void *)f.data(); }
  size_t elem_bytes() const { return bf16 ? 2 : 4; }
};

Tensor draw(size_t n, bool bf16, Normal &g) {
  Tensor t;
  t.bf16 = bf16;
  t.f.resize(n);
  for (size_t i = 0; i < n; ++i) t.f[i] = g.draw();
  if (bf16) {
    t.h.resize(n);
    for (size_t i = 0; i < n; ++i) t.h[i] = to_bf16(t.f[i]);
  }
  return t;
}

void *upload(const Tensor &t) {
  void *d = nullptr;
  const size_t bytes = t.f.size() * t.elem_bytes();
  if (!ok(hipMalloc(&d, bytes + 16), "hipMalloc")) return nullptr;
  if (!ok(hipMemcpy(d, t.host(), bytes, hipMemcpyHostToDevice), "hipMemcpy")) return nullptr;
  return d;
}

std::vector<double> download(const void *d, size_t n, bool bf16) {
  std::vector<double> out(n);
  if (bf16) {
    std::vector<uint16_t> h(n);
    if (!ok(hipMemcpy(h.data(), d, n * 2, hipMemcpyDeviceToHost), "hipMemcpy")) return {};
    for (size_t i = 0; i < n; ++i) out[i] = from_bf16(h[i]);
  } else {
    std::vector<float> h(n);
    if (!ok(hipMemcpy(h.data(), d, n * 4, hipMemcpyDeviceToHost), "hipMemcpy")) return {};
    for (size_t i = 0; i < n; ++i) out[i] = h[i];
  }
  return out;
}

bool forward_case(int B, int H, int N, bool bf16, int causal, uint64_t seed, hipStream_t s) {
  Normal g(seed);
  const size_t n = (size_t)B * H * N * 64;
  const Tensor q = draw(n, bf16, g), k = draw(n, bf16, g), v = draw(n, bf16, g);
  void *dq = upload(q), *dk = upload(k), *dv = upload(v), *dout = nullptr, *ws = nullptr;
  const linattn_dtype dt = bf16 ? LINATTN_BF16 : LINATTN_F32;
  const size_t wsb = linattn_forward_workspace_bytes(B, H, N, 64, 64, dt, causal);
  if (!dq || !dk || !dv || !ok(hipMalloc(&dout, n * q.elem_bytes() + 16), "hipMalloc")) return false;
  if (wsb > 0 && !ok(hipMalloc(&ws, wsb), "hipMalloc")) return false;
  const linattn_status st = linattn_forward(dq, dk, dv, dout, B, H, N, 64, 64, dt, causal, ws, wsb, s);
  if (st != LINATTN_OK) {
    std::printf("linattn_forward: %s\n", linattn_last_error());
    return false;
  }
  if (!ok(hipStreamSynchronize(s), "hipStreamSynchronize")) return false;
  const std::vector<double> got = download(dout, n, bf16);
  std::vector<double> ref(n), mag(n);
  const int odt = bf16 ? kOracleBf16 : kOracleF32;
  if (oracle_forward_recurrent(q.host(), k.host(), v.host(), odt, (long)B * H, N, 64, 64, causal, 0, nullptr, nullptr,
                               ref.data(), nullptr, nullptr, 0) != 0 ||
      oracle_forward_recurrent(q.host(), k.host(), v.host(), odt, (long)B * H, N, 64, 64, causal, 1, nullptr, nullptr,
                               mag.data(), nullptr, nullptr, 0) != 0)
    return false;
  char name[96];
  std::snprintf(name, sizeof name, "forward %s %s B%d H%d N%d", causal ? "causal" : "non-causal",
                bf16 ? "bf16" : "fp32", B, H, N);
  const bool pass = report(name, max_err(got, ref, mag), bf16 ? 2e-2 : 1e-4);
  (void)hipFree(dq), (void)hipFree(dk), (void)hipFree(dv), (void)hipFree(dout), (void)hipFree(ws);
  return pass;
}

bool backward_case(int B, int H, int N, bool bf16, int causal, uint64_t seed, hipStream_t s) {
  Normal g(seed);
  const size_t n = (size_t)B * H * N * 64;
  const Tensor q = draw(n, bf16, g), k = draw(n, bf16, g), v = draw(n, bf16, g), go = draw(n, bf16, g);
  void *dq = upload(q), *dk = upload(k), *dv = upload(v), *dg = upload(go);
  void *gq = nullptr, *gk = nullptr, *gv = nullptr, *ws = nullptr;
  const linattn_dtype dt = bf16 ? LINATTN_BF16 : LINATTN_F32;
  const size_t eb = q.elem_bytes();
  const size_t wsb = linattn_backward_workspace_bytes(B, H, N, 64, 64, dt, causal);
  if (!dq || !dk || !dv || !dg || !ok(hipMalloc(&gq, n * eb), "hipMalloc") || !ok(hipMalloc(&gk, n * eb), "hipMalloc") ||
      !ok(hipMalloc(&gv, n * eb), "hipMalloc") || (wsb > 0 && !ok(hipMalloc(&ws, wsb), "hipMalloc")))
    return false;
  const linattn_status st = linattn_backward(dq, dk, dv, dg, gq, gk, gv, B, H, N, 64, 64, dt, causal, ws, wsb, s);
  if (st != LINATTN_OK) {
    std::printf("linattn_backward: %s\n", linattn_last_error());
    return false;
  }
  if (!ok(hipStreamSynchronize(s), "hipStreamSynchronize")) return false;
  std::vector<double> r[3], m[3];
  for (int i = 0; i < 3; ++i) r[i].resize(n), m[i].resize(n);
  const int odt = bf16 ? kOracleBf16 : kOracleF32;
  if (oracle_backward_recurrent(q.host(), k.host(), v.host(), go.host(), odt, (long)B * H, N, 64, 64, causal, 0,
                                r[0].data(), r[1].data(), r[2].data(), 0) != 0 ||
      oracle_backward_recurrent(q.host(), k.host(), v.host(), go.host(), odt, (long)B * H, N, 64, 64, causal, 1,
                                m[0].data(), m[1].data(), m[2].data(), 0) != 0)
    return false;
  bool pass = true;
  const void *outs[3] = {gq, gk, gv};
  const char *names[3] = {"dQ", "dK", "dV"};
  for (int i = 0; i < 3; ++i) {
    char name[96];
    std::snprintf(name, sizeof name, "backward %s %s B%d H%d N%d %s", causal ? "causal" : "non-causal",
                  bf16 ? "bf16" : "fp32", B, H, N, names[i]);
    pass &= report(name, max_err(download(outs[i], n, bf16), r[i], m[i]), bf16 ? 2e-2 : 1e-4);
  }
  for (void *p : {dq, dk, dv, dg, gq, gk, gv, ws}) (void)hipFree(p);
  return pass;
}

bool decode_case(int BH, int steps, uint64_t seed, hipStream_t s) {
  Normal g(seed);
  std::vector<float> S((size_t)BH * 4096, 0.f), z((size_t)BH * 64, 0.f);
  float *dS = upload(S), *dz = upload(z), *dqkv = nullptr, *dout = nullptr;
  if (!dS || !dz || !ok(hipMalloc(&dqkv, (size_t)3 * BH * 64 * 4), "hipMalloc") ||
      !ok(hipMalloc(&dout, (size_t)BH * 64 * 4), "hipMalloc"))
    return false;
  std::vector<double> So((size_t)BH * 4096, 0.0), zo((size_t)BH * 64, 0.0), Sa = So, za = zo;
  bool pass = true;
  for (int t = 0; t < steps; ++t) {
    std::vector<float> qkv((size_t)3 * BH * 64);
    for (float &x : qkv) x = g.draw();
    if (!ok(hipMemcpy(dqkv, qkv.data(), qkv.size() * 4, hipMemcpyHostToDevice), "hipMemcpy")) return false;
    const float *dq = dqkv, *dk = dqkv + BH * 64, *dv = dqkv + 2 * BH * 64;
    const linattn_status st = linattn_decode_step(dS, dz, dq, dk, dv, dout, BH, 64, 64, LINATTN_F32, s);
    if (st != LINATTN_OK) {
      std::printf("linattn_decode_step: %s\n", linattn_last_error());
      return false;
    }
    if (!ok(hipStreamSynchronize(s), "hipStreamSynchronize")) return false;
    std::vector<double> ref((size_t)BH * 64), mag((size_t)BH * 64);
    const float *hq = qkv.data(), *hk = hq + BH * 64, *hv = hq + 2 * BH * 64;
    if (oracle_decode_step(So.data(), zo.data(), hq, hk, hv, kOracleF32, BH, 64, 64, 0, ref.data(), 0) != 0 ||
        oracle_decode_step(Sa.data(), za.data(), hq, hk, hv, kOracleF32, BH, 64, 64, 1, mag.data(), 0) != 0)
      return false;
    char name[96];
    std::snprintf(name, sizeof name, "decode fp32 BH%d step %d", BH, t);
    pass &= report(name, max_err(download(dout, (size_t)BH * 64, false), ref, mag), 1e-4);
  }
  for (void *p : {(void *)dS, (void *)dz, (void *)dqkv, (void *)dout}) (void)hipFree(p);
  return pass;
}

}  // namespace

int main() {
  std::printf("liblinattn interface version %d\n", linattn_version());
  hipStream_t s;
  if (!ok(hipStreamCreate(&s), "hipStreamCreate")) return 1;
  bool pass = true;
  pass &= forward_case(1, 3, 1000, true, 1, 11, s);
  pass &= forward_case(2, 2, 300, false, 0, 12, s);
  pass &= backward_case(1, 2, 700, true, 1, 13, s);
  pass &= decode_case(5, 4, 14, s);
  (void)hipStreamDestroy(s);
  std::printf("%s\n", pass ? "ALL PASS" : "FAILURES");
  return pass ? 0 : 1;
}
