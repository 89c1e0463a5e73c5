// c_abi_check.cpp -- drives liblinattn.so through its C ABI alone (no Python,
// no PyTorch): device buffers from hipMalloc, inputs from a seeded host
// generator, results checked element by element against the fp64 oracle
// (oracle/liboracle.so, test infrastructure).  Exit status 0 when every case
// is within its bound, 1 otherwise.
//
// Cases: causal bf16 forward on a ragged length, non-causal fp32 forward,
// causal bf16 backward, the training pair (forward_train then backward_train,
// bf16 causal), backward_after_forward (fp32 non-causal, also bit for bit
// against backward), a causal fp32 prefill split in two forward_state calls
// that carry the state (outputs and final state), and fp32 decode steps on a
// head count that is not a multiple of the kernel's four heads per workgroup,
// with packed and with strided q, k, v.  Error metric as in the
// Python tests: max |x - x_ref| / x_mag, with x_mag the oracle's magnitude
// companion; bounds 1e-4 for fp32 inputs, 2e-2 for bf16 inputs.
#include <hip/hip_runtime.h>

#include <algorithm>
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

// Backward modes: 0 linattn_backward; 1 linattn_forward then
// linattn_backward_after_forward (also compared bit for bit with mode 0's
// call); 2 linattn_forward_train then linattn_backward_train (its forward
// output checked too).
bool backward_case(int B, int H, int N, bool bf16, int causal, int mode, uint64_t seed, hipStream_t s) {
  Normal g(seed);
  const size_t n = (size_t)B * H * N * 64;
  const Tensor q = draw(n, bf16, g), k = draw(n, bf16, g), v = draw(n, bf16, g), go = draw(n, bf16, g);
  void *dq = upload(q), *dk = upload(k), *dv = upload(v), *dg = upload(go);
  void *gq = nullptr, *gk = nullptr, *gv = nullptr, *ws = nullptr, *dout = nullptr;
  const linattn_dtype dt = bf16 ? LINATTN_BF16 : LINATTN_F32;
  const size_t eb = q.elem_bytes();
  const size_t wsb = mode == 2 ? linattn_train_workspace_bytes(B, H, N, 64, 64, dt, causal)
                               : linattn_backward_workspace_bytes(B, H, N, 64, 64, dt, causal);
  if (!dq || !dk || !dv || !dg || !ok(hipMalloc(&gq, n * eb), "hipMalloc") || !ok(hipMalloc(&gk, n * eb), "hipMalloc") ||
      !ok(hipMalloc(&gv, n * eb), "hipMalloc") || !ok(hipMalloc(&dout, n * eb + 16), "hipMalloc") ||
      (wsb > 0 && !ok(hipMalloc(&ws, wsb), "hipMalloc")))
    return false;
  linattn_status st = LINATTN_OK;
  const char *what = "linattn_backward";
  if (mode == 0) {
    st = linattn_backward(dq, dk, dv, dg, gq, gk, gv, B, H, N, 64, 64, dt, causal, ws, wsb, s);
  } else if (mode == 1) {
    what = "linattn_forward / linattn_backward_after_forward";
    st = linattn_forward(dq, dk, dv, dout, B, H, N, 64, 64, dt, causal, ws, wsb, s);
    if (st == LINATTN_OK)
      st = linattn_backward_after_forward(dq, dk, dv, dg, gq, gk, gv, B, H, N, 64, 64, dt, causal, ws, wsb, s);
  } else {
    what = "linattn_forward_train / linattn_backward_train";
    st = linattn_forward_train(dq, dk, dv, dout, B, H, N, 64, 64, dt, causal, ws, wsb, s);
    if (st == LINATTN_OK)
      st = linattn_backward_train(dq, dk, dv, dout, dg, gq, gk, gv, B, H, N, 64, 64, dt, causal, ws, wsb, s);
  }
  if (st != LINATTN_OK) {
    std::printf("%s: %s\n", what, linattn_last_error());
    return false;
  }
  if (!ok(hipStreamSynchronize(s), "hipStreamSynchronize")) return false;
  static const char *kMode[3] = {"backward", "backward_after_forward", "backward_train"};
  bool pass = true;
  const int odt = bf16 ? kOracleBf16 : kOracleF32;
  if (mode == 2) {
    std::vector<double> ref(n), mag(n);
    if (oracle_forward_recurrent(q.host(), k.host(), v.host(), odt, (long)B * H, N, 64, 64, causal, 0, nullptr,
                                 nullptr, ref.data(), nullptr, nullptr, 0) != 0 ||
        oracle_forward_recurrent(q.host(), k.host(), v.host(), odt, (long)B * H, N, 64, 64, causal, 1, nullptr,
                                 nullptr, mag.data(), nullptr, nullptr, 0) != 0)
      return false;
    char name[96];
    std::snprintf(name, sizeof name, "forward_train %s %s B%d H%d N%d", causal ? "causal" : "non-causal",
                  bf16 ? "bf16" : "fp32", B, H, N);
    pass &= report(name, max_err(download(dout, n, bf16), ref, mag), bf16 ? 2e-2 : 1e-4);
  }
  std::vector<double> r[3], m[3];
  for (int i = 0; i < 3; ++i) r[i].resize(n), m[i].resize(n);
  if (oracle_backward_recurrent(q.host(), k.host(), v.host(), go.host(), odt, (long)B * H, N, 64, 64, causal, 0,
                                r[0].data(), r[1].data(), r[2].data(), 0) != 0 ||
      oracle_backward_recurrent(q.host(), k.host(), v.host(), go.host(), odt, (long)B * H, N, 64, 64, causal, 1,
                                m[0].data(), m[1].data(), m[2].data(), 0) != 0)
    return false;
  void *const outs[3] = {gq, gk, gv};
  const char *names[3] = {"dQ", "dK", "dV"};
  std::vector<double> got[3];
  for (int i = 0; i < 3; ++i) {
    char name[96];
    std::snprintf(name, sizeof name, "%s %s %s B%d H%d N%d %s", kMode[mode], causal ? "causal" : "non-causal",
                  bf16 ? "bf16" : "fp32", B, H, N, names[i]);
    got[i] = download(outs[i], n, bf16);
    pass &= report(name, max_err(got[i], r[i], m[i]), bf16 ? 2e-2 : 1e-4);
  }
  if (mode == 1) {  // the same gradients as linattn_backward, bit for bit
    st = linattn_backward(dq, dk, dv, dg, gq, gk, gv, B, H, N, 64, 64, dt, causal, ws, wsb, s);
    if (st != LINATTN_OK || !ok(hipStreamSynchronize(s), "hipStreamSynchronize")) return false;
    bool same = true;
    for (int i = 0; i < 3; ++i) same &= download(outs[i], n, bf16) == got[i];
    std::printf("%-44s %s\n", "backward_after_forward == backward (bits)", same ? "PASS" : "FAIL");
    pass &= same;
  }
  for (void *p : {dq, dk, dv, dg, gq, gk, gv, ws, dout}) (void)hipFree(p);
  return pass;
}

// Causal fp32 prefill of N tokens as two linattn_forward_state calls (the
// first N1 tokens from zero state, then the rest from the state the first
// call returned), against one oracle pass over all N tokens: the outputs of
// both calls and the final (S, z).
bool forward_state_case(int B, int H, int N, int N1, uint64_t seed, hipStream_t s) {
  Normal g(seed);
  const int units = B * H, N2 = N - N1;
  const size_t n = (size_t)units * N * 64;
  const Tensor q = draw(n, false, g), k = draw(n, false, g), v = draw(n, false, g);
  // The two calls' inputs: [units][N1][64] and [units][N2][64] slices.
  std::vector<float> parts[2][3];
  const Tensor *src[3] = {&q, &k, &v};
  for (int t = 0; t < 3; ++t)
    for (int u = 0; u < units; ++u) {
      const float *row = src[t]->f.data() + (size_t)u * N * 64;
      parts[0][t].insert(parts[0][t].end(), row, row + (size_t)N1 * 64);
      parts[1][t].insert(parts[1][t].end(), row + (size_t)N1 * 64, row + (size_t)N * 64);
    }
  float *dS = nullptr, *dz = nullptr;
  if (!ok(hipMalloc(&dS, (size_t)units * 4096 * 4), "hipMalloc") || !ok(hipMalloc(&dz, (size_t)units * 64 * 4), "hipMalloc"))
    return false;
  std::vector<double> got(n);
  for (int c = 0; c < 2; ++c) {
    const int Nc = c == 0 ? N1 : N2;
    float *in[3];
    for (int t = 0; t < 3; ++t) in[t] = upload(parts[c][t]);
    void *dout = nullptr, *ws = nullptr;
    const size_t wsb = linattn_forward_state_workspace_bytes(B, H, Nc, 64, 64, LINATTN_F32);
    if (!in[0] || !in[1] || !in[2] || !ok(hipMalloc(&dout, (size_t)units * Nc * 64 * 4 + 16), "hipMalloc") ||
        (wsb > 0 && !ok(hipMalloc(&ws, wsb), "hipMalloc")))
      return false;
    // The second call reads the state the first wrote and updates it in place.
    const linattn_status st = linattn_forward_state(in[0], in[1], in[2], dout, B, H, Nc, 64, 64, LINATTN_F32,
                                                    c == 0 ? nullptr : dS, c == 0 ? nullptr : dz, dS, dz, ws, wsb, s);
    if (st != LINATTN_OK) {
      std::printf("linattn_forward_state: %s\n", linattn_last_error());
      return false;
    }
    if (!ok(hipStreamSynchronize(s), "hipStreamSynchronize")) return false;
    const std::vector<double> o = download(dout, (size_t)units * Nc * 64, false);
    for (int u = 0; u < units; ++u)
      std::copy(o.begin() + (size_t)u * Nc * 64, o.begin() + (size_t)(u + 1) * Nc * 64,
                got.begin() + (size_t)u * N * 64 + (size_t)(c == 0 ? 0 : N1) * 64);
    for (void *p : {(void *)in[0], (void *)in[1], (void *)in[2], dout, ws}) (void)hipFree(p);
  }
  std::vector<double> ref(n), mag(n), S((size_t)units * 4096), z((size_t)units * 64), Sm(S.size()), zm(z.size());
  if (oracle_forward_recurrent(q.host(), k.host(), v.host(), kOracleF32, units, N, 64, 64, 1, 0, nullptr, nullptr,
                               ref.data(), S.data(), z.data(), 0) != 0 ||
      oracle_forward_recurrent(q.host(), k.host(), v.host(), kOracleF32, units, N, 64, 64, 1, 1, nullptr, nullptr,
                               mag.data(), Sm.data(), zm.data(), 0) != 0)
    return false;
  char name[96];
  std::snprintf(name, sizeof name, "forward_state fp32 B%d H%d N%d+%d O", B, H, N1, N2);
  bool pass = report(name, max_err(got, ref, mag), 1e-4);
  std::snprintf(name, sizeof name, "forward_state fp32 B%d H%d N%d+%d S, z", B, H, N1, N2);
  std::vector<double> gs = download(dS, S.size(), false), gz = download(dz, z.size(), false);
  gs.insert(gs.end(), gz.begin(), gz.end());
  S.insert(S.end(), z.begin(), z.end());
  Sm.insert(Sm.end(), zm.begin(), zm.end());
  pass &= report(name, max_err(gs, S, Sm), 1e-4);
  (void)hipFree(dS), (void)hipFree(dz);
  return pass;
}

// strided: q, k, v are the column slices of one [BH][192] projection output
// (linattn_decode_step_strided, row stride 192), else three packed [BH][64].
bool decode_case(int BH, int steps, bool strided, uint64_t seed, hipStream_t s) {
  Normal g(seed);
  std::vector<float> S((size_t)BH * 4096, 0.f), z((size_t)BH * 64, 0.f);
  float *dS = upload(S), *dz = upload(z), *dqkv = nullptr, *dout = nullptr;
  if (!dS || !dz || !ok(hipMalloc(&dqkv, (size_t)3 * BH * 64 * 4), "hipMalloc") ||
      !ok(hipMalloc(&dout, (size_t)BH * 64 * 4), "hipMalloc"))
    return false;
  std::vector<double> So((size_t)BH * 4096, 0.0), zo((size_t)BH * 64, 0.0), Sa = So, za = zo;
  bool pass = true;
  for (int t = 0; t < steps; ++t) {
    std::vector<float> qkv((size_t)3 * BH * 64);  // packed q, then k, then v (the oracle's layout)
    for (float &x : qkv) x = g.draw();
    linattn_status st;
    if (strided) {
      std::vector<float> proj((size_t)BH * 192);
      for (int h = 0; h < BH; ++h)
        for (int t = 0; t < 3; ++t)
          std::copy(qkv.begin() + ((size_t)t * BH + h) * 64, qkv.begin() + ((size_t)t * BH + h + 1) * 64,
                    proj.begin() + (size_t)h * 192 + 64 * t);
      if (!ok(hipMemcpy(dqkv, proj.data(), proj.size() * 4, hipMemcpyHostToDevice), "hipMemcpy")) return false;
      st = linattn_decode_step_strided(dS, dz, dqkv, dqkv + 64, dqkv + 128, dout, BH, 64, 64, LINATTN_F32, 192, s);
    } else {
      if (!ok(hipMemcpy(dqkv, qkv.data(), qkv.size() * 4, hipMemcpyHostToDevice), "hipMemcpy")) return false;
      const float *dq = dqkv, *dk = dqkv + BH * 64, *dv = dqkv + 2 * BH * 64;
      st = linattn_decode_step(dS, dz, dq, dk, dv, dout, BH, 64, 64, LINATTN_F32, s);
    }
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
    std::snprintf(name, sizeof name, "decode%s fp32 BH%d step %d", strided ? " strided" : "", BH, t);
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
  pass &= backward_case(1, 2, 700, true, 1, 0, 13, s);
  pass &= backward_case(1, 2, 700, true, 1, 2, 15, s);
  pass &= backward_case(2, 1, 333, false, 0, 1, 16, s);
  pass &= forward_state_case(1, 3, 700, 257, 17, s);
  pass &= decode_case(5, 4, false, 14, s);
  pass &= decode_case(6, 3, true, 18, s);
  (void)hipStreamDestroy(s);
  std::printf("%s\n", pass ? "ALL PASS" : "FAILURES");
  return pass ? 0 : 1;
}
