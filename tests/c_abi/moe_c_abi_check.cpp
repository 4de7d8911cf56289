// The C ABI used from C++ with nothing but the HIP runtime: no Python, no
// torch.  One layer (layout, dispatch, combine, both backward passes) on a
// small routing, checked against properties that need no reference values:
//
//   * every (token, k) pair has one receive row, inside its expert's segment,
//     in token order within the expert, and the segments tile [0, T*K);
//   * a dispatch copies each token row bit for bit into its receive rows;
//   * on small-integer rows every float32 sum below is exact, so a plain
//     combine of the dispatched rows gives K * x exactly, the combine
//     backward gives w * g rows and <g, x> router gradients exactly, and the
//     dispatch backward of those rows gives sum_k w[t,k] * g exactly.
//
// Built by the package's build step; run by tests/test_gpu_c_abi.py.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <vector>

#include "../../include/moe_layout.h"

namespace {

constexpr int64_t T = 1000;
constexpr int K = 8, E = 64, P = 8, H = 256;  // float32 rows: 64 chunks of 16 bytes

int failures = 0;

void expect(bool ok, const char* what, int64_t at = -1) {
  if (ok) return;
  if (failures++ < 10) std::printf("FAIL %s (at %lld)\n", what, (long long)at);
}

#define HIP_OK(x)                                                              \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 2;                                                                \
    }                                                                          \
  } while (0)

#define MOE_OK_(x)                                                                        \
  do {                                                                                    \
    int s_ = (x);                                                                         \
    if (s_ != MOE_OK) {                                                                   \
      std::printf("moe error %d (%s) at line %d\n", s_, moe_strerror(s_), __LINE__); \
      return 2;                                                                           \
    }                                                                                     \
  } while (0)

// test-only generator (64-bit LCG); the routing and values only need to be
// deterministic, not good
struct Lcg {
  uint64_t s;
  uint32_t next() {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(s >> 33);
  }
};

}  // namespace

int main() {
  std::printf("c-abi check: %s, T=%lld K=%d E=%d P=%d H=%d float32\n", moe_version(), (long long)T, K, E, P,
              H);
  Lcg rng{12345};
  // routing: K distinct experts per token
  std::vector<int32_t> idx(T * K);
  for (int64_t t = 0; t < T; ++t) {
    int chosen[E] = {0};
    for (int k = 0; k < K; ++k) {
      int e;
      do e = (int)(rng.next() % E); while (chosen[e]);
      chosen[e] = 1;
      idx[t * K + k] = e;
    }
  }
  // small-integer rows and power-of-two weights: every sum below is exact
  std::vector<float> x(T * H), g(T * H), w(T * K);
  for (auto& v : x) v = (float)((int)(rng.next() % 9) - 4);
  for (auto& v : g) v = (float)((int)(rng.next() % 9) - 4);
  for (auto& v : w) v = (rng.next() & 1) ? 0.5f : 2.0f;
  const int64_t R = T * K;

  size_t ws_bytes = 0;
  MOE_OK_(moe_workspace_size(T, K, E, P, &ws_bytes));
  void *d_idx, *d_ws, *d_x, *d_g, *d_w, *d_recv, *d_out, *d_gy, *d_gw, *d_gx;
  HIP_OK(hipMalloc(&d_idx, idx.size() * 4));
  HIP_OK(hipMalloc(&d_ws, ws_bytes));
  HIP_OK(hipMalloc(&d_x, x.size() * 4));
  HIP_OK(hipMalloc(&d_g, g.size() * 4));
  HIP_OK(hipMalloc(&d_w, w.size() * 4));
  HIP_OK(hipMalloc(&d_recv, R * H * 4));
  HIP_OK(hipMalloc(&d_out, T * H * 4));
  HIP_OK(hipMalloc(&d_gy, R * H * 4));
  HIP_OK(hipMalloc(&d_gw, T * K * 4));
  HIP_OK(hipMalloc(&d_gx, T * H * 4));
  HIP_OK(hipMemcpy(d_idx, idx.data(), idx.size() * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_x, x.data(), x.size() * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_g, g.data(), g.size() * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_w, w.data(), w.size() * 4, hipMemcpyHostToDevice));
  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));

  moe_handle_t h = nullptr;
  MOE_OK_(moe_handle_create(&h, nullptr));
  MOE_OK_(moe_layout(h, d_idx, MOE_I32, T, K, E, P, d_ws, ws_bytes, s));
  MOE_OK_(moe_dispatch(h, d_x, MOE_F32, H, nullptr, 0, d_recv, nullptr, s));
  MOE_OK_(moe_combine(h, d_recv, MOE_F32, H, nullptr, d_out, s));
  MOE_OK_(moe_combine_bwd(h, d_g, MOE_F32, H, (const float*)d_w, d_recv, d_gy, (float*)d_gw, s));
  MOE_OK_(moe_dispatch_bwd(h, d_gy, MOE_F32, H, nullptr, nullptr, d_gx, nullptr, s));
  int status = -1;
  MOE_OK_(moe_handle_check(h, s, &status));
  expect(status == 0, "device status");

  // handle fields
  void* fp = nullptr;
  size_t fb = 0;
  std::vector<int32_t> pos(R), n_e(E), off(E + 1);
  MOE_OK_(moe_handle_field(h, MOE_FIELD_RECV_POS, &fp, &fb));
  expect(fb == (size_t)R * 4, "recv_pos size");
  HIP_OK(hipMemcpy(pos.data(), fp, R * 4, hipMemcpyDeviceToHost));
  MOE_OK_(moe_handle_field(h, MOE_FIELD_NUM_TOKENS_PER_EXPERT, &fp, &fb));
  HIP_OK(hipMemcpy(n_e.data(), fp, E * 4, hipMemcpyDeviceToHost));
  MOE_OK_(moe_handle_field(h, MOE_FIELD_EXPERT_OFFSET, &fp, &fb));
  HIP_OK(hipMemcpy(off.data(), fp, (E + 1) * 4, hipMemcpyDeviceToHost));

  int64_t total = 0;
  for (int e = 0; e < E; ++e) {
    total += n_e[e];
    expect(off[e + 1] - off[e] == n_e[e], "segment length", e);
  }
  expect(off[0] == 0 && total == R && off[E] == R, "segments tile [0, T*K)");
  std::vector<int> seen(R, 0);
  std::vector<int32_t> last(E, -1);
  for (int64_t t = 0; t < T; ++t)
    for (int k = 0; k < K; ++k) {
      const int e = idx[t * K + k];
      const int32_t p = pos[t * K + k];
      const bool inside = p >= off[e] && p < off[e + 1];
      expect(inside, "receive row inside its expert's segment", t * K + k);
      if (!inside) continue;
      expect(seen[p]++ == 0, "one pair per receive row", p);
      expect(p > last[e], "token order within an expert", t * K + k);
      last[e] = p;
    }

  // rows
  std::vector<float> recv(R * H), out(T * H), gy(R * H), gw(T * K), gx(T * H);
  HIP_OK(hipMemcpy(recv.data(), d_recv, recv.size() * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out.data(), d_out, out.size() * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(gy.data(), d_gy, gy.size() * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(gw.data(), d_gw, gw.size() * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(gx.data(), d_gx, gx.size() * 4, hipMemcpyDeviceToHost));
  for (int64_t t = 0; t < T; ++t) {
    float wsum = 0.f;
    for (int k = 0; k < K; ++k) {
      const int64_t p = pos[t * K + k];
      if (p < 0 || p >= R) continue;  // already reported
      const float wk = w[t * K + k];
      float dot = 0.f;
      for (int c = 0; c < H; ++c) {
        expect(recv[p * H + c] == x[t * H + c], "dispatch copies the token row", p);
        expect(gy[p * H + c] == wk * g[t * H + c], "combine_bwd rows are w * g", p);
        dot += g[t * H + c] * x[t * H + c];
      }
      expect(gw[t * K + k] == dot, "combine_bwd router gradient is <g, x>", t * K + k);
      wsum += wk;
    }
    for (int c = 0; c < H; ++c) {
      expect(out[t * H + c] == (float)K * x[t * H + c], "plain combine of the dispatch is K * x", t);
      expect(gx[t * H + c] == wsum * g[t * H + c], "dispatch_bwd of w * g rows is sum_k w * g", t);
    }
  }

  MOE_OK_(moe_handle_destroy(h));
  HIP_OK(hipStreamDestroy(s));
  for (void* p : {d_idx, d_ws, d_x, d_g, d_w, d_recv, d_out, d_gy, d_gw, d_gx}) HIP_OK(hipFree(p));
  if (failures) {
    std::printf("c-abi check: %d failures\n", failures);
    return 1;
  }
  std::printf("c-abi check: ok\n");
  return 0;
}
