// Drives the host side of the C ABI -- argument validation, the offline
// preparation (smoothing, truncated SVD, residual quantization, refinement,
// LoRA), the 8-bit and NVFP4 preparations, layer files, the GEMM planner --
// in a build with the address and undefined-behaviour sanitizers and with the
// device launchers replaced by stubs (device_stubs.cpp).  Exit status 0 and
// "host sanitize ok" when every call returned the status it should.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "svdq.h"

static int g_fail = 0;
#define EXPECT(call, want)                                                                         \
  do {                                                                                             \
    const int got_ = (call);                                                                       \
    if (got_ != (want)) {                                                                          \
      std::printf("FAIL line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, got_, (int)(want), \
                  svdq_last_error());                                                              \
      ++g_fail;                                                                                    \
    }                                                                                              \
  } while (0)

static uint64_t g_state = 0x1234567ull;
static double uniform() {  // 53-bit uniform in [0, 1)
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(g_state >> 11) * (1.0 / 9007199254740992.0);
}
static float gauss() {
  const double u1 = uniform() + 1e-300, u2 = uniform();
  return (float)(std::sqrt(-2.0 * std::log(u1)) * std::cos(6.283185307179586 * u2));
}

struct Layer {
  int m, n, rank;
  std::vector<float> W, amax, lam, inv, res;
  std::vector<uint8_t> qw;
  std::vector<uint16_t> ws, l1, l2;
  Layer(int m_, int n_, int r_) : m(m_), n(n_), rank(r_) {
    W.resize((size_t)m * n);
    for (auto& v : W) v = gauss() / std::sqrt((float)m);
    amax.resize(m);
    for (auto& v : amax) v = 0.5f + (float)std::fabs(gauss()) * 4.0f;
    amax[0] = 0.0f;  // a zero statistic: lambda = 1
    lam.resize(m);
    inv.resize(m);
    res.resize((size_t)m * n);
    qw.resize((size_t)m * n / 2);
    ws.resize((size_t)(m / 64) * n);
    l1.resize((size_t)r_ * m + 1);
    l2.resize((size_t)n * r_ + 1);
  }
  int prepare(bool smooth = true, float alpha = 0.5f) {
    return svdq_prepare_weights(W.data(), smooth ? amax.data() : nullptr, m, n, rank, 64, alpha, qw.data(),
                                ws.data(), l1.data(), l2.data(), lam.data(), inv.data(), res.data());
  }
};

int main() {
  // ---- preparation on wide, tall, rank-0 and full-rank layers --------------
  for (int s = 0; s < 5; ++s) {
    const int m = (int[]){192, 512, 128, 64, 256}[s], n = (int[]){256, 96, 72, 64, 300}[s];
    const int r = (int[]){12, 20, 0, 64, 33}[s];
    Layer L(m, n, r);
    EXPECT(L.prepare(s % 2 == 0), SVDQ_OK);
    // the residual's codes are what svdq_quantize_residual gives
    std::vector<uint8_t> qw2(L.qw.size());
    std::vector<uint16_t> ws2(L.ws.size());
    EXPECT(svdq_quantize_residual(L.res.data(), m, n, 64, qw2.data(), ws2.data()), SVDQ_OK);
    if (qw2 != L.qw || ws2 != L.ws) {
      std::printf("FAIL: residual codes differ (layer %d)\n", s);
      ++g_fail;
    }
  }
  // ---- adversarial residual groups ------------------------------------------
  {
    const int m = 128, n = 8;
    std::vector<float> R((size_t)m * n);
    for (auto& v : R) v = gauss();
    for (int k = 0; k < 64; ++k) R[(size_t)k * n + 0] = 0.0f;
    for (int k = 64; k < 128; ++k) R[(size_t)k * n + 1] = 1e-9f;
    for (int k = 0; k < 64; ++k) R[(size_t)k * n + 2] = 1e30f;
    R[3] = -3e5f;
    std::vector<uint8_t> qw((size_t)m * n / 2);
    std::vector<uint16_t> ws((size_t)(m / 64) * n);
    EXPECT(svdq_quantize_residual(R.data(), m, n, 64, qw.data(), ws.data()), SVDQ_OK);
    R[5] = NAN;
    EXPECT(svdq_quantize_residual(R.data(), m, n, 64, qw.data(), ws.data()), SVDQ_ERR_NONFINITE);
  }
  // ---- refinement, LoRA, 8-bit and NVFP4 preparation ------------------------
  {
    Layer L(256, 128, 8);
    std::vector<uint16_t> xcal(16 * 256);
    for (auto& v : xcal) v = (uint16_t)(0x3F00 + (uint16_t)(uniform() * 255));
    const float alphas[3] = {0.3f, 0.5f, 0.9f};
    float a_out = 0.0f;
    int it_out = -1;
    double err = -1.0;
    EXPECT(svdq_prepare_weights_refined(L.W.data(), L.amax.data(), xcal.data(), 16, 256, 128, 8, 64, alphas, 3, 2,
                                        L.qw.data(), L.ws.data(), L.l1.data(), L.l2.data(), L.lam.data(),
                                        L.inv.data(), L.res.data(), &a_out, &it_out, &err),
           SVDQ_OK);
    std::vector<float> A(256 * 4), Bm(4 * 128);
    for (auto& v : A) v = gauss() * 0.1f;
    for (auto& v : Bm) v = gauss() * 0.1f;
    std::vector<uint16_t> l1o(12 * 256), l2o(128 * 12);
    EXPECT(svdq_append_lora(L.l1.data(), L.l2.data(), 256, 128, 8, L.lam.data(), A.data(), Bm.data(), 4, 0.5f,
                            l1o.data(), l2o.data()),
           SVDQ_OK);
    std::vector<int8_t> q8(256 * 128);
    std::vector<uint16_t> s8(128);
    EXPECT(svdq_w8a8_prepare_weights(L.W.data(), L.amax.data(), 256, 128, 8, 0.5f, q8.data(), s8.data(),
                                     L.l1.data(), L.l2.data(), L.lam.data(), L.inv.data(), nullptr),
           SVDQ_OK);
    std::vector<uint8_t> q4(256 * 128 / 2), s4(4 * 128 * 4);
    float tx = 0.0f, tw = 0.0f;
    EXPECT(svdq_fp4_prepare_weights(L.W.data(), L.amax.data(), 256, 128, 8, 0.5f, q4.data(), s4.data(),
                                    L.l1.data(), L.l2.data(), L.lam.data(), L.inv.data(), nullptr, &tx, &tw),
           SVDQ_OK);
  }
  // ---- validation errors of the preparation ---------------------------------
  {
    Layer L(128, 64, 8);
    EXPECT(svdq_prepare_weights(L.W.data(), nullptr, 100, 64, 8, 64, 0.5f, L.qw.data(), L.ws.data(), L.l1.data(),
                                L.l2.data(), L.lam.data(), L.inv.data(), nullptr),
           SVDQ_ERR_UNSUPPORTED);
    EXPECT(L.prepare(true, 1.5f), SVDQ_ERR_INVALID_ARG);
    EXPECT(svdq_prepare_weights(nullptr, nullptr, 128, 64, 8, 64, 0.5f, L.qw.data(), L.ws.data(), L.l1.data(),
                                L.l2.data(), L.lam.data(), L.inv.data(), nullptr),
           SVDQ_ERR_INVALID_ARG);
    L.W[7] = INFINITY;
    EXPECT(L.prepare(), SVDQ_ERR_NONFINITE);
    L.W[7] = 0.0f;
    L.amax[3] = -1.0f;
    EXPECT(L.prepare(), SVDQ_ERR_INVALID_ARG);
    L.amax[3] = 1.0f;
    EXPECT(svdq_test_set_svd_iteration_limit(0), 60);
    EXPECT(L.prepare(), SVDQ_ERR_NO_CONVERGENCE);
    EXPECT(svdq_test_set_svd_iteration_limit(-1), 0);
    EXPECT(L.prepare(), SVDQ_OK);
  }
  // ---- layer files -----------------------------------------------------------
  {
    Layer L(192, 80, 10);
    EXPECT(L.prepare(), SVDQ_OK);
    std::vector<uint16_t> bias(80, 0x3F80);
    svdq_host_layer h{192, 80, 10, 64, 0.5f, L.lam.data(), L.inv.data(), L.qw.data(), L.ws.data(),
                      L.l1.data(), L.l2.data(), bias.data()};
    const char* tmp = std::getenv("TMPDIR");
    const std::string path = std::string(tmp ? tmp : "/tmp") + "/svdq_host_sanitize_" +
                             std::to_string((unsigned long long)g_state % 1000000007ull) + ".svdq";
    EXPECT(svdq_save_layer(path.c_str(), &h), SVDQ_OK);
    int32_t m = 0, n = 0, r = 0, hb = 0;
    float alpha = 0.0f;
    EXPECT(svdq_load_layer_info(path.c_str(), &m, &n, &r, &hb, &alpha), SVDQ_OK);
    Layer B(192, 80, 10);
    std::vector<uint16_t> bias2(80);
    EXPECT(svdq_load_layer(path.c_str(), B.lam.data(), B.inv.data(), B.qw.data(), B.ws.data(), B.l1.data(),
                           B.l2.data(), bias2.data()),
           SVDQ_OK);
    if (m != 192 || n != 80 || r != 10 || hb != 1 || B.qw != L.qw || B.l2 != L.l2 || bias2 != bias) {
      std::printf("FAIL: layer file round trip\n");
      ++g_fail;
    }
    FILE* f = std::fopen(path.c_str(), "r+b");
    std::fseek(f, 200, SEEK_SET);
    std::fputc(0x55, f);
    std::fclose(f);
    EXPECT(svdq_load_layer(path.c_str(), B.lam.data(), B.inv.data(), B.qw.data(), B.ws.data(), B.l1.data(),
                           B.l2.data(), bias2.data()),
           SVDQ_ERR_IO);
    std::remove(path.c_str());
    EXPECT(svdq_load_layer_info(path.c_str(), &m, &n, &r, &hb, &alpha), SVDQ_ERR_IO);
  }
  // ---- the GEMM planner and workspace sizes ----------------------------------
  {
    int info[5];
    const int shapes[][3] = {{4608, 9216, 3072}, {4608, 3072, 12288}, {256, 3072, 15360}, {256, 21504, 3072},
                             {1, 7, 64}, {0, 64, 64}, {300, 520, 2368}, {4096, 4608, 1152}};
    for (const auto& sh : shapes)
      for (int setting = 0; setting < 3; ++setting) {
        EXPECT(svdq_gemm_schedule(sh[0], sh[1], sh[2], setting, info), SVDQ_OK);
        (void)svdq_linear_workspace_size(sh[0], sh[2], sh[1], 48, 64);
        (void)svdq_gemm_workspace_size(sh[0], sh[1], sh[2]);
        (void)svdq_act_workspace_size(sh[0], sh[2], 48);
      }
    EXPECT(svdq_gemm_schedule(64, 64, 64, 7, info), SVDQ_ERR_INVALID_ARG);
    EXPECT(svdq_gemm_schedule(64, 64, 100, 0, info), SVDQ_ERR_UNSUPPORTED);
  }
  // ---- device entry points: errors found on the host, and the launch stub ----
  {
    alignas(256) static uint8_t dev[1 << 20];  // stands in for device memory (never touched)
    svdq_layer L{256, 64, 16, 64, (const float*)dev, dev, (const uint16_t*)dev, (const uint16_t*)dev,
                 (const uint16_t*)dev, nullptr};
    EXPECT(svdq_linear((const uint16_t*)dev, &L, 8, dev, SVDQ_OUT_BF16, nullptr, 0, nullptr), SVDQ_ERR_WORKSPACE);
    EXPECT(svdq_linear((const uint16_t*)(dev + 2), &L, 8, dev, SVDQ_OUT_BF16, dev, sizeof dev, nullptr),
           SVDQ_ERR_ALIGNMENT);
    EXPECT(svdq_linear((const uint16_t*)dev, &L, 8, dev, 5, dev, sizeof dev, nullptr), SVDQ_ERR_INVALID_ARG);
    EXPECT(svdq_linear((const uint16_t*)dev, &L, 0, nullptr, SVDQ_OUT_BF16, nullptr, 0, nullptr), SVDQ_OK);
    EXPECT(svdq_linear((const uint16_t*)dev, &L, 8, dev, SVDQ_OUT_BF16, dev, sizeof dev, nullptr), SVDQ_ERR_HIP);
    EXPECT(svdq_linear_noalloc((const uint16_t*)dev, &L, 8, dev, SVDQ_OUT_F32, nullptr), SVDQ_ERR_HIP);
    EXPECT(svdq_linear_noalloc((const uint16_t*)dev, &L, 1 << 21, dev, SVDQ_OUT_F32, nullptr), SVDQ_ERR_WORKSPACE);
    L.group = 32;
    EXPECT(svdq_linear((const uint16_t*)dev, &L, 8, dev, SVDQ_OUT_BF16, dev, sizeof dev, nullptr),
           SVDQ_ERR_UNSUPPORTED);
    L.group = 64;
    L.rank = 300;
    EXPECT(svdq_gemm_w4a4_lowrank_up(dev, (const uint16_t*)dev, (const float*)dev, &L, 8, dev, SVDQ_OUT_BF16, dev,
                                     sizeof dev, nullptr),
           SVDQ_ERR_UNSUPPORTED);
    EXPECT(svdq_quantize_act_lowrank_down((const uint16_t*)dev, 8, 256, 16, 64, nullptr, nullptr, dev,
                                          (uint16_t*)dev, (float*)dev, nullptr, 0, nullptr),
           SVDQ_ERR_INVALID_ARG);
    EXPECT(svdq_calibrate_act_amax((const uint16_t*)dev, 4, 12, (float*)dev, 0, nullptr), SVDQ_ERR_UNSUPPORTED);
  }
  for (int st = 0; st <= 9; ++st)
    if (!svdq_status_string(st)) ++g_fail;
  if (g_fail) {
    std::printf("host sanitize: %d failed checks\n", g_fail);
    return 1;
  }
  std::printf("host sanitize ok\n");
  return 0;
}
