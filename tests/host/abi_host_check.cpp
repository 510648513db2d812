// Host-layer check of libqsa under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).
//
// Built by tests/test_abi.py with g++ from the library's own host source (qsa_api.cpp) and this
// file, which stands in for the kernel launchers: each stub records the launch arguments it was
// handed and returns a status the driver chooses, so every validation branch, the argument
// marshalling into FwdArgs / BwdArgs and the error reporting run without a GPU or hipcc.
// Exit status 0 and the last line "host checks passed" mean every check held.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <limits>
#include <string>
#include <thread>

#include "qsa.h"
#include "qsa_common.h"

namespace {

struct Seen {
  int which = -1;  // 0 f32, 1 bf16, 2 fp8, 3 backward, 4 matrix-core backward
  int d = 0, wk = -1;
  qsa::FwdArgs f = {};
  qsa::BwdArgs b = {};
} g_seen;
hipError_t g_ret = hipSuccess;

hipError_t record(int which, const qsa::FwdArgs& a, int d, int wk) {
  g_seen.which = which;
  g_seen.d = d;
  g_seen.wk = wk;
  g_seen.f = a;
  return g_ret;
}

int g_fail = 0;
#define CHECK(cond)                                                                  \
  do {                                                                               \
    if (!(cond)) {                                                                   \
      std::fprintf(stderr, "FAILED line %d: %s (last error: %s)\n", __LINE__, #cond, \
                   qsa_last_error());                                                \
      ++g_fail;                                                                      \
    }                                                                                \
  } while (0)

}  // namespace

namespace qsa {
hipError_t launch_f32(const FwdArgs& a, int d, int wk, hipStream_t) { return record(0, a, d, wk); }
hipError_t launch_bf16(const FwdArgs& a, int d, int wk, hipStream_t) { return record(1, a, d, wk); }
hipError_t launch_fp8(const FwdArgs& a, int d, int wk, hipStream_t) { return record(2, a, d, wk); }
hipError_t launch_bwd(const BwdArgs& a, int d, int wk, hipStream_t) {
  g_seen.b = a;
  return record(3, a.f, d, wk);
}
hipError_t launch_bwd_mma(const BwdArgs& a, int d, int wk, hipStream_t) {
  g_seen.b = a;
  return record(4, a.f, d, wk);
}
}  // namespace qsa

extern "C" const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "stub launch error"; }

namespace {

const float kNaN = std::numeric_limits<float>::quiet_NaN();
const float kInf = std::numeric_limits<float>::infinity();
char g_buf[4][64];  // stand-ins for device pointers: the host layer never dereferences them
void* const P0 = g_buf[0];
void* const P1 = g_buf[1];
void* const P2 = g_buf[2];
void* const P3 = g_buf[3];
float g_f[4][4];

int fwd(int B, int H, int Hkv, int N, int d, int causal, int variant, int k, float window, int dtype,
        const qsa_fwd_ex_opts* o = nullptr) {
  g_seen = Seen();
  return qsa_attn_fwd_ex(P0, P1, P2, P3, B, H, Hkv, N, d, causal, variant, k, window, dtype, o, nullptr);
}

int bwd(int variant, int k, float window, int dtype, int grad, float scale = 0.0f, int d = 64) {
  g_seen = Seen();
  return qsa_attn_bwd(P0, P1, P2, P3, g_f[0], g_f[1], g_f[2], 1, 4, 2, 128, d, 1, variant, k, window, dtype, grad,
                      scale, nullptr);
}

void status_strings() {
  CHECK(std::strcmp(qsa_status_string(QSA_OK), "QSA_OK") == 0);
  CHECK(std::strcmp(qsa_status_string(QSA_ERR_HIP), "QSA_ERR_HIP") == 0);
  CHECK(std::strcmp(qsa_status_string(-7), "QSA_ERR_UNKNOWN") == 0);
  CHECK(std::strcmp(qsa_status_string(1 << 30), "QSA_ERR_UNKNOWN") == 0);
  CHECK(qsa_version() == QSA_VERSION);
}

void shapes() {
  const int bf = QSA_DT_BF16;
  CHECK(qsa_attn_validate(1, 2, 2, 256, 64, 0, QSA_EXACT, 0, 0.0f, bf) == QSA_OK);
  CHECK(std::strlen(qsa_last_error()) == 0);
  CHECK(qsa_attn_validate(0, 2, 2, 256, 64, 0, QSA_EXACT, 0, 0.0f, bf) == QSA_ERR_SHAPE);
  CHECK(std::strstr(qsa_last_error(), "B=0") != nullptr);
  CHECK(qsa_attn_validate(1, 0, 1, 256, 64, 0, QSA_EXACT, 0, 0.0f, bf) == QSA_ERR_SHAPE);
  CHECK(qsa_attn_validate(1, 2, 0, 256, 64, 0, QSA_EXACT, 0, 0.0f, bf) == QSA_ERR_SHAPE);
  CHECK(qsa_attn_validate(1, 2, 2, 0, 64, 0, QSA_EXACT, 0, 0.0f, bf) == QSA_ERR_SHAPE);
  CHECK(qsa_attn_validate(1, 6, 4, 256, 64, 0, QSA_EXACT, 0, 0.0f, bf) == QSA_ERR_SHAPE);
  CHECK(qsa_attn_validate(1, 2, 2, (1 << 20) + 1, 64, 0, QSA_EXACT, 0, 0.0f, bf) == QSA_ERR_SHAPE);
  CHECK(qsa_attn_validate(1, 2, 2, 256, 0, 0, QSA_EXACT, 0, 0.0f, bf) == QSA_ERR_SHAPE);
  CHECK(qsa_attn_validate(1, 2, 2, 256, -64, 0, QSA_EXACT, 0, 0.0f, bf) == QSA_ERR_SHAPE);
  CHECK(qsa_attn_validate(1, 2, 2, 256, 96, 0, QSA_EXACT, 0, 0.0f, bf) == QSA_ERR_UNSUPPORTED);
  // 2^31 elements: B * H * N * d overflows 32 bits, so the product must be taken in 64 bits
  CHECK(qsa_attn_validate(1 << 10, 32, 32, 1 << 20, 128, 0, QSA_EXACT, 0, 0.0f, bf) == QSA_ERR_SHAPE);
  CHECK(qsa_attn_validate(2, 1 << 14, 1, 1 << 10, 128, 0, QSA_EXACT, 0, 0.0f, bf) == QSA_ERR_SHAPE);
  CHECK(qsa_attn_validate(1, 1 << 14, 1, 1 << 10, 128, 0, QSA_EXACT, 0, 0.0f, bf) == QSA_ERR_SHAPE);  // 2^31
  CHECK(qsa_attn_validate(1, (1 << 14) - 1, 1, 1 << 10, 128, 0, QSA_EXACT, 0, 0.0f, bf) == QSA_OK);
  CHECK(qsa_attn_validate(1, 1 << 14, 1 << 14, 1 << 10, 64, 0, QSA_EXACT, 0, 0.0f, bf) == QSA_OK);  // 2^30
  CHECK(qsa_attn_validate(2147483647, 2147483647, 1, 1 << 20, 128, 0, QSA_EXACT, 0, 0.0f, bf) == QSA_ERR_SHAPE);
  CHECK(qsa_attn_validate(1, 64, 8, 16384, 128, 1, QSA_POT, 16, 0.0f, bf) == QSA_OK);
}

void variants() {
  const int bf = QSA_DT_BF16, f8 = QSA_DT_FP8_E4M3;
  auto v = [](int variant, int k, float w, int dt) { return qsa_attn_validate(1, 2, 2, 256, 64, 1, variant, k, w, dt); };
  CHECK(v(QSA_EXACT, 0, 0.0f, 7) == QSA_ERR_PARAM);
  CHECK(v(QSA_EXACT, 0, 0.0f, -1) == QSA_ERR_PARAM);
  CHECK(v(QSA_EXACT | (1 << 7), 0, 0.0f, bf) == QSA_ERR_PARAM);
  CHECK(v(7, 0, 0.0f, bf) == QSA_ERR_PARAM);
  CHECK(v(QSA_BASE_MASK, 0, 0.0f, bf) == QSA_ERR_PARAM);
  CHECK(v(QSA_TRUNC, 0, 2.0f, bf) == QSA_OK);
  CHECK(v(QSA_TRUNC | QSA_F_FLUSH, 0, 2.0f, bf) == QSA_ERR_PARAM);
  for (float w : {0.0f, -1.0f, kNaN, kInf, -kInf}) {
    CHECK(v(QSA_TRUNC, 0, w, bf) == QSA_ERR_PARAM);
    CHECK(v(QSA_UNIFORM, 0, w, bf) == QSA_ERR_PARAM);
    CHECK(v(QSA_KINT | QSA_F_WINDOW, 4, w, bf) == QSA_ERR_PARAM);
  }
  CHECK(v(QSA_POT | QSA_F_INTERP, 8, 0.0f, bf) == QSA_ERR_PARAM);
  CHECK(v(QSA_POT | QSA_F_WINDOW, 8, 8.0f, bf) == QSA_ERR_PARAM);
  CHECK(v(QSA_EXACT | QSA_F_FLUSH, 0, 0.0f, bf) == QSA_ERR_PARAM);
  CHECK(v(QSA_EXACT_ANCHORED | QSA_F_FLUSH, 0, 0.0f, bf) == QSA_ERR_PARAM);
  CHECK(v(QSA_KINT, 0, 0.0f, bf) == QSA_ERR_PARAM);
  CHECK(v(QSA_KINT, 65, 0.0f, bf) == QSA_ERR_PARAM);
  CHECK(v(QSA_KINT, 1, 0.0f, bf) == QSA_OK);
  CHECK(v(QSA_KINT, 64, 0.0f, bf) == QSA_OK);
  CHECK(v(QSA_KINT | QSA_F_FLUSH, 4, 0.0f, bf) == QSA_OK);  // accepted, and changes nothing on min-max
  CHECK(v(QSA_POT, 0, 0.0f, bf) == QSA_ERR_PARAM);
  CHECK(v(QSA_POT, 65, 0.0f, bf) == QSA_ERR_PARAM);
  CHECK(v(QSA_POT, 64, 0.0f, bf) == QSA_OK);
  CHECK(v(QSA_POT, 17, 0.0f, f8) == QSA_ERR_PARAM);
  CHECK(v(QSA_POT, 16, 0.0f, f8) == QSA_OK);
  CHECK(v(QSA_POT_RUNNING, 1, 0.0f, bf) == QSA_ERR_PARAM);
  CHECK(v(QSA_POT_RUNNING, 2, 0.0f, bf) == QSA_OK);
  CHECK(v(QSA_POT_RUNNING, 17, 0.0f, f8) == QSA_ERR_PARAM);
  CHECK(v(QSA_POT_RUNNING | QSA_F_FLUSH, 16, 0.0f, f8) == QSA_OK);
}

void forward_calls() {
  // null pointers, each in turn
  for (int i = 0; i < 4; ++i) {
    const void* p[4] = {P0, P1, P2, P3};
    p[i] = nullptr;
    g_seen = Seen();
    CHECK(qsa_attn_fwd(p[0], p[1], p[2], (void*)p[3], 1, 2, 2, 256, 64, 0, QSA_POT, 8, 0.0f, QSA_DT_BF16,
                       nullptr) == QSA_ERR_NULL_PTR);
    CHECK(g_seen.which == -1);
  }
  // shape errors come before pointer errors, and nothing is launched
  g_seen = Seen();
  CHECK(qsa_attn_fwd(nullptr, nullptr, nullptr, nullptr, 0, 2, 2, 256, 64, 0, QSA_POT, 8, 0.0f, QSA_DT_BF16,
                     nullptr) == QSA_ERR_SHAPE);
  CHECK(g_seen.which == -1);

  // marshalling: dtype -> launcher, variant -> weight kind, scale
  CHECK(fwd(1, 2, 2, 256, 64, 1, QSA_KINT | QSA_F_WINDOW | QSA_F_FLUSH, 4, 8.0f, QSA_DT_BF16) == QSA_OK);
  CHECK(g_seen.which == 1 && g_seen.d == 64 && g_seen.wk == qsa::WK_KH_FLUSH);
  CHECK(g_seen.f.window_calib == 1 && g_seen.f.window == 8.0f && g_seen.f.levels == 4 && g_seen.f.causal == 1);
  CHECK(g_seen.f.track_min == 0);
  CHECK(std::fabs(g_seen.f.sc - 0.125f) < 1e-7f);
  CHECK(fwd(1, 2, 2, 256, 64, 0, QSA_KINT | QSA_F_FLUSH, 4, 0.0f, QSA_DT_BF16) == QSA_OK);
  CHECK(g_seen.wk == qsa::WK_KH && g_seen.f.track_min == 1 && g_seen.f.window == 0.0f);
  CHECK(fwd(1, 2, 2, 256, 128, 0, QSA_KINT | QSA_F_INTERP | QSA_F_WINDOW, 16, 8.0f, QSA_DT_F32) == QSA_OK);
  CHECK(g_seen.which == 0 && g_seen.d == 128 && g_seen.wk == qsa::WK_KI);
  CHECK(fwd(1, 32, 32, 8192, 128, 0, QSA_POT, 16, 0.0f, QSA_DT_FP8_E4M3) == QSA_OK);
  CHECK(g_seen.which == 2 && g_seen.wk == qsa::WK_POT && g_seen.f.N == 8192 && g_seen.f.H == 32);
  CHECK(fwd(1, 2, 2, 256, 64, 0, QSA_POT_RUNNING | QSA_F_FLUSH, 8, 0.0f, QSA_DT_BF16) == QSA_OK);
  CHECK(g_seen.wk == qsa::WK_POTR_FLUSH);
  CHECK(fwd(1, 2, 2, 256, 64, 0, QSA_UNIFORM, 0, 2.0f, QSA_DT_BF16) == QSA_OK);
  CHECK(g_seen.wk == qsa::WK_UNIF && g_seen.f.window == 2.0f);

  qsa_fwd_ex_opts o = {};
  o.scale = 0.5f;
  o.q_descale = 2.0f;
  o.k_descale = 0.25f;
  o.v_descale = 3.0f;
  CHECK(fwd(1, 2, 2, 256, 64, 0, QSA_POT, 8, 0.0f, QSA_DT_FP8_E4M3, &o) == QSA_OK);
  CHECK(g_seen.f.sc == 0.25f && g_seen.f.vd == 3.0f);
  CHECK(fwd(1, 2, 2, 256, 64, 0, QSA_POT, 8, 0.0f, QSA_DT_BF16, &o) == QSA_ERR_PARAM);  // descales: fp8 only
  o = qsa_fwd_ex_opts{};
  o.q_descale = 1.0f;
  CHECK(fwd(1, 2, 2, 256, 64, 0, QSA_POT, 8, 0.0f, QSA_DT_BF16, &o) == QSA_OK);
  for (float bad : {kNaN, kInf, -1.0f}) {
    o = qsa_fwd_ex_opts{};
    o.scale = bad;
    CHECK(fwd(1, 2, 2, 256, 64, 0, QSA_POT, 8, 0.0f, QSA_DT_BF16, &o) == QSA_ERR_PARAM);
    o = qsa_fwd_ex_opts{};
    o.k_descale = bad;
    CHECK(fwd(1, 2, 2, 256, 64, 0, QSA_POT, 8, 0.0f, QSA_DT_FP8_E4M3, &o) == QSA_ERR_PARAM);
  }
  o = qsa_fwd_ex_opts{};
  o.scale = 1e-30f;
  o.q_descale = 1e-30f;  // the product underflows to 0
  CHECK(fwd(1, 2, 2, 256, 64, 0, QSA_POT, 8, 0.0f, QSA_DT_FP8_E4M3, &o) == QSA_ERR_PARAM);
  CHECK(g_seen.which == -1);

  // row statistics and the grid-index dump
  o = qsa_fwd_ex_opts{};
  o.row_lo = g_f[3];
  CHECK(fwd(1, 2, 2, 256, 64, 0, QSA_EXACT, 0, 0.0f, QSA_DT_BF16, &o) == QSA_ERR_PARAM);
  CHECK(fwd(1, 2, 2, 256, 64, 0, QSA_POT_RUNNING, 8, 0.0f, QSA_DT_BF16, &o) == QSA_ERR_PARAM);
  CHECK(fwd(1, 2, 2, 256, 64, 0, QSA_POT, 8, 0.0f, QSA_DT_BF16, &o) == QSA_OK);
  CHECK(g_seen.f.track_min == 1 && g_seen.f.row_lo == g_f[3]);
  unsigned char idx[16];
  o = qsa_fwd_ex_opts{};
  o.grid_idx = idx;
  o.idx_row0 = 250;
  o.idx_rows = 6;
  CHECK(fwd(1, 2, 2, 256, 64, 0, QSA_POT, 8, 0.0f, QSA_DT_BF16, &o) == QSA_OK);
  CHECK(g_seen.f.idx_row0 == 250 && g_seen.f.idx_rows == 6 && g_seen.f.grid_idx == idx);
  o.idx_rows = 7;
  CHECK(fwd(1, 2, 2, 256, 64, 0, QSA_POT, 8, 0.0f, QSA_DT_BF16, &o) == QSA_ERR_SHAPE);
  o.idx_row0 = -1;
  o.idx_rows = 1;
  CHECK(fwd(1, 2, 2, 256, 64, 0, QSA_POT, 8, 0.0f, QSA_DT_BF16, &o) == QSA_ERR_SHAPE);
  o.idx_row0 = 2147483647;  // row0 + rows must be formed without overflow
  o.idx_rows = 2147483647;
  CHECK(fwd(1, 2, 2, 256, 64, 0, QSA_POT, 8, 0.0f, QSA_DT_BF16, &o) == QSA_ERR_SHAPE);
  o.idx_row0 = 0;
  o.idx_rows = 0;
  CHECK(fwd(1, 2, 2, 256, 64, 0, QSA_POT, 8, 0.0f, QSA_DT_BF16, &o) == QSA_ERR_SHAPE);
  o.idx_rows = 1 << 16;  // Q has 2^27 elements, the dump 2^37
  CHECK(fwd(1, 32, 8, 1 << 16, 64, 0, QSA_POT, 8, 0.0f, QSA_DT_BF16, &o) == QSA_ERR_SHAPE);
  CHECK(std::strstr(qsa_last_error(), "grid_idx") != nullptr);

  // a launch failure is reported as QSA_ERR_HIP with the runtime's text
  g_ret = hipErrorInvalidValue;
  CHECK(fwd(1, 2, 2, 256, 64, 0, QSA_POT, 8, 0.0f, QSA_DT_BF16) == QSA_ERR_HIP);
  CHECK(std::strstr(qsa_last_error(), "stub launch error") != nullptr);
  g_ret = hipSuccess;
  CHECK(fwd(1, 2, 2, 256, 64, 0, QSA_POT, 8, 0.0f, QSA_DT_BF16) == QSA_OK);
  CHECK(qsa_last_error()[0] == '\0');
}

void backward_calls() {
  CHECK(bwd(QSA_KINT, 4, 0.0f, QSA_DT_BF16, QSA_GRAD_STE_PRE) == QSA_OK);
  CHECK(g_seen.which == 3 && g_seen.b.bf16 == 1 && g_seen.b.mode == QSA_GRAD_STE_PRE && g_seen.wk == qsa::WK_KH);
  CHECK(g_seen.b.dq == g_f[0] && g_seen.b.dk == g_f[1] && g_seen.b.dv == g_f[2] && g_seen.b.dout == P3);
  CHECK(std::fabs(g_seen.f.sc - 0.125f) < 1e-7f);
  CHECK(bwd(QSA_POT, 8, 0.0f, QSA_DT_F32, QSA_GRAD_EXACT_DETACHED, 0.5f, 128) == QSA_OK);
  CHECK(g_seen.b.bf16 == 0 && g_seen.f.sc == 0.5f && g_seen.d == 128);
  CHECK(bwd(QSA_KINT, 4, 0.0f, QSA_DT_FP8_E4M3, QSA_GRAD_STE_PRE) == QSA_ERR_UNSUPPORTED);
  CHECK(bwd(QSA_POT_RUNNING, 8, 0.0f, QSA_DT_BF16, QSA_GRAD_STE_POST) == QSA_ERR_UNSUPPORTED);
  CHECK(bwd(QSA_KINT, 4, 0.0f, QSA_DT_BF16, -1) == QSA_ERR_PARAM);
  CHECK(bwd(QSA_KINT, 4, 0.0f, QSA_DT_BF16, QSA_GRAD_STE_PRE_DETACHED + 1) == QSA_ERR_PARAM);
  CHECK(bwd(QSA_KINT, 4, 0.0f, QSA_DT_BF16, QSA_GRAD_EXACT, kNaN) == QSA_ERR_PARAM);
  CHECK(bwd(QSA_KINT, 4, 0.0f, QSA_DT_BF16, QSA_GRAD_EXACT, -0.5f) == QSA_ERR_PARAM);
  CHECK(bwd(QSA_KINT, 0, 0.0f, QSA_DT_BF16, QSA_GRAD_EXACT) == QSA_ERR_PARAM);
  CHECK(g_seen.which == -1);
  g_seen = Seen();
  CHECK(qsa_attn_bwd(P0, P1, P2, P3, g_f[0], nullptr, g_f[2], 1, 4, 2, 128, 64, 1, QSA_KINT, 4, 0.0f, QSA_DT_BF16,
                     QSA_GRAD_STE_PRE, 0.0f, nullptr) == QSA_ERR_NULL_PTR);
  CHECK(g_seen.which == -1);
  g_ret = hipErrorInvalidValue;
  CHECK(bwd(QSA_KINT, 4, 0.0f, QSA_DT_BF16, QSA_GRAD_STE_PRE) == QSA_ERR_HIP);
  g_ret = hipSuccess;
}

void thread_local_errors() {
  CHECK(qsa_attn_validate(0, 1, 1, 1, 64, 0, QSA_EXACT, 0, 0.0f, QSA_DT_BF16) == QSA_ERR_SHAPE);
  std::string other;
  std::thread t([&] {
    other = qsa_last_error();  // this thread has made no failing call
    (void)qsa_attn_validate(1, 3, 2, 1, 64, 0, QSA_EXACT, 0, 0.0f, QSA_DT_BF16);
  });
  t.join();
  CHECK(other.empty());
  CHECK(std::strstr(qsa_last_error(), "B=0") != nullptr);  // unchanged by the other thread
}

}  // namespace

int main() {
  status_strings();
  shapes();
  variants();
  forward_calls();
  backward_calls();
  thread_local_errors();
  if (g_fail) {
    std::fprintf(stderr, "%d host check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("host checks passed\n");
  return 0;
}
