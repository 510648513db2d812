// Host side of libqsa: argument validation, kernel selection, launch.
// The C ABI is declared (and documented) in include/qsa.h.
#include "qsa.h"

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "qsa_common.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return QSA_OK;
}

int validate(int B, int H, int Hkv, int N, int d, int causal, int variant, int k_levels, float window,
             int dtype) {
  (void)causal;
  if (B < 1 || H < 1 || Hkv < 1 || N < 1)
    return fail(QSA_ERR_SHAPE, "B=%d H=%d Hkv=%d N=%d: each must be >= 1", B, H, Hkv, N);
  if (H % Hkv != 0) return fail(QSA_ERR_SHAPE, "H=%d is not a multiple of Hkv=%d", H, Hkv);
  if (N > (1 << 20)) return fail(QSA_ERR_SHAPE, "N=%d exceeds 2^20", N);
  if (d < 1) return fail(QSA_ERR_SHAPE, "d=%d must be >= 1", d);
  if (d != 64 && d != 128) return fail(QSA_ERR_UNSUPPORTED, "head dimension d=%d: only 64 and 128 are built", d);
  // B * H * N * d < 2^31, tested as B * H <= (2^31 - 1) / (N * d) so that no product overflows
  const int64_t per_head = (int64_t)N * d, cap = ((int64_t(1) << 31) - 1) / per_head;
  if ((int64_t)B * H > cap || (int64_t)B * Hkv > cap) return fail(QSA_ERR_SHAPE, "tensor has 2^31 or more elements");
  if (dtype != QSA_DT_F32 && dtype != QSA_DT_BF16 && dtype != QSA_DT_FP8_E4M3)
    return fail(QSA_ERR_PARAM, "unknown dtype %d", dtype);
  const int base = variant & QSA_BASE_MASK;
  const int flags = variant & ~QSA_BASE_MASK;
  if (flags & ~(QSA_F_INTERP | QSA_F_WINDOW | QSA_F_FLUSH))
    return fail(QSA_ERR_PARAM, "unknown variant flag bits 0x%x", flags);
  if (base > QSA_POT_RUNNING) return fail(QSA_ERR_PARAM, "unknown variant kind %d", base);
  if (base == QSA_TRUNC || base == QSA_UNIFORM) {
    if (flags) return fail(QSA_ERR_PARAM, "support truncation and uniform weighting take no flags");
    if (!(std::isfinite(window) && window > 0.0f))
      return fail(QSA_ERR_PARAM, "support truncation and uniform weighting need a finite window > 0 (got %g)",
                  (double)window);
  }
  if (base != QSA_KINT && (flags & (QSA_F_INTERP | QSA_F_WINDOW)))
    return fail(QSA_ERR_PARAM, "interpolation and fixed-window calibration are K-interval options");
  if ((base == QSA_EXACT || base == QSA_EXACT_ANCHORED) && (flags & QSA_F_FLUSH))
    return fail(QSA_ERR_PARAM, "flush applies to K-interval and PoT");
  if (base == QSA_KINT && (k_levels < 1 || k_levels > 64))
    return fail(QSA_ERR_PARAM, "K-interval needs 1 <= K <= 64 (got %d)", k_levels);
  if (base == QSA_POT_RUNNING) {
    if (k_levels < 2 || k_levels > 64)
      return fail(QSA_ERR_PARAM, "single-pass PoT needs 2 <= L <= 64 (got %d)", k_levels);
    if (dtype == QSA_DT_FP8_E4M3 && k_levels > 16)
      return fail(QSA_ERR_PARAM, "PoT on fp8 needs L <= 16 (got %d)", k_levels);
  }
  if (base == QSA_POT) {
    if (k_levels < 1 || k_levels > 64) return fail(QSA_ERR_PARAM, "PoT needs 1 <= L <= 64 (got %d)", k_levels);
    if (dtype == QSA_DT_FP8_E4M3 && k_levels > 16)
      return fail(QSA_ERR_PARAM, "PoT on fp8 needs L <= 16 (got %d)", k_levels);
  }
  if (flags & QSA_F_WINDOW) {
    if (!(std::isfinite(window) && window > 0.0f))
      return fail(QSA_ERR_PARAM, "fixed-window calibration needs a finite window > 0 (got %g)", (double)window);
  }
  return ok();
}

int weight_kind(int variant) {
  const int base = variant & QSA_BASE_MASK;
  const bool interp = variant & QSA_F_INTERP;
  // a min-max grid spans every visible score, so flushing removes nothing there; dropping the
  // flag keeps a rounded y = K + ulp at the row minimum from flushing the arg-min key
  const bool flush = (variant & QSA_F_FLUSH) && !(base == QSA_KINT && !(variant & QSA_F_WINDOW));
  switch (base) {
    case QSA_EXACT: return qsa::WK_EXACT;
    case QSA_EXACT_ANCHORED: return qsa::WK_EXACT_ANCH;
    case QSA_POT: return flush ? qsa::WK_POT_FLUSH : qsa::WK_POT;
    case QSA_POT_RUNNING: return flush ? qsa::WK_POTR_FLUSH : qsa::WK_POTR;
    case QSA_TRUNC: return qsa::WK_TRUNC;
    case QSA_UNIFORM: return qsa::WK_UNIF;
    default: return interp ? (flush ? qsa::WK_KI_FLUSH : qsa::WK_KI) : (flush ? qsa::WK_KH_FLUSH : qsa::WK_KH);
  }
}

bool descale_ok(float x, bool fp8) {
  if (x == 0.0f) return true;
  if (!fp8) return x == 1.0f;
  return std::isfinite(x) && x > 0.0f;
}

}  // namespace

extern "C" {

int qsa_attn_validate(int B, int H, int Hkv, int N, int d, int causal, int variant, int k_levels, float window,
                      int dtype) {
  return validate(B, H, Hkv, N, d, causal, variant, k_levels, window, dtype);
}

int qsa_attn_fwd_ex(const void* Q, const void* K, const void* V, void* O, int B, int H, int Hkv, int N, int d,
                    int causal, int variant, int k_levels, float window, int dtype, const qsa_fwd_ex_opts* opts,
                    void* stream) {
  int st = validate(B, H, Hkv, N, d, causal, variant, k_levels, window, dtype);
  if (st != QSA_OK) return st;
  if (!Q || !K || !V || !O) return fail(QSA_ERR_NULL_PTR, "Q, K, V and O must be non-NULL");
  const bool fp8 = dtype == QSA_DT_FP8_E4M3;
  qsa_fwd_ex_opts x = {};
  if (opts) x = *opts;
  if (!(std::isfinite(x.scale) && x.scale >= 0.0f))
    return fail(QSA_ERR_PARAM, "scale must be finite and >= 0 (got %g)", (double)x.scale);
  if (!descale_ok(x.q_descale, fp8) || !descale_ok(x.k_descale, fp8) || !descale_ok(x.v_descale, fp8))
    return fail(QSA_ERR_PARAM, "descales must be finite and > 0 for fp8, and 0 or 1 otherwise");
  const int base = variant & QSA_BASE_MASK;
  if (x.row_lo && (base == QSA_EXACT || base == QSA_POT_RUNNING))
    return fail(QSA_ERR_PARAM, "row_lo needs a kind with the row-extrema pre-pass");
  if (x.grid_idx) {
    if (x.idx_row0 < 0 || x.idx_rows < 1 || (int64_t)x.idx_row0 + x.idx_rows > N)
      return fail(QSA_ERR_SHAPE, "grid_idx rows [%d, %d+%d) outside [0, N=%d)", x.idx_row0, x.idx_row0,
                  x.idx_rows, N);
    if ((int64_t)B * H * x.idx_rows * N >= (int64_t(1) << 31))
      return fail(QSA_ERR_SHAPE, "grid_idx dump has 2^31 or more elements");
  }

  qsa::FwdArgs a = {};
  a.q = Q;
  a.k = K;
  a.v = V;
  a.o = O;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.N = N;
  a.causal = causal ? 1 : 0;
  a.levels = k_levels;
  a.window_calib = (base == QSA_KINT && (variant & QSA_F_WINDOW)) ? 1 : 0;
  a.window = (a.window_calib || base == QSA_TRUNC || base == QSA_UNIFORM) ? window : 0.0f;
  const float scale = x.scale > 0.0f ? x.scale : 1.0f / std::sqrt((float)d);
  const float qd = x.q_descale > 0.0f ? x.q_descale : 1.0f;
  const float kd = x.k_descale > 0.0f ? x.k_descale : 1.0f;
  a.sc = scale * qd * kd;
  a.vd = x.v_descale > 0.0f ? x.v_descale : 1.0f;
  if (!(std::isfinite(a.sc) && a.sc > 0.0f)) return fail(QSA_ERR_PARAM, "scale * descales is not a positive float");
  a.row_max = x.row_max;
  a.row_lo = x.row_lo;
  a.row_sum = x.row_sum;
  a.grid_idx = x.grid_idx;
  a.idx_row0 = x.grid_idx ? x.idx_row0 : 0;
  a.idx_rows = x.grid_idx ? x.idx_rows : 0;
  a.track_min = ((base == QSA_KINT && !a.window_calib) || x.row_lo) ? 1 : 0;

  const int wk = weight_kind(variant);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  switch (dtype) {
    case QSA_DT_F32: e = qsa::launch_f32(a, d, wk, s); break;
    case QSA_DT_BF16: e = qsa::launch_bf16(a, d, wk, s); break;
    default: e = qsa::launch_fp8(a, d, wk, s); break;
  }
  if (e != hipSuccess) return fail(QSA_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int qsa_attn_fwd(const void* Q, const void* K, const void* V, void* O, int B, int H, int Hkv, int N, int d,
                 int causal, int variant, int k_levels, float window, int dtype, void* stream) {
  return qsa_attn_fwd_ex(Q, K, V, O, B, H, Hkv, N, d, causal, variant, k_levels, window, dtype, nullptr, stream);
}

int qsa_attn_bwd(const void* Q, const void* K, const void* V, const void* dO, float* dQ, float* dK, float* dV, int B,
                 int H, int Hkv, int N, int d, int causal, int variant, int k_levels, float window, int dtype, int grad,
                 float scale, void* stream) {
  int st = validate(B, H, Hkv, N, d, causal, variant, k_levels, window, dtype);
  if (st != QSA_OK) return st;
  if (dtype == QSA_DT_FP8_E4M3) return fail(QSA_ERR_UNSUPPORTED, "the backward takes float32 or bfloat16 inputs");
  if ((variant & QSA_BASE_MASK) == QSA_POT_RUNNING)
    return fail(QSA_ERR_UNSUPPORTED, "the backward covers the kinds anchored at the row maximum");
  if (grad < QSA_GRAD_STE_POST || grad > QSA_GRAD_STE_PRE_DETACHED)
    return fail(QSA_ERR_PARAM, "unknown gradient mode %d", grad);
  if (!(std::isfinite(scale) && scale >= 0.0f))
    return fail(QSA_ERR_PARAM, "scale must be finite and >= 0 (got %g)", (double)scale);
  if (!Q || !K || !V || !dO || !dQ || !dK || !dV)
    return fail(QSA_ERR_NULL_PTR, "Q, K, V, dO, dQ, dK and dV must be non-NULL");
  const int base = variant & QSA_BASE_MASK;
  qsa::BwdArgs a = {};
  a.f.q = Q;
  a.f.k = K;
  a.f.v = V;
  a.f.B = B;
  a.f.H = H;
  a.f.Hkv = Hkv;
  a.f.N = N;
  a.f.causal = causal ? 1 : 0;
  a.f.levels = k_levels;
  a.f.window_calib = (base == QSA_KINT && (variant & QSA_F_WINDOW)) ? 1 : 0;
  a.f.window = (a.f.window_calib || base == QSA_TRUNC || base == QSA_UNIFORM) ? window : 0.0f;
  a.f.sc = scale > 0.0f ? scale : 1.0f / std::sqrt((float)d);
  a.f.vd = 1.0f;
  a.dout = dO;
  a.dq = dQ;
  a.dk = dK;
  a.dv = dV;
  a.mode = grad;
  a.bf16 = dtype == QSA_DT_BF16 ? 1 : 0;
  const hipError_t e = qsa::launch_bwd(a, d, weight_kind(variant), (hipStream_t)stream);
  if (e != hipSuccess) return fail(QSA_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

const char* qsa_status_string(int status) {
  switch (status) {
    case QSA_OK: return "QSA_OK";
    case QSA_ERR_NULL_PTR: return "QSA_ERR_NULL_PTR";
    case QSA_ERR_SHAPE: return "QSA_ERR_SHAPE";
    case QSA_ERR_PARAM: return "QSA_ERR_PARAM";
    case QSA_ERR_UNSUPPORTED: return "QSA_ERR_UNSUPPORTED";
    case QSA_ERR_HIP: return "QSA_ERR_HIP";
  }
  return "QSA_ERR_UNKNOWN";
}

const char* qsa_last_error(void) { return g_err; }

int qsa_version(void) { return QSA_VERSION; }

}  // extern "C"
