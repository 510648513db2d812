// Device helpers shared by the attention backward kernels of libqsa (the float32 vector path
// and the bf16 matrix-core path): the per-element derivatives of the weight functions, dS by
// gradient mode, the per-row grid constants and the key-tile block map.  The gradient modes
// (BwdArgs::mode) are described in qsa_bwd.hip.
#pragma once

#include <type_traits>

#include "qsa_common.h"
#include "qsa_weights.h"

namespace qsa {

constexpr int SHB = 8;   // K-interval table row shift of the backward kernels: log2(64 rows * 4)
constexpr int NPARK = 8; // floats parked per row in dQ: M, MN, l, D, dm, dlo, arg-max, arg-min

// Gradient modes (the values of BwdArgs::mode)
constexpr int G_STE_POST = 0, G_EXACT = 1, G_EXACT_DET = 2, G_STE_PRE = 3, G_STE_PRE_DET = 4;
__device__ __forceinline__ bool g_ste(int mode) { return mode == G_STE_PRE || mode == G_STE_PRE_DET; }
__device__ __forceinline__ bool g_attached(int mode) { return mode == G_EXACT || mode == G_STE_PRE; }

// Per-row constants of the K-interval derivatives: the grid step Delta in score units, its
// reciprocal and 1/K (see grid_d).
struct GridD {
  float dsc, idsc, ik, pad;
};

// Per-element derivatives of the weight for the exact and pre-normalisation surrogate modes:
// gs = dw/ds (direct, score units), cm = dw/dm, clo = dw/dlo.  gd: the row's grid step, its
// reciprocal and 1/K (K-interval).  STE: the rounding of the grid coordinate is passed straight through
// where the clip to the last level is not active.  At y = K the last interval's slope applies,
// and on a min-max grid every visible key is inside (its arg-min sits on y = K up to rounding).
// w must be Weight<WK>::w of the same acc: hard rounding reads T_l off it (w = T_l there).
template <int WK, int SHT = SHB>
__device__ __forceinline__ void partials(float acc, float w, const RowC& rc, const unsigned char* Tb, int K,
                                         const GridD& gd, bool minmax, bool ste, float& gs, float& cm, float& clo) {
  gs = cm = clo = 0.0f;
  if (WK == WK_EXACT || WK == WK_EXACT_ANCH || WK == WK_TRUNC) {  // w = exp(s - m) where kept
    gs = w;
    cm = -w;
    return;
  }
  if (WK == WK_POT || WK == WK_POT_FLUSH) {  // 2^-e with e := y = (m - s) log2(e) inside the clip
    if (ste && __builtin_rintf(fmaf(acc, -rc.c, rc.mc)) <= (float)(K - 1)) {
      gs = w;
      cm = -w;
    }
    return;
  }
  if (!wk_kint(WK) || rc.c == 0.0f) return;  // uniform weights, zero-width grids
  constexpr bool INTERP = (WK == WK_KI || WK == WK_KI_FLUSH);
  constexpr bool FLUSH = (WK == WK_KH_FLUSH || WK == WK_KI_FLUSH);  // fixed-window grids only
  const float y = fmaf(acc, -rc.c, rc.mc);  // (m - s) / Delta
  const float Kf = (float)K;
  float dwdy = 0.0f, dwdD = 0.0f;           // dw/dy, and dw/dDelta at fixed y
  if (INTERP) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    if (minmax || y <= Kf) {
      const float yc = __builtin_amdgcn_fmed3f(y, 0.0f, Kf);
      const float lf = fminf(__builtin_floorf(yc), Kf - 1.0f);
      const uint32_t l = (uint32_t)(int32_t)lf;
      const float t = yc - lf;
      const f2 e = *(const f2*)(Tb + ((l << (SHT + 1)) + rc.tab));  // (T_l, T_l+1 - T_l)
      dwdy = e.y;
      dwdD = (1.0f - t) * (-lf * e.x) + t * (-(lf + 1.0f) * (e.x + e.y));
    } else if (!FLUSH) {
      const f2 e = *(const f2*)(Tb + (((uint32_t)K << (SHT + 1)) + rc.tab));
      dwdD = -Kf * e.x;
    }
  } else {
    // Hard rounding: w = T_l = exp(-l Delta), l = min(rint(max(y, 0)), K), the level the weight
    // was read at (outside a flushed window, where w = 0 and nothing moves).  Straight through,
    // dw/dy = -Delta w, so the direct term -dw/dy / Delta is w itself; at fixed y dw/dDelta =
    // -l w, and with y = (m - s) / Delta moving as well the total is w y - l w.  Written out
    // here rather than through the general form below, which would multiply by Delta and by its
    // reciprocal.
    // As in the weight (KHardW): t = y + 2^23 holds rint(y) in its low bits and the clamp of
    // t to [2^23, 2^23 + K] gives l = min(rint(max(y, 0)), K); rint(y) <= K exactly when
    // t <= 2^23 + K.  Written the same way, the compiler shares t and the clamp with the weight.
    const float t = y + 8388608.0f;
    if (!(FLUSH && y > Kf)) {
      const float lf = __builtin_amdgcn_fmed3f(t, 8388608.0f, 8388608.0f + Kf) - 8388608.0f;
      const float wo = (ste && t <= 8388608.0f + Kf) ? w : 0.0f;
      const float dD = fmaf(wo, y, -lf * w);
      gs = wo;
      cm = minmax ? fmaf(dD, gd.ik, -wo) : -wo;
      clo = minmax ? -dD * gd.ik : 0.0f;
    }
    return;
  }
  const float inv = gd.idsc;
  gs = -dwdy * inv;
  const float dD = dwdD - dwdy * y * inv;  // total dw/dDelta with y moving with Delta
  cm = dwdy * inv + (minmax ? dD * gd.ik : 0.0f);
  clo = minmax ? -dD * gd.ik : 0.0f;
}

// Per-row grid constants of the K-interval derivatives (other kinds: unused ones): the grid
// step Delta in score units, its reciprocal and 1/K, computed once per row so that no
// element pays a division.
__device__ __forceinline__ GridD grid_d(const FwdArgs& f, float M, float MN) {
  GridD g;
  g.dsc = f.window_calib ? f.window / (float)f.levels : (M - MN) * f.sc / (float)f.levels;
  g.idsc = 1.0f / g.dsc;
  g.ik = 1.0f / (float)f.levels;
  g.pad = 0.0f;
  return g;
}

// dS_ij from the weight, the row constants and dP_ij (modes as in the file header).  at_max and
// at_min: key j is the row's arg-max (arg-min), where the attached modes add the gradient of m
// (of lo on a min-max grid).
template <int WK, int SHT = SHB>
__device__ __forceinline__ float dscore(int mode, float s, float w, float dp, bool at_max, bool at_min,
                                        const RowC& rc, const unsigned char* Tb, const FwdArgs& f, float il,
                                        float Dr, float dm, float dlo, const GridD& gd, bool minmax) {
  if (mode == G_STE_POST) return (w * il) * (dp - Dr);  // il = 1 / l
  float gs, cm, clo;
  partials<WK, SHT>(s, w, rc, Tb, f.levels, gd, minmax, g_ste(mode), gs, cm, clo);
  float ds = (dp - Dr) * il * gs;
  if (g_attached(mode)) {
    if (at_max) ds += dm;
    if (at_min && minmax) ds += dlo;
  }
  return ds;
}

// dscore with the gradient mode fixed at compile time (the matrix-core kernels instantiate their
// element loops per mode, so that no per-element branch on the mode remains)
template <int WK, int SHT, int MODE>
__device__ __forceinline__ float dscore_m(float s, float w, float dp, bool at_max, bool at_min, const RowC& rc,
                                          const unsigned char* Tb, const FwdArgs& f, float il, float Dr, float dm,
                                          float dlo, const GridD& gd, bool minmax) {
  if constexpr (MODE == G_STE_POST) {
    return (w * il) * (dp - Dr);
  } else {
    constexpr bool STE = MODE == G_STE_PRE || MODE == G_STE_PRE_DET;
    constexpr bool ATT = MODE == G_EXACT || MODE == G_STE_PRE;
    float gs, cm, clo;
    partials<WK, SHT>(s, w, rc, Tb, f.levels, gd, minmax, STE, gs, cm, clo);
    const float g = fmaf(dp, il, -Dr * il);  // (dP - D) / l; D il is the same for the whole row
    if constexpr (ATT) {
      const float ext = (at_max ? dm : 0.0f) + ((at_min && minmax) ? dlo : 0.0f);
      return fmaf(g, gs, ext);
    } else {
      return g * gs;
    }
  }
}

// Calls f(std::integral_constant<int, mode>) for the runtime gradient mode.
template <class F>
__device__ __forceinline__ void with_mode(int mode, F&& f) {
  switch (mode) {
    case G_STE_POST: f(std::integral_constant<int, G_STE_POST>()); break;
    case G_EXACT: f(std::integral_constant<int, G_EXACT>()); break;
    case G_EXACT_DET: f(std::integral_constant<int, G_EXACT_DET>()); break;
    case G_STE_PRE: f(std::integral_constant<int, G_STE_PRE>()); break;
    default: f(std::integral_constant<int, G_STE_PRE_DET>()); break;
  }
}

// Offset of accumulator register r's key from the lane's first key (acc_key(r, hh) - 4 hh).
__device__ __forceinline__ constexpr int acc_off(int r) { return 8 * (r >> 2) + (r & 3); }

// Block index -> (batch * KV head, key tile) for bwd_keys, on the same principles as the
// query-tile map of the forward: each XCD (workgroup w runs on XCD w % 8) takes a contiguous
// range of KV heads, whose query heads' Q and dO it then reads through one L2; causal key tile
// kt costs nt - kt query tiles, so causal launches go in decreasing cost (ascending kt) across
// all of the XCD's KV heads when B * Hkv is a multiple of 8.
__device__ __forceinline__ void map_key_block(const FwdArgs& f, int nt, int& bkv, int& kt) {
  const int L = blockIdx.x, BKV = f.B * f.Hkv;
  if (f.causal && (BKV & 7) == 0) {
    const int j = L % BKV;
    kt = L / BKV;
    bkv = (j & 7) * (BKV >> 3) + (j >> 3);
    return;
  }
  const int T = BKV * nt, x = L & 7, slot = L >> 3;
  const int per = T >> 3, rem = T & 7;
  const int logical = x * per + (x < rem ? x : rem) + slot;
  bkv = logical / nt;
  kt = logical - bkv * nt;
}

}  // namespace qsa
