// Per-element weight functions of the quantized-softmax attention forward
// (device code shared by every kernel of libqsa).
//
// Every function takes the raw score accumulator `acc` (the dot product of a
// query and a key in the units the MMA produced) and per-row constants in the
// same units, so the score scale is folded into the constants once per row:
//
//   y = (M - acc) * c     M = row maximum of acc over the visible keys
//
// exact / PoT / support kinds: c = scale * log2(e), so y = (m - s) log2(e);
// K-interval:  c = scale / Delta,   so y = (m - s) / Delta.
//
// Rowmax-PoT ("Approximating Softmax in Pretrained LLMs", abstract; the wiki
// summary's flowchart "Row max -> Power-of-two weights"): w = 2^-e with
// e = rint(y) clipped to L-1.  The weight is built in the float's exponent
// field with integer operations; no exponential is evaluated.
//
// K-interval attention ("Pretraining Transformers with Quantized Softmax in
// Attention", abstract and chapter 1): w is read off a table of K+1 grid
// values T_l = exp(-l Delta) kept per row in LDS; hard rounding takes the
// nearest grid point, interpolation the straight line between neighbours.
//
// Support truncation and uniform weighting (the sensitivity study of
// "Approximating Softmax in Pretrained LLMs", abstract): keys with
// s >= m - W keep exp(s - m) or 1, the others get 0; in y units the edge is
// y = W log2(e) (RowC::cut).
#pragma once

#include "qsa_common.h"

namespace qsa {

__device__ __forceinline__ uint32_t fbits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float bitsf(uint32_t x) { return __builtin_bit_cast(float, x); }

constexpr float kLog2e = 1.4426950408889634f;

// Per-row constants.
struct RowC {
  float c;      // multiplier on (M - acc)
  float mc;     // M * c
  uint32_t tab; // K-interval: byte offset of this row's column in the LDS table
  float cut;    // support kinds: the support edge W log2(e) in y units
  float step;   // K-interval: -Delta log2(e) (score units), so T_l = 2^(l step)
};

// Table layout (K-interval): entry l of local row r sits at byte
// (l * ROWS + r) * 4 (hard: T_l) or (l * ROWS + r) * 8 (interpolation:
// T_l, T_{l+1} - T_l).  Consecutive rows fall in consecutive banks, so the
// 32 rows of a half-wave look up their own tables without bank conflicts.
// SH = log2(ROWS * 4).

template <int WK> struct Weight;

// Exact exponential (both the online control and the anchored variant).
template <int WK> struct ExactW {
  template <int SH>
  static __device__ __forceinline__ float w(float acc, const RowC& r, const unsigned char*, int) {
    return __builtin_amdgcn_exp2f(fmaf(acc, r.c, -r.mc));
  }
  static __device__ __forceinline__ uint32_t idx(float, const RowC&, int) { return 0u; }
};
template <> struct Weight<WK_EXACT> : ExactW<WK_EXACT> {};
template <> struct Weight<WK_EXACT_ANCH> : ExactW<WK_EXACT_ANCH> {};

// Rowmax-PoT.  t = 2^24 - y is rounded by the subtraction itself to an
// integer (the float spacing in [2^23, 2^24] is 1), ties to even; since 2^24
// is even, t and e = 2^24 - t have the same parity, so e = rint(y) with ties
// to even.  bits(t) = 0x4B800000 - e, and shifting it left by 23 leaves
// -e << 23 (the exponent bits of 2^24 shift out), so adding 127 << 23 gives the
// binary32 pattern of 2^-e.  The clip e <= L-1 is an integer max on bits(t).
template <bool FLUSH> struct PotW {
  template <int SH>
  static __device__ __forceinline__ float w(float acc, const RowC& r, const unsigned char*, int L) {
    const float y = fmaf(acc, -r.c, r.mc);
    int32_t tb = (int32_t)fbits(16777216.0f - y);
    const int32_t lo = 0x4B800000 - (L - 1);
    if (FLUSH) {
      if (tb < lo) return 0.0f;
    } else {
      tb = tb > lo ? tb : lo;
    }
    return bitsf(((uint32_t)tb << 23) + (127u << 23));
  }
  static __device__ __forceinline__ uint32_t idx(float acc, const RowC& r, int L) {
    const float y = fmaf(acc, -r.c, r.mc);
    int32_t tb = (int32_t)fbits(16777216.0f - y);
    const int32_t lo = 0x4B800000 - (L - 1);
    if (tb < lo) return FLUSH ? 254u : (uint32_t)(L - 1);
    return (uint32_t)(0x4B800000 - tb);
  }
};
template <> struct Weight<WK_POT> : PotW<false> {};
template <> struct Weight<WK_POT_FLUSH> : PotW<true> {};
// Single-pass PoT: the same exponent against the running integer anchor A, which the kernel
// keeps in RowC::mc (with c = scale log2 e, y = A - acc c).
template <> struct Weight<WK_POTR> : PotW<false> {};
template <> struct Weight<WK_POTR_FLUSH> : PotW<true> {};

// K-interval, hard rounding.  t = y + 2^23 rounds y to the nearest integer
// (ties to even) inside the float: bits(t) = 0x4B000000 + l.  The clip of l to
// [0, K] is one v_med3_f32 on t (on [2^23, 2^23 + K] floats order as their bit
// patterns; the lower end keeps the lookup in the table when rounding puts the
// score a little above the anchor); (bits(t) << SH) drops the 0x4B000000 part
// (SH >= 8) and leaves l * ROWS * 4, the table offset of entry l.
template <bool FLUSH> struct KHardW {
  static __device__ __forceinline__ int32_t level_bits(float y, int K) {
    return (int32_t)fbits(__builtin_amdgcn_fmed3f(y + 8388608.0f, 8388608.0f, 8388608.0f + (float)K));
  }
  template <int SH>
  static __device__ __forceinline__ float w(float acc, const RowC& r, const unsigned char* tab, int K) {
    const float y = fmaf(acc, -r.c, r.mc);
    const int32_t tb = level_bits(y, K);
    const float wv = *(const float*)(tab + (((uint32_t)tb << SH) + r.tab));
    if (FLUSH && y > (float)K) return 0.0f;
    return wv;
  }
  static __device__ __forceinline__ uint32_t idx(float acc, const RowC& r, int K) {
    const float y = fmaf(acc, -r.c, r.mc);
    if (FLUSH && y > (float)K) return 254u;
    return (uint32_t)(level_bits(y, K) - 0x4B000000);
  }
};
template <> struct Weight<WK_KH> : KHardW<false> {};
template <> struct Weight<WK_KH_FLUSH> : KHardW<true> {};

// K-interval, linear interpolation between T_l and T_{l+1}, l = floor(y)
// (y clipped to [0, K]; at y = K the slope entry is 0, giving T_K).
template <bool FLUSH> struct KInterpW {
  template <int SH>
  static __device__ __forceinline__ float w(float acc, const RowC& r, const unsigned char* tab, int K) {
    const float y = fmaf(acc, -r.c, r.mc);
    const float yc = __builtin_amdgcn_fmed3f(y, 0.0f, (float)K);
    const float fl = __builtin_floorf(yc);
    const float t = yc - fl;
    const uint32_t l = (uint32_t)(int32_t)fl;
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 e = *(const f2*)(tab + ((l << (SH + 1)) + r.tab));
    if (FLUSH && y > (float)K) return 0.0f;
    return fmaf(t, e.y, e.x);
  }
  static __device__ __forceinline__ uint32_t idx(float acc, const RowC& r, int K) {
    const float y = fmaf(acc, -r.c, r.mc);
    if (FLUSH && y > (float)K) return 254u;
    const float yc = __builtin_amdgcn_fmed3f(y, 0.0f, (float)K);
    return (uint32_t)(int32_t)__builtin_floorf(yc);
  }
};
template <> struct Weight<WK_KI> : KInterpW<false> {};
template <> struct Weight<WK_KI_FLUSH> : KInterpW<true> {};

// Support truncation (UNIF = false) and uniform weighting (UNIF = true).
template <bool UNIF> struct SupportW {
  template <int SH>
  static __device__ __forceinline__ float w(float acc, const RowC& r, const unsigned char*, int) {
    const float y = fmaf(acc, -r.c, r.mc);
    if (y > r.cut) return 0.0f;
    return UNIF ? 1.0f : __builtin_amdgcn_exp2f(-y);
  }
  static __device__ __forceinline__ uint32_t idx(float acc, const RowC& r, int) {
    return fmaf(acc, -r.c, r.mc) > r.cut ? 254u : 0u;
  }
};
template <> struct Weight<WK_TRUNC> : SupportW<false> {};
template <> struct Weight<WK_UNIF> : SupportW<true> {};

// Per-row constants from the pre-pass extrema (raw units) and, for
// K-interval, the row's grid table written into LDS (unless `tab` is null:
// the weights then evaluate T_l = 2^(l step) from the index with the same
// instruction, which gives the same values without the table).  The K+1
// table entries are split between the `nsplit` lanes that share a row (this
// lane writes entries part, part + nsplit, ...).  TMODE picks the layout of
// the interpolation table (the hard-rounding table is T_l alone in every mode):
//   TAB_PAIRS  (T_l, T_l+1 - T_l), 8 bytes per entry;
//   TAB_T      T_l alone (the kernel forms T_l+1 from T_l);
//   TAB_SLOPE  the line of interval l as a function of the raw score difference
//              x = s - m (y = -c x): (A_l, B_l) with A_l = T_l - l (T_l+1 - T_l) and
//              B_l = -c (T_l+1 - T_l), so that the weight on [l, l+1] is
//              A_l + B_l x = T_l + (y - l)(T_l+1 - T_l); entry K is (T_K, 0), or
//              (0, 0) for the flushing kind, whose weight is 0 once floor(y) >= K.
enum : int { TAB_PAIRS = 0, TAB_T = 1, TAB_SLOPE = 2 };
template <int WK, int SH, int TMODE = TAB_PAIRS>
__device__ __forceinline__ RowC make_row(const FwdArgs& a, float M, float MN, int row_local,
                                         unsigned char* tab, int part, int nsplit) {
  RowC rc;
  rc.tab = 0;
  rc.cut = a.window * kLog2e;
  rc.step = 0.0f;
  if (!wk_kint(WK)) {
    rc.c = a.sc * kLog2e;
    rc.mc = M * rc.c;
    return rc;
  }
  const int K = a.levels;
  float delta_s;  // grid step in score units
  if (a.window_calib) {
    delta_s = a.window / (float)K;
    rc.c = a.sc * (float)K / a.window;
  } else {
    const float range = M - MN;
    rc.c = range > 0.0f ? (float)K / range : 0.0f;  // zero-width grid: every weight T_0 = 1
    delta_s = range * a.sc / (float)K;
  }
  rc.mc = M * rc.c;
  const float step = -delta_s * kLog2e;
  rc.step = step;
  constexpr bool INTERP = (WK == WK_KI || WK == WK_KI_FLUSH) && TMODE != TAB_T;
  constexpr int ROWS = (1 << SH) / 4;
  rc.tab = (uint32_t)row_local * (INTERP ? 8u : 4u);
  if (tab == nullptr) return rc;
  for (int l = part; l <= K; l += nsplit) {
    const float t0 = __builtin_amdgcn_exp2f(step * (float)l);
    if (INTERP) {
      const float t1 = (l < K) ? __builtin_amdgcn_exp2f(step * (float)(l + 1)) : t0;
      typedef float f2 __attribute__((ext_vector_type(2)));
      f2 e = {t0, t1 - t0};
      if (TMODE == TAB_SLOPE) {
        e = f2{fmaf(-(float)l, e.y, t0), -rc.c * e.y};
        if (WK == WK_KI_FLUSH && l == K) e = f2{0.0f, 0.0f};
      }
      *(f2*)(tab + ((size_t)l * ROWS + row_local) * 8) = e;
    } else {
      *(float*)(tab + ((size_t)l * ROWS + row_local) * 4) = t0;
    }
  }
  return rc;
}

// K-interval interpolation without the table: (T_l, T_{l+1} - T_l) for the index fl = l (a
// float), the entry the table would hold (at l = K the table's difference is 0, but there the
// interpolation parameter is 0 as well, so the weight is the same).
__device__ __forceinline__ float __attribute__((ext_vector_type(2))) kgrid_pair(float step, float fl) {
  const float t0 = __builtin_amdgcn_exp2f(step * fl);
  const float t1 = __builtin_amdgcn_exp2f(step * (fl + 1.0f));
  return {t0, t1 - t0};
}

// Table bytes a workgroup of ROWS rows needs for weight kind WK.
__host__ __device__ inline size_t table_bytes(int wk, int rows, int K) {
  if (wk == WK_KH || wk == WK_KH_FLUSH) return (size_t)rows * (K + 1) * 4;
  if (wk == WK_KI || wk == WK_KI_FLUSH) return (size_t)rows * (K + 1) * 8;
  return 0;
}

// Block index -> (batch*head, query tile).  Workgroups are dispatched round-
// robin over the 8 XCDs (workgroup w runs on XCD w % 8); the remap gives each
// XCD a contiguous range of heads, so the query tiles of one head (and the
// heads of one GQA group) share an XCD and its L2 while they sweep the same
// K/V.  Causal launches, whose query tile t costs t + 1 key tiles, are ordered
// longest first across all of the XCD's heads (list scheduling in decreasing
// cost), so the last workgroups to start are the shortest; taking each head's
// tiles in turn instead left one head's long tiles starting late (when the
// row count per head is below what an XCD holds at once).  That needs B*H to
// be a multiple of 8; otherwise the causal order is longest first per head.
__device__ __forceinline__ void map_block(const FwdArgs& a, int& bh, int& qt) {
  const int L = blockIdx.x, T = a.total_blocks;
  const int BH = a.B * a.H;
  if (a.causal && (BH & 7) == 0) {
    const int j = L % BH, t = L / BH;  // workgroup L runs on XCD L % 8 = j % 8
    bh = (j & 7) * (BH >> 3) + (j >> 3);
    qt = a.n_qtiles - 1 - t;
    return;
  }
  const int x = L & 7, slot = L >> 3;
  const int per = T >> 3, rem = T & 7;
  const int logical = x * per + (x < rem ? x : rem) + slot;
  bh = logical / a.n_qtiles;
  const int t = logical - bh * a.n_qtiles;
  qt = a.causal ? (a.n_qtiles - 1 - t) : t;
}

}  // namespace qsa
