// Internal definitions shared by the host layer and the HIP kernels of libqsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

// Weight kinds compiled into the kernels (one instantiation each).
enum WeightKind : int {
  WK_EXACT = 0,        // online softmax (running max + rescale)
  WK_EXACT_ANCH = 1,   // exp(s - m) at the pre-pass anchor
  WK_POT = 2,          // Rowmax-PoT, saturate at L-1
  WK_POT_FLUSH = 3,    // Rowmax-PoT, e >= L -> 0
  WK_KH = 4,           // K-interval, hard rounding (saturate)
  WK_KH_FLUSH = 5,     // K-interval, hard rounding, below window -> 0
  WK_KI = 6,           // K-interval, linear interpolation
  WK_KI_FLUSH = 7,     // K-interval, interpolation, below window -> 0
  WK_TRUNC = 8,        // exp(s - m) on the support s >= m - W, else 0
  WK_UNIF = 9,         // 1 on the support s >= m - W, else 0
  WK_POTR = 10,        // single-pass PoT, running integer anchor, saturate at L-1
  WK_POTR_FLUSH = 11,  // single-pass PoT, e >= L -> 0
  WK_COUNT = 12
};

// K-interval kinds (per-row grid table) and support kinds (truncation, uniform weighting).
__host__ __device__ constexpr bool wk_kint(int wk) { return wk >= WK_KH && wk <= WK_KI_FLUSH; }
__host__ __device__ constexpr bool wk_support(int wk) { return wk == WK_TRUNC || wk == WK_UNIF; }
// Power-of-two weights, anchored at the row maximum (pre-pass) or at the running anchor.
__host__ __device__ constexpr bool wk_running(int wk) { return wk == WK_POTR || wk == WK_POTR_FLUSH; }
__host__ __device__ constexpr bool wk_pot(int wk) { return wk == WK_POT || wk == WK_POT_FLUSH || wk_running(wk); }

// Everything a launch needs; passed by value as the kernel argument.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int B, H, Hkv, N;
  int causal;
  int levels;          // K (K-interval) or L (PoT)
  int window_calib;    // K-interval: 1 = fixed window, 0 = min-max
  float window;        // W (score units) when window_calib
  float sc;            // raw accumulator -> scaled score: scale * q_descale * k_descale
  float vd;            // v_descale (epilogue)
  float* row_max;
  float* row_lo;
  float* row_sum;
  uint8_t* grid_idx;
  int idx_row0, idx_rows;
  int track_min;       // pre-pass also tracks the visible row minimum
  int n_qtiles;        // query tiles per (b, h)
  int total_blocks;    // B * H * n_qtiles
};

// Backward: the forward's arguments (shapes, kind, scale, calibration; q/k/v; o unused) plus
// the output gradient and the three input gradients (float32).
struct BwdArgs {
  FwdArgs f;
  const void* dout;   // dO [B,H,N,d], the dtype of Q
  float* dq;          // [B,H,N,d]; also holds per-row constants between the launches
  float* dk;          // [B,Hkv,N,d]
  float* dv;          // [B,Hkv,N,d]
  int mode;           // 0 straight-through, 1 exact, 2 exact with the extrema detached
  int bf16;           // inputs are bf16 (else float32)
};

// Launchers (return the HIP status of the launch).
hipError_t launch_bf16(const FwdArgs& a, int d, int wk, hipStream_t s);
hipError_t launch_fp8(const FwdArgs& a, int d, int wk, hipStream_t s);
hipError_t launch_f32(const FwdArgs& a, int d, int wk, hipStream_t s);
hipError_t launch_bwd(const BwdArgs& a, int d, int wk, hipStream_t s);
hipError_t launch_bwd_mma(const BwdArgs& a, int d, int wk, hipStream_t s);  // bf16 inputs, matrix cores

}  // namespace qsa
