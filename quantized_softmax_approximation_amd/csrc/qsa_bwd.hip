// Quantized-softmax attention backward: dQ, dK, dV of sum(dO * O), float32 math.
//
// Gradient modes.  The pages train K-interval attention with a straight-through surrogate whose
// placement relative to the normalisation they vary, derive backward rules that include the
// derivatives through the calibration, and compare attached with detached row extrema
// ("Pretraining Transformers with Quantized Softmax in Attention", abstract; chapter 5 "Build
// the method").  They print no formulas, so the modes are readings:
//   0 post-normalisation surrogate: P = w / l is passed back as a softmax of the scores,
//     dS = P (dP - D) with dP = dO V^T and D_i = dO_i . O_i; the extrema do not enter.
//   1 exact: the derivative of the forward function wherever it exists.  Through each score
//     directly (the slope of the interpolated grid line; zero for hard rounding, PoT and
//     uniform weights; w itself for the exponential kinds) and through the calibration: the
//     row maximum m moves y = (m - s)/Delta and, for min-max grids, Delta = (m - lo)/K, and the
//     row minimum lo moves Delta and with it the grid values T_l = exp(-l Delta).  Those two
//     gradients land on the row's arg-max and arg-min keys (first in key order).
//   2 exact with m and lo held constant (detached extrema).
//   3 pre-normalisation surrogate: as 1, but the rounding of the grid coordinate (K-interval
//     hard rounding, PoT) is passed straight through where the clip to the last level is not
//     active, so hard rounding gets dw/ds = w and the calibration term dw/dDelta = w (y - l).
//   4 as 3 with the extrema detached.
//
// A float32 path on the vector ALU: four lanes per query row or key (lane u of a quad holds
// four groups of four consecutive dimensions, see dim_of), fp32 FMAs, 64-row or 64-key tiles
// staged in LDS and read as 16-byte vectors, quad sums by DPP, per-row reciprocals instead of
// per-element divisions.  Three launches on the caller's stream:
//   bwd_rows  per query row, two passes over its keys: the extrema and their keys; then l, D
//             and (attached modes) the gradients of m and lo, parked in the first 8 floats
//             of the row's dQ;
//   bwd_keys  per key: dK and dV, summed over the query heads that read the key's KV head;
//   bwd_dq    per query row: dQ (it reads its parked constants, then overwrites the row).
// Every launch computes scores with the same operation order, so the three agree exactly on
// every weight.
#include "qsa_bwd_common.h"
#include "qsa_common.h"
#include "qsa_weights.h"

namespace qsa {
namespace {

constexpr int TB = 64;   // rows or keys per workgroup (one quad each)
static_assert(SHB == 8, "the table shift matches TB rows");

template <typename T>
__device__ __forceinline__ float ld(const T* p) {
  return (float)*p;
}

// Sum over the four lanes of a quad with DPP lane permutes (quad_perm 1,0,3,2 then 2,3,0,1):
// every lane ends with (x0 + x1) + (x2 + x3), with no LDS round trip.
__device__ __forceinline__ float quad_sum(float x) {
  x += bitsf((uint32_t)__builtin_amdgcn_mov_dpp((int)fbits(x), 0xB1, 0xF, 0xF, false));
  x += bitsf((uint32_t)__builtin_amdgcn_mov_dpp((int)fbits(x), 0x4E, 0xF, 0xF, false));
  return x;
}

typedef float f4 __attribute__((ext_vector_type(4)));

// Dimension held in register k of lane u of a quad: groups of four consecutive dimensions,
// 16k' + 4u .. 16k' + 4u + 3 for k = 4k' .. 4k' + 3, so a lane reads a 16-byte LDS vector per
// four FMAs and the four lanes of a quad cover 16 consecutive words (no bank conflicts; every
// quad of a wave reads the same words, a broadcast).
__device__ __forceinline__ int dim_of(int k, int u) { return 16 * (k >> 2) + 4 * u + (k & 3); }

// x . row for the quad: four partial sums (one per vector component, four FMA chains in
// flight), then the quad adds up
template <int D>
__device__ __forceinline__ float qdot(const float* row, const float (&x)[D / 4], int u) {
  float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k4 = 0; k4 < D / 16; ++k4) {
    const f4 r = *(const f4*)(row + 16 * k4 + 4 * u);
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fmaf(x[4 * k4 + i], r[i], p[i]);
  }
  return quad_sum((p[0] + p[1]) + (p[2] + p[3]));
}

// acc += a * row (the quad's dimensions of one LDS row)
template <int D>
__device__ __forceinline__ void qaxpy(float a, const float* row, float (&acc)[D / 4], int u) {
#pragma unroll
  for (int k4 = 0; k4 < D / 16; ++k4) {
    const f4 r = *(const f4*)(row + 16 * k4 + 4 * u);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[4 * k4 + i] = fmaf(a, r[i], acc[4 * k4 + i]);
  }
}

template <typename T, int D, int WK>
__global__ __launch_bounds__(256) void bwd_rows(BwdArgs a) {
  const FwdArgs& f = a.f;
  constexpr int DL = D / 4;
  extern __shared__ __align__(16) unsigned char smem[];
  float* Ks = (float*)smem;
  float* Vs = Ks + TB * D;
  unsigned char* Tb = (unsigned char*)(Vs + TB * D);

  const int tid = threadIdx.x, rl = tid >> 2, u = tid & 3;
  int bh, qt;
  map_block(f, bh, qt);
  const int b = bh / f.H, h = bh - b * f.H;
  const int kvh = h / (f.H / f.Hkv);
  const int N = f.N;
  const int row = qt * TB + rl;
  const T* Qg = (const T*)f.q + (size_t)(b * f.H + h) * N * D;
  const T* Gg = (const T*)a.dout + (size_t)(b * f.H + h) * N * D;
  const T* Kg = (const T*)f.k + (size_t)(b * f.Hkv + kvh) * N * D;
  const T* Vg = (const T*)f.v + (size_t)(b * f.Hkv + kvh) * N * D;

  float q[DL], g[DL];
#pragma unroll
  for (int k = 0; k < DL; ++k) {
    q[k] = row < N ? ld(Qg + (size_t)row * D + dim_of(k, u)) : 0.0f;
    g[k] = row < N ? ld(Gg + (size_t)row * D + dim_of(k, u)) : 0.0f;
  }
  const int kt_end = f.causal ? ((min(qt * TB + TB, N) - 1) / TB + 1) : (N + TB - 1) / TB;
  const int lim = row < N ? (f.causal ? row : N - 1) : -1;  // last key this row sees
  auto load_tile = [&](float* dst, const T* src, int kt) {
    for (int e = tid; e < TB * D; e += 256) {
      const int key = kt * TB + e / D;
      dst[e] = key < N ? ld(src + (size_t)key * D + e % D) : 0.0f;
    }
  };

  // extrema over the visible keys and the first keys that reach them
  float M = -__builtin_inff(), MN = __builtin_inff();
  int amax = -1, amin = -1;
  for (int kt = 0; kt < kt_end; ++kt) {
    __syncthreads();
    load_tile(Ks, Kg, kt);
    __syncthreads();
#pragma unroll 4
    for (int j = 0; j < TB; ++j) {
      const int key = kt * TB + j;
      const float s = qdot<D>(Ks + j * D, q, u);
      if (key <= lim) {
        if (s > M) { M = s; amax = key; }
        if (s < MN) { MN = s; amin = key; }
      }
    }
  }
  if (row >= N) M = MN = 0.0f;
  const RowC rc = make_row<WK, SHB>(f, M, MN, rl, Tb, u, 4);
  const GridD gd = grid_d(f, M, MN);
  const bool minmax = wk_kint(WK) && !f.window_calib;

  // l, D = sum_j P_ij dP_ij (= dO_i . O_i) and, with the extrema attached, the gradients of m
  // and lo: dm = sum_j (dP_ij - D) cm_ij / l is linear in D, so one pass gathers
  // sum dP cm and sum cm (likewise for lo) before D is known
  const bool calib = g_attached(a.mode) &&
                     (WK == WK_TRUNC || wk_kint(WK) || ((WK == WK_POT || WK == WK_POT_FLUSH) && g_ste(a.mode)));
  float l = 0.0f, wdp = 0.0f, pm = 0.0f, sm = 0.0f, plo = 0.0f, slo = 0.0f;
  for (int kt = 0; kt < kt_end; ++kt) {
    __syncthreads();
    load_tile(Ks, Kg, kt);
    load_tile(Vs, Vg, kt);
    __syncthreads();
#pragma unroll 4
    for (int j = 0; j < TB; ++j) {
      const float s = qdot<D>(Ks + j * D, q, u);
      const float dp = qdot<D>(Vs + j * D, g, u);
      if (kt * TB + j <= lim) {
        const float w = Weight<WK>::template w<SHB>(s, rc, Tb, f.levels);
        l += w;
        wdp = fmaf(w, dp, wdp);
        if (calib) {
          float gs, cm, clo;
          partials<WK>(s, w, rc, Tb, f.levels, gd, minmax, g_ste(a.mode), gs, cm, clo);
          pm = fmaf(dp, cm, pm);
          sm += cm;
          plo = fmaf(dp, clo, plo);
          slo += clo;
        }
      }
    }
  }
  const float Dr = row < N ? wdp / l : 0.0f;
  const float dm = calib && row < N ? fmaf(-Dr, sm, pm) / l : 0.0f;
  const float dlo = calib && row < N ? fmaf(-Dr, slo, plo) / l : 0.0f;
  if (row < N && u == 0) {
    float* pk = a.dq + ((size_t)(b * f.H + h) * N + row) * D;
    pk[0] = M;
    pk[1] = MN;
    pk[2] = l;
    pk[3] = Dr;
    pk[4] = dm;
    pk[5] = dlo;
    pk[6] = __builtin_bit_cast(float, amax);
    pk[7] = __builtin_bit_cast(float, amin);
  }
}

// Waves per SIMD the register budget of bwd_keys is sized for: 4 at d = 64 (at most 128 VGPRs,
// 12-40 bytes spilled; the GPT-2 shaped backward measured 5 % faster than at the 140 VGPRs and 3
// waves the compiler picks unbounded), no bound otherwise (d = 128 spills kilobytes at 4, and the
// interpolation kinds, which spill most at d = 64, measured 1 % slower with it).
template <int D, int WK>
constexpr int keys_waves() {
  return (D == 64 && WK != WK_KI && WK != WK_KI_FLUSH) ? 4 : 1;
}

template <typename T, int D, int WK>
__global__ __launch_bounds__(256, (keys_waves<D, WK>())) void bwd_keys(BwdArgs a) {
  const FwdArgs& f = a.f;
  constexpr int DL = D / 4;
  extern __shared__ __align__(16) unsigned char smem[];
  float* Qs = (float*)smem;
  float* Gs = Qs + TB * D;
  float* Rp = Gs + TB * D;                               // [TB][NPARK] parked row constants (1/l for l)
  RowC* Rc = (RowC*)(Rp + TB * NPARK);                   // [TB] row constants
  GridD* Rg = (GridD*)(Rc + TB);                         // [TB] grid constants of the derivatives
  unsigned char* Tb = (unsigned char*)(Rg + TB);

  const int tid = threadIdx.x, kl = tid >> 2, u = tid & 3;
  const int N = f.N, nt = (N + TB - 1) / TB;
  int bkv, kt;
  map_key_block(f, nt, bkv, kt);
  const int b = bkv / f.Hkv, kvh = bkv - b * f.Hkv;
  const int group = f.H / f.Hkv;
  const int key = kt * TB + kl;
  const T* Kg = (const T*)f.k + (size_t)(b * f.Hkv + kvh) * N * D;
  const T* Vg = (const T*)f.v + (size_t)(b * f.Hkv + kvh) * N * D;
  float kk[DL], vv[DL], dk[DL], dv[DL];
#pragma unroll
  for (int k = 0; k < DL; ++k) {
    kk[k] = key < N ? ld(Kg + (size_t)key * D + dim_of(k, u)) : 0.0f;
    vv[k] = key < N ? ld(Vg + (size_t)key * D + dim_of(k, u)) : 0.0f;
    dk[k] = dv[k] = 0.0f;
  }
  const bool minmax = wk_kint(WK) && !f.window_calib;

  for (int hq = kvh * group; hq < (kvh + 1) * group; ++hq) {
    const T* Qg = (const T*)f.q + (size_t)(b * f.H + hq) * N * D;
    const T* Gg = (const T*)a.dout + (size_t)(b * f.H + hq) * N * D;
    const float* Pk = a.dq + (size_t)(b * f.H + hq) * N * D;
    for (int qt = f.causal ? kt : 0; qt < nt; ++qt) {
      __syncthreads();
      for (int e = tid; e < TB * D; e += 256) {
        const int r = qt * TB + e / D;
        Qs[e] = r < N ? ld(Qg + (size_t)r * D + e % D) : 0.0f;
        Gs[e] = r < N ? ld(Gg + (size_t)r * D + e % D) : 0.0f;
      }
      // quad kl takes row kl of the tile: its parked constants and its grid table
      {
        const int r = qt * TB + kl;
        float pk[NPARK];
#pragma unroll
        for (int c = 0; c < NPARK; ++c) pk[c] = r < N ? Pk[(size_t)r * D + c] : 0.0f;
        const RowC rc = make_row<WK, SHB>(f, pk[0], pk[1], kl, Tb, u, 4);
        if (u == 0) {
#pragma unroll
          for (int c = 0; c < NPARK; ++c) Rp[kl * NPARK + c] = pk[c];
          Rp[kl * NPARK + 2] = 1.0f / pk[2];  // l >= 1 on a row (its maximum weighs 1); unused past N
          Rc[kl] = rc;
          Rg[kl] = grid_d(f, pk[0], pk[1]);
        }
      }
      __syncthreads();
#pragma unroll 4
      for (int r = 0; r < TB; ++r) {
        const int i = qt * TB + r;
        if (i >= N) break;
        const float s = qdot<D>(Qs + r * D, kk, u);
        const float dp = qdot<D>(Gs + r * D, vv, u);
        if (key < N && (!f.causal || key <= i)) {
          const RowC rc = Rc[r];
          const float* pk = Rp + r * NPARK;
          const float w = Weight<WK>::template w<SHB>(s, rc, Tb, f.levels);
          const float il = pk[2];
          const float ds = dscore<WK>(a.mode, s, w, dp, key == __builtin_bit_cast(int, pk[6]),
                                      key == __builtin_bit_cast(int, pk[7]), rc, Tb, f, il, pk[3], pk[4], pk[5], Rg[r],
                                      minmax);
          qaxpy<D>(w * il, Gs + r * D, dv, u);
          qaxpy<D>(ds, Qs + r * D, dk, u);
        }
      }
    }
  }
  if (key < N) {
    float* dKg = a.dk + ((size_t)(b * f.Hkv + kvh) * N + key) * D;
    float* dVg = a.dv + ((size_t)(b * f.Hkv + kvh) * N + key) * D;
#pragma unroll
    for (int k = 0; k < DL; ++k) {
      dKg[dim_of(k, u)] = f.sc * dk[k];
      dVg[dim_of(k, u)] = dv[k];
    }
  }
}

template <typename T, int D, int WK>
__global__ __launch_bounds__(256) void bwd_dq(BwdArgs a) {
  const FwdArgs& f = a.f;
  constexpr int DL = D / 4;
  extern __shared__ __align__(16) unsigned char smem[];
  float* Ks = (float*)smem;
  float* Vs = Ks + TB * D;
  unsigned char* Tb = (unsigned char*)(Vs + TB * D);

  const int tid = threadIdx.x, rl = tid >> 2, u = tid & 3;
  int bh, qt;
  map_block(f, bh, qt);
  const int b = bh / f.H, h = bh - b * f.H;
  const int kvh = h / (f.H / f.Hkv);
  const int N = f.N;
  const int row = qt * TB + rl;
  const T* Qg = (const T*)f.q + (size_t)(b * f.H + h) * N * D;
  const T* Gg = (const T*)a.dout + (size_t)(b * f.H + h) * N * D;
  const T* Kg = (const T*)f.k + (size_t)(b * f.Hkv + kvh) * N * D;
  const T* Vg = (const T*)f.v + (size_t)(b * f.Hkv + kvh) * N * D;
  float* dQg = a.dq + ((size_t)(b * f.H + h) * N + row) * D;

  float q[DL], g[DL], dq[DL];
  float pk[NPARK];
#pragma unroll
  for (int k = 0; k < DL; ++k) {
    q[k] = row < N ? ld(Qg + (size_t)row * D + dim_of(k, u)) : 0.0f;
    g[k] = row < N ? ld(Gg + (size_t)row * D + dim_of(k, u)) : 0.0f;
    dq[k] = 0.0f;
  }
#pragma unroll
  for (int c = 0; c < NPARK; ++c) pk[c] = row < N ? dQg[c] : 0.0f;  // before the row is overwritten
  const RowC rc = make_row<WK, SHB>(f, pk[0], pk[1], rl, Tb, u, 4);
  const GridD gd = grid_d(f, pk[0], pk[1]);
  const float il = 1.0f / pk[2];  // unused past N (no visible key)
  const bool minmax = wk_kint(WK) && !f.window_calib;
  const int amax = __builtin_bit_cast(int, pk[6]), amin = __builtin_bit_cast(int, pk[7]);
  const int kt_end = f.causal ? ((min(qt * TB + TB, N) - 1) / TB + 1) : (N + TB - 1) / TB;
  const int lim = row < N ? (f.causal ? row : N - 1) : -1;
  auto load_tile = [&](float* dst, const T* src, int kt) {
    for (int e = tid; e < TB * D; e += 256) {
      const int key = kt * TB + e / D;
      dst[e] = key < N ? ld(src + (size_t)key * D + e % D) : 0.0f;
    }
  };
  for (int kt = 0; kt < kt_end; ++kt) {
    __syncthreads();
    load_tile(Ks, Kg, kt);
    load_tile(Vs, Vg, kt);
    __syncthreads();
#pragma unroll 4
    for (int j = 0; j < TB; ++j) {
      const int key = kt * TB + j;
      const float s = qdot<D>(Ks + j * D, q, u);
      const float dp = qdot<D>(Vs + j * D, g, u);
      if (key <= lim) {
        const float w = Weight<WK>::template w<SHB>(s, rc, Tb, f.levels);
        const float ds = dscore<WK>(a.mode, s, w, dp, key == amax, key == amin, rc, Tb, f, il, pk[3], pk[4], pk[5],
                                    gd, minmax);
        qaxpy<D>(ds, Ks + j * D, dq, u);
      }
    }
  }
  if (row < N) {
#pragma unroll
    for (int k = 0; k < DL; ++k) dQg[dim_of(k, u)] = f.sc * dq[k];
  }
}

template <typename T, int D, int WK>
hipError_t launch_typed(const BwdArgs& a0, hipStream_t st) {
  BwdArgs a = a0;
  a.f.n_qtiles = (a.f.N + TB - 1) / TB;
  a.f.total_blocks = a.f.B * a.f.H * a.f.n_qtiles;
  const size_t tab = table_bytes(WK, TB, a.f.levels);
  const size_t lds_rows = 2 * (size_t)TB * D * 4 + tab;
  const size_t lds_keys =
      2 * (size_t)TB * D * 4 + (size_t)TB * NPARK * 4 + (size_t)TB * sizeof(RowC) + (size_t)TB * sizeof(GridD) + tab;
  const void* ks[3] = {(const void*)bwd_rows<T, D, WK>, (const void*)bwd_keys<T, D, WK>, (const void*)bwd_dq<T, D, WK>};
  const size_t lds[3] = {lds_rows, lds_keys, lds_rows};
  for (int i = 0; i < 3; ++i)
    if (lds[i] > 65536) {
      const hipError_t e = hipFuncSetAttribute(ks[i], hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds[i]);
      if (e != hipSuccess) return e;
    }
  hipLaunchKernelGGL((bwd_rows<T, D, WK>), dim3(a.f.total_blocks), dim3(256), lds_rows, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int key_blocks = a.f.B * a.f.Hkv * ((a.f.N + TB - 1) / TB);
  hipLaunchKernelGGL((bwd_keys<T, D, WK>), dim3(key_blocks), dim3(256), lds_keys, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq<T, D, WK>), dim3(a.f.total_blocks), dim3(256), lds_rows, st, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_kind(const BwdArgs& a, int wk, hipStream_t st) {
  switch (wk) {
    case WK_EXACT:
    case WK_EXACT_ANCH: return launch_typed<T, D, WK_EXACT_ANCH>(a, st);  // the same function
    case WK_POT: return launch_typed<T, D, WK_POT>(a, st);
    case WK_POT_FLUSH: return launch_typed<T, D, WK_POT_FLUSH>(a, st);
    case WK_KH: return launch_typed<T, D, WK_KH>(a, st);
    case WK_KH_FLUSH: return launch_typed<T, D, WK_KH_FLUSH>(a, st);
    case WK_KI: return launch_typed<T, D, WK_KI>(a, st);
    case WK_KI_FLUSH: return launch_typed<T, D, WK_KI_FLUSH>(a, st);
    case WK_TRUNC: return launch_typed<T, D, WK_TRUNC>(a, st);
    case WK_UNIF: return launch_typed<T, D, WK_UNIF>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int d, int wk, hipStream_t st) {
  if (a.bf16) return launch_bwd_mma(a, d, wk, st);  // bf16 inputs: the matrix-core path (qsa_bwd_mma.hip)
  {
    if (d == 64) return launch_kind<float, 64>(a, wk, st);
    if (d == 128) return launch_kind<float, 128>(a, wk, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace qsa
