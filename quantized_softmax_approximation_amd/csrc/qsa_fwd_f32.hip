// Quantized-softmax attention forward for float32 Q/K/V (and float32 O).
//
// A correctness path for small fp32 problems, not a performance path: one
// wave per workgroup, one lane per query row, scores as fp32 FMAs over d and
// the weights kept in fp32.  The row extrema pre-pass and the weight
// functions are the same as the MFMA kernels'.  The single-pass PoT kind takes
// 64-key tiles (its anchor moves once per 64 keys, as in the MFMA kernels): a
// pass over a tile's scores for its maximum, then one for the weights.
#include "qsa_common.h"
#include "qsa_weights.h"

namespace qsa {
namespace {

constexpr int BMF = 64;  // query rows per workgroup (one wave)
constexpr int BNF = 32;  // keys per LDS tile

template <int WK>
constexpr int tile_keys() { return wk_running(WK) ? 64 : BNF; }

template <int D, int WK>
__global__ __launch_bounds__(64) void fwd_f32(FwdArgs a) {
  constexpr bool RUN = wk_running(WK);
  constexpr bool ANCH = (WK != WK_EXACT) && !RUN;
  constexpr int BT = tile_keys<WK>();  // keys per LDS tile
  constexpr int SH = 8;  // log2(BMF * 4)
  extern __shared__ __align__(16) unsigned char smem[];
  float* Ks = (float*)smem;
  float* Vs = Ks + BT * D;
  unsigned char* Tb = (unsigned char*)(Vs + BNF * D);

  const int lane = threadIdx.x;
  int bh, qt;
  map_block(a, bh, qt);
  const int b = bh / a.H, h = bh - b * a.H;
  const int kvh = h / (a.H / a.Hkv);
  const int N = a.N;
  const int q0 = qt * BMF;
  const int row = q0 + lane;
  const float* Qg = (const float*)a.q + (size_t)(b * a.H + h) * N * D;
  const float* Kg = (const float*)a.k + (size_t)(b * a.Hkv + kvh) * N * D;
  const float* Vg = (const float*)a.v + (size_t)(b * a.Hkv + kvh) * N * D;

  float q[D];
#pragma unroll
  for (int c = 0; c < D; ++c) q[c] = row < N ? Qg[(size_t)row * D + c] : 0.0f;

  const int qend = min(q0 + BMF, N);
  const int kt_end = a.causal ? ((qend - 1) / BT + 1) : (N + BT - 1) / BT;
  const int lim = a.causal ? min(row, N - 1) : N - 1;  // last key this row sees

  auto load_tile = [&](float* dst, const float* src, int kt) {
    for (int e = lane; e < BT * D; e += 64) {
      const int key = kt * BT + e / D;
      dst[e] = key < N ? src[(size_t)key * D + e % D] : 0.0f;
    }
  };
  auto score = [&](int j) {
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < D; ++c) acc = fmaf(q[c], Ks[j * D + c], acc);
    return acc;
  };

  float M = -__builtin_inff(), MN = __builtin_inff();
  if (ANCH) {
    for (int kt = 0; kt < kt_end; ++kt) {
      __syncthreads();
      load_tile(Ks, Kg, kt);
      __syncthreads();
      for (int j = 0; j < BT; ++j) {
        const int key = kt * BT + j;
        if (key <= lim) {
          const float s = score(j);
          M = fmaxf(M, s);
          MN = fminf(MN, s);
        }
      }
    }
  }
  RowC rc = make_row<WK, SH>(a, M, MN, lane, Tb, 0, 1);

  float o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) o[c] = 0.0f;
  float l = 0.0f;
  const bool dump_row = a.grid_idx != nullptr && row >= a.idx_row0 && row < a.idx_row0 + a.idx_rows && row < N;
  float A = -__builtin_inff();  // single-pass PoT: the running integer anchor, kept in rc.mc

  for (int kt = 0; kt < kt_end; ++kt) {
    __syncthreads();
    load_tile(Ks, Kg, kt);
    load_tile(Vs, Vg, kt);
    __syncthreads();
    if constexpr (RUN) {
      // A = ceil(running max of s log2 e); a rise by dA scales what was formed by 2^-dA
      float tm = -__builtin_inff();
      for (int j = 0; j < BT; ++j)
        if (kt * BT + j <= lim) tm = fmaxf(tm, score(j));
      const float An = fmaxf(A, __builtin_ceilf(tm * rc.c));
      if (An > A) {
        const float alpha = A > -__builtin_inff() ? __builtin_ldexpf(1.0f, (int)(A - An)) : 0.0f;
        l *= alpha;
#pragma unroll
        for (int c = 0; c < D; ++c) o[c] *= alpha;
        A = An;
        rc.mc = An;
      }
      for (int j = 0; j < BT; ++j) {
        const int key = kt * BT + j;
        const bool vis = key <= lim;
        const float sj = score(j);
        if (dump_row && key < N)
          a.grid_idx[((size_t)bh * a.idx_rows + (row - a.idx_row0)) * N + key] =
              (uint8_t)(vis ? Weight<WK>::idx(sj, rc, a.levels) : 255u);
        if (vis) {
          const float w = Weight<WK>::template w<SH>(sj, rc, Tb, a.levels);
          l += w;
#pragma unroll
          for (int c = 0; c < D; ++c) o[c] = fmaf(w, Vs[j * D + c], o[c]);
        }
      }
      continue;
    }
    float s[BNF];
#pragma unroll
    for (int j = 0; j < BNF; ++j) s[j] = (kt * BNF + j <= lim) ? score(j) : -__builtin_inff();
    if (WK == WK_EXACT) {
      float tm = -__builtin_inff();
#pragma unroll
      for (int j = 0; j < BNF; ++j) tm = fmaxf(tm, s[j]);
      if (tm > M) {
        const float alpha = __builtin_amdgcn_exp2f((M - tm) * rc.c);
        l *= alpha;
#pragma unroll
        for (int c = 0; c < D; ++c) o[c] *= alpha;
        M = tm;
        rc.mc = M * rc.c;
      }
    }
    if (dump_row) {
      uint8_t* dst = a.grid_idx + ((size_t)bh * a.idx_rows + (row - a.idx_row0)) * N;
      for (int j = 0; j < BNF; ++j) {
        const int key = kt * BNF + j;
        if (key < N) dst[key] = (uint8_t)(s[j] == -__builtin_inff() ? 255u : Weight<WK>::idx(s[j], rc, a.levels));
      }
    }
#pragma unroll
    for (int j = 0; j < BNF; ++j) {
      float w = Weight<WK>::template w<SH>(s[j], rc, Tb, a.levels);
      w = s[j] == -__builtin_inff() ? 0.0f : w;
      l += w;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] = fmaf(w, Vs[j * D + c], o[c]);
    }
  }

  if (row >= N) return;
  if (dump_row) {  // keys past the last tile are invisible to every row here (causal)
    uint8_t* dst = a.grid_idx + ((size_t)bh * a.idx_rows + (row - a.idx_row0)) * N;
    for (int key = kt_end * BT; key < N; ++key) dst[key] = 255u;
  }
  float* Og = (float*)a.o + (size_t)(b * a.H + h) * N * D;
  const float inv = a.vd / l;
#pragma unroll
  for (int c = 0; c < D; ++c) Og[(size_t)row * D + c] = o[c] * inv;
  const size_t ri = (size_t)bh * N + row;
  if (a.row_max) a.row_max[ri] = RUN ? A * 0.69314718055994531f : M * a.sc;  // single pass: A ln 2
  if (a.row_sum) a.row_sum[ri] = l;
  if (a.row_lo) a.row_lo[ri] = ((wk_kint(WK) && a.window_calib) || wk_support(WK)) ? M * a.sc - a.window : MN * a.sc;
}

template <int D, int WK>
hipError_t launch_one(const FwdArgs& a0, hipStream_t st) {
  FwdArgs a = a0;
  a.n_qtiles = (a.N + BMF - 1) / BMF;
  a.total_blocks = a.B * a.H * a.n_qtiles;
  const size_t lds = 2 * (size_t)tile_keys<WK>() * D * 4 + table_bytes(WK, BMF, a.levels);
  auto kern = fwd_f32<D, WK>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(a.total_blocks), dim3(64), lds, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a, int wk, hipStream_t st) {
  switch (wk) {
    case WK_EXACT: return launch_one<D, WK_EXACT>(a, st);
    case WK_EXACT_ANCH: return launch_one<D, WK_EXACT_ANCH>(a, st);
    case WK_POT: return launch_one<D, WK_POT>(a, st);
    case WK_POT_FLUSH: return launch_one<D, WK_POT_FLUSH>(a, st);
    case WK_POTR: return launch_one<D, WK_POTR>(a, st);
    case WK_POTR_FLUSH: return launch_one<D, WK_POTR_FLUSH>(a, st);
    case WK_KH: return launch_one<D, WK_KH>(a, st);
    case WK_KH_FLUSH: return launch_one<D, WK_KH_FLUSH>(a, st);
    case WK_KI: return launch_one<D, WK_KI>(a, st);
    case WK_KI_FLUSH: return launch_one<D, WK_KI_FLUSH>(a, st);
    case WK_TRUNC: return launch_one<D, WK_TRUNC>(a, st);
    case WK_UNIF: return launch_one<D, WK_UNIF>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_f32(const FwdArgs& a, int d, int wk, hipStream_t st) {
  if (d == 64) return launch_d<64>(a, wk, st);
  if (d == 128) return launch_d<128>(a, wk, st);
  return hipErrorInvalidValue;
}

}  // namespace qsa
