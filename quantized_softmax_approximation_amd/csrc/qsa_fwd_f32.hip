// Quantized-softmax attention forward for float32 Q/K/V (and float32 O) on the matrix cores
// (v_mfma_f32_32x32x2_f32): scores and PV in fp32 with fp32 accumulation, the weights kept in
// fp32.  The row-extrema pre-pass, the weight functions (Weight<WK> in qsa_weights.h) and the
// single-pass anchor (tiles of 64 keys) are those of the bf16 and fp8 kernels; the structure is
// simpler (one LDS tile of K and V, loaded between two barriers), as this path serves fp32
// inputs, which the pages do not time.
#include "qsa_common.h"
#include "qsa_mfma_util.h"
#include "qsa_weights.h"

namespace qsa {
namespace {

// ---- fp32 on the matrix cores (v_mfma_f32_32x32x2_f32) ----------------------------------------
// A workgroup is 4 waves = 128 query rows; a wave owns 32 rows.  Scores are computed transposed,
// S^T = K Q^T, one MMA per pair of feature columns: in k-step s lane (i, h) gives K[key i][2s + h]
// and Q[row i][2s + h], and the accumulator holds key acc_key(r, h) of row i in register r (the
// layout of every 32x32 MMA).  The weights stay in those registers and are the B operand of
// O^T += V^T P^T: k-step s of a 32-key block takes the key of register s, so lane (c, h) gives
// V[key acc_key(s, h)][c].  Tiles of 64 keys (the single-pass anchor's tile) in LDS with padded
// rows: K rows D + 2 floats apart (the k-step reads of a wave fall in distinct banks), V rows
// D + 8 apart (the two half-waves read rows four apart, half the banks away).
constexpr int MW = 4;         // waves per workgroup
constexpr int MBM = MW * 32;  // query rows per workgroup
constexpr int MBN = 64;       // keys per tile
constexpr int MSH = 9;        // log2(MBM * 4): the K-interval table stride

template <int D, int WK>
__global__ __launch_bounds__(MW * 64) void fwd_f32(FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr bool RUN = wk_running(WK);
  constexpr bool ANCH = (WK != WK_EXACT) && !RUN;
  constexpr int KS = D + 2, VS = D + 8, DB = D / 32, NS = D / 2;
  extern __shared__ __align__(16) unsigned char smem[];
  float* const Ks = (float*)smem;
  float* const Vs = Ks + MBN * KS;
  unsigned char* const Tb = (unsigned char*)(Vs + MBN * VS);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = tid >> 6, li = lane & 31, hh = lane >> 5;
  int bh, qt;
  map_block(a, bh, qt);
  const int b = bh / a.H, h = bh - b * a.H;
  const int kvh = h / (a.H / a.Hkv);
  const int N = a.N;
  const int q0 = qt * MBM, row = q0 + wave * 32 + li;
  const float* Qg = (const float*)a.q + (size_t)(b * a.H + h) * N * D;
  const float* Kg = (const float*)a.k + (size_t)(b * a.Hkv + kvh) * N * D;
  const float* Vg = (const float*)a.v + (size_t)(b * a.Hkv + kvh) * N * D;

  float qf[NS];  // Q^T operand of k-step s: Q[row][2s + hh]
#pragma unroll
  for (int s = 0; s < NS; ++s) qf[s] = row < N ? Qg[(size_t)row * D + 2 * s + hh] : 0.0f;

  const int T = a.causal ? ((min(q0 + MBM, N) - 1) / MBN + 1) : (N + MBN - 1) / MBN;
  const int lim = a.causal ? min(row, N - 1) : N - 1;  // last key visible to the lane's row

  // tile kt of K (and V) into LDS, rows past N as zero: float4 reads, float2 (K) / float4 (V) stores
  auto load = [&](int kt, bool with_v) {
    for (int e = tid; e < MBN * D / 4; e += MW * 64) {
      const int j = e / (D / 4), c = 4 * (e % (D / 4)), key = kt * MBN + j;
      const f32x4 k4 = key < N ? *(const f32x4*)(Kg + (size_t)key * D + c) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      float* kd = Ks + j * KS + c;
      kd[0] = k4[0];
      kd[1] = k4[1];
      kd[2] = k4[2];
      kd[3] = k4[3];
      if (with_v) {
        const f32x4 v4 = key < N ? *(const f32x4*)(Vg + (size_t)key * D + c) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        *(f32x4*)(Vs + j * VS + c) = v4;
      }
    }
  };
  // S^T of 32-key block kb of the tile in LDS
  auto scores = [&](int kb) {
    f32x16 acc = {};
    const float* kr = Ks + (kb * 32 + li) * KS + hh;
#pragma unroll
    for (int s = 0; s < NS; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kr[2 * s], qf[s], acc, 0, 0, 0);
    return acc;
  };
  auto visible = [&](int kt, int kb, int r) { return kt * MBN + kb * 32 + acc_key(r, hh) <= lim; };

  float M = -__builtin_inff(), MN = __builtin_inff();
  if (ANCH) {  // the row extrema over the visible keys, from the same MMA chains as the main loop
    for (int kt = 0; kt < T; ++kt) {
      __syncthreads();
      load(kt, false);
      __syncthreads();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const f32x16 sc = scores(kb);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool ok = visible(kt, kb, r);
          M = fmaxf(M, ok ? sc[r] : -__builtin_inff());
          MN = fminf(MN, ok ? sc[r] : __builtin_inff());
        }
      }
    }
    M = half_max(M);
    MN = half_min(MN);
  }
  RowC rc = make_row<WK, MSH>(a, M, MN, wave * 32 + li, Tb, hh, 2);

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float l = 0.0f;
  const bool dump_row = a.grid_idx != nullptr && row >= a.idx_row0 && row < a.idx_row0 + a.idx_rows && row < N;
  uint8_t* const dst = dump_row ? a.grid_idx + ((size_t)bh * a.idx_rows + (row - a.idx_row0)) * N : nullptr;
  float A = -__builtin_inff();  // single-pass PoT: the running integer anchor, kept in rc.mc

  for (int kt = 0; kt < T; ++kt) {
    __syncthreads();  // also publishes the K-interval tables before the first weights
    load(kt, true);
    __syncthreads();
    f32x16 sc[2] = {scores(0), scores(1)};
    if (WK == WK_EXACT || RUN) {  // the tile's maximum over the row's visible keys
      float tm = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) tm = fmaxf(tm, visible(kt, kb, r) ? sc[kb][r] : -__builtin_inff());
      tm = half_max(tm);
      if (RUN) {  // A = ceil(running max of s log2 e); a rise by dA scales what was formed by 2^-dA
        const float An = fmaxf(A, __builtin_ceilf(tm * rc.c));
        if (An > A) {
          const float alpha = A > -__builtin_inff() ? __builtin_ldexpf(1.0f, (int)(A - An)) : 0.0f;
          l *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) o[db] *= alpha;
          A = An;
          rc.mc = An;
        }
      } else if (tm > M) {  // online exact: rescale by 2^((M_old - M_new) c)
        const float alpha = __builtin_amdgcn_exp2f((M - tm) * rc.c);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
        M = tm;
        rc.mc = M * rc.c;
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 p;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool ok = visible(kt, kb, r);
        const float w = Weight<WK>::template w<MSH>(sc[kb][r], rc, Tb, a.levels);
        p[r] = ok ? w : 0.0f;
        l += p[r];
        if (dump_row) {
          const int key = kt * MBN + kb * 32 + acc_key(r, hh);
          if (key < N) dst[key] = (uint8_t)(ok ? Weight<WK>::idx(sc[kb][r], rc, a.levels) : 255u);
        }
      }
      // O^T += V^T P^T over the block's 32 keys, k-step s on the key of register s
      const float* vr = Vs + (kb * 32 + 4 * hh) * VS + li;
#pragma unroll
      for (int s = 0; s < 16; ++s)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vr[(8 * (s >> 2) + (s & 3)) * VS + 32 * db], p[s], o[db], 0, 0, 0);
    }
  }

  l = half_sum(l);
  if (row >= N) return;
  if (dump_row && hh == 0)  // keys past the last tile are invisible to every row here (causal)
    for (int key = T * MBN; key < N; ++key) dst[key] = 255u;
  float* Og = (float*)a.o + (size_t)(b * a.H + h) * N * D + (size_t)row * D;
  const float inv = a.vd / l;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)  // registers 4g .. 4g+3: columns 32 db + 8g + 4hh + 0..3
      *(f32x4*)(Og + 32 * db + 8 * g + 4 * hh) =
          f32x4{o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv};
  if (hh == 0) {
    const size_t ri = (size_t)bh * N + row;
    if (a.row_max) a.row_max[ri] = RUN ? A * 0.69314718055994531f : M * a.sc;  // single pass: A ln 2
    if (a.row_sum) a.row_sum[ri] = l;
    if (a.row_lo) a.row_lo[ri] = ((wk_kint(WK) && a.window_calib) || wk_support(WK)) ? M * a.sc - a.window : MN * a.sc;
  }
#endif
}

template <int D, int WK>
hipError_t launch_one(const FwdArgs& a0, hipStream_t st) {
  FwdArgs a = a0;
  a.n_qtiles = (a.N + MBM - 1) / MBM;
  a.total_blocks = a.B * a.H * a.n_qtiles;
  const size_t lds = (size_t)MBN * ((D + 2) + (D + 8)) * 4 + table_bytes(WK, MBM, a.levels);
  auto kern = fwd_f32<D, WK>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(a.total_blocks), dim3(MW * 64), lds, st, a);
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
