// Fused quantized-softmax attention forward, bf16 Q/K/V, gfx950 MFMA.
//
// The fused path follows the wiki summary's flowchart of the method ("QK tile
// -> Row max (anchor point) -> Power-of-two weights -> PV matmul -> Output"),
// built for CDNA4:
//
//   * one workgroup = 4 waves = BM = 128 query rows of one (batch, head);
//     each wave owns 32 rows for the whole kernel (Q stays in VGPRs);
//   * scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: lane (i, h) of a wave holds query row i of its
//     32 and 16 keys of each 32-key block, so row maxima, minima and sums are
//     in-lane reductions plus one exchange between the two half-waves;
//   * the accumulator layout of S^T is already the B operand of the PV
//     product O^T = V^T P^T, so P never moves between lanes; V is transposed
//     once on its way into LDS to match;
//   * anchored kinds (Rowmax-PoT, K-interval, exact-anchored) first run a
//     pre-pass over all key tiles for the true row maximum (and minimum for
//     min-max calibration), then the main loop forms weights against that
//     fixed anchor, so O needs no per-tile rescale.  The online exact control
//     skips the pre-pass and rescales by 2^(m_old - m_new) when a row's
//     running maximum grows;
//   * K and V tiles (64 keys) are staged in LDS; the next tile's global loads
//     are in flight while the current tile is computed.
#include "qsa_common.h"
#include "qsa_weights.h"

namespace qsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int NW = 4;   // waves per workgroup
constexpr int BN = 64;  // keys per tile

__device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Round-to-nearest-even pack of two floats into two bf16 (low = a).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Sum of the two bf16 in `p` added to `acc` (v_dot2_f32_bf16 against 1.0).
__device__ __forceinline__ float dot2_ones(uint32_t p, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p), one, acc, false);
}

__device__ __forceinline__ float half_swap(float x) { return __shfl_xor(x, 32, 64); }

// Row and key of accumulator register r of lane (li, hh) in a 32x32 block.
__device__ __forceinline__ int acc_key(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }

template <int D, int WK, int QB>
__global__ __launch_bounds__(NW * 64, 2) void fwd_bf16(FwdArgs a) {
  constexpr int BM = NW * QB * 32;
  constexpr int KC = D / 16;  // k-steps of the QK product
  constexpr int DB = D / 32;  // 32-column blocks of O^T
  constexpr int NB = BN / 32; // 32-key blocks per tile
  constexpr int C8 = D / 8;   // 16-byte chunks per K row
  constexpr bool ANCH = (WK != WK_EXACT);
  constexpr bool PACK_EXACT_BITS = (WK == WK_POT || WK == WK_POT_FLUSH);
  constexpr int SH = (BM == 128) ? 9 : (BM == 256 ? 10 : 8);
  static_assert((1 << SH) == BM * 4, "table shift");

  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* Ks = smem;
  unsigned char* Vs = smem + BN * D * 2;
  unsigned char* Tb = smem + 2 * BN * D * 2;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, hh = lane >> 5;
  int bh, qt;
  map_block(a, bh, qt);
  const int b = bh / a.H, h = bh - b * a.H;
  const int kvh = h / (a.H / a.Hkv);
  const int N = a.N;
  const int q0 = qt * BM;
  const int wr0 = q0 + wave * QB * 32;
  const __bf16* Qg = (const __bf16*)a.q + (size_t)(b * a.H + h) * N * D;
  const __bf16* Kg = (const __bf16*)a.k + (size_t)(b * a.Hkv + kvh) * N * D;
  const __bf16* Vg = (const __bf16*)a.v + (size_t)(b * a.Hkv + kvh) * N * D;

  // Q^T operand: lane (li, hh) holds Q[row][16c + 8hh .. +7].
  u32x4 qf[QB][KC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wr0 + qb * 32 + li;
#pragma unroll
    for (int c = 0; c < KC; ++c)
      qf[qb][c] = row < N ? *(const u32x4*)(Qg + (size_t)row * D + 16 * c + 8 * hh) : u32x4{0, 0, 0, 0};
  }

  const int ntile_all = (N + BN - 1) / BN;
  const int qend = min(q0 + BM, N);
  const int kt_end = a.causal ? ((qend - 1) / BN + 1) : ntile_all;
  const bool wave_active = wr0 < N;
  const int wrow_last = min(wr0 + QB * 32, N) - 1;
  const int wkt_last = a.causal ? (wrow_last / BN) : (ntile_all - 1);

  // ---- global -> register -> LDS staging --------------------------------
  constexpr int KU = BN * C8 / (NW * 64);
  constexpr int VU = (BN / 4) * C8;
  static_assert(KU >= 1 && VU <= NW * 64, "tile staging");
  u32x4 kr[KU];
  u32x4 vr[4];
  auto load_k = [&](int kt) {
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int u = tid + i * NW * 64, j = u / C8, c = u % C8, key = kt * BN + j;
      kr[i] = key < N ? *(const u32x4*)(Kg + (size_t)key * D + c * 8) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_k = [&]() {
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int u = tid + i * NW * 64, j = u / C8, c = u % C8;
      *(u32x4*)(Ks + j * D * 2 + ((c ^ (j % C8)) * 16)) = kr[i];
    }
  };
  auto load_v = [&](int kt) {
    if (tid < VU) {
      const int co = tid % C8, kq = tid / C8;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kt * BN + 4 * kq + r;
        vr[r] = key < N ? *(const u32x4*)(Vg + (size_t)key * D + co * 8) : u32x4{0, 0, 0, 0};
      }
    }
  };
  // V^T layout: 16-byte slot (g, hb, dcol) holds V[16g + 4hb + 0..3][dcol] then
  // V[16g + 8 + 4hb + 0..3][dcol]: the keys lane half hb multiplies in k-step g.
  auto vslot = [&](int g, int hb, int dcol) { return ((g * 2 + hb) * D + (dcol ^ ((dcol >> 3) & 7))) * 16; };
  auto store_v = [&]() {
    if (tid < VU) {
      const int co = tid % C8, kq = tid / C8;
      const int g = kq >> 2, hb = kq & 1, half = (kq >> 1) & 1;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const u32x2 lo = {__builtin_amdgcn_perm(vr[1][p], vr[0][p], 0x05040100u),
                          __builtin_amdgcn_perm(vr[3][p], vr[2][p], 0x05040100u)};
        const u32x2 hi = {__builtin_amdgcn_perm(vr[1][p], vr[0][p], 0x07060302u),
                          __builtin_amdgcn_perm(vr[3][p], vr[2][p], 0x07060302u)};
        *(u32x2*)(Vs + vslot(g, hb, co * 8 + 2 * p) + half * 8) = lo;
        *(u32x2*)(Vs + vslot(g, hb, co * 8 + 2 * p + 1) + half * 8) = hi;
      }
    }
  };
  auto rdK = [&](int kb, int c) -> u32x4 {
    const int j = kb * 32 + li, c8 = 2 * c + hh;
    return *(const u32x4*)(Ks + j * D * 2 + ((c8 ^ (j % C8)) * 16));
  };
  auto rdV = [&](int g, int db) -> u32x4 { return *(const u32x4*)(Vs + vslot(g, hh, db * 32 + li)); };

  auto qk = [&](f32x16 (&s)[QB][NB]) {
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb][kb] = f32x16{};
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const u32x4 ka = rdK(kb, c);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mma(ka, qf[qb][c], s[qb][kb]);
      }
    }
  };
  // -inf on keys a row cannot see (causal, or beyond N).
  auto mask = [&](f32x16 (&s)[QB][NB], int kt) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = wr0 + qb * 32 + li;
      const int lim = a.causal ? min(row, N - 1) : N - 1;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt * BN + kb * 32 + acc_key(r, hh);
          s[qb][kb][r] = key <= lim ? s[qb][kb][r] : -__builtin_inff();
        }
    }
  };
  auto needs_mask = [&](int kt) { return (a.causal && kt * BN + BN - 1 > wr0) || (kt * BN + BN > N); };

  // ---- pre-pass: true row extrema (anchored kinds) ------------------------
  float M[QB], MN[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) { M[qb] = -__builtin_inff(); MN[qb] = __builtin_inff(); }
  if (ANCH) {
    load_k(0);
    for (int kt = 0; kt < kt_end; ++kt) {
      __syncthreads();
      store_k();
      __syncthreads();
      if (kt + 1 < kt_end) load_k(kt + 1);
      if (wave_active && kt <= wkt_last) {
        f32x16 s[QB][NB];
        qk(s);
        const bool msk = needs_mask(kt);
        if (msk) mask(s, kt);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int kb = 0; kb < NB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) M[qb] = fmaxf(M[qb], s[qb][kb][r]);
        if (a.track_min) {
          if (msk) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
              for (int kb = 0; kb < NB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                  const float x = s[qb][kb][r];
                  MN[qb] = fminf(MN[qb], x == -__builtin_inff() ? __builtin_inff() : x);
                }
          } else {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
              for (int kb = 0; kb < NB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) MN[qb] = fminf(MN[qb], s[qb][kb][r]);
          }
        }
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      M[qb] = fmaxf(M[qb], half_swap(M[qb]));
      MN[qb] = fminf(MN[qb], half_swap(MN[qb]));
    }
  }

  RowC rc[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
    rc[qb] = make_row<WK, SH>(a, M[qb], MN[qb], (wave * QB + qb) * 32 + li, Tb, hh, 2);
  // (the barrier at the top of the main loop publishes the K-interval tables)

  // ---- main loop ----------------------------------------------------------
  f32x16 o[QB][DB];
  float l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    l[qb] = 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb][db] = f32x16{};
  }
  const bool dump = a.grid_idx != nullptr && wr0 < a.idx_row0 + a.idx_rows && wr0 + QB * 32 > a.idx_row0;

  load_k(0);
  load_v(0);
  for (int kt = 0; kt < kt_end; ++kt) {
    __syncthreads();
    store_k();
    store_v();
    __syncthreads();
    if (kt + 1 < kt_end) {
      load_k(kt + 1);
      load_v(kt + 1);
    }
    if (!(wave_active && kt <= wkt_last)) continue;

    f32x16 s[QB][NB];
    qk(s);
    const bool msk = needs_mask(kt);
    if (msk) mask(s, kt);

    if (WK == WK_EXACT) {
      // online softmax: grow the running max, rescale what was accumulated
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float tm = -__builtin_inff();
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) tm = fmaxf(tm, s[qb][kb][r]);
        tm = fmaxf(tm, half_swap(tm));
        const float mnew = fmaxf(M[qb], tm);
        if (__ballot(mnew > M[qb])) {
          const float alpha = (mnew > M[qb]) ? __builtin_amdgcn_exp2f((M[qb] - mnew) * rc[qb].c) : 1.0f;
          l[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) o[qb][db] *= alpha;
          M[qb] = mnew;
          rc[qb].mc = mnew * rc[qb].c;
        }
      }
    }

    if (dump) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int row = wr0 + qb * 32 + li;
        if (row >= a.idx_row0 && row < a.idx_row0 + a.idx_rows && row < N) {
          uint8_t* dst = a.grid_idx + ((size_t)bh * a.idx_rows + (row - a.idx_row0)) * N;
#pragma unroll
          for (int kb = 0; kb < NB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kt * BN + kb * 32 + acc_key(r, hh);
              if (key < N) {
                const float x = s[qb][kb][r];
                dst[key] = (uint8_t)(x == -__builtin_inff() ? 255u : Weight<WK>::idx(x, rc[qb], a.levels));
              }
            }
        }
      }
    }

    // weights -> P^T operands (bf16), row sums of the weights that enter PV
    u32x4 P[QB][2 * NB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int r0 = 8 * kc + 2 * p;
            const float x0 = s[qb][kb][r0], x1 = s[qb][kb][r0 + 1];
            float w0 = Weight<WK>::template w<SH>(x0, rc[qb], Tb, a.levels);
            float w1 = Weight<WK>::template w<SH>(x1, rc[qb], Tb, a.levels);
            if (WK != WK_EXACT && WK != WK_EXACT_ANCH && msk) {
              w0 = x0 == -__builtin_inff() ? 0.0f : w0;
              w1 = x1 == -__builtin_inff() ? 0.0f : w1;
            }
            uint32_t pk;
            if (PACK_EXACT_BITS)  // powers of two: the bf16 pattern is the top half
              pk = __builtin_amdgcn_perm(fbits(w1), fbits(w0), 0x07060302u);
            else
              pk = pack_bf16(w0, w1);
            P[qb][2 * kb + kc][p] = pk;
            l[qb] = dot2_ones(pk, l[qb]);
          }

    // O^T += V^T P^T
#pragma unroll
    for (int g = 0; g < 2 * NB; ++g)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x4 va = rdV(g, db);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) o[qb][db] = mma(va, P[qb][g], o[qb][db]);
      }
  }

  // ---- epilogue -----------------------------------------------------------
  if (!wave_active) return;
  if (dump) {  // keys past this wave's last tile are invisible to all its rows (causal)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = wr0 + qb * 32 + li;
      if (row >= a.idx_row0 && row < a.idx_row0 + a.idx_rows && row < N) {
        uint8_t* dst = a.grid_idx + ((size_t)bh * a.idx_rows + (row - a.idx_row0)) * N;
        for (int key = (wkt_last + 1) * BN + hh; key < N; key += 2) dst[key] = 255u;
      }
    }
  }
  __bf16* Og = (__bf16*)a.o + (size_t)(b * a.H + h) * N * D;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l[qb] + half_swap(l[qb]);
    const int row = wr0 + qb * 32 + li;
    if (row >= N) continue;
    const float inv = a.vd / lt;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dcol = db * 32 + 8 * g4 + 4 * hh;
        const u32x2 v = {pack_bf16(o[qb][db][4 * g4 + 0] * inv, o[qb][db][4 * g4 + 1] * inv),
                         pack_bf16(o[qb][db][4 * g4 + 2] * inv, o[qb][db][4 * g4 + 3] * inv)};
        *(u32x2*)(Og + (size_t)row * D + dcol) = v;
      }
    if (hh == 0) {
      const size_t ri = (size_t)bh * N + row;
      if (a.row_max) a.row_max[ri] = M[qb] * a.sc;
      if (a.row_sum) a.row_sum[ri] = lt;
      if (a.row_lo) {
        const bool kint = WK >= WK_KH;
        a.row_lo[ri] = (kint && a.window_calib) ? M[qb] * a.sc - a.window : MN[qb] * a.sc;
      }
    }
  }
}

template <int D, int WK>
hipError_t launch_one(const FwdArgs& a0, hipStream_t st) {
  constexpr int QB = 1;
  constexpr int BM = NW * QB * 32;
  FwdArgs a = a0;
  a.n_qtiles = (a.N + BM - 1) / BM;
  a.total_blocks = a.B * a.H * a.n_qtiles;
  const size_t lds = 2 * (size_t)BN * D * 2 + table_bytes(WK, BM, a.levels);
  auto kern = fwd_bf16<D, WK, QB>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(a.total_blocks), dim3(NW * 64), lds, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a, int wk, hipStream_t st) {
  switch (wk) {
    case WK_EXACT: return launch_one<D, WK_EXACT>(a, st);
    case WK_EXACT_ANCH: return launch_one<D, WK_EXACT_ANCH>(a, st);
    case WK_POT: return launch_one<D, WK_POT>(a, st);
    case WK_POT_FLUSH: return launch_one<D, WK_POT_FLUSH>(a, st);
    case WK_KH: return launch_one<D, WK_KH>(a, st);
    case WK_KH_FLUSH: return launch_one<D, WK_KH_FLUSH>(a, st);
    case WK_KI: return launch_one<D, WK_KI>(a, st);
    case WK_KI_FLUSH: return launch_one<D, WK_KI_FLUSH>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_bf16(const FwdArgs& a, int d, int wk, hipStream_t st) {
  if (d == 64) return launch_d<64>(a, wk, st);
  if (d == 128) return launch_d<128>(a, wk, st);
  return hipErrorInvalidValue;
}

}  // namespace qsa
