// Fused quantized-softmax attention forward, bf16 Q/K/V, gfx950 MFMA.
//
// The fused path follows the wiki summary's flowchart of the method ("QK tile
// -> Row max (anchor point) -> Power-of-two weights -> PV matmul -> Output"),
// laid out for CDNA4:
//
//   * one workgroup = 4 waves = 128 query rows of one (batch, head); each
//     wave owns 32 rows for the whole kernel (its Q^T operand stays in VGPRs);
//   * scores are computed transposed, S^T = K Q^T, on
//     v_mfma_f32_32x32x16_bf16: lane (i, h) of a wave holds query row i and 16
//     keys of each 32-key block, so row maxima, minima and sums are in-lane
//     reductions plus one exchange between the two half-waves;
//   * the accumulator layout of S^T is the B operand of O^T = V^T P^T, so P
//     never moves between lanes;
//   * anchored kinds run a pre-pass over all key tiles for the true row
//     maximum (and minimum for min-max calibration).  The main loop then
//     starts each score accumulation at -M (a register vector holding the
//     row max), so the MFMA itself delivers s' = acc - M <= 0 and the weight
//     needs no per-element subtraction; O needs no per-tile rescale;
//   * the online exact control skips the pre-pass and rescales O by
//     2^(m_old - m_new) when a row's running maximum grows;
//   * K and V tiles of 64 keys are double-buffered in LDS and filled by
//     buffer loads that write LDS directly (no staging registers; hardware
//     zero-fill past the end of the head), one tile ahead, with one workgroup
//     barrier per tile.  K rows are padded to an odd number of 16-byte slots
//     so a column read by 16 lanes hits 16 different banks; V stays row-major
//     and the V^T operand comes from transposing LDS reads (ds_read_b64_tr_b16);
//   * the scores of tile t+1 are computed on the matrix cores while the
//     weights of tile t are formed on the VALU, so the two overlap in a wave;
//   * only a wave's last tile can need masking (causal diagonal or the ragged
//     end of the sequence); it runs a separate code path, so the steady-state
//     tiles carry no mask arithmetic.
#include "qsa_common.h"
#include "qsa_mfma_util.h"
#include "qsa_weights.h"

namespace qsa {
namespace {

constexpr int NW = 4;    // waves per workgroup
constexpr int BN = 64;   // keys per tile
constexpr int BM = 128;  // query rows per workgroup
constexpr int SH = 9;    // log2(BM * 4): the row-constant template's table stride (no table is built here)
#ifndef QSA_BF16_WAVES_PER_SIMD
#define QSA_BF16_WAVES_PER_SIMD 2
#endif

template <int D, int WK, bool DUMP>
__global__ __launch_bounds__(NW * 64, QSA_BF16_WAVES_PER_SIMD) void fwd_bf16(FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass needs only the signature (for the launch stub)
  constexpr int KC = D / 16;  // k-steps of the QK product
  constexpr int DB = D / 32;  // 32-column blocks of O^T
  constexpr int C8 = D / 8;   // 16-byte chunks per K row
  constexpr int SK = D / 8 + 1;    // 16-byte slots per K row in LDS (odd: 16 rows -> 16 bank groups)
  constexpr int SV = D / 8 + 4;    // slots per V row (row stride = 64 mod 256 bytes)
  constexpr int KR = SK * 16, VR = SV * 16;
  constexpr int KT = BN * KR, VT = BN * VR;  // bytes of one K / V tile buffer
  constexpr int KIW = (SK + NW - 1) / NW;    // direct-load instructions per wave per K tile (max)
  constexpr int VIW = (SV + NW - 1) / NW;
  constexpr bool RUN = wk_running(WK);             // single-pass PoT: running integer anchor
  constexpr bool ANCH = (WK != WK_EXACT) && !RUN;  // true-row-extrema pre-pass
  constexpr bool EXACT_W = (WK == WK_EXACT || WK == WK_EXACT_ANCH);
  constexpr bool POT = wk_pot(WK);
  constexpr bool KHARD = (WK == WK_KH || WK == WK_KH_FLUSH);
  constexpr bool SUPPORT = wk_support(WK), UNIF = (WK == WK_UNIF);
  constexpr bool FLUSH = (WK == WK_POT_FLUSH || WK == WK_POTR_FLUSH || WK == WK_KH_FLUSH || WK == WK_KI_FLUSH);

  extern __shared__ __align__(16) unsigned char smem[];
  lds_u8* const lds = (lds_u8*)smem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, hh = lane >> 5;
  int bh, qt;
  map_block(a, bh, qt);
  const int b = bh / a.H, h = bh - b * a.H;
  const int kvh = h / (a.H / a.Hkv);
  const int N = a.N;
  const int q0 = qt * BM;
  const int wr0 = q0 + wave * 32;
  const int row = wr0 + li;
  const __bf16* Qg = (const __bf16*)a.q + (size_t)(b * a.H + h) * N * D;
  const size_t kv_off = (size_t)(b * a.Hkv + kvh) * N * D;
  const __bf16* const Kg = (const __bf16*)a.k + kv_off;
  const __bf16* const Vg = (const __bf16*)a.v + kv_off;

  // Q^T operand: lane (li, hh) holds Q[row][16c + 8hh .. +7].
  u32x4 qf[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c)
    qf[c] = row < N ? *(const u32x4*)(Qg + (size_t)row * D + 16 * c + 8 * hh) : u32x4{0, 0, 0, 0};

  const int T = a.causal ? ((min(q0 + BM, N) - 1) / BN + 1) : (N + BN - 1) / BN;  // tiles of this workgroup
  // last tile this wave computes (-1: none); only that tile can need masking
  const int wlast = wr0 >= N ? -1 : (a.causal ? (min(wr0 + 31, N - 1) / BN) : T - 1);
  const bool last_masked = (a.causal && wlast * BN + BN - 1 > wr0) || (wlast * BN + BN > N);

  // ---- tile staging: buffer loads straight into LDS ------------------------
  // A wave-instruction writes 64 consecutive 16-byte slots; slot s of a tile
  // is row s / SK, chunk s % SK of the padded layout (pad chunks load zeros
  // from an out-of-range offset).  The per-tile buffer resource starts at the
  // tile and ends at the end of the head, so rows past N read as zero.
  uint32_t kvo[KIW], vvo[VIW];
#pragma unroll
  for (int m = 0; m < KIW; ++m) {
    const int sl = (wave + NW * m) * 64 + lane, j = sl / SK, c = sl % SK;
    kvo[m] = c < D / 8 ? (uint32_t)(j * D + c * 8) * 2 : 0x7FFFFFF0u;
  }
#pragma unroll
  for (int m = 0; m < VIW; ++m) {
    const int sl = (wave + NW * m) * 64 + lane, j = sl / SV, c = sl % SV;
    vvo[m] = c < D / 8 ? (uint32_t)(j * D + c * 8) * 2 : 0x7FFFFFF0u;
  }
  auto tile_rsrc = [&](const __bf16* base, int kt) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (size_t)kt * BN * D), 0, (N - kt * BN) * D * 2,
                                             0x00020000);
  };
  auto load_k = [&](int kt, int buf) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(Kg, kt);
#pragma unroll
    for (int m = 0; m < KIW; ++m)
      if (wave + NW * m < SK)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds + buf * KT + (wave + NW * m) * 1024), 16,
                                                 kvo[m], 0, 0, 0);
  };
  auto load_v = [&](int kt, int buf) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(Vg, kt);
#pragma unroll
    for (int m = 0; m < VIW; ++m)
      if (wave + NW * m < SV)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)(lds + 2 * KT + buf * VT + (wave + NW * m) * 1024), 16, vvo[m], 0, 0, 0);
  };
  // this wave's LDS-direct loads have landed (before the workgroup barrier)
  auto loads_done = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  // A-operand read offsets (the tile buffer and the 32-key block are added as constants)
  const uint32_t koff = li * KR + hh * 16;  // + 32 c for k-step c
  // V^T operand: in each 16-lane group, lane 4q + p points at V[key q][4p .. 4p+3] of the
  // group's 16 columns; the transposing read hands lane l column l and keys q = 0..3.
  const uint32_t vtr = (4 * hh + ((lane & 15) >> 2)) * VR + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));

  // 32-key block kb of a tile: init + K_block Q^T  (init: the -M vector, or 0)
  auto qk1 = [&](int buf, int kb, const f32x16& init) {
    const lds_u8* kbase = lds + buf * KT + kb * 32 * KR + koff;
    f32x16 s = init;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const u32x4 ka = *(const __attribute__((address_space(3))) u32x4*)(kbase + 32 * c);
      s = mma(ka, qf[c], c == 0 ? init : s);
    }
    return s;
  };
  auto qk = [&](int buf, f32x16 (&s)[2], const f32x16& init) {
    s[0] = qk1(buf, 0, init);
    s[1] = qk1(buf, 1, init);
  };
  // O^T += V^T P^T over the 32 keys of block kb (k-steps g = 2kb, 2kb+1)
  auto pv1 = [&](int buf, int kb, const u32x4 (&P)[2], f32x16 (&o)[DB]) {
    const lds_u8* vbase = lds + 2 * KT + buf * VT + vtr;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const lds_u8* pa = vbase + (16 * (2 * kb + kc)) * VR + 64 * db;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)pa);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(pa + 8 * VR));
        const u32x4 va = {__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                          __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]};
        o[db] = mma(va, P[kc], o[db]);
      }
  };
  // keys up to `lim` are visible to this lane's row
  const int lim = a.causal ? min(row, N - 1) : N - 1;
  auto mask_fill = [&](f32x16 (&s)[2], int kt, float fill) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = (kt * BN + kb * 32 + acc_key(r, hh) <= lim) ? s[kb][r] : fill;
  };

  // ---- pre-pass: true row extrema ------------------------------------------
  float M = -__builtin_inff(), MN = __builtin_inff();
  const f32x16 zero16 = {};
  if (ANCH) {
    const bool tmin = a.track_min;
    load_k(0, 0);
    if (T > 1) load_k(1, 1);
    loads_done();
    __syncthreads();
    f32x16 s[2];
    if (wlast >= 0) qk(0, s, zero16);
    __syncthreads();  // every wave has read K tile 0 before iteration 0 refills its buffer
    // tiles before the wave's last (no masking), then the last tile and the iterations in
    // which the wave only issues its share of the other waves' loads: two loops, so that the
    // masking code stays out of the first (every wave still passes T barriers)
    // (unrolled by two with the score registers swapping roles, as in the main loop)
    auto fold = [&](const f32x16 (&cur)[2], f32x16 (&nxt)[2], int t) __attribute__((always_inline)) {
      if (t + 2 < T) load_k(t + 2, t & 1);  // buffer t&1 was last read in iteration t-1
      qk((t + 1) & 1, nxt, zero16);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) M = fmaxf(M, cur[kb][r]);
      if (tmin) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) MN = fminf(MN, cur[kb][r]);
      }
      loads_done();
      __syncthreads();
    };
    f32x16 s2[2];
    int t = 0;
    for (; t + 1 < wlast; t += 2) {
      fold(s, s2, t);
      fold(s2, s, t + 1);
    }
    if (t < wlast) {
      fold(s, s2, t);
      s[0] = s2[0];
      s[1] = s2[1];
      ++t;
    }
    for (; t < T; ++t) {
      if (t + 2 < T) load_k(t + 2, t & 1);
      if (t == wlast) {
        f32x16 sm[2] = {s[0], s[1]};
        if (last_masked) mask_fill(sm, t, -__builtin_inff());
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) M = fmaxf(M, sm[kb][r]);
        if (tmin) {
          if (last_masked) mask_fill(s, t, __builtin_inff());
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) MN = fminf(MN, s[kb][r]);
        }
      }
      loads_done();
      __syncthreads();
    }
    M = half_max(M);
    MN = half_min(MN);
  }

  RowC rc = make_row<WK, SH>(a, M, MN, wave * 32 + li, nullptr, hh, 2);
  // main-loop score accumulators start at -M: s' = acc - M
  f32x16 init16;
#pragma unroll
  for (int r = 0; r < 16; ++r) init16[r] = ANCH ? -M : 0.0f;
  // PoT rounds t = G - y to an integer in one FMA, G = 2^24 (pre-pass kinds: scores start at
  // -M, so t = 2^24 + acc' c) or G = 1.5 * 2^23 (single pass: t = (G - A) + acc c, and G - A
  // must be exact in fp32 for a negative integer anchor A too, which 2^24 - A is not).  In
  // both cases t lies in [2^23, 2^24), bits(t) = bits(G) - e, and the low 16 bits are -e.
  constexpr int32_t pot_bits = RUN ? 0x4B400000 : 0x4B800000;  // bits of G
  constexpr float pot_g = RUN ? 12582912.0f : 16777216.0f;      // G
  int32_t pot_lo = pot_bits - (a.levels - 1);                   // bits of G - (L-1): the clip e <= L-1
  // Single-pass PoT: A = ceil(running max of s log2 e), an integer.  The weights are formed
  // against a lagging integer anchor Aw <= A (tb = G - Aw) with the clip moved by the lag
  // dl = A - Aw (pot_lo = bits(G) - (L-1) + dl), so every weight carries the same factor 2^dl
  // relative to A while Aw stays; O and l are rescaled only when Aw moves, on the first tile
  // and when the lag would pass 32 (bf16 weights up to 2^32 and their sums stay well inside
  // the exponent range).
  float A = -__builtin_inff(), Aw = -__builtin_inff();
  int dlag = 0;
  float tb = pot_g;
  const int L = a.levels;
  const float Kf = (float)a.levels;

  // weights of 32-key block kb of tile kt -> 2 P^T operands (bf16) and the row sum
  auto weights = [&](const f32x16& sb, int kb, u32x4 (&P)[2], float& l, int kt, bool masked) {
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int r0 = 8 * kc + 2 * p;
          const float x0 = sb[r0], x1 = sb[r0 + 1];
          uint32_t pk;
          uint32_t i0 = 0, i1 = 0;  // grid indices (dump only)
          if (EXACT_W) {
            // exact: 2^((acc - M) c); the online kind folds -M c into the FMA
            const float y0 = ANCH ? x0 * rc.c : fmaf(x0, rc.c, -rc.mc);
            const float y1 = ANCH ? x1 * rc.c : fmaf(x1, rc.c, -rc.mc);
            pk = pack_bf16(__builtin_amdgcn_exp2f(y0), __builtin_amdgcn_exp2f(y1));
          } else if (SUPPORT) {
            // truncation / uniform weighting: keys with y = (M - acc) c > W log2 e are outside
            // the support; inside, exp(s - m) or 1
            const float y0 = -x0 * rc.c, y1 = -x1 * rc.c;
            const float e0 = UNIF ? 1.0f : __builtin_amdgcn_exp2f(x0 * rc.c);
            const float e1 = UNIF ? 1.0f : __builtin_amdgcn_exp2f(x1 * rc.c);
            pk = pack_bf16(y0 > rc.cut ? 0.0f : e0, y1 > rc.cut ? 0.0f : e1);
            if (DUMP) {
              i0 = y0 > rc.cut ? 254u : 0u;
              i1 = y1 > rc.cut ? 254u : 0u;
            }
          } else if (POT && !FLUSH) {
            // t = 2^24 + (acc - M) c = 2^24 - y, rounded to an integer by the FMA itself
            const float t0 = fmaf(x0, rc.c, tb), t1 = fmaf(x1, rc.c, tb);
            pk = pot_pair(t0, t1, pot_lo);
            if (DUMP) {
              i0 = 127u - ((pk >> 7) & 0x1FFu) + (uint32_t)dlag;  // against the running anchor
              i1 = 127u - ((pk >> 23) & 0x1FFu) + (uint32_t)dlag;
            }
          } else if (POT) {  // flush: e >= L -> 0
            const float t0 = fmaf(x0, rc.c, tb), t1 = fmaf(x1, rc.c, tb);
            const int32_t lo = pot_lo;
            const int32_t b0 = (int32_t)fbits(t0), b1 = (int32_t)fbits(t1);
            const uint32_t w0 = b0 < lo ? 0u : (((uint32_t)b0 << 23) + (127u << 23));
            const uint32_t w1 = b1 < lo ? 0u : (((uint32_t)b1 << 23) + (127u << 23));
            pk = __builtin_amdgcn_perm(w1, w0, 0x07060302u);
            if (DUMP) {
              i0 = b0 < lo ? 254u : (uint32_t)(pot_bits - b0 + dlag);
              i1 = b1 < lo ? 254u : (uint32_t)(pot_bits - b1 + dlag);
            }
          } else if (KHARD) {
            // y = (M - acc) c; t = y + 2^23 rounds y: bits(t) = 0x4B000000 + l
            const float t0 = fmaf(x0, -rc.c, 8388608.0f), t1 = fmaf(x1, -rc.c, 8388608.0f);
            int32_t b0 = (int32_t)fbits(t0), b1 = (int32_t)fbits(t1);
            b0 = min(max(b0, 0x4B000000), 0x4B000000 + L);
            b1 = min(max(b1, 0x4B000000), 0x4B000000 + L);
            float w0 = __builtin_amdgcn_exp2f(rc.step * (float)(b0 - 0x4B000000));  // T_l
            float w1 = __builtin_amdgcn_exp2f(rc.step * (float)(b1 - 0x4B000000));
            const float y0 = FLUSH ? -x0 * rc.c : 0.0f, y1 = FLUSH ? -x1 * rc.c : 0.0f;
            if (FLUSH) {  // y > K: below the window
              w0 = y0 > Kf ? 0.0f : w0;
              w1 = y1 > Kf ? 0.0f : w1;
            }
            pk = pack_bf16(w0, w1);
            if (DUMP) {
              i0 = (FLUSH && y0 > Kf) ? 254u : (uint32_t)(b0 - 0x4B000000);
              i1 = (FLUSH && y1 > Kf) ? 254u : (uint32_t)(b1 - 0x4B000000);
            }
          } else {  // K-interval, interpolation
            const float y0 = -x0 * rc.c, y1 = -x1 * rc.c;
            const float c0 = __builtin_amdgcn_fmed3f(y0, 0.0f, Kf), c1 = __builtin_amdgcn_fmed3f(y1, 0.0f, Kf);
            const float f0 = __builtin_floorf(c0), f1 = __builtin_floorf(c1);
            const uint32_t l0 = (uint32_t)(int32_t)f0, l1 = (uint32_t)(int32_t)f1;
            typedef float f2 __attribute__((ext_vector_type(2)));
            const f2 e0 = kgrid_pair(rc.step, f0);  // (T_l, T_l+1 - T_l)
            const f2 e1 = kgrid_pair(rc.step, f1);
            float w0 = fmaf(c0 - f0, e0.y, e0.x), w1 = fmaf(c1 - f1, e1.y, e1.x);
            if (FLUSH) {
              w0 = y0 > Kf ? 0.0f : w0;
              w1 = y1 > Kf ? 0.0f : w1;
            }
            pk = pack_bf16(w0, w1);
            if (DUMP) {
              i0 = (FLUSH && y0 > Kf) ? 254u : l0;
              i1 = (FLUSH && y1 > Kf) ? 254u : l1;
            }
          }
          if (masked) {
            const int k0 = kt * BN + kb * 32 + acc_key(r0, hh);  // r0 even: keys k0, k0 + 1
            const uint32_t m0 = k0 <= lim ? 0x0000FFFFu : 0u, m1 = k0 + 1 <= lim ? 0xFFFF0000u : 0u;
            pk &= (m0 | m1);
            if (DUMP) {
              i0 = k0 <= lim ? i0 : 255u;
              i1 = k0 + 1 <= lim ? i1 : 255u;
            }
          }
          if (DUMP && row >= a.idx_row0 && row < a.idx_row0 + a.idx_rows && row < N) {
            const int k0 = kt * BN + kb * 32 + acc_key(r0, hh);
            uint8_t* dst = a.grid_idx + ((size_t)bh * a.idx_rows + (row - a.idx_row0)) * N;
            if (k0 < N) dst[k0] = (uint8_t)i0;
            if (k0 + 1 < N) dst[k0 + 1] = (uint8_t)i1;
          }
          P[kc][p] = pk;
          l = dot2_ones(pk, l);
        }
  };

  // online exact: grow the running max over this tile, rescale O and l
  auto online_max = [&](const f32x16 (&s)[2], f32x16 (&o)[DB], float& l) {
    float tm = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) tm = fmaxf(tm, s[kb][r]);
    const float mnew = fmaxf(M, half_max(tm));
    if (__builtin_amdgcn_ballot_w64(mnew > M)) {
      const float alpha = mnew > M ? __builtin_amdgcn_exp2f((M - mnew) * rc.c) : 1.0f;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      M = mnew;
      rc.mc = mnew * rc.c;
    }
  };

  // single-pass PoT: fold this tile's maximum into the anchor before its weights are formed;
  // when the weight anchor Aw has to move, O and l, formed against the old Aw, are scaled by
  // 2^(Aw_old - Aw) (exact)
  auto run_anchor = [&](const f32x16 (&s)[2], f32x16 (&o)[DB], float& l, int kt, bool masked) {
    float tm = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        tm = fmaxf(tm, (!masked || kt * BN + kb * 32 + acc_key(r, hh) <= lim) ? s[kb][r] : -__builtin_inff());
    const float An = fmaxf(A, __builtin_ceilf(half_max(tm) * rc.c));
    if (__builtin_amdgcn_ballot_w64(An - Aw > 32.0f)) {  // Aw = -inf before the first tile
      const bool move = An - Aw > 32.0f;
      const float alpha = move ? (Aw > -__builtin_inff() ? __builtin_ldexpf(1.0f, (int)(Aw - An)) : 0.0f) : 1.0f;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      Aw = move ? An : Aw;
      tb = pot_g - Aw;
    }
    A = An;
    dlag = (int)(A - Aw);
    pot_lo = pot_bits - (a.levels - 1) + dlag;
  };

  // ---- main loop --------------------------------------------------------------
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float l = 0.0f;
  __syncthreads();  // pre-pass reads done before the buffers are refilled
  load_k(0, 0);
  load_v(0, 0);
  if (T > 1) load_k(1, 1);
  loads_done();
  __syncthreads();
  f32x16 s[2];
  if (wlast >= 0) qk(0, s, init16);
  __syncthreads();  // every wave has read K tile 0 before iteration 0 refills its buffer
  // Tiles before the wave's last (unmasked), then its last tile and the iterations in which it
  // only issues its share of the other waves' loads: two loops, so that the masking code stays
  // out of the first (merged into one body it ran on every tile); every wave passes T barriers.
  // the scores of tile t+1 go to the other of two register sets, whose roles swap every
  // iteration (unrolled by two), so no copy of 32 registers per tile
  auto steady = [&](f32x16 (&cur)[2], f32x16 (&nxt)[2], int t) __attribute__((always_inline)) {
    if (t + 2 < T) load_k(t + 2, t & 1);      // buffers last read in iteration t-1
    if (t + 1 < T) load_v(t + 1, (t + 1) & 1);
    // block 0 of tile t+1 on the matrix cores while block 0 of tile t is weighted
    nxt[0] = qk1((t + 1) & 1, 0, init16);
    if (WK == WK_EXACT) online_max(cur, o, l);
    if (RUN) run_anchor(cur, o, l, t, false);
    u32x4 P[2];
    weights(cur[0], 0, P, l, t, false);
    pv1(t & 1, 0, P, o);
    nxt[1] = qk1((t + 1) & 1, 1, init16);
    weights(cur[1], 1, P, l, t, false);
    pv1(t & 1, 1, P, o);
    loads_done();
    __syncthreads();
  };
  f32x16 s2[2];
  int t = 0;
  for (; t + 1 < wlast; t += 2) {
    steady(s, s2, t);
    steady(s2, s, t + 1);
  }
  if (t < wlast) {
    steady(s, s2, t);
    s[0] = s2[0];
    s[1] = s2[1];
    ++t;
  }
  for (; t < T; ++t) {
    if (t + 2 < T) load_k(t + 2, t & 1);
    if (t + 1 < T) load_v(t + 1, (t + 1) & 1);
    if (t == wlast) {
      if (WK == WK_EXACT) {
        f32x16 sm[2] = {s[0], s[1]};
        if (last_masked) mask_fill(sm, t, -__builtin_inff());
        online_max(sm, o, l);
      }
      if (RUN) run_anchor(s, o, l, t, last_masked);
      u32x4 P[2];
      weights(s[0], 0, P, l, t, last_masked);
      pv1(t & 1, 0, P, o);
      weights(s[1], 1, P, l, t, last_masked);
      pv1(t & 1, 1, P, o);
    }
    loads_done();
    __syncthreads();
  }

  // ---- epilogue -----------------------------------------------------------
  if (wlast < 0) return;
  const float lt = half_sum(l);
  if (DUMP && row >= a.idx_row0 && row < a.idx_row0 + a.idx_rows && row < N) {
    uint8_t* dst = a.grid_idx + ((size_t)bh * a.idx_rows + (row - a.idx_row0)) * N;
    for (int key = (wlast + 1) * BN + hh; key < N; key += 2) dst[key] = 255u;  // beyond the wave's last tile
  }
  if (row >= N) return;
  __bf16* Og = (__bf16*)a.o + (size_t)(b * a.H + h) * N * D;
  const float inv = a.vd / lt;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int dcol = db * 32 + 8 * g4 + 4 * hh;
      const u32x2 v = {pack_bf16(o[db][4 * g4 + 0] * inv, o[db][4 * g4 + 1] * inv),
                       pack_bf16(o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv)};
      *(u32x2*)(Og + (size_t)row * D + dcol) = v;
    }
  if (hh == 0) {
    const size_t ri = (size_t)bh * N + row;
    if (a.row_max) a.row_max[ri] = RUN ? A * 0.69314718055994531f : M * a.sc;  // single pass: A ln 2
    if (a.row_sum) a.row_sum[ri] = RUN ? __builtin_ldexpf(lt, -dlag) : lt;  // single pass: against A
    if (a.row_lo) a.row_lo[ri] = ((wk_kint(WK) && a.window_calib) || wk_support(WK)) ? M * a.sc - a.window : MN * a.sc;
  }
#endif
}

template <int D, int WK>
hipError_t launch_one(const FwdArgs& a0, hipStream_t st) {
  FwdArgs a = a0;
  a.n_qtiles = (a.N + BM - 1) / BM;
  a.total_blocks = a.B * a.H * a.n_qtiles;
  // No K-interval table: the weights evaluate T_l = 2^(l step) from the grid index (one
  // v_exp_f32 per element, interpolation two).  In bf16 that measured 25-33 % faster than the
  // per-element LDS gather from a per-row table, which also cost LDS space; the fp8 kernel,
  // whose loop is bound by VALU issue, keeps the table (there the evaluated form was slower).
  const size_t lds = 2 * (size_t)BN * ((D / 8 + 1) + (D / 8 + 4)) * 16;
  const void* kern = a.grid_idx ? (const void*)fwd_bf16<D, WK, true> : (const void*)fwd_bf16<D, WK, false>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  if (a.grid_idx)
    hipLaunchKernelGGL((fwd_bf16<D, WK, true>), dim3(a.total_blocks), dim3(NW * 64), lds, st, a);
  else
    hipLaunchKernelGGL((fwd_bf16<D, WK, false>), dim3(a.total_blocks), dim3(NW * 64), lds, st, a);
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

hipError_t launch_bf16(const FwdArgs& a, int d, int wk, hipStream_t st) {
  if (d == 64) return launch_d<64>(a, wk, st);
  if (d == 128) return launch_d<128>(a, wk, st);
  return hipErrorInvalidValue;
}

}  // namespace qsa
