// Quantized-softmax attention backward on the matrix cores: bf16 Q, K, V and dO, float32
// gradients.  The gradient modes, the per-element derivatives and the parked row constants are
// those of the float32 path (qsa_bwd.hip, qsa_bwd_common.h); here the dot products run on
// v_mfma_f32_32x32x16_bf16.  Score and dP products take the stored bf16 values exactly
// (products exact in fp32, fp32 accumulation); the weights P = w / l and the score gradients
// dS are formed in fp32 and rounded to bf16 (nearest even) as the operands of the dV, dK and
// dQ products, the usual precision of a mixed-precision attention backward.
//
// Three launches on the caller's stream, every one with a lane per query row in its score
// tiles, so each row's grid constants stay in that lane's registers:
//   bwd_rows_m  S^T = K Q^T and dP^T = V dO^T per key tile (a wave owns 32 rows): the visible
//               extrema and their first keys, then l, D and the gradients of m and lo, parked
//               in the first 8 floats of the row's dQ;
//   bwd_dq_m    the same products, dS^T per element, then dQ^T += K^T dS^T with dS^T as the B
//               operand in the score accumulator's own layout and K^T from transposing LDS
//               reads of the K tile;
//   bwd_keys_m  a wave owns 32 keys (K and V operands in registers) and sweeps the query tiles
//               of every query head of its KV head: S^T = K Q^T and dP^T = V dO^T against the
//               Q and dO tiles in LDS, P and dS per element with the row's constants, then
//               through a per-wave LDS scratch (written a row per lane, read back by
//               transposing reads as operands with a lane per key) into dV^T += dO^T P and
//               dK^T += Q^T dS.
// Every launch forms each score as the same chain of MMAs over the head dimension, so the three
// agree on every weight, grid decision and extremum.
#include "qsa_bwd_common.h"
#include "qsa_common.h"
#include "qsa_mfma_util.h"
#include "qsa_weights.h"

namespace qsa {
namespace {

constexpr int MNW = 4;     // waves per workgroup
constexpr int MBN = 64;    // rows of an LDS tile (keys, or query rows in bwd_keys_m)
constexpr int MBM = 128;   // query rows (bwd_rows_m, bwd_dq_m) or keys (bwd_keys_m) per workgroup
constexpr int MSH = 9;     // K-interval table shift for MBM rows: log2(128 * 4)
constexpr int SRS = 72;    // bytes per row of the P / dS scratch of bwd_keys_m (32 bf16 + 8 of padding)

// Slot of 16-byte chunk q of tile row r is q ^ bswz(r).  The tiles are read both ways: by row
// chunks (ds_read_b128, lane (i, h) of a wave reads chunk 2c + h of row i) and by transposing
// reads (ds_read_b64_tr_b16: rows 4h + 0..3 (+8) of a 16-row step, two chunks per row); this XOR
// of the row's low four bits is free of LDS bank conflicts for both (searched on the CPU over
// every linear swizzle of those bits, for 8-, 16- and 32-lane groups).
template <int D>
__device__ __forceinline__ int bswz(int r) {
  return D == 128 ? (((r & 1) ? 4 : 0) ^ ((r & 2) ? 9 : 0) ^ ((r & 4) ? 2 : 0) ^ ((r & 8) ? 1 : 0))
                  : (((r & 1) ? 2 : 0) ^ ((r & 2) ? 4 : 0) ^ ((r & 4) ? 1 : 0) ^ ((r & 8) ? 2 : 0));
}

template <int D> struct BT {
  static constexpr int SL = D / 8;           // 16-byte slots per row
  static constexpr int RR = D * 2;           // bytes per row
  static constexpr int TT = MBN * RR;        // bytes per tile
  static constexpr int LW = SL / MNW;        // tile-load instructions per wave
  static_assert(SL % MNW == 0, "tiles split evenly over the waves");
  static_assert((MNW * 64 / SL) % 16 == 0, "the swizzle repeats every 16 rows");
};

// Per-lane state of tile staging and operand reads, shared by the three kernels.
template <int D>
struct TileIO {
  using L = BT<D>;
  uint32_t voff;           // global byte offset of this lane's slot in load instruction 0
  uint32_t roff[D / 16];   // row-chunk read of chunk 2c + h of row i (lane (i, h))
  uint32_t toff[2][D / 32];// transposing read, rows 4h + q (+8), column block db
  __device__ __forceinline__ void init(int wave, int lane) {
    const int sl = wave * 64 + lane, j = sl / L::SL, c = sl % L::SL;
    voff = (uint32_t)(j * D + 8 * (c ^ bswz<D>(j))) * 2;
    const int li = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int c2 = 0; c2 < D / 16; ++c2) roff[c2] = li * L::RR + 16 * ((2 * c2 + hh) ^ bswz<D>(li));
    const int q = (lane & 15) >> 2, g1 = (lane >> 4) & 1, p = lane & 3;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int r = 4 * hh + q + 8 * hi;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        toff[hi][db] = r * L::RR + 16 * ((4 * db + 2 * g1 + (p >> 1)) ^ bswz<D>(r)) + 8 * (p & 1);
    }
  }
  // rows [r0, r0 + 64) of a [., D] bf16 tensor (rows past nrows read as zero) into lds + dst
  __device__ __forceinline__ void load(const __bf16* src, int r0, int nrows, lds_u8* dst, int wave) const {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(src + (size_t)r0 * D), 0, (nrows - r0) * D * 2, 0x00020000);
#pragma unroll
    for (int m = 0; m < L::LW; ++m)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + (wave + MNW * m) * 1024),
                                               16, voff, m * MNW * 64 * 16, 0, 0);
  }
  // row-chunk operand: chunk 2c + h of row 32 kb + i of the tile at t
  __device__ __forceinline__ u32x4 rows(const lds_u8* t, int kb, int c) const {
    return *(const lds_u32x4*)(t + kb * 32 * L::RR + roff[c]);
  }
  // transposing operand of k-step ks (tile rows 16 ks ..), column block db: A[m = column][k = row]
  __device__ __forceinline__ u32x4 cols(const lds_u8* t, int ks, int db) const {
    const lds_u8* pa = t + 16 * ks * L::RR;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(pa + toff[0][db]));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(pa + toff[1][db]));
    return u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1], __builtin_bit_cast(u32x2, hi)[0],
                 __builtin_bit_cast(u32x2, hi)[1]};
  }
};

// A lane's row operand of a [., D] bf16 tensor: lane (i, h) holds row[16c + 8h .. +7]
template <int D>
__device__ __forceinline__ void row_operand(const __bf16* src, int row, int nrows, int hh, u32x4 (&x)[D / 16]) {
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    x[c] = row < nrows ? *(const u32x4*)(src + (size_t)row * D + 16 * c + 8 * hh) : u32x4{0, 0, 0, 0};
}

// ---- bwd_rows_m ----------------------------------------------------------------------------
template <int D, int WK>
__global__ __launch_bounds__(MNW * 64, 2) void bwd_rows_m(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  const FwdArgs& f = a.f;
  constexpr int KC = D / 16;
  using L = BT<D>;
  extern __shared__ __align__(16) unsigned char smem[];
  lds_u8* const lds = (lds_u8*)smem;  // K stages 0, 1; V stages 0, 1; table
  unsigned char* const Tb = smem + 4 * L::TT;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hh = lane >> 5;
  int bh, qt;
  map_block(f, bh, qt);
  const int b = bh / f.H, h = bh - b * f.H;
  const int kvh = h / (f.H / f.Hkv);
  const int N = f.N;
  const int q0 = qt * MBM, wr0 = q0 + wave * 32, row = wr0 + li;
  const __bf16* Kg = (const __bf16*)f.k + (size_t)(b * f.Hkv + kvh) * N * D;
  const __bf16* Vg = (const __bf16*)f.v + (size_t)(b * f.Hkv + kvh) * N * D;
  u32x4 qf[KC], gf[KC];
  row_operand<D>((const __bf16*)f.q + (size_t)(b * f.H + h) * N * D, row, N, hh, qf);
  row_operand<D>((const __bf16*)a.dout + (size_t)(b * f.H + h) * N * D, row, N, hh, gf);
  const int T = f.causal ? ((min(q0 + MBM, N) - 1) / MBN + 1) : (N + MBN - 1) / MBN;
  const int wlast = wr0 >= N ? -1 : (f.causal ? (min(wr0 + 31, N - 1) / MBN) : T - 1);
  const int lim = f.causal ? min(row, N - 1) : N - 1;
  TileIO<D> io;
  io.init(wave, lane);
  const f32x16 zero16 = {};
  auto prod = [&](const lds_u8* t, int kb, const u32x4 (&bop)[KC]) __attribute__((always_inline)) {
    f32x16 s = zero16;
#pragma unroll
    for (int c = 0; c < KC; ++c) s = mma(io.rows(t, kb, c), bop[c], s);
    return s;
  };
  auto done = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  // tiles t < tfull are visible to every row of the wave (rows past N are never read back)
  const int tfull = ((f.causal ? min(wr0, N - 1) : N - 1) + 1) / MBN;
  const bool minmax = wk_kint(WK) && !f.window_calib;
  // the attached modes add the gradients of m and lo at the arg-max and arg-min: where those
  // are nonzero (see calib below) pass 1 tracks the first key of each extremum
  const bool calib = g_attached(a.mode) &&
                     (WK == WK_TRUNC || wk_kint(WK) || ((WK == WK_POT || WK == WK_POT_FLUSH) && g_ste(a.mode)));
  const bool need_min = minmax || calib;

  // pass 1: extrema over the visible keys, and the first keys that reach them
  float M = -__builtin_inff(), MN = __builtin_inff();
  int amax = 0x7FFFFFFF, amin = 0x7FFFFFFF;
  auto extrema = [&](const f32x16& s, int k0, auto MASK, auto TRACK) __attribute__((always_inline)) {
    constexpr bool masked = decltype(MASK)::value, track = decltype(TRACK)::value;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + acc_off(r);  // increasing in r: the first key wins a tie
      const bool ok = !masked || key <= lim;
      if (track) {
        const bool gt = ok && s[r] > M, lt = ok && s[r] < MN;
        M = gt ? s[r] : M;
        amax = gt ? key : amax;
        MN = lt ? s[r] : MN;
        amin = lt ? key : amin;
      } else {
        M = fmaxf(M, ok ? s[r] : -__builtin_inff());
        if (need_min) MN = fminf(MN, ok ? s[r] : __builtin_inff());
      }
    }
  };
  auto pass1_tile = [&](int t, auto MASK) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const f32x16 s = prod(lds + (t & 1) * L::TT, kb, qf);
      const int k0 = t * MBN + kb * 32 + 4 * hh;
      if (calib) extrema(s, k0, MASK, std::true_type());
      else extrema(s, k0, MASK, std::false_type());
    }
  };
  io.load(Kg, 0, N, lds, wave);
  done();
  for (int t = 0; t < T; ++t) {
    if (t + 1 < T) io.load(Kg, (t + 1) * MBN, N, lds + ((t + 1) & 1) * L::TT, wave);
    if (t < tfull) pass1_tile(t, std::false_type());
    else if (t <= wlast) pass1_tile(t, std::true_type());
    done();
  }
  {  // the two half-waves of a row: larger (smaller) value, then the smaller key
    auto xm = __builtin_amdgcn_permlane32_swap(fbits(M), fbits(M), false, false);
    auto xa = __builtin_amdgcn_permlane32_swap((uint32_t)amax, (uint32_t)amax, false, false);
    auto xn = __builtin_amdgcn_permlane32_swap(fbits(MN), fbits(MN), false, false);
    auto xb = __builtin_amdgcn_permlane32_swap((uint32_t)amin, (uint32_t)amin, false, false);
    const float Mo = bitsf(hh ? xm[0] : xm[1]), MNo = bitsf(hh ? xn[0] : xn[1]);
    const int ao = (int)(hh ? xa[0] : xa[1]), bo = (int)(hh ? xb[0] : xb[1]);
    if (Mo > M || (Mo == M && ao < amax)) { M = Mo; amax = ao; }
    if (MNo < MN || (MNo == MN && bo < amin)) { MN = MNo; amin = bo; }
  }
  if (row >= N) M = MN = 0.0f;
  const RowC rc = make_row<WK, MSH>(f, M, MN, wave * 32 + li, Tb, hh, 2);
  const GridD gd = grid_d(f, M, MN);

  // pass 2: l, D = sum_j P_ij dP_ij and (attached modes) the gradients of m and lo, which are
  // linear in D: sum dP cm and sum cm (likewise for lo) are gathered before D is known
  float l = 0.0f, wdp = 0.0f, pm = 0.0f, sm = 0.0f, plo = 0.0f, slo = 0.0f;
  const bool ste = g_ste(a.mode);
  auto sums = [&](const f32x16& s, const f32x16& dp, int k0, auto MASK, auto CALIB) __attribute__((always_inline)) {
    constexpr bool masked = decltype(MASK)::value, cal = decltype(CALIB)::value;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (!masked || k0 + acc_off(r) <= lim) {
        const float w = Weight<WK>::template w<MSH>(s[r], rc, Tb, f.levels);
        l += w;
        wdp = fmaf(w, dp[r], wdp);
        if (cal) {
          float gs, cm, clo;
          partials<WK, MSH>(s[r], w, rc, Tb, f.levels, gd, minmax, ste, gs, cm, clo);
          pm = fmaf(dp[r], cm, pm);
          sm += cm;
          plo = fmaf(dp[r], clo, plo);
          slo += clo;
        }
      }
    }
  };
  auto pass2_tile = [&](int t, auto MASK) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const f32x16 s = prod(lds + (t & 1) * L::TT, kb, qf);
      const f32x16 dp = prod(lds + (2 + (t & 1)) * L::TT, kb, gf);
      const int k0 = t * MBN + kb * 32 + 4 * hh;
      if (calib) sums(s, dp, k0, MASK, std::true_type());
      else sums(s, dp, k0, MASK, std::false_type());
    }
  };
  io.load(Kg, 0, N, lds, wave);
  io.load(Vg, 0, N, lds + 2 * L::TT, wave);
  done();  // also publishes the K-interval tables
  for (int t = 0; t < T; ++t) {
    if (t + 1 < T) {
      io.load(Kg, (t + 1) * MBN, N, lds + ((t + 1) & 1) * L::TT, wave);
      io.load(Vg, (t + 1) * MBN, N, lds + (2 + ((t + 1) & 1)) * L::TT, wave);
    }
    if (t < tfull) pass2_tile(t, std::false_type());
    else if (t <= wlast) pass2_tile(t, std::true_type());
    done();
  }
  l = half_sum(l);
  wdp = half_sum(wdp);
  pm = half_sum(pm);
  sm = half_sum(sm);
  plo = half_sum(plo);
  slo = half_sum(slo);
  const float Dr = row < N ? wdp / l : 0.0f;
  const float dm = calib && row < N ? fmaf(-Dr, sm, pm) / l : 0.0f;
  const float dlo = calib && row < N ? fmaf(-Dr, slo, plo) / l : 0.0f;
  if (row < N && hh == 0) {
    float* pk = a.dq + ((size_t)(b * f.H + h) * N + row) * D;
    *(f32x4*)pk = f32x4{M, MN, l, Dr};
    *(f32x4*)(pk + 4) = f32x4{dm, dlo, __builtin_bit_cast(float, amax), __builtin_bit_cast(float, amin)};
  }
#endif
}

// ---- bwd_dq_m ------------------------------------------------------------------------------
template <int D, int WK>
__global__ __launch_bounds__(MNW * 64, 2) void bwd_dq_m(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  const FwdArgs& f = a.f;
  constexpr int KC = D / 16, DB = D / 32;
  using L = BT<D>;
  extern __shared__ __align__(16) unsigned char smem[];
  lds_u8* const lds = (lds_u8*)smem;  // K stages 0, 1; V stages 0, 1; table
  unsigned char* const Tb = smem + 4 * L::TT;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hh = lane >> 5;
  int bh, qt;
  map_block(f, bh, qt);
  const int b = bh / f.H, h = bh - b * f.H;
  const int kvh = h / (f.H / f.Hkv);
  const int N = f.N;
  const int q0 = qt * MBM, wr0 = q0 + wave * 32, row = wr0 + li;
  const __bf16* Kg = (const __bf16*)f.k + (size_t)(b * f.Hkv + kvh) * N * D;
  const __bf16* Vg = (const __bf16*)f.v + (size_t)(b * f.Hkv + kvh) * N * D;
  float* dQg = a.dq + ((size_t)(b * f.H + h) * N + row) * D;
  u32x4 qf[KC], gf[KC];
  row_operand<D>((const __bf16*)f.q + (size_t)(b * f.H + h) * N * D, row, N, hh, qf);
  row_operand<D>((const __bf16*)a.dout + (size_t)(b * f.H + h) * N * D, row, N, hh, gf);
  float pk[NPARK];  // before the row is overwritten
#pragma unroll
  for (int c = 0; c < NPARK; ++c) pk[c] = row < N ? dQg[c] : 0.0f;
  const RowC rc = make_row<WK, MSH>(f, pk[0], pk[1], wave * 32 + li, Tb, hh, 2);
  const GridD gd = grid_d(f, pk[0], pk[1]);
  const float il = row < N ? 1.0f / pk[2] : 0.0f;
  const bool minmax = wk_kint(WK) && !f.window_calib;
  const int amax = __builtin_bit_cast(int, pk[6]), amin = __builtin_bit_cast(int, pk[7]);
  const int T = f.causal ? ((min(q0 + MBM, N) - 1) / MBN + 1) : (N + MBN - 1) / MBN;
  const int wlast = wr0 >= N ? -1 : (f.causal ? (min(wr0 + 31, N - 1) / MBN) : T - 1);
  const int lim = f.causal ? min(row, N - 1) : N - 1;
  TileIO<D> io;
  io.init(wave, lane);
  const f32x16 zero16 = {};
  auto prod = [&](const lds_u8* t, int kb, const u32x4 (&bop)[KC]) __attribute__((always_inline)) {
    f32x16 s = zero16;
#pragma unroll
    for (int c = 0; c < KC; ++c) s = mma(io.rows(t, kb, c), bop[c], s);
    return s;
  };
  auto done = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = zero16;

  // tiles t < tfull are visible to every row of the wave (rows past N are never stored)
  const int tfull = ((f.causal ? min(wr0, N - 1) : N - 1) + 1) / MBN;
  // dS^T of the 32 keys of block kb, bf16, as the B operand of dQ^T += K^T dS^T (the score
  // accumulator's layout: lane (i, h) holds 16 keys of query row i, packed by pairs)
  auto block = [&](const lds_u8* Kt, int t, int kb, auto MASK, auto MODE) __attribute__((always_inline)) {
    constexpr bool masked = decltype(MASK)::value;
    constexpr int mode = decltype(MODE)::value;
    const f32x16 s = prod(Kt, kb, qf);
    const f32x16 dp = prod(lds + (2 + (t & 1)) * L::TT, kb, gf);
    const int k0 = t * MBN + kb * 32 + 4 * hh;
    const int dmax = amax - k0, dmin = amin - k0;  // the extrema's offsets from the lane's first key
    u32x4 dsb[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        float ds2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 8 * kc + 2 * p + e;
          float ds = 0.0f;
          if (!masked || k0 + acc_off(r) <= lim) {
            const float w = Weight<WK>::template w<MSH>(s[r], rc, Tb, f.levels);
            ds = dscore_m<WK, MSH, mode>(s[r], w, dp[r], dmax == acc_off(r), dmin == acc_off(r), rc, Tb, f, il, pk[3],
                                         pk[4], pk[5], gd, minmax);
          }
          ds2[e] = ds;
        }
        dsb[kc][p] = pack_bf16(ds2[0], ds2[1]);
      }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int db = 0; db < DB; ++db) dq[db] = mma(io.cols(Kt, 2 * kb + kc, db), dsb[kc], dq[db]);
  };
  io.load(Kg, 0, N, lds, wave);
  io.load(Vg, 0, N, lds + 2 * L::TT, wave);
  done();  // also publishes the K-interval tables
  for (int t = 0; t < T; ++t) {
    if (t + 1 < T) {
      io.load(Kg, (t + 1) * MBN, N, lds + ((t + 1) & 1) * L::TT, wave);
      io.load(Vg, (t + 1) * MBN, N, lds + (2 + ((t + 1) & 1)) * L::TT, wave);
    }
    if (t <= wlast) {
      const lds_u8* Kt = lds + (t & 1) * L::TT;
      with_mode(a.mode, [&](auto MODE) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (t < tfull) block(Kt, t, kb, std::false_type(), MODE);
          else block(Kt, t, kb, std::true_type(), MODE);
        }
      });
    }
    done();
  }
  if (row < N) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dcol = db * 32 + 8 * g4 + 4 * hh;
        *(f32x4*)(dQg + dcol) = f32x4{f.sc * dq[db][4 * g4], f.sc * dq[db][4 * g4 + 1], f.sc * dq[db][4 * g4 + 2],
                                      f.sc * dq[db][4 * g4 + 3]};
      }
  }
#endif
}

// ---- bwd_keys_m ----------------------------------------------------------------------------
template <int D, int WK>
__global__ __launch_bounds__(MNW * 64, 1) void bwd_keys_m(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  const FwdArgs& f = a.f;
  constexpr int KC = D / 16, DB = D / 32;
  using L = BT<D>;
  extern __shared__ __align__(16) unsigned char smem[];
  lds_u8* const lds = (lds_u8*)smem;
  lds_u8* const Qt = lds;                              // query tile (64 rows)
  lds_u8* const Gt = lds + L::TT;                      // dO tile
  float* const Pk = (float*)(smem + 2 * L::TT);       // [64][NPARK] parked row constants
  lds_u8* const Sc = lds + 2 * L::TT + MBN * NPARK * 4;  // per wave: P, dS scratch [64 rows][SRS]
  unsigned char* const Tb = (unsigned char*)(Sc + MNW * 2 * MBN * SRS);  // [K+1][64] tables

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hh = lane >> 5;
  const int N = f.N, nkt = (N + MBM - 1) / MBM, nqt = (N + MBN - 1) / MBN;
  int bkv, kt;
  map_key_block(f, nkt, bkv, kt);
  const int b = bkv / f.Hkv, kvh = bkv - b * f.Hkv;
  const int group = f.H / f.Hkv;
  const int wk0 = kt * MBM + wave * 32;  // the wave's first key
  const __bf16* Kg = (const __bf16*)f.k + (size_t)(b * f.Hkv + kvh) * N * D;
  const __bf16* Vg = (const __bf16*)f.v + (size_t)(b * f.Hkv + kvh) * N * D;
  // K and V rows of the wave's keys as the A operands of S^T = K Q^T and dP^T = V dO^T
  u32x4 kf[KC], vf[KC];
  row_operand<D>(Kg, wk0 + li, N, hh, kf);
  row_operand<D>(Vg, wk0 + li, N, hh, vf);
  TileIO<D> io;
  io.init(wave, lane);
  const f32x16 zero16 = {};
  f32x16 dk[DB], dv[DB];  // dK^T, dV^T: [d][the wave's 32 keys]
#pragma unroll
  for (int db = 0; db < DB; ++db) dk[db] = dv[db] = zero16;
  const bool minmax = wk_kint(WK) && !f.window_calib;
  lds_u8* const Pw = Sc + wave * 2 * MBN * SRS;  // this wave's P scratch, then its dS scratch
  lds_u8* const Dw = Pw + MBN * SRS;
  // transposing reads of the scratch ([row][key], SRS bytes a row): lane 4q + p of group g reads
  // row 4h + q (+8) of the k-step, keys 16(g & 1) + 4p .. +3; lane l gets key l % 32
  const int sq = (lane & 15) >> 2, sg1 = (lane >> 4) & 1, sp = lane & 3;
  const uint32_t soff0 = (4 * hh + sq) * SRS + 2 * (16 * sg1 + 4 * sp), soff1 = soff0 + 8 * SRS;
  auto scols = [&](const lds_u8* t, int ks) __attribute__((always_inline)) {
    const lds_u8* pa = t + 16 * ks * SRS;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(pa + soff0));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(pa + soff1));
    return u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1], __builtin_bit_cast(u32x2, hi)[0],
                 __builtin_bit_cast(u32x2, hi)[1]};
  };
  const int q_first = f.causal ? (kt * MBM) / MBN : 0;  // query tiles with a row at or past the first key
  for (int hq = kvh * group; hq < (kvh + 1) * group; ++hq) {
    const __bf16* Qg = (const __bf16*)f.q + (size_t)(b * f.H + hq) * N * D;
    const __bf16* Gg = (const __bf16*)a.dout + (size_t)(b * f.H + hq) * N * D;
    const float* Pg = a.dq + (size_t)(b * f.H + hq) * N * D;
    for (int qt = q_first; qt < nqt; ++qt) {
      const int r0 = qt * MBN;
      io.load(Qg, r0, N, Qt, wave);
      io.load(Gg, r0, N, Gt, wave);
      if (tid < 2 * MBN) {  // parked constants of the tile's rows: thread 2r + u copies half u of row r's
        // eight, written and read back as the same vector type
        const int r = tid >> 1, u = tid & 1;
        const f32x4 v4 = r0 + r < N ? *(const f32x4*)(Pg + (size_t)(r0 + r) * D + 4 * u) : f32x4{};
        *(f32x4*)(Pk + r * NPARK + 4 * u) = v4;
      }
      {  // the K-interval table of row r (grid values split over the row's four threads)
        const int r = tid >> 2, u = tid & 3;
        const float Mr = r0 + r < N ? Pg[(size_t)(r0 + r) * D] : 0.0f;
        const float MNr = r0 + r < N ? Pg[(size_t)(r0 + r) * D + 1] : 0.0f;
        (void)make_row<WK, SHB>(f, Mr, MNr, r, Tb, u, 4);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      // P and dS of row block rb (32 query rows, a lane per row) for the wave's 32 keys, to the
      // scratch as [row][key] bf16: keys 8j + 4h .. +3 (registers 4j .. 4j+3) are one 8-byte
      // write per matrix
      auto row_block = [&](int rb, auto MASK, auto MODE) __attribute__((always_inline)) {
        constexpr bool masked = decltype(MASK)::value;
        constexpr int mode = decltype(MODE)::value;
        const int rl = 32 * rb + li, row = r0 + rl;
        const f32x4 c0 = *(const f32x4*)(Pk + rl * NPARK), c1 = *(const f32x4*)(Pk + rl * NPARK + 4);
        const RowC rc = make_row<WK, SHB>(f, c0[0], c0[1], rl, nullptr, 0, 1);
        const GridD gd = grid_d(f, c0[0], c0[1]);
        const float il = row < N ? 1.0f / c0[2] : 0.0f;
        // the arg-max and arg-min as scalars first: a bit cast of a vector element read the
        // vector's first element instead
        const float famax = c1[2], famin = c1[3];
        const int k0 = wk0 + 4 * hh;  // the lane's first key
        const int dmax = __builtin_bit_cast(int, famax) - k0, dmin = __builtin_bit_cast(int, famin) - k0;
        f32x16 s = zero16, dp = zero16;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          s = mma(kf[c], io.rows(Qt, rb, c), s);
          dp = mma(vf[c], io.rows(Gt, rb, c), dp);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float pv[4], dv4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * j + e;
            const int key = k0 + acc_off(r);
            float p = 0.0f, ds = 0.0f;
            if (!masked || (row < N && key < N && (!f.causal || key <= row))) {
              const float w = Weight<WK>::template w<SHB>(s[r], rc, Tb, f.levels);
              p = w * il;
              ds = dscore_m<WK, SHB, mode>(s[r], w, dp[r], dmax == acc_off(r), dmin == acc_off(r), rc, Tb, f, il,
                                           c0[3], c1[0], c1[1], gd, minmax);
            }
            pv[e] = p;
            dv4[e] = ds;
          }
          const uint32_t o = rl * SRS + 2 * (8 * j + 4 * hh);
          *(__attribute__((address_space(3))) u32x2*)(Pw + o) = u32x2{pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3])};
          *(__attribute__((address_space(3))) u32x2*)(Dw + o) =
              u32x2{pack_bf16(dv4[0], dv4[1]), pack_bf16(dv4[2], dv4[3])};
        }
      };
      with_mode(a.mode, [&](auto MODE) __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          // every (row, key) of the block visible: its rows and the wave's keys inside the head,
          // and (causal) the wave's last key at or before the block's first row
          const int rf = r0 + 32 * rb;
          const bool full = rf + 31 < N && wk0 + 31 < N && (!f.causal || wk0 + 31 <= rf);
          if (full) row_block(rb, std::false_type(), MODE);
          else row_block(rb, std::true_type(), MODE);
        }
      });
      // dV^T += dO^T P and dK^T += Q^T dS over the tile's 64 rows (four k-steps of 16 rows);
      // the scratch is this wave's own, written above in program order
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 pb = scols(Pw, ks), db_ = scols(Dw, ks);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dv[db] = mma(io.cols(Gt, ks, db), pb, dv[db]);
          dk[db] = mma(io.cols(Qt, ks, db), db_, dk[db]);
        }
      }
      __syncthreads();  // the tiles, constants and tables are refilled for the next query tile
    }
  }
  const int key = wk0 + li;
  if (key < N) {
    float* dKg = a.dk + ((size_t)(b * f.Hkv + kvh) * N + key) * D;
    float* dVg = a.dv + ((size_t)(b * f.Hkv + kvh) * N + key) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dcol = db * 32 + 8 * g4 + 4 * hh;
        *(f32x4*)(dKg + dcol) = f32x4{f.sc * dk[db][4 * g4], f.sc * dk[db][4 * g4 + 1], f.sc * dk[db][4 * g4 + 2],
                                      f.sc * dk[db][4 * g4 + 3]};
        *(f32x4*)(dVg + dcol) = f32x4{dv[db][4 * g4], dv[db][4 * g4 + 1], dv[db][4 * g4 + 2], dv[db][4 * g4 + 3]};
      }
  }
#endif
}

template <int D, int WK>
hipError_t launch_mma(const BwdArgs& a0, hipStream_t st) {
  BwdArgs a = a0;
  a.f.n_qtiles = (a.f.N + MBM - 1) / MBM;
  a.f.total_blocks = a.f.B * a.f.H * a.f.n_qtiles;
  using L = BT<D>;
  const size_t rows_lds = 4 * (size_t)L::TT + table_bytes(WK, MBM, a.f.levels);
  const size_t keys_lds = 2 * (size_t)L::TT + (size_t)MBN * NPARK * 4 + (size_t)MNW * 2 * MBN * SRS +
                          table_bytes(WK, MBN, a.f.levels);
  const void* ks[3] = {(const void*)bwd_rows_m<D, WK>, (const void*)bwd_keys_m<D, WK>, (const void*)bwd_dq_m<D, WK>};
  const size_t lds[3] = {rows_lds, keys_lds, rows_lds};
  for (int i = 0; i < 3; ++i)
    if (lds[i] > 65536) {
      const hipError_t e = hipFuncSetAttribute(ks[i], hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds[i]);
      if (e != hipSuccess) return e;
    }
  hipLaunchKernelGGL((bwd_rows_m<D, WK>), dim3(a.f.total_blocks), dim3(MNW * 64), rows_lds, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int key_blocks = a.f.B * a.f.Hkv * ((a.f.N + MBM - 1) / MBM);
  hipLaunchKernelGGL((bwd_keys_m<D, WK>), dim3(key_blocks), dim3(MNW * 64), keys_lds, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_m<D, WK>), dim3(a.f.total_blocks), dim3(MNW * 64), rows_lds, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_mma_kind(const BwdArgs& a, int wk, hipStream_t st) {
  switch (wk) {
    case WK_EXACT:
    case WK_EXACT_ANCH: return launch_mma<D, WK_EXACT_ANCH>(a, st);  // the same function
    case WK_POT: return launch_mma<D, WK_POT>(a, st);
    case WK_POT_FLUSH: return launch_mma<D, WK_POT_FLUSH>(a, st);
    case WK_KH: return launch_mma<D, WK_KH>(a, st);
    case WK_KH_FLUSH: return launch_mma<D, WK_KH_FLUSH>(a, st);
    case WK_KI: return launch_mma<D, WK_KI>(a, st);
    case WK_KI_FLUSH: return launch_mma<D, WK_KI_FLUSH>(a, st);
    case WK_TRUNC: return launch_mma<D, WK_TRUNC>(a, st);
    case WK_UNIF: return launch_mma<D, WK_UNIF>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_bwd_mma(const BwdArgs& a, int d, int wk, hipStream_t st) {
  if (d == 64) return launch_mma_kind<64>(a, wk, st);
  if (d == 128) return launch_mma_kind<128>(a, wk, st);
  return hipErrorInvalidValue;
}

}  // namespace qsa
