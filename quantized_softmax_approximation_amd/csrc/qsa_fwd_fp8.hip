// Fused quantized-softmax attention forward, OCP fp8 e4m3 Q/K/V with
// per-tensor descales (O in bf16), gfx950 MFMA.
//
// Same structure as the bf16 kernel (one workgroup = 4 waves = 128 query rows, 8 waves = 256
// rows at d = 128 for every kind but the single pass;
// S^T = K Q^T so a lane owns a query row; true-row-max pre-pass; main-loop
// accumulators start at -M; LDS tiles filled ahead of use with one barrier per
// tile; masking only on a wave's last tile), with the score product on the
// 8-bit matrix cores: v_mfma_f32_32x32x64_f8f6f4, 64 key-or-feature columns
// per instruction.  PoT keeps three K and three V tile buffers (K three tiles
// ahead, V two); the other kinds two of each.
//
// The PV product depends on whether the weights fit an 8-bit float exactly:
//   * Rowmax-PoT: the weights 2^-e ("Approximating Softmax in Pretrained
//     LLMs", abstract: power-of-two weights anchored at each row maximum),
//     scaled by the constant 2^(L-15), are exact in bf8 e5m2 for e <= L-1 <= 15
//     (and e = L, the flushed level, is exactly 0), so P^T is built directly as
//     bf8 bytes from the exponent and PV runs on the 8-bit matrix cores with V
//     in e4m3 (operand formats e4m3 x bf8).  The V^T operand comes from 8-bit
//     transposing LDS reads (ds_read_b64_tr_b8).  The row sum of the same bf8
//     weights is one more 8-bit MMA per tile (16x16x128 against a constant 0/1
//     selector), which keeps it off the VALU: on gfx950 VALU work of one wave
//     slows the matrix-core work of the other waves on its SIMD.
//   * exact and K-interval weights are not representable in 8 bits without
//     rounding errors of a few percent per row (e4m3 keeps 3 mantissa bits),
//     so their PV runs in bf16: V tiles are widened e4m3 -> bf16 (exactly)
//     while they are staged into LDS and P^T is bf16, as in the bf16 kernel.
#include "qsa_common.h"
#include "qsa_mfma_util.h"
#include "qsa_weights.h"

// Operand read-ahead (A/B switches): QSA_FP8_KRA reads the second score block's K operands of
// the PoT loop before the weights; QSA_FP8_RAV is the depth of the V operand reads of the
// interpolating K-interval kinds' bf16 PV product.
#ifndef QSA_FP8_KRA
#define QSA_FP8_KRA 1
#endif
#ifndef QSA_FP8_RAV
#define QSA_FP8_RAV 2
#endif
#ifndef QSA_FP8_XRA
#define QSA_FP8_XRA 0
#endif

namespace qsa {
namespace {

// Ablation build only (-DQSA_FP8_POT_PV16=1): Rowmax-PoT with the pre-pass runs the bf16 PV path
// of the exact kinds (bf16 weights built from the exponent field, V widened to bf16), so that
// its time against the exact kinds separates the exponential from the 8-bit PV product.
#ifndef QSA_FP8_POT_PV16
#define QSA_FP8_POT_PV16 0
#endif

constexpr int NW = 4;    // waves per workgroup (8 at d = 128 for most kinds, see launch_one)
constexpr int BN = 64;   // keys per tile
constexpr int BM = 128;  // query rows per workgroup of NW waves
constexpr int SH = 9;    // log2(BM * 4): K-interval table row stride shift

// Slot of 16-byte chunk c of fp8 V row r is c ^ vswz(r) (row bits 1 and 3 for d = 128, bit 3
// for d = 64 pick the chunk pair): conflict-free 8-bit transposing reads of the PoT V tile.
template <int D>
__device__ __forceinline__ int vswz_of(int r) {
  return D == 128 ? 2 * (((r >> 1) & 1) | ((r >> 2) & 2)) : 2 * ((r >> 3) & 1);
}

// Slot of 16-byte chunk q of K row r is q ^ kswz(r).  A ds_read_b128 of the score loop reads
// the same chunk of 32 consecutive rows; with unpadded 128-byte (d = 128) or 64-byte rows the
// XOR puts every 16-row lane group, and every 8-row half of one, on distinct LDS bank groups
// (rows r and r + 32 share the swizzle).
template <int D>
__device__ __forceinline__ int kswz_of(int r) {
  return D == 128 ? ((r & 7) ^ ((r >> 3) & 1)) : (((r >> 1) & 3) ^ ((r >> 3) & 1));
}

// v_pk_mad_u16: a * b + c in each 16-bit half
__device__ __forceinline__ uint32_t pk_mad_u16(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t d;
  asm("v_pk_mad_u16 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// WIDE: the score range of a row may exceed 2^15 log2 units, so the exponent is clamped in
// 32 bits before its low 16 bits are used (the launcher proves when it cannot; PoT only).
// Anchored kinds (all but the online exact control) run after rowext_fp8, which leaves each
// row's score extrema parked in O; the kernel reads them back before it writes O.
template <int D, int WK, bool DUMP, bool WIDE, int NWT = NW>
__global__ __launch_bounds__(NWT * 64, 8 / NWT) void fwd_fp8(FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass needs only the signature (for the launch stub)
  constexpr int KC = D / 64;  // k-steps of the QK product
  constexpr int SHK = NWT == 8 ? SH + 1 : SH;  // K-interval table stride shift for NWT * 32 rows
  constexpr int DB = D / 32;  // 32-column blocks of O^T
  constexpr bool RUN = wk_running(WK);                // single-pass PoT: running integer anchor
  constexpr bool ANCH = (WK != WK_EXACT) && !RUN;     // read the pre-pass extrema
  constexpr bool EXACT_W = (WK == WK_EXACT || WK == WK_EXACT_ANCH);
  constexpr bool POT = wk_pot(WK);
  constexpr bool KHARD = (WK == WK_KH || WK == WK_KH_FLUSH);
  constexpr bool SUPPORT = wk_support(WK), UNIF = (WK == WK_UNIF);
  constexpr bool FLUSH = (WK == WK_POT_FLUSH || WK == WK_POTR_FLUSH || WK == WK_KH_FLUSH || WK == WK_KI_FLUSH);
  constexpr bool PV8 = POT && !(QSA_FP8_POT_PV16 && !RUN);
  constexpr int SK = D / 16;                          // 16-byte slots per K row (swizzled)
  constexpr int SV = PV8 ? D / 16 : (D / 8 + 4);  // fp8 V rows (swizzled, unpadded), or bf16 rows (stride 64 mod 256)
  constexpr int KR = SK * 16, VR = SV * 16;
  auto vswz = [](int r) { return vswz_of<D>(r); };
  constexpr int KT = BN * KR, VT = BN * VR;
  constexpr int KIW = SK / NWT;  // K-tile load instructions per wave
  static_assert(SK % NWT == 0, "K tiles split evenly over the waves");
  constexpr int VIW = (SV + NWT - 1) / NWT;
  // LDS tile buffers: PoT three each for K and V (its loop is described there); the other
  // kinds keep K two tiles ahead and a register-staged V one tile ahead (two buffers each),
  // which measures faster for them.
  constexpr int NKB = PV8 ? 3 : 2, NVB = PV8 ? 3 : 2;
  constexpr int VB0 = NKB * KT;

  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* const Tb = smem + VB0 + NVB * VT;  // K-interval tables
  lds_u8* const lds = (lds_u8*)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  // PoT's main loop issues its prefetches inside per-wave branches: a wave index the compiler
  // knows to be uniform keeps those loads' buffer descriptors in SGPRs (the other kinds
  // prefetch outside any branch and need fewer registers without it)
  const int wave = PV8 ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int li = lane & 31, hh = lane >> 5;
  int bh, qt;
  map_block(a, bh, qt);
  const int b = bh / a.H, h = bh - b * a.H;
  const int kvh = h / (a.H / a.Hkv);
  const int N = a.N;
  const int q0 = qt * (NWT * 32);
  const int wr0 = q0 + wave * 32;
  const int row = wr0 + li;
  const uint8_t* Qg = (const uint8_t*)a.q + (size_t)(b * a.H + h) * N * D;
  const size_t kv_off = (size_t)(b * a.Hkv + kvh) * N * D;
  const uint8_t* const Kg = (const uint8_t*)a.k + kv_off;
  const uint8_t* const Vg = (const uint8_t*)a.v + kv_off;

  // Q^T operand: lane (li, hh) holds Q[row][64c + 32hh .. +31].
  i32x8 qf[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    u32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
    if (row < N) {
      lo = *(const u32x4*)(Qg + (size_t)row * D + 64 * c + 32 * hh);
      hi = *(const u32x4*)(Qg + (size_t)row * D + 64 * c + 32 * hh + 16);
    }
    qf[c] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }

  const int T = a.causal ? ((min(q0 + (NWT * 32), N) - 1) / BN + 1) : (N + BN - 1) / BN;
  const int wlast = wr0 >= N ? -1 : (a.causal ? (min(wr0 + 31, N - 1) / BN) : T - 1);
  const bool last_masked = (a.causal && wlast * BN + BN - 1 > wr0) || (wlast * BN + BN > N);

  // ---- tile staging ------------------------------------------------------
  // K (and V for PoT): buffer loads straight into LDS, 64 consecutive 16-byte
  // slots per wave-instruction; K slot s is row j = s / SK, slot s % SK of the row, which
  // holds chunk (s % SK) ^ kswz(j).
  uint32_t kvo[KIW];
#pragma unroll
  for (int m = 0; m < KIW; ++m) {
    const int sl = (wave + NWT * m) * 64 + lane, j = sl / SK;
    kvo[m] = (uint32_t)(j * D + ((sl % SK) ^ kswz_of<D>(j)) * 16);
  }
  auto tile_rsrc = [&](const uint8_t* base, int kt) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (size_t)kt * BN * D), 0, (N - kt * BN) * D, 0x00020000);
  };
  auto load_k_at = [&](int kt, int off) {  // K tile kt into the LDS bytes at off
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(Kg, kt);
#pragma unroll
    for (int m = 0; m < KIW; ++m)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(lds + off + (wave + NWT * m) * 1024), 16, kvo[m], 0, 0, 0);
  };
  auto load_k = [&](int kt, int buf) { load_k_at(kt, buf * KT); };
  uint32_t vvo[PV8 ? VIW : 1];
  if (PV8) {
#pragma unroll
    for (int m = 0; m < VIW; ++m) {
      const int sl = (wave + NWT * m) * 64 + lane, j = sl / SV;
      vvo[m] = (uint32_t)(j * D + ((sl % SV) ^ vswz(j)) * 16);  // slot (j, c') holds chunk c' ^ vswz(j)
    }
  }
  // bf16-PV kinds: each thread widens a quarter row of V (D/4 fp8 -> bf16) into LDS
  constexpr int VQ = D / NWT;      // bytes of V a thread stages (NWT threads per row)
  constexpr int VQL = VQ / 16;     // 16-byte loads per thread
  u32x4 vst[PV8 ? 1 : VQL];
  const int vrow = tid / NWT, vpart = tid % NWT;
  auto load_v = [&](int kt, int buf) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(Vg, kt);
    if (PV8) {
#pragma unroll
      for (int m = 0; m < VIW; ++m)  // SV % NWT == 0: every wave issues VIW of them
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)(lds + VB0 + buf * VT + (wave + NWT * m) * 1024), 16,
            vvo[m], 0, 0, 0);
    } else {
#pragma unroll
      for (int m = 0; m < VQL; ++m)
        vst[m] = __builtin_amdgcn_raw_buffer_load_b128(r, vrow * D + vpart * VQ + 16 * m, 0, 0);
    }
  };
  auto store_v = [&](int buf) {  // bf16-PV kinds: widen the staged quarter row into the bf16 tile
    if (!PV8) {
      lds_u8* dst = lds + VB0 + buf * VT + vrow * VR + vpart * VQ * 2;
#pragma unroll
      for (int m = 0; m < VQL; ++m) {
        u32x4 w0, w1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t x = vst[m][q];
          const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false);
          const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true);
          if (q < 2) {
            w0[2 * q] = __builtin_bit_cast(uint32_t, lo);
            w0[2 * q + 1] = __builtin_bit_cast(uint32_t, hi);
          } else {
            w1[2 * q - 4] = __builtin_bit_cast(uint32_t, lo);
            w1[2 * q - 3] = __builtin_bit_cast(uint32_t, hi);
          }
        }
        *(lds_u32x4*)(dst + 32 * m) = w0;
        *(lds_u32x4*)(dst + 32 * m + 16) = w1;
      }
    }
  };
  auto loads_done = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  // Wait for this wave's LDS-direct loads except the newest N.  Tile loads are split over the
  // waves (wave w issues slots w, w+NWT, ...): SLOTS/NWT of them, plus one when w < SLOTS % NWT.
  constexpr int NK_MIN = SK / NWT, NV_MIN = PV8 ? SV / NWT : 0;
  static_assert(!PV8 || SV % NWT == 0, "PoT V tiles split evenly over the waves");
  auto loads_done_but = [&](auto n) {
    constexpr int N = DUMP ? 0 : decltype(n)::value;  // the index dump's stores also count in vmcnt
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
  };

  // QK operand reads: lane (li, hh), k-step c: chunks 4c + 2hh and 4c + 2hh + 1 of K row li
  // (32 bytes), at their swizzled slots
  uint32_t koff[KC][2];
#pragma unroll
  for (int c = 0; c < KC; ++c)
#pragma unroll
    for (int u = 0; u < 2; ++u) koff[c][u] = li * KR + 16 * ((4 * c + 2 * hh + u) ^ kswz_of<D>(li));
  auto qk1 = [&](int buf, int kb, const f32x16& init) __attribute__((always_inline)) {
    const lds_u8* kbase = lds + buf * KT + kb * 32 * KR;
    f32x16 s = init;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const u32x4 lo = *(const lds_u32x4*)(kbase + koff[c][0]);
      const u32x4 hi = *(const lds_u32x4*)(kbase + koff[c][1]);
      const i32x8 ka = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      s = mma8<0>(ka, qf[c], c == 0 ? init : s);
    }
    return s;
  };
  auto qk = [&](int buf, f32x16 (&s)[2], const f32x16& init) {
    s[0] = qk1(buf, 0, init);
    s[1] = qk1(buf, 1, init);
  };
  // the same product split into its operand reads and its MMAs, so that the reads can be
  // issued well before the MMAs that use them
  auto kread = [&](int buf, int kb, i32x8 (&ka)[KC]) __attribute__((always_inline)) {
    const lds_u8* kbase = lds + buf * KT + kb * 32 * KR;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const u32x4 lo = *(const lds_u32x4*)(kbase + koff[c][0]);
      const u32x4 hi = *(const lds_u32x4*)(kbase + koff[c][1]);
      ka[c] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  };
  auto kmma = [&](const i32x8 (&ka)[KC], const f32x16& init) __attribute__((always_inline)) {
    f32x16 s = init;
#pragma unroll
    for (int c = 0; c < KC; ++c) s = mma8<0>(ka[c], qf[c], c == 0 ? init : s);
    return s;
  };
  // bf16 PV (exact / K-interval): V^T operand via 16-bit transposing reads of the bf16 tile
  const uint32_t vtr16 = (4 * hh + ((lane & 15) >> 2)) * VR + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
  // (MMA i = DB kc + db.  For the interpolating K-interval kinds the operand of MMA i + 2 is
  // read while MMA i runs, in a pinned order: measured 11-12 % faster at 8K.  The exact and
  // hard-rounding kinds measured 1-3 % slower with it and keep the scheduler's order.)
  auto pv1 = [&](int buf, int kb, const u32x4 (&P)[2], f32x16 (&o)[DB]) {
    const lds_u8* vbase = lds + VB0 + buf * VT + vtr16;
    auto vread = [&](int i) __attribute__((always_inline)) {
      const lds_u8* pa = vbase + (16 * (2 * kb + i / DB)) * VR + 64 * (i % DB);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)pa);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(pa + 8 * VR));
      return u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                   __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]};
    };
    constexpr int RV = (WK == WK_KI || WK == WK_KI_FLUSH) ? QSA_FP8_RAV : 0, NV = 2 * DB;
    if constexpr (RV == 0) {
#pragma unroll
      for (int i = 0; i < NV; ++i) o[i % DB] = mma(vread(i), P[i / DB], o[i % DB]);
    } else {
      u32x4 va[NV];
#pragma unroll
      for (int i = 0; i < RV && i < NV; ++i) va[i] = vread(i);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        if (i + RV < NV) va[i + RV] = vread(i + RV);
        o[i % DB] = mma(va[i], P[i / DB], o[i % DB]);
        __builtin_amdgcn_sched_barrier(0x0406);
      }
    }
  };
  // fp8 PV (PoT): byte e of the P^T operand is key 16(e/8) + 8((e/4)%2) + 4hh + sg(e%4) of the
  // tile, sg = (0, 2, 1, 3) (the byte order in which the weights are packed, see weights8);
  // 8-bit transposing reads put V[that key][dcol] in byte e of lane (dcol, hh): in each
  // 16-lane group, lane 2q + p points at V[row q][8p .. 8p+7] of the group's 16 columns,
  // row q = key 4hh + sg(q%4) + 8(q/4) (+16 per read).  16-byte chunk c of V row r sits in
  // slot c ^ vswz(r) of the row, which spreads the 32 lanes of each half-wave read over all 64
  // LDS banks (vswz depends on row bits 1-3 only, so the +16-row reads keep it).
  int vtr8[DB];
  {
    const int vq = ((lane & 15) >> 1) & 3;
    const int vr = 4 * hh + (((vq & 1) << 1) | (vq >> 1)) + 8 * ((lane & 15) >> 3);
#pragma unroll
    for (int db = 0; db < DB; ++db)
      vtr8[db] = vr * VR + 16 * ((2 * db + ((lane >> 4) & 1)) ^ vswz(vr)) + 8 * (lane & 1);
  }
  // row-sum MMA selector (16x16x128, A = 16 x 128 e4m3): lane l holds row l % 16 and k-group
  // l / 16; rows 0-7 take k-groups 0 and 2, rows 8-15 k-groups 1 and 3, as 1.0 (0x38)
  const int sel = (((lane & 15) < 8) == (((lane >> 4) & 1) == 0)) ? 0x38383838 : 0;
  const i32x8 rs_sel = {sel, sel, sel, sel, sel, sel, sel, sel};
  f32x4 rs = {0.0f, 0.0f, 0.0f, 0.0f};  // PoT row sums (see the epilogue for the layout)
  // V^T operands of the V tile in LDS buffer buf
  auto read_v8 = [&](int buf, i32x8 (&va)[DB]) __attribute__((always_inline)) {
    const lds_u8* vbase = lds + VB0 + buf * VT;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const i32x2 v2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vbase + vtr8[db] + 16 * k * VR));
        va[db][2 * k] = v2[0];
        va[db][2 * k + 1] = v2[1];
      }
  };
  // O^T += V^T P^T and the row-sum MMA
  auto mma_pv8 = [&](const i32x8 (&va)[DB], const uint32_t (&P8)[8], f32x16 (&o)[DB]) __attribute__((always_inline)) {
    const i32x8 pb = {(int)P8[0], (int)P8[1], (int)P8[2], (int)P8[3], (int)P8[4], (int)P8[5], (int)P8[6], (int)P8[7]};
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = mma8<1>(va[db], pb, o[db]);
    rs = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(rs_sel, pb, rs, 0, 1, 0, 0, 0, 0);
  };
  const int lim = a.causal ? min(row, N - 1) : N - 1;
  auto mask_fill = [&](f32x16 (&s)[2], int kt, float fill) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = (kt * BN + kb * 32 + acc_key(r, hh) <= lim) ? s[kb][r] : fill;
  };

  // ---- row extrema of the anchored kinds ------------------------------------
  // rowext_fp8 parked them as raw accumulator values, 8 bytes per row packed at the start of
  // the wave's own 32 rows of O (a contiguous 256-byte run), which this wave later overwrites
  float M = -__builtin_inff(), MN = __builtin_inff();
  if (ANCH) {
    const uint32_t* const park = (const uint32_t*)((const __bf16*)a.o + ((size_t)(b * a.H + h) * N + wr0) * D) + 2 * li;
    M = row < N ? bitsf(park[0]) : 0.0f;
    MN = row < N ? bitsf(park[1]) : 0.0f;
  }

  // interpolation: the line (A_l, B_l) of each interval per row, as in the bf16 kernel
  RowC rc = make_row<WK, SHK, (WK == WK_KI || WK == WK_KI_FLUSH) ? TAB_SLOPE : TAB_PAIRS>(a, M, MN, wave * 32 + li, Tb, hh, 2);
  f32x16 init16;
#pragma unroll
  for (int r = 0; r < 16; ++r) init16[r] = ANCH ? -M : 0.0f;
  const int L = a.levels;
  // PoT: e is clamped to ec = L-1 (or L with flush, whose level weighs 0); the weight
  // 2^(L-15-e) is the bf8 byte (L - e) << 2
  const int ec = FLUSH ? L : L - 1;
  uint32_t pot_clip = 0x00010001u * (uint32_t)(uint16_t)(-ec);  // -ec, twice (int16)
  // the exponent comes from t = G - y rounded by one FMA (see weights8): G = 2^24 for the
  // pre-pass kinds, 1.5 * 2^23 for the single pass (G - A must be exact for negative integer
  // anchors, which 2^24 - A is not); bits(t) = bits(G) - e either way
  constexpr int32_t pot_bits = RUN ? 0x4B400000 : 0x4B800000;
  constexpr float pot_g = RUN ? 12582912.0f : 16777216.0f;
  int32_t pot_lo = pot_bits - ec;                                       // bits of G - ec
  const uint32_t pot_add = 0x00010001u * (uint32_t)(4 * L * 257);     // 4L in both bytes of a half
  const float Kf = (float)a.levels;
  const float kt_hi = 8388608.0f + Kf;  // 2^23 + K
  // Single-pass PoT: A = ceil(running max of s log2 e), an integer.  The weights are formed
  // against a lagging integer anchor Aw <= A (tb = G - Aw, so the FMA below rounds
  // G - (Aw - s log2 e) = G - e_w), with the clip moved by the lag dl = A - Aw: e_w <= ec - dl,
  // i.e. e = e_w + dl <= ec against A.  Every weight then carries the same factor 2^dl
  // relative to A while Aw stays, so O and the row sums need rescaling only when Aw moves,
  // which happens when the lag would pass 30 - L (the bf8 byte (L - e_w) << 2 must stay a
  // normal number) and on the first tile; with flush the lag stays 0 (its level-L byte is 0
  // only unshifted).  The pre-pass kinds start their scores at -M and keep tb = G = 2^24.
  float A = -__builtin_inff(), Aw = -__builtin_inff();
  int dlag = 0;
  const float lagmax = FLUSH ? 0.0f : (float)(30 - L);
  float tb = pot_g;

  // bf16 weights of 32-key block kb (exact / K-interval), as in the bf16 kernel
  auto weights16 = [&](const f32x16& sb, int kb, u32x4 (&P)[2], float& l, int kt, bool masked) {
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int r0 = 8 * kc + 2 * p;
        const float x0 = sb[r0], x1 = sb[r0 + 1];
        uint32_t pk;
        uint32_t i0 = 0, i1 = 0;
        if (EXACT_W) {
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
        } else if (POT) {
          // (ablation build: PoT weights as bf16 exponent fields, as in the bf16 kernel)
          const float t0 = fmaf(x0, rc.c, tb), t1 = fmaf(x1, rc.c, tb);
          const int32_t lo = pot_bits - (L - 1);
          if (!FLUSH) {
            pk = pot_pair(t0, t1, lo);
            if (DUMP) {
              i0 = 127u - ((pk >> 7) & 0x1FFu);
              i1 = 127u - ((pk >> 23) & 0x1FFu);
            }
          } else {
            const int32_t b0 = (int32_t)fbits(t0), b1 = (int32_t)fbits(t1);
            const uint32_t w0 = b0 < lo ? 0u : (((uint32_t)b0 << 23) + (127u << 23));
            const uint32_t w1 = b1 < lo ? 0u : (((uint32_t)b1 << 23) + (127u << 23));
            pk = __builtin_amdgcn_perm(w1, w0, 0x07060302u);
            if (DUMP) {
              i0 = b0 < lo ? 254u : (uint32_t)(pot_bits - b0);
              i1 = b1 < lo ? 254u : (uint32_t)(pot_bits - b1);
            }
          }
        } else if (KHARD) {
          const float t0 = fmaf(x0, -rc.c, 8388608.0f), t1 = fmaf(x1, -rc.c, 8388608.0f);
          // the clamp of l to [0, K] as one v_med3_f32 on t (floats on [2^23, 2^23 + K] order as
          // their bit patterns)
          const int32_t b0 = (int32_t)fbits(__builtin_amdgcn_fmed3f(t0, 8388608.0f, kt_hi));
          const int32_t b1 = (int32_t)fbits(__builtin_amdgcn_fmed3f(t1, 8388608.0f, kt_hi));
          float w0 = *(const float*)(Tb + (((uint32_t)b0 << SHK) + rc.tab));
          float w1 = *(const float*)(Tb + (((uint32_t)b1 << SHK) + rc.tab));
          const float y0 = FLUSH ? -x0 * rc.c : 0.0f, y1 = FLUSH ? -x1 * rc.c : 0.0f;
          if (FLUSH) {
            w0 = y0 > Kf ? 0.0f : w0;
            w1 = y1 > Kf ? 0.0f : w1;
          }
          pk = pack_bf16(w0, w1);
          if (DUMP) {
            i0 = (FLUSH && y0 > Kf) ? 254u : (uint32_t)(b0 - 0x4B000000);
            i1 = (FLUSH && y1 > Kf) ? 254u : (uint32_t)(b1 - 0x4B000000);
          }
        } else {  // K-interval, interpolation between T_l and T_l+1, l = floor(min(y, K))
          // t = y + 2^23 - 1/2 rounded by the FMA holds floor(y) in its low bits for y >= 1/2 (at
          // an integer y either neighbour, where the weight is continuous); the v_med3_f32
          // clamps l to [0, K]; the table's line of interval l gives the weight from the raw
          // score in one FMA (flushing kind: entry K is 0)
          const float t0 = fmaf(x0, -rc.c, 8388607.5f), t1 = fmaf(x1, -rc.c, 8388607.5f);
          const uint32_t b0 = fbits(__builtin_amdgcn_fmed3f(t0, 8388608.0f, kt_hi));
          const uint32_t b1 = fbits(__builtin_amdgcn_fmed3f(t1, 8388608.0f, kt_hi));
          typedef float f2 __attribute__((ext_vector_type(2)));
          const f2 e0 = *(const f2*)(Tb + ((b0 << (SHK + 1)) + rc.tab));
          const f2 e1 = *(const f2*)(Tb + ((b1 << (SHK + 1)) + rc.tab));
          pk = pack_bf16(fmaf(x0, e0.y, e0.x), fmaf(x1, e1.y, e1.x));
          if (DUMP) {
            const uint32_t l0 = b0 - 0x4B000000u, l1 = b1 - 0x4B000000u;
            i0 = (FLUSH && l0 == (uint32_t)L) ? 254u : l0;
            i1 = (FLUSH && l1 == (uint32_t)L) ? 254u : l1;
          }
        }
        const int k0 = kt * BN + kb * 32 + acc_key(r0, hh);
        if (masked) {
          const uint32_t m0 = k0 <= lim ? 0x0000FFFFu : 0u, m1 = k0 + 1 <= lim ? 0xFFFF0000u : 0u;
          pk &= (m0 | m1);
          if (DUMP) {
            i0 = k0 <= lim ? i0 : 255u;
            i1 = k0 + 1 <= lim ? i1 : 255u;
          }
        }
        if (DUMP && row >= a.idx_row0 && row < a.idx_row0 + a.idx_rows && row < N) {
          uint8_t* dst = a.grid_idx + ((size_t)bh * a.idx_rows + (row - a.idx_row0)) * N;
          if (k0 < N) dst[k0] = (uint8_t)i0;
          if (k0 + 1 < N) dst[k0 + 1] = (uint8_t)i1;
        }
        P[kc][p] = pk;
        l = dot2_ones(pk, l);
      }
  };

  // PoT weights of a whole 64-key tile as bf8 bytes (P8); their row sum goes to rs by an MMA.
  // t = G - y rounded to an integer (y = (m - s) log2 e >= 0, or A - s log2 e for the single
  // pass; the FMA rounds to nearest even): the low 16 bits of its pattern are -e.  For four elements r0..r0+3 the clamped
  // pairs (-e0, -e1) and (-e2, -e3) become the bytes 4(L - e) in the order r0, r0+2, r0+1,
  // r0+3 by two v_pk_mad_u16: 4(-e) + 4L*257 gives byte 0 and a carry-free 4L in byte 1 of
  // each half, then 1024(-e') adds the second pair's bytes in byte 1.
  auto weights8 = [&](const f32x16 (&s)[2], uint32_t (&P8)[8], int kt, bool masked) __attribute__((always_inline)) {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int kb = w >> 2, r0 = 4 * (w & 3);
      uint32_t u[2];
#pragma unroll
      for (int hp = 0; hp < 2; ++hp) {
        const int r = r0 + 2 * hp;
        uint32_t t0 = fbits(fmaf(s[kb][r], rc.c, tb)), t1 = fbits(fmaf(s[kb][r + 1], rc.c, tb));
        if (WIDE || DUMP) {  // clamp in 32 bits: exact for any y
          t0 = (uint32_t)max((int32_t)t0, pot_lo);
          t1 = (uint32_t)max((int32_t)t1, pot_lo);
        }
        u[hp] = __builtin_amdgcn_perm(t1, t0, 0x05040100u);
        if (!(WIDE || DUMP))  // y < 2^15: the 16-bit exponent does not wrap
          u[hp] = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s16x2, u[hp]),
                                                                         __builtin_bit_cast(s16x2, pot_clip)));
        if (DUMP && row >= a.idx_row0 && row < a.idx_row0 + a.idx_rows && row < N) {
          uint8_t* dst = a.grid_idx + ((size_t)bh * a.idx_rows + (row - a.idx_row0)) * N;
          const int key0 = kt * BN + kb * 32 + acc_key(r, hh);
          const s16x2 ue = __builtin_bit_cast(s16x2, u[hp]);
          const int e0 = -(int)ue[0] + dlag, e1 = -(int)ue[1] + dlag;  // against the running anchor
          if (key0 < N) dst[key0] = key0 > lim ? 255u : (FLUSH && e0 == L) ? 254u : (uint8_t)e0;
          if (key0 + 1 < N) dst[key0 + 1] = key0 + 1 > lim ? 255u : (FLUSH && e1 == L) ? 254u : (uint8_t)e1;
        }
      }
      uint32_t p = pk_mad_u16(u[1], 0x04000400u, pk_mad_u16(u[0], 0x00040004u, pot_add));
      if (masked) {  // bytes: r0, r0+2, r0+1, r0+3
        const int key0 = kt * BN + kb * 32 + acc_key(r0, hh);
        p &= (key0 <= lim ? 0x000000FFu : 0u) | (key0 + 2 <= lim ? 0x0000FF00u : 0u) |
             (key0 + 1 <= lim ? 0x00FF0000u : 0u) | (key0 + 3 <= lim ? 0xFF000000u : 0u);
      }
      P8[w] = p;
    }
  };

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

  // Single-pass PoT: fold the maximum of the next tile into the anchor A before its weights
  // are formed; when the weight anchor Aw has to move (see above), O and the row sums, formed
  // against the old Aw, are scaled by 2^(Aw_old - Aw) (exact).  The row-sum MMA leaves the sum
  // of query q(l) in lane l (q = l, l-16, l-16, l-32 for the four 16-lane groups; see the
  // epilogue), whose factor is fetched from lane q(l).
  auto run_anchor = [&](const f32x16 (&s)[2], f32x16 (&o)[DB], int kt, bool masked) __attribute__((always_inline)) {
    float tm = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        tm = fmaxf(tm, (!masked || kt * BN + kb * 32 + acc_key(r, hh) <= lim) ? s[kb][r] : -__builtin_inff());
    const float An = fmaxf(A, __builtin_ceilf(half_max(tm) * rc.c));
    if (__builtin_amdgcn_ballot_w64(An - Aw > lagmax)) {  // Aw = -inf before the first tile
      const bool move = An - Aw > lagmax;
      const float alpha = move ? (Aw > -__builtin_inff() ? __builtin_ldexpf(1.0f, (int)(Aw - An)) : 0.0f) : 1.0f;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      const int ql = lane < 16 ? lane : (lane < 48 ? lane - 16 : lane - 32);
      rs *= bitsf(__builtin_amdgcn_ds_bpermute(4 * ql, (int)fbits(alpha)));
      Aw = move ? An : Aw;
      tb = pot_g - Aw;
    }
    A = An;
    dlag = (int)(A - Aw);
    pot_clip = 0x00010001u * (uint32_t)(uint16_t)(dlag - ec);
    pot_lo = pot_bits - ec + dlag;
  };

  // ---- main loop --------------------------------------------------------------
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float l = 0.0f;
  load_v(0, 0);
  if (PV8) load_v(min(1, T - 1), 1);  // PoT: V(1) is read before the loop's first barrier
  for (int j = 0; j < NKB; ++j)
    if (j < T) load_k(j, j);
  loads_done();
  store_v(0);
  __syncthreads();  // also publishes the K-interval tables
  f32x16 s[2];
  if constexpr (PV8) {
    // PoT, software-pipelined: iteration t multiplies P(t) by V(t) while it reads the V
    // operands of tile t+1, forms the weights of tile t+1 and issues the scores of tile t+2.
    // The PV MMAs then depend on nothing this iteration computes or reads: they are issued
    // between its weight VALU instructions (2 % faster than forming P(t) and multiplying it
    // in one iteration) and do not wait for the latency of their V reads (2 % faster than
    // reading V(t) in iteration t).  K and V tile j sit in LDS buffer j % 3.  Iteration t
    // reads K(t+2) and V(t+1), and prefetches K(t+4) into the buffer of K(t+1) and V(t+3)
    // into that of V(t), both last read in iteration t-1; at its end K(t+3) and V(t+2),
    // issued one iteration earlier, must have landed.  The prefetch is issued after the V
    // operand reads (the compiler makes transposing LDS reads wait for every LDS-direct load
    // issued before them).
    uint32_t P8c[8];  // weights of tile t, consumed by PV in iteration t
    i32x8 va[DB];     // V operands of tile t, consumed by PV in iteration t
    {
      f32x16 s0[2];
      if (wlast >= 0) {
        qk(0, s0, init16);
        read_v8(0, va);
      }
      if (wlast >= 1) qk(1, s, init16);
      __syncthreads();  // every wave has read K(0) before its buffer is refilled
      // the loads iteration -1 would have issued
      load_k(min(3, T - 1), 0);
      load_v(min(2, T - 1), 2);
      if (wlast >= 0) {
        if (RUN) run_anchor(s0, o, 0, wlast == 0 && last_masked);
        weights8(s0, P8c, 0, wlast == 0 && last_masked);
      }
    }
    int t = 0;
    // Every iteration issues the same loads, so that neither the prefetch nor the wait needs a
    // branch: past the last tile it reloads tile T-1 into a buffer no later iteration reads
    // (K(t+4) and V(t+3) would be read in iteration t+2, only if t+4 <= wlast or t+3 <= wlast).
    auto prefetch_to = [&](int b0, int b1) {
      load_k(min(t + 4, T - 1), b1);
      load_v(min(t + 3, T - 1), b0);
    };
    auto wait_tiles = [&]() {
      // K(t+3) and V(t+2) must have landed; this iteration's loads may still be in flight
      loads_done_but(std::integral_constant<int, NK_MIN + NV_MIN>());
      lds_barrier();
    };
    // steady state: tiles t, t+1 and t+2 all hold visible keys, none needs masking
    // Single pass: the wave holds a raised issue priority while it issues its MMAs, so that of
    // the two waves on a SIMD the one with matrix work ready goes first (measured: -2 % for the
    // single pass, +3.5 % for PoT with the pre-pass, which therefore runs without it).
    auto prio_hi = [&]() __attribute__((always_inline)) {
      if (RUN) __builtin_amdgcn_s_setprio(1);
    };
    auto prio_lo = [&]() __attribute__((always_inline)) {
      if (RUN) __builtin_amdgcn_s_setprio(0);
    };
    auto steady = [&](int b0, int b1, int b2) __attribute__((always_inline)) {
      prio_hi();
      mma_pv8(va, P8c, o);
      read_v8(b1, va);
      prefetch_to(b0, b1);
#if QSA_FP8_KRA
      // the second block's K operands are read before the weights, which cover their latency
      // (measured 1.5-1.9 % faster for PoT at 8K, 1-1.6 % for the single pass)
      const f32x16 sn0 = qk1(b2, 0, init16);
      i32x8 k1[KC];
      kread(b2, 1, k1);
      __builtin_amdgcn_sched_barrier(0x0406);  // (LDS reads and MMAs stay on their side)
      prio_lo();
      if (RUN) run_anchor(s, o, t + 1, false);
      weights8(s, P8c, t + 1, false);
      prio_hi();
      const f32x16 sn1 = kmma(k1, init16);
      prio_lo();
#else
      const f32x16 sn0 = qk1(b2, 0, init16);
      prio_lo();
      if (RUN) run_anchor(s, o, t + 1, false);
      weights8(s, P8c, t + 1, false);
      prio_hi();
      const f32x16 sn1 = qk1(b2, 1, init16);
      prio_lo();
#endif
      s[0] = sn0;
      s[1] = sn1;
      wait_tiles();
    };
    // (unrolling this loop by three, which makes every LDS address a constant, measured the same)
    int b0 = 0, b1 = 1, b2 = 2;  // t % 3, (t+1) % 3, (t+2) % 3
    for (; t + 2 <= wlast; ++t) {
      steady(b0, b1, b2);
      b0 = b1;
      b1 = b2;
      b2 = b2 + 1 == 3 ? 0 : b2 + 1;
    }
    // the last two tiles of this wave (the last may need masking), then the iterations in
    // which the wave only issues its share of the other waves' tile loads
    for (; t < T; ++t) {
      if (t + 1 == wlast) {
        mma_pv8(va, P8c, o);
        read_v8(b1, va);
        prefetch_to(b0, b1);
        if (RUN) run_anchor(s, o, t + 1, last_masked);
        weights8(s, P8c, t + 1, last_masked);
      } else if (t == wlast) {
        mma_pv8(va, P8c, o);
        prefetch_to(b0, b1);
      } else {
        prefetch_to(b0, b1);
      }
      wait_tiles();
      b0 = b1;
      b1 = b2;
      b2 = b2 + 1 == 3 ? 0 : b2 + 1;
    }
    loads_done();  // no LDS-direct load outlives the workgroup
  } else {
    // exact and K-interval: K two tiles ahead in two LDS buffers, V one tile ahead through
    // registers (widened to bf16 into the other V buffer at the end of the iteration)
    if (wlast >= 0) qk(0, s, init16);
    __syncthreads();  // every wave has read K tile 0 before iteration 0 refills its buffer
    int kl = 0, kn = 1;  // buffers of K(t) and K(t+1)
    for (int t = 0; t < T; ++t) {
      if (t + NKB < T) load_k(t + NKB, kl);  // buffer of K(t), last read in iteration t-1
      if (t + 1 < T) load_v(t + 1, (t + 1) & 1);
      if (t < wlast) {
        const f32x16 sn0 = qk1(kn, 0, init16);
        if (WK == WK_EXACT) online_max(s, o, l);
        u32x4 P[2];
        weights16(s[0], 0, P, l, t, false);
        pv1(t & 1, 0, P, o);
        const f32x16 sn1 = qk1(kn, 1, init16);
        weights16(s[1], 1, P, l, t, false);
        pv1(t & 1, 1, P, o);
        s[0] = sn0;
        s[1] = sn1;
      } else if (t == wlast) {
        if (WK == WK_EXACT) {
          f32x16 sm[2] = {s[0], s[1]};
          if (last_masked) mask_fill(sm, t, -__builtin_inff());
          online_max(sm, o, l);
        }
        u32x4 P[2];
        weights16(s[0], 0, P, l, t, last_masked);
        pv1(t & 1, 0, P, o);
        weights16(s[1], 1, P, l, t, last_masked);
        pv1(t & 1, 1, P, o);
      }
      loads_done();
      if (t + 1 < T) store_v((t + 1) & 1);
      __syncthreads();
      kl = kn;
      kn = kn + 1 == NKB ? 0 : kn + 1;
    }
  }

  // ---- epilogue -----------------------------------------------------------
  if (wlast < 0) return;
  // PoT: the row-sum MMA leaves the sum of query n (+16) in lanes n, n+16 (n+32, n+48), register 0
  const float lt = PV8 ? bitsf(__builtin_amdgcn_ds_bpermute(4 * (li < 16 ? li : li + 16), (int)fbits(rs[0])))
                       : half_sum(l);
  if (DUMP && row >= a.idx_row0 && row < a.idx_row0 + a.idx_rows && row < N) {
    uint8_t* dst = a.grid_idx + ((size_t)bh * a.idx_rows + (row - a.idx_row0)) * N;
    for (int key = (wlast + 1) * BN + hh; key < N; key += 2) dst[key] = 255u;
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
    // PoT P carries 2^(L-15) (and, single pass, 2^dlag against the final anchor)
    if (a.row_sum) a.row_sum[ri] = PV8 ? __builtin_ldexpf(lt, 15 - L - dlag) : lt;
    if (a.row_lo) a.row_lo[ri] = ((wk_kint(WK) && a.window_calib) || wk_support(WK)) ? M * a.sc - a.window : MN * a.sc;
  }
#endif
}

// ---- row-extrema pre-pass with two row blocks per wave ----------------------------------
// The same extrema as the pre-pass block of fwd_fp8 (the same MMAs in the same order, so the
// same fp32 scores), but a wave owns RB = 2 blocks of 32 query rows: every K operand read from
// LDS feeds two MMAs, which halves the LDS reads per MMA.  Scores of tile t+1 are issued before
// the extrema of tile t are folded.  The extrema are parked in O where fwd_fp8 reads them.
constexpr int XNW = 4;              // waves per workgroup
constexpr int XRB = 2;              // 32-row blocks per wave
constexpr int XBM = XNW * 32 * XRB;  // query rows per workgroup
constexpr int XNB = 2;              // K tile buffers (K loads run XNB tiles ahead; 2 measured 1 % faster than 3)
constexpr int XOCC = 2;             // workgroups per CU the register budget is sized for

template <int D, bool TMIN>
__global__ __launch_bounds__(XNW * 64, XOCC) void rowext_fp8(FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int KC = D / 64;
  constexpr int SK = D / 16;  // 16-byte slots per K row (swizzled as in fwd_fp8)
  constexpr int KR = SK * 16, KT = BN * KR;
  constexpr int KIW = SK / XNW;  // K-tile load instructions per wave
  static_assert(SK % XNW == 0, "K tiles split evenly over the waves");

  extern __shared__ __align__(16) unsigned char smem[];
  lds_u8* const lds = (lds_u8*)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loop control
  const int li = lane & 31, hh = lane >> 5;
  int bh, qt;
  map_block(a, bh, qt);
  const int b = bh / a.H, h = bh - b * a.H;
  const int kvh = h / (a.H / a.Hkv);
  const int N = a.N;
  const int q0 = qt * XBM;
  const int wr0 = q0 + wave * 32 * XRB;
  const uint8_t* Qg = (const uint8_t*)a.q + (size_t)(b * a.H + h) * N * D;
  const uint8_t* const Kg = (const uint8_t*)a.k + (size_t)(b * a.Hkv + kvh) * N * D;

  // Q^T operands, lane (li, hh) of block rb: Q[wr0 + 32 rb + li][64c + 32hh .. +31]
  i32x8 qf[XRB][KC];
#pragma unroll
  for (int rb = 0; rb < XRB; ++rb) {
    const int row = wr0 + 32 * rb + li;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      u32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
      if (row < N) {
        lo = *(const u32x4*)(Qg + (size_t)row * D + 64 * c + 32 * hh);
        hi = *(const u32x4*)(Qg + (size_t)row * D + 64 * c + 32 * hh + 16);
      }
      qf[rb][c] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  }

  const int T = a.causal ? ((min(q0 + XBM, N) - 1) / BN + 1) : (N + BN - 1) / BN;
  int last[XRB];
  bool lmask[XRB];
  int tclean = T;  // tiles t < tclean are visible and unmasked for every row block of the wave
#pragma unroll
  for (int rb = 0; rb < XRB; ++rb) {
    const int r0 = wr0 + 32 * rb;
    last[rb] = r0 >= N ? -1 : (a.causal ? (min(r0 + 31, N - 1) / BN) : T - 1);
    lmask[rb] = (a.causal && last[rb] * BN + BN - 1 > r0) || (last[rb] * BN + BN > N);
    tclean = min(tclean, lmask[rb] ? last[rb] : last[rb] + 1);
  }
  const int wlast = max(last[0], last[1]);

  // K tiles: slot s (64 per wave instruction) is row j = s / SK, slot s % SK of the row,
  // which holds chunk (s % SK) ^ kswz(j)
  uint32_t kvo[KIW];
#pragma unroll
  for (int m = 0; m < KIW; ++m) {
    const int sl = (wave + XNW * m) * 64 + lane, j = sl / SK;
    kvo[m] = (uint32_t)(j * D + ((sl % SK) ^ kswz_of<D>(j)) * 16);
  }
  auto load_k = [&](int kt, int buf) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Kg + (size_t)kt * BN * D), 0, (N - kt * BN) * D, 0x00020000);
#pragma unroll
    for (int m = 0; m < KIW; ++m)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(lds + buf * KT + (wave + XNW * m) * 1024), 16, kvo[m], 0, 0, 0);
  };

  uint32_t koff[KC][2];  // chunks 4c + 2hh (+1) of K row li at their swizzled slots
#pragma unroll
  for (int c = 0; c < KC; ++c)
#pragma unroll
    for (int u = 0; u < 2; ++u) koff[c][u] = li * KR + 16 * ((4 * c + 2 * hh + u) ^ kswz_of<D>(li));
  const f32x16 zero16 = {};
  // scores of tile buf for both row blocks: s[rb][kb] = 32 keys kb x 32 rows rb (S^T)
  // (operand j = KC kb + c; with QSA_FP8_XRA > 0 the operand of j + QSA_FP8_XRA is read while
  // j's MMAs run, in a pinned order)
  auto qk = [&](int buf, f32x16 (&s)[XRB][2]) {
    auto kread = [&](int j) __attribute__((always_inline)) {
      const lds_u8* kbase = lds + buf * KT + (j / KC) * 32 * KR;
      const u32x4 lo = *(const lds_u32x4*)(kbase + koff[j % KC][0]);
      const u32x4 hi = *(const lds_u32x4*)(kbase + koff[j % KC][1]);
      return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    constexpr int RX = QSA_FP8_XRA, NJ = 2 * KC;
    if constexpr (RX == 0) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int kb = j / KC, c = j % KC;
        const i32x8 ka = kread(j);
#pragma unroll
        for (int rb = 0; rb < XRB; ++rb) s[rb][kb] = mma8<0>(ka, qf[rb][c], c == 0 ? zero16 : s[rb][kb]);
      }
    } else {
      i32x8 kr[NJ];
#pragma unroll
      for (int j = 0; j < RX && j < NJ; ++j) kr[j] = kread(j);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int kb = j / KC, c = j % KC;
        if (j + RX < NJ) kr[j + RX] = kread(j + RX);
#pragma unroll
        for (int rb = 0; rb < XRB; ++rb) s[rb][kb] = mma8<0>(kr[j], qf[rb][c], c == 0 ? zero16 : s[rb][kb]);
        __builtin_amdgcn_sched_barrier(0x0406);
      }
    }
  };
  float M[XRB], MN[XRB];
#pragma unroll
  for (int rb = 0; rb < XRB; ++rb) {
    M[rb] = -__builtin_inff();
    MN[rb] = __builtin_inff();
  }
  auto fold = [&](int rb, const f32x16 (&s)[2], int kt, bool masked) {
    const int row = wr0 + 32 * rb + li;
    const int lim = a.causal ? min(row, N - 1) : N - 1;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool ok = !masked || kt * BN + kb * 32 + acc_key(r, hh) <= lim;
        M[rb] = fmaxf(M[rb], ok ? s[kb][r] : -__builtin_inff());
        if (TMIN) MN[rb] = fminf(MN[rb], ok ? s[kb][r] : __builtin_inff());
      }
  };
  auto fold_all = [&](const f32x16 (&s)[XRB][2], int t) {
#pragma unroll
    for (int rb = 0; rb < XRB; ++rb) {
      if (t < last[rb]) fold(rb, s[rb], t, false);
      else if (t == last[rb]) fold(rb, s[rb], t, lmask[rb]);
    }
  };

  for (int j = 0; j < XNB; ++j)
    if (j < T) load_k(j, j);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  f32x16 s[XRB][2];
  if (wlast >= 0) qk(0, s);
  __syncthreads();  // every wave has read K tile 0 before iteration 0 refills its buffer
  int kl = 0, kn = 1;  // buffers of K(t) and K(t+1)
  int t = 0;
  auto end_iteration = [&]() {
    // K(t+2) must have landed: with two buffers it is this iteration's load; with three,
    // this iteration's K(t+3) may stay in flight
    if (XNB == 3 && t + 3 < T) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(KIW) : "memory");
      lds_barrier();
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
    kl = kn;
    kn = kn + 1 == XNB ? 0 : kn + 1;
  };
  // steady state: tile t is unmasked for both row blocks and tile t+1 is needed.  Unrolled
  // by two so that the score sets swap roles instead of being copied.
  auto step = [&](const f32x16 (&cur)[XRB][2], f32x16 (&nxt)[XRB][2]) {
    if (t + XNB < T) load_k(t + XNB, kl);  // buffer of K(t), last read in iteration t-1
    qk(kn, nxt);
#pragma unroll
    for (int rb = 0; rb < XRB; ++rb) fold(rb, cur[rb], t, false);
    end_iteration();
  };
  f32x16 s2[XRB][2];
  for (; t + 2 < tclean; t += 2) {
    step(s, s2);
    ++t;
    step(s2, s);
    --t;
  }
  if (t + 1 < tclean) {
    step(s, s2);
#pragma unroll
    for (int rb = 0; rb < XRB; ++rb) {
      s[rb][0] = s2[rb][0];
      s[rb][1] = s2[rb][1];
    }
    ++t;
  }
  // the remaining tiles of the wave (masked or past a row block's last), then the iterations
  // in which it only issues its share of the other waves' tile loads
  for (; t < T; ++t) {
    if (t + XNB < T) load_k(t + XNB, kl);
    if (t < wlast) {
      f32x16 sn[XRB][2];
      qk(kn, sn);
      fold_all(s, t);
#pragma unroll
      for (int rb = 0; rb < XRB; ++rb) {
        s[rb][0] = sn[rb][0];
        s[rb][1] = sn[rb][1];
      }
    } else if (t == wlast) {
      fold_all(s, t);
    }
    end_iteration();
  }

#pragma unroll
  for (int rb = 0; rb < XRB; ++rb) {
    const float m = half_max(M[rb]);
    const float mn = half_min(MN[rb]);
    const int r0 = wr0 + 32 * rb;
    // packed at the start of the 32-row block's slice of O, where fwd_fp8 reads them
    uint32_t* const park = (uint32_t*)((__bf16*)a.o + ((size_t)bh * N + r0) * D) + 2 * li;
    if (hh == 0 && r0 + li < N) {
      park[0] = fbits(m);
      park[1] = fbits(mn);
    }
  }
#endif
}

template <int D, int WK>
hipError_t launch_one(const FwdArgs& a0, hipStream_t st) {
  FwdArgs a = a0;
  a.n_qtiles = (a.N + BM - 1) / BM;
  a.total_blocks = a.B * a.H * a.n_qtiles;
  constexpr bool PV8 = wk_pot(WK) && !(QSA_FP8_POT_PV16 && !wk_running(WK));
  constexpr bool ANCH = WK != WK_EXACT && !wk_running(WK);
  constexpr int SK = D / 16, SV = PV8 ? D / 16 : (D / 8 + 4);
  constexpr int NB = PV8 ? 3 : 2;  // K and V tile buffers
  // d = 128: 8 waves (256 query rows) per workgroup and one workgroup per CU, the same 2 waves
  // per SIMD; a K or V tile is then half the load instructions per wave and one LDS copy serves
  // twice the rows (the bf16-PV kinds stage V an eighth of a row per thread).  Measured at 8K
  // against 4 waves: PoT 0.649 -> 0.643 ms non-causal; the bf16-PV kinds 5-13 % faster.  The
  // single-pass kind measured 5-6 % slower with 8 and keeps 4.
  constexpr int NWK = (D == 128 && !wk_running(WK)) ? 8 : NW;
  const size_t lds = (size_t)BN * NB * (SK + SV) * 16 + table_bytes(WK, NWK * 32, a.levels);
  // PoT: |raw score| <= d * 448^2 for e4m3 inputs, so y = (m - s) * scale * log2 e stays below
  // 2^15 (no 16-bit wrap of the exponent) whenever 2 d 448^2 sc log2 e does (the single-pass
  // anchor adds less than 1 to y, inside the margin to 2^15)
  const bool wide = PV8 && 2.0 * D * 448.0 * 448.0 * (double)a.sc * 1.4426950408889634 >= 32000.0;
  a.n_qtiles = (a.N + NWK * 32 - 1) / (NWK * 32);
  a.total_blocks = a.B * a.H * a.n_qtiles;
  const void* kern = a.grid_idx ? (const void*)fwd_fp8<D, WK, true, false, NWK>
                                : wide ? (const void*)fwd_fp8<D, WK, false, PV8, NWK> : (const void*)fwd_fp8<D, WK, false, false, NWK>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  if constexpr (ANCH) {  // the row-extrema pre-pass, on its own workgroup grid
    FwdArgs x = a0;
    x.n_qtiles = (x.N + XBM - 1) / XBM;
    x.total_blocks = x.B * x.H * x.n_qtiles;
    const size_t xl = (size_t)BN * XNB * SK * 16;  // K tile buffers only
    if (x.track_min)
      hipLaunchKernelGGL((rowext_fp8<D, true>), dim3(x.total_blocks), dim3(XNW * 64), xl, st, x);
    else
      hipLaunchKernelGGL((rowext_fp8<D, false>), dim3(x.total_blocks), dim3(XNW * 64), xl, st, x);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.grid_idx)
    hipLaunchKernelGGL((fwd_fp8<D, WK, true, false, NWK>), dim3(a.total_blocks), dim3(NWK * 64), lds, st, a);
  else if (wide)
    hipLaunchKernelGGL((fwd_fp8<D, WK, false, PV8, NWK>), dim3(a.total_blocks), dim3(NWK * 64), lds, st, a);
  else
    hipLaunchKernelGGL((fwd_fp8<D, WK, false, false, NWK>), dim3(a.total_blocks), dim3(NWK * 64), lds, st, a);
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

hipError_t launch_fp8(const FwdArgs& a, int d, int wk, hipStream_t st) {
  if (d == 64) return launch_d<64>(a, wk, st);
  if (d == 128) return launch_d<128>(a, wk, st);
  return hipErrorInvalidValue;
}

}  // namespace qsa
