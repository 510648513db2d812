// Fused quantized-softmax attention forward, bf16 Q/K/V, gfx950 MFMA.
//
// The fused path follows the wiki summary's flowchart of the method ("QK tile
// -> Row max (anchor point) -> Power-of-two weights -> PV matmul -> Output"),
// laid out for CDNA4:
//
//   * one workgroup = 4 waves = 128 query rows of one (batch, head), two
//     workgroups per CU (two waves per SIMD), or at d = 128 for most kinds
//     8 waves = 256 rows, one workgroup per CU (see fwd_waves); each wave owns
//     32 rows for the whole kernel (its Q^T operand stays in VGPRs);
//   * scores are computed transposed, S^T = K Q^T, on
//     v_mfma_f32_32x32x16_bf16: lane (i, h) of a wave holds query row i and 16
//     keys of each 32-key block, so row maxima are in-lane reductions plus one
//     exchange between the two half-waves;
//   * the accumulator layout of S^T is the B operand of O^T = V^T P^T, so P
//     never moves between lanes; the row sums of P are one more MMA per P
//     operand against a constant 0/1 selector (v_dot2_f32_bf16 stalls the
//     matrix core of its SIMD for several times its issue cost);
//   * anchored kinds get the true row extrema from rowext_bf16, a kernel of
//     its own launched first (64 rows per wave, so each K operand read feeds
//     two MMAs), which parks them in O; the main loop starts each score
//     accumulation at -M, so the MFMA itself delivers s' = acc - M;
//   * the online exact control has no pre-pass and rescales O by
//     2^(m_old - m_new) when a row's running maximum grows;
//   * software pipeline, three tiles deep: iteration t multiplies P(t) (formed
//     in iteration t-1) by the V tile t, forms the weights of tile t+1 (whose
//     scores were issued in iteration t-1) and issues the scores of tile t+2,
//     so the PV MMAs and the score MMAs never wait for this iteration's VALU
//     work and the weights never wait for this iteration's MMAs;
//   * K and V tiles of 64 keys sit in two LDS stages each, unpadded, with the
//     16-byte chunks of each row XOR-swizzled so that the score operand reads
//     (ds_read_b128) and the transposing V reads (ds_read_b64_tr_b16) are free
//     of bank conflicts.  They are filled by buffer loads that write LDS
//     directly (no staging registers; hardware zero-fill past the end of the
//     head), the same number of instructions in every wave, issued right after
//     the iteration's V operand reads (the compiler makes transposing LDS reads
//     wait for every LDS-direct load issued before them);
//   * K-interval grid values come from a per-row table in LDS for K <= 16 (no
//     transcendental per element): T_l for hard rounding, and for
//     interpolation the line of each interval as a function of the raw score,
//     so that one FMA gives the weight; larger K evaluates T_l = 2^(l step)
//     per element.
#include "qsa_common.h"
#include "qsa_mfma_util.h"
#include "qsa_weights.h"

namespace qsa {
namespace {

constexpr int NW = 4;   // waves per workgroup (8 for the kinds fwd_waves names)
constexpr int BN = 64;  // keys per tile
constexpr int NS = 2;   // K and V stages in LDS
constexpr int KTAB_MAX = 16;  // largest K with a per-row grid table in LDS
constexpr int BM = NW * 32;   // query rows per workgroup of NW waves
constexpr int SH = 9;         // log2(BM * 4): the K-interval table's stride between grid values of one row

// Operand reads kept in flight ahead of their MMAs.  A 32-row wave-tile is 36 MMAs of 32 cycles
// each, every one fed by its own LDS read; issued just before its MMA, each read's full latency
// sits on the wave's critical path.  The loops below issue the reads RA_K score k-steps and
// RA_V PV MMAs ahead, and pin that order of LDS reads and MMAs for the scheduler (0: the
// scheduler's own order).  Measured at 8K, 16K GQA and the GPT-2 shape against the scheduler's
// order (bit-identical outputs): PoT and exact anchored 2-3.5 % faster, the single pass 1-3 %,
// the others unchanged; 2 and 2 beat 3 and 2 and 4 and 3.  In the pre-pass (RA_X) 2 ahead
// gains another 0.5-1.5 % on every anchored kind.  (Accumulators in AGPRs, tried alongside,
// cost a v_accvgpr_read per score and measured 2-3 % slower at 8K, 8-23 % on the GPT-2 shape.)
#ifndef QSA_BF16_RA_K
#define QSA_BF16_RA_K 2
#endif
#ifndef QSA_BF16_RA_V
#define QSA_BF16_RA_V 2
#endif
#ifndef QSA_BF16_RA_X
#define QSA_BF16_RA_X QSA_BF16_RA_K
#endif
constexpr int RA_K = QSA_BF16_RA_K;
constexpr int RA_V = QSA_BF16_RA_V;
constexpr int RA_X = QSA_BF16_RA_X;  // the same for the K operands of the row-extrema pre-pass
// Keeps LDS operations and MMAs on their side of this point; VALU, SALU and transcendental
// instructions may still be scheduled across it.
__device__ __forceinline__ void pin_lds_mma() { __builtin_amdgcn_sched_barrier(0x0406); }

// Slot of 16-byte chunk q of K row r is q ^ kswz(r): a ds_read_b128 of the score loop reads
// one chunk of 32 consecutive rows, and the XOR spreads every 16-lane group (and every 8-lane
// group) over distinct bank groups.
template <int D>
__device__ __forceinline__ int kswz_of(int r) {
  return D == 128 ? (r & 15) : ((r & 7) ^ ((r >> 3) & 1));
}
// Slot of 16-byte chunk q of V row r is q ^ vswz(r): a transposing read touches rows 4h + 0..3
// (plus multiples of 8), two chunks per row, and the XOR on the row's low bits puts those rows'
// chunks on distinct bank groups for 8-, 16- and 32-lane groups alike.
template <int D>
__device__ __forceinline__ int vswz_of(int r) {
  return D == 128 ? 4 * (r & 3) : 2 * (r & 3);
}

// Byte layout: NS K stages, then NS V stages (rows of D bf16, no padding), then the table.
template <int D> struct Lay {
  static constexpr int SL = D / 8;             // 16-byte slots per row
  static constexpr int RR = SL * 16;           // bytes per row
  static constexpr int KT = BN * RR, VT = BN * RR;
  static constexpr int V0 = NS * KT;           // first V stage
  static constexpr int TAB = NS * (KT + VT);   // K-interval table
  static constexpr int LW = SL / NW;           // tile-load instructions per wave (64 slots each)
  static_assert(SL % NW == 0, "tiles split evenly over the waves");
};

// Workgroups per CU the register budget is sized for: 3 at d = 64 (at most 168 VGPRs, which
// the d = 64 kernels fit without spills), so that the short, latency-bound rows of small heads
// have three waves per SIMD to interleave; 2 at d = 128 (the O accumulator alone is 64 VGPRs).
template <int D> constexpr int fwd_occ() { return D == 64 ? 3 : 2; }
// Waves per workgroup.  At d = 128 the exact, PoT, single-pass and K-interval kinds run 8 waves
// (256 query rows) and one workgroup per CU: the same two waves per SIMD, but each K or V tile is
// half the load instructions per wave and one LDS copy serves twice the rows, and the kernel
// fits in fewer registers (216-245 VGPRs against 245-256).  Measured at 8K against 4 waves:
// exact online 3.8 % / 2.4 % faster (non-causal / causal), single-pass PoT 3.3 % / 2.3 %, PoT
// 1.4 % / 0.7 %, exact anchored 1.8 % / 0.4 %, interpolation 1.7 % / 0.5 %; hard rounding 0.5-2 %
// once the operand reads ran ahead (before that it measured 0.6-2.5 % slower with 8).  The
// support kinds keep 4, as does d = 64, whose register budget is sized for three 4-wave
// workgroups per CU instead (fwd_occ).
template <int D, int WK> constexpr int fwd_waves() {
  return (D == 128 && (WK == WK_EXACT || WK == WK_EXACT_ANCH || wk_pot(WK) || wk_kint(WK))) ? 8 : NW;
}

template <int D, int WK, bool DUMP, bool TAB, int NWT = NW>
__global__ __launch_bounds__(NWT * 64, NWT == 8 ? 1 : fwd_occ<D>()) void fwd_bf16(FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass needs only the signature (for the launch stub)
  constexpr int KC = D / 16;  // k-steps of the QK product
  constexpr int DB = D / 32;  // 32-column blocks of O^T
  using LY = Lay<D>;
  constexpr int SHK = NWT == 8 ? SH + 1 : SH;  // K-interval table stride shift for NWT * 32 rows
  constexpr int SL = LY::SL, RR = LY::RR, KT = LY::KT, VT = LY::VT, LW = SL / NWT;
  constexpr bool RUN = wk_running(WK);             // single-pass PoT: running integer anchor
  constexpr bool ANCH = (WK != WK_EXACT) && !RUN;  // row extrema from the pre-pass
  constexpr bool EXACT_W = (WK == WK_EXACT || WK == WK_EXACT_ANCH);
  constexpr bool POT = wk_pot(WK);
  constexpr bool KHARD = (WK == WK_KH || WK == WK_KH_FLUSH);
  constexpr bool INTERP = (WK == WK_KI || WK == WK_KI_FLUSH);
  constexpr bool SUPPORT = wk_support(WK), UNIF = (WK == WK_UNIF);
  constexpr bool FLUSH = (WK == WK_POT_FLUSH || WK == WK_POTR_FLUSH || WK == WK_KH_FLUSH || WK == WK_KI_FLUSH);

  extern __shared__ __align__(16) unsigned char smem[];
  lds_u8* const lds = (lds_u8*)smem;
  unsigned char* const Tb = smem + LY::TAB;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hh = lane >> 5;
  int bh, qt;
  map_block(a, bh, qt);
  const int b = bh / a.H, h = bh - b * a.H;
  const int kvh = h / (a.H / a.Hkv);
  const int N = a.N;
  const int q0 = qt * (NWT * 32);
  const int wr0 = q0 + wave * 32;
  const int row = wr0 + li;
  const int lim = a.causal ? min(row, N - 1) : N - 1;  // last key visible to this lane's row
  const __bf16* Qg = (const __bf16*)a.q + (size_t)(b * a.H + h) * N * D;
  const size_t kv_off = (size_t)(b * a.Hkv + kvh) * N * D;
  const __bf16* const Kg = (const __bf16*)a.k + kv_off;
  const __bf16* const Vg = (const __bf16*)a.v + kv_off;

  // Q^T operand: lane (li, hh) holds Q[row][16c + 8hh .. +7] (rows past N: 0)
  u32x4 qf[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c)
    qf[c] = row < N ? *(const u32x4*)(Qg + (size_t)row * D + 16 * c + 8 * hh) : u32x4{0, 0, 0, 0};

  const int T = a.causal ? ((min(q0 + (NWT * 32), N) - 1) / BN + 1) : (N + BN - 1) / BN;  // tiles of this workgroup
  // last tile this wave computes (-1: none); only that tile can need masking
  const int wlast = wr0 >= N ? -1 : (a.causal ? (min(wr0 + 31, N - 1) / BN) : T - 1);
  const bool last_masked = (a.causal && wlast * BN + BN - 1 > wr0) || (wlast * BN + BN > N);
  const int tclean = last_masked ? wlast : wlast + 1;  // tiles t < tclean need no mask

  // ---- tile staging: buffer loads straight into LDS ------------------------------------------
  // Instruction m of a wave writes the 64 consecutive 16-byte slots (wave + NWT m) * 64 + lane:
  // slot s of a tile is row j = s / SL, position s % SL of the row, which holds chunk
  // (s % SL) ^ swz(j).  The per-tile buffer resource starts at the tile and ends at the end of
  // the head, so rows past N read as zero.
  // Instruction m covers rows 64 NWT m / SL further on than instruction 0 (a multiple of 16), the
  // same position in the row and the same swizzle (which reads row bits below 4): its global
  // offset is instruction 0's plus m * 64 NWT * 16 bytes, taken as the scalar offset.
  uint32_t kvo, vvo;
  {
    const int sl = wave * 64 + lane, j = sl / SL, c = sl % SL;
    kvo = (uint32_t)(j * D + 8 * (c ^ kswz_of<D>(j))) * 2;
    vvo = (uint32_t)(j * D + 8 * (c ^ vswz_of<D>(j))) * 2;
  }
  static_assert((NWT * 64 / SL) % 16 == 0, "the swizzles repeat every 16 rows");
  auto tile_rsrc = [&](const __bf16* base, int kt) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (size_t)kt * BN * D), 0, (N - kt * BN) * D * 2,
                                             0x00020000);
  };
  auto load_k = [&](int kt, int st) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(Kg, kt);
#pragma unroll
    for (int m = 0; m < LW; ++m)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(lds + st * KT + (wave + NWT * m) * 1024), 16, kvo,
          m * NWT * 64 * 16, 0, 0);
  };
  auto load_v = [&](int kt, int st) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(Vg, kt);
#pragma unroll
    for (int m = 0; m < LW; ++m)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(lds + LY::V0 + st * VT + (wave + NWT * m) * 1024), 16, vvo,
          m * NWT * 64 * 16, 0, 0);
  };
  auto loads_done = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // QK A-operand for k-step c: lane (li, hh) reads chunk 2c + hh of K row li (keys of the block)
  uint32_t koff[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) koff[c] = li * RR + 16 * ((2 * c + hh) ^ kswz_of<D>(li));
  // V^T operand: in each 16-lane group g, lane 4q + p points at V[key 4hh + q][4p .. 4p+3] of the
  // group's 16 columns (column block db, half g & 1): chunk 4db + 2(g & 1) + p/2 of the row,
  // at its swizzled slot; the transposing read hands lane l column l and keys q = 0..3.  The
  // row offsets 16(2kb + kc) and 8 keep the row's low bits, so the swizzle is per lane.
  const int vq = (lane & 15) >> 2, vg1 = (lane >> 4) & 1, vp = lane & 3;
  uint32_t vtr[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
    vtr[db] = (4 * hh + vq) * RR + 16 * ((4 * db + 2 * vg1 + (vp >> 1)) ^ vswz_of<D>(vq)) + 8 * (vp & 1);

  // 32-key block kb of the K tile in stage st: init + K_block Q^T  (init: the -M vector, or 0)
  // The operand of k-step c + RA_K is read while the MMA of k-step c runs (pinned order).
  auto qk1 = [&](int st, int kb, const f32x16& init) __attribute__((always_inline)) {
    const lds_u8* kbase = lds + st * KT + kb * 32 * RR;
    f32x16 s = init;
    if constexpr (RA_K == 0) {
#pragma unroll
      for (int c = 0; c < KC; ++c) s = mma(*(const lds_u32x4*)(kbase + koff[c]), qf[c], c == 0 ? init : s);
    } else {
      u32x4 kr[KC];
#pragma unroll
      for (int c = 0; c < RA_K && c < KC; ++c) kr[c] = *(const lds_u32x4*)(kbase + koff[c]);
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        if (c + RA_K < KC) kr[c + RA_K] = *(const lds_u32x4*)(kbase + koff[c + RA_K]);
        s = mma(kr[c], qf[c], c == 0 ? init : s);
        pin_lds_mma();
      }
    }
    return s;
  };

  // Row sums on the matrix core: v_mfma_f32_16x16x32_bf16 with A a constant 0/1 selector and B
  // a P^T operand as it is.  In the 16x16x32 layout lane l holds B rows (keys) 8(l/16)..+7 of
  // column l % 16; in the P^T operand the same lane holds 8 keys of query row l % 32.  The
  // selector's rows 0-7 take the k-groups 0 and 2 (query n = l % 16, both key halves) and rows
  // 8-15 the k-groups 1 and 3 (query n + 16), so C[m][n] accumulates the row sum of query n
  // (m < 8) or n + 16 (m >= 8): lane l holds the sum of query q(l) = l, l - 16, l - 16, l - 32
  // for its four 16-lane groups.
  const uint32_t rsel = (((lane & 15) < 8) == (((lane >> 4) & 1) == 0)) ? 0x3F803F80u : 0u;  // bf16 1.0 pairs
  const u32x4 rs_sel = {rsel, rsel, rsel, rsel};
  const int rs_q = lane < 16 ? lane : (lane < 48 ? lane - 16 : lane - 32);

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  f32x4 rs = {0.0f, 0.0f, 0.0f, 0.0f};
  u32x4 P[2][2];  // weights of the tile PV multiplies next: [kb][kc]
  // O^T += V^T P^T over the V tile in stage st (two transposing reads per operand), and the row sums
  // (MMA i = (2 kb + kc) DB + db; the operand of MMA i + RA_V is read while MMA i runs)
  auto pv = [&](int st) __attribute__((always_inline)) {
    const lds_u8* vbase = lds + LY::V0 + st * VT;
    auto vread = [&](int i) __attribute__((always_inline)) {
      const lds_u8* pa = vbase + (16 * (i / DB)) * RR + vtr[i % DB];
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)pa);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(pa + 8 * RR));
      return u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                   __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]};
    };
    constexpr int NV = 4 * DB;  // PV MMAs per tile
    if constexpr (RA_V == 0) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int kb = i / (2 * DB), kc = (i / DB) & 1, db = i % DB;
        o[db] = mma(vread(i), P[kb][kc], o[db]);
        if (db == DB - 1) rs = mma16(rs_sel, P[kb][kc], rs);
      }
    } else {
      u32x4 va[NV];
#pragma unroll
      for (int i = 0; i < RA_V && i < NV; ++i) va[i] = vread(i);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int kb = i / (2 * DB), kc = (i / DB) & 1, db = i % DB;
        if (i + RA_V < NV) va[i + RA_V] = vread(i + RA_V);
        o[db] = mma(va[i], P[kb][kc], o[db]);
        if (db == DB - 1) rs = mma16(rs_sel, P[kb][kc], rs);
        pin_lds_mma();
      }
    }
  };

  // ---- row extrema of the anchored kinds ----------------------------------------------------
  // rowext_bf16 parked them as raw accumulator values, 8 bytes per row packed at the start of
  // the wave's own 32 rows of O (a contiguous 256-byte run), which this wave later overwrites
  float M = -__builtin_inff(), MN = __builtin_inff();
  if (ANCH) {
    const uint32_t* const park = (const uint32_t*)((const __bf16*)a.o + ((size_t)bh * N + wr0) * D) + 2 * li;
    M = row < N ? bitsf(park[0]) : 0.0f;
    MN = row < N ? bitsf(park[1]) : 0.0f;
  }
  // hard rounding: T_l per row; interpolation: the line (A_l, B_l) of each interval per row
  RowC rc = make_row<WK, SHK, INTERP ? TAB_SLOPE : TAB_T>(a, M, MN, wave * 32 + li, TAB ? Tb : nullptr, hh, 2);
  // main-loop score accumulators start at -M: s' = acc - M
  f32x16 init;
#pragma unroll
  for (int r = 0; r < 16; ++r) init[r] = ANCH ? -M : 0.0f;

  // PoT rounds t = G - y to an integer in one FMA, G = 2^24 (pre-pass kinds: scores start at
  // -M, so t = 2^24 + acc' c) or G = 1.5 * 2^23 (single pass: t = (G - A) + acc c, and G - A
  // must be exact in fp32 for a negative integer anchor A too, which 2^24 - A is not).  In
  // both cases t lies in [2^23, 2^24), bits(t) = bits(G) - e, and the low 16 bits are -e.
  constexpr int32_t pot_bits = RUN ? 0x4B400000 : 0x4B800000;  // bits of G
  constexpr float pot_g = RUN ? 12582912.0f : 16777216.0f;      // G
  const int L = a.levels;
  const float Kf = (float)a.levels;
  const float kt_hi = 8388608.0f + Kf;  // 2^23 + K: the clamp of the rounded K-interval coordinate
  int32_t pot_lo = pot_bits - (L - 1);  // bits of G - (L-1): the clip e <= L-1
  // Single-pass PoT: A = ceil(running max of s log2 e), an integer.  The weights are formed
  // against a lagging integer anchor Aw <= A (tb = G - Aw) with the clip moved by the lag
  // dl = A - Aw (pot_lo = bits(G) - (L-1) + dl), so every weight carries the same factor 2^dl
  // relative to A while Aw stays; O and the row sums are rescaled only when Aw moves, on the
  // first tile and when the lag would pass 32 (bf16 weights up to 2^32 and their sums stay well
  // inside the exponent range).
  float A = -__builtin_inff(), Aw = -__builtin_inff();
  int dlag = 0;
  float tb = pot_g;
  // pre-pass PoT without flush at d = 64: t = 1 - ((L-1) - y) 2^-24 from one FMA whose output
  // clamp is the clip (pot_t_clamped), one VALU instruction per element fewer than the integer
  // max.  Measured 2.7 % faster per call at d = 64 (GPT-2 shape) and 0.6-0.8 % slower at
  // d = 128, where the integer max stays.
  constexpr bool POT_CLAMP = POT && !FLUSH && !RUN && D == 64;
  // With flush the clamp sits at L (pot_bf = 1 - L 2^-24): k = L - e, and k = 0 is the flushed
  // level.  The low half of bits(t) is then -k: 0 for the flushed level, at least 2^16 - 64
  // otherwise, so min_u16((-k)(-128) + (127 - L) 128, -k) is the weight (127 - e) << 7, or 0.
  constexpr bool POT_CLAMP_FLUSH = POT && FLUSH && !RUN;
  const float pot_bf = 1.0f - (float)L * 5.9604644775390625e-8f;        // 1 - L 2^-24
  const uint32_t pot_kaddf = 0x00010001u * (uint32_t)((127 - L) << 7);
  const float pot_nc = -rc.c * 5.9604644775390625e-8f;                  // -c 2^-24
  const float pot_b = 1.0f - (float)(L - 1) * 5.9604644775390625e-8f;   // 1 - (L-1) 2^-24
  const uint32_t pot_kadd = 0x00010001u * (uint32_t)((128 - L) << 7);

  // scale the row sums by each row's factor (held by the lane of that row)
  auto rs_scale = [&](float alpha) { rs *= bitsf(__builtin_amdgcn_ds_bpermute(4 * rs_q, (int)fbits(alpha))); };
  // the tile's maximum of this lane's row (masked: visible keys only), both half-waves combined
  auto tile_max = [&](const f32x16 (&s)[2], bool masked, int kt) __attribute__((always_inline)) {
    float tm = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        tm = fmaxf(tm, (!masked || kt * BN + kb * 32 + acc_key(r, hh) <= lim) ? s[kb][r] : -__builtin_inff());
    return half_max(tm);
  };
  // online exact: grow the running max over a tile, rescale O and the row sums
  auto online_max = [&](const f32x16 (&s)[2], bool masked, int kt) __attribute__((always_inline)) {
    const float mnew = fmaxf(M, tile_max(s, masked, kt));
    if (__builtin_amdgcn_ballot_w64(mnew > M)) {
      const float alpha = mnew > M ? __builtin_amdgcn_exp2f((M - mnew) * rc.c) : 1.0f;
      rs_scale(alpha);
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      M = mnew;
      rc.mc = mnew * rc.c;
    }
  };
  // single-pass PoT: fold a tile's maximum into the anchor before its weights are formed; when
  // the weight anchor Aw has to move, O and the row sums, formed against the old Aw, are scaled
  // by 2^(Aw_old - Aw) (exact)
  auto run_anchor = [&](const f32x16 (&s)[2], bool masked, int kt) __attribute__((always_inline)) {
    const float An = fmaxf(A, __builtin_ceilf(tile_max(s, masked, kt) * rc.c));
    if (__builtin_amdgcn_ballot_w64(An - Aw > 32.0f)) {  // Aw = -inf before the first tile
      const bool move = An - Aw > 32.0f;
      const float alpha = move ? (Aw > -__builtin_inff() ? __builtin_ldexpf(1.0f, (int)(Aw - An)) : 0.0f) : 1.0f;
      rs_scale(alpha);
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      Aw = move ? An : Aw;
      tb = pot_g - Aw;
    }
    A = An;
    dlag = (int)(A - Aw);
    pot_lo = pot_bits - (L - 1) + dlag;
  };

  // weights of 32-key block kb of tile kt -> the two P^T operands P[kb] (bf16)
  auto weights = [&](const f32x16& sb, int kb, int kt, bool masked) __attribute__((always_inline)) {
#pragma unroll
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
          // truncation / uniform weighting: keys with y = (M - acc) c > W log2 e are outside the
          // support; inside, exp(s - m) or 1
          const float y0 = -x0 * rc.c, y1 = -x1 * rc.c;
          const float e0 = UNIF ? 1.0f : __builtin_amdgcn_exp2f(x0 * rc.c);
          const float e1 = UNIF ? 1.0f : __builtin_amdgcn_exp2f(x1 * rc.c);
          pk = pack_bf16(y0 > rc.cut ? 0.0f : e0, y1 > rc.cut ? 0.0f : e1);
          if (DUMP) {
            i0 = y0 > rc.cut ? 254u : 0u;
            i1 = y1 > rc.cut ? 254u : 0u;
          }
        } else if (POT_CLAMP) {
          pk = pot_pair_k(pot_t_clamped(x0, pot_nc, pot_b), pot_t_clamped(x1, pot_nc, pot_b), pot_kadd);
          if (DUMP) {
            i0 = 127u - ((pk >> 7) & 0x1FFu);
            i1 = 127u - ((pk >> 23) & 0x1FFu);
          }
        } else if (POT && !FLUSH) {
          // t = G + (acc - M) c = G - y, rounded to an integer by the FMA itself
          const float t0 = fmaf(x0, rc.c, tb), t1 = fmaf(x1, rc.c, tb);
          pk = pot_pair(t0, t1, pot_lo);
          if (DUMP) {
            i0 = 127u - ((pk >> 7) & 0x1FFu) + (uint32_t)dlag;  // against the running anchor
            i1 = 127u - ((pk >> 23) & 0x1FFu) + (uint32_t)dlag;
          }
        } else if (POT_CLAMP_FLUSH) {
          const uint32_t nk = __builtin_amdgcn_perm(fbits(pot_t_clamped(x1, pot_nc, pot_bf)),
                                                    fbits(pot_t_clamped(x0, pot_nc, pot_bf)), 0x05040100u);
          uint32_t w;
          asm("v_pk_mad_u16 %0, %1, %2, %3" : "=v"(w) : "v"(nk), "v"(0xFF80FF80u), "v"(pot_kaddf));
          pk = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, w),
                                                                      __builtin_bit_cast(u16x2, nk)));
          if (DUMP) {  // e = L - k; k = 0 is flushed
            i0 = (nk & 0xFFFFu) == 0 ? 254u : (uint32_t)L - (0x10000u - (nk & 0xFFFFu));
            i1 = (nk >> 16) == 0 ? 254u : (uint32_t)L - (0x10000u - (nk >> 16));
          }
        } else if (POT) {  // flush: e >= L -> 0
          const float t0 = fmaf(x0, rc.c, tb), t1 = fmaf(x1, rc.c, tb);
          const int32_t b0 = (int32_t)fbits(t0), b1 = (int32_t)fbits(t1);
          const uint32_t w0 = b0 < pot_lo ? 0u : (((uint32_t)b0 << 23) + (127u << 23));
          const uint32_t w1 = b1 < pot_lo ? 0u : (((uint32_t)b1 << 23) + (127u << 23));
          pk = __builtin_amdgcn_perm(w1, w0, 0x07060302u);
          if (DUMP) {
            i0 = b0 < pot_lo ? 254u : (uint32_t)(pot_bits - b0 + dlag);
            i1 = b1 < pot_lo ? 254u : (uint32_t)(pot_bits - b1 + dlag);
          }
        } else if (KHARD) {
          // y = (M - acc) c; t = y + 2^23 rounds y: bits(t) = 0x4B000000 + l, clamped to [0, K]
          // by one v_med3_f32 on t (on [2^23, 2^23 + K] the floats order as their bit patterns;
          // the lower clamp keeps the table read inside the row's column when rounding puts
          // acc a little above M on a very narrow grid)
          const float t0 = fmaf(x0, -rc.c, 8388608.0f), t1 = fmaf(x1, -rc.c, 8388608.0f);
          const int32_t b0 = (int32_t)fbits(__builtin_amdgcn_fmed3f(t0, 8388608.0f, kt_hi));
          const int32_t b1 = (int32_t)fbits(__builtin_amdgcn_fmed3f(t1, 8388608.0f, kt_hi));
          float w0, w1;
          if (TAB) {  // T_l from the row's column of the table: (bits << SHK) drops 0x4B000000
            w0 = *(const float*)(Tb + (((uint32_t)b0 << SHK) + rc.tab));
            w1 = *(const float*)(Tb + (((uint32_t)b1 << SHK) + rc.tab));
          } else {
            w0 = __builtin_amdgcn_exp2f(rc.step * (float)(b0 - 0x4B000000));
            w1 = __builtin_amdgcn_exp2f(rc.step * (float)(b1 - 0x4B000000));
          }
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
        } else if (TAB) {  // K-interval, interpolation between T_l and T_l+1, l = floor(min(y, K))
          // t = y + 2^23 - 1/2 rounded by the FMA: for y >= 1/2 the low bits of t hold floor(y)
          // (at an integer y either neighbour, where the weight is continuous); one v_med3_f32
          // clamps t to [2^23, 2^23 + K], whose floats order as their bit patterns, so
          // bits(t) - 0x4B000000 = l in [0, K].  The table's line of interval l then gives the
          // weight from the raw score in one FMA (flushing kind: entry K is 0).
          const float t0 = fmaf(x0, -rc.c, 8388607.5f), t1 = fmaf(x1, -rc.c, 8388607.5f);
          const uint32_t b0 = fbits(__builtin_amdgcn_fmed3f(t0, 8388608.0f, kt_hi));
          const uint32_t b1 = fbits(__builtin_amdgcn_fmed3f(t1, 8388608.0f, kt_hi));
          typedef float f2 __attribute__((ext_vector_type(2)));
          // (b << (SHK + 1)) drops 0x4B000000: the table's stride is 2^(SHK+1) bytes per l
          const f2 e0 = *(const f2*)(Tb + ((b0 << (SHK + 1)) + rc.tab));
          const f2 e1 = *(const f2*)(Tb + ((b1 << (SHK + 1)) + rc.tab));
          pk = pack_bf16(fmaf(x0, e0.y, e0.x), fmaf(x1, e1.y, e1.x));
          if (DUMP) {
            const uint32_t l0 = b0 - 0x4B000000u, l1 = b1 - 0x4B000000u;
            i0 = (FLUSH && l0 == (uint32_t)a.levels) ? 254u : l0;
            i1 = (FLUSH && l1 == (uint32_t)a.levels) ? 254u : l1;
          }
        } else {  // interpolation for K > 16: T_l and T_l+1 evaluated per element
          const float y0 = -x0 * rc.c, y1 = -x1 * rc.c;
          const float c0 = __builtin_amdgcn_fmed3f(y0, 0.0f, Kf), c1 = __builtin_amdgcn_fmed3f(y1, 0.0f, Kf);
          const float f0 = __builtin_floorf(c0), f1 = __builtin_floorf(c1);
          const uint32_t l0 = (uint32_t)(int32_t)f0, l1 = (uint32_t)(int32_t)f1;
          typedef float f2 __attribute__((ext_vector_type(2)));
          const f2 e0 = kgrid_pair(rc.step, f0), e1 = kgrid_pair(rc.step, f1);  // (T_l, T_l+1 - T_l)
          float w0 = fmaf(c0 - f0, e0.y, e0.x);
          float w1 = fmaf(c1 - f1, e1.y, e1.x);
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
        P[kb][kc][p] = pk;
      }
  };
  // a tile's scores are weighed: the running maximum first (online kinds), then both blocks
  auto fold_max = [&](const f32x16 (&s)[2], int kt, bool masked) __attribute__((always_inline)) {
    if (WK == WK_EXACT) online_max(s, masked, kt);
    if (RUN) run_anchor(s, masked, kt);
  };
  auto weigh_tile = [&](const f32x16 (&s)[2], int kt, bool masked) __attribute__((always_inline)) {
    fold_max(s, kt, masked);
    weights(s[0], 0, kt, masked);
    weights(s[1], 1, kt, masked);
  };

  // ---- prologue -----------------------------------------------------------------------------
  // K(j) sits in K stage j % 2, V(j) in V stage j % 2.  Iteration t multiplies P(t) by V(t),
  // forms P(t+1) from the scores of tile t+1 and issues the scores of tile t+2; it loads V(t+1)
  // and K(t+3) into the stages of V(t-1) and K(t+1), both last read in iteration t-1.
  load_k(0, 0);
  load_k(min(1, T - 1), 1);
  load_v(0, 0);
  loads_done();
  __syncthreads();  // also publishes the K-interval tables
  f32x16 sc[2];  // the scores of tile t+1 during iteration t
  {
    f32x16 s0[2];
    if (wlast >= 0) {
      s0[0] = qk1(0, 0, init);
      s0[1] = qk1(0, 1, init);
    }
    if (wlast >= 1) {
      sc[0] = qk1(1, 0, init);
      sc[1] = qk1(1, 1, init);
    }
    __syncthreads();  // every wave has read K(0) before its stage is refilled
    load_k(min(2, T - 1), 0);
    if (wlast >= 0) weigh_tile(s0, 0, wlast == 0 && last_masked);
    loads_done();
    lds_barrier();
  }

  // ---- main loop ----------------------------------------------------------------------------
  // Every iteration issues the same loads, so the loop needs no branch for them: past the last
  // tile it reloads tile T-1 into a stage no later iteration reads.
  int t = 0;
  auto loads = [&]() __attribute__((always_inline)) {
    load_v(min(t + 1, T - 1), (t + 1) & 1);
    load_k(min(t + 3, T - 1), (t + 1) & 1);
  };
  // (the index dump's stores count in vmcnt as well: the wait covers them)
  auto end_iteration = [&]() __attribute__((always_inline)) {
    loads_done();
    lds_barrier();
  };
  // steady state: tiles t+1 and t+2 hold visible keys for every row and need no mask
  // (unrolling this loop by two so that the two sets of block 0 swap roles instead of being
  // copied saves 16 of 124 VALU instructions per wave-tile and measured 1-2 % slower)
  for (; t + 2 <= wlast && t + 1 < tclean; ++t) {
    pv(t & 1);
    loads();
    if constexpr (WK == WK_EXACT || RUN) {
      // the online kinds (a running maximum, a rare rescale branch) weigh tile t+1 before they
      // issue the scores of tile t+2 into the same registers: one score set live, not two
      weigh_tile(sc, t + 1, false);
      sc[0] = qk1(t & 1, 0, init);  // K(t+2) is in stage (t+2) % 2
      sc[1] = qk1(t & 1, 1, init);
    } else {
      const f32x16 n0 = qk1(t & 1, 0, init);
      weights(sc[0], 0, t + 1, false);
      weights(sc[1], 1, t + 1, false);
      const f32x16 n1 = qk1(t & 1, 1, init);
      sc[0] = n0;
      sc[1] = n1;
    }
    end_iteration();
  }
  // the last tiles of the wave (the last may need masking), then the iterations in which the
  // wave only issues its share of the other waves' tile loads
  for (; t < T; ++t) {
    if (t <= wlast) pv(t & 1);
    loads();
    if (t + 1 <= wlast) weigh_tile(sc, t + 1, t + 1 >= tclean);
    if (t + 2 <= wlast) {  // (the scores of tile t+2 reuse the registers of tile t+1's)
      sc[0] = qk1(t & 1, 0, init);
      sc[1] = qk1(t & 1, 1, init);
    }
    end_iteration();
  }

  // ---- epilogue -----------------------------------------------------------------------------
  if (wlast < 0) return;
  // the selector MMA left the sum of query n (n + 16) in lane n (n + 32), register 0
  const float lt = bitsf(__builtin_amdgcn_ds_bpermute(4 * (li < 16 ? li : li + 16), (int)fbits(rs[0])));
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

// ---- row-extrema pre-pass ---------------------------------------------------------------
// The row maximum (and minimum) over the visible keys of every query row, from the same MMAs
// in the same order as the main kernel's score tiles (zero-initialised).  A wave owns XRB
// blocks of 32 rows: with two, every K operand read from LDS feeds two MMAs; with one, a
// workgroup covers half the rows, so a small grid has twice the workgroups and its longest
// (causal, last) row block half the serial MMA chain.  The scores of tile t+1 are issued
// before the extrema of tile t are folded.  The extrema are parked in O where fwd_bf16 reads
// them.
constexpr int XNW = 4;  // waves per workgroup
constexpr int XNB = 2;  // K tile buffers
constexpr int xbm(int xrb) { return XNW * 32 * xrb; }  // query rows per workgroup

template <int D, bool TMIN, int XRB>
__global__ __launch_bounds__(XNW * 64, 2) void rowext_bf16(FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int KC = D / 16, XBM = xbm(XRB);
  using LY = Lay<D>;
  constexpr int SL = LY::SL, RR = LY::RR, KT = LY::KT;
  constexpr int KIW = SL / XNW;  // K-tile load instructions per wave
  static_assert(SL % XNW == 0, "K tiles split evenly over the waves");

  extern __shared__ __align__(16) unsigned char smem[];
  lds_u8* const lds = (lds_u8*)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hh = lane >> 5;
  int bh, qt;
  map_block(a, bh, qt);
  const int b = bh / a.H, h = bh - b * a.H;
  const int kvh = h / (a.H / a.Hkv);
  const int N = a.N;
  const int q0 = qt * XBM;
  const int wr0 = q0 + wave * 32 * XRB;
  const __bf16* Qg = (const __bf16*)a.q + (size_t)(b * a.H + h) * N * D;
  const __bf16* const Kg = (const __bf16*)a.k + (size_t)(b * a.Hkv + kvh) * N * D;

  u32x4 qf[XRB][KC];
#pragma unroll
  for (int rb = 0; rb < XRB; ++rb) {
    const int row = wr0 + 32 * rb + li;
#pragma unroll
    for (int c = 0; c < KC; ++c)
      qf[rb][c] = row < N ? *(const u32x4*)(Qg + (size_t)row * D + 16 * c + 8 * hh) : u32x4{0, 0, 0, 0};
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
  int wlast = last[0];
#pragma unroll
  for (int rb = 1; rb < XRB; ++rb) wlast = max(wlast, last[rb]);

  // K tiles as in fwd_bf16: slot s (64 per wave instruction) is row j = s / SL, position
  // s % SL of the row, which holds chunk (s % SL) ^ kswz(j)
  uint32_t kvo[KIW];
#pragma unroll
  for (int m = 0; m < KIW; ++m) {
    const int sl = (wave + XNW * m) * 64 + lane, j = sl / SL, c = sl % SL;
    kvo[m] = (uint32_t)(j * D + 8 * (c ^ kswz_of<D>(j))) * 2;
  }
  auto load_k = [&](int kt, int buf) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Kg + (size_t)kt * BN * D), 0, (N - kt * BN) * D * 2, 0x00020000);
#pragma unroll
    for (int m = 0; m < KIW; ++m)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(lds + buf * KT + (wave + XNW * m) * 1024), 16, kvo[m], 0, 0, 0);
  };

  uint32_t koff[KC];  // chunk 2c + hh of K row li at its swizzled slot
#pragma unroll
  for (int c = 0; c < KC; ++c) koff[c] = li * RR + 16 * ((2 * c + hh) ^ kswz_of<D>(li));
  const f32x16 zero16 = {};
  // scores of tile buf for both row blocks: s[rb][kb] = 32 keys kb x 32 rows rb (S^T)
  // (operand j = KC kb + c; as in fwd_bf16, the operand of j + RA_X is read while j's MMAs run)
  auto qk = [&](int buf, f32x16 (&s)[XRB][2]) {
    auto kread = [&](int j) __attribute__((always_inline)) {
      return *(const lds_u32x4*)(lds + buf * KT + (j / KC) * 32 * RR + koff[j % KC]);
    };
    if constexpr (RA_X == 0) {
#pragma unroll
      for (int j = 0; j < 2 * KC; ++j) {
        const int kb = j / KC, c = j % KC;
        const u32x4 ka = kread(j);
#pragma unroll
        for (int rb = 0; rb < XRB; ++rb) s[rb][kb] = mma(ka, qf[rb][c], c == 0 ? zero16 : s[rb][kb]);
      }
    } else {
      u32x4 kr[2 * KC];
#pragma unroll
      for (int j = 0; j < RA_X; ++j) kr[j] = kread(j);
#pragma unroll
      for (int j = 0; j < 2 * KC; ++j) {
        const int kb = j / KC, c = j % KC;
        if (j + RA_X < 2 * KC) kr[j + RA_X] = kread(j + RA_X);
#pragma unroll
        for (int rb = 0; rb < XRB; ++rb) s[rb][kb] = mma(kr[j], qf[rb][c], c == 0 ? zero16 : s[rb][kb]);
        pin_lds_mma();
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
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // K(t+2), this iteration's load
    __syncthreads();
    kl = kn;
    kn = kn + 1 == XNB ? 0 : kn + 1;
  };
  // steady state: tile t is unmasked for both row blocks and tile t+1 is needed.  Unrolled by
  // two so that the score sets swap roles instead of being copied.
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
    // packed at the start of the 32-row block's slice of O, where fwd_bf16 reads them
    uint32_t* const park = (uint32_t*)((__bf16*)a.o + ((size_t)bh * N + r0) * D) + 2 * li;
    if (hh == 0 && r0 + li < N) {
      park[0] = fbits(m);
      park[1] = fbits(mn);
    }
  }
#endif
}

template <int D, int WK, bool TAB>
hipError_t launch_main(const FwdArgs& a, hipStream_t st) {
  constexpr int NWK = fwd_waves<D, WK>();
  // hard rounding: T_l (4 bytes a row and level); interpolation: the interval lines (8 bytes)
  const size_t lds = (size_t)Lay<D>::TAB + (TAB ? table_bytes(WK, NWK * 32, a.levels) : 0);
  FwdArgs g = a;  // query tiles of NWK * 32 rows
  g.n_qtiles = (a.N + NWK * 32 - 1) / (NWK * 32);
  g.total_blocks = a.B * a.H * g.n_qtiles;
  const void* kern = a.grid_idx ? (const void*)fwd_bf16<D, WK, true, TAB, NWK> : (const void*)fwd_bf16<D, WK, false, TAB, NWK>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  if (a.grid_idx)
    hipLaunchKernelGGL((fwd_bf16<D, WK, true, TAB, NWK>), dim3(g.total_blocks), dim3(NWK * 64), lds, st, g);
  else
    hipLaunchKernelGGL((fwd_bf16<D, WK, false, TAB, NWK>), dim3(g.total_blocks), dim3(NWK * 64), lds, st, g);
  return hipGetLastError();
}

template <int D, int WK>
hipError_t launch_one(const FwdArgs& a0, hipStream_t st) {
  FwdArgs a = a0;
  a.n_qtiles = (a.N + BM - 1) / BM;
  a.total_blocks = a.B * a.H * a.n_qtiles;
  constexpr bool ANCH = WK != WK_EXACT && !wk_running(WK);
  if constexpr (ANCH) {  // the row-extrema pre-pass, on its own workgroup grid
    // two row blocks per wave unless that leaves fewer workgroups than two per CU
    FwdArgs x = a0;
    const int q2 = (x.N + xbm(2) - 1) / xbm(2);
    const bool one = (long)x.B * x.H * q2 < 512;
    x.n_qtiles = one ? (x.N + xbm(1) - 1) / xbm(1) : q2;
    x.total_blocks = x.B * x.H * x.n_qtiles;
    const size_t xl = (size_t)XNB * Lay<D>::KT;  // K tile buffers only
    const dim3 g(x.total_blocks), t(XNW * 64);
    if (x.track_min) {
      if (one) hipLaunchKernelGGL((rowext_bf16<D, true, 1>), g, t, xl, st, x);
      else hipLaunchKernelGGL((rowext_bf16<D, true, 2>), g, t, xl, st, x);
    } else {
      if (one) hipLaunchKernelGGL((rowext_bf16<D, false, 1>), g, t, xl, st, x);
      else hipLaunchKernelGGL((rowext_bf16<D, false, 2>), g, t, xl, st, x);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // K-interval grid values: from a per-row table in LDS while it fits (K <= 16), else evaluated
  // per element as 2^(l step) (one v_exp_f32, two for interpolation)
  if constexpr (wk_kint(WK)) {
    if (a.levels <= KTAB_MAX) return launch_main<D, WK, true>(a, st);
  }
  return launch_main<D, WK, false>(a, st);
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
