/*
 * qsa.h -- C ABI of libqsa, the quantized-softmax attention forward (and its
 * backward) for AMD Instinct MI355X (gfx950).
 *
 * The main operation: the fused attention forward
 *
 *     O = softmax~(scale * Q K^T) V
 *
 * in which the exponential inside softmax is either exact (the control) or
 * replaced by a coarse grid anchored at each row's maximum:
 *
 *   - K-interval attention: the exponential is read off K+1 grid values
 *     fitted to each row of scores, with per-row min-max or fixed-window
 *     calibration and hard rounding or interpolation ("Pretraining
 *     Transformers with Quantized Softmax in Attention", abstract; chapter 1
 *     "The problem"; chapter 5 "Build the method").
 *   - Rowmax-PoT: power-of-two weights 2^-e, e = rint((m - s) log2 e) clipped
 *     to L levels, anchored at each row maximum ("Approximating Softmax in
 *     Pretrained LLMs: Model Sensitivity and Kernel Acceleration", abstract;
 *     the wiki summary's flowchart: QK tile -> row max -> power-of-two
 *     weights -> PV matmul -> output).
 *
 * Notation: s_ij = scale * q_i . k_j; m_i and mn_i are the maximum and the
 * minimum of s_ij over the keys visible to row i (causal: j <= i, top-left
 * aligned; otherwise all j).  O_i = sum_j w_ij v_j / sum_j w_ij.
 *
 * Conventions shared by every entry point
 *   Layout    Q and O are [B, H, N, d], K and V are [B, Hkv, N, d], all
 *             contiguous with d innermost.  Query head h reads KV head
 *             h / (H / Hkv) (grouped-query attention when Hkv < H).
 *   Types     dtype QSA_DT_F32: Q, K, V and O are float32.
 *             dtype QSA_DT_BF16: Q, K, V and O are bfloat16.
 *             dtype QSA_DT_FP8_E4M3: Q, K, V are OCP FP8 E4M3 ("fn": no
 *             infinities, max 448) with per-tensor descales (see
 *             qsa_fwd_ex_opts); O is bfloat16.
 *   Pointers  Q, K, V, O and every optional output are DEVICE pointers owned
 *             by the caller.  The library allocates nothing, keeps no state
 *             between calls and needs no workspace.  O must not overlap Q, K
 *             or V: for bf16 and fp8 inputs and the anchored kinds the call
 *             runs two kernels on `stream`, and the first parks the rows' score
 *             extrema in O (8 bytes per row, inside the rows of the same
 *             32-row block) for the second, which then overwrites them.
 *   Streams   `stream` is a hipStream_t passed as void* (NULL: the null
 *             stream).  A call only enqueues work and returns; the caller
 *             synchronises.  Calls are reentrant and thread-safe.
 *   Errors    The return value is a qsa_status.  Arguments are validated on
 *             the host before any HIP call; nothing is launched when
 *             validation fails.  Launch failures return QSA_ERR_HIP.  Faults
 *             raised later by the asynchronous kernel surface at the caller's
 *             next synchronisation.  qsa_last_error() gives a thread-local
 *             text for the most recent failure on the calling thread.
 */
#ifndef QSA_H
#define QSA_H

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_VERSION 1

typedef enum {
  QSA_OK = 0,
  QSA_ERR_NULL_PTR = 1,    /* a required pointer is NULL                        */
  QSA_ERR_SHAPE = 2,       /* B, H, Hkv or N out of range, H % Hkv != 0, ...    */
  QSA_ERR_PARAM = 3,       /* k_levels, window, scale or descale out of range   */
  QSA_ERR_UNSUPPORTED = 4, /* a valid request the library does not implement    */
  QSA_ERR_HIP = 5          /* the HIP runtime reported an error at launch       */
} qsa_status;

typedef enum {
  QSA_DT_F32 = 0,
  QSA_DT_BF16 = 1,
  QSA_DT_FP8_E4M3 = 2
} qsa_dtype;

/*
 * variant = one base kind | any flags.
 *
 * QSA_EXACT           exact softmax with an online (running) maximum: the
 *                     control, w = exp(s - m).  One pass over the keys.
 * QSA_KINT            K-interval attention with K = k_levels intervals, i.e.
 *                     K+1 grid values T_l = exp(-l*Delta), Delta = (m - lo)/K,
 *                     l = 0..K.  Calibration lo = mn (min-max, default) or
 *                     lo = m - window (QSA_F_WINDOW).  With y = (m - s)/Delta:
 *                     hard rounding w = T_min(rint(y), K) (default) or linear
 *                     interpolation between T_floor(y) and T_floor(y)+1
 *                     (QSA_F_INTERP).  A min-max row whose visible scores are
 *                     all equal (Delta = 0) gives every visible key weight 1.
 * QSA_POT             Rowmax-PoT with L = k_levels levels: e = rint((m - s)
 *                     log2 e), saturated at L-1, w = 2^-e.
 * QSA_EXACT_ANCHORED  exact softmax anchored at the true row maximum found by
 *                     the same pre-pass the grid variants use, w = exp(s - m)
 *                     with no running rescale: the grid kernels with the
 *                     exponential put back, for like-for-like timing.
 * QSA_TRUNC           support truncation: the keys with s >= m - window keep
 *                     their exact weight exp(s - m), every other key gets 0
 *                     (the sensitivity study of "Approximating Softmax in
 *                     Pretrained LLMs", abstract: the support can be cut near
 *                     the row maximum).
 * QSA_UNIFORM         uniform weighting of the same support: weight 1 for the
 *                     keys with s >= m - window, 0 for the others, so each row
 *                     of O is the mean of the kept rows of V (the same study:
 *                     equal weights on the kept positions hurt).
 * QSA_POT_RUNNING     single-pass power-of-two weights with no row-maximum
 *                     pre-pass (the Rowmax-PoT page names a max-anchored
 *                     variant inside FlashAttention-4 without saying how the
 *                     maximum is found; this form is the library's own).  Keys
 *                     are visited in tiles of 64; after each tile the row's
 *                     anchor becomes A = ceil(running max of s log2 e), an
 *                     integer; a key's exponent e = rint(A - s log2 e) is
 *                     clipped to L-1 (or flushed) against the anchor of its
 *                     tile, and every rise of A by dA rescales the weights
 *                     formed before by 2^-dA exactly.  Without the clip the
 *                     weights are 2^rint(s log2 e), normalised.  L = k_levels
 *                     >= 2 (the row maximum lands on e = 0 or 1).
 *
 * QSA_F_INTERP        K-interval only: linear interpolation.
 * QSA_F_WINDOW        K-interval only: fixed-window calibration [m - window, m].
 * QSA_F_FLUSH         K-interval (window) and both PoT kinds: scores outside the
 *                     grid (K-interval: s < m - window; PoT: e >= L) get weight 0
 *                     instead of the last grid value.  On a min-max K-interval
 *                     grid every visible score lies inside, so the flag is
 *                     accepted and changes nothing.
 *
 * rint is round-half-to-even.  The row maximum always gets weight exactly 1.
 */
enum {
  QSA_EXACT = 0,
  QSA_KINT = 1,
  QSA_POT = 2,
  QSA_EXACT_ANCHORED = 3,
  QSA_TRUNC = 4,
  QSA_UNIFORM = 5,
  QSA_POT_RUNNING = 6,
  QSA_BASE_MASK = 0x0F,
  QSA_F_INTERP = 1 << 4,
  QSA_F_WINDOW = 1 << 5,
  QSA_F_FLUSH = 1 << 6
};

/* Index codes written to qsa_fwd_ex_opts.grid_idx for elements without a grid index. */
#define QSA_IDX_FLUSHED 254u
#define QSA_IDX_MASKED 255u

/*
 * Limits checked by validation:
 *   1 <= B, H, Hkv;  H % Hkv == 0;  1 <= N <= 2^20;  d in {64, 128};
 *   B*H*N*d < 2^31 and B*Hkv*N*d < 2^31 (element offsets are 32-bit);
 *   QSA_KINT: 1 <= k_levels <= 64;  QSA_POT: 1 <= k_levels <= 64;
 *   QSA_POT_RUNNING: 2 <= k_levels <= 64
 *   (fp8: k_levels <= 16, so the power-of-two weights stay exact in the
 *   8-bit operand of the PV product);
 *   QSA_F_WINDOW, QSA_TRUNC, QSA_UNIFORM: window finite and > 0;
 *   flags only on the kinds above (none on QSA_TRUNC and QSA_UNIFORM).
 */

/*
 * qsa_attn_fwd -- the attention forward.
 *
 *   Q, K, V   device inputs in the layout and dtype above.
 *   O         device output [B, H, N, d] (float32 for QSA_DT_F32, else bf16).
 *   B, H, Hkv batch, query heads, key/value heads.
 *   N         sequence length (queries and keys; causal is top-left aligned).
 *   d         head dimension, 64 or 128.
 *   causal    nonzero: key j is visible to query i only when j <= i.
 *   variant   base kind | flags (above).
 *   k_levels  K (K-interval intervals) or L (PoT levels); ignored by the
 *             exact kinds.
 *   window    W for QSA_F_WINDOW, QSA_TRUNC and QSA_UNIFORM, in units of the
 *             scaled score; else ignored.
 *   dtype     a qsa_dtype.
 *   stream    hipStream_t or NULL.
 * scale = 1/sqrt(d); fp8 descales 1.  Returns a qsa_status.
 */
int qsa_attn_fwd(const void* Q, const void* K, const void* V, void* O,
                 int B, int H, int Hkv, int N, int d, int causal,
                 int variant, int k_levels, float window, int dtype, void* stream);

/* Optional arguments and diagnostic outputs of qsa_attn_fwd_ex.  Zero-initialise
 * the struct and set what you need; every pointer is a device pointer or NULL. */
typedef struct {
  float scale;                 /* score scale; 0 -> 1/sqrt(d); must be finite and >= 0 */
  float q_descale;             /* fp8 per-tensor descales: stored value * descale = real */
  float k_descale;             /*   value; 0 -> 1.  Must be 1 or 0 for non-fp8 dtypes.   */
  float v_descale;
  float* row_max;              /* [B,H,N] float32: m_i (the anchor); QSA_POT_RUNNING:    */
                               /*   the final anchor A_i ln 2 (>= m_i, A_i an integer).   */
  float* row_lo;               /* [B,H,N] float32: K-interval: the calibrated lower end  */
                               /*   lo_i; QSA_TRUNC / QSA_UNIFORM: the support edge      */
                               /*   m_i - window; other anchored kinds: the visible row  */
                               /*   minimum.                                             */
                               /*   Not available for QSA_EXACT and QSA_POT_RUNNING      */
                               /*   (must be NULL).                                      */
  float* row_sum;              /* [B,H,N] float32: l_i = sum_j w_ij of the weights that  */
                               /*   entered the PV product (QSA_EXACT: relative to the   */
                               /*   final running maximum; QSA_POT_RUNNING: to the final */
                               /*   anchor).                                             */
  unsigned char* grid_idx;     /* [B,H,idx_rows,N] u8: per element the grid index l (K-  */
                               /*   interval; interpolation: floor(y) clipped to K; at   */
                               /*   an integer y either neighbour, where the weight is   */
                               /*   the same) or the exponent e (PoT); 0 for exact       */
                               /*   kinds and for the kept keys of QSA_TRUNC /           */
                               /*   QSA_UNIFORM;                                         */
                               /*   QSA_IDX_FLUSHED (also: outside the support) /        */
                               /*   QSA_IDX_MASKED otherwise.                            */
  int idx_row0;                /* first query row dumped into grid_idx                   */
  int idx_rows;                /* number of query rows dumped (0: none)                  */
} qsa_fwd_ex_opts;

/*
 * qsa_attn_fwd_ex -- qsa_attn_fwd with the options above (opts may be NULL,
 * which is qsa_attn_fwd).  The diagnostic outputs cost extra stores; the grid
 * index dump is meant for parity checks.  grid_idx requires idx_row0 >= 0,
 * idx_rows >= 1, idx_row0 + idx_rows <= N and B*H*idx_rows*N < 2^31.
 */
int qsa_attn_fwd_ex(const void* Q, const void* K, const void* V, void* O,
                    int B, int H, int Hkv, int N, int d, int causal,
                    int variant, int k_levels, float window, int dtype,
                    const qsa_fwd_ex_opts* opts, void* stream);

/*
 * Gradient modes of qsa_attn_bwd.  "Pretraining Transformers with Quantized
 * Softmax in Attention" (abstract; chapter 5 "Build the method") trains
 * K-interval attention with a straight-through surrogate placed before or
 * after the normalisation, derives backward rules through the calibration,
 * and compares attached with detached row extrema; it prints no formulas, so
 * each mode below states its reading.  P = w / l, dP = dO V^T, D_i = dO_i . O_i.
 *
 * QSA_GRAD_STE_POST        surrogate after the normalisation: P is passed back
 *                          as a softmax of the scores, dS = P (dP - D).
 * QSA_GRAD_EXACT           the derivative of the forward wherever it exists:
 *                          through each score (interpolation: the grid line's
 *                          slope; hard rounding, PoT, uniform: 0; exponential
 *                          kinds: w) and through the calibration (m moves y and,
 *                          for min-max grids, Delta = (m - lo)/K and the grid
 *                          values; lo moves Delta), those two gradients landing
 *                          on the row's first arg-max and arg-min keys.
 * QSA_GRAD_EXACT_DETACHED  QSA_GRAD_EXACT with m and lo held constant.
 * QSA_GRAD_STE_PRE         surrogate before the normalisation: QSA_GRAD_EXACT
 *                          with the rounding of the grid coordinate (K-interval
 *                          hard rounding, PoT) passed straight through where the
 *                          clip to the last level is not active.
 * QSA_GRAD_STE_PRE_DETACHED  QSA_GRAD_STE_PRE with m and lo held constant.
 *
 * At y = K the last interval's slope applies; on a min-max grid every visible
 * key counts as inside it.  A min-max row whose visible scores are all equal
 * gets no gradient through its weights in the modes other than STE_POST.
 */
enum {
  QSA_GRAD_STE_POST = 0,
  QSA_GRAD_EXACT = 1,
  QSA_GRAD_EXACT_DETACHED = 2,
  QSA_GRAD_STE_PRE = 3,
  QSA_GRAD_STE_PRE_DETACHED = 4
};

/*
 * qsa_attn_bwd -- gradients of sum(dO * O) for O = qsa_attn_fwd(Q, K, V, ...).
 *
 *   Q, K, V, dO  device inputs: Q and dO [B, H, N, d], K and V [B, Hkv, N, d],
 *                one dtype, QSA_DT_F32 or QSA_DT_BF16 (QSA_DT_FP8_E4M3 returns
 *                QSA_ERR_UNSUPPORTED).
 *   dQ           device output [B, H, N, d] float32.  Also the workspace: the
 *                first launch parks 8 floats of per-row constants at the start
 *                of each row of dQ, which the last launch reads and overwrites.
 *   dK, dV       device outputs [B, Hkv, N, d] float32, summed over the query
 *                heads of each KV head (overwritten, not accumulated).
 *   B .. dtype   as for qsa_attn_fwd (same limits, kinds and flags).
 *   grad         a QSA_GRAD_* mode.
 *   scale        score scale; 0 -> 1/sqrt(d).
 *   stream       hipStream_t or NULL.
 * dQ, dK and dV must not overlap each other or the inputs.  The forward's O is
 * not needed: the call recomputes the weights from Q and K (three kernels on
 * `stream`).  Float32 inputs: float32 arithmetic throughout.  BFloat16 inputs:
 * the products run on the matrix cores with float32 accumulation, and the
 * normalised weights P and score gradients dS enter dV = P^T dO, dK = scale
 * dS^T Q and dQ = scale dS K rounded to bfloat16; every weight and gradient
 * step between the products is float32.  Returns a qsa_status.
 */
int qsa_attn_bwd(const void* Q, const void* K, const void* V, const void* dO,
                 float* dQ, float* dK, float* dV,
                 int B, int H, int Hkv, int N, int d, int causal,
                 int variant, int k_levels, float window, int dtype,
                 int grad, float scale, void* stream);

/* Host-only validation of the scalar arguments of qsa_attn_fwd (no HIP call,
 * no pointer check).  Returns the status qsa_attn_fwd would return. */
int qsa_attn_validate(int B, int H, int Hkv, int N, int d, int causal,
                      int variant, int k_levels, float window, int dtype);

/* Static text for a status code ("QSA_OK", ...); never NULL. */
const char* qsa_status_string(int status);

/* Thread-local detail of the last failure on this thread ("" if none).  The
 * pointer stays valid until the next qsa_* call on the same thread. */
const char* qsa_last_error(void);

/* QSA_VERSION of the library. */
int qsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
