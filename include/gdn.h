/*
 * gdn.h -- C ABI of the MI355X (gfx950) chunked gated delta rule with dynamic
 * fake quantize-dequantize (QDQ) of the recurrent state and of the WY factor W.
 *
 * What is computed (the pages print no formulas; the readings are stated
 * here and checked against a float64 oracle):
 *   "[1/4] GDN state/W QAT foundation", section "What does this PR do?":
 *   GatedDeltaNet chunked training path, chunk size 64, exact triangular
 *   solve, dynamic FP8 E4M3 fake QDQ at the state and WY-activation (W) sites,
 *   identity straight-through gradients, the forward's quantized W saved for
 *   the backward, unsupported formats rejected.
 *   "[2/4] GDN/KDA decode QAT with INT8 recurrent state", section "What does
 *   this PR do?": signed symmetric dynamic INT8 state with per-head
 *   [Dk, block_v] scales, zero point zero, codes [-127, 127], nearest-even
 *   rounding; section "Testing": division by a scale is multiplication by
 *   its FP32-rounded reciprocal.
 *
 * Per (sequence, value head h) and chunk of n <= 64 tokens with incoming
 * state S (Dk x Dv, FP32):
 *   gamma_i = chunk-local cumsum of g;  Gam_ij = exp(gamma_i - gamma_j), i >= j
 *   L_ij = beta_i (k_i . k_j) Gam_ij (i > j);  T = (I + L)^-1 diag(beta)
 *   W = T diag(exp(gamma)) K;  U = T V
 *   Wq = QDQ_W(W)  (one scale per sequence, chunk and head over [n, Dk])
 *   Sq = QDQ_S(S)  (one scale per [Dk, block_v] tile)
 *   Vnew = U - Wq Sq
 *   O = scale (diag(exp(gamma)) Q Sq + ((Q K^T) * Gam) Vnew)
 *   S <- exp(gamma_n) Sq + (diag(exp(gamma_n - gamma)) K)^T Vnew
 * ht is the final S (not quantized). Grouped heads: value head h reads
 * query/key head h / (Hv / Hqk).
 * QDQ of a tile x (FP32):  d = max(fl(max|x| / q_max), 2^-126);
 *   r = fl(1/d);  c_i = RNE(fl(x_i * r)) on the code grid (E4M3FN, +-448,
 *   saturating; or integers clamped to [-127, 127]);  out_i = fl(c_i * d).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, row-major and contiguous,
 *     16-byte aligned. The caller allocates and owns every buffer; the library
 *     allocates no device memory, keeps no data between calls, never
 *     synchronizes, and enqueues work only on `stream` (a hipStream_t;
 *     NULL = default), except gdn_chunk_fwd's overlapped schedule below, whose
 *     second stream joins back into `stream` within the call's work.
 *   - Every argument check runs before any launch. A failed check returns a
 *     negative gdn_status, launches nothing and sets a message readable with
 *     gdn_last_error() (thread-local). There is no fallback path.
 *   - Errors raised by the HIP runtime at launch return GDN_E_HIP; faults
 *     inside a kernel surface asynchronously on the stream.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 8

typedef enum {
  GDN_OK = 0,
  GDN_E_INVALID = -1,      /* malformed argument: NULL, misaligned, bad shape */
  GDN_E_UNSUPPORTED = -2,  /* well formed but outside what is built          */
  GDN_E_WORKSPACE = -3,    /* workspace missing or too small                 */
  GDN_E_HIP = -4           /* HIP runtime error at launch                    */
} gdn_status;

typedef enum { GDN_QDQ_OFF = 0, GDN_QDQ_E4M3 = 1, GDN_QDQ_INT8 = 2 } gdn_qdq_fmt;
typedef enum { GDN_BF16 = 0, GDN_F32 = 1 } gdn_dtype;

/* QDQ policy ("[1/4]", "Usage": quantizer cfg + linear_attention policy). */
typedef struct {
  int32_t state_fmt;   /* gdn_qdq_fmt at the state site                      */
  int32_t w_fmt;       /* gdn_qdq_fmt at the W site                          */
  int32_t block_v;     /* state scale tile width: 16, 32, 64, 128 or 256;
                          divides Dv; at most 64 with FP32 inputs (ignored
                          when state_fmt == OFF). "[2/4] GDN/KDA decode QAT
                          with INT8 recurrent state", "Testing": all state
                          scale widths                                       */
  int32_t chunk_size;  /* must be 64                                         */
  int32_t solve_degree;/* 0: exact solve of the WY form (the default). d > 0:
                          opt-in approximate inverse ("[7/7] Experimental
                          GDN/KDA approximate-inverse QAT", "What does this PR
                          do?"): (I + L)^-1 is replaced by the Neumann
                          polynomial sum_{m=0..d} (-L)^m, in FP32. d must be
                          2^j - 1 for j = 1..6 (1, 3, 7, 15, 31, 63); any
                          other value is GDN_E_UNSUPPORTED, never rounded to
                          a supported one. Built for bf16 inputs (FP32
                          inputs return GDN_E_UNSUPPORTED for d > 0). The
                          saved buffer's x section then holds the
                          polynomial, not the inverse, and gdn_chunk_bwd
                          differentiates the polynomial itself: dL =
                          -sum_{m=1..d} sum_{a+b=m-1} (-L^T)^a dX (-L^T)^b. */
  int32_t read_fmt;    /* two-precision profile ("[5/8] ReplaySSM state QAT and
                          two-precision GDN", "What does this PR do?" and
                          "Usage"): GDN_QDQ_E4M3 keeps the state in FP32 (the
                          recurrence anchor, never quantized) and gives every
                          read of a chunk's incoming state, Vnew = U - Wq Sr
                          and O's Q Sr, a dynamic E4M3 copy Sr with one scale
                          per value column over the Dk key channels. Needs
                          state_fmt == OFF (GDN_E_INVALID otherwise), Dk == 128
                          and bf16 inputs (GDN_E_UNSUPPORTED otherwise; the
                          pages enable it for K = 128 only). INT8 reads are
                          GDN_E_UNSUPPORTED. GDN_QDQ_OFF (0): no read copy.  */
} gdn_qdq_policy;

/* Forward arguments. Shapes: without cu_seqlens there are N = B sequences of
 * T tokens; with cu_seqlens B must be 1, T is the packed length and N =
 * num_seqs. Sizes: Dk in {64, 128}; Dv in {64, 128, 256}; Hv % Hqk == 0.
 * io_dtype GDN_F32 needs Dk == 64. */
typedef struct {
  int32_t B, T, Hqk, Hv, Dk, Dv;
  int32_t num_seqs;            /* N (must equal B without cu_seqlens)         */
  int32_t io_dtype;            /* gdn_dtype of q, k, v and o                  */
  float scale;                 /* output scale (1/sqrt(Dk) is the usual one)  */
  int32_t prefix_len;          /* 0: whole sequences. > 0: only the first
                                  prefix_len tokens of every sequence are run
                                  (the exact chunk prefill of a decode
                                  continuation, "[2/4] GDN/KDA decode QAT with
                                  INT8 recurrent state", "What does this PR
                                  do?": an explicit prefix length selects
                                  chunk prefill, then token-state writes; see
                                  gdn_decode_fwd). ht is the state after the
                                  prefix; o, the saved buffer and every
                                  gradient are written for prefix tokens only,
                                  later tokens are left untouched. Negative:
                                  GDN_E_INVALID.                              */
  gdn_qdq_policy policy;
  const void* q;               /* [B, T, Hqk, Dk] io_dtype                    */
  const void* k;               /* [B, T, Hqk, Dk] io_dtype                    */
  const void* v;               /* [B, T, Hv, Dv]  io_dtype                    */
  const float* g;              /* [B, T, Hv] log-gate, g <= 0                 */
  const float* beta;           /* [B, T, Hv] write strength                   */
  const float* h0;             /* [N, Hv, Dk, Dv] initial state, or NULL = 0  */
  const int32_t* cu_seqlens;   /* [N + 1] offsets (device), or NULL           */
  void* o;                     /* out [B, T, Hv, Dv] io_dtype                 */
  float* ht;                   /* out [N, Hv, Dk, Dv] final state, or NULL    */
  void* saved;                 /* out: gdn_saved_bytes() bytes for the
                                  backward (layout gdn_saved_layout), or NULL */
  void* workspace;             /* gdn_fwd_workspace_bytes() bytes of device
                                  scratch (may be NULL when that is 0); its
                                  contents are undefined before and after    */
  size_t workspace_bytes;
} gdn_fwd_args;

/* Layout of the `saved` buffer, in bytes from its start. Chunk c of sequence
 * n (sequence-relative) uses slot n + bos_n / 64 + c (bos_n = first token of
 * n), so num_slots = N + ceil(B*T / 64).
 *   state:  state_fmt != OFF: quantized state codes Sq, one byte each
 *           (E4M3FN bit pattern, or int8), [num_slots, Hv, Dk, Dv];
 *           state_fmt == OFF: the state S in FP32, same shape.
 *   state_scale: FP32 d of each tile, [num_slots, Hv, Dv / block_v]
 *           (state_fmt != OFF only, else 0 bytes).
 *   w:      w_fmt != OFF: W codes, one byte each, token-major
 *           [B*T, Hv, Dk]; 0 bytes when w_fmt == OFF (the backward rebuilds W).
 *   w_scale: FP32 d of each W tile, [num_slots, Hv] (w_fmt != OFF only).
 *   x:      bf16 inputs only: X = (I + L)^-1 of every chunk, the inverse of
 *           the WY form's unit lower triangular matrix, FP32 row-major
 *           [num_slots, Hv, 64, 64]; the backward reads it instead of solving
 *           again. 0 bytes for FP32 inputs.
 *   anchor: read_fmt != OFF only: the FP32 state of every chunk before its
 *           reads, [num_slots, Hv, Dk, Dv]; the state section then holds the
 *           read copy Sr (FP32 values of codes times column scales).
 *   meta:   64 bytes: the policy (formats, block_v, solve_degree), shape and
 *           scale the forward ran under. gdn_chunk_bwd compares it with its
 *           own arguments on the device; on any difference every gradient
 *           output is set to NaN and GDN_DEVERR_SAVED_STAMP is raised in the
 *           device error flags (see gdn_device_errors), so a saved buffer
 *           is never read under another policy ("[7/7] Experimental GDN/KDA
 *           approximate-inverse QAT", "What does this PR do?": no silent
 *           change of degree or fallback).
 * Slots no chunk uses are left unwritten. */
typedef struct {
  int64_t num_slots;
  int64_t off_state, off_state_scale, off_w, off_w_scale, off_x, off_anchor, off_meta;
  int64_t total_bytes;
} gdn_saved_layout_t;

gdn_status gdn_saved_layout(const gdn_fwd_args* a, gdn_saved_layout_t* out);
size_t gdn_saved_bytes(const gdn_fwd_args* a);

/* Device scratch the forward needs (0 on error or for FP32 inputs). With
 * bf16 inputs the forward runs as two kernels: every (chunk, head) first
 * builds its state-independent operands (the solve, W and its QDQ, U and the
 * masked Q K^T) into this scratch; then one workgroup per (sequence, head,
 * 64-wide value block) runs the state recurrence over the chunks in order.
 * Per slot (see gdn_saved_layout) and value head: the W operand (128 * Dk
 * bytes, twice that with W QDQ off; 144 * Dk for Dk = 64), K^T (144 * Dk
 * bytes), masked Q K^T (18 KB), U (256 * Dv bytes) and one scale; about
 * 360 MB at B = 4, T = 4096, H = 16, Dk = Dv = 128. */
size_t gdn_fwd_workspace_bytes(const gdn_fwd_args* a);

/* Chunked forward. Writes o, and ht / saved when not NULL. Needs
 * a->workspace of gdn_fwd_workspace_bytes(a) bytes (GDN_E_WORKSPACE if
 * missing or too small).
 * Overlapped schedule: with bf16 inputs, full-precision reads (read_fmt off),
 * either equal-length sequences with at least 4 chunks each, or packed
 * sequences (cu_seqlens; at most 1,024 of them and 262,080 tokens in all,
 * whose chunk order and split a setup kernel derives from the lengths on the
 * device), and at least 16 CUs that the state recurrence's workgroups
 * (N * Hv * Dv / 64, or N * Hv * Dv / block_v for 128- and 256-wide scale
 * tiles) leave free, the state recurrence
 * starts once the first chunks' operands are built, and the remaining ones
 * are built meanwhile on those free CUs. The operand build runs on `stream`;
 * the state recurrence runs on a second stream that the library creates on
 * the device's first such call (with two events, kept until the process
 * ends), forked from `stream` and joined back into it, so later work on
 * `stream` waits for both. The kernels, their arithmetic and its order are
 * those of gdn_chunk_fwd_prep then gdn_chunk_fwd_state, so the results are
 * the same bits. Host threads enqueue it under a per-device lock. Code under
 * HIP graph capture uses gdn_chunk_fwd_noalloc, which always runs on
 * `stream` alone. With the environment variable GDN_NO_OVERLAP set (any
 * value, read once) this call and gdn_chunk_bwd run their stages one after
 * the other on `stream`: for profilers that serialize kernels, under which a
 * kernel waiting for another's ready flags would wait out its bound. */
gdn_status gdn_chunk_fwd(const gdn_fwd_args* a, void* stream);

/* The schedule gdn_chunk_fwd takes for these arguments on a device of `cus`
 * compute units (0: the current device's count): out[0] = 1 overlapped,
 * 0 one stage after the other; out[1] the (chunk, head) items of the
 * operand build; out[2] how many of them (whole rounds of cus, chunk-major)
 * run on every CU before the state recurrence starts; out[3] the CUs that
 * build the rest meanwhile (with a head and Dv <= 128, two operand-build
 * workgroups on each, on CUs picked on the device so that the recurrence's
 * workgroups find free CUs on every shader engine; else one workgroup each). For packed sequences out[1] and out[2] are
 * -1: the device derives them from the sequence lengths. Checks the shapes only; launches nothing.
 * The call itself runs one stage after the other if it cannot create its
 * second stream. */
gdn_status gdn_fwd_schedule(const gdn_fwd_args* a, int32_t cus, int32_t* out);

/* gdn_chunk_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments, checks, kernels and results as gdn_chunk_fwd, except that
 * a->workspace and a->workspace_bytes are not read: the forward scratch is a
 * fixed array inside the library, GDN_NOALLOC_SCRATCH_BYTES bytes on every
 * GPU it runs on, held until the process ends. A problem whose
 * gdn_fwd_workspace_bytes() exceeds that returns GDN_E_UNSUPPORTED before
 * any launch. The call allocates nothing. All calls on one GPU share that
 * GPU's array: calls that overlap on one GPU (several streams or host
 * threads at once) race on it and must be serialized by the caller. The
 * caller still owns o, ht and saved. */
#define GDN_NOALLOC_SCRATCH_BYTES (64ll << 20)
gdn_status gdn_chunk_fwd_noalloc(const gdn_fwd_args* a, void* stream);

/* The two stages of gdn_chunk_fwd, for callers that schedule or time them
 * separately: gdn_chunk_fwd_prep (every chunk and head: solve, W and its QDQ,
 * U, masked Q K^T, into the workspace; the saved W codes) then
 * gdn_chunk_fwd_state (the state recurrence and the output, from that
 * workspace) with the same arguments. For FP32 inputs the prep stage does
 * nothing and the state stage runs the whole forward. Same checks and errors
 * as gdn_chunk_fwd. */
gdn_status gdn_chunk_fwd_prep(const gdn_fwd_args* a, void* stream);
gdn_status gdn_chunk_fwd_state(const gdn_fwd_args* a, void* stream);

/* Backward arguments: the forward's arguments and `saved`, plus upstream
 * gradients. Identity straight-through at both QDQ sites; the saved Wq and
 * Sq are the values used in every product. grad_dtype applies to dq, dk, dv
 * (GDN_F32 or io_dtype). */
typedef struct {
  gdn_fwd_args fwd;            /* same values as the forward call; fwd.o,
                                  fwd.ht are not read; fwd.saved must hold the
                                  forward's saved buffer                      */
  const void* do_;             /* [B, T, Hv, Dv] io_dtype                     */
  const float* dht;            /* [N, Hv, Dk, Dv] or NULL (= 0)               */
  int32_t grad_dtype;          /* gdn_dtype of dq, dk, dv                     */
  void* dq;                    /* out [B, T, Hqk, Dk] (summed over the group) */
  void* dk;                    /* out [B, T, Hqk, Dk]                         */
  void* dv;                    /* out [B, T, Hv, Dv]                          */
  float* dg;                   /* out [B, T, Hv]                              */
  float* dbeta;                /* out [B, T, Hv]                              */
  float* dh0;                  /* out [N, Hv, Dk, Dv], or NULL                */
  void* workspace;             /* gdn_bwd_workspace_bytes() bytes, device     */
  size_t workspace_bytes;
} gdn_bwd_args;

size_t gdn_bwd_workspace_bytes(const gdn_bwd_args* a);
/* With bf16 inputs and equal-length sequences (at least 4 chunks each), where
 * the operand build of the reverse recurrence and the recurrence fit on one
 * CU together, the build of all but the last chunks' operands runs beside
 * the recurrence, on the second stream of gdn_chunk_fwd's overlapped
 * schedule (same lock, same join into `stream`, same GDN_NO_OVERLAP switch),
 * with the same kernels and arithmetic: the gradients are the same bits. */
gdn_status gdn_chunk_bwd(const gdn_bwd_args* a, void* stream);

/* Standalone state QDQ (the function used at the state site), bit-exact to
 * the FP32 definition above. x, y: [n_states, Dk, Dv] FP32 (y may alias x);
 * one scale per [Dk, block_v] tile of each state. scales ([n_states,
 * Dv / block_v] FP32) and codes ([n_states, Dk, Dv] bytes) are optional
 * outputs (NULL to skip). fmt must be E4M3 or INT8. Dk in [1, 1024],
 * block_v in {16, 32, 64, 128, 256} dividing Dv. */
gdn_status gdn_qdq_state(const float* x, float* y, float* scales, uint8_t* codes,
                         int64_t n_states, int32_t Dk, int32_t Dv, int32_t block_v,
                         int32_t fmt, void* stream);

/* ------------------------------------------------------------------------
 * Decode continuation ("[2/4] GDN/KDA decode QAT with INT8 recurrent state",
 * "What does this PR do?": an explicit prefix length selects exact chunk
 * prefill followed by token-state writes, gradients through initial states
 * and the continuation; "Testing": 257-token trajectories, nonzero initial
 * states, grouped heads, packed tails, both readouts, split carry, all state
 * scale widths, first-order input/state gradients).
 *
 * The prefill is gdn_chunk_fwd / gdn_chunk_bwd with prefix_len = P; the
 * decode steps are gdn_decode_fwd / gdn_decode_bwd with start = P on the same
 * token buffers, from the prefill's ht (and its dht from the decode's
 * dh_in). Per (sequence, value head h), from the state handed over S (h_in):
 *   S <- QDQ_S(S)                                    (the state as written)
 *   each decode token t (tokens start .. len-1 of the sequence):
 *     S <- exp(g_t) S;  u = beta_t (v_t - S^T k_t);  S <- S + k_t u^T
 *     o_before = scale S^T q_t;  S <- QDQ_S(S);  o_after = scale S^T q_t
 *     o_t = o_before or o_after, as `readout` selects
 *   ht = S, the last state written.
 * QDQ_S is the state QDQ above (one scale per [Dk, block_v] tile); with
 * state_fmt OFF it is the identity and the decode is the plain recurrence.
 * The arithmetic is FP32. */
typedef enum { GDN_READOUT_BEFORE_WRITE = 0, GDN_READOUT_AFTER_WRITE = 1 } gdn_readout;

/* Shapes as gdn_fwd_args (Dk in {64, 128}, Dv in {64, 128, 256}, either
 * io_dtype for any Dk). */
typedef struct {
  int32_t B, T, Hqk, Hv, Dk, Dv;
  int32_t num_seqs;            /* N (must equal B without cu_seqlens)         */
  int32_t io_dtype;            /* gdn_dtype of q, k, v and o                  */
  float scale;
  int32_t start;               /* first decode token of every sequence
                                  (sequence-relative, >= 0); earlier tokens
                                  are neither read nor written               */
  int32_t state_fmt;           /* gdn_qdq_fmt of the token-state writes       */
  int32_t block_v;             /* state scale tile width: 16, 32, 64, 128 or
                                  256 dividing Dv (ignored when OFF)          */
  int32_t readout;             /* gdn_readout                                 */
  const void* q;               /* [B, T, Hqk, Dk] io_dtype                    */
  const void* k;               /* [B, T, Hqk, Dk] io_dtype                    */
  const void* v;               /* [B, T, Hv, Dv]  io_dtype                    */
  const float* g;              /* [B, T, Hv] log-gate                         */
  const float* beta;           /* [B, T, Hv]                                  */
  const float* h_in;           /* [N, Hv, Dk, Dv] state handed over, or NULL  */
  const int32_t* cu_seqlens;   /* [N + 1] offsets (device), or NULL           */
  void* o;                     /* out [B, T, Hv, Dv]: decode tokens only      */
  float* ht;                   /* out [N, Hv, Dk, Dv] last written state, or NULL */
  void* saved;                 /* out: gdn_decode_saved_bytes() bytes for the
                                  backward, or NULL. Every written state: the
                                  first write of sequence n in slot
                                  lo_n + n (lo_n its first decode token, packed
                                  index), the write after decode token t in
                                  slot t + n + 1; state_fmt != OFF: codes
                                  [B*T + N, Hv, Dk, Dv] bytes, then (256-byte
                                  aligned) FP32 tile scales [B*T + N, Hv,
                                  Dv / block_v]; OFF: FP32 states
                                  [B*T + N, Hv, Dk, Dv]                      */
} gdn_decode_args;

size_t gdn_decode_saved_bytes(const gdn_decode_args* a);   /* 0 on error */

/* Decode steps. Writes o for decode tokens, ht and saved when not NULL.
 * Allocates nothing; no workspace. */
gdn_status gdn_decode_fwd(const gdn_decode_args* a, void* stream);

/* Backward of gdn_decode_fwd, identity straight-through at every write; the
 * saved written states are the values used in every product. Gradients are
 * written for decode tokens only (earlier tokens are left untouched, so the
 * prefill's gdn_chunk_bwd may fill them); dh_in (the gradient of h_in) is
 * the prefill's dht. grad_dtype applies to dq, dk, dv. */
typedef struct {
  gdn_decode_args fwd;         /* same values as the forward call; fwd.o,
                                  fwd.ht are not read; fwd.saved must hold the
                                  forward's saved buffer                      */
  const void* do_;             /* [B, T, Hv, Dv] io_dtype                     */
  const float* dht;            /* [N, Hv, Dk, Dv] or NULL (= 0)               */
  int32_t grad_dtype;
  void* dq;                    /* out [B, T, Hqk, Dk] (summed over the group) */
  void* dk;                    /* out [B, T, Hqk, Dk]                         */
  void* dv;                    /* out [B, T, Hv, Dv]                          */
  float* dg;                   /* out [B, T, Hv]                              */
  float* dbeta;                /* out [B, T, Hv]                              */
  float* dh_in;                /* out [N, Hv, Dk, Dv], or NULL                */
  void* workspace;             /* gdn_decode_bwd_workspace_bytes() bytes:
                                  partial dq, dk, dg, dbeta per token, value
                                  head and group of 64-column slabs (those of
                                  one scale tile), when a head has several
                                  groups or Hv > Hqk; 0 bytes otherwise      */
  size_t workspace_bytes;
} gdn_decode_bwd_args;

size_t gdn_decode_bwd_workspace_bytes(const gdn_decode_bwd_args* a);
gdn_status gdn_decode_bwd(const gdn_decode_bwd_args* a, void* stream);

const char* gdn_last_error(void);
int32_t gdn_abi_version(void);

/* Sticky device error flags of the current device. Kernels set them where a
 * check can only run on the device, instead of failing silently:
 *   GDN_DEVERR_LDS_WAIT     a bounded wait for another wave of the same
 *                           workgroup gave up (its outputs are not valid);
 *   GDN_DEVERR_FLAG_WAIT    a bounded wait for another workgroup gave up;
 *   GDN_DEVERR_SAVED_STAMP  gdn_chunk_bwd (or gdn_decode_bwd) got a saved
 *                           buffer written under another policy or shape
 *                           (its gradients are NaN);
 *   GDN_DEVERR_P_RANGE      with both QDQ sites on (state_fmt and w_fmt not
 *                           OFF, block_v <= 64, bf16 inputs) the forward
 *                           keeps the masked Q K^T operand, (q_i . k_j)
 *                           exp(gamma_i - gamma_j), in fp16 (11-bit
 *                           significand, range +-65504). Precondition:
 *                           |q_i . k_j| < 65504, which L2-normalised q and k
 *                           (GatedDeltaNet's) always meet. An entry beyond
 *                           it sets this flag (o and ht are then invalid).
 * Diagnostic query: unlike every other entry point it synchronizes the
 * device, then writes the flags to *flags and clears them. */
#define GDN_DEVERR_LDS_WAIT 1u
#define GDN_DEVERR_FLAG_WAIT 2u
#define GDN_DEVERR_SAVED_STAMP 4u
#define GDN_DEVERR_P_RANGE 8u
gdn_status gdn_device_errors(uint32_t* flags);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H */
