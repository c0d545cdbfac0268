// Forward, part 1: the state-independent work of every (chunk, value head)
// ("[1/4] GDN state/W QAT foundation", "What does this PR do?": exact
// triangular solve, W and its dynamic QDQ, the saved quantized W).
//
// Per chunk of n <= 64 tokens (rows past n are zero):
//   gamma = chunk-local cumsum of g;  Gam_ij = exp(gamma_i - gamma_j), i >= j
//   L = beta_i (K K^T)_ij Gam_ij (i > j);  P = (Q K^T) * Gam (i >= j)
//   X = (I + L)^-1: 16x16 diagonal blocks by substitution, then the 16- and
//       32-block merges X_BA = -X_BB L_BA X_AA (FP32 MFMA)
//   T = X diag(beta);  T' = T diag(exp(gamma))
//   W = T' K, QDQ_W over the [n, Dk] tile;  U = T V
// Outputs are the operand images described in gdn_images.h, plus the W codes
// and scale in the caller's saved buffer when it asks for them, with X
// (= (I + L)^-1) for the backward.
//
// Precision: q, k, v are bf16 and exact as MFMA operands; T and T' (FP32) are
// split as hi + lo bf16 (two passes), so W and U carry ~16 mantissa bits of T
// with FP32 accumulation. L, X and the merges stay FP32 throughout.
//
// Launch: persistent 8-wave workgroups, each walking (chunk, head) items and
// loading the next item's q, k, v, g, beta into registers while it computes
// the current one. Two workgroups share a CU where the compact LDS layout
// below fits (Dv <= 128, exact solve); the full layout runs one per CU (the
// opt-in Neumann solve, Dv = 256, and overlapped launches without a head).
#include <hip/hip_ext.h>

#include <type_traits>

#include "gdn_device.h"
#include "gdn_images.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

constexpr int NT = 512;
constexpr int NWAVE = NT / 64;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// 8 bytes at base + off (base wave-uniform, off < 2^31, 8-byte aligned): a
// device-scope buffer store (cache policy sc1) when a concurrent kernel reads
// them after a ready flag, else a plain store.
__device__ __forceinline__ void st_out8(void* base, int off, u32x2 v, bool coh) {
  if (coh) {
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7FFFFFF0, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b64(v, rsrc, off, 0, 16);
  } else {
    *reinterpret_cast<u32x2*>(reinterpret_cast<char*>(base) + off) = v;
  }
}
constexpr float LOG2E = 1.4426950408889634f;

// One item's LDS, in one of two layouts with the same accessors.
//
// Compact (Dv <= 128, exact solve): regions are reused as their contents
// die, so that it stays under 80 KB and two workgroups share a CU:
//   a: K and Q rows (phase 1 to the L / P tiles), then K^T and V^T (written
//      in the solve phase, read by W and U), then the W image planes;
//   l: L (until the 32-block merge), then the T' hi / lo planes;
//   x: the P planes (the tile phase; copied out at the start of the solve),
//      X = (I + L)^-1 (written from the 16-block merges on), then the T hi /
//      lo planes;
//   Y: the diagonal 16x16 blocks of X (the solve phase and the 16-block
//      merges), then the 32-block merge's scratch.
// Offset between the diagonal 16x16 blocks of X that the compact layout keeps
// in Y (row stride 16): four of them fill Y's 32 x 33 floats.
constexpr int kDiagY = 264;

template <int DK, int DV>
struct PrepSmemTwo {
  static constexpr bool TWO = true;
  static constexpr int LDK = DK + 8;             // K, Q rows (pperm over dk)
  static constexpr int LS = 68;                  // row stride of the FP32 64 x 64 solve matrices
  union {
    struct { bf16 K[64 * LDK]; bf16 Q[64 * LDK]; } kq;
    struct { bf16 Kt[DK * 64]; bf16 Vt[DV * 72]; } tv;   // K^T (r64_off), V^T (pperm over tokens)
    bf16 W[2 * Img<DK>::WQ];                              // W image planes
  } a;
  union { float L[64 * LS]; bf16 T[2][64 * 64]; } l;      // L; T' hi / lo (r64_off)
  union { float X[64 * LS]; bf16 T[2][64 * 64]; } x;      // X; T hi / lo (r64_off)
  float Y[32 * 33];                              // X's diagonal blocks, then 32-block merge scratch
  static_assert(4 * kDiagY <= 32 * 33, "diagonal blocks of X in Y");
  alignas(16) float Ld[4][16 * 16];              // diagonal 16x16 blocks of L, row-major
  alignas(16) float gam2[64];                    // log2-scaled gamma
  alignas(16) float bet[64];
  alignas(16) float eg[64];                      // exp(gamma)
  alignas(16) float red[NWAVE];
  __device__ bf16* Pl(int i) { return reinterpret_cast<bf16*>(x.X) + i * 64 * 64; }
  __device__ bf16* Kt() { return a.tv.Kt; }
  __device__ bf16* Vt() { return a.tv.Vt; }
  __device__ float* Lm() { return l.L; }
  __device__ float* Xm() { return x.X; }
  __device__ float* Ym() { return Y; }
  __device__ bf16* Wm() { return a.W; }
  __device__ bf16* Tp(int i) { return l.T[i]; }   // T' hi, lo
  __device__ bf16* Tt(int i) { return x.T[i]; }   // T hi, lo
  __device__ static int t_off(int row, int c0) { return r64_off(row, pperm(c0)); }
  __device__ static bf16x8 t_frag(const bf16* t, int row, int kk, int grp) { return ld_r64(t, row, 32 * kk, grp); }
};

// Full (Dv = 256, or the approximate inverse's four 64 x 64 buffers): every
// operand in its own place, one workgroup per CU. P, and the T planes of
// both kinds, sit in region c, and K^T leaves for the image with P during
// the solve.
template <int DK>
struct PrepSmemOne {
  static constexpr bool TWO = false;
  static constexpr int LDK = DK + 8;
  static constexpr int LS = 65;
  union {
    struct { bf16 K[64 * LDK]; bf16 Q[64 * LDK]; } kq;   // until the L / P tiles
    bf16 Vt[256 * 72];                                    // V^T (pperm over tokens)
  } a;
  bf16 Kt_[DK * 64];                             // K^T (pperm over tokens, r64_off)
  union {
    struct { float L[64 * 65]; float X[64 * 65]; } s;    // solve
    bf16 W[2 * Img<DK>::WQ];                              // W image planes
  } b;
  union {
    bf16 P[2][64 * 64];                          // P hi / lo (r64_off), until copied out
    float Y[32 * 33];                            // 32-block merge scratch
    bf16 T[4][64 * 72];                          // T hi, T lo, T' hi, T' lo
    float C[2][64 * 65];                         // the approximate inverse's two extra buffers
  } c;
  alignas(16) float Ld[4][16 * 16];
  alignas(16) float gam2[64];
  alignas(16) float bet[64];
  alignas(16) float eg[64];
  alignas(16) float red[NWAVE];
  __device__ bf16* Pl(int i) { return c.P[i]; }
  __device__ bf16* Kt() { return Kt_; }
  __device__ bf16* Vt() { return a.Vt; }
  __device__ float* Lm() { return b.s.L; }
  __device__ float* Xm() { return b.s.X; }
  __device__ float* Ym() { return c.Y; }
  __device__ bf16* Wm() { return b.W; }
  __device__ bf16* Tp(int i) { return c.T[2 + i]; }
  __device__ bf16* Tt(int i) { return c.T[i]; }
  __device__ static int t_off(int row, int c0) { return row * 72 + pperm(c0); }
  __device__ static bf16x8 t_frag(const bf16* t, int row, int kk, int grp) { return lds_nat(t, row, 72, 32 * kk, grp); }
};

// Whether the compact layout fits two workgroups per CU (Dv <= 128).
template <int DK, int DV>
constexpr bool prep_fits_two() { return sizeof(PrepSmemTwo<DK, DV>) <= 80 * 1024; }
template <int DK, int DV, bool CMP>
using PrepSmem = std::conditional_t<CMP, PrepSmemTwo<DK, DV>, PrepSmemOne<DK>>;

// The L and P tiles (mi >= mj) of one wave: all share the key block mj; kind
// 0 is L(mi, mj), 1 is P(mi, mj). Every lower tile of each matrix appears once
// over the 8 waves, at most three per wave.
struct PrepJobs {
  int n, mj, mi[3], kind[3];
};
__device__ __forceinline__ PrepJobs prep_jobs(int wave) {
  PrepJobs j;
  switch (wave) {
    case 0: j = {3, 0, {0, 1, 0}, {0, 0, 1}}; break;   // L(0,0) L(1,0) P(0,0)
    case 1: j = {3, 0, {2, 3, 1}, {0, 0, 1}}; break;   // L(2,0) L(3,0) P(1,0)
    case 2: j = {2, 0, {2, 3, 0}, {1, 1, 0}}; break;   // P(2,0) P(3,0)
    case 3: j = {3, 1, {1, 2, 1}, {0, 0, 1}}; break;   // L(1,1) L(2,1) P(1,1)
    case 4: j = {3, 1, {3, 2, 3}, {0, 1, 1}}; break;   // L(3,1) P(2,1) P(3,1)
    case 5: j = {3, 2, {2, 3, 2}, {0, 0, 1}}; break;   // L(2,2) L(3,2) P(2,2)
    case 6: j = {1, 2, {3, 0, 0}, {1, 0, 0}}; break;   // P(3,2)
    default: j = {2, 3, {3, 3, 0}, {0, 1, 0}}; break;  // L(3,3) P(3,3)
  }
  return j;
}

// acc += A(i0 + r, k) B(k, j0 + c) over k in [k0, k1) (FP32 MFMA 16x16x4),
// A(i, k) = A[i * ars + k], B(k, j) = B[k * brs + j].
__device__ __forceinline__ f32x4 mm32(const float* A, int ars, const float* B, int brs, int i0,
                                      int j0, int k0, int k1, int r16, int grp, f32x4 acc) {
  for (int k = k0; k < k1; k += 4)
    acc = mfma_f32(A[(i0 + r16) * ars + k + grp], B[(k + grp) * brs + j0 + r16], acc);
  return acc;
}

// acc += A(16 ti + r, k) B(k, 16 tj + c) over the key blocks tj..ti of two
// lower triangular FP32 64 x 64 matrices (row stride LS); a block's eight reads are issued
// before its four products.
template <int LS>
__device__ __forceinline__ f32x4 mm_lower(const float* A, const float* B, int ti, int tj, int r16,
                                          int grp, f32x4 acc) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    if (kb < tj || kb > ti) continue;
    float av[4], bv[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      av[s] = A[(16 * ti + r16) * LS + 16 * kb + 4 * s + grp];
      bv[s] = B[(16 * kb + 4 * s + grp) * LS + 16 * tj + r16];
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma_f32(av[s], bv[s], acc);
  }
  return acc;
}

// The two 16x16 output tiles (ti, tj) of a wave in a product of lower
// triangular 64x64 matrices: the ten lower tiles (1 to 4 key blocks each, 20
// in all) at most 4 blocks per wave, the six upper tiles (zero) on the rest.
__device__ __forceinline__ void lower_tiles(int wave, int (&ti)[2], int (&tj)[2]) {
  static constexpr int8_t tab[8][4] = {{3, 0, 2, 3}, {3, 1, 0, 0}, {2, 0, 1, 1}, {2, 1, 3, 2},
                                       {1, 0, 2, 2}, {3, 3, 0, 1}, {0, 2, 0, 3}, {1, 2, 1, 3}};
  ti[0] = tab[wave][0];
  tj[0] = tab[wave][1];
  ti[1] = tab[wave][2];
  tj[1] = tab[wave][3];
}

// Writes 4 consecutive bf16 at dst (8-byte aligned).
__device__ __forceinline__ void st4(bf16* dst, bf16 a, bf16 b, bf16 c, bf16 d) {
  *reinterpret_cast<bf16x4*>(dst) = bf16x4{a, b, c, d};
}

// A [64 tokens][D] bf16 tile of q, k or v staged through registers: TPG
// tokens x 8 columns per thread. Eight consecutive lanes hold 64 adjacent
// columns (128 bytes) of one token, so a load instruction touches eight
// 128-byte lines (issuing a load costs about a cycle per line it touches);
// wave w covers column slab w % NS and token groups 8 (w / NS) .. + 7. The
// loads are unconditional (row clamped to the chunk); rows past the chunk end
// are zeroed when the registers are written out, not when they arrive, so
// nothing waits for a prefetch until its data is used.
template <int D>
struct Stage {
  static constexpr int TPG = 8 * D / NT;         // tokens per thread (1, 2, 4)
  static constexpr int NTG = 64 / TPG;           // token groups
  static constexpr int NS = D / 64;              // 64-column slabs
  static_assert(TPG >= 1 && TPG <= 4 && NS == TPG && NTG * NS == 64, "thread layout");
  uint4 raw[TPG];
  int nc;
  __device__ int tg(int wave, int lane) const { return 8 * (wave / NS) + (lane >> 3); }
  __device__ int c8(int wave, int lane) const { return 8 * (wave % NS) + (lane & 7); }
  __device__ void load(const bf16* src, int64_t row_stride, int nc_, int wave, int lane) {
    nc = nc_;
#pragma unroll
    for (int p = 0; p < TPG; ++p) {
      const int row = TPG * tg(wave, lane) + p;
      raw[p] = *reinterpret_cast<const uint4*>(src + min(row, nc - 1) * row_stride + 8 * c8(wave, lane));
    }
  }
  __device__ bf16x8 row8(int p, int wave, int lane) const {
    const uint4 z = make_uint4(0, 0, 0, 0);
    const uint4 v = TPG * tg(wave, lane) + p < nc ? raw[p] : z;
    return *reinterpret_cast<const bf16x8*>(&v);
  }
  // dst[(8 c8 + j) * 72 + pperm(token)] (or the unpadded r64_off layout when
  // R64S); also to gdst if given
  template <bool R64S = false>
  __device__ void store_t(bf16* dst, bf16* gdst, int wave, int lane) const {
    bf16x8 r[TPG];
#pragma unroll
    for (int p = 0; p < TPG; ++p) r[p] = row8(p, wave, lane);
    const int t0 = TPG * tg(wave, lane), col0 = 8 * c8(wave, lane);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int off = R64S ? r64_off(col0 + j, pperm(t0)) : (col0 + j) * 72 + pperm(t0);
      bf16* d = dst + off;
      bf16* g = gdst ? gdst + off : nullptr;
      if constexpr (TPG == 1) {
        *d = r[0][j];
        if (g) *g = r[0][j];
      } else if constexpr (TPG == 2) {
        typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 v = bf16x2{r[0][j], r[1][j]};
        *reinterpret_cast<bf16x2*>(d) = v;
        if (g) *reinterpret_cast<bf16x2*>(g) = v;
      } else {
        const bf16x4 v = bf16x4{r[0][j], r[1][j], r[2][j], r[3][j]};
        *reinterpret_cast<bf16x4*>(d) = v;
        if (g) *reinterpret_cast<bf16x4*>(g) = v;
      }
    }
  }
  // row-major dst[token * ld + pperm(col)] (two 4-element units per row)
  __device__ void store_rows(bf16* dst, int ld, int wave, int lane) const {
    const int col0 = 8 * c8(wave, lane);
#pragma unroll
    for (int p = 0; p < TPG; ++p) {
      bf16* d = dst + (TPG * tg(wave, lane) + p) * ld;
      const bf16x8 r = row8(p, wave, lane);
      st4(d + pperm(col0), r[0], r[1], r[2], r[3]);
      st4(d + pperm(col0 + 4), r[4], r[5], r[6], r[7]);
    }
  }
};

// A (chunk, head) work item; items are numbered slot-major: i = slot * Hv + h.
struct PrepItem {
  int i, slot, h, t0, nc;
  bool valid;
};

__device__ PrepItem prep_item(const FwdKernelArgs& a, int N, int i) {
  PrepItem it;
  it.i = i;
  it.slot = i / a.Hv;
  it.h = i % a.Hv;
  // sequence of this slot (slot = n + bos_n / 64 + c, increasing in n).
  // cu_seqlens is read through the constant address space: the item index is
  // wave-uniform, so these become scalar loads, which no vector-memory wait
  // covers (a vector load here made every item start by waiting for the
  // previous item's stores)
  if (a.vplan) {
    // packed sequences, chunk-major from the setup kernel's table: item i is
    // (n Hv + h, chunk c)
    typedef const int32_t __attribute__((address_space(4)))* cptr;
    const cptr tab = (cptr)a.vplan + 4, cu = (cptr)a.cu_seqlens;
    const int code = tab[2 * i], c = tab[2 * i + 1], n = code / a.Hv;
    const int bos = cu[n];
    int eos = cu[n + 1];
    if (a.prefix_len > 0) eos = min(eos, bos + a.prefix_len);
    it.h = code - n * a.Hv;
    it.slot = n + bos / CHUNK + c;
    it.t0 = bos + CHUNK * c;
    it.valid = it.t0 < eos;
    it.nc = it.valid ? min(CHUNK, eos - it.t0) : 0;
    return it;
  }
  if (a.chunk_major) {
    // equal-length sequences, chunk c of every (sequence, head) before chunk
    // c + 1 (the overlapped forward): item = (c N + n) Hv + h
    const int nh = N * a.Hv, c = i / nh, r = i - c * nh, n = r / a.Hv;
    const int len = a.prefix_len > 0 ? min(a.T, a.prefix_len) : a.T;
    it.h = r - n * a.Hv;
    it.slot = n + (n * a.T) / CHUNK + c;
    it.t0 = n * a.T + CHUNK * c;
    it.valid = CHUNK * c < len;
    it.nc = it.valid ? min(CHUNK, len - CHUNK * c) : 0;
    return it;
  }
  if (!a.cu_seqlens && a.T % CHUNK == 0) {
    // equal lengths: T / 64 chunk slots and one spare slot per sequence
    const int per = a.T / CHUNK + 1, n = it.slot / per, c = it.slot - n * per;
    const int len = a.prefix_len > 0 ? min(a.T, a.prefix_len) : a.T;
    it.t0 = n * a.T + CHUNK * c;
    it.valid = CHUNK * c < len;
    it.nc = it.valid ? min(CHUNK, len - CHUNK * c) : 0;
    return it;
  }
  typedef const int32_t __attribute__((address_space(4)))* cptr;
  const cptr cu = (cptr)a.cu_seqlens;
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const int bos = cu ? cu[mid] : mid * a.T;
    if (mid + bos / CHUNK <= it.slot) lo = mid; else hi = mid - 1;
  }
  const int bos = cu ? cu[lo] : lo * a.T;
  int eos = cu ? cu[lo + 1] : (lo + 1) * a.T;
  if (a.prefix_len > 0) eos = min(eos, bos + a.prefix_len);   // prefix cap (see seq_span)
  const int c = it.slot - (lo + bos / CHUNK);
  it.t0 = bos + CHUNK * c;
  it.valid = c >= 0 && it.t0 < eos;               // some slots are used by no chunk
  it.nc = it.valid ? min(CHUNK, eos - it.t0) : 0;
  return it;
}

// First valid item at or after i in steps of `stride` (i >= total: none).
__device__ PrepItem next_item(const FwdKernelArgs& a, int N, int i, int stride, int total) {
  PrepItem it;
  it.valid = false;
  for (; i < total; i += stride) {
    it = prep_item(a, N, i);
    if (it.valid) break;
  }
  return it;
}

// Whether this workgroup's CU builds the rest of the items beside the state
// kernel (two prep workgroups per CU). A CU is named by its XCC (XCC_ID) and
// HW_ID bits 15:8 (cu, sh and se within the XCC). The state kernel's
// workgroups are spread evenly over the XCCs and, within each, over its four
// shader engines, and a workgroup can only start on a free CU of the engine
// it is sent to; so the rest is kept on prep_rest / 32 CUs of every engine
// (the remainder to the first engines). The first of a CU's workgroups to ask
// takes one of its engine's places, or finds them gone; the other reads that
// decision (bounded wait: on give-up it records kErrFlagWait and leaves the
// rest to the others).
__device__ bool admit_cu(const FwdKernelArgs& a) {
  const uint32_t key = (__builtin_amdgcn_s_getreg((31 << 11) | 4) >> 8) & 0xFFu;   // HW_ID
  const uint32_t xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20) & 7u;            // XCC_ID
  const int se = (int)(key >> 5) & 3, slot = (int)xcc * 4 + se;
  uint32_t* tab = a.admit + xcc * kAdmitPerXcc;
  const int quota = a.prep_rest / 32 + (slot < a.prep_rest % 32 ? 1 : 0);
  uint32_t st = atomicCAS(tab + key, 0u, 3u);      // 0 open, 3 deciding, 1 admitted, 2 refused
  if (st == 0u) {
    st = (int)atomicAdd(tab + 256 + se, 1u) < quota ? 1u : 2u;
    __hip_atomic_store(tab + key, st, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return st == 1u;
  }
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  while (st == 3u) {
    if (__builtin_amdgcn_s_memtime() - t0 > (1ull << 27)) {
      __hip_atomic_fetch_or(a.err, kErrFlagWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
    st = __hip_atomic_load(tab + key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return st == 1u;
}

// NEU: the instantiation that carries the approximate inverse (the exact-solve
// instantiation does not contain its code). CMP: the compact layout, two
// workgroups per CU.
// (the second launch bound is the minimum of waves per SIMD: two 8-wave
// workgroups per CU need four, which caps a wave at 128 VGPRs)
template <int DK, int DV, int WF, bool NEU, bool CMP>
__global__ void __launch_bounds__(NT, (CMP ? 4 : 1))
gdn_prep_kernel(FwdKernelArgs a, int N, int num_slots) {
  using I = Img<DK>;
  static_assert(!CMP || (!NEU && prep_fits_two<DK, DV>()), "the compact layout: exact solve, Dv <= 128");
  using Sm = PrepSmem<DK, DV, CMP>;
  constexpr int LDK = Sm::LDK;
  constexpr int LS = Sm::LS;
  constexpr int NW = WF == 0 ? 2 : 1;
  constexpr int NCTW = DK / 32;                   // W column tiles per wave (two waves per row tile)
  constexpr int NVB = DV / 64;
  __shared__ __align__(16) Sm sm;

  const int Hv = a.Hv, Hqk = a.Hqk;
  // (packed sequences in the overlapped forward: the item count and the head
  // split come from the setup kernel's table)
  const int total = a.vplan ? __builtin_amdgcn_readfirstlane(a.vplan[0])
                            : (a.item_hi > 0 ? a.item_hi : num_slots * Hv);
  const int split = a.vplan ? __builtin_amdgcn_readfirstlane(a.vplan[1]) : a.item_split;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int lane = fresh_lane(), tid = wave * 64 + lane, r16 = lane & 15, grp = lane >> 4;
  // per-lane LDS addresses are rebuilt in each phase, not kept live across the
  // item loop (fresh_lane in gdn_device.h)
#define GDN_REFRESH() \
  lane = fresh_lane(); tid = wave * 64 + lane; r16 = lane & 15; grp = lane >> 4

  Stage<DK> ks, qs;
  Stage<DV> vs;
  float graw = 0.f, braw = 0.f;                   // g, beta of token min(lane, nc - 1)
  auto load_kqg = [&](const PrepItem& it) {
    const int hk = it.h / (Hv / Hqk);
    ks.load(reinterpret_cast<const bf16*>(a.k) + ((int64_t)it.t0 * Hqk + hk) * DK, (int64_t)Hqk * DK,
            it.nc, wave, lane);
    qs.load(reinterpret_cast<const bf16*>(a.q) + ((int64_t)it.t0 * Hqk + hk) * DK, (int64_t)Hqk * DK,
            it.nc, wave, lane);
    if (wave == 0) {                               // the wave that forms the gates
      const int64_t gi = (int64_t)(it.t0 + min(lane, it.nc - 1)) * Hv + it.h;
      graw = a.g[gi];
      braw = a.beta[gi];
    }
  };
  auto load_v = [&](const PrepItem& it) {
    vs.load(reinterpret_cast<const bf16*>(a.v) + ((int64_t)it.t0 * Hv + it.h) * DV, (int64_t)Hv * DV,
            it.nc, wave, lane);
  };

  // Items in a fixed stride per workgroup, or (publishing to a concurrent
  // state kernel) from a shared counter: then the workgroups that are
  // resident take the lowest items left, whatever else occupies the device,
  // so the state kernel never waits on an item no running workgroup holds.
  __shared__ int tk_next;
  const bool dyn = a.ticket != nullptr;
  // With a split, counter [0] hands out the head (items below the split) to
  // every workgroup and counter [1] the rest to the first prep_rest ones. Once
  // counter [0] has passed the split it only grows, so a workgroup that has
  // seen that goes straight to counter [1]: one atomic round trip per item.
  bool in_rest = a.prep_rest > 0 && split <= 0;    // tid 0's: the head is gone
  // tid 0's: whether this workgroup builds the rest (by workgroup index with
  // one per CU, by CU with two; decided when the head is gone)
  int member = a.admit ? -1 : ((int)blockIdx.x < a.prep_rest ? 1 : 0);
  auto take = [&]() -> int {                       // tid 0: the next item, or -1
    if (!in_rest) {
      const int t = a.item_lo + (int)atomicAdd(a.ticket, 1u);
      if (a.prep_rest <= 0 || t < split) return t < total ? t : -1;
      in_rest = true;
    }
    if (member < 0) member = admit_cu(a) ? 1 : 0;
    if (member == 0) return -1;
    const int r = split + (int)atomicAdd(a.ticket + 1, 1u);
    return r < total ? r : -1;
  };
  PrepItem cur;
  if (dyn) {
    if (threadIdx.x == 0) tk_next = take();
    __syncthreads();
    const int i0 = tk_next;
    cur = i0 >= 0 ? prep_item(a, N, i0) : PrepItem{};
    if (i0 < 0) cur.valid = false;
    __syncthreads();                               // every wave has read it before the next ticket
  } else {
    cur = next_item(a, N, a.item_lo + blockIdx.x, gridDim.x, total);
  }
  if (!cur.valid) return;
  load_kqg(cur);
  load_v(cur);

  while (true) {
    GDN_REFRESH();
    PrepItem nxt;
    if (dyn) {
      nxt.valid = false;
      if (tid == 0) tk_next = take();              // read after this item's first barrier
    } else {
      nxt = next_item(a, N, cur.i + gridDim.x, gridDim.x, total);
    }
    const int h = cur.h, t0 = cur.t0, nc = cur.nc;
    const int64_t ch = (int64_t)cur.slot * Hv + h;
    bf16* img = a.ws_img + ch * I::template img<NW>();   // [W planes | K^T | P | gates]

    // ---- 1. K, Q rows (pperm over dk) and gates from registers (the full
    // layout: K^T too). P upper tiles (0, 1) and (2, 3), which the state
    // kernel reads as zeros, are zeroed in the LDS P planes
    if constexpr (Sm::TWO) {
      const int pl = tid >> 7, e = tid & 127, t = e >> 6, r = (e >> 2) & 15, g = e & 3;
      if (tid < (a.w_img_bytes ? 128 : 256))
        *reinterpret_cast<u32x2*>(sm.Pl(pl) + r64_off(32 * t + r, pperm(32 * t + 16 + 4 * g))) = u32x2{0u, 0u};
    } else {
#pragma unroll
      for (int k = 0; k < 2 * 2 * 256 / NT; ++k) {
        const int e = tid + NT * k;
        const int pl = e >> 9, t = (e >> 8) & 1, r = (e >> 4) & 15, cc = e & 15;
        sm.c.P[pl][r64_off(32 * t + r, pperm(32 * t + 16 + cc))] = to_bf16(0.f);
      }
    }
    ks.store_rows(sm.a.kq.K, LDK, wave, lane);
    qs.store_rows(sm.a.kq.Q, LDK, wave, lane);
    if constexpr (!Sm::TWO) ks.template store_t<true>(sm.Kt(), nullptr, wave, lane);   // the image copy goes out during the solve
    if (wave == 0) {
      const float gv = lane < nc ? graw : 0.f;
      const float g2 = wave_incl_scan(gv * LOG2E);
      const float g2n = read_lane(g2, nc - 1);
      const float eg = fexp2(g2);
      sm.gam2[lane] = g2;
      sm.bet[lane] = lane < nc ? braw : 0.f;
      sm.eg[lane] = eg;
      // the gate block follows the single fp16 P plane in the byte variant
      const int goff = a.w_img_bytes ? I::template p_at<NW>() + I::P1 : I::template g_at<NW>();
      float* G = reinterpret_cast<float*>(img + goff);
      const bool coh = a.flags != nullptr;
      st_out(G + lane, eg, coh);
      st_out(G + 64 + lane, lane < nc ? fexp2(g2n - g2) : 0.f, coh);
      if (lane != 1) st_out(G + 128 + lane, lane == 0 ? fexp2(g2n) : 0.f, coh);   // [129]: the W scale, below
      st_out(G + 192 + lane, 0.f, coh);
    }
    lds_barrier();
    GDN_REFRESH();
    if (dyn) {
      const int i1 = tk_next;
      if (i1 >= 0) nxt = prep_item(a, N, i1);
    }

    // ---- 2. L (FP32) and P (hi / lo, pperm over columns): 20 tiles over 8 waves.
    // Every tile of a wave shares its key block mj, whose fragments are read
    // once and serve as B of L(mi, mj) = K_mi K_mj^T and as A of the P^T tile
    // K_mj Q_mi^T (the phase is bound by LDS reads: 96 KB of operands
    // instead of 160 KB with a fresh pair per tile).
    {
      constexpr int KS = DK / 32;
      const PrepJobs jb = prep_jobs(wave);
      bf16x8 bk[KS];
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) bk[kk] = lds_nat(sm.a.kq.K, 16 * jb.mj + r16, LDK, 32 * kk, grp);
      // gate values of the key block, read with the operands (16-byte reads)
      const float gj = sm.gam2[16 * jb.mj + r16];
      const f32x4 gc = *reinterpret_cast<const f32x4*>(&sm.gam2[16 * jb.mj + 4 * grp]);
#pragma unroll
    for (int t3 = 0; t3 < 3; ++t3) {
      if (t3 >= jb.n) break;
      const int mi = jb.mi[t3], mj = jb.mj;
      const bool isP = jb.kind[t3] != 0;
      bf16x8 ao[KS];
      if (isP || mi != mj) {
        const bf16* src = isP ? sm.a.kq.Q : sm.a.kq.K;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) ao[kk] = lds_nat(src, 16 * mi + r16, LDK, 32 * kk, grp);
      } else {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) ao[kk] = bk[kk];
      }
      // this tile's row gates, also in flight over the products
      const f32x4 gr4 = *reinterpret_cast<const f32x4*>(&sm.gam2[16 * mi + 4 * grp]);
      const f32x4 br4 = *reinterpret_cast<const f32x4*>(&sm.bet[16 * mi + 4 * grp]);
      const float gr1 = sm.gam2[16 * mi + r16];
      f32x4 acc = zero4();
      if (!isP) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) acc = mfma(ao[kk], bk[kk], acc);
        const int cj = 16 * mj + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * mi + 4 * grp + i;
          const float e = fexp2(gr4[i] - gj);
          const float lv = row > cj ? br4[i] * acc[i] * e : 0.f;
          sm.Lm()[row * LS + cj] = lv;
          if (mi == mj) sm.Ld[mi][(4 * grp + i) * 16 + r16] = lv;   // aligned copy for the substitution
        }
      } else {
        // P^T tile (K_mj Q_mi^T): the lane holds P[16 mi + r16][16 mj + 4 grp + i],
        // four consecutive columns, so hi and lo go out as 8-byte writes
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) acc = mfma(bk[kk], ao[kk], acc);
        const int row = 16 * mi + r16, c0 = 16 * mj + 4 * grp;
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[i] = row >= c0 + i ? acc[i] * fexp2(gr1 - gc[i]) : 0.f;
        // to the LDS P planes, copied out during the solve
        auto put = [&](int plane, u32x2 v) {
          *reinterpret_cast<u32x2*>(sm.Pl(plane) + r64_off(row, pperm(c0))) = v;
        };
        if (a.w_img_bytes) {
          // one fp16 plane (11-bit significand: relative error <= 2^-12). Its
          // range is +-65504: an entry beyond it (|q . k| that large, which
          // L2-normalised q and k never reach) raises a device error flag
          // instead of passing an infinity on silently
          if (fmaxf(fmaxf(fabsf(pv[0]), fabsf(pv[1])), fmaxf(fabsf(pv[2]), fabsf(pv[3]))) > 65504.f)
            __hip_atomic_fetch_or(a.err, kErrPRange, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
          const f16x4 h = f16x4{(_Float16)pv[0], (_Float16)pv[1], (_Float16)pv[2], (_Float16)pv[3]};
          put(0, __builtin_bit_cast(u32x2, h));
        } else {
          bf16 hi[4], lo[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) split2(pv[i], hi[i], lo[i]);
          put(0, __builtin_bit_cast(u32x2, bf16x4{hi[0], hi[1], hi[2], hi[3]}));
          put(1, __builtin_bit_cast(u32x2, bf16x4{lo[0], lo[1], lo[2], lo[3]}));
        }
      }
    }
    }
    lds_barrier();
    GDN_REFRESH();

    // ---- 3. wave 0: diagonal blocks of X; others: V^T in, the P image out,
    // and (full layout) X's upper blocks zero and the K^T image out; in the
    // compact layout every wave writes its part of K^T (the K, Q rows are
    // dead) and the diagonal blocks go to Y (the P planes are in X's place)
    // (the approximate-inverse instantiation skips the solve's arithmetic here
    // and in the merges below, keeping their loads and barriers: X is formed
    // from L after this phase)
    if constexpr (Sm::TWO) ks.template store_t<true>(sm.Kt(), nullptr, wave, lane);   // copied out in the merges
    if (wave == 0) {
      if constexpr (!NEU) {
      // lane (b, cc): column cc of the inverse of diagonal block b, by rows;
      // row r of the block is read as 16-byte pieces (all 16 lanes of a
      // block read the same row), independent of the substitution itself
      const int b = lane >> 4, cc = lane & 15;
      const f32x4* Lr = reinterpret_cast<const f32x4*>(&sm.Ld[b][0]);
      float x[16];
      // rows go through a two-row-ahead register ring, so LDS latency overlaps
      // the substitution instead of being paid row by row
      f32x4 ring[3][4];
      auto fetch = [&](int r, f32x4 (&dst)[4]) {
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4)
          if (j4 < (r + 3) / 4) dst[j4] = Lr[r * 4 + j4];
      };
      fetch(1, ring[1]);
      fetch(2, ring[2]);
      x[0] = cc == 0 ? 1.f : 0.f;
#pragma unroll
      for (int r = 1; r < 16; ++r) {
        if (r + 2 < 16) fetch(r + 2, ring[(r + 2) % 3]);
        float s = (r == cc) ? 1.f : 0.f;
#pragma unroll
        for (int j4 = 0; j4 < (r + 3) / 4; ++j4) {
          const f32x4 l = ring[r % 3][j4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * j4 + e < r) s -= l[e] * x[4 * j4 + e];
        }
        x[r] = s;
      }
      // (compact layout: to Y, as the P planes in X's place are being copied
      // out; X gets them in the 16-block merge phase)
      if constexpr (Sm::TWO) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.Ym()[kDiagY * b + 16 * r + cc] = x[r];
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.Xm()[(16 * b + r) * LS + 16 * b + cc] = x[r];
      }
      }
    } else {
      const int t = tid - 64;
      if constexpr (!Sm::TWO) {
        // K^T and P images: 16-byte copies of the LDS tiles (adjacent in the
        // image, as they are in LDS), fixed trip counts
        static_assert(sizeof(sm.c.P) == 2 * I::P1 * 2, "P tile is the image's P section");
        constexpr int NKP = (I::KT + 2 * I::P1) / 8, NCP = (NKP + NT - 65) / (NT - 64);
        // one P plane in the byte variant: its second slot holds the gate block
        const int nkp = a.w_img_bytes ? (I::KT + I::P1) / 8 : NKP;
        const u32x4* ksrc = reinterpret_cast<const u32x4*>(sm.Kt());
        const u32x4* psrc = reinterpret_cast<const u32x4*>(&sm.c.P[0][0]);
        u32x4* kdst = reinterpret_cast<u32x4*>(img + I::template kt_at<NW>());
        const bool coh = a.flags != nullptr;
#pragma unroll
        for (int k = 0; k < NCP; ++k) {
          const int e = t + (NT - 64) * k;
          if (e < nkp) st_out16(kdst, 16 * e, e < I::KT / 8 ? ksrc[e] : psrc[e - I::KT / 8], coh);
        }
      } else {
        // P image: 16-byte copies of the LDS planes (one plane in the byte
        // variant, whose second slot holds the gate block); then, once all
        // seven waves have read theirs, X's upper blocks go over them
        constexpr int NPC = 2 * I::P1 / 8, NCP = (NPC + NT - 65) / (NT - 64);
        const int npc = a.w_img_bytes ? I::P1 / 8 : NPC;
        const u32x4* psrc = reinterpret_cast<const u32x4*>(sm.Pl(0));
        const bool coh = a.flags != nullptr;
#pragma unroll
        for (int k = 0; k < NCP; ++k) {
          const int e = t + (NT - 64) * k;
          if (e < npc) st_out16(img + I::template p_at<NW>(), 16 * e, psrc[e], coh);
        }
      }
      if constexpr (!Sm::TWO) {
        for (int e = t; e < 6 * 256; e += NT - 64) {  // upper blocks (bi < bj) of X
          const int blk = e >> 8, r = (e >> 4) & 15, cc = e & 15;
          const int bi = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
          const int bj = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
          sm.Xm()[(16 * bi + r) * LS + 16 * bj + cc] = 0.f;
        }
      }
      vs.store_t(sm.Vt(), nullptr, wave, lane);   // V^T for U
    }
    lds_barrier();
    GDN_REFRESH();
    if (wave == 0) vs.store_t(sm.Vt(), nullptr, wave, lane);
    // The next item's loads are issued where most waves have no other work
    // (issue stalls while the CU's memory path is busy): K, Q, g, beta here,
    // the merging waves after their merge; V in the X_BA phase. Every
    // register they fill has been written out to LDS by now.
    const bool merger = wave == 1 || wave == 2;
    if (nxt.valid && !merger) load_kqg(nxt);
    // 16-block merges X_BA = -X_BB (L_BA X_AA), (A, B) = (0, 1) and (2, 3)
    if (merger) {
      if constexpr (!NEU) {
        const int A = 2 * (wave - 1), B = A + 1;
        // the diagonal blocks X_AA, X_BB: in Y (row stride 16) in the compact
        // layout, in X otherwise
        const float* xaa = Sm::TWO ? &sm.Ym()[kDiagY * A] : &sm.Xm()[(16 * A) * LS + 16 * A];
        const float* xbb = Sm::TWO ? &sm.Ym()[kDiagY * B] : &sm.Xm()[(16 * B) * LS + 16 * B];
        const int xs = Sm::TWO ? 16 : LS;
        const f32x4 y = mm32(&sm.Lm()[(16 * B) * LS + 16 * A], LS, xaa, xs, 0, 0, 0, 16, r16, grp, zero4());
        f32x4 z = zero4();
#pragma unroll
        for (int i = 0; i < 4; ++i)               // K order 4 grp + i
          z = mfma_f32(xbb[r16 * xs + 4 * grp + i], y[i], z);
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.Xm()[(16 * B + 4 * grp + i) * LS + 16 * A + r16] = -z[i];
      }
      if (nxt.valid) load_kqg(nxt);
    } else if constexpr (Sm::TWO) {
      const int t = wave == 0 ? lane : tid - 128;   // the six other waves
      // X: its diagonal blocks from Y, its upper blocks (bi < bj) zero
      for (int e = t; e < 10 * 256; e += 384) {
        const int blk = e >> 8, r = (e >> 4) & 15, cc = e & 15;
        if (blk < 4) {
          sm.Xm()[(16 * blk + r) * LS + 16 * blk + cc] = sm.Ym()[kDiagY * blk + 16 * r + cc];
        } else {
          const int u = blk - 4;
          const int bi = u < 3 ? 0 : (u < 5 ? 1 : 2);
          const int bj = u < 3 ? u + 1 : (u < 5 ? u - 1 : 3);
          sm.Xm()[(16 * bi + r) * LS + 16 * bj + cc] = 0.f;
        }
      }
      // K^T image: 16-byte copies of the LDS tile
      constexpr int NKT = I::KT / 8, NCK = (NKT + 383) / 384;
      const u32x4* ksrc = reinterpret_cast<const u32x4*>(sm.Kt());
      const bool coh = a.flags != nullptr;
#pragma unroll
      for (int k = 0; k < NCK; ++k) {
        const int e = t + 384 * k;
        if (e < NKT) st_out16(img + I::template kt_at<NW>(), 16 * e, ksrc[e], coh);
      }
    }
    lds_barrier();
    GDN_REFRESH();
    // 32-block merge, Y = L_BA X_AA: each 16x16 tile of Y is split over two
    // waves along its K range (the first writes, the second adds after a barrier)
    {
      const int t4 = wave & 3, ti = t4 >> 1, tj = t4 & 1, kh = wave >> 2;
      const int k0 = 16 * tj, km = 16 + 8 * tj;    // X_AA rows < 16 tj are zero in column tile tj
      f32x4 y = zero4();
      float* yp = &sm.Ym()[(16 * ti + 4 * grp) * 33 + 16 * tj + r16];
      if constexpr (!NEU) {
        y = mm32(&sm.Lm()[32 * LS], LS, sm.Xm(), LS, 16 * ti, 16 * tj, kh ? km : k0, kh ? 32 : km,
                 r16, grp, zero4());
        if (kh == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) yp[i * 33] = y[i];
        }
      }
      lds_barrier();
      if (!NEU && kh == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) yp[i * 33] += y[i];
      }
    }
    lds_barrier();
    GDN_REFRESH();
    // X_BA = -X_BB Y (one 16x16 tile per wave 0..3; waves 4..7 issue their V loads first)
    if (wave >= 4 && nxt.valid) load_v(nxt);
    if (wave < 4) {
      if constexpr (!NEU) {
        const int ti = wave >> 1, tj = wave & 1;
        const f32x4 z = mm32(&sm.Xm()[32 * LS + 32], LS, sm.Ym(), 33, 16 * ti, 16 * tj, 0,
                             16 * ti + 16, r16, grp, zero4());
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.Xm()[(32 + 16 * ti + 4 * grp + i) * LS + 16 * tj + r16] = -z[i];
      }
      if (nxt.valid) load_v(nxt);
    }
    lds_barrier();
    GDN_REFRESH();

    // Opt-in approximate inverse: X = sum_{m <= d} (-L)^m, d = 2^j - 1 (the
    // library admits no other degree), in place of the exact solve. The
    // polynomial is the product (I - L)(I + L^2)(I + L^4)...: with P =
    // (-L)^(2^i), each step squares P and sets X <- X + X P. The factors are
    // lower triangular, so an output tile (ti, tj), ti >= tj, sums the key
    // blocks tj..ti only; upper tiles of X are written as zero, those of P are
    // never read. FP32 MFMA; four 64 x 64 buffers rotate: L, X and the two
    // extra ones of this instantiation.
    if constexpr (NEU) {
      static_assert(!Sm::TWO, "the approximate inverse runs in the full layout");
      float* const C0 = sm.c.C[0];
      auto buf = [&](int b) -> float* {
        return b == 0 ? sm.Lm() : (b == 1 ? sm.Xm() : (b == 2 ? C0 : sm.c.C[1]));
      };
      for (int e = tid; e < 64 * 64; e += NT) {
        const int i = e >> 6, j = e & 63;
        const float l = (i >> 4) >= (j >> 4) ? sm.Lm()[i * LS + j] : 0.f;   // strict lower (masked)
        C0[i * LS + j] = -l;
        sm.Xm()[i * LS + j] = j > i ? 0.f : (i == j ? 1.f : -l);
      }
      lds_barrier();
      int ip = 2, ix = 1;                          // P = -L in buffer 2, X = I - L in buffer 1
      for (int d = 1; d < a.solve_degree; d = 2 * d + 1) {
        const int np = ip == 2 ? 0 : 2, nx = ix == 1 ? 3 : 1;
        const float* P = buf(ip);
        float* Pn = buf(np);
        int ti[2], tj[2];
        lower_tiles(wave, ti, tj);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          if (ti[hh] >= tj[hh]) {
            const f32x4 z = mm_lower<LS>(P, P, ti[hh], tj[hh], r16, grp, zero4());
#pragma unroll
            for (int i = 0; i < 4; ++i) Pn[(16 * ti[hh] + 4 * grp + i) * LS + 16 * tj[hh] + r16] = z[i];
          }
        }
        lds_barrier();
        const float* X = buf(ix);
        float* Xn = buf(nx);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          f32x4 z = zero4();
          if (ti[hh] >= tj[hh]) {
#pragma unroll
            for (int i = 0; i < 4; ++i) z[i] = X[(16 * ti[hh] + 4 * grp + i) * LS + 16 * tj[hh] + r16];
            z = mm_lower<LS>(X, Pn, ti[hh], tj[hh], r16, grp, z);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) Xn[(16 * ti[hh] + 4 * grp + i) * LS + 16 * tj[hh] + r16] = z[i];
        }
        lds_barrier();
        ip = np;
        ix = nx;
      }
      if (ix != 1) {                               // an odd number of steps leaves X in buffer 3
        const float* X = buf(ix);
        for (int e = tid; e < 64 * 64; e += NT) {
          const int i = e >> 6, j = e & 63;
          sm.Xm()[i * LS + j] = X[i * LS + j];
        }
        lds_barrier();
      }
      GDN_REFRESH();
    }

    // X for the backward (saved buffer), row-major FP32
    if (a.s_X) {
      float* xg = a.s_X + ch * 4096;
      for (int e = tid; e < 1024; e += NT) {
        const int row = e >> 4, c4 = e & 15;
        const float* xs = &sm.Xm()[row * LS + 4 * c4];
        *reinterpret_cast<f32x4*>(xg + row * 64 + 4 * c4) = f32x4{xs[0], xs[1], xs[2], xs[3]};
      }
    }
    // ---- 4. T = X diag(beta), T' = T diag(exp(gamma)) as hi / lo planes (pperm
    // over columns). In the compact layout T' goes over L (dead since the
    // merges) and T over X once every wave has read its part of X.
    {
      const int row = tid >> 3, q = tid & 7;
      bf16 th[2][4], tl[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int c0 = 8 * q + 4 * u;
        const f32x4 b4 = *reinterpret_cast<const f32x4*>(&sm.bet[c0]);
        const f32x4 e4 = *reinterpret_cast<const f32x4*>(&sm.eg[c0]);
        float xv[4];
        if constexpr (Sm::TWO) {
          const f32x4 x4 = *reinterpret_cast<const f32x4*>(&sm.Xm()[row * LS + c0]);
#pragma unroll
          for (int e = 0; e < 4; ++e) xv[e] = x4[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) xv[e] = sm.Xm()[row * LS + c0 + e];
        }
        bf16 ph[4], pl[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float t = xv[e] * b4[e];
          split2(t, th[u][e], tl[u][e]);
          split2(t * e4[e], ph[e], pl[e]);
        }
        const int o = Sm::t_off(row, c0);
        if constexpr (!Sm::TWO) {
          st4(sm.Tt(0) + o, th[u][0], th[u][1], th[u][2], th[u][3]);
          st4(sm.Tt(1) + o, tl[u][0], tl[u][1], tl[u][2], tl[u][3]);
        }
        st4(sm.Tp(0) + o, ph[0], ph[1], ph[2], ph[3]);
        st4(sm.Tp(1) + o, pl[0], pl[1], pl[2], pl[3]);
      }
      if constexpr (Sm::TWO) {
        lds_barrier();
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int o = Sm::t_off(row, 8 * q + 4 * u);
          st4(sm.Tt(0) + o, th[u][0], th[u][1], th[u][2], th[u][3]);
          st4(sm.Tt(1) + o, tl[u][0], tl[u][1], tl[u][2], tl[u][3]);
        }
      }
    }
    lds_barrier();
    GDN_REFRESH();

    // ---- 5. W = T' K (row tile wave & 3, column-tile half wave >> 2), U = T V; QDQ of W
    const int mt = wave & 3, ct0 = (wave >> 2) * NCTW;
    f32x4 Wt[NCTW];
    {
      bf16x8 ah[2], al[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        ah[kk] = Sm::t_frag(sm.Tp(0), 16 * mt + r16, kk, grp);
        al[kk] = Sm::t_frag(sm.Tp(1), 16 * mt + r16, kk, grp);
      }
      // computed transposed (W^T = K^T T'^T, the same fragments with A and B
      // swapped): a lane then holds four adjacent dk of one token, which go
      // to LDS as one 8-byte write
#pragma unroll
      for (int d = 0; d < NCTW; ++d) {
        const int ct = ct0 + d;
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (kk > mt / 2) continue;              // T' is lower triangular
          const bf16x8 b = ld_r64(sm.Kt(), 16 * ct + r16, 32 * kk, grp);
          acc = mfma(b, ah[kk], acc);
          acc = mfma(b, al[kk], acc);
        }
        Wt[d] = acc;                              // W[16 mt + r16][16 ct + 4 grp + i]
      }
    }
    if constexpr (WF != 0) {
      float m = 0.f;
#pragma unroll
      for (int d = 0; d < NCTW; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(Wt[d][i]));
      m = wave_max(m);
      if (lane == 0) sm.red[wave] = m;
    }
    // U tiles (m, 4 vb + (wave & 3)) for the value blocks vb of parity wave >> 2,
    // written straight out in fragment order
    {
      const int w4 = wave & 3;
      bf16x8 th[4][2], tl[4][2];
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (kk > m / 2) continue;
          th[m][kk] = Sm::t_frag(sm.Tt(0), 16 * m + r16, kk, grp);
          tl[m][kk] = Sm::t_frag(sm.Tt(1), 16 * m + r16, kk, grp);
        }
      for (int vb = wave >> 2; vb < NVB; vb += 2) {
        const int ct = 4 * vb + w4;
        bf16x8 vbk[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) vbk[kk] = lds_nat(sm.Vt(), 16 * ct + r16, 72, 32 * kk, grp);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          f32x4 acc = zero4();
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            if (kk > m / 2) continue;
            acc = mfma(th[m][kk], vbk[kk], acc);
            acc = mfma(tl[m][kk], vbk[kk], acc);
          }
          st_out16(a.ws_u + u_off(ch, NVB, vb, w4, m, 0), 16 * lane, __builtin_bit_cast(u32x4, acc),
                   a.flags != nullptr);
        }
      }
    }
    lds_barrier();                              // W amax partials; K^T, V^T, T dead
    GDN_REFRESH();
    {
      float dW = 1.f, rW = 1.f;
      if constexpr (WF != 0) {
        static_assert(NWAVE == 8, "two 4-wide reads of the partial maxima");
        const f32x4 r0 = *reinterpret_cast<const f32x4*>(&sm.red[0]);
        const f32x4 r1 = *reinterpret_cast<const f32x4*>(&sm.red[4]);
        float amax = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) amax = fmaxf(amax, fmaxf(r0[w], r1[w]));
        dW = qdq_scale<WF>(amax);
        rW = 1.0f / dW;
      }
      const bool save = WF != 0 && a.w_codes != nullptr;
      const int tok = 16 * mt + r16;
#pragma unroll
      for (int d = 0; d < NCTW; ++d) {
        const int dk0 = 16 * (ct0 + d) + 4 * grp, o = wq_off<DK>(tok, pperm(dk0));   // dk0..dk0 + 3 adjacent
        const float w[4] = {Wt[d][0], Wt[d][1], Wt[d][2], Wt[d][3]};
        if constexpr (WF != 0) {
          float cq[4];
          uint32_t bytes;
          quant4<WF>(w, rW, cq, bytes);
          if (a.w_img_bytes)                      // the code bytes, same element order
            *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(sm.Wm()) + o) = bytes;
          else
            st4(sm.Wm() + o, to_bf16(cq[0]), to_bf16(cq[1]), to_bf16(cq[2]), to_bf16(cq[3]));
          if (save && tok < nc)
            *reinterpret_cast<uint32_t*>(a.w_codes + ((int64_t)(t0 + tok) * Hv + h) * DK + dk0) = bytes;
        } else {
          bf16 hi[4], lo[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) split2(w[i], hi[i], lo[i]);
          st4(sm.Wm() + o, hi[0], hi[1], hi[2], hi[3]);
          st4(sm.Wm() + I::WQ + o, lo[0], lo[1], lo[2], lo[3]);
        }
      }
      if (tid == 0) {
        st_out(a.ws_wscale + ch, dW, a.flags != nullptr);
        const int goff = a.w_img_bytes ? I::template p_at<NW>() + I::P1 : I::template g_at<NW>();
        st_out(reinterpret_cast<float*>(img + goff) + 129, dW, a.flags != nullptr);
        if (save) a.w_scale[ch] = dW;
      }
    }
    lds_barrier();
    GDN_REFRESH();
    {
      const u32x4* src = reinterpret_cast<const u32x4*>(sm.Wm());
      u32x4* dst = reinterpret_cast<u32x4*>(img);
      constexpr int NWP = NW * I::WQ / 8;          // 16-byte pieces of the W planes
      constexpr int NWB = I::WQ / 16;              // ... of the code bytes
      const bool coh = a.flags != nullptr;
      if (WF != 0 && a.w_img_bytes) {
#pragma unroll
        for (int k = 0; k < (NWB + NT - 1) / NT; ++k)
          if (NWB % NT == 0 || tid + NT * k < NWB) st_out16(dst, 16 * (tid + NT * k), src[tid + NT * k], coh);
      } else {
#pragma unroll
        for (int k = 0; k < (NWP + NT - 1) / NT; ++k)
          if (NWP % NT == 0 || tid + NT * k < NWP) st_out16(dst, 16 * (tid + NT * k), src[tid + NT * k], coh);
      }
    }
    // publishing to a concurrent state kernel: every wave waits for its
    // device-scope stores of this item, then after the barrier one flag store
    if (a.flags) vm_drain();
    lds_barrier();                              // LDS is reused by the next item
    if (a.flags && tid == 0)
      __hip_atomic_store(a.flags + (int64_t)cur.slot * Hv + h, 1u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    if (!nxt.valid) break;
    cur = nxt;
  }
#undef GDN_REFRESH
}

}  // namespace

// Compute units of the current device (queried once per device).
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

template <int DK, int DV, int WF>
static hipError_t launch_prep_one(const FwdConfig& cfg, const FwdKernelArgs& a, int num_slots,
                                  hipStream_t s, hipEvent_t stop) {
  const int64_t items = a.item_hi > 0 ? (int64_t)a.item_hi - a.item_lo : (int64_t)num_slots * cfg.Hv;
  // The compact layout, two workgroups per CU, where it fits (Dv <= 128,
  // exact solve), on its own and beside the state kernel with the CU
  // admission table; else the full layout, one per CU (beside the state
  // kernel the workgroups that end after the head then free whole CUs).
  const bool neu = a.solve_degree > 0;
  const bool cmp = !neu && prep_fits_two<DK, DV>() && !(a.ticket != nullptr && !a.admit);
  const int64_t cap = a.prep_blocks > 0 ? a.prep_blocks : (cmp ? 2 : 1) * (int64_t)device_cus();
  const int64_t nblk = items < cap ? items : cap;
  if (nblk <= 0) return stop ? hipEventRecord(stop, s) : hipSuccess;
  const dim3 grid((unsigned)nblk), block(NT);
  auto go = [&](auto kernel) {
    if (stop)
      hipExtLaunchKernelGGL(kernel, grid, block, 0, s, nullptr, stop, 0, a, cfg.N, num_slots);
    else
      hipLaunchKernelGGL(kernel, grid, block, 0, s, a, cfg.N, num_slots);
  };
  if (neu) {
    go(gdn_prep_kernel<DK, DV, WF, true, false>);
  } else if (cmp) {
    if constexpr (prep_fits_two<DK, DV>()) go(gdn_prep_kernel<DK, DV, WF, false, true>);
  } else {
    go(gdn_prep_kernel<DK, DV, WF, false, false>);
  }
  return hipGetLastError();
}

template <int DK, int DV>
static int prep_per_cu_dk_dv(int solve_degree) {
  return solve_degree == 0 && prep_fits_two<DK, DV>() ? 2 : 1;
}

int prep_workgroups_per_cu(const FwdConfig& cfg, int solve_degree) {
  if (cfg.Dk == 128) {
    if (cfg.Dv == 64) return prep_per_cu_dk_dv<128, 64>(solve_degree);
    if (cfg.Dv == 128) return prep_per_cu_dk_dv<128, 128>(solve_degree);
    if (cfg.Dv == 256) return prep_per_cu_dk_dv<128, 256>(solve_degree);
  } else if (cfg.Dk == 64) {
    if (cfg.Dv == 64) return prep_per_cu_dk_dv<64, 64>(solve_degree);
    if (cfg.Dv == 128) return prep_per_cu_dk_dv<64, 128>(solve_degree);
    if (cfg.Dv == 256) return prep_per_cu_dk_dv<64, 256>(solve_degree);
  }
  return 1;
}

template <int DK, int DV>
static hipError_t launch_prep_w(const FwdConfig& cfg, const FwdKernelArgs& a, int ns, hipStream_t s,
                                hipEvent_t stop) {
  if (cfg.w_fmt == 0) return launch_prep_one<DK, DV, 0>(cfg, a, ns, s, stop);
  if (cfg.w_fmt == 1) return launch_prep_one<DK, DV, 1>(cfg, a, ns, s, stop);
  if (cfg.w_fmt == 2) return launch_prep_one<DK, DV, 2>(cfg, a, ns, s, stop);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_prep(const FwdConfig& cfg, const FwdKernelArgs& a, int num_slots,
                           hipStream_t s, hipEvent_t stop) {
  if (cfg.Dk == 128) {
    if (cfg.Dv == 64) return launch_prep_w<128, 64>(cfg, a, num_slots, s, stop);
    if (cfg.Dv == 128) return launch_prep_w<128, 128>(cfg, a, num_slots, s, stop);
    if (cfg.Dv == 256) return launch_prep_w<128, 256>(cfg, a, num_slots, s, stop);
  } else if (cfg.Dk == 64) {
    if (cfg.Dv == 64) return launch_prep_w<64, 64>(cfg, a, num_slots, s, stop);
    if (cfg.Dv == 128) return launch_prep_w<64, 128>(cfg, a, num_slots, s, stop);
    if (cfg.Dv == 256) return launch_prep_w<64, 256>(cfg, a, num_slots, s, stop);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
