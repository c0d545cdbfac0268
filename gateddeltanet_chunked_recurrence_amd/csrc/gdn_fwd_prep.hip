// Forward, part 1: the state-independent work of every (chunk, value head),
// one workgroup each, all chunks in parallel ("[1/4] GDN state/W QAT
// foundation", "What does this PR do?": exact triangular solve, W and its
// dynamic QDQ, the saved quantized W).
//
// Per chunk of n <= 64 tokens (rows past n are zero):
//   gamma = chunk-local cumsum of g;  Gam_ij = exp(gamma_i - gamma_j), i >= j
//   L = beta_i (K K^T)_ij Gam_ij (i > j);  P = (Q K^T) * Gam (i >= j)
//   X = (I + L)^-1: 16x16 diagonal blocks by substitution, then the 16- and
//       32-block merges X_BA = -X_BB L_BA X_AA (FP32 MFMA)
//   T = X diag(beta);  T' = T diag(exp(gamma))
//   W = T' K, QDQ_W over the [n, Dk] tile;  U = T V
// Outputs are the operand images described in gdn_images.h, plus the W codes
// and scale in the caller's saved buffer when it asks for them.
//
// Precision: q, k, v are bf16 and exact as MFMA operands; T and T' (FP32) are
// split as hi + lo bf16 (two passes), so W and U carry ~16 mantissa bits of T
// with FP32 accumulation. L, X and the merges stay FP32 throughout.
#include "gdn_device.h"
#include "gdn_images.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

constexpr int NT = 256;
constexpr float LOG2E = 1.4426950408889634f;

template <int DK>
struct PrepSmem {
  static constexpr int LDK = DK + 8;             // K, Q rows (pperm over dk)
  union {
    struct { bf16 K[64 * LDK]; bf16 Q[64 * LDK]; } kq;   // until the L / P tiles
    bf16 Vt[256 * 72];                                    // V^T (pperm over tokens)
  } a;
  bf16 Kt[DK * 72];                              // K^T (pperm over tokens)
  union {
    struct { float L[64 * 65]; float X[64 * 65]; } s;    // solve
    bf16 W[2 * Img<DK>::WQ];                              // W image planes
  } b;
  union {
    bf16 P[2][64 * 72];                          // P hi / lo, until copied out
    float Y[32 * 33];                            // 32-block merge scratch
    bf16 T[4][64 * 72];                          // T hi, T lo, T' hi, T' lo
  } c;
  alignas(16) float gam2[64];                    // log2-scaled gamma
  alignas(16) float bet[64];
  alignas(16) float eg[64];                      // exp(gamma)
  float red[4];
};

// Lower 16x16 tiles (mi >= mj) of a 64x64 matrix in a fixed order.
__device__ __forceinline__ void lower_tile(int t, int& mi, int& mj) {
  mi = (t >= 1) + (t >= 3) + (t >= 6);
  mj = t - (mi * (mi + 1)) / 2;
}

// One 16x16 tile (mi, mj) of A B^T for [64][DK] bf16 row tiles in LDS (row
// stride LD, same K order in both), operands loaded before the MFMA chain.
template <int DK, int LD>
__device__ __forceinline__ f32x4 tile_abt(const bf16* A, const bf16* B, int mi, int mj, int r16,
                                          int grp) {
  constexpr int KS = DK / 32;
  bf16x8 a[KS], b[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    a[kk] = lds_nat(A, 16 * mi + r16, LD, 32 * kk, grp);
    b[kk] = lds_nat(B, 16 * mj + r16, LD, 32 * kk, grp);
  }
  f32x4 acc = zero4();
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) acc = mfma(a[kk], b[kk], acc);
  return acc;
}

// acc += A(i0 + r, k) B(k, j0 + c) over k in [k0, k1) (FP32 MFMA 16x16x4),
// A(i, k) = A[i * ars + k], B(k, j) = B[k * brs + j].
__device__ __forceinline__ f32x4 mm32(const float* A, int ars, const float* B, int brs, int i0,
                                      int j0, int k0, int k1, int r16, int grp, f32x4 acc) {
  for (int k = k0; k < k1; k += 4)
    acc = mfma_f32(A[(i0 + r16) * ars + k + grp], B[(k + grp) * brs + j0 + r16], acc);
  return acc;
}

// Writes 4 consecutive bf16 at dst (8-byte aligned).
__device__ __forceinline__ void st4(bf16* dst, bf16 a, bf16 b, bf16 c, bf16 d) {
  *reinterpret_cast<bf16x4*>(dst) = bf16x4{a, b, c, d};
}

// Stages a [64 tokens][D] bf16 tile (rows past nc = 0) transposed into
// dst[D][72] with the token index in pperm order. Thread layout: TPG tokens x
// 8 columns per thread, token groups fastest within a wave, so the 16 or 32
// lanes of one column group write one LDS row.
template <int D>
struct TransposeStage {
  static constexpr int TPG = D / 32;             // tokens per thread (2, 4 or 8)
  static constexpr int NTG = 64 / TPG;           // token groups
  bf16x8 raw[TPG];
  int tg, c8;
  __device__ void load(const bf16* src, int64_t row_stride, int nc, int wave, int lane) {
    tg = lane % NTG;
    c8 = lane / NTG + (64 / NTG) * wave;
    // unconditional loads (clamped row) then a select: no divergent branch
    // around the loads, so they are issued back to back
#pragma unroll
    for (int p = 0; p < TPG; ++p) {
      const int row = TPG * tg + p;
      const uint4 v = *reinterpret_cast<const uint4*>(src + min(row, nc - 1) * row_stride + 8 * c8);
      const uint4 z = make_uint4(0, 0, 0, 0);
      const uint4 w = row < nc ? v : z;
      raw[p] = *reinterpret_cast<const bf16x8*>(&w);
    }
  }
  // dst[(8 c8 + j) * 72 + pperm(token)] for this thread's tokens; also to gdst if given
  __device__ void store_t(bf16* dst, bf16* gdst) const {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int u = 0; u < (TPG + 3) / 4; ++u) {
        const int tok0 = TPG * tg + 4 * u;
        const int off = (8 * c8 + j) * 72 + pperm(tok0);
        if constexpr (TPG == 2) {
          typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
          const bf16x2 v = bf16x2{raw[0][j], raw[1][j]};
          *reinterpret_cast<bf16x2*>(dst + off) = v;
          if (gdst) *reinterpret_cast<bf16x2*>(gdst + off) = v;
        } else {
          const bf16x4 v = bf16x4{raw[4 * u][j], raw[4 * u + 1][j], raw[4 * u + 2][j], raw[4 * u + 3][j]};
          *reinterpret_cast<bf16x4*>(dst + off) = v;
          if (gdst) *reinterpret_cast<bf16x4*>(gdst + off) = v;
        }
      }
    }
  }
  // row-major dst[token * ld + pperm(col)] (two 4-element units per row)
  __device__ void store_rows(bf16* dst, int ld) const {
#pragma unroll
    for (int p = 0; p < TPG; ++p) {
      bf16* d = dst + (TPG * tg + p) * ld;
      const bf16x8& r = raw[p];
      st4(d + pperm(8 * c8), r[0], r[1], r[2], r[3]);
      st4(d + pperm(8 * c8 + 4), r[4], r[5], r[6], r[7]);
    }
  }
};

template <int DK, int DV, int WF>
__global__ void __launch_bounds__(NT, 1) gdn_prep_kernel(FwdKernelArgs a, int N, int num_slots) {
  using I = Img<DK>;
  constexpr int LDK = PrepSmem<DK>::LDK;
  constexpr int NW = WF == 0 ? 2 : 1;
  constexpr int NCT = DK / 16;                    // column tiles of W
  constexpr int NVB = DV / 64;
  __shared__ __align__(16) PrepSmem<DK> sm;

  const int h = blockIdx.x % a.Hv, slot = blockIdx.x / a.Hv;
  if (slot >= num_slots) return;
  // chunk of this slot (slot = n + bos_n / 64 + c, increasing in n)
  int n = 0;
  {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      const int bos = a.cu_seqlens ? a.cu_seqlens[mid] : mid * a.T;
      if (mid + bos / CHUNK <= slot) lo = mid; else hi = mid - 1;
    }
    n = lo;
  }
  const int bos = a.cu_seqlens ? a.cu_seqlens[n] : n * a.T;
  const int eos = a.cu_seqlens ? a.cu_seqlens[n + 1] : (n + 1) * a.T;
  const int c = slot - (n + bos / CHUNK);
  const int t0 = bos + CHUNK * c;
  if (c < 0 || t0 >= eos) return;                 // slot used by no chunk
  const int nc = min(CHUNK, eos - t0);
  const int Hv = a.Hv, Hqk = a.Hqk, hk = h / (Hv / Hqk);
  const int64_t ch = (int64_t)slot * Hv + h;
  bf16* img = a.ws_img + ch * I::template img<NW>();   // [W planes | K^T | P]

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = __lane_id(), tid = wave * 64 + lane, r16 = lane & 15, grp = lane >> 4;

  // ---- 1. stage K, Q (rows, pperm over dk), K^T (LDS + image), gates; V into registers
  const bf16* kp = reinterpret_cast<const bf16*>(a.k) + ((int64_t)t0 * Hqk + hk) * DK;
  const bf16* qp = reinterpret_cast<const bf16*>(a.q) + ((int64_t)t0 * Hqk + hk) * DK;
  const bf16* vp = reinterpret_cast<const bf16*>(a.v) + ((int64_t)t0 * Hv + h) * DV;
  TransposeStage<DK> ks, qs;
  TransposeStage<DV> vs;
  ks.load(kp, (int64_t)Hqk * DK, nc, wave, lane);
  qs.load(qp, (int64_t)Hqk * DK, nc, wave, lane);
  vs.load(vp, (int64_t)Hv * DV, nc, wave, lane);
  float gv, bv;
  {
    const int64_t gi = (int64_t)(t0 + min(lane, nc - 1)) * Hv + h;
    gv = lane < nc ? a.g[gi] : 0.f;
    bv = lane < nc ? a.beta[gi] : 0.f;
  }
  // P upper tiles (0, 1) and (2, 3) are read as zeros by the state kernel
  for (int e = tid; e < 2 * 2 * 256; e += NT) {
    const int pl = e >> 9, t = (e >> 8) & 1, r = (e >> 4) & 15, cc = e & 15;
    sm.c.P[pl][(32 * t + r) * 72 + pperm(32 * t + 16 + cc)] = to_bf16(0.f);
  }
  ks.store_rows(sm.a.kq.K, LDK);
  qs.store_rows(sm.a.kq.Q, LDK);
  ks.store_t(sm.Kt, img + I::template kt_at<NW>());
  if (wave == 0) {
    const float g2 = wave_incl_scan(lane < nc ? gv * LOG2E : 0.f, lane);
    const float g2n = __shfl(g2, nc - 1, WAVE);
    const float eg = fexp2(g2);
    sm.gam2[lane] = g2;
    sm.bet[lane] = bv;
    sm.eg[lane] = eg;
    float* G = reinterpret_cast<float*>(img + I::template g_at<NW>());
    G[lane] = eg;
    G[64 + lane] = lane < nc ? fexp2(g2n - g2) : 0.f;
    G[128 + lane] = lane == 0 ? fexp2(g2n) : 0.f;
    G[192 + lane] = 0.f;
  }
  __syncthreads();

  // ---- 2. L (FP32) and P (hi / lo, pperm over columns): 20 tiles, 5 per wave
#pragma unroll 1
  for (int job = wave; job < 20; job += 4) {
    int mi, mj;
    lower_tile(job % 10, mi, mj);
    const bool isL = job < 10;
    const f32x4 acc = tile_abt<DK, LDK>(isL ? sm.a.kq.K : sm.a.kq.Q, sm.a.kq.K, mi, mj, r16, grp);
    const int cj = 16 * mj + r16;
    const float gj = sm.gam2[cj];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * mi + 4 * grp + i;
      const float e = fexp2(sm.gam2[row] - gj);
      if (isL) {
        sm.b.s.L[row * 65 + cj] = row > cj ? sm.bet[row] * acc[i] * e : 0.f;
      } else {
        const float pv = row >= cj ? acc[i] * e : 0.f;
        bf16 hi, lo;
        split2(pv, hi, lo);
        sm.c.P[0][row * 72 + pperm(cj)] = hi;
        sm.c.P[1][row * 72 + pperm(cj)] = lo;
      }
    }
  }
  __syncthreads();

  // ---- 3. wave 0: diagonal blocks of X; waves 1-3: P image out, X upper zero, V^T in
  if (wave == 0) {
    const int b = lane >> 4, cc = lane & 15;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = (r == cc) ? 1.f : 0.f;
    const float* Lb = &sm.b.s.L[(16 * b) * 65 + 16 * b];
#pragma unroll
    for (int j = 0; j < 15; ++j)
#pragma unroll
      for (int r = j + 1; r < 16; ++r) x[r] -= Lb[r * 65 + j] * x[j];
#pragma unroll
    for (int r = 0; r < 16; ++r) sm.b.s.X[(16 * b + r) * 65 + 16 * b + cc] = x[r];
  } else {
    const int t = tid - 64;                       // 0..191
    const uint4* src = reinterpret_cast<const uint4*>(&sm.c.P[0][0]);
    uint4* dst = reinterpret_cast<uint4*>(img + I::template p_at<NW>());
    for (int e = t; e < 2 * I::P1 / 8; e += NT - 64) dst[e] = src[e];
    for (int e = t; e < 6 * 256; e += NT - 64) {  // upper blocks (bi < bj) of X
      const int blk = e >> 8, r = (e >> 4) & 15, cc = e & 15;
      const int bi = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
      const int bj = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
      sm.b.s.X[(16 * bi + r) * 65 + 16 * bj + cc] = 0.f;
    }
  }
  __syncthreads();
  vs.store_t(sm.a.Vt, nullptr);                   // K, Q rows are dead; V^T for U
  // 16-block merges X_BA = -X_BB (L_BA X_AA), (A, B) = (0, 1) and (2, 3)
  if (wave < 2) {
    const int A = 2 * wave, B = A + 1;
    const f32x4 y = mm32(&sm.b.s.L[(16 * B) * 65 + 16 * A], 65, &sm.b.s.X[(16 * A) * 65 + 16 * A], 65,
                         0, 0, 0, 16, r16, grp, zero4());
    f32x4 z = zero4();
#pragma unroll
    for (int i = 0; i < 4; ++i)                   // K order 4 grp + i
      z = mfma_f32(sm.b.s.X[(16 * B + r16) * 65 + 16 * B + 4 * grp + i], y[i], z);
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.b.s.X[(16 * B + 4 * grp + i) * 65 + 16 * A + r16] = -z[i];
  }
  __syncthreads();
  // 32-block merge: Y = L_BA X_AA, then X_BA = -X_BB Y (one 16x16 tile per wave)
  {
    const int ti = wave >> 1, tj = wave & 1;
    const f32x4 y = mm32(&sm.b.s.L[32 * 65], 65, sm.b.s.X, 65, 16 * ti, 16 * tj, 16 * tj, 32, r16,
                         grp, zero4());
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.c.Y[(16 * ti + 4 * grp + i) * 33 + 16 * tj + r16] = y[i];
  }
  __syncthreads();
  {
    const int ti = wave >> 1, tj = wave & 1;
    const f32x4 z = mm32(&sm.b.s.X[32 * 65 + 32], 65, sm.c.Y, 33, 16 * ti, 16 * tj, 0, 16 * ti + 16,
                         r16, grp, zero4());
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.b.s.X[(32 + 16 * ti + 4 * grp + i) * 65 + 16 * tj + r16] = -z[i];
  }
  __syncthreads();

  // ---- 4. T = X diag(beta), T' = T diag(exp(gamma)) as hi / lo planes (pperm over columns)
  {
    const int row = tid >> 2, q = tid & 3;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c0 = 16 * q + 4 * u;
      bf16 th[4], tl[4], ph[4], pl[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float t = sm.b.s.X[row * 65 + c0 + e] * sm.bet[c0 + e];
        split2(t, th[e], tl[e]);
        split2(t * sm.eg[c0 + e], ph[e], pl[e]);
      }
      const int o = row * 72 + pperm(c0);
      st4(&sm.c.T[0][o], th[0], th[1], th[2], th[3]);
      st4(&sm.c.T[1][o], tl[0], tl[1], tl[2], tl[3]);
      st4(&sm.c.T[2][o], ph[0], ph[1], ph[2], ph[3]);
      st4(&sm.c.T[3][o], pl[0], pl[1], pl[2], pl[3]);
    }
  }
  __syncthreads();

  // ---- 5. W = T' K (row tile = wave), U = T V; QDQ of W
  const int mt = wave;
  f32x4 Wt[NCT];
  {
    bf16x8 ah[2], al[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      ah[kk] = lds_nat(sm.c.T[2], 16 * mt + r16, 72, 32 * kk, grp);
      al[kk] = lds_nat(sm.c.T[3], 16 * mt + r16, 72, 32 * kk, grp);
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (kk > mt / 2) continue;                // T' is lower triangular
        const bf16x8 b = lds_nat(sm.Kt, 16 * ct + r16, 72, 32 * kk, grp);
        acc = mfma(ah[kk], b, acc);
        acc = mfma(al[kk], b, acc);
      }
      Wt[ct] = acc;
    }
  }
  if constexpr (WF != 0) {
    float m = 0.f;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(Wt[ct][i]));
    m = wave_max(m);
    if (lane == 0) sm.red[wave] = m;
  }
  // U tiles (mt, 4 vb + wave), written straight out in fragment order
  {
    bf16x8 th[4][2], tl[4][2];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (kk > m / 2) continue;
        th[m][kk] = lds_nat(sm.c.T[0], 16 * m + r16, 72, 32 * kk, grp);
        tl[m][kk] = lds_nat(sm.c.T[1], 16 * m + r16, 72, 32 * kk, grp);
      }
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
      const int ct = 4 * vb + wave;
      bf16x8 vbk[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) vbk[kk] = lds_nat(sm.a.Vt, 16 * ct + r16, 72, 32 * kk, grp);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (kk > m / 2) continue;
          acc = mfma(th[m][kk], vbk[kk], acc);
          acc = mfma(tl[m][kk], vbk[kk], acc);
        }
        *reinterpret_cast<f32x4*>(a.ws_u + u_off(ch, NVB, vb, wave, m, lane)) = acc;
      }
    }
  }
  __syncthreads();                                // W amax partials; X, L dead
  {
    float dW = 1.f, rW = 1.f;
    if constexpr (WF != 0) {
      dW = qdq_scale<WF>(fmaxf(fmaxf(sm.red[0], sm.red[1]), fmaxf(sm.red[2], sm.red[3])));
      rW = 1.0f / dW;
    }
    const bool save = WF != 0 && a.w_codes != nullptr;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int col = 16 * ct + r16, s = pperm(col);
      const int row0 = 16 * mt + 4 * grp;
      const float w[4] = {Wt[ct][0], Wt[ct][1], Wt[ct][2], Wt[ct][3]};
      if constexpr (WF != 0) {
        float cq[4];
        uint32_t bytes;
        quant4<WF>(w, rW, cq, bytes);
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.b.W[wq_off<DK>(row0 + i, s)] = to_bf16(cq[i]);
        if (save) {
          uint8_t* wp = a.w_codes + ((int64_t)t0 * Hv + h) * DK + col;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (row0 + i < nc) wp[(int64_t)(row0 + i) * Hv * DK] = (bytes >> (8 * i)) & 0xFFu;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bf16 hi, lo;
          split2(w[i], hi, lo);
          sm.b.W[wq_off<DK>(row0 + i, s)] = hi;
          sm.b.W[I::WQ + wq_off<DK>(row0 + i, s)] = lo;
        }
      }
    }
    if (tid == 0) {
      a.ws_wscale[ch] = dW;
      if (save) a.w_scale[ch] = dW;
    }
  }
  __syncthreads();
  {
    const uint4* src = reinterpret_cast<const uint4*>(sm.b.W);
    uint4* dst = reinterpret_cast<uint4*>(img);
    for (int e = tid; e < NW * I::WQ / 8; e += NT) dst[e] = src[e];
  }
}

}  // namespace

template <int DK, int DV, int WF>
static hipError_t launch_prep_one(const FwdConfig& cfg, const FwdKernelArgs& a, int num_slots,
                                  hipStream_t s) {
  const int64_t nblk = (int64_t)num_slots * cfg.Hv;
  hipLaunchKernelGGL((gdn_prep_kernel<DK, DV, WF>), dim3((unsigned)nblk), dim3(NT), 0, s, a, cfg.N,
                     num_slots);
  return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_prep_w(const FwdConfig& cfg, const FwdKernelArgs& a, int ns, hipStream_t s) {
  if (cfg.w_fmt == 0) return launch_prep_one<DK, DV, 0>(cfg, a, ns, s);
  if (cfg.w_fmt == 1) return launch_prep_one<DK, DV, 1>(cfg, a, ns, s);
  if (cfg.w_fmt == 2) return launch_prep_one<DK, DV, 2>(cfg, a, ns, s);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_prep(const FwdConfig& cfg, const FwdKernelArgs& a, int num_slots,
                           hipStream_t s) {
  if (cfg.Dk == 128) {
    if (cfg.Dv == 64) return launch_prep_w<128, 64>(cfg, a, num_slots, s);
    if (cfg.Dv == 128) return launch_prep_w<128, 128>(cfg, a, num_slots, s);
    if (cfg.Dv == 256) return launch_prep_w<128, 256>(cfg, a, num_slots, s);
  } else if (cfg.Dk == 64) {
    if (cfg.Dv == 64) return launch_prep_w<64, 64>(cfg, a, num_slots, s);
    if (cfg.Dv == 128) return launch_prep_w<64, 128>(cfg, a, num_slots, s);
    if (cfg.Dv == 256) return launch_prep_w<64, 256>(cfg, a, num_slots, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
