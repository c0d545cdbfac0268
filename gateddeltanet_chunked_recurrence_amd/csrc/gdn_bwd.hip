// Backward of the chunked gated delta rule with the identity straight-through
// estimator at both QDQ sites ("[1/4] GDN state/W QAT foundation", "What does
// this PR do?": identity STE, the forward's quantized W reused by the
// backward). The forward's quantized values Sq and Wq (saved as one-byte codes
// and scales) are the values used in every product, and their gradients pass
// through unchanged.
//
// Per chunk (forward, see include/gdn.h):
//   Vnew = U - Wq Sq,  U = T V,  W = T diag(e^gamma) K,  T = X diag(beta),
//   X = (I + L)^-1,  L_ij = beta_i (k_i . k_j) Gam_ij (i > j)
//   O = scale (diag(e^gamma) Q Sq + P Vnew),  P = (Q K^T) * Gam (i >= j)
//   S' = e^gamma_n Sq + Kd^T Vnew,  Kd = diag(e^(gamma_n - gamma)) K
// Reverse mode, with dS' the gradient of the state after the chunk:
//   dVnew = scale P^T dO + Kd dS'
//   dS    = e^gamma_n dS' + scale (diag(e^gamma) Q)^T dO - Wq^T dVnew   (STE)
//   dW    = -dVnew Sq^T (STE),  dU = dVnew,  dV = T^T dU
//   dQ    = scale diag(e^gamma) dO Sq^T + G K,      G = scale (dO Vnew^T) * Gam
//   dK    = G^T Q + Kd-term + diag(e^gamma) T^T dW + (dA + dA^T) K
//   dT    = dW (diag(e^gamma) K)^T + dU V^T,  dX = dT diag(beta)
//   dL    = -(X^T dX X^T) strictly lower,  dA_ij = dL_ij beta_i Gam_ij
// plus the gate terms (d gamma) and d beta; dg is the reverse chunk-local
// cumsum of d gamma.
//
// Kernels (all FP32 arithmetic, FP32 MFMA 16x16x4):
//   bwd_prep    per (chunk, head): X by the blocked solve; the W of the products
//   bwd_dstate  per (sequence, head, 64-wide value block), chunks in reverse:
//               the dS recurrence; writes dS' and dVnew of every chunk, and dh0
//               (FP32 inputs; bf16 inputs use gdn_bwd_state.hip)
//   bwd_chunk   per (chunk, head): Vnew, dv, and every chunk-local gradient
//   bwd_group   per (token, query/key head): dq, dk summed over the head group
#include "gdn_device.h"
#include "gdn_images.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

constexpr int NT = 256;          // threads per workgroup
constexpr float LOG2E = 1.4426950408889634f;

struct Gates {
  alignas(16) float gam2[64];    // log2-scaled chunk-local cumsum
  alignas(16) float eg[64];      // e^gamma
  alignas(16) float egc[64];     // e^(gamma_n - gamma), 0 past the chunk end
  alignas(16) float bet[64];
  float egC;                     // e^gamma_n
};

// Wave 0 forms the gates of one chunk (rows past nc: g = beta = 0).
__device__ void load_gates(Gates& gs, const float* g, const float* beta, int t0, int nc,
                           int Hv, int h, int wave, int lane) {
  if (wave != 0) return;
  const bool valid = lane < nc;
  const int64_t gi = (int64_t)(t0 + lane) * Hv + h;
  const float g2 = wave_incl_scan(valid ? g[gi] * LOG2E : 0.f);
  const float g2n = read_lane(g2, nc - 1);
  gs.gam2[lane] = g2;
  gs.eg[lane] = fexp2(g2);
  gs.egc[lane] = valid ? fexp2(g2n - g2) : 0.f;
  gs.bet[lane] = valid ? beta[gi] : 0.f;
  if (lane == 0) gs.egC = fexp2(g2n);
}

// acc += sum_{k in [k0, k1)} A(i0 + r, k) B(k, j0 + c) for one 16x16 tile, with
// A(i, k) = A[i * ars + k * acs] and B(k, j) = B[k * brs + j * bcs] (FP32).
__device__ __forceinline__ f32x4 mm(const float* A, int ars, int acs, const float* B, int brs,
                                    int bcs, int i0, int j0, int k0, int k1, int r16, int grp,
                                    f32x4 acc) {
  for (int k = k0; k < k1; k += 4)
    acc = mfma_f32(A[(i0 + r16) * ars + (k + grp) * acs], B[(k + grp) * brs + (j0 + r16) * bcs], acc);
  return acc;
}

// mm with the k loop unrolled by four (k1 - k0 a multiple of 16), so the LDS
// reads of four steps are in flight before their products.
__device__ __forceinline__ f32x4 mm_u(const float* A, int ars, int acs, const float* B, int brs,
                                      int bcs, int i0, int j0, int k0, int k1, int r16, int grp,
                                      f32x4 acc) {
#pragma unroll 4
  for (int k = k0; k < k1; k += 4)
    acc = mfma_f32(A[(i0 + r16) * ars + (k + grp) * acs], B[(k + grp) * brs + (j0 + r16) * bcs], acc);
  return acc;
}

// acc += A(i0 + r, .) Breg, where Breg holds KT accumulator tiles of a
// [16 KT x 16] B block (Breg[t][i] = B[16 t + 4 grp + i][c]); K runs in the
// matching order. A(i, k) = A[i * ars + k * acs].
template <int KT>
__device__ __forceinline__ f32x4 mm_reg(const float* A, int ars, int acs, const f32x4 (&Breg)[KT],
                                        int i0, int r16, int grp, f32x4 acc) {
#pragma unroll
  for (int t = 0; t < KT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = mfma_f32(A[(i0 + r16) * ars + (16 * t + 4 * grp + i) * acs], Breg[t][i], acc);
  return acc;
}

// Loads 64 rows x D columns of a [tokens, H, D_total] input (bf16 or FP32)
// starting at column col0 into an FP32 LDS tile with row stride ld; rows past
// nc become 0.
template <bool F32IN>
__device__ void stage_rows(float* dst, int ld, const void* src, int t0, int nc, int H, int h,
                           int Dtot, int col0, int D, int tid) {
  // unrolled so that several rows' loads are in flight before their LDS writes
#pragma unroll 8
  for (int e = tid; e < 64 * D; e += NT) {
    const int r = e / D, cc = e % D;
    float v = 0.f;
    if (r < nc) {
      const int64_t off = ((int64_t)(t0 + r) * H + h) * Dtot + col0 + cc;
      v = F32IN ? reinterpret_cast<const float*>(src)[off]
                : static_cast<float>(reinterpret_cast<const bf16*>(src)[off]);
    }
    dst[r * ld + cc] = v;
  }
}

// stage_rows for bf16 rows of D (a multiple of 8) columns: 16-byte loads,
// all of a thread's issued before its LDS writes.
template <int D>
__device__ void stage_rows_bf16(float* dst, int ld, const void* src, int t0, int nc, int H, int h,
                                int tid) {
  constexpr int V = 64 * D / 8, PER = (V + NT - 1) / NT;
  bf16x8 v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = tid + NT * u, r = e / (D / 8), c8 = e % (D / 8);
    if (e < V && r < nc)
      v[u] = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16*>(src) +
                                              ((int64_t)(t0 + r) * H + h) * D + 8 * c8);
    else
      v[u] = bf16x8{};
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = tid + NT * u, r = e / (D / 8), c8 = e % (D / 8);
    if (e < V) {
#pragma unroll
      for (int i = 0; i < 8; ++i) dst[r * ld + 8 * c8 + i] = static_cast<float>(v[u][i]);
    }
  }
}

// X = (I + L)^-1 for strictly lower L (FP32 [64][65] in LDS): 16x16 diagonal
// blocks by substitution, then the 16- and 32-block merges
// X_BA = -X_BB (L_BA X_AA). Yf is a [32][33] scratch. All threads call it;
// it ends after a barrier.
__device__ void solve64(const float* Lf, float* Xf, float* Yf, int wave, int lane) {
  const int r16 = lane & 15, grp = lane >> 4, tid = wave * 64 + lane;
  for (int e = tid; e < 64 * 64; e += NT) {
    const int i = e >> 6, j = e & 63;
    if ((j >> 4) > (i >> 4)) Xf[i * 65 + j] = 0.f;
  }
  if (lane < 16) {
    const int b = wave, cc = lane;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = (r == cc) ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < r; ++j) s -= Lf[(16 * b + r) * 65 + 16 * b + j] * x[j];
      x[r] = s;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Xf[(16 * b + r) * 65 + 16 * b + cc] = x[r];
  }
  __syncthreads();
  if (wave < 2) {
    const int A = 2 * wave, B = A + 1;
    const f32x4 y = mm(Lf + 16 * B * 65 + 16 * A, 65, 1, Xf + 16 * A * 65 + 16 * A, 65, 1, 0, 0,
                       0, 16, r16, grp, zero4());
    f32x4 z = zero4();
#pragma unroll
    for (int i = 0; i < 4; ++i) z = mfma_f32(Xf[(16 * B + r16) * 65 + 16 * B + 4 * grp + i], y[i], z);
#pragma unroll
    for (int i = 0; i < 4; ++i) Xf[(16 * B + 4 * grp + i) * 65 + 16 * A + r16] = -z[i];
  }
  __syncthreads();
  {
    const int ti = wave >> 1, tj = wave & 1;
    const f32x4 y = mm(Lf + 32 * 65, 65, 1, Xf, 65, 1, 16 * ti, 16 * tj, 0, 32, r16, grp, zero4());
#pragma unroll
    for (int i = 0; i < 4; ++i) Yf[(16 * ti + 4 * grp + i) * 33 + 16 * tj + r16] = y[i];
  }
  __syncthreads();
  {
    const int ti = wave >> 1, tj = wave & 1;
    const f32x4 z = mm(Xf + 32 * 65 + 32, 65, 1, Yf, 33, 1, 16 * ti, 16 * tj, 0, 32, r16, grp, zero4());
#pragma unroll
    for (int i = 0; i < 4; ++i) Xf[(32 + 16 * ti + 4 * grp + i) * 65 + 16 * tj + r16] = -z[i];
  }
  __syncthreads();
}

// L_ij = beta_i (K K^T)_ij Gam_ij for i > j (else 0) into Lf [64][65].
template <int DK>
__device__ void build_L(const float* Kf, const Gates& gs, float* Lf, int wave, int lane) {
  constexpr int LK = DK + 1;
  const int r16 = lane & 15, grp = lane >> 4;
  for (int t = wave; t < 16; t += 4) {
    const int mi = t >> 2, mj = t & 3;
    const f32x4 a = mm_u(Kf, LK, 1, Kf, 1, LK, 16 * mi, 16 * mj, 0, DK, r16, grp, zero4());
    const int cj = 16 * mj + r16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * mi + 4 * grp + i;
      Lf[row * 65 + cj] = row > cj ? gs.bet[row] * a[i] * fexp2(gs.gam2[row] - gs.gam2[cj]) : 0.f;
    }
  }
}

// ------------------------------------------------------------------ bwd_prep
template <int DK, bool F32IN, int WF>
__global__ void __launch_bounds__(NT, 1) bwd_prep(BwdKernelArgs a, int N) {
  constexpr int LK = DK + 1;
  __shared__ float Kf[64 * LK];
  __shared__ float Lf[64 * 65], Xf[64 * 65], Yf[32 * 33];
  __shared__ Gates gs;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = __lane_id();
  const int tid = wave * 64 + lane, r16 = lane & 15, grp = lane >> 4;
  const int slot = blockIdx.x, h = blockIdx.y;
  const FwdKernelArgs& f = a.f;
  const Chunk ch = locate_slot(slot, f.cu_seqlens, N, f.T, f.prefix_len);
  if (!ch.valid) return;
  const int Hv = f.Hv, Hqk = f.Hqk, hk = h / (Hv / Hqk);

  stage_rows<F32IN>(Kf, LK, f.k, ch.t0, ch.nc, Hqk, hk, DK, 0, DK, tid);
  load_gates(gs, f.g, f.beta, ch.t0, ch.nc, Hv, h, wave, lane);
  float* Xg = a.ws_X + ((int64_t)slot * Hv + h) * 4096;
  if (f.solve_degree > 0) {
    // approximate inverse: X is the forward's saved polynomial (ws_X points
    // at it), never a fresh exact solve
    for (int e = tid; e < 4096; e += NT) Xf[(e >> 6) * 65 + (e & 63)] = Xg[e];
    __syncthreads();
  } else {
    __syncthreads();
    build_L<DK>(Kf, gs, Lf, wave, lane);
    __syncthreads();
    solve64(Lf, Xf, Yf, wave, lane);
    for (int e = tid; e < 4096; e += NT) Xg[e] = Xf[(e >> 6) * 65 + (e & 63)];
  }

  float* Wg = a.ws_W + ((int64_t)ch.t0 * Hv + h) * DK;
  if constexpr (WF != 0 && !F32IN) {
    // bf16 inputs: the later kernels read the W codes themselves
  } else if constexpr (WF != 0) {
    const float dW = f.w_scale[(int64_t)slot * Hv + h];
    const uint8_t* codes = f.w_codes + ((int64_t)ch.t0 * Hv + h) * DK;
    for (int e = tid; e < ch.nc * DK; e += NT) {
      const int r = e / DK, cc = e % DK;
      const int64_t off = (int64_t)r * Hv * DK + cc;
      const uint8_t b = codes[off];
      const float cv = WF == 1 ? __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(b), 0)
                               : static_cast<float>(static_cast<int8_t>(b));
      Wg[off] = cv * dW;
    }
  } else {
    // T' = X diag(beta e^gamma) into Lf, then W = T' K
    for (int e = tid; e < 4096; e += NT) {
      const int i = e >> 6, j = e & 63;
      Lf[i * 65 + j] = Xf[i * 65 + j] * gs.bet[j] * gs.eg[j];
    }
    __syncthreads();
    for (int t = wave; t < 4 * (DK / 16); t += 4) {
      const int mt = t & 3, nt = t >> 2;
      const f32x4 w = mm(Lf, 65, 1, Kf, LK, 1, 16 * mt, 16 * nt, 0, 64, r16, grp, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * mt + 4 * grp + i;
        if (row < ch.nc) Wg[(int64_t)row * Hv * DK + 16 * nt + r16] = w[i];
      }
    }
  }
}

// --------------------------------------------------------------- bwd_neumann
// Gradient through the approximate inverse ("[7/7] Experimental GDN/KDA
// approximate-inverse QAT", "What does this PR do?": the backward
// differentiates the actual polynomial). With X = sum_{m=0..d} (-L)^m and
// G = dL/dX (its strict lower part: X's other entries do not depend on L),
//   dL = -sum_{m=1..d} sum_{a+b=m-1} (-L^T)^a G (-L^T)^b
// (the adjoint of the directional derivative of the polynomial). That double
// sum is the top-right block of sum_{m=0..d} M^m for the block matrix
// M = [[-L^T, G], [0, -L^T]] (the top-right block of M^m is exactly
// sum_{a+b=m-1} (-L^T)^a G (-L^T)^b), and for d = 2^j - 1 that sum is the
// product (I + M)(I + M^2)(I + M^4)..., the same factorization the forward
// uses. Each block product needs the diagonal block D and the top-right
// block E: P = M^(2^i) is [[Pd, Pe], [0, Pd]], the partial product is
// [[Xd, Xe], [0, Xd]], and per step
//   Pd' = Pd Pd,  Pe' = Pd Pe + Pe Pd,  Xd' = Xd + Xd Pd',  Xe' = Xd Pe' + Xe + Xe Pd'.
// Then dL = -Xe below the diagonal, and the terms of L_ij = beta_i (k_i . k_j)
// Gam_ij that bwd_local_kernel leaves out for this policy are added here:
//   dk += (dA + dA^T) K with dA = dL beta Gam;  d beta_i += sum_j dL_ij (K K^T)_ij Gam_ij;
//   d gamma_i += sum_j dL_ij L_ij, d gamma_j -= sum_i dL_ij L_ij, and dg gets
// the chunk-local suffix sums of those d gamma. dk goes to the per-value-head
// FP32 rows (the group sum follows); d beta and dg are read, added to and
// written back (one workgroup per chunk and head owns those entries).
// FP32 throughout (FP32 MFMA 16x16x4). -L^T and its powers (Pd) and the
// partial products Xd are upper triangular, L and dL strictly lower, so each
// product runs only over the 16-wide key blocks where both factors can be
// nonzero (the skipped steps would add exact zeros) and tiles known to be
// zero are written as zeros.
template <int DK>
__global__ void __launch_bounds__(NT, 1) bwd_neumann(BwdKernelArgs a, int N) {
  constexpr int LK = DK + 1;
  constexpr int M65 = 64 * 65;
  __shared__ float Kf[64 * LK];
  __shared__ float Lf[M65];
  __shared__ float Mb[6][M65];
  __shared__ Gates gs;
  __shared__ float rowB[64], rowG[64], colG[64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = __lane_id();
  const int tid = wave * 64 + lane, r16 = lane & 15, grp = lane >> 4;
  const int slot = blockIdx.x, h = blockIdx.y;
  const FwdKernelArgs& f = a.f;
  const Chunk ch = locate_slot(slot, f.cu_seqlens, N, f.T, f.prefix_len);
  if (!ch.valid) return;
  const int Hv = f.Hv, Hqk = f.Hqk, hk = h / (Hv / Hqk), nc = ch.nc;
  const int64_t chb = (int64_t)slot * Hv + h;

  stage_rows_bf16<DK>(Kf, LK, f.k, ch.t0, nc, Hqk, hk, tid);
  load_gates(gs, f.g, f.beta, ch.t0, nc, Hv, h, wave, lane);
  __syncthreads();
  build_L<DK>(Kf, gs, Lf, wave, lane);
  __syncthreads();
  // M = [[-L^T, G], [0, -L^T]]: P = M, partial product I + M
  int iPd = 0, iPe = 1, iXd = 2, iXe = 3, iT1 = 4, iT2 = 5;
  {
    // every load of dX is issued before the first use (one memory latency,
    // not one per element)
    const float* dXg = a.ws_dX + chb * 4096;
    constexpr int PER = 4096 / NT;
    float gv[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) gv[u] = dXg[tid + NT * u];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + NT * u, i = e >> 6, j = e & 63;
      const float g = (j < i && i < nc) ? gv[u] : 0.f;
      const float lt = Lf[j * 65 + i];
      Mb[iPd][i * 65 + j] = -lt;
      Mb[iXd][i * 65 + j] = (i == j ? 1.f : 0.f) - lt;
      Mb[iPe][i * 65 + j] = g;
      Mb[iXe][i * 65 + j] = g;
    }
  }
  __syncthreads();
  for (int d = 1; d < f.solve_degree; d = 2 * d + 1) {
    const float *Pd = Mb[iPd], *Pe = Mb[iPe];
    float *T1 = Mb[iT1], *T2 = Mb[iT2];
    for (int t = wave; t < 16; t += 4) {
      const int i0 = 16 * (t >> 2), j0 = 16 * (t & 3);
      // Pd(i, k) = 0 for k below i's block, Pd(k, j) = 0 for k above j's block
      f32x4 pe = mm_u(Pd, 65, 1, Pe, 65, 1, i0, j0, i0, 64, r16, grp, zero4());
      pe = mm_u(Pe, 65, 1, Pd, 65, 1, i0, j0, 0, j0 + 16, r16, grp, pe);
      const f32x4 pd = i0 <= j0 ? mm_u(Pd, 65, 1, Pd, 65, 1, i0, j0, i0, j0 + 16, r16, grp, zero4())
                                : zero4();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        T1[(i0 + 4 * grp + i) * 65 + j0 + r16] = pe[i];
        T2[(i0 + 4 * grp + i) * 65 + j0 + r16] = pd[i];
      }
    }
    __syncthreads();
    // new Xe and Xd into the buffers of the old Pe and Pd (no longer read)
    const float *Xd = Mb[iXd], *Xe = Mb[iXe];
    float *nXe = Mb[iPe], *nXd = Mb[iPd];
    for (int t = wave; t < 16; t += 4) {
      const int i0 = 16 * (t >> 2), j0 = 16 * (t & 3);
      f32x4 xe, xd;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xe[i] = Xe[(i0 + 4 * grp + i) * 65 + j0 + r16];
        xd[i] = Xd[(i0 + 4 * grp + i) * 65 + j0 + r16];
      }
      xe = mm_u(Xd, 65, 1, T1, 65, 1, i0, j0, i0, 64, r16, grp, xe);         // Xd upper
      xe = mm_u(Xe, 65, 1, T2, 65, 1, i0, j0, 0, j0 + 16, r16, grp, xe);     // Pd' upper
      if (i0 <= j0) xd = mm_u(Xd, 65, 1, T2, 65, 1, i0, j0, i0, j0 + 16, r16, grp, xd);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        nXe[(i0 + 4 * grp + i) * 65 + j0 + r16] = xe[i];
        nXd[(i0 + 4 * grp + i) * 65 + j0 + r16] = xd[i];
      }
    }
    __syncthreads();
    const int oXd = iXd, oXe = iXe;
    iXd = iPd; iXe = iPe; iPd = iT2; iPe = iT1; iT1 = oXd; iT2 = oXe;
  }
  // dL = -Xe below the diagonal (rows and columns of the chunk); dA = dL beta Gam
  const float* Xe = Mb[iXe];
  float* DA = Mb[iT1];
  float* AG = Mb[iT2];
  for (int e = tid; e < 4096; e += NT) {
    const int i = e >> 6, j = e & 63;
    const float dl = (j < i && i < nc) ? -Xe[i * 65 + j] : 0.f;
    DA[i * 65 + j] = dl * gs.bet[i] * fexp2(gs.gam2[i] - gs.gam2[j]);
  }
  // (K K^T)_ij Gam_ij below the diagonal
  for (int t = wave; t < 16; t += 4) {
    const int mi = t >> 2, mj = t & 3;
    const f32x4 kk = mi >= mj ? mm_u(Kf, LK, 1, Kf, 1, LK, 16 * mi, 16 * mj, 0, DK, r16, grp, zero4())
                              : zero4();
    const int cj = 16 * mj + r16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * mi + 4 * grp + i;
      AG[row * 65 + cj] = row > cj ? kk[i] * fexp2(gs.gam2[row] - gs.gam2[cj]) : 0.f;
    }
  }
  __syncthreads();
  // row and column sums: d beta_i = sum_j dL_ij AG_ij; d gamma parts from dL_ij L_ij
  // (four threads per row and per column, 16 entries each, combined within
  // their quad; fixed trip counts with masks so the LDS reads are issued ahead)
  {
    const int i = tid >> 2, part = tid & 3;
    float sb = 0.f, sg = 0.f, cg = 0.f;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const int j = 16 * part + jj;
      const float dl = (j < i && i < nc) ? -Xe[i * 65 + j] : 0.f;
      sb += dl * AG[i * 65 + j];
      sg += dl * Lf[i * 65 + j];
      // column i: rows j of the same range (the roles of i and j swapped)
      cg += (j > i && j < nc) ? -Xe[j * 65 + i] * Lf[j * 65 + i] : 0.f;
    }
    sb += dpp_f<0xB1>(sb);
    sb += dpp_f<0x4E>(sb);
    sg += dpp_f<0xB1>(sg);
    sg += dpp_f<0x4E>(sg);
    cg += dpp_f<0xB1>(cg);
    cg += dpp_f<0x4E>(cg);
    if (part == 0) {
      rowB[i] = sb;
      rowG[i] = sg;
      colG[i] = cg;
    }
  }
  // C = dA + dA^T into the Xe buffer's place is not needed: K products read DA twice
  __syncthreads();
  // dk += (dA + dA^T) K, added to this value head's FP32 dk rows
  // (all of a wave's tiles first, then every read of the rows they add to,
  // then the writes: one memory latency per wave, not one per tile)
  constexpr int NTW = DK / 16;                  // tiles per wave: 4 row blocks x DK / 16 over 4 waves
  f32x4 acc[NTW];
#pragma unroll
  for (int u = 0; u < NTW; ++u) {
    const int t = wave + 4 * u, mt = t & 3, nt = t >> 2;
    // DA(i, k) = 0 for k >= i; DA^T(i, k) = DA(k, i) = 0 for k <= i
    acc[u] = mm_u(DA, 65, 1, Kf, LK, 1, 16 * mt, 16 * nt, 0, 16 * mt + 16, r16, grp, zero4());
    acc[u] = mm_u(DA, 1, 65, Kf, LK, 1, 16 * mt, 16 * nt, 16 * mt, 64, r16, grp, acc[u]);
  }
  float old[NTW][4];
#pragma unroll
  for (int u = 0; u < NTW; ++u) {
    const int t = wave + 4 * u, mt = t & 3, nt = t >> 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * mt + 4 * grp + i;
      old[u][i] = row < nc ? a.ws_dqk[(((int64_t)(ch.t0 + row) * Hv + h) * 2 + 1) * DK + 16 * nt + r16]
                           : 0.f;
    }
  }
#pragma unroll
  for (int u = 0; u < NTW; ++u) {
    const int t = wave + 4 * u, mt = t & 3, nt = t >> 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * mt + 4 * grp + i;
      if (row < nc)
        a.ws_dqk[(((int64_t)(ch.t0 + row) * Hv + h) * 2 + 1) * DK + 16 * nt + r16] =
            old[u][i] + acc[u][i];
    }
  }
  if (wave == 0) {
    const int j = lane;
    const float dgam = j < nc ? rowG[j] - colG[j] : 0.f;
    float suf = dgam;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_down(suf, off, WAVE);
      if (j + off < 64) suf += y;
    }
    if (j < nc) {
      const int64_t gi = (int64_t)(ch.t0 + j) * Hv + h;
      a.dg[gi] += suf;
      a.dbeta[gi] += rowB[j];
    }
  }
}

// ----------------------------------------------------------- bwd_read_anchor
// Two-precision profile ("[5/8] ReplaySSM state QAT and two-precision GDN",
// "What does this PR do?"): the chunk's carry is exp(gamma_n) S with the FP32
// state S, while its reads use Sr. The other kernels take the saved Sr as the
// chunk's state (s_f32), which is right for every product and for the
// identity straight-through gradient of the reads, but gives the gate term of
// the carry as exp(gamma_n) <dS', Sr>. This kernel adds the rest,
// exp(gamma_n) <dS', S - Sr>, to d gamma_n, that is to dg of every token of
// the chunk (dg is the chunk-local suffix sum of d gamma). dS' (the gradient
// of the state after the chunk) is read in the reverse recurrence's fragment
// order; the sum is in a fixed order.
__global__ void __launch_bounds__(NT) bwd_read_anchor(BwdKernelArgs a, int N, int DK) {
  __shared__ float red[NT / 64];
  const int wave = threadIdx.x >> 6, lane = __lane_id(), tid = threadIdx.x;
  const int slot = blockIdx.x, h = blockIdx.y;
  const FwdKernelArgs& f = a.f;
  const Chunk ch = locate_slot(slot, f.cu_seqlens, N, f.T, f.prefix_len);
  if (!ch.valid) return;
  const int Hv = f.Hv, Dv = f.Dv, MT = DK / 16;
  const int64_t chb = (int64_t)slot * Hv + h, n = (int64_t)DK * Dv;
  const float* dSp = a.ws_dstate + chb * n;          // fragment order (frag_off)
  const float* Sa = f.s_anchor + chb * n;            // row-major
  const float* Sr = f.s_f32 + chb * n;
  float acc = 0.f;
  for (int64_t e = tid; e < n; e += NT) {
    const int i = (int)(e & 3), ln = (int)((e >> 2) & 63);
    const int64_t rest = e >> 8;
    const int mt = (int)(rest % MT), w = (int)((rest / MT) & 3), vb = (int)(rest / MT / 4);
    const int row = 16 * mt + 4 * (ln >> 4) + i, col = 64 * vb + 16 * w + (ln & 15);
    const int64_t rc = (int64_t)row * Dv + col;
    acc += dSp[e] * (Sa[rc] - Sr[rc]);
  }
  acc = wave_sum(acc);
  if (lane == 0) red[wave] = acc;
  __syncthreads();
  if (wave == 0) {
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) tot += red[w];
    const float gv = lane < ch.nc ? f.g[(int64_t)(ch.t0 + lane) * Hv + h] : 0.f;
    const float add = expf(wave_sum(gv)) * tot;
    if (lane < ch.nc) a.dg[(int64_t)(ch.t0 + lane) * Hv + h] += add;
  }
}

// ---------------------------------------------------------------- bwd_dstate
template <int DK, bool F32IN>
__global__ void __launch_bounds__(NT, 1) bwd_dstate(BwdKernelArgs a) {
  constexpr int LK = DK + 1, MK = DK / 16;
  __shared__ float Qf[64 * LK], Kf[64 * LK], Wf[64 * LK];
  __shared__ float dOf[64 * 65], Pf[64 * 65];
  __shared__ Gates gs;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = __lane_id();
  const int tid = wave * 64 + lane, r16 = lane & 15, grp = lane >> 4;
  const FwdKernelArgs& f = a.f;
  const int vb = blockIdx.x, h = blockIdx.y, n = blockIdx.z;
  const int Hv = f.Hv, Hqk = f.Hqk, Dv = f.Dv, hk = h / (Hv / Hqk);
  int bos, eos;
  seq_span(f, n, bos, eos);
  const int nchunks = (eos - bos + CHUNK - 1) / CHUNK;
  const int col = vb * 64 + 16 * wave + r16;        // this lane's value column (dht, dh0)
  const int64_t sbase = ((int64_t)n * Hv + h) * DK * Dv;

  f32x4 dS[MK];                                     // dS[mt][i] = dS[16 mt + 4 grp + i][col]
#pragma unroll
  for (int mt = 0; mt < MK; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dS[mt][i] = a.dht ? a.dht[sbase + (int64_t)(16 * mt + 4 * grp + i) * Dv + col] : 0.f;

  for (int c = nchunks - 1; c >= 0; --c) {
    const int t0 = bos + CHUNK * c, nc = min(CHUNK, eos - t0);
    const int slot = n + bos / CHUNK + c;
    stage_rows<F32IN>(Qf, LK, f.q, t0, nc, Hqk, hk, DK, 0, DK, tid);
    stage_rows<F32IN>(Kf, LK, f.k, t0, nc, Hqk, hk, DK, 0, DK, tid);
    for (int e = tid; e < 64 * DK; e += NT) {
      const int r = e / DK, cc = e % DK;
      Wf[r * LK + cc] = r < nc ? a.ws_W[((int64_t)(t0 + r) * Hv + h) * DK + cc] : 0.f;
    }
    stage_rows<F32IN>(dOf, 65, a.dout, t0, nc, Hv, h, Dv, vb * 64, 64, tid);
    load_gates(gs, f.g, f.beta, t0, nc, Hv, h, wave, lane);
    __syncthreads();

    // P = (Q K^T) * Gam, lower including the diagonal
    for (int t = wave; t < 16; t += 4) {
      const int mi = t >> 2, mj = t & 3;
      const f32x4 p = mm(Qf, LK, 1, Kf, 1, LK, 16 * mi, 16 * mj, 0, DK, r16, grp, zero4());
      const int cj = 16 * mj + r16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * mi + 4 * grp + i;
        Pf[row * 65 + cj] = row >= cj ? p[i] * fexp2(gs.gam2[row] - gs.gam2[cj]) : 0.f;
      }
    }
    __syncthreads();

    // dS' of this chunk (the gradient at its end), kept for bwd_chunk
    const int64_t chb = (int64_t)slot * Hv + h;
#pragma unroll
    for (int mt = 0; mt < MK; ++mt)
      *reinterpret_cast<f32x4*>(a.ws_dstate + frag_off(chb, Dv / 64, vb, wave, MK, mt, lane)) = dS[mt];
    // dVnew = scale P^T dO + diag(egc) K dS'
    f32x4 dVn[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const f32x4 p = mm(Pf, 1, 65, dOf, 65, 1, 16 * mt, 16 * wave, 0, 64, r16, grp, zero4());
      const f32x4 q = mm_reg<MK>(Kf, LK, 1, dS, 16 * mt, r16, grp, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * mt + 4 * grp + i;
        dVn[mt][i] = f.scale * p[i] + gs.egc[row] * q[i];
      }
      *reinterpret_cast<f32x4*>(a.ws_dvn + frag_off(chb, Dv / 64, vb, wave, 4, mt, lane)) = dVn[mt];
    }
    __syncthreads();                                 // dOf fully read
    for (int e = tid; e < 64 * 64; e += NT) dOf[(e >> 6) * 65 + (e & 63)] *= gs.eg[e >> 6];
    __syncthreads();
    // dS = e^gamma_n dS' + scale Q^T (diag(e^gamma) dO) - W^T dVnew
    const float egC = gs.egC;
#pragma unroll
    for (int mt = 0; mt < MK; ++mt) {
      const f32x4 q = mm(Qf, 1, LK, dOf, 65, 1, 16 * mt, 16 * wave, 0, 64, r16, grp, zero4());
      const f32x4 w = mm_reg<4>(Wf, 1, LK, dVn, 16 * mt, r16, grp, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) dS[mt][i] = egC * dS[mt][i] + f.scale * q[i] - w[i];
    }
    __syncthreads();                                 // LDS reused by the next chunk
  }
  if (a.dh0) {
#pragma unroll
    for (int mt = 0; mt < MK; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) a.dh0[sbase + (int64_t)(16 * mt + 4 * grp + i) * Dv + col] = dS[mt][i];
  }
}

// ----------------------------------------------------------------- bwd_chunk
template <int DK>
struct ChunkSmem {
  static constexpr int LK = DK + 1;
  union {
    struct {                    // value-block loop
      float Tf[64 * 65];        // T = X diag(beta)
      float Wf[64 * LK];
      float Vf[64 * 33], dOf[64 * 33], Vnf[64 * 33], dVnf[64 * 33];
      float Sqf[DK * 33], dSf[DK * 33];
    } p1;
    struct {                    // chunk-local finish
      float Kf[64 * LK], Qf[64 * LK];
      float Xf[64 * 65], Gf[64 * 65];
      float dWf[64 * LK];
    } p2;
  } u;
  Gates gs;
  // per-wave column partials (summed in a fixed order: deterministic)
  float colH[4][64];            // column sums of H = G * (Q K^T)
  float colHL[4][64];           // column sums of dL * L
  float colDB[4][64];           // column sums of dT * X (d beta from T = X diag(beta))
  // per-row totals (each row lives in one wave)
  float rowDG[64];              // d gamma row parts
  float rowTerm[64];            // egc_j k_j . (Vnew dS'^T)_j  (state-update gate term)
  float rowDB[64];              // d beta from L
  float red[4];                 // <dS', Sq> per wave
};

template <int DK, bool F32IN, int SF>
__global__ void __launch_bounds__(NT, 1) bwd_chunk(BwdKernelArgs a, int N) {
  constexpr int LK = DK + 1, NC = DK / 16;         // column tiles of a [64, DK] matrix
  __shared__ ChunkSmem<DK> sm;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = __lane_id();
  const int tid = wave * 64 + lane, r16 = lane & 15, grp = lane >> 4;
  const int slot = blockIdx.x, h = blockIdx.y;
  const FwdKernelArgs& f = a.f;
  const Chunk ch = locate_slot(slot, f.cu_seqlens, N, f.T, f.prefix_len);
  if (!ch.valid) return;
  const int Hv = f.Hv, Hqk = f.Hqk, Dv = f.Dv, hk = h / (Hv / Hqk);
  const int t0 = ch.t0, nc = ch.nc;
  const float scale = f.scale;
  Gates& gs = sm.gs;
  const int64_t ch_base = (int64_t)slot * Hv + h;

  load_gates(gs, f.g, f.beta, t0, nc, Hv, h, wave, lane);
  __syncthreads();
  {
    const float* Xg = a.ws_X + ch_base * 4096;
    for (int e = tid; e < 4096; e += NT) {
      const int i = e >> 6, j = e & 63;
      sm.u.p1.Tf[i * 65 + j] = Xg[e] * gs.bet[j];
    }
    for (int e = tid; e < 64 * DK; e += NT) {
      const int r = e / DK, cc = e % DK;
      sm.u.p1.Wf[r * LK + cc] = r < nc ? a.ws_W[((int64_t)(t0 + r) * Hv + h) * DK + cc] : 0.f;
    }
  }

  // accumulators over value blocks; wave w owns row tile w of each
  f32x4 dW[NC], dQi[NC], dKs[NC], dP[4], dTU[4];
#pragma unroll
  for (int q = 0; q < NC; ++q) dW[q] = dQi[q] = dKs[q] = zero4();
#pragma unroll
  for (int q = 0; q < 4; ++q) dP[q] = dTU[q] = zero4();
  float sSq = 0.f;

  for (int v0 = 0; v0 < Dv; v0 += 32) {
    auto& p1 = sm.u.p1;
    stage_rows<F32IN>(p1.Vf, 33, f.v, t0, nc, Hv, h, Dv, v0, 32, tid);
    stage_rows<F32IN>(p1.dOf, 33, a.dout, t0, nc, Hv, h, Dv, v0, 32, tid);
    {
      // dVnew and dS' come in fragment order (frag_off): the two 16-column
      // groups of columns v0..v0+31 are one contiguous block
      const int nvb = Dv / 64, vbk = v0 >> 6, w0 = (v0 & 63) >> 4;
      const float* dvg = a.ws_dvn + frag_off(ch_base, nvb, vbk, w0, 4, 0, 0);
      const float* dsg = a.ws_dstate + frag_off(ch_base, nvb, vbk, w0, NC, 0, 0);
      for (int e = tid; e < 64 * 32; e += NT) {
        const int i = e & 3, ln = (e >> 2) & 63, mt = (e >> 8) & 3, ws = e >> 10;
        p1.dVnf[(16 * mt + 4 * (ln >> 4) + i) * 33 + 16 * ws + (ln & 15)] = dvg[e];
      }
      for (int e = tid; e < DK * 32; e += NT) {
        const int i = e & 3, ln = (e >> 2) & 63, mt = (e >> 8) % NC, ws = (e >> 8) / NC;
        p1.dSf[(16 * mt + 4 * (ln >> 4) + i) * 33 + 16 * ws + (ln & 15)] = dsg[e];
      }
      for (int e = tid; e < DK * 32; e += NT) {
        const int r = e >> 5, cc = e & 31;
        float sq;
        if constexpr (SF == 0) {
          sq = f.s_f32[ch_base * DK * Dv + (int64_t)r * Dv + v0 + cc];
        } else {
          const uint8_t b = f.s_codes[ch_base * DK * Dv + (int64_t)r * Dv + v0 + cc];
          const float cv = SF == 1 ? __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(b), 0)
                                   : static_cast<float>(static_cast<int8_t>(b));
          sq = cv * f.s_scale[ch_base * (Dv / f.block_v) + (v0 + cc) / f.block_v];
        }
        p1.Sqf[r * 33 + cc] = sq;
      }
    }
    __syncthreads();
    // Vnew = T V - W Sq and dV = T^T dVnew for this block (8 tiles, 2 per wave)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int mt = wave, nt = q;
      f32x4 u = mm(p1.Tf, 65, 1, p1.Vf, 33, 1, 16 * mt, 16 * nt, 0, 64, r16, grp, zero4());
      const f32x4 ws = mm(p1.Wf, LK, 1, p1.Sqf, 33, 1, 16 * mt, 16 * nt, 0, DK, r16, grp, zero4());
      const f32x4 dv = mm(p1.Tf, 1, 65, p1.dVnf, 33, 1, 16 * mt, 16 * nt, 0, 64, r16, grp, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * mt + 4 * grp + i;
        p1.Vnf[row * 33 + 16 * nt + r16] = u[i] - ws[i];
        if (row < nc) {
          const int64_t off = ((int64_t)(t0 + row) * Hv + h) * Dv + v0 + 16 * nt + r16;
          if (a.grad_f32) reinterpret_cast<float*>(a.dv)[off] = dv[i];
          else reinterpret_cast<bf16*>(a.dv)[off] = to_bf16(dv[i]);
        }
      }
    }
    for (int e = tid; e < DK * 32; e += NT) {
      const int r = e >> 5, cc = e & 31;
      sSq += p1.dSf[r * 33 + cc] * p1.Sqf[r * 33 + cc];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NC; ++q) {
      dW[q] = mm(p1.dVnf, 33, 1, p1.Sqf, 1, 33, 16 * wave, 16 * q, 0, 32, r16, grp, dW[q]);
      dQi[q] = mm(p1.dOf, 33, 1, p1.Sqf, 1, 33, 16 * wave, 16 * q, 0, 32, r16, grp, dQi[q]);
      dKs[q] = mm(p1.Vnf, 33, 1, p1.dSf, 1, 33, 16 * wave, 16 * q, 0, 32, r16, grp, dKs[q]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      dP[q] = mm(p1.dOf, 33, 1, p1.Vnf, 1, 33, 16 * wave, 16 * q, 0, 32, r16, grp, dP[q]);
      dTU[q] = mm(p1.dVnf, 33, 1, p1.Vf, 1, 33, 16 * wave, 16 * q, 0, 32, r16, grp, dTU[q]);
    }
    __syncthreads();
  }
  // block sum of <dS', Sq>
  sSq = wave_sum(sSq);
  if (lane == 0) sm.red[wave] = sSq;

  // ----------------------------------------------------------- finish
  // Row tile `wave` (rows 16 wave + 4 grp + i) is owned by this wave for every
  // [64, *] result; row sums reduce over the 16 lanes of a row group.
  auto& p2 = sm.u.p2;
  stage_rows<F32IN>(p2.Kf, LK, f.k, t0, nc, Hqk, hk, DK, 0, DK, tid);
  stage_rows<F32IN>(p2.Qf, LK, f.q, t0, nc, Hqk, hk, DK, 0, DK, tid);
  {
    const float* Xg = a.ws_X + ch_base * 4096;
    for (int e = tid; e < 4096; e += NT) p2.Xf[(e >> 6) * 65 + (e & 63)] = Xg[e];
  }
  float dg_acc[4] = {0.f, 0.f, 0.f, 0.f};           // d gamma row parts (lane partial)
  float term_acc[4] = {0.f, 0.f, 0.f, 0.f};         // state gate term (lane partial)
  float db_acc[4] = {0.f, 0.f, 0.f, 0.f};           // d beta from L (lane partial)
  // column partial of one 16-column tile: sum the lane's 4 rows and the 4 row groups
  auto col_store = [&](float (&dst)[4][64], int q, const float (&v)[4]) {
    float t = v[0] + v[1] + v[2] + v[3];
    t += __shfl_xor(t, 16, WAVE);
    t += __shfl_xor(t, 32, WAVE);
    if (grp == 0) dst[wave][16 * q + r16] = t;
  };
  __syncthreads();
  // (1) G = scale dP * Gam (lower incl. diagonal); H = G * (Q K^T); dW to LDS
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int cj = 16 * q + r16;
    const f32x4 qk = mm(p2.Qf, LK, 1, p2.Kf, 1, LK, 16 * wave, 16 * q, 0, DK, r16, grp, zero4());
    float hc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * wave + 4 * grp + i;
      const float gv = row >= cj ? scale * dP[q][i] * fexp2(gs.gam2[row] - gs.gam2[cj]) : 0.f;
      p2.Gf[row * 65 + cj] = gv;
      hc[i] = gv * qk[i];
      dg_acc[i] += hc[i];
    }
    col_store(sm.colH, q, hc);
  }
#pragma unroll
  for (int q = 0; q < NC; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) p2.dWf[(16 * wave + 4 * grp + i) * LK + 16 * q + r16] = -dW[q][i];
  __syncthreads();
  // (2) dq = scale diag(e^gamma) dQi + G K; dK = G^T Q + diag(egc) dKs
  f32x4 dK[NC];
  {
    float* dqp = a.ws_dqk + ((int64_t)t0 * Hv + h) * 2 * DK;
#pragma unroll
    for (int q = 0; q < NC; ++q) {
      const int cc = 16 * q + r16;
      const f32x4 gk = mm(p2.Gf, 65, 1, p2.Kf, LK, 1, 16 * wave, 16 * q, 0, 64, r16, grp, zero4());
      dK[q] = mm(p2.Gf, 1, 65, p2.Qf, LK, 1, 16 * wave, 16 * q, 0, 64, r16, grp, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * wave + 4 * grp + i;
        const float qi = scale * gs.eg[row] * dQi[q][i];
        dg_acc[i] += qi * p2.Qf[row * LK + cc];      // gate of the inter-chunk output
        if (row < nc) dqp[(int64_t)row * Hv * 2 * DK + cc] = qi + gk[i];
        const float ks = gs.egc[row] * dKs[q][i];
        dK[q][i] += ks;
        term_acc[i] += ks * p2.Kf[row * LK + cc];   // egc_j k_j . dKs_j
      }
    }
  }
  __syncthreads();                                   // Gf, Qf are free from here
  // (3) dT = dW (diag(e^gamma) K)^T + dU V^T (into Gf); e^gamma T^T dW -> dK, d gamma
  float* dTf = p2.Gf;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int cj = 16 * q + r16;
    const f32x4 t = mm(p2.dWf, LK, 1, p2.Kf, 1, LK, 16 * wave, 16 * q, 0, DK, r16, grp, zero4());
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dTf[(16 * wave + 4 * grp + i) * 65 + cj] = t[i] * gs.eg[cj] + dTU[q][i];
  }
#pragma unroll
  for (int q = 0; q < NC; ++q) {
    const f32x4 tw = mm(p2.Xf, 1, 65, p2.dWf, LK, 1, 16 * wave, 16 * q, 0, 64, r16, grp, zero4());
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * wave + 4 * grp + i;
      const float v = tw[i] * gs.bet[row] * gs.eg[row];
      dK[q][i] += v;
      dg_acc[i] += v * p2.Kf[row * LK + 16 * q + r16];
    }
  }
  __syncthreads();
  // (4) d beta_j += sum_i dT_ij X_ij (this wave's rows); dX = dT diag(beta) in place
  {
    const int j = lane;
    float cs = 0.f;
#pragma unroll 4
    for (int r = 16 * wave; r < 16 * wave + 16; ++r) {
      const float dt = dTf[r * 65 + j];
      cs += dt * p2.Xf[r * 65 + j];
      dTf[r * 65 + j] = dt * gs.bet[j];
    }
    sm.colDB[wave][j] = cs;
  }
  __syncthreads();
  // (5) M1 = X^T dX (into Qf space)
  float* M1 = p2.Qf;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 m = mm(p2.Xf, 1, 65, dTf, 65, 1, 16 * wave, 16 * q, 0, 64, r16, grp, zero4());
#pragma unroll
    for (int i = 0; i < 4; ++i) M1[(16 * wave + 4 * grp + i) * 65 + 16 * q + r16] = m[i];
  }
  __syncthreads();
  // (6) dL = -(M1 X^T) on the strict lower part; with A = K K^T and L = beta A Gam:
  //     d beta_i += dL A Gam, HL = dL L, dA = dL beta_i Gam (into dWf space)
  float* dAf = p2.dWf;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int cj = 16 * q + r16;
    const f32x4 ml = mm(M1, 65, 1, p2.Xf, 1, 65, 16 * wave, 16 * q, 0, 64, r16, grp, zero4());
    const f32x4 kk = mm(p2.Kf, LK, 1, p2.Kf, 1, LK, 16 * wave, 16 * q, 0, DK, r16, grp, zero4());
    float hl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * wave + 4 * grp + i;
      const float gam = row > cj ? fexp2(gs.gam2[row] - gs.gam2[cj]) : 0.f;
      const float dl = -ml[i];
      const float ag = kk[i] * gam;
      db_acc[i] += dl * ag;
      hl[i] = gs.bet[row] * dl * ag;
      dg_acc[i] += hl[i];
      dAf[row * 65 + cj] = dl * gs.bet[row] * gam;
    }
    col_store(sm.colHL, q, hl);
  }
  __syncthreads();
  // (7) dK += (dA + dA^T) K; dk partial
  {
    float* dkp = a.ws_dqk + ((int64_t)t0 * Hv + h) * 2 * DK + DK;
#pragma unroll
    for (int q = 0; q < NC; ++q) {
      f32x4 acc = mm(dAf, 65, 1, p2.Kf, LK, 1, 16 * wave, 16 * q, 0, 64, r16, grp, zero4());
      acc = mm(dAf, 1, 65, p2.Kf, LK, 1, 16 * wave, 16 * q, 0, 64, r16, grp, acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * wave + 4 * grp + i;
        if (row < nc) dkp[(int64_t)row * Hv * 2 * DK + 16 * q + r16] = dK[q][i] + acc[i];
      }
    }
  }
  // (8) row totals over the 16 lanes of each row
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v3[3] = {dg_acc[i], term_acc[i], db_acc[i]};
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      float x = v3[t];
      x += __shfl_xor(x, 8, WAVE);
      x += __shfl_xor(x, 4, WAVE);
      x += __shfl_xor(x, 2, WAVE);
      x += __shfl_xor(x, 1, WAVE);
      v3[t] = x;
    }
    if (r16 == 0) {
      const int row = 16 * wave + 4 * grp + i;
      sm.rowDG[row] = v3[0];
      sm.rowTerm[row] = v3[1];
      sm.rowDB[row] = v3[2];
    }
  }
  __syncthreads();
  // (9) d gamma_j = row part - column parts - state term_j; the last row also
  //     gets e^gamma_n <dS', Sq> + sum_j term_j; dg = suffix sum of d gamma
  if (wave == 0) {
    const int j = lane;
    const float term = sm.rowTerm[j];
    const float term_total = wave_sum(term);
    const float sq_total = sm.red[0] + sm.red[1] + sm.red[2] + sm.red[3];
    float dgj = sm.rowDG[j] - term - (sm.colH[0][j] + sm.colH[1][j] + sm.colH[2][j] + sm.colH[3][j]) -
                (sm.colHL[0][j] + sm.colHL[1][j] + sm.colHL[2][j] + sm.colHL[3][j]);
    if (j == nc - 1) dgj += gs.egC * sq_total + term_total;
    if (j >= nc) dgj = 0.f;
    float suf = dgj;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_down(suf, off, WAVE);
      if (j + off < 64) suf += y;
    }
    const float db = sm.colDB[0][j] + sm.colDB[1][j] + sm.colDB[2][j] + sm.colDB[3][j] + sm.rowDB[j];
    if (j < nc) {
      const int64_t gi = (int64_t)(t0 + j) * Hv + h;
      a.dg[gi] = suf;
      a.dbeta[gi] = db;
    }
  }
}

// ----------------------------------------------------------------- bwd_group
template <int DK>
__global__ void bwd_group(BwdKernelArgs a, int G, int N) {
  const int tok = blockIdx.x, hk = blockIdx.y, d = threadIdx.x;
  const int Hv = a.f.Hv, Hqk = a.f.Hqk;
  if (d >= DK || !token_in_span(a.f, N, tok)) return;
  float sq = 0.f, sk = 0.f;
  for (int j = 0; j < G; ++j) {
    const float* p = a.ws_dqk + (((int64_t)tok * Hv + hk * G + j) * 2) * DK;
    sq += p[d];
    sk += p[DK + d];
  }
  const int64_t off = ((int64_t)tok * Hqk + hk) * DK + d;
  if (a.grad_f32) {
    reinterpret_cast<float*>(a.dq)[off] = sq;
    reinterpret_cast<float*>(a.dk)[off] = sk;
  } else {
    reinterpret_cast<bf16*>(a.dq)[off] = to_bf16(sq);
    reinterpret_cast<bf16*>(a.dk)[off] = to_bf16(sk);
  }
}

}  // namespace

hipError_t launch_bwd_read_anchor(const BwdConfig& c, const BwdKernelArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(bwd_read_anchor, dim3(a.num_slots, c.Hv), dim3(NT), 0, s, a, c.N, c.Dk);
  return hipGetLastError();
}

template <int DK, bool F32IN>
static hipError_t launch_bwd_dk(const BwdConfig& c, const BwdKernelArgs& a, hipStream_t s,
                                const BwdOverlap* ov) {
  const dim3 slots(a.num_slots, c.Hv);
  // bf16 inputs with W QDQ: X comes from the forward's saved buffer and the
  // later kernels read the W codes, so there is nothing to prepare
#define GDN_PREP(WFv) \
  if (c.w_fmt == WFv && (F32IN || WFv == 0)) \
    hipLaunchKernelGGL((bwd_prep<DK, F32IN, WFv>), slots, dim3(NT), 0, s, a, c.N);
  GDN_PREP(0) GDN_PREP(1) GDN_PREP(2)
#undef GDN_PREP
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (F32IN) {
    hipLaunchKernelGGL((bwd_dstate<DK, F32IN>), dim3(c.Dv / 64, c.Hv, c.N), dim3(NT), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else if (ov && a.flags) {
    // The images of the last rev_done chunks first, on every CU; then the
    // state kernel, and beside it on the second stream the image kernel for
    // the rest, in the reverse chunk-major order the state kernel consumes.
    // The flag reset records the fork.
    const int64_t nflags = (int64_t)a.num_slots * c.Hv;
    const int items = a.rev_maxc * c.N * c.Hv, head = a.rev_done * c.N * c.Hv;
    BwdKernelArgs img = a;
    img.flags = nullptr;
    img.rev_lo = 0;
    img.rev_hi = head;
    if ((e = launch_bwd_img(c, img, s)) != hipSuccess) return e;
    if ((e = launch_fill_u32(a.flags, nflags, 0u, s, ov->fork)) != hipSuccess) return e;
    if ((e = launch_bwd_state(c, a, s)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(ov->s2, ov->fork, 0)) != hipSuccess) return e;
    img = a;
    img.rev_lo = head;
    img.rev_hi = items;
    if ((e = launch_bwd_img(c, img, ov->s2, ov->join)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(s, ov->join, 0)) != hipSuccess) return e;
  } else {
    if ((e = launch_bwd_img(c, a, s)) != hipSuccess) return e;
    if ((e = launch_bwd_state(c, a, s)) != hipSuccess) return e;
  }
  if constexpr (F32IN) {
#define GDN_CHUNK(SFv) \
  if (c.state_fmt == SFv) hipLaunchKernelGGL((bwd_chunk<DK, F32IN, SFv>), slots, dim3(NT), 0, s, a, c.N);
    GDN_CHUNK(0) GDN_CHUNK(1) GDN_CHUNK(2)
#undef GDN_CHUNK
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else {
    if ((e = launch_bwd_local(c, a, s)) != hipSuccess) return e;
    if (a.f.solve_degree > 0) {                      // the dL terms of the approximate inverse
      hipLaunchKernelGGL((bwd_neumann<DK>), slots, dim3(NT), 0, s, a, c.N);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  if (!F32IN && c.Hv == c.Hqk && a.f.solve_degree == 0) return hipSuccess;   // dq, dk written directly
  hipLaunchKernelGGL((bwd_group<DK>), dim3(a.total_tokens, c.Hqk), dim3(DK), 0, s, a, c.Hv / c.Hqk,
                     c.N);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdConfig& c, const BwdKernelArgs& a, hipStream_t s, const BwdOverlap* ov) {
  if (a.total_tokens == 0 || c.Hv == 0) return hipSuccess;
  if (c.f32_io) {
    if (c.Dk == 64) return launch_bwd_dk<64, true>(c, a, s, nullptr);
    return hipErrorInvalidValue;
  }
  if (c.Dk == 64) return launch_bwd_dk<64, false>(c, a, s, ov);
  if (c.Dk == 128) return launch_bwd_dk<128, false>(c, a, s, ov);
  return hipErrorInvalidValue;
}

}  // namespace gdn
