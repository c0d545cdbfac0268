// Chunked gated delta rule forward with dynamic state/W fake QDQ, fused into
// one kernel per (sequence, value head, 64-wide value block). Used for FP32
// inputs (Dk = 64); bf16 inputs take the prep + state kernel pair.
//
// Work unit and residency. A workgroup of 4 waves owns the state tile
// S[Dk, 64] of one (sequence, head, value block) and walks the sequence's
// chunks in order; the state never leaves registers (wave w holds columns
// 16w..16w+15 in MFMA accumulator layout). Everything a chunk needs that does
// not depend on the state (gate cumsum, gated K K^T, the exact solve, W and
// its QDQ, U, masked Q K^T) is rebuilt per chunk in LDS from q, k, v, g, beta,
// so HBM traffic is one read of the inputs and one write of O (and ht). The
// next chunk's inputs are loaded into registers while the current chunk is
// computed.
//
// Precision. Operands that are bf16 inputs (q, k, v) are exact in bf16. Every
// FP32 operand of a bf16 MFMA (T, T', P, Vnew, the unquantized state) is split
// as hi + lo bf16 and multiplied in two or three passes (hi*x + lo*x [+ hi*lo]),
// keeping ~16 mantissa bits. QDQ codes (E4M3 values, integers <= 127) are
// exact in bf16, so products with quantized operands are single passes and
// the scales are applied after accumulation. The triangular solve runs in
// FP32 (VALU substitution and FP32 MFMA). Diagonal gate factors sit on the
// FP32 side of each product so bf16 inputs stay exact, and exp(gamma_i -
// gamma_j) is always formed from the difference (the split exp(gamma_i) *
// exp(-gamma_j) overflows for strong gates).
//
// Steps per chunk ("[1/4] GDN state/W QAT foundation", "What does this PR
// do?"; the chunk equations are listed in include/gdn.h):
//   A  store the prefetched K, K^T, Q, V^T tiles to LDS; gates; prefetch c+1
//   B  L = beta_i (K K^T) * Gam, strictly lower (10 16x16 tiles)
//   C  wave 0: diagonal 16x16 blocks of X = (I + L)^-1 by right-looking
//      substitution, then the two 16-block merges X_10 = -X_11 L_10 X_00
//      (FP32 MFMA); waves 1-3: P = (Q K^T) * Gam (lower incl. diagonal)
//   D  waves 0-1: 32-block merge X_BA = -X_BB L_BA X_AA (FP32 MFMA);
//      waves 2-3: rows 0..31 of W = T' K. T = X diag(beta) and
//      T' = T diag(exp(gamma)) are written as hi/lo bf16 by each producer
//   E  rows 32..63 of W; U = T V; amax partials of W and of S
//   F  QDQ_W(W) -> LDS; Sq = QDQ_S(S) per [Dk, block_v] tile
//   G  Vnew = U - Wq Sq; O = scale (exp(gamma) Q Sq + P Vnew);
//      S = exp(gamma_n) Sq + K^T (exp(gamma_n - gamma) Vnew)
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <int DK, bool F32IN, int SF, int WF>
struct FwdCfg {
  static constexpr int BV = 64;               // value columns per workgroup
  static constexpr int MK = DK / 16;          // 16-row tiles of the state
  static constexpr int LDK = DK + 8;          // bf16 row stride of [64][DK] tiles
  static constexpr int L64 = 64 + 8;          // bf16 row stride of [*][64] tiles
  static constexpr int LF = 65;               // FP32 row stride of [64][64] tiles
  static constexpr int NIN = F32IN ? 2 : 1;   // bf16 planes of an input operand
  static constexpr int NW = (WF == 0) ? 2 : 1;
  static constexpr int KP = DK / 32;          // rows per thread when staging a K/Q tile
  static constexpr int KCG = DK / 8;          // 8-element column groups of a K/Q row
  static constexpr int VP = 2;                // rows per thread when staging the V block
};

template <int DK, bool F32IN, int SF, int WF>
struct FwdSmem {
  using C = FwdCfg<DK, F32IN, SF, WF>;
  bf16 K[C::NIN][64 * C::LDK];     // K rows (row-major)
  bf16 Kt[C::NIN][DK * C::L64];    // K transposed [dk][pos]
  bf16 Q[C::NIN][64 * C::LDK];
  bf16 Vt[C::NIN][C::BV * C::L64]; // V block transposed [v][pos]
  bf16 P[2][64 * C::L64];          // (Q K^T) * Gam, hi / lo; upper tiles stay 0
  bf16 T[4][64 * C::L64];          // T hi, T lo, T' hi, T' lo; upper tiles stay 0
  union {
    struct { float L[64 * C::LF]; float X[64 * C::LF]; } s;   // B..D
    bf16 W[C::NW][64 * C::LDK];                              // F..G: W codes or hi / lo
  } u;
  alignas(16) float gam2[64];                  // log2-scaled chunk-local cumsum of g
  alignas(16) float bet[64];
  alignas(16) float eg[64];                    // exp(gamma)
  alignas(16) float egc[64];                   // exp(gamma_n - gamma), 0 past the chunk end
  float red[16];                               // 0..3 W amax, 4..7 S amax, 8 exp(gamma_n)
};

// 8 consecutive input elements as loaded from HBM.
template <bool F32IN> struct Raw8 { bf16x8 v; };
template <> struct Raw8<true> { float4 a, b; };

template <bool F32IN>
__device__ __forceinline__ Raw8<F32IN> load_raw(const void* base, int64_t off, bool valid) {
  Raw8<F32IN> r;
  if constexpr (!F32IN) {
    if (valid) {
      r.v = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16*>(base) + off);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) r.v[e] = to_bf16(0.f);
    }
  } else {
    r.a = r.b = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid) {
      const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
      r.a = p[0];
      r.b = p[1];
    }
  }
  return r;
}

template <bool F32IN>
__device__ __forceinline__ void planes(const Raw8<F32IN>& r, bf16x8& hi, bf16x8& lo) {
  if constexpr (!F32IN) {
    hi = r.v;
  } else {
    const float xs[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bf16 h, l;
      split2(xs[e], h, l);
      hi[e] = h;
      lo[e] = l;
    }
  }
}


// Lower 16x16 tiles (mi >= mj) of a 64x64 matrix, in a fixed order.
__device__ __forceinline__ void lower_tile(int t, int& mi, int& mj) {
  mi = (t >= 1) + (t >= 3) + (t >= 6);
  mj = t - (mi * (mi + 1)) / 2;
}


// One 16x16 tile (mi, mj) of A B^T (A, B: [64][DK] row-major bf16 planes in
// LDS) with all operand loads issued before the MFMA chain.
template <int DK, int LD, int NIN>
__device__ __forceinline__ f32x4 tile_abt(const bf16 (*A)[64 * LD], const bf16 (*B)[64 * LD],
                                          int mi, int mj, int r16, int grp) {
  constexpr int KS = DK / 32;
  bf16x8 a0[KS], b0[KS], a1[KS], b1[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    a0[kk] = lds_nat(A[0], 16 * mi + r16, LD, 32 * kk, grp);
    b0[kk] = lds_nat(B[0], 16 * mj + r16, LD, 32 * kk, grp);
    if constexpr (NIN == 2) {
      a1[kk] = lds_nat(A[1], 16 * mi + r16, LD, 32 * kk, grp);
      b1[kk] = lds_nat(B[1], 16 * mj + r16, LD, 32 * kk, grp);
    }
  }
  f32x4 acc = zero4();
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    acc = mfma(a0[kk], b0[kk], acc);
    if constexpr (NIN == 2) {
      acc = mfma(a1[kk], b0[kk], acc);
      acc = mfma(a0[kk], b1[kk], acc);
    }
  }
  return acc;
}

template <int DK, bool F32IN, int SF, int WF>
__global__ void __launch_bounds__(256, 1) gdn_fwd_kernel(FwdKernelArgs a) {
  using C = FwdCfg<DK, F32IN, SF, WF>;
  constexpr int MK = C::MK, LDK = C::LDK, L64 = C::L64, LF = C::LF, NIN = C::NIN;
  constexpr int KP = C::KP, VP = C::VP;
  constexpr float LOG2E = 1.4426950408889634f;
  __shared__ __align__(16) FwdSmem<DK, F32IN, SF, WF> sm;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int lane = fresh_lane(), tid = wave * 64 + lane, r16 = lane & 15, grp = lane >> 4;
#define GDN_REFRESH() \
  lane = fresh_lane(); tid = wave * 64 + lane; r16 = lane & 15; grp = lane >> 4
  const int vb = blockIdx.x, h = blockIdx.y, n = blockIdx.z;
  const int Hv = a.Hv, Dv = a.Dv, Hqk = a.Hqk;
  const int hk = h / (Hv / Hqk);
  int bos, eos;
  seq_span(a, n, bos, eos);
  const int nchunks = (eos - bos + CHUNK - 1) / CHUNK;
  const int slot0 = n + bos / CHUNK;
  const int wcol = vb * C::BV + wave * 16;          // first value column of this wave
  const int64_t state_base = ((int64_t)n * Hv + h) * DK * Dv;

  // P and T upper tiles are read as zeros and never written
  for (int e = tid; e < 64 * L64; e += 256) {
    sm.P[0][e] = to_bf16(0.f);
    sm.P[1][e] = to_bf16(0.f);
#pragma unroll
    for (int p = 0; p < 4; ++p) sm.T[p][e] = to_bf16(0.f);
  }

  // ---- state in accumulator layout: S[mt][i] = S[16 mt + 4 grp + i][col]
  f32x4 S[MK];
  if (a.h0) {
    const float* hp = a.h0 + state_base + wcol + r16;
#pragma unroll
    for (int mt = 0; mt < MK; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[mt][i] = hp[(16 * mt + 4 * grp + i) * Dv];
  } else {
#pragma unroll
    for (int mt = 0; mt < MK; ++mt) S[mt] = zero4();
  }

  // ---- prefetch registers for the next chunk
  Raw8<F32IN> kr[KP], qr[KP], vr[VP];
  float g_pre = 0.f, b_pre = 0.f;
  // K/Q: thread -> column group tid % KCG, rows KP * (tid / KCG) + p; a wave
  // reads whole rows (coalesced). V: column group tid % 8, rows 2 (tid / 8) + p.
  auto prefetch = [&](int t0, int nc) {
#pragma unroll
    for (int p = 0; p < KP; ++p) {
      const int row = KP * (tid / C::KCG) + p, c8 = (tid % C::KCG) * 8;
      const int64_t off = ((int64_t)(t0 + row) * Hqk + hk) * DK + c8;
      kr[p] = load_raw<F32IN>(a.k, off, row < nc);
      qr[p] = load_raw<F32IN>(a.q, off, row < nc);
    }
#pragma unroll
    for (int p = 0; p < VP; ++p) {
      const int row = VP * (tid / 8) + p, c8 = (tid % 8) * 8;
      const int64_t off = ((int64_t)(t0 + row) * Hv + h) * Dv + vb * C::BV + c8;
      vr[p] = load_raw<F32IN>(a.v, off, row < nc);
    }
    const int64_t gi = (int64_t)(t0 + lane) * Hv + h;
    g_pre = lane < nc ? a.g[gi] : 0.f;
    b_pre = lane < nc ? a.beta[gi] : 0.f;
  };
  if (nchunks > 0) prefetch(bos, min(CHUNK, eos - bos));

  // O of the previous chunk, stored once the next chunk's inputs have arrived:
  // loads and stores share one completion counter, so storing right before
  // the wait for the prefetched inputs would make that wait cover the stores.
  f32x4 Oprev[4];
  int64_t oprev_base = -1;
  int oprev_nc = 0;
  auto store_o = [&]() {
    if (oprev_base < 0) return;
    const int r16_ = __lane_id() & 15, grp_ = __lane_id() >> 4;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * mt + 4 * grp_ + i;
        if (row < oprev_nc) {
          const int64_t off = oprev_base + r16_ + (int64_t)row * Hv * Dv;
          if constexpr (F32IN) reinterpret_cast<float*>(a.o)[off] = Oprev[mt][i];
          else reinterpret_cast<bf16*>(a.o)[off] = to_bf16(Oprev[mt][i]);
        }
      }
  };

  for (int c = 0; c < nchunks; ++c) {
    const int t0 = bos + c * CHUNK;
    const int nc = min(CHUNK, eos - t0);
    const int slot = slot0 + c;

    // ------------------------------------- A: stage inputs, gates, prefetch
    GDN_REFRESH();
    {
      // K, Q rows in paired order along dk; K^T and V^T in paired order along
      // the position index (KP or 2 consecutive rows land contiguously).
      const int kc8 = (tid % C::KCG) * 8, kr0 = KP * (tid / C::KCG);
      const int kd0 = pperm(kc8), kd1 = pperm(kc8 + 4), kpos = pperm(kr0);
      bf16x8 kh[KP], kl[KP];
#pragma unroll
      for (int p = 0; p < KP; ++p) {
        bf16x8 qh, ql;
        planes<F32IN>(kr[p], kh[p], kl[p]);
        planes<F32IN>(qr[p], qh, ql);
#pragma unroll
        for (int pl = 0; pl < NIN; ++pl) {
          const bf16x8 kv = pl ? kl[p] : kh[p], qv = pl ? ql : qh;
          bf16* kd = &sm.K[pl][(kr0 + p) * LDK];
          bf16* qd = &sm.Q[pl][(kr0 + p) * LDK];
          *reinterpret_cast<bf16x4*>(kd + kd0) = bf16x4{kv[0], kv[1], kv[2], kv[3]};
          *reinterpret_cast<bf16x4*>(kd + kd1) = bf16x4{kv[4], kv[5], kv[6], kv[7]};
          *reinterpret_cast<bf16x4*>(qd + kd0) = bf16x4{qv[0], qv[1], qv[2], qv[3]};
          *reinterpret_cast<bf16x4*>(qd + kd1) = bf16x4{qv[4], qv[5], qv[6], qv[7]};
        }
      }
#pragma unroll
      for (int pl = 0; pl < NIN; ++pl)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          bf16* kt = &sm.Kt[pl][(kc8 + j) * L64 + kpos];
          if constexpr (KP == 4) {
            const bf16x8* src = pl ? kl : kh;
            *reinterpret_cast<bf16x4*>(kt) = bf16x4{src[0][j], src[1][j], src[2][j], src[3][j]};
          } else {
            const bf16x8* src = pl ? kl : kh;
            *reinterpret_cast<__attribute__((ext_vector_type(2))) bf16*>(kt) =
                (__attribute__((ext_vector_type(2))) bf16){src[0][j], src[1][j]};
          }
        }
      const int vc8 = (tid % 8) * 8, vpos = pperm(VP * (tid / 8));
      bf16x8 vh[VP], vl[VP];
#pragma unroll
      for (int p = 0; p < VP; ++p) planes<F32IN>(vr[p], vh[p], vl[p]);
#pragma unroll
      for (int pl = 0; pl < NIN; ++pl)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bf16x8* src = pl ? vl : vh;
          *reinterpret_cast<__attribute__((ext_vector_type(2))) bf16*>(
              &sm.Vt[pl][(vc8 + j) * L64 + vpos]) =
              (__attribute__((ext_vector_type(2))) bf16){src[0][j], src[1][j]};
        }
      // gates, one row per lane (every wave holds them; wave 0 publishes)
      if (wave == 0) {
        const bool valid = lane < nc;
        const float g2 = wave_incl_scan(valid ? g_pre * LOG2E : 0.f);
        const float g2n = read_lane(g2, nc - 1);
        sm.gam2[lane] = g2;
        sm.bet[lane] = valid ? b_pre : 0.f;
        sm.eg[lane] = fexp2(g2);
        sm.egc[lane] = valid ? fexp2(g2n - g2) : 0.f;
        if (lane == 0) sm.red[8] = fexp2(g2n);
      }
      store_o();
      if (c + 1 < nchunks) prefetch(t0 + CHUNK, min(CHUNK, eos - t0 - CHUNK));
    }
    __syncthreads();

    // ------------------------------------- B: L = beta_i (K K^T) Gam, strict lower
    GDN_REFRESH();
#pragma unroll
    for (int it = 0; it < 3; ++it) {
      const int jb = wave + 4 * it;
      if (jb >= 10) break;
      int mi, mj;
      lower_tile(jb, mi, mj);
      const f32x4 acc = tile_abt<DK, LDK, NIN>(sm.K, sm.K, mi, mj, r16, grp);
      const int cj = 16 * mj + r16;
      const float gj = sm.gam2[cj];
      float gr[4], br[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        gr[i] = sm.gam2[16 * mi + 4 * grp + i];
        br[i] = sm.bet[16 * mi + 4 * grp + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * mi + 4 * grp + i;
        const float lv = br[i] * acc[i] * fexp2(gr[i] - gj);
        sm.u.s.L[row * LF + cj] = (row > cj) ? lv : 0.f;
      }
    }
    __syncthreads();

    // Writes one FP32 entry of X as T = x beta_col and T' = T exp(gamma_col).
    auto put_T = [&](int row, int cj, float x, float bc, float ec) {
      const float t = x * bc, tp = t * ec;
      const int o = row * L64 + pperm(cj);
      bf16 hi, lo;
      split2(t, hi, lo);
      sm.T[0][o] = hi;
      sm.T[1][o] = lo;
      split2(tp, hi, lo);
      sm.T[2][o] = hi;
      sm.T[3][o] = lo;
    };

    // ----------------- C: wave 0 solve (diagonal blocks, 16-merges); 1-3 P
    GDN_REFRESH();
    if (wave == 0) {
      const int b = lane >> 4, cc = lane & 15;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = (r == cc) ? 1.f : 0.f;
      const float* Lb = &sm.u.s.L[(16 * b) * LF + 16 * b];
#pragma unroll
      for (int j = 0; j < 15; ++j)
#pragma unroll
        for (int r = j + 1; r < 16; ++r) x[r] -= Lb[r * LF + j] * x[j];
      {
        const int cj = 16 * b + cc;
        const float bc = sm.bet[cj], ec = sm.eg[cj];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sm.u.s.X[(16 * b + r) * LF + cj] = x[r];
          put_T(16 * b + r, cj, x[r], bc, ec);
        }
      }
      // X_BA = -X_BB (L_BA X_AA) for the block pairs (A, B) = (0, 1), (2, 3)
      f32x4 y[2], z[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int A = 2 * p, B = 2 * p + 1;
        y[p] = zero4();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          y[p] = mfma_f32(sm.u.s.L[(16 * B + r16) * LF + 16 * A + 4 * kk + grp],
                          sm.u.s.X[(16 * A + 4 * kk + grp) * LF + 16 * A + r16], y[p]);
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int B = 2 * p + 1;
        z[p] = zero4();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)                  // K order: 4 grp + kk
          z[p] = mfma_f32(sm.u.s.X[(16 * B + r16) * LF + 16 * B + 4 * grp + kk], y[p][kk], z[p]);
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int A = 2 * p, B = 2 * p + 1;
        const int cj = 16 * A + r16;
        const float bc = sm.bet[cj], ec = sm.eg[cj];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * B + 4 * grp + i;
          sm.u.s.X[row * LF + cj] = -z[p][i];
          put_T(row, cj, -z[p][i], bc, ec);
        }
      }
    } else {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int jb = wave - 1 + 3 * it;
        if (jb >= 10) break;
        int mi, mj;
        lower_tile(jb, mi, mj);
        const f32x4 acc = tile_abt<DK, LDK, NIN>(sm.Q, sm.K, mi, mj, r16, grp);
        const int cj = 16 * mj + r16;
        const float gj = sm.gam2[cj];
        float gr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) gr[i] = sm.gam2[16 * mi + 4 * grp + i];
        const int pc = pperm(cj);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * mi + 4 * grp + i;
          const float pv = (row >= cj) ? acc[i] * fexp2(gr[i] - gj) : 0.f;
          bf16 hi, lo;
          split2(pv, hi, lo);
          sm.P[0][row * L64 + pc] = hi;
          sm.P[1][row * L64 + pc] = lo;
        }
      }
    }
    __syncthreads();

    // --------------- D: waves 0-1 32-block merge; waves 2-3 W rows 0..31
    GDN_REFRESH();
    constexpr int NWC = DK / 32;                       // W column tiles per wave
    f32x4 Wt[2][NWC];                                 // this wave's 2 x NWC tiles of W
    // waves 2, 3: rows 0..31, column tiles (wave - 2) * NWC + d
    // waves 0, 1: rows 32..63, column tiles wave * NWC + d
    const int wrow0 = wave < 2 ? 32 : 0;
    const int wct0 = (wave & 1) * NWC;
    if (wave < 2) {
      const int tj = wave;
      f32x4 y[2] = {zero4(), zero4()};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if (s < 4 * tj) continue;                     // X_AA is lower triangular
        const float bx = sm.u.s.X[(4 * s + grp) * LF + 16 * tj + r16];
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
          y[ti] = mfma_f32(sm.u.s.L[(32 + 16 * ti + r16) * LF + 4 * s + grp], bx, y[ti]);
      }
      const int cj = 16 * tj + r16;
      const float bc = sm.bet[cj], ec = sm.eg[cj];
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) {
        f32x4 z = zero4();
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          if (kt > ti) continue;                      // X_BB is lower triangular
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)              // K order: 16 kt + 4 grp + kk
            z = mfma_f32(sm.u.s.X[(32 + 16 * ti + r16) * LF + 32 + 16 * kt + 4 * grp + kk],
                         y[kt][kk], z);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) put_T(32 + 16 * ti + 4 * grp + i, cj, -z[i], bc, ec);
      }
    } else {
      bf16x8 ta[2][2], kb[NWC][NIN];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        ta[mt][0] = lds_nat(sm.T[2], 16 * mt + r16, L64, 0, grp);
        ta[mt][1] = lds_nat(sm.T[3], 16 * mt + r16, L64, 0, grp);
      }
#pragma unroll
      for (int d = 0; d < NWC; ++d)
#pragma unroll
        for (int pl = 0; pl < NIN; ++pl)
          kb[d][pl] = lds_nat(sm.Kt[pl], 16 * (wct0 + d) + r16, L64, 0, grp);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int d = 0; d < NWC; ++d) {
          f32x4 acc = mfma(ta[mt][0], kb[d][0], zero4());
          acc = mfma(ta[mt][1], kb[d][0], acc);
          if constexpr (F32IN) acc = mfma(ta[mt][0], kb[d][NIN - 1], acc);
          Wt[mt][d] = acc;
        }
    }
    __syncthreads();

    // ------------------- E: W rows 32..63 (waves 0, 1), U = T V, amax partials
    GDN_REFRESH();
    if (wave < 2) {
      bf16x8 ta[2][2][2], kb[2][NWC][NIN];            // [t][kk][hi/lo], [kk][d][plane]
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          ta[t][kk][0] = lds_nat(sm.T[2], 16 * (2 + t) + r16, L64, 32 * kk, grp);
          ta[t][kk][1] = lds_nat(sm.T[3], 16 * (2 + t) + r16, L64, 32 * kk, grp);
        }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int d = 0; d < NWC; ++d)
#pragma unroll
          for (int pl = 0; pl < NIN; ++pl)
            kb[kk][d][pl] = lds_nat(sm.Kt[pl], 16 * (wct0 + d) + r16, L64, 32 * kk, grp);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int d = 0; d < NWC; ++d) {
          f32x4 acc = zero4();
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            acc = mfma(ta[t][kk][0], kb[kk][d][0], acc);
            acc = mfma(ta[t][kk][1], kb[kk][d][0], acc);
            if constexpr (F32IN) acc = mfma(ta[t][kk][0], kb[kk][d][NIN - 1], acc);
          }
          Wt[t][d] = acc;
        }
    }
    f32x4 U[4];
    {
      bf16x8 ua[2][4][2], vb_[2][NIN];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int pl = 0; pl < NIN; ++pl)
          vb_[kk][pl] = lds_nat(sm.Vt[pl], wave * 16 + r16, L64, 32 * kk, grp);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          if (kk > mt / 2) continue;                  // T is lower triangular
          ua[kk][mt][0] = lds_nat(sm.T[0], 16 * mt + r16, L64, 32 * kk, grp);
          ua[kk][mt][1] = lds_nat(sm.T[1], 16 * mt + r16, L64, 32 * kk, grp);
        }
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) U[mt] = zero4();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          if (kk > mt / 2) continue;
          U[mt] = mfma(ua[kk][mt][0], vb_[kk][0], U[mt]);
          U[mt] = mfma(ua[kk][mt][1], vb_[kk][0], U[mt]);
          if constexpr (F32IN) U[mt] = mfma(ua[kk][mt][0], vb_[kk][NIN - 1], U[mt]);
        }
    }
    if constexpr (WF != 0) {
      float m = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int d = 0; d < NWC; ++d)
#pragma unroll
          for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(Wt[t][d][i]));
      m = wave_max(m);
      if (lane == 0) sm.red[wave] = m;
    }
    if constexpr (SF != 0) {
      float m = 0.f;
#pragma unroll
      for (int mt = 0; mt < MK; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(S[mt][i]));
      m = wave_max(m);
      if (lane == 0) sm.red[4 + wave] = m;
    }
    __syncthreads();                                  // L, X dead; amax partials ready

    // ------------------------------------------- F: QDQ of W and of S
    GDN_REFRESH();
    float dW = 1.f;
    {
      const bool save = WF != 0 && a.w_codes != nullptr && vb == 0;
      float rW = 1.f;
      if constexpr (WF != 0) {
        const float amax = fmaxf(fmaxf(sm.red[0], sm.red[1]), fmaxf(sm.red[2], sm.red[3]));
        dW = qdq_scale<WF>(amax);
        rW = 1.0f / dW;
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int d = 0; d < NWC; ++d) {
          const int dcol = 16 * (wct0 + d) + r16, pc = pperm(dcol);
          const int row0 = wrow0 + 16 * t + 4 * grp;
          const float w[4] = {Wt[t][d][0], Wt[t][d][1], Wt[t][d][2], Wt[t][d][3]};
          if constexpr (WF != 0) {
            float cq[4];
            uint32_t bytes;
            quant4<WF>(w, rW, cq, bytes);
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.u.W[0][(row0 + i) * LDK + pc] = to_bf16(cq[i]);
            if (save) {
              uint8_t* wp = a.w_codes + ((int64_t)t0 * Hv + h) * DK + dcol;
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (row0 + i < nc) wp[(row0 + i) * Hv * DK] = (bytes >> (8 * i)) & 0xFFu;
            }
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              bf16 hi, lo;
              split2(w[i], hi, lo);
              sm.u.W[0][(row0 + i) * LDK + pc] = hi;
              sm.u.W[C::NW - 1][(row0 + i) * LDK + pc] = lo;
            }
          }
        }
      if (save && tid == 0) a.w_scale[(int64_t)slot * Hv + h] = dW;
    }
    float dS = 1.f;
    if constexpr (SF != 0) {
      const int gs = a.block_v / 16;                  // 16-col tiles per scale tile
      const int g0 = (wave / gs) * gs;
      float amax = 0.f;
      for (int t = g0; t < g0 + gs; ++t) amax = fmaxf(amax, sm.red[4 + t]);
      dS = qdq_scale<SF>(amax);
      const float rS = 1.0f / dS;
      uint8_t* sb = a.s_codes ? a.s_codes + ((int64_t)slot * Hv + h) * DK * Dv + wcol + r16 : nullptr;
#pragma unroll
      for (int mt = 0; mt < MK; ++mt) {
        const float x[4] = {S[mt][0], S[mt][1], S[mt][2], S[mt][3]};
        float cq[4];
        uint32_t bytes;
        quant4<SF>(x, rS, cq, bytes);
#pragma unroll
        for (int i = 0; i < 4; ++i) S[mt][i] = cq[i];                // codes
        if (sb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) sb[(16 * mt + 4 * grp + i) * Dv] = (bytes >> (8 * i)) & 0xFFu;
        }
      }
      if (sb && wave == g0 && lane == 0)
        a.s_scale[((int64_t)slot * Hv + h) * (Dv / a.block_v) + wcol / a.block_v] = dS;
    } else if (a.s_f32) {
      float* sb = a.s_f32 + ((int64_t)slot * Hv + h) * DK * Dv + wcol + r16;
#pragma unroll
      for (int mt = 0; mt < MK; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sb[(16 * mt + 4 * grp + i) * Dv] = S[mt][i];
    }
    __syncthreads();                                  // W in LDS

    // ------------------------------- G: Vnew, O, state update
    GDN_REFRESH();
    // state as B operand (paired-tile K order over dk)
    bf16x8 bSh[MK / 2], bSl[MK / 2];
#pragma unroll
    for (int kk = 0; kk < MK / 2; ++kk) {
      if constexpr (SF != 0) {
        bSh[kk] = pack_pair(S[2 * kk], S[2 * kk + 1]);
      } else {
        pack_pair_split(S[2 * kk], S[2 * kk + 1], bSh[kk], bSl[kk]);
      }
    }
    f32x4 accw[4], accq[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) accw[mt] = accq[mt] = zero4();
    {
      // operands of k-step kk + 1 are loaded while k-step kk multiplies
      constexpr int NA = 2 + (WF == 0 ? 1 : 0) + (F32IN ? 1 : 0);   // A planes per row tile
      bf16x8 opA[2][4][NA];
      auto load_k = [&](int kk, bf16x8 (&dst)[4][NA]) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          dst[mt][0] = lds_nat(sm.u.W[0], 16 * mt + r16, LDK, 32 * kk, grp);
          dst[mt][1] = lds_nat(sm.Q[0], 16 * mt + r16, LDK, 32 * kk, grp);
          int q = 2;
          if constexpr (WF == 0) dst[mt][q++] = lds_nat(sm.u.W[C::NW - 1], 16 * mt + r16, LDK, 32 * kk, grp);
          if constexpr (F32IN) dst[mt][q++] = lds_nat(sm.Q[NIN - 1], 16 * mt + r16, LDK, 32 * kk, grp);
        }
      };
      load_k(0, opA[0]);
#pragma unroll
      for (int kk = 0; kk < MK / 2; ++kk) {
        if (kk + 1 < MK / 2) load_k(kk + 1, opA[(kk + 1) & 1]);
        const auto& op = opA[kk & 1];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          accw[mt] = mfma(op[mt][0], bSh[kk], accw[mt]);
          accq[mt] = mfma(op[mt][1], bSh[kk], accq[mt]);
          int q = 2;
          if constexpr (WF == 0) accw[mt] = mfma(op[mt][q++], bSh[kk], accw[mt]);
          if constexpr (F32IN) accq[mt] = mfma(op[mt][q++], bSh[kk], accq[mt]);
          if constexpr (SF == 0) {
            accw[mt] = mfma(op[mt][0], bSl[kk], accw[mt]);
            accq[mt] = mfma(op[mt][1], bSl[kk], accq[mt]);
          }
        }
      }
    }
    f32x4 Vn[4];
    {
      const float sc = dW * dS;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Vn[mt][i] = U[mt][i] - sc * accw[mt][i];
          accq[mt][i] *= dS;
        }
    }
    // Vnew and exp(gamma_n - gamma) Vnew as B operands (paired order over positions)
    bf16x8 bVh[2], bVl[2], bDh[2], bDl[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      pack_pair_split(Vn[2 * kk], Vn[2 * kk + 1], bVh[kk], bVl[kk]);
      const f32x4 e0 = *reinterpret_cast<const f32x4*>(&sm.egc[32 * kk + 4 * grp]);
      const f32x4 e1 = *reinterpret_cast<const f32x4*>(&sm.egc[32 * kk + 16 + 4 * grp]);
      f32x4 d0, d1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        d0[i] = e0[i] * Vn[2 * kk][i];
        d1[i] = e1[i] * Vn[2 * kk + 1][i];
      }
      pack_pair_split(d0, d1, bDh[kk], bDl[kk]);
    }
    // O = scale (exp(gamma) Q Sq + P Vnew)
    {
      const int64_t obase = ((int64_t)t0 * Hv + h) * Dv + wcol + r16;
      f32x4 aco[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) aco[mt] = zero4();
      bf16x8 pop[2][4][2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          if (kk > mt / 2) continue;
          pop[kk][mt][0] = lds_nat(sm.P[0], 16 * mt + r16, L64, 32 * kk, grp);
          pop[kk][mt][1] = lds_nat(sm.P[1], 16 * mt + r16, L64, 32 * kk, grp);
        }
      float egr[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) egr[mt][i] = sm.eg[16 * mt + 4 * grp + i];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          if (kk > mt / 2) continue;
          aco[mt] = mfma(pop[kk][mt][0], bVh[kk], aco[mt]);
          aco[mt] = mfma(pop[kk][mt][1], bVh[kk], aco[mt]);
          aco[mt] = mfma(pop[kk][mt][0], bVl[kk], aco[mt]);
        }
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) Oprev[mt][i] = a.scale * (egr[mt][i] * accq[mt][i] + aco[mt][i]);
      oprev_base = obase - r16;
      oprev_nc = nc;
    }
    // S = exp(gamma_n) Sq + K^T (exp(gamma_n - gamma) Vnew), accumulated in place
    {
      const float egC = sm.red[8];
#pragma unroll
      for (int mt = 0; mt < MK; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[mt][i] = egC * ((SF != 0) ? S[mt][i] * dS : S[mt][i]);
      bf16x8 kop[2][MK][NIN];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int mt = 0; mt < MK; ++mt)
#pragma unroll
          for (int pl = 0; pl < NIN; ++pl)
            kop[kk][mt][pl] = lds_nat(sm.Kt[pl], 16 * mt + r16, L64, 32 * kk, grp);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int mt = 0; mt < MK; ++mt) {
          S[mt] = mfma(kop[kk][mt][0], bDh[kk], S[mt]);
          S[mt] = mfma(kop[kk][mt][0], bDl[kk], S[mt]);
          if constexpr (F32IN) S[mt] = mfma(kop[kk][mt][NIN - 1], bDh[kk], S[mt]);
        }
      }
    }
    __syncthreads();                                  // LDS reused by the next chunk
  }

  store_o();
  if (a.ht) {
    GDN_REFRESH();
#pragma unroll
    for (int mt = 0; mt < MK; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a.ht[state_base + (int64_t)(16 * mt + 4 * grp + i) * Dv + wcol + r16] = S[mt][i];
  }
#undef GDN_REFRESH
}

template <int DK, bool F32IN, int SF, int WF>
static hipError_t launch_one(const FwdConfig& cfg, const FwdKernelArgs& a, hipStream_t stream) {
  dim3 grid(cfg.Dv / 64, cfg.Hv, cfg.N);
  hipLaunchKernelGGL((gdn_fwd_kernel<DK, F32IN, SF, WF>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int DK, bool F32IN>
static hipError_t launch_fmt(const FwdConfig& cfg, const FwdKernelArgs& a, hipStream_t s) {
#define GDN_CASE(SFv, WFv) \
  if (cfg.state_fmt == SFv && cfg.w_fmt == WFv) return launch_one<DK, F32IN, SFv, WFv>(cfg, a, s);
  GDN_CASE(0, 0) GDN_CASE(0, 1) GDN_CASE(0, 2)
  GDN_CASE(1, 0) GDN_CASE(1, 1) GDN_CASE(1, 2)
  GDN_CASE(2, 0) GDN_CASE(2, 1) GDN_CASE(2, 2)
#undef GDN_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_fused(const FwdConfig& cfg, const FwdKernelArgs& a, hipStream_t stream) {
  if (cfg.N == 0 || cfg.Hv == 0) return hipSuccess;
  if (cfg.f32_io && cfg.Dk == 64) return launch_fmt<64, true>(cfg, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdn
