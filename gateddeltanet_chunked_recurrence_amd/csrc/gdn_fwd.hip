// Chunked gated delta rule forward with dynamic state/W fake QDQ, fused into
// one kernel per (sequence, value head, 64-wide value block).
//
// Work unit and residency. A workgroup of 4 waves owns the state tile
// S[Dk, 64] of one (sequence, head, value block) and walks the sequence's
// chunks in order; the state never leaves registers (wave w holds columns
// 16w..16w+15 in MFMA accumulator layout). Everything a chunk needs that does
// not depend on the state (gate cumsum, gated K K^T, the exact solve, W and
// its QDQ, U, masked Q K^T) is rebuilt per chunk in LDS from q, k, v, g, beta,
// so HBM traffic is one read of the inputs and one write of O (and ht).
//
// Precision. Operands that are bf16 inputs (q, k, v) are exact in bf16. Every
// FP32 operand (T, T', P, Vnew, the unquantized state) is split as hi + lo
// bf16 and multiplied in two or three MFMA passes (hi*x + lo*x [+ hi*lo]),
// which keeps ~16 mantissa bits. QDQ codes (E4M3 values, integers <= 127) are
// exact in bf16, so products with quantized operands are single passes and
// the scales are applied after accumulation. Diagonal gate factors are moved
// onto the FP32 side of each product so bf16 inputs stay exact, and
// exp(gamma_i - gamma_j) is always formed from the difference (the split
// exp(gamma_i) * exp(-gamma_j) overflows for strong gates).
//
// Steps per chunk ("[1/4] GDN state/W QAT foundation", "What does this PR
// do?"; the chunk equations are listed in include/gdn.h):
//   P0 load K, K^T, Q, V^T tiles to LDS; wave 0 forms the gates
//   P1 L = beta_i (K K^T) * Gam (strict lower), P = (Q K^T) * Gam (lower)
//   P2 16x16 diagonal blocks of X = (I + L)^-1 by substitution (FP32)
//   P3 off-diagonal blocks of X, block row by block row (FP32)
//   P4 T = X diag(beta), T' = T diag(exp(gamma)) -> hi/lo bf16
//   P5 W = T' K -> QDQ_W -> LDS; U = T V -> registers
//   P6 Sq = QDQ_S(S) per [Dk, block_v] tile (wave max + LDS)
//   P7 Vnew = U - Wq Sq; O = scale(exp(gamma) Q Sq + P Vnew);
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
  static constexpr int LF = 64 + 4;           // FP32 row stride of [64][64] tiles
  static constexpr int NIN = F32IN ? 2 : 1;   // bf16 planes of an input operand
  static constexpr int NW = (WF == 0) ? 2 : 1;
};

template <int DK, bool F32IN, int SF, int WF>
struct FwdSmem {
  using C = FwdCfg<DK, F32IN, SF, WF>;
  bf16 K[C::NIN][64 * C::LDK];     // K rows (row-major)
  bf16 Kt[C::NIN][DK * C::L64];    // K transposed [dk][pos]
  bf16 Q[C::NIN][64 * C::LDK];
  bf16 Vt[C::NIN][C::BV * C::L64]; // V block transposed [v][pos]
  bf16 P[2][64 * C::L64];          // (Q K^T) * Gam, hi / lo
  union {                          // region A
    struct { float L[64 * C::LF]; float R[3 * 256]; } s;   // P1..P3
    bf16 T[4][64 * C::L64];        // P4..P5: T hi, T lo, T' hi, T' lo
  } a;
  union {                          // region B
    float X[64 * C::LF];           // P2..P4
    bf16 W[C::NW][64 * C::LDK];    // P5..P7: W codes, or W hi / lo
  } b;
  float gam[64], eg[64], egc[64], bet[64];
  float red[8];
  float amax16[C::BV / 16];
};

// 8 consecutive input elements starting at `p` as bf16 planes (hi, and lo for
// FP32 inputs). Rows past the chunk end read as zeros.
template <bool F32IN>
__device__ __forceinline__ void load8(const void* base, int64_t off, bool valid,
                                      bf16x8& hi, bf16x8& lo) {
  if constexpr (!F32IN) {
    if (valid) {
      hi = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16*>(base) + off);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) hi[e] = to_bf16(0.f);
    }
  } else {
    float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
    if (valid) {
      const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
      x0 = p[0];
      x1 = p[1];
    }
    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bf16 h, l;
      split2(xs[e], h, l);
      hi[e] = h;
      lo[e] = l;
    }
  }
}

template <int DK, bool F32IN, int SF, int WF>
__global__ void __launch_bounds__(256, 1) gdn_fwd_kernel(FwdKernelArgs a) {
  using C = FwdCfg<DK, F32IN, SF, WF>;
  constexpr int MK = C::MK, LDK = C::LDK, L64 = C::L64, LF = C::LF, NIN = C::NIN;
  __shared__ __align__(16) FwdSmem<DK, F32IN, SF, WF> sm;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, grp = lane >> 4;
  const int vb = blockIdx.x, h = blockIdx.y, n = blockIdx.z;
  const int Hv = a.Hv, Dv = a.Dv;
  const int hk = h / (Hv / a.Hqk);
  int bos, eos;
  if (a.cu_seqlens) {
    bos = a.cu_seqlens[n];
    eos = a.cu_seqlens[n + 1];
  } else {
    bos = n * a.T;
    eos = bos + a.T;
  }
  const int nchunks = (eos - bos + CHUNK - 1) / CHUNK;
  const int slot0 = n + bos / CHUNK;
  const int wcol = vb * C::BV + wave * 16;          // first value column of this wave
  const int col = wcol + r16;                       // this lane's value column
  const int64_t state_base = ((int64_t)n * Hv + h) * DK * Dv;

  // ---- state in accumulator layout: S[mt][i] = S[16 mt + 4 grp + i][col]
  f32x4 S[MK];
#pragma unroll
  for (int mt = 0; mt < MK; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      S[mt][i] = a.h0 ? a.h0[state_base + (int64_t)(16 * mt + 4 * grp + i) * Dv + col] : 0.f;

  for (int c = 0; c < nchunks; ++c) {
    const int t0 = bos + c * CHUNK;
    const int nc = min(CHUNK, eos - t0);
    const int slot = slot0 + c;

    // ------------------------------------------------------------ P0: loads
    {
      constexpr int PER_ROW = DK / 8;                 // 8-element groups per row
#pragma unroll
      for (int p = 0; p < (64 * PER_ROW) / 256; ++p) {
        const int e = p * 256 + tid;
        const int row = e / PER_ROW, c8 = (e % PER_ROW) * 8;
        const bool valid = row < nc;
        const int64_t off = ((int64_t)(t0 + row) * a.Hqk + hk) * DK + c8;
        bf16x8 kh, kl, qh, ql;
        load8<F32IN>(a.k, off, valid, kh, kl);
        load8<F32IN>(a.q, off, valid, qh, ql);
        *reinterpret_cast<bf16x8*>(&sm.K[0][row * LDK + c8]) = kh;
        *reinterpret_cast<bf16x8*>(&sm.Q[0][row * LDK + c8]) = qh;
#pragma unroll
        for (int j = 0; j < 8; ++j) sm.Kt[0][(c8 + j) * L64 + row] = kh[j];
        if constexpr (F32IN) {
          *reinterpret_cast<bf16x8*>(&sm.K[1][row * LDK + c8]) = kl;
          *reinterpret_cast<bf16x8*>(&sm.Q[1][row * LDK + c8]) = ql;
#pragma unroll
          for (int j = 0; j < 8; ++j) sm.Kt[1][(c8 + j) * L64 + row] = kl[j];
        }
      }
      constexpr int VPR = C::BV / 8;
#pragma unroll
      for (int p = 0; p < (64 * VPR) / 256; ++p) {
        const int e = p * 256 + tid;
        const int row = e / VPR, c8 = (e % VPR) * 8;
        const bool valid = row < nc;
        const int64_t off = ((int64_t)(t0 + row) * Hv + h) * Dv + vb * C::BV + c8;
        bf16x8 vh, vl;
        load8<F32IN>(a.v, off, valid, vh, vl);
#pragma unroll
        for (int j = 0; j < 8; ++j) sm.Vt[0][(c8 + j) * L64 + row] = vh[j];
        if constexpr (F32IN) {
#pragma unroll
          for (int j = 0; j < 8; ++j) sm.Vt[1][(c8 + j) * L64 + row] = vl[j];
        }
      }
      if (wave == 0) {
        const bool valid = lane < nc;
        const int64_t gi = (int64_t)(t0 + lane) * Hv + h;
        const float gv = valid ? a.g[gi] : 0.f;
        const float bv = valid ? a.beta[gi] : 0.f;
        const float gam = wave_incl_scan(gv, lane);
        const float gamC = __shfl(gam, nc - 1, WAVE);
        sm.gam[lane] = gam;
        sm.eg[lane] = expf(gam);
        sm.egc[lane] = valid ? expf(gamC - gam) : 0.f;
        sm.bet[lane] = bv;
        if (lane == 0) sm.red[4] = expf(gamC);
      }
    }
    __syncthreads();

    // ------------------------------------ P1: L and P (lower 16x16 tiles)
    {
      // 20 lower tiles (10 of K K^T, 10 of Q K^T), 5 per wave.
      for (int job = wave; job < 20; job += 4) {
        const bool isP = job >= 10;
        int t = isP ? job - 10 : job;                 // t -> (mi, mj), mj <= mi
        int mi = 0;
        while (t > mi) { t -= mi + 1; ++mi; }
        const int mj = t;
        const bf16(*X)[64 * LDK] = isP ? sm.Q : sm.K;
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) {
          const bf16x8 b0 = lds_nat(sm.K[0], 16 * mj + r16, LDK, 32 * kk, grp);
          const bf16x8 a0 = lds_nat(X[0], 16 * mi + r16, LDK, 32 * kk, grp);
          acc = mfma(a0, b0, acc);
          if constexpr (F32IN) {
            const bf16x8 b1 = lds_nat(sm.K[1], 16 * mj + r16, LDK, 32 * kk, grp);
            const bf16x8 a1 = lds_nat(X[1], 16 * mi + r16, LDK, 32 * kk, grp);
            acc = mfma(a1, b0, acc);
            acc = mfma(a0, b1, acc);
          }
        }
        const int colj = 16 * mj + r16;
        const float gj = sm.gam[colj];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * mi + 4 * grp + i;
          const float gate = expf(sm.gam[row] - gj);
          if (!isP) {
            sm.a.s.L[row * LF + colj] = (row > colj) ? sm.bet[row] * acc[i] * gate : 0.f;
          } else {
            const float pv = (row >= colj) ? acc[i] * gate : 0.f;
            bf16 hi, lo;
            split2(pv, hi, lo);
            sm.P[0][row * L64 + colj] = hi;
            sm.P[1][row * L64 + colj] = lo;
          }
        }
      }
      // zero the upper tiles of P and of X (X's upper blocks stay zero)
      for (int e = tid; e < 6 * 256; e += 256) {
        int t = e / 256, rr = (e / 16) % 16, cc = e % 16;
        int bi = 0, bj = 1;                              // t -> (bi, bj), bj > bi
        while (t >= 3 - bi) { t -= 3 - bi; ++bi; }
        bj = bi + 1 + t;
        const int row = 16 * bi + rr, colj = 16 * bj + cc;
        sm.P[0][row * L64 + colj] = to_bf16(0.f);
        sm.P[1][row * L64 + colj] = to_bf16(0.f);
        sm.b.X[row * LF + colj] = 0.f;
      }
    }
    __syncthreads();

    // ------------------------------ P2: diagonal blocks of X = (I + L)^-1
    if (lane < 16) {
      const int b = wave, cc = lane;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = (r == cc) ? 1.f : 0.f;
        const float* Lr = &sm.a.s.L[(16 * b + r) * LF + 16 * b];
#pragma unroll
        for (int j = 0; j < r; ++j) s -= Lr[j] * x[j];
        x[r] = s;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.b.X[(16 * b + r) * LF + 16 * b + cc] = x[r];
    }
    __syncthreads();

    // ------------------------------ P3: off-diagonal blocks, block row i
    for (int bi = 1; bi < 4; ++bi) {
      // R_j = sum_{k=j}^{bi-1} L_{bi,k} X_{k,j}, j < bi
      for (int e = tid; e < bi * 256; e += 256) {
        const int j = e / 256, rr = (e / 16) % 16, cc = e % 16;
        const float* Lr = &sm.a.s.L[(16 * bi + rr) * LF];
        float s = 0.f;
        for (int m = 16 * j; m < 16 * bi; ++m) s += Lr[m] * sm.b.X[m * LF + 16 * j + cc];
        sm.a.s.R[e] = s;
      }
      __syncthreads();
      // X_{bi,j} = -X_{bi,bi} R_j
      for (int e = tid; e < bi * 256; e += 256) {
        const int j = e / 256, rr = (e / 16) % 16, cc = e % 16;
        const float* Xr = &sm.b.X[(16 * bi + rr) * LF + 16 * bi];
        const float* Rj = &sm.a.s.R[j * 256];
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < 16; ++m) s += Xr[m] * Rj[m * 16 + cc];
        sm.b.X[(16 * bi + rr) * LF + 16 * j + cc] = -s;
      }
      __syncthreads();
    }

    // -------------------- P4: T = X diag(beta), T' = T diag(exp(gamma))
    for (int e = tid; e < 64 * 64; e += 256) {
      const int row = e / 64, cc = e % 64;
      const float t = sm.b.X[row * LF + cc] * sm.bet[cc];
      const float tp = t * sm.eg[cc];
      bf16 hi, lo;
      split2(t, hi, lo);
      sm.a.T[0][row * L64 + cc] = hi;
      sm.a.T[1][row * L64 + cc] = lo;
      split2(tp, hi, lo);
      sm.a.T[2][row * L64 + cc] = hi;
      sm.a.T[3][row * L64 + cc] = lo;
    }
    __syncthreads();

    // ----------------------------------------- P5: W = T' K, U = T V
    constexpr int DTW = MK / 4;                       // W column tiles per wave
    f32x4 Wacc[4][DTW];
    float wmax = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int dt = 0; dt < DTW; ++dt) {
        const int dtile = wave * DTW + dt;
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (kk > mt / 2) continue;                  // T' is lower triangular
          const bf16x8 bk = lds_nat(sm.Kt[0], 16 * dtile + r16, L64, 32 * kk, grp);
          const bf16x8 th = lds_nat(sm.a.T[2], 16 * mt + r16, L64, 32 * kk, grp);
          const bf16x8 tl = lds_nat(sm.a.T[3], 16 * mt + r16, L64, 32 * kk, grp);
          acc = mfma(th, bk, acc);
          acc = mfma(tl, bk, acc);
          if constexpr (F32IN) {
            const bf16x8 bkl = lds_nat(sm.Kt[1], 16 * dtile + r16, L64, 32 * kk, grp);
            acc = mfma(th, bkl, acc);
          }
        }
        Wacc[mt][dt] = acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) wmax = fmaxf(wmax, fabsf(acc[i]));
      }
    f32x4 U[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (kk > mt / 2) continue;
        const bf16x8 bv = lds_nat(sm.Vt[0], wave * 16 + r16, L64, 32 * kk, grp);
        const bf16x8 th = lds_nat(sm.a.T[0], 16 * mt + r16, L64, 32 * kk, grp);
        const bf16x8 tl = lds_nat(sm.a.T[1], 16 * mt + r16, L64, 32 * kk, grp);
        acc = mfma(th, bv, acc);
        acc = mfma(tl, bv, acc);
        if constexpr (F32IN) {
          const bf16x8 bvl = lds_nat(sm.Vt[1], wave * 16 + r16, L64, 32 * kk, grp);
          acc = mfma(th, bvl, acc);
        }
      }
      U[mt] = acc;
    }
    float dW = 1.f;
    if constexpr (WF != 0) {
      wmax = wave_max(wmax);
      if (lane == 0) sm.red[wave] = wmax;
    }
    __syncthreads();                                  // X dead, W region free; amax ready
    if constexpr (WF != 0) {
      const float amax = fmaxf(fmaxf(sm.red[0], sm.red[1]), fmaxf(sm.red[2], sm.red[3]));
      dW = qdq_scale<WF>(amax);
      const float rW = 1.0f / dW;
      const bool save = a.w_codes != nullptr && vb == 0;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int dt = 0; dt < DTW; ++dt) {
          const int dcol = 16 * (wave * DTW + dt) + r16;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * mt + 4 * grp + i;
            const float cq = round_code<WF>(Wacc[mt][dt][i] * rW);
            sm.b.W[0][row * LDK + dcol] = to_bf16(cq);
            if (save && row < nc)
              a.w_codes[((int64_t)(t0 + row) * Hv + h) * DK + dcol] = code_byte<WF>(cq);
          }
        }
      if (save && tid == 0) a.w_scale[(int64_t)slot * Hv + h] = dW;
    } else {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int dt = 0; dt < DTW; ++dt) {
          const int dcol = 16 * (wave * DTW + dt) + r16;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * mt + 4 * grp + i;
            bf16 hi, lo;
            split2(Wacc[mt][dt][i], hi, lo);
            sm.b.W[0][row * LDK + dcol] = hi;
            sm.b.W[C::NW - 1][row * LDK + dcol] = lo;
          }
        }
    }

    // ---------------------------------------------- P6: state QDQ
    float dS = 1.f;
    if constexpr (SF != 0) {
      float m = 0.f;
#pragma unroll
      for (int mt = 0; mt < MK; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(S[mt][i]));
      m = wave_max(m);
      if (lane == 0) sm.amax16[wave] = m;
    }
    __syncthreads();                                  // W in LDS; state amax ready
    if constexpr (SF != 0) {
      const int gs = a.block_v / 16;                  // 16-col tiles per scale tile
      const int g0 = (wave / gs) * gs;
      float amax = 0.f;
      for (int t = g0; t < g0 + gs; ++t) amax = fmaxf(amax, sm.amax16[t]);
      dS = qdq_scale<SF>(amax);
      const float rS = 1.0f / dS;
#pragma unroll
      for (int mt = 0; mt < MK; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[mt][i] = round_code<SF>(S[mt][i] * rS);   // codes
      if (a.s_codes) {
        const int64_t sb = ((int64_t)slot * Hv + h) * DK * Dv;
#pragma unroll
        for (int mt = 0; mt < MK; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            a.s_codes[sb + (int64_t)(16 * mt + 4 * grp + i) * Dv + col] = code_byte<SF>(S[mt][i]);
        if (wave == g0 && lane == 0)
          a.s_scale[((int64_t)slot * Hv + h) * (Dv / a.block_v) + wcol / a.block_v] = dS;
      }
    } else if (a.s_f32) {
      const int64_t sb = ((int64_t)slot * Hv + h) * DK * Dv;
#pragma unroll
      for (int mt = 0; mt < MK; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a.s_f32[sb + (int64_t)(16 * mt + 4 * grp + i) * Dv + col] = S[mt][i];
    }

    // ------------------------------- P7: Vnew, O, state update
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
    f32x4 Vn[4], Oi[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 accw = zero4(), accq = zero4();
#pragma unroll
      for (int kk = 0; kk < MK / 2; ++kk) {
        const bf16x8 w0 = lds_pair(sm.b.W[0], 16 * mt + r16, LDK, 32 * kk, grp);
        const bf16x8 q0 = lds_pair(sm.Q[0], 16 * mt + r16, LDK, 32 * kk, grp);
        accw = mfma(w0, bSh[kk], accw);
        accq = mfma(q0, bSh[kk], accq);
        if constexpr (WF == 0) {
          const bf16x8 w1 = lds_pair(sm.b.W[C::NW - 1], 16 * mt + r16, LDK, 32 * kk, grp);
          accw = mfma(w1, bSh[kk], accw);
        }
        if constexpr (F32IN) {
          const bf16x8 q1 = lds_pair(sm.Q[NIN - 1], 16 * mt + r16, LDK, 32 * kk, grp);
          accq = mfma(q1, bSh[kk], accq);
        }
        if constexpr (SF == 0) {
          accw = mfma(w0, bSl[kk], accw);
          accq = mfma(q0, bSl[kk], accq);
        }
      }
      const float sc = dW * dS;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Vn[mt][i] = U[mt][i] - sc * accw[i];
        Oi[mt][i] = dS * accq[i];
      }
    }
    // Vnew and exp(gamma_n - gamma) Vnew as B operands (paired order over positions)
    bf16x8 bVh[2], bVl[2], bDh[2], bDl[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      pack_pair_split(Vn[2 * kk], Vn[2 * kk + 1], bVh[kk], bVl[kk]);
      f32x4 d0, d1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        d0[i] = sm.egc[32 * kk + 4 * grp + i] * Vn[2 * kk][i];
        d1[i] = sm.egc[32 * kk + 16 + 4 * grp + i] * Vn[2 * kk + 1][i];
      }
      pack_pair_split(d0, d1, bDh[kk], bDl[kk]);
    }
    // O = scale (exp(gamma) Q Sq + P Vnew)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (kk > mt / 2) continue;
        const bf16x8 ph = lds_pair(sm.P[0], 16 * mt + r16, L64, 32 * kk, grp);
        const bf16x8 pl = lds_pair(sm.P[1], 16 * mt + r16, L64, 32 * kk, grp);
        acc = mfma(ph, bVh[kk], acc);
        acc = mfma(pl, bVh[kk], acc);
        acc = mfma(ph, bVl[kk], acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * mt + 4 * grp + i;
        if (row < nc) {
          const float ov = a.scale * (sm.eg[row] * Oi[mt][i] + acc[i]);
          const int64_t off = ((int64_t)(t0 + row) * Hv + h) * Dv + col;
          if constexpr (F32IN) reinterpret_cast<float*>(a.o)[off] = ov;
          else reinterpret_cast<bf16*>(a.o)[off] = to_bf16(ov);
        }
      }
    }
    // S = exp(gamma_n) Sq + K^T (exp(gamma_n - gamma) Vnew)
    const float egC = sm.red[4];
#pragma unroll
    for (int mt = 0; mt < MK; ++mt) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 kt = lds_pair(sm.Kt[0], 16 * mt + r16, L64, 32 * kk, grp);
        acc = mfma(kt, bDh[kk], acc);
        acc = mfma(kt, bDl[kk], acc);
        if constexpr (F32IN) {
          const bf16x8 ktl = lds_pair(sm.Kt[1], 16 * mt + r16, L64, 32 * kk, grp);
          acc = mfma(ktl, bDh[kk], acc);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sq = (SF != 0) ? S[mt][i] * dS : S[mt][i];
        S[mt][i] = egC * sq + acc[i];
      }
    }
    __syncthreads();                                  // LDS reused by the next chunk
  }

  if (a.ht) {
#pragma unroll
    for (int mt = 0; mt < MK; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a.ht[state_base + (int64_t)(16 * mt + 4 * grp + i) * Dv + col] = S[mt][i];
  }
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

hipError_t launch_fwd(const FwdConfig& cfg, const FwdKernelArgs& a, hipStream_t stream) {
  if (cfg.N == 0 || cfg.Hv == 0) return hipSuccess;
  if (cfg.f32_io) {
    if (cfg.Dk == 64) return launch_fmt<64, true>(cfg, a, stream);
    return hipErrorInvalidValue;
  }
  if (cfg.Dk == 64) return launch_fmt<64, false>(cfg, a, stream);
  if (cfg.Dk == 128) return launch_fmt<128, false>(cfg, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdn
