// Backward, the chunk-local gradients for bf16 inputs: one workgroup per
// (chunk, value head), after the reverse recurrence has stored dS' (the
// gradient of the state at the chunk's end) and dVnew of every chunk
// ("[1/4] GDN state/W QAT foundation", "What does this PR do?": identity STE at
// both QDQ sites, the forward's quantized W reused; the products use the
// forward's Sq and Wq).
//
// Per chunk (forward in gdn_fwd_state.hip, reverse recurrence in
// gdn_bwd_state.hip), with T = X diag(beta), X = (I + L)^-1:
//   Vnew = T V - Wq Sq                          recomputed
//   dv   = T^T dVnew
//   dW   = -dVnew Sq^T,  dQi = dO Sq^T,  dKs = Vnew dS'^T
//   dP   = dO Vnew^T,    dTU = dVnew V^T
//   G    = scale dP * Gam (t >= s),  dq = scale e^gamma dQi + G K
//   dT   = dW (e^gamma K)^T + dTU,   dX = dT diag(beta)
//   dL   = -(X^T dX X^T) below the diagonal,  dA = dL beta_t Gam (t > s)
//   dk   = G^T Q + e^(gamma_n - gamma) dKs + beta e^gamma X^T dW + (dA + dA^T) K
// plus d beta and the gate gradient (reverse chunk-local cumsum of d gamma).
//
// All products run on bf16 MFMA 16x16x32 with FP32 accumulation: bf16 inputs
// enter exactly, FP32 factors as hi + lo pairs (three products when both
// factors are FP32, two when one is exact). An operand of a product needs its
// contraction index contiguous in each lane. Matrices live in LDS row-major as
// bf16 planes; an operand contracting over a row's columns is a plain LDS read
// (paired K order, lds_pair), and one contracting over a matrix's rows comes
// from accumulator-layout tiles of that matrix, which the matrix core makes
// exactly from the row-major planes (A times a 0/1 selection operand).
// Accumulator tiles are published to LDS transposed with 8-byte writes (a
// tile's lane holds four consecutive rows of one column), or as they are after
// a transpose through the matrix core.
//
// Work split, 8 waves: wave w owns row tile tw = w & 3 and column half
// hk = w >> 2 of every [64 x *] result (token rows; dk, dq, dW, dQi, dKs over
// k-tiles of that half, the 64 x 64 results over token tiles of that half).
#include "gdn_device.h"
#include "gdn_images.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

constexpr int NT = 512;
constexpr float LOG2E = 1.4426950408889634f;
constexpr int L64 = 72;                            // row stride of 64-wide LDS matrices

// Selection operand in paired K order (pperm): lane (grp, r16) holds
// B[k(e)][r16] = 1 exactly when k(e) = 16 h + r16, where position e stands for
// row 4 grp + e (e < 4) or 16 + 4 grp + e - 4 (e >= 4).
__device__ __forceinline__ bf16x8 sel_pair(int h, int r16, int grp) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int k = e < 4 ? 4 * grp + e : 16 + 4 * grp + (e - 4);
    r[e] = to_bf16(k == 16 * h + r16 ? 1.f : 0.f);
  }
  return r;
}

// Two named operands, not an array: a runtime index into an array of them
// would place it in private memory. q is the K = 16 selection (lane holds
// B[4 grp + e][r16] = 1 exactly when 4 grp + e = r16) of v_mfma_f32_16x16x16_bf16.
struct Sel {
  bf16x8 p0, p1;
  bf16x4 q;
  __device__ __forceinline__ bf16x8 get(int h) const {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = h ? p1[e] : p0[e];
    return r;
  }
};

// Accumulator tile (rows row0..row0+15, columns 16 ct..16 ct+15) of a
// row-major bf16 LDS matrix, exact (a transposing LDS read).
__device__ __forceinline__ f32x4 tile_of(const bf16* m, int ld, int row0, int ct, int r16, int grp,
                                         const Sel&) {
  return lds_tile(m, ld, row0, 16 * ct, r16, grp);
}
// Operand contracting over rows r0..r0+31 (paired order), free index = columns
// 16 ct..16 ct+15: the lane holds rows r0 + 4 grp + e and r0 + 16 + 4 grp + e
// of column 16 ct + r16 (no arithmetic).
__device__ __forceinline__ bf16x8 colp(const bf16* m, int ld, int r0, int ct, int r16, int grp,
                                       const Sel&) {
  return lds_col8(m, ld, r0, 16 * ct, r16, grp);
}
// Operand contracting over columns k0..k0+31 (paired order), free index = rows
// row0..row0+15.
__device__ __forceinline__ bf16x8 rowp(const bf16* m, int ld, int row0, int k0, int r16, int grp) {
  return lds_pair(m, row0 + r16, ld, k0, grp);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
// v_mfma_f32_16x16x16_bf16: lane holds A[r16][4 grp + e] and B[4 grp + e][r16].
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b),
                                                   c, 0, 0, 0);
}
// Transpose of one accumulator tile given as bf16: the lane that held
// M[row0 + 4 grp + i][col0 + r16] gets M[row0 + r16][col0 + 4 grp + i] (exact).
__device__ __forceinline__ f32x4 trans1(const bf16x4& c, const Sel& s) {
  return mfma16(c, s.q, zero4());
}

__device__ __forceinline__ bf16x4 to_bf16x4(const f32x4& v) {
  return bf16x4{to_bf16(v[0]), to_bf16(v[1]), to_bf16(v[2]), to_bf16(v[3])};
}
// x = hi + lo + O(2^-17 |x|): hi = bf16(x) (nearest even), lo = bf16(x - hi).
__device__ __forceinline__ void split4(const f32x4& x, bf16x4& hi, bf16x4& lo) {
  hi = to_bf16x4(x);
  f32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = x[i] - from_bf16(hi[i]);
  lo = to_bf16x4(r);
}

// Writes four consecutive elements of one row of a row-major bf16 matrix.
__device__ __forceinline__ void put4(bf16* m, int off, const bf16x4& v) {
  *reinterpret_cast<bf16x4*>(m + off) = v;
}
__device__ __forceinline__ void put4(bf16* m, int off, const f32x4& v) { put4(m, off, to_bf16x4(v)); }
// Splits four FP32 values into the hi and lo planes.
__device__ __forceinline__ void put4s(bf16* p0, bf16* p1, int off, const f32x4& v) {
  bf16x4 h, l;
  split4(v, h, l);
  put4(p0, off, h);
  put4(p1, off, l);
}
// Publishes an FP32 accumulator tile (rows 16 rt.., columns 16 ct..) of M as
// rows of M^T (hi and lo planes): M^T[16 ct + r16][16 rt + 4 grp + i].
__device__ __forceinline__ void put_T(bf16* p0, bf16* p1, int ld, const f32x4& c, int rt, int ct,
                                      int r16, int grp) {
  put4s(p0, p1, (16 * ct + r16) * ld + 16 * rt + 4 * grp, c);
}
// Publishes the same tile as rows of M (through a transpose).
__device__ __forceinline__ void put_N(bf16* p0, bf16* p1, int ld, const f32x4& c, int rt, int ct,
                                      int r16, int grp, const Sel& s) {
  bf16x4 h, l;
  split4(c, h, l);
  const int off = (16 * rt + r16) * ld + 16 * ct + 4 * grp;
  put4(p0, off, trans1(h, s));
  put4(p1, off, trans1(l, s));
}

__device__ __forceinline__ f32x4 mm2(f32x4 acc, bf16x8 a0, bf16x8 a1, bf16x8 b) {
  return mfma(a1, b, mfma(a0, b, acc));
}
// (a0 + a1)(b0 + b1) without the lo * lo term
__device__ __forceinline__ f32x4 mm3(f32x4 acc, bf16x8 a0, bf16x8 a1, bf16x8 b0, bf16x8 b1) {
  return mfma(a0, b1, mfma(a1, b0, mfma(a0, b0, acc)));
}

template <int DK, int VB, int NWP>
struct VLoopSmem {
  static constexpr int LDK = DK + 8, LVB = VB + 8;
  bf16 Wm[NWP][64 * LDK];
  bf16 Tm[2][64 * L64];
  bf16 Vm[64 * LVB];
  bf16 dOm[64 * LVB];
  bf16 Sqm[2][DK * LVB];
  bf16 Vnm[2][64 * LVB];
  bf16 dSm[2][DK * LVB];
};

template <int DK>
struct FinSmem {
  static constexpr int LDK = DK + 8;
  static constexpr int QM1 = (64 * LDK > 2 * 64 * L64) ? 64 * LDK : 2 * 64 * L64;
  bf16 Km[64 * LDK];
  bf16 QM1m[QM1];                                  // Q rows, later M1 planes
  bf16 Xm[2][64 * L64];
  bf16 dWm[2][64 * LDK];
  bf16 GA[2][64 * L64];                            // G rows, later dA rows
  bf16 GTA[2][64 * L64];                           // G^T rows, later dA^T rows
  bf16 dXTm[2][64 * L64];
};

struct LocalGates {
  alignas(16) float gam2[64];
  alignas(16) float eg[64];
  alignas(16) float egc[64];
  alignas(16) float bet[64];
  float egC;
};

template <int DK, int VB, int NWP>
struct LocalSmem {
  union {
    VLoopSmem<DK, VB, NWP> v;
    FinSmem<DK> f;
  } u;
  LocalGates gs;
  float colH[4][64];      // column sums of H = G * (Q K^T), by row tile
  float colHL[4][64];     // column sums of dA-side gate terms, by row tile
  float colDB[4][64];     // column sums of dT * X (d beta from T = X diag(beta))
  float rowDG[2][64];     // d gamma row parts, by column half
  float rowTerm[2][64];   // egc_s k_s . dKs_s (state-update gate term), by half
  float rowDB[2][64];     // d beta from L, by half
  float red[8];           // <dS', Sq> per wave
};

// Global loads of one value pass, issued one pass ahead into registers: V and
// dO rows (bf16), Sq (codes with their scale, or FP32) and this wave's dS'
// tiles (the first ones used).
template <int DK, int VB, int SF>
struct PassLoads {
  static constexpr int NVP = (64 * VB / 8 + NT - 1) / NT;
  static constexpr int SPC = SF != 0 ? DK * VB / 16 : DK * VB / 4;
  static constexpr int NSP = (SPC + NT - 1) / NT;
  static constexpr int NU = (DK / 16) * (VB / 16) / 8;
  u32x4 v[NVP], o[NVP], s[NSP];
  float sc[NSP];
  f32x4 ds[NU];
};

// NEU: the chunk's X is the approximate inverse (a polynomial in L). Its dL
// terms (dA, the d beta and d gamma parts from L) are left out here and dX
// is exported instead; bwd_neumann adds them (gdn_bwd.hip).
template <int DK, int SF, int WF, bool NEU>
__global__ void __launch_bounds__(NT, 1) bwd_local_kernel(BwdKernelArgs a, int N) {
  constexpr int VB = WF == 0 ? 32 : 64;            // value columns per pass
  constexpr int NWP = WF == 0 ? 2 : 1;             // W planes
  constexpr int MK = DK / 16, KH = MK / 2;         // k tiles, k tiles per half
  constexpr int NVT = VB / 16, NKV = VB / 32;      // value tiles, value K steps per pass
  constexpr int NJ = 4 * NVT / 8;                  // (value tile, token tile) units per wave
  constexpr int NU = MK * NVT / 8;                 // dS' publishing units per wave
  using VS = VLoopSmem<DK, VB, NWP>;
  using FS = FinSmem<DK>;
  using PL = PassLoads<DK, VB, SF>;
  constexpr int LDK = VS::LDK, LVB = VS::LVB;
  static_assert(sizeof(LocalSmem<DK, VB, NWP>) <= 160 * 1024, "LDS");
  __shared__ __align__(16) LocalSmem<DK, VB, NWP> sm;

  const FwdKernelArgs& f = a.f;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int lane = fresh_lane(), tid = wave * 64 + lane, r16 = lane & 15, grp = lane >> 4;
  // per-lane addresses are rebuilt in each phase instead of being kept live
  // across the passes (fresh_lane in gdn_device.h)
#define GDN_REFRESH() \
  lane = fresh_lane(); tid = wave * 64 + lane; r16 = lane & 15; grp = lane >> 4
  const int tw = wave & 3, hk = wave >> 2;
  const int slot = blockIdx.x, h = blockIdx.y;
  const Chunk ch = locate_slot(slot, f.cu_seqlens, N, f.T, f.prefix_len);
  if (!ch.valid) return;
  const int Hv = f.Hv, Hqk = f.Hqk, Dv = f.Dv, nvb = Dv / 64, hq = h / (Hv / Hqk);
  const int t0 = ch.t0, nc = ch.nc;
  const float scale = f.scale;
  const int64_t chb = (int64_t)slot * Hv + h;
  LocalGates& gs = sm.gs;
  Sel sel;
  sel.p0 = sel_pair(0, r16, grp);
  sel.p1 = sel_pair(1, r16, grp);
#pragma unroll
  for (int e = 0; e < 4; ++e) sel.q[e] = to_bf16(4 * grp + e == r16 ? 1.f : 0.f);
  // (vt, tt) units of this wave for Vnew and dv
  int jv[NJ], jt[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int idx = wave + 8 * j;
    jv[j] = idx % NVT;
    jt[j] = idx / NVT;
  }

  const bf16* vg = reinterpret_cast<const bf16*>(f.v);
  const bf16* dog = reinterpret_cast<const bf16*>(a.dout);
  auto dvn_tile = [&](int vb0, int tt, int vt) {
    const int col = vb0 + 16 * vt;
    return *reinterpret_cast<const f32x4*>(a.ws_dvn + frag_off(chb, nvb, col >> 6, (col & 63) >> 4, 4, tt, lane));
  };
  auto ds_tile = [&](int vb0, int kt, int vt) {
    const int col = vb0 + 16 * vt;
    return *reinterpret_cast<const f32x4*>(a.ws_dstate + frag_off(chb, nvb, col >> 6, (col & 63) >> 4, MK, kt, lane));
  };
  auto load_pass = [&](int vb0, PL& L) {
#pragma unroll
    for (int p = 0; p < PL::NVP; ++p) {
      const int e = min(tid + NT * p, 64 * VB / 8 - 1), row = e / (VB / 8), c8 = e % (VB / 8);
      const int64_t off = ((int64_t)(t0 + min(row, nc - 1)) * Hv + h) * Dv + vb0 + 8 * c8;
      L.v[p] = *reinterpret_cast<const u32x4*>(vg + off);
      L.o[p] = *reinterpret_cast<const u32x4*>(dog + off);
    }
#pragma unroll
    for (int p = 0; p < PL::NSP; ++p) {
      const int e = min(tid + NT * p, PL::SPC - 1);
      if constexpr (SF != 0) {
        const int row = e / (VB / 16), col = vb0 + 16 * (e % (VB / 16));
        L.s[p] = *reinterpret_cast<const u32x4*>(f.s_codes + chb * DK * Dv + (int64_t)row * Dv + col);
        L.sc[p] = f.s_scale[chb * (Dv / f.block_v) + col / f.block_v];
      } else {
        const int row = e / (VB / 4), col = vb0 + 4 * (e % (VB / 4));
        L.s[p] = *reinterpret_cast<const u32x4*>(f.s_f32 + chb * DK * Dv + (int64_t)row * Dv + col);
        L.sc[p] = 1.f;
      }
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int idx = wave + 8 * u;
      L.ds[u] = ds_tile(vb0, idx % MK, idx / MK);
    }
  };
  auto& V = sm.u.v;
  auto store_pass = [&](const PL& L) {
#pragma unroll
    for (int p = 0; p < PL::NVP; ++p) {
      const int e = tid + NT * p;
      if (e < 64 * VB / 8) {
        const int row = e / (VB / 8), c8 = e % (VB / 8);
        const bool z = row >= nc;
        *reinterpret_cast<u32x4*>(&V.Vm[row * LVB + 8 * c8]) = z ? u32x4{0u, 0u, 0u, 0u} : L.v[p];
        *reinterpret_cast<u32x4*>(&V.dOm[row * LVB + 8 * c8]) = z ? u32x4{0u, 0u, 0u, 0u} : L.o[p];
      }
    }
#pragma unroll
    for (int p = 0; p < PL::NSP; ++p) {
      const int e = tid + NT * p;
      if (e >= PL::SPC) continue;
      if constexpr (SF != 0) {
        const int row = e / (VB / 16), c16 = e % (VB / 16);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 x;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t word = L.s[p][q4] >> (8 * i);
            const float cv = SF == 1 ? __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word), 0)
                                     : static_cast<float>(static_cast<int8_t>(word & 0xFFu));
            x[i] = cv * L.sc[p];
          }
          put4s(V.Sqm[0], V.Sqm[1], row * LVB + 16 * c16 + 4 * q4, x);
        }
      } else {
        const int row = e / (VB / 4), c4 = e % (VB / 4);
        f32x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(L.s[p][i]);
        put4s(V.Sqm[0], V.Sqm[1], row * LVB + 4 * c4, x);
      }
    }
  };

  // ---------------------------------------------------------------- set-up
  // global loads: W, X and the first pass, all in flight together
  constexpr int WPC = WF != 0 ? 64 * DK / 16 : 64 * DK / 4, NWL = (WPC + NT - 1) / NT;
  u32x4 wl[NWL];
#pragma unroll
  for (int p = 0; p < NWL; ++p) {
    const int e = min(tid + NT * p, WPC - 1);
    if constexpr (WF != 0) {
      const int row = e / (DK / 16), c16 = e % (DK / 16);
      wl[p] = *reinterpret_cast<const u32x4*>(f.w_codes + ((int64_t)(t0 + min(row, nc - 1)) * Hv + h) * DK + 16 * c16);
    } else {
      const int row = e / (DK / 4), c4 = e % (DK / 4);
      wl[p] = *reinterpret_cast<const u32x4*>(a.ws_W + ((int64_t)(t0 + min(row, nc - 1)) * Hv + h) * DK + 4 * c4);
    }
  }
  constexpr int NXL = 64 * 16 / NT;
  f32x4 xl[NXL];
  {
    const float* Xg = a.ws_X + chb * 4096;
#pragma unroll
    for (int p = 0; p < NXL; ++p) {
      const int e = tid + NT * p;
      xl[p] = *reinterpret_cast<const f32x4*>(Xg + (e >> 4) * 64 + 4 * (e & 15));
    }
  }
  PL L;
  load_pass(0, L);
  const float dWs = WF != 0 ? f.w_scale[chb] : 1.f;   // W scale (W QDQ on)
  if (wave == 0) {
    const bool valid = lane < nc;
    const int64_t gi = (int64_t)(t0 + min(lane, nc - 1)) * Hv + h;
    const float g2 = wave_incl_scan(valid ? f.g[gi] * LOG2E : 0.f);
    const float g2n = read_lane(g2, nc - 1);
    gs.gam2[lane] = g2;
    gs.eg[lane] = fexp2(g2);
    gs.egc[lane] = valid ? fexp2(g2n - g2) : 0.f;
    gs.bet[lane] = valid ? f.beta[gi] : 0.f;
    if (lane == 0) gs.egC = fexp2(g2n);
  }
#pragma unroll
  for (int p = 0; p < NWL; ++p) {
    const int e = tid + NT * p;
    if (e >= WPC) continue;
    if constexpr (WF != 0) {
      const int row = e / (DK / 16), c16 = e % (DK / 16);
      bf16x8 o[2];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t word = wl[p][j >> 2] >> (8 * (j & 3));
        const float cv = WF == 1 ? __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word), 0)
                                 : static_cast<float>(static_cast<int8_t>(word & 0xFFu));
        o[j >> 3][j & 7] = to_bf16(row < nc ? cv : 0.f);
      }
      *reinterpret_cast<bf16x8*>(&V.Wm[0][row * LDK + 16 * c16]) = o[0];
      *reinterpret_cast<bf16x8*>(&V.Wm[0][row * LDK + 16 * c16 + 8]) = o[1];
    } else {
      const int row = e / (DK / 4), c4 = e % (DK / 4);
      f32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = row < nc ? __uint_as_float(wl[p][i]) : 0.f;
      put4s(V.Wm[0], V.Wm[NWP - 1], row * LDK + 4 * c4, w);
    }
  }
  store_pass(L);
  __syncthreads();                                 // gates visible
#pragma unroll
  for (int p = 0; p < NXL; ++p) {
    // T = X diag(beta), hi + lo
    const int e = tid + NT * p, row = e >> 4, c4 = e & 15;
    const f32x4 b = *reinterpret_cast<const f32x4*>(&gs.bet[4 * c4]);
    f32x4 x = xl[p];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] *= b[i];
    put4s(V.Tm[0], V.Tm[1], row * L64 + 4 * c4, x);
  }
  __syncthreads();

  // accumulators (row tile tw; k tiles hk*KH.. or token tiles 2hk, 2hk+1)
  f32x4 dW[KH], dQi[KH], dKs[KH], dP[2], dTU[2];
#pragma unroll
  for (int j = 0; j < KH; ++j) dW[j] = dQi[j] = dKs[j] = zero4();
  dP[0] = dP[1] = dTU[0] = dTU[1] = zero4();
  float sSq = 0.f;
  // finish inputs, loaded during the last pass
  constexpr int NKL = (64 * DK / 8 + NT - 1) / NT;
  u32x4 kl[NKL], ql[NKL];

  // ---------------------------------------------------------------- value passes
  for (int vb0 = 0; vb0 < Dv; vb0 += VB) {
    GDN_REFRESH();
    // this pass's dVnew tiles (tw, every value tile)
    f32x4 dvp[NVT], dvv[4];
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) dvp[vt] = dvn_tile(vb0, tw, vt);
    // (a) dS' as rows (k-major) hi + lo, and <dS', Sq>
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int idx = wave + 8 * u, kt = idx % MK, vt = idx / MK;
      bf16x4 ch_, cl_;
      split4(L.ds[u], ch_, cl_);
      const f32x4 th = trans1(ch_, sel), tl = trans1(cl_, sel);
      const int off = (16 * kt + r16) * LVB + 16 * vt + 4 * grp;
      put4(V.dSm[0], off, th);
      put4(V.dSm[1], off, tl);
      const bf16x4 s0 = *reinterpret_cast<const bf16x4*>(&V.Sqm[0][off]);
      const bf16x4 s1 = *reinterpret_cast<const bf16x4*>(&V.Sqm[1][off]);
#pragma unroll
      for (int i = 0; i < 4; ++i) sSq += (th[i] + tl[i]) * (from_bf16(s0[i]) + from_bf16(s1[i]));
    }
    // (every token tile, jv) dVnew tiles for dv, in flight during (4)(5)(6)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) dvv[tt] = dvn_tile(vb0, tt, jv[0]);
    // (4)(5)(6): rows tw; dVnew rows through the matrix core
    bf16x8 AdV[NKV][2], AdO[NKV];
    {
#pragma unroll
      for (int kk = 0; kk < NKV; ++kk) {
        f32x4 th[2], tl[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          bf16x4 ch_, cl_;
          split4(dvp[2 * kk + e], ch_, cl_);
          th[e] = trans1(ch_, sel);
          tl[e] = trans1(cl_, sel);
        }
        AdV[kk][0] = pack_pair(th[0], th[1]);
        AdV[kk][1] = pack_pair(tl[0], tl[1]);
        AdO[kk] = rowp(V.dOm, LVB, 16 * tw, 32 * kk, r16, grp);
      }
    }
#pragma unroll
    for (int j = 0; j < KH; ++j) {
      const int kt = hk * KH + j;
#pragma unroll
      for (int kk = 0; kk < NKV; ++kk) {
        const bf16x8 b0 = rowp(V.Sqm[0], LVB, 16 * kt, 32 * kk, r16, grp);
        const bf16x8 b1 = rowp(V.Sqm[1], LVB, 16 * kt, 32 * kk, r16, grp);
        dW[j] = mm3(dW[j], AdV[kk][0], AdV[kk][1], b0, b1);
        dQi[j] = mfma(AdO[kk], b1, mfma(AdO[kk], b0, dQi[j]));
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int st = 2 * hk + i;
#pragma unroll
      for (int kk = 0; kk < NKV; ++kk)
        dTU[i] = mm2(dTU[i], AdV[kk][0], AdV[kk][1], rowp(V.Vm, LVB, 16 * st, 32 * kk, r16, grp));
    }
    // (1) Vnew^T tiles -> Vnew rows (hi + lo); (7) dv^T tiles -> dv
    {
      const int vt = jv[0];                       // the same value tile for every unit
      f32x4 acc[NJ], accw[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[j] = accw[j] = zero4();
      // T V: A = V^T over tokens, B = T^T (rows of T)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 av = colp(V.Vm, LVB, 32 * kk, vt, r16, grp, sel);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[j] = mfma(av, rowp(V.Tm[1], L64, 16 * jt[j], 32 * kk, r16, grp),
                        mfma(av, rowp(V.Tm[0], L64, 16 * jt[j], 32 * kk, r16, grp), acc[j]));
      }
      // W Sq: A = Sq^T over k, B = W^T (rows of W)
#pragma unroll
      for (int kk = 0; kk < DK / 32; ++kk) {
        const bf16x8 as0 = colp(V.Sqm[0], LVB, 32 * kk, vt, r16, grp, sel);
        const bf16x8 as1 = colp(V.Sqm[1], LVB, 32 * kk, vt, r16, grp, sel);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const bf16x8 w0 = rowp(V.Wm[0], LDK, 16 * jt[j], 32 * kk, r16, grp);
          accw[j] = mfma(as1, w0, mfma(as0, w0, accw[j]));
          if constexpr (NWP == 2)
            accw[j] = mfma(as0, rowp(V.Wm[1], LDK, 16 * jt[j], 32 * kk, r16, grp), accw[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        f32x4 vn;
#pragma unroll
        for (int i = 0; i < 4; ++i) vn[i] = acc[j][i] - dWs * accw[j][i];
        put4s(V.Vnm[0], V.Vnm[1], (16 * jt[j] + r16) * LVB + 16 * vt + 4 * grp, vn);
      }
      // dv^T = dVnew^T T: A over tokens from the dVnew tiles, B = T over its rows
      f32x4 dv[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) dv[j] = zero4();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 dh, dl;
        pack_pair_split(dvv[2 * kk], dvv[2 * kk + 1], dh, dl);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          dv[j] = mm3(dv[j], dh, dl, colp(V.Tm[0], L64, 32 * kk, jt[j], r16, grp, sel),
                      colp(V.Tm[1], L64, 32 * kk, jt[j], r16, grp, sel));
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int t = 16 * jt[j] + r16;
        if (t < nc) {
          const int64_t o = ((int64_t)(t0 + t) * Hv + h) * Dv + vb0 + 16 * vt + 4 * grp;
          if (a.grad_f32) *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.dv) + o) = dv[j];
          else *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(a.dv) + o) =
                   bf16x4{to_bf16(dv[j][0]), to_bf16(dv[j][1]), to_bf16(dv[j][2]), to_bf16(dv[j][3])};
        }
      }
    }
    __syncthreads();                               // Vnew and dS' rows complete
    GDN_REFRESH();
    // the next pass's loads (or the finish's), in flight during (2)(3)
    asm volatile("" ::: "memory");
    const bool last = vb0 + VB >= Dv;
    if (!last) {
      load_pass(vb0 + VB, L);
    } else {
      const bf16* kg = reinterpret_cast<const bf16*>(f.k);
      const bf16* qg = reinterpret_cast<const bf16*>(f.q);
#pragma unroll
      for (int p = 0; p < NKL; ++p) {
        const int e = min(tid + NT * p, 64 * DK / 8 - 1), row = e / (DK / 8), c8 = e % (DK / 8);
        const int64_t off = ((int64_t)(t0 + min(row, nc - 1)) * Hqk + hq) * DK + 8 * c8;
        kl[p] = *reinterpret_cast<const u32x4*>(kg + off);
        ql[p] = *reinterpret_cast<const u32x4*>(qg + off);
      }
      const float* Xg = a.ws_X + chb * 4096;
#pragma unroll
      for (int p = 0; p < NXL; ++p) {
        const int e = tid + NT * p;
        xl[p] = *reinterpret_cast<const f32x4*>(Xg + (e >> 4) * 64 + 4 * (e & 15));
      }
    }
    // (2) dKs = Vnew dS'^T; (3) dP = dO Vnew^T
    {
      bf16x8 AVn[NKV][2];
#pragma unroll
      for (int kk = 0; kk < NKV; ++kk)
#pragma unroll
        for (int pl = 0; pl < 2; ++pl) AVn[kk][pl] = rowp(V.Vnm[pl], LVB, 16 * tw, 32 * kk, r16, grp);
#pragma unroll
      for (int j = 0; j < KH; ++j) {
        const int kt = hk * KH + j;
#pragma unroll
        for (int kk = 0; kk < NKV; ++kk)
          dKs[j] = mm3(dKs[j], AVn[kk][0], AVn[kk][1], rowp(V.dSm[0], LVB, 16 * kt, 32 * kk, r16, grp),
                       rowp(V.dSm[1], LVB, 16 * kt, 32 * kk, r16, grp));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int st = 2 * hk + i;
#pragma unroll
        for (int kk = 0; kk < NKV; ++kk)
          dP[i] = mfma(AdO[kk], rowp(V.Vnm[1], LVB, 16 * st, 32 * kk, r16, grp),
                       mfma(AdO[kk], rowp(V.Vnm[0], LVB, 16 * st, 32 * kk, r16, grp), dP[i]));
      }
    }
    __syncthreads();                               // pass buffers free
    GDN_REFRESH();
    if (!last) {
      store_pass(L);
      __syncthreads();
    }
  }

  // ---------------------------------------------------------------- finish
  auto& F = sm.u.f;
  constexpr int FLDK = FS::LDK;
  // dq, dk rows: straight to the outputs with one value head per query/key
  // head, else per value head (FP32) for the group sum
  const bool direct = Hv == Hqk && !NEU;           // NEU: bwd_neumann adds to dk first
  const bool half = direct && !a.grad_f32;         // bf16 outputs
  const int esz = half ? 2 : 4;
  const int64_t rstride = direct ? (int64_t)Hv * DK * esz : (int64_t)Hv * 2 * DK * 4;
  char* const dq_base = direct ? reinterpret_cast<char*>(a.dq) + ((int64_t)t0 * Hv + h) * DK * esz
                               : reinterpret_cast<char*>(a.ws_dqk + ((int64_t)t0 * Hv + h) * 2 * DK);
  char* const dk_base = direct ? reinterpret_cast<char*>(a.dk) + ((int64_t)t0 * Hv + h) * DK * esz
                               : reinterpret_cast<char*>(a.ws_dqk + ((int64_t)t0 * Hv + h) * 2 * DK + DK);
  auto put_grad = [&](char* base, int t, int col, float v) {
    char* p = base + t * rstride + col * esz;
    if (half) *reinterpret_cast<bf16*>(p) = to_bf16(v);
    else *reinterpret_cast<float*>(p) = v;
  };
  // One bf16 gradient tile (rows 16 tw.., columns 16 kt..; accumulator
  // layout) stored through a matrix-core transpose: the rounded values are
  // exact in bf16, and each lane then holds four adjacent columns of one row,
  // one 8-byte store instead of four 2-byte ones. (bf16 outputs only.)
  auto put_tile_half = [&](char* base, int kt, const f32x4& v) {
    const f32x4 tt = trans1(to_bf16x4(v), sel);
    const int t = 16 * tw + r16;
    if (t < nc)
      *reinterpret_cast<bf16x4*>(base + t * rstride + (16 * kt + 4 * grp) * 2) = to_bf16x4(tt);
  };
  GDN_REFRESH();
  {
#pragma unroll
    for (int p = 0; p < NKL; ++p) {
      const int e = tid + NT * p;
      if (e >= 64 * DK / 8) continue;
      const int row = e / (DK / 8), c8 = e % (DK / 8);
      const bool z = row >= nc;
      *reinterpret_cast<u32x4*>(&F.Km[row * FLDK + 8 * c8]) = z ? u32x4{0u, 0u, 0u, 0u} : kl[p];
      *reinterpret_cast<u32x4*>(&F.QM1m[row * FLDK + 8 * c8]) = z ? u32x4{0u, 0u, 0u, 0u} : ql[p];
    }
#pragma unroll
    for (int p = 0; p < NXL; ++p) {
      const int e = tid + NT * p, row = e >> 4, c4 = e & 15;
      put4s(F.Xm[0], F.Xm[1], row * L64 + 4 * c4, xl[p]);
    }
    // dW = -(accumulated dVnew Sq^T), as rows
#pragma unroll
    for (int j = 0; j < KH; ++j) {
      f32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = -dW[j][i];
      put_N(F.dWm[0], F.dWm[1], FLDK, w, tw, hk * KH + j, r16, grp, sel);
    }
  }
  __syncthreads();
  GDN_REFRESH();

  float dg_acc[4] = {0.f, 0.f, 0.f, 0.f};
  float term_acc[4] = {0.f, 0.f, 0.f, 0.f};
  float db_acc[4] = {0.f, 0.f, 0.f, 0.f};
  f32x4 KKt[2];
  // FA1: Q K^T, K K^T, dW K^T on tiles (tw, 2hk + i) -> G, H, dT, dX
  // (the gate values are read up front, as 16-byte reads where they are
  // contiguous, so no LDS read waits behind the products)
  const f32x4 gt4 = *reinterpret_cast<const f32x4*>(&gs.gam2[16 * tw + 4 * grp]);
  {
    float colh[2][4], coldb[2][4];
    float gs_s2[2], eg_s2[2], bet_s2[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int s = 16 * (2 * hk + i) + r16;
      gs_s2[i] = gs.gam2[s];
      eg_s2[i] = gs.eg[s];
      bet_s2[i] = gs.bet[s];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int st = 2 * hk + i;
      f32x4 qk = zero4(), kk2 = zero4(), wk = zero4();
#pragma unroll
      for (int kk = 0; kk < DK / 32; ++kk) {
        const bf16x8 bk = lds_nat(F.Km, 16 * st + r16, FLDK, 32 * kk, grp);
        qk = mfma(lds_nat(F.QM1m, 16 * tw + r16, FLDK, 32 * kk, grp), bk, qk);
        kk2 = mfma(lds_nat(F.Km, 16 * tw + r16, FLDK, 32 * kk, grp), bk, kk2);
        wk = mfma(lds_nat(F.dWm[1], 16 * tw + r16, FLDK, 32 * kk, grp), bk,
                  mfma(lds_nat(F.dWm[0], 16 * tw + r16, FLDK, 32 * kk, grp), bk, wk));
      }
      KKt[i] = kk2;
      const f32x4 xh = tile_of(F.Xm[0], L64, 16 * tw, st, r16, grp, sel);
      const f32x4 xl = tile_of(F.Xm[1], L64, 16 * tw, st, r16, grp, sel);
      const int s = 16 * st + r16;
      const float gs_s = gs_s2[i], eg_s = eg_s2[i], bet_s = bet_s2[i];
      f32x4 G, dX;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = 16 * tw + 4 * grp + q;
        const float gv = t >= s ? scale * dP[i][q] * fexp2(gt4[q] - gs_s) : 0.f;
        G[q] = gv;
        const float hv = gv * qk[q];
        dg_acc[q] += hv;
        colh[i][q] = hv;
        const float dt = wk[q] * eg_s + dTU[i][q];
        coldb[i][q] = dt * (xh[q] + xl[q]);
        dX[q] = dt * bet_s;
      }
      put_T(F.GTA[0], F.GTA[1], L64, G, tw, st, r16, grp);
      put_N(F.GA[0], F.GA[1], L64, G, tw, st, r16, grp, sel);
      put_T(F.dXTm[0], F.dXTm[1], L64, dX, tw, st, r16, grp);
      if constexpr (NEU) {
        float* dxg = a.ws_dX + chb * 4096 + 16 * st + r16;
#pragma unroll
        for (int q = 0; q < 4; ++q) dxg[(16 * tw + 4 * grp + q) * 64] = dX[q];
      }
    }
    // column partial sums of this wave's 16 rows
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float th = colh[i][0] + colh[i][1] + colh[i][2] + colh[i][3];
      float td = coldb[i][0] + coldb[i][1] + coldb[i][2] + coldb[i][3];
      th += __shfl_xor(th, 16, WAVE);
      th += __shfl_xor(th, 32, WAVE);
      td += __shfl_xor(td, 16, WAVE);
      td += __shfl_xor(td, 32, WAVE);
      if (grp == 0) {
        sm.colH[tw][16 * (2 * hk + i) + r16] = th;
        sm.colDB[tw][16 * (2 * hk + i) + r16] = td;
      }
    }
  }
  __syncthreads();
  GDN_REFRESH();

  // FB1: dq = scale e^gamma dQi + G K; dK = G^T Q + egc dKs + beta e^gamma X^T dW
  f32x4 dK[KH];
  {
    bf16x8 AX[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int pl = 0; pl < 2; ++pl) AX[kk][pl] = colp(F.Xm[pl], L64, 32 * kk, tw, r16, grp, sel);
    const f32x4 eg4 = *reinterpret_cast<const f32x4*>(&gs.eg[16 * tw + 4 * grp]);
    const f32x4 egc4 = *reinterpret_cast<const f32x4*>(&gs.egc[16 * tw + 4 * grp]);
    const f32x4 bet4 = *reinterpret_cast<const f32x4*>(&gs.bet[16 * tw + 4 * grp]);
#pragma unroll
    for (int j = 0; j < KH; ++j) {
      const int kt = hk * KH + j, col = 16 * kt + r16;
      f32x4 gk = zero4(), gq = zero4(), xw = zero4();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        gk = mm2(gk, rowp(F.GA[0], L64, 16 * tw, 32 * kk, r16, grp),
                 rowp(F.GA[1], L64, 16 * tw, 32 * kk, r16, grp), colp(F.Km, FLDK, 32 * kk, kt, r16, grp, sel));
        const bf16x8 cq = colp(F.QM1m, FLDK, 32 * kk, kt, r16, grp, sel);
        gq = mm2(gq, rowp(F.GTA[0], L64, 16 * tw, 32 * kk, r16, grp),
                 rowp(F.GTA[1], L64, 16 * tw, 32 * kk, r16, grp), cq);
        const bf16x8 w0 = colp(F.dWm[0], FLDK, 32 * kk, kt, r16, grp, sel);
        const bf16x8 w1 = colp(F.dWm[1], FLDK, 32 * kk, kt, r16, grp, sel);
        xw = mm3(xw, AX[kk][0], AX[kk][1], w0, w1);
      }
      const f32x4 qv = tile_of(F.QM1m, FLDK, 16 * tw, kt, r16, grp, sel);
      const f32x4 kv = tile_of(F.Km, FLDK, 16 * tw, kt, r16, grp, sel);
      f32x4 dqv;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = 16 * tw + 4 * grp + q;
        const float qi = scale * eg4[q] * dQi[j][q];
        dg_acc[q] += qi * qv[q];
        dqv[q] = qi + gk[q];
        if (!half && t < nc) put_grad(dq_base, t, col, dqv[q]);
        const float ks = egc4[q] * dKs[j][q];
        term_acc[q] += ks * kv[q];
        const float wv = xw[q] * bet4[q] * eg4[q];
        dg_acc[q] += wv * kv[q];
        dK[j][q] = gq[q] + ks + wv;
      }
      if (half) put_tile_half(dq_base, kt, dqv);
    }
  }
  // M1^T = dX^T X on tiles (tw, 2hk + i)
  f32x4 M1T[2];
  {
    bf16x8 AD[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int pl = 0; pl < 2; ++pl) AD[kk][pl] = rowp(F.dXTm[pl], L64, 16 * tw, 32 * kk, r16, grp);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ut = 2 * hk + i;
      f32x4 m = zero4();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        m = mm3(m, AD[kk][0], AD[kk][1], colp(F.Xm[0], L64, 32 * kk, ut, r16, grp, sel),
                colp(F.Xm[1], L64, 32 * kk, ut, r16, grp, sel));
      M1T[i] = m;
    }
  }
  __syncthreads();                                 // Q rows, G, G^T, dX^T no longer read
  GDN_REFRESH();
  // M1 rows (M1[u][s] = M1^T[s][u]) into the Q space
  bf16* M1p0 = F.QM1m;
  bf16* M1p1 = F.QM1m + 64 * L64;
#pragma unroll
  for (int i = 0; i < 2; ++i) put_T(M1p0, M1p1, L64, M1T[i], tw, 2 * hk + i, r16, grp);
  __syncthreads();
  GDN_REFRESH();
  // FA3: dL = -(M1 X^T) below the diagonal; dA = dL beta_t Gam
  {
    bf16x8 AM[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int pl = 0; pl < 2; ++pl) AM[kk][pl] = rowp(pl ? M1p1 : M1p0, L64, 16 * tw, 32 * kk, r16, grp);
    float colhl[2][4];
    const f32x4 bt4 = *reinterpret_cast<const f32x4*>(&gs.bet[16 * tw + 4 * grp]);
    float gu2[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) gu2[i] = gs.gam2[16 * (2 * hk + i) + r16];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ut = 2 * hk + i;
      f32x4 ml = zero4();
      if constexpr (!NEU) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          ml = mm3(ml, AM[kk][0], AM[kk][1], rowp(F.Xm[0], L64, 16 * ut, 32 * kk, r16, grp),
                   rowp(F.Xm[1], L64, 16 * ut, 32 * kk, r16, grp));
      }
      const int u = 16 * ut + r16;
      const float gu = gu2[i];
      f32x4 dA;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = 16 * tw + 4 * grp + q;
        const float gam = t > u ? fexp2(gt4[q] - gu) : 0.f;
        const float dl = -ml[q];
        const float ag = KKt[i][q] * gam;
        db_acc[q] += dl * ag;
        const float hl = bt4[q] * dl * ag;
        dg_acc[q] += hl;
        colhl[i][q] = hl;
        dA[q] = dl * bt4[q] * gam;
      }
      put_N(F.GA[0], F.GA[1], L64, dA, tw, ut, r16, grp, sel);
      put_T(F.GTA[0], F.GTA[1], L64, dA, tw, ut, r16, grp);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float t = colhl[i][0] + colhl[i][1] + colhl[i][2] + colhl[i][3];
      t += __shfl_xor(t, 16, WAVE);
      t += __shfl_xor(t, 32, WAVE);
      if (grp == 0) sm.colHL[tw][16 * (2 * hk + i) + r16] = t;
    }
  }
  __syncthreads();
  GDN_REFRESH();
  // FB2: dK += (dA + dA^T) K; dk partial out
  {
    bf16x8 AA[2][2], AAT[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int pl = 0; pl < 2; ++pl) {
        AA[kk][pl] = rowp(F.GA[pl], L64, 16 * tw, 32 * kk, r16, grp);
        AAT[kk][pl] = rowp(F.GTA[pl], L64, 16 * tw, 32 * kk, r16, grp);
      }
#pragma unroll
    for (int j = 0; j < KH; ++j) {
      f32x4 acc = dK[j];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 ck = colp(F.Km, FLDK, 32 * kk, hk * KH + j, r16, grp, sel);
        acc = mm2(acc, AA[kk][0], AA[kk][1], ck);
        acc = mm2(acc, AAT[kk][0], AAT[kk][1], ck);
      }
      const int col = 16 * (hk * KH + j) + r16;
      if (half) {
        put_tile_half(dk_base, hk * KH + j, acc);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t = 16 * tw + 4 * grp + q;
          if (t < nc) put_grad(dk_base, t, col, acc[q]);
        }
      }
    }
  }
  // row totals over the 16 lanes of each row (this wave's column half)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float v3[3] = {dg_acc[q], term_acc[q], db_acc[q]};
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
      const int row = 16 * tw + 4 * grp + q;
      sm.rowDG[hk][row] = v3[0];
      sm.rowTerm[hk][row] = v3[1];
      sm.rowDB[hk][row] = v3[2];
    }
  }
  sSq = wave_sum(sSq);
  if (lane == 0) sm.red[wave] = sSq;
  __syncthreads();
  GDN_REFRESH();
  // d gamma_j = row part - column parts - state term_j; the last row also gets
  // e^gamma_n <dS', Sq> + sum_j term_j; dg = suffix sum of d gamma
  if (wave == 0) {
    const int j = lane;
    const float term = sm.rowTerm[0][j] + sm.rowTerm[1][j];
    const float term_total = wave_sum(term);
    float sq_total = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) sq_total += sm.red[w];
    float dgj = sm.rowDG[0][j] + sm.rowDG[1][j] - term -
                (sm.colH[0][j] + sm.colH[1][j] + sm.colH[2][j] + sm.colH[3][j]) -
                (sm.colHL[0][j] + sm.colHL[1][j] + sm.colHL[2][j] + sm.colHL[3][j]);
    if (j == nc - 1) dgj += gs.egC * sq_total + term_total;
    if (j >= nc) dgj = 0.f;
    float suf = dgj;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_down(suf, off, WAVE);
      if (j + off < 64) suf += y;
    }
    const float db = sm.colDB[0][j] + sm.colDB[1][j] + sm.colDB[2][j] + sm.colDB[3][j] +
                     sm.rowDB[0][j] + sm.rowDB[1][j];
    if (j < nc) {
      const int64_t gi = (int64_t)(t0 + j) * Hv + h;
      a.dg[gi] = suf;
      a.dbeta[gi] = db;
    }
  }
#undef GDN_REFRESH
}

template <int DK>
static hipError_t launch_local_dk(const BwdConfig& c, const BwdKernelArgs& a, hipStream_t s) {
  const dim3 grid(a.num_slots, c.Hv);
#define GDN_CASE(SFv, WFv) \
  if (c.state_fmt == SFv && c.w_fmt == WFv) { \
    if (a.f.solve_degree > 0) \
      hipLaunchKernelGGL((bwd_local_kernel<DK, SFv, WFv, true>), grid, dim3(NT), 0, s, a, c.N); \
    else \
      hipLaunchKernelGGL((bwd_local_kernel<DK, SFv, WFv, false>), grid, dim3(NT), 0, s, a, c.N); \
    return hipGetLastError(); \
  }
  GDN_CASE(0, 0) GDN_CASE(0, 1) GDN_CASE(0, 2)
  GDN_CASE(1, 0) GDN_CASE(1, 1) GDN_CASE(1, 2)
  GDN_CASE(2, 0) GDN_CASE(2, 1) GDN_CASE(2, 2)
#undef GDN_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_bwd_local(const BwdConfig& c, const BwdKernelArgs& a, hipStream_t s) {
  if (c.Dk == 128) return launch_local_dk<128>(c, a, s);
  if (c.Dk == 64) return launch_local_dk<64>(c, a, s);
  return hipErrorInvalidValue;
}

}  // namespace gdn
