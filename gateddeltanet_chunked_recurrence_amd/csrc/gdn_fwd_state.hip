// Forward, part 2: the sequential state recurrence and the output, one
// workgroup per (sequence, value head, value block), chunks in order. A value
// block is 64 columns (four waves of 16), or 128 / 256 columns (8 / 16 waves)
// when the state scale tile is that wide, so that every [Dk, block_v] tile's
// maximum is reduced inside one workgroup
// ("[1/4] GDN state/W QAT foundation", "What does this PR do?": state QDQ at
// every chunk; "[2/4] GDN/KDA decode QAT with INT8 recurrent state", "What
// does this PR do?": per-head [Dk, block_v] state scales).
//
// Per chunk, with the prep kernel's images (gdn_images.h) and the state S
// (FP32, Dk x 64, in registers: wave w holds value columns 16w..16w+15 in
// accumulator layout):
//   Sq   = QDQ_S(S)                              amax from the previous chunk
//   Vnew = U - dW dS (Wc Sc)                     codes exact in bf16
//   O    = scale (exp(gamma) dS (Q Sc) + P Vnew)
//   S    = exp(gamma_n) Sq + K^T (exp(gamma_n - gamma) Vnew)
// One barrier per chunk: the next chunk's images are copied into the other
// LDS buffer from registers loaded one chunk earlier, and each wave's amax of
// the new state is exchanged through LDS for the next chunk's scale.
//
// Launch order pairs the value blocks of one head on one XCD (workgroup ids
// congruent mod 8), so the second block's reads of Q and the images hit the
// XCD's L2.
#include <hip/hip_ext.h>

#include "gdn_device.h"
#include "gdn_images.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

template <int DK, int NW>
struct StateBuf {
  bf16 Q[Img<DK>::WQ];
  bf16 W[NW * Img<DK>::WQ];
  bf16 Kt[Img<DK>::KT];
  bf16 P[2 * Img<DK>::P1];
  alignas(16) float G[Img<DK>::GB / 2];                   // exp(gamma), exp(gamma_n - gamma), exp(gamma_n)
};

// NWV waves of 16 value columns each (4, 8 or 16).
template <int DK, int NW, int NWV>
struct StateCfg {
  using I = Img<DK>;
  static constexpr int NT = 64 * NWV;
  static constexpr int NBUF = ((DK == 128 && NW == 2) || NWV == 16) ? 1 : 2;
  static constexpr int QN = 64 * DK / 8;                  // 16-byte Q pieces of a chunk
  static constexpr int QPT = (QN + NT - 1) / NT;          // ... per thread (the last ones guarded)
  static constexpr int IMGP = I::template img<NW>() / 8;  // 16-byte pieces of one image block
};

template <int DK, int NW, int NWV>
struct StateSmem {
  StateBuf<DK, NW> buf[StateCfg<DK, NW, NWV>::NBUF];
  alignas(16) bf16 ost[NWV][64 * 16];                     // per wave: O tile, row-major
  float red[2][NWV];                                      // per-wave state amax, by chunk parity
};

// Staging of one chunk's operands into an LDS buffer. The image block (W
// planes, K^T, P; contiguous in the workspace and in the buffer) goes by
// direct global-to-LDS loads, 1 KB per wave instruction (lane i fills bytes
// 16i..16i+15 of it), with no registers involved; its completion is covered
// by the vmcnt(0) before the chunk's barrier. Q is reordered (pperm +
// swizzle) on the way, through 16-byte register loads; rows past the chunk
// end repeat the last row (they only feed output rows that are not stored).
template <int DK, int NW, int NWV>
struct Stager {
  using C = StateCfg<DK, NW, NWV>;
  static constexpr int NT = C::NT;
  using I = Img<DK>;
  static constexpr int NINS = C::IMGP / 64;               // wave instructions per image block
  static_assert(C::IMGP % 64 == 0, "image block is a whole number of wave loads");
  uint4 q[C::QPT];
  __device__ void load_q(const FwdKernelArgs& a, int t0, int nc, int hk, int tid) {
    const bf16* qb = reinterpret_cast<const bf16*>(a.q);
#pragma unroll
    for (int p = 0; p < C::QPT; ++p) {
      const int e = min(tid + NT * p, C::QN - 1), row = e / (DK / 8), c8 = e % (DK / 8);
      q[p] = *reinterpret_cast<const uint4*>(
          qb + ((int64_t)(t0 + min(row, nc - 1)) * a.Hqk + hk) * DK + 8 * c8);
    }
  }
  __device__ void store_q(StateBuf<DK, NW>& b, int tid) const {
#pragma unroll
    for (int p = 0; p < C::QPT; ++p) {
      const int e = tid + NT * p, row = e / (DK / 8), c8 = e % (DK / 8);
      if (C::QN % NT != 0 && e >= C::QN) continue;
      *reinterpret_cast<uint2*>(&b.Q[wq_off<DK>(row, pperm(8 * c8))]) = make_uint2(q[p].x, q[p].y);
      *reinterpret_cast<uint2*>(&b.Q[wq_off<DK>(row, pperm(8 * c8 + 4))]) = make_uint2(q[p].z, q[p].w);
    }
  }
  // Part `part` of NP of this wave's wave loads of the image block: j = wave
  // + NWV k, clamped to the last one (a repeated load rewrites the same
  // bytes), so every wave issues the same compile-time number of loads and
  // the compiler can wait for older register loads precisely.
  template <int NP>
  static __device__ void dma_img(const FwdKernelArgs& a, int64_t ch, StateBuf<DK, NW>& b, int wave,
                                 int lane, int part) {
    constexpr int KW = (NINS + NWV - 1) / NWV;
    const uint4* src = reinterpret_cast<const uint4*>(a.ws_img + ch * I::template img<NW>());
    uint4* dst = reinterpret_cast<uint4*>(b.W);
#pragma unroll
    for (int k = KW * part / NP; k < KW * (part + 1) / NP; ++k) {
      const int j = min(wave + NWV * k, NINS - 1);
      __builtin_amdgcn_global_load_lds(src + 64 * j + lane, dst + 64 * j, 16, 0, 0);
    }
  }
};

// RF: the two-precision profile ("[5/8] ReplaySSM state QAT and two-precision
// GDN", "What does this PR do?"; SF = 0): the state S is carried in FP32 and
// only its reads (W S and Q S) use a dynamic E4M3 copy with one scale per
// value column over the Dk key channels. For the backward, the read copy of
// each chunk's incoming state (codes times scales, FP32) goes to s_f32 and the
// FP32 state itself to s_anchor.
template <int DK, int SF, int WF, int NWV, bool RF>
__global__ void __launch_bounds__(64 * NWV, 1) gdn_state_kernel(FwdKernelArgs a, int N, int num_heads) {
  static_assert(!RF || (SF == 0 && NWV == 4), "the read copy replaces the state quantizer");
  constexpr int NW = WF == 0 ? 2 : 1;
  using C = StateCfg<DK, NW, NWV>;
  using I = Img<DK>;
  constexpr int MK = DK / 16;                      // 16-row tiles of the state
  static_assert(sizeof(StateBuf<DK, NW>) == 2 * (I::WQ + I::template img<NW>()),
                "W, K^T, P and gate images are contiguous after Q");
  static_assert(sizeof(StateSmem<DK, NW, NWV>) <= 160 * 1024, "LDS");
  __shared__ __align__(16) StateSmem<DK, NW, NWV> sm;

  const int Hv = a.Hv, Dv = a.Dv, NVB = Dv / 64;  // NVB: 64-column blocks (U fragment order)
  const int NWB = Dv / (16 * NWV);                 // value blocks of this kernel
  // workgroup id -> (head index, value block); the blocks of a head share an XCD
  const int bid = blockIdx.x, xcd = bid & 7, r8 = bid >> 3;
  const int vb = r8 % NWB, hidx = xcd + 8 * (r8 / NWB);
  if (hidx >= num_heads) return;
  const int n = hidx / Hv, h = hidx % Hv;
  const int hk = h / (Hv / a.Hqk);
  int bos, eos;
  seq_span(a, n, bos, eos);
  const int nchunks = (eos - bos + CHUNK - 1) / CHUNK;
  const int slot0 = n + bos / CHUNK;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int lane = fresh_lane(), tid = wave * 64 + lane, r16 = lane & 15, grp = lane >> 4;
  // per-lane LDS addresses are rebuilt in each phase instead of being kept live
  // across the chunk loop (fresh_lane in gdn_device.h)
#define GDN_REFRESH() \
  lane = fresh_lane(); tid = wave * 64 + lane; r16 = lane & 15; grp = lane >> 4
  const int wcol = vb * 16 * NWV + wave * 16;      // first value column of this wave
  const int ug = wcol / 16;                        // 16-column group in U's fragment order
  const int64_t state_base = ((int64_t)n * Hv + h) * DK * Dv;

  // state in accumulator layout: S[mt][i] = S[16 mt + 4 grp + i][wcol + r16]
  f32x4 S[MK];
  if (a.h0) {
    const float* hp = a.h0 + state_base + wcol + r16;
#pragma unroll
    for (int mt = 0; mt < MK; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[mt][i] = hp[(int64_t)(16 * mt + 4 * grp + i) * Dv];
  } else {
#pragma unroll
    for (int mt = 0; mt < MK; ++mt) S[mt] = zero4();
  }
  if (nchunks == 0) {
    if (a.ht) {
#pragma unroll
      for (int mt = 0; mt < MK; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a.ht[state_base + (int64_t)(16 * mt + 4 * grp + i) * Dv + wcol + r16] = S[mt][i];
    }
    return;
  }

  auto chunk_t0 = [&](int c) { return bos + CHUNK * c; };
  auto chunk_nc = [&](int c) { return min(CHUNK, eos - bos - CHUNK * c); };
  auto chunk_ch = [&](int c) { return (int64_t)(slot0 + c) * Hv + h; };

  // per-chunk registers: U fragment and W scale
  f32x4 Ucur[4], Unext[4];
  float dWcur = 1.f, dWnext = 1.f;
  auto load_small = [&](int c, f32x4 (&U)[4], float& dW) {
    const int64_t ch = chunk_ch(c);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      U[mt] = *reinterpret_cast<const f32x4*>(a.ws_u + u_off(ch, NVB, ug >> 2, ug & 3, mt, lane));
    dW = a.ws_wscale[ch];
  };

  // Beside a concurrent prep kernel (flags set): before its loads of chunk
  // c's operands every wave sees that chunk's ready flag, bounded to about
  // 2^27 clocks (on give-up the error flag is set and the work goes on).
  auto wait_ready = [&](int c) {
    if (!a.flags) return;
    const uint32_t* fl = a.flags + chunk_ch(c);
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    while (__hip_atomic_load(fl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
      if (__builtin_amdgcn_s_memtime() - t0 > (1ull << 27)) {
        if (lane == 0) __hip_atomic_fetch_or(a.err, kErrFlagWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  };

  Stager<DK, NW, NWV> stg;
  stg.load_q(a, chunk_t0(0), chunk_nc(0), hk, tid);
  wait_ready(0);
  Stager<DK, NW, NWV>::template dma_img<1>(a, chunk_ch(0), sm.buf[0], wave, lane, 0);
  load_small(0, Ucur, dWcur);
  stg.store_q(sm.buf[0], tid);
  if (nchunks > 1) stg.load_q(a, chunk_t0(1), chunk_nc(1), hk, tid);
  if constexpr (SF != 0) {
    float m = 0.f;
#pragma unroll
    for (int mt = 0; mt < MK; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(S[mt][i]));
    m = wave_max(m);
    if (lane == 0) sm.red[0][wave] = m;
  }
  vm_drain();
  lds_barrier();

  const int gs = (SF != 0) ? a.block_v / 16 : 1;  // waves per scale tile
  const int g0 = (wave / gs) * gs;

  for (int c = 0; c < nchunks; ++c) {
    const int t0 = chunk_t0(c), nc = chunk_nc(c);
    const int64_t ch = chunk_ch(c);
    const StateBuf<DK, NW>& B = sm.buf[C::NBUF == 2 ? (c & 1) : 0];
    GDN_REFRESH();
    // staging of chunk c + 1 into the other buffer, issued in three parts
    // between the phases below so the loads drain while the chunk computes
    const bool more = C::NBUF == 2 && c + 1 < nchunks;
    if (c + 1 < nchunks) wait_ready(c + 1);       // before any load of chunk c + 1's operands
    auto stage_part = [&](int part) {
      if constexpr (C::NBUF == 2) {
        if (more) Stager<DK, NW, NWV>::template dma_img<3>(a, chunk_ch(c + 1), sm.buf[(c + 1) & 1], wave, lane, part);
      }
    };
    stage_part(0);
    if (more) {
      stg.store_q(sm.buf[(c + 1) & 1], tid);
      if (c + 2 < nchunks) stg.load_q(a, chunk_t0(c + 2), chunk_nc(c + 2), hk, tid);
    }
    if (c + 1 < nchunks) load_small(c + 1, Unext, dWnext);

    // ---- gates of this chunk (from the prep kernel's gate block)
    const float egC = B.G[128];
    f32x4 egr[4], egcr[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      egr[mt] = *reinterpret_cast<const f32x4*>(&B.G[16 * mt + 4 * grp]);
      egcr[mt] = *reinterpret_cast<const f32x4*>(&B.G[64 + 16 * mt + 4 * grp]);
    }

    // ---- Sq = QDQ_S(S): codes in S, scale dS
    float dS = 1.f;
    if constexpr (SF != 0) {
      float amax = 0.f;
      for (int t = g0; t < g0 + gs; ++t) amax = fmaxf(amax, sm.red[c & 1][t]);
      dS = qdq_scale<SF>(amax);
      const float rS = 1.0f / dS;
      uint8_t* sb = a.s_codes ? a.s_codes + ch * DK * Dv + wcol + r16 : nullptr;
#pragma unroll
      for (int mt = 0; mt < MK; ++mt) {
        const float x[4] = {S[mt][0], S[mt][1], S[mt][2], S[mt][3]};
        float cq[4];
        uint32_t bytes;
        quant4<SF>(x, rS, cq, bytes);
#pragma unroll
        for (int i = 0; i < 4; ++i) S[mt][i] = cq[i];
        if (sb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) sb[(int64_t)(16 * mt + 4 * grp + i) * Dv] = (bytes >> (8 * i)) & 0xFFu;
        }
      }
      if (sb && wave == g0 && lane == 0) a.s_scale[ch * (Dv / a.block_v) + wcol / a.block_v] = dS;
    } else if (!RF && a.s_f32) {
      float* sb = a.s_f32 + ch * DK * Dv + wcol + r16;
#pragma unroll
      for (int mt = 0; mt < MK; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sb[(int64_t)(16 * mt + 4 * grp + i) * Dv] = S[mt][i];
    }
    bf16x8 bSh[MK / 2], bSl[MK / 2];
    float dR = 1.f;                                // this lane's column scale of the read copy
    if constexpr (RF) {
      // the column's maximum: 32 values in this lane, then the four lanes
      // (one per lane group) that hold the same column
      float m = 0.f;
#pragma unroll
      for (int mt = 0; mt < MK; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(S[mt][i]));
      m = fmaxf(m, __shfl_xor(m, 16, WAVE));
      m = fmaxf(m, __shfl_xor(m, 32, WAVE));
      dR = qdq_scale<1>(m);
      const float rR = 1.0f / dR;
      float* sr = a.s_f32 ? a.s_f32 + ch * DK * Dv + wcol + r16 : nullptr;
      float* sa = a.s_anchor ? a.s_anchor + ch * DK * Dv + wcol + r16 : nullptr;
#pragma unroll
      for (int kk = 0; kk < MK / 2; ++kk) {
        f32x4 c2[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int mt = 2 * kk + h2;
          const float x[4] = {S[mt][0], S[mt][1], S[mt][2], S[mt][3]};
          float cq[4];
          uint32_t bytes;
          quant4<1>(x, rR, cq, bytes);
          c2[h2] = f32x4{cq[0], cq[1], cq[2], cq[3]};
          if (sr) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              sr[(int64_t)(16 * mt + 4 * grp + i) * Dv] = cq[i] * dR;
              sa[(int64_t)(16 * mt + 4 * grp + i) * Dv] = x[i];
            }
          }
        }
        bSh[kk] = pack_pair(c2[0], c2[1]);         // codes, exact in bf16
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < MK / 2; ++kk) {
        if constexpr (SF != 0) bSh[kk] = pack_pair(S[2 * kk], S[2 * kk + 1]);
        else pack_pair_split(S[2 * kk], S[2 * kk + 1], bSh[kk], bSl[kk]);
      }
    }

    stage_part(1);
    // ---- W Sq and Q Sq (A operands from the images, B from registers)
    GDN_REFRESH();
    f32x4 accw[4], accq[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) accw[mt] = accq[mt] = zero4();
    {
      bf16x8 opw[2][4][NW], opq[2][4];
      auto load_k = [&](int kk, bf16x8 (&w)[4][NW], bf16x8 (&q)[4]) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int row = 16 * mt + r16;
#pragma unroll
          for (int pl = 0; pl < NW; ++pl) w[mt][pl] = ld_wq<DK>(B.W + pl * I::WQ, row, kk, grp);
          q[mt] = ld_wq<DK>(B.Q, row, kk, grp);
        }
      };
      load_k(0, opw[0], opq[0]);
#pragma unroll
      for (int kk = 0; kk < MK / 2; ++kk) {
        if (kk + 1 < MK / 2) load_k(kk + 1, opw[(kk + 1) & 1], opq[(kk + 1) & 1]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const auto& w = opw[kk & 1][mt];
          const bf16x8& q = opq[kk & 1][mt];
          accw[mt] = mfma(w[0], bSh[kk], accw[mt]);
          accq[mt] = mfma(q, bSh[kk], accq[mt]);
          if constexpr (NW == 2) accw[mt] = mfma(w[NW - 1], bSh[kk], accw[mt]);
          if constexpr (SF == 0 && !RF) {
            accw[mt] = mfma(w[0], bSl[kk], accw[mt]);
            accq[mt] = mfma(q, bSl[kk], accq[mt]);
          }
        }
      }
    }
    f32x4 Vn[4];
    {
      const float sc = dWcur * dS * dR;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Vn[mt][i] = Ucur[mt][i] - sc * accw[mt][i];
          accq[mt][i] *= dS * dR * egr[mt][i];
        }
    }
    // Vnew and exp(gamma_n - gamma) Vnew as B operands (paired order over tokens)
    bf16x8 bVh[2], bVl[2], bDh[2], bDl[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      pack_pair_split(Vn[2 * kk], Vn[2 * kk + 1], bVh[kk], bVl[kk]);
      f32x4 d0, d1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        d0[i] = egcr[2 * kk][i] * Vn[2 * kk][i];
        d1[i] = egcr[2 * kk + 1][i] * Vn[2 * kk + 1][i];
      }
      pack_pair_split(d0, d1, bDh[kk], bDl[kk]);
    }
    stage_part(2);
    // ---- O = scale (exp(gamma) dS Q Sq + P Vnew)
    GDN_REFRESH();
    {
      bf16x8 ph[4][2], pl[4][2];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (kk > mt / 2) continue;              // P is lower triangular
          ph[mt][kk] = ld_r64(B.P, 16 * mt + r16, 32 * kk, grp);
          pl[mt][kk] = ld_r64(B.P + I::P1, 16 * mt + r16, 32 * kk, grp);
        }
      bf16* ot = sm.ost[wave];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 acc = accq[mt];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (kk > mt / 2) continue;
          acc = mfma(ph[mt][kk], bVh[kk], acc);
          acc = mfma(pl[mt][kk], bVh[kk], acc);
          acc = mfma(ph[mt][kk], bVl[kk], acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) ot[(16 * mt + 4 * grp + i) * 16 + r16] = to_bf16(a.scale * acc[i]);
      }
      // 16-byte row pieces of this wave's [64 x 16] O tile
      bf16* op = reinterpret_cast<bf16*>(a.o) + ((int64_t)t0 * Hv + h) * Dv + wcol;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int pc = lane + 64 * k, row = pc >> 1, half = pc & 1;
        const uint4 v = *reinterpret_cast<const uint4*>(&ot[row * 16 + 8 * half]);
        if (row < nc) *reinterpret_cast<uint4*>(op + (int64_t)row * Hv * Dv + 8 * half) = v;
      }
    }
    // ---- S = exp(gamma_n) Sq + K^T (exp(gamma_n - gamma) Vnew)
    GDN_REFRESH();
    {
      const float sdec = egC * dS;
#pragma unroll
      for (int mt = 0; mt < MK; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[mt][i] *= sdec;
      bf16x8 kop[2][MK];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int mt = 0; mt < MK; ++mt) kop[kk][mt] = ld_r64(B.Kt, 16 * mt + r16, 32 * kk, grp);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int mt = 0; mt < MK; ++mt) {
          S[mt] = mfma(kop[kk][mt], bDh[kk], S[mt]);
          S[mt] = mfma(kop[kk][mt], bDl[kk], S[mt]);
        }
    }
    if constexpr (SF != 0) {
      float m = 0.f;
#pragma unroll
      for (int mt = 0; mt < MK; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(S[mt][i]));
      m = wave_max(m);
      if (lane == 0) sm.red[(c + 1) & 1][wave] = m;
    }
    if constexpr (C::NBUF == 1) {
      lds_barrier();                             // every wave is done with the buffer
      GDN_REFRESH();
      if (c + 1 < nchunks) {
        Stager<DK, NW, NWV>::template dma_img<1>(a, chunk_ch(c + 1), sm.buf[0], wave, lane, 0);
        stg.store_q(sm.buf[0], tid);
        if (c + 2 < nchunks) stg.load_q(a, chunk_t0(c + 2), chunk_nc(c + 2), hk, tid);
      }
    }
    vm_drain();                                   // this wave's staging of chunk c + 1 landed
    lds_barrier();
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) Ucur[mt] = Unext[mt];
    dWcur = dWnext;
  }

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

}  // namespace

template <int DK, int SF, int WF, int NWV, bool RF = false>
static hipError_t launch_state_w(const FwdConfig& cfg, const FwdKernelArgs& a, hipStream_t s,
                                 hipEvent_t stop) {
  const int num_heads = cfg.N * cfg.Hv, nwb = cfg.Dv / (16 * NWV);
  const int64_t nblk = (int64_t)nwb * 8 * ((num_heads + 7) / 8);
  if (stop)
    hipExtLaunchKernelGGL((gdn_state_kernel<DK, SF, WF, NWV, RF>), dim3((unsigned)nblk),
                          dim3(64 * NWV), 0, s, nullptr, stop, 0, a, cfg.N, num_heads);
  else
    hipLaunchKernelGGL((gdn_state_kernel<DK, SF, WF, NWV, RF>), dim3((unsigned)nblk), dim3(64 * NWV),
                       0, s, a, cfg.N, num_heads);
  return hipGetLastError();
}

// Value block width: the state scale tile when it is wider than 64 columns.
template <int DK, int SF, int WF>
static hipError_t launch_state_one(const FwdConfig& cfg, const FwdKernelArgs& a, hipStream_t s,
                                   hipEvent_t stop) {
  if constexpr (SF != 0) {
    if (cfg.block_v == 256) return launch_state_w<DK, SF, WF, 16>(cfg, a, s, stop);
    if (cfg.block_v == 128) return launch_state_w<DK, SF, WF, 8>(cfg, a, s, stop);
  } else {
    if (cfg.read_fmt != 0) {
      if constexpr (DK == 128) return launch_state_w<DK, SF, WF, 4, true>(cfg, a, s, stop);
      return hipErrorInvalidValue;                 // the read copy is built for Dk = 128
    }
  }
  return launch_state_w<DK, SF, WF, 4>(cfg, a, s, stop);
}

template <int DK>
static hipError_t launch_state_dk(const FwdConfig& cfg, const FwdKernelArgs& a, hipStream_t s,
                                  hipEvent_t stop) {
#define GDN_CASE(SFv, WFv) \
  if (cfg.state_fmt == SFv && cfg.w_fmt == WFv) return launch_state_one<DK, SFv, WFv>(cfg, a, s, stop);
  GDN_CASE(0, 0) GDN_CASE(0, 1) GDN_CASE(0, 2)
  GDN_CASE(1, 0) GDN_CASE(1, 1) GDN_CASE(1, 2)
  GDN_CASE(2, 0) GDN_CASE(2, 1) GDN_CASE(2, 2)
#undef GDN_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_state(const FwdConfig& cfg, const FwdKernelArgs& a, hipStream_t s,
                            hipEvent_t stop) {
  if (a.w_img_bytes) return launch_fwd_state_split(cfg, a, s, stop);
  if (cfg.Dk == 128) return launch_state_dk<128>(cfg, a, s, stop);
  if (cfg.Dk == 64) return launch_state_dk<64>(cfg, a, s, stop);
  return hipErrorInvalidValue;
}

}  // namespace gdn
