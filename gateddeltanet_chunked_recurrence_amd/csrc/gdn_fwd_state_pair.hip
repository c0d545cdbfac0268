// Forward state recurrence with both QDQ sites on, 8 waves per (sequence,
// value head, 64-wide value block): two waves per SIMD share each 16-column
// group of the state ("[1/4] GDN state/W QAT foundation", "What does this PR
// do?"; "[2/4] GDN/KDA decode QAT with INT8 recurrent state", "What does this
// PR do?": per-head [Dk, block_v] state scales). Same arithmetic per chunk as
// the 4-wave kernel in gdn_fwd_state.hip:
//   Sq   = QDQ_S(S);  Vnew = U - dW dS (Wc Sc)
//   O    = scale (exp(gamma) dS (Q Sc) + P Vnew)
//   S    = exp(gamma_n) Sq + K^T (exp(gamma_n - gamma) Vnew)
//
// Wave w owns column group cg = w & 3 and half hf = w >> 2. It keeps the state
// rows dk in [Dk/2 hf, Dk/2 (hf + 1)) of its columns, and computes Vnew and O
// for two 16-token row tiles (half 0: tiles 0 and 3, half 1: tiles 1 and 2,
// which balances the work under the lower-triangular P). Per chunk:
//   1. QDQ of its state half; its half of the Sq B operand goes to LDS;
//      barrier A; the partner's half is read back
//   2. W Sq and Q Sq for its 32 tokens; Vnew (FP32) to LDS; barrier B
//   3. O for its row tiles and S for its state rows, from both halves' Vnew;
//      amax; barrier C
// Two waves per SIMD hide each other's latency and double the LDS read rate
// over one wave per SIMD. The next chunk's image block goes to the other LDS
// buffer by direct global-to-LDS loads issued at the top of the chunk (every
// wave issues the same compile-time number; the last index is clamped, so a
// repeated load rewrites the same bytes) and waited for (vmcnt) before
// barrier C. Its Q (single-buffered) is loaded into registers at the top of
// the chunk and written to LDS after barrier B, when every wave is done with
// the current one. Barriers are LDS-only (lds_barrier): loads in flight are
// not drained by them.
#include "gdn_device.h"
#include "gdn_images.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

constexpr int NT = 512;

template <int DK>
struct PairSmem {
  using I = Img<DK>;
  struct Buf {                                    // one image block (W codes, K^T, P, gates)
    bf16 W[I::WQ];
    bf16 Kt[I::KT];
    bf16 P[2 * I::P1];
    alignas(16) float G[I::GB / 2];
  };
  Buf buf[2];
  bf16 Q[I::WQ];                                  // W image layout
  union {
    bf16x8 sqx[8][DK / 64][64];                   // per wave: its Sq B-operand k-steps
    bf16 ost[8][32 * 16];                         // per wave: its [32 x 16] O tile
  } x1;
  f32x4 vnx[8][2][64];                            // per wave: Vnew of its two row tiles
  float red[2][8];                                // per-wave state amax, by chunk parity
};

template <int DK, int SF, int WF>
__global__ void __launch_bounds__(NT, 1) __attribute__((amdgpu_waves_per_eu(1, 2)))
gdn_state_pair_kernel(FwdKernelArgs a, int N, int num_heads) {
  static_assert(SF != 0 && WF != 0, "both QDQ sites on");
  using I = Img<DK>;
  using Sm = PairSmem<DK>;
  constexpr int MK = DK / 16;                     // 16-row tiles of the state
  constexpr int MKH = MK / 2;                     // ... held by one wave
  constexpr int KS = DK / 32;                     // 32-deep k-steps over dk
  constexpr int KSH = KS / 2;                     // ... from one wave
  constexpr int IMGP = I::template img<1>() / 8;  // 16-byte pieces of an image block
  static_assert(sizeof(typename Sm::Buf) == 16 * IMGP, "image block layout");
  __shared__ __align__(16) Sm sm;

  const int Hv = a.Hv, Dv = a.Dv, NVB = Dv / 64;
  // workgroup id -> (head index, value block); the blocks of a head share an XCD
  const int bid = blockIdx.x, xcd = bid & 7, r8 = bid >> 3;
  const int vb = r8 % NVB, hidx = xcd + 8 * (r8 / NVB);
  if (hidx >= num_heads) return;
  const int n = hidx / Hv, h = hidx % Hv;
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

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cg = wave & 3, hf = wave >> 2, partner = wave ^ 4;
  const int lane = __lane_id(), tid = wave * 64 + lane, r16 = lane & 15, grp = lane >> 4;
  const int wcol = vb * 64 + cg * 16;             // first value column of this wave
  const int dk0 = hf * (DK / 2);                  // first state row of this wave
  const int64_t state_base = ((int64_t)n * Hv + h) * DK * Dv;

  // own state rows in accumulator layout: S[j][i] = S[dk0 + 16 j + 4 grp + i][wcol + r16]
  f32x4 S[MKH];
  if (a.h0) {
    const float* hp = a.h0 + state_base + (int64_t)dk0 * Dv + wcol + r16;
#pragma unroll
    for (int j = 0; j < MKH; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[j][i] = hp[(int64_t)(16 * j + 4 * grp + i) * Dv];
  } else {
#pragma unroll
    for (int j = 0; j < MKH; ++j) S[j] = zero4();
  }
  auto store_ht = [&]() {
    if (!a.ht) return;
    float* hp = a.ht + state_base + (int64_t)dk0 * Dv + wcol + r16;
#pragma unroll
    for (int j = 0; j < MKH; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) hp[(int64_t)(16 * j + 4 * grp + i) * Dv] = S[j][i];
  };
  if (nchunks == 0) {
    store_ht();
    return;
  }

  auto chunk_t0 = [&](int c) { return bos + CHUNK * c; };
  auto chunk_nc = [&](int c) { return min(CHUNK, eos - bos - CHUNK * c); };
  auto chunk_ch = [&](int c) { return (int64_t)(slot0 + c) * Hv + h; };

  // Q of a chunk through registers (pperm + swizzle on the way; rows past the
  // chunk end repeat the last row and only feed unstored output rows)
  constexpr int QPT = 64 * DK / 8 / NT;           // 16-byte Q pieces per thread
  // Q rows go through registers two chunks ahead: qnext holds chunk c + 1's
  // (loaded during chunk c - 1, complete by that chunk's final wait), qreg
  // receives chunk c + 2's during chunk c. The write of qnext to LDS then needs
  // no wait, which would otherwise also wait for the image copy in flight.
  u32x4 qreg[QPT], qnext[QPT];
  auto load_q = [&](int c) {
    const bf16* qb = reinterpret_cast<const bf16*>(a.q);
    const int t0 = chunk_t0(c), nc = chunk_nc(c);
#pragma unroll
    for (int p = 0; p < QPT; ++p) {
      const int e = tid + NT * p, row = e / (DK / 8), c8 = e % (DK / 8);
      qreg[p] = *reinterpret_cast<const u32x4*>(qb + ((int64_t)(t0 + min(row, nc - 1)) * a.Hqk + hk) * DK + 8 * c8);
    }
  };
  auto store_q = [&](const u32x4 (&q)[QPT]) {
#pragma unroll
    for (int p = 0; p < QPT; ++p) {
      const int e = tid + NT * p, row = e / (DK / 8), c8 = e % (DK / 8);
      typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
      *reinterpret_cast<u32x2*>(&sm.Q[wq_off<DK>(row, pperm(8 * c8))]) = q[p].xy;
      *reinterpret_cast<u32x2*>(&sm.Q[wq_off<DK>(row, pperm(8 * c8 + 4))]) = q[p].zw;
    }
  };
  constexpr int NINS = IMGP / 64;                 // wave loads per image block
  constexpr int KW = (NINS + 7) / 8;               // ... per wave
  constexpr int KD0 = (KW + 2) / 3, KD1 = KD0 + (KW - KD0 + 1) / 2;   // split points
  static_assert(IMGP % 64 == 0, "whole wave loads");
  auto dma = [&](int c, int b, int k0, int k1) {
    const uint4* src = reinterpret_cast<const uint4*>(a.ws_img + chunk_ch(c) * I::template img<1>());
    uint4* dst = reinterpret_cast<uint4*>(sm.buf[b].W);
#pragma unroll
    for (int k = k0; k < k1; ++k) {
      const int j = min(wave + 8 * k, NINS - 1);
      __builtin_amdgcn_global_load_lds(src + 64 * j + lane, dst + 64 * j, 16, 0, 0);
    }
  };
  // token row tiles of this wave: one of the two short ones and one of the two
  // long ones under the lower-triangular P (half 0: tiles 0, 3; half 1: 1, 2)
  const int rt0 = hf, rt1 = 3 - hf;
  // U fragments of this wave's two row tiles, and the W scale
  f32x4 Ucur[2], Unext[2];
  float dWcur = 1.f, dWnext = 1.f;
  auto load_small = [&](int c, f32x4 (&U)[2], float& dW) {
    const int64_t ch = chunk_ch(c);
    U[0] = *reinterpret_cast<const f32x4*>(a.ws_u + u_off(ch, NVB, vb, cg, rt0, lane));
    U[1] = *reinterpret_cast<const f32x4*>(a.ws_u + u_off(ch, NVB, vb, cg, rt1, lane));
    dW = a.ws_wscale[ch];
  };

  load_q(0);
  dma(0, 0, 0, KW);
  load_small(0, Ucur, dWcur);
  store_q(qreg);
  load_q(min(1, nchunks - 1));
  vm_drain();                                     // chunk 0's image block landed
#pragma unroll
  for (int p = 0; p < QPT; ++p) qnext[p] = qreg[p];
  {
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < MKH; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(S[j][i]));
    m = wave_max(m);
    if (lane == 0) sm.red[0][wave] = m;
  }
  lds_barrier();

  const int gs = a.block_v / 16;                  // column groups per scale tile
  const int g0 = (cg / gs) * gs;

  for (int c = 0; c < nchunks; ++c) {
    const int t0 = chunk_t0(c), nc = chunk_nc(c);
    const int64_t ch = chunk_ch(c);
    const typename Sm::Buf& B = sm.buf[c & 1];
    // staging of chunk c + 1 (the last chunk repeats itself: the loads are
    // unconditional, which keeps the compiler's wait before store_q exact)
    const int cn = min(c + 1, nchunks - 1);
    load_q(min(c + 2, nchunks - 1));               // written to LDS in the next chunk
    // the image copy goes out in three parts (here, after barrier A, after
    // barrier B): issued at once, its wave loads stall the issuing wave
    dma(cn, (c + 1) & 1, 0, KD0);
    load_small(cn, Unext, dWnext);

    // ---- gates of this chunk: exp(gamma) of the own row tiles, and
    //      exp(gamma_n - gamma) of all four (for the state update)
    const float egC = B.G[128];
    f32x4 egr[2], egc[4];
    egr[0] = *reinterpret_cast<const f32x4*>(&B.G[16 * rt0 + 4 * grp]);
    egr[1] = *reinterpret_cast<const f32x4*>(&B.G[16 * rt1 + 4 * grp]);
#pragma unroll
    for (int t = 0; t < 4; ++t) egc[t] = *reinterpret_cast<const f32x4*>(&B.G[64 + 16 * t + 4 * grp]);

    // ---- 1. QDQ of the own state half; its B-operand k-steps to LDS
    float amax = 0.f;
    for (int t = g0; t < g0 + gs; ++t) amax = fmaxf(amax, fmaxf(sm.red[c & 1][t], sm.red[c & 1][t + 4]));
    const float dS = qdq_scale<SF>(amax);
    // codes of the saved state, stored after store_q below: with only loads
    // in flight there, the wait for Q's registers is exact and leaves the
    // next chunk's image copy and U loads in flight
    uint32_t sbytes[MKH];
    {
      const float rS = 1.0f / dS;
#pragma unroll
      for (int j = 0; j < MKH; ++j) {
        const float x[4] = {S[j][0], S[j][1], S[j][2], S[j][3]};
        float cq[4];
        quant4<SF>(x, rS, cq, sbytes[j]);
#pragma unroll
        for (int i = 0; i < 4; ++i) S[j][i] = cq[i];
      }
    }
    // own k-steps (KSH of them) to LDS; the operand for k-step kk is then
    // selected from own / partner halves with compile-time indices only
    // (hf is a runtime value: indexing register arrays with it would spill
    // them to lane moves)
    bf16x8 bOwn[KSH], bPar[KSH];
#pragma unroll
    for (int j = 0; j < KSH; ++j) {
      bOwn[j] = pack_pair(S[2 * j], S[2 * j + 1]);
      sm.x1.sqx[wave][j][lane] = bOwn[j];
    }
    lds_barrier();                               // A: Sq halves published
    dma(cn, (c + 1) & 1, KD0, KD1);
#pragma unroll
    for (int j = 0; j < KSH; ++j) bPar[j] = sm.x1.sqx[partner][j][lane];
    bf16x8 bS[KS];                                 // k-steps of the first half, then the second
#pragma unroll
    for (int j = 0; j < KSH; ++j) {
      bS[j] = hf == 0 ? bOwn[j] : bPar[j];
      bS[KSH + j] = hf == 0 ? bPar[j] : bOwn[j];
    }

    // ---- 2. W Sq and Q Sq for the own 32 tokens (row tiles 2 hf, 2 hf + 1)
    f32x4 accw[2], accq[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) accw[r] = accq[r] = zero4();
    {
      bf16x8 opw[2][2], opq[2][2];
      auto load_k = [&](int kk, bf16x8 (&w)[2], bf16x8 (&q)[2]) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int row = 16 * (r ? rt1 : rt0) + r16;
          w[r] = ld_wq<DK>(B.W, row, kk, grp);
          q[r] = ld_wq<DK>(sm.Q, row, kk, grp);
        }
      };
      load_k(0, opw[0], opq[0]);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        if (kk + 1 < KS) load_k(kk + 1, opw[(kk + 1) & 1], opq[(kk + 1) & 1]);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          accw[r] = mfma(opw[kk & 1][r], bS[kk], accw[r]);
          accq[r] = mfma(opq[kk & 1][r], bS[kk], accq[r]);
        }
      }
    }
    f32x4 Vn[2];
    {
      const float sc = dWcur * dS;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Vn[r][i] = Ucur[r][i] - sc * accw[r][i];
          accq[r][i] *= dS * egr[r][i];
        }
        sm.vnx[wave][r][lane] = Vn[r];
      }
    }
    lds_barrier();                               // B: Vnew halves published; Q, Sq reads done
    store_q(qnext);                                // chunk c + 1's Q: every wave is done with Q
    dma(cn, (c + 1) & 1, KD1, KW);
    if (a.s_codes) {
      uint8_t* sb = a.s_codes + ch * DK * Dv + (int64_t)dk0 * Dv + wcol + r16;
#pragma unroll
      for (int j = 0; j < MKH; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) sb[(int64_t)(16 * j + 4 * grp + i) * Dv] = (sbytes[j] >> (8 * i)) & 0xFFu;
      if (cg == g0 && hf == 0 && lane == 0) a.s_scale[ch * (Dv / a.block_v) + wcol / a.block_v] = dS;
    }
    // Vnew of all four token row tiles: tiles 0, 3 from half 0, tiles 1, 2 from
    // half 1 (selects with compile-time indices only)
    f32x4 Vt[4];
    {
      const f32x4 p0 = sm.vnx[partner][0][lane], p1 = sm.vnx[partner][1][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Vt[0][i] = hf == 0 ? Vn[0][i] : p0[i];
        Vt[1][i] = hf == 1 ? Vn[0][i] : p0[i];
        Vt[2][i] = hf == 1 ? Vn[1][i] : p1[i];
        Vt[3][i] = hf == 0 ? Vn[1][i] : p1[i];
      }
    }
    bf16x8 bVh[2], bVl[2], bDh[2], bDl[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      pack_pair_split(Vt[2 * t], Vt[2 * t + 1], bVh[t], bVl[t]);
      f32x4 d0, d1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        d0[i] = egc[2 * t][i] * Vt[2 * t][i];
        d1[i] = egc[2 * t + 1][i] * Vt[2 * t + 1][i];
      }
      pack_pair_split(d0, d1, bDh[t], bDl[t]);
    }

    // ---- 3a. O = scale (exp(gamma) dS Q Sq + P Vnew) for the own row tiles;
    //      under the lower-triangular P tile rt0 (0 or 1) needs k-step 0 only,
    //      tile rt1 (3 or 2) both
    {
      bf16* ot = sm.x1.ost[wave];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int mt = r ? rt1 : rt0;
        f32x4 acc = accq[r];
#pragma unroll
        for (int kk = 0; kk < 1 + r; ++kk) {
          const bf16x8 ph = lds_nat(B.P, 16 * mt + r16, I::R64, 32 * kk, grp);
          const bf16x8 pl = lds_nat(B.P + I::P1, 16 * mt + r16, I::R64, 32 * kk, grp);
          acc = mfma(ph, bVh[kk], acc);
          acc = mfma(pl, bVh[kk], acc);
          acc = mfma(ph, bVl[kk], acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) ot[(16 * r + 4 * grp + i) * 16 + r16] = to_bf16(a.scale * acc[i]);
      }
      // one 16-byte row piece of the [32 x 16] tile per lane
      const int row = lane >> 1, half = lane & 1;
      const int tok = 16 * ((row >> 4) ? rt1 : rt0) + (row & 15);
      const u32x4 v = *reinterpret_cast<const u32x4*>(&ot[row * 16 + 8 * half]);
      if (tok < nc) {
        bf16* op = reinterpret_cast<bf16*>(a.o) + ((int64_t)(t0 + tok) * Hv + h) * Dv + wcol + 8 * half;
        *reinterpret_cast<u32x4*>(op) = v;
      }
    }
    // ---- 3b. S = exp(gamma_n) Sq + K^T (exp(gamma_n - gamma) Vnew), own state rows
    {
      const float sdec = egC * dS;
#pragma unroll
      for (int j = 0; j < MKH; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[j][i] *= sdec;
      bf16x8 kop[2][MKH];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < MKH; ++j) kop[t][j] = lds_nat(B.Kt, dk0 + 16 * j + r16, I::R64, 32 * t, grp);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < MKH; ++j) {
          S[j] = mfma(kop[t][j], bDh[t], S[j]);
          S[j] = mfma(kop[t][j], bDl[t], S[j]);
        }
      float m = 0.f;
#pragma unroll
      for (int j = 0; j < MKH; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(S[j][i]));
      m = wave_max(m);
      if (lane == 0) sm.red[(c + 1) & 1][wave] = m;
    }
    vm_drain();                                   // this wave's staging of chunk c + 1 landed
    lds_barrier();                                 // C
#pragma unroll
    for (int r = 0; r < 2; ++r) Ucur[r] = Unext[r];
    dWcur = dWnext;
#pragma unroll
    for (int p = 0; p < QPT; ++p) qnext[p] = qreg[p];
  }
  store_ht();
}

}  // namespace

template <int DK, int SF, int WF>
static hipError_t launch_pair_one(const FwdConfig& cfg, const FwdKernelArgs& a, hipStream_t s) {
  const int num_heads = cfg.N * cfg.Hv, nvb = cfg.Dv / 64;
  const int64_t nblk = (int64_t)nvb * 8 * ((num_heads + 7) / 8);
  hipLaunchKernelGGL((gdn_state_pair_kernel<DK, SF, WF>), dim3((unsigned)nblk), dim3(NT), 0, s, a,
                     cfg.N, num_heads);
  return hipGetLastError();
}

template <int DK>
static hipError_t launch_pair_dk(const FwdConfig& cfg, const FwdKernelArgs& a, hipStream_t s) {
#define GDN_CASE(SFv, WFv) \
  if (cfg.state_fmt == SFv && cfg.w_fmt == WFv) return launch_pair_one<DK, SFv, WFv>(cfg, a, s);
  GDN_CASE(1, 1) GDN_CASE(1, 2) GDN_CASE(2, 1) GDN_CASE(2, 2)
#undef GDN_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_state_pair(const FwdConfig& cfg, const FwdKernelArgs& a, hipStream_t s) {
  if (cfg.Dk == 128) return launch_pair_dk<128>(cfg, a, s);
  if (cfg.Dk == 64) return launch_pair_dk<64>(cfg, a, s);
  return hipErrorInvalidValue;
}

}  // namespace gdn
