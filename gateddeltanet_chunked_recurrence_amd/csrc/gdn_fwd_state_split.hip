// Forward state recurrence with both QDQ sites on ("[1/4] GDN state/W QAT
// foundation", "What does this PR do?"; "[2/4] GDN/KDA decode QAT with INT8
// recurrent state", "What does this PR do?": per-head [Dk, block_v] state
// scales). One 12-wave workgroup per (sequence, value head, 64-wide value
// block), in three roles, one wave of each per SIMD:
//   recurrence waves 0..3: wave w keeps columns [16 w, 16 w + 16) of the
//     state, all Dk rows, in VGPRs for the whole sequence and runs only the
//     chain the next chunk depends on:
//       Sq = QDQ_S(S);  Vnew = U - dW dS (Wc Sc);
//       S  = exp(gamma_n) Sq + K^T (exp(gamma_n - gamma) Vnew)
//   output waves 4..7: wave 4 + w forms the output of the same columns from
//     the published state codes and Vnew,
//       O = scale (exp(gamma) dS (Q Sc) + P Vnew),
//     and writes the saved state codes;
//   staging waves 8..11: copy the next chunk's operands straight from global
//     memory into LDS (global-to-LDS loads): the image block (W^q code bytes,
//     K^T, P as one fp16 plane, the gates with the W scale), the rows of q,
//     and this value block's U. They are the only waves that issue global
//     loads inside the chunk loop: a wave's load issue stalls while the CU's
//     memory pipeline is busy, so the recurrence and output waves never queue
//     behind the copies.
// Every operand of a chunk sits in one double-buffered LDS block (65 KB).
// One workgroup barrier per chunk (X, at its end). Within a chunk the output
// waves wait on LDS counters that the recurrence waves (codes, then Vnew)
// raise after their LDS writes; the counters only grow, and nothing the
// recurrence or staging waves do waits on the output waves before X, so every
// wait ends. Each wait is also bounded, and one that gives up is recorded in
// the device error word.
// The output products are computed transposed (O^T = Sc^T Q^T + Vnew^T P^T):
// the published code and Vnew fragments are then A operands as they stand, and
// a lane's accumulator holds four adjacent output columns of one token, which
// leave as one 8-byte store. Sc^T Q^T contracts over dk in natural order (Q
// rows are copied unpermuted, 16-byte pieces XOR-swizzled by row); the
// recurrence waves publish the codes in that order.
#include <hip/hip_ext.h>

#include "gdn_device.h"
#include "gdn_images.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

constexpr int NT = 768;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <int DK>
struct SplitSmem {
  using I = Img<DK>;
  // W code bytes padded to whole 64-lane copies of 16 bytes (each lane of a
  // copy writes its own 16 bytes, so the copy of the last partial piece group
  // lands in this padding, not in K^T)
  static constexpr int WBP = (I::WQ / 16 + 63) / 64 * 64 * 16;
  static constexpr int QP = DK / 8;               // 16-byte pieces of a q row
  struct Buf {                                    // all operands of one chunk
    uint8_t Wb[WBP];                              // W^q codes, one byte each, W image element order
    bf16 Kt[I::KT];
    _Float16 P[I::P1];                            // masked Q K^T, one fp16 plane
    alignas(16) float G[I::GB / 2];               // gates; [129] holds the W scale
    bf16 Q[64 * DK];                              // q rows, natural order, pieces swizzled (q_off)
    f32x4 U[4][4][64];                            // U fragments: column group, row tile, lane
  };
  Buf buf[2];
  // state code bytes in natural dk order: codes[kk][col][g] holds rows
  // 32 kk + 8 g + e (byte e) of block column col
  u32x2 codes[DK / 32][64][4];
  f32x4 vnx[4][4][64];                            // Vnew: column group, row tile, lane
  alignas(16) float red[2][4];                    // per-column-group state amax, by chunk parity
  unsigned flag[2];                               // counters raised by the recurrence: codes, Vnew
};

// Element offset of 16-byte piece j (elements 8 j .. 8 j + 7) of q row `row`
// in the Q operand: pieces XOR-swizzled by row so that the 16 rows one
// fragment read touches fall in 16 distinct bank groups.
template <int DK>
__device__ __forceinline__ int q_off(int row, int j) {
  const int sw = DK == 128 ? (row & 15) : ((row >> 1) & 7);
  return row * DK + 8 * (j ^ sw);
}

// Raises an LDS counter after this wave's earlier LDS writes. The LDS executes
// one wave's operations in issue order, so the increment lands after the data
// without a wait; the fence keeps the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void lds_signal(unsigned* flag) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (__lane_id() == 0) __hip_atomic_fetch_add(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Waits until an LDS counter reaches `target` (bounded: about 2^18 polls).
// A wait that gives up records kErrLdsWait in the device error word (one
// atomic from lane 0): the outputs of that chunk are then not valid, and the
// host finds out through gdn_device_errors instead of by silent drift.
__device__ __forceinline__ void lds_wait(unsigned* flag, unsigned target, uint32_t* err) {
  bool ok = false;
  for (int it = 0; it < (1 << 18); ++it) {
    if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) {
      ok = true;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if (!ok && __lane_id() == 0)
    __hip_atomic_fetch_or(err, kErrLdsWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Eight state codes (bytes) as bf16, exact: E4M3 codes have 4 significant
// bits and INT8 codes at most 7.
// E4M3 pairs go through the scaled fp8 -> bf16 conversion with scale 1 (exact
// for every E4M3 value, subnormals included; checked against the FP32
// conversion for all 256 codes on gfx950).
template <int SF>
__device__ __forceinline__ bf16x8 codes_bf16(u32x2 w) {
  if constexpr (SF == 1) {
    typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  } else {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] = to_bf16(static_cast<float>(static_cast<int8_t>((w.x >> (8 * e)) & 0xFFu)));
      r[4 + e] = to_bf16(static_cast<float>(static_cast<int8_t>((w.y >> (8 * e)) & 0xFFu)));
    }
    return r;
  }
}

// A-operand fragment of the W codes (row `row`, stored positions 32 kk + 8 grp
// .. + 7) from the byte copy of a W image plane: the eight code bytes.
template <int DK>
__device__ __forceinline__ u32x2 ld_wb(const uint8_t* wb, int row, int kk, int grp) {
  return *reinterpret_cast<const u32x2*>(wb + wq_off<DK>(row, 32 * kk + 8 * grp));
}

template <int DK, int SF, int WF>
__global__ void __launch_bounds__(NT, 1) __attribute__((amdgpu_waves_per_eu(3, 3)))
gdn_state_split_kernel(FwdKernelArgs a, int N, int num_heads) {
  static_assert(SF != 0 && WF != 0, "both QDQ sites on");
  using I = Img<DK>;
  using Sm = SplitSmem<DK>;
  constexpr int MK = DK / 16;                     // 16-row tiles of a state column group
  constexpr int KS = DK / 32;                     // 32-deep k-steps over dk
  // the LDS block: the image block with its W slot replaced by the padded code
  // bytes, then the q rows and U
  static_assert(sizeof(typename Sm::Buf) ==
                    Sm::WBP + 2 * (I::KT + I::P1 + I::GB) + 2 * 64 * DK + 4 * 4 * 64 * 16,
                "operand block layout");
  static_assert(sizeof(Sm) <= 160 * 1024, "LDS");
  __shared__ __align__(16) Sm sm;

  const int Hv = a.Hv, Dv = a.Dv, NVB = Dv / 64;
  // workgroup id -> (head index, value block); the blocks of a head share an XCD
  const int bid = blockIdx.x, xcd = bid & 7, r8 = bid >> 3;
  const int vb = r8 % NVB, hidx = xcd + 8 * (r8 / NVB);
  if (hidx >= num_heads) return;
  const int n = hidx / Hv, h = hidx % Hv;
  const int hk = h / (Hv / a.Hqk);
  int bos, eos;
  seq_span(a, n, bos, eos);
  const int nchunks = (eos - bos + CHUNK - 1) / CHUNK;
  const int slot0 = n + bos / CHUNK;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cg = wave & 3;                        // column group of either role
  const int lane = __lane_id(), r16 = lane & 15, grp = lane >> 4;
  const int wcol = vb * 64 + cg * 16;             // first value column of the group
  const int64_t state_base = ((int64_t)n * Hv + h) * DK * Dv;
  const int gs = a.block_v / 16;                  // column groups per scale tile
  const int g0 = (cg / gs) * gs;

  auto chunk_t0 = [&](int c) { return bos + CHUNK * c; };
  auto chunk_nc = [&](int c) { return min(CHUNK, eos - bos - CHUNK * c); };
  auto chunk_ch = [&](int c) { return (int64_t)(slot0 + c) * Hv + h; };
  // state scale of chunk c from the four published column-group maxima
  auto scale_of = [&](int c) {
    const f32x4 rv = *reinterpret_cast<const f32x4*>(&sm.red[c & 1][0]);
    float amax = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (t >= g0 && t < g0 + gs) amax = fmaxf(amax, rv[t]);
    return qdq_scale<SF>(amax);
  };

  if (wave < 4) {
    // ======================= recurrence role =======================
    __builtin_amdgcn_s_setprio(3);
    // S[j][i] = S[16 j + 4 grp + i][wcol + r16]
    f32x4 S[MK];
    if (a.h0) {
      const float* hp = a.h0 + state_base + wcol + r16;
#pragma unroll
      for (int j = 0; j < MK; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[j][i] = hp[(int64_t)(16 * j + 4 * grp + i) * Dv];
    } else {
#pragma unroll
      for (int j = 0; j < MK; ++j) S[j] = zero4();
    }
    auto store_ht = [&]() {
      if (!a.ht) return;
      float* hp = a.ht + state_base + wcol + r16;
#pragma unroll
      for (int j = 0; j < MK; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) hp[(int64_t)(16 * j + 4 * grp + i) * Dv] = S[j][i];
    };
    if (nchunks == 0) {
      store_ht();
      return;
    }
    {
      float m = 0.f;
#pragma unroll
      for (int j = 0; j < MK; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(S[j][i]));
      m = wave_max(m);
      if (lane == 0) sm.red[0][cg] = m;
    }
    if (wave == 0 && lane < 2) sm.flag[lane] = 0;
    vm_drain();
    lds_barrier();                                 // P

    for (int c = 0; c < nchunks; ++c) {
      const typename Sm::Buf& B = sm.buf[c & 1];
      // operands read ahead of their products: the W fragments here, over the
      // QDQ; the K^T fragments after W Sq is issued, over Vnew
      // (two k-steps ahead: three waves per SIMD leave 168 VGPRs per wave)
      // W fragments stay code bytes until their product (8 bytes per read)
      u32x2 op[2][4];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) op[kk][mt] = ld_wb<DK>(B.Wb, 16 * mt + r16, kk, grp);
      const float dS = scale_of(c);

      // ---- QDQ; code bytes to LDS; Sq as the B operand of W Sq
      uint32_t sb[MK];
      {
        const float rS = 1.0f / dS;
#pragma unroll
        for (int j = 0; j < MK; ++j) {
          const float x[4] = {S[j][0], S[j][1], S[j][2], S[j][3]};
          float cq[4];
          quant4<SF>(x, rS, cq, sb[j]);
#pragma unroll
          for (int i = 0; i < 4; ++i) S[j][i] = cq[i];
        }
      }
      // rows 16 j + 4 grp + i are natural-order bytes 4 (grp & 1) + i of
      // piece 2 (j & 1) + (grp >> 1) of k-step j >> 1
      {
        uint8_t* cb = reinterpret_cast<uint8_t*>(&sm.codes[0][16 * cg + r16][0]);
#pragma unroll
        for (int j = 0; j < MK; ++j)
          *reinterpret_cast<uint32_t*>(cb + (j >> 1) * (64 * 4 * 8) + 8 * (2 * (j & 1) + (grp >> 1)) +
                                       4 * (grp & 1)) = sb[j];
      }
      lds_signal(&sm.flag[0]);

      // ---- W Sq over the four token row tiles
      f32x4 accw[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) accw[mt] = zero4();
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const bf16x8 b = pack_pair(S[2 * kk], S[2 * kk + 1]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) accw[mt] = mfma(codes_bf16<WF>(op[kk & 1][mt]), b, accw[mt]);
        if (kk + 2 < KS)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) op[kk & 1][mt] = ld_wb<DK>(B.Wb, 16 * mt + r16, kk + 2, grp);
      }
      bf16x8 kop[MK];                              // token k-step 0; k-step 1 reloads in place
#pragma unroll
      for (int j = 0; j < MK; ++j) kop[j] = ld_r64(B.Kt, 16 * j + r16, 0, grp);
      f32x4 Vn[4];
      {
        const float sc = B.G[129] * dS;            // dW dS
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const f32x4 u = B.U[cg][mt][lane];
#pragma unroll
          for (int i = 0; i < 4; ++i) Vn[mt][i] = u[i] - sc * accw[mt][i];
          sm.vnx[cg][mt][lane] = Vn[mt];
        }
      }
      const f32x4 e0[2] = {*reinterpret_cast<const f32x4*>(&B.G[64 + 4 * grp]),
                           *reinterpret_cast<const f32x4*>(&B.G[96 + 4 * grp])};
      const f32x4 e1[2] = {*reinterpret_cast<const f32x4*>(&B.G[80 + 4 * grp]),
                           *reinterpret_cast<const f32x4*>(&B.G[112 + 4 * grp])};
      const float sdec = B.G[128] * dS;
      lds_signal(&sm.flag[1]);

      // ---- S = exp(gamma_n) Sq + K^T (exp(gamma_n - gamma) Vnew)
      bf16x8 bDh[2], bDl[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x4 d0, d1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          d0[i] = e0[t][i] * Vn[2 * t][i];
          d1[i] = e1[t][i] * Vn[2 * t + 1][i];
        }
        pack_pair_split(d0, d1, bDh[t], bDl[t]);
      }
#pragma unroll
      for (int j = 0; j < MK; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[j][i] *= sdec;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int j = 0; j < MK; ++j) S[j] = mfma(kop[j], bDh[t], S[j]);
#pragma unroll
        for (int j = 0; j < MK; ++j) {
          S[j] = mfma(kop[j], bDl[t], S[j]);
          if (t == 0) kop[j] = ld_r64(B.Kt, 16 * j + r16, 32, grp);
        }
      }
      {
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < MK; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(S[j][i]));
        m = wave_max(m);
        if (lane == 0) sm.red[(c + 1) & 1][cg] = m;
      }
      lds_barrier();                               // X
    }
    store_ht();
  } else if (wave < 8) {
    // ========================= output role =========================
    if (nchunks == 0) return;
    __builtin_amdgcn_s_setprio(3);
    constexpr int CPL = DK / 64;                   // 4x4 code blocks per lane
    lds_barrier();                                 // P
    for (int c = 0; c < nchunks; ++c) {
      const typename Sm::Buf& B = sm.buf[c & 1];
      const int t0 = chunk_t0(c), nc = chunk_nc(c);
      const int64_t ch = chunk_ch(c);
      lds_wait(&sm.flag[0], 4u * (c + 1), a.err);        // this chunk's codes
      const float dS = scale_of(c);
      // ---- O^T = dS exp(gamma) (Sc^T Q^T) + Vnew^T P^T, four token row tiles
      f32x4 acc[4];
      {
        bf16x8 aS[KS];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) aS[kk] = codes_bf16<SF>(sm.codes[kk][16 * cg + r16][grp]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          acc[mt] = zero4();
#pragma unroll
          for (int kk = 0; kk < KS; ++kk)
            acc[mt] = mfma(aS[kk], *reinterpret_cast<const bf16x8*>(
                                       &B.Q[q_off<DK>(16 * mt + r16, 4 * kk + grp)]), acc[mt]);
          const float f = dS * B.G[16 * mt + r16];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mt][i] *= f;
        }
      }
      lds_wait(&sm.flag[1], 4u * (c + 1), a.err);        // this chunk's Vnew
      {
        // P is one fp16 plane; Vnew enters as fp16 hi + lo (22 significant bits)
        f16x8 aVh[2], aVl[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const f32x4 v0 = sm.vnx[cg][2 * t][lane], v1 = sm.vnx[cg][2 * t + 1][lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            aVh[t][e] = (_Float16)v0[e];
            aVh[t][4 + e] = (_Float16)v1[e];
            aVl[t][e] = (_Float16)(v0[e] - (float)aVh[t][e]);
            aVl[t][4 + e] = (_Float16)(v1[e] - (float)aVh[t][4 + e]);
          }
        }
        // under the lower-triangular P, row tiles 0 and 1 need k-step 0 only
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int kk = 0; kk <= (mt >> 1); ++kk) {
            const f16x8 p = *reinterpret_cast<const f16x8*>(B.P + r64_off(16 * mt + r16, 32 * kk + 8 * grp));
            acc[mt] = mfma(aVh[kk], p, acc[mt]);
            acc[mt] = mfma(aVl[kk], p, acc[mt]);
          }
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int tok = 16 * mt + r16;
        bf16x4 o4;
#pragma unroll
        for (int i = 0; i < 4; ++i) o4[i] = to_bf16(a.scale * acc[mt][i]);
        if (tok < nc) {
          bf16* op = reinterpret_cast<bf16*>(a.o) + ((int64_t)(t0 + tok) * Hv + h) * Dv + wcol + 4 * grp;
          *reinterpret_cast<u32x2*>(op) = __builtin_bit_cast(u32x2, o4);
        }
      }
      // ---- saved state codes: 4x4 byte blocks (rows row0 + i, columns 4 q..4 q + 3)
      if (a.s_codes) {
        uint8_t* sbase = a.s_codes + ch * DK * Dv + wcol;
#pragma unroll
        for (int p = 0; p < CPL; ++p) {
          const int cb = lane + 64 * p, q = cb & 3, g = (cb >> 2) & 3, hh = (cb >> 4) & 1, jj = cb >> 5;
          const int row0 = 32 * jj + 8 * g + 4 * hh;
          uint32_t w[4];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const u32x2 v = sm.codes[jj][16 * cg + 4 * q + m][g];
            w[m] = hh ? v.y : v.x;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i)
            *reinterpret_cast<uint32_t*>(sbase + (int64_t)(row0 + i) * Dv + 4 * q) =
                ((w[0] >> (8 * i)) & 0xFFu) | (((w[1] >> (8 * i)) & 0xFFu) << 8) |
                (((w[2] >> (8 * i)) & 0xFFu) << 16) | (((w[3] >> (8 * i)) & 0xFFu) << 24);
        }
        if (cg == g0 && lane == 0) a.s_scale[ch * (Dv / a.block_v) + wcol / a.block_v] = dS;
      }
      lds_barrier();                               // X
    }
  } else {
    // ========================= staging role =========================
    if (nchunks == 0) return;
    __builtin_amdgcn_s_setprio(1);
    // One chunk's copies, as whole 64-lane global-to-LDS loads of 16 bytes
    // (each lane's 16 bytes land at LDS base + 16 lane): the W code bytes (the
    // first WQ bytes of the image block's W slot; lanes past them read the
    // last piece into the padding), K^T, P and the gates (after the W slot),
    // the q rows (source pieces permuted so the LDS pieces come out
    // swizzled, rows past the chunk end repeat its last row), and U.
    constexpr int WOFF = I::WQ / 8;               // 16-byte pieces of the W slot
    constexpr int NWB = I::WQ / 16;               // ... of the W code bytes
    constexpr int NI1 = Sm::WBP / 16 / 64;        // wave loads of the codes
    constexpr int NI2 = (I::KT + I::P1 + I::GB) / 8 / 64;   // ... of K^T, P and the gates
    constexpr int NI3 = 64 * DK / 8 / 64;         // ... of the q rows
    constexpr int NI4 = 4 * 4 * 64 * 16 / 16 / 64;           // ... of U
    constexpr int NI = NI1 + NI2 + NI3 + NI4;
    constexpr int KW = (NI + 3) / 4;              // ... per staging wave
    static_assert((I::KT + I::P1 + I::GB) % 512 == 0 && NI1 * 64 >= NWB, "whole wave loads");
    static_assert(offsetof(typename Sm::Buf, Kt) == Sm::WBP &&
                  offsetof(typename Sm::Buf, Q) == Sm::WBP + 2 * (I::KT + I::P1 + I::GB) &&
                  offsetof(typename Sm::Buf, U) == offsetof(typename Sm::Buf, Q) + 2 * 64 * DK,
                  "the copies fill the buffer back to back");
    // Each lane's source offset of each of its KW copies is fixed for a full
    // chunk (bytes from a wave-uniform base: the image block, this chunk's
    // first q row of the head, or this value block's U), so a copy costs a
    // scalar base update and no vector address arithmetic.
    const char* qbase = reinterpret_cast<const char*>(a.q) + (int64_t)hk * DK * 2;
    const int64_t qrow = (int64_t)a.Hqk * DK * 2;   // bytes between consecutive tokens' q rows
    int off[KW];
#pragma unroll
    for (int k = 0; k < KW; ++k) {
      const int j = min(cg + 4 * k, NI - 1);       // a repeated last load rewrites the same bytes
      if (j < NI1) {
        off[k] = 16 * min(64 * j + lane, NWB - 1);
      } else if (j < NI1 + NI2) {
        off[k] = 16 * (WOFF + 64 * (j - NI1) + lane);
      } else if (j < NI1 + NI2 + NI3) {
        const int pc = 64 * (j - NI1 - NI2) + lane, row = pc / Sm::QP, jp = pc % Sm::QP;
        const int sw = DK == 128 ? (row & 15) : ((row >> 1) & 7);
        off[k] = (int)(row * qrow) + 16 * (jp ^ sw);
      } else {
        off[k] = 16 * (64 * (j - NI1 - NI2 - NI3) + lane);
      }
    }
    // chunks the concurrent prep kernel is still producing: wait for their
    // flags (bounded to about 2^27 clocks per chunk, some 60 ms: on give-up
    // the error flag is set and the copies go on)
    auto wait_ready = [&](int c) {
      if (!a.flags) return;
      uint32_t* f = a.flags + chunk_ch(c);
      const uint64_t t0 = __builtin_amdgcn_s_memtime();
      while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
        if (__builtin_amdgcn_s_memtime() - t0 > (1ull << 27)) {
          if (lane == 0) __hip_atomic_fetch_or(a.err, kErrFlagWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    };
    auto dma = [&](int c, int b) {
      wait_ready(c);
      const int64_t ch = chunk_ch(c);
      const char* img = reinterpret_cast<const char*>(a.ws_img + ch * I::template img<1>());
      const char* u = reinterpret_cast<const char*>(a.ws_u + u_off(ch, NVB, vb, 0, 0, 0));
      const int t0 = chunk_t0(c), nc = chunk_nc(c);
      const char* q0 = qbase + (int64_t)t0 * qrow;
      uint4* dst = reinterpret_cast<uint4*>(sm.buf[b].Wb);
#pragma unroll
      for (int k = 0; k < KW; ++k) {
        const int j = min(cg + 4 * k, NI - 1);
        const char* src;
        if (j < NI1 + NI2) {
          src = img + off[k];
        } else if (j < NI1 + NI2 + NI3) {
          if (nc == CHUNK) {
            src = q0 + off[k];
          } else {                                 // the last, partial chunk: rows past its end repeat its last row
            const int pc = 64 * (j - NI1 - NI2) + lane, row = pc / Sm::QP, jp = pc % Sm::QP;
            const int sw = DK == 128 ? (row & 15) : ((row >> 1) & 7);
            src = q0 + min(row, nc - 1) * qrow + 16 * (jp ^ sw);
          }
        } else {
          src = u + off[k];
        }
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4*>(src), dst + 64 * j, 16, 0, 0);
      }
    };
    dma(0, 0);
    vm_drain();
    lds_barrier();                                 // P
    for (int c = 0; c < nchunks; ++c) {
      dma(min(c + 1, nchunks - 1), (c + 1) & 1);
      vm_drain();                                  // next chunk's copies landed
      lds_barrier();                               // X
    }
  }
}

}  // namespace

template <int DK, int SF, int WF>
static hipError_t launch_split_one(const FwdConfig& cfg, const FwdKernelArgs& a, hipStream_t s,
                                   hipEvent_t stop) {
  const int num_heads = cfg.N * cfg.Hv, nvb = cfg.Dv / 64;
  const int64_t nblk = (int64_t)nvb * 8 * ((num_heads + 7) / 8);
  if (stop)
    hipExtLaunchKernelGGL((gdn_state_split_kernel<DK, SF, WF>), dim3((unsigned)nblk), dim3(NT), 0, s,
                          nullptr, stop, 0, a, cfg.N, num_heads);
  else
    hipLaunchKernelGGL((gdn_state_split_kernel<DK, SF, WF>), dim3((unsigned)nblk), dim3(NT), 0, s, a,
                       cfg.N, num_heads);
  return hipGetLastError();
}

template <int DK>
static hipError_t launch_split_dk(const FwdConfig& cfg, const FwdKernelArgs& a, hipStream_t s,
                                  hipEvent_t stop) {
#define GDN_CASE(SFv, WFv) \
  if (cfg.state_fmt == SFv && cfg.w_fmt == WFv) return launch_split_one<DK, SFv, WFv>(cfg, a, s, stop);
  GDN_CASE(1, 1) GDN_CASE(1, 2) GDN_CASE(2, 1) GDN_CASE(2, 2)
#undef GDN_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_state_split(const FwdConfig& cfg, const FwdKernelArgs& a, hipStream_t s,
                                  hipEvent_t stop) {
  if (!a.w_img_bytes) return hipErrorInvalidValue;   // its images carry W as code bytes
  if (cfg.Dk == 128) return launch_split_dk<128>(cfg, a, s, stop);
  if (cfg.Dk == 64) return launch_split_dk<64>(cfg, a, s, stop);
  return hipErrorInvalidValue;
}

}  // namespace gdn
