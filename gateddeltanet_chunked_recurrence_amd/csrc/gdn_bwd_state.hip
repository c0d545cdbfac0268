// Backward, the reverse state recurrence of the chunked gated delta rule for
// bf16 inputs, as two kernels ("[1/4] GDN state/W QAT foundation", "What does
// this PR do?": identity STE at both QDQ sites, so the forward's Sq and Wq are
// the values in every product and pass gradients unchanged).
//
// With dS' the gradient of the state after a chunk (dht after the last one),
// reverse mode through one chunk of the forward (gdn_fwd_state.hip) gives
//   dVnew = A1 + diag(e^(gamma_n - gamma)) K dS'
//   dS    = e^gamma_n dS' + A2 - Wq^T dVnew
// where the state-independent terms are
//   A1 = scale P^T dO,                 P = (Q K^T) * Gam (i >= j)
//   A2 = scale (diag(e^gamma) Q)^T dO.
//
// bwd_img_kernel, one workgroup per (chunk, value head), computes A1 and A2
// with bf16 MFMA (bf16 inputs exact, FP32 factors as hi + lo pairs) and writes
// the recurrence's other operands in the layout its LDS keeps them:
//   K image    [64][Dk] bf16, the forward's W image layout (pperm along dk)
//   W^T image  [Dk][72] bf16, the transposed W of the products, pperm along
//              tokens: the Wq codes (one plane; the scale is applied to the
//              other factor) or, with W QDQ off, W as hi + lo (two planes)
//   gates      256 FP32: e^(gamma_n - gamma_i) at [i] (0 past the chunk end),
//              e^gamma_n at [64], minus the W scale at [65]
// A1 and A2 are stored in fragment order (frag_off), so the recurrence loads
// its accumulator tiles with 16-byte loads.
//
// bwd_state_kernel, one workgroup per (sequence, value head, 64-wide value
// block), runs the chunks in reverse with dS in registers (wave w holds value
// columns 16w..16w+15 in accumulator layout; the columns are independent, as
// the backward has no QDQ). It stores dS' and dVnew of every chunk, fragment
// order, for the chunk-local gradients, and dh0 at the end.
//
// Transposes are transposing LDS reads (ds_read_b64_tr_b16): a row-major bf16
// tile read by columns is the tile in accumulator layout, and two such reads
// 16 rows apart are an operand with the tokens as contraction index.
#include <hip/hip_ext.h>

#include "gdn_device.h"
#include "gdn_images.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

constexpr int NT = 256;
constexpr float LOG2E = 1.4426950408889634f;

// Image block of one (slot, head) for the reverse recurrence.
template <int DK>
struct BImg {
  using I = Img<DK>;
  static constexpr int KI = I::WQ;                 // K image [64][RS]
  static constexpr int WT = DK * I::R64;           // one W^T plane [DK][72]
  static constexpr int GB = 512;                   // gate block, 256 FP32
  static constexpr int size(int nw) { return KI + nw * WT + GB; }
  static constexpr int g_at(int nw) { return KI + nw * WT; }
};

// Accumulator-layout tile of rows row0..row0+15, columns 16 ct..16 ct + 15 of
// a bf16 row-major LDS matrix (row stride ld), by a transposing LDS read.
__device__ __forceinline__ f32x4 tile_of(const bf16* m, int ld, int row0, int ct, int r16, int grp) {
  return lds_tile(m, ld, row0, 16 * ct, r16, grp);
}

template <int DK, int DV, int NW>
struct ImgSmem {
  static constexpr int LD = DK + 8;                // padded row strides (bf16)
  static constexpr int LDO = DV + 8;
  static constexpr int QB = 64 * LD * 2;           // bytes of the Q rows
  static constexpr int OB = 2 * (DV / 16) * 64 * 16;   // bytes of the dO operands
  union {
    struct {
      bf16 Kn[64 * LD];
      union {                                      // Q rows, then the dO operands
        bf16 Qn[64 * LD];
        bf16x8 dOB[2 * (DV / 16) * 64];            // [kk][value tile][lane]
        char raw[QB > OB ? QB : OB];
      } u;
    };
    // one W^T image plane [DK][72], staged once K's image copy and the
    // products are done with K and the dO operands (one W plane only)
    bf16 wt[NW == 1 ? DK * 72 : 8];
  };
  bf16 Wn[NW][64 * LD];                            // W codes, or W hi and lo
  bf16 dOn[64 * LDO];
  float gam2[64], eg[64];
};

// ---------------------------------------------------------------- bwd_img
template <int DK, int DV, int WF>
__global__ void __launch_bounds__(NT, 2) bwd_img_kernel(BwdKernelArgs a, int N) {
  constexpr int NW = WF == 0 ? 2 : 1;
  constexpr int MK = DK / 16, DPW = MK / 4;        // dk tiles, dk tiles per wave
  constexpr int NVT = DV / 16, nvb = DV / 64;
  using S = ImgSmem<DK, DV, NW>;
  using I = Img<DK>;
  using BI = BImg<DK>;
  constexpr int LD = S::LD, LDO = S::LDO;
  __shared__ __align__(16) S sm;
  const FwdKernelArgs& f = a.f;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = __lane_id();
  const int tid = wave * 64 + lane, r16 = lane & 15, grp = lane >> 4;
  const int Hv = f.Hv, Hqk = f.Hqk, Dv = DV;
  int slot = blockIdx.x, h = blockIdx.y;
  if (a.rev_maxc > 0) {
    // for the overlapped backward: item i in reverse chunk-major order, chunk
    // rev_maxc - 1 - i / (N Hv) of every (sequence, head) before the one below
    const int nh = N * Hv, i = a.rev_lo + blockIdx.x, cr = i / nh, r = i - cr * nh, n = r / Hv;
    h = r - n * Hv;
    slot = n + (n * f.T) / CHUNK + (a.rev_maxc - 1 - cr);
  }
  const bool coh = a.flags != nullptr;             // device-scope stores, then the item's flag
  const Chunk ch = locate_slot(slot, f.cu_seqlens, N, f.T, f.prefix_len);
  if (!ch.valid) return;
  const int hk = h / (Hv / Hqk), t0 = ch.t0, nc = ch.nc;
  const int64_t chb = (int64_t)slot * Hv + h;
  bf16* img = a.ws_bimg + chb * BI::size(NW);

  // ---- rows of K, Q, dO and W into LDS (rows past the chunk end are zero).
  // Every load is issued before the first LDS write, so the item pays one
  // memory latency, not one per loop trip.
  {
    const bf16* kg = reinterpret_cast<const bf16*>(f.k);
    const bf16* qg = reinterpret_cast<const bf16*>(f.q);
    const bf16* dog = reinterpret_cast<const bf16*>(a.dout);
    constexpr int NKQ = 64 * DK / 8 / NT, NDO = 64 * DV / 8 / NT;
    constexpr int WPR = WF != 0 ? DK / 16 : DK / 4;   // 16-byte pieces per W row
    constexpr int NWL = 64 * WPR / NT;
    static_assert(NKQ * NT == 64 * DK / 8 && NDO * NT == 64 * DV / 8 && NWL * NT == 64 * WPR,
                  "whole trips");
    u32x4 kv[NKQ], qv[NKQ], dv[NDO], wv[NWL];
#pragma unroll
    for (int p = 0; p < NKQ; ++p) {
      const int e = tid + NT * p, row = e / (DK / 8), c8 = e % (DK / 8);
      const int64_t off = ((int64_t)(t0 + min(row, nc - 1)) * Hqk + hk) * DK + 8 * c8;
      kv[p] = *reinterpret_cast<const u32x4*>(kg + off);
      qv[p] = *reinterpret_cast<const u32x4*>(qg + off);
    }
#pragma unroll
    for (int p = 0; p < NDO; ++p) {
      const int e = tid + NT * p, row = e / (DV / 8), c8 = e % (DV / 8);
      dv[p] = *reinterpret_cast<const u32x4*>(dog + ((int64_t)(t0 + min(row, nc - 1)) * Hv + h) * Dv + 8 * c8);
    }
#pragma unroll
    for (int p = 0; p < NWL; ++p) {
      const int e = tid + NT * p, row = e / WPR, cw = e % WPR;
      const int64_t rb = ((int64_t)(t0 + min(row, nc - 1)) * Hv + h) * DK;
      if constexpr (WF != 0) wv[p] = *reinterpret_cast<const u32x4*>(f.w_codes + rb + 16 * cw);
      else wv[p] = *reinterpret_cast<const u32x4*>(a.ws_W + rb + 4 * cw);
    }
#pragma unroll
    for (int p = 0; p < NKQ; ++p) {
      const int e = tid + NT * p, row = e / (DK / 8), c8 = e % (DK / 8);
      const bool z = row >= nc;
      *reinterpret_cast<u32x4*>(&sm.Kn[row * LD + 8 * c8]) = z ? u32x4{0u, 0u, 0u, 0u} : kv[p];
      *reinterpret_cast<u32x4*>(&sm.u.Qn[row * LD + 8 * c8]) = z ? u32x4{0u, 0u, 0u, 0u} : qv[p];
    }
#pragma unroll
    for (int p = 0; p < NDO; ++p) {
      const int e = tid + NT * p, row = e / (DV / 8), c8 = e % (DV / 8);
      *reinterpret_cast<u32x4*>(&sm.dOn[row * LDO + 8 * c8]) = row >= nc ? u32x4{0u, 0u, 0u, 0u} : dv[p];
    }
#pragma unroll
    for (int p = 0; p < NWL; ++p) {
      const int e = tid + NT * p, row = e / WPR, cw = e % WPR;
      if constexpr (WF != 0) {
        // codes (exact in bf16: E4M3 values and integers up to 127)
        bf16x8 o[2];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const uint32_t word = wv[p][j >> 2];
          float cv;
          if constexpr (WF == 1) {
            cv = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word >> (8 * (j & 3))), 0);
          } else {
            cv = static_cast<float>(static_cast<int8_t>((word >> (8 * (j & 3))) & 0xFFu));
          }
          o[j >> 3][j & 7] = to_bf16(row < nc ? cv : 0.f);
        }
        *reinterpret_cast<bf16x8*>(&sm.Wn[0][row * LD + 16 * cw]) = o[0];
        *reinterpret_cast<bf16x8*>(&sm.Wn[0][row * LD + 16 * cw + 8]) = o[1];
      } else {
        f32x4 w = __builtin_bit_cast(f32x4, wv[p]);
        if (row >= nc) w = zero4();
        bf16x4 hi, lo;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16 hj, lj;
          split2(w[j], hj, lj);
          hi[j] = hj;
          lo[j] = lj;
        }
        *reinterpret_cast<bf16x4*>(&sm.Wn[0][row * LD + 4 * cw]) = hi;
        *reinterpret_cast<bf16x4*>(&sm.Wn[NW - 1][row * LD + 4 * cw]) = lo;
      }
    }
  }
  // ---- gates (wave 0): LDS copies for this kernel, the gate block for the recurrence
  if (wave == 0) {
    const bool valid = lane < nc;
    const int64_t gi = (int64_t)(t0 + min(lane, nc - 1)) * Hv + h;
    const float g2 = wave_incl_scan(valid ? f.g[gi] * LOG2E : 0.f);
    const float g2n = read_lane(g2, nc - 1);
    sm.gam2[lane] = g2;
    sm.eg[lane] = fexp2(g2);
    float* G = reinterpret_cast<float*>(img + BI::g_at(NW));
    st_out(G + lane, valid ? fexp2(g2n - g2) : 0.f, coh);
    if (lane == 0) {
      st_out(G + 64, fexp2(g2n), coh);
      st_out(G + 65, WF != 0 ? -f.w_scale[chb] : -1.f, coh);
    }
  }
  __syncthreads();


  // ---- (e^gamma Q)^T operands for this wave's dk tiles: hi + lo
  bf16x8 aQh[DPW][2], aQl[DPW][2];
#pragma unroll
  for (int d = 0; d < DPW; ++d) {
    const int dt = DPW * wave + d;
    f32x4 cq[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      cq[it] = tile_of(sm.u.Qn, LD, 16 * it, dt, r16, grp);
      const f32x4 e = *reinterpret_cast<const f32x4*>(&sm.eg[16 * it + 4 * grp]);
#pragma unroll
      for (int q = 0; q < 4; ++q) cq[it][q] *= e[q];
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) pack_pair_split(cq[2 * kk], cq[2 * kk + 1], aQh[d][kk], aQl[d][kk]);
  }

  // ---- P^T operands for key tile jt = wave: P = (Q K^T) * Gam, i >= j
  const int jt = wave;
  bf16x8 aPh[2], aPl[2];
  {
    f32x4 pt[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      pt[it] = zero4();
      if (it < jt) continue;
#pragma unroll
      for (int kq = 0; kq < DK / 32; ++kq)
        pt[it] = mfma(lds_nat(sm.u.Qn, 16 * it + r16, LD, 32 * kq, grp),
                      lds_nat(sm.Kn, 16 * jt + r16, LD, 32 * kq, grp), pt[it]);
      const int j = 16 * jt + r16;
      const float gj = sm.gam2[j];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 16 * it + 4 * grp + q;
        pt[it][q] = i >= j ? pt[it][q] * fexp2(sm.gam2[i] - gj) : 0.f;
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) pack_pair_split(pt[2 * kk], pt[2 * kk + 1], aPh[kk], aPl[kk]);
  }
  __syncthreads();                                 // Q rows read: their space takes the dO operands
  // ---- dO operands, tokens as contraction index (shared by A1 and A2)
  for (int fi = wave; fi < 2 * NVT; fi += 4) {
    const int kk = fi & 1, vt = fi >> 1;
    sm.u.dOB[(kk * NVT + vt) * 64 + lane] = lds_col8(sm.dOn, LDO, 32 * kk, 16 * vt, r16, grp);
  }

  __syncthreads();                                 // dO operands complete

  const float scale = f.scale;
  float* a1b = a.ws_a1 + frag_off(chb, nvb, 0, 0, 4, 0, 0);      // this item's A1 and A2 blocks
  float* a2b = a.ws_a2 + frag_off(chb, nvb, 0, 0, MK, 0, 0);
  // ---- A1 = scale P^T dO, rows of key tile jt
  for (int vt = 0; vt < NVT; ++vt) {
    f32x4 acc = zero4();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      if (2 * kk + 1 < jt) continue;               // both query tiles above the diagonal
      const bf16x8 b = sm.u.dOB[(kk * NVT + vt) * 64 + lane];
      acc = mfma(aPh[kk], b, acc);
      acc = mfma(aPl[kk], b, acc);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] *= scale;
    st_out16(a1b, 4 * (int)frag_off(0, nvb, vt >> 2, vt & 3, 4, jt, lane), __builtin_bit_cast(u32x4, acc),
             coh);
  }
  // ---- A2 = scale (e^gamma Q)^T dO, this wave's dk tiles
#pragma unroll
  for (int d = 0; d < DPW; ++d) {
    const int dt = DPW * wave + d;
    for (int vt = 0; vt < NVT; ++vt) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 b = sm.u.dOB[(kk * NVT + vt) * 64 + lane];
        acc = mfma(aQh[d][kk], b, acc);
        acc = mfma(aQl[d][kk], b, acc);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] *= scale;
      st_out16(a2b, 4 * (int)frag_off(0, nvb, vt >> 2, vt & 3, MK, dt, lane),
               __builtin_bit_cast(u32x4, acc), coh);
    }
  }
  // ---- K image: pperm along dk, 16-byte chunks swizzled by row
  for (int p = tid; p < 64 * DK / 8; p += NT) {
    const int row = p / (DK / 8), cs = p % (DK / 8), b = cs >> 2, g4 = cs & 3;
    const uint2 lo = *reinterpret_cast<const uint2*>(&sm.Kn[row * LD + 32 * b + 4 * g4]);
    const uint2 hi = *reinterpret_cast<const uint2*>(&sm.Kn[row * LD + 32 * b + 16 + 4 * g4]);
    st_out16(img, 2 * (row * I::RS + ((cs ^ (row & I::SWZ)) << 3)), u32x4{lo.x, lo.y, hi.x, hi.y}, coh);
  }
  // ---- W^T image: dk rows, tokens paired along the row. With one W plane it
  // is staged in LDS in the image's own layout and copied out as whole
  // 16-byte pieces (a wave's store covers whole lines; the fragments alone
  // cover 64 of a row's 144 bytes, which beside the reverse recurrence costs
  // more as device-scope write-through stores)
  if constexpr (NW == 1) {
    static_assert(DK * 72 * 2 <= sizeof(sm.Kn) + sizeof(sm.u) && I::R64 == 72, "W^T staging");
    __syncthreads();                               // K and the dO operands are dead
    for (int fi = wave; fi < 2 * MK; fi += 4) {
      const int dt = fi >> 1, kk = fi & 1;
      *reinterpret_cast<bf16x8*>(&sm.wt[(16 * dt + r16) * I::R64 + 32 * kk + 8 * grp]) =
          lds_col8(sm.Wn[0], LD, 32 * kk, 16 * dt, r16, grp);
    }
    __syncthreads();
    constexpr int NPW = BI::WT / 8;                // 16-byte pieces of the plane
    const u32x4* src = reinterpret_cast<const u32x4*>(sm.wt);
    for (int e = tid; e < NPW; e += NT) st_out16(img, 2 * BI::KI + 16 * e, src[e], coh);
  } else {
    for (int fi = wave; fi < 2 * MK; fi += 4) {
      const int dt = fi >> 1, kk = fi & 1;
#pragma unroll
      for (int pl = 0; pl < NW; ++pl) {
        st_out16(img, 2 * (BI::KI + pl * BI::WT + (16 * dt + r16) * I::R64 + 32 * kk + 8 * grp),
                 __builtin_bit_cast(u32x4, lds_col8(sm.Wn[pl], LD, 32 * kk, 16 * dt, r16, grp)), coh);
      }
    }
  }
  if (coh) {
    // every wave's stores of this item have reached the device's coherence
    // point before the one flag store
    vm_drain();
    __syncthreads();
    if (tid == 0) __hip_atomic_store(a.flags + chb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------- bwd_state
// WG waves per workgroup, each owning 16 value columns, plus one staging wave:
// the columns are independent here, so a (sequence, head) can spread over
// several compute units, which share its image block through the XCD's L2. A
// chunk step moves the image block plus 28 KB per column wave through the
// compute unit's vector memory path, which bounds the step when four waves
// share one. The image copies are issued by the staging wave alone: issuing
// them stalls the issuing wave while the memory path is busy, and the column
// waves carry the recurrence.
template <int DK, int NW, int WG>
__global__ void __launch_bounds__(64 * (WG + 1), 1) bwd_state_kernel(BwdKernelArgs a, int N, int num_heads) {
  using BI = BImg<DK>;
  using I = Img<DK>;
  constexpr int MK = DK / 16;
  constexpr int SZ = BI::size(NW);
  static_assert((SZ / 8) % 64 == 0, "image block is a whole number of wave loads");
  constexpr int NINS = SZ / 8 / 64;                // 1 KB wave loads per block, all from the staging wave
  __shared__ __align__(16) bf16 buf[2][SZ];

  const FwdKernelArgs& f = a.f;
  const int Hv = f.Hv, Dv = f.Dv, NVB = Dv / 64, GH = Dv / 16 / WG;
  // workgroup id -> (head index, column group); the groups of a head share an XCD
  const int bid = blockIdx.x, xcd = bid & 7, r8 = bid >> 3;
  const int g = r8 % GH, hidx = xcd + 8 * (r8 / GH);
  if (hidx >= num_heads) return;
  const int n = hidx / Hv, h = hidx % Hv;
  int bos, eos;
  seq_span(f, n, bos, eos);
  const int nchunks = (eos - bos + CHUNK - 1) / CHUNK;
  const int slot0 = n + bos / CHUNK;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = __lane_id();
  const int r16 = lane & 15, grp = lane >> 4;
  auto chunk_ch = [&](int c) { return (int64_t)(slot0 + c) * Hv + h; };
  if (wave == WG) {
    // ---- staging wave: the image block of each chunk, one chunk ahead
    auto dma = [&](int c, int b) {
      const u32x4* src = reinterpret_cast<const u32x4*>(a.ws_bimg + chunk_ch(c) * SZ);
      u32x4* dst = reinterpret_cast<u32x4*>(buf[b]);
#pragma unroll
      for (int j = 0; j < NINS; ++j) __builtin_amdgcn_global_load_lds(src + 64 * j + lane, dst + 64 * j, 16, 0, 0);
    };
    // Beside the image kernel: chunk c's flag, before the barrier after which
    // the column waves load its A1 and A2 (two chunks ahead of the copies'
    // own use), bounded to about 2^27 clocks (on give-up the error flag is
    // set and the work goes on).
    auto wait_ready = [&](int c) {
      if (!a.flags || c < 0 || c >= nchunks - a.rev_done) return;
      const uint32_t* fl = a.flags + chunk_ch(c);
      const uint64_t t0 = __builtin_amdgcn_s_memtime();
      while (__hip_atomic_load(fl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
        if (__builtin_amdgcn_s_memtime() - t0 > (1ull << 27)) {
          if (lane == 0) __hip_atomic_fetch_or(f.err, kErrFlagWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    };
    if (nchunks > 0) {
      if (a.flags) {
        wait_ready(nchunks - 1);
        wait_ready(nchunks - 2);
        lds_barrier();                            // the column waves' first loads may start
      }
      dma(nchunks - 1, (nchunks - 1) & 1);
      vm_drain();
      lds_barrier();
    }
    for (int c = nchunks - 1; c >= 0; --c) {
      wait_ready(c - 2);                          // A1, A2 of chunk c - 2, loaded after this barrier
      if (c > 0) dma(c - 1, (c - 1) & 1);
      vm_drain();                                 // staging of chunk c - 1 landed
      lds_barrier();
    }
    return;
  }
  const int cgi = g * WG + wave;                   // 16-column group of this wave
  const int vb = cgi >> 2, wq = cgi & 3;           // its 64-wide block and place in it
  const int wcol = 16 * cgi;
  const int64_t sbase = ((int64_t)n * Hv + h) * DK * Dv;

  // dS in accumulator layout: dS[mt][i] = dS[16 mt + 4 grp + i][wcol + r16]
  f32x4 dS[MK];
#pragma unroll
  for (int mt = 0; mt < MK; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dS[mt][i] = a.dht ? a.dht[sbase + (int64_t)(16 * mt + 4 * grp + i) * Dv + wcol + r16] : 0.f;

  f32x4 A1c[4], A1n[4], A2c[MK], A2n[MK];
  auto load_a = [&](int c, f32x4 (&A1)[4], f32x4 (&A2)[MK]) {
    const int64_t ch = chunk_ch(c);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      A1[mt] = *reinterpret_cast<const f32x4*>(a.ws_a1 + frag_off(ch, NVB, vb, wq, 4, mt, lane));
#pragma unroll
    for (int mt = 0; mt < MK; ++mt)
      A2[mt] = *reinterpret_cast<const f32x4*>(a.ws_a2 + frag_off(ch, NVB, vb, wq, MK, mt, lane));
  };

  if (nchunks > 0) {
    if (a.flags) lds_barrier();                   // the staging wave saw the last two chunks' flags
    load_a(nchunks - 1, A1c, A2c);
    vm_drain();
    lds_barrier();
  }
  for (int c = nchunks - 1; c >= 0; --c) {
    const int64_t ch = chunk_ch(c);
    const bf16* B = buf[c & 1];
    // dS' of this chunk, for the chunk-local gradients (stores first: issued
    // behind the staging loads they would wait for them)
#pragma unroll
    for (int mt = 0; mt < MK; ++mt)
      *reinterpret_cast<f32x4*>(a.ws_dstate + frag_off(ch, NVB, vb, wq, MK, mt, lane)) = dS[mt];
    if (c > 0) load_a(c - 1, A1n, A2n);
    // dS' as B operands (paired order over dk), hi + lo
    bf16x8 bSh[MK / 2], bSl[MK / 2];
#pragma unroll
    for (int kk = 0; kk < MK / 2; ++kk) pack_pair_split(dS[2 * kk], dS[2 * kk + 1], bSh[kk], bSl[kk]);
    // K dS'
    f32x4 t1[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) t1[mt] = zero4();
#pragma unroll
    for (int kk = 0; kk < MK / 2; ++kk)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 ak = ld_wq<DK>(B, 16 * mt + r16, kk, grp);
        t1[mt] = mfma(ak, bSh[kk], t1[mt]);
        t1[mt] = mfma(ak, bSl[kk], t1[mt]);
      }
    // dVnew = A1 + e^(gamma_n - gamma) K dS'
    const float* G = reinterpret_cast<const float*>(B + BI::g_at(NW));
    f32x4 dvn[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const f32x4 egc = *reinterpret_cast<const f32x4*>(&G[16 * mt + 4 * grp]);
#pragma unroll
      for (int i = 0; i < 4; ++i) dvn[mt][i] = fmaf(egc[i], t1[mt][i], A1c[mt][i]);
      *reinterpret_cast<f32x4*>(a.ws_dvn + frag_off(ch, NVB, vb, wq, 4, mt, lane)) = dvn[mt];
    }
    // -dW dVnew as B operands (paired order over tokens), hi + lo
    const float nsc = G[65], egC = G[64];
    bf16x8 bVh[2], bVl[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      f32x4 d0, d1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        d0[i] = nsc * dvn[2 * kk][i];
        d1[i] = nsc * dvn[2 * kk + 1][i];
      }
      pack_pair_split(d0, d1, bVh[kk], bVl[kk]);
    }
    // dS = e^gamma_n dS' + A2 - dW W^T dVnew
#pragma unroll
    for (int mt = 0; mt < MK; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) dS[mt][i] = fmaf(egC, dS[mt][i], A2c[mt][i]);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int mt = 0; mt < MK; ++mt) {
        const bf16x8 aw = lds_nat(B + BI::KI, 16 * mt + r16, I::R64, 32 * kk, grp);
        dS[mt] = mfma(aw, bVh[kk], dS[mt]);
        dS[mt] = mfma(aw, bVl[kk], dS[mt]);
        if constexpr (NW == 2) {
          const bf16x8 al = lds_nat(B + BI::KI + BI::WT, 16 * mt + r16, I::R64, 32 * kk, grp);
          dS[mt] = mfma(al, bVh[kk], dS[mt]);
        }
      }
    vm_drain();                                   // this wave's loads of chunk c - 1 landed
    lds_barrier();
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) A1c[mt] = A1n[mt];
#pragma unroll
    for (int mt = 0; mt < MK; ++mt) A2c[mt] = A2n[mt];
  }
  if (a.dh0) {
#pragma unroll
    for (int mt = 0; mt < MK; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a.dh0[sbase + (int64_t)(16 * mt + 4 * grp + i) * Dv + wcol + r16] = dS[mt][i];
  }
}

template <int DK, int DV>
static hipError_t launch_img_dv(const BwdConfig& c, const BwdKernelArgs& a, hipStream_t s,
                                hipEvent_t stop) {
  // beside the state kernel: one workgroup per item of the reverse
  // chunk-major order (dispatched in that order)
  const dim3 grid = a.rev_maxc > 0 ? dim3((unsigned)(a.rev_hi - a.rev_lo)) : dim3(a.num_slots, c.Hv);
  if (grid.x == 0) return stop ? hipEventRecord(stop, s) : hipSuccess;
#define GDN_CASE(WFv) \
  if (c.w_fmt == WFv) { \
    if (stop) \
      hipExtLaunchKernelGGL((bwd_img_kernel<DK, DV, WFv>), grid, dim3(NT), 0, s, nullptr, stop, 0, a, c.N); \
    else \
      hipLaunchKernelGGL((bwd_img_kernel<DK, DV, WFv>), grid, dim3(NT), 0, s, a, c.N); \
    return hipGetLastError(); \
  }
  GDN_CASE(0) GDN_CASE(1) GDN_CASE(2)
#undef GDN_CASE
  return hipErrorInvalidValue;
}

template <int DK>
static hipError_t launch_img_dk(const BwdConfig& c, const BwdKernelArgs& a, hipStream_t s, hipEvent_t stop) {
  if (c.Dv == 64) return launch_img_dv<DK, 64>(c, a, s, stop);
  if (c.Dv == 128) return launch_img_dv<DK, 128>(c, a, s, stop);
  if (c.Dv == 256) return launch_img_dv<DK, 256>(c, a, s, stop);
  return hipErrorInvalidValue;
}

template <int DK, int NW, int WG>
static hipError_t launch_state_wg(const BwdConfig& c, const BwdKernelArgs& a, hipStream_t s) {
  const int num_heads = c.N * c.Hv, gh = c.Dv / 16 / WG;
  const int64_t nblk = (int64_t)gh * 8 * ((num_heads + 7) / 8);
  hipLaunchKernelGGL((bwd_state_kernel<DK, NW, WG>), dim3((unsigned)nblk), dim3(64 * (WG + 1)), 0, s, a,
                     c.N, num_heads);
  return hipGetLastError();
}

// As few waves per workgroup as keep every compute unit busy with one.
template <int DK, int NW>
static hipError_t launch_state_dk(const BwdConfig& c, const BwdKernelArgs& a, hipStream_t s) {
  const int64_t units = (int64_t)c.N * c.Hv * (c.Dv / 64), cus = device_cus();
  if (4 * units <= cus) return launch_state_wg<DK, NW, 1>(c, a, s);
  if (2 * units <= cus) return launch_state_wg<DK, NW, 2>(c, a, s);
  return launch_state_wg<DK, NW, 4>(c, a, s);
}

}  // namespace

int bwd_img_elems(int Dk, int w_fmt) {
  const int nw = w_fmt == 0 ? 2 : 1;
  return Dk == 128 ? BImg<128>::size(nw) : BImg<64>::size(nw);
}

hipError_t launch_bwd_img(const BwdConfig& c, const BwdKernelArgs& a, hipStream_t s, hipEvent_t stop) {
  if (c.Dk == 128) return launch_img_dk<128>(c, a, s, stop);
  if (c.Dk == 64) return launch_img_dk<64>(c, a, s, stop);
  return hipErrorInvalidValue;
}

namespace {
template <int DK, int DV, int NW>
int64_t img_state_lds() {                          // one image and one state workgroup (bytes)
  return (int64_t)sizeof(ImgSmem<DK, DV, NW>) + 2 * 2 * (int64_t)BImg<DK>::size(NW);
}
template <int DK>
int64_t img_state_lds_dk(int dv, int nw) {
  if (dv == 64) return nw == 1 ? img_state_lds<DK, 64, 1>() : img_state_lds<DK, 64, 2>();
  if (dv == 128) return nw == 1 ? img_state_lds<DK, 128, 1>() : img_state_lds<DK, 128, 2>();
  return nw == 1 ? img_state_lds<DK, 256, 1>() : img_state_lds<DK, 256, 2>();
}
}  // namespace

bool bwd_overlap_fits(const BwdConfig& c) {
  if (c.f32_io) return false;
  const int nw = c.w_fmt != 0 ? 1 : 2;
  const int64_t lds = c.Dk == 128 ? img_state_lds_dk<128>(c.Dv, nw) : img_state_lds_dk<64>(c.Dv, nw);
  int dev = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
          hipSuccess)
    return false;
  if (lds > per_cu) return false;
  // the state kernel's grid, as launch_state_dk sizes it
  const int64_t units = (int64_t)c.N * c.Hv * (c.Dv / 64), cus = device_cus();
  const int wg = 4 * units <= cus ? 1 : 2 * units <= cus ? 2 : 4;
  const int64_t heads = (int64_t)c.N * c.Hv;
  const int64_t nblk = (int64_t)(c.Dv / 16 / wg) * 8 * ((heads + 7) / 8);
  return nblk <= cus;
}

hipError_t launch_bwd_state(const BwdConfig& c, const BwdKernelArgs& a, hipStream_t s) {
  const bool w_on = c.w_fmt != 0;
  if (c.Dk == 128) return w_on ? launch_state_dk<128, 1>(c, a, s) : launch_state_dk<128, 2>(c, a, s);
  if (c.Dk == 64) return w_on ? launch_state_dk<64, 1>(c, a, s) : launch_state_dk<64, 2>(c, a, s);
  return hipErrorInvalidValue;
}

}  // namespace gdn
