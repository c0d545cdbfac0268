// Decode continuation: token-state writes through the state quantizer, the
// two readouts, and the identity straight-through backward.
//
// "[2/4] GDN/KDA decode QAT with INT8 recurrent state", "What does this PR
// do?": after an exact chunk prefill of an explicit prefix, every further
// token updates the recurrent state, which is written to the state cache
// through the dynamic E4M3 / INT8 quantizer (per-head [Dk, block_v] scales,
// nearest-even rounding, identity straight-through gradients through the
// initial state and the continuation); "Testing": both readouts, split carry,
// all state scale widths. Per (sequence, value head), from the state handed
// over (the prefill's final state or an initial state):
//   S <- QDQ(S)                                         (first write)
//   token t:  S <- exp(g_t) S;  u = beta_t (v_t - S^T k_t);  S <- S + k_t u^T
//             o_before = scale S^T q_t;  S <- QDQ(S);  o_after = scale S^T q_t
//   ht = S (the last state written)
// QDQ is the FP32 definition in gdn.h (IEEE division for d and 1/d), the
// identity when the state format is off. All arithmetic is FP32.
//
// One workgroup per (sequence, value head, group of NS 64-column slabs), NS
// the slabs of one scale tile (1 up to block_v 64): the columns are
// independent but for the tile amax, and the backward's dq, dk, dbeta and dg,
// which sum over every column, leave per-group partial sums that a second
// kernel adds up in a fixed order. Each slab is split over four waves by
// key rows. Wave w: slab s = w / 4, row quarter r = w % 4. Lane l holds an
// RPL x 8 block of S (RPL = Dk / 32): the workgroup's columns 64 s + 8 (l & 7)
// .. + 7, rows r Dk / 4 + (l >> 3) RPL .. + RPL - 1, so a
// sum over key rows is three lane exchanges and one LDS exchange across the
// four row quarters, and a sum over value columns is three DPP steps within
// eight lanes plus an LDS exchange across slabs. The per-token work is a few
// matrix-vector products: it runs on the vector ALUs, not on matrix cores.
//
// Saved written states (for the backward): the first write of sequence n is
// slot lo_n + n (lo_n = first decode token), the write after decode token t
// is slot t + n + 1; codes [slot, Hv, Dk, Dv] bytes and FP32 scales [slot,
// Hv, Dv / block_v], or FP32 states [slot, Hv, Dk, Dv] with the format off.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// N consecutive elements (N = 2, 4 or 8) of a bf16 or FP32 array, as floats.
template <int N, bool F32>
__device__ __forceinline__ void ld_vec(const void* base, int64_t off, float (&x)[N]) {
  if constexpr (F32) {
    const float* p = reinterpret_cast<const float*>(base) + off;
    if constexpr (N == 2) {
      const f32x2 v = *reinterpret_cast<const f32x2*>(p);
      x[0] = v[0];
      x[1] = v[1];
    } else {
#pragma unroll
      for (int h = 0; h < N / 4; ++h) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(p + 4 * h);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * h + e] = v[e];
      }
    }
  } else {
    const bf16* p = reinterpret_cast<const bf16*>(base) + off;
    if constexpr (N == 2) {
      const bf16x2 v = *reinterpret_cast<const bf16x2*>(p);
      x[0] = from_bf16(v[0]);
      x[1] = from_bf16(v[1]);
    } else if constexpr (N == 4) {
      const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = from_bf16(v[e]);
    } else {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = from_bf16(v[e]);
    }
  }
}

template <int N, bool F32>
__device__ __forceinline__ void st_vec(void* base, int64_t off, const float (&x)[N]) {
  if constexpr (F32) {
    float* p = reinterpret_cast<float*>(base) + off;
    if constexpr (N == 2) {
      *reinterpret_cast<f32x2*>(p) = f32x2{x[0], x[1]};
    } else {
#pragma unroll
      for (int h = 0; h < N / 4; ++h)
        *reinterpret_cast<f32x4*>(p + 4 * h) =
            f32x4{x[4 * h], x[4 * h + 1], x[4 * h + 2], x[4 * h + 3]};
    }
  } else {
    bf16* p = reinterpret_cast<bf16*>(base) + off;
    if constexpr (N == 2) {
      *reinterpret_cast<bf16x2*>(p) = bf16x2{to_bf16(x[0]), to_bf16(x[1])};
    } else if constexpr (N == 4) {
      *reinterpret_cast<bf16x4*>(p) =
          bf16x4{to_bf16(x[0]), to_bf16(x[1]), to_bf16(x[2]), to_bf16(x[3])};
    } else {
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = to_bf16(x[e]);
      *reinterpret_cast<bf16x8*>(p) = v;
    }
  }
}

// The values of lanes l ^ 16 and l ^ 32, by the gfx950 lane swaps (VALU, no
// LDS crossbar): v_permlane16_swap on two copies of x leaves rows (0, 0, 2, 2)
// in one and (1, 1, 3, 3) in the other, v_permlane32_swap halves (0, 0) and
// (1, 1); each lane then holds its own value and its partner's, one in each.
// (Written as one VALU instruction in asm: this compiler's builtin returns
// the first result in both places. The s_nop covers the wait states the
// swap needs after a VALU write of its operands.)
struct LanePair {
  float a, b;
};
__device__ __forceinline__ LanePair swap16(float x) {
  float a = x, b = x;
  asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return {a, b};
}
__device__ __forceinline__ LanePair swap32(float x) {
  float a = x, b = x;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return {a, b};
}
// N consecutive bf16 or FP32 elements at byte offset `off` of an LDS buffer.
template <int N, bool F32>
__device__ __forceinline__ void lds_vec(const char* base, int off, float (&x)[N]) {
  if constexpr (F32) {
    if constexpr (N == 2) {
      const f32x2 v = *reinterpret_cast<const f32x2*>(base + off);
      x[0] = v[0];
      x[1] = v[1];
    } else {
#pragma unroll
      for (int h = 0; h < N / 4; ++h) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(base + off + 16 * h);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * h + e] = v[e];
      }
    }
  } else {
    if constexpr (N == 2) {
      const bf16x2 v = *reinterpret_cast<const bf16x2*>(base + off);
      x[0] = from_bf16(v[0]);
      x[1] = from_bf16(v[1]);
    } else if constexpr (N == 4) {
      const bf16x4 v = *reinterpret_cast<const bf16x4*>(base + off);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = from_bf16(v[e]);
    } else {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(base + off);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = from_bf16(v[e]);
    }
  }
}

// Sum over the eight row groups of a wave (lanes l, l ^ 8, l ^ 16, ...):
// row_ror:8 within each row of 16 lanes, then the two swaps across rows.
__device__ __forceinline__ float sum_rows8(float x) {
  x += dpp_f<0x128>(x);
  LanePair p = swap16(x);
  x = p.a + p.b;
  p = swap32(x);
  return p.a + p.b;
}
// Sum over the eight column groups of a wave (lanes 8 m .. 8 m + 7): quad
// swaps, then the half-row mirror (after the quad steps all lanes of a quad
// hold the same value, so lane i and 7 - i add the two quads).
__device__ __forceinline__ float sum_cols8(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0x141>(x);
  return x;
}
// Maximum over the lanes of one [Dk / 4 rows, block_v] part of a tile
// within a wave (block_v / 8 column groups, all row groups).
__device__ __forceinline__ float max_tile_lanes(float m, int block_v) {
  m = fmaxf(m, dpp_f<0x128>(m));
  LanePair p = swap16(m);
  m = fmaxf(p.a, p.b);
  p = swap32(m);
  m = fmaxf(p.a, p.b);
  m = fmaxf(m, dpp_f<0xB1>(m));                     // block_v >= 16
  if (block_v >= 32) m = fmaxf(m, dpp_f<0x4E>(m));
  if (block_v >= 64) m = fmaxf(m, dpp_f<0x141>(m));
  return m;
}

// Eight codes (two words) of one row part -> values c * d.
template <int SF>
__device__ __forceinline__ void decode8(uint32_t w0, uint32_t w1, float d, float (&x)[8]) {
  if constexpr (SF == 1) {
    x[0] = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(w0), 0) * d;
    x[1] = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(w0), 1) * d;
    x[2] = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(w0), 2) * d;
    x[3] = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(w0), 3) * d;
    x[4] = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(w1), 0) * d;
    x[5] = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(w1), 1) * d;
    x[6] = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(w1), 2) * d;
    x[7] = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(w1), 3) * d;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = static_cast<float>(static_cast<int8_t>((w0 >> (8 * e)) & 0xFFu)) * d;
      x[4 + e] = static_cast<float>(static_cast<int8_t>((w1 >> (8 * e)) & 0xFFu)) * d;
    }
  }
}

struct Span {
  int bos, eos, lo;
};

// The gates of a window of 64 decode tokens, one token per lane (vector
// loads, read back with readlane): scalar loads of g and beta per token
// would be waited for by every LDS barrier (which waits lgkmcnt), so the
// windows are loaded one window ahead instead.
struct GateWin {
  float g, b;
};
__device__ __forceinline__ GateWin load_gate_win(const DecodeKernelArgs& a, int h, const Span& sp,
                                                 int w) {
  GateWin gw{0.f, 0.f};
  const int t = sp.lo + 64 * w + __lane_id();
  if (w >= 0 && t < sp.eos) {
    gw.g = a.g[(int64_t)t * a.Hv + h];
    gw.b = a.beta[(int64_t)t * a.Hv + h];
  }
  return gw;
}
__device__ __forceinline__ Span decode_span(const DecodeKernelArgs& a, int n) {
  Span sp;
  if (a.cu_seqlens) {
    sp.bos = a.cu_seqlens[n];
    sp.eos = a.cu_seqlens[n + 1];
  } else {
    sp.bos = n * a.T;
    sp.eos = sp.bos + a.T;
  }
  sp.lo = sp.bos + min(a.start, sp.eos - sp.bos);
  return sp;
}

// ------------------------------------------------------------------ forward
template <int DK, bool F32, int SF, int NS>
__global__ void __launch_bounds__(256 * NS, 1) decode_fwd_kernel(DecodeKernelArgs a) {
  constexpr int RPL = DK / 32;
  // Token inputs arrive in LDS windows of W tokens by global-to-LDS copies
  // issued one window ahead, so no token waits on a global load (a wait for a
  // register load would also wait for the stores issued after it): per
  // window K and Q [W][DK], V [W][Dv] in the input dtype, then g and beta
  // [W] each (FP32).
  constexpr int ES = F32 ? 4 : 2, W = 32, NWV = 4 * NS;
  constexpr int KB = W * DK * ES, VB = W * 64 * NS * ES, NBLK = (2 * KB + VB) / 1024;
  static_assert((2 * KB + VB) % 1024 == 0, "1 KB copy blocks");
  __shared__ __attribute__((aligned(16))) char win[2][2 * KB + VB + 2 * W * 4];
  __shared__ float xp[NS][4][64];   // S^T k per row quarter
  __shared__ float xo[NS][4][64];   // S^T q per row quarter
  __shared__ float xa[NS][4][8];    // tile amax per row quarter and column group
  // workgroup -> (head index, group of NS slabs): the slab groups of a head
  // share an XCD (workgroups go round-robin over the eight)
  const int Hv = a.Hv, Dv = a.Dv, ng = Dv / (64 * NS), VW = 64 * NS;
  const int bid = blockIdx.x, r8 = bid >> 3, gi = r8 % ng, hidx = (bid & 7) + 8 * (r8 / ng);
  if (hidx >= a.num_seqs * Hv) return;
  const int h = hidx % Hv, n = hidx / Hv;
  const int hk = h / (Hv / a.Hqk);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s = wave >> 2, r = wave & 3, lane = __lane_id(), cg = lane & 7, rg = lane >> 3;
  // lcol: first of the lane's 8 columns within this workgroup's slabs; col0 within the head
  const int row0 = r * (DK / 4) + rg * RPL, lcol = 64 * s + 8 * cg, col0 = VW * gi + lcol;
  const Span sp = decode_span(a, n);
  const int bv = a.block_v, nsl = bv > 64 ? bv / 64 : 1, sb = (s / nsl) * nsl;
  const bool before = a.readout == 0;
  const int64_t st_base = ((int64_t)n * Hv + h) * DK * Dv;

  float S[RPL][8];
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    if (a.h_in) {
      ld_vec<8, true>(a.h_in, st_base + (int64_t)(row0 + i) * Dv + col0, S[i]);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) S[i][c] = 0.f;
    }
  }

  // Local part of the tile amax, reduced over this wave's lanes of the tile.
  auto amax_publish = [&]() {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < RPL; ++i)
#pragma unroll
      for (int c = 0; c < 8; ++c) m = fmaxf(m, fabsf(S[i][c]));
    m = max_tile_lanes(m, bv);
    if (rg == 0) xa[s][r][cg] = m;
  };
  // After the barrier: quantize with the tile's scale and save the written
  // state into `slot` when a saved buffer is given.
  auto write_state = [&](int64_t slot) {
    if constexpr (SF != 0) {
      float amax = 0.f;
      for (int ss = 0; ss < nsl; ++ss)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) amax = fmaxf(amax, xa[sb + ss][rr][cg]);
      const float d = qdq_scale<SF>(amax);
      const float rcp = 1.0f / d;
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        float c[8];
        uint32_t w0, w1;
        quant4<SF>(*reinterpret_cast<const float(*)[4]>(&S[i][0]), rcp,
                   *reinterpret_cast<float(*)[4]>(&c[0]), w0);
        quant4<SF>(*reinterpret_cast<const float(*)[4]>(&S[i][4]), rcp,
                   *reinterpret_cast<float(*)[4]>(&c[4]), w1);
#pragma unroll
        for (int e = 0; e < 8; ++e) S[i][e] = c[e] * d;
        if (a.s_codes) {
          const int64_t off = ((slot * Hv + h) * DK + row0 + i) * (int64_t)Dv + col0;
          *reinterpret_cast<uint2*>(a.s_codes + off) = make_uint2(w0, w1);
        }
      }
      if (a.s_scale && r == 0 && rg == 0 && col0 % bv == 0)
        a.s_scale[(slot * Hv + h) * (Dv / bv) + col0 / bv] = d;
    } else {
      if (a.s_f32) {
#pragma unroll
        for (int i = 0; i < RPL; ++i)
          st_vec<8, true>(a.s_f32, ((slot * Hv + h) * DK + row0 + i) * (int64_t)Dv + col0, S[i]);
      }
    }
  };

  // copies of window w (tokens lo + W w ..) into buffer b; tokens past the
  // end repeat the last one (their values are never read)
  const int nwin = (sp.eos - sp.lo + W - 1) / W;
  auto issue_window = [&](int w, int b) {
    const int t0 = sp.lo + W * w;
    char* base = win[b];
    for (int j = wave; j < NBLK; j += NWV) {
      const int off = 1024 * j + 16 * lane;
      const char* src;
      if (off < 2 * KB) {
        const int o = off < KB ? off : off - KB;
        const int tok = min(t0 + o / (DK * ES), sp.eos - 1);
        src = reinterpret_cast<const char*>(off < KB ? a.k : a.q) +
              ((int64_t)tok * a.Hqk + hk) * (DK * ES) + o % (DK * ES);
      } else {                                      // this workgroup's VW columns of v
        const int o = off - 2 * KB;
        const int tok = min(t0 + o / (VW * ES), sp.eos - 1);
        src = reinterpret_cast<const char*>(a.v) + (((int64_t)tok * Hv + h) * Dv + VW * gi) * ES +
              o % (VW * ES);
      }
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4*>(src),
                                       reinterpret_cast<uint4*>(base + 1024 * j), 16, 0, 0);
    }
    if (wave == NWV - 1) {                          // g (lanes 0..31) and beta (32..63)
      const int tok = min(t0 + (lane & 31), sp.eos - 1);
      const float* src = (lane < 32 ? a.g : a.beta) + (int64_t)tok * Hv + h;
      __builtin_amdgcn_global_load_lds(src, reinterpret_cast<float*>(base + 2 * KB + VB), 4, 0, 0);
    }
  };
  if (nwin > 0) issue_window(0, 0);

  // first write: the state handed over, as the cache holds it
  const int64_t slot0 = (int64_t)sp.lo + n;
  if constexpr (SF != 0) {
    amax_publish();
    lds_barrier();
  }
  write_state(slot0);

  for (int t = sp.lo; t < sp.eos; ++t) {
    const int j = t - sp.lo, w = j / W, tok = j % W;
    const char* wb = win[w & 1];
    if (tok == 0) {
      vm_drain();                                   // this window's copies have landed
      lds_barrier();
      if (w + 1 < nwin) issue_window(w + 1, (w + 1) & 1);
    }
    float kk[RPL], qq[RPL], vv[8];
    lds_vec<RPL, F32>(wb, (tok * DK + row0) * ES, kk);
    lds_vec<RPL, F32>(wb, KB + (tok * DK + row0) * ES, qq);
    lds_vec<8, F32>(wb, 2 * KB + (tok * VW + lcol) * ES, vv);
    const float* gb = reinterpret_cast<const float*>(wb + 2 * KB + VB);
    const float eg = expf(gb[tok]), bt = gb[W + tok];

    // decay and the delta-rule prediction S^T k
    float pp[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      pp[c] = 0.f;
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        S[i][c] *= eg;
        pp[c] = fmaf(S[i][c], kk[i], pp[c]);
      }
      pp[c] = sum_rows8(pp[c]);
    }
    if (rg == 0) {
      *reinterpret_cast<f32x4*>(&xp[s][r][8 * cg]) = f32x4{pp[0], pp[1], pp[2], pp[3]};
      *reinterpret_cast<f32x4*>(&xp[s][r][8 * cg + 4]) = f32x4{pp[4], pp[5], pp[6], pp[7]};
    }
    lds_barrier();
    float u[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float p = xp[s][0][8 * cg + c] + xp[s][1][8 * cg + c] + xp[s][2][8 * cg + c] +
                      xp[s][3][8 * cg + c];
      u[c] = bt * (vv[c] - p);
    }
    // the write S + k u^T
#pragma unroll
    for (int i = 0; i < RPL; ++i)
#pragma unroll
      for (int c = 0; c < 8; ++c) S[i][c] = fmaf(kk[i], u[c], S[i][c]);

    auto publish_o = [&]() {
      float po[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        po[c] = 0.f;
#pragma unroll
        for (int i = 0; i < RPL; ++i) po[c] = fmaf(S[i][c], qq[i], po[c]);
        po[c] = sum_rows8(po[c]);
      }
      if (rg == 0) {
        *reinterpret_cast<f32x4*>(&xo[s][r][8 * cg]) = f32x4{po[0], po[1], po[2], po[3]};
        *reinterpret_cast<f32x4*>(&xo[s][r][8 * cg + 4]) = f32x4{po[4], po[5], po[6], po[7]};
      }
    };
    auto store_o = [&]() {
      if (r == 0 && rg == 0) {
        float o[8];
#pragma unroll
        for (int c = 0; c < 8; ++c)
          o[c] = a.scale * (xo[s][0][8 * cg + c] + xo[s][1][8 * cg + c] + xo[s][2][8 * cg + c] +
                            xo[s][3][8 * cg + c]);
        st_vec<8, F32>(a.o, ((int64_t)t * Hv + h) * Dv + col0, o);
      }
    };
    if (before) publish_o();
    if constexpr (SF != 0) amax_publish();
    if (SF != 0 || before) lds_barrier();
    write_state((int64_t)t + n + 1);
    if (before) {
      store_o();
    } else {
      publish_o();
      lds_barrier();
      store_o();
    }
  }
  if (a.ht) {
#pragma unroll
    for (int i = 0; i < RPL; ++i) st_vec<8, true>(a.ht, st_base + (int64_t)(row0 + i) * Dv + col0, S[i]);
  }
}

// ----------------------------------------------------------------- backward
// Reverse over the decode tokens with the carry dS = dL/d(state as written).
// Token t (A = exp(g_t) S_prev, S_prev the written state before t, S' the
// updated state before its write, S_t = QDQ(S') the written one; identity
// straight-through at every write, so dL/dS' = dL/dS_t):
//   dS' = dS + scale q do^T      (either readout)
//   dq  = scale S' do (before the write) or scale S_t do (after it)
//   du  = dS'^T k;  dv = beta du;  dbeta = du . (v - A^T k);  dp = -beta du
//   dk  = dS' u + A dp;  dA = dS' + k dp^T;  dg = <A, dA>;  dS <- exp(g_t) dA
// and after the first decode token dh_in = dS (through the first write).
template <int DK, bool F32, int SF, int NS>
__global__ void __launch_bounds__(256 * NS, 1) decode_bwd_kernel(DecodeKernelArgs a) {
  constexpr int RPL = DK / 32;
  __shared__ float xp[NS][4][64];   // A^T k per row quarter
  __shared__ float xu[NS][4][64];   // dS'^T k per row quarter
  __shared__ float xq[NS][DK];      // dq rows per slab
  __shared__ float xk[NS][DK];      // dk rows per slab
  __shared__ float xs[NS * 4][4];   // per wave: [0] u . do, [1] dbeta, [2] dg
  // workgroup -> (head index, group of NS slabs), as in the forward
  const int Hv = a.Hv, Dv = a.Dv, ng = Dv / (64 * NS);
  const int bid = blockIdx.x, r8 = bid >> 3, gi = r8 % ng, hidx = (bid & 7) + 8 * (r8 / ng);
  if (hidx >= a.num_seqs * Hv) return;
  const int h = hidx % Hv, n = hidx / Hv;
  const int hk = h / (Hv / a.Hqk);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s = wave >> 2, r = wave & 3, lane = __lane_id(), cg = lane & 7, rg = lane >> 3;
  const int row0 = r * (DK / 4) + rg * RPL, col0 = 64 * (NS * gi + s) + 8 * cg;
  const Span sp = decode_span(a, n);
  const int bv = a.block_v;
  const bool before = a.readout == 0;
  const int64_t st_base = ((int64_t)n * Hv + h) * DK * Dv;
  // partial sums (this workgroup's columns) of dq, dk, dg, dbeta go to the
  // workspace when a head's columns span several workgroups or its dq, dk
  // sum over a group of value heads: [token, value head, slab group][PW]
  const bool group = a.ws_dqk != nullptr;
  constexpr int PW = 2 * DK + 4;
  auto part = [&](int64_t tv) { return a.ws_dqk + (tv * ng + gi) * PW; };

  float dS[RPL][8];
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    if (a.dht) {
      ld_vec<8, true>(a.dht, st_base + (int64_t)(row0 + i) * Dv + col0, dS[i]);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) dS[i][c] = 0.f;
    }
  }

  // A written state of this lane's block: its codes and scale held in
  // registers (format on), or its slot, read from memory at each use (FP32
  // states would take 32 more registers per state).
  struct Held {
    uint32_t w[SF == 0 ? 1 : RPL][2];
    float d;
    int64_t slot;
  };
  auto load_state = [&](int64_t slot, Held& st) {
    if constexpr (SF != 0) {
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        const uint2 v = *reinterpret_cast<const uint2*>(
            a.s_codes + ((slot * Hv + h) * DK + row0 + i) * (int64_t)Dv + col0);
        st.w[i][0] = v.x;
        st.w[i][1] = v.y;
      }
      st.d = a.s_scale[(slot * Hv + h) * (Dv / bv) + col0 / bv];
    } else {
      st.slot = slot;
    }
  };
  // (the codes pass through an empty asm so that each use decodes them again
  // instead of keeping all decoded values live across the phases)
  auto row_of = [&](const Held& st, int i, float (&x)[8]) {
    if constexpr (SF != 0) {
      uint32_t w0 = st.w[i][0], w1 = st.w[i][1];
      asm volatile("" : "+v"(w0), "+v"(w1));
      decode8<SF>(w0, w1, st.d, x);
    } else {
      ld_vec<8, true>(a.s_f32, ((st.slot * Hv + h) * DK + row0 + i) * (int64_t)Dv + col0, x);
    }
  };

  Held cur, prev, pnext;           // written state after token t, before it, before t - 1
  if (sp.lo < sp.eos && !before) load_state((int64_t)(sp.eos - 1) + n + 1, cur);
  // token inputs and the written state before the token, one token ahead
  float kn[RPL], qn[RPL], vn[8], dn[8];
  auto load_token = [&](int t) {
    const int64_t qk = ((int64_t)t * a.Hqk + hk) * DK + row0;
    ld_vec<RPL, F32>(a.k, qk, kn);
    ld_vec<RPL, F32>(a.q, qk, qn);
    ld_vec<8, F32>(a.v, ((int64_t)t * Hv + h) * Dv + col0, vn);
    ld_vec<8, F32>(a.dout, ((int64_t)t * Hv + h) * Dv + col0, dn);
    load_state((int64_t)t + n, pnext);
  };
  if (sp.lo < sp.eos) load_token(sp.eos - 1);
  int wcur = sp.lo < sp.eos ? (sp.eos - 1 - sp.lo) >> 6 : 0;
  GateWin gcur = load_gate_win(a, h, sp, wcur), gnxt = load_gate_win(a, h, sp, wcur - 1);

  for (int t = sp.eos - 1; t >= sp.lo; --t) {
    float kk[RPL], qq[RPL], vv[8], dd[8];
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      kk[i] = kn[i];
      qq[i] = qn[i];
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      vv[c] = vn[c];
      dd[c] = dn[c];
    }
    prev = pnext;
    const int j = t - sp.lo;
    if ((j >> 6) != wcur) {                         // previous window of gates
      wcur = j >> 6;
      gcur = gnxt;
      gnxt = load_gate_win(a, h, sp, wcur - 1);
    }
    const float eg = expf(read_lane(gcur.g, j & 63)), bt = read_lane(gcur.b, j & 63);
    if (t > sp.lo) load_token(t - 1);               // in flight during this token

    // P1: the prediction A^T k
    float pp[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) pp[c] = 0.f;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      float x[8];
      row_of(prev, i, x);
#pragma unroll
      for (int c = 0; c < 8; ++c) pp[c] = fmaf(eg * x[c], kk[i], pp[c]);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) pp[c] = sum_rows8(pp[c]);
    if (rg == 0) {
      *reinterpret_cast<f32x4*>(&xp[s][r][8 * cg]) = f32x4{pp[0], pp[1], pp[2], pp[3]};
      *reinterpret_cast<f32x4*>(&xp[s][r][8 * cg + 4]) = f32x4{pp[4], pp[5], pp[6], pp[7]};
    }
    lds_barrier();

    // P2: u, dS', du and dq partials, u . do
    float p[8], u[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      p[c] = xp[s][0][8 * cg + c] + xp[s][1][8 * cg + c] + xp[s][2][8 * cg + c] +
             xp[s][3][8 * cg + c];
      u[c] = bt * (vv[c] - p[c]);
    }
    float du[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) du[c] = 0.f;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const float sq = a.scale * qq[i];
      float x[8];
      if (before) {
        row_of(prev, i, x);
#pragma unroll
        for (int c = 0; c < 8; ++c) x[c] *= eg;      // A; the k u^T part of S' joins below
      } else {
        row_of(cur, i, x);
      }
      float dqr = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        dS[i][c] = fmaf(sq, dd[c], dS[i][c]);
        du[c] = fmaf(dS[i][c], kk[i], du[c]);
        dqr = fmaf(x[c], dd[c], dqr);
      }
      dqr = sum_cols8(dqr);
      if (cg == 0) xq[s][row0 + i] = dqr;
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) du[c] = sum_rows8(du[c]);
    if (rg == 0) {
      *reinterpret_cast<f32x4*>(&xu[s][r][8 * cg]) = f32x4{du[0], du[1], du[2], du[3]};
      *reinterpret_cast<f32x4*>(&xu[s][r][8 * cg + 4]) = f32x4{du[4], du[5], du[6], du[7]};
    }
    float udo = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) udo = fmaf(u[c], dd[c], udo);
    udo = sum_cols8(udo);
    if (lane == 0) xs[wave][0] = udo;
    lds_barrier();

    // P3: du complete; dv, dbeta, dq; dk and dg partials; the carry
    float db = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      du[c] = xu[s][0][8 * cg + c] + xu[s][1][8 * cg + c] + xu[s][2][8 * cg + c] +
              xu[s][3][8 * cg + c];
      db = fmaf(du[c], vv[c] - p[c], db);
    }
    const int64_t tv = (int64_t)t * Hv + h;
    if (r == 0 && rg == 0) {
      float dv[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) dv[c] = bt * du[c];
      if (a.grad_f32) st_vec<8, true>(a.dv, tv * Dv + col0, dv);
      else st_vec<8, false>(a.dv, tv * Dv + col0, dv);
    }
    db = sum_cols8(db);
    if (lane == 0) xs[wave][1] = db;
    float ud = 0.f;
#pragma unroll
    for (int ss = 0; ss < NS; ++ss) ud += xs[4 * ss][0];
    if (s == 0 && cg == 0) {
      float dq[RPL];
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        float x = 0.f;
#pragma unroll
        for (int ss = 0; ss < NS; ++ss) x += xq[ss][row0 + i];
        dq[i] = a.scale * (before ? fmaf(kk[i], ud, x) : x);
      }
      if (group) {
        st_vec<RPL, true>(part(tv), row0, dq);
      } else {
        const int64_t off = ((int64_t)t * a.Hqk + hk) * DK + row0;
        if (a.grad_f32) st_vec<RPL, true>(a.dq, off, dq);
        else st_vec<RPL, false>(a.dq, off, dq);
      }
    }
    float dgp = 0.f;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      float x[8];
      row_of(prev, i, x);
      float dkr = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float A = eg * x[c], dp = -bt * du[c];
        dkr = fmaf(dS[i][c], u[c], dkr);
        dkr = fmaf(A, dp, dkr);
        const float dA = fmaf(kk[i], dp, dS[i][c]);
        dgp = fmaf(A, dA, dgp);
        dS[i][c] = eg * dA;
      }
      dkr = sum_cols8(dkr);
      if (cg == 0) xk[s][row0 + i] = dkr;
    }
    dgp = sum_rows8(sum_cols8(dgp));
    if (lane == 0) xs[wave][2] = dgp;
    lds_barrier();

    // P4: dk, dg and dbeta complete
    if (s == 0 && cg == 0) {
      float dk[RPL];
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        float x = 0.f;
#pragma unroll
        for (int ss = 0; ss < NS; ++ss) x += xk[ss][row0 + i];
        dk[i] = x;
      }
      if (group) {
        st_vec<RPL, true>(part(tv), DK + row0, dk);
      } else {
        const int64_t off = ((int64_t)t * a.Hqk + hk) * DK + row0;
        if (a.grad_f32) st_vec<RPL, true>(a.dk, off, dk);
        else st_vec<RPL, false>(a.dk, off, dk);
      }
    }
    if (threadIdx.x == 0) {
      float dg = 0.f, dbt = 0.f;
#pragma unroll
      for (int w = 0; w < NS * 4; ++w) dg += xs[w][2];
#pragma unroll
      for (int ss = 0; ss < NS; ++ss) dbt += xs[4 * ss][1];
      if (group) {
        part(tv)[2 * DK] = dg;
        part(tv)[2 * DK + 1] = dbt;
      } else {
        a.dg[tv] = dg;
        a.dbeta[tv] = dbt;
      }
    }
    cur = prev;
  }
  if (a.dh_in) {
#pragma unroll
    for (int i = 0; i < RPL; ++i)
      st_vec<8, true>(a.dh_in, st_base + (int64_t)(row0 + i) * Dv + col0, dS[i]);
  }
}

// The backward's partial sums: dq, dk of each query/key head over its G value
// heads and their ng slab groups, dg and dbeta of each of those value heads
// over its slab groups, in a fixed order; for decode tokens only (the tokens
// before `start` belong to the prefill).
template <int DK>
__global__ void decode_group(DecodeKernelArgs a, int N, int G, int ng) {
  const int tok = blockIdx.x, hk = blockIdx.y, d = threadIdx.x;
  int bos;
  if (a.cu_seqlens) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.cu_seqlens[mid] <= tok) lo = mid; else hi = mid - 1;
    }
    bos = a.cu_seqlens[lo];
  } else {
    bos = tok - tok % a.T;
  }
  if (d >= DK || tok - bos < a.start) return;
  constexpr int PW = 2 * DK + 4;
  float sq = 0.f, sk = 0.f;
  for (int j = 0; j < G; ++j) {
    const int64_t tv = (int64_t)tok * a.Hv + hk * G + j;
    for (int gi = 0; gi < ng; ++gi) {
      const float* p = a.ws_dqk + (tv * ng + gi) * PW;
      sq += p[d];
      sk += p[DK + d];
    }
    if (d == 0) {
      float dg = 0.f, db = 0.f;
      for (int gi = 0; gi < ng; ++gi) {
        dg += a.ws_dqk[(tv * ng + gi) * PW + 2 * DK];
        db += a.ws_dqk[(tv * ng + gi) * PW + 2 * DK + 1];
      }
      a.dg[tv] = dg;
      a.dbeta[tv] = db;
    }
  }
  const int64_t off = ((int64_t)tok * a.Hqk + hk) * DK + d;
  if (a.grad_f32) {
    reinterpret_cast<float*>(a.dq)[off] = sq;
    reinterpret_cast<float*>(a.dk)[off] = sk;
  } else {
    reinterpret_cast<bf16*>(a.dq)[off] = to_bf16(sq);
    reinterpret_cast<bf16*>(a.dk)[off] = to_bf16(sk);
  }
}

// The forward's 64-column slabs are independent (the prediction, the write,
// the readout and each scale tile are per column or per tile), so a
// workgroup takes as few as hold whole scale tiles, and the slab groups of
// a head run on separate CUs.
template <int DK, bool F32, int SF>
hipError_t launch_fwd_dk(const DecodeConfig& c, const DecodeKernelArgs& a, hipStream_t st) {
  const int ns = decode_slabs_per_group(SF, a.block_v);
  const int64_t heads = (int64_t)c.N * c.Hv;
  const dim3 grid((unsigned)((c.Dv / 64 / ns) * 8 * ((heads + 7) / 8)));
  switch (ns) {
    case 1: hipLaunchKernelGGL((decode_fwd_kernel<DK, F32, SF, 1>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((decode_fwd_kernel<DK, F32, SF, 2>), grid, dim3(512), 0, st, a); break;
    default: hipLaunchKernelGGL((decode_fwd_kernel<DK, F32, SF, 4>), grid, dim3(1024), 0, st, a); break;
  }
  return hipGetLastError();
}

// As the forward: a workgroup per group of the slabs of one scale tile; the
// partial sums over each group's columns are then added up by decode_group.
template <int DK, bool F32, int SF>
hipError_t launch_bwd_dk(const DecodeConfig& c, const DecodeKernelArgs& a, hipStream_t st) {
  const int ns = decode_slabs_per_group(c.state_fmt, a.block_v), ng = c.Dv / 64 / ns;
  if ((ng > 1 || c.Hv > c.Hqk) != (a.ws_dqk != nullptr)) return hipErrorInvalidValue;
  const int64_t heads = (int64_t)c.N * c.Hv;
  const dim3 grid((unsigned)(ng * 8 * ((heads + 7) / 8)));
  switch (ns) {
    case 1: hipLaunchKernelGGL((decode_bwd_kernel<DK, F32, SF, 1>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((decode_bwd_kernel<DK, F32, SF, 2>), grid, dim3(512), 0, st, a); break;
    default: hipLaunchKernelGGL((decode_bwd_kernel<DK, F32, SF, 4>), grid, dim3(1024), 0, st, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.ws_dqk) return e;
  hipLaunchKernelGGL((decode_group<DK>), dim3(a.total_tokens, c.Hqk), dim3(DK), 0, st, a, c.N,
                     c.Hv / c.Hqk, ng);
  return hipGetLastError();
}

template <int DK, bool F32>
hipError_t dispatch_fmt(const DecodeConfig& c, const DecodeKernelArgs& a, hipStream_t st, bool bwd) {
  switch (c.state_fmt) {
    case 0: return bwd ? launch_bwd_dk<DK, F32, 0>(c, a, st) : launch_fwd_dk<DK, F32, 0>(c, a, st);
    case 1: return bwd ? launch_bwd_dk<DK, F32, 1>(c, a, st) : launch_fwd_dk<DK, F32, 1>(c, a, st);
    default: return bwd ? launch_bwd_dk<DK, F32, 2>(c, a, st) : launch_fwd_dk<DK, F32, 2>(c, a, st);
  }
}

hipError_t dispatch(const DecodeConfig& c, const DecodeKernelArgs& a, hipStream_t st, bool bwd) {
  if (c.Dk == 128)
    return c.f32_io ? dispatch_fmt<128, true>(c, a, st, bwd) : dispatch_fmt<128, false>(c, a, st, bwd);
  return c.f32_io ? dispatch_fmt<64, true>(c, a, st, bwd) : dispatch_fmt<64, false>(c, a, st, bwd);
}

}  // namespace

hipError_t launch_decode_fwd(const DecodeConfig& c, const DecodeKernelArgs& a, hipStream_t s) {
  return dispatch(c, a, s, false);
}
hipError_t launch_decode_bwd(const DecodeConfig& c, const DecodeKernelArgs& a, hipStream_t s) {
  return dispatch(c, a, s, true);
}

}  // namespace gdn
