// Device helpers shared by the gfx950 kernels: bf16 MFMA tiles, hi/lo
// operand splitting, the FP32 QDQ arithmetic and wave reductions.
//
// MFMA tile used throughout: v_mfma_f32_16x16x32_bf16 (one wave, 64 lanes).
// Lane l, r16 = l & 15, grp = l >> 4:
//   A (16 x 32, M x K): lane holds A[r16][8*grp + e], e = 0..7
//   B (32 x 16, K x N): lane holds B[8*grp + e][r16]
//   C (16 x 16):        lane holds C[4*grp + i][r16], i = 0..3
// Any permutation of the K index that A and B share gives the same product;
// the kernels use that to feed accumulator tiles (C layout) straight back as
// B operands ("paired-tile" K order, see pack_pair below).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16 raw bytes as a native vector (copies of HIP's uint4 struct lower to
// memcpy through private memory, which is not promoted to registers)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr int CHUNK = 64;

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// The same tile on fp16 operands (v_mfma_f32_16x16x32_f16).
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mfma(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// FP32 MFMA tile (v_mfma_f32_16x16x4_f32): lane l holds A[l & 15][l >> 4] and
// B[l >> 4][l & 15]; accumulator layout as above.
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier for LDS traffic: waits for this wave's LDS operations and
// then for every wave. Unlike __syncthreads() it does not drain the wave's
// outstanding global loads and stores, so register prefetches and
// global-to-LDS copies stay in flight across it. LDS data written by
// global-to-LDS loads is covered by vmcnt, not by this barrier: wait for it
// (vmcnt) before the barrier that publishes it. The memory clobber keeps the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Waits for every outstanding vector memory operation of this wave (loads,
// stores and global-to-LDS copies). It is the s_waitcnt builtin, not inline
// assembly, so the compiler's own wait insertion knows that everything issued
// before it has completed: later uses of registers loaded before it need no
// further wait. (Inline assembly is opaque to that pass, which then waits
// again at the first use, for every load in flight at that point, prefetches
// included, whenever loads and stores are both outstanding.)
// Encoding: vmcnt 0, expcnt 7 and lgkmcnt 15 (no wait on those).
__device__ __forceinline__ void vm_drain() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// The lane index, opaque to the optimizer. Kernels call it at the start of
// each phase so per-lane LDS addresses are rebuilt where they are used:
// LDS arrays above 64 KB cannot use the 16-bit instruction offset, and
// otherwise every (lane, constant) address would be hoisted out of the chunk
// loop and kept live across it.
__device__ __forceinline__ int fresh_lane() {
  int l = __lane_id();
  asm volatile("" : "+v"(l));
  return l;
}

// float -> bf16 with round-to-nearest-even; exact split x = hi + lo + O(2^-17 x).
__device__ __forceinline__ bf16 to_bf16(float x) { return static_cast<bf16>(x); }
__device__ __forceinline__ float from_bf16(bf16 x) { return static_cast<float>(x); }
__device__ __forceinline__ void split2(float x, bf16& hi, bf16& lo) {
  hi = to_bf16(x);
  lo = to_bf16(x - from_bf16(hi));
}

// Paired-tile K order: a 32-deep K step built from two vertically adjacent
// accumulator tiles t0 (rows 0..15 of the step) and t1 (rows 16..31). Lane
// group grp holds rows 4*grp..4*grp+3 of each, so B element e maps to K row
//   e < 4: 4*grp + e        e >= 4: 16 + 4*grp + (e - 4).
// The matching A operand reads A[m][k0 + 4*grp .. +3] and A[m][k0 + 16 + 4*grp .. +3].
__device__ __forceinline__ bf16x8 pack_pair(const f32x4& t0, const f32x4& t1) {
  bf16x8 r;
  r[0] = to_bf16(t0[0]); r[1] = to_bf16(t0[1]); r[2] = to_bf16(t0[2]); r[3] = to_bf16(t0[3]);
  r[4] = to_bf16(t1[0]); r[5] = to_bf16(t1[1]); r[6] = to_bf16(t1[2]); r[7] = to_bf16(t1[3]);
  return r;
}
// The hi values are rounded once, as packed pairs; each one's FP32 value for
// the remainder is then a half of its packed word (bf16 is the upper half of
// an FP32 pattern).
__device__ __forceinline__ void pack_pair_split(const f32x4& t0, const f32x4& t1,
                                                bf16x8& hi, bf16x8& lo) {
  typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
  hi = pack_pair(t0, t1);
  const u32x4v hw = __builtin_bit_cast(u32x4v, hi);
  float hv[8];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    hv[2 * p] = __builtin_bit_cast(float, hw[p] << 16);
    hv[2 * p + 1] = __builtin_bit_cast(float, hw[p] & 0xFFFF0000u);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lo[e] = to_bf16(t0[e] - hv[e]);
    lo[e + 4] = to_bf16(t1[e] - hv[e + 4]);
  }
}

// Paired storage order: within each 32-wide block of a row, logical index
// 16 h + 4 g + e is stored at 8 g + 4 h + e. The paired-tile K order above
// then reads 8 contiguous elements (lds_nat at k0 + 8 grp). Any product whose
// two operands are both stored this way along the contraction index is
// unchanged, so a matrix can be kept in one order for every use.
__device__ __forceinline__ int pperm(int k) {
  return (k & ~31) + 8 * ((k & 15) >> 2) + 4 * ((k >> 4) & 1) + (k & 3);
}

// Column reads of a row-major bf16 LDS matrix by the transposing LDS read
// (ds_read_b64_tr_b16). Within each group of 16 lanes, lane j receives as
// element e the element (j & 3) of the 8 bytes that lane 4 e + (j >> 2)
// addresses (established on gfx950 with an in-LDS index pattern). So if lane
// i of the group addresses row r + (i >> 2), columns c + 4 (i & 3) .. + 3, lane
// j receives column c + j of rows r .. r + 3: the accumulator layout of a
// 16x16 tile, or half of a paired-order operand. Every lane of the wave must
// be active, and ld must be a multiple of 4 elements (8-byte alignment).
// lds_col4: lane (r16, grp) gets m[r0 + 4 grp + e][c0 + r16], e = 0..3.
__device__ __forceinline__ bf16x4 lds_col4(const bf16* m, int ld, int r0, int c0, int r16, int grp) {
  typedef short s16x4v __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4v* lds_s16x4;
  const bf16* p = m + (r0 + 4 * grp + (r16 >> 2)) * ld + c0 + 4 * (r16 & 3);
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(const_cast<bf16*>(p))));
}
// lds_col8: paired order over rows r0 .. r0 + 31 (rows r0 + 4 grp + e, then
// r0 + 16 + 4 grp + e) of column c0 + r16.
__device__ __forceinline__ bf16x8 lds_col8(const bf16* m, int ld, int r0, int c0, int r16, int grp) {
  const bf16x4 a = lds_col4(m, ld, r0, c0, r16, grp), b = lds_col4(m, ld, r0 + 16, c0, r16, grp);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// The accumulator tile (rows r0 .. r0 + 15, columns c0 .. c0 + 15) as FP32 (exact).
__device__ __forceinline__ f32x4 lds_tile(const bf16* m, int ld, int r0, int c0, int r16, int grp) {
  const bf16x4 a = lds_col4(m, ld, r0, c0, r16, grp);
  return f32x4{from_bf16(a[0]), from_bf16(a[1]), from_bf16(a[2]), from_bf16(a[3])};
}

// LDS operand loads (bf16 elements, row-major with row stride `ld`).
// Natural K order: 8 contiguous elements at A[row][k0 + 8*grp].
__device__ __forceinline__ bf16x8 lds_nat(const bf16* base, int row, int ld, int k0, int grp) {
  return *reinterpret_cast<const bf16x8*>(base + row * ld + k0 + 8 * grp);
}
// Paired-tile K order: elements k0 + 4*grp + 0..3 and k0 + 16 + 4*grp + 0..3.
__device__ __forceinline__ bf16x8 lds_pair(const bf16* base, int row, int ld, int k0, int grp) {
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(base + row * ld + k0 + 4 * grp);
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(base + row * ld + k0 + 16 + 4 * grp);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// ---------------------------------------------------------------- reductions
// A float moved between lanes by a DPP pattern within rows of 16 lanes
// (CTRL: quad_perm 0x00..0xFF, row_mirror 0x140, row_half_mirror 0x141).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float read_lane(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
// Maximum over the 64 lanes (all active), in every lane. DPP within each row
// of 16 lanes, then the four row maxima through scalar registers: no LDS
// round trip (a shuffle through the LDS crossbar costs a full LDS latency per
// step). The maximum is exact in any order.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));                   // quad_perm [1, 0, 3, 2]
  x = fmaxf(x, dpp_f<0x4E>(x));                   // quad_perm [2, 3, 0, 1]
  x = fmaxf(x, dpp_f<0x141>(x));                  // lanes i, 7 - i of each 8
  x = fmaxf(x, dpp_f<0x140>(x));                  // lanes i, 15 - i of each 16
  return fmaxf(fmaxf(read_lane(x, 0), read_lane(x, 16)), fmaxf(read_lane(x, 32), read_lane(x, 48)));
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, WAVE);
  return x;
}
// A float moved by a DPP pattern with a row mask (rows the mask leaves out,
// and lanes without a source, read 0).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_rows(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xF, false));
}
// Inclusive prefix sum over the 64 lanes of a wave, all in registers:
// shifts by 1, 2, 4, 8 within each row of 16 lanes (row_shr), then each
// row's total carried forward (lane 15 to row 1 and lane 47 to row 3 by
// row_bcast:15; lane 31 to rows 2 and 3 by row_bcast:31).
__device__ __forceinline__ float wave_incl_scan(float x) {
  x += dpp_rows<0x111, 0xF>(x);
  x += dpp_rows<0x112, 0xF>(x);
  x += dpp_rows<0x114, 0xF>(x);
  x += dpp_rows<0x118, 0xF>(x);
  x += dpp_rows<0x142, 0xA>(x);
  x += dpp_rows<0x143, 0xC>(x);
  return x;
}

// ---------------------------------------------------------------- QDQ (FP32)
// Formats as in gdn.h: 1 = E4M3FN (+-448), 2 = INT8 ([-127, 127]).
template <int FMT> struct QdqFmt;
template <> struct QdqFmt<1> { static constexpr float qmax = 448.f; };
template <> struct QdqFmt<2> { static constexpr float qmax = 127.f; };

// E4M3 rounding: nearest OCP E4M3FN value (bias 7, 3 mantissa bits,
// subnormal step 2^-9), ties to even, saturating at +-448. Done with the
// hardware round trip of two values: v_cvt_pk_fp8_f32 rounds to nearest even
// and v_cvt_f32_fp8 is exact. For |y| < 464 this equals the definition bit
// for bit (checked over every such FP32 pattern on gfx950); above 464 the
// hardware gives NaN instead of saturating, so inputs are clamped to +-448
// first (448 < |y| < 464 rounds to 448 either way).
// `bytes` receives the two one-byte codes in bits 0..15.
__device__ __forceinline__ void e4m3_pair(float y0, float y1, float& c0, float& c1,
                                          uint32_t& bytes) {
  y0 = __builtin_amdgcn_fmed3f(y0, -448.f, 448.f);
  y1 = __builtin_amdgcn_fmed3f(y1, -448.f, 448.f);
  bytes = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false)) & 0xFFFFu;
  c0 = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(bytes), 0);
  c1 = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(bytes), 1);
}

__device__ __forceinline__ float round_int8(float y) {
  return fminf(fmaxf(rintf(y), -127.f), 127.f);
}
// Codes of four values x * r (one accumulator quad), and their bytes, where
// r = fl(1/d) and d is derived from the maximum |x| of the values' own tile:
// then |fl(x r)| <= q_max (1 + 4 * 2^-24) (d >= amax / q_max (1 - 2^-24),
// r <= (1 / d)(1 + 2^-24)), so no clamp is needed before the conversion:
// E4M3 values below 464 round to at most 448 (the hardware gives NaN only
// from 464 up), and rint of |y| < 127.5 is at most 127. The two E4M3 pairs
// are converted into the low and high halves of one word.
template <int FMT> __device__ __forceinline__ void quant4(const float (&x)[4], float r,
                                                          float (&c)[4], uint32_t& bytes) {
  if constexpr (FMT == 1) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[0] * r, x[1] * r, 0, false);
    bytes = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(x[2] * r, x[3] * r, lo, true));
    c[0] = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(bytes), 0);
    c[1] = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(bytes), 1);
    c[2] = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(bytes), 2);
    c[3] = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(bytes), 3);
  } else {
    bytes = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = rintf(x[i] * r);
      bytes |= (static_cast<uint32_t>(static_cast<int8_t>(c[i])) & 0xFFu) << (8 * i);
    }
  }
}

// Scale from the tile amax: d = max(fl(amax / qmax), 2^-126) (IEEE division).
template <int FMT> __device__ __forceinline__ float qdq_scale(float amax) {
  const float d = amax / QdqFmt<FMT>::qmax;
  return fmaxf(d, 1.17549435e-38f);
}
// Stores that a kernel running at the same time reads after a ready flag.
// With coh set they are device-scope stores (sc1: written through to the
// device's coherence point, leaving no dirty L2 line behind), so waiting for
// them (vmcnt) before the flag makes them visible on every XCD; a release
// fence would instead write back the whole L2 (buffer_wbl2), which took
// about 40 us per item in the forward's operand build. Otherwise plain
// stores.
__device__ __forceinline__ void st_out(float* p, float v, bool coh) {
  if (coh) __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __builtin_bit_cast(uint32_t, v),
                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
// 16 bytes at base + off (base wave-uniform, off < 2^31): a device-scope
// buffer store (one instruction, cache policy sc1) or a plain store.
__device__ __forceinline__ void st_out16(void* base, int off, u32x4 v, bool coh) {
  if (coh) {
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7FFFFFF0, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, off, 0, 16);
  } else {
    *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(base) + off) = v;
  }
}

}  // namespace gdn
