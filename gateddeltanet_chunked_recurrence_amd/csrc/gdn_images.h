// Operand images exchanged between the forward's two kernels.
//
// The prep kernel (one workgroup per chunk and head) writes, for every chunk
// and head, the state-independent operands of the state kernel in exactly the
// layout the state kernel keeps in LDS, so that kernel stages them with plain
// 16-byte copies:
//   W image  [64][DK] bf16 per plane: W^q codes (one plane) or W as hi + lo
//            (two planes), paired order along dk (pperm), 16-byte chunks
//            XOR-swizzled by row for DK = 128 (rows padded to 72 for DK = 64).
//            With both QDQ sites on, the plane holds the code bytes instead
//            (the same element order, in the first WQ bytes of the plane's
//            slot), and the state kernel widens them to bf16 per fragment.
//            In that variant P is one fp16 plane and the gate block follows
//            it (in the second P plane's slot), so K^T, P and the gates are
//            one contiguous range
//   K^T image [DK][64] bf16: K transposed, paired order along tokens
//   P image  2 x [64][64] bf16: (Q K^T) * Gam as hi + lo, paired order along
//            the key token; upper 16x16 tiles zero (one fp16 plane in the
//            byte variant above)
//            (both [*][64] images unpadded, 16-byte pieces XOR-swizzled by
//            row, see r64_off)
//   U        FP32 in accumulator-fragment order: for value block vb, wave w,
//            row tile mt and lane l the four values U[16 mt + 4 (l >> 4) + i]
//            [64 vb + 16 w + (l & 15)], i = 0..3, contiguous
//   gates    256 FP32: exp(gamma_i) at [i], exp(gamma_n - gamma_i) at [64 + i]
//            (0 past the chunk end), exp(gamma_n) at [128], the W scale at
//            [129], rest unused
//   W scale  one FP32 per chunk and head (1 when W QDQ is off), also in a
//            separate array
// The W, K^T, P and gate images of one chunk and head are one contiguous
// block, in that order, as they are in the state kernel's LDS buffer (in the
// byte variant that buffer holds the code bytes, padded to whole 1 KB
// copies, then K^T, the fp16 P plane and the gates).
// The Q operand of the state kernel uses the W image layout and is staged
// from q directly.
#pragma once
#include "gdn_device.h"

namespace gdn {

template <int DK>
struct Img {
  static constexpr int RS = DK == 128 ? 128 : 72;   // row stride of [64][DK] images
  static constexpr int SWZ = DK == 128 ? 15 : 0;    // 16-byte chunk swizzle mask
  static constexpr int R64 = 72;                    // row stride of padded [*][64] tiles
  static constexpr int WQ = 64 * RS;                // elements of one [64][DK] plane
  static constexpr int KT = DK * 64;                // elements of the K^T image (r64_off)
  static constexpr int P1 = 64 * 64;                // elements of one P plane (r64_off)
  static constexpr int GB = 512;                    // gate block: 256 FP32 (1 KB)
  // one (slot, head) block: [W planes | K^T | P hi, P lo | gates], contiguous
  template <int NW> static constexpr int img() { return NW * WQ + KT + 2 * P1 + GB; }
  template <int NW> static constexpr int kt_at() { return NW * WQ; }
  template <int NW> static constexpr int p_at() { return NW * WQ + KT; }
  template <int NW> static constexpr int g_at() { return NW * WQ + KT + 2 * P1; }
};

// Element offset of stored (pperm) position s in row `row` of a [64][DK] image.
template <int DK>
__device__ __forceinline__ int wq_off(int row, int s) {
  using I = Img<DK>;
  return row * I::RS + ((((s >> 3) ^ (row & I::SWZ))) << 3) + (s & 7);
}

// Element offset of stored (pperm) position s in row `row` of an unpadded
// [*][64] image: row r's 16-byte pieces are XOR-swizzled by (r >> 1) & 7, so
// the 16 rows of one operand fragment read at one piece position hit 16
// distinct 16-byte bank groups (two 128-byte rows span all 64 banks).
__device__ __forceinline__ int r64_off(int row, int s) {
  return row * 64 + ((((s >> 3) ^ ((row >> 1) & 7))) << 3) + (s & 7);
}
// Operand fragment (row `row`, stored positions k0 + 8 grp..+7) of such an image.
__device__ __forceinline__ bf16x8 ld_r64(const bf16* img, int row, int k0, int grp) {
  return *reinterpret_cast<const bf16x8*>(img + r64_off(row, k0 + 8 * grp));
}

// A-operand fragment (16 rows from `row0`, stored K positions 32 kk + 8 grp..+7)
// of a [64][DK] image.
template <int DK>
__device__ __forceinline__ bf16x8 ld_wq(const bf16* img, int row, int kk, int grp) {
  return *reinterpret_cast<const bf16x8*>(img + wq_off<DK>(row, 32 * kk + 8 * grp));
}

// The chunk of a slot (slot = n + bos_n / 64 + c, increasing in n; see
// gdn.h): sequence n, chunk c, first token t0 and length nc; `valid` is false
// for the spare slot after each sequence's last chunk.
struct Chunk {
  int n, c, t0, nc;
  bool valid;
};
__device__ inline Chunk locate_slot(int slot, const int32_t* cu, int N, int T, int prefix_len) {
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const int bos = cu ? cu[mid] : mid * T;
    if (mid + bos / CHUNK <= slot) lo = mid; else hi = mid - 1;
  }
  const int bos = cu ? cu[lo] : lo * T;
  int eos = cu ? cu[lo + 1] : (lo + 1) * T;
  if (prefix_len > 0) eos = min(eos, bos + prefix_len);   // prefix cap (see seq_span)
  Chunk ch;
  ch.n = lo;
  ch.c = slot - (lo + bos / CHUNK);
  ch.t0 = bos + CHUNK * ch.c;
  ch.nc = min(CHUNK, eos - ch.t0);
  ch.valid = ch.c >= 0 && ch.t0 < eos;
  return ch;
}

// Float offset of the U fragment (ch, vb, w, mt) of lane `lane`.
__device__ __forceinline__ int64_t u_off(int64_t ch, int nvb, int vb, int w, int mt, int lane) {
  return ((((ch * nvb + vb) * 4 + w) * 4 + mt) * 64 + lane) * 4;
}

// Fragment order of an FP32 [MT * 16, Dv] matrix per (slot, head) `ch`: the
// accumulator tile (row tile mt, value block vb, 16-column group w) of lane
// `lane` is four contiguous floats, element i at row 16 mt + 4 (lane >> 4) + i,
// column 64 vb + 16 w + (lane & 15). The two column groups of a 32-column
// range are adjacent, so a consumer reads them as one contiguous block.
__device__ __forceinline__ int64_t frag_off(int64_t ch, int nvb, int vb, int w, int MT, int mt,
                                            int lane) {
  return (((((ch * nvb + vb) * 4 + w) * MT + mt) * 64) + lane) * 4;
}

}  // namespace gdn
