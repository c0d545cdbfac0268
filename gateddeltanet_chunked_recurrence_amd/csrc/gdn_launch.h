// Internal launch interface between the C-ABI layer (gdn_abi.cpp) and the
// HIP kernels. Plain C types only; all pointers are device pointers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

struct FwdKernelArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const float* h0;            // nullable
  const int32_t* cu_seqlens;  // nullable
  void* o;
  float* ht;                  // nullable
  uint8_t* s_codes;           // saved state codes (state QDQ on), nullable
  float* s_f32;               // saved FP32 state (state QDQ off), nullable
  float* s_scale;             // saved state scales, nullable
  uint8_t* w_codes;           // saved W codes (W QDQ on), nullable
  float* w_scale;             // saved W scales, nullable
  float* s_X;                 // saved X = (I + L)^-1 per chunk (bf16 io), nullable
  uint32_t* s_meta;           // saved policy stamp (SavedStamp words), nullable
  float* s_anchor;            // saved FP32 state of each chunk (two-precision profile), nullable
  uint32_t* err;              // sticky device error flags (kErr* bits), never NULL
  // forward workspace (bf16 io): operand images written by the prep kernel
  __bf16* ws_img;             // [slots * Hv][W planes | K^T | P] (gdn_images.h)
  float* ws_u;                // [slots * Hv][Dv * 64] fragment order
  float* ws_wscale;           // [slots * Hv]
  int32_t w_img_bytes;        // 1: the W plane of the images holds code bytes (both QDQ sites on)
  // overlapped forward (gdn_chunk_fwd with equal-length sequences): the prep
  // kernel runs items [item_lo, item_hi) of the chunk-major order (chunk c of
  // every sequence and head before chunk c + 1) and, when flags is set (a
  // state kernel runs meanwhile), stores its outputs at device scope, drains
  // them and then sets each item's flag [slot * Hv + head]; the state kernel
  // waits for the flag of every chunk
  uint32_t* flags;            // nullable
  uint32_t* ticket;           // nullable: items are taken from this counter (zeroed per call), so
                              // the resident workgroups always hold the lowest items left; with
                              // prep_rest > 0, [0] over the items below item_split (every
                              // workgroup), then [1] over the rest (only workgroups below
                              // prep_rest: the others end, and free their CUs)
  int32_t item_split, prep_rest;
  // nullable: with two prep workgroups per CU, the rest is built on whole
  // CUs: the first of a CU's workgroups to reach it admits the CU or not
  // (prep_rest CUs in all, spread evenly over the XCCs and their shader
  // engines), and the other follows; kAdmitWords words zeroed per call (per
  // XCC: one slot per CU key, then the count admitted per engine)
  uint32_t* admit;
  // packed sequences (cu_seqlens): the chunk-major order comes from a table
  // that varlen_setup_kernel builds from the lengths: [0] items, [1] the head
  // (taking the place of item_split), then per item (n Hv + head, chunk)
  const int32_t* vplan;       // nullable
  int32_t item_lo, item_hi;   // item_hi == 0: every slot-major item [0, slots * Hv)
  int32_t chunk_major;        // 1: items in chunk-major order (no cu_seqlens)
  int32_t prep_blocks;        // prep grid size (0: one workgroup per CU)
  int32_t solve_degree;       // 0: exact (I + L)^-1; else the Neumann polynomial of this degree (2^j - 1)
  int32_t T;                  // tokens per sequence (no cu_seqlens)
  int32_t prefix_len;         // > 0: only the first prefix_len tokens of every sequence
  int32_t Hqk, Hv, Dv, block_v;
  float scale;
};

// Tokens [bos, eos) of sequence n that the chunk path runs over: the whole
// sequence, or its first prefix_len tokens when that is set.
__device__ __forceinline__ void seq_span(const FwdKernelArgs& a, int n, int& bos, int& eos) {
  if (a.cu_seqlens) {
    bos = a.cu_seqlens[n];
    eos = a.cu_seqlens[n + 1];
  } else {
    bos = n * a.T;
    eos = bos + a.T;
  }
  if (a.prefix_len > 0) eos = min(eos, bos + a.prefix_len);
}

// Whether packed token `tok` lies in the span seq_span gives its sequence.
__device__ inline bool token_in_span(const FwdKernelArgs& a, int N, int tok) {
  if (a.prefix_len <= 0) return true;
  int bos;
  if (a.cu_seqlens) {
    int lo = 0, hi = N - 1;          // last sequence starting at or before tok
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.cu_seqlens[mid] <= tok) lo = mid; else hi = mid - 1;
    }
    bos = a.cu_seqlens[lo];
  } else {
    bos = tok - tok % a.T;
  }
  return tok - bos < a.prefix_len;
}

// Bits of the sticky device error word (gdn_device_errors in gdn.h).
constexpr uint32_t kErrLdsWait = 1u;      // a bounded LDS-counter wait gave up
constexpr uint32_t kErrFlagWait = 2u;     // a bounded wait on another workgroup gave up
constexpr uint32_t kErrSavedStamp = 4u;   // saved buffer written under another policy or shape
constexpr uint32_t kErrPRange = 8u;       // a masked Q K^T entry beyond the fp16 range

// The policy and shape a forward wrote its saved buffer under; the backward
// compares it with its own arguments on the device.
struct SavedStamp {
  static constexpr uint32_t kMagic = 0x53444E47u;   // "GDNS"
  uint32_t w[16];
};

struct FwdConfig {
  int Dk, Dv, N, Hv, state_fmt, w_fmt, f32_io;
  int block_v;                // state scale tile width (state QDQ on)
  int read_fmt;               // two-precision read copy format (0 off, 1 E4M3)
};

// FP32 io (Dk = 64): one fused kernel per (sequence, head, value block).
hipError_t launch_fwd_fused(const FwdConfig& cfg, const FwdKernelArgs& a, hipStream_t stream);
// bf16 io: prep kernel over every (chunk, head), then the state kernel.
// stop (nullable): an event that the launch itself records at its end, with
// no marker of its own on the stream
constexpr int kAdmitPerXcc = 256 + 8;
constexpr int kAdmitWords = 8 * kAdmitPerXcc;
// Prep workgroups that can share a CU: 2 where an item's compact LDS layout
// fits in half of it (Dv <= 128, exact solve), else 1.
int prep_workgroups_per_cu(const FwdConfig& cfg, int solve_degree);
hipError_t launch_fwd_prep(const FwdConfig& cfg, const FwdKernelArgs& a, int num_slots,
                           hipStream_t stream, hipEvent_t stop = nullptr);
hipError_t launch_fwd_state(const FwdConfig& cfg, const FwdKernelArgs& a, hipStream_t stream,
                            hipEvent_t stop = nullptr);
// Both QDQ sites on: recurrence and output in separate waves (gdn_fwd_state_split.hip).
hipError_t launch_fwd_state_split(const FwdConfig& cfg, const FwdKernelArgs& a, hipStream_t stream,
                                  hipEvent_t stop = nullptr);

struct BwdKernelArgs {
  FwdKernelArgs f;            // forward inputs + saved buffers (read only here)
  const void* dout;
  const float* dht;           // nullable
  void* dq;
  void* dk;
  void* dv;
  float* dg;
  float* dbeta;
  float* dh0;                 // nullable
  float* ws_X;                // [num_slots, Hv, 64, 64] FP32: X = (I + L)^-1 per chunk
  float* ws_W;                // [B*T, Hv, Dk] FP32: the W used in the products (Wq or W)
  float* ws_dstate;           // [num_slots, Hv] x [Dk, Dv] FP32 fragment order: dL/dS at each chunk end
  float* ws_dvn;              // [num_slots, Hv] x [64, Dv] FP32 fragment order: dL/dVnew per chunk
  // bf16 io: operands of the reverse recurrence, written by bwd_img_kernel
  __bf16* ws_bimg;            // [num_slots * Hv][K image | W^T planes | gates] (gdn_bwd_state.hip)
  float* ws_a1;               // [num_slots * Hv] x [64, Dv] fragment order: scale P^T dO
  float* ws_a2;               // [num_slots * Hv] x [Dk, Dv] fragment order: scale (e^gamma Q)^T dO
  float* ws_dqk;              // [B*T, Hv, 2, Dk] FP32 per-value-head dq, dk before the group sum
  float* ws_dX;               // [num_slots, Hv, 64, 64] FP32 dL/dX per chunk (approximate inverse only)
  // overlapped backward (bf16 io, equal-length sequences): bwd_img_kernel
  // runs its items in reverse chunk-major order (the last chunk of every
  // sequence and head first) beside bwd_state_kernel, storing at device
  // scope and setting flags[slot * Hv + head] after each item; the state
  // kernel waits for each chunk's flag
  uint32_t* flags;            // nullable
  int32_t rev_maxc;           // > 0: chunks per sequence, and bwd_img_kernel runs items
  int32_t rev_lo, rev_hi;     // [rev_lo, rev_hi) of that order, one workgroup each
  int32_t rev_done;           // the last rev_done chunks of every sequence were built before
  int32_t grad_f32;
  int32_t total_tokens;
  int32_t num_slots;
};

struct BwdConfig {
  int Dk, Dv, N, Hv, Hqk, state_fmt, w_fmt, f32_io;
};

// The second stream and the fork / join events of an overlapped backward
// (a.flags set): the flag reset records fork, the image kernel runs on s2
// after it and records join, and `stream` waits for join before the
// chunk-local kernels.
struct BwdOverlap {
  hipStream_t s2;
  hipEvent_t fork, join;
};
hipError_t launch_bwd(const BwdConfig& cfg, const BwdKernelArgs& a, hipStream_t stream,
                      const BwdOverlap* ov = nullptr);
// Whether the image kernel and the state kernel of this backward fit on one
// CU together (LDS), with the state kernel's grid at most one workgroup per
// CU: then some CU always has room for an image workgroup while every state
// workgroup is resident, and the overlapped backward cannot stall.
bool bwd_overlap_fits(const BwdConfig& cfg);
// Compute units of the current device (queried once per device).
int device_cus();
// bf16 io: operand images of the reverse recurrence, then the recurrence.
hipError_t launch_bwd_img(const BwdConfig& cfg, const BwdKernelArgs& a, hipStream_t stream,
                          hipEvent_t stop = nullptr);
hipError_t launch_bwd_state(const BwdConfig& cfg, const BwdKernelArgs& a, hipStream_t stream);
// bf16 io: the chunk-local gradients on bf16 MFMA.
hipError_t launch_bwd_local(const BwdConfig& cfg, const BwdKernelArgs& a, hipStream_t stream);
// Elements of the backward image block of one (slot, head).
int bwd_img_elems(int Dk, int w_fmt);

// Two-precision profile backward: dg += exp(gamma_n) <dS', S - Sr> over each
// chunk (the FP32 carry's gate term, which the backward's products took with
// the read copy Sr).
hipError_t launch_bwd_read_anchor(const BwdConfig& cfg, const BwdKernelArgs& a, hipStream_t s);

// Sets n words to v (a fill kernel: safe under graph capture, unlike a memset node).
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s, hipEvent_t stop = nullptr);
// Overlapped forward over packed sequences: zeroes the n words at `zero` (the
// ready flags and item counters) and writes the prep's item table to `plan`
// (see FwdKernelArgs::vplan): chunk-major, the sequences of each chunk index
// longest first, and the head split H = items - rest maxc / item_per_chunk in
// whole rounds of `cus` items (0 when negative, all items when past them).
// Needs num_seqs <= 1024 and at most 4095 chunks per sequence.
hipError_t launch_varlen_setup(uint32_t* zero, int64_t n, int32_t* plan, const int32_t* cu_seqlens,
                               int num_seqs, int prefix_len, int Hv, int cus, int rest,
                               float item_per_chunk, hipStream_t s, hipEvent_t stop);

// Writes the stamp into the saved buffer's meta section.
hipError_t launch_write_stamp(uint32_t* meta, const SavedStamp& st, hipStream_t s);
// After the backward's kernels: if the saved stamp differs from `want`, sets
// kErrSavedStamp and overwrites every gradient output with NaN.
hipError_t launch_check_stamp(const BwdKernelArgs& a, const SavedStamp& want, int64_t n_dqk,
                              int64_t n_dv, int64_t n_tok, int64_t n_h0, hipStream_t s);

hipError_t launch_qdq_state(const float* x, float* y, float* scales, uint8_t* codes,
                            int64_t n_states, int Dk, int Dv, int block_v, int fmt,
                            hipStream_t stream);

// Decode continuation (gdn_decode.hip): token-state writes through the state
// quantizer, forward and straight-through backward.
struct DecodeKernelArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const float* h_in;          // nullable (zero state)
  const int32_t* cu_seqlens;  // nullable
  void* o;
  float* ht;                  // nullable
  uint8_t* s_codes;           // saved written states (state QDQ on), nullable
  float* s_scale;             // their tile scales, nullable
  float* s_f32;               // saved written states (state QDQ off), nullable
  int32_t T, start, Hqk, Hv, Dv, block_v, readout;
  int32_t num_seqs;
  float scale;
  // backward
  const void* dout;
  const float* dht;           // nullable
  void* dq;
  void* dk;
  void* dv;
  float* dg;
  float* dbeta;
  float* dh_in;               // nullable
  float* ws_dqk;              // [B*T, Hv, 2, Dk] FP32 when Hv > Hqk, else NULL
  int32_t grad_f32;
  int32_t total_tokens;
};

struct DecodeConfig {
  int Dk, Dv, N, Hv, Hqk, state_fmt, f32_io;
};

// 64-column slabs per decode workgroup: those of one state scale tile.
inline int decode_slabs_per_group(int state_fmt, int block_v) {
  return state_fmt != 0 && block_v > 64 ? block_v / 64 : 1;
}

hipError_t launch_decode_fwd(const DecodeConfig& c, const DecodeKernelArgs& a, hipStream_t s);
hipError_t launch_decode_bwd(const DecodeConfig& c, const DecodeKernelArgs& a, hipStream_t s);

}  // namespace gdn
