// Saved-buffer policy stamp. The forward writes the policy and shape it ran
// under into the saved buffer; after the backward's kernels, one check
// compares the stamp with the backward's own arguments. On a mismatch (for
// example a saved buffer written with the approximate inverse read back by
// an exact-solve backward) every gradient output becomes NaN and the sticky
// error word records it, so a wrong pairing never passes silently ("[7/7]
// Experimental GDN/KDA approximate-inverse QAT", "What does this PR do?": no
// silent change of degree and no fallback).
#include <hip/hip_ext.h>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

__global__ void write_stamp_kernel(uint32_t* meta, SavedStamp st) {
  const int i = threadIdx.x;
  if (i < 16) meta[i] = st.w[i];
}

__device__ __forceinline__ bool stamp_differs(const uint32_t* meta, const SavedStamp& want) {
  bool bad = false;
#pragma unroll
  for (int i = 0; i < 16; ++i) bad |= meta[i] != want.w[i];
  return bad;
}

template <typename T>
__device__ void fill_nan(T* p, int64_t n) {
  const T v = static_cast<T>(__builtin_nanf(""));
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ void check_stamp_kernel(BwdKernelArgs a, SavedStamp want, int64_t n_dqk, int64_t n_dv,
                                   int64_t n_tok, int64_t n_h0) {
  if (!stamp_differs(a.f.s_meta, want)) return;   // the common case: one read per workgroup
  if (blockIdx.x == 0 && threadIdx.x == 0)
    __hip_atomic_fetch_or(a.f.err, kErrSavedStamp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (a.grad_f32) {
    fill_nan(reinterpret_cast<float*>(a.dq), n_dqk);
    fill_nan(reinterpret_cast<float*>(a.dk), n_dqk);
    fill_nan(reinterpret_cast<float*>(a.dv), n_dv);
  } else {
    fill_nan(reinterpret_cast<bf16*>(a.dq), n_dqk);
    fill_nan(reinterpret_cast<bf16*>(a.dk), n_dqk);
    fill_nan(reinterpret_cast<bf16*>(a.dv), n_dv);
  }
  fill_nan(a.dg, n_tok);
  fill_nan(a.dbeta, n_tok);
  if (a.dh0) fill_nan(a.dh0, n_h0);
}

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// Zeroes n words at `zero` (grid-strided) and, in workgroup 0, builds the
// overlapped forward's item table for packed sequences from their lengths.
constexpr int kMaxSeqs = 1024, kMaxChunks = 4096;
__global__ void __launch_bounds__(256) varlen_setup_kernel(uint32_t* zero, int64_t n, int32_t* plan,
                                                           const int32_t* cu, int N, int prefix_len,
                                                           int Hv, int cus, int rest, float ipc) {
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) zero[i] = 0u;
  if (blockIdx.x != 0) return;
  __shared__ int nc[kMaxSeqs], perm[kMaxSeqs], first[kMaxChunks + 1], mx;
  const int tid = threadIdx.x;
  if (tid == 0) mx = 0;
  __syncthreads();
  for (int s = tid; s < N; s += 256) {          // chunks of each sequence (prefix cap)
    int len = cu[s + 1] - cu[s];
    if (prefix_len > 0) len = min(len, prefix_len);
    nc[s] = (len + 63) / 64;
    atomicMax(&mx, nc[s]);
  }
  __syncthreads();
  const int maxc = mx;
  for (int s = tid; s < N; s += 256) {          // longest first, ties in sequence order
    int r = 0;
    for (int m = 0; m < N; ++m) r += nc[m] > nc[s] || (nc[m] == nc[s] && m < s);
    perm[r] = s;
  }
  for (int c = tid; c <= maxc; c += 256) {      // items of the chunk indices below c
    int k = 0;
    for (int m = 0; m < N; ++m) k += min(nc[m], c);
    first[c] = k * Hv;
  }
  __syncthreads();
  const int items = first[maxc];
  int32_t* tab = plan + 4;
  for (int i = tid; i < items; i += 256) {
    int lo = 0, hi = maxc - 1;                  // the chunk index c with first[c] <= i < first[c + 1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (first[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const int idx = i - first[lo];              // (rank among the sequences that reach chunk lo, head)
    tab[2 * i] = perm[idx / Hv] * Hv + idx % Hv;
    tab[2 * i + 1] = lo;
  }
  if (tid == 0) {
    const double h = (double)items - (double)rest * maxc / ipc;
    int head = h <= 0.0 ? 0 : (int)(h / cus + 0.5) * cus;
    if (head > items) head = items;
    plan[0] = items;
    plan[1] = head;
  }
}

}  // namespace

hipError_t launch_varlen_setup(uint32_t* zero, int64_t n, int32_t* plan, const int32_t* cu_seqlens,
                               int num_seqs, int prefix_len, int Hv, int cus, int rest,
                               float item_per_chunk, hipStream_t s, hipEvent_t stop) {
  if (num_seqs < 1 || num_seqs > kMaxSeqs) return hipErrorInvalidValue;
  const int64_t blocks = (n + 255) / 256 < 1024 ? ((n + 255) / 256 > 0 ? (n + 255) / 256 : 1) : 1024;
  if (stop)
    hipExtLaunchKernelGGL(varlen_setup_kernel, dim3((unsigned)blocks), dim3(256), 0, s, nullptr, stop, 0,
                          zero, n, plan, cu_seqlens, num_seqs, prefix_len, Hv, cus, rest, item_per_chunk);
  else
    hipLaunchKernelGGL(varlen_setup_kernel, dim3((unsigned)blocks), dim3(256), 0, s, zero, n, plan,
                       cu_seqlens, num_seqs, prefix_len, Hv, cus, rest, item_per_chunk);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s, hipEvent_t stop) {
  if (n <= 0) return stop ? hipEventRecord(stop, s) : hipSuccess;
  const int64_t blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  if (stop)
    hipExtLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, nullptr, stop, 0, p, n, v);
  else
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_write_stamp(uint32_t* meta, const SavedStamp& st, hipStream_t s) {
  hipLaunchKernelGGL(write_stamp_kernel, dim3(1), dim3(64), 0, s, meta, st);
  return hipGetLastError();
}

hipError_t launch_check_stamp(const BwdKernelArgs& a, const SavedStamp& want, int64_t n_dqk,
                              int64_t n_dv, int64_t n_tok, int64_t n_h0, hipStream_t s) {
  hipLaunchKernelGGL(check_stamp_kernel, dim3(256), dim3(256), 0, s, a, want, n_dqk, n_dv, n_tok,
                     n_h0);
  return hipGetLastError();
}

}  // namespace gdn
