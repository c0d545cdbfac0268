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

}  // namespace

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
