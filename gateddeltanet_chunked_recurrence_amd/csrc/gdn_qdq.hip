// Standalone state QDQ: one workgroup per [Dk, block_v] tile of one state.
// Pass 1 reduces the tile amax across the workgroup (wave shuffles + LDS);
// pass 2 re-reads the tile (L2-resident) and quantizes each element.
// Arithmetic order is the FP32 definition in gdn.h (IEEE division for d and
// 1/d, one rounding per product), so results are bit-exact to it. `y` may
// alias `x`: every element is read and written by the same thread.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

constexpr int QDQ_THREADS = 256;

template <int FMT>
__global__ void __launch_bounds__(QDQ_THREADS)
qdq_state_kernel(const float* x, float* y, float* __restrict__ scales,
                 uint8_t* __restrict__ codes, int Dk, int Dv, int block_v) {
  __shared__ float red[QDQ_THREADS / WAVE];
  const int tiles_per_state = Dv / block_v;
  const int64_t state = blockIdx.x / tiles_per_state;
  const int tile = blockIdx.x % tiles_per_state;
  const int64_t base = state * (int64_t)Dk * Dv + (int64_t)tile * block_v;
  const int n = Dk * block_v;
  const int tid = threadIdx.x;

  float amax = 0.f;
  for (int e = tid; e < n; e += QDQ_THREADS)
    amax = fmaxf(amax, fabsf(x[base + (int64_t)(e / block_v) * Dv + (e % block_v)]));
  amax = wave_max(amax);
  if ((tid & (WAVE - 1)) == 0) red[tid / WAVE] = amax;
  __syncthreads();
  amax = red[0];
#pragma unroll
  for (int w = 1; w < QDQ_THREADS / WAVE; ++w) amax = fmaxf(amax, red[w]);

  const float d = qdq_scale<FMT>(amax);
  const float r = 1.0f / d;
  for (int e = tid; e < n; e += QDQ_THREADS) {
    const int64_t off = base + (int64_t)(e / block_v) * Dv + (e % block_v);
    float c;
    uint8_t byte;
    if constexpr (FMT == 1) {
      float unused;
      uint32_t b;
      e4m3_pair(x[off] * r, 0.f, c, unused, b);
      byte = static_cast<uint8_t>(b & 0xFFu);
    } else {
      c = round_int8(x[off] * r);
      byte = static_cast<uint8_t>(static_cast<int8_t>(c));
    }
    y[off] = c * d;
    if (codes) codes[off] = byte;
  }
  if (scales && tid == 0) scales[state * tiles_per_state + tile] = d;
}

hipError_t launch_qdq_state(const float* x, float* y, float* scales, uint8_t* codes,
                            int64_t n_states, int Dk, int Dv, int block_v, int fmt,
                            hipStream_t stream) {
  const int64_t blocks = n_states * (Dv / block_v);
  if (blocks == 0) return hipSuccess;
  if (fmt == 1)
    hipLaunchKernelGGL(qdq_state_kernel<1>, dim3((unsigned)blocks), dim3(QDQ_THREADS), 0,
                       stream, x, y, scales, codes, Dk, Dv, block_v);
  else
    hipLaunchKernelGGL(qdq_state_kernel<2>, dim3((unsigned)blocks), dim3(QDQ_THREADS), 0,
                       stream, x, y, scales, codes, Dk, Dv, block_v);
  return hipGetLastError();
}

}  // namespace gdn
