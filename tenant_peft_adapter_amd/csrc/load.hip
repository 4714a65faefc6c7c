// Load-time (admission) kernels and the calibration probes.
//
// Scute paper (arXiv 2611.01089), §5.1 "The Admission Compiler": DoRA's
// scale s = m ⊘ ‖W + cAB‖_c is computed when the adapter is admitted, from
// the base weight in the engine's own layout; the norm of each output
// column runs over d_in (appendix "Tensor parallelism").  Here W is stored
// [d_out][d_in], so output column j is the contiguous row W[j].  The same
// kernel folds e = s into the owned B (Table 1: e -> B).
//
// Probes (appendix "Constants"): a streaming device copy for the bandwidth
// β, and chained one-block empty kernels for the launch cost λ.
#include "internal.h"

namespace tpa {

namespace {

constexpr int THREADS = 256;

template <typename T>
__global__ __launch_bounds__(THREADS) void dora_norm_kernel(DoraArgs a) {
  __shared__ float bcol[512];
  __shared__ float wsum[THREADS / 64];
  __shared__ float s_scale;
  const int j = blockIdx.x;
  const int tid = threadIdx.x;
  for (int k = tid; k < a.r; k += THREADS) bcol[k] = a.B[(size_t)k * a.d_out + j];
  __syncthreads();
  const T* W = static_cast<const T*>(a.W) + (size_t)j * a.d_in;
  float sum = 0.f;
  for (int i = tid; i < a.d_in; i += THREADS) {
    float v = to_f<T>(W[i]);
    for (int k = 0; k < a.r; ++k) v += a.At[(size_t)k * a.d_in + i] * bcol[k];
    sum += v * v;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_down(sum, off, 64);
  if ((tid & 63) == 0) wsum[tid >> 6] = sum;
  __syncthreads();
  if (tid == 0) {
    float tot = 0.f;
    for (int w = 0; w < THREADS / 64; ++w) tot += wsum[w];
    const float norm = sqrtf(tot);
    const float sv = a.m[j] / norm;
    if (!(norm > 0.f) || !isfinite(sv)) atomicOr(a.status, 1);
    a.s[j] = sv;
    s_scale = sv;
  }
  __syncthreads();
  if (!a.fold_e) return;
  T* bt = static_cast<T*>(a.Bt) + (size_t)j * a.r_pad;
  for (int k = tid; k < a.r_pad; k += THREADS) bt[k] = to_t<T>(k < a.r ? bcol[k] * s_scale : 0.f);
}

template <typename T>
__global__ __launch_bounds__(THREADS) void convert_kernel(const float* src, T* dst, size_t count,
                                                          float alpha) {
  for (size_t i = (size_t)blockIdx.x * THREADS + threadIdx.x; i < count; i += (size_t)gridDim.x * THREADS)
    dst[i] = to_t<T>(alpha * src[i]);
}

// dst[c][r] = alpha * src[r][c] * colscale[c]; dst is [cols_pad][ld].
template <typename T>
__global__ __launch_bounds__(THREADS) void pack_transpose_kernel(const float* src, int rows, int cols,
                                                                 float alpha, const float* colscale,
                                                                 T* dst, int cols_pad, int ld) {
  const size_t total = (size_t)cols_pad * ld;
  for (size_t i = (size_t)blockIdx.x * THREADS + threadIdx.x; i < total; i += (size_t)gridDim.x * THREADS) {
    const int c = (int)(i / ld), r = (int)(i % ld);
    float v = 0.f;
    if (c < cols && r < rows) v = alpha * src[(size_t)r * cols + c] * (colscale ? colscale[c] : 1.f);
    dst[i] = to_t<T>(v);
  }
}

__global__ __launch_bounds__(THREADS) void copy_kernel(uint4* dst, const uint4* src, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * THREADS + threadIdx.x; i < n16; i += (size_t)gridDim.x * THREADS)
    dst[i] = src[i];
}

// Read-only streaming probe: each thread folds its 16-byte loads (four in
// flight per iteration) into one word; one word per work-group is written,
// so the kernel's traffic is the read.
__global__ __launch_bounds__(THREADS) void read_kernel(const uint4* src, size_t n16, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * THREADS;
  uint32_t acc = 0;
  size_t i = (size_t)blockIdx.x * THREADS + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  __shared__ uint32_t red[THREADS / 64];
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < THREADS / 64; ++w) t ^= red[w];
    sink[blockIdx.x] = t;
  }
}

__global__ void empty_kernel() {}

// One wave that idles for `ticks` of the constant-rate device clock; the
// iteration cap (each iteration sleeps) bounds it even if the clock stalls.
__global__ void delay_kernel(unsigned long long ticks, unsigned long long max_iters) {
  const unsigned long long t0 = wall_clock64();
  for (unsigned long long i = 0; i < max_iters; ++i) {
    if (wall_clock64() - t0 >= ticks) break;
    __builtin_amdgcn_s_sleep(8);
  }
}

unsigned grid_for(size_t work) {
  size_t g = (work + THREADS - 1) / THREADS;
  if (g > 65536) g = 65536;
  if (g == 0) g = 1;
  return (unsigned)g;
}

}  // namespace

size_t dtype_size(int dtype) { return dtype == 0 ? 4 : 2; }

hipError_t launch_dora_norm(int dtype, const DoraArgs& a, hipStream_t s) {
  if (a.r > 512) return hipErrorInvalidValue;
  switch (dtype) {
    case 0: hipLaunchKernelGGL(dora_norm_kernel<float>, dim3(a.d_out), dim3(THREADS), 0, s, a); break;
    case 1: hipLaunchKernelGGL(dora_norm_kernel<f16>, dim3(a.d_out), dim3(THREADS), 0, s, a); break;
    case 2: hipLaunchKernelGGL(dora_norm_kernel<bf16>, dim3(a.d_out), dim3(THREADS), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_convert(int dtype, const float* src, void* dst, size_t count, float alpha,
                          hipStream_t s) {
  const dim3 grid(grid_for(count));
  switch (dtype) {
    case 0: hipLaunchKernelGGL(convert_kernel<float>, grid, dim3(THREADS), 0, s, src, (float*)dst, count, alpha); break;
    case 1: hipLaunchKernelGGL(convert_kernel<f16>, grid, dim3(THREADS), 0, s, src, (f16*)dst, count, alpha); break;
    case 2: hipLaunchKernelGGL(convert_kernel<bf16>, grid, dim3(THREADS), 0, s, src, (bf16*)dst, count, alpha); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_pack_transpose(int dtype, const float* src, int rows, int cols, float alpha,
                                 const float* colscale, void* dst, int cols_pad, int ld, hipStream_t s) {
  const dim3 grid(grid_for((size_t)cols_pad * ld));
  switch (dtype) {
    case 0:
      hipLaunchKernelGGL(pack_transpose_kernel<float>, grid, dim3(THREADS), 0, s, src, rows, cols, alpha,
                         colscale, (float*)dst, cols_pad, ld);
      break;
    case 1:
      hipLaunchKernelGGL(pack_transpose_kernel<f16>, grid, dim3(THREADS), 0, s, src, rows, cols, alpha,
                         colscale, (f16*)dst, cols_pad, ld);
      break;
    case 2:
      hipLaunchKernelGGL(pack_transpose_kernel<bf16>, grid, dim3(THREADS), 0, s, src, rows, cols, alpha,
                         colscale, (bf16*)dst, cols_pad, ld);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  size_t g = (n16 + THREADS * 4 - 1) / (THREADS * 4);
  if (g > 8192) g = 8192;
  if (g == 0) g = 1;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)g), dim3(THREADS), 0, s, (uint4*)dst, (const uint4*)src, n16);
  return hipGetLastError();
}

hipError_t launch_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s) {
  const size_t n16 = bytes / 16;
  size_t g = (n16 + THREADS * 4 - 1) / (THREADS * 4);
  if (g > PROBE_READ_BLOCKS) g = PROBE_READ_BLOCKS;
  if (g == 0) g = 1;
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)g), dim3(THREADS), 0, s, (const uint4*)src, n16, sink);
  return hipGetLastError();
}

hipError_t launch_empty(int count, hipStream_t s) {
  for (int i = 0; i < count; ++i) hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, s);
  return hipGetLastError();
}

hipError_t launch_delay(int microseconds, hipStream_t s) {
  int dev = 0, khz = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return e;
  if (khz <= 0) return hipErrorInvalidValue;
  const unsigned long long ticks = (unsigned long long)microseconds * (unsigned long long)khz / 1000ull;
  hipLaunchKernelGGL(delay_kernel, dim3(1), dim3(64), 0, s, ticks, ticks + 1);
  return hipGetLastError();
}

}  // namespace tpa
