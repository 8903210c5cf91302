// Ceiling probes (include/lowbit_probes.h): a streaming read, a
// matrix-core loop and an LDS read loop, each doing nothing but the one
// thing it measures; the probe of the matrix-core GEMV's per-row work sits
// next to that kernel (gemv_mfma.hip), whose expansion it runs.
// Context for the roofline of the library's kernels; not on the y = W.x path.
#include "../../include/lowbit.h"
#include "../../include/lowbit_probes.h"
#include "common.h"

namespace lowbit {
namespace {

constexpr uint32_t kSinkKey = 0x9E3779B9u;  // a fold that (practically) never occurs
constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(256) void probe_stream_read_kernel(const uint4* __restrict__ p,
                                                                int64_t nvec,
                                                                uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kReadUnroll - 1) * stride < nvec; i += kReadUnroll * stride) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int j = 0; j < kReadUnroll; ++j) v[j] = p[i + j * stride];
#pragma unroll
    for (int j = 0; j < kReadUnroll; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (; i < nvec; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == kSinkKey) sink[blockIdx.x] = acc;
}

// the same read with each work-group sweeping its own contiguous stretch
// (4 KB per step per work-group, 8 steps in flight)
__global__ __launch_bounds__(256) void probe_stream_read_blocks_kernel(const uint4* __restrict__ p,
                                                                       int64_t nvec,
                                                                       uint32_t* __restrict__ sink) {
  const int64_t per = (nvec + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per;
  const int64_t hi = lo + per < nvec ? lo + per : nvec;
  int64_t i = lo + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kReadUnroll - 1) * 256 < hi; i += kReadUnroll * 256) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int j = 0; j < kReadUnroll; ++j) v[j] = p[i + j * 256];
#pragma unroll
    for (int j = 0; j < kReadUnroll; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (; i < hi; i += 256) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == kSinkKey) sink[blockIdx.x] = acc;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void probe_mfma_bf16_kernel(int iters, float* __restrict__ sink) {
  // operands: small lane-dependent values (the data do not change the rate)
  const uint32_t l = threadIdx.x & 63;
  const uint32_t w = 0x3F803F80u ^ (l << 16) ^ l;
  const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(w, w ^ 1u, w ^ 2u, w ^ 3u));
  const bf16x8 b = __builtin_bit_cast(bf16x8, make_uint4(w ^ 4u, w ^ 5u, w ^ 6u, w ^ 7u));
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
  if (__builtin_bit_cast(uint32_t, s) == kSinkKey) sink[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void probe_lds_read_kernel(int iters, uint32_t* __restrict__ sink) {
  __shared__ uint4 buf[2048];  // 32 KB
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 8; ++j) buf[t + 256 * j] = make_uint4(t, j, t ^ j, 7u * t);
  __syncthreads();
  uint32_t acc = 0;
  int base = t;
  for (int i = 0; i < iters; ++i) {
    uint4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = buf[(base + 256 * j) & 2047];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    base += 64;  // a different 1 KB of every 4 KB next time (the loop-carried address keeps
                 // the reads from being hoisted)
  }
  if (acc == kSinkKey) sink[blockIdx.x * 256 + t] = acc;
}

}  // namespace
}  // namespace lowbit

extern "C" {

int lowbit_probe_cu_count(void) { return lowbit::device_cu_count(); }

int lowbit_probe_stream_read(const void* buf, size_t bytes, int blocks_per_cu, int order,
                             uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink || blocks_per_cu < 1 || blocks_per_cu > 64 || order < 0 || order > 1)
    return LOWBIT_ERR_ARG;
  if (bytes == 0 || bytes % 16 != 0 || bytes > (size_t(1) << 40)) return LOWBIT_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 3u))
    return LOWBIT_ERR_ALIGN;
  const unsigned blocks = (unsigned)(blocks_per_cu * lowbit::device_cu_count());
  if (order == 0)
    hipLaunchKernelGGL(lowbit::probe_stream_read_kernel, dim3(blocks), dim3(256), 0, stream,
                       static_cast<const uint4*>(buf), (int64_t)(bytes / 16), sink);
  else
    hipLaunchKernelGGL(lowbit::probe_stream_read_blocks_kernel, dim3(blocks), dim3(256), 0,
                       stream, static_cast<const uint4*>(buf), (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? LOWBIT_OK : LOWBIT_ERR_HIP;
}

int lowbit_probe_lds_read(int iters, int blocks_per_cu, uint32_t* sink, hipStream_t stream) {
  if (!sink || blocks_per_cu < 1 || blocks_per_cu > 4 || iters < 1 || iters > (1 << 24))
    return LOWBIT_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(sink) & 3u) return LOWBIT_ERR_ALIGN;
  const unsigned blocks = (unsigned)(blocks_per_cu * lowbit::device_cu_count());
  hipLaunchKernelGGL(lowbit::probe_lds_read_kernel, dim3(blocks), dim3(256), 0, stream, iters,
                     sink);
  return hipGetLastError() == hipSuccess ? LOWBIT_OK : LOWBIT_ERR_HIP;
}

int lowbit_probe_mfma_bf16(int iters, int blocks_per_cu, float* sink, hipStream_t stream) {
  if (!sink || blocks_per_cu < 1 || blocks_per_cu > 8 || iters < 1 || iters > (1 << 24))
    return LOWBIT_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(sink) & 3u) return LOWBIT_ERR_ALIGN;
  const unsigned blocks = (unsigned)(blocks_per_cu * lowbit::device_cu_count());
  hipLaunchKernelGGL(lowbit::probe_mfma_bf16_kernel, dim3(blocks), dim3(256), 0, stream, iters,
                     sink);
  return hipGetLastError() == hipSuccess ? LOWBIT_OK : LOWBIT_ERR_HIP;
}

int lowbit_probe_expand_mfma(int mode, int iters, int blocks_per_cu, float* sink,
                             hipStream_t stream) {
  if (!sink || mode < 0 || mode > 2 || blocks_per_cu < 1 || blocks_per_cu > 4 || iters < 1 ||
      iters > (1 << 24) || (mode == 2 && iters % 4 != 0))
    return LOWBIT_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(sink) & 3u) return LOWBIT_ERR_ALIGN;
  const int blocks = blocks_per_cu * lowbit::device_cu_count();
  return lowbit::launch_probe_expand_mfma(mode, iters, blocks, sink, stream) == hipSuccess
             ? LOWBIT_OK
             : LOWBIT_ERR_HIP;
}

}  // extern "C"
