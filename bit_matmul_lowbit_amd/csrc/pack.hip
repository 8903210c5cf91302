// Packing kernels: FP16 -> Q1_0_g128 quantiser, ternary packer, unpacker.
//
// [P1] 7minutos.es, "Un tutorial de codificacion para ejecutar PrismML Bonsai
//      1-bit LLM en CUDA con GGUF", section 7 "Q1_0_g128 Cuantizacion": scale
//      = largest |w| of each group of 128, bit 1 for w >= 0, 0 -> -scale.
// [P2] 7minutos.es, "PrismML lanza Bonsai 27B ...", section "Como funciona la
//      compresion": w = s_g * t_i with t in {-1, 0, +1}.
//
// Thread mapping (all three kernels): one lane per 8-weight chunk c of one
// 16-row tile.  For a fixed row, the 256 lanes of a block touch 256 adjacent
// chunks, i.e. 4 KB (FP16 in), 2 KB (int8 in) or 4 KB (FP16 out) of one row:
// every global access is a contiguous, 16-byte-per-lane sweep.  Each lane
// then writes its whole 16- or 32-byte code cell with one or two 16-byte
// stores, which are again contiguous across lanes.  The work is bound by HBM;
// the bit logic costs a few ALU operations per weight.
#include "common.h"

namespace lowbit {
namespace {

constexpr int kBlock = 256;

__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
  uint32_t lo = max(a & 0xFFFFu, b & 0xFFFFu);
  uint32_t hi = max(a >> 16, b >> 16);
  return lo | (hi << 16);
}

// FP16 pattern -> Q1 bit: 1 iff the IEEE comparison w >= 0 holds.
// +0 and -0 give 1; negative values, -inf and every NaN give 0.  Works on
// the bit pattern, so subnormals are never flushed.
__device__ __forceinline__ uint32_t q1_bit(uint32_t h) {
  const uint32_t mag = h & 0x7FFFu;
  return (h & 0x8000u) ? (mag == 0u) : (mag <= 0x7C00u);
}

__global__ __launch_bounds__(kBlock) void quantize_q1_kernel(
    const uint16_t* __restrict__ w, int64_t n, int64_t k, uint8_t* __restrict__ codes,
    uint16_t* __restrict__ scales) {
  const int64_t chunks = k / kChunk;
  const int64_t tile = blockIdx.x;
  const int64_t c = (int64_t)blockIdx.y * kBlock + threadIdx.x;
  // chunks % 16 == 0 and the block base is a multiple of 256, so the 16 lanes
  // of one group are either all in range or all out of range.
  if (c >= chunks) return;

  uint32_t bytes[4] = {0u, 0u, 0u, 0u};   // 16 code bytes, row r in byte r
  uint32_t mags[8];                       // max |w| bits of rows (2i, 2i+1)
#pragma unroll
  for (int r = 0; r < kTileRows; ++r) {
    const int64_t row = tile * kTileRows + r;
    uint32_t byte = 0u, mx = 0u;
    if (row < n) {
      const uint4 v = *reinterpret_cast<const uint4*>(w + row * k + c * kChunk);
      const uint32_t words[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        const uint32_t h = (words[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
        byte |= q1_bit(h) << j;
        mx = max(mx, h & 0x7FFFu);
      }
    }
    bytes[r >> 2] |= byte << ((r & 3) * 8);
    if (r & 1) mags[r >> 1] |= mx << 16;
    else mags[r >> 1] = mx;
  }
  *reinterpret_cast<uint4*>(codes + (tile * chunks + c) * 16) =
      make_uint4(bytes[0], bytes[1], bytes[2], bytes[3]);

  // group max over the 16 chunks of a group: 16 adjacent lanes
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1)
      mags[i] = max_u16x2(mags[i], (uint32_t)__shfl_xor((int)mags[i], d, 16));
  }
  const int j = (int)(c % kChunksPerGroup);  // this lane writes the scale of row j
  uint32_t sel = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i == (j >> 1)) sel = mags[i];
  const uint32_t mag = (j & 1) ? (sel >> 16) : (sel & 0xFFFFu);
  const int64_t groups = k / kGroup;
  const int64_t g = c / kChunksPerGroup;
  scales[(tile * groups + g) * kTileRows + j] = (uint16_t)mag;  // pad rows get 0
}

__global__ __launch_bounds__(kBlock) void pack_t2_kernel(
    const int8_t* __restrict__ t, const uint16_t* __restrict__ s, int64_t n, int64_t k,
    uint8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
  const int64_t chunks = k / kChunk;
  const int64_t tile = blockIdx.x;
  const int64_t c = (int64_t)blockIdx.y * kBlock + threadIdx.x;
  if (c >= chunks) return;
  uint32_t pos[4] = {0u, 0u, 0u, 0u}, neg[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int r = 0; r < kTileRows; ++r) {
    const int64_t row = tile * kTileRows + r;
    uint32_t pb = 0u, nb = 0u;
    if (row < n) {
      const uint2 v = *reinterpret_cast<const uint2*>(t + row * k + c * kChunk);
      const uint32_t words[2] = {v.x, v.y};
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        const int32_t b = (int32_t)(int8_t)((words[j >> 2] >> ((j & 3) * 8)) & 0xFFu);
        pb |= (uint32_t)(b > 0) << j;
        nb |= (uint32_t)(b < 0) << j;
      }
    }
    pos[r >> 2] |= pb << ((r & 3) * 8);
    neg[r >> 2] |= nb << ((r & 3) * 8);
  }
  uint8_t* cell = codes + (tile * chunks + c) * 32;
  *reinterpret_cast<uint4*>(cell) = make_uint4(pos[0], pos[1], pos[2], pos[3]);
  *reinterpret_cast<uint4*>(cell + 16) = make_uint4(neg[0], neg[1], neg[2], neg[3]);

  // one lane per group copies the 16 rows' scales of that group
  if (c % kChunksPerGroup == 0) {
    const int64_t groups = k / kGroup;
    const int64_t g = c / kChunksPerGroup;
    uint32_t sv[8];
#pragma unroll
    for (int r = 0; r < kTileRows; r += 2) {
      const int64_t row = tile * kTileRows + r;
      const uint32_t a = row < n ? s[row * groups + g] : 0u;
      const uint32_t b = row + 1 < n ? s[(row + 1) * groups + g] : 0u;
      sv[r >> 1] = a | (b << 16);
    }
    uint4* dst = reinterpret_cast<uint4*>(scales + (tile * groups + g) * kTileRows);
    dst[0] = make_uint4(sv[0], sv[1], sv[2], sv[3]);
    dst[1] = make_uint4(sv[4], sv[5], sv[6], sv[7]);
  }
}

template <int FMT>
__global__ __launch_bounds__(kBlock) void unpack_kernel(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales, int64_t n,
    int64_t k, uint16_t* __restrict__ w) {
  const int64_t chunks = k / kChunk;
  const int64_t tile = blockIdx.x;
  const int64_t c = (int64_t)blockIdx.y * kBlock + threadIdx.x;
  if (c >= chunks) return;
  const int64_t groups = k / kGroup;
  const uint8_t* cell = codes + (tile * chunks + c) * Fmt<FMT>::cell_bytes;
  const uint4 a = *reinterpret_cast<const uint4*>(cell);
  uint4 b = make_uint4(0u, 0u, 0u, 0u);
  if (FMT == 2) b = *reinterpret_cast<const uint4*>(cell + 16);
  const uint4* sp =
      reinterpret_cast<const uint4*>(scales + (tile * groups + c / kChunksPerGroup) * kTileRows);
  const uint4 s0 = sp[0], s1 = sp[1];
  const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
  const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int r = 0; r < kTileRows; ++r) {
    const int64_t row = tile * kTileRows + r;
    if (row >= n) break;
    const uint32_t sc = (sw[r >> 1] >> ((r & 1) * 16)) & 0xFFFFu;
    const uint32_t p = (aw[r >> 2] >> ((r & 3) * 8)) & 0xFFu;
    const uint32_t q = (bw[r >> 2] >> ((r & 3) * 8)) & 0xFFu;
    uint32_t out[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      uint32_t pair = 0u;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = jj * 2 + h;
        const uint32_t pb = (p >> j) & 1u;
        uint32_t v;
        if (FMT == 1) {
          v = pb ? sc : (sc ^ 0x8000u);  // bit 1 -> +s, bit 0 -> -s
        } else {
          const uint32_t nb = (q >> j) & 1u;  // t = pos - neg
          v = (pb && !nb) ? sc : ((nb && !pb) ? (sc ^ 0x8000u) : 0u);
        }
        pair |= v << (16 * h);
      }
      out[jj] = pair;
    }
    *reinterpret_cast<uint4*>(w + row * k + c * kChunk) = make_uint4(out[0], out[1], out[2], out[3]);
  }
}

dim3 pack_grid(int64_t n, int64_t k) {
  const int64_t tiles = (n + kTileRows - 1) / kTileRows;
  const int64_t chunks = k / kChunk;
  return dim3((unsigned)tiles, (unsigned)((chunks + kBlock - 1) / kBlock));
}

}  // namespace

hipError_t launch_quantize_q1(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                              uint16_t* scales, hipStream_t st) {
  hipLaunchKernelGGL(quantize_q1_kernel, pack_grid(n, k), dim3(kBlock), 0, st, w, n, k, codes,
                     scales);
  return hipGetLastError();
}

hipError_t launch_pack_t2(const int8_t* t, const uint16_t* s, int64_t n, int64_t k,
                          uint8_t* codes, uint16_t* scales, hipStream_t st) {
  hipLaunchKernelGGL(pack_t2_kernel, pack_grid(n, k), dim3(kBlock), 0, st, t, s, n, k, codes,
                     scales);
  return hipGetLastError();
}

hipError_t launch_unpack(int fmt, const uint8_t* codes, const uint16_t* scales, int64_t n,
                         int64_t k, uint16_t* w, hipStream_t st) {
  if (fmt == 1)
    hipLaunchKernelGGL(unpack_kernel<1>, pack_grid(n, k), dim3(kBlock), 0, st, codes, scales, n,
                       k, w);
  else
    hipLaunchKernelGGL(unpack_kernel<2>, pack_grid(n, k), dim3(kBlock), 0, st, codes, scales, n,
                       k, w);
  return hipGetLastError();
}

}  // namespace lowbit
