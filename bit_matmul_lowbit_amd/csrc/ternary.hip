// Ternary quantiser (FP16 -> ternary g128 codes) and base-3 storage.
//
// [P2] 7minutos.es, "PrismML lanza Bonsai 27B ...", "Como funciona la
//      compresion": w = s * t with t in {-1, 0, +1} and one FP16 scale per
//      128 weights; a ternary weight carries log2(3) bits, ~1.71 bits per
//      weight with the scale.
// The pages give no ternary rounding rule.  This library's rule: s = max |w|
// of the group (as the 1-bit worked example), and t is the nearest of
// {-1, 0, +1} to w / s with ties to 0, i.e. t = sign(w) iff 2|w| > s.
//
// Base-3 storage packs five trits per byte, byte = sum_i (t_i + 1) * 3^i
// for the weights 5j + i of a row, rows one after another with ceil(k/5)
// bytes each (positions past k hold t = 0), and keeps the scales row-major
// [n][k/128]: 8/5 + 16/128 = 1.725 bits per weight.  It is a storage
// format; the GEMV and GEMM read the two-plane codes, which these kernels
// convert to and from.
#include "common.h"

namespace lowbit {
namespace {

constexpr int kBlock = 256;

__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
  return max(a & 0xFFFFu, b & 0xFFFFu) | (max(a >> 16, b >> 16) << 16);
}

// 2 * |w| > s for FP16 magnitude patterns m = |w| and S = s (sign cleared),
// in real arithmetic; false when either is NaN.  Doubling a pattern is
// exact: a subnormal doubles its fraction, a normal value adds one to its
// exponent; at exponent 30 the double (>= 65536) exceeds every finite s.
__device__ __forceinline__ bool twice_gt(uint32_t m, uint32_t S) {
  if (m > 0x7C00u || S > 0x7C00u) return false;
  if (m >= 0x7800u) return S < 0x7C00u;
  const uint32_t d = m < 0x0400u ? 2u * m : m + 0x0400u;
  return d > S;
}

// One lane per 8-weight chunk c of one 16-row tile, as the 1-bit quantiser.
// A (rolled) loop over four blocks of four rows: load them, reduce their
// group maxima over the 16 lanes of the group (two 16-bit maxima per
// shuffle), decide their 32 weights, and shift the block's pos and neg code
// words into place.  Only one block is live at a time, so the kernel keeps
// enough waves in flight to stream at HBM speed.
__global__ __launch_bounds__(kBlock) void quantize_t2_kernel(const uint16_t* __restrict__ w,
                                                             int64_t n, int64_t k,
                                                             uint8_t* __restrict__ codes,
                                                             uint16_t* __restrict__ scales) {
  const int64_t chunks = k / kChunk;
  const int64_t tile = blockIdx.x;
  const int64_t c = (int64_t)blockIdx.y * kBlock + threadIdx.x;
  if (c >= chunks) return;  // whole 16-lane groups leave together
  const int jr = (int)(c % kChunksPerGroup);  // this lane writes the scale of row jr
  uint32_t p0 = 0u, p1 = 0u, p2 = 0u, p3 = 0u, q0 = 0u, q1 = 0u, q2 = 0u, q3 = 0u;
  uint32_t my_scale = 0u;
#pragma unroll 1
  for (int blk = 0; blk < kTileRows / 4; ++blk) {
    uint32_t hw[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t row = tile * kTileRows + 4 * blk + u;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (row < n) v = *reinterpret_cast<const uint4*>(w + row * k + c * kChunk);
      hw[u][0] = v.x; hw[u][1] = v.y; hw[u][2] = v.z; hw[u][3] = v.w;
    }
    uint32_t pw = 0u, nw = 0u;
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      // max |w| patterns of rows 2 pr (low half) and 2 pr + 1 of the block
      uint32_t mags = 0u;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        uint32_t mx = 0u;
#pragma unroll
        for (int j = 0; j < kChunk; ++j)
          mx = max(mx, (hw[2 * pr + u][j >> 1] >> ((j & 1) * 16)) & 0x7FFFu);
        mags |= mx << (16 * u);
      }
#pragma unroll
      for (int d = 8; d >= 1; d >>= 1)
        mags = max_u16x2(mags, (uint32_t)__shfl_xor((int)mags, d, 16));
      if ((jr >> 1) == 2 * blk + pr) my_scale = (jr & 1) ? (mags >> 16) : (mags & 0xFFFFu);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t S = (mags >> (16 * u)) & 0xFFFFu;
        uint32_t pb = 0u, nb = 0u;
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
          const uint32_t h = (hw[2 * pr + u][j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
          const uint32_t nz = twice_gt(h & 0x7FFFu, S) ? 1u : 0u;
          const uint32_t sgn = h >> 15;
          pb |= (nz & (sgn ^ 1u)) << j;
          nb |= (nz & sgn) << j;
        }
        pw |= pb << ((2 * pr + u) * 8);
        nw |= nb << ((2 * pr + u) * 8);
      }
    }
    // rows 4 blk .. 4 blk + 3 are code word blk: shift the words into place
    p0 = p1; p1 = p2; p2 = p3; p3 = pw;
    q0 = q1; q1 = q2; q2 = q3; q3 = nw;
  }
  uint8_t* cell = codes + (tile * chunks + c) * 32;
  *reinterpret_cast<uint4*>(cell) = make_uint4(p0, p1, p2, p3);
  *reinterpret_cast<uint4*>(cell + 16) = make_uint4(q0, q1, q2, q3);
  const int64_t groups = k / kGroup;
  scales[(tile * groups + c / kChunksPerGroup) * kTileRows + jr] = (uint16_t)my_scale;
}

// t of (row, col) from the two planes: pos - neg
__device__ __forceinline__ int trit(const uint8_t* __restrict__ codes, int64_t chunks, int64_t row,
                                    int64_t col) {
  const uint8_t* cell = codes + ((row / kTileRows) * chunks + col / kChunk) * 32;
  const int r = (int)(row % kTileRows), b = (int)(col % kChunk);
  return (int)((cell[r] >> b) & 1u) - (int)((cell[16 + r] >> b) & 1u);
}

// two-plane codes + tile-major scales -> base-3 bytes + row-major scales;
// one thread per output byte (then per output scale), grid-stride
__global__ __launch_bounds__(kBlock) void t2_to_base3_kernel(const uint8_t* __restrict__ codes,
                                                             const uint16_t* __restrict__ scales,
                                                             int64_t n, int64_t k,
                                                             uint8_t* __restrict__ out,
                                                             uint16_t* __restrict__ out_scales) {
  const int64_t chunks = k / kChunk, groups = k / kGroup, rb = (k + 4) / 5;
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  for (int64_t i = gid; i < n * rb; i += stride) {
    const int64_t row = i / rb, j = i - row * rb;
    int v = 0, p = 1;
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      const int64_t col = 5 * j + q;
      v += ((col < k ? trit(codes, chunks, row, col) : 0) + 1) * p;
      p *= 3;
    }
    out[i] = (uint8_t)v;
  }
  for (int64_t i = gid; i < n * groups; i += stride) {
    const int64_t row = i / groups, g = i - row * groups;
    out_scales[i] = scales[((row / kTileRows) * groups + g) * kTileRows + row % kTileRows];
  }
}

// base-3 bytes + row-major scales -> two-plane codes + tile-major scales;
// one lane per (tile, chunk) as the ternary packer (rows past n get zero
// codes and zero scales); a byte of 243..255 decodes with its fifth digit
// taken mod 3
__global__ __launch_bounds__(kBlock) void base3_to_t2_kernel(const uint8_t* __restrict__ in,
                                                             const uint16_t* __restrict__ in_scales,
                                                             int64_t n, int64_t k,
                                                             uint8_t* __restrict__ codes,
                                                             uint16_t* __restrict__ scales) {
  const int64_t chunks = k / kChunk, groups = k / kGroup, rb = (k + 4) / 5;
  const int64_t tile = blockIdx.x;
  const int64_t c = (int64_t)blockIdx.y * kBlock + threadIdx.x;
  if (c >= chunks) return;
  uint32_t pos[4] = {0u, 0u, 0u, 0u}, neg[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int r = 0; r < kTileRows; ++r) {
    const int64_t row = tile * kTileRows + r;
    uint32_t pb = 0u, nb = 0u;
    if (row < n) {
      const uint8_t* src = in + row * rb;
#pragma unroll
      for (int b = 0; b < kChunk; ++b) {
        const int64_t col = c * kChunk + b;
        int v = src[col / 5];
        const int q = (int)(col % 5);
        for (int e = 0; e < q; ++e) v /= 3;
        const int t = v % 3 - 1;
        pb |= (uint32_t)(t > 0) << b;
        nb |= (uint32_t)(t < 0) << b;
      }
    }
    pos[r >> 2] |= pb << ((r & 3) * 8);
    neg[r >> 2] |= nb << ((r & 3) * 8);
  }
  uint8_t* cell = codes + (tile * chunks + c) * 32;
  *reinterpret_cast<uint4*>(cell) = make_uint4(pos[0], pos[1], pos[2], pos[3]);
  *reinterpret_cast<uint4*>(cell + 16) = make_uint4(neg[0], neg[1], neg[2], neg[3]);
  if (c % kChunksPerGroup == 0) {
    const int64_t g = c / kChunksPerGroup;
    uint16_t* dst = scales + (tile * groups + g) * kTileRows;
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) {
      const int64_t row = tile * kTileRows + r;
      dst[r] = row < n ? in_scales[row * groups + g] : (uint16_t)0;
    }
  }
}

dim3 tile_grid(int64_t n, int64_t k) {
  const int64_t tiles = (n + kTileRows - 1) / kTileRows;
  const int64_t cblocks = (k / kChunk + kBlock - 1) / kBlock;
  return dim3((unsigned)tiles, (unsigned)cblocks);
}

}  // namespace

hipError_t launch_quantize_t2(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                              uint16_t* scales, hipStream_t st) {
  hipLaunchKernelGGL(quantize_t2_kernel, tile_grid(n, k), dim3(kBlock), 0, st, w, n, k, codes,
                     scales);
  return hipGetLastError();
}

hipError_t launch_t2_to_base3(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                              uint8_t* out, uint16_t* out_scales, hipStream_t st) {
  const int64_t work = n * ((k + 4) / 5);
  int64_t blocks = (work + kBlock - 1) / kBlock;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(t2_to_base3_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, st, codes,
                     scales, n, k, out, out_scales);
  return hipGetLastError();
}

hipError_t launch_base3_to_t2(const uint8_t* in, const uint16_t* in_scales, int64_t n, int64_t k,
                              uint8_t* codes, uint16_t* scales, hipStream_t st) {
  hipLaunchKernelGGL(base3_to_t2_kernel, tile_grid(n, k), dim3(kBlock), 0, st, in, in_scales, n, k,
                     codes, scales);
  return hipGetLastError();
}

}  // namespace lowbit
