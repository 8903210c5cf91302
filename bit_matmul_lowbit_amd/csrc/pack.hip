// Packing kernels: FP16 -> Q1_0_g128 quantiser, ternary packer, unpacker.
//
// [P1] 7minutos.es, "Un tutorial de codificacion para ejecutar PrismML Bonsai
//      1-bit LLM en CUDA con GGUF", section 7 "Q1_0_g128 Cuantizacion": scale
//      = largest |w| of each group of 128, bit 1 for w >= 0, 0 -> -scale.
// [P2] 7minutos.es, "PrismML lanza Bonsai 27B ...", section "Como funciona la
//      compresion": w = s_g * t_i with t in {-1, 0, +1}.
//
// Thread mapping: one lane per 8-weight chunk c of one 16-row tile (the
// quantiser and the unpacker; the ternary packer takes two adjacent chunks
// per lane, so that its int8 input also comes in 16 bytes per lane).  For a
// fixed row, the 128 lanes of a work-group touch adjacent chunks, i.e. 2 KB
// (FP16 in), 2 KB (int8 in, two chunks per lane) or 2 KB (FP16 out) of one
// row: every global access is a contiguous, 16-byte-per-lane sweep.  Each
// lane then writes its whole 16- or 32-byte code cell(s) with 16-byte stores,
// which are again contiguous across lanes.  The work is bound by HBM; the bit
// logic runs two FP16 or four int8 values per instruction.
#include "common.h"

namespace lowbit {
namespace {

constexpr int kBlock = 128;

__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
  uint32_t lo = max(a & 0xFFFFu, b & 0xFFFFu);
  uint32_t hi = max(a >> 16, b >> 16);
  return lo | (hi << 16);
}

// FP16 pattern -> Q1 bit: 1 iff the IEEE comparison w >= 0 holds, i.e.
// with m = |w| pattern: sign clear and m <= 0x7C00 (not a NaN), or sign set
// and m == 0.  +0 and -0 give 1; negative values, -inf and every NaN give 0.
// Works on the bit pattern, so subnormals are never flushed.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// The code byte (bit j = the bit of value j) and the max |w| pattern of one
// chunk (4 words, two FP16 values each), two values at a time with packed
// 16-bit operations: with m = |w| pattern, 0x7C00 - m wraps (bit 15 set)
// iff m > 0x7C00 (a NaN), and m - 1 wraps iff m == 0, so bit 15 / 31 of
// sign ? (m - 1) : ~(0x7C00 - m) is the IEEE w >= 0 of each value.  The
// four words' bits are gathered into the byte with shifts and a select.
__device__ __forceinline__ void q1_chunk(const uint32_t (&words)[4], uint32_t& byte,
                                         uint32_t& mx) {
  uint32_t keep[4];
  u16x2 mm = {0, 0};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const u16x2 m = __builtin_bit_cast(u16x2, words[p] & 0x7FFF7FFFu);
    mm = __builtin_elementwise_max(mm, m);
    const uint32_t nan_hi = __builtin_bit_cast(uint32_t, (u16x2){0x7C00, 0x7C00} - m);
    const uint32_t zero_hi = __builtin_bit_cast(uint32_t, m - (u16x2){1, 1});
    keep[p] = ((words[p] & zero_hi) | (~words[p] & ~nan_hi)) & 0x80008000u;
  }
  mx = max((uint32_t)mm.x, (uint32_t)mm.y);
  // value 2p at bit 2p, value 2p + 1 at bit 16 + 2p, then bit 2p + 1
  const uint32_t d = (keep[0] >> 15) | (keep[1] >> 13) | (keep[2] >> 11) | (keep[3] >> 9);
  byte = (d & 0x55u) | ((d >> 15) & 0xAAu);
}

__global__ __launch_bounds__(kBlock) void quantize_q1_kernel(
    const uint16_t* __restrict__ w, int64_t n, int64_t k, uint8_t* __restrict__ codes,
    uint16_t* __restrict__ scales) {
  const int64_t chunks = k / kChunk;
  const int64_t cblocks = (k / kChunk + kBlock - 1) / kBlock;
  const int64_t tile = blockIdx.x / cblocks;
  const int64_t c = (int64_t)(blockIdx.x - tile * cblocks) * kBlock + threadIdx.x;
  // chunks % 16 == 0 and the block base is a multiple of 128, so the 16 lanes
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
      q1_chunk(words, byte, mx);
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

// Bit 7 of each byte of x0 (weights 0..3) and x1 (weights 4..7) gathered
// into bits 0..7: after d = x0 >> 7 | x1 >> 3 the weights sit at bits
// 0, 8, 16, 24 (0..3) and 4, 12, 20, 28 (4..7); folding by 7 and then by
// 14 bits brings 8, 12 to 1, 5 and 16, 20, 24, 28 to 2, 6, 3, 7.  Other
// bits of x0, x1 must be clear.
__device__ __forceinline__ uint32_t gather_bit7(uint32_t x0, uint32_t x1) {
  uint32_t d = (x0 >> 7) | (x1 >> 3);
  d |= d >> 7;
  d |= d >> 14;
  return d & 0xFFu;
}

// pos and neg bytes of 8 int8 values t (two words): bit 7 of
// (t & 0x7F) + 0x7F is set iff the byte is nonzero; pos = nonzero with the
// sign clear, neg = sign set (t < 0).
__device__ __forceinline__ void t2_chunk_bits(uint32_t w0, uint32_t w1, uint32_t& pb,
                                              uint32_t& nb) {
  const uint32_t z0 = (w0 & 0x7F7F7F7Fu) + 0x7F7F7F7Fu, z1 = (w1 & 0x7F7F7F7Fu) + 0x7F7F7F7Fu;
  pb = gather_bit7(z0 & ~w0 & 0x80808080u, z1 & ~w1 & 0x80808080u);
  nb = gather_bit7(w0 & 0x80808080u, w1 & 0x80808080u);
}

// One lane per two adjacent chunks (c, c + 1) of a 16-row tile: a 16-byte
// load of int8 t per row (t is 16-byte aligned and rows are k bytes, a
// multiple of 128), two cells written.
__global__ __launch_bounds__(kBlock) void pack_t2_kernel(
    const int8_t* __restrict__ t, const uint16_t* __restrict__ s, int64_t n, int64_t k,
    uint8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
  const int64_t chunks = k / kChunk;
  const int64_t pairs = chunks / 2;  // chunks % 16 == 0
  const int64_t cblocks = (pairs + kBlock - 1) / kBlock;
  const int64_t tile = blockIdx.x / cblocks;
  const int64_t c = 2 * ((int64_t)(blockIdx.x - tile * cblocks) * kBlock + threadIdx.x);
  if (c >= chunks) return;
  uint32_t pos[2][4] = {}, neg[2][4] = {};
#pragma unroll
  for (int r = 0; r < kTileRows; ++r) {
    const int64_t row = tile * kTileRows + r;
    uint32_t pb0 = 0u, nb0 = 0u, pb1 = 0u, nb1 = 0u;
    if (row < n) {
      const uint4 v = *reinterpret_cast<const uint4*>(t + row * k + c * kChunk);
      t2_chunk_bits(v.x, v.y, pb0, nb0);
      t2_chunk_bits(v.z, v.w, pb1, nb1);
    }
    pos[0][r >> 2] |= pb0 << ((r & 3) * 8);
    neg[0][r >> 2] |= nb0 << ((r & 3) * 8);
    pos[1][r >> 2] |= pb1 << ((r & 3) * 8);
    neg[1][r >> 2] |= nb1 << ((r & 3) * 8);
  }
  uint4* cell = reinterpret_cast<uint4*>(codes + (tile * chunks + c) * 32);
  cell[0] = make_uint4(pos[0][0], pos[0][1], pos[0][2], pos[0][3]);
  cell[1] = make_uint4(neg[0][0], neg[0][1], neg[0][2], neg[0][3]);
  cell[2] = make_uint4(pos[1][0], pos[1][1], pos[1][2], pos[1][3]);
  cell[3] = make_uint4(neg[1][0], neg[1][1], neg[1][2], neg[1][3]);

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
  const int64_t cblocks = (k / kChunk + kBlock - 1) / kBlock;
  const int64_t tile = blockIdx.x / cblocks;
  const int64_t c = (int64_t)(blockIdx.x - tile * cblocks) * kBlock + threadIdx.x;
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

// One work-group per (tile, block of kBlock chunks), the chunk blocks of a
// tile consecutive: work-groups launched together read whole rows of 16 rows
// (1-bit FP16 -> Q1 at 151936 x 5120: 354 -> 325 us with kBlock = 128, from
// tile-major order with 256-chunk blocks, the last of them half empty).
dim3 pack_grid(int64_t n, int64_t k) {
  const int64_t tiles = (n + kTileRows - 1) / kTileRows;
  const int64_t chunks = k / kChunk;
  return dim3((unsigned)(tiles * ((chunks + kBlock - 1) / kBlock)));
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
  const int64_t tiles = (n + kTileRows - 1) / kTileRows;
  const int64_t pairs = k / kChunk / 2;
  hipLaunchKernelGGL(pack_t2_kernel, dim3((unsigned)(tiles * ((pairs + kBlock - 1) / kBlock))),
                     dim3(kBlock), 0, st, t, s, n, k, codes, scales);
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
