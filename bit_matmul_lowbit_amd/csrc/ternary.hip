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
constexpr int kQBlock = 128;  // quantiser: chunks per work-group

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

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2 as_u16x2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }
__device__ __forceinline__ uint32_t as_u32(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// max |w| pattern over the 8 FP16 values of a chunk (4 words)
__device__ __forceinline__ uint32_t chunk_max_mag(const uint32_t (&hw)[4]) {
  u16x2 m = as_u16x2(hw[0] & 0x7FFF7FFFu);
#pragma unroll
  for (int p = 1; p < 4; ++p) m = __builtin_elementwise_max(m, as_u16x2(hw[p] & 0x7FFF7FFFu));
  return max((uint32_t)m.x, (uint32_t)m.y);
}

// The pos and neg bytes of a chunk whose group scale pattern S is finite
// (S < 0x7C00; S is the largest |w| of the group, so every |w| here is
// finite too).  Two weights at a time: 2|w| as a pattern is m + min(m,
// 0x400) (a subnormal doubles its fraction, a normal value adds one to its
// exponent; at most 0x7FFF), and 2|w| > s is the sign bit of the wrapping
// 16-bit difference S - 2|w| (both below 0x8000).  Bit 15 / 31 of word p
// then holds weight 2p / 2p + 1; the four words' bits are gathered into a
// byte with shifts and a bitwise select.
__device__ __forceinline__ void chunk_trits_finite(const uint32_t (&hw)[4], uint32_t S,
                                                   uint32_t& pb, uint32_t& nb) {
  const u16x2 SS = {(unsigned short)S, (unsigned short)S};
  uint32_t pos[4], neg[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const u16x2 m = as_u16x2(hw[p] & 0x7FFF7FFFu);
    const u16x2 d = m + __builtin_elementwise_min(m, (u16x2){0x0400, 0x0400});
    const uint32_t gt = as_u32(SS - d);  // bit 15 / 31: 2|w| > s
    pos[p] = gt & ~hw[p] & 0x80008000u;
    neg[p] = gt & hw[p] & 0x80008000u;
  }
  // weight 2p at bit 2p, weight 2p + 1 at bit 16 + 2p, then bit 2p + 1
  const uint32_t dp = (pos[0] >> 15) | (pos[1] >> 13) | (pos[2] >> 11) | (pos[3] >> 9);
  const uint32_t dn = (neg[0] >> 15) | (neg[1] >> 13) | (neg[2] >> 11) | (neg[3] >> 9);
  pb = (dp & 0x55u) | ((dp >> 15) & 0xAAu);
  nb = (dn & 0x55u) | ((dn >> 15) & 0xAAu);
}

// One lane per 8-weight chunk c of one 16-row tile, as the 1-bit quantiser.
// A (rolled) loop over four blocks of four rows: load them, reduce their
// group maxima over the 16 lanes of the group (two 16-bit maxima per
// shuffle), decide their 32 weights, and shift the block's pos and neg code
// words into place.  Only one block is live at a time, so the kernel keeps
// enough waves in flight to stream at HBM speed (unrolling the loop so that
// all four blocks' loads go out at once measured slower).  Groups with a
// finite scale -- all but those holding an infinity or a NaN -- are decided
// two weights at a time (chunk_trits_finite).
__global__ __launch_bounds__(kQBlock) void quantize_t2_kernel(const uint16_t* __restrict__ w,
                                                              int64_t n, int64_t k,
                                                              uint8_t* __restrict__ codes,
                                                              uint16_t* __restrict__ scales) {
  const int64_t chunks = k / kChunk;
  const int64_t cblocks = (chunks + kQBlock - 1) / kQBlock;
  const int64_t tile = blockIdx.x / cblocks;
  const int64_t c = (int64_t)(blockIdx.x - tile * cblocks) * kQBlock + threadIdx.x;
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
        mags |= chunk_max_mag(hw[2 * pr + u]) << (16 * u);
      }
#pragma unroll
      for (int d = 8; d >= 1; d >>= 1)
        mags = max_u16x2(mags, (uint32_t)__shfl_xor((int)mags, d, 16));
      if ((jr >> 1) == 2 * blk + pr) my_scale = (jr & 1) ? (mags >> 16) : (mags & 0xFFFFu);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t S = (mags >> (16 * u)) & 0xFFFFu;
        uint32_t pb = 0u, nb = 0u;
        if (S < 0x7C00u) {
          chunk_trits_finite(hw[2 * pr + u], S, pb, nb);
        } else {
          // a group holding an infinity or a NaN: weight by weight
#pragma unroll
          for (int j = 0; j < kChunk; ++j) {
            const uint32_t h = (hw[2 * pr + u][j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
            const uint32_t nz = twice_gt(h & 0x7FFFu, S) ? 1u : 0u;
            const uint32_t sgn = h >> 15;
            pb |= (nz & (sgn ^ 1u)) << j;
            nb |= (nz & sgn) << j;
          }
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

// Base-3 conversions: one work-group per 16-row tile, over K-blocks of 1280
// weights (256 base-3 bytes per row; a multiple of 5, 8 and 128, so no byte
// straddles two blocks) staged in LDS, so that HBM sees whole code cells
// and whole row segments.
constexpr int kKB = 1280;
constexpr int kKBChunks = kKB / kChunk;  // 160 code cells per tile and block
constexpr int kKBBytes = kKB / 5;        // 256 base-3 bytes per row and block

// two-plane codes + tile-major scales -> base-3 bytes + row-major scales.
// Thread t writes bytes 16 (t % 16) .. + 15 of the block of row t / 16: their
// 80 weights are chunks 10 (t % 16) .. + 9, whose pos and neg bytes it reads
// from LDS; a 1024-entry table maps (pos bits, neg bits) of 5 weights to the
// byte.  VEC (rows a multiple of 16 bytes long, output 16-byte aligned): the
// 16 bytes go out as one 16-byte store.
template <bool VEC>
__global__ __launch_bounds__(kBlock) void t2_to_base3_kernel(const uint8_t* __restrict__ codes,
                                                             const uint16_t* __restrict__ scales,
                                                             int64_t n, int64_t k,
                                                             uint8_t* __restrict__ out,
                                                             uint16_t* __restrict__ out_scales) {
  __shared__ uint4 cells[kKBChunks * 2];
  __shared__ uint8_t byte_of[1024];
  const int64_t tile = blockIdx.x;
  const int64_t chunks = k / kChunk, groups = k / kGroup, rb = (k + 4) / 5;
  const int t = threadIdx.x;
  for (int e = t; e < 1024; e += kBlock) {
    const int pb = e >> 5, nb = e & 31;
    int v = 0, pw = 1;
    for (int q = 0; q < 5; ++q) {
      v += (((pb >> q) & 1) - ((nb >> q) & 1) + 1) * pw;
      pw *= 3;
    }
    byte_of[e] = (uint8_t)v;
  }
  const int r = t >> 4, bg = t & 15;
  const int64_t row = tile * kTileRows + r;
  const uint8_t* cb = reinterpret_cast<const uint8_t*>(cells);
  for (int64_t k0 = 0; k0 < k; k0 += kKB) {
    const int64_t c0 = k0 / kChunk;
    const int nc = (int)(chunks - c0 < kKBChunks ? chunks - c0 : kKBChunks);
    __syncthreads();  // the previous block's cells have been read
    for (int i = t; i < kKBChunks * 2; i += kBlock)
      cells[i] = i < nc * 2 ? reinterpret_cast<const uint4*>(codes + (tile * chunks + c0) * 32)[i]
                            : make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    if (row >= n) continue;
    // the 80 pos / neg bits of this thread's weights, in two 40-bit halves
    uint32_t ob[4] = {0u, 0u, 0u, 0u};  // the thread's 16 bytes
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint64_t P = 0, N = 0;
#pragma unroll
      for (int cc = 0; cc < 5; ++cc) {
        const int c = bg * 10 + h * 5 + cc;
        P |= (uint64_t)cb[c * 32 + r] << (8 * cc);
        N |= (uint64_t)cb[c * 32 + 16 + r] << (8 * cc);
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const uint32_t v = byte_of[(((P >> (5 * jj)) & 31) << 5) | ((N >> (5 * jj)) & 31)];
        ob[(h * 8 + jj) >> 2] |= v << (8 * (jj & 3));
      }
    }
    const int64_t jo = k0 / 5 + bg * 16;  // first byte of the row
    if constexpr (VEC) {
      // rb and jo are multiples of 16: the 16 bytes are all in the row or
      // all past it
      if (jo < rb)
        *reinterpret_cast<uint4*>(out + row * rb + jo) = make_uint4(ob[0], ob[1], ob[2], ob[3]);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (jo + i < rb) out[row * rb + jo + i] = (uint8_t)(ob[i >> 2] >> (8 * (i & 3)));
    }
  }
  for (int i = t; i < kTileRows * groups; i += kBlock) {
    const int rr = (int)(i / groups);
    const int64_t g = i - (int64_t)rr * groups, rw = tile * kTileRows + rr;
    if (rw < n) out_scales[rw * groups + g] = scales[(tile * groups + g) * kTileRows + rr];
  }
}

// base-3 bytes + row-major scales -> two-plane codes + tile-major scales.  The
// block's 16 row segments are staged in LDS (rows past n as byte 121: every
// digit 1, t = 0; VEC as one 16-byte load per thread).  A 256-entry table
// gives the five pos bits (digit 2) and neg bits (digit 0) of every byte
// value, pos in bits 0..4 and neg in bits 16..20 (a byte of 243..255 decodes
// with its fifth digit taken mod 3).  An item (chunk, row) ORs the entries of
// the three bytes that hold its 8 weights, shifted by 0, 5 and 10, and cuts
// its pos and neg bytes out of the 15-bit runs at the chunk's first digit;
// the bytes go into the block's cells in LDS, which then go out as whole
// 16-byte vectors.
constexpr int kSegPitch = kKBBytes + 16;  // LDS row: 256 bytes + the item's third byte past the end

template <bool VEC>
__global__ __launch_bounds__(kBlock) void base3_to_t2_kernel(const uint8_t* __restrict__ in,
                                                             const uint16_t* __restrict__ in_scales,
                                                             int64_t n, int64_t k,
                                                             uint8_t* __restrict__ codes,
                                                             uint16_t* __restrict__ scales) {
  __shared__ uint4 segv[kTileRows * kSegPitch / 16];
  __shared__ uint4 cells[kKBChunks * 2];
  __shared__ uint32_t pn[256];
  const int64_t tile = blockIdx.x;
  const int64_t chunks = k / kChunk, groups = k / kGroup, rb = (k + 4) / 5;
  const int t = threadIdx.x;
  {
    int d = t;
    uint32_t pos = 0u, neg = 0u;
    for (int q = 0; q < 5; ++q) {
      const int dg = d % 3;  // t + 1 of weight q
      pos |= (uint32_t)(dg == 2) << q;
      neg |= (uint32_t)(dg == 0) << q;
      d /= 3;
    }
    pn[t] = pos | (neg << 16);
  }
  uint8_t* seg = reinterpret_cast<uint8_t*>(segv);
  uint8_t* cb = reinterpret_cast<uint8_t*>(cells);
  for (int64_t k0 = 0; k0 < k; k0 += kKB) {
    const int64_t c0 = k0 / kChunk;
    const int nc = (int)(chunks - c0 < kKBChunks ? chunks - c0 : kKBChunks);
    __syncthreads();  // the previous block's segments and cells have been read
    if constexpr (VEC) {
      // thread t: row t / 16, bytes 16 (t % 16) .. + 15 of its segment; rb
      // and the offsets are multiples of 16, so a vector is all in the row
      // or all past it
      const int rr = t >> 4, vj = t & 15;
      const int64_t rw = tile * kTileRows + rr, jo = k0 / 5 + vj * 16;
      uint4 v = make_uint4(0x79797979u, 0x79797979u, 0x79797979u, 0x79797979u);
      if (rw < n && jo < rb) v = *reinterpret_cast<const uint4*>(in + rw * rb + jo);
      segv[(rr * kSegPitch) / 16 + vj] = v;
    } else {
      for (int i = t; i < kTileRows * kKBBytes; i += kBlock) {
        const int rr = i / kKBBytes, jb = i % kKBBytes;
        const int64_t rw = tile * kTileRows + rr, jo = k0 / 5 + jb;
        seg[rr * kSegPitch + jb] = (rw < n && jo < rb) ? in[rw * rb + jo] : (uint8_t)121;
      }
    }
    __syncthreads();
    for (int it = t; it < nc * kTileRows; it += kBlock) {
      const int c = it >> 4, rr = it & 15;
      const int j0 = (c * kChunk) / 5;
      const int off = c * kChunk - 5 * j0;  // digit of weight 0 of the chunk
      const uint8_t* sr = seg + rr * kSegPitch + j0;
      // bytes j0, j0 + 1 and j0 + 2 (the last only when off >= 3; at the
      // block's end it is padding, whose bits are never cut out)
      const uint32_t e = pn[sr[0]] | (pn[sr[1]] << 5) | (pn[sr[2]] << 10);
      cb[c * 32 + rr] = (uint8_t)(e >> off);
      cb[c * 32 + 16 + rr] = (uint8_t)(e >> (16 + off));
    }
    __syncthreads();
    uint4* dst = reinterpret_cast<uint4*>(codes + (tile * chunks + c0) * 32);
    for (int i = t; i < nc * 2; i += kBlock) dst[i] = cells[i];
  }
  for (int i = t; i < kTileRows * groups; i += kBlock) {
    const int rr = (int)(i / groups);
    const int64_t g = i - (int64_t)rr * groups, rw = tile * kTileRows + rr;
    scales[(tile * groups + g) * kTileRows + rr] = rw < n ? in_scales[rw * groups + g] : (uint16_t)0;
  }
}

// one work-group per (tile, block of kQBlock chunks), the blocks of a tile
// consecutive, as for the 1-bit quantiser
dim3 tile_grid(int64_t n, int64_t k) {
  const int64_t tiles = (n + kTileRows - 1) / kTileRows;
  const int64_t cblocks = (k / kChunk + kQBlock - 1) / kQBlock;
  return dim3((unsigned)(tiles * cblocks));
}

}  // namespace

hipError_t launch_quantize_t2(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                              uint16_t* scales, hipStream_t st) {
  hipLaunchKernelGGL(quantize_t2_kernel, tile_grid(n, k), dim3(kQBlock), 0, st, w, n, k, codes,
                     scales);
  return hipGetLastError();
}

// 16-byte row vectors of the base-3 buffer: rows a multiple of 16 bytes
// long (k a multiple of 80) and the buffer 16-byte aligned
static bool base3_vec(const void* p, int64_t k) {
  return ((k + 4) / 5) % 16 == 0 && (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

hipError_t launch_t2_to_base3(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                              uint8_t* out, uint16_t* out_scales, hipStream_t st) {
  const int64_t tiles = (n + kTileRows - 1) / kTileRows;
  if (base3_vec(out, k))
    hipLaunchKernelGGL(t2_to_base3_kernel<true>, dim3((unsigned)tiles), dim3(kBlock), 0, st,
                       codes, scales, n, k, out, out_scales);
  else
    hipLaunchKernelGGL(t2_to_base3_kernel<false>, dim3((unsigned)tiles), dim3(kBlock), 0, st,
                       codes, scales, n, k, out, out_scales);
  return hipGetLastError();
}

hipError_t launch_base3_to_t2(const uint8_t* in, const uint16_t* in_scales, int64_t n, int64_t k,
                              uint8_t* codes, uint16_t* scales, hipStream_t st) {
  const int64_t tiles = (n + kTileRows - 1) / kTileRows;
  if (base3_vec(in, k))
    hipLaunchKernelGGL(base3_to_t2_kernel<true>, dim3((unsigned)tiles), dim3(kBlock), 0, st, in,
                       in_scales, n, k, codes, scales);
  else
    hipLaunchKernelGGL(base3_to_t2_kernel<false>, dim3((unsigned)tiles), dim3(kBlock), 0, st, in,
                       in_scales, n, k, codes, scales);
  return hipGetLastError();
}

}  // namespace lowbit
