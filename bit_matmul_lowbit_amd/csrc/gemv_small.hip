// Decode GEMV for small matrices, b = 1..8, in ONE launch:
//   y[i][n] = sum_g s[n][g] * sum_{k in g} t[n][k] * x[i][k]
//
// [P2] 7minutos.es, "PrismML lanza Bonsai 27B ...": decode streams every
//      low-bit matrix once per token ("Rendimiento y decodificacion
//      especulativa DSpark").
// [P1] 7minutos.es tutorial, section 7: bit 0 -> -s, bit 1 -> +s.
// [P5] openclawradar.com, "Bonsai 1.7B ...", "Detalles tecnicos": decode
//      of the small model was tuned at the level of its matvec / FFN kernels.
//
// A matrix of a few MB is latency-bound: the table GEMV spends its time in
// two dependent launches (prepare, then accumulate), the table build, a
// K-sliced sweep and FP32 atomics.  Here one work-group owns one 16-row tile
// (or, for a matrix with fewer tiles than twice the CUs, half a tile) over
// the whole of K and writes its outputs with plain stores, so there is no
// prepare launch, no workspace, no atomics and no zeroed y:
//   * wave w takes K-range [512 w, 512 w + 512) (64 chunks of 8 weights);
//     lane (rho = l % 16, q = l / 16) takes row rho of the tile and chunks
//     q, q + 4, ..., q + 60 of that range (16 chunks, 4 groups); with half
//     tiles, lane (l % 8, l / 8) takes one of the 8 rows and chunks q,
//     q + 8, ..., q + 56 (8 chunks);
//   * every load of the lane is issued at once: one code dword per chunk
//     (rows 4 (rho / 4) .. + 3 of the cell; ternary: pos and neg), one scale
//     dword per group (rows rho & ~1, + 1), and, for b <= 2, x as 16-byte
//     FP16 vectors; for b >= 3 (k <= 4096) the work-group copies x into LDS
//     once while those loads are in flight, and lanes read it from there;
//   * the code byte of row rho goes to the low byte of both 16-bit halves
//     (v_perm), a packed shift and v_bitop3 turn each bit pair into FP16
//     (+s or -s; ternary also 0) and v_dot2_f32_f16 adds (+-s) x for two
//     weights at a time into an FP32 sum -- products of two FP16 numbers are
//     exact in FP32;
//   * the lanes of a row are summed across lanes, the waves' sums through
//     LDS, and y is stored once.
// The FFN variant (SILU) takes h = [gate | up] (FP32 [b][2k]) instead of x
// and forms z = RNE_fp16(SiLU(gate) * up) itself: lane l of wave w forms
// chunk 64 w + l into LDS, from where the lanes that need it read it.
#include "common.h"

namespace lowbit {
namespace {

constexpr int kWaveK = 512;           // weights of K per wave
constexpr int kLaneChunks = 16;       // chunks per lane
constexpr int kMaxWaves = 16;         // K <= 8192

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                false);
}

__device__ __forceinline__ uint32_t dload(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
}

__device__ __forceinline__ uint4 qload(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t word(const uint4& v, int p) {
  return p == 0 ? v.x : p == 1 ? v.y : p == 2 ? v.z : v.w;
}

// per-half arithmetic shift right by 15: 0xFFFF where bit 15 is set, else 0
__device__ __forceinline__ uint32_t mask15(uint32_t d) {
  const s16x2 a = __builtin_bit_cast(s16x2, d);
  return __builtin_bit_cast(uint32_t, (s16x2)(a >> (s16x2){15, 15}));
}

constexpr int kMaxKLds = 4096;        // k limit when x (or z) sits in LDS, b >= 3
constexpr int kHalfTileBelow = 2;     // half-tile work-groups below this many tiles per CU

template <int B>
constexpr int max_waves() { return B <= 2 ? kMaxWaves : kMaxKLds / kWaveK; }

// RH = rows per work-group: 16 (a tile), or 8 (half a tile, for matrices
// with fewer tiles than twice the CUs: twice the work-groups, each lane half
// the chunks).  Lane (rho, q): row rho of the work-group's RH rows, chunks
// q, q + QN, ... of the wave's range (QN = 64 / RH lanes per row).
template <int FMT, int B, bool SILU, int RH>
__global__ __launch_bounds__(64 * max_waves<B>()) void gemv_direct_kernel(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const void* __restrict__ xin, int64_t n, int64_t k, float* __restrict__ y) {
  constexpr int CB = Fmt<FMT>::cell_bytes;
  constexpr int QN = 64 / RH;               // lanes per row
  constexpr int LC = kLaneChunks * 4 / QN;  // chunks per lane
  static_assert(RH == 16 || RH == 8, "a tile or half a tile per work-group");
  constexpr bool XLDS = !SILU && B >= 3;  // x staged in LDS
  __shared__ uint4 zbuf[SILU ? max_waves<B>() * 64 * B : 1];
  __shared__ uint4 xbuf[XLDS ? B * kMaxKLds / 8 : 1];
  __shared__ float red[max_waves<B>() * RH * B];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = (int)(blockDim.x >> 6);
  const int64_t tile = RH == 16 ? blockIdx.x : blockIdx.x >> 1;
  const int r0 = RH == 16 ? 0 : (int)(blockIdx.x & 1) * 8;  // first row in the tile
  const int rho = r0 + (lane % RH), q = lane / RH;             // row in the tile, chunk lane
  const int64_t nch = k / kChunk;
  const int64_t G = k / kGroup;
  const int c0 = wave * (kWaveK / kChunk);  // first chunk of the wave
  // chunks past k (last wave of a k that is not a multiple of 512) read as
  // zeros: codes and scales past their resource, x by the kNoLoad offset
  const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(codes + tile * nch * CB, nch * CB);
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(scales + tile * G * 16, G * 32);
  constexpr uint32_t kNoLoad = 0x80000000u;

  // chunk c0 + q + QN i lies in group c0 / 16 + (q + QN i) / 16 = c0 / 16 + i / (16 / QN)
  constexpr int IPG = 16 / QN;  // a lane's chunks per group
  uint32_t cw[LC], nwd[FMT == 2 ? LC : 1], sw[LC / IPG];
#pragma unroll
  for (int i = 0; i < LC; ++i) {
    const uint32_t off = (uint32_t)((c0 + q + QN * i) * CB + (rho & 12));
    cw[i] = dload(rc, off);
    if constexpr (FMT == 2) nwd[i] = dload(rc, off + 16);
  }
#pragma unroll
  for (int j = 0; j < LC / IPG; ++j)
    sw[j] = dload(rs, (uint32_t)(((c0 / 16 + j) * 16 + (rho & 14)) * 2));

  uint4 xv[SILU || XLDS ? 1 : LC][B];
  const int pitch = nw * 64;  // chunks per x row in LDS: zeros past k
  if constexpr (XLDS) {
    // x [B][k] FP16 into LDS, 16 bytes per thread and round
    const uint4* x4 = static_cast<const uint4*>(xin);
    for (int v = threadIdx.x; v < B * pitch; v += blockDim.x) {
      const int bi = v / pitch, c = v - bi * pitch;
      xbuf[v] = c < nch ? x4[bi * nch + c] : make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();
  } else if constexpr (SILU) {
    // z of chunk c0 + lane, all batch rows, into LDS (zeros past k)
    const float* h = static_cast<const float*>(xin);
    const int64_t c = c0 + lane;
#pragma unroll
    for (int bi = 0; bi < B; ++bi) {
      uint4 z = make_uint4(0u, 0u, 0u, 0u);
      if (c < nch) {
        const float4* g4 = reinterpret_cast<const float4*>(h + bi * 2 * k + c * 8);
        const float4* u4 = reinterpret_cast<const float4*>(h + bi * 2 * k + k + c * 8);
        const float4 ga = g4[0], gb = g4[1], ua = u4[0], ub = u4[1];
        const float gv[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
        const float uv[8] = {ua.x, ua.y, ua.z, ua.w, ub.x, ub.y, ub.z, ub.w};
        z = silu_mul8(gv, uv);
      }
      zbuf[(wave * 64 + lane) * B + bi] = z;
    }
    __syncthreads();
  } else {
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(xin, B * k * 2);
#pragma unroll
    for (int i = 0; i < LC; ++i) {
      const int c = c0 + q + QN * i;
#pragma unroll
      for (int bi = 0; bi < B; ++bi)
        xv[i][bi] = qload(rx, c < nch ? (uint32_t)((bi * k + c * 8) * 2) : kNoLoad);
    }
  }

  // byte rho & 3 of a code dword in the low byte of both halves; the scale
  // of row rho in both halves
  const uint32_t bsel = 0x0C000C00u | ((uint32_t)(rho & 3) << 16) | (uint32_t)(rho & 3);
  const uint32_t ssel = (rho & 1) ? 0x03020302u : 0x01000100u;
  float acc[B];
#pragma unroll
  for (int bi = 0; bi < B; ++bi) acc[bi] = 0.0f;
#pragma unroll
  for (int i = 0; i < LC; ++i) {
    const uint32_t ss = __builtin_amdgcn_perm(sw[i / IPG], sw[i / IPG], ssel);
    uint4 xi[B];
#pragma unroll
    for (int bi = 0; bi < B; ++bi) {
      if constexpr (SILU) {
        xi[bi] = zbuf[(wave * 64 + q + QN * i) * B + bi];
      } else if constexpr (XLDS) {
        xi[bi] = xbuf[bi * pitch + c0 + q + QN * i];
      } else {
        xi[bi] = xv[i][bi];
      }
    }
    if constexpr (FMT == 1) {
      const uint32_t d = __builtin_amdgcn_perm(cw[i], cw[i], bsel);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t sh = ((uint32_t)(14 - 2 * p) << 16) | (uint32_t)(15 - 2 * p);
        const uint32_t a = ss ^ (~pk_shl(d, sh) & kSignBits);
#pragma unroll
        for (int bi = 0; bi < B; ++bi) acc[bi] = dot2(a, word(xi[bi], p), acc[bi]);
      }
    } else {
      const uint32_t dq = __builtin_amdgcn_perm(nwd[i], nwd[i], bsel);        // neg
      const uint32_t dn = __builtin_amdgcn_perm(cw[i] ^ nwd[i], cw[i] ^ nwd[i], bsel);  // nonzero
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t sh = ((uint32_t)(14 - 2 * p) << 16) | (uint32_t)(15 - 2 * p);
        const uint32_t a = (ss ^ (pk_shl(dq, sh) & kSignBits)) & mask15(pk_shl(dn, sh));
#pragma unroll
        for (int bi = 0; bi < B; ++bi) acc[bi] = dot2(a, word(xi[bi], p), acc[bi]);
      }
    }
  }
  // the QN lanes of a row, then the waves
#pragma unroll
  for (int bi = 0; bi < B; ++bi) {
    if constexpr (QN == 8) acc[bi] += __shfl_xor(acc[bi], 8);
    acc[bi] += __shfl_xor(acc[bi], 16);
    acc[bi] += __shfl_xor(acc[bi], 32);
  }
  if (q == 0) {
#pragma unroll
    for (int bi = 0; bi < B; ++bi) red[wave * RH * B + bi * RH + (rho - r0)] = acc[bi];
  }
  __syncthreads();
  // RH B outputs; a work-group of one wave (k <= 512) may have fewer threads
  for (int t = threadIdx.x; t < RH * B; t += blockDim.x) {
    float sum = 0.0f;
    for (int w = 0; w < nw; ++w) sum += red[w * RH * B + t];
    const int64_t row = tile * kTileRows + r0 + (t % RH);
    if (row < n) y[(t / RH) * n + row] = sum;
  }
}

template <int FMT, int B, bool SILU>
hipError_t launch_direct(const uint8_t* codes, const uint16_t* scales, const void* xin, int64_t n,
                         int64_t k, float* y, hipStream_t st) {
  const int64_t ntiles = (n + kTileRows - 1) / kTileRows;
  const int nw = (int)((k + kWaveK - 1) / kWaveK);
  if (ntiles < kHalfTileBelow * (int64_t)device_cu_count())
    hipLaunchKernelGGL((gemv_direct_kernel<FMT, B, SILU, 8>), dim3((unsigned)(2 * ntiles)),
                       dim3(64 * nw), 0, st, codes, scales, xin, n, k, y);
  else
    hipLaunchKernelGGL((gemv_direct_kernel<FMT, B, SILU, 16>), dim3((unsigned)ntiles),
                       dim3(64 * nw), 0, st, codes, scales, xin, n, k, y);
  return hipGetLastError();
}

template <int FMT, bool SILU>
hipError_t launch_direct_b(const uint8_t* codes, const uint16_t* scales, const void* xin,
                           int64_t n, int64_t k, int64_t b, float* y, hipStream_t st) {
  switch (b) {
    case 1: return launch_direct<FMT, 1, SILU>(codes, scales, xin, n, k, y, st);
    case 2: return launch_direct<FMT, 2, SILU>(codes, scales, xin, n, k, y, st);
    case 3: return launch_direct<FMT, 3, SILU>(codes, scales, xin, n, k, y, st);
    case 4: return launch_direct<FMT, 4, SILU>(codes, scales, xin, n, k, y, st);
    case 5: return launch_direct<FMT, 5, SILU>(codes, scales, xin, n, k, y, st);
    case 6: return launch_direct<FMT, 6, SILU>(codes, scales, xin, n, k, y, st);
    case 7: return launch_direct<FMT, 7, SILU>(codes, scales, xin, n, k, y, st);
    default: return launch_direct<FMT, 8, SILU>(codes, scales, xin, n, k, y, st);
  }
}

}  // namespace

bool gemv_direct_ok(int64_t n, int64_t k, int64_t b) {
  if (b < 1 || b > 8) return false;
  if (k > (b == 1 ? 8192 : b == 2 ? 4096 : kMaxKLds)) return false;
  return n * k * (b <= 2 ? 1 : b) <= kDirectMaxWeights * (b <= 2 ? 1 : kDirectBatchWeight);
}

hipError_t launch_gemv_direct(int fmt, const uint8_t* codes, const uint16_t* scales, int64_t n,
                              int64_t k, const uint16_t* x, int64_t b, float* y, hipStream_t st) {
  return fmt == 1 ? launch_direct_b<1, false>(codes, scales, x, n, k, b, y, st)
                  : launch_direct_b<2, false>(codes, scales, x, n, k, b, y, st);
}

hipError_t launch_gemv_direct_silu(int fmt, const uint8_t* codes, const uint16_t* scales,
                                   int64_t n, int64_t f, const float* h, int64_t b, float* y,
                                   hipStream_t st) {
  return fmt == 1 ? launch_direct_b<1, true>(codes, scales, h, n, f, b, y, st)
                  : launch_direct_b<2, true>(codes, scales, h, n, f, b, y, st);
}

}  // namespace lowbit
