// Prefill GEMM  Y[i][n] = sum_g s[n][g] * sum_{k in g} X[i][k] * t[n][k]
// with X in BF16 [m][k] and W in Q1_0_g128 or ternary g128 codes.
//
// [P2] 7minutos.es, "PrismML lanza Bonsai 27B ...", "Rendimiento y
//      decodificacion especulativa DSpark": prefill is compute-bound.
// [P1] 7minutos.es tutorial, section 7: bit 0 -> -s, bit 1 -> +s.
// [P2] "Como funciona la compresion": w = s * t, t in {-1, 0, +1}.
//
// Tiling: a 256-thread work-group owns a 128 x 128 output tile; its 4 waves
// form a 2 x 2 grid and each wave owns 64 x 64 outputs = 2 x 2 blocks of the
// 32x32x16 BF16 matrix-core instruction.  The K loop steps one scale group
// (128) at a time:
//   * X[128 rows][128] (32 KB) is copied to LDS;
//   * the codes of W[128 rows][128] (2 KB Q1 / 4 KB T2) are expanded to exact
//     BF16 {-1, 0, +1} (32 KB) in LDS -- the scale is NOT folded in, since a
//     BF16 scale would lose 3 of FP16's 11 significant bits;
//   * 8 k-steps of 16 accumulate the group's unscaled FP32 partial C_g;
//   * C += s[n][g] * C_g in FP32 (one FMA per accumulator);
// and the next group's global loads are in flight while the current group
// is contracted.  LDS rows are 256 B with 16-byte slots XOR-swizzled by the
// row index, so the 16-lane phases of every 16-byte LDS access hit 16
// different slots (no bank conflicts, no padding: 64 KB total).
// The epilogue rounds to BF16 (nearest-even) once, or stores FP32.
#include "common.h"

namespace lowbit {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kThreads = 256;
constexpr int kRowU4 = BK / 8;  // 16-byte slots per LDS row

// LDS uint4 index of 16-byte slot c of row r (XOR swizzle)
__device__ __forceinline__ int slot(int r, int c) { return r * kRowU4 + (c ^ (r & 15)); }

// 8 Q1 bits (LSB = first k) -> 8 BF16 values +1 (bit 1) / -1 (bit 0)
__device__ __forceinline__ uint4 expand_q1(uint32_t b) {
  const uint32_t nb = ~b;
  uint32_t d[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    d[q] = 0x3F803F80u | (((nb >> (2 * q)) & 1u) << 15) | (((nb >> (2 * q + 1)) & 1u) << 31);
  return make_uint4(d[0], d[1], d[2], d[3]);
}

// pos / neg bytes -> 8 BF16 values t = pos - neg in {-1, 0, +1}
__device__ __forceinline__ uint4 expand_t2(uint32_t p, uint32_t q) {
  const uint32_t nz = p ^ q;     // exactly one of pos / neg set
  const uint32_t ng = q & ~p;    // t = -1
  uint32_t d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = ((nz >> (2 * i)) & 1u) * 0x3F80u | (((ng >> (2 * i)) & 1u) << 15);
    const uint32_t hi = ((nz >> (2 * i + 1)) & 1u) * 0x3F80u | (((ng >> (2 * i + 1)) & 1u) << 15);
    d[i] = lo | (hi << 16);
  }
  return make_uint4(d[0], d[1], d[2], d[3]);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;  // NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int FMT, bool OUT_F32>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ x, int64_t m, int64_t n, int64_t k, void* __restrict__ y) {
  __shared__ uint4 xs[BM * kRowU4];  // 32 KB
  __shared__ uint4 ws[BN * kRowU4];  // 32 KB

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const int64_t groups = k / BK;
  const int64_t chunks = k / kChunk;
  const int64_t ntiles = (n + kTileRows - 1) / kTileRows;
  constexpr int CB = Fmt<FMT>::cell_bytes;

  // this thread's share of the staging copies
  // X: 2048 slots of 16 B, 8 per thread: slot i = tid + 256 j -> row i/16, col i%16
  // W: 8 row tiles x 16 cells; thread -> (tile wt = tid/32, cell wc = (tid%32)/2,
  //    half wh = tid%2): the 8 rows 8*wh .. 8*wh+7 of that cell
  const int wt = tid >> 5, wc = (tid & 31) >> 1, wh = tid & 1;
  const int64_t gtile = n0 / kTileRows + wt;
  const bool wvalid = gtile < ntiles;

  uint4 xr[8];
  uint2 cr[2];  // Q1: cr[0] = 8 row bytes; T2: cr[0] pos, cr[1] neg

  auto load_group = [&](int64_t g) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = tid + kThreads * j;
      const int64_t row = m0 + (i >> 4);
      xr[j] = row < m ? *reinterpret_cast<const uint4*>(x + row * k + g * BK + (i & 15) * 8)
                      : make_uint4(0u, 0u, 0u, 0u);
    }
    if (wvalid) {
      const uint8_t* cell = codes + (gtile * chunks + g * kChunksPerGroup + wc) * CB + 8 * wh;
      cr[0] = *reinterpret_cast<const uint2*>(cell);
      if constexpr (FMT == 2) cr[1] = *reinterpret_cast<const uint2*>(cell + 16);
    } else {
      cr[0] = make_uint2(0u, 0u);
      cr[1] = make_uint2(0u, 0u);
    }
  };

  // scales of this lane's two output columns (one per n-block)
  const int jl = lane & 31;
  int64_t ncol[2];
  bool nvalid[2];
#pragma unroll
  for (int bj = 0; bj < 2; ++bj) {
    ncol[bj] = n0 + wn * 64 + bj * 32 + jl;
    nvalid[bj] = ncol[bj] < n;
  }
  auto load_scale = [&](int64_t g, int bj) -> float {
    if (!nvalid[bj]) return 0.0f;
    const int64_t nn = ncol[bj];
    const uint16_t h = scales[((nn >> 4) * groups + g) * kTileRows + (nn & 15)];
    return (float)__builtin_bit_cast(_Float16, h);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[bi][bj][v] = 0.0f;

  load_group(0);
  const int kh = lane >> 5;  // which 8 of the 16 k of a step this lane holds

  for (int64_t g = 0; g < groups; ++g) {
    __syncthreads();  // previous group's contraction is done with LDS
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = tid + kThreads * j;
      xs[slot(i >> 4, i & 15)] = xr[j];
    }
    {
      const uint32_t pw[2] = {cr[0].x, cr[0].y};
      const uint32_t nw[2] = {cr[1].x, cr[1].y};
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const uint32_t pb = (pw[rr >> 2] >> ((rr & 3) * 8)) & 0xFFu;
        uint4 e;
        if constexpr (FMT == 1) e = expand_q1(pb);
        else e = expand_t2(pb, (nw[rr >> 2] >> ((rr & 3) * 8)) & 0xFFu);
        ws[slot(wt * 16 + wh * 8 + rr, wc)] = e;
      }
    }
    __syncthreads();
    if (g + 1 < groups) load_group(g + 1);
    const float s0 = load_scale(g, 0), s1 = load_scale(g, 1);

    f32x16 cg[2][2];
#pragma unroll
    for (int step = 0; step < BK / 16; ++step) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
        a[bi] = __builtin_bit_cast(bf16x8, xs[slot(wm * 64 + bi * 32 + jl, step * 2 + kh)]);
#pragma unroll
      for (int bj = 0; bj < 2; ++bj)
        b[bj] = __builtin_bit_cast(bf16x8, ws[slot(wn * 64 + bj * 32 + jl, step * 2 + kh)]);
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) {
          if (step == 0) {
            const f32x16 zero = {};
            cg[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[bi], b[bj], zero, 0, 0, 0);
          } else {
            cg[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[bi], b[bj], cg[bi][bj], 0, 0, 0);
          }
        }
    }
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        acc[bi][0][v] = __builtin_fmaf(s0, cg[bi][0][v], acc[bi][0][v]);
        acc[bi][1][v] = __builtin_fmaf(s1, cg[bi][1][v], acc[bi][1][v]);
      }
  }

  // epilogue: C[i][j] of a 32x32 block sits in lane j + 32*((i/4)%2), register
  // (i%4) + 4*(i/8)
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      if (!nvalid[bj]) continue;
      const int64_t nn = ncol[bj];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = 8 * (v >> 2) + 4 * kh + (v & 3);
        const int64_t mm = m0 + wm * 64 + bi * 32 + i;
        if (mm >= m) continue;
        if constexpr (OUT_F32)
          static_cast<float*>(y)[mm * n + nn] = acc[bi][bj][v];
        else
          static_cast<uint16_t*>(y)[mm * n + nn] = f32_to_bf16_rne(acc[bi][bj][v]);
      }
    }
}

template <int FMT>
hipError_t launch_fmt(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                      const uint16_t* x, int64_t m, void* y, bool out_f32, hipStream_t st) {
  const dim3 grid((unsigned)((n + BN - 1) / BN), (unsigned)((m + BM - 1) / BM));
  if (out_f32)
    hipLaunchKernelGGL((gemm_kernel<FMT, true>), grid, dim3(kThreads), 0, st, codes, scales, x, m,
                       n, k, y);
  else
    hipLaunchKernelGGL((gemm_kernel<FMT, false>), grid, dim3(kThreads), 0, st, codes, scales, x,
                       m, n, k, y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int fmt, const uint8_t* codes, const uint16_t* scales, int64_t n,
                       int64_t k, const uint16_t* x, int64_t m, void* y, bool out_f32,
                       hipStream_t st) {
  if (fmt == 1) return launch_fmt<1>(codes, scales, n, k, x, m, y, out_f32, st);
  return launch_fmt<2>(codes, scales, n, k, x, m, y, out_f32, st);
}

}  // namespace lowbit
