// Prefill GEMM  Y[i][n] = sum_g s[n][g] * sum_{k in g} X[i][k] * t[n][k]
// with X in BF16 [m][k] and W in Q1_0_g128 or ternary g128 codes.
//
// [P2] 7minutos.es, "PrismML lanza Bonsai 27B ...", "Rendimiento y
//      decodificacion especulativa DSpark": prefill is compute-bound.
// [P1] 7minutos.es tutorial, section 7: bit 0 -> -s, bit 1 -> +s.
// [P2] "Como funciona la compresion": w = s * t, t in {-1, 0, +1}.
//
// Tiling: a 256-thread work-group owns a BM x BN output tile (128 x 128 or
// 64 x 64); its 4 waves form a 2 x 2 grid of (BM/2) x (BN/2) wave tiles made
// of 32x32 blocks of the 32x32x16 BF16 matrix-core instruction.  The K loop
// steps one scale group (128) at a time through double-buffered LDS:
//   * X[BM][128] BF16, the codes of W[BN][128] and the scales are loaded
//     into registers one group ahead; after the current group's MFMAs are
//     issued they are written to the other LDS buffer, the codes expanded to
//     exact BF16 {-1, 0, +1}.  The scale is NOT folded in: a BF16 scale
//     would lose 3 of FP16's 11 significant bits;
//   * 8 k-steps of 16 accumulate the group's unscaled FP32 partial C_g, then
//     C += s[n][g] * C_g in FP32 (one FMA per accumulator).
// LDS rows are 256 B whose 16-byte slots are XOR-swizzled by the row index, so
// every 16-lane phase of a 16-byte LDS access hits 16 different slots.
// The epilogue rounds to BF16 (nearest-even) once, or stores FP32.
#include "common.h"

namespace lowbit {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int BK = 128;
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
  const uint32_t nz = p ^ q;   // exactly one of pos / neg set
  const uint32_t ng = q & ~p;  // t = -1
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

template <int FMT, bool OUT_F32, int BM, int BN>
__global__ __launch_bounds__(kThreads, (BM * BN >= 128 * 128) ? 1 : 2) void gemm_kernel(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ x, int64_t m, int64_t n, int64_t k, void* __restrict__ y) {
  constexpr int WBM = BM / 64;                    // 32-row blocks per wave
  constexpr int WBN = BN / 64;                    // 32-col blocks per wave
  constexpr int XL = BM * kRowU4 / kThreads;      // 16-B X slots per thread per group
  constexpr int CB = Fmt<FMT>::cell_bytes;
  constexpr int RPT = BN / 16;                    // W rows expanded per thread per group
  constexpr int TPC = 16 / RPT;                   // threads per code cell

  __shared__ uint4 xs[2][BM * kRowU4];
  __shared__ uint4 ws[2][BN * kRowU4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const int64_t groups = k / BK;
  const int64_t chunks = k / kChunk;
  const int64_t ntiles = (n + kTileRows - 1) / kTileRows;

  // --- X staging: slot i = tid + 256*j is row i/16, 16-byte column i%16 of
  // the group; rows past m read row m-1 (those outputs are never stored).
  const uint16_t* xsrc[XL];
  int xdst[XL];
#pragma unroll
  for (int j = 0; j < XL; ++j) {
    const int i = tid + kThreads * j;
    int64_t row = m0 + (i >> 4);
    if (row >= m) row = m - 1;
    xsrc[j] = x + row * k + (i & 15) * 8;
    xdst[j] = slot(i >> 4, i & 15);
  }

  // --- W codes: thread -> cell ci = tid / TPC (row tile ci/16, chunk ci%16
  // of the group), rows part*RPT .. part*RPT + RPT-1 of that cell
  const int ci = tid / TPC, part = tid % TPC;
  const int wt = ci >> 4, wc = ci & 15;
  const int64_t gtile = n0 / kTileRows + wt;
  const bool wvalid = gtile < ntiles;
  const uint8_t* wsrc = codes + ((wvalid ? gtile : 0) * chunks + wc) * CB + part * RPT;
  int wdst[RPT];
#pragma unroll
  for (int rr = 0; rr < RPT; ++rr) wdst[rr] = slot(wt * 16 + part * RPT + rr, wc);

  // --- scales of this lane's output columns (one per n-block)
  const int jl = lane & 31;
  int64_t ncol[WBN];
  bool nvalid[WBN];
  const uint16_t* sptr[WBN];
#pragma unroll
  for (int bj = 0; bj < WBN; ++bj) {
    ncol[bj] = n0 + wn * (BN / 2) + bj * 32 + jl;
    nvalid[bj] = ncol[bj] < n;
    const int64_t nn = nvalid[bj] ? ncol[bj] : 0;
    sptr[bj] = scales + ((nn >> 4) * groups) * kTileRows + (nn & 15);
  }

  // Prefetched data stays raw until it is used one iteration later (a
  // select on a just-loaded value would force an immediate wait).  Invalid
  // tiles / columns load from valid addresses and are zeroed at use.
  constexpr int CW = (RPT * 1 + 3) / 4;  // code words per plane per thread
  struct Stage {
    uint4 xr[XL];
    uint32_t p[CW], q[CW];
    uint16_t sh[WBN];
  };
  auto fetch = [&](int64_t g, Stage& st) {
#pragma unroll
    for (int j = 0; j < XL; ++j) st.xr[j] = *reinterpret_cast<const uint4*>(xsrc[j] + g * BK);
    const uint8_t* cell = wsrc + g * kChunksPerGroup * CB;
    if constexpr (RPT == 8) {
      const uint2 a = *reinterpret_cast<const uint2*>(cell);
      st.p[0] = a.x;
      st.p[1] = a.y;
      if constexpr (FMT == 2) {
        const uint2 c2 = *reinterpret_cast<const uint2*>(cell + 16);
        st.q[0] = c2.x;
        st.q[1] = c2.y;
      }
    } else {
      st.p[0] = *reinterpret_cast<const uint32_t*>(cell);
      if constexpr (FMT == 2) st.q[0] = *reinterpret_cast<const uint32_t*>(cell + 16);
    }
#pragma unroll
    for (int bj = 0; bj < WBN; ++bj) st.sh[bj] = sptr[bj][g * kTileRows];
  };
  auto stash = [&](const Stage& st, int b) {
#pragma unroll
    for (int j = 0; j < XL; ++j) xs[b][xdst[j]] = st.xr[j];
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
      const uint32_t pb = wvalid ? (st.p[rr >> 2] >> ((rr & 3) * 8)) & 0xFFu : 0u;
      uint4 e;
      if constexpr (FMT == 1) e = expand_q1(pb);
      else e = expand_t2(pb, wvalid ? (st.q[rr >> 2] >> ((rr & 3) * 8)) & 0xFFu : 0u);
      ws[b][wdst[rr]] = e;
    }
  };
  auto scale_of = [&](const Stage& st, int bj) {
    return nvalid[bj] ? (float)__builtin_bit_cast(_Float16, st.sh[bj]) : 0.0f;
  };

  f32x16 acc[WBM][WBN];
#pragma unroll
  for (int bi = 0; bi < WBM; ++bi)
#pragma unroll
    for (int bj = 0; bj < WBN; ++bj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[bi][bj][v] = 0.0f;

  // prologue: group 0 into LDS buffer 0
  Stage cur, nxt;
  fetch(0, cur);
  stash(cur, 0);
  float sv[WBN];
#pragma unroll
  for (int bj = 0; bj < WBN; ++bj) sv[bj] = scale_of(cur, bj);
  __syncthreads();

  const int kh = lane >> 5;  // which 8 of the 16 k of a step this lane holds
  for (int64_t g = 0; g < groups; ++g) {
    const int b = (int)(g & 1);
    // next group's data (the last iteration re-fetches the last group into
    // a buffer nobody reads, which keeps the loop body branch-free); the
    // scheduling barrier keeps these loads at the top of the iteration
    fetch(g + 1 < groups ? g + 1 : g, nxt);
    __builtin_amdgcn_sched_barrier(0);

    f32x16 cg[WBM][WBN];
#pragma unroll
    for (int step = 0; step < BK / 16; ++step) {
      bf16x8 a[WBM], bb[WBN];
#pragma unroll
      for (int bi = 0; bi < WBM; ++bi)
        a[bi] = __builtin_bit_cast(bf16x8, xs[b][slot(wm * (BM / 2) + bi * 32 + jl, step * 2 + kh)]);
#pragma unroll
      for (int bj = 0; bj < WBN; ++bj)
        bb[bj] = __builtin_bit_cast(bf16x8, ws[b][slot(wn * (BN / 2) + bj * 32 + jl, step * 2 + kh)]);
#pragma unroll
      for (int bi = 0; bi < WBM; ++bi)
#pragma unroll
        for (int bj = 0; bj < WBN; ++bj) {
          if (step == 0) {
            const f32x16 zero = {};
            cg[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[bi], bb[bj], zero, 0, 0, 0);
          } else {
            cg[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[bi], bb[bj], cg[bi][bj], 0, 0, 0);
          }
        }
    }
    // stage the next group into the other buffer (last read one iteration
    // ago, before the barrier) while the matrix cores drain; the scheduling
    // barrier keeps this work (which waits for the prefetch) below the MFMAs
    __builtin_amdgcn_sched_barrier(0);
    stash(nxt, b ^ 1);
#pragma unroll
    for (int bi = 0; bi < WBM; ++bi)
#pragma unroll
      for (int bj = 0; bj < WBN; ++bj)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[bi][bj][v] = __builtin_fmaf(sv[bj], cg[bi][bj][v], acc[bi][bj][v]);
#pragma unroll
    for (int bj = 0; bj < WBN; ++bj) sv[bj] = scale_of(nxt, bj);
    __syncthreads();
  }

  // epilogue: C[i][j] of a 32x32 block sits in lane j + 32*((i/4)%2), register
  // (i%4) + 4*(i/8)
#pragma unroll
  for (int bi = 0; bi < WBM; ++bi)
#pragma unroll
    for (int bj = 0; bj < WBN; ++bj) {
      if (!nvalid[bj]) continue;
      const int64_t nn = ncol[bj];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = 8 * (v >> 2) + 4 * kh + (v & 3);
        const int64_t mm = m0 + wm * (BM / 2) + bi * 32 + i;
        if (mm >= m) continue;
        if constexpr (OUT_F32)
          static_cast<float*>(y)[mm * n + nn] = acc[bi][bj][v];
        else
          static_cast<uint16_t*>(y)[mm * n + nn] = f32_to_bf16_rne(acc[bi][bj][v]);
      }
    }
}

int cu_count_gemm() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cached[dev] = v;
  }
  return cached[dev];
}

template <int FMT, int BM, int BN>
hipError_t launch_tile(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                       const uint16_t* x, int64_t m, void* y, bool out_f32, hipStream_t st) {
  const dim3 grid((unsigned)((n + BN - 1) / BN), (unsigned)((m + BM - 1) / BM));
  if (out_f32)
    hipLaunchKernelGGL((gemm_kernel<FMT, true, BM, BN>), grid, dim3(kThreads), 0, st, codes,
                       scales, x, m, n, k, y);
  else
    hipLaunchKernelGGL((gemm_kernel<FMT, false, BM, BN>), grid, dim3(kThreads), 0, st, codes,
                       scales, x, m, n, k, y);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                      const uint16_t* x, int64_t m, void* y, bool out_f32, hipStream_t st) {
  // 128 x 128 tiles when there are enough of them for two per CU, otherwise
  // 64 x 64 tiles (4x as many work-groups)
  const int64_t big = ((n + 127) / 128) * ((m + 127) / 128);
  if (big >= 2 * (int64_t)cu_count_gemm())
    return launch_tile<FMT, 128, 128>(codes, scales, n, k, x, m, y, out_f32, st);
  return launch_tile<FMT, 64, 64>(codes, scales, n, k, x, m, y, out_f32, st);
}

}  // namespace

hipError_t launch_gemm(int fmt, const uint8_t* codes, const uint16_t* scales, int64_t n,
                       int64_t k, const uint16_t* x, int64_t m, void* y, bool out_f32,
                       hipStream_t st) {
  if (fmt == 1) return launch_fmt<1>(codes, scales, n, k, x, m, y, out_f32, st);
  return launch_fmt<2>(codes, scales, n, k, x, m, y, out_f32, st);
}

}  // namespace lowbit
