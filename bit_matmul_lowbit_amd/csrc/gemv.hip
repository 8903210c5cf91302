// Decode GEMV  y[i][n] = sum_g s[n][g] * sum_{k in g} t[n][k] * x[i][k]
// for Q1_0_g128 and ternary g128 codes, batch 1..8.
//
// [P2] 7minutos.es, "PrismML lanza Bonsai 27B ...": decode is bound by memory
//      bandwidth ("Rendimiento y decodificacion especulativa DSpark"), and
//      every large matrix is stored low-bit ("Como funciona la compresion").
// [P1] 7minutos.es tutorial, section 7: bit 0 -> -s, bit 1 -> +s.
//
// Method: lookup tables of signed subset sums (the T-MAC idea of Wei et al.,
// 2024, redone for CDNA4's LDS).  For one 8-weight chunk of x,
//     S[e] = sum_{j<8} (bit j of e ? +x_j : -x_j),  e = 0..255.
// A Q1 code byte e of row n then contributes s * S[e].  A ternary chunk with
// pos byte p and neg byte q contributes s * (M[p] - M[q]) with M the masked
// subset sums, and M[p] - M[q] = (S[p] - S[q]) / 2, so one table serves both
// codes (the 1/2 is applied once per output).
//
// Data flow per call:
//   1. build kernel: every table S for every (column, chunk) into the
//      workspace, laid out exactly as the LDS image the main kernel wants;
//      it also zeroes y.
//   2. main kernel: a work-group owns one K-slice (the chunks held by its 64
//      lanes) and a range of 16-row tiles.  It copies the slice's 64 KB table
//      image into LDS once, then each wave streams 16-row code cells: lane l
//      loads the 16 B (Q1) / 32 B (T2) cell of its chunk, so a wave reads
//      1-2 KB contiguous per tile.  Each code byte becomes one LDS lookup
//      whose address is (byte << 8) | (lane << 2), built by one v_perm_b32:
//      table entry e of lane l sits at e*256 + 4*l, so every lane reads its
//      own bank -- conflict free.  Per-lane partial sums of the 16 rows are
//      then reduced across the lanes of the slice by a transposed butterfly
//      (permlane32/16 swaps, DPP row rotates / mirrors / quad perms) and
//      added to y with one atomic per row and K-slice.
//
// With batch b > 1 the 64 lanes are split into BP = 2, 4, 8 column groups of
// CH = 64 / BP chunks (BP = b rounded up to a power of two); the code cells
// are then re-read by each column group from cache, and the VALU work grows
// with BP.  No matrix cores: this is a streaming, not a dense, contraction.
#include "common.h"

namespace lowbit {
namespace {

constexpr int kWG = 256;               // 4 waves
constexpr int kLanes = 64;
constexpr int kEntries = 256;
constexpr int kSliceFloats = kEntries * kLanes;  // 64 KB of fp32

__device__ __forceinline__ float h2f(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return u2f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f2u(v), CTRL, 0xF, 0xF, true));
}

// DPP controls (within 16-lane rows / 4-lane quads)
constexpr int kRowRor8 = 0x128;      // lane i <- lane (i + 8) mod 16  (= i ^ 8)
constexpr int kRowHalfMirror = 0x141;  // lane i <- lane 7 - i within 8
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]

// ---------------------------------------------------------------------------
// build: tables of signed subset sums, one thread per (slice, hi nibble, lane)

__global__ __launch_bounds__(kWG) void gemv_build_kernel(const uint16_t* __restrict__ x, int64_t k,
                                                         int b, int ch, int64_t nslices,
                                                         float* __restrict__ lut,
                                                         float* __restrict__ y, int64_t ycount) {
  const int64_t gid = (int64_t)blockIdx.x * kWG + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kWG;
  for (int64_t i = gid; i < ycount; i += stride) y[i] = 0.0f;
  if (gid >= nslices * 16 * kLanes) return;
  const int lane = (int)(gid & 63);
  const int hi = (int)((gid >> 6) & 15);
  const int64_t s = gid >> 10;
  const int col = lane / ch;
  const int64_t chunk = s * ch + lane % ch;
  float* dst = lut + (s * kEntries + hi * 16) * kLanes + lane;
  if (col >= b || chunk >= k / kChunk) {
#pragma unroll
    for (int lo = 0; lo < 16; ++lo) dst[lo * kLanes] = 0.0f;
    return;
  }
  const uint4 v = *reinterpret_cast<const uint4*>(x + (int64_t)col * k + chunk * kChunk);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float xv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) xv[j] = h2f((w[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu);
  float h = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) h += ((hi >> j) & 1) ? xv[4 + j] : -xv[4 + j];
#pragma unroll
  for (int lo = 0; lo < 16; ++lo) {
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) a += ((lo >> j) & 1) ? xv[j] : -xv[j];
    dst[lo * kLanes] = a + h;
  }
}

// ---------------------------------------------------------------------------
// cross-lane reduction of 16 per-lane row partials over the CH chunk lanes
// (lane bits 0 .. log2(CH)-1).  After it, slot j of a lane holds the full
// sum of row (row_off + j); `writer` marks one lane per (column, row).

template <int STAGE_BIT>
__device__ __forceinline__ float partner(float v) {
  if constexpr (STAGE_BIT == 3) return dpp<kRowRor8>(v);
  else if constexpr (STAGE_BIT == 2) return dpp<kRowHalfMirror>(v);
  else if constexpr (STAGE_BIT == 1) return dpp<kQuadXor2>(v);
  else return dpp<kQuadXor1>(v);
}

// transposed stage on lane bit P: m values -> m/2 values
template <int P, int M>
__device__ __forceinline__ void tstage(float (&v)[16], int lane, int& row_off) {
  const bool hi = (lane >> P) & 1;
  if constexpr (P == 5) {
#pragma unroll
    for (int i = 0; i < M / 2; ++i) {
      auto r = __builtin_amdgcn_permlane32_swap(f2u(v[i]), f2u(v[i + M / 2]), false, false);
      v[i] = u2f(r[0]) + u2f(r[1]);
    }
  } else if constexpr (P == 4) {
#pragma unroll
    for (int i = 0; i < M / 2; ++i) {
      auto r = __builtin_amdgcn_permlane16_swap(f2u(v[i]), f2u(v[i + M / 2]), false, false);
      v[i] = u2f(r[0]) + u2f(r[1]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < M / 2; ++i) {
      const float a = v[i], b2 = v[i + M / 2];
      const float keep = hi ? b2 : a;
      const float send = hi ? a : b2;
      v[i] = keep + partner<P>(send);
    }
  }
  row_off += hi ? M / 2 : 0;
}

template <int P>
__device__ __forceinline__ void bstage(float (&v)[16]) {
  v[0] = v[0] + partner<P>(v[0]);
}

// returns number of valid slots; row of slot j is row_off + j
template <int CH>
__device__ __forceinline__ int reduce_rows(float (&v)[16], int lane, int& row_off, bool& writer) {
  row_off = 0;
  if constexpr (CH == 64) {
    tstage<5, 16>(v, lane, row_off);
    tstage<4, 8>(v, lane, row_off);
    tstage<3, 4>(v, lane, row_off);
    tstage<2, 2>(v, lane, row_off);
    bstage<1>(v);
    bstage<0>(v);
    writer = (lane & 3) == 0;
    return 1;
  } else if constexpr (CH == 32) {
    tstage<4, 16>(v, lane, row_off);
    tstage<3, 8>(v, lane, row_off);
    tstage<2, 4>(v, lane, row_off);
    tstage<1, 2>(v, lane, row_off);
    bstage<0>(v);
    writer = (lane & 1) == 0;
    return 1;
  } else if constexpr (CH == 16) {
    tstage<3, 16>(v, lane, row_off);
    tstage<2, 8>(v, lane, row_off);
    tstage<1, 4>(v, lane, row_off);
    tstage<0, 2>(v, lane, row_off);
    writer = true;
    return 1;
  } else {
    static_assert(CH == 8, "CH must be 64, 32, 16 or 8");
    tstage<2, 16>(v, lane, row_off);
    tstage<1, 8>(v, lane, row_off);
    tstage<0, 4>(v, lane, row_off);
    writer = true;
    return 2;
  }
}

// LDS byte address of table entry e (byte j of `word`) for this lane:
// (e << 8) | lane_base, with lane_base = 4 * lane < 256.
template <int J>
__device__ __forceinline__ uint32_t entry_addr(uint32_t word, uint32_t lane_base) {
  // v_perm_b32: result bytes [lane_base.b0, word.bJ, 0, 0]
  return __builtin_amdgcn_perm(word, lane_base, 0x0C0C0000u | ((4u + J) << 8));
}

// ---------------------------------------------------------------------------
// main kernel

template <int FMT, int CH>
__global__ __launch_bounds__(kWG, 2) void gemv_main_kernel(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const float* __restrict__ lut, float* __restrict__ y, int64_t n, int64_t k, int b,
    int64_t ntiles, int rb_tiles) {
  __shared__ float4 table[kSliceFloats / 4];
  const int64_t s = blockIdx.y;
  {
    const float4* src = reinterpret_cast<const float4*>(lut + s * kSliceFloats);
#pragma unroll 4
    for (int i = threadIdx.x; i < kSliceFloats / 4; i += kWG) table[i] = src[i];
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane / CH;
  const int64_t chunks = k / kChunk;
  const int64_t groups = k / kGroup;
  const int64_t c = s * CH + lane % CH;
  const bool active = (col < b) && (c < chunks);
  const int64_t g = c / kChunksPerGroup;
  const uint32_t lane_base = (uint32_t)lane * 4u;
  const char* tbase = reinterpret_cast<const char*>(table);

  const int64_t t0 = (int64_t)blockIdx.x * rb_tiles;
  const int64_t t1 = min(t0 + rb_tiles, ntiles);
  for (int64_t t = t0 + wave; t < t1; t += 4) {
    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    if (active) {
      const uint8_t* cell = codes + (t * chunks + c) * Fmt<FMT>::cell_bytes;
      const uint4 pa = *reinterpret_cast<const uint4*>(cell);
      uint4 na = make_uint4(0u, 0u, 0u, 0u);
      if constexpr (FMT == 2) na = *reinterpret_cast<const uint4*>(cell + 16);
      const uint4* sp = reinterpret_cast<const uint4*>(scales + (t * groups + g) * kTileRows);
      const uint4 s0 = sp[0], s1 = sp[1];
      const uint32_t pw[4] = {pa.x, pa.y, pa.z, pa.w};
      const uint32_t nw[4] = {na.x, na.y, na.z, na.w};
      const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#define LOWBIT_ROW(J)                                                                     \
  {                                                                                       \
    const int r = q * 4 + J;                                                              \
    const float sc = h2f((sw[r >> 1] >> ((r & 1) * 16)) & 0xFFFFu);                       \
    float val = *reinterpret_cast<const float*>(tbase + entry_addr<J>(pw[q], lane_base)); \
    if constexpr (FMT == 2)                                                               \
      val -= *reinterpret_cast<const float*>(tbase + entry_addr<J>(nw[q], lane_base));    \
    acc[r] = __builtin_fmaf(sc, val, acc[r]);                                             \
  }
        LOWBIT_ROW(0)
        LOWBIT_ROW(1)
        LOWBIT_ROW(2)
        LOWBIT_ROW(3)
#undef LOWBIT_ROW
      }
    }
    int row_off;
    bool writer;
    const int nv = reduce_rows<CH>(acc, lane, row_off, writer);
    if (writer && col < b) {
      const float half = (FMT == 2) ? 0.5f : 1.0f;
      for (int j = 0; j < nv; ++j) {
        const int64_t row = t * kTileRows + row_off + j;
        if (row < n) atomicAdd(y + (int64_t)col * n + row, acc[j] * half);
      }
    }
  }
}

int bp_for(int64_t b) { return b <= 1 ? 1 : b <= 2 ? 2 : b <= 4 ? 4 : 8; }

int64_t nslices_for(int64_t k, int ch) {
  const int64_t chunks = k / kChunk;
  return (chunks + ch - 1) / ch;
}

template <int FMT>
hipError_t launch_main(int ch, dim3 grid, hipStream_t st, const uint8_t* codes,
                       const uint16_t* scales, const float* lut, float* y, int64_t n, int64_t k,
                       int b, int64_t ntiles, int rb) {
  switch (ch) {
    case 64:
      hipLaunchKernelGGL((gemv_main_kernel<FMT, 64>), grid, dim3(kWG), 0, st, codes, scales, lut,
                         y, n, k, b, ntiles, rb);
      break;
    case 32:
      hipLaunchKernelGGL((gemv_main_kernel<FMT, 32>), grid, dim3(kWG), 0, st, codes, scales, lut,
                         y, n, k, b, ntiles, rb);
      break;
    case 16:
      hipLaunchKernelGGL((gemv_main_kernel<FMT, 16>), grid, dim3(kWG), 0, st, codes, scales, lut,
                         y, n, k, b, ntiles, rb);
      break;
    default:
      hipLaunchKernelGGL((gemv_main_kernel<FMT, 8>), grid, dim3(kWG), 0, st, codes, scales, lut,
                         y, n, k, b, ntiles, rb);
      break;
  }
  return hipGetLastError();
}

}  // namespace

size_t gemv_workspace_bytes(int64_t k, int64_t b) {
  const int ch = kLanes / bp_for(b);
  return (size_t)nslices_for(k, ch) * kSliceFloats * sizeof(float);
}

hipError_t launch_gemv_prepare(int64_t n, int64_t k, const uint16_t* x, int64_t b, float* y,
                               void* ws, hipStream_t st) {
  const int ch = kLanes / bp_for(b);
  const int64_t nslices = nslices_for(k, ch);
  const int64_t build_threads = nslices * 16 * kLanes;
  const int64_t build_blocks = (build_threads + kWG - 1) / kWG;
  hipLaunchKernelGGL(gemv_build_kernel, dim3((unsigned)build_blocks), dim3(kWG), 0, st, x, k,
                     (int)b, ch, nslices, static_cast<float*>(ws), y, n * b);
  return hipGetLastError();
}

hipError_t launch_gemv_accumulate(int fmt, const uint8_t* codes, const uint16_t* scales,
                                  int64_t n, int64_t k, int64_t b, float* y, const void* ws,
                                  hipStream_t st) {
  const int ch = kLanes / bp_for(b);
  const int64_t nslices = nslices_for(k, ch);
  const int64_t ntiles = (n + kTileRows - 1) / kTileRows;
  const float* lut = static_cast<const float*>(ws);
  // row blocks: enough work-groups to cover the GPU several times over, at
  // least two tiles per wave so the table copy is amortised
  const int64_t target_wgs = 4096;
  int64_t nrb = (target_wgs + nslices - 1) / nslices;
  int64_t rb = (ntiles + nrb - 1) / nrb;
  if (rb < 8) rb = 8;
  nrb = (ntiles + rb - 1) / rb;
  dim3 grid((unsigned)nrb, (unsigned)nslices);
  if (fmt == 1)
    return launch_main<1>(ch, grid, st, codes, scales, lut, y, n, k, (int)b, ntiles, (int)rb);
  return launch_main<2>(ch, grid, st, codes, scales, lut, y, n, k, (int)b, ntiles, (int)rb);
}

}  // namespace lowbit
