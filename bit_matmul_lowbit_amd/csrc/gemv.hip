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

#include <algorithm>

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

// LDS byte address of table entry e (byte J of `word`) for this lane and
// table q: bytes [lane_base.b0, word.bJ, lane_base.b2, 0], i.e.
// (e << 8) | (lane << 2) | (q << 16), with lane_base = 4*lane | q << 16.
template <int J>
__device__ __forceinline__ uint32_t entry_addr(uint32_t word, uint32_t lane_base) {
  return __builtin_amdgcn_perm(word, lane_base, 0x0C020000u | ((4u + J) << 8));
}

// ---------------------------------------------------------------------------
// main kernel

constexpr int kMainWaves = 12;                  // one 768-thread work-group per CU
constexpr int kMainThreads = kMainWaves * 64;
constexpr int kCpl = 2;                         // chunks (tables) per lane per slice

// tiles of code loads in flight per wave
template <int FMT> constexpr int kDepth = FMT == 1 ? 3 : 2;

template <int FMT>
struct TileRegs {
  uint4 pa[kCpl], na[kCpl];  // code cells: Q1 16 B (pa) / T2 pos (pa) + neg (na)
  uint4 s0[kCpl], s1[kCpl];  // 16 FP16 scales of the tile's rows for each chunk's group
};

// Tile loads go through buffer resources whose base is the tile's row of
// codes (or scales): the per-tile address arithmetic is scalar, the per-lane
// offsets are fixed VGPRs, and a resource with zero length (used for tiles
// past the end) returns zeros without touching memory.
constexpr int kRawBufferFlags = 0x00020000;  // gfx9 buffer descriptor word 3

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, (int)bytes,
                                           kRawBufferFlags);
}

__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int FMT>
__device__ __forceinline__ void load_tile(TileRegs<FMT>& r, __amdgpu_buffer_rsrc_t cr,
                                          __amdgpu_buffer_rsrc_t sr, const uint32_t (&coff)[kCpl],
                                          const uint32_t (&soff)[kCpl]) {
#pragma unroll
  for (int q = 0; q < kCpl; ++q) {
    r.pa[q] = bload(cr, coff[q]);
    if constexpr (FMT == 2) r.na[q] = bload(cr, coff[q] + 16);
    r.s0[q] = bload(sr, soff[q]);
    r.s1[q] = bload(sr, soff[q] + 16);
  }
}

// Lookups of one 16-row tile: acc[r] = sum over this lane's chunks of
// s[r] * S[code byte] (T2: s[r] * (S[pos] - S[neg])).  Branch-free: lanes
// without a chunk (a partial last K-slice, or columns beyond b) read their
// own all-zero table and, when MASKED, get zero scales, so they add exact
// zeros.
template <int FMT, bool MASKED>
__device__ __forceinline__ void tile_lookups(const TileRegs<FMT>& tr, const bool (&active)[kCpl],
                                             const char* tbase, const uint32_t (&lane_base)[kCpl],
                                             float (&acc)[16]) {
#pragma unroll
  for (int q = 0; q < kCpl; ++q) {
    const uint32_t pw[4] = {tr.pa[q].x, tr.pa[q].y, tr.pa[q].z, tr.pa[q].w};
    uint32_t nw[4] = {0u, 0u, 0u, 0u};
    if constexpr (FMT == 2) {
      nw[0] = tr.na[q].x; nw[1] = tr.na[q].y; nw[2] = tr.na[q].z; nw[3] = tr.na[q].w;
    }
    uint32_t sw[8] = {tr.s0[q].x, tr.s0[q].y, tr.s0[q].z, tr.s0[q].w,
                      tr.s1[q].x, tr.s1[q].y, tr.s1[q].z, tr.s1[q].w};
    if constexpr (MASKED) {
#pragma unroll
      for (int i = 0; i < 8; ++i) sw[i] = active[q] ? sw[i] : 0u;
    }
    const uint32_t lb = lane_base[q];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#define LOWBIT_ROW(J)                                                                   \
  {                                                                                     \
    const int r = w * 4 + J;                                                            \
    const float sc = h2f((sw[r >> 1] >> ((r & 1) * 16)) & 0xFFFFu);                     \
    float val = *reinterpret_cast<const float*>(tbase + entry_addr<J>(pw[w], lb));      \
    if constexpr (FMT == 2)                                                             \
      val -= *reinterpret_cast<const float*>(tbase + entry_addr<J>(nw[w], lb));         \
    acc[r] = (q == 0) ? sc * val : __builtin_fmaf(sc, val, acc[r]);                     \
  }
      LOWBIT_ROW(0)
      LOWBIT_ROW(1)
      LOWBIT_ROW(2)
      LOWBIT_ROW(3)
#undef LOWBIT_ROW
    }
  }
}

// Cross-lane reduction of a tile's 16 row partials and one atomic add per
// row (skipped for tiles past the end: `live` is wave-uniform).
template <int FMT, int CH>
__device__ __forceinline__ void tile_store(float (&acc)[16], bool live, int lane, int col, int b,
                                           int64_t t, int64_t n, float* __restrict__ y) {
  int row_off;
  bool writer;
  const int nv = reduce_rows<CH>(acc, lane, row_off, writer);
  const float half = (FMT == 2) ? 0.5f : 1.0f;
#pragma unroll
  for (int j = 0; j < nv; ++j) {
    const int64_t row = t * kTileRows + row_off + j;
    if (live && writer && col < b && row < n) atomicAdd(y + (int64_t)col * n + row, acc[j] * half);
  }
}

// Work decomposition.  A slice is kCpl consecutive sub-slices of CH chunks
// (a sub-slice is what one 64 KB table image covers); lane l holds chunk
// l % CH of each of them.  The grid is G x nslices work-groups: work-group j
// keeps slice s = j % nslices (one copy of its tables) and the row-tile
// blocks m, m + G, m + 2G, ... (m = j / nslices; 16 tiles per block, one per
// wave).  At any moment all work-groups are near the same block index, so
// the chip sweeps the code plane front to back in one contiguous front: HBM
// serves such a sweep measurably faster (about 6.3 TB/s on MI355X) than
// hundreds of independent streams (about 4.8 TB/s).
template <int FMT, int CH>
__global__ __launch_bounds__(kMainThreads, 3) void gemv_main_kernel(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const float* __restrict__ lut, float* __restrict__ y, int64_t n, int64_t k, int b,
    int64_t ntiles, int64_t nsub, int64_t nslices) {
  __shared__ float4 table[kCpl * kSliceFloats / 4];
  const int64_t s = blockIdx.x % nslices;
  const int64_t m = blockIdx.x / nslices;
  const int64_t G = gridDim.x / nslices;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int col = lane / CH;
  const int64_t chunks = k / kChunk;
  const int64_t groups = k / kGroup;
  const char* tbase = reinterpret_cast<const char*>(table);
  constexpr int S = kMainWaves;

  bool active[kCpl];
  uint32_t coff[kCpl], soff[kCpl], lane_base[kCpl];
  bool full = b * CH >= kLanes;  // wave-uniform: every lane holds a chunk of a real column
#pragma unroll
  for (int q = 0; q < kCpl; ++q) {
    const int64_t sub = s * kCpl + q;
    const int64_t c = sub * CH + lane % CH;
    active[q] = (col < b) && (c < chunks);
    full = full && (sub * CH + CH <= chunks);
    // every lane loads from a valid chunk; inactive lanes are masked later
    const int64_t cl = c < chunks ? c : chunks - 1;
    coff[q] = (uint32_t)(cl * Fmt<FMT>::cell_bytes);
    soff[q] = (uint32_t)((cl / kChunksPerGroup) * kTileRows * 2);
    lane_base[q] = (uint32_t)lane * 4u | ((uint32_t)q << 16);
  }
  const int stride = (int)(G * S);  // tiles between a wave's tiles
  const int tb = (int)ntiles;
  const int64_t cpitch = chunks * Fmt<FMT>::cell_bytes;  // bytes per 16-row tile
  const int64_t spitch = groups * kTileRows * 2;
  const uint8_t* cbase = codes;
  const uint8_t* sbase = reinterpret_cast<const uint8_t*>(scales);
  auto crs = [&](int t) { return t < tb ? tile_rsrc(cbase + t * cpitch, cpitch) : tile_rsrc(cbase, 0); };
  auto srs = [&](int t) { return t < tb ? tile_rsrc(sbase + t * spitch, spitch) : tile_rsrc(sbase, 0); };
  int t = (int)(m * S) + wave;

  // ring of D register sets: the loads of the next D-1 tiles of this wave
  // are in flight while one tile is contracted
  constexpr int D = kDepth<FMT>;
  TileRegs<FMT> buf[D];
#pragma unroll
  for (int i = 0; i < D - 1; ++i) load_tile<FMT>(buf[i], crs(t + i * stride), srs(t + i * stride), coff, soff);
  {
    // table images of this slice's sub-slices; a sub-slice past the end of K
    // gets an all-zero region, so its (inactive) lanes read finite zeros
#pragma unroll
    for (int q = 0; q < kCpl; ++q) {
      const int64_t sub = s * kCpl + q;
      if (sub < nsub) {
        const float4* src = reinterpret_cast<const float4*>(lut + sub * kSliceFloats);
#pragma unroll
        for (int i = threadIdx.x; i < kSliceFloats / 4; i += kMainThreads)
          table[q * (kSliceFloats / 4) + i] = src[i];
      } else {
        for (int i = threadIdx.x; i < kSliceFloats / 4; i += kMainThreads)
          table[q * (kSliceFloats / 4) + i] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  }
  __syncthreads();

  // software pipeline: the lookups of tile t + stride are issued next to the
  // reduction of tile t, two independent dependency chains
  float acc0[16], acc1[16];
  if (full) tile_lookups<FMT, false>(buf[0], active, tbase, lane_base, acc0);
  else tile_lookups<FMT, true>(buf[0], active, tbase, lane_base, acc0);
  constexpr int U = (D % 2 == 0) ? D : 2 * D;  // multiple of the ring and of 2
  while (t < tb) {
#pragma unroll
    for (int i = 0; i < U; ++i) {
      float (&cur)[16] = (i & 1) ? acc1 : acc0;
      float (&nxt)[16] = (i & 1) ? acc0 : acc1;
      const int tn = t + (D - 1) * stride;
      load_tile<FMT>(buf[(i + D - 1) % D], crs(tn), srs(tn), coff, soff);
      if (full) tile_lookups<FMT, false>(buf[(i + 1) % D], active, tbase, lane_base, nxt);
      else tile_lookups<FMT, true>(buf[(i + 1) % D], active, tbase, lane_base, nxt);
      tile_store<FMT, CH>(cur, t < tb, lane, col, b, t, n, y);
      t += stride;
    }
  }
}

int bp_for(int64_t b) { return b <= 1 ? 1 : b <= 2 ? 2 : b <= 4 ? 4 : 8; }

// table images (sub-slices of CH chunks) for this k and batch
int64_t nsub_for(int64_t k, int ch) {
  const int64_t chunks = k / kChunk;
  return (chunks + ch - 1) / ch;
}

// compute units of the current device (cached per device id)
int cu_count() {
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

template <int FMT>
hipError_t launch_main(int ch, dim3 grid, hipStream_t st, const uint8_t* codes,
                       const uint16_t* scales, const float* lut, float* y, int64_t n, int64_t k,
                       int b, int64_t ntiles, int64_t nsub, int64_t nslices) {
#define LOWBIT_LAUNCH(CHV)                                                                      \
  hipLaunchKernelGGL((gemv_main_kernel<FMT, CHV>), grid, dim3(kMainThreads), 0, st, codes,     \
                     scales, lut, y, n, k, b, ntiles, nsub, nslices)
  switch (ch) {
    case 64: LOWBIT_LAUNCH(64); break;
    case 32: LOWBIT_LAUNCH(32); break;
    case 16: LOWBIT_LAUNCH(16); break;
    default: LOWBIT_LAUNCH(8); break;
  }
#undef LOWBIT_LAUNCH
  return hipGetLastError();
}

}  // namespace

size_t gemv_workspace_bytes(int64_t k, int64_t b) {
  const int ch = kLanes / bp_for(b);
  return (size_t)nsub_for(k, ch) * kSliceFloats * sizeof(float);
}

hipError_t launch_gemv_prepare(int64_t n, int64_t k, const uint16_t* x, int64_t b, float* y,
                               void* ws, hipStream_t st) {
  const int ch = kLanes / bp_for(b);
  const int64_t nsub = nsub_for(k, ch);
  const int64_t build_threads = nsub * 16 * kLanes;
  const int64_t build_blocks = (build_threads + kWG - 1) / kWG;
  hipLaunchKernelGGL(gemv_build_kernel, dim3((unsigned)build_blocks), dim3(kWG), 0, st, x, k,
                     (int)b, ch, nsub, static_cast<float*>(ws), y, n * b);
  return hipGetLastError();
}

hipError_t launch_gemv_accumulate(int fmt, const uint8_t* codes, const uint16_t* scales,
                                  int64_t n, int64_t k, int64_t b, float* y, const void* ws,
                                  hipStream_t st) {
  const int ch = kLanes / bp_for(b);
  const int64_t nsub = nsub_for(k, ch);
  const int64_t nslices = (nsub + kCpl - 1) / kCpl;
  const int64_t ntiles = (n + kTileRows - 1) / kTileRows;
  const float* lut = static_cast<const float*>(ws);
  // G work-groups per slice: about one per CU in all, and no more than there
  // are 16-tile blocks
  int64_t G = (int64_t)cu_count() / nslices;
  if (G < 1) G = 1;
  const int64_t blocks = (ntiles + kMainWaves - 1) / kMainWaves;
  if (G > blocks) G = blocks;
  const int64_t nwg = G * nslices;
  dim3 grid((unsigned)nwg);
  if (fmt == 1)
    return launch_main<1>(ch, grid, st, codes, scales, lut, y, n, k, (int)b, ntiles, nsub, nslices);
  return launch_main<2>(ch, grid, st, codes, scales, lut, y, n, k, (int)b, ntiles, nsub, nslices);
}

}  // namespace lowbit
