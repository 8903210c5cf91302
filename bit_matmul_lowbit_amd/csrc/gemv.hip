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
// A Q1 code byte e of row n then contributes S[e]; a ternary chunk with pos
// byte p and neg byte q contributes M[p] - M[q] (M = masked subset sums), and
// M[p] - M[q] = (S[p] - S[q]) / 2, so one table serves both codes (the 1/2 is
// applied once per output).  The group scale multiplies the per-group sum.
//
// Data flow per call:
//   1. prepare kernel (lowbit_gemv_prepare): copies x into the workspace and
//      zeroes y.
//   2. main kernel (lowbit_gemv_accumulate): a work-group holds one K-slice:
//      each lane owns two adjacent chunks of one group (two 64 KB tables,
//      128 KB of LDS), and eight neighbouring lanes cover one group.  The
//      work-group computes its slice's tables straight into LDS from x.  Per
//      16-row tile a lane loads its 32 B (Q1) / 64 B (T2) of codes and one
//      dword of scales; each code byte becomes one LDS lookup at
//      (byte << 8) | (lane << 2) | (table << 16) -- a single v_perm_b32; every
//      lane reads its own bank, conflict-free.  The 16 row partials are then
//      reduced over the lanes of the same group (permlane swaps / DPP, three
//      transposed stages leave two rows per lane), multiplied by those two
//      rows' scales, reduced over the groups, and added to y with one FP32
//      atomic per row and K-slice.
//
// Two more entries serve the decode FFN (b <= 2) as two launches with
// nothing to zero beforehand: launch_gemv_partials (gate+up) reads x in
// place and stores each K-slice's row sums into a plane of its own (plain
// stores, no atomics), zeroing the FFN output as it goes;
// launch_gemv_accumulate_silu (down) adds those planes up and forms its
// activations z = RNE_fp16(SiLU(gate) * up) while the tables are built, so
// neither the sum h nor z is ever written out.
//
// With batch b > 1 the 64 lanes are split into BP = 2, 4, 8 column groups of
// CH = 64 / BP lanes (BP = b rounded up to a power of two); the code cells
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
// Lane -> chunk map of the main kernel.  Within a column group of CH lanes,
// lane l' = 8 j + i (i = l' % 8, j = l' / 8 < GW = CH / 8) owns chunks
// s * 2CH + 16 j + 2 i + q (q = 0, 1) of slice s: two adjacent chunks of
// group s * GW + j.  Eight neighbouring lanes thus cover one 128-weight group
// and read 256 (Q1) / 512 (T2) contiguous bytes of a tile.

__device__ __forceinline__ int64_t lane_chunk(int64_t s, int lanec, int ch, int q) {
  return s * 2 * ch + 16 * (lanec >> 3) + 2 * (lanec & 7) + q;
}

// prepare: x [b][k] -> workspace (read by the main kernel's table build), y = 0
__global__ __launch_bounds__(kWG) void gemv_prepare_kernel(const uint4* __restrict__ x,
                                                           int64_t nvec, uint4* __restrict__ xs,
                                                           float* __restrict__ y,
                                                           int64_t ycount) {
  const int64_t gid = (int64_t)blockIdx.x * kWG + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kWG;
  zero_f32(y, ycount, gid, stride);
  for (int64_t i = gid; i < nvec; i += stride) xs[i] = x[i];
}

// ---------------------------------------------------------------------------
// Cross-lane reduction of 16 per-lane row partials.

template <int STAGE_BIT>
__device__ __forceinline__ float partner(float v) {
  if constexpr (STAGE_BIT == 3) return dpp<kRowRor8>(v);
  else if constexpr (STAGE_BIT == 2) return dpp<kRowHalfMirror>(v);
  else if constexpr (STAGE_BIT == 1) return dpp<kQuadXor2>(v);
  else return dpp<kQuadXor1>(v);
}

// Transposed stage on lane bit P: M values -> M/2 values.  The lane with bit
// P clear keeps the low half of the rows, its partner the high half.  The
// bit-2 partner (half mirror) also flips bits 1 and 0; that is harmless as
// long as stages on bits 1 and 0 follow and the lanes involved hold partials
// that may be summed unscaled (same 128-weight group).
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

// Butterfly on lane bit P (3, 4 or 5): v[0] summed with the partner lane's.
template <int P>
__device__ __forceinline__ void bstage(float (&v)[16]) {
  if constexpr (P == 5) {
    auto r = __builtin_amdgcn_permlane32_swap(f2u(v[0]), f2u(v[0]), false, false);
    v[0] = u2f(r[0]) + u2f(r[1]);
  } else if constexpr (P == 4) {
    auto r = __builtin_amdgcn_permlane16_swap(f2u(v[0]), f2u(v[0]), false, false);
    v[0] = u2f(r[0]) + u2f(r[1]);
  } else {
    v[0] = v[0] + partner<P>(v[0]);
  }
}

// Part 1, within a group (lane bits 2..0 = i): three transposed stages leave
// rows row_off and row_off + 1 in v[0], v[1], with row_off = 2 (lane % 8).
__device__ __forceinline__ void reduce_in_group(float (&v)[16], int lane, int& row_off) {
  row_off = 0;
  tstage<2, 16>(v, lane, row_off);
  tstage<1, 8>(v, lane, row_off);
  tstage<0, 4>(v, lane, row_off);
}

// Part 2, across the GW groups of the slice (lane bits log2(CH)-1 .. 3 = j),
// after each lane has scaled its two rows.  Returns the number of valid
// slots; slot t holds row row_off + t; `writer` marks one lane per
// (column, row).
template <int CH>
__device__ __forceinline__ int reduce_groups(float (&v)[16], int lane, int& row_off, bool& writer) {
  if constexpr (CH == 64) {
    tstage<5, 2>(v, lane, row_off);
    bstage<4>(v);
    bstage<3>(v);
    writer = (lane & 0x18) == 0;
    return 1;
  } else if constexpr (CH == 32) {
    tstage<4, 2>(v, lane, row_off);
    bstage<3>(v);
    writer = (lane & 0x08) == 0;
    return 1;
  } else if constexpr (CH == 16) {
    tstage<3, 2>(v, lane, row_off);
    writer = true;
    return 1;
  } else {
    static_assert(CH == 8, "CH must be 64, 32, 16 or 8");
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

constexpr int kMainWaves = 16;                  // one 1024-thread work-group per CU
constexpr int kMainThreads = kMainWaves * 64;
constexpr int kImages = 2;                      // tables per lane (chunks q = 0, 1)

// 16-byte code cells per lane per tile, and tiles of loads in flight per wave
template <int FMT> constexpr int kCells = FMT == 1 ? 2 : 4;
template <int FMT, int CH> constexpr int kDepth = FMT == 1 ? 4 : 3;

template <int FMT>
struct TileRegs {
  uint4 c[kCells<FMT>];  // Q1: chunk 0, chunk 1; T2: pos 0, neg 0, pos 1, neg 1
  uint32_t sc;           // FP16 scales of this lane's two rows for its group
};

// Tile loads go through buffer resources whose base is the tile's row of
// codes (or scales): the per-tile address arithmetic is scalar, the per-lane
// offsets are fixed VGPRs, and a resource with zero length (used for tiles
// past the end) returns zeros without touching memory (buffer_rsrc).
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

// `off` is the per-lane (VGPR) offset, SOFF a constant added by the
// instruction itself (no extra VGPR per cell)
template <int SOFF = 0>
__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, SOFF, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int FMT>
__device__ __forceinline__ void load_tile(TileRegs<FMT>& r, __amdgpu_buffer_rsrc_t cr,
                                          __amdgpu_buffer_rsrc_t sr, uint32_t coff, uint32_t soff) {
  r.c[0] = bload<0>(cr, coff);
  r.c[1] = bload<16>(cr, coff);
  if constexpr (kCells<FMT> == 4) {
    r.c[2] = bload<32>(cr, coff);
    r.c[3] = bload<48>(cr, coff);
  }
  r.sc = __builtin_amdgcn_raw_buffer_load_b32(sr, soff, 0, 0);
}

// Lookups of one 16-row tile: acc[r] = sum over this lane's two chunks of
// S[code byte of row r] (T2: S[pos] - S[neg]).  Unscaled: both chunks belong
// to the same group.  Lanes without a chunk (past the end of K, or a column
// beyond b) read their own all-zero tables.
template <int FMT>
__device__ __forceinline__ void tile_lookups(const TileRegs<FMT>& tr, const char* tbase,
                                             uint32_t lane_base, float (&acc)[16]) {
#pragma unroll
  for (int q = 0; q < kImages; ++q) {
    const uint4 pc = tr.c[FMT == 1 ? q : 2 * q];
    const uint32_t pw[4] = {pc.x, pc.y, pc.z, pc.w};
    uint32_t nw[4] = {0u, 0u, 0u, 0u};
    if constexpr (FMT == 2) {
      const uint4 nc = tr.c[2 * q + 1];
      nw[0] = nc.x; nw[1] = nc.y; nw[2] = nc.z; nw[3] = nc.w;
    }
    const uint32_t lb = lane_base | ((uint32_t)q << 16);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#define LOWBIT_ROW(J)                                                                   \
  {                                                                                     \
    const int r = w * 4 + J;                                                            \
    float val = *reinterpret_cast<const float*>(tbase + entry_addr<J>(pw[w], lb));      \
    if constexpr (FMT == 2)                                                             \
      val -= *reinterpret_cast<const float*>(tbase + entry_addr<J>(nw[w], lb));         \
    acc[r] = (q == 0) ? val : acc[r] + val;                                             \
  }
      LOWBIT_ROW(0)
      LOWBIT_ROW(1)
      LOWBIT_ROW(2)
      LOWBIT_ROW(3)
#undef LOWBIT_ROW
    }
  }
}

// Reduction of a tile's 16 row partials: within the group, scale the two
// rows each lane is left with (scale word `sw`, zero for inactive lanes),
// across the groups, then one atomic add per row -- or, with PART, a plain
// store of the slice's partial sum into y + ybase (a [b][n] plane of its
// own per K-slice).  T2 halves its sums here.
template <int FMT, int CH, bool PART = false>
__device__ __forceinline__ void tile_store(float (&acc)[16], uint32_t sw, int lane,
                                           int col, int b, int64_t t, int64_t n,
                                           float* __restrict__ y, int64_t ybase = 0) {
  int row_off;
  bool writer;
  reduce_in_group(acc, lane, row_off);
  const float half = (FMT == 2) ? 0.5f : 1.0f;
  acc[0] *= h2f(sw & 0xFFFFu) * half;
  acc[1] *= h2f(sw >> 16) * half;
  const int nv = reduce_groups<CH>(acc, lane, row_off, writer);
#pragma unroll
  for (int j = 0; j < nv; ++j) {
    const int64_t row = t * kTileRows + row_off + j;
    if (writer && col < b && row < n) {
      if constexpr (PART)
        y[ybase + (int64_t)col * n + row] = acc[j];
      else
        atomicAdd(y + (int64_t)col * n + row, acc[j]);
    }
  }
}

// Work decomposition.  A slice is 2 CH consecutive chunks (GW = CH / 8
// groups); the grid is G x nslices work-groups: work-group w keeps slice
// s = w % nslices (one copy of its two table images in LDS) and the
// row-tile blocks m, m + G, m + 2G, ... (m = w / nslices; 16 tiles per
// block, one per wave).  At any moment all work-groups are near the same
// block index, so the chip sweeps the code plane front to back in one
// contiguous front: HBM serves such a sweep measurably faster (about
// 6.3 TB/s on MI355X) than hundreds of independent streams (about 4.8 TB/s).
// The decode FFN's two table GEMVs (b <= 2) use two variants:
// PART (gate+up): slice s stores its partial sums into plane s of y
//   (FP32 [nslices][b][n]) with plain stores, so that nothing has to be
//   zeroed first, and the work-groups zero yz[0 .. yzn) (the FFN output, to
//   which the down GEMV adds) on the way;
// ZH (down): the activations are z = RNE_fp16(SiLU(gate) * up), formed in
//   the table build (the same arithmetic as silu_mul_kernel) from h = the
//   sum of the np planes of partial sums at `h` (FP32 [np][b][2k]: k gate
//   columns, then k up columns), added in a fixed order (plane order for
//   np <= 8).
template <int FMT, int CH, bool ZH = false, bool PART = false>
__global__ __launch_bounds__(kMainThreads, kMainWaves / 4) void gemv_main_kernel(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ xs, float* __restrict__ y, int64_t n, int64_t k, int b,
    int64_t ntiles, int64_t nslices, const float* __restrict__ h, int np,
    float* __restrict__ yz, int64_t yzn) {
  __shared__ float4 table[kImages * kSliceFloats / 4];
  const int64_t s = blockIdx.x % nslices;
  const int64_t m = blockIdx.x / nslices;
  const int64_t G = gridDim.x / nslices;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int col = lane / CH;
  const int i8 = lane & 7;
  const int64_t groups = k / kGroup;
  const char* tbase = reinterpret_cast<const char*>(table);
  constexpr int S = kMainWaves;
  constexpr int GW = CH / 8;

  // this lane's group; every lane loads from a valid group, inactive lanes
  // read zero tables and get a zero scale word
  const int64_t g = s * GW + ((lane % CH) >> 3);
  const bool active = (col < b) && (g < groups);
  const int64_t gc = g < groups ? g : groups - 1;
  const uint32_t coff = (uint32_t)((gc * kChunksPerGroup + 2 * i8) * Fmt<FMT>::cell_bytes);
  const uint32_t soff = (uint32_t)((gc * kTileRows + 2 * i8) * 2);
  const uint32_t lane_base = (uint32_t)lane * 4u;

  const int stride = (int)(G * S);  // tiles between a wave's tiles
  const int tb = (int)ntiles;
  const int cpitch = (int)((k / kChunk) * Fmt<FMT>::cell_bytes);  // bytes per 16-row tile
  const int spitch = (int)(groups * kTileRows * 2);
  int t = (int)(m * S) + wave;
  // Running (scalar) bases of the next tile to load.  A tile past the end
  // gets a zero-length resource: its loads return zeros and touch nothing,
  // so its base may point past the arrays.
  int tn = t;
  const uint8_t* cn = codes + (int64_t)tn * cpitch;
  const uint8_t* sn = reinterpret_cast<const uint8_t*>(scales) + (int64_t)tn * spitch;
  const int64_t cstep = (int64_t)stride * cpitch, sstep = (int64_t)stride * spitch;
  auto load_next = [&](TileRegs<FMT>& r) {
    const bool in = tn < tb;
    load_tile<FMT>(r, buffer_rsrc(cn, in ? cpitch : 0), buffer_rsrc(sn, in ? spitch : 0), coff, soff);
    tn += stride;
    cn += cstep;
    sn += sstep;
  };

  // Table build, part 1: thread (image q, hi-nibble pair, lane L) loads the
  // 8 activations of its chunk (zeros for a lane without a chunk: a column
  // beyond b or a chunk past the end of K, so its entries are 0).  The wave
  // waits for it before any weight load goes out: behind a burst of weight
  // loads from every CU, this small load took microseconds to return and
  // held back the tables (and so every lookup).
  const int bl = threadIdx.x & 63;        // lane whose table column is built
  const int bq = (threadIdx.x >> 9) & 1;  // image
  const int bp = (threadIdx.x >> 6) & 7;  // hi nibbles 2 bp, 2 bp + 1
  if constexpr (PART)
    zero_f32(yz, yzn, (int64_t)blockIdx.x * kMainThreads + threadIdx.x,
             (int64_t)gridDim.x * kMainThreads);
  uint4 xv4;
  {
    const int bcol = bl / CH;
    const int64_t bchunk = lane_chunk(s, bl % CH, CH, bq);
    const bool bvalid = bcol < b && bchunk < k / kChunk;
    if constexpr (!ZH) {
      const __amdgpu_buffer_rsrc_t xr =
          buffer_rsrc(reinterpret_cast<const uint8_t*>(xs), (int64_t)b * k * 2);
      // an offset past the resource returns zeros
      const uint32_t xoff = bvalid ? (uint32_t)((bcol * k + bchunk * kChunk) * 2) : 0xFFFFFFF0u;
      xv4 = bload<0>(xr, xoff);
    } else {
      // The 8 waves of an image share its 64 chunks: wave bp adds planes
      // bp, bp + 8, ... of its lane's chunk (gate and up, 16 floats) and
      // stages the sums in LDS (image 0 of the table, not yet built:
      // float4 i of wave (bp, bq), lane L at (i * 16 + 2 bp + bq) * 64 + L,
      // conflict-free); wave 0 of each image adds the staged sums in wave
      // order, forms z and leaves it in zsh for the whole work-group.  The
      // build needs z: every wave waits for it here, before any weight load
      // goes out (as for x above).
      __shared__ uint4 zsh[kImages * kLanes];
      const int bw = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
      const int wp = bw & 7;  // = bp, known to be wave-uniform
      const int npw = np < 8 ? np : 8;
      const uint32_t go = bvalid ? (uint32_t)((bcol * 2 * k + bchunk * kChunk) * 4) : 0xFFFFFFE0u;
      const uint32_t uo = bvalid ? go + (uint32_t)(k * 4) : 0xFFFFFFE0u;
      const int64_t plane = (int64_t)b * 2 * k;  // floats per plane
      if (wp < npw) {
        float4 a[4] = {};
        for (int p = wp; p < np; p += 8) {
          const __amdgpu_buffer_rsrc_t hr =
              buffer_rsrc(reinterpret_cast<const uint8_t*>(h + p * plane), plane * 4);
          const uint4 v[4] = {bload<0>(hr, go), bload<16>(hr, go), bload<0>(hr, uo),
                              bload<16>(hr, uo)};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            a[i].x += u2f(v[i].x);
            a[i].y += u2f(v[i].y);
            a[i].z += u2f(v[i].z);
            a[i].w += u2f(v[i].w);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) table[(i * 16 + 2 * wp + bq) * 64 + bl] = a[i];
      }
      __syncthreads();
      if (wp == 0) {
        float4 a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = table[(i * 16 + bq) * 64 + bl];
        for (int w = 1; w < npw; ++w) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float4 v = table[(i * 16 + 2 * w + bq) * 64 + bl];
            a[i].x += v.x;
            a[i].y += v.y;
            a[i].z += v.z;
            a[i].w += v.w;
          }
        }
        const float gv[8] = {a[0].x, a[0].y, a[0].z, a[0].w, a[1].x, a[1].y, a[1].z, a[1].w};
        const float uv[8] = {a[2].x, a[2].y, a[2].z, a[2].w, a[3].x, a[3].y, a[3].z, a[3].w};
        zsh[bq * kLanes + bl] = silu_mul8(gv, uv);
      }
      __syncthreads();
      xv4 = zsh[bq * kLanes + bl];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // an empty statement that reads xv4: the compiler waits for the load here
  __asm__ volatile("" ::"v"(xv4.x), "v"(xv4.y), "v"(xv4.z), "v"(xv4.w));

  // ring of D register sets: the loads of the next D-1 tiles of this wave
  // are in flight while one tile is contracted.  The first goes out before
  // the table build, the others after it.
  constexpr int D = kDepth<FMT, CH>;
  TileRegs<FMT> buf[D];
  load_next(buf[0]);
  __builtin_amdgcn_sched_barrier(0);

  // Table build, part 2: S[e] = sum_j (bit j of e ? +x_j : -x_j) for the 32
  // entries e = 16 hi + lo of this thread (hi = 2 bp, 2 bp + 1); entry e of
  // lane L of image q sits at float q * 16384 + e * 64 + L, so a wave writes
  // 64 consecutive floats per entry.
  {
    const uint32_t w4[4] = {xv4.x, xv4.y, xv4.z, xv4.w};
    float xv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xv[j] = h2f((w4[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu);
    float lo_sum[16];
#pragma unroll
    for (int lo = 0; lo < 16; ++lo) {
      float a = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) a += ((lo >> j) & 1) ? xv[j] : -xv[j];
      lo_sum[lo] = a;
    }
    float* tabf = reinterpret_cast<float*>(table) + bq * kSliceFloats + bl;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int hi = 2 * bp + hh;
      float h = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) h += ((hi >> j) & 1) ? xv[4 + j] : -xv[4 + j];
#pragma unroll
      for (int lo = 0; lo < 16; ++lo) tabf[(hi * 16 + lo) * kLanes] = lo_sum[lo] + h;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 1; i < D - 1; ++i) load_next(buf[i]);

  // software pipeline: the lookups of the next tile are issued next to the
  // reduction of the current one, two independent dependency chains
  float acc0[16], acc1[16];
  tile_lookups<FMT>(buf[0], tbase, lane_base, acc0);
  uint32_t sw_cur = active ? buf[0].sc : 0u;
  constexpr int U = (D % 2 == 0) ? D : 2 * D;  // multiple of the ring and of 2
  // step i of a pass (i is a constant once the loops below are unrolled)
  auto step = [&](int i) __attribute__((always_inline)) {
    float (&cur)[16] = (i & 1) ? acc1 : acc0;
    float (&nxt)[16] = (i & 1) ? acc0 : acc1;
    load_next(buf[(i + D - 1) % D]);
    tile_lookups<FMT>(buf[(i + 1) % D], tbase, lane_base, nxt);
    const uint32_t sw_nxt = active ? buf[(i + 1) % D].sc : 0u;
    tile_store<FMT, CH, PART>(cur, sw_cur, lane, col, b, t, n, y, PART ? s * b * n : 0);
    sw_cur = sw_nxt;
    t += stride;
  };
  // whole passes while all U tiles of the pass exist, then the last tiles one
  // by one (a wave of a small matrix may have a single tile: the rest of a
  // pass would be spent on lookups and reductions of empty tiles)
  while (t + (U - 1) * stride < tb) {
#pragma unroll
    for (int i = 0; i < U; ++i) step(i);
  }
#pragma unroll
  for (int i = 0; i < U; ++i) {
    if (t >= tb) break;
    step(i);
  }
}

int bp_for(int64_t b) { return b <= 1 ? 1 : b <= 2 ? 2 : b <= 4 ? 4 : 8; }

// slices (2 CH chunks, two 64 KB table images each) for this k and batch
int64_t nslices_for(int64_t k, int ch) {
  const int64_t chunks = k / kChunk;
  return (chunks + 2 * ch - 1) / (2 * ch);
}

// grid of the main kernel: G work-groups per slice, about one per CU in
// all, and no more than there are 16-tile blocks
dim3 main_grid(int64_t ntiles, int64_t nslices) {
  int64_t G = (int64_t)device_cu_count() / nslices;
  if (G < 1) G = 1;
  const int64_t blocks = (ntiles + kMainWaves - 1) / kMainWaves;
  if (G > blocks) G = blocks;
  return dim3((unsigned)(G * nslices));
}

template <int FMT>
hipError_t launch_main(int ch, dim3 grid, hipStream_t st, const uint8_t* codes,
                       const uint16_t* scales, const uint16_t* xs, float* y, int64_t n, int64_t k,
                       int b, int64_t ntiles, int64_t nslices) {
#define LOWBIT_LAUNCH(CHV)                                                                      \
  hipLaunchKernelGGL((gemv_main_kernel<FMT, CHV>), grid, dim3(kMainThreads), 0, st, codes,     \
                     scales, xs, y, n, k, b, ntiles, nslices, nullptr, 0, nullptr, (int64_t)0)
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
  if (b >= kMfmaMinBatch) return (size_t)gemv_mfma_workspace_bytes(k);
  return (size_t)(b * k * 2);  // x, from which the main kernel builds its tables
}

hipError_t launch_gemv_prepare(int64_t n, int64_t k, const uint16_t* x, int64_t b, float* y,
                               void* ws, hipStream_t st) {
  if (b >= kMfmaMinBatch) return launch_gemv_mfma_prepare(n, k, x, b, y, ws, st);
  const int64_t nvec = b * k / 8;  // 16-byte vectors of x (k % 128 == 0)
  const int64_t yvec = (n * b + 3) / 4;  // y is zeroed 16 bytes at a time
  const int64_t work = nvec > yvec ? nvec : yvec;
  int64_t blocks = (work + kWG - 1) / kWG;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(gemv_prepare_kernel, dim3((unsigned)blocks), dim3(kWG), 0, st,
                     reinterpret_cast<const uint4*>(x), nvec, static_cast<uint4*>(ws), y, n * b);
  return hipGetLastError();
}

hipError_t launch_gemv_accumulate(int fmt, const uint8_t* codes, const uint16_t* scales,
                                  int64_t n, int64_t k, int64_t b, float* y, const void* ws,
                                  hipStream_t st) {
  if (b >= kMfmaMinBatch)
    return launch_gemv_mfma(fmt, codes, scales, n, k, b, y, ws, device_cu_count(), st);
  const int ch = kLanes / bp_for(b);
  const int64_t nslices = nslices_for(k, ch);
  const int64_t ntiles = (n + kTileRows - 1) / kTileRows;
  const uint16_t* xs = static_cast<const uint16_t*>(ws);
  const dim3 grid = main_grid(ntiles, nslices);
  if (fmt == 1)
    return launch_main<1>(ch, grid, st, codes, scales, xs, y, n, k, (int)b, ntiles, nslices);
  return launch_main<2>(ch, grid, st, codes, scales, xs, y, n, k, (int)b, ntiles, nslices);
}

int64_t gemv_partial_planes(int64_t k, int64_t b) { return nslices_for(k, kLanes / bp_for(b)); }

hipError_t launch_gemv_partials(int fmt, const uint8_t* codes, const uint16_t* scales, int64_t n,
                                int64_t k, int64_t b, const uint16_t* x, float* hp, float* yz,
                                int64_t yzn, hipStream_t st) {
  const int ch = kLanes / bp_for(b);  // 64 or 32: b <= 2
  const int64_t nslices = nslices_for(k, ch);
  const int64_t ntiles = (n + kTileRows - 1) / kTileRows;
  const dim3 grid = main_grid(ntiles, nslices);
#define LOWBIT_LAUNCH(F, CHV)                                                                   \
  hipLaunchKernelGGL((gemv_main_kernel<F, CHV, false, true>), grid, dim3(kMainThreads), 0, st,  \
                     codes, scales, x, hp, n, k, (int)b, ntiles, nslices, nullptr, 0, yz, yzn)
  if (fmt == 1) {
    if (ch == 64) LOWBIT_LAUNCH(1, 64);
    else LOWBIT_LAUNCH(1, 32);
  } else {
    if (ch == 64) LOWBIT_LAUNCH(2, 64);
    else LOWBIT_LAUNCH(2, 32);
  }
#undef LOWBIT_LAUNCH
  return hipGetLastError();
}

hipError_t launch_gemv_accumulate_silu(int fmt, const uint8_t* codes, const uint16_t* scales,
                                       int64_t n, int64_t k, int64_t b, float* y, const float* hp,
                                       int64_t np, hipStream_t st) {
  const int ch = kLanes / bp_for(b);  // 64 or 32: b <= 2
  const int64_t nslices = nslices_for(k, ch);
  const int64_t ntiles = (n + kTileRows - 1) / kTileRows;
  const dim3 grid = main_grid(ntiles, nslices);
#define LOWBIT_LAUNCH(F, CHV)                                                                   \
  hipLaunchKernelGGL((gemv_main_kernel<F, CHV, true>), grid, dim3(kMainThreads), 0, st, codes,  \
                     scales, nullptr, y, n, k, (int)b, ntiles, nslices, hp, (int)np, nullptr,   \
                     (int64_t)0)
  if (fmt == 1) {
    if (ch == 64) LOWBIT_LAUNCH(1, 64);
    else LOWBIT_LAUNCH(1, 32);
  } else {
    if (ch == 64) LOWBIT_LAUNCH(2, 64);
    else LOWBIT_LAUNCH(2, 32);
  }
#undef LOWBIT_LAUNCH
  return hipGetLastError();
}

}  // namespace lowbit
