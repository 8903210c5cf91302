// Prefill GEMM  Y[i][n] = sum_g s[n][g] * sum_{k in g} X[i][k] * t[n][k]
// with X in BF16 [m][k] and W in Q1_0_g128 or ternary g128 codes.
//
// [P2] 7minutos.es, "PrismML lanza Bonsai 27B ...", "Rendimiento y
//      decodificacion especulativa DSpark": prefill is compute-bound.
// [P1] 7minutos.es tutorial, section 7: bit 0 -> -s, bit 1 -> +s.
// [P2] "Como funciona la compresion": w = s * t, t in {-1, 0, +1}.
//
// Two kernels.  gemm_team_kernel (further below) takes shapes whose
// 128 x 96 tiles fill whole rounds of the CUs, such as the ternary pp512
// one; gemm_kernel takes the rest.
//
// gemm_kernel tiling: a team of WM x WN waves owns a BM x BN output tile (128 x 128 and
// 64 x 64 with 2 x 2 waves, 128 x 96 with 4 x 3); each wave's tile is made of
// 32x32 blocks of the 32x32x16 BF16 matrix-core instruction.  The K loop
// steps one scale group (128) at a time through LDS:
//   * X[BM][128] BF16, the codes of W[BN][128] and the scales are loaded
//     groups ahead and written to LDS while the matrix cores work (128 x 128
//     tiles: a four-stage register ring and two LDS buffers; 32 x 32 blocks
//     per wave: a two-stage ring, with one LDS buffer when three
//     work-groups share a CU and two when the work-group runs alone, where
//     the 128 x 96 kernel also loads X straight into LDS), the codes
//     expanded to exact BF16 {-1, 0, +1}.  The scale is NOT folded in: a
//     BF16 scale would lose 3 of FP16's 11 significant bits;
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
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = 128;
constexpr int kThreads = 256;
constexpr int kRowU4 = BK / 8;  // 16-byte slots per LDS row

// LDS uint4 index of 16-byte slot c of row r (XOR swizzle)
__device__ __forceinline__ int slot(int r, int c) { return r * kRowU4 + (c ^ (r & 15)); }

// Code byte -> 8 BF16 values, two per dword (k = 2p in the low half, 2p + 1
// in the high half).  Q1: the byte is placed in the low byte of both 16-bit
// halves (rep_byte); a packed 16-bit shift by (15 - 2p, 14 - 2p) brings bits
// 2p and 2p + 1 to bits 15 and 31, where v_bitop3 uses them as sign bits (+1
// and -1 differ only there): two VALU operations per dword.  Ternary: below.
constexpr uint32_t kOnes = 0x3F803F80u;  // BF16 +1 in both halves

// Q1: bit 1 -> +1, bit 0 -> -1
__device__ __forceinline__ uint4 expand_q1(uint32_t d) {
  uint32_t v[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t sh = p == 0 ? kPairShift<0> : p == 1 ? kPairShift<1> : p == 2 ? kPairShift<2> : kPairShift<3>;
    v[p] = kOnes | (~pk_shl(d, sh) & kSignBits);
  }
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// ternary: one row's pos xor neg byte in the low byte and its neg byte in
// the high byte of both 16-bit halves.  A packed shift by (7 - k) puts
// element k's nonzero bit at bit 7 and its neg bit at bit 15; bit 7 times
// 0x7F is exactly 0x3F80 (BF16 1.0), and v_bitop3 ORs in the sign: +1, -1
// or 0 (-0 when both bits are set).  Four VALU operations per dword.
__device__ __forceinline__ uint32_t pk_mul_lo(uint32_t a, uint32_t b) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, a) * __builtin_bit_cast(u16x2, b));
}

template <int P>
constexpr uint32_t kTritShift = ((uint32_t)(6 - 2 * P) << 16) | (uint32_t)(7 - 2 * P);

__device__ __forceinline__ uint4 expand_t2(uint32_t comb) {
  uint32_t v[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t sh = p == 0 ? kTritShift<0> : p == 1 ? kTritShift<1> : p == 2 ? kTritShift<2> : kTritShift<3>;
    const uint32_t h = pk_shl(comb, sh);
    v[p] = (h & kSignBits) | pk_mul_lo(h & 0x00800080u, 0x007F007Fu);
  }
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// the byte-J pair of a ternary row: pos xor neg (low byte of each half), neg
// (high byte)
template <int J>
__device__ __forceinline__ uint32_t trit_pair(uint32_t pw, uint32_t qw) {
  return __builtin_amdgcn_perm(qw, pw ^ qw, (uint32_t)J | ((uint32_t)(4 + J) << 8) |
                                                ((uint32_t)J << 16) | ((uint32_t)(4 + J) << 24));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;  // NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Output tile of this work-group.  The grid's work-groups go to the CU
// dies (XCDs, 8 on MI355X, each with its own L2) round-robin by linear
// index.  With `xcd` set (the launcher sets it when every tile of the grid
// runs in the first round of work-groups and the tile count is a multiple
// of 8), die x is given the tiles x T/8 .. (x + 1) T/8 - 1 in row-of-tiles
// order, so that one L2 serves a few whole rows of tiles: every X row of
// an M tile is then fetched into one L2 instead of into all eight (with the
// N tile fastest, each die held a share of every M tile and streamed all
// of X through its L2).  Grids of several rounds keep the plain order: the
// order then also decides which tiles run together, and a 2048x8192x2048
// 1-bit GEMM ran 14 % slower with the die order.
__device__ __forceinline__ void block_tile(int xcd, int64_t& tm, int64_t& tn) {
  const uint32_t nn = gridDim.x, total = gridDim.x * gridDim.y;
  uint32_t l = blockIdx.x + nn * blockIdx.y;
  if (xcd) l = (l & 7u) * (total >> 3) + (l >> 3);
  tm = l / nn;
  tn = l % nn;
}

// the die order applies: one round of work-groups, a multiple of 8 tiles
inline int xcd_order(dim3 grid) {
  const int64_t tiles = (int64_t)grid.x * grid.y;
  return tiles % 8 == 0 && tiles <= (int64_t)device_cu_count() ? 1 : 0;
}

// Waves with a single 32 x 32 block keep a single LDS buffer per team (three
// waves per SIMD fit); larger wave blocks double-buffer
template <int BM, int BN, int WM, int WN>
constexpr bool kSingleBuffer = BM == 32 * WM && BN == 32 * WN;

// A team of WM x WN waves owns a BM x BN tile (wave tiles (BM/WM) x (BN/WN),
// made of 32 x 32 blocks); KT teams split the tile's K groups.
template <int FMT, bool OUT_F32, int BM, int BN, int KT, int WM = 2, int WN = 2>
__global__ __launch_bounds__(64 * WM * WN * KT, (kSingleBuffer<BM, BN, WM, WN> ? 2 : 1)) void gemm_kernel(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ x, int64_t m, int64_t n, int64_t k, void* __restrict__ y,
    int xcd) {
  constexpr int NT = 64 * WM * WN;                // threads per team
  constexpr int WBM = BM / (32 * WM);             // 32-row blocks per wave
  constexpr int WBN = BN / (32 * WN);             // 32-col blocks per wave
  constexpr int XS = BM * kRowU4;                 // 16-B X slots per group
  constexpr int XL = (XS + NT - 1) / NT;          // X slots per thread per group
  constexpr bool kXPartial = XS % NT != 0;        // the last slot is not every thread's
  constexpr int CB = Fmt<FMT>::cell_bytes;
  constexpr int TPC = NT / BN;                    // threads per code cell
  constexpr int RPT = 16 / TPC;                   // W rows expanded per thread per group
  static_assert(NT % BN == 0 && 16 % TPC == 0 && RPT <= 8, "W cells split evenly");
  static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "wave tiles of 32 x 32 blocks");

  constexpr bool kSingle = kSingleBuffer<BM, BN, WM, WN>;
  // work-groups of more than four waves (wide tiles, or two K-teams) run
  // alone on a CU and have LDS to spare: their register ring stages into two
  // LDS buffers per team
  constexpr bool kWide = WM * WN > 4 || KT > 1;
  constexpr int NB = kSingle && !kWide ? 1 : 2;  // LDS buffers per team
  // X buffers are separate arrays so that loads straight into one of them
  // are not taken to alias reads of the other
  __shared__ uint4 xs0[KT][BM * kRowU4];
  __shared__ uint4 xs1[KT][NB > 1 ? BM * kRowU4 : 1];
  __shared__ uint4 ws[KT][NB][BN * kRowU4];

  // KT teams of NT threads share the output tile; team t takes the groups
  // g = t (mod KT) and has its own LDS buffers
  const int tid = (NT & (NT - 1)) == 0 ? (int)(threadIdx.x & (NT - 1))
                  : KT == 1             ? (int)threadIdx.x
                                        : (int)(threadIdx.x % NT);
  const int team = KT == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)(threadIdx.x / NT));
  const int lane = tid & 63;
  const int wave = tid >> 6;
  auto xbuf = [&](int b) __attribute__((always_inline)) -> uint4* {
    return b == 0 ? &xs0[team][0] : &xs1[team][0];
  };
  const int wm = wave / WN, wn = wave % WN;
  int64_t tm, tn;
  block_tile(xcd, tm, tn);
  const int64_t m0 = tm * BM;
  const int64_t n0 = tn * BN;
  const int64_t groups = k / BK;
  const int64_t chunks = k / kChunk;
  const int64_t ntiles = (n + kTileRows - 1) / kTileRows;

  // Loads go through buffer resources that cover this tile's rows of X, W
  // codes and scales: the per-lane offsets are fixed, the group offset is a
  // scalar, and an offset past a resource (rows of X past m, row tiles of W
  // past the end) returns zeros.  Every resource stays below 2^31 bytes for
  // k <= 2^22 (the library's limit).
  const int64_t xrows = m - m0 < BM ? m - m0 : BM;
  const int64_t wtiles0 = n0 / kTileRows;
  const int64_t wtiles = ntiles - wtiles0 < BN / 16 ? ntiles - wtiles0 : BN / 16;
  const __amdgpu_buffer_rsrc_t xres = buffer_rsrc(x + m0 * k, xrows * k * 2);
  const __amdgpu_buffer_rsrc_t wres = buffer_rsrc(codes + wtiles0 * chunks * CB, wtiles * chunks * CB);
  const __amdgpu_buffer_rsrc_t sres =
      buffer_rsrc(scales + wtiles0 * groups * kTileRows, wtiles * groups * kTileRows * 2);

  // --- X staging: slot i = tid + NT*j is row i/16, 16-byte column i%16 of
  // the group (rows past m read zeros; those outputs are never stored).
  // When NT does not divide the slots, the last slot exists for the first
  // XS - NT*(XL-1) threads only (whole waves): the others load a valid row
  // and store nothing.
  uint32_t xoff[XL];
  int xdst[XL];
  const bool xlast = !kXPartial || tid + NT * (XL - 1) < XS;
#pragma unroll
  for (int j = 0; j < XL; ++j) {
    const int i = (j == XL - 1 && !xlast) ? tid : tid + NT * j;
    xoff[j] = (uint32_t)((i >> 4) * k * 2 + (i & 15) * 16);
    xdst[j] = slot(i >> 4, i & 15);
  }

  // --- X straight into LDS (two-buffer kernels): DMA round j of wave w
  // fills slots w * 64 + j * NT .. + 63 (lane l the slot + l); slot p holds
  // row p / 16 and 16-byte column (p % 16) ^ (row % 16), the swizzle above.
  // The last round exists for the waves whose slots are below XS.  (The
  // two-team kernel measured slower this way and keeps the register path.)
  constexpr bool kDma = kWide && KT == 1;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  uint32_t xdma[XL];
#pragma unroll
  for (int j = 0; j < XL; ++j) {
    const int p = wv * 64 + j * NT + lane;
    const int r = p >> 4, c = (p & 15) ^ (r & 15);
    xdma[j] = (uint32_t)(r * k * 2 + c * 16);
  }
  auto dma_x = [&](int64_t g, int b) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < XL; ++j) {
      const int p0 = wv * 64 + j * NT;
      // (device pass only: the host pass has no LDS address space for the
      // builtin's operand, and would drop the kernel's launch stub)
#if defined(__HIP_DEVICE_COMPILE__)
      if (j < XL - 1 || p0 < XS)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            xres, (__attribute__((address_space(3))) void*)(xbuf(b) + p0), 16, xdma[j],
            (int)(g * BK * 2), 0, 0);
#else
      (void)p0;
#endif
    }
  };

  // --- W codes: thread -> cell ci = tid % BN (row tile ci/16, chunk ci%16
  // of the group), rows part*RPT .. part*RPT + RPT-1 of that cell, part =
  // tid / BN; eight consecutive lanes write one row, eight different slots.
  // A tile past the end reads zero codes (Q1: -1, never stored; T2: 0).
  const int ci = tid % BN, part = tid / BN;
  const int wt = ci >> 4, wc = ci & 15;
  const uint32_t woff = (uint32_t)((wt * chunks + wc) * CB + part * RPT);
  int wdst[RPT];
#pragma unroll
  for (int rr = 0; rr < RPT; ++rr) wdst[rr] = slot(wt * 16 + part * RPT + rr, wc);

  // --- scales of this lane's output columns (one per n-block)
  const int jl = lane & 31;
  int64_t ncol[WBN];
  bool nvalid[WBN];
  uint32_t soff[WBN];
#pragma unroll
  for (int bj = 0; bj < WBN; ++bj) {
    ncol[bj] = n0 + wn * (BN / WN) + bj * 32 + jl;
    nvalid[bj] = ncol[bj] < n;
    const int64_t nl = ncol[bj] - n0;
    soff[bj] = (uint32_t)((((nl >> 4) * groups) * kTileRows + (nl & 15)) * 2);
  }

  // Prefetched data stays raw until it is used one iteration later (a
  // select on a just-loaded value would force an immediate wait).  Invalid
  // columns are zeroed at use.
  constexpr int CW = (RPT * 1 + 3) / 4;  // code words per plane per thread
  struct Stage {
    u32x4 xr[XL];
    uint32_t p[CW], q[CW];
    uint32_t sh[WBN];
  };
  auto fetch = [&](int64_t g, Stage& st) __attribute__((always_inline)) {
    const int xg = (int)(g * BK * 2), wg = (int)(g * kChunksPerGroup * CB);
    if constexpr (!kDma) {
#pragma unroll
      for (int j = 0; j < XL; ++j) st.xr[j] = __builtin_amdgcn_raw_buffer_load_b128(xres, xoff[j], xg, 0);
    }
    if constexpr (RPT == 8) {
      const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(wres, woff, wg, 0);
      st.p[0] = a.x;
      st.p[1] = a.y;
      if constexpr (FMT == 2) {
        const u32x2 c2 = __builtin_amdgcn_raw_buffer_load_b64(wres, woff + 16, wg, 0);
        st.q[0] = c2.x;
        st.q[1] = c2.y;
      }
    } else if constexpr (RPT == 2) {
      st.p[0] = __builtin_amdgcn_raw_buffer_load_b16(wres, woff, wg, 0);
      if constexpr (FMT == 2) st.q[0] = __builtin_amdgcn_raw_buffer_load_b16(wres, woff + 16, wg, 0);
    } else {
      st.p[0] = __builtin_amdgcn_raw_buffer_load_b32(wres, woff, wg, 0);
      if constexpr (FMT == 2) st.q[0] = __builtin_amdgcn_raw_buffer_load_b32(wres, woff + 16, wg, 0);
    }
#pragma unroll
    for (int bj = 0; bj < WBN; ++bj)
      st.sh[bj] = __builtin_amdgcn_raw_buffer_load_b16(sres, soff[bj], (int)(g * kTileRows * 2), 0);
  };
  auto stash = [&](const Stage& st, int b) __attribute__((always_inline)) {
    if constexpr (!kDma) {
#pragma unroll
      for (int j = 0; j < XL; ++j)
        if (j < XL - 1 || xlast)
          xbuf(b)[xdst[j]] = make_uint4(st.xr[j].x, st.xr[j].y, st.xr[j].z, st.xr[j].w);
    }
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
      const uint32_t pw = st.p[rr >> 2];
      uint4 e;
      if constexpr (FMT == 1) {
        uint32_t dp;
        switch (rr & 3) {
          case 0: dp = rep_byte<0>(pw); break;
          case 1: dp = rep_byte<1>(pw); break;
          case 2: dp = rep_byte<2>(pw); break;
          default: dp = rep_byte<3>(pw); break;
        }
        e = expand_q1(dp);
      } else {
        const uint32_t qw = st.q[rr >> 2];
        uint32_t comb;
        switch (rr & 3) {
          case 0: comb = trit_pair<0>(pw, qw); break;
          case 1: comb = trit_pair<1>(pw, qw); break;
          case 2: comb = trit_pair<2>(pw, qw); break;
          default: comb = trit_pair<3>(pw, qw); break;
        }
        e = expand_t2(comb);
      }
      ws[team][b][wdst[rr]] = e;
    }
  };
  auto scale_of = [&](const Stage& st, int bj) __attribute__((always_inline)) {
    return nvalid[bj] ? (float)__builtin_bit_cast(_Float16, (uint16_t)st.sh[bj]) : 0.0f;
  };

  f32x16 acc[WBM][WBN];
#pragma unroll
  for (int bi = 0; bi < WBM; ++bi)
#pragma unroll
    for (int bj = 0; bj < WBN; ++bj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[bi][bj][v] = 0.0f;

  // local group index gl -> group gl * KT + team, clamped to the last group
  // (fetched into a stage whose result is discarded)
  const int64_t nloc = (groups + KT - 1) / KT;
  auto gof = [&](int64_t gl) __attribute__((always_inline)) {
    const int64_t g = gl * KT + team;
    return g < groups ? g : groups - 1;
  };
  const int kh = lane >> 5;  // which 8 of the 16 k of a step this lane holds
  // a single 32 x 32 block per wave runs two independent accumulation chains
  // (even and odd k-steps), so consecutive MFMAs do not wait on each other
  constexpr int NCH = (WBM * WBN == 1 && !kSingle) ? 2 : 1;
  auto read_a = [&](int b, int step, int bi) __attribute__((always_inline)) {
    return __builtin_bit_cast(bf16x8, xbuf(b)[slot(wm * (BM / WM) + bi * 32 + jl, step * 2 + kh)]);
  };
  auto read_b = [&](int b, int step, int bj) __attribute__((always_inline)) {
    return __builtin_bit_cast(bf16x8, ws[team][b][slot(wn * (BN / WN) + bj * 32 + jl, step * 2 + kh)]);
  };
  auto mfma_step = [&](f32x16 (&cg)[NCH][WBM][WBN], int step, const bf16x8 (&a)[WBM],
                       const bf16x8 (&bb)[WBN]) __attribute__((always_inline)) {
#pragma unroll
    for (int bi = 0; bi < WBM; ++bi)
#pragma unroll
      for (int bj = 0; bj < WBN; ++bj) {
        const int ch = step % NCH;
        const f32x16 zero = {};
        cg[ch][bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            a[bi], bb[bj], step < NCH ? zero : cg[ch][bi][bj], 0, 0, 0);
      }
  };
  // acc += s * (sum of the chains); a group past the end leaves acc unchanged
  // (`live` is wave-uniform: a scalar branch, not a select per accumulator)
  auto scale_add = [&](const f32x16 (&cg)[NCH][WBM][WBN], const float (&sv)[WBN], bool live)
      __attribute__((always_inline)) {
    if (!live) return;
#pragma unroll
    for (int bi = 0; bi < WBM; ++bi)
#pragma unroll
      for (int bj = 0; bj < WBN; ++bj)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float f = __builtin_fmaf(sv[bj], cg[0][bi][bj][v], acc[bi][bj][v]);
          if constexpr (NCH == 2) f = __builtin_fmaf(sv[bj], cg[NCH - 1][bi][bj][v], f);
          acc[bi][bj][v] = f;
        }
  };

  if constexpr (kSingle) {
    // Two register stages: group g + 2 is fetched (into the stage group g
    // was staged from, one body earlier) while group g is multiplied and
    // group g + 1 is staged into LDS.  The operands of g are read from LDS in
    // two halves of four k-steps.  With ONE LDS buffer (2 x 2 waves, three
    // work-groups per CU), once every wave holds the second half (barrier)
    // group g + 1 is written over them while the last four k-steps run.
    // Work-groups alone on a CU alternate between two LDS buffers:
    // group g + 1 goes to the other buffer with no mid-group barrier, for
    // ternary codes spread over all eight k-steps.  Stages are separate
    // variables and the body is written out twice, so neither a stage nor a
    // buffer is indexed at run time (buffer offsets fold into the LDS
    // instructions' immediate offsets).
    Stage s0, s1;
    float sv[WBN];
    // staging VALU per MFMA of the second half (about 10 (Q1) / 17 (T2) per
    // expanded W row)
    constexpr int kValu = (RPT * (FMT == 1 ? 10 : 17) + 3) / 4;
    constexpr int kDsw = (XL + RPT + 3) / 4;  // staging LDS writes per MFMA
    constexpr bool kSpread = kWide && FMT == 2;
    constexpr int kValu8 = (kValu + 1) / 2, kDsw8 = (XL + RPT + 7) / 8;  // spread over 8
#define LOWBIT_GEMM_ITER1(G, FAR, NEAR, BUF)                                                   \
  {                                                                                           \
    constexpr int RB = kWide ? (BUF) : 0; /* LDS buffer of group G */                         \
    if constexpr (kDma) dma_x(gof((G) + 1), RB ^ 1);                                          \
    fetch(gof((G) + 2), FAR);                                                                 \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    f32x16 cg[NCH][WBM][WBN];                                                                 \
    bf16x8 a[4][WBM], bb[4][WBN];                                                             \
    _Pragma("unroll") for (int r = 0; r < 4; ++r) {                                           \
      _Pragma("unroll") for (int bi = 0; bi < WBM; ++bi) a[r][bi] = read_a(RB, r, bi);        \
      _Pragma("unroll") for (int bj = 0; bj < WBN; ++bj) bb[r][bj] = read_b(RB, r, bj);       \
    }                                                                                         \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    /* two buffers: group G + 1 is staged into the other one, across all */                   \
    /* eight k-steps for ternary codes (1-bit ones would spill) */                            \
    if constexpr (kSpread) stash(NEAR, RB ^ 1);                                               \
    /* steps 0..3, each followed by the reads of step r + 4 into its registers */            \
    _Pragma("unroll") for (int r = 0; r < 4; ++r) {                                           \
      mfma_step(cg, r, a[r], bb[r]);                                                          \
      _Pragma("unroll") for (int bi = 0; bi < WBM; ++bi) a[r][bi] = read_a(RB, r + 4, bi);    \
      _Pragma("unroll") for (int bj = 0; bj < WBN; ++bj) bb[r][bj] = read_b(RB, r + 4, bj);   \
    }                                                                                         \
    _Pragma("unroll") for (int r = 0; r < 4 * WBM * WBN; ++r) {                               \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                      \
      __builtin_amdgcn_sched_group_barrier(0x100, (WBM + WBN) / (WBM * WBN), 0);              \
      if constexpr (kSpread) {                                                                \
        __builtin_amdgcn_sched_group_barrier(0x002, kValu8, 0);                               \
        __builtin_amdgcn_sched_group_barrier(0x200, kDsw8, 0);                                \
      }                                                                                       \
    }                                                                                         \
    /* one buffer: once every wave holds its operands (barrier), group G + 1 */              \
    /* is written over them during the last four k-steps */                                   \
    if constexpr (!kWide) __syncthreads();                                                    \
    _Pragma("unroll") for (int r = 0; r < 4; ++r) mfma_step(cg, r + 4, a[r], bb[r]);          \
    if constexpr (!kSpread) stash(NEAR, RB ^ (int)kWide);                                     \
    _Pragma("unroll") for (int r = 0; r < 4 * WBM * WBN; ++r) {                               \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                      \
      __builtin_amdgcn_sched_group_barrier(0x002, kSpread ? kValu8 : kValu, 0);               \
      __builtin_amdgcn_sched_group_barrier(0x200, kSpread ? kDsw8 : kDsw, 0);                 \
    }                                                                                         \
    scale_add(cg, sv, kAllLive || (G) * KT + team < groups);                                  \
    _Pragma("unroll") for (int bj = 0; bj < WBN; ++bj) sv[bj] = scale_of(NEAR, bj);           \
    __syncthreads();                                                                          \
  }
#define LOWBIT_GEMM_START1(FIRST, SECOND, BUF)                                                 \
  {                                                                                           \
    if constexpr (kDma) dma_x(gof(0), BUF);                                                   \
    fetch(gof(0), FIRST);                                                                     \
    fetch(gof(1), SECOND);                                                                    \
    stash(FIRST, kWide ? (BUF) : 0);                                                          \
    _Pragma("unroll") for (int bj = 0; bj < WBN; ++bj) sv[bj] = scale_of(FIRST, bj);          \
    __syncthreads();                                                                          \
  }
    // The loop body is entered with group g in LDS buffer 0, group g + 1 in
    // s1 and s0 free.  With an odd group count the first group runs before
    // the loop, with the stages and buffers named so that it leaves exactly
    // that state: no group body runs past the end (a group past the end of
    // one K-team still runs as a no-op).  The 2 x 2 wave kernels keep the
    // plain loop, whose last pass may run one body as a no-op: the extra
    // entry code would cost them their third wave per SIMD.
    constexpr bool kPeel = WM * WN > 4;
    constexpr bool kAllLive = kPeel && KT == 1;  // every body has a group: no selects
    const int64_t rem = kPeel ? nloc % 2 : 0;
    if (rem == 0) {
      LOWBIT_GEMM_START1(s0, s1, 0)
    } else {
      LOWBIT_GEMM_START1(s1, s0, 1)
      LOWBIT_GEMM_ITER1(0, s1, s0, 1)
    }
    // Branch-free body (a branch would let the compiler sink the prefetch
    // loads into the blocks that consume them).
    for (int64_t g = rem; g < nloc; g += 2) {
      LOWBIT_GEMM_ITER1(g, s0, s1, 0)
      LOWBIT_GEMM_ITER1(g + 1, s1, s0, 1)
    }
#undef LOWBIT_GEMM_START1
#undef LOWBIT_GEMM_ITER1
  } else {
  // Ring of four register stages: group g + 3 is fetched while group g is
  // multiplied and group g + 1 (fetched two iterations ago) is written to the
  // other LDS buffer, so three groups of loads are in flight.  The stages are
  // separate variables and the loop body is written out four times, so no
  // stage is ever indexed at run time.
  Stage s0, s1, s2, s3;
  fetch(gof(0), s0);
  fetch(gof(1), s1);
  fetch(gof(2), s2);
  stash(s0, 0);
  float sv[WBN];
#pragma unroll
  for (int bj = 0; bj < WBN; ++bj) sv[bj] = scale_of(s0, bj);
  __syncthreads();

  constexpr int RS = WBM * WBN >= 4 ? 2 : 8;  // k-steps whose operands are read at once
  constexpr bool kInterleave = RS == BK / 16;
  constexpr int kValuPerMfma = FMT == 1 ? 4 : 8;
  // one group: fetch group G + 3 into FAR, multiply group G from LDS buffer
  // B, then stage group G + 1 (NEAR) into buffer B ^ 1.  Written as a macro
  // so that the stages stay plain register variables.
#define LOWBIT_GEMM_ITER(G, B, FAR, NEAR)                                                      \
  {                                                                                           \
    /* clamped: the tail re-fetches the last group into a stage nobody reads; */              \
    /* the scheduling barrier keeps these loads at the top */                                 \
    fetch(gof((G) + 3), FAR);                                                                 \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    f32x16 cg[NCH][WBM][WBN];                                                                 \
    /* operands of RS k-steps are read from LDS before their MFMAs, so one LDS */            \
    /* round trip covers RS steps instead of one */                                           \
    _Pragma("unroll") for (int s0 = 0; s0 < BK / 16; s0 += RS) {                              \
      bf16x8 a[RS][WBM], bb[RS][WBN];                                                         \
      _Pragma("unroll") for (int r = 0; r < RS; ++r) {                                        \
        _Pragma("unroll") for (int bi = 0; bi < WBM; ++bi) a[r][bi] = __builtin_bit_cast(     \
            bf16x8, xbuf(B)[slot(wm * (BM / WM) + bi * 32 + jl, (s0 + r) * 2 + kh)]);              \
        _Pragma("unroll") for (int bj = 0; bj < WBN; ++bj) bb[r][bj] = __builtin_bit_cast(    \
            bf16x8, ws[team][B][slot(wn * (BN / WN) + bj * 32 + jl, (s0 + r) * 2 + kh)]);           \
      }                                                                                       \
      __builtin_amdgcn_sched_barrier(0);                                                      \
      _Pragma("unroll") for (int r = 0; r < RS; ++r)                                          \
      _Pragma("unroll") for (int bi = 0; bi < WBM; ++bi)                                      \
      _Pragma("unroll") for (int bj = 0; bj < WBN; ++bj) {                                    \
        const int ch = (s0 + r) % NCH;                                                        \
        if (s0 + r < NCH) {                                                                   \
          const f32x16 zero = {};                                                             \
          cg[ch][bi][bj] =                                                                    \
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[r][bi], bb[r][bj], zero, 0, 0, 0);    \
        } else {                                                                              \
          cg[ch][bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[r][bi], bb[r][bj],       \
                                                                   cg[ch][bi][bj], 0, 0, 0);  \
        }                                                                                     \
      }                                                                                       \
    }                                                                                         \
    /* stage group G + 1 into the other buffer (last read one iteration ago, */              \
    /* before the barrier) while the matrix cores work: when every operand */                \
    /* was read up front, the staging is interleaved with the MFMAs */                       \
    if constexpr (!kInterleave) __builtin_amdgcn_sched_barrier(0);                            \
    stash(NEAR, (B) ^ 1);                                                                     \
    if constexpr (kInterleave) {                                                              \
      _Pragma("unroll") for (int i = 0; i < WBM * WBN * (BK / 16); ++i) {                     \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                    \
        __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);                         \
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);                                    \
      }                                                                                       \
    }                                                                                         \
    /* a group past the end (the last block of four) leaves acc unchanged */                 \
    scale_add(cg, sv, (G) * KT + team < groups);                                              \
    _Pragma("unroll") for (int bj = 0; bj < WBN; ++bj) sv[bj] = scale_of(NEAR, bj);           \
    __syncthreads();                                                                          \
  }
  // Branch-free body (a branch would let the compiler sink the prefetch
  // loads into the blocks that consume them); groups past the end run as
  // no-ops.
  for (int64_t g = 0; g < nloc; g += 4) {
    LOWBIT_GEMM_ITER(g, 0, s3, s1)
    LOWBIT_GEMM_ITER(g + 1, 1, s0, s2)
    LOWBIT_GEMM_ITER(g + 2, 0, s1, s3)
    LOWBIT_GEMM_ITER(g + 3, 1, s2, s0)
  }
#undef LOWBIT_GEMM_ITER
  }

  if constexpr (KT > 1) {
    // teams 1.. leave their sums in their own (no longer read) LDS buffers;
    // team 0 adds them and stores the tile
    if (team > 0) {
      float* red = reinterpret_cast<float*>(&xs0[team][0]);
#pragma unroll
      for (int bi = 0; bi < WBM; ++bi)
#pragma unroll
        for (int bj = 0; bj < WBN; ++bj)
#pragma unroll
          for (int v = 0; v < 16; ++v) red[((bi * WBN + bj) * 16 + v) * NT + tid] = acc[bi][bj][v];
    }
    __syncthreads();
    if (team > 0) return;
#pragma unroll
    for (int t = 1; t < KT; ++t) {
      const float* red = reinterpret_cast<const float*>(&xs0[t][0]);
#pragma unroll
      for (int bi = 0; bi < WBM; ++bi)
#pragma unroll
        for (int bj = 0; bj < WBN; ++bj)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[bi][bj][v] += red[((bi * WBN + bj) * 16 + v) * NT + tid];
    }
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
        const int64_t mm = m0 + wm * (BM / WM) + bi * 32 + i;
        if (mm >= m) continue;
        if constexpr (OUT_F32)
          static_cast<float*>(y)[mm * n + nn] = acc[bi][bj][v];
        else
          static_cast<uint16_t*>(y)[mm * n + nn] = f32_to_bf16_rne(acc[bi][bj][v]);
      }
    }
}

// ---------------------------------------------------------------------------
// Team kernel.  One work-group per CU computes a BM x BN tile with KT
// K-teams of WM x WN waves; team t takes the scale groups g = t (mod KT) and
// the teams' sums are added through LDS at the end.  Each wave owns BI x BJ
// blocks of 32 x 32 (a 32 x 96 or 32 x 64 wave tile reads 1.33 / 1.5 KB of
// LDS operands per matrix-core instruction, against 2 KB for a lone block),
// and with two K-teams of four waves, or four of two, eight waves share the
// CU.  The K loop runs in stages of 64 (half a scale group) so that every
// team can double-buffer its stage in LDS:
//   * X[BM][64] BF16 goes straight from memory into LDS (buffer loads to
//     LDS, one stage ahead), its 16-byte slots XOR-swizzled by the row;
//   * the codes of W[BN][64] are loaded one stage ahead into registers,
//     one byte (and for ternary codes the neg byte) per row-chunk, then
//     expanded to exact BF16 {-1, 0, +1} and written to LDS while the
//     matrix cores work on the current stage, so each W row is expanded
//     once per BM rows of X;
//   * 4 k-steps of 16 per stage accumulate the group's unscaled FP32 sum
//     C_g (over the group's two stages), then C += s[n][g] * C_g in FP32.
// One barrier per stage.  The nearest-even rounding to BF16 happens once,
// at the store.
constexpr int SK = 64;        // k per pipeline stage: half a scale group
constexpr int kSS = SK / 8;   // 16-byte slots per LDS row of a stage

// LDS slot of 16-byte column c of row r in a stage buffer (128-byte rows).
// The XOR with (r & 7) ^ ((r >> 3) & 1) puts any 8, and any 16, consecutive
// rows' copies of one column in distinct 16-byte bank groups, whether the
// banks span 128 or 256 bytes.
__device__ __forceinline__ int sslot(int r, int c) {
  return r * kSS + (c ^ ((r & 7) ^ ((r >> 3) & 1)));
}

template <int FMT, bool OUT_F32, int BI, int BJ, int WM, int WN, int KT, bool ALL_LIVE>
__global__ __launch_bounds__(64 * WM * WN * KT, 1) void gemm_team_kernel(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ x, int64_t m, int64_t n, int64_t k, void* __restrict__ y,
    int xcd) {
  constexpr int NWT = WM * WN;        // waves per team
  constexpr int NT = 64 * NWT;        // threads per team
  constexpr int BM = 32 * BI * WM, BN = 32 * BJ * WN;
  constexpr int XI = BM * kSS / 64;   // X loads to LDS per team-stage (64 slots each)
  static_assert(XI % NWT == 0, "X stage splits evenly over a team's waves");
  constexpr int XIW = XI / NWT;
  constexpr int UPT = BN * kSS / NT;  // W row-chunks expanded per thread per stage
  static_assert((BN * kSS) % NT == 0 && (NT & (NT - 1)) == 0, "W stage splits evenly");
  static_assert(BN % 16 == 0, "whole row tiles of W");
  constexpr int CB = Fmt<FMT>::cell_bytes;

  // per team three X stage buffers (loads go out two stages ahead) and two
  // W stage buffers, all separate variables: a load into one is not taken
  // to alias the reads of another
  __shared__ uint4 xs0[KT][BM * kSS];
  __shared__ uint4 xs1[KT][BM * kSS];
  __shared__ uint4 xs2[KT][BM * kSS];
  __shared__ uint4 ws0[KT][BN * kSS];
  __shared__ uint4 ws1[KT][BN * kSS];

  const int tid = (int)(threadIdx.x & (NT - 1));
  const int team = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / NT));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, kh = lane >> 5;

  int64_t tm, tn;
  block_tile(xcd, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int G = (int)(k / BK);
  const int64_t chunks = k / kChunk;
  const int64_t ntiles = (n + kTileRows - 1) / kTileRows;
  const int64_t xrows = m - m0 < BM ? m - m0 : BM;
  const int64_t wt0 = n0 / kTileRows;
  const int64_t wtiles = ntiles - wt0 < BN / 16 ? ntiles - wt0 : BN / 16;
  // buffer resources over this tile's rows: offsets past them read zeros
  const __amdgpu_buffer_rsrc_t xres = buffer_rsrc(x + m0 * k, xrows * k * 2);
  const __amdgpu_buffer_rsrc_t wres = buffer_rsrc(codes + wt0 * chunks * CB, wtiles * chunks * CB);
  const __amdgpu_buffer_rsrc_t sres =
      buffer_rsrc(scales + wt0 * G * kTileRows, wtiles * G * kTileRows * 2);

  // X: load j of this wave fills slots (wave + NWT j) * 64 + lane of the
  // team's stage buffer; slot p holds row p / 8, 16-byte column
  // (p % 8) ^ swizzle(row) of the stage
  uint32_t xvoff[XIW];
#pragma unroll
  for (int j = 0; j < XIW; ++j) {
    const int p = (wave + NWT * j) * 64 + lane;
    const int r = p >> 3;
    const int c = (p & 7) ^ ((r & 7) ^ ((r >> 3) & 1));
    xvoff[j] = (uint32_t)(r * k * 2 + c * 16);
  }
  auto dma_x = [&](int stage_k, uint4 (*buf)[BM * kSS]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < XIW; ++j) {
#if defined(__HIP_DEVICE_COMPILE__)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xres, (__attribute__((address_space(3))) void*)(&buf[team][0] + (wave + NWT * j) * 64), 16,
          xvoff[j], stage_k * 2, 0, 0);
#else
      (void)buf;
      (void)stage_k;
#endif
    }
  };

  // W: row-chunk u = tid + NT i of a stage is row u % BN, chunk u / BN.
  // Its code byte is byte (r % 4) of the dword loaded at r % 16 rounded
  // down to 4 (whole dwords: a narrower load would be widened right where
  // it returns, which waits for it there); the byte is picked at use by a
  // per-lane v_perm selector.
  uint32_t wvoff[UPT], wsel[UPT];
  int wdst[UPT];
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = tid + NT * i;
    const int r = u % BN, c = u / BN;
    const uint32_t bj = (uint32_t)(r & 3);
    wvoff[i] = (uint32_t)(((r >> 4) * chunks + c) * CB + (r & 12));
    // Q1: byte bj in the low byte of both halves; ternary: pos ^ neg there
    // and neg in the high byte (the trit_pair layout)
    wsel[i] = FMT == 1 ? (0x0C000C00u | (bj << 16) | bj)
                       : (bj | ((4u + bj) << 8) | (bj << 16) | ((4u + bj) << 24));
    wdst[i] = sslot(r, c);
  }
  struct Codes {
    uint32_t p[UPT], q[UPT];
  };
  auto load_codes = [&](int stage_chunk, Codes& cd) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      cd.p[i] = __builtin_amdgcn_raw_buffer_load_b32(wres, wvoff[i], stage_chunk * CB, 0);
      if constexpr (FMT == 2)
        cd.q[i] = __builtin_amdgcn_raw_buffer_load_b32(wres, wvoff[i] + 16, stage_chunk * CB, 0);
    }
  };
  // expand row-chunk i of a stage into a W buffer
  auto expand_unit = [&](const Codes& cd, int i, uint4 (*buf)[BN * kSS])
                         __attribute__((always_inline)) {
    uint4 e;
    if constexpr (FMT == 1)
      e = expand_q1(__builtin_amdgcn_perm(cd.p[i], cd.p[i], wsel[i]));
    else
      e = expand_t2(__builtin_amdgcn_perm(cd.q[i], cd.p[i] ^ cd.q[i], wsel[i]));
    buf[team][wdst[i]] = e;
  };
  auto expand = [&](const Codes& cd, uint4 (*buf)[BN * kSS]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) expand_unit(cd, i, buf);
  };

  // scales of this lane's output columns: the dword holding the FP16 value
  // (whole dwords, as for the codes), shifted into place at use
  uint32_t svoff[BJ], svsh[BJ];
  bool nvalid[BJ];
#pragma unroll
  for (int bj = 0; bj < BJ; ++bj) {
    const int nl = wn * (BJ * 32) + bj * 32 + l32;
    nvalid[bj] = n0 + nl < n;
    svoff[bj] = (uint32_t)((((nl >> 4) * G) * kTileRows + (nl & 14)) * 2);
    svsh[bj] = (uint32_t)(nl & 1) * 16;
  }

  // team-local group gl is group gl * KT + team; past the end a team's
  // stages load the last group again and add nothing (team-uniform)
  const int nloc = (G + KT - 1) / KT;
  auto gclamp = [&](int gl) __attribute__((always_inline)) {
    const int g = gl * KT + team;
    return g < G ? g : G - 1;
  };
  auto stage_chunk = [&](int j) __attribute__((always_inline)) {
    return gclamp(j >> 1) * kChunksPerGroup + (j & 1) * kSS;
  };
  auto stage_k = [&](int j) __attribute__((always_inline)) { return stage_chunk(j) * kChunk; };

  // acc: the scaled sum (plain floats: element updates of a vector type
  // cost register copies); cg: the current group's unscaled sum
  float acc[BI][BJ][16];
  f32x16 cg[BI][BJ];
#pragma unroll
  for (int bi = 0; bi < BI; ++bi)
#pragma unroll
    for (int bj = 0; bj < BJ; ++bj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[bi][bj][v] = 0.0f;

  auto read_a = [&](uint4 (*buf)[BM * kSS], int s, int bi) __attribute__((always_inline)) {
    return __builtin_bit_cast(bf16x8, buf[team][sslot(wm * (BI * 32) + bi * 32 + l32, 2 * s + kh)]);
  };
  auto read_b = [&](uint4 (*buf)[BN * kSS], int s, int bj) __attribute__((always_inline)) {
    return __builtin_bit_cast(bf16x8, buf[team][sslot(wn * (BJ * 32) + bj * 32 + l32, 2 * s + kh)]);
  };

  // Pipeline, stage j (phase P = j mod 6, so that every buffer and register
  // set below is named at compile time):
  //   X_j in xs[j % 3]; X_{j+1} and X_{j+2} on their way into the others;
  //   W_j in ws[j % 2]; codes_{j+1}, codes_{j+2} in registers.
  //   1. load codes_{j+3} into c[j % 3] (codes_j were expanded in stage j-1);
  //      at the first stage of a group, load the next group's scales;
  //   2. four k-steps of MFMAs on X_j, W_j;
  //   3. expand codes_{j+1} into ws[(j+1) % 2] (read last in stage j-1);
  //   4. at the second stage of a group, acc += s * C_g;
  //   5. wait for this wave's loads of X_{j+1}, barrier;
  //   6. load X_{j+3} into xs[j % 3], which every wave has finished reading.
  Codes c0, c1, c2;
  const int S = 2 * nloc;
  auto clampj = [&](int j) __attribute__((always_inline)) { return j < S ? j : S - 1; };
  // scales of the three groups of an unrolled pass: group q of the pass in
  // sv[q], loaded at the first stage of the group before it
  // (FP16 bit patterns, converted at use: a conversion placed next to the
  // load would wait for it there)
  uint32_t sv0[BJ], sv1[BJ], sv2[BJ];
  auto load_scales = [&](int gl, uint32_t (&sv)[BJ]) __attribute__((always_inline)) {
#pragma unroll
    for (int bj = 0; bj < BJ; ++bj)
      sv[bj] = __builtin_amdgcn_raw_buffer_load_b32(sres, svoff[bj], gclamp(gl) * kTileRows * 2, 0);
  };
  auto scale_f = [&](uint32_t h, int bj) __attribute__((always_inline)) {
    return nvalid[bj] ? (float)__builtin_bit_cast(_Float16, (uint16_t)(h >> svsh[bj])) : 0.0f;
  };
  // memory loads per stage: codes, and X into LDS
  constexpr int kCodeLoads = UPT * (FMT == 2 ? 2 : 1);
  // at the end of stage j, loads issued after X_{j+1}'s: codes of two
  // stages, one set of scales, X_{j+2}
  constexpr int kVm = 2 * kCodeLoads + BJ + XIW;

  load_codes(stage_chunk(0), c0);
  dma_x(stage_k(0), xs0);
  load_codes(stage_chunk(clampj(1)), c1);
  dma_x(stage_k(clampj(1)), xs1);
  load_codes(stage_chunk(clampj(2)), c2);
  dma_x(stage_k(clampj(2)), xs2);
  load_scales(0, sv0);
  expand(c0, ws0);
  // X_0 has landed: loads issued after it are codes_1, X_1, codes_2, X_2 and
  // the scales
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kCodeLoads + 2 * XIW + BJ));
  __syncthreads();

  // One stage: the matrix-core steps on X_j and W_j, then the expansion of
  // the next stage's W; at the group's second stage, C += s * C_g.
#define LOWBIT_TEAM_MFMA(XB, WB, SV, H)                                                       \
  {                                                                                           \
    _Pragma("unroll") for (int s = 0; s < SK / 16; ++s) {                                     \
      bf16x8 a[BI], b[BJ];                                                                    \
      _Pragma("unroll") for (int bi = 0; bi < BI; ++bi) a[bi] = read_a(XB, s, bi);            \
      _Pragma("unroll") for (int bj = 0; bj < BJ; ++bj) b[bj] = read_b(WB, s, bj);            \
      _Pragma("unroll") for (int bi = 0; bi < BI; ++bi)                                       \
      _Pragma("unroll") for (int bj = 0; bj < BJ; ++bj) cg[bi][bj] =                          \
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(                                            \
              a[bi], b[bj], ((H) == 0 && s == 0) ? (f32x16){} : cg[bi][bj], 0, 0, 0);         \
    }                                                                                         \
  }
#define LOWBIT_TEAM_STAGE(P, XB, WB, WN_, CL, CE, SV, SVN)                                     \
  {                                                                                           \
    const int j = j0 + (P);                                                                   \
    constexpr int H = (P) & 1; /* half of the scale group */                                  \
    load_codes(stage_chunk(clampj(j + 3)), CL);                                               \
    if constexpr (H == 0) load_scales((j >> 1) + 1, SVN);                                     \
    LOWBIT_TEAM_MFMA(XB, WB, SV, H)                                                           \
    expand(CE, WN_);                                                                          \
    if constexpr (H == 1) {                                                                   \
      if (ALL_LIVE || (j >> 1) * KT + team < G) {                                             \
        _Pragma("unroll") for (int bi = 0; bi < BI; ++bi)                                     \
        _Pragma("unroll") for (int bj = 0; bj < BJ; ++bj) {                                   \
          const float sc = scale_f(SV[bj], bj);                                               \
          _Pragma("unroll") for (int v = 0; v < 16; ++v) acc[bi][bj][v] =                     \
              __builtin_fmaf(sc, cg[bi][bj][v], acc[bi][bj][v]);                              \
        }                                                                                     \
      }                                                                                       \
    }                                                                                         \
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lds(kVm));                                          \
    stage_barrier();                                                                          \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    dma_x(stage_k(clampj(j + 3)), XB);                                                        \
  }
  int j0 = 0;
  for (; j0 + 6 <= S; j0 += 6) {
    LOWBIT_TEAM_STAGE(0, xs0, ws0, ws1, c0, c1, sv0, sv1)
    LOWBIT_TEAM_STAGE(1, xs1, ws1, ws0, c1, c2, sv0, sv1)
    LOWBIT_TEAM_STAGE(2, xs2, ws0, ws1, c2, c0, sv1, sv2)
    LOWBIT_TEAM_STAGE(3, xs0, ws1, ws0, c0, c1, sv1, sv2)
    LOWBIT_TEAM_STAGE(4, xs1, ws0, ws1, c1, c2, sv2, sv0)
    LOWBIT_TEAM_STAGE(5, xs2, ws1, ws0, c2, c0, sv2, sv0)
  }
  // S is even: 0, 2 or 4 stages remain, starting at phase 0
  if (j0 < S) {
    LOWBIT_TEAM_STAGE(0, xs0, ws0, ws1, c0, c1, sv0, sv1)
    LOWBIT_TEAM_STAGE(1, xs1, ws1, ws0, c1, c2, sv0, sv1)
  }
  if (j0 + 2 < S) {
    LOWBIT_TEAM_STAGE(2, xs2, ws0, ws1, c2, c0, sv1, sv2)
    LOWBIT_TEAM_STAGE(3, xs0, ws1, ws0, c0, c1, sv1, sv2)
  }
#undef LOWBIT_TEAM_STAGE
#undef LOWBIT_TEAM_MFMA
  // K-teams 1.. leave their sums in LDS (after every load into it has
  // landed), team 0 adds them and stores the tile
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // element idx = (team - 1) NE + e of a team's sums, for every thread of
  // the team, in xs0, then xs1 (idx is a constant once the loops unroll)
  constexpr int NE = BI * BJ * 16;
  constexpr int CAPX = KT * BM * kSS * 4 / NT;  // elements per thread in one X buffer
  static_assert((KT - 1) * NE <= 3 * CAPX, "the team sums fit in the X buffers");
  auto red = [&](int idx) __attribute__((always_inline)) -> float* {
    return idx < CAPX       ? reinterpret_cast<float*>(&xs0[0][0]) + idx * NT + tid
           : idx < 2 * CAPX ? reinterpret_cast<float*>(&xs1[0][0]) + (idx - CAPX) * NT + tid
                            : reinterpret_cast<float*>(&xs2[0][0]) + (idx - 2 * CAPX) * NT + tid;
  };
  if (team > 0) {
#pragma unroll
    for (int t = 1; t < KT; ++t) {
      if (t != team) continue;
#pragma unroll
      for (int bi = 0; bi < BI; ++bi)
#pragma unroll
        for (int bj = 0; bj < BJ; ++bj)
#pragma unroll
          for (int v = 0; v < 16; ++v) *red((t - 1) * NE + (bi * BJ + bj) * 16 + v) = acc[bi][bj][v];
    }
  }
  __syncthreads();
  if (team > 0) return;
#pragma unroll
  for (int t = 1; t < KT; ++t)
#pragma unroll
    for (int bi = 0; bi < BI; ++bi)
#pragma unroll
      for (int bj = 0; bj < BJ; ++bj)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[bi][bj][v] += *red((t - 1) * NE + (bi * BJ + bj) * 16 + v);

  // C[i][j] of a 32 x 32 block sits in lane j + 32 ((i / 4) % 2), register
  // (i % 4) + 4 (i / 8)
#pragma unroll
  for (int bi = 0; bi < BI; ++bi)
#pragma unroll
    for (int bj = 0; bj < BJ; ++bj) {
      if (!nvalid[bj]) continue;
      const int64_t nn = n0 + wn * (BJ * 32) + bj * 32 + l32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = 8 * (v >> 2) + 4 * kh + (v & 3);
        const int64_t mm = m0 + wm * (BI * 32) + bi * 32 + i;
        if (mm >= m) continue;
        if constexpr (OUT_F32)
          static_cast<float*>(y)[mm * n + nn] = acc[bi][bj][v];
        else
          static_cast<uint16_t*>(y)[mm * n + nn] = f32_to_bf16_rne(acc[bi][bj][v]);
      }
    }
}

template <int FMT, int BI, int BJ, int WM, int WN, int KT>
hipError_t launch_team(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                       const uint16_t* x, int64_t m, void* y, bool out_f32, hipStream_t st) {
  constexpr int BM = 32 * BI * WM, BN = 32 * BJ * WN;
  const dim3 grid((unsigned)((n + BN - 1) / BN), (unsigned)((m + BM - 1) / BM));
  const dim3 block(64 * WM * WN * KT);
  const int xcd = xcd_order(grid);
  // every team has a group at every step when KT divides the group count
  const bool all_live = (k / BK) % KT == 0;
#define LOWBIT_LAUNCH(OF, AL)                                                                  \
  hipLaunchKernelGGL((gemm_team_kernel<FMT, OF, BI, BJ, WM, WN, KT, AL>), grid, block, 0, st,  \
                     codes, scales, x, m, n, k, y, xcd)
  if (out_f32) {
    if (all_live) LOWBIT_LAUNCH(true, true);
    else LOWBIT_LAUNCH(true, false);
  } else {
    if (all_live) LOWBIT_LAUNCH(false, true);
    else LOWBIT_LAUNCH(false, false);
  }
#undef LOWBIT_LAUNCH
  return hipGetLastError();
}

template <int FMT, int BM, int BN, int KT, int WM = 2, int WN = 2>
hipError_t launch_tile(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                       const uint16_t* x, int64_t m, void* y, bool out_f32, hipStream_t st) {
  const dim3 grid((unsigned)((n + BN - 1) / BN), (unsigned)((m + BM - 1) / BM));
  const dim3 block(64 * WM * WN * KT);
  const int xcd = xcd_order(grid);
  if (out_f32)
    hipLaunchKernelGGL((gemm_kernel<FMT, true, BM, BN, KT, WM, WN>), grid, block, 0, st, codes,
                       scales, x, m, n, k, y, xcd);
  else
    hipLaunchKernelGGL((gemm_kernel<FMT, false, BM, BN, KT, WM, WN>), grid, block, 0, st, codes,
                       scales, x, m, n, k, y, xcd);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                      const uint16_t* x, int64_t m, void* y, bool out_f32, hipStream_t st) {
  const int64_t cus = (int64_t)device_cu_count();
  // 128 x 128 tiles when there are enough of them for two per CU
  const int64_t big = ((n + 127) / 128) * ((m + 127) / 128);
  if (big >= 2 * cus)
    return launch_tile<FMT, 128, 128, 1>(codes, scales, n, k, x, m, y, out_f32, st);
  // 128 x 96 tiles when they fill whole rounds of the CUs: the team kernel
  // (two K-teams of four 32 x 96 waves; the ternary pp512 shape, 4 x 64 =
  // 256 tiles, ran 24.3 against 26.8 us cold with the 4 x 3-wave kernel
  // below), or, for a single scale group, twelve 32 x 32 waves (one
  // work-group per CU, three waves per SIMD): each W row is expanded once
  // per 128 rows of X instead of 64
  const int64_t t96 = ((n + 95) / 96) * ((m + 127) / 128);
  if (m >= 128 && t96 >= cus && t96 % cus == 0) {
    if (k >= 2 * BK)
      return launch_team<FMT, 1, 3, 4, 1, 2>(codes, scales, n, k, x, m, y, out_f32, st);
    return launch_tile<FMT, 128, 96, 1, 4, 3>(codes, scales, n, k, x, m, y, out_f32, st);
  }
  // with no more 64 x 64 tiles than CUs, two K-teams per tile (one 8-wave
  // work-group per CU) keep twice as many waves busy
  const int64_t small = ((n + 63) / 64) * ((m + 63) / 64);
  if (small <= cus && k >= 2 * BK)
    return launch_tile<FMT, 64, 64, 2>(codes, scales, n, k, x, m, y, out_f32, st);
  return launch_tile<FMT, 64, 64, 1>(codes, scales, n, k, x, m, y, out_f32, st);
}

}  // namespace

hipError_t launch_gemm(int fmt, const uint8_t* codes, const uint16_t* scales, int64_t n,
                       int64_t k, const uint16_t* x, int64_t m, void* y, bool out_f32,
                       hipStream_t st) {
  if (fmt == 1) return launch_fmt<1>(codes, scales, n, k, x, m, y, out_f32, st);
  return launch_fmt<2>(codes, scales, n, k, x, m, y, out_f32, st);
}

}  // namespace lowbit
