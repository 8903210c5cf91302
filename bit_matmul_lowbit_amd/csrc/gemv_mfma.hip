// Decode GEMV on matrix cores for batch 3..8:
//   y[i][n] = sum_g s[n][g] * sum_{k in g} t[n][k] * x[i][k]
//
// [P2] 7minutos.es, "PrismML lanza Bonsai 27B ...": decode is bound by memory
//      bandwidth ("Rendimiento y decodificacion especulativa DSpark"); speculative
//      decoding verifies several drafted tokens per step, so the same weights
//      meet a small batch of activation rows.
// [P1] 7minutos.es tutorial, section 7: bit 0 -> -s, bit 1 -> +s.
//
// With b > 1 the subset-sum tables of the b = 1 kernel grow with b, and so
// does their lookup traffic.  Here the weights are instead expanded in
// registers to FP16 values +s, -s (or 0 for ternary) -- exact, since s is an
// FP16 number -- and contracted with x on v_mfma_f32_16x16x32_f16, the batch
// padded to the instruction's 16 rows.  Products x * (+-s) are exact in FP32
// and are summed in FP32, as in the table kernel.
//
// MFMA operand mapping (16x16x32, f16):
//   A (16 x 32): lane l holds x[l % 16][8 (l / 16) .. +7]   (batch row, 8 k)
//   B (32 x 16): lane l holds w[8 (l / 16) .. +7][l % 16]   (8 k, one column)
//   D (16 x 16): lane l, register v holds D[4 (l / 16) + v][l % 16]
// Column l % 16 of B is row rho of tile T0 + l % 16: every lane reads whole
// 16-byte code cells (16 rows x 8 k) of its own tile, and byte rho of a cell
// feeds the MFMA of row rho, so one step issues 16 independent MFMAs
// (rho = 0..15) that share the A operand.  Step j of a 128-weight group
// takes chunks 4j .. 4j + 3, lane quarter q = l / 16 chunk 4j + q (the x
// operands are laid out to match), so the four lanes of a tile read 64
// contiguous bytes (Q1; 128 for T2) per load.
//
// Expansion of a Q1 byte e (bit j <-> k0 + j) into four FP16 pairs: with e
// in the low byte of both 16-bit halves, a packed 16-bit shift by
// (15 - 2p, 14 - 2p) brings bits 2p and 2p + 1 to bits 15 and 31, and
// v_bitop3 picks +s or -s (which differ only in those sign bits): two
// VALU operations per FP16 pair.  Ternary bytes are shifted straight from
// their code words (the packed shift reads the half that holds the byte in
// both halves, op_sel), with no byte moves.  A ternary pair also needs the mask of
// (pos xor neg), so a cell with both bits set is 0, as pos - neg is, and a
// zero weight contributes an exact 0 (five operations per pair).
// The 1-bit persistent kernel replaces this expansion with an LDS table
// lookup of +-1 patterns and applies the scale once per group (see
// group_mfma_lut below); the item kernel and ternary codes keep it.
//
// Work: an item is (16-tile block, K-piece).  The grid is persistent (two
// work-groups per CU); work-group w takes items w, w + W, ... in order, so
// all work-groups sweep the matrix together and the loads in flight at any
// time cover one contiguous stretch of it.  Inside an item the 4 waves
// take its groups round-robin; their load rings run on across items, and
// at the end of an item the waves sum their partials through LDS and add
// them to y with one coalesced FP32 atomic per (row, batch row).  A matrix
// with no more items than CUs runs one work-group per item instead.  Only
// lanes of batch rows < b load x (the others read past their resource,
// which returns zeros with no memory traffic).
#include "common.h"

namespace lowbit {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kSteps = 4;            // 32-k MFMA steps per 128-weight group
constexpr int kXStep = 64 * 16;      // bytes of A operand per step (64 lanes x 16 B)
constexpr int kRedPitch = 260;       // LDS pitch per batch row (256 rows + pad)

// Persistent kernel's item-end buffer: float4 (batch rows 4q .. 4q + 3) of
// wave w, lane quarter q < 2, row rho of tile `tile` of the item's block.
// The 16 tiles of one (w, q, rho) are contiguous (a wave's 16-byte stores
// fill 256 contiguous bytes per quarter), and rows rho are 68 floats apart
// (272 bytes, 16 mod 256), so the 16 rows read by a 16-lane phase of the
// summing threads fall in different 16-byte bank groups.
constexpr int kRedRowF4 = 17;  // float4 per (w, q, rho): 16 tiles + pad
constexpr int kRedFloats = kWaves * 2 * 16 * kRedRowF4 * 4;
__device__ __forceinline__ int red_at(int w, int q, int rho, int tile) {
  return ((w * 2 + q) * 16 + rho) * kRedRowF4 + tile;
}
constexpr uint32_t kNoLoad = 0x80000000u;  // lane offset past any resource: zeros

// byte offset of a lane's code cell i of a group, from the lane's quarter base
template <int FMT>
constexpr int cell_off(int i) {
  return FMT == 1 ? 64 * i : 128 * (i >> 1) + 16 * (i & 1);
}


template <int SOFF = 0>
__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff + SOFF, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// per-half arithmetic shift right by 15: 0xFFFF where bit 15 is set, else 0
__device__ __forceinline__ uint32_t pk_mask15(uint32_t d) {
  const s16x2 a = __builtin_bit_cast(s16x2, d);
  return __builtin_bit_cast(uint32_t, (s16x2)(a >> (s16x2){15, 15}));
}

// Q1: bit set -> +s, clear -> -s;  d = the code byte in the low byte of
// both halves, ss = s in both halves.  (Shifting the code word's half
// straight from the word, as the ternary expansion below does, issues one
// instruction fewer per row but measured 2 % slower on the 1-bit 27B
// matrices.)
__device__ __forceinline__ f16x8 expand_q1(uint32_t d, uint32_t ss) {
  u32x4 v;
  v[0] = ss ^ (~pk_shl(d, kPairShift<0>) & kSignBits);
  v[1] = ss ^ (~pk_shl(d, kPairShift<1>) & kSignBits);
  v[2] = ss ^ (~pk_shl(d, kPairShift<2>) & kSignBits);
  v[3] = ss ^ (~pk_shl(d, kPairShift<3>) & kSignBits);
  return __builtin_bit_cast(f16x8, v);
}

// T2, byte J of dn = pos xor neg (nonzero) and of dq = neg (sign);  -> +s,
// -s or 0
template <int J>
__device__ __forceinline__ f16x8 expand_t2(uint32_t dn, uint32_t dq, uint32_t ss) {
  u32x4 v;
#define LOWBIT_PAIR(P)                                                                   \
  v[P] = (ss ^ (byte_pair_bits<J, P>(dq) & kSignBits)) & pk_mask15(byte_pair_bits<J, P>(dn));
  LOWBIT_PAIR(0)
  LOWBIT_PAIR(1)
  LOWBIT_PAIR(2)
  LOWBIT_PAIR(3)
#undef LOWBIT_PAIR
  return __builtin_bit_cast(f16x8, v);
}

template <int FMT>
struct GroupRegs {
  static constexpr int kCells = FMT == 1 ? 4 : 8;  // 16-B cells per lane per group
  uint4 c[kCells];  // Q1: chunks 4q..4q+3; T2: (pos, neg) of each
  uint4 s[2];       // FP16 scales of the tile's 16 rows for this group
  uint4 x[kSteps];  // A operands of the group's four steps
};

// x operands: from the prepared workspace (vector (g, j, lane) at
// ((g * kSteps + j) * 64 + lane) * 16 bytes), or with XD from x itself
// (FP16 [b][k]: the lane's batch row and chunk 16 g + 4 j + q, i.e. the
// lane offset row * 2k + 16 q plus 256 g + 64 j)
template <int FMT, bool XD = false>
__device__ __forceinline__ void load_group(GroupRegs<FMT>& r, __amdgpu_buffer_rsrc_t rc,
                                           __amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rx,
                                           uint32_t voff_c, uint32_t voff_s, uint32_t voff_x,
                                           int g) {
  constexpr int GB = FMT == 1 ? 256 : 512;  // code bytes per tile per group
  const int sc = g * GB;
#pragma unroll
  for (int i = 0; i < GroupRegs<FMT>::kCells; ++i)
    r.c[i] = bload(rc, voff_c, sc + cell_off<FMT>(i));
  r.s[0] = bload<0>(rs, voff_s, g * 32);
  r.s[1] = bload<16>(rs, voff_s, g * 32);
#pragma unroll
  for (int j = 0; j < kSteps; ++j)
    r.x[j] = bload(rx, voff_x, XD ? g * 256 + j * 64 : (g * kSteps + j) * kXStep);
}

// the scale of row rho in both halves
template <int RHO>
__device__ __forceinline__ uint32_t scale_pair(const uint4 (&s)[2]) {
  const uint32_t w[8] = {s[0].x, s[0].y, s[0].z, s[0].w, s[1].x, s[1].y, s[1].z, s[1].w};
  constexpr uint32_t lo = (RHO & 1) * 2, hi = lo + 1;
  return __builtin_amdgcn_perm(w[RHO >> 1], w[RHO >> 1], (hi << 24) | (lo << 16) | (hi << 8) | lo);
}

template <int FMT>
__device__ __forceinline__ void group_mfma(const GroupRegs<FMT>& r, f32x4 (&acc)[16]) {
  uint32_t ss[16];
#define LOWBIT_SS(R) ss[R] = scale_pair<R>(r.s);
  LOWBIT_SS(0) LOWBIT_SS(1) LOWBIT_SS(2) LOWBIT_SS(3) LOWBIT_SS(4) LOWBIT_SS(5) LOWBIT_SS(6)
  LOWBIT_SS(7) LOWBIT_SS(8) LOWBIT_SS(9) LOWBIT_SS(10) LOWBIT_SS(11) LOWBIT_SS(12)
  LOWBIT_SS(13) LOWBIT_SS(14) LOWBIT_SS(15)
#undef LOWBIT_SS
#pragma unroll
  for (int j = 0; j < kSteps; ++j) {
    const f16x8 a = __builtin_bit_cast(f16x8, r.x[j]);
    if constexpr (FMT == 1) {
      const uint32_t cw[4] = {r.c[j].x, r.c[j].y, r.c[j].z, r.c[j].w};
#define LOWBIT_ROW(RHO)                                                                    \
  acc[RHO] = __builtin_amdgcn_mfma_f32_16x16x32_f16(                                       \
      a, expand_q1(rep_byte<(RHO) & 3>(cw[(RHO) >> 2]), ss[RHO]), acc[RHO], 0, 0, 0);
      LOWBIT_ROW(0) LOWBIT_ROW(1) LOWBIT_ROW(2) LOWBIT_ROW(3) LOWBIT_ROW(4) LOWBIT_ROW(5)
      LOWBIT_ROW(6) LOWBIT_ROW(7) LOWBIT_ROW(8) LOWBIT_ROW(9) LOWBIT_ROW(10) LOWBIT_ROW(11)
      LOWBIT_ROW(12) LOWBIT_ROW(13) LOWBIT_ROW(14) LOWBIT_ROW(15)
#undef LOWBIT_ROW
    } else {
      const uint4 p = r.c[2 * j], q = r.c[2 * j + 1];
      const uint32_t nw[4] = {p.x ^ q.x, p.y ^ q.y, p.z ^ q.z, p.w ^ q.w};
      const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
#define LOWBIT_ROW(RHO)                                                                    \
  acc[RHO] = __builtin_amdgcn_mfma_f32_16x16x32_f16(                                       \
      a,                                                                                   \
      expand_t2<(RHO) & 3>(nw[(RHO) >> 2], qw[(RHO) >> 2], ss[RHO]),                       \
      acc[RHO], 0, 0, 0);
      LOWBIT_ROW(0) LOWBIT_ROW(1) LOWBIT_ROW(2) LOWBIT_ROW(3) LOWBIT_ROW(4) LOWBIT_ROW(5)
      LOWBIT_ROW(6) LOWBIT_ROW(7) LOWBIT_ROW(8) LOWBIT_ROW(9) LOWBIT_ROW(10) LOWBIT_ROW(11)
      LOWBIT_ROW(12) LOWBIT_ROW(13) LOWBIT_ROW(14) LOWBIT_ROW(15)
#undef LOWBIT_ROW
    }
  }
}

// 1-bit codes: the expansion as an LDS lookup.  Code byte e of a cell (8 k
// of one row) selects a 16-byte entry of eight FP16 values +-1 (element i
// is +1 where bit i of e is set, -1 where it is clear); the four MFMAs of a
// 128-weight group sum +-x unscaled, and the row's FP16 scale multiplies the
// group's sums once (one v_fma_mix_f32 per accumulator element per group).
// Per row step that is a v_perm_b32 and a shift (the entry's address) and
// one ds_read_b128 in place of the eight VALU operations of expand_q1, and
// the lookups of the next two rows go out before the MFMAs of the current
// two.  The table holds 8 copies of its 256 entries, copy c of entry e at
// byte 128 e + 16 c, lane l reading copy l % 8 (32 KB: with the single
// item-end buffer the 1-bit kernel keeps, two work-groups still fit a CU).
// On register data (a probe, two waves per SIMD) a row step takes 14.3 ns
// this way against 20.5 ns with expand_q1 (16 copies: 10.9 ns, but 64 KB).
constexpr int kLutCopies = 8;
constexpr int kLutU4 = 256 * kLutCopies;  // 16-byte entries

// entry for byte J of w in this lane's copy: [lb.b0, w.bJ, 0, 0] >> 1 with
// lb = 32 (lane % 8), i.e. (byte << 7) | 16 (lane % 8)
template <int J>
__device__ __forceinline__ uint32_t lut_addr(uint32_t w, uint32_t lb) {
  return __builtin_amdgcn_perm(w, lb, 0x0C0C0000u | ((4u + J) << 8)) >> 1;
}

// the group's scale of row RHO of the lane's tile, as FP32
template <int RHO>
__device__ __forceinline__ float row_scale(const uint4 (&s)[2]) {
  const uint32_t w[8] = {s[0].x, s[0].y, s[0].z, s[0].w, s[1].x, s[1].y, s[1].z, s[1].w};
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w[RHO >> 1] >> (16 * (RHO & 1))));
}

// lookups of rows 2P and 2P + 1, steps 0..3: t[j] row 2P, t[4 + j] row 2P + 1
template <int P>
__device__ __forceinline__ void lut_pair(const GroupRegs<1>& r, const char* tb, uint32_t lb,
                                         uint4 (&t)[8]) {
  if constexpr (P < 8) {
    constexpr int R0 = 2 * P, R1 = 2 * P + 1;
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
      const uint32_t cw[4] = {r.c[j].x, r.c[j].y, r.c[j].z, r.c[j].w};
      t[j] = *reinterpret_cast<const uint4*>(tb + lut_addr<R0 & 3>(cw[R0 >> 2], lb));
      t[4 + j] = *reinterpret_cast<const uint4*>(tb + lut_addr<R1 & 3>(cw[R1 >> 2], lb));
    }
  }
}

template <int P>
__device__ __forceinline__ void lut_pair_mfma(const GroupRegs<1>& r, const uint4 (&t)[8],
                                              f32x4 (&acc)[16]) {
  constexpr int R0 = 2 * P, R1 = 2 * P + 1;
  f32x4 g0 = (f32x4){0.f, 0.f, 0.f, 0.f}, g1 = g0;
#pragma unroll
  for (int j = 0; j < kSteps; ++j) {
    const f16x8 a = __builtin_bit_cast(f16x8, r.x[j]);
    g0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(f16x8, t[j]), g0, 0, 0, 0);
    g1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(f16x8, t[4 + j]), g1, 0, 0,
                                                0);
  }
  const float s0 = row_scale<R0>(r.s), s1 = row_scale<R1>(r.s);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    acc[R0][v] = __builtin_fmaf(s0, g0[v], acc[R0][v]);
    acc[R1][v] = __builtin_fmaf(s1, g1[v], acc[R1][v]);
  }
}

// the table: entry index 8 e + copy, filled by `threads` threads
__device__ __forceinline__ void lut_fill(uint4* lut, int tid, int threads) {
  for (int i = tid; i < kLutU4; i += threads) {
    const uint32_t e = (uint32_t)i / kLutCopies;
    uint32_t d[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
      d[p] = (((e >> (2 * p)) & 1u) ? 0x3C00u : 0xBC00u) |
             ((((e >> (2 * p + 1)) & 1u) ? 0x3C00u : 0xBC00u) << 16);
    lut[i] = make_uint4(d[0], d[1], d[2], d[3]);
  }
}

__device__ __forceinline__ void group_mfma_lut(const GroupRegs<1>& r, f32x4 (&acc)[16],
                                               const char* tb, uint32_t lb) {
  uint4 t[2][8];
  lut_pair<0>(r, tb, lb, t[0]);
#define LOWBIT_PAIR(P)                            \
  lut_pair<(P) + 1>(r, tb, lb, t[((P) + 1) & 1]); \
  __builtin_amdgcn_sched_barrier(0);              \
  lut_pair_mfma<P>(r, t[(P) & 1], acc);           \
  __builtin_amdgcn_sched_barrier(0);
  LOWBIT_PAIR(0) LOWBIT_PAIR(1) LOWBIT_PAIR(2) LOWBIT_PAIR(3)
  LOWBIT_PAIR(4) LOWBIT_PAIR(5) LOWBIT_PAIR(6) LOWBIT_PAIR(7)
#undef LOWBIT_PAIR
}

// prepare: x -> A operands in step order (zeros for batch rows >= b), y = 0
__global__ __launch_bounds__(256) void gemv_mfma_prepare_kernel(const uint16_t* __restrict__ x,
                                                                int64_t k, int b,
                                                                uint4* __restrict__ xw,
                                                                int64_t nvec,
                                                                float* __restrict__ y,
                                                                int64_t ycount) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * 256;
  zero_f32(y, ycount, gid, stride);
  for (int64_t i = gid; i < nvec; i += stride) {
    // vector i = (group g, step j, lane l): batch row l % 16, chunk 16 g + 4 j + l / 16
    const int l = (int)(i & 63);
    const int64_t gj = i >> 6;
    const int64_t g = gj / kSteps;
    const int j = (int)(gj % kSteps);
    const int row = l & 15;
    const int64_t chunk = g * 16 + 4 * j + (l >> 4);
    xw[i] = row < b ? *reinterpret_cast<const uint4*>(x + row * k + chunk * kChunk)
                    : make_uint4(0u, 0u, 0u, 0u);
  }
}

// XD (the decode FFN's gate+up GEMV): x is read as given (FP16 [b][k], no
// prepare launch) and each item stores its K-piece's sums into plane
// `piece` of y (FP32 [kpieces][b][n]) instead of adding them up, so y
// needs no zeroing.
template <int FMT, bool XD = false>
__global__ __launch_bounds__(kThreads, 2) void gemv_mfma_kernel(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint4* __restrict__ xw, float* __restrict__ y, int64_t n, int64_t k, int b,
    int64_t ntiles, int kpieces, int gpp, int64_t nitems) {
  // Item-end reduction buffers.  Ternary: two, so that one barrier per
  // item suffices (the next item writes the other buffer; a wave can only
  // reach the item after that once every wave has passed the next barrier,
  // i.e. finished reading this one).  1-bit: the expansion table (at LDS
  // address 0, where an entry's address needs no add) and one buffer, with
  // a second barrier once the buffer has been read.
  constexpr int kRedBufs = FMT == 1 ? 1 : 2;
  constexpr int kTabU4 = FMT == 1 ? kLutU4 : 0;
  __shared__ uint4 smem[kTabU4 + kRedBufs * kRedFloats / 4];
  float4* red4 = reinterpret_cast<float4*>(smem + kTabU4);
  constexpr int D = 2;  // groups of loads in flight per wave, plus the one in use
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = (int)(k / kGroup);
  const int tl = lane & 15, q = lane >> 4;
  const int64_t cpitch = (k / kChunk) * Fmt<FMT>::cell_bytes;
  const int64_t spitch = (int64_t)G * kTileRows * 2;
  const uint32_t voff_c = (uint32_t)(tl * cpitch + q * Fmt<FMT>::cell_bytes);
  const uint32_t voff_s = (uint32_t)(tl * spitch);
  const uint32_t voff_x =
      tl < b ? (XD ? (uint32_t)(tl * k * 2 + q * 16) : (uint32_t)(lane * 16)) : kNoLoad;
  const __amdgpu_buffer_rsrc_t rx =
      buffer_rsrc(xw, XD ? (int64_t)b * k * 2 : (int64_t)G * kSteps * kXStep);
  const __amdgpu_buffer_rsrc_t rz = buffer_rsrc(xw, 0);  // all loads return zero

  // This work-group's items: blockIdx.x + i * gridDim.x.  Every wave runs
  // `per` group slots per item (slot i of an item is group
  // piece * gpp + wave + 4 i); a slot past the item's groups, or past the
  // last item, is loaded from a zero-length resource (codes, scales and x
  // read as zeros, with no memory traffic) and adds exact zeros.
  const int per = (gpp + kWaves - 1) / kWaves;
  const int64_t nit = nitems > (int64_t)blockIdx.x
                          ? (nitems - blockIdx.x + gridDim.x - 1) / gridDim.x : 0;
  const int64_t total = nit * per;
  auto load = [&](GroupRegs<FMT>& r, int64_t sl) {
    const int64_t it = sl / per;
    const int i = (int)(sl - it * per);
    const int64_t item = blockIdx.x + (it < nit ? it : 0) * (int64_t)gridDim.x;
    const int64_t T0 = (item / kpieces) * 16;
    const int piece = (int)(item % kpieces);
    const int g = piece * gpp + wave + kWaves * i;
    const int gend = piece * gpp + gpp < G ? piece * gpp + gpp : G;
    const bool live = sl < total && g < gend;
    const int64_t here = ntiles - T0 < 16 ? ntiles - T0 : 16;
    // lanes whose tile is past the end read past their resource: zeros
    const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(codes + T0 * cpitch, here * cpitch);
    const __amdgpu_buffer_rsrc_t rs =
        buffer_rsrc(reinterpret_cast<const uint8_t*>(scales) + T0 * spitch, here * spitch);
    load_group<FMT, XD>(r, live ? rc : rz, live ? rs : rz, live ? rx : rz, voff_c, voff_s,
                        voff_x, live ? g : 0);
  };

  f32x4 acc[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = (f32x4){0.f, 0.f, 0.f, 0.f};
  GroupRegs<FMT> ring[D];
#pragma unroll
  for (int i = 0; i < D - 1; ++i) load(ring[i], i);
  const char* tb = reinterpret_cast<const char*>(smem);
  const uint32_t lb = (uint32_t)(lane & (kLutCopies - 1)) << 5;
  if constexpr (FMT == 1) {
    // the table, while the first loads are in flight
    lut_fill(smem, threadIdx.x, kThreads);
    // LDS only: the loads above stay in flight
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lds(63));
    stage_barrier();
  }
  int rb = 0;  // reduction buffer of the next item end
  for (int64_t sl = 0; sl < total; sl += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      // the next group's loads go out before this group's MFMAs (the
      // scheduler would otherwise sink them into the MFMA sequence)
      load(ring[(u + D - 1) % D], sl + u + D - 1);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (FMT == 1)
        group_mfma_lut(ring[u], acc, tb, lb);
      else
        group_mfma<FMT>(ring[u], acc);
      __builtin_amdgcn_sched_barrier(0);
      const int64_t cur = sl + u;
      if (cur < total && (cur + 1) % per == 0) {
        // end of an item: partial sums of the waves -> LDS -> y.  Batch
        // rows 0..7 (b <= 8) sit in lanes q = 0, 1: each writes its 4 rows
        // of acc[r] as one 16-byte store, red_at(w, q, r, tile) + v
        const int64_t item = blockIdx.x + (cur / per) * (int64_t)gridDim.x;
        const int64_t T0 = (item / kpieces) * 16;
        float4* red = red4 + rb * (kRedFloats / 4);
        if (q < 2) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            red[red_at(wave, q, r, tl)] = make_float4(acc[r][0], acc[r][1], acc[r][2], acc[r][3]);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = (f32x4){0.f, 0.f, 0.f, 0.f};
        __syncthreads();
        // thread t: row T0 * 16 + t (t = 16 * tile + rho), batch rows 0..7
        const int t = threadIdx.x;
        const int64_t row = T0 * 16 + t;
        float4 s0 = make_float4(0.f, 0.f, 0.f, 0.f), s1 = s0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float4 a = red[red_at(w, 0, t & 15, t >> 4)], c = red[red_at(w, 1, t & 15, t >> 4)];
          s0.x += a.x; s0.y += a.y; s0.z += a.z; s0.w += a.w;
          s1.x += c.x; s1.y += c.y; s1.z += c.z; s1.w += c.w;
        }
        if (row < n) {
          const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
          const int64_t pb = XD ? (item % kpieces) * b : 0;  // plane of this K-piece
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            if (i < b) {
              if constexpr (XD)
                y[(pb + i) * n + row] = sv[i];
              else
                atomicAdd(y + i * n + row, sv[i]);
            }
          }
        }
        if constexpr (kRedBufs == 1) {
          // every wave has read the buffer before any writes it again
          __builtin_amdgcn_s_waitcnt(waitcnt_vm_lds(63));
          stage_barrier();
        } else {
          rb ^= 1;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// One item per work-group, for matrices with no more items than CUs: the
// item's x operands are staged in LDS once and read from there at each
// step, so x is read from memory once per work-group instead of once per
// wave and group, and a wave's registers hold codes and scales only (32
// fewer than the persistent kernel).  After the groups, the x buffer holds
// the waves' partial sums (8 batch rows: b <= 8).
constexpr int kItemMaxGroups = 8;
constexpr int kItemXBytes = kItemMaxGroups * kSteps * kXStep;
constexpr int kItemRedBytes = kWaves * 8 * kRedPitch * 4;
constexpr int kItemLds = kItemXBytes > kItemRedBytes ? kItemXBytes : kItemRedBytes;

template <int FMT>
struct CodeRegs {
  uint4 c[GroupRegs<FMT>::kCells];
  uint4 s[2];
};

// XD as for gemv_mfma_kernel: x as given, K-piece sums stored into planes
template <int FMT, bool XD = false>
__global__ __launch_bounds__(kThreads, FMT == 1 ? 3 : 2) void gemv_mfma_item_kernel(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint4* __restrict__ xw, float* __restrict__ y, int64_t n, int64_t k, int b,
    int64_t ntiles, int kpieces, int gpp) {
  __shared__ uint4 lds[kItemLds / 16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = (int)(k / kGroup);
  const int tl = lane & 15, q = lane >> 4;
  const int64_t cpitch = (k / kChunk) * Fmt<FMT>::cell_bytes;
  const int64_t spitch = (int64_t)G * kTileRows * 2;
  constexpr int GB = FMT == 1 ? 256 : 512;
  const uint32_t voff_c = (uint32_t)(tl * cpitch + q * Fmt<FMT>::cell_bytes);
  const uint32_t voff_s = (uint32_t)(tl * spitch);

  const int64_t item = blockIdx.x;
  const int64_t T0 = (item / kpieces) * 16;
  const int g0 = (int)(item % kpieces) * gpp;
  const int ng = g0 + gpp < G ? gpp : G - g0;  // groups of this item
  const int64_t here = ntiles - T0 < 16 ? ntiles - T0 : 16;
  // lanes whose tile is past the end read past their resource: zeros
  const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(codes + T0 * cpitch, here * cpitch);
  const __amdgpu_buffer_rsrc_t rs =
      buffer_rsrc(reinterpret_cast<const uint8_t*>(scales) + T0 * spitch, here * spitch);
  const __amdgpu_buffer_rsrc_t rz = buffer_rsrc(codes, 0);

  // the wave's groups g0 + wave + 4 i (i < 2), loaded first; a group past
  // the item reads zeros and adds exact zeros
  CodeRegs<FMT> cr[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int gl = wave + kWaves * i;
    const bool live = gl < ng;
    const int g = live ? g0 + gl : 0;
    constexpr int kCells = GroupRegs<FMT>::kCells;
#pragma unroll
    for (int c = 0; c < kCells; ++c)
      cr[i].c[c] = bload(live ? rc : rz, voff_c, g * GB + cell_off<FMT>(c));
    cr[i].s[0] = bload<0>(live ? rs : rz, voff_s, g * 32);
    cr[i].s[1] = bload<16>(live ? rs : rz, voff_s, g * 32);
  }
  // the item's x operands into LDS: vector (group gl, step j, lane l) at
  // (gl * kSteps + j) * 64 + l
  for (int i = threadIdx.x; i < ng * kSteps * 64; i += kThreads) {
    if constexpr (XD) {
      // batch row l % 16, chunk 16 (g0 + gl) + 4 j + l / 16 of x [b][k]
      const int l = i & 63, gl = i / (kSteps * 64), j = (i >> 6) % kSteps;
      const int64_t chunk = (int64_t)(g0 + gl) * 16 + 4 * j + (l >> 4);
      lds[i] = (l & 15) < b ? xw[((int64_t)(l & 15) * k + chunk * kChunk) / 8]
                            : make_uint4(0u, 0u, 0u, 0u);
    } else {
      lds[i] = (i & 15) < b ? xw[(int64_t)g0 * kSteps * 64 + i] : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __syncthreads();

  f32x4 acc[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int gl = wave + kWaves * i;
    if (i * kWaves >= gpp) break;  // gpp <= 4: one group per wave
    GroupRegs<FMT> r;
#pragma unroll
    for (int c = 0; c < GroupRegs<FMT>::kCells; ++c) r.c[c] = cr[i].c[c];
    r.s[0] = cr[i].s[0];
    r.s[1] = cr[i].s[1];
    // x from LDS (zeros past the item: the codes of such a group are zero
    // too, and Q1 zero codes expand to -s, so x must be zero there)
#pragma unroll
    for (int j = 0; j < kSteps; ++j)
      r.x[j] = gl < ng ? lds[(gl * kSteps + j) * 64 + lane] : make_uint4(0u, 0u, 0u, 0u);
    group_mfma<FMT>(r, acc);
  }

  // partial sums of the waves -> LDS (batch rows 0..7) -> one atomic per
  // (row, batch row)
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);
  if (q < 2) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[(wave * 8 + 4 * q + v) * kRedPitch + r * 16 + tl] = acc[r][v];
  }
  __syncthreads();
  // thread t: row T0 * 16 + t (t = 16 * tile + rho)
  const int t = threadIdx.x;
  const int64_t row = T0 * 16 + t;
  const int rr = (t & 15) * 16 + (t >> 4);
  if (row < n) {
    const int64_t pb = XD ? (item % kpieces) * b : 0;  // plane of this K-piece
    for (int i = 0; i < b; ++i) {
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) sum += red[(w * 8 + i) * kRedPitch + rr];
      if constexpr (XD)
        y[(pb + i) * n + row] = sum;
      else
        atomicAdd(y + i * n + row, sum);
    }
  }
}

// ---------------------------------------------------------------------------
// Ceiling probe (lowbit_probe_expand_mfma): the per-row work of group_mfma
// -- rep_byte + expand_q1 of one code byte into +-s FP16 operands, and one
// v_mfma_f32_16x16x32_f16 -- on register data, 16 rows per iteration, the
// code words changed every iteration.  MODE 0: expansion + MFMA as the
// ternary and small-matrix kernels run it, 1: the MFMA alone on fixed
// operands, 2: group_mfma_lut (the 1-bit persistent kernel's lookups, MFMAs
// and per-group scale FMAs) on register codes, one 128-weight group (64 row
// steps) per four iterations.
template <int MODE>
__global__ __launch_bounds__(kThreads) void probe_expand_mfma_kernel(int iters,
                                                                     float* __restrict__ sink) {
  const uint32_t l = threadIdx.x & 63;
  uint32_t cw[4] = {0x9E3779B9u * (l + 1), 0x85EBCA6Bu * (l + 3), 0xC2B2AE35u * (l + 5),
                    0x27D4EB2Fu * (l + 7)};
  const uint32_t ss = 0x3C003C00u ^ (l << 3);  // a positive FP16 scale in both halves
  const f16x8 a = __builtin_bit_cast(f16x8, (u32x4){ss, ss ^ 1u, ss ^ 2u, ss ^ 3u});
  f32x4 acc[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = (f32x4){0.f, 0.f, 0.f, 0.f};
  if constexpr (MODE == 2) {
    __shared__ uint4 lut[kLutU4];
    lut_fill(lut, threadIdx.x, kThreads);
    __syncthreads();
    GroupRegs<1> r;
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
      r.c[j] = make_uint4(cw[0] + j, cw[1] ^ j, cw[2] + 3 * j, cw[3] ^ (5 * j));
      r.x[j] = __builtin_bit_cast(uint4, a);
    }
    r.s[0] = make_uint4(ss, ss, ss, ss);
    r.s[1] = r.s[0];
    const char* tb = reinterpret_cast<const char*>(lut);
    const uint32_t lb = (l & (kLutCopies - 1)) << 5;
    for (int it = 0; it < iters; it += 4) {
      group_mfma_lut(r, acc, tb, lb);
#pragma unroll
      for (int j = 0; j < kSteps; ++j) {
        r.c[j].x += 0x01010101u;
        r.c[j].y += 0x01010101u;
        r.c[j].z += 0x01010101u;
        r.c[j].w += 0x01010101u;
      }
    }
  }
  for (int it = 0; it < (MODE == 2 ? 0 : iters); ++it) {
#define LOWBIT_PROBE_ROW(R)                                                                   \
  {                                                                                           \
    const f16x8 bb = MODE == 1 ? a : expand_q1(rep_byte<(R) & 3>(cw[(R) >> 2]), ss);          \
    acc[R] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bb, acc[R], 0, 0, 0);                  \
  }
    LOWBIT_PROBE_ROW(0) LOWBIT_PROBE_ROW(1) LOWBIT_PROBE_ROW(2) LOWBIT_PROBE_ROW(3)
    LOWBIT_PROBE_ROW(4) LOWBIT_PROBE_ROW(5) LOWBIT_PROBE_ROW(6) LOWBIT_PROBE_ROW(7)
    LOWBIT_PROBE_ROW(8) LOWBIT_PROBE_ROW(9) LOWBIT_PROBE_ROW(10) LOWBIT_PROBE_ROW(11)
    LOWBIT_PROBE_ROW(12) LOWBIT_PROBE_ROW(13) LOWBIT_PROBE_ROW(14) LOWBIT_PROBE_ROW(15)
#undef LOWBIT_PROBE_ROW
#pragma unroll
    for (int j = 0; j < 4; ++j) cw[j] += 0x01010101u;
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += acc[r][0] + acc[r][1] + acc[r][2] + acc[r][3];
  if (__builtin_bit_cast(uint32_t, s) == 0x9E3779B9u) sink[blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_probe_expand_mfma(int mode, int iters, int blocks, float* sink, hipStream_t st) {
  if (mode == 0)
    hipLaunchKernelGGL(probe_expand_mfma_kernel<0>, dim3(blocks), dim3(kThreads), 0, st, iters, sink);
  else if (mode == 2)
    hipLaunchKernelGGL(probe_expand_mfma_kernel<2>, dim3(blocks), dim3(kThreads), 0, st, iters, sink);
  else
    hipLaunchKernelGGL(probe_expand_mfma_kernel<1>, dim3(blocks), dim3(kThreads), 0, st, iters, sink);
  return hipGetLastError();
}

int64_t gemv_mfma_workspace_bytes(int64_t k) { return (k / kGroup) * kSteps * kXStep; }

hipError_t launch_gemv_mfma_prepare(int64_t n, int64_t k, const uint16_t* x, int64_t b, float* y,
                                    void* ws, hipStream_t st) {
  const int64_t nvec = (k / kGroup) * kSteps * 64;
  const int64_t yvec = (n * b + 3) / 4;
  const int64_t work = nvec > yvec ? nvec : yvec;
  int64_t blocks = (work + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(gemv_mfma_prepare_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, k,
                     (int)b, static_cast<uint4*>(ws), nvec, y, n * b);
  return hipGetLastError();
}

namespace {

// Work split of the matrix-core GEMV.  Persistent grid of up to two
// work-groups per CU.  An item's K-piece is 4 * per groups (per groups for
// each wave): per is chosen for about four items per work-group, but at
// least two groups per wave (each item ends with an LDS reduction and
// atomics) and no more than K holds.  The grid is two work-groups per CU
// (fewer only if there are fewer items), all resident at once, so a
// work-group with a second item has its loads in flight while it finishes
// the first; one work-group per item, with the items past the resident ones
// launched as a second round, ran the 27B gate+up (680 items) at b = 5 / 8
// in 15.0-15.5 / 15.5-16.0 us instead of 14.3 / 14.7 us.  A matrix whose
// two-group items would not even give every CU one takes a single group per
// wave (twice the items): 6144x2048 ternary at b = 3..8 runs 12.2 -> 11.1
// us, while larger matrices lose with it (27B gate+up at b = 5: 19 us).
struct MfmaPlan {
  int64_t ntiles, kp, nitems, nwg;
  int gpp;
  bool item;  // one item per work-group (gemv_mfma_item_kernel)
};

MfmaPlan mfma_plan(int64_t n, int64_t k, int cus) {
  MfmaPlan p;
  p.ntiles = (n + kTileRows - 1) / kTileRows;
  const int64_t nblocks = (p.ntiles + 15) / 16;
  const int G = (int)(k / kGroup);
  const int64_t nwg_max = 2 * (int64_t)cus;
  int64_t per = (int64_t)G * nblocks / (4 * kWaves * nwg_max);
  const int64_t per_max = (G + kWaves - 1) / kWaves;
  if (per < 2) per = nblocks * ((G + 2 * kWaves - 1) / (2 * kWaves)) < cus ? 1 : 2;
  if (per > per_max) per = per_max;
  p.gpp = (int)(kWaves * per);
  p.kp = (G + p.gpp - 1) / p.gpp;
  p.nitems = nblocks * p.kp;
  p.nwg = p.nitems < nwg_max ? p.nitems : nwg_max;
  // no more items than CUs: one item per work-group, x from LDS (ternary
  // 6144x2048 and 2048x6144 at b = 5: 11.1 -> 9.0 us; the 27B-class
  // matrices, 340 and 680 items, ran 12-15 % slower this way than with the
  // persistent kernel and stay on it)
  p.item = p.gpp <= kItemMaxGroups && p.nitems <= (int64_t)cus;
  return p;
}

template <bool XD>
hipError_t launch_plan(const MfmaPlan& p, int fmt, const uint8_t* codes, const uint16_t* scales,
                       int64_t n, int64_t k, int64_t b, float* y, const uint4* xin,
                       hipStream_t st) {
  if (p.item) {
    const dim3 igrid((unsigned)p.nitems);
    if (fmt == 1)
      hipLaunchKernelGGL((gemv_mfma_item_kernel<1, XD>), igrid, dim3(kThreads), 0, st, codes,
                         scales, xin, y, n, k, (int)b, p.ntiles, (int)p.kp, p.gpp);
    else
      hipLaunchKernelGGL((gemv_mfma_item_kernel<2, XD>), igrid, dim3(kThreads), 0, st, codes,
                         scales, xin, y, n, k, (int)b, p.ntiles, (int)p.kp, p.gpp);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)p.nwg);
  if (fmt == 1)
    hipLaunchKernelGGL((gemv_mfma_kernel<1, XD>), grid, dim3(kThreads), 0, st, codes, scales, xin,
                       y, n, k, (int)b, p.ntiles, (int)p.kp, p.gpp, p.nitems);
  else
    hipLaunchKernelGGL((gemv_mfma_kernel<2, XD>), grid, dim3(kThreads), 0, st, codes, scales, xin,
                       y, n, k, (int)b, p.ntiles, (int)p.kp, p.gpp, p.nitems);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_mfma(int fmt, const uint8_t* codes, const uint16_t* scales, int64_t n,
                            int64_t k, int64_t b, float* y, const void* ws, int cus,
                            hipStream_t st) {
  return launch_plan<false>(mfma_plan(n, k, cus), fmt, codes, scales, n, k, b, y,
                            static_cast<const uint4*>(ws), st);
}

int64_t gemv_mfma_max_planes(int64_t k) { return (k / kGroup + kWaves - 1) / kWaves; }

hipError_t launch_gemv_mfma_planes(int fmt, const uint8_t* codes, const uint16_t* scales,
                                   int64_t n, int64_t k, int64_t b, const uint16_t* x, float* hp,
                                   int cus, int64_t* planes, hipStream_t st) {
  const MfmaPlan p = mfma_plan(n, k, cus);
  *planes = p.kp;
  return launch_plan<true>(p, fmt, codes, scales, n, k, b, hp, reinterpret_cast<const uint4*>(x),
                           st);
}

}  // namespace lowbit
