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
// (rho = 0..15) that share the A operand.  Lane quarter q = l / 16 takes
// chunks 4q .. 4q + 3 of each 128-weight group (64 / 128 contiguous bytes).
//
// Expansion of a Q1 byte e (bit j <-> k0 + j) into four FP16 pairs: with e
// in the low byte of both 16-bit halves, a packed 16-bit shift by
// (15 - 2p, 14 - 2p) brings bits 2p and 2p + 1 to bits 15 and 31, and
// v_bitop3 picks +s or -s (which differ only in those sign bits): two
// VALU operations per FP16 pair.  A ternary pair also needs the mask of
// (pos xor neg), so a cell with both bits set is 0, as pos - neg is, and a
// zero weight contributes an exact 0 (five operations per pair).
//
// Work: an item is (16-tile block, K-piece).  The grid is persistent (two
// work-groups per CU); work-group w takes items w, w + W, ... in order, so
// all work-groups sweep the matrix together.  Inside an item the 4 waves
// take its groups round-robin; their load rings run on across items, and
// at the end of an item the waves sum their partials through LDS and add
// them to y with one coalesced FP32 atomic per (row, batch row).
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

// Q1: bit set -> +s, clear -> -s;  ss = s in both halves
__device__ __forceinline__ f16x8 expand_q1(uint32_t d, uint32_t ss) {
  u32x4 v;
  v[0] = ss ^ (~pk_shl(d, kPairShift<0>) & kSignBits);
  v[1] = ss ^ (~pk_shl(d, kPairShift<1>) & kSignBits);
  v[2] = ss ^ (~pk_shl(d, kPairShift<2>) & kSignBits);
  v[3] = ss ^ (~pk_shl(d, kPairShift<3>) & kSignBits);
  return __builtin_bit_cast(f16x8, v);
}

// T2: dn = pos xor neg (nonzero), dq = neg (sign);  -> +s, -s or 0
__device__ __forceinline__ f16x8 expand_t2(uint32_t dn, uint32_t dq, uint32_t ss) {
  u32x4 v;
#define LOWBIT_PAIR(P)                                                                   \
  v[P] = (ss ^ (pk_shl(dq, kPairShift<P>) & kSignBits)) & pk_mask15(pk_shl(dn, kPairShift<P>));
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

template <int FMT>
__device__ __forceinline__ void load_group(GroupRegs<FMT>& r, __amdgpu_buffer_rsrc_t rc,
                                           __amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rx,
                                           uint32_t voff_c, uint32_t voff_s, uint32_t voff_x,
                                           int g) {
  constexpr int GB = FMT == 1 ? 256 : 512;  // code bytes per tile per group
  const int sc = g * GB;
#pragma unroll
  for (int i = 0; i < GroupRegs<FMT>::kCells; ++i) r.c[i] = bload(rc, voff_c, sc + 16 * i);
  r.s[0] = bload<0>(rs, voff_s, g * 32);
  r.s[1] = bload<16>(rs, voff_s, g * 32);
#pragma unroll
  for (int j = 0; j < kSteps; ++j) r.x[j] = bload(rx, voff_x, (g * kSteps + j) * kXStep);
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
      expand_t2(rep_byte<(RHO) & 3>(nw[(RHO) >> 2]), rep_byte<(RHO) & 3>(qw[(RHO) >> 2]),  \
                ss[RHO]),                                                                  \
      acc[RHO], 0, 0, 0);
      LOWBIT_ROW(0) LOWBIT_ROW(1) LOWBIT_ROW(2) LOWBIT_ROW(3) LOWBIT_ROW(4) LOWBIT_ROW(5)
      LOWBIT_ROW(6) LOWBIT_ROW(7) LOWBIT_ROW(8) LOWBIT_ROW(9) LOWBIT_ROW(10) LOWBIT_ROW(11)
      LOWBIT_ROW(12) LOWBIT_ROW(13) LOWBIT_ROW(14) LOWBIT_ROW(15)
#undef LOWBIT_ROW
    }
  }
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
    // vector i = (group g, step j, lane l): batch row l % 16, chunk 16 g + 4 (l / 16) + j
    const int l = (int)(i & 63);
    const int64_t gj = i >> 6;
    const int64_t g = gj / kSteps;
    const int j = (int)(gj % kSteps);
    const int row = l & 15;
    const int64_t chunk = g * 16 + 4 * (l >> 4) + j;
    xw[i] = row < b ? *reinterpret_cast<const uint4*>(x + row * k + chunk * kChunk)
                    : make_uint4(0u, 0u, 0u, 0u);
  }
}

template <int FMT>
__global__ __launch_bounds__(kThreads, 2) void gemv_mfma_kernel(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint4* __restrict__ xw, float* __restrict__ y, int64_t n, int64_t k, int b,
    int64_t ntiles, int kpieces, int gpp, int64_t nitems) {
  __shared__ float red[kWaves * 16 * kRedPitch];
  constexpr int D = 2;  // groups of loads in flight per wave, plus the one in use
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = (int)(k / kGroup);
  const int tl = lane & 15, q = lane >> 4;
  const int64_t cpitch = (k / kChunk) * Fmt<FMT>::cell_bytes;
  const int64_t spitch = (int64_t)G * kTileRows * 2;
  constexpr int GB = FMT == 1 ? 256 : 512;
  const uint32_t voff_c = (uint32_t)(tl * cpitch + q * (GB / 4));
  const uint32_t voff_s = (uint32_t)(tl * spitch);
  const uint32_t voff_x = (uint32_t)(lane * 16);
  const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(xw, (int64_t)G * kSteps * kXStep);
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
    load_group<FMT>(r, live ? rc : rz, live ? rs : rz, live ? rx : rz, voff_c, voff_s, voff_x,
                    live ? g : 0);
  };

  f32x4 acc[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = (f32x4){0.f, 0.f, 0.f, 0.f};
  GroupRegs<FMT> ring[D];
#pragma unroll
  for (int i = 0; i < D - 1; ++i) load(ring[i], i);
  for (int64_t sl = 0; sl < total; sl += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      // the next group's loads go out before this group's MFMAs (the
      // scheduler would otherwise sink them into the MFMA sequence)
      load(ring[(u + D - 1) % D], sl + u + D - 1);
      __builtin_amdgcn_sched_barrier(0);
      group_mfma<FMT>(ring[u], acc);
      __builtin_amdgcn_sched_barrier(0);
      const int64_t cur = sl + u;
      if (cur < total && (cur + 1) % per == 0) {
        // end of an item: partial sums of the waves -> LDS -> y
        const int64_t item = blockIdx.x + (cur / per) * (int64_t)gridDim.x;
        const int64_t T0 = (item / kpieces) * 16;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            red[(wave * 16 + 4 * q + v) * kRedPitch + r * 16 + tl] = acc[r][v];
            acc[r][v] = 0.0f;
          }
        }
        __syncthreads();
        // thread t: row T0 * 16 + t (t = 16 * tile + rho)
        const int t = threadIdx.x;
        const int64_t row = T0 * 16 + t;
        const int rr = (t & 15) * 16 + (t >> 4);
        if (row < n) {
          for (int i = 0; i < b; ++i) {
            float sum = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) sum += red[(w * 16 + i) * kRedPitch + rr];
            atomicAdd(y + i * n + row, sum);
          }
        }
        __syncthreads();
      }
    }
  }
}

}  // namespace

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

hipError_t launch_gemv_mfma(int fmt, const uint8_t* codes, const uint16_t* scales, int64_t n,
                            int64_t k, int64_t b, float* y, const void* ws, int cus,
                            hipStream_t st) {
  const int64_t ntiles = (n + kTileRows - 1) / kTileRows;
  const int64_t nblocks = (ntiles + 15) / 16;
  const int G = (int)(k / kGroup);
  // Persistent grid of up to two work-groups per CU.  An item's K-piece is
  // 4 * per groups (per groups for each wave): per is chosen for about four
  // items per work-group, but at least two groups per wave (each item ends
  // with an LDS reduction and atomics) and no more than K holds.  The grid
  // is then sized so that every work-group gets the same number of items;
  // a matrix with few items (at most two per resident slot) gets one
  // work-group per item instead, as many loads in flight as possible.  A
  // matrix whose two-group items would not even give every CU one takes a
  // single group per wave (twice the items): 6144x2048 ternary at b = 3..8
  // runs 12.2 -> 11.1 us, while larger matrices lose with it.
  const int64_t nwg_max = 2 * (int64_t)cus;
  int64_t per = (int64_t)G * nblocks / (4 * kWaves * nwg_max);
  const int64_t per_max = (G + kWaves - 1) / kWaves;
  if (per < 2) per = nblocks * ((G + 2 * kWaves - 1) / (2 * kWaves)) < cus ? 1 : 2;
  if (per > per_max) per = per_max;
  const int gpp = (int)(kWaves * per);
  const int64_t kp = (G + gpp - 1) / gpp;
  const int64_t nitems = nblocks * kp;
  const int64_t rounds = (nitems + nwg_max - 1) / nwg_max;
  const int64_t nwg = nitems <= 2 * nwg_max ? nitems : (nitems + rounds - 1) / rounds;
  const dim3 grid((unsigned)nwg);
  const uint4* xw = static_cast<const uint4*>(ws);
  if (fmt == 1)
    hipLaunchKernelGGL(gemv_mfma_kernel<1>, grid, dim3(kThreads), 0, st, codes, scales, xw, y, n,
                       k, (int)b, ntiles, (int)kp, gpp, nitems);
  else
    hipLaunchKernelGGL(gemv_mfma_kernel<2>, grid, dim3(kThreads), 0, st, codes, scales, xw, y, n,
                       k, (int)b, ntiles, (int)kp, gpp, nitems);
  return hipGetLastError();
}

}  // namespace lowbit
