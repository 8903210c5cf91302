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
//   * wave w takes K-range [512 w, 512 w + 512) (64 chunks of 8 weights).
//     A code dword of a cell holds one byte of each of 4 rows, and a lane
//     takes all 4: lane (q = l % 16, m = l / 16) takes rows 4m .. 4m + 3 of
//     the tile and chunks q, q + 16, q + 32, q + 48 of the range (one per
//     group); with half tiles, lane (l % 32, l / 32) takes 4 of the 8 rows
//     and chunks q, q + 32.  The 16 (32) lanes of a row quad read 16 (32)
//     adjacent cells;
//   * loads go out in the order they are needed: first what the work-group
//     stages in LDS (x for b >= 3, k <= 4096; h for the FFN variant), then,
//     chunk by chunk, the code dword (ternary: pos and neg), the 4 rows'
//     scales of the chunk's group (8 bytes) and, for b <= 2, x as a 16-byte
//     FP16 vector.  Loads complete in order, so the staging waits for no
//     code load and each chunk's arithmetic waits only for its own loads;
//   * a packed shift fed the 16-bit half that holds a row's byte (op_sel, no
//     byte moves) and v_bitop3 turn each bit pair into FP16 (+s or -s;
//     ternary also 0) and v_dot2_f32_f16 adds (+-s) x for two weights at a
//     time into an FP32 sum -- products of two FP16 numbers are exact in
//     FP32;
//   * the lanes of a row quad are summed on DPP (two transposed stages leave
//     one row per lane), the waves' sums through LDS, and y is stored once.
// The FFN variant (SILU) takes h = [gate | up] (FP32 [b][2k]) instead of x
// and forms z = RNE_fp16(SiLU(gate) * up) itself: lane l of wave w forms
// chunk 64 w + l into LDS, from where the lanes that need it read it.
#include "common.h"

namespace lowbit {
namespace {

constexpr int kWaveK = 512;           // weights of K per wave
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

// v of the lane named by a DPP control (within rows of 16 lanes)
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
constexpr int kDppRor8 = 0x128;        // lane i <- lane (i + 8) mod 16 (= i ^ 8)
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7 - i within 8
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]

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
// the chunks).  A code dword of a cell holds 4 rows (one byte each), and a
// lane takes all 4: lane (q, m) = (l % QN, l / QN) takes rows rq .. rq + 3
// (rq = r0 + 4 m, m < RH / 4) of chunks q, q + QN, ... of the wave's range
// (QN = 256 / RH chunk lanes per row quad, LC = 64 / QN chunks each).
template <int FMT, int B, bool SILU, int RH>
__global__ __launch_bounds__(64 * max_waves<B>()) void gemv_direct_kernel(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const void* __restrict__ xin, int64_t n, int64_t k, float* __restrict__ y) {
  constexpr int CB = Fmt<FMT>::cell_bytes;
  constexpr int MQ = RH / 4;                // row quads per work-group
  constexpr int QN = 64 / MQ;               // chunk lanes per row quad
  constexpr int LC = kWaveK / kChunk / QN;  // chunks per lane
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
  const int q = lane % QN, rq = r0 + 4 * (lane / QN);       // chunk lane, first of 4 rows
  const int64_t nch = k / kChunk;
  const int64_t G = k / kGroup;
  const int c0 = wave * (kWaveK / kChunk);  // first chunk of the wave
  // chunks past k (last wave of a k that is not a multiple of 512) read as
  // zeros: codes and scales past their resource, x by the kNoLoad offset
  const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(codes + tile * nch * CB, nch * CB);
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(scales + tile * G * 16, G * 32);
  constexpr uint32_t kNoLoad = 0x80000000u;

  // Loads, in the order the work-group needs them: first what is staged in
  // LDS (x for b >= 3, h for the FFN variant: thread t takes chunk c0 + lane
  // of every batch row), then the lane's chunks one by one (code dword(s),
  // the 4 rows' scales of the chunk's group -- 8 contiguous bytes -- and,
  // for b <= 2, x).  Loads complete in order, so staging waits for no code
  // load, and the contraction of chunk i waits only for the loads up to it.
  const int pitch = nw * 64;  // chunks per x row in LDS: zeros past k
  const int64_t cs = c0 + lane;  // chunk staged by this thread
  uint4 xs[XLDS ? B : 1];
  float4 hs[SILU ? B : 1][4];
  if constexpr (XLDS) {
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(xin, B * k * 2);
#pragma unroll
    for (int bi = 0; bi < B; ++bi)
      xs[bi] = qload(rx, cs < nch ? (uint32_t)((bi * k + cs * 8) * 2) : kNoLoad);
  } else if constexpr (SILU) {
    const __amdgpu_buffer_rsrc_t rh = buffer_rsrc(xin, B * 2 * k * 4);
#pragma unroll
    for (int bi = 0; bi < B; ++bi) {
      const uint32_t go = cs < nch ? (uint32_t)((bi * 2 * k + cs * 8) * 4) : kNoLoad;
      const uint32_t uo = cs < nch ? go + (uint32_t)(k * 4) : kNoLoad;
      const uint4 a = qload(rh, go), b2 = qload(rh, go + (cs < nch ? 16u : 0u));
      const uint4 c = qload(rh, uo), d = qload(rh, uo + (cs < nch ? 16u : 0u));
      hs[bi][0] = __builtin_bit_cast(float4, a);
      hs[bi][1] = __builtin_bit_cast(float4, b2);
      hs[bi][2] = __builtin_bit_cast(float4, c);
      hs[bi][3] = __builtin_bit_cast(float4, d);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  uint32_t cw[LC], nwd[FMT == 2 ? LC : 1];
  uint2 sw[LC];
  uint4 xv[SILU || XLDS ? 1 : LC][B];
  const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(xin, B * k * 2);
#pragma unroll
  for (int i = 0; i < LC; ++i) {
    const int c = c0 + q + QN * i;
    const uint32_t off = (uint32_t)(c * CB + rq);
    cw[i] = dload(rc, off);
    if constexpr (FMT == 2) nwd[i] = dload(rc, off + 16);
    // chunk c lies in group c / 16; the 4 rows' scales of it are 8 bytes
    const auto s2 = __builtin_amdgcn_raw_buffer_load_b64(rs, (uint32_t)(((c >> 4) * 16 + rq) * 2), 0, 0);
    sw[i] = make_uint2(s2[0], s2[1]);
    if constexpr (!SILU && !XLDS) {
#pragma unroll
      for (int bi = 0; bi < B; ++bi)
        xv[i][bi] = qload(rx, c < nch ? (uint32_t)((bi * k + c * 8) * 2) : kNoLoad);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the chunks' loads in this order
  }

  if constexpr (XLDS) {
    // x [B][k] FP16 into LDS (zeros past k)
#pragma unroll
    for (int bi = 0; bi < B; ++bi) xbuf[bi * pitch + cs] = xs[bi];
  } else if constexpr (SILU) {
    // z of chunk c0 + lane, all batch rows, into LDS (zeros past k: h reads 0)
#pragma unroll
    for (int bi = 0; bi < B; ++bi) {
      const float gv[8] = {hs[bi][0].x, hs[bi][0].y, hs[bi][0].z, hs[bi][0].w,
                           hs[bi][1].x, hs[bi][1].y, hs[bi][1].z, hs[bi][1].w};
      const float uv[8] = {hs[bi][2].x, hs[bi][2].y, hs[bi][2].z, hs[bi][2].w,
                           hs[bi][3].x, hs[bi][3].y, hs[bi][3].z, hs[bi][3].w};
      zbuf[(wave * 64 + lane) * B + bi] = silu_mul8(gv, uv);
    }
  }
  if constexpr (XLDS || SILU) {
    // the LDS stores done (the staging loads are, being the oldest); the
    // code loads stay in flight across the barrier
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lds(63));
    stage_barrier();
  }

  // acc[r][bi]: row rq + r, batch row bi
  float acc[4][B];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int bi = 0; bi < B; ++bi) acc[r][bi] = 0.0f;
#pragma unroll
  for (int i = 0; i < LC; ++i) {
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
    const uint32_t dn = FMT == 2 ? cw[i] ^ nwd[i] : 0u;  // ternary: nonzero
    // row r: code byte r, scale half r of the group's 4 scales (both halves)
#define LOWBIT_DROW(R)                                                                      \
  {                                                                                         \
    const uint32_t sv = (R) < 2 ? sw[i].x : sw[i].y;                                        \
    const uint32_t ss = __builtin_amdgcn_perm(sv, sv, ((R) & 1) ? 0x03020302u : 0x01000100u); \
    LOWBIT_DPAIR(R, 0) LOWBIT_DPAIR(R, 1) LOWBIT_DPAIR(R, 2) LOWBIT_DPAIR(R, 3)             \
  }
#define LOWBIT_DPAIR(R, P)                                                                  \
  {                                                                                         \
    uint32_t a;                                                                             \
    if constexpr (FMT == 1)                                                                 \
      a = ss ^ (~byte_pair_bits<R, P>(cw[i]) & kSignBits);                                  \
    else                                                                                    \
      a = (ss ^ (byte_pair_bits<R, P>(nwd[i]) & kSignBits)) & mask15(byte_pair_bits<R, P>(dn)); \
    _Pragma("unroll") for (int bi = 0; bi < B; ++bi) acc[R][bi] = dot2(a, word(xi[bi], P), acc[R][bi]); \
  }
    LOWBIT_DROW(0) LOWBIT_DROW(1) LOWBIT_DROW(2) LOWBIT_DROW(3)
#undef LOWBIT_DPAIR
#undef LOWBIT_DROW
  }
  // Sum over the QN lanes of a row quad (lane bits 0 .. log2 QN - 1), on
  // DPP within 16-lane rows.  Two transposed stages leave each lane one of
  // the 4 rows, r = 2 bit3 + bit2: on bit 3 with lane i ^ 8, on bit 2 with
  // the half-row mirror 7 - i (which also flips bits 1 and 0: harmless, the
  // butterflies on those bits follow); bit 4 (QN = 32) by a lane shuffle.
#pragma unroll
  for (int bi = 0; bi < B; ++bi) {
    const bool h3 = (q >> 3) & 1, h2 = (q >> 2) & 1;
    const float k0 = h3 ? acc[2][bi] : acc[0][bi], s0 = h3 ? acc[0][bi] : acc[2][bi];
    const float k1 = h3 ? acc[3][bi] : acc[1][bi], s1 = h3 ? acc[1][bi] : acc[3][bi];
    const float v0 = k0 + dpp_f32<kDppRor8>(s0);
    const float v1 = k1 + dpp_f32<kDppRor8>(s1);
    float v = (h2 ? v1 : v0) + dpp_f32<kDppHalfMirror>(h2 ? v0 : v1);
    v += dpp_f32<kDppQuadXor2>(v);
    v += dpp_f32<kDppQuadXor1>(v);
    if constexpr (QN == 32) v += __shfl_xor(v, 16);
    acc[0][bi] = v;
  }
  if ((q & ~12) == 0) {
    const int row = rq + 2 * ((q >> 3) & 1) + ((q >> 2) & 1);
#pragma unroll
    for (int bi = 0; bi < B; ++bi) red[wave * RH * B + bi * RH + (row - r0)] = acc[0][bi];
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
