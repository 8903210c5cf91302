// Decode FFN:  y = W_dn ( SiLU(W_gate x) * (W_up x) )
//
// [P2] 7minutos.es, "PrismML lanza Bonsai 27B ...", "Como funciona la
//      compresion": the MLP projections are low-bit like every other matrix.
// [P5] openclawradar.com, "Bonsai 1.7B Modelo Ternario ...", "Detalles
//      tecnicos": decode kernels were tuned at the matvec / FFN level.
// The pages do not spell the MLP out; it is the gated form of the Qwen
// family the models derive from.  Gate and up are stacked in one [2f][k]
// matrix (gate rows first) so that one GEMV streams both, and the product
// SiLU(gate) * up is rounded to FP16, the activation type the down GEMV
// reads.
//
// The chain runs on the caller's stream with no host wait, so the caller
// can capture it in one HIP graph.  For b >= 3 (matrix-core GEMVs) it is
// three launches:
//   1. gate+up GEMV: x read in place, one plane of partial sums per K-piece
//      (h = the sum of the planes, FP32 [b][2f]; plain stores, so nothing
//      has to be zeroed and no prepare launch is needed)
//   2. silu_mul_kernel: h = the planes added up in plane order, z =
//      RNE_fp16(SiLU(h_gate) * h_up), written straight into the down GEMV's
//      workspace layout, and y = 0
//   3. GEMV accumulate: y += W_dn z                      (y FP32 [b][k])
// For b <= 2 (table GEMVs) it is two launches: the gate+up GEMV stores one
// plane of partial sums per K-slice (no atomics, so h needs no zeroing and
// x is read in place: no prepare) and zeroes y; the down GEMV adds the
// planes up in a fixed order and forms z from that h in its table build
// (same arithmetic as step 2).
#include "common.h"

namespace lowbit {
namespace {

// One 16-byte vector of z: 8 consecutive FP16 values of batch row `row`
// starting at column 8 * chunk, from h = the sum of np planes (FP32
// [np][b][2f], added in plane order); zeros for a row >= b.
// With NP > 0 (np = NP planes) the loads of every plane go out before the
// first add, one round trip in all; NP = 0 takes the planes one at a time.
template <int NP>
__device__ __forceinline__ uint4 z_vector(const float* __restrict__ h, int np, int64_t f, int b,
                                          int row, int64_t chunk) {
  if (row >= b) return make_uint4(0u, 0u, 0u, 0u);
  float gv[8], uv[8];
  if constexpr (NP > 0) {
    float4 v[NP][4];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const float* hr = h + ((int64_t)p * b + row) * 2 * f;
      const float4* g4 = reinterpret_cast<const float4*>(hr + chunk * 8);
      const float4* u4 = reinterpret_cast<const float4*>(hr + f + chunk * 8);
      v[p][0] = g4[0];
      v[p][1] = g4[1];
      v[p][2] = u4[0];
      v[p][3] = u4[1];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const float gp[8] = {v[p][0].x, v[p][0].y, v[p][0].z, v[p][0].w,
                           v[p][1].x, v[p][1].y, v[p][1].z, v[p][1].w};
      const float up[8] = {v[p][2].x, v[p][2].y, v[p][2].z, v[p][2].w,
                           v[p][3].x, v[p][3].y, v[p][3].z, v[p][3].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        gv[j] = p == 0 ? gp[j] : gv[j] + gp[j];
        uv[j] = p == 0 ? up[j] : uv[j] + up[j];
      }
    }
    return silu_mul8(gv, uv);
  }
  for (int p = 0; p < np; ++p) {
    const float* hr = h + ((int64_t)p * b + row) * 2 * f;
    const float4* g4 = reinterpret_cast<const float4*>(hr + chunk * 8);
    const float4* u4 = reinterpret_cast<const float4*>(hr + f + chunk * 8);
    const float4 ga = g4[0], gb = g4[1], ua = u4[0], ub = u4[1];
    const float gp[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
    const float up[8] = {ua.x, ua.y, ua.z, ua.w, ub.x, ub.y, ub.z, ub.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      gv[j] = p == 0 ? gp[j] : gv[j] + gp[j];
      uv[j] = p == 0 ? up[j] : uv[j] + up[j];
    }
  }
  return silu_mul8(gv, uv);
}

// z in one of two layouts, and (optionally) y = 0:
//   MFMA = false: [b][f] row-major FP16 (the workspace of the table GEMV, and
//                 the output of lowbit_silu_mul);
//   MFMA = true:  the matrix-core GEMV's operand order -- vector i = (group
//                 g, step j, lane l) holds batch row l % 16, chunk
//                 16 g + 4 j + l / 16, zeros for rows >= b.
template <bool MFMA, int NP = 0>
__global__ __launch_bounds__(256) void silu_mul_kernel(const float* __restrict__ h, int np,
                                                       int64_t f, int b, uint4* __restrict__ z,
                                                       int64_t nvec, float* __restrict__ y,
                                                       int64_t ycount) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * 256;
  zero_f32(y, ycount, gid, stride);
  const int64_t cpr = f / 8;  // 16-byte vectors per batch row
  for (int64_t i = gid; i < nvec; i += stride) {
    int row;
    int64_t chunk;
    if constexpr (MFMA) {
      const int l = (int)(i & 63);
      const int64_t gj = i >> 6;
      row = l & 15;
      chunk = (gj >> 2) * 16 + 4 * (gj & 3) + (l >> 4);
    } else {
      row = (int)(i / cpr);
      chunk = i - (int64_t)row * cpr;
    }
    z[i] = z_vector<NP>(h, np, f, b, row, chunk);
  }
}

int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }

hipError_t launch_silu(const float* h, int64_t np, int64_t f, int64_t b, void* z, bool mfma,
                       float* y, int64_t ycount, hipStream_t st) {
  const int64_t nvec = mfma ? (f / kGroup) * 4 * 64 : b * f / 8;
  const int64_t work = nvec > (ycount + 3) / 4 ? nvec : (ycount + 3) / 4;
  int64_t blocks = (work + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  if (mfma) {
    // the plane count as a template argument up to 8 (the K-pieces of the
    // gate+up GEMV: 5 at the 27B shape)
#define LOWBIT_SILU(NPV)                                                                        \
  hipLaunchKernelGGL((silu_mul_kernel<true, NPV>), dim3((unsigned)blocks), dim3(256), 0, st, h,  \
                     (int)np, f, (int)b, static_cast<uint4*>(z), nvec, y, ycount)
    switch (np) {
      case 1: LOWBIT_SILU(1); break;
      case 2: LOWBIT_SILU(2); break;
      case 3: LOWBIT_SILU(3); break;
      case 4: LOWBIT_SILU(4); break;
      case 5: LOWBIT_SILU(5); break;
      case 6: LOWBIT_SILU(6); break;
      case 7: LOWBIT_SILU(7); break;
      case 8: LOWBIT_SILU(8); break;
      default: LOWBIT_SILU(0); break;
    }
#undef LOWBIT_SILU
  } else
    hipLaunchKernelGGL(silu_mul_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, st, h,
                       (int)np, f, (int)b, static_cast<uint4*>(z), nvec, y, ycount);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_silu_mul(const float* h, int64_t f, int64_t b, uint16_t* z, hipStream_t st) {
  return launch_silu(h, 1, f, b, z, false, nullptr, 0, st);
}

// workspace, each part 256-byte aligned: h as P planes FP32 b x 2f, P = the
// gate+up GEMV's K-slices (table GEMV, b < kMfmaMinBatch) or at most that
// many K-pieces (matrix-core GEMV; the single-launch pair uses plane 0),
// then for b >= kMfmaMinBatch z prepared for W_dn
size_t ffn_workspace_bytes(int64_t k, int64_t f, int64_t b) {
  if (b < kMfmaMinBatch) return (size_t)align256(gemv_partial_planes(k, b) * b * 2 * f * 4);
  return (size_t)(align256(gemv_mfma_max_planes(k) * b * 2 * f * 4) +
                  align256((int64_t)gemv_workspace_bytes(f, b)));
}

hipError_t launch_ffn(int fmt, const uint8_t* gu_codes, const uint16_t* gu_scales,
                      const uint8_t* dn_codes, const uint16_t* dn_scales, int64_t k, int64_t f,
                      const uint16_t* x, int64_t b, float* y, void* ws, hipStream_t st) {
  char* base = static_cast<char*>(ws);
  if (gemv_direct_ok(2 * f, k, b) && gemv_direct_ok(k, f, b)) {
    // small matrices: two single-launch GEMVs that write h (at the start of
    // the workspace) and y outright, the second forming z from h as it
    // loads its activations
    float* h = reinterpret_cast<float*>(base);
    hipError_t e = launch_gemv_direct(fmt, gu_codes, gu_scales, 2 * f, k, x, b, h, st);
    if (e != hipSuccess) return e;
    return launch_gemv_direct_silu(fmt, dn_codes, dn_scales, k, f, h, b, y, st);
  }
  if (b < kMfmaMinBatch) {
    // table GEMVs: gate+up stores per-slice planes of h (and zeroes y), the
    // down GEMV sums them and forms z in its own table build
    float* hp = reinterpret_cast<float*>(base);
    hipError_t e = launch_gemv_partials(fmt, gu_codes, gu_scales, 2 * f, k, b, x, hp, y, b * k, st);
    if (e != hipSuccess) return e;
    return launch_gemv_accumulate_silu(fmt, dn_codes, dn_scales, k, f, b, y, hp,
                                       gemv_partial_planes(k, b), st);
  }
  // matrix-core GEMVs: gate+up stores per-K-piece planes of h, the SiLU
  // launch sums them, forms z in the down GEMV's operand order and zeroes y
  float* hp = reinterpret_cast<float*>(base);
  void* ws_z = base + align256(gemv_mfma_max_planes(k) * b * 2 * f * 4);
  int64_t np = 0;
  hipError_t e = launch_gemv_mfma_planes(fmt, gu_codes, gu_scales, 2 * f, k, b, x, hp,
                                         device_cu_count(), &np, st);
  if (e != hipSuccess) return e;
  e = launch_silu(hp, np, f, b, ws_z, true, y, b * k, st);
  if (e != hipSuccess) return e;
  return launch_gemv_accumulate(fmt, dn_codes, dn_scales, k, f, b, y, ws_z, st);
}

}  // namespace lowbit
