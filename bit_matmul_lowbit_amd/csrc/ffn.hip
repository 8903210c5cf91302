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
// four launches:
//   1. GEMV prepare: x -> workspace, h = 0
//   2. GEMV accumulate: h += W_gu x                      (h FP32 [b][2f])
//   3. silu_mul_kernel: z = RNE_fp16(SiLU(h_gate) * h_up), written straight
//      into the down GEMV's workspace layout, and y = 0
//   4. GEMV accumulate: y += W_dn z                      (y FP32 [b][k])
// For b <= 2 (table GEMVs) step 1 also zeroes y, and step 4 forms z from h
// in its table build (same arithmetic), so step 3 is not launched.
#include "common.h"

namespace lowbit {
namespace {

// One 16-byte vector of z: 8 consecutive FP16 values of batch row `row`
// starting at column 8 * chunk; zeros for a row >= b.
__device__ __forceinline__ uint4 z_vector(const float* __restrict__ h, int64_t f, int b, int row,
                                          int64_t chunk) {
  if (row >= b) return make_uint4(0u, 0u, 0u, 0u);
  const float4* g4 = reinterpret_cast<const float4*>(h + (int64_t)row * 2 * f + chunk * 8);
  const float4* u4 = reinterpret_cast<const float4*>(h + (int64_t)row * 2 * f + f + chunk * 8);
  const float4 ga = g4[0], gb = g4[1], ua = u4[0], ub = u4[1];
  const float gv[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
  const float uv[8] = {ua.x, ua.y, ua.z, ua.w, ub.x, ub.y, ub.z, ub.w};
  return silu_mul8(gv, uv);
}

// z in one of two layouts, and (optionally) y = 0:
//   MFMA = false: [b][f] row-major FP16 (the workspace of the table GEMV, and
//                 the output of lowbit_silu_mul);
//   MFMA = true:  the matrix-core GEMV's operand order -- vector i = (group
//                 g, step j, lane l) holds batch row l % 16, chunk
//                 16 g + 4 j + l / 16, zeros for rows >= b.
template <bool MFMA>
__global__ __launch_bounds__(256) void silu_mul_kernel(const float* __restrict__ h, int64_t f,
                                                       int b, uint4* __restrict__ z,
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
    z[i] = z_vector(h, f, b, row, chunk);
  }
}

int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }

hipError_t launch_silu(const float* h, int64_t f, int64_t b, void* z, bool mfma, float* y,
                       int64_t ycount, hipStream_t st) {
  const int64_t nvec = mfma ? (f / kGroup) * 4 * 64 : b * f / 8;
  const int64_t work = nvec > (ycount + 3) / 4 ? nvec : (ycount + 3) / 4;
  int64_t blocks = (work + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  if (mfma)
    hipLaunchKernelGGL(silu_mul_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, st, h, f,
                       (int)b, static_cast<uint4*>(z), nvec, y, ycount);
  else
    hipLaunchKernelGGL(silu_mul_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, st, h, f,
                       (int)b, static_cast<uint4*>(z), nvec, y, ycount);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_silu_mul(const float* h, int64_t f, int64_t b, uint16_t* z, hipStream_t st) {
  return launch_silu(h, f, b, z, false, nullptr, 0, st);
}

// workspace: [x prepared for W_gu][h FP32 b x 2f][z prepared for W_dn], each
// part 256-byte aligned; b < kMfmaMinBatch never writes z out, so has no z part
size_t ffn_workspace_bytes(int64_t k, int64_t f, int64_t b) {
  return (size_t)(align256((int64_t)gemv_workspace_bytes(k, b)) + align256(b * 2 * f * 4) +
                  (b >= kMfmaMinBatch ? align256((int64_t)gemv_workspace_bytes(f, b)) : 0));
}

hipError_t launch_ffn(int fmt, const uint8_t* gu_codes, const uint16_t* gu_scales,
                      const uint8_t* dn_codes, const uint16_t* dn_scales, int64_t k, int64_t f,
                      const uint16_t* x, int64_t b, float* y, void* ws, hipStream_t st) {
  char* base = static_cast<char*>(ws);
  void* ws_x = base;
  float* h = reinterpret_cast<float*>(base + align256((int64_t)gemv_workspace_bytes(k, b)));
  if (gemv_direct_ok(2 * f, k, b) && gemv_direct_ok(k, f, b)) {
    // small matrices: two single-launch GEMVs that write h and y outright,
    // the second forming z from h as it loads its activations
    hipError_t e = launch_gemv_direct(fmt, gu_codes, gu_scales, 2 * f, k, x, b, h, st);
    if (e != hipSuccess) return e;
    return launch_gemv_direct_silu(fmt, dn_codes, dn_scales, k, f, h, b, y, st);
  }
  if (b < kMfmaMinBatch) {
    // table GEMVs: the down GEMV forms z from h in its own table build, so
    // the chain is three launches (prepare zeroes h and y)
    hipError_t e = launch_gemv_prepare_zero2(2 * f, k, x, b, h, ws_x, y, b * k, st);
    if (e != hipSuccess) return e;
    e = launch_gemv_accumulate(fmt, gu_codes, gu_scales, 2 * f, k, b, h, ws_x, st);
    if (e != hipSuccess) return e;
    return launch_gemv_accumulate_silu(fmt, dn_codes, dn_scales, k, f, b, y, h, st);
  }
  void* ws_z = reinterpret_cast<char*>(h) + align256(b * 2 * f * 4);
  hipError_t e = launch_gemv_prepare(2 * f, k, x, b, h, ws_x, st);
  if (e != hipSuccess) return e;
  e = launch_gemv_accumulate(fmt, gu_codes, gu_scales, 2 * f, k, b, h, ws_x, st);
  if (e != hipSuccess) return e;
  e = launch_silu(h, f, b, ws_z, true, y, b * k, st);
  if (e != hipSuccess) return e;
  return launch_gemv_accumulate(fmt, dn_codes, dn_scales, k, f, b, y, ws_z, st);
}

}  // namespace lowbit
