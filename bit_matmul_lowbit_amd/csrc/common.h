// Internal declarations shared by the HIP sources of liblowbit.so.
// Layout constants follow include/lowbit.h (version 1): 16-row tiles, 8-weight
// chunks (one byte per row per chunk), 128-weight groups along K.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lowbit {

constexpr int kTileRows = 16;   // rows per tile
constexpr int kChunk = 8;       // weights per code byte
constexpr int kGroup = 128;     // weights per scale
constexpr int kChunksPerGroup = kGroup / kChunk;

// cell bytes: 16 rows x 1 byte (Q1) or 16 rows x (pos byte, neg byte) (T2)
template <int FMT> struct Fmt;
template <> struct Fmt<1> { static constexpr int cell_bytes = 16; };
template <> struct Fmt<2> { static constexpr int cell_bytes = 32; };

// Raw buffer resource over [base, base + bytes) (bytes < 2^31): a load at an
// offset past the end returns zeros without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int64_t bytes) {
  constexpr int kRawBufferFlags = 0x00020000;  // gfx9 buffer descriptor word 3
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRawBufferFlags);
}

// s_waitcnt immediate that waits until at most n memory loads of this wave
// are outstanding (LDS and export counters left at their maximum)
__host__ __device__ constexpr int waitcnt_vm(int n) {
  return (n & 0xF) | (((n >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8);
}
// the same, and every LDS access of this wave complete
__host__ __device__ constexpr int waitcnt_vm_lds(int n) {
  return (n & 0xF) | (((n >> 4) & 3) << 14) | (0x7 << 4);
}

// Work-group barrier without __syncthreads()'s release fence: that fence
// also waits for this wave's loads into LDS that are still in flight for
// later pipeline stages, which the caller leaves outstanding on purpose.
// The caller's s_waitcnt makes the LDS accesses (and loads) that the other
// waves need complete first; the empty asm statements keep the compiler
// from moving memory accesses across.
__device__ __forceinline__ void stage_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Code-byte expansion helpers shared by the matrix-core GEMV and the GEMM.
typedef short s16x2 __attribute__((ext_vector_type(2)));

// per-half shift of a packed pair of 16-bit values
__device__ __forceinline__ uint32_t pk_shl(uint32_t d, uint32_t sh) {
  const s16x2 a = __builtin_bit_cast(s16x2, d), s = __builtin_bit_cast(s16x2, sh);
  return __builtin_bit_cast(uint32_t, (s16x2)(a << s));
}

// byte J of w in the low byte of both halves
template <int J>
__device__ __forceinline__ uint32_t rep_byte(uint32_t w) {
  return __builtin_amdgcn_perm(w, w, 0x0C000C00u | ((uint32_t)J << 16) | (uint32_t)J);
}

// shift that brings bits 2p and 2p + 1 of a byte placed in the low byte of
// both halves to bits 15 and 31
template <int P>
constexpr uint32_t kPairShift = ((uint32_t)(14 - 2 * P) << 16) | (uint32_t)(15 - 2 * P);
constexpr uint32_t kSignBits = 0x80008000u;

// Bits 2P and 2P + 1 of byte J of w at bits 15 and 31 (the other bits are
// left as they fall): the 16-bit half that holds byte J feeds both halves of
// one packed shift (v_pk_lshlrev_b16 with op_sel), so the byte is not moved
// first.
template <int J, int P>
__device__ __forceinline__ uint32_t byte_pair_bits(uint32_t w) {
  const s16x2 a = __builtin_bit_cast(s16x2, w);
  const s16x2 h = __builtin_shufflevector(a, a, J >> 1, J >> 1);
  constexpr short lo = (short)(15 - 2 * P - 8 * (J & 1)), hi = (short)(14 - 2 * P - 8 * (J & 1));
  return __builtin_bit_cast(uint32_t, (s16x2)(h << (s16x2){lo, hi}));
}

// SiLU(v) = v / (1 + e^-v) in FP32 with the device library's expf; for
// v < -88 e^-v is infinite and the quotient is -0.
__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

// The FP32 product a * b rounded to FP16 (nearest-even), IEEE in every
// case including the sign of a zero.  Written plainly, the compiler turns a
// product followed by the FP16 conversion into one mixed-precision FMA with
// a +0 addend (v_fma_mixlo_f16 a, b, 0), and -0 + +0 is +0: a product that
// is -0 (SiLU(v) = -0 for v < -88, times u > 0) came out as +0.  The empty
// asm statement keeps the product in its own v_mul_f32, converted by
// v_cvt_f16_f32.
__device__ __forceinline__ _Float16 mul_to_fp16(float a, float b) {
  float p = a * b;
  __asm__("" : "+v"(p));
  return (_Float16)p;
}

// 8 FP16 values RNE_fp16(SiLU(g_j) * u_j) packed two per dword (j = 2p low half)
__device__ __forceinline__ uint4 silu_mul8(const float (&gv)[8], const float (&uv)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const _Float16 lo = mul_to_fp16(silu(gv[2 * p]), uv[2 * p]);
    const _Float16 hi = mul_to_fp16(silu(gv[2 * p + 1]), uv[2 * p + 1]);
    w[p] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// y[0 .. count) = 0 by the threads gid = 0, stride, 2 stride, ... of a grid:
// 16-byte stores (y is 16-byte aligned), then the count % 4 tail.
__device__ __forceinline__ void zero_f32(float* y, int64_t count, int64_t gid, int64_t stride) {
  const int64_t nv = count / 4;
  for (int64_t i = gid; i < nv; i += stride)
    reinterpret_cast<float4*>(y)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (gid < count - nv * 4) y[nv * 4 + gid] = 0.0f;
}

// Compute units of the current device (256 if it cannot be queried), cached
// per device id; safe to call from several host threads.
int device_cu_count();

// Kernel launchers (host side, defined in the .hip files).  All return a
// hipError_t from the launch; shapes were validated by the caller.
hipError_t launch_quantize_q1(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                              uint16_t* scales, hipStream_t st);
hipError_t launch_pack_t2(const int8_t* t, const uint16_t* s, int64_t n, int64_t k,
                          uint8_t* codes, uint16_t* scales, hipStream_t st);
hipError_t launch_unpack(int fmt, const uint8_t* codes, const uint16_t* scales, int64_t n,
                         int64_t k, uint16_t* w, hipStream_t st);
// ternary quantiser and base-3 storage
hipError_t launch_quantize_t2(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                              uint16_t* scales, hipStream_t st);
hipError_t launch_t2_to_base3(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                              uint8_t* out, uint16_t* out_scales, hipStream_t st);
hipError_t launch_base3_to_t2(const uint8_t* in, const uint16_t* in_scales, int64_t n, int64_t k,
                              uint8_t* codes, uint16_t* scales, hipStream_t st);

// decode GEMV: subset-sum tables for b < kMfmaMinBatch, matrix cores above
constexpr int kMfmaMinBatch = 3;
int64_t gemv_mfma_workspace_bytes(int64_t k);
hipError_t launch_gemv_mfma_prepare(int64_t n, int64_t k, const uint16_t* x, int64_t b, float* y,
                                    void* ws, hipStream_t st);
hipError_t launch_gemv_mfma(int fmt, const uint8_t* codes, const uint16_t* scales, int64_t n,
                            int64_t k, int64_t b, float* y, const void* ws, int cus,
                            hipStream_t st);
// b >= kMfmaMinBatch, the decode FFN's gate+up GEMV: W x with x FP16
// [b][k] read in place (no prepare), stored as one FP32 [b][n] plane per
// K-piece (plain stores: nothing to zero) at hp; *planes receives the
// number of planes, at most gemv_mfma_max_planes(k)
int64_t gemv_mfma_max_planes(int64_t k);
hipError_t launch_gemv_mfma_planes(int fmt, const uint8_t* codes, const uint16_t* scales,
                                   int64_t n, int64_t k, int64_t b, const uint16_t* x, float* hp,
                                   int cus, int64_t* planes, hipStream_t st);
// ceiling probe: the matrix-core GEMV's per-row expansion and MFMA on
// register data (mode 0: expansion + MFMA, 1: the MFMA alone), `blocks` work-groups
// of 256 threads
hipError_t launch_probe_expand_mfma(int mode, int iters, int blocks, float* sink, hipStream_t st);
size_t gemv_workspace_bytes(int64_t k, int64_t b);
hipError_t launch_gemv_prepare(int64_t n, int64_t k, const uint16_t* x, int64_t b, float* y,
                               void* ws, hipStream_t st);
// b < kMfmaMinBatch, the decode FFN's table GEMVs.  gemv_partial_planes:
// the K-slices of the table GEMV for (k, b).  launch_gemv_partials: W x
// (x FP16 [b][k] read in place) as one FP32 [b][n] plane of partial sums
// per K-slice, hp = [gemv_partial_planes(k, b)][b][n], written with plain
// stores; the kernel also zeroes yz[0 .. yzn).  launch_gemv_accumulate_silu:
// y += W z with z = RNE_fp16(SiLU(gate) * up) formed inside the GEMV from
// h = the sum of the np planes at hp (FP32 [np][b][2k], gate columns then
// up columns).
int64_t gemv_partial_planes(int64_t k, int64_t b);
hipError_t launch_gemv_partials(int fmt, const uint8_t* codes, const uint16_t* scales, int64_t n,
                                int64_t k, int64_t b, const uint16_t* x, float* hp, float* yz,
                                int64_t yzn, hipStream_t st);
hipError_t launch_gemv_accumulate_silu(int fmt, const uint8_t* codes, const uint16_t* scales,
                                       int64_t n, int64_t k, int64_t b, float* y, const float* hp,
                                       int64_t np, hipStream_t st);
hipError_t launch_gemv_accumulate(int fmt, const uint8_t* codes, const uint16_t* scales,
                                  int64_t n, int64_t k, int64_t b, float* y, const void* ws,
                                  hipStream_t st);
// lowbit_gemv with its scratch in a static device array (no workspace):
// at most gemv_noalloc_scratch_bytes() of scratch, checked by the caller
size_t gemv_noalloc_scratch_bytes();
hipError_t launch_gemv_noalloc(int fmt, const uint8_t* codes, const uint16_t* scales, int64_t n,
                               int64_t k, const uint16_t* x, int64_t b, float* y,
                               hipStream_t st);

// decode FFN: SiLU(gate) * up -> FP16, and the whole gated-MLP chain
hipError_t launch_silu_mul(const float* h, int64_t f, int64_t b, uint16_t* z, hipStream_t st);
// Single-launch GEMV for small matrices (gemv_small.hip): y = W x written
// directly (no prepare, workspace or atomics) when gemv_direct_ok(n, k, b).
constexpr int64_t kDirectMaxWeights = (int64_t)32 << 20;
constexpr int64_t kDirectBatchWeight = 4;  // b >= 3: n * k * b <= 4 * kDirectMaxWeights
bool gemv_direct_ok(int64_t n, int64_t k, int64_t b);
hipError_t launch_gemv_direct(int fmt, const uint8_t* codes, const uint16_t* scales, int64_t n,
                              int64_t k, const uint16_t* x, int64_t b, float* y, hipStream_t st);
// the same with x = RNE_fp16(SiLU(gate) * up) formed from h = [gate | up]
// (FP32 [b][2f]); the matrix is n x f
hipError_t launch_gemv_direct_silu(int fmt, const uint8_t* codes, const uint16_t* scales,
                                   int64_t n, int64_t f, const float* h, int64_t b, float* y,
                                   hipStream_t st);
size_t ffn_workspace_bytes(int64_t k, int64_t f, int64_t b);
hipError_t launch_ffn(int fmt, const uint8_t* gu_codes, const uint16_t* gu_scales,
                      const uint8_t* dn_codes, const uint16_t* dn_scales, int64_t k, int64_t f,
                      const uint16_t* x, int64_t b, float* y, void* ws, hipStream_t st);

// the ends of a decode step: embedding-row gather, top-1 of the LM head
hipError_t launch_embed(int fmt, const uint8_t* codes, const uint16_t* scales, int64_t n,
                        int64_t k, const int32_t* ids, int64_t count, uint16_t* out,
                        hipStream_t st);
size_t argmax_workspace_bytes(int64_t n, int64_t b);
hipError_t launch_argmax(const float* y, int64_t n, int64_t b, int32_t* idx, float* val,
                         void* ws, hipStream_t st);
size_t lm_head_workspace_bytes(int64_t n, int64_t k, int64_t b);
hipError_t launch_lm_head(int fmt, const uint8_t* codes, const uint16_t* scales, int64_t n,
                          int64_t k, const uint16_t* x, int64_t b, float* y, int32_t* idx,
                          float* val, void* ws, hipStream_t st);

hipError_t launch_gemm(int fmt, const uint8_t* codes, const uint16_t* scales, int64_t n,
                       int64_t k, const uint16_t* x, int64_t m, void* y, bool out_f32,
                       hipStream_t st);

}  // namespace lowbit
