// C ABI of liblowbit.so: argument validation on the host, then kernel
// dispatch.  The contract of every entry point is in include/lowbit.h.
#include "../../include/lowbit.h"

#include "common.h"

#include <atomic>

namespace lowbit {

int device_cu_count() {
  // atomics: first calls may race from several host threads (they store the
  // same value)
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
      v = 256;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

}  // namespace lowbit

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 40;
constexpr int64_t kMaxK = int64_t(1) << 22;

bool fmt_ok(int fmt) { return fmt == LOWBIT_FMT_Q1_G128 || fmt == LOWBIT_FMT_T2_G128; }

bool shape_ok(int64_t n, int64_t k) {
  if (n < 1 || k < 128 || k % 128 != 0 || k > kMaxK) return false;
  if (n > kMaxElems / k) return false;
  return ((n + 15) / 16) < (int64_t(1) << 31);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t padded(int64_t n) { return (n + 15) / 16 * 16; }

int hip_status(hipError_t e) { return e == hipSuccess ? LOWBIT_OK : LOWBIT_ERR_HIP; }

}  // namespace

extern "C" {

int lowbit_version(void) { return 1; }

const char* lowbit_status_str(int status) {
  switch (status) {
    case LOWBIT_OK: return "ok";
    case LOWBIT_ERR_ARG: return "invalid argument (null pointer, format, batch or m)";
    case LOWBIT_ERR_SHAPE: return "invalid shape (n >= 1, k >= 128, k % 128 == 0, size limits)";
    case LOWBIT_ERR_ALIGN: return "pointer not 16-byte aligned";
    case LOWBIT_ERR_UNSUPPORTED: return "unsupported request";
    case LOWBIT_ERR_HIP: return "HIP launch failed";
    case LOWBIT_ERR_WORKSPACE: return "workspace missing or too small";
    case LOWBIT_ERR_SCRATCH: return "request needs more than the static scratch (1 MiB)";
    default: return "unknown status";
  }
}

size_t lowbit_codes_bytes(int fmt, int64_t n, int64_t k) {
  if (!fmt_ok(fmt) || !shape_ok(n, k)) return 0;
  return (size_t)(padded(n) * k / (fmt == LOWBIT_FMT_Q1_G128 ? 8 : 4));
}

size_t lowbit_scales_bytes(int fmt, int64_t n, int64_t k) {
  if (!fmt_ok(fmt) || !shape_ok(n, k)) return 0;
  return (size_t)(padded(n) * (k / 128) * 2);
}

int lowbit_quantize_q1(const uint16_t* w_fp16, int64_t n, int64_t k, void* codes,
                       uint16_t* scales, hipStream_t stream) {
  if (!w_fp16 || !codes || !scales) return LOWBIT_ERR_ARG;
  if (!shape_ok(n, k)) return LOWBIT_ERR_SHAPE;
  if (!aligned16(w_fp16) || !aligned16(codes) || !aligned16(scales)) return LOWBIT_ERR_ALIGN;
  return hip_status(lowbit::launch_quantize_q1(w_fp16, n, k, static_cast<uint8_t*>(codes),
                                               scales, stream));
}

int lowbit_pack_t2(const int8_t* t, const uint16_t* s_fp16, int64_t n, int64_t k, void* codes,
                   uint16_t* scales, hipStream_t stream) {
  if (!t || !s_fp16 || !codes || !scales) return LOWBIT_ERR_ARG;
  if (!shape_ok(n, k)) return LOWBIT_ERR_SHAPE;
  // t rows are read 8 bytes at a time; s is read element-wise
  if (!aligned16(t) || !aligned16(codes) || !aligned16(scales) ||
      (reinterpret_cast<uintptr_t>(s_fp16) & 1u))
    return LOWBIT_ERR_ALIGN;
  return hip_status(lowbit::launch_pack_t2(t, s_fp16, n, k, static_cast<uint8_t*>(codes), scales,
                                           stream));
}

int lowbit_pack(int fmt, const void* src, const uint16_t* src_scales, int64_t n, int64_t k,
                void* codes, uint16_t* scales, hipStream_t stream) {
  if (fmt == LOWBIT_FMT_Q1_G128) {
    if (src_scales) return LOWBIT_ERR_ARG;
    return lowbit_quantize_q1(static_cast<const uint16_t*>(src), n, k, codes, scales, stream);
  }
  if (fmt == LOWBIT_FMT_T2_G128)
    return lowbit_pack_t2(static_cast<const int8_t*>(src), src_scales, n, k, codes, scales,
                          stream);
  return LOWBIT_ERR_ARG;
}

int lowbit_unpack(int fmt, const void* codes, const uint16_t* scales, int64_t n, int64_t k,
                  uint16_t* w_fp16, hipStream_t stream) {
  if (!fmt_ok(fmt) || !codes || !scales || !w_fp16) return LOWBIT_ERR_ARG;
  if (!shape_ok(n, k)) return LOWBIT_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(w_fp16)) return LOWBIT_ERR_ALIGN;
  return hip_status(lowbit::launch_unpack(fmt, static_cast<const uint8_t*>(codes), scales, n, k,
                                          w_fp16, stream));
}

size_t lowbit_gemv_workspace_bytes(int fmt, int64_t n, int64_t k, int64_t b) {
  if (!fmt_ok(fmt) || !shape_ok(n, k) || b < 1 || b > 8) return 0;
  return lowbit::gemv_workspace_bytes(k, b);
}

int lowbit_gemv_prepare(int64_t n, int64_t k, const uint16_t* x_fp16, int64_t b, float* y_f32,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!x_fp16 || !y_f32) return LOWBIT_ERR_ARG;
  if (b < 1 || b > 8) return LOWBIT_ERR_ARG;
  if (!shape_ok(n, k)) return LOWBIT_ERR_SHAPE;
  if (!aligned16(x_fp16) || !aligned16(y_f32)) return LOWBIT_ERR_ALIGN;
  if (!workspace || workspace_bytes < lowbit::gemv_workspace_bytes(k, b))
    return LOWBIT_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LOWBIT_ERR_ALIGN;
  return hip_status(lowbit::launch_gemv_prepare(n, k, x_fp16, b, y_f32, workspace, stream));
}

int lowbit_gemv_accumulate(int fmt, const void* codes, const uint16_t* scales, int64_t n,
                           int64_t k, int64_t b, float* y_f32, const void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  if (!fmt_ok(fmt) || !codes || !scales || !y_f32) return LOWBIT_ERR_ARG;
  if (b < 1 || b > 8) return LOWBIT_ERR_ARG;
  if (!shape_ok(n, k)) return LOWBIT_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(y_f32)) return LOWBIT_ERR_ALIGN;
  if (!workspace || workspace_bytes < lowbit::gemv_workspace_bytes(k, b))
    return LOWBIT_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LOWBIT_ERR_ALIGN;
  return hip_status(lowbit::launch_gemv_accumulate(fmt, static_cast<const uint8_t*>(codes),
                                                   scales, n, k, b, y_f32, workspace, stream));
}

int lowbit_gemv(int fmt, const void* codes, const uint16_t* scales, int64_t n, int64_t k,
                const uint16_t* x_fp16, int64_t b, float* y_f32, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  if (!fmt_ok(fmt) || !codes || !scales || !x_fp16 || !y_f32) return LOWBIT_ERR_ARG;
  if (b < 1 || b > 8) return LOWBIT_ERR_ARG;
  if (!shape_ok(n, k)) return LOWBIT_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(x_fp16) || !aligned16(y_f32))
    return LOWBIT_ERR_ALIGN;
  if (!workspace || workspace_bytes < lowbit::gemv_workspace_bytes(k, b))
    return LOWBIT_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LOWBIT_ERR_ALIGN;
  // small matrices: one kernel writes y (the workspace is not touched)
  if (lowbit::gemv_direct_ok(n, k, b))
    return hip_status(lowbit::launch_gemv_direct(fmt, static_cast<const uint8_t*>(codes), scales,
                                                 n, k, x_fp16, b, y_f32, stream));
  const int st = lowbit_gemv_prepare(n, k, x_fp16, b, y_f32, workspace, workspace_bytes, stream);
  if (st != LOWBIT_OK) return st;
  return lowbit_gemv_accumulate(fmt, codes, scales, n, k, b, y_f32, workspace, workspace_bytes,
                                stream);
}

int lowbit_gemv_noalloc(int fmt, const void* codes, const uint16_t* scales, int64_t n,
                        int64_t k, const uint16_t* x_fp16, int64_t b, float* y_f32,
                        hipStream_t stream) {
  if (!fmt_ok(fmt) || !codes || !scales || !x_fp16 || !y_f32) return LOWBIT_ERR_ARG;
  if (b < 1 || b > 8) return LOWBIT_ERR_ARG;
  if (!shape_ok(n, k)) return LOWBIT_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(x_fp16) || !aligned16(y_f32))
    return LOWBIT_ERR_ALIGN;
  if (lowbit::gemv_workspace_bytes(k, b) > lowbit::gemv_noalloc_scratch_bytes())
    return LOWBIT_ERR_SCRATCH;
  return hip_status(lowbit::launch_gemv_noalloc(fmt, static_cast<const uint8_t*>(codes), scales,
                                                n, k, x_fp16, b, y_f32, stream));
}

static int gemm_common(int fmt, const void* codes, const uint16_t* scales, int64_t n, int64_t k,
                       const uint16_t* x_bf16, int64_t m, void* y, bool out_f32,
                       hipStream_t stream) {
  if (!fmt_ok(fmt) || !codes || !scales || !x_bf16 || !y) return LOWBIT_ERR_ARG;
  if (m < 1 || m > (int64_t(1) << 22)) return LOWBIT_ERR_ARG;
  if (!shape_ok(n, k)) return LOWBIT_ERR_SHAPE;
  if (m > kMaxElems / k || m > kMaxElems / n) return LOWBIT_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(x_bf16) || !aligned16(y))
    return LOWBIT_ERR_ALIGN;
  return hip_status(lowbit::launch_gemm(fmt, static_cast<const uint8_t*>(codes), scales, n, k,
                                        x_bf16, m, y, out_f32, stream));
}

int lowbit_gemm(int fmt, const void* codes, const uint16_t* scales, int64_t n, int64_t k,
                const uint16_t* x_bf16, int64_t m, uint16_t* y_bf16, hipStream_t stream) {
  return gemm_common(fmt, codes, scales, n, k, x_bf16, m, y_bf16, false, stream);
}

int lowbit_gemm_f32(int fmt, const void* codes, const uint16_t* scales, int64_t n, int64_t k,
                    const uint16_t* x_bf16, int64_t m, float* y_f32, hipStream_t stream) {
  return gemm_common(fmt, codes, scales, n, k, x_bf16, m, y_f32, true, stream);
}

int lowbit_silu_mul(const float* h_f32, int64_t f, int64_t b, uint16_t* z_fp16,
                    hipStream_t stream) {
  if (!h_f32 || !z_fp16) return LOWBIT_ERR_ARG;
  if (b < 1 || b > (int64_t(1) << 20)) return LOWBIT_ERR_ARG;
  if (f < 8 || f % 8 != 0 || f > kMaxElems / (2 * b)) return LOWBIT_ERR_SHAPE;
  if (!aligned16(h_f32) || !aligned16(z_fp16)) return LOWBIT_ERR_ALIGN;
  return hip_status(lowbit::launch_silu_mul(h_f32, f, b, z_fp16, stream));
}

size_t lowbit_ffn_workspace_bytes(int fmt, int64_t k, int64_t f, int64_t b) {
  if (!fmt_ok(fmt) || f < 1 || f > kMaxElems || !shape_ok(2 * f, k) || !shape_ok(k, f) ||
      b < 1 || b > 8)
    return 0;
  return lowbit::ffn_workspace_bytes(k, f, b);
}

int lowbit_ffn(int fmt, const void* gu_codes, const uint16_t* gu_scales, const void* dn_codes,
               const uint16_t* dn_scales, int64_t k, int64_t f, const uint16_t* x_fp16,
               int64_t b, float* y_f32, void* workspace, size_t workspace_bytes,
               hipStream_t stream) {
  if (!fmt_ok(fmt) || !gu_codes || !gu_scales || !dn_codes || !dn_scales || !x_fp16 || !y_f32)
    return LOWBIT_ERR_ARG;
  if (b < 1 || b > 8) return LOWBIT_ERR_ARG;
  if (f < 1 || f > kMaxElems || !shape_ok(2 * f, k) || !shape_ok(k, f)) return LOWBIT_ERR_SHAPE;
  if (!aligned16(gu_codes) || !aligned16(gu_scales) || !aligned16(dn_codes) ||
      !aligned16(dn_scales) || !aligned16(x_fp16) || !aligned16(y_f32))
    return LOWBIT_ERR_ALIGN;
  if (!workspace || workspace_bytes < lowbit::ffn_workspace_bytes(k, f, b))
    return LOWBIT_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LOWBIT_ERR_ALIGN;
  return hip_status(lowbit::launch_ffn(fmt, static_cast<const uint8_t*>(gu_codes), gu_scales,
                                       static_cast<const uint8_t*>(dn_codes), dn_scales, k, f,
                                       x_fp16, b, y_f32, workspace, stream));
}

int lowbit_embed(int fmt, const void* codes, const uint16_t* scales, int64_t n, int64_t k,
                 const int32_t* ids, int64_t count, uint16_t* out_fp16, hipStream_t stream) {
  if (!fmt_ok(fmt) || !codes || !scales || !ids || !out_fp16) return LOWBIT_ERR_ARG;
  if (count < 1 || count > (int64_t(1) << 31) - 1) return LOWBIT_ERR_ARG;
  if (!shape_ok(n, k) || n > (int64_t(1) << 31) - 1) return LOWBIT_ERR_SHAPE;
  if (count > kMaxElems / k) return LOWBIT_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(out_fp16) || (reinterpret_cast<uintptr_t>(scales) & 1u) ||
      (reinterpret_cast<uintptr_t>(ids) & 3u))
    return LOWBIT_ERR_ALIGN;
  return hip_status(lowbit::launch_embed(fmt, static_cast<const uint8_t*>(codes), scales, n, k,
                                         ids, count, out_fp16, stream));
}

size_t lowbit_argmax_workspace_bytes(int64_t n, int64_t b) {
  if (n < 1 || n > (int64_t(1) << 31) - 1 || b < 1 || b > 65535) return 0;
  return lowbit::argmax_workspace_bytes(n, b);
}

int lowbit_argmax(const float* y_f32, int64_t n, int64_t b, int32_t* idx_out, float* val_out,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!y_f32 || !idx_out) return LOWBIT_ERR_ARG;
  if (b < 1 || b > 65535) return LOWBIT_ERR_ARG;
  if (n < 1 || n > (int64_t(1) << 31) - 1 || n > kMaxElems / b) return LOWBIT_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(y_f32) & 3u) || (reinterpret_cast<uintptr_t>(idx_out) & 3u) ||
      (reinterpret_cast<uintptr_t>(val_out) & 3u))
    return LOWBIT_ERR_ALIGN;
  if (!workspace || workspace_bytes < lowbit::argmax_workspace_bytes(n, b))
    return LOWBIT_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LOWBIT_ERR_ALIGN;
  return hip_status(lowbit::launch_argmax(y_f32, n, b, idx_out, val_out, workspace, stream));
}

size_t lowbit_lm_head_workspace_bytes(int fmt, int64_t n, int64_t k, int64_t b) {
  if (!fmt_ok(fmt) || !shape_ok(n, k) || n > (int64_t(1) << 31) - 1 || b < 1 || b > 8) return 0;
  return lowbit::lm_head_workspace_bytes(n, k, b);
}

int lowbit_lm_head(int fmt, const void* codes, const uint16_t* scales, int64_t n, int64_t k,
                   const uint16_t* x_fp16, int64_t b, float* y_f32, int32_t* idx_out,
                   float* val_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!fmt_ok(fmt) || !codes || !scales || !x_fp16 || !y_f32 || !idx_out) return LOWBIT_ERR_ARG;
  if (b < 1 || b > 8) return LOWBIT_ERR_ARG;
  if (!shape_ok(n, k) || n > (int64_t(1) << 31) - 1) return LOWBIT_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(x_fp16) || !aligned16(y_f32) ||
      (reinterpret_cast<uintptr_t>(idx_out) & 3u) || (reinterpret_cast<uintptr_t>(val_out) & 3u))
    return LOWBIT_ERR_ALIGN;
  if (!workspace || workspace_bytes < lowbit::lm_head_workspace_bytes(n, k, b))
    return LOWBIT_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LOWBIT_ERR_ALIGN;
  return hip_status(lowbit::launch_lm_head(fmt, static_cast<const uint8_t*>(codes), scales, n, k,
                                           x_fp16, b, y_f32, idx_out, val_out, workspace,
                                           stream));
}

int lowbit_quantize_t2(const uint16_t* w_fp16, int64_t n, int64_t k, void* codes,
                       uint16_t* scales, hipStream_t stream) {
  if (!w_fp16 || !codes || !scales) return LOWBIT_ERR_ARG;
  if (!shape_ok(n, k)) return LOWBIT_ERR_SHAPE;
  if (!aligned16(w_fp16) || !aligned16(codes) || !aligned16(scales)) return LOWBIT_ERR_ALIGN;
  return hip_status(lowbit::launch_quantize_t2(w_fp16, n, k, static_cast<uint8_t*>(codes),
                                               scales, stream));
}

size_t lowbit_base3_bytes(int64_t n, int64_t k) {
  if (!shape_ok(n, k)) return 0;
  return (size_t)(n * ((k + 4) / 5));
}

int lowbit_t2_to_base3(const void* codes, const uint16_t* scales, int64_t n, int64_t k,
                       uint8_t* base3_out, uint16_t* scales_out, hipStream_t stream) {
  if (!codes || !scales || !base3_out || !scales_out) return LOWBIT_ERR_ARG;
  if (!shape_ok(n, k)) return LOWBIT_ERR_SHAPE;
  if (!aligned16(codes) || (reinterpret_cast<uintptr_t>(scales) & 1u) ||
      (reinterpret_cast<uintptr_t>(scales_out) & 1u))
    return LOWBIT_ERR_ALIGN;
  return hip_status(lowbit::launch_t2_to_base3(static_cast<const uint8_t*>(codes), scales, n, k,
                                               base3_out, scales_out, stream));
}

int lowbit_base3_to_t2(const uint8_t* base3, const uint16_t* scales_rm, int64_t n, int64_t k,
                       void* codes, uint16_t* scales, hipStream_t stream) {
  if (!base3 || !scales_rm || !codes || !scales) return LOWBIT_ERR_ARG;
  if (!shape_ok(n, k)) return LOWBIT_ERR_SHAPE;
  if (!aligned16(codes) || (reinterpret_cast<uintptr_t>(scales) & 1u) ||
      (reinterpret_cast<uintptr_t>(scales_rm) & 1u))
    return LOWBIT_ERR_ALIGN;
  return hip_status(lowbit::launch_base3_to_t2(base3, scales_rm, n, k,
                                               static_cast<uint8_t*>(codes), scales, stream));
}

}  // extern "C"
