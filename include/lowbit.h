/*
 * lowbit.h -- C ABI of the group-scaled 1-bit / ternary y = W.x library for
 * AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page title and section; the method is described only in
 * prose on these pages, and no code or API is given there):
 *   [P1] 7minutos.es, "Un tutorial de codificacion para ejecutar PrismML Bonsai
 *        1-bit LLM en CUDA con GGUF", section 7 "Q1_0_g128 Cuantizacion"
 *        (the representation box and the Python demonstration of the rule).
 *   [P2] 7minutos.es, "PrismML lanza Bonsai 27B: compilaciones ternarias y de
 *        1 bit de Qwen3.6-27B", sections "Como funciona la compresion" and
 *        "Rendimiento y decodificacion especulativa DSpark".
 *   [P3] kerneldigest.dev, "Bonsai 2 27B y la densidad de inteligencia",
 *        section "Arquitectura del Sistema".
 *   [P4] es.news.hada.io topic 31450, "Bonsai 27B: un modelo de clase 27B que
 *        corre en un telefono", section "Configuracion multimodal y de bajo bit
 *        de extremo a extremo" and the reader comments.
 *
 * ---------------------------------------------------------------------------
 * THE TWO WEIGHT CODES
 *
 *   Q1_0_g128 [P1 s.7]: every weight is one bit; bit 0 stands for -s and bit 1
 *     for +s, where s is an FP16 scale shared by 128 consecutive weights.
 *     Quantisation from FP16: s = max |w| over the 128 weights of the group and
 *     bit = 1 when w >= 0, else 0.  1 + 16/128 = 1.125 bits per weight.
 *   Ternary g128 [P2 "Como funciona la compresion", P3]: w = s * t with
 *     t in {-1, 0, +1} and one FP16 scale s per 128 consecutive weights.  The
 *     pages count log2(3) bits per weight; this library stores two bits per
 *     weight ("four values of four states" per byte, [P4 comments]):
 *     2 + 16/128 = 2.125 bits per weight.
 *
 * The group of 128 runs along K, the reduction axis: W is logical [N][K] and
 * group g of row n holds k in [128 g, 128 g + 128).  K must be a multiple of
 * 128.  The pages do not fix a bit order or byte layout; this library defines
 * its own, below.  Both codes keep the pages' per-group byte count:
 * 16 code bytes + 2 scale bytes = 18 B per Q1 group, 32 + 2 = 34 B per
 * ternary group (stored as two separate planes, codes and scales).
 *
 * ---------------------------------------------------------------------------
 * BYTE LAYOUT (version 1)
 *
 *   Np      = N rounded up to a multiple of 16 (rows are stored in tiles of 16)
 *   tile    = n / 16, r = n % 16   (row tile and row within the tile)
 *   c       = k / 8                (8-weight chunk), j = k % 8 (bit in byte)
 *   G       = K / 128, g = k / 128 (group)
 *
 *   Q1 codes:  Np*K/8 bytes.  The bit of weight (n,k) is bit j (value 1<<j) of
 *              byte  (tile*(K/8) + c)*16 + r.
 *              A 16-byte "cell" holds one 8-weight chunk of 16 rows.
 *   T2 codes:  Np*K/4 bytes, 32-byte cells.  For weight (n,k):
 *                pos bit = bit j of byte (tile*(K/8) + c)*32 + r
 *                neg bit = bit j of byte (tile*(K/8) + c)*32 + 16 + r
 *              t = pos - neg  (so pos=neg=1 decodes as 0; packers never
 *              write that pattern).
 *   scales:    Np*G FP16 values (2 bytes each).  The scale of (n, g) is
 *              element (tile*G + g)*16 + r.
 *   Pad rows (N <= n < Np) hold zero codes and zero scales; they are written
 *   by the packers and never read into an output.
 *
 * ---------------------------------------------------------------------------
 * CONVENTIONS FOR EVERY ENTRY POINT
 *
 *   - Pointers are HIP device pointers unless stated otherwise; the caller
 *     allocates and frees every buffer.  The library never allocates,
 *     frees or synchronises, and keeps no state between calls (apart from
 *     lowbit_gemv_noalloc's static scratch, below).
 *   - Outputs that kernels accumulate with FP32 atomic adds -- y of
 *     lowbit_gemv, lowbit_gemv_accumulate, lowbit_gemv_noalloc, lowbit_ffn
 *     and lowbit_lm_head,
 *     and the FFN's h in its workspace -- must be coarse-grained device
 *     memory (hipMalloc, or torch's CUDA allocator).  The library is built
 *     with -munsafe-fp-atomics: on fine-grained or host-coherent memory
 *     such adds may be lost.
 *   - FP16 and BF16 values are passed as their 16-bit patterns (uint16_t).
 *   - Every call validates its arguments on the host, then enqueues its
 *     kernels on `stream` and returns without waiting.  On a validation
 *     error nothing is launched and the return value says why.  A failed
 *     launch returns LOWBIT_ERR_HIP.  Faults during execution surface at the
 *     caller's next synchronisation.
 *   - Shapes: n >= 1, k >= 128 and k % 128 == 0, n*k < 2^40; GEMV batch
 *     1 <= b <= 8; GEMM m >= 1.
 *   - Alignment: codes, scales, x, y, w and workspace pointers must be 16-byte
 *     aligned (torch's allocator gives 256).
 *   - Buffers of one call must not overlap, except that read-only inputs may
 *     alias each other.  Calls on different streams that share an output or
 *     a workspace race.
 *   - No C++ exception crosses this interface.
 */
#ifndef LOWBIT_H
#define LOWBIT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LOWBIT_FMT_Q1_G128 = 1, /* 1-bit codes, bit 1 -> +s, bit 0 -> -s  [P1 s.7] */
  LOWBIT_FMT_T2_G128 = 2  /* ternary codes t = pos - neg, w = s*t   [P2, P3]   */
} lowbit_fmt;

typedef enum {
  LOWBIT_OK = 0,
  LOWBIT_ERR_ARG = 1,         /* null pointer, unknown format, bad batch/m   */
  LOWBIT_ERR_SHAPE = 2,       /* n < 1, k % 128 != 0, size too large          */
  LOWBIT_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned             */
  LOWBIT_ERR_UNSUPPORTED = 4, /* valid request this build does not implement */
  LOWBIT_ERR_HIP = 5,         /* a HIP call or kernel launch failed           */
  LOWBIT_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required  */
  LOWBIT_ERR_SCRATCH = 7      /* needs more than lowbit_gemv_noalloc's scratch */
} lowbit_status;

/* Library ABI version (this header describes version 1). */
int lowbit_version(void);

/* Human-readable name of a status code; never NULL. */
const char* lowbit_status_str(int status);

/* Bytes of the code plane / scale plane for an n x k matrix in `fmt`
 * [P1 s.7: one bit per weight and one FP16 scale per 128 weights, 18 B per
 * group; P2 "Como funciona la compresion": ternary codes with one FP16
 * scale per group of 128, here two bits per weight, 34 B per group].
 * Q1: Np*k/8, T2: Np*k/4, scales: Np*(k/128)*2, with Np = n rounded up to 16.
 * Returns 0 for an invalid format or shape.  Host-only; touches no GPU. */
size_t lowbit_codes_bytes(int fmt, int64_t n, int64_t k);
size_t lowbit_scales_bytes(int fmt, int64_t n, int64_t k);

/* Q1 quantise + pack  [P1 s.7: scale = max|w| per 128, bit = 1 iff w >= 0].
 *   w_fp16 : [n][k] row-major FP16 weights (device, read-only).
 *   codes  : lowbit_codes_bytes(Q1, n, k) bytes (device, written).
 *   scales : lowbit_scales_bytes(Q1, n, k) bytes (device, written).
 * Exact integer rules on the FP16 bit pattern h (mag = h & 0x7FFF):
 *   s = max over the group of mag (as an FP16 pattern with sign 0): this is
 *       max|w| for finite/infinite input; a group holding a NaN gets the NaN
 *       pattern of largest magnitude bits.
 *   bit = 1 iff the IEEE comparison w >= 0 holds: +0 and -0 give 1, every NaN
 *       gives 0.  Subnormals are handled exactly (no flush to zero). */
int lowbit_quantize_q1(const uint16_t* w_fp16, int64_t n, int64_t k,
                       void* codes, uint16_t* scales, hipStream_t stream);

/* Ternary pack  [P2 "Como funciona la compresion": w = s_g * t_i].
 *   t      : [n][k] row-major int8 (device, read-only); the stored code is
 *            sign(t), so values outside {-1,0,1} are clamped by their sign.
 *   s_fp16 : [n][k/128] row-major FP16 group scales (device, read-only),
 *            copied bit for bit.
 *   codes, scales : as for lowbit_quantize_q1, in the T2 layout. */
int lowbit_pack_t2(const int8_t* t, const uint16_t* s_fp16, int64_t n,
                   int64_t k, void* codes, uint16_t* scales,
                   hipStream_t stream);

/* Generic pack entry  [P1 s.7 for Q1, P2 "Como funciona la compresion" for
 * ternary]: Q1 -> lowbit_quantize_q1(src as FP16, src_scales must be NULL);
 * T2 -> lowbit_pack_t2(src as int8, src_scales as FP16).  Same arguments,
 * layouts and errors as the call it forwards to. */
int lowbit_pack(int fmt, const void* src, const uint16_t* src_scales,
                int64_t n, int64_t k, void* codes, uint16_t* scales,
                hipStream_t stream);

/* Unpack / dequantise to dense FP16 [P1 s.7 dequantisation rule, P2].
 *   w_fp16 : [n][k] row-major FP16 output (device, written).
 * Q1: bit 1 -> s, bit 0 -> s with its sign bit flipped (-s).
 * T2: t = +1 -> s, t = -1 -> s with its sign bit flipped, t = 0 -> +0.0.
 * Every output value is exact (a copy of s or of its negation). */
int lowbit_unpack(int fmt, const void* codes, const uint16_t* scales,
                  int64_t n, int64_t k, uint16_t* w_fp16, hipStream_t stream);

/* Ternary quantiser  [P2 "Como funciona la compresion": w = s t, t in
 * {-1, 0, +1}, one FP16 scale per 128].  The pages give no rounding rule;
 * this library's: s = max |w| of each group of 128 (as the 1-bit worked
 * example), and t = sign(w) if 2|w| > s, else 0 -- the nearest of
 * {-1, 0, +1} to w / s, ties to 0 (a NaN weight, or a group whose maximum
 * is NaN or infinite, gives t = 0 except for 2|w| > s).
 *   w_fp16 : [n][k] row-major FP16 (device, read-only)
 *   codes  : lowbit_codes_bytes(T2, n, k) bytes, scales : [padded n][k/128]
 *            (device, written; layout v1, as lowbit_pack_t2 writes them). */
int lowbit_quantize_t2(const uint16_t* w_fp16, int64_t n, int64_t k, void* codes,
                       uint16_t* scales, hipStream_t stream);

/* Base-3 storage of ternary codes  [P2: log2(3) + 16/128 ~ 1.71 bits per
 * weight is the bound]: five trits per byte, byte = sum_i (t_i + 1) 3^i
 * for the weights 5j + i of a row, ceil(k/5) bytes per row, rows one after
 * another, positions past k holding t = 0; scales row-major [n][k/128].
 * 8/5 + 16/128 = 1.725 bits per weight.  A storage format: the GEMV and
 * GEMM read the two-plane codes, to and from which these calls convert. */
size_t lowbit_base3_bytes(int64_t n, int64_t k);   /* n * ceil(k/5); 0 on a bad shape */
int lowbit_t2_to_base3(const void* codes, const uint16_t* scales, int64_t n, int64_t k,
                       uint8_t* base3_out, uint16_t* scales_out, hipStream_t stream);
/* Inverse; a byte of 243..255 (never written above) decodes with its fifth
 * digit taken mod 3.  Rows of the last tile past n get zero codes and
 * scales. */
int lowbit_base3_to_t2(const uint8_t* base3, const uint16_t* scales_rm, int64_t n, int64_t k,
                       void* codes, uint16_t* scales, hipStream_t stream);

/* Workspace bytes lowbit_gemv needs for (fmt, n, k, b); 0 on a bad shape. */
size_t lowbit_gemv_workspace_bytes(int fmt, int64_t n, int64_t k, int64_t b);

/* GEMV phase 1: from x alone, prepare what lowbit_gemv_accumulate reads, and
 * set y to zero.  For b <= 2 that is a copy of x (each work-group of the
 * accumulate kernel builds its subset-sum tables -- one entry per signed
 * sum of 8 activations -- from it in LDS); for b >= 3 it is x laid out as
 * matrix-core operands (batch rows padded to 16 with zeros).
 *   x_fp16    : [b][k] row-major FP16 activations (device, read-only)
 *   y_f32     : [b][n] row-major FP32 (device, written with zeros)
 *   workspace : at least lowbit_gemv_workspace_bytes(fmt, n, k, b) bytes
 *               (device, written; its contents do not depend on fmt).
 * Several matrices that share x and k (e.g. gate and up projections) may be
 * accumulated from one prepared workspace. */
int lowbit_gemv_prepare(int64_t n, int64_t k, const uint16_t* x_fp16, int64_t b,
                        float* y_f32, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/* GEMV phase 2: y += W.x using what lowbit_gemv_prepare left in the
 * workspace (same k and b).  This is the kernel that streams the weights.
 * Different K-slices of a row are added to y with FP32 atomic adds. */
int lowbit_gemv_accumulate(int fmt, const void* codes, const uint16_t* scales,
                           int64_t n, int64_t k, int64_t b, float* y_f32,
                           const void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Decode GEMV  [P2 "Rendimiento ...": decode streams every low-bit matrix once
 * per token; P4: embeddings, attention, MLP and LM head are all low-bit].
 *   y[i][n] = sum_g s[n][g] * sum_{k in g} t[n][k] * x[i][k],  0 <= i < b
 *   x_fp16    : [b][k] row-major FP16 activations (device, read-only)
 *   y_f32     : [b][n] row-major FP32 output (device, written)
 *   workspace : at least lowbit_gemv_workspace_bytes(fmt, n, k, b) bytes of
 *               device scratch, contents ignored on entry and clobbered.
 * Equivalent to lowbit_gemv_prepare followed by lowbit_gemv_accumulate,
 * except for small matrices (k <= 8192 at b = 1, k <= 4096 at b >= 2, and
 * n * k <= 2^25 weights at b <= 2 or n * k * b <= 2^27 at b >= 3): those
 * take one kernel in which a work-group owns whole rows and stores y
 * directly (no atomics; the workspace is then not touched).  Accumulates in FP32; the summation order is not specified and,
 * where K-slices are combined with atomic adds, may differ from run to run
 * in the last bits. */
int lowbit_gemv(int fmt, const void* codes, const uint16_t* scales,
                int64_t n, int64_t k, const uint16_t* x_fp16, int64_t b,
                float* y_f32, void* workspace, size_t workspace_bytes,
                hipStream_t stream);

/* Decode GEMV that allocates nothing, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, result and errors as
 * lowbit_gemv without the workspace: the scratch lowbit_gemv keeps in the
 * workspace lives in a static device array of 1 MiB per GPU, held until
 * the process ends, so the call needs
 *     lowbit_gemv_workspace_bytes(fmt, n, k, b) <= 1 MiB
 * (b <= 2: 2*b*k bytes, k <= 262144 at b = 2; b >= 3: 32*k bytes,
 * k <= 32768) and returns LOWBIT_ERR_SCRATCH, launching nothing, beyond
 * that.  It calls no allocator.  Every call on one GPU uses the same array:
 * calls that overlap on one GPU (other streams, other host threads) race;
 * calls ordered on one stream do not.  Nothing in the array needs to start
 * at zero (the first kernel writes what the second reads, and zeroes y).
 * The small matrices that lowbit_gemv runs in one kernel use no scratch.
 * The array's device address is looked up once per device, on the first
 * call made with that device current. */
int lowbit_gemv_noalloc(int fmt, const void* codes, const uint16_t* scales,
                        int64_t n, int64_t k, const uint16_t* x_fp16, int64_t b,
                        float* y_f32, hipStream_t stream);

/* Prefill GEMM  [P2 "Rendimiento ...": prefill is compute-bound].
 *   Y[i][n] = RNE_bf16( sum_g s[n][g] * sum_{k in g} X[i][k] * t[n][k] )
 *   x_bf16 : [m][k] row-major BF16 (device, read-only)
 *   y_bf16 : [m][n] row-major BF16 (device, written)
 * Codes are expanded to exact BF16 {-1,0,+1}, contracted on matrix cores in
 * FP32, and each 128-wide group's partial is multiplied by its scale in FP32
 * before accumulation; the single rounding to BF16 happens at the store. */
int lowbit_gemm(int fmt, const void* codes, const uint16_t* scales,
                int64_t n, int64_t k, const uint16_t* x_bf16, int64_t m,
                uint16_t* y_bf16, hipStream_t stream);

/* Same contraction as lowbit_gemm with the FP32 sum stored unrounded:
 *   y_f32 : [m][n] row-major FP32 (device, written). */
int lowbit_gemm_f32(int fmt, const void* codes, const uint16_t* scales,
                    int64_t n, int64_t k, const uint16_t* x_bf16, int64_t m,
                    float* y_f32, hipStream_t stream);

/* SiLU-gated product of a decode FFN  [P2 "Como funciona la compresion":
 * the MLP projections are low-bit; P5 "Detalles tecnicos": decode kernels
 * were tuned at the FFN level.  The gated MLP form is that of the Qwen
 * family the models derive from; the pages do not spell it out.]
 *   z[i][j] = RNE_fp16( SiLU(h[i][j]) * h[i][f + j] ),  0 <= j < f, 0 <= i < b
 *   h_f32  : [b][2f] row-major FP32 (device, read-only): columns 0..f-1 the
 *            gate projection, f..2f-1 the up projection
 *   z_fp16 : [b][f] row-major FP16 (device, written)
 * SiLU(v) = v / (1 + e^-v) is evaluated in FP32 with the device expf; the
 * FP32 product is rounded to FP16 (nearest-even; beyond the FP16 range it
 * becomes +-inf; a zero keeps the IEEE sign of the product, e.g. -0 for
 * v < -88 and u > 0, where e^-v overflows and SiLU(v) = -0).
 * f must be a multiple of 8. */
int lowbit_silu_mul(const float* h_f32, int64_t f, int64_t b, uint16_t* z_fp16,
                    hipStream_t stream);

/* Workspace bytes lowbit_ffn needs for (fmt, k, f, b); 0 on a bad shape. */
size_t lowbit_ffn_workspace_bytes(int fmt, int64_t k, int64_t f, int64_t b);

/* Decode FFN (gated MLP) on one activation batch, as one stream-ordered
 * chain (no host synchronisation; it may be captured in a HIP graph):
 *   h = W_gu x               W_gu: [2f][k] codes + scales (gate rows 0..f-1,
 *                                  up rows f..2f-1), the lowbit_gemv kernels
 *   z = lowbit_silu_mul(h)   FP16 [b][f]
 *   y = W_dn z               W_dn: [k][f] codes + scales (k outputs)
 *   x_fp16    : [b][k] FP16 (device, read-only), 1 <= b <= 8
 *   y_f32     : [b][k] FP32 (device, written)
 *   workspace : at least lowbit_ffn_workspace_bytes(fmt, k, f, b) bytes of
 *               device scratch, contents ignored on entry and clobbered.
 * When both matrices are within lowbit_gemv's single-kernel limits the
 * chain is two kernels, the second forming z itself.  Otherwise, for
 * b <= 2, it is two kernels too: the gate+up GEMV stores the partial sums
 * of each of its K-slices (no atomics; it also zeroes y) and the down GEMV
 * adds them up in a fixed order and forms z inside its own table build;
 * for b >= 3, z is formed by a launch of its own.  z is never written out
 * except by that launch, and always with the arithmetic of
 * lowbit_silu_mul.
 * Both matrices use format fmt; k and f must be multiples of 128.  As in
 * lowbit_gemv, the down GEMV's K-slices are combined with atomic adds on
 * the larger shapes (and, for b >= 3, the gate+up GEMV's too), so the last
 * bits of y may differ from run to run, and for b >= 3 those of h, and so
 * may a z value that lies on an FP16 rounding boundary. */
int lowbit_ffn(int fmt, const void* gu_codes, const uint16_t* gu_scales,
               const void* dn_codes, const uint16_t* dn_scales, int64_t k, int64_t f,
               const uint16_t* x_fp16, int64_t b, float* y_f32, void* workspace,
               size_t workspace_bytes, hipStream_t stream);

/* Embedding-row gather  [P2 "Como funciona la compresion", P4: the
 * embeddings are low-bit too]: the rows ids[0..count) of W [n][k], each
 * dequantised exactly as lowbit_unpack does (+s, -s, or +0 for a ternary
 * zero).
 *   ids      : [count] int32 row indices (device, read-only); an id outside
 *              [0, n) gives a row of zeros (ids are not checked on the host)
 *   out_fp16 : [count][k] row-major FP16 (device, written) */
int lowbit_embed(int fmt, const void* codes, const uint16_t* scales, int64_t n, int64_t k,
                 const int32_t* ids, int64_t count, uint16_t* out_fp16, hipStream_t stream);

/* Workspace bytes lowbit_argmax needs for (n, b); 0 on a bad shape. */
size_t lowbit_argmax_workspace_bytes(int64_t n, int64_t b);

/* Top-1 of each row of y  [P5 "Detalles tecnicos": decode is checked by
 * top-1 token match].
 *   y_f32   : [b][n] FP32 (device, read-only), n < 2^31, b <= 65535
 *   idx_out : [b] int32 (device, written): the index of the largest value;
 *             among equal values the lowest index; a NaN counts as larger
 *             than every number (as numpy's and torch's argmax do); -0 and
 *             +0 are equal
 *   val_out : [b] FP32 (device, written) y at that index, or NULL
 * Two launches (per-part maxima into the workspace, then one work-group
 * per row); the workspace contents are ignored on entry. */
int lowbit_argmax(const float* y_f32, int64_t n, int64_t b, int32_t* idx_out, float* val_out,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes lowbit_lm_head needs for (fmt, n, k, b); 0 on a bad shape. */
size_t lowbit_lm_head_workspace_bytes(int fmt, int64_t n, int64_t k, int64_t b);

/* LM head with its top-1 token: lowbit_gemv followed by lowbit_argmax on the
 * same stream, one workspace for both.
 *   y_f32   : [b][n] FP32 logits (device, written)
 *   idx_out : [b] int32, val_out : [b] FP32 or NULL (device, written)
 * Because the GEMV's K-slices are combined with atomic adds, two logits
 * that differ by less than its rounding error may come out in either
 * order from run to run. */
int lowbit_lm_head(int fmt, const void* codes, const uint16_t* scales, int64_t n, int64_t k,
                   const uint16_t* x_fp16, int64_t b, float* y_f32, int32_t* idx_out,
                   float* val_out, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LOWBIT_H */
