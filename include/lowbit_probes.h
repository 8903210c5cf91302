/*
 * lowbit_probes.h -- measured ceilings for the roofline of liblowbit.so's
 * kernels on this GPU.  Context only: no probe is part of the y = W.x
 * path; bench.py times them next to the kernels, so that a kernel's rate can
 * be set against what the machine delivers to a kernel that does nothing
 * else, as well as against the vendor's peak figures.
 *
 * [P2] 7minutos.es, "PrismML lanza Bonsai 27B ...", "Rendimiento y
 * decodificacion especulativa DSpark": decode is bound by memory bandwidth,
 * prefill by compute -- hence a streaming-read and a matrix-core probe (and
 * an LDS probe for the table GEMV).  The same section's speculative verify
 * runs decode at a small batch, where the matrix-core GEMV is bound by its
 * own per-weight arithmetic rather than by memory: a fourth probe runs that
 * arithmetic alone.
 *
 * Conventions as in lowbit.h: device pointers, host-side validation, the
 * kernels are enqueued on `stream` and the call returns without waiting.
 */
#ifndef LOWBIT_PROBES_H
#define LOWBIT_PROBES_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of `bytes` bytes of device memory at `buf` (16-byte
 * aligned, bytes a multiple of 16, at most 2^40): a grid of
 * blocks_per_cu * (compute units) work-groups of 256 threads, each thread
 * keeping 8 independent 16-byte loads in flight.  order 0: the whole grid
 * reads one contiguous stretch per step (grid-stride order); order 1: each
 * work-group sweeps its own contiguous share.  The data are folded with
 * XOR; `sink` ([blocks] uint32, device) is written only if a fold equals a
 * fixed 32-bit constant, so the call writes (next to) nothing.
 * 1 <= blocks_per_cu <= 64.  Returns a lowbit_status. */
int lowbit_probe_stream_read(const void* buf, size_t bytes, int blocks_per_cu, int order,
                             uint32_t* sink, hipStream_t stream);

/* Matrix-core loop: every wave of blocks_per_cu * (compute units)
 * work-groups of 256 threads issues `iters` x 4 independent
 * v_mfma_f32_32x32x16_bf16 on register operands (2 * 32 * 32 * 16 flop
 * each) and nothing else; `sink` ([blocks * 256] float, device) is written
 * only if a result equals a fixed constant.  1 <= blocks_per_cu <= 8,
 * 1 <= iters <= 2^24.  Returns a lowbit_status. */
int lowbit_probe_mfma_bf16(int iters, int blocks_per_cu, float* sink, hipStream_t stream);

/* LDS read bandwidth: blocks_per_cu * (compute units) work-groups of 256
 * threads; each thread fills its 16-byte slots of a 32 KB LDS buffer, then
 * reads `iters` x 8 of them with 128-bit LDS loads (consecutive lanes on
 * consecutive 16-byte slots: no bank conflicts), folding them with XOR;
 * `sink` ([blocks * 256] uint32, device) is written only if a fold equals
 * a fixed constant.  Bytes read = blocks * 256 * iters * 8 * 16.
 * 1 <= blocks_per_cu <= 4, 1 <= iters <= 2^24.  Returns a lowbit_status. */
int lowbit_probe_lds_read(int iters, int blocks_per_cu, uint32_t* sink, hipStream_t stream);

/* The matrix-core GEMV's per-row work (lowbit_gemv at b >= 3): one code
 * byte expanded to eight FP16 operands +s / -s (a byte move, then four
 * packed shifts and four v_bitop3) and one v_mfma_f32_16x16x32_f16 -- 512
 * weights -- on register data, as the kernel issues them.  Every wave of
 * blocks_per_cu * (compute units) work-groups of 256 threads (so
 * blocks_per_cu waves per SIMD) runs iters x 16 such row steps.  mode 0:
 * expansion + MFMA, 1: the MFMA alone, 2: the 1-bit persistent kernel's
 * form -- each code byte an LDS table lookup of eight FP16 values +-1, four
 * MFMAs per 128-weight group and one FMA by the row's scale per group
 * (iters a multiple of 4: one group of 64 row steps per 4 iterations); `sink`
 * ([blocks * 256] float, device) is written only if a result equals a
 * fixed constant.  Time / (blocks_per_cu * iters * 16) is the time per row
 * step on one SIMD: with the kernel's two waves per SIMD, the floor that
 * this arithmetic puts under the kernel (mode 2 for 1-bit codes on the
 * persistent kernel, mode 0 otherwise).  1 <= blocks_per_cu
 * <= 4, 1 <= iters <= 2^24.  Returns a lowbit_status. */
int lowbit_probe_expand_mfma(int mode, int iters, int blocks_per_cu, float* sink,
                             hipStream_t stream);

/* Compute units of the current device, as the probes and the kernels'
 * launchers count them (256 if the query fails). */
int lowbit_probe_cu_count(void);

#ifdef __cplusplus
}
#endif

#endif /* LOWBIT_PROBES_H */
