// The two ends of a decode step: the low-bit embedding-row gather and the
// LM head's top-1 token.
//
// [P2] 7minutos.es, "PrismML lanza Bonsai 27B ...", "Como funciona la
//      compresion", and [P4] es.news.hada.io, "Configuracion multimodal y de
//      bajo bit de extremo a extremo": embeddings and the LM head are low-bit
//      like every other matrix.
// [P5] openclawradar.com, "Bonsai 1.7B Modelo Ternario ...", "Detalles
//      tecnicos": the decode kernels were checked by top-1 token match.
#include "common.h"

namespace lowbit {
namespace {

// ---------------------------------------------------------------------------
// embedding gather: out[t][:] = dequantised row ids[t] of W (FP16, exact:
// +s, -s as s with its sign bit flipped, or +0 for a ternary zero); an id
// outside [0, n) gives a row of zeros.  One work-group per token; thread i
// takes chunks i, i + 256, ... (8 weights -> one 16-byte store).

template <int FMT>
__global__ __launch_bounds__(256) void embed_kernel(const uint8_t* __restrict__ codes,
                                                    const uint16_t* __restrict__ scales,
                                                    int64_t n, int64_t k,
                                                    const int32_t* __restrict__ ids,
                                                    uint4* __restrict__ out) {
  const int64_t t = blockIdx.x;
  const int64_t id = ids[t];
  const bool valid = id >= 0 && id < n;
  const int64_t chunks = k / kChunk;
  const int64_t groups = k / kGroup;
  const int64_t tile = valid ? id / kTileRows : 0;
  const int r = valid ? (int)(id % kTileRows) : 0;
  const uint8_t* row_cells = codes + tile * chunks * Fmt<FMT>::cell_bytes;
  const uint16_t* row_scales = scales + tile * groups * kTileRows + r;
  uint4* dst = out + t * chunks;
  for (int64_t c = threadIdx.x; c < chunks; c += 256) {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (valid) {
      const uint32_t s = row_scales[(c / kChunksPerGroup) * kTileRows];
      const uint32_t neg_s = s ^ 0x8000u;
      const uint32_t p = row_cells[c * Fmt<FMT>::cell_bytes + r];  // Q1 bits / T2 pos
      const uint32_t q = FMT == 2 ? row_cells[c * Fmt<FMT>::cell_bytes + 16 + r] : 0u;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t v;
        if constexpr (FMT == 1) {
          v = ((p >> j) & 1u) ? s : neg_s;
        } else {
          const uint32_t pj = (p >> j) & 1u, qj = (q >> j) & 1u;
          v = (pj ^ qj) ? (qj ? neg_s : s) : 0u;  // pos xor neg = nonzero
        }
        w[j >> 1] |= v << ((j & 1) * 16);
      }
    }
    dst[c] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ---------------------------------------------------------------------------
// argmax: key(v, i) = (ordered bits of v) << 32 | (2^32 - 1 - i), so the
// largest key is the largest value and, among equal values, the lowest
// index.  The ordered bits map the IEEE order onto unsigned order (negative:
// all bits flipped, positive: sign bit set); a NaN with a clear sign bit
// sorts above +inf, so NaN wins as it does for numpy's and torch's argmax.

__device__ __forceinline__ uint64_t argmax_key(float v, int64_t i) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  if (__builtin_isnan(v)) u = 0x7FC00000u;  // every NaN the same, above +inf
  if (v == 0.0f) u = 0u;                    // -0 and +0 are equal values
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
}

__device__ __forceinline__ uint64_t wave_max(uint64_t k) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t o = __shfl_xor(k, off, 64);
    k = o > k ? o : k;
  }
  return k;
}

// block-wide maximum of one key per thread (256 threads)
__device__ __forceinline__ uint64_t block_max(uint64_t k, uint64_t* red) {
  k = wave_max(k);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = k;
  __syncthreads();
  uint64_t m = red[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) m = red[w] > m ? red[w] : m;
  __syncthreads();
  return m;
}

// The best key of y[row][lo .. hi) (lo < hi) over a 256-thread work-group's
// threads: four loads in flight per thread; an index past hi re-reads
// element hi - 1, whose key is already a candidate.
__device__ __forceinline__ uint64_t part_best(const float* __restrict__ y, int64_t row, int64_t n,
                                              int64_t lo, int64_t hi) {
  const float* yr = y + row * n;
  uint64_t best = 0;  // below every real key (a value's ordered bits are >= 1)
  for (int64_t i0 = lo + threadIdx.x; i0 < hi; i0 += 4 * 256) {
    float v[4];
    int64_t ix[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ix[u] = i0 + u * 256 < hi ? i0 + u * 256 : hi - 1;
      v[u] = yr[ix[u]];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint64_t kk = argmax_key(v[u], ix[u]);
      best = kk > best ? kk : best;
    }
  }
  return best;
}

// phase 1: work-group (p, row) reduces part p of batch row `row` to a key
__global__ __launch_bounds__(256) void argmax_part_kernel(const float* __restrict__ y, int64_t n,
                                                          int64_t per, uint64_t* __restrict__ part) {
  __shared__ uint64_t red[4];
  const int64_t p = blockIdx.x, row = blockIdx.y;
  const int64_t lo = p * per, hi = lo + per < n ? lo + per : n;
  uint64_t best = block_max(part_best(y, row, n, lo, hi), red);
  if (threadIdx.x == 0) part[row * gridDim.x + p] = best;
}

// phase 2: one work-group per batch row reduces the parts and decodes the key
__global__ __launch_bounds__(256) void argmax_final_kernel(const float* __restrict__ y, int64_t n,
                                                           const uint64_t* __restrict__ part,
                                                           int nparts, int32_t* __restrict__ idx,
                                                           float* __restrict__ val) {
  __shared__ uint64_t red[4];
  const int64_t row = blockIdx.x;
  uint64_t best = 0;
  for (int i = threadIdx.x; i < nparts; i += 256) {
    const uint64_t kk = part[row * nparts + i];
    best = kk > best ? kk : best;
  }
  best = block_max(best, red);
  if (threadIdx.x == 0) {
    const int64_t i = (int64_t)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
    idx[row] = (int32_t)i;
    if (val) val[row] = y[row * n + i];
  }
}

constexpr int kArgmaxParts = 256;

int argmax_parts(int64_t n) {
  // parts of at least 1024 elements, at most kArgmaxParts of them; with
  // per = ceil(n / parts) every part is non-empty, since parts * (parts - 1)
  // < n
  int64_t p = (n + 1023) / 1024;
  return (int)(p < 1 ? 1 : (p > kArgmaxParts ? kArgmaxParts : p));
}

int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }

}  // namespace

hipError_t launch_embed(int fmt, const uint8_t* codes, const uint16_t* scales, int64_t n,
                        int64_t k, const int32_t* ids, int64_t count, uint16_t* out,
                        hipStream_t st) {
  const dim3 grid((unsigned)count);
  if (fmt == 1)
    hipLaunchKernelGGL(embed_kernel<1>, grid, dim3(256), 0, st, codes, scales, n, k, ids,
                       reinterpret_cast<uint4*>(out));
  else
    hipLaunchKernelGGL(embed_kernel<2>, grid, dim3(256), 0, st, codes, scales, n, k, ids,
                       reinterpret_cast<uint4*>(out));
  return hipGetLastError();
}

size_t argmax_workspace_bytes(int64_t n, int64_t b) {
  return (size_t)align256(b * argmax_parts(n) * 8);
}

hipError_t launch_argmax(const float* y, int64_t n, int64_t b, int32_t* idx, float* val,
                         void* ws, hipStream_t st) {
  const int parts = argmax_parts(n);
  const int64_t per = (n + parts - 1) / parts;
  uint64_t* part = static_cast<uint64_t*>(ws);
  hipLaunchKernelGGL(argmax_part_kernel, dim3((unsigned)parts, (unsigned)b), dim3(256), 0, st, y,
                     n, per, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(argmax_final_kernel, dim3((unsigned)b), dim3(256), 0, st, y, n, part, parts,
                     idx, val);
  return hipGetLastError();
}

size_t lm_head_workspace_bytes(int64_t n, int64_t k, int64_t b) {
  return (size_t)align256((int64_t)gemv_workspace_bytes(k, b)) + argmax_workspace_bytes(n, b);
}

hipError_t launch_lm_head(int fmt, const uint8_t* codes, const uint16_t* scales, int64_t n,
                          int64_t k, const uint16_t* x, int64_t b, float* y, int32_t* idx,
                          float* val, void* ws, hipStream_t st) {
  char* base = static_cast<char*>(ws);
  void* ws_argmax = base + align256((int64_t)gemv_workspace_bytes(k, b));
  hipError_t e = launch_gemv_prepare(n, k, x, b, y, base, st);
  if (e != hipSuccess) return e;
  e = launch_gemv_accumulate(fmt, codes, scales, n, k, b, y, base, st);
  if (e != hipSuccess) return e;
  return launch_argmax(y, n, b, idx, val, ws_argmax, st);
}

}  // namespace lowbit
