// SpenseGPT+ dense index selection for a GLU block (SpenseGPT explainer,
// Technical Summary 2.B): a score per intermediate index i,
//   score[i] = sum_j |Wg[i,j]| sqrt(Hx_jj) + sum_j |Wu[i,j]| sqrt(Hx_jj)
//            + sum_n |Wd[n,i]| sqrt(Ha_ii),
// with Hx = X^T X over calibration inputs of gate/up and Ha = A^T A over
// calibration inputs of down, |W| the dequantised magnitude; then the k
// highest scores (ties to the lower index) form the dense set.
//
// Offline, memory-bound work: every reduction runs in a fixed order, so the
// scores are bitwise repeatable.
#include "spense_internal.h"

namespace spense {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

template <typename WT>
__device__ __forceinline__ float abs_value(WT v);

template <>
__device__ __forceinline__ float abs_value<uint8_t>(uint8_t v) {
  // e4m3: widen exactly, then drop the sign
  const f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8((int)(v & 0x7Fu), false);
  return f.x;
}

template <>
__device__ __forceinline__ float abs_value<uint16_t>(uint16_t v) {
  return __uint_as_float((uint32_t)(v & 0x7FFFu) << 16);
}

// partial[c][chunk] = sum over the chunk's rows t of X[t][c]^2, one thread per column
__global__ void colsq_partial_kernel(const uint16_t* __restrict__ X, int64_t T, int64_t C, int64_t ld, int64_t rows,
                                     float* __restrict__ partial, int64_t nchunks) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t chunk = blockIdx.y;
  if (c >= C) return;
  const int64_t t0 = chunk * rows, t1 = t0 + rows < T ? t0 + rows : T;
  float acc = 0.f;
  for (int64_t t = t0; t < t1; ++t) {
    const float x = __uint_as_float((uint32_t)X[t * ld + c] << 16);
    acc = fmaf(x, x, acc);
  }
  partial[c * nchunks + chunk] = acc;
}

// out[c] = sum of the chunk partials in chunk order
__global__ void colsq_final_kernel(const float* __restrict__ partial, int64_t nchunks, int64_t C,
                                   float* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= C) return;
  float acc = 0.f;
  for (int64_t i = 0; i < nchunks; ++i) acc += partial[c * nchunks + i];
  out[c] = acc;
}

// out[r] = |s_r| * sum_k |W[r][k]| sqrt(h[k]); one wave per row, each lane
// takes 16 consecutive weights per step (one 16-byte load for e4m3), then a
// fixed butterfly over the wave.  Rows whose start or K is not 16-aligned use
// the element-wise loop.
template <typename WT>
__global__ __launch_bounds__(256) void row_score_kernel(const WT* __restrict__ W, int64_t R, int64_t K, int64_t ld,
                                                        const float* __restrict__ scales,
                                                        const float* __restrict__ h, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  const WT* w = W + r * ld;
  float acc = 0.f;
  constexpr int kV = 16;
  const bool vec = (((uintptr_t)w) % (kV * sizeof(WT))) == 0 && K % kV == 0;
  if (vec) {
    for (int64_t k0 = (int64_t)lane * kV; k0 < K; k0 += 64 * kV) {
      WT v[kV];
#pragma unroll
      for (int q = 0; q < kV * (int)sizeof(WT) / 16; ++q)
        *(uint4*)((char*)v + 16 * q) = *(const uint4*)((const char*)(w + k0) + 16 * q);
#pragma unroll
      for (int t = 0; t < kV; ++t) acc = fmaf(abs_value<WT>(v[t]), sqrtf(h[k0 + t]), acc);
    }
  } else {
    for (int64_t k = lane; k < K; k += 64) acc = fmaf(abs_value<WT>(w[k]), sqrtf(h[k]), acc);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) out[r] = scales ? acc * fabsf(scales[r]) : acc;
}

// partial[c][chunk] = sum over the chunk's rows r of |s_r| |W[r][c]|: one
// thread per column and row chunk (consecutive threads read consecutive
// columns of a row)
template <typename WT>
__global__ void col_abs_partial_kernel(const WT* __restrict__ W, int64_t R, int64_t C, int64_t ld,
                                       const float* __restrict__ scales, int64_t rows, float* __restrict__ partial,
                                       int64_t nchunks) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t chunk = blockIdx.y;
  if (c >= C) return;
  const int64_t r0 = chunk * rows, r1 = r0 + rows < R ? r0 + rows : R;
  float acc = 0.f;
  for (int64_t r = r0; r < r1; ++r) acc = fmaf(abs_value<WT>(W[r * ld + c]), scales ? fabsf(scales[r]) : 1.f, acc);
  partial[c * nchunks + chunk] = acc;
}

// score[i] = (gate[i] + up[i]) + down_abs[i] * sqrt(ha[i]); rows [0, I) of
// rowscore are the gate rows, [I, 2I) the up rows
__global__ void combine_kernel(const float* __restrict__ rowscore, const float* __restrict__ down_abs,
                               const float* __restrict__ ha, int64_t I, float* __restrict__ score) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= I) return;
  score[i] = (rowscore[i] + rowscore[I + i]) + down_abs[i] * sqrtf(ha[i]);
}

// rank[i] += the number of indices j in this block's candidate range that
// beat i (score[j] > score[i], or equal and j < i).  Candidates are staged in
// LDS tile by tile; the ranges of the grid's second dimension are added with
// integer atomics, whose sum does not depend on their order.
constexpr int kRankTile = 256;
constexpr int kRankRange = 2048;  // candidates per workgroup
__global__ __launch_bounds__(kRankTile) void rank_partial_kernel(const float* __restrict__ score, int n,
                                                                 int* __restrict__ rank) {
  __shared__ float tile[kRankTile];
  const int i = (int)blockIdx.x * kRankTile + (int)threadIdx.x;
  const float si = i < n ? score[i] : 0.f;
  const int j_begin = (int)blockIdx.y * kRankRange;
  const int j_end = j_begin + kRankRange < n ? j_begin + kRankRange : n;
  int cnt = 0;
  for (int j0 = j_begin; j0 < j_end; j0 += kRankTile) {
    const int j = j0 + (int)threadIdx.x;
    tile[threadIdx.x] = j < j_end ? score[j] : 0.f;
    __syncthreads();
    const int lim = j_end - j0 < kRankTile ? j_end - j0 : kRankTile;
    if (lim == kRankTile) {
#pragma unroll 16
      for (int t = 0; t < kRankTile; ++t) {
        const float sj = tile[t];
        cnt += (sj > si || (sj == si && j0 + t < i)) ? 1 : 0;
      }
    } else {
      for (int t = 0; t < lim; ++t) {
        const float sj = tile[t];
        cnt += (sj > si || (sj == si && j0 + t < i)) ? 1 : 0;
      }
    }
    __syncthreads();
  }
  if (i < n && cnt) atomicAdd(rank + i, cnt);
}

// sel[i] = 1 iff rank[i] < k: the k highest scores with ties to the lower
// index; 2 marks a NaN score (NaN has no place in the order, so the host
// rejects the call)
__global__ void rank_final_kernel(const float* __restrict__ score, const int* __restrict__ rank, int n, int64_t k,
                                  uint8_t* __restrict__ sel) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < n) sel[i] = score[i] != score[i] ? 2 : (rank[i] < k ? 1 : 0);
}

__global__ void fill_zero_kernel(int* __restrict__ p, int n) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < n) p[i] = 0;
}

inline unsigned blocks(int64_t n, int t) { return (unsigned)((n + t - 1) / t); }

}  // namespace

hipError_t launch_colsq(const void* X, int64_t T, int64_t C, int64_t ld, float* partial, int64_t rows_per_chunk,
                        float* out, hipStream_t s) {
  const int64_t nchunks = (T + rows_per_chunk - 1) / rows_per_chunk;
  colsq_partial_kernel<<<dim3(blocks(C, 256), (unsigned)nchunks), 256, 0, s>>>((const uint16_t*)X, T, C, ld,
                                                                              rows_per_chunk, partial, nchunks);
  colsq_final_kernel<<<blocks(C, 256), 256, 0, s>>>(partial, nchunks, C, out);
  return hipGetLastError();
}

hipError_t launch_glu_scores(int32_t wdtype, const void* W_gu, const void* W_down, int64_t H, int64_t I, int64_t ld_gu,
                             int64_t ld_down, const float* s_gu, const float* s_down, const float* hx,
                             const float* ha, float* rowscore, float* down_abs, float* partial, float* score,
                             hipStream_t s) {
  const int64_t nchunks = (H + kColRows - 1) / kColRows;
  if (wdtype == DT_FP8) {
    row_score_kernel<uint8_t><<<blocks(2 * I, 4), 256, 0, s>>>((const uint8_t*)W_gu, 2 * I, H, ld_gu, s_gu, hx,
                                                                rowscore);
    col_abs_partial_kernel<uint8_t><<<dim3(blocks(I, 256), (unsigned)nchunks), 256, 0, s>>>(
        (const uint8_t*)W_down, H, I, ld_down, s_down, kColRows, partial, nchunks);
  } else if (wdtype == DT_BF16) {
    row_score_kernel<uint16_t><<<blocks(2 * I, 4), 256, 0, s>>>((const uint16_t*)W_gu, 2 * I, H, ld_gu, s_gu, hx,
                                                                 rowscore);
    col_abs_partial_kernel<uint16_t><<<dim3(blocks(I, 256), (unsigned)nchunks), 256, 0, s>>>(
        (const uint16_t*)W_down, H, I, ld_down, s_down, kColRows, partial, nchunks);
  } else {
    return hipErrorInvalidValue;
  }
  colsq_final_kernel<<<blocks(I, 256), 256, 0, s>>>(partial, nchunks, I, down_abs);
  combine_kernel<<<blocks(I, 256), 256, 0, s>>>(rowscore, down_abs, ha, I, score);
  return hipGetLastError();
}

hipError_t launch_rank_select(const float* score, int64_t n, int64_t k, int* rank, uint8_t* sel, hipStream_t s) {
  const int nn = (int)n;
  fill_zero_kernel<<<blocks(n, 256), 256, 0, s>>>(rank, nn);
  rank_partial_kernel<<<dim3(blocks(n, kRankTile), blocks(n, kRankRange)), kRankTile, 0, s>>>(score, nn, rank);
  rank_final_kernel<<<blocks(n, 256), 256, 0, s>>>(score, rank, nn, k, sel);
  return hipGetLastError();
}

}  // namespace spense
