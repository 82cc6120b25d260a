// HIP kernels of the Spense hybrid sparse-dense linear layer for gfx950.
//
// Method: SpenseGPT gist.science explainer, Technical Summary 2.A (a 2:4
// region and a dense region along K, input-split with accumulation into one
// output) and 2.B (dense set = last p% or a chosen set permuted into the dense
// block).  The fragment layout these kernels read and write is described in
// spense_internal.h.
#include "spense_internal.h"

namespace spense {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// shared helpers
// ---------------------------------------------------------------------------

// Group of a 64-column step that slot pair j of lane group g covers (see the
// layout notes in spense_internal.h).
__device__ __forceinline__ int group_local(int g, int j) {
  return ((((g & 1) << 1) + (j >> 1)) << 2) + ((g >> 1) << 1) + (j & 1);
}

__device__ __forceinline__ uint32_t mag_key(uint8_t w) { return w & 0x7Fu; }
__device__ __forceinline__ uint32_t mag_key(uint16_t w) { return w & 0x7FFFu; }
__device__ __forceinline__ uint32_t mag_key(uint32_t w) { return w & 0x7FFFFFFFu; }

// The two kept slots of a group of four: slot t is kept when fewer than two
// other slots beat it, where u beats t if its magnitude key is larger, or
// equal with a lower position.  Exactly two slots qualify; i0 < i1.
__device__ __forceinline__ void select_two(const uint32_t k[4], int& i0, int& i1) {
  int first = -1, second = -1;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    int beaten = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (u != t) beaten += (k[u] > k[t]) || (k[u] == k[t] && u < t);
    if (beaten < 2) {
      if (first < 0) first = t;
      else second = t;
    }
  }
  i0 = first;
  i1 = second;
}

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Eight e4m3 codes (little-endian in lo, hi) -> eight bf16.  Every e4m3 value
// is exact in fp32 and in bf16, so keeping the upper half of the fp32 word is
// exact.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  auto f0 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);
  auto f1 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
  auto f2 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
  auto f3 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
  u32x4 w;
  w.x = __builtin_amdgcn_perm(__float_as_uint(f0[1]), __float_as_uint(f0[0]), 0x07060302u);
  w.y = __builtin_amdgcn_perm(__float_as_uint(f1[1]), __float_as_uint(f1[0]), 0x07060302u);
  w.z = __builtin_amdgcn_perm(__float_as_uint(f2[1]), __float_as_uint(f2[0]), 0x07060302u);
  w.w = __builtin_amdgcn_perm(__float_as_uint(f3[1]), __float_as_uint(f3[0]), 0x07060302u);
  return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ bf16x16 as_bf16x16(u32x4 lo, u32x4 hi) {
  u32x8 w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x16, w);
}

template <typename WT>
__device__ __forceinline__ u32x4 pack16(const WT* v, int first);

template <>
__device__ __forceinline__ u32x4 pack16<uint8_t>(const uint8_t* v, int first) {
  u32x4 o;
  o.x = v[first + 0] | (v[first + 1] << 8) | (v[first + 2] << 16) | ((uint32_t)v[first + 3] << 24);
  o.y = v[first + 4] | (v[first + 5] << 8) | (v[first + 6] << 16) | ((uint32_t)v[first + 7] << 24);
  o.z = v[first + 8] | (v[first + 9] << 8) | (v[first + 10] << 16) | ((uint32_t)v[first + 11] << 24);
  o.w = v[first + 12] | (v[first + 13] << 8) | (v[first + 14] << 16) | ((uint32_t)v[first + 15] << 24);
  return o;
}

template <>
__device__ __forceinline__ u32x4 pack16<uint16_t>(const uint16_t* v, int first) {
  u32x4 o;
  o.x = v[first + 0] | ((uint32_t)v[first + 1] << 16);
  o.y = v[first + 2] | ((uint32_t)v[first + 3] << 16);
  o.z = v[first + 4] | ((uint32_t)v[first + 5] << 16);
  o.w = v[first + 6] | ((uint32_t)v[first + 7] << 16);
  return o;
}

template <typename WT>
constexpr int64_t kSparseBlock = sizeof(WT) == 1 ? 1280 : 2304;
template <typename WT>
constexpr int64_t kDenseBlock = sizeof(WT) == 1 ? 2048 : 4096;
template <typename WT>
constexpr int64_t kIdxOffset = sizeof(WT) == 1 ? 1024 : 2048;

// ---------------------------------------------------------------------------
// pack: 2:4 selection + compression into the fragment layout (bf16 / e4m3)
// ---------------------------------------------------------------------------

// One thread per (row tile, sparse macro-step, lane): eight groups of one row.
template <typename WT>
__global__ void pack_sparse_kernel(LayerDesc d, const WT* __restrict__ W, int64_t ldw) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= d.NT * d.n_sm * 64) return;
  const int lane = (int)(gid & 63);
  const int64_t rest = gid >> 6;
  const int64_t i = rest % d.n_sm, rt = rest / d.n_sm;
  const int r = lane & 15, g = lane >> 4;
  const int64_t n = rt * 16 + r;
  uint32_t idx = 0;
  WT v[16];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t G = 32 * i + 16 * q + group_local(g, j);
      uint32_t nib = 4u;  // padding group: slots (0, 1), zero values
      WT a = 0, b = 0;
      if (n < d.N && 4 * G < d.K_s) {
        WT w[4];
        uint32_t k[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          w[t] = W[n * ldw + d.pi[4 * G + t]];
          k[t] = mag_key(w[t]);
        }
        int i0, i1;
        select_two(k, i0, i1);
        nib = (uint32_t)(i0 | (i1 << 2));
        a = w[i0];
        b = w[i1];
      }
      idx |= nib << (16 * q + 4 * j);
      v[8 * q + 2 * j] = a;
      v[8 * q + 2 * j + 1] = b;
    }
  }
  uint8_t* blk = d.wpack + rt * d.tile_bytes + i * kSparseBlock<WT>;
  if constexpr (sizeof(WT) == 1) {
    *(u32x4*)(blk + 16 * lane) = pack16<WT>(v, 0);
  } else {
    *(u32x4*)(blk + 16 * lane) = pack16<WT>(v, 0);
    *(u32x4*)(blk + 1024 + 16 * lane) = pack16<WT>(v, 8);
  }
  *(uint32_t*)(blk + kIdxOffset<WT> + 4 * lane) = idx;
}

// One thread per (row tile, dense macro-step, lane): 2 x 16 dense values of one row.
template <typename WT>
__global__ void pack_dense_kernel(LayerDesc d, const WT* __restrict__ W, int64_t ldw) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= d.NT * d.n_dm * 64) return;
  const int lane = (int)(gid & 63);
  const int64_t rest = gid >> 6;
  const int64_t i = rest % d.n_dm, rt = rest / d.n_dm;
  const int r = lane & 15, g = lane >> 4;
  const int64_t n = rt * 16 + r;
  uint8_t* blk = d.wpack + rt * d.tile_bytes + d.n_sm * kSparseBlock<WT> + i * kDenseBlock<WT>;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    WT v[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int64_t c = 128 * i + 64 * q + 16 * g + t;
      v[t] = (n < d.N && c < d.K_d) ? W[n * ldw + d.pi[d.K_s + c]] : (WT)0;
    }
    if constexpr (sizeof(WT) == 1) {
      *(u32x4*)(blk + q * 1024 + 16 * lane) = pack16<WT>(v, 0);
    } else {
      *(u32x4*)(blk + q * 2048 + 16 * lane) = pack16<WT>(v, 0);
      *(u32x4*)(blk + q * 2048 + 1024 + 16 * lane) = pack16<WT>(v, 8);
    }
  }
}

// fp32: canonical form.  One thread per (row, meta word) for the sparse part.
__global__ void pack_f32_sparse_kernel(LayerDesc d, const uint32_t* __restrict__ W, int64_t ldw) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= d.N * d.meta_words) return;
  const int64_t n = gid / d.meta_words, w = gid % d.meta_words;
  uint32_t* vals = (uint32_t*)d.vals32 + n * (d.K_s / 2);
  uint32_t word = 0;
  for (int jj = 0; jj < 8; ++jj) {
    const int64_t G = 8 * w + jj;
    if (4 * G >= d.K_s) break;
    uint32_t x[4], k[4];
    for (int t = 0; t < 4; ++t) {
      x[t] = W[n * ldw + d.pi[4 * G + t]];
      k[t] = mag_key(x[t]);
    }
    int i0, i1;
    select_two(k, i0, i1);
    word |= (uint32_t)(i0 | (i1 << 2)) << (4 * jj);
    vals[2 * G] = x[i0];
    vals[2 * G + 1] = x[i1];
  }
  d.meta32[n * d.meta_words + w] = word;
}

__global__ void pack_f32_dense_kernel(LayerDesc d, const uint32_t* __restrict__ W, int64_t ldw) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= d.N * d.K_d) return;
  const int64_t n = gid / d.K_d, c = gid % d.K_d;
  ((uint32_t*)d.dense32)[n * d.K_d + c] = W[n * ldw + d.pi[d.K_s + c]];
}

// ---------------------------------------------------------------------------
// export: fragment layout -> canonical form
// ---------------------------------------------------------------------------
template <typename WT>
__global__ void export_sparse_kernel(LayerDesc d, WT* __restrict__ vals, uint32_t* __restrict__ meta,
                                     uint8_t* __restrict__ mask) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= d.N * d.meta_words) return;
  const int64_t n = gid / d.meta_words, w = gid % d.meta_words;
  const int64_t rt = n / 16;
  const int r = (int)(n % 16);
  uint32_t word = 0;
  for (int jj = 0; jj < 8; ++jj) {
    const int64_t G = 8 * w + jj;
    if (4 * G >= d.K_s) break;
    const int64_t i = G / 32;
    const int q = (int)((G % 32) / 16);
    const int gl = (int)(G % 16);
    const int hi2 = gl >> 2, mid = (gl >> 1) & 1, lo1 = gl & 1;
    const int g = (mid << 1) | (hi2 >> 1);
    const int j = ((hi2 & 1) << 1) | lo1;
    const int lane = 16 * g + r;
    const uint8_t* blk = d.wpack + rt * d.tile_bytes + i * kSparseBlock<WT>;
    const uint32_t idx = *(const uint32_t*)(blk + kIdxOffset<WT> + 4 * lane);
    const uint32_t nib = (idx >> (16 * q + 4 * j)) & 15u;
    WT v0, v1;
    if constexpr (sizeof(WT) == 1) {
      v0 = blk[16 * lane + 8 * q + 2 * j];
      v1 = blk[16 * lane + 8 * q + 2 * j + 1];
    } else {
      const uint16_t* h = (const uint16_t*)(blk + q * 1024 + 16 * lane);
      v0 = h[2 * j];
      v1 = h[2 * j + 1];
    }
    if (vals) {
      vals[n * (d.K_s / 2) + 2 * G] = v0;
      vals[n * (d.K_s / 2) + 2 * G + 1] = v1;
    }
    if (mask) {
      const int i0 = nib & 3, i1 = nib >> 2;
      for (int t = 0; t < 4; ++t) mask[n * d.K_s + 4 * G + t] = (t == i0 || t == i1) ? 1 : 0;
    }
    word |= nib << (4 * jj);
  }
  if (meta) meta[n * d.meta_words + w] = word;
}

template <typename WT>
__global__ void export_dense_kernel(LayerDesc d, WT* __restrict__ dense) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= d.N * d.K_d) return;
  const int64_t n = gid / d.K_d, c = gid % d.K_d;
  const int64_t rt = n / 16;
  const int r = (int)(n % 16);
  const int64_t i = c / 128;
  const int q = (int)((c % 128) / 64), g = (int)((c % 64) / 16), t = (int)(c % 16);
  const int lane = 16 * g + r;
  const uint8_t* blk = d.wpack + rt * d.tile_bytes + d.n_sm * kSparseBlock<WT> + i * kDenseBlock<WT>;
  WT v;
  if constexpr (sizeof(WT) == 1) {
    v = blk[q * 1024 + 16 * lane + t];
  } else {
    v = ((const uint16_t*)(blk + q * 2048 + (t >> 3) * 1024 + 16 * lane))[t & 7];
  }
  dense[n * d.K_d + c] = v;
}

// fp32 canonical form: vals / meta / dense are stored as exported; only the mask is derived.
__global__ void export_f32_mask_kernel(LayerDesc d, uint8_t* __restrict__ mask) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t G = d.K_s / 4;
  if (gid >= d.N * G) return;
  const int64_t n = gid / G, g = gid % G;
  const uint32_t nib = (d.meta32[n * d.meta_words + g / 8] >> (4 * (g % 8))) & 15u;
  for (int t = 0; t < 4; ++t) mask[n * d.K_s + 4 * g + t] = (t == (int)(nib & 3) || t == (int)(nib >> 2)) ? 1 : 0;
}

// ---------------------------------------------------------------------------
// linear: SMFMAC (sparse region) + MFMA (dense region) into one accumulator
// ---------------------------------------------------------------------------
constexpr int kPitch = 136;  // staged X'p row: 128 bf16 + 8 pad (272 B, conflict-free 16 B reads)

// Stage X'p[m0 .. m0+mloc)[col_base + 128u + (0..127)] for u < nc into LDS.
template <int MT, int CH>
__device__ __forceinline__ void stage_chunk(uint16_t (*xs)[MT * 16][kPitch], const LayerDesc& d, const LinearArgs& a,
                                            int64_t col_base, int nc, int64_t m0, int mloc) {
  const uint16_t* X = (const uint16_t*)a.X;
  const int per_macro = mloc * 16;
  const int units = nc * per_macro;
  for (int e = threadIdx.x; e < units; e += kWavesPerWG * 64) {
    const int u = e / per_macro;
    const int rem = e - u * per_macro;
    const int m = rem >> 4, c8 = rem & 15;
    const int64_t col = col_base + 128 * u + 8 * c8;
    const uint16_t* xrow = X + (m0 + m) * a.ldx;
    u32x4 val;
    if (!a.gather) {
      val = *(const u32x4*)(xrow + col);
    } else {
      uint32_t h[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int32_t src = d.pip[col + t];
        h[t] = src >= 0 ? (uint32_t)xrow[src] : 0u;
      }
      val.x = h[0] | (h[1] << 16);
      val.y = h[2] | (h[3] << 16);
      val.z = h[4] | (h[5] << 16);
      val.w = h[6] | (h[7] << 16);
    }
    *(u32x4*)&xs[u][m][8 * c8] = val;
  }
}

template <int MT>
__device__ __forceinline__ void load_b(bf16x16 (&B)[MT], const uint16_t (*xsu)[kPitch], int q, int lane, int mloc) {
  const int bcol = 64 * q + 16 * (lane >> 4);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = 16 * mt + (lane & 15);
    if (m < mloc) {
      const uint16_t* p = &xsu[m][bcol];
      B[mt] = as_bf16x16(*(const u32x4*)p, *(const u32x4*)(p + 8));
    } else {
      B[mt] = as_bf16x16(u32x4{0, 0, 0, 0}, u32x4{0, 0, 0, 0});
    }
  }
}

template <typename WT, int MT, int CH>
__global__ __launch_bounds__(kWavesPerWG * 64) void linear_kernel(LayerDesc d, LinearArgs a, LinearPlan p) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[CH][MT * 16][kPitch];
  __shared__ int last_flag;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bid = blockIdx.x;
  const int rg = bid % p.rgroups;
  const int rest = bid / p.rgroups;
  const int S = p.splits;
  const int s = rest % S;
  const int mg = rest / S;
  const int64_t rt = (int64_t)rg * kWavesPerWG + wave;
  const bool active = rt < d.NT;
  const int64_t m0 = (int64_t)mg * MT * 16;
  const int mloc = (int)(a.M - m0 < MT * 16 ? a.M - m0 : MT * 16);
  const int64_t ms0 = d.n_sm * s / S, ms1 = d.n_sm * (s + 1) / S;
  const int64_t md0 = d.n_dm * s / S, md1 = d.n_dm * (s + 1) / S;
  const uint8_t* tile = d.wpack + (active ? rt : 0) * d.tile_bytes;

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // sparse region: v_smfmac_f32_16x16x64_bf16, two steps per macro-step
  for (int64_t c0 = ms0; c0 < ms1; c0 += CH) {
    const int nc = (int)(ms1 - c0 < CH ? ms1 - c0 : CH);
    __syncthreads();
    stage_chunk<MT, CH>(xs, d, a, 128 * c0, nc, m0, mloc);
    __syncthreads();
    if (active) {
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        if (u < nc) {
          const uint8_t* blk = tile + (c0 + u) * kSparseBlock<WT>;
          bf16x8 A0, A1;
          if constexpr (sizeof(WT) == 1) {
            const u32x4 v = *(const u32x4*)(blk + 16 * lane);
            A0 = fp8x8_to_bf16(v.x, v.y);
            A1 = fp8x8_to_bf16(v.z, v.w);
          } else {
            A0 = as_bf16x8(*(const u32x4*)(blk + 16 * lane));
            A1 = as_bf16x8(*(const u32x4*)(blk + 1024 + 16 * lane));
          }
          const int idx = (int)*(const uint32_t*)(blk + kIdxOffset<WT> + 4 * lane);
          bf16x16 B[MT];
          load_b<MT>(B, xs[u], 0, lane, mloc);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[mt] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(A0, B[mt], acc[mt], idx, 0, 0);
          load_b<MT>(B, xs[u], 1, lane, mloc);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[mt] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(A1, B[mt], acc[mt], idx, 0, 1);
        }
      }
    }
  }

  // dense region: v_mfma_f32_16x16x32_bf16, four per macro-step
  for (int64_t c0 = md0; c0 < md1; c0 += CH) {
    const int nc = (int)(md1 - c0 < CH ? md1 - c0 : CH);
    __syncthreads();
    stage_chunk<MT, CH>(xs, d, a, d.K_sp + 128 * c0, nc, m0, mloc);
    __syncthreads();
    if (active) {
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        if (u < nc) {
          const uint8_t* blk = tile + d.n_sm * kSparseBlock<WT> + (c0 + u) * kDenseBlock<WT>;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            bf16x8 Alo, Ahi;
            if constexpr (sizeof(WT) == 1) {
              const u32x4 v = *(const u32x4*)(blk + q * 1024 + 16 * lane);
              Alo = fp8x8_to_bf16(v.x, v.y);
              Ahi = fp8x8_to_bf16(v.z, v.w);
            } else {
              Alo = as_bf16x8(*(const u32x4*)(blk + q * 2048 + 16 * lane));
              Ahi = as_bf16x8(*(const u32x4*)(blk + q * 2048 + 1024 + 16 * lane));
            }
            bf16x16 B[MT];
            load_b<MT>(B, xs[u], q, lane, mloc);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              const bf16x8 blo = __builtin_shufflevector(B[mt], B[mt], 0, 1, 2, 3, 4, 5, 6, 7);
              const bf16x8 bhi = __builtin_shufflevector(B[mt], B[mt], 8, 9, 10, 11, 12, 13, 14, 15);
              acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Alo, blo, acc[mt], 0, 0, 0);
              acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ahi, bhi, acc[mt], 0, 0, 0);
            }
          }
        }
      }
    }
  }

  // epilogue: accumulator lane l, register r holds Y^T[n = 16rt + 4(l/16) + r][m = m0 + 16mt + l%16]
  const int nb = 4 * (lane >> 4);
  if (S == 1) {
    if (!active) return;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int64_t m = m0 + 16 * mt + (lane & 15);
      if (m >= a.M) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t n = rt * 16 + nb + r;
        if (n >= d.N) continue;
        const float y = acc[mt][r] * (d.scales ? d.scales[n] : 1.0f);
        if (a.ydtype == DT_F32) ((float*)a.Y)[m * a.ldy + n] = y;
        else ((uint16_t*)a.Y)[m * a.ldy + n] = (uint16_t)bf16_rne(y);
      }
    }
    return;
  }

  // split-K: write the partial, the last workgroup of the tile adds all partials in split order
  const int64_t NP = d.NT * 16;
  if (active) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int64_t m = m0 + 16 * mt + (lane & 15);
      if (m < a.M) *(f32x4*)(a.ws + ((int64_t)s * a.M + m) * NP + rt * 16 + nb) = acc[mt];
    }
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t* cnt = a.counters + (int64_t)mg * p.rgroups + rg;
    const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (old == S - 1);
    if (old == S - 1) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();
  if (!active) return;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int64_t m = m0 + 16 * mt + (lane & 15);
    if (m >= a.M) continue;
    f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s2 = 0; s2 < S; ++s2) sum += *(const f32x4*)(a.ws + ((int64_t)s2 * a.M + m) * NP + rt * 16 + nb);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t n = rt * 16 + nb + r;
      if (n >= d.N) continue;
      const float y = sum[r] * (d.scales ? d.scales[n] : 1.0f);
      if (a.ydtype == DT_F32) ((float*)a.Y)[m * a.ldy + n] = y;
      else ((uint16_t*)a.Y)[m * a.ldy + n] = (uint16_t)bf16_rne(y);
    }
  }
}

// fp32 weights: VALU, one wave per output row, lanes stride over groups and dense columns.
__global__ __launch_bounds__(256) void linear_f32_kernel(LayerDesc d, LinearArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= d.N) return;
  const float* X = (const float*)a.X;
  const int64_t G = d.K_s / 4;
  const float* vals = d.vals32 + n * (d.K_s / 2);
  const uint32_t* meta = d.meta32 + n * d.meta_words;
  const float* dense = d.dense32 + n * d.K_d;
  for (int64_t m = 0; m < a.M; ++m) {
    const float* x = X + m * a.ldx;
    float acc = 0.f;
    for (int64_t gi = lane; gi < G; gi += 64) {
      const uint32_t nib = (meta[gi >> 3] >> (4 * (gi & 7))) & 15u;
      acc = fmaf(vals[2 * gi], x[d.pi[4 * gi + (nib & 3)]], acc);
      acc = fmaf(vals[2 * gi + 1], x[d.pi[4 * gi + (nib >> 2)]], acc);
    }
    for (int64_t c = lane; c < d.K_d; c += 64) acc = fmaf(dense[c], x[d.pi[d.K_s + c]], acc);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) {
      if (a.ydtype == DT_F32) ((float*)a.Y)[m * a.ldy + n] = acc;
      else ((uint16_t*)a.Y)[m * a.ldy + n] = (uint16_t)bf16_rne(acc);
    }
  }
}

__global__ void zero_i32_kernel(int32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

inline unsigned blocks_for(int64_t n, int threads) { return (unsigned)((n + threads - 1) / threads); }

template <typename WT>
hipError_t launch_pack_frag(const LayerDesc& d, const void* W, int64_t ldw, hipStream_t s) {
  if (d.n_sm > 0)
    pack_sparse_kernel<WT><<<blocks_for(d.NT * d.n_sm * 64, 256), 256, 0, s>>>(d, (const WT*)W, ldw);
  if (d.n_dm > 0)
    pack_dense_kernel<WT><<<blocks_for(d.NT * d.n_dm * 64, 256), 256, 0, s>>>(d, (const WT*)W, ldw);
  return hipGetLastError();
}

template <typename WT>
hipError_t launch_export_frag(const LayerDesc& d, void* vals, uint32_t* meta, uint8_t* mask, void* dense, hipStream_t s) {
  if (d.K_s > 0 && (vals || meta || mask))
    export_sparse_kernel<WT><<<blocks_for(d.N * d.meta_words, 256), 256, 0, s>>>(d, (WT*)vals, meta, mask);
  if (d.K_d > 0 && dense) export_dense_kernel<WT><<<blocks_for(d.N * d.K_d, 256), 256, 0, s>>>(d, (WT*)dense);
  return hipGetLastError();
}

template <typename WT, int MT, int CH>
hipError_t launch_linear_t(const LayerDesc& d, const LinearArgs& a, const LinearPlan& p, hipStream_t s) {
  const unsigned grid = (unsigned)((int64_t)p.rgroups * p.splits * p.mgroups);
  linear_kernel<WT, MT, CH><<<grid, kWavesPerWG * 64, 0, s>>>(d, a, p);
  return hipGetLastError();
}

template <typename WT>
hipError_t launch_linear_frag(const LayerDesc& d, const LinearArgs& a, const LinearPlan& p, hipStream_t s) {
  switch (p.mt) {
    case 1: return launch_linear_t<WT, 1, 4>(d, a, p, s);
    case 2: return launch_linear_t<WT, 2, 4>(d, a, p, s);
    case 4: return launch_linear_t<WT, 4, 2>(d, a, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_pack(const LayerDesc& d, const void* W, int64_t ldw, hipStream_t s) {
  switch (d.wdtype) {
    case DT_FP8: return launch_pack_frag<uint8_t>(d, W, ldw, s);
    case DT_BF16: return launch_pack_frag<uint16_t>(d, W, ldw, s);
    case DT_F32:
      if (d.K_s > 0)
        pack_f32_sparse_kernel<<<blocks_for(d.N * d.meta_words, 256), 256, 0, s>>>(d, (const uint32_t*)W, ldw);
      if (d.K_d > 0)
        pack_f32_dense_kernel<<<blocks_for(d.N * d.K_d, 256), 256, 0, s>>>(d, (const uint32_t*)W, ldw);
      return hipGetLastError();
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_export(const LayerDesc& d, void* vals, uint32_t* meta, uint8_t* mask, void* dense, hipStream_t s) {
  switch (d.wdtype) {
    case DT_FP8: return launch_export_frag<uint8_t>(d, vals, meta, mask, dense, s);
    case DT_BF16: return launch_export_frag<uint16_t>(d, vals, meta, mask, dense, s);
    case DT_F32: {
      hipError_t e = hipSuccess;
      if (vals && d.K_s > 0) e = hipMemcpyAsync(vals, d.vals32, (size_t)(d.N * (d.K_s / 2)) * 4, hipMemcpyDeviceToDevice, s);
      if (e == hipSuccess && meta && d.K_s > 0)
        e = hipMemcpyAsync(meta, d.meta32, (size_t)(d.N * d.meta_words) * 4, hipMemcpyDeviceToDevice, s);
      if (e == hipSuccess && dense && d.K_d > 0)
        e = hipMemcpyAsync(dense, d.dense32, (size_t)(d.N * d.K_d) * 4, hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return e;
      if (mask && d.K_s > 0) export_f32_mask_kernel<<<blocks_for(d.N * (d.K_s / 4), 256), 256, 0, s>>>(d, mask);
      return hipGetLastError();
    }
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_linear(const LayerDesc& d, const LinearArgs& a, const LinearPlan& p, hipStream_t s) {
  switch (d.wdtype) {
    case DT_FP8: return launch_linear_frag<uint8_t>(d, a, p, s);
    case DT_BF16: return launch_linear_frag<uint16_t>(d, a, p, s);
    case DT_F32:
      linear_f32_kernel<<<blocks_for(d.N, 4), 256, 0, s>>>(d, a);
      return hipGetLastError();
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_zero_i32(int32_t* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  zero_i32_kernel<<<blocks_for(n, 256), 256, 0, s>>>(p, n);
  return hipGetLastError();
}

}  // namespace spense
