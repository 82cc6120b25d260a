// Device helpers shared by the HIP kernel translation units of the Spense
// linear layer (spense_kernels.hip, spense_tile.hip): element conversions,
// the structured-sparse matrix instructions, buffer loads, the split-K
// hand-off and the epilogue.  Everything here is inline and file-local to
// each translation unit that includes it.
#pragma once

#include "spense_internal.h"

namespace spense {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Index word of a dense unit: abid 0 reads 0x4444 (slots at group positions 0
// and 1), abid 1 reads 0xEEEE (positions 2 and 3).
constexpr uint32_t kDenseIdx = 0xEEEE4444u;

// ---------------------------------------------------------------------------
// helpers
// ---------------------------------------------------------------------------

// Group of a 64-column step that slot pair j of lane group g covers.
__device__ __forceinline__ int group_local(int g, int j) {
  return ((((g & 1) << 1) + (j >> 1)) << 2) + ((g >> 1) << 1) + (j & 1);
}

// Inverse of group_local: group gl (0..15) -> (lane group g, pair j).
__device__ __forceinline__ void group_owner(int gl, int& g, int& j) {
  const int hi2 = gl >> 2, mid = (gl >> 1) & 1, lo1 = gl & 1;
  g = (mid << 1) | (hi2 >> 1);
  j = ((hi2 & 1) << 1) | lo1;
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
// is exact in bf16; the conversion with a unit scale widens two codes per
// instruction (code 2j to the low half of word j, code 2j + 1 to the high
// half).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  u32x4 w;
  w.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
  w.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
  w.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
  w.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
  return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ bf16x16 as_bf16x16(u32x4 lo, u32x4 hi) {
  u32x8 w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x16, w);
}

// Structured-sparse matrix instruction.  Its destination is tied to the
// accumulator input, which is live across the instruction, so the destination
// can never share registers with the A or B operands (a matrix instruction
// whose destination overlaps srcA/srcB gives wrong results; tests/test_isa.py
// checks the built code for that).
template <int ABID>
__device__ __forceinline__ f32x4 smfmac_bf16(const bf16x8& a, const bf16x16& b, const f32x4& c, int idx) {
  return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a, b, c, idx, 0, ABID);
}

// Raw buffer resource over [base, base + bytes): a load at an offset beyond
// `bytes` returns zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Split-K handshake without cache maintenance.  Partials are written and read
// with device-coherent accesses (the cache policy of relaxed agent-scope
// atomics: written through to, and read from, the level shared by all XCDs,
// so no L2 write-back or invalidate is needed), 16 bytes per lane; each thread
// waits until its partial stores have completed before the workgroup's
// arrival is counted, and the workgroup that arrives last reads every partial.
// Layout [split][row tile][m][16 rows]: a wave's store for one tile and m-tile
// is 1 KB contiguous.
constexpr int kCoherent = 16;  // sc1 cache-policy bit of buffer loads/stores
__device__ __forceinline__ void store_partial(__amdgpu_buffer_rsrc_t ws, uint32_t off, const f32x4& v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ws, (int)off, 0, kCoherent);
}

__device__ __forceinline__ f32x4 load_partial(__amdgpu_buffer_rsrc_t ws, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ws, (int)off, 0, kCoherent));
}

// Returns true in every thread of the last-arriving workgroup; that workgroup
// also rearms the counter for the next launch.
__device__ __forceinline__ bool arrive_last(int32_t* cnt, int S, int* flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = (old == S - 1);
    if (old == S - 1) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return *flag != 0;
}

// Scales and output columns of this lane's four output rows of row tile rt
// (packed rows rt*16 + 4(lane/16) + 0..3), loaded when a kernel starts so that
// its epilogue does not wait on memory.  Column -1 marks a padding row.
struct TileOut {
  f32x4 sc;
  u32x4 col;
};
__device__ __forceinline__ TileOut tile_out(const LayerDesc& d, int64_t rt, int lane) {
  TileOut t;
  t.sc = *(const f32x4*)(d.scales + rt * 16 + 4 * (lane >> 4));
  t.col = *(const u32x4*)(d.ycol + rt * 16 + 4 * (lane >> 4));
  return t;
}

__device__ __forceinline__ void store_y(const LinearArgs& a, int64_t m, int64_t n, float y) {
  if (a.ydtype == DT_F32) ((float*)a.Y)[m * a.ldy + n] = y;
  else ((uint16_t*)a.Y)[m * a.ldy + n] = (uint16_t)bf16_rne(y);
}

// Y[m][n..n+3] = y in one store: n % 4 == 0, Y 16-byte aligned, ldy % 4 == 0
__device__ __forceinline__ void store_y4(const LinearArgs& a, int64_t m, int64_t n, const f32x4& y) {
  if (a.ydtype == DT_F32) {
    *(f32x4*)((float*)a.Y + m * a.ldy + n) = y;
  } else {
    uint2 v;
    v.x = bf16_rne(y[0]) | (bf16_rne(y[1]) << 16);
    v.y = bf16_rne(y[2]) | (bf16_rne(y[3]) << 16);
    *(uint2*)((uint16_t*)a.Y + m * a.ldy + n) = v;
  }
}

// Writes Y (S == 1) or this split's partial; with S > 1 the last workgroup of
// the tile adds the partials in split order.  acc: lane l, register r =
// Y^T[n = 16rt + 4(l/16) + r][m = m0 + 16mt + l%16].
// Epilogue of a wave's NR row tiles (rt0 ..) x MT m-tiles; acc[r * MT + t],
// to[r] = tile_out of row tile rt0 + r.  Compile-time counts keep every
// accumulator index static (a dynamic index would move them to scratch).
// XS: also multiply by the per-token activation scale a.xscale[m] (W8A8).
template <int NR, int MT, bool XS = false>
__device__ __forceinline__ void finish_tile(const LayerDesc& d, const LinearArgs& a, const f32x4* acc,
                                            const TileOut* to, int64_t rt0, int64_t m0, int s, int S,
                                            int64_t cnt_index, int* last_flag) {
  const int lane = threadIdx.x & 63;
  const int nb = 4 * (lane >> 4);
  constexpr int nr = NR, mtiles = MT;
  // partial of (split, row tile, m) at byte ((split * NT + rt) * M + m) * 64 + 4 nb
  const __amdgpu_buffer_rsrc_t wsr = make_rsrc(a.ws, S > 1 ? (uint32_t)((int64_t)S * d.NT * a.M * 64) : 0u);
  auto poff = [&](int64_t split, int64_t rt, int64_t m) {
    return (uint32_t)((((split * d.NT + rt) * a.M + m) * 16 + nb) * 4);
  };
  if (S > 1) {
#pragma unroll
    for (int r = 0; r < nr; ++r) {
      const int64_t rt = rt0 + r;
      if (rt >= d.NT) break;
#pragma unroll
      for (int mt = 0; mt < mtiles; ++mt) {
        const int64_t m = m0 + 16 * mt + (lane & 15);
        if (m < a.M) store_partial(wsr, poff(s, rt, m), acc[r * mtiles + mt]);
      }
    }
    if (!arrive_last(a.counters + cnt_index, S, last_flag)) return;
  }
#pragma unroll
  for (int r = 0; r < nr; ++r) {
    const int64_t rt = rt0 + r;
    if (rt >= d.NT) break;
#pragma unroll
    for (int mt = 0; mt < mtiles; ++mt) {
      const int64_t m = m0 + 16 * mt + (lane & 15);
      if (m >= a.M) continue;
      f32x4 sum = acc[r * mtiles + mt];
      if (S > 1) {
        // the partials in split order, loaded eight at a time (one memory
        // round trip per eight splits instead of one per split); splits past
        // S read zero at an out-of-range offset and are not added
        sum = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < S; s0 += 8) {
          f32x4 part[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) part[j] = load_partial(wsr, s0 + j < S ? poff(s0 + j, rt, m) : 0x80000000u);
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (s0 + j < S) sum += part[j];
        }
      }
      if (a.glu) {
        // rows (q, q+1) of this lane are the gate and up rows of one
        // intermediate index; the gate row carries its output column
#pragma unroll
        for (int q = 0; q < 4; q += 2) {
          const int col = (int)to[r].col[q];
          const float g = sum[q] * to[r].sc[q], u = sum[q + 1] * to[r].sc[q + 1];
          if (col >= 0) store_y(a, m, col, g / (1.0f + __expf(-g)) * u);
        }
      } else {
        f32x4 y;
        if constexpr (XS) {
          const float xs = a.xscale[m];
#pragma unroll
          for (int q = 0; q < 4; ++q) y[q] = sum[q] * to[r].sc[q] * xs;
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) y[q] = sum[q] * to[r].sc[q];
        }
        // the lane's four rows are usually four consecutive output columns
        // (every input-split layer): one 8- or 16-byte store instead of four
        const u32x4 c = to[r].col;
        if (a.yvec && (int)c.x >= 0 && (c.x & 3u) == 0 && c.y == c.x + 1 && c.z == c.x + 2 && c.w == c.x + 3) {
          store_y4(a, m, c.x, y);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if ((int)c[q] >= 0) store_y(a, m, c[q], y[q]);
        }
      }
    }
  }
}

// One lane's unit in registers: A operands of two SMFMACs and the index word.
template <typename WT>
struct UnitFrag;
template <>
struct UnitFrag<uint8_t> {
  u32x4 a;
  uint32_t idx;
};
template <>
struct UnitFrag<uint16_t> {
  u32x4 a0, a1;
  uint32_t idx;
};

// Loads one unit.  The index load is issued for dense units too (from the
// unit itself, a cached address) and its value replaced by the dense index
// word at use, so sparse and dense units issue the same loads.  Weights are
// read once per call: the loads carry the non-temporal hint, which streams
// faster than the default policy.
template <typename WT>
__device__ __forceinline__ void load_unit(UnitFrag<WT>& f, const uint8_t* unit, const uint8_t* idx_addr, int lane) {
  if constexpr (sizeof(WT) == 1) {
    f.a = __builtin_nontemporal_load((const u32x4*)(unit + 16 * lane));
  } else {
    f.a0 = __builtin_nontemporal_load((const u32x4*)(unit + 16 * lane));
    f.a1 = __builtin_nontemporal_load((const u32x4*)(unit + 1024 + 16 * lane));
  }
  f.idx = __builtin_nontemporal_load((const uint32_t*)idx_addr);
}

// vector-memory loads load_unit issues
template <typename WT>
constexpr int kUnitLoads = sizeof(WT) == 1 ? 2 : 3;

// s_waitcnt vmcnt(n), other counters left alone (gfx9 encoding: vmcnt bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
#define SPENSE_WAIT_VM(n) \
  __builtin_amdgcn_s_waitcnt((int)(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8)))

// A workgroup barrier without a memory fence: the fence of __syncthreads
// would make every wave wait for all of its loads into LDS, the ones still in
// flight included.  The memory clobber keeps the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// Two SMFMACs: A0 with B0 (index half 0), A1 with B1 (index half 1).
// The unit's two A operands as bf16 (e4m3 widened exactly).
template <typename WT>
__device__ __forceinline__ void unit_a(const UnitFrag<WT>& f, bf16x8& A0, bf16x8& A1) {
  if constexpr (sizeof(WT) == 1) {
    A0 = fp8x8_to_bf16(f.a.x, f.a.y);
    A1 = fp8x8_to_bf16(f.a.z, f.a.w);
  } else {
    A0 = as_bf16x8(f.a0);
    A1 = as_bf16x8(f.a1);
  }
}

template <typename WT>
__device__ __forceinline__ void mac_unit(f32x4& acc0, f32x4& acc1, const UnitFrag<WT>& f, int idx, const bf16x16& B0,
                                         const bf16x16& B1) {
  bf16x8 A0, A1;
  unit_a<WT>(f, A0, A1);
  acc0 = smfmac_bf16<0>(A0, B0, acc0, idx);
  acc1 = smfmac_bf16<1>(A1, B1, acc1, idx);
}

// Split, row group and m-group of workgroup `block` of `grid`.  Logical id
// L = s * (rgroups * mgroups) + (position within the split).  Workgroups are
// dealt to the 8 XCDs round-robin; with the XCD remap each XCD takes a
// contiguous run of logical ids.  Within a split the order is m-group
// fastest over one row group, or, with rblock > 1, blocks of rblock row
// groups taken one m-group at a time (row group fastest), so that the
// workgroups an XCD runs together share both weight slices and activation
// rows in its L2: with R row groups x G m-groups resident, one stage moves
// R weight slices and G activation slices into the L2 instead of one slice
// and R G activation slices.
__device__ __forceinline__ void tile_coords(int b, int grid, const LinearPlan& p, int& s, int& rg, int& mg) {
  if (p.xcd_remap) b = (b % 8) * (grid / 8) + b / 8;
  const int S = p.splits;
  s = 0;
  mg = 0;
  rg = b;
  if (p.mgroups > 1 && p.rblock > 1) {
    const uint32_t per_split = (uint32_t)p.rgroups * (uint32_t)p.mgroups;
    uint32_t L = (uint32_t)b;
    if (S > 1) {
      s = (int)(L / per_split);
      L -= (uint32_t)s * per_split;
    }
    const uint32_t span = (uint32_t)p.rblock * (uint32_t)p.mgroups;
    const uint32_t blk = L / span, base = blk * (uint32_t)p.rblock;
    const uint32_t left = (uint32_t)p.rgroups - base;
    const uint32_t gb = left < (uint32_t)p.rblock ? left : (uint32_t)p.rblock;
    const uint32_t rem = L - blk * span;
    mg = (int)(rem / gb);
    rg = (int)(base + rem - (uint32_t)mg * gb);
    return;
  }
  if (p.mgroups > 1) {
    mg = (int)((uint32_t)b % (uint32_t)p.mgroups);
    rg = (int)((uint32_t)b / (uint32_t)p.mgroups);
  }
  if (S > 1) {
    s = (int)((uint32_t)rg / (uint32_t)p.rgroups);
    rg = (int)((uint32_t)rg % (uint32_t)p.rgroups);
  }
}

// Steps [n s / S, n (s + 1) / S) of split s of S.  Launch set-up runs before
// a wave's first weight load, so it avoids 64-bit division: n < 2^16 (K_p <
// 2^23) and S <= 64 keep n (s + 1) below 2^31, and one split needs none.
__device__ __forceinline__ void split_range(int64_t n, int s, int S, int& lo, int& hi) {
  if (S == 1) {
    lo = 0;
    hi = (int)n;
    return;
  }
  lo = (int)((uint32_t)((int)n * s) / (uint32_t)S);
  hi = (int)((uint32_t)((int)n * (s + 1)) / (uint32_t)S);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr uint32_t kOutOfRange = 0x80000000u;  // beyond every resource built here (all below 2 GB)

// Cache policy of buffer loads: 0 default, kNonTemporal for data read once
// (the non-temporal hint streams faster than the default policy).
constexpr int kNonTemporal = 2;
template <int POL = 0>
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, POL));
}
template <int POL = 0>
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, POL);
}

// 32 contiguous bytes of LDS as one B operand
__device__ __forceinline__ bf16x16 lds_b16(const uint8_t* p) {
  return as_bf16x16(*(const u32x4*)p, *(const u32x4*)(p + 16));
}
__device__ __forceinline__ i32x8 lds_b8(const uint8_t* p) {
  const i32x4 q0 = *(const i32x4*)p, q1 = *(const i32x4*)(p + 16);
  return __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ f32x4 smfmac_fp8(const u32x4& a, const i32x8& b, const f32x4& c, int idx) {
  return __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(__builtin_bit_cast(i32x4, a), b, c, idx, 0, 0);
}

}  // namespace
}  // namespace spense
