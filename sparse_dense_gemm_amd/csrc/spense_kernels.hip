// HIP kernels of the Spense hybrid sparse-dense linear layer for gfx950.
//
// Method: SpenseGPT gist.science explainer, Technical Summary 2.A (a 2:4
// region and a dense region along K, input-split with accumulation into one
// output) and 2.B (dense set = last p% or a chosen set permuted into the dense
// block).  The unit layout these kernels read and write is described in
// spense_internal.h.
#include "spense_device.h"

#include <algorithm>
#include <mutex>

namespace spense {
namespace {


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
constexpr int64_t kUnit = sizeof(WT) == 1 ? 1024 : 2048;

// One unit = one lane's A operands of two SMFMACs: 16 values v[0..15], A0 =
// v[0..7], A1 = v[8..15].  e4m3: 16 B at +16 lane; bf16: A0 at +16 lane, A1 at
// +1024 + 16 lane.
template <typename WT>
__device__ __forceinline__ void store_unit(uint8_t* unit, int lane, const WT* v) {
  if constexpr (sizeof(WT) == 1) {
    *(u32x4*)(unit + 16 * lane) = pack16<WT>(v, 0);
  } else {
    *(u32x4*)(unit + 16 * lane) = pack16<WT>(v, 0);
    *(u32x4*)(unit + 1024 + 16 * lane) = pack16<WT>(v, 8);
  }
}

template <typename WT>
__device__ __forceinline__ WT unit_value(const uint8_t* unit, int lane, int slot) {
  if constexpr (sizeof(WT) == 1) return unit[16 * lane + slot];
  else return ((const uint16_t*)(unit + (slot >> 3) * 1024 + 16 * lane))[slot & 7];
}

// ---------------------------------------------------------------------------
// pack: 2:4 selection + compression into the unit layout (bf16 / e4m3)
// ---------------------------------------------------------------------------

// One thread per (row tile, sparse unit, lane): eight groups of one row.
template <typename WT>
__global__ void pack_sparse_kernel(LayerDesc d, const WT* __restrict__ W, int64_t ldw) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= d.NT * d.n_sm * 64) return;
  const int lane = (int)(gid & 63);
  const int64_t rest = gid >> 6;
  const int64_t i = rest % d.n_sm, rt = rest / d.n_sm;
  const int r = lane & 15, g = lane >> 4;
  const int64_t n = rt * 16 + r;
  // packed row n holds W row wrow (a row subset of W for the parts of an output-split layer)
  const int64_t wrow = n < d.N ? (d.wrow ? (int64_t)d.wrow[n] : n) : 0;
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
          w[t] = W[wrow * ldw + d.pi[4 * G + t]];
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
  uint8_t* tile = d.wpack + rt * d.tile_bytes;
  store_unit<WT>(tile + i * kUnit<WT>, lane, v);
  *(uint32_t*)(tile + d.idx_off + i * 256 + 4 * lane) = idx;
}

// One thread per (row tile, dense unit = 64 dense columns, lane).
template <typename WT>
__global__ void pack_dense_kernel(LayerDesc d, const WT* __restrict__ W, int64_t ldw) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t units = 2 * d.n_dm;
  if (gid >= d.NT * units * 64) return;
  const int lane = (int)(gid & 63);
  const int64_t rest = gid >> 6;
  const int64_t t = rest % units, rt = rest / units;
  const int r = lane & 15, g = lane >> 4;
  const int64_t n = rt * 16 + r;
  // packed row n holds W row wrow (a row subset of W for the parts of an output-split layer)
  const int64_t wrow = n < d.N ? (d.wrow ? (int64_t)d.wrow[n] : n) : 0;
  WT v[16];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int64_t c = 64 * t + 4 * group_local(g, j) + 2 * half + w;
        v[8 * half + 2 * j + w] = (n < d.N && c < d.K_d) ? W[wrow * ldw + d.pi[d.K_s + c]] : (WT)0;
      }
  store_unit<WT>(d.wpack + rt * d.tile_bytes + (d.n_sm + t) * kUnit<WT>, lane, v);
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
// export: unit layout -> canonical form
// ---------------------------------------------------------------------------
template <typename WT>
__global__ void export_sparse_kernel(LayerDesc d, WT* __restrict__ vals, uint32_t* __restrict__ meta,
                                     uint8_t* __restrict__ mask) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= d.N * d.meta_words) return;
  const int64_t n = gid / d.meta_words, w = gid % d.meta_words;
  const int64_t rt = n / 16;
  const int r = (int)(n % 16);
  const uint8_t* tile = d.wpack + rt * d.tile_bytes;
  uint32_t word = 0;
  for (int jj = 0; jj < 8; ++jj) {
    const int64_t G = 8 * w + jj;
    if (4 * G >= d.K_s) break;
    const int64_t i = G / 32;
    const int q = (int)((G % 32) / 16);
    int g, j;
    group_owner((int)(G % 16), g, j);
    const int lane = 16 * g + r;
    const uint32_t idx = *(const uint32_t*)(tile + d.idx_off + i * 256 + 4 * lane);
    const uint32_t nib = (idx >> (16 * q + 4 * j)) & 15u;
    const uint8_t* unit = tile + i * kUnit<WT>;
    const WT v0 = unit_value<WT>(unit, lane, 8 * q + 2 * j);
    const WT v1 = unit_value<WT>(unit, lane, 8 * q + 2 * j + 1);
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
  const int64_t t = c / 64;
  const int cc = (int)(c % 64);
  int g, j;
  group_owner(cc >> 2, g, j);
  const int pos = cc & 3;
  const int lane = 16 * g + r;
  const uint8_t* unit = d.wpack + rt * d.tile_bytes + (d.n_sm + t) * kUnit<WT>;
  dense[n * d.K_d + c] = unit_value<WT>(unit, lane, 8 * (pos >> 1) + 2 * j + (pos & 1));
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
// linear, shared pieces
// ---------------------------------------------------------------------------

// B operand (16 activations of one lane) from a staged row: 32 contiguous bytes.
__device__ __forceinline__ bf16x16 lds_b(const uint16_t* p) {
  return as_bf16x16(*(const u32x4*)p, *(const u32x4*)(p + 8));
}

// Eight activations of row xr at the column indices i0, i1 (negative: zero).
__device__ __forceinline__ u32x4 gather8_from(const uint16_t* xr, const u32x4& i0, const u32x4& i1) {
  const int src[8] = {(int)i0.x, (int)i0.y, (int)i0.z, (int)i0.w, (int)i1.x, (int)i1.y, (int)i1.z, (int)i1.w};
  uint32_t h[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) h[t] = xr[src[t] >= 0 ? src[t] : 0];
#pragma unroll
  for (int t = 0; t < 8; ++t) h[t] = src[t] >= 0 ? h[t] : 0u;
  u32x4 val;
  val.x = h[0] | (h[1] << 16);
  val.y = h[2] | (h[3] << 16);
  val.z = h[4] | (h[5] << 16);
  val.w = h[6] | (h[7] << 16);
  return val;
}

// Gathers 8 activations X'p[row][col..col+8) (col a multiple of 8).
__device__ __forceinline__ u32x4 gather8(const LinearArgs& a, const LayerDesc& d, const uint16_t* xr, int64_t col) {
  if (!a.gather) return *(const u32x4*)(xr + col);
  return gather8_from(xr, *(const u32x4*)(d.pip + col), *(const u32x4*)(d.pip + col + 4));
}

// ---------------------------------------------------------------------------
// linear, decode (M <= 16): each wave streams its row tile's units straight
// into registers through a ring of P in-flight units; the activations of the
// workgroup's split are staged (and gathered) into LDS once, so the K loop
// has no barrier.  Sparse and dense units issue the same loads and the same
// two SMFMACs (only addresses and the index word differ), so the loop body is
// straight-line code and the in-order load counter stays P-1 units ahead.
// ---------------------------------------------------------------------------
template <typename WT, int NW, int P, bool GATHER, bool SWZ>
__device__ __forceinline__ void decode_body(const LayerDesc& d, const LinearArgs& a, const LinearPlan& p, int block,
                                            uint16_t* xs_dyn) {
  // the split-K arrival flag sits in the last 16 bytes of the dynamic LDS
  // (reserved by the planner only when the launch has several splits)
  int* last_flag = (int*)((uint8_t*)xs_dyn + p.lds_bytes - 16);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar address math
  const int S = p.splits;  // the grid is rgroups x S workgroups
  const int rg = S == 1 ? block : (int)((uint32_t)block % (uint32_t)p.rgroups);
  const int s = S == 1 ? 0 : (int)((uint32_t)block / (uint32_t)p.rgroups);
  const int64_t rt = (int64_t)rg * NW + wave;
  const bool active = rt < d.NT;
  int ms0, ms1, md0, md1;
  split_range(d.n_sm, s, S, ms0, ms1);
  split_range(d.n_dm, s, S, md0, md1);
  const int ns = ms1 - ms0, nd = md1 - md0;
  const int total = ns + 2 * nd;  // units
  const int M = (int)a.M;
  const int m = lane & 15, g = lane >> 4;
  const uint8_t* tile = d.wpack + (active ? rt : 0) * d.tile_bytes;
  // unit k of this split: sparse units ms0.. then dense units 2*md0..; both
  // contiguous, so the unit index within the tile is k plus a per-range offset
  const int64_t sbase = ms0, dbase = d.n_sm + 2 * md0 - ns;
  const uint8_t* sidx = tile + d.idx_off + ms0 * 256;
  // Staged rows, so that the 16 rows a B read touches at once sit on
  // different LDS banks: padded by 16 bytes (gathered rows: the split's
  // columns + 16 bytes; contiguous rows, copied in 1 KB blocks of 4
  // unit-steps: whole blocks + 16 bytes), or with SWZ unpadded whole 1 KB
  // blocks in which row r keeps the 16-byte piece c of each unit-step (16
  // pieces) at position c ^ (r & 15).  The swizzle lets 16 rows of 5120
  // activations (exactly 160 KB) fit one CU; it costs address arithmetic
  // per B read, so it is used only where the padded rows do not fit.
  const int nch = (ns + nd + 3) / 4;  // 1 KB blocks of a contiguous staged row
  const int pitch = SWZ ? 512 * nch : GATHER ? (ns + nd) * 128 + 8 : 512 * nch + 8;  // elements

  // weights of unit k (lane offset 16 lane) and its index word (lane offset
  // 4 lane; a dense unit reads a word of itself, replaced at use)
  auto unit_ptr = [&](int k) { return tile + (k + (k < ns ? sbase : dbase)) * kUnit<WT>; };
  auto idx_ptr = [&](int k) { return k < ns ? sidx + k * 256 : unit_ptr(k); };

  // weight ring; waves without units (past the last row tile, or an empty
  // split) load unit 0 of tile 0 so that every wave issues the same loads
  const bool stream = active && total > 0;
  UnitFrag<WT> wr[P];
  auto issue_ring = [&]() {
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int k = i < total ? i : total - 1;
      load_unit<WT>(wr[i], stream ? unit_ptr(k) : d.wpack, (stream ? idx_ptr(k) : d.wpack) + 4 * lane, lane);
    }
  };
  // Offsets are 32-bit: rows < 16 and the leading dimension < 2^23 (the entry
  // points refuse larger ones), columns < K_p < 2^23.
  const uint16_t* X = (const uint16_t*)a.X;
  const int ldx = (int)a.ldx;
  // X'p column of unit-step u: 128 u + (u < ns ? xcol_s : xcol_d)
  const int xcol_s = 128 * ms0, xcol_d = (int)d.K_sp + 128 * (md0 - ns);
  if constexpr (!GATHER) {
    // Contiguous activations go straight from memory into LDS (no register
    // round trip), issued before the weight ring: they land while the first
    // units are in flight, and the wait for them below leaves the ring's
    // loads outstanding.  Copy q: staged row q / nch, its bytes 1024 (q % nch)
    // onwards, 16 bytes per lane; bytes past the split's columns read out of
    // range, i.e. zero.
    // (lane l writes position l of its 1 KB block, so with SWZ it loads the
    // piece the swizzle puts there)
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, (uint32_t)(M * ldx * 2));
    const int copies = M * nch;
    for (int q = wave; q < copies; q += NW) {
      const int mrow = q / nch, t = q - mrow * nch;
      const int e = 512 * t + 8 * (SWZ ? lane ^ (mrow & 15) : lane);  // element of the staged row
      const int u = e >> 7;              // its unit-step
      const uint32_t voff = u < ns + nd ? (uint32_t)((mrow * ldx + 128 * u + (u < ns ? xcol_s : xcol_d) + (e & 127)) * 2)
                                        : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (void*)(xs_dyn + mrow * pitch + 512 * t), 16, voff, 0, 0, 0);
    }
    issue_ring();
  }

  const TileOut to = tile_out(d, active ? rt : 0, lane);

  // Gathered activations are staged through registers, one 16-byte piece (8
  // consecutive X'p columns) at a time per thread.  The column map is the
  // same for every row, so a thread loads the piece's 8 map entries once and
  // then issues the gathers of every row of that piece together (kGRows rows
  // at a time: one memory round trip for the map, one per kGRows rows for the
  // activations).  A 2-byte buffer load per activation, from a resource over
  // that row; padding columns (map entry < 0) read out of range, i.e. zero.
  // The first map loads go out before the weight ring, so the gathers that
  // depend on them do not wait for the ring.
  const int per_row = (ns + nd) * 16;  // pieces per staged row
  constexpr int kGRows = 8;
  u32x4 map0, map1;  // the piece's 8 map entries
  // (a piece past the row reads the map's first entries and stores nothing)
  auto load_map = [&](int q) {
    const int u = q >> 4, c8 = q & 15;
    const int col = q < per_row ? 128 * u + (u < ns ? xcol_s : xcol_d) + 8 * c8 : 0;
    map0 = *(const u32x4*)(d.pip + col);
    map1 = *(const u32x4*)(d.pip + col + 4);
  };
  auto gather_piece = [&](int q) {
    const bool okq = q < per_row;
    const int u = okq ? q >> 4 : 0, c8 = q & 15;
    const int src[8] = {(int)map0.x, (int)map0.y, (int)map0.z, (int)map0.w,
                        (int)map1.x, (int)map1.y, (int)map1.z, (int)map1.w};
    int sv[8];  // byte offsets in the row of the piece's source columns
#pragma unroll
    for (int t = 0; t < 8; ++t) sv[t] = src[t] >= 0 ? 2 * src[t] : (int)kOutOfRange;
    for (int m0 = 0; m0 < M; m0 += kGRows) {
      uint32_t h[kGRows][8];
#pragma unroll
      for (int r = 0; r < kGRows; ++r) {
        if (m0 + r < M) {
          const __amdgpu_buffer_rsrc_t xr = make_rsrc(X + (int64_t)(m0 + r) * ldx, (uint32_t)(2 * ldx));
#pragma unroll
          for (int t = 0; t < 8; ++t) h[r][t] = __builtin_amdgcn_raw_buffer_load_b16(xr, sv[t], 0, 0);
        }
      }
#pragma unroll
      for (int r = 0; r < kGRows; ++r) {
        if (okq && m0 + r < M) {
          u32x4 v;
          v.x = h[r][0] | (h[r][1] << 16);
          v.y = h[r][2] | (h[r][3] << 16);
          v.z = h[r][4] | (h[r][5] << 16);
          v.w = h[r][6] | (h[r][7] << 16);
          *(u32x4*)(xs_dyn + (m0 + r) * pitch + 128 * u + 8 * (SWZ ? c8 ^ ((m0 + r) & 15) : c8)) = v;
        }
      }
    }
  };
  if constexpr (GATHER) {
    // every thread loads a map and gathers (unconditionally: a load on one
    // path only would be copied at the merge, and the copy would wait for it)
    load_map(threadIdx.x);
    issue_ring();
    // keep the map's first use below the ring (a wait for the map must not
    // hold back the ring's loads)
    __builtin_amdgcn_sched_barrier(0);
    gather_piece(threadIdx.x);
    for (int q = threadIdx.x + NW * 64; q < per_row; q += NW * 64) {  // splits wider than 32 unit-steps
      load_map(q);
      gather_piece(q);
    }
    __syncthreads();
  } else {
    // this wave's copies have landed once at most the ring's loads are
    // outstanding (they were issued after the copies, and the counter retires
    // in order); the barrier then covers the other waves' copies
    SPENSE_WAIT_VM(P * kUnitLoads<WT>);
    barrier_no_fence();
  }

  f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
  if (stream) {
    // Lanes of activation rows m >= M read row 0: output column m depends only
    // on B column m, and columns m >= M are never stored.  With SWZ lane l
    // reads the pieces 8h + 2g and 8h + 2g + 1 of a unit-step (h: which
    // 64-column half) at their swizzled positions.
    const int mm = m < M ? m : 0;
    const uint16_t* xb = xs_dyn + mm * pitch + 16 * g;
    const uint8_t* xrow = (const uint8_t*)xs_dyn + mm * pitch * 2;
    const int o00 = 16 * ((2 * g) ^ mm), o01 = 16 * ((2 * g + 1) ^ mm);
    const int o10 = 16 * ((8 + 2 * g) ^ mm), o11 = 16 * ((9 + 2 * g) ^ mm);
    auto xread = [&](int col) {  // B operand at staged column col (a multiple of 64)
      if constexpr (SWZ) {
        const uint8_t* q = xrow + 256 * (col >> 7);
        const bool hi = (col >> 6) & 1;
        return as_bf16x16(*(const u32x4*)(q + (hi ? o10 : o00)), *(const u32x4*)(q + (hi ? o11 : o01)));
      } else {
        return lds_b(xb + col);
      }
    };
    // B operands of unit k (sparse: the unit-step's two 64-column halves;
    // dense: one 64-column half, read twice: a select between loaded values
    // would wait for them at once)
    auto bload = [&](int k, bf16x16& B0, bf16x16& B1) {
      const bool sp = k < ns;
      const int col0 = sp ? 128 * k : 128 * ns + 64 * (k - ns);
      B0 = xread(col0);
      B1 = xread(sp ? col0 + 64 : col0);
    };
    // The B operands are read one unit ahead (the LDS round trip of the next
    // unit overlaps this unit's products).
    bf16x16 b0, b1;
    bload(0, b0, b1);
    auto consume = [&](int i, int k) {
      bf16x16 n0, n1;
      bload(k + 1 < total ? k + 1 : k, n0, n1);
      mac_unit<WT>(acc0, acc1, wr[i], k < ns ? (int)wr[i].idx : (int)kDenseIdx, b0, b1);
      b0 = n0;
      b1 = n1;
    };
    // whole rings: every slot is consumed and refilled unconditionally, so
    // each slot waits for exactly its own loads
    int k0 = 0;
    for (; k0 + P <= total; k0 += P) {
#pragma unroll
      for (int i = 0; i < P; ++i) {
        consume(i, k0 + i);
        const int kn = k0 + i + P < total ? k0 + i + P : total - 1;
        load_unit<WT>(wr[i], unit_ptr(kn), idx_ptr(kn) + 4 * lane, lane);
      }
    }
    // drain: the last total % P units are already in the ring
#pragma unroll
    for (int i = 0; i < P; ++i)
      if (k0 + i < total) consume(i, k0 + i);
  }
  const f32x4 acc = acc0 + acc1;
  finish_tile<1, 1>(d, a, &acc, &to, rt, 0, s, S, rg, last_flag);
}

// No static LDS: the staged activations may take all 160 KB of the CU.
template <typename WT, int NW, int P, bool GATHER, bool SWZ>
__global__ __launch_bounds__(NW * 64) void linear_decode_kernel(LayerDesc d, LinearArgs a, LinearPlan p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs_dyn[];
  decode_body<WT, NW, P, GATHER, SWZ>(d, a, p, blockIdx.x, xs_dyn);
}

// Two layers in one grid (the two row classes of an output-split layer): the
// first workgroups run layer 0, the rest layer 1, with the same kernel shape.
template <typename WT, int NW, int P, bool GATHER, bool SWZ>
__global__ __launch_bounds__(NW * 64) void linear_decode2_kernel(LayerDesc d0, LinearArgs a0, LinearPlan p0,
                                                                 LayerDesc d1, LinearArgs a1, LinearPlan p1) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs_dyn[];
  const int g0 = p0.rgroups * p0.splits * p0.mgroups;
  if ((int)blockIdx.x < g0) decode_body<WT, NW, P, GATHER, SWZ>(d0, a0, p0, blockIdx.x, xs_dyn);
  else decode_body<WT, NW, P, GATHER, SWZ>(d1, a1, p1, blockIdx.x - g0, xs_dyn);
}

// ---------------------------------------------------------------------------
// linear, streamed activations: the split's activations pass through a
// double-buffered LDS ring of CH-unit chunks, so the LDS footprint does not
// grow with the split width.  One barrier per chunk; it waits on LDS only, so
// the weight ring stays in flight across it.  Each wave owns NR consecutive
// 16-row tiles and MT m-tiles of 16 activation rows: every weight unit loaded
// from HBM feeds MT products (pairs of products for bf16 activations), and
// every activation fragment read from LDS feeds NR of them.  Activations are
// read as a contiguous X'p (for a chosen dense set the host gathers, or
// quantises, it into a workspace first).
//
// All global loads are buffer loads: the wave's weight units at a per-wave
// resource plus a uniform (scalar) offset and the lane's fixed 16-byte slot,
// the activation pieces at a per-thread offset that is computed once per
// chunk.  No per-load 64-bit address arithmetic, and pieces outside the batch
// or the split take an offset beyond the resource, which reads zero.
//
// W8A8 (A8): e4m3 activation codes on v_smfmac_f32_16x16x128_fp8_fp8, one
// instruction per unit and no widening of the weights.  Operand layout of
// that instruction (16 rows x 128 columns of a 2:4 step): lane l (row l % 16,
// lane group h = l / 16) gives 16 stored values, bytes 2j, 2j+1 (j < 8) for
// group j of its 32-column slice, positions from nibble j of the index word;
// B lane l (column l % 16) gives 32 activations, and A byte pair j of lane
// group h pairs with B lane group 2(h & 1) + (j >= 4), bytes
// 16(h >> 1) + 4(j & 3) + pos.  For the unit layout (the A operands of the
// bf16 instruction pair, see spense_internal.h), B lane group h then needs
// the 32 staged columns at base = 64(h & 1) + 32(h >> 1) of a sparse unit
// (32(h >> 1) of a dense unit, whose fixed index word 0xEEEE4444 picks
// positions 0,1 of groups 0-3 and 2,3 of groups 4-7) with the middle two
// 8-column quarters swapped; the swap is done when the chunk is staged, so a
// fragment is 32 contiguous bytes of LDS.
// ---------------------------------------------------------------------------
// NTW: the weights are read once (one m-group): their loads carry the
// non-temporal hint.  With several m-groups each wave's weights are read again
// per m-group, mostly from L2, and keep the default policy (the hint makes
// those re-reads miss: 3-16% slower at M = 2048).
template <typename WT, bool A8, int NW, int NR, int P, int CH, int MT, bool NTW>
__device__ __forceinline__ void stream_body(const LayerDesc& d, const LinearArgs& a, const LinearPlan& p, int block,
                                            int grid, uint8_t* xs, int* last_flag_p) {
  static_assert(CH % P == 0, "a chunk must hold whole rings");
  static_assert(!A8 || sizeof(WT) == 1, "W8A8 takes e4m3 weights");
  constexpr int XB = A8 ? 1 : 2;           // bytes per staged activation
  constexpr int kSlot = 128 * XB;          // bytes of one unit slot (128 columns)
  constexpr int kPitch = CH * kSlot + 16;  // staged row: CH unit slots + pad
  constexpr int kPPU = kSlot / 16;         // 16-byte pieces per unit slot
  constexpr int kPPR = CH * kPPU;          // pieces per staged row
  constexpr int kThreads = NW * 64;
  static_assert(kThreads % kPPR == 0, "every piece of a thread sits at the same slot position");
  constexpr int kRowStep = kThreads / kPPR;  // rows between a thread's pieces
  constexpr int kPieces = 16 * MT / kRowStep;
  static_assert(kPieces * kRowStep == 16 * MT, "pieces must divide evenly");
  constexpr bool kSplitAcc = NR == 1 && MT == 1;  // alternate two accumulators when nothing else interleaves
  constexpr uint32_t UB = sizeof(WT) == 1 ? 1024u : 2048u;
  int& last_flag = *last_flag_p;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int S = p.splits;
  int s, rg, mg;
  tile_coords(block, grid, p, s, rg, mg);
  const int64_t rt0 = ((int64_t)rg * NW + wave) * NR;
  int ms0, ms1, md0, md1;
  split_range(d.n_sm, s, S, ms0, ms1);
  split_range(d.n_dm, s, S, md0, md1);
  const int ns = ms1 - ms0, nd = md1 - md0;
  const int total = ns + 2 * nd;  // units
  const int nchunks = (total + CH - 1) / CH;
  const int64_t m0 = (int64_t)mg * 16 * MT;
  const int mloc = (int)(a.M - m0 < 16 * MT ? a.M - m0 : 16 * MT);  // activation rows of this m-group
  const int rows = (int)(a.M < 16 * MT ? a.M : 16 * MT);            // rows of one staged buffer
  const int m = lane & 15, g = lane >> 4;

  // weights: one resource from the wave's first row tile (the last tile for a
  // wave wholly past the end); row tiles past the end read that first tile
  // (their results are never stored)
  const int64_t bt = rt0 < d.NT ? rt0 : d.NT - 1;
  const int64_t ntile = d.NT - bt < NR ? d.NT - bt : NR;
  const __amdgpu_buffer_rsrc_t wres = make_rsrc(d.wpack + bt * d.tile_bytes, (uint32_t)(ntile * d.tile_bytes));
  constexpr int kWPol = NTW ? kNonTemporal : 0;
  uint32_t roff[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) roff[r] = rt0 + r < d.NT ? (uint32_t)(r * d.tile_bytes) : 0u;
  const uint32_t s_unit0 = (uint32_t)(ms0 * UB);                              // sparse unit 0 of the split
  const uint32_t d_unit0 = (uint32_t)((d.n_sm + 2 * md0) * UB) - (uint32_t)ns * UB;  // + k * UB for dense k
  const uint32_t s_idx0 = (uint32_t)(d.idx_off + ms0 * kIdxBlock);
  auto load_step = [&](UnitFrag<WT>(&f)[NR], int k) {
    const bool sp = k < ns;
    const uint32_t uoff = (sp ? s_unit0 : d_unit0) + (uint32_t)k * UB;
    // dense units load their "index" from the unit itself and replace it at use
    const uint32_t ioff = sp ? s_idx0 + (uint32_t)k * kIdxBlock : uoff;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      if constexpr (sizeof(WT) == 1) {
        f[r].a = buf_load16<kWPol>(wres, 16u * lane, roff[r] + uoff);
      } else {
        f[r].a0 = buf_load16<kWPol>(wres, 16u * lane, roff[r] + uoff);
        f[r].a1 = buf_load16<kWPol>(wres, 16u * lane, roff[r] + uoff + 1024u);
      }
      f[r].idx = buf_load4<kWPol>(wres, 4u * lane, roff[r] + ioff);
    }
  };

  // Output scales and columns: loaded up front for small tiles (the epilogue
  // then does not wait on memory); large tiles load them at the end, since
  // 8 registers per row tile held through the K loop would not fit.
  constexpr bool kEarlyOut = NR * MT < 32;
  TileOut to[NR];
  auto load_out = [&]() {
#pragma unroll
    for (int r = 0; r < NR; ++r) to[r] = tile_out(d, rt0 + r < d.NT ? rt0 + r : 0, lane);
  };
  if constexpr (kEarlyOut) load_out();

  UnitFrag<WT> wr[P][NR];
  // every wave streams (waves whose row tiles are all past the end stream a
  // valid tile), so all waves of the workgroup meet the same barriers
  const bool stream = total > 0;
  if (stream) {
#pragma unroll
    for (int i = 0; i < P; ++i) load_step(wr[i], i < total ? i : total - 1);
  }

  // Staging: thread t owns piece position tp = t % kPPR of the staged rows
  // t / kPPR + i * kRowStep (i < kPieces): unit slot jslot, 16-byte piece cp.
  const uint8_t* Xg = (const uint8_t*)a.X + m0 * a.ldx * XB;
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(Xg, (uint32_t)((int64_t)mloc * a.ldx * XB));
  const int tp = (int)threadIdx.x % kPPR;
  const int jslot = tp / kPPU, cp = tp % kPPU;
  const int row0 = (int)threadIdx.x / kPPR;
  const uint32_t xrow0 = (uint32_t)(row0 * a.ldx * XB), xrow_step = (uint32_t)(kRowStep * a.ldx * XB);
  // LDS destination of piece 0 (the others follow every kRowStep rows); W8A8
  // pieces are written as two 8-byte halves with the middle quarters of every
  // 32-byte group swapped
  const int dst0 = row0 * kPitch + kSlot * jslot + (A8 ? 32 * (cp >> 1) + 8 * (cp & 1) : 16 * cp);
  const uint32_t s_col0 = (uint32_t)(128 * ms0 * XB) + 16u * cp;
  const uint32_t d_col0 = (uint32_t)((d.K_sp + 128 * md0) * XB) + 16u * cp;
  u32x4 xv[kPieces];
  auto issue_chunk = [&](int c) {
    const int k = c * CH + jslot;
    const bool kv = k < total && (k < ns || cp < kPPU / 2);
    const uint32_t colb = k < ns ? s_col0 + (uint32_t)(128 * XB * k) : d_col0 + (uint32_t)(64 * XB * (k - ns));
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const bool ok = kv && row0 + i * kRowStep < mloc;
      xv[i] = buf_load16(xres, ok ? xrow0 + i * xrow_step + colb : kOutOfRange, 0u);
    }
  };
  // A piece of a row beyond the batch is not stored, but its load is still
  // consumed (an empty use): a load left pending on one path would make the
  // next chunk's loads wait for every older load before reusing its registers.
  auto write_chunk = [&](uint8_t* buf) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      if (row0 + i * kRowStep < mloc) {
        uint8_t* q = buf + dst0 + i * kRowStep * kPitch;
        if constexpr (A8) {
          *(uint64_t*)q = (uint64_t)xv[i].x | ((uint64_t)xv[i].y << 32);
          *(uint64_t*)(q + 16) = (uint64_t)xv[i].z | ((uint64_t)xv[i].w << 32);
        } else {
          *(u32x4*)q = xv[i];
        }
      } else {
        asm volatile("" : : "v"(xv[i]));
      }
    }
  };

  uint8_t* xbuf0 = xs;
  uint8_t* xbuf1 = xs + rows * kPitch;
  issue_chunk(0);
  write_chunk(xbuf0);
  __syncthreads();

  f32x4 acc[NR * MT], acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < NR * MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Lanes of activation rows beyond the batch read row 0: output column m
  // depends only on B column m, and those columns are never stored.
  int xoff[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) xoff[t] = (16 * t + m < mloc ? 16 * t + m : 0) * kPitch + 32 * (A8 ? (g >> 1) : g);
  const int sp_off = A8 ? 64 * (g & 1) : 128;  // sparse-unit B offset: lane group (W8A8) or second step (bf16)
  auto consume = [&](const UnitFrag<WT>(&f)[NR], int k, int j, const uint8_t* xb) {
    const bool sp = k < ns;
    if constexpr (A8) {
      const int off = kSlot * j + (sp ? sp_off : 0);
      if constexpr (kSplitAcc) {
        const i32x8 B = lds_b8(xb + xoff[0] + off);
        const int idx = sp ? (int)f[0].idx : (int)kDenseIdx;
        if (j & 1) acc1 = smfmac_fp8(f[0].a, B, acc1, idx);
        else acc[0] = smfmac_fp8(f[0].a, B, acc[0], idx);
      } else {
        int idx[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) idx[r] = sp ? (int)f[r].idx : (int)kDenseIdx;
        if constexpr (MT <= 4) {  // every fragment of the unit up front
          i32x8 B[MT];
#pragma unroll
          for (int t = 0; t < MT; ++t) B[t] = lds_b8(xb + xoff[t] + off);
#pragma unroll
          for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int r = 0; r < NR; ++r) acc[r * MT + t] = smfmac_fp8(f[r].a, B[t], acc[r * MT + t], idx[r]);
        } else {  // one fragment ahead
          i32x8 Bc = lds_b8(xb + xoff[0] + off);
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            i32x8 Bn;
            if (t + 1 < MT) Bn = lds_b8(xb + xoff[t + 1] + off);
#pragma unroll
            for (int r = 0; r < NR; ++r) acc[r * MT + t] = smfmac_fp8(f[r].a, Bc, acc[r * MT + t], idx[r]);
            if (t + 1 < MT) Bc = Bn;
          }
        }
      }
    } else {
      const int off0 = kSlot * j, off1 = off0 + (sp ? sp_off : 0);
      if constexpr (kSplitAcc) {
        mac_unit<WT>(acc[0], acc1, f[0], sp ? (int)f[0].idx : (int)kDenseIdx, lds_b16(xb + xoff[0] + off0),
                     lds_b16(xb + xoff[0] + off1));
      } else {
        bf16x8 A0[NR], A1[NR];
        int idx[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          unit_a<WT>(f[r], A0[r], A1[r]);
          idx[r] = sp ? (int)f[r].idx : (int)kDenseIdx;
        }
        if constexpr (MT <= 4) {  // every fragment of the unit up front
          bf16x16 B0[MT], B1[MT];
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            B0[t] = lds_b16(xb + xoff[t] + off0);
            B1[t] = lds_b16(xb + xoff[t] + off1);
          }
#pragma unroll
          for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int r = 0; r < NR; ++r) acc[r * MT + t] = smfmac_bf16<0>(A0[r], B0[t], acc[r * MT + t], idx[r]);
#pragma unroll
          for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int r = 0; r < NR; ++r) acc[r * MT + t] = smfmac_bf16<1>(A1[r], B1[t], acc[r * MT + t], idx[r]);
        } else {  // one m-tile's fragment pair ahead
          bf16x16 B0c = lds_b16(xb + xoff[0] + off0), B1c = lds_b16(xb + xoff[0] + off1);
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            bf16x16 B0n, B1n;
            if (t + 1 < MT) {
              B0n = lds_b16(xb + xoff[t + 1] + off0);
              B1n = lds_b16(xb + xoff[t + 1] + off1);
            }
#pragma unroll
            for (int r = 0; r < NR; ++r) acc[r * MT + t] = smfmac_bf16<0>(A0[r], B0c, acc[r * MT + t], idx[r]);
#pragma unroll
            for (int r = 0; r < NR; ++r) acc[r * MT + t] = smfmac_bf16<1>(A1[r], B1c, acc[r * MT + t], idx[r]);
            if (t + 1 < MT) {
              B0c = B0n;
              B1c = B1n;
            }
          }
        }
      }
    }
  };
  // Full chunks: every ring slot is consumed and refilled, and the next
  // chunk is loaded and staged, unconditionally (after the last chunk that
  // stages zeros into the idle buffer), so every iteration issues the same
  // loads and the loop body has no branch around ring registers (a merge of
  // two paths would copy them, and a copy must wait for their loads to land).
  // The scheduling barriers keep each refill right after the products that
  // free its ring slot (left alone, the scheduler sinks every load of the
  // chunk below its last product, so the next chunk waits on them at once).
  const int nfull = total / CH;
  for (int c = 0; c < nfull; ++c) {
    issue_chunk(c + 1);
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* xb = (c & 1) ? xbuf1 : xbuf0;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int k = c * CH + j;
      consume(wr[j % P], k, j, xb);
      load_step(wr[j % P], k + P < total ? k + P : total - 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    write_chunk((c & 1) ? xbuf0 : xbuf1);
    __syncthreads();
  }
  // last, partial chunk (never followed by another): its first units are in the ring
  if (nfull < nchunks) {
    const int c = nfull;
    const uint8_t* xb = (c & 1) ? xbuf1 : xbuf0;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int k = c * CH + j;
      if (k < total) {
        consume(wr[j % P], k, j, xb);
        if (k + P < total) load_step(wr[j % P], k + P);
      }
    }
  }
  if constexpr (kSplitAcc) acc[0] += acc1;
  if constexpr (!kEarlyOut) load_out();
  finish_tile<NR, MT, A8>(d, a, acc, to, rt0, m0, s, S, (int64_t)mg * p.rgroups + rg, &last_flag);
}

template <typename WT, int NW, int NR, int P, int CH, int MT, bool NTW>
__global__ __launch_bounds__(NW * 64) void linear_stream_kernel(LayerDesc d, LinearArgs a, LinearPlan p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xsb_dyn[];
  __shared__ int last_flag;
  stream_body<WT, false, NW, NR, P, CH, MT, NTW>(d, a, p, blockIdx.x, gridDim.x, xsb_dyn, &last_flag);
}

template <typename WT, int NW, int NR, int P, int CH, int MT, bool NTW>
__global__ __launch_bounds__(NW * 64) void linear_stream2_kernel(LayerDesc d0, LinearArgs a0, LinearPlan p0,
                                                                 LayerDesc d1, LinearArgs a1, LinearPlan p1) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xsb_dyn[];
  __shared__ int last_flag;
  const int g0 = p0.rgroups * p0.splits * p0.mgroups;
  if ((int)blockIdx.x < g0)
    stream_body<WT, false, NW, NR, P, CH, MT, NTW>(d0, a0, p0, blockIdx.x, g0, xsb_dyn, &last_flag);
  else
    stream_body<WT, false, NW, NR, P, CH, MT, NTW>(d1, a1, p1, blockIdx.x - g0, gridDim.x - g0, xsb_dyn, &last_flag);
}

template <int NW, int NR, int P, int CH, int MT, bool NTW>
__global__ __launch_bounds__(NW * 64) void linear_stream8_kernel(LayerDesc d, LinearArgs a, LinearPlan p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xsb_dyn[];
  __shared__ int last_flag;
  stream_body<uint8_t, true, NW, NR, P, CH, MT, NTW>(d, a, p, blockIdx.x, gridDim.x, xsb_dyn, &last_flag);
}

// X'p[m][j] = X[m][pip[j]] (0 where pip[j] < 0), as a contiguous [M][K_p]
// workspace for batches staged by several m-tiles.  One thread per 8 columns.
__global__ void gather_x_kernel(LayerDesc d, const uint16_t* __restrict__ X, int64_t M, int64_t ldx,
                                uint16_t* __restrict__ Xp) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_row = d.K_p / 8;
  if (gid >= M * per_row) return;
  const int64_t mrow = gid / per_row, col = 8 * (gid % per_row);
  *(u32x4*)(Xp + mrow * d.K_p + col) =
      gather8_from(X + mrow * ldx, *(const u32x4*)(d.pip + col), *(const u32x4*)(d.pip + col + 4));
}

// The same X'p for large batches: a workgroup stages `tok` whole rows of X in
// LDS with 16-byte loads, then each thread loads the map entries of its
// 8-column pieces (kGBatch pieces at a time) once and gathers them from LDS for
// every staged row.  The 2-byte gathers run on LDS instead of the memory
// path, and the map is read once per workgroup instead of once per row.
constexpr int kGatherThreads = 512;
constexpr int kGBatch = 4;
__global__ __launch_bounds__(kGatherThreads) void gather_x_rows_kernel(LayerDesc d, const uint16_t* __restrict__ X,
                                                                     int64_t M, int64_t ldx,
                                                                     uint16_t* __restrict__ Xp, int tok) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xr[];  // tok rows of K
  const int64_t K = d.K, m0 = (int64_t)blockIdx.x * tok;
  const int nt = (int)(M - m0 < tok ? M - m0 : tok);
  const int tid = threadIdx.x;
  for (int t = 0; t < nt; ++t) {
    const uint16_t* x = X + (m0 + t) * ldx;
    uint16_t* xs = xr + (int64_t)t * K;
    if (((uintptr_t)x % 16) == 0 && K % 8 == 0) {
      for (int64_t k0 = 8 * (int64_t)tid; k0 < K; k0 += 8 * 4 * kGatherThreads) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t k = k0 + u * 8 * kGatherThreads;
          v[u] = k < K ? *(const u32x4*)(x + k) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t k = k0 + u * 8 * kGatherThreads;
          if (k < K) *(u32x4*)(xs + k) = v[u];
        }
      }
    } else {
      for (int64_t k = tid; k < K; k += kGatherThreads) xs[k] = x[k];
    }
  }
  __syncthreads();
  const int64_t pieces = d.K_p / 8;
  for (int64_t q0 = tid; q0 < pieces; q0 += (int64_t)kGatherThreads * kGBatch) {
    u32x4 i0[kGBatch], i1[kGBatch];
#pragma unroll
    for (int u = 0; u < kGBatch; ++u) {
      const int64_t q = q0 + (int64_t)u * kGatherThreads;
      const int64_t c = q < pieces ? 8 * q : 0;
      i0[u] = *(const u32x4*)(d.pip + c);
      i1[u] = *(const u32x4*)(d.pip + c + 4);
    }
    for (int t = 0; t < nt; ++t) {
#pragma unroll
      for (int u = 0; u < kGBatch; ++u) {
        const int64_t q = q0 + (int64_t)u * kGatherThreads;
        if (q < pieces)
          *(u32x4*)(Xp + (m0 + t) * d.K_p + 8 * q) = gather8_from(xr + (int64_t)t * K, i0[u], i1[u]);
      }
    }
  }
}

// Per-token e4m3 quantisation, one workgroup of 512 threads per token: the
// largest magnitude of the row (a max reduction, exact in any order), the
// scale max/448 as an fp32 quotient (1 for an all-zero row), then each code
// as the round-to-nearest-even e4m3 conversion of the fp32 quotient x / s
// (within range by construction: |x / s| <= 448 up to the quotient's own
// rounding, which still rounds to 448).  Output column j reads column
// pip[j] when a column map is given (the X'p order of a layer; -1: zero).
// With STAGE the row is kept in LDS between the two passes (the re-ordering
// then gathers from LDS); otherwise the second pass reads it again.
// threads per token: two workgroups per CU fit a 27648-column row in LDS,
// so wide workgroups keep more waves resident
constexpr int kQuantThreads = 512;

template <bool STAGE, bool PF>
__global__ __launch_bounds__(kQuantThreads) void quantize_tokens_kernel(const uint16_t* __restrict__ X, int64_t K, int64_t ldx,
                                                              const int32_t* __restrict__ pip, int64_t Kout,
                                                              uint8_t* __restrict__ Q, int64_t ldq,
                                                              float* __restrict__ sx) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xrow[];
  __shared__ float wmax[kQuantThreads / 64];
  const int64_t mrow = blockIdx.x;
  const uint16_t* x = X + mrow * ldx;
  const int tid = threadIdx.x;
  // Second pass: thread t writes 4 consecutive codes per step; the column
  // indices of kBatch steps are loaded together (one memory round trip per
  // kBatch steps instead of one per step; K = 27648: 27 steps).  With PF (few
  // tokens, at most one workgroup per CU) the first two batches are loaded
  // before the first pass, so their round trips overlap the row's; with many
  // tokens the second set of index registers would halve the workgroups a CU
  // holds, and one batch is loaded at a time.
  constexpr int kBatch = 8;
  constexpr int64_t kStep = (int64_t)4 * kQuantThreads * kBatch;
  auto load_src = [&](int64_t jb, int (&src)[kBatch][4]) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t j0 = jb + (int64_t)u * 4 * kQuantThreads;
      if (pip && j0 + 4 <= Kout) {
        const u32x4 p4 = *(const u32x4*)(pip + j0);
#pragma unroll
        for (int t = 0; t < 4; ++t) src[u][t] = (int)p4[t];
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) src[u][t] = j0 + t < Kout ? (pip ? pip[j0 + t] : (int)(j0 + t)) : -1;
      }
    }
  };
  const int64_t jb0 = 4 * (int64_t)tid;
  int sa[kBatch][4], sb[kBatch][4];
  if constexpr (PF) {
    load_src(jb0, sa);
    load_src(jb0 + kStep, sb);
  }
  float amax = 0.f;
  if (((uintptr_t)x % 16) == 0 && K % 8 == 0) {
    // eight 16-byte loads in flight per thread
    for (int64_t k0 = 8 * (int64_t)tid; k0 < K; k0 += 8 * 8 * kQuantThreads) {
      u32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t k = k0 + u * 8 * kQuantThreads;
        v[u] = k < K ? *(const u32x4*)(x + k) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t k = k0 + u * 8 * kQuantThreads;
        if (STAGE && k < K) *(u32x4*)(xrow + k) = v[u];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          amax = fmaxf(amax, __uint_as_float((v[u][q] & 0x7FFFu) << 16));
          amax = fmaxf(amax, __uint_as_float((v[u][q] >> 16 & 0x7FFFu) << 16));
        }
      }
    }
  } else {
    for (int64_t k = tid; k < K; k += kQuantThreads) {
      const uint16_t v = x[k];
      if (STAGE) xrow[k] = v;
      amax = fmaxf(amax, __uint_as_float((uint32_t)(v & 0x7FFFu) << 16));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  amax = wmax[0];
#pragma unroll
  for (int w = 1; w < kQuantThreads / 64; ++w) amax = fmaxf(amax, wmax[w]);
  const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
  if (tid == 0) sx[mrow] = scale;
  const uint16_t* src_row = STAGE ? xrow : x;
  uint8_t* q = Q + mrow * ldq;
  const bool vec_out = ((uintptr_t)q % 4) == 0;
  auto emit = [&](int64_t jb, const int (&src)[kBatch][4]) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t j0 = jb + (int64_t)u * 4 * kQuantThreads;
      if (j0 < Kout) {
        float v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          v[t] = src[u][t] >= 0 ? __uint_as_float((uint32_t)src_row[src[u][t]] << 16) / scale : 0.f;
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w, true);
        if (vec_out && j0 + 4 <= Kout) {
          *(uint32_t*)(q + j0) = (uint32_t)w;
        } else {
          for (int t = 0; t < 4 && j0 + t < Kout; ++t) q[j0 + t] = (uint8_t)((uint32_t)w >> (8 * t));
        }
      }
    }
  };
  if constexpr (!PF) {
    for (int64_t jb = jb0; jb < Kout; jb += kStep) {
      load_src(jb, sa);
      emit(jb, sa);
    }
    return;
  }
  // batches alternate between the two index sets, each refilled two batches ahead
  for (int64_t jb = jb0; jb < Kout; jb += 2 * kStep) {
    emit(jb, sa);
    if (jb + 2 * kStep < Kout) load_src(jb + 2 * kStep, sa);
    if (jb + kStep < Kout) {
      emit(jb + kStep, sb);
      if (jb + 3 * kStep < Kout) load_src(jb + 3 * kStep, sb);
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
hipError_t launch_pack_units(const LayerDesc& d, const void* W, int64_t ldw, hipStream_t s) {
  if (d.n_sm > 0)
    pack_sparse_kernel<WT><<<blocks_for(d.NT * d.n_sm * 64, 256), 256, 0, s>>>(d, (const WT*)W, ldw);
  if (d.n_dm > 0)
    pack_dense_kernel<WT><<<blocks_for(d.NT * 2 * d.n_dm * 64, 256), 256, 0, s>>>(d, (const WT*)W, ldw);
  return hipGetLastError();
}

template <typename WT>
hipError_t launch_export_units(const LayerDesc& d, void* vals, uint32_t* meta, uint8_t* mask, void* dense,
                               hipStream_t s) {
  if (d.K_s > 0 && (vals || meta || mask))
    export_sparse_kernel<WT><<<blocks_for(d.N * d.meta_words, 256), 256, 0, s>>>(d, (WT*)vals, meta, mask);
  if (d.K_d > 0 && dense) export_dense_kernel<WT><<<blocks_for(d.N * d.K_d, 256), 256, 0, s>>>(d, (WT*)dense);
  return hipGetLastError();
}

// One launch: layer 0 alone, or layers 0 and 1 in one grid (two == true).
struct Launch {
  const LayerDesc* d[2];
  const LinearArgs* a[2];
  const LinearPlan* p[2];
  bool two;
  unsigned grid() const {
    unsigned g = (unsigned)((int64_t)p[0]->rgroups * p[0]->splits * p[0]->mgroups);
    if (two) g += (unsigned)((int64_t)p[1]->rgroups * p[1]->splits * p[1]->mgroups);
    return g;
  }
  int lds() const { return two ? std::max(p[0]->lds_bytes, p[1]->lds_bytes) : p[0]->lds_bytes; }
};

// Kernels that may need more than the default 64 KB of dynamic LDS opt in once.
template <typename K>
hipError_t allow_lds(K kernel, int bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <typename WT, int NW, int P, bool GATHER, bool SWZ>
hipError_t launch_decode_k(const Launch& L, hipStream_t s) {
  hipError_t e;
  if (L.two) {
    auto k = linear_decode2_kernel<WT, NW, P, GATHER, SWZ>;
    if ((e = allow_lds(k, L.lds())) != hipSuccess) return e;
    k<<<L.grid(), NW * 64, L.lds(), s>>>(*L.d[0], *L.a[0], *L.p[0], *L.d[1], *L.a[1], *L.p[1]);
  } else {
    auto k = linear_decode_kernel<WT, NW, P, GATHER, SWZ>;
    if ((e = allow_lds(k, L.lds())) != hipSuccess) return e;
    k<<<L.grid(), NW * 64, L.lds(), s>>>(*L.d[0], *L.a[0], *L.p[0]);
  }
  return hipGetLastError();
}

template <typename WT, int NW, int P>
hipError_t launch_decode_t(const Launch& L, hipStream_t s) {
  const bool swz = L.p[0]->swz || (L.two && L.p[1]->swz);
  if (L.two && L.p[0]->swz != L.p[1]->swz) return hipErrorInvalidValue;
  if (L.a[0]->gather) return swz ? launch_decode_k<WT, NW, P, true, true>(L, s) : launch_decode_k<WT, NW, P, true, false>(L, s);
  return swz ? launch_decode_k<WT, NW, P, false, true>(L, s) : launch_decode_k<WT, NW, P, false, false>(L, s);
}

template <typename WT, int NW, int NR, int P, int CH, int MT, bool NTW>
hipError_t launch_stream_k(const Launch& L, hipStream_t s) {
  const LinearPlan& p = *L.p[0];
  if (p.waves != NW || p.nr != NR || p.depth != P || p.chunk != CH || p.mt != MT) return hipErrorInvalidValue;
  hipError_t e;
  if (L.two) {
    auto k = linear_stream2_kernel<WT, NW, NR, P, CH, MT, NTW>;
    if ((e = allow_lds(k, L.lds())) != hipSuccess) return e;
    k<<<L.grid(), NW * 64, L.lds(), s>>>(*L.d[0], *L.a[0], *L.p[0], *L.d[1], *L.a[1], *L.p[1]);
  } else {
    auto k = linear_stream_kernel<WT, NW, NR, P, CH, MT, NTW>;
    if ((e = allow_lds(k, L.lds())) != hipSuccess) return e;
    k<<<L.grid(), NW * 64, L.lds(), s>>>(*L.d[0], *L.a[0], *L.p[0]);
  }
  return hipGetLastError();
}

// single row tile and m-tile per wave (M <= 16, one m-group): X'p contiguous
// (gathered beforehand when needed)
template <typename WT, int NW, int P>
hipError_t launch_stream_t(const Launch& L, hipStream_t s) {
  if (L.a[0]->gather) return hipErrorInvalidValue;
  return launch_stream_k<WT, NW, 1, P, kStreamChunk, 1, true>(L, s);
}

// one m-group in every launched layer: each weight byte is read once
inline bool single_pass(const Launch& L) { return L.p[0]->mgroups == 1 && (!L.two || L.p[1]->mgroups == 1); }

// blocked tiles (SPENSE_TILE_PRESETS): X'p contiguous, gathered beforehand when needed
template <typename WT>
hipError_t launch_stream_preset(const Launch& L, hipStream_t s) {
  if (L.a[0]->gather) return hipErrorInvalidValue;
  switch (L.p[0]->preset) {
#define SPENSE_PRESET(i, nw, nr, pp, ch, mt) \
  case i:                                   \
    if constexpr (preset_codes_only(i)) return hipErrorInvalidValue; \
    else if constexpr (preset_single_pass_variant(i)) { \
      if (single_pass(L)) return launch_stream_k<WT, nw, nr, pp, ch, mt, true>(L, s); \
      return launch_stream_k<WT, nw, nr, pp, ch, mt, false>(L, s); \
    } else return launch_stream_k<WT, nw, nr, pp, ch, mt, false>(L, s);
    SPENSE_TILE_PRESETS(SPENSE_PRESET)
#undef SPENSE_PRESET
    default: return hipErrorInvalidValue;
  }
}

template <typename WT>
hipError_t launch_linear_units(const Launch& L, hipStream_t s) {
  const LinearPlan& p = *L.p[0];
  if (L.two) {  // both layers must run the same kernel shape
    const LinearPlan& q = *L.p[1];
    if (q.chunked != p.chunked || q.preset != p.preset || q.waves != p.waves || q.depth != p.depth ||
        q.nr != p.nr || q.mt != p.mt || q.chunk != p.chunk || L.a[1]->gather != L.a[0]->gather)
      return hipErrorInvalidValue;
  }
  if (p.chunked && p.preset >= 0) return launch_stream_preset<WT>(L, s);
  if (p.chunked) {
    switch (p.waves * 100 + p.depth) {
      case 404: return launch_stream_t<WT, 4, 4>(L, s);
      case 408: return launch_stream_t<WT, 4, 8>(L, s);
      case 804: return launch_stream_t<WT, 8, 4>(L, s);
      case 808: return launch_stream_t<WT, 8, 8>(L, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (p.waves * 100 + p.depth) {
    case 404: return launch_decode_t<WT, 4, 4>(L, s);
    case 408: return launch_decode_t<WT, 4, 8>(L, s);
    case 804: return launch_decode_t<WT, 8, 4>(L, s);
    case 808: return launch_decode_t<WT, 8, 8>(L, s);
    default: return hipErrorInvalidValue;
  }
}

template <int NW, int NR, int P, int CH, int MT, bool NTW>
hipError_t launch_stream8_k(const LayerDesc& d, const LinearArgs& a, const LinearPlan& p, hipStream_t s) {
  if (p.waves != NW || p.nr != NR || p.depth != P || p.chunk != CH || p.mt != MT) return hipErrorInvalidValue;
  auto k = linear_stream8_kernel<NW, NR, P, CH, MT, NTW>;
  const hipError_t e = allow_lds(k, p.lds_bytes);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)((int64_t)p.rgroups * p.splits * p.mgroups);
  k<<<grid, NW * 64, p.lds_bytes, s>>>(d, a, p);
  return hipGetLastError();
}

// W8A8: e4m3 weights, activations already quantised into X'p order
hipError_t launch_linear8(const LayerDesc& d, const LinearArgs& a, const LinearPlan& p, hipStream_t s) {
  if (d.wdtype != DT_FP8 || !p.chunked || a.gather || !a.xscale) return hipErrorInvalidValue;
  if (p.preset >= 0) {
    switch (p.preset) {
#define SPENSE_PRESET(i, nw, nr, pp, ch, mt)                                     \
  case i:                                                                        \
    if constexpr (preset_single_pass_variant(i)) {                               \
      if (p.mgroups == 1) return launch_stream8_k<nw, nr, pp, ch, mt, true>(d, a, p, s); \
    }                                                                            \
    return launch_stream8_k<nw, nr, pp, ch, mt, false>(d, a, p, s);
      SPENSE_TILE_PRESETS(SPENSE_PRESET)
#undef SPENSE_PRESET
      default: return hipErrorInvalidValue;
    }
  }
  switch (p.waves * 100 + p.depth) {
    case 404: return launch_stream8_k<4, 1, 4, kStreamChunk, 1, true>(d, a, p, s);
    case 408: return launch_stream8_k<4, 1, 8, kStreamChunk, 1, true>(d, a, p, s);
    case 804: return launch_stream8_k<8, 1, 4, kStreamChunk, 1, true>(d, a, p, s);
    case 808: return launch_stream8_k<8, 1, 8, kStreamChunk, 1, true>(d, a, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_quantize_tokens(const void* X, int64_t M, int64_t K, int64_t ldx, const int32_t* pip, int64_t Kout,
                                  uint8_t* Q, int64_t ldq, float* sx, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  // rows up to 32768 columns are kept in LDS between the passes (64 KB); the
  // column indices are prefetched when the tokens do not outnumber the CUs
  // (36B-class W8A8 set at M = 128: 194 -> 175 us with the tiled gate/up; at
  // M = 2048 the prefetch measured 7% slower)
  const bool pf = M <= 256;
  const bool stage = K <= 32768;
  const size_t lds = stage ? (size_t)K * 2 : 0;
  auto k = stage ? (pf ? quantize_tokens_kernel<true, true> : quantize_tokens_kernel<true, false>)
                 : (pf ? quantize_tokens_kernel<false, true> : quantize_tokens_kernel<false, false>);
  k<<<(unsigned)M, kQuantThreads, lds, s>>>((const uint16_t*)X, K, ldx, pip, Kout, Q, ldq, sx);
  return hipGetLastError();
}

hipError_t launch_pack(const LayerDesc& d, const void* W, int64_t ldw, hipStream_t s) {
  switch (d.wdtype) {
    case DT_FP8: return launch_pack_units<uint8_t>(d, W, ldw, s);
    case DT_BF16: return launch_pack_units<uint16_t>(d, W, ldw, s);
    case DT_F32:
      if (d.K_s > 0)
        pack_f32_sparse_kernel<<<blocks_for(d.N * d.meta_words, 256), 256, 0, s>>>(d, (const uint32_t*)W, ldw);
      if (d.K_d > 0)
        pack_f32_dense_kernel<<<blocks_for(d.N * d.K_d, 256), 256, 0, s>>>(d, (const uint32_t*)W, ldw);
      return hipGetLastError();
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gather_x(const LayerDesc& d, const void* X, int64_t M, int64_t ldx, void* Xp, hipStream_t s) {
  // large batches: rows staged in LDS, as many per workgroup as fit 112 KB
  // (K = 5120: 8, 10240: 5, 27648: 2), when that still gives 128 workgroups
  constexpr int64_t kGLds = 112 * 1024;
  if (d.K * 2 <= kGLds) {
    const int tok = (int)std::min<int64_t>(8, kGLds / (d.K * 2));
    if ((M + tok - 1) / tok >= 128) {
      const size_t lds = (size_t)tok * d.K * 2;
      auto k = gather_x_rows_kernel;
      if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
      }
      k<<<(unsigned)((M + tok - 1) / tok), kGatherThreads, lds, s>>>(d, (const uint16_t*)X, M, ldx, (uint16_t*)Xp, tok);
      return hipGetLastError();
    }
  }
  gather_x_kernel<<<blocks_for(M * (d.K_p / 8), 256), 256, 0, s>>>(d, (const uint16_t*)X, M, ldx, (uint16_t*)Xp);
  return hipGetLastError();
}

hipError_t launch_export(const LayerDesc& d, void* vals, uint32_t* meta, uint8_t* mask, void* dense, hipStream_t s) {
  switch (d.wdtype) {
    case DT_FP8: return launch_export_units<uint8_t>(d, vals, meta, mask, dense, s);
    case DT_BF16: return launch_export_units<uint16_t>(d, vals, meta, mask, dense, s);
    case DT_F32: {
      hipError_t e = hipSuccess;
      if (vals && d.K_s > 0)
        e = hipMemcpyAsync(vals, d.vals32, (size_t)(d.N * (d.K_s / 2)) * 4, hipMemcpyDeviceToDevice, s);
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
  if (p.lds_preset >= 0) return launch_linear_tile(d, a, p, s);
  if (a.a8) return launch_linear8(d, a, p, s);
  const Launch L{{&d, nullptr}, {&a, nullptr}, {&p, nullptr}, false};
  switch (d.wdtype) {
    case DT_FP8: return launch_linear_units<uint8_t>(L, s);
    case DT_BF16: return launch_linear_units<uint16_t>(L, s);
    case DT_F32:
      linear_f32_kernel<<<blocks_for(d.N, 4), 256, 0, s>>>(d, a);
      return hipGetLastError();
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_linear2(const LayerDesc& d0, const LinearArgs& a0, const LinearPlan& p0, const LayerDesc& d1,
                          const LinearArgs& a1, const LinearPlan& p1, hipStream_t s) {
  if (d0.wdtype != d1.wdtype || p0.lds_preset >= 0 || p1.lds_preset >= 0) return hipErrorInvalidValue;
  const Launch L{{&d0, &d1}, {&a0, &a1}, {&p0, &p1}, true};
  switch (d0.wdtype) {
    case DT_FP8: return launch_linear_units<uint8_t>(L, s);
    case DT_BF16: return launch_linear_units<uint16_t>(L, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_zero_i32(int32_t* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  zero_i32_kernel<<<blocks_for(n, 256), 256, 0, s>>>(p, n);
  return hipGetLastError();
}

// Scratch of the no-allocation entry point: split-K counters, split-K
// partials and gathered activations of one call, in a fixed array that every
// GPU holds for the life of the process.  In host code `scratch` names a
// host-side stand-in, not device memory: the device address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_area(hipStream_t s, uint8_t** base) {
  *base = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    // the counters start at zero (every launch that uses one re-arms it)
    e = launch_zero_i32((int32_t*)p, (int64_t)(kScratchCounterBytes / 4), s);
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = (uint8_t*)p;
  }
  *base = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace spense
