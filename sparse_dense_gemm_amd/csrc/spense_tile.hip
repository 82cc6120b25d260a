// HIP kernel of the Spense linear layer for batches above 16 rows, as a
// two-level tiled product: weight units and activation fragments are both
// copied straight from memory into LDS, and every wave multiplies a block of
// row tiles by a block of m-tiles out of it.
//
// Method: SpenseGPT gist.science explainer, Technical Summary 2.A (the
// input-split form: a 2:4 region and a dense region along K, both products
// accumulated into one output), on the unit layout of spense_internal.h.
//
// A workgroup of WR x WM waves owns RT = WR R row tiles (16 RT output rows)
// and one m-group of MG = WM T m-tiles (16 MG tokens); wave (wr, wm) computes
// row tiles wr R .. wr R + R - 1 against m-tiles wm T .. wm T + T - 1.  The K
// loop runs over unit-steps (a sparse unit: 128 X'p columns, two
// structured-sparse products; a dense unit: 64 columns, two products with the
// fixed index word).  One stage holds one unit-step: the RT weight units and
// their index blocks, and the activation fragments of the MG m-tiles, each
// laid out exactly as the lanes of a wave read them (16 bytes per lane, so a
// copy of 64 lanes lands as one contiguous 1 KB block and a wave reads it back
// without bank conflicts).  Every wave issues the same copies per stage
// (buffer loads with an LDS destination): its share of the weight units and
// of the m-tiles, spread over the product groups of the stage before.  The
// ring has NS stage buffers, declared as separate arrays and indexed with
// compile-time constants (the loop is unrolled by NS); NS - 1 stages are in
// flight.  The copies are assembly that the compiler does not track, so the
// kernel counts them itself.  One barrier per stage: before it each wave
// waits for its own copies of the stage (the copies of the later stages stay
// in flight) and for its LDS reads of the previous stage; after it the stage
// is complete in LDS and the previous stage's buffer may be refilled.  Each
// weight byte fetched into the CU feeds 16 MG tokens and each activation byte
// 16 RT output rows.
//
// Activations are read from the contiguous X'p (gathered or quantised
// beforehand for a chosen dense set).  Every copy is issued unconditionally:
// one past the end takes an offset beyond its buffer resource and writes
// zeros, so every wave issues the same number of copies per stage and the
// wait counts are static.
#include "spense_device.h"

namespace spense {
namespace {

// Tile configurations: X(index, waves along output rows, waves along tokens,
// row tiles per wave, m-tiles per wave, stages in the LDS ring).  The row
// tiles and the m-tiles of a workgroup must each be a multiple of its waves.
#define SPENSE_LDS_PRESETS(X) \
  X(0, 2, 2, 8, 4, 3)         \
  X(1, 2, 2, 8, 4, 2)         \
  X(2, 2, 2, 4, 4, 3)         \
  X(3, 2, 2, 8, 8, 2)         \
  X(4, 4, 2, 4, 4, 3)         \
  X(5, 2, 4, 8, 2, 3)         \
  X(6, 2, 2, 4, 2, 4)         \
  X(7, 4, 2, 8, 4, 2)

// Buffer descriptor words (the layout make_rsrc builds: base, no stride,
// num_records bytes, raw-buffer flags), uniform across the wave.
__device__ __forceinline__ i32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000;
  return r;
}

// LDS byte address of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)p;
}

// Copies into LDS (buffer loads with an LDS destination): lane l's 16 (or 4)
// bytes at voff + soff of the resource land at LDS address lds + 16 l (4 l);
// offsets beyond the resource write zeros.  They are written as assembly so
// that the compiler does not track them: it would otherwise wait for copies
// into other stage buffers before LDS reads whenever more copies are in
// flight than it follows one by one.  The kernel waits for them itself (a
// counted s_waitcnt before each stage's barrier); no other vector-memory
// load is issued while they are in flight.  NT: non-temporal cache policy.
template <bool NT>
__device__ __forceinline__ void copy16(const i32x4& r, uint32_t lds, uint32_t voff, uint32_t soff) {
  if constexpr (NT)
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen nt lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(lds) : "memory");
  else
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(lds) : "memory");
}
template <bool NT>
__device__ __forceinline__ void copy4(const i32x4& r, uint32_t lds, uint32_t voff, uint32_t soff) {
  if constexpr (NT)
    asm volatile("buffer_load_dword %0, %1, %2 offen nt lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(lds) : "memory");
  else
    asm volatile("buffer_load_dword %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(lds) : "memory");
}

// f(integral_constant<A>), ..., f(integral_constant<B - 1>), in order
template <int A, int B, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (A < B) {
    f(std::integral_constant<int, A>{});
    static_for<A + 1, B>(f);
  }
}

template <typename WT, bool A8, int WR, int WM, int R, int T>
struct TileShape {
  static constexpr int NWV = WR * WM;                       // waves per workgroup
  static constexpr int RT = WR * R;                         // row tiles per workgroup
  static constexpr int MG = WM * T;                         // m-tiles per workgroup
  static constexpr uint32_t UB = sizeof(WT) == 1 ? 1024u : 2048u;  // unit bytes
  static constexpr uint32_t XU = A8 ? 2048u : 4096u;        // activation bytes per m-tile and unit-step
  // Per row tile: its unit, its index block and 16 bytes of padding.  With
  // that stride two index reads cannot be merged into one two-word read
  // (which would lose the buffer it reads, and the compiler would then wait
  // for every copy in flight before it).
  static constexpr uint32_t RS = UB + 256u + 16u;
  static constexpr uint32_t kX = RT * RS;                   // activation fragments after the row tiles
  static constexpr uint32_t kStage = kX + MG * XU;
  static constexpr int kWU = RT / NWV;                      // weight units copied per wave and stage
  static constexpr int kXT = MG / NWV;                      // m-tiles copied per wave and stage
  static constexpr int kXB = A8 ? 2 : 4;                    // 1 KB activation blocks per m-tile
  // copies per wave and stage
  static constexpr int kCopies = kWU * (int)(UB / 1024 + 1) + kXT * kXB;
  static_assert(RT % NWV == 0 && MG % NWV == 0, "every wave copies the same share of a stage");
};

template <typename WT, bool A8, int WR, int WM, int R, int T, int NS, bool NTW>
__global__ __launch_bounds__(WR * WM * 64) void linear_tile_kernel(LayerDesc d, LinearArgs a, LinearPlan p) {
  static_assert(!A8 || sizeof(WT) == 1, "W8A8 takes e4m3 weights");
  static_assert(NS >= 2 && NS <= 4, "two to four stages");
  using S_ = TileShape<WT, A8, WR, WM, R, T>;
  constexpr int NWV = S_::NWV, RT = S_::RT, MG = S_::MG;
  constexpr uint32_t UB = S_::UB, XU = S_::XU, RS = S_::RS, kStage = S_::kStage;
  constexpr int kWait = (NS - 2) * S_::kCopies;
  static_assert(kWait < 64, "wait counts fit the counter");
  constexpr int XB = A8 ? 1 : 2;  // bytes per activation
  __shared__ __attribute__((aligned(1024))) uint8_t st0[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[NS > 2 ? kStage : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[NS > 3 ? kStage : 16];
  __shared__ int last_flag;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave % WR, wm = wave / WR;
  const int g = lane >> 4;

  const int S = p.splits;
  int s, rg, mg;
  tile_coords(blockIdx.x, gridDim.x, p, s, rg, mg);
  const int64_t rt0 = (int64_t)rg * RT;
  int ms0, ms1, md0, md1;
  split_range(d.n_sm, s, S, ms0, ms1);
  split_range(d.n_dm, s, S, md0, md1);
  const int ns = ms1 - ms0, nd = md1 - md0;
  const int total = ns + 2 * nd;  // unit-steps of this split

  // ---- copies.  Weights: one resource over the workgroup's row tiles (row
  // tiles past the last read zero); wave w copies units w, w + NWV, ... ----
  const int64_t ntile = d.NT - rt0 < RT ? d.NT - rt0 : RT;
  const i32x4 wres = rsrc_words(d.wpack + rt0 * d.tile_bytes, (uint32_t)(ntile * d.tile_bytes));
  const uint32_t tb = (uint32_t)d.tile_bytes;
  const uint32_t s_unit0 = (uint32_t)ms0 * UB;                                     // + k UB for sparse k
  const uint32_t d_unit0 = (uint32_t)(d.n_sm + 2 * md0) * UB - (uint32_t)ns * UB;  // + k UB for dense k
  const uint32_t s_idx0 = (uint32_t)(d.idx_off + (int64_t)ms0 * kIdxBlock);
  // Activations: this m-group's rows of X'p; rows past the batch lie beyond
  // the resource and read zero.  A copy takes 8 rows x 128 contiguous bytes
  // (16-byte piece c of row r at lane 8 r + (c ^ r): a row's pieces are
  // rotated so that the 16 lanes of a wave reading one piece of 16 rows hit
  // different banks).  Per m-tile and unit-step, bf16: four blocks (step q,
  // row half rh) holding columns col + 64 q .. + 63 of rows 8 rh .. 8 rh + 7
  // (a dense unit's one step in both q); e4m3 codes: two blocks (row half
  // rh) holding columns col .. col + 127, where for a dense unit piece slot c
  // holds piece c & 3, so that its fragments sit where a sparse unit's do.
  const int64_t m0 = (int64_t)mg * 16 * MG;
  const int64_t mrem = a.M - m0;
  const int mloc = (int)(mrem <= 0 ? 0 : (mrem < 16 * MG ? mrem : 16 * MG));
  const uint8_t* Xg = (const uint8_t*)a.X + (mloc > 0 ? m0 : 0) * a.ldx * XB;
  const i32x4 xres = rsrc_words(Xg, (uint32_t)((int64_t)mloc * a.ldx * XB));
  const int crow = lane >> 3, cslot = (lane & 7) ^ crow;  // copy lane: row within the block, piece slot
  const uint32_t xrow = (uint32_t)(crow * a.ldx * XB), xtile = (uint32_t)(16 * a.ldx * XB),
                 xhalf = (uint32_t)(8 * a.ldx * XB);
  const uint32_t xl_s = xrow + 16u * (uint32_t)cslot, xl_d = xrow + 16u * (uint32_t)(A8 ? (cslot & 3) : cslot);
  // X'p byte column of unit-step k: sparse unit ms0 + k starts at column
  // 128 (ms0 + k), dense unit 2 md0 + k - ns at K_sp + 64 (2 md0 + k - ns)
  const uint32_t s_col = (uint32_t)(128 * ms0) * XB, d_col = (uint32_t)(d.K_sp + 128 * md0 - 64 * ns) * XB;

  // Copy number i (0 .. kCopies - 1, a compile-time index) of this wave's
  // share of unit-step k into buf: first its weight units (each unit's 1 KB
  // pieces, then its index block), then its m-tiles' activation blocks.
  constexpr int kWC = S_::kWU * (int)(UB / 1024 + 1);  // weight copies per wave and stage
  auto issue_one = [&](int k, uint8_t* buf, auto ic) __attribute__((always_inline)) {
    constexpr int i = decltype(ic)::value;
    const bool in = k < total, sp = k < ns;
    if constexpr (i < kWC) {
      constexpr int iu = i / (int)(UB / 1024 + 1), part = i % (int)(UB / 1024 + 1);
      const int r = wave + NWV * iu;
      if constexpr (part < (int)(UB / 1024)) {
        const uint32_t uoff = in ? (uint32_t)r * tb + (sp ? s_unit0 : d_unit0) + (uint32_t)k * UB : kOutOfRange;
        copy16<NTW>(wres, lds_addr(buf + r * RS + 1024 * part), 16 * lane, uoff + 1024u * part);
      } else {
        const uint32_t ioff = in && sp ? (uint32_t)r * tb + s_idx0 + (uint32_t)k * 256u : kOutOfRange;
        copy4<NTW>(wres, lds_addr(buf + r * RS + UB), 4 * lane, ioff);
      }
    } else {
      constexpr int jx = i - kWC, it = jx / S_::kXB, blk = jx % S_::kXB;
      const int t = wave + NWV * it;
      uint8_t* xb = buf + S_::kX + t * XU;
      const uint32_t col = !in ? kOutOfRange : sp ? s_col + (uint32_t)(128 * XB) * k : d_col + (uint32_t)(64 * XB) * k;
      const uint32_t v = (uint32_t)t * xtile + (sp ? xl_s : xl_d);
      if constexpr (A8) {
        copy16<false>(xres, lds_addr(xb + 1024 * blk), v + xhalf * blk, col);
      } else {
        // blocks (step q, row half rh) at 2048 q + 1024 rh; a dense unit uses
        // its one 64-column step for both products: its second step's blocks
        // take the same columns (so that the reads of a stage have fixed LDS
        // offsets)
        constexpr int q = blk & 1, rh = blk >> 1;
        const uint32_t cq = q == 0 || !in ? col : sp ? col + 128u : col;
        copy16<false>(xres, lds_addr(xb + 2048 * q + 1024 * rh), v + xhalf * rh, cq);
      }
    }
  };
  auto issue = [&](int k, uint8_t* buf) __attribute__((always_inline)) {
    static_for<0, S_::kCopies>([&](auto ic) { issue_one(k, buf, ic); });
  };

  // this lane's two 16-byte fragment pieces within an m-tile's block pair:
  // row m = lane % 16 (block rh = m / 8, row m % 8 within it), pieces
  // 2 (lane / 16) + h of a bf16 step, or 4 (g & 1) + 2 (g >> 1) + h of an
  // e4m3 unit (the columns the instruction's B operand takes)
  const int fm = lane & 15, fr = fm & 7;
  const int fp = A8 ? 4 * (g & 1) + 2 * (g >> 1) : 2 * g;
  const uint32_t xo0 = 1024u * (fm >> 3) + 16u * (8 * fr + (fp ^ fr));
  const uint32_t xo1 = 1024u * (fm >> 3) + 16u * (8 * fr + ((fp + 1) ^ fr));

  f32x4 acc[R * T];
#pragma unroll
  for (int i = 0; i < R * T; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Products of the unit-step k staged in buf, in groups (a row tile, or a
  // row tile and step); after group g, between(g) issues the share of the
  // next stage's copies that belongs to it, so that the copies are spread
  // over the products instead of queueing at the stage's start.  Every LDS
  // read of the stage is issued before the first copy (the copies are
  // ordered with memory accesses and may not pass them).
  constexpr int kGroups = A8 ? R : 2 * R;
  auto consume = [&](const uint8_t* buf, int k, auto&& between) __attribute__((always_inline)) {
    const bool sp = k < ns;
    const uint8_t* Wb = buf + (wr * R) * RS + 16 * lane;
    const uint8_t* Ib = buf + (wr * R) * RS + UB + 4 * lane;
    const uint8_t* Xb = buf + S_::kX + (wm * T) * XU;
    // index words are read for dense units too (their blocks hold zeros) and
    // replaced by the dense word, so a stage's reads do not depend on its kind
    int idx[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int v = *(const int*)(Ib + r * RS);
      idx[r] = sp ? v : (int)kDenseIdx;
    }
    if constexpr (A8) {
      i32x8 B[T];
      u32x4 A[R];
#pragma unroll
      for (int t = 0; t < T; ++t) {
        // the instruction pairs byte quarters (0, 2, 1, 3) of the 32 codes
        const i32x4 lo = *(const i32x4*)(Xb + t * XU + xo0), hi = *(const i32x4*)(Xb + t * XU + xo1);
        B[t] = __builtin_shufflevector(lo, hi, 0, 1, 4, 5, 2, 3, 6, 7);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) A[r] = *(const u32x4*)(Wb + r * RS);
      static_for<0, kGroups>([&](auto gc) {
        constexpr int r = decltype(gc)::value;
#pragma unroll
        for (int t = 0; t < T; ++t) acc[r * T + t] = smfmac_fp8(A[r], B[t], acc[r * T + t], idx[r]);
        between(gc);
      });
    } else {
      bf16x16 B[2][T];
      u32x4 w[sizeof(WT) == 1 ? R : 2 * R];
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int t = 0; t < T; ++t)
          B[q][t] = as_bf16x16(*(const u32x4*)(Xb + t * XU + 2048 * q + xo0),
                               *(const u32x4*)(Xb + t * XU + 2048 * q + xo1));
      if constexpr (sizeof(WT) == 1) {
#pragma unroll
        for (int r = 0; r < R; ++r) w[r] = *(const u32x4*)(Wb + r * RS);
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          w[2 * r] = *(const u32x4*)(Wb + r * RS);
          w[2 * r + 1] = *(const u32x4*)(Wb + r * RS + 1024);
        }
      }
      // group g: step q = g / R of row tile r = g % R (both steps of a row
      // tile add into its accumulators in the order q = 0, 1)
      static_for<0, kGroups>([&](auto gc) {
        constexpr int g = decltype(gc)::value, q = g / R, r = g % R;
        bf16x8 A;
        if constexpr (sizeof(WT) == 1) A = q == 0 ? fp8x8_to_bf16(w[r].x, w[r].y) : fp8x8_to_bf16(w[r].z, w[r].w);
        else A = as_bf16x8(w[2 * r + q]);
#pragma unroll
        for (int t = 0; t < T; ++t) acc[r * T + t] = smfmac_bf16<q>(A, B[q][t], acc[r * T + t], idx[r]);
        between(gc);
      });
    }
  };

  uint8_t* const bufs[4] = {st0, st1, st2, st3};
#pragma unroll
  for (int c = 0; c < NS - 1; ++c) issue(c, bufs[c]);
  for (int c0 = 0; c0 < total; c0 += NS) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int c = c0 + j;
      if (c >= total) break;
      // this wave's copies of stage c have landed (those of the next NS - 2
      // stages stay in flight) and its reads of stage c - 1 are done; after
      // the barrier stage c is complete and buffer (c - 1) % NS is free
      __builtin_amdgcn_s_waitcnt((int)((kWait & 15) | ((kWait >> 4) << 14) | (7 << 4) | (0 << 8)));
      barrier_no_fence();
      uint8_t* nb = bufs[(j + NS - 1) % NS];
      consume(bufs[j], c, [&](auto gc) __attribute__((always_inline)) {
        constexpr int g = decltype(gc)::value;
        static_for<g * S_::kCopies / kGroups, (g + 1) * S_::kCopies / kGroups>(
            [&](auto ic) { issue_one(c + NS - 1, nb, ic); });
        __builtin_amdgcn_sched_barrier(0);
      });
    }
  }
  SPENSE_WAIT_VM(0);

  const int64_t rtw = rt0 + wr * R;
  TileOut to[R];
#pragma unroll
  for (int r = 0; r < R; ++r) to[r] = tile_out(d, rtw + r < d.NT ? rtw + r : 0, lane);
  finish_tile<R, T, A8>(d, a, acc, to, rtw, m0 + 16 * wm * T, s, S, (int64_t)mg * p.rgroups + rg, &last_flag);
}

template <typename WT, bool A8, int WR, int WM, int R, int T, int NS>
hipError_t launch_tile_k(const LayerDesc& d, const LinearArgs& a, const LinearPlan& p, hipStream_t s) {
  using S_ = TileShape<WT, A8, WR, WM, R, T>;
  if (p.waves != S_::NWV || p.mt != S_::MG || p.nr != S_::RT || p.chunk != 1) return hipErrorInvalidValue;
  // the ring must fit one CU's LDS (the planner does not pick such a configuration)
  constexpr int64_t kRing = (int64_t)NS * S_::kStage;
  if constexpr (kRing > 160 * 1024 - 1024 || (NS - 2) * S_::kCopies >= 64) {
    return hipErrorInvalidValue;
  } else {
    const unsigned grid = (unsigned)((int64_t)p.rgroups * p.splits * p.mgroups);
    if (p.mgroups == 1)
      linear_tile_kernel<WT, A8, WR, WM, R, T, NS, true><<<grid, S_::NWV * 64, 0, s>>>(d, a, p);
    else
      linear_tile_kernel<WT, A8, WR, WM, R, T, NS, false><<<grid, S_::NWV * 64, 0, s>>>(d, a, p);
    return hipGetLastError();
  }
}

template <typename WT, bool A8>
hipError_t launch_tile_t(const LayerDesc& d, const LinearArgs& a, const LinearPlan& p, hipStream_t s) {
  switch (p.lds_preset) {
#define SPENSE_LDS_CASE(i, wr, wm, r, t, ns) \
  case i: return launch_tile_k<WT, A8, wr, wm, r, t, ns>(d, a, p, s);
    SPENSE_LDS_PRESETS(SPENSE_LDS_CASE)
#undef SPENSE_LDS_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int lds_preset_count() {
  int n = 0;
#define SPENSE_LDS_COUNT(i, wr, wm, r, t, ns) ++n;
  SPENSE_LDS_PRESETS(SPENSE_LDS_COUNT)
#undef SPENSE_LDS_COUNT
  return n;
}

LdsPreset lds_preset(int i) {
  switch (i) {
#define SPENSE_LDS_DESC(i_, wr, wm, r, t, ns) \
  case i_: return LdsPreset{wr, wm, r, t, ns};
    SPENSE_LDS_PRESETS(SPENSE_LDS_DESC)
#undef SPENSE_LDS_DESC
    default: return LdsPreset{0, 0, 0, 0, 0};
  }
}

int64_t lds_tile_bytes(int i, int32_t wdtype, bool a8) {
  const LdsPreset c = lds_preset(i);
  const int64_t rt = (int64_t)c.wr * c.r, mg = (int64_t)c.wm * c.t;
  return (int64_t)c.ns * (rt * (unit_bytes(wdtype) + kIdxBlock + 16) + mg * (a8 ? 2048 : 4096));
}

int lds_tile_copies(int i, int32_t wdtype, bool a8) {
  const LdsPreset c = lds_preset(i);
  const int nw = c.wr * c.wm;
  return (c.wr * c.r / nw) * (int)(unit_bytes(wdtype) / 1024 + 1) + (c.wm * c.t / nw) * (a8 ? 2 : 4);
}

hipError_t launch_linear_tile(const LayerDesc& d, const LinearArgs& a, const LinearPlan& p, hipStream_t s) {
  if (a.gather || p.lds_preset < 0) return hipErrorInvalidValue;
  if (a.a8) {
    if (d.wdtype != DT_FP8 || !a.xscale) return hipErrorInvalidValue;
    return launch_tile_t<uint8_t, true>(d, a, p, s);
  }
  switch (d.wdtype) {
    case DT_FP8: return launch_tile_t<uint8_t, false>(d, a, p, s);
    case DT_BF16: return launch_tile_t<uint16_t, false>(d, a, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace spense
