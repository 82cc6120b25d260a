// HIP kernel of the Spense linear layer for batches above 16 rows: weight
// units staged through LDS and shared by waves that split the token
// dimension.
//
// Method: SpenseGPT gist.science explainer, Technical Summary 2.A (the
// input-split form: a 2:4 region and a dense region along K, both products
// accumulated into one output), on the unit layout of spense_internal.h.
//
// A workgroup owns RT row tiles (16 RT output rows) and one m-group of
// 16 MT NW activation rows.  It has NW consumer waves, wave w taking the MT
// m-tiles w MT .. w MT + MT - 1 of the group, and NP producer waves.  The
// producers copy the weight units of CH consecutive unit-steps of the RT row
// tiles (a "stage": RT CH units and their index blocks) from memory straight
// into LDS (buffer loads with an LDS destination), into a ring of NS stage
// buffers; every consumer multiplies every staged unit, so each weight byte
// fetched into the CU feeds 16 MT NW activation rows (one m-group covers
// M <= 16 MT NW and reads each weight byte once from memory).
//
// The vector-memory counter of a wave completes its loads in issue order, so
// a wave that mixed long-latency weight copies with its own activation loads
// would wait for older weight copies whenever it needs an activation.  Here
// the roles are split by wave: producers issue only weight copies (NS - 1
// stages in flight) and consumers only activation loads (a whole stage ahead,
// in two register sets by stage parity).  One barrier per stage: a producer
// reaches it once its copies of the stage have landed, a consumer once it has
// finished the previous stage; after it the stage is readable by every
// consumer, and the buffer of the previous stage may be refilled.
//
// Activations are read from the contiguous X'p (gathered or quantised
// beforehand for a chosen dense set).  Every load is issued unconditionally:
// loads past the end take an offset beyond their buffer resource and read zero.
#include "spense_device.h"

namespace spense {
namespace {

// Tile configurations: X(index, consumer waves, m-tiles per consumer, row
// tiles per workgroup, unit-steps per stage, stages in the LDS ring,
// producer waves).  RT * CH must be a multiple of the producer count.
#define SPENSE_LDS_PRESETS(X) \
  X(0, 4, 2, 8, 2, 3, 1)      \
  X(1, 4, 1, 8, 2, 3, 1)      \
  X(2, 2, 1, 8, 2, 3, 1)      \
  X(3, 6, 2, 8, 2, 3, 2)      \
  X(4, 8, 1, 8, 2, 4, 2)      \
  X(5, 4, 2, 8, 2, 4, 2)      \
  X(6, 2, 2, 8, 2, 3, 1)

template <typename WT, bool A8, int NW, int MT, int RT, int CH, int NS, int NP, bool NTW>
__global__ __launch_bounds__((NW + NP) * 64) void linear_tile_kernel(LayerDesc d, LinearArgs a, LinearPlan p) {
  static_assert(!A8 || sizeof(WT) == 1, "W8A8 takes e4m3 weights");
  static_assert(NS >= 2 && NS <= 4, "two to four stages");
  constexpr uint32_t UB = sizeof(WT) == 1 ? 1024u : 2048u;  // unit bytes
  constexpr int kUnits = RT * CH;                           // units per stage
  static_assert(kUnits % NP == 0, "every producer copies the same number of units");
  constexpr int kUP = kUnits / NP;                          // units copied per producer and stage
  constexpr int kDMA = kUP * (int)(UB / 1024 + 1);          // copies per producer and stage
  static_assert((NS - 2) * kDMA < 64, "wait counts fit the counter");
  constexpr uint32_t kIdx = (uint32_t)kUnits * UB;          // index blocks after the units
  constexpr uint32_t kStage = (uint32_t)kUnits * (UB + 256u);
  constexpr int kWPol = NTW ? kNonTemporal : 0;
  constexpr int XB = A8 ? 1 : 2;                            // bytes per activation
  constexpr int kBL = A8 ? 2 : 4;                           // 16-byte activation loads per m-tile and unit-step
  __shared__ __attribute__((aligned(16))) uint8_t ring[NS * kStage];
  __shared__ int last_flag;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;

  // logical workgroup id (s * rgroups + rg) * mgroups + mg; with several
  // m-groups, consecutive logical ids (the m-groups of one weight slice) are
  // placed on one XCD so that all but the first read the slice from its L2
  int b = blockIdx.x;
  if (p.xcd_remap) b = (b % 8) * ((int)gridDim.x / 8) + b / 8;
  const int S = p.splits;
  int mg = 0, rg = b, s = 0;
  if (p.mgroups > 1) {
    mg = (int)((uint32_t)b % (uint32_t)p.mgroups);
    rg = (int)((uint32_t)b / (uint32_t)p.mgroups);
  }
  if (S > 1) {
    s = (int)((uint32_t)rg / (uint32_t)p.rgroups);
    rg = (int)((uint32_t)rg % (uint32_t)p.rgroups);
  }
  const int64_t rt0 = (int64_t)rg * RT;
  int ms0, ms1, md0, md1;
  split_range(d.n_sm, s, S, ms0, ms1);
  split_range(d.n_dm, s, S, md0, md1);
  const int ns = ms1 - ms0, nd = md1 - md0;
  const int total = ns + 2 * nd;  // unit-steps of this split
  const int nstages = (total + CH - 1) / CH;

  if (wave >= NW) {
    // ---- producer: weight units into the ring.  Unit u = r CH + j of a
    // stage (row tile r, unit-step j) goes to ring slot u; producer q copies
    // units q, q + NP, ...  One resource over the workgroup's row tiles; row
    // tiles past the last read zero (their offsets fall beyond it) ----
    const int q = wave - NW;
    const int64_t ntile = d.NT - rt0 < RT ? d.NT - rt0 : RT;
    const __amdgpu_buffer_rsrc_t wres = make_rsrc(d.wpack + rt0 * d.tile_bytes, (uint32_t)(ntile * d.tile_bytes));
    const uint32_t tb = (uint32_t)d.tile_bytes;
    const uint32_t s_unit0 = (uint32_t)ms0 * UB;                                   // + k UB for sparse k
    const uint32_t d_unit0 = (uint32_t)(d.n_sm + 2 * md0) * UB - (uint32_t)ns * UB;  // + k UB for dense k
    const uint32_t s_idx0 = (uint32_t)(d.idx_off + (int64_t)ms0 * kIdxBlock);
    auto copy_stage = [&](int c) __attribute__((always_inline)) {
      uint8_t* buf = ring + (c % NS) * kStage;
#pragma unroll
      for (int i = 0; i < kUP; ++i) {
        const int u = q + NP * i;
        const int r = u / CH, k = c * CH + u % CH;
        const bool in = k < total;
        const uint32_t uoff = in ? (uint32_t)r * tb + (k < ns ? s_unit0 : d_unit0) + (uint32_t)k * UB : kOutOfRange;
        const uint32_t ioff = in && k < ns ? (uint32_t)r * tb + s_idx0 + (uint32_t)k * 256u : kOutOfRange;
#pragma unroll
        for (int h = 0; h < (int)(UB / 1024); ++h)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, buf + u * UB + 1024 * h, 16, 16 * lane, uoff + 1024u * h, 0,
                                                   kWPol);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, buf + kIdx + u * 256, 4, 4 * lane, ioff, 0, kWPol);
      }
    };
#pragma unroll
    for (int c = 0; c < NS - 1; ++c) copy_stage(c);
    for (int c = 0; c < nstages; ++c) {
      // this producer's copies of stage c have landed (those of the next
      // NS - 2 stages stay in flight), then the barrier; after it every
      // consumer has finished stage c - 1, whose buffer takes stage c + NS - 1
      SPENSE_WAIT_VM((NS - 2) * kDMA);
      barrier_no_fence();
      copy_stage(c + NS - 1);
    }
    SPENSE_WAIT_VM(0);
    // the split-K hand-off meets every wave of the workgroup at two barriers
    if (S > 1) {
      __syncthreads();
      __syncthreads();
    }
    return;
  }

  // ---- consumers.  Activations: this wave's rows m0 .. m0 + 16 MT of X'p;
  // rows past the batch lie beyond the resource and read zero ----
  const int64_t m0 = ((int64_t)mg * NW + wave) * 16 * MT;
  const int64_t mrem = a.M - m0;
  const int mloc = (int)(mrem <= 0 ? 0 : (mrem < 16 * MT ? mrem : 16 * MT));
  const uint8_t* Xw = (const uint8_t*)a.X + (mloc > 0 ? m0 : 0) * a.ldx * XB;
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(Xw, (uint32_t)((int64_t)mloc * a.ldx * XB));
  // per lane and m-tile: row offset plus the lane's column within a sparse
  // unit (vs) or a dense unit (vd); the unit-step's column is a scalar offset
  uint32_t vs[MT], vd[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const uint32_t row = (uint32_t)((16 * t + (lane & 15)) * a.ldx * XB);
    vs[t] = row + (A8 ? (uint32_t)(64 * (g & 1) + 32 * (g >> 1)) : (uint32_t)(32 * g));
    vd[t] = row + (A8 ? (uint32_t)(32 * (g >> 1)) : (uint32_t)(32 * g));
  }
  // X'p byte column of unit-step k: sparse unit ms0 + k starts at column
  // 128 (ms0 + k), dense unit 2 md0 + k - ns at K_sp + 64 (2 md0 + k - ns)
  const uint32_t s_col = (uint32_t)(128 * ms0) * XB, d_col = (uint32_t)(d.K_sp + 128 * md0 - 64 * ns) * XB;
  // activation fragments of a whole stage (CH unit-steps), two sets by stage parity
  u32x4 xb[2][CH][MT][kBL];
  auto load_b = [&](int set, int c) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int k = c * CH + j;
      const bool sp = k < ns;
      // unit-steps past the split read zero (an offset beyond every resource)
      const uint32_t col = k >= total ? kOutOfRange : sp ? s_col + (uint32_t)(128 * XB) * k : d_col + (uint32_t)(64 * XB) * k;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const uint32_t v = sp ? vs[t] : vd[t];
        xb[set][j][t][0] = buf_load16(xres, v, col);
        xb[set][j][t][1] = buf_load16(xres, v + 16u, col);
        if constexpr (!A8) {
          // second step of a sparse unit 64 columns on; a dense unit uses the same fragment twice
          const uint32_t col1 = k >= total ? kOutOfRange : col + (sp ? 128u : 0u);
          xb[set][j][t][2] = buf_load16(xres, v, col1);
          xb[set][j][t][3] = buf_load16(xres, v + 16u, col1);
        }
      }
    }
  };

  f32x4 acc[RT * MT];
#pragma unroll
  for (int i = 0; i < RT * MT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // products of unit-step j of the stage in buf, with activation set `set`
  auto consume = [&](const uint8_t* buf, int j, int k, int set) __attribute__((always_inline)) {
    const bool sp = k < ns;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int u = r * CH + j;
      const int idx = sp ? *(const int*)(buf + kIdx + u * 256 + 4 * lane) : (int)kDenseIdx;
      if constexpr (A8) {
        const u32x4 A = *(const u32x4*)(buf + u * UB + 16 * lane);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          // the instruction pairs byte quarters (0, 2, 1, 3) of the 32 loaded codes
          const i32x4 lo = __builtin_bit_cast(i32x4, xb[set][j][t][0]), hi = __builtin_bit_cast(i32x4, xb[set][j][t][1]);
          const i32x8 B = __builtin_shufflevector(lo, hi, 0, 1, 4, 5, 2, 3, 6, 7);
          acc[r * MT + t] = smfmac_fp8(A, B, acc[r * MT + t], idx);
        }
      } else {
        UnitFrag<WT> f;
        if constexpr (sizeof(WT) == 1) {
          f.a = *(const u32x4*)(buf + u * UB + 16 * lane);
        } else {
          f.a0 = *(const u32x4*)(buf + u * UB + 16 * lane);
          f.a1 = *(const u32x4*)(buf + u * UB + 1024 + 16 * lane);
        }
        bf16x8 A0, A1;
        unit_a<WT>(f, A0, A1);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          acc[r * MT + t] = smfmac_bf16<0>(A0, as_bf16x16(xb[set][j][t][0], xb[set][j][t][1]), acc[r * MT + t], idx);
          acc[r * MT + t] = smfmac_bf16<1>(A1, as_bf16x16(xb[set][j][t][2], xb[set][j][t][3]), acc[r * MT + t], idx);
        }
      }
    }
  };

  // Stage c: the barrier (after it stage c is in LDS), the activations of
  // stage c + 1 into the other register set, then the products of stage c.
  // Two stages per iteration keep the register set of each static.
  auto stage = [&](int c, int set) __attribute__((always_inline)) {
    barrier_no_fence();
    load_b(set ^ 1, c + 1);
    const uint8_t* buf = ring + (c % NS) * kStage;
#pragma unroll
    for (int j = 0; j < CH; ++j) consume(buf, j, c * CH + j, set);
  };
  load_b(0, 0);
  int c = 0;
  for (; c + 2 <= nstages; c += 2) {
    stage(c, 0);
    stage(c + 1, 1);
  }
  if (c < nstages) stage(c, 0);

  TileOut to[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) to[r] = tile_out(d, rt0 + r < d.NT ? rt0 + r : 0, lane);
  finish_tile<RT, MT, A8>(d, a, acc, to, rt0, m0, s, S, (int64_t)mg * p.rgroups + rg, &last_flag);
}

template <typename WT, bool A8, int NW, int MT, int RT, int CH, int NS, int NP>
hipError_t launch_tile_k(const LayerDesc& d, const LinearArgs& a, const LinearPlan& p, hipStream_t s) {
  if (p.waves != NW || p.mt != MT || p.nr != RT || p.chunk != CH) return hipErrorInvalidValue;
  // the ring must fit one CU's LDS (the planner does not pick such a configuration)
  constexpr int64_t kRing = (int64_t)NS * RT * CH * ((sizeof(WT) == 1 ? 1024 : 2048) + 256);
  if constexpr (kRing > 160 * 1024 - 64) {
    return hipErrorInvalidValue;
  } else {
  const unsigned grid = (unsigned)((int64_t)p.rgroups * p.splits * p.mgroups);
  if (p.mgroups == 1)
    linear_tile_kernel<WT, A8, NW, MT, RT, CH, NS, NP, true><<<grid, (NW + NP) * 64, 0, s>>>(d, a, p);
  else
    linear_tile_kernel<WT, A8, NW, MT, RT, CH, NS, NP, false><<<grid, (NW + NP) * 64, 0, s>>>(d, a, p);
  return hipGetLastError();
  }
}

template <typename WT, bool A8>
hipError_t launch_tile_t(const LayerDesc& d, const LinearArgs& a, const LinearPlan& p, hipStream_t s) {
  switch (p.lds_preset) {
#define SPENSE_LDS_CASE(i, nw, mt, rt, ch, ns, np) \
  case i: return launch_tile_k<WT, A8, nw, mt, rt, ch, ns, np>(d, a, p, s);
    SPENSE_LDS_PRESETS(SPENSE_LDS_CASE)
#undef SPENSE_LDS_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int lds_preset_count() {
  int n = 0;
#define SPENSE_LDS_COUNT(i, nw, mt, rt, ch, ns, np) ++n;
  SPENSE_LDS_PRESETS(SPENSE_LDS_COUNT)
#undef SPENSE_LDS_COUNT
  return n;
}

LdsPreset lds_preset(int i) {
  switch (i) {
#define SPENSE_LDS_DESC(i_, nw, mt, rt, ch, ns, np) \
  case i_: return LdsPreset{nw, mt, rt, ch, ns, np};
    SPENSE_LDS_PRESETS(SPENSE_LDS_DESC)
#undef SPENSE_LDS_DESC
    default: return LdsPreset{0, 0, 0, 0, 0, 0};
  }
}

int64_t lds_tile_bytes(int i, int32_t wdtype) {
  const LdsPreset c = lds_preset(i);
  return (int64_t)c.ns * c.rt * c.ch * (unit_bytes(wdtype) + kIdxBlock);
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
