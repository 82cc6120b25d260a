// Internal declarations shared by the host API (spense_api.cpp) and the HIP
// kernels (spense_kernels.hip).  Not part of the public interface.
//
// Device-resident packed form ("unit layout") for bf16 / e4m3 weights.
//
// Output rows are grouped in row tiles of 16 (one matrix-instruction tile).
// The permuted activation X'p is the padded column order: sparse columns
// pi[0..K_s) padded with zero columns to K_sp = 128*n_sm, then dense columns
// pi[K_s..K) padded to 128*n_dm.  Both regions run on
// v_smfmac_f32_16x16x64_bf16.  For a 64-column step at X'p column k0, lane l
// of a wave (r = l % 16, g = l / 16) supplies:
//   B (activations): X'p[m = l%16][k0 + 16g + t], t = 0..15;
//   A (weights of row r): eight values, slot pair j (0..3) covering the 2:4
//     group gl(g, j) = ((g&1)*2 + (j>>1))*4 + (g>>1)*2 + (j&1) of the step,
//     with the pair's two 2-bit positions in bits 4j..4j+3 of the 16-bit index
//     half selected by abid.
// A "unit" holds the A operands of two SMFMACs for every lane (16 values per
// lane: A0 = values 0..7, A1 = values 8..15):
//   sparse unit i (X'p columns 128i..128i+127): A0 = step q=0, A1 = step q=1,
//     plus one index dword per lane (step 0 in bits 0..15, step 1 in 16..31);
//   dense unit t (dense columns 64t..64t+63, one step): A0 = the values at
//     group positions 0 and 1, A1 = positions 2 and 3, with the fixed index
//     word 0xEEEE4444 (abid 0 -> 0x4444, abid 1 -> 0xEEEE), i.e. a dense
//     16x64 block is exactly two structured-sparse products.
// Unit bytes: e4m3 1024 ([64 lanes][16 B]); bf16 2048 ([A0: 64 lanes x 16 B]
// [A1: 64 lanes x 16 B]).  Per row tile: [n_sm sparse units][2*n_dm dense
// units][n_sm index blocks of 64 lanes x 4 B], so every wave streams whole
// 1 KB (e4m3) or 2 KB (bf16) units.  Padding rows, groups and columns hold
// zero values (sparse padding groups use positions (0, 1)).
//
// fp32 weights keep the canonical packed form on the device (vals [N][K_s/2],
// meta [N][ceil(K_s/32)], dense [N][K_d]) and run on a VALU kernel, since the
// structured-sparse matrix instructions have no fp32 form.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spense {

enum : int32_t { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };

constexpr int kRowTile = 16;   // output rows per MFMA tile
constexpr int kMacro = 128;    // X'p columns per macro-step

inline constexpr int64_t unit_bytes(int32_t wdt) { return wdt == DT_FP8 ? 1024 : 2048; }
constexpr int64_t kIdxBlock = 256;  // index dwords of one sparse unit (64 lanes x 4 B)

struct LayerDesc {
  int64_t N, K, K_s, K_d;
  int32_t wdtype;
  int32_t gather;        // 1: X'p[j] = X[pip[j]] (pip[j] < 0 -> 0); 0: X'p is X itself
  int64_t NT;            // row tiles, ceil(N / 16)
  int64_t n_sm, n_dm;    // sparse / dense macro-steps
  int64_t K_sp;          // 128 * n_sm, first dense column of X'p
  int64_t K_p;           // K_sp + 128 * n_dm
  int64_t tile_bytes;    // (n_sm + 2 n_dm) * unit_bytes + n_sm * kIdxBlock
  int64_t idx_off;       // offset of the index blocks within a row tile
  uint8_t* wpack;        // unit layout, NT * tile_bytes bytes
  const float* scales;   // [NT * 16] per packed row (1.0 for bf16 weights; 0 on padding rows)
  const int32_t* ycol;   // [NT * 16] output column of each packed row, -1 on padding rows
  const int32_t* wrow;   // [N] W row of each packed row, or nullptr for W's own row order (pack only)
  const int32_t* pi;     // [K]
  const int32_t* pip;    // [K_p] padded column map
  // fp32 canonical form
  float* vals32;
  uint32_t* meta32;
  float* dense32;
  int64_t meta_words;    // ceil(K_s / 32)
};

struct LinearArgs {
  const void* X;
  int64_t M, ldx;
  void* Y;
  int64_t ldy;
  int32_t ydtype;
  int32_t splits;
  int32_t gather;        // effective gather mode for this call
  int32_t glu;           // 1: packed rows come in (gate, up) pairs; write silu(gate) * up at the pair's column
  int32_t yvec;          // 1: Y is 16-byte aligned and ldy % 4 == 0 (four consecutive columns in one store)
  int32_t a8;            // 1: X is e4m3 codes [M][K_p] in X'p order, with per-token scales xscale (W8A8)
  const float* xscale;   // [M] (a8 only)
  float* ws;             // [splits][M][NT*16] fp32 partials (splits > 1)
  int32_t* counters;     // [row groups * m groups], zero between calls
};

// Launch configuration chosen on the host.
struct LinearPlan {
  int mt;        // m-tiles (16 rows of X each) per wave: 1, 2 or 4
  int mgroups;   // ceil(M / (16 * mt))
  int rgroups;   // ceil(NT / (waves * nr))
  int splits;
  int waves;     // waves per workgroup: 4 or 8
  int depth;     // units in flight per row tile of a wave (ring depth)
  int lds_bytes; // dynamic LDS
  int chunked;   // 0: linear_decode_kernel (whole split staged); 1: linear_stream_kernel
  int chunk;     // units per staged chunk of linear_stream_kernel
  int nr;        // row tiles per wave (linear_stream_kernel)
  int preset;    // index into SPENSE_TILE_PRESETS, or -1 (one row tile and m-tile per wave)
  int xcd_remap; // 1: logical workgroup id = XCD-major remap of blockIdx (grid a multiple of 8)
  int lds_preset = -1; // >= 0: linear_tile_kernel configuration (spense_tile.hip); waves, mt (m-tiles
                  // per workgroup) and nr (row tiles per workgroup) then describe it, chunk is 1
  int swz = 0;    // linear_decode_kernel: unpadded, swizzled staged rows (taken where padded rows do not fit)
  int rblock = 1; // > 1: several m-groups run their row groups in blocks of rblock (see tile_coords)
};

// Configurations of linear_tile_kernel (weight units and activation
// fragments both staged through LDS): waves along output rows, waves along
// tokens, row tiles per wave, m-tiles per wave, stages in the LDS ring.
struct LdsPreset {
  int wr, wm, r, t, ns;
};
int lds_preset_count();
LdsPreset lds_preset(int i);
// LDS of configuration i (its ring of stages) for weights of wdtype and bf16
// activations, or e4m3 activation codes (a8)
int64_t lds_tile_bytes(int i, int32_t wdtype, bool a8);
// copies each wave issues per stage (they must fit the wait counter)
int lds_tile_copies(int i, int32_t wdtype, bool a8);
hipError_t launch_linear_tile(const LayerDesc& d, const LinearArgs& a, const LinearPlan& p, hipStream_t s);

// Blocked configurations of linear_stream_kernel for batches above 16 rows:
// X(index, waves per workgroup, row tiles per wave, ring depth, chunk units, m-tiles).
#define SPENSE_TILE_PRESETS(X) \
  X(0, 8, 1, 4, 8, 2)          \
  X(1, 4, 2, 4, 4, 2)          \
  X(2, 8, 2, 4, 4, 2)          \
  X(3, 8, 1, 4, 4, 4)          \
  X(4, 4, 2, 4, 4, 4)          \
  X(5, 4, 2, 2, 2, 4)          \
  X(6, 8, 2, 2, 2, 4)          \
  X(7, 4, 1, 4, 8, 2)          \
  X(8, 4, 4, 2, 2, 4)          \
  X(9, 8, 4, 2, 2, 4)          \
  X(10, 4, 4, 2, 2, 2)         \
  X(11, 4, 4, 4, 4, 2)         \
  X(12, 8, 2, 4, 4, 4)         \
  X(13, 8, 4, 2, 2, 8)         \
  X(14, 8, 4, 2, 4, 4)         \
  X(15, 8, 1, 8, 8, 1)         \
  X(16, 8, 1, 4, 4, 2)

// Preset 13 runs on e4m3 activation codes only: with bf16 activations its
// eight m-tiles of operand pairs do not fit the registers of two waves per SIMD.
constexpr bool preset_codes_only(int i) { return i == 13; }
// presets the planner runs with one m-group (M <= 32): also built with
// non-temporal weight loads, used when a launch has a single m-group
constexpr bool preset_single_pass_variant(int i) { return i == 0 || i == 2; }

constexpr int kStreamChunk = 8;  // units per activation chunk of linear_stream_kernel

hipError_t launch_pack(const LayerDesc& d, const void* W, int64_t ldw, hipStream_t s);
hipError_t launch_export(const LayerDesc& d, void* vals, uint32_t* meta, uint8_t* mask, void* dense, hipStream_t s);
hipError_t launch_linear(const LayerDesc& d, const LinearArgs& a, const LinearPlan& p, hipStream_t s);
// two layers with the same kernel shape in one grid (the row classes of an output-split layer)
hipError_t launch_linear2(const LayerDesc& d0, const LinearArgs& a0, const LinearPlan& p0, const LayerDesc& d1,
                          const LinearArgs& a1, const LinearPlan& p1, hipStream_t s);
hipError_t launch_zero_i32(int32_t* p, int64_t n, hipStream_t s);

// Fixed device scratch of the no-allocation entry point (spense_kernels.hip):
// kScratchBytes per GPU, the first kScratchCounterBytes holding split-K
// counters that every completed launch leaves at zero.  scratch_area returns
// the current device's copy (its address looked up once per device, its
// counters cleared then by a fill kernel on `s`).
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr size_t kScratchCounterBytes = size_t(64) << 10;
hipError_t scratch_area(hipStream_t s, uint8_t** base);
// SpenseGPT+ scoring (spense_score.hip): diag(X^T X) of a bf16 [T, C] matrix via
// fixed-order chunk partials [C][ceil(T / rows_per_chunk)]; GLU index scores;
// exact top-k selection (ties to the lower index) as a 0/1 mask
hipError_t launch_colsq(const void* X, int64_t T, int64_t C, int64_t ld, float* partial, int64_t rows_per_chunk,
                        float* out, hipStream_t s);
constexpr int64_t kColRows = 64;  // rows per partial sum of the column reductions
// partial: [I][ceil(H / kColRows)] scratch for the down-projection column sums
hipError_t launch_glu_scores(int32_t wdtype, const void* W_gu, const void* W_down, int64_t H, int64_t I, int64_t ld_gu,
                             int64_t ld_down, const float* s_gu, const float* s_down, const float* hx,
                             const float* ha, float* rowscore, float* down_abs, float* partial, float* score,
                             hipStream_t s);
// rank: [n] int32 scratch
hipError_t launch_rank_select(const float* score, int64_t n, int64_t k, int* rank, uint8_t* sel, hipStream_t s);
// Per-token e4m3 quantisation of bf16 X [M][K]: sx[m] = max|X[m]| / 448 (1 for
// an all-zero row), Q[m][j] = e4m3 RNE of X[m][src] / sx[m] for j < Kout with
// src = pip ? pip[j] : j (pip[j] < 0: code 0)
hipError_t launch_quantize_tokens(const void* X, int64_t M, int64_t K, int64_t ldx, const int32_t* pip, int64_t Kout,
                                  uint8_t* Q, int64_t ldq, float* sx, hipStream_t s);
// X'p = X[:, pip] as a contiguous [M][K_p] bf16 buffer
hipError_t launch_gather_x(const LayerDesc& d, const void* X, int64_t M, int64_t ldx, void* Xp, hipStream_t s);

}  // namespace spense
