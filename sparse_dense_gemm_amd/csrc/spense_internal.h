// Internal declarations shared by the host API (spense_api.cpp) and the HIP
// kernels (spense_kernels.hip).  Not part of the public interface.
//
// Device-resident packed form ("fragment layout") for bf16 / e4m3 weights.
//
// Output rows are grouped in row tiles of 16 (one MFMA tile).  The permuted
// activation X'p is the padded column order: sparse columns pi[0..K_s) padded
// with zero columns to K_sp = 128*n_sm, then dense columns pi[K_s..K) padded to
// 128*n_dm.  Work proceeds in macro-steps of 128 X'p columns = two 64-column
// MFMA steps q = 0, 1.  For a 64-column step at X'p column k0, lane l of a wave
// (r = l % 16, g = l / 16) uses:
//   B operand (activations): X'p[m = l%16][k0 + 16g + t], t = 0..15.
//   sparse A (v_smfmac_f32_16x16x64_bf16): row r, eight kept values covering
//     four 2:4 groups; slot pair j (0..3) is group k0/4 + gl(g, j) with
//     gl(g, j) = ((g&1)*2 + (j>>1))*4 + (g>>1)*2 + (j&1); the pair's 2-bit
//     indices sit at bits 4j..4j+3 of the step's 16-bit index half (abid = q).
//   dense A (two v_mfma_f32_16x16x32_bf16): row r, dense columns
//     k0 + 16g + t; t = 0..7 pairs with B t = 0..7, t = 8..15 with B t = 8..15.
//
// Per row tile, blocks are stored sparse macro-steps first, then dense ones:
//   e4m3 sparse block (1280 B): [64 lanes][16 B values: step0 slots 0..7, step1 slots 0..7]
//                               [64 lanes][4 B index dword: step0 bits 0..15, step1 bits 16..31]
//   bf16 sparse block (2304 B): [step q][64 lanes][16 B = 8 values] x2, then [64 lanes][4 B]
//   e4m3 dense block (2048 B):  [step q][64 lanes][16 B = 16 values]
//   bf16 dense block (4096 B):  [step q][half h][64 lanes][16 B = 8 values, t = 8h..8h+7]
// Padding rows, padding groups and padding columns hold zero values (sparse
// padding groups use indices (0, 1)).
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

inline constexpr int64_t sparse_block_bytes(int32_t wdt) { return wdt == DT_FP8 ? 1280 : 2304; }
inline constexpr int64_t dense_block_bytes(int32_t wdt) { return wdt == DT_FP8 ? 2048 : 4096; }

struct LayerDesc {
  int64_t N, K, K_s, K_d;
  int32_t wdtype;
  int32_t gather;        // 1: X'p[j] = X[pip[j]] (pip[j] < 0 -> 0); 0: X'p is X itself
  int64_t NT;            // row tiles, ceil(N / 16)
  int64_t n_sm, n_dm;    // sparse / dense macro-steps
  int64_t K_sp;          // 128 * n_sm, first dense column of X'p
  int64_t K_p;           // K_sp + 128 * n_dm
  int64_t tile_bytes;    // n_sm * sparse_block_bytes + n_dm * dense_block_bytes
  uint8_t* wpack;        // fragment layout, NT * tile_bytes bytes
  const float* scales;   // [NT * 16] (e4m3) or nullptr
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
  float* ws;             // [splits][M][NT*16] fp32 partials (splits > 1)
  int32_t* counters;     // [row groups * m groups], zero between calls
};

// Launch configuration chosen on the host.
struct LinearPlan {
  int mt;        // m-tiles (16 rows of X each) per workgroup pass: 1, 2 or 4
  int mgroups;   // ceil(M / (16 * mt))
  int rgroups;   // ceil(NT / waves_per_wg)
  int splits;
};

constexpr int kWavesPerWG = 4;

hipError_t launch_pack(const LayerDesc& d, const void* W, int64_t ldw, hipStream_t s);
hipError_t launch_export(const LayerDesc& d, void* vals, uint32_t* meta, uint8_t* mask, void* dense, hipStream_t s);
hipError_t launch_linear(const LayerDesc& d, const LinearArgs& a, const LinearPlan& p, hipStream_t s);
hipError_t launch_zero_i32(int32_t* p, int64_t n, hipStream_t s);

}  // namespace spense
