// Host side of the Spense C interface: argument validation, dense-set
// resolution, handle ownership, launch planning.  Every check runs before the
// first HIP call, so rejected calls have no side effects.
//
// Dense-set resolution follows the SpenseGPT explainer, Technical Summary 2.A
// and 2.B: the dense region is either the last K_d = round(p*K) columns or a
// chosen column set; pi lists the sparse columns ascending, then the dense
// columns ascending, which moves the chosen set into one contiguous block.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/spense.h"
#include "spense_internal.h"

using namespace spense;

struct spense_layer {
  LayerDesc d{};
  int device = 0;
  std::vector<int32_t> pi_host;
  uint8_t* wpack = nullptr;
  float* scales = nullptr;
  int32_t* pi = nullptr;
  int32_t* pip = nullptr;
  float* vals32 = nullptr;
  uint32_t* meta32 = nullptr;
  float* dense32 = nullptr;
  float* ws = nullptr;
  size_t ws_bytes = 0;
  void* xws = nullptr;  // activations in X'p order: gathered bf16 [M][K_p] (chunked staging of a chosen
                        // dense set), or W8A8 e4m3 codes [M][K_p] followed by the token scales [M]
  size_t xws_bytes = 0;
  int32_t* counters = nullptr;
  size_t n_counters = 0;
  int32_t* ycol = nullptr;  // output column of each packed row, -1 on padding rows
  int32_t* wrow = nullptr;  // W row of each packed row (parts of an output-split layer)
  int64_t weight_bytes = 0;
  int64_t device_bytes = 0;
  // output-split layer (Technical Summary 2.A): no packed form of its own;
  // part[0] holds the 2:4 rows (no dense columns), part[1] the dense rows (no
  // sparse columns); either may be absent.  rho_host = [sparse rows | dense rows].
  int split = 0;  // 0 input-split layer, 1 output-split layer, 2 GLU block
  spense_layer* part[2] = {nullptr, nullptr};
  spense_layer* down = nullptr;  // GLU block: the down projection (input-split, read in rho order)
  int64_t N_s = 0, N_d = 0;
  std::vector<int32_t> rho_host;
};

namespace {

thread_local int g_last_hip = 0;

int hip_fail(hipError_t e) {
  g_last_hip = (int)e;
  return SPENSE_EHIP;
}

bool valid_dtype(int32_t t) { return t == SPENSE_F32 || t == SPENSE_BF16 || t == SPENSE_FP8_E4M3; }

int64_t elem_bytes(int32_t t) { return t == SPENSE_F32 ? 4 : t == SPENSE_BF16 ? 2 : 1; }

void release(spense_layer* h);
void release(spense_layer* h) {
  if (!h) return;
  release(h->part[0]);
  release(h->part[1]);
  release(h->down);
  void* ptrs[] = {h->wpack, h->scales, h->pi,      h->pip, h->vals32, h->meta32,
                  h->dense32, h->ws,   h->counters, h->xws, h->ycol,   h->wrow};
  for (void* p : ptrs)
    if (p) (void)hipFree(p);
  delete h;
}

template <typename T>
hipError_t dev_alloc(T** p, size_t bytes) {
  *p = nullptr;
  if (bytes == 0) return hipSuccess;
  return hipMalloc((void**)p, bytes);
}

// Validate the dense set and build pi.  Returns SPENSE_OK or SPENSE_EINVAL.
int resolve_dense_set(int64_t K, const int32_t* dense_cols, int64_t n_dense, double fraction, std::vector<int32_t>& pi,
                      int64_t& K_s, int64_t& K_d) {
  std::vector<char> is_dense((size_t)K, 0);
  if (dense_cols) {
    if (n_dense < 0 || n_dense > K) return SPENSE_EINVAL;
    for (int64_t i = 0; i < n_dense; ++i) {
      const int32_t c = dense_cols[i];
      if (c < 0 || c >= K) return SPENSE_EINVAL;
      if (is_dense[(size_t)c]) return SPENSE_EINVAL;  // duplicate
      is_dense[(size_t)c] = 1;
    }
    K_d = n_dense;
  } else {
    if (!(fraction >= 0.0 && fraction <= 1.0)) return SPENSE_EINVAL;  // also rejects NaN
    K_d = (int64_t)std::floor(fraction * (double)K + 0.5);
    if (K_d > K) K_d = K;
    for (int64_t c = K - K_d; c < K; ++c) is_dense[(size_t)c] = 1;
  }
  K_s = K - K_d;
  if (K_s % 4 != 0) return SPENSE_EINVAL;
  pi.resize((size_t)K);
  int64_t a = 0, b = K_s;
  for (int64_t c = 0; c < K; ++c) {
    if (is_dense[(size_t)c]) pi[(size_t)b++] = (int32_t)c;
    else pi[(size_t)a++] = (int32_t)c;
  }
  return SPENSE_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// output rows that may be written four columns at a time
int32_t y_vec_ok(const void* Y, int64_t ldy) { return aligned16(Y) && ldy % 4 == 0 ? 1 : 0; }

}  // namespace

extern "C" {

int spense_abi_version(void) { return SPENSE_ABI_VERSION; }

int spense_last_hip_error(void) { return g_last_hip; }

const char* spense_strerror(int status) {
  switch (status) {
    case SPENSE_OK: return "success";
    case SPENSE_EINVAL: return "invalid argument";
    case SPENSE_EUNSUPPORTED: return "unsupported type combination";
    case SPENSE_ENOMEM: return "out of memory";
    case SPENSE_EHIP: return "HIP runtime error";
    case SPENSE_ESCRATCH: return "the call needs more workspace than the fixed scratch of spense_linear_noalloc holds";
    default: return "unknown status";
  }
}

}  // extern "C"

namespace {

// Packs the rows `rows` of W (host list of W row indices; empty = every row in
// order) with column order pi; packed row n writes output column ycol[n]
// (empty = n).  scales (device, fp8 only) are indexed by W row.  Synchronises s.
int build_layer(const void* W, int32_t wdtype, int64_t N, int64_t K, int64_t ldw, const float* scales,
                const std::vector<int32_t>& rows, std::vector<int32_t> pi, int64_t K_s, int64_t K_d,
                const std::vector<int32_t>& ycol, hipStream_t s, spense_layer** out) {
  spense_layer* h = new (std::nothrow) spense_layer();
  if (!h) return SPENSE_ENOMEM;
  h->pi_host = std::move(pi);
  LayerDesc& d = h->d;
  d.N = N;
  d.K = K;
  d.K_s = K_s;
  d.K_d = K_d;
  d.wdtype = wdtype;
  d.NT = (N + kRowTile - 1) / kRowTile;
  d.meta_words = (K_s / 4 + 7) / 8;
  const int64_t b = elem_bytes(wdtype);
  h->weight_bytes = N * (K_s / 2 * b + K_s / 8 + K_d * b);

  hipError_t e = hipGetDevice(&h->device);
  if (e != hipSuccess) {
    release(h);
    return hip_fail(e);
  }
  e = dev_alloc(&h->pi, (size_t)K * 4);
  if (e == hipSuccess) e = hipMemcpyAsync(h->pi, h->pi_host.data(), (size_t)K * 4, hipMemcpyHostToDevice, s);
  d.pi = h->pi;
  if (!rows.empty()) {
    if (e == hipSuccess) e = dev_alloc(&h->wrow, (size_t)N * 4);
    if (e == hipSuccess) e = hipMemcpyAsync(h->wrow, rows.data(), (size_t)N * 4, hipMemcpyHostToDevice, s);
    d.wrow = h->wrow;
  }

  std::vector<int32_t> pip;
  std::vector<float> sc_host;
  std::vector<int32_t> ycol_host;
  if (wdtype != SPENSE_F32) {
    d.n_sm = (K_s + kMacro - 1) / kMacro;
    d.n_dm = (K_d + kMacro - 1) / kMacro;
    d.K_sp = d.n_sm * kMacro;
    d.K_p = d.K_sp + d.n_dm * kMacro;
    d.idx_off = (d.n_sm + 2 * d.n_dm) * unit_bytes(wdtype);
    d.tile_bytes = d.idx_off + d.n_sm * kIdxBlock;
    bool identity = (K_s % kMacro == 0) && (K_d % kMacro == 0);
    for (int64_t c = 0; identity && c < K; ++c) identity = h->pi_host[(size_t)c] == c;
    d.gather = identity ? 0 : 1;
    pip.assign((size_t)d.K_p, -1);
    for (int64_t j = 0; j < K_s; ++j) pip[(size_t)j] = h->pi_host[(size_t)j];
    for (int64_t j = 0; j < K_d; ++j) pip[(size_t)(d.K_sp + j)] = h->pi_host[(size_t)(K_s + j)];
    const size_t wbytes = (size_t)(d.NT * d.tile_bytes);
    h->device_bytes = (int64_t)wbytes;
    if (e == hipSuccess) e = dev_alloc(&h->wpack, wbytes);
    if (e == hipSuccess) e = dev_alloc(&h->pip, (size_t)d.K_p * 4);
    if (e == hipSuccess && d.K_p > 0)
      e = hipMemcpyAsync(h->pip, pip.data(), (size_t)d.K_p * 4, hipMemcpyHostToDevice, s);
    d.wpack = h->wpack;
    d.pip = h->pip;
    // per packed row: output scale (1.0 for bf16 weights) and output column,
    // padded to whole row tiles, so the kernels load both unconditionally
    const size_t tile_rows = (size_t)(d.NT * kRowTile);
    sc_host.assign(tile_rows, wdtype == SPENSE_FP8_E4M3 ? 0.0f : 1.0f);
    if (wdtype == SPENSE_FP8_E4M3) {
      const int64_t Nw = rows.empty() ? N : (int64_t)(*std::max_element(rows.begin(), rows.end())) + 1;
      std::vector<float> all((size_t)Nw);
      if (e == hipSuccess) e = hipMemcpyAsync(all.data(), scales, (size_t)Nw * 4, hipMemcpyDeviceToHost, s);
      if (e == hipSuccess) e = hipStreamSynchronize(s);
      for (int64_t n = 0; n < N && e == hipSuccess; ++n) sc_host[(size_t)n] = all[(size_t)(rows.empty() ? n : rows[(size_t)n])];
    }
    ycol_host.assign(tile_rows, -1);
    for (int64_t n = 0; n < N; ++n) ycol_host[(size_t)n] = ycol.empty() ? (int32_t)n : ycol[(size_t)n];
    if (e == hipSuccess) e = dev_alloc(&h->scales, tile_rows * 4);
    if (e == hipSuccess) e = hipMemcpyAsync(h->scales, sc_host.data(), tile_rows * 4, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = dev_alloc(&h->ycol, tile_rows * 4);
    if (e == hipSuccess) e = hipMemcpyAsync(h->ycol, ycol_host.data(), tile_rows * 4, hipMemcpyHostToDevice, s);
    d.scales = h->scales;
    d.ycol = h->ycol;
  } else {
    d.gather = 1;
    const size_t vbytes = (size_t)(N * (K_s / 2)) * 4, mbytes = (size_t)(N * d.meta_words) * 4,
                 dbytes = (size_t)(N * K_d) * 4;
    h->device_bytes = (int64_t)(vbytes + mbytes + dbytes);
    if (e == hipSuccess) e = dev_alloc(&h->vals32, vbytes);
    if (e == hipSuccess) e = dev_alloc(&h->meta32, mbytes);
    if (e == hipSuccess) e = dev_alloc(&h->dense32, dbytes);
    d.vals32 = h->vals32;
    d.meta32 = h->meta32;
    d.dense32 = h->dense32;
  }
  if (e == hipSuccess) e = launch_pack(d, W, ldw, s);
  // the host staging buffers above are released on return
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    (void)hipStreamSynchronize(s);
    release(h);
    return e == hipErrorOutOfMemory ? (g_last_hip = (int)e, SPENSE_ENOMEM) : hip_fail(e);
  }
  *out = h;
  return SPENSE_OK;
}

int validate_pack(const void* W, int32_t wdtype, int64_t N, int64_t K, int64_t ldw, const float* scales,
                  spense_handle* out) {
  if (!out) return SPENSE_EINVAL;
  *out = nullptr;
  if (!W || !valid_dtype(wdtype)) return SPENSE_EINVAL;
  if (N < 1 || K < 1 || ldw < K) return SPENSE_EINVAL;
  if (N > (int64_t(1) << 31) || K > (int64_t(1) << 31) || N * ldw > (int64_t(1) << 40)) return SPENSE_EINVAL;
  if ((wdtype == SPENSE_FP8_E4M3) != (scales != nullptr)) return SPENSE_EINVAL;
  return SPENSE_OK;
}

}  // namespace

extern "C" {

int spense_pack(const void* W, int32_t wdtype, int64_t N, int64_t K, int64_t ldw, const float* scales,
                const int32_t* dense_cols, int64_t n_dense, double dense_fraction, void* stream, spense_handle* out) {
  // ---- validation (host only) ----
  int rc = validate_pack(W, wdtype, N, K, ldw, scales, out);
  if (rc != SPENSE_OK) return rc;
  std::vector<int32_t> pi;
  int64_t K_s = 0, K_d = 0;
  rc = resolve_dense_set(K, dense_cols, n_dense, dense_fraction, pi, K_s, K_d);
  if (rc != SPENSE_OK) return rc;
  return build_layer(W, wdtype, N, K, ldw, scales, {}, std::move(pi), K_s, K_d, {}, (hipStream_t)stream, out);
}

int spense_pack_rows(const void* W, int32_t wdtype, int64_t N, int64_t K, int64_t ldw, const float* scales,
                     const int32_t* dense_rows, int64_t n_dense, double dense_fraction, void* stream,
                     spense_handle* out) {
  // ---- validation (host only) ----
  int rc = validate_pack(W, wdtype, N, K, ldw, scales, out);
  if (rc != SPENSE_OK) return rc;
  if (wdtype == SPENSE_F32) return SPENSE_EUNSUPPORTED;
  // the dense row set: rows resolve exactly like columns, with K = N; then
  // K must hold whole 2:4 groups when any row is sparse
  std::vector<int32_t> rho;
  int64_t N_s = 0, N_d = 0;
  std::vector<char> is_dense((size_t)N, 0);
  if (dense_rows) {
    if (n_dense < 0 || n_dense > N) return SPENSE_EINVAL;
    for (int64_t i = 0; i < n_dense; ++i) {
      const int32_t r = dense_rows[i];
      if (r < 0 || r >= N || is_dense[(size_t)r]) return SPENSE_EINVAL;
      is_dense[(size_t)r] = 1;
    }
    N_d = n_dense;
  } else {
    if (!(dense_fraction >= 0.0 && dense_fraction <= 1.0)) return SPENSE_EINVAL;
    N_d = std::min<int64_t>(N, (int64_t)std::floor(dense_fraction * (double)N + 0.5));
    for (int64_t r = N - N_d; r < N; ++r) is_dense[(size_t)r] = 1;
  }
  N_s = N - N_d;
  if (N_s > 0 && K % 4 != 0) return SPENSE_EINVAL;
  rho.resize((size_t)N);
  int64_t ia = 0, ib = N_s;
  for (int64_t r = 0; r < N; ++r) rho[(size_t)(is_dense[(size_t)r] ? ib++ : ia++)] = (int32_t)r;

  spense_layer* h = new (std::nothrow) spense_layer();
  if (!h) return SPENSE_ENOMEM;
  h->split = 1;
  h->N_s = N_s;
  h->N_d = N_d;
  h->rho_host = rho;
  h->d.N = N;
  h->d.K = K;
  h->d.K_s = N_s > 0 ? K : 0;
  h->d.K_d = N_d > 0 ? K : 0;
  h->d.wdtype = wdtype;
  (void)hipGetDevice(&h->device);
  std::vector<int32_t> ident((size_t)K);
  for (int64_t c = 0; c < K; ++c) ident[(size_t)c] = (int32_t)c;
  hipStream_t s = (hipStream_t)stream;
  for (int part = 0; part < 2; ++part) {
    const int64_t n = part == 0 ? N_s : N_d;
    if (n == 0) continue;
    const std::vector<int32_t> sel(rho.begin() + (part == 0 ? 0 : N_s), rho.begin() + (part == 0 ? N_s : N));
    rc = build_layer(W, wdtype, n, K, ldw, scales, sel, ident, part == 0 ? K : 0, part == 0 ? 0 : K, sel, s,
                     &h->part[part]);
    if (rc != SPENSE_OK) {
      release(h);
      return rc;
    }
    h->weight_bytes += h->part[part]->weight_bytes;
    h->device_bytes += h->part[part]->device_bytes;
  }
  *out = h;
  return SPENSE_OK;
}

int spense_pack_glu(const void* W_gu, const void* W_down, int32_t wdtype, int64_t H, int64_t I, int64_t ld_gu,
                    int64_t ld_down, const float* s_gu, const float* s_down, const int32_t* dense_idx, int64_t n_dense,
                    double dense_fraction, void* stream, spense_handle* out) {
  // ---- validation (host only) ----
  if (!out) return SPENSE_EINVAL;
  *out = nullptr;
  if (!W_gu || !W_down || !valid_dtype(wdtype)) return SPENSE_EINVAL;
  if (wdtype == SPENSE_F32) return SPENSE_EUNSUPPORTED;
  if (H < 1 || I < 1 || ld_gu < H || ld_down < I) return SPENSE_EINVAL;
  if (H > (int64_t(1) << 30) || I > (int64_t(1) << 30) || 2 * I * ld_gu > (int64_t(1) << 40) ||
      H * ld_down > (int64_t(1) << 40))
    return SPENSE_EINVAL;
  const bool fp8 = wdtype == SPENSE_FP8_E4M3;
  if (fp8 != (s_gu != nullptr) || fp8 != (s_down != nullptr)) return SPENSE_EINVAL;
  // one dense set of intermediate indices: gate/up rows and down columns
  std::vector<int32_t> rho;
  int64_t I_s = 0, I_d = 0;
  int rc = resolve_dense_set(I, dense_idx, n_dense, dense_fraction, rho, I_s, I_d);
  if (rc != SPENSE_OK) return rc;
  if (I_s > 0 && H % 4 != 0) return SPENSE_EINVAL;

  spense_layer* h = new (std::nothrow) spense_layer();
  if (!h) return SPENSE_ENOMEM;
  h->split = 2;
  h->N_s = I_s;
  h->N_d = I_d;
  h->rho_host = rho;
  h->d.N = H;
  h->d.K = H;
  h->d.wdtype = wdtype;
  (void)hipGetDevice(&h->device);
  hipStream_t s = (hipStream_t)stream;
  // Gate/up: intermediate index i contributes W_gu rows i (gate) and I + i
  // (up), packed next to each other so that one lane holds both results; the
  // pair writes column j = position of i in rho of the intermediate.
  std::vector<int32_t> ident((size_t)H);
  for (int64_t c = 0; c < H; ++c) ident[(size_t)c] = (int32_t)c;
  for (int part = 0; part < 2; ++part) {
    const int64_t n = part == 0 ? I_s : I_d, j0 = part == 0 ? 0 : I_s;
    if (n == 0) continue;
    std::vector<int32_t> wrow((size_t)(2 * n)), ycol((size_t)(2 * n));
    for (int64_t j = 0; j < n; ++j) {
      const int32_t i = rho[(size_t)(j0 + j)];
      wrow[(size_t)(2 * j)] = i;
      wrow[(size_t)(2 * j + 1)] = (int32_t)(I + i);
      ycol[(size_t)(2 * j)] = (int32_t)(j0 + j);
      ycol[(size_t)(2 * j + 1)] = -1;
    }
    rc = build_layer(W_gu, wdtype, 2 * n, H, ld_gu, s_gu, wrow, ident, part == 0 ? H : 0, part == 0 ? 0 : H, ycol, s,
                     &h->part[part]);
    if (rc != SPENSE_OK) {
      release(h);
      return rc;
    }
    h->weight_bytes += h->part[part]->weight_bytes;
    h->device_bytes += h->part[part]->device_bytes;
  }
  // Down: packed through rho (its dense columns become the contiguous tail),
  // then read with the identity map, since the intermediate is already
  // written in rho order: no runtime gather.
  rc = build_layer(W_down, wdtype, H, I, ld_down, s_down, {}, rho, I_s, I_d, {}, s, &h->down);
  if (rc != SPENSE_OK) {
    release(h);
    return rc;
  }
  LayerDesc& dd = h->down->d;
  std::vector<int32_t> pipI((size_t)dd.K_p, -1);
  for (int64_t j = 0; j < I_s; ++j) pipI[(size_t)j] = (int32_t)j;
  for (int64_t j = 0; j < I_d; ++j) pipI[(size_t)(dd.K_sp + j)] = (int32_t)(I_s + j);
  dd.gather = (I_s % kMacro == 0 && I_d % kMacro == 0) ? 0 : 1;
  hipError_t e = hipMemcpy(h->down->pip, pipI.data(), (size_t)dd.K_p * 4, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    release(h);
    return hip_fail(e);
  }
  h->weight_bytes += h->down->weight_bytes;
  h->device_bytes += h->down->device_bytes;
  *out = h;
  return SPENSE_OK;
}

// Optional tuning override "waves,depth[,chunked]" (e.g. "8,4,1") for the decode kernels.
static bool decode_override(int& waves, int& depth, int& chunked) {
  const char* e = std::getenv("SPENSE_DECODE");
  if (!e || !*e) return false;
  int w = 0, dp = 0, ch = -1;
  const int n = std::sscanf(e, "%d,%d,%d", &w, &dp, &ch);
  if (n < 2) return false;
  if ((w != 4 && w != 8) || (dp != 4 && dp != 8)) return false;
  waves = w;
  depth = dp;
  if (n == 3 && (ch == 0 || ch == 1)) chunked = ch;
  return true;
}

// dynamic LDS of the single-shot decode kernel: the whole split's activations
// in M staged rows, plus 16 bytes for the split-K arrival flag when the launch
// has several splits.  Padded rows (swz false) take the larger of the two
// pitches, since a call may run either form (gathered: the split's columns +
// 16 bytes; contiguous: whole 1 KB blocks of 4 unit-steps + 16 bytes);
// swizzled rows are whole 1 KB blocks.
static int64_t decode_lds_bytes(const LayerDesc& d, int64_t M, int64_t S, bool swz = false) {
  const int64_t steps = (d.n_sm + S - 1) / S + (d.n_dm + S - 1) / S;
  const int64_t blocks = (steps + 3) / 4 * 1024;
  const int64_t row = swz ? blocks : std::max(steps * kMacro * 2 + 16, blocks + 16);
  return M * row + (S > 1 ? 16 : 0);
}

// dynamic LDS of the chunked kernels: two chunk buffers of `rows` staged rows,
// each CH unit slots of 128 columns plus a 16-byte pad (xbytes: 2 for bf16
// activations, 1 for e4m3 codes)
static int64_t stream_lds_bytes(int64_t rows, int64_t chunk, int xbytes) {
  return 2 * rows * (chunk * kMacro * xbytes + 16);
}

constexpr int64_t kCUs = 256;             // compute units of the target GPU
// activation leading dimensions (elements) the streaming kernels address with
// 32-bit offsets (128 staged rows of bf16)
constexpr int64_t kMaxLd = int64_t(1) << 23;
constexpr int64_t kLdsPerCU = 160 * 1024;  // LDS bytes per CU
// dynamic LDS a kernel may take: the CU's LDS less room for the kernels' static
// shared variables (the decode kernels have none and may take all of it)
constexpr int64_t kMaxDynLds = kLdsPerCU - 1024;

// SPENSE_LDS=<configuration> runs linear_tile_kernel for batches above 16
// rows; without it the register-blocked streaming kernels run (measured
// faster on every layer and batch size of the workloads), and a forced
// streaming-kernel preset (SPENSE_TILE) takes precedence
static int lds_forced() {
  const char* e = std::getenv("SPENSE_LDS");
  const char* t = std::getenv("SPENSE_TILE");
  if (t && *t) return -1;
  return e && *e ? std::atoi(e) : -1;
}
static bool lds_enabled() { return lds_forced() >= 0; }

// Row groups per block of the workgroup order with several m-groups
// (tile_coords); SPENSE_RBLOCK=<n> overrides the default
static int rblock_choice(int dflt) {
  const char* e = std::getenv("SPENSE_RBLOCK");
  return e && *e ? std::max(1, std::atoi(e)) : dflt;
}

// NT_fill: row tiles launched in the same grid (the layer's own, or both row
// classes of an output-split layer); the split count and the blocking are
// chosen from it so that both classes get the same kernel shape.
static int plan_linear(const spense_layer* h, int64_t M, int32_t splits, int64_t NT_fill, LinearPlan& p,
                       bool force_chunked = false, int xbytes = 2) {
  const LayerDesc& d = h->d;
  // the streaming kernels address a wave's row tiles and a staged m-group of
  // activations with 32-bit offsets
  if (d.tile_bytes >= (int64_t(1) << 29) || d.K_p >= kMaxLd) return SPENSE_EUNSUPPORTED;
  const int64_t steps = std::max<int64_t>(d.n_sm, d.n_dm);
  const int64_t max_splits = std::max<int64_t>(1, std::min<int64_t>(steps, 64));
  if (splits < 0 || splits > max_splits) return SPENSE_EINVAL;
  p = LinearPlan{};
  p.preset = -1;
  p.lds_preset = -1;
  p.nr = 1;
  p.mt = 1;
  p.mgroups = 1;
  if (M <= 16) {
    // decode: one 16-row m-tile, weights streamed through a register ring,
    // 8 waves per workgroup, 4 units in flight per wave.  One split when the
    // row tiles alone give enough waves (each split adds a partial-sum
    // handshake at the end of the kernel), else about 1920 waves (down layer
    // 5120 x 25600: 6 splits; 4 splits measured 4-15% slower).  The split's
    // activations are staged in LDS at once when they fit in 64 KB (no
    // barrier in the K loop), else in double-buffered chunks.
    p.waves = 8;
    p.depth = 4;
    p.chunk = kStreamChunk;
    int w, dp, ch = -1;
    const bool overridden = decode_override(w, dp, ch);
    if (overridden) {
      p.waves = w;
      p.depth = dp;
    }
    int64_t S = splits;
    // Single-shot staging keeps the split's activations in LDS for the whole
    // kernel.  Beyond 64 KB only one workgroup fits on a CU, which costs
    // nothing while the grid has no more workgroups than CUs (gate/up 25600 x
    // 5120: 200); there contiguous activations beat chunked staging up to the
    // CU's 160 KB (M = 8: 19.6 -> 19.1 us, M = 12: 20.1 -> 19.3 us).  Gathered
    // activations stay at 64 KB: their staging issues one 2-byte load per
    // activation, and beyond that the gather pre-pass plus chunked staging is
    // as fast or faster (down 5120 x 25600, 6 splits, M = 8: 24.0 us chunked
    // vs 24.7 single-shot; M = 16: 26.4 vs 33.3 with the earlier staging).
    auto lds_cap = [&](int64_t splits_) {
      const int64_t wgs = (NT_fill + p.waves - 1) / p.waves * splits_;
      return wgs <= kCUs && !d.gather ? kLdsPerCU : int64_t(64) * 1024;
    };
    if (S == 0) {
      S = NT_fill >= 1024 ? 1 : std::max<int64_t>(1, (1920 + NT_fill - 1) / NT_fill);
      S = std::min<int64_t>(S, max_splits);
      if (ch == 0)  // single-shot staging requested: split until it fits
        while (S < max_splits && decode_lds_bytes(d, M, S) > lds_cap(S)) ++S;
    }
    // chunked staging keeps eight waves per workgroup as well (measured on
    // the gate/up layer at M = 8 and 16: 6-7% faster than four) with eight
    // units in flight per wave (4% faster than four there)
    // unpadded swizzled rows where padded ones do not fit (gate/up M = 13-16:
    // 16 x 5120 activations are exactly the CU's 160 KB)
    p.swz = (decode_lds_bytes(d, M, S) > lds_cap(S) && decode_lds_bytes(d, M, S, true) <= lds_cap(S)) ? 1 : 0;
    p.chunked = (force_chunked || ch == 1 || decode_lds_bytes(d, M, S, p.swz) > lds_cap(S)) ? 1 : 0;
    if (p.chunked) p.swz = 0;
    if (p.chunked && !overridden) p.depth = 8;
    p.rgroups = (int)((d.NT + p.waves - 1) / p.waves);
    if (S > 1 && S * M * d.NT * 64 >= (int64_t(1) << 31)) return SPENSE_EUNSUPPORTED;  // 32-bit partial offsets
    p.splits = (int)S;
    p.lds_bytes = (int)(p.chunked ? stream_lds_bytes(M, kStreamChunk, xbytes) : decode_lds_bytes(d, M, S, p.swz));
    return SPENSE_OK;
  }
  // More than 16 rows, one layer per launch, on request: weight units and
  // activation fragments both staged through LDS, each wave multiplying a
  // block of row tiles by a block of m-tiles (linear_tile_kernel).
  // Without a request the planner takes it where it measured faster than the
  // streaming kernels: e4m3 weights, 64 < M <= 256, and at least 3200 row
  // tiles (the gate/up projections of the 32B- and 36B-class layers; 36B-class
  // 55296 x 5120: M = 128 72.1 vs 77.8 us with bf16 activations and 60.7 vs
  // 73.3 us with e4m3 codes, M = 256 132 vs 138 / 107 vs 110 us).  Layers with
  // fewer row tiles, and smaller or larger batches, ran slower on it.
  const char* tile_forced = std::getenv("SPENSE_TILE");
  const bool lds_auto = !lds_enabled() && !(tile_forced && *tile_forced) && d.wdtype == DT_FP8 && M > 64 &&
                        M <= 256 && d.NT >= 3200;
  if (NT_fill == d.NT && (lds_auto || (lds_enabled() && lds_forced() < lds_preset_count()))) {
    const int pre = lds_auto ? (xbytes == 1 ? 5 : 4) : lds_forced();
    const LdsPreset c = lds_preset(pre);
    const bool a8 = xbytes == 1;
    const int64_t rt = (int64_t)c.wr * c.r, mg = (int64_t)c.wm * c.t;
    const int64_t lds = lds_tile_bytes(pre, d.wdtype, a8);
    // the kernel addresses the workgroup's row tiles with 32-bit offsets, its
    // stage ring must fit one CU's LDS and its copies in flight the wait counter
    if (rt * d.tile_bytes < (int64_t(1) << 31) && lds <= kLdsPerCU - 1024 &&
        (c.ns - 2) * lds_tile_copies(pre, d.wdtype, a8) < 64) {
      p.chunked = 1;
      p.lds_preset = pre;
      p.waves = c.wr * c.wm;
      p.mt = (int)mg;
      p.nr = (int)rt;
      p.chunk = 1;
      p.depth = 0;
      p.mgroups = (int)((M + 16 * mg - 1) / (16 * mg));
      p.rgroups = (int)((d.NT + rt - 1) / rt);
      p.lds_bytes = (int)lds;
      int64_t S = splits;
      if (S == 0) {
        // as for the streaming kernels: splits to fill the CUs when the tiles
        // alone do not, fp32 partials below two thirds of the packed weight
        // bytes, and of those split counts the one with the least work on the
        // busiest CU (rounds of resident workgroups, each K / S long)
        const int64_t units = (int64_t)p.rgroups * p.mgroups;
        const int64_t resident = kCUs * std::max<int64_t>(1, kLdsPerCU / lds);
        S = units >= resident / 2 ? 1 : std::max<int64_t>(1, std::min<int64_t>(resident / units, max_splits));
        S = std::max<int64_t>(1, std::min<int64_t>(S, d.tile_bytes / (192 * M)));
        int64_t best = 1;
        double best_cost = 1e30;
        for (int64_t sc = 1; sc <= S; ++sc) {
          const double cost = (double)((units * sc + resident - 1) / resident) / (double)sc;
          if (cost < best_cost * (1 - 1e-9)) {
            best_cost = cost;
            best = sc;
          }
        }
        S = best;
      }
      if (S > 1 && S * M * d.NT * 64 >= (int64_t(1) << 31)) {
        if (splits != 0) return SPENSE_EUNSUPPORTED;
        S = std::max<int64_t>(1, ((int64_t(1) << 31) - 1) / (M * d.NT * 64));
      }
      p.splits = (int)S;
      const int64_t grid = (int64_t)p.rgroups * p.mgroups * S;
      p.xcd_remap = (p.mgroups > 1 && grid % 8 == 0) ? 1 : 0;
      p.rblock = p.mgroups > 1 ? rblock_choice(8) : 1;
      return SPENSE_OK;
    }
  }
  // More than 16 rows: the chunked streaming kernel with register-blocked
  // tiles (row tiles x m-tiles per wave; every weight unit feeds each m-tile,
  // every staged activation fragment each row tile), activations contiguous
  // (a chosen dense set is gathered into a workspace first).  Enough splits
  // to fill the CUs with resident workgroups when the row tiles alone do not.
  struct Preset { int nw, nr, p, ch, mt; };
  static const Preset kPresets[] = {
#define SPENSE_PRESET(i, nw, nr, pp, ch, mt) {nw, nr, pp, ch, mt},
      SPENSE_TILE_PRESETS(SPENSE_PRESET)
#undef SPENSE_PRESET
  };
  constexpr int kNumPresets = (int)(sizeof(kPresets) / sizeof(kPresets[0]));
  // The largest blocking that still gives enough workgroups before splits
  // (thresholds fitted to a sweep of every preset over the four 36B-class
  // layers at M = 32..2048, both activation types: 6% above the best preset
  // per shape in total).  Eight waves per workgroup with four m-tiles each
  // (four row tiles per wave and four-unit chunks for bf16 activations, whose
  // activation loads then run a chunk further ahead; for e4m3 codes eight
  // m-tiles and four row tiles, else two row tiles, whose smaller staged rows
  // let more workgroups share a CU), then eight waves with two row tiles and
  // a deeper ring, then two m-tiles, then one row tile; at M <= 32 one m-group
  // of two m-tiles with two row tiles per wave, or a single row tile (eight
  // waves per workgroup: at M = 32 the QKV 10240 x 5120, O 5120 x 8192 and
  // down 5120 x 25600 layers took 20.7 / 17.0 / 38.1 us with four and 16.9 /
  // 16.8 / 33.6 us with eight).
  auto workgroups = [&](int i) {
    const Preset& c = kPresets[i];
    return (NT_fill + c.nw * c.nr - 1) / (c.nw * c.nr) * ((M + 16 * c.mt - 1) / (16 * c.mt));
  };
  // Layers with few output rows (O and down: 320 row tiles) take two row
  // tiles and two m-tiles per wave from 40 workgroups before splits, which
  // the splits then bring to one per CU (down 5120 x 25600 / 5120 x 27648,
  // weights streamed from HBM: M = 64 36.3 / 45.1 us against 43.4 / 51.9
  // with one row tile per wave; M = 96 with one row tile 58.6 / 66.3 us).
  // Eight single-row-tile waves with an eight-unit ring and one m-tile
  // (preset 15) won a sweep at M = 32 with the layer's weights resident in the
  // last-level cache but lost with them streamed from HBM (30.4 -> 34.5 us),
  // and stays available as a forced preset.
  int pre;
  if (M <= 32) {
    pre = workgroups(2) >= 150 ? 2 : 0;
  } else {
    // (preset, workgroups it needs before splits); e4m3 codes first try eight
    // m-tiles per wave (four row tiles), which halves the weight bytes loaded
    // per product (gate/up 55296x5120 at M = 2048: 574 us vs 645 us).  For
    // bf16 activations the two-row-tile, four-m-tile step takes the two-unit
    // ring and chunk (gate/up 51200 / 55296 x 5120 at M = 64: 51.8 / 54.3 us
    // against 53.7 / 56.3 with four-unit ring and chunk).
    const int64_t need_a8[4][2] = {{13, 150}, {6, 150}, {12, 120}, {2, 64}};
    const int64_t need_a16[4][2] = {{14, 150}, {14, 150}, {6, 120}, {2, 40}};
    pre = 0;
    for (const auto& c : xbytes == 1 ? need_a8 : need_a16)
      if (workgroups((int)c[0]) >= c[1]) {
        pre = (int)c[0];
        break;
      }
    // Few output rows and a long K (down projections): above M = 128 the
    // large tiles with splits beat the small tiles the counts above pick
    // without them (down 5120 x 27648, one layer, weights streamed from HBM:
    // bf16 activations M = 256 / 512 91.5 / 138.6 us against 128.3 / 213.8;
    // e4m3 codes 74.0 / 117.4 against 114.0 / 139.0; for e4m3 codes the
    // two-row-tile tile stays ahead up to M = 384: 95.8 against 103.9 us).
    // Where the counts already reach the eight-m-tile tile of e4m3 codes
    // (M = 2048) it stays: the four-m-tile one took that layer's pass from
    // 1213 to 1334 us.
    if (d.NT * kRowTile <= 8192 && d.K_p >= 16384 && M > 128 && pre != 13) pre = xbytes == 1 && M <= 384 ? 6 : 14;
  }
  if (const char* t = std::getenv("SPENSE_TILE")) {
    // a forced preset whose two staging buffers would not fit in one CU's LDS,
  // or that takes e4m3 codes only, is ignored
    const int v = std::atoi(t);
    if (v >= 0 && v < kNumPresets && (xbytes == 1 || !preset_codes_only(v)) &&
        stream_lds_bytes(std::min<int64_t>(M, 16 * kPresets[v].mt), kPresets[v].ch, xbytes) <= kMaxDynLds)
      pre = v;
  }
  const Preset& q = kPresets[pre];
  p.chunked = 1;
  p.preset = pre;
  p.waves = q.nw;
  p.nr = q.nr;
  p.depth = q.p;
  p.chunk = q.ch;
  p.mt = q.mt;
  p.mgroups = (int)((M + 16 * p.mt - 1) / (16 * p.mt));
  const int64_t rows = std::min<int64_t>(M, 16 * p.mt);
  const int64_t lds = stream_lds_bytes(rows, p.chunk, xbytes);
  p.lds_bytes = (int)lds;
  p.rgroups = (int)((d.NT + p.waves * p.nr - 1) / (p.waves * p.nr));
  int64_t S = splits;
  if (S == 0) {
    const int64_t units = (NT_fill + p.waves * p.nr - 1) / (p.waves * p.nr) * p.mgroups;
    const int64_t resident = kCUs * std::max<int64_t>(1, kLdsPerCU / lds);
    S = units >= kCUs / 2 ? 1 : std::max<int64_t>(1, std::min<int64_t>(resident / units, max_splits));
    // each split writes and reads back fp32 partials of the whole output
    // (8 M N bytes); keep that below two thirds of the packed weight bytes
    // (O 5120 x 8192 at M = 128: three splits 26.2 us, two 29.9 us)
    S = std::max<int64_t>(1, std::min<int64_t>(S, d.tile_bytes / (192 * M)));
    // Of the split counts up to that, take the one with the least work on the
    // busiest CU: a CU whose share of the grid is more than eight waves runs
    // the extra workgroups beside (or after) its first ones, so the launch
    // lasts about ceil(waves / (8 per CU)) workgroup-lengths of K / S each.
    // A grid just past one workgroup per CU is the costly case (QKV 12288 x
    // 5120 at M = 64, weights streamed from HBM: three splits, 288
    // eight-wave workgroups, 37.8 us; two splits, 192 workgroups, 30.1 us).
    int64_t best = 1;
    double best_cost = 1e30;
    for (int64_t s = 1; s <= S; ++s) {
      const int64_t rounds = (units * s * p.waves + kCUs * 8 - 1) / (kCUs * 8);
      const double cost = (double)rounds / (double)s;
      if (cost < best_cost * (1 - 1e-9)) {
        best_cost = cost;
        best = s;
      }
    }
    S = best;
  }
  // the partials are addressed with 32-bit offsets
  if (S > 1 && S * M * d.NT * 64 >= (int64_t(1) << 31)) {
    if (splits != 0) return SPENSE_EUNSUPPORTED;
    S = std::max<int64_t>(1, ((int64_t(1) << 31) - 1) / (M * d.NT * 64));
  }
  p.splits = (int)S;
  const int64_t grid = (int64_t)p.rgroups * p.mgroups * S;
  p.xcd_remap = (p.mgroups > 1 && grid % 8 == 0) ? 1 : 0;  // decided per layer (the remap stays inside it)
  if (const char* x = std::getenv("SPENSE_XCD")) p.xcd_remap = (std::atoi(x) != 0 && grid % 8 == 0) ? 1 : 0;
  // blocks of four row groups when eight or more m-groups share the weights
  // (the 36B-class e4m3 set at M = 2048, 32 m-groups: 1931 -> 1837 us, HBM
  // bytes 5.85 -> 4.07 GB per pass; at M = 128, four m-groups, the blocks
  // read about 20% more bytes for the same time)
  p.rblock = p.mgroups >= 8 ? rblock_choice(4) : 1;
  return SPENSE_OK;
}

// Workspace a call needs on one layer: activations in X'p order (gathered
// bf16 [M][K_p], or W8A8 codes [M][K_p] then the token scales [M]), split-K
// partials and the split-K hand-off counters.
struct WsNeed {
  size_t xws = 0, ws = 0, cnt = 0;
  void grow(const WsNeed& o) {
    xws = std::max(xws, o.xws);
    ws = std::max(ws, o.ws);
    cnt = std::max(cnt, o.cnt);
  }
  bool fits(const spense_layer* h) const { return xws <= h->xws_bytes && ws <= h->ws_bytes && cnt <= h->n_counters; }
};

static size_t a8_codes_bytes(int64_t M, int64_t K_p) { return ((size_t)M * (size_t)K_p + 255) / 256 * 256; }

static WsNeed call_need(const LayerDesc& d, int64_t M, const LinearPlan& p, bool gather_now, bool a8) {
  WsNeed n;
  if (a8) n.xws = a8_codes_bytes(M, d.K_p) + (size_t)M * 4;
  else if (gather_now) n.xws = (size_t)M * (size_t)d.K_p * 2;
  if (p.splits > 1) {
    n.ws = (size_t)p.splits * (size_t)M * (size_t)(d.NT * kRowTile) * 4;
    n.cnt = (size_t)p.rgroups * (size_t)p.mgroups;
  }
  return n;
}

// Batch sizes up to which the workspace of every smaller batch is planned
// exactly when a call grows it; beyond, the planner's own caps bound it.
constexpr int64_t kExactPlanM = 4096;

// Bound on the split-K workspace of any batch size above kExactPlanM: the
// planner keeps S * M below tile_bytes / 256 there, and only splits a launch
// of fewer than kCUs / 2 workgroups (so fewer counters).
static WsNeed large_batch_bound(const LayerDesc& d) {
  WsNeed n;
  n.ws = (size_t)std::min<int64_t>(d.NT * d.tile_bytes / 4, (int64_t(1) << 31) - 1);
  n.cnt = (size_t)std::max<int64_t>(128, d.NT);
  return n;
}

// Replaces h's workspaces with ones of at least `need` (synchronising the
// stream first: earlier launches may still use the old ones).  New counters
// are cleared by a fill kernel on the stream.
static int grow_workspaces(spense_layer* h, const WsNeed& need, hipStream_t s) {
  if (need.fits(h)) return SPENSE_OK;
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e);
  auto regrow = [&](void** ptr, size_t& have, size_t want) -> int {
    if (want <= have) return SPENSE_OK;
    if (*ptr) (void)hipFree(*ptr);
    *ptr = nullptr;
    have = 0;
    const hipError_t err = hipMalloc(ptr, want);
    if (err != hipSuccess) return err == hipErrorOutOfMemory ? (g_last_hip = (int)err, SPENSE_ENOMEM) : hip_fail(err);
    have = want;
    return SPENSE_OK;
  };
  int rc = regrow(&h->xws, h->xws_bytes, need.xws);
  if (rc == SPENSE_OK) rc = regrow((void**)&h->ws, h->ws_bytes, need.ws);
  if (rc == SPENSE_OK && need.cnt > h->n_counters) {
    size_t bytes = h->n_counters * 4;
    rc = regrow((void**)&h->counters, bytes, need.cnt * 4);
    h->n_counters = bytes / 4;
    if (rc == SPENSE_OK) {
      e = launch_zero_i32(h->counters, (int64_t)need.cnt, s);
      if (e != hipSuccess) rc = hip_fail(e);
    }
  }
  return rc;
}

// Workspaces of one call on one layer (the handle's, or carved from the fixed scratch).
struct WsPtrs {
  void* xws = nullptr;
  float* ws = nullptr;
  int32_t* counters = nullptr;
};

static WsPtrs handle_ws(const spense_layer* h) { return WsPtrs{h->xws, h->ws, h->counters}; }

// Points a at this call's workspaces; with gather_now, also writes X'p into
// the gather workspace and points a at it.  The workspaces must fit already.
static int bind_call(const spense_layer* h, int64_t M, const LinearPlan& p, LinearArgs& a, bool gather_now,
                     const WsPtrs& w, hipStream_t s) {
  const LayerDesc& d = h->d;
  if (gather_now) {
    hipError_t e = launch_gather_x(d, a.X, M, a.ldx, w.xws, s);
    if (e != hipSuccess) return hip_fail(e);
    a.X = w.xws;
    a.ldx = d.K_p;
    a.gather = 0;
  }
  if (p.splits > 1) {
    a.ws = w.ws;
    a.counters = w.counters;
  }
  return SPENSE_OK;
}

// Plans one call on `parts` (one layer, or the two row classes of an
// output-split layer, which share one grid and so one kernel shape).
static int plan_call(spense_layer* const* parts, int n_parts, int64_t M, int32_t splits, LinearPlan p[2]) {
  int64_t NT_fill = 0;
  for (int i = 0; i < n_parts; ++i) NT_fill += parts[i]->d.NT;
  for (int i = 0; i < n_parts; ++i) {
    const int rc = plan_linear(parts[i], M, splits, NT_fill, p[i]);
    if (rc != SPENSE_OK) return rc;
  }
  if (n_parts == 2 && splits == 0) {
    // Balance the two row classes: a dense row tile streams more bytes than a
    // 2:4 one (e4m3, K = 5120: 80 KB vs 50 KB), so the heavier class gets
    // proportionally more splits and its waves finish with the others.
    int64_t tile_bytes[2], lightest = 0;
    for (int i = 0; i < 2; ++i) {
      const LayerDesc& q = parts[i]->d;
      tile_bytes[i] = q.n_sm * (unit_bytes(q.wdtype) + kIdxBlock) + 2 * q.n_dm * unit_bytes(q.wdtype);
      lightest = i == 0 ? tile_bytes[0] : std::min(lightest, tile_bytes[i]);
    }
    bool chunk_any = false;
    int32_t S[2];
    for (int i = 0; i < 2; ++i) {
      const LayerDesc& q = parts[i]->d;
      const int64_t max_s = std::max<int64_t>(1, std::min<int64_t>(std::max(q.n_sm, q.n_dm), 64));
      const int64_t ratio = (2 * tile_bytes[i] + lightest) / (2 * lightest);  // rounded
      S[i] = (int32_t)std::min<int64_t>(max_s, (int64_t)p[i].splits * std::max<int64_t>(1, ratio));
      const int rc = plan_linear(parts[i], M, S[i], NT_fill, p[i]);
      if (rc != SPENSE_OK) return rc;
      chunk_any = chunk_any || p[i].chunked;
    }
    // both classes run in one grid, so they need the same kernel shape
    if (chunk_any && !(p[0].chunked && p[1].chunked))
      for (int i = 0; i < 2; ++i) {
        const int rc = plan_linear(parts[i], M, S[i], NT_fill, p[i], true);
        if (rc != SPENSE_OK) return rc;
      }
  }
  // ... and the same staged-row layout (swizzled rows fit wherever padded ones do)
  if (n_parts == 2 && !p[0].chunked && !p[1].chunked && p[0].swz != p[1].swz)
    for (int i = 0; i < 2; ++i) {
      p[i].swz = 1;
      p[i].lds_bytes = (int)decode_lds_bytes(parts[i]->d, M, p[i].splits, true);
    }
  return SPENSE_OK;
}

// Workspaces of every call with automatic splits at a batch size up to M
// (any activation alignment: a chunked launch is assumed to gather), so that
// after one call at M no call at a smaller batch size allocates, which keeps
// such calls capturable in a HIP graph.
static int max_need_parts(spense_layer* const* parts, int n_parts, int64_t M, WsNeed need[2]) {
  LinearPlan p[2]{};
  for (int64_t m = 1; m <= std::min(M, kExactPlanM); ++m) {
    const int rc = plan_call(parts, n_parts, m, 0, p);
    if (rc != SPENSE_OK) return rc;
    for (int i = 0; i < n_parts; ++i) need[i].grow(call_need(parts[i]->d, m, p[i], p[i].chunked && i == 0, false));
  }
  if (M > kExactPlanM) {
    for (int i = 0; i < n_parts; ++i) {
      need[i].grow(large_batch_bound(parts[i]->d));
      if (i == 0) need[i].xws = std::max(need[i].xws, (size_t)M * (size_t)parts[i]->d.K_p * 2);
    }
  }
  return SPENSE_OK;
}

static size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// Plans and launches one layer, or the two row classes of an output-split
// layer in one grid.  `base` carries X, M, Y and the output type.  With
// `scratch` the call's workspaces are carved from that fixed device area
// (counters first, then partials, then the gathered activations) instead of
// the handles' own, and a call that needs more than it holds is refused
// (SPENSE_ESCRATCH) before any launch.
static int run_layers(spense_layer* const* parts, int n_parts, int64_t M, int32_t splits, const LinearArgs& base,
                      hipStream_t s, uint8_t* scratch = nullptr) {
  const bool x_aligned = aligned16(base.X) && (base.ldx % 8) == 0;
  LinearPlan p[2]{};
  LinearArgs aa[2]{base, base};
  int rc = plan_call(parts, n_parts, M, splits, p);
  if (rc != SPENSE_OK) return rc;
  bool gather_now[2] = {false, false};
  WsNeed need[2];
  bool grow = false;
  for (int i = 0; i < n_parts; ++i) {
    aa[i].gather = parts[i]->d.gather || !x_aligned;
    aa[i].splits = p[i].splits;
    // The row classes of an output-split layer see the same activations in
    // the same column order (identity, padded to whole 128-column steps), so
    // one gathered copy serves both.
    gather_now[i] = p[i].chunked && aa[i].gather && i == 0;
    need[i] = call_need(parts[i]->d, M, p[i], gather_now[i], false);
    grow = grow || !need[i].fits(parts[i]);
  }
  WsPtrs w[2];
  if (scratch) {
    size_t cnt = 0, bytes = 0;
    for (int i = 0; i < n_parts; ++i) {
      w[i].counters = (int32_t*)scratch + cnt;
      cnt += need[i].cnt;
      w[i].ws = (float*)(scratch + kScratchCounterBytes + bytes);
      bytes += align256(need[i].ws);
    }
    for (int i = 0; i < n_parts; ++i) {
      w[i].xws = scratch + kScratchCounterBytes + bytes;
      bytes += align256(need[i].xws);
    }
    if (cnt * 4 > kScratchCounterBytes || bytes > kScratchBytes - kScratchCounterBytes) return SPENSE_ESCRATCH;
  } else {
    if (grow) {
      if (splits == 0 && (rc = max_need_parts(parts, n_parts, M, need)) != SPENSE_OK) return rc;
      for (int i = 0; i < n_parts; ++i)
        if ((rc = grow_workspaces(parts[i], need[i], s)) != SPENSE_OK) return rc;
    }
    for (int i = 0; i < n_parts; ++i) w[i] = handle_ws(parts[i]);
  }
  for (int i = 0; i < n_parts; ++i) {
    rc = bind_call(parts[i], M, p[i], aa[i], gather_now[i], w[i], s);
    if (rc != SPENSE_OK) return rc;
    if (i == 1 && p[1].chunked && aa[1].gather) {
      aa[1].X = aa[0].X;
      aa[1].ldx = aa[0].ldx;
      aa[1].gather = 0;
    }
  }
  hipError_t e = n_parts == 1 ? launch_linear(parts[0]->d, aa[0], p[0], s)
                              : launch_linear2(parts[0]->d, aa[0], p[0], parts[1]->d, aa[1], p[1], s);
  return e == hipSuccess ? SPENSE_OK : hip_fail(e);
}

// the layers one call runs: the handle itself, or the row classes of an output-split layer
static int layer_parts(spense_layer* h, spense_layer* parts[2]) {
  if (!h->split) {
    parts[0] = h;
    return 1;
  }
  int n = 0;
  for (spense_layer* q : h->part)
    if (q) parts[n++] = q;
  return n;
}

// spense_linear_splits and spense_linear_noalloc: validation, then the launch
// with the handle's workspaces or the fixed scratch.
static int linear_call(spense_handle h, const void* X, int32_t xdtype, int64_t M, int64_t ldx, void* Y,
                       int32_t ydtype, int64_t ldy, int32_t splits, void* stream, bool noalloc) {
  if (!h || !X || !Y) return SPENSE_EINVAL;
  if (h->split == 2) return SPENSE_EINVAL;  // a GLU block runs through spense_glu
  const LayerDesc& d = h->d;
  if (M < 1 || M > (int64_t(1) << 24) || ldx < d.K || ldy < d.N) return SPENSE_EINVAL;
  if (ldx >= kMaxLd) return SPENSE_EUNSUPPORTED;
  if (!valid_dtype(xdtype) || !valid_dtype(ydtype)) return SPENSE_EINVAL;
  if (ydtype == SPENSE_FP8_E4M3) return SPENSE_EUNSUPPORTED;
  const int32_t want_x = d.wdtype == SPENSE_F32 ? SPENSE_F32 : SPENSE_BF16;
  if (xdtype != want_x) return SPENSE_EUNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;

  LinearArgs a{};
  a.X = X;
  a.M = M;
  a.ldx = ldx;
  a.Y = Y;
  a.ldy = ldy;
  a.yvec = y_vec_ok(Y, ldy);
  a.ydtype = ydtype;
  if (d.wdtype == SPENSE_F32) {
    if (splits > 1) return SPENSE_EINVAL;
    a.splits = 1;
    LinearPlan p{};
    p.mt = p.mgroups = p.rgroups = p.splits = 1;
    hipError_t e = launch_linear(d, a, p, s);
    return e == hipSuccess ? SPENSE_OK : hip_fail(e);
  }
  spense_layer* parts[2] = {nullptr, nullptr};
  const int n_parts = layer_parts(h, parts);
  uint8_t* scratch = nullptr;
  if (noalloc) {
    const hipError_t e = scratch_area(s, &scratch);
    if (e != hipSuccess) return hip_fail(e);
  }
  return run_layers(parts, n_parts, M, splits, a, s, scratch);
}

int spense_linear_splits(spense_handle h, const void* X, int32_t xdtype, int64_t M, int64_t ldx, void* Y,
                         int32_t ydtype, int64_t ldy, int32_t splits, void* stream) {
  return linear_call(h, X, xdtype, M, ldx, Y, ydtype, ldy, splits, stream, false);
}

int spense_linear_noalloc(spense_handle h, const void* X, int32_t xdtype, int64_t M, int64_t ldx, void* Y,
                          int32_t ydtype, int64_t ldy, void* stream) {
  return linear_call(h, X, xdtype, M, ldx, Y, ydtype, ldy, 0, stream, true);
}

int spense_quantize_tokens(const void* X, int64_t M, int64_t K, int64_t ldx, uint8_t* Xq, int64_t ldq, float* sx,
                           void* stream) {
  if (!X || !Xq || !sx) return SPENSE_EINVAL;
  if (M < 1 || M > (int64_t(1) << 24) || K < 1 || ldx < K || ldq < K) return SPENSE_EINVAL;
  const hipError_t e = launch_quantize_tokens(X, M, K, ldx, nullptr, K, Xq, ldq, sx, (hipStream_t)stream);
  return e == hipSuccess ? SPENSE_OK : hip_fail(e);
}

int spense_linear_w8a8(spense_handle h, const void* X, int64_t M, int64_t ldx, void* Y, int32_t ydtype, int64_t ldy,
                       int32_t splits, void* stream) {
  if (!h || !X || !Y) return SPENSE_EINVAL;
  if (h->split != 0) return SPENSE_EUNSUPPORTED;  // input-split layers only
  const LayerDesc& d = h->d;
  if (d.wdtype != SPENSE_FP8_E4M3) return SPENSE_EUNSUPPORTED;
  if (M < 1 || M > (int64_t(1) << 24) || ldx < d.K || ldy < d.N) return SPENSE_EINVAL;
  if (d.K_p >= kMaxLd) return SPENSE_EUNSUPPORTED;
  if (ydtype != SPENSE_F32 && ydtype != SPENSE_BF16) return SPENSE_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  LinearPlan p{};
  int rc = plan_linear(h, M, splits, d.NT, p, true, 1);
  if (rc != SPENSE_OK) return rc;
  WsNeed need = call_need(d, M, p, false, true);
  if (!need.fits(h)) {
    if (splits == 0) {  // every smaller batch size too (graph capture after one eager call)
      LinearPlan q{};
      for (int64_t m = 1; m <= std::min(M, kExactPlanM); ++m) {
        if ((rc = plan_linear(h, m, 0, d.NT, q, true, 1)) != SPENSE_OK) return rc;
        need.grow(call_need(d, m, q, false, true));
      }
      if (M > kExactPlanM) need.grow(large_batch_bound(d));
    }
    if ((rc = grow_workspaces(h, need, s)) != SPENSE_OK) return rc;
  }
  // workspace: the codes [M][K_p] in X'p order, then the token scales [M]
  uint8_t* q = (uint8_t*)h->xws;
  float* sx = (float*)(q + a8_codes_bytes(M, d.K_p));
  // quantise and re-order the columns into X'p in one pass
  hipError_t e = launch_quantize_tokens(X, M, d.K, ldx, d.pip, d.K_p, q, d.K_p, sx, s);
  if (e != hipSuccess) return hip_fail(e);
  LinearArgs a{};
  a.X = q;
  a.M = M;
  a.ldx = d.K_p;
  a.Y = Y;
  a.ldy = ldy;
  a.yvec = y_vec_ok(Y, ldy);
  a.ydtype = ydtype;
  a.splits = p.splits;
  a.a8 = 1;
  a.xscale = sx;
  rc = bind_call(h, M, p, a, false, handle_ws(h), s);
  if (rc != SPENSE_OK) return rc;
  e = launch_linear(d, a, p, s);
  return e == hipSuccess ? SPENSE_OK : hip_fail(e);
}

int spense_glu(spense_handle h, const void* X, int64_t M, int64_t ldx, void* A, int64_t lda, void* Y, int32_t ydtype,
               int64_t ldy, void* stream) {
  if (!h || h->split != 2 || !X || !A || !Y) return SPENSE_EINVAL;
  const int64_t H = h->d.K, I = h->N_s + h->N_d;
  if (M < 1 || M > (int64_t(1) << 24) || ldx < H || lda < I || ldy < H) return SPENSE_EINVAL;
  if (ldx >= kMaxLd || lda >= kMaxLd) return SPENSE_EUNSUPPORTED;
  if (ydtype != SPENSE_F32 && ydtype != SPENSE_BF16) return SPENSE_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  // gate/up (output-split) with the SiLU * up epilogue -> A [M, I] bf16, rho order
  LinearArgs a{};
  a.X = X;
  a.M = M;
  a.ldx = ldx;
  a.Y = A;
  a.ldy = lda;
  a.yvec = y_vec_ok(A, lda);
  a.ydtype = SPENSE_BF16;
  a.glu = 1;
  spense_layer* parts[2] = {nullptr, nullptr};
  int n = 0;
  for (spense_layer* q : h->part)
    if (q) parts[n++] = q;
  int rc = run_layers(parts, n, M, 0, a, s);
  if (rc != SPENSE_OK) return rc;
  // down (input-split, dense tail) on A
  LinearArgs b{};
  b.X = A;
  b.M = M;
  b.ldx = lda;
  b.Y = Y;
  b.ldy = ldy;
  b.yvec = y_vec_ok(Y, ldy);
  b.ydtype = ydtype;
  spense_layer* dp[1] = {h->down};
  return run_layers(dp, 1, M, 0, b, s);
}

int spense_linear(spense_handle h, const void* X, int32_t xdtype, int64_t M, int64_t ldx, void* Y, int32_t ydtype,
                  int64_t ldy, void* stream) {
  return spense_linear_splits(h, X, xdtype, M, ldx, Y, ydtype, ldy, 0, stream);
}

int spense_score_glu(const void* W_gu, const void* W_down, int32_t wdtype, int64_t H, int64_t I, int64_t ld_gu,
                     int64_t ld_down, const float* s_gu, const float* s_down, const void* X_cal, int64_t T,
                     int64_t ld_x, const void* A_cal, int64_t ld_a, float* score, void* stream) {
  // ---- validation (host only) ----
  if (!W_gu || !W_down || !X_cal || !A_cal || !score) return SPENSE_EINVAL;
  if (wdtype != SPENSE_BF16 && wdtype != SPENSE_FP8_E4M3) return valid_dtype(wdtype) ? SPENSE_EUNSUPPORTED : SPENSE_EINVAL;
  if (H < 1 || I < 1 || T < 1 || ld_gu < H || ld_down < I || ld_x < H || ld_a < I) return SPENSE_EINVAL;
  if (H > (int64_t(1) << 30) || I > (int64_t(1) << 30) || T > (int64_t(1) << 30)) return SPENSE_EINVAL;
  const bool fp8 = wdtype == SPENSE_FP8_E4M3;
  if (fp8 != (s_gu != nullptr) || fp8 != (s_down != nullptr)) return SPENSE_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  // scratch: Hx [H], Ha [I], chunk partials, gate/up row scores [2I], down column sums [I]
  constexpr int64_t kRows = 64;  // calibration rows per partial sum
  const int64_t nchunks = std::max((T + kRows - 1) / kRows, (H + kColRows - 1) / kColRows);
  const size_t n_floats = (size_t)(H + I + nchunks * std::max(H, I) + 2 * I + I);
  float* tmp = nullptr;
  hipError_t e = hipMalloc((void**)&tmp, n_floats * 4);
  if (e != hipSuccess) return e == hipErrorOutOfMemory ? SPENSE_ENOMEM : hip_fail(e);
  float* hx = tmp;
  float* ha = hx + H;
  float* partial = ha + I;
  float* rowscore = partial + nchunks * std::max(H, I);
  float* down_abs = rowscore + 2 * I;
  e = launch_colsq(X_cal, T, H, ld_x, partial, kRows, hx, s);
  if (e == hipSuccess) e = launch_colsq(A_cal, T, I, ld_a, partial, kRows, ha, s);
  if (e == hipSuccess)
    e = launch_glu_scores(wdtype, W_gu, W_down, H, I, ld_gu, ld_down, s_gu, s_down, hx, ha, rowscore, down_abs,
                          partial, score, s);
  const hipError_t e2 = hipStreamSynchronize(s);  // the scratch is released on return
  (void)hipFree(tmp);
  if (e == hipSuccess) e = e2;
  return e == hipSuccess ? SPENSE_OK : hip_fail(e);
}

int spense_select_dense(const float* score, int64_t n, int64_t k, int32_t* dense_idx, void* stream) {
  if (!score || n < 1 || n > (int64_t(1) << 30) || k < 0 || k > n || (k > 0 && !dense_idx)) return SPENSE_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* sel = nullptr;  // [n] selection mask, then [n] int32 ranks (4-byte aligned)
  const size_t off = ((size_t)n + 255) / 256 * 256;
  hipError_t e = hipMalloc((void**)&sel, off + (size_t)n * 4);
  if (e != hipSuccess) return e == hipErrorOutOfMemory ? SPENSE_ENOMEM : hip_fail(e);
  std::vector<uint8_t> h_sel((size_t)n);
  e = launch_rank_select(score, n, k, (int*)(sel + off), sel, s);
  if (e == hipSuccess) e = hipMemcpyAsync(h_sel.data(), sel, (size_t)n, hipMemcpyDeviceToHost, s);
  const hipError_t e2 = hipStreamSynchronize(s);
  (void)hipFree(sel);
  if (e == hipSuccess) e = e2;
  if (e != hipSuccess) return hip_fail(e);
  for (int64_t i = 0; i < n; ++i)
    if (h_sel[(size_t)i] == 2) return SPENSE_EINVAL;  // a NaN score
  // the ranks of n numbers are a permutation of 0..n-1, so exactly k are below k
  int64_t m = 0;
  for (int64_t i = 0; i < n && m < k; ++i)
    if (h_sel[(size_t)i]) dense_idx[m++] = (int32_t)i;
  return SPENSE_OK;
}

int spense_info(spense_handle h, spense_layer_info* info) {
  if (!h || !info) return SPENSE_EINVAL;
  std::memset(info, 0, sizeof(*info));
  info->N = h->d.N;
  info->K = h->d.K;
  info->K_s = h->d.K_s;
  info->K_d = h->d.K_d;
  info->wdtype = h->d.wdtype;
  info->gather = h->split ? (h->part[0] ? h->part[0] : h->part[1])->d.gather
                          : (h->d.wdtype == SPENSE_F32 ? 1 : h->d.gather);
  info->weight_bytes = h->weight_bytes;
  info->device_bytes = h->device_bytes;
  info->split = h->split;
  info->N_s = h->split ? h->N_s : h->d.N;
  info->N_d = h->split ? h->N_d : 0;
  if (h->split == 2) {  // GLU block: K_s / K_d of the down projection, N_s / N_d intermediate indices
    info->K_s = h->down->d.K_s;
    info->K_d = h->down->d.K_d;
    info->gather = 0;
  }
  return SPENSE_OK;
}

int spense_export_rows(spense_handle h, void* vals, uint32_t* meta, uint8_t* mask, void* dense, int32_t* rho,
                       void* stream) {
  if (!h || h->split != 1) return SPENSE_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  if (rho) std::memcpy(rho, h->rho_host.data(), (size_t)h->d.N * 4);
  hipError_t e = hipSuccess;
  if (h->part[0]) e = launch_export(h->part[0]->d, vals, meta, mask, nullptr, s);
  if (e == hipSuccess && h->part[1]) e = launch_export(h->part[1]->d, nullptr, nullptr, nullptr, dense, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e == hipSuccess ? SPENSE_OK : hip_fail(e);
}

int spense_export(spense_handle h, void* vals, uint32_t* meta, uint8_t* mask, void* dense, int32_t* pi, void* stream) {
  if (!h || h->split) return SPENSE_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  if (pi) std::memcpy(pi, h->pi_host.data(), (size_t)h->d.K * 4);
  hipError_t e = launch_export(h->d, vals, meta, mask, dense, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e == hipSuccess ? SPENSE_OK : hip_fail(e);
}

int spense_free(spense_handle h) {
  if (!h) return SPENSE_EINVAL;
  release(h);
  return SPENSE_OK;
}

}  // extern "C"
