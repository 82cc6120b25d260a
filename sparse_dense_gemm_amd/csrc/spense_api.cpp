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
  void* xws = nullptr;  // gathered activations [M][K_p] bf16 (chunked staging of a chosen dense set)
  size_t xws_bytes = 0;
  int32_t* counters = nullptr;
  size_t n_counters = 0;
  int64_t weight_bytes = 0;
  int64_t device_bytes = 0;
};

namespace {

thread_local int g_last_hip = 0;

int hip_fail(hipError_t e) {
  g_last_hip = (int)e;
  return SPENSE_EHIP;
}

bool valid_dtype(int32_t t) { return t == SPENSE_F32 || t == SPENSE_BF16 || t == SPENSE_FP8_E4M3; }

int64_t elem_bytes(int32_t t) { return t == SPENSE_F32 ? 4 : t == SPENSE_BF16 ? 2 : 1; }

void release(spense_layer* h) {
  if (!h) return;
  void* ptrs[] = {h->wpack, h->scales, h->pi, h->pip, h->vals32, h->meta32, h->dense32, h->ws, h->counters, h->xws};
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
    default: return "unknown status";
  }
}

int spense_pack(const void* W, int32_t wdtype, int64_t N, int64_t K, int64_t ldw, const float* scales,
                const int32_t* dense_cols, int64_t n_dense, double dense_fraction, void* stream, spense_handle* out) {
  // ---- validation (host only) ----
  if (!out) return SPENSE_EINVAL;
  *out = nullptr;
  if (!W || !valid_dtype(wdtype)) return SPENSE_EINVAL;
  if (N < 1 || K < 1 || ldw < K) return SPENSE_EINVAL;
  if (N > (int64_t(1) << 31) || K > (int64_t(1) << 31) || N * ldw > (int64_t(1) << 40)) return SPENSE_EINVAL;
  if ((wdtype == SPENSE_FP8_E4M3) != (scales != nullptr)) return SPENSE_EINVAL;
  std::vector<int32_t> pi;
  int64_t K_s = 0, K_d = 0;
  int rc = resolve_dense_set(K, dense_cols, n_dense, dense_fraction, pi, K_s, K_d);
  if (rc != SPENSE_OK) return rc;

  spense_layer* h = new (std::nothrow) spense_layer();
  if (!h) return SPENSE_ENOMEM;
  h->pi_host = std::move(pi);
  hipStream_t s = (hipStream_t)stream;
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

  std::vector<int32_t> pip;
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
    // per-row output scales, padded to whole row tiles; 1.0 for bf16 weights,
    // so the kernels load and apply them unconditionally
    const size_t sbytes = (size_t)(d.NT * kRowTile) * 4;
    if (e == hipSuccess) e = dev_alloc(&h->scales, sbytes);
    if (wdtype == SPENSE_FP8_E4M3) {
      if (e == hipSuccess) e = hipMemsetAsync(h->scales, 0, sbytes, s);
      if (e == hipSuccess) e = hipMemcpyAsync(h->scales, scales, (size_t)N * 4, hipMemcpyDeviceToDevice, s);
    } else {
      const std::vector<float> ones((size_t)(d.NT * kRowTile), 1.0f);
      if (e == hipSuccess) e = hipMemcpyAsync(h->scales, ones.data(), sbytes, hipMemcpyHostToDevice, s);
      if (e == hipSuccess) e = hipStreamSynchronize(s);  // the host buffer is released on return
    }
    d.scales = h->scales;
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
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    (void)hipStreamSynchronize(s);
    release(h);
    return e == hipErrorOutOfMemory ? (g_last_hip = (int)e, SPENSE_ENOMEM) : hip_fail(e);
  }
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
static int64_t decode_lds_bytes(const LayerDesc& d, int64_t M, int64_t S) {
  const int64_t steps = (d.n_sm + S - 1) / S + (d.n_dm + S - 1) / S;
  return M * (steps * kMacro + 8) * 2;
}

// dynamic LDS of the chunked decode kernel: two chunk buffers
static int64_t stream_lds_bytes(int64_t M) { return 2 * M * (kStreamChunk * kMacro + 8) * 2; }

constexpr int64_t kCUs = 256;             // compute units of the target GPU
constexpr int64_t kLdsPerCU = 160 * 1024;  // LDS bytes per CU

static int plan_linear(const spense_layer* h, int64_t M, int32_t splits, LinearPlan& p) {
  const LayerDesc& d = h->d;
  const int64_t steps = std::max<int64_t>(d.n_sm, d.n_dm);
  const int64_t max_splits = std::max<int64_t>(1, std::min<int64_t>(steps, 64));
  if (splits < 0 || splits > max_splits) return SPENSE_EINVAL;
  p = LinearPlan{};
  p.preset = -1;
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
    if (S == 0) {
      S = d.NT >= 1024 ? 1 : std::max<int64_t>(1, (1920 + d.NT - 1) / d.NT);
      S = std::min<int64_t>(S, max_splits);
      if (ch == 0)  // single-shot staging requested: split until it fits
        while (S < max_splits && decode_lds_bytes(d, M, S) > 64 * 1024) ++S;
    }
    p.chunked = (ch == 1 || decode_lds_bytes(d, M, S) > 64 * 1024) ? 1 : 0;
    // chunked staging: two chunk buffers per workgroup bound the residency,
    // so smaller workgroups keep more waves per CU streaming
    if (p.chunked && !overridden) p.waves = 4;
    p.rgroups = (int)((d.NT + p.waves - 1) / p.waves);
    p.splits = (int)S;
    p.lds_bytes = (int)(p.chunked ? stream_lds_bytes(M) : decode_lds_bytes(d, M, S));
    return SPENSE_OK;
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
  // Two m-tiles per wave up to 128 rows (four need more LDS per workgroup
  // than they save there); beyond, four m-tiles and four row tiles per wave
  // (each staged activation fragment feeds four products).  Two row tiles
  // per wave halve the LDS reads per product but give fewer workgroups: used
  // when the row tiles alone still give at least one workgroup per two CUs;
  // otherwise one row tile per wave plus splits.
  const int64_t wg_nr2 = (d.NT + 15) / 16 * ((M + 31) / 32);
  int pre = M <= 32 || wg_nr2 < kCUs / 2 ? 0 : M <= 64 ? 1 : M <= 128 ? 2 : 8;
  if (const char* t = std::getenv("SPENSE_TILE")) {
    const int v = std::atoi(t);
    if (v >= 0 && v < kNumPresets) pre = v;
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
  const int64_t lds = 2 * rows * (p.chunk * kMacro + 8) * 2;
  p.lds_bytes = (int)lds;
  p.rgroups = (int)((d.NT + p.waves * p.nr - 1) / (p.waves * p.nr));
  int64_t S = splits;
  if (S == 0) {
    const int64_t units = (int64_t)p.rgroups * p.mgroups;
    const int64_t resident = kCUs * std::max<int64_t>(1, kLdsPerCU / lds);
    S = units >= kCUs / 2 ? 1 : std::max<int64_t>(1, std::min<int64_t>(resident / units, max_splits));
  }
  p.splits = (int)S;
  const int64_t grid = (int64_t)p.rgroups * p.mgroups * S;
  p.xcd_remap = (p.mgroups > 1 && grid % 8 == 0) ? 1 : 0;
  if (const char* x = std::getenv("SPENSE_XCD")) p.xcd_remap = (std::atoi(x) != 0 && grid % 8 == 0) ? 1 : 0;
  return SPENSE_OK;
}

int spense_linear_splits(spense_handle h, const void* X, int32_t xdtype, int64_t M, int64_t ldx, void* Y,
                         int32_t ydtype, int64_t ldy, int32_t splits, void* stream) {
  if (!h || !X || !Y) return SPENSE_EINVAL;
  const LayerDesc& d = h->d;
  if (M < 1 || M > (int64_t(1) << 24) || ldx < d.K || ldy < d.N) return SPENSE_EINVAL;
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
  a.ydtype = ydtype;
  if (d.wdtype == SPENSE_F32) {
    if (splits > 1) return SPENSE_EINVAL;
    a.splits = 1;
    LinearPlan p{};
    p.mt = p.mgroups = p.rgroups = p.splits = 1;
    hipError_t e = launch_linear(d, a, p, s);
    return e == hipSuccess ? SPENSE_OK : hip_fail(e);
  }
  LinearPlan p{};
  const bool x_aligned = aligned16(X) && (ldx % 8) == 0;
  a.gather = d.gather || !x_aligned;
  int rc = plan_linear(h, M, splits, p);
  if (rc != SPENSE_OK) return rc;
  a.splits = p.splits;
  if (p.chunked && a.gather) {
    // the chunked kernels stage a contiguous X'p: gather it once into the handle's workspace
    const size_t need = (size_t)M * (size_t)d.K_p * 2;
    if (need > h->xws_bytes) {
      hipError_t e = hipStreamSynchronize(s);  // earlier launches may still read the old workspace
      if (e != hipSuccess) return hip_fail(e);
      if (h->xws) (void)hipFree(h->xws);
      h->xws = nullptr;
      h->xws_bytes = 0;
      e = hipMalloc(&h->xws, need);
      if (e != hipSuccess) return e == hipErrorOutOfMemory ? SPENSE_ENOMEM : hip_fail(e);
      h->xws_bytes = need;
    }
    hipError_t e = launch_gather_x(d, X, M, ldx, h->xws, s);
    if (e != hipSuccess) return hip_fail(e);
    a.X = h->xws;
    a.ldx = d.K_p;
    a.gather = 0;
  }
  if (p.splits > 1) {
    const size_t need = (size_t)p.splits * (size_t)M * (size_t)(d.NT * kRowTile) * 4;
    const size_t need_cnt = (size_t)p.rgroups * (size_t)p.mgroups;
    if (need > h->ws_bytes || need_cnt > h->n_counters) {
      hipError_t e = hipStreamSynchronize(s);  // earlier launches may still read the old workspace
      if (e != hipSuccess) return hip_fail(e);
      if (need > h->ws_bytes) {
        if (h->ws) (void)hipFree(h->ws);
        h->ws = nullptr;
        h->ws_bytes = 0;
        e = hipMalloc((void**)&h->ws, need);
        if (e != hipSuccess) return e == hipErrorOutOfMemory ? SPENSE_ENOMEM : hip_fail(e);
        h->ws_bytes = need;
      }
      if (need_cnt > h->n_counters) {
        if (h->counters) (void)hipFree(h->counters);
        h->counters = nullptr;
        h->n_counters = 0;
        e = hipMalloc((void**)&h->counters, need_cnt * 4);
        if (e != hipSuccess) return e == hipErrorOutOfMemory ? SPENSE_ENOMEM : hip_fail(e);
        e = launch_zero_i32(h->counters, (int64_t)need_cnt, s);
        if (e != hipSuccess) return hip_fail(e);
        h->n_counters = need_cnt;
      }
    }
    a.ws = h->ws;
    a.counters = h->counters;
  }
  hipError_t e = launch_linear(d, a, p, s);
  return e == hipSuccess ? SPENSE_OK : hip_fail(e);
}

int spense_linear(spense_handle h, const void* X, int32_t xdtype, int64_t M, int64_t ldx, void* Y, int32_t ydtype,
                  int64_t ldy, void* stream) {
  return spense_linear_splits(h, X, xdtype, M, ldx, Y, ydtype, ldy, 0, stream);
}

int spense_info(spense_handle h, spense_layer_info* info) {
  if (!h || !info) return SPENSE_EINVAL;
  std::memset(info, 0, sizeof(*info));
  info->N = h->d.N;
  info->K = h->d.K;
  info->K_s = h->d.K_s;
  info->K_d = h->d.K_d;
  info->wdtype = h->d.wdtype;
  info->gather = h->d.wdtype == SPENSE_F32 ? 1 : h->d.gather;
  info->weight_bytes = h->weight_bytes;
  info->device_bytes = h->device_bytes;
  return SPENSE_OK;
}

int spense_export(spense_handle h, void* vals, uint32_t* meta, uint8_t* mask, void* dense, int32_t* pi, void* stream) {
  if (!h) return SPENSE_EINVAL;
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
