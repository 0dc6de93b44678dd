// C ABI of the MAPL codec library: host-side validation, then launches.
// The operations and their sources are documented in include/mapl.h.
#include <algorithm>
#include <atomic>
#include <cmath>

#include "../../include/mapl.h"
#include "internal.h"

using namespace mapl;

// ------------------------------------------------ dynamic-LDS limit registry --
namespace mapl {
namespace {
constexpr int kMaxLdsKernels = 256;
struct LdsEntry {
  const void* kernel;
  int bytes;
};
// filled during the library's static initialisation (constant-initialised storage, so
// registrations from any translation unit find it ready)
LdsEntry g_lds[kMaxLdsKernels];
int g_lds_count = 0;
bool g_lds_overflow = false;
std::atomic<uint64_t> g_lds_ready{0};  // devices whose limits are raised (bit = device index < 64)

// The scratch of spel_step_static, for callers that cannot allocate: one array per device
// (each GPU the library runs on holds its own copy until the process ends).  Host code never
// uses the array's name as an address: its device address is looked up once per device, with
// that device current, when the device is prepared (g_scratch), and only that address is
// passed to kernels.
constexpr size_t kScratchBytes = MAPL_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
void* g_scratch[64] = {};
}  // namespace

void lds_register(const void* kernel, int bytes) {
  if (g_lds_count < kMaxLdsKernels) g_lds[g_lds_count++] = LdsEntry{kernel, bytes};
  else g_lds_overflow = true;
}

// Device set-up, once per device (devices 0..63; others are set up on every call): the
// dynamic-LDS limits, and the device address of the static scratch array.
hipError_t lds_prepare_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t(1) << dev) : 0;
  if (bit != 0 && (g_lds_ready.load(std::memory_order_acquire) & bit)) return hipSuccess;
  if (g_lds_overflow) return hipErrorInvalidValue;
  for (int i = 0; i < g_lds_count; ++i) {
    e = hipFuncSetAttribute(g_lds[i].kernel, hipFuncAttributeMaxDynamicSharedMemorySize, g_lds[i].bytes);
    if (e != hipSuccess) return e;
  }
  if (bit != 0) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;  // a racing thread stores the same address
    g_lds_ready.fetch_or(bit, std::memory_order_acq_rel);
  }
  return hipSuccess;
}

// The current device's scratch address (after a successful lds_prepare_device), or NULL.
static void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  return g_scratch[dev];
}
}  // namespace mapl

namespace {

constexpr const char* kVersion = "mapl-gfx950 0.1.0";
constexpr int kMaxPolarSteps = 32;

// Launch status: clears any error left by an earlier call and prepares the
// current device (the dynamic-LDS limits) before anything is enqueued; an
// entry point returns MAPL_ERR_HIP without launching when that fails
// (ready() false), and reports the launch error (if any) afterwards.
struct LaunchScope {
  hipError_t prep;
  LaunchScope() {
    (void)hipGetLastError();
    prep = lds_prepare_device();
  }
  bool ready() const { return prep == hipSuccess; }
  int done() const { return hipGetLastError() == hipSuccess ? MAPL_OK : MAPL_ERR_HIP; }
};

inline bool dtype_ok(mapl_dtype dt) { return dt == MAPL_F32 || dt == MAPL_BF16; }

// Shared shape rules of the codec entry points.  ra is the anchor rank
// (0: no anchor); the id range V matters only when an anchor is read.
int check_codec_shape(int64_t B, int64_t T, int64_t d, int64_t r, int64_t ra, int64_t V, mapl_dtype dt, bool needV) {
  if (!dtype_ok(dt)) return MAPL_ERR_DTYPE;
  if (B < 0 || T < 0) return MAPL_ERR_SHAPE;
  if (B > 0 && T > INT32_MAX / B) return MAPL_ERR_SHAPE;
  if (d < 1 || r < 1 || r > d || d > (1 << 20)) return MAPL_ERR_SHAPE;
  if (ra < 0 || ra > d) return MAPL_ERR_SHAPE;
  if (needV && ra > 0 && (V < 1 || V > INT32_MAX)) return MAPL_ERR_SHAPE;
  if (dt == MAPL_BF16) {
    // r a power of two in [32, 512]; d a multiple of 128 (the compression kernel
    // splits d into four 32-column-aligned quarters); an anchor rank other than r
    // streams in 64-wide chunks
    if (d % 128 != 0 || r < 32 || r > 512 || (r & (r - 1)) != 0) return MAPL_ERR_SHAPE;
    if (ra != 0 && ra != r && (ra % 64 != 0 || r % 64 != 0)) return MAPL_ERR_SHAPE;
  } else {
    if (d > 4096) return MAPL_ERR_SHAPE;
  }
  const int64_t N = B * T;
  if (N * d > (int64_t(1) << 40)) return MAPL_ERR_SHAPE;
  return MAPL_OK;
}

// the anchor pointers a map needs: none without an anchor; tids and E, and P
// unless the anchor is the full-rank one (ra == d, P == NULL standing for I)
bool anchor_ptrs_ok(int64_t ra, int64_t d, const void* tids, const void* E, const void* P) {
  return ra == 0 || (tids && E && (P || ra == d));
}

// token splits of a backward Gram with `rows` rows (d for reconstruct_bwd,
// d + ra for compress_bwd); the workspace holds the larger count of either
int bwd_splits(int64_t N, int64_t rows, int64_t r) { return gram_splits_bf16(int(N), int(rows), int(r)); }

int check_pack(void* pk, size_t pk_bytes, int64_t d, int64_t r, int64_t ra, mapl_dtype dt) {
  if (dt != MAPL_BF16) return MAPL_OK;
  if (pk == nullptr) return MAPL_ERR_NULL;
  if (pk_bytes < pack_bytes_bf16(d, r, ra)) return MAPL_ERR_WORKSPACE;
  return MAPL_OK;
}

// bf16: the Gram partials [S][d + ra][r] of compress_bwd (reconstruct_bwd uses
// the first S d r of them) and M [ra][r]; fp32: the residual [N][d]
size_t bwd_ws_bytes(int64_t N, int64_t d, int64_t r, int64_t ra, mapl_dtype dt) {
  if (dt == MAPL_F32) return size_t(N) * d * sizeof(float);
  const int S = std::max(bwd_splits(N, d, r), bwd_splits(N, d + ra, r));
  return (size_t(S) * (d + ra) * r + size_t(ra) * r) * sizeof(float);
}

}  // namespace

extern "C" {

const char* mapl_status_string(int status) {
  switch (status) {
    case MAPL_OK: return "ok";
    case MAPL_ERR_NULL: return "a required pointer is NULL";
    case MAPL_ERR_SHAPE: return "a size is out of range or breaks an alignment rule";
    case MAPL_ERR_DTYPE: return "unsupported dtype";
    case MAPL_ERR_ARG: return "a scalar argument is out of range";
    case MAPL_ERR_WORKSPACE: return "workspace or pack buffer too small";
    case MAPL_ERR_HIP: return "the HIP runtime reported an error (device set-up or launch)";
    case MAPL_ERR_TID: return "a token id is outside [0, V)";
    default: return "unknown status";
  }
}

const char* mapl_version(void) { return kVersion; }

int mapl_init(void) {
  (void)hipGetLastError();
  return lds_prepare_device() == hipSuccess ? MAPL_OK : MAPL_ERR_HIP;
}

size_t mapl_pack_bytes(int64_t d, int64_t r, int64_t ra, mapl_dtype dt) {
  if (dt != MAPL_BF16 || check_codec_shape(1, 1, d, r, ra, 1, dt, false)) return 0;
  return pack_bytes_bf16(d, r, ra);
}

int mapl_pack(const void* P, const void* A, void* pk, size_t pk_bytes, int64_t d, int64_t r, int64_t ra,
              mapl_dtype dt, hipStream_t stream) {
  int st = check_codec_shape(1, 1, d, r, ra, 1, dt, false);
  if (st) return st;
  if (dt == MAPL_F32) return MAPL_OK;
  if (!A || (ra > 0 && !P && ra != d)) return MAPL_ERR_NULL;
  if ((st = check_pack(pk, pk_bytes, d, r, ra, dt))) return st;
  LaunchScope ls;
  if (!ls.ready()) return MAPL_ERR_HIP;
  PackView v = pack_view(pk, d, r, ra);
  launch_pack_all(static_cast<const uint16_t*>(P), static_cast<const uint16_t*>(A), v, int(d), int(r), int(ra),
                  stream);
  return ls.done();
}

// events armed by mapl_time_next_compress_kernel for this thread's next mapl_compress
static thread_local KernelEvents t_compress_events;

int mapl_time_next_compress_kernel(void* start, void* stop) {
  if ((start == nullptr) != (stop == nullptr)) return MAPL_ERR_NULL;
  t_compress_events.start = static_cast<hipEvent_t>(start);
  t_compress_events.stop = static_cast<hipEvent_t>(stop);
  return MAPL_OK;
}

int mapl_compress(const void* X, const int32_t* tids, const void* E_small, const void* P, const void* A, void* Z,
                  int64_t B, int64_t T, int64_t d, int64_t r, int64_t ra, int64_t V, mapl_dtype dt, void* pk,
                  size_t pk_bytes, int pk_ready, hipStream_t stream) {
  const KernelEvents ev = t_compress_events;  // taken by this call whatever its outcome
  t_compress_events = KernelEvents{};
  if (ev.armed() && (dt != MAPL_BF16 || r >= 512 || B * T == 0)) return MAPL_ERR_ARG;
  int st = check_codec_shape(B, T, d, r, ra, V, dt, true);
  if (st) return st;
  if (pk_ready != 0 && pk_ready != 1) return MAPL_ERR_ARG;
  const int N = int(B * T);
  if (N == 0) return MAPL_OK;  // nothing to do; outputs untouched
  if (!X || !A || !Z || !anchor_ptrs_ok(ra, d, tids, E_small, P)) return MAPL_ERR_NULL;
  if ((st = check_pack(pk, pk_bytes, d, r, ra, dt))) return st;
  LaunchScope ls;
  if (!ls.ready()) return MAPL_ERR_HIP;
  if (dt == MAPL_F32) {
    launch_compress_f32(static_cast<const float*>(X), tids, static_cast<const float*>(E_small),
                        static_cast<const float*>(P), static_cast<const float*>(A), static_cast<float*>(Z), N, int(d),
                        int(r), int(ra), int(V), stream);
    return ls.done();
  }
  PackView v = pack_view(pk, d, r, ra);
  if (!pk_ready)
    launch_pack_all(static_cast<const uint16_t*>(P), static_cast<const uint16_t*>(A), v, int(d), int(r), int(ra),
                    stream);
  launch_tok_reduce_bf16(static_cast<const uint16_t*>(X), v.AtF, tids,
                         ra > 0 ? static_cast<const uint16_t*>(E_small) : nullptr, v.QnF, static_cast<uint16_t*>(Z),
                         N, int(d), int(r), int(ra), int(V), stream, ev);
  return ls.done();
}

int mapl_reconstruct(const void* Z, const int32_t* tids, const void* E_small, const void* P, const void* A,
                     void* Xhat, int64_t B, int64_t T, int64_t d, int64_t r, int64_t ra, int64_t V, mapl_dtype dt,
                     void* pk, size_t pk_bytes, int pk_ready, hipStream_t stream) {
  int st = check_codec_shape(B, T, d, r, ra, V, dt, true);
  if (st) return st;
  if (pk_ready != 0 && pk_ready != 1) return MAPL_ERR_ARG;
  const int N = int(B * T);
  if (N == 0) return MAPL_OK;  // nothing to do; outputs untouched
  if (!Z || !A || !Xhat || !anchor_ptrs_ok(ra, d, tids, E_small, P)) return MAPL_ERR_NULL;
  if ((st = check_pack(pk, pk_bytes, d, r, ra, dt))) return st;
  LaunchScope ls;
  if (!ls.ready()) return MAPL_ERR_HIP;
  if (dt == MAPL_F32) {
    launch_reconstruct_f32(static_cast<const float*>(Z), tids, static_cast<const float*>(E_small),
                           static_cast<const float*>(P), static_cast<const float*>(A), static_cast<float*>(Xhat), N,
                           int(d), int(r), int(ra), int(V), stream);
    return ls.done();
  }
  PackView v = pack_view(pk, d, r, ra);
  if (!pk_ready)
    launch_pack_all(static_cast<const uint16_t*>(P), static_cast<const uint16_t*>(A), v, int(d), int(r), int(ra),
                    stream);
  if (ra > 0 && P == nullptr) {  // full-rank anchor: add the rows E[t] in the epilogue
    if (!launch_tok_expand_eadd_bf16(static_cast<const uint16_t*>(Z), v.AF, tids,
                                     static_cast<const uint16_t*>(E_small), static_cast<uint16_t*>(Xhat), N, int(d),
                                     int(r), int(V), stream))
      return MAPL_ERR_SHAPE;  // not reached: ra = d != r needs r % 64 == 0
    return ls.done();
  }
  if (!launch_tok_expand_bf16(static_cast<const uint16_t*>(Z), v.AF, tids,
                              ra > 0 ? static_cast<const uint16_t*>(E_small) : nullptr, v.PtF,
                              static_cast<uint16_t*>(Xhat), N, int(d), int(r), int(ra), int(V), stream))
    return MAPL_ERR_SHAPE;  // not reached: check_codec_shape admits only covered shapes
  return ls.done();
}

size_t mapl_bwd_workspace_bytes(int64_t B, int64_t T, int64_t d, int64_t r, int64_t ra, mapl_dtype dt) {
  if (check_codec_shape(B, T, d, r, ra, 1, dt, false)) return 0;
  return bwd_ws_bytes(B * T, d, r, ra, dt);
}

int mapl_reconstruct_bwd(const void* gXhat, const void* Z, const void* A, void* gZ, float* gA, int accumulate,
                         int64_t B, int64_t T, int64_t d, int64_t r, mapl_dtype dt, void* pk, size_t pk_bytes,
                         int pk_ready, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_codec_shape(B, T, d, r, 0, 1, dt, false);
  if (st) return st;
  if ((accumulate != 0 && accumulate != 1) || (pk_ready != 0 && pk_ready != 1)) return MAPL_ERR_ARG;
  const int64_t N = B * T;
  if (!gA) return MAPL_ERR_NULL;
  if (N == 0) {  // empty batch: gA = 0 (or unchanged when accumulating)
    if (accumulate) return MAPL_OK;
    LaunchScope ls0;
    if (!ls0.ready()) return MAPL_ERR_HIP;
    launch_fill_f32(gA, d * r, 0.f, stream);
    return ls0.done();
  }
  if (!gXhat || !Z || !A || !gZ) return MAPL_ERR_NULL;
  if ((st = check_pack(pk, pk_bytes, d, r, 0, dt))) return st;  // the A^T section, first in every pack
  const size_t need = bwd_ws_bytes(N, d, r, 0, dt);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return ws == nullptr ? MAPL_ERR_NULL : MAPL_ERR_WORKSPACE;
  LaunchScope ls;
  if (!ls.ready()) return MAPL_ERR_HIP;
  if (dt == MAPL_F32) {
    if (N > 0)
      launch_rowmap_f32(static_cast<const float*>(gXhat), static_cast<const float*>(A), static_cast<float*>(gZ),
                        int(N), int(d), int(r), 0, stream);
    launch_outer_f32(static_cast<const float*>(gXhat), static_cast<const float*>(Z), gA, int(N), int(d), int(r),
                     accumulate, stream);
    return ls.done();
  }
  PackView v = pack_view(pk, d, r, 0);
  if (!pk_ready) launch_pack_AtF(static_cast<const uint16_t*>(A), v.AtF, int(d), int(r), stream);
  const int S = bwd_splits(N, d, r);
  float* part = static_cast<float*>(ws);
  if (N > 0) {
    launch_tok_reduce_bf16(static_cast<const uint16_t*>(gXhat), v.AtF, nullptr, nullptr, nullptr,
                           static_cast<uint16_t*>(gZ), int(N), int(d), int(r), 0, 1, stream);
    // gA (+)= gXhat^T Z
    launch_gram_bf16(static_cast<const uint16_t*>(gXhat), d, int(d), nullptr, 1, nullptr, 0,
                     static_cast<const uint16_t*>(Z), int(r), part, int(N), S, stream);
    launch_reduce_partials(part, S, d * r, gA, d * r, accumulate, nullptr, 0, stream);
  }
  return ls.done();
}

int mapl_compress_bwd(const void* gZ, const void* X, const int32_t* tids, const void* E_small, const void* P,
                      const void* A, void* gX, float* gA, int accumulate, int64_t B, int64_t T, int64_t d, int64_t r,
                      int64_t ra, int64_t V, mapl_dtype dt, void* pk, size_t pk_bytes, int pk_ready, void* ws,
                      size_t ws_bytes, hipStream_t stream) {
  int st = check_codec_shape(B, T, d, r, ra, V, dt, true);
  if (st) return st;
  if ((accumulate != 0 && accumulate != 1) || (pk_ready != 0 && pk_ready != 1)) return MAPL_ERR_ARG;
  const int64_t N = B * T;
  if (!gA) return MAPL_ERR_NULL;
  if (N == 0) {  // empty batch: gA = 0 (or unchanged when accumulating)
    if (accumulate) return MAPL_OK;
    LaunchScope ls0;
    if (!ls0.ready()) return MAPL_ERR_HIP;
    launch_fill_f32(gA, d * r, 0.f, stream);
    return ls0.done();
  }
  if (!gZ || !X || !A || !gX || !anchor_ptrs_ok(ra, d, tids, E_small, P)) return MAPL_ERR_NULL;
  if ((st = check_pack(pk, pk_bytes, d, r, ra, dt))) return st;
  const size_t need = bwd_ws_bytes(N, d, r, ra, dt);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return ws == nullptr ? MAPL_ERR_NULL : MAPL_ERR_WORKSPACE;
  LaunchScope ls;
  if (!ls.ready()) return MAPL_ERR_HIP;
  if (dt == MAPL_F32) {
    float* R = static_cast<float*>(ws);
    if (N > 0) {
      launch_rowmap_f32(static_cast<const float*>(gZ), static_cast<const float*>(A), static_cast<float*>(gX), int(N),
                        int(d), int(r), 1, stream);
      launch_residual_f32(static_cast<const float*>(X), tids, static_cast<const float*>(E_small),
                          static_cast<const float*>(P), R, int(N), int(d), int(ra), int(V), stream);
    }
    launch_outer_f32(R, static_cast<const float*>(gZ), gA, int(N), int(d), int(r), accumulate, stream);
    return ls.done();
  }
  const int S = bwd_splits(N, d + ra, r);
  float* part = static_cast<float*>(ws);           // [S][d + ra][r]
  float* M = part + size_t(S) * (d + ra) * r;      // [ra][r]
  const uint16_t* gZ16 = static_cast<const uint16_t*>(gZ);
  PackView v = pack_view(pk, d, r, ra);
  if (!pk_ready)
    launch_pack_all(static_cast<const uint16_t*>(P), static_cast<const uint16_t*>(A), v, int(d), int(r), int(ra),
                    stream);
  // gX = gZ A^T
  launch_tok_expand_bf16(gZ16, v.AF, nullptr, nullptr, nullptr, static_cast<uint16_t*>(gX), int(N), int(d), int(r), 0,
                         1, stream);
  // gA (+)= X^T gZ - P^T (E[t]^T gZ): one Gram over the rows of [X | E[t]], then
  // the split sums (rows < d into gA, rows >= d into M) and gA -= P^T M
  launch_gram_bf16(static_cast<const uint16_t*>(X), d, int(d), tids, int(V),
                   ra > 0 ? static_cast<const uint16_t*>(E_small) : nullptr, int(ra), gZ16, int(r), part, int(N), S,
                   stream);
  launch_reduce_partials(part, S, (d + ra) * r, gA, d * r, accumulate, M, ra * r, stream);
  if (ra > 0) launch_sub_ptm(static_cast<const uint16_t*>(P), M, gA, int(d), int(r), int(ra), stream);
  return ls.done();
}

size_t mapl_anchor_grad_workspace_bytes(int64_t B, int64_t T, int64_t ra, int64_t V) {
  if (B < 0 || T < 0 || ra < 1 || V < 1 || V > (int64_t(1) << 22)) return 0;
  if (B > 0 && T > INT32_MAX / B) return 0;
  return anchor_grad_ws_bytes(B * T, ra, V);
}

int mapl_anchor_grad(const void* Y, const int32_t* tids, const void* P, float* gE, float alpha, int accumulate,
                     int64_t B, int64_t T, int64_t d, int64_t r, int64_t ra, int64_t V, mapl_dtype dt, void* pk,
                     size_t pk_bytes, int pk_ready, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_codec_shape(B, T, d, r, ra, V, dt, true);
  if (st) return st;
  if (ra < 1) return MAPL_ERR_SHAPE;  // no anchor, no table
  if ((accumulate != 0 && accumulate != 1) || (pk_ready != 0 && pk_ready != 1) || !std::isfinite(alpha))
    return MAPL_ERR_ARG;
  const int64_t N = B * T;
  // the owner kernel packs a token index into 24 bits of its queue entries
  if (V > (int64_t(1) << 22) || N >= (int64_t(1) << 24) || N * ra > (int64_t(1) << 38)) return MAPL_ERR_SHAPE;
  if (!gE) return MAPL_ERR_NULL;
  if (N == 0) {  // empty batch: gE = 0 (or unchanged when accumulating)
    if (accumulate) return MAPL_OK;
    LaunchScope ls0;
    if (!ls0.ready()) return MAPL_ERR_HIP;
    launch_fill_f32(gE, V * ra, 0.f, stream);
    return ls0.done();
  }
  if (!Y || !tids || (!P && ra != d)) return MAPL_ERR_NULL;
  if (P != nullptr && (st = check_pack(pk, pk_bytes, d, r, ra, dt))) return st;  // the identity needs no pack
  if (!ws) return MAPL_ERR_NULL;
  if (ws_bytes < anchor_grad_ws_bytes(N, ra, V)) return MAPL_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) & 15) return MAPL_ERR_ARG;
  LaunchScope ls;
  if (!ls.ready()) return MAPL_ERR_HIP;
  const uint16_t* PF = nullptr;
  if (dt == MAPL_BF16 && P != nullptr) {
    PackView v = pack_view(pk, d, r, ra);
    if (!pk_ready) launch_pack_PF(static_cast<const uint16_t*>(P), v.PF, int(d), int(ra), stream);
    PF = v.PF;
  }
  launch_anchor_grad(Y, dt == MAPL_BF16, tids, P, PF, gE, alpha, accumulate, int(N), int(d), int(ra), int(V), ws,
                     stream);
  return ls.done();
}

int mapl_check_tids(const int32_t* tids, int64_t N, int64_t V, int32_t* bad_count, hipStream_t stream) {
  if (!bad_count || (N > 0 && !tids)) return MAPL_ERR_NULL;
  if (N < 0 || N > INT32_MAX || V < 1 || V > INT32_MAX) return MAPL_ERR_SHAPE;
  LaunchScope ls;
  if (!ls.ready()) return MAPL_ERR_HIP;
  launch_check_tids(tids, int(N), int(V), bad_count, stream);
  return ls.done();
}

// ------------------------------------------------------------------ RVQ --
static int check_rvq_shape(int64_t N, int64_t r, int64_t G, int64_t K, int64_t R, int64_t stride) {
  if (N < 0 || N > INT32_MAX || r < 1 || G < 1 || K < 1 || R < 1 || R > 64) return MAPL_ERR_SHAPE;
  if (r % G != 0 || K > 256) return MAPL_ERR_SHAPE;
  if (N * r > (int64_t(1) << 40)) return MAPL_ERR_SHAPE;
  // codebook rows move as 16-byte vectors: every round's book starts 16-byte aligned
  if ((stride != 0 && stride < r * K) || stride % 4 != 0 || stride < 0 || stride > (int64_t(1) << 40))
    return MAPL_ERR_ARG;
  return MAPL_OK;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int rvq_encode(const void* Z, mapl_dtype z_dt, const float* C, int64_t C_round_stride, uint8_t* codes, int64_t N,
               int64_t r, int64_t G, int64_t K, int64_t R, hipStream_t stream) {
  int st = check_rvq_shape(N, r, G, K, R, C_round_stride);
  if (st) return st;
  if (!dtype_ok(z_dt)) return MAPL_ERR_DTYPE;
  if (!Z || !C || !codes) return MAPL_ERR_NULL;
  const int64_t w = r / G;
  if (!(w == 2 || w == 4 || w == 8 || w == 16 || w == 32 || w == 64)) return MAPL_ERR_SHAPE;
  if (!aligned16(Z) || !aligned16(C)) return MAPL_ERR_ARG;
  if (N == 0) return MAPL_OK;
  LaunchScope ls;
  if (!ls.ready()) return MAPL_ERR_HIP;
  launch_rvq_encode(Z, z_dt == MAPL_BF16, C, C_round_stride, codes, int(N), int(r), int(G), int(K), int(R), stream);
  return ls.done();
}

int rvq_decode(const uint8_t* codes, const float* C, int64_t C_round_stride, void* Zq, mapl_dtype out_dt, int64_t N,
               int64_t r, int64_t G, int64_t K, int64_t R, hipStream_t stream) {
  int st = check_rvq_shape(N, r, G, K, R, C_round_stride);
  if (st) return st;
  if (!dtype_ok(out_dt)) return MAPL_ERR_DTYPE;
  if (!codes || !C || !Zq) return MAPL_ERR_NULL;
  if (!aligned16(C)) return MAPL_ERR_ARG;
  if (N == 0) return MAPL_OK;
  LaunchScope ls;
  if (!ls.ready()) return MAPL_ERR_HIP;
  launch_rvq_decode(codes, C, C_round_stride, Zq, out_dt == MAPL_BF16, int(N), int(r), int(G), int(K), int(R),
                    stream);
  return ls.done();
}

int rvq_stream_apply(float* C, const int32_t* idx, const float* vals, int64_t n, int64_t r, int64_t G, int64_t K,
                     int64_t R_c, hipStream_t stream) {
  if (n < 0 || n > INT32_MAX || r < 1 || G < 1 || K < 1 || R_c < 1 || r % G != 0) return MAPL_ERR_SHAPE;
  if (!C || (n > 0 && (!idx || !vals))) return MAPL_ERR_NULL;
  if (n == 0) return MAPL_OK;
  LaunchScope ls;
  if (!ls.ready()) return MAPL_ERR_HIP;
  launch_rvq_stream(C, idx, vals, int(n), int(r / G), R_c * G * K, stream);
  return ls.done();
}

int rvq_stream_decode(float* C, int64_t C_round_stride, int64_t R_c, const int32_t* idx, const float* vals,
                      int64_t n, const uint8_t* codes, void* Zq, mapl_dtype out_dt, int64_t N, int64_t r, int64_t G,
                      int64_t K, int64_t R, hipStream_t stream) {
  int st = check_rvq_shape(N, r, G, K, R, C_round_stride);
  if (st) return st;
  if (n < 0 || n > INT32_MAX || R_c < 1) return MAPL_ERR_SHAPE;
  if (!dtype_ok(out_dt)) return MAPL_ERR_DTYPE;
  if (!C || !codes || !Zq || (n > 0 && (!idx || !vals))) return MAPL_ERR_NULL;
  if (!aligned16(C)) return MAPL_ERR_ARG;
  if (N == 0 && n == 0) return MAPL_OK;
  LaunchScope ls;
  if (!ls.ready()) return MAPL_ERR_HIP;
  launch_rvq_stream_decode(C, C_round_stride, R_c * G * K, idx, vals, int(n), codes, Zq, out_dt == MAPL_BF16, int(N),
                           int(r), int(G), int(K), int(R), stream);
  return ls.done();
}

// ----------------------------------------------------------------- SPEL --
size_t spel_workspace_bytes(int64_t d, int64_t r) {
  if (d < 1 || r < 1 || r > d || r > 1024 || d % 32 || r % 32 || d > (1 << 24)) return 0;
  return spel_ws_bytes(d, r);
}

int spel_step(float* A, const float* g, float* m, float alpha, float beta, int ns_iters, float* D_out,
              int32_t* status, int64_t d, int64_t r, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (d < 1 || r < 1 || r > d || r > 1024 || d % 32 || r % 32 || d > (1 << 24)) return MAPL_ERR_SHAPE;
  if (!A || !g || !m) return MAPL_ERR_NULL;
  if (!(beta >= 0.f && beta < 1.f) || !(alpha >= 0.f && alpha <= 0.7f) || ns_iters < 1 || ns_iters > 64)
    return MAPL_ERR_ARG;
  const size_t need = spel_ws_bytes(d, r);
  if (!ws) return MAPL_ERR_NULL;
  if (ws_bytes < need) return MAPL_ERR_WORKSPACE;
  // the kernels move rows of every operand as 16-byte vectors
  if ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(g) | reinterpret_cast<uintptr_t>(m) |
       reinterpret_cast<uintptr_t>(D_out) | reinterpret_cast<uintptr_t>(ws)) & 15)
    return MAPL_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(status) & 3) return MAPL_ERR_ARG;
  LaunchScope ls;
  if (!ls.ready()) return MAPL_ERR_HIP;
  launch_spel(A, g, m, alpha, beta, ns_iters, D_out, status, int(d), int(r), ws, stream);
  return ls.done();
}

int spel_step_static(float* A, const float* g, float* m, float alpha, float beta, int ns_iters, float* D_out,
                     int32_t* status, int64_t d, int64_t r, hipStream_t stream) {
  if (d < 1 || r < 1 || r > d || r > 1024 || d % 32 || r % 32 || d > (1 << 24)) return MAPL_ERR_SHAPE;
  if (!A || !g || !m) return MAPL_ERR_NULL;
  if (!(beta >= 0.f && beta < 1.f) || !(alpha >= 0.f && alpha <= 0.7f) || ns_iters < 1 || ns_iters > 64)
    return MAPL_ERR_ARG;
  if (spel_ws_bytes(d, r) > kScratchBytes) return MAPL_ERR_WORKSPACE;  // beyond the static scratch
  if ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(g) | reinterpret_cast<uintptr_t>(m) |
       reinterpret_cast<uintptr_t>(D_out)) & 15)
    return MAPL_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(status) & 3) return MAPL_ERR_ARG;
  LaunchScope ls;
  if (!ls.ready()) return MAPL_ERR_HIP;
  void* ws = device_scratch();
  if (ws == nullptr) return MAPL_ERR_HIP;
  launch_spel(A, g, m, alpha, beta, ns_iters, D_out, status, int(d), int(r), ws, stream);
  return ls.done();
}

int spel_polar_express_coefficients(double ell, int steps, double* coef, double* err) {
  if (!coef) return MAPL_ERR_NULL;
  if (!(ell > 0.0 && ell < 1.0) || steps < 1 || steps > kMaxPolarSteps) return MAPL_ERR_ARG;
  return polar_express_schedule(ell, steps, coef, err) == 0 ? MAPL_OK : MAPL_ERR_ARG;
}

int spel_step_polar_express(float* A, const float* g, float* m, float alpha, float beta, int lmo_steps,
                            int ret_steps, float ell, float* D_out, int32_t* status, int64_t d, int64_t r, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  if (d < 1 || r < 1 || r > d || r > 1024 || d % 32 || r % 32 || d > (1 << 24)) return MAPL_ERR_SHAPE;
  if (!A || !g || !m) return MAPL_ERR_NULL;
  if (!(beta >= 0.f && beta < 1.f) || !(alpha >= 0.f && alpha <= 0.7f) || !(ell > 0.f && ell < 1.f) ||
      lmo_steps < 1 || lmo_steps > kMaxPolarSteps || ret_steps < 1 || ret_steps > kMaxPolarSteps)
    return MAPL_ERR_ARG;
  const size_t need = spel_ws_bytes(d, r);
  if (!ws) return MAPL_ERR_NULL;
  if (ws_bytes < need) return MAPL_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(g) | reinterpret_cast<uintptr_t>(m) |
       reinterpret_cast<uintptr_t>(D_out) | reinterpret_cast<uintptr_t>(ws)) & 15)
    return MAPL_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(status) & 3) return MAPL_ERR_ARG;
  // the schedules, on the host, rounded once to fp32 for the kernels
  double cl[3 * kMaxPolarSteps], cr[3 * kMaxPolarSteps];
  if (polar_express_schedule(ell, lmo_steps, cl, nullptr) || polar_express_schedule(ell, ret_steps, cr, nullptr))
    return MAPL_ERR_ARG;
  float fl[3 * kMaxPolarSteps], fr[3 * kMaxPolarSteps];
  for (int i = 0; i < 3 * lmo_steps; ++i) fl[i] = float(cl[i]);
  for (int i = 0; i < 3 * ret_steps; ++i) fr[i] = float(cr[i]);
  LaunchScope ls;
  if (!ls.ready()) return MAPL_ERR_HIP;
  launch_spel_pe(A, g, m, alpha, beta, fl, lmo_steps, fr, ret_steps, D_out, status, int(d), int(r), ws, stream);
  return ls.done();
}

}  // extern "C"
