// Gradient of the trainable anchor table E_small.
//
// Source: "Learned Subspace Compression for Communication-Efficient Pipeline
// Parallelism", Section 3.2 and Eq. (3): the anchor E_small[t] P is part of
// both maps (subtracted in Eq. (1), added in Eq. (2)) and E_small is trained,
// so dL/dE[v] collects, over the tokens whose id is v, the token gradient
// pulled back through P:  gE[v] = alpha * sum_{n : t_n = v} Y[n] P^T.
//
// Two launches:
//   project  U[n] = alpha Y[n] P^T (fp32 [N][r]) on the matrix cores, plus
//            one max |U| per block (no atomics: a chain of atomics on one
//            address serialises);
//   own      each block owns the ids v with v % B == b (B blocks: frequent
//            ids, which tokenizers give small numbers, land in different
//            blocks) and one 64-column slice.  It reads every token id,
//            queues its own tokens in LDS, adds their U rows into an LDS
//            table of 64-bit integers at one power-of-two scale 2^e taken from
//            the global max |U| and N, and writes its gE rows.  Integer
//            addition is associative, so each row is the same bit pattern
//            whatever order the tokens are added in; no row is shared between
//            blocks, so there are no global atomics and no table in HBM.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace mapl {

namespace {

constexpr int kProjMaxGrid = 1024;  // project blocks along the tokens (the rest loop)
constexpr int kOwnThreads = 1024;   // 16 waves per owner block
constexpr int kOwnVR = 128;         // ids per owner block (LDS table rows)
constexpr int kOwnChunk = 8192;     // token ids scanned per round (LDS queue capacity)
constexpr int kOwnBatch = 32;       // queued tokens whose U loads one wave keeps in flight

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// block max of non-negative values (all threads must call)
template <int WAVES>
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int i = 1; i < WAVES; ++i) m = fmaxf(m, red[i]);
  __syncthreads();  // red may be reused
  return m;
}

// bf16 (d a multiple of 128, r of 32): a block takes 32-token tiles; wave w
// computes the 32 x 32 tile of U at columns 32 (4 blockIdx.y + w), over the
// whole d-long contraction.  The matrix-core A operand is 16 bytes of a row of
// P (output column j), the B operand 16 bytes of a row of Y (token n); the
// four waves read the same Y rows.
__global__ __launch_bounds__(256) void k_ag_project_bf16(const bf16_t* __restrict__ Y, const bf16_t* __restrict__ P,
                                                         float* __restrict__ U, float* __restrict__ part, float alpha,
                                                         int N, int d, int r) {
  __shared__ float red[4];
  const int lane = threadIdx.x & 63, w = wave_id();
  const int hi = lane >> 5, l32 = lane & 31;
  const int jb = blockIdx.y * 4 + w;
  const bool active = jb * 32 < r;  // uniform per wave
  const bf16_t* pr = P + size_t(min(jb * 32 + l32, r - 1)) * d + 8 * hi;
  float local = 0.f;
  for (int tile = blockIdx.x; tile * 32 < N; tile += gridDim.x) {
    if (!active) break;
    const int n = tile * 32 + l32;
    const bf16_t* yr = Y + size_t(min(n, N - 1)) * d + 8 * hi;
    f32x16 acc = f32x16{};
    for (int k0 = 0; k0 < d; k0 += 128) {
      bf16x8 a[8], b[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        a[t] = ld_bf16x8(pr + k0 + 16 * t);
        b[t] = ld_bf16x8(yr + k0 + 16 * t);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 8; ++t) acc = mfma_bf16_32x32x16(a[t], b[t], acc);
    }
    // lane (l32, hi), register 4q + e holds U[n][32 jb + 8q + 4hi + e]
    if (n < N) {
      float* ur = U + size_t(n) * r + jb * 32 + 4 * hi;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = alpha * acc[4 * q + e];
          local = fmaxf(local, fabsf(v[e]));
        }
        *reinterpret_cast<f32x4*>(ur + 8 * q) = v;
      }
    }
  }
  const float m = block_max<4>(local, red);
  if (threadIdx.x == 0) part[blockIdx.y * gridDim.x + blockIdx.x] = m;
}

// fp32: one thread per element of U (grid-stride)
__global__ __launch_bounds__(256) void k_ag_project_f32(const float* __restrict__ Y, const float* __restrict__ P,
                                                        float* __restrict__ U, float* __restrict__ part, float alpha,
                                                        int N, int d, int r) {
  __shared__ float red[4];
  float local = 0.f;
  const int64_t ne = int64_t(N) * r;
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < ne; e += int64_t(gridDim.x) * 256) {
    const int n = int(e / r), j = int(e % r);
    const float* yr = Y + size_t(n) * d;
    const float* pr = P + size_t(j) * d;
    float s = 0.f;
    for (int k = 0; k < d; ++k) s = fmaf(yr[k], pr[k], s);
    const float v = alpha * s;
    U[e] = v;
    local = fmaxf(local, fabsf(v));
  }
  const float m = block_max<4>(local, red);
  if (threadIdx.x == 0) part[blockIdx.x] = m;
}

// power-of-two scale 2^e of the fixed-point sums: with max |U| < 2^ex and at
// most 2^lgN terms per sum, every sum stays below 2^62
__device__ __forceinline__ int fixed_exponent(float m, int N) {
  int ex;
  (void)frexpf(m, &ex);  // m < 2^ex (ex = 0 for m = 0)
  const int lgN = (N > 1) ? 32 - __clz(N - 1) : 0;
  return 62 - ex - lgN;
}

// Owner block b (blockIdx.x) of B = gridDim.x holds the ids v = s B + b,
// s < kOwnVR, and columns [64 blockIdx.y, + 64): lane = column.
__global__ __launch_bounds__(kOwnThreads) void k_ag_own(const float* __restrict__ U, const int32_t* __restrict__ tids,
                                                        const float* __restrict__ part, int npart,
                                                        float* __restrict__ gE, int N, int r, int V, int accumulate) {
  __shared__ unsigned long long acc[kOwnVR * 64];
  __shared__ int q_tok[kOwnChunk];
  __shared__ uint16_t q_slot[kOwnChunk];
  __shared__ float red[16];
  __shared__ int q_count;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int B = gridDim.x, b = blockIdx.x;
  const int col = blockIdx.y * 64 + lane;
  const bool colok = col < r;

  // global scale from the per-block maxima of the projection
  float m = 0.f;
  for (int i = threadIdx.x; i < npart; i += kOwnThreads) m = fmaxf(m, part[i]);
  m = block_max<16>(m, red);
  const int ex = fixed_exponent(m, N);

  for (int i = threadIdx.x; i < kOwnVR * 64; i += kOwnThreads) acc[i] = 0ull;
  if (threadIdx.x == 0) q_count = 0;
  __syncthreads();

  for (int base = 0; base < N; base += kOwnChunk) {
    // queue this block's tokens of the chunk (one LDS atomic per wave and step)
    constexpr int PER = kOwnChunk / kOwnThreads;
    int tv[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) tv[k] = tids[min(base + k * kOwnThreads + int(threadIdx.x), N - 1)];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int n = base + k * kOwnThreads + threadIdx.x;
      const int t = tv[k];
      const bool mine = n < N && t >= 0 && t < V && (t % B) == b;
      const uint64_t mask = __ballot(mine);
      if (mask) {  // uniform per wave
        int qbase = 0;
        if (lane == 0) qbase = atomicAdd(&q_count, __popcll(mask));
        qbase = __shfl(qbase, 0);
        if (mine) {
          const int pos = qbase + __popcll(mask & ((1ull << lane) - 1));
          q_tok[pos] = n;
          q_slot[pos] = uint16_t(t / B);
        }
      }
    }
    __syncthreads();
    const int cnt = q_count;
    // add the queued rows: wave w takes entries w, w + 16, ...; kOwnBatch loads in flight
    for (int i0 = w; i0 < cnt; i0 += 16 * kOwnBatch) {
      float x[kOwnBatch];
      int sl[kOwnBatch];
#pragma unroll
      for (int k = 0; k < kOwnBatch; ++k) {
        // loads from clamped, always valid places; the mask is applied when adding
        const int i = min(i0 + 16 * k, cnt - 1);
        sl[k] = (i0 + 16 * k < cnt) ? int(q_slot[i]) : -1;
        x[k] = U[size_t(q_tok[i]) * r + min(col, r - 1)];
      }
#pragma unroll
      for (int k = 0; k < kOwnBatch; ++k)
        if (sl[k] >= 0 && colok) {
          // |x| <= max |U| < 2^(62 - e - lgN): the scaled value is exact and the integer fits
          const long long qv = static_cast<long long>(rintf(ldexpf(x[k], ex)));
          atomicAdd(&acc[sl[k] * 64 + lane], static_cast<unsigned long long>(qv));
        }
    }
    __syncthreads();  // queue consumed
    if (threadIdx.x == 0) q_count = 0;
    __syncthreads();
  }

  // write the owned rows (every one when overwriting; rows with no token add 0)
  if (!colok) return;
  for (int s = w; s < kOwnVR; s += 16) {
    const int64_t v = int64_t(s) * B + b;
    if (v >= V) break;
    const float val = float(ldexp(double(static_cast<long long>(acc[s * 64 + lane])), -ex));
    float* o = gE + size_t(v) * r + col;
    *o = accumulate ? *o + val : val;
  }
}

int proj_blocks(int N, int r, int y_bf16) {
  if (y_bf16) return std::min((N + 31) / 32, kProjMaxGrid) * ((r + 127) / 128);
  return int(std::min<int64_t>((int64_t(N) * r + 255) / 256, kProjMaxGrid));
}

size_t a256(size_t b) { return (b + 255) & ~size_t(255); }

}  // namespace

size_t anchor_grad_ws_bytes(int64_t N, int64_t r, int64_t V) {
  (void)V;
  return a256(size_t(N) * r * 4) + a256(size_t(kProjMaxGrid) * 16 * 4);
}

void launch_anchor_grad(const void* Y, int y_bf16, const int32_t* tids, const void* P, float* gE, float alpha,
                        int accumulate, int N, int d, int r, int V, void* ws, hipStream_t s) {
  char* base = static_cast<char*>(ws);
  float* U = reinterpret_cast<float*>(base);
  float* part = reinterpret_cast<float*>(base + a256(size_t(N) * r * 4));
  const int npart = proj_blocks(N, r, y_bf16);
  if (y_bf16) {
    const int gx = std::min((N + 31) / 32, kProjMaxGrid);
    hipLaunchKernelGGL(k_ag_project_bf16, dim3(unsigned(gx), unsigned((r + 127) / 128)), dim3(256), 0, s,
                       static_cast<const bf16_t*>(Y), static_cast<const bf16_t*>(P), U, part, alpha, N, d, r);
  } else {
    hipLaunchKernelGGL(k_ag_project_f32, dim3(unsigned(npart)), dim3(256), 0, s, static_cast<const float*>(Y),
                       static_cast<const float*>(P), U, part, alpha, N, d, r);
  }
  const int B = (V + kOwnVR - 1) / kOwnVR;
  hipLaunchKernelGGL(k_ag_own, dim3(unsigned(B), unsigned((r + 63) / 64)), dim3(kOwnThreads), 0, s, U, tids, part,
                     npart, gE, N, r, V, accumulate);
}

}  // namespace mapl
