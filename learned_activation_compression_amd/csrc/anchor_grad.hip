// Gradient of the trainable anchor table E_small.
//
// Source: "Learned Subspace Compression for Communication-Efficient Pipeline
// Parallelism", Section 3.2 and Eq. (3): the anchor E_small[t] P is part of
// both maps (subtracted in Eq. (1), added in Eq. (2)) and E_small is trained,
// so dL/dE[v] collects, over the tokens whose id is v, the token gradient
// pulled back through P:  gE[v] = alpha * sum_{n : t_n = v} Y[n] P^T.
//
// Three steps:
//   project  U[n] = alpha Y[n] P^T (fp32 [N][r]) on the matrix cores, and
//            max |U| (atomic max on the bit pattern of a non-negative float,
//            which is order-free);
//   scatter  table[t_n][j] += round(U[n][j] * 2^e) as 64-bit integers,
//            e chosen from max |U| and N so that no sum can overflow: integer
//            addition is associative, so the sums do not depend on the order
//            in which the atomics land;
//   finish   gE = (accumulate ? gE : 0) + table * 2^-e.
#include "common.h"
#include "internal.h"

namespace mapl {

namespace {

// zero the 64-bit accumulator (n entries) and the max cell
__global__ __launch_bounds__(256) void k_ag_zero(u32x2* __restrict__ table, int64_t n, uint32_t* __restrict__ mx) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) table[i] = u32x2{0u, 0u};
  if (i == 0) *mx = 0u;
}

__device__ __forceinline__ void record_max(float local, uint32_t* mx) {
  for (int off = 32; off > 0; off >>= 1) local = fmaxf(local, __shfl_xor(local, off));
  if ((threadIdx.x & 63) == 0) atomicMax(mx, __float_as_uint(local));
}

// bf16 (d a multiple of 128, r of 32): a block is 32 tokens; wave w computes
// the 32 x 32 tile of U at columns 32 (4 blockIdx.y + w), over the whole
// d-long contraction.  The matrix-core A operand is 16 bytes of a row of P
// (output column j), the B operand 16 bytes of a row of Y (token n); the four
// waves read the same Y rows, so Y leaves HBM once.
__global__ __launch_bounds__(256) void k_ag_project_bf16(const bf16_t* __restrict__ Y, const bf16_t* __restrict__ P,
                                                         float* __restrict__ U, uint32_t* __restrict__ mx,
                                                         float alpha, int N, int d, int r) {
  const int lane = threadIdx.x & 63, w = wave_id();
  const int hi = lane >> 5, l32 = lane & 31;
  const int jb = blockIdx.y * 4 + w;
  if (jb * 32 >= r) return;  // uniform per wave; no block barrier follows
  const int n = blockIdx.x * 32 + l32;
  const bf16_t* yr = Y + size_t(min(n, N - 1)) * d + 8 * hi;
  const bf16_t* pr = P + size_t(jb * 32 + l32) * d + 8 * hi;
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
  float local = 0.f;
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
  record_max(local, mx);
}

// fp32: one thread per element of U
__global__ __launch_bounds__(256) void k_ag_project_f32(const float* __restrict__ Y, const float* __restrict__ P,
                                                        float* __restrict__ U, uint32_t* __restrict__ mx, float alpha,
                                                        int N, int d, int r) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  float local = 0.f;
  if (e < int64_t(N) * r) {
    const int n = int(e / r), j = int(e % r);
    const float* yr = Y + size_t(n) * d;
    const float* pr = P + size_t(j) * d;
    float s = 0.f;
    for (int k = 0; k < d; ++k) s = fmaf(yr[k], pr[k], s);
    const float v = alpha * s;
    U[e] = v;
    local = fabsf(v);
  }
  record_max(local, mx);
}

// power-of-two scale 2^e for the fixed-point sums: with max |U| < 2^ex and at
// most 2^lgN terms per sum, every sum stays below 2^62
__device__ __forceinline__ int fixed_exponent(uint32_t mbits, int N) {
  const float m = __uint_as_float(mbits);
  int ex;
  (void)frexpf(m, &ex);  // m < 2^ex
  const int lgN = (N > 1) ? 32 - __clz(N - 1) : 0;
  return 62 - ex - lgN;
}

__global__ __launch_bounds__(256) void k_ag_scatter(const float* __restrict__ U, const int32_t* __restrict__ tids,
                                                    unsigned long long* __restrict__ table,
                                                    const uint32_t* __restrict__ mx, int N, int r, int V) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= int64_t(N) * r) return;
  const uint32_t mbits = *mx;
  if (mbits == 0u) return;  // every projected value is zero
  const int n = int(e / r), j = int(e % r);
  const int t = tids[n];
  if (t < 0 || t >= V) return;
  // |U| <= max |U| < 2^62 / 2^(e + lgN): the product is exact and the
  // rounded integer fits
  const long long q = static_cast<long long>(rintf(ldexpf(U[e], fixed_exponent(mbits, N))));
  atomicAdd(table + size_t(t) * r + j, static_cast<unsigned long long>(q));
}

__global__ __launch_bounds__(256) void k_ag_finish(const long long* __restrict__ table, const uint32_t* __restrict__ mx,
                                                   float* __restrict__ gE, int64_t n, int N, int accumulate) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const uint32_t mbits = *mx;
  const int ex = (mbits == 0u) ? 0 : fixed_exponent(mbits, N);
  const float v = float(ldexp(double(table[i]), -ex));
  gE[i] = accumulate ? gE[i] + v : v;
}

}  // namespace

size_t anchor_grad_ws_bytes(int64_t N, int64_t r, int64_t V) {
  auto a256 = [](size_t b) { return (b + 255) & ~size_t(255); };
  return a256(size_t(N) * r * 4) + a256(size_t(V) * r * 8) + 256;
}

void launch_anchor_grad(const void* Y, int y_bf16, const int32_t* tids, const void* P, float* gE, float alpha,
                        int accumulate, int N, int d, int r, int V, void* ws, hipStream_t s) {
  auto a256 = [](size_t b) { return (b + 255) & ~size_t(255); };
  char* base = static_cast<char*>(ws);
  float* U = reinterpret_cast<float*>(base);
  unsigned long long* table = reinterpret_cast<unsigned long long*>(base + a256(size_t(N) * r * 4));
  uint32_t* mx = reinterpret_cast<uint32_t*>(base + a256(size_t(N) * r * 4) + a256(size_t(V) * r * 8));
  const int64_t nt = int64_t(V) * r, ne = int64_t(N) * r;
  hipLaunchKernelGGL(k_ag_zero, dim3(unsigned((nt + 255) / 256)), dim3(256), 0, s, reinterpret_cast<u32x2*>(table), nt,
                     mx);
  if (y_bf16) {
    hipLaunchKernelGGL(k_ag_project_bf16, dim3(unsigned((N + 31) / 32), unsigned((r + 127) / 128)), dim3(256), 0, s,
                       static_cast<const bf16_t*>(Y), static_cast<const bf16_t*>(P), U, mx, alpha, N, d, r);
  } else {
    hipLaunchKernelGGL(k_ag_project_f32, dim3(unsigned((ne + 255) / 256)), dim3(256), 0, s,
                       static_cast<const float*>(Y), static_cast<const float*>(P), U, mx, alpha, N, d, r);
  }
  hipLaunchKernelGGL(k_ag_scatter, dim3(unsigned((ne + 255) / 256)), dim3(256), 0, s, U, tids, table, mx, N, r, V);
  hipLaunchKernelGGL(k_ag_finish, dim3(unsigned((nt + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const long long*>(table), mx, gE, nt, N, accumulate);
}

}  // namespace mapl
