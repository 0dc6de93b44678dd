// fp32 MAPL codec kernels: plain fp32 arithmetic for small boundaries.
//
// Source of the maps: "Learned Subspace Compression for Communication-
// Efficient Pipeline Parallelism", Section 3.2, Eq. (1)-(3) and their adjoints.
// These kernels take the definitions literally (the residual X - E[t] P is
// formed before the projection) and sum in a fixed order; they serve the fp32
// storage type, where the bf16 matrix cores would not meet fp32 accuracy.
// The anchor has rank ra (E [V][ra], P [ra][d]); ra == 0 is no anchor, and
// P == nullptr with ra == d is the full-rank anchor (P = I: the row E[t] itself).
#include "common.h"
#include "internal.h"

namespace mapl {

constexpr int kTokPerBlock = 4;

__device__ __forceinline__ bool tid_ok(int t, int V) { return t >= 0 && t < V; }

// anchor value at column i of token id t: sum_k E[t][k] P[k][i], or E[t][i] for P = I
__device__ __forceinline__ float anchor_at(const float* __restrict__ E, const float* __restrict__ P, int t, int ra,
                                           int d, int i) {
  if (P == nullptr) return E[size_t(t) * ra + i];
  float a = 0.f;
  for (int k = 0; k < ra; ++k) a = fmaf(E[size_t(t) * ra + k], P[size_t(k) * d + i], a);
  return a;
}

// R[n][i] = X[n][i] - sum_k E[t_n][k] P[k][i]
__global__ __launch_bounds__(256) void k_residual_f32(const float* __restrict__ X, const int32_t* __restrict__ tids,
                                                      const float* __restrict__ E, const float* __restrict__ P,
                                                      float* __restrict__ R, int N, int d, int ra, int V) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= int64_t(N) * d) return;
  const int n = int(e / d), i = int(e % d);
  float a = 0.f;
  if (ra > 0) {
    const int t = tids[n];
    if (tid_ok(t, V)) a = anchor_at(E, P, t, ra, d, i);
  }
  R[e] = X[e] - a;
}

void launch_residual_f32(const float* X, const int32_t* tids, const float* E, const float* P, float* R, int N, int d,
                         int ra, int V, hipStream_t s) {
  const int64_t tot = int64_t(N) * d;
  hipLaunchKernelGGL(k_residual_f32, dim3(unsigned((tot + 255) / 256)), dim3(256), 0, s, X, tids, E, P, R, N, d, ra,
                     V);
}

// Z[n][j] = sum_i (X[n][i] - sum_k E[t_n][k] P[k][i]) A[i][j]; 4 tokens per block.
__global__ __launch_bounds__(256) void k_compress_f32(const float* __restrict__ X, const int32_t* __restrict__ tids,
                                                      const float* __restrict__ E, const float* __restrict__ P,
                                                      const float* __restrict__ A, float* __restrict__ Z, int N, int d,
                                                      int r, int ra, int V) {
  extern __shared__ float Rs[];  // [kTokPerBlock][d]
  const int n0 = blockIdx.x * kTokPerBlock;
  for (int e = threadIdx.x; e < kTokPerBlock * d; e += 256) {
    const int tt = e / d, i = e % d, n = n0 + tt;
    float v = 0.f;
    if (n < N) {
      float a = 0.f;
      if (ra > 0) {
        const int t = tids[n];
        if (tid_ok(t, V)) a = anchor_at(E, P, t, ra, d, i);
      }
      v = X[size_t(n) * d + i] - a;
    }
    Rs[e] = v;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kTokPerBlock * r; e += 256) {
    const int tt = e / r, j = e % r, n = n0 + tt;
    if (n >= N) continue;
    float z = 0.f;
    for (int i = 0; i < d; ++i) z = fmaf(Rs[tt * d + i], A[size_t(i) * r + j], z);
    Z[size_t(n) * r + j] = z;
  }
}

void launch_compress_f32(const float* X, const int32_t* tids, const float* E, const float* P, const float* A,
                         float* Z, int N, int d, int r, int ra, int V, hipStream_t s) {
  const size_t lds = size_t(kTokPerBlock) * d * sizeof(float);
  hipLaunchKernelGGL(k_compress_f32, dim3((N + kTokPerBlock - 1) / kTokPerBlock), dim3(256), lds, s, X, tids, E, P,
                     A, Z, N, d, r, ra, V);
}

// Xh[n][i] = sum_j Z[n][j] A[i][j] + sum_k E[t_n][k] P[k][i]
__global__ __launch_bounds__(256) void k_reconstruct_f32(const float* __restrict__ Z, const int32_t* __restrict__ tids,
                                                         const float* __restrict__ E, const float* __restrict__ P,
                                                         const float* __restrict__ A, float* __restrict__ Xh, int N,
                                                         int d, int r, int ra, int V) {
  extern __shared__ float sh[];  // Zs [4][r], Es [4][ra]
  float* Zs = sh;
  float* Es = sh + kTokPerBlock * r;
  const int n0 = blockIdx.x * kTokPerBlock;
  for (int e = threadIdx.x; e < kTokPerBlock * r; e += 256) {
    const int tt = e / r, k = e % r, n = n0 + tt;
    Zs[e] = n < N ? Z[size_t(n) * r + k] : 0.f;
  }
  for (int e = threadIdx.x; e < kTokPerBlock * ra; e += 256) {
    const int tt = e / ra, k = e % ra, n = n0 + tt;
    float ev = 0.f;
    if (n < N) {
      const int t = tids[n];
      if (tid_ok(t, V)) ev = E[size_t(t) * ra + k];
    }
    Es[e] = ev;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kTokPerBlock * d; e += 256) {
    const int tt = e / d, i = e % d, n = n0 + tt;
    if (n >= N) continue;
    float x = 0.f;
    for (int j = 0; j < r; ++j) x = fmaf(Zs[tt * r + j], A[size_t(i) * r + j], x);
    float a = 0.f;
    if (P == nullptr) {
      if (ra > 0) a = Es[tt * ra + i];  // identity anchor: ra == d
    } else {
      for (int k = 0; k < ra; ++k) a = fmaf(Es[tt * ra + k], P[size_t(k) * d + i], a);
    }
    Xh[size_t(n) * d + i] = x + a;
  }
}

void launch_reconstruct_f32(const float* Z, const int32_t* tids, const float* E, const float* P, const float* A,
                            float* Xh, int N, int d, int r, int ra, int V, hipStream_t s) {
  const size_t lds = size_t(kTokPerBlock) * (r + ra) * sizeof(float);  // <= 128 KB (r, ra <= d <= 4096)
  (void)LdsLimit<k_reconstruct_f32, int(kTokPerBlock * 2 * 4096 * sizeof(float))>::bytes();  // the largest launch
  hipLaunchKernelGGL(k_reconstruct_f32, dim3((N + kTokPerBlock - 1) / kTokPerBlock), dim3(256), lds, s, Z, tids, E,
                     P, A, Xh, N, d, r, ra, V);
}

// transposeA == 0: out[n][j] = sum_i in[n][i] A[i][j]   (in [N][d], out [N][r])
// transposeA == 1: out[n][i] = sum_j in[n][j] A[i][j]   (in [N][r], out [N][d])
__global__ __launch_bounds__(256) void k_rowmap_f32(const float* __restrict__ in, const float* __restrict__ A,
                                                    float* __restrict__ out, int N, int d, int r, int transposeA) {
  extern __shared__ float Is[];
  const int kin = transposeA ? r : d, kout = transposeA ? d : r;
  const int n0 = blockIdx.x * kTokPerBlock;
  for (int e = threadIdx.x; e < kTokPerBlock * kin; e += 256) {
    const int tt = e / kin, n = n0 + tt;
    Is[e] = (n < N) ? in[size_t(n) * kin + e % kin] : 0.f;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kTokPerBlock * kout; e += 256) {
    const int tt = e / kout, o = e % kout, n = n0 + tt;
    if (n >= N) continue;
    float acc = 0.f;
    if (transposeA)
      for (int j = 0; j < r; ++j) acc = fmaf(Is[tt * r + j], A[size_t(o) * r + j], acc);
    else
      for (int i = 0; i < d; ++i) acc = fmaf(Is[tt * d + i], A[size_t(i) * r + o], acc);
    out[size_t(n) * kout + o] = acc;
  }
}

void launch_rowmap_f32(const float* in, const float* A, float* out, int N, int d, int r, int transposeA,
                       hipStream_t s) {
  const size_t lds = size_t(kTokPerBlock) * (transposeA ? r : d) * sizeof(float);
  hipLaunchKernelGGL(k_rowmap_f32, dim3((N + kTokPerBlock - 1) / kTokPerBlock), dim3(256), lds, s, in, A, out, N, d,
                     r, transposeA);
}

// gA[i][j] (+)= sum_n L[n][i] R[n][j], summed over n in order.
__global__ __launch_bounds__(256) void k_outer_f32(const float* __restrict__ L, const float* __restrict__ R,
                                                   float* __restrict__ gA, int N, int d, int r, int accumulate) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= int64_t(d) * r) return;
  const int i = int(e / r), j = int(e % r);
  float acc = 0.f;
  for (int n = 0; n < N; ++n) acc = fmaf(L[size_t(n) * d + i], R[size_t(n) * r + j], acc);
  gA[e] = accumulate ? gA[e] + acc : acc;
}

void launch_outer_f32(const float* L, const float* R, float* gA, int N, int d, int r, int accumulate,
                      hipStream_t s) {
  const int64_t tot = int64_t(d) * r;
  hipLaunchKernelGGL(k_outer_f32, dim3(unsigned((tot + 255) / 256)), dim3(256), 0, s, L, R, gA, N, d, r, accumulate);
}

__global__ __launch_bounds__(256) void k_fill_f32(float* __restrict__ p, int64_t count, float value) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e < count) p[e] = value;
}

void launch_fill_f32(float* p, int64_t count, float value, hipStream_t s) {
  if (count <= 0) return;
  hipLaunchKernelGGL(k_fill_f32, dim3(unsigned((count + 255) / 256)), dim3(256), 0, s, p, count, value);
}

// Count token ids outside [0, V).
__global__ __launch_bounds__(256) void k_check_tids(const int32_t* __restrict__ tids, int N, int V,
                                                    int32_t* __restrict__ bad) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  int b = 0;
  if (n < N) b = (tids[n] < 0 || tids[n] >= V) ? 1 : 0;
  // wave-level sum then one integer atomic per wave
  for (int off = 32; off > 0; off >>= 1) b += __shfl_xor(b, off);
  if ((threadIdx.x & 63) == 0 && b) atomicAdd(bad, b);
}

__global__ void k_zero_i32(int32_t* p) { *p = 0; }

void launch_check_tids(const int32_t* tids, int N, int V, int32_t* bad, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_i32, dim3(1), dim3(1), 0, s, bad);
  if (N > 0) hipLaunchKernelGGL(k_check_tids, dim3((N + 255) / 256), dim3(256), 0, s, tids, N, V, bad);
}

}  // namespace mapl
