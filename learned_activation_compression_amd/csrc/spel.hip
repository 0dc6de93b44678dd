// SPEL projector update on fp32 d x r matrices.
//
// Source: "Learned Subspace Compression for Communication-Efficient Pipeline
// Parallelism", Section 3.3, Eq. (4) g_R = g - A sym(A^T g), Eq. (5) heavy-ball
// momentum, Eq. (6) LMO direction Polar(m), Eq. (7) retraction
// A <- Polar(A - alpha d), in the order of Algorithm 1 step 4.  Polar(.) is
// the cubic Newton-Schulz iteration X <- X (1.5 I - 0.5 X^T X), ns_iters
// times; the LMO input is m / ||m||_F (zero when m == 0) and the retraction
// input is not rescaled.
//
// Every product is one of two shapes, both on v_mfma_f32_32x32x2_f32:
//   gram  part[s] = Xl[rows of s]^T Xr[rows of s]   (r x r, split over d rows)
//   xm    out = X M                                  (d x r, K = r)
// The r x r reduction over splits runs in a fixed order (deterministic).
// Scale factors 1/||m||_F are recomputed by each consumer from fixed-order
// partial sums written by the momentum epilogue.
#include "common.h"
#include "internal.h"

namespace mapl {

namespace {

enum { XM_TANGENT = 0, XM_NS = 1, XM_NS_LAST_LMO = 2, XM_NS_LAST_RET = 3 };
enum { RED_SYM = 0, RED_NS = 1 };

__device__ __forceinline__ float inv_norm_from_parts(const float* parts, int n) {
  if (parts == nullptr) return 1.f;
  float s = 0.f;
  for (int i = 0; i < n; ++i) s += parts[i];
  return s > 0.f ? 1.f / sqrtf(s) : 0.f;
}

// part[s][i][j] = sc^2 * sum_{k in split s} Xl[k][i] Xr[k][j]  (sc = 1 unless scale parts are given)
__global__ __launch_bounds__(256) void k_spel_gram(const float* __restrict__ Xl, const float* __restrict__ Xr,
                                                   const float* __restrict__ sparts, int nsp, float* __restrict__ part,
                                                   int d, int r, int rows_per_split) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int h = lane >> 5, l32 = lane & 31;
  const int i0 = blockIdx.x * 64 + (wave >> 1) * 32;
  const int j0 = blockIdx.y * 64 + (wave & 1) * 32;
  if (i0 >= r || j0 >= r) return;
  const int s = blockIdx.z;
  const int kb = s * rows_per_split;
  const int ke = min(d, kb + rows_per_split);
  f32x16 acc = f32x16{};
  const float* pl = Xl + size_t(kb + h) * r + i0 + l32;
  const float* pr = Xr + size_t(kb + h) * r + j0 + l32;
  int k = kb;
  for (; k + 8 <= ke; k += 8) {
    float a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u] = pl[size_t(k - kb + 2 * u) * r];
      b[u] = pr[size_t(k - kb + 2 * u) * r];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc = mfma_f32_32x32x2(a[u], b[u], acc);
  }
  for (; k < ke; k += 2) {
    const bool ok = (k + h) < ke;
    const float a = ok ? pl[size_t(k - kb) * r] : 0.f;
    const float b = ok ? pr[size_t(k - kb) * r] : 0.f;
    acc = mfma_f32_32x32x2(a, b, acc);
  }
  const float sc = inv_norm_from_parts(sparts, nsp);
  const float sc2 = sc * sc;
  float* dst = part + size_t(s) * r * r;
#pragma unroll
  for (int v = 0; v < 16; ++v) dst[size_t(i0 + mfma32_row(v, h)) * r + j0 + l32] = acc[v] * sc2;
}

// mode RED_SYM: M = (G + G^T)/2 ; mode RED_NS: M = 1.5 I - 0.5 G ; G = sum_s part[s]
__global__ __launch_bounds__(256) void k_spel_reduce(const float* __restrict__ part, int S, float* __restrict__ M,
                                                     int r, int mode) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= r * r) return;
  const int i = e / r, j = e % r;
  float gsum = 0.f;
  for (int s = 0; s < S; ++s) gsum += part[size_t(s) * r * r + e];
  if (mode == RED_SYM) {
    float gt = 0.f;
    for (int s = 0; s < S; ++s) gt += part[size_t(s) * r * r + size_t(j) * r + i];
    M[e] = 0.5f * (gsum + gt);
  } else {
    M[e] = (i == j ? 1.5f : 0.f) - 0.5f * gsum;
  }
}

// out[i][j] = sx * sum_k X[i][k] M[k][j] with the epilogue of `mode`.
// Block: 32 rows x 64 columns; wave = (column half jb, k half kh).
__global__ __launch_bounds__(256) void k_spel_xm(const float* __restrict__ X, const float* __restrict__ sparts, int nsp,
                                                 const float* __restrict__ M, float* __restrict__ out, int d, int r,
                                                 int mode, const float* __restrict__ g, float* __restrict__ m,
                                                 float beta, float* __restrict__ norm_parts,
                                                 const float* __restrict__ Acur, float alpha, float* __restrict__ Dout,
                                                 float* __restrict__ Y0) {
  __shared__ float red[2][16][64];
  __shared__ float wsum[4];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int h = lane >> 5, l32 = lane & 31;
  const int jb = wave & 1, kh = wave >> 1;
  const int i0 = blockIdx.x * 32;
  const int j0 = blockIdx.y * 64 + jb * 32;
  const bool active = j0 < r;
  const int half = r >> 1;
  const int kb = kh * half, ke = kb + half;
  f32x16 acc = f32x16{};
  if (active) {
    const float* px = X + size_t(i0 + l32) * r + h;
    const float* pm = M + size_t(h) * r + j0 + l32;
    int k = kb;
    for (; k + 8 <= ke; k += 8) {
      float a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = px[k + 2 * u];
        b[u] = pm[size_t(k + 2 * u) * r];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) acc = mfma_f32_32x32x2(a[u], b[u], acc);
    }
    for (; k < ke; k += 2) {
      const bool ok = (k + h) < ke;
      acc = mfma_f32_32x32x2(ok ? px[k] : 0.f, ok ? pm[size_t(k) * r] : 0.f, acc);
    }
  }
  if (kh == 1 && active) {
#pragma unroll
    for (int v = 0; v < 16; ++v) red[jb][v][lane] = acc[v];
  }
  __syncthreads();
  float local = 0.f;
  if (kh == 0 && active) {
    const float sx = inv_norm_from_parts(sparts, nsp);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = i0 + mfma32_row(v, h), j = j0 + l32;
      const size_t o = size_t(i) * r + j;
      const float val = (acc[v] + red[jb][v][lane]) * sx;
      if (mode == XM_TANGENT) {
        const float gR = g[o] - val;
        const float mn = beta * m[o] + (1.f - beta) * gR;
        m[o] = mn;
        local = fmaf(mn, mn, local);
      } else if (mode == XM_NS || mode == XM_NS_LAST_RET) {
        out[o] = val;
      } else {  // XM_NS_LAST_LMO
        out[o] = val;
        if (Dout) Dout[o] = val;
        Y0[o] = Acur[o] - alpha * val;
      }
    }
  }
  if (mode == XM_TANGENT) {
    // fixed-order block sum: lanes by xor-butterfly, then waves 0 and 1 in order
    for (int off = 32; off > 0; off >>= 1) local += __shfl_xor(local, off);
    if (lane == 0) wsum[wave] = local;
    __syncthreads();
    if (threadIdx.x == 0) norm_parts[blockIdx.y * gridDim.x + blockIdx.x] = wsum[0] + wsum[1];
  }
}

int spel_splits(int d, int r) {
  const int tiles = ((r + 63) / 64) * ((r + 63) / 64);
  int s = (256 + tiles - 1) / tiles;
  const int max_s = d / 64 > 0 ? d / 64 : 1;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  return s;
}

}  // namespace

size_t spel_ws_bytes(int64_t d, int64_t r) {
  const int S = spel_splits(int(d), int(r));
  const int64_t nparts = (d / 32) * ((r + 63) / 64);
  return (size_t(3) * d * r + size_t(S) * r * r + size_t(r) * r + size_t(nparts) + 64) * sizeof(float);
}

void launch_spel(float* A, const float* g, float* m, float alpha, float beta, int ns_iters, float* D_out, int d, int r,
                 void* ws, hipStream_t s) {
  const int S = spel_splits(d, r);
  int rps = (d + S - 1) / S;
  rps = (rps + 1) & ~1;
  float* base = static_cast<float*>(ws);
  float* Xa = base;
  float* Xb = Xa + size_t(d) * r;
  float* Xc = Xb + size_t(d) * r;
  float* parts = Xc + size_t(d) * r;
  float* M = parts + size_t(S) * r * r;
  float* nparts = M + size_t(r) * r;
  const int nsp = (d / 32) * ((r + 63) / 64);

  const dim3 ggrid((r + 63) / 64, (r + 63) / 64, S);
  const dim3 rgrid((r * r + 255) / 256);
  const dim3 xgrid(d / 32, (r + 63) / 64);

  // Eq. (4)-(5): S = A^T g ; m = beta m + (1 - beta)(g - A sym(S))
  hipLaunchKernelGGL(k_spel_gram, ggrid, dim3(256), 0, s, A, g, nullptr, 0, parts, d, r, rps);
  hipLaunchKernelGGL(k_spel_reduce, rgrid, dim3(256), 0, s, parts, S, M, r, int(RED_SYM));
  hipLaunchKernelGGL(k_spel_xm, xgrid, dim3(256), 0, s, A, nullptr, 0, M, nullptr, d, r, int(XM_TANGENT), g, m, beta,
                     nparts, nullptr, 0.f, nullptr, nullptr);

  // Eq. (6): D = NS(m / ||m||_F); the last iteration also forms Y0 = A - alpha D in Xc
  const float* cur = m;
  const float* cur_sc = nparts;
  int cur_nsp = nsp;
  float* bufs[2] = {Xa, Xb};
  for (int it = 0; it < ns_iters; ++it) {
    float* nxt = bufs[it & 1];
    hipLaunchKernelGGL(k_spel_gram, ggrid, dim3(256), 0, s, cur, cur, cur_sc, cur_nsp, parts, d, r, rps);
    hipLaunchKernelGGL(k_spel_reduce, rgrid, dim3(256), 0, s, parts, S, M, r, int(RED_NS));
    const int mode = (it == ns_iters - 1) ? int(XM_NS_LAST_LMO) : int(XM_NS);
    hipLaunchKernelGGL(k_spel_xm, xgrid, dim3(256), 0, s, cur, cur_sc, cur_nsp, M, nxt, d, r, mode, nullptr, nullptr,
                       0.f, nullptr, A, alpha, D_out, Xc);
    cur = nxt;
    cur_sc = nullptr;
    cur_nsp = 0;
  }

  // Eq. (7): A = NS(A - alpha D), input unscaled; the last iteration writes A
  cur = Xc;
  for (int it = 0; it < ns_iters; ++it) {
    float* nxt = (it == ns_iters - 1) ? A : bufs[it & 1];
    hipLaunchKernelGGL(k_spel_gram, ggrid, dim3(256), 0, s, cur, cur, nullptr, 0, parts, d, r, rps);
    hipLaunchKernelGGL(k_spel_reduce, rgrid, dim3(256), 0, s, parts, S, M, r, int(RED_NS));
    const int mode = (it == ns_iters - 1) ? int(XM_NS_LAST_RET) : int(XM_NS);
    hipLaunchKernelGGL(k_spel_xm, xgrid, dim3(256), 0, s, cur, nullptr, 0, M, nxt, d, r, mode, nullptr, nullptr, 0.f,
                       nullptr, nullptr, 0.f, nullptr, nullptr);
    cur = nxt;
  }
}

}  // namespace mapl
