// Packed weight layouts for the bf16 codec and a small strided fp32 GEMM.
//
// The matrix cores read each operand as runs of 8 consecutive contraction
// indices per lane.  A [d][r] is contracted over d in compression
// (Eq. (1) of the MAPL paper) and P [r][d] over r in the anchor term
// (Eq. (2)-(3)), so both are stored transposed once per optimizer step:
// At = A^T [r][d] and Pt = P^T [d][r].  Qn = -(P A)^T [r][r] is the anchor
// operand of the re-associated compression X A - E[tids] (P A).
#include "common.h"
#include "internal.h"

namespace mapl {

static inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

size_t pack_bytes_bf16(int64_t d, int64_t r) {
  return align256(size_t(r) * d * 2) + align256(size_t(d) * r * 2) + align256(size_t(r) * r * 2);
}

PackView pack_view(void* pk, int64_t d, int64_t r) {
  char* p = static_cast<char*>(pk);
  PackView v;
  v.At = reinterpret_cast<uint16_t*>(p);
  p += align256(size_t(r) * d * 2);
  v.Pt = reinterpret_cast<uint16_t*>(p);
  p += align256(size_t(d) * r * 2);
  v.Qn = reinterpret_cast<uint16_t*>(p);
  return v;
}

// out[c][rr] = in[rr][c] for a rows x cols bf16 matrix, 64x64 tiles through LDS.
__global__ __launch_bounds__(256) void k_transpose_bf16(const bf16_t* __restrict__ in, bf16_t* __restrict__ out,
                                                        int rows, int cols) {
  __shared__ bf16_t tile[64][66];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    int rr = r0 + i, cc = c0 + tx;
    tile[i][tx] = (rr < rows && cc < cols) ? in[size_t(rr) * cols + cc] : bf16_t(0);
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    int cc = c0 + i, rr = r0 + tx;
    if (cc < cols && rr < rows) out[size_t(cc) * rows + rr] = tile[tx][i];
  }
}

void launch_pack_At(const uint16_t* A, uint16_t* At, int d, int r, hipStream_t s) {
  dim3 grid((r + 63) / 64, (d + 63) / 64);
  hipLaunchKernelGGL(k_transpose_bf16, grid, dim3(256), 0, s, A, At, d, r);
}

void launch_pack_Pt(const uint16_t* P, uint16_t* Pt, int d, int r, hipStream_t s) {
  dim3 grid((d + 63) / 64, (r + 63) / 64);
  hipLaunchKernelGGL(k_transpose_bf16, grid, dim3(256), 0, s, P, Pt, r, d);
}

template <typename T> __device__ __forceinline__ float ldf(const void* p, int64_t idx) {
  return to_f32<T>(static_cast<const T*>(p)[idx]);
}

// C(i,j) = alpha * sum_k A(i,k) B(k,j) + beta * C(i,j); 64x64 tile per block,
// 4x4 outputs per thread, k tiles of 16, fp32 accumulation in k order.
template <typename TA, typename TB, typename TC>
__global__ __launch_bounds__(256) void k_small_gemm(int M, int N, int K, const void* __restrict__ A, int64_t sai,
                                                    int64_t sak, const void* __restrict__ B, int64_t sbk,
                                                    int64_t sbj, TC* __restrict__ C, int64_t sci, int64_t scj,
                                                    float alpha, float beta) {
  __shared__ float As[16][65];
  __shared__ float Bs[16][65];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const bool a_kfast = (sak == 1), b_jfast = (sbj == 1);
  float acc[4][4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int p = 0; p < 4; ++p) acc[q][p] = 0.f;
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int e = threadIdx.x; e < 1024; e += 256) {
      int ii = a_kfast ? (e >> 4) : (e & 63);
      int kk = a_kfast ? (e & 15) : (e >> 6);
      int gi = i0 + ii, gk = k0 + kk;
      As[kk][ii] = (gi < M && gk < K) ? ldf<TA>(A, gi * sai + gk * sak) : 0.f;
      int jj = b_jfast ? (e & 63) : (e >> 4);
      int kb = b_jfast ? (e >> 6) : (e & 15);
      int gj = j0 + jj, gkb = k0 + kb;
      Bs[kb][jj] = (gj < N && gkb < K) ? ldf<TB>(B, gkb * sbk + gj * sbj) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) a[q] = As[kk][ty + 16 * q];
#pragma unroll
      for (int p = 0; p < 4; ++p) b[p] = Bs[kk][tx + 16 * p];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int p = 0; p < 4; ++p) acc[q][p] = fmaf(a[q], b[p], acc[q][p]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      int i = i0 + ty + 16 * q, j = j0 + tx + 16 * p;
      if (i < M && j < N) {
        int64_t o = i * sci + j * scj;
        float v = alpha * acc[q][p];
        if (beta != 0.f) v += beta * to_f32<TC>(C[o]);
        C[o] = from_f32<TC>(v);
      }
    }
}

void launch_small_gemm(int M, int N, int K, const void* A, int a_ty, int64_t sai, int64_t sak, const void* B,
                       int b_ty, int64_t sbk, int64_t sbj, void* C, int c_ty, int64_t sci, int64_t scj, float alpha,
                       float beta, hipStream_t s) {
  dim3 grid((N + 63) / 64, (M + 63) / 64);
#define MAPL_SG(TA, TB, TC)                                                                                   \
  hipLaunchKernelGGL((k_small_gemm<TA, TB, TC>), grid, dim3(256), 0, s, M, N, K, A, sai, sak, B, sbk, sbj, \
                     static_cast<TC*>(C), sci, scj, alpha, beta)
  if (a_ty == 1 && b_ty == 1 && c_ty == 1) MAPL_SG(bf16_t, bf16_t, bf16_t);
  else if (a_ty == 1 && b_ty == 1 && c_ty == 0) MAPL_SG(bf16_t, bf16_t, float);
  else if (a_ty == 1 && b_ty == 0 && c_ty == 0) MAPL_SG(bf16_t, float, float);
  else if (a_ty == 0 && b_ty == 0 && c_ty == 0) MAPL_SG(float, float, float);
  else if (a_ty == 0 && b_ty == 1 && c_ty == 0) MAPL_SG(float, bf16_t, float);
#undef MAPL_SG
}

void launch_pack_Qn(const uint16_t* P, const uint16_t* A, uint16_t* Qn, int d, int r, hipStream_t s) {
  // Qn[j][k] = -sum_i A[i][j] P[k][i]:  M = r (j), N = r (k), K = d (i)
  launch_small_gemm(r, r, d, A, 1, /*sai*/ 1, /*sak*/ r, P, 1, /*sbk*/ 1, /*sbj*/ d, Qn, 1, r, 1, -1.f, 0.f, s);
}

}  // namespace mapl
