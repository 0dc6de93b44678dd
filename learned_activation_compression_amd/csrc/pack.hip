// Packed weight layouts for the bf16 codec.
//
// The matrix cores read each operand as runs of 8 consecutive contraction
// indices per lane.  A [d][r] is contracted over d in compression (Eq. (1) of
// the MAPL paper) and over r in reconstruction (Eq. (2)); P [r][d] is
// contracted over r in the anchor term (Eq. (2)-(3)); Q = P A [r][r] is the
// anchor operand of the re-associated compression X A - E[tids] (P A).
//
// Each is stored once per optimizer step in "fragment order": for an M x K
// operand W (rows = the matrix-core M dimension, K = contraction), fragment
// (s, mb) holds the 64 lanes x 16 bytes that lane l feeds to one
// v_mfma_f32_32x32x16_bf16 at K-step s for row block mb:
//     lane l <- W[mb*32 + (l & 31)][s*16 + 8*(l >> 5) + 0..7]
// at 16-byte unit (s * M/32 + mb) * 64 + l.  A wave's operand load is then one
// contiguous kilobyte, and the row blocks of one K-step are adjacent.
//   AtF: W = A^T (M = r, K = d)      compression, gZ = gXhat A
//   QnF: W = -(P A)^T (M = r, K = r)  anchor term of compression
//   AF : W = A   (M = d, K = r)      reconstruction, gX = gZ A^T
//   PtF: W = P^T (M = d, K = r)      anchor term of reconstruction
#include "common.h"
#include "internal.h"

namespace mapl {

static inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

size_t pack_bytes_bf16(int64_t d, int64_t r) {
  return 3 * align256(size_t(r) * d * 2) + align256(size_t(r) * r * 2);
}

PackView pack_view(void* pk, int64_t d, int64_t r) {
  char* p = static_cast<char*>(pk);
  const size_t big = align256(size_t(r) * d * 2);
  PackView v;
  v.AtF = reinterpret_cast<uint16_t*>(p);
  v.AF = reinterpret_cast<uint16_t*>(p + big);
  v.PtF = reinterpret_cast<uint16_t*>(p + 2 * big);
  v.QnF = reinterpret_cast<uint16_t*>(p + 3 * big);
  return v;
}

// Fragment-order pack of an M x K bf16 operand W(m, k) = src[m*sm + k*sk]
// (see the file comment); one thread per 16-byte unit.
__global__ __launch_bounds__(256) void k_frag_pack(const bf16_t* __restrict__ src, int64_t sm, int64_t sk, int M,
                                                   int K, bf16_t* __restrict__ dst) {
  const int64_t u = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int MB = M / 32;
  if (u >= int64_t(K / 16) * MB * 64) return;
  const int l = int(u & 63);
  const int64_t frag = u >> 6;
  const int s = int(frag / MB), mb = int(frag % MB);
  const int m = mb * 32 + (l & 31);
  const int k0 = s * 16 + 8 * (l >> 5);
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t lo = src[m * sm + int64_t(k0 + 2 * e) * sk];
    const uint32_t hi = src[m * sm + int64_t(k0 + 2 * e + 1) * sk];
    w[e] = lo | (hi << 16);
  }
  reinterpret_cast<u32x4*>(dst)[u] = u32x4{w[0], w[1], w[2], w[3]};
}

static void frag_pack(const uint16_t* src, int64_t sm, int64_t sk, int M, int K, uint16_t* dst, hipStream_t s) {
  const int64_t units = int64_t(K / 16) * (M / 32) * 64;
  hipLaunchKernelGGL(k_frag_pack, dim3(unsigned((units + 255) / 256)), dim3(256), 0, s, src, sm, sk, M, K, dst);
}

void launch_pack_AtF(const uint16_t* A, uint16_t* AtF, int d, int r, hipStream_t s) {
  frag_pack(A, /*sm*/ 1, /*sk*/ r, r, d, AtF, s);  // W(m, k) = A[k][m]
}

void launch_pack_AF(const uint16_t* A, uint16_t* AF, int d, int r, hipStream_t s) {
  frag_pack(A, /*sm*/ r, /*sk*/ 1, d, r, AF, s);  // W(m, k) = A[m][k]
}

void launch_pack_PtF(const uint16_t* P, uint16_t* PtF, int d, int r, hipStream_t s) {
  frag_pack(P, /*sm*/ 1, /*sk*/ d, d, r, PtF, s);  // W(m, k) = P[k][m]
}

// QnF from the split partials of P A: W(j, k) = -(P A)[k][j] = -sum_s part[s][k][j],
// rounded once to bf16, written in fragment order (M = K = r).
__global__ __launch_bounds__(256) void k_qn_finalize(const float* __restrict__ part, int S, bf16_t* __restrict__ QnF,
                                                     int r) {
  const int u = blockIdx.x * 256 + threadIdx.x;
  const int MB = r / 32;
  if (u >= (r / 16) * MB * 64) return;
  const int l = u & 63, frag = u >> 6;
  const int sidx = frag / MB, mb = frag % MB;
  const int j = mb * 32 + (l & 31);
  const int k0 = sidx * 16 + 8 * (l >> 5);
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    float v[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float acc = 0.f;
      for (int s = 0; s < S; ++s) acc += part[size_t(s) * r * r + size_t(k0 + e + q) * r + j];
      v[q] = -acc;
    }
    w[e >> 1] = pack2bf(v[0], v[1]);
  }
  reinterpret_cast<u32x4*>(QnF)[u] = u32x4{w[0], w[1], w[2], w[3]};
}

// Full pack.  P A is formed by the split-row bf16 Gram with L = P^T read in
// place (P is L^T) and R = A, contracting over the d columns of P; its fp32
// partials live in the AtF section, which is written afterwards.
void launch_pack_all(const uint16_t* P, const uint16_t* A, PackView v, int d, int r, hipStream_t s) {
  int S = gram_splits_bf16(d, r, r);
  if (S > d / (2 * r)) S = d / (2 * r);  // partials must fit in the AtF section (2 r d bytes)
  if (S < 1) S = 1;
  float* part = reinterpret_cast<float*>(v.AtF);
  launch_gram_bf16(P, d, /*LT*/ true, r, nullptr, 1, nullptr, 0, A, r, part, d, S, s);
  const int units = (r / 16) * (r / 32) * 64;
  hipLaunchKernelGGL(k_qn_finalize, dim3((units + 255) / 256), dim3(256), 0, s, part, S, v.QnF, r);
  launch_pack_AtF(A, v.AtF, d, r, s);
  launch_pack_AF(A, v.AF, d, r, s);
  launch_pack_PtF(P, v.PtF, d, r, s);
}

}  // namespace mapl
