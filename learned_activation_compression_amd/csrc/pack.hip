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
//   AtF: W = A^T (M = r, K = d)        compression, gZ = gXhat A
//   QnF: W = -(P A)^T (M = r, K = ra) anchor term of compression
//   AF : W = A   (M = d, K = r)        reconstruction, gX = gZ A^T
//   PtF: W = P^T (M = d, K = ra)       anchor term of reconstruction
//   PF : W = P   (M = ra, K = d)       anchor-table gradient, Y P^T
// where ra is the anchor rank (P is [ra][d]; Eq. (3) has ra = r).
// P is also contracted over d in the anchor-table gradient (Eq. (3)).
// The full-rank anchor (ra = d, P = I, passed as no P) needs only QnF = -A^T,
// i.e. AtF negated; its PtF and PF sections stay unused (the maps add or
// gather the anchor rows directly).
#include "common.h"
#include "internal.h"

namespace mapl {

static inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// sections AtF, AF (r d each), PtF (d ra), QnF (r ra), PF (ra d); ra == 0: the first two only
size_t pack_bytes_bf16(int64_t d, int64_t r, int64_t ra) {
  return 2 * align256(size_t(r) * d * 2) + 2 * align256(size_t(ra) * d * 2) + align256(size_t(r) * ra * 2);
}

PackView pack_view(void* pk, int64_t d, int64_t r, int64_t ra) {
  char* p = static_cast<char*>(pk);
  const size_t big = align256(size_t(r) * d * 2), anc = align256(size_t(ra) * d * 2);
  PackView v;
  v.AtF = reinterpret_cast<uint16_t*>(p);
  v.AF = reinterpret_cast<uint16_t*>(p + big);
  v.PtF = reinterpret_cast<uint16_t*>(p + 2 * big);
  v.QnF = reinterpret_cast<uint16_t*>(p + 2 * big + anc);
  v.PF = reinterpret_cast<uint16_t*>(p + 2 * big + anc + align256(size_t(r) * ra * 2));
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

void launch_pack_PtF(const uint16_t* P, uint16_t* PtF, int d, int ra, hipStream_t s) {
  frag_pack(P, /*sm*/ 1, /*sk*/ d, d, ra, PtF, s);  // W(m, k) = P[k][m]
}

void launch_pack_PF(const uint16_t* P, uint16_t* PF, int d, int ra, hipStream_t s) {
  frag_pack(P, /*sm*/ d, /*sk*/ 1, ra, d, PF, s);  // W(m, k) = P[m][k]
}

// Full pack in one launch of 512-thread blocks.  Blocks [0, nq) form QnF,
// one 32 x 32 tile of P A each (nq = (ra/32)(r/32); 0 without a P); the
// others write one 16-byte unit each of the concatenation [AtF | AF | PtF | PF]
// (section boundaries at multiples of 64 units) and, for the identity anchor
// (eye: P = I, no P), the matching unit of QnF = -AtF with each AtF unit.
//
// QnF tile (i, j): fragments of W = -(P A)^T (M = r, K = ra), rounded once to
// bf16.  Its 8 waves split the d-long contraction (the matrix-core A operand
// is 16 bytes of a row of P, the B operand 8 rows of one column of A, read
// directly), and the 8 partial tiles are added in LDS in a fixed order, each
// thread summing two of the tile's elements.  (512-thread blocks: 16 waves put
// the packing units on half as many CUs, 4 waves serialise the tiles' loads;
// 8.2 us at 150M against 10.8 and 9.5.)
constexpr int kQnWaves = 8;

__global__ __launch_bounds__(64 * kQnWaves) void k_pack_all(const bf16_t* __restrict__ A, const bf16_t* __restrict__ P,
                                                           bf16_t* __restrict__ AtF, bf16_t* __restrict__ AF,
                                                           bf16_t* __restrict__ PtF, bf16_t* __restrict__ PF,
                                                           bf16_t* __restrict__ QnF, int d, int r, int ra, int nq,
                                                           int eye) {
  __shared__ float red[kQnWaves * 1024];
  if (int(blockIdx.x) >= nq) {
    // ---- fragment packing: one unit per thread
    const int64_t u0 = int64_t(blockIdx.x - nq) * (64 * kQnWaves) + threadIdx.x;
    const int64_t n1 = int64_t(d / 16) * (r / 32) * 64;   // AtF, and AF, units
    const int64_t n3 = int64_t(ra / 16) * (d / 32) * 64;  // PtF, and PF, units
    const bf16_t* src;
    int64_t sm, sk, u;
    int M;
    bf16_t* dst;
    if (u0 < n1) {
      src = A, sm = 1, sk = r, M = r, dst = AtF, u = u0;  // W(m, k) = A[k][m]
    } else if (u0 < 2 * n1) {
      src = A, sm = r, sk = 1, M = d, dst = AF, u = u0 - n1;  // W(m, k) = A[m][k]
    } else if (u0 < 2 * n1 + n3) {
      src = P, sm = 1, sk = d, M = d, dst = PtF, u = u0 - 2 * n1;  // W(m, k) = P[k][m]
    } else if (u0 < 2 * n1 + 2 * n3) {
      src = P, sm = d, sk = 1, M = ra, dst = PF, u = u0 - 2 * n1 - n3;  // W(m, k) = P[m][k]
    } else {
      return;
    }
    const int MB = M / 32;
    const int l = int(u & 63);
    const int64_t frag = u >> 6;
    const int st = int(frag / MB), mb = int(frag % MB);
    const int m = mb * 32 + (l & 31);
    const int k0 = st * 16 + 8 * (l >> 5);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = src[m * sm + int64_t(k0 + 2 * e) * sk];
      const uint32_t hi = src[m * sm + int64_t(k0 + 2 * e + 1) * sk];
      w[e] = lo | (hi << 16);
    }
    const u32x4 v = u32x4{w[0], w[1], w[2], w[3]};
    reinterpret_cast<u32x4*>(dst)[u] = v;
    if (eye && dst == AtF) reinterpret_cast<u32x4*>(QnF)[u] = v ^ u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    return;
  }
  // ---- QnF tile: rows i0.. of P A (ra / 32 row blocks), column block mbj
  const int lane = threadIdx.x & 63, w = wave_id();
  const int hi = lane >> 5, l32 = lane & 31;
  const int i0 = (int(blockIdx.x) % (ra / 32)) * 32, mbj = int(blockIdx.x) / (ra / 32);
  const int MB = r / 32;
  const int S = d / 16, sb = S * w / kQnWaves, se = S * (w + 1) / kQnWaves;
  const bf16_t* prow = P + size_t(i0 + l32) * d + 8 * hi;
  const bf16_t* acol = A + size_t(8 * hi) * r + mbj * 32 + l32;  // A[16 st + 8 hi + e][mbj 32 + l32] at + (16 st + e) r
  f32x16 acc = f32x16{};
  for (int s0 = sb; s0 < se; s0 += 8) {
    bf16x8 a[8], b[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int st = min(s0 + t, se - 1);
      a[t] = ld_bf16x8(prow + 16 * st);
      u32x4 bw;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = acol[size_t(16 * st + 2 * e) * r];
        const uint32_t hi2 = acol[size_t(16 * st + 2 * e + 1) * r];
        bw[e] = lo | (hi2 << 16);
      }
      b[t] = __builtin_bit_cast(bf16x8, bw);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t)
      if (s0 + t < se) acc = mfma_bf16_32x32x16(a[t], b[t], acc);
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) red[w * 1024 + v * 64 + lane] = acc[v];
  __syncthreads();
  // element e = v 64 + lane of the tile (fragment order): the partials in wave order
  constexpr int EPT = 1024 / (64 * kQnWaves);  // elements per thread
  float sum[EPT];
#pragma unroll
  for (int x = 0; x < EPT; ++x) {
    const int e = threadIdx.x + 64 * kQnWaves * x;
    sum[x] = red[e];
#pragma unroll
    for (int q = 1; q < kQnWaves; ++q) sum[x] += red[q * 1024 + e];
  }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < EPT; ++x) red[threadIdx.x + 64 * kQnWaves * x] = sum[x];
  __syncthreads();
  if (w != 0) return;
  // lane (column j = mbj*32 + l32) holds rows i = i0 + 8 q + 4 hi + t of P A (t < 4),
  // which in W = -(P A)^T are elements 4 hi + t of unit ((i >> 4) MB + mbj) 64 + l32 + 32 (q & 1)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float v[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) v[t] = -red[(4 * q + t) * 64 + lane];
    const size_t unit = (size_t((i0 >> 4) + (q >> 1)) * MB + mbj) * 64 + l32 + 32 * (q & 1);
    *reinterpret_cast<u32x2*>(QnF + unit * 8 + 4 * hi) = u32x2{pack2bf(v[0], v[1]), pack2bf(v[2], v[3])};
  }
}

// Full pack: the four A / P sections and QnF from P and A in one launch
// (ra == 0: no anchor, the A sections only; P == nullptr with ra == d: the
// identity anchor, QnF = -AtF).
void launch_pack_all(const uint16_t* P, const uint16_t* A, PackView v, int d, int r, int ra, hipStream_t s) {
  const bool eye = ra > 0 && P == nullptr;
  const int rp = eye ? 0 : ra;  // P sections to fill
  const int64_t units = 2 * int64_t(d / 16) * (r / 32) * 64 + 2 * int64_t(rp / 16) * (d / 32) * 64;
  const int nq = (ra > 0 && !eye) ? (ra / 32) * (r / 32) : 0;
  const int per = 64 * kQnWaves;
  hipLaunchKernelGGL(k_pack_all, dim3(unsigned(nq + (units + per - 1) / per)), dim3(per), 0, s, A, P, v.AtF, v.AF,
                     v.PtF, v.PF, v.QnF, d, r, rp, nq, int(eye));
}

}  // namespace mapl
