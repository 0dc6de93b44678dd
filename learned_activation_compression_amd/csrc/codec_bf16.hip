// bf16 MAPL codec kernels on the gfx950 matrix cores (fp32 accumulation).
//
// Source of the maps: "Learned Subspace Compression for Communication-
// Efficient Pipeline Parallelism", Section 3.2, Eq. (1) Z = (X - E[t] P) A,
// Eq. (2) Xhat = Z A^T + E'[t] P', Eq. (3) factorised anchor; the backward
// maps are their adjoints (Section 3.1 "Setup", Section 3.2).
//
// Two token-streaming GEMM shapes cover the four maps:
//   reduce  out[N][r] = in[N][d] A  (+ E[t] Qn)    compress, gZ = gXhat A
//   expand  out[N][d] = in[N][r] A^T (+ E[t] P)    reconstruct, gX = gZ A^T
// and a split-token Gram covers the projector gradient:
//   part[s] = sum_{n in split s} L[n]^T R[n]        gA = gXhat^T Z, X^T gZ, E[t]^T gZ
// Every output tile is computed with the token index as the matrix-core N
// dimension so that each lane ends up holding 4 consecutive output channels of
// one token (8-byte stores of bf16).
#include "common.h"
#include "internal.h"

namespace mapl {

// ---------------------------------------------------------------- reduce --
// One block: 64 tokens x RB*32 output columns.  The contraction (d steps of
// the X A term, then r steps of the anchor term) is split over the 4 waves;
// each wave accumulates the whole 64 x RB*32 tile for its share of k, and the
// four partial tiles are summed in LDS in a fixed order.
template <int RB>
__global__ __launch_bounds__(256) void k_tok_reduce(const bf16_t* __restrict__ X, const bf16_t* __restrict__ At,
                                                    const int32_t* __restrict__ tids, const bf16_t* __restrict__ E,
                                                    const bf16_t* __restrict__ Qn, bf16_t* __restrict__ Z, int N,
                                                    int d, int r, int V) {
  __shared__ float red[2][RB][2][16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hi = lane >> 5, l32 = lane & 31;
  const int tok0 = blockIdx.x * 64;
  const int rbase = blockIdx.y * (RB * 32);
  const int Sd = d >> 4;
  const int Se = (E != nullptr) ? (r >> 4) : 0;
  const int S = Sd + Se;
  const int sb = (S * wave) >> 2, se = (S * (wave + 1)) >> 2;

  f32x16 acc[RB][2];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int n0 = tok0 + l32, n1 = tok0 + 32 + l32;
  const bool v0 = n0 < N, v1 = n1 < N;

  // ---- X A part: steps [sb, min(se, Sd))
  {
    const bf16_t* x0 = X + size_t(v0 ? n0 : 0) * d + 8 * hi;
    const bf16_t* x1 = X + size_t(v1 ? n1 : 0) * d + 8 * hi;
    const bf16_t* a0 = At + size_t(rbase + l32) * d + 8 * hi;
    const int s_end = se < Sd ? se : Sd;
    int s = sb;
    if (s < s_end) {
      bf16x8 b0 = v0 ? ld_bf16x8(x0 + s * 16) : zero_bf16x8();
      bf16x8 b1 = v1 ? ld_bf16x8(x1 + s * 16) : zero_bf16x8();
      bf16x8 a[RB];
#pragma unroll
      for (int i = 0; i < RB; ++i) a[i] = ld_bf16x8(a0 + size_t(i) * 32 * d + s * 16);
      for (; s < s_end; ++s) {
        bf16x8 nb0 = b0, nb1 = b1, na[RB];
#pragma unroll
        for (int i = 0; i < RB; ++i) na[i] = a[i];
        if (s + 1 < s_end) {
          const int k = (s + 1) * 16;
          nb0 = v0 ? ld_bf16x8(x0 + k) : zero_bf16x8();
          nb1 = v1 ? ld_bf16x8(x1 + k) : zero_bf16x8();
#pragma unroll
          for (int i = 0; i < RB; ++i) na[i] = ld_bf16x8(a0 + size_t(i) * 32 * d + k);
        }
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          acc[i][0] = mfma_bf16_32x32x16(a[i], b0, acc[i][0]);
          acc[i][1] = mfma_bf16_32x32x16(a[i], b1, acc[i][1]);
        }
        b0 = nb0;
        b1 = nb1;
#pragma unroll
        for (int i = 0; i < RB; ++i) a[i] = na[i];
      }
    }
  }
  // ---- anchor part  - E[t] (P A) = E[t] Qn^T: steps [max(sb, Sd), se)
  if (Se > 0 && se > Sd) {
    const int t0 = v0 ? tids[n0] : -1;
    const int t1 = v1 ? tids[n1] : -1;
    const bool e0 = (t0 >= 0 && t0 < V), e1 = (t1 >= 0 && t1 < V);
    const bf16_t* er0 = E + size_t(e0 ? t0 : 0) * r + 8 * hi;
    const bf16_t* er1 = E + size_t(e1 ? t1 : 0) * r + 8 * hi;
    const bf16_t* q0 = Qn + size_t(rbase + l32) * r + 8 * hi;
    for (int s = (sb > Sd ? sb : Sd); s < se; ++s) {
      const int k = (s - Sd) * 16;
      bf16x8 b0 = e0 ? ld_bf16x8(er0 + k) : zero_bf16x8();
      bf16x8 b1 = e1 ? ld_bf16x8(er1 + k) : zero_bf16x8();
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        bf16x8 a = ld_bf16x8(q0 + size_t(i) * 32 * r + k);
        acc[i][0] = mfma_bf16_32x32x16(a, b0, acc[i][0]);
        acc[i][1] = mfma_bf16_32x32x16(a, b1, acc[i][1]);
      }
    }
  }

  // ---- fixed-order sum of the four wave tiles: (w0 + w2) + (w1 + w3)
  if (wave >= 2) {
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) red[wave - 2][i][j][v][lane] = acc[i][j][v];
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] += red[wave][i][j][v][lane];
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) red[wave][i][j][v][lane] = acc[i][j][v];
  }
  __syncthreads();

  // ---- store: thread -> (token n, RB*8 consecutive output columns)
  const int n = threadIdx.x >> 2, c = threadIdx.x & 3;
  const int gn = tok0 + n;
  if (gn < N) {
    const int cb = n >> 5, ln = n & 31;
    uint32_t w[RB * 4];
#pragma unroll
    for (int e = 0; e < RB * 8; e += 2) {
      float f[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int m = c * RB * 8 + e + u;
        const int rb = m >> 5, mm = m & 31;
        const int v = 4 * (mm >> 3) + (mm & 3), h = (mm >> 2) & 1;
        const int ll = h * 32 + ln;
        f[u] = red[0][rb][cb][v][ll] + red[1][rb][cb][v][ll];
      }
      w[e >> 1] = pack2bf(f[0], f[1]);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(Z + size_t(gn) * r + rbase + c * RB * 8);
#pragma unroll
    for (int q = 0; q < RB; ++q) dst[q] = u32x4{w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]};
  }
}

void launch_tok_reduce_bf16(const uint16_t* in, const uint16_t* At, const int32_t* tids, const uint16_t* E,
                            const uint16_t* Qn, uint16_t* out, int N, int d, int r, int V, hipStream_t s) {
  const int nb = r / 32;
  const int RB = (nb % 4 == 0) ? 4 : (nb % 2 == 0) ? 2 : 1;
  dim3 grid((N + 63) / 64, r / (RB * 32));
  if (RB == 4)
    hipLaunchKernelGGL(k_tok_reduce<4>, grid, dim3(256), 0, s, in, At, tids, E, Qn, out, N, d, r, V);
  else if (RB == 2)
    hipLaunchKernelGGL(k_tok_reduce<2>, grid, dim3(256), 0, s, in, At, tids, E, Qn, out, N, d, r, V);
  else
    hipLaunchKernelGGL(k_tok_reduce<1>, grid, dim3(256), 0, s, in, At, tids, E, Qn, out, N, d, r, V);
}

// ---------------------------------------------------------------- expand --
// One block: TB*32 tokens x 4*CB*32 output channels; wave w owns channels
// [w*CB*32, (w+1)*CB*32) of the block and all its tokens.  K = r (Z A^T)
// followed by r (E[t] P via Pt) accumulate into the same fp32 registers.
template <int CB, int TB>
__global__ __launch_bounds__(256) void k_tok_expand(const bf16_t* __restrict__ in, const bf16_t* __restrict__ A,
                                                    const int32_t* __restrict__ tids, const bf16_t* __restrict__ E,
                                                    const bf16_t* __restrict__ Pt, bf16_t* __restrict__ out, int N,
                                                    int d, int r, int V, int nx, int ny) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hi = lane >> 5, l32 = lane & 31;
  const int bid = xcd_swizzle(blockIdx.x, nx * ny);
  const int bx = bid % nx, by = bid / nx;
  const int ch0 = bx * (4 * CB * 32) + wave * (CB * 32);
  const int tok0 = by * (TB * 32);
  if (ch0 >= d) return;  // whole wave outside d (d % 32 == 0 keeps blocks whole)

  f32x16 acc[CB][TB];
#pragma unroll
  for (int i = 0; i < CB; ++i)
#pragma unroll
    for (int j = 0; j < TB; ++j) acc[i][j] = f32x16{};

  bool cv[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) cv[i] = (ch0 + i * 32) < d;

  int tok[TB];
  bool tv[TB];
#pragma unroll
  for (int j = 0; j < TB; ++j) {
    tok[j] = tok0 + j * 32 + l32;
    tv[j] = tok[j] < N;
  }

  const int Sz = r >> 4;
  // Z A^T
  for (int s = 0; s < Sz; ++s) {
    const int k = s * 16 + 8 * hi;
    bf16x8 a[CB], b[TB];
#pragma unroll
    for (int i = 0; i < CB; ++i) a[i] = cv[i] ? ld_bf16x8(A + size_t(ch0 + i * 32 + l32) * r + k) : zero_bf16x8();
#pragma unroll
    for (int j = 0; j < TB; ++j) b[j] = tv[j] ? ld_bf16x8(in + size_t(tok[j]) * r + k) : zero_bf16x8();
#pragma unroll
    for (int i = 0; i < CB; ++i)
#pragma unroll
      for (int j = 0; j < TB; ++j) acc[i][j] = mfma_bf16_32x32x16(a[i], b[j], acc[i][j]);
  }
  // + E[t] P
  if (E != nullptr) {
    int trow[TB];
    bool ev[TB];
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      const int t = tv[j] ? tids[tok[j]] : -1;
      ev[j] = (t >= 0 && t < V);
      trow[j] = ev[j] ? t : 0;
    }
    for (int s = 0; s < Sz; ++s) {
      const int k = s * 16 + 8 * hi;
      bf16x8 a[CB], b[TB];
#pragma unroll
      for (int i = 0; i < CB; ++i) a[i] = cv[i] ? ld_bf16x8(Pt + size_t(ch0 + i * 32 + l32) * r + k) : zero_bf16x8();
#pragma unroll
      for (int j = 0; j < TB; ++j) b[j] = ev[j] ? ld_bf16x8(E + size_t(trow[j]) * r + k) : zero_bf16x8();
#pragma unroll
      for (int i = 0; i < CB; ++i)
#pragma unroll
        for (int j = 0; j < TB; ++j) acc[i][j] = mfma_bf16_32x32x16(a[i], b[j], acc[i][j]);
    }
  }
  // store 4 consecutive channels (8 bytes) per register group
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    if (!cv[i]) continue;
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      if (!tv[j]) continue;
      bf16_t* row = out + size_t(tok[j]) * d + ch0 + i * 32 + 4 * hi;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w = {pack2bf(acc[i][j][4 * g], acc[i][j][4 * g + 1]), pack2bf(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3])};
        *reinterpret_cast<u32x2*>(row + 8 * g) = w;
      }
    }
  }
}

void launch_tok_expand_bf16(const uint16_t* in, const uint16_t* A, const int32_t* tids, const uint16_t* E,
                            const uint16_t* Pt, uint16_t* out, int N, int d, int r, int V, hipStream_t s) {
  constexpr int CB = 2, TB = 4;
  const int nx = (d + 4 * CB * 32 - 1) / (4 * CB * 32);
  const int ny = (N + TB * 32 - 1) / (TB * 32);
  hipLaunchKernelGGL((k_tok_expand<CB, TB>), dim3(nx * ny), dim3(256), 0, s, in, A, tids, E, Pt, out, N, d, r, V,
                     nx, ny);
}

// ------------------------------------------------------------------ gram --
// part[s][i][j] = sum over tokens n of split s of L[n][i] R[n][j].
// Block: 128 rows i (4 waves x 32) x JB*32 columns j, one token split.
// Token chunks of 64 are staged into LDS transposed ([row][token]) so that
// each lane reads 8 consecutive tokens as one 16-byte operand.
constexpr int kGramChunk = 64;
constexpr int kGramPitch = kGramChunk + 8;

template <int JB>
__global__ __launch_bounds__(256) void k_gram(const bf16_t* __restrict__ L, const int32_t* __restrict__ tids, int V,
                                              const bf16_t* __restrict__ R, float* __restrict__ part, int N, int Ld,
                                              int r, int tok_per_split) {
  __shared__ __attribute__((aligned(16))) bf16_t Ls[128][kGramPitch];
  __shared__ __attribute__((aligned(16))) bf16_t Rs[JB * 32][kGramPitch];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hi = lane >> 5, l32 = lane & 31;
  const int i0 = blockIdx.x * 128, j0 = blockIdx.y * (JB * 32);
  const int sidx = blockIdx.z;
  const int nb = sidx * tok_per_split;
  const int ne = min(N, nb + tok_per_split);

  f32x16 acc[JB];
#pragma unroll
  for (int j = 0; j < JB; ++j) acc[j] = f32x16{};

  for (int c0 = nb; c0 < ne; c0 += kGramChunk) {
    // stage L: 64 tokens x 128 rows, 16 chunks of 8 per token
    for (int q = threadIdx.x; q < kGramChunk * 16; q += 256) {
      const int t = q & (kGramChunk - 1), ic = (q >> 6) * 8;
      const int n = c0 + t;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (n < ne && i0 + ic < Ld) {
        const bf16_t* row = nullptr;
        if (tids != nullptr) {
          const int tk = tids[n];
          if (tk >= 0 && tk < V) row = L + size_t(tk) * Ld;
        } else {
          row = L + size_t(n) * Ld;
        }
        if (row) v = *reinterpret_cast<const u32x4*>(row + i0 + ic);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Ls[ic + 2 * e][t] = bf16_t(v[e] & 0xffffu);
        Ls[ic + 2 * e + 1][t] = bf16_t(v[e] >> 16);
      }
    }
    // stage R: 64 tokens x JB*32 columns
    for (int q = threadIdx.x; q < kGramChunk * JB * 4; q += 256) {
      const int t = q & (kGramChunk - 1), jc = (q >> 6) * 8;
      const int n = c0 + t;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (n < ne) v = *reinterpret_cast<const u32x4*>(R + size_t(n) * r + j0 + jc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Rs[jc + 2 * e][t] = bf16_t(v[e] & 0xffffu);
        Rs[jc + 2 * e + 1][t] = bf16_t(v[e] >> 16);
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kGramChunk / 16; ++ks) {
      const int k = ks * 16 + 8 * hi;
      const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&Ls[wave * 32 + l32][k]));
#pragma unroll
      for (int j = 0; j < JB; ++j) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&Rs[j * 32 + l32][k]));
        acc[j] = mfma_bf16_32x32x16(a, b, acc[j]);
      }
    }
    __syncthreads();
  }
  float* dst = part + size_t(sidx) * Ld * r;
#pragma unroll
  for (int j = 0; j < JB; ++j) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = i0 + wave * 32 + mfma32_row(v, hi);
      if (i < Ld) dst[size_t(i) * r + j0 + j * 32 + l32] = acc[j][v];
    }
  }
}

int gram_splits_bf16(int N) {
  int s = N / 512;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return s;
}

void launch_gram_bf16(const uint16_t* L, const int32_t* tids, int V, const uint16_t* R, float* part, int N, int Ld,
                      int r, int splits, hipStream_t s) {
  int tps = (N + splits - 1) / splits;
  tps = (tps + kGramChunk - 1) / kGramChunk * kGramChunk;
  const int nb = r / 32;
  const int JB = (nb % 4 == 0) ? 4 : (nb % 2 == 0) ? 2 : 1;
  dim3 grid((Ld + 127) / 128, r / (JB * 32), splits);
  if (JB == 4)
    hipLaunchKernelGGL(k_gram<4>, grid, dim3(256), 0, s, L, tids, V, R, part, N, Ld, r, tps);
  else if (JB == 2)
    hipLaunchKernelGGL(k_gram<2>, grid, dim3(256), 0, s, L, tids, V, R, part, N, Ld, r, tps);
  else
    hipLaunchKernelGGL(k_gram<1>, grid, dim3(256), 0, s, L, tids, V, R, part, N, Ld, r, tps);
}

// ------------------------------------------------------ partial reduction --
__global__ __launch_bounds__(256) void k_reduce_partials(const float* __restrict__ part, int splits,
                                                         float* __restrict__ out, int64_t count4, int64_t count,
                                                         int accumulate) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= count4) return;
  f32x4 s = accumulate ? reinterpret_cast<const f32x4*>(out)[e] : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < splits; ++k) s += reinterpret_cast<const f32x4*>(part + size_t(k) * count)[e];
  reinterpret_cast<f32x4*>(out)[e] = s;
}

void launch_reduce_partials(const float* part, int splits, float* out, int64_t count, int accumulate,
                            hipStream_t s) {
  const int64_t c4 = count / 4;
  hipLaunchKernelGGL(k_reduce_partials, dim3(unsigned((c4 + 255) / 256)), dim3(256), 0, s, part, splits, out, c4,
                     count, accumulate);
}

}  // namespace mapl
