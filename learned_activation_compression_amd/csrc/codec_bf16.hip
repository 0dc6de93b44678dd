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
// One block: 64 tokens x RB*32 output columns.  The contraction (d/16 steps of
// the X A term, then r/16 steps of the anchor term) is split over the 4 waves;
// each wave accumulates the whole 64 x RB*32 tile for its share of k, and the
// four partial tiles are summed through LDS in a fixed order.
//
// Operands stream through a P-stage register ring: the loads of step s+P are
// issued right after step s is consumed, unconditionally (token rows and
// token ids are clamped to valid rows; a token past N only feeds an output
// column that is never stored, an invalid id is zeroed by a select), so the
// compiler can keep P steps of loads in flight.
template <int RB, int P, bool ANCHOR>
__global__ __launch_bounds__(256) void k_tok_reduce(const bf16_t* __restrict__ X, const bf16_t* __restrict__ AtF,
                                                    const int32_t* __restrict__ tids, const bf16_t* __restrict__ E,
                                                    const bf16_t* __restrict__ QnF, bf16_t* __restrict__ Z, int N,
                                                    int d, int r, int V) {
  __shared__ __attribute__((aligned(16))) float redbuf[4 * RB * 64 * 16];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int hi = lane >> 5, l32 = lane & 31;
  const int tok0 = blockIdx.x * 64;
  const int rbase = blockIdx.y * (RB * 32);
  const int Sd = d >> 4;
  const int Se = ANCHOR ? (r >> 4) : 0;
  const int S = Sd + Se;
  const int sb = (S * wave) >> 2, se = (S * (wave + 1)) >> 2;

  f32x16 acc[RB][2];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int n0 = min(tok0 + l32, N - 1), n1 = min(tok0 + 32 + l32, N - 1);
  const bf16_t* x0 = X + size_t(n0) * d + 8 * hi;
  const bf16_t* x1 = X + size_t(n1) * d + 8 * hi;
  // weight fragments of this block's row blocks: unit (s * MB + rbase/32 + i) * 64 + lane
  const int MB = r >> 5;
  const bf16_t* a0 = AtF + (size_t(rbase >> 5) * 64 + lane) * 8;
  // anchor operands (rows of E picked by token id; an invalid id reads row 0 and is zeroed)
  uint32_t m0 = ~0u, m1 = ~0u;  // anchor-operand masks (0 for an invalid id)
  const bf16_t* er0 = x0;
  const bf16_t* er1 = x1;
  const bf16_t* q0 = a0;
  if (ANCHOR) {
    const int t0 = tids[n0], t1 = tids[n1];
    const bool e0 = (t0 >= 0 && t0 < V), e1 = (t1 >= 0 && t1 < V);
    m0 = e0 ? ~0u : 0u;
    m1 = e1 ? ~0u : 0u;
    er0 = E + size_t(e0 ? t0 : 0) * r + 8 * hi;
    er1 = E + size_t(e1 ? t1 : 0) * r + 8 * hi;
    q0 = QnF + (size_t(rbase >> 5) * 64 + lane) * 8;
  }

  bf16x8 ba[P][RB], bb[P][2];
  auto issue = [&](int st, int s) {
    s = s < se ? s : se - 1;  // past the end: reload the last step (never consumed)
    const bool xs = s < Sd;
    const int sl = xs ? s : s - Sd;
    const int k = sl * 16;
    const bf16_t* pb0 = xs ? x0 + k : er0 + k;
    const bf16_t* pb1 = xs ? x1 + k : er1 + k;
    const bf16_t* pa = (xs ? a0 : q0) + size_t(sl) * MB * 512;
    constexpr size_t astr = 512;  // next row block of the same K-step
    bb[st][0] = ld_bf16x8(pb0);
    bb[st][1] = ld_bf16x8(pb1);
#pragma unroll
    for (int i = 0; i < RB; ++i) ba[st][i] = ld_bf16x8(pa + i * astr);
  };

  if (sb < se) {
#pragma unroll
    for (int u = 0; u < P; ++u) issue(u, sb + u);
    for (int s0 = sb; s0 < se; s0 += P) {
#pragma unroll
      for (int u = 0; u < P; ++u) {
        const int s = s0 + u;
        if (s < se) {
          const bool as = s >= Sd;
          const bf16x8 b0 = mask_bf16x8(bb[u][0], as ? m0 : ~0u);
          const bf16x8 b1 = mask_bf16x8(bb[u][1], as ? m1 : ~0u);
#pragma unroll
          for (int i = 0; i < RB; ++i) {
            acc[i][0] = mfma_bf16_32x32x16(ba[u][i], b0, acc[i][0]);
            acc[i][1] = mfma_bf16_32x32x16(ba[u][i], b1, acc[i][1]);
          }
        }
        issue(u, s + P);  // unconditional: keeps the in-flight count fixed
      }
    }
  }

  // ---- fixed-order sum of the four wave tiles, (w0 + w1) + (w2 + w3), in two
  // rounds (token block j = 0, then 1).  Each wave writes its 32 x 32 tiles of
  // the round to LDS as [wave][r-block][lane][4 x 16 bytes], the 16-byte chunk
  // q stored at position q ^ ((lane >> 1) & 3) so that 8 consecutive lanes hit
  // 8 different bank groups; then wave w sums r-block w of the round (RB == 4)
  // or its share of them and stores straight from registers: lane (token
  // l&31) holds 4 consecutive output columns per register group.
  float* red = &redbuf[0];
  const int sw = (lane >> 1) & 3;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      f32x4* dst = reinterpret_cast<f32x4*>(red + ((wave * RB + i) * 64 + lane) * 16);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        dst[q ^ sw] = f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    }
    __syncthreads();
    const int n = tok0 + j * 32 + l32;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      if ((i & 3) != wave) continue;  // r-block i is summed and stored by wave i % 4
      f32x4 sum[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int qs = q ^ sw;
        f32x4 t0 = reinterpret_cast<const f32x4*>(red + ((0 * RB + i) * 64 + lane) * 16)[qs];
        f32x4 t1 = reinterpret_cast<const f32x4*>(red + ((1 * RB + i) * 64 + lane) * 16)[qs];
        f32x4 t2 = reinterpret_cast<const f32x4*>(red + ((2 * RB + i) * 64 + lane) * 16)[qs];
        f32x4 t3 = reinterpret_cast<const f32x4*>(red + ((3 * RB + i) * 64 + lane) * 16)[qs];
        sum[q] = (t0 + t1) + (t2 + t3);
      }
      if (n < N) {
        bf16_t* row = Z + size_t(n) * r + rbase + i * 32 + 4 * hi;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<u32x2*>(row + 8 * q) = u32x2{pack2bf(sum[q][0], sum[q][1]), pack2bf(sum[q][2], sum[q][3])};
      }
    }
    __syncthreads();
  }
}

void launch_tok_reduce_bf16(const uint16_t* in, const uint16_t* AtF, const int32_t* tids, const uint16_t* E,
                            const uint16_t* QnF, uint16_t* out, int N, int d, int r, int V, hipStream_t s) {
  const int nb = r / 32;
  const int RB = (nb % 4 == 0) ? 4 : (nb % 2 == 0) ? 2 : 1;
  dim3 grid((N + 63) / 64, r / (RB * 32));
  // ANCHOR = true is the compress map of Eq. (1); false is the plain product (gZ = gXhat A)
  auto k = (E != nullptr) ? (RB == 4 ? k_tok_reduce<4, 4, true> : RB == 2 ? k_tok_reduce<2, 6, true>
                                                                         : k_tok_reduce<1, 8, true>)
                          : (RB == 4 ? k_tok_reduce<4, 4, false> : RB == 2 ? k_tok_reduce<2, 6, false>
                                                                          : k_tok_reduce<1, 8, false>);
  hipLaunchKernelGGL(k, grid, dim3(256), 0, s, in, AtF, tids, E, QnF, out, N, d, r, V);
}

// ---------------------------------------------------------------- expand --
// out[N][d] = in[N][r] A^T (+ E[t] P).  One block: TB*32 tokens x 256 output
// channels; wave w owns channels [64w, 64w+64) (two 32-row matrix-core blocks)
// and all tokens of the block.
//
// 1. The block's token operand rows [in[n] | E[t_n]] (S K-steps of 16, i.e.
//    2S 16-byte units per row) are loaded once with coalesced 16-byte loads
//    into LDS, unit u of row t at t*UR + (u ^ (t & 7)) so that the matrix-core
//    reads below (32 rows, one unit each) hit distinct bank groups.  All four
//    waves share them.
// 2. Each K-step: the two weight fragments of the wave come from the
//    fragment-ordered AF / PtF pack through a P-stage register ring; the TB
//    token fragments are read from LDS one step ahead.
// 3. The 256-channel output rows go back through the same LDS (8-byte chunk
//    c of row t at chunk position c ^ 2*(t & 7)) and out with 16-byte stores,
//    each row segment written by 32 consecutive lanes.
// Invalid token ids read row 0 of E and their anchor units are zeroed.
// Two blocks fit on a CU (<= 256 registers per lane, 64 KB LDS), so one
// block's loads overlap the other's matrix-core work.
template <int TB, int PER, int P>
__global__ __launch_bounds__(256, 2) void k_tok_expand(const bf16_t* __restrict__ in, const bf16_t* __restrict__ AF,
                                                    const int32_t* __restrict__ tids, const bf16_t* __restrict__ E,
                                                    const bf16_t* __restrict__ PtF, bf16_t* __restrict__ out, int N,
                                                    int d, int r, int V, int nx, int ny, int ur_log2) {
  constexpr int TT = TB * 32;
  extern __shared__ __attribute__((aligned(16))) u32x4 lds[];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int hi = lane >> 5, l32 = lane & 31;
  const int bid = xcd_swizzle(blockIdx.x, nx * ny);
  const int bx = bid % nx, by = bid / nx;
  const int chb = bx * 256;              // first channel of the block
  const int ch0 = chb + wave * 64;       // first channel of this wave
  const int tok0 = by * TT;
  const bool wave_on = ch0 < d;          // d % 64 == 0
  const int UR = 1 << ur_log2;           // 16-byte units per token row
  const int Sz = r >> 4;
  const int S = (E != nullptr) ? 2 * Sz : Sz;
  const int uz = 2 * Sz;                 // units of the `in` part
  const int msk = UR >= 8 ? 7 : UR - 1;

  // ---- 1. stage token rows: every thread first loads the token ids of its
  // PER units (PER = TT * UR / 256, a compile-time constant so that the loops
  // below carry no branches), then issues all of its row loads, then writes
  // them to LDS -- two memory round trips in total.
  int tk[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int t = (threadIdx.x + 256 * k) >> ur_log2;
    tk[k] = (E != nullptr) ? tids[min(tok0 + t, N - 1)] : 0;
  }
  u32x4 v[PER];
  uint32_t mk[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int q = threadIdx.x + 256 * k;
    const int t = q >> ur_log2, u = q & (UR - 1);
    const int n = min(tok0 + t, N - 1);
    const bool zpart = u < uz;
    const bool ok = zpart | (unsigned(tk[k]) < unsigned(V));
    const bf16_t* zsrc = in + size_t(n) * r + u * 8;
    const bf16_t* esrc = E + size_t(ok ? tk[k] : 0) * r + (u - uz) * 8;
    v[k] = *reinterpret_cast<const u32x4*>(zpart ? zsrc : esrc);
    mk[k] = ok ? ~0u : 0u;
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int q = threadIdx.x + 256 * k;
    const int t = q >> ur_log2, u = q & (UR - 1);
    lds[t * UR + (u ^ (t & msk))] = v[k] & u32x4{mk[k], mk[k], mk[k], mk[k]};
  }
  __syncthreads();

  f32x16 acc[2][TB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < TB; ++j) acc[i][j] = f32x16{};

  if (wave_on) {
    const int MBd = d >> 5;
    const bf16_t* af = AF + (size_t(ch0 >> 5) * 64 + lane) * 8;
    const bf16_t* pf = (E != nullptr) ? PtF + (size_t(ch0 >> 5) * 64 + lane) * 8 : af;
    bf16x8 ba[P][2];
    auto issue = [&](int st, int s) {
      s = s < S ? s : S - 1;
      const bool zs = s < Sz;
      const bf16_t* pa = (zs ? af : pf) + size_t(zs ? s : s - Sz) * MBd * 512;
      ba[st][0] = ld_bf16x8(pa);
      ba[st][1] = ld_bf16x8(pa + 512);
    };
    auto ldsb = [&](int s, int j) {
      const int t = j * 32 + l32;
      const int u = 2 * s + hi;
      return __builtin_bit_cast(bf16x8, lds[t * UR + (u ^ (t & msk))]);
    };
#pragma unroll
    for (int u = 0; u < P; ++u) issue(u, u);
    bf16x8 bnext[TB];
#pragma unroll
    for (int j = 0; j < TB; ++j) bnext[j] = ldsb(0, j);
    for (int s0 = 0; s0 < S; s0 += P) {
#pragma unroll
      for (int u = 0; u < P; ++u) {
        const int s = s0 + u;
        if (s < S) {
          bf16x8 b[TB];
#pragma unroll
          for (int j = 0; j < TB; ++j) b[j] = bnext[j];
          const int sn = s + 1 < S ? s + 1 : s;
#pragma unroll
          for (int j = 0; j < TB; ++j) bnext[j] = ldsb(sn, j);
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < TB; ++j) acc[i][j] = mfma_bf16_32x32x16(ba[u][i], b[j], acc[i][j]);
        }
        issue(u, s + P);
      }
    }
  }
  __syncthreads();  // token rows no longer needed: reuse LDS for the output tile

  // ---- 3. output tile [TT][256] bf16 through LDS: 8-byte chunk c of row t at c ^ 2*(t & 7)
  uint32_t* o32 = reinterpret_cast<uint32_t*>(lds);
  if (wave_on) {
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      const int t = j * 32 + l32;
      const int sw = 2 * (t & 7);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = (wave * 64 + i * 32 + 8 * g + 4 * hi) >> 2;  // 8-byte chunk within the row (0..63)
          uint32_t* dst = o32 + t * 128 + (c ^ sw) * 2;
          dst[0] = pack2bf(acc[i][j][4 * g], acc[i][j][4 * g + 1]);
          dst[1] = pack2bf(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
        }
    }
  }
  __syncthreads();
  const int units = min(256, d - chb) >> 3;  // 16-byte units of a row inside d: 32, or 8*k at the edge
#pragma unroll
  for (int pass = 0; pass < TT / 8; ++pass) {
    const int t = pass * 8 + (threadIdx.x >> 5);
    const int c16 = threadIdx.x & 31;  // 16-byte unit = 8-byte chunks 2*c16, 2*c16+1
    const int n = tok0 + t;
    if (n < N && c16 < units) {
      const u32x4 v = lds[t * 32 + (c16 ^ (t & 7))];
      *reinterpret_cast<u32x4*>(out + size_t(n) * d + chb + c16 * 8) = v;
    }
  }
}

void launch_tok_expand_bf16(const uint16_t* in, const uint16_t* AF, const int32_t* tids, const uint16_t* E,
                            const uint16_t* PtF, uint16_t* out, int N, int d, int r, int V, hipStream_t s) {
  const int S = (E != nullptr) ? r / 8 : r / 16;  // K-steps
  const int UR = 2 * S;                            // 16-byte units per token row (a power of two)
  int ur_log2 = 0;
  while ((1 << ur_log2) < UR) ++ur_log2;
  // token tile: the staged rows (TT * UR * 16 B) and the output tile (TT * 512 B) share <= 64 KB
  const int TB = (UR <= 32) ? 4 : (UR <= 64) ? 2 : 1;
  const int TT = TB * 32;
  const size_t lds = size_t(TT) * (UR * 16 > 512 ? UR * 16 : 512);
  const int nx = (d + 255) / 256;
  const int ny = (N + TT - 1) / TT;
  const int per = TT * UR / 256;  // 2, 4, 8 or 16
  constexpr int P = 4;
#define MAPL_EXPAND(TBv, PERv)                                                                                \
  hipLaunchKernelGGL((k_tok_expand<TBv, PERv, P>), dim3(nx * ny), dim3(256), lds, s, in, AF, tids, E, PtF, out, N, \
                     d, r, V, nx, ny, ur_log2)
  if (TB == 4 && per == 16) MAPL_EXPAND(4, 16);
  else if (TB == 4 && per == 8) MAPL_EXPAND(4, 8);
  else if (TB == 4 && per == 4) MAPL_EXPAND(4, 4);
  else if (TB == 4 && per == 2) MAPL_EXPAND(4, 2);
  else if (TB == 2) MAPL_EXPAND(2, 16);
  else MAPL_EXPAND(1, 16);
#undef MAPL_EXPAND
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
  const int lane = threadIdx.x & 63, wave = wave_id();
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
