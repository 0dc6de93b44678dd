// Residual multi-codebook VQ of the projected boundary activation.
//
// Source: "Learned Subspace Compression for Communication-Efficient Pipeline
// Parallelism", Section 3.5 (Z split into G groups, R rounds, each round
// quantising the previous round's residual against a per-stage codebook) and
// Appendix F (streamed codebook sync: the receiver overwrites the codewords
// the sender streams).
//
// Encode.  For every token, round and group the code is the exact argmin over
// k of ||res - c_k||^2 (lowest k on exact ties; a NaN distance never wins).
// The residual res is kept in fp64: it starts as the stored Z and each round
// subtracts the chosen fp32 codeword, which for inputs of ordinary range is
// exact, so the codes are those of exact arithmetic.  Each kernel first scores
// all K codewords on the matrix cores, a_k ~ s_k = ||c_k||^2 - 2 <res, c_k>
// (s_k orders the codewords as the distance does), with a proven bound
// |a_k - s_k| <= delta.  The exact argmin k* then has
//   a_k* <= s_k* + delta <= s_j + delta <= a_j + 2 delta   for every j,
// so it is among the codewords with a_k <= min_j a_j + 2 delta; those few get
// their exact distance sum_j (res_j - c_kj)^2 in fp64, and the smallest wins.
//
// Layout of both kernels: one block owns one group g and 256 tokens, one
// 32-token tile per wave (8 waves, two per SIMD, so that one wave's vector
// work overlaps the other's matrix-core work).  Lane half h of a wave holds
// dims [h W/2, (h+1) W/2) of token l & 31; in the 32 x 32 score tile of a
// block of 32 codewords, lane l holds that token's scores for the codewords
// 32 b + mfma32_row(v, h), v < 16.  K is padded to Kp = 32 ceil(K / 32) with
// codewords that can never win (norm +inf).
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace mapl {

constexpr int kRvqWaves = 8;  // 32-token tiles per block, one per wave
constexpr int kRvqMaxK = 256;

// The H dims of the token's residual that lane half h holds (columns
// col .. col + H - 1 of row n), widened exactly to fp64; zero past N.
template <int H, typename ZT>
__device__ __forceinline__ void rvq_load_res(const ZT* __restrict__ Z, int n, int N, int r, int col,
                                             double (&res)[H]) {
  const ZT* zr = Z + size_t(min(n, N - 1)) * r + col;
  if (sizeof(ZT) == 2 && H % 8 == 0) {  // bf16: 16-byte loads of 8 values
#pragma unroll
    for (int s = 0; s < H; s += 8) {
      const u32x4 u = *reinterpret_cast<const u32x4*>(zr + s);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        res[s + 2 * e] = double(__uint_as_float(u[e] << 16));
        res[s + 2 * e + 1] = double(__uint_as_float(u[e] & 0xffff0000u));
      }
    }
  } else if (sizeof(ZT) == 4 && H % 4 == 0) {  // fp32: 16-byte loads of 4 values
#pragma unroll
    for (int s = 0; s < H; s += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(zr + s);
#pragma unroll
      for (int e = 0; e < 4; ++e) res[s + e] = double(to_f32<float>(v[e]));
    }
  } else {
#pragma unroll
    for (int s = 0; s < H; ++s) res[s] = double(to_f32<ZT>(zr[s]));
  }
  if (n >= N) {
#pragma unroll
    for (int s = 0; s < H; ++s) res[s] = 0.0;
  }
}

// ||res||^2 of the whole token (both halves), rounded to fp32.
template <int H>
__device__ __forceinline__ float rvq_norm2(const double (&res)[H]) {
  double s2 = 0.0;
#pragma unroll
  for (int s = 0; s < H; ++s) s2 = fma(res[s], res[s], s2);
  const float f = float(s2);
  return f + __shfl_xor(f, 32);
}

// Exact fp64 rescoring of one token's candidates.  mine[] holds this lane's
// candidate bits: bit 16 (b & 1) + v of word b >> 1 marks codeword
// 32 b + mfma32_row(v, h).  The partner lane (same token, other half) holds
// its own bits.  Both lanes walk the union in the same order, each computes
// the squared distance over its H dims (part(k), fp64), and the two halves are
// added (fp addition commutes, so both lanes get the same value).  Exact ties
// keep the lower index; codewords past K (padding) are skipped; NaN never
// wins.  With no candidate (all scores NaN) the code is 0.
// Every pass takes each lane's next two candidates, wherever they sit in the
// eight mask words (picked with selects, no branches), and scores both with
// their loads and arithmetic side by side, so the wave makes
// ceil(c / 2) passes for its busiest token's candidate count c.  The order in
// which candidates are scored does not change the result: the winner is the
// smallest distance, the lowest index among equal ones.
template <typename PartFn>
__device__ __forceinline__ int rvq_rescore(const uint32_t (&mine)[4], int h, int K, PartFn part) {
  uint32_t mm[8];  // words 0-3: candidates of half 0, 4-7: of half 1 (the same in both lanes)
#pragma unroll
  for (int wd = 0; wd < 4; ++wd) {
    const uint32_t o = __shfl_xor(mine[wd], 32);
    mm[wd] = h == 0 ? mine[wd] : o;
    mm[4 + wd] = h == 0 ? o : mine[wd];
  }
  auto left = [&]() {
    uint32_t a = 0u;
#pragma unroll
    for (int q = 0; q < 8; ++q) a |= mm[q];
    return a != 0u;
  };
  // the first set bit in word order, taken out of its word; -1 when none is left
  auto pop = [&]() {
    int qi = 8;
    uint32_t wv = 0u;
#pragma unroll
    for (int q = 7; q >= 0; --q) {
      const bool nz = mm[q] != 0u;
      qi = nz ? q : qi;
      wv = nz ? mm[q] : wv;
    }
    const int bit = __builtin_ctz(wv | 0x80000000u);
    const uint32_t rest = wv & (wv - 1u);
#pragma unroll
    for (int q = 0; q < 8; ++q) mm[q] = (q == qi) ? rest : mm[q];
    return qi < 8 ? 64 * (qi & 3) + 32 * (bit >> 4) + mfma32_row(bit & 15, qi >> 2) : -1;
  };
  double best = __builtin_inf();
  int bk = 0;
  auto offer = [&](int k, double p) {
    const double dk = p + __shfl_xor(p, 32);
    if (k >= 0 && k < K && (dk < best || (dk == best && k < bk))) {
      best = dk;
      bk = k;
    }
  };
  while (__any(left())) {
    // both lanes of a token pop the same candidates, so both take the exchanges in offer()
    const int k1 = pop(), k2 = pop();
    const double p1 = part(k1 < 0 ? 0 : k1), p2 = part(k2 < 0 ? 0 : k2);
    offer(k1, p1);
    offer(k2, p2);
  }
  return bk;
}

// ------------------------------------------------- encode, fp32-scored (w < 16) --
// The round's codebook for g sits in LDS transposed ([dim][codeword], row
// pitch Kp + 2 so that the two lane halves read rows H apart in other banks)
// with its squared norms.  Scores come from v_mfma_f32_32x32x2_f32 on an
// accumulator that starts at ||c_k||^2, with -2 res (rounded to fp32) as the
// other operand.  Bound: nrm_k carries at most W roundings of ||c_k||^2,
// -2 res one rounding of 2 |res|, and the accumulator at most W + 1 roundings
// of sums no larger than ||c_k||^2 + 2 ||res|| ||c_k|| (one per product and
// per addition, whatever the hardware fuses), so with u = 2^-24
//   |a_k - s_k| <= (2 W + 4) u (||c_k||^2 + 2 ||res|| ||c_k||) (1 + small);
// delta is twice that, with max_k ||c_k|| for ||c_k||, plus 1e-30 for
// underflow.  One pass keeps, per lane, the smallest score, its codeword and
// the second smallest (v_med3); after the halves are merged, a token whose
// second score is more than 2 delta above its best has that codeword as its
// exact argmin (every other s_j > s_best).  Only tokens without that margin
// (a few in a thousand) take a second pass that marks every codeword within
// 2 delta and rescores them exactly.
template <int W, typename ZT>
__global__ __launch_bounds__(64 * kRvqWaves) void k_rvq_encode(const ZT* __restrict__ Z, const float* __restrict__ C,
                                                               int64_t stride, uint8_t* __restrict__ codes, int N,
                                                               int r, int G, int K, int R) {
  constexpr int H = W / 2;  // dims per lane (k steps of the 32x32x2 MFMA)
  extern __shared__ __attribute__((aligned(16))) float sh[];
  const int Kp = (K + 31) & ~31;
  const int P = Kp + 2;        // row pitch
  float* cbT = sh;             // [W][P]
  float* nrm = sh + W * P;     // [Kp], +inf past K
  float* bnd = nrm + Kp;       // [1]: max ||c_k||^2 over k < K
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int h = lane >> 5, l32 = lane & 31;
  const int g = blockIdx.x;
  const int n = blockIdx.y * (kRvqWaves * 32) + wave * 32 + l32;
  const float inf = __builtin_inff();

  double res[H];
  rvq_load_res<H, ZT>(Z, n, N, r, g * W + h * H, res);

  for (int rho = 0; rho < R; ++rho) {
    if (rho == 0 || stride != 0) {
      __syncthreads();
      const float* book = C + rho * stride + size_t(g) * K * W;
      if (W % 4 == 0) {
        // 16 bytes (dims j0..j0+3) per thread; the W/4 threads of a codeword are
        // consecutive lanes, whose partial squared norms are added by a butterfly
        for (int e = threadIdx.x; e < Kp * W / 4; e += 64 * kRvqWaves) {
          const int k = e / (W / 4), j0 = 4 * (e % (W / 4));
          const f32x4 v = k < K ? *reinterpret_cast<const f32x4*>(book + size_t(k) * W + j0) : f32x4{0.f, 0.f, 0.f, 0.f};
          float s2 = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            cbT[(j0 + q) * P + k] = v[q];
            s2 = fmaf(v[q], v[q], s2);
          }
#pragma unroll
          for (int off = 1; off < W / 4; off <<= 1) s2 += __shfl_xor(s2, off);
          if (j0 == 0) nrm[k] = k < K ? s2 : inf;
        }
      } else {  // W == 2: one thread per codeword
        for (int k = threadIdx.x; k < Kp; k += 64 * kRvqWaves) {
          const float c0 = k < K ? book[2 * k] : 0.f, c1 = k < K ? book[2 * k + 1] : 0.f;
          cbT[k] = c0;
          cbT[P + k] = c1;
          nrm[k] = k < K ? fmaf(c1, c1, c0 * c0) : inf;
        }
      }
      __syncthreads();
      if (wave == 0) {  // max ||c_k||^2 over the real codewords (a max: order does not matter; NaN drops out)
        float mx = 0.f;
        for (int k = lane; k < K; k += 64) mx = fmaxf(mx, nrm[k]);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        if (lane == 0) bnd[0] = mx;
      }
      __syncthreads();
    }
    float b[H];
#pragma unroll
    for (int s = 0; s < H; ++s) b[s] = float(-2.0 * res[s]);
    const float rn2 = rvq_norm2<H>(res);
    const float nmax = bnd[0];
    const float delta = float(2 * W + 4) * 0x1p-23f * fmaf(2.f * sqrtf(rn2), sqrtf(nmax), nmax) + 1e-30f;

    // accumulator row 8 q + 4 h + e (e < 4) starts at that codeword's squared norm
    auto init = [&](int kb) {
      f32x16 acc;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 nv = *reinterpret_cast<const f32x4*>(nrm + kb + 8 * q + 4 * h);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[4 * q + e] = nv[e];
      }
      return acc;
    };
    auto score = [&](int kb) {
      f32x16 acc = init(kb);
#pragma unroll
      for (int s = 0; s < H; ++s) acc = mfma_f32_32x32x2(cbT[(h * H + s) * P + kb + l32], b[s], acc);
      return acc;
    };
    float best = inf, second = inf;
    int bk = 0;
    auto pick = [&](const f32x16& acc, int kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float a = acc[v];
        second = __builtin_amdgcn_fmed3f(best, second, a);  // second smallest so far
        if (a < best) {
          best = a;
          bk = kb + mfma32_row(v, h);
        }
      }
    };
    int kb = 0;
    // two blocks of 32 codewords at a time: two independent accumulator chains
    for (; kb + 64 <= Kp; kb += 64) {
      f32x16 acc0 = init(kb), acc1 = init(kb + 32);
      float a0[H], a1[H];
#pragma unroll
      for (int s = 0; s < H; ++s) {
        a0[s] = cbT[(h * H + s) * P + kb + l32];
        a1[s] = cbT[(h * H + s) * P + kb + 32 + l32];
      }
      __builtin_amdgcn_sched_barrier(0);  // every operand read ahead of the first multiply
#pragma unroll
      for (int s = 0; s < H; ++s) {
        acc0 = mfma_f32_32x32x2(a0[s], b[s], acc0);
        acc1 = mfma_f32_32x32x2(a1[s], b[s], acc1);
      }
      pick(acc0, kb);
      pick(acc1, kb + 32);
    }
    if (kb < Kp) pick(score(kb), kb);  // Kp % 64 == 32: the last 32 codewords
    {  // merge the halves: best (lower index on ties) and the token's second smallest score
      const float ob = __shfl_xor(best, 32), os = __shfl_xor(second, 32);
      const int ok = __shfl_xor(bk, 32);
      second = fminf(fmaxf(best, ob), fminf(second, os));
      if (ob < best || (ob == best && ok < bk)) {
        best = ob;
        bk = ok;
      }
    }
    const bool need = !(second - best > 2.f * delta);  // no proven margin (NaN included)
    if (__any(need)) {
      const float lim = need ? fmaf(2.f, delta, best) : __builtin_nanf("");
      uint32_t mask[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int bb = 0; bb < kRvqMaxK / 32; ++bb) {
        if (32 * bb < Kp) {
          const f32x16 acc = score(32 * bb);
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (acc[v] <= lim) mask[bb >> 1] |= 1u << (16 * (bb & 1) + v);
        }
      }
      const int rk = rvq_rescore(mask, h, K, [&](int k) {
        double p = 0.0;
#pragma unroll
        for (int s = 0; s < H; ++s) {
          const double dd = res[s] - double(cbT[(h * H + s) * P + k]);
          p = fma(dd, dd, p);
        }
        return p;
      });
      if (need) bk = rk;
    }
    if (h == 0 && n < N) codes[(size_t(n) * R + rho) * G + g] = uint8_t(bk);
#pragma unroll
    for (int s = 0; s < H; ++s) res[s] -= double(cbT[(h * H + s) * P + bk]);
  }
}

// ---------------------------------------------- encode, bf16-scored (w >= 16) --
// The scan over the K codewords runs on bf16 matrix cores.  For token n the
// bf16 score of codeword k is
//   a_k = nrm_k + <bf16(-2 res), bf16(c_k)>    (products exact, fp32 sums)
// with nrm_k the fp32 ||c_k||^2, which starts the matrix-core accumulator.
// With u = 2^-8 the
// bf16 unit roundoff (8 significant bits): bf16(fp32(-2 res_j)) is
// -2 res_j (1 + e1), |e1| <= u (1 + 2^-15), and bf16(c_kj) is c_kj (1 + e2),
// |e2| <= u, so each product is off by at most 2^-7 (1 + 2^-8) |2 res_j c_kj|
// and their sum by 2^-6 (1 + 2^-8) ||res|| ||c_k|| (Cauchy-Schwarz).  The
// fp32 norm is within W 2^-24 of ||c_k||^2, and the fp32 sums of nrm_k and
// the W exact products add at most 2^-17 of the sum of their magnitudes.
// Together, against the exact
// s_k = ||c_k||^2 - 2 <res, c_k>,
//   |a_k - s_k| <= 2^-6 (1 + 2^-7) ||res|| ||c_k|| + 2^-15 ||c_k||^2,
// and the kernel takes, uniformly in k and with room for the fp32 rounding of
// its own norms and square roots,
//   delta = 2^-6 (1 + 2^-6) ||res|| max_k ||c_k|| + 2^-14 max_k ||c_k||^2 + 1e-30.
// A first scan finds min_j a_j, a second (the same instructions, so the same
// a_k) marks every codeword with a_k <= min_j a_j + 2 delta in a 128-bit mask
// per lane, and those are rescored exactly in fp64 (rvq_rescore): about 1.3
// codewords per token at the step's workload.
//
// The bf16 MFMA takes 8 dims per lane per K-step: at step t < W/16 lane half
// h supplies dims h W/2 + 8 t .. + 7 of codeword and residual alike.  The
// accumulator of a block of 32 codewords starts at their norms, kept in LDS in
// the accumulator's order (lane half h, register v holds codeword row
// mfma32_row(v, h)), so every lane of a half reads the same 64 bytes.
// Padding codewords (k >= K) have zero dims and norm +inf, so their score is
// +inf.
template <int W, typename ZT>
__global__ __launch_bounds__(64 * kRvqWaves) void k_rvq_encode_bf(const ZT* __restrict__ Z,
                                                                  const float* __restrict__ C, int64_t stride,
                                                                  uint8_t* __restrict__ codes, int N, int r, int G,
                                                                  int K, int R) {
  constexpr int H = W / 2, T = W / 16, FP = W + 4, WB = W + 16;  // dims per lane, K-steps, fp32 / bf16 row pitch
  constexpr float inf = __builtin_inff();
  extern __shared__ __attribute__((aligned(16))) float sh[];
  float* cbF = sh;                   // [256][FP] fp32 codewords
  float* nrm = cbF + kRvqMaxK * FP;  // [256] ||c_k||^2
  float* bnd = nrm + kRvqMaxK;       // [4]: max ||c_k||^2 (the block's reduction)
  float* nrmv = bnd + 4;             // [256] ||c_k||^2 in accumulator order: [32-codeword block][h][v]
  bf16_t* cbB = reinterpret_cast<bf16_t*>(nrmv + kRvqMaxK);  // [256][WB] bf16 codewords (W used)
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int h = lane >> 5, l32 = lane & 31;
  const int g = blockIdx.x;
  const int n = blockIdx.y * (kRvqWaves * 32) + wave * 32 + l32;
  const int Kp = (K + 31) & ~31;
  const int nb = Kp / 32;

  double res[H];
  rvq_load_res<H, ZT>(Z, n, N, r, g * W + h * H, res);

  for (int rho = 0; rho < R; ++rho) {
    if (rho == 0 || stride != 0) {
      __syncthreads();
      const float* book = C + rho * stride + size_t(g) * K * W;
      // W/4 consecutive threads per codeword (16 bytes each); squared norm by a fixed-order butterfly.
      // Every load of the thread is issued before the first is used.
      constexpr int UPT = (kRvqMaxK * W / 4 + 64 * kRvqWaves - 1) / (64 * kRvqWaves);  // units per thread at K = 256
      f32x4 cv[UPT];
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        const int e = threadIdx.x + u * 64 * kRvqWaves;
        const int k = e / (W / 4);
        cv[u] = (k < K) ? *reinterpret_cast<const f32x4*>(book + size_t(k) * W + 4 * (e % (W / 4)))
                        : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        const int e = threadIdx.x + u * 64 * kRvqWaves;
        if (e >= Kp * W / 4) continue;  // uniform over a codeword's W/4 threads
        const int k = e / (W / 4), j0 = 4 * (e % (W / 4));
        const f32x4 v = cv[u];
        *reinterpret_cast<f32x4*>(cbF + k * FP + j0) = v;
        *reinterpret_cast<u32x2*>(cbB + k * WB + j0) = u32x2{pack2bf(v[0], v[1]), pack2bf(v[2], v[3])};
        float s2 = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) s2 = fmaf(v[q], v[q], s2);
#pragma unroll
        for (int off = 1; off < W / 4; off <<= 1) s2 += __shfl_xor(s2, off);
        if (j0 == 0) {
          nrm[k] = s2;
          // codeword row rho of block k / 32 sits in lane half (rho >> 2) & 1, register 4 (rho >> 3) + (rho & 3)
          const int rho = k & 31;
          nrmv[(2 * (k >> 5) + ((rho >> 2) & 1)) * 16 + 4 * (rho >> 3) + (rho & 3)] = k < K ? s2 : inf;
        }
      }
      __syncthreads();
      if (wave == 0) {  // max ||c_k||^2 over the real codewords (a max: order does not matter; NaN drops out)
        float mx = 0.f;
        for (int k = lane; k < K; k += 64) mx = fmaxf(mx, nrm[k]);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        if (lane == 0) bnd[0] = mx;
      }
      __syncthreads();
    }
    // the residual's bf16 operand (pre-scaled by -2),
    // its norm and the per-token bound
    bf16x8 bB[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      u32x4 u;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        u[e] = pack2bf(float(-2.0 * res[8 * t + 2 * e]), float(-2.0 * res[8 * t + 2 * e + 1]));
      bB[t] = __builtin_bit_cast(bf16x8, u);
    }
    const float rn2 = rvq_norm2<H>(res);
    const float nmax = bnd[0];
    const float delta = fmaf(0x1.04p-6f * sqrtf(rn2), sqrtf(nmax), fmaf(0x1p-14f, nmax, 1e-30f));

    auto scan = [&](int b) {  // bf16 scores of codewords 32 b .. 32 b + 31 (rows of the accumulator)
      const bf16_t* row = cbB + (32 * b + l32) * WB;
      const f32x4* nv = reinterpret_cast<const f32x4*>(nrmv + (2 * b + h) * 16);
      f32x16 acc;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 n4 = nv[q];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[4 * q + e] = n4[e];
      }
#pragma unroll
      for (int t = 0; t < T; ++t) acc = mfma_bf16_32x32x16(ld_bf16x8(row + H * h + 8 * t), bB[t], acc);
      return acc;
    };
    // scan 1: the smallest bf16 score (NaN drops out of fminf)
    float amin = __builtin_inff();
#pragma unroll
    for (int b = 0; b < kRvqMaxK / 32; ++b) {
      if (b < nb) {
        const f32x16 acc = scan(b);
#pragma unroll
        for (int v = 0; v < 16; ++v) amin = fminf(amin, acc[v]);
      }
    }
    amin = fminf(amin, __shfl_xor(amin, 32));
    const float lim = fmaf(2.f, delta, amin);
    // scan 2: candidate mask, bit 16 (b & 1) + v of word b >> 1
    uint32_t mask[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int b = 0; b < kRvqMaxK / 32; ++b) {
      if (b < nb) {
        const f32x16 acc = scan(b);
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (acc[v] <= lim) mask[b >> 1] |= 1u << (16 * (b & 1) + v);
      }
    }
    const int bk = rvq_rescore(mask, h, K, [&](int k) {
      const float* ck = cbF + k * FP + h * H;
      double p = 0.0;
#pragma unroll
      for (int s = 0; s < H; s += 4) {
        const f32x4 c4 = *reinterpret_cast<const f32x4*>(ck + s);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const double dd = res[s + e] - double(c4[e]);
          p = fma(dd, dd, p);
        }
      }
      return p;
    });
    if (h == 0 && n < N) codes[(size_t(n) * R + rho) * G + g] = uint8_t(bk);
#pragma unroll
    for (int s = 0; s < H; ++s) res[s] -= double(cbF[bk * FP + h * H + s]);
  }
}

// LDS of the bf16-scored encode: fp32 codewords [256][W+4], norms [256], bound [4], norms in accumulator
// order [256], bf16 rows [256][W+16]
template <int W>
constexpr size_t rvq_bf_lds() {
  return (size_t(kRvqMaxK) * (W + 4) + 2 * kRvqMaxK + 4) * sizeof(float) + size_t(kRvqMaxK) * (W + 16) * sizeof(bf16_t);
}
// LDS of the fp32-scored encode: transposed codebook [W][Kp+2], norms [Kp], bound
inline size_t rvq_f32_lds(int W, int K) {
  const int Kp = (K + 31) & ~31;
  return (size_t(W) * (Kp + 2) + Kp + 4) * sizeof(float);
}
static_assert(rvq_bf_lds<64>() <= size_t(kMaxLdsBytes), "bf16-scored encode LDS");
static_assert((8 * (kRvqMaxK + 2) + kRvqMaxK + 4) * sizeof(float) <= 65536, "fp32-scored encode LDS");

template <int W>
static void rvq_encode_w(const void* Z, int z_bf16, const float* C, int64_t stride, uint8_t* codes, int N, int r,
                         int G, int K, int R, hipStream_t s) {
  const int tpb = kRvqWaves * 32;
  dim3 grid(G, (N + tpb - 1) / tpb);
  if constexpr (W >= 16) {
    if (z_bf16) {
      const int lds = LdsLimit<k_rvq_encode_bf<W, bf16_t>, int(rvq_bf_lds<W>())>::bytes();
      hipLaunchKernelGGL((k_rvq_encode_bf<W, bf16_t>), grid, dim3(64 * kRvqWaves), lds, s,
                         static_cast<const bf16_t*>(Z), C, stride, codes, N, r, G, K, R);
    } else {
      const int lds = LdsLimit<k_rvq_encode_bf<W, float>, int(rvq_bf_lds<W>())>::bytes();
      hipLaunchKernelGGL((k_rvq_encode_bf<W, float>), grid, dim3(64 * kRvqWaves), lds, s, static_cast<const float*>(Z),
                         C, stride, codes, N, r, G, K, R);
    }
  } else {  // w < 16: fp32 scores on the matrix cores
    const size_t lds = rvq_f32_lds(W, K);
    if (z_bf16)
      hipLaunchKernelGGL((k_rvq_encode<W, bf16_t>), grid, dim3(64 * kRvqWaves), lds, s, static_cast<const bf16_t*>(Z),
                         C, stride, codes, N, r, G, K, R);
    else
      hipLaunchKernelGGL((k_rvq_encode<W, float>), grid, dim3(64 * kRvqWaves), lds, s, static_cast<const float*>(Z),
                         C, stride, codes, N, r, G, K, R);
  }
}

void launch_rvq_encode(const void* Z, int z_bf16, const float* C, int64_t stride, uint8_t* codes, int N, int r, int G,
                       int K, int R, hipStream_t s) {
  switch (r / G) {
    case 2: rvq_encode_w<2>(Z, z_bf16, C, stride, codes, N, r, G, K, R, s); break;
    case 4: rvq_encode_w<4>(Z, z_bf16, C, stride, codes, N, r, G, K, R, s); break;
    case 8: rvq_encode_w<8>(Z, z_bf16, C, stride, codes, N, r, G, K, R, s); break;
    case 16: rvq_encode_w<16>(Z, z_bf16, C, stride, codes, N, r, G, K, R, s); break;
    case 32: rvq_encode_w<32>(Z, z_bf16, C, stride, codes, N, r, G, K, R, s); break;
    case 64: rvq_encode_w<64>(Z, z_bf16, C, stride, codes, N, r, G, K, R, s); break;
    default: break;
  }
}

// Decode: Zq[n][g*W + j] = sum_rho C[rho*stride + (g*K + code)*W + j], rounds in
// order.  A thread owns CH consecutive outputs of one (token, group): it reads
// the R codes once and moves its codeword slices as 16-byte vectors.
// PKT (the codebook sync fused in; the round stride a multiple of W, so that
// codeword k of group g in round rho has the flat index rho stride / W + g K + k,
// the numbering of the sync, and `total` codewords exist): the n <= kPktMax codewords
// idx[e] of a packet take the values vals[e] -- the last entry naming a codeword
// wins -- both in the decoded sums (a codeword named in the packet is read from
// vals, never from C) and in C itself, where global thread e < n stores entry e
// unless a later entry names the same codeword.  No thread reads from C a
// codeword that another thread stores, so the result is that of the sync
// followed by the decode.
constexpr int kPktMax = 64;

template <typename OT, int CH, bool PKT = false>
__global__ __launch_bounds__(256) void k_rvq_decode(const uint8_t* __restrict__ codes, const float* C, int64_t stride,
                                                    OT* __restrict__ Zq, int N, int r, int G, int K, int R,
                                                    float* Cw = nullptr, const int32_t* __restrict__ idx = nullptr,
                                                    const float* __restrict__ vals = nullptr, int n = 0,
                                                    int64_t total = 0) {
  const int W = r / G;
  __shared__ int32_t pid[PKT ? kPktMax : 1];
  if (PKT) {
    if (threadIdx.x < n) pid[threadIdx.x] = idx[threadIdx.x];
    __syncthreads();
    const int q = blockIdx.x * 256 + threadIdx.x;
    if (q < n) {
      const int64_t dst = pid[q];
      bool win = dst >= 0 && dst < total;
      for (int e = q + 1; e < n; ++e) win = win && pid[e] != dst;
      if (win)
        for (int j = 0; j < W; ++j) Cw[dst * W + j] = vals[size_t(q) * W + j];
    }
  }
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;  // chunk index
  const int per_tok = r / CH;
  if (e >= int64_t(N) * per_tok) return;
  const int n_tok = int(e / per_tok), col = int(e % per_tok) * CH;
  const int g = col / W, j = col % W;
  float acc[CH];
#pragma unroll
  for (int q = 0; q < CH; ++q) acc[q] = 0.f;
  for (int rho = 0; rho < R; ++rho) {
    const int k = codes[(size_t(n_tok) * R + rho) * G + g];
    if (k >= K) continue;  // a code >= K (corrupt input) adds nothing
    const float* cw = C + rho * stride + (size_t(g) * K + k) * W + j;
    if (PKT) {
      const int64_t cq = rho * (stride / W) + int64_t(g) * K + k;  // the codeword's flat index
      int slot = -1;
      for (int t = 0; t < n; ++t) slot = pid[t] == cq ? t : slot;
      if (slot >= 0) cw = vals + size_t(slot) * W + j;
    }
    if (CH >= 4) {
#pragma unroll
      for (int q = 0; q < CH; q += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(cw + q);
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) acc[q + e2] += v[e2];
      }
    } else {
#pragma unroll
      for (int q = 0; q < CH; ++q) acc[q] += cw[q];
    }
  }
  OT* o = Zq + size_t(n_tok) * r + col;
#pragma unroll
  for (int q = 0; q < CH; ++q) o[q] = from_f32<OT>(acc[q]);
}

// Narrow groups (W = 2 or 4, r % 8 == 0): a thread owns 8 consecutive outputs,
// i.e. 8 / W whole groups; per round it reads their codes with one load and
// each codeword as one W-float vector.
constexpr int kDecRounds = 4;
template <typename OT, int W>
__global__ __launch_bounds__(256) void k_rvq_decode_narrow(const uint8_t* __restrict__ codes,
                                                           const float* __restrict__ C, int64_t stride,
                                                           OT* __restrict__ Zq, int N, int r, int G, int K, int R) {
  constexpr int NG = 8 / W;  // groups per thread
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int per_tok = r / 8;
  if (e >= int64_t(N) * per_tok) return;
  const int n = int(e / per_tok), col = int(e % per_tok) * 8;
  const int g0 = col / W;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  // rounds in batches of kDecRounds: the batch's codes are loaded together, then
  // its codewords, so a thread waits for two loads per batch, not two per round
  for (int r0 = 0; r0 < R; r0 += kDecRounds) {
    uint32_t kk[kDecRounds];
#pragma unroll
    for (int u = 0; u < kDecRounds; ++u) {
      const uint8_t* cp = codes + (size_t(n) * R + min(r0 + u, R - 1)) * G + g0;
      if (NG == 4) kk[u] = *reinterpret_cast<const uint32_t*>(cp);
      else kk[u] = *reinterpret_cast<const uint16_t*>(cp);
    }
    float v[kDecRounds][8];
#pragma unroll
    for (int u = 0; u < kDecRounds; ++u) {
      const int rho = min(r0 + u, R - 1);
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        int k = int((kk[u] >> (8 * i)) & 0xffu);
        k = k < K ? k : 0;
        const float* cw = C + rho * stride + (size_t(g0 + i) * K + k) * W;
        if (W == 2) {
          const float2 t2 = *reinterpret_cast<const float2*>(cw);
          v[u][2 * i] = t2.x;
          v[u][2 * i + 1] = t2.y;
        } else {
          const f32x4 t4 = *reinterpret_cast<const f32x4*>(cw);
#pragma unroll
          for (int q = 0; q < 4; ++q) v[u][4 * i + q] = t4[q];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kDecRounds; ++u) {
      if (r0 + u >= R) break;
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        if (int((kk[u] >> (8 * i)) & 0xffu) >= K) continue;  // a code >= K (corrupt input) adds nothing
#pragma unroll
        for (int q = 0; q < W; ++q) acc[W * i + q] += v[u][W * i + q];
      }
    }
  }
  OT* o = Zq + size_t(n) * r + col;
#pragma unroll
  for (int q = 0; q < 8; ++q) o[q] = from_f32<OT>(acc[q]);
}

void launch_rvq_decode(const uint8_t* codes, const float* C, int64_t stride, void* Zq, int out_bf16, int N, int r,
                       int G, int K, int R, hipStream_t s) {
  const int W = r / G;
  // the narrow path's vector loads need: codes at a multiple of 8 / W bytes, codewords at W * 4 bytes
  const bool narrow_ok = (W == 2 || W == 4) && r % 8 == 0 && reinterpret_cast<uintptr_t>(codes) % (8 / W) == 0 &&
                         reinterpret_cast<uintptr_t>(C) % (4 * W) == 0 && stride % W == 0;
  if (narrow_ok) {
    dim3 grid(unsigned((int64_t(N) * (r / 8) + 255) / 256));
#define MAPL_DECN(OTv, Wv)                                                                                     \
  hipLaunchKernelGGL((k_rvq_decode_narrow<OTv, Wv>), grid, dim3(256), 0, s, codes, C, stride,                   \
                     static_cast<OTv*>(Zq), N, r, G, K, R)
    if (out_bf16) {
      if (W == 2) MAPL_DECN(bf16_t, 2);
      else MAPL_DECN(bf16_t, 4);
    } else {
      if (W == 2) MAPL_DECN(float, 2);
      else MAPL_DECN(float, 4);
    }
#undef MAPL_DECN
    return;
  }
  const int CH = (W % 8 == 0) ? 8 : (W % 4 == 0) ? 4 : (W % 2 == 0) ? 2 : 1;
  const int64_t tot = int64_t(N) * r / CH;
  dim3 grid(unsigned((tot + 255) / 256));
#define MAPL_DEC(OTv, CHv)                                                                                         \
  hipLaunchKernelGGL((k_rvq_decode<OTv, CHv>), grid, dim3(256), 0, s, codes, C, stride, static_cast<OTv*>(Zq), N, r, \
                     G, K, R)
  if (out_bf16) {
    if (CH == 8) MAPL_DEC(bf16_t, 8);
    else if (CH == 4) MAPL_DEC(bf16_t, 4);
    else if (CH == 2) MAPL_DEC(bf16_t, 2);
    else MAPL_DEC(bf16_t, 1);
  } else {
    if (CH == 8) MAPL_DEC(float, 8);
    else if (CH == 4) MAPL_DEC(float, 4);
    else if (CH == 2) MAPL_DEC(float, 2);
    else MAPL_DEC(float, 1);
  }
#undef MAPL_DEC
}

// Stream apply: C[idx[q]*W + j] = vals[q*W + j].  One thread per streamed
// codeword q; a later duplicate of idx[q] in the same call wins, so q writes
// only if no later entry names the same codeword.  The later entries are
// scanned in tiles of kStreamTile ids staged in LDS by the block (work n^2/2
// for n codewords, all from LDS: a full-codebook sync of 64k codewords is a
// fraction of a millisecond).
constexpr int kStreamTile = 1024;

__global__ __launch_bounds__(256) void k_rvq_stream(float* __restrict__ C, const int32_t* __restrict__ idx,
                                                    const float* __restrict__ vals, int n, int W, int64_t total) {
  __shared__ int32_t tile[kStreamTile];
  const int q = blockIdx.x * 256 + threadIdx.x;
  const int64_t dst = q < n ? idx[q] : -1;
  bool win = q < n && dst >= 0 && dst < total;
  for (int t0 = blockIdx.x * 256; t0 < n; t0 += kStreamTile) {
    __syncthreads();
    const int lim = min(kStreamTile, n - t0);
    for (int e = threadIdx.x; e < lim; e += 256) tile[e] = idx[t0 + e];
    __syncthreads();
    if (win) {
      for (int e = max(0, q + 1 - t0); e < lim; ++e)
        if (tile[e] == dst) {
          win = false;
          break;
        }
    }
  }
  if (win) {
    const float* v = vals + size_t(q) * W;
    float* c = C + dst * W;
    for (int j = 0; j < W; ++j) c[j] = v[j];
  }
}

void launch_rvq_stream(float* C, const int32_t* idx, const float* vals, int n, int w, int64_t total_codewords,
                       hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(k_rvq_stream, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, C, idx, vals, n, w,
                     total_codewords);
}

// Sync then decode in one launch where the packet fits the decode kernel's table
// (n <= kPktMax), the rows move as 16-byte vectors (w >= 8, w % 4 == 0, vals
// 16-byte aligned) and the round stride is a whole number of codewords; the
// narrow groups (w = 2, 4) keep their own decode kernel.  Otherwise the two
// launches run in that order.
void launch_rvq_stream_decode(float* C, int64_t stride, int64_t total, const int32_t* idx, const float* vals, int n,
                              const uint8_t* codes, void* Zq, int out_bf16, int N, int r, int G, int K, int R,
                              hipStream_t s) {
  const int W = r / G;
  const bool fuse = n > 0 && n <= kPktMax && W >= 8 && W % 4 == 0 && stride % W == 0 &&
                    reinterpret_cast<uintptr_t>(vals) % 16 == 0;
  if (!fuse) {
    launch_rvq_stream(C, idx, vals, n, W, total, s);
    if (N > 0) launch_rvq_decode(codes, C, stride, Zq, out_bf16, N, r, G, K, R, s);
    return;
  }
  const int CH = (W % 8 == 0) ? 8 : 4;
  const int64_t tot = int64_t(N) * r / CH;
  dim3 grid(unsigned(std::max<int64_t>(1, (tot + 255) / 256)));
#define MAPL_DECP(OTv, CHv)                                                                                      \
  hipLaunchKernelGGL((k_rvq_decode<OTv, CHv, true>), grid, dim3(256), 0, s, codes, C, stride, static_cast<OTv*>(Zq), \
                     N, r, G, K, R, C, idx, vals, n, total)
  if (out_bf16) {
    if (CH == 8) MAPL_DECP(bf16_t, 8);
    else MAPL_DECP(bf16_t, 4);
  } else {
    if (CH == 8) MAPL_DECP(float, 8);
    else MAPL_DECP(float, 4);
  }
#undef MAPL_DECP
}

}  // namespace mapl
