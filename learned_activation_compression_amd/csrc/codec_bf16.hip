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
                                                    int d, int r, int ra, int V) {
  __shared__ __attribute__((aligned(16))) float redbuf[4 * RB * 64 * 16];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int hi = lane >> 5, l32 = lane & 31;
  const int tok0 = blockIdx.x * 64;
  const int rbase = blockIdx.y * (RB * 32);
  const int Sd = d >> 4;
  const int Se = ANCHOR ? (ra >> 4) : 0;
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
    er0 = E + size_t(e0 ? t0 : 0) * ra + 8 * hi;
    er1 = E + size_t(e1 ? t1 : 0) * ra + 8 * hi;
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

// ------------------------------------------------------ reduce, streamed --
// For r >= 128.  One block: 64 tokens x 128 RBW output columns (all r, or the
// blockIdx.y-th such slice when the token tiles alone would not cover the
// chip); wave w owns the r-blocks [w RBW, (w+1) RBW) of the slice over the
// whole contraction, so no partial tiles are summed.  The contraction runs in chunks of 64 channels: d/64 chunks of
// the token rows against AtF, then (ANCHOR) r/64 chunks of the anchor rows
// E[t] against QnF.  Each chunk -- 64 token rows of 128 bytes and the chunk's
// weight fragments of every wave -- is copied by global_load_lds straight into
// slot c % S of an LDS ring, S - 1 chunks ahead of the one being multiplied,
// without passing through registers.
//   Token row t of a slot holds its eight 16-byte units at positions
//   u ^ (t & 7): the copy picks, per lane, the source unit that belongs at its
//   (fixed) destination, and the matrix-core reads (32 rows, one unit each)
//   then hit 8 different bank groups.
//   Synchronisation per chunk: each wave waits until its own copies of chunk
//   c are done (vmcnt counts the copies of the S - 2 younger chunks still in
//   flight), a barrier makes every wave's copies visible and guarantees that
//   all waves are done with chunk c - 1, whose slot then receives chunk
//   c + S - 1.  Copies past the last chunk repeat it into a slot never read.
constexpr int kRedKC = 64;  // channels per chunk

template <int RBW, int S>
struct RedRing {
  static constexpr int XU = 64 * kRedKC * 2 / 16;  // 16-byte units of token rows per slot
  static constexpr int WU = 4 * 4 * RBW * 64;      // 4 waves x 4 K-steps x RBW fragments x 64 lanes
  static constexpr int SLOT = XU + WU;
  static constexpr int PER = 2 + 4 * RBW;          // copies per wave per chunk
  static constexpr size_t BYTES = size_t(S) * SLOT * 16;
};

// OUTF: instead of bf16 Z, write fp32 rows alpha * (X A) to Uf and each output
// wave's max |value| to part[4 * blockIdx.x + w] (the anchor-table gradient's
// projection, X = Y and the weight pack PF).
template <int RBW, int S, int G, bool ANCHOR, bool OUTF = false>
__global__ __launch_bounds__(256 * G) void k_tok_reduce_dma(const bf16_t* __restrict__ X,
                                                            const bf16_t* __restrict__ AtF,
                                                            const int32_t* __restrict__ tids,
                                                            const bf16_t* __restrict__ E,
                                                            const bf16_t* __restrict__ QnF, bf16_t* __restrict__ Z,
                                                            int N, int d, int r, int ra, int V,
                                                            float* __restrict__ Uf, float alpha,
                                                            float* __restrict__ part) {
  using RR = RedRing<RBW, S>;
  static_assert(S % G == 0 && S / G >= 2, "each wave group needs its own slots");
  extern __shared__ __attribute__((aligned(16))) u32x4 ring[];
  const int lane = threadIdx.x & 63, wv = wave_id();
  const int grp = wv >> 2, w = wv & 3;  // group grp multiplies the chunks c with c % G == grp
  const int hi = lane >> 5, l32 = lane & 31;
  const int tok0 = blockIdx.x * 64;
  const int MB = r >> 5;
  const int cb = blockIdx.y * 4 * RBW;  // first 32-column block of the block's slice
  const int cx = d / kRedKC, nch = cx + (ANCHOR ? ra / kRedKC : 0);

  // copy role: this lane copies unit (lane & 7) of rows 16 w + 8 q + (lane >> 3), q = 0, 1;
  // the row's low 3 bits are lane >> 3, so the source unit is (lane & 7) ^ (lane >> 3)
  const int cu = (lane & 7) ^ (lane >> 3);
  // element offsets of the two copied rows: in X (token rows) and in E (anchor rows)
  size_t xoff[2], eoff[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int tk = min(tok0 + 16 * w + 8 * q + (lane >> 3), N - 1);
    xoff[q] = size_t(tk) * d + 8 * cu;
    eoff[q] = 8 * cu;
    if (ANCHOR) {
      const int t = tids[tk];
      eoff[q] += size_t((t >= 0 && t < V) ? t : 0) * ra;
    }
  }
  // matrix-core operand masks: token tb*32 + l32 with an invalid id reads a zero anchor row
  uint32_t bm[2] = {~0u, ~0u};
  if (ANCHOR) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int t = tids[min(tok0 + tb * 32 + l32, N - 1)];
      bm[tb] = (t >= 0 && t < V) ? ~0u : 0u;
    }
    asm volatile("" : : "v"(bm[0]), "v"(bm[1]));  // resolve the ids before the first copy is queued
  }

  // chunk c into slot c % S; past the last chunk the last one is copied again into that
  // (free) slot, which is never read
  auto issue = [&](int c) {
    u32x4* slot = ring + (c % S) * RR::SLOT;
    c = min(c, nch - 1);
    const bool xs = c < cx;
    const int ch = (xs ? c : c - cx) * kRedKC;
    copy16_to_lds((xs ? X + xoff[0] : E + eoff[0]) + ch, slot + (16 * w) * 8);
    copy16_to_lds((xs ? X + xoff[1] : E + eoff[1]) + ch, slot + (16 * w + 8) * 8);
    const bf16_t* wb = (xs ? AtF : QnF) + size_t(4 * (xs ? c : c - cx)) * MB * 512;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int i = 0; i < RBW; ++i)
        copy16_to_lds(wb + (size_t(ks * MB + cb + w * RBW + i) * 64 + lane) * 8,
                      slot + RR::XU + ((w * 4 + ks) * RBW + i) * 64);
  };

  f32x16 acc[2][RBW];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int i = 0; i < RBW; ++i) acc[tb][i] = f32x16{};

#pragma unroll
  for (int u = 0; u < S / G - 1; ++u) issue(grp + G * u);
  for (int c0 = 0; c0 < nch; c0 += G) {
    const int c = c0 + grp;
    wait_vmcnt<(S / G - 2) * RR::PER>();  // this wave's copies of chunk c are done
    __syncthreads();                       // everyone's are; chunk c - G is free
    issue(c + S - G);
    if (c < nch) {
      const u32x4* slot = ring + (c % S) * RR::SLOT;
      const bool anchor = ANCHOR && c >= cx;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int pu = (2 * ks + hi) ^ (l32 & 7);
        bf16x8 b[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          b[tb] = __builtin_bit_cast(bf16x8, slot[(tb * 32 + l32) * 8 + pu]);
          if (ANCHOR) b[tb] = mask_bf16x8(b[tb], anchor ? bm[tb] : ~0u);
        }
#pragma unroll
        for (int i = 0; i < RBW; ++i) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, slot[RR::XU + ((w * 4 + ks) * RBW + i) * 64 + lane]);
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) acc[tb][i] = mfma_bf16_32x32x16(a, b[tb], acc[tb][i]);
        }
      }
    }
  }
  wait_vmcnt<0>();  // no copy may still be writing the ring
  if (G > 1) {
    // group 1 hands its partial tiles to group 0 through the ring, added in a fixed order
    __syncthreads();
    f32x4* red = reinterpret_cast<f32x4*>(ring) + size_t(w) * (2 * RBW * 4 * 64);
    if (grp == 1) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < RBW; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            red[((tb * RBW + i) * 4 + q) * 64 + lane] =
                f32x4{acc[tb][i][4 * q], acc[tb][i][4 * q + 1], acc[tb][i][4 * q + 2], acc[tb][i][4 * q + 3]};
    }
    __syncthreads();
    if (grp == 1) return;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int i = 0; i < RBW; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 o = red[((tb * RBW + i) * 4 + q) * 64 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[tb][i][4 * q + e] += o[e];
        }
  }

  // lane holds, for token tb*32 + l32, 4 consecutive output columns per register group
  if (OUTF) {
    float local = 0.f;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int n = tok0 + tb * 32 + l32;
      if (n >= N) continue;
#pragma unroll
      for (int i = 0; i < RBW; ++i) {
        float* row = Uf + size_t(n) * r + (cb + w * RBW + i) * 32 + 4 * hi;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = alpha * acc[tb][i][4 * q + e];
            local = fmaxf(local, v[e] == v[e] ? fabsf(v[e]) : __builtin_inff());  // NaN counts as +inf
          }
          *reinterpret_cast<f32x4*>(row + 8 * q) = v;
        }
      }
    }
    for (int off = 32; off > 0; off >>= 1) local = fmaxf(local, __shfl_xor(local, off));
    if (lane == 0) part[4 * (blockIdx.y * gridDim.x + blockIdx.x) + w] = local;
    return;
  }
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int n = tok0 + tb * 32 + l32;
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
      bf16_t* row = Z + size_t(n) * r + (cb + w * RBW + i) * 32 + 4 * hi;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<u32x2*>(row + 8 * q) =
            u32x2{pack2bf(acc[tb][i][4 * q], acc[tb][i][4 * q + 1]), pack2bf(acc[tb][i][4 * q + 2], acc[tb][i][4 * q + 3])};
    }
  }
}

template <int RBW, int S, int G, bool ANCHOR, bool OUTF = false>
static void launch_reduce_dma(const uint16_t* in, const uint16_t* AtF, const int32_t* tids, const uint16_t* E,
                              const uint16_t* QnF, uint16_t* out, int N, int d, int r, int ra, int V, hipStream_t s,
                              float* Uf = nullptr, float alpha = 1.f, float* part = nullptr, KernelEvents ev = {}) {
  auto k = k_tok_reduce_dma<RBW, S, G, ANCHOR, OUTF>;
  const int lds = LdsLimit<k_tok_reduce_dma<RBW, S, G, ANCHOR, OUTF>, int(RedRing<RBW, S>::BYTES)>::bytes();
  // r / (128 RBW) column slices over blockIdx.y
  launch_k(ev, k, dim3((N + 63) / 64, r / (128 * RBW)), dim3(256 * G), uint32_t(lds), s, in, AtF, tids, E, QnF, out,
           N, d, r, ra, V, Uf, alpha, part);
}

bool launch_tok_reduce_f32out(const uint16_t* in, const uint16_t* F, float* U, float alpha, float* part, int N,
                              int d, int r, hipStream_t s) {
  if (r == 128) {
    launch_reduce_dma<1, 6, 2, false, true>(in, F, nullptr, nullptr, nullptr, nullptr, N, d, r, 0, 0, s, U, alpha,
                                            part);
    return true;
  }
  if (r == 256) {
    launch_reduce_dma<2, 3, 1, false, true>(in, F, nullptr, nullptr, nullptr, nullptr, N, d, r, 0, 0, s, U, alpha,
                                            part);
    return true;
  }
  return false;
}

void launch_tok_reduce_bf16(const uint16_t* in, const uint16_t* AtF, const int32_t* tids, const uint16_t* E,
                            const uint16_t* QnF, uint16_t* out, int N, int d, int r, int ra, int V, hipStream_t s,
                            KernelEvents ev) {
  // ANCHOR = true is the compress map of Eq. (1); false is the plain product (gZ = gXhat A).
  // `ev` (optional) brackets the one compress kernel for r < 512.
  const bool anc = E != nullptr && ra > 0;
  if (!anc) E = nullptr;
  if (r >= 512 && launch_tok_gemm_bf16(in, d, tids, V, E, anc ? ra : 0, AtF, QnF, out, N, r, s)) return;
  if (r == 128) {
    if (anc) launch_reduce_dma<1, 6, 2, true>(in, AtF, tids, E, QnF, out, N, d, r, ra, V, s, nullptr, 1.f, nullptr, ev);
    else launch_reduce_dma<1, 6, 2, false>(in, AtF, tids, E, QnF, out, N, d, r, ra, V, s, nullptr, 1.f, nullptr, ev);
    return;
  }
  if (r == 256) {
    if ((N + 63) / 64 < 256) {  // too few token tiles to fill the chip: two 128-column slices per tile
      if (anc) launch_reduce_dma<1, 6, 2, true>(in, AtF, tids, E, QnF, out, N, d, r, ra, V, s, nullptr, 1.f, nullptr, ev);
      else launch_reduce_dma<1, 6, 2, false>(in, AtF, tids, E, QnF, out, N, d, r, ra, V, s, nullptr, 1.f, nullptr, ev);
      return;
    }
    if (anc) launch_reduce_dma<2, 3, 1, true>(in, AtF, tids, E, QnF, out, N, d, r, ra, V, s, nullptr, 1.f, nullptr, ev);
    else launch_reduce_dma<2, 3, 1, false>(in, AtF, tids, E, QnF, out, N, d, r, ra, V, s, nullptr, 1.f, nullptr, ev);
    return;
  }
  if (r == 512) {
    if (anc) launch_reduce_dma<4, 2, 1, true>(in, AtF, tids, E, QnF, out, N, d, r, ra, V, s, nullptr, 1.f, nullptr, ev);
    else launch_reduce_dma<4, 2, 1, false>(in, AtF, tids, E, QnF, out, N, d, r, ra, V, s, nullptr, 1.f, nullptr, ev);
    return;
  }
  const int nb = r / 32;
  const int RB = (nb % 4 == 0) ? 4 : (nb % 2 == 0) ? 2 : 1;
  dim3 grid((N + 63) / 64, r / (RB * 32));
  auto k = anc ? (RB == 4 ? k_tok_reduce<4, 4, true> : RB == 2 ? k_tok_reduce<2, 6, true> : k_tok_reduce<1, 8, true>)
               : (RB == 4 ? k_tok_reduce<4, 4, false> : RB == 2 ? k_tok_reduce<2, 6, false>
                                                               : k_tok_reduce<1, 8, false>);
  launch_k(ev, k, grid, dim3(256), 0u, s, in, AtF, tids, E, QnF, out, N, d, r, ra, V);
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
// block's loads overlap the other's matrix-core work; with 64-token tiles
// (32 KB) four do (MINB = 4), which measured faster for 512-byte rows.
// EADD (the full-rank anchor, P = I): E is [V][d] and its rows are added to
// the output instead of entering the contraction.  Each lane loads the
// 8-byte pieces of E[t] that match its accumulators before the matrix-core
// loop, and adds them in fp32 before the one rounding to bf16.
template <int TB, int PER, int P, int MINB = 2, bool EADD = false>
__global__ __launch_bounds__(256, MINB) void k_tok_expand(const bf16_t* __restrict__ in, const bf16_t* __restrict__ AF,
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
  const int S = (E != nullptr && !EADD) ? 2 * Sz : Sz;
  const int uz = 2 * Sz;                 // units of the `in` part
  const int msk = UR >= 8 ? 7 : UR - 1;

  // EADD: this lane's pieces of the anchor rows (token j*32 + l32; channels
  // ch0 + 32 i + 8 g + 4 hi .. + 3), zero for an invalid id
  u32x2 ev[EADD ? TB : 1][2][4];
  if (EADD) {
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      const int id = tids[min(tok0 + j * 32 + l32, N - 1)];
      const bool ok = wave_on && id >= 0 && id < V;
      const bf16_t* er = E + size_t(ok ? id : 0) * d + (wave_on ? ch0 : 0) + 4 * hi;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x2 x = *reinterpret_cast<const u32x2*>(er + i * 32 + 8 * g);
          ev[j][i][g] = ok ? x : u32x2{0u, 0u};
        }
    }
  }

  // ---- 1. stage token rows: every thread first loads the token ids of its
  // PER units (PER = TT * UR / 256, a compile-time constant so that the loops
  // below carry no branches), then issues all of its row loads, then writes
  // them to LDS -- two memory round trips in total.
  int tk[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int t = (threadIdx.x + 256 * k) >> ur_log2;
    tk[k] = (E != nullptr && !EADD) ? tids[min(tok0 + t, N - 1)] : 0;
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
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = acc[i][j][4 * g + e];
          if (EADD) {
            const u32x2 x = ev[EADD ? j : 0][i][g];
            y[0] += bf2f(uint16_t(x[0] & 0xffffu));
            y[1] += bf2f(uint16_t(x[0] >> 16));
            y[2] += bf2f(uint16_t(x[1] & 0xffffu));
            y[3] += bf2f(uint16_t(x[1] >> 16));
          }
          dst[0] = pack2bf(y[0], y[1]);
          dst[1] = pack2bf(y[2], y[3]);
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

bool launch_tok_expand_bf16(const uint16_t* in, const uint16_t* AF, const int32_t* tids, const uint16_t* E,
                            const uint16_t* PtF, uint16_t* out, int N, int d, int r, int ra, int V, hipStream_t s) {
  if (ra == 0) E = nullptr;
  // the staged-row kernel takes an anchor of rank r only; other ranks use the token GEMM
  if (r >= 256 || (E != nullptr && ra != r))
    return launch_tok_gemm_bf16(in, r, tids, V, E, E != nullptr ? ra : 0, AF, PtF, out, N, d, s);
  const int S = (E != nullptr) ? r / 8 : r / 16;  // K-steps
  const int UR = 2 * S;                            // 16-byte units per token row (a power of two)
  int ur_log2 = 0;
  while ((1 << ur_log2) < UR) ++ur_log2;
  // token tile: the staged rows (TT * UR * 16 B) and the output tile (TT * 512 B) share <= 64 KB;
  // 512-byte rows (r = 128 with its anchor) take 64-token tiles, four blocks per CU
  const int TB = (UR < 32) ? 4 : (UR <= 64) ? 2 : 1;
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
  else if (TB == 2 && per == 8)
    hipLaunchKernelGGL((k_tok_expand<2, 8, P, 4>), dim3(nx * ny), dim3(256), lds, s, in, AF, tids, E, PtF, out, N, d,
                       r, V, nx, ny, ur_log2);
  else if (TB == 2) MAPL_EXPAND(2, 16);
  else MAPL_EXPAND(1, 16);
#undef MAPL_EXPAND
  return true;
}

// out[N][d] = in[N][r] A^T + E[t] for the full-rank anchor (E [V][d], P = I):
// the staged-row kernel with the anchor rows added in its epilogue for
// r <= 128, the token GEMM's epilogue otherwise.
bool launch_tok_expand_eadd_bf16(const uint16_t* in, const uint16_t* AF, const int32_t* tids, const uint16_t* E,
                                 uint16_t* out, int N, int d, int r, int V, hipStream_t s) {
  if (r > 128 || r < 64) return launch_tok_gemm_eadd_bf16(in, r, tids, V, E, AF, out, N, d, s);
  const int UR = r / 8;  // 16-byte units of a Z row (8 or 16)
  int ur_log2 = 0;
  while ((1 << ur_log2) < UR) ++ur_log2;
  constexpr int TB = 2, TT = TB * 32;
  const size_t lds = size_t(TT) * 512;  // the output tile; the staged rows are smaller
  const int nx = (d + 255) / 256, ny = (N + TT - 1) / TT;
  if (UR == 16)
    hipLaunchKernelGGL((k_tok_expand<TB, 4, 4, 2, true>), dim3(nx * ny), dim3(256), lds, s, in, AF, tids, E, nullptr,
                       out, N, d, r, V, nx, ny, ur_log2);
  else
    hipLaunchKernelGGL((k_tok_expand<TB, 2, 4, 2, true>), dim3(nx * ny), dim3(256), lds, s, in, AF, tids, E, nullptr,
                       out, N, d, r, V, nx, ny, ur_log2);
  return true;
}

// ------------------------------------------------------------------ gram --
// part[s][i][j] = sum over the tokens n of split s of L[n][i] R[n][j] for
// i < Ld + Le, j < Rd.  Row i < Ld of L is in[n][i] (in is [N][ldin]); row
// Ld + q is E[tids[n]][q] (zero for an id outside [0, V)).
//
// Block: 128 rows x TJ columns of one token split; the 4 waves tile it as
// WI x WJ (64 x 64 each for TJ = 128).  Tokens stream in chunks of 64 through
// two LDS buffers holding the chunk transposed, [row][token]: row t of a
// buffer is 8 units of 16 bytes (8 tokens each), unit c stored at position
// c ^ (t & 7), so that the matrix-core reads (32 rows, one unit each) and the
// staging writes (8 lanes, 8 different units) both spread over the banks.
// Staging: thread (tg, g) loads the 8 x 8 block of tokens 8 tg..+7 and rows
// 8 g..+7 as eight 16-byte row segments (each wave instruction reads eight
// full 128-byte lines), transposes it in registers with byte permutes and
// writes eight units.  The loads of the next three chunks are in flight while
// the current chunk is multiplied.
constexpr int kGramTok = 64;     // tokens per chunk (4 matrix-core K-steps)
constexpr int kGramRound = 512;  // tokens per block (8 chunks) unless that leaves a partial wave of blocks

__device__ __forceinline__ void transpose8x8_b16(const u32x4 (&v)[8], u32x4 (&o)[8]) {
  // o[q] word k = (element q of v[2k], element q of v[2k+1]) as (low, high)
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint32_t sel = (q & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[q][k] = __builtin_amdgcn_perm(v[2 * k + 1][q >> 1], v[2 * k][q >> 1], sel);
  }
}

template <int TJ, int NR>
__global__ __launch_bounds__(256) void k_gram2(const bf16_t* __restrict__ in, int64_t ldin, int Ld,
                                               const int32_t* __restrict__ tids, int V,
                                               const bf16_t* __restrict__ E, int Le, const bf16_t* __restrict__ R,
                                               int Rd, float* __restrict__ part, int N, int tps, int ntile_i,
                                               int ntile_j) {
  constexpr int WJ = (TJ == 128) ? 2 : 1;
  constexpr int WI = 4 / WJ;
  constexpr int MI = 128 / WI / 32, MJ = TJ / WJ / 32;
  constexpr int BUF = (128 + TJ) * 8;  // units per buffer
  __shared__ u32x4 sm[2 * BUF];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int hi = lane >> 5, l32 = lane & 31;
  const int wi = wave / WJ, wj = wave % WJ;
  const int bid = xcd_swizzle(blockIdx.x, int(gridDim.x));
  const int ti = bid % ntile_i, tj = (bid / ntile_i) % ntile_j, sp = bid / (ntile_i * ntile_j);
  const int i0 = ti * 128, j0 = tj * TJ;
  const int rows = Ld + Le;
  const int nb = sp * tps, ne = min(N, nb + tps);

  // staging role of this thread
  const int tid = threadIdx.x;
  const bool isL = tid < 128, isR = tid >= 128 && tid < 128 + TJ;
  const int tg = tid & 7, g = (isL ? tid : tid - 128) >> 3;
  const int srow = isL ? i0 + 8 * g : j0 + 8 * g;  // first row (L) or column (R) of the 8 x 8 block
  constexpr int D = 3;  // chunks whose loads are in flight while one is multiplied
  u32x4 v[D][8];
  uint32_t mk[D];  // bit e: element e of v[u] is real data (else it is zeroed when staged)
  int tq[D][8];    // anchor rows: token ids of the chunk D ahead of the one in v[u]
  // an anchor-row tile (rows >= Ld come from E[tids]); uniform over the block
  const bool tileE = __builtin_amdgcn_readfirstlane(int(Le > 0 && i0 >= Ld)) != 0;
  const bool roleL = wave < 2;             // waves 0-1 stage L, waves 2-3 stage R (uniform per wave)
  const bool active = roleL || isR;        // lanes of waves 2-3 past the TJ columns stage nothing
  const bool insideE = srow < rows;
  // element e of a load is row idx_e of `base` (stride `stride`)
  const bf16_t* base;
  int64_t stride;
  if (roleL && tileE) {
    base = E + (insideE ? srow - Ld : 0);
    stride = Le;
  } else if (roleL) {
    base = in + srow;
    stride = ldin;
  } else {
    base = R + (isR ? srow : 0);
    stride = Rd;
  }

  // Loads are unconditional from clamped addresses; what falls outside is
  // zeroed only when staged, so that no select waits on a load and the loads
  // of D chunks stay in flight.  Anchor rows need their token ids first: those
  // of chunk c + D are loaded right after the rows of chunk c, so waiting for
  // them never waits for a later chunk.
  auto load_tids = [&](int (&t)[8], int rb, int c) {
    const int n0 = rb + c * kGramTok + 8 * tg;
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = tids[min(n0 + e, ne - 1)];
  };
  auto load = [&](u32x4 (&w)[8], uint32_t& m, int (&t)[8], int rb, int c) {
    const int n0 = rb + c * kGramTok + 8 * tg;
    m = 0u;
    if (roleL && tileE) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool ok = insideE && (n0 + e < ne) && t[e] >= 0 && t[e] < V;
        w[e] = *reinterpret_cast<const u32x4*>(base + size_t(ok ? t[e] : 0) * stride);
        m |= uint32_t(ok) << e;
      }
      load_tids(t, rb, c + D);
    } else {  // token rows of X or R
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        w[e] = *reinterpret_cast<const u32x4*>(base + size_t(min(n0 + e, ne - 1)) * stride);
        m |= uint32_t(active && (n0 + e < ne)) << e;
      }
    }
  };
  auto stage = [&](const u32x4 (&w)[8], uint32_t m, int b) {
    if (!active) return;
    u32x4 x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = ((m >> e) & 1u) ? w[e] : u32x4{0u, 0u, 0u, 0u};
    u32x4* dst = sm + b * BUF + (roleL ? 0 : 128 * 8) + 8 * g * 8;  // row 8 g of the L or R part
    u32x4 o[8];
    transpose8x8_b16(x, o);
#pragma unroll
    for (int q = 0; q < 8; ++q) dst[q * 8 + (tg ^ q)] = o[q];
  };

  f32x16 acc[MI][MJ];
#pragma unroll
  for (int a = 0; a < MI; ++a)
#pragma unroll
    for (int b = 0; b < MJ; ++b) acc[a][b] = f32x16{};

  // Rounds of NR chunks, each a straight line of code (so that the compiler
  // counts the loads in flight exactly): register set u holds the chunks
  // c with c % D == u.  Chunks past the block's tokens load clamped rows and
  // are staged as zeros.
  for (int rb = nb; rb < ne; rb += NR * kGramTok) {
    if (tileE) {
#pragma unroll
      for (int u = 0; u < D; ++u) load_tids(tq[u], rb, u);
    }
#pragma unroll
    for (int u = 0; u < D; ++u) load(v[u], mk[u], tq[u], rb, u);
    stage(v[0], mk[0], 0);
    load(v[0], mk[0], tq[0], rb, D);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NR; ++c) {
      const u32x4* Ls = sm + (c & 1) * BUF;
      const u32x4* Rs = Ls + 128 * 8;
#pragma unroll
      for (int ks = 0; ks < kGramTok / 16; ++ks) {
        const int un = (2 * ks + hi) ^ (l32 & 7);
        bf16x8 a[MI], b[MJ];
#pragma unroll
        for (int m = 0; m < MI; ++m) a[m] = __builtin_bit_cast(bf16x8, Ls[(wi * MI * 32 + m * 32 + l32) * 8 + un]);
#pragma unroll
        for (int m = 0; m < MJ; ++m) b[m] = __builtin_bit_cast(bf16x8, Rs[(wj * MJ * 32 + m * 32 + l32) * 8 + un]);
#pragma unroll
        for (int x = 0; x < MI; ++x)
#pragma unroll
          for (int y = 0; y < MJ; ++y) acc[x][y] = mfma_bf16_32x32x16(a[x], b[y], acc[x][y]);
      }
      const int u1 = (c + 1) % D;
      if (c + 1 < NR) stage(v[u1], mk[u1], (c + 1) & 1);
      if (c + 1 + D < NR) load(v[u1], mk[u1], tq[u1], rb, c + 1 + D);
      __syncthreads();
    }
  }

  float* dst = part + size_t(sp) * rows * Rd;
#pragma unroll
  for (int x = 0; x < MI; ++x)
#pragma unroll
    for (int y = 0; y < MJ; ++y)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int i = i0 + wi * MI * 32 + x * 32 + mfma32_row(q, hi);
        if (i < rows) dst[size_t(i) * Rd + j0 + wj * MJ * 32 + y * 32 + l32] = acc[x][y][q];
      }
}

// Token splits: 512 tokens per block (one round of 8 chunks), or one round of
// 10, 12 or 16 chunks (the fewest that do) where 512 would leave a partial
// second wave of blocks on the chip's 256 compute units; at most 64 splits
// (bounds the partials: at most 64 d x r pieces).
constexpr int kGramWideRounds[3] = {10, 12, 16};

int gram_splits_bf16(int N, int rows, int Rd) {
  const int TJ = Rd >= 128 ? 128 : Rd;
  const int tiles = ((rows + 127) / 128) * (Rd / TJ);
  int s = (N + kGramRound - 1) / kGramRound;
  if (tiles * s > 256) {
    for (int nr : kGramWideRounds) {
      const int sw = (N + nr * kGramTok - 1) / (nr * kGramTok);
      if (tiles * sw <= 256) {
        s = sw;
        break;
      }
    }
  }
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  return s;
}

void launch_gram_bf16(const uint16_t* in, int64_t ldin, int Ld, const int32_t* tids, int V, const uint16_t* E,
                      int Le, const uint16_t* R, int Rd, float* part, int N, int splits, hipStream_t s) {
  // tokens per split: one round of 10, 12 or 16 chunks where that covers it, else rounds of 8
  int tps = (N + splits - 1) / splits;
  int nr = 8;
  if (tps > kGramRound) {
    for (int w : kGramWideRounds)
      if (tps <= w * kGramTok) {
        nr = w;
        break;
      }
  }
  tps = (tps + nr * kGramTok - 1) / (nr * kGramTok) * (nr * kGramTok);
  const int TJ = Rd >= 128 ? 128 : Rd;
  const int ti = (Ld + Le + 127) / 128, tj = Rd / TJ;
  const dim3 grid(unsigned(ti * tj * splits));
#define MAPL_GRAM(TJv, NRv)                                                                                         \
  hipLaunchKernelGGL((k_gram2<TJv, NRv>), grid, dim3(256), 0, s, in, ldin, Ld, tids, V, E, Le, R, Rd, part, N, tps, \
                     ti, tj)
#define MAPL_GRAM_NR(NRv)                 \
  if (TJ == 128) MAPL_GRAM(128, NRv);     \
  else if (TJ == 64) MAPL_GRAM(64, NRv);  \
  else MAPL_GRAM(32, NRv);
  if (nr == 10) {
    MAPL_GRAM_NR(10)
  } else if (nr == 12) {
    MAPL_GRAM_NR(12)
  } else if (nr == 16) {
    MAPL_GRAM_NR(16)
  } else {
    MAPL_GRAM_NR(8)
  }
#undef MAPL_GRAM_NR
#undef MAPL_GRAM
}

// ------------------------------------------------------ partial reduction --
// Element e < n0 + n1 of the split sums sum_s part[s * stride + e] goes to
// out0[e] (added to it when acc0) for e < n0, else to out1[e - n0]; the
// splits are added in order, eight loads in flight at a time.
__global__ __launch_bounds__(256) void k_reduce_partials(const float* __restrict__ part, int splits, int64_t stride4,
                                                         float* __restrict__ out0, int64_t n0_4, int acc0,
                                                         float* __restrict__ out1, int64_t n1_4) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= n0_4 + n1_4) return;
  const f32x4* p = reinterpret_cast<const f32x4*>(part) + e;
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < splits; k0 += 8) {
    f32x4 t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = (k0 + u < splits) ? p[size_t(k0 + u) * stride4] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 8; ++u) s += t[u];
  }
  if (e < n0_4) {
    f32x4* o = reinterpret_cast<f32x4*>(out0) + e;
    *o = acc0 ? *o + s : s;
  } else {
    reinterpret_cast<f32x4*>(out1)[e - n0_4] = s;
  }
}

void launch_reduce_partials(const float* part, int splits, int64_t stride, float* out0, int64_t n0, int acc0,
                            float* out1, int64_t n1, hipStream_t s) {
  const int64_t c4 = (n0 + n1) / 4;
  hipLaunchKernelGGL(k_reduce_partials, dim3(unsigned((c4 + 255) / 256)), dim3(256), 0, s, part, splits, stride / 4,
                     out0, n0 / 4, acc0, out1, n1 / 4);
}

// ------------------------------------------------- anchor-term correction --
// gA[i][j] -= sum_k P[k][i] M[k][j]  (P bf16 [ra][d], M fp32 [ra][r], gA fp32 [d][r]).
// One block per 32 x 32 tile of gA; the 4 waves split k and add in LDS.
__global__ __launch_bounds__(256) void k_sub_ptm(const bf16_t* __restrict__ P, const float* __restrict__ M,
                                                 float* __restrict__ gA, int d, int r, int ra) {
  __shared__ float red[4 * 1024];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int hi = lane >> 5, l32 = lane & 31;
  const int i0 = blockIdx.x * 32, j0 = blockIdx.y * 32;
  const int kq = ra >> 2;  // ra % 32 == 0: a multiple of 8
  const int kb = wave * kq, ke = kb + kq;
  const int i = threadIdx.x >> 3, j = (threadIdx.x & 7) * 4;
  f32x4* o = reinterpret_cast<f32x4*>(gA + size_t(i0 + i) * r + j0 + j);
  const f32x4 g0 = *o;  // issued with the operands' loads, not after the products
  f32x16 acc = f32x16{};
  // 32 values of k per batch, all loads issued before the batch's multiplies
  for (int kc = kb; kc < ke; kc += 32) {
    float a[16], b[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int k = min(kc + 2 * t + hi, ke - 1);
      a[t] = bf2f(P[size_t(k) * d + i0 + l32]);
      b[t] = M[size_t(k) * r + j0 + l32];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 16; ++t)
      if (kc + 2 * t < ke) acc = mfma_f32_32x32x2(a[t], b[t], acc);
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) red[wave * 1024 + v * 64 + lane] = acc[v];
  __syncthreads();
  const int fi = ((((i >> 3) << 2) | (i & 3)) << 6) + (((i >> 2) & 1) << 5) + j;
  const f32x4* r4 = reinterpret_cast<const f32x4*>(red);
  const f32x4 sum = (r4[fi / 4] + r4[(1024 + fi) / 4]) + (r4[(2048 + fi) / 4] + r4[(3072 + fi) / 4]);
  *o = g0 - sum;
}

// gA -= M elementwise (the identity anchor projector), 4 values per thread
__global__ __launch_bounds__(256) void k_sub_m(const f32x4* __restrict__ M, f32x4* __restrict__ gA, int64_t n4) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e < n4) gA[e] = gA[e] - M[e];
}

void launch_sub_ptm(const uint16_t* P, const float* M, float* gA, int d, int r, int ra, hipStream_t s) {
  if (P == nullptr) {
    const int64_t n4 = int64_t(d) * r / 4;
    hipLaunchKernelGGL(k_sub_m, dim3(unsigned((n4 + 255) / 256)), dim3(256), 0, s, reinterpret_cast<const f32x4*>(M),
                       reinterpret_cast<f32x4*>(gA), n4);
    return;
  }
  hipLaunchKernelGGL(k_sub_ptm, dim3(d / 32, r / 32), dim3(256), 0, s, P, M, gA, d, r, ra);
}

}  // namespace mapl
