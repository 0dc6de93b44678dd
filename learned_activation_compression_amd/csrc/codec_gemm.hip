// Token GEMM for the bf16 codec maps on the gfx950 matrix cores.
//
// Source of the maps: "Learned Subspace Compression for Communication-
// Efficient Pipeline Parallelism", Section 3.2, Eq. (1) Z = (X - E[t] P) A,
// Eq. (2) Xhat = Z A^T + E'[t] P', Eq. (3) factorised anchor; the backward
// maps gZ = gXhat A and gX = gZ A^T are their adjoints.
//
// All four are one product with a token-indexed left operand:
//   out[n][c] = sum_k T[n][k] W[k][c],   T[n] = [src[n] (K1 values) | E[t_n] (K2 values)]
// with W given as two fragment-ordered packs (F1 for k < K1, F2 for the
// anchor rows; see pack.hip):
//   compress      src = X,     K1 = d, K2 = r, F1 = AtF, F2 = QnF, C = r
//   gZ            src = gXhat, K1 = d, K2 = 0, F1 = AtF,           C = r
//   reconstruct   src = Z,     K1 = r, K2 = r, F1 = AF,  F2 = PtF, C = d
//   gX            src = gZ,    K1 = r, K2 = 0, F1 = AF,            C = d
// An id outside [0, V) gives a zero anchor row.
//
// The full-rank anchor (P = I, E [V][C]) adds E[t_n] to the output rows
// instead of contracting against an identity pack: reconstruct with K2 = 0
// and the rows E[t] added in fp32 in the epilogue (EADD), one rounding to
// bf16 as in the contracted form.
//
// Block: TC output columns x TT tokens, 4 waves as 2 x 2, each wave a
// (TC/2) x (TT/2) tile of 32 x 32 accumulators (columns = matrix-core rows,
// tokens = matrix-core columns): 256 x 256 with two ring slots where that
// still fills the chip (the accumulators take all 256 AGPRs), else 256 x 128
// or 128 x 128 with three or four.  The contraction runs in chunks of 64: the
// chunk's weight fragments (TC/32 row blocks x 4 K-steps, 1 KB each) and its
// TT token-row segments of 128 bytes are copied with global_load_lds straight
// into slot c % S of an LDS ring, S - 1 chunks ahead.  Token row t keeps its
// 8 units at positions u ^ (t & 7) (the copy chooses its source unit per
// lane), so the operand reads of 32 rows hit distinct bank groups.  Per chunk
// each wave waits for its own copies (vmcnt), a barrier publishes everyone's
// and frees chunk c - 1's slot for chunk c + S - 1.  The output tile goes
// back through the ring (16-byte unit u of token row t at u ^ (t & 31)) and
// out as whole 16-byte row segments.
#include "common.h"
#include "internal.h"

namespace mapl {

namespace {

constexpr int kKC = 64;  // contraction values per chunk

template <int TC, int TT, int S>
struct GemmRing {
  static constexpr int WU = (TC / 32) * 4 * 64;  // weight units (16 B) per slot
  static constexpr int TU = TT * 8;              // token-row units per slot
  static constexpr int SLOT = WU + TU;
  static constexpr int PER = (WU + TU) / 64 / 4;  // copies (1 KB each) per wave per chunk
  static constexpr size_t RING = size_t(S) * SLOT * 16;
  static constexpr size_t OUT = size_t(TC) * TT * 2;  // staged output tile (bf16)
  static constexpr size_t OUT32 = size_t(TC) * TT * 4;  // ... fp32, for the anchor-row epilogue
  static constexpr size_t BYTES = RING > OUT ? RING : OUT;

  static_assert((WU + TU) % 256 == 0, "copies must split evenly over the 4 waves");
};

template <int TC, int TT, int S, bool ANCHOR, bool EADD = false>
__global__ __launch_bounds__(256) void k_tok_gemm(const bf16_t* __restrict__ src, int K1,
                                                  const int32_t* __restrict__ tids, int V,
                                                  const bf16_t* __restrict__ E, int K2,
                                                  const bf16_t* __restrict__ F1, const bf16_t* __restrict__ F2,
                                                  bf16_t* __restrict__ out, int N, int C, int ntc) {
  using GR = GemmRing<TC, TT, S>;
  constexpr int MI = TC / 64, NJ = TT / 64;  // 32 x 32 blocks per wave
  extern __shared__ __attribute__((aligned(16))) u32x4 ring[];
  const int lane = threadIdx.x & 63, w = wave_id();
  const int hi = lane >> 5, l32 = lane & 31;
  const int wi = w >> 1, wj = w & 1;
  const int bid = xcd_swizzle(blockIdx.x, int(gridDim.x));
  const int tc = bid % ntc, tt = bid / ntc;  // the column tiles of one token tile are adjacent
  const int c0 = tc * TC, n0 = tt * TT;
  const int MB = C >> 5;                     // row blocks per K-step in the packs
  const int cx = K1 / kKC, nch = cx + (ANCHOR ? K2 / kKC : 0);

  // copy plan of this wave: units [w * PER, (w + 1) * PER) of a slot, in 1 KB pieces
  // (first the weight fragments, then token rows 8 at a time)
  const int cu = (lane & 7) ^ (lane >> 3);  // source unit of this lane in an 8-row token piece
  // element offsets of this lane's token rows for each token piece it copies
  constexpr int TP = TT / 8;                 // token pieces (8 rows) per chunk, a multiple of 4
  static_assert(TP % 4 == 0, "token pieces split evenly over the 4 waves");
  size_t soff[TP / 4], eoff[TP / 4];
#pragma unroll
  for (int q = 0; q < TP / 4; ++q) {
    const int piece = w + 4 * q;             // token piece handled by this wave
    const int tk = min(n0 + 8 * piece + (lane >> 3), N - 1);
    soff[q] = size_t(tk) * K1 + 8 * cu;
    eoff[q] = 8 * cu;
    if (ANCHOR) {
      const int t = tids[tk];
      eoff[q] += size_t((t >= 0 && t < V) ? t : 0) * K2;
    }
  }
  // operand masks: token column nb*32 + l32 with an invalid id reads a zero anchor row
  uint32_t bm[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    bm[j] = ~0u;
    if (ANCHOR) {
      const int t = tids[min(n0 + (wj * NJ + j) * 32 + l32, N - 1)];
      bm[j] = (t >= 0 && t < V) ? ~0u : 0u;
    }
  }
  if (ANCHOR) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) asm volatile("" : : "v"(bm[j]));  // resolve the ids before the first copy
  }

  // Blocks start at different chunks (rot), so that the blocks running at the
  // same time read different weight fragments rather than all the same L2 lines.
  const int rot = tt % nch;
  auto chunk_of = [&](int c) { return c + rot < nch ? c + rot : c + rot - nch; };
  auto issue = [&](int c) {
    u32x4* slot = ring + (c % S) * GR::SLOT;
    c = chunk_of(min(c, nch - 1));  // past the end: copy the last chunk again into a slot never read
    const bool xs = c < cx;
    const int kc = xs ? c : c - cx;
    // weight fragments: TC/32 row blocks x 4 K-steps
    const bf16_t* fb = (xs ? F1 : F2) + (size_t(4 * kc) * MB + c0 / 32) * 512;
#pragma unroll
    for (int q = 0; q < GR::WU / 256; ++q) {
      const int piece = w + 4 * q;           // (ks, mb) = (piece / (TC/32), piece % (TC/32))
      const int ks = piece / (TC / 32), mb = piece % (TC / 32);
      copy16_to_lds(fb + (size_t(ks) * MB + mb) * 512 + lane * 8, slot + piece * 64);
    }
    // token rows: TP pieces of 8 rows x 128 bytes
#pragma unroll
    for (int q = 0; q < TP / 4; ++q) {
      const bf16_t* p = xs ? src + soff[q] + kc * kKC : E + eoff[q] + kc * kKC;
      copy16_to_lds(p, slot + GR::WU + (w + 4 * q) * 64);
    }
  };

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};

#pragma unroll
  for (int u = 0; u < S - 1; ++u) issue(u);
  for (int c = 0; c < nch; ++c) {
    wait_vmcnt<(S - 2) * GR::PER>();  // this wave's copies of chunk c are done
    __syncthreads();                   // everyone's are; chunk c - 1's slot is free
    issue(c + S - 1);
    const u32x4* slot = ring + (c % S) * GR::SLOT;
    const bool anchor = ANCHOR && chunk_of(c) >= cx;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 a[MI], b[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i)
        a[i] = __builtin_bit_cast(bf16x8, slot[(ks * (TC / 32) + wi * MI + i) * 64 + lane]);
      const int pu = (2 * ks + hi) ^ (l32 & 7);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        b[j] = __builtin_bit_cast(bf16x8, slot[GR::WU + ((wj * NJ + j) * 32 + l32) * 8 + pu]);
        if (ANCHOR) b[j] = mask_bf16x8(b[j], anchor ? bm[j] : ~0u);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = mfma_bf16_32x32x16(a[i], b[j], acc[i][j]);
    }
  }
  wait_vmcnt<0>();  // no copy may still be writing the ring
  __syncthreads();

  if (EADD) {
    static_assert(!EADD || GR::RING >= GR::OUT32, "the fp32 output tile must fit the ring");
    // stage the tile as fp32 rows [token][TC columns] (16-byte unit u of row t at
    // u ^ (t & 31)), then out[n] = bf16(tile[n] + E[t_n]) with 16-byte loads and stores
    constexpr int RU4 = TC / 4;  // 16-byte fp32 units per staged row
    f32x4* st4 = reinterpret_cast<f32x4*>(ring);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int t = (wj * NJ + j) * 32 + l32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int u = ((wi * MI + i) * 32 + 8 * q) / 4 + hi;  // columns 4u .. 4u + 3
          const f32x16& a = acc[i][j];
          st4[t * RU4 + (u ^ (t & 31))] = f32x4{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
        }
      }
    __syncthreads();
    constexpr int RU = TC / 8;  // 16-byte bf16 units per output row
    for (int e = threadIdx.x; e < TT * RU; e += 256) {
      const int t = e / RU, p = e % RU;
      const int n = n0 + t;
      if (n >= N) continue;
      const int id = tids[n];
      u32x4 ev = u32x4{0u, 0u, 0u, 0u};
      if (id >= 0 && id < V) ev = *reinterpret_cast<const u32x4*>(E + size_t(id) * C + c0 + 8 * p);
      const f32x4 lo = st4[t * RU4 + ((2 * p) ^ (t & 31))];
      const f32x4 hi4 = st4[t * RU4 + ((2 * p + 1) ^ (t & 31))];
      u32x4 o;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4 v = h ? hi4 : lo;
        o[2 * h] = pack2bf(v[0] + bf2f(uint16_t(ev[2 * h] & 0xffffu)), v[1] + bf2f(uint16_t(ev[2 * h] >> 16)));
        o[2 * h + 1] =
            pack2bf(v[2] + bf2f(uint16_t(ev[2 * h + 1] & 0xffffu)), v[3] + bf2f(uint16_t(ev[2 * h + 1] >> 16)));
      }
      *reinterpret_cast<u32x4*>(out + size_t(n) * C + c0 + 8 * p) = o;
    }
    return;
  }

  // stage the tile as bf16 rows [token][TC columns]: lane holds, for token
  // column l32 of block j, 4 consecutive output columns per register group
  constexpr int RU = TC / 8;  // 16-byte units per staged row
  uint32_t* st = reinterpret_cast<uint32_t*>(ring);
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int t = (wj * NJ + j) * 32 + l32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = (wi * MI + i) * 32 + 8 * q;  // + 4 hi: first of the 4 columns
        const int u = col / 8;
        const int pos = t * RU + (u ^ (t & (RU - 1) & 31));
        const f32x16& a = acc[i][j];
        *reinterpret_cast<u32x2*>(st + pos * 4 + 2 * hi) =
            u32x2{pack2bf(a[4 * q], a[4 * q + 1]), pack2bf(a[4 * q + 2], a[4 * q + 3])};
      }
    }
  __syncthreads();
  for (int e = threadIdx.x; e < TT * RU; e += 256) {
    const int t = e / RU, p = e % RU;
    const int n = n0 + t;
    if (n >= N) continue;
    const int u = p ^ (t & (RU - 1) & 31);
    *reinterpret_cast<u32x4*>(out + size_t(n) * C + c0 + 8 * u) = ring[e];
  }
}

template <int TC, int TT, int S, bool ANCHOR, bool EADD = false>
void launch_gemm(const uint16_t* src, int K1, const int32_t* tids, int V, const uint16_t* E, int K2,
                 const uint16_t* F1, const uint16_t* F2, uint16_t* out, int N, int C, hipStream_t s) {
  auto k = k_tok_gemm<TC, TT, S, ANCHOR, EADD>;
  const int lds = LdsLimit<k_tok_gemm<TC, TT, S, ANCHOR, EADD>, int(GemmRing<TC, TT, S>::BYTES)>::bytes();
  const int ntc = C / TC, ntt = (N + TT - 1) / TT;
  hipLaunchKernelGGL(k, dim3(unsigned(ntc * ntt)), dim3(256), lds, s, src, K1, tids, V, E, K2, F1, F2, out, N, C, ntc);
}

}  // namespace

// out[N][C] = [src | E[t]] W; see the top of this file.  Requires K1 and K2
// multiples of 64 and C a multiple of the column tile (128 or 256).
bool launch_tok_gemm_bf16(const uint16_t* src, int K1, const int32_t* tids, int V, const uint16_t* E, int K2,
                          const uint16_t* F1, const uint16_t* F2, uint16_t* out, int N, int C, hipStream_t s) {
  const bool anc = E != nullptr && K2 > 0;
  if (K1 % kKC != 0 || (anc && K2 % kKC != 0)) return false;
  // 256 x 256 tiles (two 64 KB slots, 128 x 128 per wave) where they still give
  // every compute unit a block: fewer LDS bytes per matrix-core operation
  if (C % 256 == 0 && int64_t(C / 256) * ((N + 255) / 256) >= 256) {
    if (anc) launch_gemm<256, 256, 2, true>(src, K1, tids, V, E, K2, F1, F2, out, N, C, s);
    else launch_gemm<256, 256, 2, false>(src, K1, tids, V, E, K2, F1, F2, out, N, C, s);
    return true;
  }
  if (C % 256 == 0) {
    if (anc) launch_gemm<256, 128, 3, true>(src, K1, tids, V, E, K2, F1, F2, out, N, C, s);
    else launch_gemm<256, 128, 3, false>(src, K1, tids, V, E, K2, F1, F2, out, N, C, s);
    return true;
  }
  if (C % 128 == 0) {
    if (anc) launch_gemm<128, 128, 4, true>(src, K1, tids, V, E, K2, F1, F2, out, N, C, s);
    else launch_gemm<128, 128, 4, false>(src, K1, tids, V, E, K2, F1, F2, out, N, C, s);
    return true;
  }
  return false;
}

// out[N][C] = src[N][K1] W + E[t] (E [V][C]: the full-rank anchor rows, P = I).
bool launch_tok_gemm_eadd_bf16(const uint16_t* src, int K1, const int32_t* tids, int V, const uint16_t* E,
                               const uint16_t* F1, uint16_t* out, int N, int C, hipStream_t s) {
  if (K1 % kKC != 0) return false;
  if (C % 256 == 0) {
    launch_gemm<256, 128, 3, false, true>(src, K1, tids, V, E, 0, F1, nullptr, out, N, C, s);
    return true;
  }
  if (C % 128 == 0) {
    launch_gemm<128, 128, 4, false, true>(src, K1, tids, V, E, 0, F1, nullptr, out, N, C, s);
    return true;
  }
  return false;
}

}  // namespace mapl
