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
// The problem is small (a few MB) and the iteration is a chain of dependent
// products, so every kernel is built for latency: all operand loads of a wave
// are in flight before its first matrix-core instruction, and no launch
// exists only to reduce.
//
//   gram  part[q] = sum over row group q of Xl^T Xr (r x r, both triangles).
//         One block per (upper-triangle pair of 32 x 32 column blocks, row
//         group); its 4 waves sum in LDS.  For Eq. (4) the block stores
//         sym(.) of its piece (sym is linear, so the pieces add up to
//         sym(A^T g)).
//   xm    out = s X M  d x r with M = f(sum_q part[q]): f = identity for
//         Eq. (4), 1.5 I - 0.5 s^2 (.) for a Newton-Schulz step.  One block
//         per 32 x 32 output tile; the block first forms its 32 columns of M
//         in LDS (coalesced row reads, the pieces added in order), then the 4
//         waves split K = r and sum in LDS; the epilogue applies Eq. (4)-(5),
//         a plain Newton-Schulz step, or the last step of Eq. (6) / Eq. (7).
//
// All sums run in a fixed order, so a step is bitwise repeatable.  The scale
// s = 1/||m||_F comes from per-block partial sums of squares written by the
// momentum epilogue, added up in a fixed order by the one launch that uses it.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <utility>

#include "common.h"
#include "internal.h"

namespace mapl {

namespace {

enum { XM_TANGENT = 0, XM_NS = 1, XM_NS_LAST_LMO = 2, XM_NS_LAST_RET = 3 };

typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kChunk = 32;  // rows per wave per Gram chunk (16 matrix-core K-steps)

// Position of element (i, j) of a 32 x 32 tile in the accumulator fragment
// order [v][lane] of v_mfma_f32_32x32x2_f32 (lane = 32 h + j holds row
// 8 (v >> 2) + 4 h + (v & 3)).
__device__ __forceinline__ int frag_index(int i, int j) {
  return (((i >> 3) << 2 | (i & 3)) << 6) + (((i >> 2) & 1) << 5) + j;
}

__device__ __forceinline__ void store_frag(float* dst, const f32x16& acc, int lane) {
#pragma unroll
  for (int v = 0; v < 16; ++v) dst[v * 64 + lane] = acc[v];
}

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

// Upper-triangle pair index -> (bi, bj), bi <= bj, row-major.
__device__ __forceinline__ void pair_of(int p, int nb, int& bi, int& bj) {
  bi = 0;
  int rem = p;
  while (rem >= nb - bi) {
    rem -= nb - bi;
    ++bi;
  }
  bj = bi + rem;
}

// TWO = 1 (Eq. (4)): piece = sym(A^T g) over the group's rows, from
// acc1 = A_bi^T g_bj and acc2 = A_bj^T g_bi.  TWO = 0: piece = X_bi^T X_bj.
// Tile (bi, bj) of part[grp] gets the piece, tile (bj, bi) its transpose.
// `zero`, when given, holds nzero words cleared for the launches that follow:
// the progress counters and the timeout word of the Gram-space iteration, and
// (cleared by the step's first launch only) the step's sticky timeout word,
// which decides at the end whether the step is committed.  Each of the 256
// counters has a 64-byte line of its own (word 16 i): every workgroup of the
// iteration polls all of them, and polls of one shared line queue up behind
// each other.
constexpr int kRsFlagWords = 256;
constexpr int kRsFlagStride = 16;
constexpr int kRsTimeoutWord = kRsFlagWords * kRsFlagStride, kRsStickyWord = kRsTimeoutWord + 1;
constexpr int kRsSyncWords = kRsTimeoutWord + 4;
template <int TWO>
__global__ __launch_bounds__(256) void k_spel_gram(const float* __restrict__ Xl, const float* __restrict__ Xr,
                                                   float* __restrict__ part, int d, int r, int groups,
                                                   unsigned* __restrict__ zero, int nzero) {
  __shared__ float red[(1 + TWO) * 4 * 1024];
  __shared__ float tile[32 * 33];
  const int lane = threadIdx.x & 63, w = wave_id();
  if (zero != nullptr)
    for (int i = blockIdx.x * 256 + threadIdx.x; i < nzero; i += gridDim.x * 256) zero[i] = 0u;
  const int h = lane >> 5, l32 = lane & 31;
  const int p = blockIdx.x / groups, grp = blockIdx.x % groups;
  int bi, bj;
  pair_of(p, r >> 5, bi, bj);
  const bool two = TWO && bi != bj;

  f32x16 acc1 = f32x16{}, acc2 = f32x16{};
  for (int c = grp * 4 + w; c * kChunk < d; c += groups * 4) {
    const int k0 = c * kChunk;
    float a[kChunk / 2], b[kChunk / 2], a2[kChunk / 2], b2[kChunk / 2];
#pragma unroll
    for (int t = 0; t < kChunk / 2; ++t) {
      const size_t row = size_t(k0 + 2 * t + h) * r;
      a[t] = Xl[row + bi * 32 + l32];
      b[t] = Xr[row + bj * 32 + l32];
      if (two) {
        a2[t] = Xl[row + bj * 32 + l32];
        b2[t] = Xr[row + bi * 32 + l32];
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the first multiply
#pragma unroll
    for (int t = 0; t < kChunk / 2; ++t) acc1 = mfma_f32_32x32x2(a[t], b[t], acc1);
    if (two) {
#pragma unroll
      for (int t = 0; t < kChunk / 2; ++t) acc2 = mfma_f32_32x32x2(a2[t], b2[t], acc2);
    }
  }

  // the block's 4 waves in a fixed order
  store_frag(red + w * 1024, acc1, lane);
  if (TWO) store_frag(red + 4096 + w * 1024, acc2, lane);
  __syncthreads();
  const int i = threadIdx.x >> 3, j = (threadIdx.x & 7) * 4;
  const int fi = frag_index(i, j);
  f32x4 s1 = (ld4(red + fi) + ld4(red + 1024 + fi)) + (ld4(red + 2048 + fi) + ld4(red + 3072 + fi));
  if (TWO) {
    // sym: (G1_ij + G2_ji) / 2 off the diagonal, (G1_ij + G1_ji) / 2 on it
    const f32x4 s2 = (ld4(red + 4096 + fi) + ld4(red + 5120 + fi)) + (ld4(red + 6144 + fi) + ld4(red + 7168 + fi));
    const f32x4 tt = (bi != bj) ? s2 : s1;
#pragma unroll
    for (int q = 0; q < 4; ++q) tile[i * 33 + j + q] = tt[q];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) s1[q] = 0.5f * (s1[q] + tile[(j + q) * 33 + i]);
  }
  float* dst = part + size_t(grp) * r * r;
  st4(dst + size_t(bi * 32 + i) * r + bj * 32 + j, s1);
  if (bi != bj) {
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[size_t(bj * 32 + j + q) * r + bi * 32 + i] = s1[q];
  }
}

// acc += X[row][kc .. kc+CH) * M[kc .. kc+CH)[col] on the 32x32x2 matrix core,
// with M's column col already formed in LDS (Mt: row c of the block's slab holds
// column j0 + c of M).  At step t lane half h takes k = kc + (CH/2) h + t, so
// each lane reads CH/2 consecutive floats of its X row and of its M column as
// 16-byte loads; all of them are issued before the first multiply.
template <int CH>
__device__ __forceinline__ void xm_chunk(const float* __restrict__ xr, const float* mcol, int kc, int h,
                                         f32x16& acc) {
  constexpr int HK = CH / 2;
  f32x4 xa[HK / 4], mb[HK / 4];
  const float* xk = xr + kc + HK * h;
  const float* mk = mcol + kc + HK * h;
#pragma unroll
  for (int q = 0; q < HK / 4; ++q) xa[q] = ld4(xk + 4 * q);
#pragma unroll
  for (int q = 0; q < HK / 4; ++q) mb[q] = ld4(mk + 4 * q);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < HK; ++t) acc = mfma_f32_32x32x2(xa[t >> 2][t & 3], mb[t >> 2][t & 3], acc);
}

// 1/||m||_F from n per-block partial sums, added in a fixed order by wave 0
// and broadcast through LDS (0 when m == 0).
__device__ float block_inv_norm(const float* nparts, int n, float* slot) {
  if (wave_id() == 0) {
    const int lane = threadIdx.x & 63;
    float s = 0.f;
    for (int b0 = 0; b0 < n; b0 += 64) s += (b0 + lane < n) ? nparts[b0 + lane] : 0.f;
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) *slot = s > 0.f ? 1.f / sqrtf(s) : 0.f;
  }
  __syncthreads();
  return *slot;
}

// out = s X M for one 32 x 32 tile (block (row tile, col tile)); wave w takes
// K range [w r/4, (w+1) r/4) (r % 32 == 0, so each range is a multiple of 8).
template <int G, bool NS>
__global__ __launch_bounds__(256) void k_spel_xm(const float* __restrict__ X, const float* __restrict__ nparts_in,
                                                 const float* __restrict__ part, float* __restrict__ out, int d, int r,
                                                 int mode, const float* __restrict__ g, const float* __restrict__ m,
                                                 float beta, float* __restrict__ nparts_out,
                                                 const float* __restrict__ Acur, float alpha, float* __restrict__ Dout,
                                                 float* __restrict__ Y0, const unsigned* __restrict__ sticky,
                                                 const float* __restrict__ mnew, float* __restrict__ mcommit,
                                                 int* __restrict__ status) {
  extern __shared__ __attribute__((aligned(16))) float xm_lds[];  // the M slab; then the wave partials
  float* red = xm_lds;
  __shared__ float wsum[4];
  __shared__ float scs;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int h = lane >> 5, l32 = lane & 31;
  const int i0 = blockIdx.x * 32, j0 = blockIdx.y * 32;
  const float sx = nparts_in ? block_inv_norm(nparts_in, (d >> 5) * (r >> 5), &scs) : 1.f;
  const float sc2 = sx * sx;
  const size_t rr = size_t(r) * r;
  const int mp = r + 4;  // LDS pitch of a slab row (one column of M)

  // the block's 32 columns of M = f(sum of the G pieces), formed once: thread t reads
  // 4 consecutive columns of row k (coalesced 16-byte loads, 8 threads per row segment),
  // adds the pieces in order and stores the 4 values down the slab's rows
  for (int k0 = 0; k0 < r; k0 += 32) {
    const int k = k0 + int(threadIdx.x >> 3), c4 = int(threadIdx.x & 7) * 4;
    const float* src = part + size_t(k) * r + j0 + c4;
    f32x4 sum = ld4(src);
#pragma unroll
    for (int gq = 1; gq < G; ++gq) sum += ld4(src + gq * rr);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = NS ? ((k == j0 + c4 + e) ? 1.5f : 0.f) - 0.5f * (sc2 * sum[e]) : sum[e];
      xm_lds[(c4 + e) * mp + k] = v;
    }
  }
  __syncthreads();

  f32x16 acc = f32x16{};
  {
    const float* xr = X + size_t(i0 + l32) * r;
    const float* mcol = xm_lds + l32 * mp;
    const int kq = r >> 2;
    int kc = w * kq;
    const int ke = kc + kq;
    for (; kc + 64 <= ke; kc += 64) xm_chunk<64>(xr, mcol, kc, h, acc);
    if (kc + 32 <= ke) {
      xm_chunk<32>(xr, mcol, kc, h, acc);
      kc += 32;
    }
    if (kc + 16 <= ke) {
      xm_chunk<16>(xr, mcol, kc, h, acc);
      kc += 16;
    }
    if (kc + 8 <= ke) xm_chunk<8>(xr, mcol, kc, h, acc);
  }
  __syncthreads();  // the slab is read: its LDS takes the wave partials
  store_frag(red + w * 1024, acc, lane);
  __syncthreads();
  const int i = threadIdx.x >> 3, j = (threadIdx.x & 7) * 4;
  const int fi = frag_index(i, j);
  const f32x4 v = (ld4(red + fi) + ld4(red + 1024 + fi)) + (ld4(red + 2048 + fi) + ld4(red + 3072 + fi));
  const size_t o = size_t(i0 + i) * r + j0 + j;

  if (mode == XM_TANGENT) {
    // Eq. (4)-(5): g_R = g - A sym(A^T g) ; m_new = beta m + (1 - beta) g_R, into `out`
    // (the caller's m is updated only when the step commits)
    const f32x4 gv = ld4(g + o), mv = ld4(m + o);
    f32x4 mn;
    float local = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      mn[q] = beta * mv[q] + (1.f - beta) * (gv[q] - v[q]);
      local = fmaf(mn[q], mn[q], local);
    }
    st4(out + o, mn);
    // this block's share of ||m||_F^2: xor-butterfly within the wave, waves in order
    for (int off = 32; off > 0; off >>= 1) local += __shfl_xor(local, off);
    if (lane == 0) wsum[w] = local;
    __syncthreads();
    if (threadIdx.x == 0)
      nparts_out[blockIdx.y * gridDim.x + blockIdx.x] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    return;
  }
  const f32x4 val = v * sx;
  if (mode == XM_NS) {
    st4(out + o, val);
  } else if (mode == XM_NS_LAST_RET) {
    // commit: the new A and m, unless a wait of the Gram-space iteration timed out
    const bool ok = sticky == nullptr || *sticky == 0u;
    if (ok) {
      st4(out + o, val);
      st4(mcommit + o, ld4(mnew + o));
    }
    if (status != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *status = ok ? 0 : 1;
  } else {  // XM_NS_LAST_LMO: D = val ; Y0 = A - alpha D
    if (Dout) st4(Dout + o, val);
    const f32x4 y0 = ld4(Acur + o) - alpha * val;
    st4(Y0 + o, y0);
    if (nparts_out) {  // this block's share of ||Y0||_F^2, as for m above
      float local = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) local = fmaf(y0[q], y0[q], local);
      for (int off = 32; off > 0; off >>= 1) local += __shfl_xor(local, off);
      if (lane == 0) wsum[w] = local;
      __syncthreads();
      if (threadIdx.x == 0)
        nparts_out[blockIdx.y * gridDim.x + blockIdx.x] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    }
  }
}

// ------------------------------------------------ Gram-space Newton-Schulz --
// For X = s X0 (d x r, d >= r) every cubic Newton-Schulz iterate is X times a
// polynomial in S_0 = X^T X: X_k = X Q_k with Q_0 = I and, with
// S_k = X_k^T X_k and T_k = 1.5 I - 0.5 S_k,
//   Q_{k+1} = Q_k T_k = 1.5 Q_k - 0.5 Q_k S_k,
//   S_{k+1} = T_k S_k T_k = 2.25 S_k - 1.5 S_k^2 + 0.25 S_k^3
// (all are polynomials in S_0, so they commute).  After n steps
// NS_n(X0) = X0 (s Q_n): one Gram, n steps on r x r matrices and one product,
// in place of n Grams and n products on d x r matrices.
//
// Two steps per exchange.  Since S_{k+1} = h(S_k) with
// h(x) = 2.25 x - 1.5 x^2 + 0.25 x^3, rows of S_{k+1}, S_{k+1}^2 = S_{k+1} h(S_k)
// and S_{k+1}^3 = S_{k+1}^2 h(S_k), hence of S_{k+2}, are all rows times
// powers of S_k: each "times h(S_k)" is three products with right factor S_k
// (Horner), so S_{k+2} takes 8 products and only even S_k are ever
// exchanged.  Likewise Q_{k+2} = B (1.5 I - 0.5 h(S_k)) with B = Q_k T_k
// (4 products), and an odd step count ends with one plain step on the last
// even S_k.
//
// One launch of workgroups of 2 r threads, each owning RHO rows (one for
// r <= 128, two above): S workgroup J rows J RHO .. of the even S_k, Q
// workgroup J the same rows of the Q_k.  Only the S_k chain is sequential: the
// S workgroups wait for each other and never for the Q workgroups, which follow
// the chain one exchanged S_k at a time and hold nothing back but a buffer
// (the exchanged S_k live in a ring of kRsRing buffers; a slot is written
// again only after every Q workgroup has read what it held).
//
// Products on the vector ALUs.  Lane l of wave w owns CPT columns from
// c0 = 32 w + CPT (l / KS) and the contraction part q = l % KS, k in
// [q r/KS, (q+1) r/KS): r <= 128 two columns and lane quads (KS = 4), above
// four columns and lane octets (KS = 8).  Every thread keeps its entries of the
// exchanged S_k in registers for the exchange's products (r <= 128: copied
// into LDS first with coalesced 16-byte device-coherent loads; above, r x r no
// longer fits LDS and each thread loads its own), so a product reads only its
// left rows from LDS (16-byte reads, one address per lane group) and adds the
// contraction parts across the group with DPP (every lane of the group ends
// with the same sum).  Few rows per workgroup keep the chain of products
// between exchanges short: at r = 128 a product is 64 fused multiply-adds per
// thread, where 4 rows on v_mfma_f32_4x4x1_16b_f32 (half the matrix core's
// rate) took as long as 4 rows on the vector ALUs.
//
// Exchange.  Each workgroup owns a progress counter: an S workgroup's is the
// number of S_k whose rows it has stored, a Q workgroup's the number of S_k it
// has read.  The S_k travel as device-coherent loads and stores (the sc1
// cache policy: they bypass the per-XCD caches that the device's other XCDs
// do not see) and the counters as device-scope atomics, so no cache-wide
// write-back or invalidate is needed: a workgroup's stores are complete
// (s_waitcnt) before its counter moves, and a reader loads S_k only after it
// has seen every counter it needs.  A wait that exceeds its bound (a second or
// two) sets the timeout word, and the Q workgroups then write NaN: a wrong
// result is never silent and no wait is endless.  The launch is ordinary; its
// workgroups (256 at r = 128 and r = 256) must be resident together, which the
// host checks against the device's compute units and the kernel's occupancy
// before it takes this form.
//
// each spin is a sleep and an uncached load: 2^20 spins take about 1-2 s.  The
// environment variable MAPL_SPEL_SPIN_LIMIT lowers the bound, for tests of the
// timeout path.
constexpr unsigned kRsSpinLimit = 1u << 20;

constexpr int kRsRing = 4;  // S_k buffers

// Device-coherent (sc1) accesses through a buffer resource: the compiler
// tracks them like its own loads and stores.  Offsets in bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rs_rsrc(const float* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), 0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ f32x4 rs_ld(__amdgpu_buffer_rsrc_t rs, int off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 16));
}

// Move this workgroup's progress counter to `val` once every wave's stores are
// complete.
__device__ __forceinline__ void rs_publish(unsigned* flags, int idx, unsigned val) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(flags + kRsFlagStride * idx, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait (one wave polls) until counters [0, ns) are >= sneed and counters
// [ns, ns + nq) are >= qneed.  On timeout the iteration's timeout word and
// the step's sticky word are set and false is returned.
__device__ bool rs_wait(unsigned* flags, int ns, unsigned sneed, int nq, unsigned qneed, unsigned limit, int* slot) {
  if (threadIdx.x < 64) {
    const int l = threadIdx.x;
    unsigned spins = 0;
    int ok = 1;
    for (;;) {
      bool done = true;
      for (int i = l; i < ns + nq; i += 64) {
        const unsigned v = __hip_atomic_load(flags + kRsFlagStride * i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        done = done && v >= (i < ns ? sneed : qneed);
      }
      if (__all(done)) break;
      __builtin_amdgcn_s_sleep(1);
      if (++spins > limit) {
        ok = 0;
        if (l == 0) {
          __hip_atomic_store(flags + kRsTimeoutWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(flags + kRsStickyWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        break;
      }
    }
    if (l == 0) *slot = ok;
  }
  __syncthreads();
  const bool ok = *slot != 0;
  __syncthreads();  // every wave has read the slot before it is written again
  return ok;
}

// LDS position of row i of a staged S_k: pitch R + 4, and 8 more floats
// between row quarters, so that the four lanes of a quad (rows R/4 apart, the
// same columns) read different banks
template <int R>
__device__ __forceinline__ int rs_row(int i) {
  return i * (R + 4) + (i / (R / 4)) * 8;
}
template <int R>
constexpr int kRsStageFloats = R * (R + 4) + 32;

// S [R][R] (ring slot, row-major) -> LDS rows at rs_row, every thread's
// 16-byte loads issued before the first is stored (consecutive threads read
// consecutive 16 bytes)
template <int R, int NT>
__device__ __forceinline__ void rs_stage(__amdgpu_buffer_rsrc_t rs, int base, float* __restrict__ sh) {
  constexpr int U = R / 4, TOTAL = R * U, PER = (TOTAL + NT - 1) / NT;
  f32x4 v[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int u = threadIdx.x + NT * p;
    if (u < TOTAL) v[p] = rs_ld(rs, base + 16 * u);
  }
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int u = threadIdx.x + NT * p;
    if (u < TOTAL) st4(sh + rs_row<R>(u / U) + 4 * (u % U), v[p]);
  }
}

// sum over the KS lanes 4 j .. 4 j + KS - 1 (KS = 4: the lane quad; KS = 8:
// both quads of a half row, added by a half-row mirror), the same in all of them
template <int KS>
__device__ __forceinline__ float ksum(float v) {
  static_assert(KS == 4 || KS == 8, "lane group");
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  if (KS == 8) v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
  return v;
}

template <int N> struct FVec;
template <> struct FVec<2> { typedef f32x2 T; };
template <> struct FVec<4> { typedef f32x4 T; };
template <int N>
__device__ __forceinline__ typename FVec<N>::T rs_ldv(__amdgpu_buffer_rsrc_t rs, int off) {
  if constexpr (N == 2) return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 16));
  else return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 16));
}
template <int N>
__device__ __forceinline__ void rs_stv(__amdgpu_buffer_rsrc_t rs, int off, typename FVec<N>::T v) {
  if constexpr (N == 2) __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), rs, off, 0, 16);
  else __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, off, 0, 16);
}

// part: G Gram pieces [R][R] of X0 (their sum is X0^T X0); nparts: the nnp
// partial sums of ||X0||_F^2 (s = 1/||X0||_F, 0 for X0 = 0) or null (s = 1);
// Sring: kRsRing R x R floats; flags: kRsSyncWords words cleared by the launch
// before; M: s Q_iters [R][R]; limit: polls per wait before it gives up.
// RHO rows per workgroup; lane l of wave w owns the CPT columns from
// c0 = 32 w + CPT (l / KS) and the contraction part l % KS (R / KS values of
// k); STAGE: S_k is copied to LDS first (r <= 128), else every thread loads
// its entries itself.
template <int R, int RHO, int KS, int CPT, bool STAGE>
__global__ __launch_bounds__(2 * R) void k_spel_rsv(const float* __restrict__ part, int G,
                                                    const float* __restrict__ nparts, int nnp, int iters,
                                                    float* __restrict__ Sring, unsigned* __restrict__ flags,
                                                    float* __restrict__ M, unsigned limit) {
  typedef typename FVec<CPT>::T V;
  constexpr int KQ = R / KS, LP = KS * (KQ + 4), NS = R / RHO, SLOT = R * R * 4;
  static_assert(R % 32 == 0 && R % RHO == 0 && (64 / KS) * CPT == 32 && KQ % 4 == 0, "shape");
  static_assert(!STAGE || KS == 4, "the staged layout is padded for lane quads");
  static_assert(2 * NS <= kRsFlagWords, "one progress counter per workgroup");
  __shared__ __align__(16) float Lb[2][RHO][LP];  // left rows of a product, double-buffered
  extern __shared__ __align__(16) float Ssh[];     // S_k, staged (rows at rs_row)
  __shared__ float scs;
  __shared__ int slot;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int q = lane % KS, c0 = 32 * w + CPT * (lane / KS);
  const int lo = (c0 / KQ) * (KQ + 4) + c0 % KQ;  // position of column c0 in an LDS row
  const bool isS = blockIdx.x < NS;
  const int J = isS ? blockIdx.x : blockIdx.x - NS, r0 = J * RHO;
  const float sx = nparts ? block_inv_norm(nparts, nnp, &scs) : 1.f;
  const __amdgpu_buffer_rsrc_t rs = rs_rsrc(Sring);
  V b[KQ];  // S_k[q KQ + t][c0 .. c0 + CPT - 1]
  auto load = [&](int x) {  // S_{2x} -> b
    if constexpr (STAGE) {
      rs_stage<R, 2 * R>(rs, (x % kRsRing) * SLOT, Ssh);
      __syncthreads();
#pragma unroll
      for (int t = 0; t < KQ; ++t) b[t] = *reinterpret_cast<const V*>(Ssh + rs_row<R>(q * KQ + t) + c0);
    } else {
      const int base = (x % kRsRing) * SLOT + (q * KQ * R + c0) * 4;
#pragma unroll
      for (int t = 0; t < KQ; ++t) b[t] = rs_ldv<CPT>(rs, base + t * R * 4);
      __builtin_amdgcn_sched_barrier(0);  // every load in flight before the first use
    }
  };
  int buf = 0;
  auto put = [&](const V (&v)[RHO]) {  // v -> the next left rows, visible to every wave
    buf ^= 1;
    if (q == 0) {
#pragma unroll
      for (int i = 0; i < RHO; ++i) *reinterpret_cast<V*>(&Lb[buf][i][lo]) = v[i];
    }
    __syncthreads();
  };
  auto mul = [&](V (&out)[RHO]) {  // out = (left rows) S_k
#pragma unroll
    for (int i = 0; i < RHO; ++i) {
      float a[CPT] = {};
#pragma unroll
      for (int t = 0; t < KQ; t += 4) {
        const f32x4 l4 = ld4(&Lb[buf][i][q * (KQ + 4) + t]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int c = 0; c < CPT; ++c) a[c] = fmaf(l4[e], b[t + e][c], a[c]);
      }
#pragma unroll
      for (int c = 0; c < CPT; ++c) out[i][c] = ksum<KS>(a[c]);
    }
  };
  // (left rows) h(S_k), h(x) = 2.25 x - 1.5 x^2 + 0.25 x^3
  auto mul_h = [&](V (&out)[RHO]) {
    V a1[RHO], a2[RHO], a3[RHO];
    mul(a1);
    put(a1);
    mul(a2);
    put(a2);
    mul(a3);
#pragma unroll
    for (int i = 0; i < RHO; ++i) out[i] = (2.25f * a1[i] - 1.5f * a2[i]) + 0.25f * a3[i];
  };
  const int nx = (iters - 1) / 2;  // exchanges after S_0: S_2, S_4, .., S_{2 nx}

  if (isS) {
    // S_0 rows: s^2 times the pieces' sum, in piece order
    const float s2 = sx * sx;
    V s0[RHO];
#pragma unroll
    for (int i = 0; i < RHO; ++i) {
      const size_t o = size_t(r0 + i) * R + c0;
      V v = *reinterpret_cast<const V*>(part + o);
      for (int g = 1; g < G; ++g) v += *reinterpret_cast<const V*>(part + size_t(g) * R * R + o);
      s0[i] = v * s2;
      if (q == 0) rs_stv<CPT>(rs, int(o) * 4, s0[i]);
    }
    rs_publish(flags, J, 1u);
    for (int x = 0; x < nx; ++x) {  // S_{2x} -> S_{2x+2}
      // S_{2x} complete and, once the ring wraps, slot (x + 1) mod kRsRing (S_{2(x+1-kRsRing)})
      // read by every Q workgroup
      const int qneed = x + 2 - kRsRing;
      if (!rs_wait(flags, NS, unsigned(x + 1), qneed > 0 ? NS : 0, unsigned(max(qneed, 0)), limit, &slot)) return;
      load(x);
      V t1[RHO], t2[RHO], u[RHO], wv[RHO], y[RHO];
      put(s0);
      mul(t1);  // rows of S^2
      put(t1);
      mul(t2);  // rows of S^3
#pragma unroll
      for (int i = 0; i < RHO; ++i) u[i] = (2.25f * s0[i] - 1.5f * t1[i]) + 0.25f * t2[i];  // rows of S_{k+1}
      put(u);
      mul_h(wv);  // rows of S_{k+1}^2
      put(wv);
      mul_h(y);  // rows of S_{k+1}^3
#pragma unroll
      for (int i = 0; i < RHO; ++i) {
        s0[i] = (2.25f * u[i] - 1.5f * wv[i]) + 0.25f * y[i];  // rows of S_{k+2}
        if (q == 0) rs_stv<CPT>(rs, ((x + 1) % kRsRing) * SLOT + ((r0 + i) * R + c0) * 4, s0[i]);
      }
      rs_publish(flags, J, unsigned(x + 2));
    }
    return;
  }

  // Q workgroup: Q_{k+2} = B (1.5 I - 0.5 h(S_k)), B = Q_k T_k, for k = 0, 2, ..; an odd
  // step count ends with Q_n = Q_{n-1} T_{n-1}
  bool ok = true;
  V qv[RHO];
  for (int x = 0; 2 * x < iters; ++x) {
    if (!rs_wait(flags, NS, unsigned(x + 1), 0, 0u, limit, &slot)) {
      ok = false;
      break;
    }
    V bq[RHO];
    if (x == 0) {  // B = T_0, from this workgroup's rows of S_0
#pragma unroll
      for (int i = 0; i < RHO; ++i) {
        V srow;
        if constexpr (STAGE) srow = V{};
        else srow = rs_ldv<CPT>(rs, ((r0 + i) * R + c0) * 4);
        bq[i] = srow;
      }
    }
    load(x);
    if (x == 0) {
#pragma unroll
      for (int i = 0; i < RHO; ++i) {
        if constexpr (STAGE) bq[i] = *reinterpret_cast<const V*>(Ssh + rs_row<R>(r0 + i) + c0);
#pragma unroll
        for (int c = 0; c < CPT; ++c) bq[i][c] = (r0 + i == c0 + c ? 1.5f : 0.f) - 0.5f * bq[i][c];
      }
    }
    // the slot is rewritten only after every Q workgroup has read it, where an S
    // workgroup still has to write it (x + kRsRing <= nx)
    if (x + kRsRing <= nx) rs_publish(flags, NS + J, unsigned(x + 1));
    if (x > 0) {
      V t[RHO];
      put(qv);
      mul(t);
#pragma unroll
      for (int i = 0; i < RHO; ++i) bq[i] = 1.5f * qv[i] - 0.5f * t[i];
    }
    if (2 * x + 1 == iters) {  // the last, single step
#pragma unroll
      for (int i = 0; i < RHO; ++i) qv[i] = bq[i];
      break;
    }
    V bh[RHO];
    put(bq);
    mul_h(bh);
#pragma unroll
    for (int i = 0; i < RHO; ++i) qv[i] = 1.5f * bq[i] - 0.5f * bh[i];
  }
  if (threadIdx.x == 0) slot = int(__hip_atomic_load(flags + kRsTimeoutWord, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  __syncthreads();
  if (slot != 0) ok = false;
  if (q == 0) {
#pragma unroll
    for (int i = 0; i < RHO; ++i) {
      V o = qv[i] * sx;
      if (!ok) o = V{} + __builtin_nanf("");
      *reinterpret_cast<V*>(M + size_t(r0 + i) * R + c0) = o;
    }
  }
}

// Polar Express step matrix M = s (a I + b s^2 S + c s^4 S^2) [r][r], S the
// sum of the G Gram pieces, s = 1 / ||X||_F from per-block partial sums (the
// first step) or 1.  One block per 32 x 32 tile (bi, bj); S^2's tile is
// S[bi rows] S[bj rows]^T (S is symmetric), its r-long contraction taken in
// chunks of 128 staged in LDS -- every thread's piece loads issued before
// they are summed -- and split over the 8 waves, whose partial tiles are
// added in a fixed order (in the staging buffers, free by then).
constexpr int kPolyKC = 128;
constexpr int kPolyThreads = 512;

template <int G>
__global__ __launch_bounds__(kPolyThreads) void k_spel_poly(const float* __restrict__ part,
                                                            const float* __restrict__ nparts_in, int nparts_n,
                                                            float* __restrict__ M, int r, float ca, float cb,
                                                            float cc) {
  constexpr int NWV = kPolyThreads / 64;
  constexpr int LD = kPolyKC + 1;
  __shared__ float sm[2 * 32 * LD];  // rows bi.. and bj.. of S, one chunk; later the wave partials
  __shared__ float scs;
  static_assert(NWV * 1024 <= 2 * 32 * LD, "the wave partials reuse the staging buffers");
  float* sa = sm;
  float* sb = sm + 32 * LD;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int h = lane >> 5, l32 = lane & 31;
  const int bi = blockIdx.x, bj = blockIdx.y;
  const float sx = nparts_in ? block_inv_norm(nparts_in, nparts_n, &scs) : 1.f;
  const size_t rr = size_t(r) * r;

  f32x16 acc = f32x16{};
  for (int k0 = 0; k0 < r; k0 += kPolyKC) {
    const int kn = min(kPolyKC, r - k0);  // a multiple of 32
    const int per_row = kn / 4;           // 16-byte pieces per staged row
    // this thread's two pieces of each of the two row blocks: 4 G loads, all in flight
    f32x4 va[2][G], vb[2][G];
    int rw[2], cc4[2];
    bool ok[2];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int e = threadIdx.x + kPolyThreads * it;
      ok[it] = e < 32 * per_row;
      const int ee = ok[it] ? e : 0;
      rw[it] = ee / per_row;
      cc4[it] = (ee % per_row) * 4;
      const size_t oa = size_t(bi * 32 + rw[it]) * r + k0 + cc4[it];
      const size_t ob = size_t(bj * 32 + rw[it]) * r + k0 + cc4[it];
#pragma unroll
      for (int q = 0; q < G; ++q) {
        va[it][q] = ld4(part + q * rr + oa);
        vb[it][q] = ld4(part + q * rr + ob);
      }
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      if (!ok[it]) continue;
      f32x4 a = va[it][0], b = vb[it][0];
#pragma unroll
      for (int q = 1; q < G; ++q) {
        a += va[it][q];
        b += vb[it][q];
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        sa[rw[it] * LD + cc4[it] + t] = a[t];
        sb[rw[it] * LD + cc4[it] + t] = b[t];
      }
    }
    __syncthreads();
    // wave w: k in [w kn/NWV, (w+1) kn/NWV), two per multiply (lane half h takes k + h)
    const int kb = w * (kn / NWV);
    for (int k = kb; k < kb + kn / NWV; k += 2) acc = mfma_f32_32x32x2(sa[l32 * LD + k + h], sb[l32 * LD + k + h], acc);
    __syncthreads();
  }
  store_frag(sm + w * 1024, acc, lane);
  __syncthreads();
  if (threadIdx.x >= 256) return;
  const int i = threadIdx.x >> 3, j = (threadIdx.x & 7) * 4;
  const int fi = frag_index(i, j);
  f32x4 s2 = (ld4(sm + fi) + ld4(sm + 1024 + fi)) + (ld4(sm + 2048 + fi) + ld4(sm + 3072 + fi));
  s2 += (ld4(sm + 4096 + fi) + ld4(sm + 5120 + fi)) + (ld4(sm + 6144 + fi) + ld4(sm + 7168 + fi));
  const size_t o = size_t(bi * 32 + i) * r + bj * 32 + j;
  f32x4 s1 = ld4(part + o);
#pragma unroll
  for (int q = 1; q < G; ++q) s1 += ld4(part + q * rr + o);
  const float x2 = sx * sx, x4 = x2 * x2;
  f32x4 out;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const float id = (bi * 32 + i == bj * 32 + j + t) ? ca : 0.f;
    out[t] = sx * (id + cb * x2 * s1[t] + cc * x4 * s2[t]);
  }
  st4(M + o, out);
}

// row groups of the Gram pieces: 1, 2 or 4, about 256 rows each
int spel_groups(int64_t d) { return d >= 1024 ? 4 : d >= 512 ? 2 : 1; }

// the xm launch; `sticky`, `mnew`, `mcommit` and `status` serve only XM_NS_LAST_RET (the commit)
struct XmCommit {
  const unsigned* sticky = nullptr;
  const float* mnew = nullptr;
  float* mcommit = nullptr;
  int* status = nullptr;
};

template <bool NS>
void launch_xm(int G, dim3 grid, hipStream_t s, const float* X, const float* nparts_in, const float* part, float* out,
               int d, int r, int mode, const float* g, const float* m, float beta, float* nparts_out,
               const float* Acur, float alpha, float* Dout, float* Y0, XmCommit cm = {}) {
  auto k = G == 4 ? k_spel_xm<4, NS> : G == 2 ? k_spel_xm<2, NS> : k_spel_xm<1, NS>;
  // the M slab, 32 rows of pitch r + 4, or the 4 wave partials (16 KB) if larger; the
  // limit is raised once for the largest r (1024)
  constexpr int kXmLdsMax = 32 * (1024 + 4) * int(sizeof(float));
  (void)LdsLimit<k_spel_xm<1, NS>, kXmLdsMax>::bytes();
  (void)LdsLimit<k_spel_xm<2, NS>, kXmLdsMax>::bytes();
  (void)LdsLimit<k_spel_xm<4, NS>, kXmLdsMax>::bytes();
  const size_t lds = std::max<size_t>(size_t(32) * (r + 4) * sizeof(float), 4 * 1024 * sizeof(float));
  hipLaunchKernelGGL(k, grid, dim3(256), lds, s, X, nparts_in, part, out, d, r, mode, g, m, beta, nparts_out, Acur,
                     alpha, Dout, Y0, cm.sticky, cm.mnew, cm.mcommit, cm.status);
}

unsigned rs_spin_limit() {
  const char* e = std::getenv("MAPL_SPEL_SPIN_LIMIT");
  if (e == nullptr || *e == 0) return kRsSpinLimit;
  const unsigned long v = std::strtoul(e, nullptr, 10);
  return v < kRsSpinLimit ? unsigned(v) : kRsSpinLimit;
}

// The vector-ALU Gram-space iteration inside one launch: r <= 128 one row per
// workgroup, lane quads, S_k staged in LDS; 128 < r <= 256 two rows per
// workgroup, lane octets, S_k read straight into registers (r x r no longer
// fits LDS).  Either way 2 r / RHO workgroups that must all be resident.
template <int R>
void launch_rsv(const float* part, int G, const float* nparts, int nnp, int iters, float* Sbuf, unsigned* sync,
                float* M, hipStream_t s) {
  if constexpr (R <= 128) {
    constexpr int lds = kRsStageFloats<R> * int(sizeof(float));  // the staged S_k
    (void)LdsLimit<k_spel_rsv<R, 1, 4, 2, true>, lds>::bytes();
    hipLaunchKernelGGL((k_spel_rsv<R, 1, 4, 2, true>), dim3(2 * R), dim3(2 * R), lds, s, part, G, nparts, nnp, iters,
                       Sbuf, sync, M, rs_spin_limit());
  } else {
    hipLaunchKernelGGL((k_spel_rsv<R, 2, 8, 4, false>), dim3(R), dim3(2 * R), 0, s, part, G, nparts, nnp, iters, Sbuf,
                       sync, M, rs_spin_limit());
  }
}

// M = s Q_iters of the Gram-space iteration inside one launch (r <= 256)
void launch_rs_any(int r, const float* part, int G, const float* nparts, int nnp, int iters, float* Sbuf,
                   unsigned* sync, float* M, hipStream_t s) {
  switch (r) {
    case 32: launch_rsv<32>(part, G, nparts, nnp, iters, Sbuf, sync, M, s); break;
    case 64: launch_rsv<64>(part, G, nparts, nnp, iters, Sbuf, sync, M, s); break;
    case 96: launch_rsv<96>(part, G, nparts, nnp, iters, Sbuf, sync, M, s); break;
    case 128: launch_rsv<128>(part, G, nparts, nnp, iters, Sbuf, sync, M, s); break;
    case 160: launch_rsv<160>(part, G, nparts, nnp, iters, Sbuf, sync, M, s); break;
    case 192: launch_rsv<192>(part, G, nparts, nnp, iters, Sbuf, sync, M, s); break;
    case 224: launch_rsv<224>(part, G, nparts, nnp, iters, Sbuf, sync, M, s); break;
    default: launch_rsv<256>(part, G, nparts, nnp, iters, Sbuf, sync, M, s); break;
  }
}

// Whether every workgroup of the one-launch iteration for this r can be resident
// at once on the current device (its workgroups wait for each other), from the
// device's compute units and the kernel's occupancy; cached per device.  The
// environment variable MAPL_SPEL_GRAM_SPACE=0 answers no, for tests of the
// other form.
template <int R>
bool rsv_fits_now() {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return false;
  hipError_t e;
  int grid;
  if constexpr (R <= 128) {
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(k_spel_rsv<R, 1, 4, 2, true>),
                                                     2 * R, kRsStageFloats<R> * sizeof(float));
    grid = 2 * R;
  } else {
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(k_spel_rsv<R, 2, 8, 4, false>),
                                                     2 * R, 0);
    grid = R;
  }
  return e == hipSuccess && int64_t(per_cu) * cus >= grid;
}

bool rsv_fits(int r) {
  const char* e = std::getenv("MAPL_SPEL_GRAM_SPACE");
  if (e != nullptr && e[0] == '0' && e[1] == 0) return false;
  if (r > 256 || r % 32 != 0) return false;
  static std::atomic<int8_t> cache[64][8];  // 0 not known yet, 1 no, 2 yes
  int dev = 0;
  const bool cacheable = hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64;
  const int k = r / 32 - 1;
  if (cacheable) {
    const int8_t v = cache[dev][k].load(std::memory_order_relaxed);
    if (v != 0) return v == 2;
  }
  bool fits = false;
  switch (r) {
    case 32: fits = rsv_fits_now<32>(); break;
    case 64: fits = rsv_fits_now<64>(); break;
    case 96: fits = rsv_fits_now<96>(); break;
    case 128: fits = rsv_fits_now<128>(); break;
    case 160: fits = rsv_fits_now<160>(); break;
    case 192: fits = rsv_fits_now<192>(); break;
    case 224: fits = rsv_fits_now<224>(); break;
    default: fits = rsv_fits_now<256>(); break;
  }
  if (cacheable) cache[dev][k].store(fits ? 2 : 1, std::memory_order_relaxed);
  return fits;
}

}  // namespace

// workspace: Xa | Xb | Xc | Xm [d][r] | part [groups][r][r] | nparts
// [(d/32)(r/32)] | M [r][r] | nparts of Y0 [(d/32)(r/32)] | S ring
// [kRsRing][r][r] | progress, timeout and sticky words [kRsSyncWords], each region
// 16-byte aligned.  Xm holds the new momentum until the step commits.
static size_t a4(size_t n) { return (n + 3) & ~size_t(3); }

struct SpelWs {
  float *Xa, *Xb, *Xc, *Xm, *part, *nparts, *Mb, *nparts2, *Sbuf;
  unsigned* sync;
};

static SpelWs spel_ws(void* ws, int d, int r) {
  const size_t dr = size_t(d) * r, rr = size_t(r) * r, np = a4(size_t(d / 32) * (r / 32));
  SpelWs w;
  w.Xa = static_cast<float*>(ws);
  w.Xb = w.Xa + dr;
  w.Xc = w.Xb + dr;
  w.Xm = w.Xc + dr;
  w.part = w.Xm + dr;
  w.nparts = w.part + size_t(spel_groups(d)) * rr;
  w.Mb = w.nparts + np;
  w.nparts2 = w.Mb + rr;
  w.Sbuf = w.nparts2 + np;
  w.sync = reinterpret_cast<unsigned*>(w.Sbuf + kRsRing * rr);
  return w;
}

size_t spel_ws_bytes(int64_t d, int64_t r) {
  const size_t np = a4(size_t(d / 32) * (r / 32));
  const size_t floats =
      4 * size_t(d) * r + size_t(spel_groups(d)) * r * r + np + size_t(r) * r + np + kRsRing * size_t(r) * r + kRsSyncWords;
  return (floats + 64) * sizeof(float);
}

void launch_spel(float* A, const float* g, float* m, float alpha, float beta, int ns_iters, float* D_out, int* status,
                 int d, int r, void* ws, hipStream_t s) {
  const int G = spel_groups(d);
  const SpelWs w = spel_ws(ws, d, r);
  float* part = w.part;
  const int nb = r / 32;
  const dim3 blk(256);
  const dim3 ggrid(nb * (nb + 1) / 2 * G);
  const dim3 xgrid(d / 32, r / 32);
  // the last launch commits A and m = Xm unless the step's sticky timeout word is set
  XmCommit cm;
  cm.sticky = w.sync + kRsStickyWord;
  cm.mnew = w.Xm;
  cm.mcommit = m;
  cm.status = status;

  // Eq. (4)-(5): M = sym(A^T g) ; Xm = beta m + (1 - beta)(g - A M) ; per-block sums of Xm^2.
  // The first launch clears every sync word, the sticky one included.
  hipLaunchKernelGGL(k_spel_gram<1>, ggrid, blk, 0, s, A, g, part, d, r, G, w.sync, kRsSyncWords);
  launch_xm<false>(G, xgrid, s, A, nullptr, part, w.Xm, d, r, int(XM_TANGENT), g, m, beta, w.nparts, nullptr, 0.f,
                   nullptr, nullptr);

  if (rsv_fits(r)) {
    // Gram-space iteration in one launch (r <= 256, and all its workgroups resident at
    // once): S_0 from the pieces of Xm^T Xm, M = s Q_n, then D = Xm M and Y0 = A - alpha D
    // (Eq. (6)); the same for Y0 (unscaled) and A = Y0 M (Eq. (7)).
    const int npn = (d / 32) * (r / 32);
    hipLaunchKernelGGL(k_spel_gram<0>, ggrid, blk, 0, s, w.Xm, w.Xm, part, d, r, G, w.sync, kRsStickyWord);
    launch_rs_any(r, part, G, w.nparts, npn, ns_iters, w.Sbuf, w.sync, w.Mb, s);
    launch_xm<false>(1, xgrid, s, w.Xm, nullptr, w.Mb, nullptr, d, r, int(XM_NS_LAST_LMO), nullptr, nullptr, 0.f,
                     nullptr, A, alpha, D_out, w.Xc);
    hipLaunchKernelGGL(k_spel_gram<0>, ggrid, blk, 0, s, w.Xc, w.Xc, part, d, r, G, w.sync, kRsStickyWord);
    launch_rs_any(r, part, G, nullptr, 0, ns_iters, w.Sbuf, w.sync, w.Mb, s);
    launch_xm<false>(1, xgrid, s, w.Xc, nullptr, w.Mb, A, d, r, int(XM_NS_LAST_RET), nullptr, nullptr, 0.f, nullptr,
                     nullptr, 0.f, nullptr, nullptr, cm);
    return;
  }

  // Eq. (6): D = NS(s Xm), s = 1/||Xm||_F; the last step forms Y0 = A - alpha D in Xc
  const float* cur = w.Xm;
  const float* cur_np = w.nparts;
  float* bufs[2] = {w.Xa, w.Xb};
  for (int it = 0; it < ns_iters; ++it) {
    float* nxt = bufs[it & 1];
    hipLaunchKernelGGL(k_spel_gram<0>, ggrid, blk, 0, s, cur, cur, part, d, r, G, nullptr, 0);
    const int mode = (it == ns_iters - 1) ? int(XM_NS_LAST_LMO) : int(XM_NS);
    launch_xm<true>(G, xgrid, s, cur, cur_np, part, nxt, d, r, mode, nullptr, nullptr, 0.f, nullptr, A, alpha, D_out,
                    w.Xc);
    cur = nxt;
    cur_np = nullptr;
  }

  // Eq. (7): A = NS(A - alpha D), input unscaled; the last step writes A (and commits m)
  cur = w.Xc;
  for (int it = 0; it < ns_iters; ++it) {
    const bool last = it == ns_iters - 1;
    float* nxt = last ? A : bufs[it & 1];
    hipLaunchKernelGGL(k_spel_gram<0>, ggrid, blk, 0, s, cur, cur, part, d, r, G, nullptr, 0);
    launch_xm<true>(G, xgrid, s, cur, nullptr, part, nxt, d, r, last ? int(XM_NS_LAST_RET) : int(XM_NS), nullptr,
                    nullptr, 0.f, nullptr, nullptr, 0.f, nullptr, nullptr, last ? cm : XmCommit{});
    cur = nxt;
  }
}

}  // namespace mapl

namespace mapl {

// ------------------------------------------------------ Polar Express (host) --
// Minimax odd quintic a x + b x^3 + c x^5 for the constant 1 on [lo, hi] by
// the Remez exchange on four alternation points (the two ends and p's two
// interior critical points).  Returns E = max |1 - p| on [lo, hi].
namespace {

bool solve4(double m[4][5]) {  // Gaussian elimination with partial pivoting, in place
  for (int c = 0; c < 4; ++c) {
    int piv = c;
    for (int i = c + 1; i < 4; ++i)
      if (std::fabs(m[i][c]) > std::fabs(m[piv][c])) piv = i;
    if (m[piv][c] == 0.0) return false;
    for (int k = 0; k < 5; ++k) std::swap(m[c][k], m[piv][k]);
    for (int i = 0; i < 4; ++i) {
      if (i == c) continue;
      const double f = m[i][c] / m[c][c];
      for (int k = c; k < 5; ++k) m[i][k] -= f * m[c][k];
    }
  }
  for (int i = 0; i < 4; ++i) m[i][4] /= m[i][i];
  return true;
}

double remez_quintic(double lo, double hi, double coef[3]) {
  double xs[4] = {lo, lo + 0.25 * (hi - lo), lo + 0.75 * (hi - lo), hi};
  double E = 0.0;
  for (int it = 0; it < 60; ++it) {
    double m[4][5];
    for (int i = 0; i < 4; ++i) {
      const double x = xs[i], x2 = x * x;
      m[i][0] = x;
      m[i][1] = x * x2;
      m[i][2] = x * x2 * x2;
      m[i][3] = (i & 1) ? -1.0 : 1.0;
      m[i][4] = 1.0;
    }
    if (!solve4(m)) break;
    coef[0] = m[0][4];
    coef[1] = m[1][4];
    coef[2] = m[2][4];
    E = std::fabs(m[3][4]);
    const double a = coef[0], b = coef[1], c = coef[2];
    const double disc = 9.0 * b * b - 20.0 * a * c;  // critical points: 5 c y^2 + 3 b y + a = 0, y = x^2
    if (c == 0.0 || disc < 0.0) break;
    double y0 = (-3.0 * b - std::sqrt(disc)) / (10.0 * c), y1 = (-3.0 * b + std::sqrt(disc)) / (10.0 * c);
    if (y0 > y1) std::swap(y0, y1);
    if (y0 <= 0.0) break;
    const double x1 = std::sqrt(y0), x2 = std::sqrt(y1);
    if (!(lo < x1 && x2 < hi)) break;
    const double change = std::max(std::fabs(x1 - xs[1]), std::fabs(x2 - xs[2]));
    xs[1] = x1;
    xs[2] = x2;
    if (change <= 1e-15 * hi) break;
  }
  return E;
}

}  // namespace

int polar_express_schedule(double ell, int steps, double* coef, double* err) {
  double lo = ell, hi = 1.0;
  for (int t = 0; t < steps; ++t) {
    double* c = coef + 3 * t;
    double E;
    if (hi - lo < 1e-4) {  // the limit of the minimax quintic as the interval shrinks to {1}
      c[0] = 15.0 / 8.0;
      c[1] = -10.0 / 8.0;
      c[2] = 3.0 / 8.0;
      auto p = [&](double x) { return c[0] * x + c[1] * x * x * x + c[2] * x * x * x * x * x; };
      E = std::max(std::fabs(1.0 - p(lo)), std::fabs(1.0 - p(hi)));
    } else {
      E = remez_quintic(lo, hi, c);
    }
    if (!std::isfinite(E) || !std::isfinite(c[0]) || !std::isfinite(c[1]) || !std::isfinite(c[2])) return -1;
    if (err) err[t] = E;
    lo = 1.0 - E;
    hi = 1.0 + E;
  }
  return 0;
}

void launch_spel_pe(float* A, const float* g, float* m, float alpha, float beta, const float* coef_lmo, int lmo_steps,
                    const float* coef_ret, int ret_steps, float* D_out, int* status, int d, int r, void* ws,
                    hipStream_t s) {
  const int G = spel_groups(d);
  const SpelWs w = spel_ws(ws, d, r);
  float* part = w.part;
  const int npn = (d / 32) * (r / 32);
  const int nb = r / 32;
  const dim3 blk(256);
  const dim3 ggrid(nb * (nb + 1) / 2 * G);
  const dim3 xgrid(d / 32, r / 32);
  const dim3 pgrid(nb, nb);
  XmCommit cm;  // no waits here: the sticky word stays clear and the last launch always commits
  cm.sticky = w.sync + kRsStickyWord;
  cm.mnew = w.Xm;
  cm.mcommit = m;
  cm.status = status;

  // Eq. (4)-(5) as in launch_spel
  hipLaunchKernelGGL(k_spel_gram<1>, ggrid, blk, 0, s, A, g, part, d, r, G, w.sync, kRsSyncWords);
  launch_xm<false>(G, xgrid, s, A, nullptr, part, w.Xm, d, r, int(XM_TANGENT), g, m, beta, w.nparts, nullptr, 0.f,
                   nullptr, nullptr);

  // one Polar Express step: S from the Gram pieces, M = s (a I + b s^2 S + c s^4 S^2), out = X M
  float* bufs[2] = {w.Xa, w.Xb};
  auto step = [&](const float* cur, const float* np_in, const float* c3, float* out, int mode, float* np_out,
                  XmCommit c) {
    hipLaunchKernelGGL(k_spel_gram<0>, ggrid, blk, 0, s, cur, cur, part, d, r, G, nullptr, 0);
    auto poly = G == 8 ? k_spel_poly<8> : G == 4 ? k_spel_poly<4> : G == 2 ? k_spel_poly<2> : k_spel_poly<1>;
    hipLaunchKernelGGL(poly, pgrid, dim3(kPolyThreads), 0, s, part, np_in, npn, w.Mb, r, c3[0], c3[1], c3[2]);
    launch_xm<false>(1, xgrid, s, cur, nullptr, w.Mb, out, d, r, mode, nullptr, nullptr, 0.f, np_out, A, alpha, D_out,
                     w.Xc, c);
  };
  // Eq. (6): D = PE(Xm / ||Xm||_F); the last step forms Y0 = A - alpha D in Xc and its squares
  const float* cur = w.Xm;
  for (int t = 0; t < lmo_steps; ++t) {
    const bool last = t == lmo_steps - 1;
    float* nxt = bufs[t & 1];
    step(cur, t == 0 ? w.nparts : nullptr, coef_lmo + 3 * t, nxt, last ? int(XM_NS_LAST_LMO) : int(XM_NS),
         last ? w.nparts2 : nullptr, XmCommit{});
    cur = nxt;
  }
  // Eq. (7): A = PE(Y0 / ||Y0||_F); the last step writes A and commits m
  cur = w.Xc;
  for (int t = 0; t < ret_steps; ++t) {
    const bool last = t == ret_steps - 1;
    float* nxt = last ? A : bufs[t & 1];
    step(cur, t == 0 ? w.nparts2 : nullptr, coef_ret + 3 * t, nxt, last ? int(XM_NS_LAST_RET) : int(XM_NS), nullptr,
         last ? cm : XmCommit{});
    cur = nxt;
  }
}

}  // namespace mapl
