// Gradient of the trainable anchor table E_small.
//
// Source: "Learned Subspace Compression for Communication-Efficient Pipeline
// Parallelism", Section 3.2 and Eq. (3): the anchor E_small[t] P is part of
// both maps (subtracted in Eq. (1), added in Eq. (2)) and E_small is trained,
// so dL/dE[v] collects, over the tokens whose id is v, the token gradient
// pulled back through P:  gE[v] = alpha * sum_{n : t_n = v} Y[n] P^T.
//
// Two launches:
//   project  U[n] = alpha Y[n] P^T (fp32 [N][r]) on the matrix cores, plus a
//            max |U| per block or output wave (no atomics: a chain of atomics
//            on one address serialises).  bf16 at r = 128, 256 uses the
//            codec's streaming reduction kernel with P's fragment pack.
//   own      block b owns the ids v with v % B == b (B blocks: frequent ids,
//            which tokenizers give small numbers, land in different blocks)
//            and one 64-column slice.  It reads the token ids in chunks,
//            queues its own tokens in LDS (one LDS atomic per wave and step),
//            adds their U rows into an LDS table of 64-bit integers at one
//            power-of-two scale 2^e taken from the global max |U| and N (runs
//            of one id summed in registers first), and writes its gE rows.  Integer addition is associative, so each
//            row is the same bit pattern whatever order the tokens are added
//            in; no row is shared between blocks, so there are no global
//            atomics and no table in HBM.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace mapl {

namespace {

constexpr int kProjMaxGrid = 1024;  // project blocks along the tokens (the rest loop)
constexpr int kOwnThreads = 512;    // 8 waves per owner block, two blocks per CU
constexpr int kOwnVR = 128;         // ids per owner block (LDS table rows)
constexpr int kOwnPer = 4;          // token ids each thread loads per chunk
constexpr int kOwnChunk = kOwnThreads * kOwnPer;  // token ids per chunk
constexpr int kOwnQueue = 4000;     // LDS queue capacity (entries); two blocks fit in 160 KB
static_assert(kOwnQueue >= kOwnChunk, "a chunk must fit in an empty queue");
constexpr int kOwnBatch = 32;       // queued tokens whose U loads one wave keeps in flight
constexpr int kOwnBatchQ = 16;      // the same in 16-byte loads (4 tokens per wave instruction)

// running max |x| that lets a non-finite value through: NaN counts as +inf
// (fmaxf alone would drop it), so a non-finite projection reaches the owner
// kernel's scale, which then marks the whole table NaN
__device__ __forceinline__ float absmax_nf(float m, float x) { return fmaxf(m, x == x ? fabsf(x) : __builtin_inff()); }

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// block max of non-negative values (all threads must call)
template <int WAVES>
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int i = 1; i < WAVES; ++i) m = fmaxf(m, red[i]);
  __syncthreads();  // red may be reused
  return m;
}

// bf16 (d a multiple of 128, r of 32): a block takes 32-token tiles; wave w
// computes the 32 x 32 tile of U at columns 32 (4 blockIdx.y + w), over the
// whole d-long contraction.  The matrix-core A operand is 16 bytes of a row of
// P (output column j), the B operand 16 bytes of a row of Y (token n); the
// four waves read the same Y rows.
__global__ __launch_bounds__(256) void k_ag_project_bf16(const bf16_t* __restrict__ Y, const bf16_t* __restrict__ P,
                                                         float* __restrict__ U, float* __restrict__ part, float alpha,
                                                         int N, int d, int r) {
  __shared__ float red[4];
  const int lane = threadIdx.x & 63, w = wave_id();
  const int hi = lane >> 5, l32 = lane & 31;
  const int jb = blockIdx.y * 4 + w;
  const bool active = jb * 32 < r;  // uniform per wave
  const bf16_t* pr = P + size_t(min(jb * 32 + l32, r - 1)) * d + 8 * hi;
  float local = 0.f;
  for (int tile = blockIdx.x; tile * 32 < N; tile += gridDim.x) {
    if (!active) break;
    const int n = tile * 32 + l32;
    const bf16_t* yr = Y + size_t(min(n, N - 1)) * d + 8 * hi;
    f32x16 acc = f32x16{};
    for (int k0 = 0; k0 < d; k0 += 128) {
      bf16x8 a[8], b[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        a[t] = ld_bf16x8(pr + k0 + 16 * t);
        b[t] = ld_bf16x8(yr + k0 + 16 * t);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 8; ++t) acc = mfma_bf16_32x32x16(a[t], b[t], acc);
    }
    // lane (l32, hi), register 4q + e holds U[n][32 jb + 8q + 4hi + e]
    if (n < N) {
      float* ur = U + size_t(n) * r + jb * 32 + 4 * hi;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = alpha * acc[4 * q + e];
          local = absmax_nf(local, v[e]);
        }
        *reinterpret_cast<f32x4*>(ur + 8 * q) = v;
      }
    }
  }
  const float m = block_max<4>(local, red);
  if (threadIdx.x == 0) part[blockIdx.y * gridDim.x + blockIdx.x] = m;
}

// fp32: one thread per element of U (grid-stride)
__global__ __launch_bounds__(256) void k_ag_project_f32(const float* __restrict__ Y, const float* __restrict__ P,
                                                        float* __restrict__ U, float* __restrict__ part, float alpha,
                                                        int N, int d, int r) {
  __shared__ float red[4];
  float local = 0.f;
  const int64_t ne = int64_t(N) * r;
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < ne; e += int64_t(gridDim.x) * 256) {
    const int n = int(e / r), j = int(e % r);
    const float* yr = Y + size_t(n) * d;
    const float* pr = P + size_t(j) * d;
    float s = 0.f;
    for (int k = 0; k < d; ++k) s = fmaf(yr[k], pr[k], s);
    const float v = alpha * s;
    U[e] = v;
    local = absmax_nf(local, v);
  }
  const float m = block_max<4>(local, red);
  if (threadIdx.x == 0) part[blockIdx.x] = m;
}

// Identity projection (the full-rank anchor, P = I, r = d): U = alpha Y.
// bf16: 8 values per thread and step (d % 8 == 0); fp32: one value.  Grid-stride.
template <bool BF16>
__global__ __launch_bounds__(256) void k_ag_identity(const void* __restrict__ Yv, float* __restrict__ U,
                                                     float* __restrict__ part, float alpha, int64_t ne) {
  __shared__ float red[4];
  float local = 0.f;
  const int64_t step = int64_t(gridDim.x) * 256;
  if (BF16) {
    const u32x4* Y = static_cast<const u32x4*>(Yv);
    for (int64_t u = int64_t(blockIdx.x) * 256 + threadIdx.x; u < ne / 8; u += step) {
      const u32x4 y = Y[u];
      f32x4 v[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint32_t w = y[2 * h + e];
          v[h][2 * e] = alpha * bf2f(uint16_t(w & 0xffffu));
          v[h][2 * e + 1] = alpha * bf2f(uint16_t(w >> 16));
        }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int e = 0; e < 4; ++e) local = absmax_nf(local, v[h][e]);
        reinterpret_cast<f32x4*>(U)[2 * u + h] = v[h];
      }
    }
  } else {
    const float* Y = static_cast<const float*>(Yv);
    for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < ne; e += step) {
      const float v = alpha * Y[e];
      U[e] = v;
      local = absmax_nf(local, v);
    }
  }
  const float m = block_max<4>(local, red);
  if (threadIdx.x == 0) part[blockIdx.x] = m;
}

// power-of-two scale 2^e of the fixed-point terms: with max |U| < 2^ex every
// scaled term is below 2^30 in magnitude (an int32 after rounding), so a sum
// of at most N < 2^31 of them stays below 2^61 in 64 bits.  Each term is
// rounded once, by at most 2^-31 * 2^ex <= 2^-30 * max |U|.
__device__ __forceinline__ int fixed_exponent(float m) {
  int ex;
  (void)frexpf(m, &ex);  // m < 2^ex (ex = 0 for m = 0)
  return 30 - ex;
}

// x * 2^e rounded to the nearest integer, as an int32 (|x| <= max |U|: exact scaling, fits)
__device__ __forceinline__ long long fixed_term(float x, int e) {
  return static_cast<long long>(static_cast<int>(rintf(ldexpf(x, e))));
}

// q = t / B, rem = t % B for 0 <= t < 2^24, 1 <= B < 2^16: a float estimate of
// the quotient (off by at most one) and one correction each way, instead of
// the integer division sequence
__device__ __forceinline__ void divmod_small(int t, int B, float invB, int& q, int& rem) {
  q = int(float(t) * invB);
  rem = t - q * B;
  if (rem < 0) q -= 1, rem += B;
  if (rem >= B) q += 1, rem -= B;
}

// Owner block b (blockIdx.x) of B = gridDim.x holds the ids v = s B + b,
// s < kOwnVR, and columns [64 blockIdx.y, + 64): lane = column.  The block
// scans the ids chunk by chunk (the next chunk's loads in flight while the
// current one is queued) and adds the queued rows once the scan is done or the
// queue could overflow.  Queue entry: (slot s << 24) | token, token < 2^24.
template <bool QUAD>
__global__ __launch_bounds__(kOwnThreads, 2) void k_ag_own(const float* __restrict__ U,
                                                           const int32_t* __restrict__ tids,
                                                           const float* __restrict__ part, int npart,
                                                           float* __restrict__ gE, int N, int r, int V, int accumulate) {
  constexpr int NW = kOwnThreads / 64;
  static_assert(kOwnVR <= 256, "queue entry packing");
  __shared__ unsigned long long acc[kOwnVR * 64];
  __shared__ uint32_t q[kOwnQueue];
  __shared__ float red[NW];
  __shared__ int q_count;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int B = gridDim.x, b = blockIdx.x;
  const int col = blockIdx.y * 64 + lane;
  const bool colok = col < r;
  const int ccol = min(col, r - 1);
  const float invB = 1.0f / float(B);

  // the first chunk's ids (clamped, always valid) are requested before anything else
  int tv[kOwnPer];
#pragma unroll
  for (int k = 0; k < kOwnPer; ++k) tv[k] = tids[min(k * kOwnThreads + int(threadIdx.x), N - 1)];

  // global scale from the per-block maxima of the projection
  float m = 0.f;
  for (int i = threadIdx.x; i < npart; i += kOwnThreads) m = fmaxf(m, part[i]);
  for (int i = threadIdx.x; i < kOwnVR * 64; i += kOwnThreads) acc[i] = 0ull;
  if (threadIdx.x == 0) q_count = 0;
  m = block_max<NW>(m, red);  // its barriers also publish the zeroed table and count
  if (!(m < __builtin_inff())) {
    // a projected value is not finite (Y overflowed or holds NaN): no fixed-point scale
    // exists, and every row of the table becomes NaN rather than a silently wrong number
    if (!colok) return;
    const float nan = __builtin_nanf("");
    for (int sl = w; sl < kOwnVR; sl += NW) {
      const int64_t v = int64_t(sl) * B + b;
      if (v >= V) break;
      gE[size_t(v) * r + col] = nan;
    }
    return;
  }
  const int ex = fixed_exponent(m);

  // QUAD (r % 4 == 0): lane = (entry g = lane >> 4, columns 4 (lane & 15) + 0..3);
  // one 16-byte load per lane covers four entries per wave instruction, and
  // wave w takes entries w + NW (4 j + g).  A run of one slot in a lane's own
  // sequence of entries is summed in registers and added once.
  auto add_queue_quad = [&](int cnt) {
    const int g = lane >> 4, c4 = blockIdx.y * 64 + 4 * (lane & 15);
    const bool ok4 = c4 < r;  // r % 4 == 0: all four columns or none
    const int cc4 = min(c4, r - 4);
    for (int i0 = w + NW * g; i0 < cnt; i0 += NW * 4 * kOwnBatchQ) {
      f32x4 x[kOwnBatchQ];
      int sl[kOwnBatchQ];
#pragma unroll
      for (int k = 0; k < kOwnBatchQ; ++k) {
        const int i = i0 + NW * 4 * k;
        const uint32_t e = q[min(i, cnt - 1)];  // clamped: always a queued token
        sl[k] = (i < cnt) ? int(e >> 24) : -1;
        x[k] = *reinterpret_cast<const f32x4*>(U + size_t(e & 0xffffffu) * r + cc4);
      }
#pragma unroll
      for (int k = 0; k < kOwnBatchQ; ++k) asm volatile("" : : "v"(x[k]));
      long long run[4] = {0, 0, 0, 0};
      int run_slot = sl[0];
#pragma unroll
      for (int k = 0; k < kOwnBatchQ; ++k) {
        if (sl[k] >= 0) {
          if (sl[k] != run_slot) {
            if (ok4) {
#pragma unroll
              for (int c = 0; c < 4; ++c)
                atomicAdd(&acc[run_slot * 64 + (c4 & 63) + c], static_cast<unsigned long long>(run[c]));
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) run[c] = 0;
            run_slot = sl[k];
          }
#pragma unroll
          for (int c = 0; c < 4; ++c) run[c] += fixed_term(x[k][c], ex);
        }
      }
      if (run_slot >= 0 && ok4) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          atomicAdd(&acc[run_slot * 64 + (c4 & 63) + c], static_cast<unsigned long long>(run[c]));
      }
    }
  };

  // add queued rows [0, cnt): wave w takes entries w, w + NW, ...; a run of
  // consecutive entries with one slot is summed in registers and added once
  auto add_queue = [&](int cnt) {
    if (QUAD) {
      add_queue_quad(cnt);
      return;
    }
    for (int i0 = w; i0 < cnt; i0 += NW * kOwnBatch) {
      float x[kOwnBatch];
      int sl[kOwnBatch];
#pragma unroll
      for (int k = 0; k < kOwnBatch; ++k) {
        const uint32_t e = q[min(i0 + NW * k, cnt - 1)];  // clamped: always a queued token
        sl[k] = (i0 + NW * k < cnt) ? int(e >> 24) : -1;
        x[k] = U[size_t(e & 0xffffffu) * r + ccol];
      }
      // every row value is resolved here, after all loads were issued: otherwise
      // the compiler moves each load into the branches below and waits on it there
#pragma unroll
      for (int k = 0; k < kOwnBatch; ++k) asm volatile("" : : "v"(x[k]));
      long long run = 0;
      int run_slot = sl[0];
#pragma unroll
      for (int k = 0; k < kOwnBatch; ++k) {
        if (sl[k] < 0) break;  // uniform: the rest of the batch is padding
        if (sl[k] != run_slot) {
          if (colok) atomicAdd(&acc[run_slot * 64 + lane], static_cast<unsigned long long>(run));
          run = 0;
          run_slot = sl[k];
        }
        run += fixed_term(x[k], ex);
      }
      if (run_slot >= 0 && colok) atomicAdd(&acc[run_slot * 64 + lane], static_cast<unsigned long long>(run));
    }
  };

  for (int base = 0; base < N; base += kOwnChunk) {
#pragma unroll
    for (int k = 0; k < kOwnPer; ++k) {
      const int n = base + k * kOwnThreads + threadIdx.x;
      const int t = tv[k];
      const bool valid = n < N && t >= 0 && t < V;
      int tq, trem;
      divmod_small(valid ? t : 0, B, invB, tq, trem);
      const bool mine = valid && trem == b;
      const uint64_t mask = __ballot(mine);
      if (mask) {  // uniform per wave
        int qbase = 0;
        if (lane == 0) qbase = atomicAdd(&q_count, __popcll(mask));
        qbase = __shfl(qbase, 0);
        if (mine) q[qbase + __popcll(mask & ((1ull << lane) - 1))] = (uint32_t(tq) << 24) | uint32_t(n);
      }
    }
    const int nb = base + kOwnChunk;
    if (nb < N) {  // the next chunk's ids load while this one is queued and (maybe) added
#pragma unroll
      for (int k = 0; k < kOwnPer; ++k) tv[k] = tids[min(nb + k * kOwnThreads + int(threadIdx.x), N - 1)];
    }
    __syncthreads();
    const int cnt = q_count;
    if (nb >= N || cnt > kOwnQueue - kOwnChunk) {  // uniform
      add_queue(cnt);
      __syncthreads();  // queue consumed
      if (threadIdx.x == 0) q_count = 0;
      __syncthreads();
    }
  }

  // write the owned rows (every one when overwriting; rows with no token add 0)
  if (!colok) return;
  for (int sl = w; sl < kOwnVR; sl += NW) {
    const int64_t v = int64_t(sl) * B + b;
    if (v >= V) break;
    const float val = float(ldexp(double(static_cast<long long>(acc[sl * 64 + lane])), -ex));
    float* o = gE + size_t(v) * r + col;
    *o = accumulate ? *o + val : val;
  }
}

int proj_blocks(int N, int r, int y_bf16) {
  if (y_bf16) return std::min((N + 31) / 32, kProjMaxGrid) * ((r + 127) / 128);
  return int(std::min<int64_t>((int64_t(N) * r + 255) / 256, kProjMaxGrid));
}

size_t a256(size_t b) { return (b + 255) & ~size_t(255); }

// U [N][r] fp32 | partial maxima
size_t part_offset(int64_t N, int64_t r) { return a256(size_t(N) * r * 4); }
size_t npart_max(int64_t N) { return std::max<size_t>(size_t(kProjMaxGrid) * 4, size_t(4) * ((N + 63) / 64)); }

}  // namespace

size_t anchor_grad_ws_bytes(int64_t N, int64_t r, int64_t V) {
  (void)V;
  return part_offset(N, r) + a256(npart_max(N) * 4);
}

void launch_anchor_grad(const void* Y, int y_bf16, const int32_t* tids, const void* P, const uint16_t* PF,
                        float* gE, float alpha, int accumulate, int N, int d, int r, int V, void* ws, hipStream_t s) {
  float* U = static_cast<float*>(ws);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + part_offset(N, r));
  int npart;
  if (P == nullptr) {  // identity projection (r == d)
    const int64_t ne = int64_t(N) * d;
    npart = int(std::min<int64_t>((ne / (y_bf16 ? 8 : 1) + 255) / 256, kProjMaxGrid));
    if (y_bf16)
      hipLaunchKernelGGL(k_ag_identity<true>, dim3(unsigned(npart)), dim3(256), 0, s, Y, U, part, alpha, ne);
    else
      hipLaunchKernelGGL(k_ag_identity<false>, dim3(unsigned(npart)), dim3(256), 0, s, Y, U, part, alpha, ne);
  } else if (y_bf16 && PF != nullptr &&
      launch_tok_reduce_f32out(static_cast<const uint16_t*>(Y), PF, U, alpha, part, N, d, r, s)) {
    npart = 4 * ((N + 63) / 64);
  } else if (y_bf16) {
    npart = proj_blocks(N, r, 1);
    const int gx = std::min((N + 31) / 32, kProjMaxGrid);
    hipLaunchKernelGGL(k_ag_project_bf16, dim3(unsigned(gx), unsigned((r + 127) / 128)), dim3(256), 0, s,
                       static_cast<const bf16_t*>(Y), static_cast<const bf16_t*>(P), U, part, alpha, N, d, r);
  } else {
    npart = proj_blocks(N, r, 0);
    hipLaunchKernelGGL(k_ag_project_f32, dim3(unsigned(npart)), dim3(256), 0, s, static_cast<const float*>(Y),
                       static_cast<const float*>(P), U, part, alpha, N, d, r);
  }
  const int B = (V + kOwnVR - 1) / kOwnVR;
  auto own = (r % 4 == 0) ? k_ag_own<true> : k_ag_own<false>;
  hipLaunchKernelGGL(own, dim3(unsigned(B), unsigned((r + 63) / 64)), dim3(kOwnThreads), 0, s, U, tids, part,
                     npart, gE, N, r, V, accumulate);
}

}  // namespace mapl
