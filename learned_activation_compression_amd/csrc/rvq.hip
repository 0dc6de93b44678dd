// Residual multi-codebook VQ of the projected boundary activation.
//
// Source: "Learned Subspace Compression for Communication-Efficient Pipeline
// Parallelism", Section 3.5 (Z split into G groups, R rounds, each round
// quantising the previous round's residual against a per-stage codebook) and
// Appendix F (streamed codebook sync: the receiver overwrites the codewords
// the sender streams).
//
// Encode: one block owns one group g and a range of tokens.  The round's
// codebook for g sits in LDS transposed ([dim][codeword]) with its squared
// norms.  Each wave keeps NT tiles of 32 tokens' residuals in registers (lane
// half h holds dims [h*W/2, (h+1)*W/2) of token l&31) and scores 32 codewords
// at a time with v_mfma_f32_32x32x2_f32: score_k = ||c_k||^2 - 2 <res, c_k>.
// Candidates are visited in increasing k within a lane and merged with the
// partner half-wave preferring the lower index, so exact ties resolve to the
// lowest codeword index; NaN scores never compare smaller.
#include "common.h"
#include "internal.h"

namespace mapl {

constexpr int kRvqTilesPerWave = 2;

template <int W, typename ZT>
__global__ __launch_bounds__(256) void k_rvq_encode(const ZT* __restrict__ Z, const float* __restrict__ C,
                                                    int64_t stride, uint8_t* __restrict__ codes, int N, int r, int G,
                                                    int K, int R) {
  constexpr int H = W / 2;  // dims per lane (k steps of the 32x32x2 MFMA)
  extern __shared__ float sh[];
  float* cbT = sh;           // [W][K]
  float* nrm = sh + W * K;   // [K]
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int h = lane >> 5, l32 = lane & 31;
  const int g = blockIdx.x;
  const int tok_base = blockIdx.y * (4 * kRvqTilesPerWave * 32) + wave * (kRvqTilesPerWave * 32);

  float res[kRvqTilesPerWave][H];
#pragma unroll
  for (int t = 0; t < kRvqTilesPerWave; ++t) {
    const int n = tok_base + t * 32 + l32;
#pragma unroll
    for (int s = 0; s < H; ++s)
      res[t][s] = (n < N) ? to_f32<ZT>(Z[size_t(n) * r + g * W + h * H + s]) : 0.f;
  }

  for (int rho = 0; rho < R; ++rho) {
    if (rho == 0 || stride != 0) {
      __syncthreads();
      const float* book = C + rho * stride + size_t(g) * K * W;
      for (int e = threadIdx.x; e < K * W; e += 256) {
        const int k = e / W, j = e % W;
        cbT[j * K + k] = book[e];
      }
      __syncthreads();
      for (int k = threadIdx.x; k < K; k += 256) {
        float s2 = 0.f;
        for (int j = 0; j < W; ++j) s2 = fmaf(cbT[j * K + k], cbT[j * K + k], s2);
        nrm[k] = s2;
      }
      __syncthreads();
    }
#pragma unroll
    for (int t = 0; t < kRvqTilesPerWave; ++t) {
      float best = __builtin_inff();
      int bk = 0;
      for (int kb = 0; kb < K; kb += 32) {
        f32x16 acc = f32x16{};
#pragma unroll
        for (int s = 0; s < H; ++s) acc = mfma_f32_32x32x2(cbT[(h * H + s) * K + kb + l32], res[t][s], acc);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int k = kb + mfma32_row(v, h);
          const float sc = nrm[k] - 2.f * acc[v];
          if (sc < best) {
            best = sc;
            bk = k;
          }
        }
      }
      const float ob = __shfl_xor(best, 32);
      const int ok = __shfl_xor(bk, 32);
      if (ob < best || (ob == best && ok < bk)) {
        best = ob;
        bk = ok;
      }
      const int n = tok_base + t * 32 + l32;
      if (h == 0 && n < N) codes[(size_t(n) * R + rho) * G + g] = uint8_t(bk);
#pragma unroll
      for (int s = 0; s < H; ++s) res[t][s] -= cbT[(h * H + s) * K + bk];
    }
  }
}

template <int W>
static void rvq_encode_w(const void* Z, int z_bf16, const float* C, int64_t stride, uint8_t* codes, int N, int r,
                         int G, int K, int R, hipStream_t s) {
  const int tpb = 4 * kRvqTilesPerWave * 32;
  dim3 grid(G, (N + tpb - 1) / tpb);
  const size_t lds = (size_t(W) * K + K) * sizeof(float);
  if (z_bf16)
    hipLaunchKernelGGL((k_rvq_encode<W, bf16_t>), grid, dim3(256), lds, s, static_cast<const bf16_t*>(Z), C, stride,
                       codes, N, r, G, K, R);
  else
    hipLaunchKernelGGL((k_rvq_encode<W, float>), grid, dim3(256), lds, s, static_cast<const float*>(Z), C, stride,
                       codes, N, r, G, K, R);
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

// Decode: Zq[n][g*W + j] = sum_rho C[rho*stride + (g*K + code)*W + j], rounds in order.
template <typename OT>
__global__ __launch_bounds__(256) void k_rvq_decode(const uint8_t* __restrict__ codes, const float* __restrict__ C,
                                                    int64_t stride, OT* __restrict__ Zq, int N, int r, int G, int K,
                                                    int R) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= int64_t(N) * r) return;
  const int n = int(e / r), col = int(e % r);
  const int W = r / G;
  const int g = col / W, j = col % W;
  float acc = 0.f;
  for (int rho = 0; rho < R; ++rho) {
    const int k = codes[(size_t(n) * R + rho) * G + g];
    if (k < K) acc += C[rho * stride + (size_t(g) * K + k) * W + j];  // a code >= K (corrupt input) adds nothing
  }
  Zq[e] = from_f32<OT>(acc);
}

void launch_rvq_decode(const uint8_t* codes, const float* C, int64_t stride, void* Zq, int out_bf16, int N, int r,
                       int G, int K, int R, hipStream_t s) {
  const int64_t tot = int64_t(N) * r;
  dim3 grid(unsigned((tot + 255) / 256));
  if (out_bf16)
    hipLaunchKernelGGL(k_rvq_decode<bf16_t>, grid, dim3(256), 0, s, codes, C, stride, static_cast<bf16_t*>(Zq), N, r,
                       G, K, R);
  else
    hipLaunchKernelGGL(k_rvq_decode<float>, grid, dim3(256), 0, s, codes, C, stride, static_cast<float*>(Zq), N, r, G,
                       K, R);
}

// Stream apply: C[idx[q]*W + j] = vals[q*W + j]; a later duplicate of idx[q]
// in the same call wins, so an earlier one skips its write.
__global__ __launch_bounds__(256) void k_rvq_stream(float* __restrict__ C, const int32_t* __restrict__ idx,
                                                    const float* __restrict__ vals, int n, int W, int64_t total) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= int64_t(n) * W) return;
  const int q = int(e / W), j = int(e % W);
  const int64_t dst = idx[q];
  if (dst < 0 || dst >= total) return;
  for (int q2 = q + 1; q2 < n; ++q2)
    if (idx[q2] == dst) return;
  C[dst * W + j] = vals[e];
}

void launch_rvq_stream(float* C, const int32_t* idx, const float* vals, int n, int w, int64_t total_codewords,
                       hipStream_t s) {
  const int64_t tot = int64_t(n) * w;
  if (tot == 0) return;
  hipLaunchKernelGGL(k_rvq_stream, dim3(unsigned((tot + 255) / 256)), dim3(256), 0, s, C, idx, vals, n, w,
                     total_codewords);
}

}  // namespace mapl
