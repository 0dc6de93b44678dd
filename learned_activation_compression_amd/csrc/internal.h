// Host-side launchers of the MAPL kernels.  Each launcher assumes its
// arguments were validated by the C ABI layer and only enqueues work.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"
#include <stddef.h>
#include <stdint.h>

namespace mapl {

// ---- packed weights (bf16, fragment order; see pack.hip):
//   AtF = A^T (r x d), AF = A (d x r), PtF = P^T (d x r), QnF = -(P A)^T (r x r),
//   PF = P (r x d)
struct PackView {
  uint16_t* AtF;
  uint16_t* AF;
  uint16_t* PtF;
  uint16_t* QnF;
  uint16_t* PF;
};
size_t pack_bytes_bf16(int64_t d, int64_t r, int64_t ra);
PackView pack_view(void* pk, int64_t d, int64_t r, int64_t ra);
void launch_pack_AtF(const uint16_t* A, uint16_t* AtF, int d, int r, hipStream_t s);
void launch_pack_AF(const uint16_t* A, uint16_t* AF, int d, int r, hipStream_t s);
void launch_pack_PtF(const uint16_t* P, uint16_t* PtF, int d, int ra, hipStream_t s);
void launch_pack_PF(const uint16_t* P, uint16_t* PF, int d, int ra, hipStream_t s);
// all five sections; P == nullptr with ra > 0 packs the identity anchor (QnF = -AtF)
void launch_pack_all(const uint16_t* P, const uint16_t* A, PackView v, int d, int r, int ra, hipStream_t s);

// ---- bf16 codec
// out[N][r] = in[N][d] A  (- E[tids] (P A)) via AtF and QnF; E [V][ra]; E == nullptr or
// ra == 0 drops the anchor term
void launch_tok_reduce_bf16(const uint16_t* in, const uint16_t* AtF, const int32_t* tids,
                            const uint16_t* E, const uint16_t* QnF, uint16_t* out,
                            int N, int d, int r, int ra, int V, hipStream_t s, KernelEvents ev = {});
// U[N][r] = alpha * in[N][d] W^T with W's fragments F (M = r, K = d), fp32 rows, and
// the max |U| of each output wave in part[4 * (N / 64 block) + wave]; covers r = 128
// and 256 (returns false, launching nothing, otherwise)
bool launch_tok_reduce_f32out(const uint16_t* in, const uint16_t* F, float* U, float alpha, float* part, int N,
                              int d, int r, hipStream_t s);
// out[N][d] = in[N][r] A^T (+ E[tids] P) via AF and PtF; E [V][ra]; E == nullptr or ra == 0
// drops the anchor term.  Returns false, launching nothing, for shapes no kernel covers
// (an anchor rank other than r needs r and ra multiples of 64).
bool launch_tok_expand_bf16(const uint16_t* in, const uint16_t* AF, const int32_t* tids,
                            const uint16_t* E, const uint16_t* PtF, uint16_t* out,
                            int N, int d, int r, int ra, int V, hipStream_t s);
// token-split partial Gram: part[s][i][j] = sum_{n in split s} L[n][i] R[n][j] for
// i < Ld + Le, j < Rd.  Row i < Ld of L is in[n][i] (in [N][ldin]); row Ld + q is
// E[tids[n]][q] (zero for an invalid id).  R is [N][Rd].  part is [splits][Ld + Le][Rd].
int gram_splits_bf16(int N, int rows, int Rd);
void launch_gram_bf16(const uint16_t* in, int64_t ldin, int Ld, const int32_t* tids, int V, const uint16_t* E,
                      int Le, const uint16_t* R, int Rd, float* part, int N, int splits, hipStream_t s);
// fixed-order split sums: e < n0 -> out0[e] (+= when acc0), else out1[e - n0];
// split k of element e at part[k * stride + e]; n0, n1, stride multiples of 4
void launch_reduce_partials(const float* part, int splits, int64_t stride, float* out0, int64_t n0, int acc0,
                            float* out1, int64_t n1, hipStream_t s);
// gA[i][j] -= sum_k P[k][i] M[k][j]  (P bf16 [ra][d], M fp32 [ra][r], gA fp32 [d][r]);
// P == nullptr is the identity (ra == d): gA -= M
void launch_sub_ptm(const uint16_t* P, const float* M, float* gA, int d, int r, int ra, hipStream_t s);

// token GEMM out[N][C] = [src | E[t]] W with W from the packs F1 (k < K1) and F2
// (anchor rows, K2 of them; E == nullptr or K2 == 0 drops them).  Returns false,
// launching nothing, for shapes it does not cover (K1, K2 % 64, C % 128).
bool launch_tok_gemm_bf16(const uint16_t* src, int K1, const int32_t* tids, int V, const uint16_t* E, int K2,
                          const uint16_t* F1, const uint16_t* F2, uint16_t* out, int N, int C, hipStream_t s);
// out[N][d] = in[N][r] A^T + E[t] with E [V][d] (the full-rank anchor), one rounding; r % 64 == 0
bool launch_tok_expand_eadd_bf16(const uint16_t* in, const uint16_t* AF, const int32_t* tids, const uint16_t* E,
                                 uint16_t* out, int N, int d, int r, int V, hipStream_t s);
// the token GEMM form of the same: out[N][C] = src[N][K1] W + E[t] with E [V][C], one rounding
bool launch_tok_gemm_eadd_bf16(const uint16_t* src, int K1, const int32_t* tids, int V, const uint16_t* E,
                               const uint16_t* F1, uint16_t* out, int N, int C, hipStream_t s);

// ---- fp32 codec (small problems, plain fp32 arithmetic); anchor E [V][ra], P [ra][d]
// (P == nullptr with ra == d: the identity anchor, E[t] itself)
void launch_compress_f32(const float* X, const int32_t* tids, const float* E, const float* P,
                         const float* A, float* Z, int N, int d, int r, int ra, int V, hipStream_t s);
void launch_residual_f32(const float* X, const int32_t* tids, const float* E, const float* P,
                         float* R, int N, int d, int ra, int V, hipStream_t s);
void launch_reconstruct_f32(const float* Z, const int32_t* tids, const float* E, const float* P,
                            const float* A, float* Xh, int N, int d, int r, int ra, int V, hipStream_t s);
void launch_rowmap_f32(const float* in, const float* A, float* out, int N, int d, int r,
                       int transposeA, hipStream_t s);
void launch_outer_f32(const float* L, const float* R, float* gA, int N, int d, int r,
                      int accumulate, hipStream_t s);

void launch_fill_f32(float* p, int64_t count, float value, hipStream_t s);
void launch_check_tids(const int32_t* tids, int N, int V, int32_t* bad, hipStream_t s);

// anchor-table gradient: workspace (projected rows, partial maxima) and the two
// launches (project, own); PF (P's fragment pack) may be nullptr; P == nullptr is
// the identity projection (r == d: the rows alpha Y themselves)
size_t anchor_grad_ws_bytes(int64_t N, int64_t r, int64_t V);
void launch_anchor_grad(const void* Y, int y_bf16, const int32_t* tids, const void* P, const uint16_t* PF,
                        float* gE, float alpha, int accumulate, int N, int d, int r, int V, void* ws, hipStream_t s);

// ---- residual VQ
void launch_rvq_encode(const void* Z, int z_bf16, const float* C, int64_t stride,
                       uint8_t* codes, int N, int r, int G, int K, int R, hipStream_t s);
void launch_rvq_decode(const uint8_t* codes, const float* C, int64_t stride, void* Zq, int out_bf16,
                       int N, int r, int G, int K, int R, hipStream_t s);
void launch_rvq_stream(float* C, const int32_t* idx, const float* vals, int n, int w,
                       int64_t total_codewords, hipStream_t s);
void launch_rvq_stream_decode(float* C, int64_t stride, int64_t total, const int32_t* idx, const float* vals, int n,
                              const uint8_t* codes, void* Zq, int out_bf16, int N, int r, int G, int K, int R,
                              hipStream_t s);

// ---- SPEL
size_t spel_ws_bytes(int64_t d, int64_t r);
// Polar Express: the greedy minimax odd-quintic schedule from [ell, 1] (coef [steps][3],
// err [steps] or nullptr; returns 0, or -1 if a step is not finite), and the SPEL step
// that uses it for both polar maps (fp32 coefficients [steps][3])
int polar_express_schedule(double ell, int steps, double* coef, double* err);
// status (device int, optional): 0 when the step was committed, 1 when a wait
// between workgroups timed out and A and m were left as they were
void launch_spel_pe(float* A, const float* g, float* m, float alpha, float beta, const float* coef_lmo, int lmo_steps,
                    const float* coef_ret, int ret_steps, float* D_out, int* status, int d, int r, void* ws,
                    hipStream_t s);
void launch_spel(float* A, const float* g, float* m, float alpha, float beta, int ns_iters,
                 float* D_out, int* status, int d, int r, void* ws, hipStream_t s);

}  // namespace mapl
