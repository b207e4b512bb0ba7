// MFMA GEMM used by the SO(2) convolution (forward) and its backward.
//
//   C[m][n] (+)= sum_k A(m,k) B(n,k)
// A(m,k) = A[m*lda + k] when a_kcontig, else A[k*lda + m]; B likewise.
// C is fp32 [M][ldc].  With splits > 1 the K range is cut into `splits`
// slices and slice z writes its partial product to C + z*split_stride
// (reduced afterwards in a fixed order, so results are deterministic).
#pragma once

#include "common.h"

namespace egnn {

hipError_t gemm_f32(int M, int N, int K, const float *A, int lda, bool a_kcontig, const float *B, int ldb,
                    bool b_kcontig, float *C, int ldc, int splits, int64_t split_stride, hipStream_t stream);

// Complex product by three real products (see gemm.hip):
//   Cre + i Cim = sum_k (U+ + i U-)(m,k) (V+ + i V-)(n,k),  m < M, n < N.
// U+/U- at Up/Um (same layout, ldu).  If V3 is given, V1 = V+, V2 = V- - V+,
// V3 = V+ + V- are precomputed; otherwise V+ = V1 and V- = vsign * V2.
// Supported layouts: (U, V) K-contiguous with precomputed V; U K-contiguous,
// V not, precomputed; neither K-contiguous with V from data.  Split-K as gemm_f32.
hipError_t cgemm_f32(int M, int N, int K, const float *Up, const float *Um, int ldu, bool u_kcontig, const float *V1,
                     const float *V2, const float *V3, int ldv, bool v_kcontig, float vsign, float *Cre, float *Cim,
                     int ldc, int splits, int64_t split_stride, hipStream_t stream);

// Output tiles of gemm_f32 / cgemm_f32 for an M x N result (their tile widths
// are chosen per dimension), and of gemm_bf16_tn_splitk.
int gemm_f32_tiles(int M, int N);
int gemm_bf16_tn_tiles(int M, int N);

// Workgroups of the split-K weight-gradient kernels that one CU holds at once
// (the runtime's occupancy figure for the instantiation that the shape
// selects; at least 1): gemm_f32 and cgemm_f32 with neither operand
// K-contiguous (cgemm with V from data), and gemm_bf16_tn_splitk.
int gemm_f32_tn_blocks_per_cu(int M, int N);
int cgemm_f32_dw_blocks_per_cu(int M, int N);
int gemm_bf16_tn_blocks_per_cu();
// CUs per XCD of the current device (its CU count / 8).
int xcd_cus();

// bf16 operands (raw 16-bit), fp32 accumulate; both operands K-contiguous.
// C is written as bf16 when c_bf16, else fp32.
hipError_t gemm_bf16_nt(int M, int N, int K, const uint16_t *A, int lda, const uint16_t *B, int ldb, void *C,
                        int ldc, bool c_bf16, hipStream_t stream);

// Split-K form of gemm_bf16_nt with fp32 output: slice z of C (at C + z *
// split_stride) holds the product over the z-th K range.  K % 32 == 0.
hipError_t gemm_bf16_nt_splitk(int M, int N, int K, const uint16_t *A, int lda, const uint16_t *B, int ldb, float *C,
                               int ldc, int splits, int64_t split_stride, hipStream_t stream);

// Split-K product over the rows of two row-major bf16 matrices: slice z of C
// (at C + z * split_stride, row stride ldc) is C_z[m][n] = sum over the z-th
// range of k of P[k][m] * Q[k][n], P [K][M] (row stride ldp), Q [K][N] (row
// stride ldq), fp32 accumulate and output.  No transpose pass: the operands go
// to LDS as they lie and are read with gfx950's transposing LDS loads.
// M, N, ldp, ldq multiples of 8, P and Q 16-byte aligned.
hipError_t gemm_bf16_tn_splitk(int M, int N, int K, const uint16_t *P, int ldp, const uint16_t *Q, int ldq, float *C,
                               int ldc, int splits, int64_t split_stride, hipStream_t stream);

}  // namespace egnn
