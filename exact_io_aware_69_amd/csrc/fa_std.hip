// Standard (materialised) attention on gfx950: the computation the IO-aware
// kernels replace, kept for comparison (Stanford FlashAttention summary:
// standard attention writes the N x N attention matrix to HBM and reads it
// back; FlashAttention-2 review, Abstract: its memory grows quadratically
// with sequence length). Three steps per call, on the caller's stream:
//   1. S = (Q K^T) * scale, fp32 [B*H][N][N]      (rocBLAS strided-batched GEMM)
//   2. P = row-softmax(masked S), bf16, and lse     (fa_std_softmax_kernel)
//   3. O = P V, bf16                                (rocBLAS strided-batched GEMM)
// The matrix products are plain library GEMMs; the masking and softmax are
// this file's kernel.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include "fa_device.h"
#include "fa_params.h"

namespace fa {

// One wave per score row, four rows per workgroup; each lane handles 4
// consecutive columns per 256-column chunk.

__device__ __forceinline__ bool std_visible(int i, int j, int N, bool causal, const uint8_t* mrow) {
  return j < N && (!causal || j <= i) && (!mrow || mrow[j / MASK_BLOCK] != 0);
}

// Row r = (bh, i) of S: keys j visible iff j < N, (causal) j <= i and (mask)
// the 128 x 128 block (i/128, j/128) of head h is kept. P = exp(S - m) / l on
// visible keys, 0 elsewhere; lse = m + ln l (-inf and P = 0 when no key is
// visible). Pass 1 keeps a running (max, sum) per lane, combined across the
// wave; pass 2 writes P.
__global__ __launch_bounds__(256) void fa_std_softmax_kernel(const float* __restrict__ S, uint16_t* __restrict__ P,
                                                             float* __restrict__ lse, const uint8_t* __restrict__ mask,
                                                             int H, int N, int nb, int causal, size_t rows) {
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int i = (int)(row % N);
  const int h = (int)((row / N) % H);
  const float* s = S + row * N;
  uint16_t* pr = P + row * N;
  const uint8_t* mrow = mask ? mask + ((size_t)h * nb + i / MASK_BLOCK) * nb : nullptr;
  const int jend = causal ? min(N, i + 1) : N;  // columns past jend are never visible
  // Rows are read and written 4 columns per lane when N is a multiple of 4
  // (16-byte aligned rows, no column past N); otherwise one column per lane.
  const bool vec = (N & 3) == 0;
  float m = -INFINITY, l = 0.f;
  auto accum = [&](float x) {
    if (x > m) {
      l = l * expf(m - x) + 1.f;
      m = x;
    } else {
      l += expf(x - m);
    }
  };
  if (vec) {
    for (int j0 = 4 * lane; j0 < jend; j0 += 256) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(s + j0);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (std_visible(i, j0 + e, N, causal, mrow)) accum(x[e]);
    }
  } else {
    for (int j = lane; j < jend; j += 64)
      if (std_visible(i, j, N, causal, mrow)) accum(s[j]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float mo = __shfl_xor(m, off), lo = __shfl_xor(l, off);
    const float mn = fmaxf(m, mo);
    if (mn != -INFINITY) l = (m == -INFINITY ? 0.f : l * expf(m - mn)) + (mo == -INFINITY ? 0.f : lo * expf(mo - mn));
    m = mn;
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  if (vec) {
    for (int j0 = 4 * lane; j0 < N; j0 += 256) {
      bf16x4 out;
      if (j0 < jend) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(s + j0);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          out[e] = (__bf16)(std_visible(i, j0 + e, N, causal, mrow) ? expf(x[e] - m) * inv : 0.f);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = (__bf16)0.f;
      }
      *reinterpret_cast<bf16x4*>(pr + j0) = out;
    }
  } else {
    for (int j = lane; j < N; j += 64) {
      const float pv = (j < jend && std_visible(i, j, N, causal, mrow)) ? expf(s[j] - m) * inv : 0.f;
      pr[j] = __builtin_bit_cast(uint16_t, (__bf16)pv);
    }
  }
  if (lane == 0) lse[row] = l > 0.f ? m + logf(l) : -INFINITY;
}

namespace {

// One rocBLAS handle per device, created on first use and kept for the
// life of the process.
rocblas_handle handle_for_current_device() {
  static std::mutex mu;
  static rocblas_handle handles[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!handles[dev] && rocblas_create_handle(&handles[dev]) != rocblas_status_success) handles[dev] = nullptr;
  return handles[dev];
}

}  // namespace

size_t std_workspace_bytes(int B, int H, int N) {
  const size_t nn = (size_t)B * H * N * N;
  const size_t s_bytes = (nn * 4 + 255) & ~(size_t)255;
  return s_bytes + ((nn * 2 + 255) & ~(size_t)255);
}

// Returns 0 on success, 1 for a rocBLAS failure, 2 for a HIP launch failure.
int std_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse, int B, int H, int N,
            int d, bool causal, float scale, const uint8_t* mask, void* workspace, hipStream_t st) {
  rocblas_handle hdl = handle_for_current_device();
  if (!hdl || rocblas_set_stream(hdl, st) != rocblas_status_success) return 1;
  const int BH = B * H;
  const size_t nn = (size_t)BH * N * N;
  float* S = static_cast<float*>(workspace);
  uint16_t* P = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(workspace) + ((nn * 4 + 255) & ~(size_t)255));
  // Column-major view: S^T = K Q^T, i.e. element (key, query) of a column-
  // major N x N matrix, which is row-major S[query][key].
  const float alpha = scale, beta = 0.f;
  rocblas_status rs = rocblas_gemm_strided_batched_ex(
      hdl, rocblas_operation_transpose, rocblas_operation_none, N, N, d, &alpha, k, rocblas_datatype_bf16_r, d,
      (rocblas_stride)N * d, q, rocblas_datatype_bf16_r, d, (rocblas_stride)N * d, &beta, S, rocblas_datatype_f32_r, N,
      (rocblas_stride)N * N, S, rocblas_datatype_f32_r, N, (rocblas_stride)N * N, BH, rocblas_datatype_f32_r,
      rocblas_gemm_algo_standard, 0, 0);
  if (rs != rocblas_status_success) return 1;
  const int nb = (N + MASK_BLOCK - 1) / MASK_BLOCK;
  const size_t rows = (size_t)BH * N;
  hipLaunchKernelGGL(fa_std_softmax_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, S, P, lse, mask, H, N,
                     nb, causal ? 1 : 0, rows);
  if (hipGetLastError() != hipSuccess) return 2;
  // O^T = V^T P^T in the column-major view: a d x N result, row-major O.
  const float one = 1.f;
  rs = rocblas_gemm_strided_batched_ex(hdl, rocblas_operation_none, rocblas_operation_none, d, N, N, &one, v,
                                       rocblas_datatype_bf16_r, d, (rocblas_stride)N * d, P, rocblas_datatype_bf16_r,
                                       N, (rocblas_stride)N * N, &beta, o, rocblas_datatype_bf16_r, d,
                                       (rocblas_stride)N * d, o, rocblas_datatype_bf16_r, d, (rocblas_stride)N * d, BH,
                                       rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  return rs == rocblas_status_success ? 0 : 1;
}

}  // namespace fa
