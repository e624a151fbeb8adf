// Rank-r map of an expert's down matrix, built on the device in fp64 for large
// shapes (page "KAIST drops calibration from MoE decoding, speeds up blocks by
// up to 2.69x over vLLM", section "A reader built from weights alone": the
// compensation of skipped channels is a low-rank map built from the weights).
//
// P Q^T is the best rank-r approximation of W = W_down [d][m], from the top-r
// eigenvectors of the smaller Gram matrix. The O(n^3) work runs here: the Gram
// matrix, the Householder tridiagonalisation (one symmetric matrix-vector
// product and one rank-2 update per step, as in Golub & Van Loan) and the
// projection that forms the other factor. The tridiagonal eigen-solve and the
// back-transformation are the host code shared with the host path.
//
// Arithmetic is fp64 without contraction, so the symmetric update keeps the
// matrix exactly symmetric; every reduction has a fixed order.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <string>
#include <vector>

#include "internal.h"

#pragma clang fp contract(off)

namespace moe_sel {
namespace {

__device__ __forceinline__ double bf(uint16_t b) { return (double)__uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ double wave_sum_d(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// block sum over 1024 threads in a fixed order; every thread gets the result
__device__ double block_sum_1024(double v, double* s_w) {
  v = wave_sum_d(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) s_w[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < 16; ++w) t += s_w[w];
  __syncthreads();
  return t;
}

// C[i][j] = sum_k X(k, i) X(k, j) with X(k, i) = x[k * sk + i * si] (bf16).
// 64 x 64 output tile per block, 4 x 4 per thread, K in chunks of 16.
__global__ __launch_bounds__(256) void k_gram(const uint16_t* x, long sk, long si, int K, int n, double* C) {
  __shared__ double sa[16][65], sb[16][65];
  const int bi = blockIdx.y * 64, bj = blockIdx.x * 64;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  double acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q, kk = e >> 6, ii = e & 63;
      const int k = k0 + kk;
      sa[kk][ii] = (k < K && bi + ii < n) ? bf(x[(size_t)k * sk + (size_t)(bi + ii) * si]) : 0.0;
      sb[kk][ii] = (k < K && bj + ii < n) ? bf(x[(size_t)k * sk + (size_t)(bj + ii) * si]) : 0.0;
    }
    __syncthreads();
    for (int kk = 0; kk < 16; ++kk) {
      double a[4], b[4];
      for (int u = 0; u < 4; ++u) {
        a[u] = sa[kk][4 * ty + u];
        b[u] = sb[kk][4 * tx + u];
      }
      for (int u = 0; u < 4; ++u)
        for (int v = 0; v < 4; ++v) acc[u][v] += a[u] * b[v];
    }
    __syncthreads();
  }
  for (int u = 0; u < 4; ++u)
    for (int v = 0; v < 4; ++v) {
      const int i = bi + 4 * ty + u, j = bj + 4 * tx + v;
      if (i < n && j < n) C[(size_t)i * n + j] = acc[u][v];
    }
}

// Householder vector of step k from row k right of the diagonal, stored in place.
__global__ __launch_bounds__(1024) void k_house(double* A, int n, int k, double* off, double* beta) {
  __shared__ double s_w[16];
  __shared__ double s_x0;
  const int len = n - k - 1;
  double* v = A + (size_t)k * n + k + 1;
  double s = 0.0;
  for (int i = threadIdx.x; i < len; i += 1024) s += v[i] * v[i];
  const double xnorm2 = block_sum_1024(s, s_w);
  const double xnorm = sqrt(xnorm2);
  if (xnorm == 0.0) {
    if (threadIdx.x == 0) {
      off[k] = 0.0;
      beta[k] = 0.0;
    }
    return;
  }
  if (threadIdx.x == 0) {
    const double x0 = v[0];
    const double alpha = x0 > 0 ? -xnorm : xnorm;
    v[0] = x0 - alpha;
    s_x0 = alpha;
  }
  __syncthreads();
  s = 0.0;
  for (int i = threadIdx.x; i < len; i += 1024) s += v[i] * v[i];
  const double vnorm2 = block_sum_1024(s, s_w);
  if (threadIdx.x == 0) {
    off[k] = s_x0;
    beta[k] = 2.0 / vnorm2;
  }
}

// p = beta * A22 v, one wave per row of the trailing matrix
__global__ __launch_bounds__(256) void k_symv(const double* A, int n, int k, const double* beta, double* p) {
  const double bt = beta[k];
  if (bt == 0.0) return;
  const int len = n - k - 1;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= len) return;
  const double* v = A + (size_t)k * n + k + 1;
  const double* arow = A + (size_t)(k + 1 + row) * n + k + 1;
  double s = 0.0;
  for (int j = lane; j < len; j += 64) s += arow[j] * v[j];
  s = wave_sum_d(s);
  if (lane == 0) p[row] = bt * s;
}

// w = p - (beta / 2) (p . v) v
__global__ __launch_bounds__(1024) void k_wvec(const double* A, int n, int k, const double* beta, const double* p,
                                               double* w) {
  __shared__ double s_w[16];
  const double bt = beta[k];
  if (bt == 0.0) return;
  const int len = n - k - 1;
  const double* v = A + (size_t)k * n + k + 1;
  double s = 0.0;
  for (int i = threadIdx.x; i < len; i += 1024) s += p[i] * v[i];
  const double K = 0.5 * bt * block_sum_1024(s, s_w);
  for (int i = threadIdx.x; i < len; i += 1024) w[i] = p[i] - K * v[i];
}

// A22 -= v w^T + w v^T
__global__ __launch_bounds__(256) void k_rank2(double* A, int n, int k, const double* beta, const double* w) {
  if (beta[k] == 0.0) return;
  const int len = n - k - 1;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= len) return;
  const double* v = A + (size_t)k * n + k + 1;
  const double vj = v[j], wj = w[j];
  for (int i = blockIdx.y; i < len; i += gridDim.y) {
    double* arow = A + (size_t)(k + 1 + i) * n + k + 1;
    arow[j] -= v[i] * wj + w[i] * vj;
  }
}

// out[j][c] = sum_i X(j, i) U[i][c] with X(j, i) = x[j * sj + i * si] (bf16),
// U n x r (fp64, row-major); one 64-thread block per j, threads over c.
__global__ __launch_bounds__(64) void k_project(const uint16_t* x, long sj, long si, int len, const double* U, int r,
                                                double* out) {
  const int j = blockIdx.x;
  for (int c = threadIdx.x; c < r; c += 64) {
    double s = 0.0;
    for (int i = 0; i < len; ++i) s += bf(x[(size_t)j * sj + (size_t)i * si]) * U[(size_t)i * r + c];
    out[(size_t)j * r + c] = s;
  }
}

struct DevBuf {
  void* p = nullptr;
  ~DevBuf() {
    if (p) (void)hipFree(p);
  }
};

}  // namespace

std::string lowrank_map_device(const uint16_t* wch_dev, int d, int m, int r, uint16_t* p_out, uint16_t* q_out,
                               void* stream) {
  if (r <= 0) return std::string();
  hipStream_t s = (hipStream_t)stream;
  const int n = m <= d ? m : d;
  // W [d][m]: element (i, j) = down column j at row i = wch[j * 3d + 2d + i]
  const uint16_t* wd = wch_dev + 2 * (size_t)d;
  const long cstride = 3L * d;  // between channels
  DevBuf bA, bp, bw, boff, bbeta, bU, bout;
  const size_t nn = (size_t)n * n;
  hipError_t e = hipMalloc(&bA.p, nn * sizeof(double));
  if (e == hipSuccess) e = hipMalloc(&bp.p, (size_t)n * sizeof(double));
  if (e == hipSuccess) e = hipMalloc(&bw.p, (size_t)n * sizeof(double));
  if (e == hipSuccess) e = hipMalloc(&boff.p, (size_t)n * sizeof(double));
  if (e == hipSuccess) e = hipMalloc(&bbeta.p, (size_t)n * sizeof(double));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return std::string("device low-rank workspace: ") + hipGetErrorString(e);
  }
  double* A = (double*)bA.p;
  double* p = (double*)bp.p;
  double* w = (double*)bw.p;
  double* off = (double*)boff.p;
  double* beta = (double*)bbeta.p;
  // Gram matrix of the smaller side
  const dim3 gg((n + 63) / 64, (n + 63) / 64);
  if (m <= d)  // G = W^T W: (a, b) = sum_i W[i][a] W[i][b]; X(k = i, a) = wd[i + a * cstride]
    hipLaunchKernelGGL(k_gram, gg, dim3(256), 0, s, wd, 1L, cstride, d, n, A);
  else  // G = W W^T: (a, b) = sum_j W[a][j] W[b][j]; X(k = j, a) = wd[j * cstride + a]
    hipLaunchKernelGGL(k_gram, gg, dim3(256), 0, s, wd, cstride, 1L, m, n, A);
  for (int k = 0; k + 2 < n; ++k) {
    const int len = n - k - 1;
    hipLaunchKernelGGL(k_house, dim3(1), dim3(1024), 0, s, A, n, k, off, beta);
    hipLaunchKernelGGL(k_symv, dim3((len + 3) / 4), dim3(256), 0, s, (const double*)A, n, k, (const double*)beta, p);
    hipLaunchKernelGGL(k_wvec, dim3(1), dim3(1024), 0, s, (const double*)A, n, k, (const double*)beta,
                       (const double*)p, w);
    const int rows = len < 256 ? len : 256;
    hipLaunchKernelGGL(k_rank2, dim3((len + 255) / 256, rows), dim3(256), 0, s, A, n, k, (const double*)beta,
                       (const double*)w);
  }
  if ((e = hipGetLastError()) != hipSuccess) return std::string("device tridiagonalisation: ") + hipGetErrorString(e);
  Tridiag T;
  std::vector<double> hA(nn);
  T.off.assign(n > 1 ? n - 1 : 0, 0.0);
  T.beta.assign(n > 2 ? n - 2 : 0, 0.0);
  T.diag.assign(n, 0.0);
  e = hipMemcpyAsync(hA.data(), A, nn * sizeof(double), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess && n > 2) e = hipMemcpyAsync(T.off.data(), off, (size_t)(n - 2) * sizeof(double), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess && n > 2) e = hipMemcpyAsync(T.beta.data(), beta, (size_t)(n - 2) * sizeof(double), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return std::string("device low-rank copy: ") + hipGetErrorString(e);
  for (int i = 0; i < n; ++i) T.diag[i] = hA[(size_t)i * n + i];
  if (n >= 2) T.off[n - 2] = hA[(size_t)(n - 1) * n + (n - 2)];
  std::vector<double> vecs, vals;
  eigvecs_from_tridiag(hA.data(), n, r, T, vecs, vals);  // n x r
  hA.clear();
  hA.shrink_to_fit();
  // the other factor: m <= d: P[c][i] = sum_j W[i][j] V[j][c]; else Q[j][c] = sum_i W[i][j] U[i][c]
  const int other = m <= d ? d : m;
  e = hipMalloc(&bU.p, vecs.size() * sizeof(double));
  if (e == hipSuccess) e = hipMalloc(&bout.p, (size_t)other * r * sizeof(double));
  if (e == hipSuccess) e = hipMemcpyAsync(bU.p, vecs.data(), vecs.size() * sizeof(double), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return std::string("device low-rank projection: ") + hipGetErrorString(e);
  }
  if (m <= d)  // row i of W: X(i, j) = wd[i + j * cstride], len = m
    hipLaunchKernelGGL(k_project, dim3(d), dim3(64), 0, s, wd, 1L, cstride, m, (const double*)bU.p, r,
                       (double*)bout.p);
  else  // column j of W: X(j, i) = wd[j * cstride + i], len = d
    hipLaunchKernelGGL(k_project, dim3(m), dim3(64), 0, s, wd, cstride, 1L, d, (const double*)bU.p, r,
                       (double*)bout.p);
  std::vector<double> proj((size_t)other * r);
  e = hipGetLastError();
  if (e == hipSuccess) e = hipMemcpyAsync(proj.data(), bout.p, proj.size() * sizeof(double), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return std::string("device low-rank projection: ") + hipGetErrorString(e);
  if (m <= d) {
    for (int j = 0; j < m; ++j)
      for (int c = 0; c < r; ++c) q_out[(size_t)j * r + c] = f32_to_bf16((float)vecs[(size_t)j * r + c]);
    for (int c = 0; c < r; ++c)
      for (int i = 0; i < d; ++i) p_out[(size_t)c * d + i] = f32_to_bf16((float)proj[(size_t)i * r + c]);
  } else {
    for (int c = 0; c < r; ++c)
      for (int i = 0; i < d; ++i) p_out[(size_t)c * d + i] = f32_to_bf16((float)vecs[(size_t)i * r + c]);
    for (int j = 0; j < m; ++j)
      for (int c = 0; c < r; ++c) q_out[(size_t)j * r + c] = f32_to_bf16((float)proj[(size_t)j * r + c]);
  }
  return std::string();
}

}  // namespace moe_sel
