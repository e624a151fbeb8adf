// Rank-r maps of the experts' down matrices, built on the device in fp64 (page
// "KAIST drops calibration from MoE decoding, speeds up blocks by up to 2.69x
// over vLLM", section "A reader built from weights alone": the compensation of
// skipped channels is a low-rank map built from the weights).
//
// P Q^T is the best rank-r approximation of W = W_down [d][m], from the top-r
// eigenvectors of the smaller Gram matrix. The O(n^3) work runs here for a batch
// of experts at once (one launch per step covers every expert of the batch):
// the Gram matrices, the Householder tridiagonalisation (one symmetric
// matrix-vector product and one rank-2 update per step, as in Golub & Van Loan)
// and the projection that forms the other factor. The tridiagonal eigen-solves
// and back-transformations are the host code shared with the host path, run in
// parallel over the experts.
//
// Arithmetic is fp64 without contraction, so the symmetric update keeps each
// matrix exactly symmetric; every reduction has a fixed order.
#include <hip/hip_runtime.h>

#include <algorithm>
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

// Expert z of the batch: C_z[i][j] = sum_k X(k, i) X(k, j), X(k, i) = x_z[k * sk + i * si]
// (bf16), x_z = x + z * xe. 64 x 64 output tile per block, 4 x 4 per thread.
__global__ __launch_bounds__(256) void k_gram(const uint16_t* x, size_t xe, long sk, long si, int K, int n,
                                              double* C) {
  __shared__ double sa[16][65], sb[16][65];
  const uint16_t* xz = x + blockIdx.z * xe;
  double* Cz = C + (size_t)blockIdx.z * n * n;
  const int bi = blockIdx.y * 64, bj = blockIdx.x * 64;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  double acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q, kk = e >> 6, ii = e & 63;
      const int k = k0 + kk;
      sa[kk][ii] = (k < K && bi + ii < n) ? bf(xz[(size_t)k * sk + (size_t)(bi + ii) * si]) : 0.0;
      sb[kk][ii] = (k < K && bj + ii < n) ? bf(xz[(size_t)k * sk + (size_t)(bj + ii) * si]) : 0.0;
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
      if (i < n && j < n) Cz[(size_t)i * n + j] = acc[u][v];
    }
}

// Householder vector of step k from row k right of the diagonal, stored in place.
// One block per expert (blockIdx.x).
__global__ __launch_bounds__(1024) void k_house(double* A, int n, int k, double* off, double* beta) {
  __shared__ double s_w[16];
  __shared__ double s_alpha;
  double* Az = A + (size_t)blockIdx.x * n * n;
  const int len = n - k - 1;
  double* v = Az + (size_t)k * n + k + 1;
  double s = 0.0;
  for (int i = threadIdx.x; i < len; i += 1024) s += v[i] * v[i];
  const double xnorm = sqrt(block_sum_1024(s, s_w));
  if (xnorm == 0.0) {
    if (threadIdx.x == 0) {
      off[(size_t)blockIdx.x * n + k] = 0.0;
      beta[(size_t)blockIdx.x * n + k] = 0.0;
    }
    return;
  }
  if (threadIdx.x == 0) {
    const double x0 = v[0];
    const double alpha = x0 > 0 ? -xnorm : xnorm;
    v[0] = x0 - alpha;
    s_alpha = alpha;
  }
  __syncthreads();
  s = 0.0;
  for (int i = threadIdx.x; i < len; i += 1024) s += v[i] * v[i];
  const double vnorm2 = block_sum_1024(s, s_w);
  if (threadIdx.x == 0) {
    off[(size_t)blockIdx.x * n + k] = s_alpha;
    beta[(size_t)blockIdx.x * n + k] = 2.0 / vnorm2;
  }
}

// p = beta * A22 v, one wave per row of the trailing matrix; expert blockIdx.y
__global__ __launch_bounds__(256) void k_symv(const double* A, int n, int k, const double* beta, double* p) {
  const size_t z = blockIdx.y;
  const double bt = beta[z * n + k];
  if (bt == 0.0) return;
  const int len = n - k - 1;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= len) return;
  const double* Az = A + z * n * n;
  const double* v = Az + (size_t)k * n + k + 1;
  const double* arow = Az + (size_t)(k + 1 + row) * n + k + 1;
  double s = 0.0;
  for (int j = lane; j < len; j += 64) s += arow[j] * v[j];
  s = wave_sum_d(s);
  if (lane == 0) p[z * n + row] = bt * s;
}

// w = p - (beta / 2) (p . v) v; one block per expert
__global__ __launch_bounds__(1024) void k_wvec(const double* A, int n, int k, const double* beta, const double* p,
                                               double* w) {
  __shared__ double s_w[16];
  const size_t z = blockIdx.x;
  const double bt = beta[z * n + k];
  if (bt == 0.0) return;
  const int len = n - k - 1;
  const double* v = A + z * n * n + (size_t)k * n + k + 1;
  const double* pz = p + z * n;
  double* wz = w + z * n;
  double s = 0.0;
  for (int i = threadIdx.x; i < len; i += 1024) s += pz[i] * v[i];
  const double K = 0.5 * bt * block_sum_1024(s, s_w);
  for (int i = threadIdx.x; i < len; i += 1024) wz[i] = pz[i] - K * v[i];
}

// A22 -= v w^T + w v^T; expert blockIdx.z
__global__ __launch_bounds__(256) void k_rank2(double* A, int n, int k, const double* beta, const double* w) {
  const size_t z = blockIdx.z;
  if (beta[z * n + k] == 0.0) return;
  const int len = n - k - 1;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= len) return;
  double* Az = A + z * n * n;
  const double* v = Az + (size_t)k * n + k + 1;
  const double* wz = w + z * n;
  const double vj = v[j], wj = wz[j];
  for (int i = blockIdx.y; i < len; i += gridDim.y) {
    double* arow = Az + (size_t)(k + 1 + i) * n + k + 1;
    arow[j] -= v[i] * wj + wz[i] * vj;
  }
}

// Expert z: out_z[j][c] = sum_i X(j, i) U_z[i][c], X(j, i) = x_z[j * sj + i * si]
// (bf16), U_z len x r (fp64, row-major); one 64-thread block per (j, z).
__global__ __launch_bounds__(64) void k_project(const uint16_t* x, size_t xe, long sj, long si, int len,
                                                const double* U, int r, int rows, double* out) {
  const size_t z = blockIdx.y;
  const int j = blockIdx.x;
  const uint16_t* xz = x + z * xe;
  const double* Uz = U + z * (size_t)len * r;
  for (int c = threadIdx.x; c < r; c += 64) {
    double s = 0.0;
    for (int i = 0; i < len; ++i) s += bf(xz[(size_t)j * sj + (size_t)i * si]) * Uz[(size_t)i * r + c];
    out[(z * rows + j) * r + c] = s;
  }
}

struct DevBuf {
  void* p = nullptr;
  ~DevBuf() {
    if (p) (void)hipFree(p);
  }
};

struct EigJob {
  const std::vector<double>* A;
  const std::vector<double>* off;
  const std::vector<double>* beta;
  std::vector<double>* vecs;  // [nb][n][r]
  int n, r;
};

void eig_one(int z, void* arg) {
  EigJob* j = (EigJob*)arg;
  const int n = j->n, r = j->r;
  const double* Az = j->A->data() + (size_t)z * n * n;
  Tridiag T;
  T.diag.resize(n);
  T.off.assign(n > 1 ? n - 1 : 0, 0.0);
  T.beta.assign(n > 2 ? n - 2 : 0, 0.0);
  for (int k = 0; k + 2 < n; ++k) {
    T.off[k] = (*j->off)[(size_t)z * n + k];
    T.beta[k] = (*j->beta)[(size_t)z * n + k];
  }
  for (int i = 0; i < n; ++i) T.diag[i] = Az[(size_t)i * n + i];
  if (n >= 2) T.off[n - 2] = Az[(size_t)(n - 1) * n + (n - 2)];
  std::vector<double> vecs, vals;
  eigvecs_from_tridiag(Az, n, r, T, vecs, vals);
  std::copy(vecs.begin(), vecs.end(), j->vecs->begin() + (size_t)z * n * r);
}

}  // namespace

std::string lowrank_maps_device(const uint16_t* wch_dev, int n_experts, int d, int m, int r, uint16_t* p_out,
                                uint16_t* q_out, void* stream) {
  if (r <= 0 || n_experts <= 0) return std::string();
  hipStream_t s = (hipStream_t)stream;
  const int n = m <= d ? m : d;
  const int other = m <= d ? d : m;
  // W_e [d][m]: element (i, j) = down column j at row i = wch_e[j * 3d + 2d + i]
  const size_t xe = (size_t)m * 3 * d;  // between experts
  const long cstride = 3L * d;          // between channels
  const size_t nn = (size_t)n * n;
  // experts per batch: at most 1 GiB of fp64 matrices
  const int nb = (int)std::max<size_t>(1, std::min<size_t>((size_t)n_experts, ((size_t)1 << 30) / (nn * 8)));
  DevBuf bA, bp, bw, boff, bbeta, bU, bout;
  auto dmalloc = [](void** q, size_t bytes) { return (hipError_t)checked_device_malloc(q, bytes); };
  hipError_t e = dmalloc(&bA.p, (size_t)nb * nn * sizeof(double));
  if (e == hipSuccess) e = dmalloc(&bp.p, (size_t)nb * n * sizeof(double));
  if (e == hipSuccess) e = dmalloc(&bw.p, (size_t)nb * n * sizeof(double));
  if (e == hipSuccess) e = dmalloc(&boff.p, (size_t)nb * n * sizeof(double));
  if (e == hipSuccess) e = dmalloc(&bbeta.p, (size_t)nb * n * sizeof(double));
  if (e == hipSuccess) e = dmalloc(&bU.p, (size_t)nb * n * r * sizeof(double));
  if (e == hipSuccess) e = dmalloc(&bout.p, (size_t)nb * other * r * sizeof(double));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return std::string(kNoDeviceMemory) + "low-rank workspace: " + hipGetErrorString(e);
  }
  double* A = (double*)bA.p;
  double* p = (double*)bp.p;
  double* w = (double*)bw.p;
  double* off = (double*)boff.p;
  double* beta = (double*)bbeta.p;
  std::vector<double> hA((size_t)nb * nn), hoff((size_t)nb * n), hbeta((size_t)nb * n);
  std::vector<double> vecs((size_t)nb * n * r), proj((size_t)nb * other * r);
  for (int e0 = 0; e0 < n_experts; e0 += nb) {
    const int ne = std::min(nb, n_experts - e0);
    const uint16_t* wd = wch_dev + (size_t)e0 * xe + 2 * (size_t)d;
    const dim3 gg((n + 63) / 64, (n + 63) / 64, ne);
    if (m <= d)  // G = W^T W: (a, b) = sum_i W[i][a] W[i][b]; X(k = i, a) = wd[i + a * cstride]
      hipLaunchKernelGGL(k_gram, gg, dim3(256), 0, s, wd, xe, 1L, cstride, d, n, A);
    else  // G = W W^T: (a, b) = sum_j W[a][j] W[b][j]; X(k = j, a) = wd[j * cstride + a]
      hipLaunchKernelGGL(k_gram, gg, dim3(256), 0, s, wd, xe, cstride, 1L, m, n, A);
    for (int k = 0; k + 2 < n; ++k) {
      const int len = n - k - 1;
      hipLaunchKernelGGL(k_house, dim3(ne), dim3(1024), 0, s, A, n, k, off, beta);
      hipLaunchKernelGGL(k_symv, dim3((len + 3) / 4, ne), dim3(256), 0, s, (const double*)A, n, k,
                         (const double*)beta, p);
      hipLaunchKernelGGL(k_wvec, dim3(ne), dim3(1024), 0, s, (const double*)A, n, k, (const double*)beta,
                         (const double*)p, w);
      const int rows = len < 128 ? len : 128;
      hipLaunchKernelGGL(k_rank2, dim3((len + 255) / 256, rows, ne), dim3(256), 0, s, A, n, k,
                         (const double*)beta, (const double*)w);
    }
    if ((e = hipGetLastError()) != hipSuccess) return std::string("device tridiagonalisation: ") + hipGetErrorString(e);
    e = hipMemcpyAsync(hA.data(), A, (size_t)ne * nn * sizeof(double), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipMemcpyAsync(hoff.data(), off, (size_t)ne * n * sizeof(double), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipMemcpyAsync(hbeta.data(), beta, (size_t)ne * n * sizeof(double), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return std::string("device low-rank copy: ") + hipGetErrorString(e);
    EigJob job{&hA, &hoff, &hbeta, &vecs, n, r};
    parallel_for(ne, 0, eig_one, &job);
    // the other factor: m <= d: P[c][i] = sum_j W[i][j] V[j][c]; else Q[j][c] = sum_i W[i][j] U[i][c]
    e = hipMemcpyAsync(bU.p, vecs.data(), (size_t)ne * n * r * sizeof(double), hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return std::string("device low-rank projection: ") + hipGetErrorString(e);
    if (m <= d)  // row i of W: X(i, j) = wd[i + j * cstride], len = m
      hipLaunchKernelGGL(k_project, dim3(d, ne), dim3(64), 0, s, wd, xe, 1L, cstride, m, (const double*)bU.p, r, d,
                         (double*)bout.p);
    else  // column j of W: X(j, i) = wd[j * cstride + i], len = d
      hipLaunchKernelGGL(k_project, dim3(m, ne), dim3(64), 0, s, wd, xe, cstride, 1L, d, (const double*)bU.p, r, m,
                         (double*)bout.p);
    e = hipGetLastError();
    if (e == hipSuccess)
      e = hipMemcpyAsync(proj.data(), bout.p, (size_t)ne * other * r * sizeof(double), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return std::string("device low-rank projection: ") + hipGetErrorString(e);
    for (int z = 0; z < ne; ++z) {
      const double* vz = vecs.data() + (size_t)z * n * r;
      const double* pz = proj.data() + (size_t)z * other * r;
      uint16_t* po = p_out + (size_t)(e0 + z) * r * d;
      uint16_t* qo = q_out + (size_t)(e0 + z) * m * r;
      if (m <= d) {
        for (int j = 0; j < m; ++j)
          for (int c = 0; c < r; ++c) qo[(size_t)j * r + c] = f32_to_bf16((float)vz[(size_t)j * r + c]);
        for (int c = 0; c < r; ++c)
          for (int i = 0; i < d; ++i) po[(size_t)c * d + i] = f32_to_bf16((float)pz[(size_t)i * r + c]);
      } else {
        for (int c = 0; c < r; ++c)
          for (int i = 0; i < d; ++i) po[(size_t)c * d + i] = f32_to_bf16((float)vz[(size_t)i * r + c]);
        for (int j = 0; j < m; ++j)
          for (int c = 0; c < r; ++c) qo[(size_t)j * r + c] = f32_to_bf16((float)pz[(size_t)j * r + c]);
      }
    }
  }
  return std::string();
}

}  // namespace moe_sel
