// Host-side, weight-only preparation of one expert: ternary sketch and channel
// statistics, device-layout packing, and the rank-r map of the down matrix.
//
// Page "KAIST drops calibration from MoE decoding, speeds up blocks by up to
// 2.69x over vLLM", section "A reader built from weights alone": channels are
// filtered with a ternary sketch of the weights and skipped channels are
// compensated by a low-rank map built from the weights; nothing here looks at
// activations or calibration data.
//
// Exactness: every sum is formed exactly in a wide fixed-point accumulator and
// rounded once to double, so the statistics are a function of the weights
// alone, independent of summation order. This translation unit is compiled
// without floating-point contraction.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <new>
#include <thread>
#include <vector>

#include "internal.h"

namespace moe_sel {

uint16_t f32_to_bf16(float v) {
  uint32_t u;
  std::memcpy(&u, &v, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFF) ? 0x40 : 0));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

void parallel_for(int n, int threads, void (*fn)(int, void*), void* arg) {
  if (n <= 0) return;
  if (threads <= 0) threads = (int)std::max(1u, std::thread::hardware_concurrency());
  threads = std::min(threads, n);
  if (threads == 1) {
    for (int i = 0; i < n; ++i) fn(i, arg);
    return;
  }
  std::atomic<int> next{0};
  std::vector<std::thread> pool;
  pool.reserve(threads);
  for (int t = 0; t < threads; ++t)
    pool.emplace_back([&] {
      for (int i = next.fetch_add(1); i < n; i = next.fetch_add(1)) fn(i, arg);
    });
  for (auto& th : pool) th.join();
}

namespace {

// Non-negative integer of NL 64-bit limbs; value = integer * 2^lsb_exp.
template <int NL>
struct ExactAcc {
  uint64_t limb[NL];
  ExactAcc() { std::memset(limb, 0, sizeof(limb)); }
  // add v * 2^pos, v < 2^32
  void add(uint64_t v, int pos) {
    const int li = pos >> 6, sh = pos & 63;
    const unsigned __int128 x = (unsigned __int128)v << sh;
    uint64_t lo = (uint64_t)x, carry = (uint64_t)(x >> 64);
    uint64_t s = limb[li] + lo;
    carry += (s < lo);
    limb[li] = s;
    for (int i = li + 1; carry && i < NL; ++i) {
      s = limb[i] + carry;
      carry = (s < carry);
      limb[i] = s;
    }
  }
  int bit(int p) const { return p < 0 ? 0 : (int)((limb[p >> 6] >> (p & 63)) & 1u); }
  bool any_below(int p) const {  // any set bit at positions < p
    if (p <= 0) return false;
    const int li = p >> 6, sh = p & 63;
    for (int i = 0; i < li && i < NL; ++i)
      if (limb[i]) return true;
    if (li < NL && sh && (limb[li] & ((uint64_t(1) << sh) - 1))) return true;
    return false;
  }
  // integer * 2^lsb_exp rounded to the nearest double, ties to even
  double to_double(int lsb_exp) const {
    int top = NL - 1;
    while (top >= 0 && limb[top] == 0) --top;
    if (top < 0) return 0.0;
    int msb = top * 64 + (63 - __builtin_clzll(limb[top]));
    uint64_t mant = 0;
    for (int p = msb; p >= msb - 52; --p) mant = (mant << 1) | (uint64_t)bit(p);
    const int round_bit = bit(msb - 53);
    const bool sticky = any_below(msb - 53);
    if (round_bit && (sticky || (mant & 1u))) {
      ++mant;
      if (mant == (uint64_t(1) << 53)) {
        mant >>= 1;
        ++msb;
      }
    }
    return std::ldexp((double)mant, msb - 52 + lsb_exp);
  }
};

// |w| of a finite bf16 as M * 2^(pos - 133), M < 256, pos >= 0
inline void bf16_mag(uint16_t b, uint32_t& mant, int& pos) {
  const int e = (b >> 7) & 0xFF;
  const uint32_t f = b & 0x7F;
  if (e == 0) {
    mant = f;
    pos = 0;
  } else {
    mant = 128u + f;
    pos = e - 1;
  }
}

inline double bf16_abs_double(uint16_t b) { return std::fabs((double)bf16_to_f32(b)); }

struct RowStats {
  float alpha;
  int32_t nnz;
};

// Ternary sketch of one channel row of length d (strided access allowed).
RowStats sketch_row(const uint16_t* w, int d, double ratio, int8_t* t_out) {
  ExactAcc<5> all;
  for (int i = 0; i < d; ++i) {
    uint32_t mt;
    int pos;
    bf16_mag(w[i], mt, pos);
    if (mt) all.add(mt, pos);
  }
  const double total = all.to_double(-133);
  const double mean = total / (double)d;
  const double delta = ratio * mean;
  ExactAcc<5> kept;
  int nnz = 0;
  for (int i = 0; i < d; ++i) {
    const double a = bf16_abs_double(w[i]);
    int8_t t = 0;
    if (a > delta) {
      t = (w[i] & 0x8000) ? -1 : 1;
      uint32_t mt;
      int pos;
      bf16_mag(w[i], mt, pos);
      if (mt) kept.add(mt, pos);
      ++nnz;
    }
    t_out[i] = t;
  }
  RowStats rs;
  rs.nnz = nnz;
  rs.alpha = nnz ? (float)(kept.to_double(-133) / (double)nnz) : 0.0f;
  return rs;
}

float column_norm(const uint16_t* wd, int d, int m, int j) {
  ExactAcc<9> sq;
  for (int i = 0; i < d; ++i) {
    uint32_t mt;
    int pos;
    bf16_mag(wd[(size_t)i * m + j], mt, pos);
    if (mt) sq.add((uint64_t)mt * mt, 2 * pos);
  }
  return (float)std::sqrt(sq.to_double(-266));
}

// ---------------------------------------------------------------------------
// Symmetric eigen-solver for the top-r eigenpairs (Golub & Van Loan: Householder
// tridiagonalisation, bisection on Sturm counts, inverse iteration with full
// re-orthogonalisation, back-transformation).
// ---------------------------------------------------------------------------
// A (n x n, row-major, symmetric, overwritten with reflectors in rows k: A[k][k+1..]).
void tridiagonalize(std::vector<double>& A, int n, Tridiag& T) {
  T.diag.assign(n, 0.0);
  T.off.assign(std::max(n - 1, 0), 0.0);
  T.beta.assign(std::max(n - 2, 0), 0.0);
  std::vector<double> p(n), w(n);
  for (int k = 0; k + 2 < n; ++k) {
    double* v = &A[(size_t)k * n + k + 1];  // row k right of the diagonal == column k below it
    const int len = n - k - 1;
    double xnorm2 = 0.0;
    for (int i = 0; i < len; ++i) xnorm2 += v[i] * v[i];
    const double xnorm = std::sqrt(xnorm2);
    if (xnorm == 0.0) {
      T.off[k] = 0.0;
      T.beta[k] = 0.0;
      continue;
    }
    const double alpha = v[0] > 0 ? -xnorm : xnorm;
    v[0] -= alpha;
    double vnorm2 = 0.0;
    for (int i = 0; i < len; ++i) vnorm2 += v[i] * v[i];
    const double beta = 2.0 / vnorm2;
    T.off[k] = alpha;
    T.beta[k] = beta;
    // p = beta * A22 v (eight interleaved partial sums per row, added pairwise)
    for (int i = 0; i < len; ++i) {
      const double* row = &A[(size_t)(k + 1 + i) * n + k + 1];
      double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      int j = 0;
      for (; j + 8 <= len; j += 8)
        for (int q = 0; q < 8; ++q) acc[q] += row[j + q] * v[j + q];
      for (; j < len; ++j) acc[0] += row[j] * v[j];
      p[i] = beta * (((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7])));
    }
    double pv = 0.0;
    for (int i = 0; i < len; ++i) pv += p[i] * v[i];
    const double K = 0.5 * beta * pv;
    for (int i = 0; i < len; ++i) w[i] = p[i] - K * v[i];
    for (int i = 0; i < len; ++i) {
      double* row = &A[(size_t)(k + 1 + i) * n + k + 1];
      const double vi = v[i], wi = w[i];
      for (int j = 0; j < len; ++j) row[j] -= vi * w[j] + wi * v[j];
    }
  }
  for (int i = 0; i < n; ++i) T.diag[i] = A[(size_t)i * n + i];
  if (n >= 2) T.off[n - 2] = A[(size_t)(n - 1) * n + (n - 2)];
}

// number of eigenvalues of T strictly below x
int sturm_count(const Tridiag& T, double x, double pivmin) {
  const int n = (int)T.diag.size();
  int cnt = 0;
  double q = T.diag[0] - x;
  if (std::fabs(q) < pivmin) q = -pivmin;
  cnt += q < 0;
  for (int i = 1; i < n; ++i) {
    q = (T.diag[i] - x) - T.off[i - 1] * T.off[i - 1] / q;
    if (std::fabs(q) < pivmin) q = -pivmin;
    cnt += q < 0;
  }
  return cnt;
}

// Solve (T - lam I) y = b in place (LU with partial pivoting of a tridiagonal).
void tridiag_solve(const Tridiag& T, double lam, double tiny, std::vector<double>& b) {
  const int n = (int)T.diag.size();
  std::vector<double> dl(n), dd(n), du(n), du2(n, 0.0);
  std::vector<char> swapped(n, 0);
  for (int i = 0; i < n; ++i) dd[i] = T.diag[i] - lam;
  for (int i = 0; i + 1 < n; ++i) dl[i] = du[i] = T.off[i];
  for (int i = 0; i + 1 < n; ++i) {
    if (std::fabs(dd[i]) >= std::fabs(dl[i])) {
      if (dd[i] == 0.0) dd[i] = tiny;
      const double f = dl[i] / dd[i];
      dl[i] = f;
      dd[i + 1] -= f * du[i];
      du2[i] = 0.0;
    } else {
      const double f = dd[i] / dl[i];
      dd[i] = dl[i];
      dl[i] = f;
      const double tmp = du[i];
      du[i] = dd[i + 1];
      dd[i + 1] = tmp - f * dd[i + 1];
      if (i + 2 < n) {
        du2[i] = du[i + 1];
        du[i + 1] = -f * du[i + 1];
      }
      swapped[i] = 1;
    }
  }
  if (dd[n - 1] == 0.0) dd[n - 1] = tiny;
  for (int i = 0; i + 1 < n; ++i) {
    if (swapped[i]) std::swap(b[i], b[i + 1]);
    b[i + 1] -= dl[i] * b[i];
  }
  b[n - 1] /= dd[n - 1];
  if (n >= 2) b[n - 2] = (b[n - 2] - du[n - 2] * b[n - 1]) / dd[n - 2];
  for (int i = n - 3; i >= 0; --i) b[i] = (b[i] - du[i] * b[i + 1] - du2[i] * b[i + 2]) / dd[i];
}

}  // namespace

// Top-r eigenpairs from the tridiagonal form T and the reflectors stored in the
// rows of refl (row k, columns k+1..n-1): bisection on Sturm counts, inverse
// iteration with full re-orthogonalisation, then back-transformation of all r
// vectors together.
void eigvecs_from_tridiag(const double* refl, int n, int r, const Tridiag& T, std::vector<double>& vecs,
                          std::vector<double>& vals) {
  double tnorm = 0.0;
  for (int i = 0; i < n; ++i) {
    double s = std::fabs(T.diag[i]);
    if (i > 0) s += std::fabs(T.off[i - 1]);
    if (i + 1 < n) s += std::fabs(T.off[i]);
    tnorm = std::max(tnorm, s);
  }
  const double eps = 2.220446049250313e-16;
  const double pivmin = std::max(tnorm * eps * eps, 1e-300);
  const double tiny = std::max(tnorm * eps, 1e-300);
  vals.assign(r, 0.0);
  // eigenvalues, largest first, by bisection
  for (int i = 0; i < r; ++i) {
    const int target = n - 1 - i;  // the target-th smallest (0-based)
    double lo = -tnorm - 1.0, hi = tnorm + 1.0;
    for (int it = 0; it < 200; ++it) {
      const double mid = 0.5 * (lo + hi);
      if (mid <= lo || mid >= hi) break;
      if (sturm_count(T, mid, pivmin) > target) hi = mid;
      else lo = mid;
    }
    vals[i] = 0.5 * (lo + hi);
  }
  // eigenvectors of T by inverse iteration, re-orthogonalised against all previous ones
  std::vector<std::vector<double>> ys(r, std::vector<double>(n));
  uint64_t lcg = 0x9E3779B97F4A7C15ull;
  for (int i = 0; i < r; ++i) {
    std::vector<double>& y = ys[i];
    for (int j = 0; j < n; ++j) {
      lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
      y[j] = ((double)(lcg >> 11) / 9007199254740992.0) - 0.5;
    }
    for (int it = 0; it < 4; ++it) {
      tridiag_solve(T, vals[i], tiny, y);
      for (int pass = 0; pass < 2; ++pass)
        for (int q = 0; q < i; ++q) {
          double dot = 0.0;
          for (int j = 0; j < n; ++j) dot += ys[q][j] * y[j];
          for (int j = 0; j < n; ++j) y[j] -= dot * ys[q][j];
        }
      double nrm = 0.0;
      for (int j = 0; j < n; ++j) nrm += y[j] * y[j];
      nrm = std::sqrt(nrm);
      if (nrm == 0.0) {
        y.assign(n, 0.0);
        y[i % n] = 1.0;
        nrm = 1.0;
      }
      for (int j = 0; j < n; ++j) y[j] /= nrm;
    }
  }
  // back-transform all vectors: Y = H_0 H_1 ... H_{n-3} Y, with Y n x r row-major
  vecs.assign((size_t)n * r, 0.0);
  for (int i = 0; i < r; ++i)
    for (int j = 0; j < n; ++j) vecs[(size_t)j * r + i] = ys[i][j];
  std::vector<double> dots(r);
  for (int k = n - 3; k >= 0; --k) {
    const double beta = T.beta[k];
    if (beta == 0.0) continue;
    const double* v = refl + (size_t)k * n + k + 1;
    const int len = n - k - 1;
    std::fill(dots.begin(), dots.end(), 0.0);
    for (int j = 0; j < len; ++j) {
      const double vj = v[j];
      const double* yrow = &vecs[(size_t)(k + 1 + j) * r];
      for (int c = 0; c < r; ++c) dots[c] += vj * yrow[c];
    }
    for (int c = 0; c < r; ++c) dots[c] *= beta;
    for (int j = 0; j < len; ++j) {
      const double vj = v[j];
      double* yrow = &vecs[(size_t)(k + 1 + j) * r];
      for (int c = 0; c < r; ++c) yrow[c] -= vj * dots[c];
    }
  }
}

namespace {

// Top-r eigenvectors (columns of vecs, n x r row-major) of the symmetric matrix A.
void top_eigvecs(std::vector<double>& A, int n, int r, std::vector<double>& vecs, std::vector<double>& vals) {
  Tridiag T;
  tridiagonalize(A, n, T);
  eigvecs_from_tridiag(A.data(), n, r, T, vecs, vals);
}

// G (n x n) = sum over the rows x of X [rows][n] of x^T x. Rows of G are
// accumulated in blocks of 32 so a block stays in cache while X streams; each
// entry sums over the rows in order. Only the lower triangle is formed, then
// mirrored.
void gram_lower(const double* X, int rows, int n, double* G) {
  constexpr int kB = 32;
  for (int a0 = 0; a0 < n; a0 += kB) {
    const int a1 = std::min(n, a0 + kB);
    for (int i = 0; i < rows; ++i) {
      const double* x = X + (size_t)i * n;
      for (int a = a0; a < a1; ++a) {
        const double xa = x[a];
        double* g = G + (size_t)a * n;
        for (int b = 0; b <= a; ++b) g[b] += xa * x[b];
      }
    }
  }
  for (int a = 0; a < n; ++a)
    for (int b = 0; b < a; ++b) G[(size_t)b * n + a] = G[(size_t)a * n + b];
}

// P^T [r][d] and Q [m][r] with P Q^T = best rank-r approximation of W [d][m].
void lowrank_map(const uint16_t* wd_bits, int d, int m, int r, uint16_t* p_out, uint16_t* q_out) {
  if (r == 0) return;
  std::vector<double> W((size_t)d * m);
  for (size_t i = 0; i < W.size(); ++i) W[i] = (double)bf16_to_f32(wd_bits[i]);
  std::vector<double> vecs, vals;
  if (m <= d) {
    // G = W^T W (m x m) = sum over rows i of W[i]^T W[i]: lower triangle, one
    // row of W at a time (contiguous inner loops), mirrored at the end
    std::vector<double> G((size_t)m * m, 0.0);
    gram_lower(W.data(), d, m, G.data());
    top_eigvecs(G, m, r, vecs, vals);  // V_r: m x r
    for (int j = 0; j < m; ++j)
      for (int c = 0; c < r; ++c) q_out[(size_t)j * r + c] = f32_to_bf16((float)vecs[(size_t)j * r + c]);
    for (int c = 0; c < r; ++c)
      for (int i = 0; i < d; ++i) {
        const double* row = &W[(size_t)i * m];
        double s = 0.0;
        for (int j = 0; j < m; ++j) s += row[j] * vecs[(size_t)j * r + c];
        p_out[(size_t)c * d + i] = f32_to_bf16((float)s);
      }
  } else {
    // G = W W^T (d x d) = sum over channels j of W[:, j] W[:, j]^T
    std::vector<double> Wt((size_t)m * d);
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < m; ++j) Wt[(size_t)j * d + i] = W[(size_t)i * m + j];
    std::vector<double> G((size_t)d * d, 0.0);
    gram_lower(Wt.data(), m, d, G.data());
    top_eigvecs(G, d, r, vecs, vals);  // U_r: d x r
    for (int c = 0; c < r; ++c)
      for (int i = 0; i < d; ++i) p_out[(size_t)c * d + i] = f32_to_bf16((float)vecs[(size_t)i * r + c]);
    std::vector<double> acc((size_t)m * r, 0.0);
    for (int i = 0; i < d; ++i) {
      const double* row = &W[(size_t)i * m];
      const double* u = &vecs[(size_t)i * r];
      for (int j = 0; j < m; ++j) {
        double* a = &acc[(size_t)j * r];
        const double wij = row[j];
        for (int c = 0; c < r; ++c) a[c] += wij * u[c];
      }
    }
    for (size_t i = 0; i < acc.size(); ++i) q_out[i] = f32_to_bf16((float)acc[i]);
  }
}

}  // namespace

std::string prepare_expert(const moe_sel_config& cfg, const uint16_t* w_gate, const uint16_t* w_up,
                           const uint16_t* w_down, const ExpertPrep& out) {
  if (alloc_fault_hit()) throw std::bad_alloc();  // stands for the scratch vectors below
  const int d = cfg.d, m = cfg.m, r = cfg.rank;
  for (size_t i = 0, n = (size_t)m * d; i < n; ++i)
    if (((w_gate[i] >> 7) & 0xFF) == 0xFF || ((w_up[i] >> 7) & 0xFF) == 0xFF || ((w_down[i] >> 7) & 0xFF) == 0xFF)
      return "weights contain inf or nan";
  // the sketch may be built elsewhere (on the device): skip it when no output asks for it
  const bool sketch = out.tern_gate || out.tern_up || out.alpha_gate || out.alpha_up || out.down_norm ||
                      out.nnz_gate || out.nnz_up || out.stats || out.codes;
  std::vector<int8_t> tg((size_t)d), tu((size_t)d);
  for (int j = 0; j < m; ++j) {
    RowStats sg{0.0f, 0}, su{0.0f, 0};
    float c = 0.0f;
    if (sketch) {
      sg = sketch_row(w_gate + (size_t)j * d, d, cfg.tern_ratio, tg.data());
      su = sketch_row(w_up + (size_t)j * d, d, cfg.tern_ratio, tu.data());
      c = column_norm(w_down, d, m, j);
    }
    if (out.tern_gate) std::memcpy(out.tern_gate + (size_t)j * d, tg.data(), d);
    if (out.tern_up) std::memcpy(out.tern_up + (size_t)j * d, tu.data(), d);
    if (out.alpha_gate) out.alpha_gate[j] = sg.alpha;
    if (out.alpha_up) out.alpha_up[j] = su.alpha;
    if (out.down_norm) out.down_norm[j] = c;
    if (out.nnz_gate) out.nnz_gate[j] = sg.nnz;
    if (out.nnz_up) out.nnz_up[j] = su.nnz;
    if (out.stats) {
      out.stats[(size_t)j * 4 + 0] = sg.alpha;
      out.stats[(size_t)j * 4 + 1] = su.alpha;
      out.stats[(size_t)j * 4 + 2] = c;
      out.stats[(size_t)j * 4 + 3] = 0.0f;
    }
    if (out.codes) {
      const int g = j / kGroup, lane = j % kGroup;
      for (int mat = 0; mat < 2; ++mat) {
        const int8_t* t = mat == 0 ? tg.data() : tu.data();
        for (int b = 0; b < d / kBlock; ++b)
          for (int w = 0; w < 4; ++w) {
            uint32_t word = 0;
            for (int a = 0; a < 4; ++a)
              for (int ii = 0; ii < 4; ++ii) {
                const int i = b * kBlock + 16 * w + 4 * a + ii;
                word |= (uint32_t)(t[i] + 1) << (8 * ii + 2 * a);
              }
            out.codes[codes_dword_index(d, m, g, mat, b, lane, w)] = word;
          }
      }
    }
    if (out.wch) {
      uint16_t* dst = out.wch + (size_t)j * 3 * d;
      std::memcpy(dst, w_gate + (size_t)j * d, (size_t)d * 2);
      std::memcpy(dst + d, w_up + (size_t)j * d, (size_t)d * 2);
      for (int i = 0; i < d; ++i) dst[2 * d + i] = w_down[(size_t)i * m + j];
    }
  }
  if (r > 0 && (out.p_bf16 || out.q_bf16)) {
    std::vector<uint16_t> pbuf, qbuf;
    uint16_t* p = out.p_bf16;
    uint16_t* q = out.q_bf16;
    if (!p) {
      pbuf.resize((size_t)r * d);
      p = pbuf.data();
    }
    if (!q) {
      qbuf.resize((size_t)m * r);
      q = qbuf.data();
    }
    lowrank_map(w_down, d, m, r, p, q);
  }
  return std::string();
}

}  // namespace moe_sel
