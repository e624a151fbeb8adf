// Internal declarations shared by the host runtime, the host-side preparation
// and the device kernels. Not part of the public ABI (include/moe_sel.h).
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "moe_sel.h"

// Layout helpers are shared by host packing code and device kernels.
#if defined(__HIPCC__)
#define MOE_SEL_HD __host__ __device__
#else
#define MOE_SEL_HD
#endif

namespace moe_sel {

// ---------------------------------------------------------------------------
// Device layout (all per expert e, contiguous per expert):
//
//  codes  : 2-bit offset-binary sketch codes (t + 1 in {0, 1, 2}).
//           [E][m/64 groups][2 (gate, up)][d/64 blocks][64 lanes][4 dwords]
//           A 64-lane wave reads one (group, matrix, block) as one coalesced
//           1 KiB load: lane l holds channel 64*g + l, dword w holds the 16
//           codes of d = 64*b + 16*w .. +15, the code of d = 64b + 16w + 4a + i
//           sitting at bits [8i + 2a, 8i + 2a + 2) so that
//           (dword >> 2a) & 0x03030303 yields four byte-wide codes that line up
//           with four consecutive int8 activations.
//  stats  : float4 [E][m] = {alpha_gate, alpha_up, ||down_j||_2, 0}
//  wch    : bf16 [E][m][3][d]: channel j's gate row, up row and down column
//           stored back to back (12*d bytes per channel, contiguous).
//  pmat   : bf16 [E][r][d]   (P^T: row c is the c-th output direction)
//  qmat   : bf16 [E][m][r]   (row j: channel j's coordinates)
// ---------------------------------------------------------------------------
constexpr int kGroup = 64;   // channels per sketch group (one per lane)
constexpr int kBlock = 64;   // hidden elements per sketch block

MOE_SEL_HD inline size_t codes_dwords_per_expert(int d, int m) { return (size_t)m * 2 * (d / 16); }
MOE_SEL_HD inline size_t codes_dword_index(int d, int m, int g, int mat, int b, int lane, int w) {
  const int nb = d / kBlock;
  (void)m;
  return ((((size_t)g * 2 + mat) * nb + b) * 64 + lane) * 4 + w;
}

// Host-side preparation of one expert (prepare_host.cpp). Outputs may be null.
struct ExpertPrep {
  int8_t* tern_gate = nullptr;   // [m][d]
  int8_t* tern_up = nullptr;     // [m][d]
  float* alpha_gate = nullptr;   // [m]
  float* alpha_up = nullptr;     // [m]
  float* down_norm = nullptr;    // [m]
  int32_t* nnz_gate = nullptr;   // [m]
  int32_t* nnz_up = nullptr;     // [m]
  uint32_t* codes = nullptr;     // device layout, codes_dwords_per_expert
  float* stats = nullptr;        // [m][4]
  uint16_t* wch = nullptr;       // [m][3][d]
  uint16_t* p_bf16 = nullptr;    // [r][d]
  uint16_t* q_bf16 = nullptr;    // [m][r]
};

// Symmetric eigen-solver pieces (Golub & Van Loan): the Householder
// tridiagonal form of an n x n matrix, and the top-r eigenpairs from it.
struct Tridiag {
  std::vector<double> diag, off;  // off[i] couples i and i+1
  std::vector<double> beta;       // reflector k acts on indices k+1..n-1
};
void eigvecs_from_tridiag(const double* refl, int n, int r, const Tridiag& T, std::vector<double>& vecs,
                          std::vector<double>& vals);

// Rank-r maps of all experts built on the device in fp64 (Gram matrices,
// tridiagonalisation and projection on the GPU, batched over experts; the
// tridiagonal eigen-solves on host threads). wch_dev: the experts' channel-major
// rows on the device ([E][m][3][d]). Outputs are host arrays P^T [E][r][d] and
// Q [E][m][r] in bf16. Empty string on success.
std::string lowrank_maps_device(const uint16_t* wch_dev, int n_experts, int d, int m, int r, uint16_t* p_out,
                                uint16_t* q_out, void* stream);

// Ternary sketch codes and the stats [E][m] float4 {alpha_gate, alpha_up,
// ||down_j||, 0} of all experts built on the device from the channel-major rows
// (wch_dev, [E][m][3][d]), bit-identical to prepare_expert's. Queued on
// `stream`; empty string on success.
std::string sketch_stats_device(const uint16_t* wch_dev, int n_experts, int d, int m, double ratio,
                                uint32_t* codes_dev, float* stats_dev, void* stream);

// Returns an empty string on success, else the failure message.
std::string prepare_expert(const moe_sel_config& cfg, const uint16_t* w_gate, const uint16_t* w_up,
                           const uint16_t* w_down, const ExpertPrep& out);

// Validation shared by every entry point (validate.cpp). Empty string = valid.
std::string validate_config(const moe_sel_config* cfg);

// Round-to-nearest-even conversion of an fp32 value to bf16 bits.
uint16_t f32_to_bf16(float v);
float bf16_to_f32(uint16_t b);

// Allocation fault injection for tests of the out-of-memory paths: once armed
// with n >= 1, the n-th allocation the library attempts after that fails (and
// the injector disarms). Host allocations throw std::bad_alloc there; device
// allocations return hipErrorOutOfMemory (checked_device_malloc).
void arm_alloc_fault(int n);
bool alloc_fault_hit();
// hipMalloc behind the fault injector.
int checked_device_malloc(void** p, size_t bytes);  // a hipError_t value
// Message prefix of a device workspace that could not be allocated.
constexpr const char* kNoDeviceMemory = "out of device memory: ";

// Run fn(i) for i in [0, n) on up to `threads` host threads (0 = all cores).
void parallel_for(int n, int threads, void (*fn)(int, void*), void* arg);

}  // namespace moe_sel
