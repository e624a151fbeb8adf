// Host-only check of the weight-only preparation (ternary sketch, channel
// statistics, device-layout packing, rank-r map) and of the allocation fault
// injector, built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py. Experts of several shapes are prepared,
// including rows that are zero, constant, one-hot or subnormal, on several
// host threads at once; the program checks a few invariants and exits non-zero
// on a mismatch (the sanitizers abort on their own findings).
#include <cmath>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "internal.h"

using namespace moe_sel;

namespace {

int g_fail = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint32_t next_u32() {
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(g_state >> 33);
}
// bf16 of a value roughly N(0, 0.02): sum of uniforms, scaled
uint16_t rand_weight() {
  float s = 0.0f;
  for (int i = 0; i < 4; ++i) s += (float)(next_u32() & 0xFFFF) / 65536.0f - 0.5f;
  return f32_to_bf16(s * 0.035f);
}

struct Expert {
  int d, m, r;
  std::vector<uint16_t> wg, wu, wd;
};

Expert make_expert(int d, int m, int r) {
  Expert e{d, m, r, std::vector<uint16_t>((size_t)m * d), std::vector<uint16_t>((size_t)m * d),
           std::vector<uint16_t>((size_t)d * m)};
  for (auto& v : e.wg) v = rand_weight();
  for (auto& v : e.wu) v = rand_weight();
  for (auto& v : e.wd) v = rand_weight();
  // edge rows: zero, constant magnitude, one-hot, subnormal
  for (int i = 0; i < d; ++i) {
    e.wg[(size_t)0 * d + i] = 0;
    e.wu[(size_t)1 * d + i] = (i & 1) ? 0xBC00 : 0x3C00;  // -1/128 and 1/128 magnitude pattern
    e.wg[(size_t)2 * d + i] = i == 5 ? 0x3F80 : 0;       // one-hot 1.0
    e.wu[(size_t)3 * d + i] = (uint16_t)(1 + (i % 100));  // subnormals
  }
  return e;
}

struct Job {
  std::vector<Expert>* experts;
  std::vector<std::string>* errs;
};

void prepare_one(int idx, void* arg) {
  Job* j = (Job*)arg;
  const Expert& e = (*j->experts)[idx];
  moe_sel_config cfg{};
  cfg.struct_size = sizeof(moe_sel_config);
  cfg.d = e.d;
  cfg.m = e.m;
  cfg.rank = e.r;
  cfg.n_experts = 1;
  cfg.max_top_e = 1;
  cfg.max_batch = 1;
  cfg.tern_ratio = 0.7;
  std::vector<int8_t> tg((size_t)e.m * e.d), tu((size_t)e.m * e.d);
  std::vector<float> ag(e.m), au(e.m), dn(e.m), stats((size_t)e.m * 4);
  std::vector<int32_t> ng(e.m), nu(e.m);
  std::vector<uint32_t> codes(codes_dwords_per_expert(e.d, e.m));
  std::vector<uint16_t> wch((size_t)e.m * 3 * e.d), p((size_t)e.r * e.d + 1), q((size_t)e.m * e.r + 1);
  ExpertPrep out;
  out.tern_gate = tg.data();
  out.tern_up = tu.data();
  out.alpha_gate = ag.data();
  out.alpha_up = au.data();
  out.down_norm = dn.data();
  out.nnz_gate = ng.data();
  out.nnz_up = nu.data();
  out.codes = codes.data();
  out.stats = stats.data();
  out.wch = wch.data();
  if (e.r > 0) {
    out.p_bf16 = p.data();
    out.q_bf16 = q.data();
  }
  std::string err = prepare_expert(cfg, e.wg.data(), e.wu.data(), e.wd.data(), out);
  if (!err.empty()) {
    (*j->errs)[idx] = err;
    return;
  }
  // invariants: kept counts match the codes; the zero row keeps nothing; the
  // channel-major copy holds the rows and the down column
  for (int c = 0; c < e.m; ++c) {
    int kg = 0, ku = 0;
    for (int i = 0; i < e.d; ++i) {
      kg += tg[(size_t)c * e.d + i] != 0;
      ku += tu[(size_t)c * e.d + i] != 0;
    }
    if (kg != ng[c] || ku != nu[c]) (*j->errs)[idx] = "nnz mismatch";
  }
  if (ng[0] != 0 || ag[0] != 0.0f) (*j->errs)[idx] = "zero row kept entries";
  if (ng[2] != 1) (*j->errs)[idx] = "one-hot row";
  for (int c = 0; c < e.m; ++c)
    for (int i = 0; i < e.d; ++i)
      if (wch[((size_t)c * 3 + 0) * e.d + i] != e.wg[(size_t)c * e.d + i] ||
          wch[((size_t)c * 3 + 2) * e.d + i] != e.wd[(size_t)i * e.m + c])
        (*j->errs)[idx] = "channel-major copy";
  for (int c = 0; c < e.m; ++c)
    if (!(dn[c] >= 0.0f) || !std::isfinite(ag[c])) (*j->errs)[idx] = "statistics not finite";
}

}  // namespace

int main() {
  const int shapes[][3] = {{64, 64, 0}, {64, 64, 64}, {128, 64, 8}, {64, 192, 16}, {256, 128, 32}, {192, 64, 63}};
  std::vector<Expert> experts;
  for (const auto& s : shapes) experts.push_back(make_expert(s[0], s[1], s[2]));
  std::vector<std::string> errs(experts.size());
  Job job{&experts, &errs};
  parallel_for((int)experts.size(), 4, prepare_one, &job);
  for (size_t i = 0; i < errs.size(); ++i) {
    if (!errs[i].empty()) std::fprintf(stderr, "expert %zu: %s\n", i, errs[i].c_str());
    CHECK(errs[i].empty());
  }

  // the fault injector: the armed allocation throws once, then preparation works again
  arm_alloc_fault(1);
  bool threw = false;
  try {
    std::vector<std::string> e1(1);
    std::vector<Expert> one{experts[2]};
    Job j1{&one, &e1};
    prepare_one(0, &j1);
  } catch (const std::bad_alloc&) {
    threw = true;
  }
  CHECK(threw);
  CHECK(!alloc_fault_hit());  // disarmed after it fired
  arm_alloc_fault(3);
  CHECK(!alloc_fault_hit());
  CHECK(!alloc_fault_hit());
  CHECK(alloc_fault_hit());
  CHECK(!alloc_fault_hit());
  arm_alloc_fault(2);
  arm_alloc_fault(0);  // disarms
  CHECK(!alloc_fault_hit() && !alloc_fault_hit());

  // round trip of the bf16 conversion on ties and carries
  CHECK(f32_to_bf16(1.0f) == 0x3F80);
  CHECK(f32_to_bf16(bf16_to_f32(0x3F81)) == 0x3F81);
  std::printf("%s (%zu experts)\n", g_fail ? "FAILED" : "ok", experts.size());
  return g_fail ? 1 : 0;
}
