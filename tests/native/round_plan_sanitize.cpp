// Host-side round planner under AddressSanitizer / UndefinedBehaviorSanitizer.
//
// Built by tests/test_round_plan_sanitize.py with g++ from the library's own
// round.cpp (no GPU code), it plans seeded random rounds (separators, empty
// and repeated segments, shared and private blocks, slot ranges), checks the
// invariants of every plan and drives the error paths.  Any out-of-bounds
// access, leak or undefined operation aborts the run with a report.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "../../include/tdx.h"

namespace tdx {
// the library's error reporter lives in the C ABI file; keep the last text here
std::string g_msg;
int report(int code, const char* msg) {
  g_msg = msg;
  return code;
}
}  // namespace tdx

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint32_t next_u32() {  // xorshift64*
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (uint32_t)((g_state * 2685821657736338717ull) >> 32);
}
int uniform(int lo, int hi) { return lo + (int)(next_u32() % (uint32_t)(hi - lo + 1)); }

int fail(const char* what, int round) {
  std::fprintf(stderr, "round %d: %s\n", round, what);
  return 1;
}

int check_round(int round) {
  const int sep = 0;
  const int R = uniform(1, 12);
  std::vector<std::vector<int32_t>> pool(uniform(1, 6));
  for (auto& p : pool) {
    p.resize(uniform(1, 5));
    for (auto& t : p) t = uniform(1, 5);
  }
  std::vector<int32_t> tokens;
  std::vector<int64_t> off{0};
  for (int r = 0; r < R; ++r) {
    const int parts = uniform(0, 6);
    for (int q = 0; q < parts; ++q) {
      for (int s = uniform(0, 2); s > 0; --s) tokens.push_back(sep);
      if (uniform(0, 4) == 0) {
        for (int s = uniform(0, 4); s > 0; --s) tokens.push_back(uniform(1000, 1010));
      } else {
        const auto& p = pool[uniform(0, (int)pool.size() - 1)];
        tokens.insert(tokens.end(), p.begin(), p.end());
      }
    }
    off.push_back((int64_t)tokens.size());
  }
  std::vector<int64_t> sb(R), se(R);
  const bool slots = uniform(0, 1) == 1;
  for (int r = 0; r < R; ++r) {
    sb[r] = uniform(0, 40);
    se[r] = sb[r] + uniform(0, 15);
  }
  const int min_share = uniform(-1, R + 1);
  tdx_round_plan* plan = nullptr;
  const int rc = tdx_round_plan_build(tokens.empty() ? nullptr : tokens.data(), off.data(), R, sep, min_share,
                                      slots ? sb.data() : nullptr, slots ? se.data() : nullptr, &plan);
  if (rc != TDX_OK || plan == nullptr) return fail("build failed", round);
  const int ng = tdx_round_plan_n_groups(plan);
  if (ng < 1 || ng > R) return fail("group count", round);
  std::vector<int> seen(R, 0);
  for (int g = 0; g < ng; ++g) {
    int32_t N = -1, B = -1, T = -1;
    if (tdx_round_plan_group_dims(plan, g, &N, &B, &T) != TDX_OK) return fail("dims", round);
    std::vector<int32_t> agents(N), seg(B), bs(B + 1), src(B), dst((size_t)N * B), priv(N);
    if (tdx_round_plan_group(plan, g, agents.data(), seg.data(), bs.data(), src.data(), dst.data(), priv.data()) !=
        TDX_OK)
      return fail("group", round);
    if (bs[0] != 0 || bs[B] != T) return fail("blk_start", round);
    for (int i = 0; i < N; ++i) {
      const int r = agents[i];
      if (r < 0 || r >= R || seen[r]++) return fail("membership", round);
      const int64_t len = off[r + 1] - off[r];
      if (priv[i] != len - T) return fail("priv_len", round);
      std::vector<int32_t> map(len > 0 ? (size_t)len : 1);
      int32_t grp = -1;
      if (tdx_round_plan_request(plan, r, &grp, map.data()) != TDX_OK || grp != g) return fail("request", round);
      int64_t shared = 0;
      for (int64_t p = 0; p < len; ++p) shared += map[p] >= 0;
      if (shared != T) return fail("token map count", round);
      for (int b = 0; b < B; ++b) {
        if (src[b] != bs[b]) return fail("src_pos", round);
        const int32_t d = dst[(size_t)i * B + b];
        for (int32_t j = 0; j < bs[b + 1] - bs[b]; ++j) {
          if (d + j >= len) return fail("dst_pos out of the request", round);
          // the shared copy holds the block's content (the first member's copy)
          const int32_t want = tokens[off[agents[0]] + dst[b] + j];
          if (tokens[off[r] + d + j] != want || map[d + j] != bs[b] + j) return fail("content", round);
        }
      }
    }
  }
  for (int r = 0; r < R; ++r)
    if (seen[r] != 1) return fail("a request in no group", round);
  tdx_round_plan_free(plan);
  return 0;
}

int check_errors() {
  tdx_round_plan* plan = reinterpret_cast<tdx_round_plan*>(0x1);
  const int32_t toks[4] = {1, 2, 0, 3};
  const int64_t off[3] = {0, 2, 4}, bad[3] = {0, 3, 2};
  const int64_t sb[2] = {5, 0}, se[2] = {4, 1};
  int bad_rc = 0;
  bad_rc |= tdx_round_plan_build(toks, off, 2, 0, 0, nullptr, nullptr, nullptr) != TDX_EINVAL;
  bad_rc |= tdx_round_plan_build(toks, off, 0, 0, 0, nullptr, nullptr, &plan) != TDX_EINVAL || plan != nullptr;
  bad_rc |= tdx_round_plan_build(toks, bad, 2, 0, 0, nullptr, nullptr, &plan) != TDX_EINVAL;
  bad_rc |= tdx_round_plan_build(nullptr, off, 2, 0, 0, nullptr, nullptr, &plan) != TDX_EINVAL;
  bad_rc |= tdx_round_plan_build(toks, off, 2, 0, 0, sb, nullptr, &plan) != TDX_EINVAL;
  bad_rc |= tdx_round_plan_build(toks, off, 2, 0, 0, sb, se, &plan) != TDX_EINVAL;
  bad_rc |= tdx_round_plan_n_groups(nullptr) != TDX_EINVAL;
  if (tdx_round_plan_build(toks, off, 2, 0, 0, nullptr, nullptr, &plan) != TDX_OK) return 1;
  bad_rc |= tdx_round_plan_group_dims(plan, 5, nullptr, nullptr, nullptr) != TDX_EINVAL;
  bad_rc |= tdx_round_plan_group(plan, -1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) != TDX_EINVAL;
  bad_rc |= tdx_round_plan_request(plan, 9, nullptr, nullptr) != TDX_EINVAL;
  bad_rc |= tdx_round_plan_group(plan, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) != TDX_OK;
  tdx_round_plan_free(plan);
  tdx_round_plan_free(nullptr);
  if (bad_rc) std::fprintf(stderr, "error paths: unexpected return code\n");
  return bad_rc;
}

}  // namespace

int main(int argc, char** argv) {
  const int rounds = argc > 1 ? std::atoi(argv[1]) : 500;
  for (int r = 0; r < rounds; ++r)
    if (check_round(r)) return 1;
  if (check_errors()) return 1;
  std::printf("ok %d rounds\n", rounds);
  return 0;
}
