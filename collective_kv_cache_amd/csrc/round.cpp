// Round structure from token IDs (host only, no GPU work).
//
// TokenDance notes, §4 "Key Innovations" (Round-Aware Prompt Interface) and
// §2a (data flow: prompt assembly with separators, segment hashing, grouping
// of compatible requests); §5 "Scheduling" (group constraints: same cached
// span, disjoint slot mappings); blog §4.1 (the separator token).  From the
// token IDs of one round's requests this derives, per group of compatible
// requests, the tdx_layout arrays the collective calls take.
//
// Steps: split every request at separator tokens into segments (maximal runs
// of other tokens); give equal token sequences one block ID (a 64-bit FNV-1a
// hash indexes candidates, equality is then checked token by token, so a
// hash collision never merges different content); a block is shared when at
// least min_share requests hold it; requests with the same set of shared
// blocks form a group unless their slot ranges intersect; each group's
// blocks take the order of its first member and canonical positions from
// their prefix sums.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstring>
#include <map>
#include <memory>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/tdx.h"
#include "errors.h"

struct tdx_round_plan {
  struct Group {
    std::vector<int32_t> agents;     // [N] request indices, ascending
    std::vector<int32_t> seg;        // [B] block IDs in canonical order
    std::vector<int32_t> blk_start;  // [B+1]
    std::vector<int32_t> dst;        // [N*B]
    std::vector<int32_t> priv;       // [N]
  };
  std::vector<Group> groups;
  std::vector<int32_t> req_group;  // [R]
  std::vector<int64_t> map_off;    // [R+1] into map
  std::vector<int32_t> map;        // token maps of all requests, concatenated
};

namespace {

// FNV-1a, 64-bit (Fowler, Noll and Vo): for every byte, xor it into the
// state, then multiply by the FNV prime.  Tokens are hashed as 4 little-endian
// bytes each.
uint64_t fnv1a64(const int32_t* p, int64_t n) {
  uint64_t h = 14695981039346656037ull;
  for (int64_t i = 0; i < n; ++i) {
    const uint32_t v = static_cast<uint32_t>(p[i]);
    for (int k = 0; k < 4; ++k) {
      h ^= (v >> (8 * k)) & 0xffu;
      h *= 1099511628211ull;
    }
  }
  return h;
}

struct Seg {
  int32_t start, len, id;
};

int invalid(const char* msg) { return tdx::report(TDX_EINVAL, msg); }

}  // namespace

extern "C" {

int tdx_round_plan_build(const int32_t* tokens, const int64_t* req_off, int32_t n_req, int32_t sep_token,
                         int32_t min_share, const int64_t* slot_begin, const int64_t* slot_end,
                         tdx_round_plan** plan) {
  if (plan == nullptr) return invalid("plan is null");
  *plan = nullptr;
  if (n_req < 1) return invalid("n_req < 1");
  if (req_off == nullptr) return invalid("req_off is null");
  if ((slot_begin == nullptr) != (slot_end == nullptr)) return invalid("slot_begin and slot_end: both or neither");
  if (req_off[0] < 0) return invalid("req_off[0] < 0");
  for (int32_t r = 0; r < n_req; ++r) {
    if (req_off[r + 1] < req_off[r]) return invalid("req_off is not non-decreasing");
    if (req_off[r + 1] - req_off[r] > INT32_MAX) return invalid("a request is longer than INT32_MAX tokens");
    if (slot_begin != nullptr && slot_begin[r] > slot_end[r]) return invalid("slot_begin[r] > slot_end[r]");
  }
  if (tokens == nullptr && req_off[n_req] > req_off[0]) return invalid("tokens is null");
  try {
    const int32_t need = min_share <= 0 ? n_req : min_share;
    auto req_tokens = [&](int32_t r) { return tokens + req_off[r]; };

    // ---- segments and block IDs (dense, in order of first appearance)
    std::vector<std::vector<Seg>> segs(n_req);
    std::unordered_map<uint64_t, std::vector<int32_t>> bucket;  // hash -> IDs
    std::vector<const int32_t*> id_tok;                         // first occurrence of each ID
    std::vector<int32_t> id_len, id_count, id_last;             // length, holders, last holder
    for (int32_t r = 0; r < n_req; ++r) {
      const int32_t* t = req_tokens(r);
      const int32_t n = static_cast<int32_t>(req_off[r + 1] - req_off[r]);
      int32_t p = 0;
      while (p < n) {
        if (t[p] == sep_token) {
          ++p;
          continue;
        }
        int32_t q = p;
        while (q < n && t[q] != sep_token) ++q;
        const int32_t len = q - p;
        std::vector<int32_t>& cand = bucket[fnv1a64(t + p, len)];
        int32_t id = -1;
        for (int32_t c : cand)
          if (id_len[c] == len && std::memcmp(id_tok[c], t + p, sizeof(int32_t) * (size_t)len) == 0) {
            id = c;
            break;
          }
        if (id < 0) {
          id = static_cast<int32_t>(id_len.size());
          cand.push_back(id);
          id_tok.push_back(t + p);
          id_len.push_back(len);
          id_count.push_back(0);
          id_last.push_back(-1);
        }
        if (id_last[id] != r) {
          id_last[id] = r;
          ++id_count[id];
        }
        segs[r].push_back(Seg{p, len, id});
        p = q;
      }
    }
    const size_t n_ids = id_len.size();

    // ---- each request's shared copies (first occurrence of a shared ID)
    std::vector<std::vector<Seg>> shared(n_req);
    std::vector<int32_t> stamp(n_ids, -1);
    for (int32_t r = 0; r < n_req; ++r)
      for (const Seg& s : segs[r])
        if (id_count[s.id] >= need && stamp[s.id] != r) {
          stamp[s.id] = r;
          shared[r].push_back(s);
        }

    // ---- groups: equal cached span, pairwise disjoint slot ranges
    std::unique_ptr<tdx_round_plan> out(new tdx_round_plan());
    std::map<std::vector<int32_t>, std::vector<int32_t>> by_span;  // span -> groups
    out->req_group.assign(n_req, -1);
    for (int32_t r = 0; r < n_req; ++r) {
      std::vector<int32_t> span;
      for (const Seg& s : shared[r]) span.push_back(s.id);
      std::sort(span.begin(), span.end());
      std::vector<int32_t>& cands = by_span[span];
      int32_t g = -1;
      for (int32_t c : cands) {
        bool clash = false;
        if (slot_begin != nullptr)
          for (int32_t m : out->groups[c].agents)
            if (slot_begin[r] < slot_end[m] && slot_begin[m] < slot_end[r]) {
              clash = true;
              break;
            }
        if (!clash) {
          g = c;
          break;
        }
      }
      if (g < 0) {
        g = static_cast<int32_t>(out->groups.size());
        out->groups.emplace_back();
        cands.push_back(g);
      }
      out->groups[g].agents.push_back(r);
      out->req_group[r] = g;
    }

    // ---- per-group layout and per-request token maps
    out->map_off.resize(n_req + 1);
    out->map_off[0] = 0;
    for (int32_t r = 0; r < n_req; ++r) out->map_off[r + 1] = out->map_off[r] + (req_off[r + 1] - req_off[r]);
    out->map.assign(static_cast<size_t>(out->map_off[n_req]), -1);
    std::vector<int32_t> pos(n_ids, -1);  // start of an ID's shared copy in the current member
    for (tdx_round_plan::Group& G : out->groups) {
      for (const Seg& s : shared[G.agents[0]]) G.seg.push_back(s.id);
      const size_t B = G.seg.size();
      G.blk_start.assign(B + 1, 0);
      int64_t T = 0;
      for (size_t b = 0; b < B; ++b) {
        T += id_len[G.seg[b]];
        if (T > INT32_MAX) return invalid("a group's shared region is longer than INT32_MAX tokens");
        G.blk_start[b + 1] = static_cast<int32_t>(T);
      }
      G.dst.assign(G.agents.size() * B, 0);
      G.priv.assign(G.agents.size(), 0);
      for (size_t i = 0; i < G.agents.size(); ++i) {
        const int32_t r = G.agents[i];
        for (const Seg& s : shared[r]) pos[s.id] = s.start;
        int32_t* m = out->map.data() + out->map_off[r];
        for (size_t b = 0; b < B; ++b) {
          const int32_t d = pos[G.seg[b]];
          G.dst[i * B + b] = d;
          for (int32_t j = 0; j < id_len[G.seg[b]]; ++j) m[d + j] = G.blk_start[b] + j;
        }
        for (const Seg& s : shared[r]) pos[s.id] = -1;
        G.priv[i] = static_cast<int32_t>((req_off[r + 1] - req_off[r]) - T);
      }
    }
    *plan = out.release();
    return tdx::report(TDX_OK, "");
  } catch (const std::bad_alloc&) {
    return tdx::report(TDX_EINTERNAL, "out of host memory");
  } catch (...) {
    return tdx::report(TDX_EINTERNAL, "unexpected exception in tdx_round_plan_build");
  }
}

int tdx_round_plan_n_groups(const tdx_round_plan* plan) {
  if (plan == nullptr) return invalid("plan is null");
  return static_cast<int>(plan->groups.size());
}

int tdx_round_plan_group_dims(const tdx_round_plan* plan, int32_t group, int32_t* n_agents, int32_t* n_blocks,
                              int32_t* n_tokens) {
  if (plan == nullptr) return invalid("plan is null");
  if (group < 0 || group >= static_cast<int32_t>(plan->groups.size())) return invalid("group out of range");
  const tdx_round_plan::Group& G = plan->groups[group];
  if (n_agents) *n_agents = static_cast<int32_t>(G.agents.size());
  if (n_blocks) *n_blocks = static_cast<int32_t>(G.seg.size());
  if (n_tokens) *n_tokens = G.blk_start.back();
  return tdx::report(TDX_OK, "");
}

int tdx_round_plan_group(const tdx_round_plan* plan, int32_t group, int32_t* agents, int32_t* seg_ids,
                         int32_t* blk_start, int32_t* src_pos, int32_t* dst_pos, int32_t* priv_len) {
  if (plan == nullptr) return invalid("plan is null");
  if (group < 0 || group >= static_cast<int32_t>(plan->groups.size())) return invalid("group out of range");
  const tdx_round_plan::Group& G = plan->groups[group];
  auto put = [](int32_t* dst, const std::vector<int32_t>& v, size_t n) {
    if (dst != nullptr && n > 0) std::memcpy(dst, v.data(), n * sizeof(int32_t));
  };
  const size_t B = G.seg.size();
  put(agents, G.agents, G.agents.size());
  put(seg_ids, G.seg, B);
  put(blk_start, G.blk_start, B + 1);
  put(src_pos, G.blk_start, B);  // a block's cached K sits at its canonical position
  put(dst_pos, G.dst, G.dst.size());
  put(priv_len, G.priv, G.priv.size());
  return tdx::report(TDX_OK, "");
}

int tdx_round_plan_request(const tdx_round_plan* plan, int32_t request, int32_t* group, int32_t* token_map) {
  if (plan == nullptr) return invalid("plan is null");
  if (request < 0 || request >= static_cast<int32_t>(plan->req_group.size())) return invalid("request out of range");
  if (group) *group = plan->req_group[request];
  if (token_map) {
    const int64_t a = plan->map_off[request], b = plan->map_off[request + 1];
    if (b > a) std::memcpy(token_map, plan->map.data() + a, static_cast<size_t>(b - a) * sizeof(int32_t));
  }
  return tdx::report(TDX_OK, "");
}

void tdx_round_plan_free(tdx_round_plan* plan) { delete plan; }

}  // extern "C"
