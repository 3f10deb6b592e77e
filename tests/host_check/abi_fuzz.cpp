// Mutation fuzz of the C entry points' host-side validation, built with AddressSanitizer and
// UndefinedBehaviorSanitizer against the HIP runtime stand-in (no GPU, no kernel runs).
//
// Every entry starts from a configuration it accepts; each call mutates up to three of its size
// arguments (neighbours, powers of two, int32 extremes, random words) and draws each pointer as
// aligned, misaligned or NULL. Properties checked on every call:
//  * the status is one of the documented codes;
//  * an error returns before any HIP call (nothing launched, no attribute set);
//  * an accepted call launches what the entry promises (one kernel, one per layer, or none for an
//    empty packed batch), within HIP's launch limits and the LDS budget (the stand-in aborts
//    otherwise);
//  * no sanitizer report (they abort the process: -fno-sanitize-recover).
// The run fails if an entry never accepts a mutated call (the fuzz would not reach the launchers).
//
// Usage: abi_fuzz [iterations per entry] [seed]
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <functional>
#include <limits>
#include <string>
#include <vector>

#include "hip_runtime_stub.h"
#include "pkc.h"

namespace {

struct Rng {
  uint64_t s;
  uint64_t next() {   // splitmix64
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  int below(int n) { return (int)(next() % (uint64_t)n); }
};

const int32_t kSpecial[] = {0, 1, -1, 2, 3, 7, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128,
                            255, 256, 257, 1 << 15, 1 << 16, 1 << 20, 1 << 23, 1 << 24,
                            (1 << 24) + 1, 1 << 29, 1 << 30, std::numeric_limits<int32_t>::max(),
                            std::numeric_limits<int32_t>::min(), -(1 << 24), -(1 << 30)};

int32_t mutate(Rng& r, int32_t v) {
  switch (r.below(5)) {
    case 0: return (int32_t)((uint32_t)v + (uint32_t)(r.below(5) - 2));   // a neighbour
    case 1: return kSpecial[r.below((int)(sizeof(kSpecial) / sizeof(kSpecial[0])))];
    case 2: return (int32_t)(uint32_t)r.next();
    case 3: return (int32_t)((uint32_t)v << (1 + r.below(4)));             // larger
    default: return (int32_t)(1u << r.below(31));
  }
}

alignas(256) unsigned char g_arena[64 * 256];

// Pointer slot i: aligned (distinct per slot), misaligned, or NULL.
const void* pick_ptr(Rng& r, int slot) {
  const int k = r.below(100);
  if (k < 2) return nullptr;
  if (k < 4) return g_arena + 256 * slot + 2 + 2 * r.below(7);
  return g_arena + 256 * slot;
}

float pick_scale(Rng& r) {
  switch (r.below(6)) {
    case 0: return 0.f;
    case 1: return -1.f;
    case 2: return std::numeric_limits<float>::quiet_NaN();
    case 3: return std::numeric_limits<float>::infinity();
    default: return 0.125f;
  }
}

bool known_status(int st) {
  return st == PKC_OK || st == PKC_ERR_NULL || st == PKC_ERR_SHAPE || st == PKC_ERR_DTYPE ||
         st == PKC_ERR_UNSUPPORTED || st == PKC_ERR_CAPACITY || st == PKC_ERR_ALIGN;
}

struct Call {
  pkc_status status;
  int expected_launches;   // when accepted
};

struct Entry {
  std::string name;
  std::vector<int32_t> base;   // sizes of an accepted call
  int n_ptr;
  std::function<Call(Rng&, const std::vector<int32_t>&, const void* const*)> call;
};

#define P(i) const_cast<void*>(p[i])
#define PI(i) static_cast<const int32_t*>(p[i])

std::vector<Entry> entries() {
  std::vector<Entry> e;
  // dtype, batch, chunk, Hk, D, block, num_blocks, max_blocks, max_cache
  e.push_back({"paged_kv_append", {1, 4, 16, 2, 64, 16, 64, 8, 100}, 8,
               [](Rng&, const std::vector<int32_t>& v, const void* const* p) {
                 return Call{paged_kv_append((pkc_dtype)v[0], p[0], p[1], P(2), P(3), PI(4), PI(5),
                                             PI(6), PI(7), v[1], v[2], v[3], v[4], v[5], v[6], v[7],
                                             v[8], nullptr),
                             1};
               }});
  // dtype, pos_len, layout, batch, chunk, H, Hk, D, block, num_blocks, max_blocks, max_cache
  const std::vector<int32_t> attn = {1, 2 * (100 + 16) - 1, 0, 4, 16, 4, 2, 64, 16, 64, 8, 100};
  e.push_back({"chunk_paged_relpos_attn", attn, 11,
               [](Rng& r, const std::vector<int32_t>& v, const void* const* p) {
                 return Call{chunk_paged_relpos_attn(
                                 (pkc_dtype)v[0], p[0], p[1], p[2], PI(3), PI(4), PI(5), PI(6),
                                 p[7], v[1], v[2], p[8], p[9], P(10), v[3], v[4], v[5], v[6], v[7],
                                 v[8], v[9], v[10], v[11], pick_scale(r), nullptr),
                             1};
               }});
  e.push_back({"paged_kv_append_relpos_attn", attn, 13,
               [](Rng& r, const std::vector<int32_t>& v, const void* const* p) {
                 return Call{paged_kv_append_relpos_attn(
                                 (pkc_dtype)v[0], p[0], p[1], p[2], P(3), P(4), PI(5), PI(6),
                                 PI(7), PI(8), p[9], v[1], v[2], p[10], p[11], P(12), v[3], v[4],
                                 v[5], v[6], v[7], v[8], v[9], v[10], v[11], pick_scale(r),
                                 nullptr),
                             1};
               }});
  // dtype, pos_len, layout, batch, chunk, H, Hk, D, block, num_blocks, max_blocks, max_cache
  e.push_back({"paged_kv_append_relpos_attn_layers", attn, 13,
               [](Rng& r, const std::vector<int32_t>& v, const void* const* p) {
                 const int choices[] = {-1, 0, 1, 2, 3, 8};
                 const int n = r.below(8) < 6 ? 2 : choices[r.below(6)];
                 std::vector<const void*> q, kn, vn, pos, u, w;
                 std::vector<void*> kp, vp, out;
                 for (int l = 0; l < (n > 0 ? n : 0); ++l) {
                   // a NULL or misaligned entry now and then, in one layer only
                   const bool bad = r.below(40) == 0;
                   q.push_back(bad ? p[0] : g_arena + 256 * (16 + l));
                   kn.push_back(p[1]);
                   vn.push_back(p[2]);
                   kp.push_back(P(3));
                   vp.push_back(P(4));
                   pos.push_back(p[9]);
                   u.push_back(p[10]);
                   w.push_back(p[11]);
                   out.push_back(P(12));
                 }
                 return Call{paged_kv_append_relpos_attn_layers(
                                 (pkc_dtype)v[0], n, q.data(), kn.data(), vn.data(), kp.data(),
                                 vp.data(), PI(5), PI(6), PI(7), PI(8), pos.data(), v[1], v[2],
                                 u.data(), w.data(), out.data(), v[3], v[4], v[5], v[6], v[7],
                                 v[8], v[9], v[10], v[11], pick_scale(r), nullptr),
                             n};
               }});
  // dtype, pos_len, layout, batch, chunk, H, Hk, D, block, num_blocks, max_blocks, max_cache,
  // waves, split, reads
  std::vector<int32_t> gather = attn;
  gather.insert(gather.end(), {4, 1, 1});
  e.push_back({"pkc_gather_read", gather, 13,
               [](Rng&, const std::vector<int32_t>& v, const void* const* p) {
                 return Call{pkc_gather_read((pkc_dtype)v[0], p[0], p[1], p[2], P(3), P(4), PI(5),
                                             PI(6), p[7], v[1], v[2], p[8], p[9], P(10), v[3],
                                             v[4], v[5], v[6], v[7], v[8], v[9], v[10], v[11],
                                             v[12], v[13], v[14], nullptr),
                             1};
               }});
  // max_cached, batch, chunk, block
  e.push_back({"paged_kv_commit", {64, 4, 16, 16}, 3,
               [](Rng&, const std::vector<int32_t>& v, const void* const* p) {
                 return Call{paged_kv_commit(const_cast<int32_t*>(PI(0)), PI(1),
                                             const_cast<int32_t*>(PI(2)), v[0], v[1], v[2], v[3],
                                             nullptr),
                             1};
               }});
  // dtype, num_seqs, total, max_seqlen, H, Hk, D, mask_chunk, mask_left
  e.push_back({"varlen_packed_relpos_attn", {1, 4, 300, 120, 4, 4, 64, 0, 0}, 8,
               [](Rng& r, const std::vector<int32_t>& v, const void* const* p) {
                 const pkc_status st = varlen_packed_relpos_attn(
                     (pkc_dtype)v[0], p[0], p[1], p[2], PI(3), v[1], v[2], v[3], p[4], p[5], p[6],
                     P(7), v[4], v[5], v[6], v[7], v[8], pick_scale(r), nullptr);
                 return Call{st, (v[2] == 0 || v[3] == 0) ? 0 : 1};
               }});
  // dtype, M, N, K
  e.push_back({"pkc_linear", {1, 1000, 768, 256}, 4,
               [](Rng&, const std::vector<int32_t>& v, const void* const* p) {
                 return Call{pkc_linear((pkc_dtype)v[0], p[0], p[1], p[2], P(3), v[1], v[2], v[3],
                                        nullptr),
                             1};
               }});
  // dtype, batch, chunk, d_model, H, Hk, D, block, num_blocks, max_blocks, max_cache
  e.push_back({"paged_kv_qkv_append", {1, 4, 16, 256, 4, 2, 64, 16, 64, 8, 100}, 11,
               [](Rng&, const std::vector<int32_t>& v, const void* const* p) {
                 return Call{paged_kv_qkv_append((pkc_dtype)v[0], p[0], p[1], p[2], P(3), P(4),
                                                 P(5), PI(6), PI(7), PI(8), PI(9), v[1], v[2],
                                                 v[3], v[4], v[5], v[6], v[7], v[8], v[9], v[10],
                                                 nullptr),
                             1};
               }});
  // dtype, pos_first, pos_step, n_tables, rows, d_model, out_features
  e.push_back({"rel_pos_projection", {1, 271, -1, 1, 543, 256, 256}, 3,
               [](Rng&, const std::vector<int32_t>& v, const void* const* p) {
                 // pos_start (p[1]) is optional: NULL selects pos_first
                 return Call{rel_pos_projection((pkc_dtype)v[0], p[0], PI(1), v[1], v[2], v[3],
                                                v[4], v[5], v[6], P(2), nullptr),
                             1};
               }});
  return e;
}

}  // namespace

int main(int argc, char** argv) {
  const long iters = argc > 1 ? std::atol(argv[1]) : 20000;
  const uint64_t seed = argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 1;
  if (pkc_version() <= 0 || std::string(pkc_status_string(PKC_ERR_SHAPE)).empty()) return 2;
  int failures = 0;
  for (const Entry& en : entries()) {
    Rng r{seed * 1000003ull + std::hash<std::string>{}(en.name)};
    long accepted = 0, mutated_accepted = 0;
    for (long it = 0; it <= iters; ++it) {
      std::vector<int32_t> v = en.base;
      std::vector<const void*> p(en.n_ptr);
      const bool plain = it == 0;   // the base call: every pointer aligned, sizes unmutated
      const int n_mut = plain ? 0 : r.below(4);
      for (int m = 0; m < n_mut; ++m) {
        const int i = r.below((int)v.size());
        v[i] = mutate(r, v[i]);
      }
      for (int i = 0; i < en.n_ptr; ++i)
        p[i] = plain ? g_arena + 256 * i : pick_ptr(r, i);
      stub_clear();
      const Call c = en.call(r, v, p.data());
      const int st = c.status;
      const size_t launched = stub_launches().size();
      bool bad = false;
      if (!known_status(st)) {
        std::fprintf(stderr, "%s: unknown status %d\n", en.name.c_str(), st);
        bad = true;
      } else if (st != PKC_OK && stub_hip_calls() != 0) {
        std::fprintf(stderr, "%s: status %d after %ld HIP calls\n", en.name.c_str(), st,
                     stub_hip_calls());
        bad = true;
      } else if (st == PKC_OK && (long)launched != c.expected_launches) {
        std::fprintf(stderr, "%s: accepted with %zu launches (%ld HIP calls), expected %d\n",
                     en.name.c_str(), launched, stub_hip_calls(), c.expected_launches);
        bad = true;
      } else if (plain && st != PKC_OK) {
        std::fprintf(stderr, "%s: base call refused with status %d\n", en.name.c_str(), st);
        bad = true;
      }
      if (bad) {
        std::fprintf(stderr, "  iteration %ld sizes:", it);
        for (int32_t x : v) std::fprintf(stderr, " %d", x);
        std::fprintf(stderr, "\n");
        ++failures;
        break;
      }
      if (st == PKC_OK) {
        ++accepted;
        if (n_mut > 0) ++mutated_accepted;
      }
    }
    std::printf("%-36s accepted %ld of %ld (%ld mutated)\n", en.name.c_str(), accepted, iters + 1,
                mutated_accepted);
    if (mutated_accepted == 0) {
      std::fprintf(stderr, "%s: no mutated call accepted\n", en.name.c_str());
      ++failures;
    }
  }
  std::printf(failures ? "FAILED\n" : "OK\n");
  return failures ? 1 : 0;
}
