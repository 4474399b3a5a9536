// Host control plane: fingerprint dedup with refcounts, master/mirror delta
// tables, RoPE shifts, and the device work plan (kvpool_build_tables).
//
// Dedup follows the INMS walkthrough (sec. 2.2: fixed-size blocks, a content
// fingerprint looked up in the pool of the block's tier, hit -> reuse and
// refcount + 1, miss -> new block; sec. 3.2: a hash match must also match the
// tier) and the TokenDance write-up (sec. 1: segments indexed by their own
// content; sec. 3: one master plus block-sparse mirrors).  The fingerprint is
// word-wise FNV-1a-64 over the key (shared-memory prefix cache blog, sec. 3.2),
// kept in an open-addressing table; every hash hit is confirmed by comparing
// the full key, so hash collisions never merge different content.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <new>
#include <numeric>
#include <string>
#include <unordered_map>
#include <vector>

#include "kvpool.h"
#include "kvpool_internal.h"
#include "kvpool_mirror.h"

namespace kvp {

// fixed storage: recording a failure never allocates (and so never throws)
thread_local char g_last_error[256];
static int g_hash_bits = 64;

int fail(int code, const char* msg) {
  snprintf(g_last_error, sizeof g_last_error, "%s", msg ? msg : "");
  return code;
}

static constexpr uint64_t kFnvBasis = 1469598103934665603ull;
static constexpr uint64_t kFnvPrime = 1099511628211ull;

static inline uint64_t fnv_word(uint64_t h, uint32_t w) {
  h ^= (uint64_t)w;
  h *= kFnvPrime;
  return h;
}

}  // namespace kvp

using namespace kvp;

namespace {

// Key of one block: everything that decides whether two blocks hold the same
// cached content.  tokens point into the caller's arrays (valid for the call).
struct BlockKey {
  int32_t tier, group, priv_agent, priv_span, parent, ntok;
  const int32_t* tokens;
};

constexpr int32_t kAgentRoot = -1;
constexpr int32_t kSegRoot = -2;

uint64_t key_hash(const BlockKey& k) {
  uint64_t h = kFnvBasis;
  h = fnv_word(h, (uint32_t)k.tier);
  h = fnv_word(h, (uint32_t)k.group);
  h = fnv_word(h, (uint32_t)k.priv_agent);
  h = fnv_word(h, (uint32_t)k.priv_span);
  h = fnv_word(h, (uint32_t)k.parent);
  h = fnv_word(h, (uint32_t)k.ntok);
  for (int32_t i = 0; i < k.ntok; ++i) h = fnv_word(h, (uint32_t)k.tokens[i]);
  if (g_hash_bits < 64) h &= ((1ull << g_hash_bits) - 1);
  return h;
}

bool key_equal(const BlockKey& a, const BlockKey& b) {
  return a.tier == b.tier && a.group == b.group && a.priv_agent == b.priv_agent &&
         a.priv_span == b.priv_span && a.parent == b.parent && a.ntok == b.ntok &&
         std::memcmp(a.tokens, b.tokens, sizeof(int32_t) * (size_t)a.ntok) == 0;
}

// Open-addressing (linear probing) fingerprint table: slot -> physical id.
struct FingerprintTable {
  std::vector<uint64_t> hash;
  std::vector<int32_t> id;
  uint64_t mask_ = 0;
  explicit FingerprintTable(size_t n_keys) {
    size_t cap = 16;
    while (cap < 2 * n_keys + 16) cap <<= 1;
    hash.assign(cap, 0);
    id.assign(cap, -1);
    mask_ = cap - 1;
  }
  // Returns the id of an equal key, or inserts new_id and returns it.
  int32_t find_or_insert(const BlockKey& k, const std::vector<BlockKey>& keys, int32_t new_id) {
    uint64_t h = key_hash(k);
    uint64_t s = (h ^ (h >> 29)) * 0xbf58476d1ce4e5b9ull;
    for (uint64_t i = s & mask_;; i = (i + 1) & mask_) {
      if (id[i] < 0) {
        hash[i] = h;
        id[i] = new_id;
        return new_id;
      }
      if (hash[i] == h && key_equal(keys[(size_t)id[i]], k)) return id[i];
    }
  }
};

struct ConsRef {
  int32_t qc;       // unique (agent, shift) consumer
  bool reads;       // false: overlaid by a delta (masked out)
};

int validate_shape(const kvp_shape* s) {
  if (!s) return fail(KVP_EINVAL, "shape is NULL");
  if (s->n_layers < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1 || s->n_q_heads % s->n_kv_heads)
    return fail(KVP_EINVAL, "bad head or layer counts (n_q_heads must be a multiple of n_kv_heads)");
  if (s->n_q_heads / s->n_kv_heads > kMaxRowsValu)
    return fail(KVP_EINVAL, "more than 16 q heads per kv head is not supported");
  if (s->head_dim != 64 && s->head_dim != 128) return fail(KVP_EINVAL, "head_dim must be 64 or 128");
  if (s->block_tokens != 16 && s->block_tokens != 256) return fail(KVP_EINVAL, "block_tokens must be 16 or 256");
  if (s->kv_dtype != KVP_BF16 && s->kv_dtype != KVP_Q4G64) return fail(KVP_EINVAL, "kv_dtype");
  if (!(s->rope_theta > 0.f) || !std::isfinite(s->rope_theta)) return fail(KVP_EINVAL, "rope_theta");
  return KVP_OK;
}

}  // namespace

namespace kvp {
int check_shape(const kvp_shape* s) { return validate_shape(s); }

int64_t block_head_bytes(const kvp_shape* s, int32_t ntok) {
  int64_t per = s->kv_dtype == KVP_BF16 ? 2LL * s->head_dim * 2 : 2LL * (s->head_dim / 2 + (s->head_dim / 64) * 4);
  return per * ntok;
}
}  // namespace kvp

// ----------------------------------------------------------------------------
// work plan

namespace kvp {
void build_plan(const kvp_shape* sh, kvp_tables* t) {
  const int32_t n = t->n_agents, M = t->max_blocks;
  const int32_t group = sh->n_q_heads / sh->n_kv_heads;

  // unique (agent, shift) consumers, in first-use order
  std::unordered_map<uint64_t, int32_t> qc_of;
  auto qc_id = [&](int32_t j, int32_t s) {
    uint64_t key = ((uint64_t)(uint32_t)j << 32) | (uint32_t)s;
    auto it = qc_of.find(key);
    if (it != qc_of.end()) return it->second;
    int32_t id = (int32_t)(t->qcons.size() / 2);
    t->qcons.push_back(j);
    t->qcons.push_back(s);
    qc_of.emplace(key, id);
    return id;
  };

  // consumers of every physical block
  std::vector<std::vector<ConsRef>> users((size_t)t->n_phys);
  for (int32_t j = 0; j < n; ++j) {
    for (int32_t b = 0; b < t->n_blocks[(size_t)j]; ++b) {
      size_t e = (size_t)j * M + b;
      int32_t p = t->block_table[e], d = t->delta_table[e], s = t->shift[e];
      int32_t q = qc_id(j, s);
      users[(size_t)p].push_back({q, d < 0});
      if (d >= 0) users[(size_t)d].push_back({q, true});
    }
  }

  // group blocks that have the same consumer list into runs
  struct Run {
    std::vector<int32_t> cons;   // qcons ids, sorted
    std::vector<int32_t> blocks; // physical ids, ascending
    std::vector<std::vector<uint8_t>> reads;  // [block][consumer]
  };
  std::vector<Run> runs;
  std::unordered_map<std::string, int32_t> run_of;
  for (int32_t p = 0; p < t->n_phys; ++p) {
    auto& u = users[(size_t)p];
    bool any = false;
    for (auto& c : u) any |= c.reads;
    if (!any) continue;  // nobody reads this block
    std::sort(u.begin(), u.end(), [](const ConsRef& a, const ConsRef& b) { return a.qc < b.qc; });
    std::string sig((const char*)nullptr, 0);
    sig.reserve(u.size() * 4);
    for (auto& c : u) sig.append((const char*)&c.qc, 4);
    auto it = run_of.find(sig);
    int32_t r;
    if (it == run_of.end()) {
      r = (int32_t)runs.size();
      run_of.emplace(sig, r);
      runs.emplace_back();
      for (auto& c : u) runs.back().cons.push_back(c.qc);
    } else {
      r = it->second;
    }
    runs[(size_t)r].blocks.push_back(p);
    std::vector<uint8_t> rd(u.size());
    for (size_t i = 0; i < u.size(); ++i) rd[i] = u[i].reads ? 1 : 0;
    runs[(size_t)r].reads.push_back(std::move(rd));
  }

  int64_t total_block_heads = 0;
  for (auto& r : runs) total_block_heads += (int64_t)r.blocks.size() * sh->n_kv_heads;
  int32_t tiles_per_block = sh->block_tokens / 16;
  int64_t units = total_block_heads * tiles_per_block;
  // an item is processed by a workgroup of 4 waves; aim at ~256 (item, kv head)
  // units of 8..256 tiles each (measured: every item pays a start-up latency of
  // a few microseconds, which larger items amortise; the tail is split below)
  // Q4 tiles are bound by their conversion work rather than by HBM: aim at one
  // round of ~512 equal units (two resident workgroups per CU), see below
  const int64_t unit_div = sh->kv_dtype == KVP_Q4G64 ? 512 : 256;
  int32_t cb_tiles = (int32_t)std::min<int64_t>(256, std::max<int64_t>(8, (units + unit_div - 1) / unit_div));

  const int32_t cons_per_item = std::max(1, kMaxRowsValu / group);
  const bool mfma_rows = sh->kv_dtype == KVP_BF16;  // bf16 items of > 4 rows run on MFMA
  // blocks read by many consumers go to wide items (up to 128 rows) for bf16
  // pools of 16-token blocks; otherwise their consumers are split into narrow items
  const bool wide_rows = mfma_rows && sh->block_tokens == 16;

  // 1. chunks: (run, block range, consumer range)
  struct Chunk {
    int32_t run, b0, b1, c0, c1;
  };
  std::vector<Chunk> chunks;
  for (int32_t ri = 0; ri < (int32_t)runs.size(); ++ri) {
    const Run& r = runs[(size_t)ri];
    int32_t nb = (int32_t)r.blocks.size();
    int32_t nc = (int32_t)r.cons.size();
    // bf16 blocks read by more rows than a narrow item holds go to wide items
    const int32_t cpi = (wide_rows && nc * group > kMaxRowsValu) ? std::max(1, std::min(kMaxConsWide, kMaxRowsWide / group)) : cons_per_item;
    // VALU items' work grows with their rows: give 2..4-row bf16 items fewer tiles
    // (Q4 items of more than one row run on MFMA)
    const int32_t rows_item = std::min(nc, cpi) * group;
    const bool valu_multi = rows_item > 1 && mfma_rows && rows_item <= 4;
    int32_t run_tiles = valu_multi ? std::max(8, cb_tiles * 4 / (3 + rows_item)) : cb_tiles;
    // wide items of more than 64 rows do twice the work per tile: half the tiles
    if (mfma_rows && rows_item > 64) run_tiles = std::max(8, run_tiles / 2);
    // keep the partials an item writes (rows x (head_dim + 2) floats) under ~1/16
    // of the K/V bytes it reads (counted for at most 64 rows: wider items are
    // bound by their matrix work, and their K/V reads are shared in L2)
    const int64_t tile_bytes = block_head_bytes(sh, 16);
    const int64_t min_tiles =
        (16LL * std::min<int32_t>(rows_item, 64) * (sh->head_dim + 2) * 4 + tile_bytes - 1) / tile_bytes;
    run_tiles = (int32_t)std::max<int64_t>(run_tiles, std::min<int64_t>(min_tiles, 1024));
    int32_t cb = std::max(1, run_tiles / tiles_per_block);
    if (rows_item > kMaxRowsValu) cb = std::min(cb, kMaxBlocksWide);
    int32_t nchunk = (nb + cb - 1) / cb;
    // Q4: round the chunk count down (chunks a little above the target size) so
    // that the units fit one round
    // (never more chunks than blocks: an empty item would only write an empty partial)
    if (sh->kv_dtype == KVP_Q4G64)
      nchunk = std::min<int32_t>(nb, std::max<int32_t>(1, (int32_t)((int64_t)nb * tiles_per_block / run_tiles)));
    for (int32_t k = 0; k < nchunk; ++k) {
      int32_t b0 = (int32_t)((int64_t)nb * k / nchunk), b1 = (int32_t)((int64_t)nb * (k + 1) / nchunk);
      // consumers split into equal groups of at most cpi
      const int32_t ng = (nc + cpi - 1) / cpi;
      for (int32_t k2 = 0; k2 < ng; ++k2) chunks.push_back({ri, b0, b1, nc * k2 / ng, nc * (k2 + 1) / ng});
    }
  }
  // 2. dispatch order: more rows first (heavier per tile), then longer chunks
  //    first (the longest work starts earliest); equal chunks keep their order
  //    (consumer groups of one chunk stay adjacent)
  std::stable_sort(chunks.begin(), chunks.end(), [&](const Chunk& x, const Chunk& y) {
    const int cx = row_class((x.c1 - x.c0) * group), cy = row_class((y.c1 - y.c0) * group);
    if (cx != cy) return cx > cy;
    return (x.b1 - x.b0) > (y.b1 - y.b0);
  });
  // 2b. wide items whose (item, kv head) units need more than one round of
  //     workgroup slots (two per CU on 256 CUs) are spread through the narrow
  //     items instead of going first: the matrix-bound wide workgroups then
  //     share CUs with the HBM-bound narrow ones.  Fewer wide units go first,
  //     being the longest work.  The wide items go in bursts of whole consumer
  //     groups (the items over one block range, adjacent so that they share
  //     the block in L2) of about half a round of slots.  Measured on one box
  //     (tile pass of the scale round's layer, HBM reads over unique bytes):
  //     wide first 1202 us, spread one group at a time 1113-1119 us (1.053),
  //     in bursts of 2, 3, 4 and 6 groups 1109 (1.045), 1078-1082 (1.035),
  //     1130 (1.040) and 1187 us (1.014); TokenDance's 264 wide units spread:
  //     40 % slower.
  {
    constexpr int64_t kSlots = 512;
    std::vector<Chunk> wide, narrow;
    for (auto& c : chunks) ((wide_rows && (c.c1 - c.c0) * group > kMaxRowsValu) ? wide : narrow).push_back(c);
    if ((int64_t)wide.size() * sh->n_kv_heads > kSlots && !narrow.empty()) {
      std::vector<std::vector<Chunk>> groups;
      for (auto& c : wide) {
        if (groups.empty() || groups.back().back().run != c.run || groups.back().back().b0 != c.b0) groups.emplace_back();
        groups.back().push_back(c);
      }
      const int64_t gunits = (int64_t)groups[0].size() * sh->n_kv_heads;
      const size_t burst = (size_t)std::max<int64_t>(1, (kSlots / 2 + gunits / 2) / gunits);
      std::vector<Chunk> out;
      out.reserve(chunks.size());
      size_t ni = 0;
      for (size_t gi = 0; gi < groups.size(); ++gi) {
        const size_t until = narrow.size() * (gi / burst * burst) / groups.size();
        while (ni < until) out.push_back(narrow[ni++]);
        out.insert(out.end(), groups[gi].begin(), groups[gi].end());
      }
      while (ni < narrow.size()) out.push_back(narrow[ni++]);
      chunks.swap(out);
    }
  }
  // consecutive chunks over the same blocks (consumer groups) should share an XCD
  {
    int32_t g_max = 1;
    for (auto& r : runs) {
      const int32_t nc = (int32_t)r.cons.size();
      const int32_t cpi = (wide_rows && nc * group > kMaxRowsValu) ? std::max(1, std::min(kMaxConsWide, kMaxRowsWide / group)) : cons_per_item;
      g_max = std::max<int32_t>(g_max, (nc + cpi - 1) / cpi);
    }
    t->unit_span = std::max(1, std::min(512, g_max * sh->n_kv_heads));
    t->unit_span = std::max(t->unit_span, 2 * sh->n_kv_heads);
  }
  // 3. the last quarter of the work is cut into quarter-size items, so that the
  //    end of the launch is filled with short items (less idle time at the tail);
  //    not for Q4, whose equal units already fit one round, and not when the plan
  //    has wide items: those start first and run longest, the narrow items already
  //    fill the end, and splitting them only adds per-item start-up (measured:
  //    TokenDance and the scale round 3-4 % faster without the split, the
  //    narrow-only INMS round 1 % slower)
  {
    bool has_wide = false;
    for (auto& c : chunks) has_wide |= wide_rows && (c.c1 - c.c0) * group > kMaxRowsValu;
    int64_t total = 0;
    for (auto& c : chunks) total += c.b1 - c.b0;
    int64_t tail = 0;
    size_t first_tail = chunks.size();
    while (sh->kv_dtype != KVP_Q4G64 && !has_wide && first_tail > 0 &&
           4 * (tail + chunks[first_tail - 1].b1 - chunks[first_tail - 1].b0) <= total) {
      --first_tail;
      tail += chunks[first_tail].b1 - chunks[first_tail].b0;
    }
    std::vector<Chunk> split(chunks.begin(), chunks.begin() + (ptrdiff_t)first_tail);
    for (size_t i = first_tail; i < chunks.size(); ++i) {
      const Chunk& c = chunks[i];
      const int32_t nb = c.b1 - c.b0, np = std::min(4, nb);
      for (int32_t k = 0; k < np; ++k)
        split.push_back({c.run, c.b0 + nb * k / np, c.b0 + nb * (k + 1) / np, c.c0, c.c1});
    }
    chunks.swap(split);
  }
  // 4. items
  std::vector<std::vector<int32_t>> comb((size_t)n);
  int32_t part = 0;
  for (const Chunk& ch : chunks) {
    const Run& r = runs[(size_t)ch.run];
    const int32_t b0 = ch.b0, b1 = ch.b1, c0 = ch.c0, c1 = ch.c1;
    int32_t pb0 = (int32_t)t->plan_blocks.size();
    for (int32_t b = b0; b < b1; ++b) t->plan_blocks.push_back(r.blocks[(size_t)b]);
    int32_t pb1 = (int32_t)t->plan_blocks.size();
    // mask words only if some consumer skips some block of this chunk
    bool full = true;
    for (int32_t b = b0; b < b1 && full; ++b)
      for (int32_t c = c0; c < c1; ++c) full &= r.reads[(size_t)b][(size_t)c] != 0;
    kvp_item it{};
    it.blk_begin = pb0;
    it.blk_end = pb1;
    it.cons_begin = (int32_t)t->cons.size();
    for (int32_t c = c0; c < c1; ++c) t->cons.push_back(r.cons[(size_t)c]);
    it.cons_end = (int32_t)t->cons.size();
    it.rows = (c1 - c0) * group;
    it.part_base = part;
    it.mask_stride = (c1 - c0 + 31) / 32;
    if (full) {
      it.mask_base = -1;
    } else {
      it.mask_base = (int32_t)t->mask.size();
      for (int32_t b = b0; b < b1; ++b) {
        for (int32_t w = 0; w < it.mask_stride; ++w) {
          uint32_t word = 0;
          for (int32_t c = c0 + 32 * w; c < std::min(c1, c0 + 32 * (w + 1)); ++c)
            if (r.reads[(size_t)b][(size_t)c]) word |= 1u << (c - c0 - 32 * w);
          t->mask.push_back(word);
        }
      }
    }
    for (int32_t c = c0; c < c1; ++c) {
      int32_t j = t->qcons[2 * (size_t)r.cons[(size_t)c]];
      comb[(size_t)j].push_back(part + (c - c0) * group);
    }
    part += it.rows;
    t->items.push_back(it);
  }
  for (auto& it : t->items) t->class_items[row_class_index(it.rows)] += 1;

  // unshifted consumers first (the kernels read their queries as they are);
  // shifted ones last (their rotated queries are prepared per call)
  {
    const size_t nq = t->qcons.size() / 2;
    std::vector<int32_t> newid(nq);
    std::vector<int32_t> reordered;
    reordered.reserve(t->qcons.size());
    int32_t k = 0;
    for (int pass = 0; pass < 2; ++pass)
      for (size_t q = 0; q < nq; ++q)
        if ((t->qcons[2 * q + 1] != 0) == (pass == 1)) {
          newid[q] = k++;
          reordered.push_back(t->qcons[2 * q]);
          reordered.push_back(t->qcons[2 * q + 1]);
          if (pass == 1) t->n_qcons_shifted += 1;
        }
    t->qcons.swap(reordered);
    for (auto& c : t->cons) c = newid[(size_t)c];
  }
  t->n_part_rows = part;
  t->comb_ptr.assign((size_t)n + 1, 0);
  for (int32_t j = 0; j < n; ++j) {
    std::sort(comb[(size_t)j].begin(), comb[(size_t)j].end());
    t->comb_ptr[(size_t)j + 1] = t->comb_ptr[(size_t)j] + (int32_t)comb[(size_t)j].size();
    t->comb_rows.insert(t->comb_rows.end(), comb[(size_t)j].begin(), comb[(size_t)j].end());
  }
  // derived lookups, so that a workgroup reaches its blocks' token counts and its
  // consumers' query rows in one dependent load less
  t->plan_ntok.resize(t->plan_blocks.size());
  for (size_t i = 0; i < t->plan_blocks.size(); ++i) t->plan_ntok[i] = t->phys_ntok[(size_t)t->plan_blocks[i]];
  const int32_t n_unshifted = (int32_t)(t->qcons.size() / 2) - t->n_qcons_shifted;
  t->cons_row.resize(t->cons.size());
  for (size_t i = 0; i < t->cons.size(); ++i) {
    const int32_t c = t->cons[i];
    t->cons_row[i] = c < n_unshifted ? t->qcons[2 * (size_t)c] : c - n_unshifted;
  }
  // the rotation R(-shift) of each shifted consumer's query (INMS walkthrough
  // sec. 3.2: the compensation of a move depends on the position difference
  // only): cos and sin of -shift * theta_i, theta_i = rope_theta^(-2i/d), the
  // angle formed in double and both rounded to float
  const int32_t half = sh->head_dim / 2;
  t->rope_cs.assign((size_t)t->n_qcons_shifted * half * 2, 0.f);
  for (int32_t k = 0; k < t->n_qcons_shifted; ++k) {
    const double delta = (double)t->qcons[2 * (size_t)(n_unshifted + k) + 1];
    for (int32_t i = 0; i < half; ++i) {
      const double ang = -delta * std::pow((double)sh->rope_theta, -2.0 * (double)i / (double)sh->head_dim);
      t->rope_cs[((size_t)k * half + i) * 2] = (float)std::cos(ang);
      t->rope_cs[((size_t)k * half + i) * 2 + 1] = (float)std::sin(ang);
    }
  }
  int64_t ub = 0;
  for (int32_t p = 0; p < t->n_phys; ++p) ub += block_head_bytes(sh, t->phys_ntok[(size_t)p]);
  t->unique_kv_bytes = ub * sh->n_kv_heads;
}
}  // namespace kvp

namespace kvp {
int check_plan_bounds(const kvp_shape* sh, const kvp_tables* t) {
  char msg[160];
  auto bad = [&](const char* what, int64_t i) {
    snprintf(msg, sizeof msg, "internal: work plan index out of range (%s, entry %lld)", what, (long long)i);
    return fail(KVP_EINVAL, msg);
  };
  const int64_t n_phys = t->n_phys, n_pb = (int64_t)t->plan_blocks.size(), n_cons = (int64_t)t->cons.size();
  const int64_t n_qcons = (int64_t)t->qcons.size() / 2, n_mask = (int64_t)t->mask.size();
  const int32_t group = sh->n_q_heads / sh->n_kv_heads;
  if ((int64_t)t->phys_ntok.size() != n_phys) return bad("phys_ntok size", n_phys);
  for (int64_t p = 0; p < n_phys; ++p)
    if (t->phys_ntok[(size_t)p] < 0 || t->phys_ntok[(size_t)p] > sh->block_tokens) return bad("phys_ntok", p);
  for (int64_t i = 0; i < n_pb; ++i)
    if (t->plan_blocks[(size_t)i] < 0 || t->plan_blocks[(size_t)i] >= n_phys) return bad("plan_blocks", i);
  for (int64_t i = 0; i < n_cons; ++i)
    if (t->cons[(size_t)i] < 0 || t->cons[(size_t)i] >= n_qcons) return bad("cons", i);
  // the derived lookups agree with what they are derived from
  if ((int64_t)t->plan_ntok.size() != n_pb) return bad("plan_ntok size", n_pb);
  for (int64_t i = 0; i < n_pb; ++i)
    if (t->plan_ntok[(size_t)i] != t->phys_ntok[(size_t)t->plan_blocks[(size_t)i]]) return bad("plan_ntok", i);
  if ((int64_t)t->cons_row.size() != n_cons) return bad("cons_row size", n_cons);
  if ((int64_t)t->rope_cs.size() != (int64_t)t->n_qcons_shifted * sh->head_dim)
    return bad("rope_cs size", (int64_t)t->rope_cs.size());
  for (int64_t i = 0; i < n_cons; ++i) {
    const int64_t c = t->cons[(size_t)i], nu = n_qcons - t->n_qcons_shifted;
    if (t->cons_row[(size_t)i] != (c < nu ? t->qcons[2 * (size_t)c] : c - nu)) return bad("cons_row", i);
  }
  for (int64_t i = 0; i < n_qcons; ++i) {
    if (t->qcons[2 * (size_t)i] < 0 || t->qcons[2 * (size_t)i] >= t->n_agents) return bad("qcons agent", i);
    // shifted consumers come last (their rotated queries are indexed from the first of them)
    if ((t->qcons[2 * (size_t)i + 1] != 0) != (i >= n_qcons - t->n_qcons_shifted)) return bad("qcons order", i);
  }
  int64_t rows = 0;
  for (size_t k = 0; k < t->items.size(); ++k) {
    const kvp_item& it = t->items[k];
    const int64_t nb = (int64_t)it.blk_end - it.blk_begin, nc = (int64_t)it.cons_end - it.cons_begin;
    if (it.blk_begin < 0 || nb < 1 || it.blk_end > n_pb) return bad("item blocks", (int64_t)k);
    if (it.cons_begin < 0 || nc < 1 || it.cons_end > n_cons) return bad("item consumers", (int64_t)k);
    // wide items (more than 16 rows): bf16 pools of 16-token blocks only
    const bool wide_ok = sh->kv_dtype == KVP_BF16 && sh->block_tokens == 16;
    if (it.rows != nc * group || it.rows < 1 || it.rows > (wide_ok ? kMaxRowsWide : kMaxRowsValu) ||
        (it.rows > kMaxRowsValu && nc > kMaxConsWide))
      return bad("item rows", (int64_t)k);
    if (it.rows > kMaxRowsValu && nb > kMaxBlocksWide) return bad("wide item blocks", (int64_t)k);
    if (it.part_base != rows || (int64_t)it.part_base + it.rows > t->n_part_rows) return bad("item partial rows", (int64_t)k);
    rows += it.rows;
    if (it.mask_base >= 0) {
      if (it.mask_stride != (nc + 31) / 32 || (int64_t)it.mask_base + nb * it.mask_stride > n_mask)
        return bad("item mask", (int64_t)k);
    } else if (it.mask_base != -1) {
      return bad("item mask", (int64_t)k);
    }
  }
  if (rows != t->n_part_rows) return bad("partial row count", rows);
  if ((int64_t)t->comb_ptr.size() != (int64_t)t->n_agents + 1 || t->comb_ptr[0] != 0 ||
      t->comb_ptr[(size_t)t->n_agents] != (int32_t)t->comb_rows.size())
    return bad("comb_ptr", 0);
  for (int32_t j = 0; j < t->n_agents; ++j)
    if (t->comb_ptr[(size_t)j + 1] < t->comb_ptr[(size_t)j]) return bad("comb_ptr", j);
  for (size_t i = 0; i < t->comb_rows.size(); ++i)
    if (t->comb_rows[i] < 0 || (int64_t)t->comb_rows[i] + group > t->n_part_rows) return bad("comb_rows", (int64_t)i);
  return KVP_OK;
}
}  // namespace kvp

// ----------------------------------------------------------------------------
// tables

static int build(const kvp_shape* sh, const kvp_agent* agents, int32_t n, kvp_tables* t) {
  const int32_t B = sh->block_tokens;
  // count logical blocks and validate spans
  std::vector<int32_t> m((size_t)n, 0);
  int64_t total = 0;
  for (int32_t j = 0; j < n; ++j) {
    const kvp_agent& a = agents[j];
    if (a.n_spans < 0 || (a.n_spans > 0 && !a.spans)) return fail(KVP_EINVAL, "agent spans");
    if (a.n_delta < 0 || (a.n_delta > 0 && !a.delta_blocks)) return fail(KVP_EINVAL, "agent deltas");
    int64_t mb = 0;
    for (int32_t s = 0; s < a.n_spans; ++s) {
      const kvp_span& sp = a.spans[s];
      if (sp.n_tokens < 0 || (sp.n_tokens > 0 && !sp.tokens)) return fail(KVP_EINVAL, "span tokens");
      if (sp.tier < KVP_GLOBAL || sp.tier > KVP_PRIVATE || sp.kind < KVP_PREFIX || sp.kind > KVP_SEGMENT)
        return fail(KVP_EINVAL, "span tier or kind");
      if (sp.tier == KVP_GROUP && sp.group < 0) return fail(KVP_ETIER, "GROUP span without a group id");
      mb += (sp.n_tokens + B - 1) / B;
    }
    if (mb > INT32_MAX / 2) return fail(KVP_EINVAL, "too many blocks");
    m[(size_t)j] = (int32_t)mb;
    total += mb;
  }
  if (total > INT32_MAX / 2) return fail(KVP_EINVAL, "too many blocks");
  int32_t M = 0;
  for (auto x : m) M = std::max(M, x);
  t->n_agents = n;
  t->max_blocks = M;
  t->n_blocks = m;
  size_t cells = (size_t)n * (size_t)M;
  t->block_table.assign(cells, -1);
  t->delta_table.assign(cells, -1);
  t->ntok.assign(cells, 0);
  t->dst_pos0.assign(cells, 0);
  t->shift.assign(cells, 0);

  std::vector<BlockKey> keys;
  keys.reserve((size_t)total);
  std::vector<uint8_t> is_shared_seg(cells, 0);
  FingerprintTable ft((size_t)total);
  for (int32_t j = 0; j < n; ++j) {
    const kvp_agent& a = agents[j];
    int32_t parent = kAgentRoot;
    int64_t pos = 0;
    int32_t b = 0;
    for (int32_t s = 0; s < a.n_spans; ++s) {
      const kvp_span& sp = a.spans[s];
      if (sp.kind == KVP_SEGMENT) parent = kSegRoot;
      BlockKey k{};
      k.tier = sp.tier;
      k.group = sp.tier == KVP_GROUP ? sp.group : 0;
      k.priv_agent = sp.tier == KVP_PRIVATE ? j : -1;
      k.priv_span = sp.tier == KVP_PRIVATE ? s : -1;
      for (int32_t t0 = 0; t0 < sp.n_tokens; t0 += B, ++b) {
        k.parent = parent;
        k.ntok = std::min(B, sp.n_tokens - t0);
        k.tokens = sp.tokens + t0;
        int32_t id = ft.find_or_insert(k, keys, (int32_t)keys.size());
        if (id == (int32_t)keys.size()) {
          keys.push_back(k);
          t->src_pos0.push_back((int32_t)(pos + t0));
          t->phys_ntok.push_back(k.ntok);
          t->phys_agent.push_back(j);
          t->phys_block.push_back(b);
        }
        size_t e = (size_t)j * M + b;
        t->block_table[e] = id;
        t->ntok[e] = k.ntok;
        t->dst_pos0[e] = (int32_t)(pos + t0);
        t->shift[e] = (int32_t)(pos + t0) - t->src_pos0[(size_t)id];
        is_shared_seg[e] = (sp.kind == KVP_SEGMENT && sp.tier != KVP_PRIVATE) ? 1 : 0;
        parent = id;
      }
      pos += sp.n_tokens;
      if (pos > INT32_MAX) return fail(KVP_EINVAL, "sequence longer than 2^31 tokens");
    }
  }
  t->n_dedup = (int32_t)keys.size();

  // deltas (validated before any is numbered)
  for (int32_t j = 0; j < n; ++j) {
    const kvp_agent& a = agents[j];
    for (int32_t i = 0; i < a.n_delta; ++i) {
      int32_t b = a.delta_blocks[i];
      if (b < 0 || b >= m[(size_t)j] || (i && a.delta_blocks[i - 1] >= b))
        return fail(KVP_EINVAL, "delta index out of range or not increasing");
      if (!is_shared_seg[(size_t)j * M + b]) return fail(KVP_EINVAL, "delta on a block that is not a shared segment block");
    }
  }
  int32_t next = t->n_dedup;
  for (int32_t j = 0; j < n; ++j) {
    const kvp_agent& a = agents[j];
    for (int32_t i = 0; i < a.n_delta; ++i) {
      int32_t b = a.delta_blocks[i];
      size_t e = (size_t)j * M + b;
      int32_t master = t->block_table[e];
      t->delta_table[e] = next++;
      t->src_pos0.push_back(t->src_pos0[(size_t)master]);
      t->phys_ntok.push_back(t->ntok[e]);
      t->phys_agent.push_back(j);
      t->phys_block.push_back(b);
    }
  }
  t->n_phys = next;
  t->n_delta = next - t->n_dedup;
  t->refcount.assign((size_t)next, 0);
  for (int32_t j = 0; j < n; ++j)
    for (int32_t b = 0; b < m[(size_t)j]; ++b) {
      size_t e = (size_t)j * M + b;
      int32_t id = t->delta_table[e] >= 0 ? t->delta_table[e] : t->block_table[e];
      t->refcount[(size_t)id] += 1;
    }
  build_plan(sh, t);
  return check_plan_bounds(sh, t);
}

extern "C" {

int kvpool_build_tables(const kvp_shape* shape, const kvp_agent* agents, int32_t n_agents, kvp_tables** out) {
  g_last_error[0] = '\0';
  int rc = validate_shape(shape);
  if (rc) return rc;
  if (!out || n_agents < 0 || (n_agents > 0 && !agents)) return fail(KVP_EINVAL, "agents or out is NULL");
  kvp_tables* t = new (std::nothrow) kvp_tables();
  if (!t) return fail(KVP_ENOMEM, "out of host memory");
  try {
    rc = build(shape, agents, n_agents, t);
  } catch (const std::bad_alloc&) {
    rc = fail(KVP_ENOMEM, "out of host memory");
  } catch (...) {
    rc = fail(KVP_EINVAL, "unexpected failure");
  }
  if (rc) {
    delete t;
    return rc;
  }
  *out = t;
  return KVP_OK;
}

int kvpool_tables_view(const kvp_tables* t, kvp_tables_view* v) {
  if (!t || !v) return fail(KVP_EINVAL, "tables or view is NULL");
  v->n_agents = t->n_agents;
  v->max_blocks = t->max_blocks;
  v->n_phys = t->n_phys;
  v->n_dedup = t->n_dedup;
  v->n_delta = t->n_delta;
  v->n_blocks = t->n_blocks.data();
  v->block_table = t->block_table.data();
  v->delta_table = t->delta_table.data();
  v->ntok = t->ntok.data();
  v->dst_pos0 = t->dst_pos0.data();
  v->shift = t->shift.data();
  v->src_pos0 = t->src_pos0.data();
  v->refcount = t->refcount.data();
  v->phys_ntok = t->phys_ntok.data();
  v->phys_agent = t->phys_agent.data();
  v->phys_block = t->phys_block.data();
  v->n_items = (int32_t)t->items.size();
  v->n_plan_blocks = (int32_t)t->plan_blocks.size();
  v->n_cons = (int32_t)t->cons.size();
  v->n_qcons = (int32_t)(t->qcons.size() / 2);
  v->n_mask_words = (int32_t)t->mask.size();
  v->n_part_rows = t->n_part_rows;
  v->n_comb = (int32_t)t->comb_rows.size();
  v->items = t->items.data();
  v->plan_blocks = t->plan_blocks.data();
  v->cons = t->cons.data();
  v->qcons = t->qcons.data();
  v->mask = t->mask.data();
  v->comb_ptr = t->comb_ptr.data();
  v->comb_rows = t->comb_rows.data();
  for (int i = 0; i < kRowClasses; ++i) v->class_items[i] = t->class_items[i];
  v->n_qcons_shifted = t->n_qcons_shifted;
  v->unit_span = t->unit_span;
  v->unique_kv_bytes = t->unique_kv_bytes;
  v->plan_ntok = t->plan_ntok.data();
  v->cons_row = t->cons_row.data();
  v->rope_cs = t->rope_cs.data();
  v->n_rope_cs = (int32_t)t->rope_cs.size();
  return KVP_OK;
}

void kvpool_tables_free(kvp_tables* t) { delete t; }

int kvpool_restore_list(const kvp_tables* t, const int32_t* agents, int32_t n_agents, int32_t* out,
                        int32_t max_entries) {
  if (!t || n_agents < 0 || (n_agents > 0 && !agents) || max_entries < 0 || (max_entries > 0 && !out))
    return fail(KVP_EINVAL, "tables NULL, bad agent list, or bad output buffer");
  int64_t total = 0;
  for (int32_t a = 0; a < n_agents; ++a) {
    if (agents[a] < 0 || agents[a] >= t->n_agents) return fail(KVP_EINVAL, "agent out of range");
    total += t->n_blocks[(size_t)agents[a]];
  }
  if (total > INT32_MAX) return fail(KVP_EINVAL, "too many entries");
  if (total > max_entries) return (int)total;
  // entries in destination order, then grouped by (source, valid tokens, shift)
  // so that a run of destinations reads its source once
  std::vector<int32_t> e, order;
  try {
    e.resize((size_t)total * 4);
    order.resize((size_t)total);
  } catch (const std::bad_alloc&) {
    return fail(KVP_ENOMEM, "restore list");
  }
  int64_t i = 0;
  for (int32_t a = 0; a < n_agents; ++a) {
    const int32_t j = agents[a];
    for (int32_t b = 0; b < t->n_blocks[(size_t)j]; ++b, ++i) {
      const size_t x = (size_t)j * t->max_blocks + b;
      e[4 * i] = t->delta_table[x] >= 0 ? t->delta_table[x] : t->block_table[x];
      e[4 * i + 1] = t->shift[x];
      e[4 * i + 2] = t->ntok[x];
      e[4 * i + 3] = (int32_t)i;
    }
  }
  for (int64_t k = 0; k < total; ++k) order[(size_t)k] = (int32_t)k;
  std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
    for (int f = 0; f < 3; ++f)
      if (e[4 * (size_t)x + f] != e[4 * (size_t)y + f]) return e[4 * (size_t)x + f] < e[4 * (size_t)y + f];
    return false;
  });
  for (int64_t k = 0; k < total; ++k)
    for (int f = 0; f < 4; ++f) out[4 * k + f] = e[4 * (size_t)order[(size_t)k] + f];
  return (int)total;
}

const char* kvpool_last_error(void) { return g_last_error; }

uint64_t kvpool_fnv1a64_words(const uint32_t* w, int64_t n) {
  uint64_t h = kFnvBasis;
  for (int64_t i = 0; i < n; ++i) h = fnv_word(h, w[i]);
  return h;
}

int kvpool_debug_set_hash_bits(int32_t bits) {
  if (bits < 1 || bits > 64) return fail(KVP_EINVAL, "hash bits must be 1..64");
  g_hash_bits = bits;
  return KVP_OK;
}

}  // extern "C"
