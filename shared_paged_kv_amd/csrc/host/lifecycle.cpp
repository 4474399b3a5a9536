// Block lifecycle of the deduplicated pool (include/kvpool_lifecycle.h):
// decode-time append with copy-on-write, sequence destruction, and the leak
// audit with forced reclamation.
//
// INMS walkthrough, sec. 2.2: a write into a block whose reference count is
// above one first makes a private copy (the old count drops by one), else it
// writes in place; sec. 3.3: destroying a sequence releases its references and
// reclaims blocks at zero; sec. 5.3: an agent that dies without its destroy
// call leaks its references until a scan finds them and they are reclaimed.
#include <algorithm>
#include <cstdint>
#include <functional>
#include <new>
#include <unordered_map>
#include <vector>

#include "kvpool_internal.h"
#include "kvpool_lifecycle.h"

using namespace kvp;

namespace {

enum : uint8_t { kLive = 0, kDestroyed = 1, kLost = 2 };

struct Entry {
  int32_t table;      // block_table id (the master of an overlaid entry)
  uint32_t table_gen; // allocation generation of table when it was recorded
  int32_t delta;      // delta id or -1
  int32_t ntok;       // valid tokens
  int32_t dst_pos0;   // logical position of the first token
  int32_t eff() const { return delta >= 0 ? delta : table; }
};

}  // namespace

struct kvp_pool {
  kvp_shape shape{};
  int32_t capacity = 0, n_dedup = 0, n_delta = 0;
  std::vector<uint8_t> state;               // per agent
  std::vector<std::vector<Entry>> blocks;   // per agent
  // per physical id, [capacity]
  std::vector<int32_t> refcount, src_pos0, phys_ntok, phys_agent, phys_block;
  std::vector<uint8_t> allocated;
  std::vector<uint32_t> gen;
  // freed ids below next_id: a min-heap with room for capacity ids reserved at
  // creation, so that returning an id never allocates
  std::vector<int32_t> free_ids;
  int32_t next_id = 0;         // ids >= next_id were never allocated
  // the last append's operations
  std::vector<int32_t> copies, writes;
};

namespace {

int32_t alloc_id(kvp_pool* p) {
  int32_t id;
  if (!p->free_ids.empty()) {
    std::pop_heap(p->free_ids.begin(), p->free_ids.end(), std::greater<int32_t>());
    id = p->free_ids.back();
    p->free_ids.pop_back();
  } else if (p->next_id < p->capacity) {
    id = p->next_id++;
  } else {
    return -1;
  }
  p->allocated[(size_t)id] = 1;
  p->gen[(size_t)id] += 1;
  p->refcount[(size_t)id] = 0;
  p->phys_ntok[(size_t)id] = 0;
  p->phys_agent[(size_t)id] = -1;
  p->phys_block[(size_t)id] = -1;
  return id;
}

void free_id(kvp_pool* p, int32_t id) {
  p->allocated[(size_t)id] = 0;
  p->refcount[(size_t)id] = 0;
  p->phys_ntok[(size_t)id] = 0;
  p->free_ids.push_back(id);
  std::push_heap(p->free_ids.begin(), p->free_ids.end(), std::greater<int32_t>());
}

bool live(const kvp_pool* p, int32_t j) {
  return j >= 0 && j < (int32_t)p->state.size() && p->state[(size_t)j] == kLive;
}

// live agents' effective references per physical id
std::vector<int32_t> recount(const kvp_pool* p) {
  std::vector<int32_t> rc((size_t)p->capacity, 0);
  for (size_t j = 0; j < p->blocks.size(); ++j) {
    if (p->state[j] != kLive) continue;
    for (const Entry& e : p->blocks[j]) rc[(size_t)e.eff()] += 1;
  }
  return rc;
}

// What an append changed, for an all-or-nothing call: per agent its block count
// and last entry before the call; per physical id its state before the call;
// the free ids taken and the high-water id.
struct Undo {
  struct Agent {
    size_t size;
    Entry last;
  };
  std::unordered_map<int32_t, Agent> agents;
  struct Phys {
    int32_t refcount, src_pos0, phys_ntok, phys_agent, phys_block;
    uint8_t allocated;
    uint32_t gen;
  };
  std::unordered_map<int32_t, Phys> phys;
  std::vector<int32_t> taken;  // ids taken from the free set
  int32_t next_id = 0;

  void save_agent(const kvp_pool* p, int32_t j) {
    if (agents.count(j)) return;
    const auto& bl = p->blocks[(size_t)j];
    agents.emplace(j, Agent{bl.size(), bl.empty() ? Entry{} : bl.back()});
  }
  void save_phys(const kvp_pool* p, int32_t id) {
    if (phys.count(id)) return;
    size_t i = (size_t)id;
    phys.emplace(id, Phys{p->refcount[i], p->src_pos0[i], p->phys_ntok[i], p->phys_agent[i], p->phys_block[i],
                          p->allocated[i], p->gen[i]});
  }
  void restore(kvp_pool* p) {
    for (auto& a : agents) {
      auto& bl = p->blocks[(size_t)a.first];
      bl.resize(a.second.size);
      if (!bl.empty()) bl.back() = a.second.last;
    }
    for (auto& kv : phys) {
      size_t i = (size_t)kv.first;
      const Phys& s = kv.second;
      p->refcount[i] = s.refcount;
      p->src_pos0[i] = s.src_pos0;
      p->phys_ntok[i] = s.phys_ntok;
      p->phys_agent[i] = s.phys_agent;
      p->phys_block[i] = s.phys_block;
      p->allocated[i] = s.allocated;
      p->gen[i] = s.gen;
    }
    for (int32_t id : taken) {
      p->free_ids.push_back(id);
      std::push_heap(p->free_ids.begin(), p->free_ids.end(), std::greater<int32_t>());
    }
    p->next_id = next_id;
  }
};

// Allocation that records the id's previous state first.
int32_t alloc_logged(kvp_pool* p, Undo& u) {
  const bool from_free = !p->free_ids.empty();
  int32_t id = from_free ? p->free_ids.front() : (p->next_id < p->capacity ? p->next_id : -1);
  if (id < 0) return -1;
  u.save_phys(p, id);
  if (from_free) u.taken.push_back(id);
  return alloc_id(p);
}

int append_one(kvp_pool* p, int32_t j, int32_t row, Undo& u) {
  const int32_t B = p->shape.block_tokens;
  u.save_agent(p, j);
  std::vector<Entry>& bl = p->blocks[(size_t)j];
  if (bl.empty() || bl.back().ntok >= B) {
    // a new logical block, in its own frame
    const int32_t pos = bl.empty() ? 0 : bl.back().dst_pos0 + bl.back().ntok;
    const int32_t q = alloc_logged(p, u);
    if (q < 0) return fail(KVP_EFULL, "the pool has no free physical block");
    p->refcount[(size_t)q] = 1;
    p->src_pos0[(size_t)q] = pos;
    p->phys_ntok[(size_t)q] = 1;
    bl.push_back(Entry{q, p->gen[(size_t)q], -1, 1, pos});
    p->writes.insert(p->writes.end(), {q, 0, row, 0});
    return KVP_OK;
  }
  Entry& e = bl.back();
  int32_t eff = e.eff();
  if (p->refcount[(size_t)eff] > 1) {
    // copy-on-write: a private copy in the same stored frame
    const int32_t q = alloc_logged(p, u);
    if (q < 0) return fail(KVP_EFULL, "the pool has no free physical block");
    u.save_phys(p, eff);
    p->refcount[(size_t)eff] -= 1;
    p->refcount[(size_t)q] = 1;
    p->src_pos0[(size_t)q] = p->src_pos0[(size_t)eff];
    p->phys_ntok[(size_t)q] = p->phys_ntok[(size_t)eff];
    p->copies.insert(p->copies.end(), {eff, q});
    e.table = q;
    e.table_gen = p->gen[(size_t)q];
    e.delta = -1;
    eff = q;
  }
  u.save_phys(p, eff);
  const int32_t slot = e.ntok;
  const int32_t shift = e.dst_pos0 - p->src_pos0[(size_t)eff];
  p->writes.insert(p->writes.end(), {eff, slot, row, shift});
  e.ntok += 1;
  p->phys_ntok[(size_t)eff] = e.ntok;
  return KVP_OK;
}

}  // namespace

extern "C" {

int kvpool_pool_create(const kvp_tables* t, const kvp_shape* shape, int32_t capacity, kvp_pool** out) {
  if (!t || !shape || !out) return fail(KVP_EINVAL, "tables, shape or out is NULL");
  int rc = check_shape(shape);
  if (rc) return rc;
  if (capacity < t->n_phys) return fail(KVP_EINVAL, "capacity below the tables' physical blocks");
  kvp_pool* p = new (std::nothrow) kvp_pool();
  if (!p) return fail(KVP_ENOMEM, "out of host memory");
  try {
    p->shape = *shape;
    p->capacity = capacity;
    p->n_dedup = t->n_dedup;
    p->n_delta = t->n_delta;
    const size_t C = (size_t)capacity;
    p->refcount.assign(C, 0);
    p->src_pos0.assign(C, 0);
    p->phys_ntok.assign(C, 0);
    p->phys_agent.assign(C, -1);
    p->phys_block.assign(C, -1);
    p->allocated.assign(C, 0);
    p->gen.assign(C, 0);
    p->free_ids.reserve(C);
    for (int32_t i = 0; i < t->n_phys; ++i) {
      size_t k = (size_t)i;
      p->refcount[k] = t->refcount[k];
      p->src_pos0[k] = t->src_pos0[k];
      p->phys_ntok[k] = t->phys_ntok[k];
      p->phys_agent[k] = t->phys_agent[k];
      p->phys_block[k] = t->phys_block[k];
      p->gen[k] = 1;
      // a block that no entry reads (a master overlaid everywhere) is free
      if (t->refcount[k] > 0) p->allocated[k] = 1;
      else free_id(p, i);
    }
    p->next_id = t->n_phys;
    p->state.assign((size_t)t->n_agents, kLive);
    p->blocks.resize((size_t)t->n_agents);
    for (int32_t j = 0; j < t->n_agents; ++j) {
      auto& bl = p->blocks[(size_t)j];
      bl.reserve((size_t)t->n_blocks[(size_t)j]);
      for (int32_t b = 0; b < t->n_blocks[(size_t)j]; ++b) {
        size_t e = (size_t)j * t->max_blocks + b;
        bl.push_back(Entry{t->block_table[e], 1u, t->delta_table[e], t->ntok[e], t->dst_pos0[e]});
      }
    }
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(KVP_ENOMEM, "out of host memory");
  }
  *out = p;
  return KVP_OK;
}

void kvpool_pool_free(kvp_pool* pool) { delete pool; }

int kvpool_append(kvp_pool* pool, int32_t n, const int32_t* agents, kvp_append_ops* ops) {
  if (!pool || !ops || n < 0 || (n > 0 && !agents)) return fail(KVP_EINVAL, "pool, ops or agents is NULL, or n < 0");
  for (int32_t i = 0; i < n; ++i)
    if (!live(pool, agents[i])) return fail(KVP_EINVAL, "agent out of range or not live");
  // every change is recorded before it is made, and undoing allocates nothing,
  // so a failure part-way (no free block, or no host memory) leaves the pool as
  // it was
  Undo u;
  u.next_id = pool->next_id;
  auto undo = [&](int rc) {
    u.restore(pool);
    pool->copies.clear();
    pool->writes.clear();
    ops->n_copies = ops->n_writes = 0;
    ops->copies = ops->writes = nullptr;
    return rc;
  };
  try {
    pool->copies.clear();
    pool->writes.clear();
    for (int32_t i = 0; i < n; ++i) {
      int rc = append_one(pool, agents[i], i, u);
      if (rc) return undo(rc);
    }
  } catch (const std::bad_alloc&) {
    return undo(fail(KVP_ENOMEM, "out of host memory"));
  }
  ops->n_copies = (int32_t)(pool->copies.size() / 2);
  ops->copies = pool->copies.data();
  ops->n_writes = (int32_t)(pool->writes.size() / 4);
  ops->writes = pool->writes.data();
  return KVP_OK;
}

int kvpool_destroy(kvp_pool* pool, int32_t agent) {
  if (!pool || !live(pool, agent)) return fail(KVP_EINVAL, "agent out of range or not live");
  for (const Entry& e : pool->blocks[(size_t)agent]) {
    const int32_t id = e.eff();
    if (--pool->refcount[(size_t)id] == 0) free_id(pool, id);
  }
  pool->blocks[(size_t)agent].clear();
  pool->state[(size_t)agent] = kDestroyed;
  return KVP_OK;
}

int kvpool_lose(kvp_pool* pool, int32_t agent) {
  if (!pool || !live(pool, agent)) return fail(KVP_EINVAL, "agent out of range or not live");
  pool->blocks[(size_t)agent].clear();
  pool->state[(size_t)agent] = kLost;
  return KVP_OK;
}

int kvpool_audit(const kvp_pool* pool, kvp_audit* audit, int32_t* ids, int32_t max_ids) {
  if (!pool || !audit || max_ids < 0) return fail(KVP_EINVAL, "pool or audit is NULL, or max_ids < 0");
  std::vector<int32_t> rc = recount(pool);
  kvp_audit a{};
  int32_t written = 0;
  for (int32_t i = 0; i < pool->next_id; ++i) {
    size_t k = (size_t)i;
    if (!pool->allocated[k]) continue;
    a.n_allocated += 1;
    if (pool->refcount[k] != rc[k]) a.n_mismatched += 1;
    if (pool->refcount[k] > 0 && rc[k] == 0) {
      a.n_leaked += 1;
      a.leaked_tokens += pool->phys_ntok[k];
      if (ids && written < max_ids) ids[written++] = i;
    }
  }
  for (uint8_t s : pool->state) a.n_live_agents += s == kLive;
  *audit = a;
  return KVP_OK;
}

int kvpool_reclaim(kvp_pool* pool) {
  if (!pool) return fail(KVP_EINVAL, "pool is NULL");
  std::vector<int32_t> rc = recount(pool);
  int32_t freed = 0;
  for (int32_t i = 0; i < pool->next_id; ++i) {
    size_t k = (size_t)i;
    if (!pool->allocated[k]) continue;
    pool->refcount[k] = rc[k];
    if (rc[k] == 0) {
      free_id(pool, i);
      ++freed;
    }
  }
  return freed;
}

int kvpool_pool_tables(const kvp_pool* pool, kvp_tables** out) {
  if (!pool || !out) return fail(KVP_EINVAL, "pool or out is NULL");
  kvp_tables* t = new (std::nothrow) kvp_tables();
  if (!t) return fail(KVP_ENOMEM, "out of host memory");
  try {
    const int32_t n = (int32_t)pool->blocks.size();
    int32_t M = 0;
    for (auto& bl : pool->blocks) M = std::max(M, (int32_t)bl.size());
    t->n_agents = n;
    t->max_blocks = M;
    t->n_dedup = pool->n_dedup;
    t->n_delta = pool->n_delta;
    t->n_blocks.resize((size_t)n);
    const size_t cells = (size_t)n * (size_t)M;
    t->block_table.assign(cells, -1);
    t->delta_table.assign(cells, -1);
    t->ntok.assign(cells, 0);
    t->dst_pos0.assign(cells, 0);
    t->shift.assign(cells, 0);
    for (int32_t j = 0; j < n; ++j) {
      const auto& bl = pool->blocks[(size_t)j];
      t->n_blocks[(size_t)j] = (int32_t)bl.size();
      for (size_t b = 0; b < bl.size(); ++b) {
        const Entry& e = bl[b];
        const size_t c = (size_t)j * M + b;
        const int32_t eff = e.eff();
        // an overlaid entry names its master only while that block is the same
        // allocation; otherwise the entry is the delta block alone
        const bool master_alive = e.delta >= 0 && pool->allocated[(size_t)e.table] &&
                                  pool->gen[(size_t)e.table] == e.table_gen;
        t->block_table[c] = e.delta >= 0 && !master_alive ? e.delta : e.table;
        t->delta_table[c] = master_alive ? e.delta : -1;
        t->ntok[c] = e.ntok;
        t->dst_pos0[c] = e.dst_pos0;
        t->shift[c] = e.dst_pos0 - pool->src_pos0[(size_t)eff];
      }
    }
    // the snapshot describes the whole pool: capacity physical ids, so that the
    // decode's per-layer stride is the pool's
    t->n_phys = pool->capacity;
    t->src_pos0 = pool->src_pos0;
    t->refcount = pool->refcount;
    t->phys_ntok = pool->phys_ntok;
    t->phys_agent = pool->phys_agent;
    t->phys_block = pool->phys_block;
    build_plan(&pool->shape, t);
  } catch (const std::bad_alloc&) {
    delete t;
    return fail(KVP_ENOMEM, "out of host memory");
  }
  const int rc = check_plan_bounds(&pool->shape, t);
  if (rc) {
    delete t;
    return rc;
  }
  *out = t;
  return KVP_OK;
}

}  // extern "C"
