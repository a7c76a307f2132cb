// Host-side block manager: owns the physical block pool of a paged KV cache and produces
// the block tables and slots the decode and append kernels consume. Host code only.
//
// Pages cited by title and section:
//   [P1] "突破GPU内存瓶颈：vLLM与PagedAttention技术深度解析" §2 — fixed-size blocks, block
//        table per sequence, blocks shared between sequences; §5 — beam search shares
//        blocks between candidates.
//   [P3] "内存优化：KV Cache管理、PagedAttention原理与内存池配置" — blocks are allocated on
//        demand and appended as a request grows, returned to the global pool when it ends;
//        sharing by reference counting; free blocks kept in a list so that allocation and
//        release are O(1); prefix caching keeps a global hash index over prefix blocks and
//        reuses a block only when the prefix is exactly identical.
//   [P2] vLLM architecture deep-dive §2.3 — when no block is free, the block whose K-th
//        most recent access lies furthest back is evicted (LRU-K; LRU-2 named).
//
// Policies (where the pages leave a choice open):
//   * Free blocks form a stack: allocation pops the most recently freed block (initially
//     block 0, 1, 2, ...).
//   * With prefix caching, a block is indexed once it is full, under a key made of its
//     parent block (the previous block of the sequence, -1 for the first) and its token
//     ids; a lookup hits only if both are equal, so equal keys mean equal prefixes.
//     An indexed block whose reference count drops to zero stays indexed and becomes
//     evictable; it is reused on a hit, or evicted (and unindexed) when the free stack is
//     empty.
//   * Eviction is LRU-K over a logical clock that advances once per add, append or fork:
//     a block is accessed when a sequence gains a reference to it or writes a token into
//     it (several accesses within one operation count once). The victim is the evictable
//     block whose K-th most recent access is oldest, a block with fewer than K accesses
//     counting as infinitely old; ties go to the older most recent access, then to the
//     block deeper in its prefix chain (so a chain is evicted from its end), then to the
//     lower id. There is no swap space, so nothing is written back.
//   * Appending to a sequence whose last block is partly filled and shared (reference
//     count > 1) first gives the sequence a private copy (copy-on-write): the manager
//     allocates the new block and reports (source, destination) so that the caller copies
//     the block's K/V on the device.
#include <array>
#include <cstdint>
#include <cstring>
#include <new>
#include <set>
#include <tuple>
#include <unordered_map>
#include <vector>

#include "pa.h"

namespace pa {
namespace {

struct Seq {
  bool live = false;
  std::vector<int32_t> blocks;
  std::vector<int32_t> tokens;  // token ids, for prefix keys of blocks as they fill
};

// key of a full block: its parent block (id and the generation the parent had when this
// block was indexed, so that a parent reused for other data never matches old children)
// and the block's token ids
struct BlockKey {
  int32_t parent = -1;
  uint32_t parent_gen = 0;
  std::vector<int32_t> tokens;
  bool operator==(const BlockKey& o) const {
    return parent == o.parent && parent_gen == o.parent_gen && tokens == o.tokens;
  }
};
struct BlockKeyHash {
  size_t operator()(const BlockKey& k) const {
    // 64-bit FNV-1a over the parent id and the token ids
    uint64_t h = 1469598103934665603ull;
    auto mix = [&](uint32_t v) {
      for (int i = 0; i < 4; ++i) {
        h ^= (v >> (8 * i)) & 0xffu;
        h *= 1099511628211ull;
      }
    };
    mix((uint32_t)k.parent);
    mix(k.parent_gen);
    for (int32_t t : k.tokens) mix((uint32_t)t);
    return (size_t)h;
  }
};

constexpr int kMaxLruK = 4;

// eviction order: (K-th most recent access, most recent access, -chain depth, id), smallest
// first; -1 stands for "never"
using EvictKey = std::tuple<int64_t, int64_t, int32_t, int32_t>;

struct Manager {
  int num_blocks;
  int block_size;
  bool prefix_caching;
  int lru_k;
  int64_t clock = 0;
  std::vector<int32_t> ref;          // reference count per block
  std::vector<int32_t> free_stack;   // top = back
  std::vector<char> in_free;
  std::set<EvictKey> evictable;      // indexed blocks with no reference
  std::vector<EvictKey> evict_key;   // valid while in_evict
  std::vector<char> in_evict;
  std::vector<char> indexed;
  std::vector<BlockKey> key_of;      // valid when indexed
  std::vector<int32_t> depth;        // position in its prefix chain, valid when indexed
  std::vector<uint32_t> gen;         // bumped every time a block is taken for new data
  std::vector<std::array<int64_t, kMaxLruK>> hist;  // access times, most recent first
  std::unordered_map<BlockKey, int32_t, BlockKeyHash> index;
  std::vector<Seq> seqs;

  Manager(int nb, int bs, bool pc, int k)
      : num_blocks(nb), block_size(bs), prefix_caching(pc), lru_k(k), ref(nb, 0), in_free(nb, 1),
        evict_key(nb), in_evict(nb, 0), indexed(nb, 0), key_of(nb), depth(nb, 0), gen(nb, 0) {
    std::array<int64_t, kMaxLruK> never;
    never.fill(-1);
    hist.assign(nb, never);
    free_stack.reserve(nb);
    for (int b = nb - 1; b >= 0; --b) free_stack.push_back(b);
  }

  int available() const { return (int)free_stack.size() + (int)evictable.size(); }

  void access(int32_t b) {
    auto& h = hist[b];
    if (h[0] == clock) return;
    for (int i = kMaxLruK - 1; i > 0; --i) h[i] = h[i - 1];
    h[0] = clock;
  }

  // a block for new data: the free stack first, else the LRU-K victim among the evictable
  int32_t take() {
    int32_t b = -1;
    if (!free_stack.empty()) {
      b = free_stack.back();
      free_stack.pop_back();
      in_free[b] = 0;
    } else if (!evictable.empty()) {
      b = std::get<3>(*evictable.begin());
      evictable.erase(evictable.begin());
      in_evict[b] = 0;
      unindex(b);
    } else {
      return -1;
    }
    ref[b] = 1;
    ++gen[b];
    access(b);
    return b;
  }

  void unindex(int32_t b) {
    if (!indexed[b]) return;
    index.erase(key_of[b]);
    indexed[b] = 0;
    key_of[b] = BlockKey{};
  }

  void release(int32_t b) {
    if (--ref[b] > 0) return;
    if (prefix_caching && indexed[b]) {
      evict_key[b] = EvictKey{hist[b][lru_k - 1], hist[b][0], -depth[b], b};
      evictable.insert(evict_key[b]);
      in_evict[b] = 1;
    } else {
      unindex(b);
      free_stack.push_back(b);
      in_free[b] = 1;
    }
  }

  void acquire_cached(int32_t b) {
    if (in_evict[b]) {
      evictable.erase(evict_key[b]);
      in_evict[b] = 0;
    }
    ++ref[b];
    access(b);
  }

  // index block j of sequence s once it is full
  void index_full_block(Seq& sq, size_t j) {
    if (!prefix_caching) return;
    const int32_t b = sq.blocks[j];
    if (indexed[b]) return;
    BlockKey k;
    k.parent = j == 0 ? -1 : sq.blocks[j - 1];
    k.parent_gen = j == 0 ? 0 : gen[k.parent];
    k.tokens.assign(sq.tokens.begin() + (int64_t)j * block_size,
                    sq.tokens.begin() + (int64_t)(j + 1) * block_size);
    if (index.count(k)) return;  // an equal block is already indexed; keep this one private
    index.emplace(k, b);
    key_of[b] = std::move(k);
    indexed[b] = 1;
    depth[b] = (int32_t)j;
  }

  bool valid_seq(int s) const { return s >= 0 && s < (int)seqs.size() && seqs[s].live; }
};

}  // namespace
}  // namespace pa

struct pa_block_manager {
  pa::Manager m;
  pa_block_manager(int nb, int bs, bool pc, int k) : m(nb, bs, pc, k) {}
};

extern "C" {

pa_block_manager* pa_bm_create(int num_blocks, int block_size, int enable_prefix_caching, int lru_k) {
  if (lru_k == 0) lru_k = 2;
  if (num_blocks <= 0 || block_size <= 0 || lru_k < 1 || lru_k > pa::kMaxLruK) return nullptr;
  try {
    return new pa_block_manager(num_blocks, block_size, enable_prefix_caching != 0, lru_k);
  } catch (...) {
    return nullptr;
  }
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int pa_bm_num_free(const pa_block_manager* bm) {
  if (!bm) return PA_ERR_INVALID;
  return bm->m.available();
}

int pa_bm_add_sequence(pa_block_manager* bm, const int32_t* token_ids, int num_tokens,
                       int* num_cached_tokens) {
  if (!bm || num_tokens < 0 || (num_tokens > 0 && !token_ids)) return PA_ERR_INVALID;
  try {
    pa::Manager& m = bm->m;
    const int BS = m.block_size;
    const int nblk = (num_tokens + BS - 1) / BS;
    // prefix-cache hits over leading full blocks
    std::vector<int32_t> hit;
    if (m.prefix_caching) {
      int32_t parent = -1;
      for (int j = 0; j < num_tokens / BS; ++j) {
        pa::BlockKey k;
        k.parent = parent;
        k.parent_gen = parent < 0 ? 0 : m.gen[parent];
        k.tokens.assign(token_ids + (int64_t)j * BS, token_ids + (int64_t)(j + 1) * BS);
        auto it = m.index.find(k);
        if (it == m.index.end()) break;
        hit.push_back(it->second);
        parent = it->second;
      }
    }
    // evictable hits stop being available once acquired
    int evictable_hits = 0;
    for (int32_t b : hit) evictable_hits += m.in_evict[b] ? 1 : 0;
    if (m.available() - evictable_hits < nblk - (int)hit.size()) return PA_ERR_WORKSPACE;
    ++m.clock;
    pa::Seq sq;
    sq.live = true;
    sq.tokens.assign(token_ids, token_ids + num_tokens);
    for (int32_t b : hit) {
      m.acquire_cached(b);
      sq.blocks.push_back(b);
    }
    for (int j = (int)hit.size(); j < nblk; ++j) sq.blocks.push_back(m.take());
    for (int j = (int)hit.size(); j < num_tokens / BS; ++j) m.index_full_block(sq, (size_t)j);
    if (num_cached_tokens) *num_cached_tokens = (int)hit.size() * BS;
    m.seqs.push_back(std::move(sq));
    return (int)m.seqs.size() - 1;
  } catch (...) {
    return PA_ERR_LAUNCH;
  }
}

int pa_bm_append_token(pa_block_manager* bm, int seq, int32_t token_id, int32_t* slot,
                       int32_t* copy_src, int32_t* copy_dst) {
  if (!bm || !slot || !copy_src || !copy_dst) return PA_ERR_INVALID;
  try {
    pa::Manager& m = bm->m;
    if (!m.valid_seq(seq)) return PA_ERR_INVALID;
    pa::Seq& sq = m.seqs[seq];
    const int BS = m.block_size;
    const int64_t pos = (int64_t)sq.tokens.size();
    *copy_src = -1;
    *copy_dst = -1;
    // a new block when the last one is full (or there is none), a private copy when it is
    // partly filled and shared
    const bool fresh_block = pos % BS == 0;
    const bool cow = !fresh_block && m.ref[sq.blocks.back()] > 1;
    if ((fresh_block || cow) && m.available() < 1) return PA_ERR_WORKSPACE;
    ++m.clock;
    if (fresh_block) {
      sq.blocks.push_back(m.take());
    } else {
      const int32_t last = sq.blocks.back();
      if (cow) {
        const int32_t fresh = m.take();
        m.release(last);
        sq.blocks.back() = fresh;
        *copy_src = last;
        *copy_dst = fresh;
      }
    }
    sq.tokens.push_back(token_id);
    m.access(sq.blocks.back());
    *slot = sq.blocks.back() * BS + (int32_t)(pos % BS);
    if ((pos + 1) % BS == 0) m.index_full_block(sq, sq.blocks.size() - 1);
    return PA_OK;
  } catch (...) {
    return PA_ERR_LAUNCH;
  }
}

int pa_bm_fork(pa_block_manager* bm, int parent) {
  if (!bm) return PA_ERR_INVALID;
  try {
    pa::Manager& m = bm->m;
    if (!m.valid_seq(parent)) return PA_ERR_INVALID;
    pa::Seq child = m.seqs[parent];
    ++m.clock;
    for (int32_t b : child.blocks) {
      ++m.ref[b];
      m.access(b);
    }
    m.seqs.push_back(std::move(child));
    return (int)m.seqs.size() - 1;
  } catch (...) {
    return PA_ERR_LAUNCH;
  }
}

int pa_bm_free_sequence(pa_block_manager* bm, int seq) {
  if (!bm) return PA_ERR_INVALID;
  pa::Manager& m = bm->m;
  if (!m.valid_seq(seq)) return PA_ERR_INVALID;
  pa::Seq& sq = m.seqs[seq];
  // release in reverse so that a sequence's later blocks are evicted before its prefix
  for (auto it = sq.blocks.rbegin(); it != sq.blocks.rend(); ++it) m.release(*it);
  sq.blocks.clear();
  sq.tokens.clear();
  sq.live = false;
  return PA_OK;
}

int pa_bm_context_len(const pa_block_manager* bm, int seq) {
  if (!bm || !bm->m.valid_seq(seq)) return PA_ERR_INVALID;
  return (int)bm->m.seqs[seq].tokens.size();
}

int pa_bm_block_table(const pa_block_manager* bm, int seq, int32_t* out, int max_blocks) {
  if (!bm || !bm->m.valid_seq(seq) || max_blocks < 0 || (max_blocks > 0 && !out)) return PA_ERR_INVALID;
  const auto& blocks = bm->m.seqs[seq].blocks;
  if ((int)blocks.size() > max_blocks) return PA_ERR_WORKSPACE;
  for (int j = 0; j < max_blocks; ++j) out[j] = j < (int)blocks.size() ? blocks[j] : -1;
  return (int)blocks.size();
}

int pa_bm_ref_count(const pa_block_manager* bm, int block) {
  if (!bm || block < 0 || block >= bm->m.num_blocks) return PA_ERR_INVALID;
  return bm->m.ref[block];
}

int pa_bm_export(const pa_block_manager* bm, const int32_t* seqs, int n, int max_blocks,
                 int32_t* block_tables, int32_t* context_lens) {
  if (!bm || n < 0 || max_blocks <= 0 || (n > 0 && (!seqs || !block_tables || !context_lens)))
    return PA_ERR_INVALID;
  for (int i = 0; i < n; ++i)
    if (!bm->m.valid_seq(seqs[i]) || (int)bm->m.seqs[seqs[i]].blocks.size() > max_blocks)
      return PA_ERR_INVALID;
  for (int i = 0; i < n; ++i) {
    pa_bm_block_table(bm, seqs[i], block_tables + (int64_t)i * max_blocks, max_blocks);
    context_lens[i] = (int32_t)bm->m.seqs[seqs[i]].tokens.size();
  }
  return PA_OK;
}

}  // extern "C"
