// Host block manager with prefix caching (MinivLLM guide "vLLM 技术路线",
// Step 3 §3.2 Block: a reference count, and a content hash of a full block
// chained with its predecessor's hash so equal tokens in different contexts
// stay distinct; a cached block is reused only when the hash is found AND the
// block holds exactly the same tokens, which guards against collisions;
// §3.3 BlockManager: can_allocate / allocate_with_cache / can_append / append /
// deallocate; Step 4 §4.5: prepare_prefill writes only the uncached tokens,
// prepare_decode's new slot is block_table[-1] * block_size +
// last_block_num_tokens - 1, and the token after a full block opens a new one).
//
// Readings where the pages leave a step open are stated with each operation
// in include/pagedattn.h.  Host code only: nothing here touches the GPU.
#include <stdint.h>
#include <string.h>

#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pagedattn.h"

namespace {

constexpr uint64_t kFnvOffset = 0xCBF29CE484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001B3ull;

inline uint64_t fnv_bytes(uint64_t h, const unsigned char* p, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= kFnvPrime;
  }
  return h;
}

// FNV-1a 64 over [prefix hash, 8 bytes LE, if any] + [token ids, 4 bytes LE each].
uint64_t chained_hash(const int32_t* toks, int n, bool has_prefix, uint64_t prefix, int bits) {
  uint64_t h = kFnvOffset;
  if (has_prefix) {
    unsigned char b[8];
    for (int i = 0; i < 8; ++i) b[i] = (unsigned char)(prefix >> (8 * i));
    h = fnv_bytes(h, b, 8);
  }
  for (int t = 0; t < n; ++t) {
    const uint32_t u = (uint32_t)toks[t];
    unsigned char b[4] = {(unsigned char)u, (unsigned char)(u >> 8), (unsigned char)(u >> 16),
                          (unsigned char)(u >> 24)};
    h = fnv_bytes(h, b, 4);
  }
  return bits >= 64 ? h : (h & ((1ull << bits) - 1));
}

struct Block {
  int ref = 0;
  bool has_hash = false;
  uint64_t hash = 0;
  std::vector<int32_t> tokens;  // contents of a full, hashed block
  // free list links (FIFO, O(1) removal of any member)
  int prev = -1, next = -1;
  bool free = true;
};

struct Seq {
  std::vector<int32_t> tokens;
  std::vector<int32_t> table;
  int cached = 0;
};

}  // namespace

struct pa_block_manager {
  int block_size = 0;
  int hash_bits = 64;
  std::vector<Block> blocks;
  int head = -1, tail = -1, num_free = 0;
  std::unordered_map<uint64_t, int> hash_to_block;
  std::unordered_map<int64_t, Seq> seqs;

  void push_free(int b) {
    Block& k = blocks[b];
    k.free = true;
    k.prev = tail;
    k.next = -1;
    if (tail >= 0) blocks[tail].next = b;
    else head = b;
    tail = b;
    ++num_free;
  }
  void unlink_free(int b) {
    Block& k = blocks[b];
    if (k.prev >= 0) blocks[k.prev].next = k.next;
    else head = k.next;
    if (k.next >= 0) blocks[k.next].prev = k.prev;
    else tail = k.prev;
    k.prev = k.next = -1;
    k.free = false;
    --num_free;
  }
  // Hand out the head of the free list for new contents (its old hash entry is dropped).
  int take() {
    const int b = head;
    unlink_free(b);
    Block& k = blocks[b];
    if (k.has_hash) {
      auto it = hash_to_block.find(k.hash);
      if (it != hash_to_block.end() && it->second == b) hash_to_block.erase(it);
    }
    k.ref = 1;
    k.has_hash = false;
    k.hash = 0;
    k.tokens.clear();
    return b;
  }
  void enroll(int b, uint64_t h, const int32_t* toks) {
    Block& k = blocks[b];
    k.has_hash = true;
    k.hash = h;
    k.tokens.assign(toks, toks + block_size);
    hash_to_block[h] = b;
  }
  int blocks_for(int64_t n) const { return (int)((n + block_size - 1) / block_size); }
};

extern "C" {

int pa_bm_create(int num_blocks, int block_size, int hash_bits, pa_block_manager** out) {
  if (!out) return PA_ERR_NULL;
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0 || hash_bits < 1 || hash_bits > 64) return PA_ERR_SHAPE;
  if ((int64_t)num_blocks * block_size > INT32_MAX) return PA_ERR_SHAPE;
  pa_block_manager* m = new (std::nothrow) pa_block_manager();
  if (!m) return PA_ERR_OUT_OF_BLOCKS;
  m->block_size = block_size;
  m->hash_bits = hash_bits;
  try {
    m->blocks.resize(num_blocks);
  } catch (...) {  // host memory exhausted
    delete m;
    return PA_ERR_OUT_OF_BLOCKS;
  }
  for (int b = 0; b < num_blocks; ++b) m->push_free(b);
  *out = m;
  return PA_OK;
}

int pa_bm_destroy(pa_block_manager* m) {
  delete m;
  return PA_OK;
}

int pa_bm_num_free(const pa_block_manager* m) { return m ? m->num_free : PA_ERR_NULL; }

int pa_bm_can_allocate(const pa_block_manager* m, int num_tokens) {
  if (!m) return PA_ERR_NULL;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  return m->num_free >= m->blocks_for(num_tokens) ? 1 : 0;
}

int pa_bm_allocate(pa_block_manager* m, int64_t seq_id, const int32_t* tokens, int num_tokens,
                   int* num_cached_tokens) {
  if (!m) return PA_ERR_NULL;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (num_tokens > 0 && !tokens) return PA_ERR_NULL;
  if (m->seqs.count(seq_id)) return PA_ERR_SEQUENCE;
  if (m->num_free < m->blocks_for(num_tokens)) return PA_ERR_OUT_OF_BLOCKS;
  Seq s;
  s.tokens.assign(tokens, tokens + num_tokens);
  const int bs = m->block_size;
  const int nb = m->blocks_for(num_tokens);
  bool has_prefix = false, miss = false;
  uint64_t prefix = 0;
  for (int i = 0; i < nb; ++i) {
    const int32_t* tk = s.tokens.data() + (size_t)i * bs;
    const bool full = (int64_t)(i + 1) * bs <= num_tokens;
    uint64_t h = 0;
    int bid = -1;
    if (full) {
      h = chained_hash(tk, bs, has_prefix, prefix, m->hash_bits);
      auto it = m->hash_to_block.find(h);
      if (it != m->hash_to_block.end()) bid = it->second;
    }
    if (bid < 0 || (int)m->blocks[bid].tokens.size() != bs ||
        memcmp(m->blocks[bid].tokens.data(), tk, sizeof(int32_t) * bs) != 0)
      miss = true;
    int b;
    if (miss) {
      b = m->take();
      if (full) m->enroll(b, h, tk);
    } else {
      b = bid;
      s.cached += bs;
      Block& k = m->blocks[b];
      if (k.free) {
        m->unlink_free(b);
        k.ref = 1;
      } else {
        ++k.ref;
      }
    }
    s.table.push_back(b);
    has_prefix = full;
    prefix = h;
  }
  if (num_cached_tokens) *num_cached_tokens = s.cached;
  m->seqs.emplace(seq_id, std::move(s));
  return PA_OK;
}

int pa_bm_can_append(const pa_block_manager* m, int64_t seq_id) {
  if (!m) return PA_ERR_NULL;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PA_ERR_SEQUENCE;
  const int need = it->second.tokens.size() % (size_t)m->block_size == 0 ? 1 : 0;
  return m->num_free >= need ? 1 : 0;
}

int pa_bm_append(pa_block_manager* m, int64_t seq_id, int32_t token) {
  if (!m) return PA_ERR_NULL;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PA_ERR_SEQUENCE;
  Seq& s = it->second;
  const int bs = m->block_size;
  if (s.tokens.size() % (size_t)bs == 0 && m->num_free == 0) return PA_ERR_OUT_OF_BLOCKS;
  if (s.tokens.size() >= (size_t)INT32_MAX) return PA_ERR_SHAPE;
  s.tokens.push_back(token);
  const size_t n = s.tokens.size();
  if ((n - 1) % bs == 0) s.table.push_back(m->take());  // the token opens a block
  if (n % bs == 0) {                                     // the token fills the last block
    const int last = s.table.back();
    const bool has_prefix = s.table.size() > 1;
    const Block& pb = m->blocks[has_prefix ? s.table[s.table.size() - 2] : last];
    // a full predecessor always carries its hash
    const uint64_t h = chained_hash(s.tokens.data() + n - bs, bs, has_prefix,
                                    has_prefix ? pb.hash : 0, m->hash_bits);
    m->enroll(last, h, s.tokens.data() + n - bs);
  }
  return PA_OK;
}

int pa_bm_deallocate(pa_block_manager* m, int64_t seq_id) {
  if (!m) return PA_ERR_NULL;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PA_ERR_SEQUENCE;
  const std::vector<int32_t>& t = it->second.table;
  for (size_t i = t.size(); i-- > 0;) {
    Block& k = m->blocks[t[i]];
    if (--k.ref == 0) m->push_free(t[i]);
  }
  m->seqs.erase(it);
  return PA_OK;
}

int pa_bm_seq_info(const pa_block_manager* m, int64_t seq_id, int* num_tokens,
                   int* num_cached_tokens, int* num_blocks) {
  if (!m) return PA_ERR_NULL;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PA_ERR_SEQUENCE;
  if (num_tokens) *num_tokens = (int)it->second.tokens.size();
  if (num_cached_tokens) *num_cached_tokens = it->second.cached;
  if (num_blocks) *num_blocks = (int)it->second.table.size();
  return PA_OK;
}

int pa_bm_block_table(const pa_block_manager* m, int64_t seq_id, int32_t* out, int capacity) {
  if (!m) return PA_ERR_NULL;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PA_ERR_SEQUENCE;
  const std::vector<int32_t>& t = it->second.table;
  if (capacity > 0 && !out) return PA_ERR_NULL;
  for (int i = 0; i < capacity && i < (int)t.size(); ++i) out[i] = t[i];
  return (int)t.size();
}

int pa_bm_free_list(const pa_block_manager* m, int32_t* out, int capacity) {
  if (!m) return PA_ERR_NULL;
  if (capacity > 0 && !out) return PA_ERR_NULL;
  int i = 0;
  for (int b = m->head; b >= 0; b = m->blocks[b].next, ++i)
    if (i < capacity) out[i] = b;
  return i;
}

int pa_bm_ref_count(const pa_block_manager* m, int block_id) {
  if (!m) return PA_ERR_NULL;
  if (block_id < 0 || block_id >= (int)m->blocks.size()) return PA_ERR_SHAPE;
  return m->blocks[block_id].ref;
}

int pa_bm_prepare_decode(const pa_block_manager* m, const int64_t* seq_ids, int num_seqs,
                         int max_blocks_per_seq, int32_t* slot_mapping, int32_t* context_lens,
                         int32_t* block_tables) {
  if (!m) return PA_ERR_NULL;
  if (num_seqs < 0 || max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!seq_ids || !slot_mapping || !context_lens || !block_tables) return PA_ERR_NULL;
  const int bs = m->block_size;
  for (int i = 0; i < num_seqs; ++i) {
    auto it = m->seqs.find(seq_ids[i]);
    if (it == m->seqs.end()) return PA_ERR_SEQUENCE;
    const Seq& s = it->second;
    if ((int)s.table.size() > max_blocks_per_seq) return PA_ERR_SHAPE;
    const int n = (int)s.tokens.size();
    context_lens[i] = n;
    // new slot = table[-1] * block_size + last_block_num_tokens - 1
    const int last_block_num_tokens = n - ((int)s.table.size() - 1) * bs;
    slot_mapping[i] = n > 0 ? s.table.back() * bs + last_block_num_tokens - 1 : -1;
    int32_t* row = block_tables + (size_t)i * max_blocks_per_seq;
    for (int j = 0; j < max_blocks_per_seq; ++j)
      row[j] = j < (int)s.table.size() ? s.table[j] : -1;
  }
  return PA_OK;
}

int pa_bm_prepare_prefill(const pa_block_manager* m, const int64_t* seq_ids, int num_seqs,
                          int max_blocks_per_seq, int32_t* cu_seqlens_q, int32_t* context_lens,
                          int32_t* block_tables, int32_t* slot_mapping, int slot_capacity,
                          int* total_q, int* max_q_len) {
  if (!m) return PA_ERR_NULL;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || slot_capacity < 0) return PA_ERR_SHAPE;
  if (!cu_seqlens_q) return PA_ERR_NULL;
  cu_seqlens_q[0] = 0;
  int64_t total = 0;
  int mx = 0;
  if (num_seqs > 0 && (!seq_ids || !context_lens || !block_tables)) return PA_ERR_NULL;
  const int bs = m->block_size;
  for (int i = 0; i < num_seqs; ++i) {
    auto it = m->seqs.find(seq_ids[i]);
    if (it == m->seqs.end()) return PA_ERR_SEQUENCE;
    const Seq& s = it->second;
    if ((int)s.table.size() > max_blocks_per_seq) return PA_ERR_SHAPE;
    const int n = (int)s.tokens.size();
    const int q = n - s.cached;
    if (total + q > slot_capacity) return PA_ERR_SHAPE;
    if (q > 0 && !slot_mapping) return PA_ERR_NULL;
    for (int p = s.cached; p < n; ++p) slot_mapping[total + p - s.cached] = s.table[p / bs] * bs + p % bs;
    total += q;
    mx = q > mx ? q : mx;
    cu_seqlens_q[i + 1] = (int32_t)total;
    context_lens[i] = n;
    int32_t* row = block_tables + (size_t)i * max_blocks_per_seq;
    for (int j = 0; j < max_blocks_per_seq; ++j)
      row[j] = j < (int)s.table.size() ? s.table[j] : -1;
  }
  if (total_q) *total_q = (int)total;
  if (max_q_len) *max_q_len = mx;
  return PA_OK;
}

}  // extern "C"
