// Host-side manager of the physical blocks behind the block cache layout (no device code).
//
// Book "DeepSeek V4 模型技术大全", chapter "Attention": the hybrid cache stores compressed entries
// in blocks aligned to lcm(m, 128) = 128 tokens, so one block id covers the same 128 tokens in a
// CSA entry pool (32 entries), its indexer-key pool and an HCA entry pool (one entry); a prefix
// of whole blocks can be shared by requests that start with the same tokens, and the tokens past
// the last whole block are recomputed.
//
// The manager keeps, for n_blocks ids: a reference count (sequences mapping the block); the free
// ids; and a registry of full blocks under a key that identifies the token prefix they end (a
// hash chain over the prefix's blocks of token ids).  A registered block whose count drops to
// zero is not forgotten at once: it waits in least-recently-released order and is handed out
// again by a lookup of its key, or recycled (and unregistered) only when no never-registered
// free block is left.
#include <cstdint>
#include <cstring>
#include <list>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/csa.h"

namespace csa {

int api_fail(int code, const char* fmt, ...);  // api.hip: records the thread's last error

}  // namespace csa

struct csa_block_manager {
  std::vector<int32_t> refs;
  std::vector<int32_t> free_ids;                      // never registered (or unregistered)
  std::list<int32_t> idle;                            // registered, count 0, oldest first
  std::vector<std::list<int32_t>::iterator> idle_at;  // position in `idle`
  std::vector<uint8_t> in_idle;
  std::vector<uint64_t> key_of;
  std::vector<uint8_t> has_key;
  std::unordered_map<uint64_t, int32_t> registry;
};

namespace {

using csa::api_fail;

bool bad_id(const csa_block_manager* m, int32_t b) {
  return b < 0 || b >= static_cast<int32_t>(m->refs.size());
}

void unregister(csa_block_manager* m, int32_t b) {
  if (!m->has_key[b]) return;
  auto it = m->registry.find(m->key_of[b]);
  if (it != m->registry.end() && it->second == b) m->registry.erase(it);
  m->has_key[b] = 0;
}

void take_from_idle(csa_block_manager* m, int32_t b) {
  m->idle.erase(m->idle_at[b]);
  m->in_idle[b] = 0;
}

// 64-bit mix (the splitmix64 finaliser) used to chain block keys.
uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

}  // namespace

extern "C" {

int csa_blocks_create(int32_t n_blocks, csa_block_manager_t** out) {
  if (!out) return api_fail(CSA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (n_blocks < 1) return api_fail(CSA_ERR_INVALID_ARG, "n_blocks=%d < 1", n_blocks);
  csa_block_manager* m = new (std::nothrow) csa_block_manager;
  if (!m) return api_fail(CSA_ERR_INVALID_ARG, "out of host memory");
  m->refs.assign(n_blocks, 0);
  m->free_ids.reserve(n_blocks);
  for (int32_t b = n_blocks - 1; b >= 0; --b) m->free_ids.push_back(b);  // hands out 0, 1, ...
  m->idle_at.resize(n_blocks);
  m->in_idle.assign(n_blocks, 0);
  m->key_of.assign(n_blocks, 0);
  m->has_key.assign(n_blocks, 0);
  *out = m;
  return CSA_OK;
}

int csa_blocks_destroy(csa_block_manager_t* m) {
  delete m;
  return CSA_OK;
}

int csa_blocks_counts(const csa_block_manager_t* m, int32_t* n_free, int32_t* n_idle) {
  if (!m) return api_fail(CSA_ERR_INVALID_ARG, "manager is NULL");
  if (n_free) *n_free = static_cast<int32_t>(m->free_ids.size() + m->idle.size());
  if (n_idle) *n_idle = static_cast<int32_t>(m->idle.size());
  return CSA_OK;
}

int csa_blocks_refcount(const csa_block_manager_t* m, int32_t block, int32_t* count) {
  if (!m || !count) return api_fail(CSA_ERR_INVALID_ARG, "manager or count is NULL");
  if (bad_id(m, block)) return api_fail(CSA_ERR_INVALID_ARG, "block %d out of range", block);
  *count = m->refs[block];
  return CSA_OK;
}

int csa_blocks_alloc(csa_block_manager_t* m, int32_t n, int32_t* blocks) {
  if (!m || (n > 0 && !blocks)) return api_fail(CSA_ERR_INVALID_ARG, "manager or blocks is NULL");
  if (n < 0) return api_fail(CSA_ERR_INVALID_ARG, "n=%d < 0", n);
  if (static_cast<size_t>(n) > m->free_ids.size() + m->idle.size())
    return api_fail(CSA_ERR_UNSUPPORTED, "%d blocks requested, %zu free", n,
                    m->free_ids.size() + m->idle.size());
  for (int32_t i = 0; i < n; ++i) {
    int32_t b;
    if (!m->free_ids.empty()) {
      b = m->free_ids.back();
      m->free_ids.pop_back();
    } else {  // recycle the least recently released registered block
      b = m->idle.front();
      take_from_idle(m, b);
      unregister(m, b);
    }
    m->refs[b] = 1;
    blocks[i] = b;
  }
  return CSA_OK;
}

int csa_blocks_share(csa_block_manager_t* m, int32_t n, const int32_t* blocks) {
  if (!m || (n > 0 && !blocks)) return api_fail(CSA_ERR_INVALID_ARG, "manager or blocks is NULL");
  for (int32_t i = 0; i < n; ++i)
    if (bad_id(m, blocks[i]) || m->refs[blocks[i]] < 1)
      return api_fail(CSA_ERR_INVALID_ARG, "block %d is not in use", blocks[i]);
  for (int32_t i = 0; i < n; ++i) ++m->refs[blocks[i]];
  return CSA_OK;
}

int csa_blocks_release(csa_block_manager_t* m, int32_t n, const int32_t* blocks) {
  if (!m || (n > 0 && !blocks)) return api_fail(CSA_ERR_INVALID_ARG, "manager or blocks is NULL");
  // validate first (a block listed twice needs two references), so an error changes nothing
  std::unordered_map<int32_t, int32_t> need;
  for (int32_t i = 0; i < n; ++i) {
    if (bad_id(m, blocks[i])) return api_fail(CSA_ERR_INVALID_ARG, "block %d out of range", blocks[i]);
    if (++need[blocks[i]] > m->refs[blocks[i]])
      return api_fail(CSA_ERR_INVALID_ARG, "block %d released more often than referenced",
                      blocks[i]);
  }
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = blocks[i];
    if (--m->refs[b] > 0) continue;
    if (m->has_key[b]) {
      m->idle.push_back(b);
      m->idle_at[b] = std::prev(m->idle.end());
      m->in_idle[b] = 1;
    } else {
      m->free_ids.push_back(b);
    }
  }
  return CSA_OK;
}

int csa_blocks_publish(csa_block_manager_t* m, uint64_t key, int32_t block) {
  if (!m) return api_fail(CSA_ERR_INVALID_ARG, "manager is NULL");
  if (bad_id(m, block) || m->refs[block] < 1)
    return api_fail(CSA_ERR_INVALID_ARG, "block %d is not in use", block);
  auto it = m->registry.find(key);
  if (it != m->registry.end()) return CSA_OK;  // first publisher keeps the key
  unregister(m, block);
  m->registry.emplace(key, block);
  m->key_of[block] = key;
  m->has_key[block] = 1;
  return CSA_OK;
}

int csa_blocks_lookup(csa_block_manager_t* m, int32_t n_keys, const uint64_t* keys,
                      int32_t* blocks, int32_t* n_hit) {
  if (!m || !n_hit || (n_keys > 0 && (!keys || !blocks)))
    return api_fail(CSA_ERR_INVALID_ARG, "manager, keys, blocks or n_hit is NULL");
  int32_t h = 0;
  for (; h < n_keys; ++h) {
    auto it = m->registry.find(keys[h]);
    if (it == m->registry.end()) break;
    const int32_t b = it->second;
    if (m->in_idle[b]) take_from_idle(m, b);
    ++m->refs[b];
    blocks[h] = b;
  }
  *n_hit = h;
  return CSA_OK;
}

int csa_blocks_chain_keys(const int32_t* tokens, int32_t n_tokens, int32_t block_tokens,
                          uint64_t seed, uint64_t* keys) {
  if (n_tokens < 0 || block_tokens < 1)
    return api_fail(CSA_ERR_INVALID_ARG, "n_tokens=%d, block_tokens=%d", n_tokens, block_tokens);
  const int32_t nb = n_tokens / block_tokens;
  if (nb > 0 && (!tokens || !keys)) return api_fail(CSA_ERR_INVALID_ARG, "tokens or keys is NULL");
  uint64_t k = mix64(seed ^ 0x6a09e667f3bcc908ULL);
  for (int32_t j = 0; j < nb; ++j) {
    for (int32_t i = 0; i < block_tokens; ++i)
      k = mix64(k ^ (static_cast<uint64_t>(static_cast<uint32_t>(tokens[j * block_tokens + i])) +
                     0x9e3779b97f4a7c15ULL * static_cast<uint64_t>(i + 1)));
    k = mix64(k + static_cast<uint64_t>(j + 1));
    keys[j] = k;
  }
  return CSA_OK;
}

}  // extern "C"
