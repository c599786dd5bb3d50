// Host block manager: paging, prefix sharing and copy-on-write.
//
// "Large-model inference KV Cache memory optimisation: from PagedAttention to
// AI memory systems" (wmrh.cn) 2.2-2.3: fixed blocks come from a common pool
// on demand and go back to it when a request ends; 3.1-3.2: requests with a
// common prefix reference the same blocks, each block counts its referencing
// sequences (atomically: several threads may fork and free at once), and a
// block that others still reference is copied before a sequence writes into
// it; 7.2: getting that copy wrong corrupts the other sequences.
// "The KV Cache memory ledger" (gcssc.sfwss.com) 4: copy only at the fork.
//
// The manager only does the bookkeeping.  It hands back the slot of every
// appended token (for pkv_kv_append) and the (old, new) block pairs that
// must be copied on the device (pkv_copy_blocks) before those appends run.
#include "pkv_internal.h"

#include <atomic>
#include <memory>
#include <mutex>
#include <unordered_map>
#include <unordered_set>
#include <vector>

struct pkv_block_manager {
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t tokens = 0;
  };
  int32_t num_blocks = 0;
  int32_t block_size = 16;
  std::mutex mu;                                  // guards free_list and seqs
  std::vector<int32_t> free_list;                 // blocks are taken from the end
  std::unique_ptr<std::atomic<int32_t>[]> ref;    // readable without the lock
  std::unordered_map<int64_t, Seq> seqs;

  int32_t take() {
    const int32_t b = free_list.back();
    free_list.pop_back();
    ref[b].store(1, std::memory_order_relaxed);
    return b;
  }
  void release(int32_t b) {
    if (ref[b].fetch_sub(1, std::memory_order_acq_rel) == 1) free_list.push_back(b);
  }
};

extern "C" {

PKV_API pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order) {
  if (num_blocks <= 0 || block_size != PKV_BLOCK_SIZE) return nullptr;
  auto* bm = new (std::nothrow) pkv_block_manager();
  if (!bm) return nullptr;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ref.reset(new (std::nothrow) std::atomic<int32_t>[num_blocks]);
  if (!bm->ref) {
    delete bm;
    return nullptr;
  }
  std::vector<char> seen(num_blocks, 0);
  bm->free_list.resize(num_blocks);
  for (int32_t i = 0; i < num_blocks; ++i) {
    const int32_t b = free_order ? free_order[i] : i;
    if (b < 0 || b >= num_blocks || seen[b]) {   // not a permutation
      delete bm;
      return nullptr;
    }
    seen[b] = 1;
    bm->free_list[num_blocks - 1 - i] = b;      // free_order[0] is taken first
    bm->ref[b].store(0, std::memory_order_relaxed);
  }
  return bm;
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq) {
  if (!bm) return PKV_ERR_NULL;
  std::lock_guard<std::mutex> g(bm->mu);
  if (!bm->seqs.emplace(seq, pkv_block_manager::Seq{}).second) return PKV_ERR_SEQUENCE;
  return PKV_OK;
}

int pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child) {
  if (!bm) return PKV_ERR_NULL;
  std::lock_guard<std::mutex> g(bm->mu);
  auto p = bm->seqs.find(parent);
  if (p == bm->seqs.end() || bm->seqs.count(child)) return PKV_ERR_SEQUENCE;
  pkv_block_manager::Seq c = p->second;           // shares every block, the last one too
  for (int32_t b : c.blocks) bm->ref[b].fetch_add(1, std::memory_order_relaxed);
  bm->seqs.emplace(child, std::move(c));
  return PKV_OK;
}

int pkv_bm_append_slots(pkv_block_manager* bm, const int64_t* seqs, int32_t n, int64_t* slots_out,
                        int32_t* copy_src, int32_t* copy_dst, int32_t copy_capacity,
                        int32_t* num_copies) {
  if (!bm || (n > 0 && (!seqs || !slots_out || !copy_src || !copy_dst)) || !num_copies)
    return PKV_ERR_NULL;
  if (n < 0 || copy_capacity < n) return PKV_ERR_SHAPE;
  std::lock_guard<std::mutex> g(bm->mu);
  // check everything first: the call either fully happens or changes nothing
  std::vector<pkv_block_manager::Seq*> s(n);
  std::unordered_set<int64_t> seen;
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end() || !seen.insert(seqs[i]).second) return PKV_ERR_SEQUENCE;
    s[i] = &it->second;
    const int64_t off = s[i]->tokens % bm->block_size;
    if (off == 0 || bm->ref[s[i]->blocks.back()].load(std::memory_order_relaxed) > 1) ++need;
  }
  if (need > (int64_t)bm->free_list.size()) return PKV_ERR_NO_BLOCKS;
  int32_t nc = 0;
  for (int32_t i = 0; i < n; ++i) {
    auto& q = *s[i];
    const int64_t off = q.tokens % bm->block_size;
    if (off == 0) {
      q.blocks.push_back(bm->take());
    } else if (bm->ref[q.blocks.back()].load(std::memory_order_relaxed) > 1) {
      const int32_t fresh = bm->take();
      copy_src[nc] = q.blocks.back();
      copy_dst[nc] = fresh;
      ++nc;
      bm->release(q.blocks.back());               // still referenced by the others
      q.blocks.back() = fresh;
    }
    slots_out[i] = (int64_t)q.blocks.back() * bm->block_size + off;
    ++q.tokens;
  }
  *num_copies = nc;
  return PKV_OK;
}

int pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq) {
  if (!bm) return PKV_ERR_NULL;
  std::lock_guard<std::mutex> g(bm->mu);
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PKV_ERR_SEQUENCE;
  for (int32_t b : it->second.blocks) bm->release(b);
  bm->seqs.erase(it);
  return PKV_OK;
}

int pkv_bm_num_free(pkv_block_manager* bm) {
  if (!bm) return PKV_ERR_NULL;
  std::lock_guard<std::mutex> g(bm->mu);
  return (int)bm->free_list.size();
}

int pkv_bm_refcount(pkv_block_manager* bm, int32_t block) {
  if (!bm) return PKV_ERR_NULL;
  if (block < 0 || block >= bm->num_blocks) return PKV_ERR_SHAPE;
  return bm->ref[block].load(std::memory_order_acquire);
}

int pkv_bm_block_tables(pkv_block_manager* bm, const int64_t* seqs, int32_t n, int32_t max_blocks,
                        int32_t* tables_out, int32_t* lens_out) {
  if (!bm || (n > 0 && (!seqs || !tables_out || !lens_out))) return PKV_ERR_NULL;
  if (n < 0 || max_blocks <= 0) return PKV_ERR_SHAPE;
  std::lock_guard<std::mutex> g(bm->mu);
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return PKV_ERR_SEQUENCE;
    if ((int64_t)it->second.blocks.size() > max_blocks || it->second.tokens > 0x7FFFFFFF)
      return PKV_ERR_SHAPE;
  }
  for (int32_t i = 0; i < n; ++i) {
    const auto& q = bm->seqs.find(seqs[i])->second;
    int32_t* row = tables_out + (int64_t)i * max_blocks;
    int32_t j = 0;
    for (; j < (int32_t)q.blocks.size(); ++j) row[j] = q.blocks[j];
    for (; j < max_blocks; ++j) row[j] = -1;
    lens_out[i] = (int32_t)q.tokens;
  }
  return PKV_OK;
}

}  // extern "C"
