// Host block pool: free list (min-heap) plus reference counts.  The contract
// of every operation is in include/kvattn.h (kvattn_pool_*).
#include "block_pool.h"

#include <stdio.h>

#include <algorithm>
#include <functional>

#include "kvattn.h"

namespace kvattn {
namespace {

int64_t blocks_for(int64_t len) { return (len + KVATTN_BLOCK_TOKENS - 1) / KVATTN_BLOCK_TOKENS; }

int failmsg(std::string* err, int code, const char* fmt, long long a = 0, long long b = 0, long long c = 0) {
  char buf[256];
  snprintf(buf, sizeof(buf), fmt, a, b, c);
  *err = buf;
  return code;
}

}  // namespace

BlockPool::BlockPool(int32_t num_blocks) : ref_(num_blocks, 0), heap_(num_blocks) {
  // ascending ids form a valid min-heap as they are
  for (int32_t i = 0; i < num_blocks; ++i) heap_[i] = i;
}

int64_t BlockPool::num_free() const {
  std::lock_guard<std::mutex> g(mu_);
  return (int64_t)heap_.size();
}

int32_t BlockPool::refcount(int32_t block) const {
  std::lock_guard<std::mutex> g(mu_);
  if (block < 0 || block >= num_blocks()) return -1;
  return ref_[block];
}

int32_t BlockPool::pop_free(Undo* u) {
  if (heap_.empty()) return -1;
  std::pop_heap(heap_.begin(), heap_.end(), std::greater<int32_t>());
  const int32_t b = heap_.back();
  heap_.pop_back();
  u->heap_changed = true;
  set_ref(b, 1, u);
  return b;
}

void BlockPool::set_ref(int32_t b, int32_t v, Undo* u) {
  u->refs.emplace_back(b, ref_[b]);
  ref_[b] = v;
}

void BlockPool::set_cell(int32_t* cell, int32_t v, Undo* u) {
  u->cells.emplace_back(cell, *cell);
  *cell = v;
}

int BlockPool::dec_ref(int32_t b, Undo* u) {
  set_ref(b, ref_[b] - 1, u);
  if (ref_[b] == 0) {
    heap_.push_back(b);
    std::push_heap(heap_.begin(), heap_.end(), std::greater<int32_t>());
    u->heap_changed = true;
  }
  return KVATTN_OK;
}

void BlockPool::rollback(Undo* u) {
  for (auto it = u->cells.rbegin(); it != u->cells.rend(); ++it) *it->first = it->second;
  for (auto it = u->refs.rbegin(); it != u->refs.rend(); ++it) ref_[it->first] = it->second;
  if (u->heap_changed) {
    heap_.clear();
    for (int32_t b = 0; b < num_blocks(); ++b)
      if (ref_[b] == 0) heap_.push_back(b);  // ascending: already a min-heap
  }
  u->cells.clear();
  u->refs.clear();
  u->heap_changed = false;
}

// Every id in range, and named no more often than its count.
int BlockPool::check_held(const int32_t* ids, int32_t n, const char* what, std::string* err) const {
  std::vector<int32_t> s(ids, ids + n);
  std::sort(s.begin(), s.end());
  for (int32_t i = 0; i < n;) {
    int32_t j = i;
    while (j < n && s[j] == s[i]) ++j;
    const int32_t b = s[i];
    if (b < 0 || b >= num_blocks() || j - i > ref_[b]) {
      if (b < 0 || b >= num_blocks())
        failmsg(err, KVATTN_EINVAL, "block %lld outside [0, %lld)", b, num_blocks());
      else
        failmsg(err, KVATTN_EINVAL, "block %lld named %lld times but held %lld times", b, j - i, ref_[b]);
      *err = std::string(what) + ": " + *err;
      return KVATTN_EINVAL;
    }
    i = j;
  }
  return KVATTN_OK;
}

int BlockPool::alloc(int32_t n, int32_t* ids, std::string* err) {
  std::lock_guard<std::mutex> g(mu_);
  if (n < 0) return failmsg(err, KVATTN_EINVAL, "alloc: n = %lld < 0", n);
  if ((int64_t)n > (int64_t)heap_.size())
    return failmsg(err, KVATTN_ENOSPACE, "alloc: %lld blocks requested, %lld free", n, (long long)heap_.size());
  Undo u;
  for (int32_t i = 0; i < n; ++i) ids[i] = pop_free(&u);
  return KVATTN_OK;
}

int BlockPool::retain(int32_t n, const int32_t* ids, std::string* err) {
  std::lock_guard<std::mutex> g(mu_);
  if (n < 0) return failmsg(err, KVATTN_EINVAL, "retain: n = %lld < 0", n);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = ids[i];
    if (b < 0 || b >= num_blocks() || ref_[b] == 0)
      return failmsg(err, KVATTN_EINVAL, "retain: block %lld is out of range or free", b);
  }
  Undo u;
  for (int32_t i = 0; i < n; ++i) {
    if (ref_[ids[i]] == INT32_MAX) {
      rollback(&u);
      return failmsg(err, KVATTN_EINVAL, "retain: block %lld reference count overflows", ids[i]);
    }
    set_ref(ids[i], ref_[ids[i]] + 1, &u);
  }
  return KVATTN_OK;
}

int BlockPool::release(int32_t n, const int32_t* ids, std::string* err) {
  std::lock_guard<std::mutex> g(mu_);
  if (n < 0) return failmsg(err, KVATTN_EINVAL, "release: n = %lld < 0", n);
  int rc = check_held(ids, n, "release", err);
  if (rc) return rc;
  Undo u;
  for (int32_t i = 0; i < n; ++i) dec_ref(ids[i], &u);
  return KVATTN_OK;
}

int BlockPool::fork(const int32_t* src_row, int32_t* dst_row, int32_t max_blocks, int32_t length,
                    std::string* err) {
  std::lock_guard<std::mutex> g(mu_);
  if (max_blocks < 1 || length < 0 || blocks_for(length) > max_blocks)
    return failmsg(err, KVATTN_EINVAL, "fork: length %lld does not fit %lld blocks", length, max_blocks);
  if (src_row == dst_row) return failmsg(err, KVATTN_EINVAL, "fork: source and destination rows are one row");
  const int32_t nb = (int32_t)blocks_for(length);
  for (int32_t j = 0; j < nb; ++j) {
    const int32_t b = src_row[j];
    if (b < 0 || b >= num_blocks() || ref_[b] == 0 || ref_[b] == INT32_MAX)
      return failmsg(err, KVATTN_EINVAL, "fork: entry %lld names block %lld, which is out of range or free", j, b);
  }
  Undo u;
  for (int32_t j = 0; j < nb; ++j) set_ref(src_row[j], ref_[src_row[j]] + 1, &u);
  for (int32_t j = 0; j < max_blocks; ++j) dst_row[j] = j < nb ? src_row[j] : -1;
  return KVATTN_OK;
}

int BlockPool::free_seq(int32_t* row, int32_t max_blocks, int32_t length, std::string* err) {
  std::lock_guard<std::mutex> g(mu_);
  if (max_blocks < 1 || length < 0 || blocks_for(length) > max_blocks)
    return failmsg(err, KVATTN_EINVAL, "free_seq: length %lld does not fit %lld blocks", length, max_blocks);
  const int32_t nb = (int32_t)blocks_for(length);
  int rc = check_held(row, nb, "free_seq", err);
  if (rc) return rc;
  Undo u;
  for (int32_t j = 0; j < nb; ++j) {
    dec_ref(row[j], &u);
    row[j] = -1;
  }
  return KVATTN_OK;
}

int BlockPool::prepare_append(int32_t rows, int32_t* tables, int32_t max_blocks, const int32_t* cur_lens,
                              const int32_t* new_lens, int32_t* copy_src, int32_t* copy_dst, int32_t* n_copies,
                              std::string* err) {
  std::lock_guard<std::mutex> g(mu_);
  if (rows < 0 || max_blocks < 1) return failmsg(err, KVATTN_EINVAL, "prepare_append: rows %lld, max_blocks %lld",
                                                 rows, max_blocks);
  Undo u;
  int32_t copies = 0;
  for (int32_t b = 0; b < rows; ++b) {
    int32_t* row = tables + (int64_t)b * max_blocks;
    const int32_t cur = cur_lens[b], nw = new_lens[b];
    int rc = KVATTN_OK;
    if (cur < 0 || nw < cur || blocks_for(nw) > max_blocks)
      rc = failmsg(err, KVATTN_EINVAL, "prepare_append: row %lld grows %lld -> %lld", b, cur, nw);
    if (!rc) rc = check_held(row, (int32_t)blocks_for(cur), "prepare_append", err);
    if (!rc && nw > cur && cur % KVATTN_BLOCK_TOKENS) {
      // the partly filled last block gets written: copy it first if shared
      const int32_t j = cur / KVATTN_BLOCK_TOKENS;
      const int32_t old = row[j];
      if (ref_[old] > 1) {
        const int32_t fresh = pop_free(&u);
        if (fresh < 0) {
          rc = failmsg(err, KVATTN_ENOSPACE, "prepare_append: pool exhausted at row %lld", b);
        } else {
          dec_ref(old, &u);
          set_cell(row + j, fresh, &u);
          copy_src[copies] = old;
          copy_dst[copies] = fresh;
          ++copies;
        }
      }
    }
    for (int64_t j = blocks_for(cur); !rc && j < blocks_for(nw); ++j) {
      const int32_t fresh = pop_free(&u);
      if (fresh < 0)
        rc = failmsg(err, KVATTN_ENOSPACE, "prepare_append: pool exhausted at row %lld", b);
      else
        set_cell(row + j, fresh, &u);
    }
    if (rc) {
      rollback(&u);
      return rc;
    }
  }
  *n_copies = copies;
  return KVATTN_OK;
}

int BlockPool::reorder(int32_t n_rows, const int32_t* perm, int32_t src_rows, const int32_t* src_tables,
                       const int32_t* src_lens, int32_t max_blocks, int32_t* dst_tables, int32_t* dst_lens,
                       std::string* err) {
  std::lock_guard<std::mutex> g(mu_);
  if (n_rows < 0 || src_rows < 0 || max_blocks < 1)
    return failmsg(err, KVATTN_EINVAL, "reorder: n_rows %lld, src_rows %lld, max_blocks %lld", n_rows, src_rows,
                   max_blocks);
  const int32_t* s0 = src_tables;
  const int32_t* s1 = src_tables + (int64_t)src_rows * max_blocks;
  const int32_t* d0 = dst_tables;
  const int32_t* d1 = dst_tables + (int64_t)n_rows * max_blocks;
  if (n_rows && src_rows && s0 < d1 && d0 < s1)
    return failmsg(err, KVATTN_EINVAL, "reorder: destination tables overlap the source tables");
  // every source row must hold its blocks (all rows' references together)
  std::vector<int32_t> held;
  for (int32_t r = 0; r < src_rows; ++r) {
    const int32_t L = src_lens[r];
    if (L < 0 || blocks_for(L) > max_blocks)
      return failmsg(err, KVATTN_EINVAL, "reorder: source row %lld has length %lld", r, L);
    held.insert(held.end(), src_tables + (int64_t)r * max_blocks,
                src_tables + (int64_t)r * max_blocks + blocks_for(L));
  }
  int rc = check_held(held.data(), (int32_t)held.size(), "reorder", err);
  if (rc) return rc;
  Undo u;
  for (int32_t i = 0; i < n_rows; ++i) {
    const int32_t p = perm[i];
    const bool valid = p >= 0 && p < src_rows;
    const int32_t* srow = src_tables + (int64_t)p * max_blocks;
    const int32_t nb = valid ? (int32_t)blocks_for(src_lens[p]) : 0;
    for (int32_t j = 0; j < nb; ++j) {
      if (ref_[srow[j]] == INT32_MAX) {
        rollback(&u);
        return failmsg(err, KVATTN_EINVAL, "reorder: block %lld reference count overflows", srow[j]);
      }
      set_ref(srow[j], ref_[srow[j]] + 1, &u);
    }
  }
  for (int32_t k = 0; k < (int32_t)held.size(); ++k) dec_ref(held[k], &u);
  for (int32_t i = 0; i < n_rows; ++i) {
    const int32_t p = perm[i];
    const bool valid = p >= 0 && p < src_rows;
    for (int32_t j = 0; j < max_blocks; ++j)
      dst_tables[(int64_t)i * max_blocks + j] = valid ? src_tables[(int64_t)p * max_blocks + j] : -1;
    dst_lens[i] = valid ? src_lens[p] : 0;
  }
  return KVATTN_OK;
}

}  // namespace kvattn
