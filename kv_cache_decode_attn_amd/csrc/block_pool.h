// Host block pool of a paged KV cache: the free list of physical blocks with
// reference counts behind kvattn_pool_* (include/kvattn.h has the contract).
//
// "KV Cache, Flash Attention and Inference Optimization"
// (factory.pai-world.com), section "Exercises": a toy PagedAttention keeps
// 16-token blocks on a free list and returns a sequence's blocks to the pool
// when it ends; section "PagedAttention": parallel branches (beam search,
// parallel sampling) share blocks through the page table.  "KV Cache Fully
// Explained" (techblog.paldyn.com), section "(4) PagedAttention": requests
// with a common prefix share physical blocks, copy-on-write.
//
// A block's count is the number of table rows naming it; free at 0.  Free
// blocks sit in a min-heap, so the lowest free id is handed out first and
// allocation is O(log n).  Every operation either completes or leaves the
// pool and the caller's tables as they were: an undo log restores counts and
// table cells, and a failed operation that moved blocks on or off the free
// list rebuilds the heap (O(num_blocks), on failure only).  One mutex
// serialises the operations on a pool.
#pragma once

#include <stdint.h>

#include <mutex>
#include <string>
#include <utility>
#include <vector>

namespace kvattn {

class BlockPool {
 public:
  explicit BlockPool(int32_t num_blocks);

  int32_t num_blocks() const { return (int32_t)ref_.size(); }
  int64_t num_free() const;
  int32_t refcount(int32_t block) const;

  // Each returns KVATTN_OK or a negative kvattn_status, with a message in
  // *err on failure.
  int alloc(int32_t n, int32_t* ids, std::string* err);
  int retain(int32_t n, const int32_t* ids, std::string* err);
  int release(int32_t n, const int32_t* ids, std::string* err);
  int fork(const int32_t* src_row, int32_t* dst_row, int32_t max_blocks, int32_t length, std::string* err);
  int free_seq(int32_t* row, int32_t max_blocks, int32_t length, std::string* err);
  int prepare_append(int32_t rows, int32_t* tables, int32_t max_blocks, const int32_t* cur_lens,
                     const int32_t* new_lens, int32_t* copy_src, int32_t* copy_dst, int32_t* n_copies,
                     std::string* err);
  int reorder(int32_t n_rows, const int32_t* perm, int32_t src_rows, const int32_t* src_tables,
              const int32_t* src_lens, int32_t max_blocks, int32_t* dst_tables, int32_t* dst_lens,
              std::string* err);

 private:
  // Changes made inside one operation, undone in reverse on failure.
  struct Undo {
    std::vector<std::pair<int32_t, int32_t>> refs;   // (block, count before)
    std::vector<std::pair<int32_t*, int32_t>> cells;  // (table cell, value before)
    bool heap_changed = false;
  };
  int32_t pop_free(Undo* u);
  void set_ref(int32_t b, int32_t v, Undo* u);
  void set_cell(int32_t* cell, int32_t v, Undo* u);
  void rollback(Undo* u);
  int check_held(const int32_t* ids, int32_t n, const char* what, std::string* err) const;
  int dec_ref(int32_t b, Undo* u);  // count - 1; the block joins the free list at 0

  mutable std::mutex mu_;
  std::vector<int32_t> ref_;
  std::vector<int32_t> heap_;  // free ids, min-heap
};

}  // namespace kvattn
