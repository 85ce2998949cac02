// LIFO block free-list ("Rebuilding Kshipra Around Memory", section 1: the KV
// arena is reserved once as fixed-size blocks; the free-list starts as
// [0 .. n-1] so the first pop hands out n-1, and a released block is the next
// one handed out). Host-only; no HIP calls.
#pragma once

#include <stdint.h>

#include <vector>

namespace vla {

class BlockPool {
 public:
  explicit BlockPool(int n = 0) { reset(n); }

  void reset(int n) {
    n_ = n;
    free_.resize(n);
    is_free_.assign(n, 1);
    for (int i = 0; i < n; ++i) free_[i] = i;
  }
  int size() const { return n_; }
  int free_count() const { return (int)free_.size(); }

  // pop k blocks (in pop order) into out; false and unchanged if fewer are free
  bool alloc(int k, std::vector<int>* out) {
    if (k < 0 || k > (int)free_.size()) return false;
    for (int i = 0; i < k; ++i) {
      const int b = free_.back();
      free_.pop_back();
      is_free_[b] = 0;
      out->push_back(b);
    }
    return true;
  }
  // push blocks in the order given; false (unchanged) on a bad or already-free id
  bool release(const int* blocks, int k) {
    for (int i = 0; i < k; ++i) {
      const int b = blocks[i];
      if (b < 0 || b >= n_ || is_free_[b]) return false;
      for (int j = 0; j < i; ++j)
        if (blocks[j] == b) return false;
    }
    for (int i = 0; i < k; ++i) {
      free_.push_back(blocks[i]);
      is_free_[blocks[i]] = 1;
    }
    return true;
  }
  const std::vector<int>& free_list() const { return free_; }

 private:
  int n_ = 0;
  std::vector<int> free_;
  std::vector<char> is_free_;
};

}  // namespace vla
