// Host-side KV page allocator and per-sequence bookkeeping.  Free of HIP so
// that it can be unit-tested on a machine without a GPU.
#pragma once
#include <algorithm>
#include <cstdint>
#include <random>
#include <vector>

namespace sdm {

class PagePool {
 public:
  explicit PagePool(int64_t n_pages = 0) { reset(n_pages); }

  void reset(int64_t n_pages) {
    free_.clear();
    free_.reserve((size_t)n_pages);
    for (int64_t p = n_pages - 1; p >= 0; --p) free_.push_back((int32_t)p);  // pops ascending
    total_ = n_pages;
  }
  int64_t free_count() const { return (int64_t)free_.size(); }
  int64_t total() const { return total_; }

  // Take `count` pages; all or nothing.
  bool take(int64_t count, std::vector<int32_t>* out) {
    if (count < 0 || count > (int64_t)free_.size()) return false;
    for (int64_t i = 0; i < count; ++i) {
      out->push_back(free_.back());
      free_.pop_back();
    }
    return true;
  }
  void give_back(const std::vector<int32_t>& pages) {
    for (auto it = pages.rbegin(); it != pages.rend(); ++it) free_.push_back(*it);
  }
  void shuffle(uint64_t seed) {
    std::mt19937_64 g(seed);
    std::shuffle(free_.begin(), free_.end(), g);
  }

 private:
  std::vector<int32_t> free_;
  int64_t total_ = 0;
};

// State of one sequence slot.
//   len        committed positions (their K/V in the cache are causal)
//   pages      page ids covering positions [0, pages.size() * page_tokens)
//   prefilled  the prompt has been committed
//   verified   block size of the last causal block forward whose K/V are still
//              in the uncommitted slots (0 if none): what commit may accept
struct SeqState {
  int32_t len = 0;
  std::vector<int32_t> pages;
  bool prefilled = false;
  int32_t verified = 0;
};

// Pages needed so that positions [0, end) are covered.
inline int64_t pages_for(int64_t end, int page_tokens) { return (end + page_tokens - 1) / page_tokens; }

}  // namespace sdm
