// Host-only unit test of the KV page allocator (no GPU, no HIP).
// Built with g++ and the address / undefined-behaviour sanitizers by
// tests/test_host_cpp.py; exits non-zero on the first failed check.
#include <cstdio>
#include <cstdlib>
#include <set>
#include <vector>

#include "page_pool.hpp"

using sdm::PagePool;
using sdm::pages_for;

static int g_fail = 0;
#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                          \
    }                                                                    \
  } while (0)

int main() {
  // pages_for: ceil(end / page_tokens)
  CHECK(pages_for(0, 64) == 0);
  CHECK(pages_for(1, 64) == 1);
  CHECK(pages_for(64, 64) == 1);
  CHECK(pages_for(65, 64) == 2);
  CHECK(pages_for(8192 + 32, 64) == 129);

  // a fresh pool hands out 0, 1, 2, ... and counts what it holds
  PagePool pool(10);
  CHECK(pool.total() == 10 && pool.free_count() == 10);
  std::vector<int32_t> a;
  CHECK(pool.take(3, &a));
  CHECK(a.size() == 3 && a[0] == 0 && a[1] == 1 && a[2] == 2);
  CHECK(pool.free_count() == 7);

  // all or nothing: asking for more than is free takes nothing
  std::vector<int32_t> b;
  CHECK(!pool.take(8, &b));
  CHECK(b.empty() && pool.free_count() == 7);
  CHECK(!pool.take(-1, &b));
  CHECK(pool.take(0, &b) && b.empty());

  // exhaust, then return one sequence's pages: they come back in their order
  CHECK(pool.take(7, &b));
  CHECK(pool.free_count() == 0);
  std::vector<int32_t> none;
  CHECK(!pool.take(1, &none) && none.empty());
  pool.give_back(a);
  CHECK(pool.free_count() == 3);
  std::vector<int32_t> c;
  CHECK(pool.take(3, &c));
  CHECK(c == a);

  // every id is handed out once: no page is shared by two holders
  {
    std::set<int32_t> seen(b.begin(), b.end());
    for (int32_t p : c) CHECK(!seen.count(p));
    seen.insert(c.begin(), c.end());
    CHECK(seen.size() == 10 && *seen.begin() == 0 && *seen.rbegin() == 9);
  }

  // a shuffled pool is a permutation of the free ids, reproducible by seed
  PagePool s1(64), s2(64), s3(64);
  s1.shuffle(1234);
  s2.shuffle(1234);
  s3.shuffle(99);
  std::vector<int32_t> p1, p2, p3;
  CHECK(s1.take(64, &p1) && s2.take(64, &p2) && s3.take(64, &p3));
  CHECK(p1 == p2);
  CHECK(p1 != p3);
  std::set<int32_t> u(p1.begin(), p1.end());
  CHECK(u.size() == 64 && *u.begin() == 0 && *u.rbegin() == 63);

  // reset returns the pool to its fresh state
  s1.reset(5);
  CHECK(s1.free_count() == 5 && s1.total() == 5);
  std::vector<int32_t> r;
  CHECK(s1.take(5, &r) && r[0] == 0 && r[4] == 4);

  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("page pool: all checks passed\n");
  return 0;
}
