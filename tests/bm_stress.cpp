// Concurrency stress of the lock-free host block manager (block_manager.h),
// built by tests/test_block_manager.py with ThreadSanitizer and with
// AddressSanitizer + UBSan.  T threads run random operations on one
// manager: reserve-and-take blocks (singly or as one chain), release
// references (singly or several in one call), add
// references to blocks they hold, and add references to blocks other
// threads published (which may meanwhile have been released and handed out
// again: the manager must stay consistent either way).  After every round,
// with all threads joined, each block's reference count must equal the
// references the threads hold on it, and the free count must equal the
// blocks nobody holds: a block handed out twice, lost or freed twice breaks
// one of these.  Prints "ok" and exits 0 on success.
#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <thread>
#include <vector>

#include "block_manager.h"

int main(int argc, char** argv) {
  const int nb = argc > 1 ? atoi(argv[1]) : 1024;
  const int threads = argc > 2 ? atoi(argv[2]) : 8;
  const int rounds = argc > 3 ? atoi(argv[3]) : 6;
  const int iters = argc > 4 ? atoi(argv[4]) : 20000;
  pa::BlockManager m(nb, 16);
  std::vector<std::vector<int>> held(threads);
  std::vector<std::atomic<int>> pub(64);
  for (auto& p : pub) p.store(-1);
  std::atomic<long> failures{0};
  for (int round = 0; round < rounds; ++round) {
    std::vector<std::thread> pool;
    for (int t = 0; t < threads; ++t) {
      pool.emplace_back([&, t]() {
        std::mt19937 rng(1000u * (unsigned)round + (unsigned)t);
        std::vector<int>& h = held[t];
        for (int i = 0; i < iters; ++i) {
          const int op = (int)(rng() % 10);
          if (op < 3) {  // fresh blocks, all or nothing: one by one or as a batch
            const int n = 1 + (int)(rng() % 8);
            if (m.reserve(n)) {
              int ids[8];
              if (rng() % 2) {
                m.take_reserved_n(n, ids);
              } else {
                for (int k = 0; k < n; ++k) ids[k] = m.take_reserved();
              }
              for (int k = 0; k < n; ++k) {
                if (ids[k] < 0 || ids[k] >= nb || m.refcount(ids[k]) < 1) failures++;
                h.push_back(ids[k]);
              }
            }
          } else if (op < 6) {  // release references: one, or several in one call
            const int n = std::min<int>((int)h.size(), 1 + (int)(rng() % 4));
            int ids[4];
            for (int k = 0; k < n; ++k) {
              const size_t j = rng() % h.size();
              ids[k] = h[j];
              h[j] = h.back();
              h.pop_back();
            }
            if (n == 1 ? !m.drop(ids[0]) : m.drop_n(ids, n) != n) failures++;
          } else if (op < 7) {  // another reference to a held block
            if (!h.empty()) {
              const int id = h[rng() % h.size()];
              if (!m.share(id)) failures++;
              h.push_back(id);
            }
          } else if (op < 8) {  // publish a held block
            if (!h.empty()) pub[rng() % pub.size()].store(h[rng() % h.size()]);
          } else {  // a reference to a published block, if it is still in use
            const int id = pub[rng() % pub.size()].load();
            if (id >= 0 && m.share(id)) h.push_back(id);
          }
        }
      });
    }
    for (auto& th : pool) th.join();
    std::vector<int> refs(nb, 0);
    for (auto& h : held)
      for (int id : h) refs[id]++;
    int unheld = 0;
    for (int id = 0; id < nb; ++id) {
      if (m.refcount(id) != refs[id]) {
        std::printf("round %d: block %d refcount %d held %d\n", round, id, m.refcount(id), refs[id]);
        return 1;
      }
      unheld += refs[id] == 0;
    }
    if (m.num_free() != unheld) {
      std::printf("round %d: num_free %d, blocks held by nobody %d\n", round, m.num_free(), unheld);
      return 1;
    }
  }
  for (auto& h : held)
    for (int id : h)
      if (!m.drop(id)) failures++;
  if (m.num_free() != nb || failures.load() != 0) {
    std::printf("end: num_free %d of %d, failed operations %ld\n", m.num_free(), nb, failures.load());
    return 1;
  }
  // everything free again: all nb blocks can be taken, each exactly once
  std::vector<int> seen(nb, 0);
  if (!m.reserve(nb) || m.reserve(1)) return 1;
  for (int k = 0; k < nb; ++k) seen[m.take_reserved()]++;
  for (int id = 0; id < nb; ++id)
    if (seen[id] != 1) return 1;
  std::printf("ok\n");
  return 0;
}
