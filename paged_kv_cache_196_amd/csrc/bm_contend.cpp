// bm_contend.cpp — host timing driver for the block manager's C entry
// points under contention (no device work).  T threads share one manager;
// each allocates `batch` blocks with one pa_bm_alloc call and releases them
// with one pa_bm_release call, over and over for `ms` milliseconds.  Prints
// one JSON object: wall nanoseconds per block allocated and released,
// summed over all threads (and the same loop on one thread), and whether
// every block was back in the pool at the end.
//
//   bm_contend [threads=8] [batch=64] [ms=300] [num_blocks=100000]
#include <atomic>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <thread>
#include <vector>

#include "pagedattn.h"

namespace {

double run(int threads, int batch, int ms, int nb, bool* ok) {
  pa_block_manager* bm = pa_bm_create(nb, 16);
  if (!bm) {
    *ok = false;
    return 0.0;
  }
  std::atomic<bool> stop{false};
  std::atomic<long> blocks{0};
  std::atomic<int> failed{0};
  std::vector<std::thread> pool;
  const auto t0 = std::chrono::steady_clock::now();
  for (int t = 0; t < threads; ++t)
    pool.emplace_back([&]() {
      std::vector<int32_t> ids(batch);
      long n = 0;
      while (!stop.load(std::memory_order_relaxed)) {
        for (int i = 0; i < 64; ++i) {
          if (pa_bm_alloc(bm, batch, ids.data()) != PA_OK ||
              pa_bm_release(bm, ids.data(), batch) != PA_OK) {
            failed++;
            return;
          }
        }
        n += 64L * batch;
      }
      blocks += n;
    });
  std::this_thread::sleep_for(std::chrono::milliseconds(ms));
  stop = true;
  for (auto& th : pool) th.join();
  const double dt = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
  *ok = *ok && failed.load() == 0 && pa_bm_num_free(bm) == nb;
  pa_bm_destroy(bm);
  return blocks.load() ? dt / (double)blocks.load() * 1e9 : 0.0;
}

}  // namespace

int main(int argc, char** argv) {
  const int threads = argc > 1 ? atoi(argv[1]) : 8;
  const int batch = argc > 2 ? atoi(argv[2]) : 64;
  const int ms = argc > 3 ? atoi(argv[3]) : 300;
  const int nb = argc > 4 ? atoi(argv[4]) : 100000;
  if (threads < 1 || batch < 1 || ms < 1 || (long)threads * batch > nb) {
    std::fprintf(stderr, "bad arguments\n");
    return 2;
  }
  bool ok = true;
  const double many = run(threads, batch, ms, nb, &ok);
  const double one = run(1, batch, ms, nb, &ok);
  std::printf(
      "{\"threads\": %d, \"blocks_per_call\": %d, \"alloc_release_ns_per_block\": %.2f, "
      "\"single_thread_alloc_release_ns_per_block\": %.2f, \"pool_whole_after\": %s}\n",
      threads, batch, many, one, ok ? "true" : "false");
  return ok ? 0 : 1;
}
