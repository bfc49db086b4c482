// Host-side copy pool of the streamed fit: memcpy of one piece of pageable
// host memory into a pinned staging slot, split over a few worker threads
// and the calling thread (one thread cannot keep up with the host link).
// Host-only C++ (no HIP), so it can be built and stress-tested on its own
// (under ThreadSanitizer in the CPU test tier).  Internal to the library.
#pragma once

#include <condition_variable>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <thread>
#include <vector>

namespace km {

class CopyPool {
 public:
  explicit CopyPool(int workers) : nw_(workers) {
    for (int i = 0; i < nw_; ++i) th_.emplace_back([this, i] { run(i + 1); });
  }
  ~CopyPool() {
    {
      std::lock_guard<std::mutex> g(mu_);
      stop_ = true;
    }
    cv_.notify_all();
    for (auto& t : th_) t.join();
  }
  // memcpy(dst, src, n) split over the workers and the calling thread; returns when all parts are done.
  void copy(uint8_t* dst, const uint8_t* src, size_t n) {
    std::lock_guard<std::mutex> call(call_mu_);
    const int parts = nw_ + 1;
    {
      std::lock_guard<std::mutex> g(mu_);
      dst_ = dst;
      src_ = src;
      n_ = n;
      left_ = nw_;
      ++gen_;
    }
    cv_.notify_all();
    part(0, parts, dst, src, n);
    std::unique_lock<std::mutex> g(mu_);
    done_.wait(g, [&] { return left_ == 0; });
  }

 private:
  static size_t bound(int i, int parts, size_t n) { return i >= parts ? n : (n / parts * i) & ~(size_t)63; }
  static void part(int i, int parts, uint8_t* d, const uint8_t* s, size_t n) {
    const size_t a = bound(i, parts, n), b = bound(i + 1, parts, n);
    if (b > a) std::memcpy(d + a, s + a, b - a);
  }
  void run(int idx) {
    uint64_t seen = 0;
    for (;;) {
      uint8_t* d;
      const uint8_t* s;
      size_t n;
      {
        std::unique_lock<std::mutex> g(mu_);
        cv_.wait(g, [&] { return stop_ || gen_ != seen; });
        if (stop_) return;
        seen = gen_;
        d = dst_;
        s = src_;
        n = n_;
      }
      part(idx, nw_ + 1, d, s, n);
      std::lock_guard<std::mutex> g(mu_);
      if (--left_ == 0) done_.notify_one();
    }
  }
  int nw_;
  std::vector<std::thread> th_;
  std::mutex mu_, call_mu_;
  std::condition_variable cv_, done_;
  uint8_t* dst_ = nullptr;
  const uint8_t* src_ = nullptr;
  size_t n_ = 0;
  int left_ = 0;
  uint64_t gen_ = 0;
  bool stop_ = false;
};

}  // namespace km
