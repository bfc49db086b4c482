// Stress driver for the streamed fit's host copy pool (means_clustering_amd/csrc/copy_pool.hpp), built by
// tests/test_sanitizers.py with ThreadSanitizer (and separately with AddressSanitizer): several caller threads
// issue copies of many sizes at once through pools of 0 to 8 workers, every destination is checked byte for byte,
// and pools are created and destroyed repeatedly.  Exits 0 on success, 1 on a wrong byte; the sanitizer
// reports any data race or bad access itself (non-zero exit).
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

#include "copy_pool.hpp"

static bool check_pool(int workers, int callers, int rounds) {
  km::CopyPool pool(workers);
  const size_t sizes[] = {0, 1, 7, 63, 64, 65, 1000, 4096, 4097, 100000, 1 << 20};
  bool ok = true;
  std::vector<std::thread> th;
  std::vector<int> bad(callers, 0);
  for (int c = 0; c < callers; ++c)
    th.emplace_back([&, c] {
      std::vector<unsigned char> src(1 << 20), dst(1 << 20);
      for (int r = 0; r < rounds; ++r)
        for (size_t n : sizes) {
          for (size_t i = 0; i < n; ++i) src[i] = (unsigned char)(i * 31 + r * 7 + c * 13 + n);
          std::memset(dst.data(), 0xA5, dst.size());
          pool.copy(dst.data(), src.data(), n);
          if (std::memcmp(dst.data(), src.data(), n) != 0) bad[c]++;
          if (n < dst.size() && dst[n] != 0xA5) bad[c]++;  // nothing written past the end
        }
    });
  for (auto& t : th) t.join();
  for (int b : bad) ok = ok && b == 0;
  return ok;
}

int main() {
  bool ok = true;
  for (int workers : {0, 1, 3, 8})
    for (int callers : {1, 4}) ok = ok && check_pool(workers, callers, 3);
  for (int i = 0; i < 20; ++i) {  // construction and teardown while idle
    km::CopyPool p(i % 5);
    (void)p;
  }
  std::printf(ok ? "copy pool: ok\n" : "copy pool: WRONG BYTES\n");
  return ok ? 0 : 1;
}
