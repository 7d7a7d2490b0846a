// Prints one line per mismatch between FastDiv (exact_attention_84_amd/csrc/
// fa_fastdiv.hpp) and plain integer division, then "checked N".
#include <cstdint>
#include <cstdio>
#include <vector>

#include "fa_fastdiv.hpp"

int main() {
  std::vector<uint32_t> divs;
  for (uint32_t d = 1; d <= 4096; ++d) divs.push_back(d);
  for (int s = 12; s < 31; ++s) {
    const uint32_t p = 1u << s;
    for (uint32_t d : {p - 1, p, p + 1, p + p / 3, p + p / 2 + 7}) divs.push_back(d);
  }
  divs.push_back(0x7fffffffu);
  uint64_t x = 0x9e3779b97f4a7c15ull, checked = 0;
  int bad = 0;
  auto rnd = [&]() { x ^= x << 13; x ^= x >> 7; x ^= x << 17; return static_cast<uint32_t>(x); };
  for (int i = 0; i < 2000; ++i) divs.push_back(1 + rnd() % 0x7fffffffu);
  for (uint32_t d : divs) {
    const fa::FastDiv f = fa::FastDiv::make(d);
    std::vector<uint32_t> ns;
    for (uint32_t n = 0; n < 2048; ++n) ns.push_back(n);
    for (uint64_t k : {1ull, 2ull, 3ull, 1000ull, 0x7fffffffull / d}) {
      const uint64_t c = k * d;
      for (int64_t e = -1; e <= 1; ++e)
        if (c + e < 0x80000000ull) ns.push_back(static_cast<uint32_t>(c + e));
    }
    ns.push_back(0x7fffffffu);
    for (int i = 0; i < 200; ++i) ns.push_back(rnd() & 0x7fffffffu);
    for (uint32_t n : ns) {
      ++checked;
      if (f.div(n) != n / d) {
        if (bad++ < 20) std::printf("bad d=%u n=%u got %u want %u\n", d, n, f.div(n), n / d);
      }
    }
  }
  std::printf("checked %llu\n", static_cast<unsigned long long>(checked));
  return bad != 0;
}
