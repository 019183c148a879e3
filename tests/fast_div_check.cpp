// Host check of make_fast_div (internal.h): for every divisor the kernels can
// be given (block sizes and virtual KV head counts up to 8192), the quotient
// the kernels compute, (mulhi(n, m) + n) >> s with mulhi the high 32 bits of
// the 64-bit product, equals n / d for every n they pass (0 <= n < 2^31):
// all n below 4 d + 64, the neighbours of multiples of d across the range,
// the top of the range and a fixed pseudo-random sample.  Prints the number
// of mismatches.
#include <cstdint>
#include <cstdio>

#include "internal.h"

static uint32_t quotient(uint32_t n, pagedkv::FastDiv f) {
  const uint32_t hi = (uint32_t)(((uint64_t)n * f.m) >> 32);
  return (hi + n) >> f.s;
}

int main() {
  uint64_t checked = 0, failures = 0;
  uint64_t x = 0x9e3779b97f4a7c15ull;   // xorshift64 state
  auto check = [&](uint32_t n, uint32_t d, pagedkv::FastDiv f) {
    ++checked;
    if (quotient(n, f) != n / d) {
      if (failures < 10) std::printf("mismatch: n=%u d=%u\n", n, d);
      ++failures;
    }
  };
  const uint32_t top = 0x7fffffffu;
  for (uint32_t d = 1; d <= 8192; ++d) {
    const pagedkv::FastDiv f = pagedkv::make_fast_div(d);
    for (uint32_t n = 0; n < 4 * d + 64; ++n) check(n, d, f);
    for (uint64_t k = d; k <= top; k = k * 3 / 2 + d) {
      for (int e = -1; e <= 1; ++e) {
        const uint64_t n = (k / d) * d + (uint64_t)(int64_t)e;
        if (n <= top) check((uint32_t)n, d, f);
      }
    }
    for (uint32_t n = top; n > top - 64; --n) check(n, d, f);
    for (int i = 0; i < 512; ++i) {
      x ^= x << 13;
      x ^= x >> 7;
      x ^= x << 17;
      check((uint32_t)(x & top), d, f);
    }
  }
  std::printf("%llu checked, %llu failures\n", (unsigned long long)checked,
              (unsigned long long)failures);
  return failures != 0;
}
