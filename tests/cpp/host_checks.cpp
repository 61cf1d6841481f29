// Host-only checks of libmuseattn's pure host pieces, built with g++ and
// AddressSanitizer/UBSan: the invariant-divisor division used for row ->
// token and token -> position maps, and the packed-layout validator.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "fastdiv.hpp"
#include "muse_attn.h"

static int failures = 0;
#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      if (failures++ < 20) std::printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c); \
    }                                                                   \
  } while (0)

int main() {
  std::mt19937_64 rng(7);
  std::vector<uint32_t> divisors;
  for (uint32_t d = 1; d <= 5000; ++d) divisors.push_back(d);
  for (int i = 0; i < 3000; ++i) divisors.push_back(1 + (uint32_t)(rng() % 0x7fffffffu));
  for (uint32_t k = 0; k < 31; ++k) { divisors.push_back(1u << k); divisors.push_back((1u << k) + 1); }
  divisors.push_back(0x7fffffffu);
  for (uint32_t d : divisors) {
    muse::FastDiv f(d);
    auto check = [&](uint32_t n) { CHECK(f.div(n) == n / d); CHECK(f.mod(n) == n % d); };
    for (uint32_t n = 0; n < 2048; ++n) check(n);
    for (int i = 0; i < 200; ++i) check((uint32_t)(rng() % 0x80000000u));
    check(0x7fffffffu);
    check(0x7ffffffeu);
    for (uint32_t q = 1; q < 64; ++q) {            // around multiples of d
      const uint64_t n = (uint64_t)q * d;
      if (n < 0x80000000u) { check((uint32_t)n); check((uint32_t)n - 1); }
      if (n + 1 < 0x80000000u) check((uint32_t)n + 1);
    }
  }
  // packed layout validator
  const int32_t ok[] = {0, 3, 3, 10};
  CHECK(muse_validate_cu_seqlens(ok, 3, 10, 7) == MUSE_OK);
  CHECK(muse_validate_cu_seqlens(ok, 3, 10, 6) == MUSE_ERR_INVALID_ARG);
  CHECK(muse_validate_cu_seqlens(ok, 3, 11, 7) == MUSE_ERR_INVALID_ARG);
  CHECK(muse_validate_cu_seqlens(nullptr, 3, 10, 7) == MUSE_ERR_INVALID_ARG);
  const int32_t neg[] = {0, 5, 4};
  CHECK(muse_validate_cu_seqlens(neg, 2, 4, 5) == MUSE_ERR_INVALID_ARG);
  CHECK(muse_last_error()[0] != 0);
  CHECK(muse_validate_cu_seqlens(ok, 3, 10, 7) == MUSE_OK);
  CHECK(muse_last_error()[0] == 0);
  std::printf("%s (%d failures)\n", failures ? "FAILED" : "OK", failures);
  return failures ? 1 : 0;
}
