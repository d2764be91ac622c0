// Host check of the piece arithmetic in rank_latent_attention_amd/csrc/pieces.h
// against exact 64-bit integer division.  Built with g++ by test_pieces.py
// (__host__ / __device__ defined away); prints "ok" or the first mismatch.
#include <cstdio>
#include <cstdint>
#include <random>

#define __host__
#define __device__
#include "../rank_latent_attention_amd/csrc/pieces.h"

static long long start_ref(long long i, long long total, int nwg) { return i * total / nwg; }

static int of_ref(long long x, long long total, int nwg) {
  // largest i with start_ref(i) <= x, by bisection on the monotone starts
  int lo = 0, hi = nwg - 1;
  while (lo < hi) {
    const int mid = lo + (hi - lo + 1) / 2;
    if (start_ref(mid, total, nwg) <= x) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

static bool check(long long total, int nwg) {
  for (long long i = 0; i <= nwg; ++i) {
    if (piece_start(i, total, nwg) != start_ref(i, total, nwg)) {
      std::printf("piece_start(%lld, %lld, %d) = %lld, want %lld\n", i, total, nwg, piece_start(i, total, nwg),
                  start_ref(i, total, nwg));
      return false;
    }
  }
  // every piece boundary and its neighbours, plus the two ends
  for (long long i = 0; i <= nwg; ++i) {
    const long long b = start_ref(i, total, nwg);
    for (long long x = b - 1; x <= b + 1; ++x) {
      if (x < 0 || x >= total) continue;
      if (piece_of(x, total, nwg) != of_ref(x, total, nwg)) {
        std::printf("piece_of(%lld, %lld, %d) = %d, want %d\n", x, total, nwg, piece_of(x, total, nwg),
                    of_ref(x, total, nwg));
        return false;
      }
    }
  }
  return true;
}

int main() {
  const long long big = (1LL << 31) - 1;
  const long long totals[] = {1, 2, 3, 7, 127, 128, 129, 1000, 1024, 16641 * 32, 7225 * 64, 8LL << 20, big - 1, big};
  const int nwgs[] = {1, 2, 3, 7, 64, 255, 256, 512, 1000, 1024, 4096, 16384, (1 << 20) - 1};
  for (long long t : totals)
    for (int w : nwgs)
      if (!check(t, w)) return 1;
  std::mt19937_64 rng(12345);
  for (int k = 0; k < 2000; ++k) {
    const long long t = 1 + (long long)(rng() % (unsigned long long)big);
    const int w = 1 + (int)(rng() % ((1u << 20) - 1));
    const int wc = w > 20000 ? 20000 : w;  // keep the exhaustive boundary scan short
    if (!check(t, wc)) return 1;
  }
  // floor_div on its own over the full stated range
  for (int k = 0; k < 200000; ++k) {
    const long long n = (long long)(rng() >> 11);  // < 2^53
    const long long d = 1 + (long long)(rng() % (unsigned long long)big);
    if (floor_div(n, d) != n / d) {
      std::printf("floor_div(%lld, %lld) = %lld, want %lld\n", n, d, floor_div(n, d), n / d);
      return 1;
    }
  }
  std::printf("ok\n");
  return 0;
}
