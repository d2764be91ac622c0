// pieces.h -- cutting a flattened (head, token) range into contiguous
// per-workgroup pieces, shared by the host planner and the kernels.
#pragma once

// floor(n / d) for 0 <= n < 2^53 and d >= 1 without a 64-bit integer
// division (a long software sequence on the GPU).  The correctly rounded
// double quotient r of q = n / d is exact when q is an integer; otherwise
// |r - q| <= q 2^-53 = n / (d 2^53) < 1 / d, which is at most the distance
// from q to the next integer, and rounding is monotonic, so r truncates to
// floor(q).
__host__ __device__ inline long long floor_div(long long n, long long d) {
  return (long long)((double)n / (double)d);
}

// Piece i of `total` tokens cut into `nwg` pieces starts at
// floor(i total / nwg).  Callers keep total < 2^31 and nwg < 2^20, so every
// product is below 2^53.
__host__ __device__ inline long long piece_start(long long i, long long total, int nwg) {
  return floor_div(i * total, nwg);
}

// The piece holding token x (0 <= x < total): the largest i with
// piece_start(i) <= x, i.e. i total < (x + 1) nwg.
__host__ __device__ inline int piece_of(long long x, long long total, int nwg) {
  const long long i = floor_div((x + 1) * nwg - 1, total);
  return (int)(i < nwg ? i : nwg - 1);
}
