// sep_index_compact: exclusive prefix sum of the separator flags and the
// compacted list of separator positions (SepLLM pages: P1 "KV Cache
// Manager", compress_past_win_2_seps keeps the separators of a window in
// order; P3 §3.3, the past window keeps only its separators).
//
// One workgroup of 1024 threads per sequence walks the sequence in chunks of
// 4096 flags (4 per thread). Inside a wave, the per-thread counts (0..4) are
// prefix-summed with three ballots and mbcnt (one per bit of the count);
// the 16 wave totals go through LDS. A running carry links the chunks.
#include "common.hpp"
#include "internal.hpp"

namespace sep {

constexpr int kCompactThreads = 1024;
constexpr int kCompactWaves = kCompactThreads / kWave;

__global__ void __launch_bounds__(kCompactThreads)
    compact_kernel(const uint8_t* __restrict__ is_sep, int S, int32_t* __restrict__ rank,
                   int32_t* __restrict__ sep_pos, int32_t* __restrict__ count) {
  __shared__ int32_t wave_tot[2][kCompactWaves];
  const int b = blockIdx.x;
  const uint8_t* f = is_sep + static_cast<int64_t>(b) * S;
  int32_t* rk = rank + static_cast<int64_t>(b) * (S + 1);
  int32_t* sp = sep_pos + static_cast<int64_t>(b) * S;
  const int tid = threadIdx.x;
  const int wid = tid / kWave;
  int carry = 0;
  int parity = 0;
  for (int base = 0; base < S; base += 4 * kCompactThreads, parity ^= 1) {
    const int j0 = base + 4 * tid;
    int fl[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) fl[e] = (j0 + e < S) ? (f[j0 + e] != 0) : 0;
    const int c = fl[0] + fl[1] + fl[2] + fl[3];
    // wave-level exclusive prefix of c (c < 8 -> three bit planes)
    int pre = 0, tot = 0;
#pragma unroll
    for (int bit = 0; bit < 3; ++bit) {
      const uint64_t m = ballot((c >> bit) & 1);
      pre += static_cast<int>(mbcnt(m)) << bit;
      tot += __popcll(m) << bit;
    }
    if ((tid % kWave) == 0) wave_tot[parity][wid] = tot;
    __syncthreads();
    int before = 0, chunk = 0;
#pragma unroll
    for (int w = 0; w < kCompactWaves; ++w) {
      const int t = wave_tot[parity][w];
      before += (w < wid) ? t : 0;
      chunk += t;
    }
    int r = carry + before + pre;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = j0 + e;
      if (j < S) {
        rk[j] = r;
        if (fl[e]) sp[r] = j;
        r += fl[e];
      }
    }
    carry += chunk;
    // wave_tot is double-buffered by chunk parity, so the next chunk's
    // writes cannot race with this chunk's reads.
  }
  for (int j = carry + tid; j < S; j += kCompactThreads) sp[j] = -1;
  if (tid == 0) {
    rk[S] = carry;
    if (count) count[b] = carry;
  }
}

hipError_t launch_index_compact(const uint8_t* is_sep, int B, int S, int32_t* rank,
                                int32_t* sep_pos, int32_t* count, hipStream_t st) {
  hipLaunchKernelGGL(compact_kernel, dim3(B), dim3(kCompactThreads), 0, st, is_sep, S, rank, sep_pos,
                     count);
  return hipGetLastError();
}

}  // namespace sep
