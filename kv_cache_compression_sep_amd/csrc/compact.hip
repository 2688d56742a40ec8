// sep_index_compact: exclusive prefix sum of the separator flags and the
// compacted list of separator positions (SepLLM pages: P1 "KV Cache
// Manager", compress_past_win_2_seps keeps the separators of a window in
// order; P3 §3.3, the past window keeps only its separators).
//
// One workgroup of 1024 threads per sequence walks the sequence in chunks of
// 4096 flags (4 per thread). Inside a wave, the per-thread counts (0..4) are
// prefix-summed with three ballots and mbcnt (one per bit of the count);
// the 16 wave totals go through LDS. A running carry links the chunks.
// mask_compact_kernel does the same walk from token ids.
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

// sep_mask_compact: the flags of sep_mask_build and the compaction above in
// one launch. The same walk with 8 ids per thread (chunks of 8192 ids, so
// an 8192-token row is one chunk: one barrier): each thread reads its ids
// with two 16-byte loads when the rows allow it, tests them against the
// separator set in LDS, writes the 8 flags, then their ranks with 16-byte
// stores; the per-thread counts (0..8) take four ballot bit planes.
constexpr int kMcPer = 8;
__global__ void __launch_bounds__(kCompactThreads)
    mask_compact_kernel(const int32_t* __restrict__ ids, int S, const int32_t* __restrict__ sep_ids, int n_sep,
                        uint8_t* __restrict__ is_sep, int32_t* __restrict__ rank,
                        int32_t* __restrict__ sep_pos, int32_t* __restrict__ count) {
  __shared__ int32_t wave_tot[2][kCompactWaves];
  __shared__ int32_t set[SEP_MAX_SEP_IDS];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int wid = tid / kWave;
  const int32_t* id = ids + static_cast<int64_t>(b) * S;
  uint8_t* f = is_sep + static_cast<int64_t>(b) * S;
  int32_t* rk = rank + static_cast<int64_t>(b) * (S + 1);
  int32_t* sp = sep_pos + static_cast<int64_t>(b) * S;
  const bool vec = (S % 4) == 0;                  // rows of whole 16-byte groups (ids) and 4-byte flag groups
  const bool rvec = vec && ((static_cast<int64_t>(b) * (S + 1)) % 4) == 0;   // 16-byte aligned rank row
  constexpr int kChunk = kMcPer * kCompactThreads;
  // the ids of each chunk are loaded one chunk ahead (the first ones while
  // the separator set is staged), so a load's latency overlaps the previous
  // chunk's work
  auto load4 = [&](int j0) -> int4 {
    return (vec && j0 + 4 <= S) ? *reinterpret_cast<const int4*>(id + j0) : make_int4(0, 0, 0, 0);
  };
  int4 nx0 = load4(kMcPer * tid), nx1 = load4(kMcPer * tid + 4);
  for (int i = tid; i < n_sep; i += kCompactThreads) set[i] = sep_ids[i];
  __syncthreads();
  int carry = 0;
  int parity = 0;
  for (int base = 0; base < S; base += kChunk, parity ^= 1) {
    const int j0 = base + kMcPer * tid;
    const int4 v0 = nx0, v1 = nx1;
    if (base + kChunk < S) {
      nx0 = load4(j0 + kChunk);
      nx1 = load4(j0 + kChunk + 4);
    }
    int fl[kMcPer];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int4 v = h ? v1 : v0;
      const int jh = j0 + 4 * h;
      if (vec && jh + 4 <= S) {
        fl[4 * h + 0] = in_set(v.x, set, n_sep);
        fl[4 * h + 1] = in_set(v.y, set, n_sep);
        fl[4 * h + 2] = in_set(v.z, set, n_sep);
        fl[4 * h + 3] = in_set(v.w, set, n_sep);
        *reinterpret_cast<uchar4*>(f + jh) =
            make_uchar4(fl[4 * h], fl[4 * h + 1], fl[4 * h + 2], fl[4 * h + 3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = jh + e;
          fl[4 * h + e] = (j < S) ? in_set(id[j], set, n_sep) : 0;
          if (j < S) f[j] = static_cast<uint8_t>(fl[4 * h + e]);
        }
      }
    }
    int c = 0;
#pragma unroll
    for (int e = 0; e < kMcPer; ++e) c += fl[e];
    int pre = 0, tot = 0;
#pragma unroll
    for (int bit = 0; bit < 4; ++bit) {              // c <= 8: four bit planes
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
    int rr[kMcPer];
    rr[0] = carry + before + pre;
#pragma unroll
    for (int e = 1; e < kMcPer; ++e) rr[e] = rr[e - 1] + fl[e - 1];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int jh = j0 + 4 * h;
      if (rvec && jh + 4 <= S) {
        *reinterpret_cast<int4*>(rk + jh) = make_int4(rr[4 * h], rr[4 * h + 1], rr[4 * h + 2], rr[4 * h + 3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (jh + e < S) rk[jh + e] = rr[4 * h + e];
      }
    }
#pragma unroll
    for (int e = 0; e < kMcPer; ++e)
      if (j0 + e < S && fl[e]) sp[rr[e]] = j0 + e;
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

hipError_t launch_mask_compact(const int32_t* ids, int B, int S, const int32_t* sep_ids, int n_sep,
                               uint8_t* is_sep, int32_t* rank, int32_t* sep_pos, int32_t* count,
                               hipStream_t st) {
  hipLaunchKernelGGL(mask_compact_kernel, dim3(B), dim3(kCompactThreads), 0, st, ids, S, sep_ids, n_sep, is_sep,
                     rank, sep_pos, count);
  return hipGetLastError();
}

hipError_t launch_index_compact(const uint8_t* is_sep, int B, int S, int32_t* rank,
                                int32_t* sep_pos, int32_t* count, hipStream_t st) {
  hipLaunchKernelGGL(compact_kernel, dim3(B), dim3(kCompactThreads), 0, st, is_sep, S, rank, sep_pos,
                     count);
  return hipGetLastError();
}

}  // namespace sep
