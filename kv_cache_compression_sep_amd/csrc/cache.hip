// sep_cache_update / sep_cache_reset: the four-block streaming KV cache.
//
// Blocks and eviction (SepLLM pages: P2 §1.3; P3 §3.3 table; P1
// "KV Cache Manager"): initial tokens are fixed; the local window overflows
// into the past window; when the past window is full its separators are
// kept and the rest dropped; the separator cache holds at most s entries and
// drops its oldest. A token at position t >= a joins the recent ring R
// (= past ++ local); when the policy's trigger fires, R minus its last w
// entries is compressed (separators to the separator ring, the rest
// dropped; without SEP_ACCUMULATION the ring is emptied first).
//   fixed caps: R would hold p + w + 1 entries. The timing depends only on
//     t: after t tokens K(t) = max(0, floor((t - a - w) / (p + 1))) (t > a)
//     compressions of p + 1 entries each have happened.
//   dynamic (P1's trigger): the whole cache would hold more than
//     c = a + s + p + w entries. Pushing position x makes it hold
//     a + |S| + (x + 1 - cend) entries, so the next compression is at
//     x = cend + c - a - |S|; its timing depends on |S|, i.e. on content.
//
// A call that appends T tokens is planned once per sequence: the positions
// compressed by this call are [cend0, cend1). Their separators that can
// survive (all of them, or without accumulation those of the call's last
// compression, [wlo, cend1)) are numbered k = 0 .. nL-1 in position order,
// and only the last min(nL, s) survive, the k-th landing in ring slot
// (sep_head + k) mod s. A block-wide count gives nL; a backward walk with
// wavefront ballots finds the survivors. Under the dynamic trigger one
// thread steps through the call's compressions, counting separators in a
// bitmap of [cend0, t1) built block-wide in LDS. Surviving rows are copied
// into the separator ring before any newly arriving token overwrites a
// recent-ring slot. A call with T > 1 runs two kernels: one block per
// sequence plans and writes pos / tok / state, then one block per (head,
// sequence) copies K/V rows, reading the plan back from pos[] of the
// separator ring. T == 1 runs one fused block per sequence.
#include "common.hpp"
#include "decode.hpp"
#include "internal.hpp"

#include <type_traits>

namespace sep {

constexpr int kUpdThreads = 512;
constexpr int kUpdWaves = kUpdThreads / kWave;
// positions a dynamic-trigger plan covers at most (its bitmap): the ring
// (<= SEP_MAX_DYN_RING) plus the new tokens of one chunk of a call
constexpr int kSpan = 2 * SEP_MAX_DYN_RING;
constexpr int kSpanWords = kSpan / 32;

struct CacheArgs {
  char* k;
  char* v;
  int32_t* pos;
  int32_t* tok;
  int64_t* state;
  const char* k_new;         // rows of this call's first token
  const char* v_new;
  const int32_t* ids_new;
  const int32_t* sep_ids;
  int n_sep;
  int a, s, p, w;
  int rw;                    // recent-ring size
  int c;                     // slots per sequence
  int Hkv, D, esize;
  int T;                     // tokens of this call
  int tstride;               // tokens per (sequence, head) row of k_new / ids_new
  int dynamic, accumulate;
  int csplit;                // data_kernel: workgroups per (sequence, kv head), each a column range
};

struct PlanHead {
  int64_t t0, t1, cend0, cend1;
  int64_t wlo;       // separators in [wlo, cend1) can survive
  int64_t nL;        // separators in [wlo, cend1)
  int head0, cnt0;
  int reset;         // the separator ring is emptied first (no accumulation)
};

__device__ __forceinline__ int64_t n_compact(int64_t t, int a, int p, int w) {
  const int64_t m = t - a;
  if (m <= 0) return 0;
  const int64_t r = (m - w) / (p + 1);
  return (m - w) < 0 ? 0 : r;
}

// Ring slot of position x >= a. Positions are stored as int32, so x - a
// fits 32 bits and the remainder is taken in 32-bit arithmetic.
__device__ __forceinline__ int slot_r(int64_t x, int a, int s, int rw) {
  return a + s + static_cast<int>(static_cast<uint32_t>(x - a) % static_cast<uint32_t>(rw));
}

// i + d reduced into [0, m) for 0 <= i < m, 0 <= d < m
__device__ __forceinline__ int wrap_add(int i, int d, int m) {
  const int r = i + d;
  return r >= m ? r - m : r;
}

// Loads and stores through global-address-space pointers, so that they wait
// on the vector-memory counter only (generic pointers would also hold up
// waits for LDS results).
template <class T>
__device__ __forceinline__ T ld_global(const T* p) {
  return *(const __attribute__((address_space(1))) T*)(p);
}
template <class T>
__device__ __forceinline__ T ld_global_nt(const T* p) {
  return __builtin_nontemporal_load((const __attribute__((address_space(1))) T*)(p));
}
template <class T>
__device__ __forceinline__ void st_global(T* p, T v) {
  *(__attribute__((address_space(1))) T*)(p) = v;
}

// Separator-set membership, exact: a table of 2^kHashBits ids in LDS. Every
// slot first holds the set's first id, then each id of the set is written at
// slot h(id); id is in the set iff tab[h(id)] == id (a slot holds either an id
// of the set that hashes there, or the first id, which hashes elsewhere or is
// id itself). Two ids of the set that share a slot would lose one, so the
// block checks every id after the build; if one is missing (or the set is
// empty) the block uses SetList instead.
constexpr int kHashBits = 12;
constexpr int kHashSize = 1 << kHashBits;

__device__ __forceinline__ int sep_hash(int32_t id) {
  const uint32_t u = static_cast<uint32_t>(id);
  return static_cast<int>((u ^ (u >> kHashBits) ^ (u >> (2 * kHashBits))) & (kHashSize - 1));
}

struct SetHash {
  const int32_t* tab;
  const int32_t* set;
  int n;
  bool exact;   // uniform
  // lds_tab: kHashSize ints; lds_set: n ints. Contains barriers.
  __device__ void load(const int32_t* sep_ids, int n_, int32_t* lds_tab, int32_t* lds_set) {
    const int tid = threadIdx.x;
    n = n_;
    tab = lds_tab;
    set = lds_set;
    const int32_t first = n_ > 0 ? sep_ids[0] : 0;
    for (int q = tid; q < n_; q += blockDim.x) lds_set[q] = sep_ids[q];
    for (int e = tid; e < kHashSize; e += blockDim.x) lds_tab[e] = first;
    __syncthreads();
    for (int q = tid; q < n_; q += blockDim.x) lds_tab[sep_hash(lds_set[q])] = lds_set[q];
    __syncthreads();
    bool lost = false;
    for (int q = tid; q < n_; q += blockDim.x) lost |= lds_tab[sep_hash(lds_set[q])] != lds_set[q];
    exact = !__syncthreads_or(lost) && n_ > 0;
  }
  // valid when `exact`
  __device__ __forceinline__ bool operator()(int32_t id) const { return tab[sep_hash(id)] == id; }
};

// The set compared entry by entry: for calls that test only a few ids.
struct SetList {
  const int32_t* set;
  int n;
  __device__ void load(const int32_t* sep_ids, int n_, int32_t*, int32_t* lds_set) {
    for (int q = threadIdx.x; q < n_; q += blockDim.x) lds_set[q] = sep_ids[q];
    set = lds_set;
    n = n_;
    __syncthreads();
  }
  __device__ __forceinline__ bool operator()(int32_t id) const { return in_set(id, set, n); }
};

// Separator bitmap of positions [x0, x0 + L) (L <= kSpan): bit o of word
// o / 32 is set iff position x0 + o is a separator; pre[i] counts the set
// bits of words 0 .. i-1. Built by the whole block; ends with a barrier.
struct SepBits {
  uint32_t* bits;
  int32_t* pre;
  // separators at offsets [0, o)
  __device__ __forceinline__ int rank(int o) const {
    const int wi = o >> 5, r = o & 31;
    return pre[wi] + (r ? __popc(bits[wi] & ((1u << r) - 1u)) : 0);
  }
};

template <class Set, class IdAt>
__device__ void build_bits(SepBits& B, const Set& S, IdAt id_at, int64_t x0, int L, int32_t* wave_tot) {
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int nwords = (L + 31) / 32;
  for (int base = 0; base < L; base += kWave * kUpdWaves) {
    const int o = base + wv * kWave + lane;
    const bool f = o < L && S(id_at(x0 + o));
    const uint64_t m = ballot(f);
    const int w0 = (base + wv * kWave) / 32;
    if (lane == 0 && w0 < nwords) B.bits[w0] = static_cast<uint32_t>(m);
    if (lane == 1 && w0 + 1 < nwords) B.bits[w0 + 1] = static_cast<uint32_t>(m >> 32);
  }
  __syncthreads();
  // exclusive prefix of the word popcounts, kSpanWords / kUpdThreads words per thread
  constexpr int PER = kSpanWords / kUpdThreads;
  int c[PER], sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int wi = tid * PER + i;
    c[i] = wi < nwords ? __popc(B.bits[wi]) : 0;
    sum += c[i];
  }
  int incl = sum;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(incl, off, kWave);
    incl += (lane >= off) ? y : 0;
  }
  if (lane == kWave - 1) wave_tot[wv] = incl;
  __syncthreads();
  int before = incl - sum;
  for (int i = 0; i < wv; ++i) before += wave_tot[i];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int wi = tid * PER + i;
    if (wi <= nwords) B.pre[wi] = before;
    before += c[i];
  }
  if (tid == kUpdThreads - 1 && nwords == kSpanWords) B.pre[kSpanWords] = before;   // the total
  __syncthreads();
}

// Plan one sequence's call. Fills `ph` and the survivor list: entry (k mod s)
// of lpos/lid holds the position and id of the k-th separator of
// [wlo, cend1) for the last min(nL, s) values of k. Reads state and tok[] of
// the recent ring; nothing is written to global memory. `early(ph)` runs
// once `ph` is known, before the plan's own loads, so that a caller can put
// its own independent loads in flight. Ends with a barrier. The caller has
// loaded `S`; `sb` (bitmap storage) is used under the dynamic trigger only.
//
// nL is a block-wide count over [wlo, cend1): the positions still in the
// ring one per thread, the new ones from ids_new in 16-byte loads,
// kCountUnroll of them in flight per thread. The survivors are then found by
// walking that range backwards in chunks of kWalkPer * kUpdThreads positions
// (kWalkPer consecutive positions per thread) until min(nL, s) separators
// are seen; the first chunk is loaded together with the count.
constexpr int kCountUnroll = 16;
constexpr int kWalkPer = 8;

template <bool DYN, class Set, class Early>
__device__ void plan(const CacheArgs& A, int b, const Set& S, PlanHead& ph, int32_t* lpos, int32_t* lid,
                     int32_t* wave_tot, SepBits sb, Early early) {
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wv = tid / kWave;
  const int rw = A.rw;
  if (tid == 0) {
    const int64_t* st = A.state + kStateWords * static_cast<int64_t>(b);
    ph.t0 = st[0];
    ph.cend0 = A.a + st[1];
    ph.head0 = static_cast<int>(st[2]);
    ph.cnt0 = static_cast<int>(st[3]);
    ph.t1 = ph.t0 + A.T;
    if (!DYN) {
      ph.cend1 = A.a + n_compact(ph.t1, A.a, A.p, A.w) * (A.p + 1);
      // without accumulation only the last compression's separators count
      const bool comp = ph.cend1 > ph.cend0;
      ph.wlo = (A.accumulate || !comp) ? ph.cend0 : ph.cend1 - (A.p + 1);
      ph.reset = (!A.accumulate && comp) ? 1 : 0;
    }
  }
  __syncthreads();
  const int64_t t0 = ph.t0, cend0 = ph.cend0;
  const int32_t* tokb = A.tok + static_cast<int64_t>(b) * A.c;
  const int32_t* idsb = A.ids_new + static_cast<int64_t>(b) * A.tstride;
  // id of position x (cend0 <= x < t1): the ring's tok[] before this call,
  // the new ids from t0 on
  auto id_at = [&](int64_t x) -> int32_t {
    const int32_t* src = (x < t0) ? tokb + slot_r(x, A.a, A.s, rw) : idsb + (x - t0);
    return ld_global(src);
  };
  if (DYN) {
    // the call's compressions, one after the other (thread 0), with the
    // separators of [cend0, t1) in a bitmap
    const int L = static_cast<int>(ph.t1 - cend0 > 0 ? ph.t1 - cend0 : 0);
    build_bits(sb, S, id_at, cend0, L, wave_tot);
    if (tid == 0) {
      const int c = A.a + A.s + A.p + A.w;
      int64_t cend = cend0, last_lo = -1;
      int cnt = ph.cnt0;
      const int64_t t1 = ph.t1;
      for (;;) {
        if (A.accumulate && cnt == A.s) {
          // S stays full from here: a compression every p + 1 tokens
          const int64_t x = cend + A.p + A.w;
          if (x < t1) {
            const int64_t k = (t1 - 1 - x) / (A.p + 1) + 1;
            cend += k * (A.p + 1);
            last_lo = cend - (A.p + 1);
          }
          break;
        }
        const int64_t x = cend + (c - A.a - cnt);
        if (x >= t1) break;
        const int64_t nc = x + 1 - A.w;
        const int n = sb.rank(static_cast<int>(nc - cend0)) - sb.rank(static_cast<int>(cend - cend0));
        const int acc = A.accumulate ? cnt + n : n;
        cnt = acc < A.s ? acc : A.s;
        last_lo = cend;
        cend = nc;
      }
      ph.cend1 = cend;
      const bool comp = cend > cend0;
      ph.wlo = (A.accumulate || !comp) ? cend0 : last_lo;
      ph.reset = (!A.accumulate && comp) ? 1 : 0;
    }
    __syncthreads();
  }
  early(ph);
  const int64_t cend1 = ph.cend1, wlo = ph.wlo;

  // first chunk of the walk, loaded now
  int32_t wid[kWalkPer];
  const bool walk = (A.s > 0) && (cend1 > wlo);
  if (walk) {
#pragma unroll
    for (int u = 0; u < kWalkPer; ++u) {
      const int64_t x = cend1 - kWalkPer * kUpdThreads + kWalkPer * tid + u;
      wid[u] = id_at(x >= wlo ? x : wlo);
    }
  }

  // (1) nL = number of separators in [wlo, cend1)
  int cnt = 0;
  const int64_t xr_end = cend1 < t0 ? cend1 : t0;
  for (int64_t x = wlo + tid; x < xr_end; x += kUpdThreads) cnt += S(ld_global(tokb + slot_r(x, A.a, A.s, rw))) ? 1 : 0;
  const int64_t xn_beg = wlo > t0 ? wlo : t0;
  const int n_new = static_cast<int>(cend1 > xn_beg ? cend1 - xn_beg : 0);
  const int32_t* nb = idsb + (xn_beg - t0);
  // nb[0 .. n_head) up to a 16-byte boundary, then whole 16-byte groups, then the rest
  int n_head = static_cast<int>((16 - (reinterpret_cast<uintptr_t>(nb) & 15)) & 15) / 4;
  n_head = n_head < n_new ? n_head : n_new;
  const int n_vec = (n_new - n_head) / 4;
  const int n_tail0 = n_head + 4 * n_vec;
  if (tid < n_head) cnt += S(ld_global(nb + tid)) ? 1 : 0;
  if (tid < n_new - n_tail0) cnt += S(ld_global(nb + n_tail0 + tid)) ? 1 : 0;
  const u32x4* nv = reinterpret_cast<const u32x4*>(nb + n_head);
  for (int i0 = tid; i0 < n_vec; i0 += kCountUnroll * kUpdThreads) {
    u32x4 v[kCountUnroll];
#pragma unroll
    for (int u = 0; u < kCountUnroll; ++u) {
      const int i = i0 + u * kUpdThreads;
      v[u] = ld_global(nv + (i < n_vec ? i : 0));
    }
#pragma unroll
    for (int u = 0; u < kCountUnroll; ++u) {
      const int four = (S(static_cast<int32_t>(v[u].x)) ? 1 : 0) + (S(static_cast<int32_t>(v[u].y)) ? 1 : 0) +
                       (S(static_cast<int32_t>(v[u].z)) ? 1 : 0) + (S(static_cast<int32_t>(v[u].w)) ? 1 : 0);
      cnt += (i0 + u * kUpdThreads < n_vec) ? four : 0;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, kWave);
  if (lane == 0) wave_tot[wv] = cnt;
  __syncthreads();
  int64_t nL = 0;
#pragma unroll
  for (int i = 0; i < kUpdWaves; ++i) nL += wave_tot[i];
  const int64_t nsurv = (A.s > 0) ? (nL < A.s ? nL : A.s) : 0;
  __syncthreads();

  // (2) survivors: walk [wlo, cend1) backwards; `after` counts the
  //     separators at higher positions than the current chunk. Thread tid
  //     owns positions lo + kWalkPer*tid + u, u = 0 .. kWalkPer-1.
  int64_t after = 0;
  // entry of the last separator: (nL - 1) mod s; from_end < s steps back from it
  const int li_last = (A.s > 0 && nL > 0) ? static_cast<int>((nL - 1) % A.s) : 0;
  for (int64_t hi = cend1; hi > wlo && after < nsurv; hi -= kWalkPer * kUpdThreads) {
    const int64_t lo = hi - kWalkPer * kUpdThreads;
    if (hi != cend1) {
#pragma unroll
      for (int u = 0; u < kWalkPer; ++u) {
        const int64_t x = lo + kWalkPer * tid + u;
        wid[u] = id_at(x >= wlo ? x : wlo);
      }
    }
    uint32_t fl = 0;   // bit u: position lo + kWalkPer*tid + u is a separator
    int above = 0;     // separators of this wave at lanes above this one
    int wtot = 0;
#pragma unroll
    for (int u = 0; u < kWalkPer; ++u) {
      const bool f = lo + kWalkPer * tid + u >= wlo && S(wid[u]);
      const uint64_t m = ballot(f);
      fl |= f ? (1u << u) : 0u;
      above += (lane == 63) ? 0 : __popcll(m >> (lane + 1));
      wtot += __popcll(m);
    }
    if (lane == 0) wave_tot[kUpdWaves + wv] = wtot;
    __syncthreads();
    int later = 0, chunk = 0;
#pragma unroll
    for (int i = 0; i < kUpdWaves; ++i) {
      const int tt = wave_tot[kUpdWaves + i];
      later += (i > wv) ? tt : 0;
      chunk += tt;
    }
    if (fl) {
      int within = 0;   // this thread's separators at higher u
#pragma unroll
      for (int u = kWalkPer - 1; u >= 0; --u) {
        if ((fl >> u) & 1) {
          const int64_t from_end = after + later + above + within;   // 0 for the last separator
          if (from_end < nsurv) {
            const int back = li_last - static_cast<int>(from_end);
            const int li = back < 0 ? back + A.s : back;
            lpos[li] = static_cast<int32_t>(lo + kWalkPer * tid + u);
            lid[li] = wid[u];
          }
          ++within;
        }
      }
    }
    after += chunk;
    __syncthreads();
  }
  if (tid == 0) ph.nL = nL;
  __syncthreads();
}

// Copy `nrows` rows (head range [g0, g1), K and V) in 16-byte columns. A row
// is W = (g1 - g0) * 2 * row_bytes / 16 columns; thread t keeps one column
// and takes every R-th row (R = threads / W), so the row-to-address functor
// runs once per 16 bytes but the column split is done once. kCopyUnroll
// loads are in flight per thread before their stores. The functor maps
// (row, head, k-or-v) to (src, dst) row pointers; no destination of one call
// is a source of the same call. With parts > 1 the call copies only column
// range `part` of `parts` equal ones: workgroups that split a head's columns
// between them never touch the same bytes.
constexpr int kCopyUnroll = 8;

template <class RowFn>
__device__ __forceinline__ void copy_rows(int nrows, int g0, int g1, int row_bytes, RowFn fn, int part = 0,
                                          int parts = 1) {
  const int cpr = row_bytes / 16;
  const int Wall = (g1 - g0) * 2 * cpr;
  const int clo = Wall * part / parts;
  const int chi = Wall * (part + 1) / parts;
  const int W = chi - clo;
  const int t = threadIdx.x;
  if (W <= 0) return;
  const int R = W <= kUpdThreads ? kUpdThreads / W : 1;
  const int rbeg = W <= kUpdThreads ? t / W : 0;
  if (rbeg >= R) return;
  for (int col = clo + (W <= kUpdThreads ? t % W : t); col < chi; col += kUpdThreads) {
    const int chunk = col % cpr;
    const int kvg = col / cpr;
    const int kv = kvg & 1;
    const int g = g0 + (kvg >> 1);
    for (int r0 = rbeg; r0 < nrows; r0 += kCopyUnroll * R) {
      u32x4 val[kCopyUnroll];
      char* dst[kCopyUnroll];
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u) {
        const int r = r0 + u * R;
        dst[u] = nullptr;
        if (r < nrows) {
          const char* src;
          fn(r, g, kv, &src, &dst[u]);
          dst[u] += 16 * chunk;
          val[u] = ld_global_nt(reinterpret_cast<const u32x4*>(src + 16 * chunk));
        }
      }
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u)
        if (r0 + u * R < nrows) st_global(reinterpret_cast<u32x4*>(dst[u]), val[u]);
    }
  }
}

// K/V rows of new tokens that stay, for heads [g0, g1): initial slots, and
// recent-ring slots for positions >= cend1 (those below cend1 were compacted
// away, and the ring holds at most rw positions).
__device__ __forceinline__ void copy_new_rows(const CacheArgs& A, int b, int g0, int g1, int64_t t0,
                                              int64_t t1, int64_t cend1, int part = 0, int parts = 1) {
  const int rw = A.rw;
  const int row_bytes = A.D * A.esize;
  const int64_t cache_seq = static_cast<int64_t>(b) * A.Hkv;
  const int64_t keep_lo = t1 - rw > t0 ? t1 - rw : t0;
  const int64_t r_lo = (cend1 > keep_lo) ? cend1 : keep_lo;
  const int64_t r_start = r_lo > A.a ? r_lo : A.a;
  const int64_t init_end = t1 < A.a ? t1 : A.a;
  const int n_init_new = static_cast<int>(init_end > t0 ? init_end - t0 : 0);
  const int n_r_new = static_cast<int>(t1 > r_start ? t1 - r_start : 0);
  copy_rows(n_init_new + n_r_new, g0, g1, row_bytes, [&](int r, int g, int kv, const char** src, char** dst) {
    const int64_t y = (r < n_init_new) ? t0 + r : r_start + (r - n_init_new);
    const int dslot = (y < A.a) ? static_cast<int>(y) : slot_r(y, A.a, A.s, rw);
    const char* base_new = kv ? A.v_new : A.k_new;
    char* base_c = kv ? A.v : A.k;
    *src = base_new + ((cache_seq + g) * A.tstride + (y - t0)) * row_bytes;
    *dst = base_c + ((cache_seq + g) * A.c + dslot) * row_bytes;
  }, part, parts);
}

enum { UPD_META = 1, UPD_FUSED = 2 };

// UPD_META : grid (1, B), plan + pos / tok / state; K/V untouched.
// UPD_FUSED: grid (1, B), everything (used for T == 1).
template <int MODE, bool DYN, class Set>
__device__ void update_block(const CacheArgs& A, const Set& S, PlanHead& ph, int32_t* lpos, int32_t* lid,
                             int32_t* wave_tot, SepBits sb) {
  const int tid = threadIdx.x;
  const int b = blockIdx.y;
  const int rw = A.rw;
  const int32_t* idsb = A.ids_new + static_cast<int64_t>(b) * A.tstride;
  // New tokens that stay, as one list: i < n_init are initial positions
  // t0 + i, the rest the recent-ring tail from r_start on (positions below
  // cend1 are compacted by this call, and the ring holds at most rw). Their
  // ids are loaded before the plan's count; the stores wait for it.
  constexpr int kKeepPre = 2;
  int64_t r_start = 0;
  int n_init = 0, n_keep = 0;
  int32_t kid[kKeepPre];
  auto keep_pos = [&](int i) -> int64_t { return (i < n_init) ? ph.t0 + i : r_start + (i - n_init); };
  plan<DYN>(A, b, S, ph, lpos, lid, wave_tot, sb, [&](const PlanHead& h) {
    const int64_t keep_lo = h.t1 - rw > h.t0 ? h.t1 - rw : h.t0;
    const int64_t r_lo = (h.cend1 > keep_lo) ? h.cend1 : keep_lo;
    r_start = r_lo > A.a ? r_lo : A.a;
    const int64_t init_end = h.t1 < A.a ? h.t1 : A.a;
    n_init = static_cast<int>(init_end > h.t0 ? init_end - h.t0 : 0);
    n_keep = n_init + static_cast<int>(h.t1 > r_start ? h.t1 - r_start : 0);
#pragma unroll
    for (int u = 0; u < kKeepPre; ++u) {
      const int i = tid + u * kUpdThreads;
      kid[u] = (i < n_keep) ? ld_global(idsb + (keep_pos(i) - h.t0)) : 0;
    }
  });

  const int64_t t0 = ph.t0, t1 = ph.t1, cend1 = ph.cend1, nL = ph.nL;
  const int nsurv = static_cast<int>(nL < A.s ? nL : A.s);
  const int64_t kfirst = nL - nsurv;
  // survivor r (k = kfirst + r): list entry (li0 + r) mod s, ring slot
  // a + (d0 + r) mod s
  const int li0 = A.s > 0 ? static_cast<int>(kfirst % A.s) : 0;
  // an emptied ring restarts at its first slot, so that its layout depends
  // on the last compression only (as after single-token calls)
  const int d0 = A.s > 0 ? (ph.reset ? 0 : static_cast<int>((ph.head0 + kfirst) % A.s)) : 0;
  const int row_bytes = A.D * A.esize;
  const int64_t cache_seq = static_cast<int64_t>(b) * A.Hkv;

  if (MODE == UPD_FUSED) {
    // (1) surviving separators -> separator ring, before any new token
    //     overwrites a recent-ring slot they may come from
    copy_rows(nsurv, 0, A.Hkv, row_bytes, [&](int r, int g, int kv, const char** src, char** dst) {
      const int64_t x = lpos[wrap_add(li0, r, A.s)];
      const int dslot = A.a + wrap_add(d0, r, A.s);
      const char* base_new = kv ? A.v_new : A.k_new;
      char* base_c = kv ? A.v : A.k;
      const int64_t crow = (cache_seq + g) * A.c;
      if (x < t0) {
        *src = base_c + (crow + slot_r(x, A.a, A.s, rw)) * row_bytes;
      } else {
        *src = base_new + ((cache_seq + g) * A.tstride + (x - t0)) * row_bytes;
      }
      *dst = base_c + (crow + dslot) * row_bytes;
    });
    __syncthreads();
    // (2) new tokens that stay
    copy_new_rows(A, b, 0, A.Hkv, t0, t1, cend1);
  }

  int32_t* posb = A.pos + static_cast<int64_t>(b) * A.c;
  int32_t* tokb = A.tok + static_cast<int64_t>(b) * A.c;
  // without accumulation a compression empties the separator ring first
  if (ph.reset) {
    for (int j = tid; j < A.s; j += kUpdThreads) {
      st_global(posb + A.a + j, -1);
      st_global(tokb + A.a + j, -1);
    }
    __syncthreads();
  }
  // survivors -> separator-ring metadata (ids were captured by the plan)
  for (int r = tid; r < nsurv; r += kUpdThreads) {
    const int li = wrap_add(li0, r, A.s);
    const int dslot = A.a + wrap_add(d0, r, A.s);
    st_global(posb + dslot, lpos[li]);
    st_global(tokb + dslot, lid[li]);
  }
  // recent-ring slots of positions compacted by this call become empty
  const int64_t old_lo = ph.cend0;
  const int64_t old_hi = cend1 < t0 ? cend1 : t0;
  for (int64_t x = old_lo + tid; x < old_hi; x += kUpdThreads) {
    const int sl = slot_r(x, A.a, A.s, rw);
    st_global(posb + sl, -1);
    st_global(tokb + sl, -1);
  }
  __syncthreads();
  // new tokens that stay (a cleared slot may be one of theirs)
  auto put = [&](int i, int32_t id) {
    const int64_t y = keep_pos(i);
    const int sl = (y < A.a) ? static_cast<int>(y) : slot_r(y, A.a, A.s, rw);
    st_global(posb + sl, static_cast<int32_t>(y));
    st_global(tokb + sl, id);
  };
#pragma unroll
  for (int u = 0; u < kKeepPre; ++u)
    if (tid + u * kUpdThreads < n_keep) put(tid + u * kUpdThreads, kid[u]);
  for (int i = tid + kKeepPre * kUpdThreads; i < n_keep; i += kUpdThreads) put(i, ld_global(idsb + (keep_pos(i) - t0)));
  if (tid == 0) {
    int64_t* st = A.state + kStateWords * static_cast<int64_t>(b);
    st[0] = t1;
    st[1] = cend1 - A.a;
    st[4] = ph.cend0 - A.a;
    if (A.s > 0) {
      st[2] = ph.reset ? nsurv % A.s : (ph.head0 + nL) % A.s;
      const int64_t cnt = (ph.reset ? 0 : ph.cnt0) + nL;
      st[3] = cnt < A.s ? cnt : A.s;
    }
  }
}

template <int MODE, bool DYN>
__device__ __forceinline__ void update_body(const CacheArgs& A) {
  extern __shared__ int32_t dyn[];
  __shared__ int32_t set_lds[SEP_MAX_SEP_IDS_];
  __shared__ int32_t set_tab[MODE == UPD_FUSED ? 1 : kHashSize];
  __shared__ int32_t wave_tot[2 * kUpdWaves];
  __shared__ uint32_t sb_bits[DYN ? kSpanWords : 1];
  __shared__ int32_t sb_pre[DYN ? kSpanWords + 1 : 1];
  __shared__ PlanHead ph;
  const int smax = A.s > 0 ? A.s : 1;
  int32_t* lpos = dyn;
  int32_t* lid = dyn + smax;
  SepBits sb{sb_bits, sb_pre};
  SetList L;
  if (MODE == UPD_FUSED) {
    // T == 1. The new K/V row, its id and the state are loaded together;
    // when no compression is due the token only takes its slot: the row, one
    // pos/tok entry and the state words, with no barrier. Otherwise the
    // general block plans the compression (few ids, no table).
    const int tid = threadIdx.x;
    const int b = blockIdx.y;
    const int rw = A.rw;
    const int row_bytes = A.D * A.esize;
    const int cpr = row_bytes / 16;
    const int W = A.Hkv * 2 * cpr;
    const int64_t* st = A.state + kStateWords * static_cast<int64_t>(b);
    const int64_t t0 = ld_global(st), ncomp = ld_global(st + 1), cnt0 = ld_global(st + 3);
    const int32_t id = ld_global(A.ids_new + static_cast<int64_t>(b) * A.tstride);
    u32x4 val[2];
    int col[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      col[u] = tid + u * kUpdThreads;
      if (col[u] < W) {
        const int kv = (col[u] / cpr) & 1;
        const int g = col[u] / (2 * cpr);
        const char* src = (kv ? A.v_new : A.k_new) + (static_cast<int64_t>(b) * A.Hkv + g) * A.tstride * row_bytes;
        val[u] = ld_global_nt(reinterpret_cast<const u32x4*>(src + 16 * (col[u] % cpr)));
      }
    }
    // R after the push holds t0 + 1 - cend0 entries. Without a separator
    // ring (StreamingLLM: s = p = 0, ring of w slots) a compression drops
    // R's oldest r_after - w entries and keeps nothing; the one it drops in
    // a single-token step is the position t0 - w, whose slot the new token
    // takes, so that compression is a slot write like the others.
    const int64_t r_after = t0 + 1 - (A.a + ncomp);
    const int64_t r_cap = DYN ? (A.s + A.p + A.w - cnt0) : (A.p + A.w);
    if (t0 < A.a || r_after <= r_cap || A.s == 0) {
      // R holds at most w entries before the push when s == 0, so at most one
      // is dropped here
      const int64_t dropped = (A.s == 0 && t0 >= A.a && r_after > A.w) ? r_after - A.w : 0;
      const int slot = t0 < A.a ? static_cast<int>(t0) : slot_r(t0, A.a, A.s, rw);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (col[u] < W) {
          const int kv = (col[u] / cpr) & 1;
          const int g = col[u] / (2 * cpr);
          char* dst = (kv ? A.v : A.k) + ((static_cast<int64_t>(b) * A.Hkv + g) * A.c + slot) * row_bytes;
          st_global(reinterpret_cast<u32x4*>(dst + 16 * (col[u] % cpr)), val[u]);
        }
      }
      for (int c0 = 2 * kUpdThreads + tid; c0 < W; c0 += kUpdThreads) {
        const int kv = (c0 / cpr) & 1;
        const int g = c0 / (2 * cpr);
        const int64_t hrow = static_cast<int64_t>(b) * A.Hkv + g;
        const u32x4 v = ld_global_nt(reinterpret_cast<const u32x4*>((kv ? A.v_new : A.k_new) +
                                                                    hrow * A.tstride * row_bytes + 16 * (c0 % cpr)));
        st_global(reinterpret_cast<u32x4*>((kv ? A.v : A.k) + (hrow * A.c + slot) * row_bytes + 16 * (c0 % cpr)), v);
      }
      if (tid == 0) {
        int64_t* stw = A.state + kStateWords * static_cast<int64_t>(b);
        st_global(A.pos + static_cast<int64_t>(b) * A.c + slot, static_cast<int32_t>(t0));
        st_global(A.tok + static_cast<int64_t>(b) * A.c + slot, id);
        st_global(stw, t0 + 1);
        if (dropped > 0) st_global(stw + 1, ncomp + dropped);
        st_global(stw + 4, ncomp);
      }
      return;
    }
    L.load(A.sep_ids, A.n_sep, nullptr, set_lds);
    update_block<MODE, DYN>(A, L, ph, lpos, lid, wave_tot, sb);
  } else {
    SetHash H;
    H.load(A.sep_ids, A.n_sep, set_tab, set_lds);
    if (H.exact) {
      update_block<MODE, DYN>(A, H, ph, lpos, lid, wave_tot, sb);
    } else {
      L.set = set_lds;
      L.n = A.n_sep;
      update_block<MODE, DYN>(A, L, ph, lpos, lid, wave_tot, sb);
    }
  }
}

template <int MODE, bool DYN>
__global__ void __launch_bounds__(kUpdThreads) update_kernel(CacheArgs A) {
  update_body<MODE, DYN>(A);
}

// K/V rows of a call with T > 1, grid (Hkv * csplit, B): block x copies
// column range x % csplit of head x / csplit, in both steps below (the rows
// step (2) overwrites are read by step (1) in the same columns only, so the
// block's own barrier orders them); runs
// after update_kernel<UPD_META> of the same call and plans nothing itself.
// From the state META left it takes t1 (t0 = t1 - T), cend1 and cend0 (state
// words 1 and 4). A separator-ring slot whose pos[] is >= cend0 was written
// by this call (every older entry was compacted below cend0, or was cleared
// when the call emptied the ring); those slots form the ring range ending
// just before the new sep_head. Each such row comes from the recent ring
// (position < t0: K/V there are untouched until step (2) below) or from the
// new rows.
__global__ void __launch_bounds__(kUpdThreads) data_kernel(CacheArgs A) {
  extern __shared__ int32_t dyn[];
  __shared__ int32_t wave_tot[kUpdWaves];
  __shared__ int64_t st_s[kStateWords];
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wv = tid / kWave;
  const int b = blockIdx.y;
  const int parts = A.csplit;
  const int g = blockIdx.x / parts;
  const int part = blockIdx.x % parts;
  const int rw = A.rw;
  const int row_bytes = A.D * A.esize;
  const int64_t cache_seq = static_cast<int64_t>(b) * A.Hkv;
  if (tid < kStateWords) st_s[tid] = A.state[kStateWords * static_cast<int64_t>(b) + tid];
  __syncthreads();
  const int64_t t1 = st_s[0], t0 = t1 - A.T;
  const int64_t cend1 = A.a + st_s[1];
  const int64_t cend0 = A.a + st_s[4];

  if (A.s > 0) {
    const int head1 = static_cast<int>(st_s[2]);
    int32_t* lpos = dyn;   // pos[] of the separator ring, by ring index
    const int32_t* posb = A.pos + static_cast<int64_t>(b) * A.c + A.a;
    int cnt = 0;
    for (int j = tid; j < A.s; j += kUpdThreads) {
      const int32_t x = ld_global(posb + j);
      lpos[j] = x;
      cnt += (x >= cend0) ? 1 : 0;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, kWave);
    if (lane == 0) wave_tot[wv] = cnt;
    __syncthreads();
    int nsurv = 0;
#pragma unroll
    for (int i = 0; i < kUpdWaves; ++i) nsurv += wave_tot[i];
    const int jfirst = wrap_add(head1, A.s - nsurv, A.s);   // head1 - nsurv mod s
    // (1) surviving separators -> separator ring
    copy_rows(nsurv, g, g + 1, row_bytes, [&](int r, int gg, int kv, const char** src, char** dst) {
      const int j = wrap_add(jfirst, r, A.s);
      const int64_t x = lpos[j];
      const char* base_new = kv ? A.v_new : A.k_new;
      char* base_c = kv ? A.v : A.k;
      const int64_t crow = (cache_seq + gg) * A.c;
      if (x < t0) {
        *src = base_c + (crow + slot_r(x, A.a, A.s, rw)) * row_bytes;
      } else {
        *src = base_new + ((cache_seq + gg) * A.tstride + (x - t0)) * row_bytes;
      }
      *dst = base_c + (crow + A.a + j) * row_bytes;
    }, part, parts);
    __syncthreads();
  }
  // (2) new tokens that stay
  copy_new_rows(A, b, g, g + 1, t0, t1, cend1, part, parts);
}

__global__ void __launch_bounds__(kUpdThreads) reset_kernel(int32_t* pos, int32_t* tok, int64_t* state,
                                                            int c) {
  const int b = blockIdx.x;
  for (int i = threadIdx.x; i < c; i += kUpdThreads) {
    pos[static_cast<int64_t>(b) * c + i] = -1;
    tok[static_cast<int64_t>(b) * c + i] = -1;
  }
  if (threadIdx.x < kStateWords) state[kStateWords * static_cast<int64_t>(b) + threadIdx.x] = 0;
}

hipError_t launch_cache_reset(const sep_cache& c, hipStream_t st) {
  hipLaunchKernelGGL(reset_kernel, dim3(c.B), dim3(kUpdThreads), 0, st, c.pos, c.tok, c.state,
                     cache_slots(c));
  return hipGetLastError();
}

template <bool DYN>
static hipError_t launch_update_chunk(const sep_cache& c, const CacheArgs& A, size_t dyn, hipStream_t st) {
  if (A.T == 1) {
    hipLaunchKernelGGL((update_kernel<UPD_FUSED, DYN>), dim3(1, c.B), dim3(kUpdThreads), dyn, st, A);
    return hipGetLastError();
  }
  // metadata (and the plan) first; the K/V copy reads what it wrote
  hipLaunchKernelGGL((update_kernel<UPD_META, DYN>), dim3(1, c.B), dim3(kUpdThreads), dyn, st, A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // few (sequence, kv head) pairs: split each head's columns over several
  // workgroups, so that each takes in less (up to 8 parts, 256 blocks)
  CacheArgs D = A;
  const int wall = 2 * (A.D * A.esize / 16);
  D.csplit = 1;
  while (c.B * c.Hkv * D.csplit < 256 && D.csplit < 8 && wall % (2 * D.csplit) == 0) D.csplit *= 2;
  hipLaunchKernelGGL(data_kernel, dim3(c.Hkv * D.csplit, c.B), dim3(kUpdThreads), dyn, st, D);
  return hipGetLastError();
}

static CacheArgs cache_args(const sep_cache& c, const int32_t* sep_ids, int n_sep, int T) {
  CacheArgs A;
  A.k = static_cast<char*>(c.k);
  A.v = static_cast<char*>(c.v);
  A.pos = c.pos;
  A.tok = c.tok;
  A.state = c.state;
  A.sep_ids = sep_ids;
  A.n_sep = n_sep;
  A.a = c.a;
  A.s = c.s;
  A.p = c.p;
  A.w = c.w;
  A.rw = cache_ring(c);
  A.c = cache_slots(c);
  A.Hkv = c.Hkv;
  A.D = c.D;
  A.esize = (c.dtype == SEP_BF16) ? 2 : 4;
  A.tstride = T;
  A.dynamic = (c.policy & SEP_POLICY_DYNAMIC) ? 1 : 0;
  A.accumulate = (c.policy & SEP_POLICY_NO_ACCUM) ? 0 : 1;
  A.csplit = 1;
  return A;
}

static size_t update_dyn_bytes(const sep_cache& c) {
  return 2 * sizeof(int32_t) * static_cast<size_t>(c.s > 0 ? c.s : 1);
}

hipError_t launch_cache_update(const sep_cache& c, const void* k_new, const void* v_new,
                               const int32_t* ids_new, int T, const int32_t* sep_ids, int n_sep,
                               hipStream_t st) {
  CacheArgs A = cache_args(c, sep_ids, n_sep, T);
  const size_t dyn = update_dyn_bytes(c);
  const size_t row_bytes = static_cast<size_t>(c.D) * A.esize;
  // a dynamic-trigger plan covers the ring plus the new tokens in one
  // bitmap of kSpan positions, so a long call runs as consecutive chunks
  // (T tokens at once equal T single updates, hence any split of them)
  const int chunk = A.dynamic ? kSpan - A.rw : T;
  for (int off = 0; off < T; off += chunk) {
    A.T = T - off < chunk ? T - off : chunk;
    A.k_new = static_cast<const char*>(k_new) + off * row_bytes;
    A.v_new = static_cast<const char*>(v_new) + off * row_bytes;
    A.ids_new = ids_new + off;
    const hipError_t e = A.dynamic ? launch_update_chunk<true>(c, A, dyn, st)
                                   : launch_update_chunk<false>(c, A, dyn, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------- decode + update
// One streaming step in one launch: every workgroup (kv head g, sequence b)
// runs the decode of sep_attn_decode (8 waves), and the last of a sequence's
// Hkv workgroups to finish then runs the single-token update of
// sep_cache_update for that sequence, all heads (SepLLM pages: P1
// "Streaming-SepLLM", the forward with the cache, then the update). The
// update rewrites K/V rows and the state words that the other workgroups
// read, so it waits until all of them are done: each workgroup, once all its
// waves have consumed what they loaded, adds one to an arrival counter in
// state word kArriveWord with a device-scope atomic, and the workgroup that
// brings it to Hkv resets it and updates. No other workgroup reads anything
// the update writes, so no release or acquire fence is needed; the next
// launch sees the update at the kernel boundary.
constexpr int kArriveWord = 7;

template <int D, bool ROPE, bool DYN>
__global__ void __launch_bounds__(kUpdThreads) decode_update_kernel(DecodeArgs A, CacheArgs U) {
  static_assert(kUpdThreads == 8 * kWave, "the decode runs with 8 waves here");
  __shared__ int last;
  decode_body<D, 8, ROPE>(A, blockIdx.x, blockIdx.y, 0);
  __syncthreads();
  const int64_t sw = kStateWords * static_cast<int64_t>(blockIdx.y);
  if (threadIdx.x == 0) {
    unsigned long long* arrive = reinterpret_cast<unsigned long long*>(U.state + sw + kArriveWord);
    last = atomicAdd(arrive, 1ull) == static_cast<unsigned long long>(U.Hkv - 1) ? 1 : 0;
  }
  __syncthreads();
  if (!last) return;
  if (threadIdx.x == 0) U.state[sw + kArriveWord] = 0;
  update_body<UPD_FUSED, DYN>(U);
}

// Split decode's second launch, grid (Hkv + 1, B): workgroup 0 runs the
// single-token update of sequence b (blockIdx.y), the longest chain of the
// launch, so it is dispatched first; workgroup 1 + g merges the partials of
// kv head g. The first launch (the ranges) has finished reading the cache,
// so the update may rewrite it.
template <int D, bool DYN>
__global__ void __launch_bounds__(kUpdThreads) merge_update_kernel(DecodeArgs A, CacheArgs U) {
  if (blockIdx.x > 0) {
    merge_body<D>(A, blockIdx.x - 1, blockIdx.y, kUpdThreads);
    return;
  }
  update_body<UPD_FUSED, DYN>(U);
}

// LDS the fused kernel may add for the update's position / id lists
constexpr size_t kFusedDynMax = 32 * 1024;

template <int D, bool ROPE>
static void launch_fused(const sep_cache& c, const DecodeArgs& A, const CacheArgs& U, size_t dyn, hipStream_t st) {
  if (U.dynamic)
    hipLaunchKernelGGL((decode_update_kernel<D, ROPE, true>), dim3(c.Hkv, c.B), dim3(kUpdThreads), dyn, st, A, U);
  else
    hipLaunchKernelGGL((decode_update_kernel<D, ROPE, false>), dim3(c.Hkv, c.B), dim3(kUpdThreads), dyn, st, A, U);
}

hipError_t launch_decode_update(const void* q, const void* k_new, const void* v_new, const int32_t* ids_new,
                                const int32_t* sep_ids, int n_sep, const sep_cache& c, int Hq, float scale,
                                const float* rope, void* out, float* lse, hipStream_t st) {
  const size_t dyn = update_dyn_bytes(c);
  if (decode_uses_split(c, Hq) && dyn <= kFusedDynMax) {
    // the ranges, then the merge with the update in the same launch
    const DecodeArgs A = decode_args(q, k_new, v_new, c, Hq, scale, rope, out, lse);
    hipError_t e = launch_split_ranges(A, c, st);
    if (e != hipSuccess) return e;
    CacheArgs U = cache_args(c, sep_ids, n_sep, 1);
    U.T = 1;
    U.k_new = static_cast<const char*>(k_new);
    U.v_new = static_cast<const char*>(v_new);
    U.ids_new = ids_new;
    const dim3 grid(c.Hkv + 1, c.B);
    if (c.D == 128) {
      if (U.dynamic) hipLaunchKernelGGL((merge_update_kernel<128, true>), grid, dim3(kUpdThreads), dyn, st, A, U);
      else hipLaunchKernelGGL((merge_update_kernel<128, false>), grid, dim3(kUpdThreads), dyn, st, A, U);
    } else {
      if (U.dynamic) hipLaunchKernelGGL((merge_update_kernel<64, true>), grid, dim3(kUpdThreads), dyn, st, A, U);
      else hipLaunchKernelGGL((merge_update_kernel<64, false>), grid, dim3(kUpdThreads), dyn, st, A, U);
    }
    return hipGetLastError();
  }
  // the fused launch covers the few-pairs case, where the decode runs with 8
  // waves; otherwise the two launches it stands for
  if (!decode_uses_wide(c) || dyn > kFusedDynMax || decode_uses_split(c, Hq)) {
    hipError_t e = launch_decode(q, k_new, v_new, c, Hq, scale, rope, out, lse, st);
    if (e != hipSuccess) return e;
    return launch_cache_update(c, k_new, v_new, ids_new, 1, sep_ids, n_sep, st);
  }
  const DecodeArgs A = decode_args(q, k_new, v_new, c, Hq, scale, rope, out, lse);
  CacheArgs U = cache_args(c, sep_ids, n_sep, 1);
  U.T = 1;
  U.k_new = static_cast<const char*>(k_new);
  U.v_new = static_cast<const char*>(v_new);
  U.ids_new = ids_new;
  const bool r = rope != nullptr;
  if (c.D == 128) {
    if (r) launch_fused<128, true>(c, A, U, dyn, st);
    else launch_fused<128, false>(c, A, U, dyn, st);
  } else {
    if (r) launch_fused<64, true>(c, A, U, dyn, st);
    else launch_fused<64, false>(c, A, U, dyn, st);
  }
  return hipGetLastError();
}

}  // namespace sep
