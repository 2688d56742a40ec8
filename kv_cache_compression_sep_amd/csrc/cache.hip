// sep_cache_update / sep_cache_reset: the four-block streaming KV cache.
//
// Blocks and eviction (SepLLM pages: P2 §1.3; P3 §3.3 table; P1
// "KV Cache Manager"): initial tokens are fixed; the local window overflows
// into the past window; when the past window is full its separators are
// kept and the rest dropped; the separator cache holds at most s entries and
// drops its oldest. With fixed caps this becomes: a token at position t >= a
// joins the recent ring R (= past ++ local, cap p + w); when R would hold
// p + w + 1 entries, its oldest p + 1 are compacted first (separators to the
// separator ring, others dropped). The timing of compactions depends only on
// t, so after t tokens the number of compactions is
//   K(t) = max(0, floor((t - a - w) / (p + 1)))   (t > a), 0 otherwise,
// and the compacted prefix is [a, a + K (p + 1)).
//
// A call that appends T tokens is planned once per sequence: the positions
// compacted by this call are [cend0, cend1); their separators are numbered
// k = 0 .. nL-1 in position order, and only the last min(nL, s) survive,
// the k-th landing in ring slot (sep_head + k) mod s. A block-wide count
// gives nL; a backward walk with wavefront ballots finds the survivors.
// Surviving rows are copied into the separator ring before any newly arriving
// token overwrites a recent-ring slot. A call with T > 1 runs two kernels:
// one block per sequence plans and writes pos / tok / state, then one block
// per (head, sequence) copies K/V rows, reading the plan back from pos[] of
// the separator ring. T == 1 runs one fused block per sequence.
#include "common.hpp"
#include "internal.hpp"

#include <type_traits>

namespace sep {

constexpr int kUpdThreads = 512;
constexpr int kUpdWaves = kUpdThreads / kWave;

struct CacheArgs {
  char* k;
  char* v;
  int32_t* pos;
  int32_t* tok;
  int64_t* state;
  const char* k_new;
  const char* v_new;
  const int32_t* ids_new;
  const int32_t* sep_ids;
  int n_sep;
  int a, s, p, w, c, Hkv, D, esize, T;
};

struct PlanHead {
  int64_t t0, t1, cend0, cend1;
  int64_t nL;        // separators compacted by this call
  int head0, cnt0;
  int64_t K1;
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

// Plan one sequence's call. Fills `ph` and the survivor list: entry (k mod s)
// of lpos/lid holds the position and id of the k-th compacted separator for
// the last min(nL, s) values of k. Reads state and tok[] of the recent ring;
// nothing is written to global memory. `early(ph)` runs once `ph` is known,
// before the plan's own loads, so that a caller can put its own independent
// loads in flight. Ends with a barrier. The caller has loaded `S`.
//
// nL is a block-wide count over [cend0, cend1): the positions still in the
// ring (at most p + w) one per thread, the new ones from ids_new in 16-byte
// loads, kCountUnroll of them in flight per thread. The survivors are then
// found by walking that range backwards in chunks of kWalkPer * kUpdThreads
// positions (kWalkPer consecutive positions per thread) until min(nL, s)
// separators are seen; the first chunk is loaded together with the count.
constexpr int kCountUnroll = 16;
constexpr int kWalkPer = 8;

template <class Set, class Early>
__device__ void plan(const CacheArgs& A, int b, const Set& S, PlanHead& ph, int32_t* lpos, int32_t* lid,
                     int32_t* wave_tot, Early early) {
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wv = tid / kWave;
  const int rw = A.p + A.w;
  if (tid == 0) {
    const int64_t* st = A.state + 4 * static_cast<int64_t>(b);
    ph.t0 = st[0];
    const int64_t K0 = st[1];
    ph.head0 = static_cast<int>(st[2]);
    ph.cnt0 = static_cast<int>(st[3]);
    ph.t1 = ph.t0 + A.T;
    ph.K1 = n_compact(ph.t1, A.a, A.p, A.w);
    ph.cend0 = A.a + K0 * (A.p + 1);
    ph.cend1 = A.a + ph.K1 * (A.p + 1);
  }
  __syncthreads();
  early(ph);
  const int64_t t0 = ph.t0, cend0 = ph.cend0, cend1 = ph.cend1;
  const int32_t* tokb = A.tok + static_cast<int64_t>(b) * A.c;
  const int32_t* idsb = A.ids_new + static_cast<int64_t>(b) * A.T;
  // id of position x (cend0 <= x < t1): the ring's tok[] before this call,
  // the new ids from t0 on
  auto id_at = [&](int64_t x) -> int32_t {
    const int32_t* src = (x < t0) ? tokb + slot_r(x, A.a, A.s, rw) : idsb + (x - t0);
    return ld_global(src);
  };

  // first chunk of the walk, loaded now
  int32_t wid[kWalkPer];
  const bool walk = (A.s > 0) && (cend1 > cend0);
  if (walk) {
#pragma unroll
    for (int u = 0; u < kWalkPer; ++u) {
      const int64_t x = cend1 - kWalkPer * kUpdThreads + kWalkPer * tid + u;
      wid[u] = id_at(x >= cend0 ? x : cend0);
    }
  }

  // (1) nL = number of separators among the compacted positions
  int cnt = 0;
  const int64_t xr_end = cend1 < t0 ? cend1 : t0;
  for (int64_t x = cend0 + tid; x < xr_end; x += kUpdThreads) cnt += S(ld_global(tokb + slot_r(x, A.a, A.s, rw))) ? 1 : 0;
  const int64_t xn_beg = cend0 > t0 ? cend0 : t0;
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

  // (2) survivors: walk [cend0, cend1) backwards; `after` counts the
  //     separators at higher positions than the current chunk. Thread tid
  //     owns positions lo + kWalkPer*tid + u, u = 0 .. kWalkPer-1.
  int64_t after = 0;
  // entry of the last separator: (nL - 1) mod s; from_end < s steps back from it
  const int li_last = (A.s > 0 && nL > 0) ? static_cast<int>((nL - 1) % A.s) : 0;
  for (int64_t hi = cend1; hi > cend0 && after < nsurv; hi -= kWalkPer * kUpdThreads) {
    const int64_t lo = hi - kWalkPer * kUpdThreads;
    if (hi != cend1) {
#pragma unroll
      for (int u = 0; u < kWalkPer; ++u) {
        const int64_t x = lo + kWalkPer * tid + u;
        wid[u] = id_at(x >= cend0 ? x : cend0);
      }
    }
    uint32_t fl = 0;   // bit u: position lo + kWalkPer*tid + u is a separator
    int above = 0;     // separators of this wave at lanes above this one
    int wtot = 0;
#pragma unroll
    for (int u = 0; u < kWalkPer; ++u) {
      const bool f = lo + kWalkPer * tid + u >= cend0 && S(wid[u]);
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
// is a source of the same call.
constexpr int kCopyUnroll = 8;

template <class RowFn>
__device__ __forceinline__ void copy_rows(int nrows, int g0, int g1, int row_bytes, RowFn fn) {
  const int cpr = row_bytes / 16;
  const int W = (g1 - g0) * 2 * cpr;
  const int t = threadIdx.x;
  const int R = W <= kUpdThreads ? kUpdThreads / W : 1;
  const int rbeg = W <= kUpdThreads ? t / W : 0;
  if (rbeg >= R) return;
  for (int col = W <= kUpdThreads ? t % W : t; col < W; col += kUpdThreads) {
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
// away, and a ring holds at most p + w positions).
__device__ __forceinline__ void copy_new_rows(const CacheArgs& A, int b, int g0, int g1, int64_t t0,
                                              int64_t t1, int64_t cend1) {
  const int rw = A.p + A.w;
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
    *src = base_new + ((cache_seq + g) * A.T + (y - t0)) * row_bytes;
    *dst = base_c + ((cache_seq + g) * A.c + dslot) * row_bytes;
  });
}

enum { UPD_META = 1, UPD_FUSED = 2 };

// UPD_META : grid (1, B), plan + pos / tok / state; K/V untouched.
// UPD_FUSED: grid (1, B), everything (used for T == 1).
template <int MODE, class Set>
__device__ void update_block(const CacheArgs& A, const Set& S, PlanHead& ph, int32_t* lpos, int32_t* lid,
                             int32_t* wave_tot) {
  const int tid = threadIdx.x;
  const int b = blockIdx.y;
  const int rw = A.p + A.w;
  const int32_t* idsb = A.ids_new + static_cast<int64_t>(b) * A.T;
  // New tokens that stay, as one list: i < n_init are initial positions
  // t0 + i, the rest the recent-ring tail from r_start on (positions below
  // cend1 are compacted by this call, and a ring holds at most p + w). Their
  // ids are loaded before the plan; the stores wait for it.
  constexpr int kKeepPre = 2;
  int64_t r_start = 0;
  int n_init = 0, n_keep = 0;
  int32_t kid[kKeepPre];
  auto keep_pos = [&](int i) -> int64_t { return (i < n_init) ? ph.t0 + i : r_start + (i - n_init); };
  plan(A, b, S, ph, lpos, lid, wave_tot, [&](const PlanHead& h) {
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
  const int d0 = A.s > 0 ? static_cast<int>((ph.head0 + kfirst) % A.s) : 0;
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
        *src = base_new + ((cache_seq + g) * A.T + (x - t0)) * row_bytes;
      }
      *dst = base_c + (crow + dslot) * row_bytes;
    });
    __syncthreads();
    // (2) new tokens that stay
    copy_new_rows(A, b, 0, A.Hkv, t0, t1, cend1);
  }

  int32_t* posb = A.pos + static_cast<int64_t>(b) * A.c;
  int32_t* tokb = A.tok + static_cast<int64_t>(b) * A.c;
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
    int64_t* st = A.state + 4 * static_cast<int64_t>(b);
    st[0] = t1;
    st[1] = ph.K1;
    if (A.s > 0) {
      st[2] = (ph.head0 + nL) % A.s;
      const int64_t cnt = ph.cnt0 + nL;
      st[3] = cnt < A.s ? cnt : A.s;
    }
  }
}

template <int MODE>
__global__ void __launch_bounds__(kUpdThreads) update_kernel(CacheArgs A) {
  extern __shared__ int32_t dyn[];
  __shared__ int32_t set_lds[SEP_MAX_SEP_IDS_];
  __shared__ int32_t set_tab[MODE == UPD_FUSED ? 1 : kHashSize];
  __shared__ int32_t wave_tot[2 * kUpdWaves];
  __shared__ PlanHead ph;
  const int smax = A.s > 0 ? A.s : 1;
  int32_t* lpos = dyn;
  int32_t* lid = dyn + smax;
  SetList L;
  if (MODE == UPD_FUSED) {
    // T == 1. The new K/V row, its id and the state are loaded together;
    // when no compaction is due (K(t0 + 1) == K(t0)) the token only takes
    // its slot: the row, one pos/tok entry and state[0], with no barrier.
    // Otherwise the general block plans the compaction (p + 1 ids, no table).
    const int tid = threadIdx.x;
    const int b = blockIdx.y;
    const int rw = A.p + A.w;
    const int row_bytes = A.D * A.esize;
    const int cpr = row_bytes / 16;
    const int W = A.Hkv * 2 * cpr;
    const int64_t* st = A.state + 4 * static_cast<int64_t>(b);
    const int64_t t0 = ld_global(st), K0 = ld_global(st + 1);
    const int32_t id = ld_global(A.ids_new + b);
    u32x4 val[2];
    int col[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      col[u] = tid + u * kUpdThreads;
      if (col[u] < W) {
        const int kv = (col[u] / cpr) & 1;
        const int g = col[u] / (2 * cpr);
        const char* src = (kv ? A.v_new : A.k_new) + (static_cast<int64_t>(b) * A.Hkv + g) * row_bytes;
        val[u] = ld_global_nt(reinterpret_cast<const u32x4*>(src + 16 * (col[u] % cpr)));
      }
    }
    if (n_compact(t0 + 1, A.a, A.p, A.w) == K0) {
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
        const u32x4 v = ld_global_nt(reinterpret_cast<const u32x4*>((kv ? A.v_new : A.k_new) + hrow * row_bytes +
                                                                    16 * (c0 % cpr)));
        st_global(reinterpret_cast<u32x4*>((kv ? A.v : A.k) + (hrow * A.c + slot) * row_bytes + 16 * (c0 % cpr)), v);
      }
      if (tid == 0) {
        st_global(A.pos + static_cast<int64_t>(b) * A.c + slot, static_cast<int32_t>(t0));
        st_global(A.tok + static_cast<int64_t>(b) * A.c + slot, id);
        st_global(A.state + 4 * static_cast<int64_t>(b), t0 + 1);
      }
      return;
    }
    L.load(A.sep_ids, A.n_sep, nullptr, set_lds);
    update_block<MODE>(A, L, ph, lpos, lid, wave_tot);
  } else {
    SetHash H;
    H.load(A.sep_ids, A.n_sep, set_tab, set_lds);
    if (H.exact) {
      update_block<MODE>(A, H, ph, lpos, lid, wave_tot);
    } else {
      L.set = set_lds;
      L.n = A.n_sep;
      update_block<MODE>(A, L, ph, lpos, lid, wave_tot);
    }
  }
}

// K/V rows of a call with T > 1, grid (Hkv, B), one head per block; runs
// after update_kernel<UPD_META> of the same call and plans nothing itself.
// From the state META left (t1 = t0 + T, sep_head1) it takes t0, cend0 and
// cend1. A separator-ring slot whose pos[] is >= cend0 was written by this
// call (every earlier entry was compacted below cend0); those slots form the
// ring range ending just before sep_head1. Each such row comes from the
// recent ring (position < t0: K/V there are untouched until step (2) below)
// or from the new rows.
__global__ void __launch_bounds__(kUpdThreads) data_kernel(CacheArgs A) {
  extern __shared__ int32_t dyn[];
  __shared__ int32_t wave_tot[kUpdWaves];
  __shared__ int64_t st_s[3];
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wv = tid / kWave;
  const int b = blockIdx.y;
  const int g = blockIdx.x;
  const int rw = A.p + A.w;
  const int row_bytes = A.D * A.esize;
  const int64_t cache_seq = static_cast<int64_t>(b) * A.Hkv;
  if (tid < 3) st_s[tid] = A.state[4 * static_cast<int64_t>(b) + tid];
  __syncthreads();
  const int64_t t1 = st_s[0], t0 = t1 - A.T;
  const int64_t cend1 = A.a + st_s[1] * (A.p + 1);
  const int64_t cend0 = A.a + n_compact(t0, A.a, A.p, A.w) * (A.p + 1);

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
        *src = base_new + ((cache_seq + gg) * A.T + (x - t0)) * row_bytes;
      }
      *dst = base_c + (crow + A.a + j) * row_bytes;
    });
    __syncthreads();
  }
  // (2) new tokens that stay
  copy_new_rows(A, b, g, g + 1, t0, t1, cend1);
}

__global__ void __launch_bounds__(kUpdThreads) reset_kernel(int32_t* pos, int32_t* tok, int64_t* state,
                                                            int c) {
  const int b = blockIdx.x;
  for (int i = threadIdx.x; i < c; i += kUpdThreads) {
    pos[static_cast<int64_t>(b) * c + i] = -1;
    tok[static_cast<int64_t>(b) * c + i] = -1;
  }
  if (threadIdx.x < 4) state[4 * static_cast<int64_t>(b) + threadIdx.x] = 0;
}

hipError_t launch_cache_reset(const sep_cache& c, hipStream_t st) {
  const int cap = c.a + c.s + c.p + c.w;
  hipLaunchKernelGGL(reset_kernel, dim3(c.B), dim3(kUpdThreads), 0, st, c.pos, c.tok, c.state, cap);
  return hipGetLastError();
}

hipError_t launch_cache_update(const sep_cache& c, const void* k_new, const void* v_new,
                               const int32_t* ids_new, int T, const int32_t* sep_ids, int n_sep,
                               hipStream_t st) {
  CacheArgs A;
  A.k = static_cast<char*>(c.k);
  A.v = static_cast<char*>(c.v);
  A.pos = c.pos;
  A.tok = c.tok;
  A.state = c.state;
  A.k_new = static_cast<const char*>(k_new);
  A.v_new = static_cast<const char*>(v_new);
  A.ids_new = ids_new;
  A.sep_ids = sep_ids;
  A.n_sep = n_sep;
  A.a = c.a;
  A.s = c.s;
  A.p = c.p;
  A.w = c.w;
  A.c = c.a + c.s + c.p + c.w;
  A.Hkv = c.Hkv;
  A.D = c.D;
  A.esize = (c.dtype == SEP_BF16) ? 2 : 4;
  A.T = T;
  const size_t dyn = 2 * sizeof(int32_t) * static_cast<size_t>(c.s > 0 ? c.s : 1);
  if (T == 1) {
    hipLaunchKernelGGL(update_kernel<UPD_FUSED>, dim3(1, c.B), dim3(kUpdThreads), dyn, st, A);
    return hipGetLastError();
  }
  // metadata (and the plan) first; the K/V copy reads what it wrote
  hipLaunchKernelGGL(update_kernel<UPD_META>, dim3(1, c.B), dim3(kUpdThreads), dyn, st, A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(data_kernel, dim3(c.Hkv, c.B), dim3(kUpdThreads), dyn, st, A);
  return hipGetLastError();
}

}  // namespace sep
