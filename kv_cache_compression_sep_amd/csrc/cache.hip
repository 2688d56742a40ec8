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
// compacted by this call are [cend0, cend1); a block-wide ballot/mbcnt
// prefix sum over their separator flags numbers the new separators
// k = 0 .. nL-1, and only the last min(nL, s) survive, the k-th landing in
// ring slot (sep_head + k) mod s. Surviving rows are copied into the ring
// before any newly arriving token overwrites a recent-ring slot.
#include "common.hpp"
#include "internal.hpp"

namespace sep {

constexpr int kUpdThreads = 256;
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

__device__ __forceinline__ int slot_r(int64_t x, int a, int s, int rw) {
  return a + s + static_cast<int>((x - a) % rw);
}

// Plan one sequence's call. Fills `ph` and the survivor list: entry (k mod s)
// of lpos/lid holds the position and id of the k-th compacted separator for
// the last min(nL, s) values of k. Reads tok[] of the recent ring; nothing is
// written to global memory. Ends with a barrier.
__device__ void plan(const CacheArgs& A, int b, const int32_t* set, PlanHead& ph, int32_t* lpos,
                     int32_t* lid, int32_t* wave_tot) {
  const int tid = threadIdx.x;
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
  const int64_t t0 = ph.t0, cend0 = ph.cend0, cend1 = ph.cend1;
  const int32_t* tokb = A.tok + static_cast<int64_t>(b) * A.c;
  const int32_t* idsb = A.ids_new + static_cast<int64_t>(b) * A.T;
  int64_t carry = 0;
  int parity = 0;
  for (int64_t base = cend0; base < cend1; base += kUpdThreads, parity ^= 1) {
    const int64_t x = base + tid;
    int32_t id = -1;
    bool f = false;
    if (x < cend1) {
      id = (x < t0) ? tokb[slot_r(x, A.a, A.s, rw)] : idsb[x - t0];
      f = in_set(id, set, A.n_sep);
    }
    const uint64_t m = ballot(f);
    if ((tid % kWave) == 0) wave_tot[parity * kUpdWaves + tid / kWave] = __popcll(m);
    __syncthreads();
    int before = 0, chunk = 0;
#pragma unroll
    for (int wv = 0; wv < kUpdWaves; ++wv) {
      const int tt = wave_tot[parity * kUpdWaves + wv];
      before += (wv < tid / kWave) ? tt : 0;
      chunk += tt;
    }
    if (f && A.s > 0) {
      const int64_t k = carry + before + static_cast<int>(mbcnt(m));
      // Within one chunk, keep only ranks that can still be among the last s,
      // so no two writers of this chunk share a slot.
      if (k >= carry + chunk - A.s) {
        const int li = static_cast<int>(k % A.s);
        lpos[li] = static_cast<int32_t>(x);
        lid[li] = id;
      }
    }
    carry += chunk;
    __syncthreads();
  }
  if (tid == 0) ph.nL = carry;
  __syncthreads();
}

// Copy `nrows` rows (head range [g0, g1)) using 16-byte chunks.
// The caller passes a functor mapping a row index to (src, dst) pointers.
template <class RowFn>
__device__ __forceinline__ void copy_rows(int nrows, int g0, int g1, int row_bytes, RowFn fn) {
  const int cpr = row_bytes / 16;
  const int total = nrows * (g1 - g0) * 2 * cpr;
  for (int e = threadIdx.x; e < total; e += kUpdThreads) {
    const int chunk = e % cpr;
    int rest = e / cpr;
    const int kv = rest & 1;
    rest >>= 1;
    const int g = g0 + rest % (g1 - g0);
    const int r = rest / (g1 - g0);
    const char* src;
    char* dst;
    fn(r, g, kv, &src, &dst);
    *reinterpret_cast<u32x4*>(dst + 16 * chunk) = *reinterpret_cast<const u32x4*>(src + 16 * chunk);
  }
}

enum { UPD_DATA = 0, UPD_META = 1, UPD_FUSED = 2 };

// UPD_DATA : grid (Hkv, B), K/V rows of one head, state untouched.
// UPD_META : grid (1, B), pos / tok / state only.
// UPD_FUSED: grid (1, B), everything (used for T == 1).
template <int MODE>
__global__ void __launch_bounds__(kUpdThreads) update_kernel(CacheArgs A) {
  extern __shared__ int32_t dyn[];
  __shared__ int32_t set[SEP_MAX_SEP_IDS_];
  __shared__ int32_t wave_tot[2 * kUpdWaves];
  __shared__ PlanHead ph;
  const int tid = threadIdx.x;
  const int b = blockIdx.y;
  const int smax = A.s > 0 ? A.s : 1;
  int32_t* lpos = dyn;
  int32_t* lid = dyn + smax;
  for (int i = tid; i < A.n_sep; i += kUpdThreads) set[i] = A.sep_ids[i];
  __syncthreads();
  plan(A, b, set, ph, lpos, lid, wave_tot);

  const int rw = A.p + A.w;
  const int64_t t0 = ph.t0, t1 = ph.t1, cend1 = ph.cend1, nL = ph.nL;
  const int nsurv = static_cast<int>(nL < A.s ? nL : A.s);
  const int64_t kfirst = nL - nsurv;
  const int row_bytes = A.D * A.esize;
  const int64_t cache_seq = static_cast<int64_t>(b) * A.Hkv;

  if (MODE != UPD_META) {
    const int g0 = (MODE == UPD_DATA) ? blockIdx.x : 0;
    const int g1 = (MODE == UPD_DATA) ? blockIdx.x + 1 : A.Hkv;
    // (1) surviving separators -> separator ring
    copy_rows(nsurv, g0, g1, row_bytes, [&](int r, int g, int kv, const char** src, char** dst) {
      const int64_t k = kfirst + r;
      const int li = static_cast<int>(k % A.s);
      const int64_t x = lpos[li];
      const int dslot = A.a + static_cast<int>((ph.head0 + k) % A.s);
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
    // (2) new tokens that stay: initial slots, and recent-ring slots for
    //     positions >= cend1 (those below cend1 were compacted away).
    const int64_t keep_lo = t1 - rw > t0 ? t1 - rw : t0;  // a ring holds at most rw positions
    const int64_t r_lo = (cend1 > keep_lo) ? cend1 : keep_lo;
    const int64_t r_start = r_lo > A.a ? r_lo : A.a;
    const int n_init_new = static_cast<int>((t1 < A.a ? t1 : A.a) > t0 ? ((t1 < A.a ? t1 : A.a) - t0) : 0);
    const int n_r_new = static_cast<int>(t1 > r_start ? t1 - r_start : 0);
    copy_rows(n_init_new + n_r_new, g0, g1, row_bytes,
              [&](int r, int g, int kv, const char** src, char** dst) {
                const int64_t y = (r < n_init_new) ? t0 + r : r_start + (r - n_init_new);
                const int dslot = (y < A.a) ? static_cast<int>(y) : slot_r(y, A.a, A.s, rw);
                const char* base_new = kv ? A.v_new : A.k_new;
                char* base_c = kv ? A.v : A.k;
                *src = base_new + ((cache_seq + g) * A.T + (y - t0)) * row_bytes;
                *dst = base_c + ((cache_seq + g) * A.c + dslot) * row_bytes;
              });
  }

  if (MODE != UPD_DATA) {
    int32_t* posb = A.pos + static_cast<int64_t>(b) * A.c;
    int32_t* tokb = A.tok + static_cast<int64_t>(b) * A.c;
    const int32_t* idsb = A.ids_new + static_cast<int64_t>(b) * A.T;
    // survivors -> separator-ring metadata (ids were captured by the plan)
    for (int r = tid; r < nsurv; r += kUpdThreads) {
      const int64_t k = kfirst + r;
      const int li = static_cast<int>(k % A.s);
      const int dslot = A.a + static_cast<int>((ph.head0 + k) % A.s);
      posb[dslot] = lpos[li];
      tokb[dslot] = lid[li];
    }
    // recent-ring slots of positions compacted by this call become empty
    const int64_t old_lo = ph.cend0;
    const int64_t old_hi = cend1 < t0 ? cend1 : t0;
    for (int64_t x = old_lo + tid; x < old_hi; x += kUpdThreads) {
      const int sl = slot_r(x, A.a, A.s, rw);
      posb[sl] = -1;
      tokb[sl] = -1;
    }
    __syncthreads();
    const int64_t keep_lo = t1 - rw > t0 ? t1 - rw : t0;
    const int64_t r_lo = (cend1 > keep_lo) ? cend1 : keep_lo;
    const int64_t r_start = r_lo > A.a ? r_lo : A.a;
    for (int64_t y = t0 + tid; y < t1; y += kUpdThreads) {
      if (y < A.a) {
        posb[y] = static_cast<int32_t>(y);
        tokb[y] = idsb[y - t0];
      } else if (y >= r_start) {
        const int sl = slot_r(y, A.a, A.s, rw);
        posb[sl] = static_cast<int32_t>(y);
        tokb[sl] = idsb[y - t0];
      }
    }
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
  hipLaunchKernelGGL(update_kernel<UPD_DATA>, dim3(c.Hkv, c.B), dim3(kUpdThreads), dyn, st, A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(update_kernel<UPD_META>, dim3(1, c.B), dim3(kUpdThreads), dyn, st, A);
  return hipGetLastError();
}

}  // namespace sep
