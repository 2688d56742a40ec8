// sep_attn_prefill_chunk: C new tokens attend the live cache and themselves.
//
// SepLLM pages: P1 "SepAttention" (build_generate_mask applies the prefill
// keep rule -- initial OR separator OR local window, AND causal -- to the
// rows of new queries; a generation window and a window per layer); P2 §1.3
// (the cache holds only what was retained). Query tau = t + i of the chunk
// sees a retained entry or chunk key at position p iff p <= tau and (p < a,
// or it is a separator, or tau - p < n).
//
// The keys are laid out as one sequence of V = slots + C rows per
// (sequence, kv head), so that the bf16 prefill kernel runs on it unchanged
// apart from three arguments (key rows Skv = V, query base = slots, first
// band row key_lo):
//
//   [ I (n_init) | S, oldest first (cnt) | padding | R, oldest first (n_rec) | chunk (C) ]
//   0                                            key_lo = slots - n_rec      slots         V
//
// R ends where the chunk starts, and R and the chunk are consecutive
// positions, so a row distance there equals a position distance and the
// band's window test is the position test. Initial entries, the separator
// ring and the chunk's initial tokens are flagged like separators: visible
// to every later query, through the gathered global list (their window test
// never matters). Padding rows are zero, unflagged and below key_lo, so no
// tile ever makes them visible.
#include "common.hpp"
#include "internal.hpp"
#include "prefill.hpp"

namespace sep {
namespace {

constexpr int kRowsPerBlock = 32;

struct ChunkArgs {
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* tok;
  const int64_t* state;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* ids;
  const int32_t* sep_ids;
  uint16_t* xk;
  uint16_t* xv;
  uint8_t* xflag;
  int32_t* key_lo;
  int n_sep, a, s, rw, slots, Hkv, C, V;
};

// grid (ceil(V / kRowsPerBlock), B * Hkv): the rows [x0, x0 + 32) of one
// (sequence, kv head); 16-byte chunks, D / 8 per row
template <int D>
__global__ void __launch_bounds__(256) context_kernel(ChunkArgs A) {
  constexpr int CPR = D / 8;
  __shared__ int32_t set[SEP_MAX_SEP_IDS];
  const int bg = blockIdx.y;
  const int b = bg / A.Hkv;
  const int g = bg % A.Hkv;
  const int x0 = blockIdx.x * kRowsPerBlock;
  for (int i = threadIdx.x; i < A.n_sep; i += blockDim.x) set[i] = A.sep_ids[i];
  __syncthreads();

  const int64_t* st = A.state + kStateWords * static_cast<int64_t>(b);
  const int64_t t = st[0];
  const int64_t ncomp = st[1];
  const int head = static_cast<int>(st[2]);
  const int cnt = static_cast<int>(st[3]);
  const int n_init = static_cast<int>(t < A.a ? t : A.a);
  const int64_t cend = A.a + ncomp;
  const int64_t rec_lo = cend > A.a ? cend : A.a;
  const int n_rec = static_cast<int>(t > rec_lo ? t - rec_lo : 0);
  int s0 = 0;
  if (cnt > 0) {
    s0 = (head - cnt) % A.s;
    if (s0 < 0) s0 += A.s;
  }
  const int r0 = n_rec > 0 ? static_cast<int>((rec_lo - A.a) % A.rw) : 0;
  const int klo = A.slots - n_rec;
  if (g == 0 && blockIdx.x == 0 && threadIdx.x == 0) A.key_lo[b] = klo;

  // source of row x: 0 padding, 1 cache slot, 2 chunk row
  auto source = [&](int x, int* src, int* row) {
    if (x < n_init) {
      *src = 1; *row = x;
    } else if (x < n_init + cnt) {
      int r = s0 + (x - n_init);
      r = r >= A.s ? r - A.s : r;
      *src = 1; *row = A.a + r;
    } else if (x < klo) {
      *src = 0; *row = 0;
    } else if (x < A.slots) {
      int r = r0 + (x - klo);
      r = r >= A.rw ? r - A.rw : r;
      *src = 1; *row = A.a + A.s + r;
    } else {
      *src = 2; *row = x - A.slots;
    }
  };
  // flags (kv head 0 only): initial and separator-ring entries 1, padding 0,
  // recent entries and chunk tokens by their id (chunk tokens before a: 1)
  if (g == 0) {
    for (int x = x0 + threadIdx.x; x < min(x0 + kRowsPerBlock, A.V); x += blockDim.x) {
      int src, row;
      source(x, &src, &row);
      bool flag = false;
      if (x < n_init + cnt) flag = true;
      else if (src == 1) flag = in_set(A.tok[static_cast<int64_t>(b) * A.slots + row], set, A.n_sep);
      else if (src == 2) flag = in_set(A.ids[static_cast<int64_t>(b) * A.C + row], set, A.n_sep) || (t + row < A.a);
      A.xflag[static_cast<int64_t>(b) * A.V + x] = static_cast<uint8_t>(flag);
    }
  }

  const int64_t cbase = static_cast<int64_t>(bg) * A.slots * D;
  const int64_t nbase = static_cast<int64_t>(bg) * A.C * D;
  const int64_t xbase = static_cast<int64_t>(bg) * A.V * D;
  // every load of the thread first (one unconditional load per operand,
  // from a computed address; padding rows read cache row 0 and store
  // zeros), then the stores: kPer rows in flight
  constexpr int kPer = kRowsPerBlock * CPR / 256;
  u32x4 kk[kPer], vv[kPer];
  bool pad[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = threadIdx.x + 256 * i;
    const int x = min(x0 + e / CPR, A.V - 1);
    const int c = e % CPR;
    int src, row;
    source(x, &src, &row);
    pad[i] = src == 0;
    const uint16_t* kp = src == 2 ? A.k + nbase : A.kc + cbase;
    const uint16_t* vp = src == 2 ? A.v + nbase : A.vc + cbase;
    kk[i] = *reinterpret_cast<const u32x4*>(kp + static_cast<int64_t>(row) * D + 8 * c);
    vv[i] = *reinterpret_cast<const u32x4*>(vp + static_cast<int64_t>(row) * D + 8 * c);
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = threadIdx.x + 256 * i;
    const int x = x0 + e / CPR;
    const int c = e % CPR;
    if (x < A.V) {
      const u32x4 z = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(A.xk + xbase + static_cast<int64_t>(x) * D + 8 * c) = pad[i] ? z : kk[i];
      *reinterpret_cast<u32x4*>(A.xv + xbase + static_cast<int64_t>(x) * D + 8 * c) = pad[i] ? z : vv[i];
    }
  }
}

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct Workspace {
  size_t xk, xv, xflag, rank, sep_pos, count, key_lo, total;
};

Workspace layout(int B, int Hkv, int D, int V) {
  Workspace w;
  size_t o = 0;
  const size_t kv = static_cast<size_t>(B) * Hkv * V * D * 2;
  w.xk = o; o = align256(o + kv);
  w.xv = o; o = align256(o + kv);
  w.xflag = o; o = align256(o + static_cast<size_t>(B) * V);
  w.rank = o; o = align256(o + static_cast<size_t>(B) * (V + 1) * 4);
  w.sep_pos = o; o = align256(o + static_cast<size_t>(B) * V * 4);
  w.count = o; o = align256(o + static_cast<size_t>(B) * 4);
  w.key_lo = o; o = align256(o + static_cast<size_t>(B) * 4);
  w.total = o;
  return w;
}

}  // namespace

size_t chunk_workspace_bytes(const sep_cache& c, int C) {
  return layout(c.B, c.Hkv, c.D, cache_slots(c) + C).total;
}

hipError_t launch_prefill_chunk(const void* q, const void* k, const void* v, const int32_t* ids, int C,
                                const int32_t* sep_ids, int n_sep, const sep_cache& c, int Hq, int n,
                                float scale, void* workspace, void* out, float* lse, hipStream_t st) {
  const int slots = cache_slots(c);
  const int V = slots + C;
  const Workspace w = layout(c.B, c.Hkv, c.D, V);
  char* ws = static_cast<char*>(workspace);
  ChunkArgs A;
  A.kc = static_cast<const uint16_t*>(c.k);
  A.vc = static_cast<const uint16_t*>(c.v);
  A.tok = c.tok;
  A.state = c.state;
  A.k = static_cast<const uint16_t*>(k);
  A.v = static_cast<const uint16_t*>(v);
  A.ids = ids;
  A.sep_ids = sep_ids;
  A.xk = reinterpret_cast<uint16_t*>(ws + w.xk);
  A.xv = reinterpret_cast<uint16_t*>(ws + w.xv);
  A.xflag = reinterpret_cast<uint8_t*>(ws + w.xflag);
  A.key_lo = reinterpret_cast<int32_t*>(ws + w.key_lo);
  A.n_sep = n_sep;
  A.a = c.a;
  A.s = c.s;
  A.rw = cache_ring(c);
  A.slots = slots;
  A.Hkv = c.Hkv;
  A.C = C;
  A.V = V;
  const dim3 grid((V + kRowsPerBlock - 1) / kRowsPerBlock, c.B * c.Hkv);
  if (c.D == 128)
    hipLaunchKernelGGL(context_kernel<128>, grid, dim3(256), 0, st, A);
  else
    hipLaunchKernelGGL(context_kernel<64>, grid, dim3(256), 0, st, A);
  int32_t* rank = reinterpret_cast<int32_t*>(ws + w.rank);
  int32_t* sep_pos = reinterpret_cast<int32_t*>(ws + w.sep_pos);
  hipError_t e = launch_index_compact(A.xflag, c.B, V, rank, sep_pos, reinterpret_cast<int32_t*>(ws + w.count), st);
  if (e != hipSuccess) return e;

  PrefillArgs P;
  P.q = q;
  P.k = A.xk;
  P.v = A.xv;
  P.out = out;
  P.lse = lse;
  P.is_sep = A.xflag;
  P.rank = rank;
  P.sep_pos = sep_pos;
  P.B = c.B;
  P.Hq = Hq;
  P.Hkv = c.Hkv;
  P.S = C;
  P.Skv = V;
  P.q_base = slots;
  P.key_lo = A.key_lo;
  P.a = 0;                                        // initial entries are flagged instead
  P.n = n;
  P.G = Hq / c.Hkv;
  P.HPW = (P.G % 4 == 0) ? 4 : ((P.G % 2 == 0) ? 2 : 1);
  P.n_hg = P.G / P.HPW;
  P.scale_log2 = scale * kLog2e;
  return launch_prefill_bf16(P, c.D, st);
}

}  // namespace sep
