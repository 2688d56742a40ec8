// Tile bookkeeping shared by the Sep-Attention prefill kernels.
//
// A workgroup owns query rows [q0, q1). With band_lo = max(q0 - n + 1, 0),
// (or the first key row that may enter a band, in chunk mode),
// every key j < band_lo is visible to all of these queries iff it is an
// initial token (j < a) or a separator, and to none of them otherwise
// (SepLLM pages: P2 §1.2 mask matrix; P1 "SepAttention", initial OR window
// OR separator, AND causal). The workgroup's key list is therefore
//   global keys: [0, min(a, band_lo)) ++ separators in [a, band_lo)
//                (read through sep_pos[rank[a] .. rank[band_lo]]), no mask;
//   band keys:   [band_lo, q1), element mask where a tile is mixed;
// cut into tiles of KT keys, global tiles first.
#pragma once

#include "common.hpp"

namespace sep {

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const uint8_t* is_sep;
  const int32_t* rank;
  const int32_t* sep_pos;
  int B, Hq, Hkv, S, a, n;
  int G, HPW, QT, n_hg, n_qt;
  float scale_log2;
  // Chunk mode (sep_attn_prefill_chunk): the keys are a longer sequence of
  // Skv rows in which query row r sits at index q_base + r, and key rows
  // below key_lo[b] are never band keys. Plain prefill: Skv = S, q_base = 0,
  // key_lo = nullptr.
  int Skv, q_base;
  const int32_t* key_lo;
};

struct TileInfo {
  int band_lo, n_init, n_glob, rank_a, ntg, ntiles;
};

template <int KT>
__device__ __forceinline__ TileInfo tile_info(const int32_t* rk, int S, int a, int n, int q0, int q1,
                                              int key_lo = 0) {
  TileInfo ti;
  ti.band_lo = max(q0 - n + 1, key_lo);
  ti.n_init = min(a, ti.band_lo);
  ti.rank_a = rk[min(a, S)];
  const int n_sepg = (ti.band_lo > a) ? (rk[ti.band_lo] - ti.rank_a) : 0;
  ti.n_glob = ti.n_init + n_sepg;
  ti.ntg = (ti.n_glob + KT - 1) / KT;
  ti.ntiles = ti.ntg + (q1 - ti.band_lo + KT - 1) / KT;
  return ti;
}

// Row to load for entry u of tile t (entries past the list are clamped to a
// valid row; their scores are masked).
template <int KT>
__device__ __forceinline__ int tile_key(const TileInfo& ti, const int32_t* sp, int S, int t, int u,
                                        bool* is_band) {
  if (t < ti.ntg) {
    *is_band = false;
    const int gu = t * KT + u;
    if (gu >= ti.n_glob) return 0;
    if (gu < ti.n_init) return gu;
    return sp[ti.rank_a + gu - ti.n_init];
  }
  *is_band = true;
  const int j = ti.band_lo + (t - ti.ntg) * KT + u;
  return j < S ? j : S - 1;
}

// Work item of a workgroup: late (heavy) query tiles first; the pairs that
// share a key/value head stay on one XCD (workgroups are dealt to the 8 XCDs
// round-robin by their linear index).
__device__ __forceinline__ void work_item(const PrefillArgs& P, int id, int* pair, int* qt) {
  const int pairs = P.B * P.Hkv * P.n_hg;
  if ((pairs % 8) == 0) {
    const int per = pairs / 8;
    const int xcd = id % 8;
    const int k = id / 8;
    *pair = xcd + 8 * (k % per);
    *qt = P.n_qt - 1 - k / per;
  } else {
    *pair = id % pairs;
    *qt = P.n_qt - 1 - id / pairs;
  }
}

// Per-lane visibility word of a tile: bit u stands for key u of the tile.
// Band tiles: causal, window, initial and separator tests for query qi.
// Global tiles: the first nvalid entries.
__device__ __forceinline__ uint64_t vis_word(bool band, int qi, int jmin, int n, int a,
                                             uint64_t sepbits, int nvalid) {
  if (!band) return nvalid >= 64 ? ~0ull : ((1ull << nvalid) - 1);
  const int dq = qi - jmin;                                // causal: u <= dq
  const int wl = dq - n + 1;                               // window: u >= wl
  const int ih = a - jmin;                                 // initial: u < ih
  const uint64_t cm = dq >= 63 ? ~0ull : (dq < 0 ? 0ull : ((2ull << dq) - 1));
  const uint64_t wm = wl <= 0 ? ~0ull : (wl >= 64 ? 0ull : ~((1ull << wl) - 1));
  const uint64_t im = ih >= 64 ? ~0ull : (ih <= 0 ? 0ull : ((1ull << ih) - 1));
  return cm & (wm | im | sepbits);
}

hipError_t launch_prefill_bf16(PrefillArgs A, int D, hipStream_t st);

}  // namespace sep
