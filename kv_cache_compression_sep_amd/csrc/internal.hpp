// Internal launchers behind the C ABI (argument checking happens in api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sepattn.h"

#define SEP_MAX_SEP_IDS_ SEP_MAX_SEP_IDS

namespace sep {

// int64 words of cache state per sequence (see sep_cache in sepattn.h)
constexpr int kStateWords = 8;

// recent-ring size and slot count of a cache under its policy
inline int cache_ring(const sep_cache& c) {
  return c.p + c.w + ((c.policy & SEP_POLICY_DYNAMIC) ? c.s : 0);
}
inline int cache_slots(const sep_cache& c) { return c.a + c.s + cache_ring(c); }

// Decode geometry. Few (sequence, kv head) pairs: wider workgroups (8
// waves), so that each pair's list is read by more waves at once; and, when
// the cache carries a large enough work buffer, each list split over several
// workgroups: ranges of whole 32-entry slices, one wave per workgroup, so
// that each CU takes in as little of the list as possible (16 KB of K and V
// at D = 128); at most kMaxSplits ranges per list (longer lists take longer
// ranges). A list holds at most slots + 1 entries. The split (two launches
// and the partials' round trip) pays only while the lists are too few to
// spread over the CUs whole: up to kSplitMaxPairs (sequence, kv head) pairs.
inline bool decode_uses_wide(const sep_cache& c) { return c.B * c.Hkv < 256; }
constexpr int kSplitMaxPairs = 64;
inline bool decode_may_split(const sep_cache& c) { return c.B * c.Hkv <= kSplitMaxPairs; }
constexpr int kSplitChunk = 32;
constexpr int kMaxSplits = 32;
inline void decode_split_shape(const sep_cache& c, int* ns, int* span) {
  const int nch = (cache_slots(c) + 1 + kSplitChunk - 1) / kSplitChunk;
  *ns = nch < kMaxSplits ? nch : kMaxSplits;
  *span = kSplitChunk * ((nch + *ns - 1) / *ns);
}
// one partial per wave of a range: [B][Hkv][ns * kSplitWaves][G] rows of D + 4 floats
constexpr int kSplitWaves = kSplitChunk / 32;
inline size_t decode_split_bytes(const sep_cache& c, int Hq) {
  int ns, span;
  decode_split_shape(c, &ns, &span);
  return static_cast<size_t>(c.B) * Hq * ns * kSplitWaves * static_cast<size_t>(c.D + 4) * sizeof(float);
}
inline bool decode_uses_split(const sep_cache& c, int Hq) {
  return decode_may_split(c) && c.work != nullptr && c.work_bytes >= decode_split_bytes(c, Hq);
}

hipError_t launch_is_sep(const int32_t* ids, int64_t N, const int32_t* sep_ids, int n_sep,
                         uint8_t* is_sep, hipStream_t st);
hipError_t launch_tile_class(const uint8_t* is_sep, int B, int S, int a, int n, int tq, int tk,
                             uint8_t* tc, hipStream_t st);
hipError_t launch_dense_mask(const uint8_t* is_sep, int B, int S, int a, int n, uint8_t* M,
                             hipStream_t st);
hipError_t launch_index_compact(const uint8_t* is_sep, int B, int S, int32_t* rank,
                                int32_t* sep_pos, int32_t* count, hipStream_t st);
hipError_t launch_mask_compact(const int32_t* ids, int B, int S, const int32_t* sep_ids, int n_sep,
                               uint8_t* is_sep, int32_t* rank, int32_t* sep_pos, int32_t* count, hipStream_t st);
hipError_t launch_prefill(const void* q, const void* k, const void* v, int dtype, int B, int Hq,
                          int Hkv, int S, int D, const uint8_t* is_sep, const int32_t* rank,
                          const int32_t* sep_pos, int a, int n, float scale, void* out, float* lse,
                          hipStream_t st);
hipError_t launch_prefill_backward(const void* q, const void* k, const void* v, const void* out,
                                   const void* dout, const float* lse, int dtype, int B, int Hq, int Hkv,
                                   int S, int D, const uint8_t* is_sep, const int32_t* rank,
                                   const int32_t* sep_pos, int a, int n, float scale, float* delta, float* dq,
                                   float* dk, float* dv, hipStream_t st);
// argument checks of sep_attn_prefill_backward apart from its delta
// workspace (api.hip); SEP_OK or the status the entry point returns
int check_backward_args(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* lse, int dtype, int B, int Hq, int Hkv, int S, int D, const uint8_t* is_sep,
                        const int32_t* rank, const int32_t* sep_pos, int a, int n, float scale, const float* dq,
                        const float* dk, const float* dv);
hipError_t launch_cache_reset(const sep_cache& c, hipStream_t st);
hipError_t launch_cache_update(const sep_cache& c, const void* k_new, const void* v_new,
                               const int32_t* ids_new, int T, const int32_t* sep_ids, int n_sep,
                               hipStream_t st);
// decode then single-token update in one launch where the decode runs wide
// (else the two launches)
hipError_t launch_decode_update(const void* q, const void* k_new, const void* v_new, const int32_t* ids_new,
                                const int32_t* sep_ids, int n_sep, const sep_cache& c, int Hq, float scale,
                                const float* rope, void* out, float* lse, hipStream_t st);
hipError_t launch_decode(const void* q, const void* k_new, const void* v_new, const sep_cache& c,
                         int Hq, float scale, const float* rope, void* out, float* lse, hipStream_t st);
size_t chunk_workspace_bytes(const sep_cache& c, int C);
hipError_t launch_prefill_chunk(const void* q, const void* k, const void* v, const int32_t* ids, int C,
                                const int32_t* sep_ids, int n_sep, const sep_cache& c, int Hq, int n,
                                float scale, void* workspace, void* out, float* lse, hipStream_t st);
hipError_t launch_rope_table(double base, int D, int n_pos, float* table, hipStream_t st);

}  // namespace sep
