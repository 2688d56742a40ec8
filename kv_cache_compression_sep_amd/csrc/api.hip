// C ABI of libsepattn: host-side validation, then kernel launches.
// Every check runs before anything is enqueued; a failed check returns a
// negative sep_status and launches nothing.
#include <stdint.h>

#include "internal.hpp"
#include "sepattn.h"

namespace {

constexpr int kVersion = 1 * 10000 + 2 * 100 + 0;   // 1.2: prefill backward, RoPE decode
constexpr int kMaxSepCache = 8192;   // separator-ring cap (plan list lives in LDS)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? SEP_OK : SEP_ERR_HIP; }

int check_cache(const sep_cache* c) {
  if (c == nullptr) return SEP_ERR_NULL;
  if (c->pos == nullptr || c->tok == nullptr || c->state == nullptr) return SEP_ERR_NULL;
  if (c->B <= 0 || c->Hkv <= 0) return SEP_ERR_SHAPE;
  if (c->D != 64 && c->D != 128) return SEP_ERR_SHAPE;
  if (c->dtype != SEP_BF16 && c->dtype != SEP_F32) return SEP_ERR_DTYPE;
  // parameter contract (study notes, "Streaming 参数约束"), with c = a+s+p+w
  if (c->a < 0 || c->w < 1 || c->s < 0 || c->p < 0) return SEP_ERR_PARAM;
  const bool sepllm = c->s >= 1 && c->p >= 1;
  const bool streaming = c->s == 0 && c->p == 0;
  if (!sepllm && !streaming) return SEP_ERR_PARAM;
  if (c->s > kMaxSepCache) return SEP_ERR_PARAM;
  if ((c->policy & ~(SEP_POLICY_DYNAMIC | SEP_POLICY_NO_ACCUM)) != 0) return SEP_ERR_PARAM;
  const bool dynamic = (c->policy & SEP_POLICY_DYNAMIC) != 0;
  const int64_t ring = static_cast<int64_t>(c->p) + c->w + (dynamic ? c->s : 0);
  if (dynamic && ring > SEP_MAX_DYN_RING) return SEP_ERR_PARAM;
  const int64_t slots = static_cast<int64_t>(c->a) + c->s + ring;
  if (slots > (1 << 24)) return SEP_ERR_SHAPE;
  return SEP_OK;
}

int check_cache_kv(const sep_cache* c) {
  if (c->k == nullptr || c->v == nullptr) return SEP_ERR_NULL;
  if (!aligned16(c->k) || !aligned16(c->v)) return SEP_ERR_ALIGN;
  if (c->work != nullptr && (reinterpret_cast<uintptr_t>(c->work) & 255) != 0) return SEP_ERR_WORKSPACE;
  return SEP_OK;
}

}  // namespace

extern "C" {

int sep_version(void) { return kVersion; }

const char* sep_status_string(int s) {
  switch (s) {
    case SEP_OK: return "ok";
    case SEP_ERR_NULL: return "a required pointer is NULL";
    case SEP_ERR_SHAPE: return "a size is out of range or inconsistent";
    case SEP_ERR_PARAM: return "a parameter breaks the Sep-Attention / cache contract";
    case SEP_ERR_DTYPE: return "dtype not supported by this entry point";
    case SEP_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case SEP_ERR_HIP: return "HIP launch failure";
    case SEP_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    default: return "unknown status";
  }
}

int sep_mask_build(const int32_t* ids, int B, int S, const int32_t* sep_ids, int n_sep_ids, int a,
                   int n, uint8_t* is_sep, uint8_t* tile_class, int tq, int tk,
                   uint8_t* dense_mask, hipStream_t stream) {
  if (ids == nullptr || is_sep == nullptr) return SEP_ERR_NULL;
  if (n_sep_ids < 0 || n_sep_ids > SEP_MAX_SEP_IDS) return SEP_ERR_SHAPE;
  if (n_sep_ids > 0 && sep_ids == nullptr) return SEP_ERR_NULL;
  if (B <= 0 || S <= 0) return SEP_ERR_SHAPE;
  if (a < 0 || n < 1) return SEP_ERR_PARAM;
  if (tile_class != nullptr && (tq < 1 || tk < 1 || tq > 4096 || tk > 4096)) return SEP_ERR_SHAPE;
  if (dense_mask != nullptr && S > SEP_MAX_DENSE_S) return SEP_ERR_SHAPE;
  if (!aligned16(ids)) return SEP_ERR_ALIGN;
  hipError_t e = sep::launch_is_sep(ids, static_cast<int64_t>(B) * S, sep_ids, n_sep_ids, is_sep,
                                    stream);
  if (e != hipSuccess) return SEP_ERR_HIP;
  if (tile_class != nullptr) {
    e = sep::launch_tile_class(is_sep, B, S, a, n, tq, tk, tile_class, stream);
    if (e != hipSuccess) return SEP_ERR_HIP;
  }
  if (dense_mask != nullptr) {
    e = sep::launch_dense_mask(is_sep, B, S, a, n, dense_mask, stream);
    if (e != hipSuccess) return SEP_ERR_HIP;
  }
  return SEP_OK;
}

int sep_index_compact(const uint8_t* is_sep, int B, int S, int32_t* rank, int32_t* sep_pos,
                      int32_t* count, hipStream_t stream) {
  if (is_sep == nullptr || rank == nullptr || sep_pos == nullptr) return SEP_ERR_NULL;
  if (B <= 0 || S <= 0) return SEP_ERR_SHAPE;
  return hip_status(sep::launch_index_compact(is_sep, B, S, rank, sep_pos, count, stream));
}

int sep_mask_compact(const int32_t* ids, int B, int S, const int32_t* sep_ids, int n_sep_ids, uint8_t* is_sep,
                     int32_t* rank, int32_t* sep_pos, int32_t* count, hipStream_t stream) {
  if (ids == nullptr || is_sep == nullptr || rank == nullptr || sep_pos == nullptr) return SEP_ERR_NULL;
  if (n_sep_ids < 0 || n_sep_ids > SEP_MAX_SEP_IDS) return SEP_ERR_SHAPE;
  if (n_sep_ids > 0 && sep_ids == nullptr) return SEP_ERR_NULL;
  if (B <= 0 || S <= 0) return SEP_ERR_SHAPE;
  if (!aligned16(ids) || !aligned16(is_sep) || !aligned16(rank)) return SEP_ERR_ALIGN;
  return hip_status(sep::launch_mask_compact(ids, B, S, sep_ids, n_sep_ids, is_sep, rank, sep_pos, count, stream));
}

int sep_attn_prefill(const void* q, const void* k, const void* v, int dtype, int B, int Hq, int Hkv,
                     int S, int D, const uint8_t* is_sep, const int32_t* rank,
                     const int32_t* sep_pos, int a, int n, float scale, void* out, float* lse,
                     hipStream_t stream) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return SEP_ERR_NULL;
  if (is_sep == nullptr || rank == nullptr || sep_pos == nullptr) return SEP_ERR_NULL;
  if (dtype != SEP_BF16 && dtype != SEP_F32) return SEP_ERR_DTYPE;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0) return SEP_ERR_SHAPE;
  if (Hq % Hkv != 0 || Hq / Hkv > 16) return SEP_ERR_SHAPE;
  if (D != 64 && D != 128) return SEP_ERR_SHAPE;
  if (a < 0 || n < 1) return SEP_ERR_PARAM;
  if (!(scale > 0.0f) || scale > 1e30f) return SEP_ERR_PARAM;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return SEP_ERR_ALIGN;
  return hip_status(sep::launch_prefill(q, k, v, dtype, B, Hq, Hkv, S, D, is_sep, rank, sep_pos, a,
                                        n, scale, out, lse, stream));
}

int sep_attn_prefill_backward(const void* q, const void* k, const void* v, const void* out,
                              const void* dout, const float* lse, int dtype, int B, int Hq, int Hkv,
                              int S, int D, const uint8_t* is_sep, const int32_t* rank,
                              const int32_t* sep_pos, int a, int n, float scale, float* delta,
                              float* dq, float* dk, float* dv, hipStream_t stream) {
  if (delta == nullptr) return SEP_ERR_NULL;
  const int st = sep::check_backward_args(q, k, v, out, dout, lse, dtype, B, Hq, Hkv, S, D, is_sep, rank, sep_pos,
                                          a, n, scale, dq, dk, dv);
  if (st != SEP_OK) return st;
  return hip_status(sep::launch_prefill_backward(q, k, v, out, dout, lse, dtype, B, Hq, Hkv, S, D, is_sep,
                                                 rank, sep_pos, a, n, scale, delta, dq, dk, dv, stream));
}

}  // extern "C"

namespace sep {

int check_backward_args(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* lse, int dtype, int B, int Hq, int Hkv, int S, int D, const uint8_t* is_sep,
                        const int32_t* rank, const int32_t* sep_pos, int a, int n, float scale, const float* dq,
                        const float* dk, const float* dv) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || dout == nullptr) return SEP_ERR_NULL;
  if (lse == nullptr || dq == nullptr || dk == nullptr || dv == nullptr) return SEP_ERR_NULL;
  if (is_sep == nullptr || rank == nullptr || sep_pos == nullptr) return SEP_ERR_NULL;
  if (dtype != SEP_BF16 && dtype != SEP_F32) return SEP_ERR_DTYPE;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0) return SEP_ERR_SHAPE;
  if (Hq % Hkv != 0 || Hq / Hkv > 16) return SEP_ERR_SHAPE;
  if (D != 64 && D != 128) return SEP_ERR_SHAPE;
  if (S > SEP_MAX_BACKWARD_S) return SEP_ERR_SHAPE;
  if (a < 0 || n < 1) return SEP_ERR_PARAM;
  if (!(scale > 0.0f) || scale > 1e30f) return SEP_ERR_PARAM;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return SEP_ERR_ALIGN;
  return SEP_OK;
}

}  // namespace sep

extern "C" {

int sep_cache_reset(const sep_cache* cache, hipStream_t stream) {
  const int st = check_cache(cache);
  if (st != SEP_OK) return st;
  return hip_status(sep::launch_cache_reset(*cache, stream));
}

int sep_cache_update(const sep_cache* cache, const void* k_new, const void* v_new,
                     const int32_t* ids_new, int T, const int32_t* sep_ids, int n_sep_ids,
                     hipStream_t stream) {
  int st = check_cache(cache);
  if (st != SEP_OK) return st;
  st = check_cache_kv(cache);
  if (st != SEP_OK) return st;
  if (k_new == nullptr || v_new == nullptr || ids_new == nullptr) return SEP_ERR_NULL;
  if (T < 1) return SEP_ERR_SHAPE;
  if (n_sep_ids < 0 || n_sep_ids > SEP_MAX_SEP_IDS) return SEP_ERR_SHAPE;
  if (n_sep_ids > 0 && sep_ids == nullptr) return SEP_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new)) return SEP_ERR_ALIGN;
  return hip_status(
      sep::launch_cache_update(*cache, k_new, v_new, ids_new, T, sep_ids, n_sep_ids, stream));
}

int sep_attn_decode(const void* q, const void* k_new, const void* v_new, const sep_cache* cache,
                    int Hq, float scale, void* out, float* lse, hipStream_t stream) {
  int st = check_cache(cache);
  if (st != SEP_OK) return st;
  st = check_cache_kv(cache);
  if (st != SEP_OK) return st;
  if (q == nullptr || k_new == nullptr || v_new == nullptr || out == nullptr) return SEP_ERR_NULL;
  if (cache->dtype != SEP_BF16) return SEP_ERR_DTYPE;
  if (Hq <= 0 || Hq % cache->Hkv != 0 || Hq / cache->Hkv > 16) return SEP_ERR_SHAPE;
  if (!(scale > 0.0f) || scale > 1e30f) return SEP_ERR_PARAM;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out))
    return SEP_ERR_ALIGN;
  return hip_status(sep::launch_decode(q, k_new, v_new, *cache, Hq, scale, nullptr, out, lse, stream));
}

size_t sep_decode_work_bytes(const sep_cache* cache, int Hq) {
  if (check_cache(cache) != SEP_OK || Hq <= 0 || Hq % cache->Hkv != 0 || Hq / cache->Hkv > 16) return 0;
  if (!sep::decode_may_split(*cache)) return 0;
  return sep::decode_split_bytes(*cache, Hq);
}

size_t sep_chunk_workspace_bytes(const sep_cache* cache, int C) {
  if (check_cache(cache) != SEP_OK || C < 1) return 0;
  return sep::chunk_workspace_bytes(*cache, C);
}

int sep_attn_prefill_chunk(const void* q, const void* k, const void* v, const int32_t* ids, int C,
                           const int32_t* sep_ids, int n_sep_ids, const sep_cache* cache, int Hq, int n,
                           float scale, void* workspace, size_t workspace_bytes, void* out, float* lse,
                           hipStream_t stream) {
  int st = check_cache(cache);
  if (st != SEP_OK) return st;
  st = check_cache_kv(cache);
  if (st != SEP_OK) return st;
  if (q == nullptr || k == nullptr || v == nullptr || ids == nullptr || out == nullptr) return SEP_ERR_NULL;
  if (n_sep_ids < 0 || n_sep_ids > SEP_MAX_SEP_IDS) return SEP_ERR_SHAPE;
  if (n_sep_ids > 0 && sep_ids == nullptr) return SEP_ERR_NULL;
  if (cache->dtype != SEP_BF16) return SEP_ERR_DTYPE;
  if (C < 1) return SEP_ERR_SHAPE;
  if (Hq <= 0 || Hq % cache->Hkv != 0 || Hq / cache->Hkv > 16) return SEP_ERR_SHAPE;
  if (static_cast<int64_t>(sep::cache_slots(*cache)) + C > (1 << 24)) return SEP_ERR_SHAPE;
  if (n < 1) return SEP_ERR_PARAM;
  if (!(scale > 0.0f) || scale > 1e30f) return SEP_ERR_PARAM;
  if (workspace == nullptr || workspace_bytes < sep::chunk_workspace_bytes(*cache, C) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return SEP_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return SEP_ERR_ALIGN;
  return hip_status(sep::launch_prefill_chunk(q, k, v, ids, C, sep_ids, n_sep_ids, *cache, Hq, n, scale,
                                              workspace, out, lse, stream));
}

int sep_rope_table(double base, int D, int n_pos, float* table, hipStream_t stream) {
  if (table == nullptr) return SEP_ERR_NULL;
  if (D != 64 && D != 128) return SEP_ERR_SHAPE;
  if (n_pos < 1) return SEP_ERR_SHAPE;
  if (!(base > 1.0) || !(base < 1e300)) return SEP_ERR_PARAM;
  if (!aligned16(table)) return SEP_ERR_ALIGN;
  return hip_status(sep::launch_rope_table(base, D, n_pos, table, stream));
}

int sep_attn_decode_rope(const void* q, const void* k_new, const void* v_new, const sep_cache* cache,
                         int Hq, float scale, const float* rope, int rope_npos, void* out, float* lse,
                         hipStream_t stream) {
  int st = check_cache(cache);
  if (st != SEP_OK) return st;
  st = check_cache_kv(cache);
  if (st != SEP_OK) return st;
  if (q == nullptr || k_new == nullptr || v_new == nullptr || out == nullptr || rope == nullptr)
    return SEP_ERR_NULL;
  if (cache->dtype != SEP_BF16) return SEP_ERR_DTYPE;
  if (Hq <= 0 || Hq % cache->Hkv != 0 || Hq / cache->Hkv > 16) return SEP_ERR_SHAPE;
  if (!(scale > 0.0f) || scale > 1e30f) return SEP_ERR_PARAM;
  if (rope_npos < sep::cache_slots(*cache) + 1) return SEP_ERR_PARAM;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out) || !aligned16(rope))
    return SEP_ERR_ALIGN;
  return hip_status(sep::launch_decode(q, k_new, v_new, *cache, Hq, scale, rope, out, lse, stream));
}

int sep_decode_update(const void* q, const void* k_new, const void* v_new, const int32_t* ids_new,
                      const int32_t* sep_ids, int n_sep_ids, const sep_cache* cache, int Hq, float scale,
                      const float* rope, int rope_npos, void* out, float* lse, hipStream_t stream) {
  int st = check_cache(cache);
  if (st != SEP_OK) return st;
  st = check_cache_kv(cache);
  if (st != SEP_OK) return st;
  if (q == nullptr || k_new == nullptr || v_new == nullptr || ids_new == nullptr || out == nullptr)
    return SEP_ERR_NULL;
  if (n_sep_ids < 0 || n_sep_ids > SEP_MAX_SEP_IDS) return SEP_ERR_SHAPE;
  if (n_sep_ids > 0 && sep_ids == nullptr) return SEP_ERR_NULL;
  if (cache->dtype != SEP_BF16) return SEP_ERR_DTYPE;
  if (Hq <= 0 || Hq % cache->Hkv != 0 || Hq / cache->Hkv > 16) return SEP_ERR_SHAPE;
  if (!(scale > 0.0f) || scale > 1e30f) return SEP_ERR_PARAM;
  if (rope != nullptr && rope_npos < sep::cache_slots(*cache) + 1) return SEP_ERR_PARAM;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out) ||
      (rope != nullptr && !aligned16(rope)))
    return SEP_ERR_ALIGN;
  return hip_status(sep::launch_decode_update(q, k_new, v_new, ids_new, sep_ids, n_sep_ids, *cache, Hq, scale,
                                              rope, out, lse, stream));
}

}  // extern "C"
