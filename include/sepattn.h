/*
 * sepattn.h - C ABI of the Sep-Attention hot path for AMD Instinct MI355X (gfx950).
 *
 * Sep-Attention (SepLLM): a causal query i attends key j only when j is one of
 * the first `a` tokens (initial tokens), or j is among the `n` most recent
 * positions (0 <= i - j < n, the neighbouring window), or token j is a
 * separator, i.e. its id belongs to a given separator id set. Streaming
 * inference keeps a four-block KV cache (initial / separator / past window /
 * local window) and compacts the overflowing past window down to its
 * separators.
 *
 * Sources (web pages on SepLLM):
 *   [P1] "HKUDS047: SepLLM 作为 Long-Context Compression、KV Cache Efficiency 与
 *        Research OS Memory Compression Layer" - sections "核心机制",
 *        "SepCache", "Streaming-SepLLM", "KV Cache Manager",
 *        "Streaming 参数约束", "SepAttention", "Flex Attention Kernel".
 *   [P2] jieyibu.net SepLLM explainer - §1.2 (mask matrix, masked scaled
 *        softmax) and §1.3 (the four cache blocks).
 *   [P3] "用句号提速大模型？华为新算法SepLLM让AI推理快50%！" - §3.1 (kept
 *        tokens) and §3.3 (four-block eviction table).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never allocates, frees or synchronises, and keeps no mutable
 *     global state. Tensors are dense, row-major, in the layouts stated, and
 *     16-byte aligned.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *     the null stream). Calls on one stream execute in order.
 *   - Arguments are validated on the host before anything is launched. An
 *     invalid argument returns a negative sep_status and enqueues nothing.
 *     After enqueueing, a failed launch returns SEP_ERR_HIP. No exceptions
 *     cross this boundary and nothing calls exit().
 *   - Valid inputs cannot fail on the device: ids outside every separator
 *     set are simply not separators.
 *   - Names follow the pages: a = init_cache_size (= init_tok_max_idx + 1),
 *     n = prefill/generate_local_window_size, s = sep_cache_size,
 *     w = local_size, c = cache_size = a + s + p + w, with p the past window.
 */
#ifndef SEPATTN_H
#define SEPATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SEP_OK = 0,
  SEP_ERR_NULL = -1,      /* a required pointer is NULL                    */
  SEP_ERR_SHAPE = -2,     /* a size is out of range or inconsistent        */
  SEP_ERR_PARAM = -3,     /* a, n, s, p, w, scale break the contract       */
  SEP_ERR_DTYPE = -4,     /* dtype not supported by this entry point       */
  SEP_ERR_WORKSPACE = -5, /* reserved                                       */
  SEP_ERR_HIP = -6,       /* the HIP runtime reported a launch failure     */
  SEP_ERR_ALIGN = -7      /* a tensor pointer is not 16-byte aligned       */
} sep_status;

typedef enum { SEP_F32 = 0, SEP_BF16 = 1 } sep_dtype;

/* Largest separator set accepted (ids are compared one by one). */
#define SEP_MAX_SEP_IDS 64
/* Largest S for which sep_mask_build writes the dense mask. */
#define SEP_MAX_DENSE_S 8192

/*
 * sep_mask_build - separator flags, block classes and (optionally) the dense
 * 0/1 mask of each sequence.  [P1 "Separator Tokens", "SepAttention"
 * (build_prefill_mask); P2 §1.2 (mask matrix M); P1 "Flex Attention Kernel"
 * (block-sparse map, the role of create_block_mask)]
 *
 *   ids        [B, S] int32   token ids.
 *   sep_ids    [n_sep_ids] int32 device array, 0 <= n_sep_ids <= 64
 *              (NULL allowed when n_sep_ids == 0; duplicates allowed).
 *   a, n       initial-token count (a >= 0) and window (n >= 1).
 *   is_sep     [B, S] uint8 out (required): 1 iff ids[b,j] is in sep_ids.
 *   tile_class [B, ceil(S/tq), ceil(S/tk)] uint8 out, or NULL: for each
 *              block of tq query rows x tk key columns, 0 = no pair visible,
 *              1 = every pair visible, 2 = mixed. Edge blocks count only
 *              rows/columns < S. tq, tk in [1, 4096] when tile_class != NULL.
 *   dense_mask [B, S, S] uint8 out, or NULL: M[b,i,j] = 1 iff j <= i and
 *              (j < a or i - j < n or is_sep[b,j]). Requires S <= 8192.
 * Returns SEP_OK, SEP_ERR_NULL, SEP_ERR_SHAPE, SEP_ERR_PARAM, SEP_ERR_HIP.
 */
int sep_mask_build(const int32_t* ids, int B, int S, const int32_t* sep_ids, int n_sep_ids,
                   int a, int n, uint8_t* is_sep, uint8_t* tile_class, int tq, int tk,
                   uint8_t* dense_mask, hipStream_t stream);

/*
 * sep_index_compact - prefix-sum stream compaction of the separator flags.
 * [P1 "KV Cache Manager" (compress_past_win_2_seps keeps the separator
 * entries of a window, in order); P3 §3.3 (the past window keeps only its
 * separators)]
 *
 *   is_sep  [B, S] uint8 (0/1; any non-zero byte counts as 1).
 *   rank    [B, S+1] int32 out: rank[b,j] = number of separators at
 *           positions < j; rank[b,S] is the separator count.
 *   sep_pos [B, S] int32 out: sep_pos[b,r] = position of the r-th separator
 *           in increasing order for r < count; -1 for r >= count.
 *   count   [B] int32 out, or NULL.
 * Returns SEP_OK, SEP_ERR_NULL, SEP_ERR_SHAPE, SEP_ERR_HIP.
 */
int sep_index_compact(const uint8_t* is_sep, int B, int S, int32_t* rank, int32_t* sep_pos,
                      int32_t* count, hipStream_t stream);

/*
 * sep_mask_compact - the separator flags of sep_mask_build and the
 * compaction of sep_index_compact in one launch (one workgroup per
 * sequence), for callers that need no tile classes or dense mask.
 * [as sep_mask_build and sep_index_compact]
 *
 *   ids [B, S] int32; sep_ids [n_sep_ids] int32 device array (0..64 ids).
 *   is_sep [B, S] uint8 out; rank [B, S+1], sep_pos [B, S] int32 out; count
 *   [B] int32 out or NULL: exactly what sep_mask_build (flags only) then
 *   sep_index_compact write. ids, is_sep and rank 16-byte aligned.
 * Returns SEP_OK, SEP_ERR_NULL, SEP_ERR_SHAPE, SEP_ERR_ALIGN, SEP_ERR_HIP.
 */
int sep_mask_compact(const int32_t* ids, int B, int S, const int32_t* sep_ids, int n_sep_ids, uint8_t* is_sep,
                     int32_t* rank, int32_t* sep_pos, int32_t* count, hipStream_t stream);

/*
 * sep_attn_prefill - Sep-Attention over a whole sequence.  [P2 §1.2 (scores
 * scaled, masked entries set to -inf, softmax, weighted sum of V); P1
 * "SepAttention" (initial OR window OR separator, AND causal); P1
 * "Flex Attention Kernel" (only a kernel that sees the sparsity saves work)]
 *
 *   q        [B, Hq, S, D]; k, v [B, Hkv, S, D]; dtype SEP_BF16 or SEP_F32
 *            (the same for q, k, v and out). Query head h reads key/value
 *            head h / (Hq / Hkv). Hq % Hkv == 0, Hq / Hkv <= 16, D in {64, 128}.
 *   is_sep   [B, S] uint8 from sep_mask_build.
 *   rank     [B, S+1], sep_pos [B, S] int32 from sep_index_compact on the
 *            same is_sep.
 *   a >= 0, n >= 1; scale > 0 multiplies q.k (1/sqrt(D) is the usual value).
 *   out      [B, Hq, S, D] out, same dtype as q.
 *   lse      [B, Hq, S] float32 out, or NULL: natural-log softmax
 *            normaliser (row max + log of the row sum of exponentials).
 * Arithmetic: fp32 accumulation and online softmax; in bf16 mode the
 * softmax weights are rounded to bf16 for the P.V product.
 * Returns SEP_OK, SEP_ERR_NULL, SEP_ERR_SHAPE, SEP_ERR_PARAM, SEP_ERR_DTYPE,
 * SEP_ERR_ALIGN, SEP_ERR_HIP.
 */
int sep_attn_prefill(const void* q, const void* k, const void* v, int dtype, int B, int Hq,
                     int Hkv, int S, int D, const uint8_t* is_sep, const int32_t* rank,
                     const int32_t* sep_pos, int a, int n, float scale, void* out, float* lse,
                     hipStream_t stream);

/*
 * sep_attn_prefill_backward - gradients of sep_attn_prefill.
 * [P2 §1.2 (scaled masked softmax attention); P1 "Training-SepLLM" (training
 * runs through the same Sep-Attention mask)]
 *
 * For L = sum(dout * out): dq = dL/dq, dk = dL/dk, dv = dL/dv, with the
 * same mask and scale as the forward (see sep_attn_prefill):
 *   delta_i = sum_d dout_id out_id;  P = softmax weights, recomputed as
 *   exp(scale q_i.k_j - lse_i) on visible pairs;  dP = dout V^T;
 *   dS = P * (dP - delta);  dq = scale dS K;  dk_g = scale sum over the
 *   query heads h of group g of dS_h^T Q_h;  dv_g = sum_h P_h^T dout_h.
 *   q, out, dout [B, Hq, S, D] and k, v [B, Hkv, S, D] in `dtype`; lse
 *          [B, Hq, S] float32 as written by sep_attn_prefill (natural log);
 *   is_sep, rank, sep_pos as for sep_attn_prefill.
 *   delta  [B, Hq, S] float32 workspace, overwritten.
 *   dq     [B, Hq, S, D] float32 out; dk, dv [B, Hkv, S, D] float32 out
 *          (written, not accumulated).
 * Shapes as for sep_attn_prefill, and S <= SEP_MAX_BACKWARD_S.
 * Arithmetic, by dtype:
 *   SEP_F32   products on the fp32 MFMA; every operand, P, dP, dS and
 *             accumulator in fp32.
 *   SEP_BF16  products on the bf16 MFMA with fp32 accumulation: q, k, v,
 *             dout enter as bf16 (exactly); scores, P, dP and dS are
 *             computed in fp32, and P (for dv) and dS (for dq, dk) are
 *             rounded to bf16 (round to nearest even) before their products.
 *   Each element of dq, dk, dv lies within (e^d - 1 + r + g) * A of the
 *   exact gradient, where A is the same sum taken over absolute values, d
 *   the forward's log-sum-exp error (4e-3 bf16, 1e-5 fp32), r = 2^-8 for
 *   bf16 (its unit roundoff; 0 for fp32) and g = m u / (1 - m u) with u = 2^-24 and m = D + G S
 *   (G = Hq / Hkv): the bound the parity tests apply.
 * dk and dv of initial and separator keys are summed with fp32 atomics, so
 * their summation order varies between runs.
 * Returns SEP_OK, SEP_ERR_NULL, SEP_ERR_SHAPE, SEP_ERR_PARAM, SEP_ERR_DTYPE,
 * SEP_ERR_ALIGN, SEP_ERR_HIP.
 */
#define SEP_MAX_BACKWARD_S 2097152
int sep_attn_prefill_backward(const void* q, const void* k, const void* v, const void* out,
                              const void* dout, const float* lse, int dtype, int B, int Hq, int Hkv,
                              int S, int D, const uint8_t* is_sep, const int32_t* rank,
                              const int32_t* sep_pos, int a, int n, float scale, float* delta,
                              float* dq, float* dk, float* dv, hipStream_t stream);

/*
 * Cache policies (bits of sep_cache.policy) [P1 "KV Cache Manager": the
 * compression pseudo-code and its SEP_ACCUMULATION / USE_MAX_SEP_CACHE
 * switches].
 *   0                    fixed caps: R is compressed when it would hold
 *                        p + w + 1 entries.
 *   SEP_POLICY_DYNAMIC   the pseudo-code's trigger: R is compressed when
 *                        the whole cache (I + S + R) would hold more than
 *                        c = a + s + p + w entries; while S is not full R
 *                        grows past p + w (its ring has s + p + w slots).
 *   SEP_POLICY_NO_ACCUM  SEP_ACCUMULATION off: a compression replaces S by
 *                        the separators of the compressed entries.
 * Either way a compression takes R minus its last w entries (under fixed
 * caps exactly its oldest p + 1), and S keeps its last s separators
 * (USE_MAX_SEP_CACHE on; an unbounded S has no fixed-size form and is not
 * offered). Under SEP_POLICY_DYNAMIC, s + p + w <= SEP_MAX_DYN_RING.
 */
#define SEP_POLICY_DYNAMIC 1
#define SEP_POLICY_NO_ACCUM 2
#define SEP_MAX_DYN_RING 32768

/*
 * sep_cache - a batch of four-block KV caches in caller-owned device memory.
 * [P2 §1.3 and P3 §3.3 (initial / separator / past window / local window);
 * P1 "SepCache" (parameter names)]
 *
 * Slot layout per sequence, with the recent-ring size r = p + w (fixed
 * caps) or s + p + w (SEP_POLICY_DYNAMIC) and nslots = a + s + r:
 *   [0, a)          initial block: position x < a lives in slot x.
 *   [a, a+s)        separator ring (FIFO, cap s).
 *   [a+s, nslots)   recent ring R = past window ++ local window:
 *                   position x >= a lives in slot a + s + (x - a) mod r.
 * Device arrays:
 *   k, v   [B, Hkv, nslots, D] in `dtype`.
 *   pos    [B, nslots] int32: absolute position held by each slot, -1 if
 *          empty. Positions are below 2^31.
 *   tok    [B, nslots] int32: token id held by each slot, -1 if empty.
 *   state  [B, 8] int64 per sequence:
 *          [0] n_seen        tokens inserted so far (t);
 *          [1] n_compacted   entries taken out of R so far: the compacted
 *                            prefix is [a, a + n_compacted) and R holds
 *                            positions [a + n_compacted, t) (fixed caps:
 *                            n_compacted = K (p + 1) after K compressions);
 *          [2] sep_head      separator-ring slot the next separator takes;
 *          [3] sep_count     separators held (<= s);
 *          [4] n_compacted before the last sep_cache_update call;
 *          [5..6] reserved, 0;
 *          [7] arrival count of sep_decode_update, 0 between calls.
 *          The ring's entries, oldest first, are the slots
 *          a + (sep_head - sep_count + i) mod s, i = 0 .. sep_count-1.
 *   work   device work buffer of work_bytes bytes (256-byte aligned), or
 *          NULL. With few (sequence, kv head) pairs (B * Hkv <= 64) and
 *          work_bytes >= sep_decode_work_bytes(cache, Hq), the decode calls
 *          (sep_attn_decode, sep_attn_decode_rope, sep_decode_update) split
 *          each list over several workgroups and keep their partial results
 *          here; otherwise one workgroup reads each list and work is unused.
 *          Either way the result of a given (cache, Hq) is deterministic,
 *          and the three calls agree bit for bit. Decode calls that share a
 *          work buffer must not overlap.
 * An empty cache is state all zero and pos/tok all -1 (sep_cache_reset).
 * K/V rows of empty slots are never read.
 * Contract [P1 "Streaming 参数约束"]: a >= 0, w >= 1, and either s >= 1 and
 * p >= 1 (SepLLM: a + s + w < c) or s == 0 and p == 0 (StreamingLLM: the
 * local window is c - a); policy is a combination of the bits above.
 */
typedef struct {
  int32_t a, s, p, w;
  int32_t B, Hkv, D, dtype;
  void* k;
  void* v;
  int32_t* pos;
  int32_t* tok;
  int64_t* state;
  int32_t policy;
  void* work;
  size_t work_bytes;
} sep_cache;

/*
 * sep_decode_work_bytes - the work buffer (sep_cache.work) the decode calls
 * need to split their lists for Hq query heads: 0 when they never split
 * (B * Hkv > 64) or the cache is invalid. Split decode [P2 §1.3, only the
 * retained KV are read: more workgroups read each list at once].
 */
size_t sep_decode_work_bytes(const sep_cache* cache, int Hq);

/*
 * sep_cache_reset - make every sequence of the cache empty (state = 0,
 * pos = tok = -1). K/V contents are left as they are.
 * Returns SEP_OK, SEP_ERR_NULL, SEP_ERR_SHAPE, SEP_ERR_PARAM, SEP_ERR_HIP.
 */
int sep_cache_reset(const sep_cache* cache, hipStream_t stream);

/*
 * sep_cache_update - append T tokens to every sequence of the cache.
 * [P1 "KV Cache Manager" (compress_past_win_2_seps, keep the last
 * sep_cache_size separators, K/V and token ids move together); P3 §3.3
 * (initial fixed; local window overflows into the past window; a full past
 * window keeps its separators and drops the rest; the separator cache
 * evicts its oldest entry beyond s)]
 *
 *   k_new, v_new [B, Hkv, T, D] in cache->dtype; ids_new [B, T] int32.
 *   sep_ids [n_sep_ids] int32 device array (0..64 ids).
 * Rule, per token (positions t = n_seen, n_seen+1, ...): if fewer than a
 * tokens are held in the initial block, the token goes there. Otherwise it
 * joins R; when the policy's trigger fires (fixed caps: R would hold
 * p + w + 1 entries; SEP_POLICY_DYNAMIC: the cache would hold more than c),
 * R minus its last w entries is compressed first: under SEP_POLICY_NO_ACCUM
 * the separator ring is emptied (its next entry takes slot a, sep_head 0);
 * then each separator among the compressed
 * entries, oldest first, is copied into the separator ring (overwriting the
 * oldest entry once the ring holds s); the rest are dropped. T > 1 gives
 * exactly the state of T calls with T = 1.
 * Returns SEP_OK, SEP_ERR_NULL, SEP_ERR_SHAPE, SEP_ERR_PARAM, SEP_ERR_DTYPE,
 * SEP_ERR_ALIGN, SEP_ERR_HIP.
 */
int sep_cache_update(const sep_cache* cache, const void* k_new, const void* v_new,
                     const int32_t* ids_new, int T, const int32_t* sep_ids, int n_sep_ids,
                     hipStream_t stream);

/*
 * sep_attn_decode - one decode step of Sep-Attention over the cache.
 * [P1 "SepAttention" (build_generate_mask: the same keep rule for one query);
 * P1 "Streaming-SepLLM" (each token: forward with the cache, then update
 * and compress); P2 §1.3 (only the retained KV are read)]
 *
 *   q      [B, Hq, D] in cache->dtype (SEP_BF16 only); Hq % Hkv == 0 and
 *          Hq / Hkv <= 16; query head h reads kv head h / (Hq / Hkv).
 *   k_new, v_new [B, Hkv, D]: the current token's key/value. It attends the
 *          cache as it is (tokens before it) plus itself; call
 *          sep_cache_update afterwards to insert it.
 *   scale  > 0; out [B, Hq, D] (bf16); lse [B, Hq] float32 out or NULL.
 * Reads the cache, never writes its blocks or state (only, in split mode,
 * the work buffer; see sep_cache).
 * Returns SEP_OK, SEP_ERR_NULL, SEP_ERR_SHAPE, SEP_ERR_PARAM, SEP_ERR_DTYPE,
 * SEP_ERR_ALIGN, SEP_ERR_HIP.
 */
int sep_attn_decode(const void* q, const void* k_new, const void* v_new, const sep_cache* cache,
                    int Hq, float scale, void* out, float* lse, hipStream_t stream);

/*
 * sep_attn_prefill_chunk - a chunk of C new tokens attends the live cache
 * and itself (chunked prefill into a cache).
 * [P1 "SepAttention" (build_generate_mask: the prefill keep rule applied to
 * the rows of new queries; a generation window, and a window per layer);
 * P2 §1.3 (only the retained KV are read)]
 *
 *   q      [B, Hq, C, D]; k, v [B, Hkv, C, D] in cache->dtype (SEP_BF16
 *          only); ids [B, C] int32: the chunk of each sequence, at
 *          positions t .. t+C-1, t = its state word 0.
 *   sep_ids [n_sep_ids] int32 device array (0..64 ids), as for
 *          sep_cache_update.
 *   n      >= 1: this call's window (the layer's generation window).
 * Query tau = t + i sees a retained entry or chunk key at position p iff
 * p <= tau and (p < a, or its token id is a separator, or tau - p < n).
 * With C = 1 and n at least the cache's slot count this is sep_attn_decode.
 * The cache is read, not written: insert the chunk afterwards with
 * sep_cache_update(cache, k, v, ids, C, ...).
 *   workspace  device memory of at least sep_chunk_workspace_bytes(cache, C)
 *          bytes, 256-byte aligned, overwritten (the keys laid out as one
 *          sequence per kv head, with flags and their compaction).
 *   scale  > 0; out [B, Hq, C, D] (bf16); lse [B, Hq, C] float32 or NULL.
 * Returns SEP_OK, SEP_ERR_NULL, SEP_ERR_SHAPE, SEP_ERR_PARAM, SEP_ERR_DTYPE,
 * SEP_ERR_ALIGN, SEP_ERR_WORKSPACE, SEP_ERR_HIP.
 */
size_t sep_chunk_workspace_bytes(const sep_cache* cache, int C);
int sep_attn_prefill_chunk(const void* q, const void* k, const void* v, const int32_t* ids, int C,
                           const int32_t* sep_ids, int n_sep_ids, const sep_cache* cache, int Hq, int n,
                           float scale, void* workspace, size_t workspace_bytes, void* out, float* lse,
                           hipStream_t stream);

/*
 * sep_rope_table - cos/sin table of rotary position embedding.
 * [P1 "Streaming-SepLLM": streaming needs positional-encoding shifting (the
 * Llama pos_shift module); RoPE as published: Su et al., RoFormer, §3.4]
 *
 *   table  [n_pos, D/2, 2] float32 out: table[p][i] = (cos(p theta_i),
 *          sin(p theta_i)), theta_i = base^(-2 i / D), evaluated in fp64 and
 *          rounded once to fp32. 16-byte aligned.
 *   base   > 1 (500000 for Llama 3); D in {64, 128}; n_pos >= 1.
 * Build it once per (base, D) and cache size; sep_attn_decode_rope reads it.
 * Returns SEP_OK, SEP_ERR_NULL, SEP_ERR_SHAPE, SEP_ERR_PARAM, SEP_ERR_ALIGN,
 * SEP_ERR_HIP.
 */
int sep_rope_table(double base, int D, int n_pos, float* table, hipStream_t stream);

/*
 * sep_attn_decode_rope - sep_attn_decode with rotary position embedding and
 * position shifting.
 * [P1 "Streaming-SepLLM" and "Streaming 不是普通评测入口" (streaming needs
 * positional-encoding shifting); RoFormer §3.4 for the rotation]
 *
 * The cache holds keys before rotation (as k_new is passed: unrotated), so
 * positions are assigned at read time: the retained entries take positions
 * 0 .. L-1 in cache order (initial block, then the separator ring oldest
 * first, then the recent ring oldest first) and the current token, query
 * and key, takes position L. Pair i of a head vector is (x_i, x_{i+D/2})
 * (Llama's arrangement), rotated by p theta_i. The rotated query and keys
 * are rounded to bf16 (round to nearest even) before the products; values
 * are not rotated.
 *   q, k_new, v_new, cache, Hq, scale, out, lse as for sep_attn_decode.
 *   rope   sep_rope_table output for D = cache->D with rope_npos rows;
 *          rope_npos >= (cache slots) + 1 = a + s + ring + 1, where ring is
 *          p + w, or s + p + w under SEP_POLICY_DYNAMIC. 16-byte aligned.
 * Returns SEP_OK, SEP_ERR_NULL, SEP_ERR_SHAPE, SEP_ERR_PARAM, SEP_ERR_DTYPE,
 * SEP_ERR_ALIGN, SEP_ERR_HIP.
 */
int sep_attn_decode_rope(const void* q, const void* k_new, const void* v_new, const sep_cache* cache,
                         int Hq, float scale, const float* rope, int rope_npos, void* out, float* lse,
                         hipStream_t stream);

/* Static description of a status code. */
const char* sep_status_string(int status);

/* Library version, as major*10000 + minor*100 + patch. */
int sep_version(void);

/*
 * sep_decode_update - one streaming step: sep_attn_decode (or, with rope,
 * sep_attn_decode_rope) of the new token, then sep_cache_update of that
 * token (T = 1), in one call.
 * [P1 "Streaming-SepLLM" (each step: the forward with the cache, then the
 * cache update); P2 §1.3; P3 §3.3]
 *
 * Arguments are those of the two calls: q [B, Hq, D], k_new / v_new
 * [B, Hkv, D] in cache->dtype (SEP_BF16 only), ids_new [B] int32, sep_ids
 * [n_sep_ids] int32, scale > 0, rope NULL (plain decode) or the table of
 * sep_rope_table with rope_npos >= slots + 1 rows, out [B, Hq, D] bf16, lse
 * [B, Hq] float32 or NULL. The result (out, lse, and the cache's K/V, pos,
 * tok and state) equals the two calls in that order, bit for bit.
 * When B * Hkv < 256 and the separator ring holds at most 4096 entries it
 * is one launch (each sequence's last kv-head workgroup to finish its decode
 * runs the update, counting arrivals in state word 7, which is 0 between
 * calls); otherwise it is the two launches. Calls on one cache must not
 * overlap.
 * Returns SEP_OK, SEP_ERR_NULL, SEP_ERR_SHAPE, SEP_ERR_PARAM, SEP_ERR_DTYPE,
 * SEP_ERR_ALIGN, SEP_ERR_HIP.
 */
int sep_decode_update(const void* q, const void* k_new, const void* v_new, const int32_t* ids_new,
                      const int32_t* sep_ids, int n_sep_ids, const sep_cache* cache, int Hq, float scale,
                      const float* rope, int rope_npos, void* out, float* lse, hipStream_t stream);

/*
 * sep_attn_prefill_backward_noalloc - sep_attn_prefill_backward without the
 * delta workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops that forbid hipMalloc).
 *
 * Arguments, results, arithmetic and status codes are those of
 * sep_attn_prefill_backward. The per-row sums delta live instead in a fixed
 * device array inside the library (one copy per GPU, held until the process
 * ends) of SEP_NOALLOC_MAX_ROWS floats (16 MiB): B * Hq * S must not exceed
 * SEP_NOALLOC_MAX_ROWS, else SEP_ERR_WORKSPACE and nothing is launched. The
 * array's address is looked up on the first call from each device, which
 * must be the calling thread's current device and the device of `stream`.
 * Nothing is allocated or freed, by this call or by any call it makes.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (concurrent streams, or threads) race on it and must be serialised by
 * the caller. The array holds no state between calls (delta is rewritten in
 * full before it is read).
 */
#define SEP_NOALLOC_MAX_ROWS (1 << 22)
int sep_attn_prefill_backward_noalloc(const void* q, const void* k, const void* v, const void* out,
                                      const void* dout, const float* lse, int dtype, int B, int Hq, int Hkv,
                                      int S, int D, const uint8_t* is_sep, const int32_t* rank,
                                      const int32_t* sep_pos, int a, int n, float scale, float* dq, float* dk,
                                      float* dv, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SEPATTN_H */
