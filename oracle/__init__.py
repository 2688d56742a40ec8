"""Plain CPU oracle of the Sep-Attention hot path (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or run anything in this package. The product
path (``kv_cache_compression_sep_amd``) never does; it shares no code,
table or helper with this package, and neither imports the other.

Everything here is slow, direct and fp64 (or exact integer) NumPy, written
from the SepLLM pages. Citations use these tags:

  P1  "HKUDS047: SepLLM 作为 Long-Context Compression、KV Cache Efficiency 与
       Research OS Memory Compression Layer" (pengpengyi92.github.io), study
       notes on the SepLLM code: sections "核心机制" (Initial Tokens,
       Separator Tokens, Local Window), "SepCache", "Streaming-SepLLM",
       "KV Cache Manager", "Streaming 参数约束", "SepAttention",
       "Flex Attention Kernel".
  P2  SepLLM explainer at jieyibu.net/a/61556: §1.2 "Sep-Attention核心算法解析"
       (mask matrix M, masked scaled softmax) and §1.3 "动态KV缓存管理策略"
       (the four cache blocks).
  P3  "用句号提速大模型？华为新算法SepLLM让AI推理快50%！" (xugj520.cn):
       §3.1 (which tokens are kept) and §3.3 (the four-block eviction table).

Modules:
  mask.py       separator flags, the 0/1 mask M, prefix-sum compaction,
                tile classes.
  attention.py  dense masked softmax attention (prefill), its gradients,
                attention over an explicit key list (decode) and of a chunk
                of new tokens over a live cache.
  cache.py      list-based simulation of the four-block cache, and the
                closed form of its state.
  rope.py       rotary position embedding and the position shifting of
                streaming decode (keys re-indexed by their place in the
                cache).

Every function is pinned by tests under ``tests/`` marked "not gpu"
(brute force on tiny inputs, special cases that reduce to textbook or
library routines, invariants and a closed form). No function here is
"parity unpinned".
"""
from .mask import (is_sep, sep_mask, mask_rows, compact, tile_class,  # noqa: F401
                   tile_class_slabs)
from .attention import (attention, attention_backward, attention_backward_sampled, attention_rows,  # noqa: F401
                        chunk_attention, decode_attention)
from .rope import decode_attention_shifted, rope_angles, rotate, round_bf16  # noqa: F401
from .cache import (CacheSim, Entry, closed_form_positions, check_cache_params,  # noqa: F401
                    n_compactions, policy_positions)
