"""CPU float64 oracle for selectively-read decode attention over a paged KV cache.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The product library (``sparse_kv_recall_amd``) never imports it and
shares no code with it: no kernels, headers, helpers, tables or constants.

Every function here is the plain definition of what the decode path computes,
written in float64 from the sources below, without blocking, fusion or
reordering beyond what the definition itself states:

* "On-Demand Attention: Language Models Know When to Recall" (arxiv-wiki
  summary page): the local-first view with s sink tokens and a recent window
  of w tokens that includes the current token, the recall head
  R(h_{t-1}, E(x_t), h^L_t) -> q_t, the gate q_t > theta, recomputation of the
  current step with full attention, and commit of the selected pass's
  current-position KV ("Approach" section; the Local setting in "Main
  results"; the Local/full-view runtime and FP32 recall head in "Developer
  perspective").
* "[Paper review] Language Models Can Control Their Own Attention" (blog
  review of Declarative Attention), section 3 "Method & Key Results": the
  mask is applied at KV-block granularity by rewriting the block table so the
  attention kernel sees only kept blocks; the global / focus / local modes of
  section 1 "Key Terms" and of the chatpaper abstract page.

Parity status of each function (pinned by the ``-m "not gpu"`` tests):

* keysets.full_keys / local_keys / block_keys ......... pinned
* attention.attend ..................................... pinned
* recall.recall_score / recall.gate .................... pinned
* gather.gather_blocks / gather.da_mode_blocks ......... pinned
* bf16.f64_to_bf16_bits ................................ pinned (hand values,
  ties to even, identity on bf16 values, monotone)
* decoder.rms_norm / rope / silu ....................... pinned (closed forms,
  textbook RoPE values, norm and relative-position invariants)
* decoder.Decoder (layer, forward, oda_step) ........... pinned by invariants
  (zero weights keep the residual stream; Local = Full within s + w; the
  recall pass's own commits from layer 1 on); the layer structure is the
  published Qwen3-family layer, not the pages' (they give none)
* declare.parse_declarations ........................... pinned by a hand-worked
  token stream (the pages print none) and by an independent backward-scan
  formulation on seeded streams
* oda.local_pass / full_pass / blocks_pass / recall_pass / select / request_mode
  ...................................................... pinned by definition only
  (the pages print no worked example of a stack step; the commit, select and
  per-layer access rules are checked against their restatement, perturbation
  invariants and the Local = Full identity within s + w)
* cost.* (attention-only) .............................. pinned (golden ratio,
  closed forms)
* cost.DenseShape / decode_flops_ratio / decode_bytes_ratio  pinned to the pages'
  whole-model 24.26 % to within 0.1 point, under one reading: Qwen3-1.7B's
  dense sizes (MLP 6144, vocabulary 151936, tied embeddings) are the model's
  published configuration, not the pages'; also pinned by a loop count of a
  tiny decoder and by the exact reduction to the attention-only ratio.
"""

from . import attention, cost, declare, decoder, gather, keysets, oda, recall  # noqa: F401
from .bf16 import bf16_bits_to_f64, f64_to_bf16_bits  # noqa: F401
