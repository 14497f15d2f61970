"""MI355X-native decode-phase paged attention.

The operations sit behind a C-ABI shared library (``libpkv.so``, declared in
``include/pkv.h``) built from hand-written HIP for gfx950:

* ``kv_append``: store the step's new K/V token of each sequence into its slot
  of the block-paged cache (bf16 copy, or e4m3fn / int8 quantisation with
  a per-(block, kv head) scale);
* ``paged_decode_attention``: one query token per sequence attends over its
  whole paged history (GQA grouping, no causal mask, exact masking of
  everything past ``context_lens``), split over the context with a
  log-sum-exp merge;
* ``paged_attention``: the generalised call -- several query tokens per
  sequence with the bottom-right causal mask, and an optional sliding window
  with attention sinks;
* ``rope_kv_append``: the rotary embedding of q and of the new keys
  (Llama 3 frequency scaling) fused with the append;
* ``decode_step``: both in one call (the append runs inside the attention's
  partition kernel), bit-identical to the two calls in sequence;
  ``decode_step_rope`` the same with the rotary embedding of q and the new
  keys (size its workspace with ``decode_step_rope_workspace_bytes``);
* ``validate_inputs``: a debug check of the device-resident inputs.

The Python functions in :mod:`paged_kv_decode_06_amd.ops` only marshal
torch tensors into the C calls; every step runs in the HIP kernels.  There is
no fallback: if the library is missing the call raises.
"""
from .ops import (  # noqa: F401
    KV_BF16,
    KV_FP8,
    KV_INT8,
    PkvError,
    decode_step,
    decode_step_rope,
    kv_append,
    rope_kv_append,
    paged_attention,
    attention_workspace_bytes,
    decode_step_rope_workspace_bytes,
    paged_decode_attention,
    paged_decode_merge,
    paged_decode_partition,
    validate_inputs,
    workspace_bytes,
    library_path,
)
