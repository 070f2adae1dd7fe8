"""KV-cache size arithmetic for the Gemma 4 text decoders (fp64 / int).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The PyTorch port prints the KV-cache size of two models at 32k context, with
full-length caches on every layer and with window-sized caches on the
sliding layers [gemma4-pt-claude README, "KV Cache" table].  Those printed
numbers pin the shapes this library is built for: the layer schedule, the
KV head counts of sliding and global layers, the head widths 256 / 512 and
the bf16 storage of both keys and values.

Model shapes, from the pages:
* 31B: 60 layers at 5:1 local:global, 16 KV heads on sliding layers and 4 on
  global ones [gemma4-pt-claude README, "Supported Models"]; head_dim 256 on
  local layers, global_head_dim 512 [Gemma 4 Keras docs, ``Gemma4Model``
  table]; sliding window 1024 [vinija.ai Gemma 4 primer, "Window sizes by
  model family"].
* 26B-A4B: 30 layers at 5:1, 8 KV heads (2 global), same widths and window.

Reading: a cache stores keys and values as two tensors on every layer,
including the K=V global layers (the printed totals hold only that way).

Pin (tests/test_oracle_kv_cache.py): the printed sizes in
``tests/golden/kv_cache_sizes.json``.
"""


def layer_split(num_layers, local_per_global):
    """Sliding and global layer counts of a ``local_per_global``:1 schedule."""
    period = local_per_global + 1
    n_global = num_layers // period
    return num_layers - n_global, n_global


def kv_cache_bytes(num_layers, local_per_global, kv_heads, global_kv_heads,
                   head_dim, global_head_dim, context, window=None,
                   batch=1, bytes_per_elem=2, tensors_per_layer=2):
    """Bytes of a per-layer KV cache at ``context`` tokens.

    ``window`` set: sliding layers keep ``max(window, ...)`` slots, i.e. only
    ``min(window, context)`` rows; global layers always keep the full
    context.
    """
    n_local, n_global = layer_split(num_layers, local_per_global)
    local_rows = context if window is None else min(window, context)
    per_row_local = kv_heads * head_dim
    per_row_global = global_kv_heads * global_head_dim
    elems = n_local * per_row_local * local_rows + n_global * per_row_global * context
    return batch * tensors_per_layer * bytes_per_elem * elems
