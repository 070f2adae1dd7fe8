"""The five attention workloads, shaped like the Gemma 4 variants.

Head counts, head widths and windows come from the variant tables
[gemma4-pt-claude README, "Supported Models"; Gemma 4 Keras docs,
``Gemma4Model`` table; vinija.ai Gemma 4 primer, "Window sizes by model
family"]:

* E2B: 8 query heads, 1 KV head, window 512, head_dim 256 / global 512.
* 31B: 32 query heads, 16 KV heads on sliding layers and 4 on global ones,
  window 1024, head_dim 256 / global 512, K=V on global layers.

RoPE: theta 1e4 with every pair rotated on sliding layers; theta 1e6 with a
quarter of the head rotated (zero-padded frequencies) on global layers.
Scale ``1/sqrt(head_dim)`` everywhere.
"""

from dataclasses import dataclass
import math


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int            # seed component
    kind: str              # "prefill" | "decode"
    B: int
    S: int                 # prefill sequence length (decode: 1)
    Hq: int
    Hkv: int
    D: int
    window: int            # 0 = global (causal)
    rotary_dims: int
    theta: float
    k_eq_v: bool
    len_lo: int = 0        # decode: cache lengths drawn from [len_lo, len_hi]
    len_hi: int = 0
    images: tuple = ()     # prefill: (start, length) image blocks of every sequence

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.D)

    @property
    def cache_cap(self):
        # Global layer: room for the longest cache plus the new token's own
        # slot.  Sliding layer: a rolling cache of `window` slots.
        return self.window if self.window else self.len_hi + 1


WORKLOADS = {
    "e2b_sliding_prefill": Workload(
        "e2b_sliding_prefill", 1, "prefill", B=1, S=1024, Hq=8, Hkv=1, D=256,
        window=512, rotary_dims=256, theta=1e4, k_eq_v=False),
    "e2b_global_prefill": Workload(
        "e2b_global_prefill", 2, "prefill", B=1, S=8192, Hq=8, Hkv=1, D=512,
        window=0, rotary_dims=128, theta=1e6, k_eq_v=False),
    "31b_sliding_prefill": Workload(
        "31b_sliding_prefill", 3, "prefill", B=2, S=16384, Hq=32, Hkv=16, D=256,
        window=1024, rotary_dims=256, theta=1e4, k_eq_v=False),
    "31b_global_kv_prefill": Workload(
        "31b_global_kv_prefill", 4, "prefill", B=1, S=32768, Hq=32, Hkv=4, D=512,
        window=0, rotary_dims=128, theta=1e6, k_eq_v=True),
    "31b_global_kv_decode": Workload(
        "31b_global_kv_decode", 5, "decode", B=32, S=1, Hq=32, Hkv=4, D=512,
        window=0, rotary_dims=128, theta=1e6, k_eq_v=True,
        len_lo=32768, len_hi=131072),
    # chunked prefill of the 31B sliding layer: the last 4096 of 16384
    # positions of 2 sequences over linear K/V caches holding all of them
    "31b_sliding_chunk_prefill": Workload(
        "31b_sliding_chunk_prefill", 7, "chunk", B=2, S=4096, Hq=32, Hkv=16, D=256,
        window=1024, rotary_dims=256, theta=1e4, k_eq_v=False,
        len_lo=16384, len_hi=16384),
    # the 31B sliding prefill with 8 image blocks of 280 tokens per sequence,
    # attended bidirectionally within each block
    "31b_sliding_image_prefill": Workload(
        "31b_sliding_image_prefill", 8, "prefill", B=2, S=16384, Hq=32, Hkv=16, D=256,
        window=1024, rotary_dims=256, theta=1e4, k_eq_v=False,
        images=tuple((1000 + 1900 * i, 280) for i in range(8))),
    # the 31B K=V decode over the layer's own cache format: raw projection
    # rows plus their inverse RMS and rotated key part (V unroped)
    "31b_global_kv_decode_raw": Workload(
        "31b_global_kv_decode_raw", 9, "decode", B=32, S=1, Hq=32, Hkv=4, D=512,
        window=0, rotary_dims=128, theta=1e6, k_eq_v=True,
        len_lo=32768, len_hi=131072),
    # chunked prefill of the 31B K=V global layer: the last 4096 of 32768
    # positions over the layer's own raw-projection cache holding all of them
    "31b_global_kv_chunk_prefill": Workload(
        "31b_global_kv_chunk_prefill", 10, "chunk", B=1, S=4096, Hq=32, Hkv=4, D=512,
        window=0, rotary_dims=128, theta=1e6, k_eq_v=True,
        len_lo=32768, len_hi=32768),
    # sliding-layer decode of the same 31B batch over rolling caches
    "31b_sliding_decode": Workload(
        "31b_sliding_decode", 6, "decode", B=32, S=1, Hq=32, Hkv=16, D=256,
        window=1024, rotary_dims=256, theta=1e4, k_eq_v=False,
        len_lo=32768, len_hi=131072),
}


# Parity cases at the longest contexts the pages give (256K positions on the
# 31B model, 128K on E2B: "Gemma 4" Keras docs and the vinija.ai primer,
# context windows by variant).  Shapes of the layers above at those lengths;
# not timed by the bench (they exist to exercise 64-bit offsets and
# full-length index logic).
MAX_CONTEXT = {
    "31b_global_kv_prefill_256k": Workload(
        "31b_global_kv_prefill_256k", 11, "prefill", B=1, S=262144, Hq=32, Hkv=4, D=512,
        window=0, rotary_dims=128, theta=1e6, k_eq_v=True),
    "31b_sliding_prefill_256k": Workload(
        "31b_sliding_prefill_256k", 12, "prefill", B=1, S=262144, Hq=32, Hkv=16, D=256,
        window=1024, rotary_dims=256, theta=1e4, k_eq_v=False),
    "e2b_global_prefill_128k": Workload(
        "e2b_global_prefill_128k", 14, "prefill", B=1, S=131072, Hq=8, Hkv=1, D=512,
        window=0, rotary_dims=128, theta=1e6, k_eq_v=False),
    "e2b_sliding_prefill_128k": Workload(
        "e2b_sliding_prefill_128k", 15, "prefill", B=1, S=131072, Hq=8, Hkv=1, D=256,
        window=512, rotary_dims=256, theta=1e4, k_eq_v=False),
    # chunked prefills of the last 4096 of 262144 positions over the caches
    "31b_global_kv_chunk_256k": Workload(
        "31b_global_kv_chunk_256k", 16, "chunk", B=1, S=4096, Hq=32, Hkv=4, D=512,
        window=0, rotary_dims=128, theta=1e6, k_eq_v=True, len_lo=262144, len_hi=262144),
    "31b_sliding_chunk_256k": Workload(
        "31b_sliding_chunk_256k", 17, "chunk", B=1, S=4096, Hq=32, Hkv=16, D=256,
        window=1024, rotary_dims=256, theta=1e4, k_eq_v=False, len_lo=262144, len_hi=262144),
    # two sequences whose new token is the 262144th position
    "31b_global_kv_decode_256k": Workload(
        "31b_global_kv_decode_256k", 13, "decode", B=2, S=1, Hq=32, Hkv=4, D=512,
        window=0, rotary_dims=128, theta=1e6, k_eq_v=True,
        len_lo=262143, len_hi=262143),
}


def get(name):
    return WORKLOADS[name]
