"""KDA (Kimi Delta Attention) prefill hot path for AMD Instinct MI355X (gfx950).

Three stages, each a C-ABI entry point of libkda.so (include/kda.h):

* :func:`kda_state_gather`  -- initial states out of indexed cache rows;
* :func:`kda_chunk_prefill` -- chunkwise gated delta rule (chunk 64), varlen;
* :func:`kda_state_scatter` -- final states back into cache rows.

Decode: :func:`kda_recurrent_decode` advances each sequence by one token with
its state updated in place in its cache row.  Compressed checkpoints:
:func:`kda_ckpt_quantize_scatter` / :func:`kda_ckpt_dequantize_gather` move
states between packed buffers and an INT8 store.

The library must be built (``python -m kda_recurrent_state_amd.build``); there
is no fallback implementation.
"""
from ._lib import KDAError, load_library  # noqa: F401
from .api import (KDAStateCopy, cache_descriptor, checkpoint_offsets, int8_store_descriptor,  # noqa: F401
                  kda_chunk_prefill, kda_chunk_prefill_noalloc, kda_chunk_prefill_workspace_size,
                  kda_ckpt_dequantize_gather,
                  kda_ckpt_quantize_scatter, kda_recurrent_decode, kda_state_gather, kda_state_scatter)

__all__ = ["kda_state_gather", "kda_state_scatter", "kda_chunk_prefill", "kda_chunk_prefill_workspace_size",
           "kda_chunk_prefill_noalloc",
           "kda_recurrent_decode", "kda_ckpt_quantize_scatter", "kda_ckpt_dequantize_gather",
           "int8_store_descriptor",
           "KDAStateCopy", "KDAError", "load_library", "cache_descriptor", "checkpoint_offsets"]
