// Internal declarations shared by the host entry points and the kernel
// launchers of libkda.  Not part of the public ABI (see include/kda.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

// Copies whole state rows between a cache view and a packed buffer.
// row_stride_bytes/payload_bytes are byte counts; indices are read in their
// own width.  gather: packed <- cache (zeros for invalid/flag-false rows);
// scatter: cache <- packed for valid rows only.
hipError_t launch_state_copy(bool gather, char* cache, int64_t row_stride_bytes, int64_t num_rows,
                             int64_t payload_bytes, const void* indices, bool index64, int64_t num_selected,
                             const uint8_t* flags, char* packed, hipStream_t stream);

// Enqueues the chunked gated-delta-rule prefill; arguments already validated.
hipError_t launch_chunk_prefill(const kda_prefill_args_t& a, hipStream_t stream);

// Enqueues one recurrent decode step on validated arguments (cache and args agree).
hipError_t launch_recurrent_decode(const kda_state_cache_t& cache, const kda_decode_args_t& a, hipStream_t stream);

// INT8 checkpoint codec: quantize-scatter (packed -> store slots) or
// dequantize-gather (store slots -> packed); arguments already validated.
hipError_t launch_int8_ckpt(bool quantize, const kda_int8_store_t& store, const void* indices, bool index64,
                            int64_t num_selected, const uint8_t* flags, void* packed, bool packed_bf16,
                            hipStream_t stream);

// Workspace bytes launch_chunk_prefill uses for these sizes.
size_t chunk_prefill_workspace_bytes(int64_t T, int64_t N, int64_t H, int64_t K, int64_t V);

// Device address of the current device's copy of the library's static
// scratch array (KDA_NOALLOC_SCRATCH_BYTES bytes), looked up once per device.
hipError_t noalloc_scratch(void** ptr);

}  // namespace kda
