// State gather / scatter kernels for gfx950.
//
// Behaviour follows the copy contract of the page "vllm-ascend 的 KDA 状态复制
// Triton 集成：PR 17301 对齐的预编译 worker 生命周期方案", section "数值契约":
// gather writes every packed row (zeros for an invalid index or a false flag),
// scatter skips invalid targets and ignores flags, page gaps and the storage
// offset are never touched, and row addresses are formed in 64-bit arithmetic
// so caches spanning more than 4 GiB are addressed correctly.
//
// Design: the copy is HBM-bound, so each workgroup streams one contiguous
// tile of one row with the widest vector the alignment allows (16 B when the
// cache base, row stride, payload and packed base are all 16-byte aligned),
// every thread keeping several independent loads in flight before its stores
// (16-byte tiles: 8 KiB per workgroup for gather, 32 KiB for scatter).  Loads
// and stores are non-temporal: the rows are touched once.  Invalid /
// flag-false gather rows only store zeros, scatter skips the whole tile for an
// invalid target.  A grid-stride loop over (row, tile) pairs keeps the grid
// within the dispatch limits for any selection size.
#include "internal.h"

namespace kda {
namespace {

constexpr int kThreads = 256;
// vectors in flight per thread: gather (strided rows in, dense packed rows
// out) runs fastest with 8 KiB tiles, scatter (dense in, strided out) with
// 32 KiB tiles
constexpr int kGatherUnroll = 2;
constexpr int kScatterUnroll = 8;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <typename T>
__device__ __forceinline__ T zero_vec() {
  return T(0);
}

template <typename VecT, bool kGather, typename IdxT, int kUnroll>
__global__ __launch_bounds__(kThreads) void state_copy_kernel(char* __restrict__ cache, int64_t row_stride_bytes,
                                                               int64_t num_rows, int64_t payload_vecs,
                                                               int64_t tiles_per_row, int64_t total_tiles,
                                                               const IdxT* __restrict__ indices,
                                                               const uint8_t* __restrict__ flags,
                                                               char* __restrict__ packed) {
  constexpr int64_t kTileVecs = (int64_t)kThreads * kUnroll;
  for (int64_t t = blockIdx.x; t < total_tiles; t += gridDim.x) {
    const int64_t row = t / tiles_per_row;
    const int64_t tile = t - row * tiles_per_row;
    const int64_t idx = (int64_t)indices[row];
    const bool valid = idx >= 0 && idx < num_rows;
    const int64_t begin = tile * kTileVecs;
    const int64_t end = begin + kTileVecs < payload_vecs ? begin + kTileVecs : payload_vecs;
    VecT* pk = reinterpret_cast<VecT*>(packed + row * payload_vecs * (int64_t)sizeof(VecT));
    if (kGather) {
      const bool take = valid && (flags == nullptr || flags[row] != 0);
      if (take) {
        const VecT* src = reinterpret_cast<const VecT*>(cache + idx * row_stride_bytes);
        if (end - begin == kTileVecs) {
          VecT buf[kUnroll];
#pragma unroll
          for (int u = 0; u < kUnroll; ++u)
            buf[u] = __builtin_nontemporal_load(src + begin + u * kThreads + threadIdx.x);
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(buf[u], pk + begin + u * kThreads + threadIdx.x);
        } else {
          for (int64_t i = begin + threadIdx.x; i < end; i += kThreads)
            __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), pk + i);
        }
      } else {
        const VecT z = zero_vec<VecT>();
        for (int64_t i = begin + threadIdx.x; i < end; i += kThreads) __builtin_nontemporal_store(z, pk + i);
      }
    } else {
      if (!valid) continue;
      VecT* dst = reinterpret_cast<VecT*>(cache + idx * row_stride_bytes);
      if (end - begin == kTileVecs) {
        VecT buf[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
          buf[u] = __builtin_nontemporal_load(pk + begin + u * kThreads + threadIdx.x);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(buf[u], dst + begin + u * kThreads + threadIdx.x);
      } else {
        for (int64_t i = begin + threadIdx.x; i < end; i += kThreads)
          __builtin_nontemporal_store(__builtin_nontemporal_load(pk + i), dst + i);
      }
    }
  }
}

template <typename VecT, typename IdxT>
hipError_t launch_typed(bool gather, char* cache, int64_t row_stride_bytes, int64_t num_rows, int64_t payload_bytes,
                        const void* indices, int64_t num_selected, const uint8_t* flags, char* packed,
                        hipStream_t stream) {
  const int64_t payload_vecs = payload_bytes / (int64_t)sizeof(VecT);
  const int64_t tile_vecs = (int64_t)kThreads * (gather ? kGatherUnroll : kScatterUnroll);
  const int64_t tiles_per_row = (payload_vecs + tile_vecs - 1) / tile_vecs;
  const int64_t total = tiles_per_row * num_selected;
  const int64_t max_grid = 1 << 20;
  const unsigned grid = (unsigned)(total < max_grid ? total : max_grid);
  const IdxT* idx = static_cast<const IdxT*>(indices);
  if (gather) {
    hipLaunchKernelGGL((state_copy_kernel<VecT, true, IdxT, kGatherUnroll>), dim3(grid), dim3(kThreads), 0, stream,
                       cache, row_stride_bytes, num_rows, payload_vecs, tiles_per_row, total, idx, flags, packed);
  } else {
    hipLaunchKernelGGL((state_copy_kernel<VecT, false, IdxT, kScatterUnroll>), dim3(grid), dim3(kThreads), 0, stream,
                       cache, row_stride_bytes, num_rows, payload_vecs, tiles_per_row, total, idx, nullptr, packed);
  }
  return hipGetLastError();
}

template <typename IdxT>
hipError_t dispatch_width(bool gather, char* cache, int64_t row_stride_bytes, int64_t num_rows, int64_t payload_bytes,
                          const void* indices, int64_t num_selected, const uint8_t* flags, char* packed,
                          hipStream_t stream) {
  const uint64_t a = (uint64_t)(uintptr_t)cache | (uint64_t)row_stride_bytes | (uint64_t)payload_bytes |
                     (uint64_t)(uintptr_t)packed;
  if ((a & 15) == 0)
    return launch_typed<u32x4, IdxT>(gather, cache, row_stride_bytes, num_rows, payload_bytes, indices,
                                     num_selected, flags, packed, stream);
  if ((a & 7) == 0)
    return launch_typed<u32x2, IdxT>(gather, cache, row_stride_bytes, num_rows, payload_bytes, indices,
                                     num_selected, flags, packed, stream);
  if ((a & 3) == 0)
    return launch_typed<unsigned int, IdxT>(gather, cache, row_stride_bytes, num_rows, payload_bytes, indices,
                                            num_selected, flags, packed, stream);
  return launch_typed<unsigned short, IdxT>(gather, cache, row_stride_bytes, num_rows, payload_bytes, indices,
                                            num_selected, flags, packed, stream);
}

}  // namespace

hipError_t launch_state_copy(bool gather, char* cache, int64_t row_stride_bytes, int64_t num_rows,
                             int64_t payload_bytes, const void* indices, bool index64, int64_t num_selected,
                             const uint8_t* flags, char* packed, hipStream_t stream) {
  if (index64)
    return dispatch_width<int64_t>(gather, cache, row_stride_bytes, num_rows, payload_bytes, indices, num_selected,
                                   flags, packed, stream);
  return dispatch_width<int32_t>(gather, cache, row_stride_bytes, num_rows, payload_bytes, indices, num_selected,
                                 flags, packed, stream);
}

}  // namespace kda
