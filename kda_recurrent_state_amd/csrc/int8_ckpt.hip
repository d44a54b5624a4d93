// INT8 checkpoint codec fused into the state copies.
//
// A compressed checkpoint store keeps, per slot and head, the K x V state as
// int8 codes [V][K] plus one fp32 scale per key channel ([1][K]): the scale is
// the largest magnitude over the d_v axis divided by 127 and the codes are
// symmetric (page "【轻量化复刻大模型 / KIMI K3】KDA 对 AI Infra 的挑战与各家应对",
// section 5.3: parked checkpoints are compressed to INT8 and dequantised into
// a fresh active slot on a hit; section 6.6.2: qdata [slots, heads, d_v, d_k]
// int8, scale [slots, heads, 1, d_k], max-abs along d_v, symmetric codes).
//
//   quantize-scatter: store slot indices[i] <- Q(packed[i])   (invalid slots skipped)
//   dequantize-gather: packed[i] <- D(store slot indices[i])  (zeros for invalid
//                                                              slots or false flags)
// Q: amax_c = max_v |x[v][c]|, scale_c = amax_c / 127 (fp32 division),
//    code = clamp(rint(x / scale_c), -127, 127) (fp32 division, ties to even),
//    code = 0 where scale_c = 0.
// D: x = code * scale_c in fp32, then rounded to the packed dtype.
//
// One workgroup per (selected state, head).  Quantize: 16 lanes per row, each
// holding 8 consecutive channels; 16 row groups; the rows stay in registers
// (up to 128) between the column-max pass and the encode pass, so the source
// is read once.  Dequantize: 16 lanes per row, each holding 4 channels at c
// and 4 at c + 64, so that every store instruction of a row writes one
// contiguous run; the code loads of 8 rows are issued before their
// conversion and stores.  State rows and codes are streamed with
// non-temporal loads and stores.
#include "internal.h"

namespace kda {
namespace {

constexpr int kQThreads = 256;
constexpr int kQC = 8;                        // channels per lane, quantize
constexpr int kQLanes = 16;                   // lanes per row, quantize (kQC * kQLanes = 128 channels)
constexpr int kQGroups = kQThreads / kQLanes; // row groups, quantize
constexpr int kQRows = 8;                     // rows per thread kept in registers (V <= 128)
constexpr int kDLanes = 16;                   // lanes per row, dequantize
constexpr int kDGroups = kQThreads / kDLanes; // row groups, dequantize

struct Int8Params {
  int8_t* q;          // element (0,0,0,0) of qdata
  float* s;           // element (0,0,0,0) of scale
  int64_t qs0, ss0;   // slot strides, elements
  int64_t num_slots;
  const void* idx;
  int idx64;
  const uint8_t* flags;
  void* packed;       // [S, H, V, K]
  int pbf16;
  int64_t H, V, K;
  int vec;            // K % 8 == 0 and every row slice aligned: vector I/O
};

__device__ __forceinline__ int64_t slot_of(const Int8Params& p, int64_t i) {
  return p.idx64 ? static_cast<const int64_t*>(p.idx)[i] : (int64_t) static_cast<const int32_t*>(p.idx)[i];
}

__device__ __forceinline__ float ld_packed(const void* base, int64_t e, int bf) {
  return bf ? __uint_as_float((unsigned)static_cast<const unsigned short*>(base)[e] << 16)
            : static_cast<const float*>(base)[e];
}

__device__ __forceinline__ int encode(float x, float sc) {
  if (sc == 0.f) return 0;
  float r = rintf(x / sc);
  r = r > 127.f ? 127.f : (r < -127.f ? -127.f : r);
  return (int)r;
}

// The same code from rc = 1 / sc (correctly rounded; 0 where sc = 0), for sc
// in the normal range: z = x / sc lies in [-127.00001, 127.00001], and
// q = x * rc is within |z| * 2^-23 * (1 + 2^-24) < 2^-16 of z, while the
// correctly rounded quotient is within 2^-18 of z.  When q is at least 2^-14
// away from every half-integer, both round to the same integer as z does;
// otherwise the exact quotient decides (as in encode).
__device__ __forceinline__ int encode_rcp(float x, float sc, float rc) {
  const float q = x * rc;
  float r = rintf(q);
  if (fabsf(q - r) > 0.5f - 0x1p-14f) r = rintf(x / sc);
  r = r > 127.f ? 127.f : (r < -127.f ? -127.f : r);
  return (int)r;
}

typedef unsigned u32x2v __attribute__((ext_vector_type(2)));
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
// Streamed (non-temporal) accesses: state rows and codes are touched once.
template <typename T>
__device__ __forceinline__ T ld_nt(const void* p) {
  return __builtin_nontemporal_load(static_cast<const T*>(p));
}
template <typename T>
__device__ __forceinline__ void st_nt(void* p, T x) {
  __builtin_nontemporal_store(x, static_cast<T*>(p));
}

// kKeep: V <= kQGroups * kQRows, rows held in registers; else the encode pass
// reads the rows again.
template <bool kKeep>
__global__ __launch_bounds__(kQThreads) void quantize_scatter_kernel(Int8Params p) {
  __shared__ float red[kQGroups][128];
  __shared__ float scl[128];
  const int64_t i = blockIdx.x / p.H;
  const int64_t h = blockIdx.x - i * p.H;
  const int64_t slot = slot_of(p, i);
  if (slot < 0 || slot >= p.num_slots) return;
  const int V = (int)p.V, K = (int)p.K;
  const int tid = threadIdx.x;
  const int lane = tid % kQLanes, grp = tid / kQLanes;
  const int c0 = kQC * lane;  // this lane's first channel
  const int64_t src = (i * p.H + h) * p.V * p.K;  // element offset of the source slice
  int8_t* qd = p.q + slot * p.qs0 + h * p.V * p.K;
  float* sd = p.s + slot * p.ss0 + h * p.K;

  auto load = [&](int row, float (&x)[kQC]) {
    const int64_t e = src + (int64_t)row * K + c0;
    if (p.vec) {
      if (p.pbf16) {
        const u32x4v u = kKeep ? ld_nt<u32x4v>(static_cast<const unsigned short*>(p.packed) + e)
                               : *reinterpret_cast<const u32x4v*>(static_cast<const unsigned short*>(p.packed) + e);
        const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int t = 0; t < kQC; ++t)
          x[t] = (t & 1) ? __uint_as_float(w[t >> 1] & 0xffff0000u) : __uint_as_float(w[t >> 1] << 16);
      } else {
        const f32x4v f0 = kKeep ? ld_nt<f32x4v>(static_cast<const float*>(p.packed) + e)
                                : *reinterpret_cast<const f32x4v*>(static_cast<const float*>(p.packed) + e);
        const f32x4v f1 = kKeep ? ld_nt<f32x4v>(static_cast<const float*>(p.packed) + e + 4)
                                : *reinterpret_cast<const f32x4v*>(static_cast<const float*>(p.packed) + e + 4);
        x[0] = f0.x; x[1] = f0.y; x[2] = f0.z; x[3] = f0.w;
        x[4] = f1.x; x[5] = f1.y; x[6] = f1.z; x[7] = f1.w;
      }
    } else {
#pragma unroll
      for (int t = 0; t < kQC; ++t) x[t] = c0 + t < K ? ld_packed(p.packed, e + t, p.pbf16) : 0.f;
    }
  };

  // pass 1: column max over this thread's rows
  float keep[kKeep ? kQRows : 1][kQC];
  float m[kQC];
#pragma unroll
  for (int t = 0; t < kQC; ++t) m[t] = 0.f;
  if (c0 < K) {
    if constexpr (kKeep) {
#pragma unroll
      for (int r = 0; r < kQRows; ++r) {
        int row = grp + kQGroups * r;
        row = row < V ? row : V - 1;  // clamped duplicates do not change the max
        load(row, keep[r]);
      }
#pragma unroll
      for (int r = 0; r < kQRows; ++r)
#pragma unroll
        for (int t = 0; t < kQC; ++t) m[t] = fmaxf(m[t], fabsf(keep[r][t]));
    } else {
      for (int row = grp; row < V; row += kQGroups) {
        float x[kQC];
        load(row, x);
#pragma unroll
        for (int t = 0; t < kQC; ++t) m[t] = fmaxf(m[t], fabsf(x[t]));
      }
    }
#pragma unroll
    for (int t = 0; t < kQC; ++t) red[grp][c0 + t] = m[t];
  }
  __syncthreads();
  if (tid < K) {
    float a = red[0][tid];
#pragma unroll
    for (int g = 1; g < kQGroups; ++g) a = fmaxf(a, red[g][tid]);
    scl[tid] = a / 127.f;  // scale
    sd[tid] = a / 127.f;
  }
  __syncthreads();
  if (c0 >= K) return;
  float sc[kQC], rc[kQC];
  bool tiny = false;  // a nonzero scale below the normal range of 1 / sc: exact quotients
#pragma unroll
  for (int t = 0; t < kQC; ++t) {
    sc[t] = c0 + t < K ? scl[c0 + t] : 0.f;
    rc[t] = sc[t] == 0.f ? 0.f : 1.f / sc[t];
    tiny |= sc[t] != 0.f && sc[t] < 0x1p-120f;
  }
  auto store = [&](int row, const float (&x)[kQC]) {
    int8_t* dst = qd + (int64_t)row * K + c0;
    int qq[kQC];
    if (tiny) {
#pragma unroll
      for (int t = 0; t < kQC; ++t) qq[t] = encode(x[t], sc[t]);
    } else {
#pragma unroll
      for (int t = 0; t < kQC; ++t) qq[t] = encode_rcp(x[t], sc[t], rc[t]);
    }
    if (p.vec) {
      unsigned w[2] = {0u, 0u};
#pragma unroll
      for (int t = 0; t < kQC; ++t) w[t >> 2] |= (unsigned)(qq[t] & 0xff) << (8 * (t & 3));
      st_nt<u32x2v>(dst, u32x2v{w[0], w[1]});
    } else {
#pragma unroll
      for (int t = 0; t < kQC; ++t)
        if (c0 + t < K) dst[t] = (int8_t)qq[t];
    }
  };
  if constexpr (kKeep) {
#pragma unroll
    for (int r = 0; r < kQRows; ++r) {
      const int row = grp + kQGroups * r;
      if (row < V) store(row, keep[r]);
    }
  } else {
    for (int row = grp; row < V; row += kQGroups) {
      float x[kQC];
      load(row, x);
      store(row, x);
    }
  }
}

constexpr int kDRows = 8;  // rows per thread per batch, dequantize (loads issued together)

__global__ __launch_bounds__(kQThreads) void dequantize_gather_kernel(Int8Params p) {
  const int64_t i = blockIdx.x / p.H;
  const int64_t h = blockIdx.x - i * p.H;
  const int64_t slot = slot_of(p, i);
  const bool take = slot >= 0 && slot < p.num_slots && (p.flags == nullptr || p.flags[i] != 0);
  const int V = (int)p.V, K = (int)p.K;
  const int tid = threadIdx.x;
  const int lane = tid % kDLanes, grp = tid / kDLanes;
  const int64_t dst = (i * p.H + h) * p.V * p.K;  // element offset of the packed slice
  const int8_t* qs = take ? p.q + slot * p.qs0 + h * p.V * p.K : nullptr;
  const float* ss = take ? p.s + slot * p.ss0 + h * p.K : nullptr;
  if (p.vec) {
    // groups of 4 channels at ca and ca + 64: each store instruction of a
    // row's 16 lanes covers one contiguous run
    for (int cb = 0; cb < K; cb += 8 * kDLanes) {
      const int ca = cb + 4 * lane, cc = ca + 4 * kDLanes;
      if (ca >= K) continue;
      const bool hc = cc < K;
      float sc[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        sc[t] = take ? ss[ca + t] : 0.f;
        sc[4 + t] = take && hc ? ss[cc + t] : 0.f;
      }
      for (int r0 = grp; r0 < V; r0 += kDGroups * kDRows) {
        unsigned ua[kDRows], uc[kDRows];
        if (take) {
#pragma unroll
          for (int r = 0; r < kDRows; ++r) {
            int row = r0 + kDGroups * r;
            row = row < V ? row : V - 1;
            ua[r] = ld_nt<unsigned>(qs + (int64_t)row * K + ca);
            uc[r] = hc ? ld_nt<unsigned>(qs + (int64_t)row * K + cc) : 0u;
          }
        }
#pragma unroll
        for (int r = 0; r < kDRows; ++r) {
          const int row = r0 + kDGroups * r;
          if (row >= V) break;
          float x[8];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            x[t] = take ? (float)(int8_t)((ua[r] >> (8 * t)) & 0xff) * sc[t] : 0.f;
            x[4 + t] = take ? (float)(int8_t)((uc[r] >> (8 * t)) & 0xff) * sc[4 + t] : 0.f;
          }
          const int64_t e = dst + (int64_t)row * K;
          if (p.pbf16) {
            typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
            __bf16* d = static_cast<__bf16*>(p.packed) + e;
            st_nt<bf4>(d + ca, bf4{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]});
            if (hc) st_nt<bf4>(d + cc, bf4{(__bf16)x[4], (__bf16)x[5], (__bf16)x[6], (__bf16)x[7]});
          } else {
            float* d = static_cast<float*>(p.packed) + e;
            st_nt<f32x4v>(d + ca, f32x4v{x[0], x[1], x[2], x[3]});
            if (hc) st_nt<f32x4v>(d + cc, f32x4v{x[4], x[5], x[6], x[7]});
          }
        }
      }
    }
    return;
  }
  // element path (K not a multiple of 8 or unaligned rows): lane covers 8 channels
  for (int cb = 0; cb < K; cb += 8 * kDLanes) {
    const int c0 = cb + 8 * lane;
    if (c0 >= K) continue;
    float sc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) sc[t] = (take && c0 + t < K) ? ss[c0 + t] : 0.f;
    for (int row = grp; row < V; row += kDGroups) {
      const int64_t e = dst + (int64_t)row * K + c0;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (c0 + t >= K) continue;
        const float x = take ? (float)qs[(int64_t)row * K + c0 + t] * sc[t] : 0.f;
        if (p.pbf16)
          static_cast<__bf16*>(p.packed)[e + t] = (__bf16)x;
        else
          static_cast<float*>(p.packed)[e + t] = x;
      }
    }
  }
}

}  // namespace

hipError_t launch_int8_ckpt(bool quantize, const kda_int8_store_t& st, const void* indices, bool index64,
                            int64_t num_selected, const uint8_t* flags, void* packed, bool packed_bf16,
                            hipStream_t stream) {
  Int8Params p;
  p.q = st.qdata;
  p.s = st.scale;
  p.qs0 = st.qdata_stride0;
  p.ss0 = st.scale_stride0;
  p.num_slots = st.num_slots;
  p.idx = indices;
  p.idx64 = index64;
  p.flags = flags;
  p.packed = packed;
  p.pbf16 = packed_bf16;
  p.H = st.H;
  p.V = st.V;
  p.K = st.K;
  const int64_t eb = packed_bf16 ? 2 : 4;
  // vector I/O: 8-channel groups whole, packed rows 16-byte aligned, int8 rows 8-byte aligned
  p.vec = st.K % 8 == 0 && (uintptr_t)packed % 16 == 0 && (st.K * eb) % 16 == 0 && (uintptr_t)st.qdata % 8 == 0 &&
          st.qdata_stride0 % 8 == 0;
  const dim3 grid((unsigned)(num_selected * st.H)), block(kQThreads);
  if (quantize) {
    if (st.V <= kQGroups * kQRows)
      hipLaunchKernelGGL(quantize_scatter_kernel<true>, grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL(quantize_scatter_kernel<false>, grid, block, 0, stream, p);
  } else {
    hipLaunchKernelGGL(dequantize_gather_kernel, grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace kda
