// Recurrent decode: one new token per sequence, the state updated in place in
// its cache row.
//
// Per (sequence n, head h), with S the K x V state held in cache row
// state_indices[n] (element (r, h, v, c) = S[c][v]) -- the gated delta rule of
// "【轻量化复刻大模型 / KIMI K3】KDA 对 AI Infra 的挑战与各家应对", section 1.1,
// applied to one token:
//   S <- (I - beta k^ k^T) Diag(exp g) S + beta k^ v^T,   o = scale * S^T q^
// with k^, q^ the l2-normalised key and query.  Decode runs the recurrent
// form rather than the chunk form (page "vllm-ascend 的 KDA 状态复制 Triton
// 集成", section "背景": decode takes its own recurrent kernel; page "PR #33465
// 完整报告", section "实现拆解": decode is a separate packed kernel that takes
// the state indices).  An index outside [0, num_rows) marks a padding slot:
// its output is zero and no cache row is touched.
//
// Column v of S is row v of the cache layout: K contiguous elements.  Every
// row is independent once k^, q^, exp(g) and beta are known:
//   x_c = exp(g_c) S[c][v];  u = sum_c k^_c x_c;  x_c += beta k^_c (v_v - u);
//   o_v = scale * sum_c q^_c x_c.
// So a row is owned by 16 lanes (one DPP row), each holding EPL = KP/16
// consecutive elements, and the two row sums are 4-step DPP reductions within
// those 16 lanes.  A workgroup of 256 threads owns one (n, h): 16 row groups,
// each taking rows grp, grp+16, ... in batches of RB rows whose loads are all
// issued before any arithmetic.  The token's k, q and exp(g) are staged in
// LDS once per workgroup.  Only the raw row words stay in registers; the
// decayed values are recomputed for the second pass.  The kernel moves
// 2 x K x V state elements per (n, h) and is HBM-bound.
#include <type_traits>

#include "internal.h"

namespace kda {
namespace {

constexpr int kDecThreads = 256;
constexpr int kRowGroups = kDecThreads / 16;
constexpr int kRB = 8;  // rows per row group per batch
constexpr float kDecL2Eps = 1e-6f;
constexpr float kDecLog2e = 1.4426950408889634f;

struct DecodeParams {
  char* cache;             // element (0,0,0,0)
  int64_t stride0;         // row stride, elements
  int64_t num_rows;
  const void* idx;
  int idx64;
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const void* beta;
  void* out;
  int64_t N, H, K, V;
  float scale;
  int l2norm, x_bf16, beta_bf16;
  int vec;                 // K == KP and 16-lane row slices are aligned: vector state I/O
};

__device__ __forceinline__ float dec_bf2f(unsigned short u) { return __uint_as_float((unsigned)u << 16); }

template <int kCtrl>
__device__ __forceinline__ float dec_dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the same bits
// (each step adds two equal partial sums in either order).
__device__ __forceinline__ float row16_sum(float x) {
  x += dec_dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dec_dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dec_dpp<0x141>(x);  // row_half_mirror
  x += dec_dpp<0x140>(x);  // row_mirror
  return x;
}

// Load / store of a T at a 32-bit byte offset from a uniform base (lets the
// compiler use the scalar-base + 32-bit-offset addressing form).
template <typename T>
__device__ __forceinline__ T ldo(const void* base, uint32_t off) {
  return *reinterpret_cast<const T*>(static_cast<const char*>(base) + off);
}
template <typename T>
__device__ __forceinline__ void sto(void* base, uint32_t off, T x) {
  *reinterpret_cast<T*>(static_cast<char*>(base) + off) = x;
}
typedef unsigned u32x2v __attribute__((ext_vector_type(2)));
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
// Streamed (non-temporal) state traffic: each row is read and written once.
template <typename T>
__device__ __forceinline__ T ldo_nt(const void* base, uint32_t off) {
  return __builtin_nontemporal_load(reinterpret_cast<const T*>(static_cast<const char*>(base) + off));
}
template <typename T>
__device__ __forceinline__ void sto_nt(void* base, uint32_t off, T x) {
  __builtin_nontemporal_store(x, reinterpret_cast<T*>(static_cast<char*>(base) + off));
}

// Raw words of EPL state elements: EPL/2 words for bf16, EPL for fp32.
template <int EPL, bool kSB>
struct RowWords {
  static constexpr int W = kSB ? EPL / 2 : EPL;
  unsigned w[W];
};

// Loads this lane's EPL elements of the row at byte offset off from base.
// kVec: the slice is whole and aligned (vector loads); otherwise element by
// element with columns past K clamped (their values are masked later).
template <int EPL, bool kSB, bool kVec>
__device__ __forceinline__ void load_words(const char* base, uint32_t off, int j, int K, RowWords<EPL, kSB>& r) {
  constexpr int W = RowWords<EPL, kSB>::W;
  if constexpr (kVec) {
    const uint32_t o = off + 4u * W * (uint32_t)j;
    if constexpr (W == 2) {
      const u32x2v a = ldo_nt<u32x2v>(base, o);
      r.w[0] = a.x; r.w[1] = a.y;
    } else {
#pragma unroll
      for (int i = 0; i < W; i += 4) {
        const u32x4v a = ldo_nt<u32x4v>(base, o + 4u * i);
        r.w[i] = a.x; r.w[i + 1] = a.y; r.w[i + 2] = a.z; r.w[i + 3] = a.w;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int c = EPL * j + e;
      const uint32_t cs = (uint32_t)(c < K ? c : K - 1);
      if (kSB) {
        const unsigned u = ldo<unsigned short>(base, off + 2u * cs);
        if (e & 1) r.w[e >> 1] |= u << 16; else r.w[e >> 1] = u;
      } else {
        r.w[e] = ldo<unsigned>(base, off + 4u * cs);
      }
    }
  }
}

template <int EPL, bool kSB>
__device__ __forceinline__ void unpack_words(const RowWords<EPL, kSB>& r, float (&x)[EPL]) {
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    if (kSB)
      x[e] = (e & 1) ? __uint_as_float(r.w[e >> 1] & 0xffff0000u) : __uint_as_float(r.w[e >> 1] << 16);
    else
      x[e] = __uint_as_float(r.w[e]);
  }
}

template <int EPL, bool kSB, bool kVec>
__device__ __forceinline__ void store_row(char* base, uint32_t off, int j, int K, const float (&x)[EPL]) {
  if constexpr (kVec) {
    if constexpr (kSB) {
      typedef __bf16 bfv __attribute__((ext_vector_type(EPL)));
      bfv o;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = (__bf16)x[e];
      sto_nt<bfv>(base, off + 2u * EPL * (uint32_t)j, o);
    } else {
#pragma unroll
      for (int i = 0; i < EPL; i += 4)
        sto_nt<f32x4v>(base, off + 4u * (EPL * (uint32_t)j + i), f32x4v{x[i], x[i + 1], x[i + 2], x[i + 3]});
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int c = EPL * j + e;
      if (c >= K) continue;
      if (kSB)
        sto<__bf16>(base, off + 2u * (uint32_t)c, (__bf16)x[e]);
      else
        sto<float>(base, off + 4u * (uint32_t)c, x[e]);
    }
  }
}

template <bool kBF16>
__device__ __forceinline__ float dec_ldx(const void* base, uint32_t i) {
  if (kBF16) return dec_bf2f(ldo<unsigned short>(base, 2u * i));
  return ldo<float>(base, 4u * i);
}

// One batch of kRowGroups * kRB state rows starting at row v0 of one
// (sequence, head): load, update in place, write the outputs.
template <int EPL, bool kSB, bool kXB, bool kBB, bool kVec, typename XT>
__device__ __forceinline__ void decode_batch(const DecodeParams& p, int64_t item, int v0, char* base, const XT* qrow,
                                             const XT* krow, const XT* vrow, const float* grow, XT* orow, int j,
                                             int grp, int K, int V) {
  constexpr int eb = kSB ? 2 : 4;
  // this batch's state rows: every load issued before any arithmetic
  RowWords<EPL, kSB> raw[kRB];
  float vv[kRB];
#pragma unroll
  for (int i = 0; i < kRB; ++i) {
    int row = v0 + kRowGroups * i + grp;
    row = row < V ? row : V - 1;
    load_words<EPL, kSB, kVec>(base, (uint32_t)(row * K * eb), j, K, raw[i]);
    vv[i] = dec_ldx<kXB>(vrow, (uint32_t)row);
  }
  const float b = dec_ldx<kBB>(p.beta, (uint32_t)item);
  // key-side values of this lane's EPL columns: k, q and exp(g) staged in LDS
  // once per workgroup (loading them in every row group repeated a third of
  // the workgroup's load instructions and the exponentials 16 times)
  __shared__ __attribute__((aligned(16))) float sx[3][16 * EPL];
  if (v0 == 0) {
    const int t = threadIdx.x;
    if (t < 16 * EPL) {
      const bool in = t < K;
      sx[0][t] = in ? dec_ldx<kXB>(krow, (uint32_t)t) : 0.f;
      sx[1][t] = in ? dec_ldx<kXB>(qrow, (uint32_t)t) : 0.f;
      sx[2][t] = in ? __builtin_amdgcn_exp2f(grow[t] * kDecLog2e) : 0.f;
    }
    __syncthreads();
  }
  float kh[EPL], qh[EPL], dk[EPL];
#pragma unroll
  for (int e = 0; e < EPL; e += 4) {
    const float4 a = *reinterpret_cast<const float4*>(&sx[0][EPL * j + e]);
    const float4 c = *reinterpret_cast<const float4*>(&sx[1][EPL * j + e]);
    const float4 d = *reinterpret_cast<const float4*>(&sx[2][EPL * j + e]);
    kh[e] = a.x; kh[e + 1] = a.y; kh[e + 2] = a.z; kh[e + 3] = a.w;
    qh[e] = c.x; qh[e + 1] = c.y; qh[e + 2] = c.z; qh[e + 3] = c.w;
    dk[e] = d.x; dk[e + 1] = d.y; dk[e + 2] = d.z; dk[e + 3] = d.w;
  }
  float sk = 0.f, sq = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    sk += kh[e] * kh[e];
    sq += qh[e] * qh[e];
  }
  if (p.l2norm) {
    const float rk = __frsqrt_rn(row16_sum(sk) + kDecL2Eps);
    const float rq = __frsqrt_rn(row16_sum(sq) + kDecL2Eps);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      kh[e] *= rk;
      qh[e] *= rq;
    }
  }
  // u = k^T Diag(exp g) S for every row
  float u[kRB];
#pragma unroll
  for (int i = 0; i < kRB; ++i) {
    float x[EPL];
    unpack_words<EPL, kSB>(raw[i], x);
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) a += (kh[e] * dk[e]) * x[e];
    u[i] = a;
  }
#pragma unroll
  for (int i = 0; i < kRB; ++i) u[i] = row16_sum(u[i]);
  // new rows and outputs
  float o[kRB];
#pragma unroll
  for (int i = 0; i < kRB; ++i) {
    float x[EPL];
    unpack_words<EPL, kSB>(raw[i], x);
    const float wv = b * (vv[i] - u[i]);
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      x[e] = dk[e] * x[e] + kh[e] * wv;
      a += qh[e] * x[e];
    }
    o[i] = a;
    const int row = v0 + kRowGroups * i + grp;
    if (row < V) store_row<EPL, kSB, kVec>(base, (uint32_t)(row * K * eb), j, K, x);
  }
#pragma unroll
  for (int i = 0; i < kRB; ++i) o[i] = row16_sum(o[i]);
  if (j == 0) {
#pragma unroll
    for (int i = 0; i < kRB; ++i) {
      const int row = v0 + kRowGroups * i + grp;
      if (row >= V) continue;
      const float ov = p.scale * o[i];
      if constexpr (kXB)
        reinterpret_cast<__bf16*>(orow)[row] = (__bf16)ov;
      else
        orow[row] = ov;
    }
  }
}

// One workgroup per (sequence, head).  kSB: bf16 state; kXB: bf16 q/k/v/out;
// kBB: bf16 beta; kVec: vector state I/O, K = 16 * EPL and 16-byte aligned
// q/k/g rows.  Byte offsets inside one head's state (V*K elements) and inside
// one token-head's q/k/v/g rows fit in 32 bits.
template <int EPL, bool kSB, bool kXB, bool kBB, bool kVec>
__global__ __launch_bounds__(kDecThreads) void recurrent_decode_kernel(DecodeParams p) {
  const int64_t item = blockIdx.x;  // (n, h)
  const int64_t n = item / p.H;
  const int64_t h = item - n * p.H;
  const int K = (int)p.K, V = (int)p.V;
  const int tid = threadIdx.x;
  const int j = tid & 15;    // lane within the row's 16
  const int grp = tid >> 4;  // row group
  const int64_t r = p.idx64 ? static_cast<const int64_t*>(p.idx)[n] : (int64_t) static_cast<const int32_t*>(p.idx)[n];
  // this token-head's rows of q/k/g (K elements) and v/out (V elements)
  typedef typename std::conditional<kXB, unsigned short, float>::type XT;
  const XT* qrow = static_cast<const XT*>(p.q) + item * p.K;
  const XT* krow = static_cast<const XT*>(p.k) + item * p.K;
  const XT* vrow = static_cast<const XT*>(p.v) + item * p.V;
  const float* grow = p.g + item * p.K;
  XT* orow = static_cast<XT*>(p.out) + item * p.V;
  if (r < 0 || r >= p.num_rows) {  // padding slot
    for (int vv = tid; vv < V; vv += kDecThreads) orow[vv] = 0;
    return;
  }
  constexpr int eb = kSB ? 2 : 4;
  char* base = p.cache + (r * p.stride0 + h * p.V * p.K) * eb;  // row v of this head at base + v*K*eb
  // the first batch (all rows when V <= 128) outside any loop, so that its
  // loads are straight-line code
  decode_batch<EPL, kSB, kXB, kBB, kVec>(p, item, 0, base, qrow, krow, vrow, grow, orow, j, grp, K, V);
  for (int v0 = kRowGroups * kRB; v0 < V; v0 += kRowGroups * kRB)
    decode_batch<EPL, kSB, kXB, kBB, kVec>(p, item, v0, base, qrow, krow, vrow, grow, orow, j, grp, K, V);
}

template <int EPL, bool kSB, bool kXB, bool kBB>
void launch_bb(const DecodeParams& prm, hipStream_t stream) {
  const dim3 grid((unsigned)(prm.N * prm.H)), block(kDecThreads);
  if (prm.vec)
    hipLaunchKernelGGL((recurrent_decode_kernel<EPL, kSB, kXB, kBB, true>), grid, block, 0, stream, prm);
  else
    hipLaunchKernelGGL((recurrent_decode_kernel<EPL, kSB, kXB, kBB, false>), grid, block, 0, stream, prm);
}

template <int EPL, bool kSB>
hipError_t launch_sb(const DecodeParams& prm, bool xb, hipStream_t stream) {
  if (xb) {
    if (prm.beta_bf16) launch_bb<EPL, kSB, true, true>(prm, stream);
    else launch_bb<EPL, kSB, true, false>(prm, stream);
  } else {
    if (prm.beta_bf16) launch_bb<EPL, kSB, false, true>(prm, stream);
    else launch_bb<EPL, kSB, false, false>(prm, stream);
  }
  return hipGetLastError();
}

template <int EPL>
hipError_t launch_epl(const DecodeParams& prm, bool state_bf16, bool xb, hipStream_t stream) {
  return state_bf16 ? launch_sb<EPL, true>(prm, xb, stream) : launch_sb<EPL, false>(prm, xb, stream);
}

}  // namespace

hipError_t launch_recurrent_decode(const kda_state_cache_t& c, const kda_decode_args_t& a, hipStream_t stream) {
  DecodeParams prm;
  prm.cache = static_cast<char*>(c.data);
  prm.stride0 = c.stride[0];
  prm.num_rows = c.num_rows;
  prm.idx = a.state_indices;
  prm.idx64 = a.index_type == KDA_I64;
  prm.q = a.q;
  prm.k = a.k;
  prm.v = a.v;
  prm.g = a.g;
  prm.beta = a.beta;
  prm.out = a.out;
  prm.N = a.N;
  prm.H = a.H;
  prm.K = a.K;
  prm.V = a.V;
  prm.scale = a.scale;
  prm.l2norm = a.use_qk_l2norm != 0;
  prm.x_bf16 = a.qkv_dtype == KDA_BF16;
  prm.beta_bf16 = a.beta_dtype == KDA_BF16;
  const bool sb = c.dtype == KDA_BF16;
  const int64_t eb = sb ? 2 : 4;
  const int epl = a.K <= 64 ? 4 : 8;
  // vector I/O: every lane's slice of a row is EPL whole elements, aligned to its width
  const int64_t slice = epl * eb;
  const int64_t al = slice >= 16 ? 16 : slice;
  const uintptr_t xal = (uintptr_t)a.q | (uintptr_t)a.k | (uintptr_t)a.g;
  prm.vec = a.K == 16 * epl && (uintptr_t)c.data % al == 0 && (c.stride[0] * eb) % al == 0 && xal % 16 == 0;
  if (epl == 4) return launch_epl<4>(prm, sb, prm.x_bf16, stream);
  return launch_epl<8>(prm, sb, prm.x_bf16, stream);
}

}  // namespace kda
