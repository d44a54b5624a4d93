// Chunkwise gated delta rule (KDA prefill) for gfx950.
//
// What is computed: for every sequence n and head h of a varlen batch, with a
// K x V fp32 state S, each token t applies
//     S <- (I - beta_t k_t k_t^T) Diag(exp g_t) S + beta_t k_t v_t^T,
//     o_t = scale * S^T q_t,
// after L2-normalising q and k (page "【轻量化复刻大模型 / KIMI K3】KDA 对 AI Infra
// 的挑战与各家应对", section 1.1; page "PR #33465 完整报告", section "关键源码片段",
// for the normalisation, the K^-1/2 scale and the chunk size of 64).
//
// How: a chunk of L <= 64 tokens acts on S as an affine map (section 1.3 of the
// first page), evaluated with the stage order of the second page -- l2norm,
// in-chunk cumulative gate sum in log2 units, gated K K^T and Q K^T, unit
// lower-triangular solve, W/U recompute, inter-chunk state update, output:
//   gamma_i  = log2(e) * sum_{s<=i} g_s                     (per key channel)
//   A_kk     = strict_lower(beta_i * sum_c k_ic k_jc 2^(gamma_ic - gamma_jc))
//   A_qk     = lower(scale * sum_c q_ic k_jc 2^(gamma_ic - gamma_jc))
//   T        = (I + A_kk)^-1
//   W = T diag(beta) (K * 2^gamma),  U = T diag(beta) V,  Kbar = K * 2^(gamma_L - gamma)
//   V_new    = U - W S
//   O        = scale (Q * 2^gamma) S + A_qk V_new
//   S        = diag(2^gamma_L) S + Kbar^T V_new
//
// MI355X mapping (one workgroup of BV/16 wave64s -- 4 or 8 -- per (sequence,
// head, V-block of BV = 64 or 128 value columns)):
//  * The workgroup walks its sequence chunk by chunk; the fp32 state block
//    (K x BV) never leaves registers.  It is held in MFMA accumulator layout,
//    wave w owning 16 value columns, and converted to bf16 B-operands for the
//    W S and Q S products.  The serial chain (V_new, O, S update) touches no
//    barrier: each wave works on its own columns with operands that the whole
//    workgroup prepared in LDS.
//  * Everything the serial chain needs -- the gated key/query tiles, -W, A_qk,
//    Kbar^T, V^T, T -- is built per chunk in LDS (~150 KiB, so one workgroup per
//    CU).  The chunk's inputs are read from HBM exactly once; outputs and the
//    final state are written once.
//  * All dense contractions use v_mfma_f32_16x16x32_bf16 with fp32
//    accumulation.  A C-layout accumulator holds 4 consecutive rows per lane;
//    two such tiles give the 8 contraction values a B-operand lane needs, so a
//    product's C-layout result feeds the next product directly; the LDS tiles
//    that meet such operands store their contraction index in the matching
//    permuted order, so each lane reads its 8 values as one 16-byte run.
//  * Gate factors 2^(gamma_i - gamma_j) are split around a reference row m of
//    the chunk: 2^(gamma_i - gamma_m) * 2^(gamma_m - gamma_j), one exp2 per
//    (row, channel) for each side.  A chunk whose factors would leave the
//    range |log2| <= 100 is re-processed as shorter chunks (64 -> 16 -> 4 -> 1
//    tokens); the chunk formulas are exact for any length, so this changes
//    nothing but speed.
//  * Work items are issued longest sequence first (a small planning kernel
//    ranks the sequences by length) so the long serial chains start early, and
//    the V-block siblings of one (sequence, head) land on the same XCD so the
//    shared q/k/g tiles are served from one L2.
//  * Batches of many chains with K = V = 128 and bf16 q/k/v run a 4-wave
//    variant in 80 KiB of LDS (chunk_prefill_2wg_kernel), so that two chains
//    share each CU and the phases of one fill the idle issue slots of the
//    other.
#include "internal.h"

#include <mutex>
#include <type_traits>

namespace kda {
namespace {

constexpr int kC = 64;  // chunk length
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRangeLimit = 100.f;
constexpr float kL2Eps = 1e-6f;
constexpr float kL2EpsLane = kL2Eps / 64;  // each lane's share of eps in a 64-lane row sum

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// KP: key dim padded to 64 or 128.  BV: value columns per workgroup (64 or 128).
// The workgroup has NW = BV/16 waves; wave w owns value columns [16w, 16w+16)
// of the block in the state phase and rows [RPW*w, RPW*w + RPW) of the chunk
// in the elementwise phase.
template <int KP, int BV>
struct Cfg {
  static constexpr int NW = BV / 16;       // waves
  static constexpr int NT = NW * 64;       // threads
  static constexpr int RPW = kC / NW;      // chunk rows per wave, elementwise phase
  static constexpr int CPL = KP / 64;      // key channels per lane, elementwise phase
  static constexpr int VPL = BV / 64;      // value columns per lane, elementwise phase
  static constexpr int KT = KP / 16;       // 16-row key tiles
  static constexpr int KS = KP / 32;       // 32-deep contraction steps over the key dim
  // Row strides (bf16 elements).  On gfx950, 16 rows read at 4 column offsets
  // hit distinct LDS banks when the stride is 8 (mod 32) dwords for 16-byte
  // reads and 2 (mod 4) dwords for 8-byte reads, and conflict-free 16-byte
  // reads move about twice the bytes per clock of 8-byte reads (measured), so
  // the tiles the serial chain reads as MFMA operands are read 16 bytes per
  // lane: Qg and -W at stride LDK, A_qk at LDA, Kbar^T unpadded with a
  // swizzle (kb_pos).
  static constexpr int LDK = KP + 16;      // [64][KP] tiles (KL, QL, KR, Qg, -W)
  static constexpr int LDT = kC + 4;       // [X][64] tiles read 8 B/lane (KE, (beta V)^T, A_kk)
  static constexpr int LDA = kC + 16;      // A_qk [64][64]
  static constexpr int LDO = BV + 8;       // row stride (bf16) of the output staging tile
  static constexpr int SZ_ROW = kC * LDK * 2;
  static constexpr int SZ_KT = KP * LDT * 2;
  static constexpr int SZ_VT = BV * LDT * 2;
  static constexpr int SZ_T = kC * LDT * 2;
  static constexpr int SZ_A = kC * LDA * 2;
  static constexpr int SZ_KB = KP * kC * 2;  // Kbar^T: unpadded rows, 16-byte runs swizzled (kb_pos)
  // LDS map (bytes).  KL, QL and KR die after the A products; QL's space is
  // reused for -W and KR's for the output staging tile.  With KP = 64, Qg
  // is held in registers through phase B and then written over KL, and the
  // gate totals share the fp32 diagonal blocks' region, so that a workgroup
  // fits in 80 KiB and two share a CU.
  static constexpr bool kCompact = KP == 64;
  static constexpr int R_KL = 0;                    // KL [64][KP]      (-> Qg when compact)
  static constexpr int R_QL = R_KL + SZ_ROW;        // QL [64][KP]      -> -W [64][KP]
  static constexpr int R_KR = R_QL + SZ_ROW;        // KR [64][KP]      -> O staging [64][BV]
  static constexpr int R_QG = kCompact ? R_KL : R_KR + SZ_ROW;  // Qg [64][KP]
  static constexpr int R_KE = R_KR + SZ_ROW + (kCompact ? 0 : SZ_ROW);  // (beta K 2^gamma)^T [KP][64]
  static constexpr int R_KB = R_KE + SZ_KT;         // Kbar^T [KP][64]
  static constexpr int R_VT = R_KB + SZ_KB;         // (beta V)^T [BV][64]
  static constexpr int R_AB = R_VT + SZ_VT;         // bf16 [64][LDT]: -A_kk below the diagonal blocks, D_b on them
  // fp32 diagonal blocks of A_kk, column-major: element (row, col) of block b
  // at b * AD_B + col * AD_C + row (16-byte aligned columns, blocks on
  // different banks)
  static constexpr int AD_C = 20, AD_B = 16 * AD_C + 4;
  static constexpr int R_AD = R_AB + SZ_T;
  static constexpr int R_AQK = R_AD + 4 * AD_B * 4;  // A_qk bf16 [64][LDA]
  static constexpr int R_TOT = kCompact ? R_AD : R_AQK + SZ_A;  // per-wave gate sums fp32 [NW][KP]
  static constexpr int R_DEC = R_AQK + SZ_A + (kCompact ? 0 : NW * KP * 4);  // 2^gamma_L fp32 [KP]
  static constexpr int R_RED = R_DEC + KP * 4;      // range guard fp32 [NW]
  static constexpr int R_DIAG = R_RED + 64;         // fp32 [64] diagonal of A_qk
  static constexpr int LDS = R_DIAG + kC * 4;
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(!kCompact || (LDS <= 80 * 1024 && NW * KP * 4 <= 4 * AD_B * 4), "two workgroups per CU");
  static_assert(kC * LDO * 2 <= SZ_ROW, "output staging fits in the KR region");
  static_assert(RPW == 8 || RPW == 16, "rows per wave");
};

__device__ __forceinline__ float bf2f(unsigned short u) { return __uint_as_float((unsigned)u << 16); }

// A T at a 32-bit byte offset from a uniform base (lets the compiler use the
// scalar-base + 32-bit vector-offset addressing form).
template <typename T>
__device__ __forceinline__ T ld_at(const char* base, uint32_t off) {
  return *reinterpret_cast<const T*>(base + off);
}

template <bool kBF16>
__device__ __forceinline__ float ld_in(const void* p, int64_t i) {
  if (kBF16) return bf2f(static_cast<const unsigned short*>(p)[i]);
  return static_cast<const float*>(p)[i];
}

// Cross-lane reductions: DPP within each 16-lane row (quad swaps, half-row and
// row mirrors), then across rows by row broadcasts or the gfx950 half- and
// quarter-wave swaps, and readlane.  Every lane ends with the same bits.
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}

__device__ __forceinline__ float lane_f(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// DPP move of x from the lanes named by kCtrl into the rows of kRowMask; the
// other rows get 0.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_rows(float x) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, kRowMask, 0xF, false));
}

// Sums over the wave's 64 lanes of x[r] for R rows at once, reduce-scattered:
// the half-wave swap pairs row j with row j + R/2 (lanes 0-31 keep row j,
// lanes 32-63 row j + R/2), the quarter-wave swap pairs those sums again, so
// each 16-lane group holds one row of every register, and DPP finishes the
// sums inside the groups.  On return lane group g holds in u[j] the sum of
// row j + g * R/4, the same bits in each of its 16 lanes.
template <int R>
__device__ __forceinline__ void rows_reduce(const float (&x)[R], float (&u)[R / 4]) {
  static_assert(R % 4 == 0, "rows");
  constexpr int R2 = R / 2, R4 = R / 4;
  float t[R2];
#pragma unroll
  for (int j = 0; j < R2; ++j) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x[j]),
                                                     __builtin_bit_cast(unsigned, x[j + R2]), false, false);
    const unsigned lo = sw[0], hi = sw[1];  // scalar copies before the bit casts
    t[j] = __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
  }
#pragma unroll
  for (int j = 0; j < R4; ++j) {
    const auto sw = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, t[j]),
                                                     __builtin_bit_cast(unsigned, t[j + R4]), false, false);
    const unsigned lo = sw[0], hi = sw[1];
    u[j] = __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
  }
#pragma unroll
  for (int j = 0; j < R4; ++j) {
    u[j] += dpp<0xB1>(u[j]);   // quad_perm [1,0,3,2]
    u[j] += dpp<0x4E>(u[j]);   // quad_perm [2,3,0,1]
    u[j] += dpp<0x141>(u[j]);  // row_half_mirror
    u[j] += dpp<0x140>(u[j]);  // row_mirror: every lane of a group holds the group's row
  }
}

// out[r] = 1 / sqrt(sum over the wave's 64 lanes of x[r]) for R rows at once,
// the same bits in every lane: one rsqrt per register of the reduce-scattered
// sums covers four rows, and readlane hands each row to the wave.
template <int R>
__device__ __forceinline__ void rows_rsqrt(const float (&x)[R], float (&out)[R]) {
  constexpr int R4 = R / 4;
  float u[R4];
  rows_reduce(x, u);
#pragma unroll
  for (int j = 0; j < R4; ++j) u[j] = __frsqrt_rn(u[j]);
#pragma unroll
  for (int r = 0; r < R; ++r) out[r] = lane_f(u[r % R4], 16 * (r / R4));
}

// Per-row factors of a wave's R chunk rows (rows row0 .. row0 + R - 1), from
// each lane's shares of the row sums sk = |k|^2 (+ eps), sq = |q|^2 (+ eps)
// and dq = k . q: rk[r] = 1 / |k_r| and rq[r] = 1 / |q_r| (1 without l2norm),
// the same bits in every lane, and diag[r] = scale q^_r . k^_r, the
// diagonal of A_qk, written by one lane per row.  That fp32 diagonal replaces
// the one the operand tiles give: their bf16 rounding errors do not cancel
// when q^_r . k^_r is small.  It matters only where that term is a token's
// whole output -- a sequence's first token from a zero state; every later
// token also sees earlier tokens or the state -- so the kernels compute it in
// each work item's first chunk only.
template <int R>
__device__ __forceinline__ void rows_norms_diag(const float (&sk)[R], const float (&sq)[R], const float (&dq)[R],
                                                bool l2norm, float scale, int lane, float (&rk)[R], float (&rq)[R],
                                                float* diag) {
  constexpr int R4 = R / 4;
  float uk[R4], uq[R4], ud[R4];
  rows_reduce(dq, ud);
#pragma unroll
  for (int j = 0; j < R4; ++j) uk[j] = uq[j] = 1.f;
  if (l2norm) {
    rows_reduce(sk, uk);
    rows_reduce(sq, uq);
#pragma unroll
    for (int j = 0; j < R4; ++j) {
      uk[j] = __frsqrt_rn(uk[j]);
      uq[j] = __frsqrt_rn(uq[j]);
      ud[j] *= uk[j] * uq[j];
    }
  }
  if ((lane & 15) == 0) {  // group g holds rows j + g R/4
#pragma unroll
    for (int j = 0; j < R4; ++j) diag[j + (lane >> 4) * R4] = ud[j] * scale;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {  // (1 in every lane without l2norm)
    rk[r] = lane_f(uk[r % R4], 16 * (r / R4));
    rq[r] = lane_f(uq[r % R4], 16 * (r / R4));
  }
}

// (for x >= 0: rows outside the broadcast masks receive 0)
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  x = fmaxf(x, dpp_rows<0x142, 0xA>(x));
  x = fmaxf(x, dpp_rows<0x143, 0xC>(x));
  return lane_f(x, 63);
}

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Storage position of contraction index c in the tiles read as 16-byte MFMA
// operands (Qg and -W over key channels, A_qk over tokens): within each
// 32-block, c = 16h + 4g + j is stored at 8g + 4h + j, so the eight values
// lane group g needs for one product (the k order pack_perm gives the other
// operand) are one contiguous 16-byte run.  Runs of 4 from a multiple of 4
// stay contiguous.
__device__ __forceinline__ int kpos(int c) { return (c & ~31) | ((c & 12) << 1) | ((c & 16) >> 2) | (c & 3); }

// Position of token t of row r in Kbar^T: rows of 64 tokens in kpos order
// with no padding, the 16-byte run index XORed with bits 1-3 of the row.
// The 16 rows x 4 runs of a 16-byte operand read then fall on distinct
// banks, and the 8-byte transposed writes of rows 2l, 2l + 1 meet at most
// 2 to a bank.
__device__ __forceinline__ int kb_pos(int r, int t) {
  const int p = kpos(t);
  return r * kC + ((((p >> 3) ^ (r >> 1)) & 7) << 3) + (p & 7);
}

__device__ __forceinline__ bf16x8 pack_perm(const f32x4& lo, const f32x4& hi) {
  return bf16x8{(__bf16)lo[0], (__bf16)lo[1], (__bf16)lo[2], (__bf16)lo[3],
                (__bf16)hi[0], (__bf16)hi[1], (__bf16)hi[2], (__bf16)hi[3]};
}

__device__ __forceinline__ bf16x8 ld8(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

typedef short s16x4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x16_bf16: A lane l holds A[l%16][4(l/16)+e], B lane l holds
// B[4(l/16)+e][l%16] -- the same rows a C-layout lane holds, so a C tile
// packed to bf16 is directly a B operand.
__device__ __forceinline__ f32x4 mfma16(const s16x4& a, const s16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Four floats to bf16, converted in pairs (one v_cvt_pk_bf16_f32 each; a
// bf16x4 built element by element converts one at a time and permutes).
__device__ __forceinline__ bf16x4 to_bf16x4(float a, float b, float c, float d) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const bf16x2 lo = bf16x2{(__bf16)a, (__bf16)b}, hi = bf16x2{(__bf16)c, (__bf16)d};
  return __builtin_bit_cast(bf16x4, u32x2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)});
}

__device__ __forceinline__ s16x4 pack4(const f32x4& x) {
  const float a = x[0], b = x[1], c = x[2], d = x[3];  // scalar copies of the lanes' elements
  return __builtin_bit_cast(s16x4, to_bf16x4(a, b, c, d));
}

__device__ __forceinline__ s16x4 ld4s(const __bf16* p) { return *reinterpret_cast<const s16x4*>(p); }

__device__ __forceinline__ f32x4 widen4(const __bf16* p) {
  const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}

// Workgroup barrier that orders LDS only.  __syncthreads() would also wait
// for every outstanding global store of the wave (vmcnt(0)); the chunk loop
// has no cross-wave traffic through global memory, so its output stores are
// left in flight across barriers.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

constexpr int64_t kPlanMaxN = 2048;

// Relative cost of one chunk of a chain in the two-chains-per-CU kernel, with
// the 8-wave kernel (one chain per CU) as 1: with another chain on its CU,
// and alone on its CU (K = V = 128, bf16; measured on batches of equal
// sequences).  The two-chains kernel is chosen only where its estimate is
// below kTwoPerCuMargin of the 8-wave one.
constexpr double kPairCost = 1.78, kLoneCost = 1.32, kTwoPerCuMargin = 0.95;

// Ranks sequences by length, longest first (ties by index).  One workgroup.
// With sel, it also picks the chunk kernel for the batch (H heads per
// sequence, cus CUs), from makespan estimates in chunk units with chain i of
// the batch (longest first) of c_i chunks and sum C:
//   one chain per CU : max(C / cus, max_k (k + 1) c_{k cus}) -- among the
//                      k cus + 1 longest chains some CU runs k + 1 in turn
//   two chains per CU: max(kPairCost C / (2 cus), kLoneCost c_0)
// and writes 1 (two chains per CU) or 0 to *sel.
__global__ __launch_bounds__(1024) void plan_order_kernel(const int32_t* __restrict__ cu, int64_t N, int64_t T,
                                                          int64_t H, int32_t cus, int32_t* __restrict__ order,
                                                          int32_t* __restrict__ sel) {
  __shared__ int32_t len_s[kPlanMaxN];
  __shared__ int32_t ord_s[kPlanMaxN];
  __shared__ unsigned long long tot_s, lpt_s;
  if (threadIdx.x == 0) tot_s = lpt_s = 0;
  for (int64_t s = threadIdx.x; s < N; s += blockDim.x) {
    int64_t b = cu[s], e = cu[s + 1];
    b = b < 0 ? 0 : (b > T ? T : b);
    e = e < b ? b : (e > T ? T : e);
    len_s[s] = (int32_t)(e - b);
  }
  __syncthreads();
  for (int64_t s = threadIdx.x; s < N; s += blockDim.x) {
    const int32_t ls = len_s[s];
    int32_t rank = 0;
    for (int64_t o = 0; o < N; ++o) {
      const int32_t lo = len_s[o];
      rank += (lo > ls) || (lo == ls && o < s);
    }
    order[rank] = (int32_t)s;
    ord_s[rank] = (int32_t)s;
  }
  if (!sel) return;  // (uniform)
  __syncthreads();
  unsigned long long part = 0;
  for (int64_t s = threadIdx.x; s < N; s += blockDim.x) part += (unsigned long long)((len_s[s] + 63) / 64);
  for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);  // one LDS atomic per wave
  if ((threadIdx.x & 63) == 0 && part) atomicAdd(&tot_s, part * (unsigned long long)H);
  // chain i is one of the H heads of sequence ord_s[i / H]
  const int64_t n = N * H;
  for (int64_t k = threadIdx.x; k * cus < n; k += blockDim.x) {
    const int64_t c = (len_s[ord_s[(k * cus) / H]] + 63) / 64;
    atomicMax(&lpt_s, (unsigned long long)((k + 1) * c));
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const double mean = (double)tot_s / cus;
    const double c0 = (double)((len_s[ord_s[0]] + 63) / 64);
    const double one = fmax(mean, (double)lpt_s);
    const double two = fmax(0.5 * kPairCost * mean, kLoneCost * c0);
    *sel = two < kTwoPerCuMargin * one ? 1 : 0;
  }
}

struct Params {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const void* beta;
  const int32_t* cu;
  const void* init;
  void* out;
  void* fin;
  const int32_t* order;  // NULL: natural order
  int64_t T, N, H, K, V;
  int nvb;               // V-blocks per (sequence, head)
  float scale;
  int beta_bf16, init_bf16, fin_bf16, l2norm;
  int pair;              // K, V even and q/k/v/g 8-byte aligned: two channels per load
  int ovec;              // V % 8 == 0 and out 16-byte aligned: 16-byte output stores
  int svec;              // K % 4 == 0 and state pointers aligned: vector state I/O
  // segment maps (kOut = false): fin receives b = F(0) and mmap receives M
  // (the state propagated from the identity with zero values, rows [seg, H,
  // K, K]: row x of a (segment, head) tile is M's column x), written by the
  // first value block of each (segment, head)
  float* mmap;
  // chunk-boundary checkpoints: the state after every ckpt_iv tokens of a
  // sequence goes to row ckpt_cu[seq] + j of ckpt (rows outside [0, num_ckpt)
  // are skipped)
  void* ckpt;            // NULL: none
  const int32_t* ckpt_cu;
  int64_t ckpt_iv, num_ckpt;
  int ckpt_bf16;
  // segments: seq_of[n] is the sequence that work item n belongs to, seq_cu
  // the sequences' token offsets and seg_first[s] the first segment of
  // sequence s (seq_of NULL: items are whole sequences).  seg_role picks the
  // items of a pass and where their states come from and go:
  //   kSegMaps  : the maps of the middle segments (neither first nor last of
  //               their sequence; kOut = false)
  //   kSegFirst : the first segment of each sequence, from the sequence's
  //               initial state (row seq_of[n] of init): outputs, and its final
  //               state to row n + 1 of sin_next (fp32), or to row seq_of[n] of
  //               fin when it is also the last
  //   kSegRest  : every other segment, from row n of init: outputs, the last
  //               one of each sequence writing row seq_of[n] of fin
  // Only segments below *seg_total are real.
  const int32_t* seq_of;
  const int32_t* seq_cu;
  const int32_t* seg_first;
  int seg_role;
  const int32_t* seg_total;
  float* sin_next;
  // kernel chosen on the device (NULL: none): a launch whose sel_want differs
  // from *sel returns at once
  const int32_t* sel;
  int sel_want;
};

constexpr int kSegMaps = 1, kSegFirst = 2, kSegRest = 3;

// Raw bits of one chunk's inputs as loaded (bf16 pairs packed in one word, a
// bf16 beta in the low half), kept in registers from the time the loads are
// issued until phase 0.
template <int RPW, int CPL, int VPL, bool kBF16>
struct RawChunk {
  static constexpr int KW = (kBF16 && CPL == 2) ? 1 : CPL;  // words per row of q/k
  static constexpr int VW = (kBF16 && VPL == 2) ? 1 : VPL;  // words per row of v
  unsigned k[RPW][KW], q[RPW][KW], v[RPW][VW], b[RPW];
  float g[RPW][CPL];
};

// Writes one lane's state columns (MFMA C layout, S[ct][e] = S(16ct + 4kg + e,
// vc)) to rows [row, row + V) of a [.., V, K] state array.
template <int KT>
__device__ __forceinline__ void store_state(const f32x4 (&S)[KT], void* dst, int bf, int svec, int64_t row, int kg,
                                            int64_t vc, int64_t K, int64_t V) {
  if (vc >= V) return;
  if (svec) {
#pragma unroll
    for (int ct = 0; ct < KT; ++ct) {
      const int64_t c0 = 16 * ct + 4 * kg;
      if (c0 >= K) continue;
      const int64_t o = (row + vc) * K + c0;
      if (bf)
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(dst) + o) =
            to_bf16x4(S[ct][0], S[ct][1], S[ct][2], S[ct][3]);
      else
        *reinterpret_cast<f32x4*>(static_cast<float*>(dst) + o) = S[ct];
    }
  } else {
#pragma unroll
    for (int ct = 0; ct < KT; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t c = 16 * ct + 4 * kg + e;
        if (c >= K) continue;
        const int64_t o = (row + vc) * K + c;
        if (bf)
          static_cast<__bf16*>(dst)[o] = (__bf16)S[ct][e];
        else
          static_cast<float*>(dst)[o] = S[ct][e];
      }
  }
}

// kOut = false: affine maps F(S) = M S + b of segments (out == NULL): from a
// zero state with the chunk's values (-> b) and, in the same pass, from the
// identity with zero values (-> M, propagated through the same W, Kbar and
// decays; its U is zero); q, the query tiles, A_qk and the output products
// are not computed.  Launched with BV == KP so that the K columns of M are
// one 16-column tile per wave.
// kSeg: the items are segments (p.seq_of set; segment passes only).
template <int KP, int BV, bool kBF16, bool kOut, bool kSeg>
__device__ __forceinline__ void chunk_body(const Params& p, char* smem) {
  using C = Cfg<KP, BV>;
  constexpr int NW = C::NW, NT = C::NT, RPW = C::RPW, CPL = C::CPL, VPL = C::VPL;
  static_assert(NT == BV * 4, "launch bounds");
  __bf16* sKL = reinterpret_cast<__bf16*>(smem + C::R_KL);
  __bf16* sQL = reinterpret_cast<__bf16*>(smem + C::R_QL);
  __bf16* sW = reinterpret_cast<__bf16*>(smem + C::R_QL);
  __bf16* sKR = reinterpret_cast<__bf16*>(smem + C::R_KR);
  __bf16* sO = reinterpret_cast<__bf16*>(smem + C::R_KR);
  __bf16* sQg = reinterpret_cast<__bf16*>(smem + C::R_QG);
  __bf16* sKE = reinterpret_cast<__bf16*>(smem + C::R_KE);
  __bf16* sKB = reinterpret_cast<__bf16*>(smem + C::R_KB);
  __bf16* sVT = reinterpret_cast<__bf16*>(smem + C::R_VT);
  __bf16* sAb = reinterpret_cast<__bf16*>(smem + C::R_AB);
  float* sAd = reinterpret_cast<float*>(smem + C::R_AD);
  __bf16* sAqk = reinterpret_cast<__bf16*>(smem + C::R_AQK);
  float* sTot = reinterpret_cast<float*>(smem + C::R_TOT);
  float* sDec = reinterpret_cast<float*>(smem + C::R_DEC);
  float* sRed = reinterpret_cast<float*>(smem + C::R_RED);
  float* sDiag = reinterpret_cast<float*>(smem + C::R_DIAG);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, provably uniform
  const int l = tid & 63;
  const int lr = l & 15;  // MFMA row (A) / column (B, C) within a 16-tile
  const int lg = l >> 4;  // MFMA k-group

  // ---- work item: XCD-aware mapping, V-block siblings share blockIdx % 8 ----
  const int64_t H = p.H, K = p.K, V = p.V;
  const int nvb = p.nvb;
  const int64_t b = blockIdx.x;
  const int64_t grp = b / (8 * nvb);
  const int64_t rem = b - grp * 8 * nvb;
  const int64_t item = grp * 8 + (rem & 7);
  const int vb = (int)(rem >> 3);
  if (item >= p.N * H) return;
  const int64_t rank = item / H;
  const int64_t h = item - rank * H;
  const int64_t n = p.order ? (int64_t)p.order[rank] : rank;
  int64_t bos = p.cu[n], eos = p.cu[n + 1];
  bos = bos < 0 ? 0 : (bos > p.T ? p.T : bos);
  eos = eos < bos ? bos : (eos > p.T ? p.T : eos);
  const int64_t len = eos - bos;
  const int64_t v0 = (int64_t)vb * BV;   // first value column of this block
  const int64_t vcol = v0 + 16 * w + lr; // this lane's state column (state phase)
  const int64_t vcl = vcol < V ? vcol : V - 1;
  const int64_t srow = (n * H + h) * V;  // state row base of (n, h), in units of K elements
  // initial-state row, final-state destination and row, and whether this
  // item writes it (segments: see Params)
  int64_t irow = srow, frow = srow;
  void* fdst = p.fin;
  int fbf16 = p.fin_bf16;
  bool fin_ok = true;
  if constexpr (kSeg) {
    const int64_t sq = p.seq_of[n];
    int64_t se = p.seq_cu[sq + 1];
    se = se < 0 ? 0 : (se > p.T ? p.T : se);
    const bool last = eos == se, first = p.seg_first[sq] == n;
    const bool real = n < (int64_t)*p.seg_total;
    if (p.seg_role == kSegMaps) {
      if (first || last) return;
    } else if (p.seg_role == kSegFirst) {
      if (!first || !real) return;
      irow = (sq * H + h) * V;
      if (last) {
        frow = irow;
      } else {
        fdst = p.sin_next;
        fbf16 = 0;
        frow = srow + H * V;  // row n + 1
      }
    } else {
      if (first) return;
      fin_ok = last && real;
      frow = (sq * H + h) * V;
    }
  }

  // A_qk upper blocks are read by the output product but never written: zero once.
  if constexpr (kOut) {
    for (int e = tid; e < kC * kC; e += NT) {
      const int r = e >> 6, c = e & 63;
      if ((c >> 4) > (r >> 4)) sAqk[r * C::LDA + kpos(c)] = (__bf16)0.f;
    }
  }

  // ---- initial state, MFMA C layout: S[ct][e] = S(c = 16ct + 4lg + e, vcol) ----
  f32x4 S[C::KT];
  // maps: M's column mcol of this lane, from the identity (first value block only)
  const int mcol = 16 * w + lr;
  const bool map_m = !kOut && vb == 0 && p.mmap;  // uniform
  f32x4 SM[kOut ? 1 : C::KT];
  if constexpr (!kOut) {
    static_assert(kOut || BV == KP, "maps run with BV == KP");
#pragma unroll
    for (int ct = 0; ct < C::KT; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) SM[ct][e] = (16 * ct + 4 * lg + e == mcol && mcol < K) ? 1.f : 0.f;
  }
  if (p.init) {
    if (p.svec) {
#pragma unroll
      for (int ct = 0; ct < C::KT; ++ct) {
        const int64_t c0 = 16 * ct + 4 * lg;
        const int64_t cs = c0 < K ? c0 : K - 4;
        const int64_t o = (irow + vcl) * K + cs;
        if (p.init_bf16) {
          const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const unsigned short*>(p.init) + o);
          S[ct] = f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                        __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
        } else {
          S[ct] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.init) + o);
        }
      }
    } else {
#pragma unroll
      for (int ct = 0; ct < C::KT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t c = 16 * ct + 4 * lg + e;
          const int64_t o = (irow + vcl) * K + (c < K ? c : K - 1);
          S[ct][e] = p.init_bf16 ? bf2f(static_cast<const unsigned short*>(p.init)[o])
                                 : static_cast<const float*>(p.init)[o];
        }
    }
#pragma unroll
    for (int ct = 0; ct < C::KT; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[ct][e] = (vcol < V && 16 * ct + 4 * lg + e < K) ? S[ct][e] : 0.f;
  } else {
#pragma unroll
    for (int ct = 0; ct < C::KT; ++ct) S[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const float scale = p.scale;
  const int64_t c_lo = (int64_t)l * CPL;       // first key channel of this lane (elementwise phase)
  const int64_t vc_lo = v0 + (int64_t)l * VPL; // first value column of this lane (elementwise phase)
  // Loads of one chunk's rows [tb, tb + min(64, len - tb)): every load is
  // unconditional (row clamped to the span's last row, channel to the last
  // valid one) so they are all in flight together; values outside the chunk
  // or the key/value range are zeroed in phase 0.
  using Raw = RawChunk<RPW, CPL, VPL, kBF16>;
  Raw raw;
  const void* const vsrc = p.v;
  const int64_t vstride = V;
  // Loads of rows RPW*w + r, r in [r0, r1), of the chunk starting at tb (r0
  // and r1 are constants at every call, so the loop unrolls to the rows
  // asked for): rows past the span re-read its last row, channels past K and
  // columns past V re-read the last valid one.
  // (wv: the wave index as the caller has it, opaque inside the chunk loop)
  auto issue_rows = [&](int64_t tb, int r0, int r1, int wv) __attribute__((always_inline)) {
    const int64_t span = (len - tb) < (int64_t)kC ? (len - tb) : (int64_t)kC;
    if (p.pair) {
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        if (r < r0 || r >= r1) continue;
        const int i = RPW * wv + r;
        const int64_t ir = i < span ? i : span - 1;
        // Uniform 64-bit bases at the chunk's first (token, head) row and
        // 32-bit offsets from them (H * max(K, V) <= 2^22 keeps a chunk's
        // offsets below 2^31 bytes); two key channels (CPL == 2) / value
        // columns (VPL == 2) per access.
        constexpr uint32_t eb = kBF16 ? 2 : 4;
        const int64_t row0 = (bos + tb) * H + h;
        const char* kb = static_cast<const char*>(p.k) + row0 * K * eb;
        const char* qb = static_cast<const char*>(p.q) + row0 * K * eb;
        const char* vb = static_cast<const char*>(vsrc) + row0 * vstride * eb;
        const char* gb = reinterpret_cast<const char*>(p.g) + row0 * K * 4;
        const char* bb = static_cast<const char*>(p.beta) + row0 * (p.beta_bf16 ? 2 : 4);
        const uint32_t cs = (uint32_t)(CPL == 2 ? (c_lo + 1 < K ? c_lo : K - 2) : (c_lo < K ? c_lo : K - 1));
        const uint32_t vs = (uint32_t)(VPL == 2 ? (vc_lo + 1 < V ? vc_lo : V - 2) : (vc_lo < V ? vc_lo : V - 1));
        const uint32_t ri = (uint32_t)(ir * H);  // (token, head) rows after row0
        if (p.beta_bf16)
          raw.b[r] = ld_at<unsigned short>(bb, 2 * ri);
        else
          raw.b[r] = ld_at<unsigned>(bb, 4 * ri);
        const uint32_t ek = ri * (uint32_t)K + cs;        // element offset in k, q, g
        const uint32_t ev = ri * (uint32_t)vstride + vs;  // element offset in v
        if (kBF16) {
          if (CPL == 2) {
            // rows are read once: non-temporal loads (and stores of the outputs)
            raw.k[r][0] = __builtin_nontemporal_load(reinterpret_cast<const unsigned*>(kb + 2 * ek));
            raw.q[r][0] = __builtin_nontemporal_load(reinterpret_cast<const unsigned*>(qb + 2 * ek));
          } else {
            raw.k[r][0] = ld_at<unsigned short>(kb, 2 * ek);
            raw.q[r][0] = ld_at<unsigned short>(qb, 2 * ek);
          }
          raw.v[r][0] = VPL == 2 ? __builtin_nontemporal_load(reinterpret_cast<const unsigned*>(vb + 2 * ev))
                                 : (unsigned)ld_at<unsigned short>(vb, 2 * ev);
        } else {
          if (CPL == 2) {
            const uint2 a = ld_at<uint2>(kb, 4 * ek), c = ld_at<uint2>(qb, 4 * ek);
            raw.k[r][0] = a.x; raw.k[r][CPL - 1] = a.y;
            raw.q[r][0] = c.x; raw.q[r][CPL - 1] = c.y;
          } else {
            raw.k[r][0] = ld_at<unsigned>(kb, 4 * ek);
            raw.q[r][0] = ld_at<unsigned>(qb, 4 * ek);
          }
          if (VPL == 2) {
            const uint2 a = ld_at<uint2>(vb, 4 * ev);
            raw.v[r][0] = a.x; raw.v[r][VPL - 1] = a.y;
          } else {
            raw.v[r][0] = ld_at<unsigned>(vb, 4 * ev);
          }
        }
        if (CPL == 2) {
          typedef float f32x2 __attribute__((ext_vector_type(2)));
          const f32x2 fg = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(gb + 4 * ek));
          raw.g[r][0] = fg[0];
          raw.g[r][CPL - 1] = fg[1];
        } else {
          raw.g[r][0] = ld_at<float>(gb, 4 * ek);
        }
      }
    } else {
      // element by element (odd K or V, or unaligned tensors); bf16 pairs are
      // packed after the loads return
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        if (r < r0 || r >= r1) continue;
        const int i = RPW * wv + r;
        const int64_t ir = i < span ? i : span - 1;
        const int64_t th = (bos + tb + ir) * H + h;
        raw.b[r] = p.beta_bf16 ? (unsigned)static_cast<const unsigned short*>(p.beta)[th]
                               : static_cast<const unsigned*>(p.beta)[th];
        unsigned kk[CPL], qq[CPL], vv2[VPL];
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
          const int64_t cs = c_lo + cc < K ? c_lo + cc : K - 1;
          kk[cc] = kBF16 ? (unsigned)static_cast<const unsigned short*>(p.k)[th * K + cs]
                         : static_cast<const unsigned*>(p.k)[th * K + cs];
          qq[cc] = kBF16 ? (unsigned)static_cast<const unsigned short*>(p.q)[th * K + cs]
                         : static_cast<const unsigned*>(p.q)[th * K + cs];
          raw.g[r][cc] = p.g[th * K + cs];
        }
#pragma unroll
        for (int vv = 0; vv < VPL; ++vv) {
          const int64_t vs = vc_lo + vv < V ? vc_lo + vv : V - 1;
          vv2[vv] = kBF16 ? (unsigned)static_cast<const unsigned short*>(vsrc)[th * vstride + vs]
                          : static_cast<const unsigned*>(vsrc)[th * vstride + vs];
        }
        if (kBF16 && CPL == 2) {
          raw.k[r][0] = kk[0] | (kk[CPL - 1] << 16);
          raw.q[r][0] = qq[0] | (qq[CPL - 1] << 16);
        } else {
#pragma unroll
          for (int cc = 0; cc < Raw::KW; ++cc) {
            raw.k[r][cc] = kk[cc];
            raw.q[r][cc] = qq[cc];
          }
        }
        if (kBF16 && VPL == 2) {
          raw.v[r][0] = vv2[0] | (vv2[VPL - 1] << 16);
        } else {
#pragma unroll
          for (int vv = 0; vv < Raw::VW; ++vv) raw.v[r][vv] = vv2[vv];
        }
      }
    }
  };
  auto issue_loads = [&](int64_t tb, int wv) __attribute__((always_inline)) { issue_rows(tb, 0, RPW, wv); };

  // Checkpoints: ck_next is the next checkpoint position relative to bos and
  // ck_row its row (both uniform).  Chunks never straddle a multiple of 64
  // tokens and ckpt_iv is a multiple of 64, so every checkpoint position is
  // a chunk end.
  int64_t ck_next = INT64_MAX, ck_row = 0, ck_end = 0;
  if (p.ckpt) {
    int64_t seq = n, off = 0;
    if constexpr (kSeg) {
      seq = p.seq_of[n];
      int64_t sb = p.seq_cu[seq];
      sb = sb < 0 ? 0 : (sb > p.T ? p.T : sb);
      off = bos - sb;
    }
    const int64_t j = off / p.ckpt_iv;  // checkpoints that end at or before this item's start
    ck_next = (j + 1) * p.ckpt_iv - off;
    ck_row = (int64_t)p.ckpt_cu[seq] + j;
    ck_end = p.ckpt_cu[seq + 1];
    ck_end = ck_end < p.num_ckpt ? ck_end : p.num_ckpt;
  }

  int64_t t0 = 0;
  int Lcap = kC;
  if (len > 0) issue_loads(0, w);
  while (t0 < len) {
    // chunk length: the cap, the tokens left, and the next multiple of 64
    int L = (int)((len - t0) < (int64_t)Lcap ? (len - t0) : (int64_t)Lcap);
    L = L < kC - (int)(t0 & (kC - 1)) ? L : kC - (int)(t0 & (kC - 1));
    // No barrier here: before phase 0's barrier this chunk writes only (beta
    // V)^T and the gate totals, which the previous chunk read before its
    // phase-E and phase-A barriers; every tile the previous chunk's phase E
    // and output still read is rewritten only after phase 0's barrier.
    // Per-iteration copies of the lane indices, opaque to the optimiser: this
    // keeps every lane-dependent LDS address from being hoisted out of the
    // loop into a register of its own (which would force spills).
    int tid_i = tid;
    asm volatile("" : "+v"(tid_i));
    // The wave index, opaque per iteration too: the wave-uniform tile offsets
    // derived from it are recomputed in each chunk rather than hoisted out of
    // the loop, where they would stay live in (and spill out of) the scalar
    // registers.
    int w_i = w;
    asm volatile("" : "+s"(w_i));
    const int w = w_i;
    const int l = tid_i & 63;
    const int lr = l & 15;
    const int lg = l >> 4;
    const int64_t c_lo = (int64_t)l * CPL;
    const int64_t vc_lo = v0 + (int64_t)l * VPL;
    const int tid_l = tid_i;

    // ---------------- phase 0: loads, (beta V)^T, gate sums, norms ----------
    // The chunk's rows were loaded by issue_loads (for this chunk's start) while
    // the previous chunk computed; unpack them and zero what lies outside.
    // Rows past the chunk, channels past K and value columns past V were
    // loaded clamped: zero their bits before anything is unpacked (a full
    // chunk has none; uniform branch).  Masking the loaded words in place
    // keeps a single unpack path after the branch.
    if (!(L == kC && K == KP && v0 + BV <= V)) {
      unsigned mk[Raw::KW], mv[Raw::VW];  // this lane's channel / column masks per word
#pragma unroll
      for (int cw = 0; cw < Raw::KW; ++cw) {
        if (kBF16 && CPL == 2)
          mk[cw] = (c_lo < K ? 0xffffu : 0u) | (c_lo + 1 < K ? 0xffff0000u : 0u);
        else
          mk[cw] = c_lo + cw < K ? ~0u : 0u;
      }
#pragma unroll
      for (int vw = 0; vw < Raw::VW; ++vw) {
        if (kBF16 && VPL == 2)
          mv[vw] = (vc_lo < V ? 0xffffu : 0u) | (vc_lo + 1 < V ? 0xffff0000u : 0u);
        else
          mv[vw] = vc_lo + vw < V ? ~0u : 0u;
      }
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const bool okr = RPW * w + r < L;  // uniform
        raw.b[r] = okr ? raw.b[r] : 0u;
#pragma unroll
        for (int cw = 0; cw < Raw::KW; ++cw) {
          raw.k[r][cw] = okr ? raw.k[r][cw] & mk[cw] : 0u;
          raw.q[r][cw] = okr ? raw.q[r][cw] & mk[cw] : 0u;
        }
#pragma unroll
        for (int vw = 0; vw < Raw::VW; ++vw) raw.v[r][vw] = okr ? raw.v[r][vw] & mv[vw] : 0u;
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) raw.g[r][cc] = (okr && c_lo + cc < K) ? raw.g[r][cc] : 0.f;
      }
    }
    float kx[RPW][CPL], qx[RPW][CPL], gx[RPW][CPL], vx[RPW][VPL], bt[RPW];
    // bf16 beta arrives as the raw 16 bits (widening at load time would make
    // the load wait for its data right there)
    if (p.beta_bf16) {
#pragma unroll
      for (int r = 0; r < RPW; ++r) raw.b[r] <<= 16;
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      bt[r] = __uint_as_float(raw.b[r]);
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) {
        if (kBF16 && CPL == 2) {
          kx[r][cc] = __uint_as_float(cc == 0 ? raw.k[r][0] << 16 : raw.k[r][0] & 0xffff0000u);
          qx[r][cc] = __uint_as_float(cc == 0 ? raw.q[r][0] << 16 : raw.q[r][0] & 0xffff0000u);
        } else if (kBF16) {
          kx[r][cc] = __uint_as_float(raw.k[r][cc] << 16);
          qx[r][cc] = __uint_as_float(raw.q[r][cc] << 16);
        } else {
          kx[r][cc] = __uint_as_float(raw.k[r][cc]);
          qx[r][cc] = __uint_as_float(raw.q[r][cc]);
        }
        gx[r][cc] = raw.g[r][cc];
      }
#pragma unroll
      for (int vv = 0; vv < VPL; ++vv) {
        if (kBF16 && VPL == 2)
          vx[r][vv] = __uint_as_float(vv == 0 ? raw.v[r][0] << 16 : raw.v[r][0] & 0xffff0000u);
        else if (kBF16)
          vx[r][vv] = __uint_as_float(raw.v[r][vv] << 16);
        else
          vx[r][vv] = __uint_as_float(raw.v[r][vv]);
      }
    }
    // squared row norms of k and q and the dot products k . q (bf16 pairs: one
    // dot2 per pair), each lane adding its share of eps to the norms
    float sk[RPW], sq[RPW], dq[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      if (kBF16 && CPL == 2) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        sk[r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, raw.k[r][0]),
                                                __builtin_bit_cast(bf16x2, raw.k[r][0]), kL2EpsLane, false);
        sq[r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, raw.q[r][0]),
                                                __builtin_bit_cast(bf16x2, raw.q[r][0]), kL2EpsLane, false);
        dq[r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, raw.k[r][0]),
                                                __builtin_bit_cast(bf16x2, raw.q[r][0]), 0.f, false);
      } else {
        sk[r] = kL2EpsLane;
        sq[r] = kL2EpsLane;
        dq[r] = 0.f;
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
          sk[r] += kx[r][cc] * kx[r][cc];
          sq[r] += qx[r][cc] * qx[r][cc];
          dq[r] += kx[r][cc] * qx[r][cc];
        }
      }
    }
    // (beta V)^T: this lane's RPW consecutive rows of each of its value columns
#pragma unroll
    for (int vv = 0; vv < VPL; ++vv) {
      bf16x4* pv = reinterpret_cast<bf16x4*>(sVT + (l * VPL + vv) * C::LDT + RPW * w);
#pragma unroll
      for (int h4 = 0; h4 < RPW / 4; ++h4) {
        bf16x4 x;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = (__bf16)(bt[4 * h4 + j] * vx[4 * h4 + j][vv]);
        pv[h4] = x;
      }
    }
    // inclusive sum of g over this wave's rows; the wave totals go to LDS
    float tw[CPL];
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
      float run = 0.f;
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        run += gx[r][cc];
        gx[r][cc] = run;
      }
      tw[cc] = run;
    }
    if (CPL == 2)
      *reinterpret_cast<float2*>(sTot + w * KP + c_lo) = float2{tw[0], tw[CPL - 1]};
    else
      sTot[w * KP + c_lo] = tw[0];
    // 1 / |row| for q and k (1 without l2norm) and, in the first chunk, the
    // diagonal of A_qk (uniform branches)
    float rk[RPW], rq[RPW];
    const bool exact_diag = kOut && t0 == 0;
    if (exact_diag) {
      rows_norms_diag(sk, sq, dq, p.l2norm != 0, scale, l, rk, rq, sDiag + RPW * w);
    } else if (p.l2norm) {
      rows_rsqrt(sk, rk);
      rows_rsqrt(sq, rq);
    } else {
#pragma unroll
      for (int r = 0; r < RPW; ++r) rk[r] = rq[r] = 1.f;
    }
    lds_barrier();

    // gamma in log2 units, the reference row m and the range guard
    const int mw = (L > 32 ? 32 : 16) / RPW;  // waves whose rows precede the reference boundary
    float gm[CPL], gL[CPL];
    float guard = 0.f;
    float totw[NW][CPL];  // every wave's totals of this lane's channels
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      if (CPL == 2) {
        const float2 t2 = *reinterpret_cast<const float2*>(sTot + ww * KP + c_lo);
        totw[ww][0] = t2.x;
        totw[ww][CPL - 1] = t2.y;
      } else {
        totw[ww][0] = sTot[ww * KP + c_lo];
      }
    }
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
      // prefix sums of the wave totals: off = before this wave, ref = before
      // the reference row, tot = the whole chunk (w and mw are uniform)
      float pre[NW + 1];
      pre[0] = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) pre[ww + 1] = pre[ww] + totw[ww][cc];
      const float tot = pre[NW];
      const float ref = mw == 32 / RPW ? pre[32 / RPW] : pre[16 / RPW];
      float off = pre[0];
      off = pre[w];  // uniform index: one indexed register move
      gm[cc] = ref * kLog2e;
      gL[cc] = tot * kLog2e;
      // gx becomes gamma_i - gamma_m = log2(e) * (in-wave prefix + off - ref)
      const float nref = (off - ref) * kLog2e;
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        gx[r][cc] = fmaf(gx[r][cc], kLog2e, nref);
        guard = fmaxf(guard, fabsf(gx[r][cc]));
      }
      guard = fmaxf(guard, fmaxf(gm[cc], gL[cc] - gm[cc]));
    }
    guard = wave_max(guard);
    if (l == 0) sRed[w] = guard;  // checked after phase A's barrier

    // ---------------- phase A: gated operand tiles into LDS ----------------
    __bf16 qgh[C::kCompact ? RPW : 1];  // Qg of this lane's channel, stored after phase B (compact map)
    {
      float cg[CPL], cb[CPL];
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) {
        cg[cc] = __builtin_amdgcn_exp2f(gm[cc]);           // 2^gamma_m
        cb[cc] = __builtin_amdgcn_exp2f(gL[cc] - gm[cc]);  // 2^(gamma_L - gamma_m)
        if (w == 0) sDec[c_lo + cc] = __builtin_amdgcn_exp2f(gL[cc]);
      }
      __bf16 ke[CPL][RPW], kb[CPL][RPW];
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const int i = RPW * w + r;
        const float bk = bt[r] * rk[r];   // beta / |k| of this row
        const float sq = scale * rq[r];   // scale / |q|
        __bf16 kl[CPL], ql[CPL], kr[CPL], qg[CPL];
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
          const float d = gx[r][cc];                     // gamma_i - gamma_m
          const float e1 = __builtin_amdgcn_exp2f(d);   // 2^(gamma_i - gamma_m)
          const float e2 = __builtin_amdgcn_exp2f(-d);  // 2^(gamma_m - gamma_i)
          const float fkl = kx[r][cc] * e1 * bk;        // beta k^ 2^(gamma_i - gamma_m)
          const float fkr = kx[r][cc] * e2 * rk[r];     // k^ 2^(gamma_m - gamma_i)
          kl[cc] = (__bf16)fkl;
          kr[cc] = (__bf16)fkr;
          if constexpr (kOut) {
            const float fql = qx[r][cc] * e1 * sq;      // scale q^ 2^(gamma_i - gamma_m)
            ql[cc] = (__bf16)fql;
            qg[cc] = (__bf16)(fql * cg[cc]);            // scale q^ 2^gamma_i
          }
          ke[cc][r] = (__bf16)(fkl * cg[cc]);           // beta k^ 2^gamma_i
          kb[cc][r] = (__bf16)(fkr * cb[cc]);           // k^ 2^(gamma_L - gamma_i)
        }
        if (CPL == 2) {
          typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
          *reinterpret_cast<bf16x2*>(sKL + i * C::LDK + c_lo) = bf16x2{kl[0], kl[CPL - 1]};
          *reinterpret_cast<bf16x2*>(sKR + i * C::LDK + c_lo) = bf16x2{kr[0], kr[CPL - 1]};
          if constexpr (kOut) {
            *reinterpret_cast<bf16x2*>(sQL + i * C::LDK + c_lo) = bf16x2{ql[0], ql[CPL - 1]};
            *reinterpret_cast<bf16x2*>(sQg + i * C::LDK + kpos((int)c_lo)) = bf16x2{qg[0], qg[CPL - 1]};
          }
        } else {
          sKL[i * C::LDK + c_lo] = kl[0];
          sKR[i * C::LDK + c_lo] = kr[0];
          if constexpr (kOut) {
            sQL[i * C::LDK + c_lo] = ql[0];
            if constexpr (C::kCompact)
              qgh[r] = qg[0];
            else
              sQg[i * C::LDK + kpos((int)c_lo)] = qg[0];
          }
        }
      }
      // transposed tiles: RPW consecutive rows of one channel, 16-byte stores
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) {
        bf16x4* pe = reinterpret_cast<bf16x4*>(sKE + (c_lo + cc) * C::LDT + RPW * w);
        const int rb = (int)c_lo + cc;
#pragma unroll
        for (int h4 = 0; h4 < RPW / 4; ++h4) {
          bf16x4 xe, xb;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            xe[j] = ke[cc][4 * h4 + j];
            xb[j] = kb[cc][4 * h4 + j];
          }
          pe[h4] = xe;
          *reinterpret_cast<bf16x4*>(sKB + kb_pos(rb, RPW * w + 4 * h4)) = xb;
        }
      }
    }
    // The next chunk's loads: the first half of the waves (which the SIMD
    // arbiter favours, so they finish phase A first) issue theirs now, while
    // their SIMD partners finish phase A; the other half issue theirs after
    // phase B's first step, while wave 0 computes phase C.
    const bool early = w < NW / 2;
    if (early && t0 + L < len) issue_loads(t0 + L, w);
    lds_barrier();
    {
      // range guard of every wave (written before the barrier above): a span
      // whose gate factors would leave 2^+-100 is re-processed as shorter
      // chunks, discarding this pass's tiles
      float gmax = sRed[0];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) gmax = fmaxf(gmax, sRed[ww]);
      if (gmax > kRangeLimit && L > 1) {
        Lcap = L > 16 ? 16 : (L > 4 ? 4 : 1);
        // this chunk's rows again (the early half has overwritten them; reloading
        // in every wave also ends the rows' live range at phase 0)
        issue_loads(t0, w);
        continue;
      }
    }

    // ---------------- phase B: A_kk (fp32) and A_qk (bf16) -----------------
    // The ten lower 16x16 block pairs (bi >= bj) in two steps.  Step 1: waves
    // 0-3 take the diagonal pair of block w (A_kk's fp32 diagonal blocks are
    // all phase C needs), waves 4.. the first pairs below the diagonal.  Step
    // 2: wave 0 inverts the diagonal blocks (phase C) while other waves take
    // the remaining pairs.  A_kk and A_qk of a pair share the key operand,
    // and a wave's pairs run as interleaved independent accumulator chains.
    // A_qk is taken transposed (K Q^T) so that each lane holds four
    // consecutive columns of one row.  The pairs below the diagonal are
    // numbered e = 0..5: (1,0) (2,0) (2,1) (3,0) (3,1) (3,2).
    auto pairs = [&](auto npc, auto pick) {
      constexpr int NP = decltype(npc)::value;
      int bi[NP], bj[NP];
#pragma unroll
      for (int m = 0; m < NP; ++m) pick(m, bi[m], bj[m]);
      f32x4 akk[NP], aqk[NP];
      bf16x8 oL[2][NP], oR[2][NP], oQ[2][NP];
      auto fetch = [&](int ks, int bf) {
#pragma unroll
        for (int m = 0; m < NP; ++m) {
          oR[bf][m] = ld8(sKR + (16 * bj[m] + lr) * C::LDK + 32 * ks + 8 * lg);
          oL[bf][m] = ld8(sKL + (16 * bi[m] + lr) * C::LDK + 32 * ks + 8 * lg);
          if constexpr (kOut) oQ[bf][m] = ld8(sQL + (16 * bi[m] + lr) * C::LDK + 32 * ks + 8 * lg);
        }
      };
#pragma unroll
      for (int m = 0; m < NP; ++m) {
        akk[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        aqk[m] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      fetch(0, 0);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        if (ks + 1 < C::KS) fetch(ks + 1, (ks + 1) & 1);
#pragma unroll
        for (int m = 0; m < NP; ++m) {
          akk[m] = mfma(oL[ks & 1][m], oR[ks & 1][m], akk[m]);
          if constexpr (kOut) aqk[m] = mfma(oR[ks & 1][m], oQ[ks & 1][m], aqk[m]);
        }
      }
#pragma unroll
      for (int m = 0; m < NP; ++m) {
        const int col = 16 * bj[m] + lr;
        if (bi[m] != bj[m]) {
#pragma unroll
          for (int e = 0; e < 4; ++e) sAb[(16 * bi[m] + 4 * lg + e) * C::LDT + col] = (__bf16)(-akk[m][e]);
        } else {  // rows 4lg..4lg+3 of column lr: one 16-byte store
          f32x4 d;
#pragma unroll
          for (int e = 0; e < 4; ++e) d[e] = 4 * lg + e > lr ? akk[m][e] : 0.f;
          *reinterpret_cast<f32x4*>(sAd + bi[m] * C::AD_B + lr * C::AD_C + 4 * lg) = d;
        }
        if constexpr (kOut) {  // row 16bi + lr, columns 16bj + 4lg + e; the fp32 diagonal from sDiag
          const int i = 16 * bi[m] + lr, j0 = 16 * bj[m] + 4 * lg;
          f32x4 a;
#pragma unroll
          for (int e = 0; e < 4; ++e) a[e] = i >= j0 + e ? aqk[m][e] : 0.f;
          if (exact_diag && bi[m] == bj[m] && (lr >> 2) == lg) a[lr & 3] = sDiag[i];
          *reinterpret_cast<bf16x4*>(sAqk + i * C::LDA + kpos(j0)) = to_bf16x4(a[0], a[1], a[2], a[3]);
        }
      }
    };
    // pair e below the diagonal: (bi, bj)
    auto below = [](int e, int& bi, int& bj) {
      bi = e < 1 ? 1 : (e < 3 ? 2 : 3);
      bj = e - ((bi - 1) * bi) / 2;
    };
    if (w < 4)
      pairs(std::integral_constant<int, 1>{}, [&](int, int& bi, int& bj) { bi = bj = w; });
    else  // 8 waves: pairs 0-3 below the diagonal
      pairs(std::integral_constant<int, 1>{}, [&](int, int& bi, int& bj) { below(w - 4, bi, bj); });
    lds_barrier();

    // ---------------- phase C: D_b = (I + A_bb)^-1 for the diagonal blocks --
    // beside it, the pairs left below the diagonal: 8 waves, pairs 4 and 5 on
    // waves 1 and 2; 4 waves, all six on waves 1-3, two each
    if (w == 0) {
      // fp32 forward substitution; lane = (block, column).  Step j needs
      // column j of the block: four 16-byte reads, issued one step ahead.
      const int bb = l >> 4;
      int col = l & 15;
      asm volatile("" : "+v"(col));  // keep the identity column below from being hoisted out of the chunk loop
      const f32x4* Ab = reinterpret_cast<const f32x4*>(sAd + bb * C::AD_B);
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = (i == col) ? 1.f : 0.f;
      // columns j + 1 and j + 2 in flight during step j (a ring of three)
      f32x4 cr[3][4];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) cr[c][q] = Ab[c * (C::AD_C / 4) + q];
#pragma unroll
      for (int j = 0; j < 15; ++j) {
        if (j + 2 < 15) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (4 * q + 3 > j + 2) cr[(j + 2) % 3][q] = Ab[(j + 2) * (C::AD_C / 4) + q];
        }
#pragma unroll
        for (int i = j + 1; i < 16; ++i) x[i] -= cr[j % 3][i >> 2][i & 3] * x[j];
        __builtin_amdgcn_sched_barrier(0);  // (register pressure)
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sAb[(16 * bb + i) * C::LDT + 16 * bb + col] = (__bf16)x[i];
    } else if constexpr (NW == 8) {
      if (w < 3) pairs(std::integral_constant<int, 1>{}, [&](int, int& bi, int& bj) { below(w + 3, bi, bj); });
    } else {
      pairs(std::integral_constant<int, 2>{}, [&](int m, int& bi, int& bj) { below(2 * (w - 1) + m, bi, bj); });
    }
    // the other half's loads (they land while phases D-E compute)
    if (!early && t0 + L < len) issue_loads(t0 + L, w);
    lds_barrier();
    if constexpr (kOut && C::kCompact) {
      // Qg over KL, which phase B has finished reading; phase E reads it
      // after phase D's barrier
#pragma unroll
      for (int r = 0; r < RPW; ++r) sQg[(RPW * w + r) * C::LDK + kpos((int)c_lo)] = qgh[r];
    }

    // ---------------- phase D: [W | U] = (I + A_kk)^-1 [beta K 2^gamma | beta V] --
    // Blocked forward substitution, one 16-column tile at a time, no barriers:
    //   X_b = D_b (R_b - sum_{c<b} A_bc X_c),  b = 0..3
    // R is read from the transposed tiles (4 consecutive rows per lane = C layout).
    // The wave's key-column tiles (-> W) and its own value tile (-> U) are
    // solved together, as independent interleaved chains.  Each W block is
    // also taken transposed (same operands swapped) so that a lane holds four
    // consecutive channels of one token for the -W store.
    constexpr int NWT = C::KT / NW;  // W tiles per wave
    static_assert(C::KT % NW == 0, "every wave owns the same number of W tiles");
    f32x4 X[NWT + 1][4];
    {
      f32x4 Xt[NWT][4];
      const __bf16* rhs[NWT + 1];
#pragma unroll
      for (int m = 0; m < NWT; ++m) rhs[m] = sKE + (16 * (w + m * NW) + lr) * C::LDT;
      rhs[NWT] = sVT + (16 * w + lr) * C::LDT;
      // every operand of the substitution is read up front: the block rows of
      // (I + A_kk)^-1's factors (A_bc below the diagonal, D_b on it) and the
      // right-hand sides
      s16x4 ab[4][4];
      bf16x4 rb[NWT + 1][4];
#pragma unroll
      for (int bk = 0; bk < 4; ++bk) {
#pragma unroll
        for (int c = 0; c <= bk; ++c) ab[bk][c] = ld4s(sAb + (16 * bk + lr) * C::LDT + 16 * c + 4 * lg);
#pragma unroll
        for (int m = 0; m <= NWT; ++m) rb[m][bk] = *reinterpret_cast<const bf16x4*>(rhs[m] + 16 * bk + 4 * lg);
      }
      __builtin_amdgcn_sched_barrier(0);  // all reads issued before the chain starts
      s16x4 xb[NWT + 1][4];
#pragma unroll
      for (int bk = 0; bk < 4; ++bk) {
        f32x4 acc[NWT + 1];
#pragma unroll
        for (int m = 0; m <= NWT; ++m)
          acc[m] = f32x4{(float)rb[m][bk][0], (float)rb[m][bk][1], (float)rb[m][bk][2], (float)rb[m][bk][3]};
#pragma unroll
        for (int c = 0; c < bk; ++c) {
#pragma unroll
          for (int m = 0; m <= NWT; ++m) acc[m] = mfma16(ab[bk][c], xb[m][c], acc[m]);
        }
        const s16x4 d = ab[bk][bk];
#pragma unroll
        for (int m = 0; m <= NWT; ++m) {
          const s16x4 r = pack4(acc[m]);
          X[m][bk] = mfma16(d, r, f32x4{0.f, 0.f, 0.f, 0.f});
          xb[m][bk] = pack4(X[m][bk]);
          if (m < NWT) Xt[m][bk] = mfma16(r, d, f32x4{0.f, 0.f, 0.f, 0.f});
        }
      }
      // -W into LDS (QL is dead)
#pragma unroll
      for (int m = 0; m < NWT; ++m) {
        const int ct = w + m * NW;
#pragma unroll
        for (int bk = 0; bk < 4; ++bk)
          *reinterpret_cast<bf16x4*>(sW + (16 * bk + lr) * C::LDK + kpos(16 * ct + 4 * lg)) =
              to_bf16x4(-Xt[m][bk][0], -Xt[m][bk][1], -Xt[m][bk][2], -Xt[m][bk][3]);
      }
    }
    // U for this wave's own value columns stays in registers
    f32x4 (&U)[4] = X[NWT];
    lds_barrier();

    // ---------------- phase E: the serial chain on this wave's 16 columns ----
    // V_new = U - W S, O = Qg S + A_qk V_new, S = D S + Kbar^T V_new.  Each
    // product reads its LDS operands ahead of the MFMAs that use them, so the
    // read latency overlaps the MFMAs already issued.
    // Vn -= W St: contraction step outer, row tile inner (the four
    // accumulators advance together, so consecutive MFMAs are independent);
    // the next step's four operands are read before this step's MFMAs
    auto sub_w_product = [&](const bf16x8 (&bSt)[C::KS], f32x4 (&Vn)[4]) __attribute__((always_inline)) {
      bf16x8 a[2][4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) a[0][rt] = ld8(sW + (16 * rt + lr) * C::LDK + 8 * lg);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        if (ks + 1 < C::KS) {
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
            a[(ks + 1) & 1][rt] = ld8(sW + (16 * rt + lr) * C::LDK + 32 * (ks + 1) + 8 * lg);
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) Vn[rt] = mfma(a[ks & 1][rt], bSt[ks], Vn[rt]);
      }
    };
    // St += Kbar^T V_new: a ring of four Kbar^T operands in flight
    auto add_kbar_product = [&](f32x4 (&St)[C::KT], const bf16x8 (&bV)[2]) __attribute__((always_inline)) {
      constexpr int NU = 2 * C::KT;  // (q2, ct) steps, q2 outer
      // 16-byte run 4 q2 + lg of row 16 ct + lr (kb_pos; the swizzle depends on lr only)
      const int kb0 = lr * kC + 8 * (lg ^ ((lr >> 1) & 7)), kb1 = lr * kC + 8 * ((4 + lg) ^ ((lr >> 1) & 7));
      bf16x8 kr[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        kr[t] = ld8(sKB + 16 * kC * (t % C::KT) + (t / C::KT ? kb1 : kb0));
#pragma unroll
      for (int t = 0; t < NU; ++t) {
        const int q2 = t / C::KT, ct = t % C::KT;
        St[ct] = mfma(kr[t & 3], bV[q2], St[ct]);
        if (t + 4 < NU) {
          const int q2n = (t + 4) / C::KT, ctn = (t + 4) % C::KT;
          kr[t & 3] = ld8(sKB + 16 * kC * ctn + (q2n ? kb1 : kb0));
        }
      }
    };
    // 2^gamma_L of this lane's state rows, read now so that the reads overlap V_new
    f32x4 dec[C::KT];
#pragma unroll
    for (int ct = 0; ct < C::KT; ++ct) dec[ct] = *reinterpret_cast<const f32x4*>(sDec + 16 * ct + 4 * lg);
    bf16x8 bS[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) bS[ks] = pack_perm(S[2 * ks], S[2 * ks + 1]);
    f32x4 Vn[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) Vn[rt] = U[rt];
    sub_w_product(bS, Vn);
    bf16x8 bV[2];
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) bV[q2] = pack_perm(Vn[2 * q2], Vn[2 * q2 + 1]);
#pragma unroll
    for (int ct = 0; ct < C::KT; ++ct) S[ct] *= dec[ct];
    // The output is computed transposed, O^T = S^T Qg^T + V_new^T A_qk^T (the
    // operands of each product swapped): tile rt then holds, per lane, the
    // four consecutive value columns 16w + 4lg.. of token 16rt + lr.
    f32x4 O[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) O[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (kOut) {
      bf16x8 a[2][4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) a[0][rt] = ld8(sQg + (16 * rt + lr) * C::LDK + 8 * lg);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        if (ks + 1 < C::KS) {
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
            a[(ks + 1) & 1][rt] = ld8(sQg + (16 * rt + lr) * C::LDK + 32 * (ks + 1) + 8 * lg);
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) O[rt] = mfma(bS[ks], a[ks & 1][rt], O[rt]);
      }
      // the six A_qk tiles on or below the diagonal, (q2, rt) with 32 q2 <= 16 rt + 15
      bf16x8 aq[6];
#pragma unroll
      for (int t = 0; t < 6; ++t) {
        const int q2 = t < 4 ? 0 : 1, rt = t < 4 ? t : t - 2;
        aq[t] = ld8(sAqk + (16 * rt + lr) * C::LDA + 32 * q2 + 8 * lg);
      }
#pragma unroll
      for (int t = 0; t < 6; ++t) {
        const int q2 = t < 4 ? 0 : 1, rt = t < 4 ? t : t - 2;
        O[rt] = mfma(bV[q2], aq[t], O[rt]);
      }
    }
    add_kbar_product(S, bV);
    if constexpr (!kOut) {
      // segment maps, M part (after the b part, whose U and V_new are then
      // dead): V_new = -W S_M (zero values), S_M = D S_M + Kbar^T V_new
      if (map_m) {
        __builtin_amdgcn_sched_barrier(0);  // the b part's registers are free before the M part starts
        bf16x8 bM[C::KS];
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) bM[ks] = pack_perm(SM[2 * ks], SM[2 * ks + 1]);
        f32x4 Vm[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) Vm[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        sub_w_product(bM, Vm);
        bf16x8 bVm[2];
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) bVm[q2] = pack_perm(Vm[2 * q2], Vm[2 * q2 + 1]);
#pragma unroll
        for (int ct = 0; ct < C::KT; ++ct) SM[ct] *= *reinterpret_cast<const f32x4*>(sDec + 16 * ct + 4 * lg);
        add_kbar_product(SM, bVm);
      }
    }

    // ---------------- output rows of this chunk ---------------------------
    if constexpr (!kOut) {
      // maps of a segment only (no outputs)
    } else if (kBF16 && p.ovec) {
      // stage through LDS (KR is dead), one 8-byte write per tile, and store
      // whole 16-byte runs of rows
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
        *reinterpret_cast<bf16x4*>(sO + (16 * rt + lr) * C::LDO + 16 * w + 4 * lg) =
            to_bf16x4(O[rt][0], O[rt][1], O[rt][2], O[rt][3]);
      lds_barrier();
      constexpr int VPR = BV / 8;  // 16-byte runs per row
      // uniform base at (token bos + t0, head h, column v0), 32-bit lane
      // offsets (H * V <= 2^22 keeps them below 2^31 bytes)
      char* const ob = static_cast<char*>(p.out) + (((bos + t0) * H + h) * V + v0) * 2;
      const uint32_t row_b = (uint32_t)(H * V) * 2;
      typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int u0 = 0; u0 < kC * VPR; u0 += NT) {
        const int u = u0 + tid_l;
        const int i = u / VPR, cv = u - i * VPR;
        if (i < L && v0 + 8 * cv < V)
          __builtin_nontemporal_store(__builtin_bit_cast(u32x4, ld8(sO + i * C::LDO + 8 * cv)),
                                      reinterpret_cast<u32x4*>(ob + ((uint32_t)i * row_b + 16 * (uint32_t)cv)));
      }
    } else {
      const int64_t vb = v0 + 16 * w + 4 * lg;  // this lane's first output column
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int i = 16 * rt + lr;
        if (i >= L) continue;
        const int64_t o = ((bos + t0 + i) * H + h) * V + vb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (vb + e >= V) continue;
          if (kBF16)
            static_cast<__bf16*>(p.out)[o + e] = (__bf16)O[rt][e];
          else
            static_cast<float*>(p.out)[o + e] = O[rt][e];
        }
      }
    }
    t0 += L;
    Lcap = kC;
    if (t0 == ck_next) {
      if (ck_row >= 0 && ck_row < ck_end) {
        int tid_c = tid;
        asm volatile("" : "+v"(tid_c));
        store_state(S, p.ckpt, p.ckpt_bf16, p.svec, (ck_row * H + h) * V, (tid_c & 63) >> 4, v0 + 16 * w + (tid_c & 15),
                    K, V);
      }
      ck_next += p.ckpt_iv;
      ++ck_row;
    }
  }

  // ---- final state ----
  if (fdst && fin_ok) store_state(S, fdst, fbf16, p.svec, frow, lg, vcol, K, V);
  if constexpr (!kOut) {
    if (map_m) store_state(SM, p.mmap, 0, p.svec, (n * H + h) * K, lg, (int64_t)mcol, K, K);
  }
}

template <int KP, int BV, bool kBF16, bool kSeg>
__global__ __launch_bounds__(BV * 4, (Cfg<KP, BV>::kCompact ? 2 : 1)) void chunk_prefill_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) char smem[Cfg<KP, BV>::LDS];
  if (p.sel && *p.sel != p.sel_want) return;
  chunk_body<KP, BV, kBF16, true, kSeg>(p, smem);
}

// Pass 1 of the segment-parallel path in one launch: the first segment of
// each sequence runs as an output item (pout, kSegFirst) and the middle
// segments as map items (pmap, kSegMaps), side by side on the GPU.  Both
// parameter sets describe the same segments and value blocks, so the
// work-item mapping of chunk_body gives the same segment for a workgroup
// under either.
template <int KP, int BV, bool kBF16>
__global__ __launch_bounds__(BV * 4, (Cfg<KP, BV>::kCompact ? 2 : 1)) void chunk_prefill_seg1_kernel(Params pout, Params pmap) {
  __shared__ __attribute__((aligned(16))) char smem[Cfg<KP, BV>::LDS];
  const int64_t b = blockIdx.x;
  const int64_t grp = b / (8 * pout.nvb);
  const int64_t rem = b - grp * 8 * pout.nvb;
  const int64_t item = grp * 8 + (rem & 7);
  if (item >= pout.N * pout.H) return;
  const int64_t n = item / pout.H;
  if (pout.seg_first[pout.seq_of[n]] == n)
    chunk_body<KP, BV, kBF16, true, true>(pout, smem);
  else
    chunk_body<KP, BV, kBF16, false, true>(pmap, smem);
}

// ---------------------------------------------------------------------------
// Two workgroups per CU.  The kernel above runs one (sequence, head) chain per
// CU: its phases follow one another (elementwise VALU work, block products
// bound by LDS latency, MFMA chains, load issue), and with ~150 KiB of LDS
// nothing overlaps them.  This variant, for K = V = 128 with bf16 q, k, v,
// runs a chain with 4 waves (16 chunk rows and 32 value columns each) in at
// most 80 KiB of LDS, so two chains share each CU and the phases of one fill
// the gaps of the other.  Arithmetic and operand layouts are those of the
// kernel above; what changes is where the tiles live:
//  * tiles are unpadded, bank conflicts avoided by swizzling 16-byte runs
//    (row-major tiles) or 8-byte runs (transposed tiles);
//  * the gated tiles of phase B (KL, KR, QL) and those of phases D-E
//    (beta K 2^gamma, Kbar^T, Qg) share one region: the latter are written
//    from registers once phase B is done;
//  * -W is written over beta K 2^gamma: wave w solves, and alone reads, the
//    32-channel pair w, whose 4 KiB it overwrites (token-major, for phase E);
//  * A_kk / D_b and A_qk keep only their blocks on or below the diagonal;
//  * the output staging tile reuses the (beta V)^T region, which the next
//    chunk's phase 0 writes only after its first barrier.
// The next chunk's loads are issued after phase E (registers are short before
// then); the other workgroup on the CU computes while they are in flight.
// ---------------------------------------------------------------------------
namespace w2 {
constexpr int NW = 4, NT = 256, RPW = 16, KT = 8, KS = 4;
// LDS map, bytes
constexpr int R1 = 0;        // KL, KR, QL [64][128] each  ->  beta K 2^gamma (-> -W) [128][64], Kbar^T, Qg
constexpr int R2 = 49152;    // (beta V)^T [128][64]  ->  output staging [64][128]
constexpr int R_AB = 65536;  // 10 bf16 blocks 16x16: -A_kk below the diagonal, D_b on it
constexpr int R_AQK = 70656; // 6 bf16 blocks [16][32] of A_qk (kpos columns)
constexpr int AD_B = 260;    // fp32 stride of the diagonal blocks of A_kk (4 banks apart)
constexpr int R_AD = 76800;  // fp32 4 x [16 columns][16 rows] diagonal blocks of A_kk  /  gate totals [4][128]
constexpr int R_DEC = R_AD + 4 * AD_B * 4;  // fp32 [128] 2^gamma_L
constexpr int R_RED = R_DEC + 512;          // fp32 [4] range guard
constexpr int R_DIAG = R_RED + 16;          // fp32 [64] diagonal of A_qk
constexpr int LDS = R_DIAG + 256;
static_assert(LDS <= 81920, "two workgroups per CU");
static_assert(NW * 128 <= 4 * AD_B, "gate totals fit in the A_kk diagonal region");
// [64][128] row-major tiles (KL, KR, QL, Qg, output): 16-byte run of column c
// in row t XORed with t mod 16
__device__ __forceinline__ int rs_pos(int t, int c) { return t * 128 + ((((c >> 3) ^ (t & 15)) << 3) | (c & 7)); }
// [128][64] transposed tiles ((beta V)^T, beta K 2^gamma): rows in pairs of
// 256 bytes (one sweep of the banks) of 32 runs of 4 tokens; run (r, t) at
// 16 ((r & 1) ^ bit 5 of r) + ((t >> 2) ^ 2 (bits 1-3 of r) ^ bit 4 of r).
// The 16 rows x 2 token runs of a 32-lane operand read, and the rows 2l + x
// of a 32-lane store, fall on distinct banks.
__device__ __forceinline__ int tu_pos(int r, int t) {
  const int hi = (r & 1) ^ ((r >> 5) & 1);
  const int lo = ((t >> 2) ^ (((r >> 1) & 7) << 1) ^ ((r >> 4) & 1)) & 15;
  return (r >> 1) * 128 + ((hi << 4) | lo) * 4 + (t & 3);
}
// Bank rules (gfx950, measured): 32 banks of 4 bytes; a read is served per
// half-wave, a 16-byte write per 8 lanes and an 8-byte write per 16 lanes.
// -W of channel pair w: [64 tokens][32 kpos channels] over pair w's rows of
// beta K 2^gamma (elements [2048 w, 2048 w + 2048)); 16-byte runs XORed with
// bits 1-2 of the token, which keeps the 16 rows x 2 runs of a half-wave's
// operand read off each other's banks
__device__ __forceinline__ int w_pos(int t, int kp) { return t * 32 + ((((kp >> 3) ^ ((t >> 1) & 3)) << 3) | (kp & 7)); }
// A_kk / D_b block (bi >= bj), element (i, j): 8-byte runs XORed with bit 3 of i
__device__ __forceinline__ int ab_pos(int bi, int bj, int i, int j) {
  return ((bi * (bi + 1)) / 2 + bj) * 256 + i * 16 + ((((j >> 2) ^ ((i >> 3) << 1)) << 2) | (j & 3));
}
// A_qk block of row tile rt and 32-column block q2 (32 q2 <= 16 rt + 15), row
// i, kpos column kp; swizzled as -W
__device__ __forceinline__ int aqk_pos(int q2, int rt, int i, int kp) {
  return (q2 ? rt + 2 : rt) * 512 + i * 32 + ((((kp >> 3) ^ ((i >> 1) & 3)) << 3) | (kp & 7));
}
// fp32 diagonal block b of A_kk, element (row, col): columns of 16 floats,
// the 16-byte row groups XORed with bits 1-2 of the column (the 16-byte
// column stores of phase B then hit distinct banks)
__device__ __forceinline__ int ad_pos(int b, int row, int col) {
  return b * AD_B + col * 16 + ((((row >> 2) ^ (col >> 1)) & 3) << 2) + (row & 3);
}
}  // namespace w2

// Requires K == V == 128, bf16 q/k/v, p.pair, p.ovec, outputs (no maps);
// kBetaBF16 == p.beta_bf16.
template <bool kBetaBF16>
__global__ __launch_bounds__(256, 2) void chunk_prefill_2wg_kernel(Params p) {
  using namespace w2;
  __shared__ __attribute__((aligned(16))) char smem[LDS];
  __bf16* sKL = reinterpret_cast<__bf16*>(smem + R1);
  __bf16* sKR = reinterpret_cast<__bf16*>(smem + R1 + 16384);
  __bf16* sQL = reinterpret_cast<__bf16*>(smem + R1 + 32768);
  __bf16* sKE = reinterpret_cast<__bf16*>(smem + R1);  // -> -W, pair by pair
  __bf16* sKB = reinterpret_cast<__bf16*>(smem + R1 + 16384);
  __bf16* sQg = reinterpret_cast<__bf16*>(smem + R1 + 32768);
  __bf16* sVT = reinterpret_cast<__bf16*>(smem + R2);
  __bf16* sO = reinterpret_cast<__bf16*>(smem + R2);
  __bf16* sAb = reinterpret_cast<__bf16*>(smem + R_AB);
  __bf16* sAqk = reinterpret_cast<__bf16*>(smem + R_AQK);
  float* sAd = reinterpret_cast<float*>(smem + R_AD);
  float* sTot = reinterpret_cast<float*>(smem + R_AD);
  float* sDec = reinterpret_cast<float*>(smem + R_DEC);
  float* sRed = reinterpret_cast<float*>(smem + R_RED);
  float* sDiag = reinterpret_cast<float*>(smem + R_DIAG);
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

  if (p.sel && *p.sel != p.sel_want) return;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int lr = l & 15;
  const int lg = l >> 4;

  // ---- work item: one workgroup per (sequence, head) ----
  const int64_t H = p.H, K = p.K, V = p.V;
  const int64_t item = blockIdx.x;
  if (item >= p.N * H) return;
  const int64_t rank = item / H;
  const int64_t h = item - rank * H;
  const int64_t n = p.order ? (int64_t)p.order[rank] : rank;
  int64_t bos = p.cu[n], eos = p.cu[n + 1];
  bos = bos < 0 ? 0 : (bos > p.T ? p.T : bos);
  eos = eos < bos ? bos : (eos > p.T ? p.T : eos);
  const int64_t len = eos - bos;
  const int64_t srow = (n * H + h) * V;
  int64_t frow = srow;
  bool fin_ok = true;
  if (p.seq_of) {  // output pass over segments
    const int64_t sq = p.seq_of[n];
    int64_t se = p.seq_cu[sq + 1];
    se = se < 0 ? 0 : (se > p.T ? p.T : se);
    fin_ok = eos == se && n < (int64_t)*p.seg_total;
    frow = (sq * H + h) * V;
  }

  // A_qk: the upper halves of the two diagonal 32-column blocks are read by
  // the output product but never written
  for (int e = tid; e < 2 * 16 * 16; e += NT) {
    const int q2 = e >> 8, i = (e >> 4) & 15, jj = e & 15;
    sAqk[aqk_pos(q2, 2 * q2, i, kpos(16 + jj))] = (__bf16)0.f;
  }

  // ---- initial state: S[m][ct][e] = S(c = 16ct + 4lg + e, value column 32w + 16m + lr) ----
  f32x4 S[2][KT];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int64_t vcol = 32 * w + 16 * m + lr;
    if (p.init) {
#pragma unroll
      for (int ct = 0; ct < KT; ++ct) {
        const int64_t o = (srow + vcol) * K + 16 * ct + 4 * lg;
        if (p.svec) {
          if (p.init_bf16) {
            const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const unsigned short*>(p.init) + o);
            S[m][ct] = f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                             __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
          } else {
            S[m][ct] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.init) + o);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            S[m][ct][e] = p.init_bf16 ? bf2f(static_cast<const unsigned short*>(p.init)[o + e])
                                      : static_cast<const float*>(p.init)[o + e];
        }
      }
    } else {
#pragma unroll
      for (int ct = 0; ct < KT; ++ct) S[m][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  const float scale = p.scale;
  // raw bits of this wave's 16 rows of a chunk: two channels (k, q, g) or
  // value columns (v) per lane, bf16 pairs in one word
  unsigned rk_[RPW], rq_[RPW], rv_[RPW], rb_[RPW];
  float rg_[RPW][2];
  // This chain's tensors at the current chunk's first (token, head) row; the
  // pointers advance chunk by chunk, so the loop carries six 64-bit bases
  // and 32-bit counters only (scalar registers are the scarce resource here).
  const int64_t crow = bos * H + h;
  const char* kp = static_cast<const char*>(p.k) + crow * 256;
  const char* qp = static_cast<const char*>(p.q) + crow * 256;
  const char* vp = static_cast<const char*>(p.v) + crow * 256;
  const char* gp = reinterpret_cast<const char*>(p.g) + crow * 512;
  const char* bp = static_cast<const char*>(p.beta) + crow * (kBetaBF16 ? 2 : 4);
  char* op = static_cast<char*>(p.out) + crow * 256;
  const uint32_t Hu = (uint32_t)H;
  const uint32_t lenu = (uint32_t)len;
  // Loads of the chunk that starts dr tokens after the current one, span
  // (1..64) tokens of it: rows past the span re-read its last row.  32-bit
  // offsets: (dr + 63) H 512 < 2^32 for H <= 65535.
  // (wv: the wave index as the caller has it, opaque inside the chunk loop)
  auto issue_loads = [&](uint32_t dr, uint32_t span, int wv) __attribute__((always_inline)) {
    const uint32_t cl = (uint32_t)(tid & 63) * 2;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const uint32_t i = (uint32_t)(RPW * wv + r);
      const uint32_t ri = ((i < span ? i : span - 1) + dr) * Hu;  // (token, head) rows after the current one
      if (kBetaBF16)
        rb_[r] = ld_at<unsigned short>(bp, 2 * ri);
      else
        rb_[r] = ld_at<unsigned>(bp, 4 * ri);
      const uint32_t ek = ri * 128u + cl;
      // read once: non-temporal (-1 % on the e2e batch, -1.5 % with 2048 chains)
      rk_[r] = __builtin_nontemporal_load(reinterpret_cast<const unsigned*>(kp + 2 * ek));
      rq_[r] = __builtin_nontemporal_load(reinterpret_cast<const unsigned*>(qp + 2 * ek));
      rv_[r] = __builtin_nontemporal_load(reinterpret_cast<const unsigned*>(vp + 2 * ek));
      typedef float f32x2 __attribute__((ext_vector_type(2)));
      const f32x2 fg = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(gp + 4 * ek));
      rg_[r][0] = fg[0];
      rg_[r][1] = fg[1];
    }
  };

  // checkpoints (32-bit: positions within a sequence, rows of ckpt)
  uint32_t ck_next = 0xffffffffu, ck_iv = 0;
  int32_t ck_row = 0, ck_end = 0;
  if (p.ckpt) {
    int64_t seq = n, off = 0;
    if (p.seq_of) {
      seq = p.seq_of[n];
      int64_t sb = p.seq_cu[seq];
      sb = sb < 0 ? 0 : (sb > p.T ? p.T : sb);
      off = bos - sb;
    }
    const int64_t j = off / p.ckpt_iv;
    ck_next = (uint32_t)((j + 1) * p.ckpt_iv - off);
    ck_iv = (uint32_t)p.ckpt_iv;
    ck_row = (int32_t)(p.ckpt_cu[seq] + j);
    const int64_t ce = p.ckpt_cu[seq + 1];
    ck_end = (int32_t)(ce < p.num_ckpt ? ce : p.num_ckpt);
  }

  uint32_t t0 = 0;
  uint32_t Lcap = kC;
  if (lenu > 0) issue_loads(0, lenu < (uint32_t)kC ? lenu : (uint32_t)kC, w);
  while (t0 < lenu) {
    uint32_t L = lenu - t0 < Lcap ? lenu - t0 : Lcap;
    L = L < kC - (t0 & (kC - 1)) ? L : kC - (t0 & (kC - 1));
    int tid_i = tid;
    asm volatile("" : "+v"(tid_i));
    // The wave index, opaque per iteration too: the wave-uniform tile offsets
    // derived from it are recomputed in each chunk rather than hoisted out of
    // the loop, where they would stay live in (and spill out of) the scalar
    // registers.
    int w_i = w;
    asm volatile("" : "+s"(w_i));
    const int w = w_i;
    const int l = tid_i & 63;
    const int lr = l & 15;
    const int lg = l >> 4;
    const int c_lo = 2 * l;  // this lane's channels / value columns in the elementwise phases

    // ---------------- phase 0: unpack, gate sums, norms ----------------
    if (L != kC) {
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const bool okr = RPW * w + r < L;  // uniform
        rb_[r] = okr ? rb_[r] : 0u;
        rk_[r] = okr ? rk_[r] : 0u;
        rq_[r] = okr ? rq_[r] : 0u;
        rv_[r] = okr ? rv_[r] : 0u;
        rg_[r][0] = okr ? rg_[r][0] : 0.f;
        rg_[r][1] = okr ? rg_[r][1] : 0.f;
      }
    }
    float gx[RPW][2], bt[RPW];
    // beta v of this lane's two value columns, packed as bf16 pairs of
    // consecutive rows of one column (the layout of the transposed tile)
    unsigned bvc[2][RPW / 2];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      bt[r] = __uint_as_float(kBetaBF16 ? rb_[r] << 16 : rb_[r]);
      gx[r][0] = rg_[r][0];
      gx[r][1] = rg_[r][1];
    }
#pragma unroll
    for (int r = 0; r < RPW; r += 2) {
#pragma unroll
      for (int vv = 0; vv < 2; ++vv) {
        const float v0 = __uint_as_float(vv ? rv_[r] & 0xffff0000u : rv_[r] << 16);
        const float v1 = __uint_as_float(vv ? rv_[r + 1] & 0xffff0000u : rv_[r + 1] << 16);
        bvc[vv][r / 2] = __builtin_bit_cast(unsigned, bf16x2{(__bf16)(bt[r] * v0), (__bf16)(bt[r + 1] * v1)});
      }
    }
    float sk[RPW], sq[RPW], dq[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      sk[r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, rk_[r]), __builtin_bit_cast(bf16x2, rk_[r]),
                                              kL2EpsLane, false);
      sq[r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, rq_[r]), __builtin_bit_cast(bf16x2, rq_[r]),
                                              kL2EpsLane, false);
      dq[r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, rk_[r]), __builtin_bit_cast(bf16x2, rq_[r]),
                                              0.f, false);
    }
    float tw[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      float run = 0.f;
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        run += gx[r][cc];
        gx[r][cc] = run;
      }
      tw[cc] = run;
    }
    *reinterpret_cast<float2*>(sTot + w * 128 + c_lo) = float2{tw[0], tw[1]};
    // 1 / |row| for q and k and, in the first chunk, the diagonal of A_qk
    float rkn[RPW], rqn[RPW];
    const bool exact_diag = t0 == 0;
    if (exact_diag) {
      rows_norms_diag(sk, sq, dq, p.l2norm != 0, scale, l, rkn, rqn, sDiag + RPW * w);
    } else if (p.l2norm) {
      rows_rsqrt(sk, rkn);
      rows_rsqrt(sq, rqn);
    } else {
#pragma unroll
      for (int r = 0; r < RPW; ++r) rkn[r] = rqn[r] = 1.f;
    }
    lds_barrier();
    // (beta V)^T, after the barrier: the region held the previous chunk's
    // output staging, read before it
#pragma unroll
    for (int vv = 0; vv < 2; ++vv) {
#pragma unroll
      for (int j = 0; j < RPW / 4; ++j)
        *reinterpret_cast<uint2*>(sVT + tu_pos(c_lo + vv, RPW * w + 4 * j)) = uint2{bvc[vv][2 * j], bvc[vv][2 * j + 1]};
    }

    // gamma in log2 units relative to the reference row m, the range guard
    const int mw = L > 32 ? 2 : 1;  // waves whose rows precede the reference row
    float gm[2], gL[2];
    float guard = 0.f;
    float totw[NW][2];
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float2 t2 = *reinterpret_cast<const float2*>(sTot + ww * 128 + c_lo);
      totw[ww][0] = t2.x;
      totw[ww][1] = t2.y;
    }
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      float pre[NW + 1];
      pre[0] = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) pre[ww + 1] = pre[ww] + totw[ww][cc];
      const float tot = pre[NW];
      const float ref = mw == 2 ? pre[2] : pre[1];
      float off = pre[0];
      off = pre[w];
      gm[cc] = ref * kLog2e;
      gL[cc] = tot * kLog2e;
      const float nref = (off - ref) * kLog2e;
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        gx[r][cc] = fmaf(gx[r][cc], kLog2e, nref);
        guard = fmaxf(guard, fabsf(gx[r][cc]));
      }
      guard = fmaxf(guard, fmaxf(gm[cc], gL[cc] - gm[cc]));
    }
    guard = wave_max(guard);
    if (l == 0) sRed[w] = guard;

    // ---------------- phase A: KL, KR, QL; KE, KB, Qg kept as bf16 pairs ----
    // KE and KB as bf16 pairs of consecutive rows of one channel (the layout
    // of their transposed tiles), Qg as pairs of this lane's two channels
    unsigned kec[2][RPW / 2], kbc[2][RPW / 2], qgp[RPW];
    {
      float pke[2], pkb[2];  // the even row's values, packed with the odd row's
      float cg[2], cb[2];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        cg[cc] = __builtin_amdgcn_exp2f(gm[cc]);           // 2^gamma_m
        cb[cc] = __builtin_amdgcn_exp2f(gL[cc] - gm[cc]);  // 2^(gamma_L - gamma_m)
        if (w == 0) sDec[c_lo + cc] = __builtin_amdgcn_exp2f(gL[cc]);
      }
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const int i = RPW * w + r;
        const float bk = bt[r] * rkn[r];
        const float sqr = scale * rqn[r];
        float fkl[2], fkr[2], fql[2];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const float kx = __uint_as_float(cc == 0 ? rk_[r] << 16 : rk_[r] & 0xffff0000u);
          const float qx = __uint_as_float(cc == 0 ? rq_[r] << 16 : rq_[r] & 0xffff0000u);
          const float d = gx[r][cc];                     // gamma_i - gamma_m
          const float e1 = __builtin_amdgcn_exp2f(d);
          const float e2 = __builtin_amdgcn_exp2f(-d);
          fkl[cc] = kx * e1 * bk;      // beta k^ 2^(gamma_i - gamma_m)
          fkr[cc] = kx * e2 * rkn[r];  // k^ 2^(gamma_m - gamma_i)
          fql[cc] = qx * e1 * sqr;     // scale q^ 2^(gamma_i - gamma_m)
        }
        *reinterpret_cast<bf16x2*>(sKL + rs_pos(i, c_lo)) = bf16x2{(__bf16)fkl[0], (__bf16)fkl[1]};
        *reinterpret_cast<bf16x2*>(sKR + rs_pos(i, c_lo)) = bf16x2{(__bf16)fkr[0], (__bf16)fkr[1]};
        *reinterpret_cast<bf16x2*>(sQL + rs_pos(i, c_lo)) = bf16x2{(__bf16)fql[0], (__bf16)fql[1]};
        qgp[r] = __builtin_bit_cast(unsigned, bf16x2{(__bf16)(fql[0] * cg[0]), (__bf16)(fql[1] * cg[1])});
        // packed here: left to itself the compiler keeps the fp32 products
        // live through phase B and converts them at their stores
        asm volatile("" : "+v"(qgp[r]));
        if (r & 1) {
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            kec[cc][r / 2] = __builtin_bit_cast(unsigned, bf16x2{(__bf16)pke[cc], (__bf16)(fkl[cc] * cg[cc])});
            kbc[cc][r / 2] = __builtin_bit_cast(unsigned, bf16x2{(__bf16)pkb[cc], (__bf16)(fkr[cc] * cb[cc])});
            asm volatile("" : "+v"(kec[cc][r / 2]), "+v"(kbc[cc][r / 2]));
          }
        } else {
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            pke[cc] = fkl[cc] * cg[cc];
            pkb[cc] = fkr[cc] * cb[cc];
          }
        }
      }
    }
    lds_barrier();
    bool retry;
    {
      // range guard of every wave: a span whose gate factors would leave
      // 2^+-100 is re-processed as shorter chunks
      float gmax = sRed[0];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) gmax = fmaxf(gmax, sRed[ww]);
      retry = gmax > kRangeLimit && L > 1;
    }
    // The next rows are loaded at one place for both paths (below): the
    // structurised control flow of a `continue`, or of loads on both sides
    // of an if/else, keeps the words loaded on one path live (undefined)
    // through the other path's phases.
    uint32_t dr = 0;  // the chunk whose rows are loaded next starts dr tokens after this one
    if (retry) {
      Lcap = L > 16 ? 16 : (L > 4 ? 4 : 1);
    } else {
      // ---------------- phase B: A_kk (fp32 diagonal / bf16 below) and A_qk ----
      // The ten 16x16 block pairs (bi >= bj) in two steps: each wave first
      // takes the diagonal pair of its own rows (A_kk's fp32 diagonal blocks
      // are all phase C needs), then wave 0 inverts them (phase C) while waves
      // 1-3 take the six pairs below the diagonal, two each.
      auto pairs = [&](auto npc, auto pick) __attribute__((always_inline)) {
        constexpr int NP = decltype(npc)::value;
        int bi[NP], bj[NP];
#pragma unroll
        for (int m = 0; m < NP; ++m) pick(m, bi[m], bj[m]);
        f32x4 akk[NP], aqk[NP];
        bf16x8 oL[2][NP], oR[2][NP], oQ[2][NP];
        auto fetch = [&](int ks, int bf) __attribute__((always_inline)) {
#pragma unroll
          for (int m = 0; m < NP; ++m) {
            oR[bf][m] = ld8(sKR + rs_pos(16 * bj[m] + lr, 32 * ks + 8 * lg));
            oL[bf][m] = ld8(sKL + rs_pos(16 * bi[m] + lr, 32 * ks + 8 * lg));
            oQ[bf][m] = ld8(sQL + rs_pos(16 * bi[m] + lr, 32 * ks + 8 * lg));
          }
        };
#pragma unroll
        for (int m = 0; m < NP; ++m) {
          akk[m] = f32x4{0.f, 0.f, 0.f, 0.f};
          aqk[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        fetch(0, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ks + 1 < KS) fetch(ks + 1, (ks + 1) & 1);
#pragma unroll
          for (int m = 0; m < NP; ++m) {
            akk[m] = mfma(oL[ks & 1][m], oR[ks & 1][m], akk[m]);
            aqk[m] = mfma(oR[ks & 1][m], oQ[ks & 1][m], aqk[m]);
          }
        }
#pragma unroll
        for (int m = 0; m < NP; ++m) {
          if (bi[m] != bj[m]) {
#pragma unroll
            for (int e = 0; e < 4; ++e) sAb[ab_pos(bi[m], bj[m], 4 * lg + e, lr)] = (__bf16)(-akk[m][e]);
          } else {  // rows 4lg..4lg+3 of column lr, fp32, one 16-byte store
            f32x4 d;
#pragma unroll
            for (int e = 0; e < 4; ++e) d[e] = 4 * lg + e > lr ? akk[m][e] : 0.f;
            *reinterpret_cast<f32x4*>(sAd + ad_pos(bi[m], 4 * lg, lr)) = d;
          }
          // A_qk row 16bi + lr, columns 16bj + 4lg + e: kpos 8lg + 4(bj & 1) + e of 32-block bj >> 1;
          // the fp32 diagonal from sDiag
          const int i = 16 * bi[m] + lr, j0 = 16 * bj[m] + 4 * lg;
          f32x4 a;
#pragma unroll
          for (int e = 0; e < 4; ++e) a[e] = i >= j0 + e ? aqk[m][e] : 0.f;
          if (exact_diag && bi[m] == bj[m] && (lr >> 2) == lg) a[lr & 3] = sDiag[i];
          *reinterpret_cast<bf16x4*>(sAqk + aqk_pos(bj[m] >> 1, bi[m], lr, 8 * lg + 4 * (bj[m] & 1))) =
              to_bf16x4(a[0], a[1], a[2], a[3]);
        }
      };
      pairs(std::integral_constant<int, 1>{}, [&](int, int& bi, int& bj) { bi = bj = w; });
      lds_barrier();

      // ---------------- phase C: D_b = (I + A_bb)^-1; the pairs below the diagonal --
      if (w == 0) {
        // fp32 forward substitution; lane = (block, column)
        const int bb = l >> 4;
        int col = l & 15;
        asm volatile("" : "+v"(col));
        const float* Ab = sAd + bb * AD_B;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (i == col) ? 1.f : 0.f;
        // columns j + 1 and j + 2 in flight during step j (a ring of three)
        f32x4 cr[3][4];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int q = 0; q < 4; ++q) cr[c][q] = *reinterpret_cast<const f32x4*>(Ab + ad_pos(0, 4 * q, c));
#pragma unroll
        for (int j = 0; j < 15; ++j) {
          if (j + 2 < 15) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (4 * q + 3 > j + 2) cr[(j + 2) % 3][q] = *reinterpret_cast<const f32x4*>(Ab + ad_pos(0, 4 * q, j + 2));
          }
#pragma unroll
          for (int i = j + 1; i < 16; ++i) x[i] -= cr[j % 3][i >> 2][i & 3] * x[j];
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sAb[ab_pos(bb, bb, i, col)] = (__bf16)x[i];
      } else {
        // wave w: entries 2(w - 1) and 2w - 1 of (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
        pairs(std::integral_constant<int, 2>{}, [&](int m, int& bi, int& bj) {
          const int e = 2 * (w - 1) + m;
          bi = e < 1 ? 1 : (e < 3 ? 2 : 3);
          bj = e - ((bi - 1) * bi) / 2;
        });
      }
      lds_barrier();

      // ---------------- KE, KB, Qg over KL, KR, QL (phase B has read them) ----
#pragma unroll
      for (int r = 0; r < RPW; ++r) *reinterpret_cast<unsigned*>(sQg + rs_pos(RPW * w + r, kpos(c_lo))) = qgp[r];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
        for (int j = 0; j < RPW / 4; ++j) {
          *reinterpret_cast<uint2*>(sKE + tu_pos(c_lo + cc, RPW * w + 4 * j)) = uint2{kec[cc][2 * j], kec[cc][2 * j + 1]};
          *reinterpret_cast<uint2*>(sKB + kb_pos(c_lo + cc, RPW * w + 4 * j)) = uint2{kbc[cc][2 * j], kbc[cc][2 * j + 1]};
        }
      }
      lds_barrier();

      // ---------------- phase D: [W | U] = (I + A_kk)^-1 [beta K 2^gamma | beta V] --
      // wave w: the W tiles of channels 32w + 16m + lr (m = 0, 1) and the U
      // tiles of its value columns 32w + 16m + lr (m = 2, 3), four independent
      // chains of the blocked substitution X_b = D_b (R_b - sum_{c<b} A_bc X_c).
      // Each W block is also taken transposed (operands swapped), so that a lane
      // holds four consecutive channels of one token, and stored as -W at once
      // over this wave's own pair of beta K 2^gamma (all of it read up front).
      f32x4 U[2][4];
      // O^T = S^T Qg^T + V_new^T A_qk^T, its first term here: it needs only Qg
      // and this wave's S, and its MFMAs fill the gaps of the dependent chain
      f32x4 O[2][4];
      {
        s16x4 ab[4][4];
        bf16x4 rb[4][4];
#pragma unroll
        for (int bk = 0; bk < 4; ++bk) {
#pragma unroll
          for (int c = 0; c <= bk; ++c) ab[bk][c] = ld4s(sAb + ab_pos(bk, c, lr, 4 * lg));
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            rb[m][bk] = *reinterpret_cast<const bf16x4*>(sKE + tu_pos(32 * w + 16 * m + lr, 16 * bk + 4 * lg));
            rb[2 + m][bk] = *reinterpret_cast<const bf16x4*>(sVT + tu_pos(32 * w + 16 * m + lr, 16 * bk + 4 * lg));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        // the bf16 identity as an A operand (lane: row lr, columns 4lg..4lg+3):
        // an MFMA with it widens a right-hand side to the C layout in fp32
        // exactly, on the matrix cores instead of four VALU conversions
        s16x4 ident;
#pragma unroll
        for (int e = 0; e < 4; ++e) ident[e] = (short)(lr == 4 * lg + e ? 0x3f80 : 0);
        s16x4 xb[4][4];
#pragma unroll
        for (int bk = 0; bk < 4; ++bk) {
          s16x4 r[4];
          if (bk == 0) {  // R_0 as loaded: bf16 already
#pragma unroll
            for (int m = 0; m < 4; ++m) r[m] = __builtin_bit_cast(s16x4, rb[m][0]);
          } else {
            f32x4 acc[4];
#pragma unroll
            for (int m = 0; m < 4; ++m)
              acc[m] = mfma16(ident, __builtin_bit_cast(s16x4, rb[m][bk]), f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int c = 0; c < bk; ++c) {
#pragma unroll
              for (int m = 0; m < 4; ++m) acc[m] = mfma16(ab[bk][c], xb[m][c], acc[m]);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) r[m] = pack4(acc[m]);
          }
          const s16x4 d = ab[bk][bk];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const f32x4 x = mfma16(d, r[m], f32x4{0.f, 0.f, 0.f, 0.f});
            if (bk < 3) xb[m][bk] = pack4(x);
            if (m >= 2) {
              U[m - 2][bk] = x;
            } else {
              const f32x4 xt = mfma16(r[m], d, f32x4{0.f, 0.f, 0.f, 0.f});
              *reinterpret_cast<bf16x4*>(sKE + 2048 * w + w_pos(16 * bk + lr, 8 * lg + 4 * m)) =
                  to_bf16x4(-xt[0], -xt[1], -xt[2], -xt[3]);
            }
          }
        }
      }
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) O[m][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 aq[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) aq[rt] = ld8(sQg + rs_pos(16 * rt + lr, 32 * ks + 8 * lg));
        const bf16x8 b0 = pack_perm(S[0][2 * ks], S[0][2 * ks + 1]);
        const bf16x8 b1 = pack_perm(S[1][2 * ks], S[1][2 * ks + 1]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          O[0][rt] = mfma(b0, aq[rt], O[0][rt]);
          O[1][rt] = mfma(b1, aq[rt], O[1][rt]);
        }
      }
      lds_barrier();

      // ---------------- phase E: the serial chain on this wave's 32 columns ----
      // V_new = U - W S, O = Qg S + A_qk V_new, S = D S + Kbar^T V_new; each LDS
      // operand read serves both column tiles.  The output is computed
      // transposed, O^T = S^T Qg^T + V_new^T A_qk^T: tile rt holds, per lane,
      // value columns 32w + 16m + 4lg.. of token 16rt + lr.  The two products
      // with S run together, one contraction step at a time, the next step's
      // W and Qg operands read ahead.
      f32x4 (&Vn)[2][4] = U;
      {
        bf16x8 aw[2][4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) aw[0][rt] = ld8(sKE + w_pos(16 * rt + lr, 8 * lg));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ks + 1 < KS) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) aw[(ks + 1) & 1][rt] = ld8(sKE + 2048 * (ks + 1) + w_pos(16 * rt + lr, 8 * lg));
          }
          const bf16x8 b0 = pack_perm(S[0][2 * ks], S[0][2 * ks + 1]);
          const bf16x8 b1 = pack_perm(S[1][2 * ks], S[1][2 * ks + 1]);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            Vn[0][rt] = mfma(aw[ks & 1][rt], b0, Vn[0][rt]);
            Vn[1][rt] = mfma(aw[ks & 1][rt], b1, Vn[1][rt]);
          }
        }
      }
      bf16x8 bV[2][2];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) bV[m][q2] = pack_perm(Vn[m][2 * q2], Vn[m][2 * q2 + 1]);
      {
        bf16x8 aq[6];
#pragma unroll
        for (int t = 0; t < 6; ++t) {
          const int q2 = t < 4 ? 0 : 1, rt = t < 4 ? t : t - 2;
          aq[t] = ld8(sAqk + aqk_pos(q2, rt, lr, 8 * lg));
        }
#pragma unroll
        for (int t = 0; t < 6; ++t) {
          const int q2 = t < 4 ? 0 : 1, rt = t < 4 ? t : t - 2;
          O[0][rt] = mfma(bV[0][q2], aq[t], O[0][rt]);
          O[1][rt] = mfma(bV[1][q2], aq[t], O[1][rt]);
        }
      }
      {
        // S = D S + Kbar^T V_new: a ring of four Kbar^T operands in flight
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) {
          const f32x4 dec = *reinterpret_cast<const f32x4*>(sDec + 16 * ct + 4 * lg);
          S[0][ct] *= dec;
          S[1][ct] *= dec;
        }
        constexpr int NU = 2 * KT;
        const int kb0 = lr * kC + 8 * (lg ^ ((lr >> 1) & 7)), kb1 = lr * kC + 8 * ((4 + lg) ^ ((lr >> 1) & 7));
        bf16x8 kr[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) kr[t] = ld8(sKB + 16 * kC * (t % KT) + (t / KT ? kb1 : kb0));
#pragma unroll
        for (int t = 0; t < NU; ++t) {
          const int q2 = t / KT, ct = t % KT;
          S[0][ct] = mfma(kr[t & 3], bV[0][q2], S[0][ct]);
          S[1][ct] = mfma(kr[t & 3], bV[1][q2], S[1][ct]);
          if (t + 4 < NU) {
            const int q2n = (t + 4) / KT, ctn = (t + 4) % KT;
            kr[t & 3] = ld8(sKB + 16 * kC * ctn + (q2n ? kb1 : kb0));
          }
        }
      }
      // ---------------- output rows of this chunk ---------------------------
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          *reinterpret_cast<bf16x4*>(sO + rs_pos(16 * rt + lr, 32 * w + 16 * m + 4 * lg)) =
              to_bf16x4(O[m][rt][0], O[m][rt][1], O[m][rt][2], O[m][rt][3]);
      dr = L;
    }
    // the next chunk's rows (zeros past the end: the loaded words then hold
    // constants, not this chunk's values, across the loop's back edge)
    if (t0 + dr < lenu) {
      const uint32_t left = lenu - t0 - dr;
      issue_loads(dr, left < (uint32_t)kC ? left : (uint32_t)kC, w);
    } else {
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        rk_[r] = rq_[r] = rv_[r] = rb_[r] = 0u;
        rg_[r][0] = rg_[r][1] = 0.f;
      }
    }
    if (!retry) {
      lds_barrier();
      {
        // 32-bit lane offsets from the chain's output pointer; written once,
        // non-temporal
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        const uint32_t row_b = Hu * 256;
#pragma unroll
        for (int u0 = 0; u0 < kC * 16; u0 += NT) {
          const int u = u0 + tid_i;
          const int i = u >> 4, cv = u & 15;
          if ((uint32_t)i < L)
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4, ld8(sO + rs_pos(i, 8 * cv))),
                                        reinterpret_cast<u32x4*>(op + ((uint32_t)i * row_b + 16 * (uint32_t)cv)));
        }
      }
      // advance the chain's pointers past this chunk
      const int64_t adv = (int64_t)L * H;
      kp += adv * 256;
      qp += adv * 256;
      vp += adv * 256;
      gp += adv * 512;
      bp += adv * (kBetaBF16 ? 2 : 4);
      op += adv * 256;
      t0 += L;
      Lcap = kC;
      if (t0 == ck_next) {
        if (ck_row >= 0 && ck_row < ck_end) {
          int tid_c = tid;
          asm volatile("" : "+v"(tid_c));
#pragma unroll
          for (int m = 0; m < 2; ++m)
            store_state(S[m], p.ckpt, p.ckpt_bf16, p.svec, ((int64_t)ck_row * H + h) * V, (tid_c & 63) >> 4,
                        32 * w + 16 * m + (tid_c & 15), K, V);
        }
        ck_next += ck_iv;
        ++ck_row;
      }
    }
  }

  if (p.fin && fin_ok) {
#pragma unroll
    for (int m = 0; m < 2; ++m) store_state(S[m], p.fin, p.fin_bf16, p.svec, frow, lg, 32 * w + 16 * m + lr, K, V);
  }
}

// First-segment length for segments of lc tokens: a map chunk costs about
// 0.8 of an output chunk (measured at K = V = 128, with both in one launch),
// so a first segment of 0.8 lc tokens (its outputs, in pass 1) ends with the
// middle segments' maps; a multiple of 64, at least 64.
__host__ __device__ inline int64_t seg_first_len(int64_t lc) {
  const int64_t l0 = (lc * 800 / 1000 + 32) / 64 * 64;
  return l0 < 64 ? 64 : l0;
}

// ---------------------------------------------------------------------------
// Segment-parallel prefill of long sequences.  When a batch has too few
// (sequence, head) chains to fill the GPU, every sequence is cut into a first
// segment of l0 tokens and further segments of lc tokens.  A segment acts on
// the state as an affine map F(S) = M S + b (maps compose in order; the
// composition is associative):
//   pass 1 : in one launch, side by side: the first segment of each sequence
//            from the sequence's initial state -> its outputs and its final
//            state (S_in of the second segment); and every middle segment
//            (neither first nor last): from a zero state -> b, and from the
//            identity with zero values -> M (the same chunk operators act on
//            both)
//   scan   : S_in(next) = M S_in + b from the second segment on
//   pass 2 : every segment but the first from its S_in -> outputs; the last
//            segment of each sequence writes the sequence's final state
// A map chunk costs about l0 / lc (0.8) of an output chunk, so the first
// segment's outputs end with the maps.  When splitting would not pay (the
// planning kernel estimates both ways from the lengths), every sequence is
// one segment and pass 1 runs whole sequences.
// All segments of all sequences run in parallel in passes 1 and 2.
// ---------------------------------------------------------------------------

// Segment table: scu[0..nmax] token offsets of the segments (entries past the
// last real segment are T, i.e. empty segments); sfirst[n] is the first
// segment of sequence n, sfirst[N] the number of real segments; sseq[s] is
// the sequence of segment s (0 for the empty ones).
__global__ __launch_bounds__(1024) void seg_plan_kernel(const int32_t* __restrict__ cu, int64_t N, int64_t T,
                                                        int64_t H, int64_t lc_min, int64_t nmax,
                                                        int32_t* __restrict__ scu, int32_t* __restrict__ sfirst,
                                                        int32_t* __restrict__ sseq) {
  __shared__ int32_t cnt[1025], first[1025];
  __shared__ int64_t lens[2];
  if (threadIdx.x == 0) {
    // lc: the smallest multiple of 64 from lc_min whose segments after the
    // first make at most 256 pass-2 items (H per segment), by bisection (the
    // count does not grow with lc); l0 = seg_first_len(lc)
    auto items = [&](int64_t lc) {
      const int64_t l0 = seg_first_len(lc);
      int64_t c = 0;
      for (int64_t n = 0; n < N; ++n) {
        int64_t b0 = cu[n], e0 = cu[n + 1];
        b0 = b0 < 0 ? 0 : (b0 > T ? T : b0);
        e0 = e0 < b0 ? b0 : (e0 > T ? T : e0);
        const int64_t len = e0 - b0;
        c += len <= l0 ? 0 : (len - l0 + lc - 1) / lc;
      }
      return c * H;
    };
    int64_t lo = lc_min / 64, hi = (T + 63) / 64 + lo;  // items(64 hi) <= H N <= 256
    while (lo < hi) {
      const int64_t mid = (lo + hi) / 2;
      if (items(64 * mid) <= 256) hi = mid; else lo = mid + 1;
    }
    lens[0] = seg_first_len(64 * lo);
    lens[1] = 64 * lo;
  }
  __syncthreads();
  const int64_t l0 = lens[0], lc = lens[1];
  for (int64_t n = threadIdx.x; n < N; n += blockDim.x) {
    int64_t b0 = cu[n], e0 = cu[n + 1];
    b0 = b0 < 0 ? 0 : (b0 > T ? T : b0);
    e0 = e0 < b0 ? b0 : (e0 > T ? T : e0);
    // the first segment takes l0 tokens, the others lc; an empty sequence
    // keeps one (empty) segment
    const int64_t len = e0 - b0;
    cnt[n] = (int32_t)(len <= l0 ? 1 : 1 + (len - l0 + lc - 1) / lc);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    // Split only where it pays, in thousandths of one output chunk (64
    // tokens): whole sequences take the longest one's chunks; split, pass 1
    // takes max(l0, 0.825 lc) (the first segments' outputs beside the maps),
    // pass 2 lc, the scan about 0.95 per composed map and the two extra
    // launches about 6 (measured at K = V = 128, H = 32).
    int32_t cmax = 0;
    int64_t lmax = 0;
    for (int64_t n = 0; n < N; ++n) {
      cmax = cnt[n] > cmax ? cnt[n] : cmax;
      int64_t b0 = cu[n], e0 = cu[n + 1];
      b0 = b0 < 0 ? 0 : (b0 > T ? T : b0);
      e0 = e0 < b0 ? b0 : (e0 > T ? T : e0);
      lmax = e0 - b0 > lmax ? e0 - b0 : lmax;
    }
    const int64_t whole = 1000 * ((lmax + 63) / 64);
    const int64_t p1 = cmax >= 3 ? (1000 * l0 > 825 * lc ? 1000 * l0 : 825 * lc) / 64 : 1000 * l0 / 64;
    const int64_t split = p1 + 1000 * lc / 64 + (cmax >= 3 ? 950 * (cmax - 2) : 0) + 6000;
    const bool seg = cmax >= 2 && split < whole;
    // prefix sums, clamped to nmax so that offsets that break the cu_seqlens
    // precondition still cannot index past the workspace
    int64_t run = 0;
    for (int64_t n = 0; n < N; ++n) {
      const int64_t c = seg ? cnt[n] : 1;
      first[n] = (int32_t)run;
      run = run + c < nmax ? run + c : nmax;
    }
    first[N] = (int32_t)run;
  }
  __syncthreads();
  for (int64_t n = threadIdx.x; n <= N; n += blockDim.x) sfirst[n] = first[n];
  for (int64_t n = threadIdx.x; n < N; n += blockDim.x) {
    int64_t b0 = cu[n], e0 = cu[n + 1];
    b0 = b0 < 0 ? 0 : (b0 > T ? T : b0);
    e0 = e0 < b0 ? b0 : (e0 > T ? T : e0);
    for (int64_t j = 0; first[n] + j < first[n + 1]; ++j) {
      scu[first[n] + j] = (int32_t)(j == 0 ? b0 : b0 + l0 + (j - 1) * lc);
      sseq[first[n] + j] = (int32_t)n;
    }
  }
  for (int64_t s = first[N] + threadIdx.x; s <= nmax; s += blockDim.x) {
    scu[s] = (int32_t)T;
    if (s < nmax) sseq[s] = 0;
  }
}

// Composes the segment maps of one (sequence, head) in fp32, for one block
// of kScanCols value columns (the columns of S evolve independently under
// S <- M S + b); 256 threads, K, V <= 128.  Starts from the initial state of
// the sequence's second segment (row sfirst[n] + 1 of S_in, [nmax, H, V, K]
// fp32, written by pass 1) and writes those of the third segment on.  The
// first segment has no map (pass 1 ran it from the true initial state) and
// neither has the last (its pass-2 run writes the final state).
//
// The map of a segment is stored as the state that pass 1 propagated from
// the identity: row x of the [K][K] tile holds M's column x, so
// S_new[r] = b[r] + sum_x T[x][r] S[x].  T is kept in LDS as stored (thread
// r reads column r: consecutive addresses across lanes) and the next
// segment's T and b are loaded into registers while this segment's product
// runs (K % 4 == 0: 16-byte loads; other K: element loads, not prefetched).
constexpr int kScanCols = 8;
constexpr int kScanT = 256;                      // threads
constexpr int kScanSL = kScanCols + 4;           // sS row stride (16-byte aligned rows)
constexpr int kScanML = 128 + 4;                 // sT row stride
constexpr int kScanV4 = 128 * 128 / 4 / kScanT;  // float4 of a 128 x 128 tile per thread

__global__ __launch_bounds__(kScanT) void seg_scan_kernel(const int32_t* __restrict__ sfirst, const float* __restrict__ bmap,
                                                          const float* __restrict__ mmap, float* __restrict__ sin,
                                                          int64_t H, int64_t K, int64_t V) {
  __shared__ __attribute__((aligned(16))) float sS[128 * kScanSL];  // S[c][v - v0]
  __shared__ __attribute__((aligned(16))) float sT[128 * kScanML];  // T[x][c]
  const int64_t ncb = (V + kScanCols - 1) / kScanCols;
  const int64_t item = blockIdx.x / ncb;
  const int64_t v0 = (blockIdx.x - item * ncb) * kScanCols;
  const int64_t n = item / H, h = item % H;
  const int tid = threadIdx.x;
  // the maps of segments s0 .. s1 - 2 are composed (uniform)
  const int64_t s0 = sfirst[n] + 1, s1 = sfirst[n + 1];
  if (s0 + 1 >= s1) return;
  const bool vec = (K & 3) == 0;
  const int nv4 = (int)(K * K / 4);      // float4 of a K x K tile
  // coalesced element order: e -> (column vl, channel c), c fastest
  for (int e = tid; e < kScanCols * 128; e += kScanT) {
    const int c = e & 127, vl = e >> 7;
    float x = 0.f;
    if (c < K && v0 + vl < V) x = sin[((s0 * H + h) * V + v0 + vl) * K + c];
    sS[c * kScanSL + vl] = x;
  }
  const int r = tid >> 1;                      // this thread's state row (key channel)
  const int j0 = (tid & 1) * (kScanCols / 2);  // and its kScanCols / 2 columns
  f32x4 tr[kScanV4];        // the next segment's T (vector path)
  float br[kScanCols / 2];  // and this thread's b entries
  auto fetch = [&](int64_t sg) {
    const float* tb = mmap + (sg * H + h) * K * K;
    if (vec) {
#pragma unroll
      for (int u = 0; u < kScanV4; ++u) {
        const int f = u * kScanT + tid;
        if (f < nv4) tr[u] = *reinterpret_cast<const f32x4*>(tb + 4 * (int64_t)f);
      }
    }
#pragma unroll
    for (int j = 0; j < kScanCols / 2; ++j) {
      const int64_t v = v0 + j0 + j;
      br[j] = (r < K && v < V) ? bmap[((sg * H + h) * V + v) * K + r] : 0.f;
    }
  };
  fetch(s0);
  __syncthreads();
  for (int64_t sg = s0; sg < s1; ++sg) {
    if (sg > s0) {  // S_in of segment sg (that of s0 came from pass 1)
      const int64_t srow_s = (sg * H + h) * V;
      for (int e = tid; e < kScanCols * 128; e += kScanT) {
        const int c = e & 127, vl = e >> 7;
        if (v0 + vl < V && c < K) sin[(srow_s + v0 + vl) * K + c] = sS[c * kScanSL + vl];
      }
    }
    if (sg + 1 == s1) break;  // uniform: the last segment's map is not composed
    if (vec) {
      const int q4 = (int)(K / 4);  // float4 per row
#pragma unroll
      for (int u = 0; u < kScanV4; ++u) {
        const int f = u * kScanT + tid;
        if (f < nv4) {
          const int x = f / q4, c4 = f - x * q4;
          *reinterpret_cast<f32x4*>(sT + x * kScanML + 4 * c4) = tr[u];
        }
      }
    } else {
      const float* tb = mmap + (sg * H + h) * K * K;
      for (int e = tid; e < K * K; e += kScanT) {
        const int x = (int)(e / K), c = (int)(e - x * K);
        sT[x * kScanML + c] = tb[e];
      }
    }
    float acc[kScanCols / 2];
#pragma unroll
    for (int j = 0; j < kScanCols / 2; ++j) acc[j] = br[j];
    __syncthreads();
    if (sg + 2 < s1) fetch(sg + 1);  // lands while the product below runs
    if (r < K) {
      for (int x = 0; x < K; ++x) {
        const float m = sT[x * kScanML + r];
#pragma unroll
        for (int q = 0; q < kScanCols / 8; ++q) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(sS + x * kScanSL + j0 + 4 * q);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[4 * q + j] += m * a[j];
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kScanCols / 2; ++j) sS[r * kScanSL + j0 + j] = acc[j];
    __syncthreads();
  }
}

// K = V = 128 with bf16 q/k/v can run two chains per CU
// (chunk_prefill_2wg_kernel).  Whether that pays depends on the batch: on a
// CU of its own one chain of it is about a third slower than on the 8 waves of
// chunk_prefill_kernel, and two on a CU take 1.78 of that time per chunk each
// (H = 32, K = V = 128 against the 8-wave kernel: 8x4096 tokens +32 %, 12x4096
// -13 %, 16x2048 -9 %, 20x2048 and 24x2048 -5 %, 32x2048 -8 %, 64x1024 -11 %,
// 200 sequences of 64-8192 tokens -12 %; 16 sequences of 512-4096 tokens -2 %
// to +17 %, as the longest chains share their CUs).  With more chains than
// CUs the planning kernel chooses from the lengths and both kernels are
// launched, the one not chosen returning at once; without a plan (one
// sequence) the two-chains kernel runs from this many chains on.
constexpr int64_t kTwoPerCuMinChains = 1024;

bool two_per_cu_shape(const Params& prm, bool bf16) {
  return bf16 && prm.K == 128 && prm.V == 128 && prm.pair && prm.ovec && prm.T <= INT32_MAX && prm.H <= 65535 &&
         !prm.seq_of;
}

// Compute units of the current device (cached per device).
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int cus[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (!cus[dev]) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
    cus[dev] = c;
  }
  return cus[dev];
}

template <int KP, int BV>
hipError_t launch_cfg(const Params& prm, bool bf16, hipStream_t stream) {
  const int64_t items = prm.N * prm.H;
  const int64_t groups = (items + 7) / 8;
  const int64_t grid = groups * 8 * prm.nvb;
  constexpr int nt = Cfg<KP, BV>::NT;
  const dim3 g3((unsigned)grid), b3(nt);
  // the 8-wave kernel obeys the plan's choice only beside the two-chains one
  Params p8 = prm;
  p8.sel = nullptr;
  if constexpr (KP == 128 && BV == 128) {
    if (two_per_cu_shape(prm, bf16) && (prm.sel || items >= kTwoPerCuMinChains)) {
      Params p2 = prm;
      p2.sel_want = 1;
      if (prm.beta_bf16)
        hipLaunchKernelGGL(chunk_prefill_2wg_kernel<true>, dim3((unsigned)items), dim3(w2::NT), 0, stream, p2);
      else
        hipLaunchKernelGGL(chunk_prefill_2wg_kernel<false>, dim3((unsigned)items), dim3(w2::NT), 0, stream, p2);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess || !prm.sel) return e;
      // the 8-wave kernel below runs when the plan chose it
      p8.sel = prm.sel;
      p8.sel_want = 0;
    }
  }
  if (prm.seq_of) {
    if (bf16)
      hipLaunchKernelGGL((chunk_prefill_kernel<KP, BV, true, true>), g3, b3, 0, stream, p8);
    else
      hipLaunchKernelGGL((chunk_prefill_kernel<KP, BV, false, true>), g3, b3, 0, stream, p8);
  } else {
    if (bf16)
      hipLaunchKernelGGL((chunk_prefill_kernel<KP, BV, true, false>), g3, b3, 0, stream, p8);
    else
      hipLaunchKernelGGL((chunk_prefill_kernel<KP, BV, false, false>), g3, b3, 0, stream, p8);
  }
  return hipGetLastError();
}

// Vector-access flags of a parameter set (from sizes and pointer alignment).
void set_access_flags(Params& prm) {
  const uintptr_t al = (uintptr_t)prm.q | (uintptr_t)prm.k | (uintptr_t)prm.v | (uintptr_t)prm.g;
  prm.pair = (prm.K % 2 == 0) && (prm.V % 2 == 0) && (al % 8 == 0);
  prm.ovec = (prm.V % 8 == 0) && ((uintptr_t)prm.out % 16 == 0);
  const uintptr_t sal = (uintptr_t)prm.init | (uintptr_t)prm.fin | (uintptr_t)prm.ckpt | (uintptr_t)prm.mmap |
                        (uintptr_t)prm.sin_next;
  prm.svec = (prm.K % 4 == 0) && (sal % 16 == 0);
}

// Pass 1 of the segment-parallel path (chunk_prefill_seg1_kernel): both roles
// with the value blocks of the map pass (128 columns, 64 for K <= 64).
hipError_t launch_seg1(Params pout, Params pmap, bool bf16, hipStream_t stream) {
  set_access_flags(pout);
  set_access_flags(pmap);
  pmap.svec = pout.svec = pout.svec && pmap.svec;
  const bool small = pout.K <= 64;
  pout.nvb = pmap.nvb = (int)(small ? (pout.V + 63) / 64 : (pout.V + 127) / 128);
  const int64_t grid = (pout.N * pout.H + 7) / 8 * 8 * pout.nvb;
  const dim3 g3((unsigned)grid), b3(small ? 256 : 512);
  if (small) {
    if (bf16)
      hipLaunchKernelGGL((chunk_prefill_seg1_kernel<64, 64, true>), g3, b3, 0, stream, pout, pmap);
    else
      hipLaunchKernelGGL((chunk_prefill_seg1_kernel<64, 64, false>), g3, b3, 0, stream, pout, pmap);
  } else {
    if (bf16)
      hipLaunchKernelGGL((chunk_prefill_seg1_kernel<128, 128, true>), g3, b3, 0, stream, pout, pmap);
    else
      hipLaunchKernelGGL((chunk_prefill_seg1_kernel<128, 128, false>), g3, b3, 0, stream, pout, pmap);
  }
  return hipGetLastError();
}

// Picks the kernel variant for these sizes and launches it.
hipError_t launch_variant(Params prm, bool bf16, hipStream_t stream) {
  set_access_flags(prm);
  if (prm.K <= 64) {
    prm.nvb = (int)((prm.V + 63) / 64);
    return launch_cfg<64, 64>(prm, bf16, stream);
  }
  // 128-column value blocks for K > 64, also for few (sequence, head) chains
  // and for V <= 64: 64-column blocks double the workgroups, but each repeats
  // the key-side phases with half the waves, which costs more than the CUs it
  // fills (1.2-2.2x slower from 8 to 480 chains of 2048-8192 tokens); with
  // V <= 64 the 8 waves of a 128-column block, half of its columns idle, are
  // still 27-29 % faster than 4 waves on 64 columns (one wave per SIMD).
  prm.nvb = (int)((prm.V + 127) / 128);
  return launch_cfg<128, 128>(prm, bf16, stream);
}

// Smallest length of the segments after the first when a batch is cut into
// segments, 0 when it is not: with a first segment of l0 = 0.8 lc tokens,
// H (T - N l0) / lc = 256 pass-2 items gives lc = H T / (256 + 0.8 N H)
// (the planning kernel may take longer segments, never shorter).
int64_t segment_length(int64_t T, int64_t N, int64_t H, int64_t K, int64_t V) {
  if (N * H >= 256 || T < 16384 || K > 128 || V > 128 || N > 1024) return 0;
  const int64_t den = 256000 + 800 * N * H;
  int64_t lc = (H * T * 1000 + den - 1) / den;
  lc = (lc + 63) / 64 * 64;
  return lc < 2048 ? 2048 : lc;
}

struct SegLayout {
  int64_t seg_len = 0, nmax = 0;
  size_t off_scu = 0, off_sfirst = 0, off_sseq = 0, off_b = 0, off_m = 0, off_sin = 0, total = 0;
};

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

SegLayout seg_layout(int64_t T, int64_t N, int64_t H, int64_t K, int64_t V) {
  SegLayout L;
  L.seg_len = segment_length(T, N, H, K, V);
  if (!L.seg_len) return L;
  // a sequence of len > l0 tokens has 1 + ceil((len - l0) / lc) segments, at
  // most 2 + (len - l0) / lc < 1.25 + len / lc (l0 >= 0.8 lc - 32, lc >=
  // seg_len >= 2048; one segment when len <= l0): fewer than
  // 1.25 N + T / seg_len + 1 in all
  L.nmax = N + (4 * T + N * L.seg_len) / (4 * L.seg_len) + 1;
  size_t o = 0;
  L.off_scu = o;     o += round256(sizeof(int32_t) * (size_t)(L.nmax + 1));
  L.off_sfirst = o;  o += round256(sizeof(int32_t) * (size_t)(N + 1));
  L.off_sseq = o;    o += round256(sizeof(int32_t) * (size_t)L.nmax);
  L.off_b = o;       o += round256(sizeof(float) * (size_t)(L.nmax * H * V * K));
  L.off_m = o;       o += round256(sizeof(float) * (size_t)(L.nmax * H * K * K));
  L.off_sin = o;     o += round256(sizeof(float) * (size_t)(L.nmax * H * V * K));
  L.total = o;
  return L;
}
}  // namespace

size_t chunk_prefill_workspace_bytes(int64_t T, int64_t N, int64_t H, int64_t K, int64_t V) {
  const SegLayout L = seg_layout(T, N, H, K, V);
  if (L.seg_len) return L.total;
  if (N < 2 || N > kPlanMaxN) return 0;
  return round256((size_t)N * 4 + 4);  // the order, the kernel choice
}

hipError_t launch_chunk_prefill(const kda_prefill_args_t& a, hipStream_t stream) {
  Params prm;
  prm.q = a.q;
  prm.k = a.k;
  prm.v = a.v;
  prm.g = a.g;
  prm.beta = a.beta;
  prm.cu = a.cu_seqlens;
  prm.init = a.initial_state;
  prm.out = a.out;
  prm.fin = a.final_state;
  prm.T = a.T;
  prm.N = a.N;
  prm.H = a.H;
  prm.K = a.K;
  prm.V = a.V;
  prm.scale = a.scale;
  prm.beta_bf16 = a.beta_dtype == KDA_BF16;
  prm.init_bf16 = a.initial_dtype == KDA_BF16;
  prm.fin_bf16 = a.final_dtype == KDA_BF16;
  prm.l2norm = a.use_qk_l2norm != 0;
  prm.order = nullptr;
  prm.mmap = nullptr;
  prm.nvb = 1;
  prm.ckpt = a.ckpt_states;
  prm.ckpt_cu = a.ckpt_cu;
  prm.ckpt_iv = a.ckpt_interval;
  prm.num_ckpt = a.num_ckpt;
  prm.ckpt_bf16 = a.ckpt_dtype == KDA_BF16;
  prm.seq_of = nullptr;
  prm.seq_cu = nullptr;
  prm.seg_first = nullptr;
  prm.seg_role = 0;
  prm.seg_total = nullptr;
  prm.sin_next = nullptr;
  prm.sel = nullptr;
  prm.sel_want = 0;
  const bool bf16 = a.qkv_dtype == KDA_BF16;
  hipError_t e;

  const SegLayout L = seg_layout(a.T, a.N, a.H, a.K, a.V);
  if (L.seg_len) {
    char* ws = static_cast<char*>(a.workspace);
    int32_t* scu = reinterpret_cast<int32_t*>(ws + L.off_scu);
    int32_t* sfirst = reinterpret_cast<int32_t*>(ws + L.off_sfirst);
    int32_t* sseq = reinterpret_cast<int32_t*>(ws + L.off_sseq);
    float* bmap = reinterpret_cast<float*>(ws + L.off_b);
    float* mmap = reinterpret_cast<float*>(ws + L.off_m);
    float* sin = reinterpret_cast<float*>(ws + L.off_sin);
    hipLaunchKernelGGL(seg_plan_kernel, dim3(1), dim3(1024), 0, stream, a.cu_seqlens, a.N, a.T, a.H, L.seg_len,
                       L.nmax, scu, sfirst, sseq);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    Params seg = prm;
    seg.cu = scu;
    seg.N = L.nmax;
    seg.seq_of = sseq;
    seg.seq_cu = a.cu_seqlens;
    seg.seg_first = sfirst;
    seg.seg_total = sfirst + a.N;
    // pass 1: the first segments' outputs (from the sequences' initial
    // states) beside the middle segments' maps (M, b)
    Params pf = seg;
    pf.seg_role = kSegFirst;
    pf.sin_next = sin;
    Params pm = seg;
    pm.seg_role = kSegMaps;
    pm.init = nullptr;
    pm.out = nullptr;
    pm.ckpt = nullptr;
    pm.fin = bmap;
    pm.fin_bf16 = 0;
    pm.mmap = mmap;
    if ((e = launch_seg1(pf, pm, bf16, stream)) != hipSuccess) return e;
    // scan: S_in of every segment after the second
    const int64_t ncb = (a.V + kScanCols - 1) / kScanCols;
    hipLaunchKernelGGL(seg_scan_kernel, dim3((unsigned)(a.N * a.H * ncb)), dim3(256), 0, stream, sfirst, bmap, mmap,
                       sin, a.H, a.K, a.V);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // pass 2: outputs of the other segments from their initial states
    Params pr = seg;
    pr.seg_role = kSegRest;
    pr.init = sin;
    pr.init_bf16 = 0;
    return launch_variant(pr, bf16, stream);
  }

  if (a.N >= 2 && a.N <= kPlanMaxN) {
    int32_t* order = static_cast<int32_t*>(a.workspace);
    // more chains than CUs: the plan also picks the chunk kernel
    Params pa = prm;
    set_access_flags(pa);
    const int cus = device_cus();
    int32_t* sel = two_per_cu_shape(pa, bf16) && a.N * a.H > cus ? order + a.N : nullptr;
    hipLaunchKernelGGL(plan_order_kernel, dim3(1), dim3(1024), 0, stream, a.cu_seqlens, a.N, a.T, a.H,
                       (int32_t)cus, order, sel);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    prm.order = order;
    prm.sel = sel;
  }
  return launch_variant(prm, bf16, stream);
}

}  // namespace kda

// Scratch of the allocation-free entry point (kda_chunk_prefill_noalloc): the
// workspace of the sequence-order plan and of the segment maps, one copy per
// device, held until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: its device address on the current
// device comes from hipGetSymbolAddress, and only that address is handed to
// kernels.  Nothing in it needs to start at zero (every kernel that reads a
// part of it reads only what an earlier kernel of the same call wrote).
static __device__ __align__(256) char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace kda {

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace kda
