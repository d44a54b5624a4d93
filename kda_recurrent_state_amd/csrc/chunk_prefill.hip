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
// MI355X mapping (one workgroup of 4 wave64s per (sequence, head, V-block)):
//  * The workgroup walks its sequence chunk by chunk; the fp32 state block
//    (K x BV) never leaves registers.  It is held in MFMA accumulator layout,
//    wave w owning BV/4 value columns, and converted to bf16 B-operands for the
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
//    product's C-layout result feeds the next product directly, with the A
//    operand read from LDS in the matching (permuted) k order.
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
#include "internal.h"

namespace kda {
namespace {

constexpr int kC = 64;          // chunk length
constexpr int kThreads = 256;   // 4 wave64s
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRangeLimit = 100.f;
constexpr float kL2Eps = 1e-6f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int KP, int BV>
struct Cfg {
  static constexpr int CPL = KP / 64;   // key channels per lane in the elementwise phase
  static constexpr int VPL = BV / 64;   // value columns per lane in the elementwise phase
  static constexpr int NVW = BV / 4;    // value columns owned by each wave in the state phase
  static constexpr int NVT = NVW / 16;  // 16-wide value tiles per wave
  static constexpr int KT = KP / 16;    // 16-row key tiles
  static constexpr int KS = KP / 32;    // 32-deep contraction steps over the key dim
  static constexpr int LDK = KP + 8;    // row stride (bf16) of [64][KP] tiles
  static constexpr int LDT = kC + 8;    // row stride (bf16) of [X][64] tiles
  static constexpr int LDA = kC + 4;    // row stride (fp32) of the [64][64] solve tile
  // LDS map (bytes).  R_KL/R_QL/R_KR are dead after the A products and are
  // reused for T, -W and the output staging.
  static constexpr int SZ_ROW = kC * LDK * 2;
  static constexpr int SZ_KT = KP * LDT * 2;
  static constexpr int SZ_VT = BV * LDT * 2;
  static constexpr int SZ_T = kC * LDT * 2;
  static constexpr int R_KL = 0;                        // KL  [64][KP]  -> T [64][64]
  static constexpr int R_QL = R_KL + SZ_ROW;            // QL  [64][KP]  -> -W [64][KP]
  static constexpr int R_KR = R_QL + SZ_ROW;            // KR  [64][KP]
  static constexpr int R_QG = R_KR + SZ_ROW;            // Qg  [64][KP]
  static constexpr int R_KE = R_QG + SZ_ROW;            // KE^T [KP][64]
  static constexpr int R_KB = R_KE + SZ_KT;             // Kbar^T [KP][64]
  static constexpr int R_VT = R_KB + SZ_KT;             // (beta V)^T [BV][64]
  static constexpr int R_A = R_VT + SZ_VT;              // A_kk / T fp32 [64][LDA]
  static constexpr int R_AQK = R_A + kC * LDA * 4;      // A_qk bf16 [64][LDT]
  static constexpr int R_TOT = R_AQK + SZ_T;            // gate block totals fp32 [4][KP]
  static constexpr int R_DEC = R_TOT + 4 * KP * 4;      // 2^gamma_L fp32 [KP]
  static constexpr int R_RED = R_DEC + KP * 4;          // range guard, fp32 [4]
  static constexpr int R_X = R_RED + 64;                // solve temps fp32 [3 waves][2][16][16]
  static constexpr int LDS = R_X + 3 * 2 * 256 * 4;
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(SZ_T <= SZ_ROW, "T fits in the KL region");
};

__device__ __forceinline__ float bf2f(unsigned short u) { return __uint_as_float((unsigned)u << 16); }

template <bool kBF16>
__device__ __forceinline__ float ld_in(const void* p, int64_t i) {
  if (kBF16) return bf2f(static_cast<const unsigned short*>(p)[i]);
  return static_cast<const float*>(p)[i];
}

__device__ __forceinline__ float ld_any(const void* p, int64_t i, bool bf16) {
  return bf16 ? bf2f(static_cast<const unsigned short*>(p)[i]) : static_cast<const float*>(p)[i];
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 bf16 from two 4-element runs: k-slots 0..3 <- p[0..3], 4..7 <- p[16..19].
__device__ __forceinline__ bf16x8 ld_perm(const __bf16* p) {
  bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
  bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 16);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ bf16x8 pack_perm(const f32x4& lo, const f32x4& hi) {
  return bf16x8{(__bf16)lo[0], (__bf16)lo[1], (__bf16)lo[2], (__bf16)lo[3],
                (__bf16)hi[0], (__bf16)hi[1], (__bf16)hi[2], (__bf16)hi[3]};
}

// Ranks sequences by length, longest first (ties by index).  One workgroup.
__global__ __launch_bounds__(1024) void plan_order_kernel(const int32_t* __restrict__ cu, int64_t N, int64_t T,
                                                          int32_t* __restrict__ order) {
  __shared__ int32_t len_s[2048];
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
};

template <int KP, int BV, bool kBF16>
__global__ __launch_bounds__(kThreads, 1) void chunk_prefill_kernel(Params p) {
  using C = Cfg<KP, BV>;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  __bf16* sKL = reinterpret_cast<__bf16*>(smem + C::R_KL);
  __bf16* sT = reinterpret_cast<__bf16*>(smem + C::R_KL);
  __bf16* sQL = reinterpret_cast<__bf16*>(smem + C::R_QL);
  __bf16* sW = reinterpret_cast<__bf16*>(smem + C::R_QL);
  __bf16* sKR = reinterpret_cast<__bf16*>(smem + C::R_KR);
  __bf16* sQg = reinterpret_cast<__bf16*>(smem + C::R_QG);
  __bf16* sKE = reinterpret_cast<__bf16*>(smem + C::R_KE);
  __bf16* sKB = reinterpret_cast<__bf16*>(smem + C::R_KB);
  __bf16* sVT = reinterpret_cast<__bf16*>(smem + C::R_VT);
  float* sA = reinterpret_cast<float*>(smem + C::R_A);
  __bf16* sAqk = reinterpret_cast<__bf16*>(smem + C::R_AQK);
  float* sTot = reinterpret_cast<float*>(smem + C::R_TOT);
  float* sDec = reinterpret_cast<float*>(smem + C::R_DEC);
  float* sRed = reinterpret_cast<float*>(smem + C::R_RED);
  float* sX = reinterpret_cast<float*>(smem + C::R_X);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int lr = l & 15;  // MFMA row/col within a 16-tile
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
  const int64_t v0 = (int64_t)vb * BV;  // first value column of this block

  // A_qk upper blocks are read by the output product but never written: zero once.
  for (int e = tid; e < kC * kC; e += kThreads) {
    const int r = e >> 6, c = e & 63;
    if ((c >> 4) > (r >> 4)) sAqk[r * C::LDT + c] = (__bf16)0.f;
  }

  // ---- initial state into MFMA C-layout registers ----
  // S[ct][vt][e] = S(c = 16ct + 4lg + e, v = v0 + w*NVW + 16vt + lr)
  f32x4 S[C::KT][C::NVT];
#pragma unroll
  for (int ct = 0; ct < C::KT; ++ct)
#pragma unroll
    for (int vt = 0; vt < C::NVT; ++vt) {
      const int64_t vcol = v0 + w * C::NVW + 16 * vt + lr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t c = 16 * ct + 4 * lg + e;
        float x = 0.f;
        if (p.init && vcol < V && c < K) x = ld_any(p.init, ((n * H + h) * V + vcol) * K + c, p.init_bf16);
        S[ct][vt][e] = x;
      }
    }

  const float scale = p.scale;
  int64_t t0 = 0;
  int Lcap = kC;
  while (t0 < len) {
    int L = (int)((len - t0) < (int64_t)Lcap ? (len - t0) : (int64_t)Lcap);
    __syncthreads();  // previous chunk's readers of LDS are done

    // ---------------- phase 0: loads, l2norm, gate cumsum -----------------
    float kx[16][C::CPL], qx[16][C::CPL], gx[16][C::CPL], vx[16][C::VPL], bt[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 16 * w + r;
      const bool ok = i < L;
      const int64_t t = bos + t0 + i;
      const int64_t bk = (t * H + h) * K;
#pragma unroll
      for (int cc = 0; cc < C::CPL; ++cc) {
        const int64_t c = l * C::CPL + cc;
        const bool okc = ok && c < K;
        kx[r][cc] = okc ? ld_in<kBF16>(p.k, bk + c) : 0.f;
        qx[r][cc] = okc ? ld_in<kBF16>(p.q, bk + c) : 0.f;
        gx[r][cc] = okc ? p.g[bk + c] : 0.f;
      }
      const int64_t bv = (t * H + h) * V + v0;
#pragma unroll
      for (int vv = 0; vv < C::VPL; ++vv) {
        const int64_t vc = l * C::VPL + vv;
        vx[r][vv] = (ok && v0 + vc < V) ? ld_in<kBF16>(p.v, bv + vc) : 0.f;
      }
      bt[r] = ok ? ld_any(p.beta, t * H + h, p.beta_bf16) : 0.f;
    }
    // inclusive cumsum of g over this wave's 16 rows
#pragma unroll
    for (int cc = 0; cc < C::CPL; ++cc) {
      float run = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        run += gx[r][cc];
        gx[r][cc] = run;
      }
      sTot[w * KP + l * C::CPL + cc] = run;
    }
    // row norms
    float rk[16], rq[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float sk = 0.f, sq = 0.f;
#pragma unroll
      for (int cc = 0; cc < C::CPL; ++cc) {
        sk += kx[r][cc] * kx[r][cc];
        sq += qx[r][cc] * qx[r][cc];
      }
      sk = wave_sum(sk);
      sq = wave_sum(sq);
      rk[r] = p.l2norm ? __frsqrt_rn(sk + kL2Eps) : 1.f;
      rq[r] = p.l2norm ? __frsqrt_rn(sq + kL2Eps) : 1.f;
    }
    __syncthreads();

    // gamma (log2 units), reference row and range guard
    const int mb = L > 32 ? 2 : 1;  // reference = last row of block mb-1
    float gm[C::CPL], gL[C::CPL];
    float guard = 0.f;
#pragma unroll
    for (int cc = 0; cc < C::CPL; ++cc) {
      const int c = l * C::CPL + cc;
      float off = 0.f, ref = 0.f, tot = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float x = sTot[ww * KP + c];
        off += ww < w ? x : 0.f;
        ref += ww < mb ? x : 0.f;
        tot += x;
      }
      gm[cc] = ref * kLog2e;
      gL[cc] = tot * kLog2e;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        gx[r][cc] = (gx[r][cc] + off) * kLog2e;
        guard = fmaxf(guard, fabsf(gx[r][cc] - gm[cc]));
      }
      guard = fmaxf(guard, fmaxf(gm[cc], gL[cc] - gm[cc]));
    }
    guard = wave_max(guard);
    if (l == 0) sRed[w] = guard;
    __syncthreads();
    const float gmax = fmaxf(fmaxf(sRed[0], sRed[1]), fmaxf(sRed[2], sRed[3]));
    if (gmax > kRangeLimit && L > 1) {
      Lcap = L > 16 ? 16 : (L > 4 ? 4 : 1);
      continue;  // re-process this span as shorter chunks
    }

    // ---------------- phase A: gated operand tiles into LDS ----------------
#pragma unroll
    for (int cc = 0; cc < C::CPL; ++cc) {
      const int c = l * C::CPL + cc;
      const float cg = __builtin_amdgcn_exp2f(gm[cc]);           // 2^gamma_m
      const float cb = __builtin_amdgcn_exp2f(gL[cc] - gm[cc]);  // 2^(gamma_L - gamma_m)
      if (w == 0) sDec[c] = __builtin_amdgcn_exp2f(gL[cc]);
      __bf16 ke[16], kb[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 16 * w + r;
        const float e1 = __builtin_amdgcn_exp2f(gx[r][cc] - gm[cc]);  // 2^(gamma_i - gamma_m)
        const float e2 = __builtin_amdgcn_exp2f(gm[cc] - gx[r][cc]);  // 2^(gamma_m - gamma_i)
        const float kh = kx[r][cc] * rk[r];
        const float qh = qx[r][cc] * rq[r];
        sKL[i * C::LDK + c] = (__bf16)(bt[r] * kh * e1);
        sQL[i * C::LDK + c] = (__bf16)(scale * qh * e1);
        sKR[i * C::LDK + c] = (__bf16)(kh * e2);
        sQg[i * C::LDK + c] = (__bf16)(scale * qh * (e1 * cg));
        ke[r] = (__bf16)(bt[r] * kh * (e1 * cg));
        kb[r] = (__bf16)(kh * (e2 * cb));
      }
      // transposed tiles: 16 consecutive rows of one channel = two 16-byte stores
      bf16x8* pe = reinterpret_cast<bf16x8*>(sKE + c * C::LDT + 16 * w);
      bf16x8* pb = reinterpret_cast<bf16x8*>(sKB + c * C::LDT + 16 * w);
      pe[0] = bf16x8{ke[0], ke[1], ke[2], ke[3], ke[4], ke[5], ke[6], ke[7]};
      pe[1] = bf16x8{ke[8], ke[9], ke[10], ke[11], ke[12], ke[13], ke[14], ke[15]};
      pb[0] = bf16x8{kb[0], kb[1], kb[2], kb[3], kb[4], kb[5], kb[6], kb[7]};
      pb[1] = bf16x8{kb[8], kb[9], kb[10], kb[11], kb[12], kb[13], kb[14], kb[15]};
    }
#pragma unroll
    for (int vv = 0; vv < C::VPL; ++vv) {
      const int vc = l * C::VPL + vv;
      __bf16 bvv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) bvv[r] = (__bf16)(bt[r] * vx[r][vv]);
      bf16x8* pv = reinterpret_cast<bf16x8*>(sVT + vc * C::LDT + 16 * w);
      pv[0] = bf16x8{bvv[0], bvv[1], bvv[2], bvv[3], bvv[4], bvv[5], bvv[6], bvv[7]};
      pv[1] = bf16x8{bvv[8], bvv[9], bvv[10], bvv[11], bvv[12], bvv[13], bvv[14], bvv[15]};
    }
    __syncthreads();

    // ---------------- phase B: A_kk (fp32) and A_qk (bf16) -----------------
    // 10 lower block pairs x {kk, qk} = 20 tile jobs, round-robin over waves.
    for (int job = w; job < 20; job += 4) {
      const int pair = job >> 1;
      const bool is_qk = job & 1;
      // pair -> (bi, bj), bj <= bi
      const int bi = pair >= 6 ? 3 : (pair >= 3 ? 2 : (pair >= 1 ? 1 : 0));
      const int bj = pair - (bi * (bi + 1)) / 2;
      const __bf16* left = is_qk ? sQL : sKL;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(left + (16 * bi + lr) * C::LDK + 32 * ks + 8 * lg);
        const bf16x8 bb = *reinterpret_cast<const bf16x8*>(sKR + (16 * bj + lr) * C::LDK + 32 * ks + 8 * lg);
        acc = mfma(a, bb, acc);
      }
      const int col = 16 * bj + lr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * bi + 4 * lg + e;
        if (is_qk)
          sAqk[row * C::LDT + col] = (__bf16)(row >= col ? acc[e] : 0.f);
        else
          sA[row * C::LDA + col] = row > col ? acc[e] : 0.f;
      }
    }
    __syncthreads();

    // ---------------- phase C: T = (I + A_kk)^-1, in place in sA ----------
    if (w == 0) {
      // diagonal 16x16 blocks by forward substitution; lane = (block, column)
      const int bb = l >> 4, col = l & 15;
      const float* Ab = sA + (16 * bb) * C::LDA + 16 * bb;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float s = (i == col) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < i; ++j) s -= Ab[i * C::LDA + j] * x[j];
        x[i] = s;
      }
      float* Tb = sA + (16 * bb) * C::LDA + 16 * bb;
#pragma unroll
      for (int i = 0; i < 16; ++i) Tb[i * C::LDA + col] = x[i];
    }
    __syncthreads();
    // off-diagonal blocks, one block row at a time:
    //   T[bi][bj] = -D_bi * sum_{k=bj}^{bi-1} A[bi][k] T[k][bj]
    for (int bi = 1; bi < 4; ++bi) {
      if (w < bi) {
        const int bj = w;
        const int r = l >> 2, c0 = 4 * (l & 3);
        float* X = sX + w * 512;
        float* Y = X + 256;
        f32x4 xs = {0.f, 0.f, 0.f, 0.f};
        for (int kb = bj; kb < bi; ++kb) {
#pragma unroll
          for (int kk = 0; kk < 16; ++kk) {
            const float a = sA[(16 * bi + r) * C::LDA + 16 * kb + kk];
            const f32x4 t4 = *reinterpret_cast<const f32x4*>(sA + (16 * kb + kk) * C::LDA + 16 * bj + c0);
            xs += a * t4;
          }
        }
        *reinterpret_cast<f32x4*>(X + r * 16 + c0) = xs;
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): X visible to the wave
        __builtin_amdgcn_wave_barrier();
        f32x4 ys = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
          const float d = sA[(16 * bi + r) * C::LDA + 16 * bi + kk];
          const f32x4 x4 = *reinterpret_cast<const f32x4*>(X + kk * 16 + c0);
          ys -= d * x4;
        }
        *reinterpret_cast<f32x4*>(Y + r * 16 + c0) = ys;
      }
      __syncthreads();
      if (w < bi) {
        const int bj = w;
        const int r = l >> 2, c0 = 4 * (l & 3);
        const float* Y = sX + w * 512 + 256;
        *reinterpret_cast<f32x4*>(sA + (16 * bi + r) * C::LDA + 16 * bj + c0) =
            *reinterpret_cast<const f32x4*>(Y + r * 16 + c0);
      }
      __syncthreads();
    }
    // T to bf16 [64][LDT] with zeros above the diagonal (overwrites KL)
    for (int e = tid; e < kC * kC; e += kThreads) {
      const int r = e >> 6, c = e & 63;
      sT[r * C::LDT + c] = (__bf16)(c <= r ? sA[r * C::LDA + c] : 0.f);
    }
    __syncthreads();

    // ---------------- phase D: U (registers) and -W (LDS) ------------------
    f32x4 U[4][C::NVT];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int vt = 0; vt < C::NVT; ++vt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if (32 * ks > 16 * rt + 15) continue;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sT + (16 * rt + lr) * C::LDT + 32 * ks + 8 * lg);
          const bf16x8 bb =
              *reinterpret_cast<const bf16x8*>(sVT + (w * C::NVW + 16 * vt + lr) * C::LDT + 32 * ks + 8 * lg);
          acc = mfma(a, bb, acc);
        }
        U[rt][vt] = acc;
      }
    // W^T[c][i] = sum_j KE^T[c][j] T[i][j]; stored as -W[i][c]
    for (int ct = w; ct < C::KT; ct += 4) {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if (32 * ks > 16 * it + 15) continue;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sKE + (16 * ct + lr) * C::LDT + 32 * ks + 8 * lg);
          const bf16x8 bb = *reinterpret_cast<const bf16x8*>(sT + (16 * it + lr) * C::LDT + 32 * ks + 8 * lg);
          acc = mfma(a, bb, acc);
        }
        *reinterpret_cast<bf16x4*>(sW + (16 * it + lr) * C::LDK + 16 * ct + 4 * lg) =
            bf16x4{(__bf16)(-acc[0]), (__bf16)(-acc[1]), (__bf16)(-acc[2]), (__bf16)(-acc[3])};
      }
    }
    __syncthreads();

    // ---------------- phase E: the serial chain, per wave ------------------
    bf16x8 bS[C::KS][C::NVT];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int vt = 0; vt < C::NVT; ++vt) bS[ks][vt] = pack_perm(S[2 * ks][vt], S[2 * ks + 1][vt]);
    // V_new = U - W S
    f32x4 Vn[4][C::NVT];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int vt = 0; vt < C::NVT; ++vt) Vn[rt][vt] = U[rt][vt];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 a = ld_perm(sW + (16 * rt + lr) * C::LDK + 32 * ks + 4 * lg);
#pragma unroll
        for (int vt = 0; vt < C::NVT; ++vt) Vn[rt][vt] = mfma(a, bS[ks][vt], Vn[rt][vt]);
      }
    bf16x8 bV[2][C::NVT];
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
      for (int vt = 0; vt < C::NVT; ++vt) bV[q2][vt] = pack_perm(Vn[2 * q2][vt], Vn[2 * q2 + 1][vt]);
    // O = Qg S_in + A_qk V_new
    f32x4 O[4][C::NVT];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
      for (int vt = 0; vt < C::NVT; ++vt) O[rt][vt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 a = ld_perm(sQg + (16 * rt + lr) * C::LDK + 32 * ks + 4 * lg);
#pragma unroll
        for (int vt = 0; vt < C::NVT; ++vt) O[rt][vt] = mfma(a, bS[ks][vt], O[rt][vt]);
      }
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        if (32 * q2 > 16 * rt + 15) continue;
        const bf16x8 a = ld_perm(sAqk + (16 * rt + lr) * C::LDT + 32 * q2 + 4 * lg);
#pragma unroll
        for (int vt = 0; vt < C::NVT; ++vt) O[rt][vt] = mfma(a, bV[q2][vt], O[rt][vt]);
      }
    }
    // S = diag(2^gamma_L) S + Kbar^T V_new
#pragma unroll
    for (int ct = 0; ct < C::KT; ++ct) {
      const f32x4 dec = *reinterpret_cast<const f32x4*>(sDec + 16 * ct + 4 * lg);
#pragma unroll
      for (int vt = 0; vt < C::NVT; ++vt) S[ct][vt] *= dec;
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const bf16x8 a = ld_perm(sKB + (16 * ct + lr) * C::LDT + 32 * q2 + 4 * lg);
#pragma unroll
        for (int vt = 0; vt < C::NVT; ++vt) S[ct][vt] = mfma(a, bV[q2][vt], S[ct][vt]);
      }
    }
    // output rows of this chunk
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int vt = 0; vt < C::NVT; ++vt) {
        const int64_t vcol = v0 + w * C::NVW + 16 * vt + lr;
        if (vcol >= V) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * rt + 4 * lg + e;
          if (i >= L) continue;
          const int64_t o = ((bos + t0 + i) * H + h) * V + vcol;
          if (kBF16)
            static_cast<__bf16*>(p.out)[o] = (__bf16)O[rt][vt][e];
          else
            static_cast<float*>(p.out)[o] = O[rt][vt][e];
        }
      }
    t0 += L;
    Lcap = kC;
  }

  // ---- final state ----
  if (p.fin) {
#pragma unroll
    for (int ct = 0; ct < C::KT; ++ct)
#pragma unroll
      for (int vt = 0; vt < C::NVT; ++vt) {
        const int64_t vcol = v0 + w * C::NVW + 16 * vt + lr;
        if (vcol >= V) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t c = 16 * ct + 4 * lg + e;
          if (c >= K) continue;
          const int64_t o = ((n * H + h) * V + vcol) * K + c;
          if (p.fin_bf16)
            static_cast<__bf16*>(p.fin)[o] = (__bf16)S[ct][vt][e];
          else
            static_cast<float*>(p.fin)[o] = S[ct][vt][e];
        }
      }
  }
}

constexpr int64_t kPlanMaxN = 2048;

template <int KP, int BV>
hipError_t launch_cfg(const Params& prm, bool bf16, hipStream_t stream) {
  const int64_t items = prm.N * prm.H;
  const int64_t groups = (items + 7) / 8;
  const int64_t grid = groups * 8 * prm.nvb;
  if (bf16)
    hipLaunchKernelGGL((chunk_prefill_kernel<KP, BV, true>), dim3((unsigned)grid), dim3(kThreads), 0, stream, prm);
  else
    hipLaunchKernelGGL((chunk_prefill_kernel<KP, BV, false>), dim3((unsigned)grid), dim3(kThreads), 0, stream, prm);
  return hipGetLastError();
}

}  // namespace

size_t chunk_prefill_workspace_bytes(int64_t T, int64_t N, int64_t H, int64_t K, int64_t V) {
  (void)T; (void)H; (void)K; (void)V;
  if (N < 2 || N > kPlanMaxN) return 0;
  return (size_t)(((N * 4) + 255) / 256 * 256);
}

hipError_t launch_chunk_prefill(const kda_prefill_args_t& a, hipStream_t stream) {
  Params prm;
  prm.q = a.q; prm.k = a.k; prm.v = a.v; prm.g = a.g; prm.beta = a.beta; prm.cu = a.cu_seqlens;
  prm.init = a.initial_state; prm.out = a.out; prm.fin = a.final_state;
  prm.T = a.T; prm.N = a.N; prm.H = a.H; prm.K = a.K; prm.V = a.V;
  prm.scale = a.scale;
  prm.beta_bf16 = a.beta_dtype == KDA_BF16;
  prm.init_bf16 = a.initial_dtype == KDA_BF16;
  prm.fin_bf16 = a.final_dtype == KDA_BF16;
  prm.l2norm = a.use_qk_l2norm != 0;
  prm.order = nullptr;
  if (a.N >= 2 && a.N <= kPlanMaxN) {
    int32_t* order = static_cast<int32_t*>(a.workspace);
    hipLaunchKernelGGL(plan_order_kernel, dim3(1), dim3(1024), 0, stream, a.cu_seqlens, a.N, a.T, order);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    prm.order = order;
  }
  const bool bf16 = a.qkv_dtype == KDA_BF16;
  // Fewer than ~2 workgroups per CU from (sequence, head) chains alone: split V.
  const int64_t chains = a.N * a.H;
  if (a.K <= 64) {
    prm.nvb = (int)((a.V + 63) / 64);
    return launch_cfg<64, 64>(prm, bf16, stream);
  }
  if (a.V <= 64 || chains < 512) {
    prm.nvb = (int)((a.V + 63) / 64);
    return launch_cfg<128, 64>(prm, bf16, stream);
  }
  prm.nvb = (int)((a.V + 127) / 128);
  return launch_cfg<128, 128>(prm, bf16, stream);
}

}  // namespace kda
