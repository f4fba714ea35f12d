// Chunked causal prefill of SATA for bfloat16 inputs on gfx950 (CDNA4).
//
// Same split of the output as the float32 path [SATA page, section
// "Engineering of constant compute cost": a fixed-size state of
// phi(k) v^T sums, read out per token through the weighted feature map]:
//   num_i = (intra-window part, exact polynomial)      prefill_intra_mfma
//         + (order 0 before the window, exact sums)    prefill_carry
//         + sum_{m of order >= 1} w_m phi_m(q_i) S_m   prefill_scan_b16
// over readout windows of 512 tokens, and likewise for den with v -> 1.
//
// Kernels of one call window (launch order):
//   prefill_amax     max |q|, |k|, |v| per head (32 token slices).
//   prefill_stage    per (64-token chunk, head): q, k, v converted once into
//                    the scan's 16-bit tables (f16 after exact power-of-two
//                    scaling, or bf16 as is) in four layouts: keys and values
//                    index-major, queries index-major and token-major; plus
//                    exact fp32 sums of v per chunk.
//   prefill_carry    order-0 prefix at each readout-window start, and the
//                    order-0 row of the state (a parallel scan over the
//                    readout windows, one block per column and head).
//   prefill_scan_b16 grid = (row tiles) x (heads), 8 waves.  Per chunk the
//                    staged tables arrive in LDS by DMA (global_load_lds,
//                    double-buffered, one chunk ahead; the loop runs chunk
//                    pairs so each buffer's offsets are constants); the state
//                    slice of the tile stays in registers.  Two
//                    barrier-separated segments per chunk, each with MFMA work:
//                      1  readout  phi_q(Q) Sb  into the cross-wave buffer
//                      2  cross-wave sum into the tile's records, key
//                         features of the next chunk's parent slots (order 2,
//                         and order 3 when P = 5), and the update
//                         S += phi_k(K)^T [V 1].
//   prefill_reduce_b16  out = (intra + records + carry) / den per token.
// The state-only scan (the first pass over sequence segments) keeps the
// update, the key/value DMA and the parent slots, and drops the readout,
// its 16-bit operand and the records; no intra-window or reduce kernel runs.
// state_copy, state_zero and state_prefix move the segment states.
//
// Feature map.  Rows of a tile come in runs of four children (P, c..c+3) of
// one parent multiset P (the nested i1 <= ... <= ip index structure); a
// child's feature is the parent's times one coordinate.  Features are plain
// monomials prod k_i and prod q_i: the weights w_m = 1 / (prod count! c^p)
// multiply the state when it is rounded to the 16-bit readout operand Sb
// (once per readout window), so the state itself is the canonical S (times
// exact powers of two on the f16 path).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "sata_device.h"
#include "sata_internal.h"

namespace sata {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kL = 64;   // tokens per chunk

// Tile records of the f16 operand path (d >= 32): the cross-wave sum of eight
// partials (below 2^18) times 2^-kRecShift, as f16, with the chunk's scale
// 2^(ew + kRecShift) in a side array.
constexpr int kRecShift = 3;

// Two floats rounded (nearest even) to bf16 / f16 and packed in one register.
// The empty asm pins the conversion here so the fp32 inputs die early.
__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
  bf16x2 v = {static_cast<__bf16>(x), static_cast<__bf16>(y)};
  uint32_t r = __builtin_bit_cast(uint32_t, v);
  asm volatile("" : "+v"(r));
  return r;
}
__device__ __forceinline__ uint32_t pack_f16(float x, float y) {
  f16x2 v = {static_cast<_Float16>(x), static_cast<_Float16>(y)};
  uint32_t r = __builtin_bit_cast(uint32_t, v);
  asm volatile("" : "+v"(r));
  return r;
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

// Barrier for LDS traffic only: waits for this wave's LDS operations, not for
// its global stores.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// 16 bytes a lane from global memory straight into LDS (lane l writes bytes
// [16 l, 16 l + 16) after the wave-uniform LDS address).
__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, lds_dst, 16, 0, 0);
}
// The same after this wave's LDS DMA (global_load_lds) has landed.
__device__ __forceinline__ void dma_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  lds_barrier();
}

// Per-head scale exponents of the f16 operand path, from the window's
// max-abs values: k' = k 2^-ek, q' = q 2^ek, v' = v 2^-ev (exact; q'.k' =
// q.k).  ek splits the magnitude evenly between the two sides: with |q| <
// 2^eq and |k| < 2^ekk, ek = (ekk - eq) / 2 leaves |q'| < 2^(eq + ek) and
// |k'| < 2^(ekk - ek), so a query feature (at most P-1 coordinates) is below
// 2^fq, fq = (P-1) max(eq + ek, 0), and a key feature below 2^fk likewise.
// ev is zero unless |v| is outside [2^-8, 2^15), so |v'| < 2^15.  The path
// is taken when fq, fk <= 12 (and every value is finite), far inside the f16
// range.  The readout operand Sb of a tile is then scaled so that its
// largest entry lies in [2^(sb-1), 2^sb), sb = min(14, 9 - fq): a wave's
// readout partial over at most 64 rows stays below 2^6 2^fq 2^sb <= 2^15 <
// 65504 and goes to the cross-wave sum as f16.  (Entries of Sb more than
// 2^(sb+14) below the largest are subnormal; their absolute error is
// negligible next to the largest entries'.)  Otherwise the head runs with
// bf16 operands.
struct HalfScales {
  bool safe;
  int ek;
  int ev;
  int sb;
};

__device__ __forceinline__ HalfScales half_scales(const float* amax, int P, int ec) {
  float mq = 0.f, mk = 0.f, mv = 0.f;
#pragma unroll 4
  for (int s = 0; s < kAmaxSplit; ++s) {
    mq = fmaxf(mq, amax[4 * s]);
    mk = fmaxf(mk, amax[4 * s + 1]);
    mv = fmaxf(mv, amax[4 * s + 2]);
  }
  HalfScales h;
  int eq = 0, ekk = 0, e = 0;
  if (mq > 0.f) (void)frexpf(mq, &eq);    // mq < 2^eq
  if (mk > 0.f) (void)frexpf(mk, &ekk);   // mk < 2^ekk
  eq -= ec;                               // the staged queries carry 2^-ec (the power of two of c)
  h.ek = (ekk - eq) / 2;
  h.ev = 0;
  if (mv > 0.f) {
    (void)frexpf(mv, &e);
    if (e > 15) h.ev = e - 15;
    else if (e < -7) h.ev = e;
  }
  const int fq = (P - 1) * max(eq + h.ek, 0);
  const int fk = (P - 1) * max(ekk - h.ek, 0);
  h.sb = min(14, 9 - fq);
  h.safe = isfinite(mq) && isfinite(mk) && isfinite(mv) && fq <= 12 && fk <= 12 && h.ek > -40 &&
           h.ek < 40 && h.ev > -40 && h.ev < 40;
  return h;
}

__device__ __forceinline__ const HalfScales head_scales(const PrefillWs& ws, int head, int P, int ec) {
  return half_scales(ws.amax + static_cast<int64_t>(head) * kAmaxSplit * 4, P, ec);
}

// ---------------------------------------------------------------------------
// Max |x| of q, k, v over a slice of the window's tokens, per head.  Grid =
// (kAmaxSplit slices, heads); absolute values compared as bf16 bit patterns
// (monotone for non-NaN values; a NaN pattern exceeds every finite one and
// makes the head take the bf16 path), eight per 16-byte load.
template <int DK>
__global__ __launch_bounds__(256) void prefill_amax(ScanArgs a) {
  const int sp = blockIdx.x;
  const int head = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t per = (a.nw + kAmaxSplit - 1) / kAmaxSplit;
  const int64_t t_begin = static_cast<int64_t>(sp) * per;
  const int64_t t_end = min(static_cast<int64_t>(head_tokens(a.lens, head, a.t0, a.nw, a.n_total)), t_begin + per);
  __shared__ uint32_t wmax[3][4];
  uint32_t m[3] = {0u, 0u, 0u};
  if (t_begin < t_end) {
    const int64_t e0 = (a.t0 + t_begin) * DK, e1 = (a.t0 + t_end) * DK;   // DK % 8 == 0
    const int64_t hoff = static_cast<int64_t>(head) * a.n_total * DK;
    const uint16_t* src[3] = {static_cast<const uint16_t*>(a.q) + hoff, static_cast<const uint16_t*>(a.k) + hoff,
                              static_cast<const uint16_t*>(a.v) + hoff};
    auto fold = [&](uint32_t& acc, const u32x4& v) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w2 = v[j] & 0x7fff7fffu;
        acc = max(acc, max(w2 & 0xffffu, w2 >> 16));
      }
    };
    // q, k and v together, four strides deep: twelve loads in flight
    constexpr int64_t STR = 8 * 256;
    int64_t e = e0 + 8 * tid;
    for (; e + 3 * STR < e1; e += 4 * STR) {
      u32x4 v[3][4];
#pragma unroll
      for (int x = 0; x < 3; ++x)
#pragma unroll
        for (int u = 0; u < 4; ++u) v[x][u] = *reinterpret_cast<const u32x4*>(src[x] + e + u * STR);
#pragma unroll
      for (int x = 0; x < 3; ++x)
#pragma unroll
        for (int u = 0; u < 4; ++u) fold(m[x], v[x][u]);
    }
    for (; e < e1; e += STR) {
      u32x4 v[3];
#pragma unroll
      for (int x = 0; x < 3; ++x) v[x] = *reinterpret_cast<const u32x4*>(src[x] + e);
#pragma unroll
      for (int x = 0; x < 3; ++x) fold(m[x], v[x]);
    }
  }
#pragma unroll
  for (int x = 0; x < 3; ++x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m[x] = max(m[x], static_cast<uint32_t>(__shfl_xor(static_cast<int>(m[x]), o)));
    if ((tid & 63) == 0) wmax[x][tid >> 6] = m[x];
  }
  __syncthreads();
  if (tid < 3) {
    const uint32_t r = max(max(wmax[tid][0], wmax[tid][1]), max(wmax[tid][2], wmax[tid][3]));
    a.ws.amax[(static_cast<int64_t>(head) * kAmaxSplit + sp) * 4 + tid] = __uint_as_float(r << 16);
  }
}

// ---------------------------------------------------------------------------
// Staging pre-pass.  Block = (64-token chunk, head).  Writes the chunk's four
// 16-bit tables (each DK x 128 bytes, tokens past the window zero):
//   KT[i][t] = k'_t[i]   VT[c][t] = v'_t[c]   QT[i][t] = q'_t[i]   QN[t][i] = q'_t[i]
// and vsum[c] = sum_t v_t[c] (fp32, from the bf16 values), vsum[DV] = tokens.
template <int DK>
__global__ __launch_bounds__(256) void prefill_stage(ScanArgs a) {
  constexpr int DV = DK, L = kL, NU = DK / 8, DVP = padded_dv(DV);
  constexpr int TS = L + 8;   // LDS row stride of the transposes (16-bit elements)
  __shared__ __attribute__((aligned(16))) uint16_t tr[3][DK * TS];
  __shared__ float vraw[L][DV + 1];
  const int ch = blockIdx.x;
  const int head = blockIdx.y;
  const int tid = threadIdx.x;
  const HalfScales hs = head_scales(a.ws, head, a.P, a.ec);
  const int nvalid = max(0, min(L, head_tokens(a.lens, head, a.t0, a.nw, a.n_total) - ch * L));
  const int64_t tok0 = a.t0 + static_cast<int64_t>(ch) * L;
  const int nchp = a.ws.nwp / L;
  // k, v, q; q also takes 2^-ec, the power of two of c (the row weights
  // of this layout use c 2^-ec), on both operand paths
  float mul[3] = {1.f, 1.f, ldexpf(1.f, -a.ec)};
  if (hs.safe) {
    mul[0] = ldexpf(1.f, -hs.ek);
    mul[1] = ldexpf(1.f, -hs.ev);
    mul[2] = ldexpf(1.f, hs.ek - a.ec);
  }
  uint16_t* rec = a.ws.stg + (static_cast<int64_t>(head) * nchp + ch) * (4 * DK * L);
  const uint16_t* src[3] = {static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                            static_cast<const uint16_t*>(a.q)};
  // Every load of the chunk first (a token past the window reads the chunk's
  // first token and is zeroed), then the conversions and LDS writes.
  constexpr int NI = (3 * L * NU + 255) / 256;
  u32x4 raws[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int e = tid + 256 * i;
    const int x = e / (L * NU);
    const int r = e % (L * NU);
    const int t = r / NU, u = r % NU;
    const bool ok = e < 3 * L * NU && t < nvalid;
    const uint16_t* sx = !ok || x == 0 ? src[0] : x == 1 ? src[1] : src[2];
    raws[i] = *reinterpret_cast<const u32x4*>(sx + (static_cast<int64_t>(head) * a.n_total + tok0 + (ok ? t : 0)) * DK +
                                              (ok ? 8 * u : 0));
    if (!ok) raws[i] = u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int e = tid + 256 * i;
    if (e >= 3 * L * NU) break;
    const int x = e / (L * NU);
    const int r = e % (L * NU);
    const int t = r / NU, u = r % NU;
    const u32x4 raw = raws[i];
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t wj = raw[j];
      const float lo = bf16_lo(wj), hi = bf16_hi(wj);
      if (x == 1) {
        vraw[t][8 * u + 2 * j] = lo;
        vraw[t][8 * u + 2 * j + 1] = hi;
      }
      const float mx = x == 0 ? mul[0] : x == 1 ? mul[1] : mul[2];   // no indexed private array
      o[j] = hs.safe ? pack_f16(lo * mx, hi * mx) : (x == 2 && a.ec != 0 ? pack_bf16(lo * mx, hi * mx) : wj);
      tr[x][(8 * u + 2 * j) * TS + t] = static_cast<uint16_t>(o[j] & 0xffffu);
      tr[x][(8 * u + 2 * j + 1) * TS + t] = static_cast<uint16_t>(o[j] >> 16);
    }
    if (x == 2) *reinterpret_cast<u32x4*>(rec + 3 * DK * L + t * DK + 8 * u) = o;
  }
  __syncthreads();
  for (int e = tid; e < 3 * DK * 8; e += 256) {
    const int x = e / (DK * 8);
    const int i = (e / 8) % DK, u = e % 8;
    *reinterpret_cast<u32x4*>(rec + x * DK * L + i * L + 8 * u) =
        *reinterpret_cast<const u32x4*>(&tr[x][i * TS + 8 * u]);
  }
  if (tid <= DV) {
    float s = 0.f;
    if (tid < DV) {
      for (int t = 0; t < nvalid; ++t) s += vraw[t][tid];
    } else {
      s = static_cast<float>(nvalid);
    }
    a.ws.vsum[(static_cast<int64_t>(head) * nchp + ch) * DVP + tid] = s;
  }
}

// ---------------------------------------------------------------------------
// Order-0 carry.  Block = (column c <= DV, head): carry[r][c] = (order-0 entry
// c of the state) + (sum of v[c], or the token count for c = DV, over the
// chunks before readout window r); the state's entry ends as the sum over the
// whole window.  Thread t takes windows [t k, (t + 1) k): the sum of its
// windows, an exclusive scan of the block's sums in LDS, then the carries of
// its windows in order.  One wave a block while the window count is small,
// four waves beyond.
template <int DK, int kCarryThreads>
__global__ __launch_bounds__(kCarryThreads) void prefill_carry(ScanArgs a) {
  constexpr int DV = DK, DVP = padded_dv(DV), L = kL, SC = prefill_window(true) / kL;
  const int c = blockIdx.x;
  const int head = blockIdx.y;
  const int tid = threadIdx.x;
  float* st = a.state + static_cast<int64_t>(head) * a.stride;
  const int64_t zoff = static_cast<int64_t>(a.D) * DV;
  const float s0 = c < DV ? st[c] : st[zoff];
  const int nch = (a.nw + L - 1) / L;
  const int nchp = a.ws.nwp / L;
  const int R = (nch + SC - 1) / SC;
  const int k = (R + kCarryThreads - 1) / kCarryThreads;
  const int r0 = min(R, tid * k), r1 = min(R, r0 + k);
  const float* vs = a.ws.vsum + static_cast<int64_t>(head) * nchp * DVP + c;
  float* carry = a.ws.carry + static_cast<int64_t>(head) * ((a.ws.nwp + SC * L - 1) / (SC * L)) * DVP + c;
  auto window_sum = [&](int r) {
    float v[SC];
#pragma unroll
    for (int j = 0; j < SC; ++j) v[j] = r * SC + j < nch ? vs[static_cast<int64_t>(r * SC + j) * DVP] : 0.f;
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < SC; ++j) s += v[j];
    return s;
  };
  float tot = 0.f;
  for (int r = r0; r < r1; ++r) tot += window_sum(r);
  // inclusive scan of the threads' sums (Hillis-Steele over two buffers)
  __shared__ float sh[2][kCarryThreads];
  int cur = 0;
  sh[0][tid] = tot;
  __syncthreads();
  for (int o = 1; o < kCarryThreads; o <<= 1) {
    const float x = sh[cur][tid] + (tid >= o ? sh[cur][tid - o] : 0.f);
    sh[cur ^ 1][tid] = x;
    cur ^= 1;
    __syncthreads();
  }
  float pre = s0 + (sh[cur][tid] - tot);
  for (int r = r0; r < r1; ++r) {
    carry[static_cast<int64_t>(r) * DVP] = pre;
    pre += window_sum(r);
  }
  if (tid == kCarryThreads - 1) {
    const float fin = s0 + sh[cur][tid];
    if (c < DV)
      st[c] = fin;
    else
      st[zoff] = fin;
  }
}

// ---------------------------------------------------------------------------
// The scan.
template <int DK>
struct CfgS {
  static constexpr int DV = DK;
  static constexpr int L = kL;
  static constexpr int T = prefill_window(true);
  static constexpr int SC = T / L;                 // chunks per readout window
  static constexpr int NW = prefill_waves(true);
  static constexpr int RB = prefill_rb(DK, true);  // 16-row blocks per wave
  static constexpr int NKS = RB / 2;               // readout K-slices (two blocks each)
  static constexpr int NB = col_blocks(DV);        // 16-column blocks incl. den
  static constexpr int NSLOT = prefill_slots(DK, true);
  static constexpr int NU = DK / 8;                // 16-byte units per QN / red row
  static constexpr int ROW_ZERO = DK, ROW_ONES = DK + 1, ROW_SLOT = DK + 2;
  static constexpr int KT_ROWS = ROW_SLOT + NSLOT;
  // LDS carve-up (bytes); tables of 64-token rows are 128 bytes a row.
  static constexpr int KT_B = KT_ROWS * 128;
  static constexpr int VT_B = DV * 128;
  static constexpr int QT_B = (DK + 1) * 128;
  static constexpr int QN_B = L * 2 * DK;
  static constexpr int RED_B = NW * L * 2 * DV;
  // bf16 operand path at d <= 32: the low bf16 half of every wave partial
  static constexpr int REDL_B = DK <= 32 ? RED_B : 0;
  static constexpr int DEN_B = NW * L * 4;
  static constexpr int WL_B = NW * RB * 16 * 4;
  static constexpr int O_KT = 0;
  static constexpr int O_VT = O_KT + 2 * KT_B;
  static constexpr int O_QT = O_VT + 2 * VT_B;
  static constexpr int O_QN = O_QT + 2 * QT_B;
  static constexpr int O_RED = O_QN + 2 * QN_B;
  static constexpr int O_REDL = O_RED + RED_B;
  static constexpr int O_DEN = O_REDL + REDL_B;
  static constexpr int O_WL = O_DEN + DEN_B;
  static constexpr int O_MAX = O_WL + WL_B;
  static constexpr int LDS_B = O_MAX + 16 * NW;
  // DMA: 4 tables of DK/8 blocks of 1 KB per chunk.
  static constexpr int NBLK = 4 * NU;
  static constexpr int NDMA = (NBLK + NW - 1) / NW;
  // Where the den column sits in the readout output (C layout of a block).
  static constexpr int NB_DEN = DV / 16, G_DEN = (DV % 16) / 4, R_DEN = DV % 4;
  static_assert(LDS_B <= 160 * 1024, "LDS budget");
  static_assert(RB % 2 == 0, "readout K-slices pair row blocks");
};

// Swizzles (16-byte units).  A 64-token row of KT / VT / QT / slots keeps its
// eight 8-token units in the order u ^ ((row >> 1) & 7); a QN row (one
// token) keeps its DK/8 units in the order u ^ (((t >> 2) ^ (t >> 5)) & (DK/8 - 1)).
__device__ __forceinline__ int swz_row(int row) { return (row >> 1) & 7; }
template <int NU>
__device__ __forceinline__ int swz_tok(int t) { return ((t >> 2) ^ (t >> 5)) & (NU - 1); }
// Cross-wave buffer row rho (d >= 32): 16-byte unit u at u ^ ((rho ^ (rho >> 3)) & (DV/8 - 1)).
template <int NU>
__device__ __forceinline__ int swz_red(int rho) { return (rho ^ (rho >> 3)) & (NU - 1); }

template <bool H16>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (H16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Elementwise product of three packed 16-bit 8-vectors: f16, two rounded
// products; bf16, the exact fp32 product (8 + 8 + 8 significant bits) rounded
// once.
template <bool H16>
__device__ __forceinline__ u32x4 mul8x3(u32x4 x, u32x4 y, u32x4 z) {
  if constexpr (H16) {
    return __builtin_bit_cast(
        u32x4, __builtin_bit_cast(f16x8, x) * __builtin_bit_cast(f16x8, y) * __builtin_bit_cast(f16x8, z));
  } else {
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t xj = x[j], yj = y[j], zj = z[j];
      r[j] = pack_bf16(bf16_lo(xj) * bf16_lo(yj) * bf16_lo(zj), bf16_hi(xj) * bf16_hi(yj) * bf16_hi(zj));
    }
    return r;
  }
}

// Elementwise product of two packed 16-bit 8-vectors (one MFMA operand).
// f16: packed f16 multiplies; bf16: exact fp32 products rounded once.
template <bool H16>
__device__ __forceinline__ u32x4 mul8(u32x4 x, u32x4 y) {
  if constexpr (H16) {
    return __builtin_bit_cast(u32x4, __builtin_bit_cast(f16x8, x) * __builtin_bit_cast(f16x8, y));
  } else {
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t xj = x[j], yj = y[j];
      r[j] = pack_bf16(bf16_lo(xj) * bf16_lo(yj), bf16_hi(xj) * bf16_hi(yj));
    }
    return r;
  }
}

// One head-tile of the scan with one operand type (the kernel below picks it
// per head).
// P5: orders 0..4, whose order-3 parents carry a third coordinate on both
// sides (a separate instantiation keeps the registers of P <= 4 as they are).
// SO (state only): the state update alone, for the first pass of a prefill
// over sequence segments; no readout operand, readout or records.
template <int DK, bool H16, bool P5, bool SO>
__device__ __forceinline__ void scan_tile(const ScanArgs& a, const HalfScales& hs, unsigned char* lds) {
  using C = CfgS<DK>;
  constexpr int DV = C::DV, L = C::L, NW = C::NW, RB = C::RB, NKS = C::NKS, NB = C::NB, NU = C::NU;
  // d >= 32: a cross-wave buffer unit holds four columns of two adjacent
  // column blocks (one 16-byte write per block pair)
  constexpr bool PAIRED = DV >= 32;
  constexpr int NSLOT = C::NSLOT;
  // bf16 operands at d <= 32: the readout operand and the wave partials are
  // carried as bf16 pairs (value and rounding residual), 16 significant bits,
  // where a single bf16 (8 bits) would pass its rounding to outputs that
  // average few rows.
  constexpr bool LOX = !H16 && DK <= 32;

  const int tile = blockIdx.x;
  const int head = blockIdx.y;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int lr = l & 15;
  const int g = l >> 4;
  const int lay_base = (tile * NW + w) * RB;
  const int nch = (head_tokens(a.lens, head, a.t0, a.nw, a.n_total) + L - 1) / L;
  const int nchp = a.ws.nwp / L;

  // ---- constant rows, row weights -----------------------------------------
  const uint32_t one2 = H16 ? 0x3c003c00u : 0x3f803f80u;
  for (int e = tid; e < 6 * 32; e += NW * 64) {
    const int r = e / 32, j = e % 32;   // KT zero (x2), KT ones (x2), QT ones (x2)
    int off;
    uint32_t val;
    if (r < 2) {
      off = C::O_KT + r * C::KT_B + C::ROW_ZERO * 128;
      val = 0u;
    } else if (r < 4) {
      off = C::O_KT + (r - 2) * C::KT_B + C::ROW_ONES * 128;
      val = one2;
    } else {
      off = C::O_QT + (r - 4) * C::QT_B + DK * 128;
      val = one2;
    }
    *reinterpret_cast<uint32_t*>(lds + off + 4 * j) = val;
  }
  float* wl = reinterpret_cast<float*>(lds + C::O_WL);
  for (int e = tid; e < NW * RB * 16; e += NW * 64)
    wl[e] = a.lay.rweight[static_cast<int64_t>(tile) * NW * RB * 16 + e];

  // ---- per-lane layout constants --------------------------------------------
  // Update: KT byte offsets of the parent and child rows of lane row lr in
  // block b, for the 8-token unit g of the first 32 tokens (the second 32
  // tokens: offset ^ 64).
  uint32_t okpc[RB];   // parent offset | child offset << 16
  // Readout: QT byte offsets of the two parent coordinates of the run of
  // lane group g in block b at tokens 4 lr .. 4 lr + 3, and the QN byte
  // offset of its four children for token block 0 (block mb: + 2 DK mb, odd
  // blocks also - d4).
  uint32_t oq12[RB], oqc[RB];   // oq12: first | second coordinate offset << 16
  uint32_t oq3[RB];             // third coordinate offset (P5 only)
  // Token slot lr of token block mb is token 4 lr + (mb ^ (lr & 1)) (rows of
  // both parities in every QN load); QN offsets of odd blocks are d4 lower.
  const bool odd = lr & 1;
  const uint32_t d4 = odd ? 2 * 2 * DK : 0;   // two token rows
  {
    const int sq = (lr ^ (lr >> 3)) & (NU - 1);
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const uint32_t ks = a.lay.kside[(lay_base + b) * 16 + lr];
      const int pr = ks & 0xffff, cr = ks >> 16;
      okpc[b] = static_cast<uint32_t>(pr * 128 + 16 * (g ^ swz_row(pr))) |
                (static_cast<uint32_t>(cr * 128 + 16 * (g ^ swz_row(cr))) << 16);
      const uint32_t qs = a.lay.qside[(lay_base + b) * 4 + g];
      const int i1 = qs & 255, i2 = (qs >> 8) & 255, c0 = (qs >> 16) & 255, i3 = qs >> 24;
      oq12[b] = static_cast<uint32_t>(i1 * 128 + 16 * ((lr >> 1) ^ swz_row(i1)) + 8 * (lr & 1)) |
                (static_cast<uint32_t>(i2 * 128 + 16 * ((lr >> 1) ^ swz_row(i2)) + 8 * (lr & 1)) << 16);
      oq3[b] = P5 ? static_cast<uint32_t>(i3 * 128 + 16 * ((lr >> 1) ^ swz_row(i3)) + 8 * (lr & 1)) : 0u;
      oqc[b] = (4 * lr + (odd ? 1 : 0)) * 2 * DK + 16 * ((c0 >> 3) ^ sq) + 8 * ((c0 >> 2) & 1);
    }
  }
  // Update, values: VT byte offset of row lr (column block 0), unit g; the
  // rows of block nb are 2048 nb bytes further.
  const uint32_t ovt = (DV >= 16 ? lr : (lr & (DV - 1))) * 128 + 16 * (g ^ swz_row(lr));
  // Parent slots: items (slot, 8-token unit), at most one per thread.
  constexpr int NSI = (NSLOT * 8 + NW * 64 - 1) / (NW * 64);
  const int nslot = a.lay.nslot[tile];
  uint32_t so12[NSI], sod[NSI], so3[NSI];
#pragma unroll
  for (int i = 0; i < NSI; ++i) {
    const int e = tid + i * NW * 64;
    sod[i] = 0xffffffffu;
    so12[i] = 0u;
    so3[i] = 0u;
    if (e < nslot * 8) {
      const int s = e >> 3, u = e & 7;
      const uint32_t par = a.lay.parents[tile * NSLOT + s];
      const int i1 = par & 255, i2 = (par >> 8) & 255, i3 = (par >> 16) & 255, R = C::ROW_SLOT + s;
      so12[i] = static_cast<uint32_t>(i1 * 128 + 16 * (u ^ swz_row(i1))) |
                (static_cast<uint32_t>(i2 * 128 + 16 * (u ^ swz_row(i2))) << 16);
      if constexpr (P5) so3[i] = static_cast<uint32_t>(i3 * 128 + 16 * (u ^ swz_row(i3)));
      sod[i] = R * 128 + 16 * (u ^ swz_row(R));
    }
  }
  // DMA: this wave's blocks of a chunk record: global byte offset per lane,
  // LDS destination per block (buffer 0; buffer 1 adds the table size).
  uint32_t gofs[(C::NDMA + 1) / 2];       // two 16-bit offsets a register
  int ldst[C::NDMA], lstep[C::NDMA];   // wave-uniform
#pragma unroll
  for (int i = 0; i < (C::NDMA + 1) / 2; ++i) gofs[i] = 0u;
#pragma unroll
  for (int i = 0; i < C::NDMA; ++i) {
    const int beta = w + NW * i;
    ldst[i] = -1;
    lstep[i] = 0;
    // the state-only scan reads the key and value tables only
    if (beta < C::NBLK && (!SO || beta / NU < 2)) {
      const int tau = beta / NU, bb = beta % NU;
      const int p = 64 * bb + l;   // 16-byte unit of the table
      if (tau < 3) {
        const int row = p >> 3, q = p & 7;
        gofs[i / 2] |= static_cast<uint32_t>(tau * DK * 128 + (row * 8 + (q ^ swz_row(row))) * 16) << (16 * (i & 1));
      } else {
        const int t = p / NU, q = p % NU;
        gofs[i / 2] |= static_cast<uint32_t>(3 * DK * 128 + (t * NU + (q ^ swz_tok<NU>(t))) * 16) << (16 * (i & 1));
      }
      const int base = tau == 0 ? C::O_KT : tau == 1 ? C::O_VT : tau == 2 ? C::O_QT : C::O_QN;
      lstep[i] = __builtin_amdgcn_readfirstlane(tau == 0 ? C::KT_B : tau == 1 ? C::VT_B : tau == 2 ? C::QT_B : C::QN_B);
      ldst[i] = __builtin_amdgcn_readfirstlane(base + 1024 * bb);
    }
  }
  const unsigned char* stg = reinterpret_cast<const unsigned char*>(a.ws.stg) +
                             static_cast<int64_t>(head) * nchp * (8 * DK * L);
  // Block i of this wave's share of chunk ch into buffer X.
  auto dma_one = [&](int i, int ch, int X) {
    if ((!SO && C::NBLK % NW == 0) || ldst[i] >= 0)
      dma16(stg + static_cast<int64_t>(ch) * (8 * DK * L) + ((gofs[i / 2] >> (16 * (i & 1))) & 0xffffu),
            lds + __builtin_amdgcn_readfirstlane(ldst[i] + X * lstep[i]));
  };
  auto dma = [&](int ch, int X) {
#pragma unroll
    for (int i = 0; i < C::NDMA; ++i) dma_one(i, ch, X);
  };

  // ---- state tile into registers (C layout: lane holds column 16 nb + lr of
  // rows 4 g + r of block b); f16 path: times 2^-(p ek + ev) for a value
  // column of an order-p row, 2^-(p ek) for den.
  float* st = a.state + static_cast<int64_t>(head) * a.stride;
  const int64_t zoff = static_cast<int64_t>(a.D) * DV;
  const int64_t off2 = 1 + DK, off3 = 1 + DK + static_cast<int64_t>(DK) * (DK + 1) / 2;
  const int64_t off4 = off3 + static_cast<int64_t>(DK) * (DK + 1) * (DK + 2) / 6;
  auto row_exp = [&](int64_t m, bool value_col) {
    const int p = (P5 && m >= off4) ? 4 : m >= off3 ? 3 : m >= off2 ? 2 : m >= 1 ? 1 : 0;
    return p * hs.ek + (value_col ? hs.ev : 0);
  };
  // Every row index first, then every load with no branch between them (a
  // pad row or a column past den reads a valid word and is zeroed after), so
  // the loads are all in flight at once; offsets are 32-bit (a head's state
  // is below 2^32 bytes).
  uint32_t info[RB][4];
  float wr_lane[RB][4];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      info[b][r] = a.lay.rowinfo[(lay_base + b) * 16 + 4 * g + r];
      wr_lane[b][r] = a.lay.rweight[(lay_base + b) * 16 + 4 * g + r];
    }
  f32x4 S[RB][NB];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t m = info[b][r] ? info[b][r] - 1 : 0u;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = nb * 16 + lr;
        const uint32_t off = col < DV ? m * DV + col : static_cast<uint32_t>(zoff) + m;
        S[b][nb][r] = st[off];
      }
    }
  // Chunk 0's tables go out behind the state loads (loads retire in order, so
  // the wait for the state does not wait for these).
  if (nch > 0) dma(0, 0);
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t m = info[b][r] ? info[b][r] - 1 : 0u;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = nb * 16 + lr;
        float val = S[b][nb][r];
        if constexpr (H16) val = ldexpf(val, -row_exp(m, col < DV));
        S[b][nb][r] = (info[b][r] != 0u && col <= DV) ? val : 0.f;
      }
    }

  // ---- readout operand: Sb = S w 2^-ew, one ew per tile and readout window
  // (f16: max |S| max(w) 2^-ew in [2^(sb-1), 2^sb); bf16: ew = 0).  Two steps around a
  // barrier: each wave posts its max |S|, then every wave derives ew from
  // the tile's max and rounds its slice.
  u32x4 Sb[NKS][NB];
  u32x4 Sbl[LOX ? NKS : 1][NB];   // residual of Sb (LOX)
  int ew = 0;
  float* wmx = reinterpret_cast<float*>(lds + C::O_MAX);
  // Largest row weight of the lane's rows: max |S| times it bounds max |S w|.
  float wlmax = 0.f;
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) wlmax = fmaxf(wlmax, fabsf(wr_lane[b][r]));
  auto post_max = [&]() {
    if constexpr (H16) {
      float mx = 0.f;
#pragma unroll
      for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(S[b][nb][r]));
      mx = wave_max(mx * wlmax);
      if (l == 0) wmx[w] = mx;
    }
  };
  auto refresh = [&]() {
    float sc = 1.f;
    if constexpr (H16) {
      float mx = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) mx = fmaxf(mx, wmx[ww]);
      int e = 0;
      if (mx > 0.f) (void)frexpf(mx, &e);
      ew = __builtin_amdgcn_readfirstlane(mx > 0.f ? e - hs.sb : 0);
      sc = ldexpf(1.f, -ew);
    }
    const float* wb = wl + (w * RB) * 16 + 4 * g;
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const f32x4 wr = *reinterpret_cast<const f32x4*>(wb + 16 * b) * sc;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const f32x4 x = S[b][nb] * wr;
        if constexpr (H16) {
          Sb[b / 2][nb][2 * (b % 2)] = pack_f16(x[0], x[1]);
          Sb[b / 2][nb][2 * (b % 2) + 1] = pack_f16(x[2], x[3]);
        } else {
          const uint32_t h0 = pack_bf16(x[0], x[1]), h1 = pack_bf16(x[2], x[3]);
          Sb[b / 2][nb][2 * (b % 2)] = h0;
          Sb[b / 2][nb][2 * (b % 2) + 1] = h1;
          if constexpr (LOX) {
            Sbl[b / 2][nb][2 * (b % 2)] = pack_bf16(x[0] - bf16_lo(h0), x[1] - bf16_hi(h0));
            Sbl[b / 2][nb][2 * (b % 2) + 1] = pack_bf16(x[2] - bf16_lo(h1), x[3] - bf16_hi(h1));
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- records ---------------------------------------------------------------
  using RedT = typename std::conditional<prefill_bf16_records(DK, true), uint16_t, float>::type;
  const int nwp = a.ws.nwp;
  RedT* rech = static_cast<RedT*>(a.ws.rec) + (static_cast<int64_t>(head) * a.lay.n_tiles + tile) * nwp * DV;
  float* reczh = a.ws.recz + (static_cast<int64_t>(head) * a.lay.n_tiles + tile) * nwp;
  // chunk scales [head][chunk][tile]: a reduce block reads its chunk's tiles contiguously
  float* recsh = a.ws.recs + static_cast<int64_t>(head) * (nwp / L) * a.lay.n_tiles + tile;
  static_assert(NW * 32768 <= (32768 << kRecShift), "f16 records stay in range");
  const uint16_t* red = reinterpret_cast<const uint16_t*>(lds + C::O_RED);
  const uint16_t* redl = reinterpret_cast<const uint16_t*>(lds + C::O_REDL);
  const float* den = reinterpret_cast<const float*>(lds + C::O_DEN);
  // Two stacked 16 x 16 identities as an MFMA A operand (16-bit ones of the
  // partials' type): lane (lr, g) holds row lr, K = 8 g .. 8 g + 7; entry 1
  // where K % 16 == lr (built at use).
  auto eye2 = [&]() {
    const uint32_t one = H16 ? 0x3c00u : 0x3f80u;
    u32x4 e;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = 8 * (g & 1) + 2 * j == lr ? one : 0u;
      const uint32_t hi = 8 * (g & 1) + 2 * j + 1 == lr ? one : 0u;
      e[j] = lo | (hi << 16);
    }
    return e;
  };

  // Cross-wave sum of chunk ch's readout, times 2^ew, into the records.
  // Value columns on MFMA: for a block of 16 tokens x 16 buffer positions,
  //   sum_w P_w^T = sum over wave pairs p of [I I] [P_2p; P_2p+1]^T,
  // A = two stacked 16 x 16 identities, B = the 16-bit partials of two waves
  // (K = wave x position); D^T gives lane (lr, g) token slot lr, positions
  // 4 g + r (four consecutive columns).  Red row rho = lr + 16 mb holds token
  // 4 lr + (mb ^ (lr & 1)).  den: fp32 partials summed by the last wave, one
  // token per lane.
  constexpr int NCB = (DV + 15) / 16;        // 16-position blocks of a row
  constexpr int NITEM = 4 * NCB;             // (token block, position block)
  constexpr int NIW = (NITEM + NW - 1) / NW; // items per wave
  auto red_sum = [&](int ch) {
    const float sc = ldexpf(1.f, ew);
    const u32x4 eye = eye2();
#pragma unroll
    for (int i = 0; i < NIW; ++i) {
      const int item = w + NW * i;
      if (item < NITEM) {
        const int tb = item / NCB, cb = item % NCB;
        const int rho = 16 * tb + lr;
        const int unit = 2 * cb + (g & 1);
        const int upos = PAIRED ? (unit ^ swz_red<NU>(rho)) : (unit ^ (swz_row(rho) % NU));
        f32x4 D = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int pq = 0; pq < NW / 2; ++pq) {
          const int ww = 2 * pq + (g >> 1);
          u32x4 x = {0u, 0u, 0u, 0u};
          if (DV >= 16 || (g & 1) == 0)
            x = *reinterpret_cast<const u32x4*>(&red[ww * L * DV + rho * DV + 8 * upos]);
          D = mfma16<H16>(eye, x, D);
          if constexpr (LOX) {
            u32x4 xl = {0u, 0u, 0u, 0u};
            if (DV >= 16 || (g & 1) == 0)
              xl = *reinterpret_cast<const u32x4*>(&redl[ww * L * DV + rho * DV + 8 * upos]);
            D = mfma16<H16>(eye, xl, D);
          }
        }
        const int t = 4 * lr + (tb ^ (lr & 1));
        // positions 4 g .. 4 g + 3 of block cb = units 2 cb + (g >> 1), half g & 1
        const int col = PAIRED ? 32 * (cb >> 1) + 16 * (g & 1) + 8 * (cb & 1) + 4 * (g >> 1) : 16 * cb + 4 * g;
        if (col < DV) {
          const int64_t ro = (static_cast<int64_t>(ch) * L + t) * DV + col;
          if constexpr (std::is_same<RedT, uint16_t>::value && H16) {
            constexpr float rs = 1.f / (1 << kRecShift);
            const u32x2 o = {pack_f16(D[0] * rs, D[1] * rs), pack_f16(D[2] * rs, D[3] * rs)};
            __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(&rech[ro]));   // read once, later
          } else if constexpr (std::is_same<RedT, uint16_t>::value) {
            const u32x2 o = {pack_bf16(D[0] * sc, D[1] * sc), pack_bf16(D[2] * sc, D[3] * sc)};
            __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(&rech[ro]));
          } else {
            __builtin_nontemporal_store(D * sc, reinterpret_cast<f32x4*>(&rech[ro]));
          }
        }
      }
    }
    if constexpr (std::is_same<RedT, uint16_t>::value && H16) {
      if (tid == 0) recsh[static_cast<int64_t>(ch) * a.lay.n_tiles] = ldexpf(1.f, ew + kRecShift);
    }
    if (tid >= (NW - 1) * 64) {
      float sz = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) sz += den[ww * L + l];
      __builtin_nontemporal_store(sz * sc, &reczh[static_cast<int64_t>(ch) * L + l]);
    }
  };

  // Parent features of the parent slots of a chunk (buffer X): products of
  // two key rows (order 2) or three (order 3, orders 0..4 only).
  auto slots = [&](int X) {
    unsigned char* kt = lds + C::O_KT + X * C::KT_B;
#pragma unroll
    for (int i = 0; i < NSI; ++i) {
      if (sod[i] != 0xffffffffu) {
        const u32x4 x1 = *reinterpret_cast<const u32x4*>(kt + (so12[i] & 0xffffu));
        const u32x4 x2 = *reinterpret_cast<const u32x4*>(kt + (so12[i] >> 16));
        if constexpr (P5) {
          const u32x4 x3 = *reinterpret_cast<const u32x4*>(kt + so3[i]);
          *reinterpret_cast<u32x4*>(kt + sod[i]) = mul8x3<H16>(x1, x2, x3);
        } else {
          *reinterpret_cast<u32x4*>(kt + sod[i]) = mul8<H16>(x1, x2);
        }
      }
    }
  };

  static_assert(RB * 16 <= 64, "the f16 partial bound assumes at most 64 rows a wave");
  auto pack_red = [&](float x, float y) {
    if constexpr (H16)
      return pack_f16(x, y);
    else
      return pack_bf16(x, y);
  };

  // Readout of chunk X's queries against Sb into the cross-wave buffer.
  // MFMA: A = Sb^T (16 value columns x 32 rows), B = phi_q^T (32 rows x 16
  // tokens), so lane (lr, g) gets token slot lr, columns 16 nb + 4 g + r.
  // Token slot lr of token block mb is token 4 lr + (mb ^ (lr & 1)).
  auto readout = [&](int X, auto&& hook) {
    const unsigned char* qt = lds + C::O_QT + X * C::QT_B;
    const unsigned char* qn = lds + C::O_QN + X * C::QN_B;
    uint16_t* redw = reinterpret_cast<uint16_t*>(lds + C::O_RED) + w * L * DV;
    uint16_t* redwl = reinterpret_cast<uint16_t*>(lds + C::O_REDL) + w * L * DV;
    // Parent products for the lane's four tokens, in token-block order
    // (element mb holds token 4 lr + (mb ^ (lr & 1))).
    u32x2 pp[RB];
    float pf[RB][4];
    const uint32_t psel = odd ? 0x01000302u : 0x03020100u;   // byte select: swap the halves
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const u32x2 x1 = *reinterpret_cast<const u32x2*>(qt + (oq12[b] & 0xffffu));
      const u32x2 x2 = *reinterpret_cast<const u32x2*>(qt + (oq12[b] >> 16));
      // third coordinate (the ones row unless the parent has order 3)
      const u32x2 x3 = P5 ? *reinterpret_cast<const u32x2*>(qt + oq3[b]) : u32x2{one2, one2};
      if constexpr (H16) {
        f16x4 p = __builtin_bit_cast(f16x4, x1) * __builtin_bit_cast(f16x4, x2);
        if constexpr (P5) p = p * __builtin_bit_cast(f16x4, x3);
        const u32x2 pw = __builtin_bit_cast(u32x2, p);
        pp[b] = u32x2{__builtin_amdgcn_perm(pw[0], pw[0], psel), __builtin_amdgcn_perm(pw[1], pw[1], psel)};
      } else {
        float v[4] = {bf16_lo(x1[0]) * bf16_lo(x2[0]), bf16_hi(x1[0]) * bf16_hi(x2[0]),
                      bf16_lo(x1[1]) * bf16_lo(x2[1]), bf16_hi(x1[1]) * bf16_hi(x2[1])};
        if constexpr (P5) {
          v[0] *= bf16_lo(x3[0]);
          v[1] *= bf16_hi(x3[0]);
          v[2] *= bf16_lo(x3[1]);
          v[3] *= bf16_hi(x3[1]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) pf[b][j] = odd ? v[j ^ 1] : v[j];
      }
    }
    float dn[4] = {0.f, 0.f, 0.f, 0.f};
    auto load_c = [&](int mb, int kk, u32x2 (&c)[2]) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        c[h] = *reinterpret_cast<const u32x2*>(qn + (oqc[2 * kk + h] - ((mb & 1) ? d4 : 0u)) + 2 * DK * mb);
    };
    auto build = [&](int mb, int kk, const u32x2 (&c)[2]) {
      u32x4 B;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int b = 2 * kk + h;
        if constexpr (H16) {
          const uint32_t pw = pp[b][mb >> 1];   // scalar copy: bit_cast of a vector element is miscompiled
          const _Float16 p = __builtin_bit_cast(f16x2, pw)[mb & 1];
          const f16x4 x = __builtin_bit_cast(f16x4, c[h]) * p;
          const u32x2 xw = __builtin_bit_cast(u32x2, x);
          B[2 * h] = xw[0];
          B[2 * h + 1] = xw[1];
        } else {
          const float p = pf[b][mb];
          B[2 * h] = pack_bf16(bf16_lo(c[h][0]) * p, bf16_hi(c[h][0]) * p);
          B[2 * h + 1] = pack_bf16(bf16_lo(c[h][1]) * p, bf16_hi(c[h][1]) * p);
        }
      }
      return B;
    };
    constexpr int NST = 4 * NKS;
    // child loads run two steps ahead of their use (a ring of two)
    u32x2 cr[2][2];
    load_c(0, 0, cr[0]);
    u32x4 Bcur = build(0, 0, cr[0]);
    if (NST > 1) load_c(1 / NKS, 1 % NKS, cr[1]);
    if (NST > 2) load_c(2 / NKS, 2 % NKS, cr[0]);
    f32x4 acc[NB];
#pragma unroll
    for (int s_ = 0; s_ < NST; ++s_) {
      const int mb = s_ / NKS, kk = s_ % NKS;
      hook(s_);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        acc[nb] = mfma16<H16>(Sb[kk][nb], Bcur, kk == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[nb]);
        if constexpr (LOX) acc[nb] = mfma16<H16>(Sbl[kk][nb], Bcur, acc[nb]);
      }
      u32x4 Bnext = Bcur;
      if (s_ + 1 < NST) Bnext = build((s_ + 1) / NKS, (s_ + 1) % NKS, cr[(s_ + 1) & 1]);
      if (s_ + 3 < NST) load_c((s_ + 3) / NKS, (s_ + 3) % NKS, cr[(s_ + 1) & 1]);
      if (kk == NKS - 1) {
        const int rho = lr + 16 * mb;
        if constexpr (PAIRED) {
          // unit 4 P + g = columns 32 P + 4 g .. +3 and 32 P + 16 + 4 g .. +3
#pragma unroll
          for (int P = 0; P < DV / 32; ++P) {
            const uint32_t o0 = pack_red(acc[2 * P][0], acc[2 * P][1]), o1 = pack_red(acc[2 * P][2], acc[2 * P][3]);
            const uint32_t o2 = pack_red(acc[2 * P + 1][0], acc[2 * P + 1][1]);
            const uint32_t o3 = pack_red(acc[2 * P + 1][2], acc[2 * P + 1][3]);
            const int ro = rho * DV + 8 * ((4 * P + g) ^ swz_red<NU>(rho));
            *reinterpret_cast<u32x4*>(&redw[ro]) = u32x4{o0, o1, o2, o3};
            if constexpr (LOX) {
              const u32x4 ol = {pack_bf16(acc[2 * P][0] - bf16_lo(o0), acc[2 * P][1] - bf16_hi(o0)),
                                pack_bf16(acc[2 * P][2] - bf16_lo(o1), acc[2 * P][3] - bf16_hi(o1)),
                                pack_bf16(acc[2 * P + 1][0] - bf16_lo(o2), acc[2 * P + 1][1] - bf16_hi(o2)),
                                pack_bf16(acc[2 * P + 1][2] - bf16_lo(o3), acc[2 * P + 1][3] - bf16_hi(o3))};
              *reinterpret_cast<u32x4*>(&redwl[ro]) = ol;
            }
          }
        } else {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            if (16 * nb < DV && (16 * nb + 16 <= DV || 4 * g < DV % 16)) {
              const int cu = 2 * nb + (g >> 1);
              const uint32_t o0 = pack_red(acc[nb][0], acc[nb][1]), o1 = pack_red(acc[nb][2], acc[nb][3]);
              const int ro = rho * DV + 8 * (cu ^ (swz_row(rho) % NU)) + 4 * (g & 1);
              *reinterpret_cast<u32x2*>(&redw[ro]) = u32x2{o0, o1};
              if constexpr (LOX) {
                const u32x2 ol = {pack_bf16(acc[nb][0] - bf16_lo(o0), acc[nb][1] - bf16_hi(o0)),
                                  pack_bf16(acc[nb][2] - bf16_lo(o1), acc[nb][3] - bf16_hi(o1))};
                *reinterpret_cast<u32x2*>(&redwl[ro]) = ol;
              }
            }
          }
        }
        dn[mb] = acc[C::NB_DEN][C::R_DEN];
      }
      __builtin_amdgcn_sched_barrier(0);
      Bcur = Bnext;
    }
    if (g == C::G_DEN)   // tokens 4 lr + j, j = mb ^ (lr & 1)
      *reinterpret_cast<f32x4*>(lds + C::O_DEN + (w * L + 4 * lr) * 4) =
          odd ? f32x4{dn[1], dn[0], dn[3], dn[2]} : f32x4{dn[0], dn[1], dn[2], dn[3]};
  };

  // State update of chunk X: S += phi_k(K)^T [V 1].  A = key features (16
  // rows x 32 tokens) = parent row x child row; B = V' (32 tokens x 16
  // columns), the den block a constant.
  auto update = [&](int X, auto&& hook) {
    const unsigned char* kt = lds + C::O_KT + X * C::KT_B;
    const unsigned char* vt = lds + C::O_VT + X * C::VT_B;
    constexpr int NST = 2 * RB;
    auto load_k = [&](int st_, u32x4 (&d)[2]) {
      const int kst = st_ / RB, b = st_ % RB;
      d[0] = *reinterpret_cast<const u32x4*>(kt + ((okpc[b] & 0xffffu) ^ (64 * kst)));
      d[1] = *reinterpret_cast<const u32x4*>(kt + ((okpc[b] >> 16) ^ (64 * kst)));
    };
    u32x4 Bv[NB];
    auto load_v = [&](int kst) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = 16 * nb + lr;
        const uint32_t cst = col == DV ? one2 & 0xffffu : 0u;   // den column: ones
        if (16 * nb >= DV) {
          const uint32_t c2 = cst | (cst << 16);
          Bv[nb] = u32x4{c2, c2, c2, c2};
        } else {
          const u32x4 x = *reinterpret_cast<const u32x4*>(vt + ((ovt ^ (64 * kst)) + 2048 * nb));
          if (16 * nb + 16 <= DV) {
            Bv[nb] = x;
          } else {
            const uint32_t c2 = cst | (cst << 16);
            Bv[nb] = col < DV ? x : u32x4{c2, c2, c2, c2};
          }
        }
      }
    };
    u32x4 dk[2];
    load_k(0, dk);
    u32x4 Acur = mul8<H16>(dk[0], dk[1]);
    if (NST > 1) load_k(1, dk);
#pragma unroll
    for (int st_ = 0; st_ < NST; ++st_) {
      const int kst = st_ / RB, b = st_ % RB;
      hook(st_);
      if (b == 0) load_v(kst);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) S[b][nb] = mfma16<H16>(Acur, Bv[nb], S[b][nb]);
      u32x4 Anext = Acur;
      if (st_ + 1 < NST) Anext = mul8<H16>(dk[0], dk[1]);
      if (st_ + 2 < NST) load_k(st_ + 2, dk);
      __builtin_amdgcn_sched_barrier(0);
      Acur = Anext;
    }
  };

  // ---- prologue: chunk 0's parent slots, the first Sb ---------------------------
  if constexpr (!SO) post_max();
  dma_barrier();
  slots(0);
  if constexpr (!SO) refresh();
  lds_barrier();

  // ---- chunks -------------------------------------------------------------------
  // One chunk with its table buffer X as a compile-time constant (the loop
  // below runs chunk pairs), so every buffer base folds into the immediate
  // offset of the LDS instructions instead of costing address arithmetic.
  auto chunk = [&](auto Xc, int ch) {
    constexpr int X = decltype(Xc)::value;
#pragma unroll
    for (int b = 0; b < RB; ++b) asm volatile("" : "+v"(okpc[b]));
    if constexpr (SO) {
      // the next chunk's tables, then this chunk's update and the next
      // chunk's parent slots
      dma(ch + 1 < nch ? ch + 1 : ch, X ^ 1);
      update(X, [](int) {});
      dma_barrier();
      if (ch + 1 < nch) slots(X ^ 1);
      lds_barrier();
      return;
    }
    // segment 1: read out this chunk; the next chunk's DMA goes out one
    // block per readout step
    if (ch > 0 && ch % C::SC == 0) refresh();
    // No branch around the DMA (a branch there splits the readout steps
    // and undoes their software pipelining): the last chunk re-fetches
    // itself into the idle buffer, which is never read again.
    const int chn = ch + 1 < nch ? ch + 1 : ch;
    readout(X, [&](int step) {
      if (step < C::NDMA) dma_one(step, chn, X ^ 1);
    });
    dma_barrier();
    // segment 2: records of this chunk, parent slots of the next, update;
    // the two waves sharing a SIMD take these in opposite orders
    auto side = [&]() {
      red_sum(ch);
      if (ch + 1 < nch) slots(X ^ 1);
    };
    auto none = [&](int) {};
    if (w < NW / 2) {
      update(X, none);
      side();
    } else {
      side();
      update(X, none);
    }
    if (ch % C::SC == C::SC - 1 && ch + 1 < nch) post_max();
    lds_barrier();
  };
  for (int ch = 0; ch < nch; ch += 2) {
    chunk(std::integral_constant<int, 0>{}, ch);
    if (ch + 1 < nch) chunk(std::integral_constant<int, 1>{}, ch + 1);
  }

  // ---- state tile back (f16 path: unscaled) --------------------------------------
  // Row indices again (the loop leaves no registers to keep them), all
  // loaded before the first store.
  const uint32_t* rowinfo = a.lay.rowinfo;
  float* stw = st;
  asm volatile("" : "+s"(rowinfo), "+s"(stw));
  uint32_t info2[RB][4];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) info2[b][r] = rowinfo[(lay_base + b) * 16 + 4 * g + r];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t m = info2[b][r] - 1;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = nb * 16 + lr;
        float val = S[b][nb][r];
        if constexpr (H16) val = ldexpf(val, row_exp(m, col < DV));
        if (info2[b][r] != 0u && col <= DV) stw[col < DV ? m * DV + col : static_cast<uint32_t>(zoff) + m] = val;
      }
    }
  }
}

template <int DK, bool P5, bool SO>
__global__ __launch_bounds__(prefill_waves(true) * 64, 1) void prefill_scan_b16(ScanArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[CfgS<DK>::LDS_B];
  // no tokens of this head in the window: the state is left as it is
  if (head_tokens(a.lens, blockIdx.y, a.t0, a.nw, a.n_total) == 0) return;
  const HalfScales hs = head_scales(a.ws, blockIdx.y, a.P, a.ec);
  if (hs.safe)
    scan_tile<DK, true, P5, SO>(a, hs, lds);
  else
    scan_tile<DK, false, P5, SO>(a, hs, lds);
}

// ---------------------------------------------------------------------------
// out = (intra + sum over tiles of the records + carry) for num / for den,
// summed in a fixed order.  Block = (32 tokens, head); den per token first
// (eight interleaved tile sums, combined in order), then value items of 8
// columns.  Records are read once: non-temporal loads, sixteen (or eight)
// tiles in flight a thread.
// Reduce blocks: 32 tokens x 256 threads (64 x 256: 1.5 % slower; 16 x 128
// and 32 x 128: 5-17 % slower, 64 heads x 4096 tokens at d = 64).
constexpr int kRedTok = 32;           // tokens per reduce block
constexpr int kRedThr = 256;          // threads per reduce block
template <int DK>
__global__ __launch_bounds__(kRedThr) void prefill_reduce_b16(ReduceArgs a) {
  constexpr int DV = DK, DVP = padded_dv(DV), T = prefill_window(true), NU = DV / 8, TB = kRedTok;
  constexpr int QQ = kRedThr / TB;    // interleaved den sums per token
  static_assert(QQ >= 1 && QQ * TB == kRedThr, "reduce block shape");
  using RedT = typename std::conditional<prefill_bf16_records(DK, true), uint16_t, float>::type;
  __shared__ float dsh[TB];
  __shared__ float dpart[QQ][TB];
  const int head = blockIdx.y;
  const int t0 = blockIdx.x * TB;
  const int tid = threadIdx.x;
  const int nwp = a.ws.nwp;
  const int nt = a.n_tiles;
  const int ntok = min(TB, head_tokens(a.lens, head, a.t0, a.nw, a.n_total) - t0);   // may be <= 0
  const int nout = min(TB, a.nw - t0);   // rows of the block; those past ntok are written as zeros
  const HalfScales hs = head_scales(a.ws, head, a.P, a.ec);
  const float rscale = hs.safe ? ldexpf(1.f, hs.ev) : 1.f;   // value-column records carry 2^-ev
  const float* intra = a.ws.intra + static_cast<int64_t>(head) * nwp * DVP;
  const float* carry = a.ws.carry + static_cast<int64_t>(head) * ((nwp + T - 1) / T) * DVP;
  {
    const int tt = tid % TB, qq = tid / TB;   // QQ interleaved sums per token
    float s = 0.f;
    if (tt < ntok) {
      const float* rz = a.ws.recz + static_cast<int64_t>(head) * nt * nwp + t0 + tt;
      // groups of eight loads in flight, summed in tile order
      int tl = qq;
      for (; tl + 7 * QQ < nt; tl += 8 * QQ) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = __builtin_nontemporal_load(rz + static_cast<int64_t>(tl + QQ * i) * nwp);
#pragma unroll
        for (int i = 0; i < 8; ++i) s += x[i];
      }
      for (; tl < nt; tl += QQ) s += __builtin_nontemporal_load(rz + static_cast<int64_t>(tl) * nwp);
    }
    dpart[qq][tt] = s;
  }
  __syncthreads();
  if (tid < TB) {
    const int t = t0 + tid;
    float s = dpart[0][tid];
#pragma unroll
    for (int j = 1; j < QQ; ++j) s += dpart[j][tid];
    if (tid < ntok) {
      s += intra[static_cast<int64_t>(t) * DVP + DV];
      s += carry[(t / T) * DVP + DV];
    }
    dsh[tid] = s;
  }
  __syncthreads();
  const RedT* rec = static_cast<const RedT*>(a.ws.rec) + static_cast<int64_t>(head) * nt * nwp * DV;
  float* out = a.out + (static_cast<int64_t>(head) * a.n_total + a.t0) * DV;
  // f16 records: scale of this block's chunk (32 | 64) per tile
  const int nchp = nwp / 64;
  const float* rsc = a.ws.recs + (static_cast<int64_t>(head) * nchp + t0 / 64) * nt;
  for (int e = tid; e < ntok * NU; e += kRedThr) {
    const int tt = e / NU, u = e % NU;
    const int t = t0 + tt;
    float r[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = 0.f;
    const RedT* rp = rec + static_cast<int64_t>(t) * DV + 8 * u;
    const int64_t tstride = static_cast<int64_t>(nwp) * DV;
    int tl = 0;
    if constexpr (std::is_same<RedT, uint16_t>::value) {
      // groups of G record loads in flight, folded in tile order; f16
      // records (heads on the f16 operand path) times their chunk scale.
      // G = 16 up to 256 tiles (eight: 4 % slower at d = 64, P = 4, 101
      // tiles), else 8 (sixteen: 25-40 % slower at d = 64, P = 5, 1745 tiles
      // whose records lie 512 KB apart)
      auto sum16 = [&](auto f16c, auto gc) {
        constexpr bool F16 = decltype(f16c)::value;
        constexpr int G = decltype(gc)::value;
        for (; tl + G - 1 < nt; tl += G) {
          u32x4 x[G];
          float sv[G];
#pragma unroll
          for (int i = 0; i < G; ++i) {
            x[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rp + (tl + i) * tstride));
            sv[i] = F16 ? rsc[tl + i] : 1.f;
          }
#pragma unroll
          for (int i = 0; i < G; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint32_t xj = x[i][j];
              if constexpr (F16) {
                r[2 * j] = fmaf(f16_lo(xj), sv[i], r[2 * j]);
                r[2 * j + 1] = fmaf(f16_hi(xj), sv[i], r[2 * j + 1]);
              } else {
                r[2 * j] += bf16_lo(xj);
                r[2 * j + 1] += bf16_hi(xj);
              }
            }
        }
        for (; tl < nt; ++tl) {
          const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rp + tl * tstride));
          const float sv = F16 ? rsc[tl] : 1.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if constexpr (F16) {
              r[2 * j] = fmaf(f16_lo(x[j]), sv, r[2 * j]);
              r[2 * j + 1] = fmaf(f16_hi(x[j]), sv, r[2 * j + 1]);
            } else {
              r[2 * j] += bf16_lo(x[j]);
              r[2 * j + 1] += bf16_hi(x[j]);
            }
          }
        }
      };
      using G16 = std::integral_constant<int, 16>;
      using G8 = std::integral_constant<int, 8>;
      if (nt <= 256) {
        if (hs.safe)
          sum16(std::true_type{}, G16{});
        else
          sum16(std::false_type{}, G16{});
      } else {
        if (hs.safe)
          sum16(std::true_type{}, G8{});
        else
          sum16(std::false_type{}, G8{});
      }
    } else {
#pragma unroll 4
      for (; tl < nt; ++tl) {
        const f32x4 x0 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(rp + tl * tstride));
        const f32x4 x1 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(rp + tl * tstride + 4));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          r[j] += x0[j];
          r[4 + j] += x1[j];
        }
      }
    }
    const float* ip = intra + static_cast<int64_t>(t) * DVP + 8 * u;
    const float* cp = carry + (t / T) * DVP + 8 * u;
    const float dinv = 1.f / dsh[tt];
    f32x4 o0, o1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o0[j] = (ip[j] + r[j] * rscale + cp[j]) * dinv;
      o1[j] = (ip[4 + j] + r[4 + j] * rscale + cp[4 + j]) * dinv;
    }
    *reinterpret_cast<f32x4*>(out + static_cast<int64_t>(t) * DV + 8 * u) = o0;
    *reinterpret_cast<f32x4*>(out + static_cast<int64_t>(t) * DV + 8 * u + 4) = o1;
  }
  // rows past the head's length
  const int nz = max(ntok, 0);
  for (int e = tid; e < (nout - nz) * DV; e += kRedThr)
    out[static_cast<int64_t>(t0 + nz) * DV + e] = 0.f;
}

template <int D>
hipError_t launch_b16_t(int BH, const ScanArgs& a, hipStream_t s) {
  const int nch = (a.nw + kL - 1) / kL;
  prefill_amax<D><<<dim3(kAmaxSplit, BH), 256, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prefill_stage<D><<<dim3(nch, BH), 256, 0, s>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int windows = (nch + prefill_window(true) / kL - 1) / (prefill_window(true) / kL);
  if (windows <= 256)
    prefill_carry<D, 64><<<dim3(D + 1, BH), 64, 0, s>>>(a);
  else
    prefill_carry<D, 256><<<dim3(D + 1, BH), 256, 0, s>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const dim3 grid(a.lay.n_tiles, BH);
  constexpr int NT = prefill_waves(true) * 64;
  if (a.state_only) {
    if (a.P == 5)
      prefill_scan_b16<D, true, true><<<grid, NT, 0, s>>>(a);
    else
      prefill_scan_b16<D, false, true><<<grid, NT, 0, s>>>(a);
  } else {
    if (a.P == 5)
      prefill_scan_b16<D, true, false><<<grid, NT, 0, s>>>(a);
    else
      prefill_scan_b16<D, false, false><<<grid, NT, 0, s>>>(a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_reduce_b16_t(int BH, const ReduceArgs& a, hipStream_t s) {
  prefill_reduce_b16<D><<<dim3((a.nw + kRedTok - 1) / kRedTok, BH), kRedThr, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

namespace {
constexpr int kStateThreads = 256;
// Elementwise kernels over segment states (grid-stride over nf floats).
__global__ __launch_bounds__(kStateThreads) void state_copy(float* dst, const float* src, int64_t nf) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kStateThreads + threadIdx.x; i < nf;
       i += static_cast<int64_t>(gridDim.x) * kStateThreads)
    dst[i] = src[i];
}
__global__ __launch_bounds__(kStateThreads) void state_zero(float* T, int64_t ts, int64_t nf) {
  float* t = T + static_cast<int64_t>(blockIdx.y) * ts;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kStateThreads + threadIdx.x; i < nf;
       i += static_cast<int64_t>(gridDim.x) * kStateThreads)
    t[i] = 0.f;
}
__global__ __launch_bounds__(kStateThreads) void state_prefix(float* T, int64_t ts, int G, int64_t nf) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kStateThreads + threadIdx.x; i < nf;
       i += static_cast<int64_t>(gridDim.x) * kStateThreads) {
    float acc = T[ts + i];
    for (int s = 2; s < G; ++s) {
      acc += T[s * ts + i];
      T[s * ts + i] = acc;
    }
  }
}
unsigned state_blocks(int64_t nf) {
  return static_cast<unsigned>(std::min<int64_t>((nf + kStateThreads - 1) / kStateThreads, 4096));
}
}  // namespace

hipError_t launch_state_copy(float* dst, const float* src, int64_t nf, hipStream_t s) {
  state_copy<<<state_blocks(nf), kStateThreads, 0, s>>>(dst, src, nf);
  return hipGetLastError();
}
hipError_t launch_state_zero(float* T, int64_t ts, int count, int64_t nf, hipStream_t s) {
  state_zero<<<dim3(state_blocks(nf), count), kStateThreads, 0, s>>>(T, ts, nf);
  return hipGetLastError();
}
hipError_t launch_state_prefix(float* T, int64_t ts, int G, int64_t nf, hipStream_t s) {
  state_prefix<<<state_blocks(nf), kStateThreads, 0, s>>>(T, ts, G, nf);
  return hipGetLastError();
}

hipError_t launch_prefill_b16(int d, int BH, const ScanArgs& a, hipStream_t s) {
  switch (d) {
    case 8: return launch_b16_t<8>(BH, a, s);
    case 16: return launch_b16_t<16>(BH, a, s);
    case 32: return launch_b16_t<32>(BH, a, s);
    case 64: return launch_b16_t<64>(BH, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_reduce_b16(int d, int BH, const ReduceArgs& a, hipStream_t s) {
  switch (d) {
    case 8: return launch_reduce_b16_t<8>(BH, a, s);
    case 16: return launch_reduce_b16_t<16>(BH, a, s);
    case 32: return launch_reduce_b16_t<32>(BH, a, s);
    case 64: return launch_reduce_b16_t<64>(BH, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sata
