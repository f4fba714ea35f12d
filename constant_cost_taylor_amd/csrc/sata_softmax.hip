// Exact causal softmax attention on gfx950: the baseline SATA is measured
// against.  out_i = sum_{j<=i} exp(q_i.k_j/c) v_j / sum_{j<=i} exp(q_i.k_j/c),
// computed stably (running maximum) as in the MoA page's section "DNF
// derivation"; its per-token cost grows with the position, n (2 d_k + 2 d_v + 3)
// FLOPs at position n (SATA page, "Scale bottleneck of conventional
// self-attention"), which is what SATA's fixed-size state avoids.
//
// bfloat16 inputs: softmax_mfma.  Block = (256 queries, head), four waves of 64
// queries; key tiles of 64 keys are staged in LDS (K row-major, V'^T with a
// ones row at column d_v, so the MFMA that forms sum_j p_j v_j also forms
// sum_j p_j).  Per 32-key slice and wave:
//   X^T = K_s Q^T                      (bf16 MFMA, fp32 accumulate)
//   m'  = max(m, max_j x_j / c) per query; O *= exp(m - m')
//   p_j = exp(x_j / c - m'), zero for keys after the query
//   O^T += V'^T_s p_hi + V'^T_s p_lo    (p = p_hi + p_lo, two bf16 parts:
//                                         about 2^-17 relative)
// float32 inputs: softmax_f32, one query per thread in fp32 arithmetic (the
// reference-precision path; key tiles of 64 staged in LDS).
#include <hip/hip_runtime.h>

#include "sata_internal.h"

namespace sata {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2(float x, float y) {
  bf16x2 v = {static_cast<__bf16>(x), static_cast<__bf16>(y)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float lo16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

constexpr int kQB = 256;   // queries per block (four waves of 64)
constexpr int kKT = 64;    // keys per staged tile

template <int DK>
__global__ __launch_bounds__(kQB) void softmax_mfma(SoftmaxArgs a) {
  constexpr int DV = DK;
  constexpr int KP = DK < 32 ? 32 : DK;        // head dim padded to the MFMA K
  constexpr int KSTEPS = KP / 32;
  constexpr int KSTR = KP + 8;                 // bf16 per staged key row
  constexpr int NB = col_blocks(DV), NC = NB * 16;
  constexpr int VSTR = kKT + 8;                // bf16 per staged V' row
  __shared__ __attribute__((aligned(16))) uint16_t ks_[kKT * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t vt[NC * VSTR];
  const int qblk = blockIdx.x;
  const int head = blockIdx.y;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int lr = l & 15;
  const int g = l >> 4;
  const int64_t n = a.n;
  const int64_t q0 = static_cast<int64_t>(qblk) * kQB + 64 * w;   // first query of this wave
  const uint16_t* qh = static_cast<const uint16_t*>(a.q) + static_cast<int64_t>(head) * n * DK;
  const uint16_t* kh = static_cast<const uint16_t*>(a.k) + static_cast<int64_t>(head) * n * DK;
  const uint16_t* vh = static_cast<const uint16_t*>(a.v) + static_cast<int64_t>(head) * n * DV;

  // Query operands (B of X^T): lane holds query q0 + 16 qb + lr, dims 32 kst + 8 g ..
  bf16x8 qop[4][KSTEPS];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb)
#pragma unroll
    for (int kst = 0; kst < KSTEPS; ++kst) {
      const int64_t qi = q0 + 16 * qb + lr;
      const int d0 = 32 * kst + 8 * g;
      const bool ok = qi < n && d0 < DK;
      u32x4 val = *reinterpret_cast<const u32x4*>(qh + (ok ? qi : 0) * DK + (ok ? d0 : 0));
      if (!ok) val = u32x4{0u, 0u, 0u, 0u};
      qop[qb][kst] = __builtin_bit_cast(bf16x8, val);
    }

  f32x4 O[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) O[nb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};   // running max of x / c per query

  // keys [0, kend) matter for this block; this wave needs keys <= its last query
  const int64_t kend = min(n, static_cast<int64_t>(qblk + 1) * kQB);
  const int64_t wend = min(n, q0 + 64);
  const int ntile = static_cast<int>((kend + kKT - 1) / kKT);
  constexpr int KI = kKT * (KP / 8) / kQB, VI = kKT * (DV / 8) / kQB;
  for (int tile = 0; tile < ntile; ++tile) {
    const int64_t kb = static_cast<int64_t>(tile) * kKT;
    __syncthreads();   // the previous tile's LDS reads are done
    // stage K (zero past n / past DK) and V'^T (ones row at DV)
    for (int e = tid; e < kKT * (KP / 8); e += kQB) {
      const int t = e / (KP / 8), c8 = (e % (KP / 8)) * 8;
      const bool ok = kb + t < n && c8 < DK;
      u32x4 val = *reinterpret_cast<const u32x4*>(kh + (ok ? kb + t : 0) * DK + (ok ? c8 : 0));
      if (!ok) val = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(&ks_[t * KSTR + c8]) = val;
    }
    for (int e = tid; e < kKT * (DV / 8); e += kQB) {
      const int t = e % kKT, c8 = (e / kKT) * 8;
      const bool ok = kb + t < n;
      u32x4 val = *reinterpret_cast<const u32x4*>(vh + (ok ? kb + t : 0) * DV + c8);
      if (!ok) val = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 8; ++j)
        vt[(c8 + j) * VSTR + t] = static_cast<uint16_t>((j & 1) ? (val[j / 2] >> 16) : (val[j / 2] & 0xffffu));
    }
    for (int e = tid; e < (NC - DV) * kKT; e += kQB) {
      const int c = DV + e / kKT;
      const int t = e % kKT;
      vt[c * VSTR + t] = (c == DV && kb + t < n) ? static_cast<uint16_t>(0x3f80) : static_cast<uint16_t>(0);
    }
    (void)KI;
    (void)VI;
    __syncthreads();
    if (kb >= wend) continue;   // every key of the tile is after this wave's queries
#pragma unroll
    for (int sl = 0; sl < kKT / 32; ++sl) {
      const int64_t ks0 = kb + 32 * sl;
      if (ks0 >= wend) break;
      f32x4 X[2][4];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) X[kk][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kst = 0; kst < KSTEPS; ++kst)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const bf16x8 A = *reinterpret_cast<const bf16x8*>(&ks_[(32 * sl + 16 * kk + lr) * KSTR + 32 * kst + 8 * g]);
#pragma unroll
          for (int qb = 0; qb < 4; ++qb)
            X[kk][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, qop[qb][kst], X[kk][qb], 0, 0, 0);
        }
      // lane holds query q0 + 16 qb + lr and keys ks0 + 16 (j / 4) + 4 g + j % 4
      bf16x8 Bh[4], Bl[4];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const int64_t qi = q0 + 16 * qb + lr;
        float x[8];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int64_t key = ks0 + 16 * (j / 4) + 4 * g + (j % 4);
          x[j] = key <= qi && key < n ? X[j / 4][qb][j % 4] * a.inv_c : -INFINITY;
          mx = fmaxf(mx, x[j]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(m[qb], mx);
        // rescale the running sums when the maximum grows (a query with no
        // key yet keeps m = -inf and O = 0)
        const float alpha = mn == -INFINITY ? 1.f : __expf(m[qb] - mn);
        if (alpha != 1.f) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) O[nb][qb] *= alpha;
        }
        m[qb] = mn;
        float p[8], r[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = x[j] == -INFINITY ? 0.f : __expf(x[j] - mn);
        const u32x4 ph = {pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7])};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t w2 = ph[j / 2];
          r[j] = p[j] - ((j & 1) ? hi16(w2) : lo16(w2));
        }
        const u32x4 pl = {pack2(r[0], r[1]), pack2(r[2], r[3]), pack2(r[4], r[5]), pack2(r[6], r[7])};
        Bh[qb] = __builtin_bit_cast(bf16x8, ph);
        Bl[qb] = __builtin_bit_cast(bf16x8, pl);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint16_t* vr = &vt[(16 * nb + lr) * VSTR + 32 * sl + 4 * g];
        const u32x2 lo = *reinterpret_cast<const u32x2*>(__builtin_assume_aligned(vr, 8));
        const u32x2 hi = *reinterpret_cast<const u32x2*>(__builtin_assume_aligned(vr + 16, 8));
        const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
        const bf16x8 A = __builtin_bit_cast(bf16x8, av);
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
          O[nb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bh[qb], O[nb][qb], 0, 0, 0);
          O[nb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bl[qb], O[nb][qb], 0, 0, 0);
        }
      }
    }
  }
  // O^T in C layout: lane holds query q0 + 16 qb + lr, columns 16 nb + 4 g + r;
  // the den column DV sits in block DV / 16, lane group (DV % 16) / 4, element DV % 4.
  constexpr int NBD = DV / 16, GD = (DV % 16) / 4, RD = DV % 4;
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const int64_t qi = q0 + 16 * qb + lr;
    const float den = __shfl(O[NBD][qb][RD], lr + 16 * GD);   // lane (lr, GD) holds it
    if (qi >= n) continue;
    float* out = a.out + (static_cast<int64_t>(head) * n + qi) * DV;
    const float inv = 1.f / den;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = 16 * nb + 4 * g;
      if (col + 4 <= DV) *reinterpret_cast<f32x4*>(&out[col]) = O[nb][qb] * inv;
    }
  }
}

// float32 inputs: thread = query, fp32 arithmetic throughout.
template <int DK>
__global__ __launch_bounds__(128) void softmax_f32(SoftmaxArgs a) {
  constexpr int DV = DK;
  constexpr int KT = 32;
  __shared__ float sk[KT][DK];
  __shared__ float sv[KT][DV];
  const int head = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t n = a.n;
  const int64_t qi = static_cast<int64_t>(blockIdx.x) * 128 + tid;
  const float* qh = static_cast<const float*>(a.q) + static_cast<int64_t>(head) * n * DK;
  const float* kh = static_cast<const float*>(a.k) + static_cast<int64_t>(head) * n * DK;
  const float* vh = static_cast<const float*>(a.v) + static_cast<int64_t>(head) * n * DV;
  float q[DK], o[DV];
#pragma unroll
  for (int d = 0; d < DK; ++d) q[d] = qi < n ? qh[qi * DK + d] * a.inv_c : 0.f;
#pragma unroll
  for (int d = 0; d < DV; ++d) o[d] = 0.f;
  float m = -INFINITY, den = 0.f;
  const int64_t kend = min(n, static_cast<int64_t>(blockIdx.x + 1) * 128);
  for (int64_t kb = 0; kb < kend; kb += KT) {
    __syncthreads();
    for (int e = tid; e < KT * DK; e += 128) {
      const int t = e / DK, d = e % DK;
      sk[t][d] = kb + t < n ? kh[(kb + t) * DK + d] : 0.f;
      sv[t][d] = kb + t < n ? vh[(kb + t) * DV + d] : 0.f;
    }
    __syncthreads();
    if (qi >= n || kb > qi) continue;
    float x[KT];
    float mx = m;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < DK; ++d) s = fmaf(q[d], sk[t][d], s);
      x[t] = kb + t <= qi ? s : -INFINITY;
      mx = fmaxf(mx, x[t]);
    }
    const float alpha = m == -INFINITY ? 0.f : expf(m - mx);
    den *= alpha;
#pragma unroll
    for (int d = 0; d < DV; ++d) o[d] *= alpha;
    m = mx;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const float p = x[t] == -INFINITY ? 0.f : expf(x[t] - mx);
      den += p;
#pragma unroll
      for (int d = 0; d < DV; ++d) o[d] = fmaf(p, sv[t][d], o[d]);
    }
  }
  if (qi < n) {
    float* out = a.out + (static_cast<int64_t>(head) * n + qi) * DV;
#pragma unroll
    for (int d = 0; d < DV; ++d) out[d] = o[d] / den;
  }
}

template <int D>
hipError_t launch_softmax_t(bool bf16, int BH, const SoftmaxArgs& a, hipStream_t s) {
  if (bf16)
    softmax_mfma<D><<<dim3(static_cast<unsigned>((a.n + kQB - 1) / kQB), BH), kQB, 0, s>>>(a);
  else
    softmax_f32<D><<<dim3(static_cast<unsigned>((a.n + 127) / 128), BH), 128, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_softmax(int d, bool bf16, int BH, const SoftmaxArgs& a, hipStream_t s) {
  switch (d) {
    case 8: return launch_softmax_t<8>(bf16, BH, a, s);
    case 16: return launch_softmax_t<16>(bf16, BH, a, s);
    case 32: return launch_softmax_t<32>(bf16, BH, a, s);
    case 64: return launch_softmax_t<64>(bf16, BH, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sata
