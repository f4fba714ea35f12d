// Chunked causal prefill of SATA on gfx950 (CDNA4).
//
// The sequence is cut into chunks of kChunk tokens.  For a query i in chunk t
//   num_i = sum_{j <= i, j in t} T_P(x_ij) v_j            (intra-chunk, exact polynomial)
//         + sum_m w_m phi_m(q_i) S_m(<t)                  (inter-chunk, through the state)
// and likewise for den with v replaced by 1.  The state S(<t) holds every
// key before chunk t [SATA page, section "Engineering of constant compute
// cost": the fixed-size state accumulates phi(k) v over the processed
// tokens, one scan per Taylor order].
//
// Kernels:
//   prefill_scan   grid = (row tiles) x (heads).  A workgroup owns a tile of
//                  basis rows of order >= 1 and keeps its fp32 state slice in
//                  MFMA accumulators for the whole window.  Per chunk it builds
//                  the query and key features of its rows from LDS-staged q/k
//                  (each row = parent feature x one more coordinate, the
//                  nested i1 <= ... <= ip structure of the index matrices),
//                  reads out  phi_q(Q_t) S  and updates  S += phi_k(K_t)^T [V_t 1]
//                  on MFMA (bf16 operands for bf16 inputs, fp32 otherwise).
//                  The order-0 row (the running sum of v and the token count)
//                  is carried exactly in fp32 by tile 0.
//   prefill_intra  grid = (chunks) x (heads): the intra-chunk part, fp32.
//   prefill_reduce sums the per-tile readout records in a fixed order and divides.
//
// Internal row order.  The rows of a tile are grouped in runs of four
// children (P, c0..c0+3) of one parent multiset P (c0 a multiple of 4,
// children below max(P) masked).  Inside the scan the state of row
// m = P + {c} is kept divided by cnt_c(m), the multiplicity of c in m; the
// query features then factor as [w(P) prod_{i in P} q_i/c] * q_c/c, with w(P)
// = 1/prod(count!) of the parent, and the key features as
// [prod_{i in P} k_i] * k_c/cnt_c(m).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "sata_internal.h"

namespace sata {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Two floats rounded to bf16 (nearest even) and packed in one register.  The
// empty asm pins the conversion at this point of the program, so the
// compiler cannot defer it and keep the fp32 inputs alive instead.
__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
  bf16x2 v = {static_cast<__bf16>(x), static_cast<__bf16>(y)};
  uint32_t r = __builtin_bit_cast(uint32_t, v);
  asm volatile("" : "+v"(r));
  return r;
}

// 16-byte LDS load at an offset the caller guarantees to be a multiple of 4 floats.
__device__ __forceinline__ float4 lds4(const float* base, int off) {
  return *reinterpret_cast<const float4*>(__builtin_assume_aligned(base + off, 16));
}

__device__ __forceinline__ float load_in(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_in(const uint16_t* p, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

// One thread's share of a chunk of q, k or v: EPT consecutive elements of one
// token, fetched with 16-byte (or narrower) vector loads.
template <typename IT, int EPT>
struct ChunkRegs {
  static constexpr int kBytes = EPT * static_cast<int>(sizeof(IT));
  static constexpr int kVec = kBytes < 16 ? kBytes : 16;   // bytes per load
  static constexpr int kLoads = kBytes / kVec;
  struct alignas(kVec) Piece {
    unsigned char b[kVec];
  };
  Piece p[kLoads];
  __device__ __forceinline__ void load(const IT* src, bool valid) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      if (valid) {
        p[j] = reinterpret_cast<const Piece*>(src)[j];
      } else {
#pragma unroll
        for (int x = 0; x < kVec; ++x) p[j].b[x] = 0;
      }
    }
  }
  __device__ __forceinline__ IT raw(int e) const {
    IT v;
    __builtin_memcpy(&v, reinterpret_cast<const unsigned char*>(p) + e * sizeof(IT), sizeof(IT));
    return v;
  }
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }

template <int DK, bool BF16, int RB>
struct ScanShape {
  static constexpr int DV = DK;
  static constexpr int L = kChunk;
  static constexpr int NB = col_blocks(DV);     // 16-wide column blocks incl. z
  static constexpr int NC = NB * 16;
  static constexpr int DVP = padded_dv(DV);
  static constexpr int NSLOT = 4 * RB * kWaves;  // bound on distinct parents per tile
  static constexpr int KSTR = kKStride;          // xk / pk row stride (floats)
  static constexpr int QSTR = L + 1;             // pq row stride
  static constexpr int XQSTR = DK + 4;           // xq row stride
  static constexpr int RSTR = NC + 4;            // readout reduction row stride
  static constexpr int VSTR = L + 8;             // bf16 V' row stride (elements)
  static constexpr int XK_ZERO = 3 * DK * KSTR;  // dword offset of the zero row
  static constexpr int NKS = (RB + 1) / 2;       // bf16 readout K-slices (2 blocks each)
};

template <int DK, bool BF16, int RB>
__global__ __launch_bounds__(kWaves * 64, 1) void prefill_scan(ScanArgs a) {
  using Sh = ScanShape<DK, BF16, RB>;
  constexpr int DV = Sh::DV, L = Sh::L, NB = Sh::NB, NC = Sh::NC, DVP = Sh::DVP;
  constexpr int NSLOT = Sh::NSLOT, KSTR = Sh::KSTR, QSTR = Sh::QSTR, XQSTR = Sh::XQSTR;
  constexpr int RSTR = Sh::RSTR, VSTR = Sh::VSTR, XK_ZERO = Sh::XK_ZERO;
  using IT = typename std::conditional<BF16, uint16_t, float>::type;

  __shared__ __attribute__((aligned(16))) float xk[(3 * DK + 1) * KSTR];
  __shared__ __attribute__((aligned(16))) float pk[NSLOT * KSTR];
  __shared__ __attribute__((aligned(16))) float pq[NSLOT * QSTR];
  __shared__ __attribute__((aligned(16))) float xq[L * XQSTR];
  __shared__ __attribute__((aligned(16))) float red[kWaves * L * RSTR];
  __shared__ __attribute__((aligned(16))) uint16_t vt[BF16 ? NC * VSTR : 8];
  __shared__ __attribute__((aligned(16))) float vv[BF16 ? 4 : L * NC];
  __shared__ float carry[NC];
  __shared__ uint32_t spar[NSLOT];
  __shared__ float spw[NSLOT];

  const int tile = blockIdx.x;
  const int head = blockIdx.y;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int lr = l & 15;
  const int g = l >> 4;
  const int n_tiles = a.lay.n_tiles;
  const int lay_base = (tile * kWaves + w) * RB;

  // Per-lane run metadata (fixed for the whole window).
  uint32_t ks[RB], qs[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    ks[b] = a.lay.kside[(lay_base + b) * 16 + lr];
    qs[b] = a.lay.qside[(lay_base + b) * 4 + g];
  }
  const int nslot = a.lay.nslot[tile];
  for (int s = tid; s < nslot; s += kWaves * 64) {
    spar[s] = a.lay.parents[tile * NSLOT + s];
    spw[s] = a.lay.pweight[tile * NSLOT + s];
  }
  for (int i = tid; i < KSTR; i += kWaves * 64) xk[XK_ZERO + i] = 0.f;
  if constexpr (BF16) {
    // Constant columns of V' = [v, 1, 0...]: the ones column feeds z.
    for (int e = tid; e < (NC - DV) * VSTR; e += kWaves * 64) {
      const int c = DV + e / VSTR;
      vt[c * VSTR + e % VSTR] = (c == DV) ? static_cast<uint16_t>(0x3f80) : static_cast<uint16_t>(0);
    }
  } else {
    for (int e = tid; e < L * (NC - DV); e += kWaves * 64) {
      const int t = e / (NC - DV);
      const int c = DV + e % (NC - DV);
      vv[t * NC + c] = (c == DV) ? 1.f : 0.f;
    }
  }

  // Load the state tile into the accumulators (C layout: lane holds column
  // nb*16 + lr of rows 4g + r), divided by the multiplicity of each row's
  // last index.
  float* st = a.state + static_cast<int64_t>(head) * a.stride;
  const int64_t zoff = static_cast<int64_t>(a.D) * DV;
  f32x4 S[RB][NB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t info = a.lay.rowinfo[(lay_base + b) * 16 + 4 * g + r];
      const int64_t m = info ? static_cast<int64_t>(info & 0x0fffffffu) - 1 : 0;
      const float inv_cnt = info ? 1.f / static_cast<float>(info >> 28) : 0.f;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = nb * 16 + lr;
        float val = 0.f;
        if (col < DV) val = st[m * DV + col];
        else if (col == DV) val = st[zoff + m];
        S[b][nb][r] = val * inv_cnt;
      }
    }
    // Move the block into accumulator registers right away, so the whole
    // tile is never held in VGPRs at once.
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) asm volatile("" : "+a"(S[b][nb]));
    __builtin_amdgcn_sched_barrier(0);  // one row block of loads in flight at a time
  }
  // bf16 copy of the state used as the readout operand; refreshed right
  // after every update so the fp32 tile never has to leave the accumulators.
  uint32_t Sb[BF16 ? RB : 1][BF16 ? NB : 1][2];
  if constexpr (BF16) {
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        Sb[b][nb][0] = pack_bf16(S[b][nb][0], S[b][nb][1]);
        Sb[b][nb][1] = pack_bf16(S[b][nb][2], S[b][nb][3]);
      }
  }
  if (tile == 0 && tid < NC) carry[tid] = tid < DV ? st[tid] : (tid == DV ? st[zoff] : 0.f);

  const IT* qh = static_cast<const IT*>(a.q) + static_cast<int64_t>(head) * a.n_total * DK;
  const IT* kh = static_cast<const IT*>(a.k) + static_cast<int64_t>(head) * a.n_total * DK;
  const IT* vh = static_cast<const IT*>(a.v) + static_cast<int64_t>(head) * a.n_total * DV;
  float* parth = a.part + static_cast<int64_t>(head) * (n_tiles + 1) * a.nw * DVP +
                 static_cast<int64_t>(tile) * a.nw * DVP;

  // Each thread stages EPT consecutive elements of one token per tensor.
  constexpr int EPT = L * DK / (kWaves * 64);
  const int st_t = (tid * EPT) / DK;
  const int st_i = (tid * EPT) % DK;
  ChunkRegs<IT, EPT> rq, rk, rv;
  {
    const bool ok = st_t < min(L, a.nw);
    rq.load(qh + (a.t0 + st_t) * DK + st_i, ok);
    rk.load(kh + (a.t0 + st_t) * DK + st_i, ok);
    rv.load(vh + (a.t0 + st_t) * DV + st_i, ok);
  }

  const int nch = (a.nw + L - 1) / L;
  for (int ch = 0; ch < nch; ++ch) {
    const int64_t tb = a.t0 + static_cast<int64_t>(ch) * L;
    const int nvalid = min(L, a.nw - ch * L);
    // Launder the run metadata so the LDS addresses derived from it are
    // recomputed each chunk (a few integer ops) instead of held live.
#pragma unroll
    for (int b = 0; b < RB; ++b) asm volatile("" : "+v"(ks[b]), "+v"(qs[b]));
    __syncthreads();  // previous chunk is done with every LDS buffer

    // Stage the chunk from the registers prefetched during the previous
    // chunk: xq[t][i] = q/c, xk[code][i][t] = k/code, V' columns.
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const float qv = to_f32(rq.raw(e)) * a.inv_c;
      const float kv = to_f32(rk.raw(e));
      xq[st_t * XQSTR + st_i + e] = qv;
      xk[(st_i + e) * KSTR + st_t] = kv;
      xk[(DK + st_i + e) * KSTR + st_t] = kv * 0.5f;
      xk[(2 * DK + st_i + e) * KSTR + st_t] = kv * (1.f / 3.f);
      if constexpr (BF16)
        vt[(st_i + e) * VSTR + st_t] = rv.raw(e);
      else
        vv[st_t * NC + st_i + e] = rv.raw(e);
    }
    // Prefetch the next chunk; the loads stay in flight through this chunk.
    if (ch + 1 < nch) {
      const int64_t tn = tb + L + st_t;
      const bool ok = st_t < min(L, a.nw - (ch + 1) * L);
      rq.load(qh + tn * DK + st_i, ok);
      rk.load(kh + tn * DK + st_i, ok);
      rv.load(vh + tn * DV + st_i, ok);
    }
    __syncthreads();

    // Parent features of the tile's distinct parents (order <= 2).
    for (int e = tid; e < nslot * L; e += kWaves * 64) {
      const int s = e / L;
      const int t = e % L;
      const uint32_t pw = spar[s];
      const int np = (pw >> 16) & 3;
      const int i1 = pw & 255;
      const int i2 = (pw >> 8) & 255;
      float fk = 1.f, fq = spw[s];
      if (np >= 1) {
        fk *= xk[i1 * KSTR + t];
        fq *= xq[t * XQSTR + i1];
      }
      if (np >= 2) {
        fk *= xk[i2 * KSTR + t];
        fq *= xq[t * XQSTR + i2];
      }
      pk[s * KSTR + t] = fk;
      pq[s * QSTR + t] = fq;
    }
    __syncthreads();

    // Readout against the state before this chunk: acc[mb] = phi_q(Q) S.
    f32x4 acc[L / 16][NB];
#pragma unroll
    for (int mb = 0; mb < L / 16; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    if constexpr (BF16) {
#pragma unroll
      for (int kk = 0; kk < Sh::NKS; ++kk) {
        const int b0 = 2 * kk;
        const int b1 = (2 * kk + 1 < RB) ? 2 * kk + 1 : 2 * kk;
        const bool has1 = 2 * kk + 1 < RB;
        // Query features of both token blocks for this K-slice (8 rows per lane).
        bf16x8 A[L / 16];
        const int slot0 = qs[b0] & 0xffff;
        const int c00 = qs[b0] >> 16;
        const int slot1 = qs[b1] & 0xffff;
        const int c01 = qs[b1] >> 16;
#pragma unroll
        for (int mb = 0; mb < L / 16; ++mb) {
          const int t = mb * 16 + lr;
          const float p0 = pq[slot0 * QSTR + t];
          const float4 x0 = lds4(xq, t * XQSTR + c00);
          float p1 = 0.f;
          float4 x1 = make_float4(0.f, 0.f, 0.f, 0.f);
          if (has1) {
            p1 = pq[slot1 * QSTR + t];
            x1 = lds4(xq, t * XQSTR + c01);
          }
          A[mb][0] = static_cast<__bf16>(p0 * x0.x);
          A[mb][1] = static_cast<__bf16>(p0 * x0.y);
          A[mb][2] = static_cast<__bf16>(p0 * x0.z);
          A[mb][3] = static_cast<__bf16>(p0 * x0.w);
          A[mb][4] = static_cast<__bf16>(p1 * x1.x);
          A[mb][5] = static_cast<__bf16>(p1 * x1.y);
          A[mb][6] = static_cast<__bf16>(p1 * x1.z);
          A[mb][7] = static_cast<__bf16>(p1 * x1.w);
        }
        // State rows of the K-slice as the bf16 B operand, one column block at a time.
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const u32x4 bw = {Sb[b0][nb][0], Sb[b0][nb][1], has1 ? Sb[b1][nb][0] : 0u,
                            has1 ? Sb[b1][nb][1] : 0u};
          const bf16x8 Bop = __builtin_bit_cast(bf16x8, bw);
#pragma unroll
          for (int mb = 0; mb < L / 16; ++mb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mb], Bop, acc[mb][nb], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const int slot = qs[b] & 0xffff;
        const int c0 = qs[b] >> 16;
#pragma unroll
        for (int mb = 0; mb < L / 16; ++mb) {
          const int t = mb * 16 + lr;
          const float p = pq[slot * QSTR + t];
          const float4 x = lds4(xq, t * XQSTR + c0);
          const float av[4] = {p * x.x, p * x.y, p * x.z, p * x.w};
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[r], S[b][nb][r], acc[mb][nb], 0, 0, 0);
        }
      }
    }

    // Sum the waves' readouts (fixed order) and write this tile's records.
#pragma unroll
    for (int mb = 0; mb < L / 16; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          red[(w * L + mb * 16 + 4 * g + r) * RSTR + nb * 16 + lr] = acc[mb][nb][r];
    __syncthreads();
    for (int e = tid; e < nvalid * (DV + 1); e += kWaves * 64) {
      const int t = e / (DV + 1);
      const int c = e % (DV + 1);
      float sum = red[t * RSTR + c];
#pragma unroll
      for (int ww = 1; ww < kWaves; ++ww) sum += red[(ww * L + t) * RSTR + c];
      if (tile == 0) sum += carry[c];
      parth[static_cast<int64_t>(ch * L + t) * DVP + c] = sum;
    }
    if (tile == 0) {
      __syncthreads();  // carry was read above
      if (tid < DV) {
        float s = 0.f;
        for (int t = 0; t < nvalid; ++t) {
          if constexpr (BF16)
            s += __uint_as_float(static_cast<uint32_t>(vt[tid * VSTR + t]) << 16);
          else
            s += vv[t * NC + tid];
        }
        carry[tid] += s;
      } else if (tid == DV) {
        carry[DV] += static_cast<float>(nvalid);
      }
    }

    // State update: S += phi_k(K)^T [V 1] for every row block.  Software
    // pipelined per row block (LDS loads of block b+1 in flight while block b
    // runs on MFMA) with scheduling fences, so only a couple of blocks'
    // temporaries are live.
    if constexpr (BF16) {
      bf16x8 Bv[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        Bv[nb] = *reinterpret_cast<const bf16x8*>(&vt[(nb * 16 + lr) * VSTR + 8 * g]);
      float4 cp0, cp1, cx0, cx1;
      {
        const int pko = ks[0] & 0xffff;
        const int xko = ks[0] >> 16;
        cp0 = lds4(pk, pko + 8 * g);
        cp1 = lds4(pk, pko + 8 * g + 4);
        cx0 = lds4(xk, xko + 8 * g);
        cx1 = lds4(xk, xko + 8 * g + 4);
      }
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        float4 np0, np1, nx0, nx1;
        if (b + 1 < RB) {
          const int pko = ks[b + 1 < RB ? b + 1 : b] & 0xffff;
          const int xko = ks[b + 1 < RB ? b + 1 : b] >> 16;
          np0 = lds4(pk, pko + 8 * g);
          np1 = lds4(pk, pko + 8 * g + 4);
          nx0 = lds4(xk, xko + 8 * g);
          nx1 = lds4(xk, xko + 8 * g + 4);
        }
        const u32x4 aw = {pack_bf16(cp0.x * cx0.x, cp0.y * cx0.y), pack_bf16(cp0.z * cx0.z, cp0.w * cx0.w),
                          pack_bf16(cp1.x * cx1.x, cp1.y * cx1.y), pack_bf16(cp1.z * cx1.z, cp1.w * cx1.w)};
        const bf16x8 A = __builtin_bit_cast(bf16x8, aw);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          S[b][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bv[nb], S[b][nb], 0, 0, 0);
        if (b > 0) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const int bp = b > 0 ? b - 1 : 0;
            Sb[bp][nb][0] = pack_bf16(S[bp][nb][0], S[bp][nb][1]);
            Sb[bp][nb][1] = pack_bf16(S[bp][nb][2], S[bp][nb][3]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (b + 1 < RB) {
          cp0 = np0;
          cp1 = np1;
          cx0 = nx0;
          cx1 = nx1;
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        Sb[RB - 1][nb][0] = pack_bf16(S[RB - 1][nb][0], S[RB - 1][nb][1]);
        Sb[RB - 1][nb][1] = pack_bf16(S[RB - 1][nb][2], S[RB - 1][nb][3]);
      }
    } else {
#pragma unroll
      for (int kst = 0; kst < L / 4; ++kst) {
        const int t = 4 * kst + g;
        float bv[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) bv[nb] = vv[t * NC + nb * 16 + lr];
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const int pko = ks[b] & 0xffff;
          const int xko = ks[b] >> 16;
          const float av = pk[pko + t] * xk[xko + t];
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            S[b][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv[nb], S[b][nb], 0, 0, 0);
        }
      }
    }
  }

  // Write the state tile back in canonical layout.  The row table pointer is
  // laundered so the addresses are recomputed here instead of being kept live
  // (in registers) from the initial load across the whole chunk loop.
  const uint32_t* rowinfo = a.lay.rowinfo;
  float* stw = st;
  asm volatile("" : "+s"(rowinfo), "+s"(stw));
#pragma unroll
  for (int b = 0; b < RB; ++b) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t info = rowinfo[(lay_base + b) * 16 + 4 * g + r];
      if (info) {
        const int64_t m = static_cast<int64_t>(info & 0x0fffffffu) - 1;
        const float cnt = static_cast<float>(info >> 28);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int col = nb * 16 + lr;
          const float val = S[b][nb][r] * cnt;
          if (col < DV) stw[m * DV + col] = val;
          else if (col == DV) stw[zoff + m] = val;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (tile == 0) {
    __syncthreads();
    if (tid < DV) st[tid] = carry[tid];
    else if (tid == DV) st[zoff] = carry[DV];
  }
}

// Intra-chunk part: for each token i of a chunk, sum over the chunk's tokens
// j <= i of T_P(q_i.k_j/c) (v_j, 1), in fp32 with Horner's rule.
template <int DK, typename IT>
__global__ __launch_bounds__(256) void prefill_intra(IntraArgs a) {
  constexpr int DV = DK, L = kChunk, DVP = padded_dv(DV);
  constexpr int TPT = 256 / L;                 // threads per token
  constexpr int CPT = (DV + TPT - 1) / TPT;    // columns per thread
  __shared__ float sq[L][DK + 1];
  __shared__ float sk[L][DK + 1];
  __shared__ float sv[L][DV + 1];
  const int ch = blockIdx.x;
  const int head = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t tb = a.t0 + static_cast<int64_t>(ch) * L;
  const int nvalid = min(L, a.nw - ch * L);
  const IT* qh = static_cast<const IT*>(a.q) + static_cast<int64_t>(head) * a.n_total * DK;
  const IT* kh = static_cast<const IT*>(a.k) + static_cast<int64_t>(head) * a.n_total * DK;
  const IT* vh = static_cast<const IT*>(a.v) + static_cast<int64_t>(head) * a.n_total * DV;
  for (int e = tid; e < L * DK; e += 256) {
    const int t = e / DK, i = e % DK;
    sq[t][i] = t < nvalid ? load_in(qh, (tb + t) * DK + i) * a.inv_c : 0.f;
    sk[t][i] = t < nvalid ? load_in(kh, (tb + t) * DK + i) : 0.f;
  }
  for (int e = tid; e < L * DV; e += 256) {
    const int t = e / DV, c = e % DV;
    sv[t][c] = t < nvalid ? load_in(vh, (tb + t) * DV + c) : 0.f;
  }
  __syncthreads();
  const int i = tid / TPT;
  const int sub = tid % TPT;
  if (i >= nvalid) return;
  float rcp[4] = {0.f, 1.f, 0.5f, 1.f / 3.f};
  float num[CPT];
#pragma unroll
  for (int cc = 0; cc < CPT; ++cc) num[cc] = 0.f;
  float den = 0.f;
  for (int j = 0; j <= i; ++j) {
    float x = 0.f;
#pragma unroll
    for (int d = 0; d < DK; ++d) x = fmaf(sq[i][d], sk[j][d], x);
    float wgt = 1.f;
    for (int p = a.P - 1; p >= 1; --p) wgt = fmaf(wgt, x * rcp[p], 1.f);
    den += wgt;
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) {
      const int c = sub + TPT * cc;
      if (c < DV) num[cc] = fmaf(wgt, sv[j][c], num[cc]);
    }
  }
  float* rec = a.part + ((static_cast<int64_t>(head) * (a.n_tiles + 1) + a.n_tiles) * a.nw +
                         static_cast<int64_t>(ch) * L + i) * DVP;
#pragma unroll
  for (int cc = 0; cc < CPT; ++cc) {
    const int c = sub + TPT * cc;
    if (c < DV) rec[c] = num[cc];
  }
  if (sub == 0) rec[DV] = den;
}

// out = (sum over records of num) / (sum over records of den), fixed order.
template <int DV>
__global__ __launch_bounds__(256) void prefill_reduce(ReduceArgs a) {
  constexpr int DVP = padded_dv(DV);
  constexpr int TB = 64;
  __shared__ __attribute__((aligned(16))) float acc[TB * DVP];
  const int head = blockIdx.y;
  const int t0 = blockIdx.x * TB;
  const int ntok = min(TB, a.nw - t0);
  const int tid = threadIdx.x;
  const int n4 = ntok * DVP / 4;
  const float4* base = reinterpret_cast<const float4*>(a.part) +
                       (static_cast<int64_t>(head) * a.nslots * a.nw + t0) * (DVP / 4);
  const int64_t sstride = static_cast<int64_t>(a.nw) * (DVP / 4);
  for (int e = tid; e < n4; e += 256) {
    float4 s = base[e];
    for (int sl = 1; sl < a.nslots; ++sl) {
      const float4 x = base[sl * sstride + e];
      s.x += x.x;
      s.y += x.y;
      s.z += x.z;
      s.w += x.w;
    }
    reinterpret_cast<float4*>(acc)[e] = s;
  }
  __syncthreads();
  float* out = a.out + (static_cast<int64_t>(head) * a.n_total + a.t0 + t0) * DV;
  for (int e = tid; e < ntok * DV; e += 256) {
    const int t = e / DV, c = e % DV;
    out[static_cast<int64_t>(t) * DV + c] = acc[t * DVP + c] / acc[t * DVP + DV];
  }
}

template <int D, bool BF16>
hipError_t launch_scan_t(int BH, const ScanArgs& a, hipStream_t s) {
  constexpr int RB = prefill_rb(D, BF16);
  dim3 grid(a.lay.n_tiles, BH);
  prefill_scan<D, BF16, RB><<<grid, kWaves * 64, 0, s>>>(a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_intra_t(bool bf16, int BH, const IntraArgs& a, hipStream_t s) {
  dim3 grid((a.nw + kChunk - 1) / kChunk, BH);
  if (bf16)
    prefill_intra<D, uint16_t><<<grid, 256, 0, s>>>(a);
  else
    prefill_intra<D, float><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_scan(int d, bool bf16, int BH, const ScanArgs& a, hipStream_t s) {
  switch (d) {
    case 8: return bf16 ? launch_scan_t<8, true>(BH, a, s) : launch_scan_t<8, false>(BH, a, s);
    case 16: return bf16 ? launch_scan_t<16, true>(BH, a, s) : launch_scan_t<16, false>(BH, a, s);
    case 32: return bf16 ? launch_scan_t<32, true>(BH, a, s) : launch_scan_t<32, false>(BH, a, s);
    case 64: return bf16 ? launch_scan_t<64, true>(BH, a, s) : launch_scan_t<64, false>(BH, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill_intra(int d, bool bf16, int BH, const IntraArgs& a, hipStream_t s) {
  switch (d) {
    case 8: return launch_intra_t<8>(bf16, BH, a, s);
    case 16: return launch_intra_t<16>(bf16, BH, a, s);
    case 32: return launch_intra_t<32>(bf16, BH, a, s);
    case 64: return launch_intra_t<64>(bf16, BH, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill_reduce(int d, int BH, const ReduceArgs& a, hipStream_t s) {
  dim3 grid((a.nw + 63) / 64, BH);
  switch (d) {
    case 8: prefill_reduce<8><<<grid, 256, 0, s>>>(a); break;
    case 16: prefill_reduce<16><<<grid, 256, 0, s>>>(a); break;
    case 32: prefill_reduce<32><<<grid, 256, 0, s>>>(a); break;
    case 64: prefill_reduce<64><<<grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sata
