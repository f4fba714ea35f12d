// Chunked causal prefill of SATA on gfx950 (CDNA4) for float32 inputs, and
// the intra-window kernel of the bfloat16 path (prefill_intra_mfma; the rest
// of that path is in sata_prefill_b16.hip).
//
// The sequence is cut into chunks of L tokens.  For a query i in chunk t
//   num_i = sum_{j <= i, j in t} T_P(x_ij) v_j            (intra-chunk, exact polynomial)
//         + sum_{j before t} v_j                          (order 0, carried exactly)
//         + sum_{m of order >= 1} w_m phi_m(q_i) S_m(<t)  (inter-chunk, through the state)
// and likewise for den with v replaced by 1.  S(<t) holds every key before
// chunk t [SATA page, section "Engineering of constant compute cost": the
// fixed-size state accumulates phi(k) v over the processed tokens, one scan
// per Taylor order].
//
// Kernels:
//   prefill_scan   grid = (row tiles) x (heads).  A workgroup owns a tile of
//                  basis rows of order >= 1 and keeps its fp32 state slice in
//                  MFMA accumulators for the whole window.  Per chunk it builds
//                  the query and key features of its rows from LDS-staged q/k
//                  (each row = parent feature x one more coordinate, the
//                  nested i1 <= ... <= ip structure of the index matrices),
//                  reads out  phi_q(Q_t) S  and updates  S += phi_k(K_t)^T [V_t 1]
//                  on fp32 MFMA, and writes one readout record per token.
//                  Where d_v is a multiple of 16, z and phi_q.z run on VALU
//                  (the den column would take an MFMA block of its own).
//                  Tile 0 also records the exact order-0 prefix of every chunk.
//   prefill_intra  grid = (chunks) x (heads): the intra-chunk part, fp32.
//   prefill_reduce sums the records in a fixed order and divides.
//
// Internal row order.  The rows of a tile are grouped in runs of four
// children (P, c0..c0+3) of one parent multiset P (c0 a multiple of 4,
// children below max(P) masked).  Inside the scan the state of row
// m = P + {c} is kept divided by cnt_c(m), the multiplicity of c in m; the
// query features then factor as [w(P) prod_{i in P} q_i/c] * q_c/c, with w(P)
// = 1/prod(count!) of the parent, and the key features as
// [prod_{i in P} k_i] * k_c/cnt_c(m) (the 1/3 of the (i, i, i) rows sits on a
// parent slot of its own).
//
// One chunk takes three barrier-separated phases:
//   A  cross-wave sum of the previous chunk's readout (writes its records)
//      and staging of this chunk from registers prefetched a chunk earlier;
//   B  parent features of the tile's parent slots (+ the order-0 carry);
//   C  readout into the LDS reduction buffer, then the state update.
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
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }

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
  bool ok;
  // The load is unconditional (src must be a valid address): a select on
  // the loaded value would make the wave wait for it here, turning the
  // prefetch into a synchronous load.  Invalid tokens are zeroed at use.
  __device__ __forceinline__ void load(const IT* src, bool valid) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) p[j] = reinterpret_cast<const Piece*>(src)[j];
    ok = valid;
  }
  __device__ __forceinline__ IT raw(int e) const {
    IT v;
    __builtin_memcpy(&v, reinterpret_cast<const unsigned char*>(p) + e * sizeof(IT), sizeof(IT));
    return ok ? v : IT(0);
  }
};

template <int DK, int RB_>
struct Cfg {
  static constexpr int DV = DK;
  static constexpr int L = prefill_chunk(false);
  static constexpr int T = prefill_window(false);    // readout window (tokens)
  static constexpr int SC = T / L;                   // chunks per readout window
  static constexpr int RB = RB_;                     // 16-row blocks a wave
  static constexpr int NB = col_blocks(DV);        // 16-wide column blocks incl. z
  static constexpr int NC = NB * 16;
  static constexpr int DVP = padded_dv(DV);
  static constexpr int NSLOT = prefill_slots_rb(RB_, false);
  static constexpr int KSTR = prefill_kstride(false); // xk / pk row stride (floats)
  static constexpr int QSTR = L + 1;                 // pq row stride
  static constexpr int XQSTR = DK + 4;               // xq row stride
  static constexpr int RSTR = L + 4;                 // reduction row stride (floats)
  static constexpr int XK_ZERO = 2 * DK * KSTR;      // offset of the zero row
  static constexpr int MB = L / 16;                  // 16-token blocks per chunk
  static constexpr int EPT = L * DK / (kWaves * 64); // staged elements per thread and tensor
  static constexpr int TPG = L / 4;                  // token groups of the cross-wave sum
};

template <int DK, int RB_>
__global__ __launch_bounds__(kWaves * 64, 1) void prefill_scan(ScanArgs a) {
  // tokens of this head in the window; none: the state is left as it is
  const int nwh = head_tokens(a.lens, blockIdx.y, a.t0, a.nw, a.n_total);
  if (nwh == 0) return;
  using C = Cfg<DK, RB_>;
  constexpr int DV = C::DV, L = C::L, RB = C::RB, NB = C::NB, NC = C::NC, DVP = C::DVP;
  constexpr int NSLOT = C::NSLOT, KSTR = C::KSTR, QSTR = C::QSTR, XQSTR = C::XQSTR;
  // d_v a multiple of 16: the denominator column would fill a 16-wide MFMA
  // block of its own (half the blocks at d = 16), so z and phi_q.z run on
  // VALU instead; the MFMA blocks hold value columns only.
  constexpr bool VDEN = DV % 16 == 0;
  constexpr int NBM = VDEN ? NB - 1 : NB;
  constexpr int RSTR = C::RSTR, XK_ZERO = C::XK_ZERO, MB = C::MB, EPT = C::EPT;
  using IT = float;
  using RedT = float;

  __shared__ __attribute__((aligned(16))) float xk[(2 * DK + 1) * KSTR];
  __shared__ __attribute__((aligned(16))) float pk[NSLOT * KSTR];
  __shared__ __attribute__((aligned(16))) float pq[NSLOT * QSTR];
  __shared__ __attribute__((aligned(16))) float xq[L * XQSTR];
  __shared__ __attribute__((aligned(16))) RedT red[kWaves * (DV + 1) * RSTR];
  __shared__ __attribute__((aligned(16))) float vv[L * NC];
  __shared__ float carry[NC];
  __shared__ uint32_t spar[NSLOT];
  __shared__ float spwq[NSLOT];
  __shared__ float spwk[NSLOT];

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
    spwq[s] = a.lay.pweight[tile * NSLOT + s];
    spwk[s] = a.lay.kscale[tile * NSLOT + s];
  }
  for (int i = tid; i < KSTR; i += kWaves * 64) xk[XK_ZERO + i] = 0.f;
  for (int e = tid; e < L * (NC - DV); e += kWaves * 64) {
    const int t = e / (NC - DV);
    const int c = DV + e % (NC - DV);
    vv[t * NC + c] = (c == DV) ? 1.f : 0.f;
  }


  // Load the state tile into the accumulators (C layout: lane holds column
  // nb*16 + lr of rows 4g + r), divided by the multiplicity of each row's
  // last index.
  float* st = a.state + static_cast<int64_t>(head) * a.stride;
  const int64_t zoff = static_cast<int64_t>(a.D) * DV;
  // Row indices first; within a block every load is unconditional (a pad
  // row or a column past den reads a valid word and is zeroed), so a block's
  // loads are in flight together.  32-bit offsets: a head's state is below
  // 2^32 bytes.
  uint32_t info[RB][4];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) info[b][r] = a.lay.rowinfo[(lay_base + b) * 16 + 4 * g + r];
  f32x4 S[RB][NBM];
  // VDEN: z of rows 4 g + r of block b, the same in every lane of group g
  float zr[VDEN ? RB : 1][4];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t m = info[b][r] ? (info[b][r] & 0x0fffffffu) - 1 : 0u;
#pragma unroll
      for (int nb = 0; nb < NBM; ++nb) {
        const int col = nb * 16 + lr;
        S[b][nb][r] = st[col < DV ? m * DV + col : static_cast<uint32_t>(zoff) + m];
      }
      if constexpr (VDEN) zr[b][r] = st[static_cast<uint32_t>(zoff) + m];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float inv_cnt = info[b][r] ? 1.f / static_cast<float>(info[b][r] >> 28) : 0.f;
#pragma unroll
      for (int nb = 0; nb < NBM; ++nb) S[b][nb][r] = (nb * 16 + lr <= DV) ? S[b][nb][r] * inv_cnt : 0.f;
      if constexpr (VDEN) zr[b][r] *= inv_cnt;
    }
    // Move the block into accumulator registers right away, so the whole
    // tile is never held in VGPRs at once.
#pragma unroll
    for (int nb = 0; nb < NBM; ++nb) asm volatile("" : "+a"(S[b][nb]));
    __builtin_amdgcn_sched_barrier(0);
  }
  if (tile == 0 && tid < NC) carry[tid] = tid < DV ? st[tid] : (tid == DV ? st[zoff] : 0.f);

  const IT* qh = static_cast<const IT*>(a.q) + static_cast<int64_t>(head) * a.n_total * DK;
  const IT* kh = static_cast<const IT*>(a.k) + static_cast<int64_t>(head) * a.n_total * DK;
  const IT* vh = static_cast<const IT*>(a.v) + static_cast<int64_t>(head) * a.n_total * DV;
  const int nwp = a.ws.nwp;
  RedT* rech = static_cast<RedT*>(a.ws.rec) +
               (static_cast<int64_t>(head) * n_tiles + tile) * DVP * static_cast<int64_t>(nwp);
  const int nch = (nwh + L - 1) / L;
  float* carryh = a.ws.carry + static_cast<int64_t>(head) * ((nwp + C::T - 1) / C::T) * DVP;

  // Cross-wave sum of one chunk's readout (LDS red) into its records.
  auto red_sum = [&](int ch) {
    for (int e = tid; e < (DV + 1) * C::TPG; e += kWaves * 64) {
      const int c = e / C::TPG;
      const int tg = e % C::TPG;
      f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww)
        sum += *reinterpret_cast<const f32x4*>(&red[(ww * (DV + 1) + c) * RSTR + 4 * tg]);
      *reinterpret_cast<f32x4*>(&rech[static_cast<int64_t>(c) * nwp + ch * L + 4 * tg]) = sum;
    }
  };

  // Each thread stages EPT consecutive elements of one token per tensor;
  // consecutive lanes take consecutive tokens (conflict-free transposed writes).
  const int st_t = tid % L;
  const int st_i = (tid / L) * EPT;
  ChunkRegs<IT, EPT> rq, rk, rv;
  {
    // Tokens past the window read the window's first token (always valid).
    const bool ok = st_t < min(L, nwh);
    const int64_t tn = a.t0 + (ok ? st_t : 0);
    rq.load(qh + tn * DK + st_i, ok);
    rk.load(kh + tn * DK + st_i, ok);
    rv.load(vh + tn * DV + st_i, ok);
  }

  // Chunks grouped by readout window (here a window is one chunk: the readout
  // reads the live fp32 state).
  for (int ch0 = 0; ch0 < nch; ch0 += C::SC) {
  const int ch_end = min(nch, ch0 + C::SC);
  for (int ch = ch0; ch < ch_end; ++ch) {
    const int64_t tb = a.t0 + static_cast<int64_t>(ch) * L;
    const int nvalid = min(L, nwh - ch * L);
    // Launder the run metadata so the LDS addresses derived from it are
    // recomputed each chunk (a few integer ops) instead of held live.
#pragma unroll
    for (int b = 0; b < RB; ++b) asm volatile("" : "+v"(ks[b]), "+v"(qs[b]));

    // ---- phase A: previous chunk's records, then stage this chunk --------
    if (ch > 0) red_sum(ch - 1);
#pragma unroll
    for (int e = 0; e < EPT; e += 4) {
      float4 q4;
      q4.x = to_f32(rq.raw(e)) * a.inv_c;
      q4.y = to_f32(rq.raw(e + 1 < EPT ? e + 1 : e)) * a.inv_c;
      q4.z = to_f32(rq.raw(e + 2 < EPT ? e + 2 : e)) * a.inv_c;
      q4.w = to_f32(rq.raw(e + 3 < EPT ? e + 3 : e)) * a.inv_c;
      if constexpr (EPT >= 4) {
        *reinterpret_cast<float4*>(__builtin_assume_aligned(&xq[st_t * XQSTR + st_i + e], 16)) = q4;
      } else {
        xq[st_t * XQSTR + st_i + e] = q4.x;
        if (EPT > 1) xq[st_t * XQSTR + st_i + e + 1] = q4.y;
      }
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const float kv = to_f32(rk.raw(e));
      xk[(st_i + e) * KSTR + st_t] = kv;
      xk[(DK + st_i + e) * KSTR + st_t] = kv * 0.5f;
      vv[st_t * NC + st_i + e] = rv.raw(e);
    }
    // Prefetch the next chunk; the loads stay in flight through this chunk.
    if (ch + 1 < nch) {
      const bool ok = st_t < min(L, nwh - (ch + 1) * L);
      const int64_t tn = tb + L + (ok ? st_t : 0);
      rq.load(qh + tn * DK + st_i, ok);
      rk.load(kh + tn * DK + st_i, ok);
      rv.load(vh + tn * DV + st_i, ok);
    }
    __syncthreads();

    // ---- phase B: parent features (order <= 3) and the order-0 carry -----
    for (int e = tid; e < nslot * L; e += kWaves * 64) {
      const int s = e / L;
      const int t = e % L;
      const uint32_t pw = spar[s];
      const int np = pw >> 24;
      float fk = spwk[s], fq = spwq[s];
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        if (r < np) {
          const int i = (pw >> (8 * r)) & 255;
          fk *= xk[i * KSTR + t];
          fq *= xq[t * XQSTR + i];
        }
      }
      pk[s * KSTR + t] = fk;
      pq[s * QSTR + t] = fq;
    }
    if (tile == 0) {
      // Order-0 prefix at each readout window's start, then add the chunk
      // (exact fp32).
      const bool wstart = ch % C::SC == 0;
      if (tid < DV) {
        if (wstart) carryh[static_cast<int64_t>(ch / C::SC) * DVP + tid] = carry[tid];
        float s = 0.f;
        for (int t = 0; t < nvalid; ++t) {
          s += vv[t * NC + tid];
        }
        carry[tid] += s;
      } else if (tid == DV) {
        if (wstart) carryh[static_cast<int64_t>(ch / C::SC) * DVP + DV] = carry[DV];
        carry[DV] += static_cast<float>(nvalid);
      }
    }
    __syncthreads();

    // ---- phase C: readout against the state before this chunk -----------
    // (two 16-token blocks at a time), written to the reduction buffer.
#pragma unroll
    for (int half = 0; half < MB / 2; ++half) {
      f32x4 acc[2][NBM];
      float dn[2] = {0.f, 0.f};   // VDEN: phi_q.z over the lane's rows, token 16 mb + lr
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBM; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const int slot = qs[b] & 0xffff;
        const int c0 = qs[b] >> 16;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int t = (2 * half + mb) * 16 + lr;
          const float p = pq[slot * QSTR + t];
          const float4 x = lds4(xq, t * XQSTR + c0);
          const float av[4] = {p * x.x, p * x.y, p * x.z, p * x.w};
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int nb = 0; nb < NBM; ++nb)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[r], S[b][nb][r], acc[mb][nb], 0, 0, 0);
          if constexpr (VDEN) {
#pragma unroll
            for (int r = 0; r < 4; ++r) dn[mb] = fmaf(av[r], zr[b][r], dn[mb]);
          }
        }
      }
      if constexpr (VDEN) {
        // over the four lane groups (rows 4 g + r), then one store a token
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          float d = dn[mb];
          d += __shfl_xor(d, 16);
          d += __shfl_xor(d, 32);
          if (g == 0) red[(w * (DV + 1) + DV) * RSTR + (2 * half + mb) * 16 + lr] = d;
        }
      }

      // C layout: lane holds column nb*16 + lr of tokens 4g..4g+3 -> one
      // 4-token vector store per (block, column block).
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBM; ++nb) {
          const int col = nb * 16 + lr;
          if (col <= DV) {
            RedT* dst = &red[(w * (DV + 1) + col) * RSTR + (2 * half + mb) * 16 + 4 * g];
            *reinterpret_cast<f32x4*>(__builtin_assume_aligned(dst, 16)) = acc[mb][nb];
          
          }
        }
    }

    // ---- phase C: state update S += phi_k(K)^T [V 1] ----------------------
    float zinc[VDEN ? RB : 1];   // VDEN: sum of phi_k(row lr) over the lane's tokens
#pragma unroll
    for (int b = 0; b < (VDEN ? RB : 1); ++b) zinc[b] = 0.f;
#pragma unroll
    for (int kst = 0; kst < L / 4; ++kst) {
      const int t = 4 * kst + g;
      float bv[NBM];
#pragma unroll
      for (int nb = 0; nb < NBM; ++nb) bv[nb] = vv[t * NC + nb * 16 + lr];
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const int pko = ks[b] & 0xffff;
        const int xko = ks[b] >> 16;
        const float av = pk[pko + t] * xk[xko + t];
#pragma unroll
        for (int nb = 0; nb < NBM; ++nb)
          S[b][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv[nb], S[b][nb], 0, 0, 0);
        if constexpr (VDEN) zinc[b] += av;
      }
    }
    if constexpr (VDEN) {
      // z of row lr gains the sum over the four token groups; lane (lr, g)
      // keeps rows 4 g + r, found in lanes 4 g + r of group 0
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        float x = zinc[b];
        x += __shfl_xor(x, 16);
        x += __shfl_xor(x, 32);
#pragma unroll
        for (int r = 0; r < 4; ++r) zr[b][r] += __shfl(x, 4 * g + r);
      }
    }
  
    __syncthreads();
  }
  }
  if (nch > 0) red_sum(nch - 1);

  // Write the state tile back in canonical layout.  The row table pointer is
  // laundered so the addresses are recomputed here instead of being kept live
  // (in registers) from the initial load across the whole chunk loop.
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
      const uint32_t m = (info2[b][r] & 0x0fffffffu) - 1;
      const float cnt = static_cast<float>(info2[b][r] >> 28);
#pragma unroll
      for (int nb = 0; nb < NBM; ++nb) {
        const int col = nb * 16 + lr;
        if (info2[b][r] != 0u && col <= DV)
          stw[col < DV ? m * DV + col : static_cast<uint32_t>(zoff) + m] = S[b][nb][r] * cnt;
      }
      if constexpr (VDEN) {
        if (info2[b][r] != 0u && lr == 0) stw[static_cast<uint32_t>(zoff) + m] = zr[b][r] * cnt;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (tile == 0) {
    if (tid < DV) st[tid] = carry[tid];
    else if (tid == DV) st[zoff] = carry[DV];
  }
}

// Intra-window part for float32 inputs, on fp32 MFMA (16x16x4): for the
// window's queries i and keys j <= i, sum T_P(q_i.k_j/c) (v_j, 1).  Block =
// (window of T = 32 tokens, head), one wave.  With A the 16 x 4 and B the
// 4 x 16 operand (lane (lr, g) holds A[lr][g] and B[g][lr]) and the 16 x 16
// result in C layout (lane (lr, g) holds rows 4 g .. 4 g + 3 of column lr):
//   X^T[key][query] = sum over dims of K Q^T    (tiles of 16 keys x 16 queries)
//   W^T = T_P(X^T / c) by Horner's rule, zero for keys after the query
//   O^T[col][query] += V'^T W^T                  (V' = [v, 1, 0...])
// For K-step s of a key tile, lane (lr, g) feeds key 4 g + s: its own C-layout
// element s of W^T is the B operand, and the A operand is V' at that key, so
// no value crosses lanes.  Writes record columns [DVP][nwp].
template <int DK>
__global__ __launch_bounds__(64) void prefill_intra(IntraArgs a) {
  constexpr int DV = DK, T = prefill_window(false);
  static_assert(T == 32, "two 16-token tiles per window");
  constexpr int NB = col_blocks(DV), NC = NB * 16;
  constexpr int KS = DK + 1;                  // LDS row stride of q and k (floats)
  constexpr int VS = NC + 1;                  // LDS row stride of v'
  __shared__ float sq[T * KS];
  __shared__ float sk[T * KS];
  __shared__ float sv[T * VS];
  const int win = blockIdx.x;
  const int head = blockIdx.y;
  const int l = threadIdx.x;
  const int lr = l & 15;
  const int g = l >> 4;
  const int64_t tb = a.t0 + static_cast<int64_t>(win) * T;
  const int nvalid = min(T, head_tokens(a.lens, head, a.t0, a.nw, a.n_total) - win * T);
  if (nvalid <= 0) return;
  const float* qh = static_cast<const float*>(a.q) + static_cast<int64_t>(head) * a.n_total * DK;
  const float* kh = static_cast<const float*>(a.k) + static_cast<int64_t>(head) * a.n_total * DK;
  const float* vh = static_cast<const float*>(a.v) + static_cast<int64_t>(head) * a.n_total * DV;
  for (int e = l; e < T * DK; e += 64) {
    const int t = e / DK, d = e % DK;
    const bool ok = t < nvalid;
    sq[t * KS + d] = ok ? qh[(tb + t) * DK + d] * a.inv_c : 0.f;
    sk[t * KS + d] = ok ? kh[(tb + t) * DK + d] : 0.f;
  }
  for (int e = l; e < T * NC; e += 64) {
    const int t = e / NC, c = e % NC;
    const bool ok = t < nvalid;
    sv[t * VS + c] = !ok ? 0.f : c < DV ? vh[(tb + t) * DV + c] : (c == DV ? 1.f : 0.f);
  }
  __syncthreads();
  const float rcp[5] = {0.f, 1.f, 0.5f, 1.f / 3.f, 0.25f};
  float* rec = a.ws.intra + static_cast<int64_t>(head) * padded_dv(DV) * a.ws.nwp + static_cast<int64_t>(win) * T;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    f32x4 O[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) O[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int qi = 16 * qt + lr;                 // this lane's query (window-relative)
#pragma unroll
    for (int kt = 0; kt <= qt; ++kt) {           // key tiles at or before the query tile
      f32x4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kst = 0; kst < DK / 4; ++kst)
        X = __builtin_amdgcn_mfma_f32_16x16x4f32(sk[(16 * kt + lr) * KS + 4 * kst + g],
                                                 sq[(16 * qt + lr) * KS + 4 * kst + g], X, 0, 0, 0);
      f32x4 Wt;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kj = 16 * kt + 4 * g + r;      // key of element r
        float wgt = 1.f;
        for (int p = a.P - 1; p >= 1; --p) wgt = fmaf(wgt, X[r] * rcp[p], 1.f);
        Wt[r] = (kj <= qi && kj < nvalid) ? wgt : 0.f;
      }
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          O[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(sv[(16 * kt + 4 * g + st) * VS + 16 * nb + lr], Wt[st], O[nb],
                                                       0, 0, 0);
    }
    if (qi < nvalid) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = 16 * nb + 4 * g + r;
          if (c <= DV) rec[static_cast<int64_t>(c) * a.ws.nwp + qi] = O[nb][r];
        }
    }
  }
}

// Intra-window part on MFMA, for bf16 inputs.  Block = (readout window of T
// tokens, head); each wave owns 64 queries of the window, the groups paired
// so that the two waves sharing a SIMD (w and w + 4 of 8) take one early and
// one late group (equal causal work per SIMD).  For every 32-key slice up to
// the wave's last query:
//   X^T = K_s Q_w^T                       (bf16 MFMA, fp32 accumulate)
//   W'  = T_P(X / c) - 1 in fp32 (nested with the coefficients 1/(p! c^p),
//         zero past order P - 1), zero for keys after the query
//   O^T += V'^T_s M + V'^T_s W_hi + V'^T_s W_lo   (M = the 0/1 causal mask)
// V' = [v, 1, 0...]: its ones row gives the denominator.  The order-0 term
// goes through the exact 0/1 mask, and the higher-order weights W' as two
// bf16 parts (W_hi = bf16(W'), W_lo = bf16(W' - W_hi)), about 2^-17 relative.
// P5: orders 0..4 (a fourth nesting step; P <= 4 takes three).
template <int DK, bool P5>
__global__ __launch_bounds__(prefill_window(true)) void prefill_intra_mfma(IntraArgs a) {
  constexpr int DV = DK, T = prefill_window(true);
  constexpr int NT = T;                        // threads: one 64-query wave per 64 tokens
  constexpr int KP = DK < 32 ? 32 : DK;        // head dim padded to the MFMA K
  constexpr int KSTEPS = KP / 32;
  constexpr int KSTR = KP + 8;                 // bf16 per staged key row
  constexpr int NB = col_blocks(DV), NC = NB * 16;
  constexpr int VSTR = T + 8;                  // bf16 per staged V' row
  constexpr int DVP = padded_dv(DV);
  static_assert(T % 64 == 0 && DK % 8 == 0, "window of 64-query waves");
  __shared__ __attribute__((aligned(16))) uint16_t ks_[T * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t vt[NC * VSTR];
  const int win = blockIdx.x;
  const int head = blockIdx.y;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int lr = l & 15;
  const int g = l >> 4;
  const int64_t tb = a.t0 + static_cast<int64_t>(win) * T;
  const int nvalid = min(T, head_tokens(a.lens, head, a.t0, a.nw, a.n_total) - win * T);
  if (nvalid <= 0) return;
  const uint16_t* qh = static_cast<const uint16_t*>(a.q) + static_cast<int64_t>(head) * a.n_total * DK;
  const uint16_t* kh = static_cast<const uint16_t*>(a.k) + static_cast<int64_t>(head) * a.n_total * DK;
  const uint16_t* vh = static_cast<const uint16_t*>(a.v) + static_cast<int64_t>(head) * a.n_total * DV;

  // Stage K row-major (zero-padded to KP, zero past the window) and V'^T.
  // Every load first, from a valid address (the window's first token for
  // items outside it, zeroed after), so they are in flight together.
  constexpr int KI = T * (KP / 8) / NT, VI = T * (DV / 8) / NT;
  static_assert(KI * NT == T * (KP / 8) && VI * NT == T * (DV / 8), "staging items per thread");
  u32x4 kv[KI], vv[VI];
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int e = tid + i * NT;
    const int t = e / (KP / 8), c8 = (e % (KP / 8)) * 8;
    const bool ok = t < nvalid && c8 < DK;
    kv[i] = *reinterpret_cast<const u32x4*>(kh + (tb + (ok ? t : 0)) * DK + (ok ? c8 : 0));
    if (!ok) kv[i] = u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < VI; ++i) {
    const int e = tid + i * NT;
    const int t = e % T, c8 = (e / T) * 8;
    const bool ok = t < nvalid;
    vv[i] = *reinterpret_cast<const u32x4*>(vh + (tb + (ok ? t : 0)) * DV + c8);
    if (!ok) vv[i] = u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int e = tid + i * NT;
    *reinterpret_cast<u32x4*>(&ks_[(e / (KP / 8)) * KSTR + (e % (KP / 8)) * 8]) = kv[i];
  }
#pragma unroll
  for (int i = 0; i < VI; ++i) {
    const int e = tid + i * NT;
    const int t = e % T, c8 = (e / T) * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      vt[(c8 + j) * VSTR + t] = static_cast<uint16_t>((j & 1) ? (vv[i][j / 2] >> 16) : (vv[i][j / 2] & 0xffffu));
  }
  for (int e = tid; e < (NC - DV) * T; e += NT) {
    const int c = DV + e / T;
    const int t = e % T;
    vt[c * VSTR + t] = (c == DV && t < nvalid) ? static_cast<uint16_t>(0x3f80) : static_cast<uint16_t>(0);
  }

  // Query group of this wave (64 queries): early groups on waves 0..W/2-1,
  // late ones (in reverse) on the waves sharing their SIMDs.
  constexpr int NWV = NT / 64;
  const int qg = w < NWV / 2 ? w : 3 * NWV / 2 - 1 - w;
  // Query operands (B of X^T): lane holds query 16 qb + lr, dims 32 kst + 8 g ...
  bf16x8 qop[4][KSTEPS];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb)
#pragma unroll
    for (int kst = 0; kst < KSTEPS; ++kst) {
      const int qi = 64 * qg + 16 * qb + lr;
      const int d0 = 32 * kst + 8 * g;
      const bool ok = qi < nvalid && d0 < DK;
      u32x4 val = *reinterpret_cast<const u32x4*>(qh + (tb + (ok ? qi : 0)) * DK + (ok ? d0 : 0));
      if (!ok) val = u32x4{0u, 0u, 0u, 0u};
      qop[qb][kst] = __builtin_bit_cast(bf16x8, val);
    }
  __syncthreads();

  f32x4 O[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) O[nb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // W' = T_P(x/c) - 1 = x (a1 + x (a2 + x (a3 + x a4))), a_p = 1 / (p! c^p)
  // for p < P and 0 beyond: the same nesting for every P, no per-order select
  const float ic = a.inv_c;
  const float a1 = a.P > 1 ? ic : 0.f;
  const float a2 = a.P > 2 ? ic * ic * 0.5f : 0.f;
  const float a3 = a.P > 3 ? ic * ic * ic * (1.f / 6.f) : 0.f;
  const float a4 = P5 && a.P > 4 ? ic * ic * ic * ic * (1.f / 24.f) : 0.f;
  const int nslice = min(2 * qg + 2, (nvalid + 31) / 32);
  for (int sl = 0; sl < nslice; ++sl) {
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
    // Weights in B layout: lane holds query 16 qb + lr and keys
    // 32 sl + 16 (j / 4) + 4 g + j % 4 for j = 0..7.
    bf16x8 Bm[4], Bw[4], Bl[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const int qi = 64 * qg + 16 * qb + lr;
      float wv[8], mv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = 32 * sl + 16 * (j / 4) + 4 * g + (j % 4);
        const float x = X[j / 4][qb][j % 4];
        float h = P5 ? fmaf(x, a4, a3) : a3;
        h = fmaf(x, h, a2);
        h = fmaf(x, h, a1);
        h *= x;
        const bool ok = key <= qi;
        wv[j] = ok ? h : 0.f;
        mv[j] = ok ? 1.f : 0.f;
      }
      const u32x4 ww = {pack_bf16(wv[0], wv[1]), pack_bf16(wv[2], wv[3]), pack_bf16(wv[4], wv[5]),
                        pack_bf16(wv[6], wv[7])};
      // W' = hi + lo: the residual of the bf16 rounding, itself in bf16,
      // carries W' to about 2^-17 relative
      float rv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t w2 = ww[j / 2];
        rv[j] = wv[j] - __uint_as_float((j & 1) ? (w2 & 0xffff0000u) : (w2 << 16));
      }
      const u32x4 wl = {pack_bf16(rv[0], rv[1]), pack_bf16(rv[2], rv[3]), pack_bf16(rv[4], rv[5]),
                        pack_bf16(rv[6], rv[7])};
      const u32x4 mm = {pack_bf16(mv[0], mv[1]), pack_bf16(mv[2], mv[3]), pack_bf16(mv[4], mv[5]),
                        pack_bf16(mv[6], mv[7])};
      Bw[qb] = __builtin_bit_cast(bf16x8, ww);
      Bl[qb] = __builtin_bit_cast(bf16x8, wl);
      Bm[qb] = __builtin_bit_cast(bf16x8, mm);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint16_t* vr = &vt[(16 * nb + lr) * VSTR + 32 * sl + 4 * g];
      const u32x2 lo = *reinterpret_cast<const u32x2*>(__builtin_assume_aligned(vr, 8));
      const u32x2 hi = *reinterpret_cast<const u32x2*>(__builtin_assume_aligned(vr + 16, 8));
      const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
      const bf16x8 A = __builtin_bit_cast(bf16x8, av);
      // the three products of one accumulator four instructions apart
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) O[nb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bm[qb], O[nb][qb], 0, 0, 0);
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) O[nb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bw[qb], O[nb][qb], 0, 0, 0);
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) O[nb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bl[qb], O[nb][qb], 0, 0, 0);
    }
  }
  // O^T in C layout: lane holds query 16 qb + lr, value columns 16 nb + 4 g + r;
  // records are token-major, DVP columns a token.
  float* rec = a.ws.intra + (static_cast<int64_t>(head) * a.ws.nwp + static_cast<int64_t>(win) * T) * DVP;
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const int qi = 64 * qg + 16 * qb + lr;
    if (qi >= nvalid) continue;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = 16 * nb + 4 * g;
      if (col + 4 <= DVP) *reinterpret_cast<f32x4*>(&rec[static_cast<int64_t>(qi) * DVP + col]) = O[nb][qb];
    }
  }
}

// out = (tile records + intra record + order-0 carry) for num / for den,
// summed in a fixed order.  Block = (64 tokens, head).
template <int DK>
__global__ __launch_bounds__(256) void prefill_reduce(ReduceArgs a) {
  constexpr int DV = DK, DVP = padded_dv(DV), T = prefill_window(false);
  constexpr int TB = 64;
  __shared__ float acc[(DV + 1) * (TB + 1)];
  const int head = blockIdx.y;
  const int t0 = blockIdx.x * TB;
  const int tid = threadIdx.x;
  const int nwp = a.ws.nwp;
  const int64_t slab = static_cast<int64_t>(DVP) * nwp;
  const float* intra = a.ws.intra + head * slab;
  const float* carry = a.ws.carry + static_cast<int64_t>(head) * ((nwp + T - 1) / T) * DVP;
  const float* rec = static_cast<const float*>(a.ws.rec) + static_cast<int64_t>(head) * a.n_tiles * slab;
  for (int e = tid; e < (DV + 1) * (TB / 4); e += 256) {
    const int c = e / (TB / 4);
    const int t = 4 * (e % (TB / 4));
    const int64_t off = static_cast<int64_t>(c) * nwp + t0 + t;
    f32x4 r = {0.f, 0.f, 0.f, 0.f};
    for (int tl = 0; tl < a.n_tiles; ++tl) r += *reinterpret_cast<const f32x4*>(&rec[tl * slab + off]);
    f32x4 s = *reinterpret_cast<const f32x4*>(&intra[off]);
#pragma unroll
    for (int j = 0; j < 4; ++j) s[j] += r[j];
#pragma unroll
    for (int j = 0; j < 4; ++j) s[j] += carry[((t0 + t + j) / T) * DVP + c];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[c * (TB + 1) + t + j] = s[j];
  }
  __syncthreads();
  const int ntok = min(TB, a.nw - t0);
  const int nlive = min(ntok, head_tokens(a.lens, head, a.t0, a.nw, a.n_total) - t0);
  float* out = a.out + (static_cast<int64_t>(head) * a.n_total + a.t0 + t0) * DV;
  for (int e = tid; e < ntok * DV; e += 256) {
    const int t = e / DV, c = e % DV;
    out[static_cast<int64_t>(t) * DV + c] = t < nlive ? acc[c * (TB + 1) + t] / acc[DV * (TB + 1) + t] : 0.f;
  }
}

// The scan and reduce here take float32 inputs; bfloat16 inputs have their
// own scan and reduce (launch_prefill_b16, launch_reduce_b16).
template <int D, bool BF16>
hipError_t launch_scan_t(int BH, const ScanArgs& a, hipStream_t s) {
  if (BF16) return hipErrorInvalidValue;
  dim3 grid(a.lay.n_tiles, BH);
  constexpr int RB = prefill_rb(D, false), RBS = prefill_rb_small(D);
  if (a.lay.rb == RB) {
    prefill_scan<D, RB><<<grid, kWaves * 64, 0, s>>>(a);
  } else if constexpr (RBS > 0) {
    if (a.lay.rb != RBS) return hipErrorInvalidValue;
    prefill_scan<D, RBS><<<grid, kWaves * 64, 0, s>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_intra_t(int BH, const IntraArgs& a, hipStream_t s) {
  constexpr int T = prefill_window(BF16);
  dim3 grid((a.nw + T - 1) / T, BH);
  if (!BF16)
    prefill_intra<D><<<grid, 64, 0, s>>>(a);
  else if (a.P == 5)
    prefill_intra_mfma<D, true><<<grid, T, 0, s>>>(a);
  else
    prefill_intra_mfma<D, false><<<grid, T, 0, s>>>(a);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_reduce_t(int BH, const ReduceArgs& a, hipStream_t s) {
  if (BF16) return hipErrorInvalidValue;
  dim3 grid((a.nw + 63) / 64, BH);
  prefill_reduce<D><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

#define SATA_DISPATCH(fn, d, bf16, ...)                                   \
  switch (d) {                                                            \
    case 8: return bf16 ? fn<8, true>(__VA_ARGS__) : fn<8, false>(__VA_ARGS__);     \
    case 16: return bf16 ? fn<16, true>(__VA_ARGS__) : fn<16, false>(__VA_ARGS__);  \
    case 32: return bf16 ? fn<32, true>(__VA_ARGS__) : fn<32, false>(__VA_ARGS__);  \
    case 64: return bf16 ? fn<64, true>(__VA_ARGS__) : fn<64, false>(__VA_ARGS__);  \
    default: return hipErrorInvalidValue;                                 \
  }

}  // namespace

hipError_t launch_prefill_scan(int d, bool bf16, int BH, const ScanArgs& a, hipStream_t s) {
  SATA_DISPATCH(launch_scan_t, d, bf16, BH, a, s)
}

hipError_t launch_prefill_intra(int d, bool bf16, int BH, const IntraArgs& a, hipStream_t s) {
  SATA_DISPATCH(launch_intra_t, d, bf16, BH, a, s)
}

hipError_t launch_prefill_reduce(int d, bool bf16, int BH, const ReduceArgs& a, hipStream_t s) {
  SATA_DISPATCH(launch_reduce_t, d, bf16, BH, a, s)
}

}  // namespace sata
