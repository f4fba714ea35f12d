// Decode step of causal SATA on gfx950: one new token per resident state.
//
// Each state takes its token's key into every basis row (S_m += phi_m(k) v,
// z_m += phi_m(k)) and then reads out num = sum_m w_m phi_m(q) S_m and
// den = sum_m w_m phi_m(q) z_m, so the token attends to itself
// [SATA page, section "Engineering of constant compute cost": the per-token
// step maps the key through the index matrix, accumulates, and forms the
// output from the weighted sum over orders].
//
// The step is bound by HBM: every state value is read once and written once.
// Layout of the work: grid = (row tiles) x (states), blocks of 128 threads,
// tiles of two rows per thread (16 rows of 64 floats at d_v = 64: 4 KB of
// state per block).  A block
// issues the loads of its S rows and z values first, builds the features of
// its rows (phi_k unweighted, phi_q with the row weight) while they are in
// flight, then applies the rank-1 update, stores, and forms its readout
// partial sums; a second kernel reduces the per-tile partials in a fixed
// order and divides (with few states and many tiles, in two passes so the
// reduce still spreads over the chip).  Small one-shot blocks stream this read-modify-write at
// 6.2 TB/s where 512-row blocks that loop over their rows reach 5.3.  With
// bf16 inputs the value partials go out as 16-bit records (f16 with a
// power-of-two scale per tile; fp32 for the tiles of the order-0 and order-1
// rows), half the bytes the reduce reads.  The state is touched once per step and
// is far larger than the caches, so its loads and stores carry the
// non-temporal hint.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "sata_device.h"
#include "sata_internal.h"

namespace sata {
namespace {

__device__ __forceinline__ float load_in(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_in(const uint16_t* p, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

// Four floats as a clang vector (the non-temporal builtins take vector types).
typedef float f4v __attribute__((ext_vector_type(4)));

// One float4 slot of a state row, non-temporal.  AL: the state base is
// 16-byte aligned and the head stride a multiple of 4 floats (the padded
// layout), so the slot is one dwordx4 access; otherwise (the packed layout,
// heads state_floats apart) four dword accesses.
template <bool AL>
__device__ __forceinline__ f4v ld4(const float* p) {
  if constexpr (AL) {
    return __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p));
  } else {
    return f4v{__builtin_nontemporal_load(p), __builtin_nontemporal_load(p + 1), __builtin_nontemporal_load(p + 2),
               __builtin_nontemporal_load(p + 3)};
  }
}
template <bool AL>
__device__ __forceinline__ void st4(f4v x, float* p) {
  if constexpr (AL) {
    __builtin_nontemporal_store(x, reinterpret_cast<f4v*>(p));
  } else {
    __builtin_nontemporal_store(x.x, p);
    __builtin_nontemporal_store(x.y, p + 1);
    __builtin_nontemporal_store(x.z, p + 2);
    __builtin_nontemporal_store(x.w, p + 3);
  }
}

__device__ __forceinline__ f4v fma4(float s, f4v v, f4v acc) {
  acc.x = fmaf(s, v.x, acc.x);
  acc.y = fmaf(s, v.y, acc.y);
  acc.z = fmaf(s, v.z, acc.z);
  acc.w = fmaf(s, v.w, acc.w);
  return acc;
}

// Features of the tile's rows, phi_k = prod k[i_r] and phi_q = w_m prod q[i_r],
// into fk / fq (thread t < R builds row t; rows past nrows get 0).
template <int R>
__device__ __forceinline__ void tile_features(const float* xq, const float* xk, uint32_t pk, float wr, int nrows,
                                              float* fk, float* fq) {
  const int tid = threadIdx.x;
  if (tid < R) {
    const int p = static_cast<int>(pk >> 24);
    float fkk = 1.f, fqq = wr;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < p) {
        const int i = (pk >> (6 * t)) & 63;
        fkk *= xk[i];
        fqq *= xq[i];
      }
    }
    fk[tid] = tid < nrows ? fkk : 0.f;
    fq[tid] = tid < nrows ? fqq : 0.f;
  }
}

// Fixed-order reductions of a tile's readout: over the row groups of a
// column (red[RPP][DV]) and over the block for den (one value per wave), into
// the tile's partial record.
template <int DV, int RPP>
__device__ __forceinline__ void tile_partials(const float* red, const float* dred, float* part, float* partz) {
  const int tid = threadIdx.x;
  if (tid < DV) {
    float sum = 0.f;
    for (int j = 0; j < RPP; ++j) sum += red[j * DV + tid];
    *(part + tid) = sum;
  }
  if (tid == DV) {
    float sum = 0.f;
    for (int j = 0; j < kDecodeThreads / 64; ++j) sum += dred[j];
    *partz = sum;
  }
}

// The same sums as 16-bit records (bf16 inputs): the value partials of tile
// `tile` of state s as f16 times a power of two that puts the tile's largest
// below 2^15 (the first lo_t tiles, the rows of orders 0 and 1, keep fp32
// records), den as fp32.
template <int DV, int RPP, typename A>
__device__ __forceinline__ void tile_partials_c16(const float* red, const float* dred, const A& a, int s, int tile) {
  static_assert(DV <= 64, "the value columns fit one wave");
  const int tid = threadIdx.x;
  const int64_t pi = static_cast<int64_t>(s) * a.n_tiles + tile;
  if (tid < 64) {
    float sum = 0.f;
    if (tid < DV)
      for (int j = 0; j < RPP; ++j) sum += red[j * DV + tid];
    if (tile < a.lo_t) {
      if (tid < DV) a.partlo[(static_cast<int64_t>(s) * a.lo_t + tile) * DV + tid] = sum;
    } else {
      const float m = wave_max(fabsf(sum));
      int e = 0;
      if (m > 0.f) (void)frexpf(m, &e);     // m < 2^e
      const int es = m > 0.f ? max(e - 15, -100) : 0;
      if (tid < DV)
        a.part16[pi * DV + tid] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(sum * ldexpf(1.f, -es)));
      if (tid == 0) a.psc[pi] = ldexpf(1.f, es);
    }
  }
  if (tid == DV) {
    float sum = 0.f;
    for (int j = 0; j < kDecodeThreads / 64; ++j) sum += dred[j];
    a.partz[pi] = sum;
  }
}

// One tile of fp32 rows [r0, r0 + nrows) of state s: S4 = its first row, z =
// its first z value.  Rank-1 update, store, readout partial into part/partz
// (C16: the 16-bit records of tile `tile`).
template <int DK, typename IT, bool AL, bool C16>
__device__ __forceinline__ void f32_tile(const DecodeArgs& a, int s, float* S4, float* z, int r0, int nrows,
                                         float* part, float* partz, int tile) {
  constexpr int DV = DK;
  constexpr int TPR = DV / 4;          // threads per S row, one float4 each
  constexpr int RPP = kDecodeThreads / TPR;  // rows per pass of the block
  constexpr int R = decode_rows(DV);   // rows of the tile
  constexpr int U = R / RPP;           // rows per thread, all in flight at once
  static_assert(U * RPP == R && R <= kDecodeThreads, "decode tile shape");
  static_assert(DV < kDecodeThreads, "one thread per value column plus one for den");

  __shared__ float xq[DK], xk[DK], xv[DV];
  __shared__ float fk[R], fq[R];
  __shared__ float red[RPP * DV];
  __shared__ float dred[kDecodeThreads / 64];

  const int tid = threadIdx.x;
  // The tile's state rows and z values go out first (a row past the tail
  // reads the tile's first row and is not written back); the features are
  // built while they are in flight.
  const int c4 = tid % TPR;
  const int rs = tid / TPR;
  f4v x[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int row = rs + u * RPP;
    x[u] = ld4<AL>(S4 + ((row < nrows ? row : 0) * TPR + c4) * 4);
  }
  const float zv = __builtin_nontemporal_load(&z[tid < nrows ? tid : 0]);

  const IT* q = static_cast<const IT*>(a.q) + static_cast<int64_t>(s) * DK;
  const IT* k = static_cast<const IT*>(a.k) + static_cast<int64_t>(s) * DK;
  const IT* v = static_cast<const IT*>(a.v) + static_cast<int64_t>(s) * DV;
  if (tid < DK) {
    xq[tid] = load_in(q, tid);
    xk[tid] = load_in(k, tid);
  }
  if (tid < DV) xv[tid] = load_in(v, tid);
  uint32_t pk = 0u;
  float wr = 0.f;
  if (tid < nrows) {
    pk = a.rows[r0 + tid];
    wr = a.weight[r0 + tid];
  }
  __syncthreads();
  tile_features<R>(xq, xk, pk, wr, nrows, fk, fq);
  __syncthreads();

  const f4v vv = {xv[4 * c4], xv[4 * c4 + 1], xv[4 * c4 + 2], xv[4 * c4 + 3]};
  f4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int row = rs + u * RPP;
    if (row < nrows) {
      x[u] = fma4(fk[row], vv, x[u]);
      st4<AL>(x[u], S4 + (row * TPR + c4) * 4);
      acc = fma4(fq[row], x[u], acc);
    }
  }
  float dacc = 0.f;
  if (tid < nrows) {
    const float zz = zv + fk[tid];
    __builtin_nontemporal_store(zz, &z[tid]);
    dacc = fq[tid] * zz;
  }

  red[rs * DV + 4 * c4 + 0] = acc.x;
  red[rs * DV + 4 * c4 + 1] = acc.y;
  red[rs * DV + 4 * c4 + 2] = acc.z;
  red[rs * DV + 4 * c4 + 3] = acc.w;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) dacc += __shfl_xor(dacc, o);
  if ((tid & 63) == 0) dred[tid >> 6] = dacc;
  __syncthreads();
  if constexpr (C16)
    tile_partials_c16<DV, RPP>(red, dred, a, s, tile);
  else
    tile_partials<DV, RPP>(red, dred, part, partz);
}

// bf16 inputs write 16-bit records, fp32 inputs fp32 ones.
template <int DK, typename IT, bool AL>
__global__ __launch_bounds__(kDecodeThreads) void decode_update_readout(DecodeArgs a) {
  constexpr int R = decode_rows(DK);
  const int tile = blockIdx.x;
  const int s = blockIdx.y;
  const int r0 = tile * R;
  const int nrows = min(R, a.D - r0);
  float* st = a.state + static_cast<int64_t>(s) * a.stride;
  const int64_t pi = static_cast<int64_t>(s) * a.n_tiles + tile;
  constexpr bool C16 = std::is_same<IT, uint16_t>::value;
  f32_tile<DK, IT, AL, C16>(a, s, st + static_cast<int64_t>(r0) * DK, st + static_cast<int64_t>(a.D) * DK + r0, r0,
                            nrows, C16 ? nullptr : a.part + pi * DK, C16 ? nullptr : a.partz + pi, tile);
}

// ---------------------------------------------------------------------------
// Mixed-precision state [SATA page, "Precision/efficiency trade-off
// parameter" and "Hardware optimisation path and current limitations": a
// 16-bit state roughly halves the bytes of the memory-bound step].  Rows of
// orders 0 and 1 of S and all of z stay fp32; rows of order >= 2 of S are
// f16, each tile of mixed_rows(d_v) rows scaled by a power of two.  The block
// that owns a tile reads it, updates it in fp32, reads out from the fp32
// values, and writes it back with a freshly chosen scale that puts the tile's
// largest entry below 2^15 (so a growing state never overflows f16; entries
// 2^29 below the tile's largest are subnormal).

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// One f16 tile (t16) of state s: rows [lo + t16 R, ...), record index pi.
template <int DK, typename IT, bool C16>
__device__ __forceinline__ void f16_tile(const MixedDecodeArgs& a, int s, int t16, float* part, float* partz) {
  constexpr int DV = DK;
  constexpr int TPR = DV / 8;                 // threads per f16 row, 8 halves (16 bytes) each
  constexpr int RPP = kDecodeThreads / TPR;   // rows per pass
  constexpr int R = mixed_rows(DV);
  constexpr int U = R / RPP;
  static_assert(U * RPP == R && R <= kDecodeThreads, "mixed tile shape");

  __shared__ float xq[DK], xk[DK], xv[DV];
  __shared__ float fk[R], fq[R];
  __shared__ float red[RPP * DV];
  __shared__ float dred[kDecodeThreads / 64];
  __shared__ float wmx[kDecodeThreads / 64];

  const int tid = threadIdx.x;
  unsigned char* base = a.state + static_cast<int64_t>(s) * a.stride_bytes;
  const int r0 = a.lo + t16 * R;                       // canonical first row
  const int nrows = min(R, a.D - r0);
  uint16_t* H = reinterpret_cast<uint16_t*>(base + a.off_h) + static_cast<int64_t>(t16) * R * DV;
  float* z = reinterpret_cast<float*>(base + a.off_z) + r0;
  float* sc = reinterpret_cast<float*>(base + a.off_sc) + t16;
  const int c8 = tid % TPR;
  const int rs = tid / TPR;
  u32x4 raw[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int row = rs + u * RPP;
    raw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(H + (row < nrows ? row : 0) * DV + 8 * c8));
  }
  const float zv = __builtin_nontemporal_load(&z[tid < nrows ? tid : 0]);
  const float scale = *sc;

  const IT* q = static_cast<const IT*>(a.q) + static_cast<int64_t>(s) * DK;
  const IT* k = static_cast<const IT*>(a.k) + static_cast<int64_t>(s) * DK;
  const IT* v = static_cast<const IT*>(a.v) + static_cast<int64_t>(s) * DV;
  if (tid < DK) {
    xq[tid] = load_in(q, tid);
    xk[tid] = load_in(k, tid);
  }
  if (tid < DV) xv[tid] = load_in(v, tid);
  uint32_t pk = 0u;
  float wr = 0.f;
  if (tid < nrows) {
    pk = a.rows[r0 + tid];
    wr = a.weight[r0 + tid];
  }
  __syncthreads();
  tile_features<R>(xq, xk, pk, wr, nrows, fk, fq);
  __syncthreads();

  float vv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) vv[j] = xv[8 * c8 + j];
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float x[U][8];
  float mx = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int row = rs + u * RPP;
    const bool live = row < nrows;
    const float f = live ? fk[row] : 0.f;
    const float g = live ? fq[row] : 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = raw[u][j];
      const f16x2 h = __builtin_bit_cast(f16x2, w);
      x[u][2 * j] = fmaf(f, vv[2 * j], static_cast<float>(h[0]) * scale);
      x[u][2 * j + 1] = fmaf(f, vv[2 * j + 1], static_cast<float>(h[1]) * scale);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[j] = fmaf(g, x[u][j], acc[j]);
      if (live) mx = fmaxf(mx, fabsf(x[u][j]));
    }
  }
  float dacc = 0.f;
  if (tid < nrows) {
    const float zz = zv + fk[tid];
    __builtin_nontemporal_store(zz, &z[tid]);
    dacc = fq[tid] * zz;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) red[rs * DV + 8 * c8 + j] = acc[j];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    dacc += __shfl_xor(dacc, o);
    mx = fmaxf(mx, __shfl_xor(mx, o));
  }
  if ((tid & 63) == 0) {
    dred[tid >> 6] = dacc;
    wmx[tid >> 6] = mx;
  }
  __syncthreads();
  // the tile's new scale: its largest |entry| times 2^-e below 2^15
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < kDecodeThreads / 64; ++j) m = fmaxf(m, wmx[j]);
  int e = 0;
  if (m > 0.f) (void)frexpf(m, &e);           // m < 2^e
  const int es = m > 0.f ? e - 15 : 0;
  const float inv = ldexpf(1.f, -es);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int row = rs + u * RPP;
    if (row < nrows) {
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f16x2 h = {static_cast<_Float16>(x[u][2 * j] * inv), static_cast<_Float16>(x[u][2 * j + 1] * inv)};
        o[j] = __builtin_bit_cast(uint32_t, h);
      }
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(H + row * DV + 8 * c8));
    }
  }
  if (tid == 0) *sc = ldexpf(1.f, es);
  if constexpr (C16)
    tile_partials_c16<DV, RPP>(red, dred, a, s, a.nt32 + t16);
  else
    tile_partials<DV, RPP>(red, dred, part, partz);
}

// Mixed-state decode: blocks [0, nt32) take fp32 tiles of rows [0, lo),
// blocks [nt32, nt32 + nt16) the f16 tiles; records in block order (bf16
// inputs: 16-bit records, fp32 ones for the fp32 tiles).
template <int DK, typename IT>
__global__ __launch_bounds__(kDecodeThreads) void decode_mixed(MixedDecodeArgs a) {
  constexpr int R32 = decode_rows(DK);
  constexpr bool C16 = std::is_same<IT, uint16_t>::value;
  const int tile = blockIdx.x;
  const int s = blockIdx.y;
  const int64_t pi = static_cast<int64_t>(s) * a.n_tiles + tile;
  float* part = C16 ? nullptr : a.part + pi * DK;
  float* partz = C16 ? nullptr : a.partz + pi;
  if (tile < a.nt32) {
    unsigned char* base = a.state + static_cast<int64_t>(s) * a.stride_bytes;
    float* st = reinterpret_cast<float*>(base);
    const int r0 = tile * R32;
    DecodeArgs d{};
    d.q = a.q;
    d.k = a.k;
    d.v = a.v;
    d.rows = a.rows;
    d.weight = a.weight;
    d.partz = a.partz;
    d.n_tiles = a.n_tiles;
    d.part16 = a.part16;
    d.psc = a.psc;
    d.partlo = a.partlo;
    d.lo_t = a.lo_t;
    f32_tile<DK, IT, true, C16>(d, s, st + static_cast<int64_t>(r0) * DK,
                                reinterpret_cast<float*>(base + a.off_z) + r0, r0, min(R32, a.lo - r0), part, partz,
                                tile);
  } else {
    f16_tile<DK, IT, C16>(a, s, tile - a.nt32, part, partz);
  }
}

// Conversion between the fp32 state ([S][stride] floats) and the mixed one.
// Grid x: nt16 f16 tiles, then blocks of kDecodeThreads * 4 floats over the
// fp32 rows and then over z; grid y: states.
template <int DK, bool TO_MIXED>
__global__ __launch_bounds__(kDecodeThreads) void mixed_convert(MixedConvArgs a) {
  constexpr int DV = DK;
  constexpr int R = mixed_rows(DV);
  __shared__ float wmx[kDecodeThreads / 64];
  const int s = blockIdx.y;
  const int tid = threadIdx.x;
  float* st = a.state + static_cast<int64_t>(s) * a.stride;
  unsigned char* base = a.mixed + static_cast<int64_t>(s) * a.stride_bytes;
  const int bx = blockIdx.x;
  if (bx < a.nt16) {
    const int r0 = a.lo + bx * R;
    const int nrows = min(R, a.D - r0);
    const int n = nrows * DV;
    const float* src = st + static_cast<int64_t>(r0) * DV;
    uint16_t* H = reinterpret_cast<uint16_t*>(base + a.off_h) + static_cast<int64_t>(bx) * R * DV;
    float* sc = reinterpret_cast<float*>(base + a.off_sc) + bx;
    if constexpr (TO_MIXED) {
      float mx = 0.f;
      for (int i = tid; i < n; i += kDecodeThreads) mx = fmaxf(mx, fabsf(src[i]));
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      if ((tid & 63) == 0) wmx[tid >> 6] = mx;
      __syncthreads();
      float m = 0.f;
#pragma unroll
      for (int j = 0; j < kDecodeThreads / 64; ++j) m = fmaxf(m, wmx[j]);
      int e = 0;
      if (m > 0.f) (void)frexpf(m, &e);
      const int es = m > 0.f ? e - 15 : 0;
      const float inv = ldexpf(1.f, -es);
      for (int i = tid; i < n; i += kDecodeThreads)
        H[i] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(src[i] * inv));
      if (tid == 0) *sc = ldexpf(1.f, es);
    } else {
      const float scale = *sc;
      float* dst = st + static_cast<int64_t>(r0) * DV;
      for (int i = tid; i < n; i += kDecodeThreads)
        dst[i] = static_cast<float>(__builtin_bit_cast(_Float16, H[i])) * scale;
    }
    return;
  }
  // plain fp32 copies: rows [0, lo) of S, then z
  const int64_t n32 = static_cast<int64_t>(a.lo) * DV;
  const int64_t i0 = static_cast<int64_t>(bx - a.nt16) * kDecodeThreads * 4;
  float* m32 = reinterpret_cast<float*>(base);
  float* mz = reinterpret_cast<float*>(base + a.off_z);
  const float* sz = st + static_cast<int64_t>(a.D) * DV;
  float* szw = st + static_cast<int64_t>(a.D) * DV;
  for (int j = 0; j < 4; ++j) {
    const int64_t i = i0 + j * kDecodeThreads + tid;
    if (i < n32) {
      if constexpr (TO_MIXED) m32[i] = st[i];
      else st[i] = m32[i];
    } else if (i < n32 + a.D) {
      if constexpr (TO_MIXED) mz[i - n32] = sz[i - n32];
      else szw[i - n32] = mz[i - n32];
    }
  }
}

// Sums, in a fixed order, the readout records [t0, t1) of one state: value
// records part[s][t][DV], den records partz[s][t] (nrec records a state).
// Block (g, s) takes the range g of length per; FINAL: out[s] = num / den,
// else the sums become record (s, g) of the next level (nxt, nxtz).  One
// block of kRedThreads: groups of DV/4 threads sum interleaved records
// (float4 columns, 8 loads in flight), then a fixed-order combine.
constexpr int kRedThreads = 1024;
// C16: value records as written by tile_partials_c16 (p16: f16 records, psc
// their scales, plo the fp32 records of the first lo_t tiles).
template <int DV, bool FINAL, bool C16>
__global__ __launch_bounds__(kRedThreads) void decode_reduce(const float* __restrict__ part_in,
                                                             const float* __restrict__ partz_in, int nrec,
                                                             int per, float* nxt, float* nxtz, float* out,
                                                             const uint16_t* __restrict__ p16,
                                                             const float* __restrict__ psc,
                                                             const float* __restrict__ plo, int lo_t) {
  constexpr int Q = DV / 4;              // float4 columns per record
  constexpr int G = kRedThreads / Q;     // record groups
  __shared__ float4 red[G * Q];
  __shared__ float dz[kRedThreads];
  __shared__ float dz2[32];
  __shared__ float tot[DV + 1];
  const int s = blockIdx.y;
  const int t0 = blockIdx.x * per;
  const int t1 = min(nrec, t0 + per);
  const int tid = threadIdx.x;
  const int grp = tid / Q;
  const int c = tid % Q;
  const float4* part = C16 ? nullptr : reinterpret_cast<const float4*>(part_in + static_cast<int64_t>(s) * nrec * DV);
  const float* partz = partz_in + static_cast<int64_t>(s) * nrec;
  {
    float z = 0.f;
    for (int t = t0 + tid; t < t1; t += kRedThreads) z += partz[t];
    dz[tid] = z;
  }
  if (grp < G) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    int t = t0 + grp;
    if constexpr (C16) {
      // the records in the same order as fp32 ones: an fp32 record of a
      // low-order tile first (t < lo_t <= G happens only for t = grp of the
      // first block), then f16 records times their scales
      if (t < lo_t && t < t1) {
        const float4 x = reinterpret_cast<const float4*>(plo + (static_cast<int64_t>(s) * lo_t + t) * DV)[c];
        acc.x += x.x;
        acc.y += x.y;
        acc.z += x.z;
        acc.w += x.w;
        t += G;
      }
      const uint2* q16 = reinterpret_cast<const uint2*>(p16 + static_cast<int64_t>(s) * nrec * DV);
      const float* sc = psc + static_cast<int64_t>(s) * nrec;
      auto add16 = [&](uint2 x, float f) {
        const _Float16 h0 = __builtin_bit_cast(_Float16, static_cast<uint16_t>(x.x & 0xffffu));
        const _Float16 h1 = __builtin_bit_cast(_Float16, static_cast<uint16_t>(x.x >> 16));
        const _Float16 h2 = __builtin_bit_cast(_Float16, static_cast<uint16_t>(x.y & 0xffffu));
        const _Float16 h3 = __builtin_bit_cast(_Float16, static_cast<uint16_t>(x.y >> 16));
        acc.x += static_cast<float>(h0) * f;
        acc.y += static_cast<float>(h1) * f;
        acc.z += static_cast<float>(h2) * f;
        acc.w += static_cast<float>(h3) * f;
      };
      for (; t + 7 * G < t1; t += 8 * G) {
        uint2 x[8];
        float f[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          x[u] = q16[static_cast<int64_t>(t + u * G) * Q + c];
          f[u] = sc[t + u * G];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) add16(x[u], f[u]);
      }
      for (; t < t1; t += G) add16(q16[static_cast<int64_t>(t) * Q + c], sc[t]);
    } else {
      for (; t + 7 * G < t1; t += 8 * G) {
        float4 x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = part[static_cast<int64_t>(t + u * G) * Q + c];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          acc.x += x[u].x;
          acc.y += x[u].y;
          acc.z += x[u].z;
          acc.w += x[u].w;
        }
      }
      for (; t < t1; t += G) {
        const float4 x = part[static_cast<int64_t>(t) * Q + c];
        acc.x += x.x;
        acc.y += x.y;
        acc.z += x.z;
        acc.w += x.w;
      }
    }
    red[grp * Q + c] = acc;
  }
  __syncthreads();
  if (tid < DV) {
    const float* redf = reinterpret_cast<const float*>(red);
    float sum = 0.f;
    for (int gg = 0; gg < G; ++gg) sum += redf[gg * DV + tid];
    tot[tid] = sum;
  } else if (tid >= 64 && tid < 96) {
    // den: 32 sums of 32 consecutive thread totals, then their sum (below)
    float sum = 0.f;
    for (int j = 0; j < kRedThreads / 32; ++j) sum += dz[(tid - 64) * (kRedThreads / 32) + j];
    dz2[tid - 64] = sum;
  }
  __syncthreads();
  if (tid == 0) {
    float sum = 0.f;
    for (int j = 0; j < 32; ++j) sum += dz2[j];
    tot[DV] = sum;
  }
  __syncthreads();
  if constexpr (FINAL) {
    if (tid < DV) out[static_cast<int64_t>(s) * DV + tid] = tot[tid] / tot[DV];
  } else {
    const int64_t r = static_cast<int64_t>(s) * gridDim.x + blockIdx.x;
    if (tid < DV) nxt[r * DV + tid] = tot[tid];
    else if (tid == DV) nxtz[r] = tot[DV];
  }
}

// The fixed-order reduce of a step's partial records (one or two passes).
// C16: the step's records are 16-bit ones (a.part16, a.psc, a.partlo).
template <int D, bool C16, typename A>
hipError_t launch_reduce(const float* part, const float* partz, float* out, int S, int n_tiles, int groups,
                         float* part2, float* partz2, const A& a, hipStream_t st) {
  const uint16_t* p16 = C16 ? a.part16 : nullptr;
  const float* psc = C16 ? a.psc : nullptr;
  const float* plo = C16 ? a.partlo : nullptr;
  const int lo_t = C16 ? a.lo_t : 0;
  if (groups <= 1) {
    decode_reduce<D, true, C16><<<dim3(1, S), kRedThreads, 0, st>>>(part, partz, n_tiles, n_tiles, nullptr, nullptr,
                                                                     out, p16, psc, plo, lo_t);
    return hipGetLastError();
  }
  // Few states: the tiles of a state are split over `groups` blocks, whose
  // sums a second pass combines (in group order).
  const int per = (n_tiles + groups - 1) / groups;
  decode_reduce<D, false, C16><<<dim3(groups, S), kRedThreads, 0, st>>>(part, partz, n_tiles, per, part2, partz2,
                                                                         nullptr, p16, psc, plo, lo_t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_reduce<D, true, false><<<dim3(1, S), kRedThreads, 0, st>>>(part2, partz2, groups, groups, nullptr, nullptr,
                                                                     out, nullptr, nullptr, nullptr, 0);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(bool bf16, const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.n_tiles, a.S);
  const bool al = a.stride % 4 == 0 && reinterpret_cast<uintptr_t>(a.state) % 16 == 0;
  if (bf16 && al)
    decode_update_readout<D, uint16_t, true><<<grid, kDecodeThreads, 0, st>>>(a);
  else if (bf16)
    decode_update_readout<D, uint16_t, false><<<grid, kDecodeThreads, 0, st>>>(a);
  else if (al)
    decode_update_readout<D, float, true><<<grid, kDecodeThreads, 0, st>>>(a);
  else
    decode_update_readout<D, float, false><<<grid, kDecodeThreads, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (bf16) return launch_reduce<D, true>(a.part, a.partz, a.out, a.S, a.n_tiles, a.groups, a.part2, a.partz2, a, st);
  return launch_reduce<D, false>(a.part, a.partz, a.out, a.S, a.n_tiles, a.groups, a.part2, a.partz2, a, st);
}

template <int D>
hipError_t launch_mixed_d(bool bf16, const MixedDecodeArgs& a, hipStream_t st) {
  dim3 grid(a.n_tiles, a.S);
  if (bf16)
    decode_mixed<D, uint16_t><<<grid, kDecodeThreads, 0, st>>>(a);
  else
    decode_mixed<D, float><<<grid, kDecodeThreads, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (bf16) return launch_reduce<D, true>(a.part, a.partz, a.out, a.S, a.n_tiles, a.groups, a.part2, a.partz2, a, st);
  return launch_reduce<D, false>(a.part, a.partz, a.out, a.S, a.n_tiles, a.groups, a.part2, a.partz2, a, st);
}

template <int D>
hipError_t launch_convert_d(bool to_mixed, const MixedConvArgs& a, hipStream_t st) {
  const int64_t n = static_cast<int64_t>(a.lo) * D + a.D;
  dim3 grid(a.nt16 + static_cast<int>((n + kDecodeThreads * 4 - 1) / (kDecodeThreads * 4)), a.S);
  if (to_mixed)
    mixed_convert<D, true><<<grid, kDecodeThreads, 0, st>>>(a);
  else
    mixed_convert<D, false><<<grid, kDecodeThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mixed(int d, bool bf16, const MixedDecodeArgs& a, hipStream_t s) {
  switch (d) {
    case 8: return launch_mixed_d<8>(bf16, a, s);
    case 16: return launch_mixed_d<16>(bf16, a, s);
    case 32: return launch_mixed_d<32>(bf16, a, s);
    case 64: return launch_mixed_d<64>(bf16, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_mixed_convert(int d, bool to_mixed, const MixedConvArgs& a, hipStream_t s) {
  switch (d) {
    case 8: return launch_convert_d<8>(to_mixed, a, s);
    case 16: return launch_convert_d<16>(to_mixed, a, s);
    case 32: return launch_convert_d<32>(to_mixed, a, s);
    case 64: return launch_convert_d<64>(to_mixed, a, s);
    default: return hipErrorInvalidValue;
  }
}

// Scratch of sata_decode_step_noalloc: the per-tile partial records of a
// decode step (the same regions as the caller's workspace of
// sata_decode_step).  Host code reaches it only through the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch_address(void** ptr) { return hipGetSymbolAddress(ptr, HIP_SYMBOL(scratch)); }

hipError_t launch_decode(int d, bool bf16, const DecodeArgs& a, hipStream_t s) {
  switch (d) {
    case 8: return launch_d<8>(bf16, a, s);
    case 16: return launch_d<16>(bf16, a, s);
    case 32: return launch_d<32>(bf16, a, s);
    case 64: return launch_d<64>(bf16, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sata
