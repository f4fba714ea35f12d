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
// 6.2 TB/s where 512-row blocks that loop over their rows reach 5.3 (the
// partials add 3.3 % to the traffic).  The state is touched once per step and
// is far larger than the caches, so its loads and stores carry the
// non-temporal hint.
#include <hip/hip_runtime.h>

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

template <int DK, typename IT, bool AL>
__global__ __launch_bounds__(kDecodeThreads) void decode_update_readout(DecodeArgs a) {
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

  const int tile = blockIdx.x;
  const int s = blockIdx.y;
  const int tid = threadIdx.x;
  const int r0 = tile * R;
  const int nrows = min(R, a.D - r0);

  // The tile's state rows and z values go out first (a row past the tail
  // reads the tile's first row and is not written back); the features are
  // built while they are in flight.
  float* st = a.state + static_cast<int64_t>(s) * a.stride;
  float* S4 = st + static_cast<int64_t>(r0) * DV;
  float* z = st + static_cast<int64_t>(a.D) * DV + r0;
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
  // Features of this tile's rows: phi_k = prod k[i_r], phi_q = w_m prod q[i_r].
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

  // Fixed-order reductions: over the row groups of a column, and over the block for den.
  red[rs * DV + 4 * c4 + 0] = acc.x;
  red[rs * DV + 4 * c4 + 1] = acc.y;
  red[rs * DV + 4 * c4 + 2] = acc.z;
  red[rs * DV + 4 * c4 + 3] = acc.w;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) dacc += __shfl_xor(dacc, o);
  if ((tid & 63) == 0) dred[tid >> 6] = dacc;
  __syncthreads();
  const int64_t pi = static_cast<int64_t>(s) * a.n_tiles + tile;
  if (tid < DV) {
    float sum = 0.f;
    for (int j = 0; j < RPP; ++j) sum += red[j * DV + tid];
    a.part[pi * DV + tid] = sum;
  }
  if (tid == DV) {
    float sum = 0.f;
    for (int j = 0; j < kDecodeThreads / 64; ++j) sum += dred[j];
    a.partz[pi] = sum;
  }
}

// Sums, in a fixed order, the readout records [t0, t1) of one state: value
// records part[s][t][DV], den records partz[s][t] (nrec records a state).
// Block (g, s) takes the range g of length per; FINAL: out[s] = num / den,
// else the sums become record (s, g) of the next level (nxt, nxtz).  One
// block of kRedThreads: groups of DV/4 threads sum interleaved records
// (float4 columns, 8 loads in flight), then a fixed-order combine.
constexpr int kRedThreads = 1024;
template <int DV, bool FINAL>
__global__ __launch_bounds__(kRedThreads) void decode_reduce(const float* __restrict__ part_in,
                                                             const float* __restrict__ partz_in, int nrec,
                                                             int per, float* nxt, float* nxtz, float* out) {
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
  const float4* part = reinterpret_cast<const float4*>(part_in + static_cast<int64_t>(s) * nrec * DV);
  const float* partz = partz_in + static_cast<int64_t>(s) * nrec;
  {
    float z = 0.f;
    for (int t = t0 + tid; t < t1; t += kRedThreads) z += partz[t];
    dz[tid] = z;
  }
  if (grp < G) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    int t = t0 + grp;
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
  if (a.groups <= 1) {
    decode_reduce<D, true><<<dim3(1, a.S), kRedThreads, 0, st>>>(a.part, a.partz, a.n_tiles, a.n_tiles, nullptr,
                                                                 nullptr, a.out);
    return hipGetLastError();
  }
  // Few states: the tiles of a state are split over `groups` blocks, whose
  // sums a second pass combines (in group order).
  const int per = (a.n_tiles + a.groups - 1) / a.groups;
  decode_reduce<D, false><<<dim3(a.groups, a.S), kRedThreads, 0, st>>>(a.part, a.partz, a.n_tiles, per, a.part2,
                                                                       a.partz2, nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  decode_reduce<D, true><<<dim3(1, a.S), kRedThreads, 0, st>>>(a.part2, a.partz2, a.groups, a.groups, nullptr,
                                                               nullptr, a.out);
  return hipGetLastError();
}

}  // namespace

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
