// Internal declarations shared by the host library (sata_host.cpp) and the
// HIP kernels (sata_prefill.hip, sata_decode.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>

namespace sata {

// Waves per prefill workgroup and tokens per prefill chunk.
constexpr int kWaves = 4;
constexpr int kChunk = 32;

// Rows of one decode tile and threads of every decode / reduce block.
constexpr int kDecodeRows = 1024;
constexpr int kThreads = 256;

// Row blocks of 16 rows per wave held on chip by the prefill scan, per
// (head dim, input dtype).  Sized so that the fp32 state tile plus the readout
// accumulators fit the 512 registers a lane owns at one wave per SIMD.
constexpr int prefill_rb(int d, bool bf16) {
  return d == 64 ? (bf16 ? 12 : 8) : d == 32 ? 8 : d == 16 ? (bf16 ? 8 : 4) : (bf16 ? 2 : 1);
}

// Floats between consecutive heads' states: the state size rounded up to a
// multiple of 64 floats, so every head's S rows start 256-byte aligned.
constexpr int64_t state_stride(int64_t state_floats) { return (state_floats + 63) & ~int64_t(63); }

// LDS row strides of the prefill scan (floats): key / parent-feature tables.
constexpr int kKStride = kChunk + 4;

// Padded widths of the per-token readout records written to the workspace.
constexpr int padded_dv(int dv) { return (dv + 1 + 3) & ~3; }
// Column blocks of 16 (value columns plus the z column).
constexpr int col_blocks(int dv) { return (dv + 1 + 15) / 16; }

// One internal tile layout of the prefill scan (device arrays).
//   kside[tile][wave][rb][16]: LDS dword offsets used by lane row j of a row
//       block to build its key features: low 16 bits = parent row in the
//       parent-feature table, high 16 bits = child row in the scaled key table.
//   qside[tile][wave][rb][4]: parent slot (low 16 bits) and first child index
//       (high 16 bits) of the run held by lane group g.
//   rowinfo[tile][wave][rb][16]: (canonical row + 1) | (count << 28), 0 = pad.
//   parents[tile][slot]: i1 | i2 << 8 | order << 16 of each distinct parent,
//   pweight[tile][slot]: 1 / prod(count!) of that parent.
//   nslot[tile]: number of distinct parents of the tile.
struct PrefillLayout {
  int rb = 0;
  int n_tiles = 0;
  uint32_t* kside = nullptr;
  uint32_t* qside = nullptr;
  uint32_t* rowinfo = nullptr;
  uint32_t* parents = nullptr;
  float* pweight = nullptr;
  int32_t* nslot = nullptr;
};

struct ScanArgs {
  const void* q;
  const void* k;
  const void* v;
  float* state;          // [BH][stride]
  int64_t stride;        // floats between consecutive heads' states
  float* part;           // [BH][n_tiles + 1][nw][DVP]
  PrefillLayout lay;
  int64_t n_total;       // tokens per head in q/k/v/out
  int64_t t0;            // first token of this window
  int nw;                // tokens in this window
  int D;                 // total basis rows (incl. order 0)
  float inv_c;           // 1 / c
};

struct IntraArgs {
  const void* q;
  const void* k;
  const void* v;
  float* part;           // slot n_tiles of [BH][n_tiles + 1][nw][DVP]
  int64_t n_total;
  int64_t t0;
  int nw;
  int n_tiles;
  int P;
  float inv_c;
};

struct ReduceArgs {
  const float* part;
  float* out;            // [BH][n_total][dv]
  int64_t n_total;
  int64_t t0;
  int nw;
  int nslots;            // n_tiles + 1
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  float* state;          // [S][stride]
  int64_t stride;        // floats between consecutive states
  float* part;           // [S][n_tiles][DVP]
  float* out;            // [S][dv]
  const uint32_t* rows;  // packed multiset of every row
  const float* weight;   // w_m of every row
  int S;
  int D;
  int n_tiles;
};

// Launchers (defined in the .hip translation units).  Return hipSuccess or
// the launch error.
hipError_t launch_prefill_scan(int d, bool bf16, int BH, const ScanArgs& a, hipStream_t s);
hipError_t launch_prefill_intra(int d, bool bf16, int BH, const IntraArgs& a, hipStream_t s);
hipError_t launch_prefill_reduce(int d, int BH, const ReduceArgs& a, hipStream_t s);
hipError_t launch_decode(int d, bool bf16, const DecodeArgs& a, hipStream_t s);

}  // namespace sata
