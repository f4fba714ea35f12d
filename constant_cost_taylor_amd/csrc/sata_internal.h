// Internal declarations shared by the host library (sata_host.cpp) and the
// HIP kernels (sata_prefill.hip, sata_decode.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>

namespace sata {

// Waves per prefill workgroup of the fp32 scan (and of the intra-window and
// reduce kernels).
constexpr int kWaves = 4;

// Waves per prefill scan workgroup: the bf16 scan runs two waves per SIMD so
// one wave's LDS traffic and operand building overlap the other's MFMAs.
constexpr int prefill_waves(bool bf16) { return bf16 ? 8 : kWaves; }

// Threads of every decode / prefill-reduce block.
constexpr int kThreads = 256;

// Decode tiles: blocks of kDecodeThreads threads, kDecodeU rows of d_v
// floats per thread (one float4 per thread and row).  Small one-shot blocks
// stream a read-modify-write faster than long-running ones on this part
// (decode step, 256 states at d = 64: 128 threads x 2 rows 1.027 ms; 256 x 2
// 1.054; 512 x 2 1.054; 128 x 3 1.121; 128 x 4 1.094; 512-row tiles looping
// over their rows 1.200).
constexpr int kDecodeU = 2;
constexpr int kDecodeThreads = 128;
constexpr int decode_rows(int dv) {
  // at most one row per thread (features and z are one row a thread)
  int u = kDecodeU;
  while (u > 1 && u * (kDecodeThreads / (dv / 4)) > kDecodeThreads) --u;
  return u * (kDecodeThreads / (dv / 4));
}

// Tokens per prefill chunk: 64 for bf16 inputs (the readout operand of the
// state is refreshed once per chunk, so longer chunks amortise it), 32 for
// fp32 inputs (fp32 cross-wave buffers would not fit LDS at 64).
constexpr int prefill_chunk(bool bf16) { return bf16 ? 64 : 32; }

// Tokens per readout window: the readout of every chunk in a window uses the
// state as it stood at the window's start (for bf16 inputs, whose readout
// operand is a 16-bit copy of the state refreshed once per window), and the
// keys of the window before the query are summed exactly by the intra-window
// kernel.  fp32 inputs read the live state, so their window is one chunk.
constexpr int prefill_window(bool bf16) { return bf16 ? 512 : prefill_chunk(bf16); }

// Row blocks of 16 rows per wave held on chip by the prefill scan, per
// (head dim, input dtype).  fp32 (one wave per SIMD): the state tile
// (rb * column blocks * 4 registers) plus the readout accumulators fit the
// 256 accumulator registers of a lane; at d = 16 two blocks (128-row tiles)
// rather than four: the same speed at 256 heads, and twice the workgroups
// for small batches (32 heads x 4096 tokens: 0.70 -> 0.575 ms).  bf16 (two
// waves per SIMD): state, its bf16 copy and the working set fit 256
// registers per lane.
constexpr int prefill_rb(int d, bool bf16) {
  return bf16 ? (d >= 16 ? 4 : 2) : (d >= 32 ? 8 : d == 16 ? 2 : 1);
}
// fp32 inputs, batches of few heads: a second tiling with one row block a
// wave at d = 16 (64-row tiles, twice the workgroups, two of them sharing a
// CU; 32 heads x 4096 tokens 0.533 -> 0.449 ms, while 256 heads run
// 2.31 -> 2.61 ms and keep the default); 0 where none is built.
constexpr int prefill_rb_small(int d) { return d == 16 ? 1 : 0; }
// The small tiling serves a call whose default tiling gives fewer than this
// many workgroups (two per CU of the 256).
constexpr int kSmallGridWorkgroups = 512;

// Runs of four rows per tile and the cap on distinct parent multisets per
// tile (the per-chunk parent-feature tables are sized by it), for rb row
// blocks a wave.
constexpr int prefill_runs_per_tile_rb(int rb, bool bf16) { return 4 * rb * prefill_waves(bf16); }
constexpr int prefill_slots_rb(int rb, bool bf16) {
  // bf16 scan: 64 slots x 8 token groups = one item per thread of its 512
  return prefill_runs_per_tile_rb(rb, bf16) < (bf16 ? 64 : 80) ? prefill_runs_per_tile_rb(rb, bf16) : (bf16 ? 64 : 80);
}
constexpr int prefill_runs_per_tile(int d, bool bf16) { return prefill_runs_per_tile_rb(prefill_rb(d, bf16), bf16); }
constexpr int prefill_slots(int d, bool bf16) { return prefill_slots_rb(prefill_rb(d, bf16), bf16); }

// LDS row stride (floats) of the key / parent-feature tables.
constexpr int prefill_kstride(bool bf16) { return prefill_chunk(bf16) + 4; }

// Readout records are 16-bit for bf16 inputs at d >= 32 (f16 with a
// per-chunk scale on the f16 operand path, bf16 on the bf16 operand path;
// half the record traffic of fp32), fp32 otherwise.
constexpr bool prefill_bf16_records(int d, bool bf16) { return bf16 && d >= 32; }

// Floats between consecutive heads' states: the state size rounded up to a
// multiple of 64 floats, so every head's S rows start 256-byte aligned.
constexpr int64_t state_stride(int64_t state_floats) { return (state_floats + 63) & ~int64_t(63); }

// Padded widths of the per-token readout records (value columns + den).
constexpr int padded_dv(int dv) { return (dv + 1 + 3) & ~3; }
// Column blocks of 16 (value columns plus the z column).
constexpr int col_blocks(int dv) { return (dv + 1 + 15) / 16; }

// One internal tile layout of the prefill scan (device arrays).  Two
// encodings.  float32 inputs:
//   kside[tile][wave][rb][16]: LDS offsets (floats) used by lane row j of a
//       row block to build its key features: low 16 bits = parent row of the
//       parent-feature table, high 16 bits = child row of the key table.
//   qside[tile][wave][rb][4]: parent slot (low 16 bits) and first child index
//       (high 16 bits) of the run held by lane group g.
//   rowinfo[tile][wave][rb][16]: (canonical row + 1) | (count << 28), 0 = pad.
//   parents[tile][slot]: i1 | i2 << 8 | i3 << 16 | order << 24 of each
//       parent slot (order <= 3, unused indices zero);
//   pweight[tile][slot]: 1 / prod(count!) of that parent (query side);
//   kscale[tile][slot]: factor of the key-side parent feature (1, or 1/3 for
//       the slot that feeds the (i, i, i) rows).
// bfloat16 inputs (key table rows: d key rows, a zero row, a ones row, then
// one row per parent slot of order 2 or 3):
//   kside: key-table row of the parent feature (low 16 bits) and of the
//       child coordinate (high 16 bits) of lane row j;
//   qside: i1 | i2 << 8 | c0 << 16 | i3 << 24 of the run of lane group g
//       (index d = the constant 1);
//   rowinfo: canonical row + 1, 0 = pad;  rweight: w_m of the row computed
//       with c' = c 2^-ec in place of c (0 = pad), the queries being staged
//       times 2^-ec;
//   parents[tile][slot]: key-table rows r1 | r2 << 8 | r3 << 16 of the
//       factors of each parent slot (r3 = the ones row for order 2).
// Both: nslot[tile] = number of parent slots of the tile.
struct PrefillLayout {
  int rb = 0;
  int n_tiles = 0;
  uint32_t* kside = nullptr;
  uint32_t* qside = nullptr;
  uint32_t* rowinfo = nullptr;
  uint32_t* parents = nullptr;
  float* pweight = nullptr;
  float* kscale = nullptr;
  float* rweight = nullptr;
  int32_t* nslot = nullptr;
};

// Token slices of the max-abs pre-pass of the bf16 prefill (per head).
constexpr int kAmaxSplit = 32;

// Prefill workspace of one window of nw tokens (nwp = nw rounded up to 64).
// float32 inputs:
//   rec:   [BH][n_tiles][DVP][nwp]  per-tile readout records (fp32)
//   intra: [BH][DVP][nwp]           intra-chunk records (fp32)
//   carry: [BH][nchunks][DVP]       order-0 prefix at each chunk start (fp32)
// bfloat16 inputs:
//   rec:   [BH][n_tiles][nwp][DV]   per-tile readout records of the value
//                                   columns (16-bit at d >= 32: f16 for heads
//                                   on the f16 operand path, else bf16; fp32
//                                   below d = 32)
//   recs:  [BH][nwp/64][n_tiles]    scale of each 64-token chunk of f16
//                                   records (d >= 32)
//   recz:  [BH][n_tiles][nwp]       per-tile den records (fp32)
//   intra: [BH][nwp][DVP]           intra-window records (fp32)
//   carry: [BH][nrwin][DVP]         order-0 prefix at each readout window start (fp32)
//   amax:  [BH][kAmaxSplit][4]      max |q|, |k|, |v| per token slice
//   stg:   [BH][nwp/64][4][DK][64]  staged 16-bit tables of each 64-token chunk
//   vsum:  [BH][nwp/64][DVP]        sum of v per chunk (fp32), token count at DV
struct PrefillWs {
  void* rec;
  float* intra;
  float* carry;
  float* amax;
  int nwp;
  float* recz;
  uint16_t* stg;
  float* vsum;
  float* recs;
};

struct ScanArgs {
  const void* q;
  const void* k;
  const void* v;
  float* state;          // [BH][stride]
  int64_t stride;        // floats between consecutive heads' states
  PrefillWs ws;
  PrefillLayout lay;
  int64_t n_total;       // tokens per head in q/k/v/out
  int64_t t0;            // first token of this window
  int nw;                // tokens in this window
  int D;                 // total basis rows (incl. order 0)
  float inv_c;           // 1 / c
  int P;                 // orders 0..P-1
  const int32_t* lens;   // [BH] tokens of each head (device), or null: n_total for every head
  int ec;                // c = c' 2^ec, c' in [1, 2): bf16 inputs fold 2^-ec into the staged queries
  int state_only;        // bf16 scan: update the state only (no readout, no records)
};

struct IntraArgs {
  const void* q;
  const void* k;
  const void* v;
  PrefillWs ws;
  int64_t n_total;
  int64_t t0;
  int nw;
  int P;
  float inv_c;
  const int32_t* lens;
};

struct ReduceArgs {
  PrefillWs ws;
  float* out;            // [BH][n_total][dv]
  int64_t n_total;
  int64_t t0;
  int nw;
  int n_tiles;
  float inv_c;           // 1 / c
  int P;                 // orders 0..P-1 (with the max-abs values, selects the bf16 scan's operand type)
  const int32_t* lens;
  int ec;                // as in ScanArgs
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  float* state;          // [S][stride]
  int64_t stride;        // floats between consecutive states
  float* part;           // [S][n_tiles][dv]  readout partials of the value columns (fp32 records)
  float* partz;          // [S][n_tiles]      readout partials of den
  float* out;            // [S][dv]
  const uint32_t* rows;  // packed multiset of every row
  const float* weight;   // w_m of every row
  int S;
  int D;
  int n_tiles;
  int groups;            // reduce blocks per state (1: one pass)
  float* part2;          // [S][groups][dv]   second-level partials (groups > 1)
  float* partz2;         // [S][groups]
  // 16-bit records (bf16 inputs): value partials of tiles >= lo_t as f16
  // times a per-tile power of two, those of the first lo_t tiles (the rows
  // of orders 0 and 1) in fp32; part is unused then.
  uint16_t* part16;      // [S][n_tiles][dv]  (tiles < lo_t unused)
  float* psc;            // [S][n_tiles]      scale of each f16 record
  float* partlo;         // [S][lo_t][dv]
  int lo_t;
};

// Decode tiles whose rows include orders 0 and 1 (rows [0, 1 + d)): their
// readout partials carry most of the output and stay fp32 in the 16-bit
// record format.
constexpr int decode_lo_tiles(int d) { return (1 + d + decode_rows(d) - 1) / decode_rows(d); }

// Reduce blocks per decode state: enough to give the chip about 256 blocks
// when there are few states, each summing at least 256 tile records (a
// second pass then combines the groups); one when S >= 256.
constexpr int decode_groups(int S, int tiles) {
  const int want = (256 + S - 1) / S;
  const int cap = tiles / 256;
  const int g = want < cap ? want : cap;
  return g > 1 ? g : 1;
}

// Launchers (defined in the .hip translation units).  Return hipSuccess or
// the launch error.
hipError_t launch_prefill_scan(int d, bool bf16, int BH, const ScanArgs& a, hipStream_t s);
hipError_t launch_prefill_intra(int d, bool bf16, int BH, const IntraArgs& a, hipStream_t s);
hipError_t launch_prefill_reduce(int d, bool bf16, int BH, const ReduceArgs& a, hipStream_t s);
hipError_t launch_decode(int d, bool bf16, const DecodeArgs& a, hipStream_t s);

// Mixed-precision decode state: rows of orders 0 and 1 of S fp32, rows of
// order >= 2 f16 in tiles of mixed_rows(dv) rows (two 16-byte slots of eight
// halves per thread of a kDecodeThreads block, at most one row per thread),
// each tile with one power-of-two scale; z fp32.  Bytes of one state, from
// its base: [lo][dv] fp32 rows, then off_h: [D - lo][dv] f16 rows, then
// off_z: [D] fp32, then off_sc: [nt16] fp32 tile scales; stride_bytes apart.
constexpr int mixed_rows(int dv) {
  return 2 * (kDecodeThreads / (dv / 8)) > kDecodeThreads ? kDecodeThreads : 2 * (kDecodeThreads / (dv / 8));
}

struct MixedDecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  unsigned char* state;  // [S][stride_bytes]
  int64_t stride_bytes;
  int64_t off_h, off_z, off_sc;
  float* part;           // [S][n_tiles][dv]
  float* partz;          // [S][n_tiles]
  float* out;            // [S][dv]
  const uint32_t* rows;
  const float* weight;
  int S;
  int D;
  int lo;                // rows of orders 0 and 1 (fp32)
  int nt32;              // fp32 tiles (decode_rows rows each)
  int nt16;              // f16 tiles (mixed_rows rows each)
  int n_tiles;           // nt32 + nt16
  int groups;
  float* part2;
  float* partz2;
  // 16-bit records (bf16 inputs), as for DecodeArgs; lo_t = nt32
  uint16_t* part16;
  float* psc;
  float* partlo;
  int lo_t;
};

struct MixedConvArgs {
  float* state;          // fp32 states [S][stride]
  int64_t stride;
  unsigned char* mixed;  // mixed states [S][stride_bytes]
  int64_t stride_bytes;
  int64_t off_h, off_z, off_sc;
  int S;
  int D;
  int lo;
  int nt16;
};

hipError_t launch_decode_mixed(int d, bool bf16, const MixedDecodeArgs& a, hipStream_t s);

// Exact causal softmax attention (the baseline): q, k, v [BH][n][d], out [BH][n][d] fp32.
struct SoftmaxArgs {
  const void* q;
  const void* k;
  const void* v;
  float* out;
  int64_t n;
  float inv_c;
};
hipError_t launch_softmax(int d, bool bf16, int BH, const SoftmaxArgs& a, hipStream_t s);
hipError_t launch_mixed_convert(int d, bool to_mixed, const MixedConvArgs& a, hipStream_t s);

// The allocation-free decode entry point keeps its partial records in a
// file-scope device array of this many bytes (one copy per device, held
// until the process ends).
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
// Device address of that array on the current device (hipGetSymbolAddress).
hipError_t noalloc_scratch_address(void** ptr);
// bfloat16 inputs: max-abs pre-pass, staging, order-0 carry and the scan of
// one call window; then the reduce (after the intra-window kernel).
hipError_t launch_prefill_b16(int d, int BH, const ScanArgs& a, hipStream_t s);
// Segment states of a prefill over sequence segments: nf floats each, T[s]
// at T + s * ts.  copy: dst = src; zero: T[0 .. count) = 0; prefix: T[s] +=
// T[s - 1] for s = 2 .. G - 1, in order.
hipError_t launch_state_copy(float* dst, const float* src, int64_t nf, hipStream_t s);
hipError_t launch_state_zero(float* T, int64_t ts, int count, int64_t nf, hipStream_t s);
hipError_t launch_state_prefix(float* T, int64_t ts, int G, int64_t nf, hipStream_t s);
hipError_t launch_reduce_b16(int d, int BH, const ReduceArgs& a, hipStream_t s);

}  // namespace sata
