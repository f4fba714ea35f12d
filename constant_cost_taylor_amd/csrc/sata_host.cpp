// Host side of the SATA library: minimal-basis and coefficient tables, the
// internal tile layout of the prefill scan, argument validation and dispatch.
//
// Basis (SATA page, section "Core insight: symmetric tensor decomposition"):
// for every order p < P the rows are the multisets i1 <= ... <= ip over
// [0, d) in lexicographic order, concatenated by ascending p; the number of
// index tuples a multiset stands for is mult = p!/prod(count!), and its query
// weight is w = mult / (p! c^p) = 1/(prod(count!) c^p).  The index matrices are
// fixed once d and P are known, so they are built once per handle (section
// "Hardware optimisation path and current limitations" notes they are
// precomputable and nested: every order-p row extends an order-(p-1) row by
// one index not below its last one).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/sata.h"
#include "sata_internal.h"

using sata::PrefillLayout;

struct sata_basis {
  int d = 0;
  int P = 0;
  double c = 1.0;
  int64_t D = 0;
  std::vector<int64_t> offset;               // first row of each order
  std::vector<std::vector<int32_t>> idx;     // per order: rows * p
  std::vector<std::vector<uint32_t>> mult;   // per order
  std::vector<uint32_t> packed;              // per row: i1 | i2<<8 | i3<<16 | p<<24
  std::vector<float> weight;                 // per row: w_m
  int device = -1;
  uint32_t* d_rows = nullptr;
  float* d_weight = nullptr;
  PrefillLayout lay[2];                      // [0] float32 inputs, [1] bfloat16 inputs
  PrefillLayout lay_small;                   // float32 inputs, few heads (rb = 0: none)
  std::vector<void*> allocations;
  void* scratch = nullptr;                   // device address of the no-alloc decode scratch
  int ec = 0;                                // c = c' 2^ec with c' in [1, 2) (bf16 prefill layout)
};

namespace {

bool supported_dim(int d) { return d == 8 || d == 16 || d == 32 || d == 64; }

uint64_t factorial(int n) {
  uint64_t f = 1;
  for (int i = 2; i <= n; ++i) f *= static_cast<uint64_t>(i);
  return f;
}

// Six bits per index (d_k <= 64), order in bits 24..30.
uint32_t pack_multiset(const int32_t* m, int p) {
  uint32_t key = static_cast<uint32_t>(p) << 24;
  for (int r = 0; r < p; ++r) key |= static_cast<uint32_t>(m[r]) << (6 * r);
  return key;
}
int key_index(uint32_t key, int r) { return static_cast<int>((key >> (6 * r)) & 63u); }

// All multisets of size p over [0, d) in lexicographic order.
std::vector<int32_t> enumerate_multisets(int d, int p, int64_t* count) {
  std::vector<int32_t> out;
  std::vector<int32_t> cur(p, 0);
  int64_t n = 0;
  while (true) {
    out.insert(out.end(), cur.begin(), cur.end());
    ++n;
    int r = p - 1;
    while (r >= 0 && cur[r] == d - 1) --r;
    if (r < 0) break;
    const int32_t nv = cur[r] + 1;
    for (int t = r; t < p; ++t) cur[t] = nv;
  }
  *count = n;
  return out;
}

template <typename T>
int upload(sata_basis* b, const std::vector<T>& host, T** dev) {
  *dev = nullptr;
  if (host.empty()) return SATA_OK;
  void* p = nullptr;
  if (hipMalloc(&p, host.size() * sizeof(T)) != hipSuccess) return SATA_ERR_OOM;
  b->allocations.push_back(p);
  if (hipMemcpy(p, host.data(), host.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess)
    return SATA_ERR_HIP;
  *dev = static_cast<T*>(p);
  return SATA_OK;
}

struct Run {
  uint32_t parent_key;   // packed parent multiset (order p-1); bit 31 = key-side 1/3 slot
  float parent_weight;   // 1 / prod(count!) of the parent (query side)
  float kscale;          // factor of the key-side parent feature
  int c0;                // first child index (multiple of 4)
  int64_t row[4];        // canonical row of each child, -1 = masked
  int code[4];           // key table of each child: 0 = masked, 1 = k, 2 = k/2
  int cnt[4];            // multiplicity of the child index in the child row
};

// Runs of four children (P, c0..c0+3) over every parent of order 0..P-2, in
// canonical row order.  With split_iii, a child whose index already occurs
// twice in the parent (the (i, i, i) rows) gets a run of its own, fed by a
// parent slot whose key feature carries the 1/3, so only the k and k/2 tables
// are needed (float32 encoding); otherwise it stays in its parent's run.
std::vector<Run> build_runs(const sata_basis& b, const std::unordered_map<uint32_t, int64_t>& rank,
                            bool split_iii) {
  std::vector<Run> runs;
  for (int p = 1; p < b.P; ++p) {
    const int pp = p - 1;
    const int64_t nparents = static_cast<int64_t>(b.mult[pp].size());
    for (int64_t r = 0; r < nparents; ++r) {
      const int32_t* par = b.idx[pp].data() + r * pp;
      const int lo = pp > 0 ? par[pp - 1] : 0;
      uint64_t cf = 1;   // prod(count!) of the parent
      for (int s = 0; s < pp;) {
        int e = s;
        while (e < pp && par[e] == par[s]) ++e;
        cf *= factorial(e - s);
        s = e;
      }
      auto child_row = [&](int c, int* cnt) {
        int32_t child[4];
        for (int s = 0; s < pp; ++s) child[s] = par[s];
        child[pp] = c;
        int k = 1;
        for (int s = 0; s < pp; ++s) k += (par[s] == c);
        *cnt = k;
        return rank.at(pack_multiset(child, p));
      };
      for (int c0 = (lo / 4) * 4; c0 < b.d; c0 += 4) {
        Run run;
        run.parent_key = pack_multiset(par, pp);
        run.parent_weight = static_cast<float>(1.0 / static_cast<double>(cf));
        run.kscale = 1.f;
        run.c0 = c0;
        bool any = false;
        for (int j = 0; j < 4; ++j) {
          const int c = c0 + j;
          run.row[j] = -1;
          run.code[j] = 0;
          run.cnt[j] = 0;
          if (c < lo) continue;
          int cnt = 0;
          const int64_t row = child_row(c, &cnt);
          if (cnt > 2 && split_iii) continue;   // handled by its own run below
          run.row[j] = row;
          run.code[j] = cnt;
          run.cnt[j] = cnt;
          any = true;
        }
        if (any) runs.push_back(run);
      }
      // The child equal to a twice-repeated last index: k^3/3 = (k^2/3) * k.
      int cnt = 0;
      if (pp >= 2 && split_iii) {
        const int64_t row = child_row(lo, &cnt);
        if (cnt > 2) {
          Run run;
          run.parent_key = pack_multiset(par, pp) | (1u << 31);
          run.parent_weight = static_cast<float>(1.0 / static_cast<double>(cf));
          run.kscale = static_cast<float>(1.0 / cnt);
          run.c0 = (lo / 4) * 4;
          for (int j = 0; j < 4; ++j) {
            run.row[j] = -1;
            run.code[j] = 0;
            run.cnt[j] = 0;
          }
          const int j = lo - run.c0;
          run.row[j] = row;
          run.code[j] = 1;
          run.cnt[j] = cnt;
          runs.push_back(run);
        }
      }
    }
  }
  return runs;
}

// Tile layouts.  Two encodings:
//  * float32 inputs: parent slots for every parent; key side reads a parent
//    table and a separate key table; the query side reads a per-slot table
//    and the scan keeps rows divided by the multiplicity of their last index.
//  * bfloat16 inputs: one key table (d key rows, a zero row, a ones row, then
//    one slot row per parent of order 2 or 3 of the tile); key and query
//    features are plain monomials (the query side from two coordinates, three
//    when P = 5, index d = the constant 1, and the run's four children) and
//    the row weights w_m are applied to the state when the scan rounds it to
//    its readout operand.
int build_layout(sata_basis* b, const std::unordered_map<uint32_t, int64_t>& rank, bool bf16,
                 bool upload_tables, PrefillLayout* lay, int rb) {
  const int per_tile = sata::prefill_runs_per_tile_rb(rb, bf16);
  const int max_slots = sata::prefill_slots_rb(rb, bf16);
  const int kstr = sata::prefill_kstride(bf16);
  const int xk_zero = 2 * b->d * kstr;
  const bool v2 = bf16;
  const int row_zero = b->d, row_ones = b->d + 1, row_slot = b->d + 2;
  lay->rb = rb;
  const std::vector<Run> runs = build_runs(*b, rank, !bf16);
  auto parent_order = [](uint32_t key) { return static_cast<int>((key >> 24) & 0x7f); };
  auto needs_slot = [&](const Run& r) { return !v2 || parent_order(r.parent_key) >= 2; };
  // Greedy tiling in canonical order: a tile takes runs until it is full or
  // one more run would exceed the parent-slot cap.  With P = 1 there are no
  // runs, but one (empty) tile still carries the order-0 row.
  std::vector<std::vector<int>> tiles;
  {
    std::vector<int> cur;
    std::unordered_map<uint32_t, int> keys;
    for (int ri = 0; ri < static_cast<int>(runs.size()); ++ri) {
      const bool new_key = needs_slot(runs[ri]) && keys.find(runs[ri].parent_key) == keys.end();
      if (static_cast<int>(cur.size()) == per_tile ||
          (new_key && static_cast<int>(keys.size()) == max_slots)) {
        tiles.push_back(cur);
        cur.clear();
        keys.clear();
      }
      if (needs_slot(runs[ri])) keys.emplace(runs[ri].parent_key, 0);
      cur.push_back(ri);
    }
    if (!cur.empty() || tiles.empty()) tiles.push_back(cur);
  }
  const int n_tiles = static_cast<int>(tiles.size());
  const int nw = sata::prefill_waves(bf16);
  const size_t nblk = static_cast<size_t>(n_tiles) * nw * rb;
  std::vector<uint32_t> kside(nblk * 16, 0);
  std::vector<uint32_t> qside(nblk * 4, 0);
  std::vector<uint32_t> rowinfo(nblk * 16, 0);
  std::vector<uint32_t> parents(static_cast<size_t>(n_tiles) * max_slots, 0);
  std::vector<float> pweight(static_cast<size_t>(n_tiles) * max_slots, 0.f);
  std::vector<float> kscale(static_cast<size_t>(n_tiles) * max_slots, 0.f);
  std::vector<float> rweight(v2 ? nblk * 16 : 0, 0.f);
  std::vector<int32_t> nslot(n_tiles, 0);
  for (int t = 0; t < n_tiles; ++t) {
    std::unordered_map<uint32_t, int> slot_of;
    for (int u = 0; u < per_tile; ++u) {
      const int w = u / (4 * rb);
      const int bl = (u / 4) % rb;
      const int g = u % 4;
      const size_t blk = (static_cast<size_t>(t) * nw + w) * rb + bl;
      if (u >= static_cast<int>(tiles[t].size())) {
        // Empty run: masked children reading the zero row (parent slot 0, or
        // the ones row / the constant query coordinate).
        for (int j = 0; j < 4; ++j)
          kside[blk * 16 + 4 * g + j] =
              v2 ? static_cast<uint32_t>(row_ones) | (static_cast<uint32_t>(row_zero) << 16)
                 : static_cast<uint32_t>(xk_zero) << 16;
        qside[blk * 4 + g] =
            v2 ? static_cast<uint32_t>(b->d) | (static_cast<uint32_t>(b->d) << 8) | (static_cast<uint32_t>(b->d) << 24)
               : 0u;
        continue;
      }
      const Run& run = runs[tiles[t][u]];
      if (v2) {
        const int pp = parent_order(run.parent_key);
        const int i1 = pp >= 1 ? key_index(run.parent_key, 0) : b->d;
        const int i2 = pp >= 2 ? key_index(run.parent_key, 1) : b->d;
        const int i3 = pp >= 3 ? key_index(run.parent_key, 2) : b->d;
        int prow;
        if (pp == 0) {
          prow = row_ones;
        } else if (pp == 1) {
          prow = i1;
        } else {
          auto it = slot_of.find(run.parent_key);
          int slot;
          if (it == slot_of.end()) {
            slot = static_cast<int>(slot_of.size());
            slot_of.emplace(run.parent_key, slot);
            const size_t si = static_cast<size_t>(t) * max_slots + slot;
            // third factor: the ones row for an order-2 parent
            const int i3r = pp >= 3 ? i3 : row_ones;
            parents[si] = static_cast<uint32_t>(i1) | (static_cast<uint32_t>(i2) << 8) |
                          (static_cast<uint32_t>(i3r) << 16);
          } else {
            slot = it->second;
          }
          prow = row_slot + slot;
        }
        qside[blk * 4 + g] = static_cast<uint32_t>(i1) | (static_cast<uint32_t>(i2) << 8) |
                             (static_cast<uint32_t>(run.c0) << 16) | (static_cast<uint32_t>(i3) << 24);
        for (int j = 0; j < 4; ++j) {
          const int xrow = run.row[j] >= 0 ? run.c0 + j : row_zero;
          kside[blk * 16 + 4 * g + j] = static_cast<uint32_t>(prow) | (static_cast<uint32_t>(xrow) << 16);
          if (run.row[j] >= 0) {
            rowinfo[blk * 16 + 4 * g + j] = static_cast<uint32_t>(run.row[j] + 1);
            // w_m with c' = c 2^-ec (the staged queries carry the 2^-ec)
            const int po = pp + 1;   // order of the child row
            rweight[blk * 16 + 4 * g + j] = static_cast<float>(
                static_cast<double>(b->mult[po][run.row[j] - b->offset[po]]) /
                (static_cast<double>(factorial(po)) * std::pow(std::ldexp(b->c, -b->ec), po)));
          }
        }
        continue;
      }
      auto it = slot_of.find(run.parent_key);
      int slot;
      if (it == slot_of.end()) {
        slot = static_cast<int>(slot_of.size());
        slot_of.emplace(run.parent_key, slot);
        const size_t si = static_cast<size_t>(t) * max_slots + slot;
        {
          const int np = parent_order(run.parent_key);
          uint32_t pw = static_cast<uint32_t>(np) << 24;
          for (int r = 0; r < np; ++r) pw |= static_cast<uint32_t>(key_index(run.parent_key, r)) << (8 * r);
          parents[si] = pw;
        }
        pweight[si] = run.parent_weight;
        kscale[si] = run.kscale;
      } else {
        slot = it->second;
      }
      qside[blk * 4 + g] = static_cast<uint32_t>(slot) | (static_cast<uint32_t>(run.c0) << 16);
      for (int j = 0; j < 4; ++j) {
        const int code = run.code[j];
        const uint32_t pko = static_cast<uint32_t>(slot * kstr);
        const uint32_t xko = code == 0 ? static_cast<uint32_t>(xk_zero)
                                       : static_cast<uint32_t>(((code - 1) * b->d + run.c0 + j) * kstr);
        kside[blk * 16 + 4 * g + j] = pko | (xko << 16);
        if (run.row[j] >= 0)
          rowinfo[blk * 16 + 4 * g + j] =
              static_cast<uint32_t>(run.row[j] + 1) | (static_cast<uint32_t>(run.cnt[j]) << 28);
      }
    }
    // Every tile has at least one parent slot so empty runs read finite
    // features (the bfloat16 encoding needs none).
    nslot[t] = v2 ? static_cast<int32_t>(slot_of.size()) : std::max(1, static_cast<int32_t>(slot_of.size()));
  }
  lay->n_tiles = n_tiles;
  if (!upload_tables) return SATA_OK;
  int st;
  if ((st = upload(b, kside, &lay->kside)) != SATA_OK) return st;
  if ((st = upload(b, qside, &lay->qside)) != SATA_OK) return st;
  if ((st = upload(b, rowinfo, &lay->rowinfo)) != SATA_OK) return st;
  if ((st = upload(b, parents, &lay->parents)) != SATA_OK) return st;
  if ((st = upload(b, pweight, &lay->pweight)) != SATA_OK) return st;
  if ((st = upload(b, kscale, &lay->kscale)) != SATA_OK) return st;
  if ((st = upload(b, rweight, &lay->rweight)) != SATA_OK) return st;
  if ((st = upload(b, nslot, &lay->nslot)) != SATA_OK) return st;
  return SATA_OK;
}

void release(sata_basis* b) {
  if (!b) return;
  if (b->device >= 0) {
    int prev = -1;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(b->device);
    for (void* p : b->allocations) (void)hipFree(p);
    if (prev >= 0) (void)hipSetDevice(prev);
  }
  delete b;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Device address of the no-alloc decode scratch on the current device,
// resolved once per device (nullptr if the lookup failed).
void* scratch_for_current_device() {
  static std::mutex mu;
  static std::vector<std::pair<int, void*>> known;   // (device, address)
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& e : known)
    if (e.first == dev) return e.second;
  void* p = nullptr;
  if (sata::noalloc_scratch_address(&p) != hipSuccess) p = nullptr;
  known.emplace_back(dev, p);
  return p;
}

int check_device(const sata_basis* b) {
  if (b->device < 0 || !b->d_rows) return SATA_ERR_INVALID_ARG;  // host-only handle
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SATA_ERR_HIP;
  return dev == b->device ? SATA_OK : SATA_ERR_INVALID_ARG;
}

// Upper bound on the prefill workspace: 16 GiB, or the byte count in the
// environment variable SATA_PREFILL_WS_CAP, read at every call (the workspace
// query and the prefill call must see the same value).
size_t prefill_ws_cap() {
  const char* e = std::getenv("SATA_PREFILL_WS_CAP");
  if (e && *e) {
    char* end = nullptr;
    const unsigned long long v = std::strtoull(e, &end, 10);
    if (end && *end == 0 && v > 0) return static_cast<size_t>(v);
  }
  return size_t(16) << 30;
}

// How a prefill call is cut: the heads in `groups` groups of at most `heads`
// heads each (sizes differ by at most one), each group's tokens in call
// windows of nw tokens.  Every kernel of the prefill runs once per (group,
// window); the workspace holds one group's records of one window.
struct PrefillPlan {
  int64_t groups = 0;
  int64_t heads = 0;      // heads of the largest group
  int64_t nw = 0;         // tokens per window
  int64_t nwp = 0;        // nw rounded up to 64
  size_t rec_bytes = 0;   // per-tile records
  size_t recz_bytes = 0;  // per-tile den records (bfloat16 inputs)
  size_t intra_bytes = 0;
  size_t carry_bytes = 0;
  size_t amax_bytes = 0;
  size_t stg_bytes = 0;   // staged 16-bit tables (bfloat16 inputs)
  size_t vsum_bytes = 0;  // per-chunk sums of v (bfloat16 inputs)
  size_t recs_bytes = 0;  // per-chunk scales of 16-bit records (bfloat16 inputs, d >= 32)
  size_t total = 0;
  double cost = 0.0;
};

// The prefill tiling of a call over BH heads: for float32 inputs, the small
// tiling when the default one gives too few workgroups to fill the chip.
const PrefillLayout& prefill_layout(const sata_basis* b, int dtype, int64_t BH) {
  const PrefillLayout& lay = b->lay[dtype];
  if (dtype == SATA_F32 && b->lay_small.rb > 0 && BH * lay.n_tiles < sata::kSmallGridWorkgroups)
    return b->lay_small;
  return lay;
}

// Workspace of G heads and windows of nw tokens.
PrefillPlan prefill_sizes(const sata_basis* b, const PrefillLayout& lay, int64_t G, int64_t nw, int dtype) {
  const bool bf16 = dtype == SATA_BF16;
  const int nt = lay.n_tiles;
  const int d = b->d;
  const int dvp = sata::padded_dv(d);
  const int T = sata::prefill_window(bf16);
  const size_t rec_elt = sata::prefill_bf16_records(d, bf16) ? 2 : 4;
  PrefillPlan pl;
  pl.heads = G;
  pl.nw = nw;
  pl.nwp = (nw + 63) / 64 * 64;
  pl.rec_bytes = static_cast<size_t>(G) * nt * (bf16 ? d : dvp) * pl.nwp * rec_elt;
  pl.recz_bytes = bf16 ? static_cast<size_t>(G) * nt * pl.nwp * 4 : 0;
  pl.intra_bytes = static_cast<size_t>(G) * dvp * pl.nwp * 4;
  pl.carry_bytes = static_cast<size_t>(G) * ((pl.nwp + T - 1) / T) * dvp * 4;
  pl.amax_bytes = bf16 ? static_cast<size_t>(G) * sata::kAmaxSplit * 4 * 4 : 0;
  pl.stg_bytes = bf16 ? static_cast<size_t>(G) * pl.nwp * 4 * d * 2 : 0;
  pl.vsum_bytes = bf16 ? static_cast<size_t>(G) * (pl.nwp / 64) * dvp * 4 : 0;
  pl.recs_bytes = rec_elt == 2 ? static_cast<size_t>(G) * nt * (pl.nwp / 64) * 4 : 0;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  pl.total = up(pl.rec_bytes) + up(pl.recz_bytes) + up(pl.intra_bytes) + up(pl.carry_bytes) +
             up(pl.amax_bytes) + up(pl.stg_bytes) + up(pl.vsum_bytes) + up(pl.recs_bytes);
  return pl;
}

// Plans of the prefill, in units of one scan chunk of one workgroup: a scan
// launch of g heads runs ceil(g * tiles / 256) rounds of workgroups on the
// 256 compute units; each round costs its chunks plus about 5 for the state
// tile's load and store (once per window); every (group, window) adds about
// 10 for its six launches.  Head groups thus cost only the rounding of the
// rounds, while windows cost a state reload each.  For each group count k the
// longest window that fits `budget` is taken (groups = 0 when not even one
// head and one readout window fit).  Of the plans whose modelled time is
// within (1 + slack) of the least and whose groups each keep the 256 units
// busy for at least 8 rounds (the model ignores the under-filled kernels of
// smaller groups: 4 heads at d = 64 in two groups ran 8 % slower), the one
// with the smallest workspace is returned (ties: the faster); the least-time
// plan always qualifies.  The workspace query passes slack 0.02, so the
// default workspace stays small where more groups cost nothing (256 heads of
// 4096 tokens at d = 64: 2.5 instead of 14.8 GB at the same speed); the call
// passes 0, so a workspace of the queried size selects the same plan and a
// larger one the least-time plan.
PrefillPlan prefill_plan(const sata_basis* b, int64_t BH, int64_t n, int dtype, size_t budget, double slack) {
  const bool bf16 = dtype == SATA_BF16;
  const PrefillLayout& lay = prefill_layout(b, dtype, BH);
  const int64_t nt = lay.n_tiles;
  const int64_t T = sata::prefill_window(bf16);
  const int64_t L = sata::prefill_chunk(bf16);
  constexpr int64_t kCUs = 256;
  constexpr double kStateLoad = 5.0, kLaunches = 10.0;
  const int64_t nround = std::max<int64_t>(64, (n + 63) / 64 * 64);
  const int64_t chunks = (n + L - 1) / L;
  const int64_t m = (nround + T - 1) / T;
  auto window = [&](int64_t i) { return std::min<int64_t>(i * T, nround); };
  std::vector<PrefillPlan> cands;
  double least = 0.0;
  int64_t last_g = -1;
  for (int64_t k = 1; k <= BH; ++k) {
    const int64_t G = (BH + k - 1) / k;
    if (G == last_g) continue;  // same largest group with more launches
    last_g = G;
    // the longest window that fits: min(i T, nround) for the largest i (the
    // workspace grows with the window)
    if (prefill_sizes(b, lay, G, window(1), dtype).total > budget) continue;
    int64_t lo = 1, hi = m;
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) / 2;
      if (prefill_sizes(b, lay, G, window(mid), dtype).total <= budget)
        lo = mid;
      else
        hi = mid - 1;
    }
    const int64_t w = window(lo);
    PrefillPlan pl = prefill_sizes(b, lay, G, w, dtype);
    const int64_t small = BH / k, nbig = BH - small * k;
    const int64_t rounds = nbig * ((G * nt + kCUs - 1) / kCUs) + (k - nbig) * ((small * nt + kCUs - 1) / kCUs);
    const int64_t windows = (n + w - 1) / w;
    pl.groups = k;
    pl.cost = static_cast<double>(rounds) * (static_cast<double>(chunks) + kStateLoad * windows) +
              kLaunches * static_cast<double>(k * windows);
    least = cands.empty() ? pl.cost : std::min(least, pl.cost);
    cands.push_back(pl);
  }
  PrefillPlan best;
  for (const PrefillPlan& pl : cands) {
    const bool filled = pl.groups == 1 || (BH / pl.groups) * nt >= 8 * kCUs;
    if (pl.cost > least * (1.0 + slack) || (pl.cost > least && !filled)) continue;
    if (best.groups == 0 || pl.total < best.total || (pl.total == best.total && pl.cost < best.cost)) best = pl;
  }
  return best;
}

// The prefill kernels of BH heads of n tokens under plan pl (every head
// group and call window), workspace at ws.  state_only (bf16 inputs): the
// state update alone, no outputs.
static int run_plan(const sata_basis* b, const PrefillPlan& pl, const PrefillLayout& lay, int64_t BH, int64_t n,
                    int d_v, bool bf16, const char* q, const char* k, const char* v, const int32_t* lens,
                    float* out, float* state, int64_t stride, char* ws, bool state_only, hipStream_t s) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t off = 0;
  auto carve = [&](size_t bytes) -> char* {
    if (bytes == 0) return nullptr;
    char* p = ws + off;
    off += up(bytes);
    return p;
  };
  sata::PrefillWs pw{};
  pw.rec = carve(pl.rec_bytes);
  pw.intra = reinterpret_cast<float*>(carve(pl.intra_bytes));
  pw.carry = reinterpret_cast<float*>(carve(pl.carry_bytes));
  pw.amax = reinterpret_cast<float*>(carve(pl.amax_bytes));
  pw.nwp = static_cast<int>(pl.nwp);
  pw.recz = reinterpret_cast<float*>(carve(pl.recz_bytes));
  pw.stg = reinterpret_cast<uint16_t*>(carve(pl.stg_bytes));
  pw.vsum = reinterpret_cast<float*>(carve(pl.vsum_bytes));
  pw.recs = reinterpret_cast<float*>(carve(pl.recs_bytes));
  const float inv_c = static_cast<float>(1.0 / b->c);
  const size_t esz = bf16 ? 2 : 4;
  const int64_t small = BH / pl.groups, nbig = BH - small * pl.groups;
  int64_t h0 = 0;
  for (int64_t gi = 0; gi < pl.groups; ++gi) {
    const int64_t G = small + (gi < nbig ? 1 : 0);
    if (G == 0) continue;   // a plan made for more heads than this call has
    const int gh = static_cast<int>(G);
    const char* qg = q + h0 * n * b->d * esz;
    const char* kg = k + h0 * n * b->d * esz;
    const char* vg = v + h0 * n * d_v * esz;
    float* og = out ? out + h0 * n * d_v : nullptr;
    float* sg = state + h0 * stride;
    const int32_t* lg = lens ? lens + h0 : nullptr;
    for (int64_t t0 = 0; t0 < n; t0 += pl.nw) {
      const int w = static_cast<int>(std::min<int64_t>(pl.nw, n - t0));
      sata::IntraArgs ia{qg, kg, vg, pw, n, t0, w, b->P, inv_c, lg};
      sata::ScanArgs sa{qg, kg, vg, sg, stride, pw, lay, n, t0, w, static_cast<int>(b->D), inv_c, b->P, lg, b->ec,
                        state_only ? 1 : 0};
      sata::ReduceArgs ra{pw, og, n, t0, w, lay.n_tiles, inv_c, b->P, lg, b->ec};
      if (bf16) {
        if (sata::launch_prefill_b16(b->d, gh, sa, s) != hipSuccess) return SATA_ERR_HIP;
        if (state_only) continue;
        if (sata::launch_prefill_intra(b->d, true, gh, ia, s) != hipSuccess) return SATA_ERR_HIP;
        if (sata::launch_reduce_b16(b->d, gh, ra, s) != hipSuccess) return SATA_ERR_HIP;
      } else {
        if (sata::launch_prefill_intra(b->d, false, gh, ia, s) != hipSuccess) return SATA_ERR_HIP;
        if (sata::launch_prefill_scan(b->d, false, gh, sa, s) != hipSuccess) return SATA_ERR_HIP;
        if (sata::launch_prefill_reduce(b->d, false, gh, ra, s) != hipSuccess) return SATA_ERR_HIP;
      }
    }
    h0 += G;
  }
  return SATA_OK;
}

// Sequence segments for batches of few heads (bfloat16 inputs, one length for
// every head).  The scan gives each workgroup a tile of one head's basis rows
// for the whole sequence, so a batch of few heads leaves CUs idle however long
// the sequence.  The state composes over token ranges [SATA page, "Engineering
// of constant compute cost": the state is a plain sum over the keys], so each
// head runs as G segments of Ls tokens in parallel:
//   pass 1  state-only scans of segments 0 .. G-2, the first from the head's
//           state, the others from zero: P_1 and the increments dS_s;
//   prefix  P_s = P_{s-1} + dS_{s-1};
//   pass 2  the full prefill of the G segments, segment s from P_s (P_0 the
//           head's state); the last segment's state is the head's new state;
//   tail    the n - G Ls tokens past the segments, a plain continuation.
// Pass 1 repeats the update of all but the last segment (about half a scan's
// cost a token), so segments pay only where they fill idle CUs.  Model, in
// chunk units as in prefill_plan, per head: ceil((G-1) tiles / 256) rounds of
// state-only chunks (0.5 each) and ceil(G tiles / 256) rounds of full chunks
// over Ls tokens, 5 per round for the state tiles, 30 for the launches, plus
// the tail; taken when it beats one launch of all heads by 20 %.  The
// environment variable SATA_PREFILL_SEGMENTS=0 turns segments off.
struct SegPlan {
  int G = 1;              // segments per head (1: none)
  int64_t Ls = 0;         // tokens a segment (a multiple of the 512-token readout window)
  int64_t rest = 0;       // tokens after the G segments
  int64_t ts = 0;         // floats between segment states
  size_t tmp_bytes = 0;   // G segment states
  PrefillPlan inner;      // G segments as heads of Ls tokens
  PrefillPlan tail;       // one head of `rest` tokens
  size_t total = 0;
};

bool segments_enabled() {
  const char* e = std::getenv("SATA_PREFILL_SEGMENTS");
  return !(e && e[0] == '0' && e[1] == 0);
}

SegPlan segment_plan(const sata_basis* b, int64_t BH, int64_t n, int dtype, bool varlen, size_t budget,
                     double slack) {
  SegPlan sp;
  if (dtype != SATA_BF16 || varlen || !segments_enabled()) return sp;
  constexpr int64_t kCUs = 256, T = sata::prefill_window(true), L = sata::prefill_chunk(true);
  const int64_t nt = b->lay[SATA_BF16].n_tiles;
  if (nt < 1 || BH * nt >= kCUs) return sp;
  const double plain = static_cast<double>((BH * nt + kCUs - 1) / kCUs) * ((n + L - 1) / L + 5) + 10;
  double best = 0.8 * plain;
  for (int64_t G = 2; G <= std::min<int64_t>(kCUs / nt, n / T); ++G) {
    const int64_t Ls = T * (n / (T * G));
    const int64_t rest = n - G * Ls;
    const double ch = static_cast<double>(Ls / L);
    double c = static_cast<double>(((G - 1) * nt + kCUs - 1) / kCUs) * (0.5 * ch + 5) +
               static_cast<double>((G * nt + kCUs - 1) / kCUs) * (ch + 5) + 30;
    if (rest > 0) c += static_cast<double>((nt + kCUs - 1) / kCUs) * ((rest + L - 1) / L + 5) + 10;
    c *= static_cast<double>(BH);
    if (c < best) {
      best = c;
      sp.G = static_cast<int>(G);
      sp.Ls = Ls;
      sp.rest = rest;
    }
  }
  if (sp.G == 1) return sp;
  sp.ts = sata::state_stride(static_cast<int64_t>(b->d + 1) * b->D);
  sp.tmp_bytes = (static_cast<size_t>(sp.G) * sp.ts * 4 + 255) / 256 * 256;
  if (sp.tmp_bytes >= budget) return SegPlan{};
  sp.inner = prefill_plan(b, sp.G, sp.Ls, dtype, budget - sp.tmp_bytes, slack);
  if (sp.rest > 0) sp.tail = prefill_plan(b, 1, sp.rest, dtype, budget - sp.tmp_bytes, slack);
  if (sp.inner.groups == 0 || (sp.rest > 0 && sp.tail.groups == 0)) return SegPlan{};
  sp.total = sp.tmp_bytes + std::max(sp.inner.total, sp.rest > 0 ? sp.tail.total : size_t(0));
  return sp;
}

// One head through segments (see segment_plan); q, k, v, out and state point
// at the head.
static int run_segments(const sata_basis* b, const SegPlan& sp, int64_t n, int d_v, const char* q, const char* k,
                        const char* v, float* out, float* state, char* ws, hipStream_t s) {
  const PrefillLayout& lay = b->lay[SATA_BF16];
  const int64_t nf = static_cast<int64_t>(d_v + 1) * b->D;
  float* T = reinterpret_cast<float*>(ws);
  char* inner_ws = ws + sp.tmp_bytes;
  const int G = sp.G;
  // pass 1: segment 0 from the head's state into T[1], segments 1..G-2 from
  // zero into T[2..G-1]
  if (sata::launch_state_copy(T + sp.ts, state, nf, s) != hipSuccess) return SATA_ERR_HIP;
  if (G > 2 && sata::launch_state_zero(T + 2 * sp.ts, sp.ts, G - 2, nf, s) != hipSuccess) return SATA_ERR_HIP;
  PrefillPlan p1 = sp.inner;   // G - 1 of the G segment heads fit the same plan
  int st = run_plan(b, p1, lay, G - 1, sp.Ls, d_v, true, q, k, v, nullptr, nullptr, T + sp.ts, sp.ts, inner_ws,
                    true, s);
  if (st != SATA_OK) return st;
  // prefix: T[s] = P_s for s >= 1
  if (G > 2 && sata::launch_state_prefix(T, sp.ts, G, nf, s) != hipSuccess) return SATA_ERR_HIP;
  // pass 2 from P_0 = the head's state
  if (sata::launch_state_copy(T, state, nf, s) != hipSuccess) return SATA_ERR_HIP;
  st = run_plan(b, sp.inner, lay, G, sp.Ls, d_v, true, q, k, v, nullptr, out, T, sp.ts, inner_ws, false, s);
  if (st != SATA_OK) return st;
  if (sata::launch_state_copy(state, T + static_cast<int64_t>(G - 1) * sp.ts, nf, s) != hipSuccess)
    return SATA_ERR_HIP;
  if (sp.rest == 0) return SATA_OK;
  const int64_t t = static_cast<int64_t>(G) * sp.Ls;
  return run_plan(b, sp.tail, lay, 1, sp.rest, d_v, true, q + t * b->d * 2, k + t * b->d * 2, v + t * d_v * 2,
                  nullptr, out + t * d_v, state, 0, inner_ws, false, s);
}

int decode_tiles(const sata_basis* b) {
  const int rows = sata::decode_rows(b->d);
  return static_cast<int>((b->D + rows - 1) / rows);
}

// Decode workspace regions (sata_decode_step and, with tiles = nt32 + nt16 and
// lo_t = nt32, sata_decode_step_mixed).  fp32 inputs: value records [S][tiles][d_v] and
// den records [S][tiles], fp32.  bf16 inputs (16-bit records): f16 value
// records [S][tiles][d_v], their scales [S][tiles], the fp32 value records of
// the first lo_t tiles [S][lo_t][d_v], den records [S][tiles].  Then, with
// more than one reduce group a state, the fp32 second-level partials
// [S][groups][d_v] and [S][groups].  Each region 256-byte aligned.
struct DecodeWs {
  size_t part = 0, p16 = 0, psc = 0, plo = 0, partz = 0, part2 = 0, partz2 = 0, total = 0;
};
DecodeWs decode_ws_tiles(int S, int tiles, int lo_t, int d_v, bool c16) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const int groups = sata::decode_groups(S, tiles);
  const size_t ST = static_cast<size_t>(S) * tiles;
  DecodeWs w;
  size_t off = 0;
  if (c16) {
    w.p16 = off;
    off += up(ST * d_v * 2);
    w.psc = off;
    off += up(ST * 4);
    w.plo = off;
    off += up(static_cast<size_t>(S) * lo_t * d_v * 4);
  } else {
    w.part = off;
    off += up(ST * d_v * 4);
  }
  w.partz = off;
  off += up(ST * 4);
  if (groups > 1) {
    w.part2 = off;
    off += up(static_cast<size_t>(S) * groups * d_v * 4);
    w.partz2 = off;
    off += up(static_cast<size_t>(S) * groups * 4);
  }
  w.total = off;
  return w;
}
DecodeWs decode_ws(const sata_basis* b, int S, int d_v, bool c16) {
  return decode_ws_tiles(S, decode_tiles(b), sata::decode_lo_tiles(b->d), d_v, c16);
}

// Mixed-precision state layout of one state (bytes from its base).
struct MixedPlan {
  int lo = 0, nt32 = 0, nt16 = 0;
  int64_t off_h = 0, off_z = 0, off_sc = 0, bytes = 0;
};
MixedPlan mixed_plan(const sata_basis* b) {
  auto up = [](int64_t x, int64_t a) { return (x + a - 1) / a * a; };
  MixedPlan m;
  const int64_t d = b->d;
  m.lo = static_cast<int>(std::min<int64_t>(1 + d, b->D));
  const int r32 = sata::decode_rows(b->d), r16 = sata::mixed_rows(b->d);
  m.nt32 = (m.lo + r32 - 1) / r32;
  m.nt16 = static_cast<int>((b->D - m.lo + r16 - 1) / r16);
  m.off_h = up(m.lo * d * 4, 256);
  m.off_z = up(m.off_h + (b->D - m.lo) * d * 2, 256);
  m.off_sc = up(m.off_z + b->D * 4, 256);
  m.bytes = up(m.off_sc + static_cast<int64_t>(m.nt16) * 4, 256);
  return m;
}

}  // namespace

extern "C" {

static int build_basis_impl(int d_k, int P, double c, bool upload_tables, sata_basis** out) {
  if (!out) return SATA_ERR_INVALID_ARG;
  *out = nullptr;
  if (!(std::isfinite(c) && c > 0.0)) return SATA_ERR_INVALID_ARG;
  if (!supported_dim(d_k) || P < 1 || P > 5) return SATA_ERR_UNSUPPORTED;
  sata_basis* b = new (std::nothrow) sata_basis;
  if (!b) return SATA_ERR_OOM;
  b->d = d_k;
  b->P = P;
  b->c = c;
  {
    int e = 0;
    (void)std::frexp(c, &e);   // c = f 2^e, f in [0.5, 1)
    b->ec = (e - 1 >= -30 && e - 1 <= 30) ? e - 1 : 0;
  }
  std::unordered_map<uint32_t, int64_t> rank;
  int64_t total = 0;
  for (int p = 0; p < P; ++p) {
    int64_t cnt = 0;
    b->idx.push_back(enumerate_multisets(d_k, p, &cnt));
    b->offset.push_back(total);
    std::vector<uint32_t> mult(cnt);
    const double scale = 1.0 / (static_cast<double>(factorial(p)) * std::pow(c, p));
    for (int64_t r = 0; r < cnt; ++r) {
      const int32_t* m = b->idx[p].data() + r * p;
      uint64_t den = 1;
      for (int s = 0; s < p;) {
        int e = s;
        while (e < p && m[e] == m[s]) ++e;
        den *= factorial(e - s);
        s = e;
      }
      mult[r] = static_cast<uint32_t>(factorial(p) / den);
      const uint32_t key = pack_multiset(m, p);
      rank.emplace(key, total + r);
      b->packed.push_back(key);
      b->weight.push_back(static_cast<float>(static_cast<double>(mult[r]) * scale));
    }
    b->mult.push_back(std::move(mult));
    total += cnt;
  }
  b->D = total;
  if (!upload_tables) {
    int st = build_layout(b, rank, false, false, &b->lay[0], sata::prefill_rb(d_k, false));
    if (st == SATA_OK) st = build_layout(b, rank, true, false, &b->lay[1], sata::prefill_rb(d_k, true));
    if (st == SATA_OK && sata::prefill_rb_small(d_k) > 0)
      st = build_layout(b, rank, false, false, &b->lay_small, sata::prefill_rb_small(d_k));
    if (st != SATA_OK) {
      release(b);
      return st;
    }
    *out = b;
    return SATA_OK;
  }
  if (hipGetDevice(&b->device) != hipSuccess) {
    b->device = -1;
    release(b);
    return SATA_ERR_HIP;
  }
  int st = upload(b, b->packed, &b->d_rows);
  if (st == SATA_OK) st = upload(b, b->weight, &b->d_weight);
  if (st == SATA_OK) st = build_layout(b, rank, false, true, &b->lay[0], sata::prefill_rb(d_k, false));
  if (st == SATA_OK) st = build_layout(b, rank, true, true, &b->lay[1], sata::prefill_rb(d_k, true));
  if (st == SATA_OK && sata::prefill_rb_small(d_k) > 0)
    st = build_layout(b, rank, false, true, &b->lay_small, sata::prefill_rb_small(d_k));
  if (st != SATA_OK) {
    release(b);
    return st;
  }
  b->scratch = scratch_for_current_device();
  *out = b;
  return SATA_OK;
}

int sata_build_basis(int d_k, int P, double c, sata_basis** out) {
  try {
    return build_basis_impl(d_k, P, c, true, out);
  } catch (...) {
    if (out) *out = nullptr;
    return SATA_ERR_OOM;
  }
}

int sata_build_basis_host(int d_k, int P, double c, sata_basis** out) {
  try {
    return build_basis_impl(d_k, P, c, false, out);
  } catch (...) {
    if (out) *out = nullptr;
    return SATA_ERR_OOM;
  }
}

void sata_free_basis(sata_basis* basis) { release(basis); }

int sata_basis_info(const sata_basis* b, int* d_k, int* P, double* c, int64_t* total_rows) {
  if (!b) return SATA_ERR_INVALID_ARG;
  if (d_k) *d_k = b->d;
  if (P) *P = b->P;
  if (c) *c = b->c;
  if (total_rows) *total_rows = b->D;
  return SATA_OK;
}

int sata_basis_rows(const sata_basis* b, int p, int64_t* rows) {
  if (!b || !rows || p < 0 || p >= b->P) return SATA_ERR_INVALID_ARG;
  *rows = static_cast<int64_t>(b->mult[p].size());
  return SATA_OK;
}

int sata_basis_copy_tables(const sata_basis* b, int p, int32_t* idx, uint32_t* mult) {
  if (!b || p < 0 || p >= b->P) return SATA_ERR_INVALID_ARG;
  if (idx && !b->idx[p].empty()) std::memcpy(idx, b->idx[p].data(), b->idx[p].size() * sizeof(int32_t));
  if (mult) std::memcpy(mult, b->mult[p].data(), b->mult[p].size() * sizeof(uint32_t));
  return SATA_OK;
}

int sata_basis_download_rows(const sata_basis* b, uint32_t* packed, float* weight) {
  if (!b || !packed || !weight) return SATA_ERR_INVALID_ARG;
  if (check_device(b) != SATA_OK) return SATA_ERR_INVALID_ARG;
  if (hipMemcpy(packed, b->d_rows, b->D * sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess)
    return SATA_ERR_HIP;
  if (hipMemcpy(weight, b->d_weight, b->D * sizeof(float), hipMemcpyDeviceToHost) != hipSuccess)
    return SATA_ERR_HIP;
  return SATA_OK;
}

int64_t sata_state_floats(const sata_basis* b, int d_v) {
  if (!b || d_v != b->d) return -1;
  return static_cast<int64_t>(d_v + 1) * b->D;
}

int64_t sata_state_stride(const sata_basis* b, int d_v) {
  const int64_t f = sata_state_floats(b, d_v);
  return f < 0 ? -1 : sata::state_stride(f);
}

int sata_prefill_workspace(const sata_basis* b, int B, int H, int n, int d_v, int dtype, size_t* bytes) {
  if (!b || !bytes || B < 1 || H < 1 || n < 0) return SATA_ERR_INVALID_ARG;
  if (dtype != SATA_F32 && dtype != SATA_BF16) return SATA_ERR_INVALID_ARG;
  if (d_v != b->d) return SATA_ERR_UNSUPPORTED;
  if (n == 0) {
    *bytes = 0;
    return SATA_OK;
  }
  const int64_t BH = static_cast<int64_t>(B) * H;
  const SegPlan sp = segment_plan(b, BH, n, dtype, false, prefill_ws_cap(), 0.02);
  if (sp.G > 1) {
    *bytes = sp.total;
    return SATA_OK;
  }
  const PrefillPlan pl = prefill_plan(b, BH, n, dtype, prefill_ws_cap(), 0.02);
  if (pl.groups == 0) return SATA_ERR_WORKSPACE;
  *bytes = pl.total;
  return SATA_OK;
}

static int prefill_impl(const sata_basis* b, int B, int H, int n, int d_v, int dtype, const void* q,
                        const void* k, const void* v, const int32_t* lens, float* out, float* state,
                        int64_t state_stride, void* ws, size_t ws_bytes, void* stream) {
  if (!b || B < 1 || H < 1 || n < 0) return SATA_ERR_INVALID_ARG;
  if (dtype != SATA_F32 && dtype != SATA_BF16) return SATA_ERR_INVALID_ARG;
  if (d_v != b->d) return SATA_ERR_UNSUPPORTED;
  if (n == 0) return SATA_OK;
  if (!q || !k || !v || !out || !state) return SATA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(state, 4))
    return SATA_ERR_INVALID_ARG;
  if (state_stride < static_cast<int64_t>(d_v + 1) * b->D) return SATA_ERR_INVALID_ARG;
  const int64_t BH = static_cast<int64_t>(B) * H;
  if (BH > 65535) return SATA_ERR_UNSUPPORTED;  // grid y limit
  if (!ws) return SATA_ERR_WORKSPACE;
  const size_t budget = std::min(ws_bytes, prefill_ws_cap());
  const SegPlan sp = segment_plan(b, BH, n, dtype, lens != nullptr, budget, 0.0);
  PrefillPlan pl;
  if (sp.G == 1) {
    pl = prefill_plan(b, BH, n, dtype, budget, 0.0);
    if (pl.groups == 0) return SATA_ERR_WORKSPACE;
  }
  if (!aligned(ws, 256)) return SATA_ERR_INVALID_ARG;
  if (check_device(b) != SATA_OK) return SATA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = dtype == SATA_BF16;
  const char* qc = static_cast<const char*>(q);
  const char* kc = static_cast<const char*>(k);
  const char* vc = static_cast<const char*>(v);
  char* wsc = static_cast<char*>(ws);
  if (sp.G > 1) {
    const size_t esz = 2;
    for (int64_t h = 0; h < BH; ++h) {
      const int st = run_segments(b, sp, n, d_v, qc + h * n * b->d * esz, kc + h * n * b->d * esz,
                                  vc + h * n * d_v * esz, out + h * n * d_v, state + h * state_stride, wsc, s);
      if (st != SATA_OK) return st;
    }
    return SATA_OK;
  }
  return run_plan(b, pl, prefill_layout(b, dtype, BH), BH, n, d_v, bf16, qc, kc, vc, lens, out, state,
                  state_stride, wsc, false, s);
}

int sata_prefill_strided(const sata_basis* b, int B, int H, int n, int d_v, int dtype, const void* q,
                         const void* k, const void* v, float* out, float* state, int64_t state_stride,
                         void* ws, size_t ws_bytes, void* stream) {
  return prefill_impl(b, B, H, n, d_v, dtype, q, k, v, nullptr, out, state, state_stride, ws, ws_bytes, stream);
}

int sata_prefill_varlen(const sata_basis* b, int B, int H, int n, int d_v, int dtype, const void* q,
                        const void* k, const void* v, const int32_t* lengths, float* out, float* state,
                        int64_t state_stride, void* ws, size_t ws_bytes, void* stream) {
  if (n > 0 && (!lengths || !aligned(lengths, 4))) return SATA_ERR_INVALID_ARG;
  return prefill_impl(b, B, H, n, d_v, dtype, q, k, v, lengths, out, state, state_stride, ws, ws_bytes, stream);
}

int sata_prefill(const sata_basis* b, int B, int H, int n, int d_v, int dtype, const void* q,
                 const void* k, const void* v, float* out, float* state, void* ws, size_t ws_bytes,
                 void* stream) {
  if (!b) return SATA_ERR_INVALID_ARG;
  if (d_v != b->d) return SATA_ERR_UNSUPPORTED;
  return sata_prefill_strided(b, B, H, n, d_v, dtype, q, k, v, out, state, sata_state_floats(b, d_v), ws,
                              ws_bytes, stream);
}

int sata_decode_workspace(const sata_basis* b, int S, int d_v, int dtype, size_t* bytes) {
  if (!b || !bytes || S < 0) return SATA_ERR_INVALID_ARG;
  if (dtype != SATA_F32 && dtype != SATA_BF16) return SATA_ERR_INVALID_ARG;
  if (d_v != b->d) return SATA_ERR_UNSUPPORTED;
  *bytes = decode_ws(b, S, d_v, dtype == SATA_BF16).total;
  return SATA_OK;
}

static int decode_check(const sata_basis* b, int S, int d_v, int dtype, const void* q, const void* k,
                        const void* v, const float* out, const float* state, int64_t state_stride) {
  if (!b || S < 0) return SATA_ERR_INVALID_ARG;
  if (dtype != SATA_F32 && dtype != SATA_BF16) return SATA_ERR_INVALID_ARG;
  if (d_v != b->d) return SATA_ERR_UNSUPPORTED;
  if (S == 0) return SATA_OK;
  if (S > 65535) return SATA_ERR_UNSUPPORTED;
  const size_t esz = dtype == SATA_BF16 ? 2 : 4;
  if (!q || !k || !v || !out || !state) return SATA_ERR_INVALID_ARG;
  if (!aligned(q, esz) || !aligned(k, esz) || !aligned(v, esz) || !aligned(out, 16) ||
      !aligned(state, 4))
    return SATA_ERR_INVALID_ARG;
  if (state_stride < static_cast<int64_t>(d_v + 1) * b->D) return SATA_ERR_INVALID_ARG;
  return SATA_OK;
}

// Launches the decode step with its partial records in ws (already checked
// to hold sata_decode_workspace bytes and to be 256-byte aligned).
static int decode_launch(const sata_basis* b, int S, int d_v, int dtype, const void* q, const void* k,
                         const void* v, float* out, float* state, int64_t state_stride, void* ws,
                         void* stream) {
  const int tiles = decode_tiles(b);
  const int groups = sata::decode_groups(S, tiles);
  const bool c16 = dtype == SATA_BF16;
  const DecodeWs w = decode_ws(b, S, d_v, c16);
  char* base = static_cast<char*>(ws);
  auto at = [&](size_t off) { return reinterpret_cast<float*>(base + off); };
  sata::DecodeArgs a{q, k, v, state, state_stride,
                     c16 ? nullptr : at(w.part), at(w.partz), out, b->d_rows, b->d_weight, S,
                     static_cast<int>(b->D), tiles, groups,
                     groups > 1 ? at(w.part2) : nullptr, groups > 1 ? at(w.partz2) : nullptr,
                     c16 ? reinterpret_cast<uint16_t*>(base + w.p16) : nullptr, c16 ? at(w.psc) : nullptr,
                     c16 ? at(w.plo) : nullptr, c16 ? sata::decode_lo_tiles(b->d) : 0};
  if (sata::launch_decode(b->d, dtype == SATA_BF16, a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return SATA_ERR_HIP;
  return SATA_OK;
}

int sata_decode_step_strided(const sata_basis* b, int S, int d_v, int dtype, const void* q, const void* k,
                             const void* v, float* out, float* state, int64_t state_stride, void* ws,
                             size_t ws_bytes, void* stream) {
  int st = decode_check(b, S, d_v, dtype, q, k, v, out, state, state_stride);
  if (st != SATA_OK || S == 0) return st;
  size_t need = 0;
  sata_decode_workspace(b, S, d_v, dtype, &need);
  if (!ws || ws_bytes < need) return SATA_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return SATA_ERR_INVALID_ARG;
  if (check_device(b) != SATA_OK) return SATA_ERR_INVALID_ARG;
  return decode_launch(b, S, d_v, dtype, q, k, v, out, state, state_stride, ws, stream);
}

int sata_decode_step_noalloc(const sata_basis* b, int S, int d_v, int dtype, const void* q, const void* k,
                             const void* v, float* out, float* state, int64_t state_stride, void* stream) {
  int st = decode_check(b, S, d_v, dtype, q, k, v, out, state, state_stride);
  if (st != SATA_OK || S == 0) return st;
  size_t need = 0;
  sata_decode_workspace(b, S, d_v, dtype, &need);
  if (need > sata::kNoAllocScratchBytes) return SATA_ERR_SCRATCH;
  if (check_device(b) != SATA_OK) return SATA_ERR_INVALID_ARG;
  if (!b->scratch) return SATA_ERR_HIP;
  return decode_launch(b, S, d_v, dtype, q, k, v, out, state, state_stride, b->scratch, stream);
}

size_t sata_decode_noalloc_max_bytes(void) { return sata::kNoAllocScratchBytes; }

int sata_softmax_attention(int B, int H, int n, int d, int dtype, double c, const void* q, const void* k,
                           const void* v, float* out, void* stream) {
  if (B < 1 || H < 1 || n < 0 || !(std::isfinite(c) && c > 0.0)) return SATA_ERR_INVALID_ARG;
  if (dtype != SATA_F32 && dtype != SATA_BF16) return SATA_ERR_INVALID_ARG;
  if (!supported_dim(d)) return SATA_ERR_UNSUPPORTED;
  if (n == 0) return SATA_OK;
  const int64_t BH = static_cast<int64_t>(B) * H;
  if (BH > 65535) return SATA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !out) return SATA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return SATA_ERR_INVALID_ARG;
  sata::SoftmaxArgs a{q, k, v, out, n, static_cast<float>(1.0 / c)};
  if (sata::launch_softmax(d, dtype == SATA_BF16, static_cast<int>(BH), a, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return SATA_ERR_HIP;
  return SATA_OK;
}

int64_t sata_mixed_state_bytes(const sata_basis* b, int d_v) {
  if (!b || d_v != b->d) return -1;
  return mixed_plan(b).bytes;
}

static int mixed_convert(const sata_basis* b, int S, int d_v, float* state, int64_t state_stride, void* mixed,
                         bool to_mixed, void* stream) {
  if (!b || S < 0) return SATA_ERR_INVALID_ARG;
  if (d_v != b->d) return SATA_ERR_UNSUPPORTED;
  if (S == 0) return SATA_OK;
  if (S > 65535) return SATA_ERR_UNSUPPORTED;
  if (!state || !mixed || !aligned(state, 4) || !aligned(mixed, 256)) return SATA_ERR_INVALID_ARG;
  if (state_stride < static_cast<int64_t>(d_v + 1) * b->D) return SATA_ERR_INVALID_ARG;
  if (check_device(b) != SATA_OK) return SATA_ERR_INVALID_ARG;
  const MixedPlan m = mixed_plan(b);
  sata::MixedConvArgs a{state, state_stride, static_cast<unsigned char*>(mixed), m.bytes, m.off_h, m.off_z,
                        m.off_sc, S, static_cast<int>(b->D), m.lo, m.nt16};
  if (sata::launch_mixed_convert(b->d, to_mixed, a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return SATA_ERR_HIP;
  return SATA_OK;
}

int sata_state_to_mixed(const sata_basis* b, int S, int d_v, const float* state, int64_t state_stride,
                        void* mixed, void* stream) {
  return mixed_convert(b, S, d_v, const_cast<float*>(state), state_stride, mixed, true, stream);
}

int sata_state_from_mixed(const sata_basis* b, int S, int d_v, const void* mixed, float* state,
                          int64_t state_stride, void* stream) {
  return mixed_convert(b, S, d_v, state, state_stride, const_cast<void*>(mixed), false, stream);
}

int sata_decode_mixed_workspace(const sata_basis* b, int S, int d_v, int dtype, size_t* bytes) {
  if (!b || !bytes || S < 0) return SATA_ERR_INVALID_ARG;
  if (dtype != SATA_F32 && dtype != SATA_BF16) return SATA_ERR_INVALID_ARG;
  if (d_v != b->d) return SATA_ERR_UNSUPPORTED;
  const MixedPlan m = mixed_plan(b);
  *bytes = decode_ws_tiles(S, m.nt32 + m.nt16, m.nt32, d_v, dtype == SATA_BF16).total;
  return SATA_OK;
}

int sata_decode_step_mixed(const sata_basis* b, int S, int d_v, int dtype, const void* q, const void* k,
                           const void* v, float* out, void* mixed, void* ws, size_t ws_bytes, void* stream) {
  if (!b || S < 0) return SATA_ERR_INVALID_ARG;
  if (dtype != SATA_F32 && dtype != SATA_BF16) return SATA_ERR_INVALID_ARG;
  if (d_v != b->d) return SATA_ERR_UNSUPPORTED;
  if (S == 0) return SATA_OK;
  if (S > 65535) return SATA_ERR_UNSUPPORTED;
  const size_t esz = dtype == SATA_BF16 ? 2 : 4;
  if (!q || !k || !v || !out || !mixed) return SATA_ERR_INVALID_ARG;
  if (!aligned(q, esz) || !aligned(k, esz) || !aligned(v, esz) || !aligned(out, 16) || !aligned(mixed, 256))
    return SATA_ERR_INVALID_ARG;
  size_t need = 0;
  sata_decode_mixed_workspace(b, S, d_v, dtype, &need);
  if (!ws || ws_bytes < need) return SATA_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return SATA_ERR_INVALID_ARG;
  if (check_device(b) != SATA_OK) return SATA_ERR_INVALID_ARG;
  const MixedPlan m = mixed_plan(b);
  const int tiles = m.nt32 + m.nt16;
  const int groups = sata::decode_groups(S, tiles);
  const bool c16 = dtype == SATA_BF16;
  const DecodeWs w = decode_ws_tiles(S, tiles, m.nt32, d_v, c16);
  char* base = static_cast<char*>(ws);
  auto at = [&](size_t off) { return reinterpret_cast<float*>(base + off); };
  sata::MixedDecodeArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.state = static_cast<unsigned char*>(mixed);
  a.stride_bytes = m.bytes;
  a.off_h = m.off_h;
  a.off_z = m.off_z;
  a.off_sc = m.off_sc;
  a.part = c16 ? nullptr : at(w.part);
  a.partz = at(w.partz);
  a.out = out;
  a.rows = b->d_rows;
  a.weight = b->d_weight;
  a.S = S;
  a.D = static_cast<int>(b->D);
  a.lo = m.lo;
  a.nt32 = m.nt32;
  a.nt16 = m.nt16;
  a.n_tiles = tiles;
  a.groups = groups;
  a.part2 = groups > 1 ? at(w.part2) : nullptr;
  a.partz2 = groups > 1 ? at(w.partz2) : nullptr;
  a.part16 = c16 ? reinterpret_cast<uint16_t*>(base + w.p16) : nullptr;
  a.psc = c16 ? at(w.psc) : nullptr;
  a.partlo = c16 ? at(w.plo) : nullptr;
  a.lo_t = c16 ? m.nt32 : 0;
  if (sata::launch_decode_mixed(b->d, dtype == SATA_BF16, a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return SATA_ERR_HIP;
  return SATA_OK;
}

int sata_decode_step(const sata_basis* b, int S, int d_v, int dtype, const void* q, const void* k,
                     const void* v, float* out, float* state, void* ws, size_t ws_bytes, void* stream) {
  if (!b) return SATA_ERR_INVALID_ARG;
  if (d_v != b->d) return SATA_ERR_UNSUPPORTED;
  return sata_decode_step_strided(b, S, d_v, dtype, q, k, v, out, state, sata_state_floats(b, d_v), ws,
                                  ws_bytes, stream);
}

const char* sata_status_string(int status) {
  switch (status) {
    case SATA_OK: return "SATA_OK";
    case SATA_ERR_INVALID_ARG: return "SATA_ERR_INVALID_ARG: invalid argument";
    case SATA_ERR_UNSUPPORTED: return "SATA_ERR_UNSUPPORTED: unsupported d_k, d_v or P";
    case SATA_ERR_WORKSPACE: return "SATA_ERR_WORKSPACE: workspace too small";
    case SATA_ERR_HIP: return "SATA_ERR_HIP: HIP runtime or launch failure";
    case SATA_ERR_OOM: return "SATA_ERR_OOM: allocation failed";
    case SATA_ERR_SCRATCH:
      return "SATA_ERR_SCRATCH: the call needs more scratch than the static array of "
             "sata_decode_step_noalloc holds (sata_decode_noalloc_max_bytes)";
    default: return "unknown SATA status";
  }
}

}  // extern "C"
