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
  std::vector<void*> allocations;
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
                 bool upload_tables, PrefillLayout* lay) {
  const int rb = sata::prefill_rb(b->d, bf16);
  const int per_tile = sata::prefill_runs_per_tile(b->d, bf16);
  const int max_slots = sata::prefill_slots(b->d, bf16);
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
            rweight[blk * 16 + 4 * g + j] = b->weight[run.row[j]];
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

int check_device(const sata_basis* b) {
  if (b->device < 0 || !b->d_rows) return SATA_ERR_INVALID_ARG;  // host-only handle
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SATA_ERR_HIP;
  return dev == b->device ? SATA_OK : SATA_ERR_INVALID_ARG;
}

// Tokens per prefill window and the workspace it needs (records of one
// window; the window is bounded so that they fit the workspace cap: 16 GiB,
// or the byte count in the environment variable SATA_PREFILL_WS_CAP, read at
// every call, so the workspace query and the prefill call must see the same
// value).
size_t prefill_ws_cap() {
  const char* e = std::getenv("SATA_PREFILL_WS_CAP");
  if (e && *e) {
    char* end = nullptr;
    const unsigned long long v = std::strtoull(e, &end, 10);
    if (end && *end == 0 && v > 0) return static_cast<size_t>(v);
  }
  return size_t(16) << 30;
}

struct PrefillPlan {
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
};

PrefillPlan prefill_plan(const sata_basis* b, int64_t BH, int64_t n, int dtype) {
  const bool bf16 = dtype == SATA_BF16;
  const int nt = b->lay[dtype].n_tiles;
  const int d = b->d;
  const int dvp = sata::padded_dv(d);
  const int T = sata::prefill_window(bf16);
  const size_t rec_elt = sata::prefill_bf16_records(d, bf16) ? 2 : 4;
  // bytes per token of window: records, intra, staged tables, chunk sums
  const size_t per_token =
      bf16 ? static_cast<size_t>(BH) * (nt * (d * rec_elt + 4) + nt / 16 + 1 + dvp * 4 + 8 * d + dvp)
           : static_cast<size_t>(BH) * dvp * (nt * rec_elt + 4);
  int64_t w = static_cast<int64_t>(prefill_ws_cap() / per_token);
  // windows start on readout-window boundaries
  w = std::max<int64_t>(T, (w / T) * T);
  const int64_t nround = std::max<int64_t>(64, (n + 63) / 64 * 64);
  PrefillPlan pl;
  pl.nw = std::min(w, nround);
  pl.nwp = (pl.nw + 63) / 64 * 64;
  pl.rec_bytes = static_cast<size_t>(BH) * nt * (bf16 ? d : dvp) * pl.nwp * rec_elt;
  pl.recz_bytes = bf16 ? static_cast<size_t>(BH) * nt * pl.nwp * 4 : 0;
  pl.intra_bytes = static_cast<size_t>(BH) * dvp * pl.nwp * 4;
  pl.carry_bytes = static_cast<size_t>(BH) * ((pl.nwp + T - 1) / T) * dvp * 4;
  pl.amax_bytes = bf16 ? static_cast<size_t>(BH) * sata::kAmaxSplit * 4 * 4 : 0;
  pl.stg_bytes = bf16 ? static_cast<size_t>(BH) * pl.nwp * 4 * d * 2 : 0;
  pl.vsum_bytes = bf16 ? static_cast<size_t>(BH) * (pl.nwp / 64) * dvp * 4 : 0;
  pl.recs_bytes = rec_elt == 2 ? static_cast<size_t>(BH) * nt * (pl.nwp / 64) * 4 : 0;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  pl.total = up(pl.rec_bytes) + up(pl.recz_bytes) + up(pl.intra_bytes) + up(pl.carry_bytes) +
             up(pl.amax_bytes) + up(pl.stg_bytes) + up(pl.vsum_bytes) + up(pl.recs_bytes);
  return pl;
}

// Decode workspace: value partials [S][tiles][d_v] then den partials
// [S][tiles]; with more than one reduce group a state, then the second-level
// partials [S][groups][d_v] and [S][groups].  Each region 256-byte aligned.
size_t decode_part_bytes(int S, int tiles, int d_v) {
  return (static_cast<size_t>(S) * tiles * d_v * sizeof(float) + 255) / 256 * 256;
}
size_t decode_partz_bytes(int S, int tiles) {
  return (static_cast<size_t>(S) * tiles * sizeof(float) + 255) / 256 * 256;
}

int decode_tiles(const sata_basis* b) {
  const int rows = sata::decode_rows(b->d);
  return static_cast<int>((b->D + rows - 1) / rows);
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
    int st = build_layout(b, rank, false, false, &b->lay[0]);
    if (st == SATA_OK) st = build_layout(b, rank, true, false, &b->lay[1]);
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
  if (st == SATA_OK) st = build_layout(b, rank, false, true, &b->lay[0]);
  if (st == SATA_OK) st = build_layout(b, rank, true, true, &b->lay[1]);
  if (st != SATA_OK) {
    release(b);
    return st;
  }
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
  *bytes = n == 0 ? 0 : prefill_plan(b, static_cast<int64_t>(B) * H, n, dtype).total;
  return SATA_OK;
}

int sata_prefill(const sata_basis* b, int B, int H, int n, int d_v, int dtype, const void* q,
                 const void* k, const void* v, float* out, float* state, void* ws, size_t ws_bytes,
                 void* stream) {
  if (!b || B < 1 || H < 1 || n < 0) return SATA_ERR_INVALID_ARG;
  if (dtype != SATA_F32 && dtype != SATA_BF16) return SATA_ERR_INVALID_ARG;
  if (d_v != b->d) return SATA_ERR_UNSUPPORTED;
  if (n == 0) return SATA_OK;
  if (!q || !k || !v || !out || !state) return SATA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(state, 16))
    return SATA_ERR_INVALID_ARG;
  const int64_t BH = static_cast<int64_t>(B) * H;
  if (BH > 65535) return SATA_ERR_UNSUPPORTED;  // grid y limit
  const PrefillPlan pl = prefill_plan(b, BH, n, dtype);
  if (!ws || ws_bytes < pl.total) return SATA_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return SATA_ERR_INVALID_ARG;
  if (check_device(b) != SATA_OK) return SATA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = dtype == SATA_BF16;
  const PrefillLayout& lay = b->lay[dtype];
  const int64_t stride = sata::state_stride(static_cast<int64_t>(d_v + 1) * b->D);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  char* base = static_cast<char*>(ws);
  size_t off = 0;
  auto carve = [&](size_t bytes) -> char* {
    if (bytes == 0) return nullptr;
    char* p = base + off;
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
  for (int64_t t0 = 0; t0 < n; t0 += pl.nw) {
    const int w = static_cast<int>(std::min<int64_t>(pl.nw, n - t0));
    sata::IntraArgs ia{q, k, v, pw, n, t0, w, b->P, inv_c};
    sata::ScanArgs sa{q, k, v, state, stride, pw, lay, n, t0, w, static_cast<int>(b->D), inv_c, b->P};
    sata::ReduceArgs ra{pw, out, n, t0, w, lay.n_tiles, inv_c, b->P};
    if (bf16) {
      if (sata::launch_prefill_b16(b->d, static_cast<int>(BH), sa, s) != hipSuccess) return SATA_ERR_HIP;
      if (sata::launch_prefill_intra(b->d, true, static_cast<int>(BH), ia, s) != hipSuccess)
        return SATA_ERR_HIP;
      if (sata::launch_reduce_b16(b->d, static_cast<int>(BH), ra, s) != hipSuccess) return SATA_ERR_HIP;
    } else {
      if (sata::launch_prefill_intra(b->d, false, static_cast<int>(BH), ia, s) != hipSuccess)
        return SATA_ERR_HIP;
      if (sata::launch_prefill_scan(b->d, false, static_cast<int>(BH), sa, s) != hipSuccess)
        return SATA_ERR_HIP;
      if (sata::launch_prefill_reduce(b->d, false, static_cast<int>(BH), ra, s) != hipSuccess)
        return SATA_ERR_HIP;
    }
  }
  return SATA_OK;
}

int sata_decode_workspace(const sata_basis* b, int S, int d_v, int dtype, size_t* bytes) {
  if (!b || !bytes || S < 0) return SATA_ERR_INVALID_ARG;
  if (dtype != SATA_F32 && dtype != SATA_BF16) return SATA_ERR_INVALID_ARG;
  if (d_v != b->d) return SATA_ERR_UNSUPPORTED;
  const int tiles = decode_tiles(b);
  const int groups = sata::decode_groups(S, tiles);
  *bytes = decode_part_bytes(S, tiles, d_v) + decode_partz_bytes(S, tiles);
  if (groups > 1) *bytes += decode_part_bytes(S, groups, d_v) + decode_partz_bytes(S, groups);
  return SATA_OK;
}

int sata_decode_step(const sata_basis* b, int S, int d_v, int dtype, const void* q, const void* k,
                     const void* v, float* out, float* state, void* ws, size_t ws_bytes, void* stream) {
  if (!b || S < 0) return SATA_ERR_INVALID_ARG;
  if (dtype != SATA_F32 && dtype != SATA_BF16) return SATA_ERR_INVALID_ARG;
  if (d_v != b->d) return SATA_ERR_UNSUPPORTED;
  if (S == 0) return SATA_OK;
  if (S > 65535) return SATA_ERR_UNSUPPORTED;
  const size_t esz = dtype == SATA_BF16 ? 2 : 4;
  if (!q || !k || !v || !out || !state) return SATA_ERR_INVALID_ARG;
  if (!aligned(q, esz) || !aligned(k, esz) || !aligned(v, esz) || !aligned(out, 16) ||
      !aligned(state, 16))
    return SATA_ERR_INVALID_ARG;
  size_t need = 0;
  sata_decode_workspace(b, S, d_v, dtype, &need);
  if (!ws || ws_bytes < need) return SATA_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return SATA_ERR_INVALID_ARG;
  if (check_device(b) != SATA_OK) return SATA_ERR_INVALID_ARG;
  const int tiles = decode_tiles(b);
  float* part = static_cast<float*>(ws);
  float* partz = reinterpret_cast<float*>(static_cast<char*>(ws) + decode_part_bytes(S, tiles, d_v));
  const int groups = sata::decode_groups(S, tiles);
  char* lvl2 = static_cast<char*>(ws) + decode_part_bytes(S, tiles, d_v) + decode_partz_bytes(S, tiles);
  float* part2 = groups > 1 ? reinterpret_cast<float*>(lvl2) : nullptr;
  float* partz2 = groups > 1 ? reinterpret_cast<float*>(lvl2 + decode_part_bytes(S, groups, d_v)) : nullptr;
  sata::DecodeArgs a{q, k, v, state,
                     sata::state_stride(static_cast<int64_t>(d_v + 1) * b->D),
                     part, partz, out, b->d_rows, b->d_weight, S,
                     static_cast<int>(b->D), tiles, groups, part2, partz2};
  if (sata::launch_decode(b->d, dtype == SATA_BF16, a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return SATA_ERR_HIP;
  return SATA_OK;
}

const char* sata_status_string(int status) {
  switch (status) {
    case SATA_OK: return "SATA_OK";
    case SATA_ERR_INVALID_ARG: return "SATA_ERR_INVALID_ARG: invalid argument";
    case SATA_ERR_UNSUPPORTED: return "SATA_ERR_UNSUPPORTED: unsupported d_k, d_v or P";
    case SATA_ERR_WORKSPACE: return "SATA_ERR_WORKSPACE: workspace too small";
    case SATA_ERR_HIP: return "SATA_ERR_HIP: HIP runtime or launch failure";
    case SATA_ERR_OOM: return "SATA_ERR_OOM: allocation failed";
    default: return "unknown SATA status";
  }
}

}  // extern "C"
