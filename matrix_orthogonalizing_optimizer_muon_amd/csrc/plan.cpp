// Host-side planner of the Muon step (see plan.hpp).
#include "plan.hpp"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <fstream>
#include <map>
#include <sstream>

namespace muon {

namespace {

constexpr uint64_t kAlign = 256;
constexpr uint64_t kDefaultCap = 96ull << 30;   // a third of a 288 GB part
constexpr int kEw = 64;           // elementwise tile edge
constexpr int kOld = 128;         // tile edge of the fp32 (register-staged) kernel
constexpr int kXcds = 8;          // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kCus = 256;
constexpr double kLaunchUs = 4.0; // per-launch cost used by the model

// Tile plans: (sym config, apply config, k-major reads of X in B X).
// Plans 8 and 9 are plans 6 and 5 with 64 x 64 tiles (config 4) for the
// symmetric products.
constexpr TilePlan kTilePlans[10] = {{0, 0, 0}, {0, 1, 0}, {1, 1, 0}, {0, 2, 0}, {0, 3, 0},
                                     {0, 0, 1}, {0, 1, 1}, {1, 1, 1}, {4, 1, 1}, {4, 0, 1}};

uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }
int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// Byte sizes of each buffer of one matrix; returns the total with offsets.
uint64_t layout(const ShapeKey& k, int32_t form, int32_t tile, uint64_t* off, bool* has) {
  int64_t mp64 = 0, np64 = 0;
  padded_dims(k, form, tile, &mp64, &np64);
  const uint64_t mp = (uint64_t)mp64, np = (uint64_t)np64;
  const uint64_t es = k.path ? 2 : 4;
  const uint64_t mn = mp * np, mm = mp * mp;
  uint64_t sizes[kPlanBufs] = {0};
  sizes[bX0] = es * mn;
  sizes[bXT] = 4 * mn;
  // transposed copies of X only where B X reads them (not with k-major reads)
  const bool copies = k.path && !tile_plan(tile).qt;
  if (form == kFormDirect) {
    sizes[bX1] = es * mn;
    sizes[bA] = es * mm;
    sizes[bB] = es * mm;
    if (copies) sizes[bX0T] = sizes[bX1T] = 2 * mn;
  } else {
    sizes[bA] = sizes[bH] = sizes[bQX] = sizes[bQY] = sizes[bT1] = 4 * mm;
    if (k.path) sizes[bQH] = 2 * mm;
    if (copies) sizes[bX0T] = 2 * mn;
  }
  uint64_t cur = 0;
  for (int b = 0; b < kPlanBufs; ++b) {
    if (off) off[b] = sizes[b] ? cur : 0;
    if (has) has[b] = sizes[b] != 0;
    cur = align_up(cur + sizes[b], kAlign);
  }
  return cur;
}

// Hands XCD x the contiguous run [x n / 8, ...) of a list of n items (blocks
// are dealt to the XCDs round-robin: block b runs on XCD b % 8).
void remap_xcd(std::vector<ItemHost>& v) {
  const size_t n = v.size();
  if (n < 2 * kXcds) return;
  std::vector<ItemHost> out(n);
  const size_t per = n / kXcds, rem = n % kXcds;
  for (size_t p = 0; p < n; ++p) {
    const size_t x = p % kXcds, idx = p / kXcds;
    const size_t start = x * per + std::min(x, rem);
    out[p] = v[start + idx];
  }
  v.swap(out);
}

// Deals a launch's items window by window.  The blocks the GPU runs side by
// side are about one window of W = kXcds * per_xcd consecutive block indices
// (per_xcd = the CUs of an XCD times the blocks per CU), so each window takes W
// consecutive list items and XCD x gets per_xcd consecutive ones of them.  The
// whole GPU then works within one or two matrices of the list at a time, whose
// operands stay in the last-level cache, and each XCD on a compact group of
// tiles that share row and column panels in its L2.  (Handing each XCD one
// contiguous run of the whole list instead keeps eight far-apart matrices in
// flight; on launches shaped like the Llama-7B set's, X X^T ran at 934 against
// 1430 TFLOP/s dealt by windows.)  A last, partial window is dealt as one run
// per XCD.
void deal_windows(std::vector<ItemHost>& v, size_t per_xcd) {
  const size_t n = v.size(), W = kXcds * per_xcd;
  if (n < 2 * kXcds || per_xcd == 0) return;
  std::vector<ItemHost> out(n);
  size_t w0 = 0;
  for (; w0 + W <= n; w0 += W)
    for (size_t q = 0; q < W; ++q) out[w0 + q] = v[w0 + (q % kXcds) * per_xcd + q / kXcds];
  if (w0 < n) {
    std::vector<ItemHost> tail(v.begin() + (std::ptrdiff_t)w0, v.end());
    remap_xcd(tail);
    std::copy(tail.begin(), tail.end(), out.begin() + (std::ptrdiff_t)w0);
  }
  v.swap(out);
}

// Tiles of one product in super-tile order: 4 x 8 blocks of output tiles are
// consecutive, so the 32 work items an XCD runs side by side (remap_xcd hands
// each XCD a contiguous run) share 4 row panels and 8 column panels in its L2.
// Products with 16 or more rows of tiles use 16 x 8 blocks: the XCD's next
// waves of 32 items then reuse the same 8 column panels (measured on the
// 4096-row products of a Llama-7B matrix set: 457 against 466 ms per step; the
// smaller sets measured flat or slightly slower with taller blocks).
constexpr int kSuperM = 4, kSuperMTall = 16, kTallRows = 16, kSuperN = 8;

void add_tiles(std::vector<ItemHost>& v, int32_t slot, int32_t ntm, int32_t ntn, bool upper) {
  const int32_t rows = ntm >= kTallRows ? kSuperMTall : kSuperM;
  for (int32_t sm = 0; sm < ntm; sm += rows)
    for (int32_t sn = 0; sn < ntn; sn += kSuperN)
      for (int32_t a = sm; a < std::min(sm + rows, ntm); ++a)
        for (int32_t b = sn; b < std::min(sn + kSuperN, ntn); ++b)
          if (!upper || b >= a) v.push_back({slot, a, b});
}

void add_sym(std::vector<ItemHost>& v, int32_t slot, int64_t m_pad, int edge) {
  const int32_t nt = (int32_t)(m_pad / edge);
  add_tiles(v, slot, nt, nt, true);
}

void add_full(std::vector<ItemHost>& v, int32_t slot, int64_t m_pad, int64_t n_pad, TileShape t) {
  add_tiles(v, slot, (int32_t)(m_pad / t.bm), (int32_t)(n_pad / t.bn), false);
}

double sym_tiles(int64_t m_pad, int edge) {
  const double nt = (double)(m_pad / edge);
  return nt * (nt + 1) / 2;
}

// Per-block rate (flop/s) and blocks per CU of each NT configuration, as measured
// on MI355X for large bf16 products; the fp32 kernel for the fp32 path.
double nt_rate(int cfg) {
  switch (cfg) {
    case 1: return 4.6e12;
    case 2: case 3: return 3.4e12;
    case 4: return 0.8e12;
    default: return 1.8e12;
  }
}
int nt_blocks_per_cu(int cfg) { return cfg == 0 ? 2 : cfg == 4 ? 4 : 1; }
constexpr double kOldRateBf16 = 0.9e12;   // fp32-kernel blocks, bf16 operands
constexpr double kOldRateF32 = 0.25e12;   // fp32-kernel blocks, fp32 operands (per block, 2 per CU)

// Time of one launch of `tiles` blocks each doing `flops_per_tile`.
double launch_us(double tiles, double flops_per_tile, double rate, int per_cu) {
  if (tiles <= 0) return 0;
  const double waves = std::ceil(tiles / (double)(kCus * per_cu));
  return waves * flops_per_tile / rate * 1e6 + kLaunchUs;
}

}  // namespace

TileShape nt_cfg_shape(int cfg) {
  if (cfg < 0 || cfg >= kNtTiles) cfg = 0;
  return kNtTileShapes[cfg];
}

int num_tile_plans() { return (int)(sizeof kTilePlans / sizeof kTilePlans[0]); }

TilePlan tile_plan(int t) {
  if (t < 0 || t >= num_tile_plans()) t = 0;
  return kTilePlans[t];
}

ShapeKey shape_key(int64_t rows, int64_t cols, int32_t dtype, int32_t precision) {
  ShapeKey k;
  k.m = std::min(rows, cols);
  k.n = std::max(rows, cols);
  if (precision == 1) k.path = 0;
  else if (precision == 2) k.path = 1;
  else k.path = dtype == 0 ? 0 : 1;
  return k;
}

void padded_dims(const ShapeKey& k, int32_t form, int32_t tile, int64_t* m_pad, int64_t* n_pad) {
  (void)form;
  int64_t em = kOld, en = kOld;
  if (k.path) {
    const TilePlan tp = tile_plan(tile);
    const TileShape s = nt_cfg_shape(tp.sym), a = nt_cfg_shape(tp.apply);
    em = std::max<int64_t>({em, s.bm, a.bm});
    en = std::max<int64_t>(en, a.bn);
  }
  *m_pad = round_up(k.m, em);
  *n_pad = round_up(k.n, en);
}

bool dims_supported(int64_t rows, int64_t cols) {
  const int64_t m = std::min(rows, cols), n = std::max(rows, cols);
  if (m < 1 || m > 16384 || n > (1 << 20)) return false;
  // every bf16 operand and each fp32 m x m iterate stays under 2^31 bytes
  return round_up(m, 256) * round_up(n, 256) <= (int64_t(1) << 30);
}

uint64_t matrix_ws_bytes(const ShapeKey& k, int32_t form, int32_t tile) {
  return layout(k, form, tile, nullptr, nullptr);
}

std::vector<std::pair<int32_t, int32_t>> candidates(const ShapeKey& k, int32_t forced_form,
                                                    int32_t forced_tile) {
  std::vector<std::pair<int32_t, int32_t>> out;
  const bool dir = forced_form != kFormGram, gram = forced_form != kFormDirect;
  if (!k.path) {
    if (dir) out.push_back({kFormDirect, 0});
    if (gram) out.push_back({kFormGram, 0});
    return out;
  }
  auto want = [&](int t) { return forced_tile < 0 || forced_tile == t; };
  if (dir)
    for (int t = 0; t < num_tile_plans(); ++t)
      if (want(t)) out.push_back({kFormDirect, t});
  if (gram)
    for (int t : {0, 1, 2, 5, 6, 7, 8, 9})
      if (want(t)) out.push_back({kFormGram, t});
  return out;
}

double model_cost_us(const ShapeKey& k, int32_t form, int32_t tile, int count) {
  const int T = 5;
  const double c = std::max(count, 1);
  int64_t mp64 = 0, np64 = 0;
  padded_dims(k, form, tile, &mp64, &np64);
  const double mp = (double)mp64, np = (double)np64;
  double us = 0;
  if (!k.path) {
    // the tile edge the plan takes for a set of c such matrices (64 when their
    // m x n products have fewer 128-tiles than CUs); a 64-block does a quarter
    // of the work at half the per-block rate, four blocks per CU
    const bool small = (mp / kOld) * (np / kOld) * c < kCus;
    const int e = small ? kOld / 2 : kOld;
    const double rate = small ? kOldRateF32 / 2 : kOldRateF32;
    const int per_cu = small ? 4 : 2;
    const double st = sym_tiles(mp64, e) * c, ft = (mp / e) * (np / e) * c;
    const double tf = 2.0 * e * e;
    const double g = launch_us(st, tf * np, rate, per_cu);
    const double sq = launch_us(st, tf * mp, rate, per_cu);
    const double ap = launch_us(ft, tf * mp, rate, per_cu);
    us = form == kFormDirect ? T * (g + sq + ap) : g + ap + (4 * T - 3) * sq;
    return us / c;
  }
  const TilePlan tp = tile_plan(tile);
  const TileShape s = nt_cfg_shape(tp.sym), a = nt_cfg_shape(tp.apply);
  const double st = sym_tiles(mp64, s.bm) * c, ft = (mp / a.bm) * (np / a.bn) * c;
  const double g = launch_us(st, 2.0 * s.bm * s.bn * np, nt_rate(tp.sym), nt_blocks_per_cu(tp.sym));
  // k-major reads: about 10% slower main loop, no X'^T stores; the model
  // rates them slightly behind the transposed copies (timing decides)
  const double ap = launch_us(ft, 2.0 * a.bm * a.bn * mp, nt_rate(tp.apply), nt_blocks_per_cu(tp.apply)) *
                    (tp.qt ? 1.02 : 1.0);
  if (form == kFormDirect) {
    const double sq = launch_us(st, 2.0 * s.bm * s.bn * mp, nt_rate(tp.sym), nt_blocks_per_cu(tp.sym));
    us = T * (g + sq + ap);
  } else {
    const double ost = sym_tiles(mp64, kOld) * c;
    const double sq = launch_us(ost, 2.0 * kOld * kOld * mp, kOldRateBf16 * 0.3, 2);  // fp32 iterates
    us = g + ap + (4 * T - 3) * sq;
  }
  return us / c;
}

ShapeChoice model_choice(const ShapeKey& k, int32_t forced_form, int32_t forced_tile, int count) {
  ShapeChoice best;
  double best_us = 0;
  bool first = true;
  for (const auto& cand : candidates(k, forced_form, forced_tile)) {
    const double us = model_cost_us(k, cand.first, cand.second, count);
    if (first || us < 0.97 * best_us) {
      best.form = cand.first;
      best.tile = cand.second;
      best_us = us;
      first = false;
    }
  }
  best.us = 0;
  best.timed = false;
  return best;
}

std::string build_plan(const std::vector<int64_t>& rows, const std::vector<int64_t>& cols,
                       const std::vector<int32_t>& dtypes, const PlanOptions& opts,
                       const std::map<ShapeKey, ShapeChoice>& choices, PlanHost* out) {
  PlanHost P;
  P.opts = opts;
  const size_t n = rows.size();
  P.mats.resize(n);
  std::map<ShapeKey, std::vector<int32_t>> by_key;
  for (size_t i = 0; i < n; ++i) {
    MatPlan& M = P.mats[i];
    M.rows = rows[i];
    M.cols = cols[i];
    M.dtype = dtypes[i];
    const ShapeKey k = shape_key(rows[i], cols[i], dtypes[i], opts.precision);
    M.path = k.path;
    M.m = k.m;
    M.n = k.n;
    M.trans = rows[i] > cols[i] ? 1 : 0;
    M.s = (float)(opts.rms_scale * std::sqrt((double)k.n));
    by_key[k].push_back((int32_t)i);
  }
  for (auto& kv : by_key) {
    auto it = choices.find(kv.first);
    if (it == choices.end()) return "internal: no choice for a shape key";
    GroupPlan g;
    g.key = kv.first;
    g.form = it->second.form;
    g.tile = kv.first.path ? it->second.tile : 0;
    g.members = kv.second;
    const int32_t gi = (int32_t)P.groups.size();
    // estimated step time of one member: the NS time its shape measured when
    // timed (else the cost model at the group's count) plus its elementwise
    // bytes at 5 TB/s
    const double ns_us = it->second.timed && it->second.us > 0
                             ? it->second.us
                             : model_cost_us(kv.first, g.form, g.tile, (int)g.members.size());
    for (int32_t i : g.members) {
      MatPlan& M = P.mats[i];
      M.form = g.form;
      M.tile = g.tile;
      M.group = gi;
      {
        const double e = (double)M.rows * M.cols, pes = M.dtype ? 2 : 4, es = M.path ? 2 : 4;
        const bool dt = M.path && !tile_plan(g.tile).qt;   // D^T written by the momentum kernel
        const double ew = e * (pes + 8 + es + (dt ? es : 0) + 2 * pes + (M.path ? 0 : 4));
        M.cost_us = ns_us + ew / 5e12 * 1e6;
      }
      padded_dims(kv.first, g.form, g.tile, &M.m_pad, &M.n_pad);
      M.ws_bytes = layout(kv.first, g.form, g.tile, M.off, M.has);
      M.ew_tiles = (M.m_pad / kEw) * (M.n_pad / kEw);
      if (g.form == kFormGram) P.n_gram++;
    }
    P.groups.push_back(std::move(g));
  }
  // chunks under the workspace cap, in group order
  const uint64_t cap = opts.workspace_cap ? opts.workspace_cap : kDefaultCap;
  for (const GroupPlan& g : P.groups) {
    for (int32_t i : g.members) {
      MatPlan& M = P.mats[i];
      if (M.ws_bytes > cap) {
        char msg[160];
        snprintf(msg, sizeof msg, "matrix %d needs %llu workspace bytes, over the cap of %llu", i,
                 (unsigned long long)M.ws_bytes, (unsigned long long)cap);
        return msg;
      }
      if (P.chunks.empty() || P.chunks.back().ws_bytes + M.ws_bytes > cap) P.chunks.emplace_back();
      ChunkPlan& C = P.chunks.back();
      for (int b = 0; b < kPlanBufs; ++b) M.off[b] += C.ws_bytes;
      C.ws_bytes += M.ws_bytes;
      C.ew_tiles += M.ew_tiles;
      M.chunk = (int32_t)(P.chunks.size() - 1);
      C.mats.push_back(i);
    }
  }
  const int32_t lanes = std::min<int32_t>(std::max<int32_t>(opts.lanes, 1), kMaxLanes);
  P.lanes = lanes;
  for (ChunkPlan& C : P.chunks) {
    P.ws_bytes = std::max(P.ws_bytes, C.ws_bytes);
    // lane of each matrix: the chunk's matrices in order, cut where the running
    // NS work crosses multiples of total / lanes (by each matrix's midpoint)
    std::vector<double> work(C.mats.size());
    double total = 0;
    for (size_t k = 0; k < C.mats.size(); ++k) {
      const MatPlan& M = P.mats[C.mats[k]];
      const double m = (double)M.m, nn = (double)M.n;
      work[k] = nn * m * (m + 1) + m * m * (m + 1) + 2.0 * m * m * nn;
      total += work[k];
    }
    double run = 0;
    for (size_t k = 0; k < C.mats.size(); ++k) {
      MatPlan& M = P.mats[C.mats[k]];
      const double mid = run + 0.5 * work[k];
      run += work[k];
      M.lane = total > 0 ? std::min<int32_t>(lanes - 1, (int32_t)(mid * lanes / total)) : 0;
      C.n_lanes = std::max(C.n_lanes, M.lane + 1);
    }
    // fp32-path sets: 128-tiles of their m x n products, which sets the tile edge
    std::map<std::pair<int32_t, int32_t>, int64_t> fp32_tiles;   // (form, lane) -> tiles
    for (int32_t i : C.mats) {
      const MatPlan& M = P.mats[i];
      if (!M.path) fp32_tiles[{M.form, M.lane}] += (M.m_pad / kOld) * (M.n_pad / kOld);
    }
    for (int32_t i : C.mats) {
      const MatPlan& M = P.mats[i];
      LaunchSetPlan* S = nullptr;
      for (LaunchSetPlan& s : C.sets)
        if (s.path == M.path && s.form == M.form && s.lane == M.lane) S = &s;
      if (!S) {
        C.sets.emplace_back();
        S = &C.sets.back();
        S->path = M.path;
        S->form = M.form;
        S->lane = M.lane;
        if (!M.path && fp32_tiles[{M.form, M.lane}] < kCus) S->old_edge = kOld / 2;
      }
      const int32_t slot = (int32_t)S->mats.size();
      S->mats.push_back(i);
      const double m = (double)M.m, nn = (double)M.n, mp = (double)M.m_pad, np = (double)M.n_pad;
      const double fg = nn * m * (m + 1), fs = m * m * (m + 1), fa = 2.0 * m * m * nn;
      S->flops_gram_min += fg;
      S->flops_square_min += fs;
      S->flops_apply_min += fa;
      const double old_tf = 2.0 * kOld * kOld;
      if (M.path) {
        const TilePlan tp = tile_plan(M.tile);
        const TileShape s = nt_cfg_shape(tp.sym), a = nt_cfg_shape(tp.apply);
        add_sym(S->nt_sym[tp.sym], slot, M.m_pad, s.bm);
        add_full(S->nt_full[full_list(tp.apply, tp.qt)], slot, M.m_pad, M.n_pad, a);
        S->fl_gram[tp.sym] += fg;
        S->fl_square[tp.sym] += fs;
        S->fl_apply[full_list(tp.apply, tp.qt)] += fa;
        const double st = sym_tiles(M.m_pad, s.bm);
        S->flops_gram_issued += st * 2.0 * s.bm * s.bn * np;
        S->flops_apply_issued += (mp / a.bm) * (np / a.bn) * 2.0 * a.bm * a.bn * mp;
        if (M.form == kFormDirect) {
          S->flops_square_issued += st * 2.0 * s.bm * s.bn * mp;
        } else {
          add_sym(S->old_sym, slot, M.m_pad, kOld);
          S->flops_square_issued_fp32 += sym_tiles(M.m_pad, kOld) * old_tf * mp;
        }
      } else {
        const int e = S->old_edge;
        const double etf = 2.0 * e * e;
        add_sym(S->old_sym, slot, M.m_pad, e);
        add_full(S->old_full, slot, M.m_pad, M.n_pad, TileShape{e, e});
        S->fl_gram[0] += fg;
        S->fl_square[0] += fs;
        S->fl_apply[0] += fa;
        const double st = sym_tiles(M.m_pad, e);
        S->flops_gram_issued += st * etf * np;
        S->flops_apply_issued += (mp / e) * (np / e) * etf * mp;
        if (M.form == kFormDirect) S->flops_square_issued += st * etf * mp;
        else S->flops_square_issued_fp32 += st * etf * mp;
      }
    }
    for (LaunchSetPlan& S : C.sets) {
      // longest contraction first, then dealt to the XCDs window by window
      auto kn = [&](const ItemHost& it) { return P.mats[S.mats[it.slot]].n_pad; };
      auto km = [&](const ItemHost& it) { return P.mats[S.mats[it.slot]].m_pad; };
      // blocks per CU: the NT configuration's, two of the 128-edge fp32
      // kernel, four of its 64-edge variant
      const size_t cus_per_xcd = kCus / kXcds;
      const size_t old_per_cu = S.old_edge == kOld ? 2 : 4;
      std::vector<std::pair<std::vector<ItemHost>*, size_t>> sym{{&S.old_sym, old_per_cu}},
          full{{&S.old_full, old_per_cu}};
      for (int c = 0; c < kNtTiles; ++c) sym.push_back({&S.nt_sym[c], (size_t)nt_blocks_per_cu(c)});
      for (int c = 0; c < 2 * kNtTiles; ++c)
        full.push_back({&S.nt_full[c], (size_t)nt_blocks_per_cu(c % kNtTiles)});
      for (auto& vp : sym) {
        std::stable_sort(vp.first->begin(), vp.first->end(),
                         [&](const ItemHost& x, const ItemHost& y) { return kn(x) > kn(y); });
        deal_windows(*vp.first, cus_per_xcd * vp.second);
      }
      for (auto& vp : full) {
        std::stable_sort(vp.first->begin(), vp.first->end(),
                         [&](const ItemHost& x, const ItemHost& y) { return km(x) > km(y); });
        deal_windows(*vp.first, cus_per_xcd * vp.second);
      }
    }
  }
  *out = std::move(P);
  return "";
}

std::string serialize_plan(const PlanHost& p) {
  std::ostringstream o;
  o << "muon-plan v4\n";
  o << "opts nesterov=" << p.opts.nesterov << " eps=" << std::hexfloat << p.opts.eps
    << " rms=" << p.opts.rms_scale << std::defaultfloat << " precision=" << p.opts.precision
    << " form=" << p.opts.form << " tile=" << p.opts.tile << " cap=" << p.opts.workspace_cap
    << " lanes=" << p.lanes << "\n";
  for (size_t i = 0; i < p.mats.size(); ++i) {
    const MatPlan& M = p.mats[i];
    o << "mat " << i << " " << M.rows << "x" << M.cols << " dtype=" << M.dtype << " path=" << M.path
      << " trans=" << M.trans << " pad=" << M.m_pad << "x" << M.n_pad << " form=" << M.form
      << " tile=" << M.tile << " group=" << M.group << " chunk=" << M.chunk << " lane=" << M.lane
      << " ws=" << M.ws_bytes
      << " off=" << M.off[0] << "\n";
  }
  for (size_t g = 0; g < p.groups.size(); ++g) {
    const GroupPlan& G = p.groups[g];
    o << "group " << g << " m=" << G.key.m << " n=" << G.key.n << " path=" << G.key.path
      << " form=" << G.form << " tile=" << G.tile << " members=" << G.members.size() << "\n";
  }
  for (size_t c = 0; c < p.chunks.size(); ++c) {
    const ChunkPlan& C = p.chunks[c];
    o << "chunk " << c << " mats=" << C.mats.size() << " ws=" << C.ws_bytes << " ew_tiles=" << C.ew_tiles
      << " lanes=" << C.n_lanes << "\n";
    for (const LaunchSetPlan& S : C.sets) {
      o << " set path=" << S.path << " form=" << S.form << " lane=" << S.lane << " mats=" << S.mats.size()
        << " edge=" << S.old_edge << " items=";
      for (int c = 0; c < kNtTiles; ++c)
        o << S.nt_sym[c].size() << "/" << S.nt_full[c].size() << "/" << S.nt_full[c + kNtTiles].size() << ",";
      o << S.old_sym.size() << "/" << S.old_full.size() << " order=";
      uint64_t h = 1469598103934665603ull;
      auto mix = [&](int32_t v) { for (int b = 0; b < 4; ++b) { h ^= (uint8_t)(v >> (8 * b)); h *= 1099511628211ull; } };
      std::vector<const std::vector<ItemHost>*> lists;
      for (int c = 0; c < kNtTiles; ++c) {
        lists.push_back(&S.nt_sym[c]);
        lists.push_back(&S.nt_full[c]);
        lists.push_back(&S.nt_full[c + kNtTiles]);
      }
      lists.push_back(&S.old_sym);
      lists.push_back(&S.old_full);
      for (const std::vector<ItemHost>* v : lists)
        for (const ItemHost& it : *v) { mix(it.slot); mix(it.tm); mix(it.tn); }
      o << std::hex << h << std::dec << "\n";
    }
  }
  return o.str();
}

uint64_t fnv1a(const std::string& s) {
  uint64_t h = 1469598103934665603ull;
  for (unsigned char c : s) {
    h ^= c;
    h *= 1099511628211ull;
  }
  return h;
}

TuneCache read_cache(const std::string& path, const std::string& device_tag) {
  TuneCache out;
  if (path.empty()) return out;
  std::ifstream f(path);
  std::string line;
  while (std::getline(f, line)) {
    std::istringstream is(line);
    std::string magic, tag;
    if (!(is >> magic >> tag) || magic != "muon-tune-v4" || tag != device_tag) continue;
    ShapeKey k{-1, -1, -1};
    ShapeChoice c;
    c.form = -1;
    c.tile = -1;
    std::string set, kv;
    bool bad = false, have_tile = false;
    int32_t lanes = 1;
    while (is >> kv) {
      const size_t eq = kv.find('=');
      if (eq == std::string::npos) { bad = true; break; }
      const std::string key = kv.substr(0, eq), val = kv.substr(eq + 1);
      if (key == "set") {
        set = val;
        continue;
      }
      char* end = nullptr;
      const double v = std::strtod(val.c_str(), &end);
      if (val.empty() || !end || *end) { bad = true; break; }
      if (key == "m") k.m = (int64_t)v;
      else if (key == "n") k.n = (int64_t)v;
      else if (key == "path") k.path = (int32_t)v;
      else if (key == "form") c.form = (int32_t)v;
      else if (key == "tile") { c.tile = (int32_t)v; have_tile = true; }
      else if (key == "lanes") lanes = (int32_t)v;
      else if (key == "us") c.us = v;
    }
    if (bad) continue;
    if (!set.empty()) {
      if (set.size() != 16 || set.find_first_not_of("0123456789abcdef") != std::string::npos) continue;
      if (!have_tile || c.tile < -1 || c.tile >= num_tile_plans() || lanes < 1 || lanes > kMaxLanes) continue;
      out.sets[set] = SetChoice{c.tile, lanes, c.us};
      continue;
    }
    if (k.m < 1 || k.n < k.m || (k.path != 0 && k.path != 1)) continue;
    if ((c.form != kFormDirect && c.form != kFormGram) || c.tile < 0 || c.tile >= num_tile_plans()) continue;
    if (k.path == 0 && c.tile != 0) continue;
    c.timed = true;
    out.shapes[k] = c;
  }
  return out;
}

bool write_cache(const std::string& path, const std::string& device_tag, const TuneCache& entries) {
  if (path.empty()) return false;
  // keep other devices' lines, replace this device's
  std::vector<std::string> keep;
  {
    std::ifstream f(path);
    std::string line;
    while (std::getline(f, line)) {
      std::istringstream is(line);
      std::string magic, tag;
      if ((is >> magic >> tag) && magic == "muon-tune-v4" && tag == device_tag) continue;
      if (!line.empty()) keep.push_back(line);
    }
  }
  const std::string tmp = path + ".tmp";
  {
    std::ofstream f(tmp, std::ios::trunc);
    if (!f) return false;
    for (const std::string& l : keep) f << l << "\n";
    char buf[256];
    for (const auto& kv : entries.shapes) {
      snprintf(buf, sizeof buf, "muon-tune-v4 %s m=%lld n=%lld path=%d form=%d tile=%d us=%.3f\n",
               device_tag.c_str(), (long long)kv.first.m, (long long)kv.first.n, kv.first.path,
               kv.second.form, kv.second.tile, kv.second.us);
      f << buf;
    }
    for (const auto& kv : entries.sets) {
      snprintf(buf, sizeof buf, "muon-tune-v4 %s set=%s tile=%d lanes=%d us=%.3f\n",
               device_tag.c_str(), kv.first.c_str(), kv.second.tile, kv.second.lanes, kv.second.us);
      f << buf;
    }
    if (!f) return false;
  }
  return std::rename(tmp.c_str(), path.c_str()) == 0;
}

std::string set_key(const std::map<ShapeKey, int>& counts,
                    const std::map<ShapeKey, ShapeChoice>& choices, int32_t forced_lanes) {
  std::ostringstream o;
  for (const auto& kv : counts) {
    const auto it = choices.find(kv.first);
    o << kv.first.m << "," << kv.first.n << "," << kv.first.path << "," << kv.second << ","
      << (it == choices.end() ? -1 : it->second.form) << "," << (it == choices.end() ? -1 : it->second.tile)
      << ";";
  }
  o << "lanes=" << forced_lanes;
  char buf[17];
  snprintf(buf, sizeof buf, "%016llx", (unsigned long long)fnv1a(o.str()));
  return buf;
}

void plan_flops(const PlanHost& p, int T, double* min_flops, double* issued_flops) {
  double mn = 0, is = 0;
  for (const ChunkPlan& C : p.chunks)
    for (const LaunchSetPlan& S : C.sets) {
      if (T <= 0) continue;
      if (S.form == kFormDirect) {
        mn += T * (S.flops_gram_min + S.flops_square_min + S.flops_apply_min);
        is += T * (S.flops_gram_issued + S.flops_square_issued + S.flops_apply_issued);
      } else {
        mn += S.flops_gram_min + S.flops_apply_min + (4.0 * T - 3) * S.flops_square_min;
        is += S.flops_gram_issued + S.flops_apply_issued + (4.0 * T - 3) * S.flops_square_issued_fp32;
      }
    }
  if (min_flops) *min_flops = mn;
  if (issued_flops) *issued_flops = is;
}

double plan_ew_bytes(const PlanHost& p) {
  double b = 0;
  for (const MatPlan& M : p.mats) {
    const double e = (double)M.rows * M.cols;
    const double pes = M.dtype ? 2 : 4, es = M.path ? 2 : 4;
    const double dt = M.has[bX0T] ? es : 0;   // transposed copy of d for the bf16 path
    b += e * (pes + 8 + es + dt);  // momentum: g, buf in/out, d (and d^T) out
    b += e * (4 + 2 * pes);        // apply: X_T in, W in/out
  }
  return b;
}

}  // namespace muon
