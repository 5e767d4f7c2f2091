// Host-side planner of the Muon step (see plan.hpp).
#include "plan.hpp"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <fstream>
#include <sstream>

namespace muon {

namespace {

constexpr uint64_t kAlign = 256;
constexpr uint64_t kDefaultCap = 48ull << 30;
constexpr int kEw = 64;           // elementwise tile edge
constexpr int kXcds = 8;          // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr double kLaunchUs = 4.0; // per-launch cost used by the model

uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }
int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// Buffer ids (same numbering as kernels.hpp BufId).
enum { bX0 = 0, bX1, bXT, bA, bB, bH, bQX, bQY, bT1, bQH };

// Byte offsets of each buffer of one matrix, relative to its start; returns the total.
uint64_t layout(const ShapeKey& k, int32_t form, int32_t tile, uint64_t* off) {
  const TileShape t = tile_shape(tile);
  const int64_t pad = std::max(t.bm, t.bn);
  const uint64_t mp = (uint64_t)round_up(k.m, pad), np = (uint64_t)round_up(k.n, pad);
  const uint64_t es = k.path ? 2 : 4;
  const uint64_t mn = mp * np, mm = mp * mp;
  uint64_t sizes[10] = {0};
  sizes[bX0] = es * mn;
  sizes[bXT] = 4 * mn;
  if (form == kFormDirect) {
    sizes[bX1] = es * mn;
    sizes[bA] = es * mm;
    sizes[bB] = es * mm;
  } else {
    sizes[bA] = sizes[bH] = sizes[bQX] = sizes[bQY] = sizes[bT1] = 4 * mm;
    if (k.path) sizes[bQH] = 2 * mm;
  }
  uint64_t cur = 0;
  for (int b = 0; b < 10; ++b) {
    if (off) off[b] = sizes[b] ? cur : 0;
    cur = align_up(cur + sizes[b], kAlign);
  }
  return cur;
}

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

}  // namespace

TileShape tile_shape(int tile) {
  switch (tile) {
    default:
    case 0: return {128, 128};
  }
}
int num_tiles() { return 1; }

ShapeKey shape_key(int64_t rows, int64_t cols, int32_t dtype, int32_t precision) {
  ShapeKey k;
  k.m = std::min(rows, cols);
  k.n = std::max(rows, cols);
  if (precision == 1) k.path = 0;
  else if (precision == 2) k.path = 1;
  else k.path = dtype == 0 ? 0 : 1;
  return k;
}

uint64_t matrix_ws_bytes(const ShapeKey& k, int32_t form, int32_t tile) {
  return layout(k, form, tile, nullptr);
}

double model_cost_us(const ShapeKey& k, int32_t form, int32_t tile) {
  const int T = 5;
  const TileShape t = tile_shape(tile);
  const double mp = (double)round_up(k.m, std::max(t.bm, t.bn));
  const double np = (double)round_up(k.n, std::max(t.bm, t.bn));
  const double ntm = mp / t.bm;
  const double sym_tiles = ntm * (ntm + 1) / 2;
  const double tile_flops = 2.0 * t.bm * t.bn;
  const double gram = sym_tiles * tile_flops * np;
  const double square = sym_tiles * tile_flops * mp;
  const double apply = ntm * (np / t.bn) * tile_flops * mp;
  const double fast = (k.path ? 2.5e15 : 157e12) * 0.5;   // NS dtype rate
  const double f32 = 157e12 * 0.5;                          // Gram iterates run in fp32
  if (form == kFormDirect) return T * (gram + square + apply) / fast * 1e6 + 3 * T * kLaunchUs;
  return (gram + apply) / fast * 1e6 + (4 * T - 3) * square / f32 * 1e6 + (4 * T - 1) * kLaunchUs;
}

ShapeChoice model_choice(const ShapeKey& k, int32_t forced_form) {
  ShapeChoice c;
  c.tile = 0;
  if (forced_form == kFormDirect || forced_form == kFormGram) {
    c.form = forced_form;
    return c;
  }
  const double d = model_cost_us(k, kFormDirect, 0), g = model_cost_us(k, kFormGram, 0);
  c.form = g < 0.97 * d ? kFormGram : kFormDirect;
  return c;
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
    g.tile = it->second.tile;
    g.members = kv.second;
    const int32_t gi = (int32_t)P.groups.size();
    for (int32_t i : g.members) {
      MatPlan& M = P.mats[i];
      M.form = g.form;
      M.tile = g.tile;
      M.group = gi;
      const TileShape t = tile_shape(g.tile);
      const int64_t pad = std::max(t.bm, t.bn);
      M.m_pad = round_up(M.m, pad);
      M.n_pad = round_up(M.n, pad);
      M.ws_bytes = layout(kv.first, g.form, g.tile, M.off);
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
      for (int b = 0; b < 10; ++b) M.off[b] += C.ws_bytes;
      C.ws_bytes += M.ws_bytes;
      C.ew_tiles += M.ew_tiles;
      M.chunk = (int32_t)(P.chunks.size() - 1);
      C.mats.push_back(i);
    }
  }
  for (ChunkPlan& C : P.chunks) {
    P.ws_bytes = std::max(P.ws_bytes, C.ws_bytes);
    for (int32_t i : C.mats) {
      const MatPlan& M = P.mats[i];
      LaunchSetPlan* S = nullptr;
      for (LaunchSetPlan& s : C.sets)
        if (s.path == M.path && s.form == M.form && s.tile == M.tile) S = &s;
      if (!S) {
        C.sets.emplace_back();
        S = &C.sets.back();
        S->path = M.path;
        S->form = M.form;
        S->tile = M.tile;
      }
      const int32_t slot = (int32_t)S->mats.size();
      S->mats.push_back(i);
      const TileShape t = tile_shape(M.tile);
      const int32_t ntm = (int32_t)(M.m_pad / t.bm), ntn = (int32_t)(M.n_pad / t.bn);
      for (int32_t a = 0; a < ntm; ++a)
        for (int32_t b = a; b < ntm; ++b) S->items_sym.push_back({slot, a, b});
      for (int32_t a = 0; a < ntm; ++a)
        for (int32_t b = 0; b < ntn; ++b) S->items_full.push_back({slot, a, b});
      const double m = (double)M.m, nn = (double)M.n, mp = (double)M.m_pad, np = (double)M.n_pad;
      const double symt = (double)ntm * (ntm + 1) / 2, tf = 2.0 * t.bm * t.bn;
      S->flops_gram_min += nn * m * (m + 1);
      S->flops_square_min += m * m * (m + 1);
      S->flops_apply_min += 2.0 * m * m * nn;
      S->flops_gram_issued += symt * tf * np;
      S->flops_square_issued += symt * tf * mp;
      S->flops_apply_issued += (double)ntm * ntn * tf * mp;
    }
    for (LaunchSetPlan& S : C.sets) {
      // longest contraction first, then XCD-contiguous placement
      auto kgram = [&](const ItemHost& it) { return P.mats[S.mats[it.slot]].n_pad; };
      auto kfull = [&](const ItemHost& it) { return P.mats[S.mats[it.slot]].m_pad; };
      std::stable_sort(S.items_sym.begin(), S.items_sym.end(),
                       [&](const ItemHost& x, const ItemHost& y) { return kgram(x) > kgram(y); });
      std::stable_sort(S.items_full.begin(), S.items_full.end(),
                       [&](const ItemHost& x, const ItemHost& y) { return kfull(x) > kfull(y); });
      remap_xcd(S.items_sym);
      remap_xcd(S.items_full);
    }
  }
  *out = std::move(P);
  return "";
}

std::string serialize_plan(const PlanHost& p) {
  std::ostringstream o;
  o << "muon-plan v1\n";
  o << "opts nesterov=" << p.opts.nesterov << " eps=" << std::hexfloat << p.opts.eps
    << " rms=" << p.opts.rms_scale << std::defaultfloat << " precision=" << p.opts.precision
    << " form=" << p.opts.form << " cap=" << p.opts.workspace_cap << "\n";
  for (size_t i = 0; i < p.mats.size(); ++i) {
    const MatPlan& M = p.mats[i];
    o << "mat " << i << " " << M.rows << "x" << M.cols << " dtype=" << M.dtype << " path=" << M.path
      << " trans=" << M.trans << " pad=" << M.m_pad << "x" << M.n_pad << " form=" << M.form
      << " tile=" << M.tile << " group=" << M.group << " chunk=" << M.chunk << " ws=" << M.ws_bytes
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
      << "\n";
    for (const LaunchSetPlan& S : C.sets) {
      o << " set path=" << S.path << " form=" << S.form << " tile=" << S.tile << " mats=" << S.mats.size()
        << " sym=" << S.items_sym.size() << " full=" << S.items_full.size() << " order=";
      uint64_t h = 1469598103934665603ull;
      auto mix = [&](int32_t v) { for (int b = 0; b < 4; ++b) { h ^= (uint8_t)(v >> (8 * b)); h *= 1099511628211ull; } };
      for (const ItemHost& it : S.items_sym) { mix(it.slot); mix(it.tm); mix(it.tn); }
      for (const ItemHost& it : S.items_full) { mix(it.slot); mix(it.tm); mix(it.tn); }
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

std::map<ShapeKey, ShapeChoice> read_cache(const std::string& path, const std::string& device_tag) {
  std::map<ShapeKey, ShapeChoice> out;
  if (path.empty()) return out;
  std::ifstream f(path);
  std::string line;
  while (std::getline(f, line)) {
    std::istringstream is(line);
    std::string magic, tag;
    if (!(is >> magic >> tag) || magic != "muon-tune-v1" || tag != device_tag) continue;
    ShapeKey k{-1, -1, -1};
    ShapeChoice c;
    c.form = -1;
    c.tile = -1;
    std::string kv;
    bool bad = false;
    while (is >> kv) {
      const size_t eq = kv.find('=');
      if (eq == std::string::npos) { bad = true; break; }
      const std::string key = kv.substr(0, eq), val = kv.substr(eq + 1);
      char* end = nullptr;
      const double v = std::strtod(val.c_str(), &end);
      if (!end || *end) { bad = true; break; }
      if (key == "m") k.m = (int64_t)v;
      else if (key == "n") k.n = (int64_t)v;
      else if (key == "path") k.path = (int32_t)v;
      else if (key == "form") c.form = (int32_t)v;
      else if (key == "tile") c.tile = (int32_t)v;
      else if (key == "us_direct") c.us_direct = v;
      else if (key == "us_gram") c.us_gram = v;
    }
    if (bad || k.m < 1 || k.n < k.m || (k.path != 0 && k.path != 1)) continue;
    if ((c.form != kFormDirect && c.form != kFormGram) || c.tile < 0 || c.tile >= num_tiles()) continue;
    c.timed = true;
    out[k] = c;
  }
  return out;
}

bool write_cache(const std::string& path, const std::string& device_tag,
                 const std::map<ShapeKey, ShapeChoice>& entries) {
  if (path.empty()) return false;
  // keep other devices' lines, replace this device's
  std::vector<std::string> keep;
  {
    std::ifstream f(path);
    std::string line;
    while (std::getline(f, line)) {
      std::istringstream is(line);
      std::string magic, tag;
      if ((is >> magic >> tag) && magic == "muon-tune-v1" && tag == device_tag) continue;
      if (!line.empty()) keep.push_back(line);
    }
  }
  const std::string tmp = path + ".tmp";
  {
    std::ofstream f(tmp, std::ios::trunc);
    if (!f) return false;
    for (const std::string& l : keep) f << l << "\n";
    for (const auto& kv : entries) {
      char buf[256];
      snprintf(buf, sizeof buf, "muon-tune-v1 %s m=%lld n=%lld path=%d form=%d tile=%d us_direct=%.3f us_gram=%.3f\n",
               device_tag.c_str(), (long long)kv.first.m, (long long)kv.first.n, kv.first.path,
               kv.second.form, kv.second.tile, kv.second.us_direct, kv.second.us_gram);
      f << buf;
    }
    if (!f) return false;
  }
  return std::rename(tmp.c_str(), path.c_str()) == 0;
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
        is += S.flops_gram_issued + S.flops_apply_issued + (4.0 * T - 3) * S.flops_square_issued;
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
    b += e * (pes + 8 + es);    // momentum: g, buf in/out, d out
    b += e * (4 + 2 * pes);     // apply: X_T in, W in/out
  }
  return b;
}

}  // namespace muon
