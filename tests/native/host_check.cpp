// Host-only driver of the planner (plan.cpp) and the owner-assignment solver
// (assign.cpp) for sanitizer builds: the CPU tests compile this file together
// with those two sources under -fsanitize=address,undefined and compare what
// it prints with what the library itself returns for the same inputs.
//
//   host_check plan <tile> <form> <lanes> <cap_bytes> <precision>
//       stdin: "rows cols dtype" per matrix; prints the canonical plan text
//       (per-shape choices from the cost model, as a plan created with tuning
//       off does).
//   host_check assign <owners> <node_limit>
//       stdin: one cost per line; prints "makespan optimal" then the owners.
//   host_check cache <path>
//       writes a cache, reads it back (and a damaged copy), prints the entries.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <iostream>
#include <map>
#include <string>
#include <vector>

#include "assign.hpp"
#include "plan.hpp"

using namespace muon;

static int do_plan(int argc, char** argv) {
  if (argc < 7) return 2;
  PlanOptions po;
  po.tile = std::atoi(argv[2]);
  po.form = std::atoi(argv[3]);
  po.lanes = std::max(1, std::atoi(argv[4]));
  po.workspace_cap = std::strtoull(argv[5], nullptr, 10);
  po.precision = std::atoi(argv[6]);
  po.host_only = 1;
  std::vector<int64_t> rows, cols;
  std::vector<int32_t> dts;
  long long r, c;
  int dt;
  while (std::cin >> r >> c >> dt) {
    rows.push_back(r);
    cols.push_back(c);
    dts.push_back(dt);
  }
  std::map<ShapeKey, int> counts;
  for (size_t i = 0; i < rows.size(); ++i) counts[shape_key(rows[i], cols[i], dts[i], po.precision)]++;
  std::map<ShapeKey, ShapeChoice> choices;
  for (const auto& kv : counts) {
    const auto all = candidates(kv.first, po.form, po.tile);
    double best = 0;
    for (const auto& cd : all) {
      const double us = model_cost_us(kv.first, cd.first, cd.second, kv.second);
      best = (best == 0 || us < best) ? us : best;
    }
    std::vector<std::pair<int32_t, int32_t>> cands;
    for (const auto& cd : all)
      if (model_cost_us(kv.first, cd.first, cd.second, kv.second) <= 2.0 * best) cands.push_back(cd);
    if (cands.size() == 1) {
      ShapeChoice ch;
      ch.form = cands[0].first;
      ch.tile = cands[0].second;
      choices[kv.first] = ch;
    } else {
      choices[kv.first] = model_choice(kv.first, po.form, po.tile, kv.second);
    }
  }
  PlanHost H;
  const std::string err = build_plan(rows, cols, dts, po, choices, &H);
  if (!err.empty()) {
    std::printf("ERROR %s\n", err.c_str());
    return 0;
  }
  const std::string s = serialize_plan(H);
  std::fwrite(s.data(), 1, s.size(), stdout);
  double mn = 0, iss = 0;
  plan_flops(H, 5, &mn, &iss);
  std::fprintf(stderr, "flops %.17g %.17g bytes %.17g hash %llu\n", mn, iss, plan_ew_bytes(H),
               (unsigned long long)fnv1a(s));
  return 0;
}

static int do_assign(int argc, char** argv) {
  if (argc < 4) return 2;
  const int owners = std::atoi(argv[2]);
  const long long limit = std::atoll(argv[3]);
  std::vector<double> costs;
  double x;
  while (std::cin >> x) costs.push_back(x);
  const AssignResult res = assign_owners(costs, owners, limit);
  std::printf("%.17g %d\n", res.makespan, res.optimal ? 1 : 0);
  for (int32_t o : res.owner) std::printf("%d\n", o);
  return 0;
}

static int do_cache(int argc, char** argv) {
  if (argc < 3) return 2;
  const std::string path = argv[2];
  TuneCache c;
  const ShapeKey k1{1024, 4096, 1}, k2{256, 512, 0};
  ShapeChoice a;
  a.form = kFormDirect;
  a.tile = 6;
  a.us = 123.5;
  a.timed = true;
  ShapeChoice b;
  b.form = kFormGram;
  b.tile = 0;
  b.us = 7.25;
  b.timed = true;
  c.shapes[k1] = a;
  c.shapes[k2] = b;
  SetChoice sc;
  sc.tile = 2;
  sc.lanes = 3;
  sc.us = 99.0;
  std::map<ShapeKey, int> counts{{k1, 4}, {k2, 1}};
  const std::string sk = set_key(counts, c.shapes, 0);
  c.sets[sk] = sc;
  if (!write_cache(path, "host", c)) return 3;
  const TuneCache back = read_cache(path, "host");
  const TuneCache other = read_cache(path, "gfx950-cu256-abi1");
  std::printf("shapes %zu sets %zu other %zu\n", back.shapes.size(), back.sets.size(), other.shapes.size());
  for (const auto& kv : back.shapes)
    std::printf("m=%lld n=%lld path=%d form=%d tile=%d\n", (long long)kv.first.m, (long long)kv.first.n,
                kv.first.path, kv.second.form, kv.second.tile);
  for (const auto& kv : back.sets)
    std::printf("set %s tile=%d lanes=%d\n", kv.first == sk ? "key" : "other", kv.second.tile, kv.second.lanes);
  // a damaged copy: truncated lines and garbage are ignored, never read past
  std::FILE* f = std::fopen(path.c_str(), "ab");
  if (!f) return 3;
  std::fputs("muon-tune-v4 host m=12 n=\nmuon-tune-v4 host m=99999999999999999999 n=1 path=1 form=1 tile=1\n"
             "\x01\x02garbage\nmuon-tune-v4 host set=", f);
  std::fclose(f);
  const TuneCache dam = read_cache(path, "host");
  std::printf("damaged shapes %zu sets %zu\n", dam.shapes.size(), dam.sets.size());
  return 0;
}

int main(int argc, char** argv) {
  if (argc < 2) return 2;
  if (!std::strcmp(argv[1], "plan")) return do_plan(argc, argv);
  if (!std::strcmp(argv[1], "assign")) return do_assign(argc, argv);
  if (!std::strcmp(argv[1], "cache")) return do_cache(argc, argv);
  return 2;
}
