// Host-side planner of the Muon step: pure C++, no device calls.
//
// The plan is a pure function of (matrix descriptors, options, per-shape
// choices).  The per-shape choices (NS form and tile plan) come from the tune
// cache, one-time timing, or the analytic cost model; everything downstream
// of them - groups, chunks, workspace offsets, work-item order - is derived
// deterministically here, so equal inputs give byte-equal plans.
//
// DMuon announcement (wjxwpt.net), improvement 2 "shape-adaptive execution
// stack": the mathematical form, the execution mode (alone or batched) and
// the kernel are chosen per shape.  DMuon announcement (zaocj.com), second of
// the three moves: a new shape is measured once and the winner is reused for
// that shape.
#pragma once
#include <stdint.h>

#include <map>
#include <string>
#include <tuple>
#include <vector>

namespace muon {

enum PlanForm : int32_t { kFormDirect = 1, kFormGram = 2 };

// Buffer ids of a matrix's workspace (same numbering as kernels.hpp BufId).
enum PlanBuf : int32_t {
  bX0 = 0, bX1, bXT, bA, bB, bH, bQX, bQY, bT1, bQH, bX0T, bX1T, kPlanBufs
};

// Output tiles of the bf16 NT kernel configurations (kernels.hpp NtCfg; abi.cpp
// checks at compile time that the two tables agree).
struct TileShape { int32_t bm, bn; };
constexpr int kNtTiles = 5;
constexpr TileShape kNtTileShapes[kNtTiles] = {{128, 128}, {256, 256}, {256, 128}, {128, 256}, {64, 64}};
TileShape nt_cfg_shape(int cfg);

// A tile plan: the NT kernel configuration of the symmetric m x m products
// (X X^T, A A; square tiles), that of the m x n product B X, and how B X
// reads X: from a transposed copy X^T kept beside X (qt = 0: the epilogue of
// every B X also writes X'^T), or k-major from X itself with LDS transpose
// reads (qt = 1: no transposed copies; slower main loop).  The fp32 path runs
// the 128 x 128 register-staged kernel and has the single plan 0.
struct TilePlan { int32_t sym, apply, qt; };

// Work-item list of the m x n product for NT configuration cfg and read mode qt.
constexpr int full_list(int cfg, int qt) { return cfg + kNtTiles * qt; }
int num_tile_plans();
TilePlan tile_plan(int t);

struct ShapeKey {
  int64_t m, n;     // canonical (min, max)
  int32_t path;     // NS dtype: 0 fp32, 1 bf16
  bool operator<(const ShapeKey& o) const {
    return std::tie(path, m, n) < std::tie(o.path, o.m, o.n);
  }
  bool operator==(const ShapeKey& o) const { return m == o.m && n == o.n && path == o.path; }
};

struct ShapeChoice {
  int32_t form = kFormDirect;
  int32_t tile = 0;
  double us = 0;        // measured NS time per matrix of the chosen candidate (0: not timed)
  bool timed = false;
};

struct PlanOptions {
  int32_t nesterov = 1;
  float eps = 1e-7f;
  float rms_scale = 0.2f;
  int32_t precision = 0;  // muon_precision
  int32_t form = 0;       // muon_form
  int32_t tile = -1;      // forced tile plan, -1: chosen per shape
  int32_t tune = 0;
  int32_t host_only = 0;
  int32_t lanes = 0;      // NS lanes per chunk; 0: 1 (build_plan) or tuned (plan creation)
  uint64_t workspace_cap = 0;
  std::string cache_path;
};

struct MatPlan {
  int64_t rows = 0, cols = 0;
  int32_t dtype = 0;       // parameter dtype
  int32_t path = 0;        // NS dtype
  int32_t trans = 0;
  int64_t m = 0, n = 0, m_pad = 0, n_pad = 0;
  int32_t form = kFormDirect;
  int32_t tile = 0;
  int32_t group = -1;
  int32_t chunk = -1;
  int32_t lane = 0;
  float s = 0.f;                  // RMS-matching scale
  uint64_t off[kPlanBufs] = {0};  // workspace byte offsets per buffer id (within the chunk region)
  bool has[kPlanBufs] = {false};  // buffer present
  uint64_t ws_bytes = 0;
  int64_t ew_tiles = 0;           // 64 x 64 tiles of the padded canonical extent
  double cost_us = 0;             // estimated step time (owner assignment input)
};

struct GroupPlan {
  ShapeKey key;
  int32_t form = kFormDirect, tile = 0;
  std::vector<int32_t> members;  // matrix indices, ascending
};

struct ItemHost { int32_t slot, tm, tn; };

// Matrices of one chunk that share (path, form, lane): one launch per NS stage and
// kernel configuration.  On the bf16 path every NT configuration has its own
// item lists, so matrices whose tile plans differ in one product still share
// the launches of the other (a plan {128 sym, 256 apply} and a plan {128, 128}
// run X X^T and A A together).
struct LaunchSetPlan {
  int32_t path = 0, form = kFormDirect;
  int32_t lane = 0;                        // NS lane (stream) the set's launches go to
  std::vector<int32_t> mats;               // matrix indices, in slot order
  std::vector<ItemHost> nt_sym[kNtTiles];  // upper-triangle m x m tiles per NT configuration
  std::vector<ItemHost> nt_full[2 * kNtTiles]; // m x n tiles per (NT configuration, read mode)
  std::vector<ItemHost> old_sym;           // upper-triangle tiles of the fp32 kernel (edge old_edge)
  std::vector<ItemHost> old_full;          // m x n tiles of the fp32 kernel
  // tile edge of the fp32 kernel in this set: 128, or 64 on the fp32 path when
  // the set's m x n products have fewer 128-tiles than the GPU has CUs (the
  // bf16 Gram iterates keep 128)
  int32_t old_edge = 128;
  // symmetric-aware algorithmic flops of one product over the matrices of each
  // NT configuration's launch (bf16 path) or of the whole set (fp32 path: index 0)
  double fl_gram[kNtTiles] = {0}, fl_square[kNtTiles] = {0}, fl_apply[2 * kNtTiles] = {0};
  double flops_gram_min = 0;       // one X X^T over the set
  double flops_square_min = 0;     // one symmetric m x m product over the set
  double flops_apply_min = 0;      // one (m x m)(m x n) product over the set
  double flops_gram_issued = 0, flops_square_issued = 0, flops_apply_issued = 0;
  double flops_square_issued_fp32 = 0;   // Gram iterates on the fp32 kernel
};

// NS lanes: a chunk's matrices (in group order) are cut into runs of about
// equal NS work, one per lane; each lane's sets are enqueued on a stream of
// their own, so one lane's launch fills the CUs another lane's tail leaves idle.
constexpr int kMaxLanes = 4;

struct ChunkPlan {
  std::vector<int32_t> mats;         // in group order
  int32_t n_lanes = 1;               // lanes holding at least one matrix are 0 .. n_lanes-1
  uint64_t ws_bytes = 0;
  int64_t ew_tiles = 0;
  std::vector<LaunchSetPlan> sets;
};

struct PlanHost {
  PlanOptions opts;
  int32_t lanes = 1;           // lanes per chunk the plan was cut for
  std::vector<MatPlan> mats;
  std::vector<GroupPlan> groups;
  std::vector<ChunkPlan> chunks;
  uint64_t ws_bytes = 0;       // max over chunks
  int32_t n_gram = 0;
};

// Canonical key of a matrix under the options (path from dtype and precision).
ShapeKey shape_key(int64_t rows, int64_t cols, int32_t dtype, int32_t precision);

// Candidates (form, tile plan) of a key, in the fixed tie-break order.
std::vector<std::pair<int32_t, int32_t>> candidates(const ShapeKey& k, int32_t forced_form,
                                                    int32_t forced_tile);

// Analytic cost of one matrix of `count` equal ones for a (form, tile plan),
// in microseconds at the rates the kernels reach on MI355X (used when not timing).
double model_cost_us(const ShapeKey& k, int32_t form, int32_t tile, int count);
ShapeChoice model_choice(const ShapeKey& k, int32_t forced_form, int32_t forced_tile, int count);

// Padded canonical extents of a key under a (form, tile plan).
void padded_dims(const ShapeKey& k, int32_t form, int32_t tile, int64_t* m_pad, int64_t* n_pad);

// Largest canonical extents the kernels address (32-bit byte offsets per operand).
bool dims_supported(int64_t rows, int64_t cols);

// Builds the plan.  choices must hold an entry for every distinct key.
// Returns "" on success or an error message (workspace cap exceeded by one matrix).
std::string build_plan(const std::vector<int64_t>& rows, const std::vector<int64_t>& cols,
                       const std::vector<int32_t>& dtypes, const PlanOptions& opts,
                       const std::map<ShapeKey, ShapeChoice>& choices, PlanHost* out);

// Canonical serialization (text) and its FNV-1a hash.
std::string serialize_plan(const PlanHost& p);
uint64_t fnv1a(const std::string& s);

// Workspace bytes of one matrix of the given key/form/tile (as laid out by build_plan).
uint64_t matrix_ws_bytes(const ShapeKey& k, int32_t form, int32_t tile);

// Whole-set choice: one tile plan for every bf16 direct-form shape of a
// matrix set (-1: the per-shape choices stand) and the NS lane count.
struct SetChoice {
  int32_t tile = -1;
  int32_t lanes = 1;
  double us = 0;   // measured NS time of the whole set
};

// Tune cache: one line per shape key and one per matrix set (keyed by
// set_key of the set's per-shape choices); unknown or malformed lines are
// ignored.
struct TuneCache {
  std::map<ShapeKey, ShapeChoice> shapes;
  std::map<std::string, SetChoice> sets;
};
TuneCache read_cache(const std::string& path, const std::string& device_tag);
bool write_cache(const std::string& path, const std::string& device_tag, const TuneCache& entries);

// Key of a matrix set: hex FNV-1a of its shape keys, their counts, their
// per-shape choices and the forced lane count (0: free).
std::string set_key(const std::map<ShapeKey, int>& counts,
                    const std::map<ShapeKey, ShapeChoice>& choices, int32_t forced_lanes);

// Per-step flops of the plan at ns_steps T: symmetric-aware minimum and issued by the tiles.
void plan_flops(const PlanHost& p, int ns_steps, double* min_flops, double* issued_flops);
double plan_ew_bytes(const PlanHost& p);

}  // namespace muon
