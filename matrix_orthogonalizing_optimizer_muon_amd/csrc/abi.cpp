// C ABI of the Muon step: plan objects, device tables, the per-step launch
// sequence, one-time per-shape timing with a persisted cache, and profiling.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "muon.h"
#include "errors.hpp"
#include "kernels.hpp"
#include "probe.hpp"
#include "assign.hpp"
#include "plan.hpp"

using namespace muon;

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

}  // namespace

int muon::report_error(int code, const std::string& msg) { return fail(code, msg); }

namespace {

#define HIP_TRY(x)                                                                        \
  do {                                                                                    \
    hipError_t e_ = (x);                                                                  \
    if (e_ != hipSuccess) return fail(MUON_EHIP, std::string(#x) + ": " + hipGetErrorString(e_)); \
  } while (0)

enum Kind { kEwMom = 0, kNorm, kNsSyrk, kNsComb, kNsApply, kGramXxt, kGramSquare, kGramFinal, kEwApply, kKinds };
const char* kKindNames[kKinds] = {"ew_momentum", "ew_norm", "ns_syrk", "ns_comb", "ns_apply",
                                  "gram_xxt", "gram_square", "gram_final", "ew_apply"};

// One list of work items on the device.
struct Items {
  WorkItem* d = nullptr;
  int n = 0;
};

struct SetDev {
  int path = 0, form = kFormDirect;
  int lane = 0;
  int nmats = 0;
  NsMat* mats = nullptr;
  Items nt_sym[kNumNtCfgs], nt_full[2 * kNumNtCfgs], old_sym, old_full;   // nt_full: full_list(cfg, qt)
  int old_cfg = 0;   // fp32 kernel configuration of old_sym / old_full (kTileCfgs index)
  // algorithmic (symmetric-aware) flops of each launch: per NT configuration
  // (and read mode for B X) on the bf16 path, index 0 for the fp32 kernel
  double fl_gram[kNumNtCfgs] = {0}, fl_square[kNumNtCfgs] = {0}, fl_apply[2 * kNumNtCfgs] = {0};
};

static_assert(kNumNtCfgs == kNtTiles && sizeof(kNtTileShapes) / sizeof(kNtTileShapes[0]) == kNtTiles,
              "tables");
static_assert(kNtCfgs[0].bm == kNtTileShapes[0].bm && kNtCfgs[0].bn == kNtTileShapes[0].bn &&
              kNtCfgs[1].bm == kNtTileShapes[1].bm && kNtCfgs[1].bn == kNtTileShapes[1].bn &&
              kNtCfgs[2].bm == kNtTileShapes[2].bm && kNtCfgs[2].bn == kNtTileShapes[2].bn &&
              kNtCfgs[3].bm == kNtTileShapes[3].bm && kNtCfgs[3].bn == kNtTileShapes[3].bn &&
              kNtCfgs[4].bm == kNtTileShapes[4].bm && kNtCfgs[4].bn == kNtTileShapes[4].bn,
              "planner and kernel tile tables agree");
static_assert((int)kPlanBufs == (int)kNumBufs && (int)bX0T == (int)kX0T && (int)bX1T == (int)kX1T &&
              (int)bQH == (int)kQH, "buffer ids agree");

struct ChunkDev {
  std::vector<int> mats;          // global indices, chunk order
  EwMat* ew = nullptr;
  int64_t* prefix = nullptr;
  EwDyn* dyn = nullptr;
  EwDyn* dyn_pinned = nullptr;
  std::vector<EwDyn> dyn_last;
  bool dyn_valid = false;
  hipEvent_t upload_ev = nullptr;
  bool upload_pending = false;
  float* partials = nullptr;
  int64_t total_tiles = 0;
  double bytes_apply = 0;
  bool all_fused = false;     // every matrix's update is applied by its last NS product
  double bytes_apply_unfused = 0;   // k_ew_apply bytes when fused matrices are skipped
  double bytes_store = 0;   // orthogonalization alone: X_T -> out
  std::vector<SetDev> sets;
  int n_lanes = 1;
  // lane l's matrices: mats[lane_first[l] .. lane_first[l + 1]) (contiguous in
  // chunk order); tile_first[k]: first elementwise tile of mats[k] (k = nm: the
  // total); per-matrix bytes of the momentum kernel and of the input load
  // (orthogonalization alone: input -> D, and D^T when kept)
  std::vector<int> lane_first;
  std::vector<int64_t> tile_first;
  std::vector<double> mat_bytes_mom, mat_bytes_load;
};

// Kernel symbol labels for the profiling records (one per template instance;
// ",qt": the instance that reads Q k-major).
const char* nt_name(int cfg, int odt, int qt = 0) {
  static const char* names[2][kNumNtCfgs][2] = {
      {{"k_nt<128,128,f32>", "k_nt<128,128,bf16>"}, {"k_nt<256,256,f32>", "k_nt<256,256,bf16>"},
       {"k_nt<256,128,f32>", "k_nt<256,128,bf16>"}, {"k_nt<128,256,f32>", "k_nt<128,256,bf16>"},
       {"k_nt<64,64,f32>", "k_nt<64,64,bf16>"}},
      {{"k_nt<128,128,f32,qt>", "k_nt<128,128,bf16,qt>"}, {"k_nt<256,256,f32,qt>", "k_nt<256,256,bf16,qt>"},
       {"k_nt<256,128,f32,qt>", "k_nt<256,128,bf16,qt>"}, {"k_nt<128,256,f32,qt>", "k_nt<128,256,bf16,qt>"},
       {"k_nt<64,64,f32,qt>", "k_nt<64,64,bf16,qt>"}}};
  return names[qt ? 1 : 0][cfg][odt == kBF16 ? 1 : 0];
}
const char* rs_name(bool nn, int idt, int odt) {
  if (idt == kF32) return nn ? "k_gemm<f32,f32,NN>" : "k_gemm<f32,f32,NT>";
  if (odt == kF32) return nn ? "k_gemm<bf16,f32,NN>" : "k_gemm<bf16,f32,NT>";
  return nn ? "k_gemm<bf16,bf16,NN>" : "k_gemm<bf16,bf16,NT>";
}

struct ProfRec {
  int kind;
  const char* kern;
  double flops, bytes;
  hipEvent_t a, b;
};

struct Totals {
  int64_t launches = 0;
  double ms = 0, flops = 0, bytes = 0;
};

}  // namespace

struct muon_plan {
  PlanHost host;
  std::string serialized;
  uint64_t hash = 0;
  int device = -1;
  int grid_cap = 2048;
  char* ws = nullptr;
  float* rscale = nullptr;
  uint32_t* flags = nullptr;
  std::vector<void*> dev_allocs;
  std::vector<void*> host_allocs;
  std::vector<ChunkDev> chunks;
  // NS lanes 1 .. lanes-1: a stream each (default priority, non-blocking);
  // lane_front[l]: lane l's front is done (lane l+1 starts on it); lane_join:
  // lanes 1.. joined back into the caller's stream
  std::vector<hipStream_t> lane_streams;
  std::vector<hipEvent_t> lane_front, lane_join;
  std::vector<float*> capture;
  bool profiling = false;
  std::vector<ProfRec> recs;
  hipEvent_t prof_epoch = nullptr;              // first recorded event since enable / reset
  std::vector<muon_launch_interval> intervals;  // folded launches, in launch order
  std::vector<hipEvent_t> ev_pool;
  std::map<std::pair<int, std::string>, Totals> tot;   // (stage, kernel) -> totals
  // graph replay of muon_step (muon_plan_set_graph): the instantiated graph of
  // the step whose arguments give graph_key; pending_key: the arguments of the
  // last eager step, captured if the next step repeats them
  bool graph_on = false;
  hipGraphExec_t graph_exec = nullptr;
  std::string graph_key, pending_key;
};

namespace {

template <typename T>
int dev_alloc(muon_plan* p, T** ptr, size_t bytes) {
  void* v = nullptr;
  if (bytes == 0) bytes = 256;
  hipError_t e = hipMalloc(&v, bytes);
  if (e != hipSuccess) return fail(MUON_ENOMEM, std::string("hipMalloc: ") + hipGetErrorString(e));
  p->dev_allocs.push_back(v);
  *ptr = static_cast<T*>(v);
  return MUON_OK;
}

template <typename T>
int host_alloc(muon_plan* p, T** ptr, size_t bytes) {
  void* v = nullptr;
  if (bytes == 0) bytes = 64;
  hipError_t e = hipHostMalloc(&v, bytes, hipHostMallocDefault);
  if (e != hipSuccess) return fail(MUON_ENOMEM, std::string("hipHostMalloc: ") + hipGetErrorString(e));
  p->host_allocs.push_back(v);
  *ptr = static_cast<T*>(v);
  return MUON_OK;
}

void drop_graph(muon_plan* p) {
  if (p->graph_exec) (void)hipGraphExecDestroy(p->graph_exec);
  p->graph_exec = nullptr;
  p->graph_key.clear();
}

void free_plan_memory(muon_plan* p) {
  if (!p) return;
  if (!p->host.opts.host_only) (void)hipDeviceSynchronize();
  drop_graph(p);
  for (ChunkDev& c : p->chunks)
    if (c.upload_ev) (void)hipEventDestroy(c.upload_ev);
  for (ProfRec& r : p->recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  for (hipEvent_t e : p->ev_pool) (void)hipEventDestroy(e);
  if (p->prof_epoch) (void)hipEventDestroy(p->prof_epoch);
  p->prof_epoch = nullptr;
  for (hipEvent_t e : p->lane_join) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->lane_front) (void)hipEventDestroy(e);
  for (hipStream_t st : p->lane_streams) (void)hipStreamDestroy(st);
  p->lane_join.clear();
  p->lane_front.clear();
  p->lane_streams.clear();
  for (void* v : p->dev_allocs) (void)hipFree(v);
  for (void* v : p->host_allocs) (void)hipHostFree(v);
  p->dev_allocs.clear();
  p->host_allocs.clear();
}

std::string device_tag(int dev) {
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return "unknown";
  std::string arch = prop.gcnArchName;
  const size_t colon = arch.find(':');
  if (colon != std::string::npos) arch = arch.substr(0, colon);
  return arch + "-cu" + std::to_string(prop.multiProcessorCount) + "-abi" + std::to_string(MUON_ABI_VERSION);
}

// Uploads the static tables of a host plan and wires the workspace.
int materialize(muon_plan* p) {
  const PlanHost& H = p->host;
  const size_t n = H.mats.size();
  int rc;
  if ((rc = dev_alloc(p, &p->ws, H.ws_bytes))) return rc;
  if ((rc = dev_alloc(p, &p->rscale, n * sizeof(float)))) return rc;
  if ((rc = dev_alloc(p, &p->flags, sizeof(uint32_t)))) return rc;
  HIP_TRY(hipMemset(p->flags, 0, sizeof(uint32_t)));
  HIP_TRY(hipMemset(p->rscale, 0, n * sizeof(float)));
  p->capture.assign(n, nullptr);
  p->chunks.resize(H.chunks.size());
  for (size_t c = 0; c < H.chunks.size(); ++c) {
    const ChunkPlan& CP = H.chunks[c];
    ChunkDev& C = p->chunks[c];
    C.mats.assign(CP.mats.begin(), CP.mats.end());
    const size_t nm = C.mats.size();
    std::vector<EwMat> ew(nm);
    std::vector<int64_t> prefix(nm);
    int64_t tb = 0;
    for (size_t k = 0; k < nm; ++k) {
      const MatPlan& M = H.mats[C.mats[k]];
      EwMat& E = ew[k];
      std::memset(&E, 0, sizeof E);
      E.rows = M.rows;
      E.cols = M.cols;
      E.m = M.m;
      E.n = M.n;
      E.ldd = M.n_pad;
      E.tile_begin = tb;
      E.tiles_i = (int32_t)(M.m_pad / kEwTile);
      E.tiles_j = (int32_t)(M.n_pad / kEwTile);
      E.trans = M.trans;
      E.pdtype = M.dtype;
      E.ddtype = M.path;
      E.mat = C.mats[k];
      E.d = p->ws + M.off[kX0];
      E.dt = M.has[bX0T] ? static_cast<void*>(p->ws + M.off[kX0T]) : nullptr;
      E.ldt = M.m_pad;
      E.xt = reinterpret_cast<float*>(p->ws + M.off[kXT]);
      E.s = M.s;
      E.fused = M.path ? 1 : 0;
      prefix[k] = tb;
      C.tile_first.push_back(tb);
      tb += M.ew_tiles;
      const double e = (double)M.rows * M.cols, pes = M.dtype ? 2 : 4, es = M.path ? 2 : 4;
      C.mat_bytes_mom.push_back(e * (pes + 8 + es + (M.has[bX0T] ? es : 0)));
      C.mat_bytes_load.push_back(e * (pes + es + (M.has[bX0T] ? es : 0)));
      C.bytes_apply += e * (4 + 2 * pes);
      C.bytes_store += e * (4 + 4);
    }
    C.tile_first.push_back(tb);
    C.total_tiles = tb;
    C.all_fused = true;
    for (size_t k = 0; k < nm; ++k) {
      const MatPlan& M = H.mats[C.mats[k]];
      if (!M.path) {
        C.all_fused = false;
        const double e = (double)M.rows * M.cols, pes = M.dtype ? 2 : 4;
        C.bytes_apply_unfused += e * (4 + 2 * pes);
      }
    }
    if ((rc = dev_alloc(p, &C.ew, nm * sizeof(EwMat)))) return rc;
    if ((rc = dev_alloc(p, &C.prefix, nm * sizeof(int64_t)))) return rc;
    if ((rc = dev_alloc(p, &C.dyn, nm * sizeof(EwDyn)))) return rc;
    if ((rc = dev_alloc(p, &C.partials, std::max<int64_t>(tb, 1) * sizeof(float)))) return rc;
    if ((rc = host_alloc(p, &C.dyn_pinned, nm * sizeof(EwDyn)))) return rc;
    HIP_TRY(hipMemcpy(C.ew, ew.data(), nm * sizeof(EwMat), hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(C.prefix, prefix.data(), nm * sizeof(int64_t), hipMemcpyHostToDevice));
    HIP_TRY(hipEventCreateWithFlags(&C.upload_ev, hipEventDisableTiming));
    C.n_lanes = CP.n_lanes;
    if (C.n_lanes > H.lanes) return fail(MUON_EINVAL, "plan: chunk lane count above the plan's");
    C.lane_first.assign(C.n_lanes + 1, (int)nm);
    for (size_t k = nm; k-- > 0;) {
      const int l = H.mats[C.mats[k]].lane;
      if (l < 0 || l >= C.n_lanes || (k + 1 < nm && l > H.mats[C.mats[k + 1]].lane))
        return fail(MUON_EINVAL, "plan: lanes are not contiguous runs of the chunk");
      for (int q = 0; q <= l; ++q) C.lane_first[q] = (int)k;
    }
    for (const LaunchSetPlan& S : CP.sets) {
      SetDev D;
      D.path = S.path;
      D.form = S.form;
      D.lane = S.lane;
      D.nmats = (int)S.mats.size();
      D.old_cfg = -1;
      for (int c = 0; c < kNumTileCfgs; ++c)
        if (kTileCfgs[c].bm == S.old_edge && kTileCfgs[c].bn == S.old_edge) D.old_cfg = c;
      if (D.old_cfg < 0) return fail(MUON_EINVAL, "plan: no fp32 kernel for the set's tile edge");
      std::vector<NsMat> nsm(S.mats.size());
      for (size_t k = 0; k < S.mats.size(); ++k) {
        const MatPlan& M = H.mats[S.mats[k]];
        NsMat& N = nsm[k];
        std::memset(&N, 0, sizeof N);
        for (int b = 0; b < kNumBufs; ++b) N.buf[b] = M.has[b] ? p->ws + M.off[b] : nullptr;
        N.m = (int32_t)M.m;
        N.n = (int32_t)M.n;
        N.m_pad = (int32_t)M.m_pad;
        N.n_pad = (int32_t)M.n_pad;
        N.mat = S.mats[k];
        N.dyn = (int32_t)(std::find(C.mats.begin(), C.mats.end(), S.mats[k]) - C.mats.begin());
        N.trans = M.trans;
        N.pdtype = M.dtype;
        N.cols = M.cols;
        N.s = M.s;
      }
      for (int c = 0; c < kNumNtCfgs; ++c) {
        D.fl_gram[c] = S.fl_gram[c];
        D.fl_square[c] = S.fl_square[c];
      }
      for (int c = 0; c < 2 * kNumNtCfgs; ++c) D.fl_apply[c] = S.fl_apply[c];
      if ((rc = dev_alloc(p, &D.mats, nsm.size() * sizeof(NsMat)))) return rc;
      HIP_TRY(hipMemcpy(D.mats, nsm.data(), nsm.size() * sizeof(NsMat), hipMemcpyHostToDevice));
      auto upload = [&](const std::vector<ItemHost>& v, Items* out) -> int {
        out->n = (int)v.size();
        if (v.empty()) return MUON_OK;
        std::vector<WorkItem> w(v.size());
        for (size_t i = 0; i < v.size(); ++i) w[i] = WorkItem{v[i].slot, v[i].tm, v[i].tn, 0};
        int r = dev_alloc(p, &out->d, w.size() * sizeof(WorkItem));
        if (r) return r;
        HIP_TRY(hipMemcpy(out->d, w.data(), w.size() * sizeof(WorkItem), hipMemcpyHostToDevice));
        return MUON_OK;
      };
      for (int c = 0; c < kNumNtCfgs; ++c)
        if ((rc = upload(S.nt_sym[c], &D.nt_sym[c]))) return rc;
      for (int c = 0; c < 2 * kNumNtCfgs; ++c)
        if ((rc = upload(S.nt_full[c], &D.nt_full[c]))) return rc;
      if ((rc = upload(S.old_sym, &D.old_sym)) || (rc = upload(S.old_full, &D.old_full))) return rc;
      C.sets.push_back(D);
    }
  }
  for (int l = 1; l < H.lanes; ++l) {
    hipStream_t st = nullptr;
    hipEvent_t ev = nullptr, ef = nullptr;
    HIP_TRY(hipStreamCreateWithFlags(&st, hipStreamNonBlocking));
    p->lane_streams.push_back(st);
    HIP_TRY(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
    p->lane_join.push_back(ev);
    HIP_TRY(hipEventCreateWithFlags(&ef, hipEventDisableTiming));
    p->lane_front.push_back(ef);
  }
  return MUON_OK;
}

hipEvent_t pool_event(muon_plan* p) {
  if (!p->ev_pool.empty()) {
    hipEvent_t e = p->ev_pool.back();
    p->ev_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

template <typename F>
int run(muon_plan* p, int kind, const char* kern, double flops, double bytes, hipStream_t s,
        F&& launch) {
  hipEvent_t a = nullptr, b = nullptr;
  if (p->profiling) {
    // the launch's dispatch start and end go into a and b
    a = pool_event(p);
    b = pool_event(p);
    if (!a || !b) return fail(MUON_EHIP, "hipEventCreate failed");
    set_launch_events(a, b);
  }
  const hipError_t e = launch();
  const bool did = launched();
  if (p->profiling) set_launch_events(nullptr, nullptr);
  if (e != hipSuccess)
    return fail(MUON_EHIP, std::string(kKindNames[kind]) + " launch: " + hipGetErrorString(e));
  if (p->profiling) {
    if (!did) {   // nothing to launch: an empty interval
      HIP_TRY(hipEventRecord(a, s));
      HIP_TRY(hipEventRecord(b, s));
    }
    p->recs.push_back({kind, kern, flops, bytes, a, b});
  }
  return MUON_OK;
}

GemmParams gp(const SetDev& S, const Items& it, bool sym, int shape, int pid, int qid, int cid,
              int oid, int o2id, int otid, float alpha, float beta, float gamma, int scale_pow,
              const float* rscale) {
  GemmParams g;
  std::memset(&g, 0, sizeof g);
  g.items = it.d;
  g.n_items = it.n;
  g.mats = S.mats;
  g.rscale = rscale;
  g.shape = shape;
  g.scale_pow = scale_pow;
  g.sym = sym ? 1 : 0;
  g.p_id = pid;
  g.q_id = qid;
  g.c_id = cid;
  g.o_id = oid;
  g.o2_id = o2id;
  g.ot_id = otid;
  g.alpha = alpha;
  g.beta = beta;
  g.gamma = gamma;
  return g;
}

// A bf16-tile NT launch whose staged outputs add up to more than the
// last-level cache (256 MB on MI355X) stores them nontemporally: they cannot
// stay cached for the next launch anyway, and streaming them frees the
// write path sooner (measured: MoE stack 164.0 -> 158.0 ms, VLA set 44.1 ->
// 43.3 ms, Llama-7B set 395-397 -> 393-394 ms; the transformer block set,
// whose launches write a few MB, ran 5% slower with them).
constexpr double kStreamOutBytes = 256.0 * 1024 * 1024;
void set_stream_out(GemmParams* g, int cfg, int copies) {
  const double bytes = (double)g->n_items * kNtCfgs[cfg].bm * kNtCfgs[cfg].bn * 2.0 * copies;
  g->stream_out = bytes > kStreamOutBytes ? 1 : 0;
}

// Makes the last NS product apply the parameter update instead of storing X_T.
void fuse_update(GemmParams* g, const EwDyn* dyn, float lr, float wd) {
  g->fuse = 1;
  g->dyn = dyn;
  g->lr = lr;
  g->wd = wd;
}

// The NS stages of one launch set (T steps, coefficient schedule sched[3*T]).
// On the bf16 path each stage is one launch per NT configuration that the
// set's matrices use for it.
//
// bf16 path, direct form, step k (X = X_k, X^T kept alongside):
//   A  = s_k X X^T                     NT, symmetric tiles           (s_0 = r^2, else 1)
//   B  = a I + b A + c A A             NT, symmetric tiles
//   X' = t_k B X                       NT with Q = X^T; writes X' and X'^T (t_0 = r, else 1)
//   the last step applies the update from X' (or, without parameters, writes
//   X' in fp32 to X_T).  B carries the a X term as a I: in exact arithmetic
//   B X equals a X + (b A + c A A) X, and the product then reads no third
//   operand.  Rounding B to bf16 perturbs a X no more than rounding X' does.
// bf16 path, Gram form: G = r^2 X0 X0^T (NT, fp32 out); the m x m recursion in
// fp32 on the register-staged kernel; X_T = r Q_T X0 (NT, Q_T rounded to bf16).
// fp32 path: the same stages on the register-staged kernel.
int enqueue_ns(muon_plan* p, const SetDev& S, int T, const float* sched, const EwDyn* dyn,
               float lr, float wd, hipStream_t s) {
  if (T <= 0) return MUON_OK;
  int rc;
  const float* rs = p->rscale;
  if (S.path) {
    if (S.form == kFormDirect) {
      for (int k = 0; k < T; ++k) {
        const float a = sched[3 * k], b = sched[3 * k + 1], c = sched[3 * k + 2];
        const bool even = k % 2 == 0, last = k == T - 1;
        const int src = even ? kX0 : kX1, srcT = even ? kX0T : kX1T;
        const int dst = last ? kXT : (even ? kX1 : kX0);
        const int dstT = last ? -1 : (even ? kX1T : kX0T);
        for (int cfg = 0; cfg < kNumNtCfgs; ++cfg) {
          if (!S.nt_sym[cfg].n) continue;
          GemmParams g1 = gp(S, S.nt_sym[cfg], true, kShapeGram, src, src, -1, kA, -1, -1, 1.f, 0.f,
                             0.f, k == 0 ? 2 : 0, rs);
          set_stream_out(&g1, cfg, 2);
          if ((rc = run(p, kNsSyrk, nt_name(cfg, kBF16), S.fl_gram[cfg], 0, s, [&] { return launch_gemm_nt(cfg, kBF16, g1, s); }))) return rc;
        }
        for (int cfg = 0; cfg < kNumNtCfgs; ++cfg) {
          if (!S.nt_sym[cfg].n) continue;
          GemmParams g2 = gp(S, S.nt_sym[cfg], true, kShapeSquare, kA, kA, kA, kB, -1, -1, c, b, a, 0, rs);
          set_stream_out(&g2, cfg, 2);
          if ((rc = run(p, kNsComb, nt_name(cfg, kBF16), S.fl_square[cfg], 0, s, [&] { return launch_gemm_nt(cfg, kBF16, g2, s); }))) return rc;
        }
        const int odt = last ? kF32 : kBF16;
        for (int fi = 0; fi < 2 * kNumNtCfgs; ++fi) {
          if (!S.nt_full[fi].n) continue;
          const int cfg = fi % kNumNtCfgs, qt = fi / kNumNtCfgs;
          // qt: B X reads X itself k-major and no transposed copy is written
          GemmParams g3 = gp(S, S.nt_full[fi], false, kShapeApplyT, kB, qt ? src : srcT, -1, dst, -1,
                             qt ? -1 : dstT, 1.f, 0.f, 0.f, k == 0 ? 1 : 0, rs);
          g3.qt = qt;
          set_stream_out(&g3, cfg, last || qt ? 1 : 2);
          if (last && dyn) fuse_update(&g3, dyn, lr, wd);
          if ((rc = run(p, kNsApply, nt_name(cfg, odt, qt), S.fl_apply[fi], 0, s, [&] { return launch_gemm_nt(cfg, odt, g3, s); }))) return rc;
        }
      }
      return MUON_OK;
    }
    // Gram space
    double fl_square = 0;
    for (int cfg = 0; cfg < kNumNtCfgs; ++cfg) {
      fl_square += S.fl_square[cfg];
      if (!S.nt_sym[cfg].n) continue;
      GemmParams g0 = gp(S, S.nt_sym[cfg], true, kShapeGram, kX0, kX0, -1, kA, -1, -1, 1.f, 0.f, 0.f, 2, rs);
      if ((rc = run(p, kGramXxt, nt_name(cfg, kF32), S.fl_gram[cfg], 0, s, [&] { return launch_gemm_nt(cfg, kF32, g0, s); }))) return rc;
    }
    int cur = kQX;
    for (int k = 0; k < T; ++k) {
      const float a = sched[3 * k], b = sched[3 * k + 1], c = sched[3 * k + 2];
      const bool last = k == T - 1;
      const int hbuf = (k == 0) ? kQX : kH;
      // H = a I + b A + c A^2 (at k = 0 this is Q_1 itself)
      GemmParams gh = gp(S, S.old_sym, true, kShapeSquare, kA, kA, kA, hbuf, (k == 0 && last) ? kQH : -1,
                         -1, c, b, a, 0, rs);
      if ((rc = run(p, kGramSquare, rs_name(false, kF32, kF32), fl_square, 0, s, [&] { return launch_gemm(S.old_cfg, kF32, kF32, gh, s); }))) return rc;
      if (k > 0) {
        const int nxt = cur == kQX ? kQY : kQX;
        GemmParams gq = gp(S, S.old_sym, true, kShapeSquare, kH, cur, -1, nxt, last ? kQH : -1, -1, 1.f,
                           0.f, 0.f, 0, rs);
        if ((rc = run(p, kGramSquare, rs_name(false, kF32, kF32), fl_square, 0, s, [&] { return launch_gemm(S.old_cfg, kF32, kF32, gq, s); }))) return rc;
        cur = nxt;
      }
      if (!last) {
        GemmParams gt = gp(S, S.old_sym, true, kShapeSquare, hbuf, kA, -1, kT1, -1, -1, 1.f, 0.f, 0.f, 0, rs);
        if ((rc = run(p, kGramSquare, rs_name(false, kF32, kF32), fl_square, 0, s, [&] { return launch_gemm(S.old_cfg, kF32, kF32, gt, s); }))) return rc;
        GemmParams ga = gp(S, S.old_sym, true, kShapeSquare, kT1, hbuf, -1, kA, -1, -1, 1.f, 0.f, 0.f, 0, rs);
        if ((rc = run(p, kGramSquare, rs_name(false, kF32, kF32), fl_square, 0, s, [&] { return launch_gemm(S.old_cfg, kF32, kF32, ga, s); }))) return rc;
      }
    }
    for (int fi = 0; fi < 2 * kNumNtCfgs; ++fi) {
      if (!S.nt_full[fi].n) continue;
      const int cfg = fi % kNumNtCfgs, qt = fi / kNumNtCfgs;
      GemmParams gf = gp(S, S.nt_full[fi], false, kShapeApplyT, kQH, qt ? kX0 : kX0T, -1, kXT, -1, -1,
                         1.f, 0.f, 0.f, 1, rs);
      gf.qt = qt;
      set_stream_out(&gf, cfg, 1);
      if (dyn) fuse_update(&gf, dyn, lr, wd);
      if ((rc = run(p, kGramFinal, nt_name(cfg, kF32, qt), S.fl_apply[fi], 0, s, [&] { return launch_gemm_nt(cfg, kF32, gf, s); }))) return rc;
    }
    return MUON_OK;
  }
  // fp32 path
  if (S.form == kFormDirect) {
    for (int k = 0; k < T; ++k) {
      const float a = sched[3 * k], b = sched[3 * k + 1], c = sched[3 * k + 2];
      const int src = (k % 2 == 0) ? kX0 : kX1;
      const int dst = (k == T - 1) ? kXT : (src == kX0 ? kX1 : kX0);
      GemmParams g1 = gp(S, S.old_sym, true, kShapeGram, src, src, -1, kA, -1, -1, 1.f, 0.f, 0.f, k == 0 ? 2 : 0, rs);
      if ((rc = run(p, kNsSyrk, rs_name(false, kF32, kF32), S.fl_gram[0], 0, s, [&] { return launch_gemm(S.old_cfg, kF32, kF32, g1, s); }))) return rc;
      GemmParams g2 = gp(S, S.old_sym, true, kShapeSquare, kA, kA, kA, kB, -1, -1, c, b, 0.f, 0, rs);
      if ((rc = run(p, kNsComb, rs_name(false, kF32, kF32), S.fl_square[0], 0, s, [&] { return launch_gemm(S.old_cfg, kF32, kF32, g2, s); }))) return rc;
      GemmParams g3 = gp(S, S.old_full, false, kShapeApply, kB, src, src, dst, -1, -1, 1.f, a, 0.f, k == 0 ? 1 : 0, rs);
      if ((rc = run(p, kNsApply, rs_name(true, kF32, kF32), S.fl_apply[0], 0, s, [&] { return launch_gemm(S.old_cfg, kF32, kF32, g3, s); }))) return rc;
    }
    return MUON_OK;
  }
  GemmParams g0 = gp(S, S.old_sym, true, kShapeGram, kX0, kX0, -1, kA, -1, -1, 1.f, 0.f, 0.f, 2, rs);
  if ((rc = run(p, kGramXxt, rs_name(false, kF32, kF32), S.fl_gram[0], 0, s, [&] { return launch_gemm(S.old_cfg, kF32, kF32, g0, s); }))) return rc;
  int cur = kQX;
  for (int k = 0; k < T; ++k) {
    const float a = sched[3 * k], b = sched[3 * k + 1], c = sched[3 * k + 2];
    const bool last = k == T - 1;
    const int hbuf = (k == 0) ? kQX : kH;
    GemmParams gh = gp(S, S.old_sym, true, kShapeSquare, kA, kA, kA, hbuf, -1, -1, c, b, a, 0, rs);
    if ((rc = run(p, kGramSquare, rs_name(false, kF32, kF32), S.fl_square[0], 0, s, [&] { return launch_gemm(S.old_cfg, kF32, kF32, gh, s); }))) return rc;
    if (k > 0) {
      const int nxt = cur == kQX ? kQY : kQX;
      GemmParams gq = gp(S, S.old_sym, true, kShapeSquare, kH, cur, -1, nxt, -1, -1, 1.f, 0.f, 0.f, 0, rs);
      if ((rc = run(p, kGramSquare, rs_name(false, kF32, kF32), S.fl_square[0], 0, s, [&] { return launch_gemm(S.old_cfg, kF32, kF32, gq, s); }))) return rc;
      cur = nxt;
    }
    if (!last) {
      GemmParams gt = gp(S, S.old_sym, true, kShapeSquare, hbuf, kA, -1, kT1, -1, -1, 1.f, 0.f, 0.f, 0, rs);
      if ((rc = run(p, kGramSquare, rs_name(false, kF32, kF32), S.fl_square[0], 0, s, [&] { return launch_gemm(S.old_cfg, kF32, kF32, gt, s); }))) return rc;
      GemmParams ga = gp(S, S.old_sym, true, kShapeSquare, kT1, hbuf, -1, kA, -1, -1, 1.f, 0.f, 0.f, 0, rs);
      if ((rc = run(p, kGramSquare, rs_name(false, kF32, kF32), S.fl_square[0], 0, s, [&] { return launch_gemm(S.old_cfg, kF32, kF32, ga, s); }))) return rc;
    }
  }
  GemmParams gf = gp(S, S.old_full, false, kShapeApply, cur, kX0, -1, kXT, -1, -1, 1.f, 0.f, 0.f, 1, rs);
  if ((rc = run(p, kGramFinal, rs_name(true, kF32, kF32), S.fl_apply[0], 0, s, [&] { return launch_gemm(S.old_cfg, kF32, kF32, gf, s); }))) return rc;
  return MUON_OK;
}

// A chunk's front and NS stages.  front(a, b, stream, ev) enqueues the front
// (momentum or input load, then k_norm) of the chunk's matrices [a, b) and,
// when ev is set, records it once the HBM-heavy part is done.  The whole
// chunk's front runs on s as one launch pair; then, with more than one lane
// (and T > 0), lane l's NS launch sets run on a stream of their own (lane 0
// on s), all lanes starting when the front is done, and lanes 1.. are
// joined back into s.  While profiling, the same launches run lane after lane
// on s, so each recorded dispatch time is the kernel's own, not shared with
// another lane.
template <class Front>
int enqueue_chunk(muon_plan* p, const ChunkDev& C, int T, const float* sched, const EwDyn* dyn,
                  float lr, float wd, hipStream_t s, Front&& front) {
  int rc;
  const int L = T > 0 ? C.n_lanes : 1;
  if (L > (int)p->lane_streams.size() + 1) return fail(MUON_EINVAL, "plan: lane without a stream");
  if (L <= 1) {
    if ((rc = front(0, (int)C.mats.size(), s, nullptr))) return rc;
    for (const SetDev& S : C.sets)
      if ((rc = enqueue_ns(p, S, T, sched, dyn, lr, wd, s))) return rc;
    return MUON_OK;
  }
  const bool serial = p->profiling;
  if ((rc = front(0, (int)C.mats.size(), s, nullptr))) return rc;
  if (!serial) HIP_TRY(hipEventRecord(p->lane_front[0], s));
  for (int l = 0; l < L; ++l) {
    hipStream_t ls = (l == 0 || serial) ? s : p->lane_streams[l - 1];
    if (l > 0 && !serial) HIP_TRY(hipStreamWaitEvent(ls, p->lane_front[0], 0));
    for (const SetDev& S : C.sets)
      if (S.lane == l && (rc = enqueue_ns(p, S, T, sched, dyn, lr, wd, ls))) return rc;
  }
  for (int l = 1; l < L && !serial; ++l) {
    HIP_TRY(hipEventRecord(p->lane_join[l - 1], p->lane_streams[l - 1]));
    HIP_TRY(hipStreamWaitEvent(s, p->lane_join[l - 1], 0));
  }
  return MUON_OK;
}

// Front of matrices [a, b) of a chunk: k_ew_momentum (load_only: d is the
// input itself) over their tiles, then k_norm over them; ev (if set) is
// recorded between the two.
int enqueue_front(muon_plan* p, const ChunkDev& C, int a, int b, float beta, int load_only,
                  hipStream_t s, hipEvent_t ev) {
  if (a >= b) {
    if (ev) HIP_TRY(hipEventRecord(ev, s));
    return MUON_OK;
  }
  double bytes = 0;
  for (int k = a; k < b; ++k) bytes += load_only ? C.mat_bytes_load[k] : C.mat_bytes_mom[k];
  const int nm = (int)C.mats.size();
  const int64_t t0 = C.tile_first[a], t1 = C.tile_first[b];
  const int nesterov = load_only ? 1 : p->host.opts.nesterov;
  int rc;
  if ((rc = run(p, kEwMom, "k_ew_momentum", 0, bytes, s, [&] {
         return launch_ew_momentum(C.ew, C.dyn, C.prefix, nm, t0, t1, C.partials, beta, nesterov,
                                   load_only, p->grid_cap, s);
       }))) return rc;
  if (ev) HIP_TRY(hipEventRecord(ev, s));
  return run(p, kNorm, "k_norm", 0, 0, s, [&] {
    return launch_norm(C.ew + a, b - a, C.partials, p->rscale, p->flags, p->host.opts.eps, s);
  });
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

// Whether stream s is being captured into a graph (the null stream never is).
int stream_capturing(hipStream_t s, bool* capturing) {
  *capturing = false;
  if (!s) return MUON_OK;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  HIP_TRY(hipStreamIsCapturing(s, &cs));
  *capturing = cs != hipStreamCaptureStatusNone;
  return MUON_OK;
}

// Pointer tables are uploaded outside graphs only: a graph captured by the
// caller reads the table from device memory at every replay, and a copy
// recorded into it would read the pinned staging buffer that later uploads
// overwrite.
const char* kCaptureTableMsg =
    "stream capture: the plan's device pointer table differs from these pointers; "
    "run one call with the same pointers outside the capture first";

// Per-matrix pointers of a chunk to the device (skipped when unchanged).
// momenta NULL: no momentum buffers (orthogonalization alone); use_capture 0:
// no update capture.  capturing: s is being captured (a changed table is
// then refused).
int upload_dyn(muon_plan* p, ChunkDev& C, void* const* params, const void* const* grads,
               float* const* momenta, bool use_capture, bool capturing, hipStream_t s) {
  const size_t nm = C.mats.size();
  std::vector<EwDyn> d(nm);
  for (size_t k = 0; k < nm; ++k) {
    const int i = C.mats[k];
    const MatPlan& M = p->host.mats[i];
    EwDyn& e = d[k];
    std::memset(&e, 0, sizeof e);
    e.w = params[i];
    e.g = grads[i];
    e.buf = momenta ? momenta[i] : nullptr;
    e.upd = use_capture ? p->capture[i] : nullptr;
    e.vec = (M.cols % 8 == 0 && aligned16(e.w) && aligned16(e.g) && aligned16(e.buf) &&
             (!e.upd || aligned16(e.upd))) ? 1 : 0;
  }
  if (C.dyn_valid && std::memcmp(d.data(), C.dyn_last.data(), nm * sizeof(EwDyn)) == 0) return MUON_OK;
  if (capturing) return fail(MUON_ESTATE, kCaptureTableMsg);
  if (C.upload_pending) HIP_TRY(hipEventSynchronize(C.upload_ev));
  std::memcpy(C.dyn_pinned, d.data(), nm * sizeof(EwDyn));
  HIP_TRY(hipMemcpyAsync(C.dyn, C.dyn_pinned, nm * sizeof(EwDyn), hipMemcpyHostToDevice, s));
  HIP_TRY(hipEventRecord(C.upload_ev, s));
  C.upload_pending = true;
  C.dyn_last = d;
  C.dyn_valid = true;
  return MUON_OK;
}

int step_impl(muon_plan* p, void* const* params, const void* const* grads, float* const* momenta,
              float lr, float beta, float wd, int T, const float* sched, void* stream) {
  if (!p) return fail(MUON_EINVAL, "plan is NULL");
  if (p->host.opts.host_only) return fail(MUON_ESTATE, "muon_step on a host-only plan");
  if (!params || !grads || !momenta) return fail(MUON_EINVAL, "NULL pointer array");
  if (T < 0 || T > 64) return fail(MUON_EINVAL, "ns_steps must be in [0, 64]");
  if (!std::isfinite(lr) || !std::isfinite(beta) || !std::isfinite(wd))
    return fail(MUON_EINVAL, "non-finite lr, beta or wd");
  for (int k = 0; k < 3 * T; ++k)
    if (!std::isfinite(sched[k])) return fail(MUON_EINVAL, "non-finite NS coefficient");
  const size_t n = p->host.mats.size();
  for (size_t i = 0; i < n; ++i)
    if (!params[i] || !grads[i] || !momenta[i]) return fail(MUON_EINVAL, "NULL matrix pointer at index " + std::to_string(i));
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc;
  bool capturing = false;
  if ((rc = stream_capturing(s, &capturing))) return rc;
  // every chunk's per-matrix pointers first (uploaded only when they changed;
  // each chunk has its own table), then the kernels
  for (ChunkDev& C : p->chunks)
    if ((rc = upload_dyn(p, C, params, grads, momenta, true, capturing, s))) return rc;
  auto enqueue = [&]() -> int {
    for (ChunkDev& C : p->chunks) {
      const int nm = (int)C.mats.size();
      int r;
      if ((r = enqueue_chunk(p, C, T, sched, C.dyn, lr, wd, s, [&](int a, int b, hipStream_t ls, hipEvent_t ev) {
             return enqueue_front(p, C, a, b, beta, 0, ls, ev);
           }))) return r;
      // with T >= 1 the last NS product of every bf16-path matrix applied its update
      if (T >= 1 && C.all_fused) continue;
      if ((r = run(p, kEwApply, "k_ew_apply", 0, T >= 1 ? C.bytes_apply_unfused : C.bytes_apply, s, [&] {
             return launch_ew_apply(C.ew, C.dyn, C.prefix, nm, C.total_tiles, p->rscale, lr, wd,
                                    T == 0 ? 1 : 0, T >= 1 ? 1 : 0, 0, p->grid_cap, s);
           }))) return r;
    }
    return MUON_OK;
  };
  if (!p->graph_on || p->profiling) return enqueue();
  if (!s) return fail(MUON_EINVAL, "graph replay needs a stream other than the null stream");
  if (capturing) return enqueue();   // the caller captures the step itself
  // the step's launches depend on the pointers (through the uploaded tables,
  // which the key pins), the update capture buffers and the scalars
  std::string key;
  const size_t n_ptr = p->host.mats.size();
  auto put = [&key](const void* v, size_t bytes) { key.append(static_cast<const char*>(v), bytes); };
  put(params, n_ptr * sizeof(void*));
  put(grads, n_ptr * sizeof(void*));
  put(momenta, n_ptr * sizeof(void*));
  if (!p->capture.empty()) put(p->capture.data(), p->capture.size() * sizeof(float*));
  const float sc[3] = {lr, beta, wd};
  put(sc, sizeof sc);
  put(&T, sizeof T);
  put(sched, 3 * (size_t)T * sizeof(float));
  if (p->graph_exec && key == p->graph_key) {
    HIP_TRY(hipGraphLaunch(p->graph_exec, s));
    return MUON_OK;
  }
  if (key != p->pending_key) {
    // first step with these arguments: eager; the next one like it is captured
    p->pending_key = key;
    return enqueue();
  }
  if (p->graph_exec) HIP_TRY(hipDeviceSynchronize());   // the old graph may still run
  drop_graph(p);
  HIP_TRY(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
  rc = enqueue();
  hipGraph_t g = nullptr;
  const hipError_t e = hipStreamEndCapture(s, &g);
  if (rc || e != hipSuccess || !g) {
    if (g) (void)hipGraphDestroy(g);
    if (rc) return rc;
    return fail(MUON_EHIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(e));
  }
  const hipError_t ie = hipGraphInstantiate(&p->graph_exec, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  if (ie != hipSuccess) {
    p->graph_exec = nullptr;
    return fail(MUON_EHIP, std::string("hipGraphInstantiate: ") + hipGetErrorString(ie));
  }
  p->graph_key = key;
  HIP_TRY(hipGraphLaunch(p->graph_exec, s));
  return MUON_OK;
}

// Orthogonalization alone: X0 = M / (||M||_F + eps), T NS steps, X_T to out.
int ortho_impl(muon_plan* p, const void* const* inputs, float* const* outputs, int T,
               const float* sched, void* stream) {
  if (!p) return fail(MUON_EINVAL, "plan is NULL");
  if (p->host.opts.host_only) return fail(MUON_ESTATE, "muon_orthogonalize on a host-only plan");
  if (!inputs || !outputs) return fail(MUON_EINVAL, "NULL pointer array");
  if (T < 0 || T > 64) return fail(MUON_EINVAL, "ns_steps must be in [0, 64]");
  for (int k = 0; k < 3 * T; ++k)
    if (!std::isfinite(sched[k])) return fail(MUON_EINVAL, "non-finite NS coefficient");
  const size_t n = p->host.mats.size();
  for (size_t i = 0; i < n; ++i)
    if (!inputs[i] || !outputs[i]) return fail(MUON_EINVAL, "NULL matrix pointer at index " + std::to_string(i));
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<void*> outs(outputs, outputs + n);
  int rc;
  bool capturing = false;
  if ((rc = stream_capturing(s, &capturing))) return rc;
  for (ChunkDev& C : p->chunks)
    if ((rc = upload_dyn(p, C, outs.data(), inputs, nullptr, false, capturing, s))) return rc;
  for (ChunkDev& C : p->chunks) {
    const int nm = (int)C.mats.size();
    // no parameters: the last NS product writes X_T (fp32) to the workspace
    if ((rc = enqueue_chunk(p, C, T, sched, nullptr, 0.f, 0.f, s, [&](int a, int b, hipStream_t ls, hipEvent_t ev) {
           return enqueue_front(p, C, a, b, 0.f, 1, ls, ev);
         }))) return rc;
    if ((rc = run(p, kEwApply, "k_ew_apply", 0, C.bytes_store, s, [&] {
           return launch_ew_apply(C.ew, C.dyn, C.prefix, nm, C.total_tiles, p->rscale, 0.f, 0.f,
                                  T == 0 ? 1 : 0, 0, 1, p->grid_cap, s);
         }))) return rc;
  }
  return MUON_OK;
}

const float kQuintic[3] = {3.4445f, -4.7750f, 2.0315f};

// Times the NS stages (T = 5) of a host plan on bounded synthetic operands:
// the workspace filled with random bf16 values of magnitude [2^-7, 2^-6)
// (read as fp32, values of the same size), X0 scaled to about unit Frobenius
// norm, so the MFMAs see real data's switching activity.  with_front: each
// chunk's front runs too, as in a step (the momentum kernel on gradients and
// momenta filled the same way, then k_norm).  best_ms: the time per step of
// the best of 3 timed repetitions.
int time_ns(PlanHost&& H, bool with_front, float* best_ms) {
  muon_plan tp;
  tp.host = std::move(H);
  int rc = materialize(&tp);
  if (rc) { free_plan_memory(&tp); return rc; }
  const size_t n = tp.host.mats.size();
  // front operands: per chunk, each matrix's gradient (its parameter dtype)
  // then its fp32 momentum, 256-byte aligned; chunks run one after another
  // and share the memory
  std::vector<void*> grads(n, nullptr);
  std::vector<float*> moms(n, nullptr);
  if (with_front) {
    auto gbytes = [](const MatPlan& M) {
      return ((size_t)M.rows * (size_t)M.cols * (M.dtype ? 2 : 4) + 255) / 256 * 256;
    };
    auto mbytes = [](const MatPlan& M) { return ((size_t)M.rows * (size_t)M.cols * 4 + 255) / 256 * 256; };
    std::vector<size_t> at(n, 0);
    size_t most = 0;
    for (const ChunkDev& C : tp.chunks) {
      size_t off = 0;
      for (int i : C.mats) {
        at[i] = off;
        off += gbytes(tp.host.mats[i]) + mbytes(tp.host.mats[i]);
      }
      most = std::max(most, off);
    }
    char* fm = nullptr;
    if ((rc = dev_alloc(&tp, &fm, most))) { free_plan_memory(&tp); return rc; }
    if (launch_fill_random_bf16(fm, most, 2, nullptr) != hipSuccess) {
      free_plan_memory(&tp);
      return fail(MUON_EHIP, "tuning setup failed");
    }
    for (size_t i = 0; i < n; ++i) {
      grads[i] = fm + at[i];
      moms[i] = reinterpret_cast<float*>(fm + at[i] + gbytes(tp.host.mats[i]));
    }
  }
  std::vector<float> r(n);
  for (size_t i = 0; i < n; ++i) {
    const MatPlan& M = tp.host.mats[i];
    r[i] = (float)(1.0 / (kTuneFillRms * std::sqrt((double)M.m_pad * M.n_pad)));
  }
  hipStream_t s = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  auto cleanup = [&] {
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (s) (void)hipStreamDestroy(s);
    free_plan_memory(&tp);
  };
  if (launch_fill_random_bf16(tp.ws, tp.host.ws_bytes, 1, nullptr) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(tp.rscale, r.data(), n * sizeof(float), hipMemcpyHostToDevice) != hipSuccess ||
      hipStreamCreate(&s) != hipSuccess || hipEventCreate(&e0) != hipSuccess ||
      hipEventCreate(&e1) != hipSuccess) {
    cleanup();
    return fail(MUON_EHIP, "tuning setup failed");
  }
  float sched[15];
  for (int i = 0; i < 5; ++i) std::memcpy(sched + 3 * i, kQuintic, sizeof kQuintic);
  // one untimed step, then 3 timed repetitions of `steps` consecutive steps
  // (enough for about 4 ms, so that short steps are not timed one by one);
  // the best repetition's time per step
  float best = 1e30f;
  int steps = 1;
  for (int rep = 0; rep < 4; ++rep) {
    (void)hipEventRecord(e0, s);
    for (int st = 0; st < steps; ++st)
    for (ChunkDev& C : tp.chunks) {
      if (with_front) {
        // the parameters are never touched (no update is applied here)
        rc = upload_dyn(&tp, C, grads.data(), grads.data(), moms.data(), false, false, s);
        if (!rc)
          rc = enqueue_chunk(&tp, C, 5, sched, nullptr, 0.f, 0.f, s, [&](int a, int b, hipStream_t ls, hipEvent_t ev) {
            return enqueue_front(&tp, C, a, b, 0.95f, 0, ls, ev);
          });
      } else {
        rc = enqueue_chunk(&tp, C, 5, sched, nullptr, 0.f, 0.f, s,
                           [](int, int, hipStream_t ls, hipEvent_t ev) {
                             if (ev) HIP_TRY(hipEventRecord(ev, ls));
                             return (int)MUON_OK;
                           });
      }
      if (rc) {
        cleanup();
        return rc;
      }
    }
    (void)hipEventRecord(e1, s);
    if (hipEventSynchronize(e1) != hipSuccess) { cleanup(); return fail(MUON_EHIP, "tuning sync failed"); }
    float ms = 0;
    (void)hipEventElapsedTime(&ms, e0, e1);
    if (rep == 0) steps = std::max(1, std::min(64, (int)std::ceil(4.0f / std::max(ms, 1e-3f))));
    else best = std::min(best, ms / steps);
  }
  cleanup();
  *best_ms = best;
  return MUON_OK;
}

// Times every candidate (form, tile plan) of one shape on a batch of equal
// matrices and keeps the fastest; a later candidate must beat the best so far
// by 3% to replace it.
int time_shape(const ShapeKey& k, const PlanOptions& base, int count,
               const std::vector<std::pair<int32_t, int32_t>>& cands, ShapeChoice* out) {
  double best_us = 0;
  bool have = false;
  for (const auto& cand : cands) {
    // the shape's real count of matrices (at most 64 and 16 GiB of workspace), so
    // the timed launches have the real launch's tile count and wave quantization
    const uint64_t per = matrix_ws_bytes(k, cand.first, cand.second);
    const int by_mem = (int)std::max<uint64_t>(1, (16ull << 30) / std::max<uint64_t>(per, 1));
    const int batch = std::max(1, std::min({64, count, by_mem}));
    PlanHost H;
    std::map<ShapeKey, ShapeChoice> ch;
    ShapeChoice c;
    c.form = cand.first;
    c.tile = cand.second;
    ch[k] = c;
    PlanOptions o = base;
    o.workspace_cap = 0;
    std::vector<int64_t> rows(batch, k.m), cols(batch, k.n);
    std::vector<int32_t> dts(batch, k.path ? MUON_BF16 : MUON_F32);
    o.precision = k.path ? MUON_PRECISION_BF16 : MUON_PRECISION_FP32;
    std::string err = build_plan(rows, cols, dts, o, ch, &H);
    if (!err.empty()) return fail(MUON_ENOMEM, "tuning: " + err);
    float ms = 0;
    const int rc = time_ns(std::move(H), false, &ms);
    if (rc) return rc;
    const double us = ms * 1000.0 / batch;
    if (!have || us < 0.97 * best_us) {
      out->form = cand.first;
      out->tile = cand.second;
      best_us = us;
      have = true;
    }
  }
  out->us = best_us;
  out->timed = true;
  return MUON_OK;
}

// Whole-set refinement.  Shapes are timed one at a time, but a stage's launch
// is shared by every matrix that uses the same kernel configuration for it, and
// lanes overlap one lane's launches with another's tails; neither shows in a
// one-shape timing.  So the whole set is timed with the per-shape choices and
// with every uniform tile plan (all bf16 direct-form shapes on plan t), each at
// 1, 2 and 4 lanes (when free), and the fastest is kept; a candidate must be
// 1.5% faster than the best so far (whole-set timings repeat to well under 1%).
int refine_set(const std::vector<int64_t>& rows, const std::vector<int64_t>& cols,
               const std::vector<int32_t>& dts, const PlanOptions& po,
               const std::map<ShapeKey, ShapeChoice>& choices, bool tiles_free, bool lanes_free,
               SetChoice* out) {
  auto with_tile = [&](int t) {
    std::map<ShapeKey, ShapeChoice> u = choices;
    if (t >= 0)
      for (auto& kv : u)
        if (kv.first.path && kv.second.form == kFormDirect) kv.second.tile = t;
    return u;
  };
  std::vector<int> tiles{-1};
  if (tiles_free)
    for (int t = 0; t < num_tile_plans(); ++t) {
      bool same = true;
      for (const auto& kv : choices)
        if (kv.first.path && kv.second.form == kFormDirect && kv.second.tile != t) same = false;
      if (!same) tiles.push_back(t);
    }
  std::vector<int> lanes{std::max(po.lanes, 1)};
  if (lanes_free) lanes = {1, 2, 3, 4};
  bool have = false;
  float best = 0;
  for (int t : tiles)
    for (int L : lanes) {
      PlanOptions o = po;
      o.lanes = L;
      PlanHost H;
      const std::string err = build_plan(rows, cols, dts, o, with_tile(t), &H);
      if (!err.empty()) return fail(MUON_ENOMEM, "tuning: " + err);
      float ms = 0;
      const int rc = time_ns(std::move(H), true, &ms);
      if (rc) return rc;
      if (!have || ms < 0.985f * best) {
        best = ms;
        out->tile = t;
        out->lanes = L;
        out->us = ms * 1000.0;
        have = true;
      }
    }
  return MUON_OK;
}

}  // namespace

extern "C" {

int muon_abi_version(void) { return MUON_ABI_VERSION; }

// ---------------------------------------------------------------- ceiling probes

namespace {

// Stream, events and device buffers of one probe run, released on every path.
struct ProbeRun {
  hipStream_t s = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  float* out = nullptr;
  ~ProbeRun() {
    if (s) (void)hipStreamSynchronize(s);
    if (out) (void)hipFree(out);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (s) (void)hipStreamDestroy(s);
  }
  int init() {
    // the probe's stream does not order itself after the caller's streams:
    // let every earlier piece of device work (e.g. the buffers' fill) finish
    HIP_TRY(hipDeviceSynchronize());
    HIP_TRY(hipStreamCreateWithFlags(&s, hipStreamNonBlocking));
    HIP_TRY(hipEventCreate(&e0));
    HIP_TRY(hipEventCreate(&e1));
    return MUON_OK;
  }
  int elapsed(double* ms) {
    HIP_TRY(hipEventSynchronize(e1));
    float f = 0.f;
    HIP_TRY(hipEventElapsedTime(&f, e0, e1));
    *ms = f;
    return MUON_OK;
  }
};

int device_cus(int* cus) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  HIP_TRY(hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev));
  if (*cus < 1) return fail(MUON_EHIP, "no compute units reported");
  return MUON_OK;
}

}  // namespace

static int probe_mfma(int iters, bool random_operands, double* tflops, double* flops) {
  if (iters < 1 || iters > (1 << 24) || !tflops) return fail(MUON_EINVAL, "iters out of [1, 2^24] or NULL tflops");
  int cus = 0, rc;
  if ((rc = device_cus(&cus))) return rc;
  const int blocks = 2 * cus;   // 8 waves per CU, two per SIMD
  ProbeRun r;
  if ((rc = r.init())) return rc;
  HIP_TRY(hipMalloc(&r.out, (size_t)blocks * 256 * sizeof(float)));
  HIP_TRY(launch_probe_mfma(blocks, iters, random_operands, r.out, r.s));   // warm-up: clocks settle
  HIP_TRY(hipEventRecord(r.e0, r.s));
  HIP_TRY(launch_probe_mfma(blocks, iters, random_operands, r.out, r.s));
  HIP_TRY(hipEventRecord(r.e1, r.s));
  double ms = 0;
  if ((rc = r.elapsed(&ms))) return rc;
  const double fl = (double)blocks * 4 * (double)iters * kProbeChains * (2.0 * 32 * 32 * 16);
  if (flops) *flops = fl;
  *tflops = ms > 0 ? fl / (ms * 1e-3) / 1e12 : 0.0;
  return MUON_OK;
}

int muon_probe_mfma_bf16(int iters, double* tflops, double* flops) {
  return probe_mfma(iters, false, tflops, flops);
}

int muon_probe_mfma_bf16_random(int iters, double* tflops, double* flops) {
  return probe_mfma(iters, true, tflops, flops);
}

int muon_probe_nt_bf16(const void* P, const void* Q, int m, int n, int k, int reps, double* tflops,
                       double* checksum) {
  if (!P || !Q || !tflops) return fail(MUON_EINVAL, "NULL pointer");
  if (m <= 0 || n <= 0 || k <= 0 || m % kProbeNtTile || n % kProbeNtTile || k % 64)
    return fail(MUON_EINVAL, "m and n must be positive multiples of 256, k a positive multiple of 64");
  if ((int64_t)m * k >= (1ll << 31) || (int64_t)n * k >= (1ll << 31))
    return fail(MUON_EINVAL, "m k and n k must stay below 2^31");
  if (!aligned16(P) || !aligned16(Q)) return fail(MUON_EINVAL, "P and Q must be 16-byte aligned");
  if (reps < 1 || reps > 100) return fail(MUON_EINVAL, "reps out of [1, 100]");
  const int64_t outn = (int64_t)(m / kProbeNtTile) * (n / kProbeNtTile) * kProbeNtThreads;
  int rc;
  ProbeRun r;
  if ((rc = r.init())) return rc;
  HIP_TRY(hipMalloc(&r.out, (size_t)outn * sizeof(float)));
  HIP_TRY(launch_probe_nt(P, Q, m, n, k, r.out, r.s));   // warm-up
  HIP_TRY(hipEventRecord(r.e0, r.s));
  for (int i = 0; i < reps; ++i) HIP_TRY(launch_probe_nt(P, Q, m, n, k, r.out, r.s));
  HIP_TRY(hipEventRecord(r.e1, r.s));
  double ms = 0;
  if ((rc = r.elapsed(&ms))) return rc;
  const double fl = 2.0 * m * (double)n * k * reps;
  *tflops = ms > 0 ? fl / (ms * 1e-3) / 1e12 : 0.0;
  if (checksum) {
    std::vector<float> h((size_t)outn);
    HIP_TRY(hipMemcpy(h.data(), r.out, h.size() * sizeof(float), hipMemcpyDeviceToHost));
    double t = 0.0;
    for (float v : h) t += v;
    *checksum = t;
  }
  return MUON_OK;
}

int muon_probe_nt_out_bf16(const void* P, const void* Q, void* C, void* CT, int m, int n, int k, int mode,
                           int reps, double* tflops) {
  if (!P || !Q || !C || !tflops || (mode >= 2 && !CT)) return fail(MUON_EINVAL, "NULL pointer");
  if (mode < 1 || mode > 3) return fail(MUON_EINVAL, "mode must be 1, 2 or 3");
  if (m <= 0 || n <= 0 || k <= 0 || m % kProbeNtTile || n % kProbeNtTile || k % 64)
    return fail(MUON_EINVAL, "m and n must be positive multiples of 256, k a positive multiple of 64");
  if ((int64_t)m * k >= (1ll << 31) || (int64_t)n * k >= (1ll << 31) || (int64_t)m * n >= (1ll << 30))
    return fail(MUON_EINVAL, "m k and n k must stay below 2^31, m n below 2^30");
  if (!aligned16(P) || !aligned16(Q) || !aligned16(C) || (mode >= 2 && !aligned16(CT)))
    return fail(MUON_EINVAL, "P, Q, C and CT must be 16-byte aligned");
  if (reps < 1 || reps > 100) return fail(MUON_EINVAL, "reps out of [1, 100]");
  int rc;
  ProbeRun r;
  if ((rc = r.init())) return rc;
  HIP_TRY(launch_probe_nt_out(P, Q, C, CT, m, n, k, mode, r.s));   // warm-up
  HIP_TRY(hipEventRecord(r.e0, r.s));
  for (int i = 0; i < reps; ++i) HIP_TRY(launch_probe_nt_out(P, Q, C, CT, m, n, k, mode, r.s));
  HIP_TRY(hipEventRecord(r.e1, r.s));
  double ms = 0;
  if ((rc = r.elapsed(&ms))) return rc;
  *tflops = ms > 0 ? 2.0 * m * (double)n * k * reps / (ms * 1e-3) / 1e12 : 0.0;
  return MUON_OK;
}

int muon_probe_hbm_copy(void* dst, const void* src, uint64_t bytes, int reps, double* gbs) {
  if (!dst || !src || !gbs) return fail(MUON_EINVAL, "NULL pointer");
  if (bytes == 0 || bytes % 16 || !aligned16(dst) || !aligned16(src))
    return fail(MUON_EINVAL, "bytes must be a non-zero multiple of 16 and both buffers 16-byte aligned");
  if (reps < 1 || reps > 1000) return fail(MUON_EINVAL, "reps out of [1, 1000]");
  const uintptr_t d = reinterpret_cast<uintptr_t>(dst), q = reinterpret_cast<uintptr_t>(src);
  if (d < q + bytes && q < d + bytes) return fail(MUON_EINVAL, "source and destination overlap");
  int cus = 0, rc;
  if ((rc = device_cus(&cus))) return rc;
  const int64_t n16 = (int64_t)(bytes / 16);
  ProbeRun r;
  if ((rc = r.init())) return rc;
  double best = 0.0;
  for (int nontemporal = 0; nontemporal < 2; ++nontemporal)
    for (int per_cu : {4, 8, 16, 0}) {
      const int blocks = per_cu * cus;   // 0: a block per 16 KiB run
      HIP_TRY(launch_probe_copy(src, dst, n16, blocks, nontemporal != 0, r.s));   // warm-up
      HIP_TRY(hipEventRecord(r.e0, r.s));
      for (int k = 0; k < reps; ++k) HIP_TRY(launch_probe_copy(src, dst, n16, blocks, nontemporal != 0, r.s));
      HIP_TRY(hipEventRecord(r.e1, r.s));
      double ms = 0;
      if ((rc = r.elapsed(&ms))) return rc;
      if (ms > 0) best = std::max(best, 2.0 * (double)bytes * reps / (ms * 1e-3) / 1e9);
    }
  *gbs = best;
  return MUON_OK;
}

const char* muon_last_error(void) { return g_err.c_str(); }

int muon_plan_opts_default(muon_plan_opts* o) {
  if (!o) return fail(MUON_EINVAL, "opts is NULL");
  std::memset(o, 0, sizeof *o);
  o->struct_size = sizeof(muon_plan_opts);
  o->nesterov = 1;
  o->eps = 1e-7f;
  o->rms_scale = 0.2f;
  o->precision = MUON_PRECISION_AUTO;
  o->form = MUON_FORM_AUTO;
  o->tile = -1;
  o->tune = MUON_TUNE_ONCE;
  o->host_only = 0;
  o->lanes = 0;
  o->workspace_cap_bytes = 0;
  o->cache_path = nullptr;
  return MUON_OK;
}

int muon_plan_create(const muon_matrix_desc* descs, int n, const muon_plan_opts* opts_in,
                     muon_plan** out) {
  g_err.clear();
  if (!out) return fail(MUON_EINVAL, "out is NULL");
  *out = nullptr;
  if (!descs || n <= 0) return fail(MUON_EINVAL, "descs is NULL or n <= 0");
  muon_plan_opts o;
  muon_plan_opts_default(&o);
  if (opts_in) {
    if (opts_in->struct_size != sizeof(muon_plan_opts)) return fail(MUON_EINVAL, "opts.struct_size mismatch");
    o = *opts_in;
  }
  if (!(o.eps >= 0.f) || !std::isfinite(o.eps) || !(o.rms_scale > 0.f) || !std::isfinite(o.rms_scale))
    return fail(MUON_EINVAL, "eps must be >= 0 and rms_scale > 0, both finite");
  if (o.precision < 0 || o.precision > 2 || o.form < 0 || o.form > 2 || o.tune < 0 || o.tune > 2 ||
      o.tile < -1 || o.tile >= num_tile_plans() || o.lanes < 0 || o.lanes > kMaxLanes)
    return fail(MUON_EINVAL, "precision, form, tile, lanes or tune out of range");
  std::vector<int64_t> rows(n), cols(n);
  std::vector<int32_t> dts(n);
  for (int i = 0; i < n; ++i) {
    if (descs[i].reserved != 0) return fail(MUON_EINVAL, "desc.reserved must be 0");
    if (descs[i].dtype != MUON_F32 && descs[i].dtype != MUON_BF16)
      return fail(MUON_EUNSUPPORTED, "unsupported dtype at index " + std::to_string(i));
    if (descs[i].rows < 1 || descs[i].cols < 1)
      return fail(MUON_EUNSUPPORTED, "zero-size matrix at index " + std::to_string(i));
    if (!dims_supported(descs[i].rows, descs[i].cols))
      return fail(MUON_EUNSUPPORTED, "matrix too large at index " + std::to_string(i));
    rows[i] = descs[i].rows;
    cols[i] = descs[i].cols;
    dts[i] = descs[i].dtype;
  }
  PlanOptions po;
  po.nesterov = o.nesterov ? 1 : 0;
  po.eps = o.eps;
  po.rms_scale = o.rms_scale;
  po.precision = o.precision;
  po.form = o.form;
  po.tile = o.tile;
  po.host_only = o.host_only ? 1 : 0;
  po.lanes = o.lanes;
  po.workspace_cap = o.workspace_cap_bytes;
  if (o.cache_path) po.cache_path = o.cache_path;
  else if (const char* env = std::getenv("MUON_TUNE_CACHE")) po.cache_path = env;
  po.tune = po.cache_path.empty() ? MUON_TUNE_OFF : o.tune;
  if (const char* env = std::getenv("MUON_TUNE")) {
    if (!std::strcmp(env, "off")) po.tune = MUON_TUNE_OFF;
  }
  int dev = -1;
  std::string tag = "host";
  if (!po.host_only) {
    if (hipGetDevice(&dev) != hipSuccess) return fail(MUON_EUNSUPPORTED, "no HIP device");
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(MUON_EHIP, "hipGetDeviceProperties failed");
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
      return fail(MUON_EUNSUPPORTED, std::string("device is ") + prop.gcnArchName + ", not gfx950");
    tag = device_tag(dev);
  }
  // per-shape choices: forced form, cache, timing, or cost model
  std::map<ShapeKey, int> counts;
  for (int i = 0; i < n; ++i) counts[shape_key(rows[i], cols[i], dts[i], po.precision)]++;
  // a host-only plan reads the cache (tag "host") but never times
  TuneCache cache;
  if (po.tune != MUON_TUNE_OFF) cache = read_cache(po.cache_path, tag);
  std::map<ShapeKey, ShapeChoice> choices;
  bool cache_dirty = false;
  for (const auto& kv : counts) {
    const ShapeKey& k = kv.first;
    // candidates worth timing: within 2x of the cost model's best
    std::vector<std::pair<int32_t, int32_t>> cands;
    {
      const auto all = candidates(k, po.form, po.tile);
      double best = 0;
      for (const auto& c : all) {
        const double us = model_cost_us(k, c.first, c.second, kv.second);
        best = (best == 0 || us < best) ? us : best;
      }
      for (const auto& c : all)
        if (model_cost_us(k, c.first, c.second, kv.second) <= 2.0 * best) cands.push_back(c);
    }
    const bool forced = po.form != MUON_FORM_AUTO || (po.tile >= 0 && k.path);
    if (cands.size() == 1) {
      ShapeChoice c;
      c.form = cands[0].first;
      c.tile = cands[0].second;
      choices[k] = c;
      continue;
    }
    auto it = cache.shapes.find(k);
    if (!forced && it != cache.shapes.end() && (po.tune == MUON_TUNE_ONCE || po.host_only)) {
      choices[k] = it->second;
      continue;
    }
    if (po.tune == MUON_TUNE_OFF || po.host_only) {
      choices[k] = model_choice(k, po.form, po.tile, kv.second);
      continue;
    }
    ShapeChoice c;
    const int rc = time_shape(k, po, kv.second, cands, &c);
    if (rc) return rc;
    choices[k] = c;
    if (!forced) {
      cache.shapes[k] = c;
      cache_dirty = true;
    }
  }
  // whole-set refinement (tuned plans; the tile plan when neither form nor tile
  // is forced, the lane count when not forced): the cached set choice, or a
  // timing when the set's workspace fits 16 GiB
  {
    bool direct_bf16 = false;
    for (const auto& kv : choices) direct_bf16 |= kv.first.path && kv.second.form == kFormDirect;
    const bool tiles_free = po.form == MUON_FORM_AUTO && po.tile < 0 && direct_bf16;
    const bool lanes_free = po.lanes == 0;
    SetChoice sc;
    sc.lanes = std::max(po.lanes, 1);
    if (po.tune != MUON_TUNE_OFF && (tiles_free || lanes_free)) {
      const std::string sk = set_key(counts, choices, po.lanes);
      const auto it = cache.sets.find(sk);
      if (it != cache.sets.end() && (po.tune == MUON_TUNE_ONCE || po.host_only)) {
        sc = it->second;
      } else if (!po.host_only) {
        PlanHost probe;
        if (build_plan(rows, cols, dts, po, choices, &probe).empty() && probe.ws_bytes <= (16ull << 30)) {
          const int rc = refine_set(rows, cols, dts, po, choices, tiles_free, lanes_free, &sc);
          if (rc) return rc;
          cache.sets[sk] = sc;
          cache_dirty = true;
        }
      }
      if (!tiles_free) sc.tile = -1;
      if (!lanes_free) sc.lanes = std::max(po.lanes, 1);
    }
    if (sc.tile >= 0)
      for (auto& kv : choices)
        if (kv.first.path && kv.second.form == kFormDirect) kv.second.tile = sc.tile;
    po.lanes = sc.lanes;
  }
  if (cache_dirty) (void)write_cache(po.cache_path, tag, cache);

  muon_plan* p = new muon_plan;
  const std::string err = build_plan(rows, cols, dts, po, choices, &p->host);
  if (!err.empty()) {
    delete p;
    return fail(MUON_ENOMEM, err);
  }
  p->serialized = serialize_plan(p->host);
  p->hash = fnv1a(p->serialized);
  p->device = dev;
  if (!po.host_only) {
    hipDeviceProp_t prop;
    // elementwise launches: up to 32 blocks per CU in flight (grid-stride beyond)
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) p->grid_cap = prop.multiProcessorCount * 32;
    const int rc = materialize(p);
    if (rc) {
      const std::string keep = g_err;
      free_plan_memory(p);
      delete p;
      g_err = keep;
      return rc;
    }
  }
  *out = p;
  return MUON_OK;
}

int muon_plan_destroy(muon_plan* p) {
  if (!p) return MUON_OK;
  free_plan_memory(p);
  delete p;
  return MUON_OK;
}

int muon_step(muon_plan* p, void* const* params, const void* const* grads, float* const* momenta,
              float lr, float beta, float wd, int ns_steps, const float* coeffs, void* stream) {
  if (ns_steps < 0 || ns_steps > 64) return fail(MUON_EINVAL, "ns_steps must be in [0, 64]");
  const float* c = coeffs ? coeffs : kQuintic;
  std::vector<float> sched(3 * (size_t)ns_steps);
  for (int k = 0; k < ns_steps; ++k) std::memcpy(&sched[3 * k], c, 3 * sizeof(float));
  return step_impl(p, params, grads, momenta, lr, beta, wd, ns_steps, sched.data(), stream);
}

int muon_step_schedule(muon_plan* p, void* const* params, const void* const* grads,
                       float* const* momenta, float lr, float beta, float wd, int ns_steps,
                       const float* coeffs, void* stream) {
  if (ns_steps > 0 && !coeffs) return fail(MUON_EINVAL, "coeffs is NULL");
  return step_impl(p, params, grads, momenta, lr, beta, wd, ns_steps, coeffs ? coeffs : kQuintic, stream);
}

int muon_orthogonalize(muon_plan* p, const void* const* inputs, float* const* outputs, int ns_steps,
                       const float* coeffs, void* stream) {
  if (ns_steps < 0 || ns_steps > 64) return fail(MUON_EINVAL, "ns_steps must be in [0, 64]");
  std::vector<float> sched(3 * (size_t)ns_steps);
  for (int k = 0; k < ns_steps; ++k)
    std::memcpy(&sched[3 * k], coeffs ? coeffs + 3 * k : kQuintic, 3 * sizeof(float));
  return ortho_impl(p, inputs, outputs, ns_steps, sched.data(), stream);
}

}  // extern "C" (reopened below)

struct muon_adamw_plan {
  int device = -1;
  int grid_cap = 2048;
  std::vector<int64_t> numels;
  std::vector<int32_t> dtypes;
  std::vector<int64_t> prefix;    // first chunk of each tensor
  int64_t total_chunks = 0;
  muon::AdamTensor* dev_tensors = nullptr;
  int64_t* dev_prefix = nullptr;
  muon::AdamTensor* pinned = nullptr;
  std::vector<muon::AdamTensor> last;
  bool valid = false, pending = false;
  hipEvent_t upload_ev = nullptr;
};

namespace {
void free_adamw(muon_adamw_plan* a) {
  if (!a) return;
  (void)hipDeviceSynchronize();
  if (a->upload_ev) (void)hipEventDestroy(a->upload_ev);
  if (a->dev_tensors) (void)hipFree(a->dev_tensors);
  if (a->dev_prefix) (void)hipFree(a->dev_prefix);
  if (a->pinned) (void)hipHostFree(a->pinned);
}
}  // namespace

extern "C" {

int muon_adamw_plan_create(const int64_t* numels, const int32_t* dtypes, int n, muon_adamw_plan** out) {
  g_err.clear();
  if (!out) return fail(MUON_EINVAL, "out is NULL");
  *out = nullptr;
  if (!numels || !dtypes || n <= 0) return fail(MUON_EINVAL, "NULL arrays or n <= 0");
  for (int i = 0; i < n; ++i) {
    if (dtypes[i] != MUON_F32 && dtypes[i] != MUON_BF16)
      return fail(MUON_EUNSUPPORTED, "unsupported dtype at index " + std::to_string(i));
    if (numels[i] < 1) return fail(MUON_EUNSUPPORTED, "empty tensor at index " + std::to_string(i));
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MUON_EUNSUPPORTED, "no HIP device");
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(MUON_EHIP, "hipGetDeviceProperties failed");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(MUON_EUNSUPPORTED, std::string("device is ") + prop.gcnArchName + ", not gfx950");
  muon_adamw_plan* a = new muon_adamw_plan;
  a->device = dev;
  a->grid_cap = 1 << 20;   // one block per chunk: measured faster than a grid-stride loop here
  a->numels.assign(numels, numels + n);
  a->dtypes.assign(dtypes, dtypes + n);
  a->prefix.resize(n);
  for (int i = 0; i < n; ++i) {
    a->prefix[i] = a->total_chunks;
    a->total_chunks += (numels[i] + kAdamChunk - 1) / kAdamChunk;
  }
  auto bad = [&](const char* what) {
    free_adamw(a);
    delete a;
    return fail(MUON_ENOMEM, what);
  };
  if (hipMalloc(&a->dev_tensors, n * sizeof(AdamTensor)) != hipSuccess) return bad("hipMalloc (AdamW table)");
  if (hipMalloc(&a->dev_prefix, n * sizeof(int64_t)) != hipSuccess) return bad("hipMalloc (AdamW prefix)");
  if (hipHostMalloc(&a->pinned, n * sizeof(AdamTensor), hipHostMallocDefault) != hipSuccess)
    return bad("hipHostMalloc (AdamW table)");
  if (hipMemcpy(a->dev_prefix, a->prefix.data(), n * sizeof(int64_t), hipMemcpyHostToDevice) != hipSuccess ||
      hipEventCreateWithFlags(&a->upload_ev, hipEventDisableTiming) != hipSuccess) {
    free_adamw(a);
    delete a;
    return fail(MUON_EHIP, "AdamW plan setup failed");
  }
  *out = a;
  return MUON_OK;
}

int muon_adamw_step(muon_adamw_plan* a, void* const* params, const void* const* grads,
                    float* const* exp_avg, float* const* exp_avg_sq, double lr, double beta1,
                    double beta2, double eps, double wd, int64_t step, void* stream) {
  g_err.clear();
  if (!a) return fail(MUON_EINVAL, "plan is NULL");
  if (!params || !grads || !exp_avg || !exp_avg_sq) return fail(MUON_EINVAL, "NULL pointer array");
  if (step < 1) return fail(MUON_EINVAL, "step must be >= 1");
  if (!(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0))
    return fail(MUON_EINVAL, "beta1 and beta2 must be in [0, 1)");
  if (!std::isfinite(lr) || !std::isfinite(wd) || !std::isfinite(eps) || eps < 0.0)
    return fail(MUON_EINVAL, "non-finite lr or wd, or eps not finite and >= 0");
  const size_t n = a->numels.size();
  std::vector<AdamTensor> t(n);
  for (size_t i = 0; i < n; ++i) {
    if (!params[i] || !grads[i] || !exp_avg[i] || !exp_avg_sq[i])
      return fail(MUON_EINVAL, "NULL tensor pointer at index " + std::to_string(i));
    AdamTensor& e = t[i];
    std::memset(&e, 0, sizeof e);
    e.p = params[i];
    e.g = grads[i];
    e.m = exp_avg[i];
    e.v = exp_avg_sq[i];
    e.n = a->numels[i];
    e.chunk_begin = a->prefix[i];
    e.pdtype = a->dtypes[i];
    e.vec = (aligned16(e.p) && aligned16(e.g) && aligned16(e.m) && aligned16(e.v)) ? 1 : 0;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!a->valid || std::memcmp(t.data(), a->last.data(), n * sizeof(AdamTensor)) != 0) {
    bool capturing = false;
    int rc;
    if ((rc = stream_capturing(s, &capturing))) return rc;
    if (capturing) return fail(MUON_ESTATE, kCaptureTableMsg);
    if (a->pending) HIP_TRY(hipEventSynchronize(a->upload_ev));
    std::memcpy(a->pinned, t.data(), n * sizeof(AdamTensor));
    HIP_TRY(hipMemcpyAsync(a->dev_tensors, a->pinned, n * sizeof(AdamTensor), hipMemcpyHostToDevice, s));
    HIP_TRY(hipEventRecord(a->upload_ev, s));
    a->pending = true;
    a->last = t;
    a->valid = true;
  }
  // bias corrections in double on the host
  const double bc1 = 1.0 - std::pow(beta1, (double)step);
  const double bc2 = 1.0 - std::pow(beta2, (double)step);
  AdamScalars sc;
  sc.beta1 = (float)beta1;
  sc.beta2 = (float)beta2;
  sc.eps = (float)eps;
  sc.omb1 = (float)(1.0 - beta1);
  sc.omb2 = (float)(1.0 - beta2);
  sc.decay = (float)(1.0 - lr * wd);
  sc.step_size = (float)(lr / bc1);
  sc.inv_bc2_sqrt = (float)(1.0 / std::sqrt(bc2));
  const hipError_t e = launch_adamw(a->dev_tensors, a->dev_prefix, (int)n, a->total_chunks, sc, a->grid_cap, s);
  if (e != hipSuccess) return fail(MUON_EHIP, std::string("adamw launch: ") + hipGetErrorString(e));
  return MUON_OK;
}

int muon_adamw_plan_destroy(muon_adamw_plan* a) {
  if (!a) return MUON_OK;
  free_adamw(a);
  delete a;
  return MUON_OK;
}

int muon_plan_set_update_capture(muon_plan* p, float* const* dst) {
  if (!p) return fail(MUON_EINVAL, "plan is NULL");
  for (size_t i = 0; i < p->capture.size(); ++i) p->capture[i] = dst ? dst[i] : nullptr;
  return MUON_OK;
}

int muon_plan_get_flags(muon_plan* p, uint32_t* flags, int clear) {
  if (!p || !flags) return fail(MUON_EINVAL, "NULL argument");
  if (p->host.opts.host_only) return fail(MUON_ESTATE, "host-only plan");
  HIP_TRY(hipDeviceSynchronize());
  HIP_TRY(hipMemcpy(flags, p->flags, sizeof(uint32_t), hipMemcpyDeviceToHost));
  if (clear) HIP_TRY(hipMemset(p->flags, 0, sizeof(uint32_t)));
  return MUON_OK;
}

int muon_plan_serialize(const muon_plan* p, void* buf, size_t* len) {
  if (!p || !len) return fail(MUON_EINVAL, "NULL argument");
  const size_t need = p->serialized.size();
  if (!buf) {
    *len = need;
    return MUON_OK;
  }
  if (*len < need) return fail(MUON_EINVAL, "buffer too small");
  std::memcpy(buf, p->serialized.data(), need);
  *len = need;
  return MUON_OK;
}

int muon_plan_info_get(const muon_plan* p, muon_plan_info* info) {
  if (!p || !info) return fail(MUON_EINVAL, "NULL argument");
  std::memset(info, 0, sizeof *info);
  info->n_matrices = (int32_t)p->host.mats.size();
  info->n_groups = (int32_t)p->host.groups.size();
  info->n_chunks = (int32_t)p->host.chunks.size();
  info->n_gram = p->host.n_gram;
  info->workspace_bytes = p->host.ws_bytes;
  plan_flops(p->host, 5, &info->ns_flops_min, &info->ns_flops_issued);
  info->ew_bytes = plan_ew_bytes(p->host);
  info->plan_hash = p->hash;
  info->n_lanes = p->host.lanes;
  return MUON_OK;
}

int muon_plan_matrix_choice(const muon_plan* p, int i, int32_t* form, int32_t* tile, int32_t* group,
                            int32_t* chunk, int32_t* lane) {
  if (!p || i < 0 || i >= (int)p->host.mats.size()) return fail(MUON_EINVAL, "bad plan or index");
  const MatPlan& M = p->host.mats[i];
  if (form) *form = M.form;
  if (tile) *tile = M.tile;
  if (group) *group = M.group;
  if (chunk) *chunk = M.chunk;
  if (lane) *lane = M.lane;
  return MUON_OK;
}

int muon_plan_matrix_cost(const muon_plan* p, int i, double* us) {
  if (!p || !us || i < 0 || i >= (int)p->host.mats.size()) return fail(MUON_EINVAL, "bad plan, index or pointer");
  *us = p->host.mats[i].cost_us;
  return MUON_OK;
}

int muon_assign_owners(const double* costs, int n, int n_owners, int64_t node_limit, int32_t* owner,
                       double* makespan, int32_t* optimal) {
  g_err.clear();
  if (n < 0 || n_owners < 1) return fail(MUON_EINVAL, "n < 0 or n_owners < 1");
  if (n > 0 && (!costs || !owner)) return fail(MUON_EINVAL, "NULL costs or owner");
  std::vector<double> c(costs ? costs : nullptr, costs ? costs + n : nullptr);
  for (int i = 0; i < n; ++i)
    if (!std::isfinite(c[i]) || c[i] < 0) return fail(MUON_EINVAL, "cost " + std::to_string(i) + " is negative or not finite");
  const AssignResult r = assign_owners(c, n_owners, node_limit > 0 ? node_limit : 2000000);
  for (int i = 0; i < n; ++i) owner[i] = r.owner[i];
  if (makespan) *makespan = r.makespan;
  if (optimal) *optimal = r.optimal ? 1 : 0;
  return MUON_OK;
}

int muon_plan_set_graph(muon_plan* p, int enable) {
  if (!p) return fail(MUON_EINVAL, "plan is NULL");
  if (p->host.opts.host_only) return fail(MUON_ESTATE, "graph replay on a host-only plan");
  if (!enable) {
    if (p->graph_exec) HIP_TRY(hipDeviceSynchronize());
    drop_graph(p);
    p->pending_key.clear();
  }
  p->graph_on = enable != 0;
  return MUON_OK;
}

int muon_plan_set_profiling(muon_plan* p, int enable) {
  if (!p) return fail(MUON_EINVAL, "plan is NULL");
  if (enable && !p->profiling) p->intervals.clear();
  p->profiling = enable != 0;
  return MUON_OK;
}

int muon_plan_get_launch_intervals(const muon_plan* p, muon_launch_interval* out, int max, int* n_out) {
  if (!p || !n_out || (max > 0 && !out)) return fail(MUON_EINVAL, "NULL argument");
  const int n = std::min<int>((int)p->intervals.size(), std::max(max, 0));
  for (int i = 0; i < n; ++i) out[i] = p->intervals[i];
  *n_out = n;
  return MUON_OK;
}

int muon_plan_get_kernel_times(muon_plan* p, muon_kernel_time* out, int max, int* n_out, int reset) {
  if (!p || !n_out || (max > 0 && !out)) return fail(MUON_EINVAL, "NULL argument");
  for (ProfRec& r : p->recs) {
    HIP_TRY(hipEventSynchronize(r.b));
    float ms = 0;
    HIP_TRY(hipEventElapsedTime(&ms, r.a, r.b));
    if (!p->prof_epoch) {
      // the first pair after a reset: its start event becomes the time origin
      p->prof_epoch = r.a;
      r.a = pool_event(p);
      if (!r.a) return fail(MUON_EHIP, "hipEventCreate failed");
    }
    float t0 = 0;
    HIP_TRY(hipEventElapsedTime(&t0, p->prof_epoch, r.b));
    muon_launch_interval iv;
    std::memset(&iv, 0, sizeof iv);
    std::strncpy(iv.name, kKindNames[r.kind], sizeof(iv.name) - 1);
    std::strncpy(iv.kernel, r.kern, sizeof(iv.kernel) - 1);
    iv.end_ms = t0;
    iv.start_ms = t0 - ms;
    p->intervals.push_back(iv);
    Totals& t = p->tot[{r.kind, std::string(r.kern)}];
    t.launches++;
    t.ms += ms;
    t.flops += r.flops;
    t.bytes += r.bytes;
    p->ev_pool.push_back(r.a);
    p->ev_pool.push_back(r.b);
  }
  p->recs.clear();
  int k = 0;
  for (const auto& kv : p->tot) {
    if (kv.second.launches == 0) continue;
    if (k < max) {
      muon_kernel_time& o = out[k];
      std::memset(&o, 0, sizeof o);
      std::strncpy(o.name, kKindNames[kv.first.first], sizeof(o.name) - 1);
      std::strncpy(o.kernel, kv.first.second.c_str(), sizeof(o.kernel) - 1);
      o.launches = kv.second.launches;
      o.total_ms = kv.second.ms;
      o.flops = kv.second.flops;
      o.bytes = kv.second.bytes;
    }
    ++k;
  }
  *n_out = std::min(k, std::max(max, 0));
  if (reset) {
    p->tot.clear();
    p->intervals.clear();
    if (p->prof_epoch) p->ev_pool.push_back(p->prof_epoch);
    p->prof_epoch = nullptr;
  }
  return MUON_OK;
}

}  // extern "C"
