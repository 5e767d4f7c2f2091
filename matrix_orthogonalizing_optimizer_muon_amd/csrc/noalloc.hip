// muon_step_noalloc: the Muon step of one matrix with no device allocation,
// for callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// It runs the same kernels as a plan's step with a fixed configuration:
// direct NS form, 128 x 128 tiles for every product; on the bf16 path B X
// reads X k-major (no transposed copies), so the workspace is X0, X1, A, B;
// on the fp32 path it is X0, X1, X_T, A, B.  Everything a plan keeps in its
// own device memory - the workspace, the per-tile norm partials, the scale,
// the non-finite flag, the matrix descriptors and the work-item lists - lives
// in one file-scope device array, `scratch`, of kScratchBytes per device.
// The descriptors and item lists are written into it by a small set-up kernel
// that takes them by value, so a call enqueues kernels only (no copy or
// memory-set nodes when captured).
//
// Every call on a device shares that device's array and leaves its contents
// behind: calls that overlap on one device (different streams, or threads
// without ordering) race.  Calls on one stream are ordered and safe.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>
#include <string>

#include "errors.hpp"
#include "kernels.hpp"
#include "muon.h"
#include "plan.hpp"

using namespace muon;

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // per device
constexpr int kMaxDevices = 64;
constexpr int kTile = 128;                             // NS tile edge, both paths
constexpr size_t kAlign = 256;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};   // device address of `scratch`, per device
int g_grid_cap[kMaxDevices] = {};

// the message goes to the library's muon_last_error()
int fail(int code, const std::string& msg) { return report_error(code, msg); }

// The scratch array's address and the elementwise grid cap of the current
// device, looked up once per device with that device current.
int device_setup(void** ptr, int* grid_cap) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MUON_EHIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MUON_EUNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(MUON_EHIP, std::string("hipGetDeviceProperties: ") + hipGetErrorString(e));
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
      return fail(MUON_EUNSUPPORTED, std::string("device is ") + prop.gcnArchName + ", not gfx950");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MUON_EHIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_grid_cap[dev] = prop.multiProcessorCount * 32;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  *grid_cap = g_grid_cap[dev];
  return MUON_OK;
}

// Tables the set-up kernel writes into the scratch array (by value: no copy).
struct SetupArgs {
  EwMat ew;
  EwDyn dyn;
  NsMat ns;
  EwMat* ew_dst;
  EwDyn* dyn_dst;
  NsMat* ns_dst;
  int64_t* prefix;
  uint32_t* flags;
  WorkItem* sym;     // upper-triangle tiles (tm <= tn) of the m x m products
  WorkItem* full;    // every tile of the m x n product
  int32_t tm, tn;    // tiles along m_pad and n_pad
};

__global__ __launch_bounds__(256) void k_noalloc_setup(SetupArgs a) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    *a.ew_dst = a.ew;
    *a.dyn_dst = a.dyn;
    *a.ns_dst = a.ns;
    a.prefix[0] = 0;
    a.flags[0] = 0u;   // the non-finite flag starts clear every call
  }
  const int nsym = a.tm * (a.tm + 1) / 2, nfull = a.tm * a.tn;
  for (int k = tid; k < nsym; k += blockDim.x) {
    // k-th upper-triangle tile in row order: row i holds tm - i tiles
    int i = 0, base = 0;
    while (base + (a.tm - i) <= k) {
      base += a.tm - i;
      ++i;
    }
    a.sym[k] = WorkItem{0, i, i + (k - base), 0};
  }
  for (int k = tid; k < nfull; k += blockDim.x) a.full[k] = WorkItem{0, k / a.tn, k % a.tn, 0};
}

size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

GemmParams params(const WorkItem* items, int n_items, const NsMat* mats, const float* rscale,
                  int shape, bool sym, int p_id, int q_id, int c_id, int o_id, float alpha,
                  float beta, float gamma, int scale_pow) {
  GemmParams g;
  std::memset(&g, 0, sizeof g);
  g.items = items;
  g.n_items = n_items;
  g.mats = mats;
  g.rscale = rscale;
  g.shape = shape;
  g.scale_pow = scale_pow;
  g.sym = sym ? 1 : 0;
  g.p_id = p_id;
  g.q_id = q_id;
  g.c_id = c_id;
  g.o_id = o_id;
  g.o2_id = -1;
  g.ot_id = -1;
  g.alpha = alpha;
  g.beta = beta;
  g.gamma = gamma;
  return g;
}

#define LAUNCH_TRY(what, x)                                                                   \
  do {                                                                                        \
    hipError_t e_ = (x);                                                                      \
    if (e_ != hipSuccess) return fail(MUON_EHIP, std::string(what) + ": " + hipGetErrorString(e_)); \
  } while (0)

}  // namespace

extern "C" int muon_step_noalloc(const muon_matrix_desc* desc, const muon_plan_opts* opts,
                                 void* param, const void* grad, float* momentum, float lr,
                                 float beta, float wd, int ns_steps, const float* coeffs,
                                 void* stream) {
  report_error(MUON_OK, "");
  if (!desc || !param || !grad || !momentum) return fail(MUON_EINVAL, "NULL descriptor or pointer");
  if (desc->reserved != 0) return fail(MUON_EINVAL, "desc.reserved must be 0");
  if (desc->dtype != MUON_F32 && desc->dtype != MUON_BF16) return fail(MUON_EUNSUPPORTED, "unsupported dtype");
  if (desc->rows < 1 || desc->cols < 1) return fail(MUON_EUNSUPPORTED, "zero-size matrix");
  if (!dims_supported(desc->rows, desc->cols)) return fail(MUON_EUNSUPPORTED, "matrix too large");
  int nesterov = 1;
  float eps = 1e-7f, rms = 0.2f;
  if (opts) {
    if (opts->struct_size != sizeof(muon_plan_opts)) return fail(MUON_EINVAL, "opts.struct_size mismatch");
    if (opts->form == MUON_FORM_GRAM || opts->precision != MUON_PRECISION_AUTO)
      return fail(MUON_EUNSUPPORTED, "muon_step_noalloc runs the direct form at the matrix's own precision");
    nesterov = opts->nesterov ? 1 : 0;
    eps = opts->eps;
    rms = opts->rms_scale;
  }
  if (!(eps >= 0.f) || !std::isfinite(eps) || !(rms > 0.f) || !std::isfinite(rms))
    return fail(MUON_EINVAL, "eps must be >= 0 and rms_scale > 0, both finite");
  if (ns_steps < 0 || ns_steps > 64) return fail(MUON_EINVAL, "ns_steps must be in [0, 64]");
  if (!std::isfinite(lr) || !std::isfinite(beta) || !std::isfinite(wd))
    return fail(MUON_EINVAL, "non-finite lr, beta or wd");
  static const float kQuintic[3] = {3.4445f, -4.7750f, 2.0315f};
  const float* co = coeffs ? coeffs : kQuintic;
  for (int k = 0; k < 3; ++k)
    if (!std::isfinite(co[k])) return fail(MUON_EINVAL, "non-finite NS coefficient");

  const int64_t rows = desc->rows, cols = desc->cols;
  const bool bf16 = desc->dtype == MUON_BF16;
  const bool trans = rows > cols;
  const int64_t m = trans ? cols : rows, n = trans ? rows : cols;
  const int64_t m_pad = (m + kTile - 1) / kTile * kTile, n_pad = (n + kTile - 1) / kTile * kTile;
  const int32_t tm = (int32_t)(m_pad / kTile), tn = (int32_t)(n_pad / kTile);
  const int64_t tiles = (m_pad / kEwTile) * (n_pad / kEwTile);
  const size_t es = bf16 ? 2 : 4;
  // scratch layout: tables, partials, item lists, then the workspace buffers
  size_t off = 0;
  const size_t o_ew = off; off = up(off + sizeof(EwMat));
  const size_t o_dyn = off; off = up(off + sizeof(EwDyn));
  const size_t o_ns = off; off = up(off + sizeof(NsMat));
  const size_t o_prefix = off; off = up(off + sizeof(int64_t));
  const size_t o_rscale = off; off = up(off + sizeof(float));
  const size_t o_flags = off; off = up(off + sizeof(uint32_t));
  const size_t o_part = off; off = up(off + (size_t)tiles * sizeof(float));
  const size_t o_sym = off; off = up(off + (size_t)tm * (tm + 1) / 2 * sizeof(WorkItem));
  const size_t o_full = off; off = up(off + (size_t)tm * tn * sizeof(WorkItem));
  const size_t mn = (size_t)m_pad * n_pad * es, mm = (size_t)m_pad * m_pad * es;
  const size_t o_x0 = off; off = up(off + mn);
  const size_t o_x1 = off; off = up(off + mn);
  const size_t o_a = off; off = up(off + mm);
  const size_t o_b = off; off = up(off + mm);
  size_t o_xt = 0;
  if (!bf16) { o_xt = off; off = up(off + (size_t)m_pad * n_pad * 4); }
  if (off > kScratchBytes)
    return fail(MUON_ENOMEM, "matrix " + std::to_string(rows) + "x" + std::to_string(cols) + " needs " +
                                 std::to_string(off) + " bytes of scratch; muon_step_noalloc holds " +
                                 std::to_string(kScratchBytes) + " per device");

  void* base = nullptr;
  int grid_cap = 0;
  int rc = device_setup(&base, &grid_cap);
  if (rc) return rc;
  char* S = static_cast<char*>(base);
  hipStream_t s = static_cast<hipStream_t>(stream);

  SetupArgs a;
  std::memset(&a, 0, sizeof a);
  EwMat& E = a.ew;
  E.rows = rows;
  E.cols = cols;
  E.m = m;
  E.n = n;
  E.ldd = n_pad;
  E.tile_begin = 0;
  E.tiles_i = (int32_t)(m_pad / kEwTile);
  E.tiles_j = (int32_t)(n_pad / kEwTile);
  E.trans = trans ? 1 : 0;
  E.pdtype = bf16 ? kBF16 : kF32;
  E.ddtype = bf16 ? kBF16 : kF32;
  E.mat = 0;
  E.d = S + o_x0;
  E.dt = nullptr;
  E.ldt = m_pad;
  E.xt = bf16 ? nullptr : reinterpret_cast<float*>(S + o_xt);
  E.s = (float)(rms * std::sqrt((double)n));   // as the planner forms it
  E.fused = bf16 ? 1 : 0;
  EwDyn& D = a.dyn;
  D.w = param;
  D.g = grad;
  D.buf = momentum;
  D.upd = nullptr;
  D.vec = (cols % 8 == 0 && aligned16(param) && aligned16(grad) && aligned16(momentum)) ? 1 : 0;
  NsMat& N = a.ns;
  N.buf[kX0] = S + o_x0;
  N.buf[kX1] = S + o_x1;
  N.buf[kA] = S + o_a;
  N.buf[kB] = S + o_b;
  N.buf[kXT] = bf16 ? nullptr : S + o_xt;
  N.m = (int32_t)m;
  N.n = (int32_t)n;
  N.m_pad = (int32_t)m_pad;
  N.n_pad = (int32_t)n_pad;
  N.mat = 0;
  N.dyn = 0;
  N.trans = trans ? 1 : 0;
  N.pdtype = E.pdtype;
  N.cols = cols;
  N.s = E.s;
  a.ew_dst = reinterpret_cast<EwMat*>(S + o_ew);
  a.dyn_dst = reinterpret_cast<EwDyn*>(S + o_dyn);
  a.ns_dst = reinterpret_cast<NsMat*>(S + o_ns);
  a.prefix = reinterpret_cast<int64_t*>(S + o_prefix);
  a.flags = reinterpret_cast<uint32_t*>(S + o_flags);
  a.sym = reinterpret_cast<WorkItem*>(S + o_sym);
  a.full = reinterpret_cast<WorkItem*>(S + o_full);
  a.tm = tm;
  a.tn = tn;
  hipLaunchKernelGGL(k_noalloc_setup, dim3(1), dim3(256), 0, s, a);
  LAUNCH_TRY("set-up launch", hipGetLastError());

  const EwMat* ew = a.ew_dst;
  const EwDyn* dyn = a.dyn_dst;
  const NsMat* nsm = a.ns_dst;
  float* partials = reinterpret_cast<float*>(S + o_part);
  float* rscale = reinterpret_cast<float*>(S + o_rscale);
  const int nsym = tm * (tm + 1) / 2, nfull = tm * tn;
  LAUNCH_TRY("momentum launch", launch_ew_momentum(ew, dyn, a.prefix, 1, 0, tiles, partials, beta,
                                                   nesterov, 0, grid_cap, s));
  LAUNCH_TRY("norm launch", launch_norm(ew, 1, partials, rscale, a.flags, eps, s));
  const int T = ns_steps;
  for (int k = 0; k < T; ++k) {
    const float ca = co[0], cb = co[1], cc = co[2];
    const bool even = k % 2 == 0, last = k == T - 1;
    const int src = even ? kX0 : kX1;
    const int dst = last ? kXT : (even ? kX1 : kX0);
    if (bf16) {
      // A = s X X^T; B = a I + b A + c A A; X' = t B X (X read k-major); the
      // last product applies the update to the parameters
      GemmParams g1 = params(a.sym, nsym, nsm, rscale, kShapeGram, true, src, src, -1, kA, 1.f, 0.f, 0.f,
                             k == 0 ? 2 : 0);
      LAUNCH_TRY("X X^T launch", launch_gemm_nt(kNt128, kBF16, g1, s));
      GemmParams g2 = params(a.sym, nsym, nsm, rscale, kShapeSquare, true, kA, kA, kA, kB, cc, cb, ca, 0);
      LAUNCH_TRY("A A launch", launch_gemm_nt(kNt128, kBF16, g2, s));
      GemmParams g3 = params(a.full, nfull, nsm, rscale, kShapeApplyT, false, kB, src, -1, dst, 1.f, 0.f,
                             0.f, k == 0 ? 1 : 0);
      g3.qt = 1;
      if (last) {
        g3.fuse = 1;
        g3.dyn = dyn;
        g3.lr = lr;
        g3.wd = wd;
      }
      LAUNCH_TRY("B X launch", launch_gemm_nt(kNt128, last ? kF32 : kBF16, g3, s));
    } else {
      GemmParams g1 = params(a.sym, nsym, nsm, rscale, kShapeGram, true, src, src, -1, kA, 1.f, 0.f, 0.f,
                             k == 0 ? 2 : 0);
      LAUNCH_TRY("X X^T launch", launch_gemm(0, kF32, kF32, g1, s));
      GemmParams g2 = params(a.sym, nsym, nsm, rscale, kShapeSquare, true, kA, kA, kA, kB, cc, cb, 0.f, 0);
      LAUNCH_TRY("A A launch", launch_gemm(0, kF32, kF32, g2, s));
      GemmParams g3 = params(a.full, nfull, nsm, rscale, kShapeApply, false, kB, src, src, dst, 1.f, ca,
                             0.f, k == 0 ? 1 : 0);
      LAUNCH_TRY("B X launch", launch_gemm(0, kF32, kF32, g3, s));
    }
  }
  // fp32 path (and ns_steps = 0 on either): decay and the scaled step applied
  // from X_T (or from r D when there is no NS step)
  if (!bf16 || T == 0)
    LAUNCH_TRY("apply launch", launch_ew_apply(ew, dyn, a.prefix, 1, tiles, rscale, lr, wd, T == 0 ? 1 : 0,
                                               0, 0, grid_cap, s));
  return MUON_OK;
}
