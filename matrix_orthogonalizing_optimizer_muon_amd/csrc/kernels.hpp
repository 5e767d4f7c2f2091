// Device-side tables and kernel launchers of the Muon step (gfx950).
//
// Layout conventions shared by the planner, the sequencer and the kernels:
//  * "canonical" orientation: m = min(rows, cols) rows, n = max(rows, cols)
//    columns.  A tall stored matrix (rows > cols) is transposed while the
//    elementwise kernels move it between the caller's buffers and the
//    workspace, so every NS kernel sees one row-major layout.
//  * every workspace matrix is zero-padded to multiples of the NS tile size in
//    both dimensions (m_pad x n_pad, m_pad x m_pad); the kernels write the pads
//    as exact zeros each step, so the NS contractions need no bounds checks.
//  * the elementwise kernels walk 64 x 64 tiles of the padded canonical
//    extent; tile t of a chunk belongs to the matrix whose tile range holds it.
#pragma once
#include <stdint.h>
#include <hip/hip_runtime.h>

namespace muon {

constexpr int kEwTile = 64;   // elementwise tile edge (canonical elements)

enum DType : int32_t { kF32 = 0, kBF16 = 1 };

// Per matrix, static for the life of a plan (uploaded once).
struct EwMat {
  int64_t rows, cols;        // stored shape
  int64_t m, n;              // canonical real shape
  int64_t ldd;               // leading dimension of D and XT (n_pad)
  int64_t tile_begin;        // first elementwise tile of this matrix in its chunk
  int32_t tiles_i, tiles_j;  // 64-tiles along m_pad and n_pad
  int32_t trans;             // 1: canonical = stored^T
  int32_t pdtype;            // parameter / gradient dtype
  int32_t ddtype;            // NS operand dtype (D buffer)
  int32_t mat;               // index into the plan's per-matrix scale array
  void* d;                   // D: canonical NS input (m_pad x n_pad, ddtype)
  void* dt;                  // D^T (n_pad x m_pad, ddtype) or null when the NS path does not use it
  int64_t ldt;               // leading dimension of D^T (m_pad)
  float* xt;                 // X_T: final NS output (m_pad x n_pad, fp32)
  float s;                   // RMS-matching scale
  int32_t fused;             // 1: the last NS product applies the update (bf16 NT path)
};

// One tensor of a fused AdamW step: caller pointers and its place in the
// launch's chunk sequence (kAdamChunk elements per chunk).
constexpr int kAdamChunk = 2048;
struct AdamTensor {
  void* p;             // params (pdtype), n elements
  const void* g;       // grads (pdtype)
  float* m;            // first moment (fp32)
  float* v;            // second moment (fp32)
  int64_t n;
  int64_t chunk_begin; // first chunk of this tensor in the launch
  int32_t pdtype;
  int32_t vec;         // 1: all four pointers 16-byte aligned
};

// Per step scalars of AdamW (host-computed bias corrections).
struct AdamScalars {
  float beta1, beta2, eps;
  float omb1, omb2;    // 1 - beta1, 1 - beta2 (computed in double: 1 - 0.999f would be off by 1e-5)
  float decay;         // 1 - lr * wd
  float step_size;     // lr / (1 - beta1^t)
  float inv_bc2_sqrt;  // 1 / sqrt(1 - beta2^t)
};

// Per matrix, caller pointers of the current step (uploaded when they change).
struct EwDyn {
  void* w;           // params (pdtype), rows x cols
  const void* g;     // grads (pdtype)
  float* buf;        // momentum (fp32)
  float* upd;        // optional fp32 capture of the update, or null
  int32_t vec;       // 1: all four pointers 16-byte aligned and cols % 8 == 0
  int32_t pad_;
};

// Workspace buffers of one matrix in NS (ids index NsMat::buf).
enum BufId : int32_t {
  kX0 = 0,  // D / X_0 (m_pad x n_pad, NS dtype); also X ping
  kX1 = 1,  // X pong (m_pad x n_pad, NS dtype)
  kXT = 2,  // X_T (m_pad x n_pad, fp32)
  kA = 3,   // A = X X^T (direct, NS dtype) or G / A_k (Gram, fp32); m_pad x m_pad
  kB = 4,   // B = b A + c A^2 (direct, NS dtype)
  kH = 5,   // H = a I + b A + c A^2 (Gram, fp32)
  kQX = 6,  // Q ping (Gram, fp32)
  kQY = 7,  // Q pong (Gram, fp32)
  kT1 = 8,  // H A (Gram, fp32)
  kQH = 9,  // bf16 copy of Q_T (Gram, bf16 path)
  kX0T = 10, // D^T / X_0^T (n_pad x m_pad, bf16 path): the k-contiguous operand of B X
  kX1T = 11, // X pong, transposed (bf16 direct path)
  kNumBufs = 12
};

// Per matrix of a launch set: its workspace buffers and extents.
struct NsMat {
  void* buf[kNumBufs];
  int32_t m, n;          // canonical real extents
  int32_t m_pad, n_pad;  // padded extents (multiples of the tile sizes)
  int32_t mat;           // scale index
  int32_t dyn;           // index of the matrix's EwDyn in its chunk
  int32_t trans;         // 1: stored = canonical^T
  int32_t pdtype;        // parameter dtype
  int64_t cols;          // stored columns (row pitch of W)
  float s;               // RMS-matching scale
  int32_t pad_;
};

// Contraction shapes, derived per matrix from (m_pad, n_pad):
enum GemmShape : int32_t {
  kShapeGram = 0,   // (m x n)(m x n)^T -> m x m, K = n_pad        (NT, symmetric)
  kShapeSquare = 1, // (m x m)(m x m)   -> m x m, K = m_pad        (NT, Q symmetric)
  kShapeApply = 2,  // (m x m)(m x n)   -> m x n, K = m_pad        (NN)
  kShapeApplyT = 3  // (m x m)(n x m)^T -> m x n, K = m_pad        (NT, Q = X^T)
};

struct WorkItem {
  int32_t slot;      // NsMat index
  int32_t tm, tn;    // output tile coordinates
  int32_t pad_;
};

// out = s * (alpha * acc + beta * Cin) + gamma * [i == j],  s = rscale[mat]^scale_pow;
// entries outside the real extents are written as 0.
struct GemmParams {
  const WorkItem* items;
  const NsMat* mats;
  const float* rscale;
  int32_t n_items;
  int32_t shape;       // GemmShape
  int32_t scale_pow;   // 0, 1 or 2
  int32_t sym;         // 1: items are upper-triangle tiles; off-diagonal tiles are mirrored
  int32_t p_id, q_id, c_id, o_id, o2_id;   // BufId; c_id / o2_id may be -1 (none)
  int32_t ot_id;       // NT kernel: also store out^T (bf16) into this buffer, or -1
  float alpha, beta, gamma;
  // NT kernel, last NS product: instead of storing X_T, apply
  // W <- W - lr (wd W + s X_T) to the caller's parameters (and write the
  // update to the capture buffer when one is set).
  int32_t fuse;
  const EwDyn* dyn;
  float lr, wd;
  // NT kernel, kShapeApplyT: 1 = Q is X itself (m_pad x n_pad, read k-major
  // with LDS transpose reads) instead of X^T
  int32_t qt;
  // NT kernel: 1 = the staged bf16 tiles go out with nontemporal stores (set
  // when the launch writes more than the last-level cache holds, so that its
  // outputs would not stay cached for the next launch anyway)
  int32_t stream_out;
};

// Kernel configurations (the planner's tile choices).
struct TileCfg {
  int32_t bm, bn;  // output tile (rows, cols); k-tile is always 128 bytes
};
constexpr int kNumTileCfgs = 2;
constexpr TileCfg kTileCfgs[kNumTileCfgs] = {{128, 128}, {64, 64}};

// Tile configurations of the bf16 NT kernel (mfma_nt.hpp): output tile BM x BN,
// 64-element k-tiles, two LDS stages.
enum NtCfg : int32_t { kNt128 = 0, kNt256 = 1, kNt256x128 = 2, kNt128x256 = 3, kNt64 = 4, kNumNtCfgs = 5 };
constexpr TileCfg kNtCfgs[kNumNtCfgs] = {{128, 128}, {256, 256}, {256, 128}, {128, 256}, {64, 64}};

// Launchers (kernels.hip).  All return hipError_t of the launch.
// Tiles [tile_begin, tile_end) of the chunk (mats, tile_prefix: the whole chunk).
hipError_t launch_ew_momentum(const EwMat* mats, const EwDyn* dyn, const int64_t* tile_prefix,
                              int nmats, int64_t tile_begin, int64_t tile_end, float* partials,
                              float beta, int nesterov, int load_only, int grid_cap, hipStream_t s);
// One block per matrix of mats[0 .. nmats).
hipError_t launch_norm(const EwMat* mats, int nmats, const float* partials, float* rscale,
                       uint32_t* flags, float eps, hipStream_t s);
// Fused AdamW over a list of tensors (chunk_prefix[i] = tensors[i].chunk_begin).
hipError_t launch_adamw(const AdamTensor* tensors, const int64_t* chunk_prefix, int ntensors,
                        int64_t total_chunks, AdamScalars sc, int grid_cap, hipStream_t s);
// skip_fused != 0: matrices whose update the last NS product applied are skipped.
hipError_t launch_ew_apply(const EwMat* mats, const EwDyn* dyn, const int64_t* tile_prefix,
                           int nmats, int64_t total_tiles, const float* rscale, float lr,
                           float wd, int src_is_d, int skip_fused, int store_x, int grid_cap,
                           hipStream_t s);
// kShapeApply runs the NN kernel, the other shapes the NT kernel.
hipError_t launch_gemm(int tile_cfg, int in_dtype, int out_dtype, const GemmParams& p,
                       hipStream_t s);
// bf16 operands on the LDS-DMA MFMA core; shapes kShapeGram, kShapeSquare, kShapeApplyT.
// out_dtype: kF32 or kBF16; Cin (c_id) and out^T (ot_id) are bf16.
hipError_t launch_gemm_nt(int nt_cfg, int out_dtype, const GemmParams& p, hipStream_t s);

// Tuning operands: fills `bytes` (a multiple of 16) at p with random bf16
// values of random sign and magnitude in [2^-7, 2^-6) (root mean square
// 0.01193), from a hash of (seed, position).  Read as fp32, each pair of them
// is a value of the same magnitude.  Random operands make the timed kernels
// draw the power real data does (constant operands run the MFMAs faster).
constexpr double kTuneFillRms = 0.011934;
hipError_t launch_fill_random_bf16(void* p, uint64_t bytes, uint32_t seed, hipStream_t s);

// Profiling: the next kernel launched by any launcher above on this thread
// records its dispatch start and end in these events (hipExtLaunchKernel), the
// times a kernel-trace profiler reports even when streams overlap.  launched()
// says whether a kernel has been launched since the events were set.
void set_launch_events(hipEvent_t start, hipEvent_t stop);
bool launched();

}  // namespace muon
