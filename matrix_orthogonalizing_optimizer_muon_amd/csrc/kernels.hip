// gfx950 kernels of the Muon update step.
//
//  k_ew_momentum  Nesterov momentum (the "momentum-based update" Muon
//                 orthogonalizes, per "DeepSpeed now supports Muon",
//                 technical deep dive), fused with the move of d into the
//                 canonical NS workspace (transposed through LDS for tall
//                 matrices) and per-tile partial sums of d^2.  HBM-bound.
//  k_norm         fixed-order reduction of those partials: r = 1/(||d||_F + eps).
//  k_gemm         the Newton-Schulz contractions on MFMA with fp32 accumulation:
//                 A = X X^T, B = b A + c A^2, X <- a X + B X, and the m x m
//                 Gram-space products (DMuon announcement, improvement 2,
//                 item 1).  LDS-staged 128-byte k-tiles, double buffered.
//  k_ew_apply     decoupled weight decay plus the RMS-matched orthogonal step
//                 (same deep-dive section), transposing back through LDS.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"
#include "mfma_nt.hpp"

namespace muon {
namespace {

// profiling events of the next launch on this thread (see set_launch_events)
thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;
thread_local bool t_launched = false;

template <typename F, typename... Args>
void launch_kernel(F kernel, dim3 grid, dim3 block, uint32_t smem, hipStream_t s, Args... args) {
  if (t_ev_start)
    hipExtLaunchKernelGGL(kernel, grid, block, smem, s, t_ev_start, t_ev_stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, smem, s, args...);
  t_ev_start = t_ev_stop = nullptr;
  t_launched = true;
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
#define GLOBAL_AS __attribute__((address_space(1)))

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 by gfx950's v_cvt_pk_bf16_f32 (two values per instruction):
// round to nearest, ties to even; NaN stays NaN.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

// 16-byte global accesses.  (Nontemporal variants were measured slower for
// every elementwise kernel here.)
__device__ __forceinline__ u32x4_t ld_u4(const void* p) {
  return *(const GLOBAL_AS u32x4_t*)p;
}

__device__ __forceinline__ void st_u4(void* p, u32x4_t v) {
  *(GLOBAL_AS u32x4_t*)p = v;
}

__device__ __forceinline__ float load1(const void* base, int dt, int64_t off) {
  if (dt == kBF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[off]);
  return static_cast<const float*>(base)[off];
}

__device__ __forceinline__ void store1(void* base, int dt, int64_t off, float v) {
  if (dt == kBF16) static_cast<uint16_t*>(base)[off] = static_cast<uint16_t>(f32_to_bf16(v));
  else static_cast<float*>(base)[off] = v;
}

// Workgroup barrier for LDS traffic only: this wave's LDS accesses complete
// (lgkmcnt(0)), then s_barrier.  __syncthreads() would also wait for every
// outstanding global access of the wave (vmcnt(0)), draining the global
// stores just issued at each barrier; no wave of these kernels reads global
// memory that another wave of its block writes.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(nt::kWaitLgkm0);
  nt::block_barrier();
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Matrix of chunk tile t: the last matrix whose first tile is <= t.
__device__ __forceinline__ int find_mat(const int64_t* prefix, int nmats, int64_t t) {
  int lo = 0, hi = nmats - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ------------------------------------------------------------ elementwise: momentum

// Four consecutive elements of dtype dt at element offset off (a multiple of
// 4 on a 16-byte aligned base): one 8-byte (bf16) or 16-byte (fp32) access.
__device__ __forceinline__ void load4_vec(const void* base, int dt, int64_t off, float* v) {
  if (dt == kBF16) {
    const u32x2_t a = *(const GLOBAL_AS u32x2_t*)(static_cast<const uint16_t*>(base) + off);
    v[0] = bf16_to_f32(a[0] & 0xffffu);
    v[1] = bf16_to_f32(a[0] >> 16);
    v[2] = bf16_to_f32(a[1] & 0xffffu);
    v[3] = bf16_to_f32(a[1] >> 16);
  } else {
    const u32x4_t t = ld_u4(static_cast<const float*>(base) + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(t[e]);
  }
}

__device__ __forceinline__ void store4_vec(void* base, int dt, int64_t off, const float* v) {
  if (dt == kBF16) {
    *(GLOBAL_AS u32x2_t*)(static_cast<uint16_t*>(base) + off) =
        u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  } else {
    st_u4(static_cast<float*>(base) + off, u32x4_t{__float_as_uint(v[0]), __float_as_uint(v[1]),
                                                   __float_as_uint(v[2]), __float_as_uint(v[3])});
  }
}

// Thread layout on a 64 x 64 tile (stored orientation): 16 lanes span one
// 64-element row segment, 4 consecutive columns each, so every wave-wide
// access covers four whole row segments (128 contiguous bytes of bf16, 256 of
// fp32).  Thread tid holds rows rq + 16 k (rq = tid / 16, k = 0..3) at
// columns cq .. cq + 3 (cq = 4 (tid % 16)).  The LDS transpose below (row
// pitch 65 floats) has two-way bank conflicts (lanes 8 apart in a row group
// share a bank; 41% of its LDS cycles on the Llama-7B set, measured), which
// this HBM-bound kernel's time does not show.
__global__ __launch_bounds__(256) void k_ew_momentum(
    const EwMat* __restrict__ mats, const EwDyn* __restrict__ dyn,
    const int64_t* __restrict__ prefix, int nmats, int64_t t_begin, int64_t t_end,
    float* __restrict__ partials, float beta, int nesterov, int load_only) {
  __shared__ float tT[kEwTile][kEwTile + 1];
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int rq = tid >> 4, cq = (tid & 15) * 4;
  for (int64_t t = t_begin + blockIdx.x; t < t_end; t += gridDim.x) {
    const int mi = find_mat(prefix, nmats, t);
    const EwMat& M = mats[mi];
    const EwDyn& D = dyn[mi];
    const int64_t lt = t - M.tile_begin;
    const int64_t i0 = (lt / M.tiles_j) * kEwTile, j0 = (lt % M.tiles_j) * kEwTile;
    const int64_t sr0 = M.trans ? j0 : i0, sc0 = M.trans ? i0 : j0;
    const bool full = D.vec && sr0 + kEwTile <= M.rows && sc0 + kEwTile <= M.cols;
    float dv[4][4];
    if (load_only) {
      // d = the input itself (orthogonalization alone: no momentum buffer)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t sr = sr0 + rq + 16 * k;
        if (full) {
          load4_vec(D.g, M.pdtype, sr * M.cols + sc0 + cq, dv[k]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t sc = sc0 + cq + e;
            dv[k][e] = (sr < M.rows && sc < M.cols) ? load1(D.g, M.pdtype, sr * M.cols + sc) : 0.f;
          }
        }
      }
    } else if (full) {
      float g[4][4], b[4][4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t off = (sr0 + rq + 16 * k) * M.cols + sc0 + cq;
        load4_vec(D.g, M.pdtype, off, g[k]);
        load4_vec(D.buf, kF32, off, b[k]);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          b[k][e] = beta * b[k][e] + g[k][e];
          dv[k][e] = nesterov ? g[k][e] + beta * b[k][e] : b[k][e];
        }
        store4_vec(D.buf, kF32, (sr0 + rq + 16 * k) * M.cols + sc0 + cq, b[k]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t sr = sr0 + rq + 16 * k;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t sc = sc0 + cq + e;
          dv[k][e] = 0.f;
          if (sr < M.rows && sc < M.cols) {
            const int64_t off = sr * M.cols + sc;
            const float g = load1(D.g, M.pdtype, off);
            const float b = beta * D.buf[off] + g;
            D.buf[off] = b;
            dv[k][e] = nesterov ? g + beta * b : b;
          }
        }
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) ss += dv[k][e] * dv[k][e];
    // dv[k] is row rq + 16 k of the tile in stored orientation: canonical row
    // i0 + rq + 16 k of D (stored = canonical) or canonical column j0 + rq +
    // 16 k, i.e. a row of D^T (tall matrices).  That orientation is stored
    // directly; the other one, when the NS path uses it, goes through an LDS
    // transpose.
    void* direct = M.trans ? M.dt : M.d;
    void* other = M.trans ? M.d : M.dt;
    const int64_t ld_dir = M.trans ? M.ldt : M.ldd, ld_oth = M.trans ? M.ldd : M.ldt;
    if (direct) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        store4_vec(direct, M.ddtype, (sr0 + rq + 16 * k) * ld_dir + sc0 + cq, dv[k]);
    }
    if (other) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) tT[cq + e][rq + 16 * k] = dv[k][e];
      lds_barrier();
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = tT[rq + 16 * k][cq + e];
        store4_vec(other, M.ddtype, (sc0 + rq + 16 * k) * ld_oth + sr0 + cq, o);
      }
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    lds_barrier();
    if (tid == 0) partials[t] = (red[0] + red[1]) + (red[2] + red[3]);
    lds_barrier();   // red and tT are reused by the next tile
  }
}

// One block per matrix: fixed-order sum of its tiles' partials.
__global__ __launch_bounds__(256) void k_norm(const EwMat* __restrict__ mats,
                                              const float* __restrict__ partials,
                                              float* __restrict__ rscale,
                                              uint32_t* __restrict__ flags, float eps) {
  __shared__ float red[4];
  const EwMat& M = mats[blockIdx.x];
  const int64_t nt = (int64_t)M.tiles_i * M.tiles_j;
  float ss = 0.f;
  for (int64_t k = threadIdx.x; k < nt; k += blockDim.x) ss += partials[M.tile_begin + k];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float nu = sqrtf(tot);
    rscale[M.mat] = 1.0f / (nu + eps);
    if (!isfinite(tot)) atomicOr(flags, 1u);
  }
}

// ------------------------------------------------------------ elementwise: AdamW
//
// "DeepSpeed now supports Muon" (setupai.cc), technical deep dive: the usual
// hybrid runs Muon on the weight matrices and AdamW on the other parameters
// (embeddings, biases, the final classifier).  AdamW with decoupled weight
// decay, per element, t the step count:
//   m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2
//   p <- p (1 - lr wd) - lr / (1 - b1^t) * m / (sqrt(v) / sqrt(1 - b2^t) + eps)
// Block: 256 threads x 8 consecutive elements = one 2048-element chunk.
__device__ __forceinline__ void adam8(float* p, const float* g, float* m, float* v,
                                      const AdamScalars& c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    m[e] = c.beta1 * m[e] + c.omb1 * g[e];
    v[e] = c.beta2 * v[e] + c.omb2 * (g[e] * g[e]);
    const float denom = sqrtf(v[e]) * c.inv_bc2_sqrt + c.eps;
    p[e] = p[e] * c.decay - c.step_size * (m[e] / denom);
  }
}

__global__ __launch_bounds__(256) void k_adamw(const AdamTensor* __restrict__ ts,
                                               const int64_t* __restrict__ prefix, int nt,
                                               int64_t total, AdamScalars c) {
  for (int64_t ch = blockIdx.x; ch < total; ch += gridDim.x) {
    const int ti = find_mat(prefix, nt, ch);
    const AdamTensor& T = ts[ti];
    const int64_t off = (ch - T.chunk_begin) * kAdamChunk + (int64_t)threadIdx.x * 8;
    if (off >= T.n) continue;
    float p[8], g[8], m[8], v[8];
    if (T.vec && off + 8 <= T.n) {
      if (T.pdtype == kBF16) {
        const u32x4_t qp = ld_u4(static_cast<const uint16_t*>(T.p) + off);
        const u32x4_t qg = ld_u4(static_cast<const uint16_t*>(T.g) + off);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[2 * e] = bf16_to_f32(qp[e] & 0xffffu);
          p[2 * e + 1] = bf16_to_f32(qp[e] >> 16);
          g[2 * e] = bf16_to_f32(qg[e] & 0xffffu);
          g[2 * e + 1] = bf16_to_f32(qg[e] >> 16);
        }
      } else {
        const float* sp = static_cast<const float*>(T.p) + off;
        const float* sg = static_cast<const float*>(T.g) + off;
        const u32x4_t a0 = ld_u4(sp), a1 = ld_u4(sp + 4);
        const u32x4_t b0 = ld_u4(sg), b1 = ld_u4(sg + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[e] = __uint_as_float(a0[e]); p[4 + e] = __uint_as_float(a1[e]);
          g[e] = __uint_as_float(b0[e]); g[4 + e] = __uint_as_float(b1[e]);
        }
      }
      const u32x4_t m0 = ld_u4(T.m + off), m1 = ld_u4(T.m + off + 4);
      const u32x4_t v0 = ld_u4(T.v + off), v1 = ld_u4(T.v + off + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        m[e] = __uint_as_float(m0[e]); m[4 + e] = __uint_as_float(m1[e]);
        v[e] = __uint_as_float(v0[e]); v[4 + e] = __uint_as_float(v1[e]);
      }
      adam8(p, g, m, v, c);
      auto u4 = [](const float* x) {
        return u32x4_t{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
      };
      st_u4(T.m + off, u4(m));
      st_u4(T.m + off + 4, u4(m + 4));
      st_u4(T.v + off, u4(v));
      st_u4(T.v + off + 4, u4(v + 4));
      if (T.pdtype == kBF16) {
        st_u4(static_cast<uint16_t*>(T.p) + off,
                    u32x4_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                            pack_bf16x2(p[6], p[7])});
      } else {
        float* dp = static_cast<float*>(T.p) + off;
        st_u4(dp, u4(p));
        st_u4(dp + 4, u4(p + 4));
      }
    } else {
      const int cnt = (int)(T.n - off < 8 ? T.n - off : 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool in = e < cnt;
        p[e] = in ? load1(T.p, T.pdtype, off + e) : 0.f;
        g[e] = in ? load1(T.g, T.pdtype, off + e) : 0.f;
        m[e] = in ? T.m[off + e] : 0.f;
        v[e] = in ? T.v[off + e] : 0.f;
      }
      adam8(p, g, m, v, c);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e < cnt) {
          store1(T.p, T.pdtype, off + e, p[e]);
          T.m[off + e] = m[e];
          T.v[off + e] = v[e];
        }
    }
  }
}

// ------------------------------------------------------------ elementwise: apply

// The update of one element: U = -lr (wd W + s x), one fused multiply-add
// written out so that every kernel that applies it rounds the same way.
__device__ __forceinline__ float update_u(float w, float x, float lr, float wd, float s) {
  return -lr * fmaf(wd, w, s * x);
}

// Same thread layout as k_ew_momentum (rows rq + 16 k, columns cq .. cq + 3).
__global__ __launch_bounds__(256) void k_ew_apply(
    const EwMat* __restrict__ mats, const EwDyn* __restrict__ dyn,
    const int64_t* __restrict__ prefix, int nmats, int64_t total,
    const float* __restrict__ rscale, float lr, float wd, int src_is_d, int skip_fused,
    int store_x) {
  __shared__ float tT[kEwTile][kEwTile + 1];
  const int tid = threadIdx.x;
  const int rq = tid >> 4, cq = (tid & 15) * 4;
  for (int64_t t = blockIdx.x; t < total; t += gridDim.x) {
    const int mi = find_mat(prefix, nmats, t);
    const EwMat& M = mats[mi];
    const EwDyn& D = dyn[mi];
    const int64_t lt = t - M.tile_begin;
    const int64_t i0 = (lt / M.tiles_j) * kEwTile, j0 = (lt % M.tiles_j) * kEwTile;
    if (i0 >= M.m || j0 >= M.n) continue;   // padding-only tile (uniform per block)
    if (skip_fused && M.fused) continue;     // the last NS product applied this matrix
    const float sx = src_is_d ? rscale[M.mat] : 1.0f;
    const void* src = src_is_d ? M.d : static_cast<const void*>(M.xt);
    const int sdt = src_is_d ? M.ddtype : kF32;
    float x[4][4];
    int64_t sr0, sc0;   // the tile's origin in stored orientation
    if (!M.trans) {
#pragma unroll
      for (int k = 0; k < 4; ++k) load4_vec(src, sdt, (i0 + rq + 16 * k) * M.ldd + j0 + cq, x[k]);
      sr0 = i0;
      sc0 = j0;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float o[4];
        load4_vec(src, sdt, (i0 + rq + 16 * k) * M.ldd + j0 + cq, o);
#pragma unroll
        for (int e = 0; e < 4; ++e) tT[rq + 16 * k][cq + e] = o[e];
      }
      lds_barrier();
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[k][e] = tT[cq + e][rq + 16 * k];
      lds_barrier();
      sr0 = j0;
      sc0 = i0;
    }
    const float s = M.s;
    const int64_t sc = sc0 + cq;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t sr = sr0 + rq + 16 * k;
      const bool vec = D.vec && sr < M.rows && sc + 4 <= M.cols;
      if (store_x) {
        // orthogonalization alone: the NS output itself, fp32, stored orientation
#pragma unroll
        for (int e = 0; e < 4; ++e) x[k][e] *= sx;
        if (vec) {
          store4_vec(D.w, kF32, sr * M.cols + sc, x[k]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (sr < M.rows && sc + e < M.cols) static_cast<float*>(D.w)[sr * M.cols + sc + e] = x[k][e];
        }
        continue;
      }
      if (vec) {
        const int64_t off = sr * M.cols + sc;
        float w[4], u[4];
        load4_vec(D.w, M.pdtype, off, w);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          u[e] = update_u(w[e], sx * x[k][e], lr, wd, s);
          w[e] = w[e] + u[e];
        }
        store4_vec(D.w, M.pdtype, off, w);
        if (D.upd) store4_vec(D.upd, kF32, off, u);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (sr < M.rows && sc + e < M.cols) {
            const int64_t off = sr * M.cols + sc + e;
            const float w = load1(D.w, M.pdtype, off);
            const float u = update_u(w, sx * x[k][e], lr, wd, s);
            store1(D.w, M.pdtype, off, w + u);
            if (D.upd) D.upd[off] = u;
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ NS contractions
//
// Block: 256 threads = 4 waves in a 2 x 2 grid, each wave a (BM/2) x (BN/2)
// sub-tile made of 32 x 32 MFMA tiles.  k advances in 128-byte tiles (64 bf16
// or 32 fp32).  Both operands sit in LDS as [row][k] with a 144-byte row pitch
// (16 bytes of padding keep the 16-byte fragment reads conflict-free); the NN
// operand is transposed on its way into LDS.  A lane's MFMA fragment is the
// 16 bytes at row (lane % 32), byte (lane / 32) * 16 of a 32-byte k-group:
// eight bf16 for one 32x32x16 MFMA, or four fp32 feeding four 32x32x2 MFMAs
// (the k order inside a group is the same permutation for both operands, so
// the sum is unchanged).

template <typename TI>
struct Mma;

template <>
struct Mma<uint16_t> {
  static __device__ __forceinline__ void run(const u32x4_t& a, const u32x4_t& b, f32x16_t& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};

template <>
struct Mma<float> {
  static __device__ __forceinline__ void run(const u32x4_t& a, const u32x4_t& b, f32x16_t& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[0]), __uint_as_float(b[0]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[1]), __uint_as_float(b[1]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[2]), __uint_as_float(b[2]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[3]), __uint_as_float(b[3]), c, 0, 0, 0);
  }
};

// Element access to workspace buffers (device global memory).
template <typename T>
__device__ __forceinline__ float ld_elem(const void* base, int64_t off) {
  if constexpr (sizeof(T) == 2)
    return bf16_to_f32(((__attribute__((address_space(1))) const uint16_t*)(base))[off]);
  else return ((__attribute__((address_space(1))) const float*)(base))[off];
}

template <typename T>
__device__ __forceinline__ void st_elem(void* base, int64_t off, float v) {
  if constexpr (sizeof(T) == 2)
    ((__attribute__((address_space(1))) uint16_t*)(base))[off] = static_cast<uint16_t>(f32_to_bf16(v));
  else ((__attribute__((address_space(1))) float*)(base))[off] = v;
}

// Four consecutive elements (one row, columns off..off+3).
template <typename T>
__device__ __forceinline__ void st_elem4(void* base, int64_t off, const float* v) {
  if constexpr (sizeof(T) == 2) {
    *((__attribute__((address_space(1))) u32x2_t*)(static_cast<uint16_t*>(base) + off)) =
        u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  } else {
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    *((__attribute__((address_space(1))) f32x4_t*)(static_cast<float*>(base) + off)) =
        f32x4_t{v[0], v[1], v[2], v[3]};
  }
}

__device__ __forceinline__ uint32_t half16(const u32x4_t& v, int e) {
  const uint32_t w = v[e >> 1];
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}
__device__ __forceinline__ uint32_t word32(const u32x4_t& v, int e) { return v[e]; }

typedef GLOBAL_AS const u32x4_t gu32x4_c;

template <int BM, int BN, bool NN, int ES>
struct GemmGeom {
  static constexpr int V = 16 / ES;      // elements per 16-byte chunk
  static constexpr int BK = 128 / ES;    // elements per k-tile
  static constexpr int ROWB = 144;       // LDS row pitch (bytes)
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int MT = WM / 32, NT = WN / 32;
  static constexpr int PCH = BM / 32;    // 16-byte P chunks per thread per k-tile
  static constexpr int QCH = BN / 32;    // Q chunks per thread (NN: consecutive k rows)
  static constexpr int STAGE = (BM + BN) * ROWB;
};

template <int BM, int BN, bool NN, int ES>
__device__ __forceinline__ void gemm_gload(u32x4_t (&pr)[BM / 32], u32x4_t (&qr)[BN / 32],
                                           const char* Pg, const char* Qg, int ldp, int ldq,
                                           int m0, int n0, int kt, int tid, int qcc, int qrg) {
  using G = GemmGeom<BM, BN, NN, ES>;
  const int64_t k0 = (int64_t)kt * G::BK;
#pragma unroll
  for (int u = 0; u < G::PCH; ++u) {
    const int c = tid + 256 * u, row = c >> 3, cc = c & 7;
    pr[u] = *(gu32x4_c*)(Pg + (((int64_t)(m0 + row) * ldp + k0) * ES) + cc * 16);
  }
  if constexpr (!NN) {
#pragma unroll
    for (int u = 0; u < G::QCH; ++u) {
      const int c = tid + 256 * u, row = c >> 3, cc = c & 7;
      qr[u] = *(gu32x4_c*)(Qg + (((int64_t)(n0 + row) * ldq + k0) * ES) + cc * 16);
    }
  } else {
#pragma unroll
    for (int u = 0; u < G::QCH; ++u) {
      const int64_t krow = k0 + qrg * G::QCH + u;
      qr[u] = *(gu32x4_c*)(Qg + ((krow * ldq + n0) * ES) + qcc * 16);
    }
  }
}

template <int BM, int BN, bool NN, int ES>
__device__ __forceinline__ void gemm_lstore(const u32x4_t (&pr)[BM / 32], const u32x4_t (&qr)[BN / 32],
                                            char* Ps, int tid, int qcc, int qrg) {
  using G = GemmGeom<BM, BN, NN, ES>;
  char* Qs = Ps + BM * G::ROWB;
#pragma unroll
  for (int u = 0; u < G::PCH; ++u) {
    const int c = tid + 256 * u, row = c >> 3, cc = c & 7;
    *reinterpret_cast<u32x4_t*>(Ps + row * G::ROWB + cc * 16) = pr[u];
  }
  if constexpr (!NN) {
#pragma unroll
    for (int u = 0; u < G::QCH; ++u) {
      const int c = tid + 256 * u, row = c >> 3, cc = c & 7;
      *reinterpret_cast<u32x4_t*>(Qs + row * G::ROWB + cc * 16) = qr[u];
    }
  } else {
    // element e of each loaded chunk is column n = qcc*V + e; its QCH k values
    // (rows qrg*QCH ..) become one contiguous run of LDS row n.
#pragma unroll
    for (int e = 0; e < G::V; ++e) {
      char* dst = Qs + (qcc * G::V + e) * G::ROWB + qrg * G::QCH * ES;
      if constexpr (ES == 2) {
        uint32_t w[G::QCH / 2];
#pragma unroll
        for (int h = 0; h < G::QCH / 2; ++h) w[h] = half16(qr[2 * h], e) | (half16(qr[2 * h + 1], e) << 16);
        if constexpr (G::QCH == 2) {
          *reinterpret_cast<uint32_t*>(dst) = w[0];
        } else if constexpr (G::QCH == 4) {
          *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{w[0], w[1]};
        } else {
#pragma unroll
          for (int h = 0; h < G::QCH / 8; ++h)
            *reinterpret_cast<u32x4_t*>(dst + 16 * h) = u32x4_t{w[4 * h], w[4 * h + 1], w[4 * h + 2], w[4 * h + 3]};
        }
      } else if constexpr (G::QCH == 2) {
        *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{word32(qr[0], e), word32(qr[1], e)};
      } else {
#pragma unroll
        for (int h = 0; h < G::QCH / 4; ++h)
          *reinterpret_cast<u32x4_t*>(dst + 16 * h) =
              u32x4_t{word32(qr[4 * h], e), word32(qr[4 * h + 1], e), word32(qr[4 * h + 2], e),
                      word32(qr[4 * h + 3], e)};
      }
    }
  }
}

template <typename TI, int BM, int BN, bool NN>
__device__ __forceinline__ void gemm_compute(f32x16_t (&acc)[BM / 64][BN / 64], const char* Ps,
                                             int lane, int wy, int wx) {
  using G = GemmGeom<BM, BN, NN, (int)sizeof(TI)>;
  const char* Qs = Ps + BM * G::ROWB;
  const int lr = lane & 31, lk = (lane >> 5) * 16;
#pragma unroll
  for (int kg = 0; kg < 4; ++kg) {
    u32x4_t af[G::MT], bfr[G::NT];
#pragma unroll
    for (int a = 0; a < G::MT; ++a)
      af[a] = *reinterpret_cast<const u32x4_t*>(Ps + (wy * G::WM + a * 32 + lr) * G::ROWB + kg * 32 + lk);
#pragma unroll
    for (int b = 0; b < G::NT; ++b)
      bfr[b] = *reinterpret_cast<const u32x4_t*>(Qs + (wx * G::WN + b * 32 + lr) * G::ROWB + kg * 32 + lk);
#pragma unroll
    for (int a = 0; a < G::MT; ++a)
#pragma unroll
      for (int b = 0; b < G::NT; ++b) Mma<TI>::run(af[a], bfr[b], acc[a][b]);
  }
}

template <typename TI, typename TO, bool NN, int BM, int BN>
__global__ __launch_bounds__(256) void k_gemm(const GemmParams p) {
  constexpr int ES = sizeof(TI);
  using G = GemmGeom<BM, BN, NN, ES>;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wy = wid >> 1, wx = wid & 1;
  const WorkItem it = p.items[blockIdx.x];
  const NsMat* nmp = p.mats + it.slot;
  const int m_pad = nmp->m_pad, n_pad = nmp->n_pad;
  const int shape = p.shape;
  int K, ldp, ldq, ldc, Mr, Nr;
  if (shape == kShapeGram) { K = n_pad; ldp = n_pad; ldq = n_pad; ldc = m_pad; Mr = nmp->m; Nr = nmp->m; }
  else if (shape == kShapeSquare) { K = m_pad; ldp = m_pad; ldq = m_pad; ldc = m_pad; Mr = nmp->m; Nr = nmp->m; }
  else { K = m_pad; ldp = m_pad; ldq = n_pad; ldc = n_pad; Mr = nmp->m; Nr = nmp->n; }
  const char* Pg = static_cast<const char*>(nmp->buf[p.p_id]);
  const char* Qg = static_cast<const char*>(nmp->buf[p.q_id]);
  const int m0 = it.tm * BM, n0 = it.tn * BN;
  const int nk = K / G::BK;
  const int qcc = tid % (BN / G::V), qrg = tid / (BN / G::V);

  u32x4_t pr[G::PCH], qr[G::QCH];
  f32x16_t acc[G::MT][G::NT];
#pragma unroll
  for (int a = 0; a < G::MT; ++a)
#pragma unroll
    for (int b = 0; b < G::NT; ++b)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[a][b][q] = 0.f;

  gemm_gload<BM, BN, NN, ES>(pr, qr, Pg, Qg, ldp, ldq, m0, n0, 0, tid, qcc, qrg);
  gemm_lstore<BM, BN, NN, ES>(pr, qr, smem, tid, qcc, qrg);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) gemm_gload<BM, BN, NN, ES>(pr, qr, Pg, Qg, ldp, ldq, m0, n0, kt + 1, tid, qcc, qrg);
    gemm_compute<TI, BM, BN, NN>(acc, smem + cur * G::STAGE, lane, wy, wx);
    if (more) gemm_lstore<BM, BN, NN, ES>(pr, qr, smem + (cur ^ 1) * G::STAGE, tid, qcc, qrg);
    __syncthreads();
  }

  // ---- epilogue
  float s = 1.0f;
  if (p.scale_pow) {
    const float rr = p.rscale[nmp->mat];
    s = p.scale_pow == 2 ? rr * rr : rr;
  }
  const float alpha = p.alpha, beta = p.beta, gamma = p.gamma;
  void* Out = nmp->buf[p.o_id];
  void* Out2 = p.o2_id >= 0 ? nmp->buf[p.o2_id] : nullptr;
  const void* Cin = p.c_id >= 0 ? nmp->buf[p.c_id] : nullptr;
  const int ldo = ldc;
  const bool mirror = p.sym && it.tm != it.tn;
#pragma unroll
  for (int a = 0; a < G::MT; ++a) {
#pragma unroll
    for (int b = 0; b < G::NT; ++b) {
      const int j = n0 + wx * G::WN + b * 32 + (lane & 31);
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int ib = m0 + wy * G::WM + a * 32 + rg * 8 + (lane >> 5) * 4;
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = ib + q;
          float x = alpha * acc[a][b][rg * 4 + q];
          if (Cin) x += beta * ld_elem<TI>(Cin, (int64_t)i * ldc + j);
          x *= s;
          if (i == j) x += gamma;
          if (i >= Mr || j >= Nr) x = 0.f;
          v[q] = x;
          st_elem<TO>(Out, (int64_t)i * ldo + j, x);
          if (Out2) st_elem<uint16_t>(Out2, (int64_t)i * ldo + j, x);
        }
        if (mirror) {
          st_elem4<TO>(Out, (int64_t)j * ldo + ib, v);
          if (Out2) st_elem4<uint16_t>(Out2, (int64_t)j * ldo + ib, v);
        }
      }
    }
  }
}

template <typename TI, typename TO, bool NN, int BM, int BN>
hipError_t launch_gemm_t(const GemmParams& p, hipStream_t s) {
  constexpr int smem = 2 * (BM + BN) * 144;
  static bool attr_done = false;
  auto kern = &k_gemm<TI, TO, NN, BM, BN>;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  if (p.n_items <= 0) return hipSuccess;
  launch_kernel(kern, dim3(p.n_items), dim3(256), smem, s, p);
  return hipGetLastError();
}

template <int BM, int BN>
hipError_t launch_gemm_cfg(int in_dt, int out_dt, const GemmParams& p, hipStream_t s) {
  const bool nn = p.shape == kShapeApply;
  if (in_dt == kBF16 && out_dt == kBF16)
    return nn ? launch_gemm_t<uint16_t, uint16_t, true, BM, BN>(p, s)
              : launch_gemm_t<uint16_t, uint16_t, false, BM, BN>(p, s);
  if (in_dt == kBF16 && out_dt == kF32)
    return nn ? launch_gemm_t<uint16_t, float, true, BM, BN>(p, s)
              : launch_gemm_t<uint16_t, float, false, BM, BN>(p, s);
  if (in_dt == kF32 && out_dt == kF32)
    return nn ? launch_gemm_t<float, float, true, BM, BN>(p, s)
              : launch_gemm_t<float, float, false, BM, BN>(p, s);
  return hipErrorInvalidValue;
}

// ------------------------------------------------------- bf16 NT contractions
//
// The NS products on the LDS-DMA MFMA core of mfma_nt.hpp.  Both operands are
// row-major with k contiguous:
//   kShapeGram    A = X X^T       P = Q = X (m_pad x n_pad), K = n_pad, out m x m
//   kShapeSquare  C = A A         P = Q = A (m_pad x m_pad, symmetric), K = m_pad
//   kShapeApplyT  C = B X         P = B (m_pad x m_pad), Q = X^T (n_pad x m_pad), K = m_pad
// (B X needs X^T because its k index runs down the columns of X; every NS
// step therefore keeps X in both orientations.)  Epilogue as GemmParams: the
// output in TO, optionally its transpose (bf16) and, for upper-triangle
// symmetric tiles, the mirrored tile.

// Pipeline of each NT configuration: k-tile (elements) and LDS stages.  One
// setting serves all five: k-tiles of 32 with three or four stages were
// measured slower on the 128x128 and the 256x256 tiles.
// LDS_CAP: the LDS a block may take without lowering the blocks per CU its
// registers allow (two 128x128 blocks per CU, one of any other).
// One random bf16 (sign, fixed exponent 2^-7, 7 random mantissa bits) from a
// 32-bit hash of its key.
__device__ __forceinline__ uint32_t tune_bf16(uint32_t key) {
  key ^= key >> 16;
  key *= 0x7feb352du;
  key ^= key >> 15;
  key *= 0x846ca68bu;
  key ^= key >> 16;
  return (key & 0x8000u) | (120u << 7) | (key & 0x7fu);
}

__global__ __launch_bounds__(256) void k_fill_random_bf16(u32x4_t* __restrict__ p, int64_t n16, uint32_t seed) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const uint32_t b = (uint32_t)(i * 8) ^ (seed * 0x9e3779b9u) ^ (uint32_t)(i >> 29);
    u32x4_t v;
#pragma unroll
    for (int w = 0; w < 4; ++w) v[w] = tune_bf16(b + 2 * w) | (tune_bf16(b + 2 * w + 1) << 16);
    p[i] = v;
  }
}

template <int BM, int BN, int WGM, int WGN>
struct NtPipe {
  static constexpr int BK = 64, S = 2;
  static constexpr int LDS_CAP = (BM == 64 && BN == 64)     ? 32 * 1024
                                 : (BM == 128 && BN == 128) ? 80 * 1024
                                                            : 160 * 1024;
};

// Rows of the output tile staged in LDS at a time: the largest power of two
// whose fp32 slab (row pitch BN + 4 floats) fits the block's LDS budget.
template <int BM, int BN, int WGM, int WGN>
constexpr int slab_rows() {
  int sh = BM;
  while (sh > 8 && sh * (BN + 4) * 4 > NtPipe<BM, BN, WGM, WGN>::LDS_CAP) sh /= 2;
  return sh;
}

// Row pitch (elements) of the bf16 epilogue tile.
template <int BN>
constexpr int bf16_pitch() { return BN + 8; }

// Dynamic LDS of a block: the main loop's stages, the fp32 epilogue slab or the
// whole output tile in bf16, whichever is largest (they never live at once).
template <int BM, int BN, int WGM, int WGN>
constexpr int nt_lds() {
  using P = NtPipe<BM, BN, WGM, WGN>;
  constexpr int stages = nt::Geom<BM, BN, P::BK, P::S, WGM, WGN>::LDS;
  constexpr int slab = slab_rows<BM, BN, WGM, WGN>() * (BN + 4) * 4;
  constexpr int tile16 = BM * bf16_pitch<BN>() * 2;
  static_assert(stages <= P::LDS_CAP && slab <= P::LDS_CAP && tile16 <= P::LDS_CAP, "LDS budget");
  constexpr int m = stages > slab ? stages : slab;
  return m > tile16 ? m : tile16;
}

template <typename TO>
__device__ __forceinline__ void st8(void* base, int64_t off, const float* v) {
  if constexpr (sizeof(TO) == 2) {
    *(GLOBAL_AS u32x4_t*)(static_cast<uint16_t*>(base) + off) =
        u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                pack_bf16x2(v[6], v[7])};
  } else {
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    GLOBAL_AS f32x4_t* d = (GLOBAL_AS f32x4_t*)(static_cast<float*>(base) + off);
    d[0] = f32x4_t{v[0], v[1], v[2], v[3]};
    d[1] = f32x4_t{v[4], v[5], v[6], v[7]};
  }
}

// A 16-byte output store of the staged epilogues (element offset off of a
// bf16 buffer), nontemporal when the launch streams its outputs
// (GemmParams::stream_out).  The nontemporal form is a buffer store whose
// cache policy is an immediate, so the compiler cannot fold the two forms
// into one store and drop the hint; its descriptor spans 4 GiB from base,
// and every output buffer is smaller than 2 GiB.
constexpr int kCpolNt = 2;   // cache-policy operand: the nt bit
__device__ __forceinline__ void st_out16(void* base, int64_t off, u32x4_t v, bool stream) {
  if (stream) {
    const __amdgpu_buffer_rsrc_t r = nt::make_rsrc(base, 0xFFFFFFFFu);
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (uint32_t)(off * 2), 0, kCpolNt);
  } else {
    *(GLOBAL_AS u32x4_t*)(static_cast<uint16_t*>(base) + off) = v;
  }
}

// What the weight update applied in an epilogue needs, read once per block
// (the output stores may alias the descriptor tables, so nothing is re-read).
struct UpdCtx {
  void* w;          // stored W (rows x cols, row-major)
  float* upd;       // capture of U, or null
  int64_t cols;
  float s, lr, wd;  // RMS-matching scale, learning rate, weight decay
  int32_t pdtype;
  int32_t vec;      // W (and the capture) aligned for 16-byte runs, cols % 8 == 0
};

// Decoupled weight decay and the RMS-scaled orthogonal step on 8 consecutive
// stored bf16 elements of W at element offset `off`, whose current values wq
// were loaded ahead: U = -lr (wd W + s x), W <- RNE(W + U); U also goes to the
// capture buffer when one is set.
__device__ __forceinline__ void apply_update8_bf16(const UpdCtx& c, int64_t off, u32x4_t wq,
                                                   const float* x) {
  float w[8], u[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    w[2 * e] = bf16_to_f32(wq[e] & 0xffffu);
    w[2 * e + 1] = bf16_to_f32(wq[e] >> 16);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    u[e] = update_u(w[e], x[e], c.lr, c.wd, c.s);
    w[e] = w[e] + u[e];
  }
  *(GLOBAL_AS u32x4_t*)(static_cast<uint16_t*>(c.w) + off) =
      u32x4_t{pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]), pack_bf16x2(w[4], w[5]),
              pack_bf16x2(w[6], w[7])};
  if (c.upd) {
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    GLOBAL_AS f32x4_t* dst = (GLOBAL_AS f32x4_t*)(c.upd + off);
    dst[0] = f32x4_t{u[0], u[1], u[2], u[3]};
    dst[1] = f32x4_t{u[4], u[5], u[6], u[7]};
  }
}

// The same update on `nvalid` (<= 8) consecutive stored elements of W starting
// at (row, col0), loading W itself (any parameter dtype, any alignment).
__device__ __forceinline__ void apply_update8(const UpdCtx& c, int64_t row, int64_t col0, int nvalid,
                                              const float* x) {
  if (nvalid <= 0) return;
  const int64_t off = row * c.cols + col0;
  const float sc = c.s, lr = c.lr, wd = c.wd;
  const int dt = c.pdtype;
  if (c.vec && nvalid == 8) {
    if (dt == kBF16) {
      apply_update8_bf16(c, off, *(GLOBAL_AS const u32x4_t*)(static_cast<const uint16_t*>(c.w) + off), x);
      return;
    }
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    GLOBAL_AS f32x4_t* src = (GLOBAL_AS f32x4_t*)(static_cast<float*>(c.w) + off);
    const f32x4_t a = src[0], b = src[1];
    float w[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}, u[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      u[e] = update_u(w[e], x[e], lr, wd, sc);
      w[e] = w[e] + u[e];
    }
    src[0] = f32x4_t{w[0], w[1], w[2], w[3]};
    src[1] = f32x4_t{w[4], w[5], w[6], w[7]};
    if (c.upd) {
      GLOBAL_AS f32x4_t* dst = (GLOBAL_AS f32x4_t*)(c.upd + off);
      dst[0] = f32x4_t{u[0], u[1], u[2], u[3]};
      dst[1] = f32x4_t{u[4], u[5], u[6], u[7]};
    }
    return;
  }
  for (int e = 0; e < nvalid; ++e) {
    const float w = load1(c.w, dt, off + e);
    const float u = update_u(w, x[e], lr, wd, sc);
    store1(c.w, dt, off + e, w + u);
    if (c.upd) c.upd[off + e] = u;
  }
}

// Epilogue of the NT kernel.  With only bf16 outputs to write (no Cin or
// update: the row-major output and possibly its transposed copy or mirrored
// tile) the values are finished in registers and the whole tile goes through
// LDS once, as bf16, for a row pass and a column pass.  Otherwise it goes
// through LDS in fp32 slabs of SH rows:
//  1. each wave writes its accumulators of the slab's rows into an fp32 tile;
//  2. row pass: every thread takes 8 consecutive columns of a row, applies
//     out = (s alpha) acc + (s beta) Cin + gamma [i == j] (0 outside the real
//     extents) and stores 16-byte runs of the output (Cin read the same way);
//  3. column pass (transposed copy or mirrored tile only): every thread takes 8
//     consecutive rows of one column and stores them as a 16-byte run; the
//     lanes of a wave cover 4 columns x 16 row groups, so each store
//     instruction writes four 256-byte runs of the transposed output.
template <int BM, int BN, int WGM, int WGN, typename TO>
__device__ __forceinline__ void nt_epilogue(const nt::f32x16_t (&acc)[BM / 32 / WGM][BN / 32 / WGN],
                                            MUON_LDS float* C, const GemmParams& p,
                                            const NsMat* nmp, int m0, int n0, int ldo, int Mr,
                                            int Nr) {
  using PP = NtPipe<BM, BN, WGM, WGN>;
  using G = nt::Geom<BM, BN, PP::BK, PP::S, WGM, WGN>;
  constexpr int NT = G::THREADS;
  constexpr int SH = slab_rows<BM, BN, WGM, WGN>();
  constexpr int PITCH = BN + 4;
  constexpr int TPR = BN / 8, RPP = NT / TPR;
  static_assert(SH % 32 == 0 && PITCH % 4 == 0 && SH * PITCH * 4 <= nt_lds<BM, BN, WGM, WGN>() &&
                NT % TPR == 0, "slab");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wy = w / WGN, wx = w % WGN;
  float sc = 1.0f;
  if (p.scale_pow) {
    const float rr = p.rscale[nmp->mat];
    sc = p.scale_pow == 2 ? rr * rr : rr;
  }
  const float gamma = p.gamma;
  const float as = p.alpha * sc, bs = p.beta * sc;
  // only tiles that reach past the real extents, or that the diagonal crosses
  // when gamma is added there, need the per-element checks
  const bool edge = m0 + BM > Mr || n0 + BN > Nr || (gamma != 0.f && m0 < n0 + BN && n0 < m0 + BM);
  void* Out = nmp->buf[p.o_id];
  void* OutT = p.ot_id >= 0 ? nmp->buf[p.ot_id] : nullptr;
  const void* Cin = p.c_id >= 0 ? nmp->buf[p.c_id] : nullptr;
  const WorkItem it = p.items[blockIdx.x];
  const bool mirror = p.sym && it.tm != it.tn;
  const bool fuse = p.fuse != 0, ftrans = fuse && nmp->trans;
  const bool stream = p.stream_out != 0;
  const bool colpass = mirror || OutT != nullptr || ftrans;
  const int m_pad = nmp->m_pad;
  UpdCtx uc = {nullptr, nullptr, 0, 0.f, 0.f, 0.f, 0, 0};
  if (fuse) {
    const EwDyn* d = p.dyn + nmp->dyn;
    uc = UpdCtx{d->w, d->upd, nmp->cols, nmp->s, p.lr, p.wd, nmp->pdtype, d->vec};
  }
  // the update's W runs are loaded ahead when they are aligned bf16 runs
  const bool wvec = fuse && uc.pdtype == kBF16 && uc.vec;
  const bool wrow = wvec && !ftrans, wcol = wvec && ftrans;
  if constexpr (sizeof(TO) == 2) {
    {
      // bf16 outputs (the row-major output, with or without a transposed copy
      // or mirrored tile; the launcher refuses an update fused into a bf16
      // launch): each lane finishes its values in registers (4
      // consecutive columns of a row per register group) and the whole tile is
      // staged once in LDS as bf16, element (r, col) at r PB + (col ^ 8 ((r >>
      // 3) & 7)).  The XOR keeps 8-element (16-byte) groups whole and puts the
      // eight 8-row groups of a column on distinct bank quads.  A row pass
      // stores 16-byte row runs; for the transposed copy or mirror a column
      // pass follows in which the 4 lanes of a quad take 4 columns and
      // consecutive quads consecutive 8-row groups, so every store instruction
      // writes four 256-byte runs of transposed rows and the 2-byte LDS reads
      // of a column spread over the banks.  With Cin, its tile is first copied into the same
      // staging layout (16-byte row runs), and each lane combines the values
      // at its own positions in fp32 before they are rounded once to bf16.
      constexpr int PB = bf16_pitch<BN>();
      constexpr int TPR = BN / 8, RPP = NT / TPR;
      MUON_LDS uint16_t* Cb = reinterpret_cast<MUON_LDS uint16_t*>(C);
      auto at = [&](int r, int col) { return Cb + r * PB + (col ^ (8 * ((r >> 3) & 7))); };
      const int cc = (tid % TPR) * 8;
      if (Cin) {
        // rows of this thread in batches of CB 16-byte loads (all of a batch
        // in flight at once, within the registers the accumulators leave)
        constexpr int CR = BM / RPP, CB = CR < 8 ? CR : 8;
        static_assert(BM % RPP == 0 && CR % CB == 0, "Cin rows per thread");
#pragma unroll
        for (int t0 = 0; t0 < CR; t0 += CB) {
          u32x4_t cr[CB];
#pragma unroll
          for (int t = 0; t < CB; ++t)
            cr[t] = *(GLOBAL_AS const u32x4_t*)(static_cast<const uint16_t*>(Cin) +
                                                (int64_t)(m0 + tid / TPR + (t0 + t) * RPP) * ldo + n0 + cc);
          if (t0 == 0) lds_barrier();   // every wave is done with the main loop's LDS
#pragma unroll
          for (int t = 0; t < CB; ++t) *(MUON_LDS u32x4_t*)at(tid / TPR + (t0 + t) * RPP, cc) = cr[t];
        }
      }
      lds_barrier();   // the main loop's LDS is free; Cin (if any) is staged
#pragma unroll
      for (int a = 0; a < G::MT; ++a) {
        const int r = wy * G::WM + a * 32 + (lane & 31), i = m0 + r;
#pragma unroll
        for (int b = 0; b < G::NT; ++b)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int c = wx * G::WN + b * 32 + g * 8 + (lane >> 5) * 4, j = n0 + c;
            float v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = as * acc[a][b][4 * g + q];
            if (Cin) {
              const u32x2_t c2 = *(const MUON_LDS u32x2_t*)at(r, c);
              v[0] = fmaf(bs, bf16_to_f32(c2[0] & 0xffffu), v[0]);
              v[1] = fmaf(bs, bf16_to_f32(c2[0] >> 16), v[1]);
              v[2] = fmaf(bs, bf16_to_f32(c2[1] & 0xffffu), v[2]);
              v[3] = fmaf(bs, bf16_to_f32(c2[1] >> 16), v[3]);
            }
            if (edge) {
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                if (i == j + q) v[q] += gamma;
                if (i >= Mr || j + q >= Nr) v[q] = 0.f;
              }
            }
            *(MUON_LDS u32x2_t*)at(r, c) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          }
      }
      lds_barrier();
#pragma unroll 4
      for (int r = tid / TPR; r < BM; r += RPP)
        st_out16(Out, (int64_t)(m0 + r) * ldo + n0 + cc, *(const MUON_LDS u32x4_t*)at(r, cc), stream);
      if (colpass) {
        // items (column jc, 8-row group r0): item wi is column 4 (wi / (4 GR))
        // + wi % 4 and row group (wi / 4) % GR; with NT a multiple of 4 GR a
        // thread keeps its row group and steps its column by NT / GR
        constexpr int GR = BM / 8;
        static_assert(BN * GR % NT == 0 && NT % (4 * GR) == 0, "column items per thread");
        const int jc0 = 4 * (tid / (4 * GR)) + tid % 4, r0 = ((tid / 4) % GR) * 8;
        const int i0 = m0 + r0;
#pragma unroll 2
        for (int ci = 0; ci < BN * GR / NT; ++ci) {
          const int jc = jc0 + ci * (NT / GR), j = n0 + jc;
          uint32_t w[4];
#pragma unroll
          for (int h = 0; h < 4; ++h)
            w[h] = (uint32_t)*at(r0 + 2 * h, jc) | ((uint32_t)*at(r0 + 2 * h + 1, jc) << 16);
          const u32x4_t q = u32x4_t{w[0], w[1], w[2], w[3]};
          if (OutT) st_out16(OutT, (int64_t)j * m_pad + i0, q, stream);
          if (mirror) st_out16(Out, (int64_t)j * ldo + i0, q, stream);
        }
      }
      return;
    }
  }
  if constexpr (sizeof(TO) == 4) {
    if (wvec && !edge) {
      // The update applied to an interior tile of bf16 parameters: W's tile
      // is staged in LDS as bf16 in the layout of the bf16 epilogue above (W's
      // row runs, or for a transposed matrix its column runs, scattered 2 bytes
      // at a time the way the column pass gathers them), each lane updates the
      // elements at its own accumulator positions in fp32 and rounds each once,
      // and the tile goes back to W in 16-byte runs (the row pass, or for a
      // transposed matrix the column pass).  The capture of U, when set, is
      // written from the lanes' registers.
      constexpr int PB = bf16_pitch<BN>();
      constexpr int TPR = BN / 8, RPP = NT / TPR, GR = BM / 8, CI = BN * GR / NT;
      static_assert(BM % RPP == 0 && BN * GR % NT == 0 && NT % (4 * GR) == 0, "staged update items");
      MUON_LDS uint16_t* Cb = reinterpret_cast<MUON_LDS uint16_t*>(C);
      auto at = [&](int r, int col) { return Cb + r * PB + (col ^ (8 * ((r >> 3) & 7))); };
      uint16_t* W = static_cast<uint16_t*>(uc.w);
      const int64_t ldw = uc.cols;
      const int cc = (tid % TPR) * 8;
      const int jc0 = 4 * (tid / (4 * GR)) + tid % 4, r0 = ((tid / 4) % GR) * 8;
      if (!ftrans) {
        constexpr int CR = BM / RPP, CB = CR < 8 ? CR : 8;
        static_assert(CR % CB == 0, "W rows per thread");
#pragma unroll
        for (int t0 = 0; t0 < CR; t0 += CB) {
          u32x4_t q[CB];
#pragma unroll
          for (int t = 0; t < CB; ++t)
            q[t] = *(GLOBAL_AS const u32x4_t*)(W + (int64_t)(m0 + tid / TPR + (t0 + t) * RPP) * ldw + n0 + cc);
          if (t0 == 0) lds_barrier();   // every wave is done with the main loop's LDS
#pragma unroll
          for (int t = 0; t < CB; ++t) *(MUON_LDS u32x4_t*)at(tid / TPR + (t0 + t) * RPP, cc) = q[t];
        }
      } else {
        constexpr int CB = CI < 8 ? CI : 8;
        static_assert(CI % CB == 0, "W column runs per thread");
#pragma unroll
        for (int t0 = 0; t0 < CI; t0 += CB) {
          u32x4_t q[CB];
#pragma unroll
          for (int t = 0; t < CB; ++t)
            q[t] = *(GLOBAL_AS const u32x4_t*)(W + (int64_t)(n0 + jc0 + (t0 + t) * (NT / GR)) * ldw + m0 + r0);
          if (t0 == 0) lds_barrier();   // every wave is done with the main loop's LDS
#pragma unroll
          for (int t = 0; t < CB; ++t) {
            const int jc = jc0 + (t0 + t) * (NT / GR);
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              *at(r0 + 2 * h, jc) = (uint16_t)(q[t][h] & 0xffffu);
              *at(r0 + 2 * h + 1, jc) = (uint16_t)(q[t][h] >> 16);
            }
          }
        }
      }
      lds_barrier();
#pragma unroll
      for (int a = 0; a < G::MT; ++a) {
        const int r = wy * G::WM + a * 32 + (lane & 31);
#pragma unroll
        for (int b = 0; b < G::NT; ++b)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int c = wx * G::WN + b * 32 + g * 8 + (lane >> 5) * 4;
            const u32x2_t w2 = *(const MUON_LDS u32x2_t*)at(r, c);
            float w[4] = {bf16_to_f32(w2[0] & 0xffffu), bf16_to_f32(w2[0] >> 16), bf16_to_f32(w2[1] & 0xffffu),
                          bf16_to_f32(w2[1] >> 16)};
            float u[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              u[q] = update_u(w[q], as * acc[a][b][4 * g + q], uc.lr, uc.wd, uc.s);
              w[q] = w[q] + u[q];
            }
            if (uc.upd) {
              const int64_t i = m0 + r, j = n0 + c;
              if (!ftrans) {
                *(GLOBAL_AS nt::f32x4_t*)(uc.upd + i * ldw + j) = nt::f32x4_t{u[0], u[1], u[2], u[3]};
              } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) uc.upd[(j + q) * ldw + i] = u[q];
              }
            }
            *(MUON_LDS u32x2_t*)at(r, c) = u32x2_t{pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3])};
          }
      }
      lds_barrier();
      if (!ftrans) {
#pragma unroll 4
        for (int r = tid / TPR; r < BM; r += RPP)
          st_out16(W, (int64_t)(m0 + r) * ldw + n0 + cc, *(const MUON_LDS u32x4_t*)at(r, cc), stream);
      } else {
#pragma unroll 2
        for (int ci = 0; ci < CI; ++ci) {
          const int jc = jc0 + ci * (NT / GR);
          uint32_t w[4];
#pragma unroll
          for (int h = 0; h < 4; ++h)
            w[h] = (uint32_t)*at(r0 + 2 * h, jc) | ((uint32_t)*at(r0 + 2 * h + 1, jc) << 16);
          st_out16(W, (int64_t)(n0 + jc) * ldw + m0 + r0, u32x4_t{w[0], w[1], w[2], w[3]}, stream);
        }
      }
      return;
    }
  }
  lds_barrier();   // every wave is done with the main loop's LDS
  // With the whole tile in one slab (SW), slab element (r, col) sits at
  // r * PITCH + (col ^ 4 ((r >> 3) & 7)).  The XOR keeps 4-aligned column
  // quads whole (the 16-byte accesses of the accumulator writes and the row
  // pass keep their shape) and puts the eight 8-row groups of a column on
  // distinct bank quads, so the column pass can hand consecutive lanes
  // consecutive 8-row groups of one column: its 16-byte stores then form
  // 256-byte runs of the transposed rows, and its LDS reads stay
  // conflict-free.  (A tile staged in two slabs keeps half its accumulators
  // live through the first; there the extra addressing spilled registers and
  // cost more than the coalescing gained, so it keeps the plain layout.)
  constexpr bool SW = SH == BM;
  auto slab = [&](int r, int col) {
    if constexpr (SW) return C + r * PITCH + (col ^ (4 * ((r >> 3) & 7)));
    else return C + r * PITCH + col;
  };
#pragma unroll 1
  for (int s0 = 0; s0 < BM; s0 += SH) {
    // lane l holds row l % 32 of each MFMA tile, 4 consecutive columns per
    // register group: one 16-byte LDS write each (rows 16 bytes apart in bank
    // terms, so any 16 lanes cover all banks)
#pragma unroll
    for (int a = 0; a < G::MT; ++a) {
      const int rbase = wy * G::WM + a * 32;   // 32-row MFMA tile, uniform per wave
      if (rbase < s0 || rbase >= s0 + SH) continue;
      const int r = rbase - s0 + (lane & 31);
#pragma unroll
      for (int b = 0; b < G::NT; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = wx * G::WN + b * 32 + g * 8 + (lane >> 5) * 4;
          *(MUON_LDS nt::f32x4_t*)slab(r, c) =
              nt::f32x4_t{acc[a][b][4 * g], acc[a][b][4 * g + 1], acc[a][b][4 * g + 2], acc[a][b][4 * g + 3]};
        }
    }
    lds_barrier();
    // row pass: this thread's RPT consecutive rows of the slab, 8 columns
    // each (consecutive rows share the slab swizzle); Cin for all of them (or,
    // for an update applied here, the bf16 W rows) is requested before any is
    // used
    constexpr int RPT = SH / RPP;
    static_assert(SH % RPP == 0, "rows per thread");
    // rows of this thread: RPT consecutive ones (one swizzle) or, in the plain
    // layout, every RPP-th
    const int c = (tid % TPR) * 8, r_first = SW ? (tid / TPR) * RPT : tid / TPR;
    constexpr int RS = SW ? 1 : RPP;   // row step
    const int j = n0 + c;
    u32x4_t craw[RPT];
    if (Cin) {
#pragma unroll
      for (int t = 0; t < RPT; ++t)
        craw[t] = *(GLOBAL_AS const u32x4_t*)(static_cast<const uint16_t*>(Cin) +
                                              (int64_t)(m0 + s0 + r_first + t * RS) * ldo + j);
    } else if (wrow) {
#pragma unroll
      for (int t = 0; t < RPT; ++t) {
        const int i = m0 + s0 + r_first + t * RS;
        if (i < Mr && j + 8 <= Nr)
          craw[t] = *(GLOBAL_AS const u32x4_t*)(static_cast<const uint16_t*>(uc.w) +
                                                (int64_t)i * uc.cols + j);
      }
    }
#pragma unroll
    for (int t = 0; t < RPT; ++t) {
      const int r = r_first + t * RS;
      const int i = m0 + s0 + r;
      float v[8];
      {
        const nt::f32x4_t a4 = *(const MUON_LDS nt::f32x4_t*)slab(r, c);
        const nt::f32x4_t b4 = *(const MUON_LDS nt::f32x4_t*)slab(r, c + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = a4[e];
          v[4 + e] = b4[e];
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = as * v[e];
        if (Cin) x = fmaf(bs, bf16_to_f32((e & 1) ? (craw[t][e >> 1] >> 16) : (craw[t][e >> 1] & 0xffffu)), x);
        v[e] = x;
      }
      if (edge) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (i == j + e) v[e] += gamma;
          if (i >= Mr || j + e >= Nr) v[e] = 0.f;
        }
      }
      if (!fuse) {
        st8<TO>(Out, (int64_t)i * ldo + j, v);
      } else if (!ftrans && i < Mr) {
        const int nv = Nr - j;
        if (wrow && nv >= 8) apply_update8_bf16(uc, (int64_t)i * uc.cols + j, craw[t], v);
        else apply_update8(uc, i, j, nv < 8 ? nv : 8, v);
      }
      if (colpass) {
        *(MUON_LDS nt::f32x4_t*)slab(r, c) = nt::f32x4_t{v[0], v[1], v[2], v[3]};
        *(MUON_LDS nt::f32x4_t*)slab(r, c + 4) = nt::f32x4_t{v[4], v[5], v[6], v[7]};
      }
    }
    if (colpass) {
      lds_barrier();
      // every thread takes CI (column, 8-row group) items.  Swizzled layout:
      // item wi = tid + ci NT is column 4 (wi / (4 GR)) + wi % 4 and row group
      // (wi / 4) % GR, so the 4 lanes of a quad take 4 columns and the next
      // quads the next row groups (with NT a multiple of 4 GR a thread keeps
      // its row group and steps its column by NT / GR per item).  Plain
      // layout: column wi % BN, row group wi / BN.
      constexpr int GR = SH / 8;
      constexpr int CI = BN * GR / NT;
      static_assert(BN * GR % NT == 0 && CI % 2 == 0 && (SW ? NT % (4 * GR) == 0 : NT % BN == 0),
                    "column items per thread");
      const int jc0 = SW ? 4 * (tid / (4 * GR)) + tid % 4 : tid % BN;
      const int rg0 = SW ? ((tid / 4) % GR) * 8 : (tid / BN) * 8;
      auto col_of = [&](int ci) { return SW ? jc0 + ci * (NT / GR) : jc0; };
      auto grp_of = [&](int ci) { return SW ? rg0 : rg0 + ci * (NT / BN) * 8; };
      auto item = [&](int ci, bool have_w, u32x4_t wq) {
        const int jc = col_of(ci), r0 = grp_of(ci);
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = *slab(r0 + e, jc);
        const int j = n0 + jc, i0 = m0 + s0 + r0;
        if (OutT) st8<uint16_t>(OutT, (int64_t)j * m_pad + i0, v);
        if (mirror) st8<TO>(Out, (int64_t)j * ldo + i0, v);
        if (ftrans && j < Nr) {
          const int nv = Mr - i0;
          if (have_w && nv >= 8) apply_update8_bf16(uc, (int64_t)j * uc.cols + i0, wq, v);
          else apply_update8(uc, j, i0, nv < 8 ? nv : 8, v);
        }
      };
      if (wcol) {
        // the update of a tall matrix: items in pairs, both bf16 W runs
        // requested before either is used
        auto wrun = [&](int ci) {
          const int j = n0 + col_of(ci), i0 = m0 + s0 + grp_of(ci);
          u32x4_t q = {0, 0, 0, 0};
          if (j < Nr && i0 + 8 <= Mr)
            q = *(GLOBAL_AS const u32x4_t*)(static_cast<const uint16_t*>(uc.w) +
                                            (int64_t)j * uc.cols + i0);
          return q;
        };
#pragma unroll 1
        for (int ci = 0; ci < CI; ci += 2) {
          const u32x4_t q0 = wrun(ci), q1 = wrun(ci + 1);
          item(ci, true, q0);
          item(ci + 1, true, q1);
        }
      } else {
#pragma unroll 1
        for (int ci = 0; ci < CI; ++ci) item(ci, false, u32x4_t{0, 0, 0, 0});
      }
    }
    lds_barrier();   // the slab buffer is reused
  }
}

template <int BM, int BN, int WGM, int WGN, typename TO, bool QT>
__global__ __launch_bounds__(64 * WGM * WGN) void k_nt(const GemmParams p) {
  extern __shared__ __attribute__((aligned(1024))) char nt_smem[];
  using PP = NtPipe<BM, BN, WGM, WGN>;
  using G = nt::Geom<BM, BN, PP::BK, PP::S, WGM, WGN>;
  const WorkItem it = p.items[blockIdx.x];
  const NsMat* nmp = p.mats + it.slot;
  const int m_pad = nmp->m_pad, n_pad = nmp->n_pad;
  int K, ldp, ldq, ldo, Mr, Nr;
  uint32_t p_rows, q_rows;
  if (p.shape == kShapeGram) {
    K = n_pad; ldp = ldq = n_pad; ldo = m_pad; Mr = Nr = nmp->m; p_rows = q_rows = m_pad;
  } else if (p.shape == kShapeSquare) {
    K = m_pad; ldp = ldq = m_pad; ldo = m_pad; Mr = Nr = nmp->m; p_rows = q_rows = m_pad;
  } else if (!QT) {
    K = m_pad; ldp = ldq = m_pad; ldo = n_pad; Mr = nmp->m; Nr = nmp->n; p_rows = m_pad; q_rows = n_pad;
  } else {
    // Q = X itself, m_pad rows (k) of n_pad
    K = m_pad; ldp = m_pad; ldq = n_pad; ldo = n_pad; Mr = nmp->m; Nr = nmp->n; p_rows = m_pad;
    q_rows = m_pad;
  }
  const void* Pg = nmp->buf[p.p_id];
  const void* Qg = nmp->buf[p.q_id];
  const __amdgpu_buffer_rsrc_t Pr = nt::make_rsrc(Pg, p_rows * (uint32_t)ldp * 2u);
  const __amdgpu_buffer_rsrc_t Qr = nt::make_rsrc(Qg, q_rows * (uint32_t)ldq * 2u);
  const int m0 = it.tm * BM, n0 = it.tn * BN;
  nt::f32x16_t acc[G::MT][G::NT];
  nt::mainloop<BM, BN, PP::BK, PP::S, WGM, WGN, QT>(acc, (MUON_LDS char*)nt_smem, Pr, Qr, (uint32_t)ldp,
                                            (uint32_t)ldq, (uint32_t)m0, (uint32_t)n0, K);

  nt_epilogue<BM, BN, WGM, WGN, TO>(acc, (MUON_LDS float*)nt_smem, p, nmp, m0, n0, ldo, Mr, Nr);
}

template <int BM, int BN, int WGM, int WGN, typename TO, bool QT>
hipError_t launch_nt_t(const GemmParams& p, hipStream_t s) {
  using PP = NtPipe<BM, BN, WGM, WGN>;
  using G = nt::Geom<BM, BN, PP::BK, PP::S, WGM, WGN, QT>;
  static_assert(G::LDS == nt::Geom<BM, BN, PP::BK, PP::S, WGM, WGN>::LDS, "k-major Q tile, same bytes");
  constexpr int smem = nt_lds<BM, BN, WGM, WGN>();
  static bool attr_done = false;
  auto kern = &k_nt<BM, BN, WGM, WGN, TO, QT>;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  if (p.n_items <= 0) return hipSuccess;
  launch_kernel(kern, dim3(p.n_items), dim3(G::THREADS), smem, s, p);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN>
hipError_t launch_nt_cfg(int out_dt, const GemmParams& p, hipStream_t s) {
  if (p.fuse && out_dt != kF32) return hipErrorInvalidValue;   // the update is applied from fp32 tiles
  if (p.qt) {
    if (p.shape != kShapeApplyT) return hipErrorInvalidValue;
    if constexpr (BN >= 128) {   // k-major Q tiles need rows of >= 256 bytes
      if (out_dt == kBF16) return launch_nt_t<BM, BN, WGM, WGN, uint16_t, true>(p, s);
      if (out_dt == kF32) return launch_nt_t<BM, BN, WGM, WGN, float, true>(p, s);
    }
    return hipErrorInvalidValue;
  }
  if (out_dt == kBF16) return launch_nt_t<BM, BN, WGM, WGN, uint16_t, false>(p, s);
  if (out_dt == kF32) return launch_nt_t<BM, BN, WGM, WGN, float, false>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_ew_momentum(const EwMat* mats, const EwDyn* dyn, const int64_t* tile_prefix,
                              int nmats, int64_t tile_begin, int64_t tile_end, float* partials,
                              float beta, int nesterov, int load_only, int grid_cap, hipStream_t s) {
  const int64_t n = tile_end - tile_begin;
  if (n <= 0) return hipSuccess;
  const int64_t grid = n < grid_cap ? n : grid_cap;
  launch_kernel(k_ew_momentum, dim3((unsigned)grid), dim3(256), 0, s, mats, dyn, tile_prefix,
                     nmats, tile_begin, tile_end, partials, beta, nesterov, load_only);
  return hipGetLastError();
}

hipError_t launch_adamw(const AdamTensor* tensors, const int64_t* chunk_prefix, int ntensors,
                        int64_t total_chunks, AdamScalars sc, int grid_cap, hipStream_t s) {
  if (total_chunks <= 0) return hipSuccess;
  const int64_t grid = total_chunks < grid_cap ? total_chunks : grid_cap;
  launch_kernel(k_adamw, dim3((unsigned)grid), dim3(256), 0, s, tensors, chunk_prefix, ntensors,
                     total_chunks, sc);
  return hipGetLastError();
}

hipError_t launch_norm(const EwMat* mats, int nmats, const float* partials, float* rscale,
                       uint32_t* flags, float eps, hipStream_t s) {
  if (nmats <= 0) return hipSuccess;
  launch_kernel(k_norm, dim3(nmats), dim3(256), 0, s, mats, partials, rscale, flags, eps);
  return hipGetLastError();
}

hipError_t launch_ew_apply(const EwMat* mats, const EwDyn* dyn, const int64_t* tile_prefix,
                           int nmats, int64_t total_tiles, const float* rscale, float lr,
                           float wd, int src_is_d, int skip_fused, int store_x, int grid_cap,
                           hipStream_t s) {
  if (total_tiles <= 0) return hipSuccess;
  const int64_t grid = total_tiles < grid_cap ? total_tiles : grid_cap;
  launch_kernel(k_ew_apply, dim3((unsigned)grid), dim3(256), 0, s, mats, dyn, tile_prefix,
                     nmats, total_tiles, rscale, lr, wd, src_is_d, skip_fused, store_x);
  return hipGetLastError();
}

hipError_t launch_gemm(int tile_cfg, int in_dtype, int out_dtype, const GemmParams& p,
                       hipStream_t s) {
  switch (tile_cfg) {
    case 0: return launch_gemm_cfg<128, 128>(in_dtype, out_dtype, p, s);
    // 64 x 64 tiles: four times the blocks for products too small to fill the CUs
    case 1: return launch_gemm_cfg<64, 64>(in_dtype, out_dtype, p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fill_random_bf16(void* p, uint64_t bytes, uint32_t seed, hipStream_t s) {
  if (bytes % 16 || (bytes && !p)) return hipErrorInvalidValue;
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const int64_t want = (n16 + 255) / 256;
  const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(k_fill_random_bf16, dim3(blocks), dim3(256), 0, s, static_cast<u32x4_t*>(p), n16, seed);
  return hipGetLastError();
}

hipError_t launch_gemm_nt(int nt_cfg, int out_dtype, const GemmParams& p, hipStream_t s) {
  if (p.shape != kShapeGram && p.shape != kShapeSquare && p.shape != kShapeApplyT)
    return hipErrorInvalidValue;
  switch (nt_cfg) {
    // 256 x 256 runs 8 waves (2 per SIMD, 128 x 64 each); the others 4 waves
    case kNt128: return launch_nt_cfg<128, 128, 2, 2>(out_dtype, p, s);
    case kNt256: return launch_nt_cfg<256, 256, 2, 4>(out_dtype, p, s);
    case kNt256x128: return launch_nt_cfg<256, 128, 2, 2>(out_dtype, p, s);
    case kNt128x256: return launch_nt_cfg<128, 256, 2, 2>(out_dtype, p, s);
    // 64 x 64 (4 waves of 32 x 32, 32 KiB of LDS): four times the blocks of
    // 128 x 128 for m x m products too small to fill the CUs
    case kNt64: return launch_nt_cfg<64, 64, 2, 2>(out_dtype, p, s);
    default: return hipErrorInvalidValue;
  }
}

void set_launch_events(hipEvent_t start, hipEvent_t stop) {
  t_ev_start = start;
  t_ev_stop = stop;
  t_launched = false;
}

bool launched() { return t_launched; }

}  // namespace muon
