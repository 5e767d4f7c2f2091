// Ceiling probes (declared in probe.hpp): the rates this part sustains for
// dense bf16 MFMA work, for the NT contraction core and for streaming HBM
// copies when nothing else limits them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mfma_nt.hpp"
#include "probe.hpp"

namespace muon {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

namespace {

// One bf16 operand value from a hash of (thread, index): random sign and
// 7-bit mantissa, magnitude in [2^-7, 2^-5), so every multiplier input bit
// toggles between consecutive MFMAs as it does on real data.
__device__ __forceinline__ __bf16 probe_rand_bf16(uint32_t key) {
  key ^= key >> 16;
  key *= 0x7feb352du;
  key ^= key >> 15;
  key *= 0x846ca68bu;
  key ^= key >> 16;
  const uint16_t bits = (uint16_t)((key & 0x8000u) | ((120u + ((key >> 8) & 1u)) << 7) | (key & 0x7fu));
  return __builtin_bit_cast(__bf16, bits);
}

// RAND = false: every MFMA of a wave takes the same register operands.
// RAND = true: eight operand pairs of random values, a different pair for
// each MFMA of a round of eight (the register file still feeds them, no
// memory traffic), which is the switching activity of random data.
template <bool RAND>
__global__ __launch_bounds__(256) void k_probe_mfma(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  constexpr int NOP = RAND ? 8 : 1;
  bf16x8_t a[NOP], b[NOP];
  const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x;
#pragma unroll
  for (int k = 0; k < NOP; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (RAND) {
        a[k][e] = probe_rand_bf16(tid * 131u + (uint32_t)(k * 8 + e) * 2u);
        b[k][e] = probe_rand_bf16(tid * 131u + (uint32_t)(k * 8 + e) * 2u + 1u);
      } else {
        a[k][e] = (__bf16)(0.001f * (float)(lane + e));
        b[k][e] = (__bf16)(0.002f * (float)(lane - e));
      }
    }
  f32x16_t acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  int i = 0;
  if constexpr (RAND) {
    for (; i + 8 <= iters; i += 8) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int c = 0; c < kProbeChains; ++c)
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(j + c) % 8], b[(j + 3 * c + 1) % 8], acc[c], 0, 0, 0);
    }
  }
  for (; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], acc[c], 0, 0, 0);
  }
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += acc[c][r];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

using ProbeNtGeom = nt::Geom<kProbeNtTile, kProbeNtTile, 64, 2, 2, 4>;
static_assert(ProbeNtGeom::THREADS == kProbeNtThreads, "probe block");

__global__ __launch_bounds__(kProbeNtThreads) void k_probe_nt(const uint16_t* __restrict__ P,
                                                              const uint16_t* __restrict__ Q, int m,
                                                              int n, int k, float* __restrict__ out) {
  extern __shared__ __attribute__((aligned(1024))) char probe_smem[];
  using G = ProbeNtGeom;
  const int tn_count = n / kProbeNtTile;
  const int tm = blockIdx.x / tn_count, tn = blockIdx.x % tn_count;
  const __amdgpu_buffer_rsrc_t Pr = nt::make_rsrc(P, (uint32_t)((size_t)m * k * 2));
  const __amdgpu_buffer_rsrc_t Qr = nt::make_rsrc(Q, (uint32_t)((size_t)n * k * 2));
  nt::f32x16_t acc[G::MT][G::NT];
  nt::mainloop<kProbeNtTile, kProbeNtTile, 64, 2, 2, 4, false>(
      acc, (MUON_LDS char*)probe_smem, Pr, Qr, (uint32_t)k, (uint32_t)k, (uint32_t)(tm * kProbeNtTile),
      (uint32_t)(tn * kProbeNtTile), k);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < G::MT; ++i)
#pragma unroll
    for (int j = 0; j < G::NT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += acc[i][j][r];
  out[(int64_t)blockIdx.x * kProbeNtThreads + threadIdx.x] = sum;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t probe_pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// 16-byte store of the probe's output, nontemporal when NTS (a buffer store
// whose cache-policy immediate carries the nt bit; the descriptor spans 4 GiB
// from base, the outputs stay below 2 GiB).
template <bool NTS>
__device__ __forceinline__ void probe_out16(uint16_t* base, int64_t off, u32x4_t v) {
  if constexpr (NTS) {
    const __amdgpu_buffer_rsrc_t r = nt::make_rsrc(base, 0xFFFFFFFFu);
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (uint32_t)(off * 2), 0, 2);
  } else {
    *reinterpret_cast<u32x4_t*>(base + off) = v;
  }
}

constexpr int kProbeOutPitch = kProbeNtTile + 8;   // staged bf16 row pitch (elements)
constexpr int kProbeOutLds = kProbeNtTile * kProbeOutPitch * 2 > ProbeNtGeom::LDS
                                 ? kProbeNtTile * kProbeOutPitch * 2
                                 : ProbeNtGeom::LDS;

// The core plus an epilogue of the library's shape: every lane rounds its
// accumulators to bf16 and writes them into one staged tile (element (r, col)
// at r pitch + (col ^ 8 ((r >> 3) & 7))); a row pass stores 16-byte row runs
// into C; with COL a column pass gathers 8-row runs of a column (4 lanes of a
// quad on 4 columns, consecutive quads on consecutive 8-row groups) and
// stores them into CT.
template <bool COL, bool NTS>
__global__ __launch_bounds__(kProbeNtThreads) void k_probe_nt_out(const uint16_t* __restrict__ P,
                                                                  const uint16_t* __restrict__ Q, int m,
                                                                  int n, int k, uint16_t* __restrict__ C,
                                                                  uint16_t* __restrict__ CT) {
  extern __shared__ __attribute__((aligned(1024))) char probe_smem[];
  using G = ProbeNtGeom;
  constexpr int BM = kProbeNtTile, BN = kProbeNtTile, NT = kProbeNtThreads, PB = kProbeOutPitch;
  const int tn_count = n / BN;
  const int m0 = (blockIdx.x / tn_count) * BM, n0 = (blockIdx.x % tn_count) * BN;
  const __amdgpu_buffer_rsrc_t Pr = nt::make_rsrc(P, (uint32_t)((size_t)m * k * 2));
  const __amdgpu_buffer_rsrc_t Qr = nt::make_rsrc(Q, (uint32_t)((size_t)n * k * 2));
  nt::f32x16_t acc[G::MT][G::NT];
  nt::mainloop<BM, BN, 64, 2, 2, 4, false>(acc, (MUON_LDS char*)probe_smem, Pr, Qr, (uint32_t)k, (uint32_t)k,
                                           (uint32_t)m0, (uint32_t)n0, k);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wy = w / 4, wx = w % 4;
  MUON_LDS uint16_t* Cb = (MUON_LDS uint16_t*)probe_smem;
  auto at = [&](int r, int col) { return Cb + r * PB + (col ^ (8 * ((r >> 3) & 7))); };
  __builtin_amdgcn_s_waitcnt(nt::kWaitLgkm0);   // the main loop's LDS is free
  nt::block_barrier();
#pragma unroll
  for (int a = 0; a < G::MT; ++a) {
    const int r = wy * G::WM + a * 32 + (lane & 31);
#pragma unroll
    for (int b = 0; b < G::NT; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = wx * G::WN + b * 32 + g * 8 + (lane >> 5) * 4;
        *(MUON_LDS u32x2_t*)at(r, c) = u32x2_t{probe_pack_bf16x2(acc[a][b][4 * g], acc[a][b][4 * g + 1]),
                                               probe_pack_bf16x2(acc[a][b][4 * g + 2], acc[a][b][4 * g + 3])};
      }
  }
  __builtin_amdgcn_s_waitcnt(nt::kWaitLgkm0);
  nt::block_barrier();
  constexpr int TPR = BN / 8, RPP = NT / TPR;
  const int cc = (tid % TPR) * 8;
#pragma unroll 4
  for (int r = tid / TPR; r < BM; r += RPP)
    probe_out16<NTS>(C, (int64_t)(m0 + r) * n + n0 + cc, *(const MUON_LDS u32x4_t*)at(r, cc));
  if constexpr (COL) {
    constexpr int GR = BM / 8;
    const int jc0 = 4 * (tid / (4 * GR)) + tid % 4, r0 = ((tid / 4) % GR) * 8;
#pragma unroll 2
    for (int ci = 0; ci < BN * GR / NT; ++ci) {
      const int jc = jc0 + ci * (NT / GR);
      uint32_t q[4];
#pragma unroll
      for (int h = 0; h < 4; ++h)
        q[h] = (uint32_t)*at(r0 + 2 * h, jc) | ((uint32_t)*at(r0 + 2 * h + 1, jc) << 16);
      probe_out16<NTS>(CT, (int64_t)(n0 + jc) * m + m0 + r0, u32x4_t{q[0], q[1], q[2], q[3]});
    }
  }
}

template <bool NTMP>
__device__ __forceinline__ u32x4_t probe_ld(const u32x4_t* p) {
  if constexpr (NTMP) return __builtin_nontemporal_load(p);
  return *p;
}

template <bool NTMP>
__device__ __forceinline__ void probe_st(u32x4_t* p, u32x4_t v) {
  if constexpr (NTMP) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// NTMP: nontemporal loads and stores (streaming cache policy)
template <bool NTMP>
__global__ __launch_bounds__(256) void k_probe_copy(const u32x4_t* __restrict__ src,
                                                    u32x4_t* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4_t v0 = probe_ld<NTMP>(src + i), v1 = probe_ld<NTMP>(src + i + stride);
    const u32x4_t v2 = probe_ld<NTMP>(src + i + 2 * stride), v3 = probe_ld<NTMP>(src + i + 3 * stride);
    probe_st<NTMP>(dst + i, v0);
    probe_st<NTMP>(dst + i + stride, v1);
    probe_st<NTMP>(dst + i + 2 * stride, v2);
    probe_st<NTMP>(dst + i + 3 * stride, v3);
  }
  for (; i < n16; i += stride) probe_st<NTMP>(dst + i, probe_ld<NTMP>(src + i));
}

// One contiguous 16 KiB run per block (256 threads x 4 words), as many blocks
// as runs.
template <bool NTMP>
__global__ __launch_bounds__(256) void k_probe_copy_runs(const u32x4_t* __restrict__ src,
                                                         u32x4_t* __restrict__ dst, int64_t n16) {
  const int64_t base = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  u32x4_t v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (base + u * 256 < n16) v[u] = probe_ld<NTMP>(src + base + u * 256);
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (base + u * 256 < n16) probe_st<NTMP>(dst + base + u * 256, v[u]);
}

}  // namespace

hipError_t launch_probe_mfma(int blocks, int iters, bool random_operands, float* out, hipStream_t s) {
  if (random_operands)
    hipLaunchKernelGGL(k_probe_mfma<true>, dim3((unsigned)blocks), dim3(256), 0, s, iters, out);
  else
    hipLaunchKernelGGL(k_probe_mfma<false>, dim3((unsigned)blocks), dim3(256), 0, s, iters, out);
  return hipGetLastError();
}

hipError_t launch_probe_nt(const void* P, const void* Q, int m, int n, int k, float* out, hipStream_t s) {
  if (m <= 0 || n <= 0 || k <= 0 || m % kProbeNtTile || n % kProbeNtTile || k % 64 ||
      (int64_t)m * k >= (1ll << 31) || (int64_t)n * k >= (1ll << 31))
    return hipErrorInvalidValue;
  static bool attr_done = false;
  if (!attr_done) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_probe_nt),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, ProbeNtGeom::LDS);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int tiles = (m / kProbeNtTile) * (n / kProbeNtTile);
  hipLaunchKernelGGL(k_probe_nt, dim3((unsigned)tiles), dim3(kProbeNtThreads), ProbeNtGeom::LDS, s,
                     static_cast<const uint16_t*>(P), static_cast<const uint16_t*>(Q), m, n, k, out);
  return hipGetLastError();
}

template <bool COL, bool NTS>
hipError_t launch_probe_nt_out_t(const void* P, const void* Q, void* C, void* CT, int m, int n, int k,
                                 hipStream_t s) {
  static bool attr_done = false;
  auto kern = &k_probe_nt_out<COL, NTS>;
  if (!attr_done) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kProbeOutLds);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int tiles = (m / kProbeNtTile) * (n / kProbeNtTile);
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(kProbeNtThreads), kProbeOutLds, s,
                     static_cast<const uint16_t*>(P), static_cast<const uint16_t*>(Q), m, n, k,
                     static_cast<uint16_t*>(C), static_cast<uint16_t*>(CT));
  return hipGetLastError();
}

hipError_t launch_probe_nt_out(const void* P, const void* Q, void* C, void* CT, int m, int n, int k, int mode,
                               hipStream_t s) {
  if (m <= 0 || n <= 0 || k <= 0 || m % kProbeNtTile || n % kProbeNtTile || k % 64 ||
      (int64_t)m * k >= (1ll << 31) || (int64_t)n * k >= (1ll << 31) || (int64_t)m * n >= (1ll << 30) ||
      !C || (mode >= 2 && !CT))
    return hipErrorInvalidValue;
  if (mode == 1) return launch_probe_nt_out_t<false, false>(P, Q, C, CT, m, n, k, s);
  if (mode == 2) return launch_probe_nt_out_t<true, false>(P, Q, C, CT, m, n, k, s);
  if (mode == 3) return launch_probe_nt_out_t<true, true>(P, Q, C, CT, m, n, k, s);
  return hipErrorInvalidValue;
}

hipError_t launch_probe_copy(const void* src, void* dst, int64_t n16, int blocks, bool nontemporal,
                             hipStream_t s) {
  if (blocks <= 0) {
    const int64_t runs = (n16 + 1023) / 1024;
    if (runs > 0x7fffffff) return hipErrorInvalidValue;
    if (nontemporal)
      hipLaunchKernelGGL(k_probe_copy_runs<true>, dim3((unsigned)runs), dim3(256), 0, s,
                         static_cast<const u32x4_t*>(src), static_cast<u32x4_t*>(dst), n16);
    else
      hipLaunchKernelGGL(k_probe_copy_runs<false>, dim3((unsigned)runs), dim3(256), 0, s,
                         static_cast<const u32x4_t*>(src), static_cast<u32x4_t*>(dst), n16);
    return hipGetLastError();
  }
  if (nontemporal)
    hipLaunchKernelGGL(k_probe_copy<true>, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const u32x4_t*>(src), static_cast<u32x4_t*>(dst), n16);
  else
    hipLaunchKernelGGL(k_probe_copy<false>, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const u32x4_t*>(src), static_cast<u32x4_t*>(dst), n16);
  return hipGetLastError();
}

}  // namespace muon
