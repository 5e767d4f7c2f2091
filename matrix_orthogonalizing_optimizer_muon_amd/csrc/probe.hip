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
