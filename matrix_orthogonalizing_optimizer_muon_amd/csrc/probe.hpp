// Ceiling probes of the gfx950 device (measurement only, never part of a
// step): a dense bf16 MFMA loop without memory traffic, the NT contraction
// core alone and an HBM copy.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

// k_probe_mfma: `blocks` blocks of 4 waves; every wave runs `iters` rounds of
// kProbeChains independent v_mfma_f32_32x32x16_bf16 accumulations with no
// memory traffic, then stores one float per thread into out (blocks * 256).
// random_operands: each MFMA takes another of eight random register operand
// pairs (real data's switching activity) instead of the same pair.
constexpr int kProbeChains = 4;
hipError_t launch_probe_mfma(int blocks, int iters, bool random_operands, float* out, hipStream_t s);
// k_probe_nt: the NT contraction core (mfma_nt.hpp, 256x256 tiles of 8
// waves, the configuration of the large NS products) without an epilogue:
// block t computes tile (t / (n / 256), t % (n / 256)) of P Q^T over k (P m x
// k, Q n x k, bf16 row-major) and stores the sum of its accumulators, one
// float per thread, into out ((m / 256) * (n / 256) * 512 floats).  m, n
// multiples of 256, k a multiple of 64, m k and n k below 2^31.
constexpr int kProbeNtTile = 256, kProbeNtThreads = 512;
hipError_t launch_probe_nt(const void* P, const void* Q, int m, int n, int k, float* out, hipStream_t s);
// k_probe_nt_out: the same core with an epilogue that writes the product:
// each 256x256 tile is rounded to bf16 (RNE), staged once in LDS and stored
// by a row pass into C (m x n row-major); mode 2 adds a column pass storing
// the transposed tile into CT (n x m row-major); mode 3 is mode 2 with
// nontemporal stores.  m n below 2^30.
hipError_t launch_probe_nt_out(const void* P, const void* Q, void* C, void* CT, int m, int n, int k, int mode,
                               hipStream_t s);
// k_probe_copy: dst[i] = src[i] for n16 16-byte words (grid-stride, `blocks`
// blocks of 256 threads, 4 words in flight per thread), plain or nontemporal
// loads and stores; blocks <= 0: one block per contiguous 1024-word run.
hipError_t launch_probe_copy(const void* src, void* dst, int64_t n16, int blocks, bool nontemporal,
                             hipStream_t s);

}  // namespace muon
