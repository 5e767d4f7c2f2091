// Ceiling probes of the gfx950 device (measurement only, never part of a
// step): a dense bf16 MFMA loop without memory traffic and an HBM copy.
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
// k_probe_copy: dst[i] = src[i] for n16 16-byte words (grid-stride, `blocks`
// blocks of 256 threads, 4 words in flight per thread), plain or nontemporal
// loads and stores; blocks <= 0: one block per contiguous 1024-word run.
hipError_t launch_probe_copy(const void* src, void* dst, int64_t n16, int blocks, bool nontemporal,
                             hipStream_t s);

}  // namespace muon
