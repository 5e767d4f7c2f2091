// bf16 "NT" contraction core for gfx950: acc(i, j) += sum_k P[i][k] * Q[j][k]
// with P and Q row-major and k contiguous in both, fp32 accumulation on
// v_mfma_f32_32x32x16_bf16.
//
// Block: 256 threads = 4 waves in a 2 x 2 grid; wave tile (BM/2) x (BN/2)
// made of 32 x 32 MFMA tiles, accumulators in AGPRs (one wave per SIMD).
// k advances in 64-element (128-byte) tiles.  Each k-tile of P (BM rows) and
// Q (BN rows) is copied global -> LDS by buffer_load ... lds (16 bytes per
// lane, no VGPR staging), two stages in flight.  LDS rows are 128 bytes with
// no padding; 16-byte chunk c of row r is stored at slot c ^ ((r >> 1) & 7),
// so the 16-byte fragment reads of any 16 consecutive lanes (16 rows, one
// chunk) hit 16 distinct 16-byte bank groups.  A lane's MFMA fragment is the
// 16 bytes of chunk (2*kg + lane/32) of row (lane % 32) of a 32-row slab.
//
// With QT the second operand is stored the other way, Q[k][j] (k-major, j
// contiguous): acc(i, j) += sum_k P[i][k] * Q[k][j].  Its k-tile is copied as
// BK rows of BN elements and the MFMA B fragments are read with the gfx950
// LDS transpose read (ds_read_b64_tr_b16), so no transposed copy of Q has to
// exist in memory.
//
// The buffer descriptors carry the byte size of each operand, so an access
// outside it reads zeros instead of faulting; the callers still only issue
// in-bounds tiles (every extent is padded to the tile size).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {
namespace nt {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
#define MUON_LDS __attribute__((address_space(3)))

constexpr int kThreads = 256;

// Raw buffer descriptor word 3 for gfx9-class targets: 32-bit untyped data.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 encoding: vmcnt
// bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
constexpr int waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x70 | 0xF00; }
static_assert(waitcnt_vm(0) == 0xF70, "encoding");
constexpr int kWaitVmLgkm0 = 0x0070;   // vmcnt(0) lgkmcnt(0)
constexpr int kWaitLgkm0 = 0xC07F;     // lgkmcnt(0) only (vmcnt 63, expcnt 7 leave them be)
static_assert((waitcnt_vm(63) & ~0x0F00) == kWaitLgkm0, "encoding");

// BM x BN output tile, BK bf16 per k-tile (32 or 64), S LDS stages, a WGM x WGN
// grid of waves (each owns a (BM/WGM) x (BN/WGN) tile).
template <int BM, int BN, int BK, int S, int WGM = 2, int WGN = 2, bool QT = false>
struct Geom {
  static constexpr int NW = WGM * WGN;                 // waves per block
  static constexpr int THREADS = 64 * NW;
  static constexpr int ROWB = BK * 2;                  // bytes per LDS row
  static constexpr int CPR = ROWB / 16;                // 16-byte chunks per row
  static constexpr int R256 = 256 / ROWB;              // rows per 256 bytes
  static constexpr int KG = BK / 16;                   // MFMA k-groups per k-tile
  static constexpr int WM = BM / WGM, WN = BN / WGN;   // wave tile
  static constexpr int MT = WM / 32, NT = WN / 32;     // MFMA tiles per wave
  static constexpr int PB = BM * ROWB, QB = BN * ROWB;
  static constexpr int STAGE = PB + QB;                // bytes per stage
  static constexpr int LDS = S * STAGE;
  static constexpr int RPI = 1024 / ROWB;              // rows per wave copy instruction
  static constexpr int RPR = NW * RPI;                 // rows per round of all waves
  // Q tile: BN rows of BK (NT) or, with QT, BK rows of BN elements
  static constexpr int QROWB = QT ? BN * 2 : ROWB;     // bytes per Q tile row
  static constexpr int QCPR = QROWB / 16;
  static constexpr int QRPI = 1024 / QROWB;
  static constexpr int QRPR = NW * QRPI;
  static constexpr int QROWS = QT ? BK : BN;
  static constexpr bool QT_ = QT;
  static constexpr int NDS = MT + (QT ? 2 : 1) * NT;   // LDS fragment reads per k-group
  static constexpr int PR = BM / RPR, QR = QROWS / QRPR;   // copy rounds per operand
  static constexpr int NI = PR + QR;                   // copy instructions per wave per tile
  static_assert(BK == 32 || BK == 64, "k-tile");
  static_assert(WM % 32 == 0 && WN % 32 == 0 && BM % RPR == 0 && QROWS % QRPR == 0, "tile edges");
  static_assert(!QT || (QCPR >= 16 && QRPI >= 1), "k-major Q tiles need rows of >= 256 bytes");
  static_assert(S >= 2 && LDS <= 160 * 1024, "LDS budget");
  static_assert((S - 1) * NI <= 63, "vmcnt range");
};

// LDS slot of 16-byte chunk c of tile row r: c ^ swz(r).  Any 16 consecutive
// rows read at one chunk hit 16 distinct 16-byte bank groups.
template <int ROWB>
__device__ __forceinline__ int swz(int r) {
  return (r / (256 / ROWB)) % (ROWB / 16);
}

// LDS slot of 16-byte chunk c of row k of a k-major Q tile: c ^ swzt(k).  A
// transpose read by 16 lanes covers rows k..k+3 (k a multiple of 4) at two
// adjacent chunks; the pattern puts those 4 pairs on 4 distinct 32-byte bank
// groups of a 128-byte window, and the pairs of the next 16 lanes (the next
// two chunks, same rows) on the rest of the 256-byte window.
__device__ __forceinline__ int swzt(int k) { return 4 * (k & 3) + 2 * ((k >> 1) & 1); }

// Global -> LDS copies of one operand.  Wave w copies the contiguous run of
// tile rows [w * NR * RPI, (w+1) * NR * RPI): copy u writes LDS bytes
// [(w*NR + u) KiB, +1 KiB), i.e. RPI whole rows, lane l into row l / CPR,
// slot l % CPR, so it fetches chunk (l % CPR) ^ swz(row) of that row.  M0
// (the LDS base) changes every fourth copy; the 12-bit immediate supplies the
// 1 KiB steps in between.  The immediate also advances the global address, so
// the scalar offset takes it back out.
template <class G, int NR, bool T = false>
struct Copier {
  // geometry of the copied tile: the P / NT layout, or the k-major Q tile
  static constexpr int RPI = T ? G::QRPI : G::RPI;
  static constexpr int CPR = T ? G::QCPR : G::CPR;
  static constexpr int ROWB = T ? G::QROWB : G::ROWB;
  static_assert(T || NR % 2 == 0 || G::ROWB == 64, "the swizzle phase must follow the copy index");
  static_assert(!T || RPI == 2 || RPI == 4, "k-major rows per copy");
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t voff[2];   // per-lane offsets for even / odd copies (swizzle phase)
  uint32_t soff;      // bytes to the wave's first row (row-block origin added per call)
  uint32_t step;      // bytes per copy (RPI rows)

  __device__ __forceinline__ void init(__amdgpu_buffer_rsrc_t r, uint32_t ld_bytes, int lane, int w) {
    rsrc = r;
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int row = (w * NR + par) * RPI + lane / CPR;   // any copy of this parity
      int sw;
      if constexpr (T) sw = swzt(row);
      else sw = swz<ROWB>(row);
      const int chunk = (lane % CPR) ^ sw;
      voff[par] = (uint32_t)(lane / CPR) * ld_bytes + (uint32_t)chunk * 16u;
    }
    step = (uint32_t)RPI * ld_bytes;
    soff = (uint32_t)(w * NR) * step;
  }

  // Copy U of the run (the immediate must be a compile-time constant).
  template <int U>
  __device__ __forceinline__ void issue_from(MUON_LDS char* dst, uint32_t origin, int w) const {
    if constexpr (U < NR) {
      constexpr int kImm = (U & 3) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst + (w * NR + (U & ~3)) * 1024, 16,
                                               voff[U & 1], origin + soff + U * step - kImm, kImm, 0);
      issue_from<U + 1>(dst, origin, w);
    }
  }

  // Copies rows [0, NR*4*RPI) of the row block whose byte origin is `origin`
  // (row-block start + k offset) into `dst` (this operand's region of a stage).
  __device__ __forceinline__ void issue(MUON_LDS char* dst, uint32_t origin, int w) const {
    issue_from<0>(dst, origin, w);
  }
};

template <class G>
struct Frags {
  u32x4_t a[G::MT], b[G::NT];
};

// Fragments of k-group kg (16 k values) of the stage at `st`: lane l reads
// chunk (2 kg + l / 32) of row (l % 32) of every 32-row slab of its wave tile.
template <class G>
__device__ __forceinline__ void load_frags_qt(u32x4_t (&b)[G::NT], const MUON_LDS char* stq, int kg,
                                              int lane, int wx);

template <class G>
__device__ __forceinline__ void load_frags(Frags<G>& f, const MUON_LDS char* st, int kg, int lane,
                                           int wy, int wx) {
  const int lr = lane & 31, hi = lane >> 5;
  const int q = ((kg * 2 + hi) ^ swz<G::ROWB>(lr)) * 16;
  const MUON_LDS char* pa = st + (wy * G::WM + lr) * G::ROWB + q;
#pragma unroll
  for (int i = 0; i < G::MT; ++i) f.a[i] = *(const MUON_LDS u32x4_t*)(pa + i * 32 * G::ROWB);
  if constexpr (G::QT_) {
    load_frags_qt<G>(f.b, st + G::PB, kg, lane, wx);
  } else {
    const MUON_LDS char* qa = st + G::PB + (wx * G::WN + lr) * G::ROWB + q;
#pragma unroll
    for (int j = 0; j < G::NT; ++j) f.b[j] = *(const MUON_LDS u32x4_t*)(qa + j * 32 * G::ROWB);
  }
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// B fragments of k-group kg from a k-major Q tile (G::QT).  A 32x32x16 B
// fragment is lane l: Q[k0 + 8 (l / 32) + 0..7][j0 + l % 32].  The transpose
// read gives lane i of each 16-lane group element (i % 4) of the 8 bytes that
// lane 4e + i / 4 addresses, for e = 0..3; so lane s of group g addresses row
// k0 + 8 (g / 2) + s / 4 (then 4 rows further for the second read), columns
// j0 + 16 (g % 2) + 4 (s % 4) .. + 3, and receives its column's 4 + 4 k values.
template <class G>
__device__ __forceinline__ void load_frags_qt(u32x4_t (&b)[G::NT], const MUON_LDS char* stq, int kg,
                                              int lane, int wx) {
  const int g = lane >> 4, sl = lane & 15;
  const int k = kg * 16 + 8 * (g >> 1) + (sl >> 2);
  const int off = ((g & 1) * 16 + 4 * (sl & 3)) * 2;       // byte offset of the lane's 4 columns
  const int sw = swzt(k);                                   // = swzt(k + 4)
#pragma unroll
  for (int j = 0; j < G::NT; ++j) {
    const int byte = (wx * G::WN + j * 32) * 2 + off;
    const int a = (((byte >> 4) ^ sw) << 4) + (byte & 15);
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (MUON_LDS s16x4_t*)(stq + k * G::QROWB + a));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (MUON_LDS s16x4_t*)(stq + (k + 4) * G::QROWB + a));
    const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
    b[j] = u32x4_t{l2[0], l2[1], h2[0], h2[1]};
  }
}

// The fragments go into the MFMA as (Q, P), so it accumulates the transposed
// 32 x 32 tile and acc[i][j] comes out row-major friendly: lane l holds row
// l % 32 of tile (i, j), columns 8 g + 4 (l / 32) + 0..3 in registers 4 g + 0..3.
template <class G>
__device__ __forceinline__ void mfma_group(f32x16_t (&acc)[G::MT][G::NT], const Frags<G>& f) {
#pragma unroll
  for (int i = 0; i < G::MT; ++i)
#pragma unroll
    for (int j = 0; j < G::NT; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, f.b[j]),
                                                         __builtin_bit_cast(bf16x8_t, f.a[i]),
                                                         acc[i][j], 0, 0, 0);
}

// Scheduling hints: keep `n` instructions of class `mask` in this slot of the
// schedule (classes: 0x008 MFMA, 0x020 VMEM read, 0x100 DS read).
#define MUON_SCHED(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)

// MFMAs of one k-group interleaved with `nvm` copy instructions and `nds`
// LDS fragment reads issued by the surrounding code (one of each per MFMA
// until they run out).
template <class G, int NVM, int NDS>
__device__ __forceinline__ void interleave_hint() {
#pragma unroll
  for (int i = 0; i < G::MT * G::NT; ++i) {
    MUON_SCHED(0x008, 1);
    if (i < NVM) MUON_SCHED(0x020, 1);
    if (i < NDS) MUON_SCHED(0x100, 1);
  }
}

// Workgroup barrier without the memory-model fences of __syncthreads (those
// would force vmcnt(0) and drain every copy in flight).  Callers wait on the
// counters they need first; the "memory" clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Full k loop: acc = P[m0 : m0+BM, 0:K] * Q[n0 : n0+BN, 0:K]^T.
// ldp / ldq: leading dimensions in elements; K a multiple of BK.
// lds: Geom::LDS bytes of dynamic shared memory.
//
// Tile kt sits in stage kt % S.  Its k-groups run on fragments loaded one
// group ahead.  After the reads of its last group have been issued, the wave
// waits for those reads and for its copies of tile kt+1, then one barrier:
// every wave is done with stage kt % S and tile kt+1 has landed everywhere.
// The copies of tile kt+S then go into stage kt % S, interleaved with the
// last group's MFMAs and the reads of group 0 of tile kt+1.  Copies past the
// last tile re-read the last tile (in bounds, never consumed) so the steady
// state has no branches and always S-1 tiles in flight.
template <int BM, int BN, int BK, int S, int WGM = 2, int WGN = 2, bool QT = false>
__device__ __forceinline__ void mainloop(
    f32x16_t (&acc)[BM / 32 / WGM][BN / 32 / WGN],
    MUON_LDS char* lds, __amdgpu_buffer_rsrc_t P, __amdgpu_buffer_rsrc_t Q, uint32_t ldp,
    uint32_t ldq, uint32_t m0, uint32_t n0, int K) {
  using G = Geom<BM, BN, BK, S, WGM, WGN, QT>;
  static_assert(G::KG % 2 == 0, "the last group's fragments are in f1");
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wy = w / WGN, wx = w % WGN;
#pragma unroll
  for (int i = 0; i < G::MT; ++i)
#pragma unroll
    for (int j = 0; j < G::NT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  Copier<G, G::PR> cp;
  Copier<G, G::QR, QT> cq;
  cp.init(P, ldp * 2u, lane, w);
  cq.init(Q, ldq * 2u, lane, w);
  // k-tile byte steps: along a P row; along a Q row (NT) or down BK Q rows (QT)
  const uint32_t sp = m0 * ldp * 2u, sq = QT ? n0 * 2u : n0 * ldq * 2u;
  const uint32_t kq = QT ? (uint32_t)BK * ldq * 2u : (uint32_t)G::ROWB;
  const int nk = K / BK;
  const uint32_t klast = (uint32_t)(nk - 1) * G::ROWB, klast_q = (uint32_t)(nk - 1) * kq;
#pragma unroll
  for (int t = 0; t < S; ++t) {
    const uint32_t kb = t < nk ? (uint32_t)t * G::ROWB : klast;
    const uint32_t kbq = t < nk ? (uint32_t)t * kq : klast_q;
    cp.issue(lds + t * G::STAGE, sp + kb, w);
    cq.issue(lds + t * G::STAGE + G::PB, sq + kbq, w);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm((S - 1) * G::NI));   // tile 0 landed
  block_barrier();
  Frags<G> f0, f1;
  load_frags<G>(f0, lds, 0, lane, wy, wx);
  int stage = 0;
  uint32_t knext = (uint32_t)S * G::ROWB, knext_q = (uint32_t)S * kq;
  for (int kt = 0; kt < nk; ++kt) {
    const MUON_LDS char* st = lds + stage * G::STAGE;
#pragma unroll
    for (int g = 0; g + 1 < G::KG; ++g) {
      if (g & 1) { load_frags<G>(f0, st, g + 1, lane, wy, wx); mfma_group<G>(acc, f1); }
      else       { load_frags<G>(f1, st, g + 1, lane, wy, wx); mfma_group<G>(acc, f0); }
      interleave_hint<G, 0, G::NDS>();
    }
    // tile kt+1 landed (S-2 later tiles may stay in flight), own reads done
    constexpr int kWait = waitcnt_vm((S - 2) * G::NI) & ~0xF00;
    __builtin_amdgcn_s_waitcnt(kWait);
    block_barrier();
    const uint32_t kb = knext <= klast ? knext : klast;
    const uint32_t kbq = knext_q <= klast_q ? knext_q : klast_q;
    knext += G::ROWB;
    knext_q += kq;
    MUON_LDS char* dst = lds + stage * G::STAGE;
    cp.issue(dst, sp + kb, w);
    cq.issue(dst + G::PB, sq + kbq, w);
    stage = stage + 1 == S ? 0 : stage + 1;
    load_frags<G>(f0, lds + stage * G::STAGE, 0, lane, wy, wx);
    mfma_group<G>(acc, f1);
    interleave_hint<G, G::NI, G::NDS>();
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);   // no copy outlives the loop
}

}  // namespace nt
}  // namespace muon
