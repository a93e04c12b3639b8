// flce_device.h -- gfx950 device building blocks: element types, MFMA
// wrappers and the LDS-staged "NT" GEMM tile (C = A . B^T with both operands
// K-contiguous) that the forward logit pass, the backward recompute pass and
// the two gradient contractions share.
//
// Tile geometry: a workgroup owns a 256 x 256 fp32 output tile, split over
// its 4 or 8 wave64s as blocks of the 32x32 MFMA (Gemm<W> below); operands
// stream through a four-stage LDS ring fed by direct global-to-LDS copies
// (see gemm_nt_tile below).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

enum Dt : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int D> struct Elem;
template <> struct Elem<DT_F32> { typedef float T; static constexpr int bytes = 4; };
template <> struct Elem<DT_F16> { typedef _Float16 T; static constexpr int bytes = 2; };
template <> struct Elem<DT_BF16> { typedef __bf16 T; static constexpr int bytes = 2; };

template <int D> __device__ __forceinline__ float to_f32(typename Elem<D>::T x) { return (float)x; }
template <int D> __device__ __forceinline__ typename Elem<D>::T from_f32(float x) {
  return (typename Elem<D>::T)x;  // round to nearest even (v_cvt_pk_bf16_f32 / v_cvt_f16_f32)
}

constexpr int TILE = 256;          // output tile edge (rows and columns)

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// One 16-byte fragment pair -> MFMA update of one 32x32 block.
//  16-bit types: lane l holds row (l&31), k = 8*(l>>5) .. +7 of the 16-deep slab.
//  fp32: the same 16 bytes are 4 consecutive k of the 8-deep slab; four
//  32x32x2 MFMAs contract (k, k+4) pairs so every k is used exactly once.
template <int D> __device__ __forceinline__ void mfma_frag(f32x16_t& acc, uint4 a, uint4 b);

template <> __device__ __forceinline__ void mfma_frag<DT_BF16>(f32x16_t& acc, uint4 a, uint4 b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}
template <> __device__ __forceinline__ void mfma_frag<DT_F16>(f32x16_t& acc, uint4 a, uint4 b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                               __builtin_bit_cast(f16x8_t, b), acc, 0, 0, 0);
}
template <> __device__ __forceinline__ void mfma_frag<DT_F32>(f32x16_t& acc, uint4 a, uint4 b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

// Output element (row, col) of accumulator register r of a 32x32 block, for lane l:
//   col = l & 31,  row = 8*(r>>2) + 4*(l>>5) + (r&3).
__device__ __forceinline__ int acc_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

// An operand panel: 256 rows starting at `base` (rows past `rows` re-read the
// last valid row; their results are never stored), `ld` bytes apart,
// `kbytes` bytes of K (a multiple of 16; a ragged last stage reads zeros).
struct Panel {
  const char* base;
  int64_t ld;
  int rows;
  int64_t kbytes;
};

// ---------------------------------------------------------------------------
// Multi-stage operand pipeline.  Global memory is copied straight into LDS
// (global_load_lds_dwordx4, 16 bytes per lane) three K-stages ahead of use,
// into a ring of NSTAGES buffers.  A stage is 64 bytes of K for all 256 rows
// of A and of B (32 KB).  Rows are stored 64 bytes apart with the four 16-byte
// chunks of a row XOR-swizzled by (row>>2)&3, so that the 16 lanes that read
// one chunk of 16 consecutive rows hit all 64 LDS banks once.  Each stage has
// two 32-byte slabs; the fragments of the next slab are read while the MFMAs
// of the current one run, and the single barrier per stage sits between the
// two slabs' MFMAs.

constexpr int ROWB = 64;                 // K bytes per row per stage
constexpr int OPB = TILE * ROWB;         // one operand, one stage: 16 KB
constexpr int STB = 2 * OPB;             // A + B: 32 KB
constexpr int NSTAGES = 4;               // 128 KB of LDS

__shared__ __attribute__((aligned(1024))) char g_stage0[STB];
__shared__ __attribute__((aligned(1024))) char g_stage1[STB];
__shared__ __attribute__((aligned(1024))) char g_stage2[STB];
__shared__ __attribute__((aligned(1024))) char g_stage3[STB];

// Separate arrays per stage (not one array with offsets) so that no access
// to one stage's buffer is mistaken for an access to another's.
template <int S> __device__ __forceinline__ char* stage_buf() {
  if constexpr (S == 0) return g_stage0;
  else if constexpr (S == 1) return g_stage1;
  else if constexpr (S == 2) return g_stage2;
  else return g_stage3;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One wave-wide copy of 16 bytes per lane from global memory into LDS: lane l
// writes LDS bytes [lds + 16*l, +16).  Issued through inline asm so that only
// the pipeline's explicit vmcnt waits order it (the compiler would otherwise
// wait for every outstanding copy before any LDS read of a stage buffer).
// `gbase` and `lds` are wave-uniform; `voff` is the lane's byte offset.
__device__ __forceinline__ void lds_copy16(const char* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(gbase), "s"(lds)
               : "memory");
}

// A wave-uniform pointer forced into scalar registers (a uniform value the
// compiler computed in vector registers, e.g. after an integer division,
// would otherwise be handed to the "s" operand of lds_copy16).
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// s_waitcnt vmcnt(N) only (gfx9 encoding: expcnt and lgkmcnt left at max).
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier that waits for this wave's LDS accesses (lgkmcnt(0)) but
// not for its in-flight global copies; the signal fences keep the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Keeps the instruction scheduler from moving anything across this point,
// so that the source order is the issue order.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Wave layout of a workgroup of W waves over the 256 x 256 tile: a GM x GN
// grid of wave tiles of WI x WJ 32x32 blocks.
//   W = 4: one wave per SIMD, 128 x 128 per wave (256 accumulator registers).
//   W = 8: two waves per SIMD, 128 x 64 per wave (128 accumulator registers);
//          while one wave of a SIMD waits (a copy being issued, a barrier),
//          the other keeps the MFMA unit busy.
template <int W> struct Geo;
template <> struct Geo<4> { static constexpr int WI = 4, WJ = 4; };
template <> struct Geo<8> { static constexpr int WI = 4, WJ = 2; };
template <int W> struct Gemm {
  static constexpr int WI = Geo<W>::WI, WJ = Geo<W>::WJ;
  static constexpr int GN = TILE / (32 * WJ);   // wave columns
  static constexpr int NCOP = 2 * TILE / 16 / W;  // 16-row copies per thread per stage
  static constexpr int NREAD = WI + WJ;         // fragment reads per slab
  __device__ static int wm(int wave) { return wave / GN; }
  __device__ static int wn(int wave) { return wave % GN; }
};

template <int W> struct Frags {
  uint4 a[Gemm<W>::WI], b[Gemm<W>::WJ];
};

// Per-thread global byte offsets of its copies.  A stage is 32 copies of 16
// rows x 64 bytes (1 KB): block b = 0..31 is operand b>>4, rows (b&15)*16 ..
// +16.  Copy i of wave w is block w + W*i (so copies 0 .. NCOP/2-1 are of
// operand A, the rest of B).  Lane L covers row (b&15)*16 + L/4 (clamped to
// the panel) and LDS chunk position L&3, which holds global chunk
// (L&3) ^ ((row>>2)&3) of that row.
template <int W> struct CopyPlan {
  uint32_t off[Gemm<W>::NCOP];
};

template <int W> __device__ __forceinline__ constexpr int copy_block(int i, int wave) { return wave + W * i; }

template <int W>
__device__ __forceinline__ void copy_plan(CopyPlan<W>& cp, const Panel& A, const Panel& B, int t) {
  const int wave = t >> 6, L = t & 63;
#pragma unroll
  for (int i = 0; i < Gemm<W>::NCOP; ++i) {
    const int blk = copy_block<W>(i, wave);
    const Panel& p = blk < 16 ? A : B;
    int row = (blk & 15) * 16 + (L >> 2);
    const int c = (L & 3) ^ ((row >> 2) & 3);
    row = row < p.rows ? row : p.rows - 1;
    cp.off[i] = (uint32_t)(row * p.ld) + (uint32_t)(c * 16);
  }
}

// Copy I of stage kc into buffer S.  `masked` (ragged last stage only): a
// chunk past K is read from the row's last valid 16 bytes instead (the offset
// stays non-negative, so the address stays inside the row) and zeroed after
// it lands.  The choice is a select, not a branch.
template <int W, int S, int I>
__device__ __forceinline__ void copy_one_any(const CopyPlan<W>& cp, const Panel& A, const Panel& B, int kc,
                                            bool masked, int t) {
  const int wave = t >> 6, L = t & 63;
  const int64_t k0 = (int64_t)kc * ROWB;
  constexpr bool OPA = I < Gemm<W>::NCOP / 2;
  const Panel& p = OPA ? A : B;
  const int blk = copy_block<W>(I, wave);
  const int c = ((((blk & 15) * 16 + (L >> 2)) >> 2) & 3) ^ (L & 3);
  const uint32_t off = (masked && k0 + c * 16 >= p.kbytes)
                           ? cp.off[I] - (uint32_t)(c * 16) + (uint32_t)(p.kbytes - 16 - k0)
                           : cp.off[I];
  const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(stage_buf<S>() + blk * 1024));
  lds_copy16(uniform_ptr(p.base + k0), off, dst);
}

template <int W, int S, int I = 0>
__device__ __forceinline__ void copy_any(const CopyPlan<W>& cp, const Panel& A, const Panel& B, int kt,
                                         int nk, bool ragged, int t) {
  if constexpr (I < Gemm<W>::NCOP) {
    copy_one_any<W, S, I>(cp, A, B, kt, ragged && kt == nk - 1, t);
    copy_any<W, S, I + 1>(cp, A, B, kt, nk, ragged, t);
  }
}

// Zeroes this thread's LDS chunks of ragged stage kt that lie past K.
template <int W, int S>
__device__ __forceinline__ void zero_tail(const Panel& A, int kt, int t) {
  const int wave = t >> 6, L = t & 63;
  const int64_t k0 = (int64_t)kt * ROWB;
  char* base = stage_buf<S>();
#pragma unroll
  for (int i = 0; i < Gemm<W>::NCOP; ++i) {
    const int blk = copy_block<W>(i, wave);
    const int c = ((((blk & 15) * 16 + (L >> 2)) >> 2) & 3) ^ (L & 3);
    if (k0 + c * 16 >= A.kbytes) *reinterpret_cast<uint4*>(base + blk * 1024 + L * 16) = make_uint4(0u, 0u, 0u, 0u);
  }
}

// Byte offsets, inside a stage buffer, of this lane's fragment chunk for
// slab 0 and slab 1, for its first A and first B row block.  The lane reads
// rows r0 + 32*i + (l&31): they differ by multiples of 32, so the swizzle
// term (row>>2)&3 = ((l&31)>>2)&3 is the same for all its blocks, which then
// sit 32*ROWB bytes apart (an immediate offset).
struct FragBase {
  uint32_t a[2], b[2];
};

template <int W>
__device__ __forceinline__ void frag_base(FragBase& fb, int wave, int lane) {
  const int r32 = lane & 31, half = lane >> 5, x = (r32 >> 2) & 3;
  const int ra = Gemm<W>::wm(wave) * 32 * Gemm<W>::WI, rb = Gemm<W>::wn(wave) * 32 * Gemm<W>::WJ;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const uint32_t coff = (uint32_t)(((2 * s + half) ^ x) << 4);
    fb.a[s] = (uint32_t)((ra + r32) * ROWB) + coff;
    fb.b[s] = (uint32_t)(OPB + (rb + r32) * ROWB) + coff;
  }
}

// Fragment P (0..WI-1: A row block P; WI..: B row block P-WI) of slab `slab`
// of buffer S: lane (l&31, l>>5) reads chunk 2*slab + (l>>5) of its row.
template <int W, int S, int P>
__device__ __forceinline__ void frag_read_one(Frags<W>& f, const FragBase& fb, int slab) {
  constexpr int WI = Gemm<W>::WI;
  const char* base = stage_buf<S>();
  if constexpr (P < WI)
    f.a[P] = *reinterpret_cast<const uint4*>(base + fb.a[slab] + P * 32 * ROWB);
  else
    f.b[P - WI] = *reinterpret_cast<const uint4*>(base + fb.b[slab] + (P - WI) * 32 * ROWB);
}

// The order in which a slab's fragments are read: A0, B0 .. B(WJ-1), A1 ..
// A(WI-1) -- the MFMAs run row block by row block (A0 with every B, then
// A1, ...), so each fragment is read in the order it is first needed.
template <int W> __device__ __forceinline__ constexpr int read_order(int k) {
  constexpr int WI = Gemm<W>::WI, WJ = Gemm<W>::WJ;
  return k == 0 ? 0 : (k <= WJ ? WI + k - 1 : k - WJ);
}

// What follows MFMA step s of a slab: read k (0..NREAD-1), copy c (100 + c)
// or nothing (-1).  W = 4: 16 MFMAs | a read after every even step, a copy
// after every fourth (1, 5, 9, 13).  W = 8: 8 MFMAs | reads after steps
// 0 1 3 4 6 7, copies after 2 and 5.
template <int W> __device__ __forceinline__ constexpr int slab_action(int s) {
  if constexpr (W == 4) {
    return (s & 1) == 0 ? s / 2 : ((s & 3) == 1 ? 100 + s / 4 : -1);
  } else {
    return s == 2 ? 100 : (s == 5 ? 101 : (s < 2 ? s : (s < 5 ? s - 1 : s - 2)));
  }
}

// Copy issuers for slab_phase.  PlainCopy: a stage that lies wholly inside K
// (no clamp, no mask); everything but the lane's fixed offset cp.off[I] is
// scalar (the stage's global base and the LDS destination in m0).
template <int W> struct PlainCopy {
  const CopyPlan<W>& cp;
  const char* base;   // operand base + this stage's K offset (wave-uniform)
  uint32_t wave_lds;  // wave * 1024 (wave-uniform)
  template <int S, int I> __device__ __forceinline__ void issue() const {
    lds_copy16(base, cp.off[I], lds_addr(stage_buf<S>() + W * I * 1024) + wave_lds);
  }
};

// EdgeCopy: a stage at the end of K -- clamped to the last stage and masked
// when that one is ragged (copy_one_any).
template <int W> struct EdgeCopy {
  const CopyPlan<W>& cp;
  const Panel& A;
  const Panel& B;
  int kc;
  bool masked;
  int t;
  template <int S, int I> __device__ __forceinline__ void issue() const {
    copy_one_any<W, S, I>(cp, A, B, kc, masked, t);
  }
};

// One slab's WI x WJ MFMAs on `fm`, with the NREAD fragment reads of the next
// slab (buffer RS, slab `rslab`, into `fr`) and NCOP/2 copies (C0.. into
// buffer CS) placed between them as slab_action says: a wave issues in order
// and would otherwise stall its MFMAs behind a burst of copies or reads.
template <int D, int W, int RS, int CS, int C0, int STEP = 0, class Copy>
__device__ __forceinline__ void slab_phase(f32x16_t (&acc)[Gemm<W>::WI][Gemm<W>::WJ], const Frags<W>& fm,
                                           Frags<W>& fr, const FragBase& fb, int rslab, const Copy& cp) {
  constexpr int WJ = Gemm<W>::WJ;
  if constexpr (STEP < Gemm<W>::WI * WJ) {
    constexpr int I = STEP / WJ, J = STEP % WJ;
    mfma_frag<D>(acc[I][J], fm.a[I], fm.b[J]);
    constexpr int act = slab_action<W>(STEP);
    if constexpr (act >= 100) cp.template issue<CS, C0 + act - 100>();
    else if constexpr (act >= 0) frag_read_one<W, RS, read_order<W>(act)>(fr, fb, rslab);
    sched_fence();
    slab_phase<D, W, RS, CS, C0, STEP + 1>(acc, fm, fr, fb, rslab, cp);
  }
}

// All NREAD fragments of a slab, in read_order (so that every path into a
// stage has the same reads pending).
template <int W, int S, int K = 0>
__device__ __forceinline__ void frag_read(Frags<W>& f, const FragBase& fb, int slab) {
  if constexpr (K < Gemm<W>::NREAD) {
    frag_read_one<W, S, read_order<W>(K)>(f, fb, slab);
    frag_read<W, S, K + 1>(f, fb, slab);
  }
}

// Stage kt from buffer S (f0 holds its slab 0).  Every stage copies stage
// kt+3 into buffer (S+3)%4 (that buffer was last read in stage kt-1, before
// that stage's barrier):
//   phase A: slab-0 MFMAs | slab-1 reads of buffer S | operand-A copies
//   wait for stage kt+1's copies, zero its ragged tail, barrier
//   phase B: slab-1 MFMAs | slab-0 reads of buffer S+1 | operand-B copies
// Copies issued after stage kt+1's when the wait runs: stage kt+2's NCOP and
// stage kt+3's first NCOP/2.
template <int W> constexpr int kStageWait = Gemm<W>::NCOP + Gemm<W>::NCOP / 2;

// kstage_plain: stage kt+3 lies wholly inside K.
template <int D, int W, int S>
__device__ __forceinline__ void kstage_plain(f32x16_t (&acc)[Gemm<W>::WI][Gemm<W>::WJ], Frags<W>& f0,
                                             Frags<W>& f1, const CopyPlan<W>& cp, const FragBase& fb,
                                             const Panel& A, const Panel& B, int kt, uint32_t wave_lds) {
  constexpr int SN = (S + 1) % NSTAGES, SC = (S + NSTAGES - 1) % NSTAGES, H = Gemm<W>::NCOP / 2;
  const int64_t k0 = (int64_t)(kt + NSTAGES - 1) * ROWB;
  const PlainCopy<W> ca{cp, uniform_ptr(A.base + k0), wave_lds};
  const PlainCopy<W> cb{cp, uniform_ptr(B.base + k0), wave_lds};
  sched_fence();
  slab_phase<D, W, S, SC, 0>(acc, f0, f1, fb, 1, ca);
  wait_vmcnt<kStageWait<W>>();
  lds_barrier();
  slab_phase<D, W, SN, SC, H>(acc, f1, f0, fb, 0, cb);
}

// kstage_edge: any stage; past the end of K the copy re-reads the last stage
// (never used), so the schedule still has no branches.
template <int D, int W, int S>
__device__ __forceinline__ void kstage_edge(f32x16_t (&acc)[Gemm<W>::WI][Gemm<W>::WJ], Frags<W>& f0,
                                            Frags<W>& f1, const CopyPlan<W>& cp, const FragBase& fb,
                                            const Panel& A, const Panel& B, int kt, int nk, bool ragged,
                                            int t) {
  constexpr int SN = (S + 1) % NSTAGES, SC = (S + NSTAGES - 1) % NSTAGES, H = Gemm<W>::NCOP / 2;
  const int kc = min(kt + NSTAGES - 1, nk - 1);
  const EdgeCopy<W> c{cp, A, B, kc, ragged && kc == nk - 1, t};
  sched_fence();
  slab_phase<D, W, S, SC, 0>(acc, f0, f1, fb, 1, c);
  wait_vmcnt<kStageWait<W>>();
  if (ragged && kt + 1 == nk - 1) zero_tail<W, SN>(A, kt + 1, t);
  lds_barrier();
  slab_phase<D, W, SN, SC, H>(acc, f1, f0, fb, 0, c);
}

// acc[i][j] (this wave's WI x WJ blocks) = A_panel . B_panel^T over all of K.
// Uses the stage buffers; returns after a barrier with no copy in flight, so
// the caller may reuse them (e.g. g_stage0) right away.
template <int D, int W>
__device__ __forceinline__ void gemm_nt_tile(f32x16_t (&acc)[Gemm<W>::WI][Gemm<W>::WJ], const Panel& A,
                                             const Panel& B) {
  static_assert(NSTAGES == 4, "the unrolled loops below assume four stages");
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
#pragma unroll
  for (int i = 0; i < Gemm<W>::WI; ++i)
#pragma unroll
    for (int j = 0; j < Gemm<W>::WJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int nk = (int)((A.kbytes + ROWB - 1) / ROWB);
  const bool ragged = (A.kbytes % ROWB) != 0;
  const uint32_t wave_lds = (uint32_t)__builtin_amdgcn_readfirstlane(wave) * 1024u;
  CopyPlan<W> cp;
  copy_plan<W>(cp, A, B, t);
  lds_barrier();  // every wave is done with the buffers of any previous use
  // stages 0..2 (clamped to the last stage, as in kstage_edge)
  copy_any<W, 0>(cp, A, B, 0, nk, ragged, t);
  copy_any<W, 1>(cp, A, B, min(1, nk - 1), nk, ragged, t);
  copy_any<W, 2>(cp, A, B, min(2, nk - 1), nk, ragged, t);
  wait_vmcnt<2 * Gemm<W>::NCOP>();
  if (ragged && nk == 1) zero_tail<W, 0>(A, 0, t);
  lds_barrier();
  FragBase fb;
  frag_base<W>(fb, wave, lane);
  Frags<W> f0, f1;
  frag_read<W, 0>(f0, fb, 0);
  // Whole rounds of four plain stages (each copies a stage that is neither
  // past K nor ragged: kt+3+3 <= last_plain), then rounds of edge stages.
  // A loop header with only two predecessors keeps the waitcnt pass from
  // falling back to a full wait at the top of every round.
  const int last_plain = ragged ? nk - 2 : nk - 1;
  int kt = 0;
  for (; kt + 6 <= last_plain; kt += 4) {
    kstage_plain<D, W, 0>(acc, f0, f1, cp, fb, A, B, kt, wave_lds);
    kstage_plain<D, W, 1>(acc, f0, f1, cp, fb, A, B, kt + 1, wave_lds);
    kstage_plain<D, W, 2>(acc, f0, f1, cp, fb, A, B, kt + 2, wave_lds);
    kstage_plain<D, W, 3>(acc, f0, f1, cp, fb, A, B, kt + 3, wave_lds);
  }
  for (; kt < nk; kt += 4) {
    kstage_edge<D, W, 0>(acc, f0, f1, cp, fb, A, B, kt, nk, ragged, t);
    if (kt + 1 < nk) {
      kstage_edge<D, W, 1>(acc, f0, f1, cp, fb, A, B, kt + 1, nk, ragged, t);
      if (kt + 2 < nk) {
        kstage_edge<D, W, 2>(acc, f0, f1, cp, fb, A, B, kt + 2, nk, ragged, t);
        if (kt + 3 < nk) kstage_edge<D, W, 3>(acc, f0, f1, cp, fb, A, B, kt + 3, nk, ragged, t);
      }
    }
  }
  wait_vmcnt<0>();
  lds_barrier();
}

// Bijective remap of a 1-D workgroup id so that consecutive logical ids land
// on the same XCD (workgroups are dispatched round-robin over 8 XCDs).
__device__ __forceinline__ int xcd_logical_id(int bid, int nblocks) {
  const int q = nblocks / 8, rem = nblocks % 8;
  const int xcd = bid % 8, k = bid / 8;
  return xcd < rem ? xcd * (q + 1) + k : rem * (q + 1) + (xcd - rem) * q + k;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace flce
