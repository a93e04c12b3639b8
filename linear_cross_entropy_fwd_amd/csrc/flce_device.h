// flce_device.h -- gfx950 device building blocks: element types, MFMA
// wrappers and the LDS-staged "NT" GEMM tile (C = A . B^T with both operands
// K-contiguous) that the forward logit pass, the backward recompute pass and
// the two gradient contractions share.
//
// Tile geometry: a workgroup owns a 256 x 256 fp32 output tile, split over
// its 8 wave64s as blocks of the 16x16 MFMA (Gemm<W> below); operands stream
// through two LDS stage buffers fed by direct global-to-LDS copies (see
// gemm_nt_tile below).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

enum Dt : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

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

// One 16-byte fragment pair -> MFMA update of one 16x16 block.
//  16-bit types: lane l holds row (l&15), k = 8*(l>>4) .. +7 of the 32-deep
//  slab (v_mfma_f32_16x16x32).
//  fp32: the same 16 bytes are k = 4*(l>>4) .. +3 of the 16-deep slab; four
//  16x16x4 MFMAs each take element c of every lane (k = 4*(l>>4) + c), so
//  together they use every k of the slab exactly once.
template <int D> __device__ __forceinline__ void mfma_frag(f32x4_t& acc, uint4 a, uint4 b);

template <> __device__ __forceinline__ void mfma_frag<DT_BF16>(f32x4_t& acc, uint4 a, uint4 b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}
template <> __device__ __forceinline__ void mfma_frag<DT_F16>(f32x4_t& acc, uint4 a, uint4 b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                               __builtin_bit_cast(f16x8_t, b), acc, 0, 0, 0);
}
template <> __device__ __forceinline__ void mfma_frag<DT_F32>(f32x4_t& acc, uint4 a, uint4 b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

// Output element (row, col) of accumulator register e (0..3) of a 16x16
// block, for lane l:  col = l & 15,  row = 4*(l>>4) + e.
__device__ __forceinline__ int acc_row(int e, int lane) { return 4 * (lane >> 4) + e; }

// An operand panel: 256 rows starting at `base`, `ld` bytes apart, `kbytes`
// bytes of K (a multiple of 16).  Only rows < `rows` and bytes < kbytes of
// them are read from memory: reads past the panel's last valid byte return
// zeros, K past kbytes is zeroed in LDS, and results of rows past `rows` are
// never stored.
struct Panel {
  const char* base;
  int64_t ld;
  int rows;
  int64_t kbytes;
};

// ---------------------------------------------------------------------------
// Two-stage operand pipeline.  Global memory is copied straight into LDS
// (buffer_load_dwordx4 ... lds, 16 bytes per lane) one K-stage ahead of use
// into two buffers.  A stage is 128 bytes of K (one cache line per row) for all
// 256 rows of A and of B (64 KB); one copy instruction moves 8 whole rows
// (1 KB).  Rows are stored 128 bytes apart with the eight 16-byte chunks of
// row r at positions c ^ ((r>>1)&7), so that the 16 lanes that read one
// chunk of 16 consecutive rows hit all 64 LDS banks once.  A stage has two
// 64-byte slabs; the fragments of the next slab are read while the MFMAs of
// the current one run, and the one barrier per stage sits between them.

constexpr int ROWB = 128;                // K bytes per row per stage
constexpr int OPB = TILE * ROWB;         // one operand, one stage: 32 KB
constexpr int STB = 2 * OPB;             // A + B: 64 KB
constexpr int NSTAGES = 2;               // 128 KB of LDS
constexpr int NSLABS = ROWB / 64;        // 64-byte MFMA slabs per stage

__shared__ __attribute__((aligned(1024))) char g_stage0[STB];
__shared__ __attribute__((aligned(1024))) char g_stage1[STB];

// Separate arrays per stage (not one array with offsets) so that no access
// to one stage's buffer is mistaken for an access to another's.
template <int S> __device__ __forceinline__ char* stage_buf() {
  if constexpr (S == 0) return g_stage0;
  else return g_stage1;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

// One wave-wide copy of 16 bytes per lane from a buffer into LDS: lane l
// writes LDS bytes [lds + 16*l, +16) with the 16 bytes at byte offset `voff`
// of the buffer `rsrc`, or zeros where voff lies past its num_records (the
// range check that makes clamping unnecessary).  Issued through inline asm
// so that only the pipeline's explicit vmcnt waits order it (the compiler
// would otherwise wait for every outstanding copy before any LDS read of a
// stage buffer).  `rsrc` and `lds` are wave-uniform.
__device__ __forceinline__ void lds_copy16(const i32x4_t& rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds)
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
// grid of wave tiles of WI x WJ 16x16 blocks.  W = 8: two waves per SIMD,
// 128 x 64 per wave (128 accumulator registers); while one wave of a SIMD
// waits (a copy being issued, a barrier), the other keeps the MFMA unit busy.
// (One wave per SIMD with 128 x 128 each, the 256 accumulators in AGPRs,
// measured no faster in the K loops of the real kernels and slower in
// their epilogues, where no second wave fills the latencies.)
template <int W> struct Geo;
template <> struct Geo<8> { static constexpr int WI = 8, WJ = 4; };
template <int W> struct Gemm {
  static constexpr int WI = Geo<W>::WI, WJ = Geo<W>::WJ;
  static constexpr int GN = TILE / (16 * WJ);       // wave columns
  static constexpr int NBLK = 2 * TILE / 8;         // 8-row copy blocks per stage (64)
  static constexpr int NCOP = NBLK / W;             // copies per thread per stage
  static constexpr int NSTEP = WI * WJ;             // MFMAs per slab
  __device__ static int wm(int wave) { return wave / GN; }
  __device__ static int wn(int wave) { return wave % GN; }
};

// Fragment registers.  The MFMAs of a slab run row block by row block (A
// fragment i with every B fragment, then i+1), so A fragment i is dead after
// its last MFMA and is refilled in place with the next slab's; the B
// fragments are used until the end of the slab and alternate between two
// sets (slab 0 of a stage uses b[0], slab 1 b[1]).
template <int W> struct Frags {
  uint4 a[Gemm<W>::WI], b[2][Gemm<W>::WJ];
};

// Raw buffer resource (stride 0) over a panel's valid bytes, rows 0 ..
// rows-1 up to kbytes in the last one; everything in it is wave-uniform.
// The host keeps 256 row pitches below 2^32 bytes.
__device__ __forceinline__ i32x4_t panel_rsrc(const Panel& p) {
  const uint64_t u = (uint64_t)(uintptr_t)p.base;
  const int64_t extent = (int64_t)(p.rows - 1) * p.ld + p.kbytes;
  i32x4_t r;
  r[0] = (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)u);
  r[1] = (int32_t)(__builtin_amdgcn_readfirstlane((uint32_t)(u >> 32)) & 0xFFFFu);
  r[2] = (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)extent);
  r[3] = 0x00020000;  // gfx9 data format word: 32-bit, no swizzle
  return r;
}

// The copies of a stage.  Block b = 0..63 of a stage is operand b>>5, rows
// (b&31)*8 .. +8.  Copy i of wave w is block w + W*i (copies 0 .. NCOP/2-1
// are of operand A, the rest of B), so copy i of an operand covers rows
// 8*W*i + 8*w + L/8 for lane L: its offset is the lane's first one plus
// 8*W*i row pitches.  Lane L fills LDS chunk position L&7 of its row, which
// holds global chunk (L&7) ^ ((row>>1)&7) -- the same for every i.
template <int W> struct CopyPlan {
  i32x4_t ra, rb;   // buffer resources of A and B
  uint32_t oa, ob;  // the lane's byte offset in copy 0 of A / of B
  uint32_t sa, sb;  // 8*W row pitches of A / of B (wave-uniform)
  uint32_t kb;      // B bytes per stage: ROWB, or 64 row pitches when B is K-major
};

// K-major B (16-bit types): the B panel is stored [k][col], 256 columns
// (512 bytes) per K row, and a stage holds 64 K rows of it (the same 32 KB).
// Copy block bb = 0..31 of B is K rows 2 bb, 2 bb + 1; lane L fills chunk
// position L & 31 of row 2 bb + L / 32.  Chunk c of K row r sits at position
// c ^ kswz(r): the 16 rows that one transposed fragment read touches
// (8 g + [0, 4) and 8 g + 4 + [0, 4) for g = 0..3) then spread their 32-byte
// pieces over all eight 32-byte bank groups, two rows each.  kswz depends on
// bits 0, 1 and 3 of r only, so it is the same for rows 16 apart (the copies
// of one lane), 4 apart (a fragment's two reads) and 32 apart (the slabs).
__device__ __forceinline__ constexpr int kswz(int r) { return 2 * ((r & 3) | (((r >> 3) & 1) << 2)); }

template <int W> __device__ __forceinline__ constexpr int copy_block(int i, int wave) { return wave + W * i; }
__device__ __forceinline__ int copy_row(int blk, int L) { return (blk & 31) * 8 + (L >> 3); }
__device__ __forceinline__ int copy_chunk(int row, int L) { return (L & 7) ^ ((row >> 1) & 7); }

// BK: B is K-major (B.rows = K rows, B.kbytes = the last row's valid column bytes; the host
// keeps every K-row offset of the panel below 2^32 bytes).
template <int W, bool BK = false>
__device__ __forceinline__ void copy_plan(CopyPlan<W>& cp, const Panel& A, const Panel& B, int t) {
  const int wave = t >> 6, L = t & 63;
  const int row = copy_row(copy_block<W>(0, wave), L);
  const uint32_t c16 = (uint32_t)(copy_chunk(row, L) * 16);
  cp.ra = panel_rsrc(A);
  cp.rb = panel_rsrc(B);
  cp.oa = (uint32_t)(row * A.ld) + c16;
  cp.sa = __builtin_amdgcn_readfirstlane((uint32_t)(8 * W * A.ld));
  if constexpr (BK) {
    static_assert(W == 8, "four B copies of 2 K rows per wave and stage");
    const int kr = 2 * wave + (L >> 5);  // K row of copy 0; copy i adds 16 i
    cp.ob = (uint32_t)(kr * B.ld) + (uint32_t)((((L & 31) ^ kswz(kr))) * 16);
    cp.sb = __builtin_amdgcn_readfirstlane((uint32_t)(16 * B.ld));
    cp.kb = __builtin_amdgcn_readfirstlane((uint32_t)(64 * B.ld));
  } else {
    cp.ob = (uint32_t)(row * B.ld) + c16;
    cp.sb = __builtin_amdgcn_readfirstlane((uint32_t)(8 * W * B.ld));
    cp.kb = (uint32_t)ROWB;
  }
}

// Copy I of the stage at K byte offset k0 into buffer S.  Stages past K (the
// pipeline runs two ahead) and rows past the panel read zeros.
template <int W> struct StageCopy {
  const CopyPlan<W>& cp;
  uint32_t k0;        // wave-uniform
  uint32_t wave_lds;  // wave * 1024 (wave-uniform)
  uint32_t kb0;       // B's offset of the stage (k0 unless B is K-major)
  template <int S, int I> __device__ __forceinline__ void issue() const {
    constexpr int H = Gemm<W>::NCOP / 2;
    constexpr bool OPA = I < H;
    constexpr uint32_t ii = OPA ? I : I - H;
    const uint32_t soff = (OPA ? k0 : kb0) + ii * (OPA ? cp.sa : cp.sb);
    lds_copy16(OPA ? cp.ra : cp.rb, (OPA ? cp.oa : cp.ob) + soff,
               lds_addr(stage_buf<S>() + W * I * 1024) + wave_lds);
  }
};

template <int W, int S, int I = 0>
__device__ __forceinline__ void copy_stage(const StageCopy<W>& c) {
  if constexpr (I < Gemm<W>::NCOP) {
    c.template issue<S, I>();
    copy_stage<W, S, I + 1>(c);
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
    const int c = copy_chunk(copy_row(blk, L), L);
    if (k0 + c * 16 >= A.kbytes) *reinterpret_cast<uint4*>(base + blk * 1024 + L * 16) = make_uint4(0u, 0u, 0u, 0u);
  }
}

// Byte offsets, inside a stage buffer, of this lane's fragment chunk of each
// slab for its first A and first B row block.  The lane reads rows
// r0 + 16*i + (l&15): they differ by multiples of 16, so the swizzle term
// ((row>>1)&7) = ((l&15)>>1)&7 is the same for all its blocks, which then sit
// 16*ROWB bytes apart (an immediate offset).
struct FragBase {
  uint32_t a[NSLABS], b[NSLABS];
};

template <int W, bool BK = false>
__device__ __forceinline__ void frag_base(FragBase& fb, int wave, int lane) {
  const int r16 = lane & 15, q = lane >> 4, x = (r16 >> 1) & 7;
  const int ra = Gemm<W>::wm(wave) * 16 * Gemm<W>::WI, rb = Gemm<W>::wn(wave) * 16 * Gemm<W>::WJ;
#pragma unroll
  for (int s = 0; s < NSLABS; ++s) {
    const uint32_t coff = (uint32_t)(((4 * s + q) ^ x) << 4);
    fb.a[s] = (uint32_t)((ra + r16) * ROWB) + coff;
    fb.b[s] = (uint32_t)(OPB + (rb + r16) * ROWB) + coff;
  }
  if constexpr (BK) {
    // K-major B, first read of fragment 0 of slab 0: lane 16 g + i addresses
    // K row 8 g + i / 4, columns rb + 4 (i & 3) .. +3 (chunk rb / 8 + (i & 3) / 2,
    // byte 8 (i & 1) in it).  Fragment J flips chunk bits 1-2 (offset ^ 32 J),
    // the second read is 4 rows on (+2048), slab 1 is 32 rows on (+16384).
    const int kr = 8 * q + (r16 >> 2);
    const int chunk = rb / 8 + ((r16 & 3) >> 1);
    fb.b[0] = (uint32_t)(OPB + kr * 512 + ((chunk ^ kswz(kr)) << 4) + 8 * (r16 & 1));
    fb.b[1] = fb.b[0] + 16384u;
  }
}

// A fragment I / B fragment J of slab SL of buffer S: lane (l&15, l>>4)
// reads chunk 4*SL + (l>>4) of its row.  B fragments of slab SL go to set SL.
template <int W, int S, int SL, int I>
__device__ __forceinline__ void read_a(Frags<W>& f, const FragBase& fb) {
  f.a[I] = *reinterpret_cast<const uint4*>(stage_buf<S>() + fb.a[SL] + I * 16 * ROWB);
}
template <int W, int S, int SL, int J, bool BK = false>
__device__ __forceinline__ void read_b(Frags<W>& f, const FragBase& fb) {
  if constexpr (BK) {
    // two transposed reads: lane 16 g + i gets column i of K rows 8 g + [0, 4)
    // and 8 g + 4 + [0, 4) of the fragment, i.e. its k = 8 g .. 8 g + 7
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4* lp;
    const uint32_t off = fb.b[SL] ^ (uint32_t)(32 * J);
    const uint32_t base = lds_addr(stage_buf<S>());
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lp>(base + off));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lp>(base + off + 2048u));
    const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
    f.b[SL][J] = make_uint4(l2.x, l2.y, h2.x, h2.y);
  } else {
    f.b[SL][J] = *reinterpret_cast<const uint4*>(stage_buf<S>() + fb.b[SL] + J * 16 * ROWB);
  }
}

// Item k of M spread evenly over N steps goes after step floor(k*N/M).
__device__ __forceinline__ constexpr int spread(int s, int M, int N) {
  const int k = (s * M + N - 1) / N;
  return (k < M && (k * N) / M == s) ? k : -1;
}

// What follows MFMA step s = (i, j) of a slab (i = s / WJ, j = s % WJ):
//  - after the last MFMA of row block i (j = WJ-1): the next slab's A fragment i;
//  - the next slab's B fragment k after step 2k (early: the next slab needs
//    all of them in its first WJ steps);
//  - with COPIES (every copy of a stage in one slab): copy k after step
//    floor(k * NSTEP / NCOP), the first right after the barrier.
template <int W> __device__ __forceinline__ constexpr int step_read_b(int s) {
  return (s & 1) == 0 && s < 2 * Gemm<W>::WJ ? s / 2 : -1;
}
template <int W, bool COPIES> __device__ __forceinline__ constexpr int step_copy(int s) {
  if constexpr (!COPIES) return -1;
  else return spread(s, Gemm<W>::NCOP, Gemm<W>::NSTEP);
}

struct NoCopy {
  template <int S, int I> __device__ __forceinline__ void issue() const {}
};

// Extra work a kernel may run on stage kt's operands while they sit in
// buffer S, in two parts per stage, called in stage order:
//   run<S>(kt):   after the stage's MFMAs have read all of buffer S and the
//                 copies of stage kt+1 have landed, just before the barrier
//                 after which buffer S is overwritten (its LDS writes are
//                 complete and visible after that barrier);
//   after<S>(kt): right after that barrier, before the stage's second slab.
// Neither should add a branch to the K loop.  NoSide: none.
struct NoSide {
  template <int S> __device__ __forceinline__ void run(int) {}
  template <int S> __device__ __forceinline__ void after(int) {}
};

// One slab's WI x WJ MFMAs on A fragments f.a and B fragments f.b[SC], with
// the fragment reads of the next slab (slab RSL of buffer RS) and, if COPIES,
// the stage's NCOP copies (into buffer CS) placed between them as the step
// functions above say: a wave issues in order and would otherwise stall its
// MFMAs behind a burst of copies or reads.
template <int D, int W, int SC, int RS, int RSL, int CS, bool COPIES, bool BK, int STEP = 0, class Copy>
__device__ __forceinline__ void slab_phase(f32x4_t (&acc)[Gemm<W>::WI][Gemm<W>::WJ], Frags<W>& f,
                                           const FragBase& fb, const Copy& cp) {
  constexpr int WJ = Gemm<W>::WJ;
  if constexpr (STEP < Gemm<W>::NSTEP) {
    constexpr int I = STEP / WJ, J = STEP % WJ;
    mfma_frag<D>(acc[I][J], f.a[I], f.b[SC][J]);
    if constexpr (J == WJ - 1) read_a<W, RS, RSL, I>(f, fb);
    constexpr int rb = step_read_b<W>(STEP), cpy = step_copy<W, COPIES>(STEP);
    if constexpr (rb >= 0) read_b<W, RS, RSL, rb, BK>(f, fb);
    if constexpr (cpy >= 0) cp.template issue<CS, cpy>();
    sched_fence();
    slab_phase<D, W, SC, RS, RSL, CS, COPIES, BK, STEP + 1>(acc, f, fb, cp);
  }
}

// Every fragment of slab SL of buffer S.
template <int W, int S, int SL, bool BK, int K = 0>
__device__ __forceinline__ void frag_read(Frags<W>& f, const FragBase& fb) {
  if constexpr (K < Gemm<W>::WI) {
    read_a<W, S, SL, K>(f, fb);
    frag_read<W, S, SL, BK, K + 1>(f, fb);
  } else if constexpr (K < Gemm<W>::WI + Gemm<W>::WJ) {
    read_b<W, S, SL, K - Gemm<W>::WI, BK>(f, fb);
    frag_read<W, S, SL, BK, K + 1>(f, fb);
  }
}

// Stage kt from buffer S (f holds its slab 0; stage kt+1's copies are in
// flight into S^1):
//   slab 0: MFMAs | reads of slab 1
//   wait for every copy (stage kt+1), zero its ragged tail, barrier: every
//   wave is done reading buffer S and stage kt+1 is visible
//   slab 1: MFMAs | reads of slab 0 of stage kt+1 (S^1) | every copy of
//   stage kt+2 (into S), as early as the buffer allows
template <int D, int W, int S, bool BK, class C, class Side>
__device__ __forceinline__ void kstage(f32x4_t (&acc)[Gemm<W>::WI][Gemm<W>::WJ], Frags<W>& f,
                                       const FragBase& fb, const C& c, bool zero_next, const Panel& A, int kt,
                                       int t, Side& side) {
  static_assert(NSLABS == 2, "the schedule below assumes two slabs");
  constexpr int SN = S ^ 1;
  const NoCopy nc;
  sched_fence();
  slab_phase<D, W, 0, S, 1, SN, false, BK>(acc, f, fb, nc);
  wait_vmcnt<0>();
  if (zero_next) zero_tail<W, SN>(A, kt + 1, t);
  sched_fence();
  side.template run<S>(kt);
  sched_fence();
  lds_barrier();
  side.template after<S>(kt);
  sched_fence();
  slab_phase<D, W, 1, SN, 0, S, true, BK>(acc, f, fb, c);
}

// Stage kt; the copies it issues are of stage kt+2.  zero_next: stage kt+1
// is the ragged last one.
template <int D, int W, int S, bool EDGE, bool BK, class Side>
__device__ __forceinline__ void kstage_at(f32x4_t (&acc)[Gemm<W>::WI][Gemm<W>::WJ], Frags<W>& f,
                                          const CopyPlan<W>& cp, const FragBase& fb, const Panel& A, int kt,
                                          int nk, bool ragged, uint32_t wave_lds, int t, Side& side) {
  const uint32_t k0 = (uint32_t)(kt + 2) * ROWB;
  uint32_t kb0 = k0;
  if constexpr (BK) kb0 = (uint32_t)(kt + 2) * cp.kb;
  const StageCopy<W> c{cp, k0, wave_lds, kb0};
  kstage<D, W, S, BK>(acc, f, fb, c, EDGE && ragged && kt + 1 == nk - 1, A, kt, t, side);
}

// The first two stages of a tile: the copy plan and the copies of stages 0
// and 1.  Waits (at a barrier) until every wave is done with the stage
// buffers of any previous use; the caller may then run code that touches
// neither the stage buffers nor vector memory counters it waits on exactly
// (e.g. the previous tile's epilogue) before gemm_run.
template <int W, bool BK = false>
__device__ __forceinline__ void gemm_prefetch(CopyPlan<W>& cp, const Panel& A, const Panel& B) {
  const int t = threadIdx.x;
  const uint32_t wave_lds = (uint32_t)__builtin_amdgcn_readfirstlane(t >> 6) * 1024u;
  copy_plan<W, BK>(cp, A, B, t);
  lds_barrier();  // every wave is done with the buffers of any previous use
  copy_stage<W, 0>(StageCopy<W>{cp, 0u, wave_lds, 0u});
  copy_stage<W, 1>(StageCopy<W>{cp, (uint32_t)ROWB, wave_lds, BK ? cp.kb : (uint32_t)ROWB});
}

// acc[i][j] (this wave's WI x WJ blocks) = A_panel . B_panel^T over all of K,
// from a gemm_prefetch of the same panels.  Uses the stage buffers; returns
// after a barrier with no copy in flight, so the caller may reuse them (e.g.
// g_stage0) right away.
// ZERO = false: acc arrives holding values to add to (loaded by the caller
// before gemm_prefetch, so that those loads complete in order ahead of the
// stage copies and the first wait below covers them).
template <int D, int W, class Side, bool ZERO = true, bool BK = false>
__device__ __forceinline__ void gemm_run(f32x4_t (&acc)[Gemm<W>::WI][Gemm<W>::WJ], const CopyPlan<W>& cp,
                                         const Panel& A, Side& side) {
  static_assert(NSTAGES == 2, "the loops below alternate two buffers");
  constexpr int H = Gemm<W>::NCOP / 2;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if constexpr (ZERO) {
#pragma unroll
    for (int i = 0; i < Gemm<W>::WI; ++i)
#pragma unroll
      for (int j = 0; j < Gemm<W>::WJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;
  }
  const int nk = (int)((A.kbytes + ROWB - 1) / ROWB);
  const bool ragged = (A.kbytes % ROWB) != 0;
  const uint32_t wave_lds = (uint32_t)__builtin_amdgcn_readfirstlane(wave) * 1024u;
  // stage 0 has landed once at most the 2H younger copies (stage 1, and any
  // later vector memory op) are outstanding: they complete in order
  wait_vmcnt<2 * H>();
  if (ragged && nk == 1) zero_tail<W, 0>(A, 0, t);
  lds_barrier();
  FragBase fb;
  frag_base<W, BK>(fb, wave, lane);
  Frags<W> f;
  frag_read<W, 0, 0, BK>(f, fb);
  // Pairs of stages none of whose successors is the ragged last stage, then
  // the rest.  A loop header with only two predecessors keeps the waitcnt
  // pass from falling back to a full wait at the top of every round.
  const int last_plain = ragged ? nk - 2 : nk - 1;
  int kt = 0;
  for (; kt + 3 <= last_plain; kt += 2) {
    kstage_at<D, W, 0, false, BK>(acc, f, cp, fb, A, kt, nk, ragged, wave_lds, t, side);
    kstage_at<D, W, 1, false, BK>(acc, f, cp, fb, A, kt + 1, nk, ragged, wave_lds, t, side);
  }
  for (; kt < nk; kt += 2) {
    kstage_at<D, W, 0, true, BK>(acc, f, cp, fb, A, kt, nk, ragged, wave_lds, t, side);
    if (kt + 1 < nk) kstage_at<D, W, 1, true, BK>(acc, f, cp, fb, A, kt + 1, nk, ragged, wave_lds, t, side);
  }
  wait_vmcnt<0>();
  lds_barrier();
}

template <int D, int W, class Side>
__device__ __forceinline__ void gemm_nt_tile(f32x4_t (&acc)[Gemm<W>::WI][Gemm<W>::WJ], const Panel& A,
                                             const Panel& B, Side& side) {
  CopyPlan<W> cp;
  gemm_prefetch<W>(cp, A, B);
  gemm_run<D, W>(acc, cp, A, side);
}

// acc = A_panel . B^T with B K-major (16-bit types): B.base is column 0 of
// K row 0, B.ld the K-row pitch, B.rows the valid K rows and B.kbytes the
// valid column bytes of the last of them (at most 512): the copies read 512
// bytes of every K row, zeros past that range.  A's K must be whole stages
// (a multiple of ROWB bytes).  ZERO = false: acc arrives holding values to
// add to, as in gemm_run.
template <int D, int W, bool ZERO = true>
__device__ __forceinline__ void gemm_tile_kmajor_b(f32x4_t (&acc)[Gemm<W>::WI][Gemm<W>::WJ], const Panel& A,
                                                   const Panel& B) {
  static_assert(Elem<D>::bytes == 2, "transposed fragment reads are of 16-bit elements");
  NoSide none;
  CopyPlan<W> cp;
  gemm_prefetch<W, true>(cp, A, B);
  gemm_run<D, W, NoSide, ZERO, true>(acc, cp, A, none);
}

template <int D, int W>
__device__ __forceinline__ void gemm_nt_tile(f32x4_t (&acc)[Gemm<W>::WI][Gemm<W>::WJ], const Panel& A,
                                             const Panel& B) {
  NoSide none;
  gemm_nt_tile<D, W>(acc, A, B, none);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace flce
