// flce_device.h -- gfx950 device building blocks: element types, MFMA
// wrappers and the LDS-staged "NT" GEMM tile (C = A . B^T with both operands
// K-contiguous) that the forward logit pass, the backward recompute pass and
// the two gradient contractions share.
//
// Tile geometry: a workgroup of 256 threads (4 wave64s, one per SIMD) owns a
// 256 x 256 fp32 output tile; wave w covers rows [128*(w>>1), +128) and
// columns [128*(w&1), +128) as 4 x 4 blocks of the 32x32 MFMA.  K advances
// 128 bytes per stage (64 bf16/f16 or 32 fp32 values); two LDS stages of
// 256 rows x 144 bytes per operand (16 bytes of padding per row keep the
// 16-byte fragment reads bank-conflict free), refilled from registers that
// were loaded from global memory one stage ahead.
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
constexpr int NTHREADS = 256;      // 4 waves
constexpr int KBYTES = 128;        // K bytes per stage
constexpr int PITCH = 144;         // LDS row pitch (bytes)
constexpr int OP_BYTES = TILE * PITCH;           // one operand, one stage
constexpr int STAGE_BYTES = 2 * OP_BYTES;        // A + B
constexpr int LDS_BYTES = 2 * STAGE_BYTES;       // double buffered: 147456

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

template <bool MASKED>
__device__ __forceinline__ void panel_load(uint4 (&r)[8], const Panel& p, int64_t k0, int t) {
  const int seg = t & 7, rb = t >> 3;
  const int64_t koff = k0 + seg * 16;
  const bool kin = !MASKED || koff < p.kbytes;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int row = rb + 32 * i;
    row = row < p.rows ? row : p.rows - 1;
    const uint4* src = reinterpret_cast<const uint4*>(p.base + (int64_t)row * p.ld + koff);
    if (MASKED) r[i] = kin ? *src : make_uint4(0u, 0u, 0u, 0u);
    else r[i] = *src;
  }
}

// Loads K-stage `kt`; only a ragged last stage (K not a multiple of 128
// bytes) takes the masked path.
__device__ __forceinline__ void stage_load(uint4 (&ra)[8], uint4 (&rb)[8], const Panel& A,
                                           const Panel& B, int kt, int nfull, int t) {
  const int64_t k0 = (int64_t)kt * KBYTES;
  if (kt < nfull) {
    panel_load<false>(ra, A, k0, t);
    panel_load<false>(rb, B, k0, t);
  } else {
    panel_load<true>(ra, A, k0, t);
    panel_load<true>(rb, B, k0, t);
  }
}

__device__ __forceinline__ void panel_store_lds(char* lds_op, const uint4 (&r)[8], int t) {
  const int seg = t & 7, rb = t >> 3;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<uint4*>(lds_op + (rb + 32 * i) * PITCH + seg * 16) = r[i];
}

template <int D>
__device__ __forceinline__ void stage_mfma(f32x16_t (&acc)[4][4], const char* la, const char* lb,
                                           int wm, int wn, int lane) {
  const int r32 = lane & 31, half = lane >> 5;
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) {
    uint4 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *reinterpret_cast<const uint4*>(la + (wm * 128 + i * 32 + r32) * PITCH + kc * 32 + half * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = *reinterpret_cast<const uint4*>(lb + (wn * 128 + j * 32 + r32) * PITCH + kc * 32 + half * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) mfma_frag<D>(acc[i][j], a[i], b[j]);
  }
}

// acc[i][j] (this wave's 4x4 blocks) = A_panel . B_panel^T over all of K.
// Ends with a barrier, so the caller may reuse `lds` right away.
template <int D>
__device__ __forceinline__ void gemm_nt_tile(f32x16_t (&acc)[4][4], const Panel& A, const Panel& B,
                                             char* lds) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nfull = (int)(A.kbytes / KBYTES);
  const int nk = (int)((A.kbytes + KBYTES - 1) / KBYTES);
  uint4 ra[8], rb[8];
  stage_load(ra, rb, A, B, 0, nfull, t);
  panel_store_lds(lds, ra, t);
  panel_store_lds(lds + OP_BYTES, rb, t);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const char* cur = lds + (kt & 1) * STAGE_BYTES;
    char* nxt = lds + ((kt + 1) & 1) * STAGE_BYTES;
    const bool more = kt + 1 < nk;
    if (more) stage_load(ra, rb, A, B, kt + 1, nfull, t);
    stage_mfma<D>(acc, cur, cur + OP_BYTES, wm, wn, lane);
    if (more) {
      panel_store_lds(nxt, ra, t);
      panel_store_lds(nxt + OP_BYTES, rb, t);
    }
    __syncthreads();
  }
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
