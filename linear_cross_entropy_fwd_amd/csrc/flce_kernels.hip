// flce_kernels.hip -- gfx950 kernels of fused linear cross-entropy.
//
// Forward (trl-lib "fused-linear-ce" card, "Algorithm" and "Metrics for
// free"): each workgroup computes 256 x 256 logit tiles z^T = W . hidden^T
// with bf16/f16 (or fp32) MFMA into fp32 registers, applies bias / scale /
// soft cap, and folds every tile into per-row online log-sum-exp state
// (running max m and rescaled sum S), together with the target-logit gather,
// the running argmax and the entropy sum U = sum e^{z-m} (z-m).  Vocabulary
// ids run along the MFMA row axis, so each lane owns 4 token columns and
// reduces its 32 logits per column in registers; the four lanes that share
// a column merge by lane shuffles every tile, and the two waves that share a
// token merge once per split.  Nothing of size N x V
// is written: per (row, split) a record of m and S (plus U and the argmax
// value and id with metrics, plus the logit sum with label smoothing), and
// per row the target logit from the split that holds the target.
//
// Backward (card: "Algorithm", backward): per vocabulary chunk of Cv ids,
// recompute the logit tiles and form G = (p - onehot) * coef * dz/draw in the
// input dtype, then contract
//   grad_hidden += G . W_c        (fp32 accumulator across chunks)
//   grad_weight[c] = G^T . hidden (complete per chunk, written once)
// with the same GEMM tile.  For 16-bit types both contractions read their B
// operand K-major through transposed LDS fragment reads (G itself for
// grad_weight, the chunk's weight rows for grad_hidden), so only hidden is
// transposed, once per call.  The fp32 path, which has no transposed
// 32-bit fragment read, has the recompute kernel write G^T as well and
// transposes the chunk's weight rows into W_c^T.  grad_bias sums G over rows
// per tile, then over tiles in a fixed order.  No atomics: results are
// deterministic.
#include <math.h>

#include <mutex>
#include <type_traits>

#include "flce_device.h"
#include "flce_plan.h"

namespace flce {

// ------------------------------------------------------------------ helpers

// An int the compiler cannot see through: per-tile epilogue indices derived
// from it are recomputed after each tile's GEMM instead of being hoisted out
// of the tile loop and kept live (in registers the K-loop needs) across it.
__device__ __forceinline__ int opaque_int(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// tanh u from its definition, 1 - 2 / (e^{2u} + 1), given x = 2 u log2(e)
// (so that e^{2u} = 2^x is one hardware exp2), with the hardware reciprocal:
// an absolute error of a few 1e-7 (so cap * tanh is off by a few 1e-7 cap at
// most).  No sign handling is needed: 2^x = inf (u past ~44) gives exactly 1,
// 2^x = 0 gives exactly -1, and NaN stays NaN.
__device__ __forceinline__ float tanh_of_exp2_arg(float x) {
  return fmaf(-2.f, __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(x) + 1.f), 1.f);
}

// Merge online-softmax state (m2,S2,U2) into (m,S,U).  Symmetric in its two
// operands (fp add / mul commute), so the merge order of a pair never
// changes the bits.  U = sum e^{z-m}(z-m) rescales as e^{m-M}(U + (m-M) S).
template <bool METRICS>
__device__ __forceinline__ void lse_merge(float& m, float& S, float& U, float m2, float S2, float U2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  float s1 = 0.f, s2 = 0.f, u1 = 0.f, u2 = 0.f;
  if (m != -INFINITY) {
    const float d = m - M;
    const float al = fast_exp2(d * LOG2E);
    s1 = S * al;
    if (METRICS) u1 = al * fmaf(d, S, U);
  }
  if (m2 != -INFINITY) {
    const float d = m2 - M;
    const float al = fast_exp2(d * LOG2E);
    s2 = S2 * al;
    if (METRICS) u2 = al * fmaf(d, S2, U2);
  }
  m = M;
  S = s1 + s2;
  if (METRICS) U = u1 + u2;
}

// First-index argmax merge: larger value wins, ties go to the smaller id.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

// Bias of the rows this lane holds: row vq + 16*i + e of accumulator
// element [i][.][e] (vq = the wave's first row + 4*(lane>>4)).
template <int D, bool BIAS, int WI>
__device__ __forceinline__ void load_bias_rows(float (&bv)[WI][4], const char* bias, int vq, int64_t V) {
  typedef typename Elem<D>::T T;
  const T* b = reinterpret_cast<const T*>(bias);
#pragma unroll
  for (int i = 0; i < WI; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (BIAS) {
        int64_t v = (int64_t)vq + 16 * i + e;
        v = v < V ? v : V - 1;
        bv[i][e] = to_f32<D>(b[v]);
      } else {
        bv[i][e] = 0.f;
      }
    }
}

// The four lanes l, l^16, l^32, l^48 hold the same accumulator column over
// disjoint rows.  Butterfly reductions over them: every lane ends with the
// same bits (each step adds or compares a pair in either order).
__device__ __forceinline__ float col_max4(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float col_sum4(float x) {
  x = x + __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}
// Sum over the 16 lanes of a row (lanes 16 r .. 16 r + 15, one token column
// each) by rotations within the row (DPP row_ror: VALU operands, no LDS):
// every lane ends with the row's sum, lane 16 r in the order it is used.
template <int N> __device__ __forceinline__ float row_ror(float x) {
  static_assert(N >= 1 && N <= 15, "row_ror range");
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x120 + N, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_sum16(float x) {
  x = x + row_ror<8>(x);
  x = x + row_ror<4>(x);
  x = x + row_ror<2>(x);
  return x + row_ror<1>(x);
}
__device__ __forceinline__ int col_min4(int x) {
  x = min(x, __shfl_xor(x, 16));
  return min(x, __shfl_xor(x, 32));
}

// ------------------------------------------------------------------ forward tiles

// Per-column online state between vocabulary tiles, in LDS so that it does
// not occupy registers across the GEMM: 8 values (m, S, U, target logit,
// argmax value and id, target id, logit sum) x WJ column blocks x 16 columns
// per wave (16 KB next to the 128 KB stage buffers).
__shared__ float g_fwd_state[8 * 4 * 8 * 16];

template <int D, bool METRICS, bool BIAS, bool CAP, int W>
__global__ __launch_bounds__(W * 64) void fwd_tiles_kernel(FwdArgs a) {
  constexpr int EB = Elem<D>::bytes, WI = Gemm<W>::WI, WJ = Gemm<W>::WJ, GN = Gemm<W>::GN;
  static_assert(8 * WJ * W * 16 <= 8 * 4 * 8 * 16, "online state does not fit g_fwd_state");
  static_assert(GN * 16 * WJ == TILE && 2 * 16 * WI == TILE, "two wave rows share each column");
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = Gemm<W>::wm(wave), wn = Gemm<W>::wn(wave), c16 = lane & 15, q = lane >> 4;

  const TileAB ti = grouped_tile<kFwdGA, kFwdGB, kFwdXcd>(blockIdx.x, gridDim.x, a.n_tok_tiles, a.n_groups);
  if (!ti.valid) return;
  const int tt = ti.a;
  const int split_first = ti.b * a.splits_per_wg;
  const int split_last = min(split_first + a.splits_per_wg, a.n_splits);  // one past
  const int64_t n0 = (int64_t)tt * TILE;
  const int wg_vt_end = min(split_last * a.tiles_per_split, a.n_voc_tiles);
  const int64_t rowb = a.H * EB;

  Panel B{a.hidden + n0 * rowb, rowb, (int)min<int64_t>(TILE, a.N - n0), rowb};

  // Slot k of column block j of this lane's column: 0 m, 1 S, 2 U,
  // 3 z_target, 4 argmax value, 5 argmax id, 6 target id (-1 when the row is
  // ignored or its target is out of range), 7 sum of z (label smoothing).  The four lanes of a column hold
  // the same m, S, U and argmax (they are merged every tile); z_target is
  // written only by the lane that holds the target's row.  Slot 6 holds for
  // the whole workgroup, the others start again with each split.
  const int so = wave * 16 + c16;  // this lane's column slots
#define FST(k, j) g_fwd_state[so + ((k) * WJ + (j)) * (W * 16)]
  if (q == 0) {
#pragma unroll
    for (int j = 0; j < WJ; ++j) {
      const int64_t n = n0 + wn * 16 * WJ + 16 * j + c16;
      const int64_t tv = n < a.N ? a.targets[n] : a.ignore_index;
      FST(6, j) = __int_as_float((tv != a.ignore_index && tv >= 0 && tv < a.V) ? (int)tv : -1);
    }
  }

  f32x4_t acc[WI][WJ];
  // The first two stages of each next vocabulary tile, also the next
  // split's first, are copied before this tile's epilogue (which touches
  // only registers and g_fwd_state), so the copies' latency hides behind it.
  CopyPlan<W> cp;
  {
    const int64_t v0 = (int64_t)split_first * a.tiles_per_split * TILE;
    gemm_prefetch<W>(cp, Panel{a.weight + v0 * rowb, rowb, (int)min<int64_t>(TILE, a.V - v0), rowb}, B);
  }
  for (int split = split_first; split < split_last; ++split) {
    if (q == 0) {
#pragma unroll
      for (int j = 0; j < WJ; ++j) {
        FST(0, j) = -INFINITY;
        FST(1, j) = 0.f;
        FST(2, j) = 0.f;
        FST(3, j) = 0.f;
        FST(4, j) = -INFINITY;
        FST(5, j) = __int_as_float(0x7fffffff);
        FST(7, j) = 0.f;
      }
    }
    const int vt_end = min((split + 1) * a.tiles_per_split, a.n_voc_tiles);
    for (int vt = split * a.tiles_per_split; vt < vt_end; ++vt) {
      const int64_t v0 = (int64_t)vt * TILE;
      Panel A{a.weight + v0 * rowb, rowb, (int)min<int64_t>(TILE, a.V - v0), rowb};
      NoSide none;
      gemm_run<D, W>(acc, cp, A, none);
      if (vt + 1 < wg_vt_end)
        gemm_prefetch<W>(cp, Panel{A.base + TILE * rowb, rowb, (int)min<int64_t>(TILE, a.V - v0 - TILE), rowb}, B);

      const int to = opaque_int(t);
      const int qo = (to >> 4) & 3;
      const int vbase = (int)v0 + Gemm<W>::wm(to >> 6) * 16 * WI;  // this wave's first row
      const int vq = vbase + 4 * qo;                                // row of acc[i][.][e]: vq + 16 i + e
      // rows of this lane at or past V (only in the last, ragged tile): vq + 16 i + e >= V
      const int vrem = (int)min<int64_t>(a.V - vq, 1 << 20);
      const bool ragged = vrem < 16 * WI;  // wave-uniform
      // Each logit as a key that orders like it: with a soft cap the tanh t
      // (z = cap t, cap > 0), else z itself.  The bias folds into one FMA:
      // with a cap, x = 2 log2(e) s (y + b) / cap is the exp2 argument of t.
      const float kscale = CAP ? a.s * a.inv_cap * (2.f * LOG2E) : a.s;
      float bv[WI][4];
      load_bias_rows<D, BIAS, WI>(bv, a.bias, vq, a.V);
      if (BIAS) {
#pragma unroll
        for (int i = 0; i < WI; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) bv[i][e] = bv[i][e] * kscale;
      }
      const float kz = CAP ? a.cap : 1.f;  // z = kz * key

#pragma unroll
      for (int j = 0; j < WJ; ++j) {
        float z[WI][4];  // the keys
#pragma unroll
        for (int i = 0; i < WI; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = BIAS ? fmaf(acc[i][j][e], kscale, bv[i][e]) : acc[i][j][e] * kscale;
            z[i][e] = CAP ? tanh_of_exp2_arg(x) : x;
          }
        if (ragged) {  // a branch only the last tile takes, not a select per element
#pragma unroll
          for (int i = 0; i < WI; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (16 * i + e >= vrem) z[i][e] = -INFINITY;
        }
        float zl = -INFINITY;
#pragma unroll
        for (int i = 0; i < WI; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) zl = fmaxf(zl, z[i][e]);
        if (a.zsum) {  // label smoothing: the sum of z over the vocabulary
          float zs = 0.f;
#pragma unroll
          for (int i = 0; i < WI; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (!ragged || 16 * i + e < vrem) zs = zs + z[i][e];
          zs = col_sum4(zs);
          if (q == 0) FST(7, j) = fmaf(kz, zs, FST(7, j));
        }
        const float kmax = col_max4(zl);
        const float zmax = kz * kmax;
        const float mold = FST(0, j);
        const float mnew = fmaxf(mold, zmax);
        if (mnew != -INFINITY) {
          // four independent partial sums (one per accumulator register), so
          // that the adds do not wait on each exp in turn.  The exp argument
          // (z - m) log2(e) is one FMA of the key, and the entropy term
          // e^{z-m} (z - m) is taken in those units (times ln 2 per column).
          float sp[4] = {0.f, 0.f, 0.f, 0.f}, up[4] = {0.f, 0.f, 0.f, 0.f};
          const float ml = mnew * LOG2E, kl = kz * LOG2E;
#pragma unroll
          for (int i = 0; i < WI; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float arg = fmaf(z[i][e], kl, -ml);
              const float ex = fast_exp2(arg);
              sp[e] = sp[e] + ex;
              // (the floor keeps a logit of -inf, a row past V or a bias of
              // -inf, at 0 * -1e30 = 0 instead of 0 * -inf = NaN)
              if (METRICS) up[e] = fmaf(ex, fmaxf(arg, -1e30f), up[e]);
            }
          float sum = (sp[0] + sp[1]) + (sp[2] + sp[3]), usum = 0.f;
          if (METRICS) usum = (up[0] + up[1]) + (up[2] + up[3]);
          sum = col_sum4(sum);
          if (METRICS) usum = col_sum4(usum) * LN2;
          if (q == 0) {
            if (mold == -INFINITY) {
              FST(1, j) = sum;
              if (METRICS) FST(2, j) = usum;
            } else {
              const float dm = mold - mnew;
              const float al = fast_exp2(dm * LOG2E);
              const float Sold = FST(1, j);
              if (METRICS) FST(2, j) = fmaf(al, fmaf(dm, Sold, FST(2, j)), usum);
              FST(1, j) = fmaf(Sold, al, sum);
            }
            FST(0, j) = mnew;
          }
        }
        if (METRICS && zmax > FST(4, j)) {
          // the first row of the column's largest key: a select per element,
          // from the last row to the first
          int loc = -1;
#pragma unroll
          for (int i = WI - 1; i >= 0; --i)
#pragma unroll
            for (int e = 3; e >= 0; --e) loc = z[i][e] == kmax ? 16 * i + e : loc;
          const int idx = col_min4(loc >= 0 ? vq + loc : 0x7fffffff);
          if (q == 0) {
            FST(4, j) = zmax;
            FST(5, j) = __int_as_float(idx);
          }
        }
        const int local = __float_as_int(FST(6, j)) - vbase;
        if (local >= 0 && local < 16 * WI && ((local & 15) >> 2) == qo) {
          const int ti = local >> 4, te = local & 3;
          float zv = 0.f;
#pragma unroll
          for (int i = 0; i < WI; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (i == ti && e == te) zv = z[i][e];
          FST(3, j) = kz * zv;
        }
      }
    }

    // The split is complete.  Waves wm = 0 and wm = 1 hold the same token
    // columns over disjoint vocabulary rows: the first merges the second's
    // state (read from its LDS slots) into its own and writes the split's
    // record.  The stage buffers may hold the next split's first copies; the
    // record's stores are issued after them, so the next GEMM's first wait
    // covers the stores too (once per split, not per tile).
    lds_barrier();
    if (wm == 0) {
      // rows of part and zt_rows are padded to whole tiles (pitch npad), so no
      // lane needs a predicate: the four lanes of a column store the same
      // values, columns past N land in the padding, and a split that does
      // not hold a row's target writes the row's slot in zt_rows' second half
      // (indices from an opaque copy of the thread id: derived from it
      // outside, they would be kept live, and spilled, across the K loops)
      const int tm = opaque_int(t), wv = tm >> 6, cm = tm & 15;
      const int64_t stride = (int64_t)a.n_splits * a.npad;
      const int po = (wv + GN) * 16 + cm;  // the partner's slots
#define PST(k, j) g_fwd_state[po + ((k) * WJ + (j)) * (W * 16)]
#pragma unroll
      for (int j = 0; j < WJ; ++j) {
        float m = FST(0, j), S = FST(1, j), U = FST(2, j), av = FST(4, j);
        int ai = __float_as_int(FST(5, j));
        lse_merge<METRICS>(m, S, U, PST(0, j), PST(1, j), PST(2, j));
        if (METRICS) argmax_merge(av, ai, PST(4, j), __float_as_int(PST(5, j)));
        const int col = Gemm<W>::wn(wv) * 16 * WJ + 16 * j + cm;
        float* p = a.part + (int64_t)split * a.npad + n0 + col;
        p[0] = m;
        p[stride] = S;
        if (METRICS) {
          p[2 * stride] = U;
          p[3 * stride] = av;
          p[4 * stride] = __int_as_float(ai);
        }
        if (a.zsum) p[part_zs_field(METRICS) * stride] = FST(7, j) + PST(7, j);
        const int tv = __float_as_int(FST(6, j));
        const bool own = tv >= 0 && tv / TILE / a.tiles_per_split == split;
        a.zt_rows[(own ? 0 : a.npad) + n0 + col] = FST(3, j) + PST(3, j);  // the non-owner holds +0
      }
#undef PST
    }
    lds_barrier();  // before the next split resets the state
  }
#undef FST
}

// ------------------------------------------------------------------ forward combine / reduce

// One workgroup per 32 rows; the 8 groups of 32 threads each fold the
// splits k = p, p+8, p+16, ... of their row into a partial state, then the
// first group merges the 8 partials in the order p = 0..7 (a fixed order, so
// a row's result does not depend on the launch or on N).
template <bool METRICS>
__global__ __launch_bounds__(256) void fwd_combine_kernel(CombineArgs a) {
  constexpr int ROWS = 32, PARTS = 8;
  __shared__ float sh[6][PARTS][ROWS];
  const int t = threadIdx.x, rl = t % ROWS, p = t / ROWS;
  const int64_t n = (int64_t)blockIdx.x * ROWS + rl;
  const bool in = n < a.N;
  const int64_t stride = (int64_t)a.n_splits * a.npad;
  const float* pm = a.part + (in ? n : 0);
  const int64_t zsf = part_zs_field(METRICS);
  float M = -INFINITY, S = 0.f, U = 0.f, av = -INFINITY, Z = 0.f;
  int ai = 0x7fffffff;
  if (in) {
    for (int k = p; k < a.n_splits; k += PARTS) M = fmaxf(M, pm[(int64_t)k * a.npad]);
    if (a.zsum)
      for (int k = p; k < a.n_splits; k += PARTS) Z = Z + pm[zsf * stride + (int64_t)k * a.npad];
    for (int k = p; k < a.n_splits; k += PARTS) {
      const float mk = pm[(int64_t)k * a.npad];
      if (mk != -INFINITY) {
        const float d = mk - M;
        const float al = fast_exp2(d * LOG2E);
        const float sk = pm[stride + (int64_t)k * a.npad];
        S = S + sk * al;
        if (METRICS) U = U + al * fmaf(d, sk, pm[2 * stride + (int64_t)k * a.npad]);
      }
      if (METRICS)
        argmax_merge(av, ai, pm[3 * stride + (int64_t)k * a.npad],
                     __float_as_int(pm[4 * stride + (int64_t)k * a.npad]));
    }
  }
  sh[0][p][rl] = M;
  sh[1][p][rl] = S;
  sh[2][p][rl] = U;
  sh[3][p][rl] = av;
  sh[4][p][rl] = __int_as_float(ai);
  sh[5][p][rl] = Z;
  __syncthreads();
  if (p != 0 || !in) return;
  for (int q = 1; q < PARTS; ++q) {
    lse_merge<METRICS>(M, S, U, sh[0][q][rl], sh[1][q][rl], sh[2][q][rl]);
    if (METRICS) argmax_merge(av, ai, sh[3][q][rl], __float_as_int(sh[4][q][rl]));
    Z = Z + sh[5][q][rl];
  }
  const int64_t tv = a.targets[n];
  const bool valid = tv != a.ignore_index;
  const bool foreign = a.shard && tv == a.foreign;  // another shard's id: no target logit here
  const bool bad = valid && !foreign && (tv < 0 || tv >= a.V);
  const float logS = logf(S);
  const float lse = M + logS;
  float row = 0.f, rw = 0.f;
  if (valid && !foreign) {
    if (bad) {
      row = NAN;
    } else if (a.shard) {
      row = a.zt_rows[n];  // the target logit (no variants with shards)
    } else {
      const float zt = a.zt_rows[n];
      // smoothed cross-entropy + z-loss, times the row's class weight (all
      // of it exact for the plain loss: eps = 0, z_loss = 0, weight 1)
      rw = a.class_weight ? a.class_weight[tv] : 1.f;
      row = rw * ((lse - (1.f - a.eps) * zt) - (a.eps / (float)a.V) * Z + a.z_loss * (lse * lse));
    }
  }
  if (a.row_w) a.row_w[n] = rw;
  if (a.lse_out) a.lse_out[n] = lse;
  if (a.loss_rows) a.loss_rows[n] = row;
  a.row_loss[n] = row;
  int flag = (valid ? 1 : 0) | (bad ? 4 : 0);
  if (METRICS) {
    if (a.predictions) a.predictions[n] = (int64_t)ai;
    if (valid && !foreign && !bad && ai == tv) flag |= 2;
    a.row_ent[n] = valid ? logS - U / S : 0.f;
    if (a.shard) {
      a.shard_max[n] = av;
      a.shard_argmax[n] = (int64_t)ai + a.voff;
      a.shard_ent[n] = logS - U / S;
    }
  }
  a.row_flag[n] = flag;
}

template <bool METRICS>
__global__ __launch_bounds__(1024) void fwd_reduce_kernel(ReduceArgs a) {
  __shared__ double sh_l[1024], sh_e[1024], sh_w[1024];
  __shared__ int sh_v[1024], sh_h[1024], sh_b[1024];
  const int t = threadIdx.x;
  double sl = 0.0, se = 0.0, sw = 0.0;
  int nv = 0, nh = 0, nb = 0;
  for (int64_t n = t; n < a.N; n += 1024) {
    const int f = a.row_flag[n];
    sl += (double)a.row_loss[n];
    if (a.row_w) sw += (double)a.row_w[n];
    nv += f & 1;
    nh += (f >> 1) & 1;
    nb |= (f >> 2) & 1;
    if (METRICS) se += (double)a.row_ent[n];
  }
  sh_l[t] = sl;
  sh_e[t] = se;
  sh_w[t] = sw;
  sh_v[t] = nv;
  sh_h[t] = nh;
  sh_b[t] = nb;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (t < w) {
      sh_l[t] += sh_l[t + w];
      sh_e[t] += sh_e[t + w];
      sh_w[t] += sh_w[t + w];
      sh_v[t] += sh_v[t + w];
      sh_h[t] += sh_h[t + w];
      sh_b[t] |= sh_b[t + w];
    }
    __syncthreads();
  }
  if (t == 0) {
    const int64_t nvalid = sh_v[0];
    // mean: over the count of valid rows, or over their class-weight total
    const double den = a.row_w ? sh_w[0] : (double)nvalid;
    if (a.reduction == 0) a.loss[0] = nvalid > 0 ? (float)(sh_l[0] / den) : NAN;
    if (a.reduction == 1) a.loss[0] = (float)sh_l[0];
    if (METRICS && a.metrics) {
      a.metrics[0] = nvalid > 0 ? (float)((double)sh_h[0] / (double)nvalid) : NAN;
      a.metrics[1] = nvalid > 0 ? (float)(sh_e[0] / (double)nvalid) : NAN;
    }
    a.status[0] = (uint32_t)sh_b[0];
  }
}

// The loss of a vocabulary split into shards.  Each shard's forward gives a
// row's log-sum-exp over the shard's ids and, at the shard that holds the
// row's target, the target logit (0 at the others).  Here lse = M + log sum_k
// e^{lse_k - M} (M the largest, k in shard order) and the row loss is lse
// minus the sum of the target logits.  One thread per row.
__global__ __launch_bounds__(256) void shard_combine_kernel(ShardCombineArgs a) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= a.N) return;
  float M = -INFINITY;
  for (int k = 0; k < a.n_shards; ++k) M = fmaxf(M, a.shard_lse[(int64_t)k * a.N + n]);
  float S = 0.f, zt = 0.f;
  for (int k = 0; k < a.n_shards; ++k) {
    const float lk = a.shard_lse[(int64_t)k * a.N + n];
    if (lk != -INFINITY) S = S + fast_exp2((lk - M) * LOG2E);
    zt = zt + a.target_logit[(int64_t)k * a.N + n];
  }
  const float lse = M + logf(S);
  const int64_t tv = a.targets[n];
  const bool valid = tv != a.ignore_index;
  const bool bad = valid && (tv < 0 || tv >= a.V);
  const float row = !valid ? 0.f : bad ? NAN : lse - zt;
  if (a.lse_out) a.lse_out[n] = lse;
  if (a.loss_rows) a.loss_rows[n] = row;
  a.row_loss[n] = row;
  int flag = (valid ? 1 : 0) | (bad ? 4 : 0);
  if (a.shard_max) {
    // The argmax: the first shard holding the largest value (shards in id
    // order keep the first index on ties).  The entropy: with q_k the
    // shard's softmax and w_k = e^{lse_k - lse} its share of the whole,
    // E_p[z] = sum_k w_k (lse_k - H_k), so H = lse - sum_k w_k (lse_k - H_k).
    float best = -INFINITY, ez = 0.f;
    int64_t id = 0;
    for (int k = 0; k < a.n_shards; ++k) {
      const int64_t o = (int64_t)k * a.N + n;
      const float mk = a.shard_max[o];
      if (k == 0 || mk > best) {
        best = mk;
        id = a.shard_argmax[o];
      }
      const float lk = a.shard_lse[o];
      if (lk != -INFINITY) ez = ez + fast_exp2((lk - lse) * LOG2E) * (lk - a.shard_ent[o]);
    }
    if (a.predictions) a.predictions[n] = id;
    if (valid && !bad && id == tv) flag |= 2;
    a.row_ent[n] = valid ? lse - ez : 0.f;
  }
  a.row_flag[n] = flag;
}

// ------------------------------------------------------------------ backward helpers

__global__ __launch_bounds__(1024) void bwd_prep_kernel(PrepArgs a) {
  // the mean's denominator: the count of non-ignored rows, or with class
  // weights their weight total (in-range targets only; a bad target makes
  // the gradient NaN anyway), summed in fp64 in a fixed order
  __shared__ double sh[1024];
  const int t = threadIdx.x;
  double nv = 0.0;
  for (int64_t n = t; n < a.N; n += 1024) {
    const int64_t tv = a.targets[n];
    if (tv == a.ignore_index) continue;
    if (!a.class_weight) nv += 1.0;
    else if (tv >= 0 && tv < a.V) nv += (double)a.class_weight[tv];
  }
  sh[t] = nv;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (t < w) sh[t] += sh[t + w];
    __syncthreads();
  }
  if (t == 0) {
    float scale = 1.f;
    if (a.reduction != 2) {
      const float g = a.grad_loss ? a.grad_loss[0] : 1.f;
      if (a.reduction == 0) scale = sh[0] > 0.0 ? (float)((double)g / sh[0]) : 0.f;
      else scale = g;
    }
    a.scale[0] = scale * a.s;
  }
}

// dst[c][r] (row pitch dst_ld) = src[r][c] for r < rows, 0 for rows <= r < rpad.  A workgroup
// moves a 64-row x 256-byte tile: 16-byte loads along src rows, through LDS,
// 16-byte stores along dst rows.  Needs cols*EB and src_ld*EB multiples of 16
// (hidden*bytes % 16 == 0 is checked at the boundary) and rpad % 64 == 0.
template <int EB>
__global__ __launch_bounds__(256) void transpose_kernel(TransposeArgs a) {
  typedef typename std::conditional<EB == 4, uint32_t, uint16_t>::type U;
  constexpr int E = 16 / EB;           // elements per 16 bytes
  constexpr int TR = 64, TC = 16 * E;  // tile: TR src rows x TC src cols
  constexpr int PITCH = TC + E;        // LDS row pitch: 16-byte aligned, not a multiple of 128 bytes
  constexpr int SEGS = TR / E;         // 16-byte pieces per dst row of the tile
  __shared__ __attribute__((aligned(16))) U tile[TR * PITCH];
  const int64_t r0 = (int64_t)blockIdx.x * TR, c0 = (int64_t)blockIdx.y * TC;
  const U* src = reinterpret_cast<const U*>(a.src);
  U* dst = reinterpret_cast<U*>(a.dst);
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = t + 256 * i, row = q >> 4, seg = q & 15;
    const int64_t r = r0 + row, c = c0 + seg * E;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < a.rows && c < a.cols) v = *reinterpret_cast<const uint4*>(src + r * a.src_ld + c);
    *reinterpret_cast<uint4*>(tile + row * PITCH + seg * E) = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = t + 256 * i, cc = q / SEGS, sg = q % SEGS;
    const int64_t c = c0 + cc, r = r0 + sg * E;
    if (c >= a.cols || r >= a.rpad) continue;
    alignas(16) U e[E];
#pragma unroll
    for (int k = 0; k < E; ++k) e[k] = tile[(sg * E + k) * PITCH + cc];
    *reinterpret_cast<uint4*>(dst + c * a.dst_ld + r) = *reinterpret_cast<const uint4*>(e);
  }
}

__global__ void fill_zero_kernel(uint8_t* p, int64_t bytes) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < bytes;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// ------------------------------------------------------------------ backward G (recompute)

// A 256 x 256 tile of 16-bit values, row r's 16-byte chunk c stored at chunk
// position c ^ (r & 31) (rows 512 bytes apart), rows 0..127 in g_stage0 and
// 128..255 in g_stage1 (both free once gemm_nt_tile has returned).  Lanes
// writing 8 bytes of 16 different rows then spread over the LDS banks, and a
// row can be read back as 16-byte pieces and stored fully coalesced.
__device__ __forceinline__ char* tile16_addr(int row, int col) {
  char* buf = row < 128 ? g_stage0 : g_stage1;
  const int r = row & 127;
  return buf + r * 512 + ((((col >> 3) ^ (r & 31))) << 4) + (col & 7) * 2;
}

// Four consecutive columns col..col+3 (col % 4 == 0) of row `row`.
template <int D>
__device__ __forceinline__ void tile16_put4(int row, int col, float x0, float x1, float x2, float x3) {
  typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
  u16x4 v;
  v[0] = __builtin_bit_cast(uint16_t, from_f32<D>(x0));
  v[1] = __builtin_bit_cast(uint16_t, from_f32<D>(x1));
  v[2] = __builtin_bit_cast(uint16_t, from_f32<D>(x2));
  v[3] = __builtin_bit_cast(uint16_t, from_f32<D>(x3));
  *reinterpret_cast<u16x4*>(tile16_addr(row, col)) = v;
}

// Stores the staged tile: row r, columns c0.. go to dst + r * ld (elements),
// for r < rows and chunk columns below cols (a multiple of 8).  Callers put a
// barrier between the last tile16_put4 and this.  STREAM: non-temporal
// stores, which do not keep the lines in the caches.
template <int NT, bool STREAM = false>
__device__ __forceinline__ void tile16_store(uint16_t* dst, int64_t ld, int rows, int cols, int t) {
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
#pragma unroll 4
  for (int k = t; k < TILE * 32; k += NT) {
    const int r = k >> 5, c = k & 31;
    if (r < rows && 8 * c < cols) {
      const u32x4v v = *reinterpret_cast<const u32x4v*>(tile16_addr(r, 8 * c));
      u32x4v* p = reinterpret_cast<u32x4v*>(dst + (int64_t)r * ld + 8 * c);
      if constexpr (STREAM) __builtin_nontemporal_store(v, p);
      else *p = v;
    }
  }
}

// Stores the staged tile transposed: dst[c][r] (row pitch ld elements) for
// tile row r < rows, column c < cols, from transposed LDS reads.  In a group
// of 16 lanes, lane i reads row r0 + i/4, columns c0 + 4*(i%4) .. +3 (8
// bytes); ds_read_b64_tr_b16 hands lane j the four values of column c0 + j
// in rows r0 .. r0+3.  Two such reads give a lane 8 consecutive rows of one
// column: a 16-byte piece of a dst row.  The four groups of a wave take
// consecutive 8-row pieces of the same 16 columns, so a wave stores 16 dst
// row pieces of 64 bytes.  Callers put a barrier between the last
// tile16_put4 and this.
__device__ __forceinline__ void tile16_store_t(uint16_t* dst, int64_t ld, int rows, int cols, int t) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const int w = t >> 6, gw = (t >> 4) & 3, i = t & 15;
#pragma unroll 2
  for (int it = 0; it < 16; ++it) {
    const int cb = w + 8 * (it & 1);        // 16-column block (tile column = dst row)
    const int rb = 4 * (it >> 1) + gw;      // 8-row block (tile row = dst column)
    const int r0 = 8 * rb, c0 = 16 * cb;
    const int rr = r0 + (i >> 2), cc = c0 + 4 * (i & 3);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) s16x4*>(lds_addr(tile16_addr(rr, cc))));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) s16x4*>(lds_addr(tile16_addr(rr + 4, cc))));
    const int c = c0 + i;
    if (c < cols && r0 < rows) {
      uint4 v;
      v.x = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
      v.y = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
      v.z = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
      v.w = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
      *reinterpret_cast<uint4*>(dst + (int64_t)c * ld + r0) = v;
    }
  }
}

// Side job of the recompute kernel (16-bit types): while stage kt of the
// weight tile (256 vocabulary rows x 64 hidden columns) sits in LDS, one of
// the workgroups that share the vocabulary tile also writes it transposed
// into W_c^T[h][vl] (row pitch ld), so grad_hidden needs no separate
// transpose of the chunk.  Token tile tt takes the stages kt = tt mod
// n_tok_tiles (the host asks for this only with at least 4 token tiles).
//
// Part 1, before the stage's barrier: the stage is transposed into a 32 KB
// LDS tile T[h][vl] (64 rows of 512 bytes; 16-byte chunk c of row h sits at
// c ^ (h & 31), conflict-free for both passes).  Wave w takes hidden
// columns 16 (w >> 1) + [0, 16) and, in each of the four 64-row parts p of
// the stage, rows 64 p + 32 (w & 1) + [0, 32).  Lane L = 16 g + i reads row
// 64 p + 32 (w & 1) + L / 4 and 16 + that row, 4 columns at 4 (i % 4), with
// ds_read_b64_tr_b16, which hands lane i column i of rows 4 g + [0, 4)
// (and 16 + those): two 8-byte writes into row h = 16 (w >> 1) + i of T.
// The stage's row swizzle (row >> 1) & 7 is the same for all eight rows a
// lane reads, so they are one address at immediate offsets; in T, part p
// and the second read are the first write address xor 128 p and xor 32.
// Part 2, after the barrier: wave w stores rows 8 w + [0, 8) of T, two rows
// of 512 bytes per instruction (whole cache lines; 8-byte stores straight
// from the transposed reads ran several times slower).
// Each part is one asm block that the other workgroups jump over (exec mask
// empty): the K loop gets no branch and no register that lives across it.
__shared__ __attribute__((aligned(1024))) char g_wct_tile[64 * 512];

struct WcTSide {
  uint16_t* wct;
  int64_t H;
  int cvpad, ld, vl0, ntt;  // columns of this chunk, row pitch of W_c^T
  uint32_t wave;  // wave-uniform
  int ks;         // next stage of this workgroup
  uint64_t m;     // this stage: exec if selected, else 0
  template <int S> __device__ __forceinline__ void run(int kt) {
    const bool in = kt == ks;  // wave-uniform
    ks += in ? ntt : 0;
    m = __builtin_amdgcn_ballot_w64(in);  // exec or 0, without a branch
    const int hrem = (int)min<int64_t>(64, H - (int64_t)kt * (ROWB / 2));
    const int vrem = cvpad - vl0;  // rows of the tile inside W_c^T (a multiple of 64)
    const uint32_t hb16 = 16u * (wave >> 1), w32 = 32u * (wave & 1u), ch16 = 32u * (wave >> 1);
    const uint32_t lb = lds_addr(stage_buf<S>()) + 128u * w32;
    const uint32_t tb = lds_addr(g_wct_tile);
    uint64_t save, lo, hi;
    uint32_t t0, t1, t2, t3;
#define FLCE_WCT_PART(P, NEXT)                                            \
  "s_cmp_gt_i32 %[vr], " #P "*64\n\t"                                     \
  "s_cbranch_scc0 1f\n\t"                                                 \
  "ds_read_b64_tr_b16 %[lo], %[t0] offset:" #P "*8192\n\t"                \
  "ds_read_b64_tr_b16 %[hi], %[t0] offset:" #P "*8192+2048\n\t"           \
  "s_waitcnt lgkmcnt(0)\n\t"                                              \
  "ds_write_b64 %[t1], %[lo]\n\t"                                         \
  "v_xor_b32 %[t3], 32, %[t1]\n\t"                                        \
  "ds_write_b64 %[t3], %[hi]\n\t"                                         \
  "v_xor_b32 %[t1], " #NEXT ", %[t1]\n\t"
    asm volatile(
        "s_mov_b64 %[sv], exec\n\t"
        "s_mov_b64 exec, %[m]\n\t"
        "s_cbranch_execz 1f\n\t"
        "v_mbcnt_lo_u32_b32 %[t2], -1, 0\n\t"
        "v_mbcnt_hi_u32_b32 %[t2], -1, %[t2]\n\t"   // L
        // transposed-read address: 128 (L / 4) + 16 ((2 hb + (L >> 1) & 1) ^ ((L >> 3) & 7)) + 8 (L & 1)
        "v_and_b32 %[t0], -4, %[t2]\n\t"
        "v_lshlrev_b32 %[t0], 5, %[t0]\n\t"
        "v_xor_b32 %[t0], %[ch], %[t0]\n\t"
        "v_lshlrev_b32 %[t1], 3, %[t2]\n\t"
        "v_and_b32 %[t1], 24, %[t1]\n\t"
        "v_xor_b32 %[t0], %[t0], %[t1]\n\t"
        "v_lshlrev_b32 %[t1], 1, %[t2]\n\t"
        "v_and_b32 %[t1], 0x70, %[t1]\n\t"
        "v_xor_b32 %[t0], %[t0], %[t1]\n\t"
        "v_add_u32 %[t0], %[lb], %[t0]\n\t"
        "v_and_b32 %[t1], 15, %[t2]\n\t"
        "v_add_u32 %[t1], %[hb], %[t1]\n\t"          // hl
        "v_cmp_gt_i32 vcc, %[hr], %[t1]\n\t"         // hl < hrem
        "s_mov_b64 exec, vcc\n\t"
        "s_cbranch_execz 1f\n\t"
        // T write address of part 0: tb + 512 hl + ((8 g + 64 (w & 1)) ^ 16 (hl & 31))
        "v_and_b32 %[t3], 31, %[t1]\n\t"
        "v_lshlrev_b32 %[t3], 4, %[t3]\n\t"
        "v_lshrrev_b32 %[t2], 1, %[t2]\n\t"
        "v_and_b32 %[t2], 24, %[t2]\n\t"
        "v_or_b32 %[t2], %[w64], %[t2]\n\t"
        "v_xor_b32 %[t2], %[t2], %[t3]\n\t"
        "v_lshl_add_u32 %[t1], %[t1], 9, %[t2]\n\t"
        "v_add_u32 %[t1], %[tb], %[t1]\n\t"
        FLCE_WCT_PART(0, 128) FLCE_WCT_PART(1, 384) FLCE_WCT_PART(2, 128) FLCE_WCT_PART(3, 0)
        "1:\n\t"
        "s_mov_b64 exec, %[sv]"
        : [sv] "=&s"(save), [lo] "=&v"(lo), [hi] "=&v"(hi), [t0] "=&v"(t0), [t1] "=&v"(t1), [t2] "=&v"(t2),
          [t3] "=&v"(t3)
        : [m] "s"(m), [hr] "s"(hrem), [vr] "s"(vrem), [lb] "s"(lb), [tb] "s"(tb), [hb] "s"(hb16),
          [w64] "s"(2u * w32), [ch] "s"(ch16)
        : "memory", "vcc", "scc");
#undef FLCE_WCT_PART
  }
  template <int S> __device__ __forceinline__ void after(int kt) {
    const int hrem = (int)min<int64_t>(64, H - (int64_t)kt * (ROWB / 2));
    const int vrem = cvpad - vl0;
    const uint32_t tb = lds_addr(g_wct_tile);
    const char* sb = uniform_ptr(reinterpret_cast<const char*>(wct + (int64_t)kt * (ROWB / 2) * ld + vl0));
    uint64_t save, rows;
    uint4 d;
    uint32_t t0, t1, t2, t3;
    // row h = 8 w + 2 J + L / 32, chunk c = L & 31: T at tb + 512 h + 16 (c ^ (h & 31)),
    // W_c^T at sb + 2 ld h + 16 c
#define FLCE_WCT_ROW(J)                                                   \
  "s_mov_b64 exec, %[rw]\n\t"                                             \
  "v_add3_u32 %[t0], %[h8], " #J "*2, %[t2]\n\t"                          \
  "v_cmp_gt_i32 vcc, %[hr], %[t0]\n\t"                                    \
  "s_mov_b64 exec, vcc\n\t"                                               \
  "s_cbranch_execz 2f\n\t"                                                \
  "v_and_b32 %[t1], 31, %[t0]\n\t"                                        \
  "v_xor_b32 %[t1], %[t1], %[t3]\n\t"                                     \
  "v_lshlrev_b32 %[t1], 4, %[t1]\n\t"                                     \
  "v_lshl_add_u32 %[t1], %[t0], 9, %[t1]\n\t"                             \
  "v_add_u32 %[t1], %[tb], %[t1]\n\t"                                     \
  "ds_read_b128 %[d], %[t1]\n\t"                                          \
  "v_mul_lo_u32 %[t0], %[t0], %[cp2]\n\t"                                 \
  "v_lshl_add_u32 %[t0], %[t3], 4, %[t0]\n\t"                             \
  "s_waitcnt lgkmcnt(0)\n\t"                                              \
  "global_store_dwordx4 %[t0], %[d], %[sb]\n"                             \
  "2:\n\t"
    asm volatile(
        "s_mov_b64 %[sv], exec\n\t"
        "s_mov_b64 exec, %[m]\n\t"
        "s_cbranch_execz 1f\n\t"
        "v_mbcnt_lo_u32_b32 %[t2], -1, 0\n\t"
        "v_mbcnt_hi_u32_b32 %[t2], -1, %[t2]\n\t"   // L
        "v_and_b32 %[t3], 31, %[t2]\n\t"             // c
        "v_lshlrev_b32 %[t0], 3, %[t3]\n\t"
        "v_cmp_gt_i32 vcc, %[vr], %[t0]\n\t"         // 8 c < vrem
        "s_mov_b64 exec, vcc\n\t"
        "s_cbranch_execz 1f\n\t"
        "s_mov_b64 %[rw], exec\n\t"
        "v_lshrrev_b32 %[t2], 5, %[t2]\n\t"          // L / 32
        FLCE_WCT_ROW(0) FLCE_WCT_ROW(1) FLCE_WCT_ROW(2) FLCE_WCT_ROW(3)
        "1:\n\t"
        "s_mov_b64 exec, %[sv]"
        : [sv] "=&s"(save), [rw] "=&s"(rows), [d] "=&v"(d), [t0] "=&v"(t0), [t1] "=&v"(t1), [t2] "=&v"(t2),
          [t3] "=&v"(t3)
        : [m] "s"(m), [hr] "s"(hrem), [vr] "s"(vrem), [tb] "s"(tb), [sb] "s"(sb), [h8] "s"(8u * wave),
          [cp2] "s"(2 * ld)
        : "memory", "vcc");
#undef FLCE_WCT_ROW
  }
};

// Per-token inputs of the recompute tile (see g_tile).
__shared__ int g_col_code[TILE];
__shared__ float g_col_lse[TILE];
__shared__ float g_col_gr[TILE];

// Recompute one (token tile, vocabulary tile) of the chunk and write
// G = coef * (softmax - onehot) * dz/draw (G^T too when asked, grad_bias partials).
// A = weight rows (vocabulary on the MFMA row axis), B = hidden rows.
// Workgroup `bid` of a grid of `nblocks` (the tile order of grouped_tile).
// WCT: the W_c^T side job may be asked for (16-bit types).
template <int D, bool BIAS, bool CAP, int W, bool WCT>
__device__ __forceinline__ void g_tile(const GArgs& a, int bid, int nblocks) {
  typedef typename Elem<D>::T T;
  constexpr int EB = Elem<D>::bytes, WI = Gemm<W>::WI, WJ = Gemm<W>::WJ;
  static_assert(Gemm<W>::GN == kBiasParts || W != kRecomputeWaves, "grad_bias partials per token tile");
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = Gemm<W>::wm(wave), wn = Gemm<W>::wn(wave), c16 = lane & 15, q = lane >> 4;

  const TileAB ti = grouped_tile<kRecGA, kRecGB, kRecXcd>(bid, nblocks, a.n_tok_tiles, a.n_voc_tiles);
  if (!ti.valid) return;
  const int tt = ti.a, vt = ti.b;
  const int64_t n0 = (int64_t)tt * TILE;
  const int vl0 = vt * TILE;              // chunk-local first id of the tile
  const int64_t v0 = a.c0 + vl0;          // global first id
  const int64_t rowb = a.H * EB;

  Panel A{a.weight + v0 * rowb, rowb, (int)min<int64_t>(TILE, a.V - v0), rowb};
  Panel B{a.hidden + n0 * rowb, rowb, (int)min<int64_t>(TILE, a.N - n0), rowb};
  // Without the W_c^T side job (whose LDS tile leaves no room), the tile's
  // per-token inputs are loaded ahead of the operand copies (their latency
  // then passes with the first stages') and parked in LDS until the
  // epilogue: thread c < 256 takes token n0 + c.  Target code: the id, -1
  // for a dead token (past N or ignored), -2 for an id outside [0, V), -3
  // for another vocabulary shard's id.
  constexpr bool PARK = !WCT;
  f32x4_t acc[WI][WJ];
  if constexpr (PARK) {
    const int64_t cn = n0 + t;
    int64_t col_tv = a.ignore_index;
    float col_lse = 0.f, col_gr = 1.f;
    if (t < TILE && cn < a.N) {
      col_tv = a.targets[cn];
      col_lse = a.lse[cn];
      if (a.none_reduction && a.grad_rows) col_gr = a.grad_rows[cn];
    }
    CopyPlan<W> cp;
    gemm_prefetch<W>(cp, A, B);
    sched_fence();  // the loads' first use stays behind the copies
    if (t < TILE) {
      g_col_code[t] = col_tv == a.ignore_index ? -1
                      : col_tv == a.foreign          ? -3
                      : (col_tv < 0 || col_tv >= a.V) ? -2
                                                      : (int)col_tv;
      g_col_lse[t] = col_lse;
      g_col_gr[t] = col_gr;
    }
    NoSide none;
    gemm_run<D, W>(acc, cp, A, none);
  } else if constexpr (EB == 2) {
    // no W_c^T wanted: a first stage past every stage selects none
    WcTSide side{reinterpret_cast<uint16_t*>(a.WcT), a.H, a.cvpad, a.wct_ld, vl0, a.n_tok_tiles,
                 (uint32_t)__builtin_amdgcn_readfirstlane(t >> 6), a.WcT != nullptr ? tt : (1 << 30), 0ull};
    gemm_nt_tile<D, W>(acc, A, B, side);
  } else {
    gemm_nt_tile<D, W>(acc, A, B);
  }

  // Per column: lse, the gradient factor (row weight times the per-row
  // upstream gradient), the softmax factor 1 + 2 z_loss lse and the target
  // id.  A dead column (past N or ignored) gets lse = +inf and factor 0, so
  // its p is 0 and its G column 0 without a select per element.
  //   dL/dz_j = w (pscale p_j - keep [j = t] - eps/V),  keep = 1 - eps
  // (parked: g_col_* were written before the K loop's barriers)
  float lse[WJ], coef[WJ], pscale[WJ];
  int tgt[WJ];
#pragma unroll
  for (int j = 0; j < WJ; ++j) {
    const int col = wn * 16 * WJ + 16 * j + c16;
    const int64_t n = n0 + col;
    int code = -1;
    float cl = 0.f, gr = 1.f;
    if constexpr (PARK) {
      code = g_col_code[col];
      cl = g_col_lse[col];
      gr = g_col_gr[col];
    } else if (n < a.N) {
      const int64_t tv = a.targets[n];
      code = tv == a.ignore_index ? -1 : tv == a.foreign ? -3 : (tv < 0 || tv >= a.V) ? -2 : (int)tv;
      if (code != -1) cl = a.lse[n];
      if (code != -1 && a.none_reduction && a.grad_rows) gr = a.grad_rows[n];
    }
    tgt[j] = -1;
    lse[j] = INFINITY;
    coef[j] = 0.f;
    pscale[j] = 1.f;
    if (code != -1) {
      lse[j] = cl;
      pscale[j] = fmaf(a.zl2, lse[j], 1.f);
      if (code == -2) {
        coef[j] = NAN;
      } else {
        tgt[j] = code;  // -3 (another shard's id) matches no row: no one-hot term
        coef[j] = gr;
        if (a.class_weight && code >= 0) coef[j] = coef[j] * a.class_weight[code];
      }
    }
  }

  const int vq = (int)v0 + wm * 16 * WI + 4 * q;  // row of acc[i][.][e]: vq + 16 i + e
  // The logit's key as in the forward: with a soft cap the exp2 argument
  // x = 2 log2(e) s (y + b) / cap of th = tanh(s (y + b) / cap), else
  // s (y + b); the bias folds into one FMA.
  const float kscale = CAP ? a.s * a.inv_cap * (2.f * LOG2E) : a.s;
  float bv[WI][4];
  load_bias_rows<D, BIAS, WI>(bv, a.bias, vq, a.V);
  if (BIAS) {
#pragma unroll
    for (int i = 0; i < WI; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) bv[i][e] = bv[i][e] * kscale;
  }
  // The one-hot term: column j's target row, as 16 i + e relative to vq, when
  // this lane holds it (rare), and its value dz/draw * factor there.
  int tl[WJ];
  bool any_t = false;
#pragma unroll
  for (int j = 0; j < WJ; ++j) {
    tl[j] = tgt[j] - vq;
    const bool here = tgt[j] >= 0 && tl[j] >= 0 && tl[j] < 16 * WI && (tl[j] & 15) < 4;
    if (!here) tl[j] = -1;
    any_t |= here;
  }
  float onehot[WJ];
#pragma unroll
  for (int j = 0; j < WJ; ++j) onehot[j] = 0.f;
  if (any_t) {
#pragma unroll
    for (int j = 0; j < WJ; ++j) {
      float xr = 0.f;
#pragma unroll
      for (int i = 0; i < WI; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (16 * i + e == tl[j]) xr = BIAS ? fmaf(acc[i][j][e], kscale, bv[i][e]) : acc[i][j][e] * kscale;
      float cf = 1.f;
      if (CAP) {
        const float qc = tanh_of_exp2_arg(xr);  // z / cap
        cf = fmaf(-qc, qc, 1.f);
      }
      if (tl[j] >= 0) onehot[j] = cf * (coef[j] * a.keep);
    }
  }
  // G = coef (pscale exp2(z log2e - lse log2e) - eps/V) [* (1 - (z/cap)^2)]:
  // FMAs around the exp, the per-column factors folded ahead (a dead column
  // has lse = +inf and coef = 0: exp2(-inf) = 0 and both factors 0).
  float ll[WJ], pc[WJ], ec[WJ];
#pragma unroll
  for (int j = 0; j < WJ; ++j) {
    ll[j] = lse[j] * LOG2E;
    pc[j] = pscale[j] * coef[j];
    ec[j] = a.eps_v * coef[j];
  }
  if constexpr (CAP) {
    // z = cap th; dz/dy = s (1 - th^2).  Two passes over the tile, each
    // element's th kept in its accumulator in between: the elements of a
    // pass are independent, so their exp2 / reciprocal latencies overlap
    // (done per element in one go, the chain ran one element at a time).
    const float cl = a.cap * LOG2E;
#pragma unroll
    for (int i = 0; i < WI; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < WJ; ++j)
          acc[i][j][e] = tanh_of_exp2_arg(BIAS ? fmaf(acc[i][j][e], kscale, bv[i][e]) : acc[i][j][e] * kscale);
#pragma unroll
    for (int i = 0; i < WI; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < WJ; ++j) {
          const float th = acc[i][j][e];
          acc[i][j][e] = fmaf(fast_exp2(fmaf(th, cl, -ll[j])), pc[j], -ec[j]) * fmaf(-th, th, 1.f);
        }
  } else if constexpr (BIAS) {
#pragma unroll
    for (int i = 0; i < WI; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < WJ; ++j) {
          const float z = fmaf(acc[i][j][e], kscale, bv[i][e]);
          acc[i][j][e] = fmaf(fast_exp2(fmaf(z, LOG2E, -ll[j])), pc[j], -ec[j]);
        }
  } else {
    const float sl = a.s * LOG2E;
#pragma unroll
    for (int i = 0; i < WI; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < WJ; ++j) acc[i][j][e] = fmaf(fast_exp2(fmaf(acc[i][j][e], sl, -ll[j])), pc[j], -ec[j]);
  }
  if (any_t) {
#pragma unroll
    for (int j = 0; j < WJ; ++j)
#pragma unroll
      for (int i = 0; i < WI; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (16 * i + e == tl[j]) acc[i][j][e] = acc[i][j][e] - onehot[j];
  }
  // rows past V or past the chunk (only in a ragged last tile): G = 0
  const int vrem = (int)min<int64_t>(min<int64_t>(a.V, a.c0 + a.cv) - vq, 1 << 20);
  if (vrem < 16 * WI) {
#pragma unroll
    for (int i = 0; i < WI; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (16 * i + e >= vrem) {
#pragma unroll
          for (int j = 0; j < WJ; ++j) acc[i][j][e] = 0.f;
        }
  }

  const int vlq = vl0 + wm * 16 * WI + 4 * q;  // chunk-local row of acc[i][.][e]: vlq + 16 i + e
  // 16-bit types: the tile goes to LDS as [n][v] and leaves as G rows and,
  // read transposed, as G^T rows.
  if constexpr (EB == 2) {
    if (a.G || a.GT) {
#pragma unroll
      for (int j = 0; j < WJ; ++j)
#pragma unroll
        for (int i = 0; i < WI; ++i)
          tile16_put4<D>(wn * 16 * WJ + 16 * j + c16, wm * 16 * WI + 16 * i + 4 * q, acc[i][j][0], acc[i][j][1],
                         acc[i][j][2], acc[i][j][3]);
      __syncthreads();
      const int rows = (int)min<int64_t>(TILE, a.npad - n0), cols = min(TILE, a.cvpad - vl0);
      if (a.G) {
        uint16_t* gdst = reinterpret_cast<uint16_t*>(a.G) + n0 * a.g_ld + vl0;
        if (a.g_stream) tile16_store<W * 64, true>(gdst, a.g_ld, rows, cols, t);
        else tile16_store<W * 64>(gdst, a.g_ld, rows, cols, t);
      }
      if (a.GT) tile16_store_t(reinterpret_cast<uint16_t*>(a.GT) + (int64_t)vl0 * a.npad + n0, a.npad, rows, cols, t);
    }
  }
  // fp32: G[n][vl] (row pitch g_ld) and G^T[vl][n] (row pitch npad) directly.
  if constexpr (EB == 4) {
    if (a.G) {
      float* G = reinterpret_cast<float*>(a.G);
#pragma unroll
      for (int j = 0; j < WJ; ++j) {
        const int64_t n = n0 + wn * 16 * WJ + 16 * j + c16;
        if (n >= a.npad) continue;
#pragma unroll
        for (int i = 0; i < WI; ++i) {
          const int vl = vlq + 16 * i;
          if (vl < a.cvpad)
            *reinterpret_cast<float4*>(G + n * a.g_ld + vl) =
                make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
      }
    }
  }
  if (EB == 4 && a.GT) {
    T* GT = reinterpret_cast<T*>(a.GT);
#pragma unroll
    for (int i = 0; i < WI; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int vl = vlq + 16 * i + e;
        if (vl >= a.cvpad) continue;
#pragma unroll
        for (int j = 0; j < WJ; ++j) {
          const int64_t n = n0 + wn * 16 * WJ + 16 * j + c16;
          if (n < a.npad) GT[(int64_t)vl * a.npad + n] = from_f32<D>(acc[i][j][e]);
        }
      }
  }
  // grad_bias partials: sum over this wave's 16*WJ tokens, per vocabulary id.
  if (a.dbpart) {
#pragma unroll
    for (int i = 0; i < WI; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float sb = acc[i][0][e];
#pragma unroll
        for (int j = 1; j < WJ; ++j) sb = sb + acc[i][j][e];
        sb = row_sum16(sb);
        const int v = vq + 16 * i + e;
        const int vl = v - (int)a.c0;
        if (c16 == 0 && v < a.V && vl < a.cv) a.dbpart[(int64_t)(Gemm<W>::GN * tt + wn) * a.V + v] = sb;
      }
  }
}

template <int D, bool BIAS, bool CAP, int W>
__global__ __launch_bounds__(W * 64) void bwd_g_kernel(GArgs a) {
  g_tile<D, BIAS, CAP, W, true>(a, blockIdx.x, gridDim.x);
}

// ------------------------------------------------------------------ backward contractions

template <int D>
__device__ __forceinline__ void store4(typename Elem<D>::T* p, float x0, float x1, float x2, float x3) {
  if constexpr (Elem<D>::bytes == 2) {
    typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
    u16x4 v;
    v[0] = __builtin_bit_cast(uint16_t, from_f32<D>(x0));
    v[1] = __builtin_bit_cast(uint16_t, from_f32<D>(x1));
    v[2] = __builtin_bit_cast(uint16_t, from_f32<D>(x2));
    v[3] = __builtin_bit_cast(uint16_t, from_f32<D>(x3));
    *reinterpret_cast<u16x4*>(p) = v;
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(x0, x1, x2, x3);
  }
}

// Both contractions put H on the MFMA row axis, so that a lane's four
// accumulator rows are four consecutive hidden indices of one output row.
//
// grad_hidden[n][h] (+)= scale * sum_v G[n][v] W[v][h] over one vocabulary
// chunk: A = W_c^T (h rows), B = G (n rows), K = the chunk.  The fp32
// accumulator is read and written 16 bytes per lane.
// Workgroup `bid` of a grid of `nblocks` (the tile order of grouped_tile), K
// split `ks`.
template <int D, int W, bool BK>
__device__ __forceinline__ void dh_tile(const DhArgs& a, int bid, int nblocks, int ks) {
  typedef typename Elem<D>::T T;
  constexpr int EB = Elem<D>::bytes, WI = Gemm<W>::WI, WJ = Gemm<W>::WJ;
  const TileAB ti = grouped_tile<kDhGA, kDhGB, kDhXcd>(bid, nblocks, a.n_h_tiles, a.n_tok_tiles);
  if (!ti.valid) return;
  const int ht = ti.a, tt = ti.b;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = Gemm<W>::wm(wave), wn = Gemm<W>::wn(wave), c16 = lane & 15, q = lane >> 4;
  const int64_t n0 = (int64_t)tt * TILE, h0 = (int64_t)ht * TILE;
  const int64_t kb = (int64_t)a.ld * EB;
  // split ks takes ids [k0, k0 + kn) of the chunk into its own accumulator
  const int k0 = ks * a.kpart, kn = min(a.kpart, a.kdim - k0);
  // The chunks' contributions accumulate unscaled; the running sum is read
  // into the accumulators before the K loop (its loads overlap the first
  // stages' copies instead of following the last MFMA), and the scale is
  // applied once, when grad_hidden is written.
  float* accbuf = a.acc + (int64_t)ks * a.acc_stride;
  f32x4_t acc[WI][WJ];
  if constexpr (BK) {
    // Tokens on the MFMA row axis (A = G), hidden on the column axis (B = the
    // chunk's weight rows, K-major): acc[i][j][e] is token nr + 16 i + e,
    // hidden hc + 16 j.  The running sum moves one float per lane, 64
    // contiguous bytes per quarter-wave.
    // The running sum is private to these kernels and kept in their own tile
    // layout: block (i, j) of thread t of tile (tt, ht) is the float4 at
    // ((tt * n_h_tiles + ht) * WI * WJ + i * WJ + j) * 512 + t, so each wave
    // moves 1 KB per instruction.  Tiles past N or H hold entries that are
    // never written out.
    float4* tp = reinterpret_cast<float4*>(accbuf) + ((int64_t)(tt * a.n_h_tiles + ht) * (WI * WJ)) * (W * 64) + t;
#pragma unroll
    for (int i = 0; i < WI; ++i)
#pragma unroll
      for (int j = 0; j < WJ; ++j) {
        if (a.first) {
          acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        } else if (a.acc_stream) {
          acc[i][j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(tp + (i * WJ + j) * (W * 64)));
        } else {
          const float4 o = tp[(i * WJ + j) * (W * 64)];
          acc[i][j] = f32x4_t{o.x, o.y, o.z, o.w};
        }
      }
    // K ids past the weight's last row (padding of the last chunk, whose G
    // columns are zero) add nothing: a split that holds only those is skipped
    const int64_t wr = min<int64_t>(kn, a.wrows - k0);
    if (kn > 0 && wr > 0) {
      const int64_t hb = a.H * EB;
      Panel A{a.G + n0 * kb + (int64_t)k0 * EB, kb, (int)min<int64_t>(TILE, a.N - n0), (int64_t)kn * EB};
      Panel B{a.Wk + (int64_t)k0 * hb + h0 * EB, hb, (int)wr, min<int64_t>(TILE, a.H - h0) * EB};
      gemm_tile_kmajor_b<D, W, false>(acc, A, B);
    }
    if (a.last && a.ksplit == 1) {
      // grad_hidden in the dtype through the LDS tile ([h][n] in, read
      // transposed into whole 16-byte pieces of grad_hidden rows); as fp32
      // straight from the accumulators, four tokens of one hidden column a
      // lane (a quarter-wave covers 64 contiguous bytes of each row)
      const float scale = a.scale[0];
      if (a.out_f32) {
        float* out = reinterpret_cast<float*>(a.out);
        const int nr = wm * 16 * WI + 4 * q, hc = wn * 16 * WJ + c16;
#pragma unroll
        for (int j = 0; j < WJ; ++j) {
          const int64_t h = h0 + hc + 16 * j;
          if (h >= a.H) continue;
#pragma unroll
          for (int i = 0; i < WI; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int64_t n = n0 + nr + 16 * i + e;
              if (n < a.N) out[n * a.H + h] = acc[i][j][e] * scale;
            }
        }
      } else if constexpr (EB == 2) {
#pragma unroll
        for (int i = 0; i < WI; ++i)
#pragma unroll
          for (int j = 0; j < WJ; ++j)
            tile16_put4<D>(wn * 16 * WJ + 16 * j + c16, wm * 16 * WI + 16 * i + 4 * q, acc[i][j][0] * scale,
                           acc[i][j][1] * scale, acc[i][j][2] * scale, acc[i][j][3] * scale);
        __syncthreads();
        tile16_store_t(reinterpret_cast<uint16_t*>(a.out) + n0 * a.H + h0, a.H, (int)min<int64_t>(TILE, a.H - h0),
                       (int)min<int64_t>(TILE, a.N - n0), t);
      }
    } else if (a.acc_stream) {
#pragma unroll
      for (int i = 0; i < WI; ++i)
#pragma unroll
        for (int j = 0; j < WJ; ++j)
          __builtin_nontemporal_store(acc[i][j], reinterpret_cast<f32x4_t*>(tp + (i * WJ + j) * (W * 64)));
    } else {
#pragma unroll
      for (int i = 0; i < WI; ++i)
#pragma unroll
        for (int j = 0; j < WJ; ++j)
          tp[(i * WJ + j) * (W * 64)] = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < WJ; ++j) {
    const int64_t n = n0 + wn * 16 * WJ + 16 * j + c16;
#pragma unroll
    for (int i = 0; i < WI; ++i) {
      const int64_t h = h0 + wm * 16 * WI + 16 * i + 4 * q;  // H % 4 == 0: all four in range
      acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (!a.first && n < a.N && h < a.H) {
        const float4 o = *reinterpret_cast<const float4*>(accbuf + n * a.H + h);
        acc[i][j] = f32x4_t{o.x, o.y, o.z, o.w};
      }
    }
  }
  if (kn > 0) {  // a split past a short last chunk adds nothing
    Panel A{a.WcT + h0 * kb + (int64_t)k0 * EB, kb, (int)min<int64_t>(TILE, a.H - h0), (int64_t)kn * EB};
    Panel B{a.G + n0 * kb + (int64_t)k0 * EB, kb, (int)min<int64_t>(TILE, a.N - n0), (int64_t)kn * EB};
    CopyPlan<W> cp;
    gemm_prefetch<W>(cp, A, B);
    NoSide none;
    gemm_run<D, W, NoSide, false>(acc, cp, A, none);
  }
  const bool finish = a.last && a.ksplit == 1;  // else a separate pass sums the splits
  const float scale = a.scale[0];
  T* out = reinterpret_cast<T*>(a.out);
#pragma unroll
  for (int j = 0; j < WJ; ++j) {
    const int64_t n = n0 + wn * 16 * WJ + 16 * j + c16;
    if (n >= a.N) continue;
#pragma unroll
    for (int i = 0; i < WI; ++i) {
      const int64_t h = h0 + wm * 16 * WI + 16 * i + 4 * q;
      if (h >= a.H) continue;
      const int64_t idx = n * a.H + h;
      if (finish && a.out_f32)
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + idx) = make_float4(
            acc[i][j][0] * scale, acc[i][j][1] * scale, acc[i][j][2] * scale, acc[i][j][3] * scale);
      else if (finish)
        store4<D>(out + idx, acc[i][j][0] * scale, acc[i][j][1] * scale, acc[i][j][2] * scale,
                  acc[i][j][3] * scale);
      else
        *reinterpret_cast<float4*>(accbuf + idx) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
    }
  }
}

template <int D, int W, bool BK>
__global__ __launch_bounds__(W * 64) void bwd_dh_kernel(DhArgs a) {
  dh_tile<D, W, BK>(a, blockIdx.x, gridDim.x, blockIdx.y);
}

// grad_hidden = scale * (sum over s = 0, 1, ... of the split accumulators,
// in that order), four elements per thread.
template <int D>
__global__ __launch_bounds__(256) void bwd_dh_final_kernel(DhFinalArgs a) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= a.count) return;
  if (a.bk) {
    // tile layout of the K-major grad_hidden kernel (8 waves, 8 x 4 blocks a
    // wave): float4 f = ((tile * 32 + blk) * 512 + t) holds tokens
    // n0 + wm 128 + 16 (blk / 4) + 4 q + [0, 4) of hidden h0 + wn 64 + 16 (blk % 4) + (t & 15)
    const int64_t f = i / 4;
    const int t = (int)(f % 512), blk = (int)((f / 512) % 32);
    const int64_t tile = f / (512 * 32);
    const int wave = t >> 6, lane = t & 63;
    const int64_t n = (tile / a.n_h_tiles) * TILE + (wave / 4) * 128 + 16 * (blk / 4) + 4 * (lane >> 4);
    const int64_t h = (tile % a.n_h_tiles) * TILE + (wave % 4) * 64 + 16 * (blk % 4) + (lane & 15);
    if (h >= a.H) return;
    float4 v = *reinterpret_cast<const float4*>(a.acc + i);
    for (int s = 1; s < a.ksplit; ++s) {
      const float4 o = *reinterpret_cast<const float4*>(a.acc + (int64_t)s * a.acc_stride + i);
      v.x = v.x + o.x;
      v.y = v.y + o.y;
      v.z = v.z + o.z;
      v.w = v.w + o.w;
    }
    const float sc = a.scale[0];
    typename Elem<D>::T* out = reinterpret_cast<typename Elem<D>::T*>(a.out);
    float* out32 = reinterpret_cast<float*>(a.out);
    const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (n + e < a.N) {
        if (a.out_f32) out32[(n + e) * a.H + h] = x[e] * sc;
        else out[(n + e) * a.H + h] = from_f32<D>(x[e] * sc);
      }
    return;
  }
  float4 v = *reinterpret_cast<const float4*>(a.acc + i);
  for (int s = 1; s < a.ksplit; ++s) {
    const float4 o = *reinterpret_cast<const float4*>(a.acc + (int64_t)s * a.acc_stride + i);
    v.x = v.x + o.x;
    v.y = v.y + o.y;
    v.z = v.z + o.z;
    v.w = v.w + o.w;
  }
  const float sc = a.scale[0];
  if (a.out_f32)
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + i) = make_float4(v.x * sc, v.y * sc, v.z * sc, v.w * sc);
  else
    store4<D>(reinterpret_cast<typename Elem<D>::T*>(a.out) + i, v.x * sc, v.y * sc, v.z * sc, v.w * sc);
}

// grad_weight[v][h] = scale * sum_n G[n][v] H[n][h] for one vocabulary chunk:
// A = H^T (h rows), B = G^T (v rows), K = tokens; with BK (16-bit types) B
// is G itself, read K-major (token rows of the chunk's columns, transposed in
// the fragment reads), so the recompute kernel writes no G^T.  16-bit results go through
// the LDS tile and leave as whole 512-byte row pieces; fp32 results (fp32
// inputs, or out_f32) are stored straight from the accumulators, each
// quarter-wave writing 64 contiguous bytes of one row.
template <int D, int W, bool BK>
__device__ __forceinline__ void dw_tile(const DwArgs& a, int bid, int nblocks) {
  constexpr int EB = Elem<D>::bytes, WI = Gemm<W>::WI, WJ = Gemm<W>::WJ;
  const TileAB ti = grouped_tile<kDwGA, kDwGB, kDwXcd>(bid, nblocks, a.n_h_tiles, a.n_voc_tiles);
  if (!ti.valid) return;
  const int ht = ti.a, vt = ti.b;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = Gemm<W>::wm(wave), wn = Gemm<W>::wn(wave), c16 = lane & 15, q = lane >> 4;
  const int64_t v0 = (int64_t)vt * TILE, h0 = (int64_t)ht * TILE;
  const int64_t kb = (int64_t)a.npad * EB;
  Panel A{a.HT + h0 * kb, kb, (int)min<int64_t>(TILE, a.H - h0), kb};
  f32x4_t acc[WI][WJ];
  if constexpr (BK) {
    // columns v0 .. v0 + 255 of G's npad token rows (pitch gld elements).  The
    // panel's range ends at column cv of the last row, inside G; columns past
    // the chunk in earlier rows read the next ones' data and feed only
    // outputs that are never stored.
    const int64_t cb = (int64_t)min(TILE, a.cv - (int)v0) * EB;
    gemm_tile_kmajor_b<D, W>(acc, A, Panel{a.GT + v0 * EB, (int64_t)a.gld * EB, a.npad, cb});
  } else {
    gemm_nt_tile<D, W>(acc, A, Panel{a.GT + v0 * kb, kb, (int)min<int64_t>(TILE, a.cv - v0), kb});
  }
  const float scale = a.scale[0];
  if constexpr (EB == 2) {
    if (!a.out_f32) {
#pragma unroll
      for (int j = 0; j < WJ; ++j)
#pragma unroll
        for (int i = 0; i < WI; ++i)
          tile16_put4<D>(wn * 16 * WJ + 16 * j + c16, wm * 16 * WI + 16 * i + 4 * q, acc[i][j][0] * scale,
                         acc[i][j][1] * scale, acc[i][j][2] * scale, acc[i][j][3] * scale);
      __syncthreads();
      tile16_store<W * 64>(reinterpret_cast<uint16_t*>(a.out) + v0 * a.H + h0, a.H,
                           (int)min<int64_t>(TILE, a.cv - v0), (int)min<int64_t>(TILE, a.H - h0), t);
      return;
    }
  }
  float* out = reinterpret_cast<float*>(a.out);
#pragma unroll
  for (int j = 0; j < WJ; ++j) {
    const int64_t v = v0 + wn * 16 * WJ + 16 * j + c16;
    if (v >= a.cv) continue;
#pragma unroll
    for (int i = 0; i < WI; ++i) {
      const int64_t h = h0 + wm * 16 * WI + 16 * i + 4 * q;
      if (h < a.H)
        *reinterpret_cast<float4*>(out + v * a.H + h) = make_float4(
            acc[i][j][0] * scale, acc[i][j][1] * scale, acc[i][j][2] * scale, acc[i][j][3] * scale);
    }
  }
}

template <int D, int W, bool BK>
__global__ __launch_bounds__(W * 64) void bwd_dw_kernel(DwArgs a) {
  dw_tile<D, W, BK>(a, blockIdx.x, gridDim.x);
}

// One backward step of the 16-bit K-major path in one launch: grad_hidden of
// a finished chunk (or pair of chunks), grad_weight of the last finished
// chunk and the recompute of the next chunk into the other G buffer.  The
// three grids are laid end to end (grad_hidden's, the longest workgroups,
// first); each part's size is a multiple of 8, so a workgroup's XCD
// (block id mod 8) is the same as in a launch of its own.  The parts touch
// disjoint outputs and read only G written by an earlier launch.
template <int D, bool BIAS, bool CAP>
__global__ __launch_bounds__(kContractWaves * 64) void bwd_step_kernel(StepArgs a) {
  static_assert(kContractWaves == kRecomputeWaves, "one workgroup shape for every part");
  int b = blockIdx.x;
  if (b < a.nb_dh) {
    dh_tile<D, kContractWaves, true>(a.dh, b % a.dh_grid, a.dh_grid, b / a.dh_grid);
    return;
  }
  b -= a.nb_dh;
  if (b < a.nb_dw) {
    dw_tile<D, kContractWaves, true>(a.dw, b, a.nb_dw);
    return;
  }
  b -= a.nb_dw;
  g_tile<D, BIAS, CAP, kRecomputeWaves, false>(a.g, b, a.nb_g);
}

template <int D>
__global__ __launch_bounds__(256) void bwd_db_kernel(DbArgs a) {
  typedef typename Elem<D>::T T;
  const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (v >= a.V) return;
  float s = 0.f;
  for (int p = 0; p < a.n_parts; ++p) s = s + a.dbpart[(int64_t)p * a.V + v];
  if (a.out_f32) reinterpret_cast<float*>(a.out)[v] = s * a.scale[0];
  else reinterpret_cast<T*>(a.out)[v] = from_f32<D>(s * a.scale[0]);
}

// ------------------------------------------------------------------ strided token layouts

// One workgroup per token row: 16-byte pieces of the row (row_bytes is a
// multiple of 16, and so are both source strides).
__global__ __launch_bounds__(256) void gather_rows_kernel(GatherRowsArgs a) {
  const int64_t n = blockIdx.x, s = n / a.T, t = n - s * a.T;
  const char* src = a.src + s * a.seq_bytes + t * a.row_pitch;
  char* dst = a.dst + n * a.row_bytes;
  for (int64_t c = (int64_t)threadIdx.x * 16; c < a.row_bytes; c += 256 * 16)
    *reinterpret_cast<uint4*>(dst + c) = *reinterpret_cast<const uint4*>(src + c);
}

__global__ __launch_bounds__(256) void gather_targets_kernel(GatherTargetsArgs a) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= a.N) return;
  const int64_t s = n / a.T, t = n - s * a.T;
  int64_t tv = a.src[s * a.seq_stride + t * a.stride];
  if (a.shard) {
    const int64_t local = tv - a.voff;
    tv = tv == a.ignore_index              ? kShardIgnored
         : (local >= 0 && local < a.vshard) ? local
         : (tv >= 0 && tv < a.vtotal)       ? kShardForeign
                                            : kShardBad;
  }
  a.dst[n] = tv;
}

// ------------------------------------------------------------------ launchers

static inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

template <int D>
static hipError_t fwd_tiles_dispatch(bool metrics, bool bias, bool cap, const FwdArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)grouped_grid<kFwdXcd>(a.n_tok_tiles, a.n_groups)), block(kFwdWaves * 64);
#define FLCE_FWD(M, B, C)                                                                \
  if (metrics == M && bias == B && cap == C) {                                           \
    hipLaunchKernelGGL((fwd_tiles_kernel<D, M, B, C, kFwdWaves>), grid, block, 0, st, a); \
    return hipGetLastError();                                                     \
  }
  FLCE_FWD(false, false, false) FLCE_FWD(false, false, true) FLCE_FWD(false, true, false)
  FLCE_FWD(false, true, true) FLCE_FWD(true, false, false) FLCE_FWD(true, false, true)
  FLCE_FWD(true, true, false) FLCE_FWD(true, true, true)
#undef FLCE_FWD
  return hipErrorInvalidValue;
}

hipError_t launch_forward_tiles(int dtype, bool metrics, bool bias, bool cap, const FwdArgs& a,
                                hipStream_t st) {
  switch (dtype) {
    case DT_F32: return fwd_tiles_dispatch<DT_F32>(metrics, bias, cap, a, st);
    case DT_F16: return fwd_tiles_dispatch<DT_F16>(metrics, bias, cap, a, st);
    case DT_BF16: return fwd_tiles_dispatch<DT_BF16>(metrics, bias, cap, a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_forward_combine(bool metrics, const CombineArgs& a, hipStream_t st) {
  const dim3 grid(blocks_for(a.N, 32)), block(256);
  if (metrics) hipLaunchKernelGGL(fwd_combine_kernel<true>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(fwd_combine_kernel<false>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_forward_reduce(bool metrics, const ReduceArgs& a, hipStream_t st) {
  if (metrics) hipLaunchKernelGGL(fwd_reduce_kernel<true>, dim3(1), dim3(1024), 0, st, a);
  else hipLaunchKernelGGL(fwd_reduce_kernel<false>, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_shard_combine(const ShardCombineArgs& a, hipStream_t st) {
  if (a.N <= 0) return hipSuccess;
  hipLaunchKernelGGL(shard_combine_kernel, dim3(blocks_for(a.N, 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_backward_prep(const PrepArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(bwd_prep_kernel, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_transpose(int dtype, const TransposeArgs& a, hipStream_t st) {
  const int tc = dtype == DT_F32 ? 64 : 128;
  const dim3 grid(blocks_for(a.rpad, 64), blocks_for(a.cols, tc)), block(256);
  if (dtype == DT_F32) hipLaunchKernelGGL(transpose_kernel<4>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(transpose_kernel<2>, grid, block, 0, st, a);
  return hipGetLastError();
}

template <int D>
static hipError_t g_dispatch(bool bias, bool cap, const GArgs& a, hipStream_t st) {
  constexpr int W = kRecomputeWaves;
  const dim3 grid((unsigned)grouped_grid<kRecXcd>(a.n_tok_tiles, a.n_voc_tiles)), block(W * 64);
  if (!bias && !cap) hipLaunchKernelGGL((bwd_g_kernel<D, false, false, W>), grid, block, 0, st, a);
  else if (!bias && cap) hipLaunchKernelGGL((bwd_g_kernel<D, false, true, W>), grid, block, 0, st, a);
  else if (bias && !cap) hipLaunchKernelGGL((bwd_g_kernel<D, true, false, W>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((bwd_g_kernel<D, true, true, W>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_backward_g(int dtype, bool bias, bool cap, const GArgs& a, hipStream_t st) {
  switch (dtype) {
    case DT_F32: return g_dispatch<DT_F32>(bias, cap, a, st);
    case DT_F16: return g_dispatch<DT_F16>(bias, cap, a, st);
    case DT_BF16: return g_dispatch<DT_BF16>(bias, cap, a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_backward_dh(int dtype, const DhArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)grouped_grid<kDhXcd>(a.n_h_tiles, a.n_tok_tiles), (unsigned)a.ksplit),
      block(kContractWaves * 64);
  switch (dtype) {
    case DT_F32: hipLaunchKernelGGL((bwd_dh_kernel<DT_F32, kContractWaves, false>), grid, block, 0, st, a); break;
    case DT_F16:
      if (a.bk) hipLaunchKernelGGL((bwd_dh_kernel<DT_F16, kContractWaves, true>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((bwd_dh_kernel<DT_F16, kContractWaves, false>), grid, block, 0, st, a);
      break;
    case DT_BF16:
      if (a.bk) hipLaunchKernelGGL((bwd_dh_kernel<DT_BF16, kContractWaves, true>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((bwd_dh_kernel<DT_BF16, kContractWaves, false>), grid, block, 0, st, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_backward_dh_final(int dtype, const DhFinalArgs& a, hipStream_t st) {
  if (a.count <= 0) return hipSuccess;
  const dim3 grid(blocks_for(a.count / 4, 256)), block(256);
  switch (dtype) {
    case DT_F32: hipLaunchKernelGGL(bwd_dh_final_kernel<DT_F32>, grid, block, 0, st, a); break;
    case DT_F16: hipLaunchKernelGGL(bwd_dh_final_kernel<DT_F16>, grid, block, 0, st, a); break;
    case DT_BF16: hipLaunchKernelGGL(bwd_dh_final_kernel<DT_BF16>, grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_backward_dw(int dtype, const DwArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)grouped_grid<kDwXcd>(a.n_h_tiles, a.n_voc_tiles)), block(kContractWaves * 64);
  switch (dtype) {
    case DT_F32: hipLaunchKernelGGL((bwd_dw_kernel<DT_F32, kContractWaves, false>), grid, block, 0, st, a); break;
    case DT_F16:
      if (a.gk) hipLaunchKernelGGL((bwd_dw_kernel<DT_F16, kContractWaves, true>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((bwd_dw_kernel<DT_F16, kContractWaves, false>), grid, block, 0, st, a);
      break;
    case DT_BF16:
      if (a.gk) hipLaunchKernelGGL((bwd_dw_kernel<DT_BF16, kContractWaves, true>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((bwd_dw_kernel<DT_BF16, kContractWaves, false>), grid, block, 0, st, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
static hipError_t step_dispatch(bool bias, bool cap, const StepArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.nb_dh + a.nb_dw + a.nb_g)), block(kContractWaves * 64);
  if (!bias && !cap) hipLaunchKernelGGL((bwd_step_kernel<D, false, false>), grid, block, 0, st, a);
  else if (!bias && cap) hipLaunchKernelGGL((bwd_step_kernel<D, false, true>), grid, block, 0, st, a);
  else if (bias && !cap) hipLaunchKernelGGL((bwd_step_kernel<D, true, false>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((bwd_step_kernel<D, true, true>), grid, block, 0, st, a);
  return hipGetLastError();
}

int backward_g_grid(int n_tok_tiles, int n_voc_tiles) { return grouped_grid<kRecXcd>(n_tok_tiles, n_voc_tiles); }
int backward_dh_grid(int n_h_tiles, int n_tok_tiles) { return grouped_grid<kDhXcd>(n_h_tiles, n_tok_tiles); }
int backward_dw_grid(int n_h_tiles, int n_voc_tiles) { return grouped_grid<kDwXcd>(n_h_tiles, n_voc_tiles); }

hipError_t launch_backward_step(int dtype, bool bias, bool cap, const StepArgs& a, hipStream_t st) {
  if (a.nb_dh + a.nb_dw + a.nb_g == 0) return hipSuccess;
  switch (dtype) {
    case DT_F16: return step_dispatch<DT_F16>(bias, cap, a, st);
    case DT_BF16: return step_dispatch<DT_BF16>(bias, cap, a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_backward_db(int dtype, const DbArgs& a, hipStream_t st) {
  const dim3 grid(blocks_for(a.V, 256)), block(256);
  switch (dtype) {
    case DT_F32: hipLaunchKernelGGL(bwd_db_kernel<DT_F32>, grid, block, 0, st, a); break;
    case DT_F16: hipLaunchKernelGGL(bwd_db_kernel<DT_F16>, grid, block, 0, st, a); break;
    case DT_BF16: hipLaunchKernelGGL(bwd_db_kernel<DT_BF16>, grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* dst, size_t bytes, hipStream_t st) {
  if (bytes == 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<int64_t>(4096, ((int64_t)bytes + 255) / 256);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0, st, reinterpret_cast<uint8_t*>(dst),
                     (int64_t)bytes);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const GatherRowsArgs& a, hipStream_t st) {
  if (a.N <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)a.N), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gather_targets(const GatherTargetsArgs& a, hipStream_t st) {
  if (a.N <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_targets_kernel, dim3(blocks_for(a.N, 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ fixed scratch

// The workspace of the allocation-free forward entry point: one array per
// device, of kScratchBytes, alive until the process ends.  Host code never
// passes this name to a kernel (on the host it is only a stand-in for the
// symbol): it takes the device address hipGetSymbolAddress gives, once per
// device, with that device current.  Every call on a device shares the
// array, so calls that overlap on one device race.
static __device__ __align__(256) char scratch[kScratchBytes];

hipError_t scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace flce
