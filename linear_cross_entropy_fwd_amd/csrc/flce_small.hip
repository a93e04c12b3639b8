// flce_small.hip -- fp32 problems of at most 256 tokens (a vocabulary of at
// most 8192 ids and a hidden size of at most 1024): the same loss and
// gradients as the tiled path (trl-lib "fused-linear-ce" card, "Algorithm"
// and "Metrics for free"), computed with plain fp32 FMAs, because at these
// sizes the tiled path's 256 x 256 fp32 MFMA tiles leave all but a few CUs
// idle and the time goes to latency.
//
//   small_fwd_kernel  one workgroup per token: the row's logits into LDS,
//                     then max, sum of exp, target logit, first-index argmax,
//                     entropy sum and sum of z, and the row's loss as the
//                     split combine of the tiled path forms it;
//   small_dh_kernel   one workgroup per token: the row's logits again, G for
//                     the row, grad_hidden row = G . weight;
//   small_dw_kernel   one workgroup per 8 vocabulary rows, one thread per
//                     token: G for those columns, grad_weight rows = G^T .
//                     hidden and grad_bias.
// Every sum runs in a fixed order, so results are deterministic; the
// transform and the gradient factors are the tiled path's formulas.
#include <math.h>

#include "flce_device.h"
#include "flce_plan.h"

namespace flce {

namespace {

constexpr int kT = 256;  // threads per workgroup

__device__ __forceinline__ float tanh_def(float x) {
  // tanh x = sign(x) (1 - 2 / (e^{2|x|} + 1)) with the hardware exp2 and
  // reciprocal (the tiled path's form)
  const float t = __builtin_amdgcn_exp2f(fabsf(x) * (2.f * LOG2E));
  return copysignf(fmaf(-2.f, __builtin_amdgcn_rcpf(t + 1.f), 1.f), x);
}

// z = cap tanh(s (raw + b) / cap) or s (raw + b): bias, then scale, then cap.
__device__ __forceinline__ float transform(const SmallArgs& a, float raw, int64_t j) {
  float y = raw;
  if (a.bias) y = y + reinterpret_cast<const float*>(a.bias)[j];
  return a.has_cap ? a.cap * tanh_def(y * (a.s * a.inv_cap)) : a.s * y;
}

// raw logit of hidden row h (in LDS) against weight row w: four running
// sums over k = 0, 1, 2, 3 mod 4 (independent FMA chains), added in a fixed
// order at the end.
__device__ __forceinline__ float dot_row(const float* h, const float* w, int64_t H) {
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  for (int64_t k = 0; k < H; k += 4) {
    const float4 wv = *reinterpret_cast<const float4*>(w + k);
    a0 = fmaf(h[k], wv.x, a0);
    a1 = fmaf(h[k + 1], wv.y, a1);
    a2 = fmaf(h[k + 2], wv.z, a2);
    a3 = fmaf(h[k + 3], wv.w, a3);
  }
  return (a0 + a1) + (a2 + a3);
}

template <class Op>
__device__ __forceinline__ float block_reduce(float* red, float v, Op op) {
  const int t = threadIdx.x;
  red[t] = v;
  __syncthreads();
  for (int w = kT / 2; w > 0; w >>= 1) {
    if (t < w) red[t] = op(red[t], red[t + w]);
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

// The reduction's uniform gradient factor (times the logit scale): the
// tiled path's prep kernel, a fixed-order fp64 sum over the targets.
__device__ __forceinline__ float uniform_scale(const SmallArgs& a) {
  __shared__ float sc;
  if (threadIdx.x == 0) {
    float scale = 1.f;
    if (a.reduction != 2) {
      double den = 0.0;
      for (int64_t n = 0; n < a.N; ++n) {
        const int64_t tv = a.targets[n];
        if (tv == a.ignore_index) continue;
        if (!a.class_weight) den += 1.0;
        else if (tv >= 0 && tv < a.V) den += (double)a.class_weight[tv];
      }
      const float g = a.grad_loss ? a.grad_loss[0] : 1.f;
      if (a.reduction == 0) scale = den > 0.0 ? (float)((double)g / den) : 0.f;
      else scale = g;
    }
    sc = scale * a.s;
  }
  __syncthreads();
  return sc;
}

// Per-row factors of dL/dz_j = coef (pscale p_j - keep [j = t] - eps/V):
// coef = row weight times the per-row upstream gradient (NaN for an
// out-of-range target, 0 for an ignored row).
struct RowGrad {
  float lse, coef, pscale;
  int64_t t;  // -1 when the row is ignored or its target is out of range
};

__device__ __forceinline__ RowGrad row_grad(const SmallArgs& a, int64_t n) {
  RowGrad r{INFINITY, 0.f, 1.f, -1};
  const int64_t tv = a.targets[n];
  if (tv == a.ignore_index) return r;
  r.lse = a.lse[n];
  r.pscale = fmaf(a.zl2, r.lse, 1.f);
  if (tv < 0 || tv >= a.V) {
    r.coef = NAN;
    return r;
  }
  r.t = tv;
  r.coef = (a.reduction == 2 && a.grad_loss) ? a.grad_loss[n] : 1.f;
  if (a.class_weight) r.coef = r.coef * a.class_weight[tv];
  return r;
}

// G_j (before the uniform scale): dL/dz_j times dz/dy (1 - (z/cap)^2 with a cap).
__device__ __forceinline__ float g_of(const SmallArgs& a, const RowGrad& r, float z, int64_t j) {
  if (r.coef == 0.f) return 0.f;
  const float p = __builtin_amdgcn_exp2f(fmaf(z, LOG2E, -r.lse * LOG2E));
  float g = r.coef * (fmaf(r.pscale, p, -a.eps_v) - (j == r.t ? a.keep : 0.f));
  if (a.has_cap) {
    const float th = z * a.inv_cap;
    g = g * fmaf(-th, th, 1.f);
  }
  return g;
}

}  // namespace

template <bool METRICS>
__global__ __launch_bounds__(kT) void small_fwd_kernel(SmallArgs a) {
  __shared__ float hrow[kSmallMaxH];
  __shared__ float zr[kSmallMaxV];
  __shared__ float red[kT];
  __shared__ int redi[kT];
  const int t = threadIdx.x;
  const int64_t n = blockIdx.x, H = a.H, V = a.V;
  const float* h = reinterpret_cast<const float*>(a.hidden) + n * H;
  const float* W = reinterpret_cast<const float*>(a.weight);
  for (int64_t k = t; k < H; k += kT) hrow[k] = h[k];
  __syncthreads();
  float m = -INFINITY, zs = 0.f, av = -INFINITY;
  int ai = 0x7fffffff;
  for (int64_t j = t; j < V; j += kT) {
    const float z = transform(a, dot_row(hrow, W + j * H, H), j);
    zr[j] = z;
    m = fmaxf(m, z);
    zs = zs + z;
    if (z > av) {  // ids rise within a thread: strict > keeps the first
      av = z;
      ai = (int)j;
    }
  }
  m = block_reduce(red, m, [](float x, float y) { return fmaxf(x, y); });
  float s = 0.f, u = 0.f;
  for (int64_t j = t; j < V; j += kT) {
    const float d = zr[j] - m;
    const float e = __builtin_amdgcn_exp2f(d * LOG2E);
    s = s + e;
    if (METRICS) u = fmaf(e, d, u);
  }
  s = block_reduce(red, s, [](float x, float y) { return x + y; });
  if (METRICS) u = block_reduce(red, u, [](float x, float y) { return x + y; });
  if (a.eps > 0.f) zs = block_reduce(red, zs, [](float x, float y) { return x + y; });
  if (METRICS) {
    // first-index argmax over the block: larger value, then smaller id
    red[t] = av;
    redi[t] = ai;
    __syncthreads();
    for (int w = kT / 2; w > 0; w >>= 1) {
      if (t < w) {
        const float v2 = red[t + w];
        const int i2 = redi[t + w];
        if (v2 > red[t] || (v2 == red[t] && i2 < redi[t])) {
          red[t] = v2;
          redi[t] = i2;
        }
      }
      __syncthreads();
    }
    ai = redi[0];
  }
  if (t != 0) return;
  const int64_t tv = a.targets[n];
  const bool valid = tv != a.ignore_index;
  const bool bad = valid && (tv < 0 || tv >= V);
  const float logS = logf(s);
  const float lse = m + logS;
  float row = 0.f, rw = 0.f;
  if (valid) {
    if (bad) {
      row = NAN;
    } else {
      const float zt = zr[tv];
      rw = a.class_weight ? a.class_weight[tv] : 1.f;
      const float zsum = a.eps > 0.f ? zs : 0.f;  // the sum of z only enters with smoothing
      row = rw * ((lse - (1.f - a.eps) * zt) - (a.eps / (float)V) * zsum + a.z_loss * (lse * lse));
    }
  }
  if (a.row_w) a.row_w[n] = rw;
  if (a.lse_out) a.lse_out[n] = lse;
  if (a.loss_rows) a.loss_rows[n] = row;
  a.row_loss[n] = row;
  int flag = (valid ? 1 : 0) | (bad ? 4 : 0);
  if (METRICS) {
    if (a.predictions) a.predictions[n] = (int64_t)ai;
    if (valid && !bad && ai == tv) flag |= 2;
    a.row_ent[n] = valid ? logS - u / s : 0.f;
  }
  a.row_flag[n] = flag;
}

// grad_hidden row: thread t owns the float4 of columns 4 (t % C) .. +3
// (C = H / 4 threads per row) in group t / C, and group g sums the ids
// j = g, g + NG, ... (NG = 256 / C groups); the NG partial sums are then
// added in the order g = 0, 1, ...
__global__ __launch_bounds__(kT) void small_dh_kernel(SmallArgs a) {
  __shared__ float hrow[kSmallMaxH];
  __shared__ float gr[kSmallMaxV];
  __shared__ float4 part[kT];
  const int t = threadIdx.x;
  const int64_t n = blockIdx.x, H = a.H, V = a.V;
  const float scale = uniform_scale(a);
  const RowGrad r = row_grad(a, n);
  const float* h = reinterpret_cast<const float*>(a.hidden) + n * H;
  const float* W = reinterpret_cast<const float*>(a.weight);
  for (int64_t k = t; k < H; k += kT) hrow[k] = h[k];
  __syncthreads();
  for (int64_t j = t; j < V; j += kT) gr[j] = g_of(a, r, transform(a, dot_row(hrow, W + j * H, H), j), j);
  __syncthreads();
  const int C = (int)(H / 4), NG = kT / C;  // H <= 1024: C <= 256, NG >= 1
  const int c = t % C, grp = t / C;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (grp < NG) {
    for (int64_t j = grp; j < V; j += NG) {
      const float4 wv = *reinterpret_cast<const float4*>(W + j * H + 4 * c);
      const float gj = gr[j];
      acc.x = fmaf(gj, wv.x, acc.x);
      acc.y = fmaf(gj, wv.y, acc.y);
      acc.z = fmaf(gj, wv.z, acc.z);
      acc.w = fmaf(gj, wv.w, acc.w);
    }
  }
  part[t] = acc;
  __syncthreads();
  if (t < C) {
    float4 sum = part[t];
    for (int g2 = 1; g2 < NG; ++g2) {
      const float4 o = part[g2 * C + t];
      sum.x = sum.x + o.x;
      sum.y = sum.y + o.y;
      sum.z = sum.z + o.z;
      sum.w = sum.w + o.w;
    }
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.grad_hidden) + n * H + 4 * t) =
        make_float4(sum.x * scale, sum.y * scale, sum.z * scale, sum.w * scale);
  }
}

__global__ __launch_bounds__(kT) void small_dw_kernel(SmallArgs a) {
  constexpr int R = kSmallDwRows;
  __shared__ float wrows[R * kSmallMaxH];
  __shared__ float gc[R][kT];
  const int t = threadIdx.x;
  const int64_t j0 = (int64_t)blockIdx.x * R, H = a.H, V = a.V, N = a.N;
  const int rows = (int)min<int64_t>(R, V - j0);
  const float scale = uniform_scale(a);
  const float* W = reinterpret_cast<const float*>(a.weight);
  const float* Hd = reinterpret_cast<const float*>(a.hidden);
  for (int64_t i = t; i < (int64_t)rows * H; i += kT) wrows[i] = W[j0 * H + i];
  __syncthreads();
  // thread t: token t's G for these vocabulary rows (R independent dot
  // products, each with the four k-mod-4 running sums of dot_row)
  if (t < N) {
    const RowGrad r = row_grad(a, t);
    const float* h = Hd + (int64_t)t * H;
    float acc[R][4];
    for (int q = 0; q < R; ++q) acc[q][0] = acc[q][1] = acc[q][2] = acc[q][3] = 0.f;
    for (int64_t k = 0; k < H; k += 4) {
      const float4 hv = *reinterpret_cast<const float4*>(h + k);
#pragma unroll
      for (int q = 0; q < R; ++q) {
        const float* w = wrows + q * H + k;
        acc[q][0] = fmaf(hv.x, w[0], acc[q][0]);
        acc[q][1] = fmaf(hv.y, w[1], acc[q][1]);
        acc[q][2] = fmaf(hv.z, w[2], acc[q][2]);
        acc[q][3] = fmaf(hv.w, w[3], acc[q][3]);
      }
    }
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const float raw = (acc[q][0] + acc[q][1]) + (acc[q][2] + acc[q][3]);
      gc[q][t] = q < rows ? g_of(a, r, transform(a, raw, j0 + q), j0 + q) : 0.f;
    }
  }
  __syncthreads();
  if (a.grad_weight) {
    // thread t: the float4 of columns 4 (t % C) .. +3 for rows q = t / C, t / C + NQ, ...
    float* out = reinterpret_cast<float*>(a.grad_weight);
    const int C = (int)(H / 4), NQ = kT / C > R ? R : kT / C;
    const int c = t % C, q0 = t / C;
    for (int q = q0; q < rows && q0 < NQ; q += NQ) {
      float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int64_t i = 0; i < N; ++i) {
        const float4 hv = *reinterpret_cast<const float4*>(Hd + i * H + 4 * c);
        const float g = gc[q][i];
        s4.x = fmaf(g, hv.x, s4.x);
        s4.y = fmaf(g, hv.y, s4.y);
        s4.z = fmaf(g, hv.z, s4.z);
        s4.w = fmaf(g, hv.w, s4.w);
      }
      *reinterpret_cast<float4*>(out + (j0 + q) * H + 4 * c) =
          make_float4(s4.x * scale, s4.y * scale, s4.z * scale, s4.w * scale);
    }
  }
  if (a.grad_bias && t < rows) {
    float acc = 0.f;
    for (int64_t i = 0; i < N; ++i) acc = acc + gc[t][i];
    reinterpret_cast<float*>(a.grad_bias)[j0 + t] = acc * scale;
  }
}

hipError_t launch_small_forward(bool metrics, const SmallArgs& a, hipStream_t st) {
  if (a.N <= 0) return hipSuccess;
  if (metrics) hipLaunchKernelGGL(small_fwd_kernel<true>, dim3((unsigned)a.N), dim3(kT), 0, st, a);
  else hipLaunchKernelGGL(small_fwd_kernel<false>, dim3((unsigned)a.N), dim3(kT), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_small_backward(const SmallArgs& a, hipStream_t st) {
  if (a.N <= 0) return hipSuccess;
  if (a.grad_hidden) {
    hipLaunchKernelGGL(small_dh_kernel, dim3((unsigned)a.N), dim3(kT), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.grad_weight || a.grad_bias) {
    const unsigned grid = (unsigned)((a.V + kSmallDwRows - 1) / kSmallDwRows);
    hipLaunchKernelGGL(small_dw_kernel, dim3(grid), dim3(kT), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace flce
