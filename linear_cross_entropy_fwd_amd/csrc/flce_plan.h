// flce_plan.h -- host/device shared argument blocks and the launch plan.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace flce {

// Waves per workgroup of the GEMM-shaped kernels (each 256 x 256 output
// tile; 4 = one wave per SIMD with 128 x 128 per wave, 8 = two per SIMD with
// 128 x 64 per wave).
constexpr int kFwdWaves = 8;        // forward logit tiles
constexpr int kRecomputeWaves = 8;  // backward recompute (G; G^T on the fp32 path; grad_bias partials)
constexpr int kContractWaves = 8;   // grad_hidden and grad_weight contractions

// Tile orders (grouped_tile): GA x GB blocks, remapped per XCD or not
// (measured at 4096 x 4096 x 128256 bf16: the forward sweep is 3-4 % faster
// in dispatch order, the backward launches are fastest remapped).
constexpr int kFwdGA = 4, kFwdGB = 8;
constexpr bool kFwdXcd = false;
constexpr int kRecGA = 4, kRecGB = 8;
constexpr bool kRecXcd = true;
constexpr int kDhGA = 4, kDhGB = 8;
constexpr bool kDhXcd = true;
constexpr int kDwGA = 4, kDwGB = 8;
constexpr bool kDwXcd = true;

// Tile order of a GEMM-shaped grid over na x nb output tiles (a: the
// dimension whose operand panels are shared along b, and the reverse).  The
// tiles are numbered in blocks of up to GA x GB: rows of blocks GB tiles deep
// in b, GA-wide blocks along a within a row, a fastest inside a block; a
// block at the far edge of a or b is as wide as what is left, so the numbers
// 0 .. na nb - 1 are exactly the tiles.
//
// Workgroups run one per CU and are dealt round robin to the 8 XCDs
// (workgroup id mod 8), in order: when the next workgroup's XCD has no free
// CU, the ones queued behind it wait too, even for other XCDs.  Without XCD,
// workgroup bid takes tile number bid (grid na nb), and a block of 32 spreads
// over all XCDs, its panels meeting in the last-level cache.  With XCD, the
// grid is na nb rounded up to a multiple of 8 and each XCD is given one
// contiguous range of tile numbers, all of equal length (the last XCDs one
// shorter when na nb is not a multiple of 8: their last workgroup gets
// valid = false and must exit at once), so that a block's panels meet in one
// XCD's L2 and every XCD holds the same share of the work: an XCD with more
// of a launch's long workgroups than the others would hold back the
// dispatch of everything queued after them.
struct TileAB {
  int a, b;
  bool valid;
};

template <bool XCD>
__host__ __device__ inline int grouped_grid(int na, int nb) {
  return XCD ? (na * nb + 7) / 8 * 8 : na * nb;
}

template <int GA, int GB, bool XCD>
__host__ __device__ inline TileAB grouped_tile(int bid, int nblocks, int na, int nb) {
  TileAB r{0, 0, false};
  const int T = na * nb;
  int L = bid;
  if (XCD) {
    // nblocks = grouped_grid<true>: XCDs [full, 8) get q - 1 tiles, the rest q
    const int q = nblocks / 8, full = 8 - (nblocks - T);
    const int x = bid % 8, k = bid / 8;
    if (k >= (x < full ? q : q - 1)) return r;
    L = x * q - (x > full ? x - full : 0) + k;
  }
  if (L >= T) return r;
  const int gb = L / (na * GB), r0 = L - gb * (na * GB);
  const int wb = nb - gb * GB < GB ? nb - gb * GB : GB;
  const int ga = r0 / (GA * wb), r1 = r0 - ga * (GA * wb);
  const int wa = na - ga * GA < GA ? na - ga * GA : GA;
  r.a = ga * GA + r1 % wa;
  r.b = gb * GB + r1 / wa;
  r.valid = true;
  return r;
}
// grad_bias partial sums per 256-token tile: one per wave column (64 tokens
// each with 8 waves, 128 with 4).
constexpr int kBiasParts = kRecomputeWaves == 8 ? 4 : 2;

// Fields of a forward partial record, part[field][split][row] (floats): m
// and S; then U, the argmax value and the argmax id with metrics; then the
// sum of z with label smoothing.
__host__ __device__ inline int part_fields(bool metrics, bool zsum) {
  return 2 + (metrics ? 3 : 0) + (zsum ? 1 : 0);
}
__host__ __device__ inline int part_zs_field(bool metrics) { return metrics ? 5 : 2; }

// Forward: a split is a run of consecutive 256-id vocabulary tiles whose
// per-row online state is carried in LDS between tiles (so that the state
// takes no registers from the K loop) and ends in one partial record per
// row.  The split size depends on V only, so a row's result does not depend
// on how many rows share the call.  One workgroup per (token tile, group of
// splits_per_wg consecutive splits), walking the group's tiles in order; the
// group size depends on N and changes no result.
struct FwdArgs {
  const char* hidden;
  const char* weight;
  const char* bias;
  const int64_t* targets;
  float* part;     // [part_fields][n_splits][npad]
  float* zt_rows;  // [2 npad]: the target's logit (from the split that holds the target), then scratch
  int64_t N, H, V, ignore_index;
  int64_t npad;    // N rounded up to whole tiles
  int n_tok_tiles, n_voc_tiles, tiles_per_split, n_splits;
  int splits_per_wg, n_groups;  // n_groups = ceil(n_splits / splits_per_wg)
  int zsum;  // 1: also the sum of z over the vocabulary (label smoothing)
  float s, cap, inv_cap;
};

struct CombineArgs {
  const int64_t* targets;
  const float* part;     // [part_fields][n_splits][npad]
  const float* zt_rows;  // [2 npad]
  float* lse_out;   // may be null
  float* loss_rows; // [N] output for reduction "none", else null
  float* row_loss;  // workspace [N]
  float* row_ent;   // workspace [N]
  int* row_flag;    // workspace [N]: bit0 valid, bit1 hit, bit2 bad target
  const float* class_weight;  // [V] or null
  float* row_w;     // workspace [N]: the row's weight (0 if ignored or bad), or null
  int64_t* predictions;  // [N] argmax ids (needs METRICS), or null
  int64_t N, V, ignore_index;
  int64_t npad;          // row pitch of part
  int tiles_per_split, n_splits;
  int zsum;         // the partial records hold the sum of z
  float eps, z_loss;  // label smoothing, z-loss coefficient
  // Vocabulary shard: loss_rows receives each row's target logit when the
  // target code is a local id, 0 for ignored rows and for code `foreign`
  // (another shard's id), NaN for a bad id (flagged as for the whole vocabulary).
  // With metrics, per row: the largest logit, its first id (plus voff, an id
  // of the whole vocabulary) and the entropy of the shard's softmax.
  int shard;
  int64_t foreign, voff;
  float* shard_max;
  int64_t* shard_argmax;
  float* shard_ent;
};

// The loss of a vocabulary split into shards, from each shard's per-row
// log-sum-exp and target logit (the target's owner holds it, the others 0).
struct ShardCombineArgs {
  const float* shard_lse;     // [n_shards][N]
  const float* target_logit;  // [n_shards][N]
  const int64_t* targets;     // [N] ids of the whole vocabulary
  float* lse_out;             // [N] or null
  float* loss_rows;           // [N] for reduction "none", else null
  float* row_loss;            // workspace [N]
  int* row_flag;              // workspace [N]: bit0 valid, bit1 hit, bit2 bad target
  int64_t N, V, ignore_index; // V: the whole vocabulary
  int n_shards;
  // metrics (all null without): each shard's row max, its id and its entropy
  const float* shard_max;        // [n_shards][N]
  const int64_t* shard_argmax;   // [n_shards][N]
  const float* shard_ent;        // [n_shards][N]
  float* row_ent;                // workspace [N]: the row's entropy (0 if ignored)
  int64_t* predictions;          // [N] the row's first-index argmax, or null
};

struct ReduceArgs {
  const float* row_loss;
  const float* row_ent;
  const int* row_flag;
  const float* row_w;  // null: mean over the count of valid rows; else over the sum of row_w
  float* loss;      // [1] (mean/sum), unused for none
  float* metrics;   // [2] or null
  uint32_t* status;
  int64_t N;
  int reduction;
};

struct PrepArgs {
  const int64_t* targets;
  const float* grad_loss;  // null = 1
  const float* class_weight;  // [V] or null: mean over the weight total
  float* scale;            // out [1]: uniform gradient factor (reduction * upstream * s)
  int64_t N, V, ignore_index;
  int reduction;
  float s;
};

struct TransposeArgs {
  const char* src;   // rows x cols, leading dim src_ld elements
  char* dst;         // cols x rpad, leading dim dst_ld elements; zeros for rows <= r < rpad
  int64_t rows, cols, src_ld, rpad, dst_ld;
};

// Token n = s * T + t of a strided layout into contiguous rows: hidden row
// bytes at src + s * seq_bytes + t * row_pitch, targets at element
// s * seq_stride + t * stride.
struct GatherRowsArgs {
  const char* src;
  char* dst;           // [N][row_bytes]
  int64_t N, T, row_bytes, row_pitch, seq_bytes;
};
struct GatherTargetsArgs {
  const int64_t* src;
  int64_t* dst;        // [N]
  int64_t N, T, stride, seq_stride;
  // Vocabulary shard (shard = 1): dst holds the codes the shard's kernels
  // read instead of ids: t - voff for the shard's ids [voff, voff + vshard),
  // kShardIgnored for ignore_index, kShardForeign for another shard's id
  // (inside [0, vtotal)), kShardBad for an id outside [0, vtotal).
  int shard;
  int64_t ignore_index, voff, vshard, vtotal;
};

// Target codes of a vocabulary shard (all negative, so none is a local id).
constexpr int64_t kShardIgnored = -1, kShardBad = -2, kShardForeign = -3;

struct GArgs {
  const char* hidden;
  const char* weight;   // full (V,H)
  const char* bias;
  const int64_t* targets;
  const float* lse;
  const float* grad_rows;  // reduction "none": per-row upstream gradient (null = 1)
  char* G;                 // [npad][g_ld] (this chunk's cvpad columns) or null
  char* GT;                // [cvpad][npad] or null
  char* WcT;               // [H][wct_ld] (this chunk's cvpad columns): W_c^T, 16-bit types only, or null
  float* dbpart;           // [kBiasParts*n_tok_tiles][V] or null
  int64_t N, H, V, ignore_index, c0;
  int cv, cvpad, npad, n_tok_tiles, n_voc_tiles;
  int g_ld, wct_ld;        // row pitches (elements) of G and W_c^T
  int g_stream;            // store G with streaming (non-temporal) stores
  int none_reduction;
  int64_t foreign;         // target code of another shard's id: no one-hot term, a finite factor
                           // (ignore_index outside a vocabulary shard, which makes it unused)
  float s, cap, inv_cap;
  const float* class_weight;  // [V] or null
  float eps_v, keep, zl2;     // eps / V, 1 - eps, 2 * z_loss
};

struct DhArgs {
  const char* G;     // [npad][ld]: K = kdim columns (one or two chunks side by side)
  const char* WcT;   // [H][ld]
  float* acc;        // ksplit x [N][H] fp32 unscaled running sums across chunks (split s at acc + s * acc_stride)
  char* out;         // grad_hidden (N,H)
  const float* scale;
  int64_t N, H, acc_stride;
  int ld, kdim, n_tok_tiles, n_h_tiles, first, last;
  int ksplit, kpart;  // K in ksplit parts of kpart ids (grid.y = ksplit)
  // bk (16-bit types): no W_c^T; B is the weight rows themselves, read K-major:
  // K id k is weight row k of Wk, valid for k < wrows
  int bk;
  const char* Wk;
  int64_t wrows;
  int acc_stream;  // bk: read and write the running sums with streaming (non-temporal) accesses
  int out_f32;     // 1: grad_hidden is written as fp32 whatever the input dtype
};

// grad_hidden = the fixed-order sum of the ksplit accumulators, in the dtype.
struct DhFinalArgs {
  const float* acc;
  const float* scale;
  char* out;
  int64_t count, acc_stride;  // count = N * H (a multiple of 4); with bk, float4 blocks of the tiles
  int ksplit;
  int bk;                      // accumulators in the tile layout of the K-major grad_hidden kernel
  int64_t N, H;
  int n_h_tiles;
  int out_f32;                 // 1: out is fp32 whatever the input dtype
};

struct DwArgs {
  const char* GT;    // [cvpad][npad]; with gk, G itself: [npad][gld] from the chunk's first column
  const char* HT;    // [H][npad]
  char* out;         // grad_weight rows [c0, c0+cv)
  const float* scale;
  int64_t H;
  int cv, npad, n_voc_tiles, n_h_tiles;
  int out_f32;       // 1: out is fp32 whatever the input dtype
  int gk;            // 1 (16-bit types): GT is G, read K-major
  int gld;           // row pitch of G in elements (gk only)
};

struct DbArgs {
  const float* dbpart;
  char* out;
  const float* scale;
  int64_t V;
  int n_parts;
  int out_f32;       // 1: out is fp32 whatever the input dtype
};

// One launch of the 16-bit K-major backward: nb_dh grad_hidden workgroups
// (dh_grid per K split), then nb_dw grad_weight workgroups, then nb_g
// recompute workgroups; a part with 0 workgroups is skipped.
struct StepArgs {
  GArgs g;
  DwArgs dw;
  DhArgs dh;
  int nb_dh, dh_grid, nb_dw, nb_g;
};

// The small fp32 path (flce_small.hip): at most kSmallMaxN tokens,
// kSmallMaxV ids and a hidden size of kSmallMaxH.
constexpr int64_t kSmallMaxN = 256, kSmallMaxV = 8192, kSmallMaxH = 1024;
constexpr int kSmallDwRows = 8;  // vocabulary rows per grad_weight workgroup

struct SmallArgs {
  const char* hidden;      // [N][H] fp32, contiguous rows
  const char* weight;      // [V][H] fp32
  const char* bias;        // [V] fp32 or null
  const int64_t* targets;  // [N], contiguous
  int64_t N, H, V, ignore_index;
  float s, cap, inv_cap;   // cap = inv_cap = 1 without a soft cap
  int has_cap;
  const float* class_weight;  // [V] or null
  float eps, z_loss;       // label smoothing, z-loss coefficient
  // forward outputs (as the split combine of the tiled path writes them)
  float* lse_out;          // [N] or null
  float* loss_rows;        // [N] for reduction "none", else null
  float* row_loss;         // [N] workspace
  float* row_ent;          // [N] workspace (metrics)
  int* row_flag;           // [N] workspace
  float* row_w;            // [N] workspace or null
  int64_t* predictions;    // [N] or null
  // backward
  const float* lse;        // [N]
  const float* grad_loss;  // [1] (mean / sum) or [N] (none), null = 1
  int reduction;
  float eps_v, keep, zl2;  // eps / V, 1 - eps, 2 z_loss
  char* grad_hidden;       // [N][H] or null
  char* grad_weight;       // [V][H] or null
  char* grad_bias;         // [V] or null
};

// Launchers (flce_kernels.hip, flce_small.hip).  All asynchronous on `st`.
hipError_t launch_forward_tiles(int dtype, bool metrics, bool bias, bool cap, const FwdArgs& a,
                                hipStream_t st);
hipError_t launch_forward_combine(bool metrics, const CombineArgs& a, hipStream_t st);
hipError_t launch_forward_reduce(bool metrics, const ReduceArgs& a, hipStream_t st);
hipError_t launch_shard_combine(const ShardCombineArgs& a, hipStream_t st);
hipError_t launch_backward_prep(const PrepArgs& a, hipStream_t st);
hipError_t launch_transpose(int dtype, const TransposeArgs& a, hipStream_t st);
hipError_t launch_backward_g(int dtype, bool bias, bool cap, const GArgs& a, hipStream_t st);
hipError_t launch_backward_dh(int dtype, const DhArgs& a, hipStream_t st);
hipError_t launch_backward_dh_final(int dtype, const DhFinalArgs& a, hipStream_t st);
hipError_t launch_backward_dw(int dtype, const DwArgs& a, hipStream_t st);
hipError_t launch_backward_db(int dtype, const DbArgs& a, hipStream_t st);
hipError_t launch_backward_step(int dtype, bool bias, bool cap, const StepArgs& a, hipStream_t st);
hipError_t launch_small_forward(bool metrics, const SmallArgs& a, hipStream_t st);
hipError_t launch_small_backward(const SmallArgs& a, hipStream_t st);
// Grid sizes (workgroups: grouped_grid of each part's tile grid, a multiple
// of 8) of the three parts.
int backward_g_grid(int n_tok_tiles, int n_voc_tiles);
int backward_dh_grid(int n_h_tiles, int n_tok_tiles);
int backward_dw_grid(int n_h_tiles, int n_voc_tiles);
hipError_t launch_fill_zero(void* dst, size_t bytes, hipStream_t st);
hipError_t launch_gather_rows(const GatherRowsArgs& a, hipStream_t st);
hipError_t launch_gather_targets(const GatherTargetsArgs& a, hipStream_t st);

// The allocation-free forward's fixed workspace (a device array of this many
// bytes in flce_kernels.hip): its device address on the current device,
// looked up once per device.
constexpr size_t kScratchBytes = size_t(32) << 20;
hipError_t scratch_address(void** out);

}  // namespace flce
