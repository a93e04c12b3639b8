// flce_api.cpp -- the C ABI (include/flce.h): argument validation, the
// launch plan, workspace layout and the launch sequence of each pass.
// Host code only; kernels live in flce_kernels.hip.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>

#include "../../include/flce.h"
#include "flce_plan.h"

namespace {

thread_local std::string g_last_error;

flce_status_t fail(flce_status_t s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
flce_status_t fail(flce_status_t s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

flce_status_t hip_fail(hipError_t e, const char* what) {
  return fail(FLCE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kTile = 256;
constexpr int64_t kAlign = 256;
// At most 48 vocabulary tiles per backward chunk: at the head shape (16
// token tiles, 16 hidden tiles) the recompute and grad_weight grids are then
// three full rounds of 256 workgroups, and the fp32 grad_hidden accumulator
// is re-read 11 times at V = 128256 instead of 16 (measured 0.45 ms faster
// than 8192 there); larger chunks measured slower (their G buffers outgrow
// the last-level cache).
constexpr int64_t kMaxChunkTiles = 48;
constexpr int64_t kCUs = 256;  // MI355X compute units: one workgroup of a GEMM grid each at a time
constexpr int64_t kLastLevelCacheBytes = int64_t(256) << 20;  // MI355X Infinity Cache

// Forward vocabulary splits: at least kMinSplitTiles tiles and at most
// kMaxSplits splits (both by V only); a workgroup walks the splits of a run of
// consecutive ones, at most kMaxWgTiles tiles in all (longer runs of one
// workgroup through the vocabulary lose the operand sharing in L2 and the
// last-level cache: 256 tiles a workgroup halved the forward's speed at
// N = 16384, V = 262144).
constexpr int kMinSplitTiles = 4;
constexpr int kMaxSplits = 128;
constexpr int kMaxWgTiles = 16;

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
int64_t cdiv(int64_t x, int64_t m) { return (x + m - 1) / m; }

// The default backward chunk, in vocabulary tiles.  It depends on V and H
// only, never on N, so that a row's gradient does not depend on how many
// rows share the call (the chunking fixes grad_hidden's summation order).
// At most cap = min(a quarter of V rounded up to whole tiles, kMaxChunkTiles)
// tiles, so the chunk buffers stay far below N x V.  (Rounded down, V = 32000
// got 31-tile chunks: with 32 the recompute and grad_weight grids at
// N = 2048, H = 2048 are whole rounds, 0.4-0.8 % off that backward.)  The
// candidates are cap and the multiples of
// 16 tiles below it (with those the recompute grid, token tiles x chunk
// tiles, is whole rounds over the CUs whenever N is a multiple of 4096).
// Each is scored by how full the last round of its grad_weight grid is
// (hidden tiles x chunk tiles workgroups, each a full-K GEMM tile); the
// largest candidate within 5 % of the best score wins (fewer chunks re-read
// the grad_hidden accumulator fewer times).  Measured with N = 16384,
// H = 2048: 32 tiles (one round of 256) against 48 (1.5 rounds), 4.8 % off
// the backward; a 36-tile chunk at H = 3584 (a full last grad_weight round
// but 4.5 recompute rounds) was 8 % slower than 48.
int64_t default_chunk_tiles(int64_t H, int64_t V) {
  const int64_t cap = std::max<int64_t>(1, std::min<int64_t>(kMaxChunkTiles, cdiv(V, 4 * kTile)));
  const int64_t h_tiles = cdiv(H, kTile);
  auto eff = [&](int64_t k) {
    const int64_t wg = h_tiles * k;
    return (double)wg / (double)(cdiv(wg, kCUs) * kCUs);
  };
  double best_eff = eff(cap);
  for (int64_t k = 16; k < cap; k += 16) best_eff = std::max(best_eff, eff(k));
  if (eff(cap) >= best_eff - 0.05) return cap;
  int64_t best = 16;
  for (int64_t k = 16; k < cap; k += 16)
    if (eff(k) >= best_eff - 0.05) best = k;
  return best;
}
int elem_bytes(int dtype) { return dtype == FLCE_F32 ? 4 : 2; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

flce_status_t check_problem(const flce_problem_t* p) {
  if (!p) return fail(FLCE_ERR_INVALID_ARGUMENT, "problem is NULL");
  if (p->dtype != FLCE_F32 && p->dtype != FLCE_F16 && p->dtype != FLCE_BF16)
    return fail(FLCE_ERR_INVALID_ARGUMENT, "unknown dtype %d", p->dtype);
  if (p->reduction != FLCE_MEAN && p->reduction != FLCE_SUM && p->reduction != FLCE_NONE)
    return fail(FLCE_ERR_INVALID_ARGUMENT, "unknown reduction %d", p->reduction);
  if (p->n_tokens < 0) return fail(FLCE_ERR_INVALID_ARGUMENT, "n_tokens < 0");
  if (p->hidden < 1) return fail(FLCE_ERR_INVALID_ARGUMENT, "hidden < 1");
  if (p->vocab < 1) return fail(FLCE_ERR_INVALID_ARGUMENT, "vocab < 1");
  if (p->n_tokens >= (int64_t(1) << 31) || p->vocab >= (int64_t(1) << 31))
    return fail(FLCE_ERR_UNSUPPORTED, "n_tokens and vocab must be < 2^31");
  if (p->hidden > (int64_t(1) << 20)) return fail(FLCE_ERR_UNSUPPORTED, "hidden > 2^20");
  if ((p->hidden * elem_bytes(p->dtype)) % 16 != 0)
    return fail(FLCE_ERR_UNSUPPORTED, "hidden * sizeof(dtype) must be a multiple of 16 bytes (H=%lld)",
                (long long)p->hidden);
  if (!isfinite(p->logit_scale)) return fail(FLCE_ERR_INVALID_ARGUMENT, "logit_scale is not finite");
  if (!(p->softcap >= 0.f) || isinf(p->softcap))
    return fail(FLCE_ERR_INVALID_ARGUMENT, "softcap must be 0 (none) or a finite value > 0");
  if (p->return_metrics != 0 && p->return_metrics != 1)
    return fail(FLCE_ERR_INVALID_ARGUMENT, "return_metrics must be 0 or 1");
  if (p->has_bias != 0 && p->has_bias != 1) return fail(FLCE_ERR_INVALID_ARGUMENT, "has_bias must be 0 or 1");
  if (p->fwd_tiles_per_split < 0) return fail(FLCE_ERR_INVALID_ARGUMENT, "fwd_tiles_per_split < 0");
  if (p->bwd_vocab_chunk < 0 || p->bwd_vocab_chunk % kTile != 0)
    return fail(FLCE_ERR_INVALID_ARGUMENT, "bwd_vocab_chunk must be 0 or a positive multiple of 256");
  if (!(p->label_smoothing >= 0.f && p->label_smoothing <= 1.f))
    return fail(FLCE_ERR_INVALID_ARGUMENT, "label_smoothing must be in [0, 1]");
  if (!isfinite(p->z_loss)) return fail(FLCE_ERR_INVALID_ARGUMENT, "z_loss is not finite");
  if (p->class_weight && !aligned(p->class_weight, 4))
    return fail(FLCE_ERR_INVALID_ARGUMENT, "class_weight is misaligned");
  if (p->predictions && !aligned(p->predictions, 8))
    return fail(FLCE_ERR_INVALID_ARGUMENT, "predictions is misaligned");
  if (p->grad_weight_fp32 != 0 && p->grad_weight_fp32 != 1)
    return fail(FLCE_ERR_INVALID_ARGUMENT, "grad_weight_fp32 must be 0 or 1");
  if (p->predictions && !p->return_metrics)
    return fail(FLCE_ERR_INVALID_ARGUMENT, "predictions need return_metrics=1");
  if (p->seq_len < 0 || p->hidden_row_stride < 0 || p->hidden_seq_stride < 0 || p->targets_stride < 0 ||
      p->targets_seq_stride < 0)
    return fail(FLCE_ERR_INVALID_ARGUMENT, "seq_len and strides must be >= 0");
  constexpr int64_t kMaxStride = int64_t(1) << 40;  // elements; keeps every offset product in range
  if (p->hidden_row_stride >= kMaxStride || p->hidden_seq_stride >= kMaxStride ||
      p->targets_stride >= kMaxStride || p->targets_seq_stride >= kMaxStride)
    return fail(FLCE_ERR_INVALID_ARGUMENT, "strides must be below 2^40 elements");
  if (p->seq_len > 0 && p->n_tokens % p->seq_len != 0)
    return fail(FLCE_ERR_INVALID_ARGUMENT, "n_tokens (%lld) must be a multiple of seq_len (%lld)",
                (long long)p->n_tokens, (long long)p->seq_len);
  if ((p->hidden_row_stride * elem_bytes(p->dtype)) % 16 != 0 ||
      (p->hidden_seq_stride * elem_bytes(p->dtype)) % 16 != 0)
    return fail(FLCE_ERR_INVALID_ARGUMENT, "hidden strides times sizeof(dtype) must be multiples of 16 bytes");
  if (p->vocab_offset < 0 || p->vocab_total < 0)
    return fail(FLCE_ERR_INVALID_ARGUMENT, "vocab_offset and vocab_total must be >= 0");
  if (p->vocab_total == 0 && p->vocab_offset != 0)
    return fail(FLCE_ERR_INVALID_ARGUMENT, "vocab_offset needs vocab_total > 0 (a vocabulary shard)");
  if (p->vocab_total > 0) {
    if (p->vocab_total >= (int64_t(1) << 31)) return fail(FLCE_ERR_UNSUPPORTED, "vocab_total must be < 2^31");
    if (p->vocab_offset + p->vocab > p->vocab_total)
      return fail(FLCE_ERR_INVALID_ARGUMENT, "the shard [vocab_offset, vocab_offset + vocab) = [%lld, %lld) must lie "
                  "inside [0, vocab_total = %lld)", (long long)p->vocab_offset,
                  (long long)(p->vocab_offset + p->vocab), (long long)p->vocab_total);
    if (p->label_smoothing != 0.f || p->z_loss != 0.f || p->class_weight || p->predictions)
      return fail(FLCE_ERR_UNSUPPORTED, "a vocabulary shard takes no label smoothing, z-loss, class weights or "
                  "predictions (the combine writes predictions)");
  }
  if (p->grad_hidden_fp32 != 0 && p->grad_hidden_fp32 != 1)
    return fail(FLCE_ERR_INVALID_ARGUMENT, "grad_hidden_fp32 must be 0 or 1");
  return FLCE_OK;
}

// ---------------------------------------------------------------- token layout

// Token n = s * T + t.  Hidden rows and targets that are not contiguous are
// gathered into contiguous workspace rows first: the GEMM tiles keep one
// compile-time-shaped panel per tile (a runtime row pitch there costs
// registers in the K loop).
struct TokLayout {
  int64_t T, hr, hs, ts, tss;  // hidden strides in elements, target strides in elements
  bool h_gather, t_gather;
};

TokLayout tok_layout(const flce_problem_t& p) {
  TokLayout L{};
  const int64_t N = p.n_tokens;
  L.T = p.seq_len > 0 ? p.seq_len : std::max<int64_t>(N, 1);
  const bool one_seq = N <= L.T;
  L.hr = p.hidden_row_stride > 0 ? p.hidden_row_stride : p.hidden;
  L.hs = p.hidden_seq_stride > 0 ? p.hidden_seq_stride : L.T * L.hr;
  L.ts = p.targets_stride > 0 ? p.targets_stride : 1;
  L.tss = p.targets_seq_stride > 0 ? p.targets_seq_stride : L.T * L.ts;
  L.h_gather = N > 0 && !(L.hr == p.hidden && (one_seq || L.hs == L.T * L.hr));
  // a vocabulary shard's kernels read target codes (the mapping rides on the gather)
  L.t_gather = N > 0 && (p.vocab_total > 0 || !(L.ts == 1 && (one_seq || L.tss == L.T)));
  return L;
}

// The hidden rows and targets the kernels read: in place, or gathered into
// the workspace at off_h / off_t.
struct TokInputs {
  const char* hidden;  // N contiguous rows of H elements
  const int64_t* targets;
};

hipError_t tok_inputs(const flce_problem_t& p, const TokLayout& L, const void* hidden, const int64_t* targets,
                      char* ws, size_t off_h, size_t off_t, hipStream_t st, TokInputs& out) {
  const int eb = elem_bytes(p.dtype);
  out.hidden = reinterpret_cast<const char*>(hidden);
  out.targets = targets;
  hipError_t e;
  if (L.h_gather) {
    flce::GatherRowsArgs a{out.hidden, ws + off_h, p.n_tokens, L.T, p.hidden * eb, L.hr * eb, L.hs * eb};
    if ((e = flce::launch_gather_rows(a, st)) != hipSuccess) return e;
    out.hidden = ws + off_h;
  }
  if (L.t_gather) {
    int64_t* dst = reinterpret_cast<int64_t*>(ws + off_t);
    flce::GatherTargetsArgs a{targets, dst, p.n_tokens, L.T, L.ts, L.tss};
    if (p.vocab_total > 0) {
      a.shard = 1;
      a.ignore_index = p.ignore_index;
      a.voff = p.vocab_offset;
      a.vshard = p.vocab;
      a.vtotal = p.vocab_total;
    }
    if ((e = flce::launch_gather_targets(a, st)) != hipSuccess) return e;
    out.targets = dst;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------- forward plan

struct FwdLayout {
  int n_tok_tiles, n_voc_tiles, tiles_per_split, n_splits, splits_per_wg, n_groups;
  TokLayout tok;
  size_t off_status, off_part, off_zt, off_rowloss, off_rowent, off_rowflag, off_roww, off_hrows, off_tgt, total;
};

// Splits a forward workgroup walks, one after the other (each still ends in
// its own partial record, so the grouping changes no result and may depend
// on N): the fewest rounds of kCUs workgroups times the tiles each walks, at
// most kMaxWgTiles tiles; a tie goes to the longer run (fewer workgroups, so
// fewer pipeline fills, and the next tile's copies overlap each epilogue).
int fwd_splits_per_wg(int n_tok_tiles, int n_splits, int tiles_per_split) {
  int best_g = 1;
  int64_t best = INT64_MAX;
  for (int g = 1; g <= n_splits && (g == 1 || g * tiles_per_split <= kMaxWgTiles); ++g) {
    const int64_t wgs = (int64_t)n_tok_tiles * cdiv(n_splits, g);
    const int64_t cost = cdiv(wgs, kCUs) * g * tiles_per_split;
    if (cost <= best) {
      best = cost;
      best_g = g;
    }
  }
  return best_g;
}

FwdLayout fwd_layout(const flce_problem_t& p) {
  FwdLayout L{};
  const int64_t N = p.n_tokens, V = p.vocab;
  L.n_tok_tiles = (int)cdiv(N, kTile);
  L.n_voc_tiles = (int)cdiv(V, kTile);
  // Depends on V only (not N): a row's result must not depend on the batch.
  L.tiles_per_split = p.fwd_tiles_per_split > 0
                          ? std::min(p.fwd_tiles_per_split, L.n_voc_tiles)
                          : (int)std::min<int64_t>(L.n_voc_tiles, std::max<int64_t>(kMinSplitTiles,
                                                                                   cdiv(L.n_voc_tiles, kMaxSplits)));
  L.n_splits = (int)cdiv(L.n_voc_tiles, L.tiles_per_split);
  L.splits_per_wg = fwd_splits_per_wg(L.n_tok_tiles, L.n_splits, L.tiles_per_split);
  L.n_groups = (int)cdiv(L.n_splits, L.splits_per_wg);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (size_t)round_up((int64_t)(off + bytes), kAlign);
    return o;
  };
  L.off_status = take(16);
  // records and target logits at a row pitch of whole tiles (the tile
  // kernel stores whole tiles' columns without a predicate)
  const int64_t npad = (int64_t)L.n_tok_tiles * kTile;
  L.off_part = take((size_t)flce::part_fields(p.return_metrics != 0, p.label_smoothing > 0.f) * L.n_splits * npad * 4);
  L.off_zt = take((size_t)2 * npad * 4);
  L.off_rowloss = take((size_t)N * 4);
  L.off_rowent = take((size_t)N * 4);
  L.off_rowflag = take((size_t)N * 4);
  L.off_roww = take((size_t)N * 4);
  L.tok = tok_layout(p);
  L.off_hrows = take(L.tok.h_gather ? (size_t)N * p.hidden * elem_bytes(p.dtype) : 0);
  L.off_tgt = take(L.tok.t_gather ? (size_t)N * 8 : 0);
  L.total = off;
  return L;
}

// ---------------------------------------------------------------- backward plan

constexpr int64_t kMaxPanelPitch = int64_t(1) << 24;  // bytes

struct BwdLayout {
  int64_t chunk, last_chunk, npad, cvpad_max;  // chunks of `chunk` ids, the last of last_chunk
  int64_t cvpad_reg, gld;  // a full chunk's padded width; row pitch of the G and W_c^T buffers
  int n_chunks, n_tok_tiles, n_h_tiles, dh_split, dh_pair;
  bool gk;  // grad_weight reads G K-major (no G^T buffer)
  bool dk;  // grad_hidden reads the weight rows K-major (no W_c^T buffer)
  // gk and dk: one launch per chunk runs the recompute of the next chunk with
  // both contractions of the last one (bwd_step_kernel), so G is kept twice
  // (the chunk, or pair of chunks, being contracted and the one being written)
  bool fused;
  // caching hints: G stored with streaming stores; grad_hidden's running
  // sums read and written with streaming accesses
  bool g_stream, acc_stream;
  TokLayout tok;
  size_t off_scale, off_ht, off_wct, off_g, off_gt, off_dh, off_db, off_hrows, off_tgt, total;
};

BwdLayout bwd_layout(const flce_problem_t& p) {
  BwdLayout L{};
  const int64_t N = p.n_tokens, H = p.hidden, V = p.vocab;
  const int eb = elem_bytes(p.dtype);
  if (p.bwd_vocab_chunk > 0) {
    L.chunk = p.bwd_vocab_chunk;
  } else {
    L.chunk = default_chunk_tiles(H, V) * kTile;
  }
  L.chunk = std::min<int64_t>(L.chunk, round_up(V, kTile));
  L.n_chunks = (int)cdiv(V, L.chunk);
  // A default plan's last chunk of under a quarter of a chunk joins the one
  // before it (three launches and a grad_hidden read-modify-write saved).
  if (p.bwd_vocab_chunk <= 0 && L.n_chunks > 1 && 4 * (V - (int64_t)(L.n_chunks - 1) * L.chunk) < L.chunk)
    --L.n_chunks;
  L.last_chunk = V - (int64_t)(L.n_chunks - 1) * L.chunk;
  L.npad = round_up(std::max<int64_t>(N, 1), 64);
  L.cvpad_max = round_up(std::max(std::min(L.chunk, V), L.last_chunk), 64);
  L.n_tok_tiles = (int)cdiv(N, kTile);
  L.n_h_tiles = (int)cdiv(H, kTile);
  // With many chunks grad_hidden runs once per pair of them: the pair's G
  // and W_c^T sit side by side in K (a full chunk, then the next), so the
  // fp32 running sum is read and written half as often, for one more chunk
  // of G and W_c^T in the workspace.  Measured: 0.9-2.2 % off the backward
  // with 32 chunks (N = 16384, H = 2048, V = 262144), within noise with the
  // head shape's 11, so it is kept to 16 chunks or more.  (It depends on V
  // and H only, like the chunks.)
  L.dh_pair = L.n_chunks >= 16 ? 2 : 1;
  L.cvpad_reg = round_up(std::min(L.chunk, V), 64);
  L.gld = L.dh_pair == 2 ? L.cvpad_reg + L.cvpad_max : L.cvpad_max;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (size_t)round_up((int64_t)(off + bytes), kAlign);
    return o;
  };
  // 16-bit types: grad_hidden reads the chunk's weight rows as a K-major
  // operand, so W_c^T is neither written (the recompute kernel's side job,
  // 22 us of its time a chunk at the head shape) nor read.  Its copy offsets
  // span a pair's K ids plus two stages of weight rows.
  L.dk = eb == 2 && (L.gld + 128) * H * eb + 512 < (int64_t(1) << 32);
  // 16-bit types: grad_weight reads G itself as a K-major operand, so the
  // recompute kernel writes no G^T (measured 29 us of its 348 us a chunk at
  // the head shape).  The tile's 32-bit copy offsets must reach two stages
  // past the last token row.
  L.gk = eb == 2 && (L.npad + 128) * L.gld * eb + 512 < (int64_t(1) << 32);
  L.fused = L.dk && L.gk;
  L.off_scale = take(16);
  L.off_ht = take((size_t)H * L.npad * eb);
  L.off_wct = take(L.dk ? 0 : (size_t)H * L.gld * eb);
  L.off_g = take((size_t)(L.fused ? 2 : 1) * L.npad * L.gld * eb);
  L.off_gt = take(L.gk ? 0 : (size_t)L.cvpad_max * L.npad * eb);
  // grad_hidden's grid is token tiles x hidden tiles; when that is a small
  // part of the CUs, the chunk's K is split over 2 or 4 workgroups per tile,
  // each into an accumulator of its own, summed in a fixed order at the end.
  // In the one-launch steps grad_hidden shares the CUs with the other two
  // parts, so it only needs its workgroups no longer than a few of theirs:
  // 2 splits up to a quarter of the CUs' worth of tiles, else none.
  // (Rows of grad_hidden then depend on N only through this split: calls
  // whose grids fall in the same class give bit-identical rows.)
  const int64_t dh_tiles = (int64_t)L.n_tok_tiles * L.n_h_tiles;
  if (L.fused)
    L.dh_split = dh_tiles <= kCUs / 4 ? 2 : 1;
  else
    L.dh_split = dh_tiles <= kCUs / 4 ? 4 : dh_tiles <= kCUs / 2 ? 2 : 1;
  // (the K-major grad_hidden kernel keeps whole 256 x 256 tiles)
  const int64_t acc_elems = L.dk ? (int64_t)L.n_tok_tiles * L.n_h_tiles * kTile * kTile : N * H;
  L.off_dh = take(L.n_chunks > L.dh_pair || L.dh_split > 1 ? (size_t)L.dh_split * acc_elems * 4 : 0);
  L.off_db = take(p.has_bias ? (size_t)flce::kBiasParts * L.n_tok_tiles * V * 4 : 0);
  // Caching hints (results are the same bits either way), from alternated
  // A/B runs on one device each.  G buffers larger than the last-level cache: G
  // leaves with streaming stores (1.5-1.7 % off the backward at N = 16384,
  // H = 2048, V = 262144, 0.2-0.7 % at N = 8192, H = 3584, V = 152064; at
  // N = 4096, H = 4096, V = 128256, whose two buffers fit, plain stores are
  // 0.4-1 % faster).  A launch's data (G buffers, running sums, the chunk's
  // weight rows, hidden and hidden^T) larger than that cache: the running
  // sums, read once at the start of a launch and written once at its end,
  // bypass it (1.7-2.1 % off the backward at N = 4096, H = 4096,
  // V = 128256, 0.8-1.3 % at the two above; at N = 2048, H = 2048,
  // V = 32000, where everything fits, 1.5 % slower).
  const int64_t g_bytes = (L.fused ? 2 : 1) * L.npad * L.gld * eb;
  L.g_stream = g_bytes > kLastLevelCacheBytes;
  {
    const int64_t sums = (L.n_chunks > L.dh_pair || L.dh_split > 1) ? (int64_t)L.dh_split * acc_elems * 4 : 0;
    const int64_t rows = std::min<int64_t>(L.chunk * L.dh_pair, V) * H * eb;
    const int64_t set = g_bytes + sums + rows + 2 * L.npad * H * eb;
    L.acc_stream = set > kLastLevelCacheBytes;
  }
  L.tok = tok_layout(p);
  L.off_hrows = take(L.tok.h_gather ? (size_t)N * H * eb : 0);
  L.off_tgt = take(L.tok.t_gather ? (size_t)N * 8 : 0);
  L.total = off;
  return L;
}

// One workspace for flce_forward_backward: [forward][lse][backward].
struct FwdBwdLayout {
  size_t fwd_bytes, off_lse, off_bwd, total;
};

FwdBwdLayout fwdbwd_layout(const flce_problem_t& p) {
  FwdBwdLayout L{};
  L.fwd_bytes = (size_t)round_up((int64_t)fwd_layout(p).total, kAlign);
  L.off_lse = L.fwd_bytes;
  L.off_bwd = (size_t)round_up((int64_t)(L.off_lse + (size_t)p.n_tokens * 4), kAlign);
  L.total = L.off_bwd + bwd_layout(p).total;
  return L;
}

flce_status_t check_workspace(const void* ws, size_t bytes, size_t need) {
  if (need == 0) return FLCE_OK;
  if (!ws) return fail(FLCE_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (bytes < need) return fail(FLCE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", bytes, need);
  if (!aligned(ws, 256)) return fail(FLCE_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  return FLCE_OK;
}

float cap_of(const flce_problem_t& p) { return p.softcap > 0.f ? p.softcap : 1.f; }

// fp32 problems small enough that the 256 x 256 tiles would leave most CUs
// idle run the small path (flce_small.hip) when the plan is the default one
// (the plan overrides address the tiled path).
bool small_path(const flce_problem_t& p) {
  return p.dtype == FLCE_F32 && p.n_tokens <= flce::kSmallMaxN && p.vocab <= flce::kSmallMaxV &&
         p.hidden <= flce::kSmallMaxH && p.fwd_tiles_per_split == 0 && p.bwd_vocab_chunk == 0 &&
         p.vocab_total == 0;
}

flce::SmallArgs small_args(const flce_problem_t& p, const char* hidden, const void* weight, const void* bias,
                           const int64_t* targets) {
  flce::SmallArgs a{};
  a.hidden = hidden;
  a.weight = reinterpret_cast<const char*>(weight);
  a.bias = reinterpret_cast<const char*>(bias);
  a.targets = targets;
  a.N = p.n_tokens;
  a.H = p.hidden;
  a.V = p.vocab;
  a.ignore_index = p.ignore_index;
  a.s = p.logit_scale;
  a.cap = cap_of(p);
  a.inv_cap = 1.f / a.cap;
  a.has_cap = p.softcap > 0.f;
  a.class_weight = p.class_weight;
  a.eps = p.label_smoothing;
  a.z_loss = p.z_loss;
  a.reduction = p.reduction;
  a.eps_v = p.label_smoothing / (float)p.vocab;
  a.keep = 1.f - p.label_smoothing;
  a.zl2 = 2.f * p.z_loss;
  return a;
}

}  // namespace

extern "C" {

flce_status_t flce_forward_plan(const flce_problem_t* p, int32_t* tiles_per_split, int32_t* n_splits,
                                int32_t* splits_per_workgroup) {
  const flce_status_t s = check_problem(p);
  if (s != FLCE_OK) return s;
  const FwdLayout L = fwd_layout(*p);
  const bool small = small_path(*p);
  if (tiles_per_split) *tiles_per_split = small ? 0 : L.tiles_per_split;
  if (n_splits) *n_splits = small ? 0 : L.n_splits;
  if (splits_per_workgroup) *splits_per_workgroup = small ? 0 : L.splits_per_wg;
  return FLCE_OK;
}

flce_status_t flce_backward_plan(const flce_problem_t* p, int64_t* chunk, int64_t* n_chunks,
                                 int64_t* last_chunk, int32_t* one_launch_per_chunk) {
  const flce_status_t s = check_problem(p);
  if (s != FLCE_OK) return s;
  const BwdLayout L = bwd_layout(*p);
  const bool small = small_path(*p);  // no chunks: the whole vocabulary at once
  if (chunk) *chunk = small ? p->vocab : L.chunk;
  if (n_chunks) *n_chunks = small ? 1 : L.n_chunks;
  if (last_chunk) *last_chunk = small ? p->vocab : L.last_chunk;
  if (one_launch_per_chunk) *one_launch_per_chunk = L.fused && !small ? 1 : 0;
  return FLCE_OK;
}

size_t flce_forward_workspace_size(const flce_problem_t* p) {
  if (check_problem(p) != FLCE_OK) return 0;
  return fwd_layout(*p).total;
}

size_t flce_backward_workspace_size(const flce_problem_t* p) {
  if (check_problem(p) != FLCE_OK) return 0;
  return bwd_layout(*p).total;
}

}  // extern "C"

namespace {

// flce_combine_shards' workspace: the status word first (where
// flce_forward_status reads it), the per-row loss and flags the reduce
// kernel sums, and gathered targets for a strided layout.
struct CombineLayout {
  TokLayout tok;
  size_t off_status, off_rowloss, off_rowflag, off_rowent, off_tgt, total;
};

CombineLayout combine_layout(const flce_problem_t& p) {
  CombineLayout L{};
  const int64_t N = p.n_tokens;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (size_t)round_up((int64_t)(off + bytes), kAlign);
    return o;
  };
  L.off_status = take(16);
  L.off_rowloss = take((size_t)N * 4);
  L.off_rowflag = take((size_t)N * 4);
  L.off_rowent = take(p.return_metrics ? (size_t)N * 4 : 0);
  L.tok = tok_layout(p);
  L.off_tgt = take(L.tok.t_gather ? (size_t)N * 8 : 0);
  L.total = off;
  return L;
}

flce_status_t check_combine_problem(const flce_problem_t* p) {
  const flce_status_t s = check_problem(p);
  if (s != FLCE_OK) return s;
  if (p->vocab_total != 0)
    return fail(FLCE_ERR_INVALID_ARGUMENT, "flce_combine_shards takes the whole problem: vocab = the whole "
                "vocabulary, vocab_offset and vocab_total 0");
  if (p->label_smoothing != 0.f || p->z_loss != 0.f || p->class_weight)
    return fail(FLCE_ERR_UNSUPPORTED, "flce_combine_shards takes no label smoothing, z-loss or class weights");
  return FLCE_OK;
}

// The forward of flce_forward and, with `shard` (a vocabulary shard), of
// flce_forward_shard: then `loss` receives the per-row target logits and
// `lse` the shard's per-row log-sum-exp, and no reduction is applied.
struct ShardMetrics {
  float* max;
  int64_t* argmax;
  float* ent;
};

flce_status_t forward_impl(const flce_problem_t* p, bool shard, const void* hidden, const void* weight,
                           const int64_t* targets, const void* bias, float* loss, float* lse, float* metrics,
                           void* workspace, size_t workspace_bytes, void* stream, ShardMetrics sm = {}) {
  flce_status_t s = check_problem(p);
  if (s != FLCE_OK) return s;
  if (!shard && p->vocab_total > 0)
    return fail(FLCE_ERR_INVALID_ARGUMENT, "a vocabulary shard (vocab_total > 0) runs flce_forward_shard");
  if (shard && p->vocab_total == 0)
    return fail(FLCE_ERR_INVALID_ARGUMENT, "flce_forward_shard needs a vocabulary shard (vocab_total > 0)");
  const int64_t N = p->n_tokens;
  if (N > 0 && (!hidden || !weight || !targets))
    return fail(FLCE_ERR_INVALID_ARGUMENT, "hidden, weight and targets must be non-NULL");
  if (p->has_bias && !bias) return fail(FLCE_ERR_INVALID_ARGUMENT, "has_bias=1 but bias is NULL");
  if (!p->has_bias && bias) return fail(FLCE_ERR_INVALID_ARGUMENT, "bias given but has_bias=0");
  if (shard && N > 0 && (!loss || !lse))
    return fail(FLCE_ERR_INVALID_ARGUMENT, "shard_lse and target_logit must be non-NULL");
  if (!shard && !loss && !(p->reduction == FLCE_NONE && N == 0))
    return fail(FLCE_ERR_INVALID_ARGUMENT, "loss is NULL");
  if (shard && (!aligned(loss, 4) || !aligned(lse, 4)))
    return fail(FLCE_ERR_INVALID_ARGUMENT, "shard_lse / target_logit misaligned");
  if (shard) {
    const bool any = sm.max || sm.argmax || sm.ent, all = sm.max && sm.argmax && sm.ent;
    if (p->return_metrics && N > 0 && !all)
      return fail(FLCE_ERR_INVALID_ARGUMENT, "return_metrics=1 needs shard_max, shard_argmax and shard_entropy");
    if (!p->return_metrics && any)
      return fail(FLCE_ERR_INVALID_ARGUMENT, "shard metrics given but return_metrics=0");
    if (!aligned(sm.max, 4) || !aligned(sm.argmax, 8) || !aligned(sm.ent, 4))
      return fail(FLCE_ERR_INVALID_ARGUMENT, "shard metric outputs misaligned");
  } else {
    if (p->return_metrics && !metrics) return fail(FLCE_ERR_INVALID_ARGUMENT, "return_metrics=1 but metrics is NULL");
    if (!p->return_metrics && metrics) return fail(FLCE_ERR_INVALID_ARGUMENT, "metrics given but return_metrics=0");
  }
  if (!aligned(hidden, 16) || !aligned(weight, 16))
    return fail(FLCE_ERR_INVALID_ARGUMENT, "hidden and weight must be 16-byte aligned");
  if (!aligned(targets, 8)) return fail(FLCE_ERR_INVALID_ARGUMENT, "targets must be 8-byte aligned");
  if (bias && !aligned(bias, (uintptr_t)elem_bytes(p->dtype)))
    return fail(FLCE_ERR_INVALID_ARGUMENT, "bias is misaligned");
  const FwdLayout L = fwd_layout(*p);
  s = check_workspace(workspace, workspace_bytes, L.total);
  if (s != FLCE_OK) return s;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  const bool metrics_on = p->return_metrics != 0;
  hipError_t e;
  if (N > 0) {
    TokInputs in{};
    if ((e = tok_inputs(*p, L.tok, hidden, targets, ws, L.off_hrows, L.off_tgt, st, in)) != hipSuccess)
      return hip_fail(e, "gather kernel");
    targets = in.targets;
    if (small_path(*p)) {
      flce::SmallArgs sa = small_args(*p, in.hidden, weight, bias, targets);
      sa.lse_out = lse;
      sa.loss_rows = p->reduction == FLCE_NONE ? loss : nullptr;
      sa.row_loss = reinterpret_cast<float*>(ws + L.off_rowloss);
      sa.row_ent = reinterpret_cast<float*>(ws + L.off_rowent);
      sa.row_flag = reinterpret_cast<int*>(ws + L.off_rowflag);
      sa.row_w = p->class_weight ? reinterpret_cast<float*>(ws + L.off_roww) : nullptr;
      sa.predictions = p->predictions;
      e = flce::launch_small_forward(metrics_on, sa, st);
      if (e != hipSuccess) return hip_fail(e, "small forward kernel");
    } else {
      flce::FwdArgs fa{};
      fa.hidden = in.hidden;
      fa.weight = reinterpret_cast<const char*>(weight);
      fa.bias = reinterpret_cast<const char*>(bias);
      fa.targets = targets;
      fa.part = reinterpret_cast<float*>(ws + L.off_part);
      fa.zt_rows = reinterpret_cast<float*>(ws + L.off_zt);
      fa.N = N;
      fa.npad = (int64_t)L.n_tok_tiles * kTile;
      fa.H = p->hidden;
      fa.V = p->vocab;
      fa.ignore_index = shard ? flce::kShardIgnored : p->ignore_index;
      fa.n_tok_tiles = L.n_tok_tiles;
      fa.n_voc_tiles = L.n_voc_tiles;
      fa.tiles_per_split = L.tiles_per_split;
      fa.n_splits = L.n_splits;
      fa.splits_per_wg = L.splits_per_wg;
      fa.n_groups = L.n_groups;
      fa.s = p->logit_scale;
      fa.cap = cap_of(*p);
      fa.inv_cap = 1.f / fa.cap;
      fa.zsum = p->label_smoothing > 0.f;
      e = flce::launch_forward_tiles(p->dtype, metrics_on, p->has_bias != 0, p->softcap > 0.f, fa, st);
      if (e != hipSuccess) return hip_fail(e, "forward tile kernel");

      flce::CombineArgs ca{};
      ca.targets = targets;
      ca.part = fa.part;
      ca.zt_rows = fa.zt_rows;
      ca.lse_out = lse;
      ca.loss_rows = shard || p->reduction == FLCE_NONE ? loss : nullptr;
      ca.row_loss = reinterpret_cast<float*>(ws + L.off_rowloss);
      ca.row_ent = reinterpret_cast<float*>(ws + L.off_rowent);
      ca.row_flag = reinterpret_cast<int*>(ws + L.off_rowflag);
      ca.N = N;
      ca.npad = fa.npad;
      ca.V = p->vocab;
      ca.ignore_index = fa.ignore_index;
      ca.shard = shard ? 1 : 0;
      ca.foreign = flce::kShardForeign;
      ca.voff = p->vocab_offset;
      ca.shard_max = sm.max;
      ca.shard_argmax = sm.argmax;
      ca.shard_ent = sm.ent;
      ca.tiles_per_split = L.tiles_per_split;
      ca.n_splits = L.n_splits;
      ca.zsum = fa.zsum;
      ca.eps = p->label_smoothing;
      ca.z_loss = p->z_loss;
      ca.class_weight = p->class_weight;
      ca.row_w = p->class_weight ? reinterpret_cast<float*>(ws + L.off_roww) : nullptr;
      ca.predictions = p->predictions;
      e = flce::launch_forward_combine(metrics_on, ca, st);
      if (e != hipSuccess) return hip_fail(e, "forward combine kernel");
    }
  }
  flce::ReduceArgs ra{};
  ra.row_loss = reinterpret_cast<const float*>(ws + L.off_rowloss);
  ra.row_ent = reinterpret_cast<const float*>(ws + L.off_rowent);
  ra.row_flag = reinterpret_cast<const int*>(ws + L.off_rowflag);
  ra.row_w = p->class_weight ? reinterpret_cast<const float*>(ws + L.off_roww) : nullptr;
  ra.loss = shard ? nullptr : loss;
  ra.metrics = metrics;
  ra.status = reinterpret_cast<uint32_t*>(ws + L.off_status);
  ra.N = N;
  ra.reduction = shard ? FLCE_NONE : p->reduction;  // a shard: the status word only
  e = flce::launch_forward_reduce(metrics_on, ra, st);
  if (e != hipSuccess) return hip_fail(e, "forward reduce kernel");
  return FLCE_OK;
}

}  // namespace

extern "C" {

flce_status_t flce_forward(const flce_problem_t* p, const void* hidden, const void* weight,
                           const int64_t* targets, const void* bias, float* loss, float* lse,
                           float* metrics, void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl(p, false, hidden, weight, targets, bias, loss, lse, metrics, workspace, workspace_bytes,
                      stream);
}

flce_status_t flce_forward_shard(const flce_problem_t* p, const void* hidden, const void* weight,
                                 const int64_t* targets, const void* bias, float* shard_lse,
                                 float* target_logit, float* shard_max, int64_t* shard_argmax,
                                 float* shard_entropy, void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl(p, true, hidden, weight, targets, bias, target_logit, shard_lse, nullptr, workspace,
                      workspace_bytes, stream, ShardMetrics{shard_max, shard_argmax, shard_entropy});
}

size_t flce_combine_shards_workspace_size(const flce_problem_t* p) {
  if (check_combine_problem(p) != FLCE_OK) return 0;
  return combine_layout(*p).total;
}

flce_status_t flce_combine_shards(const flce_problem_t* p, int32_t n_shards, const float* shard_lse,
                                  const float* target_logit, const float* shard_max,
                                  const int64_t* shard_argmax, const float* shard_entropy,
                                  const int64_t* targets, float* loss, float* lse, float* metrics,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  flce_status_t s = check_combine_problem(p);
  if (s != FLCE_OK) return s;
  if (n_shards < 1) return fail(FLCE_ERR_INVALID_ARGUMENT, "n_shards must be >= 1");
  const int64_t N = p->n_tokens;
  if (N > 0 && (!shard_lse || !target_logit || !targets))
    return fail(FLCE_ERR_INVALID_ARGUMENT, "shard_lse, target_logit and targets must be non-NULL");
  if (!loss && !(p->reduction == FLCE_NONE && N == 0)) return fail(FLCE_ERR_INVALID_ARGUMENT, "loss is NULL");
  if (!aligned(shard_lse, 4) || !aligned(target_logit, 4) || !aligned(loss, 4) || !aligned(lse, 4) ||
      !aligned(targets, 8) || !aligned(shard_max, 4) || !aligned(shard_argmax, 8) || !aligned(shard_entropy, 4) ||
      !aligned(metrics, 4))
    return fail(FLCE_ERR_INVALID_ARGUMENT, "shard arrays / loss / lse / targets / metrics misaligned");
  const bool mon = p->return_metrics != 0;
  if (mon && (!metrics || (N > 0 && (!shard_max || !shard_argmax || !shard_entropy))))
    return fail(FLCE_ERR_INVALID_ARGUMENT, "return_metrics=1 needs metrics, shard_max, shard_argmax and shard_entropy");
  if (!mon && (metrics || shard_max || shard_argmax || shard_entropy))
    return fail(FLCE_ERR_INVALID_ARGUMENT, "metrics or shard metric arrays given but return_metrics=0");
  if ((int64_t)n_shards * N >= (int64_t(1) << 40))
    return fail(FLCE_ERR_UNSUPPORTED, "n_shards * n_tokens must be below 2^40");
  const CombineLayout L = combine_layout(*p);
  s = check_workspace(workspace, workspace_bytes, L.total);
  if (s != FLCE_OK) return s;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  hipError_t e;
  float* row_loss = reinterpret_cast<float*>(ws + L.off_rowloss);
  int* row_flag = reinterpret_cast<int*>(ws + L.off_rowflag);
  if (N > 0) {
    const int64_t* tg = targets;
    if (L.tok.t_gather) {
      int64_t* dst = reinterpret_cast<int64_t*>(ws + L.off_tgt);
      flce::GatherTargetsArgs ga{targets, dst, N, L.tok.T, L.tok.ts, L.tok.tss};
      if ((e = flce::launch_gather_targets(ga, st)) != hipSuccess) return hip_fail(e, "gather kernel");
      tg = dst;
    }
    flce::ShardCombineArgs a{shard_lse, target_logit, tg, lse, p->reduction == FLCE_NONE ? loss : nullptr,
                             row_loss, row_flag, N, p->vocab, p->ignore_index, n_shards};
    if (mon) {
      a.shard_max = shard_max;
      a.shard_argmax = shard_argmax;
      a.shard_ent = shard_entropy;
      a.row_ent = reinterpret_cast<float*>(ws + L.off_rowent);
      a.predictions = p->predictions;
    }
    if ((e = flce::launch_shard_combine(a, st)) != hipSuccess) return hip_fail(e, "shard combine kernel");
  }
  flce::ReduceArgs ra{};
  ra.row_loss = row_loss;
  ra.row_flag = row_flag;
  ra.row_ent = mon ? reinterpret_cast<const float*>(ws + L.off_rowent) : nullptr;
  ra.loss = loss;
  ra.metrics = metrics;
  ra.status = reinterpret_cast<uint32_t*>(ws + L.off_status);
  ra.N = N;
  ra.reduction = p->reduction;
  if ((e = flce::launch_forward_reduce(mon, ra, st)) != hipSuccess) return hip_fail(e, "forward reduce kernel");
  return FLCE_OK;
}

flce_status_t flce_forward_noalloc(const flce_problem_t* p, const void* hidden, const void* weight,
                                   const int64_t* targets, const void* bias, float* loss, float* lse,
                                   float* metrics, void* stream) {
  const flce_status_t s = check_problem(p);
  if (s != FLCE_OK) return s;
  const size_t need = fwd_layout(*p).total;
  if (need > flce::kScratchBytes)
    return fail(FLCE_ERR_WORKSPACE,
                "flce_forward_noalloc: this problem needs %zu bytes of workspace; the fixed scratch holds %zu "
                "(use flce_forward with a workspace)", need, flce::kScratchBytes);
  void* ws = nullptr;
  const hipError_t e = flce::scratch_address(&ws);
  if (e != hipSuccess) return hip_fail(e, "scratch address");
  return flce_forward(p, hidden, weight, targets, bias, loss, lse, metrics, ws, flce::kScratchBytes, stream);
}

// The backward's argument checks (no launch): flce_backward and
// flce_forward_backward run them before anything is enqueued.
static flce_status_t check_backward_args(const flce_problem_t* p, const void* hidden, const void* weight,
                                         const int64_t* targets, const void* bias, const float* lse,
                                         const float* grad_loss, void* grad_hidden, void* grad_weight,
                                         void* grad_bias) {
  const int64_t N = p->n_tokens;
  const int eb = elem_bytes(p->dtype);
  if (grad_bias && !p->has_bias) return fail(FLCE_ERR_INVALID_ARGUMENT, "grad_bias given but has_bias=0");
  if (p->has_bias && !bias) return fail(FLCE_ERR_INVALID_ARGUMENT, "has_bias=1 but bias is NULL");
  if (!p->has_bias && bias) return fail(FLCE_ERR_INVALID_ARGUMENT, "bias given but has_bias=0");
  const int geb = p->grad_weight_fp32 ? 4 : eb;  // bytes per grad_weight / grad_bias element
  if (!(grad_hidden && N > 0) && !grad_weight && !grad_bias) return FLCE_OK;
  if (N > 0 && (!hidden || !weight || !targets || !lse))
    return fail(FLCE_ERR_INVALID_ARGUMENT, "hidden, weight, targets and lse must be non-NULL");
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(grad_hidden, 16) || !aligned(grad_weight, 16))
    return fail(FLCE_ERR_INVALID_ARGUMENT, "hidden, weight, grad_hidden and grad_weight must be 16-byte aligned");
  if (!aligned(targets, 8) || !aligned(lse, 4) || !aligned(grad_loss, 4))
    return fail(FLCE_ERR_INVALID_ARGUMENT, "targets / lse / grad_loss misaligned");
  if ((bias && !aligned(bias, (uintptr_t)eb)) || (grad_bias && !aligned(grad_bias, (uintptr_t)geb)))
    return fail(FLCE_ERR_INVALID_ARGUMENT, "bias / grad_bias misaligned");
  const BwdLayout L = bwd_layout(*p);
  // The GEMM tiles read their operand panels through 32-bit buffer offsets:
  // 256 row pitches (tokens or chunk ids times the element size) stay below 4 GiB.
  if (L.npad * eb >= kMaxPanelPitch || L.gld * eb >= kMaxPanelPitch)
    return fail(FLCE_ERR_UNSUPPORTED, "backward needs n_tokens and the vocabulary chunk times sizeof(dtype) "
                "below 16 MiB (n_tokens=%lld, chunk=%lld)", (long long)N, (long long)L.chunk);
  return FLCE_OK;
}

// The backward of the 16-bit K-major path as n_chunks + 1 launches of
// bwd_step_kernel: launch k recomputes chunk k (if k < n_chunks) into G
// buffer (k / dh_pair) % 2 and contracts chunk k - 1 (grad_weight, and
// grad_hidden once its pair is complete), which an earlier launch wrote into
// the other buffer or into the other column slot of the same pair.
static hipError_t backward_fused(const flce_problem_t& p, const BwdLayout& L, const flce::GArgs& gbase,
                                 const char* weight, const char* ht, char* g, float* dh, const float* scale,
                                 void* grad_hidden, void* grad_weight, bool want_dh, bool want_dw, hipStream_t st) {
  const int64_t H = p.hidden, V = p.vocab;
  const int eb = elem_bytes(p.dtype);
  const int geb = p.grad_weight_fp32 ? 4 : eb;
  const size_t gbuf = (size_t)L.npad * L.gld * eb;
  auto chunk_cv = [&](int c) { return (int)(c == L.n_chunks - 1 ? L.last_chunk : L.chunk); };
  auto g_of = [&](int c) {  // this chunk's G columns: its pair's buffer, its slot in the pair
    const int pair = c / L.dh_pair, slot = c % L.dh_pair;
    return g + (size_t)(pair % 2) * gbuf + (size_t)(slot == 0 ? 0 : L.cvpad_reg) * eb;
  };
  hipError_t e;
  for (int k = 0; k <= L.n_chunks; ++k) {
    flce::StepArgs sa{};
    if (k < L.n_chunks) {
      const int cv = chunk_cv(k);
      sa.g = gbase;
      sa.g.G = (want_dh || want_dw) ? g_of(k) : nullptr;
      sa.g.c0 = (int64_t)k * L.chunk;
      sa.g.cv = cv;
      sa.g.cvpad = (int)round_up(cv, 64);
      sa.g.n_voc_tiles = (int)cdiv(cv, kTile);
      sa.nb_g = flce::backward_g_grid(L.n_tok_tiles, sa.g.n_voc_tiles);
    }
    const int c = k - 1;  // the chunk contracted in this launch
    if (c >= 0 && want_dw) {
      const int cv = chunk_cv(c);
      flce::DwArgs& wa = sa.dw;
      wa.GT = g_of(c);
      wa.gk = 1;
      wa.gld = (int)L.gld;
      wa.HT = ht;
      wa.out = reinterpret_cast<char*>(grad_weight) + (int64_t)c * L.chunk * H * geb;
      wa.out_f32 = p.grad_weight_fp32;
      wa.scale = scale;
      wa.H = H;
      wa.cv = cv;
      wa.npad = (int)L.npad;
      wa.n_voc_tiles = (int)cdiv(cv, kTile);
      wa.n_h_tiles = L.n_h_tiles;
      sa.nb_dw = flce::backward_dw_grid(L.n_h_tiles, wa.n_voc_tiles);
    }
    const int slot = c >= 0 ? c % L.dh_pair : 0;
    if (c >= 0 && want_dh && (slot == L.dh_pair - 1 || c == L.n_chunks - 1)) {
      const int pair = c / L.dh_pair;
      const int64_t col = slot == 0 ? 0 : L.cvpad_reg;
      flce::DhArgs& da = sa.dh;
      da.G = g + (size_t)(pair % 2) * gbuf;
      da.WcT = nullptr;
      da.acc = dh;
      da.out = reinterpret_cast<char*>(grad_hidden);
      da.scale = scale;
      da.N = p.n_tokens;
      da.H = H;
      da.ld = (int)L.gld;
      da.kdim = (int)(col + round_up(chunk_cv(c), 64));
      da.n_tok_tiles = L.n_tok_tiles;
      da.n_h_tiles = L.n_h_tiles;
      da.first = pair == 0;
      da.last = c == L.n_chunks - 1;
      da.ksplit = L.dh_split;
      da.kpart = (int)round_up(cdiv(da.kdim, L.dh_split), 64);
      da.acc_stride = (int64_t)L.n_tok_tiles * L.n_h_tiles * kTile * kTile;
      da.bk = 1;
      da.Wk = weight + (int64_t)(c - slot) * L.chunk * H * eb;
      da.wrows = V - (int64_t)(c - slot) * L.chunk;
      da.acc_stream = L.acc_stream;
      da.out_f32 = p.grad_hidden_fp32;
      sa.dh_grid = flce::backward_dh_grid(L.n_h_tiles, L.n_tok_tiles);
      sa.nb_dh = sa.dh_grid * L.dh_split;
    }
    if ((e = flce::launch_backward_step(p.dtype, p.has_bias != 0, p.softcap > 0.f, sa, st)) != hipSuccess) return e;
    if (sa.nb_dh > 0 && sa.dh.last && L.dh_split > 1) {
      flce::DhFinalArgs fa{dh, scale, reinterpret_cast<char*>(grad_hidden), sa.dh.acc_stride, sa.dh.acc_stride,
                           L.dh_split, 1, p.n_tokens, H, L.n_h_tiles, p.grad_hidden_fp32};
      if ((e = flce::launch_backward_dh_final(p.dtype, fa, st)) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

flce_status_t flce_backward(const flce_problem_t* p, const void* hidden, const void* weight,
                            const int64_t* targets, const void* bias, const float* lse,
                            const float* grad_loss, void* grad_hidden, void* grad_weight,
                            void* grad_bias, void* workspace, size_t workspace_bytes, void* stream) {
  flce_status_t s = check_problem(p);
  if (s != FLCE_OK) return s;
  s = check_backward_args(p, hidden, weight, targets, bias, lse, grad_loss, grad_hidden, grad_weight, grad_bias);
  if (s != FLCE_OK) return s;
  const int64_t N = p->n_tokens, H = p->hidden, V = p->vocab;
  const int eb = elem_bytes(p->dtype);
  const bool want_dh = grad_hidden != nullptr && N > 0;
  const bool want_dw = grad_weight != nullptr;
  const bool want_db = grad_bias != nullptr;
  const int geb = p->grad_weight_fp32 ? 4 : eb;  // bytes per grad_weight / grad_bias element
  if (!want_dh && !want_dw && !want_db) return FLCE_OK;
  const BwdLayout L = bwd_layout(*p);
  s = check_workspace(workspace, workspace_bytes, L.total);
  if (s != FLCE_OK) return s;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  hipError_t e;
  if (N == 0) {  // every gradient is zero
    if (want_dw && (e = flce::launch_fill_zero(grad_weight, (size_t)V * H * geb, st)) != hipSuccess)
      return hip_fail(e, "zero fill");
    if (want_db && (e = flce::launch_fill_zero(grad_bias, (size_t)V * geb, st)) != hipSuccess)
      return hip_fail(e, "zero fill");
    return FLCE_OK;
  }

  TokInputs in{};
  if ((e = tok_inputs(*p, L.tok, hidden, targets, ws, L.off_hrows, L.off_tgt, st, in)) != hipSuccess)
    return hip_fail(e, "gather kernel");
  targets = in.targets;
  if (small_path(*p)) {
    flce::SmallArgs sa = small_args(*p, in.hidden, weight, bias, targets);
    sa.lse = lse;
    sa.grad_loss = grad_loss;
    sa.grad_hidden = want_dh ? reinterpret_cast<char*>(grad_hidden) : nullptr;
    sa.grad_weight = want_dw ? reinterpret_cast<char*>(grad_weight) : nullptr;
    sa.grad_bias = want_db ? reinterpret_cast<char*>(grad_bias) : nullptr;
    if ((e = flce::launch_small_backward(sa, st)) != hipSuccess) return hip_fail(e, "small backward kernel");
    return FLCE_OK;
  }
  float* scale = reinterpret_cast<float*>(ws + L.off_scale);
  // a vocabulary shard's kernels read target codes (tok_inputs mapped them)
  const bool shard = p->vocab_total > 0;
  const int64_t ignore = shard ? flce::kShardIgnored : p->ignore_index;
  const int64_t foreign = shard ? flce::kShardForeign : p->ignore_index;
  flce::PrepArgs pa{targets, grad_loss, p->class_weight, scale, N, V, ignore, p->reduction, p->logit_scale};
  if ((e = flce::launch_backward_prep(pa, st)) != hipSuccess) return hip_fail(e, "backward prep kernel");

  char* ht = ws + L.off_ht;
  char* wct = ws + L.off_wct;
  char* g = ws + L.off_g;
  char* gt = ws + L.off_gt;
  float* dh = reinterpret_cast<float*>(ws + L.off_dh);
  float* db = reinterpret_cast<float*>(ws + L.off_db);
  if (want_dw) {
    flce::TransposeArgs ta{in.hidden, ht, N, H, H, L.npad, L.npad};
    if ((e = flce::launch_transpose(p->dtype, ta, st)) != hipSuccess) return hip_fail(e, "transpose kernel");
  }
  if (L.fused) {
    flce::GArgs gb{};
    gb.hidden = in.hidden;
    gb.weight = reinterpret_cast<const char*>(weight);
    gb.bias = reinterpret_cast<const char*>(bias);
    gb.targets = targets;
    gb.lse = lse;
    gb.grad_rows = p->reduction == FLCE_NONE ? grad_loss : nullptr;
    gb.GT = nullptr;
    gb.WcT = nullptr;
    gb.g_ld = (int)L.gld;
    gb.wct_ld = (int)L.gld;
    gb.g_stream = L.g_stream;
    gb.dbpart = want_db ? db : nullptr;
    gb.N = N;
    gb.H = H;
    gb.V = V;
    gb.ignore_index = ignore;
    gb.foreign = foreign;
    gb.npad = (int)L.npad;
    gb.n_tok_tiles = L.n_tok_tiles;
    gb.none_reduction = p->reduction == FLCE_NONE;
    gb.s = p->logit_scale;
    gb.cap = cap_of(*p);
    gb.inv_cap = 1.f / gb.cap;
    gb.class_weight = p->class_weight;
    gb.eps_v = p->label_smoothing / (float)V;
    gb.keep = 1.f - p->label_smoothing;
    gb.zl2 = 2.f * p->z_loss;
    if ((e = backward_fused(*p, L, gb, reinterpret_cast<const char*>(weight), ht, g, dh, scale, grad_hidden,
                            grad_weight, want_dh, want_dw, st)) != hipSuccess)
      return hip_fail(e, "backward step kernel");
  }
  for (int c = 0; c < (L.fused ? 0 : L.n_chunks); ++c) {
    const int64_t c0 = (int64_t)c * L.chunk;
    const int cv = (int)(c == L.n_chunks - 1 ? L.last_chunk : L.chunk);
    const int cvpad = (int)round_up(cv, 64);
    // slot 0 of a pair is a full chunk at column 0 of G and W_c^T; slot 1 follows it
    const int slot = c % L.dh_pair;
    const int64_t col = slot == 0 ? 0 : L.cvpad_reg;
    char* g_c = g + col * eb;
    char* wct_c = wct + col * eb;
    // W_c^T, when grad_hidden does not read the weight rows K-major: with
    // 16-bit types and at least 4 token tiles the recompute kernel writes it
    // as a side job, otherwise the transpose kernel does.
    const bool fused_wct = want_dh && eb == 2 && L.n_tok_tiles >= 4 && !L.dk;
    if (want_dh && !fused_wct && !L.dk) {
      flce::TransposeArgs ta{reinterpret_cast<const char*>(weight) + c0 * H * eb, wct_c, cv, H, H, cvpad, L.gld};
      if ((e = flce::launch_transpose(p->dtype, ta, st)) != hipSuccess) return hip_fail(e, "transpose kernel");
    }
    flce::GArgs ga{};
    ga.hidden = in.hidden;
    ga.weight = reinterpret_cast<const char*>(weight);
    ga.bias = reinterpret_cast<const char*>(bias);
    ga.targets = targets;
    ga.lse = lse;
    ga.grad_rows = p->reduction == FLCE_NONE ? grad_loss : nullptr;
    ga.G = want_dh || (want_dw && L.gk) ? g_c : nullptr;
    ga.GT = want_dw && !L.gk ? gt : nullptr;
    ga.WcT = fused_wct ? wct_c : nullptr;
    ga.g_ld = (int)L.gld;
    ga.wct_ld = (int)L.gld;
    ga.dbpart = want_db ? db : nullptr;
    ga.N = N;
    ga.H = H;
    ga.V = V;
    ga.ignore_index = ignore;
    ga.foreign = foreign;
    ga.c0 = c0;
    ga.cv = cv;
    ga.cvpad = cvpad;
    ga.npad = (int)L.npad;
    ga.n_tok_tiles = L.n_tok_tiles;
    ga.n_voc_tiles = (int)cdiv(cv, kTile);
    ga.none_reduction = p->reduction == FLCE_NONE;
    ga.s = p->logit_scale;
    ga.cap = cap_of(*p);
    ga.inv_cap = 1.f / ga.cap;
    ga.class_weight = p->class_weight;
    ga.eps_v = p->label_smoothing / (float)V;
    ga.keep = 1.f - p->label_smoothing;
    ga.zl2 = 2.f * p->z_loss;
    if ((e = flce::launch_backward_g(p->dtype, p->has_bias != 0, p->softcap > 0.f, ga, st)) != hipSuccess)
      return hip_fail(e, "backward G kernel");
    if (want_dw) {
      flce::DwArgs wa{};
      wa.GT = L.gk ? g_c : gt;
      wa.gk = L.gk ? 1 : 0;
      wa.gld = (int)L.gld;
      wa.HT = ht;
      wa.out = reinterpret_cast<char*>(grad_weight) + c0 * H * geb;
      wa.out_f32 = p->grad_weight_fp32;
      wa.scale = scale;
      wa.H = H;
      wa.cv = cv;
      wa.npad = (int)L.npad;
      wa.n_voc_tiles = (int)cdiv(cv, kTile);
      wa.n_h_tiles = L.n_h_tiles;
      if ((e = flce::launch_backward_dw(p->dtype, wa, st)) != hipSuccess) return hip_fail(e, "grad_weight kernel");
    }
    // grad_hidden once the pair is complete (or at the last chunk); after
    // grad_weight, which needs this chunk's G (or G^T) before the next chunk's
    // recompute overwrites it
    if (want_dh && (slot == L.dh_pair - 1 || c == L.n_chunks - 1)) {
      const int pair = c / L.dh_pair;
      flce::DhArgs da{};
      da.G = g;
      da.WcT = wct;
      da.acc = dh;
      da.out = reinterpret_cast<char*>(grad_hidden);
      da.scale = scale;
      da.N = N;
      da.H = H;
      da.ld = (int)L.gld;
      da.kdim = (int)(col + cvpad);
      da.n_tok_tiles = L.n_tok_tiles;
      da.n_h_tiles = L.n_h_tiles;
      da.first = pair == 0;
      da.last = c == L.n_chunks - 1;
      da.ksplit = L.dh_split;
      da.kpart = (int)round_up(cdiv(da.kdim, L.dh_split), 64);
      da.acc_stride = L.dk ? (int64_t)L.n_tok_tiles * L.n_h_tiles * kTile * kTile : N * H;
      da.bk = L.dk ? 1 : 0;
      da.Wk = reinterpret_cast<const char*>(weight) + (int64_t)(c - slot) * L.chunk * H * eb;
      da.wrows = V - (int64_t)(c - slot) * L.chunk;
      da.acc_stream = L.acc_stream;
      da.out_f32 = p->grad_hidden_fp32;
      if ((e = flce::launch_backward_dh(p->dtype, da, st)) != hipSuccess) return hip_fail(e, "grad_hidden kernel");
      if (da.last && L.dh_split > 1) {
        flce::DhFinalArgs fa{dh, scale, reinterpret_cast<char*>(grad_hidden), da.acc_stride, da.acc_stride,
                             L.dh_split, L.dk ? 1 : 0, N, H, L.n_h_tiles, p->grad_hidden_fp32};
        if ((e = flce::launch_backward_dh_final(p->dtype, fa, st)) != hipSuccess)
          return hip_fail(e, "grad_hidden sum kernel");
      }
    }
  }
  if (want_db) {
    flce::DbArgs ba{db, reinterpret_cast<char*>(grad_bias), scale, V, flce::kBiasParts * L.n_tok_tiles,
                    p->grad_weight_fp32};
    if ((e = flce::launch_backward_db(p->dtype, ba, st)) != hipSuccess) return hip_fail(e, "grad_bias kernel");
  }
  return FLCE_OK;
}

size_t flce_forward_backward_workspace_size(const flce_problem_t* p) {
  if (check_problem(p) != FLCE_OK) return 0;
  const FwdBwdLayout L = fwdbwd_layout(*p);
  return L.total;
}

flce_status_t flce_forward_backward(const flce_problem_t* p, const void* hidden, const void* weight,
                                    const int64_t* targets, const void* bias, float* loss, float* lse,
                                    float* metrics, const float* grad_loss, void* grad_hidden,
                                    void* grad_weight, void* grad_bias, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  flce_status_t s = check_problem(p);
  if (s != FLCE_OK) return s;
  if (p->vocab_total > 0)
    return fail(FLCE_ERR_INVALID_ARGUMENT, "a vocabulary shard needs the combined lse before its backward: "
                "flce_forward_shard, flce_combine_shards, flce_backward");
  const FwdBwdLayout L = fwdbwd_layout(*p);
  s = check_workspace(workspace, workspace_bytes, L.total);
  if (s != FLCE_OK) return s;
  char* ws = reinterpret_cast<char*>(workspace);
  float* lse_use = lse ? lse : reinterpret_cast<float*>(ws + L.off_lse);
  // the backward's checks first, so that a call it would refuse enqueues nothing
  s = check_backward_args(p, hidden, weight, targets, bias, lse_use, grad_loss, grad_hidden, grad_weight,
                          grad_bias);
  if (s != FLCE_OK) return s;
  s = flce_forward(p, hidden, weight, targets, bias, loss, lse_use, metrics, ws, L.fwd_bytes, stream);
  if (s != FLCE_OK) return s;
  return flce_backward(p, hidden, weight, targets, bias, lse_use, grad_loss, grad_hidden, grad_weight,
                       grad_bias, ws + L.off_bwd, L.total - L.off_bwd, stream);
}

flce_status_t flce_forward_status(const flce_problem_t* p, const void* workspace, uint32_t* status_out,
                                  void* stream) {
  flce_status_t s = check_problem(p);
  if (s != FLCE_OK) return s;
  if (!workspace || !status_out) return fail(FLCE_ERR_INVALID_ARGUMENT, "workspace and status_out must be non-NULL");
  const FwdLayout L = fwd_layout(*p);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(status_out, reinterpret_cast<const char*>(workspace) + L.off_status,
                                sizeof(uint32_t), hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return hip_fail(e, "status copy");
  if ((e = hipStreamSynchronize(st)) != hipSuccess) return hip_fail(e, "status sync");
  return FLCE_OK;
}

const char* flce_status_str(flce_status_t s) {
  switch (s) {
    case FLCE_OK: return "FLCE_OK";
    case FLCE_ERR_INVALID_ARGUMENT: return "FLCE_ERR_INVALID_ARGUMENT";
    case FLCE_ERR_UNSUPPORTED: return "FLCE_ERR_UNSUPPORTED";
    case FLCE_ERR_WORKSPACE: return "FLCE_ERR_WORKSPACE";
    case FLCE_ERR_HIP: return "FLCE_ERR_HIP";
  }
  return "FLCE_ERR_UNKNOWN";
}

const char* flce_last_error(void) { return g_last_error.c_str(); }

const char* flce_version(void) { return "flce-gfx950 0.1.0"; }
size_t flce_problem_size(void) { return sizeof(flce_problem_t); }

}  // extern "C"
