// Host-only driver of the C ABI (test infrastructure): calls every entry
// point over a sweep of problems with fake device addresses, against the
// launcher stand-ins of flce_host_stubs.cpp, so that AddressSanitizer and
// UndefinedBehaviorSanitizer check the host layer and the stubs check every
// workspace range it hands a kernel.  Prints "ok <calls> <launches>" and
// exits 0 when nothing was flagged.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "flce.h"
#include "flce_plan.h"

namespace hoststub {
extern int violations, launches;
extern const void* hidden_ptr;
void begin(const void* ws, size_t bytes);
int end();
}  // namespace hoststub

static char* A(uint64_t x) { return reinterpret_cast<char*>(uintptr_t(x)); }
// Fake device address ranges (never dereferenced), 1 TiB apart.
static char* const HID = A(0x100000000000ull);
static char* const WGT = A(0x110000000000ull);
static char* const TGT = A(0x120000000000ull);
static char* const BIA = A(0x130000000000ull);
static char* const OUT = A(0x140000000000ull);
static char* const WSP = A(0x200000000000ull);
static char* const NOALLOC = A(0x7f0000000000ull);  // the stubs' scratch address

static int calls = 0, failures = 0;

static void expect(flce_status_t got, flce_status_t want, const char* what, const flce_problem_t& p) {
  ++calls;
  if (got != want) {
    ++failures;
    fprintf(stderr, "FAIL %s: status %d (want %d) N=%lld H=%lld V=%lld dtype=%d: %s\n", what, got, want,
            (long long)p.n_tokens, (long long)p.hidden, (long long)p.vocab, p.dtype, flce_last_error());
  }
}

static flce_problem_t base(int64_t n, int64_t h, int64_t v, int dtype) {
  flce_problem_t p;
  memset(&p, 0, sizeof p);
  p.n_tokens = n;
  p.hidden = h;
  p.vocab = v;
  p.ignore_index = -100;
  p.dtype = dtype;
  p.reduction = FLCE_MEAN;
  p.logit_scale = 1.0f;
  return p;
}

static void run(flce_problem_t p, bool strided = false) {
  const bool none = p.reduction == FLCE_NONE;
  float* loss = reinterpret_cast<float*>(OUT);
  float* lse = reinterpret_cast<float*>(OUT + (1ull << 36));
  float* metrics = p.return_metrics ? reinterpret_cast<float*>(OUT + (2ull << 36)) : nullptr;
  float* gl = reinterpret_cast<float*>(OUT + (3ull << 36));
  void* gh = OUT + (4ull << 36);
  void* gw = OUT + (5ull << 36);
  void* gb = p.has_bias ? OUT + (6ull << 36) : nullptr;
  const void* bias = p.has_bias ? BIA : nullptr;
  if (strided) {
    p.seq_len = p.n_tokens / 4;
    p.hidden_row_stride = p.hidden + 8 * (p.dtype == FLCE_F32 ? 4 : 8);
    p.hidden_seq_stride = (p.seq_len + 1) * p.hidden_row_stride;
    p.targets_stride = 2;
    p.targets_seq_stride = 2 * (p.seq_len + 1);
  }
  hoststub::hidden_ptr = HID;
  int32_t tps = -1, nsp = -1, gsp = -1;
  expect(flce_forward_plan(&p, &tps, &nsp, &gsp), FLCE_OK, "forward plan", p);
  expect(flce_forward_plan(&p, nullptr, nullptr, nullptr), FLCE_OK, "forward plan, no outputs", p);
  const size_t fs = flce_forward_workspace_size(&p), bs = flce_backward_workspace_size(&p);
  const size_t fbs = flce_forward_backward_workspace_size(&p);
  hoststub::begin(WSP, fs);
  expect(flce_forward(&p, HID, WGT, reinterpret_cast<const int64_t*>(TGT), bias, loss, lse, metrics, WSP, fs, nullptr),
         FLCE_OK, "forward", p);
  hoststub::end();
  hoststub::begin(WSP, bs);
  expect(flce_backward(&p, HID, WGT, reinterpret_cast<const int64_t*>(TGT), bias, lse, none ? gl : nullptr, gh, gw,
                       gb, WSP, bs, nullptr),
         FLCE_OK, "backward", p);
  hoststub::end();
  // only some gradients wanted
  hoststub::begin(WSP, bs);
  expect(flce_backward(&p, HID, WGT, reinterpret_cast<const int64_t*>(TGT), bias, lse, nullptr, gh, nullptr,
                       nullptr, WSP, bs, nullptr),
         FLCE_OK, "backward grad_hidden only", p);
  hoststub::end();
  hoststub::begin(WSP, bs);
  expect(flce_backward(&p, HID, WGT, reinterpret_cast<const int64_t*>(TGT), bias, lse, nullptr, nullptr, gw, gb,
                       WSP, bs, nullptr),
         FLCE_OK, "backward grad_weight only", p);
  hoststub::end();
  hoststub::begin(WSP, fbs);
  expect(flce_forward_backward(&p, HID, WGT, reinterpret_cast<const int64_t*>(TGT), bias, loss, nullptr, metrics,
                               none ? gl : nullptr, gh, gw, gb, WSP, fbs, nullptr),
         FLCE_OK, "forward_backward", p);
  hoststub::end();
  if (fs <= (size_t(32) << 20)) {
    hoststub::begin(NOALLOC, size_t(32) << 20);
    expect(flce_forward_noalloc(&p, HID, WGT, reinterpret_cast<const int64_t*>(TGT), bias, loss, lse, metrics, nullptr),
           FLCE_OK, "forward_noalloc", p);
    hoststub::end();
  }
  // a workspace one byte short is refused before any launch
  if (fs > 0) {
    const int before = hoststub::launches;
    expect(flce_forward(&p, HID, WGT, reinterpret_cast<const int64_t*>(TGT), bias, loss, lse, metrics, WSP, fs - 1,
                        nullptr),
           FLCE_ERR_WORKSPACE, "forward short workspace", p);
    if (hoststub::launches != before) {
      ++failures;
      fprintf(stderr, "FAIL: a refused forward launched something\n");
    }
  }
}

// A vocabulary split into shards of the whole problem p: each shard's
// forward and backward (fp32 grad_hidden), then the combine of the whole.
// The entry points that refuse a shard do so before any launch.
static void run_shards(flce_problem_t whole, const int64_t* bounds, int n_shards, bool strided = false) {
  const bool none = whole.reduction == FLCE_NONE;
  float* gl = reinterpret_cast<float*>(OUT + (3ull << 36));
  float* slse = reinterpret_cast<float*>(OUT + (7ull << 36));
  float* stl = reinterpret_cast<float*>(OUT + (8ull << 36));
  float* loss = reinterpret_cast<float*>(OUT);
  float* lse = reinterpret_cast<float*>(OUT + (1ull << 36));
  if (strided) {
    whole.seq_len = whole.n_tokens / 4;
    whole.hidden_row_stride = whole.hidden + 8 * (whole.dtype == FLCE_F32 ? 4 : 8);
    whole.hidden_seq_stride = (whole.seq_len + 1) * whole.hidden_row_stride;
    whole.targets_stride = 2;
    whole.targets_seq_stride = 2 * (whole.seq_len + 1);
  }
  hoststub::hidden_ptr = HID;
  for (int k = 0; k < n_shards; ++k) {
    flce_problem_t p = whole;
    p.vocab_offset = bounds[k];
    p.vocab = bounds[k + 1] - bounds[k];
    p.vocab_total = whole.vocab;
    p.grad_hidden_fp32 = 1;
    const void* bias = p.has_bias ? BIA : nullptr;
    const size_t fs = flce_forward_workspace_size(&p), bs = flce_backward_workspace_size(&p);
    hoststub::begin(WSP, fs);
    float* smax = p.return_metrics ? reinterpret_cast<float*>(OUT + (9ull << 36)) + k * p.n_tokens : nullptr;
    int64_t* sarg = p.return_metrics ? reinterpret_cast<int64_t*>(OUT + (10ull << 36)) + k * p.n_tokens : nullptr;
    float* sent = p.return_metrics ? reinterpret_cast<float*>(OUT + (11ull << 36)) + k * p.n_tokens : nullptr;
    expect(flce_forward_shard(&p, HID, WGT, reinterpret_cast<const int64_t*>(TGT), bias, slse + k * p.n_tokens,
                              stl + k * p.n_tokens, smax, sarg, sent, WSP, fs, nullptr),
           FLCE_OK, "forward shard", p);
    hoststub::end();
    hoststub::begin(WSP, bs);
    expect(flce_backward(&p, HID, WGT, reinterpret_cast<const int64_t*>(TGT), bias, lse, none ? gl : nullptr,
                         OUT + (4ull << 36), OUT + (5ull << 36), p.has_bias ? OUT + (6ull << 36) : nullptr, WSP, bs,
                         nullptr),
           FLCE_OK, "backward shard", p);
    hoststub::end();
    const int before = hoststub::launches;
    float l;
    expect(flce_forward(&p, HID, WGT, reinterpret_cast<const int64_t*>(TGT), bias, &l, lse, nullptr, WSP, fs, nullptr),
           FLCE_ERR_INVALID_ARGUMENT, "flce_forward of a shard", p);
    expect(flce_forward_backward(&p, HID, WGT, reinterpret_cast<const int64_t*>(TGT), bias, &l, lse, nullptr, nullptr,
                                 OUT + (4ull << 36), nullptr, nullptr, WSP, size_t(1) << 40, nullptr),
           FLCE_ERR_INVALID_ARGUMENT, "forward_backward of a shard", p);
    if (hoststub::launches != before) {
      ++failures;
      fprintf(stderr, "FAIL: a refused shard call launched something\n");
    }
  }
  const size_t cs = flce_combine_shards_workspace_size(&whole);
  const bool m = whole.return_metrics != 0;
  hoststub::begin(WSP, cs);
  expect(flce_combine_shards(&whole, n_shards, slse, stl, m ? reinterpret_cast<float*>(OUT + (9ull << 36)) : nullptr,
                             m ? reinterpret_cast<int64_t*>(OUT + (10ull << 36)) : nullptr,
                             m ? reinterpret_cast<float*>(OUT + (11ull << 36)) : nullptr,
                             reinterpret_cast<const int64_t*>(TGT), loss, lse,
                             m ? reinterpret_cast<float*>(OUT + (2ull << 36)) : nullptr, WSP, cs, nullptr),
         FLCE_OK, "combine shards", whole);
  hoststub::end();
}

// Tile orders: every tile of the grid exactly once; with the XCD remap, a
// grid of a multiple of 8 and per-XCD tile counts at most one apart; and for
// grids of whole 4 x 8 blocks the plain block order (blocks along a, then b;
// a fastest inside a block; XCD x taking the x-th eighth of it).
template <bool XCD>
static void check_order(int na, int nb) {
  const int nblocks = flce::grouped_grid<XCD>(na, nb);
  std::vector<int> seen((size_t)na * nb, 0);
  int per_xcd[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  bool whole = na % 4 == 0 && nb % 8 == 0;
  if (XCD && nblocks % 8 != 0) ++failures;
  for (int bid = 0; bid < nblocks; ++bid) {
    const flce::TileAB t = flce::grouped_tile<4, 8, XCD>(bid, nblocks, na, nb);
    if (!t.valid) continue;
    if (t.a < 0 || t.a >= na || t.b < 0 || t.b >= nb) {
      ++failures;
      fprintf(stderr, "FAIL tile order %d x %d (xcd %d): block %d -> (%d, %d)\n", na, nb, XCD, bid, t.a, t.b);
      continue;
    }
    ++seen[(size_t)t.b * na + t.a];
    ++per_xcd[bid % 8];
    if (whole) {
      const int L = XCD ? (bid % 8) * (nblocks / 8) + bid / 8 : bid;
      const int g = L / 32, w = L % 32, nga = na / 4;
      if (t.a != (g % nga) * 4 + w % 4 || t.b != (g / nga) * 8 + w / 4) whole = false;
    }
  }
  for (size_t i = 0; i < seen.size(); ++i)
    if (seen[i] != 1) {
      ++failures;
      fprintf(stderr, "FAIL tile order %d x %d (xcd %d): tile %zu taken %d times\n", na, nb, XCD, i, seen[i]);
      break;
    }
  if (XCD) {
    int lo = per_xcd[0], hi = per_xcd[0];
    for (int x = 1; x < 8; ++x) lo = per_xcd[x] < lo ? per_xcd[x] : lo, hi = per_xcd[x] > hi ? per_xcd[x] : hi;
    if (hi - lo > 1) {
      ++failures;
      fprintf(stderr, "FAIL tile order %d x %d: XCD counts %d .. %d\n", na, nb, lo, hi);
    }
  }
  if (na % 4 == 0 && nb % 8 == 0 && !whole) {
    ++failures;
    fprintf(stderr, "FAIL tile order %d x %d (xcd %d): not the plain block order\n", na, nb, XCD);
  }
  ++calls;
}

int main() {
  for (int na = 1; na <= 40; ++na)
    for (int nb = 1; nb <= 72; ++nb) {
      check_order<false>(na, nb);
      check_order<true>(na, nb);
    }
  const int big[][2] = {{16, 501}, {32, 594}, {64, 1024}, {14, 48}, {14, 32}, {8, 31}, {32, 48}, {16, 48}, {125, 8}};
  for (const auto& g : big) {
    check_order<false>(g[0], g[1]);
    check_order<true>(g[0], g[1]);
  }
  const int dts[3] = {FLCE_F32, FLCE_F16, FLCE_BF16};
  // the five workloads
  {
    flce_problem_t p = base(64, 128, 1000, FLCE_F32);
    p.return_metrics = 1;
    run(p);
    run(base(2048, 2048, 32000, FLCE_BF16));
    run(base(4096, 4096, 128256, FLCE_BF16));
    p = base(8192, 3584, 152064, FLCE_BF16);
    p.has_bias = 1;
    p.logit_scale = 0.5f;
    p.softcap = 30.f;
    p.reduction = FLCE_SUM;
    p.return_metrics = 1;
    run(p);
    run(base(16384, 2048, 262144, FLCE_BF16));
    p = base(16384, 2048, 262144, FLCE_BF16);
    p.reduction = FLCE_NONE;
    run(p);
  }
  // a sweep of shapes, dtypes, options and plans
  const int64_t ns[] = {0, 1, 63, 256, 300, 1030};
  const int64_t hs[] = {8, 64, 200, 256, 1024, 1032};
  const int64_t vs[] = {1, 37, 1000, 2600, 8192, 8193, 33000};
  for (int d = 0; d < 3; ++d)
    for (int64_t n : ns)
      for (int64_t h : hs)
        for (int64_t v : vs) {
          if ((h * (dts[d] == FLCE_F32 ? 4 : 2)) % 16) continue;
          flce_problem_t p = base(n, h, v, dts[d]);
          const int k = (int)(n + h + v) % 5;
          p.reduction = k % 3;
          p.has_bias = k & 1;
          p.return_metrics = (k >> 1) & 1;
          p.softcap = k == 4 ? 5.f : 0.f;
          p.label_smoothing = k == 3 ? 0.1f : 0.f;
          p.z_loss = k == 2 ? 1e-3f : 0.f;
          p.grad_weight_fp32 = k == 1;
          run(p);
          p.bwd_vocab_chunk = 256;
          p.fwd_tiles_per_split = 3;
          run(p);
          if (n >= 4 && n % 4 == 0) run(p, true);
        }
  // vocabulary shards
  {
    const int64_t b2[] = {0, 1000, 2600}, b3[] = {0, 300, 301, 2600}, b8[9] = {0, 16032, 32064, 48096, 64128,
                                                                               80160, 96192, 112224, 128256};
    for (int d = 1; d < 3; ++d)
      for (int r = 0; r < 3; ++r) {
        flce_problem_t p = base(300, 256, 2600, dts[d]);
        p.reduction = r;
        p.has_bias = r == 1;
        p.softcap = r == 2 ? 30.f : 0.f;
        p.return_metrics = r != 1;
        run_shards(p, b2, 2);
        run_shards(p, b3, 3);
        run_shards(p, b3, 3, true);
      }
    run_shards(base(4096, 4096, 128256, FLCE_BF16), b8, 8);
    flce_problem_t p = base(64, 128, 1000, FLCE_F32);  // not the small path with a shard
    const int64_t bf[] = {0, 500, 1000};
    run_shards(p, bf, 2);
    // refused shard descriptions: a status, nothing launched
    const int before = hoststub::launches;
    p = base(300, 256, 1000, FLCE_BF16);
    p.vocab_offset = 1700;
    p.vocab_total = 2600;
    float l;
    expect(flce_forward_shard(&p, HID, WGT, reinterpret_cast<const int64_t*>(TGT), nullptr, &l, &l, nullptr, nullptr,
                              nullptr, WSP, 1 << 30, nullptr),
           FLCE_ERR_INVALID_ARGUMENT, "shard past the vocabulary", p);
    p.vocab_offset = 1600;
    p.z_loss = 1e-3f;
    expect(flce_forward_shard(&p, HID, WGT, reinterpret_cast<const int64_t*>(TGT), nullptr, &l, &l, nullptr, nullptr,
                              nullptr, WSP, 1 << 30, nullptr),
           FLCE_ERR_UNSUPPORTED, "shard with z-loss", p);
    p.z_loss = 0.f;
    p.return_metrics = 1;
    expect(flce_forward_shard(&p, HID, WGT, reinterpret_cast<const int64_t*>(TGT), nullptr, &l, &l, nullptr, nullptr,
                              nullptr, WSP, 1 << 30, nullptr),
           FLCE_ERR_INVALID_ARGUMENT, "shard metrics without their outputs", p);
    p.return_metrics = 0;
    p.vocab_total = 0;
    expect(flce_forward_shard(&p, HID, WGT, reinterpret_cast<const int64_t*>(TGT), nullptr, &l, &l, nullptr, nullptr,
                              nullptr, WSP, 1 << 30, nullptr),
           FLCE_ERR_INVALID_ARGUMENT, "offset without a vocabulary total", p);
    p.vocab_offset = 0;
    expect(flce_forward_shard(&p, HID, WGT, reinterpret_cast<const int64_t*>(TGT), nullptr, &l, &l, nullptr, nullptr,
                              nullptr, WSP, 1 << 30, nullptr),
           FLCE_ERR_INVALID_ARGUMENT, "forward shard without a shard", p);
    p.vocab_total = 2600;
    expect(flce_combine_shards(&p, 2, &l, &l, nullptr, nullptr, nullptr, reinterpret_cast<const int64_t*>(TGT), &l, &l,
                               nullptr, WSP, 1 << 30, nullptr),
           FLCE_ERR_INVALID_ARGUMENT, "combine of a shard problem", p);
    p.vocab_total = 0;
    expect(flce_combine_shards(&p, 0, &l, &l, nullptr, nullptr, nullptr, reinterpret_cast<const int64_t*>(TGT), &l, &l,
                               nullptr, WSP, 1 << 30, nullptr),
           FLCE_ERR_INVALID_ARGUMENT, "combine of no shards", p);
    p.return_metrics = 1;
    expect(flce_combine_shards(&p, 2, &l, &l, nullptr, nullptr, nullptr, reinterpret_cast<const int64_t*>(TGT), &l, &l,
                               &l, WSP, 1 << 30, nullptr),
           FLCE_ERR_INVALID_ARGUMENT, "combine metrics without the shard arrays", p);
    if (hoststub::launches != before) {
      ++failures;
      fprintf(stderr, "FAIL: a refused shard description launched something\n");
    }
  }
  // invalid arguments: a status, nothing launched
  {
    flce_problem_t p = base(64, 128, 1000, FLCE_BF16);
    const int before = hoststub::launches;
    float loss;
    expect(flce_forward(&p, nullptr, WGT, reinterpret_cast<const int64_t*>(TGT), nullptr, &loss, nullptr, nullptr, WSP,
                        1 << 20, nullptr),
           FLCE_ERR_INVALID_ARGUMENT, "null hidden", p);
    expect(flce_forward(&p, HID + 8, WGT, reinterpret_cast<const int64_t*>(TGT), nullptr, &loss, nullptr, nullptr, WSP,
                        1 << 20, nullptr),
           FLCE_ERR_INVALID_ARGUMENT, "misaligned hidden", p);
    p.softcap = -1.f;
    expect(flce_forward(&p, HID, WGT, reinterpret_cast<const int64_t*>(TGT), nullptr, &loss, nullptr, nullptr, WSP,
                        1 << 20, nullptr),
           FLCE_ERR_INVALID_ARGUMENT, "negative softcap", p);
    p = base(64, 100, 1000, FLCE_BF16);
    expect(flce_forward(&p, HID, WGT, reinterpret_cast<const int64_t*>(TGT), nullptr, &loss, nullptr, nullptr, WSP,
                        1 << 20, nullptr),
           FLCE_ERR_UNSUPPORTED, "row bytes not a multiple of 16", p);
    expect(flce_forward_status(nullptr, WSP, nullptr, nullptr), FLCE_ERR_INVALID_ARGUMENT, "status of null problem", p);
    if (hoststub::launches != before) {
      ++failures;
      fprintf(stderr, "FAIL: an invalid call launched something\n");
    }
    if (strcmp(flce_status_str((flce_status_t)77), "FLCE_ERR_UNKNOWN") != 0) ++failures;
  }
  if (failures || hoststub::violations) {
    fprintf(stderr, "%d failures, %d violations\n", failures, hoststub::violations);
    return 1;
  }
  printf("ok %d %d\n", calls, hoststub::launches);
  return 0;
}
