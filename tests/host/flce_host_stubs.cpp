// Host-only stand-ins for the kernel launchers of libflce (test
// infrastructure): built with the host layer (flce_api.cpp) under
// AddressSanitizer and UndefinedBehaviorSanitizer, they launch nothing and
// instead check that every workspace pointer the host layer hands a kernel,
// with the extent that kernel touches, lies inside the caller's workspace,
// and that the named workspace buffers of one call never overlap.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <string>

#include "flce_plan.h"

namespace hoststub {
uintptr_t ws_lo = 0, ws_hi = 0;  // the registered workspace of the current call
const void* hidden_ptr = nullptr; // the caller's hidden rows of the current call
int violations = 0;
std::map<std::string, std::pair<uintptr_t, uintptr_t>> regions;  // name -> [lo, hi) touched

// Regions are named per pass: flce_forward_backward runs the forward (which
// ends with the reduce launch) and then the backward in one workspace, and
// the two passes may reuse each other's bytes.
int pass = 0;

void begin(const void* ws, size_t bytes) {
  ws_lo = reinterpret_cast<uintptr_t>(ws);
  ws_hi = ws_lo + bytes;
  regions.clear();
  pass = 0;
}

static void fail(const char* what, const char* name, uintptr_t p, size_t n) {
  ++violations;
  fprintf(stderr, "VIOLATION %s: %s [%#lx, %#lx) outside workspace [%#lx, %#lx)\n", what, name,
          (unsigned long)p, (unsigned long)(p + n), (unsigned long)ws_lo, (unsigned long)ws_hi);
}

// A pointer that must be inside the workspace, touched over `n` bytes.
void ws(const char* what, const char* name, const void* p, size_t n) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  if (!p) return;
  if (a < ws_lo || a + n > ws_hi || a + n < a) {
    fail(what, name, a, n);
    return;
  }
  const std::string key = "pass" + std::to_string(pass) + ":" + name;
  auto it = regions.find(key);
  if (it == regions.end()) regions[key] = {a, a + n};
  else it->second = {std::min(it->second.first, a), std::max(it->second.second, a + n)};
}

// A pointer that may be a caller buffer or (when gathered) inside the workspace.
void maybe_ws(const char* what, const char* name, const void* p, size_t n) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  if (p && a >= ws_lo && a < ws_hi) ws(what, name, p, n);
}

// Named regions of one call must be pairwise disjoint.
int end() {
  for (auto i = regions.begin(); i != regions.end(); ++i)
    for (auto j = std::next(i); j != regions.end(); ++j)
      if (i->second.first < j->second.second && j->second.first < i->second.second) {
        ++violations;
        fprintf(stderr, "VIOLATION overlap: %s [%#lx, %#lx) and %s [%#lx, %#lx)\n", i->first.c_str(),
                (unsigned long)i->second.first, (unsigned long)i->second.second, j->first.c_str(),
                (unsigned long)j->second.first, (unsigned long)j->second.second);
      }
  return violations;
}

int launches = 0;
}  // namespace hoststub

using namespace hoststub;

extern "C" {
const char* hipGetErrorString(hipError_t) { return "hip stub"; }
hipError_t hipMemcpyAsync(void* dst, const void*, size_t n, hipMemcpyKind, hipStream_t) {
  memset(dst, 0, n);  // the status word reads as 0
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
}

namespace flce {

static int eb_of(int dtype) { return dtype == 0 ? 4 : 2; }  // fp32 is dtype 0
int backward_g_grid(int a, int b) { return grouped_grid<kRecXcd>(a, b); }
int backward_dh_grid(int a, int b) { return grouped_grid<kDhXcd>(a, b); }
int backward_dw_grid(int a, int b) { return grouped_grid<kDwXcd>(a, b); }

static char fake_scratch_tag;
hipError_t scratch_address(void** out) {
  // a fake device address; the driver registers [it, it + kScratchBytes) as the workspace
  *out = reinterpret_cast<void*>(uintptr_t(0x7f0000000000ull));
  (void)fake_scratch_tag;
  return hipSuccess;
}

hipError_t launch_forward_tiles(int dtype, bool metrics, bool, bool, const FwdArgs& a, hipStream_t) {
  ++launches;
  maybe_ws("fwd_tiles", "hrows", a.hidden, (size_t)a.N * a.H * eb_of(dtype));
  maybe_ws("fwd_tiles", "tgt", a.targets, (size_t)a.N * 8);
  ws("fwd_tiles", "part", a.part, (size_t)part_fields(metrics, a.zsum != 0) * a.n_splits * a.npad * 4);
  ws("fwd_tiles", "zt", a.zt_rows, (size_t)2 * a.npad * 4);
  if (a.npad < (a.N + 255) / 256 * 256) {
    ++violations;
    fprintf(stderr, "VIOLATION forward row pitch %lld for %lld rows\n", (long long)a.npad, (long long)a.N);
  }
  // the launch covers every split: groups of splits_per_wg
  if (a.splits_per_wg < 1 || (int64_t)a.n_groups * a.splits_per_wg < a.n_splits ||
      (int64_t)(a.n_groups - 1) * a.splits_per_wg >= a.n_splits ||
      (int64_t)a.n_splits * a.tiles_per_split < a.n_voc_tiles ||
      (int64_t)(a.n_splits - 1) * a.tiles_per_split >= a.n_voc_tiles) {
    ++violations;
    fprintf(stderr, "VIOLATION forward plan: %d splits of %d tiles in %d groups of %d, %d tiles\n", a.n_splits,
            a.tiles_per_split, a.n_groups, a.splits_per_wg, a.n_voc_tiles);
  }
  return hipSuccess;
}
hipError_t launch_forward_combine(bool metrics, const CombineArgs& a, hipStream_t) {
  ++launches;
  maybe_ws("combine", "tgt", a.targets, (size_t)a.N * 8);
  ws("combine", "part", a.part, (size_t)part_fields(metrics, a.zsum != 0) * a.n_splits * a.npad * 4);
  ws("combine", "zt", a.zt_rows, (size_t)2 * a.npad * 4);
  ws("combine", "rowloss", a.row_loss, (size_t)a.N * 4);
  ws("combine", "rowent", a.row_ent, (size_t)a.N * 4);
  ws("combine", "rowflag", a.row_flag, (size_t)a.N * 4);
  ws("combine", "roww", a.row_w, (size_t)a.N * 4);
  return hipSuccess;
}
hipError_t launch_forward_reduce(bool, const ReduceArgs& a, hipStream_t) {
  ++launches;
  ws("reduce", "rowloss", a.row_loss, (size_t)a.N * 4);
  ws("reduce", "rowent", a.row_ent, (size_t)a.N * 4);
  ws("reduce", "rowflag", a.row_flag, (size_t)a.N * 4);
  ws("reduce", "roww", a.row_w, (size_t)a.N * 4);
  ws("reduce", "status", a.status, 4);
  ++pass;
  return hipSuccess;
}
hipError_t launch_shard_combine(const ShardCombineArgs& a, hipStream_t) {
  ++launches;
  maybe_ws("shard_combine", "tgt", a.targets, (size_t)a.N * 8);
  ws("shard_combine", "rowloss", a.row_loss, (size_t)a.N * 4);
  ws("shard_combine", "rowflag", a.row_flag, (size_t)a.N * 4);
  ws("shard_combine", "rowent", a.row_ent, (size_t)a.N * 4);
  return hipSuccess;
}
hipError_t launch_backward_prep(const PrepArgs& a, hipStream_t) {
  ++launches;
  maybe_ws("prep", "tgt", a.targets, (size_t)a.N * 8);
  ws("prep", "scale", a.scale, 4);
  return hipSuccess;
}
hipError_t launch_transpose(int dtype, const TransposeArgs& a, hipStream_t) {
  ++launches;
  const int e = eb_of(dtype);
  maybe_ws("transpose", "hrows", a.src, (size_t)a.rows * a.src_ld * e);
  // hidden^T (of the caller's or the gathered hidden rows) or a chunk's W_c^T
  const uintptr_t src = reinterpret_cast<uintptr_t>(a.src);
  const bool hid = a.src == hidden_ptr || (src >= ws_lo && src < ws_hi);
  ws("transpose", hid ? "ht" : "wct", a.dst, (size_t)((a.cols - 1) * a.dst_ld + a.rpad) * e);
  return hipSuccess;
}
static void check_g(int dtype, const GArgs& a) {
  const int e = eb_of(dtype);
  maybe_ws("recompute", "hrows", a.hidden, (size_t)a.N * a.H * e);
  maybe_ws("recompute", "tgt", a.targets, (size_t)a.N * 8);
  ws("recompute", "g", a.G, (size_t)((int64_t)(a.npad - 1) * a.g_ld + a.cvpad) * e);
  ws("recompute", "gt", a.GT, (size_t)a.cvpad * a.npad * e);
  ws("recompute", "wct", a.WcT, (size_t)((a.H - 1) * a.wct_ld + a.cvpad) * e);
  ws("recompute", "db", a.dbpart, (size_t)kBiasParts * a.n_tok_tiles * a.V * 4);
}
static void check_dh(int dtype, const DhArgs& a) {
  const int e = eb_of(dtype);
  ws("grad_hidden", "g", a.G, (size_t)((a.N - 1) * a.ld + a.kdim) * e);
  if (!a.bk) ws("grad_hidden", "wct", a.WcT, (size_t)((a.H - 1) * a.ld + a.kdim) * e);
  ws("grad_hidden", "dh", a.acc, (size_t)a.ksplit * a.acc_stride * 4);
}
static void check_dw(int dtype, const DwArgs& a) {
  const int e = eb_of(dtype);
  if (a.gk) ws("grad_weight", "g", a.GT, (size_t)((int64_t)(a.npad - 1) * a.gld + a.cv) * e);
  else ws("grad_weight", "gt", a.GT, (size_t)a.cv * a.npad * e);
  ws("grad_weight", "ht", a.HT, (size_t)a.H * a.npad * e);
}
hipError_t launch_backward_g(int dtype, bool, bool, const GArgs& a, hipStream_t) {
  ++launches;
  check_g(dtype, a);
  return hipSuccess;
}
hipError_t launch_backward_dh(int dtype, const DhArgs& a, hipStream_t) {
  ++launches;
  check_dh(dtype, a);
  return hipSuccess;
}
hipError_t launch_backward_dh_final(int, const DhFinalArgs& a, hipStream_t) {
  ++launches;
  ws("grad_hidden_sum", "dh", a.acc, (size_t)a.ksplit * a.acc_stride * 4);
  ws("grad_hidden_sum", "scale", a.scale, 4);
  return hipSuccess;
}
hipError_t launch_backward_dw(int dtype, const DwArgs& a, hipStream_t) {
  ++launches;
  check_dw(dtype, a);
  return hipSuccess;
}
hipError_t launch_backward_db(int, const DbArgs& a, hipStream_t) {
  ++launches;
  ws("grad_bias", "db", a.dbpart, (size_t)a.n_parts * a.V * 4);
  ws("grad_bias", "scale", a.scale, 4);
  return hipSuccess;
}
hipError_t launch_backward_step(int dtype, bool, bool, const StepArgs& a, hipStream_t) {
  ++launches;
  if (a.nb_g) check_g(dtype, a.g);
  if (a.nb_dw) check_dw(dtype, a.dw);
  if (a.nb_dh) check_dh(dtype, a.dh);
  return hipSuccess;
}
hipError_t launch_fill_zero(void*, size_t, hipStream_t) {
  ++launches;
  return hipSuccess;
}
hipError_t launch_gather_rows(const GatherRowsArgs& a, hipStream_t) {
  ++launches;
  ws("gather_rows", "hrows", a.dst, (size_t)a.N * a.row_bytes);
  return hipSuccess;
}
hipError_t launch_gather_targets(const GatherTargetsArgs& a, hipStream_t) {
  ++launches;
  ws("gather_targets", "tgt", a.dst, (size_t)a.N * 8);
  return hipSuccess;
}
hipError_t launch_small_forward(bool, const SmallArgs& a, hipStream_t) {
  ++launches;
  maybe_ws("small_fwd", "hrows", a.hidden, (size_t)a.N * a.H * 4);
  maybe_ws("small_fwd", "tgt", a.targets, (size_t)a.N * 8);
  ws("small_fwd", "rowloss", a.row_loss, (size_t)a.N * 4);
  ws("small_fwd", "rowent", a.row_ent, (size_t)a.N * 4);
  ws("small_fwd", "rowflag", a.row_flag, (size_t)a.N * 4);
  ws("small_fwd", "roww", a.row_w, (size_t)a.N * 4);
  return hipSuccess;
}
hipError_t launch_small_backward(const SmallArgs& a, hipStream_t) {
  ++launches;
  maybe_ws("small_bwd", "hrows", a.hidden, (size_t)a.N * a.H * 4);
  maybe_ws("small_bwd", "tgt", a.targets, (size_t)a.N * 8);
  return hipSuccess;
}

}  // namespace flce
