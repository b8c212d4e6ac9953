// Host side of the C ABI in include/pa.h: argument validation, the split planner,
// and kernel dispatch.  Nothing here allocates device memory or synchronises.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <functional>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <tuple>
#include <vector>

#include "pa.h"
#include "pa_internal.hpp"
#include "kv_append.hpp"

using namespace pa;

namespace {

thread_local std::string g_err;

pa_status fail(pa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}
pa_status ok() {
  g_err.clear();
  return PA_OK;
}
pa_status hip_fail(int err, const char* what) {
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString((hipError_t)err));
}

int ilog2_exact(int v) {
  if (v <= 0 || (v & (v - 1))) return -1;
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Enum arguments come from C callers and may hold any int: read them as their int bits
// (loading an out-of-range value as a C++ enum is undefined), and validate before use.
template <class E>
int raw(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "enum arguments are int-sized");
  int v;
  memcpy(&v, &e, sizeof v);
  return v;
}

// Partial outputs of split requests: float32, except with one-byte KV codes (FP8, INT8),
// whose bar (2e-2) leaves room for bf16 partials (2^-9 relative) and half the bytes
// written by stage 1 and read back by the merge.
int partial_o_elem_bytes(int kv_dtype) { return kv_dtype == PA_DTYPE_BF16 ? 4 : 2; }

}  // namespace

namespace pa {
// Tile configurations stage 1 is instantiated for (its dispatcher in stage1.hip uses the
// same list).
bool stage1_cfg_supported(const KernelCfg& c) {
  if (c.qm && (c.kr || c.dh == 512)) return false;
  // keys with a rotary part (stage1_kr.hip): bf16 192/128, or the MLA latent cache 576/512
  // with e4m3 latent codes and e4m3 latent queries; one, two or four 16-row blocks per
  // item, the four waves splitting each tile's tokens between the blocks' teams
  if (c.kr) {
    if ((c.wq != 1 && c.wq != 2 && c.wq != 4) || c.nqb != 1) return false;   // blocks per item
    if (c.mla) return c.dv == 512 && c.dh == 576 && c.qf8 && c.kvf8 && !c.i8;
    return c.dv == 128 && c.dh == 192 && !c.qf8 && !c.kvf8 && !c.pt;
  }
  // head_dim 512: bf16 KV, or per-token-head FP8 KV with bf16 queries; up to four 16-row
  // query blocks (one per wave), one workgroup per CU (its accumulators and query
  // operand need the whole register file of a SIMD)
  if (c.dh == 512)
    return !c.qf8 && !c.i8 && (c.kvf8 ? c.pt : !c.pt) && c.wq == 4 && c.nqb == 1;
  if (c.dh != 128 && c.dh != 256) return false;
  if (c.qm) {
    // query rows on the MFMA M axis (the alternative orientation): bf16 KV, or
    // per-token-head FP8 KV with bf16 queries; not the two tile shapes whose registers
    // would spill (bf16 KV with two query-block waves at head_dim 256, three blocks per
    // wave at head_dim 128)
    if (c.qf8 || c.i8 || (c.kvf8 != c.pt)) return false;
    if (c.nqb == 1 && c.wq == 1) return c.dh == 128;
    if (c.nqb == 1 && c.wq == 2) return c.dh == 128 || c.kvf8;
    if (c.nqb == 1 && c.wq == 4) return true;
    if (c.wq == 4 && c.nqb == 2) return c.dh == 128;
    return c.wq == 4 && c.nqb == 3 && c.dh == 128 && c.kvf8;
  }
  if (c.qf8 && !c.kvf8) return false;
  if (!c.kvf8 && c.pt) return false;
  if (c.i8 && (!c.kvf8 || !c.pt || c.qf8)) return false;    // INT8 KV: bf16 queries, per-token scale path
  const bool pv_fp8 = c.kvf8 && !c.pt;
  if (c.dh == 256 && pv_fp8 && !c.qf8 && c.wq == 2) return false;
  const int nmax = c.dh == 128 ? (pv_fp8 ? 2 : 3) : 1;
  if (c.nqb == 1) return (c.wq == 1 && c.dh == 128) || c.wq == 2 || c.wq == 4;
  return c.wq == 4 && c.nqb >= 2 && c.nqb <= nmax;
}
}  // namespace pa

namespace {

// Tile configuration for the planned shape.
bool choose_cfg(const pa_plan_args& a, KernelCfg* c) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const int mq = a.max_q_len * G;
  const int nqb = (mq + 15) / 16;
  c->dh = a.head_dim;
  c->dv = a.head_dim_v > 0 ? a.head_dim_v : a.head_dim;
  c->qm = a.orientation == PA_ORIENT_Q_ON_M;
  if (c->dv != c->dh) {               // keys with a rotary part: up to four blocks per item
    c->kr = 1;
    c->mla = a.kv_scale_mode == PA_SCALE_PER_TOKEN_BLOCK128;
    c->qf8 = a.q_dtype == PA_DTYPE_FP8_E4M3;
    c->kvf8 = a.kv_dtype != PA_DTYPE_BF16;
    c->i8 = a.kv_dtype == PA_DTYPE_INT8;
    c->pt = c->mla;
    c->wq = nqb <= 1 ? 1 : nqb == 2 ? 2 : 4;     // blocks per item; 4 / wq waves per block
    c->nqb = 1;
    return stage1_cfg_supported(*c);
  }
  c->qf8 = a.q_dtype == PA_DTYPE_FP8_E4M3;
  c->kvf8 = a.kv_dtype != PA_DTYPE_BF16;            // one-byte codes
  c->i8 = a.kv_dtype == PA_DTYPE_INT8;
  // INT8 KV always runs the per-token scale path (bf16 MFMA on upconverted K and V); a
  // per-tensor INT8 scale is read through zero scale strides
  c->pt = a.kv_scale_mode == PA_SCALE_PER_TOKEN_HEAD || c->i8;
  // head_dim 256 with one query block: 64-token tiles (two token groups of two waves)
  // keep two LDS stages; 128-token tiles of d256 would fit only one
  // head_dim 512 and 256 run one 16-row block per wave; a request with more than four
  // blocks per KV head is cut into groups of four, one work item per (group, KV split)
  // (at head_dim 256 two blocks per wave would need more than the 256 registers a wave
  // has at two workgroups per CU).  For head_dim 128 the waves take several blocks each
  // instead: groups measured slower on the ragged group-24 workload, 124 -> 132 us,
  // since every group re-reads the split's K and V.
  const bool d256_bf16q_pt8 = c->dh == 256 && c->kvf8 && !c->pt && !c->qf8;   // no two-wave variant
  if (c->dh == 512 || (c->dh == 256 && nqb > 4)) { c->wq = 4; c->nqb = 1; }
  else if (nqb <= 1) { c->wq = c->dh == 256 ? (d256_bf16q_pt8 ? 4 : 2) : 1; c->nqb = 1; }
  else if (nqb == 2) { c->wq = d256_bf16q_pt8 ? 4 : 2; c->nqb = 1; }
  else if (nqb <= 4) { c->wq = 4; c->nqb = 1; }
  else { c->wq = 4; c->nqb = (nqb + 3) / 4; }
  return stage1_cfg_supported(*c);
}

// Query-block groups of request b: its rows x heads in 16-row blocks, cut into runs of
// the blocks one workgroup covers (waves x blocks per wave).
int query_groups(const pa_plan_args& a, const KernelCfg& cfg, int b) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const int nb16 = ((a.qo_indptr[b + 1] - a.qo_indptr[b]) * G + 15) / 16;
  const int per = cfg.wq * cfg.nqb;
  return (nb16 + per - 1) / per;
}

// ---- split-count cost model --------------------------------------------------------
// Every CU holds two stage-1 workgroups at once (the kernels' LDS and register
// budgets are sized for that), and a CU running only one of them leaves its memory
// pipeline half idle.  So the model schedules items onto 2 x num_cus slots, each with
// half of a CU's share of the HBM bandwidth.  An item costs the larger of its KV
// streaming time and its compute time (which grows with the number of 16-row query
// blocks each wave runs per token), plus its partial-output write when the request is
// split, plus a fixed prologue.  Items are placed longest-first on the least loaded
// slot; the merge reads every partial back.  The candidate split plan with the smallest
// estimated step time wins (ties go to fewer, longer splits).
constexpr double kHbmBytesPerS = 6.5e12;     // MI355X HBM3E, sustained streaming rate
constexpr int kSlotsPerCu = 2;
constexpr double kItemOverheadS = 1.5e-6;    // item prologue + pipeline fill
constexpr double kMergeBytesPerS = 4.0e12;   // partials are re-read from the last-level cache
constexpr double kMergeLaunchS = 3.0e-6;
// Workgroup p of a launch runs on XCD p mod 8.  Measured with per-workgroup timelines
// (equal items, random pages, one round): the odd-numbered XCDs stream KV about 10%
// slower than the even ones (c3 161 against 145 us, c4 R1 340 against 309 us, median
// finish per XCD, on three machines); compute-bound items differ by 2-3%.
constexpr int kXcds = 8;
constexpr double kOddXcdStreamRate = 0.9;

// Seconds of compute per KV token for one 16-row query block per wave, one workgroup
// in a slot, by head_dim and KV format (measured with the KV loads switched off; for
// per-token scales the constant that planned the ragged group-24 mix fastest: 14, 18, 22
// and 28 ns gave 128.5, 138.6, 119 and 118.5 us of stage 1 -- its three-block waves
// cost more per block than the one-block shapes the first figure came from).
// Keys with a rotary part: the latent-cache kernel computes about 64 ns per token and
// workgroup with its four waves on one block (all loads served from cache: 33 us for the
// 512-token items of the latent workload), i.e. 256 ns per 16-row block for one wave; the
// 192/128 kernel is bound by its loads (20 ns).  The planned split counts of both
// workloads measured best in forced-split sweeps.
double compute_s_per_token_block(const pa_plan_args& a) {
  if (a.head_dim_v > 0 && a.head_dim_v != a.head_dim)      // keys with a rotary part
    return (a.kv_scale_mode == PA_SCALE_PER_TOKEN_BLOCK128 ? 256.0 : 20.0) * 1e-9;
  const bool f8 = a.kv_dtype != PA_DTYPE_BF16;
  const bool pt = a.kv_scale_mode == PA_SCALE_PER_TOKEN_HEAD || a.kv_dtype == PA_DTYPE_INT8;
  const double d_scale = a.head_dim / 128.0;
  double ns;
  if (!f8) ns = 16.0;            // two-term bf16 P
  else if (pt) ns = 22.0;        // fp8 -> bf16 upconversion of K and V, per-token scales
  else ns = 8.0;                 // fp8 MFMA for both products
  return ns * d_scale * 1e-9;
}

// Per-request item costs of the split model.
struct CostModel {
  int slots = 0;
  double bw_slot = 0, kv_tok = 0;
  std::vector<double> comp_tok;                  // compute seconds per token of request b's items
  std::vector<double> part;                      // partial-output bytes one item of b writes when split
  std::vector<int> ngrp;                         // query-block groups (items per split and KV head)
  // Seconds of one item of request b over tok tokens: its KV bytes (plus its partial
  // output when the request is split) at the slot's share of HBM, or its compute,
  // whichever is longer, plus a fixed prologue.
  double item_cost(int b, double tok, bool split) const {
    const double mem = (tok * kv_tok + (split ? part[b] : 0.0)) / bw_slot;
    return std::max(mem, tok * comp_tok[b]) + kItemOverheadS;
  }
};

CostModel cost_model(const pa_plan_args& a, const KernelCfg& cfg, int num_cus) {
  CostModel m;
  const int B = a.batch;
  const int G = a.num_q_heads / a.num_kv_heads;
  m.kv_tok = 2.0 * a.head_dim * (a.kv_dtype != PA_DTYPE_BF16 ? 1 : 2) +
             (a.kv_scale_mode == PA_SCALE_PER_TOKEN_HEAD ? 8 : 0);
  if (cfg.kr)                           // key rows of dh channels, value rows of dv (MLA: shared)
    m.kv_tok = cfg.mla ? cfg.dv + 2.0 * 64 + 4.0 * cfg.dv / 128 : 2.0 * (cfg.dh + cfg.dv);
  // head_dim 512 and the latent cache with four query blocks per item: one workgroup per
  // CU (registers, LDS)
  m.slots = (cfg.dh == 512 || (cfg.mla && cfg.wq == 4) ? 1 : kSlotsPerCu) * num_cus;
  m.bw_slot = kHbmBytesPerS / m.slots;
  const int wt = 4 / cfg.wq;                     // waves sharing the tokens of a tile
  const double comp_blk = compute_s_per_token_block(a);
  m.comp_tok.resize(B);
  m.part.resize(B);
  m.ngrp.resize(B);
  for (int b = 0; b < B; ++b) {
    const int n = a.qo_indptr[b + 1] - a.qo_indptr[b];
    const int nb16 = (n * G + 15) / 16;
    m.ngrp[b] = query_groups(a, cfg, b);
    const int per_item = std::min(nb16, cfg.wq * cfg.nqb);
    const int rounds = (per_item + cfg.wq - 1) / cfg.wq;
    m.comp_tok[b] = comp_blk * rounds / wt;
    m.part[b] = (double)std::min(n * G, 16 * per_item) * (cfg.dv * partial_o_elem_bytes(a.kv_dtype) + 4.0);
  }
  return m;
}

void choose_splits(const pa_plan_args& a, const CostModel& cm, const std::vector<int>& span, int split_cap,
                   std::vector<int>* nsp) {
  const int B = a.batch;
  const int slots = cm.slots;
  // Split counts: every request's items should cost about the same, so a request whose
  // tokens are more expensive (more 16-row query blocks per wave: compute-bound) is cut
  // into shorter splits than a memory-bound one.  The candidates are the item costs
  // C = W_max / S, S = 1, 2, ..., where W_max is the cost of the heaviest request's whole
  // range; request b then gets ceil(W_b / C) splits (at most its 64-token blocks and the
  // cap).  On uniform batches this is the same as cutting every request into equal runs.
  std::vector<int> nblk(B);
  std::vector<double> ctok(B);                   // seconds per token of request b's items
  double heavy = 0;
  int heavy_b = 0;
  for (int b = 0; b < B; ++b) {
    nblk[b] = std::max(1, (span[b] + kSplitAlign - 1) / kSplitAlign);
    ctok[b] = std::max(cm.kv_tok / cm.bw_slot, cm.comp_tok[b]);
    const double wb = (double)span[b] * ctok[b] * cm.ngrp[b];
    if (wb > heavy) {
      heavy = wb;
      heavy_b = b;
    }
  }
  const int s_heavy = std::max(1, std::min(split_cap, nblk[heavy_b]));
  std::vector<int> best(B, 1), cur(B), prev;
  double best_t = 1e30;
  std::vector<std::pair<double, int>> groups;       // (item cost, item count)
  std::vector<double> heap;
  // Fewest splits first, so that an equal estimate keeps the plan with fewer splits.  A
  // candidate whose lower bound -- its work spread evenly over the CUs, or its longest
  // item, plus its merge -- cannot beat the best estimate so far is not scheduled at all.
  for (int S = 1; S <= s_heavy; ++S) {
    const double target = heavy / S;
    for (int b = 0; b < B; ++b) {
      const double wb = (double)span[b] * ctok[b] * cm.ngrp[b];
      const int sb = (int)std::ceil(wb / target * (1 - 1e-12));
      cur[b] = std::max(1, std::min(sb, std::min(split_cap, nblk[b])));
    }
    if (cur == prev) continue;
    prev = cur;
    groups.clear();
    double merge_bytes = 0, total = 0, longest = 0;
    for (int b = 0; b < B; ++b) {
      const int sb = cur[b];
      const double cost = cm.item_cost(b, (double)span[b] / sb, sb > 1);
      const int count = sb * a.num_kv_heads * cm.ngrp[b];
      groups.push_back({cost, count});
      if (sb > 1) merge_bytes += cm.part[b] * count;
      total += cost * count;
      longest = std::max(longest, cost);
    }
    const double merge_t = merge_bytes > 0 ? merge_bytes / kMergeBytesPerS + kMergeLaunchS : 0.0;
    if (std::max(total / slots, longest) + merge_t >= best_t * (1 - 1e-9)) continue;
    std::sort(groups.begin(), groups.end(), [](const auto& x, const auto& y) { return x.first > y.first; });
    heap.assign(slots, 0.0);                         // min-heap of slot loads
    for (const auto& gi : groups) {
      for (int k = 0; k < gi.second; ++k) {
        std::pop_heap(heap.begin(), heap.end(), std::greater<double>());
        heap.back() += gi.first;
        std::push_heap(heap.begin(), heap.end(), std::greater<double>());
      }
    }
    const double t = *std::max_element(heap.begin(), heap.end()) + merge_t;
    if (t < best_t * (1 - 1e-9)) {
      best_t = t;
      best = cur;
    }
  }
  *nsp = best;
}

}  // namespace

namespace pa {
// Error reporting for entry points defined in other source files (same message slot
// that pa_last_error returns).
int report_error(int st, const char* msg) {
  if (st == PA_OK) return (int)ok();
  return (int)fail((pa_status)st, "%s", msg);
}
}  // namespace pa

extern "C" {

const char* pa_last_error(void) { return g_err.c_str(); }

const char* pa_version(void) { return "paged_split_kv_stage1_amd 0.1 (gfx950)"; }

pa_status pa_plan_splits(const pa_plan_args* a, void* plan_host, size_t plan_capacity, pa_plan_info* info) {
  if (!a || !info) return fail(PA_ERR_INVALID_ARGUMENT, "pa_plan_splits: args and info must be non-NULL");
  const int B = a->batch;
  if (B < 1) return fail(PA_ERR_INVALID_ARGUMENT, "batch must be >= 1 (got %d)", B);
  if (!a->qo_indptr || !a->kv_indptr || !a->kv_len)
    return fail(PA_ERR_INVALID_ARGUMENT, "qo_indptr, kv_indptr and kv_len must be non-NULL host arrays");
  if (a->max_q_len < 1) return fail(PA_ERR_INVALID_ARGUMENT, "max_q_len must be >= 1 (got %d)", a->max_q_len);
  if (a->max_q_len > 8)
    return fail(PA_ERR_UNSUPPORTED, "max_q_len %d: at most 8 query rows per request are supported", a->max_q_len);
  if (a->num_q_heads < 1 || a->num_kv_heads < 1 || a->num_q_heads % a->num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                a->num_q_heads, a->num_kv_heads);
  const int dv = a->head_dim_v > 0 ? a->head_dim_v : a->head_dim;
  if (a->head_dim_v < 0) return fail(PA_ERR_INVALID_ARGUMENT, "head_dim_v must be >= 0");
  if (dv == a->head_dim && a->head_dim != 128 && a->head_dim != 256 && a->head_dim != 512)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d: only 128, 256 and 512 are supported", a->head_dim);
  if (dv != a->head_dim && !((a->head_dim == 192 && dv == 128) || (a->head_dim == 576 && dv == 512)))
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d with head_dim_v %d: separate key and value widths are supported "
                                    "as 192/128 and 576/512 (keys with a 64-channel rotary part)", a->head_dim, dv);
  const int page_shift = ilog2_exact(a->page_size);
  if (page_shift < 4 || a->page_size > 1024)
    return fail(PA_ERR_UNSUPPORTED, "page_size %d: must be a power of two in [16, 1024]", a->page_size);
  const int qd = raw(a->q_dtype), kd = raw(a->kv_dtype), sm = raw(a->kv_scale_mode);
  if (qd != PA_DTYPE_BF16 && qd != PA_DTYPE_FP8_E4M3)
    return fail(PA_ERR_INVALID_ARGUMENT, "q_dtype must be BF16 or FP8_E4M3");
  if (kd != PA_DTYPE_BF16 && kd != PA_DTYPE_FP8_E4M3 && kd != PA_DTYPE_INT8)
    return fail(PA_ERR_INVALID_ARGUMENT, "kv_dtype must be BF16, FP8_E4M3 or INT8");
  if (kd == PA_DTYPE_BF16 && sm != PA_SCALE_NONE)
    return fail(PA_ERR_INVALID_ARGUMENT, "bf16 KV takes kv_scale_mode NONE");
  if (kd == PA_DTYPE_FP8_E4M3 && sm != PA_SCALE_PER_TENSOR && sm != PA_SCALE_PER_HEAD &&
      sm != PA_SCALE_PER_TOKEN_HEAD && sm != PA_SCALE_PER_TOKEN_BLOCK128)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "FP8 KV takes kv_scale_mode PER_TENSOR, PER_HEAD, PER_TOKEN_HEAD or PER_TOKEN_BLOCK128");
  if ((sm == PA_SCALE_PER_TOKEN_BLOCK128) != (a->head_dim == 576 && dv == 512))
    return fail(PA_ERR_UNSUPPORTED, "PER_TOKEN_BLOCK128 scales are the latent cache of 576/512 keys/values "
                                    "(and that cache takes no other mode)");
  if (dv != a->head_dim && dv == 128 && (qd != PA_DTYPE_BF16 || kd != PA_DTYPE_BF16))
    return fail(PA_ERR_UNSUPPORTED, "192/128 keys/values take bf16 queries and a bf16 cache");
  if (sm == PA_SCALE_PER_TOKEN_BLOCK128 && qd != PA_DTYPE_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "the latent cache takes e4m3 latent queries (with bf16 rotary parts)");
  if (kd == PA_DTYPE_INT8 && sm != PA_SCALE_PER_TENSOR &&
      sm != PA_SCALE_PER_TOKEN_HEAD)
    return fail(PA_ERR_INVALID_ARGUMENT, "INT8 KV takes kv_scale_mode PER_TENSOR or PER_TOKEN_HEAD");
  if (qd == PA_DTYPE_FP8_E4M3 && kd != PA_DTYPE_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "FP8 queries need an FP8 KV cache");
  if (a->max_splits < 0 || a->force_splits < 0 || a->num_cus < 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_splits, force_splits and num_cus must be >= 0");
  const int split_cap = a->max_splits > 0 ? std::min(a->max_splits, kMaxSplits) : kMaxSplits;
  if (a->force_splits > split_cap)
    return fail(PA_ERR_INVALID_ARGUMENT, "force_splits %d exceeds the split cap %d", a->force_splits, split_cap);

  if (a->orientation != PA_ORIENT_KV_ON_M && a->orientation != PA_ORIENT_Q_ON_M)
    return fail(PA_ERR_INVALID_ARGUMENT, "orientation must be PA_ORIENT_KV_ON_M or PA_ORIENT_Q_ON_M (got %d)",
                a->orientation);
  KernelCfg cfg;
  if (!choose_cfg(*a, &cfg) && cfg.qm)
    return fail(PA_ERR_UNSUPPORTED, "query rows on the MFMA M axis are built for bf16 KV and per-token-head FP8 KV "
                                    "with bf16 queries at head_dim 128/256, except bf16 KV at head_dim 256 with at "
                                    "most 32 and at head_dim 128 with more than 128 query rows x heads per KV head");
  if (!choose_cfg(*a, &cfg))
    return fail(PA_ERR_UNSUPPORTED, "max_q_len x group = %d query rows per KV head is beyond the tile limit "
                                    "for head_dim %d and this dtype combination",
                a->max_q_len * (a->num_q_heads / a->num_kv_heads), a->head_dim);

  // ---- validate the index arrays ------------------------------------------------
  if (a->qo_indptr[0] != 0) return fail(PA_ERR_INVALID_ARGUMENT, "qo_indptr[0] must be 0");
  for (int b = 0; b < B; ++b) {
    const int n = a->qo_indptr[b + 1] - a->qo_indptr[b];
    if (n < 1 || n > a->max_q_len)
      return fail(PA_ERR_INVALID_ARGUMENT, "request %d has %d query rows (must be 1..max_q_len=%d)", b, n,
                  a->max_q_len);
    const int L = a->kv_len[b];
    if (L < n) return fail(PA_ERR_INVALID_ARGUMENT, "request %d: kv_len %d < its %d query rows", b, L, n);
    const int64_t pages = ((int64_t)L + a->page_size - 1) / a->page_size;
    if ((int64_t)a->kv_indptr[b + 1] - a->kv_indptr[b] != pages)
      return fail(PA_ERR_INVALID_ARGUMENT, "request %d: kv_indptr spans %d pages but kv_len %d needs %lld", b,
                  a->kv_indptr[b + 1] - a->kv_indptr[b], L, (long long)pages);
    if (a->kv_indptr[b] < 0) return fail(PA_ERR_INVALID_ARGUMENT, "kv_indptr[%d] is negative", b);
    if (a->window && a->window[b] < 0)
      return fail(PA_ERR_INVALID_ARGUMENT, "request %d: window %d is negative", b, a->window[b]);
  }
  const int T = a->qo_indptr[B];
  const int Hkv = a->num_kv_heads;

  int num_cus = a->num_cus;
  if (num_cus == 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "pa_plan_splits: hipGetDevice");
    e = hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "pa_plan_splits: hipDeviceGetAttribute");
  }

  // ---- split plan -------------------------------------------------------------------
  // Each request's visible token range [lo_b, L_b) (union over its rows) is aligned
  // down to a multiple of 64 tokens and cut into S_b equal runs of 64-token blocks.
  std::vector<int> begin(B), span(B), nsp(B);
  int64_t total_tok = 0;
  for (int b = 0; b < B; ++b) {
    const int n = a->qo_indptr[b + 1] - a->qo_indptr[b];
    const int L = a->kv_len[b];
    const int W = a->window ? a->window[b] : 0;
    const int lo = W > 0 ? std::max(0, L - n - W + 1) : 0;
    begin[b] = (lo / kSplitAlign) * kSplitAlign;
    span[b] = L - begin[b];
    total_tok += (int64_t)span[b] * Hkv;
  }
  const CostModel cm = cost_model(*a, cfg, num_cus);
  if (a->force_splits > 0) {
    for (int b = 0; b < B; ++b) nsp[b] = a->force_splits;
  } else {
    choose_splits(*a, cm, span, split_cap, &nsp);
  }
  int s_max = 1;
  int64_t n_items = 0;
  for (int b = 0; b < B; ++b) {
    s_max = std::max(s_max, nsp[b]);
    n_items += (int64_t)nsp[b] * Hkv * query_groups(*a, cfg, b);
  }
  if (n_items > 0x7fffffff) return fail(PA_ERR_UNSUPPORTED, "too many work items (%lld)", (long long)n_items);
  // split s of request b covers 64-token blocks [s * nblk / S, (s + 1) * nblk / S) from begin[b]
  auto split_range = [&](int b, int s, int* t0, int* t1) {
    const int L = a->kv_len[b];
    const int nblk = (span[b] + kSplitAlign - 1) / kSplitAlign;
    const int64_t blk0 = (int64_t)s * nblk / nsp[b];
    const int64_t blk1 = (int64_t)(s + 1) * nblk / nsp[b];
    *t0 = (int)std::min<int64_t>(begin[b] + blk0 * kSplitAlign, L);
    *t1 = (int)std::min<int64_t>(begin[b] + blk1 * kSplitAlign, L);
  };
  // ---- emit work items, heaviest first ----------------------------------------------
  std::vector<PaItem> items;
  items.reserve((size_t)n_items);
  for (int b = 0; b < B; ++b) {
    const int n = a->qo_indptr[b + 1] - a->qo_indptr[b];
    const int L = a->kv_len[b];
    const int ng = query_groups(*a, cfg, b);
    for (int g = 0; g < Hkv; ++g) {
      for (int s = 0; s < nsp[b]; ++s) {
        for (int qg = 0; qg < ng; ++qg) {
          PaItem it;
          memset(&it, 0, sizeof it);
          it.row0 = a->qo_indptr[b];
          it.nrows = n;
          it.kv_len = L;
          it.page_base = a->kv_indptr[b];
          it.window = a->window ? a->window[b] : 0;
          it.kvh = g;
          it.split = s;
          it.nsplit = nsp[b];
          split_range(b, s, &it.tok_begin, &it.tok_end);
          it.req = b;
          it.qblk0 = qg * cfg.wq * cfg.nqb;
          items.push_back(it);
        }
      }
    }
  }
  // heaviest first: workgroups are dispatched in order to whichever slot frees up first,
  // which makes the launch a longest-first list schedule.  The weight is tokens x (a fixed
  // cost + the item's own rows x heads): on the ragged group-24 mix this order measured
  // 119 us of stage 1 against 137 us when ordered by the split model's item cost.
  const int G = a->num_q_heads / Hkv;
  const int rows_per_item = 16 * cfg.wq * cfg.nqb;
  auto weight = [G, rows_per_item](const PaItem& x) {
    const int m = std::min(x.nrows * G - 16 * x.qblk0, rows_per_item);
    return (int64_t)(x.tok_end - x.tok_begin) * (64 + m);
  };
  std::stable_sort(items.begin(), items.end(),
                   [&weight](const PaItem& x, const PaItem& y) { return weight(x) > weight(y); });
  // One round (every item has its own workgroup slot): the splits of each memory-bound
  // range are cut in proportion to the streaming rate of the XCD their position lands on,
  // so that the odd XCDs' shorter items end with the even XCDs' longer ones (equal-width
  // kernel: c3 175 -> 172.5 us, c3 R1 171 -> 167.6, c4 R1 342.5 -> 338; the 192/128
  // kernel measured 0.6% slower with it and keeps equal splits).
  if (n_items <= cm.slots && cm.slots % (2 * kXcds) == 0 && a->force_splits == 0 && !cfg.kr) {
    // item positions grouped by range (request, KV head, query-block group)
    std::vector<std::pair<std::tuple<int, int, int>, int>> keyed;
    keyed.reserve(items.size());
    for (int p = 0; p < (int)items.size(); ++p) {
      const PaItem& x = items[p];
      keyed.push_back({std::make_tuple(x.req, x.kvh, x.qblk0), p});
    }
    std::stable_sort(keyed.begin(), keyed.end());
    for (size_t i = 0; i < keyed.size();) {
      size_t j = i;
      while (j < keyed.size() && keyed[j].first == keyed[i].first) ++j;
      const int b = items[keyed[i].second].req;
      const bool mem_bound = cm.kv_tok / cm.bw_slot >= cm.comp_tok[b];
      const int S = nsp[b];
      if (mem_bound && S > 1 && (int)(j - i) == S) {
        std::vector<int> at(S);                  // position of split s
        for (size_t k = i; k < j; ++k) at[items[keyed[k].second].split] = keyed[k].second;
        const int nblk = (span[b] + kSplitAlign - 1) / kSplitAlign;
        double wsum = 0;
        for (int sp = 0; sp < S; ++sp) wsum += (at[sp] % 2) ? kOddXcdStreamRate : 1.0;
        double acc = 0;
        int blk_prev = 0;
        for (int sp = 0; sp < S; ++sp) {
          acc += (at[sp] % 2) ? kOddXcdStreamRate : 1.0;
          int blk = sp + 1 == S ? nblk : (int)std::lround(nblk * acc / wsum);
          blk = std::max(blk, blk_prev + 1);
          blk = std::min(blk, nblk - (S - 1 - sp));
          PaItem& x = items[at[sp]];
          x.tok_begin = (int)std::min<int64_t>(begin[b] + (int64_t)blk_prev * kSplitAlign, x.kv_len);
          x.tok_end = (int)std::min<int64_t>(begin[b] + (int64_t)blk * kSplitAlign, x.kv_len);
          blk_prev = blk;
        }
      }
      i = j;
    }
  }
  int64_t max_item_tokens = 0;
  for (const PaItem& x : items) max_item_tokens = std::max<int64_t>(max_item_tokens, x.tok_end - x.tok_begin);
  const int64_t th_count = (int64_t)T * a->num_q_heads;

  memset(info, 0, sizeof *info);
  info->batch = B;
  info->total_rows = T;
  info->num_q_heads = a->num_q_heads;
  info->num_kv_heads = Hkv;
  info->head_dim = a->head_dim;
  info->head_dim_v = dv;
  info->page_size = a->page_size;
  info->max_q_len = a->max_q_len;
  info->q_dtype = a->q_dtype;
  info->kv_dtype = a->kv_dtype;
  info->kv_scale_mode = a->kv_scale_mode;
  info->num_items = (int32_t)n_items;
  info->max_splits = s_max;
  info->needs_merge = s_max > 1;
  info->num_cus = num_cus;
  info->variant = pack_cfg(cfg);
  info->plan_bytes = plan_bytes_for(n_items, T);
  info->partial_o_bytes = s_max > 1 ? th_count * s_max * dv * partial_o_elem_bytes(a->kv_dtype) : 0;
  info->partial_lse_bytes = s_max > 1 ? th_count * s_max * 4 : 0;
  info->max_item_tokens = max_item_tokens;
  if (!plan_host) return ok();
  if ((int64_t)plan_capacity < info->plan_bytes)
    return fail(PA_ERR_INSUFFICIENT_WORKSPACE, "plan buffer holds %zu bytes, %lld needed", plan_capacity,
                (long long)info->plan_bytes);

  uint8_t* out = static_cast<uint8_t*>(plan_host);
  memcpy(out, items.data(), items.size() * sizeof(PaItem));
  int32_t* row_ns = reinterpret_cast<int32_t*>(out + items.size() * sizeof(PaItem));
  for (int b = 0; b < B; ++b)
    for (int t = a->qo_indptr[b]; t < a->qo_indptr[b + 1]; ++t) row_ns[t] = nsp[b];
  return ok();
}

pa_status pa_decode_stage1(const pa_plan_info* info, const void* plan_dev, const void* q, const float* q_scale,
                           const void* k_cache, const void* v_cache, const pa_kv_layout* kv, const float* k_scale,
                           const float* v_scale, const pa_scale_layout* sc, const int32_t* page_indices,
                           float sm_scale, void* partial_o, float* partial_lse, void* out, pa_dtype out_dtype,
                           float* out_lse, void* stream) {
  if (!info || !plan_dev || !q || !k_cache || !v_cache || !kv || !page_indices || !out)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_stage1: a required pointer is NULL");
  if (raw(out_dtype) != PA_DTYPE_BF16 && raw(out_dtype) != PA_DTYPE_FP32)
    return fail(PA_ERR_INVALID_ARGUMENT, "out_dtype must be BF16 or FP32");
  const KernelCfg cfg = unpack_cfg(info->variant);
  if (!stage1_cfg_supported(cfg) || cfg.dh != info->head_dim)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_plan_info was not produced by pa_plan_splits");
  if (cfg.kr)
    return fail(PA_ERR_INVALID_ARGUMENT, "this plan has keys wider than values: use pa_decode_stage1_rope");
  if (info->needs_merge && (!partial_o || !partial_lse))
    return fail(PA_ERR_INVALID_ARGUMENT, "this plan has several splits: partial_o and partial_lse are required");
  if (cfg.qf8 && !q_scale) return fail(PA_ERR_INVALID_ARGUMENT, "FP8 queries need q_scale");
  if (cfg.kvf8 && (!k_scale || !v_scale))
    return fail(PA_ERR_INVALID_ARGUMENT, "FP8 and INT8 KV need k_scale and v_scale");
  const bool per_token = info->kv_scale_mode == PA_SCALE_PER_TOKEN_HEAD;
  if (per_token && !sc) return fail(PA_ERR_INVALID_ARGUMENT, "per-token-head scales need a scale layout");
  const int esz = cfg.kvf8 ? 1 : 2;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(q) || !aligned16(out))
    return fail(PA_ERR_INVALID_ARGUMENT, "q, k_cache, v_cache and out must be 16-byte aligned");
  if ((kv->page * esz) % 16 || (kv->head * esz) % 16 || (kv->slot * esz) % 16 || kv->page < 0 || kv->head < 0 ||
      kv->slot < 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "KV strides must be non-negative multiples of 16 bytes");
  if (info->needs_merge && (((uintptr_t)partial_o & 15u) != 0))
    return fail(PA_ERR_INVALID_ARGUMENT, "partial_o must be 16-byte aligned");
  const int ps = ilog2_exact(info->page_size);
  Stage1Args s;
  memset(&s, 0, sizeof s);
  s.items = static_cast<const PaItem*>(plan_dev);
  s.q = q;
  s.q_scale = q_scale;
  s.k = k_cache;
  s.v = v_cache;
  s.kv_sp = kv->page;
  s.kv_sh = kv->head;
  s.kv_ss = kv->slot;
  s.k_scale = k_scale;
  s.v_scale = v_scale;
  s.scale_per_head = info->kv_scale_mode == PA_SCALE_PER_HEAD;
  if (per_token) {          // (per-tensor INT8 runs the per-token path with all strides 0)
    s.sc_sp = sc->page;
    s.sc_sh = sc->head;
    s.sc_ss = sc->slot;
  }
  s.page_indices = page_indices;
  s.sm_scale = sm_scale;
  s.partial_o = partial_o;
  s.partial_lse = partial_lse;
  s.part_bf16 = partial_o_elem_bytes(info->kv_dtype) == 2;
  s.out = out;
  s.out_bf16 = out_dtype == PA_DTYPE_BF16;
  s.out_lse = out_lse;
  s.hq = info->num_q_heads;
  s.group = info->num_q_heads / info->num_kv_heads;
  s.page_shift = ps;
  s.s_max = info->max_splits;
  s.fair = info->num_items <= kSlotsPerCu * info->num_cus;
  const int e = launch_stage1(cfg, s, info->num_items, stream);
  if (e) return hip_fail(e, "pa_decode_stage1 launch");
  return ok();
}

pa_status pa_decode_stage1_rope(const pa_plan_info* info, const void* plan_dev, const void* q, const float* q_scale,
                                const void* q_rope, const void* k_cache, const pa_kv_layout* k_layout,
                                const void* k_rope, const pa_kv_layout* k_rope_layout, const float* k_scale,
                                const pa_kv_layout* k_scale_layout, const void* v_cache, const pa_kv_layout* v_layout,
                                const int32_t* page_indices, float sm_scale, void* partial_o, float* partial_lse,
                                void* out, pa_dtype out_dtype, float* out_lse, void* stream) {
  if (!info || !plan_dev || !q || !k_cache || !k_layout || !page_indices || !out)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_stage1_rope: a required pointer is NULL");
  if (raw(out_dtype) != PA_DTYPE_BF16 && raw(out_dtype) != PA_DTYPE_FP32)
    return fail(PA_ERR_INVALID_ARGUMENT, "out_dtype must be BF16 or FP32");
  const KernelCfg cfg = unpack_cfg(info->variant);
  if (!stage1_cfg_supported(cfg) || !cfg.kr || cfg.dh != info->head_dim)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_stage1_rope needs a plan with keys wider than values");
  if (info->needs_merge && (!partial_o || !partial_lse))
    return fail(PA_ERR_INVALID_ARGUMENT, "this plan has several splits: partial_o and partial_lse are required");
  if (cfg.mla && (!q_scale || !q_rope || !k_rope || !k_rope_layout || !k_scale || !k_scale_layout))
    return fail(PA_ERR_INVALID_ARGUMENT, "the latent cache needs q_scale, q_rope, k_rope and k_scale with layouts");
  if (!cfg.mla && (!v_cache || !v_layout))
    return fail(PA_ERR_INVALID_ARGUMENT, "192/128 keys/values need v_cache and v_layout");
  const bool ok_align = aligned16(q) && aligned16(k_cache) && aligned16(out) && (!q_rope || aligned16(q_rope)) &&
                        (!k_rope || aligned16(k_rope)) && (!v_cache || aligned16(v_cache)) &&
                        (!info->needs_merge || aligned16(partial_o));
  if (!ok_align) return fail(PA_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
  auto strides_ok = [](const pa_kv_layout* l, int esz) {
    return l->page >= 0 && l->head >= 0 && l->slot >= 0 && (l->page * esz) % 16 == 0 && (l->head * esz) % 16 == 0 &&
           (l->slot * esz) % 16 == 0;
  };
  if (!strides_ok(k_layout, cfg.mla ? 1 : 2) || (cfg.mla && !strides_ok(k_rope_layout, 2)) ||
      (!cfg.mla && !strides_ok(v_layout, 2)))
    return fail(PA_ERR_INVALID_ARGUMENT, "cache strides must be non-negative multiples of 16 bytes");
  if (cfg.mla && (k_scale_layout->page < 0 || k_scale_layout->head < 0 || k_scale_layout->slot < 0))
    return fail(PA_ERR_INVALID_ARGUMENT, "scale strides must be non-negative");
  KrArgs s;
  memset(&s, 0, sizeof s);
  s.items = static_cast<const PaItem*>(plan_dev);
  s.q = q;
  s.q_scale = q_scale;
  s.q_rope = q_rope;
  s.k_main = k_cache;
  s.m_sp = k_layout->page; s.m_sh = k_layout->head; s.m_ss = k_layout->slot;
  if (cfg.mla) {
    s.k_rope = k_rope;
    s.r_sp = k_rope_layout->page; s.r_sh = k_rope_layout->head; s.r_ss = k_rope_layout->slot;
    s.k_scale = k_scale;
    s.s_sp = k_scale_layout->page; s.s_sh = k_scale_layout->head; s.s_ss = k_scale_layout->slot;
  } else {                            // the rotary channels are the last 64 of each key row
    s.k_rope = static_cast<const uint8_t*>(k_cache) + 2 * cfg.dv;
    s.r_sp = s.m_sp; s.r_sh = s.m_sh; s.r_ss = s.m_ss;
    s.v = v_cache;
    s.v_sp = v_layout->page; s.v_sh = v_layout->head; s.v_ss = v_layout->slot;
  }
  s.page_indices = page_indices;
  s.sm_scale = sm_scale;
  s.partial_o = partial_o;
  s.partial_lse = partial_lse;
  s.part_bf16 = partial_o_elem_bytes(info->kv_dtype) == 2;
  s.out = out;
  s.out_bf16 = raw(out_dtype) == PA_DTYPE_BF16;
  s.out_lse = out_lse;
  s.hq = info->num_q_heads;
  s.group = info->num_q_heads / info->num_kv_heads;
  s.page_shift = ilog2_exact(info->page_size);
  s.s_max = info->max_splits;
  s.fair = info->num_items <= kSlotsPerCu * info->num_cus;
  const int e = cfg.mla ? launch_stage1_mla(cfg.wq, s, info->num_items, stream)
                        : launch_stage1_kr(cfg.dv, cfg.wq, s, info->num_items, stream);
  if (e) return hip_fail(e, "pa_decode_stage1_rope launch");
  return ok();
}

pa_status pa_decode_merge(const pa_plan_info* info, const void* plan_dev, const void* partial_o,
                          const float* partial_lse, void* out, pa_dtype out_dtype, float* out_lse, void* stream) {
  if (!info || !plan_dev || !out) return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_merge: a required pointer is NULL");
  if (raw(out_dtype) != PA_DTYPE_BF16 && raw(out_dtype) != PA_DTYPE_FP32)
    return fail(PA_ERR_INVALID_ARGUMENT, "out_dtype must be BF16 or FP32");
  if (!info->needs_merge) return ok();
  if (!partial_o || !partial_lse) return fail(PA_ERR_INVALID_ARGUMENT, "partial_o and partial_lse are required");
  if (!aligned16(out) || !aligned16(partial_o))
    return fail(PA_ERR_INVALID_ARGUMENT, "out and partial_o must be 16-byte aligned");
  MergeArgs m;
  m.row_nsplit = reinterpret_cast<const int32_t*>(static_cast<const uint8_t*>(plan_dev) +
                                                  (int64_t)info->num_items * sizeof(PaItem));
  m.partial_o = partial_o;
  m.partial_lse = partial_lse;
  m.part_bf16 = partial_o_elem_bytes(info->kv_dtype) == 2;
  m.out = out;
  m.out_bf16 = out_dtype == PA_DTYPE_BF16;
  m.out_lse = out_lse;
  m.total_rows = info->total_rows;
  m.hq = info->num_q_heads;
  m.dh = info->head_dim_v > 0 ? info->head_dim_v : info->head_dim;
  m.s_max = info->max_splits;
  const int e = launch_merge(m, stream);
  if (e) return hip_fail(e, "pa_decode_merge launch");
  return ok();
}

pa_status pa_kv_quantize_fp8(const void* src, pa_dtype src_dtype, int64_t n_rows, int32_t head_dim,
                             pa_scale_mode mode, uint8_t* dst, float* scale, void* stream) {
  if (!src || !dst || !scale) return fail(PA_ERR_INVALID_ARGUMENT, "pa_kv_quantize_fp8: NULL pointer");
  if (raw(src_dtype) != PA_DTYPE_BF16 && raw(src_dtype) != PA_DTYPE_FP32)
    return fail(PA_ERR_INVALID_ARGUMENT, "src_dtype must be BF16 or FP32");
  if (raw(mode) != PA_SCALE_PER_TENSOR && raw(mode) != PA_SCALE_PER_TOKEN_HEAD)   // per-head: pa_kv_quantize_fp8_per_head
    return fail(PA_ERR_INVALID_ARGUMENT, "mode must be PER_TENSOR or PER_TOKEN_HEAD");
  if (n_rows < 0) return fail(PA_ERR_INVALID_ARGUMENT, "n_rows must be >= 0");
  if (head_dim < 64 || head_dim > 1024 || ilog2_exact(head_dim / 64) < 0 || head_dim % 64)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d: must be 64 times a power of two, at most 1024", head_dim);
  if (!aligned16(src) || ((uintptr_t)dst & 7u) != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_kv_quantize_fp8: src must be 16-byte and dst 8-byte aligned");
  const int e = launch_quant(src, src_dtype == PA_DTYPE_BF16, n_rows, head_dim, mode == PA_SCALE_PER_TENSOR, 0, dst,
                             scale, stream);
  if (e) return hip_fail(e, "pa_kv_quantize_fp8 launch");
  return ok();
}

pa_status pa_kv_quantize_int8(const void* src, pa_dtype src_dtype, int64_t n_rows, int32_t head_dim,
                              pa_scale_mode mode, int8_t* dst, float* scale, void* stream) {
  if (!src || !dst || !scale) return fail(PA_ERR_INVALID_ARGUMENT, "pa_kv_quantize_int8: NULL pointer");
  if (raw(src_dtype) != PA_DTYPE_BF16 && raw(src_dtype) != PA_DTYPE_FP32)
    return fail(PA_ERR_INVALID_ARGUMENT, "src_dtype must be BF16 or FP32");
  if (raw(mode) != PA_SCALE_PER_TENSOR && raw(mode) != PA_SCALE_PER_TOKEN_HEAD)
    return fail(PA_ERR_INVALID_ARGUMENT, "mode must be PER_TENSOR or PER_TOKEN_HEAD");
  if (n_rows < 0) return fail(PA_ERR_INVALID_ARGUMENT, "n_rows must be >= 0");
  if (head_dim < 64 || head_dim > 1024 || ilog2_exact(head_dim / 64) < 0 || head_dim % 64)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d: must be 64 times a power of two, at most 1024", head_dim);
  if (!aligned16(src) || ((uintptr_t)dst & 7u) != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_kv_quantize_int8: src must be 16-byte and dst 8-byte aligned");
  const int e = launch_quant(src, src_dtype == PA_DTYPE_BF16, n_rows, head_dim, mode == PA_SCALE_PER_TENSOR, 1,
                             reinterpret_cast<uint8_t*>(dst), scale, stream);
  if (e) return hip_fail(e, "pa_kv_quantize_int8 launch");
  return ok();
}

pa_status pa_kv_quantize_fp8_per_head(const void* src, pa_dtype src_dtype, int64_t n_tokens, int32_t num_heads,
                                      int32_t head_dim, uint8_t* dst, float* scale, void* stream) {
  if (!src || !dst || !scale) return fail(PA_ERR_INVALID_ARGUMENT, "pa_kv_quantize_fp8_per_head: NULL pointer");
  if (raw(src_dtype) != PA_DTYPE_BF16 && raw(src_dtype) != PA_DTYPE_FP32)
    return fail(PA_ERR_INVALID_ARGUMENT, "src_dtype must be BF16 or FP32");
  if (n_tokens < 0) return fail(PA_ERR_INVALID_ARGUMENT, "n_tokens must be >= 0");
  if (num_heads < 1 || num_heads > 1024)
    return fail(PA_ERR_UNSUPPORTED, "num_heads %d: must be in [1, 1024]", num_heads);
  if (head_dim < 64 || head_dim > 1024 || ilog2_exact(head_dim / 64) < 0 || head_dim % 64)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d: must be 64 times a power of two, at most 1024", head_dim);
  if (!aligned16(src) || ((uintptr_t)dst & 7u) != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_kv_quantize_fp8_per_head: src must be 16-byte and dst 8-byte aligned");
  const int e = launch_quant_heads(src, src_dtype == PA_DTYPE_BF16, n_tokens, num_heads, head_dim, dst, scale, stream);
  if (e) return hip_fail(e, "pa_kv_quantize_fp8_per_head launch");
  return ok();
}

pa_status pa_kv_append(const void* k_new, const void* v_new, pa_dtype src_dtype, int64_t n_tokens,
                       int32_t num_kv_heads, int32_t head_dim, int32_t page_size, const int64_t* slot_mapping,
                       void* k_cache, void* v_cache, pa_dtype kv_dtype, pa_scale_mode mode,
                       const pa_kv_layout* kv, float* k_scale, float* v_scale, const pa_scale_layout* sc,
                       void* stream) {
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache || !kv)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_kv_append: NULL pointer");
  if (raw(src_dtype) != PA_DTYPE_BF16 && raw(src_dtype) != PA_DTYPE_FP32)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_kv_append: src_dtype must be BF16 or FP32");
  int m;
  const int kd = raw(kv_dtype), md = raw(mode);
  if (kd == PA_DTYPE_BF16 && md == PA_SCALE_NONE) m = 0;
  else if (kd == PA_DTYPE_FP8_E4M3 && (md == PA_SCALE_PER_TENSOR || md == PA_SCALE_PER_HEAD)) m = 1;
  else if (kd == PA_DTYPE_FP8_E4M3 && md == PA_SCALE_PER_TOKEN_HEAD) m = 2;
  else if (kd == PA_DTYPE_INT8 && md == PA_SCALE_PER_TENSOR) m = 1;
  else if (kd == PA_DTYPE_INT8 && md == PA_SCALE_PER_TOKEN_HEAD) m = 2;
  else return fail(PA_ERR_INVALID_ARGUMENT,
                   "pa_kv_append: kv_dtype/mode must be BF16/NONE, FP8 with PER_TENSOR, PER_HEAD or PER_TOKEN_HEAD, "
                   "or INT8 with PER_TENSOR or PER_TOKEN_HEAD");
  if (m > 0 && (!k_scale || !v_scale))
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_kv_append: FP8 and INT8 caches need k_scale and v_scale");
  if (m == 2 && !sc) return fail(PA_ERR_INVALID_ARGUMENT, "pa_kv_append: per-token-head scales need a scale layout");
  if (n_tokens < 0 || num_kv_heads < 1) return fail(PA_ERR_INVALID_ARGUMENT, "pa_kv_append: n_tokens >= 0, num_kv_heads >= 1");
  if (2 * n_tokens * num_kv_heads >= (int64_t(1) << 31))
    return fail(PA_ERR_UNSUPPORTED, "pa_kv_append: 2 * n_tokens * num_kv_heads must be below 2^31");
  if (head_dim < 64 || head_dim > 1024 || head_dim % 64 || ilog2_exact(head_dim / 64) < 0)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d: must be 64 times a power of two, at most 1024", head_dim);
  const int shift = ilog2_exact(page_size);
  if (shift < 0) return fail(PA_ERR_UNSUPPORTED, "page_size %d: must be a power of two", page_size);
  const int esz = kv_dtype == PA_DTYPE_BF16 ? 2 : 1;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_kv_append: sources and caches must be 16-byte aligned");
  if ((kv->page * esz) % 16 || (kv->head * esz) % 16 || (kv->slot * esz) % 16 || kv->page < 0 || kv->head < 0 ||
      kv->slot < 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_kv_append: cache strides must be non-negative and 16-byte multiples");
  AppendArgs a;
  a.k_new = k_new; a.v_new = v_new; a.slots = slot_mapping;
  a.k_cache = k_cache; a.v_cache = v_cache; a.k_scale = k_scale; a.v_scale = v_scale;
  a.n_tokens = n_tokens; a.hkv = num_kv_heads; a.page_shift = shift;
  a.kv_sp = kv->page; a.kv_sh = kv->head; a.kv_ss = kv->slot;
  a.sc_sp = m == 2 ? sc->page : 0; a.sc_sh = m == 2 ? sc->head : 0; a.sc_ss = m == 2 ? sc->slot : 0;
  a.scale_hstride = mode == PA_SCALE_PER_HEAD ? 1 : 0;
  a.i8 = kv_dtype == PA_DTYPE_INT8;
  const int e = launch_append(a, src_dtype == PA_DTYPE_BF16, head_dim, m, stream);
  if (e) return hip_fail(e, "pa_kv_append launch");
  return ok();
}

pa_status pa_debug_gather(const pa_plan_info* info, const void* plan_dev, const int32_t* page_indices,
                          const pa_kv_layout* kv, const pa_scale_layout* sc, int64_t* kv_off_out,
                          int64_t* scale_off_out, void* stream) {
  if (!info || !plan_dev || !page_indices || !kv || !kv_off_out)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_debug_gather: NULL pointer");
  const KernelCfg cfg = unpack_cfg(info->variant);
  if (!stage1_cfg_supported(cfg) || cfg.dh != info->head_dim)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_plan_info was not produced by pa_plan_splits");
  if (cfg.kr) return fail(PA_ERR_UNSUPPORTED, "pa_debug_gather covers the equal-width stage-1 kernel only");
  // INT8 KV runs the per-token scale path for both scale modes (per tensor: zero strides)
  const bool per_token = info->kv_scale_mode == PA_SCALE_PER_TOKEN_HEAD || info->kv_dtype == PA_DTYPE_INT8;
  if (per_token && !scale_off_out)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_debug_gather: per-token scales need scale_off_out");
  if (info->kv_scale_mode == PA_SCALE_PER_TOKEN_HEAD && !sc)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_debug_gather: per-token-head scales need a scale layout");
  GatherArgs g;
  memset(&g, 0, sizeof g);
  g.items = static_cast<const PaItem*>(plan_dev);
  g.page_indices = page_indices;
  g.kv_sp = kv->page;
  g.kv_sh = kv->head;
  g.kv_ss = kv->slot;
  if (per_token && info->kv_scale_mode == PA_SCALE_PER_TOKEN_HEAD) {
    g.sc_sp = sc->page;
    g.sc_sh = sc->head;
    g.sc_ss = sc->slot;
  }
  g.kv_off = kv_off_out;
  g.sc_off = per_token ? scale_off_out : nullptr;
  g.max_tok = info->max_item_tokens;
  g.page_shift = ilog2_exact(info->page_size);
  const int e = launch_gather(cfg, g, info->num_items, stream);
  if (e) return hip_fail(e, "pa_debug_gather launch");
  return ok();
}

pa_status pa_debug_gather_rope(const pa_plan_info* info, const void* plan_dev, const int32_t* page_indices,
                               const pa_kv_layout* k_layout, const pa_kv_layout* k_rope_layout,
                               const pa_kv_layout* v_layout, const pa_scale_layout* k_scale_layout, int64_t* off_out,
                               void* stream) {
  if (!info || !plan_dev || !page_indices || !k_layout || !off_out)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_debug_gather_rope: NULL pointer");
  const KernelCfg cfg = unpack_cfg(info->variant);
  if (!stage1_cfg_supported(cfg) || cfg.dh != info->head_dim)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_plan_info was not produced by pa_plan_splits");
  if (!cfg.kr) return fail(PA_ERR_UNSUPPORTED, "equal key and value widths: use pa_debug_gather");
  if (cfg.mla && (!k_rope_layout || !k_scale_layout))
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_debug_gather_rope: the latent cache needs rotary and scale layouts");
  if (!cfg.mla && !v_layout) return fail(PA_ERR_INVALID_ARGUMENT, "pa_debug_gather_rope: 192/128 needs v_layout");
  GatherRopeArgs g;
  memset(&g, 0, sizeof g);
  g.items = static_cast<const PaItem*>(plan_dev);
  g.page_indices = page_indices;
  g.m_sp = k_layout->page;
  g.m_sh = k_layout->head;
  g.m_ss = k_layout->slot;
  const pa_kv_layout* rl = cfg.mla ? k_rope_layout : k_layout;   // 192/128: rotary part of the K row
  g.r_sp = rl->page;
  g.r_sh = rl->head;
  g.r_ss = rl->slot;
  if (!cfg.mla) {
    g.v_sp = v_layout->page;
    g.v_sh = v_layout->head;
    g.v_ss = v_layout->slot;
  } else {
    g.s_sp = k_scale_layout->page;
    g.s_sh = k_scale_layout->head;
    g.s_ss = k_scale_layout->slot;
  }
  g.off = off_out;
  g.max_tok = info->max_item_tokens;
  g.page_shift = ilog2_exact(info->page_size);
  const int e = launch_gather_rope(cfg, g, info->num_items, stream);
  if (e) return hip_fail(e, "pa_debug_gather_rope launch");
  return ok();
}

}  // extern "C"
