// Randomised inputs for the split planner (pa_plan_splits), built with the address and
// undefined-behaviour sanitizers: malformed and extreme arguments must come back as a
// status, never as an out-of-bounds access or undefined arithmetic, and every accepted
// plan must cover each (request, KV head, query-block group)'s visible token range
// exactly once with well-formed items.  Host arrays are sized exactly (std::vector) so
// that any read past them is caught.  Usage: planner_fuzz [cases] [seed]
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <vector>

#include "pa.h"
#include "pa_internal.hpp"

namespace {

uint64_t rng_state;
uint64_t next() {                       // xorshift64*
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 2685821657736338717ull;
}
int uni(int lo, int hi) { return lo + (int)(next() % (uint64_t)(hi - lo + 1)); }
template <typename T, size_t N>
T pick(const T (&v)[N]) { return v[next() % N]; }

int fails = 0;
#define CHECK(c, ...) do { if (!(c)) { ++fails; fprintf(stderr, "case %d: ", cs); fprintf(stderr, __VA_ARGS__); fprintf(stderr, "\n"); return; } } while (0)

void one_case(int cs) {
  const bool wild = next() % 4 == 0;                 // a quarter of the cases break a rule
  const int B = wild ? uni(-1, 20) : uni(1, 16);
  const int nb = B > 0 ? B : 1;
  const int psizes[] = {16, 32, 64, 1024, 8, 48, 2048};
  const int P = wild ? pick(psizes) : pick(psizes) % 2048 > 0 && pick(psizes) >= 16 ? 16 << uni(0, 6) : 16;
  const int dims[] = {128, 256, 512, 192, 576, 64, 96};
  int d = wild ? pick(dims) : dims[uni(0, 4)];
  const int hkvs[] = {1, 2, 8};
  const int Hkv = pick(hkvs);
  const int gs[] = {1, 2, 8, 24, 3};
  const int G = pick(gs);
  const int Hq = Hkv * G + (wild && next() % 3 == 0 ? 1 : 0);
  const int max_q = wild ? uni(0, 10) : uni(1, 8);
  std::vector<int32_t> qo(nb + 1), kvi(nb + 1), kv(nb), win(nb);
  qo[0] = wild && next() % 8 == 0 ? 1 : 0;
  kvi[0] = 0;
  for (int b = 0; b < nb; ++b) {
    const int n = wild && next() % 10 == 0 ? uni(-1, 9) : uni(1, max_q > 0 ? (max_q < 8 ? max_q : 8) : 1);
    qo[b + 1] = qo[b] + n;
    kv[b] = wild && next() % 10 == 0 ? uni(-5, n) : n + uni(0, next() % 3 == 0 ? 70000 : 3000);
    const int64_t pages = kv[b] > 0 ? ((int64_t)kv[b] + P - 1) / (P > 0 ? P : 1) : 0;
    kvi[b + 1] = kvi[b] + (int32_t)pages + (wild && next() % 10 == 0 ? 1 : 0);
    win[b] = next() % 2 ? 0 : (wild && next() % 10 == 0 ? -3 : uni(1, 2000));
  }
  // keys wider than values: 192/128 bf16 or the 576/512 latent cache; sometimes a wrong pair
  const int dvs[] = {0, 128, 512, 100};
  const int dv = d == 192 ? 128 : d == 576 ? 512 : (wild ? pick(dvs) : 0);
  const pa_dtype qd[] = {PA_DTYPE_BF16, PA_DTYPE_FP8_E4M3};
  const pa_dtype kd[] = {PA_DTYPE_BF16, PA_DTYPE_FP8_E4M3, PA_DTYPE_INT8};
  pa_plan_args a;
  memset(&a, 0, sizeof a);
  a.batch = B;
  a.qo_indptr = qo.data();
  a.kv_indptr = kvi.data();
  a.kv_len = kv.data();
  a.window = next() % 3 ? win.data() : nullptr;
  a.max_q_len = max_q;
  a.page_size = P;
  a.num_q_heads = Hq;
  a.num_kv_heads = Hkv;
  a.head_dim = d;
  a.q_dtype = wild && next() % 6 == 0 ? (pa_dtype)7 : pick(qd);
  a.kv_dtype = pick(kd);
  a.kv_scale_mode = a.kv_dtype == PA_DTYPE_BF16 ? PA_SCALE_NONE
                    : (pa_scale_mode)(a.kv_dtype == PA_DTYPE_INT8 ? (next() % 2 ? 1 : 2) : uni(1, 3));
  if (d == 576 && !wild) {
    a.q_dtype = PA_DTYPE_FP8_E4M3;
    a.kv_dtype = PA_DTYPE_FP8_E4M3;
    a.kv_scale_mode = PA_SCALE_PER_TOKEN_BLOCK128;
  } else if (d == 192 && !wild) {
    a.q_dtype = PA_DTYPE_BF16;
    a.kv_dtype = PA_DTYPE_BF16;
    a.kv_scale_mode = PA_SCALE_NONE;
  }
  a.head_dim_v = dv;
  if (wild && next() % 6 == 0) a.kv_scale_mode = (pa_scale_mode)uni(0, 5);
  const int cus[] = {1, 8, 256, 304};
  a.num_cus = pick(cus);
  a.max_splits = next() % 3 ? 0 : uni(1, 64);
  a.force_splits = next() % 5 ? 0 : uni(1, a.max_splits > 0 ? a.max_splits : 32);
  if (wild && next() % 10 == 0) a.force_splits = -1;

  pa_plan_info info;
  const pa_status st = pa_plan_splits(&a, nullptr, 0, &info);
  if (st != PA_OK) {
    CHECK(st == PA_ERR_INVALID_ARGUMENT || st == PA_ERR_UNSUPPORTED, "unexpected status %d", (int)st);
    CHECK(pa_last_error()[0] != 0, "failure without a message");
    return;
  }
  CHECK(!wild || B >= 1, "accepted batch %d", B);
  CHECK(info.plan_bytes == (int64_t)info.num_items * 64 + (int64_t)qo[B] * 4, "plan bytes");
  std::vector<uint8_t> small(8);
  CHECK(pa_plan_splits(&a, small.data(), small.size(), &info) == PA_ERR_INSUFFICIENT_WORKSPACE, "small buffer");
  std::vector<uint8_t> plan((size_t)info.plan_bytes);
  CHECK(pa_plan_splits(&a, plan.data(), plan.size(), &info) == PA_OK, "second call");
  std::vector<pa::PaItem> items(info.num_items);
  memcpy(items.data(), plan.data(), items.size() * sizeof(pa::PaItem));
  std::vector<int32_t> row_ns(qo[B]);
  memcpy(row_ns.data(), plan.data() + items.size() * sizeof(pa::PaItem), row_ns.size() * 4);
  // coverage: per (request, KV head, first block) the ranges tile [begin, kv_len) exactly
  std::vector<std::map<int, std::vector<uint8_t>>> cover(B);   // (KV head, first block) -> per token
  int64_t max_tok = 0;
  for (const pa::PaItem& it : items) {
    const int b = it.req;
    CHECK(b >= 0 && b < B, "request %d", b);
    CHECK(it.row0 == qo[b] && it.nrows == qo[b + 1] - qo[b] && it.kv_len == kv[b] && it.page_base == kvi[b],
          "request fields");
    CHECK(it.kvh >= 0 && it.kvh < Hkv && it.qblk0 >= 0 && it.qblk0 < 64, "kvh %d qblk0 %d", it.kvh, it.qblk0);
    CHECK(it.split >= 0 && it.split < it.nsplit && it.nsplit <= info.max_splits, "split");
    CHECK(0 <= it.tok_begin && it.tok_begin <= it.tok_end && it.tok_end <= kv[b], "range");
    CHECK(it.tok_begin % 64 == 0 || it.tok_begin == kv[b], "alignment");
    max_tok = it.tok_end - it.tok_begin > max_tok ? it.tok_end - it.tok_begin : max_tok;
    std::vector<uint8_t>& cv = cover[b][it.kvh * 64 + it.qblk0];
    if (cv.empty()) cv.assign(kv[b], 0);
    for (int t = it.tok_begin; t < it.tok_end; ++t) cv[t] += 1;
  }
  CHECK(max_tok == info.max_item_tokens, "max_item_tokens %lld vs %lld", (long long)info.max_item_tokens,
        (long long)max_tok);
  for (int b = 0; b < B; ++b) {
    const int n = qo[b + 1] - qo[b];
    const int W = a.window ? win[b] : 0;
    const int lo = W > 0 ? (kv[b] - n - W + 1 > 0 ? kv[b] - n - W + 1 : 0) : 0;
    for (int r = qo[b]; r < qo[b + 1]; ++r) CHECK(row_ns[r] >= 1 && row_ns[r] <= info.max_splits, "row_nsplit");
    // every KV head has items, with the same query-block groups
    CHECK(kv[b] <= lo || (int)cover[b].size() % Hkv == 0, "request %d: groups not the same for every KV head", b);
    for (const auto& kvc : cover[b])
      for (int t = 0; t < kv[b]; ++t)
        CHECK(kvc.second[t] == (t >= lo ? 1 : 0) || (t < lo && kvc.second[t] <= 1),
              "request %d head/block %d token %d covered %d times (visible from %d)", b, kvc.first, t,
              (int)kvc.second[t], lo);
  }
}

}  // namespace

int main(int argc, char** argv) {
  const int cases = argc > 1 ? atoi(argv[1]) : 2000;
  rng_state = argc > 2 ? strtoull(argv[2], nullptr, 10) : 0x9E3779B97F4A7C15ull;
  if (!rng_state) rng_state = 1;
  for (int cs = 0; cs < cases && fails < 5; ++cs) one_case(cs);
  printf("%d cases, %d failures\n", cases, fails);
  return fails ? 1 : 0;
}
