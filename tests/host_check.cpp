// Host-side exercise of the C ABI for a build with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_sanitizers.py
// builds it, device code compiled as usual, and runs it on the CPU). It drives descriptor
// validation, the workspace and reserve layouts, the launch planner and the
// argument checks of the entry points over a seeded sweep of valid, edge and
// invalid descriptors and length arrays. Nothing here needs a GPU: every
// call either returns before touching a device or fails on the missing one.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <vector>

#include "rnn.h"

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint32_t next_u32() {  // xorshift64*
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (uint32_t)((g_state * 0x2545F4914F6CDD1Dull) >> 32);
}
int pick(const std::vector<int>& v) { return v[next_u32() % v.size()]; }
int range(int lo, int hi) { return lo + (int)(next_u32() % (uint32_t)(hi - lo + 1)); }

const std::vector<int> kSizes = {-1, 0, 1, 2, 3, 7, 16, 17, 31, 33, 64, 100, 200, 256, 511, 1024, 4096, 65536, 1 << 30};
const std::vector<int> kSmall = {-1, 0, 1, 2, 3, 4, 5, 8, 9};

RnnDesc random_desc() {
  RnnDesc d;
  std::memset(&d, 0, sizeof(d));
  const bool tame = next_u32() % 3 != 0;  // two thirds mostly-valid descriptors
  d.mode = tame ? range(0, 4) : pick({-1, 0, 1, 2, 3, 4, 5, 99});
  d.dtype = tame ? range(0, 1) : pick({-1, 0, 1, 2});
  d.layout = tame ? (d.mode >= 3 ? 2 : range(0, 1)) : pick({-1, 0, 1, 2, 3});
  d.T = tame ? range(1, 40) : pick(kSizes);
  d.B = tame ? range(1, 70) : pick(kSizes);
  d.input_size = tame ? range(1, 300) : pick(kSizes);
  d.hidden_size = tame ? range(1, 300) : pick(kSizes);
  d.proj_size = d.mode == 2 ? (tame ? range(1, d.hidden_size > 0 ? d.hidden_size : 1) : pick(kSizes))
                            : (tame ? 0 : pick(kSmall));
  d.num_layers = tame ? range(1, 3) : pick(kSmall);
  d.bidirectional = tame ? range(0, 1) : pick({-1, 0, 1, 2});
  d.has_bias = tame ? range(0, 1) : pick({-1, 0, 1, 2});
  d.state_dim = tame ? range(1, 40) : pick(kSizes);
  d.action_dim = tame ? range(1, 8) : pick(kSizes);
  d.embed_dim = tame ? range(1, 260) : pick(kSizes);
  d.belief_dim = tame ? range(1, 260) : pick(kSizes);
  d.scale_lb = next_u32() % 17 == 0 ? std::numeric_limits<float>::quiet_NaN() : 0.1f;
  d.tile_batch = next_u32() % 4 == 0 ? pick({-1, 0, 1, 2, 3, 16, 17, 32, 48, 64, 65, 128}) : 0;
  d.tile_hidden = next_u32() % 4 == 0 ? pick({-1, 0, 1, 4, 16, 32, 33, 64, 256, 300}) : 0;
  d.placement = next_u32() % 4 == 0 ? pick({-1, 0, 1, 2, 3}) : 0;
  d.weights = next_u32() % 4 == 0 ? pick({-1, 0, 1, 2, 3}) : 0;
  d.clip = next_u32() % 5 == 0 ? pick({-1, 0, 1, 2, 3, 4}) : 0;
  d.cell_clip_lo = next_u32() % 7 == 0 ? std::numeric_limits<float>::quiet_NaN() : -2.0f;
  d.cell_clip_hi = next_u32() % 7 == 0 ? -std::numeric_limits<float>::infinity() : 2.0f;
  d.proj_clip = next_u32() % 7 == 0 ? -1.0f : 0.5f;
  d.actor_dim = d.mode == 4 ? (tame ? range(1, 64) : pick(kSizes)) : (next_u32() % 9 == 0 ? 3 : 0);
  d.gx_dtype = next_u32() % 6 == 0 ? pick({-1, 0, 1, 2}) : 0;
  d.layer_pipeline = next_u32() % 6 == 0 ? pick({-1, 0, 1, 2, 3}) : 0;
  if (next_u32() % 25 == 0) d.reserved[0] = 1;
  return d;
}

// Lengths for B rows: none, valid sorted, valid unsorted, or out of range.
std::vector<int32_t> random_lengths(const RnnDesc& d, int* kind) {
  std::vector<int32_t> L;
  const int B = d.B > 0 && d.B <= 4096 ? d.B : 0;
  *kind = (int)(next_u32() % 4);
  if (*kind == 0 || B == 0) {
    *kind = 0;
    return L;
  }
  const int T = d.T > 0 ? d.T : 1;
  L.resize(B);
  for (int b = 0; b < B; ++b) L[b] = range(1, T);
  if (*kind == 1)
    for (int i = 1; i < B; ++i)
      for (int j = i; j > 0 && L[j] > L[j - 1]; --j) std::swap(L[j], L[j - 1]);
  if (*kind == 3) L[next_u32() % B] = pick({-5, 0, T + 1, 1 << 30});
  return L;
}

}  // namespace

int main(int argc, char** argv) {
  // --self-test: a heap read one element past a vector's end (host memory),
  // which an instrumented build must report; proves the sanitizer is active
  if (argc > 1 && std::strcmp(argv[1], "--self-test") == 0) {
    std::vector<int> v((size_t)range(3, 5));
    volatile int* p = v.data();
    std::printf("read %d\n", p[v.size()]);
    return 0;
  }
  int fails = 0;
  if (rnn_abi_version() <= 0) {
    std::printf("bad abi version\n");
    ++fails;
  }
  for (int s = -20; s <= 5; ++s)
    if (!rnn_strerror(s) || !*rnn_strerror(s)) {
      std::printf("empty strerror(%d)\n", s);
      ++fails;
    }

  // NULL handling of every host-only query
  size_t bytes = 0;
  int info[16];
  if (rnn_workspace_bytes(nullptr, nullptr, &bytes) != RNN_E_NULL) ++fails;
  if (rnn_reserve_bytes(nullptr, nullptr, &bytes) != RNN_E_NULL) ++fails;
  if (rnn_backward_workspace_bytes(nullptr, nullptr, &bytes) != RNN_E_NULL) ++fails;
  if (rnn_plan_info(nullptr, nullptr, 256, 8, info, 16) != RNN_E_NULL) ++fails;
  if (rnn_forward(nullptr, nullptr, nullptr, nullptr, 0, nullptr) == RNN_OK) ++fails;
  if (rnn_forward_noalloc(nullptr, nullptr, nullptr, nullptr, nullptr) == RNN_OK) ++fails;

  long counts[32] = {0};
  const int kIters = 20000;
  for (int it = 0; it < kIters; ++it) {
    RnnDesc d = random_desc();
    int kind = 0;
    std::vector<int32_t> L = random_lengths(d, &kind);
    const int32_t* lp = L.empty() ? nullptr : L.data();
    const int st = rnn_workspace_bytes(&d, lp, &bytes);
    counts[-st < 32 && st <= 0 ? -st : 31]++;
    rnn_reserve_bytes(&d, lp, &bytes);
    rnn_backward_workspace_bytes(&d, lp, &bytes);
    const int cus = pick({256, 304, 80, 1, 0, -1});
    const int xcds = pick({8, 1, 0, 3});
    const int n_info = pick({0, 5, 13, 16});
    const int sp = rnn_plan_info(&d, lp, cus, xcds, info, n_info);
    // for a descriptor rnn_workspace_bytes accepts: too small an info array
    // is RNN_E_NULL, an impossible device RNN_E_SHAPE, else a plan or
    // RNN_E_PLAN (the problem does not fit the device)
    const int want = n_info < 9 ? RNN_E_NULL : (cus < 1 || xcds < 1 || cus % xcds != 0) ? RNN_E_SHAPE : 1;
    if (st == RNN_OK && (want != 1 ? sp != want : (sp != RNN_OK && sp != RNN_E_PLAN))) {
      std::printf("plan_info status %d for a valid descriptor (cus %d xcds %d n_info %d)\n", sp, cus, xcds, n_info);
      ++fails;
    }
    // argument checks of the launching entry points: missing weights, I/O
    // or workspace return an error before anything is enqueued
    RnnWeights w;
    std::memset(&w, 0, sizeof(w));
    RnnIO io;
    std::memset(&io, 0, sizeof(io));
    io.lengths_host = lp;
    if (rnn_forward(&d, &w, &io, nullptr, 0, nullptr) == RNN_OK) {
      std::printf("rnn_forward accepted NULL buffers\n");
      ++fails;
    }
  }
  std::printf("host_check: %d descriptors; status histogram:", kIters);
  for (int i = 0; i < 32; ++i)
    if (counts[i]) std::printf(" %d:%ld", -i, counts[i]);
  std::printf("\nfailures %d\n", fails);
  return fails ? 1 : 0;
}
