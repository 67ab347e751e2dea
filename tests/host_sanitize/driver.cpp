// Host-side exercise of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer: the block manager through long random traces
// (with a block-conservation check after every operation), and every
// entry point's argument checks, which must return before any HIP call.
// Built and run by tests/test_host_sanitizers.py; needs no GPU.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <map>
#include <random>
#include <set>
#include <vector>

#include "pa.h"
#include "pa_blocks.h"

static int failures = 0;
#define CHECK(c)                                                     \
  do {                                                               \
    if (!(c)) {                                                      \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++failures;                                                    \
    }                                                                \
  } while (0)

// ---------------------------------------------------------------------------
// block manager: random traces
// ---------------------------------------------------------------------------
static void bm_trace(uint32_t seed) {
  std::mt19937 rng(seed);
  auto pick = [&](int n) { return (int)(rng() % (uint32_t)n); };
  const int nb = 1 + pick(40), bs = 1 << pick(5), nh = pick(30);
  std::vector<int32_t> order(nb);
  for (int i = 0; i < nb; ++i) order[i] = i;
  std::shuffle(order.begin(), order.end(), rng);
  pa_bm* bm = nullptr;
  CHECK(pa_bm_create(nb, bs, order.data(), nh, &bm) == PA_OK && bm);
  std::map<int64_t, int> state;   // 0 running, 1 swapping, 2 swapped out
  int64_t next = 1;
  std::vector<int64_t> buf(2 * (nb + nh + 8) + 512);
  for (int step = 0; step < 600; ++step) {
    const int op = pick(10);
    std::vector<int64_t> ids;
    for (auto& kv : state) ids.push_back(kv.first);
    const int64_t any = ids.empty() ? 999999 : ids[pick((int)ids.size())];
    int32_t n = 0, ncow = 0;
    switch (op) {
      case 0: if (pa_bm_add(bm, next) == PA_OK) state[next] = 0; ++next; break;
      case 1: case 2: case 3: {
        const int32_t k = pick(3) ? 1 : pick(200);
        std::vector<int64_t> slots(k + 1);
        const pa_status s = pa_bm_append(bm, any, k, slots.data(), buf.data(), &ncow);
        CHECK(s == PA_OK || s == PA_ERR_NO_SPACE || s == PA_ERR_INVALID_ARG);
        if (s == PA_OK)
          for (int32_t i = 0; i < k; ++i) CHECK(slots[i] >= 0 && slots[i] < (int64_t)nb * bs);
        break;
      }
      case 4: if (pa_bm_fork(bm, any, next) == PA_OK) state[next] = 0; ++next; break;
      case 5: pa_bm_copy_last_block(bm, any, buf.data()); break;
      case 6: if (pa_bm_release(bm, any) == PA_OK) state.erase(any); break;
      case 7: {
        int64_t v = -1;
        if (pa_bm_newest_running(bm, &v) == PA_OK &&
            pa_bm_swap_out(bm, v, buf.data(), (int32_t)buf.size() / 2, &n) == PA_OK) {
          state[v] = 1;
          if (pick(2)) { CHECK(pa_bm_swap_out_done(bm, v) == PA_OK); state[v] = 2; }
        }
        break;
      }
      case 8:
        for (auto& kv : state)
          if (kv.second == 1 && pa_bm_swap_out_done(bm, kv.first) == PA_OK) kv.second = 2;
        if (pa_bm_swap_in(bm, any, buf.data(), (int32_t)buf.size() / 2, &n) == PA_OK) state[any] = 0;
        break;
      default: {
        // outputs too small and null pointers: refused, nothing changes
        int32_t tb[1], nbk = 0, nt = 0;
        CHECK(pa_bm_table(bm, any, nullptr, 0, nullptr, &nt) == PA_ERR_INVALID_ARG);
        pa_bm_table(bm, any, tb, 0, &nbk, &nt);
        CHECK(pa_bm_append(bm, any, 1, nullptr, buf.data(), &ncow) == PA_ERR_INVALID_ARG);
        CHECK(pa_bm_swap_out(nullptr, any, buf.data(), 1, &n) == PA_ERR_INVALID_ARG);
        CHECK(pa_bm_blocks_needed(bm, any, -5) == 0);
        break;
      }
    }
    // conservation: free device blocks + distinct blocks held by running or
    // swapping sequences = all blocks
    std::set<int32_t> held;
    std::vector<int32_t> t(nb + 1);
    for (auto& kv : state) {
      int32_t nbk = 0, nt = 0;
      CHECK(pa_bm_table(bm, kv.first, t.data(), (int32_t)t.size(), &nbk, &nt) == PA_OK);
      if (kv.second != 2)
        for (int32_t i = 0; i < nbk; ++i) held.insert(t[i]);
    }
    CHECK(pa_bm_num_free(bm, 0) + (int32_t)held.size() == nb);
    CHECK(pa_bm_num_free(bm, 1) >= 0 && pa_bm_num_free(bm, 1) <= nh);
  }
  pa_bm_destroy(bm);
}

// ---------------------------------------------------------------------------
// entry points: argument checks that return before any HIP call
// ---------------------------------------------------------------------------
static void* const FAKE = (void*)(uintptr_t)0x100000;

static pa_kv_cache cache(pa_dtype dt, int32_t blocks, int32_t layers, int32_t heads, int32_t bs,
                         int32_t dim, float ks = 1.f, float vs = 1.f) {
  pa_kv_cache c;
  c.k = FAKE;
  c.v = FAKE;
  c.dtype = dt;
  c.num_blocks = blocks;
  c.num_layers = layers;
  c.num_kv_heads = heads;
  c.block_size = bs;
  c.head_dim = dim;
  c.layer_stride = (int64_t)heads * bs * dim;
  c.block_stride = (int64_t)layers * c.layer_stride;
  c.k_scale = ks;
  c.v_scale = vs;
  return c;
}

static bool refused(pa_status s) { return s == PA_ERR_INVALID_ARG || s == PA_ERR_UNSUPPORTED || s == PA_ERR_WORKSPACE; }

static void geometry_cases(std::vector<pa_kv_cache>& bad) {
  pa_kv_cache c = cache(PA_BF16, 100, 2, 8, 16, 128);
  auto push = [&](auto f) { pa_kv_cache x = c; f(x); bad.push_back(x); };
  push([](pa_kv_cache& x) { x.block_size = 12; });
  push([](pa_kv_cache& x) { x.block_size = 512; });
  push([](pa_kv_cache& x) { x.num_blocks = 0; });
  push([](pa_kv_cache& x) { x.num_layers = -1; });
  push([](pa_kv_cache& x) { x.head_dim = 0; });
  push([](pa_kv_cache& x) { x.dtype = (pa_dtype)9; });
  push([](pa_kv_cache& x) { x.k = nullptr; });
  push([](pa_kv_cache& x) { x.layer_stride = 10; });                       // slabs overlap
  push([](pa_kv_cache& x) { x.block_stride = -4096; });
  push([](pa_kv_cache& x) { x.k_scale = 2.f; });                           // not FP8
  push([](pa_kv_cache& x) { x.dtype = PA_FP8_E4M3; x.k_scale = 0.f; });
  push([](pa_kv_cache& x) { x.dtype = PA_FP8_E4M3; x.v_scale = -1.f; });
  // extreme sizes: products that do not fit 64 bits must be refused, not
  // wrapped
  push([](pa_kv_cache& x) { x.num_layers = 0x7fffffff; x.layer_stride = INT64_MAX / 4; });
  push([](pa_kv_cache& x) { x.num_blocks = 0x7fffffff; x.block_stride = INT64_MAX / 2; });
  push([](pa_kv_cache& x) {
    x.num_kv_heads = 0x7fffffff; x.block_size = 256; x.head_dim = 0x7fffff00;
  });
  push([](pa_kv_cache& x) { x.layer_stride = INT64_MAX; x.block_stride = INT64_MAX; });
}

static void api_cases() {
  std::vector<pa_kv_cache> bad;
  geometry_cases(bad);
  int64_t pairs_host[8] = {0, 1, 2, 1, 5, 200, -1, 3};     // duplicate dst, out of range
  int32_t tables[64] = {0}, ctx[8] = {0};
  for (const pa_kv_cache& c : bad) {
    CHECK(refused(pa_write_kv(&c, 0, FAKE, FAKE, PA_BF16, (const int64_t*)FAKE, 4, nullptr)));
    CHECK(refused(pa_decode(&c, 0, FAKE, PA_BF16, FAKE, tables, 8, ctx, 100, 4, 32, 0.1f, FAKE,
                            1 << 30, nullptr)));
    CHECK(refused(pa_decode_no_alloc(&c, 0, FAKE, PA_BF16, FAKE, tables, 8, ctx, 100, 4, 32,
                                     0.1f, nullptr)));
    CHECK(refused(pa_decode_shared(&c, 0, FAKE, PA_BF16, FAKE, tables, 8, ctx, 100, 4, 32, 0.1f,
                                   0, FAKE, 1 << 30, nullptr)));
    CHECK(refused(pa_prefill(&c, 0, FAKE, PA_BF16, FAKE, tables, 8, ctx, 100, (const int32_t*)FAKE,
                             16, 4, 64, 32, 0.1f, nullptr)));
    CHECK(refused(pa_copy_blocks(&c, &c, pairs_host, 2, PA_COPY_H2D, nullptr)));
    CHECK(refused(pa_copy_blocks_staged(&c, &c, pairs_host, 2, PA_COPY_D2H, FAKE, 1 << 30, nullptr)));
    if (c.k) {   // the size queries need no data pointers
      CHECK(pa_decode_workspace_size(&c, 4, 32, 100) == 0);
      CHECK(pa_decode_shared_workspace_size(&c, 4, 32) == 0);
      CHECK(pa_copy_staging_size(&c, 4) == 0);
      CHECK(pa_decode_partition_tokens(&c, 4, 32, 100) == 0);
    }
  }
  // well-formed pool, bad call arguments
  pa_kv_cache c = cache(PA_BF16, 100, 2, 8, 16, 128);
  CHECK(pa_write_kv(&c, 2, FAKE, FAKE, PA_BF16, (const int64_t*)FAKE, 4, nullptr) == PA_ERR_INVALID_ARG);
  CHECK(pa_write_kv(&c, 0, FAKE, FAKE, PA_F16, (const int64_t*)FAKE, 4, nullptr) == PA_ERR_INVALID_ARG);
  CHECK(pa_write_kv(&c, 0, nullptr, FAKE, PA_BF16, (const int64_t*)FAKE, 4, nullptr) == PA_ERR_INVALID_ARG);
  CHECK(pa_write_kv(&c, 0, FAKE, FAKE, PA_BF16, (const int64_t*)FAKE, -1, nullptr) == PA_ERR_INVALID_ARG);
  CHECK(pa_write_kv(&c, 0, (char*)FAKE + 2, FAKE, PA_BF16, (const int64_t*)FAKE, 4, nullptr) == PA_ERR_UNSUPPORTED);
  CHECK(pa_decode(&c, 0, FAKE, PA_BF16, FAKE, tables, 8, ctx, 100, 4, 30, 0.1f, FAKE, 1 << 30, nullptr) == PA_ERR_INVALID_ARG);
  CHECK(pa_decode(&c, 0, FAKE, PA_BF16, FAKE, tables, 8, ctx, 100, 4, 32, 0.1f, nullptr, 0, nullptr) == PA_ERR_WORKSPACE);
  CHECK(pa_decode(&c, 0, FAKE, PA_BF16, FAKE, tables, 8, ctx, -1, 4, 32, 0.1f, FAKE, 1 << 30, nullptr) == PA_ERR_INVALID_ARG);
  CHECK(pa_decode(&c, 0, FAKE, PA_BF16, FAKE, tables, 0x7fffffff, ctx, 100, 4, 32, 0.1f, FAKE, 1 << 30, nullptr) != PA_OK);
  CHECK(pa_decode(&c, 0, FAKE, PA_BF16, FAKE, tables, 8, ctx, 100, 4, 32, 1.f / 0.f, FAKE, 1 << 30, nullptr) == PA_ERR_INVALID_ARG);
  CHECK(pa_decode(&c, 0, FAKE, PA_F16, FAKE, tables, 8, ctx, 100, 4, 32, 0.1f, FAKE, 1 << 30, nullptr) == PA_ERR_UNSUPPORTED);
  CHECK(pa_decode(&c, 0, FAKE, PA_BF16, FAKE, tables, 8, ctx, 100, 4, 8 * 32, 0.1f, FAKE, 1 << 30, nullptr) == PA_ERR_UNSUPPORTED);
  CHECK(pa_decode_no_alloc(&c, 0, FAKE, PA_BF16, FAKE, tables, 8, ctx, 4000, 8192, 32, 0.1f, nullptr) == PA_ERR_WORKSPACE);
  CHECK(pa_decode_no_alloc(&c, 0, nullptr, PA_BF16, FAKE, tables, 8, ctx, 100, 4, 32, 0.1f, nullptr) == PA_ERR_INVALID_ARG);
  CHECK(pa_decode_shared(&c, 0, FAKE, PA_BF16, FAKE, tables, 8, ctx, 100, 4, 32, 0.1f, 2, FAKE, 1 << 30, nullptr) == PA_ERR_INVALID_ARG);
  CHECK(pa_decode_shared(&c, 0, FAKE, PA_BF16, FAKE, tables, 8, ctx, 100, 4, 32, 0.1f, 0, FAKE, 16, nullptr) == PA_ERR_WORKSPACE);
  CHECK(pa_prefill(&c, 0, FAKE, PA_BF16, FAKE, tables, 8, ctx, 100, nullptr, 16, 4, 64, 32, 0.1f, nullptr) == PA_ERR_INVALID_ARG);
  CHECK(pa_prefill(&c, 0, FAKE, PA_F32, FAKE, tables, 8, ctx, 100, (const int32_t*)FAKE, 16, 4, 64, 32, 0.1f, nullptr) == PA_ERR_UNSUPPORTED);
  CHECK(pa_prefill(&c, 0, FAKE, PA_BF16, FAKE, tables, 8, ctx, 100, (const int32_t*)FAKE, 0x7fffffff, 4, 64, 32, 0.1f, nullptr) == PA_ERR_UNSUPPORTED);
  // host pair lists: out of range or duplicate destinations, before any copy
  pa_kv_cache h = c;
  CHECK(pa_copy_blocks(&c, &h, pairs_host, 4, PA_COPY_H2D, nullptr) == PA_ERR_INVALID_ARG);
  CHECK(pa_copy_blocks(&h, &c, pairs_host + 4, 2, PA_COPY_D2H, nullptr) == PA_ERR_INVALID_ARG);
  CHECK(pa_copy_blocks(&c, &h, pairs_host, 2, (pa_copy_dir)7, nullptr) == PA_ERR_INVALID_ARG);
  CHECK(pa_copy_blocks(&c, &h, nullptr, 2, PA_COPY_H2D, nullptr) == PA_ERR_INVALID_ARG);
  CHECK(pa_copy_blocks(&c, &h, pairs_host, -2, PA_COPY_H2D, nullptr) == PA_ERR_INVALID_ARG);
  pa_kv_cache other = cache(PA_BF16, 100, 2, 8, 16, 64);
  CHECK(pa_copy_blocks(&c, &other, pairs_host, 1, PA_COPY_D2D, nullptr) == PA_ERR_INVALID_ARG);
  CHECK(pa_copy_blocks_staged(&c, &h, pairs_host, 4, PA_COPY_H2D, FAKE, 1 << 30, nullptr) == PA_ERR_INVALID_ARG);
  CHECK(pa_copy_blocks_staged(&c, &h, pairs_host, 1, PA_COPY_H2D, FAKE, 16, nullptr) == PA_ERR_WORKSPACE);
  CHECK(pa_copy_blocks_staged(&c, &h, pairs_host, 1, PA_COPY_D2D, FAKE, 1 << 30, nullptr) == PA_ERR_INVALID_ARG);
  // queries on valid geometry
  CHECK(pa_decode_workspace_size(&c, 256, 32, 4000) > 0);
  CHECK(pa_decode_shared_workspace_size(&c, 256, 32) > 0);
  CHECK(pa_copy_staging_size(&c, 94) == (size_t)94 * 2 * 2 * 8 * 16 * 128 * 2);
  CHECK(pa_decode_partition_tokens(&c, 256, 32, 4000) == 16);
  for (int s = -1; s < 8; ++s) CHECK(pa_status_string((pa_status)s) != nullptr);
  CHECK(pa_version() != nullptr);
  CHECK(pa_bm_create(0, 16, nullptr, 0, nullptr) == PA_ERR_INVALID_ARG);
  pa_bm* bm = nullptr;
  const int32_t not_perm[3] = {0, 0, 1};
  CHECK(pa_bm_create(3, 16, not_perm, 0, &bm) == PA_ERR_INVALID_ARG && !bm);
  CHECK(pa_bm_create(3, 0, nullptr, 0, &bm) == PA_ERR_INVALID_ARG && !bm);
}

int main() {
  for (uint32_t seed = 1; seed <= 200; ++seed) bm_trace(seed);
  api_cases();
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("host sanitizer driver: all checks passed\n");
  return 0;
}
