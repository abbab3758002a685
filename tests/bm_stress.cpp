// Stress driver for the host block manager through its C ABI, meant to be
// built with AddressSanitizer and UndefinedBehaviorSanitizer (see
// tests/test_block_manager_sanitized.py).  Random allocate / append / fork /
// free sequences on small pools; after every operation the state seen through
// the inspection calls must be consistent:
//   - every live sequence's table has ceil(tokens / block_size) blocks and its
//     length is the number of tokens the driver gave it;
//   - a block's reference count is the number of live tables naming it;
//   - the free queue holds exactly the blocks nobody references, once each,
//     and its length is pa_bm_num_free;
//   - a copy-on-write pair moves off a block still referenced elsewhere.
// Exit status 0 when every check holds.
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <vector>

#include "pa_block_manager.h"

namespace {

int fail(const char* what, long a = 0, long b = 0) {
  std::fprintf(stderr, "bm_stress: %s (%ld, %ld)\n", what, a, b);
  std::exit(1);
}

void check_state(pa_block_manager* m, int nb, int bs, const std::map<long, int>& live) {
  std::vector<int> refs(nb, 0);
  for (const auto& kv : live) {
    const long id = kv.first;
    std::vector<int32_t> row(nb > 0 ? nb : 1);
    int32_t len = -1;
    if (pa_bm_tables(m, &id, 1, nb, row.data(), &len) != PA_OK) fail("tables", id);
    if (len != kv.second) fail("length", len, kv.second);
    const int want = (kv.second + bs - 1) / bs;
    for (int j = 0; j < nb; ++j) {
      if (j < want) {
        if (row[j] < 0 || row[j] >= nb) fail("block id", row[j]);
        ++refs[row[j]];
      } else if (row[j] != -1) {
        fail("padding", j, row[j]);
      }
    }
  }
  std::vector<int32_t> queue(nb > 0 ? nb : 1);
  int32_t count = -1;
  if (pa_bm_free_queue(m, queue.data(), nb, &count) != PA_OK) fail("free queue");
  if (count != pa_bm_num_free(m)) fail("queue length", count, pa_bm_num_free(m));
  std::vector<int> in_queue(nb, 0);
  for (int i = 0; i < count; ++i) {
    if (queue[i] < 0 || queue[i] >= nb) fail("queued id", queue[i]);
    if (in_queue[queue[i]]++) fail("queued twice", queue[i]);
  }
  for (int b = 0; b < nb; ++b) {
    int32_t ref = -1, has = -1, reg = -1;
    uint8_t digest[32];
    if (pa_bm_block_info(m, b, &ref, &has, digest, &reg) != PA_OK) fail("block info", b);
    if (ref != refs[b]) fail("reference count", b, ref);
    if ((ref == 0) != (in_queue[b] == 1)) fail("free queue membership", b, ref);
    if (reg && !has) fail("registered without a digest", b);
  }
}

}  // namespace

int main() {
  const int configs[][3] = {{24, 4, 1}, {40, 2, 1}, {30, 4, 0}, {64, 8, 1}, {12, 1, 1}, {0, 16, 1}};
  std::mt19937 rng(12345);
  long total_ops = 0, cows = 0, out_of_blocks = 0;
  for (const auto& cfg : configs) {
    const int nb = cfg[0], bs = cfg[1];
    pa_block_manager* m = nullptr;
    if (pa_bm_create(nb, bs, cfg[2], &m) != PA_OK || !m) fail("create");
    std::map<long, int> live;
    long next_id = 0;
    std::vector<std::vector<int32_t>> bases(3);
    for (auto& b : bases)
      for (int i = 0; i < 3 * bs + 1; ++i) b.push_back(int32_t(rng() % 50));
    for (int step = 0; step < 3000; ++step, ++total_ops) {
      const double r = std::uniform_real_distribution<double>(0, 1)(rng);
      std::vector<long> ids;
      for (const auto& kv : live) ids.push_back(kv.first);
      if (r < 0.2 || ids.empty()) {
        const auto& base = bases[rng() % 3];
        std::vector<int32_t> prompt(base.begin(), base.begin() + rng() % (base.size() + 1));
        for (int i = rng() % (bs + 2); i > 0; --i) prompt.push_back(int32_t(rng() % 50));
        const char salt[] = "tenant";
        const bool salted = rng() % 3 == 0;
        int32_t hit = -1;
        const pa_status s = pa_bm_allocate(m, next_id, prompt.data(), int32_t(prompt.size()),
                                           salted ? salt : nullptr, salted ? 6 : 0, &hit);
        if (s == PA_OK) {
          if (hit < 0 || hit % bs != 0 || (hit > 0 && hit >= int32_t(prompt.size())))
            fail("cached tokens", hit, long(prompt.size()));
          live[next_id] = int(prompt.size());
        } else if (s == PA_ERR_OUT_OF_BLOCKS) {
          ++out_of_blocks;
        } else {
          fail("allocate status", s);
        }
        // a live id is refused, and changes nothing
        if (!live.empty() && pa_bm_allocate(m, live.begin()->first, nullptr, 0, nullptr, 0,
                                            nullptr) != PA_ERR_INVALID_ARGUMENT)
          fail("duplicate id accepted");
        ++next_id;
      } else if (r < 0.75) {
        const int k = 1 + int(rng() % 3);
        std::vector<int64_t> seqs;
        std::vector<int32_t> toks;
        for (int i = 0; i < k; ++i) {
          seqs.push_back(ids[rng() % ids.size()]);
          toks.push_back(int32_t(rng() % 50));
        }
        std::vector<int32_t> slots(k), pairs(2 * k);
        int32_t ncow = -1;
        const pa_status s =
            pa_bm_append(m, seqs.data(), toks.data(), k, slots.data(), pairs.data(), &ncow);
        if (s == PA_OK) {
          for (int i = 0; i < k; ++i) {
            if (slots[i] < 0 || slots[i] >= nb * bs) fail("slot", slots[i]);
            ++live[seqs[i]];
          }
          if (ncow < 0 || ncow > k) fail("copy-on-write count", ncow);
          for (int i = 0; i < ncow; ++i) {
            int32_t ref = -1;
            pa_bm_block_info(m, pairs[2 * i], &ref, nullptr, nullptr, nullptr);
            if (ref < 1) fail("copied block has no other reader", pairs[2 * i], ref);
          }
          cows += ncow;
        } else if (s == PA_ERR_OUT_OF_BLOCKS) {
          ++out_of_blocks;
          if (!ids.empty()) {
            pa_bm_free(m, ids.front());
            live.erase(ids.front());
          }
        } else {
          fail("append status", s);
        }
      } else if (r < 0.87) {
        const long parent = ids[rng() % ids.size()];
        if (pa_bm_fork(m, parent, next_id) != PA_OK) fail("fork");
        live[next_id] = live[parent];
        ++next_id;
      } else {
        const long id = ids[rng() % ids.size()];
        if (pa_bm_free(m, id) != PA_OK) fail("free");
        live.erase(id);
        if (pa_bm_free(m, id) != PA_ERR_INVALID_ARGUMENT) fail("double free accepted");
      }
      check_state(m, nb, bs, live);
    }
    pa_bm_destroy(m);
  }
  std::printf("bm_stress: %ld operations, %ld copy-on-write pairs, %ld out-of-blocks refusals\n",
              total_ops, cows, out_of_blocks);
  return 0;
}
