// Random operation sequences, valid and invalid, against the host side of
// libpkv (allocator, copy-on-write, retention pool, prepare_step, planner,
// table validation).  Built with AddressSanitizer and UBSan on the CPU by
// test_host_sanitized.py: it looks for memory errors, leaks and undefined
// behaviour only; results are checked against the oracle elsewhere.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>
#include "pkv.h"
int main() {
  std::mt19937 rng(1234);
  for (int trial = 0; trial < 300; ++trial) {
    int np = 1 + rng() % 64, ps = 1 + rng() % 17;
    pkv_alloc* a = nullptr;
    std::vector<int32_t> order(np);
    for (int i = 0; i < np; ++i) order[i] = i;
    std::shuffle(order.begin(), order.end(), rng);
    if (pkv_alloc_create(np, ps, (rng() & 1) ? order.data() : nullptr, &a) != PKV_OK) return 1;
    std::vector<int32_t> seqs;
    for (int op = 0; op < 400; ++op) {
      int k = rng() % 13;
      int32_t s = seqs.empty() ? -1 : seqs[rng() % seqs.size()];
      int32_t t = seqs.empty() ? -1 : seqs[rng() % seqs.size()];
      int32_t n = (int32_t)(rng() % 40) - 3;
      int32_t out2[2], nc, avail, len;
      int64_t pages;
      switch (k) {
        case 0: { int32_t id; if (pkv_seq_new(a, &id) == PKV_OK) seqs.push_back(id); break; }
        case 1: pkv_reserve(a, s, n); break;
        case 2: pkv_truncate(a, s, n); break;
        case 3: pkv_release(a, s); break;
        case 4: pkv_share_prefix(a, t, s, n * ps / 4); break;
        case 5: pkv_fork(a, t, s); break;
        case 6: pkv_reserve_cow(a, s, n, out2, &nc); break;
        case 7: pkv_retention_add(a, s, (rng() % 100) / 100.0, (rng() % 100) / 10.0); break;
        case 8: { std::vector<int32_t> ev(rng() % 5); int32_t ne; pkv_retention_evict(a, rng() % 80, ev.data(), (int32_t)ev.size(), &ne); break; }
        case 9: pkv_retention_take(a, s, &avail); pkv_retention_pages(a, &pages); break;
        case 10: {
          int stride = rng() % 8;
          std::vector<int32_t> ids(seqs.begin(), seqs.begin() + std::min<size_t>(seqs.size(), 5));
          std::vector<int32_t> bt(ids.size() * (size_t)std::max(stride, 1));
          pkv_block_tables(a, ids.data(), (int32_t)ids.size(), stride, bt.data());
          break;
        }
        case 11: {
          if (pkv_seq_len(a, s, &len) == PKV_OK && len > 0) {
            int32_t st0 = rng() % len, cnt = rng() % (len - st0 + 2);
            std::vector<int64_t> sl(cnt + 1);
            pkv_slots(a, s, st0, cnt, sl.data());
          }
          break;
        }
        case 12: {
          std::vector<int32_t> ids;
          for (int32_t x : seqs) if (rng() % 3 == 0 && ids.size() < 6) ids.push_back(x);
          std::vector<int32_t> nn(ids.size());
          for (auto& x : nn) x = rng() % 9;
          int stride = rng() % 10;
          int64_t tot = 0; for (auto x : nn) tot += x;
          std::vector<int64_t> sl(tot + 1);
          std::vector<int32_t> bt(ids.size() * (size_t)std::max(stride, 1) + 1), ln(ids.size() + 1);
          pkv_prepare_step(a, ids.data(), (int32_t)ids.size(), nn.data(), stride, sl.data(), stride ? bt.data() : nullptr, ln.data());
          break;
        }
      }
    }
    pkv_alloc_destroy(a);
  }
  // planner
  for (int trial = 0; trial < 200; ++trial) {
    int nd = rng() % 12;
    std::vector<int64_t> off(nd + 1, 0);
    std::vector<int32_t> tok;
    for (int d = 0; d < nd; ++d) { int L = rng() % 30; for (int i = 0; i < L; ++i) tok.push_back(rng() % 3); off[d + 1] = tok.size(); }
    std::vector<int32_t> o(nd + 1), p(nd + 1), sh(nd + 1);
    tok.push_back(0);
    pkv_plan_prefix(tok.data(), off.data(), nd, 1 + rng() % 5, o.data(), p.data(), sh.data());
  }
  // validate_tables
  pkv_pool_desc d{PKV_BF16, 50, 16, 8, 128};
  for (int trial = 0; trial < 200; ++trial) {
    int n = rng() % 6, stride = rng() % 6;
    std::vector<int32_t> bt(n * std::max(stride, 1) + 1), ln(n + 1), cu(n + 2);
    for (auto& x : bt) x = (int32_t)(rng() % 70) - 5;
    for (auto& x : ln) x = (int32_t)(rng() % 120) - 5;
    cu[0] = 0; for (int i = 1; i <= n; ++i) cu[i] = cu[i - 1] + rng() % 4;
    pkv_validate_tables(&d, bt.data(), n, stride, ln.data(), (rng() & 1) ? cu.data() : nullptr, rng() % 5);
  }
  std::printf("fuzz done\n");
  return 0;
}
