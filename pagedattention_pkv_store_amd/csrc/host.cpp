// Host half of libpkv: the page allocator, slot computation, block-table
// export, the prefix-sharing planner and the host-side table validator.
//
// Sources for the behaviour (see include/pkv.h for each call's contract):
//  * TileInfer.jl docs "KV cache", "Pages and block tables" (free-page stack,
//    block tables, slots = page and offset) and "Growing, rolling back,
//    releasing" (reserve!, truncate!, release!, OutOfPagesError).
//  * "KV Cache Management and PagedAttention", Figures 1-3 (a block is taken
//    only when the last one is full) and "Return blocks after a request ends"
//    (reference counts).
//  * Quail docs "KV", "Paged KV" (pages shared by reference, free when
//    unreferenced), "The sharing plan" (sorted-adjacent planning) and
//    "Execution" (adoption without copying).
//
// Nothing here touches the GPU; the allocator runs in microseconds per call
// and produces the int32/int64 arrays the kernels consume.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <numeric>
#include <set>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/pkv.h"
#include "status.h"

namespace pkv {

static thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

}  // namespace pkv

using pkv::fail;

struct pkv_alloc {
  struct Seq {
    std::vector<int32_t> table;
    int32_t len = 0;
    bool live = false;
  };
  int32_t num_pages = 0;
  int32_t page_size = 1;
  std::vector<int32_t> free_stack;  // top = back()
  std::vector<int32_t> refcount;
  std::vector<Seq> seqs;            // index = sequence id

  // KV retention pool: (priority, entry order, sequence), lowest first, and
  // each retained sequence's page count at entry (0 = not retained).
  std::set<std::tuple<double, int64_t, int32_t>> retained;
  std::vector<int32_t> ret_pages_of;
  std::vector<std::pair<double, int64_t>> ret_key_of;
  int64_t ret_pages = 0;
  int64_t ret_order = 0;
  void retention_drop(int32_t seq) {
    if (seq < static_cast<int32_t>(ret_pages_of.size()) && ret_pages_of[seq] > 0) {
      retained.erase(std::make_tuple(ret_key_of[seq].first, ret_key_of[seq].second, seq));
      ret_pages -= ret_pages_of[seq];
      ret_pages_of[seq] = 0;
    }
  }

  const Seq* find(int32_t id) const {
    if (id < 0 || id >= static_cast<int32_t>(seqs.size()) || !seqs[id].live) return nullptr;
    return &seqs[id];
  }
  Seq* find(int32_t id) {
    return const_cast<Seq*>(static_cast<const pkv_alloc*>(this)->find(id));
  }
  static int64_t blocks_for(int64_t len, int32_t ps) { return (len + ps - 1) / ps; }

  // Drop references to logical blocks >= keep_blocks, last block first.
  void drop_blocks(Seq& s, size_t keep_blocks) {
    for (size_t i = s.table.size(); i > keep_blocks; --i) {
      int32_t page = s.table[i - 1];
      if (--refcount[page] == 0) free_stack.push_back(page);
    }
    s.table.resize(keep_blocks);
  }
};

extern "C" {

const char* pkv_last_error(void) { return pkv::g_last_error.c_str(); }

int pkv_alloc_create(int32_t num_pages, int32_t page_size, const int32_t* free_order,
                     pkv_alloc** out) {
  if (!out) return fail(PKV_ERR_INVALID_ARG, "pkv_alloc_create: out is NULL");
  *out = nullptr;
  if (num_pages < 0) return fail(PKV_ERR_INVALID_ARG, "pkv_alloc_create: num_pages < 0");
  if (page_size < 1) return fail(PKV_ERR_INVALID_ARG, "pkv_alloc_create: page_size < 1");
  std::vector<int32_t> order(num_pages);
  if (free_order) {
    std::vector<char> seen(num_pages, 0);
    for (int32_t i = 0; i < num_pages; ++i) {
      int32_t p = free_order[i];
      if (p < 0 || p >= num_pages || seen[p])
        return fail(PKV_ERR_INVALID_ARG, "pkv_alloc_create: free_order is not a permutation");
      seen[p] = 1;
      order[i] = p;
    }
  } else {
    std::iota(order.begin(), order.end(), 0);
  }
  auto* a = new pkv_alloc;
  a->num_pages = num_pages;
  a->page_size = page_size;
  a->free_stack.assign(order.rbegin(), order.rend());  // first pop = order[0]
  a->refcount.assign(num_pages, 0);
  *out = a;
  return PKV_OK;
}

void pkv_alloc_destroy(pkv_alloc* a) { delete a; }

int pkv_seq_new(pkv_alloc* a, int32_t* seq_out) {
  if (!a || !seq_out) return fail(PKV_ERR_INVALID_ARG, "pkv_seq_new: NULL argument");
  if (a->seqs.size() >= static_cast<size_t>(INT32_MAX))
    return fail(PKV_ERR_INVALID_ARG, "pkv_seq_new: sequence ids exhausted");
  a->seqs.emplace_back();
  a->seqs.back().live = true;
  *seq_out = static_cast<int32_t>(a->seqs.size() - 1);
  return PKV_OK;
}

int pkv_reserve(pkv_alloc* a, int32_t seq, int32_t n) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "pkv_reserve: NULL allocator");
  pkv_alloc::Seq* s = a->find(seq);
  if (!s) return fail(PKV_ERR_INVALID_ARG, "pkv_reserve: unknown sequence " + std::to_string(seq));
  if (n < 0) return fail(PKV_ERR_INVALID_ARG, "pkv_reserve: n < 0");
  const int32_t ps = a->page_size;
  const int64_t new_len = static_cast<int64_t>(s->len) + n;
  if (new_len > INT32_MAX) return fail(PKV_ERR_INVALID_ARG, "pkv_reserve: length overflows int32");
  if (n > 0 && s->len % ps != 0 && a->refcount[s->table[s->len / ps]] > 1)
    return fail(PKV_ERR_SHARED_PAGE,
                "pkv_reserve: next position falls in a page other sequences reference");
  const int64_t need = pkv_alloc::blocks_for(new_len, ps) - static_cast<int64_t>(s->table.size());
  if (need > static_cast<int64_t>(a->free_stack.size()))
    return fail(PKV_ERR_OUT_OF_PAGES, "pkv_reserve: need " + std::to_string(need) + " pages, " +
                                          std::to_string(a->free_stack.size()) + " free");
  for (int64_t i = 0; i < need; ++i) {
    int32_t page = a->free_stack.back();
    a->free_stack.pop_back();
    a->refcount[page] = 1;
    s->table.push_back(page);
  }
  s->len = static_cast<int32_t>(new_len);
  return PKV_OK;
}

int pkv_truncate(pkv_alloc* a, int32_t seq, int32_t n_keep) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "pkv_truncate: NULL allocator");
  pkv_alloc::Seq* s = a->find(seq);
  if (!s) return fail(PKV_ERR_INVALID_ARG, "pkv_truncate: unknown sequence " + std::to_string(seq));
  if (n_keep < 0 || n_keep > s->len)
    return fail(PKV_ERR_INVALID_ARG, "pkv_truncate: n_keep outside 0..len");
  a->drop_blocks(*s, static_cast<size_t>(pkv_alloc::blocks_for(n_keep, a->page_size)));
  s->len = n_keep;
  return PKV_OK;
}

int pkv_release(pkv_alloc* a, int32_t seq) {
  int rc = pkv_truncate(a, seq, 0);
  if (rc != PKV_OK) return rc;
  a->retention_drop(seq);
  a->seqs[seq].live = false;
  a->seqs[seq].table.shrink_to_fit();
  return PKV_OK;
}

int pkv_share_prefix(pkv_alloc* a, int32_t child, int32_t parent, int32_t n_tokens) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "pkv_share_prefix: NULL allocator");
  pkv_alloc::Seq* c = a->find(child);
  const pkv_alloc::Seq* p = a->find(parent);
  if (!c || !p) return fail(PKV_ERR_INVALID_ARG, "pkv_share_prefix: unknown sequence");
  if (child == parent) return fail(PKV_ERR_INVALID_ARG, "pkv_share_prefix: child == parent");
  if (c->len != 0) return fail(PKV_ERR_INVALID_ARG, "pkv_share_prefix: child is not empty");
  if (n_tokens < 0 || n_tokens % a->page_size != 0 || n_tokens > p->len)
    return fail(PKV_ERR_INVALID_ARG,
                "pkv_share_prefix: n_tokens must be whole pages within the parent");
  const size_t npg = static_cast<size_t>(n_tokens / a->page_size);
  c->table.assign(p->table.begin(), p->table.begin() + npg);
  for (int32_t page : c->table) ++a->refcount[page];
  c->len = n_tokens;
  return PKV_OK;
}

int pkv_fork(pkv_alloc* a, int32_t child, int32_t parent) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "pkv_fork: NULL allocator");
  pkv_alloc::Seq* c = a->find(child);
  const pkv_alloc::Seq* p = a->find(parent);
  if (!c || !p) return fail(PKV_ERR_INVALID_ARG, "pkv_fork: unknown sequence");
  if (child == parent) return fail(PKV_ERR_INVALID_ARG, "pkv_fork: child == parent");
  if (c->len != 0) return fail(PKV_ERR_INVALID_ARG, "pkv_fork: child is not empty");
  c->table = p->table;
  for (int32_t page : c->table) ++a->refcount[page];
  c->len = p->len;
  return PKV_OK;
}

int pkv_reserve_cow(pkv_alloc* a, int32_t seq, int32_t n, int32_t* copy_out, int32_t* n_copies) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "pkv_reserve_cow: NULL allocator");
  if (!copy_out || !n_copies) return fail(PKV_ERR_INVALID_ARG, "pkv_reserve_cow: NULL output");
  pkv_alloc::Seq* s = a->find(seq);
  if (!s) return fail(PKV_ERR_INVALID_ARG, "pkv_reserve_cow: unknown sequence " + std::to_string(seq));
  if (n < 0) return fail(PKV_ERR_INVALID_ARG, "pkv_reserve_cow: n < 0");
  const int32_t ps = a->page_size;
  const int64_t new_len = static_cast<int64_t>(s->len) + n;
  if (new_len > INT32_MAX) return fail(PKV_ERR_INVALID_ARG, "pkv_reserve_cow: length overflows int32");
  const bool copy = n > 0 && s->len % ps != 0 && a->refcount[s->table[s->len / ps]] > 1;
  const int64_t need =
      pkv_alloc::blocks_for(new_len, ps) - static_cast<int64_t>(s->table.size()) + (copy ? 1 : 0);
  if (need > static_cast<int64_t>(a->free_stack.size()))
    return fail(PKV_ERR_OUT_OF_PAGES, "pkv_reserve_cow: need " + std::to_string(need) + " pages, " +
                                          std::to_string(a->free_stack.size()) + " free");
  *n_copies = 0;
  if (copy) {
    // the writer takes a fresh page first; the shared one loses its reference
    const size_t blk = static_cast<size_t>(s->len / ps);
    const int32_t shared = s->table[blk];
    const int32_t fresh = a->free_stack.back();
    a->free_stack.pop_back();
    --a->refcount[shared];
    a->refcount[fresh] = 1;
    s->table[blk] = fresh;
    copy_out[0] = shared;
    copy_out[1] = fresh;
    *n_copies = 1;
  }
  return pkv_reserve(a, seq, n);   // cannot fail now: pages were counted above
}

int pkv_retention_add(pkv_alloc* a, int32_t seq, double probability_of_reuse, double recompute_seconds) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "pkv_retention_add: NULL allocator");
  const pkv_alloc::Seq* s = a->find(seq);
  if (!s) return fail(PKV_ERR_INVALID_ARG, "pkv_retention_add: unknown sequence " + std::to_string(seq));
  if (seq < static_cast<int32_t>(a->ret_pages_of.size()) && a->ret_pages_of[seq] > 0)
    return fail(PKV_ERR_INVALID_ARG, "pkv_retention_add: sequence already retained");
  if (s->table.empty()) return fail(PKV_ERR_INVALID_ARG, "pkv_retention_add: an empty sequence holds no KV");
  if (!(probability_of_reuse >= 0.0) || !(recompute_seconds >= 0.0) || !std::isfinite(probability_of_reuse) ||
      !std::isfinite(recompute_seconds))
    return fail(PKV_ERR_INVALID_ARG, "pkv_retention_add: probability and seconds must be finite and >= 0");
  const int32_t pages = static_cast<int32_t>(s->table.size());
  const double prio = probability_of_reuse * recompute_seconds / pages;   // saving per page
  if (a->ret_pages_of.size() < a->seqs.size()) {
    a->ret_pages_of.resize(a->seqs.size(), 0);
    a->ret_key_of.resize(a->seqs.size());
  }
  const int64_t order = a->ret_order++;
  a->retained.emplace(prio, order, seq);
  a->ret_key_of[seq] = {prio, order};
  a->ret_pages_of[seq] = pages;
  a->ret_pages += pages;
  return PKV_OK;
}

int pkv_retention_evict(pkv_alloc* a, int64_t limit_pages, int32_t* evicted, int32_t max_evicted,
                        int32_t* n_evicted) {
  if (!a || !n_evicted) return fail(PKV_ERR_INVALID_ARG, "pkv_retention_evict: NULL argument");
  if (limit_pages < 0 || max_evicted < 0) return fail(PKV_ERR_INVALID_ARG, "pkv_retention_evict: negative size");
  // choose first, so a too-small output array leaves everything unchanged
  std::vector<int32_t> chosen;
  int64_t pages = a->ret_pages;
  for (auto it = a->retained.begin(); it != a->retained.end() && pages > limit_pages; ++it) {
    const int32_t seq = std::get<2>(*it);
    chosen.push_back(seq);
    pages -= a->ret_pages_of[seq];
  }
  if (static_cast<int64_t>(chosen.size()) > max_evicted || (!chosen.empty() && !evicted))
    return fail(PKV_ERR_BUFFER_TOO_SMALL, "pkv_retention_evict: " + std::to_string(chosen.size()) +
                                              " sequences to evict");
  for (size_t i = 0; i < chosen.size(); ++i) {
    evicted[i] = chosen[i];
    pkv_release(a, chosen[i]);   // drops it from the pool too
  }
  *n_evicted = static_cast<int32_t>(chosen.size());
  return PKV_OK;
}

int pkv_retention_take(pkv_alloc* a, int32_t seq, int32_t* available) {
  if (!a || !available) return fail(PKV_ERR_INVALID_ARG, "pkv_retention_take: NULL argument");
  *available = (seq >= 0 && seq < static_cast<int32_t>(a->ret_pages_of.size()) && a->ret_pages_of[seq] > 0) ? 1 : 0;
  if (*available) a->retention_drop(seq);
  return PKV_OK;
}

int pkv_retention_pages(const pkv_alloc* a, int64_t* pages) {
  if (!a || !pages) return fail(PKV_ERR_INVALID_ARG, "pkv_retention_pages: NULL argument");
  *pages = a->ret_pages;
  return PKV_OK;
}

int pkv_seq_len(const pkv_alloc* a, int32_t seq, int32_t* len) {
  if (!a || !len) return fail(PKV_ERR_INVALID_ARG, "pkv_seq_len: NULL argument");
  const pkv_alloc::Seq* s = a->find(seq);
  if (!s) return fail(PKV_ERR_INVALID_ARG, "pkv_seq_len: unknown sequence " + std::to_string(seq));
  *len = s->len;
  return PKV_OK;
}

int pkv_num_free(const pkv_alloc* a, int32_t* n) {
  if (!a || !n) return fail(PKV_ERR_INVALID_ARG, "pkv_num_free: NULL argument");
  *n = static_cast<int32_t>(a->free_stack.size());
  return PKV_OK;
}

int pkv_page_refcount(const pkv_alloc* a, int32_t page, int32_t* count) {
  if (!a || !count) return fail(PKV_ERR_INVALID_ARG, "pkv_page_refcount: NULL argument");
  if (page < 0 || page >= a->num_pages)
    return fail(PKV_ERR_INVALID_ARG, "pkv_page_refcount: page out of range");
  *count = a->refcount[page];
  return PKV_OK;
}

int pkv_seq_num_blocks(const pkv_alloc* a, int32_t seq, int32_t* n) {
  if (!a || !n) return fail(PKV_ERR_INVALID_ARG, "pkv_seq_num_blocks: NULL argument");
  const pkv_alloc::Seq* s = a->find(seq);
  if (!s) return fail(PKV_ERR_INVALID_ARG, "pkv_seq_num_blocks: unknown sequence");
  *n = static_cast<int32_t>(s->table.size());
  return PKV_OK;
}

int pkv_block_tables(const pkv_alloc* a, const int32_t* seqs, int32_t n_seqs, int32_t stride,
                     int32_t* out) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "pkv_block_tables: NULL allocator");
  if (n_seqs < 0 || stride < 0) return fail(PKV_ERR_INVALID_ARG, "pkv_block_tables: negative size");
  if (n_seqs > 0 && (!seqs || !out)) return fail(PKV_ERR_INVALID_ARG, "pkv_block_tables: NULL array");
  for (int32_t b = 0; b < n_seqs; ++b) {
    const pkv_alloc::Seq* s = a->find(seqs[b]);
    if (!s) return fail(PKV_ERR_INVALID_ARG, "pkv_block_tables: unknown sequence " + std::to_string(seqs[b]));
    if (s->table.size() > static_cast<size_t>(stride))
      return fail(PKV_ERR_BUFFER_TOO_SMALL, "pkv_block_tables: a table is longer than stride");
  }
  for (int32_t b = 0; b < n_seqs; ++b) {
    const pkv_alloc::Seq* s = a->find(seqs[b]);
    int32_t* row = out + static_cast<int64_t>(b) * stride;
    std::copy(s->table.begin(), s->table.end(), row);
    std::fill(row + s->table.size(), row + stride, 0);
  }
  return PKV_OK;
}

int pkv_slots(const pkv_alloc* a, int32_t seq, int32_t start, int32_t n, int64_t* out) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "pkv_slots: NULL allocator");
  const pkv_alloc::Seq* s = a->find(seq);
  if (!s) return fail(PKV_ERR_INVALID_ARG, "pkv_slots: unknown sequence " + std::to_string(seq));
  if (start < 0 || n < 0 || static_cast<int64_t>(start) + n > s->len)
    return fail(PKV_ERR_INVALID_ARG, "pkv_slots: range outside the sequence");
  if (n > 0 && !out) return fail(PKV_ERR_INVALID_ARG, "pkv_slots: NULL out");
  const int32_t ps = a->page_size;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t p = start + i;
    out[i] = static_cast<int64_t>(s->table[p / ps]) * ps + p % ps;
  }
  return PKV_OK;
}

int pkv_prepare_step(pkv_alloc* a, const int32_t* seqs, int32_t n_seqs, const int32_t* n_new,
                     int32_t bt_stride, int64_t* slots_out, int32_t* bt_out,
                     int32_t* seq_lens_out) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "pkv_prepare_step: NULL allocator");
  if (n_seqs < 0 || bt_stride < 0) return fail(PKV_ERR_INVALID_ARG, "pkv_prepare_step: negative size");
  if (n_seqs == 0) return PKV_OK;
  if (!seqs || !n_new) return fail(PKV_ERR_INVALID_ARG, "pkv_prepare_step: NULL array");
  {
    std::vector<int32_t> ids(seqs, seqs + n_seqs);
    std::sort(ids.begin(), ids.end());
    if (std::adjacent_find(ids.begin(), ids.end()) != ids.end())
      return fail(PKV_ERR_INVALID_ARG, "pkv_prepare_step: a sequence appears twice");
  }
  for (int32_t b = 0; b < n_seqs; ++b) {
    if (!a->find(seqs[b]))
      return fail(PKV_ERR_INVALID_ARG, "pkv_prepare_step: unknown sequence " + std::to_string(seqs[b]));
    if (n_new[b] < 0) return fail(PKV_ERR_INVALID_ARG, "pkv_prepare_step: n_new < 0");
  }
  std::vector<int32_t> old_len(n_seqs);
  int rc = PKV_OK;
  std::string msg;
  int32_t done = 0;
  for (; done < n_seqs; ++done) {
    pkv_alloc::Seq* s = a->find(seqs[done]);
    old_len[done] = s->len;
    rc = pkv_reserve(a, seqs[done], n_new[done]);
    if (rc != PKV_OK) break;
    if (bt_out && s->table.size() > static_cast<size_t>(bt_stride)) {
      ++done;  // this reserve succeeded and must be undone too
      rc = fail(PKV_ERR_BUFFER_TOO_SMALL, "pkv_prepare_step: a block table is longer than bt_stride");
      break;
    }
  }
  if (rc != PKV_OK) {
    msg = pkv_last_error();
    for (int32_t b = done - 1; b >= 0; --b) pkv_truncate(a, seqs[b], old_len[b]);
    return fail(rc, msg);
  }
  int64_t k = 0;
  const int32_t ps = a->page_size;
  for (int32_t b = 0; b < n_seqs; ++b) {
    const pkv_alloc::Seq* s = a->find(seqs[b]);
    if (slots_out) {
      for (int32_t p = old_len[b]; p < s->len; ++p)
        slots_out[k++] = static_cast<int64_t>(s->table[p / ps]) * ps + p % ps;
    }
    if (bt_out) {
      int32_t* row = bt_out + static_cast<int64_t>(b) * bt_stride;
      std::copy(s->table.begin(), s->table.end(), row);
      std::fill(row + s->table.size(), row + bt_stride, 0);
    }
    if (seq_lens_out) seq_lens_out[b] = s->len;
  }
  return PKV_OK;
}

int pkv_plan_prefix(const int32_t* tokens, const int64_t* offsets, int32_t n_docs,
                    int32_t page_size, int32_t* order, int32_t* parent, int32_t* shared) {
  if (n_docs < 0) return fail(PKV_ERR_INVALID_ARG, "pkv_plan_prefix: n_docs < 0");
  if (page_size < 1) return fail(PKV_ERR_INVALID_ARG, "pkv_plan_prefix: page_size < 1");
  if (n_docs == 0) return PKV_OK;
  if (!offsets || !order || !parent || !shared)
    return fail(PKV_ERR_INVALID_ARG, "pkv_plan_prefix: NULL array");
  if (offsets[0] != 0) return fail(PKV_ERR_INVALID_ARG, "pkv_plan_prefix: offsets[0] != 0");
  for (int32_t d = 0; d < n_docs; ++d)
    if (offsets[d + 1] < offsets[d])
      return fail(PKV_ERR_INVALID_ARG, "pkv_plan_prefix: offsets decrease");
  if (offsets[n_docs] > 0 && !tokens) return fail(PKV_ERR_INVALID_ARG, "pkv_plan_prefix: NULL tokens");

  auto first = [&](int32_t d) { return tokens + offsets[d]; };
  auto last = [&](int32_t d) { return tokens + offsets[d + 1]; };
  auto length = [&](int32_t d) { return offsets[d + 1] - offsets[d]; };

  std::vector<int32_t> idx(n_docs);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(), [&](int32_t x, int32_t y) {
    return std::lexicographical_compare(first(x), last(x), first(y), last(y));
  });
  std::vector<int32_t> par(n_docs, -1);
  std::vector<int64_t> shr(n_docs, 0);
  for (int32_t k = 1; k < n_docs; ++k) {
    const int32_t d = idx[k];
    const int32_t q = idx[k - 1];
    const int64_t n = std::min(length(d), length(q));
    const auto mm = std::mismatch(first(d), first(d) + n, first(q));
    const int64_t lcp = mm.first - first(d);
    const int64_t computable = std::max<int64_t>(0, std::min(lcp, length(d) - 1));
    const int64_t s = page_size * (computable / page_size);
    if (s == 0) continue;
    int32_t p = q;
    while (par[p] != -1 && shr[p] >= s) p = par[p];
    par[d] = p;
    shr[d] = s;
  }
  for (int32_t d = 0; d < n_docs; ++d) {
    if (shr[d] > INT32_MAX) return fail(PKV_ERR_INVALID_ARG, "pkv_plan_prefix: shared overflows int32");
  }
  for (int32_t k = 0; k < n_docs; ++k) order[k] = idx[k];
  for (int32_t d = 0; d < n_docs; ++d) {
    parent[d] = par[d];
    shared[d] = static_cast<int32_t>(shr[d]);
  }
  return PKV_OK;
}

int pkv_validate_tables(const pkv_pool_desc* desc, const int32_t* block_tables, int32_t n_seqs,
                        int32_t bt_stride, const int32_t* seq_lens, const int32_t* cu_q,
                        int32_t max_q_per_seq) {
  if (!desc) return fail(PKV_ERR_INVALID_ARG, "pkv_validate_tables: NULL desc");
  if (n_seqs < 0 || bt_stride < 0) return fail(PKV_ERR_INVALID_ARG, "pkv_validate_tables: negative size");
  if (n_seqs > 0 && (!block_tables || !seq_lens))
    return fail(PKV_ERR_INVALID_ARG, "pkv_validate_tables: NULL array");
  const int64_t ps = desc->page_size;
  if (ps < 1) return fail(PKV_ERR_INVALID_ARG, "pkv_validate_tables: page_size < 1");
  for (int32_t b = 0; b < n_seqs; ++b) {
    const int64_t len = seq_lens[b];
    if (len < 1 || len > bt_stride * ps)
      return fail(PKV_ERR_INVALID_ARG, "pkv_validate_tables: seq_lens[" + std::to_string(b) +
                                           "] outside 1..bt_stride*page_size");
    const int64_t nblk = (len + ps - 1) / ps;
    for (int64_t i = 0; i < nblk; ++i) {
      const int32_t page = block_tables[static_cast<int64_t>(b) * bt_stride + i];
      if (page < 0 || page >= desc->num_pages)
        return fail(PKV_ERR_INVALID_ARG, "pkv_validate_tables: block table entry out of range");
    }
  }
  if (cu_q) {
    if (cu_q[0] != 0) return fail(PKV_ERR_INVALID_ARG, "pkv_validate_tables: cu_q[0] != 0");
    for (int32_t b = 0; b < n_seqs; ++b) {
      const int32_t n = cu_q[b + 1] - cu_q[b];
      if (n < 0) return fail(PKV_ERR_INVALID_ARG, "pkv_validate_tables: cu_q decreases");
      if (n > seq_lens[b])
        return fail(PKV_ERR_INVALID_ARG, "pkv_validate_tables: more queries than positions");
      if (max_q_per_seq > 0 && n > max_q_per_seq)
        return fail(PKV_ERR_INVALID_ARG, "pkv_validate_tables: n_b > max_q_per_seq");
    }
  }
  return PKV_OK;
}

}  // extern "C"
