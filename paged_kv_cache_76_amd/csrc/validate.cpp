// Index-precondition checks over host copies of the index arrays.
//
// The kernels take slots, block ids and lengths as preconditions: they skip
// ids outside the pool (so memory stays in bounds) but a duplicated copy
// destination, a destination that is also a source, or two tokens written to
// one slot make the result depend on the order in which workgroups run.
// These checks state the preconditions exactly:
// * copy-on-write copies ("vLLM / PagedAttention", awesome.papernotes.org,
//   key design 3: the writer of a shared block copies it into a newly
//   allocated block; key design 5: the copies of a step are batched) go to
//   distinct, freshly allocated blocks, never to a block another pair reads;
// * a step's new tokens ([P2] "PagedAttention 原理": each token's K/V go to
//   the slot the block table maps it to) occupy distinct slots;
// * every block a table maps for a sequence's context is a block of the pool;
// * an appending decode's new tokens go to distinct slots that no other
//   sequence of the batch reads (the copy-on-write rule of key design 3 makes
//   the block that receives a token private to its sequence).
// They run on the host over plain arrays, so they never touch a device.
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pa_internal.h"

namespace pa {

pa_status check_fail(pa_status st, const char* fmt, ...);

}  // namespace pa

extern "C" {

pa_status pa_check_copy_pairs(const int64_t* pairs, int32_t n, int32_t src_blocks, int32_t dst_blocks,
                              int32_t same_pool) {
  const char* fn = "pa_check_copy_pairs";
  if (n < 0 || src_blocks < 0 || dst_blocks < 0) return pa::check_fail(PA_ERR_INVALID_ARG, "%s: negative size", fn);
  if (n == 0) return PA_OK;
  if (!pairs) return pa::check_fail(PA_ERR_INVALID_ARG, "%s: pairs is NULL", fn);
  std::unordered_set<int64_t> dsts;
  dsts.reserve((size_t)n * 2);
  for (int32_t i = 0; i < n; ++i) {
    const int64_t s = pairs[2 * i], d = pairs[2 * i + 1];
    if (s < 0 || s >= src_blocks)
      return pa::check_fail(PA_ERR_INVALID_ARG, "%s: pair %d: source block %lld outside [0, %d)", fn, i,
                            (long long)s, src_blocks);
    if (d < 0 || d >= dst_blocks)
      return pa::check_fail(PA_ERR_INVALID_ARG, "%s: pair %d: destination block %lld outside [0, %d)", fn, i,
                            (long long)d, dst_blocks);
    if (!dsts.insert(d).second)
      return pa::check_fail(PA_ERR_INVALID_ARG, "%s: pair %d: destination block %lld appears twice", fn, i,
                            (long long)d);
  }
  if (same_pool) {
    for (int32_t i = 0; i < n; ++i) {
      if (dsts.count(pairs[2 * i]))
        return pa::check_fail(PA_ERR_INVALID_ARG, "%s: pair %d: source block %lld is also a destination", fn, i,
                              (long long)pairs[2 * i]);
    }
  }
  return PA_OK;
}

pa_status pa_check_slot_mapping(const int64_t* slot_mapping, int32_t T, int64_t num_slots) {
  const char* fn = "pa_check_slot_mapping";
  if (T < 0 || num_slots < 0) return pa::check_fail(PA_ERR_INVALID_ARG, "%s: negative size", fn);
  if (T == 0) return PA_OK;
  if (!slot_mapping) return pa::check_fail(PA_ERR_INVALID_ARG, "%s: slot_mapping is NULL", fn);
  std::vector<int64_t> used;
  used.reserve(T);
  for (int32_t t = 0; t < T; ++t) {
    const int64_t slot = slot_mapping[t];
    if (slot < 0) continue;  // a skipped token
    if (slot >= num_slots)
      return pa::check_fail(PA_ERR_INVALID_ARG, "%s: token %d: slot %lld outside [0, %lld)", fn, t,
                            (long long)slot, (long long)num_slots);
    used.push_back(slot);
  }
  std::sort(used.begin(), used.end());
  const auto dup = std::adjacent_find(used.begin(), used.end());
  if (dup != used.end())
    return pa::check_fail(PA_ERR_INVALID_ARG, "%s: slot %lld is written by two tokens", fn, (long long)*dup);
  return PA_OK;
}

pa_status pa_check_block_tables(const int32_t* block_tables, int32_t S, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t max_context_len, int32_t block_size,
                                int32_t num_blocks) {
  const char* fn = "pa_check_block_tables";
  if (S < 0 || max_blocks_per_seq < 0 || block_size < 1 || num_blocks < 0)
    return pa::check_fail(PA_ERR_INVALID_ARG, "%s: bad size", fn);
  if (S == 0) return PA_OK;
  if (!block_tables || !context_lens) return pa::check_fail(PA_ERR_INVALID_ARG, "%s: NULL array", fn);
  for (int32_t s = 0; s < S; ++s) {
    const int32_t L = context_lens[s];
    if (L < 1 || L > max_context_len)
      return pa::check_fail(PA_ERR_INVALID_ARG, "%s: sequence %d: context length %d outside [1, %d]", fn, s, L,
                            max_context_len);
    const int64_t nblk = ((int64_t)L + block_size - 1) / block_size;
    if (nblk > max_blocks_per_seq)
      return pa::check_fail(PA_ERR_INVALID_ARG, "%s: sequence %d: %lld blocks exceed the table row of %d", fn, s,
                            (long long)nblk, max_blocks_per_seq);
    const int32_t* row = block_tables + (int64_t)s * max_blocks_per_seq;
    for (int64_t j = 0; j < nblk; ++j) {
      if (row[j] < 0 || row[j] >= num_blocks)
        return pa::check_fail(PA_ERR_INVALID_ARG, "%s: sequence %d: logical block %lld maps to %d outside [0, %d)",
                              fn, s, (long long)j, row[j], num_blocks);
    }
  }
  return PA_OK;
}

pa_status pa_check_append_slots(const int32_t* block_tables, int32_t S, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t block_size, const int32_t* cow_src,
                                int32_t num_blocks) {
  const char* fn = "pa_check_append_slots";
  if (S < 0 || max_blocks_per_seq < 0 || block_size < 1)
    return pa::check_fail(PA_ERR_INVALID_ARG, "%s: bad size", fn);
  if (S == 0) return PA_OK;
  if (!block_tables || !context_lens) return pa::check_fail(PA_ERR_INVALID_ARG, "%s: NULL array", fn);
  // (physical block, offset) of each row's newest token; rows with no
  // token are the caller's error, reported by pa_check_block_tables
  struct Slot {
    int32_t block, off, row;
  };
  std::vector<Slot> fresh;
  fresh.reserve((size_t)S);
  for (int32_t s = 0; s < S; ++s) {
    const int32_t L = context_lens[s];
    if (L < 1 || (int64_t)(L - 1) / block_size >= max_blocks_per_seq)
      return pa::check_fail(PA_ERR_INVALID_ARG, "%s: sequence %d: context length %d outside its table row", fn, s,
                            L);
    const int32_t pos = L - 1;
    fresh.push_back({block_tables[(int64_t)s * max_blocks_per_seq + pos / block_size], pos % block_size, s});
  }
  std::sort(fresh.begin(), fresh.end(), [](const Slot& x, const Slot& y) {
    return x.block != y.block ? x.block < y.block : x.off < y.off;
  });
  for (size_t i = 1; i < fresh.size(); ++i) {
    if (fresh[i].block == fresh[i - 1].block && fresh[i].off == fresh[i - 1].off)
      return pa::check_fail(PA_ERR_INVALID_ARG, "%s: sequences %d and %d append to the same slot (block %d, offset %d)",
                            fn, fresh[i - 1].row, fresh[i].row, fresh[i].block, fresh[i].off);
  }
  // every other row's reads of a block that receives a new token: offsets
  // below its own count of tokens in that block
  std::unordered_map<int32_t, std::pair<size_t, size_t>> by_block;  // block -> range in fresh
  for (size_t i = 0; i < fresh.size();) {
    size_t j = i;
    while (j < fresh.size() && fresh[j].block == fresh[i].block) ++j;
    by_block[fresh[i].block] = {i, j};
    i = j;
  }
  for (int32_t s = 0; s < S; ++s) {
    const int32_t L = context_lens[s];
    const int64_t nblk = ((int64_t)L + block_size - 1) / block_size;
    const int32_t* row = block_tables + (int64_t)s * max_blocks_per_seq;
    for (int64_t j = 0; j < nblk; ++j) {
      const auto it = by_block.find(row[j]);
      if (it == by_block.end()) continue;
      const int64_t count = std::min<int64_t>(block_size, L - j * block_size);  // tokens of s in this block
      for (size_t k = it->second.first; k < it->second.second; ++k) {
        if (fresh[k].row != s && fresh[k].off < count)
          return pa::check_fail(PA_ERR_INVALID_ARG,
                                "%s: sequence %d appends to block %d offset %d, which sequence %d reads", fn,
                                fresh[k].row, fresh[k].block, fresh[k].off, s);
      }
    }
  }
  if (!cow_src) return PA_OK;
  // Copy-on-write folded in: row s's newest-token block d first receives a
  // copy of block c = cow_src[s] (the slots before the newest token's, which
  // its own write fills; the slots after it hold no token).  d must belong to
  // s alone, and no write of the call may land in a slot of c that the copy
  // reads.
  std::unordered_map<int32_t, int32_t> owner;  // newest-token block -> row, for rows that copy
  for (int32_t s = 0; s < S; ++s) {
    const int32_t c = cow_src[s];
    if (c < 0) continue;
    const int32_t pos = context_lens[s] - 1;
    const int32_t d = block_tables[(int64_t)s * max_blocks_per_seq + pos / block_size];
    if (c >= num_blocks)
      return pa::check_fail(PA_ERR_INVALID_ARG, "%s: sequence %d: copy source %d outside [0, %d)", fn, s, c,
                            num_blocks);
    if (c == d) return pa::check_fail(PA_ERR_INVALID_ARG, "%s: sequence %d copies block %d onto itself", fn, s, c);
    owner[d] = s;
  }
  for (int32_t s = 0; s < S; ++s) {  // nobody else maps a block that receives a copy
    const int64_t nblk = ((int64_t)context_lens[s] + block_size - 1) / block_size;
    const int32_t* row = block_tables + (int64_t)s * max_blocks_per_seq;
    for (int64_t j = 0; j < nblk; ++j) {
      const auto it = owner.find(row[j]);
      if (it != owner.end() && it->second != s)
        return pa::check_fail(PA_ERR_INVALID_ARG, "%s: block %d receives sequence %d's copy but sequence %d maps it",
                              fn, row[j], it->second, s);
    }
  }
  for (const Slot& f : fresh) {  // every write of the call against every copy's source
    for (int32_t s = 0; s < S; ++s) {
      if (cow_src[s] != f.block) continue;
      if (f.off < (context_lens[s] - 1) % block_size)
        return pa::check_fail(PA_ERR_INVALID_ARG,
                              "%s: sequence %d writes block %d offset %d, which sequence %d's copy reads", fn, f.row,
                              f.block, f.off, s);
    }
  }
  for (int32_t s = 0; s < S; ++s) {  // a copy's source is no other copy's destination
    if (cow_src[s] >= 0 && owner.count(cow_src[s]))
      return pa::check_fail(PA_ERR_INVALID_ARG, "%s: sequence %d copies from block %d, which receives a copy", fn, s,
                            cow_src[s]);
  }
  return PA_OK;
}

pa_status pa_check_prefill_rows(const int32_t* cu_q_lens, const int32_t* context_lens, int32_t S,
                                int32_t max_q_len) {
  const char* fn = "pa_check_prefill_rows";
  if (S < 0) return pa::check_fail(PA_ERR_INVALID_ARG, "%s: negative size", fn);
  if (S == 0) return PA_OK;
  if (!cu_q_lens || !context_lens) return pa::check_fail(PA_ERR_INVALID_ARG, "%s: NULL array", fn);
  if (cu_q_lens[0] != 0) return pa::check_fail(PA_ERR_INVALID_ARG, "%s: cu_q_lens[0] = %d, not 0", fn, cu_q_lens[0]);
  for (int32_t s = 0; s < S; ++s) {
    const int64_t q = (int64_t)cu_q_lens[s + 1] - cu_q_lens[s];
    if (q < 0 || q > max_q_len)
      return pa::check_fail(PA_ERR_INVALID_ARG, "%s: sequence %d: %lld queries outside [0, %d]", fn, s,
                            (long long)q, max_q_len);
    if (q > context_lens[s])
      return pa::check_fail(PA_ERR_INVALID_ARG, "%s: sequence %d: %lld queries but a context of %d", fn, s,
                            (long long)q, context_lens[s]);
  }
  return PA_OK;
}

}  // extern "C"
