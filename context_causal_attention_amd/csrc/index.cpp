// Host index builder: the zigzag deal of a sequence (or of packed documents)
// over 2*cp chunks, the ring source of each step and exact allowed-pair counts.
//
// Context parallelism shards the sequence dimension across ranks (Accelerate
// concept guide, "Technical details"); the length must be a multiple of 2*cp
// (hierarchical-CP skill page, "Required constraints"), and rank r holds chunk r
// and chunk 2*cp-1-r, so every rank gets the same number of causal pairs.
#include <algorithm>
#include <climits>
#include <vector>

#include "internal.h"

using cpattn::fail;

namespace {

int check_cp_rank(int32_t cp, int32_t rank) {
  if (cp < 1) return fail(CP_EINVAL, "cp must be >= 1 (got %d)", cp);
  if (rank < 0 || rank >= cp) return fail(CP_EINVAL, "rank %d outside [0, %d)", rank, cp);
  return CP_OK;
}

int check_seq(int64_t S, int32_t cp) {
  if (S < 0 || S > INT32_MAX) return fail(CP_EINVAL, "sequence length %lld outside [0, INT32_MAX]", (long long)S);
  if (S % (2 * (int64_t)cp) != 0)
    return fail(CP_ESHAPE, "sequence length %lld is not a multiple of 2*cp = %lld", (long long)S,
                2 * (long long)cp);
  return CP_OK;
}

void deal(int64_t base, int64_t len, int32_t cp, int32_t rank, int32_t* out) {
  const int64_t c = len / (2 * (int64_t)cp);
  const int64_t a = rank, b = 2 * (int64_t)cp - 1 - rank;
  for (int64_t i = 0; i < c; ++i) out[i] = (int32_t)(base + a * c + i);
  for (int64_t i = 0; i < c; ++i) out[c + i] = (int32_t)(base + b * c + i);
}

// Causal pairs of rows [a, b) of a document that starts at s.
int64_t piece_work(int64_t s, int64_t a, int64_t b) { return (b - a) * ((a - s + 1) + (b - s)) / 2; }

// Whole-document placement over all ranks (rule in cpattn.h); writes rank's
// positions, ascending.
void whole_doc(const int32_t* cu, int32_t n_docs, int32_t cp, int32_t rank, int32_t* out) {
  const int64_t S = cu[n_docs];
  std::vector<int64_t> room(cp, S / cp), load(cp, 0);
  std::vector<std::pair<int64_t, int64_t>> mine;  // pieces [a, b) of this rank
  std::vector<int32_t> order(n_docs);
  for (int32_t i = 0; i < n_docs; ++i) order[i] = i;
  std::sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
    const int64_t lx = (int64_t)cu[x + 1] - cu[x], ly = (int64_t)cu[y + 1] - cu[y];
    return lx != ly ? lx > ly : x < y;
  });
  auto place = [&](int32_t r, int64_t s, int64_t a, int64_t b) {
    room[r] -= b - a;
    load[r] += piece_work(s, a, b);
    if (r == rank) mine.emplace_back(a, b);
  };
  for (int32_t i : order) {
    const int64_t s = cu[i], e = cu[i + 1];
    if (e == s) continue;
    int32_t best = -1;
    for (int32_t r = 0; r < cp; ++r)
      if (room[r] >= e - s && (best < 0 || load[r] < load[best])) best = r;
    if (best >= 0) {
      place(best, s, s, e);
      continue;
    }
    for (int64_t a = s; a < e;) {
      int32_t r = 0;
      for (int32_t q = 1; q < cp; ++q)
        if (room[q] > room[r]) r = q;
      const int64_t m = std::min(room[r], e - a);
      place(r, s, a, a + m);
      a += m;
    }
  }
  std::sort(mine.begin(), mine.end());
  int64_t k = 0;
  for (const auto& pc : mine)
    for (int64_t p = pc.first; p < pc.second; ++p) out[k++] = (int32_t)p;
}

}  // namespace

extern "C" int cp_shard_zigzag(int64_t S, int32_t cp, int32_t rank, int32_t* pos_out) {
  cpattn::clear_error();
  if (!pos_out) return fail(CP_EINVAL, "pos_out is null");
  if (int rc = check_cp_rank(cp, rank)) return rc;
  if (int rc = check_seq(S, cp)) return rc;
  deal(0, S, cp, rank, pos_out);
  return CP_OK;
}

extern "C" int cp_unshard_zigzag(int64_t S, int32_t cp, int32_t* perm_out) {
  cpattn::clear_error();
  if (!perm_out) return fail(CP_EINVAL, "perm_out is null");
  if (cp < 1) return fail(CP_EINVAL, "cp must be >= 1 (got %d)", cp);
  if (int rc = check_seq(S, cp)) return rc;
  const int64_t per = S / cp;
  for (int32_t r = 0; r < cp; ++r) deal(0, S, cp, r, perm_out + r * per);
  return CP_OK;
}

extern "C" int cp_varlen_index(const int32_t* cu, int32_t n_docs, int32_t cp, int32_t rank,
                               int32_t mode, int32_t* pos_out, int32_t* lo_out) {
  cpattn::clear_error();
  if (!cu || !pos_out || !lo_out) return fail(CP_EINVAL, "null pointer argument");
  if (n_docs < 1) return fail(CP_EINVAL, "n_docs must be >= 1 (got %d)", n_docs);
  if (int rc = check_cp_rank(cp, rank)) return rc;
  if (mode != CP_STREAM && mode != CP_PER_DOC && mode != CP_WHOLE_DOC)
    return fail(CP_EINVAL, "unknown shard mode %d", mode);
  if (cu[0] != 0) return fail(CP_ESHAPE, "cu_seqlens[0] must be 0 (got %d)", cu[0]);
  for (int32_t i = 0; i < n_docs; ++i)
    if (cu[i + 1] < cu[i]) return fail(CP_ESHAPE, "cu_seqlens decreases at index %d", i);
  const int64_t S = cu[n_docs];
  if (int rc = check_seq(S, cp)) return rc;
  const int64_t per = S / cp;
  if (mode == CP_STREAM) {
    deal(0, S, cp, rank, pos_out);
  } else if (mode == CP_WHOLE_DOC) {
    whole_doc(cu, n_docs, cp, rank, pos_out);
  } else {
    int64_t off = 0;
    for (int32_t i = 0; i < n_docs; ++i) {
      const int64_t len = (int64_t)cu[i + 1] - cu[i];
      if (len % (2 * (int64_t)cp) != 0)
        return fail(CP_ESHAPE, "document %d has length %lld, not a multiple of 2*cp = %lld", i,
                    (long long)len, 2 * (long long)cp);
      deal(cu[i], len, cp, rank, pos_out + off);
      off += len / cp;
    }
    if (off != per) return fail(CP_ESHAPE, "internal: per-document deal produced %lld rows", (long long)off);
  }
  // Start of the document holding each position: the last boundary <= p.
  for (int64_t i = 0; i < per; ++i) {
    const int32_t p = pos_out[i];
    const int32_t* it = std::upper_bound(cu, cu + n_docs + 1, p);
    lo_out[i] = *(it - 1);
  }
  return CP_OK;
}

extern "C" int cp_ring_source(int32_t cp, int32_t rank, int32_t step) {
  cpattn::clear_error();
  if (check_cp_rank(cp, rank) != CP_OK) return -1;
  if (step < 0 || step >= cp) {
    fail(CP_EINVAL, "step %d outside [0, %d)", step, cp);
    return -1;
  }
  return (int32_t)(((int64_t)rank - step + cp) % cp);
}

extern "C" int64_t cp_pairs(const int32_t* q_pos, const int32_t* q_lo, int64_t nq, const int32_t* k_pos,
                            int64_t nk) {
  cpattn::clear_error();
  if (nq < 0 || nk < 0) {
    fail(CP_EINVAL, "negative length");
    return -1;
  }
  if ((nq > 0 && !q_pos) || (nk > 0 && !k_pos)) {
    fail(CP_EINVAL, "null array with nonzero length");
    return -1;
  }
  std::vector<int32_t> ks(k_pos, k_pos + nk);
  std::sort(ks.begin(), ks.end());
  int64_t total = 0;
  for (int64_t i = 0; i < nq; ++i) {
    const int32_t lo = q_lo ? q_lo[i] : 0;
    const int32_t hi = q_pos[i];
    if (hi < lo) continue;
    auto a = std::lower_bound(ks.begin(), ks.end(), lo);
    auto b = std::upper_bound(ks.begin(), ks.end(), hi);
    total += (int64_t)(b - a);
  }
  return total;
}
