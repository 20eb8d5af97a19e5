// Host layout builder: offsets, per-token descriptors, key spans and the
// FLOP-balanced work list of the attention launch.
//
// Layout: "Preference Packing" (technical framework) stores each prompt once,
// followed by its responses; the verl prefix_grouper_utils.py page describes
// the grouped batch by per-group prefix_len and suffix_lens (sections 1-2).
// Work list: query blocks of all groups go into one launch, ordered so the
// hardware dispatcher balances them ("PackInfer", abstract: batched requests
// organised into load-balanced execution groups, one unified kernel launch,
// thread-block execution balanced, shared-prefix requests co-located).
#include <algorithm>
#include <cmath>
#include <cstring>
#include <numeric>

#include "pg_internal.h"

namespace {

constexpr int64_t kMaxTokens = int64_t(1) << 30;   // keeps every int32 key index + tile size in range

int gcd_int(int a, int b) {
  while (b) {
    int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

// Allowed keys of one query token: the group prefix up to the token for
// prefix tokens; the whole prefix plus its own segment up to itself for
// suffix tokens.
inline int64_t keys_of(int32_t t, int32_t g0, int32_t pe, int32_t ss) {
  if (t < pe) return int64_t(t - g0 + 1);
  return int64_t(pe - g0) + int64_t(t - ss + 1);
}

// Launch order over the XCDs. Workgroups are dispatched round-robin over the
// XCDs (workgroup p runs on XCD p % 8), and each XCD has its own L2. All items
// of one cluster (same group and KV head) read the same K/V (forward) or Q/dO
// (backward), so a cluster is placed on one XCD: clusters go to the XCD with
// the least load so far, largest first (LPT over cluster costs); inside an XCD,
// clusters run largest first and the items of a cluster in the order `before`
// gives, so each XCD's queue is in LPT order and the cluster's shared rows stay
// hot in its L2. Returns item indices by launch position, -1 where an XCD
// whose queue ran out needs a padding item; trailing padding is dropped.
template <class Before>
std::vector<int32_t> xcd_launch_order(const std::vector<int64_t>& cost,
                                      const std::vector<int64_t>& cluster, int64_t ncl,
                                      Before before, std::vector<int64_t>* xcd_load_out) {
  std::vector<int64_t> cl_cost(static_cast<size_t>(ncl), 0);
  std::vector<std::vector<int32_t>> cl_items(static_cast<size_t>(ncl));
  for (size_t i = 0; i < cost.size(); ++i) {
    cl_cost[size_t(cluster[i])] += cost[i];
    cl_items[size_t(cluster[i])].push_back(int32_t(i));
  }
  std::vector<int64_t> order;
  for (int64_t c = 0; c < ncl; ++c)
    if (!cl_items[size_t(c)].empty()) order.push_back(c);
  std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t b) {
    return cl_cost[size_t(a)] > cl_cost[size_t(b)];
  });
  std::vector<int64_t> xcd_load(PG_XCDS, 0);
  std::vector<std::vector<int32_t>> xcd_queue(PG_XCDS);
  for (int64_t c : order) {
    int x = 0;
    for (int j = 1; j < PG_XCDS; ++j)
      if (xcd_load[j] < xcd_load[x]) x = j;
    xcd_load[x] += cl_cost[size_t(c)];
    std::vector<int32_t>& its = cl_items[size_t(c)];
    std::stable_sort(its.begin(), its.end(), before);
    xcd_queue[x].insert(xcd_queue[x].end(), its.begin(), its.end());
  }
  size_t rows = 0;
  for (const auto& qx : xcd_queue) rows = std::max(rows, qx.size());
  std::vector<int32_t> launch;
  launch.reserve(rows * PG_XCDS);
  for (size_t i = 0; i < rows; ++i)
    for (int x = 0; x < PG_XCDS; ++x)
      launch.push_back(i < xcd_queue[x].size() ? xcd_queue[x][i] : -1);
  while (!launch.empty() && launch.back() < 0) launch.pop_back();
  if (xcd_load_out) *xcd_load_out = xcd_load;
  return launch;
}

}  // namespace

pg_status pg_layout_build_host(pg_layout& L, int32_t num_groups, const int32_t* prefix_lens,
                               const int32_t* suffix_counts, const int32_t* suffix_lens,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               double rope_theta) {
  // ---------------------------------------------------------- validation --
  if (num_groups < 0) return pg_fail(PG_ERR_INVALID_ARG, "num_groups %d < 0", num_groups);
  if (num_groups > 0 && (!prefix_lens || !suffix_counts))
    return pg_fail(PG_ERR_INVALID_ARG, "prefix_lens / suffix_counts is NULL");
  if (num_q_heads < 1 || num_kv_heads < 1)
    return pg_fail(PG_ERR_INVALID_ARG, "head counts must be >= 1 (Hq=%d, Hkv=%d)", num_q_heads,
                   num_kv_heads);
  if (num_q_heads % num_kv_heads != 0)
    return pg_fail(PG_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", num_q_heads,
                   num_kv_heads);
  if (head_dim != 64 && head_dim != 128)
    return pg_fail(PG_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (!(rope_theta > 0.0) || !std::isfinite(rope_theta))
    return pg_fail(PG_ERR_INVALID_ARG, "rope_theta must be finite and > 0");

  int64_t nsuf = 0, total = 0;
  for (int32_t g = 0; g < num_groups; ++g) {
    if (prefix_lens[g] < 0) return pg_fail(PG_ERR_INVALID_ARG, "prefix_lens[%d] < 0", g);
    if (suffix_counts[g] < 0) return pg_fail(PG_ERR_INVALID_ARG, "suffix_counts[%d] < 0", g);
    nsuf += suffix_counts[g];
    total += prefix_lens[g];
    if (nsuf > kMaxTokens || total > kMaxTokens)
      return pg_fail(PG_ERR_INVALID_ARG, "layout too large");
  }
  if (nsuf > 0 && !suffix_lens) return pg_fail(PG_ERR_INVALID_ARG, "suffix_lens is NULL");
  for (int64_t i = 0; i < nsuf; ++i) {
    if (suffix_lens[i] < 0) return pg_fail(PG_ERR_INVALID_ARG, "suffix_lens[%lld] < 0", (long long)i);
    total += suffix_lens[i];
    if (total > kMaxTokens)
      return pg_fail(PG_ERR_INVALID_ARG, "total tokens exceed 2^30");
  }

  try {
    L.G = num_groups;
    L.Hq = num_q_heads;
    L.Hkv = num_kv_heads;
    L.d = head_dim;
    L.T = total;
    L.rope_theta = rope_theta;
    L.prefix_lens.assign(prefix_lens, prefix_lens + num_groups);
    L.suffix_counts.assign(suffix_counts, suffix_counts + num_groups);
    L.suffix_lens.assign(suffix_lens, suffix_lens + nsuf);
    L.num_segments = int32_t(num_groups + nsuf);

    // ------------------------------------------------ offsets + tokens ----
    L.group_off.assign(size_t(num_groups) + 1, 0);
    L.seg_off.clear();
    L.seg_off.reserve(size_t(L.num_segments) + 1);
    L.tok_g0.resize(size_t(total));
    L.tok_pe.resize(size_t(total));
    L.tok_ss.resize(size_t(total));
    L.tok_owner.resize(size_t(total));
    L.suffix_group.assign(size_t(nsuf), 0);
    L.max_prefix_len = 0;
    L.max_suffix_len = 0;
    L.max_position = -1;
    L.useful_pairs = 0;
    L.unpacked_pairs = 0;
    int32_t cur = 0;
    int64_t k = 0;
    for (int32_t g = 0; g < num_groups; ++g) {
      const int32_t g0 = cur, P = prefix_lens[g], pe = g0 + P;
      L.group_off[g] = g0;
      L.seg_off.push_back(g0);
      for (int32_t t = g0; t < pe; ++t) {
        L.tok_g0[t] = g0;
        L.tok_pe[t] = pe;
        L.tok_ss[t] = g0;
        L.tok_owner[t] = g;
      }
      L.max_prefix_len = std::max(L.max_prefix_len, P);
      if (P > 0) L.max_position = std::max(L.max_position, P - 1);
      const int64_t Pl = P;
      L.useful_pairs += Pl * (Pl + 1) / 2;
      cur = pe;
      if (suffix_counts[g] == 0) L.unpacked_pairs += Pl * (Pl + 1) / 2;
      for (int32_t j = 0; j < suffix_counts[g]; ++j, ++k) {
        const int32_t S = suffix_lens[k];
        L.seg_off.push_back(cur);
        for (int32_t t = cur; t < cur + S; ++t) {
          L.tok_g0[t] = g0;
          L.tok_pe[t] = pe;
          L.tok_ss[t] = cur;
          L.tok_owner[t] = int32_t(k);
        }
        L.suffix_group[size_t(k)] = g;
        L.max_suffix_len = std::max(L.max_suffix_len, S);
        if (S > 0) L.max_position = std::max(L.max_position, P + S - 1);
        const int64_t Sl = S;
        L.useful_pairs += Sl * Pl + Sl * (Sl + 1) / 2;
        L.unpacked_pairs += (Pl + Sl) * (Pl + Sl + 1) / 2;
        cur += S;
      }
    }
    L.group_off[num_groups] = cur;
    L.seg_off.push_back(cur);
    L.max_group_len = 0;
    for (int32_t g = 0; g < num_groups; ++g)
      L.max_group_len = std::max(L.max_group_len, L.group_off[g + 1] - L.group_off[g]);

    // ------------------------------------------------ rotary frequencies --
    L.inv_freq.resize(size_t(head_dim / 2));
    for (int i = 0; i < head_dim / 2; ++i)
      L.inv_freq[i] = std::pow(rope_theta, -2.0 * double(i) / double(head_dim));

    // --------------------------------------------------------- work list --
    // One item = query tokens [t0, t1) of one group x `hpw` query heads of one
    // KV head. hpw = gcd(r, 8) heads share each LDS K/V tile (GQA reuse); the
    // eight waves of an item cover hpw heads x (8 / hpw) blocks of 32 tokens.
    const int r = num_q_heads / num_kv_heads;
    const int hpw = gcd_int(r, PG_ITEM_WAVES);
    const int BT = PG_WAVE_QUERIES * PG_ITEM_WAVES / hpw;
    L.heads_per_item = hpw;
    L.block_tokens = BT;
    L.items.clear();
    L.spans.clear();
    L.max_item_cost = 0;
    std::vector<int32_t> item_group;
    k = 0;
    int32_t seg = 0;   // index of the group's prefix segment in seg_off
    for (int32_t g = 0; g < num_groups; ++g) {
      const int32_t g0 = L.group_off[g], g1 = L.group_off[g + 1];
      const int32_t pe = g0 + prefix_lens[g];
      const int32_t nseg = suffix_counts[g];
      int32_t first_suffix = 0;   // first suffix segment that may still overlap a block
      for (int32_t t0 = g0; t0 < g1; t0 += BT) {
        const int32_t t1 = std::min<int32_t>(t0 + BT, g1);
        const int32_t span0 = int32_t(L.spans.size());
        if (pe > g0) L.spans.push_back({g0, std::min(pe, t1)});
        while (first_suffix < nseg && L.seg_off[seg + 2 + first_suffix] <= t0) ++first_suffix;
        for (int32_t j = first_suffix; j < nseg; ++j) {
          const int32_t a = L.seg_off[seg + 1 + j], b = L.seg_off[seg + 2 + j];
          if (a >= t1) break;
          if (b > a && b > t0) L.spans.push_back({a, std::min(b, t1)});
        }
        const int32_t nspan = int32_t(L.spans.size()) - span0;
        int32_t ntiles = 0;
        for (int32_t s = span0; s < span0 + nspan; ++s)
          ntiles += (L.spans[size_t(s)].k1 - L.spans[size_t(s)].k0 + PG_KEY_TILE - 1) / PG_KEY_TILE;
        int64_t pairs = 0;
        for (int32_t t = t0; t < t1; ++t) pairs += keys_of(t, L.tok_g0[t], L.tok_pe[t], L.tok_ss[t]);
        for (int32_t hk = 0; hk < num_kv_heads; ++hk) {
          for (int32_t sub = 0; sub < r / hpw; ++sub) {
            pg_work_item it;
            it.t0 = t0;
            it.t1 = t1;
            it.hq0 = hk * r + sub * hpw;
            it.pe = pe;
            it.span0 = span0;
            it.nspan = nspan;
            it.ntiles = ntiles;
            it.k0 = nspan > 0 ? L.spans[size_t(span0)].k0 : 0;
            it.k1 = nspan > 0 ? L.spans[size_t(span0)].k1 : 0;
            it.reserved = 0;
            it.cost = pairs * hpw;
            L.max_item_cost = std::max(L.max_item_cost, it.cost);
            L.items.push_back(it);
            item_group.push_back(g);
          }
        }
      }
      seg += 1 + nseg;
      k += nseg;
    }
    // Launch order: see xcd_launch_order.
    std::vector<int64_t> costs(L.items.size()), clusters(L.items.size());
    for (size_t i = 0; i < L.items.size(); ++i) {
      costs[i] = L.items[i].cost;
      clusters[i] = int64_t(item_group[i]) * num_kv_heads + L.items[i].hq0 / r;
    }
    std::vector<int64_t> xcd_load;
    const std::vector<int32_t> pos = xcd_launch_order(
        costs, clusters, int64_t(num_groups) * num_kv_heads,
        [&](int32_t a, int32_t b) {
          const pg_work_item &ia = L.items[size_t(a)], &ib = L.items[size_t(b)];
          if (ia.cost != ib.cost) return ia.cost > ib.cost;
          if (ia.t0 != ib.t0) return ia.t0 < ib.t0;
          return ia.hq0 < ib.hq0;
        },
        &xcd_load);
    std::vector<pg_work_item> launch;
    launch.reserve(pos.size());
    pg_work_item empty{};
    for (int32_t i : pos) launch.push_back(i >= 0 ? L.items[size_t(i)] : empty);
    L.items.swap(launch);
    L.xcd_load = xcd_load;


    // Backward work list (dK, dV): blocks of PG_KV_BLOCK keys of one KV head
    // that never cross a segment. The queries that read key j form one
    // contiguous range [j, qend): a prompt key is read by every later token of
    // its group (the rest of the prompt and all responses), a response key by
    // the rest of its own response. qend is the group end or the response end.
    std::vector<pg_kv_item> kv;
    std::vector<int64_t> kv_cluster;
    {
      int32_t sg = 0;   // index of the group's prefix segment in seg_off
      for (int32_t g = 0; g < num_groups; ++g) {
        const int32_t nseg = suffix_counts[g];
        const int32_t gend = L.group_off[g + 1];
        for (int32_t j = 0; j <= nseg; ++j) {
          const int32_t a = L.seg_off[sg + j], b = L.seg_off[sg + j + 1];
          const int32_t qend = j == 0 ? gend : b;
          for (int32_t k0 = a; k0 < b; k0 += PG_KV_BLOCK) {
            const int32_t k1 = std::min<int32_t>(k0 + PG_KV_BLOCK, b);
            const int64_t n = k1 - k0;
            // sum over keys of the queries reading them, times the r query heads
            const int64_t pairs = n * int64_t(qend) - (int64_t(k0) + k1 - 1) * n / 2;
            for (int32_t hk = 0; hk < num_kv_heads; ++hk) {
              kv.push_back(pg_kv_item{k0, k1, hk, qend, pairs * r});
              kv_cluster.push_back(int64_t(g) * num_kv_heads + hk);
            }
          }
        }
        sg += 1 + nseg;
      }
      std::vector<int64_t> kv_cost(kv.size());
      for (size_t i = 0; i < kv.size(); ++i) kv_cost[i] = kv[i].cost;
      const std::vector<int32_t> kpos = xcd_launch_order(
          kv_cost, kv_cluster, int64_t(num_groups) * num_kv_heads,
          [&](int32_t a, int32_t b) {
            const pg_kv_item &ia = kv[size_t(a)], &ib = kv[size_t(b)];
            if (ia.cost != ib.cost) return ia.cost > ib.cost;
            if (ia.k0 != ib.k0) return ia.k0 < ib.k0;
            return ia.hk < ib.hk;
          },
          nullptr);
      L.kv_items.clear();
      L.kv_items.reserve(kpos.size());
      for (int32_t i : kpos)
        L.kv_items.push_back(i >= 0 ? kv[size_t(i)] : pg_kv_item{0, 0, 0, 0, 0});
    }

    // Decode work list: every segment of a group that has responses, split
    // into balanced chunks (multiples of 32 rows) per KV head and per block of
    // at most PG_DEC_ROWS query rows. The chunk length aims at about
    // PG_DEC_TARGET items for the whole step (several waves per CU on small
    // batches), between 64 and PG_DEC_CHUNK rows. A prompt chunk
    // serves the rows of all the group's responses, so each prompt row is read
    // once per step (plus once per extra row block when n * r > 32); a
    // response chunk serves its own r rows. Each chunk (with its row blocks) is
    // one cluster for the XCD placement: its row blocks re-read the same rows.
    {
      const int64_t N = int64_t(L.suffix_lens.size());
      std::vector<pg_dec_item> dec;
      std::vector<int64_t> dcost, dcluster;
      std::vector<std::vector<int32_t>> refs(size_t(N * num_kv_heads));
      int64_t ncl = 0;
      int64_t dec_rows = 0;   // cache rows a step may read, summed over KV heads
      {
        int32_t sg = 0;
        for (int32_t g = 0; g < num_groups; ++g) {
          const int32_t n = suffix_counts[g];
          if (n > 0) dec_rows += int64_t(L.seg_off[sg + 1 + n] - L.seg_off[sg]) * num_kv_heads;
          sg += 1 + n;
        }
      }
      const int64_t per_item = (dec_rows + PG_DEC_TARGET - 1) / PG_DEC_TARGET;
      const int32_t chunk =
          int32_t(std::min<int64_t>(PG_DEC_CHUNK, std::max<int64_t>(64, (per_item + 31) / 32 * 32)));
      L.dec_chunk = chunk;
      // A prompt much longer than a chunk is cut into fewer, longer pieces:
      // every piece of it already has enough rows to stream, and each extra
      // piece adds a partial result to write and merge and a work item to
      // start (a 16K-row prompt: 14 % faster steps with 1024-row pieces).
      auto chunked = [&](int32_t a, int32_t b, int32_t resp, int32_t rows0, int32_t nrows) {
        if (b <= a || nrows <= 0) return;
        const int32_t len = b - a;
        const int32_t ck = (resp < 0 && len > PG_DEC_LONG_PROMPT) ? PG_DEC_CHUNK_LONG : chunk;
        const int32_t nch = (len + ck - 1) / ck;
        const int32_t step = ((len + nch - 1) / nch + 31) / 32 * 32;
        for (int32_t k0 = a; k0 < b; k0 += step) {
          const int32_t k1 = std::min(b, k0 + step);
          for (int32_t hk = 0; hk < num_kv_heads; ++hk) {
            const int64_t cl = ncl++;
            for (int32_t b0 = 0; b0 < nrows; b0 += PG_DEC_ROWS) {
              const int32_t row0 = rows0 + b0, nrow = std::min(PG_DEC_ROWS, nrows - b0);
              const int32_t idx = int32_t(dec.size());
              dec.push_back(pg_dec_item{k0, k1, hk, resp, a, b, row0, nrow});
              dcost.push_back(int64_t(k1 - k0) + 64);   // rows read, plus a fixed start-up
              dcluster.push_back(cl);
              for (int32_t k = row0 / r; k <= (row0 + nrow - 1) / r; ++k)
                refs[size_t(int64_t(k) * num_kv_heads + hk)].push_back(idx);
            }
          }
        }
      };
      int32_t sg = 0, kresp = 0;
      for (int32_t g = 0; g < num_groups; ++g) {
        const int32_t n = suffix_counts[g];
        if (n > 0) chunked(L.seg_off[sg], L.seg_off[sg + 1], -1, kresp * r, n * r);
        for (int32_t j = 0; j < n; ++j)
          chunked(L.seg_off[sg + 1 + j], L.seg_off[sg + 2 + j], kresp + j, (kresp + j) * r, r);
        sg += 1 + n;
        kresp += n;
      }
      const std::vector<int32_t> dpos = xcd_launch_order(
          dcost, dcluster, ncl,
          [&](int32_t a, int32_t b) {
            const pg_dec_item &ia = dec[size_t(a)], &ib = dec[size_t(b)];
            if (ia.row0 != ib.row0) return ia.row0 < ib.row0;
            return ia.k0 < ib.k0;
          },
          nullptr);
      std::vector<int32_t> launch_of(dec.size(), -1);
      L.dec_items.clear();
      L.dec_items.reserve(dpos.size());
      for (size_t p = 0; p < dpos.size(); ++p) {
        const int32_t i = dpos[p];
        if (i >= 0) launch_of[size_t(i)] = int32_t(p);
        L.dec_items.push_back(i >= 0 ? dec[size_t(i)] : pg_dec_item{0, 0, 0, -1, 0, 0, 0, 0});
      }
      L.dec_ref_off.assign(size_t(N * num_kv_heads + 1), 0);
      L.dec_refs.clear();
      for (size_t u = 0; u < refs.size(); ++u) {
        for (int32_t i : refs[u]) L.dec_refs.push_back(launch_of[size_t(i)]);
        L.dec_ref_off[u + 1] = int32_t(L.dec_refs.size());
      }
    }
  } catch (const std::bad_alloc&) {
    return pg_fail(PG_ERR_OOM, "host allocation failed");
  }
  return PG_OK;
}
