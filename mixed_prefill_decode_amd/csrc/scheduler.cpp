// SLO-aware scheduling around the waterfill dispatcher (host only).
//
// ConfluxServe §6.4 and Algorithm 1: one scheduling iteration takes the
// dispatcher's reference budget B0 (no candidate, nothing selected), admits
// the pending prefills by Moore-Hodgson under B0 (App. G, Algorithm 4), then
// walks the admitted requests in EDF order and the removed ones in SJF order,
// asking the dispatcher (App. E, Algorithm 2) for each one's TBT-safe chunk.
// A zero chunk ends the iteration.  A chunk that finishes its prompt needs a
// decode host from the dual-mode placement (§6.3, App. F, Algorithm 3): worst
// fit on the smallest aggregate decode context while a feasible rank is below
// the KV-utilization threshold, best fit on the highest utilization once none
// is; a chunk with no feasible host is dropped and ends the iteration.
//
// Readings where the pages leave a detail open:
//   - K_i = max(0, floor((d_i - t) / tau)) * B0: whole iterations left before the
//     deadline times the per-iteration budget (the floor brackets of App. G),
//     with the iteration count clamped at 2^40.
//   - Ties: EDF by (deadline, index); the heap removes the largest m, the later
//     in EDF order among equal m; SJF by (m, EDF position); placement ties go to
//     the lowest rank index.
//   - A placed request needs c + m KV tokens and adds one decode token and
//     c + m of context to its host's tentative state; headroom h is a count of
//     KV tokens that must stay free on the host after the placement;
//     utilization is kv_used / kv_capacity before the placement.
//   - The dispatcher sees the current decode state (the new decodes start in
//     the next iteration); only placement sees the tentative state.
//   - B0's level search is bounded by max_r n_d^r + sum_i m_i: a budget beyond
//     all pending work changes no admission decision.
#pragma clang fp contract(off)

#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <numeric>
#include <queue>
#include <vector>

#include "../../include/xp.h"

namespace xp {
xp_status fail(xp_status code, const char* fmt, ...);
}
using xp::fail;

namespace {

constexpr double kMaxIterations = 1099511627776.0;  // 2^40

xp_status check_queue(const xp_prefill_queue* q, const char* who) {
  if (!q || q->n < 0) return fail(XP_EINVAL, "%s: null or negative queue", who);
  if (q->n > 0 && (!q->m_remaining || !q->c_processed || !q->deadline))
    return fail(XP_EINVAL, "%s: null queue array", who);
  for (int i = 0; i < q->n; ++i) {
    if (q->m_remaining[i] < 1) return fail(XP_EINVAL, "%s: m_remaining[%d] = %d", who, i, q->m_remaining[i]);
    if (q->c_processed[i] < 0) return fail(XP_EINVAL, "%s: c_processed[%d] < 0", who, i);
    if (!isfinite(q->deadline[i])) return fail(XP_EINVAL, "%s: deadline[%d] not finite", who, i);
  }
  return XP_OK;
}

xp_status check_state(const xp_decode_state* s, const char* who) {
  if (!s || s->n_ranks < 1) return fail(XP_EINVAL, "%s: null state or n_ranks < 1", who);
  if (!s->n_decode_tokens || !s->decode_ctx_sum || !s->kv_used || !s->kv_capacity)
    return fail(XP_EINVAL, "%s: null state array", who);
  for (int r = 0; r < s->n_ranks; ++r) {
    if (s->n_decode_tokens[r] < 0 || s->decode_ctx_sum[r] < 0 || s->kv_used[r] < 0)
      return fail(XP_EINVAL, "%s: negative load on rank %d", who, r);
    if (s->kv_capacity[r] <= 0) return fail(XP_EINVAL, "%s: kv_capacity[%d] <= 0", who, r);
  }
  return XP_OK;
}

// EDF order, then Moore-Hodgson removals; returns the number admitted.
int admit(const xp_prefill_queue& q, int64_t b0, double now, double tau, int32_t* order) {
  const int R = q.n;
  std::vector<int> edf(R);
  std::iota(edf.begin(), edf.end(), 0);
  std::sort(edf.begin(), edf.end(), [&](int a, int b) {
    return q.deadline[a] != q.deadline[b] ? q.deadline[a] < q.deadline[b] : a < b;
  });
  std::vector<int> pos(R);
  for (int k = 0; k < R; ++k) pos[edf[k]] = k;
  // max-heap on (m, EDF position)
  auto lower = [&](int a, int b) {
    return q.m_remaining[a] != q.m_remaining[b] ? q.m_remaining[a] < q.m_remaining[b] : pos[a] < pos[b];
  };
  std::priority_queue<int, std::vector<int>, decltype(lower)> heap(lower);
  std::vector<char> removed(R, 0);
  __int128 total = 0;
  for (int k = 0; k < R; ++k) {
    const int i = edf[k];
    total += q.m_remaining[i];
    heap.push(i);
    double iters = floor((q.deadline[i] - now) / tau);
    iters = iters < 0.0 ? 0.0 : std::min(iters, kMaxIterations);
    const __int128 cap = __int128(int64_t(iters)) * b0;
    if (total > cap) {
      const int j = heap.top();
      heap.pop();
      total -= q.m_remaining[j];
      removed[j] = 1;
    }
  }
  int n = 0;
  for (int k = 0; k < R; ++k)
    if (!removed[edf[k]]) order[n++] = edf[k];
  const int n_adm = n;
  std::vector<int> rej;
  for (int k = 0; k < R; ++k)
    if (removed[edf[k]]) rej.push_back(edf[k]);
  std::stable_sort(rej.begin(), rej.end(), [&](int a, int b) { return q.m_remaining[a] < q.m_remaining[b]; });
  for (int i : rej) order[n++] = i;
  return n_adm;
}

int place(int N, const int64_t* ctx_sum, const int64_t* used, const int64_t* cap, int64_t need, double eta,
          int64_t headroom) {
  int worst = -1, best = -1;
  for (int r = 0; r < N; ++r) {
    if (__int128(used[r]) + need + headroom > cap[r]) continue;  // not feasible
    if (double(used[r]) / double(cap[r]) < eta) {
      if (worst < 0 || ctx_sum[r] < ctx_sum[worst]) worst = r;
    }
    // highest utilization: used[r]/cap[r] > used[best]/cap[best], exactly
    if (best < 0 || __int128(used[r]) * cap[best] > __int128(used[best]) * cap[r]) best = r;
  }
  return worst >= 0 ? worst : best;
}

}  // namespace

extern "C" {

xp_status xp_admission(const xp_prefill_queue* queue, int64_t ref_budget, double now, double tbt_slo,
                       int32_t* order, int32_t* n_admitted) {
  xp_status st = check_queue(queue, "xp_admission");
  if (st) return st;
  if (!n_admitted || (queue->n > 0 && !order)) return fail(XP_EINVAL, "xp_admission: null output");
  if (!(tbt_slo > 0.0) || !isfinite(now)) return fail(XP_EINVAL, "xp_admission: tbt_slo / now");
  if (ref_budget < 0) return fail(XP_EINVAL, "xp_admission: ref_budget < 0");
  *n_admitted = admit(*queue, ref_budget, now, tbt_slo, order);
  return XP_OK;
}

xp_status xp_decode_placement(const xp_decode_state* state, int64_t kv_need, double kv_util_threshold,
                              int64_t kv_headroom, int32_t* rank) {
  xp_status st = check_state(state, "xp_decode_placement");
  if (st) return st;
  if (!rank) return fail(XP_EINVAL, "xp_decode_placement: null output");
  if (kv_need < 0 || kv_headroom < 0) return fail(XP_EINVAL, "xp_decode_placement: kv_need / headroom < 0");
  *rank = place(state->n_ranks, state->decode_ctx_sum, state->kv_used, state->kv_capacity, kv_need, kv_util_threshold,
                kv_headroom);
  return XP_OK;
}

xp_status xp_schedule(const xp_decode_state* state, const xp_prefill_queue* queue, const xp_sched_params* p,
                      xp_schedule_out* out) {
  xp_status st;
  if ((st = check_state(state, "xp_schedule"))) return st;
  if ((st = check_queue(queue, "xp_schedule"))) return st;
  if (!p || !p->model || !out) return fail(XP_EINVAL, "xp_schedule: null params / model / out");
  if (!(p->tbt_slo > 0.0) || !isfinite(p->now) || p->quantum < 1 || p->kv_headroom < 0)
    return fail(XP_EINVAL, "xp_schedule: tbt_slo / now / quantum / headroom");
  const int N = state->n_ranks, R = queue->n;
  if (!out->prefill_assign || (R > 0 && (!out->order || !out->chunk_len || !out->decode_rank)))
    return fail(XP_EINVAL, "xp_schedule: null output array");

  int64_t max_load = 0, pending = 0;
  for (int r = 0; r < N; ++r) max_load = std::max<int64_t>(max_load, state->n_decode_tokens[r]);
  for (int i = 0; i < R; ++i) pending += queue->m_remaining[i];
  const int64_t level_hi = max_load + pending;
  if (level_hi > INT32_MAX) return fail(XP_EINVAL, "xp_schedule: pending work exceeds int32 levels");

  // Line 2: B0 with nothing selected and no candidate
  std::vector<int32_t> inc(N), ap(N, 0);
  xp_waterfill_in wi{};
  wi.n_ranks = N;
  wi.n_decode_tokens = state->n_decode_tokens;
  wi.decode_ctx_sum = state->decode_ctx_sum;
  wi.existing_assign = ap.data();
  wi.fixed_target = -1;
  wi.level_hi = int32_t(level_hi);
  wi.quantum = p->quantum;
  wi.tbt_slo = p->tbt_slo;
  wi.model = p->model;
  xp_waterfill_out wo{0, 0, 0, inc.data()};
  if ((st = xp_waterfill(&wi, &wo))) return st;
  out->ref_budget = wo.budget;

  // Lines 3-4: admission and ordering
  out->n_admitted = R > 0 ? admit(*queue, wo.budget, p->now, p->tbt_slo, out->order) : 0;
  for (int i = 0; i < R; ++i) {
    out->chunk_len[i] = 0;
    out->decode_rank[i] = -1;
  }
  if (out->request_assign)
    for (int64_t k = 0; k < int64_t(R) * N; ++k) out->request_assign[k] = 0;

  // tentative decode state for placement
  std::vector<int64_t> t_ctx(state->decode_ctx_sum, state->decode_ctx_sum + N);
  std::vector<int64_t> t_used(state->kv_used, state->kv_used + N);
  std::vector<int32_t> sel_len;
  std::vector<int64_t> sel_ctx;
  out->stop = XP_SCHED_DONE;
  out->n_selected = 0;
  for (int k = 0; k < R; ++k) {  // Lines 5-13
    const int i = out->order[k];
    wi.n_selected = int32_t(sel_len.size());
    wi.sel_len = sel_len.data();
    wi.sel_ctx = sel_ctx.data();
    wi.has_candidate = 1;
    wi.m_remaining = queue->m_remaining[i];
    wi.c_processed = queue->c_processed[i];
    wi.level_hi = 0;
    if ((st = xp_waterfill(&wi, &wo))) return st;
    if (wo.chunk_len == 0) {
      out->stop = XP_SCHED_BUDGET;
      break;
    }
    if (wo.chunk_len == queue->m_remaining[i]) {  // the chunk completes the prompt
      const int64_t need = queue->c_processed[i] + queue->m_remaining[i];
      const int g = place(N, t_ctx.data(), t_used.data(), state->kv_capacity, need, p->kv_util_threshold,
                          p->kv_headroom);
      if (g < 0) {
        out->stop = XP_SCHED_NO_HOST;
        break;
      }
      t_ctx[g] += need;
      t_used[g] += need;
      out->decode_rank[i] = g;
    }
    for (int r = 0; r < N; ++r) {
      ap[r] += inc[r];
      if (out->request_assign) out->request_assign[int64_t(i) * N + r] = inc[r];
    }
    sel_len.push_back(wo.chunk_len);
    sel_ctx.push_back(queue->c_processed[i]);
    out->chunk_len[i] = wo.chunk_len;
    out->n_selected = k + 1;
  }
  for (int r = 0; r < N; ++r) out->prefill_assign[r] = ap[r];
  return XP_OK;
}

}  // extern "C"
