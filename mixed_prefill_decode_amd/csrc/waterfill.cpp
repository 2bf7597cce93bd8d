// Waterfill dispatch and the latency model it queries (host only).
//
// ConfluxServe §6.2: T_iter = L (T_GEMM + T_ATTN) (Eq. 2) with
//   T_GEMM = f_GEMM(max_r (n_p^r + n_d^r))                      (Eq. 3)
//   T_ATTN = max(beta T_P, alpha T_D)                            (Eq. 4)
//   T_D    = max_r f_D(sum of the decode contexts on rank r)     (Eq. 5)
//   T_P    = f_comm(max_r n_p^r) + f_P((1/N) sum_i l_i (c_i + (l_i + 1)/2))   (Eq. 6, 9)
// and the affine base functions of App. D (Eq. 7, 8, 10, 11).  A path with no
// work in the iteration contributes 0.
//
// §6.3 / App. E (Algorithm 2): the dispatcher binary-searches the largest
// level n_target (a multiple of the alignment quantum q) whose iteration
// latency stays within the TBT SLO tau, with the latency evaluated on the
// dispatch that level implies (the candidate's chunk min(m, B(n)) filled
// toward n); rank r then has capacity max(0, n_target - n_d^r - n_p^r(A_p)),
// B is their sum, l = min(m, B), and the chunk is filled toward n_target
// lowest combined load first, the remainder one token each to the lowest
// rank indices at the fill level.  The paper-daily summary's worked example
// (loads 40/10/10/0, level 300 -> capacities 260/290/290/300, B = 1140) is the
// fixed-target case.
//
// Expressions are evaluated without floating-point contraction so every
// latency is the same IEEE result on every compiler.
#pragma clang fp contract(off)

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../include/xp.h"

namespace xp {
xp_status fail(xp_status code, const char* fmt, ...);
}
using xp::fail;

namespace {

double t_iter(const xp_latency_model& m, int N, const int32_t* nd, const int64_t* ctx_sum, const int64_t* np,
              int n_chunks, const int64_t* len, const int64_t* cctx) {
  int64_t max_load = 0, max_np = 0, sum_nd = 0, sum_np = 0;
  for (int r = 0; r < N; ++r) {
    max_load = std::max<int64_t>(max_load, int64_t(nd[r]) + np[r]);
    max_np = std::max<int64_t>(max_np, np[r]);
    sum_nd += nd[r];
    sum_np += np[r];
  }
  const double t_gemm = max_load > 0 ? m.gamma * double(max_load) + m.gamma0 : 0.0;
  double t_d = 0.0;
  if (sum_nd > 0) {
    t_d = m.a_d * double(ctx_sum[0]) + m.a_d0;
    for (int r = 1; r < N; ++r) t_d = std::max(t_d, m.a_d * double(ctx_sum[r]) + m.a_d0);
  }
  double t_p = 0.0;
  if (sum_np > 0) {
    int64_t w = 0;
    for (int j = 0; j < n_chunks; ++j) w += len[j] * cctx[j] + len[j] * (len[j] + 1) / 2;
    t_p = (m.a_comm * double(max_np) + m.a_comm0) + (m.a_p * (double(w) / double(N)) + m.a_p0);
  }
  const double t_attn = std::max(m.beta * t_p, m.alpha * t_d);
  return double(m.n_layers) * (t_gemm + t_attn);
}

int64_t capacity_sum(const std::vector<int64_t>& load, int64_t level) {
  int64_t b = 0;
  for (int64_t l : load) b += std::max<int64_t>(0, level - l);
  return b;
}

// fill `tokens` toward `level`; false if they do not fit
bool fill(const std::vector<int64_t>& load, int64_t tokens, int64_t level, std::vector<int64_t>& out) {
  const size_t N = load.size();
  out.assign(N, 0);
  if (tokens <= 0) return true;
  if (tokens > capacity_sum(load, level)) return false;
  int64_t lo = *std::min_element(load.begin(), load.end()), hi = level;
  while (lo < hi) {  // largest L with capacity_sum(L) <= tokens
    const int64_t mid = lo + (hi - lo + 1) / 2;
    if (capacity_sum(load, mid) <= tokens) lo = mid;
    else hi = mid - 1;
  }
  int64_t rest = tokens;
  for (size_t r = 0; r < N; ++r) {
    out[r] = std::max<int64_t>(0, lo - load[r]);
    rest -= out[r];
  }
  for (size_t r = 0; r < N && rest > 0; ++r)
    if (load[r] <= lo) {
      ++out[r];
      --rest;
    }
  return rest == 0;
}

struct Problem {
  const xp_waterfill_in* in;
  std::vector<int64_t> load, existing, lens, ctxs;
  // latency of the dispatch level n implies
  bool feasible(int64_t n, std::vector<int64_t>& add) const {
    const int N = in->n_ranks;
    const int64_t b = capacity_sum(load, n);
    const int64_t l = in->has_candidate ? std::min<int64_t>(in->m_remaining, b) : b;
    fill(load, l, n, add);
    std::vector<int64_t> np(N), len(lens), cx(ctxs);
    for (int r = 0; r < N; ++r) np[r] = existing[r] + add[r];
    if (in->has_candidate && l > 0) {
      len.push_back(l);
      cx.push_back(in->c_processed);
    }
    const double t = t_iter(*in->model, N, in->n_decode_tokens, in->decode_ctx_sum, np.data(), int(len.size()),
                            len.data(), cx.data());
    return t <= in->tbt_slo;
  }
};

}  // namespace

extern "C" {

xp_status xp_iteration_latency(const xp_latency_model* model, int32_t N, const int32_t* nd, const int64_t* ctx_sum,
                               const int32_t* np, int32_t n_chunks, const int32_t* len, const int64_t* cctx,
                               double* t) {
  if (!model || !nd || !ctx_sum || !np || !t || N < 1 || n_chunks < 0 || (n_chunks > 0 && (!len || !cctx)))
    return fail(XP_EINVAL, "xp_iteration_latency: bad argument");
  std::vector<int64_t> np64(np, np + N), len64(len, len + n_chunks), cx(cctx, cctx + n_chunks);
  *t = t_iter(*model, N, nd, ctx_sum, np64.data(), n_chunks, len64.data(), cx.data());
  return XP_OK;
}

xp_status xp_waterfill(const xp_waterfill_in* in, xp_waterfill_out* out) {
  if (!in || !out) return fail(XP_EINVAL, "xp_waterfill: null argument");
  const int N = in->n_ranks;
  if (N < 1 || !in->n_decode_tokens || !in->decode_ctx_sum || !in->model || !out->assign)
    return fail(XP_EINVAL, "xp_waterfill: n_ranks / null array");
  if (in->quantum < 1) return fail(XP_EINVAL, "xp_waterfill: quantum %d", in->quantum);
  if (in->n_selected < 0 || (in->n_selected > 0 && (!in->sel_len || !in->sel_ctx)))
    return fail(XP_EINVAL, "xp_waterfill: selected chunks");
  if (in->has_candidate && in->m_remaining < 0) return fail(XP_EINVAL, "xp_waterfill: m_remaining %d", in->m_remaining);
  if (!in->has_candidate && in->fixed_target < 0 && in->level_hi < 0)
    return fail(XP_EINVAL, "xp_waterfill: level_hi %d", in->level_hi);
  Problem p;
  p.in = in;
  p.load.resize(N);
  p.existing.resize(N);
  for (int r = 0; r < N; ++r) {
    if (in->n_decode_tokens[r] < 0 || (in->existing_assign && in->existing_assign[r] < 0))
      return fail(XP_EINVAL, "xp_waterfill: negative load on rank %d", r);
    p.existing[r] = in->existing_assign ? in->existing_assign[r] : 0;
    p.load[r] = int64_t(in->n_decode_tokens[r]) + p.existing[r];
  }
  for (int j = 0; j < in->n_selected; ++j) {
    p.lens.push_back(in->sel_len[j]);
    p.ctxs.push_back(in->sel_ctx[j]);
  }
  std::vector<int64_t> add;
  int64_t n_target;
  if (in->fixed_target >= 0) {
    n_target = in->fixed_target;
  } else {
    const int64_t q = in->quantum;
    const int64_t hi = in->has_candidate ? *std::max_element(p.load.begin(), p.load.end()) + in->m_remaining
                                         : int64_t(in->level_hi);
    if (!p.feasible(0, add)) {
      n_target = 0;
    } else {
      int64_t lo_k = 0, hi_k = (hi + q - 1) / q;
      while (lo_k < hi_k) {
        const int64_t mid = lo_k + (hi_k - lo_k + 1) / 2;
        if (p.feasible(mid * q, add)) lo_k = mid;
        else hi_k = mid - 1;
      }
      n_target = lo_k * q;
    }
  }
  const int64_t budget = capacity_sum(p.load, n_target);
  const int64_t l = in->has_candidate ? std::min<int64_t>(in->m_remaining, budget) : budget;
  if (l > INT32_MAX || n_target > INT32_MAX) return fail(XP_EINVAL, "xp_waterfill: result exceeds int32");
  if (!fill(p.load, l, n_target, add)) return fail(XP_EINVAL, "xp_waterfill: internal fill failure");
  out->n_target = int32_t(n_target);
  out->budget = budget;
  out->chunk_len = int32_t(l);
  for (int r = 0; r < N; ++r) out->assign[r] = int32_t(add[r]);
  return XP_OK;
}

}  // extern "C"
