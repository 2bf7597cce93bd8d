// C ABI: context, validation, workspace layout and the layer step.
//
// The layer step follows ConfluxServe §4 (Fig. 7): one co-batched QKV
// projection over the rank-local [prefill-chunk || decode] rows, a split
// attention region, then co-batched O projection and FFN.  The split region
// follows §6.1 (coordinated attention overlap): prefill and decode attention
// are enqueued on two streams between a fork and a join event, optionally on
// disjoint CU sets (hipExtStreamCreateWithCUMask) with decode given the fewest
// CUs that keep most of its standalone HBM bandwidth.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <memory>
#include <string>
#include <vector>

#include "xp_internal.h"

namespace xp {

static thread_local std::string g_err;

xp_status fail(xp_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

}  // namespace xp

using namespace xp;

// Timing events of the layer stages (xp_ctx_stage_timing): per stage, `cap` pairs of
// (begin, end) events, of which the first n[stage] hold recorded runs.
struct StageTimer {
  int cap = 0;
  int n[XP_STAGE_COUNT] = {};
  std::vector<hipEvent_t> ev;   // [stage][cap][2]
  hipEvent_t* pair(int stage, int i) { return &ev[(size_t(stage) * cap + i) * 2]; }
};

struct xp_ctx {
  int device = 0;
  int n_cus = 0;
  int decode_cus = 0;  // 0 serialized, -1 concurrent unmasked, k masked
  int pps = 0;
  hipStream_t s_dec = nullptr, s_pre = nullptr;
  hipEvent_t e_fork = nullptr, e_dec = nullptr, e_pre = nullptr;
  uint32_t mask_dec[8] = {}, mask_pre[8] = {};
  StageTimer timer;
};

extern "C" {

const char* xp_last_error(void) { return g_err.c_str(); }

const char* xp_build_info(void) {
  return "xp: gfx950 HIP kernels (MFMA bf16/fp32), hipcc " __clang_version__;
}

}  // extern "C"

namespace {

struct ScopedDevice {
  int prev = -1;
  explicit ScopedDevice(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    (void)hipSetDevice(dev);
  }
  ~ScopedDevice() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

// CU mask of `k` CUs spread evenly over the XCDs, assuming mask bit i lands on
// XCD i % n_xcd (the interleaving the runtime applies on multi-XCD parts); the
// hardware ids each mask reaches are checked with xp_probe_hw_ids.
void spread_mask(int n_cus, int k, uint32_t* dec, uint32_t* pre) {
  for (int w = 0; w < 8; ++w) dec[w] = pre[w] = 0;
  const int n_xcd = 8;
  for (int bit = 0; bit < n_cus && bit < 256; ++bit) {
    const int slot = bit / n_xcd;  // position of this CU inside its XCD
    const int xcd = bit % n_xcd;
    // the first k CUs in (slot, xcd) order: slot-major so every XCD gains one before any gains two
    const int order = slot * n_xcd + xcd;
    if (order < k)
      dec[bit / 32] |= 1u << (bit % 32);
    else
      pre[bit / 32] |= 1u << (bit % 32);
  }
}

int rows_of(const xp_batch_desc* d) { return d->n_prefill_local + d->n_decode; }

xp_status check_shape(const xp_layer_shape* sh) {
  if (!sh) return fail(XP_EINVAL, "null shape");
  if (sh->dtype != XP_BF16 && sh->dtype != XP_F32) return fail(XP_EINVAL, "dtype %d", sh->dtype);
  if (sh->hidden <= 0 || sh->n_q_heads <= 0 || sh->n_kv_heads <= 0 || sh->head_dim <= 0 || sh->ffn_dim <= 0)
    return fail(XP_ESHAPE, "non-positive layer dimension");
  if (sh->head_dim != 64 && sh->head_dim != 128) return fail(XP_EUNSUPPORTED, "head_dim %d (64 or 128)", sh->head_dim);
  if (sh->page_size != 16) return fail(XP_EUNSUPPORTED, "page_size %d (16)", sh->page_size);
  if (sh->n_q_heads % sh->n_kv_heads) return fail(XP_ESHAPE, "Hq %d not a multiple of Hkv %d", sh->n_q_heads, sh->n_kv_heads);
  if (sh->n_q_heads / sh->n_kv_heads > 16) return fail(XP_EUNSUPPORTED, "GQA group %d > 16", sh->n_q_heads / sh->n_kv_heads);
  const int bk = 128 / dtype_bytes(sh->dtype);
  if (sh->hidden % bk || sh->ffn_dim % bk || (sh->n_q_heads * sh->head_dim) % bk)
    return fail(XP_EUNSUPPORTED, "hidden, ffn_dim and Hq*d must be multiples of %d", bk);
  if (!(sh->rms_eps >= 0.f) || !(sh->rope_base > 0.0)) return fail(XP_EINVAL, "rms_eps / rope_base");
  return XP_OK;
}

xp_status check_desc(const xp_layer_shape* sh, const xp_batch_desc* d) {
  if (!d) return fail(XP_EINVAL, "null batch descriptor");
  const int P = d->sp_degree;
  if (d->n_prefill_local < 0 || d->n_decode < 0 || d->chunk_len < 0 || d->prior_len < 0)
    return fail(XP_ESHAPE, "negative row count");
  if (P < 1 || d->sp_rank < 0 || d->sp_rank >= P) return fail(XP_ESHAPE, "sp_degree %d / sp_rank %d", P, d->sp_rank);
  if (sh->n_q_heads % P || sh->n_kv_heads % P)
    return fail(XP_ESHAPE, "heads %d/%d not divisible by sp_degree %d", sh->n_q_heads, sh->n_kv_heads, P);
  if (d->n_prefill_local > d->chunk_len) return fail(XP_ESHAPE, "n_prefill_local > chunk_len");
  if (d->local_row_offset < 0 || d->local_row_offset + d->n_prefill_local > d->chunk_len)
    return fail(XP_ESHAPE, "local rows [%d, %d) outside the chunk of %d", d->local_row_offset,
                d->local_row_offset + d->n_prefill_local, d->chunk_len);
  if (P == 1 && d->n_prefill_local != d->chunk_len) return fail(XP_ESHAPE, "sp_degree 1 needs every chunk row local");
  if (rows_of(d) > 0 && !d->x) return fail(XP_EINVAL, "null x");
  if (d->n_decode > 0) {
    if (!d->dec_ctx || !d->dec_pages) return fail(XP_EINVAL, "null decode table");
    if (d->dec_max_blocks < 1) return fail(XP_ESHAPE, "dec_max_blocks %d", d->dec_max_blocks);
  }
  if (d->chunk_len > 0) {
    if (!d->pre_pages) return fail(XP_EINVAL, "null prefill table");
    if (long(d->pre_max_blocks) * sh->page_size < long(d->prior_len) + d->chunk_len)
      return fail(XP_EPAGE, "prefill table of %d blocks cannot hold %d positions", d->pre_max_blocks,
                  d->prior_len + d->chunk_len);
    const int n_peer = d->chunk_len - d->n_prefill_local;
    if (n_peer > 0 && (!d->peer_qkv_in || !d->peer_attn_out)) return fail(XP_EINVAL, "null peer_qkv_in / peer_attn_out");
    if (P > 1 && d->n_prefill_local > 0 && (!d->peer_qkv_out || !d->peer_attn_in))
      return fail(XP_EINVAL, "null peer_qkv_out / peer_attn_in");
  }
  return XP_OK;
}

// CUs the prefill key-split plan assumes: the CUs the prefill attention runs on (the
// whole device when serialized or unmasked, the prefill side of a CU partition
// otherwise), so that its work units fill them in few rounds.  The split points, and
// so the order in which a row's partial sums are merged, follow from that count: a
// CU-partitioned step can differ from a serialized one in the last bits of the
// prefill rows (each is within the attention tolerance of the oracle).
int prefill_cus(const xp_ctx* ctx) {
  if (!ctx) return device_cus();
  return ctx->decode_cus > 0 ? ctx->n_cus - ctx->decode_cus : ctx->n_cus;
}
int plan_cus_or_device(int plan_cus) { return plan_cus > 0 ? plan_cus : device_cus(); }

// Prefill side of a step's workspace: the rotated chunk queries and the key-split
// partials, for one chunk (the descriptor's) or a list of chunks run one after another.
struct PrefillNeed {
  size_t q_bytes = 0;     // [Hq/P, rows, d] T per chunk, chunks back to back
  size_t part_bytes = 0;  // the largest chunk's partials (chunks share them in turn)
};

xp_ws_layout make_layout_core(const xp_ctx* ctx, const xp_layer_shape* sh, const xp_batch_desc* d, size_t M,
                              const PrefillNeed& pn) {
  xp_ws_layout L;
  memset(&L, 0, sizeof(L));
  const size_t eb = dtype_bytes(sh->dtype);
  const size_t H = sh->hidden, F = sh->ffn_dim, Hq = sh->n_q_heads, Hkv = sh->n_kv_heads, D = sh->head_dim;
  const int pps = decode_pick_pps(ctx ? ctx->pps : 0, d->n_decode, int(Hkv), d->dec_max_blocks);
  const int splits = d->n_decode > 0 ? decode_splits(d->dec_max_blocks, pps) : 0;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align_up(std::max<size_t>(bytes, 1), 256);
    return o;
  };
  L.status = take(sizeof(uint32_t));
  L.hn = take(M * H * eb);
  L.qkv = take(M * (Hq + 2 * Hkv) * D * 4);
  L.q_dec = take(size_t(d->n_decode) * Hq * D * eb);
  L.q_pre = take(pn.q_bytes);
  L.attn = take(M * Hq * D * eb);
  const size_t units = size_t(d->n_decode) * Hq * splits;
  L.dec_ml = take(units * 2 * sizeof(float));
  L.dec_o = take(units * D * sizeof(float));
  L.pre_part = take(pn.part_bytes);
  {
    const int dt = sh->dtype;
    const size_t g = std::max(std::max(gemm_ws_bytes(dt, XP_EPI_F32, int(M), int((Hq + 2 * Hkv) * D), int(H)),
                                       gemm_ws_bytes(dt, XP_EPI_ADD_T, int(M), int(H), int(Hq * D))),
                              std::max(gemm_ws_bytes(dt, XP_EPI_SWIGLU, int(M), int(F), int(H)),
                                       gemm_ws_bytes(dt, XP_EPI_ADD_F32, int(M), int(H), int(F))));
    L.gemm_part = take(g);
  }
  L.h1 = take(M * H * 4);
  L.act = take(M * F * eb);
  L.total = off;
  L.dec_splits = splits;
  L.dec_pages_per_split = pps;
  return L;
}

xp_ws_layout make_layout(const xp_ctx* ctx, const xp_layer_shape* sh, const xp_batch_desc* d) {
  const size_t eb = dtype_bytes(sh->dtype), Hq = sh->n_q_heads, Hkv = sh->n_kv_heads, D = sh->head_dim;
  PrefillNeed pn;
  pn.q_bytes = size_t(Hq / d->sp_degree) * d->chunk_len * D * eb;
  pn.part_bytes = prefill_ws_bytes(int(Hq) / d->sp_degree, int(Hkv) / d->sp_degree, int(D), d->prior_len,
                                   d->chunk_len, prefill_cus(ctx));
  return make_layout_core(ctx, sh, d, size_t(rows_of(d)), pn);
}

// A multi-chunk step: the descriptor carries x, the decodes and sp_degree 1 with no
// chunk of its own; the chunks' rows come first in x, in list order.
xp_status check_chunks(const xp_layer_shape* sh, const xp_batch_desc* d, int n_chunks, const xp_chunk* ch) {
  if (d->sp_degree != 1) return fail(XP_EUNSUPPORTED, "multi-chunk steps need sp_degree 1");
  if (d->chunk_len != 0 || d->n_prefill_local != 0)
    return fail(XP_ESHAPE, "multi-chunk steps take their chunks from the list (descriptor chunk_len %d)",
                d->chunk_len);
  if (n_chunks < 0 || (n_chunks > 0 && !ch)) return fail(XP_EINVAL, "chunk list");
  long rows = d->n_decode;
  for (int j = 0; j < n_chunks; ++j) {
    const xp_chunk& c = ch[j];
    if (c.chunk_len < 1 || c.prior_len < 0) return fail(XP_ESHAPE, "chunk %d: length %d, prior %d", j, c.chunk_len, c.prior_len);
    if (!c.pre_pages) return fail(XP_EINVAL, "chunk %d: null table", j);
    if (long(c.pre_max_blocks) * sh->page_size < long(c.prior_len) + c.chunk_len)
      return fail(XP_EPAGE, "chunk %d: table of %d blocks cannot hold %d positions", j, c.pre_max_blocks,
                  c.prior_len + c.chunk_len);
    rows += c.chunk_len;
  }
  if (rows > INT32_MAX / 2) return fail(XP_ESHAPE, "too many rows");
  if (rows > 0 && !d->x) return fail(XP_EINVAL, "null x");
  return XP_OK;
}

xp_ws_layout make_layout_chunks(const xp_ctx* ctx, const xp_layer_shape* sh, const xp_batch_desc* d, int n_chunks,
                                const xp_chunk* ch) {
  const size_t eb = dtype_bytes(sh->dtype), Hq = sh->n_q_heads, Hkv = sh->n_kv_heads, D = sh->head_dim;
  PrefillNeed pn;
  size_t rows = 0;
  for (int j = 0; j < n_chunks; ++j) {  // one launch runs them all: each chunk keeps its own partials
    rows += size_t(ch[j].chunk_len);
    pn.part_bytes += align_up(prefill_ws_bytes(int(Hq), int(Hkv), int(D), ch[j].prior_len, ch[j].chunk_len,
                                               prefill_cus(ctx)), 256);
  }
  pn.q_bytes = Hq * rows * D * eb;
  return make_layout_core(ctx, sh, d, rows + size_t(d->n_decode), pn);
}

}  // namespace

extern "C" {

xp_status xp_ctx_create(xp_ctx** out, int32_t device, int32_t decode_cus, int32_t pages_per_split) {
  if (!out) return fail(XP_EINVAL, "null ctx out");
  *out = nullptr;
  int n_dev = 0;
  XP_HIP_TRY(hipGetDeviceCount(&n_dev));
  if (device < 0 || device >= n_dev) return fail(XP_EINVAL, "device %d of %d", device, n_dev);
  if (pages_per_split < 0 || pages_per_split > 64) return fail(XP_EINVAL, "pages_per_split %d (0..64)", pages_per_split);
  ScopedDevice sd(device);
  hipDeviceProp_t prop;
  XP_HIP_TRY(hipGetDeviceProperties(&prop, device));
  xp_ctx* c = new xp_ctx();
  c->device = device;
  c->n_cus = prop.multiProcessorCount;
  c->pps = pages_per_split;  // 0: chosen per batch
  if (decode_cus < -1 || decode_cus >= c->n_cus) {
    const int n_cus = c->n_cus;
    delete c;
    return fail(XP_EINVAL, "decode_cus %d (valid: -1, 0, 1..%d)", decode_cus, n_cus - 1);
  }
  c->decode_cus = decode_cus;
  hipError_t e = hipSuccess;
  if (decode_cus > 0) {
    spread_mask(c->n_cus, decode_cus, c->mask_dec, c->mask_pre);
    e = hipExtStreamCreateWithCUMask(&c->s_dec, 8, c->mask_dec);
    if (e == hipSuccess) e = hipExtStreamCreateWithCUMask(&c->s_pre, 8, c->mask_pre);
  } else {
    for (int w = 0; w < 8; ++w) c->mask_dec[w] = c->mask_pre[w] = 0xffffffffu;
    if (decode_cus == -1) {
      e = hipStreamCreateWithFlags(&c->s_dec, hipStreamNonBlocking);
      if (e == hipSuccess) e = hipStreamCreateWithFlags(&c->s_pre, hipStreamNonBlocking);
    }
  }
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->e_fork, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->e_dec, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->e_pre, hipEventDisableTiming);
  if (e != hipSuccess) {
    xp_ctx_destroy(c);
    return fail(XP_EHIP, "xp_ctx_create: %s", hipGetErrorString(e));
  }
  *out = c;
  return XP_OK;
}

xp_status xp_ctx_destroy(xp_ctx* c) {
  if (!c) return XP_OK;
  ScopedDevice sd(c->device);
  for (hipEvent_t e : c->timer.ev) (void)hipEventDestroy(e);
  if (c->s_dec) (void)hipStreamDestroy(c->s_dec);
  if (c->s_pre) (void)hipStreamDestroy(c->s_pre);
  if (c->e_fork) (void)hipEventDestroy(c->e_fork);
  if (c->e_dec) (void)hipEventDestroy(c->e_dec);
  if (c->e_pre) (void)hipEventDestroy(c->e_pre);
  delete c;
  return XP_OK;
}

xp_status xp_ctx_cu_masks(const xp_ctx* c, uint32_t* dec, uint32_t* pre, int32_t* n_cus) {
  if (!c) return fail(XP_EINVAL, "null ctx");
  for (int w = 0; w < 8; ++w) {
    if (dec) dec[w] = c->mask_dec[w];
    if (pre) pre[w] = c->mask_pre[w];
  }
  if (n_cus) *n_cus = c->n_cus;
  return XP_OK;
}

xp_status xp_ctx_streams(const xp_ctx* c, void** dec, void** pre) {
  if (!c) return fail(XP_EINVAL, "null ctx");
  if (dec) *dec = c->s_dec;
  if (pre) *pre = c->s_pre;
  return XP_OK;
}

xp_status xp_ctx_stage_timing(xp_ctx* c, int32_t capacity) {
  if (!c) return fail(XP_EINVAL, "null ctx");
  if (capacity < 0 || capacity > 4096) return fail(XP_EINVAL, "stage timing capacity %d (0..4096)", capacity);
  ScopedDevice sd(c->device);
  StageTimer& t = c->timer;
  for (int k = 0; k < XP_STAGE_COUNT; ++k) t.n[k] = 0;
  if (capacity == t.cap) return XP_OK;
  for (hipEvent_t e : t.ev) (void)hipEventDestroy(e);
  t.ev.clear();
  t.cap = 0;
  std::vector<hipEvent_t> ev(size_t(XP_STAGE_COUNT) * capacity * 2, nullptr);
  for (hipEvent_t& e : ev) {
    const hipError_t r = hipEventCreateWithFlags(&e, hipEventReleaseToDevice);
    if (r != hipSuccess) {
      for (hipEvent_t x : ev)
        if (x) (void)hipEventDestroy(x);
      return fail(XP_EHIP, "hipEventCreate: %s", hipGetErrorString(r));
    }
  }
  t.ev.swap(ev);
  t.cap = capacity;
  return XP_OK;
}

xp_status xp_ctx_stage_time(xp_ctx* c, int32_t stage, int32_t* count, double* total_ms) {
  if (!c || !count || !total_ms) return fail(XP_EINVAL, "null argument");
  if (stage < 0 || stage >= XP_STAGE_COUNT) return fail(XP_EINVAL, "stage %d (0..%d)", stage, XP_STAGE_COUNT - 1);
  ScopedDevice sd(c->device);
  StageTimer& t = c->timer;
  double sum = 0;
  for (int i = 0; i < t.n[stage]; ++i) {
    hipEvent_t* e = t.pair(stage, i);
    XP_HIP_TRY(hipEventSynchronize(e[1]));
    float ms = 0.f;
    XP_HIP_TRY(hipEventElapsedTime(&ms, e[0], e[1]));
    sum += ms;
  }
  *count = t.n[stage];
  *total_ms = sum;
  return XP_OK;
}

xp_status xp_layer_workspace_layout(const xp_ctx* ctx, const xp_layer_shape* sh, const xp_batch_desc* d,
                                    xp_ws_layout* out) {
  if (!out) return fail(XP_EINVAL, "null layout out");
  xp_status st = check_shape(sh);
  if (st) return st;
  if ((st = check_desc(sh, d))) return st;
  *out = make_layout(ctx, sh, d);
  return XP_OK;
}

}  // extern "C"

namespace {

// Marks the pages a step touches; fails on an id outside the pool or named twice.
struct PageCheck {
  std::string seen;
  int n_pages;
  explicit PageCheck(int n) : seen(size_t(n), '\0'), n_pages(n) {}
  xp_status use(int p, const char* what) {
    if (p < 0 || p >= n_pages) return fail(XP_EPAGE, "%s page id %d outside [0, %d)", what, p, n_pages);
    if (seen[size_t(p)]) return fail(XP_EPAGE, "%s page id %d named twice", what, p);
    seen[size_t(p)] = 1;
    return XP_OK;
  }
  xp_status decodes(const xp_layer_shape* sh, const xp_batch_desc* d, const int32_t* dec_ctx_h,
                    const int32_t* dec_pages_h) {
    if (d->n_decode == 0) return XP_OK;
    if (!dec_ctx_h || !dec_pages_h) return fail(XP_EINVAL, "null host decode tables");
    const int S = sh->page_size, Hkv = sh->n_kv_heads;
    for (int i = 0; i < d->n_decode; ++i) {
      const int c = dec_ctx_h[i];
      if (c < 0) return fail(XP_ESHAPE, "decode %d: context %d", i, c);
      const int nb = c / S + 1;
      if (nb > d->dec_max_blocks) return fail(XP_EPAGE, "decode %d: context %d needs %d blocks > %d", i, c, nb, d->dec_max_blocks);
      for (int g = 0; g < Hkv; ++g)
        for (int b = 0; b < nb; ++b) {
          xp_status st = use(dec_pages_h[(long(i) * Hkv + g) * d->dec_max_blocks + b], "decode");
          if (st) return st;
        }
    }
    return XP_OK;
  }
  // one prefill table: heads rows of max_blocks, positions [0, prior + len)
  xp_status chunk(const int32_t* t, int heads, int max_blocks, int prior, int len, int S, const char* what) {
    const int nb = cdiv(long(prior) + len, S);
    for (int g = 0; g < heads; ++g)
      for (int b = 0; b < nb; ++b) {
        xp_status st = use(t[long(g) * max_blocks + b], what);
        if (st) return st;
      }
    return XP_OK;
  }
};

}  // namespace

extern "C" {

xp_status xp_validate_batch(const xp_layer_shape* sh, const xp_batch_desc* d, int32_t n_pages,
                            const int32_t* dec_ctx_h, const int32_t* dec_pages_h, const int32_t* pre_pages_h) {
  xp_status st = check_shape(sh);
  if (st) return st;
  if ((st = check_desc(sh, d))) return st;
  if (n_pages <= 0) return fail(XP_ESHAPE, "n_pages %d", n_pages);
  PageCheck pc(n_pages);
  if ((st = pc.decodes(sh, d, dec_ctx_h, dec_pages_h))) return st;
  if (d->chunk_len > 0) {
    if (!pre_pages_h) return fail(XP_EINVAL, "null host prefill table");
    return pc.chunk(pre_pages_h, sh->n_kv_heads / d->sp_degree, d->pre_max_blocks, d->prior_len, d->chunk_len,
                    sh->page_size, "prefill");
  }
  return XP_OK;
}

xp_status xp_validate_chunks(const xp_layer_shape* sh, const xp_batch_desc* d, int32_t n_chunks, const xp_chunk* chunks,
                             int32_t n_pages, const int32_t* dec_ctx_h, const int32_t* dec_pages_h,
                             const int32_t* chunk_pages_h) {
  xp_status st = check_shape(sh);
  if (st) return st;
  if ((st = check_desc(sh, d)) || (st = check_chunks(sh, d, n_chunks, chunks))) return st;
  if (n_pages <= 0) return fail(XP_ESHAPE, "n_pages %d", n_pages);
  PageCheck pc(n_pages);
  if ((st = pc.decodes(sh, d, dec_ctx_h, dec_pages_h))) return st;
  if (n_chunks > 0 && !chunk_pages_h) return fail(XP_EINVAL, "null host chunk tables");
  long off = 0;
  for (int j = 0; j < n_chunks; ++j) {
    const xp_chunk& c = chunks[j];
    if ((st = pc.chunk(chunk_pages_h + off, sh->n_kv_heads, c.pre_max_blocks, c.prior_len, c.chunk_len, sh->page_size,
                       "chunk")))
      return st;
    off += long(sh->n_kv_heads) * c.pre_max_blocks;
  }
  return XP_OK;
}

xp_status xp_layer_read_status(const void* ws, const xp_ws_layout* L, uint32_t* status, void* stream) {
  if (!ws || !L || !status) return fail(XP_EINVAL, "null argument");
  hipStream_t s = static_cast<hipStream_t>(stream);
  XP_HIP_TRY(hipMemcpyAsync(status, static_cast<const char*>(ws) + L->status, sizeof(uint32_t),
                            hipMemcpyDeviceToHost, s));
  XP_HIP_TRY(hipStreamSynchronize(s));
  return XP_OK;
}

}  // extern "C"

namespace {

// The optional host copies of a step's tables (xp_batch_desc, xp_chunk): none given
// leaves the page ids to the device-side check; otherwise every table the step reads
// must have its copy, and the copies are checked like xp_validate_batch /
// xp_validate_chunks before anything is launched.
xp_status check_host_tables(const xp_layer_shape* sh, const xp_batch_desc* d, int n_pages, int n_chunks,
                            const xp_chunk* ch) {
  bool given = d->dec_ctx_host || d->dec_pages_host || d->pre_pages_host;
  for (int j = 0; j < n_chunks; ++j) given = given || ch[j].pre_pages_host;
  if (!given) return XP_OK;
  if (d->n_decode > 0 && (!d->dec_ctx_host || !d->dec_pages_host))
    return fail(XP_EINVAL, "host table copies: dec_ctx_host and dec_pages_host are both needed");
  if (d->chunk_len > 0 && !d->pre_pages_host) return fail(XP_EINVAL, "host table copies: pre_pages_host is needed");
  for (int j = 0; j < n_chunks; ++j)
    if (!ch[j].pre_pages_host) return fail(XP_EINVAL, "host table copies: chunk %d has no pre_pages_host", j);
  PageCheck pc(n_pages);
  xp_status st = pc.decodes(sh, d, d->dec_ctx_host, d->dec_pages_host);
  if (st) return st;
  if (d->chunk_len > 0 &&
      (st = pc.chunk(d->pre_pages_host, sh->n_kv_heads / d->sp_degree, d->pre_max_blocks, d->prior_len,
                     d->chunk_len, sh->page_size, "prefill")))
    return st;
  for (int j = 0; j < n_chunks; ++j)
    if ((st = pc.chunk(ch[j].pre_pages_host, sh->n_kv_heads, ch[j].pre_max_blocks, ch[j].prior_len, ch[j].chunk_len,
                       sh->page_size, "chunk")))
      return st;
  return XP_OK;
}

// One prefill chunk as the step runs it: chunk rows [off, off + n_local) are the
// rank's local rows [row0, row0 + n_local) of x; its rotated queries sit q_off bytes
// into the workspace's q region.
struct ChunkRun {
  int len, prior, off, n_local, row0;
  const int32_t* pages;
  int max_blocks;
  const void* peer_qkv_in;
  void* peer_qkv_out;
  const void* peer_attn_in;
  void* peer_attn_out;
  size_t q_off;
};

xp_status check_weights(const xp_layer_weights* w, const xp_kv_pages* kv) {
  if (!w || !w->w_qkv || !w->w_o || !w->w_gate || !w->w_up || !w->w_down || !w->g_attn || !w->g_ffn)
    return fail(XP_EINVAL, "null weight");
  if (!kv || !kv->pool || kv->n_pages <= 0) return fail(XP_EINVAL, "null or empty KV pool");
  return XP_OK;
}

// The step of ConfluxServe §4 (Fig. 7) over rows [chunk rows of every chunk || decode],
// in the three pieces a stack runs separately (§6.1, Fig. 10: graph-captured shared-linear
// segments around an eager attention region):
//   pre:    co-batched RMSNorm + QKV, RoPE and the appends;
//   attend: the split attention region (every chunk's prefill attention in turn on the
//           prefill side; serialized on `s` when split is false or the context is);
//   post:   co-batched O projection + residual, RMSNorm, gate/up + SwiGLU, down + residual.
// The layer input is `x`: [M, H] of the workload type, or fp32 when x_f32 (a stack's
// residual stream); the first RMSNorm and the O projection's residual are its only
// readers, so `out` may alias an fp32 `x`.  Every member is held by value, so a run
// outlives the caller's structs (a captured stack keeps its runs for later replays).
struct LayerRun {
  xp_ctx* ctx;
  xp_layer_shape shape;
  xp_batch_desc desc;
  std::vector<ChunkRun> ch;
  int rows_pre;
  xp_layer_weights weights;
  xp_kv_pages pool;
  float* out;
  xp_ws_layout L;
  void* workspace;
  const void* x;
  bool x_f32;
  bool clear_status;  // the first layer of a call resets the device status word
  bool timed = true;  // eager runs record the context's stage events (graph captures do not)

  // runs f() (launches on stream s) between the stage's timing events when the
  // context times stages and the stage has room left
  template <typename F>
  xp_status stage(int id, hipStream_t s, F&& f) const {
    StageTimer& t = ctx->timer;
    if (!timed || t.n[id] >= t.cap) return f();
    hipEvent_t* e = t.pair(id, t.n[id]++);
    XP_HIP_TRY(hipEventRecord(e[0], s));
    const xp_status st = f();
    XP_HIP_TRY(hipEventRecord(e[1], s));
    return st;
  }

  xp_status pre(hipStream_t s) const;
  xp_status attend(hipStream_t s, bool split) const;
  xp_status post(hipStream_t s) const;
  // RoPE + appends (+ the peer stand-ins) of one chunk's rows, the decodes with the last
  // chunk (their rows follow it in x) or alone when there is no chunk
  PostQkvArgs post_args(const ChunkRun* c, int nd, bool rope_done) const;
  // with at most one chunk the QKV projection rotates and appends in its epilogue
  bool fused_qkv() const { return ch.size() <= 1 && gemm_rope_supported(shape.dtype, shape.head_dim); }
};

PostQkvArgs LayerRun::post_args(const ChunkRun* c, int nd, bool rope_done) const {
  const xp_layer_shape* sh = &shape;
  const xp_batch_desc* d = &desc;
  const int Hq = sh->n_q_heads, Hkv = sh->n_kv_heads, D = sh->head_dim;
  const int ldq = (Hq + 2 * Hkv) * D;
  char* ws = static_cast<char*>(workspace);
  float* qkv = reinterpret_cast<float*>(ws + L.qkv);
  const size_t attn_row = size_t(Hq) * D * dtype_bytes(sh->dtype);
  const int row0 = c ? c->row0 : rows_pre;
  PostQkvArgs pa{qkv + size_t(row0) * ldq, c ? c->n_local : 0, nd, Hq, Hkv, D, sh->page_size, sh->rope_base,
                 d->dec_ctx, d->dec_pages, d->dec_max_blocks, c ? c->prior : 0, c ? c->len : 0, d->sp_degree,
                 d->sp_rank, c ? c->off : 0, c ? c->pages : nullptr, c ? c->max_blocks : 0,
                 c ? c->peer_qkv_in : nullptr, c ? c->peer_qkv_out : nullptr, c ? c->peer_attn_in : nullptr,
                 pool.pool, pool.n_pages, ws + L.q_dec, c ? ws + L.q_pre + c->q_off : nullptr,
                 ws + L.attn + size_t(row0) * attn_row, reinterpret_cast<uint32_t*>(ws + L.status)};
  pa.rope_done = rope_done ? 1 : 0;
  return pa;
}

xp_status LayerRun::pre(hipStream_t s) const {
  xp_status st;
  const xp_layer_shape* sh = &shape;
  const xp_batch_desc* d = &desc;
  const int dt = sh->dtype, H = sh->hidden, Hq = sh->n_q_heads, Hkv = sh->n_kv_heads, D = sh->head_dim;
  const int n_d = d->n_decode, M = rows_pre + n_d;
  const int ldq = (Hq + 2 * Hkv) * D;
  char* ws = static_cast<char*>(workspace);
  uint32_t* status = reinterpret_cast<uint32_t*>(ws + L.status);
  float* qkv = reinterpret_cast<float*>(ws + L.qkv);
  auto args_of = [&](const ChunkRun* c, int nd, bool rope_done) { return post_args(c, nd, rope_done); };

  // shared linear region (1): RMSNorm + QKV over all M rows.  With at most one chunk the
  // QKV projection rotates and appends in its epilogue (the RMSNorm forms each row's
  // RoPE table in the qkv region, which then holds no projection); several chunks rotate
  // per chunk afterwards.
  const ChunkRun* c0 = ch.empty() ? nullptr : &ch[0];
  const bool fused = fused_qkv();
  RopeTab rt{};
  if (fused) {
    rt.tab = reinterpret_cast<float2*>(qkv);
    rt.half = D / 2;
    rt.n_pl = c0 ? c0->n_local : 0;
    rt.pos0 = c0 ? c0->prior + c0->off : 0;
    rt.dec_ctx = d->dec_ctx;
    rope_frequencies(sh->rope_base, D, rt.inv_freq);
  }
  if ((st = stage(XP_STAGE_NORM1, s, [&] {
         return launch_rmsnorm(dt, x, x_f32 ? 1 : 0, weights.g_attn, ws + L.hn, M, H, sh->rms_eps,
                               clear_status ? status : nullptr, s, fused ? &rt : nullptr);
       })))
    return st;
  if (fused) {
    PostQkvArgs pa = args_of(c0, n_d, false);
    pa.rope_tab = rt.tab;
    if (M > 0 && (st = stage(XP_STAGE_QKV, s, [&] { return launch_gemm_rope(dt, ws + L.hn, weights.w_qkv, M, ldq, H, pa, s); })))
      return st;
    // what is left before attention: the chunk's peer rows (sequence parallel); the
    // peer_attn_in copies follow decode attention (attend)
    PostQkvArgs pp = args_of(c0, n_d, true);
    pp.only = 2;
    return stage(XP_STAGE_ROPE_APPEND, s, [&] { return launch_post_qkv(dt, pp, s); });
  }
  if (M > 0 && (st = stage(XP_STAGE_QKV, s, [&] {
                  return launch_gemm(dt, XP_EPI_F32, ws + L.hn, weights.w_qkv, nullptr, nullptr, qkv, M, ldq, H,
                                     ws + L.gemm_part, L.h1 - L.gemm_part, s);
                })))
    return st;
  return stage(XP_STAGE_ROPE_APPEND, s, [&] {
    if (ch.empty()) return launch_post_qkv(dt, args_of(nullptr, n_d, false), s);
    for (size_t j = 0; j < ch.size(); ++j) {
      const xp_status e = launch_post_qkv(dt, args_of(&ch[j], j + 1 == ch.size() ? n_d : 0, false), s);
      if (e) return e;
    }
    return xp_status(XP_OK);
  });
}

xp_status LayerRun::attend(hipStream_t s, bool split) const {
  xp_status st;
  const xp_layer_shape* sh = &shape;
  const xp_batch_desc* d = &desc;
  const xp_kv_pages* kv = &pool;
  const int dt = sh->dtype, Hq = sh->n_q_heads, Hkv = sh->n_kv_heads, D = sh->head_dim;
  const int P = d->sp_degree, r = d->sp_rank, hq_loc = Hq / P, hkv_loc = Hkv / P, n_d = d->n_decode;
  const size_t eb = dtype_bytes(dt);
  char* ws = static_cast<char*>(workspace);
  uint32_t* status = reinterpret_cast<uint32_t*>(ws + L.status);
  char* attn = ws + L.attn;
  const size_t attn_row = size_t(Hq) * D * eb;

  // Concurrent on unmasked streams, the two kernels share every CU: in bf16 both take
  // their co-resident forms, whose register and LDS budgets leave each CU room for one
  // prefill workgroup and four decode waves at once (same arithmetic, same bits; the
  // fp32 kernels do not fit those budgets).
  const bool concurrent = split && ctx->s_dec && n_d > 0 && !ch.empty();
  const bool cores = concurrent && ctx->decode_cus == XP_SPLIT_UNMASKED && dt == XP_BF16;
  auto decode = [&](hipStream_t q) {
    return launch_decode(dt, ws + L.q_dec, kv->pool, kv->n_pages, sh->page_size, d->dec_pages, d->dec_max_blocks,
                         d->dec_ctx, n_d, Hq, Hkv, D, attn + size_t(rows_pre) * attn_row, Hq * D,
                         reinterpret_cast<float*>(ws + L.dec_ml), reinterpret_cast<float*>(ws + L.dec_o),
                         L.dec_pages_per_split, status, q, cores);
  };
  // the other ranks' heads of the local prefill rows (peer_attn_in), which only the O
  // projection reads: copied on decode's stream after decode (in the concurrent modes
  // decode ends before prefill, so the copy leaves the path to attention; outside the
  // decode stage's events)
  auto peer_heads = [&](hipStream_t q) {
    if (!fused_qkv()) return xp_status(XP_OK);
    PostQkvArgs pc = post_args(ch.empty() ? nullptr : &ch[0], n_d, true);
    pc.only = 1;
    return launch_post_qkv(dt, pc, q);
  };
  auto prefill = [&](hipStream_t q) {
    if (ch.size() == 1) {
      const ChunkRun& c = ch[0];
      return launch_prefill(dt, ws + L.q_pre + c.q_off, kv->pool, kv->n_pages, sh->page_size, c.pages, c.max_blocks,
                            hq_loc, hkv_loc, D, c.prior, c.len, c.off, c.n_local,
                            attn + size_t(c.row0) * attn_row + size_t(r) * hq_loc * D * eb, Hq * D, c.peer_attn_out,
                            hq_loc * D, ws + L.pre_part, status, prefill_cus(ctx), q, cores);
    }
    // several chunks: one grouped launch, each chunk with its own partials
    std::vector<PrefillJob> jobs;
    size_t part = 0;
    for (const ChunkRun& c : ch) {
      jobs.push_back(PrefillJob{ws + L.q_pre + c.q_off, c.pages, c.max_blocks, c.prior, c.len, c.off, c.n_local,
                                attn + size_t(c.row0) * attn_row + size_t(r) * hq_loc * D * eb, Hq * D,
                                c.peer_attn_out, hq_loc * D, ws + L.pre_part + part});
      part += align_up(prefill_ws_bytes(hq_loc, hkv_loc, D, c.prior, c.len, prefill_cus(ctx)), 256);
    }
    return launch_prefill_group(dt, kv->pool, kv->n_pages, sh->page_size, hq_loc, hkv_loc, D, int(jobs.size()),
                                jobs.data(), status, prefill_cus(ctx), q, cores);
  };
  if (!concurrent) {
    if ((st = stage(XP_STAGE_DECODE, s, [&] { return decode(s); }))) return st;
    if ((st = peer_heads(s))) return st;
    if ((st = stage(XP_STAGE_PREFILL, s, [&] { return prefill(s); }))) return st;
  } else {
    XP_HIP_TRY(hipEventRecord(ctx->e_fork, s));
    XP_HIP_TRY(hipStreamWaitEvent(ctx->s_dec, ctx->e_fork, 0));
    XP_HIP_TRY(hipStreamWaitEvent(ctx->s_pre, ctx->e_fork, 0));
    if ((st = stage(XP_STAGE_DECODE, ctx->s_dec, [&] { return decode(ctx->s_dec); }))) return st;
    if ((st = peer_heads(ctx->s_dec))) return st;
    XP_HIP_TRY(hipEventRecord(ctx->e_dec, ctx->s_dec));
    if ((st = stage(XP_STAGE_PREFILL, ctx->s_pre, [&] { return prefill(ctx->s_pre); }))) return st;
    XP_HIP_TRY(hipEventRecord(ctx->e_pre, ctx->s_pre));
    XP_HIP_TRY(hipStreamWaitEvent(s, ctx->e_dec, 0));
    XP_HIP_TRY(hipStreamWaitEvent(s, ctx->e_pre, 0));
  }
  return XP_OK;
}

xp_status LayerRun::post(hipStream_t s) const {
  xp_status st;
  const int dt = shape.dtype, H = shape.hidden, HqD = shape.n_q_heads * shape.head_dim, F = shape.ffn_dim;
  const int M = rows_pre + desc.n_decode;
  if (M == 0) return XP_OK;
  char* ws = static_cast<char*>(workspace);
  float* h1 = reinterpret_cast<float*>(ws + L.h1);
  void* gp = ws + L.gemm_part;                  // GEMM K-split partials
  const size_t gpb = L.h1 - L.gemm_part;
  const xp_layer_weights* w = &weights;

  // shared linear region (2): O projection + residual, RMSNorm, gate/up + SwiGLU, down + residual
  if ((st = stage(XP_STAGE_O, s, [&] {
         return launch_gemm(dt, x_f32 ? XP_EPI_ADD_F32 : XP_EPI_ADD_T, ws + L.attn, w->w_o, nullptr, x, h1, M, H, HqD,
                            gp, gpb, s);
       })))
    return st;
  if ((st = stage(XP_STAGE_NORM2, s,
                  [&] { return launch_rmsnorm(dt, h1, 1, w->g_ffn, ws + L.hn, M, H, shape.rms_eps, nullptr, s); })))
    return st;
  if ((st = stage(XP_STAGE_GATE_UP, s, [&] {
         return launch_gemm(dt, XP_EPI_SWIGLU, ws + L.hn, w->w_gate, w->w_up, nullptr, ws + L.act, M, F, H, gp, gpb, s);
       })))
    return st;
  return stage(XP_STAGE_DOWN, s, [&] {
    return launch_gemm(dt, XP_EPI_ADD_F32, ws + L.act, w->w_down, nullptr, h1, out, M, H, F, gp, gpb, s);
  });
}

xp_status run_layer(const LayerRun& run, hipStream_t s) {
  xp_status st;
  if ((st = run.pre(s)) || (st = run.attend(s, true)) || (st = run.post(s))) return st;
  return XP_OK;
}


// A layer stack: sp_degree 1, a weight set and a pool per layer.
xp_status check_stack(const xp_layer_shape* sh, const xp_batch_desc* d, int n_layers, const xp_layer_weights* w,
                      const xp_kv_pages* kv) {
  xp_status st = check_shape(sh);
  if (st) return st;
  if ((st = check_desc(sh, d))) return st;
  if (d->sp_degree != 1) return fail(XP_EUNSUPPORTED, "layer stack: sp_degree %d (supported: 1)", d->sp_degree);
  if (n_layers < 1 || !w || !kv) return fail(XP_EINVAL, "layer stack: %d layers, weights %p, pools %p", n_layers,
                                             static_cast<const void*>(w), static_cast<const void*>(kv));
  int n_pages = INT32_MAX;
  for (int l = 0; l < n_layers; ++l) {
    if ((st = check_weights(w + l, kv + l))) return st;
    n_pages = std::min(n_pages, int(kv[l].n_pages));
  }
  // every layer reads the same tables: a page id must lie inside every layer's pool
  return check_host_tables(sh, d, n_pages, 0, nullptr);
}

// The runs of a stack, layer after layer over one batch: layer 0 reads desc->x; every
// layer writes `out`, which the next one reads as its fp32 input (the residual stream).
std::vector<LayerRun> stack_runs(xp_ctx* ctx, const xp_layer_shape* sh, const xp_batch_desc* d, int n_layers,
                                 const xp_layer_weights* w, const xp_kv_pages* kv, float* out, const xp_ws_layout& L,
                                 void* workspace) {
  std::vector<ChunkRun> ch;
  if (d->chunk_len > 0)
    ch.push_back(ChunkRun{d->chunk_len, d->prior_len, 0, d->n_prefill_local, 0, d->pre_pages, d->pre_max_blocks,
                          nullptr, nullptr, nullptr, nullptr, 0});
  std::vector<LayerRun> runs;
  for (int l = 0; l < n_layers; ++l)
    runs.push_back(LayerRun{ctx, *sh, *d, ch, d->n_prefill_local, w[l], kv[l], out, L, workspace,
                            l == 0 ? d->x : static_cast<const void*>(out), l > 0, l == 0});
  return runs;
}

}  // namespace

// A captured stack: segment k holds layer k-1's post piece (k > 0) and layer k's pre
// piece (k < n), so n layers give n + 1 graphs around n eager attention regions.
struct xp_graph {
  std::vector<LayerRun> runs;
  std::vector<hipGraph_t> graphs;
  std::vector<hipGraphExec_t> execs;
  ~xp_graph() {
    for (hipGraphExec_t e : execs) (void)hipGraphExecDestroy(e);
    for (hipGraph_t g : graphs) (void)hipGraphDestroy(g);
  }
};

extern "C" {

xp_status xp_layer_forward(xp_ctx* ctx, const xp_layer_shape* sh, const xp_batch_desc* d, const xp_layer_weights* w,
                           const xp_kv_pages* kv, float* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!ctx) return fail(XP_EINVAL, "null ctx");
  xp_status st = check_shape(sh);
  if (st) return st;
  if ((st = check_desc(sh, d))) return st;
  if ((st = check_weights(w, kv))) return st;
  if ((st = check_host_tables(sh, d, kv->n_pages, 0, nullptr))) return st;
  const int M = rows_of(d);
  if (M > 0 && !out) return fail(XP_EINVAL, "null out");
  const xp_ws_layout L = make_layout(ctx, sh, d);
  if (!workspace || workspace_bytes < L.total)
    return fail(XP_EWORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, L.total);
  std::vector<ChunkRun> ch;
  if (d->chunk_len > 0)
    ch.push_back(ChunkRun{d->chunk_len, d->prior_len, d->local_row_offset, d->n_prefill_local, 0, d->pre_pages,
                          d->pre_max_blocks, d->peer_qkv_in, d->peer_qkv_out, d->peer_attn_in, d->peer_attn_out, 0});
  return run_layer(LayerRun{ctx, *sh, *d, ch, d->n_prefill_local, *w, *kv, out, L, workspace, d->x, false, true},
                   static_cast<hipStream_t>(stream));
}

xp_status xp_layer_workspace_layout_chunks(const xp_ctx* ctx, const xp_layer_shape* sh, const xp_batch_desc* d,
                                           int32_t n_chunks, const xp_chunk* chunks, xp_ws_layout* out) {
  if (!out) return fail(XP_EINVAL, "null layout out");
  xp_status st = check_shape(sh);
  if (st) return st;
  if ((st = check_desc(sh, d)) || (st = check_chunks(sh, d, n_chunks, chunks))) return st;
  *out = make_layout_chunks(ctx, sh, d, n_chunks, chunks);
  return XP_OK;
}

xp_status xp_layer_forward_chunks(xp_ctx* ctx, const xp_layer_shape* sh, const xp_batch_desc* d, int32_t n_chunks,
                                  const xp_chunk* chunks, const xp_layer_weights* w, const xp_kv_pages* kv, float* out,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (!ctx) return fail(XP_EINVAL, "null ctx");
  xp_status st = check_shape(sh);
  if (st) return st;
  if ((st = check_desc(sh, d)) || (st = check_chunks(sh, d, n_chunks, chunks))) return st;
  if ((st = check_weights(w, kv))) return st;
  if ((st = check_host_tables(sh, d, kv->n_pages, n_chunks, chunks))) return st;
  const xp_ws_layout L = make_layout_chunks(ctx, sh, d, n_chunks, chunks);
  if (!workspace || workspace_bytes < L.total)
    return fail(XP_EWORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, L.total);
  std::vector<ChunkRun> ch;
  int rows = 0;
  size_t q_off = 0;
  const size_t q_row = size_t(sh->n_q_heads) * sh->head_dim * dtype_bytes(sh->dtype);
  for (int j = 0; j < n_chunks; ++j) {
    const xp_chunk& c = chunks[j];
    ch.push_back(ChunkRun{c.chunk_len, c.prior_len, 0, c.chunk_len, rows, c.pre_pages, c.pre_max_blocks, nullptr,
                          nullptr, nullptr, nullptr, q_off});
    rows += c.chunk_len;
    q_off += size_t(c.chunk_len) * q_row;
  }
  if (rows + d->n_decode > 0 && !out) return fail(XP_EINVAL, "null out");
  return run_layer(LayerRun{ctx, *sh, *d, ch, rows, *w, *kv, out, L, workspace, d->x, false, true},
                   static_cast<hipStream_t>(stream));
}

xp_status xp_stack_forward(xp_ctx* ctx, const xp_layer_shape* sh, const xp_batch_desc* d, int32_t n_layers,
                           const xp_layer_weights* w, const xp_kv_pages* kv, float* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!ctx) return fail(XP_EINVAL, "null ctx");
  xp_status st = check_stack(sh, d, n_layers, w, kv);
  if (st) return st;
  if (rows_of(d) > 0 && !out) return fail(XP_EINVAL, "null out");
  const xp_ws_layout L = make_layout(ctx, sh, d);
  if (!workspace || workspace_bytes < L.total)
    return fail(XP_EWORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, L.total);
  for (const LayerRun& run : stack_runs(ctx, sh, d, n_layers, w, kv, out, L, workspace))
    if ((st = run_layer(run, static_cast<hipStream_t>(stream)))) return st;
  return XP_OK;
}

xp_status xp_stack_graph_create(xp_ctx* ctx, const xp_layer_shape* sh, const xp_batch_desc* d, int32_t n_layers,
                                const xp_layer_weights* w, const xp_kv_pages* kv, float* out, void* workspace,
                                size_t workspace_bytes, void* stream, xp_graph** graph) {
  if (!graph) return fail(XP_EINVAL, "null graph out");
  *graph = nullptr;
  if (!ctx) return fail(XP_EINVAL, "null ctx");
  if (!stream) return fail(XP_EINVAL, "graph capture needs a stream other than the null stream");
  xp_status st = check_stack(sh, d, n_layers, w, kv);
  if (st) return st;
  if (rows_of(d) == 0) return fail(XP_EINVAL, "graph of an empty batch");
  if (!out) return fail(XP_EINVAL, "null out");
  const xp_ws_layout L = make_layout(ctx, sh, d);
  if (!workspace || workspace_bytes < L.total)
    return fail(XP_EWORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, L.total);
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::unique_ptr<xp_graph> g(new xp_graph);
  g->runs = stack_runs(ctx, sh, d, n_layers, w, kv, out, L, workspace);
  for (LayerRun& r : g->runs) r.timed = false;
  for (int k = 0; k <= n_layers; ++k) {
    XP_HIP_TRY(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
    st = k > 0 ? g->runs[k - 1].post(s) : XP_OK;
    if (!st && k < n_layers) st = g->runs[k].pre(s);
    hipGraph_t gr = nullptr;
    const hipError_t e = hipStreamEndCapture(s, &gr);
    if (gr) g->graphs.push_back(gr);
    if (st) return st;
    if (e != hipSuccess || !gr) return fail(XP_EHIP, "hipStreamEndCapture: %s", hipGetErrorString(e));
    hipGraphExec_t x = nullptr;
    XP_HIP_TRY(hipGraphInstantiate(&x, gr, nullptr, nullptr, 0));
    g->execs.push_back(x);
  }
  *graph = g.release();
  return XP_OK;
}

xp_status xp_graph_launch(xp_graph* graph, void* stream) {
  if (!graph) return fail(XP_EINVAL, "null graph");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t n = graph->runs.size();
  for (size_t k = 0; k <= n; ++k) {
    XP_HIP_TRY(hipGraphLaunch(graph->execs[k], s));
    if (k < n) {
      const xp_status st = graph->runs[k].attend(s, true);
      if (st) return st;
    }
  }
  return XP_OK;
}

xp_status xp_graph_destroy(xp_graph* graph) {
  delete graph;
  return XP_OK;
}

// ---- kernel-level entry points ------------------------------------------------

xp_status xp_rmsnorm(int32_t dtype, const void* x, int32_t x_is_f32, const void* gamma, void* y, int32_t M,
                     int32_t H, float eps, void* stream) {
  return launch_rmsnorm(dtype, x, x_is_f32, gamma, y, M, H, eps, nullptr, static_cast<hipStream_t>(stream));
}

size_t xp_gemm_workspace_size(int32_t dtype, int32_t epi, int32_t M, int32_t N, int32_t K) {
  if ((dtype != XP_BF16 && dtype != XP_F32) || epi < XP_EPI_F32 || epi > XP_EPI_SWIGLU) return 0;
  return gemm_ws_bytes(dtype, epi, M, N, K);
}

xp_status xp_gemm_tile(int32_t dtype, int32_t epi, int32_t M, int32_t N, int32_t K, int32_t* bm, int32_t* bn,
                       int32_t* splits) {
  if (dtype != XP_BF16 && dtype != XP_F32) return fail(XP_EINVAL, "xp_gemm_tile: dtype %d", dtype);
  if (epi < XP_EPI_F32 || epi > XP_EPI_SWIGLU) return fail(XP_EINVAL, "xp_gemm_tile: unknown epilogue %d", epi);
  if (M <= 0 || N <= 0 || K <= 0) return fail(XP_ESHAPE, "xp_gemm_tile: M=%d N=%d K=%d", M, N, K);
  if (!bm || !bn || !splits) return fail(XP_EINVAL, "xp_gemm_tile: null output");
  int a = 0, b = 0, sp = 0;
  gemm_tile(dtype, epi, M, N, K, &a, &b, &sp);
  *bm = a;
  *bn = b;
  *splits = sp;
  return XP_OK;
}

xp_status xp_gemm(int32_t dtype, int32_t epi, const void* A, const void* B, const void* B2, const void* R, void* C,
                  int32_t M, int32_t N, int32_t K, void* workspace, size_t workspace_bytes, void* stream) {
  return launch_gemm(dtype, epi, A, B, B2, R, C, M, N, K, workspace, workspace_bytes,
                     static_cast<hipStream_t>(stream));
}

xp_status xp_kv_append(int32_t dtype, void* pool, int32_t n_pages, int32_t S, int32_t d, const int32_t* table,
                       int32_t table_stride, const int32_t* seq, const int32_t* pos, const void* k, const void* v,
                       int32_t n, void* stream) {
  if (dtype != XP_BF16 && dtype != XP_F32) return fail(XP_EINVAL, "xp_kv_append: dtype %d", dtype);
  if (n < 0 || S <= 0 || d <= 0 || table_stride <= 0 || n_pages <= 0) return fail(XP_ESHAPE, "xp_kv_append: sizes");
  if (n > 0 && (!pool || !table || !seq || !pos || !k || !v)) return fail(XP_EINVAL, "xp_kv_append: null pointer");
  return launch_kv_append(dtype, pool, n_pages, S, d, table, table_stride, seq, pos, k, v, n, nullptr,
                          static_cast<hipStream_t>(stream));
}

xp_status xp_kv_gather(int32_t dtype, const void* pool, int32_t n_pages, int32_t S, int32_t d, const int32_t* table,
                       int32_t table_stride, const int32_t* len, int32_t n_seq, int32_t max_len, void* k_out,
                       void* v_out, void* stream) {
  if (dtype != XP_BF16 && dtype != XP_F32) return fail(XP_EINVAL, "xp_kv_gather: dtype %d", dtype);
  if (n_seq < 0 || max_len < 0 || S <= 0 || d <= 0 || table_stride <= 0 || n_pages <= 0)
    return fail(XP_ESHAPE, "xp_kv_gather: sizes");
  if (n_seq > 0 && max_len > 0 && (!pool || !table || !len || !k_out || !v_out))
    return fail(XP_EINVAL, "xp_kv_gather: null pointer");
  return launch_kv_gather(dtype, pool, n_pages, S, d, table, table_stride, len, n_seq, max_len, k_out, v_out,
                          static_cast<hipStream_t>(stream));
}

size_t xp_decode_workspace_size(int32_t n_d, int32_t Hq, int32_t Hkv, int32_t d, int32_t max_blocks, int32_t pps) {
  if (n_d <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || max_blocks <= 0 || pps < 0) return 0;
  return decode_ws_bytes(n_d, Hq, d, decode_splits(max_blocks, decode_pick_pps(pps, n_d, Hkv, max_blocks)));
}

xp_status xp_decode_attention(int32_t dtype, const void* q, const void* pool, int32_t n_pages, int32_t S,
                              const int32_t* dec_pages, int32_t max_blocks, const int32_t* dec_ctx, int32_t n_d,
                              int32_t Hq, int32_t Hkv, int32_t d, void* out, int32_t out_stride, void* workspace,
                              int32_t pps, void* stream) {
  if (n_d < 0) return fail(XP_ESHAPE, "xp_decode_attention: n_decode %d", n_d);
  if (n_d == 0) return XP_OK;
  if (!q || !pool || !dec_pages || !dec_ctx || !out || !workspace) return fail(XP_EINVAL, "xp_decode_attention: null pointer");
  if (out_stride < Hq * d) return fail(XP_ESHAPE, "xp_decode_attention: out_stride %d < Hq*d", out_stride);
  if (pps < 0) return fail(XP_EINVAL, "xp_decode_attention: pages_per_split %d", pps);
  if (Hkv <= 0 || max_blocks <= 0) return fail(XP_ESHAPE, "xp_decode_attention: Hkv %d max_blocks %d", Hkv, max_blocks);
  pps = decode_pick_pps(pps, n_d, Hkv, max_blocks);
  const int splits = decode_splits(max_blocks, pps);
  const size_t ml_bytes = align_up(size_t(n_d) * Hq * splits * 2 * sizeof(float), 256);
  float* ml = static_cast<float*>(workspace);
  float* po = reinterpret_cast<float*>(static_cast<char*>(workspace) + ml_bytes);
  return launch_decode(dtype, q, pool, n_pages, S, dec_pages, max_blocks, dec_ctx, n_d, Hq, Hkv, d, out, out_stride,
                       ml, po, pps, nullptr, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// Times `launch` (enqueued on the given stream) on every CU, then on CU-masked streams
// of cu_step, 2 cu_step, ... CUs: `repeats` untimed launches, then `repeats` timed
// between two events.  `stop(us_all, us_k)` ends the sweep early.  Every stream and
// event made here is destroyed before returning.
template <typename Launch, typename Stop>
xp_status cu_sweep(int device, int cu_step, int repeats, Launch&& launch, Stop&& stop, xp_cu_curve* curve) {
  ScopedDevice sd(device);
  hipDeviceProp_t prop;
  XP_HIP_TRY(hipGetDeviceProperties(&prop, device));
  const int n_cus = prop.multiProcessorCount;
  memset(curve, 0, sizeof(*curve));
  curve->n_cus = n_cus;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipStream_t s = nullptr;
  auto cleanup = [&]() {
    if (s) (void)hipStreamDestroy(s);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    s = nullptr;
  };
  auto time_on = [&](double* us) -> xp_status {
    for (int i = 0; i < repeats; ++i) {
      xp_status st = launch(s);
      if (st) return st;
    }
    XP_HIP_TRY(hipEventRecord(e0, s));
    for (int i = 0; i < repeats; ++i) {
      xp_status st = launch(s);
      if (st) return st;
    }
    XP_HIP_TRY(hipEventRecord(e1, s));
    XP_HIP_TRY(hipEventSynchronize(e1));
    float ms = 0.f;
    XP_HIP_TRY(hipEventElapsedTime(&ms, e0, e1));
    *us = 1e3 * double(ms) / repeats;
    return XP_OK;
  };
  xp_status st = XP_OK;
  hipError_t e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
  if (e != hipSuccess) {
    cleanup();
    return fail(XP_EHIP, "CU sweep set-up: %s", hipGetErrorString(e));
  }
  st = time_on(&curve->us_all);
  (void)hipStreamDestroy(s);
  s = nullptr;
  for (int k = cu_step; !st && k < n_cus && curve->n_points < XP_CU_CURVE_MAX; k += cu_step) {
    uint32_t dec[8], pre[8];
    spread_mask(n_cus, k, dec, pre);
    e = hipExtStreamCreateWithCUMask(&s, 8, dec);
    if (e != hipSuccess) {
      st = fail(XP_EHIP, "hipExtStreamCreateWithCUMask(%d CUs): %s", k, hipGetErrorString(e));
      break;
    }
    double us = 0.0;
    st = time_on(&us);
    (void)hipStreamSynchronize(s);
    (void)hipStreamDestroy(s);
    s = nullptr;
    if (st) break;
    curve->cus[curve->n_points] = k;
    curve->us[curve->n_points] = us;
    ++curve->n_points;
    if (stop(curve->us_all, us)) break;
  }
  cleanup();
  return st;
}

}  // namespace

extern "C" {

xp_status xp_calibrate_decode_cus(int32_t device, int32_t dtype, const void* q, const void* pool, int32_t n_pages,
                                  int32_t S, const int32_t* dec_pages, int32_t max_blocks, const int32_t* dec_ctx,
                                  int32_t n_d, int32_t Hq, int32_t Hkv, int32_t d, void* out, int32_t out_stride,
                                  void* workspace, int32_t pps, double keep_fraction, int32_t cu_step,
                                  int32_t repeats, int32_t stop_at_rule, int32_t* decode_cus, xp_cu_curve* curve) {
  if (!decode_cus || !curve) return fail(XP_EINVAL, "xp_calibrate_decode_cus: null output");
  if (!(keep_fraction > 0.0 && keep_fraction <= 1.0) || cu_step < 1 || repeats < 1)
    return fail(XP_EINVAL, "xp_calibrate_decode_cus: keep_fraction %g, cu_step %d, repeats %d", keep_fraction,
                cu_step, repeats);
  if (n_d < 1) return fail(XP_ESHAPE, "xp_calibrate_decode_cus: no decode requests");
  int n_dev = 0;
  XP_HIP_TRY(hipGetDeviceCount(&n_dev));
  if (device < 0 || device >= n_dev) return fail(XP_EINVAL, "xp_calibrate_decode_cus: device %d of %d", device, n_dev);
  auto launch = [&](hipStream_t s) {
    return xp_decode_attention(dtype, q, pool, n_pages, S, dec_pages, max_blocks, dec_ctx, n_d, Hq, Hkv, d, out,
                               out_stride, workspace, pps, s);
  };
  auto meets = [&](double us_all, double us) { return us_all >= keep_fraction * us; };
  xp_status st = cu_sweep(device, cu_step, repeats, launch,
                          [&](double a, double u) { return stop_at_rule != 0 && meets(a, u); }, curve);
  if (st) return st;
  if (curve->n_points == 0) return fail(XP_EINVAL, "xp_calibrate_decode_cus: cu_step %d leaves no partition", cu_step);
  *decode_cus = curve->cus[curve->n_points - 1];
  for (int i = 0; i < curve->n_points; ++i)
    if (meets(curve->us_all, curve->us[i])) {
      *decode_cus = curve->cus[i];
      break;
    }
  return XP_OK;
}

xp_status xp_probe_read_curve(int32_t device, const void* src, size_t bytes, uint32_t* sink, int32_t cu_step,
                              int32_t repeats, xp_cu_curve* curve) {
  if (!curve || !src || !sink || cu_step < 1 || repeats < 1 || bytes == 0 || bytes % 16)
    return fail(XP_EINVAL, "xp_probe_read_curve: bad argument");
  int n_dev = 0;
  XP_HIP_TRY(hipGetDeviceCount(&n_dev));
  if (device < 0 || device >= n_dev) return fail(XP_EINVAL, "xp_probe_read_curve: device %d of %d", device, n_dev);
  return cu_sweep(device, cu_step, repeats, [&](hipStream_t s) { return xp_probe_read(src, bytes, sink, s); },
                  [](double, double) { return false; }, curve);
}

size_t xp_prefill_workspace_size(int32_t hq, int32_t hkv, int32_t d, int32_t prior, int32_t chunk,
                                 int32_t plan_cus) {
  if (hq <= 0 || hkv <= 0 || hq % hkv || d <= 0 || prior < 0 || chunk <= 0 || plan_cus < 0) return 0;
  return prefill_ws_bytes(hq, hkv, d, prior, chunk, plan_cus_or_device(plan_cus));
}

xp_status xp_prefill_attention(int32_t dtype, const void* q, const void* pool, int32_t n_pages, int32_t S,
                               const int32_t* pre_pages, int32_t pre_max_blocks, int32_t hq, int32_t hkv, int32_t d,
                               int32_t prior, int32_t chunk, int32_t off, int32_t n_local, void* out_local,
                               int32_t out_local_stride, void* out_peer, int32_t out_peer_stride, void* workspace,
                               int32_t plan_cus, uint32_t* status, void* stream) {
  if (chunk < 0 || prior < 0) return fail(XP_ESHAPE, "xp_prefill_attention: chunk/prior");
  if (plan_cus < 0) return fail(XP_EINVAL, "xp_prefill_attention: plan_cus %d", plan_cus);
  if (chunk == 0) return XP_OK;
  if (!q || !pool || !pre_pages) return fail(XP_EINVAL, "xp_prefill_attention: null pointer");
  if (n_local > 0 && (!out_local || out_local_stride < hq * d)) return fail(XP_EINVAL, "xp_prefill_attention: out_local");
  if (chunk - n_local > 0 && (!out_peer || out_peer_stride < hq * d)) return fail(XP_EINVAL, "xp_prefill_attention: out_peer");
  return launch_prefill(dtype, q, pool, n_pages, S, pre_pages, pre_max_blocks, hq, hkv, d, prior, chunk, off, n_local,
                        out_local, out_local_stride, out_peer, out_peer_stride, workspace, status,
                        plan_cus_or_device(plan_cus),
                        static_cast<hipStream_t>(stream));
}

}  // extern "C"
