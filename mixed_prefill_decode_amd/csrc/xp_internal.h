// Host-side internals shared by the library's translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>

#include "../../include/xp.h"

namespace xp {

// Records the message of a failing call for xp_last_error() and returns `code`.
xp_status fail(xp_status code, const char* fmt, ...);

#define XP_HIP_TRY(expr)                                                        \
  do {                                                                          \
    hipError_t e_ = (expr);                                                     \
    if (e_ != hipSuccess) return ::xp::fail(XP_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

#define XP_CHECK_LAUNCH()                                                       \
  do {                                                                          \
    hipError_t e_ = hipGetLastError();                                          \
    if (e_ != hipSuccess) return ::xp::fail(XP_EHIP, "kernel launch: %s", hipGetErrorString(e_)); \
  } while (0)

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline int cdiv(long a, long b) { return int((a + b - 1) / b); }
inline int dtype_bytes(int dtype) { return dtype == XP_BF16 ? 2 : 4; }

// ---- launchers (each validates its own arguments) ------------------------------
struct RopeTab;
struct PostQkvArgs;
// `rope` (optional): also form each row's RoPE table (see RopeTab)
xp_status launch_rmsnorm(int dtype, const void* x, int x_is_f32, const void* gamma, void* y, int M,
                         int H, float eps, uint32_t* status_clear, hipStream_t s, const RopeTab* rope = nullptr);
// The QKV projection with RoPE and the appends fused into its epilogue (no qkv output):
// rows [0, M) are the step's local rows as PostQkvArgs describes them.  XP_EUNSUPPORTED
// when the head dimension does not divide the candidate tiles' widths.
bool gemm_rope_supported(int dtype, int d);
xp_status launch_gemm_rope(int dtype, const void* A, const void* B, int M, int N, int K, const PostQkvArgs& ra,
                           hipStream_t s);

int device_cus();   // CUs of the current device (256 when none is visible)
int gemm_chunks(int dtype, int epi, int N, int K);
int gemm_split_count(int dtype, int epi, int M, int N, int K);
size_t gemm_ws_bytes(int dtype, int epi, int M, int N, int K);
void gemm_tile(int dtype, int epi, int M, int N, int K, int* bm, int* bn, int* splits);
xp_status launch_gemm(int dtype, int epi, const void* A, const void* B, const void* B2, const void* R,
                      void* C, int M, int N, int K, void* ws, size_t ws_bytes, hipStream_t s);

struct PostQkvArgs {
  const float* qkv;
  int n_pl, n_d;
  int Hq, Hkv, d, S;
  double rope_base;
  const int32_t* dec_ctx;
  const int32_t* dec_pages;
  int dec_max_blocks;
  int prior, chunk, P, r, off;
  const int32_t* pre_pages;
  int pre_max_blocks;
  const void* peer_qkv_in;
  void* peer_qkv_out;
  const void* peer_attn_in;
  void* pool;
  int n_pages;
  void* q_dec;
  void* q_pre;
  void* attn;
  uint32_t* status;
  double inv_freq[64];       // base^(-2i/d), i < d/2: filled by launch_post_qkv
  const float2* rope_tab;    // [rows][d/2] (cos, sin) of each local row's position (fused epilogue)
  int rope_done;             // the QKV GEMM's epilogue already rotated and appended the local rows
  int only;                  // 0: every task; 1: the local rows' tasks; 2: the chunk's peer rows
  int task0;                 // first task of the launch (set by launch_post_qkv)
};

// Each row's RoPE (cos, sin) pairs, formed by the first RMSNorm launch of a step for the
// QKV GEMM's fused epilogue: tab[row][i] for i < half, at position pos0 + row for
// rows < n_pl (the chunk's local rows) and dec_ctx[row - n_pl] after them.
struct RopeTab {
  float2* tab;
  int half, n_pl, pos0;
  const int32_t* dec_ctx;
  double inv_freq[64];
};
void rope_frequencies(double base, int d, double* inv_freq);
xp_status launch_post_qkv(int dtype, const PostQkvArgs& a, hipStream_t s);

xp_status launch_kv_append(int dtype, void* pool, int n_pages, int S, int d, const int32_t* table,
                           int table_stride, const int32_t* seq, const int32_t* pos, const void* k,
                           const void* v, int n, uint32_t* status, hipStream_t s);
xp_status launch_kv_gather(int dtype, const void* pool, int n_pages, int S, int d, const int32_t* table,
                           int table_stride, const int32_t* len, int n_seq, int max_len, void* k_out,
                           void* v_out, hipStream_t s);

int decode_splits(int dec_max_blocks, int pages_per_split);
int decode_grid(int n_d, int Hkv, int n_splits);
int decode_pick_pps(int requested, int n_d, int Hkv, int dec_max_blocks);
size_t decode_ws_bytes(int n_d, int Hq, int d, int n_splits);
// `cores`: the co-resident form (four-wave workgroups that leave each CU room for one
// prefill workgroup beside them), for decode running concurrently with prefill attention
xp_status launch_decode(int dtype, const void* q, const void* pool, int n_pages, int S,
                        const int32_t* dec_pages, int dec_max_blocks, const int32_t* dec_ctx, int n_d,
                        int Hq, int Hkv, int d, void* out, int out_stride, float* part_ml,
                        float* part_o, int pages_per_split, uint32_t* status, hipStream_t s, bool cores = false);

size_t prefill_ws_bytes(int hq, int hkv, int d, int prior, int chunk, int cus);
// one chunk of a grouped prefill launch; ws holds its own partials (prefill_ws_bytes)
struct PrefillJob {
  const void* q;
  const int32_t* pre_pages;
  int pre_max_blocks;
  int prior, chunk, off, n_local;
  void* out_local;
  int out_local_stride;
  void* out_peer;
  int out_peer_stride;
  void* ws;
};
// Every job's prefill attention, up to eight chunks per launch, longest key range first.
// `cores`: the co-resident form (within 168 registers per wave, one key set), for prefill
// running concurrently with decode's co-resident form on the same CUs.
xp_status launch_prefill_group(int dtype, const void* pool, int n_pages, int S, int hq, int hkv, int d, int n,
                               const PrefillJob* jobs, uint32_t* status, int cus, hipStream_t s,
                               bool cores = false);
xp_status launch_prefill(int dtype, const void* q, const void* pool, int n_pages, int S,
                         const int32_t* pre_pages, int pre_max_blocks, int hq, int hkv, int d,
                         int prior, int chunk, int off, int n_local, void* out_local,
                         int out_local_stride, void* out_peer, int out_peer_stride, void* ws,
                         uint32_t* status, int cus, hipStream_t s, bool cores = false);

}  // namespace xp
