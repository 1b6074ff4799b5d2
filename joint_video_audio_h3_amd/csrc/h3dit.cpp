// C ABI of the H3 DiT block forward: argument checks, workspace carve-up and
// the launch sequence of one block / one forward.  All checks happen on the
// host before the first launch; nothing is enqueued on an error.
#include "../../include/h3dit.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <string>

#include "launch.h"

namespace {

thread_local std::string g_err;

h3_status fail(h3_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxRows = int64_t(1) << 24;

int64_t pad_rows(int64_t n) { return (n + 255) / 256 * 256; }

h3_status check_dims(const h3_dims* d) {
  if (!d) return fail(H3_ERR_INVALID_ARG, "dims is NULL");
  if (d->hidden <= 0 || d->heads <= 0 || d->head_dim <= 0 || d->ffn <= 0 || d->n_tags <= 0)
    return fail(H3_ERR_INVALID_ARG, "dims fields must be positive");
  if (d->hidden % 256 != 0 || d->hidden > 8192)
    return fail(H3_ERR_UNSUPPORTED, "hidden=%d: need a multiple of 256, at most 8192", d->hidden);
  if (d->head_dim != 96 && d->head_dim != 128)
    return fail(H3_ERR_UNSUPPORTED, "head_dim=%d: supported 96 or 128", d->head_dim);
  if ((d->heads * d->head_dim) % 64 != 0)
    return fail(H3_ERR_UNSUPPORTED, "heads*head_dim=%d must be a multiple of 64",
                d->heads * d->head_dim);
  if (d->ffn % 128 != 0) return fail(H3_ERR_UNSUPPORTED, "ffn=%d must be a multiple of 128", d->ffn);
  // the GEMM addresses a weight tile with 32-bit offsets from its first row
  if ((int64_t)(d->ffn + 256) * d->hidden * 2 >= ((int64_t)1 << 32))
    return fail(H3_ERR_UNSUPPORTED, "ffn=%d, hidden=%d: (ffn + 256) * hidden * 2 must be below 2^32",
                d->ffn, d->hidden);
  if (d->n_tags > 8) return fail(H3_ERR_UNSUPPORTED, "n_tags=%d: at most 8", d->n_tags);
  if (d->wfmt != H3_W_BF16 && (d->heads * d->head_dim) % 128 != 0)
    return fail(H3_ERR_UNSUPPORTED, "INT8 weights need heads*head_dim=%d to be a multiple of 128",
                d->heads * d->head_dim);
  int sum = 0;
  for (int i = 0; i < 3; ++i) {
    if (d->rope_split[i] < 0 || d->rope_split[i] % 2 != 0)
      return fail(H3_ERR_INVALID_ARG, "rope_split[%d]=%d must be even and >= 0", i, d->rope_split[i]);
    sum += d->rope_split[i];
  }
  if (sum != d->head_dim)
    return fail(H3_ERR_INVALID_ARG, "rope_split sums to %d, head_dim is %d", sum, d->head_dim);
  if (!(d->rope_theta > 0.f) || !(d->ln_eps >= 0.f) || !(d->qk_eps >= 0.f) ||
      !std::isfinite(d->rope_theta))
    return fail(H3_ERR_INVALID_ARG, "rope_theta must be > 0 and epsilons >= 0");
  if (d->wfmt != H3_W_BF16 && d->wfmt != H3_W_INT8_G32 && d->wfmt != H3_W_W8A8)
    return fail(H3_ERR_INVALID_ARG, "wfmt=%d unknown", d->wfmt);
  if (d->wfmt == H3_W_W8A8) {
    const int g = d->w8a8_group;
    if (g != 64 && g != 256 && g != 448 && g != 896)
      return fail(H3_ERR_UNSUPPORTED, "w8a8_group=%d: accepted 64, 256, 448, 896", g);
    if (d->w8a8_row_fc2 != 0 && d->w8a8_row_fc2 != 1)
      return fail(H3_ERR_INVALID_ARG, "w8a8_row_fc2=%d must be 0 or 1", d->w8a8_row_fc2);
    const int di = d->heads * d->head_dim;
    if (d->hidden % g != 0 || di % g != 0 || (!d->w8a8_row_fc2 && d->ffn % g != 0))
      return fail(H3_ERR_UNSUPPORTED,
                  "w8a8_group=%d must divide hidden=%d, heads*head_dim=%d%s (ffn=%d)", g, d->hidden, di,
                  d->w8a8_row_fc2 ? "" : " and ffn", d->ffn);
  }
  return H3_OK;
}

// W8A8: the scale group of the linear with input width K (FC2 with per-row
// scales: one group spanning K).
int w8_group(const h3_dims& d, int K, bool fc2) { return (fc2 && d.w8a8_row_fc2) ? K : d.w8a8_group; }
// the same for GemmArgs::group: 0 selects the per-row kernel
int gemm_group(const h3_dims& d, int K, bool fc2) { return (fc2 && d.w8a8_row_fc2) ? 0 : w8_group(d, K, fc2); }

h3_status check_rows(int64_t n) {
  if (n <= 0 || n > kMaxRows) return fail(H3_ERR_INVALID_ARG, "n_rows=%lld out of [1, 2^24]", (long long)n);
  return H3_OK;
}

#define H3_NEED(ptr, name)                                                          \
  do {                                                                              \
    if (!(ptr)) return fail(H3_ERR_INVALID_ARG, "%s is NULL", name);               \
    if (!al16(ptr)) return fail(H3_ERR_INVALID_ARG, "%s is not 16-byte aligned", name); \
  } while (0)
#define H3_OPT(ptr, name)                                                           \
  do {                                                                              \
    if ((ptr) && !al16(ptr)) return fail(H3_ERR_INVALID_ARG, "%s is not 16-byte aligned", name); \
  } while (0)

h3_status check_linear(const h3_dims* d, const void* w, const uint16_t* s, const uint16_t* b,
                       const char* wn, const char* sn, const char* bn) {
  H3_NEED(w, wn);
  if (d->wfmt != H3_W_BF16) H3_NEED(s, sn);
  H3_OPT(b, bn);
  return H3_OK;
}

h3_status check_weights(const h3_dims* d, const h3_block_weights* w, bool qkv, bool out, bool fc1,
                        bool fc2) {
  if (!w) return fail(H3_ERR_INVALID_ARG, "weights is NULL");
  h3_status st;
  if (qkv && (st = check_linear(d, w->w_qkv, w->s_qkv, w->b_qkv, "w_qkv", "s_qkv", "b_qkv")) != H3_OK)
    return st;
  if (out && (st = check_linear(d, w->w_out, w->s_out, w->b_out, "w_out", "s_out", "b_out")) != H3_OK)
    return st;
  if (fc1 && (st = check_linear(d, w->w_fc1, w->s_fc1, w->b_fc1, "w_fc1", "s_fc1", "b_fc1")) != H3_OK)
    return st;
  if (fc2 && (st = check_linear(d, w->w_fc2, w->s_fc2, w->b_fc2, "w_fc2", "s_fc2", "b_fc2")) != H3_OK)
    return st;
  if (qkv) {
    H3_OPT(w->q_norm, "q_norm");
    H3_OPT(w->k_norm, "k_norm");
  }
  return H3_OK;
}

h3_status check_device() {
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return fail(H3_ERR_NO_DEVICE, "no HIP device available (%s)", hipGetErrorString(e));
  }
  return H3_OK;
}

h3_status hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(H3_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return H3_OK;
}

// ---------------------------------------------------------------- workspace
struct Arena {
  float* cs;
  uint16_t *h, *q, *k, *vt, *o, *a;
  int8_t* qa;   // W8A8: int8 codes of the activation about to be consumed (h, o, h2 or a)
  float* qs;    // W8A8: its scales [K/G][n_pad]
  uint16_t* wdq;  // INT8 weights, when the workspace holds it: one linear's bf16 weights at a time
  float* tmp;     // H3_UNFUSED=1: one GEMM's fp32 output (acc + bias) before its separate epilogue
  size_t bytes;
};

// H3_UNFUSED=1 in the environment (read at every call, so it must not change
// between sizing a workspace and using it): the bf16-weight block forward runs
// each GEMM with a plain fp32 store and its epilogue (QK-norm + RoPE + scatter,
// SwiGLU, gated residual) as a separate elementwise kernel, to A/B the fused
// epilogues on the device.  Other weight formats ignore it.
bool unfused_mode(const h3_dims& d) {
  const char* e = std::getenv("H3_UNFUSED");
  return d.wfmt == H3_W_BF16 && e && std::strcmp(e, "1") == 0;
}

size_t up256(size_t b) { return (b + 255) / 256 * 256; }

// Lifetimes inside a block: cs (whole forward); h (norm1 -> QKV, then norm2 ->
// FC1); q/k/vt (QKV -> attention); o (attention -> out-proj); a (FC1 -> FC2)
// reuses the q/k/vt arena, which is dead once attention has run.  With INT8
// weights and `wdq`, one more buffer takes each linear's dequantised bf16
// weights just before its GEMM (sized for FC1's, the largest).
Arena carve(const h3_dims& d, int64_t n, char* base, bool wdq = false) {
  const size_t np = (size_t)pad_rows(n);
  const size_t D = d.hidden, Di = (size_t)d.heads * d.head_dim, F = d.ffn;
  Arena a{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += up256(bytes);
    return p;
  };
  a.cs = reinterpret_cast<float*>(take(np * d.head_dim * 4));
  a.h = reinterpret_cast<uint16_t*>(take(np * D * 2));
  const size_t head_buf = np * Di * 2;
  const size_t qkv_bytes = std::max(3 * up256(head_buf), up256(np * F * 2));
  char* qkv = take(qkv_bytes);
  a.q = reinterpret_cast<uint16_t*>(qkv);
  a.k = reinterpret_cast<uint16_t*>(qkv ? qkv + up256(head_buf) : nullptr);
  a.vt = reinterpret_cast<uint16_t*>(qkv ? qkv + 2 * up256(head_buf) : nullptr);
  a.a = reinterpret_cast<uint16_t*>(qkv);
  a.o = reinterpret_cast<uint16_t*>(take(np * Di * 2));
  if (d.wfmt == H3_W_W8A8) {
    // W8A8: the codes and scales of one activation at a time (h, o, h2, a in
    // turn), sized for the widest input and the most groups
    const size_t kmax = std::max<size_t>(std::max<size_t>(D, Di), F);
    const size_t ng = std::max<size_t>(std::max<size_t>(D / w8_group(d, (int)D, false),
                                                        Di / w8_group(d, (int)Di, false)),
                                       F / w8_group(d, (int)F, true));
    a.qa = reinterpret_cast<int8_t*>(take(np * kmax));
    a.qs = reinterpret_cast<float*>(take(np * ng * 4));
  }
  if (wdq && d.wfmt == H3_W_INT8_G32) {
    const size_t wmax = std::max(std::max(3 * Di * D, D * Di), std::max(2 * F * D, D * F));
    a.wdq = reinterpret_cast<uint16_t*>(take(wmax * 2));
  }
  if (unfused_mode(d)) a.tmp = reinterpret_cast<float*>(take(np * std::max(std::max(3 * Di, 2 * F), D) * 4));
  a.bytes = off;
  return a;
}

// The full workspace of a forward: with the dequantised-weight buffer for INT8
// weights (what h3_workspace_size reports).  A smaller workspace that still
// holds the rest runs the INT8 GEMMs on the dequantising kernel instead.
size_t full_arena_bytes(const h3_dims& d, int64_t n) { return carve(d, n, nullptr, true).bytes; }
Arena carve_ws(const h3_dims& d, int64_t n, void* ws, size_t ws_bytes) {
  return carve(d, n, static_cast<char*>(ws), ws_bytes >= full_arena_bytes(d, n));
}

// W8A8 activation buffer of the step entry points: codes [n][K], then the fp32
// row scales at byte offset roundup(n*K, 256).
size_t qa_scale_offset(int64_t n, int64_t K) { return up256((size_t)n * (size_t)K); }

// ---------------------------------------------------------------- launches
h3::GemmArgs gemm_base(const h3_dims& d, const uint16_t* A, const void* B, const uint16_t* Bs,
                       const uint16_t* bias, int M, int K, int n_out) {
  h3::GemmArgs g{};
  g.A = A;
  g.B = B;
  g.Bs = Bs;
  g.bias = bias;
  g.M = M;
  g.K = K;
  g.n_out = n_out;
  return g;
}

hipError_t do_rope(const h3_dims& d, const float* pos, int64_t n, float* cs, hipStream_t s) {
  h3::RopeArgs r{};
  r.pos = pos;
  r.cs = cs;
  r.n = (int)n;
  r.n_pad = (int)pad_rows(n);
  r.d = d.head_dim;
  r.split0 = d.rope_split[0];
  r.split1 = d.rope_split[1];
  r.split2 = d.rope_split[2];
  r.theta = d.rope_theta;
  return h3::launch_rope_table(r, s);
}

hipError_t do_adaln(const h3_dims& d, const float* x, const int32_t* tag, const uint16_t* table,
                    int which, int64_t n, uint16_t* h, hipStream_t s) {
  h3::AdalnArgs a{};
  a.x = x;
  a.tag = tag;
  a.table = table;
  a.h = h;
  a.n = (int)n;
  a.D = d.hidden;
  a.k_shift = 3 * which;
  a.k_scale = 3 * which + 1;
  a.eps = d.ln_eps;
  return h3::launch_adaln(a, s);
}

// int8 codes and scales [K/group][n_pad] of a bf16 activation [n][K]
hipError_t do_quant(const uint16_t* in, int64_t n, int K, int group, int8_t* q, float* sc, hipStream_t s) {
  h3::QuantArgs a{};
  a.in = in;
  a.q = q;
  a.s = sc;
  a.n = (int)n;
  a.K = K;
  a.group = group;
  a.ld = (int)pad_rows(n);
  return h3::launch_quant(a, s);
}

// W8A8 operands of a GEMM: the activation's scales (row stride n_pad) and the
// linear's scale group (nothing for other formats)
void set_w8(const h3_dims& d, h3::GemmArgs& g, const float* sa, int64_t n, bool fc2) {
  if (d.wfmt != H3_W_W8A8) return;
  g.sa = sa;
  g.sa_ld = (int)pad_rows(n);
  g.group = gemm_group(d, g.K, fc2);
}

// sa: the W8A8 scales of the int8 activation h (ignored otherwise)
// INT8 weights with a dequantisation buffer: the layer's bf16 weights are
// formed there first and the GEMM runs on them as bf16 (wfmt is updated)
hipError_t predequant(const h3_dims& d, h3::GemmArgs& g, int rows, uint16_t* wdq, int& wfmt,
                      hipStream_t s) {
  wfmt = d.wfmt;
  if (!wdq || d.wfmt != H3_W_INT8_G32) return hipSuccess;
  h3::DequantArgs a{};
  a.q = static_cast<const int8_t*>(g.B);
  a.s = g.Bs;
  a.out = wdq;
  a.rows = rows;
  a.K = g.K;
  hipError_t e = h3::launch_dequant_w8(a, s);
  if (e != hipSuccess) return e;
  g.B = wdq;
  g.Bs = nullptr;
  wfmt = H3_W_BF16;
  return hipSuccess;
}

hipError_t do_qkv(const h3_dims& d, const uint16_t* h, const h3_block_weights& w, const float* cs,
                  int64_t n, uint16_t* q, uint16_t* k, uint16_t* vt, hipStream_t s,
                  const float* sa = nullptr, uint16_t* wdq = nullptr) {
  const int Di = d.heads * d.head_dim;
  h3::GemmArgs g = gemm_base(d, h, w.w_qkv, w.s_qkv, w.b_qkv, (int)n, d.hidden, 3 * Di);
  int wfmt;
  if (hipError_t e = predequant(d, g, 3 * Di, wdq, wfmt, s); e != hipSuccess) return e;
  set_w8(d, g, sa, n, false);
  g.q = q;
  g.k = k;
  g.vt = vt;
  g.n_pad = (int)pad_rows(n);
  g.heads = d.heads;
  g.head_dim = d.head_dim;
  g.gq = w.q_norm;
  g.gk = w.k_norm;
  g.cs = cs;
  g.qk_eps = d.qk_eps;
  g.q_scale = (float)(1.4426950408889634 / std::sqrt((double)d.head_dim));
  return h3::launch_gemm(h3::EPI_QKV, wfmt, g, s);
}

// Block-sparse attention selection of one block (null = full attention).
struct Sparse {
  int tile;
  const int32_t* off;   // [heads * ceil(n / tile) + 1]
  const int32_t* idx;
};

hipError_t do_attn(const h3_dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* vt,
                   int64_t n, uint16_t* o, hipStream_t s, const Sparse* sp = nullptr) {
  h3::AttnArgs a{};
  if (sp) {
    a.tile = sp->tile;
    a.tile_off = sp->off;
    a.tile_idx = sp->idx;
  }
  a.q = q;
  a.k = k;
  a.vt = vt;
  a.o = o;
  a.n = (int)n;
  a.n_pad = (int)pad_rows(n);
  a.heads = d.heads;
  a.head_dim = d.head_dim;
  return h3::launch_attention(a, s);
}

hipError_t do_resid(const h3_dims& d, const uint16_t* A, const void* W, const uint16_t* S,
                    const uint16_t* b, int K, const uint16_t* table, int kgate, const int32_t* tag,
                    int64_t n, float* x, hipStream_t s, const float* sa = nullptr, uint16_t* wdq = nullptr) {
  h3::GemmArgs g = gemm_base(d, A, W, S, b, (int)n, K, d.hidden);
  int wfmt;
  if (hipError_t e = predequant(d, g, d.hidden, wdq, wfmt, s); e != hipSuccess) return e;
  set_w8(d, g, sa, n, kgate == 5);
  g.x = x;
  g.ldx = d.hidden;
  g.gate_tab = table + (size_t)kgate * d.hidden;
  g.tag = tag;
  g.tag_stride = 6 * d.hidden;
  return h3::launch_gemm(h3::EPI_RESID, wfmt, g, s);
}

hipError_t do_fc1(const h3_dims& d, const uint16_t* h2, const h3_block_weights& w, int64_t n,
                  uint16_t* a, hipStream_t s, const float* sa = nullptr, uint16_t* wdq = nullptr) {
  h3::GemmArgs g = gemm_base(d, h2, w.w_fc1, w.s_fc1, w.b_fc1, (int)n, d.hidden, 2 * d.ffn);
  int wfmt;
  if (hipError_t e = predequant(d, g, 2 * d.ffn, wdq, wfmt, s); e != hipSuccess) return e;
  set_w8(d, g, sa, n, false);
  g.out = a;
  g.ffn = d.ffn;
  return h3::launch_gemm(h3::EPI_SWIGLU, wfmt, g, s);
}

// W8A8 block: each linear's bf16 input is quantized (per row and scale group)
// right after it is made, into the arena's code and scale buffers.
h3_status run_block_w8a8(const h3_dims& d, float* x, const int32_t* tag, const uint16_t* table,
                         const h3_block_weights& w, int64_t n, const Arena& ar, hipStream_t s,
                         const Sparse* sp) {
  const int D = d.hidden, Di = d.heads * d.head_dim, F = d.ffn;
  const uint16_t* qa = reinterpret_cast<const uint16_t*>(ar.qa);
  h3_status st;
  if ((st = hip_ok(do_adaln(d, x, tag, table, 0, n, ar.h, s), "adaln (attention)")) != H3_OK) return st;
  if ((st = hip_ok(do_quant(ar.h, n, D, w8_group(d, D, false), ar.qa, ar.qs, s), "quantize h")) != H3_OK)
    return st;
  if ((st = hip_ok(do_qkv(d, qa, w, ar.cs, n, ar.q, ar.k, ar.vt, s, ar.qs), "qkv+rope")) != H3_OK) return st;
  if ((st = hip_ok(do_attn(d, ar.q, ar.k, ar.vt, n, ar.o, s, sp), "attention")) != H3_OK) return st;
  if ((st = hip_ok(do_quant(ar.o, n, Di, w8_group(d, Di, false), ar.qa, ar.qs, s), "quantize o")) != H3_OK)
    return st;
  if ((st = hip_ok(do_resid(d, qa, w.w_out, w.s_out, w.b_out, Di, table, 2, tag, n, x, s, ar.qs),
                   "out-proj+gate")) != H3_OK)
    return st;
  if ((st = hip_ok(do_adaln(d, x, tag, table, 1, n, ar.h, s), "adaln (mlp)")) != H3_OK) return st;
  if ((st = hip_ok(do_quant(ar.h, n, D, w8_group(d, D, false), ar.qa, ar.qs, s), "quantize h2")) != H3_OK)
    return st;
  if ((st = hip_ok(do_fc1(d, qa, w, n, ar.a, s, ar.qs), "fc1+swiglu")) != H3_OK) return st;
  if ((st = hip_ok(do_quant(ar.a, n, F, w8_group(d, F, true), ar.qa, ar.qs, s), "quantize a")) != H3_OK)
    return st;
  if ((st = hip_ok(do_resid(d, qa, w.w_fc2, w.s_fc2, w.b_fc2, F, table, 5, tag, n, x, s, ar.qs),
                   "fc2+gate")) != H3_OK)
    return st;
  return H3_OK;
}

// H3_UNFUSED=1: a GEMM's output acc + bias stored as fp32 [n][n_out] into tmp
hipError_t do_store_f32(const h3_dims& d, const uint16_t* A, const void* W, const uint16_t* b, int K, int n_out,
                        int64_t n, float* tmp, hipStream_t s) {
  h3::GemmArgs g = gemm_base(d, A, W, nullptr, b, (int)n, K, n_out);
  g.x = tmp;
  g.ldx = n_out;
  return h3::launch_gemm(h3::EPI_STORE, H3_W_BF16, g, s);
}

// The bf16 block with every GEMM epilogue run as its own kernel (H3_UNFUSED=1).
h3_status run_block_unfused(const h3_dims& d, float* x, const int32_t* tag, const uint16_t* table,
                            const h3_block_weights& w, int64_t n, const Arena& ar, hipStream_t s,
                            const Sparse* sp) {
  const int D = d.hidden, Di = d.heads * d.head_dim, F = d.ffn;
  h3_status st;
  if ((st = hip_ok(do_adaln(d, x, tag, table, 0, n, ar.h, s), "adaln (attention)")) != H3_OK) return st;
  h3::UnfusedQkvArgs qa{};
  qa.u = ar.tmp;
  qa.gq = w.q_norm;
  qa.gk = w.k_norm;
  qa.cs = ar.cs;
  qa.q = ar.q;
  qa.k = ar.k;
  qa.vt = ar.vt;
  qa.n = (int)n;
  qa.n_pad = (int)pad_rows(n);
  qa.heads = d.heads;
  qa.head_dim = d.head_dim;
  qa.eps = d.qk_eps;
  qa.q_scale = (float)(1.4426950408889634 / std::sqrt((double)d.head_dim));
  if ((st = hip_ok(do_store_f32(d, ar.h, w.w_qkv, w.b_qkv, D, 3 * Di, n, ar.tmp, s), "qkv (unfused)")) != H3_OK ||
      (st = hip_ok(h3::launch_unfused_qkv(qa, s), "qk-norm+rope (unfused)")) != H3_OK)
    return st;
  if ((st = hip_ok(do_attn(d, ar.q, ar.k, ar.vt, n, ar.o, s, sp), "attention")) != H3_OK) return st;
  if ((st = hip_ok(do_store_f32(d, ar.o, w.w_out, w.b_out, Di, D, n, ar.tmp, s), "out-proj (unfused)")) != H3_OK ||
      (st = hip_ok(h3::launch_unfused_resid(ar.tmp, n, D, table + (size_t)2 * D, tag, 6 * D, x, s),
                   "gate1 residual (unfused)")) != H3_OK)
    return st;
  if ((st = hip_ok(do_adaln(d, x, tag, table, 1, n, ar.h, s), "adaln (mlp)")) != H3_OK) return st;
  if ((st = hip_ok(do_store_f32(d, ar.h, w.w_fc1, w.b_fc1, D, 2 * F, n, ar.tmp, s), "fc1 (unfused)")) != H3_OK ||
      (st = hip_ok(h3::launch_unfused_swiglu(ar.tmp, n, F, ar.a, s), "swiglu (unfused)")) != H3_OK)
    return st;
  if ((st = hip_ok(do_store_f32(d, ar.a, w.w_fc2, w.b_fc2, F, D, n, ar.tmp, s), "fc2 (unfused)")) != H3_OK ||
      (st = hip_ok(h3::launch_unfused_resid(ar.tmp, n, D, table + (size_t)5 * D, tag, 6 * D, x, s),
                   "gate2 residual (unfused)")) != H3_OK)
    return st;
  return H3_OK;
}

h3_status run_block(const h3_dims& d, float* x, const int32_t* tag, const uint16_t* table,
                    const h3_block_weights& w, int64_t n, const Arena& ar, hipStream_t s,
                    const Sparse* sp = nullptr) {
  if (d.wfmt == H3_W_W8A8) return run_block_w8a8(d, x, tag, table, w, n, ar, s, sp);
  if (ar.tmp && d.wfmt == H3_W_BF16) return run_block_unfused(d, x, tag, table, w, n, ar, s, sp);
  const int Di = d.heads * d.head_dim;
  h3_status st;
  if ((st = hip_ok(do_adaln(d, x, tag, table, 0, n, ar.h, s), "adaln (attention)")) != H3_OK) return st;
  if ((st = hip_ok(do_qkv(d, ar.h, w, ar.cs, n, ar.q, ar.k, ar.vt, s, nullptr, ar.wdq), "qkv+rope")) != H3_OK)
    return st;
  if ((st = hip_ok(do_attn(d, ar.q, ar.k, ar.vt, n, ar.o, s, sp), "attention")) != H3_OK) return st;
  if ((st = hip_ok(do_resid(d, ar.o, w.w_out, w.s_out, w.b_out, Di, table, 2, tag, n, x, s, nullptr, ar.wdq),
                   "out-proj+gate")) != H3_OK)
    return st;
  if ((st = hip_ok(do_adaln(d, x, tag, table, 1, n, ar.h, s), "adaln (mlp)")) != H3_OK) return st;
  if ((st = hip_ok(do_fc1(d, ar.h, w, n, ar.a, s, nullptr, ar.wdq), "fc1+swiglu")) != H3_OK) return st;
  if ((st = hip_ok(do_resid(d, ar.a, w.w_fc2, w.s_fc2, w.b_fc2, d.ffn, table, 5, tag, n, x, s, nullptr,
                            ar.wdq),
                   "fc2+gate")) != H3_OK)
    return st;
  return H3_OK;
}

// With H3_CHECK=1 in the environment, the modality tags are checked on the
// device before anything else is enqueued: one small kernel counting into a
// static device counter, then a wait for the stream (so not for use under
// stream capture, and check-mode calls that overlap on one device share the
// counter).  Any tag outside [0, n_tags) fails the call with nothing else
// enqueued.
h3_status check_tags(const h3_dims& d, const int32_t* tag, int64_t n, hipStream_t s) {
  const char* e = std::getenv("H3_CHECK");
  if (!e || std::strcmp(e, "1") != 0) return H3_OK;
  unsigned int* bad = nullptr;
  unsigned int host = 0;
  h3_status st;
  if ((st = hip_ok(h3::bad_tags_counter(&bad), "H3_CHECK counter")) != H3_OK) return st;
  hipError_t r = hipMemsetAsync(bad, 0, sizeof(unsigned int), s);
  if (r == hipSuccess) r = h3::launch_count_bad_tags(tag, n, d.n_tags, bad, s);
  if (r == hipSuccess) r = hipMemcpyAsync(&host, bad, sizeof(unsigned int), hipMemcpyDeviceToHost, s);
  if (r == hipSuccess) r = hipStreamSynchronize(s);
  if ((st = hip_ok(r, "H3_CHECK tag scan")) != H3_OK) return st;
  if (host != 0)
    return fail(H3_ERR_INVALID_ARG, "%u modality tags outside [0, %d) (H3_CHECK)", host, d.n_tags);
  return H3_OK;
}

h3_status check_forward_common(const h3_dims* dims, const float* x, const int32_t* tag,
                               const float* pos, const uint16_t* table, int64_t n, void* ws,
                               size_t ws_bytes) {
  h3_status st;
  if ((st = check_dims(dims)) != H3_OK) return st;
  if ((st = check_rows(n)) != H3_OK) return st;
  H3_NEED(x, "x");
  H3_NEED(tag, "modality_tag");
  H3_NEED(pos, "positions");
  H3_NEED(table, "mod_table");
  H3_NEED(ws, "workspace");
  const size_t need = carve(*dims, n, nullptr).bytes;
  if (ws_bytes < need)
    return fail(H3_ERR_WORKSPACE, "workspace is %zu bytes, %zu needed", ws_bytes, need);
  return H3_OK;
}

// ---------------------------------------------------------------- around the block stack
bool patch_ok(int p) { return p == 32 || p == 64 || p == 96 || p == 128; }

h3_status check_io(const h3_dims* d, const h3_io_dims* io, const h3_segments* sg) {
  h3_status st;
  if ((st = check_dims(d)) != H3_OK) return st;
  if (!io) return fail(H3_ERR_INVALID_ARG, "io_dims is NULL");
  if (!sg) return fail(H3_ERR_INVALID_ARG, "segments is NULL");
  if (sg->text < 0 || sg->cond < 0 || sg->audio < 0 || sg->video < 0)
    return fail(H3_ERR_INVALID_ARG, "segment row counts must be >= 0");
  if ((st = check_rows(sg->text + sg->cond + sg->audio + sg->video)) != H3_OK) return st;
  if (io->text_dim <= 0 || io->text_dim % 64 != 0)
    return fail(H3_ERR_UNSUPPORTED, "text_dim=%d must be a positive multiple of 64", io->text_dim);
  if (!patch_ok(io->video_patch) || !patch_ok(io->audio_patch))
    return fail(H3_ERR_UNSUPPORTED, "patch widths video=%d audio=%d: supported 32, 64, 96, 128",
                io->video_patch, io->audio_patch);
  return H3_OK;
}

h3_status check_embed_ptrs(const h3_segments& sg, const h3_io_weights* w, const void* text,
                           const void* cond, const void* audio, const void* video, const void* x) {
  if (!w) return fail(H3_ERR_INVALID_ARG, "io_weights is NULL");
  H3_NEED(x, "x_packed");
  if (sg.text > 0) {
    H3_NEED(text, "text");
    H3_NEED(w->w_text, "w_text");
    H3_OPT(w->b_text, "b_text");
  }
  if (sg.cond > 0) H3_NEED(cond, "cond");
  if (sg.video > 0) H3_NEED(video, "video");
  if (sg.cond > 0 || sg.video > 0) {
    H3_NEED(w->w_video, "w_video");
    H3_OPT(w->b_video, "b_video");
  }
  if (sg.audio > 0) {
    H3_NEED(audio, "audio");
    H3_NEED(w->w_audio, "w_audio");
    H3_OPT(w->b_audio, "b_audio");
  }
  return H3_OK;
}

h3_status check_head_ptrs(const h3_segments& sg, const h3_io_weights* w, const void* x,
                          const void* final_table, const void* vel_audio, const void* vel_video) {
  if (!w) return fail(H3_ERR_INVALID_ARG, "io_weights is NULL");
  H3_NEED(x, "x_packed");
  H3_NEED(final_table, "final_table");
  if (sg.audio > 0) {
    H3_NEED(vel_audio, "vel_audio");
    H3_NEED(w->w_head_audio, "w_head_audio");
    H3_OPT(w->b_head_audio, "b_head_audio");
  }
  if (sg.video > 0) {
    H3_NEED(vel_video, "vel_video");
    H3_NEED(w->w_head_video, "w_head_video");
    H3_OPT(w->b_head_video, "b_head_video");
  }
  return H3_OK;
}

size_t heads_ws_bytes(const h3_dims& d, const h3_segments& sg) {
  return up256((size_t)std::max(sg.audio, sg.video) * d.hidden * 2);
}

hipError_t do_patch(const h3_dims& d, const float* in, const float* W, const float* b, int P,
                    int64_t rows, float* out, hipStream_t s) {
  h3::PatchArgs a{};
  a.in = in;
  a.W = W;
  a.bias = b;
  a.out = out;
  a.rows = (int)rows;
  a.P = P;
  a.D = d.hidden;
  return h3::launch_patch_embed(a, s);
}

h3_status run_embed(const h3_dims& d, const h3_io_dims& io, const h3_io_weights& w,
                    const h3_segments& sg, const uint16_t* text, const float* cond,
                    const float* audio, const float* video, float* x, hipStream_t s) {
  const size_t D = d.hidden;
  h3_status st;
  if (sg.text > 0) {
    h3::GemmArgs g = gemm_base(d, text, w.w_text, nullptr, w.b_text, (int)sg.text, io.text_dim, d.hidden);
    g.x = x;
    g.ldx = d.hidden;
    if ((st = hip_ok(h3::launch_gemm(h3::EPI_STORE, H3_W_BF16, g, s), "text projection")) != H3_OK)
      return st;
  }
  float* xc = x + (size_t)sg.text * D;
  float* xa = xc + (size_t)sg.cond * D;
  float* xv = xa + (size_t)sg.audio * D;
  if (sg.cond > 0 &&
      (st = hip_ok(do_patch(d, cond, w.w_video, w.b_video, io.video_patch, sg.cond, xc, s),
                   "condition patch projection")) != H3_OK)
    return st;
  if (sg.audio > 0 &&
      (st = hip_ok(do_patch(d, audio, w.w_audio, w.b_audio, io.audio_patch, sg.audio, xa, s),
                   "audio patch projection")) != H3_OK)
    return st;
  if (sg.video > 0 &&
      (st = hip_ok(do_patch(d, video, w.w_video, w.b_video, io.video_patch, sg.video, xv, s),
                   "video patch projection")) != H3_OK)
    return st;
  return H3_OK;
}

// Final AdaLN of one modality's slice (one (shift, scale) pair for all its rows)
// into h, then its output head into vel.
h3_status run_head(const h3_dims& d, const float* x_rows, int64_t rows, const uint16_t* tab_m,
                   const uint16_t* w_head, const uint16_t* b_head, int P, uint16_t* h, float* vel,
                   hipStream_t s, const char* what) {
  h3_status st;
  if ((st = hip_ok(do_adaln(d, x_rows, nullptr, tab_m, 0, rows, h, s), what)) != H3_OK) return st;
  h3::GemmArgs g = gemm_base(d, h, w_head, nullptr, b_head, (int)rows, d.hidden, P);
  g.x = vel;
  g.ldx = P;
  return hip_ok(h3::launch_gemm(h3::EPI_STORE, H3_W_BF16, g, s), what);
}

h3_status run_heads(const h3_dims& d, const h3_io_dims& io, const h3_io_weights& w,
                    const h3_segments& sg, const float* x, const uint16_t* final_table,
                    float* vel_audio, float* vel_video, uint16_t* h, hipStream_t s) {
  const size_t D = d.hidden;
  const float* xa = x + (size_t)(sg.text + sg.cond) * D;
  const float* xv = xa + (size_t)sg.audio * D;
  h3_status st;
  if (sg.audio > 0 &&
      (st = run_head(d, xa, sg.audio, final_table, w.w_head_audio, w.b_head_audio, io.audio_patch,
                     h, vel_audio, s, "audio head")) != H3_OK)
    return st;
  if (sg.video > 0 &&
      (st = run_head(d, xv, sg.video, final_table + 2 * D, w.w_head_video, w.b_head_video,
                     io.video_patch, h, vel_video, s, "video head")) != H3_OK)
    return st;
  return H3_OK;
}

h3_status check_sparse(int tile, const int32_t* off, const int32_t* idx) {
  if (tile != 64 && tile != 128) return fail(H3_ERR_UNSUPPORTED, "tile=%d: supported 64 or 128", tile);
  if (!off || !idx) return fail(H3_ERR_INVALID_ARG, "tile_off / tile_idx is NULL");
  if ((reinterpret_cast<uintptr_t>(off) | reinterpret_cast<uintptr_t>(idx)) & 3u)
    return fail(H3_ERR_INVALID_ARG, "tile_off / tile_idx is not 4-byte aligned");
  return H3_OK;
}

// Scales of a step entry point's activation buffer (W8A8), else null.
const float* act_scales(const h3_dims& d, const void* act, int64_t n, int64_t K) {
  if (d.wfmt != H3_W_W8A8) return nullptr;
  return reinterpret_cast<const float*>(static_cast<const char*>(act) + qa_scale_offset(n, K));
}

// Velocity history of the denoising loop, after the block arena: two slots per
// modality (the last two fresh velocities), each 256-byte aligned.
struct VelHistory {
  size_t a_bytes, v_bytes, bytes;
};
VelHistory vel_history(const h3_io_dims& io, const h3_segments& sg) {
  VelHistory h{};
  h.a_bytes = up256((size_t)sg.audio * io.audio_patch * 4);
  h.v_bytes = up256((size_t)sg.video * io.video_patch * 4);
  h.bytes = 2 * (h.a_bytes + h.v_bytes);
  return h;
}

}  // namespace

extern "C" {

int64_t h3_padded_rows(int64_t n_rows) { return n_rows <= 0 ? 0 : pad_rows(n_rows); }

h3_status h3_attention_sparse(const h3_dims* dims, const uint16_t* q, const uint16_t* k,
                              const uint16_t* vt, int64_t n_rows, int32_t tile,
                              const int32_t* tile_off, const int32_t* tile_idx, uint16_t* o,
                              void* stream) {
  g_err.clear();
  h3_status st;
  if ((st = check_dims(dims)) != H3_OK || (st = check_rows(n_rows)) != H3_OK) return st;
  H3_NEED(q, "q");
  H3_NEED(k, "k");
  H3_NEED(vt, "vt");
  H3_NEED(o, "o");
  if ((st = check_sparse(tile, tile_off, tile_idx)) != H3_OK) return st;
  if ((st = check_device()) != H3_OK) return st;
  const Sparse sp{tile, tile_off, tile_idx};
  return hip_ok(do_attn(*dims, q, k, vt, n_rows, o, reinterpret_cast<hipStream_t>(stream), &sp),
                "sparse attention");
}

h3_status h3_dit_forward_sparse(const h3_dims* dims, float* x, const int32_t* tag,
                                const float* positions, const uint16_t* mod_table,
                                const h3_block_weights* weights, int32_t n_blocks, int64_t n_rows,
                                int32_t tile, const int32_t* tile_off, const int32_t* tile_idx,
                                void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  h3_status st;
  if ((st = check_forward_common(dims, x, tag, positions, mod_table, n_rows, workspace,
                                 workspace_bytes)) != H3_OK)
    return st;
  if (n_blocks <= 0) return fail(H3_ERR_INVALID_ARG, "n_blocks=%d must be positive", n_blocks);
  if (!weights) return fail(H3_ERR_INVALID_ARG, "weights is NULL");
  for (int b = 0; b < n_blocks; ++b) {
    if ((st = check_weights(dims, &weights[b], true, true, true, true)) != H3_OK) {
      std::string m = g_err;
      return fail(st, "block %d: %s", b, m.c_str());
    }
  }
  if ((st = check_sparse(tile, tile_off, tile_idx)) != H3_OK) return st;
  if ((st = check_device()) != H3_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((st = check_tags(*dims, tag, n_rows, s)) != H3_OK) return st;
  const Arena ar = carve_ws(*dims, n_rows, workspace, workspace_bytes);
  if ((st = hip_ok(do_rope(*dims, positions, n_rows, ar.cs, s), "rope table")) != H3_OK) return st;
  const size_t tstride = (size_t)dims->n_tags * 6 * dims->hidden;
  const int64_t nq = (n_rows + tile - 1) / tile;
  for (int b = 0; b < n_blocks; ++b) {
    const Sparse sp{tile, tile_off + (size_t)b * (dims->heads * nq + 1), tile_idx};
    if ((st = run_block(*dims, x, tag, mod_table + b * tstride, weights[b], n_rows, ar, s, &sp)) != H3_OK) {
      std::string m = g_err;
      return fail(st, "block %d: %s", b, m.c_str());
    }
  }
  return H3_OK;
}

h3_status h3_sigma_schedule(int32_t n_steps, double shift, double* sigmas) {
  g_err.clear();
  if (n_steps <= 0 || n_steps > 100000) return fail(H3_ERR_INVALID_ARG, "n_steps=%d out of [1, 100000]", n_steps);
  if (!(shift > 0.0) || !std::isfinite(shift)) return fail(H3_ERR_INVALID_ARG, "shift must be > 0");
  if (!sigmas) return fail(H3_ERR_INVALID_ARG, "sigmas is NULL");
  for (int i = 0; i < n_steps; ++i) {
    const double b = 1.0 - (double)i / (double)n_steps;
    sigmas[i] = shift * b / (1.0 + (shift - 1.0) * b);
  }
  sigmas[n_steps] = 0.0;
  return H3_OK;
}

h3_status h3_denoise(const h3_dims* dims, const h3_io_dims* io_dims, const h3_io_weights* io_weights,
                     const h3_segments* segments, const uint16_t* text, const float* cond,
                     float* audio, float* video, const int32_t* tag, const float* positions,
                     const uint16_t* mod_tables, const h3_block_weights* weights, int32_t n_blocks,
                     const uint16_t* final_tables, const double* sigmas_audio,
                     const double* sigmas_video, int32_t n_steps, int32_t reuse, float* x_packed,
                     void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  h3_status st;
  if ((st = check_io(dims, io_dims, segments)) != H3_OK) return st;
  const h3_segments sg = *segments;
  const int64_t n = sg.text + sg.cond + sg.audio + sg.video;
  if (n_steps <= 0) return fail(H3_ERR_INVALID_ARG, "n_steps=%d must be positive", n_steps);
  if (reuse <= 0) return fail(H3_ERR_INVALID_ARG, "reuse=%d must be positive", reuse);
  if (n_blocks <= 0) return fail(H3_ERR_INVALID_ARG, "n_blocks=%d must be positive", n_blocks);
  if (!sigmas_audio || !sigmas_video) return fail(H3_ERR_INVALID_ARG, "sigmas_audio / sigmas_video is NULL");
  if ((st = check_embed_ptrs(sg, io_weights, text, cond, audio, video, x_packed)) != H3_OK) return st;
  if ((st = check_head_ptrs(sg, io_weights, x_packed, final_tables, audio, video)) != H3_OK) return st;
  if ((st = check_forward_common(dims, x_packed, tag, positions, mod_tables, n, workspace,
                                 workspace_bytes)) != H3_OK)
    return st;
  const size_t arena = full_arena_bytes(*dims, n);
  const VelHistory vh = vel_history(*io_dims, sg);
  if (workspace_bytes < arena + vh.bytes)
    return fail(H3_ERR_WORKSPACE, "workspace is %zu bytes, %zu needed (h3_denoise_workspace_size)",
                workspace_bytes, arena + vh.bytes);
  if (!weights) return fail(H3_ERR_INVALID_ARG, "weights is NULL");
  for (int b = 0; b < n_blocks; ++b) {
    if ((st = check_weights(dims, &weights[b], true, true, true, true)) != H3_OK) {
      std::string m = g_err;
      return fail(st, "block %d: %s", b, m.c_str());
    }
  }
  if ((st = check_device()) != H3_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((st = check_tags(*dims, tag, n, s)) != H3_OK) return st;
  const Arena ar = carve(*dims, n, static_cast<char*>(workspace), true);
  char* hist = static_cast<char*>(workspace) + arena;
  float* vel_a[2] = {reinterpret_cast<float*>(hist), reinterpret_cast<float*>(hist + vh.a_bytes)};
  float* vel_v[2] = {reinterpret_cast<float*>(hist + 2 * vh.a_bytes),
                     reinterpret_cast<float*>(hist + 2 * vh.a_bytes + vh.v_bytes)};
  if ((st = hip_ok(do_rope(*dims, positions, n, ar.cs, s), "rope table")) != H3_OK) return st;
  const size_t tstride = (size_t)dims->n_tags * 6 * dims->hidden;
  const size_t fstride = (size_t)4 * dims->hidden;
  const int64_t na = sg.audio * io_dims->audio_patch, nv = sg.video * io_dims->video_patch;
  int fresh_count = 0, j0 = -1, j1 = -1;   // the last two fresh passes (j0 < j1)
  for (int i = 0; i < n_steps; ++i) {
    const bool fresh = i % reuse == 0 || i == n_steps - 1;
    if (fresh) {
      // the new velocities go to the slot not holding the last fresh ones
      const int slot = fresh_count % 2;
      if ((st = run_embed(*dims, *io_dims, *io_weights, sg, text, cond, audio, video, x_packed, s)) != H3_OK)
        return fail(st, "step %d: %s", i, std::string(g_err).c_str());
      const uint16_t* tab = mod_tables + (size_t)i * n_blocks * tstride;
      for (int b = 0; b < n_blocks; ++b) {
        if ((st = run_block(*dims, x_packed, tag, tab + b * tstride, weights[b], n, ar, s)) != H3_OK)
          return fail(st, "step %d block %d: %s", i, b, std::string(g_err).c_str());
      }
      if ((st = run_heads(*dims, *io_dims, *io_weights, sg, x_packed, final_tables + i * fstride,
                          vel_a[slot], vel_v[slot], ar.h, s)) != H3_OK)
        return fail(st, "step %d: %s", i, std::string(g_err).c_str());
      ++fresh_count;
      j0 = j1;
      j1 = i;
    }
    const int cur = (fresh_count - 1) % 2, prev = 1 - cur;
    const double dta = sigmas_audio[i + 1] - sigmas_audio[i];
    const double dtv = sigmas_video[i + 1] - sigmas_video[i];
    if (fresh || j0 < 0) {
      // a fresh velocity, or the only one there is
      if ((st = hip_ok(h3::launch_euler(audio, vel_a[cur], (float)dta, na, s), "euler audio")) != H3_OK) return st;
      if ((st = hip_ok(h3::launch_euler(video, vel_v[cur], (float)dtv, nv, s), "euler video")) != H3_OK) return st;
    } else {
      // extrapolated on each modality's own schedule through (sigma[j0], v0) and (sigma[j1], v1)
      const double ca = (sigmas_audio[i] - sigmas_audio[j1]) / (sigmas_audio[j1] - sigmas_audio[j0]);
      const double cv = (sigmas_video[i] - sigmas_video[j1]) / (sigmas_video[j1] - sigmas_video[j0]);
      if ((st = hip_ok(h3::launch_euler2(audio, vel_a[cur], vel_a[prev], (float)(dta * (1.0 + ca)),
                                         (float)(-dta * ca), na, s), "euler audio")) != H3_OK)
        return st;
      if ((st = hip_ok(h3::launch_euler2(video, vel_v[cur], vel_v[prev], (float)(dtv * (1.0 + cv)),
                                         (float)(-dtv * cv), nv, s), "euler video")) != H3_OK)
        return st;
    }
  }
  return H3_OK;
}

size_t h3_denoise_workspace_size(const h3_dims* dims, const h3_io_dims* io_dims,
                                 const h3_segments* segments) {
  if (check_io(dims, io_dims, segments) != H3_OK) return 0;
  const h3_segments& sg = *segments;
  return full_arena_bytes(*dims, sg.text + sg.cond + sg.audio + sg.video) +
         vel_history(*io_dims, sg).bytes;
}

size_t h3_quantized_bytes(int64_t n_rows, int32_t width, int32_t group) {
  if (n_rows <= 0 || n_rows > kMaxRows || width <= 0 || group <= 0 || width % group != 0) return 0;
  return qa_scale_offset(n_rows, width) + up256((size_t)(width / group) * (size_t)pad_rows(n_rows) * 4);
}

h3_status h3_quantize_groups(const uint16_t* in, int64_t n_rows, int32_t width, int32_t group,
                             void* out, void* stream) {
  g_err.clear();
  h3_status st;
  if ((st = check_rows(n_rows)) != H3_OK) return st;
  if (width <= 0 || width % 8 != 0 || width > 16384)
    return fail(H3_ERR_UNSUPPORTED, "width=%d: need a positive multiple of 8, at most 16384", width);
  if (group != width && group != 64 && group != 256 && group != 448 && group != 896)
    return fail(H3_ERR_UNSUPPORTED, "group=%d: accepted 64, 256, 448, 896, or the width (one per row)", group);
  if (width % group != 0) return fail(H3_ERR_UNSUPPORTED, "group=%d does not divide width=%d", group, width);
  H3_NEED(in, "in");
  H3_NEED(out, "out");
  if ((st = check_device()) != H3_OK) return st;
  char* base = static_cast<char*>(out);
  return hip_ok(do_quant(in, n_rows, width, group, reinterpret_cast<int8_t*>(base),
                         reinterpret_cast<float*>(base + qa_scale_offset(n_rows, width)),
                         reinterpret_cast<hipStream_t>(stream)),
                "quantize groups");
}

size_t h3_workspace_size(const h3_dims* dims, int64_t n_rows) {
  if (check_dims(dims) != H3_OK || check_rows(n_rows) != H3_OK) return 0;
  return full_arena_bytes(*dims, n_rows);
}

const char* h3_last_error(void) { return g_err.c_str(); }

h3_status h3_dit_block_forward(const h3_dims* dims, float* x, const int32_t* tag,
                               const float* positions, const uint16_t* mod_table,
                               const h3_block_weights* weights, int64_t n_rows, void* workspace,
                               size_t workspace_bytes, void* stream) {
  g_err.clear();
  h3_status st;
  if ((st = check_forward_common(dims, x, tag, positions, mod_table, n_rows, workspace,
                                 workspace_bytes)) != H3_OK)
    return st;
  if ((st = check_weights(dims, weights, true, true, true, true)) != H3_OK) return st;
  if ((st = check_device()) != H3_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((st = check_tags(*dims, tag, n_rows, s)) != H3_OK) return st;
  const Arena ar = carve_ws(*dims, n_rows, workspace, workspace_bytes);
  if ((st = hip_ok(do_rope(*dims, positions, n_rows, ar.cs, s), "rope table")) != H3_OK) return st;
  return run_block(*dims, x, tag, mod_table, *weights, n_rows, ar, s);
}

h3_status h3_dit_forward(const h3_dims* dims, float* x, const int32_t* tag, const float* positions,
                         const uint16_t* mod_table, const h3_block_weights* weights,
                         int32_t n_blocks, int64_t n_rows, void* workspace, size_t workspace_bytes,
                         void* stream) {
  g_err.clear();
  h3_status st;
  if ((st = check_forward_common(dims, x, tag, positions, mod_table, n_rows, workspace,
                                 workspace_bytes)) != H3_OK)
    return st;
  if (n_blocks <= 0) return fail(H3_ERR_INVALID_ARG, "n_blocks=%d must be positive", n_blocks);
  if (!weights) return fail(H3_ERR_INVALID_ARG, "weights is NULL");
  for (int b = 0; b < n_blocks; ++b) {
    if ((st = check_weights(dims, &weights[b], true, true, true, true)) != H3_OK) {
      std::string m = g_err;
      return fail(st, "block %d: %s", b, m.c_str());
    }
  }
  if ((st = check_device()) != H3_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((st = check_tags(*dims, tag, n_rows, s)) != H3_OK) return st;
  const Arena ar = carve_ws(*dims, n_rows, workspace, workspace_bytes);
  if ((st = hip_ok(do_rope(*dims, positions, n_rows, ar.cs, s), "rope table")) != H3_OK) return st;
  const size_t tstride = (size_t)dims->n_tags * 6 * dims->hidden;
  for (int b = 0; b < n_blocks; ++b) {
    if ((st = run_block(*dims, x, tag, mod_table + b * tstride, weights[b], n_rows, ar, s)) != H3_OK) {
      std::string m = g_err;
      return fail(st, "block %d: %s", b, m.c_str());
    }
  }
  return H3_OK;
}

h3_status h3_dit_forward_noalloc(const h3_dims* dims, float* x, const int32_t* tag,
                                 const float* positions, const uint16_t* mod_table,
                                 const h3_block_weights* weights, int32_t n_blocks, int64_t n_rows,
                                 void* stream) {
  g_err.clear();
  h3_status st;
  if ((st = check_dims(dims)) != H3_OK || (st = check_rows(n_rows)) != H3_OK) return st;
  const size_t need = carve(*dims, n_rows, nullptr).bytes;
  if (need > H3_NOALLOC_SCRATCH_BYTES)
    return fail(H3_ERR_WORKSPACE,
                "h3_dit_forward_noalloc: %lld rows need a %zu-byte workspace, above the %zu-byte "
                "static scratch array (use h3_dit_forward with a caller workspace)",
                (long long)n_rows, need, (size_t)H3_NOALLOC_SCRATCH_BYTES);
  if ((st = check_device()) != H3_OK) return st;
  void* ws = nullptr;
  if ((st = hip_ok(h3::noalloc_scratch(&ws), "scratch array address")) != H3_OK) return st;
  return h3_dit_forward(dims, x, tag, positions, mod_table, weights, n_blocks, n_rows, ws,
                        H3_NOALLOC_SCRATCH_BYTES, stream);
}

h3_status h3_rope_table(const h3_dims* dims, const float* positions, int64_t n_rows, float* cs,
                        void* stream) {
  g_err.clear();
  h3_status st;
  if ((st = check_dims(dims)) != H3_OK || (st = check_rows(n_rows)) != H3_OK) return st;
  H3_NEED(positions, "positions");
  H3_NEED(cs, "cs");
  if ((st = check_device()) != H3_OK) return st;
  return hip_ok(do_rope(*dims, positions, n_rows, cs, reinterpret_cast<hipStream_t>(stream)),
                "rope table");
}

h3_status h3_adaln_modulate(const h3_dims* dims, const float* x, const int32_t* tag,
                            const uint16_t* mod_table, int32_t which, int64_t n_rows, uint16_t* h,
                            void* stream) {
  g_err.clear();
  h3_status st;
  if ((st = check_dims(dims)) != H3_OK || (st = check_rows(n_rows)) != H3_OK) return st;
  H3_NEED(x, "x");
  H3_NEED(tag, "modality_tag");
  H3_NEED(mod_table, "mod_table");
  H3_NEED(h, "h");
  if (which != 0 && which != 1) return fail(H3_ERR_INVALID_ARG, "which=%d must be 0 or 1", which);
  if ((st = check_device()) != H3_OK) return st;
  if ((st = check_tags(*dims, tag, n_rows, reinterpret_cast<hipStream_t>(stream))) != H3_OK) return st;
  return hip_ok(do_adaln(*dims, x, tag, mod_table, which, n_rows, h,
                         reinterpret_cast<hipStream_t>(stream)),
                "adaln");
}

h3_status h3_qkv_rope(const h3_dims* dims, const uint16_t* h, const h3_block_weights* weights,
                      const float* cs, int64_t n_rows, uint16_t* q, uint16_t* k, uint16_t* vt,
                      void* stream) {
  g_err.clear();
  h3_status st;
  if ((st = check_dims(dims)) != H3_OK || (st = check_rows(n_rows)) != H3_OK) return st;
  if ((st = check_weights(dims, weights, true, false, false, false)) != H3_OK) return st;
  H3_NEED(h, "h");
  H3_NEED(cs, "cs");
  H3_NEED(q, "q");
  H3_NEED(k, "k");
  H3_NEED(vt, "vt");
  if ((st = check_device()) != H3_OK) return st;
  return hip_ok(do_qkv(*dims, h, *weights, cs, n_rows, q, k, vt, reinterpret_cast<hipStream_t>(stream),
                       act_scales(*dims, h, n_rows, dims->hidden)),
                "qkv+rope");
}

h3_status h3_attention(const h3_dims* dims, const uint16_t* q, const uint16_t* k,
                       const uint16_t* vt, int64_t n_rows, uint16_t* o, void* stream) {
  g_err.clear();
  h3_status st;
  if ((st = check_dims(dims)) != H3_OK || (st = check_rows(n_rows)) != H3_OK) return st;
  H3_NEED(q, "q");
  H3_NEED(k, "k");
  H3_NEED(vt, "vt");
  H3_NEED(o, "o");
  if ((st = check_device()) != H3_OK) return st;
  return hip_ok(do_attn(*dims, q, k, vt, n_rows, o, reinterpret_cast<hipStream_t>(stream)),
                "attention");
}

h3_status h3_out_proj_residual(const h3_dims* dims, const uint16_t* o,
                               const h3_block_weights* weights, const uint16_t* mod_table,
                               const int32_t* tag, int64_t n_rows, float* x, void* stream) {
  g_err.clear();
  h3_status st;
  if ((st = check_dims(dims)) != H3_OK || (st = check_rows(n_rows)) != H3_OK) return st;
  if ((st = check_weights(dims, weights, false, true, false, false)) != H3_OK) return st;
  H3_NEED(o, "o");
  H3_NEED(mod_table, "mod_table");
  H3_NEED(tag, "modality_tag");
  H3_NEED(x, "x");
  if ((st = check_device()) != H3_OK) return st;
  if ((st = check_tags(*dims, tag, n_rows, reinterpret_cast<hipStream_t>(stream))) != H3_OK) return st;
  return hip_ok(do_resid(*dims, o, weights->w_out, weights->s_out, weights->b_out,
                         dims->heads * dims->head_dim, mod_table, 2, tag, n_rows, x,
                         reinterpret_cast<hipStream_t>(stream),
                         act_scales(*dims, o, n_rows, dims->heads * dims->head_dim)),
                "out-proj+gate");
}

h3_status h3_mlp_fc1_swiglu(const h3_dims* dims, const uint16_t* h2, const h3_block_weights* weights,
                            int64_t n_rows, uint16_t* a, void* stream) {
  g_err.clear();
  h3_status st;
  if ((st = check_dims(dims)) != H3_OK || (st = check_rows(n_rows)) != H3_OK) return st;
  if ((st = check_weights(dims, weights, false, false, true, false)) != H3_OK) return st;
  H3_NEED(h2, "h2");
  H3_NEED(a, "a");
  if ((st = check_device()) != H3_OK) return st;
  return hip_ok(do_fc1(*dims, h2, *weights, n_rows, a, reinterpret_cast<hipStream_t>(stream),
                       act_scales(*dims, h2, n_rows, dims->hidden)),
                "fc1+swiglu");
}

h3_status h3_mlp_fc2_residual(const h3_dims* dims, const uint16_t* a,
                              const h3_block_weights* weights, const uint16_t* mod_table,
                              const int32_t* tag, int64_t n_rows, float* x, void* stream) {
  g_err.clear();
  h3_status st;
  if ((st = check_dims(dims)) != H3_OK || (st = check_rows(n_rows)) != H3_OK) return st;
  if ((st = check_weights(dims, weights, false, false, false, true)) != H3_OK) return st;
  H3_NEED(a, "a");
  H3_NEED(mod_table, "mod_table");
  H3_NEED(tag, "modality_tag");
  H3_NEED(x, "x");
  if ((st = check_device()) != H3_OK) return st;
  if ((st = check_tags(*dims, tag, n_rows, reinterpret_cast<hipStream_t>(stream))) != H3_OK) return st;
  return hip_ok(do_resid(*dims, a, weights->w_fc2, weights->s_fc2, weights->b_fc2, dims->ffn,
                         mod_table, 5, tag, n_rows, x, reinterpret_cast<hipStream_t>(stream),
                         act_scales(*dims, a, n_rows, dims->ffn)),
                "fc2+gate");
}

size_t h3_heads_workspace_size(const h3_dims* dims, const h3_segments* segments) {
  if (check_dims(dims) != H3_OK) return 0;
  if (!segments || segments->audio < 0 || segments->video < 0) {
    fail(H3_ERR_INVALID_ARG, "segments is NULL or negative");
    return 0;
  }
  const size_t b = heads_ws_bytes(*dims, *segments);
  return b ? b : 256;
}

h3_status h3_embed_inputs(const h3_dims* dims, const h3_io_dims* io_dims,
                          const h3_io_weights* io_weights, const h3_segments* segments,
                          const uint16_t* text, const float* cond, const float* audio,
                          const float* video, float* x_packed, void* stream) {
  g_err.clear();
  h3_status st;
  if ((st = check_io(dims, io_dims, segments)) != H3_OK) return st;
  if ((st = check_embed_ptrs(*segments, io_weights, text, cond, audio, video, x_packed)) != H3_OK)
    return st;
  if ((st = check_device()) != H3_OK) return st;
  return run_embed(*dims, *io_dims, *io_weights, *segments, text, cond, audio, video, x_packed,
                   reinterpret_cast<hipStream_t>(stream));
}

h3_status h3_final_heads(const h3_dims* dims, const h3_io_dims* io_dims,
                         const h3_io_weights* io_weights, const h3_segments* segments,
                         const float* x_packed, const uint16_t* final_table, float* vel_audio,
                         float* vel_video, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  h3_status st;
  if ((st = check_io(dims, io_dims, segments)) != H3_OK) return st;
  if ((st = check_head_ptrs(*segments, io_weights, x_packed, final_table, vel_audio, vel_video)) != H3_OK)
    return st;
  H3_NEED(workspace, "workspace");
  const size_t need = heads_ws_bytes(*dims, *segments);
  if (workspace_bytes < need)
    return fail(H3_ERR_WORKSPACE, "workspace is %zu bytes, %zu needed", workspace_bytes, need);
  if ((st = check_device()) != H3_OK) return st;
  return run_heads(*dims, *io_dims, *io_weights, *segments, x_packed, final_table, vel_audio,
                   vel_video, static_cast<uint16_t*>(workspace), reinterpret_cast<hipStream_t>(stream));
}

h3_status h3_velocity_forward(const h3_dims* dims, const h3_io_dims* io_dims,
                              const h3_io_weights* io_weights, const h3_segments* segments,
                              const uint16_t* text, const float* cond, const float* audio,
                              const float* video, const int32_t* tag, const float* positions,
                              const uint16_t* mod_table, const h3_block_weights* weights,
                              int32_t n_blocks, const uint16_t* final_table, float* x_packed,
                              float* vel_audio, float* vel_video, void* workspace,
                              size_t workspace_bytes, void* stream) {
  g_err.clear();
  h3_status st;
  if ((st = check_io(dims, io_dims, segments)) != H3_OK) return st;
  const h3_segments sg = *segments;
  const int64_t n = sg.text + sg.cond + sg.audio + sg.video;
  if ((st = check_embed_ptrs(sg, io_weights, text, cond, audio, video, x_packed)) != H3_OK) return st;
  if ((st = check_head_ptrs(sg, io_weights, x_packed, final_table, vel_audio, vel_video)) != H3_OK)
    return st;
  if (n_blocks < 0) return fail(H3_ERR_INVALID_ARG, "n_blocks=%d must be >= 0", n_blocks);
  if (n_blocks > 0) {
    if ((st = check_forward_common(dims, x_packed, tag, positions, mod_table, n, workspace,
                                   workspace_bytes)) != H3_OK)
      return st;
    if (!weights) return fail(H3_ERR_INVALID_ARG, "weights is NULL");
    for (int b = 0; b < n_blocks; ++b) {
      if ((st = check_weights(dims, &weights[b], true, true, true, true)) != H3_OK) {
        std::string m = g_err;
        return fail(st, "block %d: %s", b, m.c_str());
      }
    }
  } else {
    H3_NEED(workspace, "workspace");
    const size_t need = heads_ws_bytes(*dims, sg);
    if (workspace_bytes < need)
      return fail(H3_ERR_WORKSPACE, "workspace is %zu bytes, %zu needed", workspace_bytes, need);
  }
  if ((st = check_device()) != H3_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // the tags are read only by the blocks (tag may be NULL when none runs)
  if (n_blocks > 0 && (st = check_tags(*dims, tag, n, s)) != H3_OK) return st;
  if ((st = run_embed(*dims, *io_dims, *io_weights, sg, text, cond, audio, video, x_packed, s)) != H3_OK)
    return st;
  uint16_t* h = static_cast<uint16_t*>(workspace);
  if (n_blocks > 0) {
    const Arena ar = carve_ws(*dims, n, workspace, workspace_bytes);
    if ((st = hip_ok(do_rope(*dims, positions, n, ar.cs, s), "rope table")) != H3_OK) return st;
    const size_t tstride = (size_t)dims->n_tags * 6 * dims->hidden;
    for (int b = 0; b < n_blocks; ++b) {
      if ((st = run_block(*dims, x_packed, tag, mod_table + b * tstride, weights[b], n, ar, s)) != H3_OK) {
        std::string m = g_err;
        return fail(st, "block %d: %s", b, m.c_str());
      }
    }
    h = ar.h;   // dead after the last block; holds max(audio, video) rows
  }
  return run_heads(*dims, *io_dims, *io_weights, sg, x_packed, final_table, vel_audio, vel_video, h, s);
}

}  // extern "C"
