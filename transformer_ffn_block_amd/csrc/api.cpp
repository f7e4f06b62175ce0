// C ABI of libffn (declared in include/ffn.h): argument validation, schedule
// selection and kernel launches on the caller's stream.  No device memory is
// allocated here, nothing synchronises (except ffn_timing_collect), nothing
// prints.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/ffn.h"
#include "launch.h"

namespace {

thread_local std::string g_err;

ffn_status fail(ffn_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

ffn_status ok() {
  g_err.clear();
  return FFN_OK;
}

// ---- per-kernel timing ---------------------------------------------------
// Timing state belongs to the calling thread: only kernels enqueued by the
// thread that enabled timing are timed, and the totals are that thread's.
// Each dispatch gets its own event pair, bound to the kernel by
// hipExtLaunchKernel (ffn::dispatch_events); a launcher's first kernel is
// named after the launch site, its later ones "<name>/2", "<name>/3".
// Events are created on first use (so enabling touches no device) and
// destroyed when the thread disables timing.  No HIP call is made from a
// thread-exit destructor: a thread that ends with timing still enabled
// leaks its events.
struct Timing {
  bool on = false;
  int cap = 0;
  int used = 0;
  const char* site = nullptr;  // launch site being issued (set by timed())
  int sub = 0;                 // dispatches issued so far by that site
  std::vector<hipEvent_t> ev;  // 2 per dispatch slot, created on demand
  std::vector<std::string> name;
  std::map<std::string, std::pair<int64_t, double>> total;
  std::vector<std::string> order;
};
thread_local Timing t_timing;

template <class F>
hipError_t timed(const char* name, hipStream_t s, F&& f) {
  (void)s;
  Timing& T = t_timing;
  if (!T.on) return f();
  T.site = name;
  T.sub = 0;
  const hipError_t e = f();
  T.site = nullptr;
  return e;
}

void release_events() {
  Timing& T = t_timing;
  for (hipEvent_t e : T.ev)
    if (e) (void)hipEventDestroy(e);
  T.ev.clear();
  T.name.clear();
  T.cap = T.used = 0;
}

// ---- validation helpers ----------------------------------------------------
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

constexpr int64_t kMaxChunks = 0x7FFFFFFF;  // 16-byte chunks addressable with int32 offsets

size_t elem_size(ffn_dtype dt) { return dt == FFN_BF16 ? 2 : 4; }

ffn_status check_dtype(ffn_dtype dt) {
  if (dt != FFN_F32 && dt != FFN_BF16)
    return fail(FFN_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dt);
  return FFN_OK;
}

ffn_status check_eps(float eps) {
  if (!(eps >= 0.f) || !std::isfinite(eps))
    return fail(FFN_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  return FFN_OK;
}

// sizes shared by the dense and Q8 blocks
ffn_status check_block_dims(int64_t M, int64_t d, int64_t f, int64_t mult) {
  if (M < 0 || d <= 0 || f <= 0)
    return fail(FFN_ERR_INVALID_ARGUMENT, "need M >= 0, d > 0, f > 0 (got %lld, %lld, %lld)",
                (long long)M, (long long)d, (long long)f);
  if (d % mult || f % mult)
    return fail(FFN_ERR_UNSUPPORTED, "d and f must be multiples of %lld (got %lld, %lld)",
                (long long)mult, (long long)d, (long long)f);
  if (M > 0x7FFFFFFF || d > 0x7FFFFFFF || f > 0x7FFFFFFF)
    return fail(FFN_ERR_UNSUPPORTED, "dimension exceeds 2^31-1");
  const int64_t mx = M > f ? M : f;
  if (mx * (d / 8) > kMaxChunks || (M > d ? M : d) * (f / 8) > kMaxChunks)
    return fail(FFN_ERR_UNSUPPORTED, "tensor too large for 32-bit chunk offsets");
  return FFN_OK;
}

struct WsLayout {
  size_t n = 0, h = 0, G = 0, U = 0, part = 0, ctr = 0, total = 0;
};

// The decode regime (bf16, fused schedule, M <= decode_max_tokens()) keeps h
// in the decode kernels' blocked layout: whole 16-token tiles of ceil(f/128)
// 128-k stages each.
bool decode_regime(size_t es, int64_t M, bool split, bool persistent) {
  return es == 2 && !split && !persistent && M <= ffn::decode_max_tokens();
}
size_t decode_h_row_elems(int64_t f) {  // elements per token of blocked h
  return ffn::decode_h_blocked() ? (size_t)((f + 127) / 128) * 128 : (size_t)f;
}

// Split-K plans of the prefill GEMMs (bf16, more than decode_max_tokens()
// tokens): columns [0, main) unsplit, the rest over z K ranges.  The gate/up
// plan applies to the fused GEMM (not SPLIT, not the register-staged
// FUSED_NORM kernel, which never splits).
struct PrefillSplits {
  ffn::PrefillPlan gu, dn;
};
PrefillSplits prefill_splits(size_t es, int64_t M, int64_t d, int64_t f, bool split, bool persistent) {
  PrefillSplits p;
  p.gu.main = (int)std::min<int64_t>(f, INT32_MAX);
  p.dn.main = (int)std::min<int64_t>(d, INT32_MAX);
  if (es != 2 || persistent || M <= ffn::decode_max_tokens() || M > INT32_MAX || d > INT32_MAX ||
      f > INT32_MAX)
    return p;
  if (!split) p.gu = ffn::prefill_gateup_plan((int)M, (int)d, (int)f);
  p.dn = ffn::prefill_down_plan((int)M, (int)d, (int)f);
  return p;
}

WsLayout ws_layout(size_t es, int64_t M, int64_t d, int64_t f, bool split, bool persistent = false) {
  WsLayout w;
  size_t at = 0;
  w.n = at;
  at += round256((size_t)M * d * es);
  w.h = at;
  if (decode_regime(es, M, split, persistent) && ffn::decode_h_blocked())
    at += round256((size_t)((M + 15) / 16) * 16 * decode_h_row_elems(f) * es);
  else
    at += round256((size_t)M * f * es);
  if (split) {
    w.G = at;
    at += round256((size_t)M * f * es);
    w.U = at;
    at += round256((size_t)M * f * es);
  }
  if (persistent) {
    const int sp = ffn::decode_persistent_splits((int)d, (int)f);
    w.part = at;
    at += round256((size_t)sp * M * d * 4);
    w.ctr = at;
    at += round256(ffn::decode_persistent_counters((int)d, sp) * 4);
  }
  // fp32 partial sums of split-K prefill GEMMs (gate/up planes, then reused
  // for the down projection's)
  const PrefillSplits ps = prefill_splits(es, M, d, f, split, persistent);
  const size_t pgu = ps.gu.z > 1 ? (size_t)2 * ps.gu.z * M * (f - ps.gu.main) * 4 : 0;
  const size_t pdn = ps.dn.z > 1 ? (size_t)ps.dn.z * M * (d - ps.dn.main) * 4 : 0;
  if (pgu || pdn) {
    w.part = at;
    at += round256(pgu > pdn ? pgu : pdn);
  }
  w.total = at;
  return w;
}

#define FFN_TRY(expr)                 \
  do {                                \
    ffn_status st_ = (expr);          \
    if (st_ != FFN_OK) return st_;    \
  } while (0)

#define FFN_LAUNCH(name, s, call)                                                          \
  do {                                                                                     \
    hipError_t e_ = timed(name, s, [&] { return (call); });                               \
    if (e_ != hipSuccess)                                                                  \
      return fail(FFN_ERR_LAUNCH, "%s: %s", name, hipGetErrorString(e_));                  \
  } while (0)

bool use_split(ffn_variant v) { return v == FFN_VARIANT_SPLIT; }
bool use_persistent(ffn_variant v) { return v == FFN_VARIANT_PERSISTENT; }

}  // namespace

extern "C" {

const char* ffn_status_string(ffn_status s) {
  switch (s) {
    case FFN_OK: return "FFN_OK";
    case FFN_ERR_INVALID_ARGUMENT: return "FFN_ERR_INVALID_ARGUMENT";
    case FFN_ERR_UNSUPPORTED: return "FFN_ERR_UNSUPPORTED";
    case FFN_ERR_WORKSPACE: return "FFN_ERR_WORKSPACE";
    case FFN_ERR_LAUNCH: return "FFN_ERR_LAUNCH";
  }
  return "FFN_ERR_UNKNOWN";
}

const char* ffn_last_error(void) { return g_err.c_str(); }

// ---------------------------------------------------------------------------
ffn_status ffn_rmsnorm(ffn_dtype dt, const void* x, const void* g, void* y, int64_t rows,
                       int64_t d, float eps, void* stream) {
  FFN_TRY(check_dtype(dt));
  if (!x || !g || !y) return fail(FFN_ERR_INVALID_ARGUMENT, "null pointer");
  if (rows < 0 || d <= 0)
    return fail(FFN_ERR_INVALID_ARGUMENT, "need rows >= 0 and d > 0");
  FFN_TRY(check_eps(eps));
  const size_t es = elem_size(dt);
  const int64_t mult = 16 / (int64_t)es;
  if (d % mult) return fail(FFN_ERR_UNSUPPORTED, "d must be a multiple of %lld", (long long)mult);
  if (d / mult > kMaxChunks || rows > 0x7FFFFFFFLL)
    return fail(FFN_ERR_UNSUPPORTED, "too large");
  if (!aligned(x, 16) || !aligned(g, 16) || !aligned(y, 16))
    return fail(FFN_ERR_UNSUPPORTED, "x, g and y must be 16-byte aligned");
  const size_t nb = (size_t)rows * d * es;
  if (overlap(y, nb, x, nb) || overlap(y, nb, g, (size_t)d * es))
    return fail(FFN_ERR_INVALID_ARGUMENT, "y overlaps an input");
  if (rows == 0) return ok();
  hipStream_t s = (hipStream_t)stream;
  FFN_LAUNCH("rmsnorm", s, ffn::launch_rmsnorm((int)es, x, g, y, rows, d, eps, s));
  return ok();
}

size_t ffn_swiglu_block_workspace_size(ffn_dtype dt, int64_t M, int64_t d, int64_t f,
                                       ffn_variant variant) {
  if (dt != FFN_F32 && dt != FFN_BF16) return 0;
  if (M < 0 || d <= 0 || f <= 0) return 0;
  if (variant != FFN_VARIANT_AUTO && variant != FFN_VARIANT_FUSED && variant != FFN_VARIANT_SPLIT &&
      variant != FFN_VARIANT_PERSISTENT && variant != FFN_VARIANT_FUSED_NORM)
    return 0;
  if (use_persistent(variant) && (dt != FFN_BF16 || M > 16 || d > INT32_MAX || f > INT32_MAX))
    return 0;
  return ws_layout(elem_size(dt), M, d, f, use_split(variant), use_persistent(variant)).total;
}

size_t ffn_swiglu_block_persistent_status_offset(int64_t M, int64_t d, int64_t f) {
  if (M < 1 || M > 16 || d <= 0 || f <= 0 || d > INT32_MAX || f > INT32_MAX) return 0;
  return ws_layout(2, M, d, f, false, true).ctr + 4;
}

}  // extern "C"

namespace {

// Every check of a block call that does not involve the workspace.
ffn_status check_block_args(ffn_dtype dt, const void* x, const void* g, const void* w_gate,
                            const void* w_up, const void* w_down, const void* y, int64_t M,
                            int64_t d, int64_t f, float eps, ffn_variant variant) {
  FFN_TRY(check_dtype(dt));
  if (!x || !g || !w_gate || !w_up || !w_down || !y)
    return fail(FFN_ERR_INVALID_ARGUMENT, "null pointer");
  if (variant != FFN_VARIANT_AUTO && variant != FFN_VARIANT_FUSED && variant != FFN_VARIANT_SPLIT &&
      variant != FFN_VARIANT_PERSISTENT && variant != FFN_VARIANT_FUSED_NORM)
    return fail(FFN_ERR_INVALID_ARGUMENT, "unknown variant %d", (int)variant);
  FFN_TRY(check_eps(eps));
  const size_t es = elem_size(dt);
  FFN_TRY(check_block_dims(M, d, f, 16 / (int64_t)es));
  if (use_persistent(variant) && (dt != FFN_BF16 || M > 16))
    return fail(FFN_ERR_UNSUPPORTED, "the persistent schedule takes bf16 and at most 16 tokens");
  if (!aligned(x, 16) || !aligned(g, 16) || !aligned(w_gate, 16) || !aligned(w_up, 16) ||
      !aligned(w_down, 16) || !aligned(y, 16))
    return fail(FFN_ERR_UNSUPPORTED, "tensors must be 16-byte aligned");
  if ((size_t)f * d * es >= ((size_t)1 << 31))
    return fail(FFN_ERR_UNSUPPORTED, "weight matrices must be smaller than 2 GiB");
  const size_t ny = (size_t)M * d * es, nw = (size_t)f * d * es;
  if (overlap(y, ny, x, ny) || overlap(y, ny, g, (size_t)d * es) || overlap(y, ny, w_gate, nw) ||
      overlap(y, ny, w_up, nw) || overlap(y, ny, w_down, nw))
    return fail(FFN_ERR_INVALID_ARGUMENT, "y overlaps an input or the workspace");
  return FFN_OK;
}

}  // namespace

extern "C" {

ffn_status ffn_swiglu_block(ffn_dtype dt, const void* x, const void* g, const void* w_gate,
                            const void* w_up, const void* w_down, void* y, int64_t M, int64_t d,
                            int64_t f, float eps, ffn_variant variant, void* workspace,
                            size_t workspace_bytes, void* stream) {
  FFN_TRY(check_block_args(dt, x, g, w_gate, w_up, w_down, y, M, d, f, eps, variant));
  const size_t es = elem_size(dt);
  const bool persistent = use_persistent(variant);
  const bool split = use_split(variant);
  const WsLayout L = ws_layout(es, M, d, f, split, persistent);
  if (M > 0 && (!workspace || workspace_bytes < L.total))
    return fail(FFN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total,
                workspace ? workspace_bytes : (size_t)0);
  if (workspace && !aligned(workspace, 256))
    return fail(FFN_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  const size_t ny = (size_t)M * d * es;
  if (overlap(y, ny, workspace, workspace ? L.total : 0))
    return fail(FFN_ERR_INVALID_ARGUMENT, "y overlaps an input or the workspace");
  if (M == 0) return ok();

  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  void* n = ws + L.n;
  void* h = ws + L.h;
  float* part = (float*)(ws + L.part);
  const PrefillSplits sp = prefill_splits(es, M, d, f, split, persistent);
  const int Mi = (int)M, di = (int)d, fi = (int)f;

  if (persistent) {
    FFN_LAUNCH("decode_persistent", s,
               ffn::launch_decode_persistent(x, g, w_gate, w_up, w_down, h, (float*)(ws + L.part),
                                             (unsigned*)(ws + L.ctr), y, Mi, di, fi, eps, s));
    return ok();
  }
  const bool decode = decode_regime(es, M, split, false);
  // prefill with the norm folded into the fused gate/up GEMM
  const bool fold_prefill = dt == FFN_BF16 && variant == FFN_VARIANT_FUSED_NORM && !decode;
  if (!decode && !fold_prefill) FFN_LAUNCH("rmsnorm", s, ffn::launch_rmsnorm((int)es, x, g, n, M, d, eps, s));
  if (dt == FFN_F32) {
    const float* nf = (const float*)n;
    float* hf = (float*)h;
    if (split) {
      float* G = (float*)(ws + L.G);
      float* U = (float*)(ws + L.U);
      FFN_LAUNCH("f32_gemm_gate", s, ffn::launch_gemm_f32(ffn::F32_STORE, nf, (const float*)w_gate, nullptr, nullptr, G, Mi, fi, di, s));
      FFN_LAUNCH("f32_gemm_up", s, ffn::launch_gemm_f32(ffn::F32_STORE, nf, (const float*)w_up, nullptr, nullptr, U, Mi, fi, di, s));
      FFN_LAUNCH("f32_swiglu", s, ffn::launch_swiglu_f32(G, U, hf, (int64_t)M * f, s));
    } else {
      FFN_LAUNCH("f32_gemm_gateup_fused", s, ffn::launch_gemm_f32(ffn::F32_SWIGLU, nf, (const float*)w_gate, (const float*)w_up, nullptr, hf, Mi, fi, di, s));
    }
    FFN_LAUNCH("f32_gemm_down_residual", s, ffn::launch_gemm_f32(ffn::F32_RESIDUAL, hf, (const float*)w_down, nullptr, (const float*)x, (float*)y, Mi, di, fi, s));
    return ok();
  }

  if (split) {
    void* G = ws + L.G;
    void* U = ws + L.U;
    FFN_LAUNCH("gemm_gate", s, ffn::launch_gemm_store(n, w_gate, G, Mi, fi, di, s));
    FFN_LAUNCH("gemm_up", s, ffn::launch_gemm_store(n, w_up, U, Mi, fi, di, s));
    FFN_LAUNCH("swiglu", s, ffn::launch_swiglu_bf16(G, U, h, (int64_t)M * f, s));
  } else if (fold_prefill) {
    FFN_LAUNCH("gemm_gateup_fused_norm", s,
               ffn::launch_gemm_gateup_fused_norm(x, g, w_gate, w_up, h, Mi, di, fi, eps, s));
  } else if (!decode) {
    // columns [0, c) unsplit, [c, f) split over K (row stride f throughout)
    const int c = sp.gu.main;
    if (c > 0)
      FFN_LAUNCH("gemm_gateup_fused", s,
                 ffn::launch_gemm_gateup_fused(n, w_gate, w_up, h, Mi, di, c, s, fi));
    if (sp.gu.z > 1) {
      const size_t wo = (size_t)c * d * 2;
      char* hc = (char*)h + (size_t)c * 2;
      FFN_LAUNCH("gemm_gateup_fused_splitk", s,
                 ffn::launch_gemm_gateup_fused_part(n, (const char*)w_gate + wo, (const char*)w_up + wo,
                                                    part, sp.gu.z, Mi, di, fi - c, s));
      FFN_LAUNCH("splitk_swiglu", s, ffn::launch_splitk_swiglu(part, sp.gu.z, hc, Mi, fi - c, s, fi));
    }
  }
  if (Mi > ffn::decode_max_tokens()) {
    const int c = sp.dn.main;
    if (c > 0)
      FFN_LAUNCH("gemm_down_residual", s, ffn::launch_gemm_residual(h, w_down, x, y, Mi, c, fi, s, di));
    if (sp.dn.z > 1) {
      const size_t co = (size_t)c * 2;
      FFN_LAUNCH("gemm_down_splitk", s,
                 ffn::launch_gemm_down_part(h, (const char*)w_down + (size_t)c * f * 2, part, sp.dn.z,
                                            Mi, di - c, fi, s));
      FFN_LAUNCH("splitk_residual", s,
                 ffn::launch_splitk_residual(part, sp.dn.z, (const char*)x + co, (char*)y + co, Mi,
                                             di - c, s, di));
    }
    return ok();
  }
  // decode regime: gate/up launches of at most decode_gateup_tokens() tokens
  // with h blocked, decode_chunk_tokens() otherwise (the norm is folded in,
  // so n is never materialised; every chunk but the last is a whole number
  // of 16-token tiles).  With h blocked, one down launch takes every token
  // (it reads h straight into registers, so up to four token tiles fit).
  // Row-major h (SPLIT) is read in chunks like the gate/up side.
  const bool hblk = decode && ffn::decode_h_blocked();
  const int step = hblk ? ffn::decode_gateup_tokens() : ffn::decode_chunk_tokens();
  for (int m0 = 0; m0 < Mi; m0 += step) {
    const int mc = Mi - m0 < step ? Mi - m0 : step;
    const char* xc = (const char*)x + (size_t)m0 * d * es;
    char* hc = (char*)h + (size_t)m0 * (hblk ? decode_h_row_elems(f) : (size_t)f) * es;
    if (decode)
      FFN_LAUNCH("decode_gateup", s, ffn::launch_decode_gateup_norm(xc, g, w_gate, w_up, hc, mc, di, fi, eps, s));
    if (!hblk)
      FFN_LAUNCH("decode_down", s, ffn::launch_decode_down(hc, w_down, xc, (char*)y + (size_t)m0 * d * es, mc, di, fi, false, s));
  }
  if (hblk) FFN_LAUNCH("decode_down", s, ffn::launch_decode_down(h, w_down, x, y, Mi, di, fi, true, s));
  return ok();
}

}  // extern "C"

namespace {

// Q8_0 and Q4_0 blocks share validation and the launch sequence; the traits
// give the storage of one matrix and its kernels, and whether the gate/up
// kernel folds the norm in (then n is never materialised).
#ifndef FFN_Q8_FOLD
#define FFN_Q8_FOLD 1
#endif
#ifndef FFN_Q4_FOLD
#define FFN_Q4_FOLD 1
#endif
#ifndef FFN_Q4_FOLD_MAX
#define FFN_Q4_FOLD_MAX 10240
#endif
struct Q8Traits {
  using Mat = ffn_q8_matrix;
  static constexpr const char* name = "Q8";
  static constexpr int64_t k_multiple = 32;
  static constexpr const char* gateup_name = "q8_gateup";
  static constexpr const char* down_name = "q8_down";
  static size_t quant_bytes(size_t weights) { return weights; }
  static int max_tokens() { return ffn::q8_max_tokens(); }
  // fp32 partial sums of the split-K down projection for Mc tokens
  static size_t part_bytes(int64_t Mc, int64_t d, int64_t f) {
    const int sp = ffn::q8_down_splits((int)Mc, (int)d, (int)f);
    return sp > 1 ? (size_t)sp * (size_t)Mc * (size_t)d * 4 : 0;
  }
  // The norm folds into the gate/up kernel for every call of up to 8
  // tokens: the fold removes the norm launch (~5 us) and the n round trip.
  // Measured with the deeper quantised pipeline: block 26.4 -> 23.8 us at
  // f = 2176 and 74.2 -> 72.8 us at f = 17408 (8 tokens); at 16 and 32
  // tokens the folded kernel was slower, so those calls keep the norm kernel.
  static bool fold(int64_t M, int64_t d, int64_t f) {
    (void)d;
    (void)f;
    return FFN_Q8_FOLD != 0 && M <= 8;
  }
  static hipError_t gateup(const void* act, const void* gain, float eps, const Mat* g, const Mat* u,
                           void* h, int M, int d, int f, hipStream_t s) {
    return ffn::launch_q8_gateup(act, gain, eps, g->qs, g->scales, u->qs, u->scales, h, M, d, f, s);
  }
  static hipError_t down(const void* h, const Mat* w, const void* x, void* y, float* part, int M,
                         int d, int f, hipStream_t s) {
    return ffn::launch_q8_down(h, w->qs, w->scales, x, y, part, M, d, f, s);
  }
};
struct Q4Traits {
  using Mat = ffn_q4_matrix;
  static constexpr const char* name = "Q4";
  static constexpr int64_t k_multiple = 32;
  static constexpr const char* gateup_name = "q4_gateup";
  static constexpr const char* down_name = "q4_down";
  static size_t quant_bytes(size_t weights) { return weights / 2; }
  static int max_tokens() { return ffn::q4_max_tokens(); }
  // fp32 partial sums of the split-K down projection for Mc tokens
  static size_t part_bytes(int64_t Mc, int64_t d, int64_t f) {
    const int sp = ffn::q4_down_splits((int)Mc, (int)d, (int)f);
    return sp > 1 ? (size_t)sp * (size_t)Mc * (size_t)d * 4 : 0;
  }
  // the same bound as Q8_0 (measured: block 23.5 -> 21.0 us at f = 2176,
  // 55.5 -> 58.1 us if folded at f = 17408)
  static bool fold(int64_t M, int64_t d, int64_t f) {
    return FFN_Q4_FOLD != 0 && M <= 8 && ((f + 15) / 16) * ((d + 255) / 256) <= FFN_Q4_FOLD_MAX;
  }
  static hipError_t gateup(const void* act, const void* gain, float eps, const Mat* g, const Mat* u,
                           void* h, int M, int d, int f, hipStream_t s) {
    return ffn::launch_q4_gateup(act, gain, eps, g->qs, g->scales, u->qs, u->scales, h, M, d, f, s);
  }
  static hipError_t down(const void* h, const Mat* w, const void* x, void* y, float* part, int M,
                         int d, int f, hipStream_t s) {
    return ffn::launch_q4_down(h, w->qs, w->scales, x, y, part, M, d, f, s);
  }
};

// The quantised blocks stream every weight once per launch of at most
// T::max_tokens() tokens, so their cost grows with M in steps of whole
// weight passes; they take the weight-streaming regime only (two launches
// at most), and larger token counts are rejected.
constexpr int64_t kQuantMaxTokens = 64;

// Workspace of a quantised block: n [M,d] (unless the norm is folded) and
// h [M,f] in bf16, then the down projection's split-K partials for one
// chunk of tokens.
struct QuantWs {
  size_t n = 0, h = 0, part = 0, total = 0;
};
template <class T>
static QuantWs quant_ws(int64_t M, int64_t d, int64_t f) {
  QuantWs w;
  size_t at = 0;
  if (!T::fold(M, d, f)) {
    w.n = at;
    at += round256((size_t)M * d * 2);
  }
  w.h = at;
  at += round256((size_t)M * f * 2);
  const int64_t mc = M < T::max_tokens() ? M : T::max_tokens();
  w.part = at;
  at += round256(T::part_bytes(mc, d, f));
  w.total = at;
  return w;
}

template <class T>
static ffn_status quant_block(const void* x, const void* g, const typename T::Mat* w_gate,
                              const typename T::Mat* w_up, const typename T::Mat* w_down, void* y,
                              int64_t M, int64_t d, int64_t f, float eps, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!x || !g || !y || !w_gate || !w_up || !w_down)
    return fail(FFN_ERR_INVALID_ARGUMENT, "null pointer");
  const typename T::Mat* mats[3] = {w_gate, w_up, w_down};
  for (const typename T::Mat* m : mats) {
    if (!m->qs || !m->scales) return fail(FFN_ERR_INVALID_ARGUMENT, "null %s matrix pointer", T::name);
    if (!aligned(m->qs, 16) || !aligned(m->scales, 2))
      return fail(FFN_ERR_UNSUPPORTED, "%s quants must be 16-byte aligned, scales 2-byte", T::name);
  }
  FFN_TRY(check_eps(eps));
  FFN_TRY(check_block_dims(M, d, f, T::k_multiple));
  if (M > kQuantMaxTokens)
    return fail(FFN_ERR_UNSUPPORTED,
                "%s block takes at most %d tokens (weight-streaming regime; got %lld)", T::name,
                kQuantMaxTokens, (long long)M);
  if (T::quant_bytes((size_t)f * d) >= ((size_t)1 << 31))
    return fail(FFN_ERR_UNSUPPORTED, "%s quant arrays must be smaller than 2 GiB", T::name);
  if (!aligned(x, 16) || !aligned(g, 16) || !aligned(y, 16))
    return fail(FFN_ERR_UNSUPPORTED, "x, g and y must be 16-byte aligned");
  const QuantWs L = quant_ws<T>(M, d, f);
  const size_t ws_total = L.total;
  if (M > 0 && (!workspace || workspace_bytes < ws_total))
    return fail(FFN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", ws_total,
                workspace ? workspace_bytes : (size_t)0);
  if (workspace && !aligned(workspace, 256))
    return fail(FFN_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  const size_t ny = (size_t)M * d * 2, nq = T::quant_bytes((size_t)f * d), ns = (size_t)f * d / 32 * 2;
  bool ov = overlap(y, ny, x, ny) || overlap(y, ny, g, (size_t)d * 2) ||
            overlap(y, ny, workspace, workspace ? ws_total : 0);
  for (const typename T::Mat* m : mats)
    ov = ov || overlap(y, ny, m->qs, nq) || overlap(y, ny, m->scales, ns);
  if (ov) return fail(FFN_ERR_INVALID_ARGUMENT, "y overlaps an input or the workspace");
  if (M == 0) return ok();

  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  char* n = ws + L.n;
  char* h = ws + L.h;
  float* part = (float*)(ws + L.part);
  const bool fold = T::fold(M, d, f);
  if (!fold) FFN_LAUNCH("rmsnorm", s, ffn::launch_rmsnorm(2, x, g, n, M, d, eps, s));
  const char* act = fold ? (const char*)x : n;
  const int step = T::max_tokens();
  for (int64_t m0 = 0; m0 < M; m0 += step) {
    const int mc = (int)(M - m0 < step ? M - m0 : step);
    FFN_LAUNCH(T::gateup_name, s,
               T::gateup(act + m0 * d * 2, fold ? g : nullptr, eps, w_gate, w_up, h + m0 * f * 2, mc,
                         (int)d, (int)f, s));
    FFN_LAUNCH(T::down_name, s,
               T::down(h + m0 * f * 2, w_down, (const char*)x + m0 * d * 2, (char*)y + m0 * d * 2,
                       part, mc, (int)d, (int)f, s));
  }
  return ok();
}

}  // namespace

extern "C" {

size_t ffn_swiglu_block_q8_workspace_size(int64_t M, int64_t d, int64_t f) {
  if (M < 0 || M > kQuantMaxTokens || d <= 0 || f <= 0 || d > INT32_MAX || f > INT32_MAX) return 0;
  return quant_ws<Q8Traits>(M, d, f).total;
}

ffn_status ffn_swiglu_block_q8(const void* x, const void* g, const ffn_q8_matrix* w_gate,
                               const ffn_q8_matrix* w_up, const ffn_q8_matrix* w_down, void* y,
                               int64_t M, int64_t d, int64_t f, float eps, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return quant_block<Q8Traits>(x, g, w_gate, w_up, w_down, y, M, d, f, eps, workspace,
                               workspace_bytes, stream);
}

size_t ffn_swiglu_block_q4_workspace_size(int64_t M, int64_t d, int64_t f) {
  if (M < 0 || M > kQuantMaxTokens || d <= 0 || f <= 0 || d > INT32_MAX || f > INT32_MAX) return 0;
  return quant_ws<Q4Traits>(M, d, f).total;
}

ffn_status ffn_swiglu_block_q4(const void* x, const void* g, const ffn_q4_matrix* w_gate,
                               const ffn_q4_matrix* w_up, const ffn_q4_matrix* w_down, void* y,
                               int64_t M, int64_t d, int64_t f, float eps, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return quant_block<Q4Traits>(x, g, w_gate, w_up, w_down, y, M, d, f, eps, workspace,
                               workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
int ffn_probe_read_groups(int waves_per_cu) { return ffn::probe_read_groups(waves_per_cu); }

ffn_status ffn_probe_read(const void* src, size_t bytes, void* sink, int waves_per_cu,
                          void* stream) {
  if (!src || !sink) return fail(FFN_ERR_INVALID_ARGUMENT, "null pointer");
  if (bytes < 16 || bytes % 16 || waves_per_cu < 1 || waves_per_cu > 32)
    return fail(FFN_ERR_INVALID_ARGUMENT, "bytes must be a positive multiple of 16, waves 1..32");
  if (!aligned(src, 16) || !aligned(sink, 16)) return fail(FFN_ERR_UNSUPPORTED, "alignment");
  hipStream_t s = (hipStream_t)stream;
  FFN_LAUNCH("probe_read", s, ffn::launch_probe_read(src, bytes, sink, waves_per_cu, s));
  return ok();
}

ffn_status ffn_probe_copy(const void* src, void* dst, size_t bytes, int groups_per_cu,
                          int nontemporal, void* stream) {
  if (!src || !dst) return fail(FFN_ERR_INVALID_ARGUMENT, "null pointer");
  if (bytes % 16) return fail(FFN_ERR_INVALID_ARGUMENT, "bytes must be a multiple of 16");
  if (groups_per_cu < 0 || groups_per_cu > 64)
    return fail(FFN_ERR_INVALID_ARGUMENT, "groups_per_cu must be 0..64");
  if (!aligned(src, 16) || !aligned(dst, 16)) return fail(FFN_ERR_UNSUPPORTED, "alignment");
  if (overlap(src, bytes, dst, bytes)) return fail(FFN_ERR_INVALID_ARGUMENT, "overlap");
  if (bytes / 16 / 1024 > 0x7FFFFFFFull) return fail(FFN_ERR_UNSUPPORTED, "too large");
  if (bytes == 0) return ok();
  hipStream_t s = (hipStream_t)stream;
  FFN_LAUNCH("probe_copy", s,
             ffn::launch_probe_copy(src, dst, bytes, groups_per_cu, nontemporal != 0, s));
  return ok();
}

int ffn_probe_mfma_groups(int waves_per_cu) {
  return waves_per_cu < 1 || waves_per_cu > 32 ? 0 : ffn::probe_mfma_groups(waves_per_cu);
}

ffn_status ffn_probe_mfma(int iters, int waves_per_cu, void* sink, void* stream) {
  if (!sink) return fail(FFN_ERR_INVALID_ARGUMENT, "null pointer");
  if (iters < 1 || waves_per_cu < 1 || waves_per_cu > 32)
    return fail(FFN_ERR_INVALID_ARGUMENT, "iters >= 1, waves_per_cu 1..32");
  if (!aligned(sink, 16)) return fail(FFN_ERR_UNSUPPORTED, "alignment");
  hipStream_t s = (hipStream_t)stream;
  FFN_LAUNCH("probe_mfma", s, ffn::launch_probe_mfma(iters, waves_per_cu, (float*)sink, s));
  return ok();
}

// ---------------------------------------------------------------------------
ffn_status ffn_timing_enable(int on, int max_launches) {
  Timing& T = t_timing;
  if (!on) {
    T.on = false;
    release_events();
    return ok();
  }
  if (max_launches < 1 || max_launches > (1 << 20))
    return fail(FFN_ERR_INVALID_ARGUMENT, "max_launches must be 1..2^20");
  if (T.cap != max_launches) {
    release_events();
    T.ev.assign(2 * (size_t)max_launches, nullptr);
    T.name.assign(max_launches, std::string());
    T.cap = max_launches;
  }
  T.used = 0;
  T.on = true;
  return ok();
}

int ffn_timing_enabled(void) { return t_timing.on ? 1 : 0; }

ffn_status ffn_timing_collect(void) {
  Timing& T = t_timing;
  for (int i = 0; i < T.used; ++i) {
    if (hipEventSynchronize(T.ev[2 * i + 1]) != hipSuccess)
      return fail(FFN_ERR_LAUNCH, "event synchronize failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, T.ev[2 * i], T.ev[2 * i + 1]) != hipSuccess)
      return fail(FFN_ERR_LAUNCH, "event elapsed time failed");
    const std::string& nm = T.name[i];
    auto it = T.total.find(nm);
    if (it == T.total.end()) {
      T.order.push_back(nm);
      T.total[nm] = {1, (double)ms};
    } else {
      it->second.first += 1;
      it->second.second += ms;
    }
  }
  T.used = 0;
  return ok();
}

int ffn_timing_count(void) { return (int)t_timing.order.size(); }

ffn_status ffn_timing_get(int index, const char** name, int64_t* launches, double* total_ms) {
  Timing& T = t_timing;
  if (index < 0 || index >= (int)T.order.size() || !name || !launches || !total_ms)
    return fail(FFN_ERR_INVALID_ARGUMENT, "bad timing index or null output");
  const std::string& nm = T.order[index];
  *name = nm.c_str();
  *launches = T.total[nm].first;
  *total_ms = T.total[nm].second;
  return ok();
}

void ffn_timing_reset(void) {
  Timing& T = t_timing;
  T.total.clear();
  T.order.clear();
  T.used = 0;
}

}  // extern "C"

// ---------------------------------------------------------------------------
namespace ffn {

void dispatch_events(hipEvent_t* start, hipEvent_t* stop) {
  *start = *stop = nullptr;
  Timing& T = t_timing;
  if (!T.on || !T.site || T.used >= T.cap) return;
  const int i = T.used;
  for (int k = 2 * i; k < 2 * i + 2; ++k)
    if (!T.ev[k] && hipEventCreate(&T.ev[k]) != hipSuccess) {
      T.ev[k] = nullptr;
      return;  // this dispatch runs untimed
    }
  T.name[i] = T.sub == 0 ? std::string(T.site) : std::string(T.site) + "/" + std::to_string(T.sub + 1);
  ++T.sub;
  T.used = i + 1;
  *start = T.ev[2 * i];
  *stop = T.ev[2 * i + 1];
}

}  // namespace ffn

// ---------------------------------------------------------------------------
// The block for callers that cannot allocate: its workspace is `scratch`, a
// file-scope device array each GPU holds from the library's load until the
// process ends.  In host code `scratch` names a host-side stand-in, so the
// array's device address is looked up once per device (with that device
// current) and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[FFN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kNoAllocScratchBytes = (size_t)FFN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // written once per device under the mutex

ffn_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FFN_ERR_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FFN_ERR_UNSUPPORTED, "device ordinal %d beyond the %d the library tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(FFN_ERR_LAUNCH, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FFN_OK;
}

}  // namespace

extern "C" {

ffn_status ffn_swiglu_block_noalloc(ffn_dtype dt, const void* x, const void* g, const void* w_gate,
                                    const void* w_up, const void* w_down, void* y, int64_t M,
                                    int64_t d, int64_t f, float eps, ffn_variant variant,
                                    void* stream) {
  // every argument is checked before the device's array is looked up
  FFN_TRY(check_block_args(dt, x, g, w_gate, w_up, w_down, y, M, d, f, eps, variant));
  const size_t need = ffn_swiglu_block_workspace_size(dt, M, d, f, variant);
  if (need > kNoAllocScratchBytes)
    return fail(FFN_ERR_UNSUPPORTED,
                "this shape needs %zu bytes of workspace; the library's scratch array holds %zu "
                "(use ffn_swiglu_block with a caller workspace)",
                need, kNoAllocScratchBytes);
  if (M == 0) return ok();
  void* ws = nullptr;
  FFN_TRY(scratch_for_current_device(&ws));
  return ffn_swiglu_block(dt, x, g, w_gate, w_up, w_down, y, M, d, f, eps, variant, ws,
                          kNoAllocScratchBytes, stream);
}

}  // extern "C"
