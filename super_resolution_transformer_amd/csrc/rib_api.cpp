// rib_api.cpp -- the C ABI declared in include/rib.h: argument validation,
// variant selection and error reporting.  Validation runs entirely on the host
// and makes no HIP call, so every error path can be exercised without a GPU.
#include "../../include/rib.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "rib_bwd.hpp"
#include "rib_launch.hpp"

namespace {

thread_local char g_err[512] = "";

rib_status fail(rib_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
rib_status fail(rib_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

rib_status ok() {
  g_err[0] = '\0';
  return RIB_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

rib_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(RIB_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

int rib_abi_version(void) { return RIB_ABI_VERSION; }

const char* rib_last_error(void) { return g_err; }

rib_status rib_encode(int window, int L, int hidden, int R, const float* weights, float* qp,
                      float* kp, void* stream) {
  if (!weights || !qp || !kp) return fail(RIB_ERR_INVALID_ARG, "rib_encode: null pointer");
  if (window < 2) return fail(RIB_ERR_INVALID_ARG, "rib_encode: window must be >= 2 (got %d)", window);
  if (L < 0 || hidden < 1 || R < 1)
    return fail(RIB_ERR_INVALID_ARG, "rib_encode: need L >= 0, hidden >= 1, R >= 1 (got %d, %d, %d)", L,
                hidden, R);
  if (window > 128 || L > 16 || hidden > 256 || R > 64)
    return fail(RIB_ERR_UNSUPPORTED,
                "rib_encode: limits are window <= 128, L <= 16, hidden <= 256, R <= 64 (got %d, %d, %d, %d)",
                window, L, hidden, R);
  if (!aligned(weights, 4) || !aligned(qp, 4) || !aligned(kp, 4))
    return fail(RIB_ERR_INVALID_ARG, "rib_encode: pointers must be 4-byte aligned");
  const size_t nw = sizeof(float) * ((size_t)(2 + 4 * L) * hidden + hidden + 2 * (size_t)hidden * R);
  const size_t no = sizeof(float) * (size_t)window * window * R;
  if (overlap(qp, no, kp, no) || overlap(qp, no, weights, nw) || overlap(kp, no, weights, nw))
    return fail(RIB_ERR_INVALID_ARG, "rib_encode: qp, kp and weights must not overlap");
  return hip_status(rib::launch_encode(window, L, hidden, R, weights, qp, kp, (hipStream_t)stream),
                    "rib_encode launch");
}

rib_status rib_attn_supported(int dh, int R, int window, rib_dtype dtype) {
  if (dh < 1 || R < 1 || window < 2) return fail(RIB_ERR_INVALID_ARG, "dh, R >= 1 and window >= 2 required");
  if (dtype != RIB_F32 && dtype != RIB_BF16) return fail(RIB_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (window > 128) return fail(RIB_ERR_UNSUPPORTED, "window %d > 128", window);
  if (dtype == RIB_F32) {
    if (dh > 64 || R > 64) return fail(RIB_ERR_UNSUPPORTED, "fp32 path: dh and R must be <= 64");
    return ok();
  }
  if (!rib::attn_bf16_supported(dh, R))
    return fail(RIB_ERR_UNSUPPORTED, "bf16 path: no compiled variant for (dh=%d, R=%d)", dh, R);
  return ok();
}

}  // extern "C"

namespace {
// shared by rib_window_attn (one (qp, kp) pair) and rib_window_attn_heads (a pair per head)
// T, wt: frames of the map and of a window (1, 1 for images)
rib_status check_attn(const char* fn, bool per_head, const void* qc, const void* kc, const void* v,
                      const void* g, const float* qp, const float* kp, void* o, float* lse, int B, int T, int H,
                      int W, int heads, int dh, int R, int wt, int window, rib_dtype dtype, rib::AttnArgs& a) {
  if (!qc || !kc || !v || !g || !qp || !kp || !o)
    return fail(RIB_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (B < 1 || T < 1 || H < 1 || W < 1 || heads < 1 || dh < 1 || R < 1 || wt < 1)
    return fail(RIB_ERR_INVALID_ARG, "%s: B, T, H, W, heads, dh, R, frames per window must be >= 1", fn);
  if (window < 2) return fail(RIB_ERR_INVALID_ARG, "%s: window must be >= 2 (got %d)", fn, window);
  if (wt > 64 || (long)wt * window * window > 16384)
    return fail(RIB_ERR_UNSUPPORTED, "%s: a window holds at most 16384 tokens (got %d x %d x %d)", fn, wt, window,
                window);
  if (dtype != RIB_F32 && dtype != RIB_BF16)
    return fail(RIB_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
  const rib_status sup = rib_attn_supported(dh, R, window, dtype);
  if (sup != RIB_OK) return sup;
  const uint64_t elems = (uint64_t)B * T * H * W * (uint64_t)heads * dh;
  if (elems >= (1ull << 31))
    return fail(RIB_ERR_UNSUPPORTED, "%s: B*T*H*W*heads*dh must be < 2^31", fn);
  // maps: the kernels read and write them in dwords (head slices of bf16 maps start on any
  // dword: 60 bytes apart for 30-channel heads), and their buffer loads need only dword
  // alignment; tables: the query side reads float pairs
  if (!aligned(qc, 4) || !aligned(kc, 4) || !aligned(v, 4) || !aligned(g, 4) || !aligned(o, 4))
    return fail(RIB_ERR_INVALID_ARG, "%s: map pointers must be 4-byte aligned", fn);
  if (!aligned(qp, 8) || !aligned(kp, 8))
    return fail(RIB_ERR_INVALID_ARG, "%s: qp and kp must be 8-byte aligned", fn);
  const size_t nb = (size_t)elems * (dtype == RIB_F32 ? 4 : 2);
  const size_t np = sizeof(float) * (size_t)wt * window * window * R * (per_head ? heads : 1);
  if (overlap(o, nb, qc, nb) || overlap(o, nb, kc, nb) || overlap(o, nb, v, nb) || overlap(o, nb, g, nb) ||
      overlap(o, nb, qp, np) || overlap(o, nb, kp, np))
    return fail(RIB_ERR_INVALID_ARG, "%s: output overlaps an input", fn);
  if (lse) {
    const size_t nl = sizeof(float) * (size_t)B * T * H * W * heads;
    const void* ins[] = {qc, kc, v, g, o};
    for (const void* p : ins)
      if (overlap(lse, nl, p, nb)) return fail(RIB_ERR_INVALID_ARG, "%s: lse overlaps a map", fn);
    if (overlap(lse, nl, qp, np) || overlap(lse, nl, kp, np))
      return fail(RIB_ERR_INVALID_ARG, "%s: lse overlaps a positional table", fn);
  }
  const long tstride = per_head ? (long)wt * window * window * R : 0;
  a = rib::AttnArgs{qc, kc, v, g, qp, kp, o, B, H, W, heads, dh, R, window, tstride, lse, T, wt};
  return RIB_OK;
}

rib_status window_attn(const char* fn, bool per_head, const void* qc, const void* kc, const void* v,
                       const void* g, const float* qp, const float* kp, void* o, float* lse, int B, int T, int H,
                       int W, int heads, int dh, int R, int wt, int window, rib_dtype dtype, void* stream) {
  rib::AttnArgs a{};
  const rib_status st = check_attn(fn, per_head, qc, kc, v, g, qp, kp, o, lse, B, T, H, W, heads, dh, R, wt,
                                   window, dtype, a);
  if (st != RIB_OK) return st;
  const hipError_t e = dtype == RIB_F32 ? rib::launch_attn_f32(a, (hipStream_t)stream)
                                        : rib::launch_attn_bf16(a, (hipStream_t)stream);
  return hip_status(e, fn);
}
}  // namespace

extern "C" {

rib_status rib_window_attn(const void* qc, const void* kc, const void* v, const void* g,
                           const float* qp, const float* kp, void* o, int B, int H, int W,
                           int heads, int dh, int R, int window, rib_dtype dtype, void* stream) {
  return window_attn("rib_window_attn", false, qc, kc, v, g, qp, kp, o, nullptr, B, 1, H, W, heads, dh, R, 1,
                     window, dtype, stream);
}

rib_status rib_window_attn_lnq(const void* x, const float* gamma, const float* beta, const float* w,
                               const float* bias, const void* kc, const void* v, const void* g, const float* qp,
                               const float* kp, void* o, int B, int H, int W, int heads, int dh, int R, int window,
                               float eps, rib_dtype dtype, void* stream) {
  const char* fn = "rib_window_attn_lnq";
  if (!gamma || !beta || !w || !bias) return fail(RIB_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (dtype != RIB_BF16) return fail(RIB_ERR_UNSUPPORTED, "%s: bf16 maps only", fn);
  if (!(eps >= 0.0f) || eps > 1.0f) return fail(RIB_ERR_INVALID_ARG, "%s: eps must be in [0, 1]", fn);
  if (!((dh == 30 && R == 16) || (dh == 16 && R == 16)))
    return fail(RIB_ERR_UNSUPPORTED, "%s: (dh, R) must be (30, 16) or (16, 16) (got %d, %d)", fn, dh, R);
  if ((long)heads * dh > 192) return fail(RIB_ERR_UNSUPPORTED, "%s: heads * dh must be <= 192", fn);
  rib::AttnArgs a{};
  const rib_status st = check_attn(fn, false, x, kc, v, g, qp, kp, o, nullptr, B, 1, H, W, heads, dh, R, 1,
                                   window, dtype, a);
  if (st != RIB_OK) return st;
  const void* par[] = {gamma, beta, w, bias};
  for (const void* p : par)
    if (!aligned(p, 4)) return fail(RIB_ERR_INVALID_ARG, "%s: parameter pointers must be 4-byte aligned", fn);
  const size_t C = (size_t)heads * dh;
  const size_t nb = (size_t)B * H * W * C * 2;
  const size_t psz[] = {4 * C, 4 * C, 12 * C * C, 12 * C};
  for (int i = 0; i < 4; ++i)
    if (overlap(o, nb, par[i], psz[i])) return fail(RIB_ERR_INVALID_ARG, "%s: output overlaps a parameter", fn);
  return hip_status(rib::launch_attn_bf16_lnq(a, x, gamma, beta, w, bias, eps, (hipStream_t)stream), fn);
}

rib_status rib_window_attn_train(const void* qc, const void* kc, const void* v, const void* g,
                                 const float* qp, const float* kp, void* o, float* lse, int B, int H, int W,
                                 int heads, int dh, int R, int window, rib_dtype dtype, void* stream) {
  if (!lse) return fail(RIB_ERR_INVALID_ARG, "rib_window_attn_train: null pointer");
  return window_attn("rib_window_attn_train", false, qc, kc, v, g, qp, kp, o, lse, B, 1, H, W, heads, dh, R,
                     1, window, dtype, stream);
}

rib_status rib_window_attn_heads(const void* qc, const void* kc, const void* v, const void* g,
                                 const float* qp, const float* kp, void* o, int B, int H, int W,
                                 int heads, int dh, int R, int window, rib_dtype dtype, void* stream) {
  return window_attn("rib_window_attn_heads", true, qc, kc, v, g, qp, kp, o, nullptr, B, 1, H, W, heads, dh,
                     R, 1, window, dtype, stream);
}

rib_status rib_window_attn_heads_train(const void* qc, const void* kc, const void* v, const void* g,
                                       const float* qp, const float* kp, void* o, float* lse, int B, int H, int W,
                                       int heads, int dh, int R, int window, rib_dtype dtype, void* stream) {
  if (!lse) return fail(RIB_ERR_INVALID_ARG, "rib_window_attn_heads_train: null pointer");
  return window_attn("rib_window_attn_heads_train", true, qc, kc, v, g, qp, kp, o, lse, B, 1, H, W, heads, dh,
                     R, 1, window, dtype, stream);
}

rib_status rib_window_attn_multi(int n, const rib_attn_call* calls, rib_dtype dtype, void* stream) {
  const char* fn = "rib_window_attn_multi";
  if (!calls) return fail(RIB_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (n < 1 || n > RIB_MAX_CALLS)
    return fail(RIB_ERR_INVALID_ARG, "%s: n must be in [1, %d] (got %d)", fn, RIB_MAX_CALLS, n);
  rib::AttnArgs args[RIB_MAX_CALLS];
  size_t bytes[RIB_MAX_CALLS];
  for (int i = 0; i < n; ++i) {
    const rib_attn_call& c = calls[i];
    const rib_status st = check_attn(fn, false, c.qc, c.kc, c.v, c.g, c.qp, c.kp, c.o, nullptr, c.B, 1, c.H, c.W,
                                     c.heads, c.dh, c.R, 1, c.window, dtype, args[i]);
    if (st != RIB_OK) return st;
    bytes[i] = (size_t)c.B * c.H * c.W * (size_t)c.heads * c.dh * (dtype == RIB_F32 ? 4 : 2);
  }
  // no call may write what another call reads or writes
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) {
      if (i == j) continue;
      const rib_attn_call& a = calls[i];
      const rib_attn_call& b = calls[j];
      const size_t np = sizeof(float) * (size_t)b.window * b.window * b.R;
      if (overlap(a.o, bytes[i], b.qc, bytes[j]) || overlap(a.o, bytes[i], b.kc, bytes[j]) ||
          overlap(a.o, bytes[i], b.v, bytes[j]) || overlap(a.o, bytes[i], b.g, bytes[j]) ||
          overlap(a.o, bytes[i], b.o, bytes[j]) || overlap(a.o, bytes[i], b.qp, np) ||
          overlap(a.o, bytes[i], b.kp, np))
        return fail(RIB_ERR_INVALID_ARG, "%s: the output of call %d overlaps an argument of call %d", fn, i, j);
    }
  hipError_t e = hipSuccess;
  if (dtype == RIB_F32) {
    for (int i = 0; i < n && e == hipSuccess; ++i) e = rib::launch_attn_f32(args[i], (hipStream_t)stream);
  } else {
    // one multi launch per (dh, R) variant present, in order of first appearance
    bool done[RIB_MAX_CALLS] = {};
    for (int i = 0; i < n && e == hipSuccess; ++i) {
      if (done[i]) continue;
      rib::AttnArgs sel[RIB_MAX_CALLS];
      int m = 0;
      for (int j = i; j < n; ++j)
        if (!done[j] && args[j].dh == args[i].dh && args[j].R == args[i].R) {
          sel[m++] = args[j];
          done[j] = true;
        }
      e = rib::launch_attn_bf16_multi(sel, m, (hipStream_t)stream);
    }
  }
  return hip_status(e, fn);
}


rib_status rib_cla_gate(const void* x, const float* dw_w, const float* dw_b, const float* pw_w,
                        const float* pw_b, void* g, int B, int H, int W, int C, rib_dtype dtype,
                        void* stream) {
  if (!x || !dw_w || !dw_b || !pw_w || !pw_b || !g) return fail(RIB_ERR_INVALID_ARG, "rib_cla_gate: null pointer");
  if (B < 1 || H < 1 || W < 1 || C < 1)
    return fail(RIB_ERR_INVALID_ARG, "rib_cla_gate: B, H, W, C must be >= 1 (got %d, %d, %d, %d)", B, H, W, C);
  if (dtype != RIB_F32 && dtype != RIB_BF16) return fail(RIB_ERR_INVALID_ARG, "rib_cla_gate: unknown dtype %d", (int)dtype);
  if (C % 2 != 0 || C > 256)
    return fail(RIB_ERR_UNSUPPORTED, "rib_cla_gate: C must be even and <= 256 (got %d)", C);
  const size_t elems = (size_t)B * H * W * C;
  if (elems >= ((size_t)1 << 31)) return fail(RIB_ERR_UNSUPPORTED, "rib_cla_gate: B*H*W*C must be < 2^31");
  if (!aligned(x, 4) || !aligned(g, 4) || !aligned(dw_w, 4) || !aligned(dw_b, 4) || !aligned(pw_w, 4) ||
      !aligned(pw_b, 4))
    return fail(RIB_ERR_INVALID_ARG, "rib_cla_gate: pointers must be 4-byte aligned");
  const size_t es = dtype == RIB_F32 ? 4 : 2;
  const size_t nmap = elems * es;
  if (overlap(g, nmap, x, nmap) || overlap(g, nmap, dw_w, 36 * (size_t)C) || overlap(g, nmap, dw_b, 4 * (size_t)C) ||
      overlap(g, nmap, pw_w, 4 * (size_t)C * C) || overlap(g, nmap, pw_b, 4 * (size_t)C))
    return fail(RIB_ERR_INVALID_ARG, "rib_cla_gate: g must not overlap x or the weights");
  rib::GateArgs a{x, dw_w, dw_b, pw_w, pw_b, g, B, H, W, C};
  return hip_status(rib::launch_cla_gate(a, dtype == RIB_BF16, (hipStream_t)stream), "rib_cla_gate launch");
}
}  // extern "C"

namespace {
// Workspace of rib_window_attn_backward: dA (storage type), D, the per-row
// dQp and dKp (fp32), and on the matrix-core path the two packed operand
// images; each region 256-byte aligned.
struct BwdLayout {
  size_t da, dsum, qrows, krows, pk, pq, total;
};

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

BwdLayout bwd_layout(int B, int H, int W, int heads, int dh, int R, int window, rib_dtype dtype) {
  const size_t rows = (size_t)B * H * W * heads;
  const size_t es = dtype == RIB_F32 ? 4 : 2;
  BwdLayout l;
  l.da = 0;
  l.dsum = up256(rows * dh * es);
  l.qrows = l.dsum + up256(rows * 4);
  l.krows = l.qrows + up256(rows * R * 4);
  l.pk = l.krows + up256(rows * R * 4);
  const bool mfma = dtype == RIB_BF16 && rib::attn_bwd_bf16_supported(dh, R);
  const size_t img = mfma ? rib::attn_bwd_bf16_image_bytes(B, H, W, heads, window) : 0;
  l.pq = l.pk + up256(img);
  l.total = l.pq + up256(img);
  return l;
}
}  // namespace

extern "C" {

size_t rib_window_attn_backward_workspace(int B, int H, int W, int heads, int dh, int R, int window,
                                          rib_dtype dtype) {
  if (B < 1 || H < 1 || W < 1 || heads < 1 || dh < 1 || R < 1 || window < 2 ||
      (dtype != RIB_F32 && dtype != RIB_BF16))
    return 0;
  return bwd_layout(B, H, W, heads, dh, R, window, dtype).total;
}

}  // extern "C"

namespace {
// shared by rib_window_attn_backward (one (qp, kp) pair; table gradients summed
// over heads) and rib_window_attn_heads_backward (a pair and a gradient per head)
rib_status window_attn_backward(const char* fn, bool per_head, const void* qc, const void* kc, const void* v,
                                const void* g, const float* qp, const float* kp, const void* o, const float* lse,
                                const void* dout, void* dqc, void* dkc, void* dv, void* dg, float* dqp,
                                float* dkp, void* workspace, size_t workspace_bytes, int B, int H, int W,
                                int heads, int dh, int R, int window, rib_dtype dtype, void* stream) {
  if (!qc || !kc || !v || !g || !qp || !kp || !o || !lse || !dout || !dqc || !dkc || !dv || !dg || !dqp ||
      !dkp || !workspace)
    return fail(RIB_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (B < 1 || H < 1 || W < 1 || heads < 1 || dh < 1 || R < 1)
    return fail(RIB_ERR_INVALID_ARG, "%s: B, H, W, heads, dh, R must be >= 1", fn);
  if (window < 2) return fail(RIB_ERR_INVALID_ARG, "%s: window must be >= 2 (got %d)", fn, window);
  if (dtype != RIB_F32 && dtype != RIB_BF16) return fail(RIB_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
  if (window > 128 || dh > 64 || R > 64)
    return fail(RIB_ERR_UNSUPPORTED, "%s: limits are window <= 128, dh <= 64, R <= 64 (got %d, %d, %d)", fn,
                window, dh, R);
  const uint64_t elems = (uint64_t)B * H * W * (uint64_t)heads * dh;
  if (elems >= (1ull << 31) || (uint64_t)B * H * W * heads * (uint64_t)R >= (1ull << 31))
    return fail(RIB_ERR_UNSUPPORTED, "%s: B*H*W*heads*max(dh, R) must be < 2^31", fn);
  const void* all[] = {qc, kc, v, g, qp, kp, o, lse, dout, dqc, dkc, dv, dg, dqp, dkp, workspace};
  for (const void* p : all)
    if (!aligned(p, 4)) return fail(RIB_ERR_INVALID_ARG, "%s: pointers must be 4-byte aligned", fn);
  if (!aligned(qp, 8) || !aligned(kp, 8))
    return fail(RIB_ERR_INVALID_ARG, "%s: qp and kp must be 8-byte aligned", fn);
  if (!aligned(workspace, 16))
    return fail(RIB_ERR_INVALID_ARG, "%s: the workspace must be 16-byte aligned", fn);
  const BwdLayout lay = bwd_layout(B, H, W, heads, dh, R, window, dtype);
  if (workspace_bytes < lay.total)
    return fail(RIB_ERR_INVALID_ARG, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, lay.total);
  const size_t nb = (size_t)elems * (dtype == RIB_F32 ? 4 : 2);
  const size_t np = sizeof(float) * (size_t)window * window * R * (per_head ? heads : 1);
  const size_t nl = sizeof(float) * (size_t)B * H * W * heads;
  const size_t sizes[] = {nb, nb, nb, nb, np, np, nb, nl, nb, nb, nb, nb, nb, np, np, lay.total};
  // every output (indices 9..15, the workspace included) is disjoint from every other buffer
  for (int i = 9; i < 16; ++i)
    for (int j = 0; j < 16; ++j)
      if (j != i && overlap(all[i], sizes[i], all[j], sizes[j]))
        return fail(RIB_ERR_INVALID_ARG, "%s: an output or the workspace overlaps another buffer", fn);
  char* w = (char*)workspace;
  rib::BwdArgs a{qc, kc, v, g, qp, kp, o, lse, dout, dqc, dkc, dv, dg, dqp, dkp,
                 w + lay.da, (float*)(w + lay.dsum), (float*)(w + lay.qrows), (float*)(w + lay.krows),
                 (uint32_t*)(w + lay.pk), (uint32_t*)(w + lay.pq), B, H, W, heads, dh, R, window,
                 rib::bwd_tiles_per_unit(window)};
  a.tstride = per_head ? (long)window * window * R : 0;
  a.tab_heads = per_head ? heads : 1;
  const hipStream_t st = (hipStream_t)stream;
  const bool bf16 = dtype == RIB_BF16;
  hipError_t e = rib::launch_attn_bwd_prep(a, bf16, st);
  if (e == hipSuccess)
    e = bf16 && rib::attn_bwd_bf16_supported(dh, R) ? rib::launch_attn_bwd_bf16(a, st)
                                                    : rib::launch_attn_bwd_rows(a, bf16, st);
  if (e == hipSuccess) e = rib::launch_attn_bwd_reduce(a, st);
  return hip_status(e, fn);
}
}  // namespace

extern "C" {

rib_status rib_window_attn_backward(const void* qc, const void* kc, const void* v, const void* g,
                                    const float* qp, const float* kp, const void* o, const float* lse,
                                    const void* dout, void* dqc, void* dkc, void* dv, void* dg, float* dqp,
                                    float* dkp, void* workspace, size_t workspace_bytes, int B, int H, int W,
                                    int heads, int dh, int R, int window, rib_dtype dtype, void* stream) {
  return window_attn_backward("rib_window_attn_backward", false, qc, kc, v, g, qp, kp, o, lse, dout, dqc, dkc,
                              dv, dg, dqp, dkp, workspace, workspace_bytes, B, H, W, heads, dh, R, window, dtype,
                              stream);
}

rib_status rib_window_attn_heads_backward(const void* qc, const void* kc, const void* v, const void* g,
                                          const float* qp, const float* kp, const void* o, const float* lse,
                                          const void* dout, void* dqc, void* dkc, void* dv, void* dg,
                                          float* dqp, float* dkp, void* workspace, size_t workspace_bytes, int B,
                                          int H, int W, int heads, int dh, int R, int window, rib_dtype dtype,
                                          void* stream) {
  return window_attn_backward("rib_window_attn_heads_backward", true, qc, kc, v, g, qp, kp, o, lse, dout, dqc,
                              dkc, dv, dg, dqp, dkp, workspace, workspace_bytes, B, H, W, heads, dh, R, window,
                              dtype, stream);
}

size_t rib_encode_backward_workspace(int window, int L, int hidden, int R) {
  if (window < 2 || window > 128 || L < 0 || L > 16 || hidden < 1 || hidden > 256 || R < 1 || R > 64) return 0;
  return sizeof(float) * (size_t)rib::encode_bwd_blocks(window) *
         ((size_t)(2 + 4 * L) * hidden + hidden + 2 * (size_t)hidden * R);
}

rib_status rib_encode_backward(int window, int L, int hidden, int R, const float* weights, const float* dqp,
                               const float* dkp, float* dweights, void* workspace, size_t workspace_bytes,
                               void* stream) {
  const char* fn = "rib_encode_backward";
  if (!weights || !dqp || !dkp || !dweights || !workspace) return fail(RIB_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (window < 2) return fail(RIB_ERR_INVALID_ARG, "%s: window must be >= 2 (got %d)", fn, window);
  if (L < 0 || hidden < 1 || R < 1)
    return fail(RIB_ERR_INVALID_ARG, "%s: need L >= 0, hidden >= 1, R >= 1 (got %d, %d, %d)", fn, L, hidden, R);
  if (window > 128 || L > 16 || hidden > 256 || R > 64)
    return fail(RIB_ERR_UNSUPPORTED, "%s: limits are window <= 128, L <= 16, hidden <= 256, R <= 64", fn);
  const void* all[] = {weights, dqp, dkp, dweights, workspace};
  for (const void* p : all)
    if (!aligned(p, 4)) return fail(RIB_ERR_INVALID_ARG, "%s: pointers must be 4-byte aligned", fn);
  const size_t need = rib_encode_backward_workspace(window, L, hidden, R);
  if (workspace_bytes < need)
    return fail(RIB_ERR_INVALID_ARG, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
  const size_t nw = sizeof(float) * ((size_t)(2 + 4 * L) * hidden + hidden + 2 * (size_t)hidden * R);
  const size_t no = sizeof(float) * (size_t)window * window * R;
  const size_t sizes[] = {nw, no, no, nw, need};
  for (int i = 3; i < 5; ++i)
    for (int j = 0; j < 5; ++j)
      if (j != i && overlap(all[i], sizes[i], all[j], sizes[j]))
        return fail(RIB_ERR_INVALID_ARG, "%s: dweights or the workspace overlaps another buffer", fn);
  return hip_status(rib::launch_encode_backward(window, L, hidden, R, weights, dqp, dkp, dweights,
                                                (float*)workspace, rib::encode_bwd_blocks(window),
                                                (hipStream_t)stream),
                    "rib_encode_backward launch");
}

rib_status rib_encode_backward_noalloc(int window, int L, int hidden, int R, const float* weights,
                                       const float* dqp, const float* dkp, float* dweights, void* stream) {
  const char* fn = "rib_encode_backward_noalloc";
  if (!weights || !dqp || !dkp || !dweights) return fail(RIB_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (window < 2) return fail(RIB_ERR_INVALID_ARG, "%s: window must be >= 2 (got %d)", fn, window);
  if (L < 0 || hidden < 1 || R < 1)
    return fail(RIB_ERR_INVALID_ARG, "%s: need L >= 0, hidden >= 1, R >= 1 (got %d, %d, %d)", fn, L, hidden, R);
  if (window > 128 || L > 16 || hidden > 256 || R > 64)
    return fail(RIB_ERR_UNSUPPORTED, "%s: limits are window <= 128, L <= 16, hidden <= 256, R <= 64", fn);
  const size_t nw = (size_t)(2 + 4 * L) * hidden + hidden + 2 * (size_t)hidden * R;
  const int rows = rib::encode_scratch_rows(window, L, hidden, R);
  if (rows < 1)
    return fail(RIB_ERR_UNSUPPORTED, "%s: %zu weights exceed the fixed workspace of %ld floats", fn, nw,
                rib::ENC_SCRATCH_FLOATS);
  const void* all[] = {weights, dqp, dkp, dweights};
  for (const void* p : all)
    if (!aligned(p, 4)) return fail(RIB_ERR_INVALID_ARG, "%s: pointers must be 4-byte aligned", fn);
  const size_t no = sizeof(float) * (size_t)window * window * R;
  const size_t sizes[] = {sizeof(float) * nw, no, no, sizeof(float) * nw};
  for (int j = 0; j < 3; ++j)
    if (overlap(all[3], sizes[3], all[j], sizes[j]))
      return fail(RIB_ERR_INVALID_ARG, "%s: dweights overlaps another buffer", fn);
  float* work = nullptr;
  const hipError_t e = rib::encode_scratch(&work);
  if (e != hipSuccess) return hip_status(e, "rib_encode_backward_noalloc workspace lookup");
  return hip_status(rib::launch_encode_backward(window, L, hidden, R, weights, dqp, dkp, dweights, work, rows,
                                                (hipStream_t)stream),
                    "rib_encode_backward_noalloc launch");
}

}  // extern "C"

extern "C" {

rib_status rib_ln_qkv(const void* x, const float* gamma, const float* beta, const float* w, const float* bias,
                      void* q, void* k, void* v, void* xn, int B, int H, int W, int C, float eps, rib_dtype dtype,
                      void* stream) {
  const char* fn = "rib_ln_qkv";
  if (!x || !gamma || !beta || !w || !bias || !k || !v) return fail(RIB_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (B < 1 || H < 1 || W < 1 || C < 1)
    return fail(RIB_ERR_INVALID_ARG, "%s: B, H, W, C must be >= 1 (got %d, %d, %d, %d)", fn, B, H, W, C);
  if (dtype != RIB_F32 && dtype != RIB_BF16) return fail(RIB_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
  if (!(eps >= 0.0f) || eps > 1.0f) return fail(RIB_ERR_INVALID_ARG, "%s: eps must be in [0, 1]", fn);
  if (C > 256 || (dtype == RIB_BF16 && C % 2 != 0))
    return fail(RIB_ERR_UNSUPPORTED, "%s: C must be <= 256 (and even for bf16), got %d", fn, C);
  const size_t elems = (size_t)B * H * W * C;
  if (elems >= ((size_t)1 << 30)) return fail(RIB_ERR_UNSUPPORTED, "%s: B*H*W*C must be < 2^30", fn);
  const void* all[] = {x, q, k, v, xn, gamma, beta, w, bias};
  for (const void* p : all)
    if (p && !aligned(p, 16)) return fail(RIB_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", fn);
  const size_t nm = elems * (dtype == RIB_F32 ? 4 : 2);
  const size_t sizes[] = {nm, nm, nm, nm, nm, 4 * (size_t)C, 4 * (size_t)C, 12 * (size_t)C * C, 12 * (size_t)C};
  // outputs (1..4) are disjoint from every other buffer
  for (int i = 1; i < 5; ++i) {
    if (!all[i]) continue;
    for (int j = 0; j < 9; ++j)
      if (j != i && all[j] && overlap(all[i], sizes[i], all[j], sizes[j]))
        return fail(RIB_ERR_INVALID_ARG, "%s: an output overlaps another buffer", fn);
  }
  const rib::LnQkvArgs a{x, gamma, beta, w, bias, q, k, v, xn, B, H, W, C, eps};
  return hip_status(rib::launch_ln_qkv(a, dtype == RIB_BF16, (hipStream_t)stream), "rib_ln_qkv launch");
}

}  // extern "C"

extern "C" {

rib_status rib_encode3d(int frames, int window, int L, int hidden, int R, const float* weights, float* qp,
                        float* kp, void* stream) {
  const char* fn = "rib_encode3d";
  if (!weights || !qp || !kp) return fail(RIB_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (frames < 1 || window < 2)
    return fail(RIB_ERR_INVALID_ARG, "%s: need frames >= 1, window >= 2 (got %d, %d)", fn, frames, window);
  if (L < 0 || hidden < 1 || R < 1)
    return fail(RIB_ERR_INVALID_ARG, "%s: need L >= 0, hidden >= 1, R >= 1 (got %d, %d, %d)", fn, L, hidden, R);
  if (window > 128 || frames > 64 || (long)frames * window * window > 16384 || L > 16 || hidden > 256 || R > 64)
    return fail(RIB_ERR_UNSUPPORTED,
                "%s: limits are frames*window^2 <= 16384, window <= 128, L <= 16, hidden <= 256, R <= 64", fn);
  if (!aligned(weights, 4) || !aligned(qp, 4) || !aligned(kp, 4))
    return fail(RIB_ERR_INVALID_ARG, "%s: pointers must be 4-byte aligned", fn);
  const size_t nw = sizeof(float) * ((size_t)(3 + 6 * L) * hidden + hidden + 2 * (size_t)hidden * R);
  const size_t no = sizeof(float) * (size_t)frames * window * window * R;
  if (overlap(qp, no, kp, no) || overlap(qp, no, weights, nw) || overlap(kp, no, weights, nw))
    return fail(RIB_ERR_INVALID_ARG, "%s: qp, kp and weights must not overlap", fn);
  return hip_status(rib::launch_encode3d(frames, window, L, hidden, R, weights, qp, kp, (hipStream_t)stream),
                    "rib_encode3d launch");
}

rib_status rib_window_attn3d(const void* qc, const void* kc, const void* v, const void* g, const float* qp,
                             const float* kp, void* o, int B, int T, int H, int W, int heads, int dh, int R,
                             int frames, int window, rib_dtype dtype, void* stream) {
  return window_attn("rib_window_attn3d", false, qc, kc, v, g, qp, kp, o, nullptr, B, T, H, W, heads, dh, R, frames,
                     window, dtype, stream);
}

}  // extern "C"
