// C-ABI entry points of libswattn: argument validation, workspace carving and
// kernel launches.  Declarations and the full contract are in include/swattn.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/swattn.h"
#include "band.h"
#include "kernels.h"

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shared checks of the forward / backward entry points.  Returns ATTN_OK to
// proceed, or a status; *empty is set for problems with no rows.
int check_common(int B, int T, int H, int H_kv, int D, int window, int causal, float eps,
                 bool* empty) {
  *empty = false;
  if (B < 0 || T < 0 || H < 0 || H_kv < 0 || D < 1) return ATTN_ERR_INVALID_ARG;
  if (H > 0 && (H_kv < 1 || H % H_kv != 0)) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(eps) || !(eps > 0.f)) return ATTN_ERR_INVALID_ARG;
  if (window < -1) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (causal == 0) return ATTN_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (B == 0 || T == 0 || H == 0) {
    *empty = true;
    return ATTN_OK;
  }
  const long long elems = (long long)B * T * H * D;
  if (elems >= (1LL << 31)) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

size_t stats_bytes(int B, int T, int H) { return round_up((size_t)B * H * T * sizeof(float)); }

// Row length of the transposed V copy of the forward: T rounded up to 64.
int vt_cols(int T) { return (T + 63) / 64 * 64; }
size_t vt_bytes(int B, int T, int H, int D) { return round_up((size_t)B * H * D * vt_cols(T) * 2); }

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
    default: return "ATTN_UNKNOWN_STATUS";
  }
}

int attn_version(void) { return 100; }

int attn_layer_windows(const char* pattern, int n_layer, int seq_len, int* windows_out) {
  if (!pattern || !windows_out || n_layer < 1 || seq_len < 1) return ATTN_ERR_INVALID_ARG;
  const size_t n = std::strlen(pattern);
  if (n == 0) return ATTN_ERR_INVALID_ARG;
  for (size_t i = 0; i < n; ++i) {
    const char ch = pattern[i];
    if (ch != 'S' && ch != 's' && ch != 'L' && ch != 'l') return ATTN_ERR_INVALID_ARG;
  }
  for (int l = 0; l < n_layer; ++l) {
    const char ch = pattern[l % n];
    windows_out[l] = (ch == 'L' || ch == 'l') ? seq_len : seq_len / 2;
  }
  windows_out[n_layer - 1] = seq_len;
  return ATTN_OK;
}

long long attn_visible_pairs(int T, int window) {
  if (T < 0 || window < -1) return -1;
  const long long W = swattn::eff_window(T, window);
  // rows i <= W see i + 1 keys; later rows see W + 1
  const long long t = T;
  const long long head = (W + 1 < t) ? W + 1 : t;  // rows 0 .. head-1
  return head * (head + 1) / 2 + (t - head) * (W + 1);
}

int attn_band_tiles(int T, int window, int rows, int cols, int by_key, int* first, int* last,
                    int* n_partial, int* n_empty) {
  if (T < 1 || window < -1 || rows < 1 || cols < 1 || !first || !last || !n_partial || !n_empty ||
      (by_key != 0 && by_key != 1))
    return ATTN_ERR_INVALID_ARG;
  const int W = swattn::eff_window(T, window);
  const int nr = (T + rows - 1) / rows;
  for (int r = 0; r < nr; ++r) {
    const int a = r * rows, bnd = a + rows - 1;
    int lo, hi;
    bool any = by_key ? swattn::q_range(a, bnd, T, W, &lo, &hi) : swattn::kv_range(a, bnd, T, W, &lo, &hi);
    first[r] = any ? lo / cols : 0;
    last[r] = any ? hi / cols : -1;
    int np = 0, ne = 0;
    for (int cb = first[r]; cb <= last[r]; ++cb) {
      const int x = cb * cols, y = x + cols - 1;
      const int cls = by_key ? swattn::tile_class(x, y, a, bnd, T, W) : swattn::tile_class(a, bnd, x, y, T, W);
      np += cls == swattn::TILE_PARTIAL;
      ne += cls == swattn::TILE_EMPTY;
    }
    n_partial[r] = np;
    n_empty[r] = ne;
  }
  return ATTN_OK;
}

size_t attn_fwd_gqa_workspace_bytes(int B, int T, int H, int H_kv, int D) {
  if (B < 0 || T < 0 || H < 0 || H_kv < 0 || D < 1) return 0;
  return stats_bytes(B, T, H_kv) + vt_bytes(B, T, H_kv, D);
}

size_t attn_fwd_workspace_bytes(int B, int T, int H, int D) {
  return attn_fwd_gqa_workspace_bytes(B, T, H, H, D);
}

size_t attn_fwd_rope_workspace_bytes(int B, int T, int H, int H_kv, int D) {
  if (B < 0 || T < 0 || H < 0 || H_kv < 0 || D < 1) return 0;
  return attn_fwd_gqa_workspace_bytes(B, T, H, H_kv, D) + round_up((size_t)B * T * H_kv * D * 2);
}

size_t attn_bwd_gqa_workspace_bytes(int B, int T, int H, int H_kv, int D) {
  if (B < 0 || T < 0 || H < 0 || H_kv < 0 || D < 1) return 0;
  return round_up((size_t)B * T * H * D * 2) + 3 * stats_bytes(B, T, H);
}

size_t attn_bwd_workspace_bytes(int B, int T, int H, int D) {
  return attn_bwd_gqa_workspace_bytes(B, T, H, H, D);
}

size_t attn_bwd_rope_workspace_bytes(int B, int T, int H, int H_kv, int D) {
  if (B < 0 || T < 0 || H < 0 || H_kv < 0 || D < 1) return 0;
  return attn_bwd_gqa_workspace_bytes(B, T, H, H_kv, D) + round_up((size_t)B * T * H_kv * D * 2);
}

}  // extern "C"

namespace {

// Forward with or without the rotary embedding (rcos == nullptr: none).
int fwd_impl(const void* q, const void* k, const void* v, const void* rcos, const void* rsin,
             void* o, float* lse, void* workspace, size_t workspace_bytes, int B, int T, int H,
             int H_kv, int D, int window, int causal, float eps, void* stream, bool rope) {
  bool empty;
  int st = check_common(B, T, H, H_kv, D, window, causal, eps, &empty);
  if (st != ATTN_OK || empty) return st;
  const void* ins[5] = {q, k, v, rcos, rsin};
  const int nin = rope ? 5 : 3;
  for (int i = 0; i < nin; ++i)
    if (!ins[i] || !aligned(ins[i], 16)) return ATTN_ERR_INVALID_ARG;
  if (!o || !lse || !aligned(o, 16) || !aligned(lse, 16)) return ATTN_ERR_INVALID_ARG;
  for (int i = 0; i < nin; ++i)
    if (ins[i] == o || ins[i] == (const void*)lse) return ATTN_ERR_INVALID_ARG;
  const size_t need = rope ? attn_fwd_rope_workspace_bytes(B, T, H, H_kv, D)
                           : attn_fwd_gqa_workspace_bytes(B, T, H, H_kv, D);
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return ATTN_ERR_WORKSPACE;

  swattn::FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.kscale = static_cast<float*>(workspace);
  a.vt = static_cast<char*>(workspace) + stats_bytes(B, T, H_kv);
  a.LT = vt_cols(T);
  a.rcos = rope ? rcos : nullptr;
  a.rsin = rope ? rsin : nullptr;
  a.kr = rope ? static_cast<char*>(workspace) + attn_fwd_gqa_workspace_bytes(B, T, H, H_kv, D) : nullptr;
  a.B = B; a.T = T; a.H = H; a.Hkv = H_kv; a.D = D; a.window = window; a.eps = eps;
  hipError_t e = swattn::launch_fwd(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int bwd_impl(const void* q, const void* k, const void* v, const void* rcos, const void* rsin,
             const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
             void* workspace, size_t workspace_bytes, int B, int T, int H, int H_kv, int D,
             int window, int causal, float eps, void* stream, bool rope) {
  bool empty;
  int st = check_common(B, T, H, H_kv, D, window, causal, eps, &empty);
  if (st != ATTN_OK || empty) return st;
  const void* ins[8] = {q, k, v, o, lse, dout, rcos, rsin};
  const int nin = rope ? 8 : 6;
  void* outs[3] = {dq, dk, dv};
  for (int i = 0; i < nin; ++i)
    if (!ins[i] || !aligned(ins[i], 16)) return ATTN_ERR_INVALID_ARG;
  for (void* p : outs) {
    if (!p || !aligned(p, 16)) return ATTN_ERR_INVALID_ARG;
    for (int i = 0; i < nin; ++i)
      if (ins[i] == p) return ATTN_ERR_INVALID_ARG;
  }
  if (dq == dk || dq == dv || dk == dv) return ATTN_ERR_INVALID_ARG;
  const size_t need = rope ? attn_bwd_rope_workspace_bytes(B, T, H, H_kv, D)
                           : attn_bwd_gqa_workspace_bytes(B, T, H, H_kv, D);
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return ATTN_ERR_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  const size_t qh_bytes = round_up((size_t)B * T * H * D * 2);
  const size_t sb = stats_bytes(B, T, H);
  swattn::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dout = dout;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.qhat = ws;
  a.kscale = reinterpret_cast<float*>(ws + qh_bytes);
  a.delta = reinterpret_cast<float*>(ws + qh_bytes + sb);
  a.lse2 = reinterpret_cast<float*>(ws + qh_bytes + 2 * sb);
  a.rcos = rope ? rcos : nullptr;
  a.rsin = rope ? rsin : nullptr;
  a.kr = rope ? ws + attn_bwd_gqa_workspace_bytes(B, T, H, H_kv, D) : nullptr;
  a.B = B; a.T = T; a.H = H; a.Hkv = H_kv; a.D = D; a.window = window; a.eps = eps;
  hipError_t e = swattn::launch_bwd(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

extern "C" {

int attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                 void* workspace, size_t workspace_bytes, int B, int T, int H, int H_kv, int D,
                 int window, int causal, float eps, void* stream) {
  return fwd_impl(q, k, v, nullptr, nullptr, o, lse, workspace, workspace_bytes, B, T, H, H_kv, D,
                  window, causal, eps, stream, false);
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
             size_t workspace_bytes, int B, int T, int H, int D, int window, int causal, float eps,
             void* stream) {
  return fwd_impl(q, k, v, nullptr, nullptr, o, lse, workspace, workspace_bytes, B, T, H, H, D,
                  window, causal, eps, stream, false);
}

int attn_fwd_rope(const void* q, const void* k, const void* v, const void* rope_cos,
                  const void* rope_sin, void* o, float* lse, void* workspace,
                  size_t workspace_bytes, int B, int T, int H, int H_kv, int D, int window,
                  int causal, float eps, void* stream) {
  return fwd_impl(q, k, v, rope_cos, rope_sin, o, lse, workspace, workspace_bytes, B, T, H, H_kv,
                  D, window, causal, eps, stream, true);
}

int attn_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, void* workspace,
                 size_t workspace_bytes, int B, int T, int H, int H_kv, int D, int window,
                 int causal, float eps, void* stream) {
  return bwd_impl(q, k, v, nullptr, nullptr, o, lse, dout, dq, dk, dv, workspace, workspace_bytes,
                  B, T, H, H_kv, D, window, causal, eps, stream, false);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, void* workspace,
             size_t workspace_bytes, int B, int T, int H, int D, int window, int causal,
             float eps, void* stream) {
  return bwd_impl(q, k, v, nullptr, nullptr, o, lse, dout, dq, dk, dv, workspace, workspace_bytes,
                  B, T, H, H, D, window, causal, eps, stream, false);
}

int attn_bwd_rope(const void* q, const void* k, const void* v, const void* rope_cos,
                  const void* rope_sin, const void* o, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B,
                  int T, int H, int H_kv, int D, int window, int causal, float eps,
                  void* stream) {
  return bwd_impl(q, k, v, rope_cos, rope_sin, o, lse, dout, dq, dk, dv, workspace,
                  workspace_bytes, B, T, H, H_kv, D, window, causal, eps, stream, true);
}

}  // extern "C"
