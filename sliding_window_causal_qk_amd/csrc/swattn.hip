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

// Byte range [lo, hi) of one buffer, for the no-overlap rules: an output may
// share no byte with an input, another output or the workspace, and the
// workspace none with any input or output.
struct Span {
  uintptr_t lo = 0, hi = 0;
};
Span span(const void* p, size_t nbytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Span{a, a + nbytes};
}
bool overlap(const Span& a, const Span& b) {
  return a.hi > a.lo && b.hi > b.lo && a.lo < b.hi && b.lo < a.hi;
}
bool overlaps_any(const Span& a, const Span* set, int n) {
  for (int i = 0; i < n; ++i)
    if (overlap(a, set[i])) return true;
  return false;
}

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
  if (D != 64 && D != 128 && D != 256) return ATTN_ERR_UNSUPPORTED;
  if (B == 0 || T == 0 || H == 0) {
    *empty = true;
    return ATTN_OK;
  }
  const long long elems = (long long)B * T * H * D;
  if (elems >= (1LL << 31)) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

size_t stats_bytes(int B, int T, int H) { return round_up((size_t)B * H * T * sizeof(float)); }

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
  return stats_bytes(B, T, H_kv);
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

size_t attn_fwd_ve_workspace_bytes(int B, int T, int H, int H_kv, int D) {
  if (B < 0 || T < 0 || H < 0 || H_kv < 0 || D < 1) return 0;
  return attn_fwd_rope_workspace_bytes(B, T, H, H_kv, D) + round_up((size_t)B * T * H_kv * D * 2) +
         stats_bytes(B, T, H_kv);
}

size_t attn_bwd_ve_workspace_bytes(int B, int T, int H, int H_kv, int D) {
  if (B < 0 || T < 0 || H < 0 || H_kv < 0 || D < 1) return 0;
  return attn_bwd_rope_workspace_bytes(B, T, H, H_kv, D) + round_up((size_t)B * T * H_kv * D * 2) +
         2 * stats_bytes(B, T, H_kv) +
         round_up(((size_t)B * T + swattn::kGateTokens - 1) / swattn::kGateTokens * H_kv * 32 * 4);
}

}  // extern "C"

namespace {

// Optional parts of a call: rotary tables, and the value-embedding gate's
// inputs and (backward) gradient outputs.
struct Extras {
  bool rope = false;
  const void* rcos = nullptr;
  const void* rsin = nullptr;
  bool gate = false;
  const void* ve = nullptr;
  const void* xg = nullptr;
  int xs = 0;
  const float* gate_w = nullptr;
  void* dve = nullptr;
  void* dxg = nullptr;
  float* dgate_w = nullptr;
};

constexpr int kGateMaxKvHeads = 16;

// Checks of the optional inputs; appends their byte ranges to `ins` for the
// overlap rules.
int check_extras(const Extras& x, int B, int T, int H_kv, int D, Span* ins, int* nin) {
  if (x.rope) {
    if (!x.rcos || !x.rsin || !aligned(x.rcos, 16) || !aligned(x.rsin, 16)) return ATTN_ERR_INVALID_ARG;
    const size_t tb = (size_t)T * (D / 2) * 2;
    ins[(*nin)++] = span(x.rcos, tb);
    ins[(*nin)++] = span(x.rsin, tb);
  }
  if (x.gate) {
    if (!x.ve || !x.xg || !x.gate_w || !aligned(x.ve, 16) || !aligned(x.xg, 16) || !aligned(x.gate_w, 16))
      return ATTN_ERR_INVALID_ARG;
    if (x.xs < 32 || x.xs % 8 != 0) return ATTN_ERR_INVALID_ARG;
    if (H_kv > kGateMaxKvHeads) return ATTN_ERR_UNSUPPORTED;
    ins[(*nin)++] = span(x.ve, (size_t)B * T * H_kv * D * 2);
    ins[(*nin)++] = span(x.xg, (((size_t)B * T - 1) * x.xs + 32) * 2);   // the 32 channels read per token
    ins[(*nin)++] = span(x.gate_w, (size_t)H_kv * 32 * 4);
  }
  return ATTN_OK;
}

int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
             size_t workspace_bytes, int B, int T, int H, int H_kv, int D, int window, int causal,
             float eps, void* stream, const Extras& x) {
  bool empty;
  int st = check_common(B, T, H, H_kv, D, window, causal, eps, &empty);
  if (st != ATTN_OK || empty) return st;
  for (const void* p : {q, k, v})
    if (!p || !aligned(p, 16)) return ATTN_ERR_INVALID_ARG;
  const size_t qb = (size_t)B * T * H * D * 2, kb = (size_t)B * T * H_kv * D * 2;
  Span ins[8] = {span(q, qb), span(k, kb), span(v, kb)};
  int nin = 3;
  st = check_extras(x, B, T, H_kv, D, ins, &nin);
  if (st != ATTN_OK) return st;
  if (!o || !lse || !aligned(o, 16) || !aligned(lse, 16)) return ATTN_ERR_INVALID_ARG;
  const Span outs[2] = {span(o, qb), span(lse, (size_t)B * H * T * 4)};
  for (int j = 0; j < 2; ++j)
    if (overlaps_any(outs[j], ins, nin) || overlaps_any(outs[j], outs, j)) return ATTN_ERR_INVALID_ARG;
  const size_t need = x.gate   ? attn_fwd_ve_workspace_bytes(B, T, H, H_kv, D)
                      : x.rope ? attn_fwd_rope_workspace_bytes(B, T, H, H_kv, D)
                               : attn_fwd_gqa_workspace_bytes(B, T, H, H_kv, D);
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return ATTN_ERR_WORKSPACE;
  const Span wsp = span(workspace, need);
  if (overlaps_any(wsp, ins, nin) || overlaps_any(wsp, outs, 2)) return ATTN_ERR_WORKSPACE;

  swattn::FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.kscale = static_cast<float*>(workspace);
  a.rcos = x.rope ? x.rcos : nullptr;
  a.rsin = x.rope ? x.rsin : nullptr;
  a.kr = x.rope ? static_cast<char*>(workspace) + attn_fwd_gqa_workspace_bytes(B, T, H, H_kv, D) : nullptr;
  a.vr = x.gate ? static_cast<char*>(workspace) + attn_fwd_rope_workspace_bytes(B, T, H, H_kv, D) : nullptr;
  a.gate = x.gate ? reinterpret_cast<float*>(static_cast<char*>(a.vr) + round_up((size_t)B * T * H_kv * D * 2))
                  : nullptr;
  a.ve = x.gate ? x.ve : nullptr;
  a.xg = x.xg;
  a.xs = x.xs;
  a.gate_w = x.gate_w;
  a.B = B; a.T = T; a.H = H; a.Hkv = H_kv; a.D = D; a.window = window; a.eps = eps;
  hipError_t e = swattn::launch_fwd(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

// reuse: fwd_ws is the workspace of the forward call that produced o and
// lse; its key scales (and rotated keys, gated values, gate) are used instead
// of running the key pre-pass again.
int bwd_impl(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, void* workspace,
             size_t workspace_bytes, int B, int T, int H, int H_kv, int D, int window, int causal,
             float eps, void* stream, const Extras& x, bool reuse = false, const void* fwd_ws = nullptr,
             size_t fwd_ws_bytes = 0) {
  bool empty;
  int st = check_common(B, T, H, H_kv, D, window, causal, eps, &empty);
  if (st != ATTN_OK || empty) return st;
  for (const void* p : {q, k, v, o, (const void*)lse, dout})
    if (!p || !aligned(p, 16)) return ATTN_ERR_INVALID_ARG;
  const size_t qb = (size_t)B * T * H * D * 2, kb = (size_t)B * T * H_kv * D * 2;
  const size_t sb_h = (size_t)B * H * T * 4;
  Span ins[12] = {span(q, qb), span(k, kb), span(v, kb), span(o, qb), span(lse, sb_h), span(dout, qb)};
  int nin = 6;
  st = check_extras(x, B, T, H_kv, D, ins, &nin);
  if (st != ATTN_OK) return st;
  void* const outp[6] = {dq, dk, dv, x.dve, x.dxg, x.dgate_w};
  const size_t outb[6] = {qb, kb, kb, kb, (size_t)B * T * 32 * 2, (size_t)H_kv * 32 * 4};
  const int nout = x.gate ? 6 : 3;
  Span outs[6];
  for (int j = 0; j < nout; ++j) {
    if (!outp[j] || !aligned(outp[j], 16)) return ATTN_ERR_INVALID_ARG;
    outs[j] = span(outp[j], outb[j]);
    if (overlaps_any(outs[j], ins, nin) || overlaps_any(outs[j], outs, j)) return ATTN_ERR_INVALID_ARG;
  }
  const size_t need = x.gate   ? attn_bwd_ve_workspace_bytes(B, T, H, H_kv, D)
                      : x.rope ? attn_bwd_rope_workspace_bytes(B, T, H, H_kv, D)
                               : attn_bwd_gqa_workspace_bytes(B, T, H, H_kv, D);
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return ATTN_ERR_WORKSPACE;
  const Span wsp = span(workspace, need);
  if (overlaps_any(wsp, ins, nin) || overlaps_any(wsp, outs, nout)) return ATTN_ERR_WORKSPACE;
  if (reuse) {
    if (!fwd_ws) return ATTN_ERR_WORKSPACE;
    const size_t need_f = x.gate   ? attn_fwd_ve_workspace_bytes(B, T, H, H_kv, D)
                          : x.rope ? attn_fwd_rope_workspace_bytes(B, T, H, H_kv, D)
                                   : attn_fwd_gqa_workspace_bytes(B, T, H, H_kv, D);
    if (fwd_ws_bytes < need_f || !aligned(fwd_ws, kAlign)) return ATTN_ERR_WORKSPACE;
    const Span fws = span(fwd_ws, need_f);
    if (overlap(fws, wsp)) return ATTN_ERR_WORKSPACE;
    if (overlaps_any(fws, outs, nout)) return ATTN_ERR_INVALID_ARG;
  }

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
  a.rcos = x.rope ? x.rcos : nullptr;
  a.rsin = x.rope ? x.rsin : nullptr;
  a.kr = x.rope ? ws + attn_bwd_gqa_workspace_bytes(B, T, H, H_kv, D) : nullptr;
  a.ve = x.gate ? x.ve : nullptr;
  a.xg = x.xg;
  a.xs = x.xs;
  a.gate_w = x.gate_w;
  a.dve = x.dve;
  a.dxg = x.dxg;
  a.dgate_w = x.dgate_w;
  a.vr = a.gate = a.dz = a.dw_part = nullptr;
  if (x.gate) {
    char* g = ws + attn_bwd_rope_workspace_bytes(B, T, H, H_kv, D);
    a.vr = g;
    g += round_up((size_t)B * T * H_kv * D * 2);
    a.gate = reinterpret_cast<float*>(g);
    g += stats_bytes(B, T, H_kv);
    a.dz = reinterpret_cast<float*>(g);
    g += stats_bytes(B, T, H_kv);
    a.dw_part = reinterpret_cast<float*>(g);
  }
  a.keys_ready = false;
  if (reuse) {   // the forward's key pre-pass, in the forward workspace's layout
    char* f = static_cast<char*>(const_cast<void*>(fwd_ws));
    a.kscale = reinterpret_cast<float*>(f);
    if (x.rope) a.kr = f + attn_fwd_gqa_workspace_bytes(B, T, H, H_kv, D);
    if (x.gate) {
      a.vr = f + attn_fwd_rope_workspace_bytes(B, T, H, H_kv, D);
      a.gate = reinterpret_cast<float*>(static_cast<char*>(a.vr) + round_up((size_t)B * T * H_kv * D * 2));
    }
    a.keys_ready = true;
  }
  a.B = B; a.T = T; a.H = H; a.Hkv = H_kv; a.D = D; a.window = window; a.eps = eps;
  hipError_t e = swattn::launch_bwd(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

Extras rope_extras(const void* rcos, const void* rsin) {
  Extras x;
  x.rope = true;
  x.rcos = rcos;
  x.rsin = rsin;
  return x;
}

Extras gate_extras(const void* ve, const void* xg, int xs, const float* gate_w, const void* rcos,
                   const void* rsin) {
  Extras x;
  x.rope = rcos != nullptr || rsin != nullptr;   // tables optional: both or neither
  x.rcos = rcos;
  x.rsin = rsin;
  x.gate = true;
  x.ve = ve;
  x.xg = xg;
  x.xs = xs;
  x.gate_w = gate_w;
  return x;
}

}  // namespace

extern "C" {

int attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                 void* workspace, size_t workspace_bytes, int B, int T, int H, int H_kv, int D,
                 int window, int causal, float eps, void* stream) {
  return fwd_impl(q, k, v, o, lse, workspace, workspace_bytes, B, T, H, H_kv, D, window, causal, eps,
                  stream, Extras());
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
             size_t workspace_bytes, int B, int T, int H, int D, int window, int causal, float eps,
             void* stream) {
  return fwd_impl(q, k, v, o, lse, workspace, workspace_bytes, B, T, H, H, D, window, causal, eps,
                  stream, Extras());
}

int attn_fwd_rope(const void* q, const void* k, const void* v, const void* rope_cos,
                  const void* rope_sin, void* o, float* lse, void* workspace,
                  size_t workspace_bytes, int B, int T, int H, int H_kv, int D, int window,
                  int causal, float eps, void* stream) {
  return fwd_impl(q, k, v, o, lse, workspace, workspace_bytes, B, T, H, H_kv, D, window, causal, eps,
                  stream, rope_extras(rope_cos, rope_sin));
}

int attn_fwd_ve(const void* q, const void* k, const void* v, const void* ve, const void* xg,
                int xg_stride, const float* gate_w, const void* rope_cos, const void* rope_sin,
                void* o, float* lse, void* workspace, size_t workspace_bytes, int B, int T, int H,
                int H_kv, int D, int window, int causal, float eps, void* stream) {
  return fwd_impl(q, k, v, o, lse, workspace, workspace_bytes, B, T, H, H_kv, D, window, causal, eps,
                  stream, gate_extras(ve, xg, xg_stride, gate_w, rope_cos, rope_sin));
}

int attn_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, void* workspace,
                 size_t workspace_bytes, int B, int T, int H, int H_kv, int D, int window,
                 int causal, float eps, void* stream) {
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, T, H, H_kv, D,
                  window, causal, eps, stream, Extras());
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, void* workspace,
             size_t workspace_bytes, int B, int T, int H, int D, int window, int causal,
             float eps, void* stream) {
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, T, H, H, D,
                  window, causal, eps, stream, Extras());
}

int attn_bwd_rope(const void* q, const void* k, const void* v, const void* rope_cos,
                  const void* rope_sin, const void* o, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B,
                  int T, int H, int H_kv, int D, int window, int causal, float eps,
                  void* stream) {
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, T, H, H_kv, D,
                  window, causal, eps, stream, rope_extras(rope_cos, rope_sin));
}

int attn_bwd_ve(const void* q, const void* k, const void* v, const void* ve, const void* xg,
                int xg_stride, const float* gate_w, const void* rope_cos, const void* rope_sin,
                const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                void* dve, void* dxg, float* dgate_w, void* workspace, size_t workspace_bytes,
                int B, int T, int H, int H_kv, int D, int window, int causal, float eps,
                void* stream) {
  Extras x = gate_extras(ve, xg, xg_stride, gate_w, rope_cos, rope_sin);
  x.dve = dve;
  x.dxg = dxg;
  x.dgate_w = dgate_w;
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, T, H, H_kv, D,
                  window, causal, eps, stream, x);
}

int attn_bwd_gqa_reuse(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, const void* fwd_workspace,
                       size_t fwd_workspace_bytes, void* workspace, size_t workspace_bytes, int B,
                       int T, int H, int H_kv, int D, int window, int causal, float eps,
                       void* stream) {
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, T, H, H_kv, D,
                  window, causal, eps, stream, Extras(), true, fwd_workspace, fwd_workspace_bytes);
}

int attn_bwd_rope_reuse(const void* q, const void* k, const void* v, const void* rope_cos,
                        const void* rope_sin, const void* o, const float* lse, const void* dout,
                        void* dq, void* dk, void* dv, const void* fwd_workspace,
                        size_t fwd_workspace_bytes, void* workspace, size_t workspace_bytes, int B,
                        int T, int H, int H_kv, int D, int window, int causal, float eps,
                        void* stream) {
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, T, H, H_kv, D,
                  window, causal, eps, stream, rope_extras(rope_cos, rope_sin), true, fwd_workspace,
                  fwd_workspace_bytes);
}

int attn_bwd_ve_reuse(const void* q, const void* k, const void* v, const void* ve, const void* xg,
                      int xg_stride, const float* gate_w, const void* rope_cos,
                      const void* rope_sin, const void* o, const float* lse, const void* dout,
                      void* dq, void* dk, void* dv, void* dve, void* dxg, float* dgate_w,
                      const void* fwd_workspace, size_t fwd_workspace_bytes, void* workspace,
                      size_t workspace_bytes, int B, int T, int H, int H_kv, int D, int window,
                      int causal, float eps, void* stream) {
  Extras x = gate_extras(ve, xg, xg_stride, gate_w, rope_cos, rope_sin);
  x.dve = dve;
  x.dxg = dxg;
  x.dgate_w = dgate_w;
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, T, H, H_kv, D,
                  window, causal, eps, stream, x, true, fwd_workspace, fwd_workspace_bytes);
}

}  // extern "C"
