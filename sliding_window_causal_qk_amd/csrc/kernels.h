// Internal launch interface between the C-ABI host code and the kernels.
// Arguments are validated by the caller (swattn.hip) before any launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace swattn {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* kscale;  // workspace: [B, Hkv, T]
  const void* rcos;  // bf16 [T, D/2] rotary tables, or null: no rotary embedding
  const void* rsin;
  void* kr;          // workspace (rotary only): bf16 [B, T, Hkv, D], the rotated keys
  void* vr;          // workspace (gate only): bf16 [B, T, Hkv, D], v + gate ve
  float* gate;       // workspace (gate only): [B, Hkv, T], kept for a backward that reuses it
  const void* ve;    // bf16 [B, T, Hkv, D] value embedding, or null: no gate
  const void* xg;    // bf16 gate input: token (b, t) at xg + (b T + t) xs, channels 0..31
  int xs;
  const float* gate_w;  // fp32 [Hkv, 32]
  int B, T, H, D;
  int Hkv;        // key/value heads (H is a multiple); q, o: H heads, k, v: Hkv
  int window;
  float eps;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  // workspace carve-up
  void* qhat;     // bf16 [B, T, H, D]: normalised queries
  float* kscale;  // [B, Hkv, T]: log2(e) / sqrt(D) / rms(k)
  float* delta;   // [B, H, T]: rowsum(dO * O)
  float* lse2;    // [B, H, T]: lse * log2(e)
  const void* rcos;  // bf16 [T, D/2] rotary tables, or null: no rotary embedding
  const void* rsin;
  void* kr;          // workspace (rotary only): bf16 [B, T, Hkv, D], the rotated keys
  // value-embedding gate (ve null: none)
  const void* ve;    // bf16 [B, T, Hkv, D]
  const void* xg;    // bf16 gate input: token (b, t) at xg + (b T + t) xs, channels 0..31
  int xs;
  const float* gate_w;  // fp32 [Hkv, 32]
  void* dve;         // bf16 [B, T, Hkv, D]
  void* dxg;         // bf16 [B, T, 32]
  float* dgate_w;    // fp32 [Hkv, 32]
  void* vr;          // workspace: bf16 [B, T, Hkv, D], v + gate ve
  float* gate;       // workspace: [B, Hkv, T]
  float* dz;         // workspace: [B, T, Hkv], gradient of the gate's pre-sigmoid input
  float* dw_part;    // workspace: [ceil(B T / kGateTokens), Hkv, 32], per-block partial sums of dgate_w
  bool keys_ready;   // kscale, kr, vr and gate already hold the forward's key pre-pass
  int B, T, H, D;
  int Hkv;        // key/value heads (H is a multiple); k, v, dk, dv have Hkv heads
  int window;
  float eps;
};

// (batch, head) slices per group of the query-tiled kernels' heaviest-first
// order (see query_tile_of); measured best on the SSSL stack's layers.  dQ
// takes wider groups when its grid is at most kDqFewWaves times the
// workgroups the CUs hold at once: measured faster on the B = 8 layers (by
// 16% at W = 2048) and on the T = 8192 stack, slower (2%) at eight times.
constexpr int kTileGroupFwd = 4;
constexpr int kTileGroupDq = 2;
constexpr int kTileGroupDqFew = 4;
constexpr int kDqFewWaves = 4;

// tokens per block of the first pass of the gate's weight-gradient reduction
constexpr int kGateTokens = 64;

// The key-side pre-pass of both passes (prep.hip): kscale, and the rotated
// keys (rcos not null) and gated values (ve not null) the attention kernels
// read.  gate may be null (the forward does not keep it).
struct KeyPrepArgs {
  const void* k;
  const void* v;
  const void* rcos;
  const void* rsin;
  const void* ve;
  const void* xg;
  int xs;
  const float* gate_w;
  float* kscale;
  void* kr;
  void* vr;
  float* gate;
  int B, T, Hkv, D;
  float eps;
};

hipError_t launch_key_prep(const KeyPrepArgs& a, int prof_kernel, hipStream_t stream);
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);
// The dQ kernel of the backward (attn_bwd_dq.hip), launched by launch_bwd
// first: kk, vv are the keys and values the products read (rotated keys, gated
// values), W the window as eff_window gives it, ncu the device's CU count.
hipError_t launch_bwd_dq(const BwdArgs& a, const uint16_t* kk, const uint16_t* vv, int W, int ncu,
                         hipStream_t stream);

}  // namespace swattn
