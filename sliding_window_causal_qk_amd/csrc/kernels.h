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
  void* vt;       // workspace: bf16 [B, Hkv, D, LT], V transposed, keys permuted (tpos16)
  int LT;         // row length of vt: T rounded up to a multiple of 64
  const void* rcos;  // bf16 [T, D/2] rotary tables, or null: no rotary embedding
  const void* rsin;
  void* kr;          // workspace (rotary only): bf16 [B, T, Hkv, D], the rotated keys
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
  int B, T, H, D;
  int Hkv;        // key/value heads (H is a multiple); k, v, dk, dv have Hkv heads
  int window;
  float eps;
};

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);

}  // namespace swattn
