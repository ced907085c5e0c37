// Key-side pre-pass shared by the forward and the backward: per key row, the
// logit scale of the RMSNorm of K and, with the rotary embedding or the
// value-embedding gate, the rotated keys and the gated values that the
// attention kernels read.
#include "common.h"
#include "kernels.h"
#include "profile.h"

namespace swattn {

// ------------------------------------------------------------------ key rows
// kscale[b, h, t] = log2(e) / sqrt(D) * r(k[b, t, h, :]) for the attention
// kernels (H here is the number of key/value heads).  D / 8 lanes share one
// key row (16 bytes each); a thread handles KR rows 256 / (D / 8) apart, so
// each has KR loads in flight.
// ROPE: the rows are rotated first (a lane's rotation partner is the lane
// D / 16 away) and written to kr, the K of the attention kernels; kscale is
// taken from the rotated bf16 rows.
// VE: the same pass writes vr = v + gate ve (the V of the attention kernels)
// and, when gate_out is not null, the gate of every key,
// gate = 2 sigmoid(W_g x[:32]).
template <int D, bool ROPE, bool VE>
__global__ __launch_bounds__(256) void key_prep_kernel(const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ rcos,
                                                       const uint16_t* __restrict__ rsin,
                                                       const uint16_t* __restrict__ v,
                                                       const uint16_t* __restrict__ ve,
                                                       const uint16_t* __restrict__ xg, int xs,
                                                       const float* __restrict__ gate_w,
                                                       float* __restrict__ kscale,
                                                       uint16_t* __restrict__ kr,
                                                       uint16_t* __restrict__ vr,
                                                       float* __restrict__ gate_out, int nrows,
                                                       int T, int H, float eps) {
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;     // rows per block pass
  constexpr int KR = 4;
  const int part = threadIdx.x % LPR;
  const int rb = blockIdx.x * RPB * KR;   // first row of the block
  const int row0 = rb + threadIdx.x / LPR;
  // descriptor from the block's first row: rows past nrows read as zero
  const rsrc_t rk = make_rsrc(k + (size_t)rb * D, (long long)(nrows - rb) * D * 2);
  u32x4 kv[KR];
#pragma unroll
  for (int i = 0; i < KR; ++i) kv[i] = bload16(rk, ((threadIdx.x / LPR + RPB * i) * D + part * 8) * 2);
  if constexpr (VE) {
    const rsrc_t rv = make_rsrc(v + (size_t)rb * D, (long long)(nrows - rb) * D * 2);
    const rsrc_t rve = make_rsrc(ve + (size_t)rb * D, (long long)(nrows - rb) * D * 2);
    const rsrc_t rvr = make_rsrc(vr + (size_t)rb * D, (long long)(nrows - rb) * D * 2);
#pragma unroll
    for (int i = 0; i < KR; ++i) {
      const int row = row0 + RPB * i;   // (b T + t) H + h
      const bool ok = row < nrows;
      const int hk = row % H, bt = row / H;
      const float gate = ve_gate_sum<LPR>(xg + (size_t)(ok ? bt : 0) * xs, gate_w + hk * 32, part, ok);
      const int off = ((threadIdx.x / LPR + RPB * i) * D + part * 8) * 2;
      u32x4 vv = bload16(rv, off);
      const u32x4 ee = bload16(rve, off);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        vv[e] = pack_bf16(bf_lo(vv[e]) + gate * bf_lo(ee[e]), bf_hi(vv[e]) + gate * bf_hi(ee[e]));
      bstore16(vv, rvr, off);
      if (gate_out && ok && part == 0) {
        const int t = bt % T, b = bt / T;
        gate_out[((size_t)b * H + hk) * T + t] = gate;
      }
    }
  }
  if constexpr (ROPE) {
    const rsrc_t rc = make_rsrc(rcos, (long long)T * D), rn = make_rsrc(rsin, (long long)T * D);
    const rsrc_t rkr = make_rsrc(kr + (size_t)rb * D, (long long)(nrows - rb) * D * 2);
    const bool second = part >= LPR / 2;   // this lane holds second-half channels
#pragma unroll
    for (int i = 0; i < KR; ++i) {
      const int t = ((row0 + RPB * i) / H) % T;
      const int off = (t * (D / 2) + 8 * (part % (LPR / 2))) * 2;
      u32x4 other;
#pragma unroll
      for (int e = 0; e < 4; ++e) other[e] = __shfl_xor(kv[i][e], LPR / 2);
      float y1[8], y2[8];
      rope8(second ? other : kv[i], second ? kv[i] : other, bload16(rc, off), bload16(rn, off), y1, y2);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        kv[i][e] = second ? pack_bf16(y2[2 * e], y2[2 * e + 1]) : pack_bf16(y1[2 * e], y1[2 * e + 1]);
      bstore16(kv[i], rkr, ((threadIdx.x / LPR + RPB * i) * D + part * 8) * 2);
    }
  }
  // The block's RPB * KR scales go out through LDS, one row per thread of its
  // first RPB * KR threads: the rows of one key/value head are consecutive
  // positions, so a wave's stores form runs of neighbouring words instead of
  // one isolated word per row.
  __shared__ float ks[RPB * KR];
#pragma unroll
  for (int i = 0; i < KR; ++i) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = bf_lo(kv[i][e]), b = bf_hi(kv[i][e]);
      ss += a * a + b * b;
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, LPR);
    if (part == 0) ks[threadIdx.x / LPR + RPB * i] = (1.0f / sqrtf(ss * (1.0f / D) + eps)) * (kLog2e / sqrtf((float)D));
  }
  __syncthreads();
  const int row = rb + threadIdx.x;
  if (threadIdx.x < RPB * KR && row < nrows) {
    const int h = row % H, bt = row / H, t = bt % T, b = bt / T;
    kscale[((size_t)b * H + h) * T + t] = ks[threadIdx.x];
  }
}

template <int D, bool ROPE, bool VE>
static void launch_key_prep_d(const KeyPrepArgs& a, hipStream_t stream) {
  const int nrows = a.B * a.T * a.Hkv;
  const int nblk = (int)(((long long)nrows * (D / 8) + 4 * 256 - 1) / (4 * 256));
  hipLaunchKernelGGL((key_prep_kernel<D, ROPE, VE>), dim3(nblk), dim3(256), 0, stream,
                     (const uint16_t*)a.k, (const uint16_t*)a.rcos, (const uint16_t*)a.rsin,
                     (const uint16_t*)a.v, (const uint16_t*)a.ve, (const uint16_t*)a.xg, a.xs, a.gate_w,
                     a.kscale, (uint16_t*)a.kr, (uint16_t*)a.vr, a.gate, nrows, a.T, a.Hkv, a.eps);
}

template <int D>
static void launch_key_prep_dd(const KeyPrepArgs& a, hipStream_t stream) {
  const bool rope = a.rcos != nullptr, ve = a.ve != nullptr;
  if (rope) {
    if (ve) launch_key_prep_d<D, true, true>(a, stream);
    else launch_key_prep_d<D, true, false>(a, stream);
  } else {
    if (ve) launch_key_prep_d<D, false, true>(a, stream);
    else launch_key_prep_d<D, false, false>(a, stream);
  }
}

hipError_t launch_key_prep(const KeyPrepArgs& a, int prof_kernel, hipStream_t stream) {
  ProfToken t = prof_begin(prof_kernel, stream);
  if (a.D == 256) launch_key_prep_dd<256>(a, stream);
  else if (a.D == 128) launch_key_prep_dd<128>(a, stream);
  else launch_key_prep_dd<64>(a, stream);
  prof_end(t);
  return hipGetLastError();
}

}  // namespace swattn
