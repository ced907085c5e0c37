// Forward pass: RMSNorm of Q and K, causal sliding-window attention, O and the
// logsumexp of the scaled logits.
//
// What is computed (per batch b, head h, query i):
//   q_hat = q * r_q,  k_hat = k * r_k,  r = 1 / sqrt(mean_d x^2 + eps)
//       (RMSNorm with unit gain on queries and keys right before the attention
//        product: okx.com line-by-line review of karpathy/autoresearch, the
//        QK-norm paragraph; "Autoresearch 深度教程" §7.3, the `norm` helper)
//   s_ij = q_hat_i . k_hat_j / sqrt(D) for the keys of the (W, 0) window
//       ("Autoresearch 深度教程" §5.2.2; FlashAttention-3 call of §5.2.1)
//   o_i = softmax_j(s_ij) v,   lse_i = ln sum_j exp(s_ij)
//
// MI355X design:
//  * QK-norm bounds every logit: |s_ij| <= |q_hat||k_hat|/sqrt(D) < sqrt(D).
//    The softmax therefore uses the fixed shift sqrt(D) instead of a running
//    row maximum: exp(s - sqrt(D)) lies in [exp(-2 sqrt(D)), ~1], far from fp32
//    overflow and underflow.  No row-max reduction and no rescaling of the
//    output accumulator are needed; lse = sqrt(D) + ln(sum).
//  * r_k is applied after the MFMA: the kernel multiplies raw bf16 K tiles with
//    the normalised query and scales each logit by kscale_j = log2(e) r_k / sqrt(D)
//    (one pre-pass over K writes kscale), so no workgroup re-normalises K.
//  * S^T = K Q^T is formed on the 32x32x16 bf16 MFMA so that each lane owns one
//    query column: its probabilities are already in the B-operand layout of the
//    next product O^T = V^T P^T, and row sums are lane-local.
//  * K and V tiles stay row-major in LDS (double-buffered; one barrier per
//    tile); the V^T operand of the PV product comes from the gfx950
//    transposing LDS read (ds_read_b64_tr_b16), two per MFMA.
//  * Loads go through buffer descriptors rebased per tile: rows past T read as
//    zero, so ragged tails need no branches; stores past T are dropped.
//  * Band-aware tile loop: a query tile visits only the key tiles that
//    intersect its window; fully visible tiles skip the mask.
#include "common.h"
#include "band.h"
#include "kernels.h"
#include "profile.h"

namespace swattn {

// ------------------------------------------------------------ kscale pre-pass
// kscale[b, h, t] = log2(e) / sqrt(D) * r(k[b, t, h, :]).  Rows of K are
// contiguous in [B, T, H, D]; D / 8 lanes share one row (16 bytes each).
template <int D>
__global__ __launch_bounds__(256) void k_scale_kernel(const uint16_t* __restrict__ k,
                                                      float* __restrict__ kscale, int nrows,
                                                      int T, int H, float eps) {
  constexpr int LPR = D / 8;  // lanes per row
  const int tid = blockIdx.x * 256 + threadIdx.x;
  const int row = tid / LPR;
  const int part = tid % LPR;
  float ss = 0.f;
  if (row < nrows) {
    u32x4 v = ld16(k + (size_t)row * D + part * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float a = bf_lo(v[e]), b = bf_hi(v[e]);
      ss += a * a + b * b;
    }
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, LPR);
  if (row < nrows && part == 0) {
    const int h = row % H;
    const int bt = row / H;
    const int t = bt % T;
    const int b = bt / T;
    float r = 1.0f / sqrtf(ss * (1.0f / D) + eps);
    kscale[((size_t)b * H + h) * T + t] = r * (kLog2e / sqrtf((float)D));
  }
}

// ------------------------------------------------------------ forward kernel
// Workgroup: 4 waves; wave w owns query rows i0 + 32 w .. i0 + 32 w + 31.
// Key tiles of BN = 64 rows, double-buffered in LDS; each wave forms S^T
// (64 keys x 32 queries) in two 32x32 blocks, then O^T += V^T P^T.
template <int D>
struct FwdCfg {
  static constexpr int BM = 128;
  static constexpr int BN = 64;
  static constexpr int KS = D / 16;          // MFMA k-steps over D
  static constexpr int NB = D / 32;          // 32-wide blocks of D in O^T
  static constexpr int KP = D + 8;           // K row pitch (bf16): 16-byte reads of 8 rows hit 8 bank groups
  static constexpr int VP = D + 16;          // V row pitch (bf16): transposed reads of 4 rows hit 4 bank groups
  static constexpr int K_LDS = BN * KP;
  static constexpr int V_LDS = BN * VP;
  static constexpr int STAGE = (K_LDS + V_LDS) * 2 + BN * 4;   // bytes of one buffer
  static constexpr int LDS_BYTES = 2 * STAGE;
  static constexpr int CH = D / 8;           // 16-byte chunks per row
  static constexpr int RPP = 256 / CH;       // rows staged per pass
  static constexpr int PASSES = BN / RPP;
};

template <int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ kscale,
    uint16_t* __restrict__ o, float* __restrict__ lse, int T, int H, int W, float eps) {
  using C = FwdCfg<D>;
  extern __shared__ __align__(16) unsigned char smem[];

  const int nqt = (T + C::BM - 1) / C::BM;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lid / nqt;
  const int qt = nqt - 1 - (lid % nqt);  // heaviest query tiles of a head first
  const int b = bh / H, h = bh % H;
  const int i0 = qt * C::BM;

  const int tid = threadIdx.x;
  const int w = uniform(tid >> 6);
  const int lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int rs = H * D;                                   // row stride (elements) along T
  const long long rsb = 2LL * rs;                         // ... in bytes
  const long long slice_bytes = (long long)(T - 1) * rsb + 2 * D;
  const size_t sbase = ((size_t)b * T * H + h) * D;       // element offset of row 0 of the slice
  const uint16_t* qs = q + sbase;
  const uint16_t* ksl = k + sbase;
  const uint16_t* vsl = v + sbase;

  // ---- query fragment: normalised q row (i0 + 32 w + c), B operand of S^T = K Q^T
  const int qw0 = i0 + 32 * w;
  const int qi = qw0 + c;
  u32x4 qf[C::KS];
  {
    const rsrc_t rq = make_rsrc(qs + (size_t)qw0 * rs, slice_bytes - qw0 * rsb);
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      qf[ks] = bload16(rq, (c * rs + 16 * ks + 8 * g) * 2);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float a = bf_lo(qf[ks][e]), bb = bf_hi(qf[ks][e]);
        ss += a * a + bb * bb;
      }
    }
    ss += __shfl_xor(ss, 32);
    const float r = 1.0f / sqrtf(ss * (1.0f / D) + eps);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[ks][e] = pack_bf16(bf_lo(qf[ks][e]) * r, bf_hi(qf[ks][e]) * r);
  }

  f32x16 acc_o[C::NB];
#pragma unroll
  for (int n = 0; n < C::NB; ++n) acc_o[n] = f32x16{};
  float lsum = 0.f;
  const float shift = sqrtf((float)D) * kLog2e;  // fixed softmax shift, log2 units

  int kv_lo, kv_hi;
  kv_range(i0, i0 + C::BM - 1, T, W, &kv_lo, &kv_hi);
  const int jt0 = kv_lo / C::BN, jt1 = kv_hi / C::BN;

  // staging: thread -> rows tid / CH + RPP p, 16-byte chunk tid % CH (K and V alike)
  const int srow = tid / C::CH, sch = tid % C::CH;
  u32x4 kreg[C::PASSES], vreg[C::PASSES];
  float ksreg = 0.f;
  const rsrc_t rks = make_rsrc(kscale + (size_t)bh * T, 4LL * T);

  auto load_tile = [&](int jt) {
    const int j0 = jt * C::BN;
    const rsrc_t rk = make_rsrc(ksl + (size_t)j0 * rs, slice_bytes - j0 * rsb);
    const rsrc_t rv = make_rsrc(vsl + (size_t)j0 * rs, slice_bytes - j0 * rsb);
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p) {
      const int off = ((srow + C::RPP * p) * rs + 8 * sch) * 2;
      kreg[p] = bload16(rk, off);
      vreg[p] = bload16(rv, off);
    }
    if (tid < C::BN) ksreg = bload4f(rks, (j0 + tid) * 4);
  };
  auto store_tile = [&](int buf) {
    uint16_t* Ks = reinterpret_cast<uint16_t*>(smem + buf * C::STAGE);
    uint16_t* Vs = Ks + C::K_LDS;
    float* KSs = reinterpret_cast<float*>(Vs + C::V_LDS);
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p) {
      st16(Ks + (srow + C::RPP * p) * C::KP + 8 * sch, kreg[p]);
      st16(Vs + (srow + C::RPP * p) * C::VP + 8 * sch, vreg[p]);
    }
    if (tid < C::BN) KSs[tid] = ksreg;
  };

  // per-lane LDS offsets of the MFMA operands
  const int k_off = c * C::KP + 8 * g;                                  // K rows, 16-byte reads
  const int li = lane & 15;
  const int v_off = (4 * g + (li >> 2)) * C::VP + 16 * ((lane >> 4) & 1) + 4 * (li & 3);  // V^T via tr reads

  if (jt0 <= jt1) {
    load_tile(jt0);
    store_tile(0);
  }
  __syncthreads();
  for (int jt = jt0; jt <= jt1; ++jt) {
    const int buf = (jt - jt0) & 1;
    if (jt < jt1) load_tile(jt + 1);

    const int j0 = jt * C::BN;
    const int cls = uniform(tile_class(qw0, qw0 + 31, j0, j0 + C::BN - 1, T, W));
    if (cls != TILE_EMPTY) {
      const uint16_t* Ks = reinterpret_cast<const uint16_t*>(smem + buf * C::STAGE);
      const uint16_t* Vs = Ks + C::K_LDS;
      const float* KSs = reinterpret_cast<const float*>(Vs + C::V_LDS);

      // S^T blocks: keys j0 + 32 mb + (8 (r/4) + 4 g + r%4), query qi
      f32x16 st[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        st[mb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
          st[mb] = mfma32(ld16(Ks + k_off + 32 * mb * C::KP + 16 * ks), qf[ks], st[mb]);
      }

      // probabilities (log2 domain, fixed shift), packed to bf16 in MFMA k order
      u32x4 pf[4];
      const int t0 = j0 + 4 * g + W - qi;   // key kv visible iff 0 <= kv - (qi - W) <= W
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int jl = 32 * mb + 8 * q4 + 4 * g;
          const f32x4 ks4 = *reinterpret_cast<const f32x4*>(KSs + jl);
          float p[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(st[mb][4 * q4 + e] * ks4[e] - shift);
          if (cls == TILE_PARTIAL) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              p[e] = ((unsigned)(t0 + 32 * mb + 8 * q4 + e) <= (unsigned)W) ? p[e] : 0.f;
          }
          const uint32_t p01 = pack_bf16(p[0], p[1]), p23 = pack_bf16(p[2], p[3]);
          pf[2 * mb + (q4 >> 1)][2 * (q4 & 1) + 0] = p01;
          pf[2 * mb + (q4 >> 1)][2 * (q4 & 1) + 1] = p23;
          // the row sum adds the bf16-rounded probabilities the PV product uses,
          // so the output weights sum to one (W = 0 gives o = v exactly)
          lsum = sum_bf16x2(p01, lsum);
          lsum = sum_bf16x2(p23, lsum);
        }
      }

      // O^T[d, q] += V^T[d, keys] P^T[keys, q]; key k-order matches pf:
      // element j of k-step s is key 16 s + 4 g + (j % 4) + 8 (j / 4)
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
#pragma unroll
        for (int n = 0; n < C::NB; ++n) {
          const u32x2 lo = lds_tr4(Vs + v_off + 16 * s2 * C::VP + 32 * n);
          const u32x2 hi = lds_tr4(Vs + v_off + (16 * s2 + 8) * C::VP + 32 * n);
          acc_o[n] = mfma32(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf[s2], acc_o[n]);
        }
      }
    }
    if (jt < jt1) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, lse = shift + ln l  (stores past T are dropped)
  lsum += __shfl_xor(lsum, 32);
  const float inv = 1.0f / lsum;
  const rsrc_t ro = make_rsrc(o + sbase + (size_t)qw0 * rs, slice_bytes - qw0 * rsb);
#pragma unroll
  for (int n = 0; n < C::NB; ++n)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * n + 8 * q4 + 4 * g;
      const u32x2 val = {pack_bf16(acc_o[n][4 * q4 + 0] * inv, acc_o[n][4 * q4 + 1] * inv),
                         pack_bf16(acc_o[n][4 * q4 + 2] * inv, acc_o[n][4 * q4 + 3] * inv)};
      bstore8(val, ro, (c * rs + d) * 2);
    }
  if (g == 0) {
    const rsrc_t rl = make_rsrc(lse + (size_t)bh * T, 4LL * T);
    bstore4f(sqrtf((float)D) + __logf(lsum), rl, qi * 4);
  }
}

template <int D>
static hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t stream) {
  using C = FwdCfg<D>;
  const int nrows = a.B * a.T * a.H;
  const int lpr = D / 8;
  const int nblk_s = (int)(((long long)nrows * lpr + 255) / 256);
  ProfToken t0 = prof_begin(K_SCALE, stream);
  hipLaunchKernelGGL(k_scale_kernel<D>, dim3(nblk_s), dim3(256), 0, stream,
                     (const uint16_t*)a.k, a.kscale, nrows, a.T, a.H, a.eps);
  prof_end(t0);
  const int nqt = (a.T + C::BM - 1) / C::BM;
  const int nblk = nqt * a.B * a.H;
  const int W = eff_window(a.T, a.window);
  // more than 64 KiB of dynamic LDS must be opted into, once per kernel
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(attn_fwd_kernel<D>),
      hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  ProfToken t1 = prof_begin(K_FWD, stream);
  hipLaunchKernelGGL(attn_fwd_kernel<D>, dim3(nblk), dim3(256), C::LDS_BYTES, stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (const float*)a.kscale, (uint16_t*)a.o, a.lse, a.T, a.H, W, a.eps);
  prof_end(t1);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  if (a.D == 128) return launch_fwd_d<128>(a, stream);
  return launch_fwd_d<64>(a, stream);
}

}  // namespace swattn
