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
//  * V is stored transposed in LDS (written through registers while staging),
//    so the V^T operand is one 16-byte LDS read per MFMA.
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
// Key tiles of BN = 64 rows; each wave forms S^T (64 x 32) in two 32x32 blocks.
template <int D>
struct FwdCfg {
  static constexpr int BM = 128;
  static constexpr int BN = 64;
  static constexpr int KS = D / 16;          // MFMA k-steps over D
  static constexpr int NB = D / 32;          // 32-wide blocks of D in O^T
  static constexpr int KP = D + 8;           // K tile pitch (bf16), rows 16 B apart in bank
  static constexpr int VP = BN + 8;          // V^T tile pitch (bf16)
  static constexpr int K_LDS = BN * KP;      // bf16 elements
  static constexpr int V_LDS = D * VP;
  static constexpr int LDS_BYTES = (K_LDS + V_LDS) * 2 + BN * 4;
  // staging: 256 threads, each 4 x 16 bytes of K and 4 x 16 bytes of V
  static constexpr int CH = D / 8;           // 16-byte chunks per row
};

template <int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ kscale,
    uint16_t* __restrict__ o, float* __restrict__ lse, int T, int H, int W, float eps) {
  using C = FwdCfg<D>;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Vt = Ks + C::K_LDS;
  float* KSs = reinterpret_cast<float*>(Vt + C::V_LDS);

  const int nqt = (T + C::BM - 1) / C::BM;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lid / nqt;
  const int qt = nqt - 1 - (lid % nqt);  // heaviest query tiles of a head first
  const int b = bh / H, h = bh % H;
  const int i0 = qt * C::BM;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const size_t rs = (size_t)H * D;  // row stride (elements) along T
  const size_t base = ((size_t)b * T) * rs + (size_t)h * D;
  const float* ksc = kscale + (size_t)bh * T;

  // ---- query fragment: normalised q row (i0 + 32 w + c), B operand of S^T = K Q^T
  const int qi = i0 + 32 * w + c;
  u32x4 qf[C::KS];
  {
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      qf[ks] = qi < T ? ld16(q + base + (size_t)qi * rs + 16 * ks + 8 * g) : u32x4{0, 0, 0, 0};
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

  // staging assignment
  //  K: thread -> chunk (tid % CH), rows (tid / CH) + (256 / CH) * p
  //  V: thread -> key quad (tid % 16), d-chunk (tid / 16) (for D = 64: rows 2 passes)
  constexpr int KROWS_PER_PASS = 256 / C::CH;
  constexpr int KPASS = C::BN / KROWS_PER_PASS;
  constexpr int VQ = C::BN / 4;                       // 16 key quads
  constexpr int VITEMS = VQ * C::CH;                  // (key quad, d-chunk) items
  constexpr int VPASS = (VITEMS + 255) / 256;
  u32x4 kreg[KPASS];
  u32x4 vreg[VPASS][4];
  float ksreg = 0.f;

  auto load_tile = [&](int jt) {
    const int j0 = jt * C::BN;
#pragma unroll
    for (int p = 0; p < KPASS; ++p) {
      const int r = tid / C::CH + KROWS_PER_PASS * p;
      const int j = j0 + r;
      kreg[p] = j < T ? ld16(k + base + (size_t)j * rs + 8 * (tid % C::CH)) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int p = 0; p < VPASS; ++p) {
      const int idx = tid + 256 * p;
      const int quad = idx % VQ, dch = idx / VQ;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + 4 * quad + e;
        vreg[p][e] = (idx < VITEMS && j < T) ? ld16(v + base + (size_t)j * rs + 8 * dch)
                                             : u32x4{0, 0, 0, 0};
      }
    }
    if (tid < C::BN) {
      const int j = j0 + tid;
      ksreg = j < T ? ksc[j] : 0.f;
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int p = 0; p < KPASS; ++p) {
      const int r = tid / C::CH + KROWS_PER_PASS * p;
      st16(Ks + r * C::KP + 8 * (tid % C::CH), kreg[p]);
    }
#pragma unroll
    for (int p = 0; p < VPASS; ++p) {
      const int idx = tid + 256 * p;
      if (idx >= VITEMS) continue;
      const int quad = idx % VQ, dch = idx / VQ;
      // keys 4 quad .. 4 quad + 3 -> columns tpos16 within their 16-group
      const int col = (quad >> 2) * 16 + tpos16((4 * quad) & 15);
      // transpose 4 keys x 8 d -> 8 rows (d) x 4 keys; dword e of a key row holds
      // d = 8 dch + 2 e (low half) and 8 dch + 2 e + 1 (high half)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t r0 = vreg[p][0][e], r1 = vreg[p][1][e], r2 = vreg[p][2][e], r3 = vreg[p][3][e];
        u32x2 lo = {__builtin_amdgcn_perm(r1, r0, 0x05040100u), __builtin_amdgcn_perm(r3, r2, 0x05040100u)};
        u32x2 hi = {__builtin_amdgcn_perm(r1, r0, 0x07060302u), __builtin_amdgcn_perm(r3, r2, 0x07060302u)};
        st8(Vt + (8 * dch + 2 * e) * C::VP + col, lo);
        st8(Vt + (8 * dch + 2 * e + 1) * C::VP + col, hi);
      }
    }
    if (tid < C::BN) KSs[tid] = ksreg;
  };

  if (jt0 <= jt1) load_tile(jt0);
  for (int jt = jt0; jt <= jt1; ++jt) {
    __syncthreads();  // previous tile fully consumed
    store_tile();
    __syncthreads();
    if (jt < jt1) load_tile(jt + 1);

    const int j0 = jt * C::BN;
    const int cls = tile_class(i0 + 32 * w, i0 + 32 * w + 31, j0, j0 + C::BN - 1, T, W);
    if (cls == TILE_EMPTY) continue;

    // S^T blocks: keys j0 + 32 mb + (8 (r/4) + 4 g + r%4), query qi
    f32x16 st[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      st[mb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        u32x4 a = ld16(Ks + (32 * mb + c) * C::KP + 16 * ks + 8 * g);
        st[mb] = mfma32(a, qf[ks], st[mb]);
      }
    }

    // probabilities (log2 domain, fixed shift), packed to bf16 in MFMA order
    u32x4 pf[4];  // k-steps of 16 keys: (mb, half)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int jl = 32 * mb + 8 * q4 + 4 * g;     // local key of r = 4 q4
        f32x4 ks4 = *reinterpret_cast<const f32x4*>(KSs + jl);
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = st[mb][4 * q4 + e] * ks4[e] - shift;
          float pe = __builtin_amdgcn_exp2f(x);
          if (cls == TILE_PARTIAL && !visible(qi, j0 + jl + e, T, W)) pe = 0.f;
          p[e] = pe;
        }
        // register r = 4 q4 + e; k-step half = q4 / 2, element j = 4 (q4 % 2) + e
        const uint32_t p01 = pack_bf16(p[0], p[1]), p23 = pack_bf16(p[2], p[3]);
        pf[2 * mb + (q4 >> 1)][2 * (q4 & 1) + 0] = p01;
        pf[2 * mb + (q4 >> 1)][2 * (q4 & 1) + 1] = p23;
        // the row sum adds the bf16-rounded probabilities the PV product uses,
        // so the output weights sum to one (W = 0 gives o = v exactly)
        lsum = sum_bf16x2(p01, lsum);
        lsum = sum_bf16x2(p23, lsum);
      }
    }

    // O^T[d, q] += V^T[d, keys] P^T[keys, q]
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int n = 0; n < C::NB; ++n) {
        u32x4 a = ld16(Vt + (32 * n + c) * C::VP + 16 * s + 8 * g);
        acc_o[n] = mfma32(a, pf[s], acc_o[n]);
      }
    }
  }

  // ---- epilogue: O = O^T / l, lse = shift + ln l
  lsum += __shfl_xor(lsum, 32);
  const float inv = 1.0f / lsum;
  if (qi < T) {
    uint16_t* orow = o + base + (size_t)qi * rs;
#pragma unroll
    for (int n = 0; n < C::NB; ++n)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * n + 8 * q4 + 4 * g;
        u32x2 val = {pack_bf16(acc_o[n][4 * q4 + 0] * inv, acc_o[n][4 * q4 + 1] * inv),
                     pack_bf16(acc_o[n][4 * q4 + 2] * inv, acc_o[n][4 * q4 + 3] * inv)};
        st8(orow + d, val);
      }
    if (g == 0) lse[(size_t)bh * T + qi] = sqrtf((float)D) + __logf(lsum);
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
