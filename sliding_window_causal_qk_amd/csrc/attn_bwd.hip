// Backward pass of QK-RMSNorm causal sliding-window attention: dQ, dK, dV with
// respect to the pre-norm q, k and v, recomputing the probabilities from the
// saved logsumexp.
//
// Chain rule through the forward of attn_fwd.hip (per batch b, head h):
//   P_ij  = exp(s_ij - lse_i)              (recomputed; masked pairs are 0)
//   dV    = P^T dO
//   dP    = dO V^T,   Delta_i = dO_i . o_i
//   dS    = P * (dP - Delta)
//   dq_hat = dS k_hat / sqrt(D),  dk_hat = dS^T q_hat / sqrt(D)
//   dx    = r (dx_hat - x_hat mean_d(dx_hat x_hat))   for x in {q, k}
//       (gradient of the unit-gain RMSNorm that the okx.com review and
//        "Autoresearch 深度教程" §7.3 place on q and k before the product)
//
// Kernels:
//   bwd_prep:  Delta, r_q, q_hat (bf16, to the workspace) and kscale for K.
//   bwd_dkdv:  a workgroup owns 128 keys (32 per wave) and walks the query
//              blocks of its band; dV^T and dK_hat^T stay in registers; the
//              RMSNorm backward of K runs in the epilogue.
//   bwd_dq:    a workgroup owns 128 queries (32 per wave) and walks the key
//              tiles of its band, recomputing S and dP; the RMSNorm backward
//              of Q runs in the epilogue.  No atomics: dQ is deterministic.
#include "common.h"
#include "band.h"
#include "kernels.h"
#include "profile.h"

namespace swattn {

// ------------------------------------------------------------------ prep
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
    uint16_t* __restrict__ qhat, float* __restrict__ rq, float* __restrict__ kscale,
    float* __restrict__ delta, int nrows, int T, int H, float eps) {
  constexpr int LPR = D / 8;
  const int tid = blockIdx.x * 256 + threadIdx.x;
  const int row = tid / LPR;
  const int part = tid % LPR;
  float ssq = 0.f, ssk = 0.f, dot = 0.f;
  u32x4 qv = {0, 0, 0, 0};
  if (row < nrows) {
    const size_t off = (size_t)row * D + part * 8;
    qv = ld16(q + off);
    u32x4 kv = ld16(k + off), ov = ld16(o + off), dv = ld16(dout + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float a = bf_lo(qv[e]), b = bf_hi(qv[e]);
      ssq += a * a + b * b;
      a = bf_lo(kv[e]); b = bf_hi(kv[e]);
      ssk += a * a + b * b;
      dot += bf_lo(ov[e]) * bf_lo(dv[e]) + bf_hi(ov[e]) * bf_hi(dv[e]);
    }
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) {
    ssq += __shfl_xor(ssq, m, LPR);
    ssk += __shfl_xor(ssk, m, LPR);
    dot += __shfl_xor(dot, m, LPR);
  }
  if (row < nrows) {
    const float r = 1.0f / sqrtf(ssq * (1.0f / D) + eps);
    u32x4 qh;
#pragma unroll
    for (int e = 0; e < 4; ++e) qh[e] = pack_bf16(bf_lo(qv[e]) * r, bf_hi(qv[e]) * r);
    st16(qhat + (size_t)row * D + part * 8, qh);
    if (part == 0) {
      const int h = row % H;
      const int bt = row / H;
      const int t = bt % T;
      const int b = bt / T;
      const size_t s = ((size_t)b * H + h) * T + t;
      rq[s] = r;
      kscale[s] = (1.0f / sqrtf(ssk * (1.0f / D) + eps)) * (kLog2e / sqrtf((float)D));
      delta[s] = dot;
    }
  }
}

// Shared staging helper: 4 consecutive rows x one 16-byte chunk per item.
// Writes the rows row-major (pitch RP) and, optionally, transposed (pitch TP)
// with the tpos16 column order the MFMA k-steps read.
template <int D, int ROWS>
struct Stage {
  static constexpr int CH = D / 8;
  static constexpr int QUADS = ROWS / 4;
  static constexpr int ITEMS = QUADS * CH;
  static constexpr int PASS = (ITEMS + 255) / 256;

  u32x4 r[PASS][4];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, size_t base, size_t rs,
                                       int row0, int T, int tid) {
#pragma unroll
    for (int p = 0; p < PASS; ++p) {
      const int idx = tid + 256 * p;
      const int quad = idx % QUADS, dch = idx / QUADS;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = row0 + 4 * quad + e;
        r[p][e] = (idx < ITEMS && t < T) ? ld16(src + base + (size_t)t * rs + 8 * dch)
                                         : u32x4{0, 0, 0, 0};
      }
    }
  }

  template <bool ROWMAJOR, bool TRANS>
  __device__ __forceinline__ void store(uint16_t* rowmaj, int RP, uint16_t* trans, int TP,
                                        int tid) const {
#pragma unroll
    for (int p = 0; p < PASS; ++p) {
      const int idx = tid + 256 * p;
      if (idx >= ITEMS) continue;
      const int quad = idx % QUADS, dch = idx / QUADS;
      if (ROWMAJOR) {
#pragma unroll
        for (int e = 0; e < 4; ++e) st16(rowmaj + (4 * quad + e) * RP + 8 * dch, r[p][e]);
      }
      if (TRANS) {
        const int col = (quad >> 2) * 16 + tpos16((4 * quad) & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t r0 = r[p][0][e], r1 = r[p][1][e], r2 = r[p][2][e], r3 = r[p][3][e];
          u32x2 lo = {__builtin_amdgcn_perm(r1, r0, 0x05040100u), __builtin_amdgcn_perm(r3, r2, 0x05040100u)};
          u32x2 hi = {__builtin_amdgcn_perm(r1, r0, 0x07060302u), __builtin_amdgcn_perm(r3, r2, 0x07060302u)};
          st8(trans + (8 * dch + 2 * e) * TP + col, lo);
          st8(trans + (8 * dch + 2 * e + 1) * TP + col, hi);
        }
      }
    }
  }
};

// ------------------------------------------------------------------ dK / dV
template <int D>
struct DkdvCfg {
  static constexpr int BNK = 128;       // keys per workgroup (32 per wave)
  static constexpr int BMQ = 64;        // queries per step
  static constexpr int KS = D / 16;
  static constexpr int NB = D / 32;
  static constexpr int RP = D + 8;      // row-major pitch
  static constexpr int TP = BMQ + 8;    // transposed pitch
  static constexpr int Q_LDS = BMQ * RP;
  static constexpr int QT_LDS = D * TP;
  static constexpr int LDS_BYTES = (2 * Q_LDS + 2 * QT_LDS) * 2 + 2 * BMQ * 4;
};

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ qhat, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta,
    const float* __restrict__ kscale, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
    int T, int H, int W) {
  using C = DkdvCfg<D>;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* Qs = reinterpret_cast<uint16_t*>(smem);
  uint16_t* dOs = Qs + C::Q_LDS;
  uint16_t* QTs = dOs + C::Q_LDS;
  uint16_t* dOTs = QTs + C::QT_LDS;
  float* Ls = reinterpret_cast<float*>(dOTs + C::QT_LDS);
  float* Dls = Ls + C::BMQ;

  const int nkt = (T + C::BNK - 1) / C::BNK;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lid / nkt;
  const int kt = lid % nkt;  // causal: the first key blocks see the most queries
  const int b = bh / H, h = bh % H;
  const int j0 = kt * C::BNK;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const size_t rs = (size_t)H * D;
  const size_t base = ((size_t)b * T) * rs + (size_t)h * D;
  const size_t sb = (size_t)bh * T;

  // ---- owned key / value rows (kv = j0 + 32 w + c), B operands of S and dP
  const int kj = j0 + 32 * w + c;
  u32x4 kf[C::KS], vf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    kf[ks] = kj < T ? ld16(k + base + (size_t)kj * rs + 16 * ks + 8 * g) : u32x4{0, 0, 0, 0};
    vf[ks] = kj < T ? ld16(v + base + (size_t)kj * rs + 16 * ks + 8 * g) : u32x4{0, 0, 0, 0};
  }
  const float ksc = kj < T ? kscale[sb + kj] : 0.f;

  f32x16 acc_dv[C::NB], acc_dk[C::NB];
#pragma unroll
  for (int n = 0; n < C::NB; ++n) { acc_dv[n] = f32x16{}; acc_dk[n] = f32x16{}; }

  int q_lo, q_hi;
  const bool any = q_range(j0, j0 + C::BNK - 1, T, W, &q_lo, &q_hi);
  const int qb0 = any ? q_lo / C::BMQ : 0, qb1 = any ? q_hi / C::BMQ : -1;

  Stage<D, C::BMQ> sq, sdo;
  float lreg = 0.f;
  auto load_blk = [&](int qb) {
    const int r0 = qb * C::BMQ;
    sq.load(qhat, base, rs, r0, T, tid);
    sdo.load(dout, base, rs, r0, T, tid);
    if (tid < C::BMQ) {
      const int t = r0 + tid;
      lreg = t < T ? lse[sb + t] * kLog2e : 0.f;
    } else if (tid < 2 * C::BMQ) {
      const int t = r0 + tid - C::BMQ;
      lreg = t < T ? delta[sb + t] : 0.f;
    }
  };

  if (qb0 <= qb1) load_blk(qb0);
  for (int qb = qb0; qb <= qb1; ++qb) {
    __syncthreads();
    sq.template store<true, true>(Qs, C::RP, QTs, C::TP, tid);
    sdo.template store<true, true>(dOs, C::RP, dOTs, C::TP, tid);
    if (tid < 2 * C::BMQ) Ls[tid] = lreg;  // Ls and Dls are contiguous
    __syncthreads();
    if (qb < qb1) load_blk(qb + 1);

    const int q0 = qb * C::BMQ;
    const int cls = tile_class(q0, q0 + C::BMQ - 1, j0 + 32 * w, j0 + 32 * w + 31, T, W);
    if (cls == TILE_EMPTY) continue;

    u32x4 pf[C::BMQ / 16], dsf[C::BMQ / 16];
#pragma unroll
    for (int mb = 0; mb < C::BMQ / 32; ++mb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        s = mfma32(ld16(Qs + (32 * mb + c) * C::RP + 16 * ks + 8 * g), kf[ks], s);
        dp = mfma32(ld16(dOs + (32 * mb + c) * C::RP + 16 * ks + 8 * g), vf[ks], dp);
      }
      // lane (g, c), register r: query q0 + 32 mb + 8 (r/4) + 4 g + r%4, key kj
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int ql = 32 * mb + 8 * q4 + 4 * g;
        f32x4 l4 = *reinterpret_cast<const f32x4*>(Ls + ql);
        f32x4 d4 = *reinterpret_cast<const f32x4*>(Dls + ql);
        float p[4], ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float pe = __builtin_amdgcn_exp2f(s[4 * q4 + e] * ksc - l4[e]);
          if (cls == TILE_PARTIAL && !visible(q0 + ql + e, kj, T, W)) pe = 0.f;
          p[e] = pe;
          ds[e] = pe * (dp[4 * q4 + e] - d4[e]);
        }
        const int st = 2 * mb + (q4 >> 1), el = 2 * (q4 & 1);
        pf[st][el] = pack_bf16(p[0], p[1]);
        pf[st][el + 1] = pack_bf16(p[2], p[3]);
        dsf[st][el] = pack_bf16(ds[0], ds[1]);
        dsf[st][el + 1] = pack_bf16(ds[2], ds[3]);
      }
    }
    // dV^T[d, kv] += dO^T[d, q] P[q, kv];  dK_hat^T[d, kv] += Q_hat^T[d, q] dS[q, kv]
#pragma unroll
    for (int s = 0; s < C::BMQ / 16; ++s) {
#pragma unroll
      for (int n = 0; n < C::NB; ++n) {
        acc_dv[n] = mfma32(ld16(dOTs + (32 * n + c) * C::TP + 16 * s + 8 * g), pf[s], acc_dv[n]);
        acc_dk[n] = mfma32(ld16(QTs + (32 * n + c) * C::TP + 16 * s + 8 * g), dsf[s], acc_dk[n]);
      }
    }
  }

  // ---- epilogue: lane (g, c) holds key kj, d = 32 n + 8 q4 + 4 g + e
  if (kj < T) {
    const float rk = ksc * (sqrtf((float)D) / kLog2e);
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    const uint16_t* krow = k + base + (size_t)kj * rs;
    float dot = 0.f;
    f32x16 khat[C::NB];
#pragma unroll
    for (int n = 0; n < C::NB; ++n)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        u32x2 kk = ld8(krow + 32 * n + 8 * q4 + 4 * g);
        float x[4] = {bf_lo(kk[0]), bf_hi(kk[0]), bf_lo(kk[1]), bf_hi(kk[1])};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          khat[n][4 * q4 + e] = x[e] * rk;
          acc_dk[n][4 * q4 + e] *= inv_sqrt_d;
          dot += acc_dk[n][4 * q4 + e] * khat[n][4 * q4 + e];
        }
      }
    dot += __shfl_xor(dot, 32);
    const float mean = dot * (1.0f / D);
    uint16_t* dkrow = dk + base + (size_t)kj * rs;
    uint16_t* dvrow = dv + base + (size_t)kj * rs;
#pragma unroll
    for (int n = 0; n < C::NB; ++n)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * n + 8 * q4 + 4 * g;
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = rk * (acc_dk[n][4 * q4 + e] - khat[n][4 * q4 + e] * mean);
        st8(dkrow + d, u32x2{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])});
        st8(dvrow + d, u32x2{pack_bf16(acc_dv[n][4 * q4 + 0], acc_dv[n][4 * q4 + 1]),
                             pack_bf16(acc_dv[n][4 * q4 + 2], acc_dv[n][4 * q4 + 3])});
      }
  }
  // (the two lanes of a key row share kj, so the partner exchange above always
  //  pairs two active lanes)
}

// ------------------------------------------------------------------ dQ
template <int D>
struct DqCfg {
  static constexpr int BM = 128;   // queries per workgroup (32 per wave)
  static constexpr int BN = 64;    // keys per step
  static constexpr int KS = D / 16;
  static constexpr int NB = D / 32;
  static constexpr int RP = D + 8;
  static constexpr int TP = BN + 8;
  static constexpr int K_LDS = BN * RP;
  static constexpr int KT_LDS = D * TP;
  static constexpr int LDS_BYTES = (2 * K_LDS + KT_LDS) * 2 + BN * 4;
};

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ qhat,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, const float* __restrict__ rq,
    const float* __restrict__ kscale, uint16_t* __restrict__ dq, int T, int H, int W) {
  using C = DqCfg<D>;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Vs = Ks + C::K_LDS;
  uint16_t* KTs = Vs + C::K_LDS;
  float* KSs = reinterpret_cast<float*>(KTs + C::KT_LDS);

  const int nqt = (T + C::BM - 1) / C::BM;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lid / nqt;
  const int qt = nqt - 1 - (lid % nqt);
  const int b = bh / H, h = bh % H;
  const int i0 = qt * C::BM;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const size_t rs = (size_t)H * D;
  const size_t base = ((size_t)b * T) * rs + (size_t)h * D;
  const size_t sb = (size_t)bh * T;

  const int qi = i0 + 32 * w + c;
  u32x4 qf[C::KS], df[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    qf[ks] = qi < T ? ld16(qhat + base + (size_t)qi * rs + 16 * ks + 8 * g) : u32x4{0, 0, 0, 0};
    df[ks] = qi < T ? ld16(dout + base + (size_t)qi * rs + 16 * ks + 8 * g) : u32x4{0, 0, 0, 0};
  }
  const float lq = qi < T ? lse[sb + qi] * kLog2e : 0.f;
  const float dlt = qi < T ? delta[sb + qi] : 0.f;

  f32x16 acc[C::NB];
#pragma unroll
  for (int n = 0; n < C::NB; ++n) acc[n] = f32x16{};

  int kv_lo, kv_hi;
  kv_range(i0, i0 + C::BM - 1, T, W, &kv_lo, &kv_hi);
  const int jt0 = kv_lo / C::BN, jt1 = kv_hi / C::BN;

  Stage<D, C::BN> sk, sv;
  float ksreg = 0.f;
  auto load_tile = [&](int jt) {
    const int r0 = jt * C::BN;
    sk.load(k, base, rs, r0, T, tid);
    sv.load(v, base, rs, r0, T, tid);
    if (tid < C::BN) {
      const int t = r0 + tid;
      ksreg = t < T ? kscale[sb + t] : 0.f;
    }
  };

  if (jt0 <= jt1) load_tile(jt0);
  for (int jt = jt0; jt <= jt1; ++jt) {
    __syncthreads();
    sk.template store<true, true>(Ks, C::RP, KTs, C::TP, tid);
    sv.template store<true, false>(Vs, C::RP, nullptr, 0, tid);
    if (tid < C::BN) KSs[tid] = ksreg;
    __syncthreads();
    if (jt < jt1) load_tile(jt + 1);

    const int j0 = jt * C::BN;
    const int cls = tile_class(i0 + 32 * w, i0 + 32 * w + 31, j0, j0 + C::BN - 1, T, W);
    if (cls == TILE_EMPTY) continue;

    u32x4 dsf[C::BN / 16];
#pragma unroll
    for (int mb = 0; mb < C::BN / 32; ++mb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        s = mfma32(ld16(Ks + (32 * mb + c) * C::RP + 16 * ks + 8 * g), qf[ks], s);
        dp = mfma32(ld16(Vs + (32 * mb + c) * C::RP + 16 * ks + 8 * g), df[ks], dp);
      }
      // lane (g, c), register r: key j0 + 32 mb + 8 (r/4) + 4 g + r%4, query qi
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int jl = 32 * mb + 8 * q4 + 4 * g;
        f32x4 k4 = *reinterpret_cast<const f32x4*>(KSs + jl);
        float ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float pe = __builtin_amdgcn_exp2f(s[4 * q4 + e] * k4[e] - lq);
          if (cls == TILE_PARTIAL && !visible(qi, j0 + jl + e, T, W)) pe = 0.f;
          ds[e] = pe * (dp[4 * q4 + e] - dlt) * k4[e];
        }
        const int st = 2 * mb + (q4 >> 1), el = 2 * (q4 & 1);
        dsf[st][el] = pack_bf16(ds[0], ds[1]);
        dsf[st][el + 1] = pack_bf16(ds[2], ds[3]);
      }
    }
    // dQ^T[d, q] += K^T[d, kv] (dS kscale)^T[kv, q]
#pragma unroll
    for (int s = 0; s < C::BN / 16; ++s)
#pragma unroll
      for (int n = 0; n < C::NB; ++n)
        acc[n] = mfma32(ld16(KTs + (32 * n + c) * C::TP + 16 * s + 8 * g), dsf[s], acc[n]);
  }

  // ---- epilogue: dq_hat = acc / log2(e); RMSNorm backward of q
  if (qi < T) {
    const float r = rq[sb + qi];
    const uint16_t* qrow = q + base + (size_t)qi * rs;
    float dot = 0.f;
    f32x16 xh[C::NB];
#pragma unroll
    for (int n = 0; n < C::NB; ++n)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        u32x2 qq = ld8(qrow + 32 * n + 8 * q4 + 4 * g);
        float x[4] = {bf_lo(qq[0]), bf_hi(qq[0]), bf_lo(qq[1]), bf_hi(qq[1])};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xh[n][4 * q4 + e] = x[e] * r;
          acc[n][4 * q4 + e] *= (1.0f / kLog2e);
          dot += acc[n][4 * q4 + e] * xh[n][4 * q4 + e];
        }
      }
    dot += __shfl_xor(dot, 32);
    const float mean = dot * (1.0f / D);
    uint16_t* dqrow = dq + base + (size_t)qi * rs;
#pragma unroll
    for (int n = 0; n < C::NB; ++n)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = r * (acc[n][4 * q4 + e] - xh[n][4 * q4 + e] * mean);
        st8(dqrow + 32 * n + 8 * q4 + 4 * g, u32x2{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])});
      }
  }
}

template <int D>
static hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t stream) {
  const int nrows = a.B * a.T * a.H;
  const int nblk_p = (int)(((long long)nrows * (D / 8) + 255) / 256);
  ProfToken t0 = prof_begin(K_BWD_PREP, stream);
  hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3(nblk_p), dim3(256), 0, stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.o,
                     (const uint16_t*)a.dout, (uint16_t*)a.qhat, a.rq, a.kscale, a.delta, nrows,
                     a.T, a.H, a.eps);
  prof_end(t0);
  const int W = eff_window(a.T, a.window);
  {
    using C = DkdvCfg<D>;
    // more than 64 KiB of dynamic LDS must be opted into, once per kernel
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(bwd_dkdv_kernel<D>),
        hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (attr != hipSuccess) return attr;
    const int nkt = (a.T + C::BNK - 1) / C::BNK;
    ProfToken t1 = prof_begin(K_BWD_DKDV, stream);
    hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3(nkt * a.B * a.H), dim3(256), C::LDS_BYTES, stream,
                       (const uint16_t*)a.qhat, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, a.lse, (const float*)a.delta,
                       (const float*)a.kscale, (uint16_t*)a.dk, (uint16_t*)a.dv, a.T, a.H, W);
    prof_end(t1);
  }
  {
    using C = DqCfg<D>;
    const int nqt = (a.T + C::BM - 1) / C::BM;
    ProfToken t2 = prof_begin(K_BWD_DQ, stream);
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3(nqt * a.B * a.H), dim3(256), C::LDS_BYTES, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.qhat, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (const uint16_t*)a.dout, a.lse,
                       (const float*)a.delta, (const float*)a.rq, (const float*)a.kscale,
                       (uint16_t*)a.dq, a.T, a.H, W);
    prof_end(t2);
  }
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  if (a.D == 128) return launch_bwd_d<128>(a, stream);
  return launch_bwd_d<64>(a, stream);
}

}  // namespace swattn
