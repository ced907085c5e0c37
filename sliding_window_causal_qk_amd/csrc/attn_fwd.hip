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
//   With grouped key/value heads (n_kv_head < n_head, "Autoresearch 深度教程"
//   §7.3), query head h reads key/value head h / G, G = H / H_kv.
//   With the rotary embedding (§7.4), q and k are rotated before the norm:
//   channel pair (i, i + D/2) at position t turns by the angle of the bf16
//   tables cos[t, i], sin[t, i].
//   With the value-embedding gate (§5.2.3), attention uses
//   v + 2 sigmoid(W_g x[:32]) ve in place of v.
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
//  * The pre-pass also writes V transposed ([B, H, D, T]) with the keys of every
//    16-key group permuted (tpos16) into the k order of the MFMA operands, so
//    the V^T operand is one conflict-free 16-byte LDS read per MFMA instead of
//    two transposing reads.
//  * K tiles (padded rows) and V^T tiles (xor-swizzled 16-byte chunks) are
//    copied global -> LDS by direct-to-LDS buffer loads into three rotating
//    buffers, one step ahead; one barrier per 32-key step.
//  * Loads go through buffer descriptors rebased per tile: rows past T read as
//    zero, so ragged tails need no branches; stores past T are dropped.
//  * Band-aware tile loop: a query tile visits only the key blocks that
//    intersect its window; fully visible blocks skip the mask.
#include <type_traits>

#include "common.h"
#include "band.h"
#include "kernels.h"
#include "profile.h"

namespace swattn {

// ------------------------------------------------------------ forward pre-pass
// One workgroup per (batch, key/value head, block of 64 keys); H is the number
// of key/value heads here:
//   kscale[b, h, t] = log2(e) / sqrt(D) * r(k[b, t, h, :])
//   vt[b, h, d, tpos(t)] = v[b, t, h, d]   (V transposed; inside every group of
//       16 keys the columns are permuted by tpos16, so that the 8 keys one lane
//       feeds to an MFMA k-step are one contiguous 16-byte chunk)
// Columns of vt past T are written as zero.
// ROPE: the key rows are rotated first; the rotated rows (bf16) go to kr, the
// K the attention kernel reads, and kscale is taken from them.
// VE: the rows transposed into vt are v + gate ve, gate = 2 sigmoid(W_g x[:32])
// of the token and key/value head (x row t of batch b at xg + (b T + t) xs).
template <int D, bool ROPE, bool VE>
__global__ __launch_bounds__(256) void fwd_prep_kernel(const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v,
                                                       const uint16_t* __restrict__ rcos,
                                                       const uint16_t* __restrict__ rsin,
                                                       const uint16_t* __restrict__ ve,
                                                       const uint16_t* __restrict__ xg, int xs,
                                                       const float* __restrict__ gate_w,
                                                       float* __restrict__ kscale,
                                                       uint16_t* __restrict__ vt,
                                                       uint16_t* __restrict__ kr, int T, int H,
                                                       int LT, float eps) {
  constexpr int KB = 64;                 // keys per workgroup
  constexpr int CH = D / 8;              // 16-byte chunks per row
  constexpr int TPR = 256 / KB;          // threads per key row (4)
  constexpr int CPT = CH / TPR;          // chunks per thread
  constexpr int LP = D + 2;              // LDS pitch (bf16) of the V block: column reads hit distinct banks
  __shared__ uint32_t vs[KB * LP / 2];

  const int nkb = LT / KB;
  const int bh = blockIdx.x / nkb, kb = blockIdx.x % nkb;
  const int b = bh / H, h = bh % H;
  const int t0 = kb * KB;
  const int tid = threadIdx.x;
  const int rs = H * D;
  const long long slice_bytes = (long long)(T - 1) * rs * 2 + 2 * D;
  const size_t sbase = ((size_t)b * T * H + h) * D;
  const rsrc_t rk = make_rsrc(k + sbase + (size_t)t0 * rs, slice_bytes - (long long)t0 * rs * 2);
  const rsrc_t rv = make_rsrc(v + sbase + (size_t)t0 * rs, slice_bytes - (long long)t0 * rs * 2);

  // rows: thread -> key t0 + tid / TPR, CPT chunks: the first half of them
  // first-half channels, the rest their rotation partners (the same split
  // with and without ROPE, so that kscale sums in the same order)
  const int r = tid / TPR, part = tid % TPR;
  auto chunk = [&](int i) {
    return i < CPT / 2 ? part * (CPT / 2) + i : CH / 2 + part * (CPT / 2) + i - CPT / 2;
  };
  u32x4 kk[CPT];
  float gate = 0.f;
  if constexpr (VE)
    gate = ve_gate_sum<TPR>(xg + ((size_t)b * T + t0 + r) * xs, gate_w + h * 32, part, t0 + r < T);
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int ch = chunk(i);
    kk[i] = bload16(rk, (r * rs + 8 * ch) * 2);
    u32x4 vv = bload16(rv, (r * rs + 8 * ch) * 2);
    if constexpr (VE) {
      const rsrc_t rve = make_rsrc(ve + sbase + (size_t)t0 * rs, slice_bytes - (long long)t0 * rs * 2);
      const u32x4 ee = bload16(rve, (r * rs + 8 * ch) * 2);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        vv[e] = pack_bf16(bf_lo(vv[e]) + gate * bf_lo(ee[e]), bf_hi(vv[e]) + gate * bf_hi(ee[e]));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) vs[(r * LP + 8 * ch) / 2 + e] = vv[e];
  }
  if constexpr (ROPE) {
    const long long tb = (long long)(T - t0) * D;   // table rows t0 .. T-1 (D / 2 bf16 each)
    const rsrc_t rc = make_rsrc(rcos + (size_t)t0 * (D / 2), tb);
    const rsrc_t rn = make_rsrc(rsin + (size_t)t0 * (D / 2), tb);
    const rsrc_t rkr = make_rsrc(kr + sbase + (size_t)t0 * rs, slice_bytes - (long long)t0 * rs * 2);
#pragma unroll
    for (int i = 0; i < CPT / 2; ++i) {
      const int ch = chunk(i);
      const u32x4 c = bload16(rc, (r * (D / 2) + 8 * ch) * 2), sn = bload16(rn, (r * (D / 2) + 8 * ch) * 2);
      float y1[8], y2[8];
      rope8(kk[i], kk[i + CPT / 2], c, sn, y1, y2);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kk[i][e] = pack_bf16(y1[2 * e], y1[2 * e + 1]);
        kk[i + CPT / 2][e] = pack_bf16(y2[2 * e], y2[2 * e + 1]);
      }
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) bstore16(kk[i], rkr, (r * rs + 8 * chunk(i)) * 2);
  }
  float ss = 0.f;   // of the keys the attention kernel multiplies (rotated, bf16)
#pragma unroll
  for (int i = 0; i < CPT; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = bf_lo(kk[i][e]), bb = bf_hi(kk[i][e]);
      ss += a * a + bb * bb;
    }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, TPR);
  if (part == 0 && t0 + r < T) {
    const float rr = 1.0f / sqrtf(ss * (1.0f / D) + eps);
    kscale[(size_t)bh * T + t0 + r] = rr * (kLog2e / sqrtf((float)D));
  }
  __syncthreads();

  // columns: thread -> (d, 8-key chunk); consecutive threads write consecutive
  // 16-byte chunks of one row of vt
  const uint16_t* vsh = reinterpret_cast<const uint16_t*>(vs);
  uint16_t* vrow = vt + (size_t)bh * D * LT + t0;
#pragma unroll
  for (int p = 0; p < D * (KB / 8) / 256; ++p) {
    const int idx = tid + 256 * p;
    const int d = idx / (KB / 8), ch = idx % (KB / 8);
    uint32_t w4[4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      // position 8 ch + j holds key tpos16^-1 (tpos16 is an involution)
      const int k0 = (8 * ch + j) & ~15, x0 = (8 * ch + j) & 15;
      const uint32_t lo = vsh[(k0 + tpos16(x0)) * LP + d];
      const uint32_t hi = vsh[(k0 + tpos16(x0 + 1)) * LP + d];
      w4[j / 2] = lo | (hi << 16);
    }
    st16(vrow + (size_t)d * LT + 8 * ch, u32x4{w4[0], w4[1], w4[2], w4[3]});
  }
}

// ------------------------------------------------------------ forward kernel
// Workgroup: 4 waves; wave w owns queries i0 + 32 w + c.  Key blocks of 32
// (K rows, V^T columns and kscale) stream through the band in three LDS
// buffers filled by direct-to-LDS loads one step ahead.  Per block i:
//   A(i): S^T = K Q_hat^T                      (queries in lanes, keys in registers)
//   B(i): P = exp2(S^T kscale - sqrt(D) log2 e), masked on edge blocks; row sums
//   C(i): O^T += V^T P^T                       (V^T from the transposed copy)
// The loop issues A(i+1), then C(i) interleaved with B(i+1).  Every MFMA
// operand read from LDS is one conflict-free 16-byte read.
template <int D, bool ROPE>
struct FwdCfg {
  static constexpr int BM = 128;   // queries per workgroup (32 per wave)
  static constexpr int BN = 32;    // keys per step
  static constexpr int NBUF = 3;
  static constexpr int KS = D / 16;
  static constexpr int NB = D / 32;
  static constexpr int PK = D + 8;                     // K row pitch (bf16): 16-byte reads conflict-free
  using KTile = DmaTileV<BN * PK / 8, 4, 8 + ROPE>;
  using VTile = DmaTileV<D * BN / 8, 4, 8 + ROPE>;     // D rows of 64 bytes, xor-swizzled chunks
  static constexpr int V_B = KTile::BYTES;
  static constexpr int ST_B = V_B + VTile::BYTES;      // kscale (128 bytes used of 256)
  static constexpr int STAGE = ST_B + 256;
  static constexpr int LDS_BYTES = NBUF * STAGE;
  static_assert(LDS_BYTES <= 160 * 1024, "fits the LDS of one CU");
};

// Chunk slot of logical chunk ch (0..3) in row r of a transposed 32-column tile.
__device__ __forceinline__ int vt_slot(int r, int ch) { return ch ^ ((r >> 2) & 3); }

// ROPE: k is the rotated copy written by the pre-pass, and the queries are
// rotated in the prologue.
template <int D, bool ROPE>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ vt, const float* __restrict__ kscale,
    const uint16_t* __restrict__ rcos, const uint16_t* __restrict__ rsin,
    uint16_t* __restrict__ o, float* __restrict__ lse, int T, int H, int G, int LT, int W,
    float eps) {
  using C = FwdCfg<D, ROPE>;
  extern __shared__ __align__(16) unsigned char smem[];

  const int nqt = (T + C::BM - 1) / C::BM;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  int bh, qt;
  query_tile_of(lid, nqt, gridDim.x / nqt, kTileGroupFwd, &bh, &qt);
  const int b = bh / H, h = bh % H;
  const int Hkv = H / G;
  const int bhk = b * Hkv + h / G;        // key/value slice read by this head
  const int i0 = qt * C::BM;

  const int tid = threadIdx.x;
  const int w = uniform(tid >> 6);
  const int lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int rs = H * D;
  const long long rsb = 2LL * rs;
  const long long slice_bytes = (long long)(T - 1) * rsb + 2 * D;
  const size_t sbase = ((size_t)b * T * H + h) * D;
  const int rs_kv = Hkv * D;               // K row stride (elements)
  const long long rsb_kv = 2LL * rs_kv;
  const long long kslice_bytes = (long long)(T - 1) * rsb_kv + 2 * D;

  // ---- query fragment: normalised q row (i0 + 32 w + c), B operand of S^T = K Q^T
  const int qw0 = i0 + 32 * w;
  const int qi = qw0 + c;
  u32x4 qf[C::KS];
  {
    const rsrc_t rq = make_rsrc(q + sbase + (size_t)qw0 * rs, slice_bytes - qw0 * rsb);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[ks] = bload16(rq, (c * rs + 16 * ks + 8 * g) * 2);
    normalise_query<D, ROPE>(qf, rcos, rsin, qw0, c, g, T, eps);
  }

  f32x16 acc[C::NB];
#pragma unroll
  for (int n = 0; n < C::NB; ++n) acc[n] = f32x16{};
  float lsum = 0.f;
  const float shift = sqrtf((float)D) * kLog2e;  // fixed softmax shift, log2 units

  int kv_lo, kv_hi;
  kv_range(i0, i0 + C::BM - 1, T, W, &kv_lo, &kv_hi);
  const int jb0 = kv_lo / C::BN;
  const int nsteps = kv_hi / C::BN - jb0 + 1;

  // ---- direct-to-LDS staging of one key step
  typename C::KTile ktile;
  ktile.init(w, lane, [&](int qc) {
    const int r = qc / (C::PK / 8), ch = qc % (C::PK / 8);
    return (r < C::BN && ch < D / 8) ? (r * rs_kv + 8 * ch) * 2 : -1;
  });
  typename C::VTile vtile;
  vtile.init(w, lane, [&](int qc) {
    const int r = qc >> 2, s = qc & 3;
    return (r * LT + 8 * vt_slot(r, s)) * 2;
  });
  const rsrc_t rks = make_rsrc(kscale + (size_t)bhk * T, 4LL * T);
  const uint16_t* k_s = k + ((size_t)b * T * Hkv + (h / G)) * D;
  const uint16_t* vt_s = vt + (size_t)bhk * D * LT;
  const long long vt_bytes = 2LL * D * LT;
  // remaining bytes of the slices from key j0 on, below 2^32 (unsigned arithmetic)
  const uint32_t kbytes_u = (uint32_t)kslice_bytes, krow_u = (uint32_t)rsb_kv, vtbytes_u = (uint32_t)vt_bytes;
  auto issue_step = [&](int step, int base) {
    const int j0 = (jb0 + step) * C::BN;
    ktile.issue(make_rsrc_u(k_s + (size_t)j0 * rs_kv, kbytes_u - (uint32_t)j0 * krow_u), smem, base, w);
    vtile.issue(make_rsrc_u(vt_s + j0, vtbytes_u - 2u * (uint32_t)j0), smem, base + C::V_B, w);
    if (w == 0) dma_row4(rks, smem, base + C::ST_B, (j0 + lane) * 4);   // wave 0 loads kscale
  };

  const int a_off = 2 * (c * C::PK + 8 * g);                 // K rows: row c, chunk 2 ks + g
  const int v_off0 = 64 * c + 16 * vt_slot(c, g);            // V^T rows 32 n + c, chunk g (k-step 0)
  const int v_off1 = 64 * c + 16 * vt_slot(c, 2 + g);        // ... chunk 2 + g (k-step 1)
  const int k_off = C::ST_B + 16 * g;                        // kscale of the lane's key quads

  f32x16 s_acc;
  u32x4 pf[2];

  auto stage_a = [&](int base) {
    const int va = base + a_off;
    s_acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) s_acc = mfma32(lds16(smem, va + 32 * ks), qf[ks], s_acc);
  };
  // lane (g, c), register r: key j0 + 8 (r/4) + 4 g + r%4, query qi
  auto stage_b = [&](int base, int step, auto masked_c) {
    constexpr bool MASKED = decltype(masked_c)::value;
    const int vk = base + k_off;
    const int t0 = (jb0 + step) * C::BN + 4 * g + W - qi;  // key kv visible iff 0 <= kv - (qi - W) <= W
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 k4 = lds16f(smem, vk + 32 * q4);
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(s_acc[4 * q4 + e] * k4[e] - shift);
      if (MASKED) {
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = ((unsigned)(t0 + 8 * q4 + e) <= (unsigned)W) ? p[e] : 0.f;
      }
      const uint32_t p01 = pack_bf16(p[0], p[1]), p23 = pack_bf16(p[2], p[3]);
      const int st = q4 >> 1, el = 2 * (q4 & 1);
      pf[st][el] = p01;
      pf[st][el + 1] = p23;
      // the row sum adds the bf16-rounded probabilities the PV product uses,
      // so the output weights sum to one (W = 0 gives o = v exactly)
      lsum = sum_bf16x2(p01, lsum);
      lsum = sum_bf16x2(p23, lsum);
    }
  };
  // O^T[d, q] += V^T[d, kv] P^T[kv, q]; element j of k-step s2 is key
  // 16 s2 + 4 g + (j % 4) + 8 (j / 4), the order of the tpos16 columns
  auto stage_c = [&](int base) {
    const int vb = base + C::V_B;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int n = 0; n < C::NB; ++n)
        acc[n] = mfma32(lds16(smem, vb + (s2 ? v_off1 : v_off0) + 2048 * n), pf[s2], acc[n]);
  };

  // ---- prologue: steps 0, 1 in LDS, step 2 in flight; A(0), B(0)
  int b0 = 0, b1 = C::STAGE, b2 = 2 * C::STAGE;
  if (nsteps > 0) issue_step(0, b0);
  if (nsteps > 1) issue_step(1, b1);
  wait_vmcnt<0>();
  __syncthreads();
  if (nsteps > 2) issue_step(2, b2);
  const std::integral_constant<bool, true> masked{};
  const std::integral_constant<bool, false> unmasked{};
  if (nsteps > 0) {
    stage_a(b0);
    stage_b(b0, 0, masked);
  }

  auto step_body = [&](int it, auto masked_c) {
    stage_a(b1);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < C::KS - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
    stage_c(b0);
    stage_b(b1, it + 1, masked_c);
    asm volatile("" ::"v"(pf[0]), "v"(pf[1]), "v"(lsum));
    wait_vmcnt<0>();            // step it + 2 landed
    __syncthreads();
    if (it + 3 < nsteps) issue_step(it + 3, b0);   // buffer of step it, consumed
    const int t = b0;
    b0 = b1;
    b1 = b2;
    b2 = t;
  };

  // steps visible in full to every query of the workgroup: keys kv0 .. kv0 + 31
  // with kv0 + 31 <= i0 and (i0 + BM - 1) - kv0 <= W (and all inside T)
  int full_lo = nsteps, full_hi = -1;
  if (nsteps > 0 && i0 + C::BM - 1 < T) {
    const int lo_kv = i0 + C::BM - 1 - W;                  // first key visible to every query
    full_lo = imax(0, (lo_kv + C::BN - 1) / C::BN - jb0);
    full_hi = (i0 - (C::BN - 1)) >= 0 ? (i0 - (C::BN - 1)) / C::BN - jb0 : -1;
    full_hi = imin(full_hi, nsteps - 1);
  }
  const int u0 = imax(full_lo - 1, 0), u1 = full_hi - 1;   // body it prepares B(it + 1)
  const int nloop = nsteps - 1;
  int it = 0;
  for (; it < imin(u0, nloop); ++it) step_body(it, masked);
  for (; it <= u1 && it < nloop; ++it) step_body(it, unmasked);
  for (; it < nloop; ++it) step_body(it, masked);
  if (nsteps > 0) stage_c(b0);

  // ---- epilogue: O = O^T / l, lse = shift + ln l  (stores past T are dropped)
  lsum += __shfl_xor(lsum, 32);
  const float inv = 1.0f / lsum;
  // O leaves through LDS (the step buffers are free once every wave is past
  // its last product) so that global memory sees whole rows
  using RS = RowStage32<D>;
  static_assert(4 * RS::BYTES <= C::LDS_BYTES, "output staging fits in the step buffers");
  __syncthreads();
  const int slot = RS::BYTES * w;
#pragma unroll
  for (int n = 0; n < C::NB; ++n)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      RS::put(smem, slot, c, 32 * n + 8 * q4 + 4 * g,
              u32x2{pack_bf16(acc[n][4 * q4 + 0] * inv, acc[n][4 * q4 + 1] * inv),
                    pack_bf16(acc[n][4 * q4 + 2] * inv, acc[n][4 * q4 + 3] * inv)});
  RS::store_rows(smem, slot, make_rsrc(o + sbase + (size_t)qw0 * rs, slice_bytes - qw0 * rsb), rs, lane);
  if (g == 0) {
    const rsrc_t rl = make_rsrc(lse + (size_t)bh * T, 4LL * T);
    bstore4f(sqrtf((float)D) + __logf(lsum), rl, qi * 4);
  }
}

template <int D, bool ROPE>
static hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t stream) {
  using C = FwdCfg<D, ROPE>;
  const int nkb = a.LT / 64;
  ProfToken t0 = prof_begin(K_FWD_PREP, stream);
  hipLaunchKernelGGL((a.ve ? fwd_prep_kernel<D, ROPE, true> : fwd_prep_kernel<D, ROPE, false>),
                     dim3(nkb * a.B * a.Hkv), dim3(256), 0, stream,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.rcos,
                     (const uint16_t*)a.rsin, (const uint16_t*)a.ve, (const uint16_t*)a.xg, a.xs,
                     a.gate_w, a.kscale, (uint16_t*)a.vt, (uint16_t*)a.kr, a.T, a.Hkv, a.LT, a.eps);
  prof_end(t0);
  const int nqt = (a.T + C::BM - 1) / C::BM;
  const int nblk = nqt * a.B * a.H;
  const int W = eff_window(a.T, a.window);
  // more than 64 KiB of dynamic LDS must be opted into, once per kernel
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(attn_fwd_kernel<D, ROPE>),
      hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  ProfToken t1 = prof_begin(K_FWD, stream);
  hipLaunchKernelGGL((attn_fwd_kernel<D, ROPE>), dim3(nblk), dim3(256), C::LDS_BYTES, stream,
                     (const uint16_t*)a.q, (const uint16_t*)(ROPE ? a.kr : a.k), (const uint16_t*)a.vt,
                     (const float*)a.kscale, (const uint16_t*)a.rcos, (const uint16_t*)a.rsin,
                     (uint16_t*)a.o, a.lse, a.T, a.H, a.H / a.Hkv, a.LT, W, a.eps);
  prof_end(t1);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  const bool rope = a.rcos != nullptr;
  if (a.D == 256) return rope ? launch_fwd_d<256, true>(a, stream) : launch_fwd_d<256, false>(a, stream);
  if (a.D == 128) return rope ? launch_fwd_d<128, true>(a, stream) : launch_fwd_d<128, false>(a, stream);
  return rope ? launch_fwd_d<64, true>(a, stream) : launch_fwd_d<64, false>(a, stream);
}

}  // namespace swattn
