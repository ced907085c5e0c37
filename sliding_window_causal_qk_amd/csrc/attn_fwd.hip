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
//  * The V^T operand of that product comes from V rows in LDS by transposing
//    reads (ds_read_b64_tr_b16), so V needs no transposed copy in HBM.
//  * K tiles (padded rows) and V tiles (xor-swizzled 16-byte chunks) are
//    copied global -> LDS by direct-to-LDS buffer loads into three rotating
//    buffers, one step ahead; one barrier per 32-key step.
//  * Loads go through buffer descriptors rebased per tile: rows past T read as
//    zero, so ragged tails need no branches; stores past T are dropped.
//  * Band-aware tile loop: a query tile visits only the key blocks that
//    intersect its window; a block visible in full to a wave's 32 queries
//    skips the mask in that wave.
#include <type_traits>

#include "common.h"
#include "band.h"
#include "kernels.h"
#include "profile.h"

namespace swattn {

// ------------------------------------------------------------ forward kernel
// Workgroup: 4 waves; wave w owns queries i0 + 32 w + c.  Key blocks of 32
// (K rows, V rows and kscale) stream through the band in three LDS buffers
// filled by direct-to-LDS loads one step ahead.  Per block i:
//   A(i): S^T = K Q_hat^T                      (queries in lanes, keys in registers)
//   B(i): P = exp2(S^T kscale - sqrt(D) log2 e), masked on edge blocks; row sums
//   C(i): O^T += V^T P^T                       (V^T by transposing reads of V)
// The loop issues A(i+1), then C(i) interleaved with B(i+1).  Every LDS read
// is free of bank conflicts.
template <int D, bool ROPE>
struct FwdCfg {
  static constexpr int BM = 128;   // queries per workgroup (32 per wave)
  static constexpr int BN = 32;    // keys per step
  static constexpr int NBUF = 3;
  static constexpr int KS = D / 16;
  static constexpr int NB = D / 32;
  static constexpr int PK = D + 8;                     // K row pitch (bf16): 16-byte reads conflict-free
  using KTile = DmaTileV<BN * PK / 8, 4, 8 + ROPE>;
  using VTile = DmaTileV<BN * D / 8, 4, 8 + ROPE>;     // BN rows of D bf16, xor-swizzled chunks
  static constexpr int V_B = KTile::BYTES;
  static constexpr int ST_B = V_B + VTile::BYTES;      // kscale (128 bytes used of 256)
  static constexpr int STAGE = ST_B + 256;
  static constexpr int LDS_BYTES = NBUF * STAGE;
  static_assert(LDS_BYTES <= 160 * 1024, "fits the LDS of one CU");
};

// LDS slot of 16-byte chunk ch of V row r.  A transposing read takes two
// chunks of each of 4 consecutive rows (32 bytes each); xor-ing bits 1-2 of
// the chunk index with the row's position in its group of 4 spreads those 8
// chunks over distinct banks without padding the rows.
__device__ __forceinline__ int v_slot(int r, int ch) { return ch ^ (2 * (r & 3)); }

// ROPE: k is the rotated copy written by the pre-pass, and the queries are
// rotated in the prologue.  At D = 256 the three stage buffers take 100 KB of
// LDS, so one workgroup runs per CU: the kernel is then built for one wave per
// SIMD, whose 512 registers hold the accumulators and every operand in flight.
// At D = 128 three workgroups share a CU (52 KB of LDS each), and the launch
// bounds hold the kernel to the 168 registers that three waves per SIMD allow;
// at D = 64, four.
template <int D, bool ROPE>
__global__ __launch_bounds__(256, D >= 256 ? 1 : (D >= 128 ? 3 : 4)) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ kscale,
    const uint16_t* __restrict__ rcos, const uint16_t* __restrict__ rsin,
    uint16_t* __restrict__ o, float* __restrict__ lse, int T, int H, int G, int W, float eps,
    int cpx) {
  using C = FwdCfg<D, ROPE>;
  extern __shared__ __align__(16) unsigned char smem[];

  const int nqt = (T + C::BM - 1) / C::BM;
  const int lid = xcd_remap_paired(blockIdx.x, gridDim.x, cpx);
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
  // Step i visits key block blk(i) = jb0 + ((i - jb0) mod nsteps): the band
  // rotated so that every query tile whose band has the same length visits
  // block j at step j mod nsteps.  The tiles of one (batch, head) run at the
  // same time, and with the rotation they read the same key block at about
  // the same time, so most of their reads hit in L2.  (The softmax shift is
  // fixed, so the order of the blocks changes nothing but rounding.)
  const int rot = nsteps > 0 ? (nsteps - jb0 % nsteps) % nsteps : 0;
  auto blk = [&](int i) {   // 0 <= i < nsteps
    const int x = i + rot;
    return jb0 + (x >= nsteps ? x - nsteps : x);
  };

  // ---- direct-to-LDS staging of one key step
  typename C::KTile ktile;
  ktile.init(w, lane, [&](int qc) {
    const int r = qc / (C::PK / 8), ch = qc % (C::PK / 8);
    return (r < C::BN && ch < D / 8) ? (r * rs_kv + 8 * ch) * 2 : -1;
  });
  typename C::VTile vtile;
  vtile.init(w, lane, [&](int qc) {   // LDS chunk qc: row qc / (D / 8), slot qc % (D / 8)
    const int r = qc / (D / 8), sl = qc % (D / 8);
    return (r * rs_kv + 8 * v_slot(r, sl)) * 2;   // v_slot is its own inverse
  });
  const u32x4 rks = make_desc(kscale + (size_t)bhk * T, 4LL * T);
  const size_t kvbase = ((size_t)b * T * Hkv + (h / G)) * D;
  const uint16_t* k_s = k + kvbase;
  const uint16_t* v_s = v + kvbase;
  // remaining bytes of the slices from key j0 on, below 2^32 (unsigned arithmetic)
  const uint32_t kbytes_u = (uint32_t)kslice_bytes, krow_u = (uint32_t)rsb_kv;
  auto issue_step = [&](int step, int base) {
    const int j0 = blk(step) * C::BN;
    const uint32_t nb = kbytes_u - (uint32_t)j0 * krow_u;
    ktile.issue(make_desc_u(k_s + (size_t)j0 * rs_kv, nb), smem, base, w);
    vtile.issue(make_desc_u(v_s + (size_t)j0 * rs_kv, nb), smem, base + C::V_B, w);
    if (w == 0) dma_row4(rks, smem, base + C::ST_B, (j0 + lane) * 4);   // wave 0 loads kscale
  };

  const int a_off = 2 * (c * C::PK + 8 * g);                 // K rows: row c, chunk 2 ks + g
  // transposing reads of the V rows (16-lane group: lane i = 4 a + e reads
  // slot j from the 8-byte piece addressed by lane a + 4 j): lane (g, c)
  // addresses row 4 g + li / 4 (+ 16 s2, + 8), channels 32 n + 16 hb + 4 (li % 4)
  // .. + 3, i.e. chunk 4 n + x, x = 2 hb + (li % 4) / 2, 8-byte half li % 2.
  // The row's swizzle xors the chunk with 2 kr, kr = li / 4: bit 0 of kr flips
  // bit 1 of x, bit 1 of kr flips the parity of n, so even and odd n take two
  // lane offsets and n / 2 a fixed step of 128 bytes.
  const int li = lane & 15, hb = (lane >> 4) & 1, kr4 = li >> 2;
  const int xs4 = (2 * hb + ((li & 3) >> 1)) ^ (2 * (kr4 & 1));
  const int vrow = 2 * D * (4 * g + kr4) + 16 * xs4 + 8 * (li & 1);
  const int v_even = vrow + 64 * (kr4 >> 1);
  const int v_odd = vrow + 64 * (1 - (kr4 >> 1));
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
    const int t0 = blk(step) * C::BN + 4 * g + W - qi;  // key kv visible iff 0 <= kv - (qi - W) <= W
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
  // 16 s2 + 4 g + (j % 4) + 8 (j / 4), the k order of the probabilities
  auto stage_c = [&](int base) {
    const int vb = base + C::V_B;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int n = 0; n < C::NB; ++n) {
        const int off = vb + ((n & 1) ? v_odd : v_even) + 128 * (n >> 1) + 2 * D * 16 * s2;
        const u32x2 a0 = lds_tr4b(smem, off), a1 = lds_tr4b(smem, off + 2 * D * 8);
        acc[n] = mfma32(u32x4{a0[0], a0[1], a1[0], a1[1]}, pf[s2], acc[n]);
      }
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

  // In the masked steps at the band's two ends a wave skips a key block that
  // none of its 32 queries sees (all keys after the last query, or before the
  // first one's window): no S products, P = 0, and then no PV products for
  // it.  Adding those zeros changed nothing, so the results are unchanged;
  // the other waves on the SIMD take the issue slots (D <= 128: two or three
  // workgroups per CU; at D = 256 one wave per SIMD has nobody to give them to).
  bool c_zero = false;   // P of the block C works on is all zero for this wave
  // At D = 256 (one wave per SIMD) the step's order is written out in fenced
  // regions: S's products with the K operands read KA ahead, then C's
  // products, each after the transposing V reads of the product CA places
  // later, with B's elements (the exponential, the mask, the bf16 packing
  // and the row sum) between them.  B writes separate registers that C takes
  // over at the step's end.
  auto step_written = [&](int it, auto masked_c) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_c)::value;
    constexpr int KA = 4, CA = 2, NC = 2 * C::NB, EPM = 16 / NC;
    const int va = b1 + a_off, vk = b1 + k_off, vb = b0 + C::V_B;
    auto v_read = [&](int m) {
      const int s2 = m / C::NB, n = m % C::NB;
      const int off = vb + ((n & 1) ? v_odd : v_even) + 128 * (n >> 1) + 2 * D * 16 * s2;
      const u32x2 a0 = lds_tr4b(smem, off), a1 = lds_tr4b(smem, off + 2 * D * 8);
      return u32x4{a0[0], a0[1], a1[0], a1[1]};
    };
    u32x4 ka[C::KS], cop[NC];
    f32x4 k4s[4];
#pragma unroll
    for (int ks = 0; ks < KA; ++ks) ka[ks] = lds16(smem, va + 32 * ks);
#pragma unroll
    for (int m = 0; m < CA; ++m) cop[m] = v_read(m);
    __builtin_amdgcn_sched_barrier(0);
    s_acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      if (ks + KA < C::KS) ka[ks + KA] = lds16(smem, va + 32 * (ks + KA));
      s_acc = mfma32(ka[ks], qf[ks], s_acc);
      if (ks == C::KS - 2) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) k4s[q4] = lds16f(smem, vk + 32 * q4);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    const int t0 = blk(it + 1) * C::BN + 4 * g + W - qi;   // key kv visible iff 0 <= kv - (qi - W) <= W
    float pe[16];
    u32x4 pn[2];
#pragma unroll
    for (int m = 0; m < NC; ++m) {
      if (m + CA < NC) cop[m + CA] = v_read(m + CA);
      const int s2 = m / C::NB, n = m % C::NB;
      acc[n] = mfma32(cop[m], pf[s2], acc[n]);
#pragma unroll
      for (int k = 0; k < EPM; ++k) {
        const int r = EPM * m + k, q4 = r >> 2, e = r & 3;
        float pr = __builtin_amdgcn_exp2f(s_acc[r] * k4s[q4][e] - shift);
        if (MASKED) pr = ((unsigned)(t0 + 8 * q4 + e) <= (unsigned)W) ? pr : 0.f;
        pe[r] = pr;
        asm volatile("" : "+v"(pe[r]));
        if (e & 1) {
          const uint32_t pk = pack_bf16(pe[r - 1], pe[r]);
          pn[q4 >> 1][2 * (q4 & 1) + (e >> 1)] = pk;
          lsum = sum_bf16x2(pk, lsum);
          asm volatile("" : "+v"(pn[q4 >> 1][2 * (q4 & 1) + (e >> 1)]), "+v"(lsum));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    pf[0] = pn[0];
    pf[1] = pn[1];
  };
  auto step_body = [&](int it, auto masked_c) {
    if constexpr (D >= 256) {
      step_written(it, masked_c);
      wait_vmcnt<0>();            // step it + 2 landed
      __syncthreads();
      if (it + 3 < nsteps) issue_step(it + 3, b0);   // buffer of step it, consumed
      const int t = b0;
      b0 = b1;
      b1 = b2;
      b2 = t;
      return;
    }
    constexpr bool MASKED = decltype(masked_c)::value && D <= 128;
    const int kb = blk(it + 1) * C::BN;
    const bool seen = !MASKED || (kb <= qw0 + 31 && kb + C::BN - 1 >= qw0 - W);
    if (seen) {
      stage_a(b1);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < C::KS - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (!MASKED || !c_zero) stage_c(b0);
    if (seen) {
      stage_b(b1, it + 1, masked_c);
    } else {
      pf[0] = u32x4{};
      pf[1] = u32x4{};
    }
    if constexpr (MASKED) c_zero = !seen;
    else c_zero = false;
    asm volatile("" ::"v"(pf[0]), "v"(pf[1]), "v"(lsum));
    wait_vmcnt<0>();            // step it + 2 landed
    __syncthreads();
    if (it + 3 < nsteps) issue_step(it + 3, b0);   // buffer of step it, consumed
    const int t = b0;
    b0 = b1;
    b1 = b2;
    b2 = t;
  };

  // steps visible in full to every query of this wave: keys kv0 .. kv0 + 31
  // with kv0 + 31 <= qw0 and (qw0 + 31) - kv0 <= W (and all inside T).  The
  // ranges differ between the waves, which pass the same number of barriers.
  int full_lo = nsteps, full_hi = -1;
  if (nsteps > 0 && qw0 + 31 < T) {
    const int lo_kv = qw0 + 31 - W;                        // first key visible to every query
    full_lo = imax(0, (lo_kv + C::BN - 1) / C::BN - jb0);
    full_hi = (qw0 - (C::BN - 1)) >= 0 ? (qw0 - (C::BN - 1)) / C::BN - jb0 : -1;
    full_hi = imin(full_hi, nsteps - 1);
  }
  // Body it prepares B(it + 1), unmasked iff block blk(it + 1) lies in that
  // range.  With the rotation those bodies form at most two runs: j = it + 1
  // in [full_lo - rot, full_hi - rot] (the part at or above 1) and the same
  // range moved up by nsteps (the part below nsteps).
  const int nloop = nsteps - 1;
  int ua0 = nloop, ua1 = nloop - 1, ub0 = nloop, ub1 = nloop - 1;
  if (full_lo <= full_hi) {
    const int a0 = full_lo - rot, a1 = full_hi - rot;
    ua0 = imax(a0, 1) - 1;
    ua1 = imin(a1, nsteps - 1) - 1;
    ub0 = imax(a0 + nsteps, 1) - 1;
    ub1 = imin(a1 + nsteps, nsteps - 1) - 1;
  }
  int it = 0;
  for (; it < imin(ua0, nloop); ++it) step_body(it, masked);
  for (; it <= ua1 && it < nloop; ++it) step_body(it, unmasked);
  for (; it < imin(ub0, nloop); ++it) step_body(it, masked);
  for (; it <= ub1 && it < nloop; ++it) step_body(it, unmasked);
  for (; it < nloop; ++it) step_body(it, masked);
  if (nsteps > 0 && !c_zero) stage_c(b0);

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
  KeyPrepArgs kp;
  kp.k = a.k; kp.v = a.v; kp.rcos = a.rcos; kp.rsin = a.rsin; kp.ve = a.ve; kp.xg = a.xg; kp.xs = a.xs;
  kp.gate_w = a.gate_w; kp.kscale = a.kscale; kp.kr = a.kr; kp.vr = a.vr; kp.gate = a.gate;
  kp.B = a.B; kp.T = a.T; kp.Hkv = a.Hkv; kp.D = D; kp.eps = a.eps;
  const hipError_t ep = launch_key_prep(kp, K_FWD_PREP, stream);
  if (ep != hipSuccess) return ep;
  const int nqt = (a.T + C::BM - 1) / C::BM;
  const int nblk = nqt * a.B * a.H;
  const int W = eff_window(a.T, a.window);
  // a grid that the CUs hold at once pairs heavy with light tiles per CU
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1)
    return hipErrorInvalidDevice;
  const long long slots = (long long)ncu * (D >= 256 ? 1 : (D >= 128 ? 3 : 4));
  const int cpx = (nblk <= slots && ncu % 8 == 0) ? ncu / 8 : 0;
  // more than 64 KiB of dynamic LDS must be opted into, once per kernel
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(attn_fwd_kernel<D, ROPE>),
      hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  ProfToken t1 = prof_begin(K_FWD, stream);
  hipLaunchKernelGGL((attn_fwd_kernel<D, ROPE>), dim3(nblk), dim3(256), C::LDS_BYTES, stream,
                     (const uint16_t*)a.q, (const uint16_t*)(ROPE ? a.kr : a.k),
                     (const uint16_t*)(a.ve ? a.vr : a.v), (const float*)a.kscale,
                     (const uint16_t*)a.rcos, (const uint16_t*)a.rsin, (uint16_t*)a.o, a.lse, a.T, a.H,
                     a.H / a.Hkv, W, a.eps, cpx);
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
