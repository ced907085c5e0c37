// dQ kernel of the backward pass (see attn_bwd.hip for the chain rule and the
// other kernels).  It lives in its own source because the build schedules it
// with the machine scheduler's ILP-maximising strategy, which suits dQ and
// spills registers in the dK/dV kernels.
//
// dq_hat = dS k_hat / sqrt(D), dq = r (dq_hat - q_hat mean_d(dq_hat q_hat))
//   (gradient of the unit-gain RMSNorm that the okx.com review and
//    "Autoresearch 深度教程" §7.3 place on q before the product)
#include <type_traits>

#include "common.h"
#include "band.h"
#include "kernels.h"
#include "profile.h"

namespace swattn {

// ------------------------------------------------------------------ dQ
// Workgroup: 4 waves; wave w owns queries i0 + 32 w + c.  Key blocks of 32
// rows (K, V and their kscale) stream through the band in three LDS buffers
// filled by direct-to-LDS loads one step ahead.  Per block i:
//   A(i): S^T = K Q_hat^T and dP^T = V dO^T   (queries in lanes, keys in registers)
//   B(i): dS' = exp2(S^T kscale - lse log2 e) (dP^T - Delta) kscale      (VALU)
//   C(i): dQ^T += K^T dS'^T   (K^T read transposed from the row-major K tile)
// As in the dK/dV kernel the loop issues A(i+1), C(i), then B(i+1).  The
// kernel fits two waves per SIMD (three at D = 64), so the hardware also
// overlaps several workgroups' phases.
template <int D, bool ROPE>
struct DqCfg {
  static constexpr int BM = 128;   // queries per workgroup (32 per wave)
  static constexpr int BN = 32;    // keys per step
  static constexpr int NBUF = 3;
  static constexpr int KS = D / 16;
  static constexpr int NB = D / 32;
  static constexpr int P = D + 24;
  using Tile = DmaTile<D, BN, P, 1 + ROPE>;
  static constexpr int V_B = Tile::BYTES;          // V tile after the K tile
  static constexpr int ST_B = 2 * Tile::BYTES;     // kscale (256 B), 3 spare
  static constexpr int STAGE = ST_B + 1024;
  static constexpr int LDS_BYTES = NBUF * STAGE;
  static constexpr int NPS = 2 * Tile::NIW + 1;    // direct loads per wave per step
};

// ROPE: k holds the rotated keys; the queries are rotated in the prologue and
// dQ goes back through the transposed rotation in the epilogue.
template <int D, bool ROPE>
__global__ __launch_bounds__(256, D >= 256 ? 1 : (D <= 64 ? 3 : 2)) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ o,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ kscale, const uint16_t* __restrict__ rcos,
    const uint16_t* __restrict__ rsin, uint16_t* __restrict__ qhat, float* __restrict__ delta,
    float* __restrict__ lse2, uint16_t* __restrict__ dq, int T, int H, int G, int W, float eps,
    int tile_group, int cpx) {
  using C = DqCfg<D, ROPE>;
  extern __shared__ __align__(16) unsigned char smem[];

  const int nqt = (T + C::BM - 1) / C::BM;
  const int lid = xcd_remap_paired(blockIdx.x, gridDim.x, cpx);
  int bh, qt;
  query_tile_of(lid, nqt, gridDim.x / nqt, tile_group, &bh, &qt);
  const int b = bh / H, h = bh % H;
  const int i0 = qt * C::BM;

  const int tid = threadIdx.x;
  const int w = uniform(tid >> 6);
  const int lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int rs = H * D;
  const long long rsb = 2LL * rs;
  const long long slice_bytes = (long long)(T - 1) * rsb + 2 * D;
  const size_t sbase = ((size_t)b * T * H + h) * D;
  const size_t sb = (size_t)bh * T;
  const int Hkv = H / G;
  const int rs_kv = Hkv * D;               // K / V row stride (elements)
  const long long rsb_kv = 2LL * rs_kv;
  const long long kslice_bytes = (long long)(T - 1) * rsb_kv + 2 * D;
  const size_t kvbase = ((size_t)b * T * Hkv + h / G) * D;

  // ---- the backward's per-query preparation, for this kernel and the dK/dV
  // kernel that runs after it: r_q and q_hat = q r_q (bf16), Delta = dO . o,
  // lse log2(e).  Lane (g, c) holds query qw0 + c, d = 16 ks + 8 g + 0..7.
  const int qw0 = i0 + 32 * w;
  const int qi = qw0 + c;
  using RS = RowStage32<D>;
  static_assert(4 * RS::BYTES <= C::LDS_BYTES, "row staging fits in the step buffers");
  u32x4 qf[C::KS], df[C::KS];
  float r_q, dlt, lse_q;
  {
    const rsrc_t rqr = make_rsrc(q + sbase + (size_t)qw0 * rs, slice_bytes - qw0 * rsb);
    const rsrc_t rdo = make_rsrc(dout + sbase + (size_t)qw0 * rs, slice_bytes - qw0 * rsb);
    const rsrc_t ror = make_rsrc(o + sbase + (size_t)qw0 * rs, slice_bytes - qw0 * rsb);
    // every load goes out before the first use: left to itself the compiler
    // issued a few, waited, and issued the rest, several round trips in a row
    u32x4 of[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      qf[ks] = bload16(rqr, (c * rs + 16 * ks + 8 * g) * 2);
      df[ks] = bload16(rdo, (c * rs + 16 * ks + 8 * g) * 2);
      of[ks] = bload16(ror, (c * rs + 16 * ks + 8 * g) * 2);
    }
    lse_q = bload4f(make_rsrc(lse + sb, 4LL * T), qi * 4);
    __builtin_amdgcn_sched_barrier(0);
    float dd = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dd += bf_lo(df[ks][e]) * bf_lo(of[ks][e]) + bf_hi(df[ks][e]) * bf_hi(of[ks][e]);
    }
    dd += __shfl_xor(dd, 32);
    dlt = dd;
    r_q = normalise_query<D, ROPE>(qf, rcos, rsin, qw0, c, g, T, eps);
    // q_hat rows leave through LDS (whole-row stores); the step buffers are
    // not in use yet
    const int slot = RS::BYTES * w;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      RS::put(smem, slot, c, 16 * ks + 8 * g, u32x2{qf[ks][0], qf[ks][1]});
      RS::put(smem, slot, c, 16 * ks + 8 * g + 4, u32x2{qf[ks][2], qf[ks][3]});
    }
    RS::store_rows(smem, slot, make_rsrc(qhat + sbase + (size_t)qw0 * rs, slice_bytes - qw0 * rsb), rs, lane);
  }
  const float lq = lse_q * kLog2e;
  if (g == 0) {
    bstore4f(dlt, make_rsrc(delta + sb, 4LL * T), qi * 4);
    bstore4f(lq, make_rsrc(lse2 + sb, 4LL * T), qi * 4);
  }
  __syncthreads();   // every wave is done with its staging slot before the loads land there

  f32x16 acc[C::NB];
#pragma unroll
  for (int n = 0; n < C::NB; ++n) acc[n] = f32x16{};

  int kv_lo, kv_hi;
  kv_range(i0, i0 + C::BM - 1, T, W, &kv_lo, &kv_hi);
  const int jb0 = kv_lo / C::BN;
  const int nsteps = kv_hi / C::BN - jb0 + 1;
  // Step i visits key block blk(i) = jb0 + ((i - jb0) mod nsteps): the band
  // rotated so that the query tiles of one (batch, head) whose bands have the
  // same length, which run at the same time, read the same key block at
  // about the same time (most reads then hit in L2).  dQ sums over the blocks
  // in that order.
  const int rot = nsteps > 0 ? (nsteps - jb0 % nsteps) % nsteps : 0;
  auto blk = [&](int i) {   // 0 <= i < nsteps
    const int x = i + rot;
    return jb0 + (x >= nsteps ? x - nsteps : x);
  };

  // ---- direct-to-LDS staging of one key step
  typename C::Tile tile;
  tile.init(w, lane, rs_kv);
  const u32x4 rks = make_desc(kscale + (size_t)(b * Hkv + h / G) * T, w == 0 ? 4LL * T : 0);   // wave 0 loads kscale
  const uint16_t* k_s = k + kvbase;
  const uint16_t* v_s = v + kvbase;
  // remaining bytes of the key slices from row r0 on, below 2^32 (unsigned arithmetic)
  const uint32_t kbytes_u = (uint32_t)kslice_bytes, krow_u = (uint32_t)rsb_kv;
  auto issue_step = [&](int step, int base) {
    const int r0 = blk(step) * C::BN;
    const uint32_t nb = kbytes_u - (uint32_t)r0 * krow_u;
    tile.issue(make_desc_u(k_s + (size_t)r0 * rs_kv, nb), smem, base, w);
    tile.issue(make_desc_u(v_s + (size_t)r0 * rs_kv, nb), smem, base + C::V_B, w);
    dma_row4(rks, smem, base + C::ST_B + 256 * w, (r0 + lane) * 4);
  };

  const int a_off = 2 * (c * C::P + 8 * g);
  const int t_off = 2 * tr_off(lane, C::P);
  const int k_off = C::ST_B + 16 * g;   // kscale of the lane's key quads

  f32x16 s_acc, dp_acc;
  u32x4 dsf[2];

  auto stage_a = [&](int base) {
    const int va = base + a_off;
    s_acc = f32x16{};
    dp_acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      s_acc = mfma32(lds16(smem, va + 32 * ks), qf[ks], s_acc);
      dp_acc = mfma32(lds16(smem, va + C::V_B + 32 * ks), df[ks], dp_acc);
    }
  };
  // lane (g, c), register r: key j0 + 8 (r/4) + 4 g + r%4, query qi
  auto stage_b = [&](int base, int step, auto masked_c) {
    constexpr bool MASKED = decltype(masked_c)::value;
    const int vk = base + k_off;
    const int t0 = blk(step) * C::BN + 4 * g + W - qi;  // kv visible iff 0 <= kv - (qi - W) <= W
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 k4 = lds16f(smem, vk + 32 * q4);
      float p[4], ds[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(s_acc[4 * q4 + e] * k4[e] - lq);
      if (MASKED) {
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = ((unsigned)(t0 + 8 * q4 + e) <= (unsigned)W) ? p[e] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) ds[e] = p[e] * (dp_acc[4 * q4 + e] - dlt) * k4[e];
      const int st = q4 >> 1, el = 2 * (q4 & 1);
      dsf[st][el] = pack_bf16(ds[0], ds[1]);
      dsf[st][el + 1] = pack_bf16(ds[2], ds[3]);
    }
  };
  // dQ^T[d, q] += K^T[d, kv] (dS kscale)^T[kv, q]
  auto stage_c = [&](int base) {
    const int vt = base + t_off;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int n = 0; n < C::NB; ++n) {
        constexpr int R8 = 2 * 8 * C::P;
        const int o = 2 * (16 * s2 * C::P + 32 * n);
        const u32x2 a0 = lds_tr4b(smem, vt + o), a1 = lds_tr4b(smem, vt + o + R8);
        acc[n] = mfma32(u32x4{a0[0], a0[1], a1[0], a1[1]}, dsf[s2], acc[n]);
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

  // One step: A(it+1), C(it), B(it+1), with the order written out in fenced
  // regions, as in the dK/dV kernel: S's products (the V operands read among
  // them), then dP's with twelve of B's sixteen exponentials (P needs only S),
  // then C's products, each after the transposing reads of the product CA
  // places later, with the last four exponentials and dS' = P (dP - Delta)
  // kscale with its packing.  B(it+1) writes separate registers that C(it+1)
  // takes over.
  auto step_body = [&](int it, auto masked_c) {
    {
      constexpr bool MASKED = decltype(masked_c)::value;
      constexpr int NC = 2 * C::NB;   // C's products, m = NB s2 + n
      constexpr int CA = 2;
      constexpr int R8 = 2 * 8 * C::P;
      const int va = b1 + a_off, vk = b1 + k_off, vt = b0 + t_off;
      auto c_read = [&](int m) {
        const int s2 = m / C::NB, n = m % C::NB;
        const int off = vt + 2 * (16 * s2 * C::P + 32 * n);
        const u32x2 x0 = lds_tr4b(smem, off), x1 = lds_tr4b(smem, off + R8);
        return u32x4{x0[0], x0[1], x1[0], x1[1]};
      };
      constexpr int KA = 4;   // S operands read ahead
      u32x4 ka[C::KS], vv[C::KS], cop[NC];
      f32x4 k4s[4];
#pragma unroll
      for (int ks = 0; ks < KA; ++ks) ka[ks] = lds16(smem, va + 32 * ks);
#pragma unroll
      for (int m = 0; m < CA; ++m) cop[m] = c_read(m);
      __builtin_amdgcn_sched_barrier(0);
      s_acc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        if (ks + KA < C::KS) ka[ks + KA] = lds16(smem, va + 32 * (ks + KA));
        s_acc = mfma32(ka[ks], qf[ks], s_acc);
        if (ks >= C::KS - KA) vv[ks - (C::KS - KA)] = lds16(smem, va + C::V_B + 32 * (ks - (C::KS - KA)));
        if (ks == C::KS - 2) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) k4s[q4] = lds16f(smem, vk + 32 * q4);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // B(it+1) element r (register r: key j0 + 8 (r / 4) + 4 g + r % 4, query
      // qi), as stage_b computes it, each value pinned where it is made
      const int t0 = blk(it + 1) * C::BN + 4 * g + W - qi;
      float pe[16], de[16];
      auto p_elem = [&](int r) {
        const int q4 = r >> 2, i = r & 3;
        float pr = __builtin_amdgcn_exp2f(s_acc[r] * k4s[q4][i] - lq);
        if (MASKED) pr = ((unsigned)(t0 + 8 * q4 + i) <= (unsigned)W) ? pr : 0.f;
        pe[r] = pr;
        asm volatile("" : "+v"(pe[r]));
      };
      constexpr int NPA = 12;
      dp_acc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        if (ks + KA < C::KS) vv[ks + KA] = lds16(smem, va + C::V_B + 32 * (ks + KA));
        dp_acc = mfma32(vv[ks], df[ks], dp_acc);
#pragma unroll
        for (int r = NPA * ks / C::KS; r < NPA * (ks + 1) / C::KS; ++r) p_elem(r);
        __builtin_amdgcn_sched_barrier(0);
      }
      constexpr int EPM = 16 / NC;   // dS elements per product of C
      u32x4 dn[2];
#pragma unroll
      for (int m = 0; m < NC; ++m) {
        if (m + CA < NC) cop[m + CA] = c_read(m + CA);
        const int s2 = m / C::NB, n = m % C::NB;
        acc[n] = mfma32(cop[m], dsf[s2], acc[n]);
#pragma unroll
        for (int r = NPA + (16 - NPA) * m / NC; r < NPA + (16 - NPA) * (m + 1) / NC; ++r) p_elem(r);
#pragma unroll
        for (int k = 0; k < EPM; ++k) {
          const int r = EPM * m + k, q4 = r >> 2, i = r & 3;
          de[r] = pe[r] * (dp_acc[r] - dlt) * k4s[q4][i];
          asm volatile("" : "+v"(de[r]));
          if (r & 1) {
            const int st = q4 >> 1, el = 2 * (q4 & 1) + (i >> 1);
            dn[st][el] = pack_bf16(de[r - 1], de[r]);
            asm volatile("" : "+v"(dn[st][el]));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      dsf[0] = dn[0];
      dsf[1] = dn[1];
    }
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
  const int nloop = nsteps - 1;
  // At D <= 128 (two or three waves per SIMD) a wave passes over the blocks
  // none of its queries sees (keys after its last query, or before its first
  // query's window) with only the step's wait, barrier and loads, and the
  // other waves on the SIMD take the issue slots.  Blocks sv_lo .. sv_hi may
  // be seen.  A skipped step has blocks it and it + 1 both unseen: the dS of
  // an unseen block is zero (its P is masked), so C adds nothing for it.  The
  // steps on either side of the skipped runs take the masked body, whose C or
  // A and B then work on an unseen block and add zeros.
  int sv_lo = 0, sv_hi = nsteps - 1;
  if constexpr (D <= 128) {
    const int lo = qw0 - W - (C::BN - 1);           // a block starting below lo is unseen
    sv_lo = imax(0, (lo > 0 ? (lo + C::BN - 1) / C::BN : 0) - jb0);
    sv_hi = imin(nsteps - 1, (qw0 + 31) / C::BN - jb0);
  }
  auto skip_step = [&](int it) {
    wait_vmcnt<0>();            // step it + 2 landed
    __syncthreads();
    if (it + 3 < nsteps) issue_step(it + 3, b0);   // buffer of step it, consumed
    const int t = b0;
    b0 = b1;
    b1 = b2;
    b2 = t;
  };
  // Body it works on A and B of block b = blk(it + 1) - jb0 (relative) and C
  // of the block before it.  In band order (b rising) the bodies run: skipped
  // while b < sv_lo, masked while b < full_lo, unmasked up to full_hi, masked
  // up to sv_hi + 1 (C of block sv_hi), skipped after.  The rotation splits
  // the steps into two such runs: b = rot + 1 .. nsteps - 1, then b = 0 ..
  // rot - 1, whose first step (b = 0) takes C of block nsteps - 1 and runs
  // masked unless that block is unseen too.
  for (int pass = 0; pass < 2; ++pass) {
    const int b_lo = pass == 0 ? rot + 1 : 0, b_hi = pass == 0 ? nsteps - 1 : rot - 1;
    const int off = pass == 0 ? -rot : nsteps - rot;   // it = b - 1 + off
    const int w0 = (pass == 1 && sv_hi >= nsteps - 1) ? 1 : 0;
    const int it_end = b_hi + off;
    int it = b_lo - 1 + off;
    for (; it < imin(b_lo - 1 + off + w0, it_end); ++it) step_body(it, masked);
    for (; it < imin(sv_lo - 1 + off, it_end); ++it) skip_step(it);
    for (; it < imin(full_lo - 1 + off, it_end); ++it) step_body(it, masked);
    for (; it < imin(full_hi + off, it_end); ++it) step_body(it, unmasked);
    for (; it < imin(sv_hi + 1 + off, it_end); ++it) step_body(it, masked);
    for (; it < it_end; ++it) skip_step(it);
  }
  if (nsteps > 0 && blk(nsteps - 1) - jb0 >= sv_lo && blk(nsteps - 1) - jb0 <= sv_hi) stage_c(b0);

  // ---- epilogue: dq_hat = acc / log2(e); RMSNorm backward of q (stores past
  // T dropped).  The norm's output x_hat is the bf16 q_hat that fed the S
  // products (qf); it moves from the fragment layout (d = 16 ks + 8 g + j) to
  // the accumulators' (d = 32 n + 8 q4 + 4 g + e) through the wave's LDS slot,
  // and dq goes out through the same slot (the step buffers, free once every
  // wave is past its last product), so global memory sees whole rows.
  const float r = r_q;
  // rotary tables of query qi (channels 32 n + 8 q4 + 4 g + e, n < NB / 2,
  // pair with n + NB / 2), in flight with the last products
  u32x2 tc[C::NB / 2][4], tsn[C::NB / 2][4];
  if constexpr (ROPE) {
    const long long tb = (long long)(T - qw0) * D;
    const rsrc_t rc = make_rsrc(rcos + (size_t)qw0 * (D / 2), tb);
    const rsrc_t rn = make_rsrc(rsin + (size_t)qw0 * (D / 2), tb);
#pragma unroll
    for (int n = 0; n < C::NB / 2; ++n)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int off = (c * (D / 2) + 32 * n + 8 * q4 + 4 * g) * 2;
        tc[n][q4] = bload8(rc, off);
        tsn[n][q4] = bload8(rn, off);
      }
  }
  __syncthreads();
  const int slot = RS::BYTES * w;
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    RS::put(smem, slot, c, 16 * ks + 8 * g, u32x2{qf[ks][0], qf[ks][1]});
    RS::put(smem, slot, c, 16 * ks + 8 * g + 4, u32x2{qf[ks][2], qf[ks][3]});
  }
  float dot = 0.f;
  f32x16 xh[C::NB];
  if constexpr (ROPE) {
    // the norm's input is the rotated q (x_hat is its normalised form); the
    // table entries take the gradient back through the rotation
#pragma unroll
    for (int n = 0; n < C::NB; ++n)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const u32x2 qq = RS::get(smem, slot, c, 32 * n + 8 * q4 + 4 * g);
        const float x[4] = {bf_lo(qq[0]), bf_hi(qq[0]), bf_lo(qq[1]), bf_hi(qq[1])};
#pragma unroll
        for (int e = 0; e < 4; ++e) xh[n][4 * q4 + e] = x[e];
      }
#pragma unroll
    for (int n = 0; n < C::NB; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        acc[n][i] *= (1.0f / kLog2e);
        dot += acc[n][i] * xh[n][i];
      }
    dot += __shfl_xor(dot, 32);
    const float mean = dot * (1.0f / D);
#pragma unroll
    for (int n = 0; n < C::NB / 2; ++n)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float y1[4], y2[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y1[e] = r * (acc[n][4 * q4 + e] - xh[n][4 * q4 + e] * mean);
          y2[e] = r * (acc[n + C::NB / 2][4 * q4 + e] - xh[n + C::NB / 2][4 * q4 + e] * mean);
        }
        rope4_bwd(y1, y2, tc[n][q4], tsn[n][q4]);
        RS::put(smem, slot, c, 32 * n + 8 * q4 + 4 * g, u32x2{pack_bf16(y1[0], y1[1]), pack_bf16(y1[2], y1[3])});
        RS::put(smem, slot, c, 32 * (n + C::NB / 2) + 8 * q4 + 4 * g,
                u32x2{pack_bf16(y2[0], y2[1]), pack_bf16(y2[2], y2[3])});
      }
  } else {
#pragma unroll
  for (int n = 0; n < C::NB; ++n)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const u32x2 qq = RS::get(smem, slot, c, 32 * n + 8 * q4 + 4 * g);
      const float x[4] = {bf_lo(qq[0]), bf_hi(qq[0]), bf_lo(qq[1]), bf_hi(qq[1])};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xh[n][4 * q4 + e] = x[e];
        acc[n][4 * q4 + e] *= (1.0f / kLog2e);
        dot += acc[n][4 * q4 + e] * xh[n][4 * q4 + e];
      }
    }
  dot += __shfl_xor(dot, 32);
  const float mean = dot * (1.0f / D);
#pragma unroll
  for (int n = 0; n < C::NB; ++n)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = r * (acc[n][4 * q4 + e] - xh[n][4 * q4 + e] * mean);
      RS::put(smem, slot, c, 32 * n + 8 * q4 + 4 * g, u32x2{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])});
    }
  }
  RS::store_rows(smem, slot, make_rsrc(dq + sbase + (size_t)qw0 * rs, slice_bytes - qw0 * rsb), rs, lane);
}


template <int D, bool ROPE>
static hipError_t launch_bwd_dq_d(const BwdArgs& a, const uint16_t* kk, const uint16_t* vv, int W, int ncu,
                                  hipStream_t stream) {
  using C = DqCfg<D, ROPE>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(bwd_dq_kernel<D, ROPE>),
      hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  const int G = a.H / a.Hkv;
  const int nqt = (a.T + C::BM - 1) / C::BM;
  // slices per group of the heaviest-first order: wider when the grid fills
  // the CUs' workgroup slots only a few times over
  const long long slots = (long long)ncu * (D >= 256 ? 1 : (D <= 64 ? 3 : 2));
  const long long nblk = (long long)nqt * a.B * a.H;
  const int tile_group = nblk <= kDqFewWaves * slots ? kTileGroupDqFew : kTileGroupDq;
  // a grid that the CUs hold at once pairs heavy with light tiles per CU
  const int cpx = (nblk <= slots && ncu % 8 == 0) ? ncu / 8 : 0;
  ProfToken t2 = prof_begin(K_BWD_DQ, stream);
  hipLaunchKernelGGL((bwd_dq_kernel<D, ROPE>), dim3(nqt * a.B * a.H), dim3(256), C::LDS_BYTES, stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.o, kk, vv,
                     (const uint16_t*)a.dout, a.lse, (const float*)a.kscale,
                     (const uint16_t*)a.rcos, (const uint16_t*)a.rsin, (uint16_t*)a.qhat, a.delta,
                     a.lse2, (uint16_t*)a.dq, a.T, a.H, G, W, a.eps, tile_group, cpx);
  prof_end(t2);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, const uint16_t* kk, const uint16_t* vv, int W, int ncu,
                         hipStream_t stream) {
  const bool rope = a.rcos != nullptr;
  if (a.D == 256)
    return rope ? launch_bwd_dq_d<256, true>(a, kk, vv, W, ncu, stream)
                : launch_bwd_dq_d<256, false>(a, kk, vv, W, ncu, stream);
  if (a.D == 128)
    return rope ? launch_bwd_dq_d<128, true>(a, kk, vv, W, ncu, stream)
                : launch_bwd_dq_d<128, false>(a, kk, vv, W, ncu, stream);
  return rope ? launch_bwd_dq_d<64, true>(a, kk, vv, W, ncu, stream)
              : launch_bwd_dq_d<64, false>(a, kk, vv, W, ncu, stream);
}

}  // namespace swattn
