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
// With grouped key/value heads (G = H / H_kv query heads read one key/value
// head, "Autoresearch 深度教程" §7.3), dk and dv of a shared head sum the
// contributions of its G query heads.  With the rotary embedding (§7.4) the
// norm's input is the rotated q or k, and dq, dk go back through the
// transposed rotation.
//
// Kernels, in launch order:
//   key_prep:   kscale = log2(e) / sqrt(D) / rms(k) for every key (prep.hip).
//   bwd_dq:     (attn_bwd_dq.hip) a workgroup owns 128 queries (32 per wave):
//               it normalises its queries, computes Delta = dO . o and writes
//               q_hat, Delta and lse log2(e) for bwd_dkdv, then walks the key
//               tiles of its band, recomputing S and dP; the RMSNorm backward
//               of Q runs in the epilogue.  No atomics: dQ is deterministic.
//   bwd_dkdv:   persistent; a tile is 128 keys (32 per wave) of one key/value
//               head, walking the query blocks of its band in each of the
//               head's G query heads; dV^T and dK_hat^T stay in registers; the
//               RMSNorm backward of K runs in the epilogue.  At head size 256,
//               bwd_dkdv_split takes its place: two waves share each 32-key
//               block, one for S, P and dV, the other for dP, dS and dK.
#include <type_traits>

#include "common.h"
#include "band.h"
#include "kernels.h"
#include "profile.h"

namespace swattn {

// ------------------------------------------------------------------ dK / dV
// Persistent: one workgroup per CU (two at head size 64, whose registers and
// LDS fit twice) walks a list of key tiles of 128 keys.  In
// a tile, wave w owns keys j0 + 32 w + c; query blocks of 32 rows (q_hat, dO
// and their lse, Delta) stream through three LDS buffers filled by
// direct-to-LDS loads one step ahead, and the stream runs on across tile
// boundaries, so a tile's first blocks are in LDS when its predecessor ends.
// The next tile's K and V rows are prefetched into LDS during the current
// tile.  Per block i:
//   A(i): S = Q_hat K^T and dP = dO V^T    (keys in lanes, queries in registers)
//   B(i): P = exp2(S kscale - lse log2 e), dS = P (dP - Delta)      (VALU)
//   C(i): dV^T += dO^T P, dK_hat^T += Q_hat^T dS  (transposed operands read
//         straight from the row-major tiles)
// The loop issues A(i+1) and C(i) back to back, then B(i+1): the softmax of
// the next block runs on the VALU while the matrix cores still work through
// C(i), and LDS reads for both products are in flight together.
//
// A tile of a key/value head shared by G query heads walks its band G times,
// once per query head, and accumulates all of them before the epilogue.
//
// Tiles are split into 8 contiguous ranges, one per XCD (workgroup b runs on
// XCD b % 8), so the tiles of one (batch, head) share that XCD's L2; inside a
// range, rounds of G8 consecutive tiles go to the G8 workgroups in the order
// of persistent_tile (band.h), which spreads the light tiles of the causal
// tail over the workgroups.
template <int D, bool GROUPED, bool ROPE>
struct DkdvCfg {
  static constexpr int BNK = 128;       // keys per tile (32 per wave)
  static constexpr int BMQ = 32;        // queries per step
  static constexpr int NBUF = 3;
  static constexpr int KS = D / 16;
  static constexpr int NB = D / 32;
  // q_hat / dO row pitch (bf16): an odd multiple of 16 bytes; at D = 64 the
  // narrower pitch keeps the workgroup within half the LDS
  static constexpr int P = D + (D <= 64 ? 8 : 24);
  static constexpr int PK = D + 8;      // K / V row pitch in the prefetch region
  using Tile = DmaTileV<BMQ * P / 8, 4, 1 + GROUPED + 2 * ROPE>;
  using KVTile = DmaTileV<BNK * PK / 8, 4, 1 + GROUPED + 2 * ROPE>;
  static constexpr int DO_B = Tile::BYTES;          // dO tile after the q_hat tile
  static constexpr int ST_B = 2 * Tile::BYTES;      // 4 x 256 B: spare, spare, lse2, Delta
  static constexpr int STAGE = ST_B + 1024;
  static constexpr int KV_B = NBUF * STAGE;         // K rows, then V rows of the next tile
  static constexpr int OP = D + 8;                  // output staging row pitch (bf16)
  static constexpr int OUT_SLOT = 32 * OP * 2;      // one wave's 32 x D bf16 block
  static constexpr int XO_B = KV_B + 2 * KVTile::BYTES;   // staging slots of waves 2 and 3
  static constexpr int LDS_BYTES = XO_B + 2 * OUT_SLOT;
  static constexpr int NSTORE = 2 * (32 * D / 8 / 64);    // epilogue stores per lane (dK and dV)
  static_assert(2 * OUT_SLOT <= STAGE, "waves 0 and 1 stage their outputs in a freed step buffer");
  static_assert(LDS_BYTES <= (D <= 64 ? 80 : 160) * 1024, "fits the LDS of one CU (half of it at D = 64)");
  static_assert(D <= 128, "head size 256 takes bwd_dkdv_split_kernel");
};

// GROUPED = false is the plain multi-head case, compiled with G = 1 so that the
// walk over the query heads of a group folds away.  ROPE: k holds the rotated
// keys, and dK goes back through the transposed rotation in the epilogue.
// With the value-embedding gate (ve not null), v holds v + gate ve and the
// epilogue also writes dve = gate dV and dz = (dV . ve) gate (1 - gate / 2),
// the gradient of the gate's pre-sigmoid input ([B, T, Hkv]).
// At D = 128 a wave holds its accumulators and K / V rows in 512 registers, one
// wave per SIMD; at D = 64 they fit in 256, and two workgroups share a CU.
template <int D, bool GROUPED, bool ROPE, bool MIRROR>
__global__ __launch_bounds__(256, D <= 64 ? 2 : 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ qhat, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse2, const float* __restrict__ delta,
    const float* __restrict__ kscale, const uint16_t* __restrict__ rcos,
    const uint16_t* __restrict__ rsin, const uint16_t* __restrict__ ve,
    const float* __restrict__ gate, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
    uint16_t* __restrict__ dve, float* __restrict__ dz, int T, int H, int G_arg, int W, int nkt,
    int ntiles, int mirror0) {
  using C = DkdvCfg<D, GROUPED, ROPE>;
  const int G = GROUPED ? G_arg : 1;
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x;
  const int w = uniform(tid >> 6);
  const int lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int rs = H * D;                 // query-side row stride (q_hat, dO)
  const long long rsb = 2LL * rs;
  const long long slice_bytes = (long long)(T - 1) * rsb + 2 * D;
  const int Hkv = H / G;
  const int rs_kv = Hkv * D;            // key-side row stride (K, V, dK, dV)
  const long long rsb_kv = 2LL * rs_kv;
  const long long kslice_bytes = (long long)(T - 1) * rsb_kv + 2 * D;

  // ---- tile list of this workgroup
  int xr = 0, ws = blockIdx.x, G8 = gridDim.x, N8 = ntiles;
  if ((ntiles & 7) == 0 && (gridDim.x & 7) == 0) {
    xr = blockIdx.x & 7;
    ws = blockIdx.x >> 3;
    G8 = gridDim.x >> 3;
    N8 = ntiles >> 3;
  }
  // MIRROR: the schedule mirrors rounds mirror0 .. of rounds 0 .. (band.h);
  // without it, the plain rotation
  auto tile_at = [&](int i) {   // i-th tile of this workgroup, or -1
    if constexpr (MIRROR) {
      const int r = schedule_tile(i, ws, G8, N8, mirror0);
      return r >= 0 ? xr * N8 + r : -1;
    } else {
      const int r = i * G8 + (ws + 7 * i) % G8;
      return (i * G8 < N8 && r < N8) ? xr * N8 + r : -1;
    }
  };
  struct TileGeo {
    int bh, b, hk, j0, qb0, nsteps;   // bh = b Hkv + hk: the key/value slice
  };
  auto geo = [&](int t) {
    TileGeo tg;
    tg.bh = t / nkt;
    tg.b = tg.bh / Hkv;
    tg.hk = tg.bh - tg.b * Hkv;
    tg.j0 = (t % nkt) * C::BNK;
    int q_lo, q_hi;
    const bool any = q_range(tg.j0, tg.j0 + C::BNK - 1, T, W, &q_lo, &q_hi);
    tg.qb0 = any ? q_lo / C::BMQ : 0;
    tg.nsteps = any ? q_hi / C::BMQ - tg.qb0 + 1 : 0;
    return tg;
  };
  auto kv_base = [&](const TileGeo& tg) { return ((size_t)tg.b * T * Hkv + tg.hk) * D; };

  // ---- direct-to-LDS staging
  typename C::Tile tile;
  tile.init(w, lane, [&](int qc) {
    const int r = qc / (C::P / 8), ch = qc % (C::P / 8);
    return (r < C::BMQ && ch < D / 8) ? (r * rs + 8 * ch) * 2 : -1;
  });
  typename C::KVTile kvtile;
  kvtile.init(w, lane, [&](int qc) {
    const int r = qc / (C::PK / 8), ch = qc % (C::PK / 8);
    return (ch < D / 8) ? (r * rs_kv + 8 * ch) * 2 : -1;
  });
  // The stream of query blocks runs across tiles (and, in a tile, across the
  // G query heads of its key/value head).  A plan holds the source
  // of the next block (computed with scalar control flow outside the
  // scheduled regions); issuing it is branch-free, so the loads interleave
  // with the MFMAs.  Past the end of the stream a plan has no bytes in range
  // and its loads write zeros into a free buffer.  Waves 2 and 3 (fewer tile
  // loads) fetch lse2 and Delta; waves 0 and 1 load into spare slots.
  struct DmaPlan {
    const uint16_t* qh;
    const uint16_t* dO;
    const float* st;
    uint32_t nbytes;    // remaining bytes of the slice, below 2^32
    int nst;
    int r0;
  };
  // The cursor: the next block is step ds of query head dgi of the dt-th tile.
  // Its source pointers advance by one block per step and are recomputed only
  // when the cursor moves to another query head or tile.
  int dt = 0, ds = 0, dgi = 0;
  TileGeo dgeo;
  const uint16_t* cq = qhat;
  const uint16_t* cdo = dout;
  const float* cst = w == 2 ? lse2 : delta;
  uint32_t cbytes = 0;
  int cr0 = 0;
  auto seek_head = [&]() {
    const int hq = dgeo.hk * G + dgi;
    const size_t sbase = ((size_t)dgeo.b * T * H + hq) * D;
    cr0 = dgeo.qb0 * C::BMQ;
    cq = qhat + sbase + (size_t)cr0 * rs;
    cdo = dout + sbase + (size_t)cr0 * rs;
    cbytes = (uint32_t)(slice_bytes - cr0 * rsb);
    cst = (w == 2 ? lse2 : delta) + (size_t)(dgeo.b * H + hq) * T;
  };
  int tcur = tile_at(0);
  if (tcur >= 0) {
    dgeo = geo(tcur);
    seek_head();
  }
  auto plan_next = [&]() {
    while (tcur >= 0 && ds >= dgeo.nsteps) {
      ds = 0;
      if (++dgi >= G) {
        dgi = 0;
        ++dt;
        tcur = tile_at(dt);
        if (tcur >= 0) dgeo = geo(tcur);
      }
      if (tcur >= 0) seek_head();
    }
    DmaPlan pl;
    const bool ok = tcur >= 0;
    pl.qh = cq;
    pl.dO = cdo;
    pl.st = cst;
    pl.r0 = ok ? cr0 : 0;
    pl.nbytes = ok ? cbytes : 0u;
    pl.nst = (ok && w >= 2) ? 4 * T : 0;
    if (ok) {
      ++ds;
      cq += (size_t)C::BMQ * rs;
      cdo += (size_t)C::BMQ * rs;
      cbytes -= (uint32_t)(C::BMQ * rsb);
      cr0 += C::BMQ;
    }
    return pl;
  };
  auto issue_plan = [&](const DmaPlan& pl, int base) {
    tile.issue(make_desc_u(pl.qh, pl.nbytes), smem, base, w);
    tile.issue(make_desc_u(pl.dO, pl.nbytes), smem, base + C::DO_B, w);
    dma_row4(make_desc(pl.st, pl.nst), smem, base + C::ST_B + 256 * w, (pl.r0 + lane) * 4);
  };
  // the same loads one instruction at a time: j < NDMA (q_hat, then dO, then
  // the statistics row)
  constexpr int NDMA = 2 * C::Tile::NIW + 1;
  auto issue_plan_one = [&](const u32x4& dq_, const u32x4& ddo, const u32x4& dst, const DmaPlan& pl, int base,
                            int j) {
    if (j < C::Tile::NIW) tile.issue_one(dq_, smem, base, w, j);
    else if (j < 2 * C::Tile::NIW) tile.issue_one(ddo, smem, base + C::DO_B, w, j - C::Tile::NIW);
    else dma_row4(dst, smem, base + C::ST_B + 256 * w, (pl.r0 + lane) * 4);
  };
  auto issue_kv = [&](const TileGeo& tg) {
    const size_t sbase = kv_base(tg);
    kvtile.issue(make_desc(k + sbase + (size_t)tg.j0 * rs_kv, kslice_bytes - tg.j0 * rsb_kv), smem,
                 C::KV_B, w);
    kvtile.issue(make_desc(v + sbase + (size_t)tg.j0 * rs_kv, kslice_bytes - tg.j0 * rsb_kv), smem,
                 C::KV_B + C::KVTile::BYTES, w);
  };

  // per-lane byte offsets inside a stage buffer
  const int a_off = 2 * (c * C::P + 8 * g);          // row-major A operands (16-byte reads)
  const int t_off = 2 * tr_off(lane, C::P);          // transposed A operands
  const int l_off = C::ST_B + 512 + 16 * g;          // lse2 / Delta of the lane's query quads
  const int kv_off = C::KV_B + 2 * ((32 * w + c) * C::PK + 8 * g);   // owned K / V row

  // prologue of the stream: K / V rows of the first tile, blocks 0 and 1.
  // Invariant at a step's start: b0 holds block it, b1 block it + 1, b2 is free.
  int b0 = 2 * C::STAGE, b1 = 0, b2 = C::STAGE;
  if (tcur >= 0) issue_kv(dgeo);
  issue_plan(plan_next(), b1);
  issue_plan(plan_next(), b2);
  DmaPlan pnext = plan_next();

  u32x4 kf[C::KS], vf[C::KS];
  f32x16 acc_dv[C::NB], acc_dk[C::NB];
  f32x16 s_acc, dp_acc;
  u32x4 pf[2], dsf[2];
  const std::integral_constant<bool, true> masked{};
  const std::integral_constant<bool, false> unmasked{};

  for (int ti = 0;; ++ti) {
    const int t = tile_at(ti);
    if (t < 0) break;
    const TileGeo tg = geo(t);
    const int bh = tg.bh, j0 = tg.j0, qb0 = tg.qb0, nsteps = tg.nsteps;
    const size_t sbase = kv_base(tg);
    const int kw0 = j0 + 32 * w;
    const int kj = kw0 + c;

    // ---- tile prologue: the key scale is issued first; then steps 0 and 1 of
    // this tile and its K / V rows have landed (they are older than the
    // previous tile's dK / dV stores and that load, which may stay in flight);
    // the buffer of the previous tile's last step takes step 2
    const float ksc = bload4f(make_rsrc(kscale + (size_t)bh * T, 4LL * T), kj * 4);
    if (ti == 0) wait_vmcnt<0>();
    else wait_vmcnt<C::NSTORE + 1>();
    __syncthreads();
    // visibility on partial blocks: 0 <= q - kj <= lim, lim = min(W, T - 1 - kj)
    const int lim = imin(W, T - 1 - kj);
    {
      const int t_ = b0;
      b0 = b1;
      b1 = b2;
      b2 = t_;
    }
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      kf[ks] = lds16(smem, kv_off + 32 * ks);
      vf[ks] = lds16(smem, kv_off + C::KVTile::BYTES + 32 * ks);
    }
#pragma unroll
    for (int n = 0; n < C::NB; ++n) { acc_dv[n] = f32x16{}; acc_dk[n] = f32x16{}; }
    const bool kv_pending = tile_at(ti + 1) >= 0;   // prefetch of the next tile's K / V rows

    // A: scores and dP of one step
    auto stage_a = [&](int base) {
      const int va = base + a_off;
      s_acc = f32x16{};
      dp_acc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        s_acc = mfma32(lds16(smem, va + 32 * ks), kf[ks], s_acc);
        dp_acc = mfma32(lds16(smem, va + C::DO_B + 32 * ks), vf[ks], dp_acc);
      }
    };
    // B for the quad q4 of one step: probabilities and dS of the lane's queries
    // q0 + 8 q4 + 4 g + {0..3} (registers 4 q4 .. 4 q4 + 3 of S and dP), key kj,
    // given their lse2 (l4) and Delta (d4); the packed bf16 results go to
    // po / dso.  MASKED is a compile-time flag so each version is straight-line.
    auto stage_b4 = [&](int step, int q4, f32x4 l4, f32x4 d4, u32x4* po, u32x4* dso, auto masked_c) {
      constexpr bool MASKED = decltype(masked_c)::value;
      const int tq = (qb0 + step) * C::BMQ + 4 * g - kj;
      float p[4], dsv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(s_acc[4 * q4 + e] * ksc - l4[e]);
      if (MASKED) {
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = ((unsigned)(tq + 8 * q4 + e) <= (unsigned)lim) ? p[e] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) dsv[e] = p[e] * (dp_acc[4 * q4 + e] - d4[e]);
      const int st = q4 >> 1, el = 2 * (q4 & 1);
      po[st][el] = pack_bf16(p[0], p[1]);
      po[st][el + 1] = pack_bf16(p[2], p[3]);
      dso[st][el] = pack_bf16(dsv[0], dsv[1]);
      dso[st][el + 1] = pack_bf16(dsv[2], dsv[3]);
    };
    // B of a whole step (the first step of a tile)
    auto stage_b = [&](int base, int step, auto masked_c) {
      const int vl = base + l_off;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        stage_b4(step, q4, lds16f(smem, vl + 32 * q4), lds16f(smem, vl + 256 + 32 * q4), pf, dsf, masked_c);
    };
    // C: dV^T[d, kv] += dO^T[d, q] P[q, kv];  dK_hat^T[d, kv] += Q_hat^T[d, q] dS[q, kv]
    // (element j of a k-step s2 is query 16 s2 + 4 g + (j % 4) + 8 (j / 4)).
    // Product m = 2 (NB s2 + n) + x: x = 0 adds to dV^T block n, x = 1 to
    // dK_hat^T block n; its A operand comes from two transposing reads.
    constexpr int NM = 4 * C::NB;
    auto c_read = [&](int base, int m) {
      constexpr int R8 = 2 * 8 * C::P;
      const int s2 = m / (2 * C::NB), n = (m >> 1) % C::NB;
      const int off = base + t_off + ((m & 1) ? 0 : C::DO_B) + 2 * (16 * s2 * C::P + 32 * n);
      const u32x2 x0 = lds_tr4b(smem, off), x1 = lds_tr4b(smem, off + R8);
      return u32x4{x0[0], x0[1], x1[0], x1[1]};
    };
    auto c_mfma = [&](int m, u32x4 a) {
      const int s2 = m / (2 * C::NB), n = (m >> 1) % C::NB;
      if (m & 1) acc_dk[n] = mfma32(a, dsf[s2], acc_dk[n]);
      else acc_dv[n] = mfma32(a, pf[s2], acc_dv[n]);
    };
    auto stage_c = [&](int base) {
#pragma unroll
      for (int m = 0; m < NM; ++m) c_mfma(m, c_read(base, m));
    };

    stage_a(b0);
    stage_b(b0, 0, masked);

    // One pipelined step: A(it+1), C(it), B(it+1), then the hand-off of the
    // buffers.  At D = 128 one wave per SIMD issues in order, so a VALU,
    // scalar or memory instruction costs nothing only in the shadow of a
    // product it does not depend on.  Left to itself the compiler issued each LDS read right before
    // its product and waited for it there, and sank the softmax next to C's
    // products alone; the order is therefore written out in regions fenced with
    // scheduling barriers:
    //   the reads of S's first QA operands;
    //   S's products, with block it + 2's loads between them (one each) and
    //   the other reads of A(it+1) and B's lse2 (a burst of every read at the
    //   step's start left the matrix pipe idle until most had landed);
    //   dP's products, with NPA of B(it+1)'s exponentials between them (P needs
    //   only S), C(it)'s first CA operand reads and B's Delta read;
    //   C(it)'s products, each after the reads of the product CA places later,
    //   with the remaining exponentials, dS = P (dP - Delta) and the bf16
    //   packing between them, and the next block's plan halfway.
    // B(it+1) writes separate registers that C(it+1) takes over at the step's
    // end.
    auto step_body = [&](int s_next, auto masked_c) {   // B for step s_next of its query head
      {
        constexpr int CA = 4;     // C operands read ahead
        const int va = b1 + a_off, vl = b1 + l_off;
        constexpr int QA = C::KS / 2;   // S operands read before the first product
        u32x4 qa[C::KS], da[C::KS], cop[NM];
#pragma unroll
        for (int ks = 0; ks < QA; ++ks) qa[ks] = lds16(smem, va + 32 * ks);
        // block it + 2's loads go out one instruction per product of S, in the
        // shadow of the matrix pipe
        const u32x4 dq_ = make_desc_u(pnext.qh, pnext.nbytes), ddo = make_desc_u(pnext.dO, pnext.nbytes);
        const u32x4 dst = make_desc(pnext.st, pnext.nst);
        constexpr bool MASKED = decltype(masked_c)::value;
        const int tq = (qb0 + s_next) * C::BMQ + 4 * g - kj;
        f32x4 l4s[4], d4s[4];
        __builtin_amdgcn_sched_barrier(0);
        s_acc = f32x16{};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          s_acc = mfma32(qa[ks], kf[ks], s_acc);
          // the remaining operand reads of A(it+1) and B's lse2, in the
          // products' shadow: each lands a few products before its use
          if (ks + QA < C::KS) qa[ks + QA] = lds16(smem, va + 32 * (ks + QA));
          da[ks] = lds16(smem, va + C::DO_B + 32 * ks);
          if (ks >= C::KS - 4) l4s[ks - (C::KS - 4)] = lds16f(smem, vl + 32 * (ks - (C::KS - 4)));
          if (ks < NDMA) issue_plan_one(dq_, ddo, dst, pnext, b2, ks);
          __builtin_amdgcn_sched_barrier(0);
        }
        // B(it+1) element r (register r of S and dP: query q0 + 8 (r / 4) + 4 g
        // + r % 4, key kj), as stage_b4 computes it, in two halves: P (the
        // exponential and the mask) needs only S and runs beside dP's products,
        // NPA elements there and the rest beside C's first; dS = P (dP - Delta)
        // and the bf16 packing run beside C(it)'s products.  Each value is pinned
        // where it is made.
        float pe[16], de[16];
        auto p_elem = [&](int r) {
          const int q4 = r >> 2, i = r & 3;
          float pr = __builtin_amdgcn_exp2f(s_acc[r] * ksc - l4s[q4][i]);
          if (MASKED) pr = ((unsigned)(tq + 8 * q4 + i) <= (unsigned)lim) ? pr : 0.f;
          pe[r] = pr;
          asm volatile("" : "+v"(pe[r]));
        };
        constexpr int NPA = 12;
        dp_acc = f32x16{};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          dp_acc = mfma32(da[ks], vf[ks], dp_acc);
          if (ks < CA) cop[ks] = c_read(b0, ks);     // C(it)'s first operands
          if (ks + C::KS < NDMA) issue_plan_one(dq_, ddo, dst, pnext, b2, ks + C::KS);
          if (ks == 0) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) d4s[q4] = lds16f(smem, vl + 256 + 32 * q4);
          }
#pragma unroll
          for (int r = NPA * ks / C::KS; r < NPA * (ks + 1) / C::KS; ++r) p_elem(r);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 2 * C::KS; j < NDMA; ++j) issue_plan_one(dq_, ddo, dst, pnext, b2, j);
        constexpr int EPM = 16 / NM;   // dS elements per product of C
        u32x4 pn[2], dn[2];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          if (m + CA < NM) cop[m + CA] = c_read(b0, m + CA);
          c_mfma(m, cop[m]);
          if (NPA + m < 16) p_elem(NPA + m);
#pragma unroll
          for (int k = 0; k < EPM; ++k) {
            const int r = EPM * m + k, q4 = r >> 2, i = r & 3;
            de[r] = pe[r] * (dp_acc[r] - d4s[q4][i]);
            asm volatile("" : "+v"(de[r]));
            if (r & 1) {
              const int st = q4 >> 1, el = 2 * (q4 & 1) + (i >> 1);
              pn[st][el] = pack_bf16(pe[r - 1], pe[r]);
              dn[st][el] = pack_bf16(de[r - 1], de[r]);
              asm volatile("" : "+v"(pn[st][el]), "+v"(dn[st][el]));
            }
          }
          if (m == NM / 2) pnext = plan_next();   // scalar work beside the products
          __builtin_amdgcn_sched_barrier(0);
        }
        pf[0] = pn[0];
        pf[1] = pn[1];
        dsf[0] = dn[0];
        dsf[1] = dn[1];
      }
      // the buffer rotation is scalar work that overlaps the last MFMAs still in
      // flight; the barrier only orders the buffers' contents
      const int t_ = b0;
      b0 = b1;
      b1 = b2;
      b2 = t_;
      wait_vmcnt<0>();            // block it + 2 has landed
      __syncthreads();
    };

    // Steps whose B needs the element mask sit at both ends of the band; the
    // middle runs the unmasked body.  `full_lo .. full_hi` are the steps
    // visible in full to every key of the tile: q0 >= j0 + BNK - 1 and
    // q0 + BMQ - 1 <= j0 + W, q0 + BMQ <= T.
    const int kv_last = imin(j0 + C::BNK - 1, T - 1);
    int full_lo = 0, full_hi = -1;
    if (nsteps > 0) {
      const int qf0 = kv_last;                                  // first fully causal query
      const int qf1 = imin(j0 + W, T) - (C::BMQ - 1);           // last start of a fully inside step
      full_lo = imax(0, (qf0 + C::BMQ - 1) / C::BMQ - qb0);
      full_hi = qf1 >= 0 ? qf1 / C::BMQ - qb0 : -1;
      full_hi = imin(full_hi, nsteps - 1);
    }
    // The tile runs G nsteps steps: step it + 1 = gi nsteps + s is step s of
    // query head gi.  Body `it` prepares B(it + 1), unmasked iff step s is full.
    const int nloop = G * nsteps - 1;   // steps with a successor
    int it = 0;
    if (nloop > 0) {   // step 1 of head 0, or step 0 of head 1
      step_body(nsteps > 1 ? 1 : 0, masked);
      it = 1;
    }
    if (kv_pending) {   // after a barrier that follows every wave's K / V reads
      if (nloop == 0) __syncthreads();
      issue_kv(geo(tile_at(ti + 1)));
    }
    for (int gi = 0; gi < G; ++gi) {
      const int base = gi * nsteps;                         // it + 1 = base + s
      const int it_end = imin(base + nsteps - 1, nloop);
      for (; it < imin(base + full_lo - 1, it_end); ++it) step_body(it + 1 - base, masked);
      for (; it < imin(base + full_hi, it_end); ++it) step_body(it + 1 - base, unmasked);
      for (; it < it_end; ++it) step_body(it + 1 - base, masked);
    }
    // rotary tables of key kj for the epilogue: channels 32 n + 8 q4 + 4 g + e
    // (n < NB / 2) pair with n + NB / 2; loaded during the last products
    u32x2 tc[C::NB / 2][4], tsn[C::NB / 2][4];
    if constexpr (ROPE) {
      const long long tb = (long long)(T - kw0) * D;
      const rsrc_t rc = make_rsrc(rcos + (size_t)kw0 * (D / 2), tb);
      const rsrc_t rn = make_rsrc(rsin + (size_t)kw0 * (D / 2), tb);
#pragma unroll
      for (int n = 0; n < C::NB / 2; ++n)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int off = (c * (D / 2) + 32 * n + 8 * q4 + 4 * g) * 2;
          tc[n][q4] = bload8(rc, off);
          tsn[n][q4] = bload8(rn, off);
        }
    }
    // value embedding and gate of key kj (channels as above, all n)
    const bool has_ve = ve != nullptr;
    u32x2 vef[C::NB][4];
    float gk = 0.f;
    if (has_ve) {
      const rsrc_t rve = make_rsrc(ve + sbase + (size_t)kw0 * rs_kv, kslice_bytes - kw0 * rsb_kv);
#pragma unroll
      for (int n = 0; n < C::NB; ++n)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) vef[n][q4] = bload8(rve, (c * rs_kv + 32 * n + 8 * q4 + 4 * g) * 2);
      gk = bload4f(make_rsrc(gate + (size_t)bh * T, 4LL * T), kj * 4);
    }
    issue_plan(pnext, b2);          // the next tile's block 1 (or later) into the free buffer
    pnext = plan_next();
    stage_c(b0);

    // ---- epilogue: lane (g, c) holds key kj, d = 32 n + 8 q4 + 4 g + e.
    // K of the key in that order comes from kf (d = 16 ks + 8 g + j): the
    // lane's own kf holds the quads with (q4 & 1) == g, its partner lane c + 32
    // (or c - 32) the others.
    const float rk = ksc * (sqrtf((float)D) / kLog2e);
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    float dot = 0.f;
    f32x16 khat[C::NB];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      // words (2 g + {0, 1}) of kf[ks]: elements 4 g .. 4 g + 3 of this lane's half
      const uint32_t send0 = g ? kf[ks][0] : kf[ks][2], send1 = g ? kf[ks][1] : kf[ks][3];
      const uint32_t got0 = __shfl_xor(send0, 32), got1 = __shfl_xor(send1, 32);
      const uint32_t own0 = g ? kf[ks][2] : kf[ks][0], own1 = g ? kf[ks][3] : kf[ks][1];
      // k-step ks covers d = 16 ks .. 16 ks + 15 = n = ks / 2, q4 = 2 (ks % 2) + {0, 1}
      const int n = ks >> 1, qa = 2 * (ks & 1);
      // quad q4 = qa + g comes from this lane, q4 = qa + 1 - g from the partner
      const uint32_t mine[2] = {own0, own1}, other[2] = {got0, got1};
#pragma unroll
      for (int hq = 0; hq < 2; ++hq) {
        const uint32_t* src = (hq == g) ? mine : other;   // quad qa + hq
        const float x[4] = {bf_lo(src[0]), bf_hi(src[0]), bf_lo(src[1]), bf_hi(src[1])};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * (qa + hq) + e;
          khat[n][r] = x[e] * rk;
          acc_dk[n][r] *= inv_sqrt_d;
          dot += acc_dk[n][r] * khat[n][r];
        }
      }
    }
    dot += __shfl_xor(dot, 32);
    const float mean = dot * (1.0f / D);
    if constexpr (ROPE) {
      // dk of the rotated key, then back through the rotation of key kj
#pragma unroll
      for (int n = 0; n < C::NB; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_dk[n][r] = rk * (acc_dk[n][r] - khat[n][r] * mean);
#pragma unroll
      for (int n = 0; n < C::NB / 2; ++n)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          float g1[4], g2[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            g1[e] = acc_dk[n][4 * q4 + e];
            g2[e] = acc_dk[n + C::NB / 2][4 * q4 + e];
          }
          rope4_bwd(g1, g2, tc[n][q4], tsn[n][q4]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc_dk[n][4 * q4 + e] = g1[e];
            acc_dk[n + C::NB / 2][4 * q4 + e] = g2[e];
          }
        }
    }
    if (has_ve) {
      float dg = 0.f;   // dV . ve of key kj, this lane's half of the channels
#pragma unroll
      for (int n = 0; n < C::NB; ++n)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float x[4] = {bf_lo(vef[n][q4][0]), bf_hi(vef[n][q4][0]), bf_lo(vef[n][q4][1]),
                              bf_hi(vef[n][q4][1])};
#pragma unroll
          for (int e = 0; e < 4; ++e) dg += acc_dv[n][4 * q4 + e] * x[e];
        }
      dg += __shfl_xor(dg, 32);
      if (g == 0)
        bstore4f(dg * gk * (1.0f - 0.5f * gk),
                 make_rsrc(dz + (size_t)tg.b * T * Hkv, 4LL * T * Hkv), (kj * Hkv + tg.hk) * 4);
    }
    // outputs leave through LDS so that every store writes whole rows: the
    // lane's values (key c, d = 32 n + 8 q4 + 4 g + e) go to a row-major
    // 32 x D block, then each lane stores 16-byte chunks of 4 rows per
    // instruction.  Waves 0 and 1 use the buffer of the last step (free after
    // the barrier), waves 2 and 3 their own slots.
    __syncthreads();
    const int slot = w < 2 ? b0 + C::OUT_SLOT * w : C::XO_B + C::OUT_SLOT * (w - 2);
    const rsrc_t rdk = make_rsrc(dk + sbase + (size_t)kw0 * rs_kv, kslice_bytes - kw0 * rsb_kv);
    const rsrc_t rdv = make_rsrc(dv + sbase + (size_t)kw0 * rs_kv, kslice_bytes - kw0 * rsb_kv);
    const rsrc_t rdve = make_rsrc(dve + sbase + (size_t)kw0 * rs_kv, has_ve ? kslice_bytes - kw0 * rsb_kv : 0);
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
      if (pass == 2 && !has_ve) break;
#pragma unroll
      for (int n = 0; n < C::NB; ++n)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            y[e] = pass == 2   ? gk * acc_dv[n][4 * q4 + e]
                   : pass == 1 ? acc_dv[n][4 * q4 + e]
                   : ROPE      ? acc_dk[n][4 * q4 + e]
                               : rk * (acc_dk[n][4 * q4 + e] - khat[n][4 * q4 + e] * mean);
          st8(smem + slot + 2 * (c * C::OP + 32 * n + 8 * q4 + 4 * g),
              u32x2{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])});
        }
      const rsrc_t ro = pass == 0 ? rdk : pass == 1 ? rdv : rdve;
#pragma unroll
      for (int i = 0; i < 32 * D / 8 / 64; ++i) {
        const int idx = lane + 64 * i, r = idx / (D / 8), ch = idx % (D / 8);
        const u32x4 val = lds16(smem, slot + 2 * (r * C::OP + 8 * ch));
        __builtin_amdgcn_raw_buffer_store_b128(val, ro, (r * rs_kv + 8 * ch) * 2, 0, 0);
      }
    }
  }
  wait_vmcnt<0>();   // the stream's last (zero-filling) block loads land before the workgroup ends
}

// ------------------------------------------------------------ dK / dV, D = 256
// At D = 256 one wave of the kernel above would need 2 x 128 accumulation
// registers for the dV and dK blocks of its 32 keys plus 128 for their K and
// V rows: more than a wave's 512.  Here two waves share each 32-key block
// and split the work by role:
//   role 0 (waves 0, 2): S = Q_hat K^T, P = exp2(S kscale - lse log2 e),
//                        dV^T += dO^T P
//   role 1 (waves 1, 3): dP = dO V^T, dS = P (dP - Delta),
//                        dK_hat^T += Q_hat^T dS
// Each wave holds one accumulator (128 registers) and one operand row set
// (K for role 0, V for role 1: 64 registers), and issues per step the same
// 32 products as a wave of the kernel above.  A tile is 64 keys (two pairs
// of waves).  Role 0 hands P to role 1 through LDS in fp32, so dS is formed
// from the unrounded probabilities as in the kernel above: role 0 writes P of
// block it + 1 during step it, role 1 reads it after the step's barrier and
// forms dS of that block beside its next dP products, one step behind role 0
// (it keeps dP of two blocks: the one it forms dS from and the one its
// products build).  The query-block stream, the tile list and the epilogues
// are those of the kernel above; the K and V rows go straight to registers at
// each tile's start.
template <bool GROUPED, bool ROPE>
struct DkdvSplitCfg {
  static constexpr int D = 256;
  static constexpr int BNK = 64;        // keys per tile (32 per pair of waves)
  static constexpr int BMQ = 32;        // queries per step
  static constexpr int NBUF = 3;
  static constexpr int KS = D / 16;
  static constexpr int NB = D / 32;
  static constexpr int P = D + 24;      // q_hat / dO row pitch (bf16): odd multiple of 16 bytes
  using Tile = DmaTileV<BMQ * P / 8, 4, 12 + GROUPED + 2 * ROPE>;
  static constexpr int DO_B = Tile::BYTES;          // dO tile after the q_hat tile
  static constexpr int ST_B = 2 * Tile::BYTES;      // 4 x 256 B: spare, spare, lse2, Delta
  static constexpr int STAGE = ST_B + 1024;
  static constexpr int XP_B = NBUF * STAGE;         // P of each pair, two buffers: 16 fp32 per lane
  static constexpr int XP_SLOT = 64 * 64;
  static constexpr int OP = D + 8;                  // output staging row pitch (bf16)
  static constexpr int OUT_SLOT = 32 * OP * 2;      // one wave's 32 x D bf16 block
  static constexpr int XO_B = XP_B + 4 * XP_SLOT;   // staging slots of waves 2 and 3
  static constexpr int LDS_BYTES = XO_B + 2 * OUT_SLOT;
  static constexpr int NSTORE = 32 * D / 8 / 64;    // epilogue stores per lane of one output
  static_assert(2 * OUT_SLOT <= STAGE, "waves 0 and 1 stage their outputs in a freed step buffer");
  static_assert(LDS_BYTES <= 160 * 1024, "fits the LDS of one CU");
};

template <bool GROUPED, bool ROPE, bool MIRROR>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_split_kernel(
    const uint16_t* __restrict__ qhat, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse2, const float* __restrict__ delta,
    const float* __restrict__ kscale, const uint16_t* __restrict__ rcos,
    const uint16_t* __restrict__ rsin, const uint16_t* __restrict__ ve,
    const float* __restrict__ gate, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
    uint16_t* __restrict__ dve, float* __restrict__ dz, int T, int H, int G_arg, int W, int nkt,
    int ntiles, int mirror0) {
  using C = DkdvSplitCfg<GROUPED, ROPE>;
  constexpr int D = C::D;
  const int G = GROUPED ? G_arg : 1;
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x;
  const int w = uniform(tid >> 6);
  const int pair = w >> 1;
  const int lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int rs = H * D;                 // query-side row stride (q_hat, dO)
  const long long rsb = 2LL * rs;
  const long long slice_bytes = (long long)(T - 1) * rsb + 2 * D;
  const int Hkv = H / G;
  const int rs_kv = Hkv * D;            // key-side row stride (K, V, dK, dV)
  const long long rsb_kv = 2LL * rs_kv;
  const long long kslice_bytes = (long long)(T - 1) * rsb_kv + 2 * D;

  // Each role runs its own copy of the whole walk (the role is fixed per
  // wave), so the two roles' registers never meet; both copies pass the same
  // barriers in the same order.
  auto run = [&](auto role_c) __attribute__((always_inline)) {
  constexpr int role = decltype(role_c)::value ? 1 : 0;
    // ---- tile list of this workgroup (as in the kernel above)
    int xr = 0, ws = blockIdx.x, G8 = gridDim.x, N8 = ntiles;
    if ((ntiles & 7) == 0 && (gridDim.x & 7) == 0) {
      xr = blockIdx.x & 7;
      ws = blockIdx.x >> 3;
      G8 = gridDim.x >> 3;
      N8 = ntiles >> 3;
    }
    auto tile_at = [&](int i) {
      if constexpr (MIRROR) {
        const int r = schedule_tile(i, ws, G8, N8, mirror0);
        return r >= 0 ? xr * N8 + r : -1;
      } else {
        const int r = i * G8 + (ws + 7 * i) % G8;
        return (i * G8 < N8 && r < N8) ? xr * N8 + r : -1;
      }
    };
    struct TileGeo {
      int bh, b, hk, j0, qb0, nsteps;
    };
    auto geo = [&](int t) {
      TileGeo tg;
      tg.bh = t / nkt;
      tg.b = tg.bh / Hkv;
      tg.hk = tg.bh - tg.b * Hkv;
      tg.j0 = (t % nkt) * C::BNK;
      int q_lo, q_hi;
      const bool any = q_range(tg.j0, tg.j0 + C::BNK - 1, T, W, &q_lo, &q_hi);
      tg.qb0 = any ? q_lo / C::BMQ : 0;
      tg.nsteps = any ? q_hi / C::BMQ - tg.qb0 + 1 : 0;
      return tg;
    };
  
    // ---- the stream of query blocks across tiles and query heads (as above)
    typename C::Tile tile;
    tile.init(w, lane, [&](int qc) {
      const int r = qc / (C::P / 8), ch = qc % (C::P / 8);
      return (r < C::BMQ && ch < D / 8) ? (r * rs + 8 * ch) * 2 : -1;
    });
    struct DmaPlan {
      const uint16_t* qh;
      const uint16_t* dO;
      const float* st;
      uint32_t nbytes;
      int nst;
      int r0;
    };
    int dt = 0, ds = 0, dgi = 0;
    TileGeo dgeo;
    const uint16_t* cq = qhat;
    const uint16_t* cdo = dout;
    const float* cst = w == 2 ? lse2 : delta;
    uint32_t cbytes = 0;
    int cr0 = 0;
    auto seek_head = [&]() {
      const int hq = dgeo.hk * G + dgi;
      const size_t sbase = ((size_t)dgeo.b * T * H + hq) * D;
      cr0 = dgeo.qb0 * C::BMQ;
      cq = qhat + sbase + (size_t)cr0 * rs;
      cdo = dout + sbase + (size_t)cr0 * rs;
      cbytes = (uint32_t)(slice_bytes - cr0 * rsb);
      cst = (w == 2 ? lse2 : delta) + (size_t)(dgeo.b * H + hq) * T;
    };
    int tcur = tile_at(0);
    if (tcur >= 0) {
      dgeo = geo(tcur);
      seek_head();
    }
    auto plan_next = [&]() {
      while (tcur >= 0 && ds >= dgeo.nsteps) {
        ds = 0;
        if (++dgi >= G) {
          dgi = 0;
          ++dt;
          tcur = tile_at(dt);
          if (tcur >= 0) dgeo = geo(tcur);
        }
        if (tcur >= 0) seek_head();
      }
      DmaPlan pl;
      const bool ok = tcur >= 0;
      pl.qh = cq;
      pl.dO = cdo;
      pl.st = cst;
      pl.r0 = ok ? cr0 : 0;
      pl.nbytes = ok ? cbytes : 0u;
      pl.nst = (ok && w >= 2) ? 4 * T : 0;
      if (ok) {
        ++ds;
        cq += (size_t)C::BMQ * rs;
        cdo += (size_t)C::BMQ * rs;
        cbytes -= (uint32_t)(C::BMQ * rsb);
        cr0 += C::BMQ;
      }
      return pl;
    };
    auto issue_plan = [&](const DmaPlan& pl, int base) {
      tile.issue(make_desc_u(pl.qh, pl.nbytes), smem, base, w);
      tile.issue(make_desc_u(pl.dO, pl.nbytes), smem, base + C::DO_B, w);
      dma_row4(make_desc(pl.st, pl.nst), smem, base + C::ST_B + 256 * w, (pl.r0 + lane) * 4);
    };
    constexpr int NDMA = 2 * C::Tile::NIW + 1;
    auto issue_plan_one = [&](const u32x4& dq_, const u32x4& ddo, const u32x4& dst, const DmaPlan& pl, int base,
                              int j) {
      if (j < C::Tile::NIW) tile.issue_one(dq_, smem, base, w, j);
      else if (j < 2 * C::Tile::NIW) tile.issue_one(ddo, smem, base + C::DO_B, w, j - C::Tile::NIW);
      else dma_row4(dst, smem, base + C::ST_B + 256 * w, (pl.r0 + lane) * 4);
    };
  
    // per-lane byte offsets inside a stage buffer
    const int a_off = 2 * (c * C::P + 8 * g);          // row-major A operands (16-byte reads)
    const int t_off = 2 * tr_off(lane, C::P);          // transposed A operands
    const int l_off = C::ST_B + 512 + 16 * g;          // lse2 (+ 0) / Delta (+ 256) of the lane's query quads
    const int x_off = C::XP_B + 2 * C::XP_SLOT * pair + 16 * lane;   // P of the pair: + XP_SLOT * buffer + 1024 q4
  
    int b0 = 2 * C::STAGE, b1 = 0, b2 = C::STAGE;
    issue_plan(plan_next(), b1);
    issue_plan(plan_next(), b2);
    DmaPlan pnext = plan_next();
  
    u32x4 kv[C::KS];              // role 0: the tile's K rows of the pair's keys; role 1: V rows
    f32x16 acc[C::NB];            // role 0: dV^T blocks; role 1: dK_hat^T blocks
    f32x16 dpa, dpb;              // role 0: S in dpa; role 1: dP of block it in dpa, of block it + 1 in dpb
    u32x4 pf[2];                  // role 0: bf16 P of the block C works on
    const std::integral_constant<bool, true> masked{};
    const std::integral_constant<bool, false> unmasked{};
  
    for (int ti = 0;; ++ti) {
      const int t = tile_at(ti);
      if (t < 0) break;
      const TileGeo tg = geo(t);
      const int bh = tg.bh, j0 = tg.j0, qb0 = tg.qb0, nsteps = tg.nsteps;
      const size_t sbase = ((size_t)tg.b * T * Hkv + tg.hk) * D;
      const int kw0 = j0 + 32 * pair;
      const int kj = kw0 + c;
  
      // ---- tile prologue.  The pair's K (role 0) or V (role 1) rows and key
      // scale go straight from global memory to registers (C::KS + 1 loads),
      // issued ahead of the wait and barrier so that they are in flight while
      // the slower role finishes the previous tile's epilogue.  Blocks 0 and 1
      // have landed after the wait (they are older than the previous tile's
      // output stores and these loads, which may stay in flight).
      {
        const rsrc_t rkv = make_rsrc((role == 0 ? k : v) + sbase + (size_t)kw0 * rs_kv, kslice_bytes - kw0 * rsb_kv);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) kv[ks] = bload16(rkv, (c * rs_kv + 16 * ks + 8 * g) * 2);
      }
      const float ksc = bload4f(make_rsrc(kscale + (size_t)bh * T, 4LL * T), kj * 4);
      if (ti == 0) wait_vmcnt<0>();
      else wait_vmcnt<C::NSTORE + C::KS + 1>();
      __syncthreads();
      const int lim = imin(W, T - 1 - kj);
      {
        const int t_ = b0;
        b0 = b1;
        b1 = b2;
        b2 = t_;
      }
#pragma unroll
      for (int n = 0; n < C::NB; ++n) acc[n] = f32x16{};
  
      // C's transposed A operand of product m = NB s2 + n: dO^T (role 0) or
      // Q_hat^T (role 1) of the block in buffer `base`, rows 16 s2 .., column
      // block n (element j of k-step s2 is query 16 s2 + 4 g + (j % 4) + 8 (j / 4))
      constexpr int NC = 2 * C::NB;
      auto c_read = [&](int base, int m) {
        constexpr int R8 = 2 * 8 * C::P;
        const int s2 = m / C::NB, n = m % C::NB;
        const int off = base + t_off + (role == 0 ? C::DO_B : 0) + 2 * (16 * s2 * C::P + 32 * n);
        const u32x2 x0 = lds_tr4b(smem, off), x1 = lds_tr4b(smem, off + R8);
        return u32x4{x0[0], x0[1], x1[0], x1[1]};
      };
      // role 0: P of the block's register r (query q0 + 8 (r / 4) + 4 g + r % 4, key kj)
      auto p_value = [&](int r, f32x4 l4, int tq, bool msk) {
        float p = __builtin_amdgcn_exp2f(dpa[r] * ksc - l4[r & 3]);
        if (msk) p = ((unsigned)(tq + 8 * (r >> 2) + (r & 3)) <= (unsigned)lim) ? p : 0.f;
        return p;
      };
  
      // prologue products: role 0 S and P of block 0 (P to the exchange buffer
      // 0), role 1 dP of block 0
      if constexpr (role == 0) {
        const int va = b0 + a_off, vl = b0 + l_off;
        dpa = f32x16{};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) dpa = mfma32(lds16(smem, va + 32 * ks), kv[ks], dpa);
        const int tq = qb0 * C::BMQ + 4 * g - kj;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 l4 = lds16f(smem, vl + 32 * q4);
          float p[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) p[e] = p_value(4 * q4 + e, l4, tq, true);
          *reinterpret_cast<f32x4*>(smem + x_off + 1024 * q4) = f32x4{p[0], p[1], p[2], p[3]};
          const int st = q4 >> 1, el = 2 * (q4 & 1);
          pf[st][el] = pack_bf16(p[0], p[1]);
          pf[st][el + 1] = pack_bf16(p[2], p[3]);
        }
      } else {
        const int va = b0 + a_off + C::DO_B;
        dpa = f32x16{};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) dpa = mfma32(lds16(smem, va + 32 * ks), kv[ks], dpa);
      }
      __syncthreads();   // P of block 0 is visible to role 1
  
      // One step `it`: A(it+1), B, C(it) as in the kernel above, written out in
      // fenced regions.  Role 0: S(it+1)'s products with block it + 2's loads
      // between them, then C(it)'s dV products, each beside one element of
      // P(it+1) (written to the exchange buffer (it + 1) % 2 by quads).  Role 1:
      // dP(it+1)'s products with the loads, each beside one element of dS(it) =
      // P(it) (dP(it) - Delta(it)) (P(it) from the exchange buffer it % 2), then
      // C(it)'s dK products; dP(it + 1) then moves to dP(it)'s registers.  (A
      // body that alternated the two by the parity of it was two bodies in one
      // loop, and the compiler copied the accumulators between them.)
      auto step_body = [&](int it, int s_next, auto masked_c) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_c)::value;
        constexpr int KA = 2, CA = 2;
        const u32x4 dq_ = make_desc_u(pnext.qh, pnext.nbytes), ddo = make_desc_u(pnext.dO, pnext.nbytes);
        const u32x4 dst = make_desc(pnext.st, pnext.nst);
        u32x4 opa[C::KS], cop[NC];
        if constexpr (role == 0) {
          const int va = b1 + a_off, vl = b1 + l_off;
          f32x4 l4s[4];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) l4s[q4] = lds16f(smem, vl + 32 * q4);
#pragma unroll
          for (int ks = 0; ks < KA; ++ks) opa[ks] = lds16(smem, va + 32 * ks);
#pragma unroll
          for (int m = 0; m < CA; ++m) cop[m] = c_read(b0, m);
          __builtin_amdgcn_sched_barrier(0);
          dpa = f32x16{};
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks) {
            if (ks + KA < C::KS) opa[ks + KA] = lds16(smem, va + 32 * (ks + KA));
            dpa = mfma32(opa[ks], kv[ks], dpa);
            if (ks < NDMA) issue_plan_one(dq_, ddo, dst, pnext, b2, ks);
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int j = C::KS; j < NDMA; ++j) issue_plan_one(dq_, ddo, dst, pnext, b2, j);
          const int tq = (qb0 + s_next) * C::BMQ + 4 * g - kj;
          const int xw = x_off + C::XP_SLOT * ((it + 1) & 1);
          float pe[16];
          u32x4 pn[2];
#pragma unroll
          for (int m = 0; m < NC; ++m) {
            if (m + CA < NC) cop[m + CA] = c_read(b0, m + CA);
            acc[m % C::NB] = mfma32(cop[m], pf[m / C::NB], acc[m % C::NB]);
            const int r = m, q4 = r >> 2;
            pe[r] = p_value(r, l4s[q4], tq, MASKED);
            asm volatile("" : "+v"(pe[r]));
            if (r & 1) {
              const int st = q4 >> 1, el = 2 * (q4 & 1) + ((r & 3) >> 1);
              pn[st][el] = pack_bf16(pe[r - 1], pe[r]);
              asm volatile("" : "+v"(pn[st][el]));
            }
            if ((r & 3) == 3)
              *reinterpret_cast<f32x4*>(smem + xw + 1024 * q4) = f32x4{pe[r - 3], pe[r - 2], pe[r - 1], pe[r]};
            if (m == NC / 2) pnext = plan_next();
            __builtin_amdgcn_sched_barrier(0);
          }
          pf[0] = pn[0];
          pf[1] = pn[1];
        } else {
          f32x16& dp_cur = dpa;   // dP(it)
          f32x16& dp_nxt = dpb;   // dP(it + 1)
          const int va = b1 + a_off + C::DO_B, vd = b0 + l_off + 256;
          const int xr_ = x_off + C::XP_SLOT * (it & 1);
          f32x4 d4s[4], xp[4];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            xp[q4] = lds16f(smem, xr_ + 1024 * q4);
            d4s[q4] = lds16f(smem, vd + 32 * q4);
          }
#pragma unroll
          for (int ks = 0; ks < KA; ++ks) opa[ks] = lds16(smem, va + 32 * ks);
#pragma unroll
          for (int m = 0; m < CA; ++m) cop[m] = c_read(b0, m);
          __builtin_amdgcn_sched_barrier(0);
          dp_nxt = f32x16{};
          float de[16];
          u32x4 dn[2];
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks) {
            if (ks + KA < C::KS) opa[ks + KA] = lds16(smem, va + 32 * (ks + KA));
            dp_nxt = mfma32(opa[ks], kv[ks], dp_nxt);
            if (ks < NDMA) issue_plan_one(dq_, ddo, dst, pnext, b2, ks);
            const int r = ks, q4 = r >> 2, i = r & 3;
            de[r] = xp[q4][i] * (dp_cur[r] - d4s[q4][i]);
            asm volatile("" : "+v"(de[r]));
            if (r & 1) {
              const int st = q4 >> 1, el = 2 * (q4 & 1) + (i >> 1);
              dn[st][el] = pack_bf16(de[r - 1], de[r]);
              asm volatile("" : "+v"(dn[st][el]));
            }
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int j = C::KS; j < NDMA; ++j) issue_plan_one(dq_, ddo, dst, pnext, b2, j);
#pragma unroll
          for (int m = 0; m < NC; ++m) {
            if (m + CA < NC) cop[m + CA] = c_read(b0, m + CA);
            acc[m % C::NB] = mfma32(cop[m], dn[m / C::NB], acc[m % C::NB]);
            if (m == NC / 2) pnext = plan_next();
            __builtin_amdgcn_sched_barrier(0);
          }
          dp_cur = dp_nxt;
        }
        const int t_ = b0;
        b0 = b1;
        b1 = b2;
        b2 = t_;
        wait_vmcnt<0>();            // block it + 2 has landed
        __syncthreads();            // and P(it + 1) is visible to role 1
      };
      auto step = [&](int it, int s_next, auto masked_c) __attribute__((always_inline)) {
        step_body(it, s_next, masked_c);
      };
  
      // masked head, unmasked middle and masked tail of each query head's band
      // (as in the kernel above; body `it` prepares block it + 1)
      const int kv_last = imin(j0 + C::BNK - 1, T - 1);
      int full_lo = 0, full_hi = -1;
      if (nsteps > 0) {
        const int qf0 = kv_last;
        const int qf1 = imin(j0 + W, T) - (C::BMQ - 1);
        full_lo = imax(0, (qf0 + C::BMQ - 1) / C::BMQ - qb0);
        full_hi = qf1 >= 0 ? qf1 / C::BMQ - qb0 : -1;
        full_hi = imin(full_hi, nsteps - 1);
      }
      const int nloop = G * nsteps - 1;
      int it = 0;
      for (int gi = 0; gi < G; ++gi) {
        const int base = gi * nsteps;
        const int it_end = imin(base + nsteps - 1, nloop);
        for (; it < imin(base + full_lo - 1, it_end); ++it) step(it, it + 1 - base, masked);
        for (; it < imin(base + full_hi, it_end); ++it) step(it, it + 1 - base, unmasked);
        for (; it < it_end; ++it) step(it, it + 1 - base, masked);
      }
  
      // rotary tables of key kj for role 1's epilogue, in flight with the last
      // products
      u32x2 tc[C::NB / 2][4], tsn[C::NB / 2][4];
      if constexpr (ROPE && role == 1) {
        const long long tb = (long long)(T - kw0) * D;
        const rsrc_t rc = make_rsrc(rcos + (size_t)kw0 * (D / 2), tb);
        const rsrc_t rn = make_rsrc(rsin + (size_t)kw0 * (D / 2), tb);
#pragma unroll
        for (int n = 0; n < C::NB / 2; ++n)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int off = (c * (D / 2) + 32 * n + 8 * q4 + 4 * g) * 2;
            tc[n][q4] = bload8(rc, off);
            tsn[n][q4] = bload8(rn, off);
          }
      }
      const bool has_ve = ve != nullptr;
      issue_plan(pnext, b2);          // the next tile's block 1 (or later) into the free buffer
      pnext = plan_next();
      // the last block's C: role 0 with its P, role 1 with dS formed from the
      // P in exchange buffer nloop % 2
#pragma unroll
      for (int m = 0; m < NC; ++m) {
        if constexpr (role == 0) acc[m % C::NB] = mfma32(c_read(b0, m), pf[m / C::NB], acc[m % C::NB]);
      }
      if constexpr (role == 1) {
        const f32x16 dpl = dpa;
        const int xr_ = x_off + C::XP_SLOT * (nloop & 1), vd = b0 + l_off + 256;
        u32x4 dn[2];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 xp = lds16f(smem, xr_ + 1024 * q4), d4 = lds16f(smem, vd + 32 * q4);
          float de[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) de[e] = xp[e] * (dpl[4 * q4 + e] - d4[e]);
          const int st = q4 >> 1, el = 2 * (q4 & 1);
          dn[st][el] = pack_bf16(de[0], de[1]);
          dn[st][el + 1] = pack_bf16(de[2], de[3]);
        }
#pragma unroll
        for (int m = 0; m < NC; ++m) acc[m % C::NB] = mfma32(c_read(b0, m), dn[m / C::NB], acc[m % C::NB]);
      }
  
      // ---- epilogue.  Lane (g, c) holds key kj, d = 32 n + 8 q4 + 4 g + e.
      // Role 1: dK, the RMSNorm backward of K with the rotary embedding turned
      // back; K of the key is read again in that order (role 1 held V), in
      // pieces, twice (the second time from L2), so it never occupies 64
      // registers beside the accumulators.  Role 0: dV, and with the gate
      // dve = gate dV and dz = (dV . ve) gate (1 - gate / 2).  The outputs
      // leave through LDS as whole rows (waves 0 and 1 stage in the buffer of
      // the last step, free after the barrier; waves 2 and 3 in their own
      // slots).  Addresses are one per-lane base plus uniform or immediate
      // offsets.
      const float rk = ksc * (sqrtf((float)D) / kLog2e);
      const float inv_sqrt_d = 1.0f / sqrtf((float)D);
      const int lane_kv = (c * rs_kv + 4 * g) * 2;                 // + 2 (32 n + 8 q4): key kj's pieces
      const int slot = w < 2 ? b0 + C::OUT_SLOT * w : C::XO_B + C::OUT_SLOT * (w - 2);
      const int st_lane = slot + 2 * (c * C::OP + 4 * g);          // + 2 (32 n + 8 q4)
      const int rd_lane = slot + 2 * ((lane >> 5) * C::OP + 8 * (lane & 31));   // + 4 OP i
      const int gl_lane = ((lane >> 5) * rs_kv + 8 * (lane & 31)) * 2;         // + 4 rs_kv i (bytes)
      const rsrc_t rrow = make_rsrc(k + sbase + (size_t)kw0 * rs_kv, kslice_bytes - kw0 * rsb_kv);
      auto stage8 = [&](int n, int q4, const float* y) {
        st8(smem + st_lane + 2 * (32 * n + 8 * q4), u32x2{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])});
      };
      auto store_rows = [&](uint16_t* dst) {
        const rsrc_t ro = make_rsrc(dst + sbase + (size_t)kw0 * rs_kv, kslice_bytes - kw0 * rsb_kv);
#pragma unroll
        for (int i = 0; i < C::NSTORE; ++i)
          __builtin_amdgcn_raw_buffer_store_b128(lds16(smem, rd_lane + 4 * C::OP * i), ro, gl_lane,
                                                 4 * rs_kv * i, 0);
      };
      if constexpr (role == 1) {
        auto khat4 = [&](int n, int q4, float* x) {
          const u32x2 u = bload8(rrow, lane_kv + 2 * (32 * n + 8 * q4));
          x[0] = bf_lo(u[0]) * rk;
          x[1] = bf_hi(u[0]) * rk;
          x[2] = bf_lo(u[1]) * rk;
          x[3] = bf_hi(u[1]) * rk;
        };
        float dot = 0.f;
#pragma unroll
        for (int n = 0; n < C::NB; ++n)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            float x[4];
            khat4(n, q4, x);
#pragma unroll
            for (int e = 0; e < 4; ++e) dot += acc[n][4 * q4 + e] * x[e];
          }
        dot = (dot + __shfl_xor(dot, 32)) * inv_sqrt_d;
        const float mean = dot * (1.0f / D);
        __syncthreads();
#pragma unroll
        for (int n = 0; n < (ROPE ? C::NB / 2 : C::NB); ++n)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            float x1[4], y1[4];
            khat4(n, q4, x1);
#pragma unroll
            for (int e = 0; e < 4; ++e) y1[e] = rk * (acc[n][4 * q4 + e] * inv_sqrt_d - x1[e] * mean);
            if constexpr (ROPE) {
              float x2[4], y2[4];
              khat4(n + C::NB / 2, q4, x2);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                y2[e] = rk * (acc[n + C::NB / 2][4 * q4 + e] * inv_sqrt_d - x2[e] * mean);
              rope4_bwd(y1, y2, tc[n][q4], tsn[n][q4]);
              stage8(n + C::NB / 2, q4, y2);
            }
            stage8(n, q4, y1);
          }
        store_rows(dk);
      } else {
        float gk = 0.f;
        if (has_ve) {   // dz of key kj: dV . ve over the key's 256 channels
          const rsrc_t rve = make_rsrc(ve + sbase + (size_t)kw0 * rs_kv, kslice_bytes - kw0 * rsb_kv);
          gk = bload4f(make_rsrc(gate + (size_t)bh * T, 4LL * T), kj * 4);
          float dg = 0.f;
#pragma unroll
          for (int n = 0; n < C::NB; ++n)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const u32x2 u = bload8(rve, lane_kv + 2 * (32 * n + 8 * q4));
              const float x[4] = {bf_lo(u[0]), bf_hi(u[0]), bf_lo(u[1]), bf_hi(u[1])};
#pragma unroll
              for (int e = 0; e < 4; ++e) dg += acc[n][4 * q4 + e] * x[e];
            }
          dg += __shfl_xor(dg, 32);
          if (g == 0)
            bstore4f(dg * gk * (1.0f - 0.5f * gk),
                     make_rsrc(dz + (size_t)tg.b * T * Hkv, 4LL * T * Hkv), (kj * Hkv + tg.hk) * 4);
        }
        __syncthreads();
#pragma unroll
        for (int n = 0; n < C::NB; ++n)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const float y[4] = {acc[n][4 * q4], acc[n][4 * q4 + 1], acc[n][4 * q4 + 2], acc[n][4 * q4 + 3]};
            stage8(n, q4, y);
          }
        store_rows(dv);
        if (has_ve) {
#pragma unroll
          for (int n = 0; n < C::NB; ++n)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              float y[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) y[e] = gk * acc[n][4 * q4 + e];
              stage8(n, q4, y);
            }
          store_rows(dve);
        }
      }
    }
  };
  if (w & 1) run(std::integral_constant<bool, true>{});
  else run(std::integral_constant<bool, false>{});
  wait_vmcnt<0>();   // the stream's last (zero-filling) block loads land before the workgroup ends
}

// ------------------------------------------------------------ gate gradients
// The last step of the value-embedding gate's backward, from dz [B T, Hkv]:
//   dx[bt, c]   = sum_h dz[bt, h] W_g[h, c]            (c < 32, bf16 out)
//   dW_g[h, c]  = sum_bt dz[bt, h] x[bt, c]
// ve_gate_bwd_kernel: block i takes tokens 64 i .. 64 i + 63 as 8 groups of
// 32 lanes; lane c of group j handles channel c of tokens j, j + 8, .., with
// all 8 tokens' loads in flight.  The groups' sums of dW_g meet in LDS and the
// block writes one partial [Hkv, 32].  ve_gate_dw_kernel (one block per head)
// adds the partials in a fixed order, so dW_g is deterministic.
constexpr int kGateMaxH = 16;   // key/value heads the gate kernels support

__global__ __launch_bounds__(256) void ve_gate_bwd_kernel(const float* __restrict__ dz,
                                                          const uint16_t* __restrict__ xg, int xs,
                                                          const float* __restrict__ gate_w,
                                                          uint16_t* __restrict__ dxg,
                                                          float* __restrict__ part, int nbt, int Hkv) {
  __shared__ float red[8][kGateMaxH * 32];
  const int c = threadIdx.x & 31, grp = threadIdx.x >> 5;
  const int t0 = blockIdx.x * kGateTokens + grp;
  float xv[8], dx[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int bt = t0 + 8 * i;
    xv[i] = bt < nbt ? __uint_as_float((uint32_t)xg[(size_t)bt * xs + c] << 16) : 0.f;
    dx[i] = 0.f;
  }
  for (int h = 0; h < Hkv; ++h) {
    const float w = gate_w[h * 32 + c];
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int bt = t0 + 8 * i;
      const float d = bt < nbt ? dz[(size_t)bt * Hkv + h] : 0.f;
      dx[i] += d * w;
      acc += d * xv[i];
    }
    red[grp][h * 32 + c] = acc;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int bt = t0 + 8 * i;
    if (bt < nbt) dxg[(size_t)bt * 32 + c] = (uint16_t)(pack_bf16(dx[i], 0.f) & 0xffff);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < Hkv * 32; i += 256) {
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) sum += red[j][i];
    part[(size_t)blockIdx.x * Hkv * 32 + i] = sum;
  }
}

// block h: lane c of group j adds the partials j, j + 8, .. of channel c
__global__ __launch_bounds__(256) void ve_gate_dw_kernel(const float* __restrict__ part,
                                                         float* __restrict__ dw, int nblk, int Hkv) {
  __shared__ float red[8][32];
  const int c = threadIdx.x & 31, grp = threadIdx.x >> 5, h = blockIdx.x;
  float sum[4] = {0.f, 0.f, 0.f, 0.f};
  int b = grp;
  for (; b + 24 < nblk; b += 32)
#pragma unroll
    for (int u = 0; u < 4; ++u) sum[u] += part[((size_t)(b + 8 * u) * Hkv + h) * 32 + c];
  for (; b < nblk; b += 8) sum[0] += part[((size_t)b * Hkv + h) * 32 + c];
  red[grp][c] = (sum[0] + sum[1]) + (sum[2] + sum[3]);
  __syncthreads();
  if (grp == 0) {
    float t = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) t += red[j][c];
    dw[h * 32 + c] = t;
  }
}

template <int D, bool GROUPED, bool ROPE, bool MIRROR>
static hipError_t set_dkdv_lds() {
  using C = DkdvCfg<D, GROUPED, ROPE>;
  // more than 64 KiB of dynamic LDS must be opted into, once per kernel
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(bwd_dkdv_kernel<D, GROUPED, ROPE, MIRROR>),
      hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  return attr;
}

template <bool GROUPED, bool ROPE, bool MIRROR>
static hipError_t set_dkdv_split_lds() {
  using C = DkdvSplitCfg<GROUPED, ROPE>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(bwd_dkdv_split_kernel<GROUPED, ROPE, MIRROR>),
      hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  return attr;
}

// The persistent dK/dV launch's schedule, as its kernels derive it: the
// tiles split into 8 XCD ranges when both counts allow; the first mirrored
// round (persistent_tile in band.h), and whether any round is mirrored.
static int dkdv_mirror_from(int ntiles, int grid, int nkt, bool* mirror) {
  const bool split = (ntiles & 7) == 0 && (grid & 7) == 0;
  const int g8 = split ? grid / 8 : grid, n8 = split ? ntiles / 8 : ntiles;
  const int m0 = mirror_from(g8, n8, nkt);
  *mirror = m0 < (n8 + g8 - 1) / g8;
  return m0;
}

template <int D, bool ROPE>
static hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t stream) {
  const int G = a.H / a.Hkv;
  // with the rotary embedding, the backward kernels read the rotated keys;
  // with the value-embedding gate, the gated values
  const uint16_t* kk = (const uint16_t*)(ROPE ? a.kr : a.k);
  const uint16_t* vv = (const uint16_t*)(a.ve ? a.vr : a.v);
  KeyPrepArgs kp;
  kp.k = a.k; kp.v = a.v; kp.rcos = a.rcos; kp.rsin = a.rsin; kp.ve = a.ve; kp.xg = a.xg; kp.xs = a.xs;
  kp.gate_w = a.gate_w; kp.kscale = a.kscale; kp.kr = a.kr; kp.vr = a.vr; kp.gate = a.gate;
  kp.B = a.B; kp.T = a.T; kp.Hkv = a.Hkv; kp.D = D; kp.eps = a.eps;
  if (!a.keys_ready) {
    const hipError_t ep = launch_key_prep(kp, K_BWD_KSCALE, stream);
    if (ep != hipSuccess) return ep;
  }
  const int W = eff_window(a.T, a.window);
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1)
    return hipErrorInvalidDevice;
  {
    // dQ first (attn_bwd_dq.hip): it also writes q_hat, Delta and lse log2(e)
    // for dK/dV
    const hipError_t eq = launch_bwd_dq(a, kk, vv, W, ncu, stream);
    if (eq != hipSuccess) return eq;
  }
  {
    if constexpr (D <= 128) {
      using C = DkdvCfg<D, false, ROPE>;
      static_assert(C::LDS_BYTES == DkdvCfg<D, true, ROPE>::LDS_BYTES, "one LDS size for both versions");
      const int nkt = (a.T + C::BNK - 1) / C::BNK;
      const int ntiles = nkt * a.B * a.Hkv;
      const int grid = imin(D <= 64 ? 2 * ncu : ncu, ntiles);   // persistent: workgroups per CU as fit
      bool mirror = false;
      const int mirror0 = dkdv_mirror_from(ntiles, grid, nkt, &mirror);
      auto go = [&](auto grouped_c, auto mirror_c) -> hipError_t {
        constexpr bool GR = decltype(grouped_c)::value, MI = decltype(mirror_c)::value;
        const hipError_t attr = set_dkdv_lds<D, GR, ROPE, MI>();
        if (attr != hipSuccess) return attr;
        ProfToken t1 = prof_begin(K_BWD_DKDV, stream);
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, GR, ROPE, MI>), dim3(grid), dim3(256), C::LDS_BYTES, stream,
                           (const uint16_t*)a.qhat, kk, vv, (const uint16_t*)a.dout,
                           (const float*)a.lse2, (const float*)a.delta, (const float*)a.kscale,
                           (const uint16_t*)a.rcos, (const uint16_t*)a.rsin, (const uint16_t*)a.ve,
                           (const float*)a.gate, (uint16_t*)a.dk, (uint16_t*)a.dv, (uint16_t*)a.dve, a.dz,
                           a.T, a.H, G, W, nkt, ntiles, mirror0);
        prof_end(t1);
        return hipSuccess;
      };
      using T_ = std::true_type;
      using F_ = std::false_type;
      const hipError_t e = G == 1 ? (mirror ? go(F_{}, T_{}) : go(F_{}, F_{}))
                                  : (mirror ? go(T_{}, T_{}) : go(T_{}, F_{}));
      if (e != hipSuccess) return e;
    } else {
      using C = DkdvSplitCfg<false, ROPE>;
      static_assert(C::LDS_BYTES == DkdvSplitCfg<true, ROPE>::LDS_BYTES, "one LDS size for both versions");
      const int nkt = (a.T + C::BNK - 1) / C::BNK;
      const int ntiles = nkt * a.B * a.Hkv;
      const int grid = imin(ncu, ntiles);   // persistent: one workgroup per CU
      bool mirror = false;
      const int mirror0 = dkdv_mirror_from(ntiles, grid, nkt, &mirror);
      auto go = [&](auto grouped_c, auto mirror_c) -> hipError_t {
        constexpr bool GR = decltype(grouped_c)::value, MI = decltype(mirror_c)::value;
        const hipError_t attr = set_dkdv_split_lds<GR, ROPE, MI>();
        if (attr != hipSuccess) return attr;
        ProfToken t1 = prof_begin(K_BWD_DKDV, stream);
        hipLaunchKernelGGL((bwd_dkdv_split_kernel<GR, ROPE, MI>), dim3(grid), dim3(256), C::LDS_BYTES, stream,
                           (const uint16_t*)a.qhat, kk, vv, (const uint16_t*)a.dout,
                           (const float*)a.lse2, (const float*)a.delta, (const float*)a.kscale,
                           (const uint16_t*)a.rcos, (const uint16_t*)a.rsin, (const uint16_t*)a.ve,
                           (const float*)a.gate, (uint16_t*)a.dk, (uint16_t*)a.dv, (uint16_t*)a.dve, a.dz,
                           a.T, a.H, G, W, nkt, ntiles, mirror0);
        prof_end(t1);
        return hipSuccess;
      };
      using T_ = std::true_type;
      using F_ = std::false_type;
      const hipError_t e = G == 1 ? (mirror ? go(F_{}, T_{}) : go(F_{}, F_{}))
                                  : (mirror ? go(T_{}, T_{}) : go(T_{}, F_{}));
      if (e != hipSuccess) return e;
    }
  }
  if (a.ve) {
    const int nbt = a.B * a.T;
    const int nblk = (nbt + kGateTokens - 1) / kGateTokens;
    ProfToken t3 = prof_begin(K_BWD_GATE, stream);
    hipLaunchKernelGGL(ve_gate_bwd_kernel, dim3(nblk), dim3(256), 0, stream, (const float*)a.dz,
                       (const uint16_t*)a.xg, a.xs, a.gate_w, (uint16_t*)a.dxg, a.dw_part, nbt, a.Hkv);
    hipLaunchKernelGGL(ve_gate_dw_kernel, dim3(a.Hkv), dim3(256), 0, stream, (const float*)a.dw_part,
                       a.dgate_w, nblk, a.Hkv);
    prof_end(t3);
  }
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  const bool rope = a.rcos != nullptr;
  if (a.D == 256) return rope ? launch_bwd_d<256, true>(a, stream) : launch_bwd_d<256, false>(a, stream);
  if (a.D == 128) return rope ? launch_bwd_d<128, true>(a, stream) : launch_bwd_d<128, false>(a, stream);
  return rope ? launch_bwd_d<64, true>(a, stream) : launch_bwd_d<64, false>(a, stream);
}

}  // namespace swattn
