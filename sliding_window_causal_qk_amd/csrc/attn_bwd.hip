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
//   bwd_dq:     a workgroup owns 128 queries (32 per wave): it normalises its
//               queries, computes Delta = dO . o and writes q_hat, Delta and
//               lse log2(e) for bwd_dkdv, then walks the key tiles of its band,
//               recomputing S and dP; the RMSNorm backward of Q runs in the
//               epilogue.  No atomics: dQ is deterministic.
//   bwd_dkdv:   persistent; a tile is 128 keys (32 per wave) of one key/value
//               head, walking the query blocks of its band in each of the
//               head's G query heads; dV^T and dK_hat^T stay in registers; the
//               RMSNorm backward of K runs in the epilogue.
#include <type_traits>

#include "common.h"
#include "band.h"
#include "kernels.h"
#include "profile.h"

namespace swattn {

// A-operand of a 32x32x16 MFMA whose k index runs along the rows of a row-major
// LDS tile (two transposing reads): lane (g, c) gets column col0 + c of rows
// row0 + 4 g + {0,1,2,3} and row0 + 8 + 4 g + {0,1,2,3}, i.e. element j is row
// row0 + 4 g + (j % 4) + 8 (j / 4) -- the k order of probabilities held in the
// C layout of a previous product.  `off` is the per-lane part from tr_off().
__device__ __forceinline__ int tr_off(int lane, int P) {
  const int li = lane & 15, g = lane >> 5;
  return (4 * g + (li >> 2)) * P + 16 * ((lane >> 4) & 1) + 4 * (li & 3);
}

// ------------------------------------------------------------------ dK / dV
// Persistent: one workgroup per CU walks a list of key tiles of 128 keys.  In
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
// range, round i gives workgroup s the tile i G8 + (s + 7 i) mod G8, which
// rotates the light tiles of the causal tail through all workgroups.
template <int D, bool GROUPED, bool ROPE>
struct DkdvCfg {
  static constexpr int BNK = 128;       // keys per tile (32 per wave)
  static constexpr int BMQ = 32;        // queries per step
  static constexpr int NBUF = 3;
  static constexpr int KS = D / 16;
  static constexpr int NB = D / 32;
  static constexpr int P = D + 24;      // q_hat / dO row pitch (bf16): odd multiple of 16 bytes
  static constexpr int PK = D + 8;      // K / V row pitch in the prefetch region
  using Tile = DmaTileV<BMQ * P / 8, 4, 1 + GROUPED + 2 * ROPE>;
  using KVTile = DmaTileV<BNK * PK / 8, 4, 1 + GROUPED + 2 * ROPE>;
  static constexpr int DO_B = Tile::BYTES;          // dO tile after the q_hat tile
  static constexpr int ST_B = 2 * Tile::BYTES;      // 4 x 256 B: spare, spare, lse2, Delta
  static constexpr int STAGE = ST_B + 1024;
  static constexpr int KV_B = NBUF * STAGE;         // K rows, then V rows of the next tile
  // the next tile's K / V rows are prefetched into LDS up to D = 128; at
  // D = 256 they would not fit, and each tile loads them into registers
  static constexpr bool KV_PREFETCH = D <= 128;
  static constexpr int OP = D + 8;                  // output staging row pitch (bf16)
  static constexpr int OUT_SLOT = 32 * OP * 2;      // one wave's 32 x D bf16 block
  static constexpr int XO_B = KV_B + (KV_PREFETCH ? 2 * KVTile::BYTES : 0);   // staging slots of waves 2 and 3
  static constexpr int LDS_BYTES = XO_B + 2 * OUT_SLOT;
  static constexpr int NSTORE = 2 * (32 * D / 8 / 64);    // epilogue stores per lane (dK and dV)
  static_assert(2 * OUT_SLOT <= STAGE, "waves 0 and 1 stage their outputs in a freed step buffer");
  static_assert(LDS_BYTES <= 160 * 1024, "fits the LDS of one CU");
};

// GROUPED = false is the plain multi-head case, compiled with G = 1 so that the
// walk over the query heads of a group folds away.  ROPE: k holds the rotated
// keys, and dK goes back through the transposed rotation in the epilogue.
// With the value-embedding gate (ve not null), v holds v + gate ve and the
// epilogue also writes dve = gate dV and dz = (dV . ve) gate (1 - gate / 2),
// the gradient of the gate's pre-sigmoid input ([B, T, Hkv]).
template <int D, bool GROUPED, bool ROPE>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ qhat, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse2, const float* __restrict__ delta,
    const float* __restrict__ kscale, const uint16_t* __restrict__ rcos,
    const uint16_t* __restrict__ rsin, const uint16_t* __restrict__ ve,
    const float* __restrict__ gate, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
    uint16_t* __restrict__ dve, float* __restrict__ dz, int T, int H, int G_arg, int W, int nkt,
    int ntiles) {
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
  auto tile_at = [&](int i) {   // i-th tile of this workgroup, or -1
    const int r = i * G8 + (ws + 7 * i) % G8;
    return (i * G8 < N8 && r < N8) ? xr * N8 + r : -1;
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
  if (C::KV_PREFETCH && tcur >= 0) issue_kv(dgeo);
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

    // ---- tile prologue: steps 0 and 1 of this tile and its K / V rows have
    // landed (they are older than the previous tile's dK / dV stores, which
    // may stay in flight); the buffer of the previous tile's last step takes
    // step 2
    if (ti == 0) wait_vmcnt<0>();
    else wait_vmcnt<C::NSTORE>();
    __syncthreads();
    const float ksc = bload4f(make_rsrc(kscale + (size_t)bh * T, 4LL * T), kj * 4);
    // visibility on partial blocks: 0 <= q - kj <= lim, lim = min(W, T - 1 - kj)
    const int lim = imin(W, T - 1 - kj);
    {
      const int t_ = b0;
      b0 = b1;
      b1 = b2;
      b2 = t_;
    }
    if constexpr (C::KV_PREFETCH) {
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        kf[ks] = lds16(smem, kv_off + 32 * ks);
        vf[ks] = lds16(smem, kv_off + C::KVTile::BYTES + 32 * ks);
      }
    } else {
      const rsrc_t rk = make_rsrc(k + sbase + (size_t)kw0 * rs_kv, kslice_bytes - kw0 * rsb_kv);
      const rsrc_t rv = make_rsrc(v + sbase + (size_t)kw0 * rs_kv, kslice_bytes - kw0 * rsb_kv);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        kf[ks] = bload16(rk, (c * rs_kv + 16 * ks + 8 * g) * 2);
        vf[ks] = bload16(rv, (c * rs_kv + 16 * ks + 8 * g) * 2);
      }
    }
#pragma unroll
    for (int n = 0; n < C::NB; ++n) { acc_dv[n] = f32x16{}; acc_dk[n] = f32x16{}; }
    const bool kv_pending = C::KV_PREFETCH && tile_at(ti + 1) >= 0;   // prefetch of the next tile's K / V rows

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
    // buffers.  One wave per SIMD issues in order, so a VALU, scalar or memory
    // instruction costs nothing only in the shadow of a product it does not
    // depend on.  Left to itself the compiler issued each LDS read right before
    // its product and waited for it there, and sank the softmax next to C's
    // products alone; the order is therefore written out in regions fenced with
    // scheduling barriers:
    //   every read of A(it+1), C(it)'s first CA and B's lse2;
    //   S's products, with block it + 2's loads between them (one each);
    //   dP's products, with NPA of B(it+1)'s exponentials between them (P needs
    //   only S) and B's Delta read;
    //   C(it)'s products, each after the reads of the product CA places later,
    //   with the remaining exponentials, dS = P (dP - Delta) and the bf16
    //   packing between them, and the next block's plan halfway.
    // B(it+1) writes separate registers that C(it+1) takes over at the step's
    // end.  At D = 256 the operands of that order do not fit in registers and
    // the step keeps the compiler's order.
    auto step_body = [&](int s_next, auto masked_c) {   // B for step s_next of its query head
      if constexpr (D <= 128) {
        constexpr int CA = 4;     // C operands read ahead
        const int va = b1 + a_off, vl = b1 + l_off;
        u32x4 qa[C::KS], da[C::KS], cop[NM];
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          qa[ks] = lds16(smem, va + 32 * ks);
          da[ks] = lds16(smem, va + C::DO_B + 32 * ks);
        }
#pragma unroll
        for (int m = 0; m < CA; ++m) cop[m] = c_read(b0, m);
        // block it + 2's loads go out one instruction per product of S, in the
        // shadow of the matrix pipe
        const u32x4 dq_ = make_desc_u(pnext.qh, pnext.nbytes), ddo = make_desc_u(pnext.dO, pnext.nbytes);
        const u32x4 dst = make_desc(pnext.st, pnext.nst);
        constexpr bool MASKED = decltype(masked_c)::value;
        const int tq = (qb0 + s_next) * C::BMQ + 4 * g - kj;
        f32x4 l4s[4], d4s[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) l4s[q4] = lds16f(smem, vl + 32 * q4);
        __builtin_amdgcn_sched_barrier(0);
        s_acc = f32x16{};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          s_acc = mfma32(qa[ks], kf[ks], s_acc);
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
      } else {
        issue_plan(pnext, b2);      // block it + 2 into the free buffer
        stage_a(b1);
        __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
#pragma unroll
        for (int i = 0; i < 2 * C::KS - 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        __builtin_amdgcn_sched_barrier(0);   // A stays ahead of C and B
        stage_c(b0);
        stage_b(b1, s_next, masked_c);
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int i = 0; i < 4 * C::NB - 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // DS reads
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // VALU
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        }
        // keep B's results inside this step (the compiler would otherwise sink
        // the softmax below the barrier, away from the MFMAs it should overlap)
        asm volatile("" ::"v"(pf[0]), "v"(pf[1]), "v"(dsf[0]), "v"(dsf[1]));
      }
      // the buffer rotation is scalar work that overlaps the last MFMAs still in
      // flight; the barrier only orders the buffers' contents
      if constexpr (D > 128) pnext = plan_next();
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

// ------------------------------------------------------------------ dQ
// Workgroup: 4 waves; wave w owns queries i0 + 32 w + c.  Key blocks of 32
// rows (K, V and their kscale) stream through the band in three LDS buffers
// filled by direct-to-LDS loads one step ahead.  Per block i:
//   A(i): S^T = K Q_hat^T and dP^T = V dO^T   (queries in lanes, keys in registers)
//   B(i): dS' = exp2(S^T kscale - lse log2 e) (dP^T - Delta) kscale      (VALU)
//   C(i): dQ^T += K^T dS'^T   (K^T read transposed from the row-major K tile)
// As in the dK/dV kernel the loop issues A(i+1), C(i), then B(i+1).  The
// kernel fits two waves per SIMD, so the hardware also overlaps two
// workgroups' phases.
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
__global__ __launch_bounds__(256, D >= 256 ? 1 : 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ o,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ kscale, const uint16_t* __restrict__ rcos,
    const uint16_t* __restrict__ rsin, uint16_t* __restrict__ qhat, float* __restrict__ delta,
    float* __restrict__ lse2, uint16_t* __restrict__ dq, int T, int H, int G, int W, float eps) {
  using C = DqCfg<D, ROPE>;
  extern __shared__ __align__(16) unsigned char smem[];

  const int nqt = (T + C::BM - 1) / C::BM;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  int bh, qt;
  query_tile_of(lid, nqt, gridDim.x / nqt, kTileGroupDq, &bh, &qt);
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
  float r_q, dlt;
  {
    const rsrc_t rqr = make_rsrc(q + sbase + (size_t)qw0 * rs, slice_bytes - qw0 * rsb);
    const rsrc_t rdo = make_rsrc(dout + sbase + (size_t)qw0 * rs, slice_bytes - qw0 * rsb);
    const rsrc_t ror = make_rsrc(o + sbase + (size_t)qw0 * rs, slice_bytes - qw0 * rsb);
    float dd = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      qf[ks] = bload16(rqr, (c * rs + 16 * ks + 8 * g) * 2);
      df[ks] = bload16(rdo, (c * rs + 16 * ks + 8 * g) * 2);
      const u32x4 of = bload16(ror, (c * rs + 16 * ks + 8 * g) * 2);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dd += bf_lo(df[ks][e]) * bf_lo(of[e]) + bf_hi(df[ks][e]) * bf_hi(of[e]);
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
  const float lq = bload4f(make_rsrc(lse + sb, 4LL * T), qi * 4) * kLog2e;
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

  // ---- direct-to-LDS staging of one key step
  typename C::Tile tile;
  tile.init(w, lane, rs_kv);
  const u32x4 rks = make_desc(kscale + (size_t)(b * Hkv + h / G) * T, w == 0 ? 4LL * T : 0);   // wave 0 loads kscale
  const uint16_t* k_s = k + kvbase;
  const uint16_t* v_s = v + kvbase;
  // remaining bytes of the key slices from row r0 on, below 2^32 (unsigned arithmetic)
  const uint32_t kbytes_u = (uint32_t)kslice_bytes, krow_u = (uint32_t)rsb_kv;
  auto issue_step = [&](int step, int base) {
    const int r0 = (jb0 + step) * C::BN;
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
    const int t0 = (jb0 + step) * C::BN + 4 * g + W - qi;  // kv visible iff 0 <= kv - (qi - W) <= W
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

  // One step: A(it+1), C(it), B(it+1).  At D <= 128 the order is written out
  // in fenced regions, as in the dK/dV kernel: S's products (the V operands
  // read among them), then dP's with twelve of B's sixteen exponentials (P
  // needs only S), then C's products, each after the transposing reads of the
  // product CA places later, with the last four exponentials and dS' = P (dP -
  // Delta) kscale with its packing.  B(it+1) writes separate registers that
  // C(it+1) takes over.  At D = 256 the compiler orders the step.
  auto step_body = [&](int it, auto masked_c) {
    if constexpr (D <= 128) {
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
      const int t0 = (jb0 + it + 1) * C::BN + 4 * g + W - qi;
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
    } else {
      stage_a(b1);
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < 2 * C::KS - 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      __builtin_amdgcn_sched_barrier(0);
      stage_c(b0);
      stage_b(b1, it + 1, masked_c);
      asm volatile("" ::"v"(dsf[0]), "v"(dsf[1]));
    }
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

  // ---- epilogue: dq_hat = acc / log2(e); RMSNorm backward of q (stores past
  // T dropped).  The raw q rows come in and dq goes out through LDS (the step
  // buffers, free once every wave is past its last product), so global memory
  // sees whole rows.
  const float r = r_q;
  // rotary tables of query qi (channels 32 n + 8 q4 + 4 g + e, n < NB / 2,
  // pair with n + NB / 2), in flight with the reload of the q rows
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
  RS::load_rows(smem, slot, make_rsrc(q + sbase + (size_t)qw0 * rs, slice_bytes - qw0 * rsb), rs, lane);
  float dot = 0.f;
  f32x16 xh[C::NB];
  if constexpr (ROPE) {
    // the norm's input is the rotated q; the table entries serve the way back too
#pragma unroll
    for (int n = 0; n < C::NB / 2; ++n)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const u32x2 q1 = RS::get(smem, slot, c, 32 * n + 8 * q4 + 4 * g);
        const u32x2 q2 = RS::get(smem, slot, c, 32 * (n + C::NB / 2) + 8 * q4 + 4 * g);
        float x1[4] = {bf_lo(q1[0]), bf_hi(q1[0]), bf_lo(q1[1]), bf_hi(q1[1])};
        float x2[4] = {bf_lo(q2[0]), bf_hi(q2[0]), bf_lo(q2[1]), bf_hi(q2[1])};
        rope4(x1, x2, tc[n][q4], tsn[n][q4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xh[n][4 * q4 + e] = x1[e] * r;
          xh[n + C::NB / 2][4 * q4 + e] = x2[e] * r;
        }
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
        xh[n][4 * q4 + e] = x[e] * r;
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

template <int D, bool GROUPED, bool ROPE>
static hipError_t set_dkdv_lds() {
  using C = DkdvCfg<D, GROUPED, ROPE>;
  // more than 64 KiB of dynamic LDS must be opted into, once per kernel
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(bwd_dkdv_kernel<D, GROUPED, ROPE>),
      hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  return attr;
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
  {
    // dQ first: it also writes q_hat, Delta and lse log2(e) for dK/dV
    using C = DqCfg<D, ROPE>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(bwd_dq_kernel<D, ROPE>),
        hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (attr != hipSuccess) return attr;
    const int nqt = (a.T + C::BM - 1) / C::BM;
    ProfToken t2 = prof_begin(K_BWD_DQ, stream);
    hipLaunchKernelGGL((bwd_dq_kernel<D, ROPE>), dim3(nqt * a.B * a.H), dim3(256), C::LDS_BYTES, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.o, kk, vv,
                       (const uint16_t*)a.dout, a.lse, (const float*)a.kscale,
                       (const uint16_t*)a.rcos, (const uint16_t*)a.rsin, (uint16_t*)a.qhat, a.delta,
                       a.lse2, (uint16_t*)a.dq, a.T, a.H, G, W, a.eps);
    prof_end(t2);
  }
  {
    using C = DkdvCfg<D, false, ROPE>;
    static_assert(C::LDS_BYTES == DkdvCfg<D, true, ROPE>::LDS_BYTES, "one LDS size for both versions");
    const hipError_t attr = G == 1 ? set_dkdv_lds<D, false, ROPE>() : set_dkdv_lds<D, true, ROPE>();
    if (attr != hipSuccess) return attr;
    const int nkt = (a.T + C::BNK - 1) / C::BNK;
    const int ntiles = nkt * a.B * a.Hkv;
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1)
      return hipErrorInvalidDevice;
    const int grid = imin(ncu, ntiles);   // persistent: one workgroup per CU
    ProfToken t1 = prof_begin(K_BWD_DKDV, stream);
    hipLaunchKernelGGL((G == 1 ? bwd_dkdv_kernel<D, false, ROPE> : bwd_dkdv_kernel<D, true, ROPE>),
                       dim3(grid), dim3(256), C::LDS_BYTES, stream,
                       (const uint16_t*)a.qhat, kk, vv, (const uint16_t*)a.dout,
                       (const float*)a.lse2, (const float*)a.delta, (const float*)a.kscale,
                       (const uint16_t*)a.rcos, (const uint16_t*)a.rsin, (const uint16_t*)a.ve,
                       (const float*)a.gate, (uint16_t*)a.dk, (uint16_t*)a.dv, (uint16_t*)a.dve, a.dz,
                       a.T, a.H, G, W, nkt, ntiles);
    prof_end(t1);
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
