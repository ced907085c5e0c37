// Device-side building blocks for the gfx950 (CDNA4) attention kernels:
// vector types, bf16 packing, 16-byte loads, the 32x32x16 bf16 MFMA and the
// XCD-aware workgroup remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D = 16 * (number of k-steps of the 32x32x16 MFMA); rows of D bf16 values.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// acc + lo + hi of a packed bf16 pair (one v_dot2c_f32_bf16 against (1, 1)).
__device__ __forceinline__ float sum_bf16x2(uint32_t pk, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), one, acc, false);
}

// C[32x32] += A[32x16] * B[16x32], bf16 inputs, fp32 accumulate.
// Operand layout (lane l, g = l / 32, c = l % 32): A supplies row c, B column c,
// each as 8 consecutive k values of the k-group g; C lane l holds column c,
// rows 8 * (r / 4) + 4 * g + (r % 4) for r = 0..15.
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ---- buffer loads: a descriptor covers one (batch, head) slice from a given
// row on; loads past its num_records (checked on the per-lane offset) return
// zero, which pads ragged tails without branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcFlags = 0x00020000;  // dword 3 of a raw gfx9-family buffer descriptor

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, long long nbytes) {
  const int n = nbytes <= 0 ? 0 : (nbytes >= 0x7fffffffLL ? 0x7fffffff : (int)nbytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kRsrcFlags);
}

// The same for a byte count known to be non-negative and below 2^32 (the
// remaining bytes of one (batch, head) slice): the clamp is one unsigned
// scalar compare instead of a 64-bit vector compare.
__device__ __forceinline__ rsrc_t make_rsrc_u(const void* base, uint32_t nbytes) {
  const int n = nbytes > 0x7fffffffu ? 0x7fffffff : (int)nbytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kRsrcFlags);
}

#define SW_LDS __attribute__((address_space(3)))   // LDS pointers

// The same descriptor as four scalar words, for the direct-to-LDS loads below.
__device__ __forceinline__ u32x4 make_desc(const void* base, long long nbytes) {
  const uint32_t n = nbytes <= 0 ? 0u : (nbytes >= 0x7fffffffLL ? 0x7fffffffu : (uint32_t)nbytes);
  const uint64_t a = (uint64_t)base;
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, n, (uint32_t)kRsrcFlags};
}
__device__ __forceinline__ u32x4 make_desc_u(const void* base, uint32_t nbytes) {
  const uint32_t n = nbytes > 0x7fffffffu ? 0x7fffffffu : nbytes;
  const uint64_t a = (uint64_t)base;
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, n, (uint32_t)kRsrcFlags};
}

// ---- direct-to-LDS loads (buffer_load_dword{,x4} ... lds): lane l's 4 or 16
// bytes land at LDS (M0 + 4 l) or (M0 + 16 l); lanes whose offset is past the
// descriptor's range write zeros.  They are written as inline assembly so that
// the compiler does not track them.  It cannot tell which buffer a transposing
// LDS read touches, and before each one it would otherwise wait for every such
// load in flight -- including the one just issued for a later step, which
// would cut the pipelines' prefetch distance to a fraction of a step.  The
// kernels order these loads themselves: a buffer is read only after
// s_waitcnt vmcnt and a workgroup barrier that follow its loads, a buffer is
// refilled only after a barrier that follows its last reads, and no load is in
// flight when a kernel exits.  The assembly sets no registers; M0 is an input
// and the one wait state between writing M0 and the load is the s_nop.
__device__ __forceinline__ uint32_t lds_addr(unsigned char* smem, int off) {
  return (uint32_t)(uintptr_t)(SW_LDS void*)(smem + off);
}
__device__ __forceinline__ void lds_dma16(u32x4 desc, unsigned char* smem, int lds_off, int voff) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(desc),
               "{m0}"(lds_addr(smem, lds_off)));
}
__device__ __forceinline__ void lds_dma4(u32x4 desc, unsigned char* smem, int lds_off, int voff) {
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(desc),
               "{m0}"(lds_addr(smem, lds_off)));
}

__device__ __forceinline__ u32x4 bload16(rsrc_t r, int voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
}
__device__ __forceinline__ u32x2 bload8(rsrc_t r, int voff) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0);
}
__device__ __forceinline__ float bload4f(rsrc_t r, int voff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}

__device__ __forceinline__ void bstore8(u32x2 v, rsrc_t r, int voff) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, 0, 0);
}
__device__ __forceinline__ void bstore4f(float v, rsrc_t r, int voff) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, 0, 0);
}

__device__ __forceinline__ void bstore16(u32x4 v, rsrc_t r, int voff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, 0, 0);
}

// ---- rotary embedding.  A head's channels pair up as (i, i + D/2); position t
// rotates pair i by the angle whose cosine and sine are the bf16 table entries
// c = cos[t, i], s = sin[t, i]:  y1 = x1 c + x2 s,  y2 = x2 c - x1 s.  The
// gradient goes back through the transpose:  g1' = g1 c - g2 s,
// g2' = g1 s + g2 c.
// rope8: x1, x2 are 8 channels (bf16 pairs) of the first and second half, c, s
// the matching 8 table entries; the rotated channels come back in fp32.
__device__ __forceinline__ void rope8(u32x4 x1, u32x4 x2, u32x4 c, u32x4 s, float* y1, float* y2) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a[2] = {bf_lo(x1[e]), bf_hi(x1[e])}, b[2] = {bf_lo(x2[e]), bf_hi(x2[e])};
    const float cc[2] = {bf_lo(c[e]), bf_hi(c[e])}, ss[2] = {bf_lo(s[e]), bf_hi(s[e])};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      y1[2 * e + h] = a[h] * cc[h] + b[h] * ss[h];
      y2[2 * e + h] = b[h] * cc[h] - a[h] * ss[h];
    }
  }
}
// rope4 / rope4_bwd: 4 fp32 channels of each half in place, tables as 4 bf16.
__device__ __forceinline__ void rope4(float* x1, float* x2, u32x2 c, u32x2 s) {
  const float cc[4] = {bf_lo(c[0]), bf_hi(c[0]), bf_lo(c[1]), bf_hi(c[1])};
  const float ss[4] = {bf_lo(s[0]), bf_hi(s[0]), bf_lo(s[1]), bf_hi(s[1])};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = x1[e], b = x2[e];
    x1[e] = a * cc[e] + b * ss[e];
    x2[e] = b * cc[e] - a * ss[e];
  }
}
__device__ __forceinline__ void rope4_bwd(float* g1, float* g2, u32x2 c, u32x2 s) {
  const float cc[4] = {bf_lo(c[0]), bf_hi(c[0]), bf_lo(c[1]), bf_hi(c[1])};
  const float ss[4] = {bf_lo(s[0]), bf_hi(s[0]), bf_lo(s[1]), bf_hi(s[1])};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = g1[e], b = g2[e];
    g1[e] = a * cc[e] - b * ss[e];
    g2[e] = a * ss[e] + b * cc[e];
  }
}

// ---- value-embedding gate: gate = 2 sigmoid(sum_c w[c] x[c]) over the 32
// gate channels of a token (x bf16, w fp32).  NL consecutive lanes share a
// token, each summing 32 / NL channels starting at 32 / NL * part; every lane
// of the group returns the gate.
template <int NL>
__device__ __forceinline__ float ve_gate_sum(const uint16_t* xrow, const float* w, int part, bool valid) {
  constexpr int NC = 32 / NL;
  static_assert(NC >= 1 && 32 % NL == 0, "lanes per token divide the 32 gate channels");
  float z = 0.f;
  if (valid) {
    if constexpr (NC == 1) {   // one channel per lane
      z = __uint_as_float((uint32_t)xrow[part] << 16) * w[part];
    } else {
#pragma unroll
      for (int j = 0; j < NC; j += 2) {
        const uint32_t xx = *reinterpret_cast<const uint32_t*>(xrow + NC * part + j);
        z += bf_lo(xx) * w[NC * part + j] + bf_hi(xx) * w[NC * part + j + 1];
      }
    }
  }
#pragma unroll
  for (int m = NL / 2; m >= 1; m >>= 1) z += __shfl_xor(z, m, NL);
  return 2.0f / (1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// Wave-uniform value moved to a scalar register.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// ---- transposed LDS reads (ds_read_b64_tr_b16).  In each group of 16 lanes,
// lane i receives slot j = element (i % 4) of the 8-byte chunk addressed by lane
// (i / 4 + 4 j) of the group.  tr4x16 reads a 4 (rows) x 16 (columns) bf16 block
// of a row-major LDS array: lane i of the group gets the column `col0 + i`, rows
// row0 .. row0 + 3, as two packed bf16 pairs.
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_tr4(const uint16_t* p) {
  const SW_LDS bf16x4* q = (const SW_LDS bf16x4*)(p);
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(const_cast<SW_LDS bf16x4*>(q)));
}

// LDS accesses at a per-lane byte address plus a compile-time displacement,
// which the compiler folds into the instruction's offset field.
__device__ __forceinline__ u32x4 lds16(const unsigned char* smem, int addr) {
  return *reinterpret_cast<const u32x4*>(smem + addr);
}
__device__ __forceinline__ f32x4 lds16f(const unsigned char* smem, int addr) {
  return *reinterpret_cast<const f32x4*>(smem + addr);
}
__device__ __forceinline__ u32x2 lds_tr4b(const unsigned char* smem, int addr) {
  return lds_tr4(reinterpret_cast<const uint16_t*>(smem + addr));
}

// ---- direct-to-LDS tiles.  A buffer_load ... lds instruction writes the 16
// bytes of lane l at LDS (M0 base + 16 l), i.e. one contiguous KiB per wave.
// DmaTile fills a tile of R rows of D bf16 stored with a padded row pitch of
// P bf16 (P * 2 an odd multiple of 16 bytes, so row-wise and transposed LDS
// reads avoid bank conflicts): LDS chunk q (16 bytes) of the tile holds row
// q / CPR, chunk q % CPR of the source; pad chunks and rows past R read out of
// the descriptor's range, i.e. zero.  The tile is covered by NI wave
// instructions (a multiple of 4, so each wave of a 256-thread workgroup issues
// the same number, NIW); wave w issues instructions w, w + 4, ...
// KERNEL only makes the instantiation distinct per kernel: with two kernels
// calling one instantiation of issue(), the host pass of this ROCm clang emits
// no launch stub for the second kernel (an undefined symbol at load time).
template <int D, int R, int P, int KERNEL>
struct DmaTile {
  static constexpr int CPR = P / 8;
  static constexpr int NCH = R * CPR;
  static constexpr int NI = ((NCH + 63) / 64 + 3) / 4 * 4;
  static constexpr int NIW = NI / 4;
  static constexpr int BYTES = NI * 1024;
  static_assert((P * 2) % 16 == 0, "pitch must be a whole number of 16-byte chunks");

  int voff[NIW];   // per-lane byte offset into the source, per instruction

  // rs: source row stride in elements
  __device__ __forceinline__ void init(int w, int lane, int rs) {
#pragma unroll
    for (int i = 0; i < NIW; ++i) {
      const int q = 64 * (w + 4 * i) + lane;
      const int r = q / CPR, ch = q % CPR;
      voff[i] = (r < R && ch < D / 8) ? (r * rs + 8 * ch) * 2 : 0x7ffffff0;
    }
  }
  // rs_tile: descriptor starting at the tile's first source row;
  // lds_base: byte offset of the tile in dynamic LDS (wave-uniform)
  __device__ __forceinline__ void issue(u32x4 desc, unsigned char* smem, int lds_base, int w) const {
#pragma unroll
    for (int i = 0; i < NIW; ++i) lds_dma16(desc, smem, lds_base + 1024 * (w + 4 * i), voff[i]);
  }
};

// Direct-to-LDS tile with a per-wave instruction count: the tile's NCH 16-byte
// chunks take NI = ceil(NCH / 64) wave instructions (so waves may issue
// different numbers).  Only for pipelines that wait for
// all outstanding loads (vmcnt 0).  NW waves share the work (wave w issues
// w, w + NW, ...).  The LDS region written is NI KiB; lanes past the tile read
// out of range and write zero there.  Chunk q of the tile
// maps to the source byte offset returned by src(q) (a functor), or to an
// out-of-range offset when src returns a negative value.  TAG keeps the
// instantiations of different kernels apart (see DmaTile).
template <int NCH_, int NW = 4, int TAG = 0>
struct DmaTileV {
  static constexpr int NCH = NCH_;
  static constexpr int NI = (NCH + 63) / 64;
  static constexpr int NIW = (NI + NW - 1) / NW;
  static constexpr int BYTES = NI * 1024;
  int voff[NIW];

  template <typename F>
  __device__ __forceinline__ void init(int w, int lane, F src) {
#pragma unroll
    for (int i = 0; i < NIW; ++i) {
      const int q = 64 * (w + NW * i) + lane;
      const int o = q < NCH ? src(q) : -1;
      voff[i] = o >= 0 ? o : 0x7ffffff0;
    }
  }
  __device__ __forceinline__ void issue(u32x4 desc, unsigned char* smem, int lds_base, int w) const {
#pragma unroll
    for (int i = 0; i < NIW; ++i) issue_one(desc, smem, lds_base, w, i);
  }
  // the wave's i-th instruction alone (i < NIW), for spreading a tile's loads
  __device__ __forceinline__ void issue_one(u32x4 desc, unsigned char* smem, int lds_base, int w, int i) const {
    if (i + 1 < NIW || w + NW * i < NI) lds_dma16(desc, smem, lds_base + 1024 * (w + NW * i), voff[i]);
  }
};

// Row-major LDS staging of one wave's 32 x D block of bf16 values.  The MFMA
// C layout gives lane (g, c) row c, columns 32 n + 8 q4 + 4 g + {0..3}: stored
// straight to global memory those are 8-byte pieces spread over 32 rows.
// Through LDS, global memory sees whole rows instead: 16-byte chunks, four
// rows per wave instruction.  The pitch D + 8 keeps both the 8-byte
// scattered accesses and the 16-byte row accesses free of bank conflicts.
template <int D>
struct RowStage32 {
  static constexpr int OP = D + 8;
  static constexpr int BYTES = 32 * OP * 2;
  static constexpr int NCHUNK = 32 * D / 8 / 64;   // 16-byte chunks per lane
  // 8-byte piece of row c at column col (a multiple of 4)
  static __device__ __forceinline__ void put(unsigned char* smem, int slot, int c, int col, u32x2 v) {
    st8(smem + slot + 2 * (c * OP + col), v);
  }
  static __device__ __forceinline__ u32x2 get(const unsigned char* smem, int slot, int c, int col) {
    return ld8(smem + slot + 2 * (c * OP + col));
  }
  // global rows (row stride rs elements, descriptor at row 0) <-> staging
  static __device__ __forceinline__ void store_rows(const unsigned char* smem, int slot, rsrc_t r, int rs, int lane) {
#pragma unroll
    for (int i = 0; i < NCHUNK; ++i) {
      const int idx = lane + 64 * i, row = idx / (D / 8), ch = idx % (D / 8);
      __builtin_amdgcn_raw_buffer_store_b128(ld16(smem + slot + 2 * (row * OP + 8 * ch)), r,
                                             (row * rs + 8 * ch) * 2, 0, 0);
    }
  }
  // the same rows in two halves: the loads into registers, then their stores
  // to the staging block, so that the loads can fly while other work runs
  static __device__ __forceinline__ void load_regs(u32x4* t, rsrc_t r, int rs, int lane) {
#pragma unroll
    for (int i = 0; i < NCHUNK; ++i) {
      const int idx = lane + 64 * i, row = idx / (D / 8), ch = idx % (D / 8);
      t[i] = bload16(r, (row * rs + 8 * ch) * 2);
    }
  }
  static __device__ __forceinline__ void put_regs(unsigned char* smem, int slot, const u32x4* t, int lane) {
#pragma unroll
    for (int i = 0; i < NCHUNK; ++i) {
      const int idx = lane + 64 * i, row = idx / (D / 8), ch = idx % (D / 8);
      st16(smem + slot + 2 * (row * OP + 8 * ch), t[i]);
    }
  }
};

// One 64-lane 4-byte direct-to-LDS load (256 bytes at lds_base + 4 lane).
__device__ __forceinline__ void dma_row4(u32x4 desc, unsigned char* smem, int lds_base, int voff) {
  lds_dma4(desc, smem, lds_base, voff);
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left unconstrained), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroups are handed to the 8 XCDs round-robin by id.  Remap so that each
// XCD walks one contiguous range of logical ids (neighbouring tiles of the same
// (batch, head) then share that XCD's L2).
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
  if ((nblk & 7) != 0) return bid;
  return (bid & 7) * (nblk >> 3) + (bid >> 3);
}

// The same for a grid that the CUs hold all at once (cpx = CUs per XCD; 0:
// plain xcd_remap).  An XCD's k-th workgroup then lands, round by round, on
// CU k mod cpx, so round j = k / cpx takes the logical ids of its range in
// reverse when j is odd: with the ids in heaviest-first order, the CU that
// gets the heaviest tile of round 0 gets the lightest of round 1.
__device__ __forceinline__ int xcd_remap_paired(int bid, int nblk, int cpx) {
  if ((nblk & 7) != 0) return bid;
  const int per = nblk >> 3;
  int k = bid >> 3;
  if (cpx > 0) {
    const int j = k / cpx, c = k - j * cpx;
    if (j & 1) k = j * cpx + (min(cpx, per - j * cpx) - 1 - c);
  }
  return (bid & 7) * per + k;
}

// Query tile of logical workgroup `lid` for the query-tiled kernels (forward,
// dQ), heaviest first: the nbh (batch, head) slices go in groups of gb; inside
// a group, tile rank r (0 = the last, heaviest query tile) of every slice
// comes before rank r + 1.  Light tiles of all slices thus end the grid, and
// each XCD's contiguous range of logical ids still covers few slices.
__device__ __forceinline__ void query_tile_of(int lid, int nqt, int nbh, int gb, int* bh, int* qt) {
  const int per = gb * nqt;
  const int grp = lid / per, r = lid - grp * per;
  const int gsz = min(gb, nbh - grp * gb);
  const int rank = r / gsz;
  *bh = grp * gb + (r - rank * gsz);
  *qt = nqt - 1 - rank;
}


// Query prologue shared by the forward and dQ kernels: lane (g, c) holds
// channels 16 ks + 8 g + 0..7 (ks < D / 16) of query qw0 + c as bf16 pairs.
// With ROPE they are rotated first (the partner of k-step ks is ks + D / 32,
// channels + D / 2, in the same lane).  On return they hold q_hat = x r,
// r = 1 / sqrt(mean x^2 + eps), as bf16; the function returns r.
template <int D, bool ROPE>
__device__ __forceinline__ float normalise_query(u32x4* qf, const uint16_t* rcos, const uint16_t* rsin,
                                                 int qw0, int c, int g, int T, float eps) {
  constexpr int KS = D / 16;
  float x[KS][8];
  if constexpr (ROPE) {
    const long long tb = (long long)(T - qw0) * D;
    const rsrc_t rc = make_rsrc(rcos + (size_t)qw0 * (D / 2), tb);
    const rsrc_t rn = make_rsrc(rsin + (size_t)qw0 * (D / 2), tb);
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks) {
      const int off = (c * (D / 2) + 16 * ks + 8 * g) * 2;
      rope8(qf[ks], qf[ks + KS / 2], bload16(rc, off), bload16(rn, off), x[ks], x[ks + KS / 2]);
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[ks][2 * e] = bf_lo(qf[ks][e]);
        x[ks][2 * e + 1] = bf_hi(qf[ks][e]);
      }
  }
  float ss = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += x[ks][j] * x[ks][j];
  ss += __shfl_xor(ss, 32);
  const float r = 1.0f / sqrtf(ss * (1.0f / D) + eps);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 4; ++e) qf[ks][e] = pack_bf16(x[ks][2 * e] * r, x[ks][2 * e + 1] * r);
  return r;
}

// A-operand of a 32x32x16 MFMA whose k index runs along the rows of a row-major
// LDS tile (two transposing reads): lane (g, c) gets column col0 + c of rows
// row0 + 4 g + {0,1,2,3} and row0 + 8 + 4 g + {0,1,2,3}, i.e. element j is row
// row0 + 4 g + (j % 4) + 8 (j / 4) -- the k order of probabilities held in the
// C layout of a previous product.  `off` is the per-lane part from tr_off().
__device__ __forceinline__ int tr_off(int lane, int P) {
  const int li = lane & 15, g = lane >> 5;
  return (4 * g + (li >> 2)) * P + 16 * ((lane >> 4) & 1) + 4 * (li & 3);
}

}  // namespace swattn
