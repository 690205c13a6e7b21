// attn_bwd_bf16.hip -- backward of RIB window attention on bf16 matrix cores
// (gfx950, v_mfma_f32_32x32x16_bf16 and v_mfma_f32_16x16x32_bf16).
//
// The gradients of O = (softmax(S) V) * sigmoid(G), S = Qt Kt^T with the
// augmented rows Qt = [Qp/sqrt(R), Qc/sqrt(dh)], Kt = [Kp, Kc] ("Rank-
// Factorized Implicit Neural Bias", gist.science summaries part A, the
// concatenation identity; omica.com.cn explainer sections 2.2, 2.3 and the
// training iteration of 4.1), given dA = dO * sigmoid(G) and D = dO . O from
// the prep pass and the forward's row log-sum-exp:
//   P = exp(S - lse),  dS = P * (dA V^T - D)
//   dQt = dS Kt,  dKt = dS^T Qt,  dV = P^T dA
//
// Both passes put every per-row constant into the contractions, so an
// element of the score tile costs one exp2, one multiply and one convert:
//  * the score rows carry log2(e) (base-2 softmax) and two extra columns: the
//    query side holds -lse*log2(e) split into a bf16 high part and a bf16
//    remainder, the key side holds (1, 1).  The MFMA returns t = s*log2(e) -
//    lse*log2(e) and P = exp2(t);
//  * the value rows V' = [V | 1 1 | 0] and gradient rows dA' = [dA | -D_hi
//    -D_lo | 0] (the head dimension padded to 32 has the room) make the MFMA
//    return dP - D directly.
//  * padded rows (past the window's real tokens) are all zero on every side:
//    their P is exp2(0) = 1 but their dP - D is 0 (padded keys, dq pass) or
//    their dA' row is 0 (padded queries, dkv pass), so they add nothing; no
//    masking instructions are needed.
//
// dq pass (query-major): a workgroup of 4 waves owns 256 queries of one
// (image, window, head); each wave keeps the B operands of its 64 queries
// (augmented query rows and dA' rows) in VGPRs and streams the window's keys
// through LDS in tiles of 64.  S^T = Kt Qt^T and (dP - D)^T = V' dA'^T come
// out with lane = query, 16 keys per lane; dS^T, rounded to bf16, is then the
// B operand of dQt^T += Kt^T dS^T, whose A operand is read from the same LDS
// rows with the transposing ds_read_b64_tr_b16 (the forward kernel's PV
// trick).  dkv pass (key-major): the mirror image, lane = key: S = Qt Kt^T,
// dP - D = dA' V'^T, then dV'^T += dA'^T P and dKt^T += Qt^T dS.
// Where the augmented gradient has 33-48 columns (dh = 30, R = 16: 46), its
// columns 32-47 come from two 16x16x32 products per 32-row block instead of a
// 32x32 tile whose upper half would be padding: both operands are regrouped
// across 16-lane rows with v_permlane16_swap (4 per operand), half the matrix
// core time of the padded tile (4.6% off the whole backward at 32 x 96x96).
// Two workgroups share a CU (164 and 255 registers per lane), each waiting only at
// its own per-tile barrier; one workgroup of 8 waves and 512 rows per CU took
// 4% longer on the 32 x 96x96 workload (bit-identical gradients).
//
// LDS layout (both passes): a tile of TT rows is stored chunk-major, one
// 16-byte chunk = 8 consecutive bf16 columns of a row, chunk c of row j at
// dword c*CS + 4j with the chunk stride CS = 4*TT + 16.  A row read of a
// score A operand (16 lanes = 16 rows of one chunk) and a staging write are
// 256 contiguous bytes; a 16-lane group of a transposing read takes 4 rows x
// 16 bytes from two neighbouring chunks, which the 16-dword pad puts on
// disjoint banks.  All three access kinds are free of bank conflicts.
#include "rib_bwd.hpp"
#include "rib_device.hpp"

namespace rib {

namespace {

constexpr int NWV = 4;         // waves per workgroup (two workgroups per CU, each with its own barriers)
constexpr int RW = 64;         // own rows per wave (two 32-row MFMA blocks)
constexpr int RB = NWV * RW;   // own rows per workgroup
constexpr int TT = 64;         // streamed rows per LDS tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr int CS = 4 * TT + 16;  // dwords between consecutive 8-column chunks of a tile

template <int DH, int R>
struct BS {
  static_assert(DH % 2 == 0 && R % 2 == 0, "even head dim and rank");
  static constexpr int C0 = R + DH;                  // first of the two constant columns
  static constexpr int KC = (R + DH + 2 + 15) / 16;  // 16-column chunks of an augmented row
  static constexpr int DC = (DH + 2 + 15) / 16;      // 16-column chunks of a value / gradient row
  static constexpr int MT = (R + DH + 31) / 32;      // 32-column tiles of an augmented gradient
  // the last tile holds at most 16 useful columns: computed as two 16x16x32
  // products (columns 32-47 only) instead of a 32-column tile
  static constexpr bool H16 = MT == 2 && R + DH <= 48;
  static constexpr int MF = H16 ? 1 : MT;            // 32-column tiles computed as such
  static constexpr int AP = 2 * KC;                  // 8-column pieces of an augmented row
  static constexpr int NP = AP + 2 * DC;             // pieces staged per streamed row
  static constexpr int A_DW = 2 * KC * CS;           // dwords of the augmented tile
  static constexpr int V_DW = 2 * DC * CS;           // dwords of the value / gradient tile
  static constexpr int ST_DW = A_DW + V_DW;
  static_assert(DC == 2, "value rows are one 32-column tile");
  static_assert(NP == 10, "packed rows of 160 bytes");
  static_assert(NP <= 3 * NWV, "at most three staging pieces per thread");
};

// dword of chunk c (columns 8c .. 8c+7) of row j of a tile
__device__ __forceinline__ int chunk_dw(int c, int j) { return c * CS + 4 * j; }

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

__device__ __forceinline__ u32x2_t ds_read_tr16(const uint32_t* p) {
  const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4_t*)(__attribute__((address_space(3))) void*)(const_cast<uint32_t*>(p)));
  return __builtin_bit_cast(u32x2_t, r);
}

// A operand of X^T B for the 32 columns [c32, c32+32) of a tile and its rows
// [kofs, kofs+16): lane (column, 8 rows) in the row order of a 32x32
// accumulator's registers (the forward kernel's V^T reads).  In a 16-lane
// group q of the transposing read, input lane j = 4k + m supplies columns
// 16(q%2) + 4m .. +3 of row 4(q/2) + k (and of row +8 for the second read).
// tbase = dword index of the tile, lbase = tr_lane_base(lane).
__device__ __forceinline__ u32x4_t tr_operand(const uint32_t* lds, int tbase, int lbase, int kofs, int c32) {
  const int off = (c32 >> 3) * CS + 4 * kofs;
  const u32x2_t lo = ds_read_tr16(lds + tbase + lbase + off);
  const u32x2_t hi = ds_read_tr16(lds + tbase + lbase + off + 32);
  return (u32x4_t){lo[0], lo[1], hi[0], hi[1]};
}

__device__ __forceinline__ int tr_lane_base(int lane) {
  const int q = lane >> 4, j = lane & 15;
  const int row = 4 * (q >> 1) + (j >> 2);
  const int col = 16 * (q & 1) + 4 * (j & 3);
  return chunk_dw(col >> 3, row) + 2 * ((col >> 2) & 1);
}

__device__ __forceinline__ float f32(uint32_t x) { return __builtin_bit_cast(float, x); }

// ---- operand rows ------------------------------------------------------------
// Raw loads of one 8-column piece (4 column pairs) of a row, converted later:
// pair k of the piece sits in raw[2k] (and raw[2k+1] for fp32 sources).
struct Raw {
  uint32_t w[8];
};

// Sources of the four row kinds; `tok` = token index, `n` = in-window index.
struct RowSrc {
  const uint32_t* map;   // bf16 pairs of the NHWC map of the content part (dword index = element / 2)
  const float* pos;      // positional table [ws*ws][R]
  const uint32_t* val;   // bf16 pairs of the value / gradient map
  const float* rowc;     // per (token, head) constant: lse (query rows) or D (gradient rows)
};

// augmented row [P | content | const pair | 0]: P = positional factor (fp32),
// content = bf16 map slice.  kind 0: key row (const pair 1, 1);
// kind 1: query row (P * sp, content * sc, const pair = -lse*log2e split).
template <int DH, int R, int P, int KIND>
__device__ __forceinline__ void load_aug(const RowSrc& s, long tok, int n, long cofs, long crow, Raw& raw) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int col = 8 * P + 2 * k;
    if (col < R) {
      const float2 f = *reinterpret_cast<const float2*>(s.pos + (long)n * R + col);
      raw.w[2 * k] = __builtin_bit_cast(uint32_t, f.x);
      raw.w[2 * k + 1] = __builtin_bit_cast(uint32_t, f.y);
    } else if (col < R + DH) {
      raw.w[2 * k] = s.map[(cofs + col - R) >> 1];
    } else if (col == R + DH && KIND == 1) {
      raw.w[2 * k] = __builtin_bit_cast(uint32_t, s.rowc[crow]);
    }
  }
}

// -x split into a bf16 high part and a bf16 remainder, packed (low half = high part)
__device__ __forceinline__ uint32_t neg_split(float x) {
  const float hi = round_bf16(x);
  return pack_bf16(-hi, -(x - hi));
}

template <int DH, int R, int P, int KIND>
__device__ __forceinline__ u32x4_t cvt_aug(const Raw& raw, bool real, float sp, float sc) {
  uint32_t d[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int col = 8 * P + 2 * k;
    uint32_t x = 0u;
    if (col < R) {
      x = KIND == 1 ? pack_bf16(f32(raw.w[2 * k]) * sp, f32(raw.w[2 * k + 1]) * sp)
                    : pack_bf16(f32(raw.w[2 * k]), f32(raw.w[2 * k + 1]));
    } else if (col < R + DH) {
      x = KIND == 1 ? pack_bf16(bf16_lo(raw.w[2 * k]) * sc, bf16_hi(raw.w[2 * k]) * sc) : raw.w[2 * k];
    } else if (col == R + DH) {
      x = KIND == 1 ? neg_split(f32(raw.w[2 * k]) * LOG2E) : 0x3F803F80u;
    }
    d[k] = real ? x : 0u;
  }
  return (u32x4_t){d[0], d[1], d[2], d[3]};
}

// value-like row [x | const pair | 0] over 32 columns: kind 0: V with (1, 1);
// kind 1: dA with (-D_hi, -D_lo).  P = piece 0..3.
template <int DH, int P, int KIND>
__device__ __forceinline__ void load_val(const RowSrc& s, long vofs, long crow, Raw& raw) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int col = 8 * P + 2 * k;
    if (col < DH) raw.w[2 * k] = s.val[(vofs + col) >> 1];
    else if (col == DH && KIND == 1) raw.w[2 * k] = __builtin_bit_cast(uint32_t, s.rowc[crow]);
  }
}

template <int DH, int P, int KIND>
__device__ __forceinline__ u32x4_t cvt_val(const Raw& raw, bool real) {
  uint32_t d[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int col = 8 * P + 2 * k;
    uint32_t x = 0u;
    if (col < DH) x = raw.w[2 * k];
    else if (col == DH) x = KIND == 1 ? neg_split(f32(raw.w[2 * k])) : 0x3F803F80u;
    d[k] = real ? x : 0u;
  }
  return (u32x4_t){d[0], d[1], d[2], d[3]};
}

// Piece p of a row (p < AP: augmented row, else value-like row).
// KIND 0: key-side rows (Kt, V'), KIND 1: query-side rows (Qt, dA').
template <int DH, int R, int P, int KIND>
__device__ __forceinline__ void load_piece(const RowSrc& aug, const RowSrc& val, long tok, int n, long cofs,
                                           long crow, Raw& raw) {
  using S = BS<DH, R>;
  if constexpr (P < S::AP) load_aug<DH, R, P, KIND>(aug, tok, n, cofs, crow, raw);
  else load_val<DH, P - S::AP, KIND>(val, cofs, crow, raw);
}

template <int DH, int R, int KIND, int P = 0>
__device__ __forceinline__ u32x4_t make_chunk(int c, const RowSrc& aug, const RowSrc& val, long tok, int n, long cofs,
                                              long crow, bool real, float sp, float sc) {
  using S = BS<DH, R>;
  if constexpr (P < S::NP) {
    if (c == P) {
      Raw raw = {};
      if (real) load_piece<DH, R, P, KIND>(aug, val, tok, n, cofs, crow, raw);
      if constexpr (P < S::AP) return cvt_aug<DH, R, P, KIND>(raw, real, sp, sc);
      else return cvt_val<DH, P - S::AP, KIND>(raw, real);
    }
    return make_chunk<DH, R, KIND, P + 1>(c, aug, val, tok, n, cofs, crow, real, sp, sc);
  } else {
    return (u32x4_t){0u, 0u, 0u, 0u};
  }
}

// ---- pack pass -----------------------------------------------------------------
// Writes the operand rows of one side of every unit in the LDS tile image:
// [unit][tile][chunk][row][16 bytes] (1 KB per chunk of 64 rows); rows past
// the window's real tokens are zero.  One thread per (unit, tile, chunk, row),
// one wave per chunk.  KIND 0: key side (Kt with (1, 1), V' with (1, 1));
// KIND 1: query side (Qt with -lse*log2e, dA' with -D).
template <int DH, int R, int KIND>
__global__ void __launch_bounds__(256)
bwd_pack_kernel(BwdArgs a, long total) {
  using S = BS<DH, R>;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int row = (int)(idx & 63);
  long t = idx >> 6;
  const int c = (int)(t % S::NP);
  t /= S::NP;
  const int tile = (int)(t % a.tu);
  const int unit = (int)(t / a.tu);
  Unit u;
  decode_unit(unit, a, a.ws * a.ws, u);
  const int r = tile * TT + row;
  const bool real = r < u.n_real;
  long tok;
  int n;
  locate(u, a, real ? r : 0, tok, n);
  const long cofs = tok * (long)(a.heads * DH) + (long)u.h * DH;
  const long crow = tok * a.heads + u.h;
  const float sp = LOG2E / sqrtf((float)R), sc = LOG2E / sqrtf((float)DH);
  u32x4_t out;
  if constexpr (KIND == 0) {
    const RowSrc aug{(const uint32_t*)a.kc, a.kp + u.h * a.tstride, nullptr, nullptr};
    const RowSrc val{nullptr, nullptr, (const uint32_t*)a.v, nullptr};
    out = make_chunk<DH, R, 0>(c, aug, val, tok, n, cofs, crow, real, sp, sc);
  } else {
    const RowSrc aug{(const uint32_t*)a.qc, a.qp + u.h * a.tstride, nullptr, a.lse};
    const RowSrc val{nullptr, nullptr, (const uint32_t*)a.da, a.dsum};
    out = make_chunk<DH, R, 1>(c, aug, val, tok, n, cofs, crow, real, sp, sc);
  }
  reinterpret_cast<u32x4_t*>(KIND == 0 ? a.pk : a.pq)[idx] = out;
}

__device__ __forceinline__ f32x16_t mfma(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int e = 0; e < 16; ++e) z[e] = 0.0f;
  return z;
}

// A 16 x 16 product over 32 contraction rows: lane l holds row (A) or column
// (B) l % 16 with contraction rows 8(l/16) .. +7, and the result rows
// 4(l/16) .. +3 of column l % 16.
__device__ __forceinline__ f32x4_t mfma16(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// Two 32x32x16 operands x (contraction rows 0-15) and y (rows 16-31) of one
// 32-row block, regrouped for 16x16x32 products by swapping 16-lane rows
// (v_permlane16_swap: the odd rows of x trade places with the even rows of
// y).  Lane half h of x holds rows {4h..4h+3, 8+4h..8+4h+3} of the block's
// first 16, of y the same rows of the second 16.  Afterwards lo holds rows
// 0-15 of the block (columns or rows l % 16) and hi rows 16-31, and in both
// the lane groups l/16 = 0..3 carry the contraction rows of (x, h = 0),
// (y, h = 0), (x, h = 1), (y, h = 1): all 32, the same in lo and hi.
struct Halves {
  u32x4_t lo, hi;
};
__device__ __forceinline__ Halves regroup16(const u32x4_t& x, const u32x4_t& y) {
  Halves r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto p = __builtin_amdgcn_permlane16_swap(x[i], y[i], false, false);
    r.lo[i] = p[0];
    r.hi[i] = p[1];
  }
  return r;
}

// Shared frame of both passes: the unit, this wave's own rows and the
// streamed side's packed image.
template <int DH, int R>
struct Frame {
  using S = BS<DH, R>;
  Unit u;
  int unit, r0, wave, lane, l32, hh, ntiles;
  bool active;
  const uint32_t* own;     // packed image of the own side of this unit
  __amdgpu_buffer_rsrc_t other;  // packed image of the streamed side of this unit

  __device__ __forceinline__ bool init(const BwdArgs& a, int total, const uint32_t* own_img,
                                       const uint32_t* other_img) {
    const int logical = xcd_swizzle(blockIdx.x, gridDim.x);
    if (logical >= total) return false;
    if (!decode_unit(logical, a, RB, u)) return false;
    unit = logical / ((a.ws * a.ws + RB - 1) / RB);
    const int tid = threadIdx.x;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    lane = tid & 63;
    l32 = lane & 31;
    hh = lane >> 5;
    r0 = u.blk * RB + wave * RW;
    active = r0 < u.n_real;
    ntiles = (u.n_real + TT - 1) / TT;
    const long img = (long)unit * a.tu * S::NP * 256;  // dwords per unit image
    own = own_img + img;
    other = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(other_img + img), (short)0,
                                              a.tu * S::NP * 1024, (int)0x00020000u);
    return true;
  }

  // B operands of own row r: augmented chunks 2c + hh and value-like chunks
  __device__ __forceinline__ void own_row(int r, u32x4_t (&at)[S::KC], u32x4_t (&vt)[2]) const {
    const bool real = r < u.n_real;
    const uint32_t* base = own + ((r >> 6) * S::NP) * 256 + (r & 63) * 4;
#pragma unroll
    for (int c = 0; c < S::KC; ++c)
      at[c] = real ? *reinterpret_cast<const u32x4_t*>(base + (2 * c + hh) * 256) : (u32x4_t){0u, 0u, 0u, 0u};
#pragma unroll
    for (int c = 0; c < 2; ++c)
      vt[c] = real ? *reinterpret_cast<const u32x4_t*>(base + (S::AP + 2 * c + hh) * 256) : (u32x4_t){0u, 0u, 0u, 0u};
  }

  // LDS-direct copy of streamed tile t into the stage `dst`: wave w copies
  // chunks w, w + 4 and w + 8; lane l writes row l of the chunk.
  __device__ __forceinline__ void issue(uint32_t* dst, int t) const {
#pragma unroll
    for (int k = 0; k < (S::NP + NWV - 1) / NWV; ++k) {
      const int cc = wave + NWV * k;
      if (cc < S::NP) {
        const unsigned off = (unsigned)(((t * S::NP + cc) * 256 + lane * 4) * 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(other, (__attribute__((address_space(3))) void*)(dst + cc * CS),
                                                 16, off, 0, 0, 0);
      }
    }
  }
};

// ---- dq pass -------------------------------------------------------------------
template <int DH, int R>
__global__ void __launch_bounds__(RB, 2)
bwd_dq_bf16_kernel(BwdArgs a, int total) {
  using S = BS<DH, R>;
  // two stages as two arrays (not one double buffer): the compiler then sees
  // that reads of one stage do not depend on the copies landing in the other
  // and does not wait for those copies before every read
  __shared__ __attribute__((aligned(16))) uint32_t lds0[S::ST_DW];
  __shared__ __attribute__((aligned(16))) uint32_t lds1[S::ST_DW];
  Frame<DH, R> f;
  if (!f.init(a, total, a.pq, a.pk)) return;
  const int l32 = f.l32, hh = f.hh;

  u32x4_t qt[2][S::KC], dat[2][2];
  f32x16_t acc[2][S::MF];
  f32x4_t acc16[2][2];  // H16: columns 32-47 of rows 0-15 and 16-31 of each block
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    f.own_row(f.r0 + qb * 32 + l32, qt[qb], dat[qb]);
#pragma unroll
    for (int mt = 0; mt < S::MF; ++mt) acc[qb][mt] = zero16();
    acc16[qb][0] = acc16[qb][1] = (f32x4_t){0.0f, 0.0f, 0.0f, 0.0f};
  }

  f.issue(lds0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int lb = tr_lane_base(f.lane);
  // tile t from stage `cur` while tile t + 1 lands in `nxt`
  auto tile = [&](const uint32_t* cur, uint32_t* nxt, int t) {
    if (t + 1 < f.ntiles) f.issue(nxt, t + 1);
    if (f.active) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        u32x4_t ka[S::KC], va[2], kt[S::MT][2];
#pragma unroll
        for (int c = 0; c < S::KC; ++c)
          ka[c] = *reinterpret_cast<const u32x4_t*>(cur + chunk_dw(2 * c + hh, kb * 32 + l32));
#pragma unroll
        for (int c = 0; c < 2; ++c)
          va[c] = *reinterpret_cast<const u32x4_t*>(cur + S::A_DW + chunk_dw(2 * c + hh, kb * 32 + l32));
#pragma unroll
        for (int mt = 0; mt < S::MT; ++mt)
#pragma unroll
          for (int c2 = 0; c2 < 2; ++c2) kt[mt][c2] = tr_operand(cur, 0, lb, kb * 32 + 16 * c2, 32 * mt);
        u32x4_t k16;  // H16: the last tile's operand for columns 32-47
        if constexpr (S::H16) k16 = regroup16(kt[1][0], kt[1][1]).lo;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          f32x16_t s = zero16(), d = zero16();
#pragma unroll
          for (int c = 0; c < S::KC; ++c) s = mfma(ka[c], qt[qb][c], s);
#pragma unroll
          for (int c = 0; c < 2; ++c) d = mfma(va[c], dat[qb][c], d);
          uint32_t ds[8];
#pragma unroll
          for (int i = 0; i < 8; ++i)
            ds[i] = pack_bf16(__builtin_amdgcn_exp2f(s[2 * i]) * d[2 * i],
                              __builtin_amdgcn_exp2f(s[2 * i + 1]) * d[2 * i + 1]);
          const u32x4_t db[2] = {{ds[0], ds[1], ds[2], ds[3]}, {ds[4], ds[5], ds[6], ds[7]}};
#pragma unroll
          for (int mt = 0; mt < S::MF; ++mt)
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) acc[qb][mt] = mfma(kt[mt][c2], db[c2], acc[qb][mt]);
          if constexpr (S::H16) {
            const Halves b = regroup16(db[0], db[1]);
            acc16[qb][0] = mfma16(k16, b.lo, acc16[qb][0]);
            acc16[qb][1] = mfma16(k16, b.hi, acc16[qb][1]);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of the next tile have landed
    __syncthreads();
  };
  for (int t = 0; t < f.ntiles; t += 2) {
    tile(lds0, lds1, t);
    if (t + 1 < f.ntiles) tile(lds1, lds0, t + 1);
  }
  if (!f.active) return;

  // ---- epilogue: register e of acc[qb][mt] is column 32mt + 8(e/4) + 4hh + e%4
  // of row l32; register i of acc16[qb][h] column 32 + 4(lane/16) + i of row
  // 16h + lane%16
  const Unit& u = f.u;
  const int C = a.heads * DH;
  const float gq = 1.0f / sqrtf((float)R), gc = 1.0f / sqrtf((float)DH);
  uint32_t* dqc = (uint32_t*)a.dqc;
  // columns c0 .. c0+3 of the own row at token tok
  auto put4 = [&](long tok, int c0, float x0, float x1, float x2, float x3) {
    if (c0 + 4 <= R) {
      float* qrow = a.qrows + (((long)u.h * a.B + u.b) * a.H * a.W + (tok - (long)u.b * a.H * a.W)) * R;
      *reinterpret_cast<float4*>(qrow + c0) = make_float4(x0 * gq, x1 * gq, x2 * gq, x3 * gq);
    } else if (c0 >= R && c0 < R + DH) {
      const long e = (tok * C + (long)u.h * DH + c0 - R) >> 1;
      dqc[e] = pack_bf16(x0 * gc, x1 * gc);
      if (c0 + 2 < R + DH) dqc[e + 1] = pack_bf16(x2 * gc, x3 * gc);
    }
  };
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int r = f.r0 + qb * 32 + l32;
    long tok;
    int n;
    if (r < u.n_real) {
      locate(u, a, r, tok, n);
#pragma unroll
      for (int mt = 0; mt < S::MF; ++mt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x16_t& x = acc[qb][mt];
          put4(tok, 32 * mt + 8 * g4 + 4 * hh, x[4 * g4], x[4 * g4 + 1], x[4 * g4 + 2], x[4 * g4 + 3]);
        }
    }
    if constexpr (S::H16) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r16 = f.r0 + qb * 32 + 16 * h + (f.lane & 15);
        const f32x4_t& x = acc16[qb][h];
        if (r16 < u.n_real) {
          locate(u, a, r16, tok, n);
          put4(tok, 32 + 4 * (f.lane >> 4), x[0], x[1], x[2], x[3]);
        }
      }
    }
  }
}

// ---- dkv pass ------------------------------------------------------------------
template <int DH, int R>
__global__ void __launch_bounds__(RB, 2)
bwd_dkv_bf16_kernel(BwdArgs a, int total) {
  using S = BS<DH, R>;
  // two stages as two arrays, as in the dq pass
  __shared__ __attribute__((aligned(16))) uint32_t lds0[S::ST_DW];
  __shared__ __attribute__((aligned(16))) uint32_t lds1[S::ST_DW];
  Frame<DH, R> f;
  if (!f.init(a, total, a.pk, a.pq)) return;
  const int l32 = f.l32, hh = f.hh;

  u32x4_t kt[2][S::KC], vt[2][2];
  f32x16_t accv[2], acck[2][S::MF];
  f32x4_t acck16[2][2];  // H16: columns 32-47 of rows 0-15 and 16-31 of each block
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    f.own_row(f.r0 + kb * 32 + l32, kt[kb], vt[kb]);
    accv[kb] = zero16();
#pragma unroll
    for (int mt = 0; mt < S::MF; ++mt) acck[kb][mt] = zero16();
    acck16[kb][0] = acck16[kb][1] = (f32x4_t){0.0f, 0.0f, 0.0f, 0.0f};
  }

  f.issue(lds0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int lb = tr_lane_base(f.lane);
  // tile t from stage `cur` while tile t + 1 lands in `nxt`
  auto tile = [&](const uint32_t* cur, uint32_t* nxt, int t) {
    if (t + 1 < f.ntiles) f.issue(nxt, t + 1);
    if (f.active) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        u32x4_t qa[S::KC], ga[2], gT[2], qT[S::MT][2];
#pragma unroll
        for (int c = 0; c < S::KC; ++c)
          qa[c] = *reinterpret_cast<const u32x4_t*>(cur + chunk_dw(2 * c + hh, qb * 32 + l32));
#pragma unroll
        for (int c = 0; c < 2; ++c)
          ga[c] = *reinterpret_cast<const u32x4_t*>(cur + S::A_DW + chunk_dw(2 * c + hh, qb * 32 + l32));
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) gT[c2] = tr_operand(cur, S::A_DW, lb, qb * 32 + 16 * c2, 0);
#pragma unroll
        for (int mt = 0; mt < S::MT; ++mt)
#pragma unroll
          for (int c2 = 0; c2 < 2; ++c2) qT[mt][c2] = tr_operand(cur, 0, lb, qb * 32 + 16 * c2, 32 * mt);
        u32x4_t q16;  // H16: the last tile's operand for columns 32-47
        if constexpr (S::H16) q16 = regroup16(qT[1][0], qT[1][1]).lo;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          f32x16_t s = zero16(), d = zero16();
#pragma unroll
          for (int c = 0; c < S::KC; ++c) s = mfma(qa[c], kt[kb][c], s);
#pragma unroll
          for (int c = 0; c < 2; ++c) d = mfma(ga[c], vt[kb][c], d);
          uint32_t pp[8], ds[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float p0 = __builtin_amdgcn_exp2f(s[2 * i]), p1 = __builtin_amdgcn_exp2f(s[2 * i + 1]);
            pp[i] = pack_bf16(p0, p1);
            ds[i] = pack_bf16(p0 * d[2 * i], p1 * d[2 * i + 1]);
          }
          const u32x4_t db[2] = {{ds[0], ds[1], ds[2], ds[3]}, {ds[4], ds[5], ds[6], ds[7]}};
#pragma unroll
          for (int c2 = 0; c2 < 2; ++c2) {
            const u32x4_t pb = {pp[4 * c2], pp[4 * c2 + 1], pp[4 * c2 + 2], pp[4 * c2 + 3]};
            accv[kb] = mfma(gT[c2], pb, accv[kb]);
#pragma unroll
            for (int mt = 0; mt < S::MF; ++mt) acck[kb][mt] = mfma(qT[mt][c2], db[c2], acck[kb][mt]);
          }
          if constexpr (S::H16) {
            const Halves b = regroup16(db[0], db[1]);
            acck16[kb][0] = mfma16(q16, b.lo, acck16[kb][0]);
            acck16[kb][1] = mfma16(q16, b.hi, acck16[kb][1]);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  for (int t = 0; t < f.ntiles; t += 2) {
    tile(lds0, lds1, t);
    if (t + 1 < f.ntiles) tile(lds1, lds0, t + 1);
  }
  if (!f.active) return;

  // ---- epilogue: register e is row/column 32mt + 8(e/4) + 4hh + e%4 of the key's gradient
  const Unit& u = f.u;
  const int C = a.heads * DH;
  uint32_t* dkc = (uint32_t*)a.dkc;
  uint32_t* dvo = (uint32_t*)a.dv;
  auto krows_of = [&](long tok) {
    return a.krows + (((long)u.h * a.B + u.b) * a.H * a.W + (tok - (long)u.b * a.H * a.W)) * R;
  };
  // columns c0 .. c0+3 of a key's gradient row (krow: its table row, cofs: its first channel)
  auto put4 = [&](float* krow, long cofs, int c0, float x0, float x1, float x2, float x3) {
    if (c0 + 4 <= R) {
      *reinterpret_cast<float4*>(krow + c0) = make_float4(x0 * LN2, x1 * LN2, x2 * LN2, x3 * LN2);
    } else if (c0 >= R && c0 < R + DH) {
      const long e = (cofs + c0 - R) >> 1;
      dkc[e] = pack_bf16(x0 * LN2, x1 * LN2);
      if (c0 + 2 < R + DH) dkc[e + 1] = pack_bf16(x2 * LN2, x3 * LN2);
    }
  };
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int r = f.r0 + kb * 32 + l32;
    if (r >= u.n_real) continue;
    long tok;
    int n;
    locate(u, a, r, tok, n);
    const long cofs = tok * C + (long)u.h * DH;
    float* krow = krows_of(tok);
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int c0 = 8 * g4 + 4 * hh;
      const f32x16_t& x = accv[kb];
      if (c0 < DH) {
        const long e = (cofs + c0) >> 1;
        dvo[e] = pack_bf16(x[4 * g4], x[4 * g4 + 1]);
        if (c0 + 2 < DH) dvo[e + 1] = pack_bf16(x[4 * g4 + 2], x[4 * g4 + 3]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < S::MF; ++mt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x16_t& x = acck[kb][mt];
        put4(krow, cofs, 32 * mt + 8 * g4 + 4 * hh, x[4 * g4], x[4 * g4 + 1], x[4 * g4 + 2], x[4 * g4 + 3]);
      }
  }
  if constexpr (S::H16) {
    // register i of acck16[kb][h] is column 32 + 4(lane/16) + i of key row 16h + lane%16
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = f.r0 + kb * 32 + 16 * h + (f.lane & 15);
        if (r >= u.n_real) continue;
        long tok;
        int n;
        locate(u, a, r, tok, n);
        const f32x4_t& x = acck16[kb][h];
        put4(krows_of(tok), tok * C + (long)u.h * DH, 32 + 4 * (f.lane >> 4), x[0], x[1], x[2], x[3]);
      }
  }
}

template <int DH, int R>
hipError_t launch_variant(const BwdArgs& a, hipStream_t stream) {
  using S = BS<DH, R>;
  const int nWy = (a.H + a.ws - 1) / a.ws, nWx = (a.W + a.ws - 1) / a.ws;
  const long pack_total = (long)a.B * nWy * nWx * a.heads * a.tu * S::NP * TT;
  const int pgrid = (int)((pack_total + 255) / 256);
  hipLaunchKernelGGL((bwd_pack_kernel<DH, R, 0>), dim3(pgrid), dim3(256), 0, stream, a, pack_total);
  hipLaunchKernelGGL((bwd_pack_kernel<DH, R, 1>), dim3(pgrid), dim3(256), 0, stream, a, pack_total);
  const int total = bwd_units(a, RB);
  const int grid = 8 * ((total + 7) / 8);
  hipLaunchKernelGGL((bwd_dq_bf16_kernel<DH, R>), dim3(grid), dim3(RB), 0, stream, a, total);
  hipLaunchKernelGGL((bwd_dkv_bf16_kernel<DH, R>), dim3(grid), dim3(RB), 0, stream, a, total);
  return hipGetLastError();
}

}  // namespace

bool attn_bwd_bf16_supported(int dh, int R) { return (dh == 30 && R == 16) || (dh == 16 && R == 16); }

size_t attn_bwd_bf16_image_bytes(int B, int H, int W, int heads, int ws) {
  const size_t units = (size_t)B * ((H + ws - 1) / ws) * ((W + ws - 1) / ws) * heads;
  return units * (size_t)bwd_tiles_per_unit(ws) * 10 * 1024;
}

hipError_t launch_attn_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  if (a.dh == 30 && a.R == 16) return launch_variant<30, 16>(a, stream);
  if (a.dh == 16 && a.R == 16) return launch_variant<16, 16>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace rib
