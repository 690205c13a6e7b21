// attn_bf16.hip -- bf16 MFMA RIB window attention with the CLA gate (gfx950).
//
// Per image, window and head ("Rank-Factorized Implicit Neural Bias",
// gist.science summaries part A mechanism steps 3-4 and part B; omica.com.cn
// explainer sections 2.2 "attention rewrite" and 2.3):
//   Q~ = [Qp/sqrt(R), Qc/sqrt(dh)],  K~ = [Kp, Kc]
//   S  = Q~ K~^T  (content score + positional bias in one contraction)
//   O  = (softmax(S) V) * sigmoid(G)
// (The pages concatenate content first; the column order of a contraction does
// not change its value, and positional-first keeps the LDS rows aligned.)
//
// Three kernels: the whole-window kernel (windows of up to 256 tokens), the
// chunked kernel (larger windows; both below) and the tiled kernel, whose
// design follows (it takes the head shapes whose chunked kernel spills
// registers, and the fused LayerNorm + Q projection).  Most points below hold
// for all three; the ping-pong is the tiled kernel's own.
//
// Tiled kernel (one workgroup = 8 waves = 512 queries of one (image, window, head)):
//
//  * Scores are computed transposed, S^T = K~ Q~^T, with
//    v_mfma_f32_32x32x16_bf16: K~ rows are the A operand (read from LDS), the
//    wave's 64 queries are the B operand (kept in VGPRs for the whole loop).
//    In the 32x32 accumulator each lane then owns ONE query and 16 of the 32
//    keys of a block, so softmax row statistics are in-lane plus one
//    v_permlane32_swap.
//  * The same accumulator registers, rounded to bf16, are exactly the B
//    operand of O^T = V^T P^T.  V stays token-major in LDS; the A operand
//    (8 keys of one channel per lane) is assembled with ds_read_b64_tr_b16,
//    whose 16-lane transpose is addressed so that the keys come out in the
//    accumulator's row order.  P never leaves registers.
//  * Softmax runs in base 2 (log2 e folded into the query scales).  Two spare
//    contraction columns carry the running maximum: column "m" holds -m_hat
//    in Q~ (a bf16 value) against 1 in K~, column "o" holds -OFF against 1
//    (2^14 for padded keys, which masks them; those have 0 in column m).  The
//    MFMA returns t = s*log2(e) - m_hat - OFF and the fast path is p = exp2(t).
//  * P is packed to bf16 by truncation with one v_perm_b32 per pair; the same
//    P feeds PV and the row sum, so O = PV / l sees a consistent set of
//    weights and the truncation's bias cancels (its spread is that of
//    rounding; the rounding convert costs the same).
//  * Rescaling is lazy: p <= 2^-OFF * 2^(growth of the maximum).  The packed
//    bf16 P values are OR-reduced; bit 14 of a half is set iff p >= 2, i.e.
//    the maximum grew by more than OFF+1 = 8 (a factor 256).  Only then (and on
//    the first tile) does the wave take the slow path: exact row maximum, new
//    m_hat rounded to bf16, recompute, rescale O.
//  * The row sum l comes for free from the PV MFMA: V channel dh is all ones
//    (a head of 32 channels, which has no spare channel, sums P with v_dot2).
//  * Ping-pong over key tiles of KT = 64.  A workgroup has 8 waves, two per
//    SIMD, in two groups (waves 0-3 and 4-7) that run half a step apart and
//    swap roles at every barrier: while one group runs its MFMA phase
//    (operand reads, its share of staging the next tiles into LDS, QK^T of
//    tile t and PV of tile t-1: 20 MFMAs per wave), the wave of the other
//    group on the same SIMD runs its softmax phase (exp2, packing and
//    overflow check of tile t, and the next tile's K~ operand reads).  The
//    matrix core thus runs while the other wave's exponentials, which hold
//    the SIMD's vector issue for about 8 cycles each, go through.  Three LDS
//    stages; tile loads are issued a full step before they are stored.
//  * Window partitioning is index arithmetic on the NHWC arrays: a window's
//    real tokens are enumerated row-major, r = iy*nx + ix, so padded positions
//    are never loaded, and only the last tile can hold padded keys.
//  * Workgroups are numbered so that the q-blocks of one (image, window, head)
//    run on one XCD (shared K/V in that XCD's L2) and the window units are
//    dealt round-robin over the XCDs (edge windows spread evenly).
#include "rib_device.hpp"
#include "rib_launch.hpp"

namespace rib {

namespace {

constexpr int KT = 64;             // keys per tile
constexpr int NWAVE = 8;           // waves per workgroup (two groups of four)
constexpr int QW = 64;             // queries per wave (two 32-query MFMA blocks)
constexpr int QB = QW * NWAVE;     // queries per workgroup
constexpr int NSTAGE = 3;          // LDS stages of the key-tile pipeline
constexpr float OFF = 7.0f;        // p = exp2(s - m_hat - OFF) <= 2^-OFF normally
constexpr float OFF_FAST = 64.0f;  // offset of the unchecked first pass (whole-window and chunked kernels)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr uint32_t RSRC_WORD3 = 0x00020000u;  // gfx9 raw buffer: 32-bit data format

template <int DH, int R>
struct Shape {
  static_assert(DH % 2 == 0 && R % 8 == 0, "head dim must be even, rank a multiple of 8");
  static constexpr int KC = (R + DH + 2 + 15) / 16;  // 16-wide contraction chunks
  // The row sum l rides along the PV product as V channel DH (all ones) when the
  // last 32-channel output tile has room for it; a head of 32 channels would
  // need a whole second tile for it, so there l is summed from P with v_dot2.
  static constexpr bool ONES = DH % 32 != 0;
  static constexpr int DT = (DH + (ONES ? 1 : 0) + 31) / 32;  // 32-channel output tiles
  static constexpr int ROWDW = 8 * KC;               // dwords per Q~/K~ row
  static constexpr int KCH = 2 * KC;                 // 16-byte chunks per K~ row
  static constexpr int KSTR = ROWDW + 4;             // row stride of the Q~ staging rows (bank spread)
  static constexpr int CONSTDW = R / 2 + DH / 2;     // dword with columns (m, o)
  static constexpr int CM = CONSTDW / 8;             // chunk holding it
  static constexpr int GM = (CONSTDW % 8) / 4;       // lane half holding it
  static constexpr int DM = CONSTDW % 4;             // dword inside the 16-byte operand
  static constexpr int VSTR = 16 * DT;               // dwords of V per key
  static constexpr int KS_DW = KT * ROWDW;           // K~ tile, chunk-major: [chunk][key][4 dwords]
  static constexpr int VS_DW = KT * VSTR;            // V tile, swizzled for the transposing reads
  static constexpr int STAGE_DW = KS_DW + VS_DW;
  static constexpr int QS_DW = QB * KSTR;
  static constexpr int LDS_DW = (NSTAGE * STAGE_DW > QS_DW) ? NSTAGE * STAGE_DW : QS_DW;
  // accumulator position of the row sum (V channel DH)
  static constexpr int LT = DH / 32;
  static constexpr int LW = DH % 32;
  static constexpr int LR = 4 * (LW / 8) + (LW % 4);
  static constexpr int LG = (LW / 4) % 2;
  static_assert(KC <= 4 && DT <= 2 && DH <= 32 && R <= 32, "variant too large");
  static_assert(!(R > 16 && DT > 1), "wave 3 stages either Kp[16..32) or the second V tile");
};

// A window spans wt frames x ws rows x ws columns of a [B][T][H][W][C] map
// (T = wt = 1 for images); its real tokens are enumerated frame-major, then
// row-major: r = (it*ny + iy)*nx + ix with ny, nx the window's real rows and
// columns.  In-window index n = (it*ws + iy)*ws + ix.
struct Geo {
  int T, H, W, C, wt, ws, b, tw, wy, wx, h, ny, nx, n_real;
  float inv_nx, inv_ny;
};

// real index r of a window -> element offset of the token's head slice and
// in-window index n
template <int DH>
__device__ __forceinline__ void locate(const Geo& G, int r, int& off, int& n) {
  const int rr = (int)(((float)r + 0.5f) * G.inv_nx);  // real row, frame-major
  const int ix = r - rr * G.nx;
  const int it = (int)(((float)rr + 0.5f) * G.inv_ny);
  const int iy = rr - it * G.ny;
  off = (((G.b * G.T + G.tw * G.wt + it) * G.H + G.wy * G.ws + iy) * G.W + G.wx * G.ws + ix) * G.C + G.h * DH;
  n = (it * G.ws + iy) * G.ws + ix;
}

// window decode of a logical unit u = (((b*nWt + tw)*nWy + wy)*nWx + wx)*heads + h
template <int DH>
__device__ __forceinline__ void decode_window(Geo& G, int u, int T, int H, int W, int heads, int wt, int ws) {
  const int nWy = (H + ws - 1) / ws, nWx = (W + ws - 1) / ws, nWt = (T + wt - 1) / wt;
  G.h = u % heads; u /= heads;
  G.wx = u % nWx; u /= nWx;
  G.wy = u % nWy; u /= nWy;
  G.tw = u % nWt;
  G.b = u / nWt;
  G.T = T; G.H = H; G.W = W; G.C = heads * DH; G.wt = wt; G.ws = ws;
  G.nx = min(ws, W - G.wx * ws);
  G.ny = min(ws, H - G.wy * ws);
  G.n_real = min(wt, T - G.tw * wt) * G.ny * G.nx;
  G.inv_nx = 1.0f / (float)G.nx;
  G.inv_ny = 1.0f / (float)G.ny;
}

// ---- LDS layouts of a key tile ----------------------------------------------
// K~: chunk-major, 16-byte chunk c of key j at dword (c*KT + j)*4.  The A
// operand of chunk c for 32 keys is then 512 contiguous bytes per lane half,
// and a staging write of one chunk for 64 keys is 1 KB contiguous.
__device__ __forceinline__ int kchunk_dw(int c, int j) { return (c * KT + j) * 4; }
// V: 8-byte pieces (4 channels) of 4 consecutive keys and one 16-channel half
// form a 128-byte block; piece (key, ch) sits at 8-byte index
//   ((key/4) * 2DT + ch/16) * 16 + (key%4) * 4 + (ch%16)/4,
// so each 16-lane group of a transposing read covers one contiguous block.
template <int DT>
__device__ __forceinline__ int vpiece_dw(int key, int ch) {
  return 2 * ((((key >> 2) * (2 * DT) + (ch >> 4)) << 4) + ((key & 3) << 2) + ((ch & 15) >> 2));
}

// ---- staging of one key tile ------------------------------------------------
// Each wave loads two 16-byte chunks per lane (lane = key) and tile with the
// same code; only the wave-uniform buffer descriptor and offset differ:
//   wave 0 / 1: Kp[n][0..8) / Kp[n][8..16)  (fp32)      waves 6 / 7: Kp[n][16..32) when R = 32
//   wave 2 / 3: Kc dwords [0, 8) / [8, 16)   (bf16)
//   wave 4 / 5: V  dwords [0, 8) / [8, 16)   (bf16)
// A wave without a load role gets a zero-length descriptor (its loads return
// zeros and touch no memory).  Buffer loads are bounds-checked by the
// hardware, so the last head slice of the map may over-read its last chunk.
// At the store each role converts its chunks into its part of the LDS rows:
// K~ row = [bf16 Kp (R/2 dwords) | Kc (dh/2) | (m, o) column pair | zeros],
// V row = [V (dh/2 dwords), ones pair (1, 0) at channel dh, zeros].
struct Stage {
  u32x4_t raw[2];
};

template <int DH, int R>
struct Roles {
  static constexpr bool KP1 = R >= 16;           // wave 1 loads Kp[8..16)
  static constexpr bool KP67 = R == 32;          // waves 6/7 load Kp[16..32)
  static constexpr bool KC1 = DH / 2 > 8;        // wave 3 loads Kc dwords [8, 16)
  static constexpr bool V1 = DH / 2 > 8;         // wave 5 loads V dwords [8, 16)
  static constexpr int KCREG = Shape<DH, R>::ROWDW - R / 2;  // dwords of the K~ row after Kp
  // every K~ part is staged by waves 0-3: the K~ operands of the next tile can
  // then be read during the softmax phase (see the main loop)
  static constexpr bool KPREF = !KP67 && KCREG <= 16;
};

// Per-lane position of the key this lane loads, advanced by KT keys per tile
// without divisions: (ix, column of the window) and the byte offset of the
// lane's chunks in this wave's source buffer.  Offsets of lanes past the last
// real key run on beyond the window; those keys are masked at the store and
// reads past the buffer end return zeros (bounds-checked buffer loads).
struct Cursor {
  int ix, iy;  // column, and row within the frame, of the lane's key
  unsigned voff;
};

struct CursorStep {
  unsigned col;    // bytes per window column (uniform)
  unsigned wrap;   // bytes from the end of one window row to the start of the next (uniform)
  unsigned fskip;  // bytes from past the window's last row of a frame to its first row of the next
};

__device__ __forceinline__ void cursor_advance(Cursor& c, const CursorStep& cs, int nx, int ny) {
  c.ix += KT;
  c.voff += KT * cs.col;
  while (c.ix >= nx) {
    c.ix -= nx;
    c.voff += cs.wrap;
    if (++c.iy == ny) {
      c.iy = 0;
      c.voff += cs.fskip;
    }
  }
}

__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t rsrc, const Cursor& c, Stage& st) {
  st.raw[0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, c.voff, 0, 0));
  st.raw[1] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, c.voff + 16u, 0, 0));
}

// Kp fp32 chunks (8 floats) -> 4 packed bf16 dwords
__device__ __forceinline__ u32x4_t kp_to_bf16(const u32x4_t& x, const u32x4_t& y, bool real) {
  const f32x4_t a = __builtin_bit_cast(f32x4_t, x);
  const f32x4_t b = __builtin_bit_cast(f32x4_t, y);
  const u32x4_t out = {pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]), pack_bf16(b[0], b[1]), pack_bf16(b[2], b[3])};
  return real ? out : (u32x4_t){0u, 0u, 0u, 0u};
}

// dword w of the K~ row region after Kp: content, the (m, o) pair, or zero
template <int DH>
__device__ __forceinline__ uint32_t kc_word(int w, uint32_t data, bool real) {
  if (w < DH / 2) return real ? data : 0u;
  if (w == DH / 2) return real ? 0x3F803F80u : 0x46800000u;  // (1,1) real, (0,2^14) padded
  return 0u;
}
// dword w of the V row: value, the ones pair at channel DH (when the tile has
// room for it), or zero
template <int DH>
__device__ __forceinline__ uint32_t v_word(int w, uint32_t data, bool real) {
  uint32_t val = w < DH / 2 ? data : (w == DH / 2 && DH % 32 != 0 ? 0x00003F80u : 0u);
  return real ? val : 0u;
}

// MASK: the tile may hold padded keys (only the last tile of a window can)
template <int DH, int R, bool MASK>
__device__ __forceinline__ void store_tile(uint32_t* stage, int wave, int j, bool real_key, const Stage& st) {
  using S = Shape<DH, R>;
  using RL = Roles<DH, R>;
  const bool real = MASK ? real_key : true;
  uint32_t* vs = stage + S::KS_DW;
  // dword w (a multiple of 4) of key j's K~ row
  auto kdst = [&](int w) { return reinterpret_cast<u32x4_t*>(stage + kchunk_dw(w >> 2, j)); };
  // V channels [ch, ch+8) of key j (ch a multiple of 8)
  auto vdst = [&](int ch) { return reinterpret_cast<u32x4_t*>(vs + vpiece_dw<S::DT>(j, ch)); };
  if (wave == 0 || (wave == 1 && RL::KP1) || (wave >= 6 && RL::KP67)) {
    const int q = wave >= 6 ? wave - 4 : wave;  // which 8-float group of Kp
    *kdst(4 * q) = kp_to_bf16(st.raw[0], st.raw[1], real);
  }
  if (wave == 2 || wave == 3) {
    const int w0 = wave == 2 ? 0 : 8;
    if (w0 < RL::KCREG) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (w0 + 4 * i >= RL::KCREG) break;
        uint32_t d[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e] = kc_word<DH>(w0 + 4 * i + e, st.raw[i][e], real);
        *kdst(R / 2 + w0 + 4 * i) = (u32x4_t){d[0], d[1], d[2], d[3]};
      }
    }
  }
  if constexpr (RL::KCREG > 16) {
    // the K~ row continues past 16 dwords after Kp: (m, o) pair and zeros only
    if (wave == 7) {
#pragma unroll
      for (int i = 0; i < (RL::KCREG - 16) / 4; ++i) {
        uint32_t d[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e] = kc_word<DH>(16 + 4 * i + e, 0u, real);
        *kdst(R / 2 + 16 + 4 * i) = (u32x4_t){d[0], d[1], d[2], d[3]};
      }
    }
  }
  if (wave == 4 || wave == 5) {
    const int w0 = wave == 4 ? 0 : 8;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      uint32_t d[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) d[e] = v_word<DH>(w0 + 4 * i + e, st.raw[i][e], real);
      *vdst(2 * (w0 + 4 * i)) = (u32x4_t){d[0], d[1], d[2], d[3]};
    }
  }
  if constexpr (S::DT > 1) {
    // V channels [32, 64): the ones pair (dh = 32) and zeros
    if (wave == 6) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t d[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e] = v_word<DH>(16 + 4 * i + e, 0u, real);
        *vdst(32 + 8 * i) = (u32x4_t){d[0], d[1], d[2], d[3]};
      }
    }
  }
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// 4 bf16 of the transposing LDS read (16-lane groups: output lane i, element k
// comes from input lane 4k + i/4, element i%4)
__device__ __forceinline__ u32x2_t ds_read_tr16(const uint32_t* p) {
  const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4_t*)(__attribute__((address_space(3))) void*)(const_cast<uint32_t*>(p)));
  return __builtin_bit_cast(u32x2_t, r);
}

// per-wave state of NQ 32-query blocks
template <int DH, int R, int NQ = 2>
struct Regs {
  using S = Shape<DH, R>;
  f32x16_t O[NQ][S::DT];
  u32x4_t qt[NQ][S::KC];
  float mhat[NQ];
  float lpart[NQ];  // this lane's share of l (only when l is not a V channel)
};

// l of the lane's query of block qb: the ones channel of the PV product, or
// the two lane halves' partial sums
template <int DH, int R, int NQ>
__device__ __forceinline__ float row_sum(const Regs<DH, R, NQ>& rg, int qb) {
  using S = Shape<DH, R>;
  if constexpr (S::ONES) {
    const LanePair pr = lane_pair(rg.O[qb][S::LT][S::LR]);
    return S::LG ? pr.hi : pr.lo;
  } else {
    const LanePair pr = lane_pair(rg.lpart[qb]);
    return pr.lo + pr.hi;
  }
}

// Operands of one MFMA phase, all read from LDS before the first MFMA issues:
// the K~ rows of the tile being scored (A operand of S^T = K~ Q~^T) and the
// transposed V of the tile being accumulated (A operand of O^T = V^T P^T).
template <int DH, int R>
struct PhaseOps {
  u32x4_t ka[2][Shape<DH, R>::KC];
  u32x4_t va[2][2][Shape<DH, R>::DT];
};

// Keeps an LDS dword index in a register as computed: every read of a phase
// then addresses base + immediate offset, instead of the compiler hoisting one
// address register per read out of the loop.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// K~ operands of one tile; kst = dword index of the stage's K~ block
template <int DH, int R>
__device__ __forceinline__ void read_k_ops(const uint32_t* lds, int kst, int l32, int gh, PhaseOps<DH, R>& ops) {
  using S = Shape<DH, R>;
  const uint32_t* base = lds + opaque(kchunk_dw(gh, l32)) + kst;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int c = 0; c < S::KC; ++c)
      ops.ka[kb][c] = *reinterpret_cast<const u32x4_t*>(base + kchunk_dw(2 * c, kb * 32));
}

// S^T = K~ Q~^T for 64 keys x the wave's 32 NQ queries
template <int DH, int R, int NQ>
__device__ __forceinline__ void qk_tile(const PhaseOps<DH, R>& ops, const Regs<DH, R, NQ>& rg,
                                        f32x16_t (&Sacc)[NQ][2]) {
  using S = Shape<DH, R>;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int qb = 0; qb < NQ; ++qb) {
      f32x16_t acc;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
      for (int c = 0; c < S::KC; ++c)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ops.ka[kb][c]),
                                                      __builtin_bit_cast(bf16x8_t, rg.qt[qb][c]), acc, 0, 0, 0);
      Sacc[qb][kb] = acc;
    }
}

// p = exp2(t - shift) packed to bf16 pairs (truncated: P feeds both the PV
// product and, through the ones channel of V, the row sum, so the rounding of
// P cancels in O = PV / l); returns the OR of all packed words
template <int NQ>
__device__ __forceinline__ uint32_t exp_tile(const f32x16_t (&Sacc)[NQ][2], uint32_t (&P)[NQ][2][8],
                                             const float (&shift)[NQ]) {
  uint32_t orv = 0;
#pragma unroll
  for (int qb = 0; qb < NQ; ++qb) {
    const float sh = shift[qb];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        P[qb][kb][i] = pack_bf16_trunc(__builtin_amdgcn_exp2f(Sacc[qb][kb][2 * i] - sh),
                                       __builtin_amdgcn_exp2f(Sacc[qb][kb][2 * i + 1] - sh));
        orv |= P[qb][kb][i];
      }
  }
  return orv;
}

// fast-path exponentials (no shift)
template <int NQ>
__device__ __forceinline__ uint32_t exp_tile_fast(const f32x16_t (&Sacc)[NQ][2], uint32_t (&P)[NQ][2][8]) {
  uint32_t orv = 0;
#pragma unroll
  for (int qb = 0; qb < NQ; ++qb)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        P[qb][kb][i] = pack_bf16_trunc(__builtin_amdgcn_exp2f(Sacc[qb][kb][2 * i]),
                                       __builtin_amdgcn_exp2f(Sacc[qb][kb][2 * i + 1]));
        orv |= P[qb][kb][i];
      }
  return orv;
}

// Slow path for the tile whose scores are in Sacc: exact row maximum, new
// reference m_hat (rounded to bf16), exponentials again, rescale of O
// (unless this is the first tile) and the new -m_hat in the Q~ operand.
template <int DH, int R, int NQ>
__device__ __forceinline__ void rescale_tile(Regs<DH, R, NQ>& rg, const f32x16_t (&Sacc)[NQ][2],
                                             uint32_t (&P)[NQ][2][8], bool first, int gh, float off = OFF) {
  using S = Shape<DH, R>;
  float shift[NQ];
#pragma unroll
  for (int qb = 0; qb < NQ; ++qb) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, Sacc[qb][kb][e]);
    const LanePair pr = lane_pair(mx);
    mx = fmaxf(pr.lo, pr.hi);
    const bool grow = first || (mx + off > 0.0f);
    const float mnew = grow ? round_bf16(rg.mhat[qb] + mx + off) : rg.mhat[qb];
    shift[qb] = mnew - rg.mhat[qb];
    rg.mhat[qb] = mnew;
    if (!first) {
      const float sc = __builtin_amdgcn_exp2f(-shift[qb]);
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) rg.O[qb][dt][e] *= sc;
      if constexpr (!S::ONES) rg.lpart[qb] *= sc;
    }
    const uint32_t cd = pack_bf16(-mnew, -off);
    if (gh == S::GM) rg.qt[qb][S::CM][S::DM] = cd;
  }
  exp_tile(Sacc, P, shift);
}

// transposed V operands of one tile (see pv_tile); vst = dword index of the
// stage's V block
template <int DH, int R>
__device__ __forceinline__ void read_v_ops(const uint32_t* lds, int vst, int lane, PhaseOps<DH, R>& ops) {
  using S = Shape<DH, R>;
  // transposing read: 16-lane group q = lane/16 covers channels 16*(q%2) + i of the
  // 32-channel tile for keys 4g + k (g = q/2); input lane j = 4k + m addresses
  // channels 16*(q%2) + 4m .. +3 of key 4g + k (+8 for the second read).
  // Keys kb*32 + 16*c2 (+8) and channel tiles dt shift the address by constants.
  const int j = lane & 15, q = lane >> 4;
  const int key0 = 4 * (q >> 1) + (j >> 2);
  const int ch0 = 16 * (q & 1) + 4 * (j & 3);
  const uint32_t* base = lds + opaque(vpiece_dw<S::DT>(key0, ch0)) + vst;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt) {
        const int kofs = kb * 32 + 16 * c2;
        const u32x2_t lo = ds_read_tr16(base + vpiece_dw<S::DT>(kofs, dt * 32));
        const u32x2_t hi = ds_read_tr16(base + vpiece_dw<S::DT>(kofs + 8, dt * 32));
        ops.va[kb][c2][dt] = (u32x4_t){lo[0], lo[1], hi[0], hi[1]};
      }
}

// Byte offsets in a staging array of this lane's K~ and V operand reads,
// carried from key tile to key tile of a run of consecutive tiles (stride
// `tile` dwords): each read addresses the carried register plus an immediate
// offset, and the next tile costs one add per array.  The carried values pass
// through opaque() in place, so that the compiler keeps one register instead
// of one hoisted address per read.
template <int DH, int R>
struct OpsWalk {
  int kb, vb;
  __device__ __forceinline__ OpsWalk(int l32, int gh, int lane, int kst, int vst) {
    using S = Shape<DH, R>;
    const int j = lane & 15, q = lane >> 4;
    kb = 4 * (kst + kchunk_dw(gh, l32));
    vb = 4 * (vst + vpiece_dw<S::DT>(4 * (q >> 1) + (j >> 2), 16 * (q & 1) + 4 * (j & 3)));
  }
  // operands of the current tile, then advance by `tile` dwords
  __device__ __forceinline__ void read(const uint32_t* lds, int tile, PhaseOps<DH, R>& ops) {
    using S = Shape<DH, R>;
    kb = opaque(kb);
    vb = opaque(vb);
    const uint32_t* kbase = reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(lds) + kb);
    const uint32_t* vbase = reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(lds) + vb);
#pragma unroll
    for (int kblk = 0; kblk < 2; ++kblk)
#pragma unroll
      for (int c = 0; c < S::KC; ++c)
        ops.ka[kblk][c] = *reinterpret_cast<const u32x4_t*>(kbase + kchunk_dw(2 * c, kblk * 32));
#pragma unroll
    for (int kblk = 0; kblk < 2; ++kblk)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt) {
          const int kofs = kblk * 32 + 16 * c2;
          const u32x2_t lo = ds_read_tr16(vbase + vpiece_dw<S::DT>(kofs, dt * 32));
          const u32x2_t hi = ds_read_tr16(vbase + vpiece_dw<S::DT>(kofs + 8, dt * 32));
          ops.va[kblk][c2][dt] = (u32x4_t){lo[0], lo[1], hi[0], hi[1]};
        }
    kb += 4 * tile;
    vb += 4 * tile;
  }
};

// O^T += V^T P^T (and, without a ones channel, l += the lane's p values)
template <int DH, int R, int NQ>
__device__ __forceinline__ void pv_tile(const PhaseOps<DH, R>& ops, Regs<DH, R, NQ>& rg, const uint32_t (&P)[NQ][2][8]) {
  using S = Shape<DH, R>;
  if constexpr (!S::ONES) {
#pragma unroll
    for (int qb = 0; qb < NQ; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          rg.lpart[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, P[qb][kb][i]),
                                                         __builtin_bit_cast(bf16x2_t, 0x3F803F80u), rg.lpart[qb], false);
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int qb = 0; qb < NQ; ++qb) {
        const u32x4_t pb = {P[qb][kb][4 * c2], P[qb][kb][4 * c2 + 1], P[qb][kb][4 * c2 + 2], P[qb][kb][4 * c2 + 3]};
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt)
          rg.O[qb][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ops.va[kb][c2][dt]),
                                                                 __builtin_bit_cast(bf16x8_t, pb), rg.O[qb][dt], 0, 0, 0);
      }
}

// ---- LayerNorm and the Q projection inside the tiled kernel's Q~ build ---------
// (omica.com.cn explainer section 3.1: LayerNorm, then the attention's Q/K/V
// projection).  For its 512 queries and head h a workgroup computes, per query token,
//   xn = (x - mu) / sqrt(var + eps) * gamma + beta   (biased variance, fp32)
//   q  = bf16(xn W_q[:, h dh .. h dh + dh) + bias_q)
// with the affine part folded into the weights, so that the raw bf16 x goes into
// the matrix core as it is:
//   q_d = inv * (sum_c x_c W'_cd - mu * sum_c W'_cd) + b'_d,
//   W'_cd = bf16(gamma_c W_cd),  b'_d = bias_d + sum_c beta_c W_cd,  inv = 1/sqrt(var + eps).
// W'^T (dh rows, padded to 32), its row sums and b' are built in LDS once per
// workgroup from coalesced reads of W; the product x W' runs as q^T = W'^T x^T on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  mu and var come from fp32 sums
// of x and x^2 (v_dot2_f32_bf16: the products of bf16 values are exact), with
// var = E[x^2] - mu^2 -- a quarter of the vector work of a second pass over
// (x - mu), which a 16-lane SIMD pays four cycles per wave64 instruction for.  Rounding: W' is rounded once,
// x is exact, and the subtraction of mu * sum_c W'_cd cancels the token offset in
// fp32; rib_ln_qkv instead rounds xn before its product, so the two paths' q may
// differ by about one bf16 unit.
struct LnqArgs {
  const uint32_t* x;   // block input, [B][T][H][W][C] bf16
  const float* gamma;  // [C]
  const float* beta;   // [C]
  const float* w;      // [C][3C], columns Q | K | V (only Q is read)
  const float* bias;   // [3C]
  float eps;
};
constexpr int LNQ_CP = 192;              // channels of the contraction (C <= 192, zero padded)
constexpr int LNQ_WST = LNQ_CP / 2 + 4;  // dwords per staged W'^T row (16-byte pad)
constexpr int LNQ_NG = 16;               // channel groups of the staging (512 threads = 16 x 32)
// LDS of the fused prologue after the Q~ rows: W'^T rows, then per-group partial
// sums (row sum of W', beta W) and the final (sum_c W'_cd, b'_d) pairs
constexpr int LNQ_DW = 32 * LNQ_WST + LNQ_NG * 64 + 64;

// thread (d = tid & 31, group tid >> 5) handles channel pairs c = 2 (group + 16 i)
template <int DH>
__device__ __forceinline__ void lnq_stage_w(uint32_t* wt, const LnqArgs& L, int C, int h) {
  const int d = threadIdx.x & 31, grp = threadIdx.x >> 5;
  const int oc = h * DH + d;
  const long C3 = 3L * C;
  float cs = 0.0f, bb = 0.0f;
#pragma unroll
  for (int cp = grp; cp < LNQ_CP / 2; cp += LNQ_NG) {
    const int c = 2 * cp;
    float a = 0.0f, b = 0.0f;
    if (d < DH && c < C) {
      const float w0 = L.w[c * C3 + oc];
      a = round_bf16(w0 * L.gamma[c]);
      bb = fmaf(L.beta[c], w0, bb);
      if (c + 1 < C) {
        const float w1 = L.w[(c + 1) * C3 + oc];
        b = round_bf16(w1 * L.gamma[c + 1]);
        bb = fmaf(L.beta[c + 1], w1, bb);
      }
    }
    cs += a + b;
    wt[d * LNQ_WST + cp] = pack_bf16(a, b);
  }
  float* part = reinterpret_cast<float*>(wt + 32 * LNQ_WST);
  part[grp * 64 + d] = cs;
  part[grp * 64 + 32 + d] = bb;
}

// after a barrier: threads 0..31 sum the groups' partials into (sum_c W'_cd, b'_d)
template <int DH>
__device__ __forceinline__ void lnq_reduce(uint32_t* wt, const LnqArgs& L, int h) {
  const int d = threadIdx.x;
  if (d >= 32) return;
  const float* part = reinterpret_cast<const float*>(wt + 32 * LNQ_WST);
  float cs = 0.0f, bb = 0.0f;
#pragma unroll
  for (int g = 0; g < LNQ_NG; ++g) {
    cs += part[g * 64 + d];
    bb += part[g * 64 + 32 + d];
  }
  float* fin = reinterpret_cast<float*>(wt + 32 * LNQ_WST + LNQ_NG * 64);
  fin[2 * d] = cs;
  fin[2 * d + 1] = d < DH ? bb + L.bias[h * DH + d] : 0.0f;
}

// Qc of the lane's query (block qb of this wave) into its Q~ row in LDS: dwords
// R/2 + 4i + 2gh (+1) hold channels 8i + 4gh .. +3 (those below DH)
constexpr int LNQ_KS = LNQ_CP / 16;  // 16-channel steps of the contraction

// the lane's channels 16s + 8gh .. +7 of its token (s < ceil(C / 16); the words
// past C are cleared by lnq_block)
__device__ __forceinline__ void lnq_load(u32x4_t (&xw)[LNQ_KS], __amdgpu_buffer_rsrc_t rx, int tok_off, int C, int gh) {
#pragma unroll
  for (int s = 0; s < LNQ_KS; ++s) {
    const int c0 = 16 * s + 8 * gh;
    xw[s] = (u32x4_t){0u, 0u, 0u, 0u};
    if (c0 < C) xw[s] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rx, 2u * (unsigned)(tok_off + c0), 0, 0));
  }
}

template <int DH, int R>
__device__ __forceinline__ void lnq_block(uint32_t* rows, const uint32_t* wt, const LnqArgs& L, u32x4_t (&xw)[LNQ_KS],
                                          bool real, int row, int C, int l32, int gh, float sc) {
  using S = Shape<DH, R>;
  constexpr int KS = LNQ_KS;
  const int ks = (C + 15) >> 4;  // 16-channel steps that hold channels
  // clear the words past C (C is even, so words are whole; only the last step holds any)
#pragma unroll
  for (int s = 0; s < KS; ++s)
    if (16 * s + 16 > C) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (16 * s + 8 * gh + 2 * e >= C) xw[s][e] = 0u;
    }
  f32x16_t acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
  for (int s = 0; s < KS; ++s)
    if (s < ks) {
      const u32x4_t wa = *reinterpret_cast<const u32x4_t*>(wt + l32 * LNQ_WST + 8 * s + 4 * gh);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, wa), __builtin_bit_cast(bf16x8_t, xw[s]),
                                                    acc, 0, 0, 0);
    }
  // token statistics: sum x and sum x^2 as bf16 pair dot products (the products are
  // exact in fp32), over the lane pair's channels; var = E[x^2] - mu^2
  float sum = 0.0f, sq = 0.0f;
  const bf16x2_t one = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
#pragma unroll
  for (int s = 0; s < KS; ++s)
    if (s < ks) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // through a scalar: hipcc lowers a bit_cast of an ext_vector element
        // (xw[s][e] directly) to element 0 for every e
        const uint32_t word = xw[s][e];
        const bf16x2_t xv = __builtin_bit_cast(bf16x2_t, word);
        sum = __builtin_amdgcn_fdot2_f32_bf16(xv, one, sum, false);
        sq = __builtin_amdgcn_fdot2_f32_bf16(xv, xv, sq, false);
      }
    }
  {
    const LanePair ps = lane_pair(sum), pq = lane_pair(sq);
    sum = ps.lo + ps.hi;
    sq = pq.lo + pq.hi;
  }
  const float mu = sum / (float)C;
  sq = fmaxf(sq / (float)C - mu * mu, 0.0f);
  const float inv = 1.0f / sqrtf(sq + L.eps);
  if (!real) return;  // padded query rows keep their zeros
  const float* fin = reinterpret_cast<const float*>(wt + 32 * LNQ_WST + LNQ_NG * 64);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      const int d = 8 * i + 4 * gh + 2 * jp;
      if (d < DH) {
        const float4 f = *reinterpret_cast<const float4*>(fin + 2 * d);  // (sum W', b') of d, d + 1
        const float q0 = round_bf16(fmaf(inv, acc[4 * i + 2 * jp] - mu * f.x, f.y));
        const float q1 = round_bf16(fmaf(inv, acc[4 * i + 2 * jp + 1] - mu * f.z, f.w));
        rows[row * S::KSTR + R / 2 + d / 2] = pack_bf16(q0 * sc, q1 * sc);
      }
    }
}

// One workgroup of the tiled kernel: logical = (window unit) * qblocks + query block.
// FUSEQ: Qc is computed from the block input (LnqArgs) instead of read from qc.
template <int DH, int R, bool FUSEQ = false>
__device__ __forceinline__ void attn_tiled_body(const uint32_t* __restrict__ qc, const uint32_t* __restrict__ kc,
                 const uint32_t* __restrict__ v, const uint32_t* __restrict__ g,
                 const float* __restrict__ qp, const float* __restrict__ kp,
                 uint32_t* __restrict__ o, int B, int T, int H, int W, int heads, int wt, int ws, int total,
                 long tstride, float* __restrict__ lse, int logical, const LnqArgs* lnq = nullptr) {
  using S = Shape<DH, R>;
  constexpr int LDS_N = FUSEQ && S::QS_DW + LNQ_DW > S::LDS_DW ? S::QS_DW + LNQ_DW : S::LDS_DW;
  __shared__ __attribute__((aligned(16))) uint32_t lds[LDS_N];

  if (logical >= total) return;
  const int NW = wt * ws * ws;  // tokens of a full window
  const int qblocks = (NW + QB - 1) / QB;
  Geo G;
  int q0;
  {
    decode_window<DH>(G, logical / qblocks, T, H, W, heads, wt, ws);
    q0 = (logical % qblocks) * QB;
    if (q0 >= G.n_real) return;
  }
  qp += (long)G.h * tstride;  // per-head positional tables (tstride 0: one shared pair)
  kp += (long)G.h * tstride;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int gh = lane >> 5;  // lane half

  // ---- prologue: build the workgroup's Q~ rows in LDS, then pick up the B operands
  const unsigned map_bytes = (unsigned)(B * T * H * W * heads * DH) * 2u;
  {
    const int r = q0 + tid;
    const bool real = r < G.n_real;
    int off, n;
    locate<DH>(G, real ? r : G.n_real - 1, off, n);
    const float sp = LOG2E / sqrtf((float)R);
    const float sc = LOG2E / sqrtf((float)DH);
    // the row's R Qp floats and DH/2 Qc dwords in 16-byte buffer loads (bounds-checked: the
    // last load of a head slice may read into the next slice, whose dwords are not used)
    constexpr int NQP = R / 4, NQC = (DH / 2 + 3) / 4;
    const __amdgpu_buffer_rsrc_t rqp = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(qp), (short)0, (int)((unsigned)(wt * ws * ws * R) * 4u), (int)RSRC_WORD3);
    const __amdgpu_buffer_rsrc_t rqc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qc), (short)0, (int)map_bytes, (int)RSRC_WORD3);
    u32x4_t xp[NQP], xc[NQC];
#pragma unroll
    for (int k = 0; k < NQP; ++k)
      xp[k] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rqp, (unsigned)(n * R + 4 * k) * 4u, 0, 0));
#pragma unroll
    for (int k = 0; k < NQC; ++k)
      xc[k] = FUSEQ ? (u32x4_t){0u, 0u, 0u, 0u}
                    : __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rqc, 2u * (unsigned)off + 16u * k, 0, 0));
    uint32_t row[S::ROWDW];
#pragma unroll
    for (int w = 0; w < S::ROWDW; ++w) {
      uint32_t val;
      if (w < R / 2) {
        const uint32_t a = xp[w / 2][2 * (w % 2)], b = xp[w / 2][2 * (w % 2) + 1];
        val = pack_bf16(__builtin_bit_cast(float, a) * sp, __builtin_bit_cast(float, b) * sp);
      } else if (w < R / 2 + DH / 2) {
        const int q = w - R / 2;
        const uint32_t x = xc[q / 4][q % 4];
        val = FUSEQ ? 0u : pack_bf16(bf16_lo(x) * sc, bf16_hi(x) * sc);  // fused: written below
      } else if (w == S::CONSTDW) {
        val = 0xC0E00000u;  // (-m_hat = 0, -OFF = -7)
      } else {
        val = 0u;
      }
      row[w] = (real || w == S::CONSTDW) ? val : 0u;
    }
    uint32_t* dst = lds + tid * S::KSTR;
#pragma unroll
    for (int w = 0; w < S::ROWDW; w += 4)
      *reinterpret_cast<u32x4_t*>(dst + w) = (u32x4_t){row[w], row[w + 1], row[w + 2], row[w + 3]};
  }
  if constexpr (FUSEQ) {
    // Qc = bf16(LN(x) W_q + b_q) of the wave's own rows (same wave as the row writes above)
    uint32_t* wtl = lds + S::QS_DW;
    lnq_stage_w<DH>(wtl, *lnq, G.C, G.h);
    __syncthreads();
    lnq_reduce<DH>(wtl, *lnq, G.h);
    // both query blocks' x rows are requested before either is used
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(lnq->x), (short)0, (int)map_bytes, (int)RSRC_WORD3);
    u32x4_t xw[2][LNQ_KS];
    bool real[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int r = q0 + wave * QW + qb * 32 + l32;
      real[qb] = r < G.n_real;
      int off, n;
      locate<DH>(G, real[qb] ? r : G.n_real - 1, off, n);
      lnq_load(xw[qb], rx, off - G.h * DH, G.C, gh);
    }
    __syncthreads();
    const float scq = LOG2E / sqrtf((float)DH);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
      lnq_block<DH, R>(lds, wtl, *lnq, xw[qb], real[qb], wave * QW + qb * 32 + l32, G.C, l32, gh, scq);
  }
  __syncthreads();
  Regs<DH, R> rg;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
    for (int c = 0; c < S::KC; ++c)
      rg.qt[qb][c] = *reinterpret_cast<const u32x4_t*>(lds + (wave * QW + qb * 32 + l32) * S::KSTR + 8 * c + 4 * gh);
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) rg.O[qb][dt][e] = 0.0f;
    rg.mhat[qb] = 0.0f;
    rg.lpart[qb] = 0.0f;
  }
  __syncthreads();

  const int ntiles = (G.n_real + KT - 1) / KT;
  const bool active = q0 + wave * QW < G.n_real;
  const int grp = wave >> 2;  // 0: waves 0-3 lead, 1: waves 4-7 follow half a step behind
  // this wave's load source (wave-uniform): see the staging notes above
  using RL = Roles<DH, R>;
  const unsigned pos_bytes = (unsigned)(NW * R) * 4u;
  const void* src = (wave == 2 || wave == 3) ? (const void*)kc
                  : (wave == 4 || wave == 5) ? (const void*)v : (const void*)kp;
  const bool loads = wave == 0 || (wave == 1 && RL::KP1) || wave == 2 || (wave == 3 && RL::KC1) ||
                     wave == 4 || (wave == 5 && RL::V1) || (wave >= 6 && RL::KP67);
  const unsigned nbytes = !loads ? 0u : (wave >= 2 && wave <= 5) ? map_bytes : pos_bytes;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(src), (short)0, (int)nbytes, (int)RSRC_WORD3);
  // load cursor of this lane, starting at key r = lane of tile 0
  const bool pos = (wave == 0) | (wave == 1) | (wave >= 6);
  const unsigned sub = wave >= 6 ? (unsigned)(wave - 4) : (unsigned)(wave & 1);  // 32-byte sub-chunk
  CursorStep cs;
  cs.col = pos ? (unsigned)(R * 4) : (unsigned)(G.C * 2);
  const unsigned row_bytes = pos ? (unsigned)(ws * R * 4) : (unsigned)(W * G.C * 2);
  const unsigned frame_bytes = pos ? (unsigned)(ws * ws * R * 4) : (unsigned)(H * W * G.C * 2);
  cs.wrap = row_bytes - (unsigned)G.nx * cs.col;
  cs.fskip = (unsigned)((pos ? ws : H) - G.ny) * row_bytes;
  Cursor cur;
  {
    const int rr = (int)(((float)lane + 0.5f) * G.inv_nx);
    cur.ix = lane - rr * G.nx;
    const int it = (int)(((float)rr + 0.5f) * G.inv_ny);
    cur.iy = rr - it * G.ny;
    const unsigned base =
        pos ? 0u
            : 2u * (unsigned)((((G.b * T + G.tw * wt) * H + G.wy * ws) * W + G.wx * ws) * G.C + G.h * DH);
    cur.voff = base + (unsigned)it * frame_bytes + (unsigned)cur.iy * row_bytes + (unsigned)cur.ix * cs.col + 32u * sub;
  }

  // ---- prologue: tile 0 staged by everyone, tile 1 loaded into registers
  Stage st;
  load_tile(rsrc, cur, st);
  if (ntiles > 1) {
    store_tile<DH, R, false>(lds, wave, lane, true, st);
    cursor_advance(cur, cs, G.nx, G.ny);
    load_tile(rsrc, cur, st);
  } else {
    store_tile<DH, R, true>(lds, wave, lane, lane < G.n_real, st);
  }
  __syncthreads();

  f32x16_t Sacc[2][2];
  uint32_t P[2][2][8];
  // Half-steps: the leading group (waves 0-3) runs MFMA(0), softmax(0),
  // MFMA(1), ..., softmax(T-1), MFMA(T), idle; the following group (waves
  // 4-7) runs idle, MFMA(0), ..., softmax(T-1), MFMA(T).  MFMA(t) = QK^T of
  // tile t (t < T) and PV of tile t-1 (t >= 1), plus this wave's share of
  // staging: store tile t+1 (loaded one step earlier) and load tile t+2,
  // issued while the operand reads are in flight.  softmax(t) = exp2,
  // convert and overflow check of tile t, no LDS traffic.  Tile x is stored
  // in half-steps 2x-2 (leading group) and 2x-1 (following group) and read
  // in half-steps 2x .. 2x+3; its stage is rewritten in half-step 2x+4.
  PhaseOps<DH, R> ops;
  auto stage = [&](int x) {  // store tile x, load tile x+1
    if (x < ntiles) {
      uint32_t* dst = lds + (x % NSTAGE) * S::STAGE_DW;
      if (x + 1 < ntiles) {
        store_tile<DH, R, false>(dst, wave, lane, true, st);
        cursor_advance(cur, cs, G.nx, G.ny);
        load_tile(rsrc, cur, st);
      } else {
        store_tile<DH, R, true>(dst, wave, lane, x * KT + lane < G.n_real, st);
      }
    }
  };
  auto softmax = [&](int t) {
    if (active) {
      if constexpr (RL::KPREF) {
        if (t + 1 < ntiles) read_k_ops<DH, R>(lds, ((t + 1) % NSTAGE) * S::STAGE_DW, l32, gh, ops);
      }
      const uint32_t orv = exp_tile_fast(Sacc, P);
      const bool first = t == 0;
      if (__builtin_amdgcn_ballot_w64(first || (orv & 0x40004000u))) rescale_tile<DH, R>(rg, Sacc, P, first, gh);
    }
  };
  if (grp == 1) __syncthreads();
  if (active) read_k_ops<DH, R>(lds, 0, l32, gh, ops);
  stage(1);
  if (active) {
    __builtin_amdgcn_sched_barrier(0);
    qk_tile<DH, R>(ops, rg, Sacc);
  }
  __syncthreads();
  for (int t = 0; t + 1 < ntiles; ++t) {
    softmax(t);
    __syncthreads();
    // The MFMA phase (operand reads, staging, MFMAs) takes issue priority over
    // the other group's softmax on the same SIMD; with equal priority the
    // older wave wins every tie and the following group's MFMA phase starves.
    __builtin_amdgcn_s_setprio(2);
    if (active) {
      if constexpr (!RL::KPREF) read_k_ops<DH, R>(lds, ((t + 1) % NSTAGE) * S::STAGE_DW, l32, gh, ops);
      read_v_ops<DH, R>(lds, (t % NSTAGE) * S::STAGE_DW + S::KS_DW, lane, ops);
    }
    stage(t + 2);
    if (active) {
      __builtin_amdgcn_sched_barrier(0);  // operand reads and staging issue before the first MFMA
      qk_tile<DH, R>(ops, rg, Sacc);
      __builtin_amdgcn_sched_barrier(0);  // QK first: its operands are the earliest ready
      pv_tile<DH, R>(ops, rg, P);
    }
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
  }
  // the gate values of the epilogue are loaded now, so that their latency hides behind the
  // last tile's softmax and product instead of following them
  // (channels d0 .. d0+3 of the lane's token: one 8-byte buffer load; where the head slice ends
  // inside the 4 channels the second dword belongs to the next slice and is not used)
  int goff[2];
  uint32_t gv[2][S::DT][4][2];
  const __amdgpu_buffer_rsrc_t rgt =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(g), (short)0, (int)map_bytes, (int)RSRC_WORD3);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int r = q0 + wave * QW + qb * 32 + l32;
    int n;
    locate<DH>(G, r < G.n_real ? r : G.n_real - 1, goff[qb], n);
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = dt * 32 + 8 * q4 + 4 * gh;
        u32x2_t w2 = {0u, 0u};
        if (active && d0 < DH)
          w2 = __builtin_bit_cast(u32x2_t,
                                  __builtin_amdgcn_raw_buffer_load_b64(rgt, 2u * (unsigned)(goff[qb] + d0), 0, 0));
        gv[qb][dt][q4][0] = w2[0];
        gv[qb][dt][q4][1] = w2[1];
      }
  }
  softmax(ntiles - 1);
  __syncthreads();
  if (active) {
    read_v_ops<DH, R>(lds, ((ntiles - 1) % NSTAGE) * S::STAGE_DW + S::KS_DW, lane, ops);
    pv_tile<DH, R>(ops, rg, P);
  }
  __syncthreads();
  if (grp == 0) __syncthreads();

  if (!active) return;
  // ---- epilogue: O / l * sigmoid(G), bf16, NHWC; 4 channels per 8-byte buffer store
  const __amdgpu_buffer_rsrc_t rot = __builtin_amdgcn_make_buffer_rsrc(o, (short)0, (int)map_bytes, (int)RSRC_WORD3);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int r = q0 + wave * QW + qb * 32 + l32;
    const float lsum = row_sum(rg, qb);
    if (r >= G.n_real) continue;
    const float inv = rcp_approx(lsum);
    const int off = goff[qb];
    if (lse) lse[(off - G.h * DH) / G.C * heads + G.h] = (rg.mhat[qb] + OFF + __log2f(lsum)) * LN2;
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = dt * 32 + 8 * q4 + 4 * gh;
        if (d0 >= DH) continue;
        const int e0 = 4 * q4;
        const int gw = (off + d0) >> 1;  // dword index of channels (d0, d0+1)
        const uint32_t g01 = gv[qb][dt][q4][0];
        const uint32_t r01 = pack_bf16(rg.O[qb][dt][e0 + 0] * inv * sigmoidf(bf16_lo(g01)),
                                       rg.O[qb][dt][e0 + 1] * inv * sigmoidf(bf16_hi(g01)));
        if (d0 + 4 <= DH) {
          const uint32_t g23 = gv[qb][dt][q4][1];
          const uint32_t r23 = pack_bf16(rg.O[qb][dt][e0 + 2] * inv * sigmoidf(bf16_lo(g23)),
                                         rg.O[qb][dt][e0 + 3] * inv * sigmoidf(bf16_hi(g23)));
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) int,
                                                                   (u32x2_t){r01, r23}),
                                                rot, 4u * (unsigned)gw, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b32((int)r01, rot, 4u * (unsigned)gw, 0, 0);
        }
      }
  }
}

// ---- small windows (window^2 <= 256) ------------------------------------------
// One workgroup of four waves covers a whole window and head: every thread
// stages one key (all roles of the staging scheme above) into its 64-key tile,
// so all key tiles are resident in LDS after a single barrier and the key loop
// runs without barriers.  Each wave takes its 64 queries as two blocks of 32,
// one after the other, which keeps it under 168 registers: three workgroups
// (four below 128 registers) share a CU, so the grid of a small map is
// resident at once.  The first block's Q~ operands and gate values come
// straight from global memory before that barrier, so the loads of a
// workgroup are all in flight together.  16x16 windows hold 4 key tiles.
constexpr int SQ = 256;        // queries (and keys) per workgroup
constexpr int SNT = SQ / KT;   // key tiles, all resident

// Dwords w0 .. w0+3 (w0 = 8c + 4gh, the lane's half of chunk c) of a Q~ row:
// [Qp/sqrt(R), Qc/sqrt(dh)] (log2 e folded in), the (-m_hat = 0, -offset) pair
// `cw`, zeros; a padded query row keeps only the constant pair.  R/2 and w0 are
// multiples of 4, so a group is all Qp, or Qc up to the end of the slice, or
// neither: one pair of 16-byte Qp loads or one 16-byte Qc load (bounds-checked
// buffer loads; past the end of the head slice the dwords are not used).
template <int DH, int R>
__device__ __forceinline__ u32x4_t qrow_group(int w0, int off, int n, bool real, __amdgpu_buffer_rsrc_t rqp,
                                              __amdgpu_buffer_rsrc_t rqc, float sp, float sc, uint32_t cw) {
  using S = Shape<DH, R>;
  static_assert(R % 8 == 0, "Qp groups of 4 dwords");
  u32x4_t q;
  if (w0 < R / 2) {
    const f32x4_t a =
        __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rqp, (unsigned)(n * R + 2 * w0) * 4u, 0, 0));
    const f32x4_t b = __builtin_bit_cast(
        f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rqp, (unsigned)(n * R + 2 * w0) * 4u + 16u, 0, 0));
    q = (u32x4_t){pack_bf16(a[0] * sp, a[1] * sp), pack_bf16(a[2] * sp, a[3] * sp), pack_bf16(b[0] * sp, b[1] * sp),
                  pack_bf16(b[2] * sp, b[3] * sp)};
  } else if (w0 < R / 2 + DH / 2) {
    const u32x4_t x = __builtin_bit_cast(
        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rqc, 2u * (unsigned)off + 4u * (unsigned)(w0 - R / 2), 0, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int w = w0 + i;
      q[i] = w < R / 2 + DH / 2 ? pack_bf16(bf16_lo(x[i]) * sc, bf16_hi(x[i]) * sc) : (w == S::CONSTDW ? cw : 0u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = w0 + i == S::CONSTDW ? cw : 0u;
  }
  if (!real) {
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = w0 + i == S::CONSTDW ? cw : 0u;
  }
  return q;
}

// gate channels d0 .. d0+3 of the head slice at element offset `off` (one 8-byte
// buffer load; where the slice ends inside the 4 channels the second dword is
// not used)
__device__ __forceinline__ u32x2_t gate4(__amdgpu_buffer_rsrc_t rg, int off, int d0) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rg, 2u * (unsigned)(off + d0), 0, 0));
}

// output channels d0 .. d0+3 (both dwords) or d0 .. d0+1 (the slice ends there)
__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t ro, int off, int d0, uint32_t r01, uint32_t r23,
                                       bool both) {
  if (both)
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) int,
                                                             (u32x2_t){r01, r23}),
                                          ro, 2u * (unsigned)(off + d0), 0, 0);
  else
    __builtin_amdgcn_raw_buffer_store_b32((int)r01, ro, 2u * (unsigned)(off + d0), 0, 0);
}

// buffer descriptors of a call's maps and positional table (num_records bounds every access)
struct MapRsrc {
  __amdgpu_buffer_rsrc_t qp, qc, g, o;
};
__device__ __forceinline__ MapRsrc map_rsrc(const float* qp, const uint32_t* qc, const uint32_t* g, uint32_t* o,
                                            unsigned map_bytes, unsigned pos_bytes) {
  MapRsrc m;
  m.qp = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(qp), (short)0, (int)pos_bytes, (int)RSRC_WORD3);
  m.qc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qc), (short)0, (int)map_bytes, (int)RSRC_WORD3);
  m.g = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(g), (short)0, (int)map_bytes, (int)RSRC_WORD3);
  m.o = __builtin_amdgcn_make_buffer_rsrc(o, (short)0, (int)map_bytes, (int)RSRC_WORD3);
  return m;
}

// Stages key r of window G (every role of the staging scheme: Kp, Kc and V
// parts, padded keys masked) into row r % 64 of tile (r / 64) % 4 of `lds`;
// the calling thread is thread r % 256 of a 256-thread workgroup.  MASK =
// false: the caller knows key r is real (no selects on the stored words).
template <int DH, int R, bool MASK = true>
__device__ __forceinline__ void stage_key(const Geo& G, uint32_t* lds, int r, const uint32_t* __restrict__ kc,
                                          const uint32_t* __restrict__ v, const float* __restrict__ kp,
                                          int map_elems, int window_tokens) {
  using S = Shape<DH, R>;
  using RL = Roles<DH, R>;
  const bool real = r < G.n_real;
  int off, n;
  locate<DH>(G, real ? r : G.n_real - 1, off, n);
  const unsigned map_bytes = (unsigned)map_elems * 2u;
  const unsigned pos_bytes = (unsigned)(window_tokens * R) * 4u;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(kc), (short)0,
                                                                      (int)map_bytes, (int)RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(v), (short)0,
                                                                      (int)map_bytes, (int)RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(kp), (short)0,
                                                                      (int)pos_bytes, (int)RSRC_WORD3);
  uint32_t* stage = lds + ((r >> 6) & (SNT - 1)) * S::STAGE_DW;
  const int lane = r & 63;
  Stage st[8];
#pragma unroll
  for (int role = 0; role < 8; ++role) {
    const bool loads = role == 0 || (role == 1 && RL::KP1) || role == 2 || (role == 3 && RL::KC1) ||
                       role == 4 || (role == 5 && RL::V1) || (role >= 6 && RL::KP67);
    if (loads) {
      const bool pos = role == 0 || role == 1 || role >= 6;
      const unsigned sub = role >= 6 ? (unsigned)(role - 4) : (unsigned)(role & 1);
      const unsigned voff = (pos ? (unsigned)(n * (R * 4)) : 2u * (unsigned)off) + 32u * sub;
      const __amdgpu_buffer_rsrc_t rs = (role == 2 || role == 3) ? rk : (role == 4 || role == 5) ? rv : rp;
      st[role].raw[0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0));
      st[role].raw[1] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16u, 0, 0));
    } else {
      st[role].raw[0] = (u32x4_t){0u, 0u, 0u, 0u};
      st[role].raw[1] = (u32x4_t){0u, 0u, 0u, 0u};
    }
  }
#pragma unroll
  for (int role = 0; role < 8; ++role) store_tile<DH, R, MASK>(stage, role, lane, real, st[role]);
}

// One workgroup of the whole-window kernel: logical = window unit.
template <int DH, int R>
__device__ __forceinline__ void attn_small_body(const uint32_t* __restrict__ qc, const uint32_t* __restrict__ kc,
                       const uint32_t* __restrict__ v, const uint32_t* __restrict__ g,
                       const float* __restrict__ qp, const float* __restrict__ kp,
                       uint32_t* __restrict__ o, int B, int T, int H, int W, int heads, int wt, int ws,
                       int total, long tstride, float* __restrict__ lse, int logical,
                       uint32_t* lds) {
  using S = Shape<DH, R>;

  if (logical >= total) return;
  Geo G;
  decode_window<DH>(G, logical, T, H, W, heads, wt, ws);
  qp += (long)G.h * tstride;  // per-head positional tables (tstride 0: one shared pair)
  kp += (long)G.h * tstride;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int gh = lane >> 5;

  // ---- key r = tid: every staging role of the key, into tile r / 64 = wave
  stage_key<DH, R>(G, lds, tid, kc, v, kp, B * T * H * W * heads * DH, wt * ws * ws);

  // ---- the wave's 64 queries run as two passes of 32 (NQ = 1): fewer live
  // registers, so three workgroups fit on a CU.  A pass picks up its Q~
  // operands and gate values straight from global memory; the first pass
  // issues those loads before the staging barrier.
  const float sp = LOG2E / sqrtf((float)R);
  const float sc = LOG2E / sqrtf((float)DH);
  Regs<DH, R, 1> rg;
  uint32_t gv[S::DT][4][2];
  int offq = 0;
  const MapRsrc mr = map_rsrc(qp, qc, g, o, (unsigned)(B * T * H * W * heads * DH) * 2u,
                              (unsigned)(wt * ws * ws * R) * 4u);
  auto load_block = [&](int qb) {
    const int r = wave * QW + qb * 32 + l32;
    const bool real = r < G.n_real;
    int off, n;
    locate<DH>(G, real ? r : G.n_real - 1, off, n);
    offq = off;
#pragma unroll
    for (int c = 0; c < S::KC; ++c)
      rg.qt[0][c] = qrow_group<DH, R>(8 * c + 4 * gh, off, n, real, mr.qp, mr.qc, sp, sc, 0xC2800000u);  // (0, -OFF_FAST)
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = dt * 32 + 8 * q4 + 4 * gh;
        u32x2_t w2 = {0u, 0u};
        if (d0 < DH) w2 = gate4(mr.g, off, d0);
        gv[dt][q4][0] = w2[0];
        gv[dt][q4][1] = w2[1];
      }
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) rg.O[0][dt][e] = 0.0f;
    rg.mhat[0] = 0.0f;
    rg.lpart[0] = 0.0f;
  };
  load_block(0);
  __syncthreads();

  const int ntiles = (G.n_real + KT - 1) / KT;
  for (int qb = 0; qb < 2; ++qb) {
    if (wave * QW + qb * 32 >= G.n_real) return;  // no real query left in this wave; no barrier follows
    if (qb > 0) load_block(qb);
    PhaseOps<DH, R> ops;
    f32x16_t Sacc[1][2];
    uint32_t P[1][2][8];
    // First pass: every tile exponentiated against the fixed reference m_hat = 0 with the
    // offset OFF_FAST = 64, p = 2^(s - 64), without a check (s: score in base-2 units; no
    // row maximum is taken).  bf16 P keeps fp32's exponent range, so the pass is exact up
    // to rounding while p and the fp32 sums stay finite and the row's largest p is a
    // normal number.  Its result is kept when the row sum l and the output are finite and
    // l >= 2^-86; since l <= 256 * 2^(s_max - 64), that means s_max >= -30, so keys that
    // flush to zero (more than 62 below 0) weigh less than 2^-32 of the row's largest.
    // Rows with s_max >= -22 always pass the test; finite sums hold for s_max up to about
    // 170 with |V| < 2^14.  A block that fails repeats its tiles with the checked loop:
    // exact maximum on the first tile, offset OFF, an OR over the packed P of every tile,
    // and a rescale whenever a score exceeds the reference by more than 8.
    OpsWalk<DH, R> walk(l32, gh, lane, 0, S::KS_DW);
    for (int x = 0; x < ntiles; ++x) {
      walk.read(lds, S::STAGE_DW, ops);
      qk_tile<DH, R>(ops, rg, Sacc);
      (void)exp_tile_fast(Sacc, P);
      pv_tile<DH, R>(ops, rg, P);
    }
    float off_used = OFF_FAST;
    {
      float t = row_sum(rg, 0);
      int bad = !(t >= 0x1p-86f);
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) t += rg.O[0][dt][e];
      bad |= !__builtin_isfinite(t);
      if (__builtin_amdgcn_ballot_w64(bad)) {
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e) rg.O[0][dt][e] = 0.0f;
        rg.mhat[0] = 0.0f;
        rg.lpart[0] = 0.0f;
        if (gh == S::GM) rg.qt[0][S::CM][S::DM] = 0xC0E00000u;  // (-m_hat = 0, -OFF = -7)
        OpsWalk<DH, R> rwalk(l32, gh, lane, 0, S::KS_DW);
        for (int x = 0; x < ntiles; ++x) {
          rwalk.read(lds, S::STAGE_DW, ops);
          qk_tile<DH, R>(ops, rg, Sacc);
          const uint32_t orv = exp_tile_fast(Sacc, P);
          const bool first = x == 0;
          if (__builtin_amdgcn_ballot_w64(first || (orv & 0x40004000u))) rescale_tile<DH, R>(rg, Sacc, P, first, gh);
          pv_tile<DH, R>(ops, rg, P);
        }
        off_used = OFF;
      }
    }

    // ---- epilogue of the block: O / l * sigmoid(G), bf16, NHWC
    const int r = wave * QW + qb * 32 + l32;
    const float lsum = row_sum(rg, 0);
    if (r < G.n_real) {
      const float inv = rcp_approx(lsum);
      if (lse) lse[(offq - G.h * DH) / G.C * heads + G.h] = (rg.mhat[0] + off_used + __log2f(lsum)) * LN2;
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d0 = dt * 32 + 8 * q4 + 4 * gh;
          if (d0 >= DH) continue;
          const int e0 = 4 * q4;
          const uint32_t g01 = gv[dt][q4][0], g23 = gv[dt][q4][1];
          const uint32_t r01 = pack_bf16(rg.O[0][dt][e0 + 0] * inv * sigmoidf(bf16_lo(g01)),
                                         rg.O[0][dt][e0 + 1] * inv * sigmoidf(bf16_hi(g01)));
          const uint32_t r23 = pack_bf16(rg.O[0][dt][e0 + 2] * inv * sigmoidf(bf16_lo(g23)),
                                         rg.O[0][dt][e0 + 3] * inv * sigmoidf(bf16_hi(g23)));
          store4(mr.o, offq, d0, r01, r23, d0 + 4 <= DH);
        }
    }
  }
}

// ---- windows of more than 256 tokens: the chunked kernel ----------------------
// One workgroup of four waves takes the queries of NB 32-query blocks per wave
// (256, 384 or 512) of one (window, head); the window's keys pass through LDS
// in chunks of 256 (four 64-key tiles), every thread staging one key of a
// chunk as in the whole-window kernel.  Each wave keeps its blocks (Q~
// operands, O, reference) in registers across the chunks; per tile it reads
// the K~ and V operands once for all of them and takes the blocks in pairs:
// both blocks' score products, then the first block's exponentials while the
// second block's scores are still on the matrix core.
// The softmax first runs unchecked, as the whole-window kernel's first pass
// does: every tile against the fixed reference 0 with the offset OFF_FAST.  A
// 32-query block whose row sum ends below 2^-80 or whose row sum or output is
// not finite is computed again, all chunks staged again for the whole
// workgroup, with the tiled kernel's checked loop: exact maximum on the first
// tile, offset OFF, an OR over the packed P of every later tile and a rescale
// when the maximum grew by more than 8.  A kept row has l >= 2^-80 and
// l <= n 2^(s_max - 64) over its n <= 16,384 keys, so s_max >= -30 base-2
// units: keys that flush to zero (more than 62 below 0) each weigh under 2^-32
// of the row's largest.  There is no hand-off between
// waves: three workgroups (two with three or four blocks per wave) share a CU,
// and while one stages a chunk the others compute.
// NB 32-query blocks per wave: NB = 2 (64 queries per wave, 256 per workgroup,
// three workgroups per CU), 3 or 4 (96 or 128 per wave, 384 or 512 per
// workgroup, two workgroups per CU: each staged chunk and each tile's operand
// reads then serve 1.5 or 2 times the queries).
template <int DH, int R, int NB = 2>
__device__ __forceinline__ void attn_chunk_body(const uint32_t* __restrict__ qc, const uint32_t* __restrict__ kc,
                       const uint32_t* __restrict__ v, const uint32_t* __restrict__ g,
                       const float* __restrict__ qp, const float* __restrict__ kp,
                       uint32_t* __restrict__ o, int B, int T, int H, int W, int heads, int wt, int ws,
                       int total, long tstride, float* __restrict__ lse, int logical,
                       uint32_t* lds) {
  using S = Shape<DH, R>;
  constexpr int WQ = 32 * NB;      // queries per wave
  constexpr int CQ = 4 * WQ;       // queries per workgroup

  if (logical >= total) return;
  const int qblocks = (wt * ws * ws + CQ - 1) / CQ;
  Geo G;
  decode_window<DH>(G, logical / qblocks, T, H, W, heads, wt, ws);
  const int q0 = (logical % qblocks) * CQ;
  if (q0 >= G.n_real) return;
  qp += (long)G.h * tstride;  // per-head positional tables (tstride 0: one shared pair)
  kp += (long)G.h * tstride;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int gh = lane >> 5;

  // Q~ operands of the wave's query blocks, straight from global memory
  const float sp = LOG2E / sqrtf((float)R);
  const float sc = LOG2E / sqrtf((float)DH);
  Regs<DH, R, 1> rg[NB];
  const MapRsrc mr = map_rsrc(qp, qc, g, o, (unsigned)(B * T * H * W * heads * DH) * 2u,
                              (unsigned)(wt * ws * ws * R) * 4u);
  const int wq0 = q0 + wave * WQ;  // first query of the wave
  auto init_block = [&](Regs<DH, R, 1>& r_, int qb) {
    const int r = wq0 + qb * 32 + l32;
    const bool real = r < G.n_real;
    int off, n;
    locate<DH>(G, real ? r : G.n_real - 1, off, n);
#pragma unroll
    for (int c = 0; c < S::KC; ++c)
      r_.qt[0][c] = qrow_group<DH, R>(8 * c + 4 * gh, off, n, real, mr.qp, mr.qc, sp, sc, 0xC2800000u);  // (0, -OFF_FAST)
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) r_.O[0][dt][e] = 0.0f;
    r_.mhat[0] = 0.0f;
    r_.lpart[0] = 0.0f;
  };
#pragma unroll
  for (int b = 0; b < NB; ++b) init_block(rg[b], b);
  // blocks holding a real query: a prefix of the wave's blocks (wave-uniform)
  const int nact = G.n_real <= wq0 ? 0 : min(NB, (G.n_real - wq0 + 31) / 32);
  const int map_elems = B * T * H * W * heads * DH;

  PhaseOps<DH, R> ops;
  f32x16_t Sacc[1][2];
  uint32_t P[1][2][8];
  auto run_tiles = [&](Regs<DH, R, 1>& r_, int nt, bool first_chunk) {
    OpsWalk<DH, R> walk(l32, gh, lane, 0, S::KS_DW);
    for (int x = 0; x < nt; ++x) {
      walk.read(lds, S::STAGE_DW, ops);
      qk_tile<DH, R>(ops, r_, Sacc);
      const uint32_t orv = exp_tile_fast(Sacc, P);
      const bool first = first_chunk && x == 0;
      if (__builtin_amdgcn_ballot_w64(first || (orv & 0x40004000u))) rescale_tile<DH, R>(r_, Sacc, P, first, gh);
      pv_tile<DH, R>(ops, r_, P);
    }
  };
  const int nchunks = (G.n_real + SQ - 1) / SQ;
  // stage each chunk of the window's keys (the whole workgroup), then run `tiles` on it
  auto over_chunks = [&](auto&& tiles) {
    for (int ch = 0; ch < nchunks; ++ch) {
      if (ch > 0) __syncthreads();  // every wave is done with the previous chunk's tiles
      const int left = G.n_real - ch * SQ;
      if (left >= SQ)  // every key of the chunk is real: no masking selects
        stage_key<DH, R, false>(G, lds, ch * SQ + tid, kc, v, kp, map_elems, wt * ws * ws);
      else
        stage_key<DH, R, true>(G, lds, ch * SQ + tid, kc, v, kp, map_elems, wt * ws * ws);
      __syncthreads();
      tiles(ch, left >= SQ ? SNT : (left + KT - 1) / KT);
    }
  };
  // unchecked pass; a pair of blocks at a time: one operand read per tile for all
  // blocks, the second block's scores issue on the matrix core while the first
  // block's exponentials run
  over_chunks([&](int, int nt) {
    if (nact == 0) return;
    f32x16_t Sb[1][2];
    uint32_t Pb[1][2][8];
    OpsWalk<DH, R> walk(l32, gh, lane, 0, S::KS_DW);
    for (int x = 0; x < nt; ++x) {
      walk.read(lds, S::STAGE_DW, ops);
#pragma unroll
      for (int p = 0; p < (NB + 1) / 2; ++p) {
        const int q1 = 2 * p + 1 < NB ? 2 * p + 1 : 2 * p;  // the pair's second block, if any
        if (2 * p + 1 < NB && q1 < nact) {
          qk_tile<DH, R>(ops, rg[2 * p], Sacc);
          qk_tile<DH, R>(ops, rg[q1], Sb);
          (void)exp_tile_fast(Sacc, P);
          pv_tile<DH, R>(ops, rg[2 * p], P);
          (void)exp_tile_fast(Sb, Pb);
          pv_tile<DH, R>(ops, rg[q1], Pb);
        } else if (2 * p < nact) {
          qk_tile<DH, R>(ops, rg[2 * p], Sacc);
          (void)exp_tile_fast(Sacc, P);
          pv_tile<DH, R>(ops, rg[2 * p], P);
        }
      }
    }
  });
  // a block fails if its row sum is below 2^-80 or its row sum or output is not finite
  // (wave-uniform)
  auto failed = [&](Regs<DH, R, 1>& r_) -> bool {
    float t = row_sum(r_, 0);
    int bad = !(t >= 0x1p-80f);
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) t += r_.O[0][dt][e];
    bad |= !__builtin_isfinite(t);
    return __builtin_amdgcn_ballot_w64(bad) != 0;
  };
  bool redo[NB];
  bool any = false;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    redo[b] = b < nact && failed(rg[b]);
    any |= redo[b];
  }
  // every wave is past its tiles here, so the re-run may stage over the last chunk
  if (__syncthreads_or(any)) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (redo[b]) {
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e) rg[b].O[0][dt][e] = 0.0f;
        rg[b].mhat[0] = 0.0f;
        rg[b].lpart[0] = 0.0f;
        if (gh == S::GM) rg[b].qt[0][S::CM][S::DM] = 0xC0E00000u;  // (-m_hat = 0, -OFF = -7)
      }
    over_chunks([&](int ch, int nt) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
        if (redo[b]) run_tiles(rg[b], nt, ch == 0);
    });
  }

  // ---- epilogue: O / l * sigmoid(G), bf16, NHWC
  auto finish = [&](const Regs<DH, R, 1>& r_, int qb, bool redone) {
    const int r = wq0 + qb * 32 + l32;
    const float lsum = row_sum(r_, 0);
    if (r >= G.n_real) return;
    int off, n;
    locate<DH>(G, r, off, n);
    const float inv = rcp_approx(lsum);
    if (lse) lse[(off - G.h * DH) / G.C * heads + G.h] = (r_.mhat[0] + (redone ? OFF : OFF_FAST) + __log2f(lsum)) * LN2;
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = dt * 32 + 8 * q4 + 4 * gh;
        if (d0 >= DH) continue;
        const int e0 = 4 * q4;
        const u32x2_t g4 = gate4(mr.g, off, d0);
        const uint32_t r01 = pack_bf16(r_.O[0][dt][e0 + 0] * inv * sigmoidf(bf16_lo(g4[0])),
                                       r_.O[0][dt][e0 + 1] * inv * sigmoidf(bf16_hi(g4[0])));
        const uint32_t r23 = pack_bf16(r_.O[0][dt][e0 + 2] * inv * sigmoidf(bf16_lo(g4[1])),
                                       r_.O[0][dt][e0 + 3] * inv * sigmoidf(bf16_hi(g4[1])));
        store4(mr.o, off, d0, r01, r23, d0 + 4 <= DH);
      }
  };
#pragma unroll
  for (int b = 0; b < NB; ++b)
    if (b < nact) finish(rg[b], b, redo[b]);
}

// Workgroup -> logical index (window * heads + head) * qblocks + query block
// for the chunked kernel, on a grid of 8 * ceil(windows / 8) * heads * qblocks
// workgroups: all workgroups of a window (every head and query block) go to
// one XCD, whose L2 then holds the window's token rows once for all of them,
// and windows are dealt round-robin over the XCDs.  Indices past the last
// window are padding.
__device__ __forceinline__ int window_block(int bid, int per_window) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int k = slot / per_window;
  return (k * 8 + xcd) * per_window + (slot - k * per_window);
}

// As window_block, with the workgroups of a window numbered query block first:
// the heads of one query block take consecutive workgroups, so the resident
// workgroups of an XCD cover every head of the window at once and read each
// cache line of the window's token rows (which hold every head's slice)
// together.  Returns the logical index (window * heads + head) * qblocks + qb.
__device__ __forceinline__ int window_block_qb(int bid, int heads, int qblocks) {
  const int per = heads * qblocks;
  const int L = window_block(bid, per);
  const int win = L / per, j = L - win * per;
  const int qb = j / heads, h = j - qb * heads;
  return (win * heads + h) * qblocks + qb;
}

// Workgroup -> logical index (window unit * qblocks + query block) for a grid
// of 8 * ceil(units / 8) * qblocks workgroups.  Window unit 8k + x takes the
// workgroups whose index is x mod 8, which the dispatcher's round-robin sends
// to one XCD: the query blocks of a (window, head) share that XCD's L2, and
// every XCD gets every eighth window unit, so the smaller edge windows of a
// map spread evenly over the XCDs.  Logical indices past the last unit are
// padding and return at once.
__device__ __forceinline__ int interleave_logical(int bid, int qblocks) {
  const int per = 8 * qblocks;
  return ((bid / per) * 8 + bid % 8) * qblocks + (bid % per) / 8;
}

// Workgroup -> window unit for the whole-window kernel, on a grid of 8 * ceil(windows / 8) *
// heads workgroups.  The heads of a window take consecutive workgroups of one XCD (the
// dispatcher sends workgroup i to XCD i % 8), so the token rows they share (a row holds every
// head's slice) are fetched once into that XCD's L2; windows are dealt round-robin over the
// XCDs, so the smaller edge windows spread evenly.  Units past the last are padding.
__device__ __forceinline__ int window_unit(int bid, int heads) {
  const int xcd = bid & 7, slot = bid >> 3;  // slot-th workgroup this XCD receives
  const int k = slot / heads;
  return (k * 8 + xcd) * heads + (slot - k * heads);
}

// the tiled kernel with LayerNorm and the Q projection in its Q~ build (qc unused)
template <int DH, int R>
__global__ void __launch_bounds__(QB, 1)
attn_bf16_lnq_kernel(const uint32_t* __restrict__ kc, const uint32_t* __restrict__ v,
                     const uint32_t* __restrict__ g, const float* __restrict__ qp, const float* __restrict__ kp,
                     uint32_t* __restrict__ o, int B, int T, int H, int W, int heads, int wt, int ws, int total,
                     long tstride, float* __restrict__ lse, int whole_windows, const LnqArgs L) {
  const int qblocks = (wt * ws * ws + QB - 1) / QB;
  attn_tiled_body<DH, R, true>(nullptr, kc, v, g, qp, kp, o, B, T, H, W, heads, wt, ws, total, tstride, lse,
                               whole_windows ? window_block_qb(blockIdx.x, heads, qblocks)
                                             : interleave_logical(blockIdx.x, qblocks),
                               &L);
}

// whole_windows: the window count is a multiple of 8, so whole windows (every head and query
// block) can be dealt to the XCDs evenly (window_block); else window units are (interleave_logical)
template <int DH, int R>
__global__ void __launch_bounds__(QB, 1)
attn_bf16_kernel(const uint32_t* __restrict__ qc, const uint32_t* __restrict__ kc,
                 const uint32_t* __restrict__ v, const uint32_t* __restrict__ g,
                 const float* __restrict__ qp, const float* __restrict__ kp,
                 uint32_t* __restrict__ o, int B, int T, int H, int W, int heads, int wt, int ws, int total,
                 long tstride, float* __restrict__ lse, int whole_windows) {
  const int qblocks = (wt * ws * ws + QB - 1) / QB;
  attn_tiled_body<DH, R>(qc, kc, v, g, qp, kp, o, B, T, H, W, heads, wt, ws, total, tstride, lse,
                         whole_windows ? window_block(blockIdx.x, heads * qblocks)
                                       : interleave_logical(blockIdx.x, qblocks));
}

template <int DH, int R>
__global__ void __launch_bounds__(SQ, 3)
attn_bf16_small_kernel(const uint32_t* __restrict__ qc, const uint32_t* __restrict__ kc,
                       const uint32_t* __restrict__ v, const uint32_t* __restrict__ g,
                       const float* __restrict__ qp, const float* __restrict__ kp,
                       uint32_t* __restrict__ o, int B, int T, int H, int W, int heads, int wt, int ws,
                       int total, long tstride, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[SNT * Shape<DH, R>::STAGE_DW];
  attn_small_body<DH, R>(qc, kc, v, g, qp, kp, o, B, T, H, W, heads, wt, ws, total, tstride, lse,
                         window_unit(blockIdx.x, heads), lds);
}

// More than two blocks per wave (two workgroups per CU) only for the shapes
// whose blocks then still fit 256 registers.
constexpr bool chunk_more_blocks(int dh, int R) {
  return (dh == 30 && R == 16) || (dh == 16 && R == 16) || (dh == 8 && R == 8);
}

template <int DH, int R, int NB>
__global__ void __launch_bounds__(SQ, NB == 2 ? 3 : 2)
attn_bf16_chunk_kernel(const uint32_t* __restrict__ qc, const uint32_t* __restrict__ kc,
                       const uint32_t* __restrict__ v, const uint32_t* __restrict__ g,
                       const float* __restrict__ qp, const float* __restrict__ kp,
                       uint32_t* __restrict__ o, int B, int T, int H, int W, int heads, int wt, int ws,
                       int total, long tstride, float* __restrict__ lse, int whole_windows) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[SNT * Shape<DH, R>::STAGE_DW];
  const int qblocks = (wt * ws * ws + 128 * NB - 1) / (128 * NB);
  attn_chunk_body<DH, R, NB>(qc, kc, v, g, qp, kp, o, B, T, H, W, heads, wt, ws, total, tstride, lse,
                             whole_windows ? window_block_qb(blockIdx.x, heads, qblocks)
                                           : interleave_logical(blockIdx.x, qblocks), lds);
}

// Which kernel a call takes: the whole-window kernel up to SQ tokens per
// window, the chunked kernel above that.  The (dh, R) shapes whose chunked
// kernel spills registers ((32, 16), (16, 32), (30, 32): 52-124 bytes per lane
// against at most 8 for the others; not timed on the chunked kernel) keep the
// tiled kernel for windows of more than CHUNK_MAX tokens, unless the chunked
// grid is resident at once (three workgroups per CU, up to CHUNK_FIT tokens).
// Measured on the (30, 16) and (16, 16) shapes (same process, interleaved
// rounds): against the tiled kernel the chunked kernel takes 4% less time on
// 32 x 96x96 windows at C = 180, 1% less on 1x360x640 with 96x96 windows, 0.4%
// less on 64x64 windows at C = 180 and 5% less at C = 48; on 32x32 windows
// 8-23% less.
// XCD dealing of chunked calls: whole windows (every head and query block of a
// window on one XCD, window_block_qb) when the windows have at most CHUNK_MAX
// tokens or their number is a multiple of 8; otherwise window units one by one
// (interleave_logical), as the tiled kernel deals them.  Whole windows of 4,096
// or 9,216 tokens are too coarse to spread 15 or 28 windows evenly over 8 XCDs:
// 64x64 windows at C = 48 took 0.133 ms dealt whole and 0.126 ms by unit,
// 1x360x640 with 96x96 windows 2.18 against 1.80 ms; 32x32 windows (60 on a
// 180x320 map) are faster dealt whole (0.037 against 0.040 ms at C = 48).
constexpr int CHUNK_MAX = 2048;
constexpr int CHUNK_FIT = 4096;
enum Kind { WHOLE = 0, CHUNKED = 1, TILED = 2 };

// ---- several independent calls in one launch ---------------------------------
// The calls of a group share (dh, R) and the workgroup size, and otherwise
// differ freely (maps, window sizes, tables): one group takes whole-window and
// chunked calls together (256 threads), another tiled calls (512).  Each call
// owns a contiguous range of the grid, a multiple of 8 workgroups long, so that
// the dispatcher's round-robin over the 8 XCDs gives every XCD the same share
// of every call; inside a call, workgroups map to their work as in a single
// call (window_unit, window_block, interleave_logical), so every output is
// bit-identical to the single call's.  The host orders the calls longest first.
constexpr int GROUP_MAX = 8;

struct CallDesc {
  const uint32_t* qc;
  const uint32_t* kc;
  const uint32_t* v;
  const uint32_t* g;
  const float* qp;
  const float* kp;
  uint32_t* o;
  float* lse;
  long tstride;
  int B, T, H, W, heads, wt, ws, units, qblocks, kind;
  int whole;  // chunked calls: 1 = whole windows per XCD (window_block), 0 = by unit
};

struct CallGroup {
  int n;
  int first[GROUP_MAX + 1];  // first workgroup of each call; first[n] = grid size
  CallDesc c[GROUP_MAX];
};

// this workgroup's call (every index static: the selection stays in SGPRs)
__device__ __forceinline__ int group_call(const CallGroup& grp, int bid, CallDesc& c) {
  int i = 0;
  c = grp.c[0];
#pragma unroll
  for (int k = 1; k < GROUP_MAX; ++k)
    if (k < grp.n && bid >= grp.first[k]) {
      c = grp.c[k];
      i = k;
    }
  return bid - grp.first[i];
}

template <int DH, int R>
__global__ void __launch_bounds__(QB, 1) attn_bf16_group_kernel(const CallGroup grp) {
  CallDesc c;
  const int lb = group_call(grp, blockIdx.x, c);
  attn_tiled_body<DH, R>(c.qc, c.kc, c.v, c.g, c.qp, c.kp, c.o, c.B, c.T, c.H, c.W, c.heads, c.wt, c.ws,
                         c.units * c.qblocks, c.tstride, c.lse, interleave_logical(lb, c.qblocks));
}

// whole-window and chunked calls: a uniform branch per workgroup on its call's kind
template <int DH, int R>
__global__ void __launch_bounds__(SQ, 3) attn_bf16_window_group_kernel(const CallGroup grp) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[SNT * Shape<DH, R>::STAGE_DW];
  CallDesc c;
  const int lb = group_call(grp, blockIdx.x, c);
  if (c.kind == WHOLE)
    attn_small_body<DH, R>(c.qc, c.kc, c.v, c.g, c.qp, c.kp, c.o, c.B, c.T, c.H, c.W, c.heads, c.wt, c.ws,
                           c.units, c.tstride, c.lse, window_unit(lb, c.heads), lds);
  else
    attn_chunk_body<DH, R, 2>(c.qc, c.kc, c.v, c.g, c.qp, c.kp, c.o, c.B, c.T, c.H, c.W, c.heads, c.wt, c.ws,
                           c.units * c.qblocks, c.tstride, c.lse,
                           c.whole ? window_block_qb(lb, c.heads, c.qblocks) : interleave_logical(lb, c.qblocks), lds);
}

// window units of a call
inline int call_units(const AttnArgs& a) {
  const int nWy = (a.H + a.ws - 1) / a.ws, nWx = (a.W + a.ws - 1) / a.ws, nWt = (a.T + a.wt - 1) / a.wt;
  return a.B * nWt * nWy * nWx * a.heads;
}
// cus: compute units of the device
inline Kind call_kind(const AttnArgs& a, int cus) {
  const int NW = a.wt * a.ws * a.ws;
  if (NW <= SQ) return WHOLE;
  if (NW <= CHUNK_MAX) return CHUNKED;
  const bool spills = (a.dh == 32 && a.R == 16) || (a.dh == 16 && a.R == 32) || (a.dh == 30 && a.R == 32);
  if (!spills) return CHUNKED;
  const long wgs = (long)call_units(a) * ((NW + SQ - 1) / SQ);
  return NW <= CHUNK_FIT && wgs <= 3L * cus ? CHUNKED : TILED;
}
// chunked calls: whole windows to an XCD (see above)
inline bool chunk_whole(const AttnArgs& a) {
  return a.wt * a.ws * a.ws <= CHUNK_MAX || (call_units(a) / a.heads) % 8 == 0;
}
// 32-query blocks per wave of a chunked call's own launch (a grouped launch
// always takes two).  More blocks stage each key chunk and read each tile's
// operands for more queries, but make fewer, larger workgroups at two per CU.
// Measured, same box, interleaved rounds, bit-identical outputs (ms with 2 / 3 /
// 4 blocks): 32 x 96x96 at C = 180 2.426 / 2.408 / 2.355; 1x360x640 with 96x96
// windows 1.784 / 1.796 / 1.718; 64x64 windows at C = 180 0.2321 / 0.2286 /
// 0.2317; 32x32 windows at C = 180 0.0717 / 0.0783 / 0.0709; 8 frames with
// 2x32x32 windows 0.945 / 1.009 / 0.921, with 4x16x16 windows 0.571 / 0.617 /
// 0.572; 32x32 and 64x64 windows at C = 48 (SST-lite): 0.0349 / 0.0430 / 0.0408
// and 0.108 / 0.115 / 0.122.  Four blocks pay once the grid fills four rounds of
// two workgroups per CU; three only on windows of 4,096 tokens or more (a
// 384-query block wastes up to a third of a workgroup on smaller ones) whose
// grid still fills 1.75 rounds.
inline int chunk_blocks(const AttnArgs& a, int cus) {
  if (!chunk_more_blocks(a.dh, a.R)) return 2;
  const int NW = a.wt * a.ws * a.ws;
  const long units = call_units(a);
  if (units * ((NW + 511) / 512) >= 8L * cus) return 4;
  if (NW >= 4096 && 2 * units * ((NW + 383) / 384) >= 7L * cus) return 3;
  return 2;
}
// query blocks per window unit for a kernel kind (nb: 32-query blocks per wave
// of a chunked call)
inline int kind_qblocks(const AttnArgs& a, Kind k, int nb = 2) {
  const int NW = a.wt * a.ws * a.ws, CQ = 128 * nb;
  return k == WHOLE ? 1 : k == CHUNKED ? (NW + CQ - 1) / CQ : (NW + QB - 1) / QB;
}
// workgroups of a call's grid range
inline int kind_grid(const AttnArgs& a, Kind k, int nb = 2) {
  const int units = call_units(a), windows = units / a.heads, qb = kind_qblocks(a, k, nb);
  const bool by_unit = k == TILED || (k == CHUNKED && !chunk_whole(a));
  return by_unit ? 8 * ((units + 7) / 8) * qb                // see interleave_logical
                 : 8 * ((windows + 7) / 8) * a.heads * qb;   // see window_unit, window_block
}

template <int DH, int R>
hipError_t launch_variant(const AttnArgs& a, hipStream_t stream) {
  const int cus = device_cus();
  const Kind kind = call_kind(a, cus);
  const int nb = kind == CHUNKED ? chunk_blocks(a, cus) : 2;
  const int units = call_units(a), qb = kind_qblocks(a, kind, nb), grid = kind_grid(a, kind, nb);
  const uint32_t* qc = (const uint32_t*)a.qc;
  const uint32_t* kc = (const uint32_t*)a.kc;
  const uint32_t* v = (const uint32_t*)a.v;
  const uint32_t* g = (const uint32_t*)a.g;
  if (kind == WHOLE)
    hipLaunchKernelGGL((attn_bf16_small_kernel<DH, R>), dim3(grid), dim3(SQ), 0, stream, qc, kc, v, g, a.qp, a.kp,
                       (uint32_t*)a.o, a.B, a.T, a.H, a.W, a.heads, a.wt, a.ws, units, a.tstride, a.lse);
  else if (kind == CHUNKED) {
    auto launch = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(grid), dim3(SQ), 0, stream, qc, kc, v, g, a.qp, a.kp, (uint32_t*)a.o, a.B, a.T,
                         a.H, a.W, a.heads, a.wt, a.ws, units * qb, a.tstride, a.lse, chunk_whole(a) ? 1 : 0);
    };
    bool done = false;
    if constexpr (chunk_more_blocks(DH, R)) {
      if (nb == 4) launch(attn_bf16_chunk_kernel<DH, R, 4>), done = true;
      if (nb == 3) launch(attn_bf16_chunk_kernel<DH, R, 3>), done = true;
    }
    if (!done) launch(attn_bf16_chunk_kernel<DH, R, 2>);
  }
  else
    hipLaunchKernelGGL((attn_bf16_kernel<DH, R>), dim3(grid), dim3(QB), 0, stream, qc, kc, v, g, a.qp, a.kp,
                       (uint32_t*)a.o, a.B, a.T, a.H, a.W, a.heads, a.wt, a.ws, units * qb, a.tstride, a.lse,
                       (units / a.heads) % 8 == 0 ? 1 : 0);
  return hipGetLastError();
}

template <int DH, int R>
hipError_t launch_group(const AttnArgs* const* calls, const Kind* kinds, int n, bool tiled, hipStream_t stream) {
  CallGroup grp{};
  grp.n = n;
  int first = 0;
  for (int i = 0; i < n; ++i) {
    const AttnArgs& a = *calls[i];
    CallDesc& c = grp.c[i];
    c.qc = (const uint32_t*)a.qc;
    c.kc = (const uint32_t*)a.kc;
    c.v = (const uint32_t*)a.v;
    c.g = (const uint32_t*)a.g;
    c.qp = a.qp;
    c.kp = a.kp;
    c.o = (uint32_t*)a.o;
    c.lse = a.lse;
    c.tstride = a.tstride;
    c.B = a.B; c.T = a.T; c.H = a.H; c.W = a.W; c.heads = a.heads; c.wt = a.wt; c.ws = a.ws;
    c.units = call_units(a);
    c.qblocks = kind_qblocks(a, kinds[i]);
    c.kind = kinds[i];
    c.whole = chunk_whole(a) ? 1 : 0;
    grp.first[i] = first;
    first += kind_grid(a, kinds[i]);
  }
  grp.first[n] = first;
  if (tiled)
    hipLaunchKernelGGL((attn_bf16_group_kernel<DH, R>), dim3(first), dim3(QB), 0, stream, grp);
  else
    hipLaunchKernelGGL((attn_bf16_window_group_kernel<DH, R>), dim3(first), dim3(SQ), 0, stream, grp);
  return hipGetLastError();
}

// all calls share (dh, R): whole-window and chunked calls in groups of the
// 256-thread kernel, tiled calls in groups of the tiled kernel, each group's
// longest windows first
template <int DH, int R>
hipError_t launch_multi_variant(const AttnArgs* calls, int n, hipStream_t stream) {
  const int cus = device_cus();
  for (int tiled = 0; tiled <= 1; ++tiled) {
    const AttnArgs* sel[64];
    Kind kinds[64];
    int m = 0;
    for (int i = 0; i < n && m < 64; ++i) {
      const Kind k = call_kind(calls[i], cus);  // the kernel the single call takes
      if ((k == TILED) == (tiled != 0)) {
        sel[m] = &calls[i];
        kinds[m++] = k;
      }
    }
    // longest first: key tiles per window (stable insertion sort)
    for (int i = 1; i < m; ++i) {
      const AttnArgs* x = sel[i];
      const Kind kxk = kinds[i];
      const int kx = x->wt * x->ws * x->ws;
      int j = i - 1;
      while (j >= 0 && sel[j]->wt * sel[j]->ws * sel[j]->ws < kx) {
        sel[j + 1] = sel[j];
        kinds[j + 1] = kinds[j];
        --j;
      }
      sel[j + 1] = x;
      kinds[j + 1] = kxk;
    }
    for (int i = 0; i < m; i += GROUP_MAX) {
      const hipError_t e = launch_group<DH, R>(sel + i, kinds + i, m - i < GROUP_MAX ? m - i : GROUP_MAX,
                                               tiled != 0, stream);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace

bool attn_bf16_supported(int dh, int R) {
  return (dh == 8 && R == 8) || (dh == 16 && R == 16) || (dh == 30 && R == 16) ||
         (dh == 32 && R == 16) || (dh == 16 && R == 32) || (dh == 30 && R == 32);
}

hipError_t launch_attn_bf16_multi(const AttnArgs* calls, int n, hipStream_t stream) {
  if (n < 1 || n > 64) return hipErrorInvalidValue;
  const int dh = calls[0].dh, R = calls[0].R;
  for (int i = 1; i < n; ++i)
    if (calls[i].dh != dh || calls[i].R != R) return hipErrorInvalidValue;
  if (dh == 8 && R == 8) return launch_multi_variant<8, 8>(calls, n, stream);
  if (dh == 16 && R == 16) return launch_multi_variant<16, 16>(calls, n, stream);
  if (dh == 30 && R == 16) return launch_multi_variant<30, 16>(calls, n, stream);
  if (dh == 32 && R == 16) return launch_multi_variant<32, 16>(calls, n, stream);
  if (dh == 16 && R == 32) return launch_multi_variant<16, 32>(calls, n, stream);
  if (dh == 30 && R == 32) return launch_multi_variant<30, 32>(calls, n, stream);
  return hipErrorInvalidValue;
}

template <int DH, int R>
hipError_t launch_lnq_variant(const AttnArgs& a, const LnqArgs& L, hipStream_t stream) {
  const int units = call_units(a), qb = kind_qblocks(a, TILED), grid = kind_grid(a, TILED);
  hipLaunchKernelGGL((attn_bf16_lnq_kernel<DH, R>), dim3(grid), dim3(QB), 0, stream, (const uint32_t*)a.kc,
                     (const uint32_t*)a.v, (const uint32_t*)a.g, a.qp, a.kp, (uint32_t*)a.o, a.B, a.T, a.H, a.W,
                     a.heads, a.wt, a.ws, units * qb, a.tstride, a.lse, (units / a.heads) % 8 == 0 ? 1 : 0, L);
  return hipGetLastError();
}

hipError_t launch_attn_bf16_lnq(const AttnArgs& a, const void* x, const float* gamma, const float* beta,
                                const float* w, const float* bias, float eps, hipStream_t stream) {
  const LnqArgs L{(const uint32_t*)x, gamma, beta, w, bias, eps};
  if (a.dh == 30 && a.R == 16) return launch_lnq_variant<30, 16>(a, L, stream);
  if (a.dh == 16 && a.R == 16) return launch_lnq_variant<16, 16>(a, L, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t stream) {
  if (a.dh == 8 && a.R == 8) return launch_variant<8, 8>(a, stream);
  if (a.dh == 16 && a.R == 16) return launch_variant<16, 16>(a, stream);
  if (a.dh == 30 && a.R == 16) return launch_variant<30, 16>(a, stream);
  if (a.dh == 32 && a.R == 16) return launch_variant<32, 16>(a, stream);
  if (a.dh == 16 && a.R == 32) return launch_variant<16, 32>(a, stream);
  if (a.dh == 30 && a.R == 32) return launch_variant<30, 32>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace rib
