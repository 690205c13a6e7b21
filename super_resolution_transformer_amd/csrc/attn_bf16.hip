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
// Design (one workgroup = 4 waves = 256 queries of one (image, window, head)):
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
//  * Rescaling is lazy: p <= 2^-OFF * 2^(growth of the maximum).  The packed
//    bf16 P values are OR-reduced; bit 14 of a half is set iff p >= 2, i.e.
//    the maximum grew by more than OFF+1 = 8 (a factor 256).  Only then (and on
//    the first tile) does the wave take the slow path: exact row maximum, new
//    m_hat rounded to bf16, recompute, rescale O.
//  * The row sum l comes for free from the PV MFMA: V channel dh is all ones.
//  * Software pipeline over key tiles of KT = 64: iteration i issues the
//    global loads of tile i+1, the QK^T MFMAs of tile i and the exp2/convert
//    work of tile i-1 in one basic block, so the matrix cores, the
//    transcendental unit and the VALU work side by side; then the PV MFMAs of
//    tile i-1 and the LDS store of tile i+1.  Three LDS stages, one barrier
//    per tile.
//  * Window partitioning is index arithmetic on the NHWC arrays: a window's
//    real tokens are enumerated row-major, r = iy*nx + ix, so padded positions
//    are never loaded, and only the last tile can hold padded keys.
//  * Workgroups are numbered so that the q-blocks of one (image, window, head)
//    are consecutive on one XCD (shared K/V in that XCD's L2).
#include "rib_device.hpp"
#include "rib_launch.hpp"

namespace rib {

namespace {

constexpr int KT = 64;             // keys per tile
constexpr int NWAVE = 4;           // waves per workgroup
constexpr int QW = 64;             // queries per wave (two 32-query MFMA blocks)
constexpr int QB = QW * NWAVE;     // queries per workgroup
constexpr int NSTAGE = 3;          // LDS stages of the key-tile pipeline
constexpr float OFF = 7.0f;        // p = exp2(s - m_hat - OFF) <= 2^-OFF normally
constexpr float LOG2E = 1.4426950408889634f;
constexpr uint32_t RSRC_WORD3 = 0x00020000u;  // gfx9 raw buffer: 32-bit data format

template <int DH, int R>
struct Shape {
  static_assert(DH % 2 == 0 && R % 8 == 0, "head dim must be even, rank a multiple of 8");
  static constexpr int KC = (R + DH + 2 + 15) / 16;  // 16-wide contraction chunks
  static constexpr int DT = (DH + 1 + 31) / 32;      // 32-channel output tiles (ones row at DH)
  static constexpr int ROWDW = 8 * KC;               // dwords per Q~/K~ row
  static constexpr int KSTR = ROWDW + 4;             // LDS row stride in dwords (bank spread)
  static constexpr int CONSTDW = R / 2 + DH / 2;     // dword with columns (m, o)
  static constexpr int CM = CONSTDW / 8;             // chunk holding it
  static constexpr int GM = (CONSTDW % 8) / 4;       // lane half holding it
  static constexpr int DM = CONSTDW % 4;             // dword inside the 16-byte operand
  static constexpr int VSTR = 16 * DT + 4;           // dwords per token-major V row in LDS
  static constexpr int KS_DW = KT * KSTR;
  static constexpr int VS_DW = KT * VSTR;
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

struct Geo {
  int H, W, C, ws, b, wy, wx, h, nx, n_real;
  float inv_nx;
};

// real index r of a window -> element offset of the token's head slice and
// in-window index n
template <int DH>
__device__ __forceinline__ void locate(const Geo& G, int r, int& off, int& n) {
  const int iy = (int)(((float)r + 0.5f) * G.inv_nx);
  const int ix = r - iy * G.nx;
  off = ((G.b * G.H + G.wy * G.ws + iy) * G.W + G.wx * G.ws + ix) * G.C + G.h * DH;
  n = iy * G.ws + ix;
}

// ---- staging of one key tile ------------------------------------------------
// Every wave issues the same four 16-byte buffer loads per lane and tile; only
// the wave-uniform buffer descriptor and the offset formula differ:
//   wave 0: the key's positional factor Kp[n][0..16)     (fp32, from kp)
//   wave 1: the key's content slice Kc (dh bf16)          (from kc)
//   wave 2: the key's value slice V (dh bf16)             (from v)
//   wave 3: Kp[n][16..32) when R = 32, otherwise nothing  (zero-length buffer)
// Buffer loads are bounds-checked by the hardware (reads past the descriptor's
// size return 0), so the last head slice of the map may over-read its 16-byte
// chunk safely.  Keeping the load code identical across waves keeps the
// prefetch free of branches, so its latency stays hidden behind the MFMAs;
// all role-specific conversion happens at the LDS store.
struct Stage {
  u32x4_t raw[4];
};

template <int DH, int R>
__device__ __forceinline__ void load_tile(const Geo& G, __amdgpu_buffer_rsrc_t rsrc, int wave, int r,
                                          Stage& st) {
  int off, n;
  locate<DH>(G, r < G.n_real ? r : G.n_real - 1, off, n);
  const bool pos = (wave == 0) | (wave == 3);
  const unsigned voff = pos ? (unsigned)(n * (R * 4) + (wave == 3 ? 64 : 0)) : 2u * (unsigned)off;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    st.raw[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff + 16u * i, 0, 0));
}

__device__ __forceinline__ uint32_t pick(const Stage& st, int w) { return st.raw[w >> 2][w & 3]; }

// Kp fp32 chunks (8 floats) -> 4 packed bf16 dwords
__device__ __forceinline__ u32x4_t kp_to_bf16(const u32x4_t& x, const u32x4_t& y, bool real) {
  const f32x4_t a = __builtin_bit_cast(f32x4_t, x);
  const f32x4_t b = __builtin_bit_cast(f32x4_t, y);
  const u32x4_t out = {pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]), pack_bf16(b[0], b[1]), pack_bf16(b[2], b[3])};
  return real ? out : (u32x4_t){0u, 0u, 0u, 0u};
}

template <int DH, int R>
__device__ __forceinline__ void store_tile(uint32_t* stage, int wave, int j, bool real, const Stage& st) {
  using S = Shape<DH, R>;
  if (wave == 0 || (wave == 3 && R > 16)) {
    // positional columns: dwords [0, R/2) of the K~ row (wave 3: the second half when R = 32)
    uint32_t* dst = stage + j * S::KSTR + (wave == 3 ? 8 : 0);
    constexpr int NQ = (R > 16 ? 16 : R) / 8;
#pragma unroll
    for (int i = 0; i < NQ; ++i)
      *reinterpret_cast<u32x4_t*>(dst + 4 * i) = kp_to_bf16(st.raw[2 * i], st.raw[2 * i + 1], real);
  } else if (wave == 1) {
    // content columns + the (m, o) pair + zero padding: dwords [R/2, ROWDW)
    uint32_t* dst = stage + j * S::KSTR + R / 2;
#pragma unroll
    for (int i = 0; i < (S::ROWDW - R / 2) / 4; ++i) {
      uint32_t d[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int w = 4 * i + e;
        uint32_t val;
        if (w < DH / 2) val = real ? pick(st, w) : 0u;
        else if (w == DH / 2) val = real ? 0x3F803F80u : 0x46800000u;  // (1,1) real, (0,2^14) padded
        else val = 0u;
        d[e] = val;
      }
      *reinterpret_cast<u32x4_t*>(dst + 4 * i) = (u32x4_t){d[0], d[1], d[2], d[3]};
    }
  }
  if (wave == 2 || (wave == 3 && S::DT > 1)) {
    // token-major V row: wave 2 channels [0, 32), wave 3 channels [32, 64)
    uint32_t* dst = stage + S::KS_DW + j * S::VSTR + (wave == 3 ? 16 : 0);
    const int base = wave == 3 ? 16 : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t d[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int w = base + 4 * i + e;
        uint32_t val = (w < DH / 2 && base == 0) ? pick(st, 4 * i + e) : 0u;
        val = w == DH / 2 ? 0x00003F80u : val;  // (1, 0): ones at channel DH
        d[e] = real ? val : 0u;
      }
      *reinterpret_cast<u32x4_t*>(dst + 4 * i) = (u32x4_t){d[0], d[1], d[2], d[3]};
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

template <int DH, int R>
struct Regs {
  using S = Shape<DH, R>;
  f32x16_t O[2][S::DT];
  u32x4_t qt[2][S::KC];
  float mhat[2];
};

// S^T = K~ Q~^T for the tile in `stage` (64 keys x the wave's 64 queries)
template <int DH, int R>
__device__ __forceinline__ void qk_tile(const uint32_t* stage, int l32, int gh, const Regs<DH, R>& rg,
                                        f32x16_t (&Sacc)[2][2]) {
  using S = Shape<DH, R>;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    u32x4_t a[S::KC];
#pragma unroll
    for (int c = 0; c < S::KC; ++c)
      a[c] = *reinterpret_cast<const u32x4_t*>(stage + (kb * 32 + l32) * S::KSTR + 8 * c + 4 * gh);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16_t acc;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
      for (int c = 0; c < S::KC; ++c)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[c]),
                                                      __builtin_bit_cast(bf16x8_t, rg.qt[qb][c]), acc, 0, 0, 0);
      Sacc[qb][kb] = acc;
    }
  }
}

// p = exp2(t - shift) packed to bf16 pairs; returns the OR of all packed words
__device__ __forceinline__ uint32_t exp_tile(const f32x16_t (&Sacc)[2][2], uint32_t (&P)[2][2][8], float shift0,
                                             float shift1) {
  uint32_t orv = 0;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float sh = qb ? shift1 : shift0;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        P[qb][kb][i] = pack_bf16(__builtin_amdgcn_exp2f(Sacc[qb][kb][2 * i] - sh),
                                 __builtin_amdgcn_exp2f(Sacc[qb][kb][2 * i + 1] - sh));
        orv |= P[qb][kb][i];
      }
  }
  return orv;
}

// fast-path exponentials (no shift)
__device__ __forceinline__ uint32_t exp_tile_fast(const f32x16_t (&Sacc)[2][2], uint32_t (&P)[2][2][8]) {
  uint32_t orv = 0;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        P[qb][kb][i] = pack_bf16(__builtin_amdgcn_exp2f(Sacc[qb][kb][2 * i]),
                                 __builtin_amdgcn_exp2f(Sacc[qb][kb][2 * i + 1]));
        orv |= P[qb][kb][i];
      }
  return orv;
}

// Slow path for the tile whose scores are in Sacc: exact row maximum, new
// reference m_hat, exponentials again, rescale of O (unless first), and the
// correction of the already computed next-tile scores Snext by the shift.
template <int DH, int R, bool NEXT>
__device__ __forceinline__ void rescale_tile(Regs<DH, R>& rg, const f32x16_t (&Sacc)[2][2], uint32_t (&P)[2][2][8],
                                             f32x16_t (&Snext)[2][2], bool first, int gh) {
  using S = Shape<DH, R>;
  float shift[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, Sacc[qb][kb][e]);
    const LanePair pr = lane_pair(mx);
    mx = fmaxf(pr.lo, pr.hi);
    const bool grow = first || (mx + OFF > 0.0f);
    const float mnew = grow ? round_bf16(rg.mhat[qb] + mx + OFF) : rg.mhat[qb];
    shift[qb] = mnew - rg.mhat[qb];
    rg.mhat[qb] = mnew;
    if (!first) {
      const float sc = __builtin_amdgcn_exp2f(-shift[qb]);
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) rg.O[qb][dt][e] *= sc;
    }
    const uint32_t cd = pack_bf16(-mnew, -OFF);
    if (gh == S::GM) rg.qt[qb][S::CM][S::DM] = cd;
    if constexpr (NEXT) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) Snext[qb][kb][e] -= shift[qb];
    }
  }
  exp_tile(Sacc, P, shift[0], shift[1]);
}

// O^T += V^T P^T for the tile whose V rows are in `stage`
template <int DH, int R>
__device__ __forceinline__ void pv_tile(const uint32_t* stage, int lane, Regs<DH, R>& rg, const uint32_t (&P)[2][2][8]) {
  using S = Shape<DH, R>;
  const uint32_t* vs = stage + S::KS_DW;
  // transposing read: 16-lane group q = lane/16 covers channels 16*(q%2) + i of the
  // 32-channel tile for keys 4g + k (g = q/2); input lane j = 4k + m addresses
  // channels 16*(q%2) + 4m .. +3 of key 4g + k (+8 for the second read).
  const int j = lane & 15, q = lane >> 4;
  const int key0 = 4 * (q >> 1) + (j >> 2);
  const int ch0 = 16 * (q & 1) + 4 * (j & 3);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      u32x4_t va[S::DT];
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt) {
        const uint32_t* p = vs + (kb * 32 + 16 * c2 + key0) * S::VSTR + ((dt * 32 + ch0) >> 1);
        const u32x2_t lo = ds_read_tr16(p);
        const u32x2_t hi = ds_read_tr16(p + 8 * S::VSTR);
        va[dt] = (u32x4_t){lo[0], lo[1], hi[0], hi[1]};
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const u32x4_t pb = {P[qb][kb][4 * c2], P[qb][kb][4 * c2 + 1], P[qb][kb][4 * c2 + 2], P[qb][kb][4 * c2 + 3]};
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt)
          rg.O[qb][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, va[dt]),
                                                                 __builtin_bit_cast(bf16x8_t, pb), rg.O[qb][dt], 0, 0, 0);
      }
    }
}

template <int DH, int R>
__global__ void __launch_bounds__(QB, 2)
attn_bf16_kernel(const uint32_t* __restrict__ qc, const uint32_t* __restrict__ kc,
                 const uint32_t* __restrict__ v, const uint32_t* __restrict__ g,
                 const float* __restrict__ qp, const float* __restrict__ kp,
                 uint32_t* __restrict__ o, int B, int H, int W, int heads, int ws, int total) {
  using S = Shape<DH, R>;
  __shared__ __attribute__((aligned(16))) uint32_t lds[S::LDS_DW];

  const int logical = xcd_swizzle(blockIdx.x, gridDim.x);
  if (logical >= total) return;
  const int nWy = (H + ws - 1) / ws, nWx = (W + ws - 1) / ws;
  const int qblocks = (ws * ws + QB - 1) / QB;
  Geo G;
  int q0;
  {
    int t = logical;
    const int qblk = t % qblocks; t /= qblocks;
    G.h = t % heads; t /= heads;
    G.wx = t % nWx; t /= nWx;
    G.wy = t % nWy;
    G.b = t / nWy;
    G.H = H; G.W = W; G.C = heads * DH; G.ws = ws;
    G.nx = min(ws, W - G.wx * ws);
    G.n_real = min(ws, H - G.wy * ws) * G.nx;
    G.inv_nx = 1.0f / (float)G.nx;
    q0 = qblk * QB;
    if (q0 >= G.n_real) return;
  }
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int gh = lane >> 5;  // lane half

  // ---- prologue: build the workgroup's Q~ rows in LDS, then pick up the B operands
  {
    const int r = q0 + tid;
    const bool real = r < G.n_real;
    int off, n;
    locate<DH>(G, real ? r : G.n_real - 1, off, n);
    const float sp = LOG2E / sqrtf((float)R);
    const float sc = LOG2E / sqrtf((float)DH);
    uint32_t row[S::ROWDW];
#pragma unroll
    for (int w = 0; w < S::ROWDW; ++w) {
      uint32_t val;
      if (w < R / 2) {
        const float2 pq = *reinterpret_cast<const float2*>(qp + n * R + 2 * w);
        val = pack_bf16(pq.x * sp, pq.y * sp);
      } else if (w < R / 2 + DH / 2) {
        const uint32_t x = qc[(off >> 1) + (w - R / 2)];
        val = pack_bf16(bf16_lo(x) * sc, bf16_hi(x) * sc);
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
  }
  __syncthreads();

  const int ntiles = (G.n_real + KT - 1) / KT;
  const bool active = q0 + wave * QW < G.n_real;
  // this wave's load source (wave-uniform): see load_tile
  const unsigned map_bytes = (unsigned)(B * H * W * heads * DH) * 2u;
  const unsigned pos_bytes = (unsigned)(ws * ws * R) * 4u;
  const void* src = wave == 1 ? (const void*)kc : wave == 2 ? (const void*)v : (const void*)kp;
  const unsigned nbytes = wave == 1 || wave == 2 ? map_bytes : (wave == 0 || R > 16 ? pos_bytes : 0u);
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(src), (short)0, (int)nbytes, (int)RSRC_WORD3);

  // ---- pipeline prologue: tile 0 staged and scored, tile 1 staged
  Stage st;
  load_tile<DH, R>(G, rsrc, wave, lane, st);
  store_tile<DH, R>(lds, wave, lane, lane < G.n_real, st);
  __syncthreads();
  if (ntiles > 1) load_tile<DH, R>(G, rsrc, wave, KT + lane, st);
  f32x16_t SA[2][2], SB[2][2];
  uint32_t P[2][2][8];
  if (active) qk_tile<DH, R>(lds, l32, gh, rg, SA);
  if (ntiles > 1) {
    store_tile<DH, R>(lds + S::STAGE_DW, wave, lane, KT + lane < G.n_real, st);
    __syncthreads();
  }

  // One pipeline step: the scores of tile `it` go into Snew while the softmax
  // and PV of tile it-1 (scores in Sprev) run.  Stages: s_cur holds tile it,
  // the one before it tile it-1, the one after it receives tile it+1.
  int s_cur = 1;
  auto step = [&](int it, f32x16_t (&Sprev)[2][2], f32x16_t (&Snew)[2][2]) {
    const int s_prev = s_cur == 0 ? NSTAGE - 1 : s_cur - 1;
    const int s_next = s_cur == NSTAGE - 1 ? 0 : s_cur + 1;
    const bool more = it + 1 < ntiles;
    if (more) load_tile<DH, R>(G, rsrc, wave, (it + 1) * KT + lane, st);
    if (active) {
      qk_tile<DH, R>(lds + s_cur * S::STAGE_DW, l32, gh, rg, Snew);
      const uint32_t orv = exp_tile_fast(Sprev, P);
      const bool need = (it == 1) || (orv & 0x40004000u);
      if (__builtin_amdgcn_ballot_w64(need)) rescale_tile<DH, R, true>(rg, Sprev, P, Snew, it == 1, gh);
      pv_tile<DH, R>(lds + s_prev * S::STAGE_DW, lane, rg, P);
    }
    if (more) store_tile<DH, R>(lds + s_next * S::STAGE_DW, wave, lane, (it + 1) * KT + lane < G.n_real, st);
    __syncthreads();
    s_cur = s_next;
  };
  // the last tile: softmax + PV only (its scores are in Slast, its stage before s_cur)
  auto finish = [&](f32x16_t (&Slast)[2][2]) {
    if (!active) return;
    const uint32_t orv = exp_tile_fast(Slast, P);
    const bool need = (ntiles == 1) || (orv & 0x40004000u);
    if (__builtin_amdgcn_ballot_w64(need)) rescale_tile<DH, R, false>(rg, Slast, P, Slast, ntiles == 1, gh);
    pv_tile<DH, R>(lds + (s_cur == 0 ? NSTAGE - 1 : s_cur - 1) * S::STAGE_DW, lane, rg, P);
  };
  int it = 1;
  for (; it + 1 < ntiles; it += 2) {
    step(it, SA, SB);
    step(it + 1, SB, SA);
  }
  if (it < ntiles) {
    step(it, SA, SB);
    finish(SB);
  } else {
    finish(SA);  // also the single-tile case
  }

  if (!active) return;
  // ---- epilogue: O / l * sigmoid(G), bf16, NHWC
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int r = q0 + wave * QW + qb * 32 + l32;
    const LanePair pr = lane_pair(rg.O[qb][S::LT][S::LR]);
    const float lsum = S::LG ? pr.hi : pr.lo;
    if (r >= G.n_real) continue;
    const float inv = 1.0f / lsum;
    int off, n;
    locate<DH>(G, r, off, n);
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = dt * 32 + 8 * q4 + 4 * gh;
        if (d0 >= DH) continue;
        const int e0 = 4 * q4;
        const int gw = (off + d0) >> 1;  // dword index of channels (d0, d0+1)
        const uint32_t g01 = g[gw];
        const uint32_t r01 = pack_bf16(rg.O[qb][dt][e0 + 0] * inv * sigmoidf(bf16_lo(g01)),
                                       rg.O[qb][dt][e0 + 1] * inv * sigmoidf(bf16_hi(g01)));
        if (d0 + 4 <= DH) {
          const uint32_t g23 = g[gw + 1];
          const uint32_t r23 = pack_bf16(rg.O[qb][dt][e0 + 2] * inv * sigmoidf(bf16_lo(g23)),
                                         rg.O[qb][dt][e0 + 3] * inv * sigmoidf(bf16_hi(g23)));
          o[gw] = r01;
          o[gw + 1] = r23;
        } else {
          o[gw] = r01;
        }
      }
  }
}

template <int DH, int R>
hipError_t launch_variant(const AttnArgs& a, hipStream_t stream) {
  const int nWy = (a.H + a.ws - 1) / a.ws, nWx = (a.W + a.ws - 1) / a.ws;
  const int qblocks = (a.ws * a.ws + QB - 1) / QB;
  const int total = a.B * nWy * nWx * a.heads * qblocks;
  const int grid = 8 * ((total + 7) / 8);
  hipLaunchKernelGGL((attn_bf16_kernel<DH, R>), dim3(grid), dim3(QB), 0, stream,
                     (const uint32_t*)a.qc, (const uint32_t*)a.kc, (const uint32_t*)a.v,
                     (const uint32_t*)a.g, a.qp, a.kp, (uint32_t*)a.o, a.B, a.H, a.W, a.heads, a.ws,
                     total);
  return hipGetLastError();
}

}  // namespace

bool attn_bf16_supported(int dh, int R) {
  return (dh == 8 && R == 8) || (dh == 16 && R == 16) || (dh == 30 && R == 16) ||
         (dh == 32 && R == 16) || (dh == 16 && R == 32) || (dh == 30 && R == 32);
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
