// cla_gate.hip -- the gate producer of Convolutional Local Attention (gfx950).
//
// The gating map of CLA comes from a depth-wise separable convolution of the
// block input (omica.com.cn explainer section 2.3: G = PWConv(DWConv3x3(X));
// gist.science summaries part B: depth-wise 3x3 then point-wise 1x1):
//   D[b,y,x,c] = dw_b[c] + sum_{dy,dx} X[b,y+dy,x+dx,c] * dw_w[c][dy+1][dx+1]
//                (zero padding, stride 1: G keeps the map's shape)
//   G[b,y,x,o] = pw_b[o] + sum_c D[b,y,x,c] * pw_w[c][o]
// on NHWC maps.  G then gates the attention output element-wise.
//
// Design: persistent workgroups (one wave per 32-channel output block, at least
// four), as many as fit on the chip at once, each take one contiguous range of
// tiles of 32 tokens (one segment of a map row), numbered so that a range walks
// down 32-token columns of the map.  The input row segments (with a one-token
// halo on each side) live in a ring of four LDS row buffers, loaded straight
// into LDS (buffer loads with the LDS destination, so a whole row is in flight
// without registers), one token per 16-byte-aligned LDS slot, tokens outside
// the map as zeros.  A tile reads rows y-1, y, y+1 from three of the buffers
// while the row y+2 of the next tile lands in the fourth: every input row is
// loaded once per column range instead of once for each of the three tiles
// that read it, and its latency hides behind a whole tile.
// Phase 1 computes the depth-wise stencil from LDS with v_dot2_f32_bf16 (bf16
// taps and inputs, exact products, fp32 sums): each thread owns one channel
// pair, keeps its taps in registers and walks a run of 8 consecutive tokens,
// so every input column is read and permuted once; it writes D, rounded to
// bf16, into a D tile.
// Phase 2 is the point-wise product as G^T = W_pw^T D^T on
// v_mfma_f32_32x32x16_bf16: each wave keeps its 32-channel output blocks of
// W_pw^T as A operands in VGPRs for the whole launch and reads the B operands
// (8 channels of one token per lane) from the D tile; in the accumulator each
// lane holds one token and 4 groups of 4 consecutive output channels (the
// accumulator starts from their biases), which are rounded and written into an
// LDS output tile; the tile's tokens are one contiguous span of G, stored with
// 16-byte writes.  The two phases are software-pipelined: a step computes the
// stencil of one tile while the matrix core runs the point-wise product of the
// previous one, and stores the tile before that.  The fp32 path keeps the
// weights and D in fp32 and does the point-wise sum with FMAs.
#include "rib_device.hpp"
#include "rib_launch.hpp"

namespace rib {

namespace {

constexpr int GT = 32;          // tokens per tile
constexpr int GTHREADS = 256;   // four waves
constexpr int GCMAX = 256;      // largest channel count

__device__ __forceinline__ void tile_coords(long tile, int nseg, int H, int& b, int& y, int& x0) {
  const int seg = (int)(tile % nseg);
  const long t2 = tile / nseg;
  y = (int)(t2 % H);
  b = (int)(t2 / H);
  x0 = seg * GT;
}

// ---------------------------------------------------------------- fp32
__global__ void __launch_bounds__(GTHREADS)
cla_gate_f32_kernel(const float* __restrict__ x, const float* __restrict__ dw_w, const float* __restrict__ dw_b,
                    const float* __restrict__ pw_w, const float* __restrict__ pw_b, float* __restrict__ g,
                    int B, int H, int W, int C, int nseg, long ntiles) {
  __shared__ float d[GT * GCMAX];
  for (long tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    int b, y, x0;
    tile_coords(tile, nseg, H, b, y, x0);
    for (int e = threadIdx.x; e < GT * C; e += GTHREADS) {
      const int t = e / C, c = e - t * C;
      const int xx = x0 + t;
      float acc = 0.0f;
      if (xx < W) {
        acc = dw_b[c];
        for (int dy = -1; dy <= 1; ++dy)
          for (int dx = -1; dx <= 1; ++dx) {
            const int yy = y + dy, xs = xx + dx;
            if (yy < 0 || yy >= H || xs < 0 || xs >= W) continue;
            acc = fmaf(x[(((long)b * H + yy) * W + xs) * C + c], dw_w[c * 9 + (dy + 1) * 3 + (dx + 1)], acc);
          }
      }
      d[t * GCMAX + c] = acc;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < GT * C; e += GTHREADS) {
      const int t = e / C, o = e - t * C;
      const int xx = x0 + t;
      if (xx >= W) continue;
      float acc = pw_b[o];
      for (int c = 0; c < C; ++c) acc = fmaf(d[t * GCMAX + c], pw_w[c * C + o], acc);
      g[(((long)b * H + y) * W + xx) * C + o] = acc;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- bf16
// NB = 32-channel output blocks (C <= 32*NB); NW = max(4, NB) waves, wave w owns output
// block w.  Phase 1 splits the tile into 4 runs of 8 tokens: thread (pair cp, run) with
// 16*NW >= C/2 threads per run.
template <int NB>
struct GateShape {
  static constexpr int NW = NB > 4 ? 8 : 4;   // waves per workgroup (2 per SIMD for wide maps)
  static constexpr int NT = 64 * NW;          // threads
  static constexpr int KCH = 2 * NB;          // 16-channel contraction chunks
  static constexpr int DSTR = 8 * KCH + 4;    // dwords per token row of the D tile (bank spread)
  static constexpr int XT = GT + 2;           // tokens of an input row segment (left/right halo)
  // one input row segment as 16-byte chunks (at most XT tokens of 16*NB dwords), loaded in
  // NPASS passes of NT lanes; a wave's 64 chunks of a pass are loaded only if the first is
  // in the row, so a buffer holds the row's chunks rounded up to 64
  static constexpr int NPASS = (XT * 4 * NB + NT - 1) / NT;
  static constexpr int ROW_DW = (XT * 4 * NB + 63) / 64 * 64 * 4;
  static constexpr int OS_DW = GT * 16 * NB;  // output tile, NHWC order
  static constexpr int TPR = 16 * NW;         // phase-1 threads per run
  static constexpr int NRUN = GT / 4;         // tokens per run
};

// Row ring: the input rows y-1, y, y+1 of the current tile and the prefetched row y+2 live
// in four LDS arrays.  Separate arrays (not one indexed array) let the compiler see that
// reading three of them never waits for the copies into the fourth.
#define GATE_RING(I) ((I) == 0 ? rb0 : (I) == 1 ? rb1 : (I) == 2 ? rb2 : rb3)

template <int NB>
__global__ void __launch_bounds__(GateShape<NB>::NT, 2)
cla_gate_bf16_kernel(const uint32_t* __restrict__ x, const float* __restrict__ dw_w,
                     const float* __restrict__ dw_b, const float* __restrict__ pw_w,
                     const float* __restrict__ pw_b, uint32_t* __restrict__ g, int B, int H, int W, int C,
                     int nseg, long ntiles) {
  using S = GateShape<NB>;
  constexpr int XT = S::XT, KCH = S::KCH, DSTR = S::DSTR, NRUN = S::NRUN, NPASS = S::NPASS;
  __shared__ __attribute__((aligned(16))) uint32_t dt0[GT * DSTR];  // D tiles, by tile parity
  __shared__ __attribute__((aligned(16))) uint32_t dt1[GT * DSTR];
  __shared__ __attribute__((aligned(16))) uint32_t rb0[S::ROW_DW];
  __shared__ __attribute__((aligned(16))) uint32_t rb1[S::ROW_DW];
  __shared__ __attribute__((aligned(16))) uint32_t rb2[S::ROW_DW];
  __shared__ __attribute__((aligned(16))) uint32_t rb3[S::ROW_DW];
  __shared__ __attribute__((aligned(16))) uint32_t ot0[S::OS_DW];  // output tiles, by tile parity
  __shared__ __attribute__((aligned(16))) uint32_t ot1[S::OS_DW];
  __shared__ __attribute__((aligned(16))) float pbias[GCMAX];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int gh = lane >> 5;
  const int CP = C >> 1;  // channel pairs
  // C in 162..192 (NB = 6): the product runs as 16x16x32 blocks, each of the 8 waves taking
  // one 16-token half of the tile (th) and three 16-channel output blocks (3 g4 .. 3 g4 + 2),
  // so every SIMD issues the same matrix-core work and a wave reads half of the D tile.
  // Otherwise wave w owns the 32-channel output block w (32x32x16 blocks).
  constexpr bool SPLIT = NB == 6;
  constexpr int NWA = SPLIT ? 3 * NB : KCH;  // A operands held by a wave
  const int th = wave >> 2, g4 = wave & 3, l16 = lane & 15, kg = lane >> 4;
  const bool has_block = SPLIT ? true : (wave < NB && wave * 32 < C);

  // ---- point-wise weights as A operands of this wave's output block: row = output
  // channel, 8 input channels per lane
  u32x4_t wa[NWA];
  if constexpr (SPLIT) {
    // operand m = j NB + ks: output channel 16 (3 g4 + j) + l16, input channels 32 ks + 8 kg ..
#pragma unroll
    for (int m = 0; m < NWA; ++m) {
      const int o = 16 * (3 * g4 + m / NB) + l16;
      uint32_t w4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 32 * (m % NB) + 8 * kg + 2 * i;
        const float a = (o < C && c < C) ? pw_w[c * C + o] : 0.0f;
        const float b2 = (o < C && c + 1 < C) ? pw_w[(c + 1) * C + o] : 0.0f;
        w4[i] = pack_bf16(a, b2);
      }
      wa[m] = (u32x4_t){w4[0], w4[1], w4[2], w4[3]};
    }
  } else {
    const int o = wave * 32 + l32;
#pragma unroll
    for (int kc = 0; kc < KCH; ++kc) {
      uint32_t w4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 16 * kc + 8 * gh + 2 * i;
        const float a = (has_block && o < C && c < C) ? pw_w[c * C + o] : 0.0f;
        const float b2 = (has_block && o < C && c + 1 < C) ? pw_w[(c + 1) * C + o] : 0.0f;
        w4[i] = pack_bf16(a, b2);
      }
      wa[kc] = (u32x4_t){w4[0], w4[1], w4[2], w4[3]};
    }
  }
  // the product's accumulator: one 32x32 block, or three 16x16 blocks
  struct AccSplit { f32x4_t a[3]; };
  using Acc = std::conditional_t<SPLIT, AccSplit, f32x16_t>;

  // ---- depth-wise taps of this thread's channel pair (channel 2cp + h); it computes tokens
  // t0 .. t0+NRUN-1.  The taps are bf16 operands of v_dot2_f32_bf16: w01[h][j] holds the
  // taps of rows y-1 and y in input column j (x-1, x, x+1), w2[h][j] the row y+1 tap in
  // half h and zero in the other half, so that it can be dotted with the input word of the
  // channel pair as read
  const int cp = tid % S::TPR;
  const int t0 = (tid / S::TPR) * NRUN;
  const bool has_pair = cp < CP;
  uint32_t w01[2][3], w2[2][3];
  float tb[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = 2 * cp + h;
    float tap[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) tap[k] = has_pair ? dw_w[c * 9 + k] : 0.0f;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      w01[h][j] = pack_bf16(tap[j], tap[3 + j]);
      w2[h][j] = h == 0 ? pack_bf16(tap[6 + j], 0.0f) : pack_bf16(0.0f, tap[6 + j]);
    }
    tb[h] = has_pair ? dw_b[c] : 0.0f;
  }
  // contraction channels [C, 16*KCH) stay zero in the D tile
  for (int e = tid; e < GT * (8 * KCH - CP); e += S::NT) {
    const int t = e / (8 * KCH - CP), p = CP + e % (8 * KCH - CP);
    dt0[t * DSTR + p] = 0u;
    dt1[t * DSTR + p] = 0u;
  }
  for (int o = tid; o < GCMAX; o += S::NT) pbias[o] = o < C ? pw_b[o] : 0.0f;

  // Input staging: an LDS row buffer holds tokens x0-1 .. x0+GT of one map row as 16-byte
  // chunks, chunk f = token * CH + k at dwords 4f, one token every TS dwords (C/2 rounded up
  // to 4) so that a chunk never spans two tokens.  The chunks are loaded straight into LDS
  // (buffer_load ... lds: lane l of a wave writes base + 16 l), so a whole row is in flight
  // without registers; rows and tokens outside the map get an out-of-range offset, which the
  // buffer bounds check turns into zeros.
  const int TS = (CP + 3) & ~3;
  const int CH = TS >> 2;  // chunks per token
  const int NCHK = XT * CH;
  const float inv_ch = 1.0f / (float)CH;
  const unsigned map_bytes = (unsigned)((long)B * H * W * C * 2);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(x), (short)0,
                                                                      (int)map_bytes, 0x00020000);
  // Per-lane chunk geometry is the same for every row: for pass j of this wave, chunk
  // f = wave*64 + j*NT + lane is sub-chunk k of token p (-1: past the row), at byte offset
  // pre[j] from the row's first token.
  int ptok[NPASS];
  unsigned pre[NPASS];
#pragma unroll
  for (int j = 0; j < NPASS; ++j) {
    const int f = wave * 64 + j * S::NT + lane;
    const int q = (int)(((float)f + 0.5f) * inv_ch);  // token (exact: f < 2^16)
    const int k = f - q * CH;
    ptok[j] = f < NCHK ? q : -1;
    pre[j] = (unsigned)((q * CP + 4 * k) * 4);
  }
  auto issue_row = [&](uint32_t* dst, int b, int yrow, int x0) {
    const bool row_ok = yrow >= 0 && yrow < H;
    const long base = ((((long)b * H + yrow) * W + (x0 - 1)) * CP) * 4;  // may be negative
#pragma unroll
    for (int j = 0; j < NPASS; ++j) {
      if (wave * 64 + j * S::NT >= NCHK) break;  // wave-uniform
      const int xt = x0 - 1 + ptok[j];
      const bool valid = row_ok && ptok[j] >= 0 && xt >= 0 && xt < W;
      const unsigned off = valid ? (unsigned)(base + (long)pre[j]) : 0xFFFFFFF0u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)(dst + 4 * (wave * 64 + j * S::NT)),
                                               16, off, 0, 0, 0);
    }
  };


  // the product's pieces: accumulators from the bias, and product m of the wave's NWA
  auto acc_init = [&](Acc& acc) {
    if constexpr (SPLIT) {
#pragma unroll
      for (int j = 0; j < 3; ++j)
        acc.a[j] = *reinterpret_cast<const f32x4_t*>(pbias + 16 * (3 * g4 + j) + 4 * kg);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4_t bq = *reinterpret_cast<const f32x4_t*>(pbias + wave * 32 + 8 * q + 4 * gh);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[4 * q + e] = bq[e];
      }
    }
  };
  auto mma_step = [&](const uint32_t* dt, int m, Acc& acc) {
    if constexpr (SPLIT) {
      // B operand: token 16 th + l16, input channels 32 ks + 8 kg .. +7
      const int ks = m % NB;
      const u32x4_t bo = *reinterpret_cast<const u32x4_t*>(dt + (16 * th + l16) * DSTR + 16 * ks + 4 * kg);
      acc.a[m / NB] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wa[m]),
                                                             __builtin_bit_cast(bf16x8_t, bo), acc.a[m / NB], 0, 0, 0);
    } else {
      const u32x4_t bo = *reinterpret_cast<const u32x4_t*>(dt + l32 * DSTR + 8 * m + 4 * gh);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, wa[m]),
                                                    __builtin_bit_cast(bf16x8_t, bo), acc, 0, 0, 0);
    }
  };

  // ---- one tile's stencil, with the point-wise product of the previous tile spread over it.
  // Phase 1: D = depth-wise 3x3 of the tile over this thread's run (bf16 products with fp32
  // accumulation, six v_dot2_f32_bf16 per channel and token), rounded to bf16 into a D tile;
  // a column of three input words is read and permuted once and used by three tokens.  Phase 2 (MMA): G^T = W_pw^T D^T of the previous tile for this wave's
  // output block, started from the bias, its KCH matrix-core products issued one or two per
  // token of the run so that they execute while the wave's vector work goes on.  Threads
  // without a channel pair read pair 0 (one broadcast address) and store nothing.  The
  // token loop has no branches.
  auto work = [&](auto mma_c, const uint32_t* up, const uint32_t* mid, const uint32_t* dn, uint32_t* dtw,
                  const uint32_t* dtr, Acc& acc) {
    constexpr bool MMA = decltype(mma_c)::value;
    // the run's NRUN + 2 input columns, all read up front so that no token waits for LDS
    const int cpr = has_pair ? cp : 0;
    uint32_t raw[NRUN + 2][3];
#pragma unroll
    for (int p = 0; p < NRUN + 2; ++p) {
      raw[p][0] = up[(t0 + p) * TS + cpr];
      raw[p][1] = mid[(t0 + p) * TS + cpr];
      raw[p][2] = dn[(t0 + p) * TS + cpr];
    }
    if constexpr (MMA) acc_init(acc);
    // an input column as dot-product operands: lo = (row y-1, row y) of channel 2cp, hi = the
    // same of channel 2cp+1 (one byte permute each), r2 = the row y+1 word as read
    struct Col { uint32_t lo, hi, r2; };
    auto column = [&](int p) {
      return Col{__builtin_amdgcn_perm(raw[p][1], raw[p][0], 0x05040100u),
                 __builtin_amdgcn_perm(raw[p][1], raw[p][0], 0x07060302u), raw[p][2]};
    };
    auto dot2 = [](uint32_t a, uint32_t b, float c) {
      return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                             false);
    };
    Col c0 = column(0), c1 = column(1);
    uint32_t dv[NRUN];
#pragma unroll
    for (int i = 0; i < NRUN; ++i) {
      if constexpr (MMA) {
#pragma unroll
        for (int m = i; m < NWA; m += NRUN) mma_step(dtr, m, acc);
      }
      const Col c2 = column(i + 2);
      float a0 = tb[0], a1 = tb[1];
      a0 = dot2(c0.lo, w01[0][0], a0);
      a1 = dot2(c0.hi, w01[1][0], a1);
      a0 = dot2(c1.lo, w01[0][1], a0);
      a1 = dot2(c1.hi, w01[1][1], a1);
      a0 = dot2(c2.lo, w01[0][2], a0);
      a1 = dot2(c2.hi, w01[1][2], a1);
      a0 = dot2(c0.r2, w2[0][0], a0);
      a1 = dot2(c0.r2, w2[1][0], a1);
      a0 = dot2(c1.r2, w2[0][1], a0);
      a1 = dot2(c1.r2, w2[1][1], a1);
      a0 = dot2(c2.r2, w2[0][2], a0);
      a1 = dot2(c2.r2, w2[1][2], a1);
      c0 = c1;
      c1 = c2;
      dv[i] = pack_bf16(a0, a1);
    }
    // tokens past the map's right edge get a value too: their G rows are never stored
    if (has_pair) {
#pragma unroll
      for (int i = 0; i < NRUN; ++i) dtw[(t0 + i) * DSTR + cp] = dv[i];
    }
  };
  // phase 2 alone (the last tile of a column range): products from the bias start
  auto pointwise = [&](const uint32_t* dt, Acc& acc) {
    acc_init(acc);
#pragma unroll
    for (int m = 0; m < NWA; ++m) mma_step(dt, m, acc);
  };
  // the accumulator rounded into an output tile (NHWC order: token row t holds C/2 dwords)
  // (with C % 4 == 0 the row stride C/2 and oc/2 are even: a pair of dwords is one aligned
  // 8-byte write; otherwise two 4-byte writes)
  auto put = [&](const Acc& acc, uint32_t* ot) {
    const bool pair8 = (CP & 1) == 0;
    // four consecutive outputs oc .. oc+3 of one token
    auto put4 = [&](uint32_t* orow, int oc, float v0, float v1, float v2, float v3) {
      const uint32_t lo = pack_bf16(v0, v1);
      const uint32_t hi = pack_bf16(v2, v3);
      if (pair8 && oc + 2 < C) {
        *reinterpret_cast<u32x2_t*>(orow + (oc >> 1)) = (u32x2_t){lo, hi};
      } else {
        if (oc < C) orow[oc >> 1] = lo;
        if (oc + 2 < C) orow[(oc >> 1) + 1] = hi;
      }
    };
    if constexpr (SPLIT) {
      uint32_t* orow = ot + (16 * th + l16) * CP;
#pragma unroll
      for (int j = 0; j < 3; ++j)
        put4(orow, 16 * (3 * g4 + j) + 4 * kg, acc.a[j][0], acc.a[j][1], acc.a[j][2], acc.a[j][3]);
    } else {
      uint32_t* orow = ot + l32 * CP;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        put4(orow, wave * 32 + 8 * q + 4 * gh, acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
    }
  };
  // an output tile's tokens are one contiguous span of G: 16-byte stores
  auto store = [&](const uint32_t* ot, int b, int y, int x0) {
    const int ntok = min(GT, W - x0);
    const int ndw = ntok * CP;
    uint32_t* gs = g + (((long)b * H + y) * W + x0) * CP;
    for (int c4 = tid; 4 * c4 < ndw; c4 += S::NT) {
      const int d = 4 * c4;
      if (d + 4 <= ndw) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ot + d);
        *reinterpret_cast<u32x4_t*>(gs + d) = v;
      } else {
        for (int i = d; i < ndw; ++i) gs[i] = ot[i];
      }
    }
  };

  // One step of the pipeline, for tile i (output row y) of a column range: the stencil of
  // tile i, the point-wise product of tile i-1 and the stores of tile i-2.  The product's
  // matrix-core work is issued first and runs while the same waves compute the stencil on
  // the vector units.  Rows y-1, y, y+1 have landed; the row y+2 of tile i+1 (if this
  // workgroup computes it) is loaded meanwhile.  Tile i's D and output tiles are dt and ot
  // of parity (i+1) & 1 = K & 1 with K = (i+1) mod 4, the ring rotation.  One barrier per
  // step (before it) orders everything: every LDS array written in a step is read only in
  // a later step, and every array read in a step is rewritten only in a later one.
  auto step = [&](auto kc, int b, int y, int x0, bool more, bool prev, bool prev2) {
    constexpr int K = decltype(kc)::value;
    uint32_t* dtw = (K & 1) ? dt1 : dt0;
    const uint32_t* dtr = (K & 1) ? dt0 : dt1;
    uint32_t* otw = (K & 1) ? ot0 : ot1;
    const uint32_t* otr = (K & 1) ? ot1 : ot0;
    if (more) issue_row(GATE_RING((K + 2) & 3), b, y + 2, x0);  // that array held row y-2
    if (prev2) store(otr, b, y - 2, x0);
    const uint32_t* up = GATE_RING((K + 3) & 3);
    const uint32_t* mid = GATE_RING(K);
    const uint32_t* dn = GATE_RING((K + 1) & 3);
    Acc acc;
    if (prev && has_block) {  // wave-uniform
      work(std::true_type{}, up, mid, dn, dtw, dtr, acc);
      put(acc, otw);
    } else {
      work(std::false_type{}, up, mid, dn, dtw, dtr, acc);
    }
  };

  // Tiles are numbered column by column: tile t is row t mod H of column t / H, a column
  // being one 32-token segment of one image.  Each workgroup takes one contiguous range of
  // tiles and walks down its columns, so every input row is loaded once per column range
  // (plus one halo row above and below), not once per tile that reads it.
  const long t_begin = (long)blockIdx.x * ntiles / gridDim.x;
  const long t_end = (long)(blockIdx.x + 1) * ntiles / gridDim.x;
  long t = t_begin;
  while (t < t_end) {
    const long col = t / H;
    const int y0 = (int)(t - col * H);
    const int b = (int)(col / nseg);
    const int x0 = (int)(col - (long)b * nseg) * GT;
    const int yend = (int)min((long)H, y0 + (t_end - t));
    // all waves are past the previous column's last step, whose stencil ended the row reads;
    // row r sits in ring array (r - y0 + 1) mod 4 for this column range, so the steps take
    // the arrays in a fixed rotation (straight-line code: each step's arrays are known
    // statically)
    issue_row(rb0, b, y0 - 1, x0);
    issue_row(rb1, b, y0, x0);
    issue_row(rb2, b, y0 + 1, x0);
    int y = y0;
    for (;;) {
      __builtin_amdgcn_s_waitcnt(0);  // this wave's rows have landed (and its last stores)
      __syncthreads();
      step(std::integral_constant<int, 1>{}, b, y, x0, y + 1 < yend, y > y0, y > y0 + 1);
      if (++y >= yend) break;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      step(std::integral_constant<int, 2>{}, b, y, x0, y + 1 < yend, y > y0, y > y0 + 1);
      if (++y >= yend) break;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      step(std::integral_constant<int, 3>{}, b, y, x0, y + 1 < yend, y > y0, y > y0 + 1);
      if (++y >= yend) break;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      step(std::integral_constant<int, 0>{}, b, y, x0, y + 1 < yend, y > y0, y > y0 + 1);
      if (++y >= yend) break;
    }
    // drain: with n = yend - y0 tiles, the last (n-1) still needs its point-wise product and
    // both the last two their stores; tile i's arrays have parity (i+1) & 1
    const int n = yend - y0;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (n >= 2) store((n & 1) ? ot0 : ot1, b, yend - 2, x0);
    if (has_block) {
      Acc acc;
      pointwise((n & 1) ? dt1 : dt0, acc);
      put(acc, (n & 1) ? ot1 : ot0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    store((n & 1) ? ot1 : ot0, b, yend - 1, x0);
    t = (long)col * H + yend;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
}

#undef GATE_RING


template <int NB>
hipError_t launch_gate_bf16(const GateArgs& a, int nseg, long ntiles, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((cla_gate_bf16_kernel<NB>), dim3(grid), dim3(GateShape<NB>::NT), 0, stream, (const uint32_t*)a.x,
                     a.dw_w, a.dw_b, a.pw_w, a.pw_b, (uint32_t*)a.g, a.B, a.H, a.W, a.C, nseg, ntiles);
  return hipGetLastError();
}

}  // namespace

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      n > 0)
    return n;
  return 256;
}

hipError_t launch_cla_gate(const GateArgs& a, bool bf16, hipStream_t stream) {
  const int nseg = (a.W + GT - 1) / GT;
  const long ntiles = (long)a.B * a.H * nseg;
  if (!bf16) {
    const long cap = 2L * device_cus();
    const int grid = (int)(ntiles < cap ? ntiles : cap);
    hipLaunchKernelGGL(cla_gate_f32_kernel, dim3(grid), dim3(GTHREADS), 0, stream, (const float*)a.x, a.dw_w,
                       a.dw_b, a.pw_w, a.pw_b, (float*)a.g, a.B, a.H, a.W, a.C, nseg, ntiles);
    return hipGetLastError();
  }
  // bf16: persistent workgroups, as many as are resident at once (two per CU up to 128
  // channels, one beyond: LDS and registers), each walking a contiguous range of tiles
  const int nb = (a.C + 31) / 32;
  const long cap = (nb > 4 ? 1L : 2L) * device_cus();
  const int grid = (int)(ntiles < cap ? ntiles : cap);
  switch (nb) {
    case 1: return launch_gate_bf16<1>(a, nseg, ntiles, grid, stream);
    case 2: return launch_gate_bf16<2>(a, nseg, ntiles, grid, stream);
    case 3: return launch_gate_bf16<3>(a, nseg, ntiles, grid, stream);
    case 4: return launch_gate_bf16<4>(a, nseg, ntiles, grid, stream);
    case 5: return launch_gate_bf16<5>(a, nseg, ntiles, grid, stream);
    case 6: return launch_gate_bf16<6>(a, nseg, ntiles, grid, stream);
    case 7: return launch_gate_bf16<7>(a, nseg, ntiles, grid, stream);
    case 8: return launch_gate_bf16<8>(a, nseg, ntiles, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rib
