// ln_qkv.hip -- the block input projection that produces the attention's
// operands: LayerNorm over the channels of each token, then one linear map
// C -> 3C (omica.com.cn explainer section 3.1: an SST block runs LayerNorm,
// then the RIB attention; the attention's Q, K and V are projections of the
// normalised block input):
//   mu = mean_c x_c,  var = mean_c (x_c - mu)^2,  xn = (x - mu)/sqrt(var + eps)*gamma + beta
//   [q | k | v] = xn W + b,  W [C][3C] row-major (y = x W)
// q, k, v (and optionally xn, the gate producer's input) are NHWC maps.
//
// bf16 path (C % 4 == 0, C <= 192): persistent workgroups of 8 waves walk
// tiles of 32 consecutive tokens.  Each wave keeps its 16-output blocks of W^T
// (rounded to bf16; block b belongs to wave b % 8) in VGPRs for the whole
// launch; a tile is
//   1. copied into LDS with buffer_load ... lds (16 bytes per lane, 64C bytes
//      per tile, the next tile's copy in flight during this tile's work);
//   2. normalised in fp32, 16 threads per token, into a chunk-major B-operand
//      tile (8 channels = 16 bytes per chunk, 32 tokens per chunk, padded so
//      the MFMA operand reads are free of bank conflicts);
//   3. multiplied: y^T = W^T xn^T with v_mfma_f32_16x16x32_bf16 on blocks of
//      16 outputs x 16 tokens (lane = token, 4 consecutive outputs per lane);
//   4. biased, rounded to bf16 and written through an LDS output tile, so
//      that each of q, k, v (and xn) leaves as one contiguous span of the
//      map with 16-byte stores.
// Everything else (fp32 maps, other C) takes a plain kernel: LayerNorm of 16
// tokens into LDS in fp32, then one output per thread with fp32 FMAs.
#include "rib_device.hpp"
#include "rib_launch.hpp"

namespace rib {

namespace {

constexpr int LQ_TT = 32;          // tokens per tile
constexpr int LQ_NW = 8;           // waves per workgroup
constexpr int LQ_NT = 64 * LQ_NW;  // threads per workgroup
constexpr uint32_t RSRC_WORD3 = 0x00020000u;

template <int KC>  // KC = 32-channel steps of the contraction (C rounded up to 32)
struct LqShape {
  static constexpr int KP = 32 * KC;                 // padded channels
  static constexpr int BCS = 4 * LQ_TT + 16;         // dwords between 8-channel chunks of the B tile
  static constexpr int B_DW = 4 * KC * BCS;          // B-operand tile
  static constexpr int XT_DW = LQ_TT * KP / 2;       // one X tile (bf16, token-major, up to KP channels)
  static constexpr int O_DW = 3 * LQ_TT * KP / 2;    // output tile q | k | v (token-major per part)
};

__device__ __forceinline__ f32x4_t lq_mfma(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// Sum over the 16 lanes of a DPP row (lanes 16k .. 16k+15), result in every lane of the row:
// swap within pairs, then within quads, then mirror the half-row (quad 0 <-> quad 1) and the
// row (half 0 <-> half 1).  Four DPP-modified adds, no LDS round trip.
__device__ __forceinline__ float row16_sum(float v) {
  auto dpp = [](float x, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 decltype(ctrl)::value, 0xF, 0xF, false));
  };
  v += dpp(v, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
  v += dpp(v, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
  v += dpp(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
  v += dpp(v, std::integral_constant<int, 0x140>{});  // row_mirror
  return v;
}

// Wait until at most n of this wave's vector memory operations are in flight
// (they complete in issue order): the next tile's copies are issued before the
// current tile's output stores, so waiting for the copies leaves the stores
// in flight.
__device__ __forceinline__ void lq_wait_vm(int n) {
  switch (n) {  // vmcnt(n), expcnt and lgkmcnt unconstrained
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
    case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
    case 11: __builtin_amdgcn_s_waitcnt(0x0F7B); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;  // n == 0, or more than tracked: wait for all
  }
}

// NBW = output blocks of 16 per wave (wave w owns blocks w, w + 8, ...)
template <int KC, int NBW>
__global__ void __launch_bounds__(LQ_NT, 1)
ln_qkv_bf16_kernel(const uint32_t* __restrict__ x, const float* __restrict__ gamma, const float* __restrict__ beta,
                   const float* __restrict__ w, const float* __restrict__ bias, uint32_t* __restrict__ q,
                   uint32_t* __restrict__ k, uint32_t* __restrict__ v, uint32_t* __restrict__ xn, long ntok, int C,
                   float eps) {
  using S = LqShape<KC>;
  // two X tile buffers as separate LDS objects: the loop below alternates them at compile time, so
  // the compiler can see that a copy in flight into one never aliases the reads of the other
  __shared__ __attribute__((aligned(16))) uint32_t s_xa[S::XT_DW];
  __shared__ __attribute__((aligned(16))) uint32_t s_xb[S::XT_DW];
  __shared__ __attribute__((aligned(16))) uint32_t s_b[S::B_DW];
  __shared__ __attribute__((aligned(16))) uint32_t s_o[S::O_DW];
  __shared__ __attribute__((aligned(16))) float s_gb[2][S::KP];
  __shared__ __attribute__((aligned(16))) float s_bias[3 * S::KP];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int C3 = 3 * C;
  const long ntiles = (ntok + LQ_TT - 1) / LQ_TT;
  const unsigned tile_bytes = (unsigned)(LQ_TT * C * 2);
  const unsigned map_bytes = (unsigned)(ntok * C * 2);  // < 2^31, checked by the caller
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(x), (short)0,
                                                                      (int)map_bytes, (int)RSRC_WORD3);

  // ---- once: W^T blocks in VGPRs (bf16, zero past C and 3C), affine and bias in LDS, B tile padding zero
  // A operand of block b, step kc: lane = (output 16b + l16, channels 32kc + 8g .. +7)
  u32x4_t wa[NBW][KC];
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int o = 16 * (wave + LQ_NW * i) + l16;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      uint32_t d[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int c0 = 32 * kc + 8 * g + 2 * p;
        const float w0 = (o < C3 && c0 < C) ? w[(long)c0 * C3 + o] : 0.0f;
        const float w1 = (o < C3 && c0 + 1 < C) ? w[(long)(c0 + 1) * C3 + o] : 0.0f;
        d[p] = pack_bf16(w0, w1);
      }
      wa[i][kc] = (u32x4_t){d[0], d[1], d[2], d[3]};
    }
  }
  for (int c = tid; c < S::KP; c += LQ_NT) {
    s_gb[0][c] = c < C ? gamma[c] : 0.0f;
    s_gb[1][c] = c < C ? beta[c] : 0.0f;
  }
  for (int o = tid; o < 3 * S::KP; o += LQ_NT) s_bias[o] = o < C3 ? bias[o] : 0.0f;
  for (int i = tid; i < S::B_DW; i += LQ_NT) s_b[i] = 0u;

  // copy of tile `tile` into X buffer `xbuf`: 16-byte chunk j of the tile's 64C bytes
  // goes to dword 4j; chunks are dealt to waves 64 at a time
  const int nchunk = LQ_TT * C / 8;
  auto issue = [&](long tile, uint32_t* xbuf) {
    const unsigned base = (unsigned)tile * tile_bytes;
    for (int j0 = wave * 64; j0 < nchunk; j0 += LQ_NW * 64) {  // wave-uniform
      const unsigned off = base + (unsigned)(j0 + lane) * 16u;
      const bool in = j0 + lane < nchunk;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)(xbuf + 4 * j0), 16,
                                               in ? off : 0xFFFFFFF0u, 0, 0, 0);
    }
  };

  int pending_stores = 0;  // store instructions this wave issued after the current tile's copies
  // one tile in X buffer xcur, the next tile's copy going into xnext
  auto body = [&](long tile, uint32_t* xcur, uint32_t* xnext) {
    const long t0 = tile * LQ_TT;
    const int nt = (int)min((long)LQ_TT, ntok - t0);
    lq_wait_vm(pending_stores);  // this wave's copies of the tile have landed
    __syncthreads();
    if (tile + gridDim.x < ntiles) issue(tile + gridDim.x, xnext);

    // ---- LayerNorm: 16 threads per token, thread `sub` owns channels [sub*CPT, sub*CPT + CPT)
    //      (groups of 4 never straddle an 8-channel chunk: CPT and the start are multiples of 4)
    {
      constexpr int CPT = 4 * ((S::KP + 63) / 64);
      const int t = tid >> 4, sub = tid & 15;
      const int c0 = sub * CPT;
      const uint32_t* xrow = xcur + t * (C / 2);  // the token's C bf16 (C % 4 == 0: 8-byte aligned)
      float xv[CPT];
#pragma unroll
      for (int g4 = 0; g4 < CPT / 4; ++g4) {
        const int c = c0 + 4 * g4;
        u32x2_t pr = {0u, 0u};
        if (c < C) pr = *reinterpret_cast<const u32x2_t*>(xrow + c / 2);
        xv[4 * g4] = bf16_lo(pr[0]);
        xv[4 * g4 + 1] = bf16_hi(pr[0]);
        xv[4 * g4 + 2] = bf16_lo(pr[1]);
        xv[4 * g4 + 3] = bf16_hi(pr[1]);
      }
      float sum = 0.0f;
#pragma unroll
      for (int i = 0; i < CPT; ++i) sum += xv[i];  // channels past C hold 0
      sum = row16_sum(sum);
      const float mu = sum * (1.0f / (float)C);
      float sq = 0.0f;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const float d = c0 + i < C ? xv[i] - mu : 0.0f;
        sq = fmaf(d, d, sq);
      }
      sq = row16_sum(sq);
      // v_rsq_f32 (about 1 ulp): LN(x) is rounded to bf16 next, and the correctly rounded
      // sqrt and divide this library is built with would cost some 25 instructions here
      const float inv = __builtin_amdgcn_rsqf(sq * (1.0f / (float)C) + eps);
      uint32_t* xo = xcur + t * (C / 2);
#pragma unroll
      for (int g4 = 0; g4 < CPT / 4; ++g4) {
        const int c = c0 + 4 * g4;
        if (c < C) {
          const f32x4_t gm = *reinterpret_cast<const f32x4_t*>(&s_gb[0][c]);
          const f32x4_t bt = *reinterpret_cast<const f32x4_t*>(&s_gb[1][c]);
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = t < nt ? (xv[4 * g4 + e] - mu) * inv * gm[e] + bt[e] : 0.0f;
          const u32x2_t pk = {pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])};
          *reinterpret_cast<u32x2_t*>(s_b + (c >> 3) * S::BCS + 4 * t + ((c & 7) >> 1)) = pk;  // chunk c/8, token t
          if (xn) *reinterpret_cast<u32x2_t*>(xo + c / 2) = pk;  // the tile's own copy becomes LN(X)
        }
      }
    }
    __syncthreads();

    // ---- y^T = W^T xn^T per 16 tokens (tg), then + bias, bf16, into the output tile [part][token][C]
    // accumulators start from the bias of the lane's 4 outputs (blocks past 3C compute nothing;
    // for the others ob + 15 < 3C rounded up to 16 <= 3 KP, inside s_bias)
    f32x4_t acc[NBW][2];
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      const int ob = 16 * (wave + LQ_NW * i);
      const f32x4_t b4 = ob < C3 ? *reinterpret_cast<const f32x4_t*>(s_bias + ob + 4 * g)
                                 : (f32x4_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int tg = 0; tg < 2; ++tg) acc[i][tg] = b4;
    }
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      // B operand: lane = (token 16 tg + l16, channels 32kc + 8g .. +7) = chunk 4kc + g
      const uint32_t* bp = s_b + (4 * kc + g) * S::BCS + 4 * l16;
      const u32x4_t xb0 = *reinterpret_cast<const u32x4_t*>(bp);
      const u32x4_t xb1 = *reinterpret_cast<const u32x4_t*>(bp + 64);
#pragma unroll
      for (int i = 0; i < NBW; ++i)
        if (16 * (wave + LQ_NW * i) < C3) {
          acc[i][0] = lq_mfma(wa[i][kc], xb0, acc[i][0]);
          acc[i][1] = lq_mfma(wa[i][kc], xb1, acc[i][1]);
        }
    }
    uint16_t* ot = reinterpret_cast<uint16_t*>(s_o);
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      const int o0 = 16 * (wave + LQ_NW * i) + 4 * g;  // 4 consecutive outputs, one part (C % 4 == 0)
      if (o0 < C3) {
        const int part = o0 / C, ch = o0 - part * C;
#pragma unroll
        for (int tg = 0; tg < 2; ++tg) {
          const uint32_t lo = pack_bf16(acc[i][tg][0], acc[i][tg][1]);
          const uint32_t hi = pack_bf16(acc[i][tg][2], acc[i][tg][3]);
          *reinterpret_cast<u32x2_t*>(ot + (part * LQ_TT + 16 * tg + l16) * C + ch) = (u32x2_t){lo, hi};
        }
      }
    }
    __syncthreads();

    // ---- copy out: each part's tile is nt*C contiguous bf16 of its map.  The parts are unrolled so
    // every store addresses a kernel argument (global stores; a flat store could alias LDS and would
    // make the compiler drain it before the next LDS read).
    const long gdw = t0 * C / 2;  // dword offset of the tile in a map
    const int ndw = nt * C / 2;
    // one store instruction per loop trip of the wave: trips = ceil((total - 64 wave) / LQ_NT)
    auto trips = [&](int total) { return total > 64 * wave ? (total - 64 * wave + LQ_NT - 1) / LQ_NT : 0; };
    auto copy_part = [&](uint32_t* __restrict__ dst, const uint32_t* src) {
      if (nt == LQ_TT) {
        const int n16 = ndw / 4;  // 32 * C / 8 chunks of 16 bytes
        for (int j = tid; j < n16; j += LQ_NT)
          *reinterpret_cast<u32x4_t*>(dst + gdw + 4 * j) = *reinterpret_cast<const u32x4_t*>(src + 4 * j);
        return trips(n16);
      }
      for (int j = tid; j < ndw; j += LQ_NT) dst[gdw + j] = src[j];
      return trips(ndw);
    };
    pending_stores = q ? copy_part(q, s_o) : 0;  // q is null when the caller fuses Q into the attention
    pending_stores += copy_part(k, s_o + LQ_TT * C / 2);
    pending_stores += copy_part(v, s_o + LQ_TT * C);
    if (xn) pending_stores += copy_part(xn, xcur);
  };
  long tile = blockIdx.x;
  if (tile < ntiles) issue(tile, s_xa);
  for (; tile < ntiles; tile += 2 * (long)gridDim.x) {
    body(tile, s_xa, s_xb);
    if (tile + gridDim.x < ntiles) body(tile + gridDim.x, s_xb, s_xa);
  }
}

// ---- plain path: 16 tokens per workgroup, fp32 LayerNorm in LDS, one output per thread
template <typename T>
__device__ __forceinline__ float lq_ld(const T* p, long i);
template <>
__device__ __forceinline__ float lq_ld<float>(const float* p, long i) { return p[i]; }
template <>
__device__ __forceinline__ float lq_ld<uint16_t>(const uint16_t* p, long i) {
  return __builtin_bit_cast(float, (uint32_t)p[i] << 16);
}
template <typename T>
__device__ __forceinline__ void lq_st(T* p, long i, float v);
template <>
__device__ __forceinline__ void lq_st<float>(float* p, long i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void lq_st<uint16_t>(uint16_t* p, long i, float v) {
  p[i] = (uint16_t)(pack_bf16(v, 0.0f) & 0xFFFFu);
}

constexpr int LP_T = 16;  // tokens per workgroup

template <typename T>
__global__ void __launch_bounds__(256)
ln_qkv_plain_kernel(const T* __restrict__ x, const float* __restrict__ gamma, const float* __restrict__ beta,
                    const float* __restrict__ w, const float* __restrict__ bias, T* __restrict__ q, T* __restrict__ k,
                    T* __restrict__ v, T* __restrict__ xn, long ntok, int C, float eps) {
  __shared__ float s_xn[LP_T][256];
  const long t0 = (long)blockIdx.x * LP_T;
  const int nt = (int)min((long)LP_T, ntok - t0);
  const int t = threadIdx.x >> 4, sub = threadIdx.x & 15;
  if (t < nt) {
    const T* xt = x + (t0 + t) * C;
    float sum = 0.0f;
    for (int c = sub; c < C; c += 16) sum += lq_ld(xt, c);
    sum = row16_sum(sum);  // the 16 threads of token t are one DPP row, active together
    const float mu = sum / (float)C;
    float sq = 0.0f;
    for (int c = sub; c < C; c += 16) {
      const float d = lq_ld(xt, c) - mu;
      sq = fmaf(d, d, sq);
    }
    sq = row16_sum(sq);
    const float inv = 1.0f / sqrtf(sq / (float)C + eps);
    for (int c = sub; c < C; c += 16) {
      const float y = (lq_ld(xt, c) - mu) * inv * gamma[c] + beta[c];
      s_xn[t][c] = y;
      if (xn) lq_st(xn, (t0 + t) * C + c, y);
    }
  }
  __syncthreads();
  const int C3 = 3 * C;
  for (int j = threadIdx.x; j < nt * C3; j += 256) {
    const int tt = j / C3, o = j - tt * C3;
    float acc = bias[o];
    for (int c = 0; c < C; ++c) acc = fmaf(s_xn[tt][c], w[(long)c * C3 + o], acc);
    T* dst = o < C ? q : (o < 2 * C ? k : v);
    if (dst) lq_st(dst, (t0 + tt) * C + o % C, acc);  // q may be null
  }
}

template <int KC, int NBW>
hipError_t launch_mfma(const LnQkvArgs& a, hipStream_t stream) {
  const long ntok = (long)a.B * a.H * a.W;
  const long ntiles = (ntok + LQ_TT - 1) / LQ_TT;
  const int grid = (int)min(ntiles, (long)device_cus());
  hipLaunchKernelGGL((ln_qkv_bf16_kernel<KC, NBW>), dim3(grid), dim3(LQ_NT), 0, stream, (const uint32_t*)a.x,
                     a.gamma, a.beta, a.w, a.bias, (uint32_t*)a.q, (uint32_t*)a.k, (uint32_t*)a.v, (uint32_t*)a.xn,
                     ntok, a.C, a.eps);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_plain(const LnQkvArgs& a, hipStream_t stream) {
  const long ntok = (long)a.B * a.H * a.W;
  const int grid = (int)((ntok + LP_T - 1) / LP_T);
  hipLaunchKernelGGL((ln_qkv_plain_kernel<T>), dim3(grid), dim3(256), 0, stream, (const T*)a.x, a.gamma, a.beta,
                     a.w, a.bias, (T*)a.q, (T*)a.k, (T*)a.v, (T*)a.xn, ntok, a.C, a.eps);
  return hipGetLastError();
}

}  // namespace

bool ln_qkv_mfma(int C) { return C % 4 == 0 && C <= 192; }

hipError_t launch_ln_qkv(const LnQkvArgs& a, bool bf16, hipStream_t stream) {
  if (!bf16) return launch_plain<float>(a, stream);
  if (!ln_qkv_mfma(a.C)) return launch_plain<uint16_t>(a, stream);
  switch ((a.C + 31) / 32) {  // 32-channel steps; blocks of 16 outputs per wave = ceil(ceil(3C/16)/8)
    case 1: return launch_mfma<1, 1>(a, stream);
    case 2: return launch_mfma<2, 2>(a, stream);
    case 3: return launch_mfma<3, 3>(a, stream);
    case 4: return launch_mfma<4, 3>(a, stream);
    case 5: return launch_mfma<5, 4>(a, stream);
    case 6: return launch_mfma<6, 5>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rib
