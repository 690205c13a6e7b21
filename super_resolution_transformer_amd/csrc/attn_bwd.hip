// attn_bwd.hip -- backward of RIB window attention with the CLA gate.
//
// Forward, per image, window and head ("Rank-Factorized Implicit Neural
// Bias", omica.com.cn explainer sections 2.2 "attention rewrite" and 2.3;
// gist.science summaries part A, the concatenation identity):
//   s_ij = Qt_i . Kt_j,  Qt = [Qc/sqrt(dh), Qp/sqrt(R)],  Kt = [Kc, Kp]
//   P = softmax_j(s),  A = P V,  O = A * sigmoid(G)
// Given dO, the chain rule gives (sg = sigmoid(G)):
//   dA = dO * sg,   dG = dO * A * sg * (1 - sg) = dO * O * (1 - sg)
//   D_i = sum_j P_ij (dA_i . V_j) = dA_i . A_i = dO_i . O_i
//   dS_ij = P_ij (dA_i . V_j - D_i)
//   dQt = dS Kt  -> dQc = dQt_c / sqrt(dh),  dQp rows = dQt_p / sqrt(R)
//   dKt = dS^T Qt -> dKc = dKt_c,            dKp rows = dKt_p
//   dV  = P^T dA
// and the shared positional tables collect dQp[n], dKp[n] from every window,
// head and image at in-window index n.  The explainer times a training
// iteration (section 4.1); this is the backward half of it.
//
// Passes (all on one stream):
//   prep   per token and head: dA, D and dG from dO, O, G
//   dq     query-major: P = exp(s - lse) from the forward's row log-sum-exp,
//          accumulates dQt, writes dQc and the per-row dQp
//   dkv    key-major: the same P, accumulates dV and dKt, writes dKc, dV and
//          the per-row dKp
//   reduce per (n, r): sums the per-row dQp / dKp over images, windows, heads
// The dq and dkv kernels here keep one row per thread in fp32 registers and
// stage the other side through LDS; they serve every (dh, R) and both storage
// types.  The bf16 MFMA kernels in attn_bwd_bf16.hip replace them for the
// head shapes they are compiled for.
#include "rib_bwd.hpp"
#include "rib_device.hpp"

namespace rib {

namespace {

constexpr int BW_QB = 256;  // rows (threads) per workgroup
constexpr int BW_KT = 64;   // rows of the other side per LDS tile

template <typename T>
__device__ __forceinline__ float ldf(const T* p, long i);
template <>
__device__ __forceinline__ float ldf<float>(const float* p, long i) { return p[i]; }
template <>
__device__ __forceinline__ float ldf<uint16_t>(const uint16_t* p, long i) {
  return __builtin_bit_cast(float, (uint32_t)p[i] << 16);
}

template <typename T>
__device__ __forceinline__ void stf(T* p, long i, float v);
template <>
__device__ __forceinline__ void stf<float>(float* p, long i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void stf<uint16_t>(uint16_t* p, long i, float v) {
  p[i] = (uint16_t)(pack_bf16(v, 0.0f) & 0xFFFFu);
}

// prep, staged: a workgroup takes NT whole tokens (NT*C contiguous elements of
// each map), copies dO, O, G into LDS with coalesced dword loads, computes one
// (token, head) row per thread, writes dA and dG over the staged dO and O and
// stores them back coalesced.  LDS: 3 * NT * C elements.
template <typename T>
__global__ void __launch_bounds__(256)
bwd_prep_staged_kernel(const T* __restrict__ dout, const T* __restrict__ o, const T* __restrict__ g,
                       T* __restrict__ da, T* __restrict__ dg, float* __restrict__ dsum, long ntok, int heads,
                       int dh, int NT) {
  extern __shared__ uint32_t sm[];
  const int C = heads * dh;
  const long tok0 = (long)blockIdx.x * NT;
  const int nt = (int)min((long)NT, ntok - tok0);
  const int ndw = nt * C * (int)sizeof(T) / 4;   // C * sizeof(T) is a multiple of 4
  const int cap = NT * C * (int)sizeof(T) / 4;
  uint32_t* s_do = sm;
  uint32_t* s_o = sm + cap;
  uint32_t* s_g = sm + 2 * cap;
  const long base = tok0 * C * (long)sizeof(T) / 4;
  const uint32_t* gdo = reinterpret_cast<const uint32_t*>(dout) + base;
  const uint32_t* go = reinterpret_cast<const uint32_t*>(o) + base;
  const uint32_t* gg = reinterpret_cast<const uint32_t*>(g) + base;
  for (int i = threadIdx.x; i < ndw; i += 256) {
    s_do[i] = gdo[i];
    s_o[i] = go[i];
    s_g[i] = gg[i];
  }
  __syncthreads();
  T* e_do = reinterpret_cast<T*>(s_do);
  T* e_o = reinterpret_cast<T*>(s_o);
  const T* e_g = reinterpret_cast<const T*>(s_g);
  for (int row = threadIdx.x; row < nt * heads; row += 256) {
    const int e0 = (row / heads) * C + (row % heads) * dh;
    float D = 0.0f;
    for (int d = 0; d < dh; ++d) {
      const float dov = ldf(e_do, e0 + d), ov = ldf(e_o, e0 + d);
      const float s = 1.0f / (1.0f + expf(-ldf(e_g, e0 + d)));
      D = fmaf(dov, ov, D);
      stf(e_do, e0 + d, dov * s);
      stf(e_o, e0 + d, dov * ov * (1.0f - s));
    }
    dsum[tok0 * heads + row] = D;
  }
  __syncthreads();
  uint32_t* gda = reinterpret_cast<uint32_t*>(da) + base;
  uint32_t* gdg = reinterpret_cast<uint32_t*>(dg) + base;
  for (int i = threadIdx.x; i < ndw; i += 256) {
    gda[i] = s_do[i];
    gdg[i] = s_o[i];
  }
}

// prep, bf16 maps with dh <= 32: the same staging with 16-byte copies (NT even, so a tile
// starts 16-byte aligned whenever C is a multiple of 4), and the rows computed by 16 lanes
// each (one DPP row): lane p takes channel pair p of its (token, head) row as one dword, D is
// the row's DPP sum.  Lanes past dh/2 or past the tile's rows compute zeros and store nothing.
__device__ __forceinline__ float prep_row16_sum(float v) {
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

__global__ void __launch_bounds__(256)
bwd_prep_pairs_kernel(const uint32_t* __restrict__ dout, const uint32_t* __restrict__ o,
                      const uint32_t* __restrict__ g, uint32_t* __restrict__ da, uint32_t* __restrict__ dg,
                      float* __restrict__ dsum, long ntok, int heads, int dh, int NT) {
  extern __shared__ uint32_t sm[];
  const int C2 = heads * dh / 2;  // dwords per token
  const long tok0 = (long)blockIdx.x * NT;
  const int nt = (int)min((long)NT, ntok - tok0);
  const int ndw = nt * C2;
  const int cap = NT * C2;
  uint32_t* s_do = sm;
  uint32_t* s_o = sm + cap;
  uint32_t* s_g = sm + 2 * cap;
  const long base = tok0 * C2;
  // 16-byte copies when every map is 16-byte aligned: C2 and NT even keep the tile and the three
  // LDS arrays 16-byte aligned; otherwise dword copies (the maps need only 4-byte alignment)
  const uintptr_t ptrs = (uintptr_t)dout | (uintptr_t)o | (uintptr_t)g | (uintptr_t)da | (uintptr_t)dg;
  const bool vec = (C2 % 2 == 0) && (base & 3) == 0 && (ptrs & 15) == 0;
  auto copy_in = [&](uint32_t* dst, const uint32_t* __restrict__ src) {
    if (vec) {
      for (int i = 4 * (int)threadIdx.x; i + 4 <= ndw; i += 1024)
        *reinterpret_cast<u32x4_t*>(dst + i) = *reinterpret_cast<const u32x4_t*>(src + base + i);
      for (int i = (ndw & ~3) + (int)threadIdx.x; i < ndw; i += 256) dst[i] = src[base + i];
    } else {
      for (int i = threadIdx.x; i < ndw; i += 256) dst[i] = src[base + i];
    }
  };
  copy_in(s_do, dout);
  copy_in(s_o, o);
  copy_in(s_g, g);
  __syncthreads();
  const int pr = threadIdx.x & 15;
  const int hp = dh / 2;
  const int rows = nt * heads;
  for (int r0 = 0; r0 < rows; r0 += 16) {
    const int row = r0 + ((int)threadIdx.x >> 4);
    const bool live = row < rows && pr < hp;
    const int e = live ? (row / heads) * C2 + (row % heads) * hp + pr : 0;
    const uint32_t wdo = live ? s_do[e] : 0u, wo = live ? s_o[e] : 0u, wg = live ? s_g[e] : 0u;
    const float do0 = bf16_lo(wdo), do1 = bf16_hi(wdo), o0 = bf16_lo(wo), o1 = bf16_hi(wo);
    const float s0 = 1.0f / (1.0f + expf(-bf16_lo(wg))), s1 = 1.0f / (1.0f + expf(-bf16_hi(wg)));
    const float D = prep_row16_sum(fmaf(do1, o1, do0 * o0));
    if (live) {
      s_do[e] = pack_bf16(do0 * s0, do1 * s1);
      s_o[e] = pack_bf16(do0 * o0 * (1.0f - s0), do1 * o1 * (1.0f - s1));
      if (pr == 0) dsum[tok0 * heads + row] = D;
    }
  }
  __syncthreads();
  auto copy_out = [&](uint32_t* __restrict__ dst, const uint32_t* src) {
    if (vec) {
      for (int i = 4 * (int)threadIdx.x; i + 4 <= ndw; i += 1024)
        *reinterpret_cast<u32x4_t*>(dst + base + i) = *reinterpret_cast<const u32x4_t*>(src + i);
      for (int i = (ndw & ~3) + (int)threadIdx.x; i < ndw; i += 256) dst[base + i] = src[i];
    } else {
      for (int i = threadIdx.x; i < ndw; i += 256) dst[base + i] = src[i];
    }
  };
  copy_out(da, s_do);
  copy_out(dg, s_o);
}

// prep for rows too wide to stage (C * sizeof(T) > 16 KB): one thread per (token, head).
template <typename T>
__global__ void __launch_bounds__(256)
bwd_prep_kernel(const T* __restrict__ dout, const T* __restrict__ o, const T* __restrict__ g,
                T* __restrict__ da, T* __restrict__ dg, float* __restrict__ dsum, long rows, int heads, int dh) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows) return;
  const long tok = idx / heads;
  const int h = (int)(idx - tok * heads);
  const long base = tok * (long)heads * dh + (long)h * dh;
  float D = 0.0f;
  for (int d = 0; d < dh; ++d) {
    const float dov = ldf(dout, base + d), ov = ldf(o, base + d);
    const float s = 1.0f / (1.0f + expf(-ldf(g, base + d)));
    D = fmaf(dov, ov, D);
    stf(da, base + d, dov * s);
    stf(dg, base + d, dov * ov * (1.0f - s));
  }
  dsum[idx] = D;
}

// dq pass: one thread per query row.  (Padded queries of the last row block
// compute on a copy of the last real row and store nothing.)
template <typename T, int DHM, int RM>
__global__ void __launch_bounds__(BW_QB)
bwd_dq_kernel(BwdArgs a, int total) {
  __shared__ float sk[BW_KT][DHM];
  __shared__ float sv[BW_KT][DHM];
  __shared__ float skp[BW_KT][RM];
  const int logical = xcd_swizzle(blockIdx.x, gridDim.x);
  if (logical >= total) return;
  Unit u;
  if (!decode_unit(logical, a, BW_QB, u)) return;
  const T* qc = (const T*)a.qc;
  const T* kc = (const T*)a.kc;
  const T* v = (const T*)a.v;
  const T* da = (const T*)a.da;
  const int dh = a.dh, R = a.R, C = a.heads * a.dh;
  const float sc = 1.0f / sqrtf((float)dh), sp = 1.0f / sqrtf((float)R);

  const int r = u.blk * BW_QB + (int)threadIdx.x;
  const bool valid = r < u.n_real;
  long qtok;
  int qn;
  locate(u, a, min(r, u.n_real - 1), qtok, qn);
  const long qoff = qtok * C + (long)u.h * dh;
  const long qrow = qtok * a.heads + u.h;
  float q[DHM], qpos[RM], dav[DHM], accc[DHM], accp[RM];
#pragma unroll
  for (int d = 0; d < DHM; ++d) {
    q[d] = d < dh ? ldf(qc, qoff + d) * sc : 0.0f;
    dav[d] = d < dh ? ldf(da, qoff + d) : 0.0f;
    accc[d] = 0.0f;
  }
#pragma unroll
  for (int k = 0; k < RM; ++k) {
    qpos[k] = k < R ? a.qp[u.h * a.tstride + qn * R + k] * sp : 0.0f;
    accp[k] = 0.0f;
  }
  const float D = a.dsum[qrow];

  const float lrow = a.lse[qrow];
  for (int k0 = 0; k0 < u.n_real; k0 += BW_KT) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < BW_KT * DHM; idx += BW_QB) {
      const int j = idx / DHM, d = idx % DHM;
      float kv = 0.0f, vv = 0.0f;
      if (k0 + j < u.n_real && d < dh) {
        long tok;
        int n;
        locate(u, a, k0 + j, tok, n);
        kv = ldf(kc, tok * C + (long)u.h * dh + d);
        vv = ldf(v, tok * C + (long)u.h * dh + d);
      }
      sk[j][d] = kv;
      sv[j][d] = vv;
    }
    for (int idx = threadIdx.x; idx < BW_KT * RM; idx += BW_QB) {
      const int j = idx / RM, k = idx % RM;
      float pv = 0.0f;
      if (k0 + j < u.n_real && k < R) {
        long tok;
        int n;
        locate(u, a, k0 + j, tok, n);
        pv = a.kp[u.h * a.tstride + n * R + k];
      }
      skp[j][k] = pv;
    }
    __syncthreads();
    const int kend = min(BW_KT, u.n_real - k0);
    for (int j = 0; j < kend; ++j) {
      float s = 0.0f, bias = 0.0f, dp = 0.0f;
#pragma unroll
      for (int d = 0; d < DHM; ++d) {
        s = fmaf(q[d], sk[j][d], s);
        dp = fmaf(dav[d], sv[j][d], dp);
      }
#pragma unroll
      for (int k = 0; k < RM; ++k) bias = fmaf(qpos[k], skp[j][k], bias);
      const float p = expf(s + bias - lrow);
      const float ds = p * (dp - D);
#pragma unroll
      for (int d = 0; d < DHM; ++d) accc[d] = fmaf(ds, sk[j][d], accc[d]);
#pragma unroll
      for (int k = 0; k < RM; ++k) accp[k] = fmaf(ds, skp[j][k], accp[k]);
    }
  }
  if (!valid) return;
  T* dqc = (T*)a.dqc;
#pragma unroll
  for (int d = 0; d < DHM; ++d)
    if (d < dh) stf(dqc, qoff + d, accc[d] * sc);
  float* qrows = a.qrows + (((long)u.h * a.B + u.b) * a.H * a.W + (qtok - (long)u.b * a.H * a.W)) * R;
#pragma unroll
  for (int k = 0; k < RM; ++k)
    if (k < R) qrows[k] = accp[k] * sp;
}

// dkv pass: one thread per key row.
template <typename T, int DHM, int RM>
__global__ void __launch_bounds__(BW_QB)
bwd_dkv_kernel(BwdArgs a, int total) {
  __shared__ float sq[BW_KT][DHM];
  __shared__ float sa[BW_KT][DHM];
  __shared__ float sqp[BW_KT][RM];
  __shared__ float slse[BW_KT];
  __shared__ float sd[BW_KT];
  const int logical = xcd_swizzle(blockIdx.x, gridDim.x);
  if (logical >= total) return;
  Unit u;
  if (!decode_unit(logical, a, BW_QB, u)) return;
  const T* qc = (const T*)a.qc;
  const T* kc = (const T*)a.kc;
  const T* v = (const T*)a.v;
  const T* da = (const T*)a.da;
  const int dh = a.dh, R = a.R, C = a.heads * a.dh;
  const float sc = 1.0f / sqrtf((float)dh), sp = 1.0f / sqrtf((float)R);

  const int r = u.blk * BW_QB + (int)threadIdx.x;
  const bool valid = r < u.n_real;
  long ktok;
  int kn;
  locate(u, a, min(r, u.n_real - 1), ktok, kn);
  const long koff = ktok * C + (long)u.h * dh;
  float k[DHM], kpos[RM], vv[DHM], dk[DHM], dkp[RM], dv[DHM];
#pragma unroll
  for (int d = 0; d < DHM; ++d) {
    k[d] = d < dh ? ldf(kc, koff + d) : 0.0f;
    vv[d] = d < dh ? ldf(v, koff + d) : 0.0f;
    dk[d] = 0.0f;
    dv[d] = 0.0f;
  }
#pragma unroll
  for (int x = 0; x < RM; ++x) {
    kpos[x] = x < R ? a.kp[u.h * a.tstride + kn * R + x] : 0.0f;
    dkp[x] = 0.0f;
  }

  for (int q0 = 0; q0 < u.n_real; q0 += BW_KT) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < BW_KT * DHM; idx += BW_QB) {
      const int i = idx / DHM, d = idx % DHM;
      float qv = 0.0f, av = 0.0f;
      if (q0 + i < u.n_real && d < dh) {
        long tok;
        int n;
        locate(u, a, q0 + i, tok, n);
        qv = ldf(qc, tok * C + (long)u.h * dh + d) * sc;
        av = ldf(da, tok * C + (long)u.h * dh + d);
      }
      sq[i][d] = qv;
      sa[i][d] = av;
    }
    for (int idx = threadIdx.x; idx < BW_KT * RM; idx += BW_QB) {
      const int i = idx / RM, x = idx % RM;
      float pv = 0.0f;
      if (q0 + i < u.n_real && x < R) {
        long tok;
        int n;
        locate(u, a, q0 + i, tok, n);
        pv = a.qp[u.h * a.tstride + n * R + x] * sp;
      }
      sqp[i][x] = pv;
    }
    for (int i = threadIdx.x; i < BW_KT; i += BW_QB) {
      float lv = 0.0f, dv0 = 0.0f;
      if (q0 + i < u.n_real) {
        long tok;
        int n;
        locate(u, a, q0 + i, tok, n);
        lv = a.lse[tok * a.heads + u.h];
        dv0 = a.dsum[tok * a.heads + u.h];
      }
      slse[i] = lv;
      sd[i] = dv0;
    }
    __syncthreads();
    const int qend = min(BW_KT, u.n_real - q0);
    for (int i = 0; i < qend; ++i) {
      float s = 0.0f, bias = 0.0f, dp = 0.0f;
#pragma unroll
      for (int d = 0; d < DHM; ++d) {
        s = fmaf(sq[i][d], k[d], s);
        dp = fmaf(sa[i][d], vv[d], dp);
      }
#pragma unroll
      for (int x = 0; x < RM; ++x) bias = fmaf(sqp[i][x], kpos[x], bias);
      const float p = expf(s + bias - slse[i]);
      const float ds = p * (dp - sd[i]);
#pragma unroll
      for (int d = 0; d < DHM; ++d) {
        dv[d] = fmaf(p, sa[i][d], dv[d]);
        dk[d] = fmaf(ds, sq[i][d], dk[d]);
      }
#pragma unroll
      for (int x = 0; x < RM; ++x) dkp[x] = fmaf(ds, sqp[i][x], dkp[x]);
    }
  }
  if (!valid) return;
  T* dkc = (T*)a.dkc;
  T* dvo = (T*)a.dv;
#pragma unroll
  for (int d = 0; d < DHM; ++d)
    if (d < dh) {
      stf(dkc, koff + d, dk[d]);
      stf(dvo, koff + d, dv[d]);
    }
  float* krows = a.krows + (((long)u.h * a.B + u.b) * a.H * a.W + (ktok - (long)u.b * a.H * a.W)) * R;
#pragma unroll
  for (int x = 0; x < RM; ++x)
    if (x < R) krows[x] = dkp[x];
}

// reduce: thread per (table head, table, n, r); sums the per-row gradients of
// every real token at in-window index n over images and windows, and over the
// heads too unless each head has its own table (tab_heads = heads).
__global__ void __launch_bounds__(256)
bwd_table_reduce_kernel(BwdArgs a) {
  const int N = a.ws * a.ws;
  int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= a.tab_heads * 2 * N * a.R) return;
  const int th = idx / (2 * N * a.R);  // table head (0 when the heads share one table)
  idx -= th * 2 * N * a.R;
  const int tab = idx / (N * a.R);
  const int rem = idx - tab * N * a.R;
  const int n = rem / a.R, r = rem - (rem / a.R) * a.R;
  const int iy = n / a.ws, ix = n - (n / a.ws) * a.ws;
  const float* rows = tab ? a.krows : a.qrows;
  const int nWy = (a.H + a.ws - 1) / a.ws, nWx = (a.W + a.ws - 1) / a.ws;
  const int hb0 = a.tab_heads > 1 ? th * a.B : 0;                 // rows are [heads][B][H][W][R]
  const int hb1 = a.tab_heads > 1 ? (th + 1) * a.B : a.heads * a.B;
  // every (window, image-head) term of this table entry; eight independent partial sums keep
  // eight loads of the image-head loop in flight
  const long hstride = (long)a.H * a.W * a.R;
  float acc = 0.0f;
  for (int wy = 0; wy < nWy; ++wy) {
    const int y = wy * a.ws + iy;
    if (y >= a.H) break;
    for (int wx = 0; wx < nWx; ++wx) {
      const int x = wx * a.ws + ix;
      if (x >= a.W) break;
      const float* p = rows + (((long)hb0 * a.H + y) * a.W + x) * a.R + r;
      float s[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
      int hb = hb0;
      for (; hb + 8 <= hb1; hb += 8, p += 8 * hstride) {
#pragma unroll
        for (int k = 0; k < 8; ++k) s[k] += p[k * hstride];
      }
      for (; hb < hb1; ++hb, p += hstride) s[0] += p[0];
      acc += ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
    }
  }
  (tab ? a.dkp : a.dqp)[(long)th * N * a.R + n * a.R + r] = acc;
}

template <typename T, int DHM, int RM>
hipError_t launch_rows(const BwdArgs& a, hipStream_t stream) {
  const int total = bwd_units(a, BW_QB);
  const int grid = 8 * ((total + 7) / 8);
  hipLaunchKernelGGL((bwd_dq_kernel<T, DHM, RM>), dim3(grid), dim3(BW_QB), 0, stream, a, total);
  hipLaunchKernelGGL((bwd_dkv_kernel<T, DHM, RM>), dim3(grid), dim3(BW_QB), 0, stream, a, total);
  return hipGetLastError();
}

template <typename T, int DHM>
hipError_t launch_rows_r(const BwdArgs& a, hipStream_t stream) {
  if (a.R <= 16) return launch_rows<T, DHM, 16>(a, stream);
  if (a.R <= 32) return launch_rows<T, DHM, 32>(a, stream);
  return launch_rows<T, DHM, 64>(a, stream);
}

template <typename T>
hipError_t launch_rows_dh(const BwdArgs& a, hipStream_t stream) {
  if (a.dh <= 16) return launch_rows_r<T, 16>(a, stream);
  if (a.dh <= 32) return launch_rows_r<T, 32>(a, stream);
  return launch_rows_r<T, 64>(a, stream);
}

template <typename T>
hipError_t launch_prep(const BwdArgs& a, hipStream_t stream) {
  const long ntok = (long)a.B * a.H * a.W;
  const int C = a.heads * a.dh;
  const int row_bytes = C * (int)sizeof(T);
  if (sizeof(T) == 2 && a.dh % 2 == 0 && a.dh <= 32 && row_bytes % 4 == 0 && row_bytes <= 16384) {
    const int NT = max(2, (6144 / row_bytes) & ~1);  // even; <= 18 KB of LDS: eight workgroups per CU
    const int grid = (int)((ntok + NT - 1) / NT);
    const size_t lds = 3 * (size_t)NT * row_bytes;
    hipLaunchKernelGGL(bwd_prep_pairs_kernel, dim3(grid), dim3(256), lds, stream, (const uint32_t*)a.dout,
                       (const uint32_t*)a.o, (const uint32_t*)a.g, (uint32_t*)a.da, (uint32_t*)a.dg, a.dsum, ntok,
                       a.heads, a.dh, NT);
    return hipGetLastError();
  }
  if (row_bytes % 4 == 0 && row_bytes <= 16384) {
    const int NT = max(1, 16384 / row_bytes);  // <= 48 KB of LDS for the three maps
    const int grid = (int)((ntok + NT - 1) / NT);
    const size_t lds = 3 * (size_t)NT * row_bytes;
    hipLaunchKernelGGL((bwd_prep_staged_kernel<T>), dim3(grid), dim3(256), lds, stream, (const T*)a.dout,
                       (const T*)a.o, (const T*)a.g, (T*)a.da, (T*)a.dg, a.dsum, ntok, a.heads, a.dh, NT);
    return hipGetLastError();
  }
  const long rows = ntok * a.heads;
  const int grid = (int)((rows + 255) / 256);
  hipLaunchKernelGGL((bwd_prep_kernel<T>), dim3(grid), dim3(256), 0, stream, (const T*)a.dout, (const T*)a.o,
                     (const T*)a.g, (T*)a.da, (T*)a.dg, a.dsum, rows, a.heads, a.dh);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_prep(const BwdArgs& a, bool bf16, hipStream_t stream) {
  return bf16 ? launch_prep<uint16_t>(a, stream) : launch_prep<float>(a, stream);
}

hipError_t launch_attn_bwd_rows(const BwdArgs& a, bool bf16, hipStream_t stream) {
  return bf16 ? launch_rows_dh<uint16_t>(a, stream) : launch_rows_dh<float>(a, stream);
}

hipError_t launch_attn_bwd_reduce(const BwdArgs& a, hipStream_t stream) {
  const int n = a.tab_heads * 2 * a.ws * a.ws * a.R;
  hipLaunchKernelGGL(bwd_table_reduce_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rib
