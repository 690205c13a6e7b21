// attn_f32.hip -- fp32 RIB window attention with the CLA gate.
//
// Computes, per image, window and head ("Rank-Factorized Implicit Neural
// Bias", gist.science summaries part A mechanism steps 3-4 and part B;
// omica.com.cn explainer sections 2.2 "attention rewrite" and 2.3):
//   s_ij = [Qc_i/sqrt(dh), Qp_i/sqrt(R)] . [Kc_j, Kp_j]
//   O_i  = (sum_j softmax_j(s_ij) V_j) * sigmoid(G_i)
// in fp32 throughout.  This is the precision path (fp32 inputs); the bf16
// MFMA kernel in attn_bf16.hip is the throughput path.
//
// One thread owns one query row: its augmented query (content scaled by
// 1/sqrt(dh), positional factor scaled by 1/sqrt(R)) lives in registers, key
// tiles of KT tokens of the same window are staged through LDS, and the
// softmax is accumulated online (running max, running sum, rescale on a new
// maximum).  Window partitioning is index arithmetic on the NHWC arrays:
// window w's real tokens are enumerated row-major as r = iy*nx + ix with
// nx = the number of real columns, so padded positions never enter the loops.
#include "rib_device.hpp"
#include "rib_launch.hpp"

namespace rib {

namespace {

constexpr int F32_QB = 256;  // queries (threads) per workgroup
constexpr int F32_KT = 64;   // keys per LDS tile

template <int DHM, int RM>
__global__ void __launch_bounds__(F32_QB)
attn_f32_kernel(const float* __restrict__ qc, const float* __restrict__ kc,
                const float* __restrict__ v, const float* __restrict__ g,
                const float* __restrict__ qp, const float* __restrict__ kp, float* __restrict__ o,
                int B, int T, int H, int W, int heads, int dh, int R, int wt, int ws, int total, long tstride,
                float* __restrict__ lse) {
  __shared__ float sk[F32_KT][DHM];
  __shared__ float sv[F32_KT][DHM];
  __shared__ float skp[F32_KT][RM];

  const int logical = xcd_swizzle(blockIdx.x, gridDim.x);
  if (logical >= total) return;
  const int nWy = (H + ws - 1) / ws, nWx = (W + ws - 1) / ws, nWt = (T + wt - 1) / wt;
  const int qblocks = (wt * ws * ws + F32_QB - 1) / F32_QB;
  int t = logical;
  const int qblk = t % qblocks; t /= qblocks;
  const int h = t % heads; t /= heads;
  const int wx = t % nWx; t /= nWx;
  const int wy = t % nWy; t /= nWy;
  const int tw = t % nWt;
  const int b = t / nWt;
  qp += (long)h * tstride;  // per-head positional tables (tstride 0: one shared pair)
  kp += (long)h * tstride;
  const int ny = min(ws, H - wy * ws), nx = min(ws, W - wx * ws);
  const int n_real = min(wt, T - tw * wt) * ny * nx;
  const int q0 = qblk * F32_QB;
  if (q0 >= n_real) return;
  const int C = heads * dh;
  // real index r (frame-major, then row-major over the window's real tokens) ->
  // (element offset of the token's head slice, in-window index n = (it*ws + iy)*ws + ix)
  auto locate = [&](int r, int& off, int& n) {
    const int rr = r / nx, ix = r - rr * nx;
    const int it = rr / ny, iy = rr - it * ny;
    off = (((b * T + tw * wt + it) * H + wy * ws + iy) * W + wx * ws + ix) * C + h * dh;
    n = (it * ws + iy) * ws + ix;
  };

  const int r = q0 + (int)threadIdx.x;
  const bool valid = r < n_real;
  int qoff, qn;
  locate(min(r, n_real - 1), qoff, qn);
  const float sc = 1.0f / sqrtf((float)dh);
  const float sp = 1.0f / sqrtf((float)R);
  float q[DHM], qpos[RM], acc[DHM];
#pragma unroll
  for (int d = 0; d < DHM; ++d) {
    q[d] = d < dh ? qc[qoff + d] * sc : 0.0f;
    acc[d] = 0.0f;
  }
#pragma unroll
  for (int k = 0; k < RM; ++k) qpos[k] = k < R ? qp[qn * R + k] * sp : 0.0f;

  float m = -INFINITY, l = 0.0f;
  for (int k0 = 0; k0 < n_real; k0 += F32_KT) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < F32_KT * DHM; idx += F32_QB) {
      const int j = idx / DHM, d = idx % DHM;
      const int key = k0 + j;
      float kv = 0.0f, vv = 0.0f;
      if (key < n_real && d < dh) {
        int off, n;
        locate(key, off, n);
        kv = kc[off + d];
        vv = v[off + d];
      }
      sk[j][d] = kv;
      sv[j][d] = vv;
    }
    for (int idx = threadIdx.x; idx < F32_KT * RM; idx += F32_QB) {
      const int j = idx / RM, k = idx % RM;
      const int key = k0 + j;
      float pv = 0.0f;
      if (key < n_real && k < R) {
        int off, n;
        locate(key, off, n);
        pv = kp[n * R + k];
      }
      skp[j][k] = pv;
    }
    __syncthreads();
    const int kend = min(F32_KT, n_real - k0);
    for (int j = 0; j < kend; ++j) {
      float s = 0.0f, bias = 0.0f;
#pragma unroll
      for (int d = 0; d < DHM; ++d) s = fmaf(q[d], sk[j][d], s);
#pragma unroll
      for (int k = 0; k < RM; ++k) bias = fmaf(qpos[k], skp[j][k], bias);
      s += bias;
      if (s > m) {
        const float c = expf(m - s);
        l *= c;
#pragma unroll
        for (int d = 0; d < DHM; ++d) acc[d] *= c;
        m = s;
      }
      const float p = expf(s - m);
      l += p;
#pragma unroll
      for (int d = 0; d < DHM; ++d) acc[d] = fmaf(p, sv[j][d], acc[d]);
    }
  }
  if (!valid) return;
  if (lse) lse[(qoff - h * dh) / C * heads + h] = m + logf(l);
#pragma unroll
  for (int d = 0; d < DHM; ++d)
    if (d < dh) o[qoff + d] = acc[d] / l * (1.0f / (1.0f + expf(-g[qoff + d])));
}

template <int DHM, int RM>
hipError_t launch_f32(const AttnArgs& a, hipStream_t stream) {
  const int nWy = (a.H + a.ws - 1) / a.ws, nWx = (a.W + a.ws - 1) / a.ws, nWt = (a.T + a.wt - 1) / a.wt;
  const int qblocks = (a.wt * a.ws * a.ws + F32_QB - 1) / F32_QB;
  const int total = a.B * nWt * nWy * nWx * a.heads * qblocks;
  const int grid = 8 * ((total + 7) / 8);
  hipLaunchKernelGGL((attn_f32_kernel<DHM, RM>), dim3(grid), dim3(F32_QB), 0, stream,
                     (const float*)a.qc, (const float*)a.kc, (const float*)a.v, (const float*)a.g,
                     a.qp, a.kp, (float*)a.o, a.B, a.T, a.H, a.W, a.heads, a.dh, a.R, a.wt, a.ws, total,
                     a.tstride, a.lse);
  return hipGetLastError();
}

template <int DHM>
hipError_t launch_f32_r(const AttnArgs& a, hipStream_t stream) {
  if (a.R <= 16) return launch_f32<DHM, 16>(a, stream);
  if (a.R <= 32) return launch_f32<DHM, 32>(a, stream);
  return launch_f32<DHM, 64>(a, stream);
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t stream) {
  if (a.dh <= 16) return launch_f32_r<16>(a, stream);
  if (a.dh <= 32) return launch_f32_r<32>(a, stream);
  return launch_f32_r<64>(a, stream);
}

}  // namespace rib
