// encode.hip -- the coordinate encoder and implicit neural field that produce
// the rank-R positional factors Qp, Kp of one window size ("Rank-Factorized
// Implicit Neural Bias", omica.com.cn explainer section 2.2: coordinate
// encoding layer and implicit neural field; gist.science summaries, part A,
// mechanism steps 1-2).
//
// One workgroup handles ENC_TOK in-window positions in three phases that meet
// in LDS: Fourier features (2+4L per position), the ReLU hidden layer (hidden
// per position), then the two rank heads.  The whole job is at most a few tens
// of MFLOP per window size and runs once per size.  It keeps exact fp32
// semantics (correctly rounded coordinate division, precise sinf/cosf, one FMA
// chain per output in input order).  Each thread's dense-layer work is a serial
// chain of LDS reads and FMAs, so the time is latency: small workgroups (8
// positions; 1152 of them for a 96x96 window) put several on each CU to hide
// it, and the weights are staged in LDS once per workgroup when they fit.
#include "rib_device.hpp"
#include "rib_bwd.hpp"
#include "rib_launch.hpp"

#include <mutex>

namespace rib {

constexpr int ENC_TOK = 8;
constexpr int ENC_THREADS = 256;

// Fourier features of TOK consecutive positions starting at n0 (clamped to N-1):
// item (t, i) writes the raw coordinates (i == 0) or the sin/cos pair of
// frequency 2^(i-1) for both axes.  Coordinates are the correctly rounded fp32
// value of -1 + 2k/(ws-1).
static __device__ void fourier_features(int n0, int N, int ws, int L, int TOK, int F, float* feat) {
  const float den = (float)(ws - 1);
  for (int item = threadIdx.x; item < TOK * (L + 1); item += blockDim.x) {
    const int t = item / (L + 1), i = item % (L + 1);
    const int n = min(n0 + t, N - 1);
    const int iy = n / ws, ix = n - (n / ws) * ws;
    const float cy = (float)(2 * iy - (ws - 1)) / den;
    const float cx = (float)(2 * ix - (ws - 1)) / den;
    float* f = feat + t * F;
    if (i == 0) {
      f[0] = cy;
      f[1] = cx;
    } else {
      const float fr = ldexpf(1.0f, i - 1);
      float* g = f + 2 + 4 * (i - 1);
      g[0] = sinf(fr * cy);
      g[1] = sinf(fr * cx);
      g[2] = cosf(fr * cy);
      g[3] = cosf(fr * cx);
    }
  }
}

// Space-time windows (explainer section 6, video): position n = (it*ws + iy)*ws + ix
// of a wt x ws x ws window has coordinates (c_t, c_y, c_x), c_t = 0 for wt = 1;
// features [c_t, c_y, c_x], then for each frequency 2^(i-1): sin t, sin y,
// sin x, cos t, cos y, cos x.
static __device__ void fourier_features3(int n0, int N, int wt, int ws, int L, int TOK, int F, float* feat) {
  for (int item = threadIdx.x; item < TOK * (L + 1); item += blockDim.x) {
    const int t = item / (L + 1), i = item % (L + 1);
    const int n = min(n0 + t, N - 1);
    const int it = n / (ws * ws), r2 = n - it * ws * ws;
    const int iy = r2 / ws, ix = r2 - (r2 / ws) * ws;
    const float c[3] = {wt == 1 ? 0.0f : (float)(2 * it - (wt - 1)) / (float)(wt - 1),
                        (float)(2 * iy - (ws - 1)) / (float)(ws - 1), (float)(2 * ix - (ws - 1)) / (float)(ws - 1)};
    float* f = feat + t * F;
    if (i == 0) {
      f[0] = c[0];
      f[1] = c[1];
      f[2] = c[2];
    } else {
      const float fr = ldexpf(1.0f, i - 1);
      float* g = f + 3 + 6 * (i - 1);
      for (int a = 0; a < 3; ++a) {
        g[a] = sinf(fr * c[a]);
        g[3 + a] = cosf(fr * c[a]);
      }
    }
  }
}

// wt = 0: image windows (2 coordinates); wt >= 1: space-time windows of wt frames.
// kLdsW: the weights are first copied to LDS, so the two dense layers read
// their operands from LDS instead of waiting on a global load per FMA.  Every
// output keeps the same FMA order either way, so both variants give the same
// bits.
template <bool kLdsW>
__global__ void __launch_bounds__(ENC_THREADS)
encode_kernel(int wt, int ws, int L, int hidden, int R, const float* __restrict__ wg,
              float* __restrict__ qp, float* __restrict__ kp) {
  extern __shared__ float sm[];
  const int F = wt ? 3 + 6 * L : 2 + 4 * L;
  float* feat = sm;                     // [ENC_TOK][F]
  float* hid = sm + ENC_TOK * F;        // [ENC_TOK][hidden]
  const int N = (wt ? wt : 1) * ws * ws;
  const int n0 = blockIdx.x * ENC_TOK;

  const float* w = wg;
  if constexpr (kLdsW) {
    float* sw = hid + ENC_TOK * hidden;  // [F*hidden + hidden + 2*hidden*R]
    const int nw = F * hidden + hidden + 2 * hidden * R;
    for (int i = threadIdx.x; i < nw; i += ENC_THREADS) sw[i] = wg[i];
    w = sw;
  }

  if (wt) fourier_features3(n0, N, wt, ws, L, ENC_TOK, F, feat);
  else fourier_features(n0, N, ws, L, ENC_TOK, F, feat);
  __syncthreads();

  // Hidden layer h = ReLU(r W_h + b_h).
  const float* Wh = w;
  const float* bh = w + F * hidden;
  for (int item = threadIdx.x; item < ENC_TOK * hidden; item += ENC_THREADS) {
    const int t = item / hidden, j = item % hidden;
    const float* f = feat + t * F;
    float acc = bh[j];
    for (int k = 0; k < F; ++k) acc = fmaf(f[k], Wh[k * hidden + j], acc);
    hid[t * hidden + j] = fmaxf(acc, 0.0f);
  }
  __syncthreads();

  // Rank heads Qp = h Wp_q, Kp = h Wp_k (no bias).
  const float* Wq = bh + hidden;
  const float* Wk = Wq + hidden * R;
  for (int item = threadIdx.x; item < ENC_TOK * 2 * R; item += ENC_THREADS) {
    const int t = item / (2 * R), rr = item % (2 * R);
    const int n = n0 + t;
    if (n >= N) continue;
    const bool is_k = rr >= R;
    const int r = is_k ? rr - R : rr;
    const float* Wm = is_k ? Wk : Wq;
    const float* hh = hid + t * hidden;
    float acc = 0.0f;
    for (int j = 0; j < hidden; ++j) acc = fmaf(hh[j], Wm[j * R + r], acc);
    (is_k ? kp : qp)[n * R + r] = acc;
  }
}

// Weights at most this many bytes go through LDS (the headline encoder, L = 10,
// hidden 64, R = 16, holds 18.7 KB).
constexpr size_t ENC_LDS_W_MAX = 48 * 1024;

static hipError_t launch_encode_any(int wt, int ws, int L, int hidden, int R, const float* w, float* qp, float* kp,
                                    hipStream_t stream) {
  const int N = (wt ? wt : 1) * ws * ws;
  const int F = wt ? 3 + 6 * L : 2 + 4 * L;
  const int blocks = (N + ENC_TOK - 1) / ENC_TOK;
  const size_t lds = sizeof(float) * ENC_TOK * (size_t)(F + hidden);
  const size_t wbytes = sizeof(float) * ((size_t)F * hidden + hidden + 2 * (size_t)hidden * R);
  if (wbytes <= ENC_LDS_W_MAX)
    hipLaunchKernelGGL(encode_kernel<true>, dim3(blocks), dim3(ENC_THREADS), lds + wbytes, stream, wt, ws, L, hidden,
                       R, w, qp, kp);
  else
    hipLaunchKernelGGL(encode_kernel<false>, dim3(blocks), dim3(ENC_THREADS), lds, stream, wt, ws, L, hidden, R, w,
                       qp, kp);
  return hipGetLastError();
}

hipError_t launch_encode(int ws, int L, int hidden, int R, const float* w, float* qp, float* kp,
                         hipStream_t stream) {
  return launch_encode_any(0, ws, L, hidden, R, w, qp, kp, stream);
}

hipError_t launch_encode3d(int wt, int ws, int L, int hidden, int R, const float* w, float* qp, float* kp,
                           hipStream_t stream) {
  return launch_encode_any(wt, ws, L, hidden, R, w, qp, kp, stream);
}

// Backward of the encoder (explainer section 2.2, the same three layers): for
// upstream dQp, dKp ([ws*ws][R]),
//   dWp_q = sum_n h_n (x) dQp_n,   dWp_k = sum_n h_n (x) dKp_n
//   dpre_n = (dQp_n Wp_q^T + dKp_n Wp_k^T) * [pre_n > 0]
//   dW_h = sum_n r_n (x) dpre_n,   db_h = sum_n dpre_n
// The window's positions fall into chunks of EB_TOK; workgroup g of a grid of
// `rows` handles chunks g, g + rows, ... in that order and accumulates its
// partial gradient of the whole packed weight vector in its own row of the
// workspace (each thread owns the same weights in every chunk, so the row needs
// no clearing and no atomics); a second kernel sums the rows in a fixed order.
// With one chunk per workgroup (rows = chunk count) a row is one chunk's sum.
// pre_n is recomputed with the forward's exact arithmetic so the ReLU mask
// matches the forward's.
constexpr int EB_TOK = 16;

int encode_bwd_blocks(int ws) { return (ws * ws + EB_TOK - 1) / EB_TOK; }

__global__ void __launch_bounds__(ENC_THREADS)
encode_bwd_kernel(int ws, int L, int hidden, int R, const float* __restrict__ w, const float* __restrict__ dqp,
                  const float* __restrict__ dkp, float* __restrict__ work, int chunks) {
  extern __shared__ float sm[];
  const int F = 2 + 4 * L;
  float* feat = sm;                        // [EB_TOK][F]
  float* hid = feat + EB_TOK * F;          // [EB_TOK][hidden]  ReLU output
  float* dpre = hid + EB_TOK * hidden;     // [EB_TOK][hidden]
  float* gq = dpre + EB_TOK * hidden;      // [EB_TOK][R]
  float* gk = gq + EB_TOK * R;             // [EB_TOK][R]
  const int N = ws * ws;
  const float* Wh = w;
  const float* bh = w + F * hidden;
  const float* Wq = bh + hidden;
  const float* Wk = Wq + hidden * R;
  const int nw = F * hidden + hidden + 2 * hidden * R;
  float* out = work + (long)blockIdx.x * nw;
  for (int chunk = blockIdx.x; chunk < chunks; chunk += gridDim.x) {
    const bool first = chunk == (int)blockIdx.x;
    if (!first) __syncthreads();  // the previous chunk's last phase still reads the LDS arrays
    const int n0 = chunk * EB_TOK;
    fourier_features(n0, N, ws, L, EB_TOK, F, feat);
    for (int item = threadIdx.x; item < EB_TOK * R; item += ENC_THREADS) {
      const int t = item / R, r = item % R;
      const bool in = n0 + t < N;
      gq[item] = in ? dqp[(n0 + t) * R + r] : 0.0f;
      gk[item] = in ? dkp[(n0 + t) * R + r] : 0.0f;
    }
    __syncthreads();
    for (int item = threadIdx.x; item < EB_TOK * hidden; item += ENC_THREADS) {
      const int t = item / hidden, j = item % hidden;
      const float* f = feat + t * F;
      float acc = bh[j];
#pragma unroll 8
      for (int k = 0; k < F; ++k) acc = fmaf(f[k], Wh[k * hidden + j], acc);  // 8 weight loads in flight
      float dh = 0.0f;
#pragma unroll 8
      for (int r = 0; r < R; ++r) dh = fmaf(gq[t * R + r], Wq[j * R + r], fmaf(gk[t * R + r], Wk[j * R + r], dh));
      hid[item] = fmaxf(acc, 0.0f);
      dpre[item] = acc > 0.0f ? dh : 0.0f;
    }
    __syncthreads();
    // this chunk's sum for one weight
    auto partial = [&](int item) {
      float acc = 0.0f;
      if (item < F * hidden) {
        const int f = item / hidden, j = item % hidden;
        for (int t = 0; t < EB_TOK; ++t) acc = fmaf(feat[t * F + f], dpre[t * hidden + j], acc);
      } else if (item < F * hidden + hidden) {
        const int j = item - F * hidden;
        for (int t = 0; t < EB_TOK; ++t) acc += dpre[t * hidden + j];
      } else {
        const int k = item - F * hidden - hidden;
        const bool is_k = k >= hidden * R;
        const int jr = is_k ? k - hidden * R : k;
        const int j = jr / R, r = jr % R;
        const float* gg = is_k ? gk : gq;
        for (int t = 0; t < EB_TOK; ++t) acc = fmaf(hid[t * hidden + j], gg[t * R + r], acc);
      }
      return acc;
    };
    // two loops, so that the first chunk's stores come with no read of the row
    if (first) {
      for (int item = threadIdx.x; item < nw; item += ENC_THREADS) out[item] = partial(item);
    } else {
      for (int item = threadIdx.x; item < nw; item += ENC_THREADS) out[item] += partial(item);
    }
  }
}

// Sum of the workgroup rows: a workgroup takes 16 weights; thread (g, w)
// adds rows g, g+16, ... of weight w, then group sums are added in order g.
__global__ void __launch_bounds__(256)
encode_bwd_reduce_kernel(int nw, int blocks, const float* __restrict__ work, float* __restrict__ dw) {
  __shared__ float part[16][17];
  const int w = threadIdx.x & 15, g = threadIdx.x >> 4;
  const int item = blockIdx.x * 16 + w;
  float acc = 0.0f;
  if (item < nw)
    for (int b = g; b < blocks; b += 16) acc += work[(long)b * nw + item];
  part[g][w] = acc;
  __syncthreads();
  if (g == 0 && item < nw) {
    float sum = 0.0f;
    for (int k = 0; k < 16; ++k) sum += part[k][w];
    dw[item] = sum;
  }
}

hipError_t launch_encode_backward(int ws, int L, int hidden, int R, const float* w, const float* dqp,
                                  const float* dkp, float* dw, float* work, int rows, hipStream_t stream) {
  const int chunks = encode_bwd_blocks(ws);
  rows = rows < chunks ? rows : chunks;
  const int F = 2 + 4 * L;
  const int nw = F * hidden + hidden + 2 * hidden * R;
  const size_t lds = sizeof(float) * EB_TOK * (size_t)(F + 2 * hidden + 2 * R);
  hipLaunchKernelGGL(encode_bwd_kernel, dim3(rows), dim3(ENC_THREADS), lds, stream, ws, L, hidden, R, w,
                     dqp, dkp, work, chunks);
  hipLaunchKernelGGL(encode_bwd_reduce_kernel, dim3((nw + 15) / 16), dim3(256), 0, stream, nw, rows, work, dw);
  return hipGetLastError();
}

// Fixed workspace for callers that cannot allocate: one array per device,
// resident from the code object's load until the process ends.  Host code
// never passes the array's name to a kernel (on the host it is only a handle);
// it passes the device address that hipGetSymbolAddress returns, looked up
// once per device and kept.
static __device__ __align__(256) float scratch[ENC_SCRATCH_FLOATS];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex scratch_mutex;
float* scratch_ptr[MAX_DEVICES] = {};
}  // namespace

hipError_t encode_scratch(float** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    scratch_ptr[dev] = static_cast<float*>(p);
  }
  *ptr = scratch_ptr[dev];
  return hipSuccess;
}

int encode_scratch_rows(int ws, int L, int hidden, int R) {
  const long nw = (long)(2 + 4 * L) * hidden + hidden + 2L * hidden * R;
  const long fit = (long)ENC_SCRATCH_FLOATS / nw;
  const long chunks = encode_bwd_blocks(ws);
  return (int)(fit < chunks ? fit : chunks);
}

}  // namespace rib
