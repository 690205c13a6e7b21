// encode.hip -- the coordinate encoder and implicit neural field that produce
// the rank-R positional factors Qp, Kp of one window size ("Rank-Factorized
// Implicit Neural Bias", omica.com.cn explainer section 2.2: coordinate
// encoding layer and implicit neural field; gist.science summaries, part A,
// mechanism steps 1-2).
//
// One workgroup handles TOK in-window positions in three phases that meet in
// LDS: Fourier features (2+4L per position), the ReLU hidden layer (hidden per
// position), then the two rank heads.  The whole job is at most a few tens of
// MFLOP per window size and runs once per size, so it is written for clarity
// and exact fp32 semantics (correctly rounded coordinate division, precise
// sinf/cosf), not for speed.
#include "rib_device.hpp"
#include "rib_launch.hpp"

namespace rib {

constexpr int ENC_TOK = 32;
constexpr int ENC_THREADS = 256;

__global__ void __launch_bounds__(ENC_THREADS)
encode_kernel(int ws, int L, int hidden, int R, const float* __restrict__ w,
              float* __restrict__ qp, float* __restrict__ kp) {
  extern __shared__ float sm[];
  const int F = 2 + 4 * L;
  float* feat = sm;                     // [ENC_TOK][F]
  float* hid = sm + ENC_TOK * F;        // [ENC_TOK][hidden]
  const int N = ws * ws;
  const int n0 = blockIdx.x * ENC_TOK;
  const float den = (float)(ws - 1);

  // Fourier features: item (t, i) writes the raw coordinates (i == 0) or the
  // sin/cos pair of frequency 2^(i-1) for both axes.
  for (int item = threadIdx.x; item < ENC_TOK * (L + 1); item += ENC_THREADS) {
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

hipError_t launch_encode(int ws, int L, int hidden, int R, const float* w, float* qp, float* kp,
                         hipStream_t stream) {
  const int N = ws * ws;
  const int blocks = (N + ENC_TOK - 1) / ENC_TOK;
  const size_t lds = sizeof(float) * ENC_TOK * (size_t)(2 + 4 * L + hidden);
  hipLaunchKernelGGL(encode_kernel, dim3(blocks), dim3(ENC_THREADS), lds, stream, ws, L, hidden, R,
                     w, qp, kp);
  return hipGetLastError();
}

}  // namespace rib
