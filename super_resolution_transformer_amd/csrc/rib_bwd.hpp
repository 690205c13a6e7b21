// rib_bwd.hpp -- internal launchers of the backward passes (arguments already validated).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rib {

struct BwdArgs {
  // forward inputs and output, upstream gradient: NHWC maps of the storage type
  const void* qc;
  const void* kc;
  const void* v;
  const void* g;
  const float* qp;  // [ws*ws][R] shared positional pair, or [heads][ws*ws][R] (tstride > 0)
  const float* kp;
  const void* o;
  const float* lse;  // row log-sum-exp per (token, head), natural log, from the forward
  const void* dout;
  // gradients
  void* dqc;
  void* dkc;
  void* dv;
  void* dg;
  float* dqp;  // [ws*ws][R] summed over heads, or [heads][ws*ws][R] (tab_heads = heads)
  float* dkp;
  // workspace
  void* da;      // dO * sigmoid(G), NHWC, storage type
  float* dsum;   // D = dO . O per (token, head)
  float* qrows;  // per-row dQp, [heads][B][H][W][R]
  float* krows;  // per-row dKp, same layout
  uint32_t* pk;  // matrix-core path: packed key-side operand rows (tile images)
  uint32_t* pq;  // matrix-core path: packed query-side operand rows
  int B, H, W, heads, dh, R, ws;
  int tu;        // 64-row tiles per unit in the packed images
  long tstride = 0;   // floats between the positional pairs of consecutive heads (0: one shared pair)
  int tab_heads = 1;  // table gradients per head (heads) or summed over heads (1)
};

inline int bwd_tiles_per_unit(int ws) { return (ws * ws + 63) / 64; }

// Decode of a workgroup's logical index into (b, wy, wx, h, row block) and the
// real-token enumeration of a window: real index r -> (iy, ix) = (r / nx, r % nx).
struct Unit {
  int b, wy, wx, h, blk, nx, n_real;
};

__device__ __forceinline__ bool decode_unit(int logical, const BwdArgs& a, int rows_per_block, Unit& u) {
  const int nWy = (a.H + a.ws - 1) / a.ws, nWx = (a.W + a.ws - 1) / a.ws;
  const int rblocks = (a.ws * a.ws + rows_per_block - 1) / rows_per_block;
  int t = logical;
  u.blk = t % rblocks; t /= rblocks;
  u.h = t % a.heads; t /= a.heads;
  u.wx = t % nWx; t /= nWx;
  u.wy = t % nWy;
  u.b = t / nWy;
  const int ny = min(a.ws, a.H - u.wy * a.ws);
  u.nx = min(a.ws, a.W - u.wx * a.ws);
  u.n_real = ny * u.nx;
  return u.blk * rows_per_block < u.n_real;
}

// token index (b, y, x) and in-window index n of real token r of the unit
__device__ __forceinline__ void locate(const Unit& u, const BwdArgs& a, int r, long& tok, int& n) {
  const int iy = r / u.nx, ix = r - iy * u.nx;
  tok = ((long)u.b * a.H + u.wy * a.ws + iy) * a.W + u.wx * a.ws + ix;
  n = iy * a.ws + ix;
}

inline int bwd_units(const BwdArgs& a, int rows_per_block) {
  const int nWy = (a.H + a.ws - 1) / a.ws, nWx = (a.W + a.ws - 1) / a.ws;
  return a.B * nWy * nWx * a.heads * ((a.ws * a.ws + rows_per_block - 1) / rows_per_block);
}

hipError_t launch_attn_bwd_prep(const BwdArgs& a, bool bf16, hipStream_t stream);
// dq then dkv, fp32-register kernels for any dh <= 64, R <= 64
hipError_t launch_attn_bwd_rows(const BwdArgs& a, bool bf16, hipStream_t stream);
hipError_t launch_attn_bwd_reduce(const BwdArgs& a, hipStream_t stream);
// dq then dkv on bf16 matrix cores; false if (dh, R) has no compiled variant
bool attn_bwd_bf16_supported(int dh, int R);
// bytes of one packed operand image (pk or pq) for this problem
size_t attn_bwd_bf16_image_bytes(int B, int H, int W, int heads, int ws);
hipError_t launch_attn_bwd_bf16(const BwdArgs& a, hipStream_t stream);

// encoder backward: `rows` workgroups (at most encode_bwd_blocks(ws), one per
// position chunk when equal) each fill one row of weight-count floats of `work`
int encode_bwd_blocks(int ws);
hipError_t launch_encode_backward(int ws, int L, int hidden, int R, const float* w, const float* dqp,
                                  const float* dkp, float* dw, float* work, int rows, hipStream_t stream);
// the per-device fixed workspace (4 MiB) and the rows of it one problem uses
// (0 when one row does not fit)
constexpr long ENC_SCRATCH_FLOATS = 1L << 20;
hipError_t encode_scratch(float** ptr);
int encode_scratch_rows(int ws, int L, int hidden, int R);

}  // namespace rib
