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
  const float* qp;  // [ws*ws][R] shared positional pair
  const float* kp;
  const void* o;
  const void* dout;
  // gradients
  void* dqc;
  void* dkc;
  void* dv;
  void* dg;
  float* dqp;  // [ws*ws][R]
  float* dkp;
  // workspace
  void* da;      // dO * sigmoid(G), NHWC, storage type
  float* dsum;   // D = dO . O per (token, head)
  float* lse;    // row log-sum-exp per (token, head)
  float* qrows;  // per-row dQp, [heads][B][H][W][R]
  float* krows;  // per-row dKp, same layout
  int B, H, W, heads, dh, R, ws;
};

hipError_t launch_attn_bwd_prep(const BwdArgs& a, bool bf16, hipStream_t stream);
// dq then dkv, fp32-register kernels for any dh <= 64, R <= 64
hipError_t launch_attn_bwd_rows(const BwdArgs& a, bool bf16, hipStream_t stream);
hipError_t launch_attn_bwd_reduce(const BwdArgs& a, hipStream_t stream);

// encoder backward: workspace of encode_bwd_blocks(ws) * weight count floats
int encode_bwd_blocks(int ws);
hipError_t launch_encode_backward(int ws, int L, int hidden, int R, const float* w, const float* dqp,
                                  const float* dkp, float* dw, float* work, hipStream_t stream);

}  // namespace rib
