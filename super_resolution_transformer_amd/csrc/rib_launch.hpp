// rib_launch.hpp -- internal launchers behind the C ABI (arguments already validated).
#pragma once
#include <hip/hip_runtime.h>

namespace rib {

struct AttnArgs {
  const void* qc;
  const void* kc;
  const void* v;
  const void* g;
  const float* qp;
  const float* kp;
  void* o;
  int B, H, W, heads, dh, R, ws;
  long tstride;  // floats between the (qp, kp) tables of consecutive heads; 0 = one shared pair
  float* lse;    // optional: row log-sum-exp per (token, head), natural log
  int T = 1;     // frames of a [B][T][H][W][C] video map (1: images)
  int wt = 1;    // frames per space-time window (1: 2-D windows)
};

hipError_t launch_encode(int ws, int L, int hidden, int R, const float* w, float* qp, float* kp,
                         hipStream_t stream);
// space-time encoder over wt x ws x ws windows (3 coordinates, 3 + 6L features)
hipError_t launch_encode3d(int wt, int ws, int L, int hidden, int R, const float* w, float* qp, float* kp,
                           hipStream_t stream);

// tiled bf16 kernel with LayerNorm + the Q projection of x fused into its Q~ build
// ((dh, R) in {(30, 16), (16, 16)}, C = heads * dh <= 192); a.qc is not read
hipError_t launch_attn_bf16_lnq(const AttnArgs& a, const void* x, const float* gamma, const float* beta,
                                const float* w, const float* bias, float eps, hipStream_t stream);

// fp32 path: any dh <= 64, R <= 64.
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t stream);

// bf16 MFMA path: returns hipErrorInvalidValue if (dh, R) has no compiled variant.
bool attn_bf16_supported(int dh, int R);
hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t stream);
// several independent bf16 calls sharing (dh, R) in as few launches as possible
// (one per kernel kind and per 8 calls); n <= 64
hipError_t launch_attn_bf16_multi(const AttnArgs* calls, int n, hipStream_t stream);

struct GateArgs {
  const void* x;
  const float* dw_w;
  const float* dw_b;
  const float* pw_w;
  const float* pw_b;
  void* g;
  int B, H, W, C;
};

// CLA gate producer; bf16 = false: fp32 maps.  C even, C <= 256.
hipError_t launch_cla_gate(const GateArgs& a, bool bf16, hipStream_t stream);

// compute units of the current device (queried on every call)
int device_cus();

struct LnQkvArgs {
  const void* x;
  const float* gamma;
  const float* beta;
  const float* w;     // [C][3C]
  const float* bias;  // [3C]
  void* q;
  void* k;
  void* v;
  void* xn;           // optional (nullptr)
  int B, H, W, C;
  float eps;
};

// LayerNorm + Q/K/V projection; bf16 = false: fp32 maps.  C <= 256.
bool ln_qkv_mfma(int C);
hipError_t launch_ln_qkv(const LnQkvArgs& a, bool bf16, hipStream_t stream);

}  // namespace rib
