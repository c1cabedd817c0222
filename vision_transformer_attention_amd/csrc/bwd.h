// Arguments of the float32 backward kernels (bwd.hip), filled on the host by
// rpe_attn_bwd.  Pure C++ (no HIP types).
#pragma once

#include <cstdint>

namespace rpe {

struct BwdArgs {
  // inputs ([B][H][N][D] in the input dtype; tables [H or 1][nb](x D))
  const void* q; const void* k; const void* v; const void* dout;
  const void* rq; const void* rk; const void* rv;
  const float* bias;
  const float* lse;         // [B][H][N], natural log, from the forward
  // outputs (float32)
  float* dq; float* dk; float* dv;
  float* dbias; float* drq; float* drk; float* drv;
  // workspace
  float* P; float* dL;      // [n_units][T][Ts]
  float* Wq; float* Wk; float* Wv;   // [n_units][T][nb] (null when not needed)
  const int16_t* bmap;      // [T][T] table row of each pair of one unit (-1: prefix pair)
  const int16_t* bmap1;     // [T][T] its second table row (Cross), or null: one row per pair
  // geometry
  int bf16;
  int D, N, H, U, T;
  int Ts;                   // row stride of P and dL: T rounded up to a multiple of 32
  int npre;                 // prefix tokens
  int C;                    // positioned columns of a unit
  int M;                    // window side (0: global)
  int gw;                   // grid width
  int wpr;                  // windows per grid row
  int nb;                   // table rows (S*S Product, 2S Cross, S undirected)
  int tables_per_head;
  int64_t n_units;          // B * H * U
  float scale;              // logit scale s
};

// Workspace of the allocation-free backward (rpe_attn_bwd_noalloc): a device
// array of this many bytes per GPU, owned by the library (bwd.hip).
constexpr uint64_t kBwdScratchBytes = uint64_t{64} << 20;

// Device address of that array on the device `stream` (a hipStream_t, NULL: the
// current device) belongs to; looked up once per device.  Returns a hipError_t.
int bwd_scratch(void* stream, void** ptr);

}  // namespace rpe
