// Host-side launchers of the attention kernels (internal to the library).
// Arguments are already validated by the C-ABI layer: pointers are non-null
// device pointers, bh * n > 0, d is a built head dimension.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int bh;       // B * H independent heads
  int n;        // sequence length (queries = keys)
  int d;        // head dimension
  float scale;  // multiplies Q K^T before the softmax
  bool causal;
  hipStream_t stream;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* workspace;  // bwd_workspace_bytes(bh, n) bytes: per-row statistics
  int bh;
  int n;
  int d;
  float scale;
  bool causal;
  hipStream_t stream;
};

hipError_t launch_fwd_bf16(const FwdArgs& a);
hipError_t launch_fwd_f32(const FwdArgs& a);
hipError_t launch_bwd_bf16(const BwdArgs& a);
// Workspace of fa_bwd: two floats per query row, rows padded to 64 per head.
size_t bwd_workspace_bytes(long long bh, int n);

}  // namespace fa
