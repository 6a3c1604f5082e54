// Host-side launchers of the attention kernels (internal to the library).
// Arguments are already validated by the C-ABI layer: pointers are non-null
// device pointers, the problem is not empty, d is a built head dimension,
// strides keep every 16-byte access aligned and every head's rows within
// 32-bit buffer offsets, and window bounds are clamped to [-1, nq + nk].
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

// Element type codes (the values of the C ABI's fa_dtype).
constexpr int kDtypeBf16 = 0;
constexpr int kDtypeF32 = 1;
constexpr int kDtypeF16 = 2;

// Mask kinds, a template argument of the 16-bit kernels: no mask, an upper
// bound only (causal-like: key j <= i + nk - nq + wr), or both bounds. The
// upper-only kind carries no lower-bound test at all.
constexpr int kMaskNone = 0;
constexpr int kMaskUpper = 1;
constexpr int kMaskBand = 2;

// Strides of one [B, H, rows, d] tensor, in elements; d is contiguous.
struct Strides {
  long long b, h, r;
};

// Shape and mask shared by the forward and backward passes. Query i is
// aligned with key i + nk - nq; with a band, key j is visible to query i iff
// i + nk - nq - wl <= j <= i + nk - nq + wr, where a bound of -1 is absent.
struct Geometry {
  int batch, heads;
  int nq, nk, d;
  int wl, wr;
  bool banded() const { return wl >= 0 || wr >= 0; }
  int mask_kind() const { return !banded() ? kMaskNone : wl < 0 ? kMaskUpper : kMaskBand; }
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // contiguous [B, H, nq]
  const float* bias;  // additive bias on the scaled scores, or null
  Strides sq, sk, sv, so, sbias;  // sbias: batch, head, query-row strides; keys contiguous
  Geometry g;
  float scale;  // multiplies Q K^T before the softmax
  int dtype;
  hipStream_t stream;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;  // contiguous [B, H, nq]
  const float* bias;  // additive bias on the scaled scores, or null
  void* dq;
  void* dk;
  void* dv;
  float* workspace;  // bwd_workspace_bytes(B * H, nq) bytes: per-row statistics
  Strides sq, sk, sv, so, sdo, sdq, sdk, sdv, sbias;
  Geometry g;
  float scale;
  int dtype;
  hipStream_t stream;
};

hipError_t launch_fwd_mfma(const FwdArgs& a);  // bf16 and fp16
hipError_t launch_fwd_f32(const FwdArgs& a);
hipError_t launch_bwd_mfma(const BwdArgs& a);  // bf16 and fp16
// Workspace of the backward: two floats per query row, rows padded to 64 per head.
size_t bwd_workspace_bytes(long long bh, int nq);

// Size of the library's own device scratch (the backward's workspace for the
// entry point that allocates nothing), and its address on the current device
// (looked up once per device; every call on a device shares it).
constexpr size_t kScratchBytes = size_t(16) << 20;
hipError_t scratch_address(void** out);

}  // namespace fa
