// C-ABI entry points: argument validation, dispatch to the gfx950 kernels,
// status codes. Every check runs on the host before any HIP call, so invalid
// requests never reach the device. There is no fallback path: a request the
// kernels do not cover returns FA_ERR_UNSUPPORTED.
#include "fa.h"

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "fa_kernels.h"

#define FA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_detail[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return status;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return na && nb && a0 < b0 + nb && b0 < a0 + na;
}

struct Problem {
  long long bh = 0;
  long long elems = 0;   // B * H * N * d
  size_t tensor_bytes = 0;
  size_t lse_bytes = 0;
  bool empty = true;
};

// Shared scalar checks of fa_fwd / fa_bwd / fa_bwd_workspace_bytes.
int check_shape(int B, int H, int N, int d, int dtype, Problem* pr) {
  if (B < 0 || H < 0 || N < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "negative size (B=%d, H=%d, N=%d)", B, H, N);
  if (d <= 0) return fail(FA_ERR_INVALID_ARGUMENT, "head dimension d=%d must be positive", d);
  if (dtype != FA_BF16 && dtype != FA_FP32) return fail(FA_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension d=%d is not built (64 or 128)", d);
  const long long bh = (long long)B * H;
  if (bh > INT_MAX) return fail(FA_ERR_INVALID_ARGUMENT, "B*H=%lld exceeds INT_MAX", bh);
  const long long rows = bh * N;
  if (N > 0 && rows / N != bh) return fail(FA_ERR_INVALID_ARGUMENT, "B*H*N overflows");
  if (rows > (LLONG_MAX / 8) / d) return fail(FA_ERR_INVALID_ARGUMENT, "B*H*N*d overflows");
  // grids use 64-row blocks at the finest: B*H*ceil(N/64) work-groups must fit in int
  if (bh * ((N + 63LL) / 64) > INT_MAX)
    return fail(FA_ERR_INVALID_ARGUMENT, "problem needs more than INT_MAX work-groups");
  // the bf16 kernels address one head through 32-bit buffer offsets
  if (dtype == FA_BF16 && (long long)N * d * 2 > INT_MAX)
    return fail(FA_ERR_UNSUPPORTED, "N*d=%lld: one head exceeds 2 GiB", (long long)N * d);
  pr->bh = bh;
  pr->elems = rows * d;
  pr->tensor_bytes = (size_t)pr->elems * (dtype == FA_BF16 ? 2 : 4);
  pr->lse_bytes = (size_t)rows * 4;
  pr->empty = rows == 0;
  return FA_OK;
}

int check_flags(float scale, int causal) {
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARGUMENT, "scale must be finite");
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1 (got %d)", causal);
  return FA_OK;
}

int check_ptr(const void* p, const char* name) {
  if (!p) return fail(FA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned16(p)) return fail(FA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
  return FA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return FA_OK;
  return fail(FA_ERR_HIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
}

}  // namespace

FA_EXPORT int fa_version(void) { return 100; }

FA_EXPORT const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARGUMENT: return "FA_ERR_INVALID_ARGUMENT";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    default: return "FA_UNKNOWN_STATUS";
  }
}

FA_EXPORT const char* fa_last_error_detail(void) { return g_detail; }

FA_EXPORT int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int N, int d,
                     float scale, int causal, int dtype, void* stream) {
  g_detail[0] = '\0';
  Problem pr;
  int st = check_shape(B, H, N, d, dtype, &pr);
  if (st != FA_OK) return st;
  if ((st = check_flags(scale, causal)) != FA_OK) return st;
  if (pr.empty) return FA_OK;
  if ((st = check_ptr(Q, "Q")) || (st = check_ptr(K, "K")) || (st = check_ptr(V, "V")) ||
      (st = check_ptr(O, "O")) || (st = check_ptr(LSE, "LSE")))
    return st;
  const size_t tb = pr.tensor_bytes, lb = pr.lse_bytes;
  const void* ins[3] = {Q, K, V};
  for (const void* in : ins) {
    if (overlap(O, tb, in, tb)) return fail(FA_ERR_INVALID_ARGUMENT, "O overlaps an input");
    if (overlap(LSE, lb, in, tb)) return fail(FA_ERR_INVALID_ARGUMENT, "LSE overlaps an input");
  }
  if (overlap(O, tb, LSE, lb)) return fail(FA_ERR_INVALID_ARGUMENT, "O overlaps LSE");

  fa::FwdArgs a{Q, K, V, O, LSE, (int)pr.bh, N, d, scale, causal == 1, (hipStream_t)stream};
  const hipError_t e = dtype == FA_BF16 ? fa::launch_fwd_bf16(a) : fa::launch_fwd_f32(a);
  return hip_status(e, "fa_fwd launch");
}

FA_EXPORT size_t fa_bwd_workspace_bytes(int B, int H, int N, int d, int dtype) {
  Problem pr;
  if (check_shape(B, H, N, d, dtype, &pr) != FA_OK || dtype != FA_BF16 || pr.empty) return 0;
  return fa::bwd_workspace_bytes(pr.bh, N);
}

FA_EXPORT int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE,
                     void* dQ, void* dK, void* dV, int B, int H, int N, int d, float scale, int causal, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream) {
  g_detail[0] = '\0';
  Problem pr;
  int st = check_shape(B, H, N, d, dtype, &pr);
  if (st != FA_OK) return st;
  if ((st = check_flags(scale, causal)) != FA_OK) return st;
  if (dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "fa_bwd is built for bf16 only");
  if (pr.empty) return FA_OK;
  if ((st = check_ptr(Q, "Q")) || (st = check_ptr(K, "K")) || (st = check_ptr(V, "V")) ||
      (st = check_ptr(O, "O")) || (st = check_ptr(dO, "dO")) || (st = check_ptr(LSE, "LSE")) ||
      (st = check_ptr(dQ, "dQ")) || (st = check_ptr(dK, "dK")) || (st = check_ptr(dV, "dV")) ||
      (st = check_ptr(workspace, "workspace")))
    return st;
  const size_t need = fa_bwd_workspace_bytes(B, H, N, d, dtype);
  if (workspace_bytes < need)
    return fail(FA_ERR_INVALID_ARGUMENT, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes,
                need);
  const size_t tb = pr.tensor_bytes, lb = pr.lse_bytes;
  struct Buf {
    const void* p;
    size_t n;
    const char* name;
  };
  const Buf ins[6] = {{Q, tb, "Q"}, {K, tb, "K"}, {V, tb, "V"}, {O, tb, "O"}, {dO, tb, "dO"}, {LSE, lb, "LSE"}};
  const Buf outs[4] = {{dQ, tb, "dQ"}, {dK, tb, "dK"}, {dV, tb, "dV"}, {workspace, need, "workspace"}};
  for (const Buf& o : outs) {
    for (const Buf& i : ins)
      if (overlap(o.p, o.n, i.p, i.n)) return fail(FA_ERR_INVALID_ARGUMENT, "%s overlaps %s", o.name, i.name);
    for (const Buf& o2 : outs)
      if (&o2 != &o && overlap(o.p, o.n, o2.p, o2.n))
        return fail(FA_ERR_INVALID_ARGUMENT, "%s overlaps %s", o.name, o2.name);
  }
  fa::BwdArgs a{Q, K, V, O, dO, LSE, dQ, dK, dV, (float*)workspace, (int)pr.bh, N, d, scale, causal == 1,
                (hipStream_t)stream};
  return hip_status(fa::launch_bwd_bf16(a), "fa_bwd launch");
}
