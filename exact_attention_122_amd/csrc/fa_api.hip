// C-ABI entry points: argument validation, dispatch to the gfx950 kernels,
// status codes. Every check runs on the host before any HIP call, so invalid
// requests never reach the device. There is no fallback path: a request the
// kernels do not cover returns FA_ERR_UNSUPPORTED.
#include "fa.h"

#include <algorithm>
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

int elem_bytes(int dtype) { return dtype == FA_FP32 ? 4 : 2; }

// Byte range [lo, hi) that a tensor's elements can touch.
struct Extent {
  uintptr_t lo = 0, hi = 0;
  bool empty() const { return hi <= lo; }
};

bool overlap(const Extent& a, const Extent& b) { return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi; }

// One [B, H, rows, d] operand as the caller describes it.
struct Tensor {
  const void* ptr;
  const char* name;
  int rows;
  fa::Strides st;
  Extent ext;
};

struct Problem {
  int B = 0, H = 0, nq = 0, nk = 0, d = 0, dtype = 0;
  long long bh = 0;
};

int check_dims(int B, int H, int nq, int nk, int d, int dtype, Problem* pr) {
  if (B < 0 || H < 0 || nq < 0 || nk < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "negative size (B=%d, H=%d, Nq=%d, Nk=%d)", B, H, nq, nk);
  if (d <= 0) return fail(FA_ERR_INVALID_ARGUMENT, "head dimension d=%d must be positive", d);
  if (dtype != FA_BF16 && dtype != FA_FP32 && dtype != FA_FP16)
    return fail(FA_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  if (d != 32 && d != 64 && d != 96 && d != 128 && d != 256)
    return fail(FA_ERR_UNSUPPORTED, "head dimension d=%d is not built (32, 64, 96, 128 or 256)", d);
  if (dtype == FA_FP32 && d > 128)
    return fail(FA_ERR_UNSUPPORTED, "head dimension d=%d is not built for fp32 (at most 128)", d);
  const long long bh = (long long)B * H;
  if (bh > INT_MAX) return fail(FA_ERR_INVALID_ARGUMENT, "B*H=%lld exceeds INT_MAX", bh);
  const long long n = std::max(nq, nk);
  // the grids use 64-row blocks at the finest: B*H*ceil(N/64) work-groups must fit in int
  if (bh * ((n + 63) / 64) > INT_MAX) return fail(FA_ERR_INVALID_ARGUMENT, "problem needs more than INT_MAX work-groups");
  // row indices and band bounds stay far from int overflow
  if (n > (1 << 28)) return fail(FA_ERR_UNSUPPORTED, "sequence length %lld exceeds 2^28", n);
  pr->B = B, pr->H = H, pr->nq = nq, pr->nk = nk, pr->d = d, pr->dtype = dtype, pr->bh = bh;
  return FA_OK;
}

int check_scale(float scale) {
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARGUMENT, "scale must be finite");
  return FA_OK;
}

int check_window(int wl, int wr) {
  if (wl < -1 || wr < -1)
    return fail(FA_ERR_INVALID_ARGUMENT, "window bounds must be -1 (absent) or >= 0 (got %d, %d)", wl, wr);
  return FA_OK;
}

// Fills t->st (contiguous when `strides` is NULL) and t->ext, and checks what
// the kernels assume of a strided operand: d contiguous, non-negative strides,
// rows at least d apart, 16-byte aligned rows and bases, offsets of one head
// within 32-bit buffer offsets, and (outputs) no two elements at one address.
int describe(Tensor* t, const long long* strides, const Problem& pr, bool output) {
  const long long esz = elem_bytes(pr.dtype);
  if (strides) {
    t->st = fa::Strides{strides[0], strides[1], strides[2]};
  } else {
    t->st = fa::Strides{(long long)pr.H * t->rows * pr.d, (long long)t->rows * pr.d, (long long)pr.d};
  }
  // the stride of a dimension of size 1 is never used: normalise it (to 0,
  // or to d for rows, which keeps rows past the end outside the buffer)
  if (pr.B == 1) t->st.b = 0;
  if (pr.H == 1) t->st.h = 0;
  if (t->rows == 1) t->st.r = pr.d;
  const fa::Strides& s = t->st;
  const long long count = pr.bh * t->rows;
  t->ext = Extent{};
  if (count == 0) return FA_OK;  // no element: the pointer is never used
  if (!t->ptr) return fail(FA_ERR_INVALID_ARGUMENT, "%s is NULL", t->name);
  if (!aligned16(t->ptr)) return fail(FA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", t->name);
  if (s.b < 0 || s.h < 0 || s.r < 0)
    return fail(FA_ERR_UNSUPPORTED, "%s has a negative stride (%lld, %lld, %lld)", t->name, s.b, s.h, s.r);
  if (s.r < pr.d)
    return fail(FA_ERR_UNSUPPORTED, "%s row stride %lld is below d=%d (rows would overlap)", t->name, s.r, pr.d);
  const long long unit = 16 / esz;  // elements per 16 bytes
  if (s.b % unit || s.h % unit || s.r % unit)
    return fail(FA_ERR_UNSUPPORTED, "%s strides (%lld, %lld, %lld) are not multiples of %lld elements (16 bytes)",
                t->name, s.b, s.h, s.r, unit);
  // one head's rows, plus a tile of zero-filled rows past the end, must stay
  // addressable with 32-bit byte offsets
  if ((long long)(t->rows + 256) * s.r * esz > INT_MAX)
    return fail(FA_ERR_UNSUPPORTED, "%s: one head spans more than 2 GiB of addresses", t->name);
  if (s.b > LLONG_MAX / 4 / std::max(pr.B, 1) || s.h > LLONG_MAX / 4 / std::max(pr.H, 1))
    return fail(FA_ERR_INVALID_ARGUMENT, "%s strides overflow", t->name);
  const long long span = ((long long)(pr.B - 1) * s.b + (long long)(pr.H - 1) * s.h +
                          (long long)(t->rows - 1) * s.r + pr.d) * esz;
  t->ext.lo = reinterpret_cast<uintptr_t>(t->ptr);
  t->ext.hi = t->ext.lo + (uintptr_t)span;
  if (output) {
    // Injective layout: sorted by stride, every dimension of size > 1 must
    // step past everything the smaller dimensions reach.
    struct Dim {
      long long stride, size;
    } dims[4] = {{1, pr.d}, {s.r, t->rows}, {s.h, pr.H}, {s.b, pr.B}};
    std::sort(dims, dims + 4, [](const Dim& a, const Dim& b) { return a.stride < b.stride; });
    long long reach = 0;  // largest offset reachable with the dimensions so far
    for (const Dim& dm : dims) {
      if (dm.size <= 1) continue;
      if (dm.stride <= reach)
        return fail(FA_ERR_INVALID_ARGUMENT, "%s: strides (%lld, %lld, %lld) map two elements to one address",
                    t->name, s.b, s.h, s.r);
      reach += dm.stride * (dm.size - 1);
    }
  }
  return FA_OK;
}

// The optional fp32 bias [B, H, Nq, Nk] (keys contiguous): strides >= 0 (0
// broadcasts), rows 16-byte aligned. Fills *st and *ext; a null bias is none.
int describe_bias(const float* bias, const long long* strides, const Problem& pr, fa::Strides* st, Extent* ext) {
  *ext = Extent{};
  const long long nk = pr.nk;
  *st = strides ? fa::Strides{strides[0], strides[1], strides[2]}
                : fa::Strides{(long long)pr.H * pr.nq * nk, (long long)pr.nq * nk, nk};
  // strides of dimensions of size 1 are never used
  if (pr.B == 1) st->b = 0;
  if (pr.H == 1) st->h = 0;
  if (pr.nq == 1) st->r = 0;
  if (!bias || pr.bh * pr.nq * nk == 0) return FA_OK;
  if (!aligned16(bias)) return fail(FA_ERR_INVALID_ARGUMENT, "bias is not 16-byte aligned");
  if (st->b < 0 || st->h < 0 || st->r < 0)
    return fail(FA_ERR_UNSUPPORTED, "bias has a negative stride (%lld, %lld, %lld)", st->b, st->h, st->r);
  if (st->b % 4 || st->h % 4 || st->r % 4)
    return fail(FA_ERR_UNSUPPORTED, "bias strides (%lld, %lld, %lld) are not multiples of 4 floats (16 bytes)", st->b,
                st->h, st->r);
  if (st->b > LLONG_MAX / 8 / std::max(pr.B, 1) || st->h > LLONG_MAX / 8 / std::max(pr.H, 1) ||
      st->r > LLONG_MAX / 8 / std::max(pr.nq, 1))
    return fail(FA_ERR_INVALID_ARGUMENT, "bias strides overflow");
  // the kernels index a bias row with a 32-bit row stride
  if (st->r > INT_MAX)
    return fail(FA_ERR_UNSUPPORTED, "bias row stride %lld exceeds 2^31 - 1 floats", st->r);
  const long long span =
      ((long long)(pr.B - 1) * st->b + (long long)(pr.H - 1) * st->h + (long long)(pr.nq - 1) * st->r + nk) * 4;
  ext->lo = reinterpret_cast<uintptr_t>(bias);
  ext->hi = ext->lo + (uintptr_t)span;
  return FA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return FA_OK;
  return fail(FA_ERR_HIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
}

// Shared body of fa_fwd and fa_fwd_ex.
int forward(const void* Q, const void* K, const void* V, void* O, float* LSE, const Problem& pr,
            const long long* q_strides, const long long* k_strides, const long long* v_strides,
            const long long* o_strides, const float* bias, const long long* bias_strides, float scale, int wl, int wr,
            void* stream) {
  int st;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if ((st = check_window(wl, wr)) != FA_OK) return st;
  if (pr.bh * pr.nq == 0) return FA_OK;  // no query row: nothing to compute
  Tensor q{Q, "Q", pr.nq}, k{K, "K", pr.nk}, v{V, "V", pr.nk}, o{O, "O", pr.nq};
  if ((st = describe(&q, q_strides, pr, false)) || (st = describe(&k, k_strides, pr, false)) ||
      (st = describe(&v, v_strides, pr, false)) || (st = describe(&o, o_strides, pr, true)))
    return st;
  if (!LSE) return fail(FA_ERR_INVALID_ARGUMENT, "LSE is NULL");
  if (!aligned16(LSE)) return fail(FA_ERR_INVALID_ARGUMENT, "LSE is not 16-byte aligned");
  fa::Strides sbias;
  Extent bext;
  if ((st = describe_bias(bias, bias_strides, pr, &sbias, &bext)) != FA_OK) return st;
  if (bias && pr.dtype == FA_FP32) return fail(FA_ERR_UNSUPPORTED, "a bias is built for bf16 and fp16 only");
  const Extent lse{reinterpret_cast<uintptr_t>(LSE), reinterpret_cast<uintptr_t>(LSE) + (uintptr_t)(pr.bh * pr.nq * 4)};
  Tensor bt{bias, "bias", pr.nq, sbias, bext};
  for (const Tensor* in : {&q, &k, &v, &bt}) {
    if (overlap(o.ext, in->ext)) return fail(FA_ERR_INVALID_ARGUMENT, "O overlaps %s", in->name);
    if (overlap(lse, in->ext)) return fail(FA_ERR_INVALID_ARGUMENT, "LSE overlaps %s", in->name);
  }
  if (overlap(o.ext, lse)) return fail(FA_ERR_INVALID_ARGUMENT, "O overlaps LSE");

  fa::FwdArgs a;
  a.q = Q, a.k = K, a.v = V, a.o = O, a.lse = LSE;
  a.bias = (bias && pr.nk > 0) ? bias : nullptr;
  a.sq = q.st, a.sk = k.st, a.sv = v.st, a.so = o.st, a.sbias = sbias;
  const int wmax = pr.nq + pr.nk;
  a.g = fa::Geometry{pr.B, pr.H, pr.nq, pr.nk, pr.d, std::min(wl, wmax), std::min(wr, wmax)};
  a.scale = scale;
  a.dtype = pr.dtype;
  a.stream = (hipStream_t)stream;
  const hipError_t e = pr.dtype == FA_FP32 ? fa::launch_fwd_f32(a) : fa::launch_fwd_mfma(a);
  return hip_status(e, "forward launch");
}

size_t workspace_bytes(const Problem& pr) {
  if (pr.dtype == FA_FP32 || pr.bh * pr.nq == 0) return 0;
  return fa::bwd_workspace_bytes(pr.bh, pr.nq);
}

// Shared body of fa_bwd, fa_bwd_ex and fa_bwd_noalloc. With use_scratch the
// workspace arguments are ignored: after every other check, the statistics go
// to the library's own device scratch (kScratchBytes at most).
int backward(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE, void* dQ,
             void* dK, void* dV, const Problem& pr, const long long* const strides[8], const float* bias,
             const long long* bias_strides, float scale, int wl, int wr, void* workspace,
             size_t workspace_bytes_given, void* stream, bool use_scratch = false) {
  int st;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if ((st = check_window(wl, wr)) != FA_OK) return st;
  if (pr.dtype == FA_FP32) return fail(FA_ERR_UNSUPPORTED, "the backward pass is built for bf16 and fp16 only");
  if (pr.bh * std::max(pr.nq, pr.nk) == 0) return FA_OK;  // no element in any output
  Tensor q{Q, "Q", pr.nq}, k{K, "K", pr.nk}, v{V, "V", pr.nk}, o{O, "O", pr.nq}, g{dO, "dO", pr.nq};
  Tensor dq{dQ, "dQ", pr.nq}, dk{dK, "dK", pr.nk}, dv{dV, "dV", pr.nk};
  Tensor* ins[5] = {&q, &k, &v, &o, &g};
  Tensor* outs[3] = {&dq, &dk, &dv};
  for (int i = 0; i < 5; ++i)
    if ((st = describe(ins[i], strides[i], pr, false)) != FA_OK) return st;
  for (int i = 0; i < 3; ++i)
    if ((st = describe(outs[i], strides[5 + i], pr, true)) != FA_OK) return st;
  const size_t need = workspace_bytes(pr);
  Extent lse{}, ws{};
  if (use_scratch && need > fa::kScratchBytes)
    return fail(FA_ERR_UNSUPPORTED,
                "the problem needs %zu bytes of row statistics, more than the %zu-byte scratch of fa_bwd_noalloc "
                "(B*H*ceil(N/64)*64 must be at most %zu): use fa_bwd with a workspace",
                need, fa::kScratchBytes, fa::kScratchBytes / 8);
  if (pr.nq > 0) {
    if (!LSE) return fail(FA_ERR_INVALID_ARGUMENT, "LSE is NULL");
    if (!aligned16(LSE)) return fail(FA_ERR_INVALID_ARGUMENT, "LSE is not 16-byte aligned");
    lse = Extent{reinterpret_cast<uintptr_t>(LSE), reinterpret_cast<uintptr_t>(LSE) + (uintptr_t)(pr.bh * pr.nq * 4)};
    if (!use_scratch) {
      if (!workspace) return fail(FA_ERR_INVALID_ARGUMENT, "workspace is NULL");
      if (!aligned16(workspace)) return fail(FA_ERR_INVALID_ARGUMENT, "workspace is not 16-byte aligned");
      ws = Extent{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + need};
    }
  }
  if (!use_scratch && workspace_bytes_given < need)
    return fail(FA_ERR_INVALID_ARGUMENT, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes_given,
                need);
  fa::Strides sbias;
  Extent bext;
  if ((st = describe_bias(bias, bias_strides, pr, &sbias, &bext)) != FA_OK) return st;
  const Extent* out_ext[4] = {&dq.ext, &dk.ext, &dv.ext, &ws};
  const char* out_name[4] = {"dQ", "dK", "dV", "workspace"};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 5; ++j)
      if (overlap(*out_ext[i], ins[j]->ext)) return fail(FA_ERR_INVALID_ARGUMENT, "%s overlaps %s", out_name[i], ins[j]->name);
    if (overlap(*out_ext[i], lse)) return fail(FA_ERR_INVALID_ARGUMENT, "%s overlaps LSE", out_name[i]);
    if (overlap(*out_ext[i], bext)) return fail(FA_ERR_INVALID_ARGUMENT, "%s overlaps the bias", out_name[i]);
    for (int j = i + 1; j < 4; ++j)
      if (overlap(*out_ext[i], *out_ext[j]))
        return fail(FA_ERR_INVALID_ARGUMENT, "%s overlaps %s", out_name[i], out_name[j]);
  }

  if (use_scratch && need > 0) {
    // the library's own device memory (a distinct symbol, so it overlaps no
    // caller buffer); its address is looked up once per device
    int e;
    if ((e = hip_status(fa::scratch_address(&workspace), "scratch lookup")) != FA_OK) return e;
  }

  fa::BwdArgs a;
  a.q = Q, a.k = K, a.v = V, a.o = O, a.dout = dO, a.lse = LSE;
  a.dq = dQ, a.dk = dK, a.dv = dV;
  a.bias = (bias && pr.nk > 0 && pr.nq > 0) ? bias : nullptr;
  a.sbias = sbias;
  a.workspace = (float*)workspace;
  a.sq = q.st, a.sk = k.st, a.sv = v.st, a.so = o.st, a.sdo = g.st;
  a.sdq = dq.st, a.sdk = dk.st, a.sdv = dv.st;
  const int wmax = pr.nq + pr.nk;
  a.g = fa::Geometry{pr.B, pr.H, pr.nq, pr.nk, pr.d, std::min(wl, wmax), std::min(wr, wmax)};
  a.scale = scale;
  a.dtype = pr.dtype;
  a.stream = (hipStream_t)stream;
  return hip_status(fa::launch_bwd_mfma(a), "backward launch");
}

}  // namespace

FA_EXPORT int fa_version(void) { return 200; }

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
  int st = check_dims(B, H, N, N, d, dtype, &pr);
  if (st != FA_OK) return st;
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1 (got %d)", causal);
  return forward(Q, K, V, O, LSE, pr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, scale, -1, causal ? 0 : -1,
                 stream);
}

FA_EXPORT int fa_fwd_ex(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int Nq,
                        int Nk, int d, const long long* q_strides, const long long* k_strides,
                        const long long* v_strides, const long long* o_strides, const float* bias,
                        const long long* bias_strides, float scale, int window_left, int window_right, int dtype,
                        void* stream) {
  g_detail[0] = '\0';
  Problem pr;
  int st = check_dims(B, H, Nq, Nk, d, dtype, &pr);
  if (st != FA_OK) return st;
  return forward(Q, K, V, O, LSE, pr, q_strides, k_strides, v_strides, o_strides, bias, bias_strides, scale,
                 window_left, window_right, stream);
}

FA_EXPORT size_t fa_bwd_workspace_bytes(int B, int H, int N, int d, int dtype) {
  Problem pr;
  if (check_dims(B, H, N, N, d, dtype, &pr) != FA_OK) return 0;
  return workspace_bytes(pr);
}

FA_EXPORT size_t fa_bwd_ex_workspace_bytes(int B, int H, int Nq, int Nk, int d, int dtype) {
  Problem pr;
  if (check_dims(B, H, Nq, Nk, d, dtype, &pr) != FA_OK) return 0;
  return workspace_bytes(pr);
}

FA_EXPORT int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE,
                     void* dQ, void* dK, void* dV, int B, int H, int N, int d, float scale, int causal, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream) {
  g_detail[0] = '\0';
  Problem pr;
  int st = check_dims(B, H, N, N, d, dtype, &pr);
  if (st != FA_OK) return st;
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1 (got %d)", causal);
  const long long* const none[8] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  return backward(Q, K, V, O, dO, LSE, dQ, dK, dV, pr, none, nullptr, nullptr, scale, -1, causal ? 0 : -1, workspace,
                  workspace_bytes, stream);
}

FA_EXPORT int fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                             const float* LSE, void* dQ, void* dK, void* dV, int B, int H, int N, int d, float scale,
                             int causal, int dtype, void* stream) {
  g_detail[0] = '\0';
  Problem pr;
  int st = check_dims(B, H, N, N, d, dtype, &pr);
  if (st != FA_OK) return st;
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1 (got %d)", causal);
  const long long* const none[8] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  return backward(Q, K, V, O, dO, LSE, dQ, dK, dV, pr, none, nullptr, nullptr, scale, -1, causal ? 0 : -1, nullptr, 0,
                  stream, true);
}

FA_EXPORT int fa_bwd_ex(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE,
                        void* dQ, void* dK, void* dV, int B, int H, int Nq, int Nk, int d,
                        const long long* q_strides, const long long* k_strides, const long long* v_strides,
                        const long long* o_strides, const long long* do_strides, const long long* dq_strides,
                        const long long* dk_strides, const long long* dv_strides, const float* bias,
                        const long long* bias_strides, float scale, int window_left, int window_right, int dtype,
                        void* workspace, size_t workspace_bytes, void* stream) {
  g_detail[0] = '\0';
  Problem pr;
  int st = check_dims(B, H, Nq, Nk, d, dtype, &pr);
  if (st != FA_OK) return st;
  const long long* const strides[8] = {q_strides, k_strides, v_strides, o_strides,
                                       do_strides, dq_strides, dk_strides, dv_strides};
  return backward(Q, K, V, O, dO, LSE, dQ, dK, dV, pr, strides, bias, bias_strides, scale, window_left, window_right,
                  workspace, workspace_bytes, stream);
}
