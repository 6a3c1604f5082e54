// Forward attention in float32 end to end (no reduced-precision modes).
//
// Same method as the bf16 kernel ('FlashAttention', josueisai.com, section on
// the softmax trick): K/V tiles are staged in LDS, every query row keeps a
// running max m, a running sum l and an output accumulator, rescaled by
// exp(m_old - m_new) whenever m grows; after the last tile O = acc / l and
// LSE = m + ln l. Here one thread owns one query row and the dot products run
// on plain fp32 FMAs: this kernel serves small fp32 problems, where latency,
// not throughput, sets the time.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kRows = 64;   // query rows per work-group (one wave)
constexpr int kKeys = 32;   // keys per LDS tile

struct F32Params {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int n;
  int nqb;
  float c;          // |scale| * log2(e)
  float scale_abs;
  float qsign;      // -1 when scale < 0 (exact sign flip of Q), else +1
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kRows) void fwd_f32_kernel(F32Params p) {
  __shared__ float k_lds[kKeys][D];
  __shared__ float v_lds[kKeys][D];
  const int tid = threadIdx.x;
  const int n = p.n;
  const int head = blockIdx.x / p.nqb;
  const int qblk = blockIdx.x - head * p.nqb;
  const size_t head_off = (size_t)head * n * D;
  const int qi = qblk * kRows + tid;

  float q[D], acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = qi < n ? p.q[head_off + (size_t)qi * D + e] * p.qsign : 0.f;
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  const int q_last = min(n, qblk * kRows + kRows) - 1;
  const int n_tiles = CAUSAL ? q_last / kKeys + 1 : (n + kKeys - 1) / kKeys;
  for (int j = 0; j < n_tiles; ++j) {
    const int key0 = j * kKeys;
    __syncthreads();
    for (int e = tid; e < kKeys * D / 4; e += kRows) {
      const int row = e / (D / 4);
      const int c4 = e % (D / 4);
      float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
      if (key0 + row < n) {
        kx = *(const float4*)(p.k + head_off + (size_t)(key0 + row) * D + 4 * c4);
        vx = *(const float4*)(p.v + head_off + (size_t)(key0 + row) * D + 4 * c4);
      }
      *(float4*)&k_lds[row][4 * c4] = kx;
      *(float4*)&v_lds[row][4 * c4] = vx;
    }
    __syncthreads();

    float s[kKeys];
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < kKeys; ++kk) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) dot = fmaf(q[e], k_lds[kk][e], dot);
      const int key = key0 + kk;
      const bool dead = key >= n || (CAUSAL && key > qi);
      s[kk] = dead ? -INFINITY : dot;
      mx = fmaxf(mx, s[kk]);
    }
    const float mnew = fmaxf(m, mx);
    const float ms = mnew == -INFINITY ? 0.f : mnew * p.c;
    const float alpha = m == -INFINITY ? 0.f : exp2f(m * p.c - ms);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < D; ++e) acc[e] *= alpha;
#pragma unroll
    for (int kk = 0; kk < kKeys; ++kk) {
      const float pk = s[kk] == -INFINITY ? 0.f : exp2f(fmaf(s[kk], p.c, -ms));
      l += pk;
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] = fmaf(pk, v_lds[kk][e], acc[e]);
    }
    m = mnew;
  }

  if (qi < n) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* orow = p.o + head_off + (size_t)qi * D;
#pragma unroll
    for (int e = 0; e < D; e += 4)
      *(float4*)(orow + e) = make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
    p.lse[(size_t)head * n + qi] = l > 0.f ? m * p.scale_abs + logf(l) : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a) {
  F32Params p;
  p.q = (const float*)a.q;
  p.k = (const float*)a.k;
  p.v = (const float*)a.v;
  p.o = (float*)a.o;
  p.lse = a.lse;
  p.n = a.n;
  p.nqb = (a.n + kRows - 1) / kRows;
  p.scale_abs = fabsf(a.scale);
  p.c = p.scale_abs * kLog2e;
  p.qsign = a.scale < 0.f ? -1.f : 1.f;
  const long long blocks = (long long)p.nqb * a.bh;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(kRows), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a) {
  if (a.d == 64) return a.causal ? launch<64, true>(a) : launch<64, false>(a);
  return a.causal ? launch<128, true>(a) : launch<128, false>(a);
}

}  // namespace fa
