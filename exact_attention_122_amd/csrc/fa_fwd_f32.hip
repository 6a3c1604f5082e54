// Forward attention in float32 end to end (no reduced-precision modes).
//
// Same method as the bf16 kernel ('FlashAttention', josueisai.com, section on
// the softmax trick): K/V tiles are staged in LDS, every query row keeps a
// running max m, a running sum l and an output accumulator, rescaled by
// exp(m_old - m_new) whenever m grows; after the last tile O = acc / l and
// LSE = m + ln l. The dot products run on plain fp32 FMAs: this kernel serves
// small fp32 problems, where latency, not throughput, sets the time. A query
// row is shared by threads_per_row<D>() adjacent lanes, each holding D / that
// many elements of q and of the output accumulator (a whole row of both per
// lane does not fit the registers at d = 96 and 128); their partial dot
// products are summed with lane shuffles, and every lane of a row then runs
// the same softmax arithmetic. Shapes, strides and band masks follow the same
// rules as the 16-bit kernels.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kThreadsF32 = 64;  // one wave per work-group
constexpr int kKeys = 32;        // keys per LDS tile

template <int D>
constexpr int threads_per_row() {
  return D <= 32 ? 1 : D <= 64 ? 2 : 4;
}

struct F32Params {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  long long q_sb, q_sh, q_sr, k_sb, k_sh, k_sr, v_sb, v_sh, v_sr, o_sb, o_sh, o_sr;  // strides (elements)
  int heads;
  int nq, nk;
  int diag;         // nk - nq: the key aligned with query 0
  int wl, wr;       // band (banded kernels only), both >= 0
  int nqb;
  float c;          // |scale| * log2(e)
  float scale_abs;
  float qsign;      // -1 when scale < 0 (exact sign flip of Q), else +1
};

template <int D, bool BAND>
__global__ __launch_bounds__(kThreadsF32) void fwd_f32_kernel(F32Params p) {
  constexpr int kTpr = threads_per_row<D>();
  constexpr int kDl = D / kTpr;              // elements of a row per lane
  constexpr int kRows = kThreadsF32 / kTpr;  // query rows per work-group
  __shared__ float k_lds[kKeys][D];
  __shared__ float v_lds[kKeys][D];
  const int tid = threadIdx.x;
  const int part = tid % kTpr;  // this lane's slice [part * kDl, +kDl) of a row
  const int nq = p.nq, nk = p.nk;
  const int head = blockIdx.x / p.nqb;
  const int qblk = blockIdx.x - head * p.nqb;
  const int hb = head / p.heads, hh = head - hb * p.heads;
  const float* qh = p.q + hb * p.q_sb + hh * p.q_sh;
  const float* kh = p.k + hb * p.k_sb + hh * p.k_sh;
  const float* vh = p.v + hb * p.v_sb + hh * p.v_sh;
  const int q_row0 = qblk * kRows;
  const int qi = q_row0 + tid / kTpr;
  const int e0 = part * kDl;

  float q[kDl], acc[kDl];
#pragma unroll
  for (int e = 0; e < kDl; ++e) {
    q[e] = qi < nq ? qh[qi * p.q_sr + e0 + e] * p.qsign : 0.f;
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  // live keys of this row: [lo, hi]
  const int lo = BAND ? qi + p.diag - p.wl : 0;
  const int hi = BAND ? min(qi + p.diag + p.wr, nk - 1) : nk - 1;

  // key tiles of this work-group's band
  const int q_last = min(nq, q_row0 + kRows) - 1;
  int key_base = 0, n_tiles = (nk + kKeys - 1) / kKeys;
  if (BAND) {
    const int k_lo = max(0, q_row0 + p.diag - p.wl);
    const int k_hi = min(nk - 1, q_last + p.diag + p.wr);
    key_base = k_lo / kKeys * kKeys;
    n_tiles = k_hi < k_lo ? 0 : (k_hi - key_base) / kKeys + 1;
  }
  for (int j = 0; j < n_tiles; ++j) {
    const int key0 = key_base + j * kKeys;
    __syncthreads();
    for (int e = tid; e < kKeys * D / 4; e += kThreadsF32) {
      const int row = e / (D / 4);
      const int c4 = e % (D / 4);
      float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
      if (key0 + row < nk) {
        kx = *(const float4*)(kh + (key0 + row) * p.k_sr + 4 * c4);
        vx = *(const float4*)(vh + (key0 + row) * p.v_sr + 4 * c4);
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
      for (int e = 0; e < kDl; ++e) dot = fmaf(q[e], k_lds[kk][e0 + e], dot);
      // the row's partial sums live in kTpr adjacent lanes
#pragma unroll
      for (int off = 1; off < kTpr; off <<= 1) dot += __shfl_xor(dot, off);
      const int key = key0 + kk;
      const bool dead = key > hi || key < lo;
      s[kk] = dead ? -INFINITY : dot;
      mx = fmaxf(mx, s[kk]);
    }
    const float mnew = fmaxf(m, mx);
    const float ms = mnew == -INFINITY ? 0.f : mnew * p.c;
    const float alpha = m == -INFINITY ? 0.f : exp2f(m * p.c - ms);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < kDl; ++e) acc[e] *= alpha;
#pragma unroll
    for (int kk = 0; kk < kKeys; ++kk) {
      const float pk = s[kk] == -INFINITY ? 0.f : exp2f(fmaf(s[kk], p.c, -ms));
      l += pk;
#pragma unroll
      for (int e = 0; e < kDl; ++e) acc[e] = fmaf(pk, v_lds[kk][e0 + e], acc[e]);
    }
    m = mnew;
  }

  if (qi < nq) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* orow = p.o + hb * p.o_sb + hh * p.o_sh + qi * p.o_sr + e0;
#pragma unroll
    for (int e = 0; e < kDl; e += 4)
      *(float4*)(orow + e) = make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
    if (part == 0) p.lse[(long long)head * nq + qi] = l > 0.f ? m * p.scale_abs + logf(l) : -INFINITY;
  }
}

template <int D, bool BAND>
hipError_t launch(const FwdArgs& a) {
  F32Params p;
  p.q = (const float*)a.q;
  p.k = (const float*)a.k;
  p.v = (const float*)a.v;
  p.o = (float*)a.o;
  p.lse = a.lse;
  p.q_sb = a.sq.b, p.q_sh = a.sq.h, p.q_sr = a.sq.r;
  p.k_sb = a.sk.b, p.k_sh = a.sk.h, p.k_sr = a.sk.r;
  p.v_sb = a.sv.b, p.v_sh = a.sv.h, p.v_sr = a.sv.r;
  p.o_sb = a.so.b, p.o_sh = a.so.h, p.o_sr = a.so.r;
  p.heads = a.g.heads;
  p.nq = a.g.nq;
  p.nk = a.g.nk;
  p.diag = a.g.nk - a.g.nq;
  p.wl = a.g.wl < 0 ? a.g.nq + a.g.nk : a.g.wl;
  p.wr = a.g.wr < 0 ? a.g.nq + a.g.nk : a.g.wr;
  constexpr int kRows = kThreadsF32 / threads_per_row<D>();
  p.nqb = (a.g.nq + kRows - 1) / kRows;
  p.scale_abs = fabsf(a.scale);
  p.c = p.scale_abs * kLog2e;
  p.qsign = a.scale < 0.f ? -1.f : 1.f;
  const long long blocks = (long long)p.nqb * a.g.batch * a.g.heads;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_f32_kernel<D, BAND>), dim3((unsigned)blocks), dim3(kThreadsF32), 0, a.stream, p);
  return hipGetLastError();
}


template <int D>
hipError_t launch_b(const FwdArgs& a) {
  return a.g.banded() ? launch<D, true>(a) : launch<D, false>(a);
}

}  // namespace

// d = 256 is not built here: a lane would hold 64 elements each of q and of
// the output accumulator (or a row would span 8 lanes); fp32 serves small
// problems, and 16-bit types cover d = 256.
hipError_t launch_fwd_f32(const FwdArgs& a) {
  switch (a.g.d) {
    case 32: return launch_b<32>(a);
    case 64: return launch_b<64>(a);
    case 96: return launch_b<96>(a);
    default: return launch_b<128>(a);
  }
}

}  // namespace fa
