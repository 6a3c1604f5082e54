// Backward attention, bf16 in / bf16 out, fp32 accumulation, MFMA on gfx950.
//
// The backward keeps no score or probability matrix: both are recomputed from
// Q, K and the saved log-sum-exp ('FlashAttention', josueisai.com, section on
// recomputing instead of remembering), P = exp(scale * Q K^T - LSE). The
// gradient formulas are the chain rule of the forward definition:
//   dV = P^T dO;  dP = dO V^T;  D_i = sum_k dO_ik O_ik = sum_j P_ij dP_ij;
//   dS = P * (dP - D);  dQ = scale dS K;  dK = scale dS^T Q.
//
// Three launches on one stream, no atomics, deterministic:
//  1. row_stats_kernel: per query row, D_i from O and dO, and LSE_i * log2(e)
//     (so the kernels below form P with one FMA and exp2). Stored per head in
//     64-row tiles [64 x LSE*log2e | 64 x D] (512 bytes, zeros past N).
//  2. dkdv_kernel: a work-group owns 128 keys (32 per wave, K and V rows held
//     in registers) and streams 64-row query tiles (Q, dO and their row
//     statistics) through LDS. Scores are computed as S = Q K^T so each lane
//     holds one key; P and dS then feed dV += P^T dO and dK += dS^T Q directly
//     as A operands, with dO and Q read transposed out of LDS
//     (ds_read_b64_tr_b16).
//  3. dq_kernel: a work-group owns 128 query rows (32 per wave, Q and dO rows
//     in registers) and streams 64-key K/V tiles through LDS. Scores are
//     computed transposed, S^T = K Q^T, so each lane holds one query (its LSE
//     and D are per-lane scalars); dS^T feeds dQ^T += K^T dS^T as the B
//     operand, with K read transposed out of LDS.
// Tiles are copied global -> LDS directly (no staging registers). Rows past
// the sequence end arrive as zeros and have zero statistics: a zero Q / dO row
// (dkdv) or a zero K row (dq) then contributes exactly nothing, so ragged
// tails need no masking. Only the causal mask is applied, on diagonal tiles.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;            // rows per LDS tile
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerBlock = 128;   // keys (dkdv) or queries (dq) per work-group
constexpr int kStatTileBytes = 2 * kTile * 4;

struct BwdParams {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const bf16_t* dout;
  const float* stats;  // per head: n_pad / 64 tiles of [64 LSE*log2e | 64 D]
  bf16_t* dq;
  bf16_t* dk;
  bf16_t* dv;
  int n;
  int n_pad;     // n rounded up to a multiple of 64
  int nblk;      // row blocks per head
  int nblocks;   // work-groups in the grid
  float c;       // scale * log2(e)
  float scale;
};

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// One thread group of D/8 lanes per padded row.
template <int D>
__global__ __launch_bounds__(kThreads) void row_stats_kernel(const bf16_t* o, const bf16_t* dout, const float* lse,
                                                             float* stats, int n, int n_pad, long long padded_rows) {
  constexpr int kLanesPerRow = D / 8;
  const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long prow = gid / kLanesPerRow;
  const int part = (int)(gid % kLanesPerRow);
  const long long head = prow / n_pad;
  const int r = (int)(prow - head * n_pad);
  const bool valid = prow < padded_rows && r < n;
  const long long row = head * n + r;
  float acc = 0.f;
  if (valid) {
    const u32x4 a = *(const u32x4*)(o + row * D + part * 8);
    const u32x4 b = *(const u32x4*)(dout + row * D + part * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(bf16_lo(a[i]), bf16_lo(b[i]), acc);
      acc = fmaf(bf16_hi(a[i]), bf16_hi(b[i]), acc);
    }
  }
#pragma unroll
  for (int off = kLanesPerRow / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (prow < padded_rows && part == 0) {
    float* tile = stats + (head * n_pad + (r & ~(kTile - 1))) * 2;
    tile[r & (kTile - 1)] = valid ? lse[row] * kLog2e : 0.f;
    tile[kTile + (r & (kTile - 1))] = acc;
  }
}

// ---------------------------------------------------------------- dK, dV ---

template <int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_tile(const bf16_t* qt, const bf16_t* dt, const float* st,
                                          const RowRead<D>& rrd, const TrRead<D>& trd, const bf16x8 (&kf)[D / 16],
                                          const bf16x8 (&vf)[D / 16], f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32],
                                          float c, int q0, int key, int lane, bool masked) {
  const int hw = lane >> 5;
  f32x16 s[2], dp[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    s[qb] = f32x16{};
    dp[qb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      s[qb] = mfma32(rrd(qt, qb, ks), kf[ks], s[qb]);
      dp[qb] = mfma32(rrd(dt, qb, ks), vf[ks], dp[qb]);
    }
  }
  // lane holds key `key`; register r of block qb holds query
  // q0 + 32 qb + 8 (r / 4) + 4 hw + r % 4
  bf16x8 pa[4], da[4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int r0 = qb * 32 + 8 * g + 4 * hw;
      const f32x4 Lv = *(const FA_LDS f32x4*)((const FA_LDS float*)st + r0);
      const f32x4 Rv = *(const FA_LDS f32x4*)((const FA_LDS float*)st + kTile + r0);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int i = 4 * g + rr;
        float arg = fmaf(s[qb][i], c, -Lv[rr]);
        if (CAUSAL && masked) arg = key > q0 + r0 + rr ? -INFINITY : arg;
        const float pv = fast_exp2(arg);
        const int t = qb * 2 + (g >> 1), e = 4 * (g & 1) + rr;
        pa[t][e] = (__bf16)pv;
        da[t][e] = (__bf16)(pv * (dp[qb][i] - Rv[rr]));
      }
    }
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      dv[db] = mfma32(pa[t], trd(dt, t, db), dv[db]);
      dk[db] = mfma32(da[t], trd(qt, t, db), dk[db]);
    }
}

struct QTileBufs {
  bf16_t* q;
  bf16_t* d;
  float* st;
};

template <int D>
struct DkdvCopy {
  TileDma<kTile, D, kThreads> dma;
  __amdgpu_buffer_rsrc_t qrs, drs, srs;
  int wave, lane;
  // query tile starting at row q0 -> LDS
  __device__ __forceinline__ void issue(const QTileBufs& b, int q0) const {
    dma.issue(qrs, b.q, q0);
    dma.issue(drs, b.d, q0);
    if (wave == 0 && lane < kStatTileBytes / 16) {
      FA_LDS void* dst = (FA_LDS void*)(FA_LDS float*)b.st;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, dst, 16, (uint32_t)(q0 / kTile) * kStatTileBytes + 16 * lane,
                                               0, 0, 0);
    }
  }
};

template <int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_step(int t, int t_end, const QTileBufs& cur, const QTileBufs& nxt,
                                          const DkdvCopy<D>& cp, const RowRead<D>& rrd, const TrRead<D>& trd,
                                          const bf16x8 (&kf)[D / 16], const bf16x8 (&vf)[D / 16],
                                          f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32], const BwdParams& p, int wk0,
                                          int key, int lane) {
  const int q0 = t * kTile;
  if (t + 1 < t_end) cp.issue(nxt, q0 + kTile);
  if (wk0 < p.n && (!CAUSAL || q0 + kTile - 1 >= wk0)) {
    const bool masked = CAUSAL && q0 < wk0 + kRowsPerWave - 1;
    dkdv_tile<D, CAUSAL>(cur.q, cur.d, cur.st, rrd, trd, kf, vf, dk, dv, p.c, q0, key, lane, masked);
  }
  wait_vmem();
  __syncthreads();
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void dkdv_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) bf16_t q_lds0[kTile * D];
  __shared__ __attribute__((aligned(1024))) bf16_t q_lds1[kTile * D];
  __shared__ __attribute__((aligned(1024))) bf16_t d_lds0[kTile * D];
  __shared__ __attribute__((aligned(1024))) bf16_t d_lds1[kTile * D];
  __shared__ __attribute__((aligned(16))) float s_lds0[2 * kTile];
  __shared__ __attribute__((aligned(16))) float s_lds1[2 * kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hw = lane >> 5;
  const int col = lane & 31;
  const int n = p.n;

  const int logical = xcd_logical_block(blockIdx.x, p.nblocks);
  const int head = logical / p.nblk;
  const int kblk = logical - head * p.nblk;
  const size_t head_off = (size_t)head * n * D;
  const int key_wg = kblk * kRowsPerBlock;
  const int wk0 = key_wg + wave * kRowsPerWave;
  const int key = wk0 + col;
  const int t_begin = CAUSAL ? key_wg / kTile : 0;
  const int t_end = (n + kTile - 1) / kTile;

  DkdvCopy<D> cp;
  cp.dma.init(wave, lane);
  cp.qrs = make_rsrc(p.q + head_off, (uint32_t)n * D * 2);
  cp.drs = make_rsrc(p.dout + head_off, (uint32_t)n * D * 2);
  cp.srs = make_rsrc(p.stats + (size_t)head * p.n_pad * 2, (uint32_t)p.n_pad * 8);
  cp.wave = wave;
  cp.lane = lane;
  const QTileBufs b0{q_lds0, d_lds0, s_lds0}, b1{q_lds1, d_lds1, s_lds1};
  cp.issue(b0, t_begin * kTile);

  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 kx = u32x4{0u, 0u, 0u, 0u}, vx = kx;
    if (key < n) {
      kx = *(const u32x4*)(p.k + head_off + (size_t)key * D + 16 * ks + 8 * hw);
      vx = *(const u32x4*)(p.v + head_off + (size_t)key * D + 16 * ks + 8 * hw);
    }
    kf[ks] = __builtin_bit_cast(bf16x8, kx);
    vf[ks] = __builtin_bit_cast(bf16x8, vx);
  }
  RowRead<D> rrd;
  rrd.init(lane);
  TrRead<D> trd;
  trd.init(lane);
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  wait_vmem();
  __syncthreads();
  for (int t = t_begin; t < t_end; t += 2) {
    dkdv_step<D, CAUSAL>(t, t_end, b0, b1, cp, rrd, trd, kf, vf, dk, dv, p, wk0, key, lane);
    if (t + 1 < t_end) dkdv_step<D, CAUSAL>(t + 1, t_end, b1, b0, cp, rrd, trd, kf, vf, dk, dv, p, wk0, key, lane);
  }

  // lane holds d = 32 db + col for keys wk0 + 8 g + 4 hw + rr
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int kr = wk0 + 8 * g + 4 * hw + rr;
        if (kr < n) {
          const size_t off = head_off + (size_t)kr * D + 32 * db + col;
          p.dk[off] = __builtin_bit_cast(bf16_t, (__bf16)(dk[db][4 * g + rr] * p.scale));
          p.dv[off] = __builtin_bit_cast(bf16_t, (__bf16)dv[db][4 * g + rr]);
        }
      }
}

// -------------------------------------------------------------------- dQ ---

template <int D, bool CAUSAL>
__device__ __forceinline__ void dq_tile(const bf16_t* kt, const bf16_t* vt, const RowRead<D>& rrd,
                                        const TrRead<D>& trd, const bf16x8 (&qf)[D / 16],
                                        const bf16x8 (&df)[D / 16], f32x16 (&dq)[D / 32], float lse2, float drow,
                                        float c, int key0, int qi, int lane, bool masked) {
  const int hw = lane >> 5;
  f32x16 s[2], dpt[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    s[kb] = f32x16{};
    dpt[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      s[kb] = mfma32(rrd(kt, kb, ks), qf[ks], s[kb]);
      dpt[kb] = mfma32(rrd(vt, kb, ks), df[ks], dpt[kb]);
    }
  }
  bf16x8 ds[4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float arg = fmaf(s[kb][i], c, -lse2);
      if (CAUSAL && masked) {
        const int key = key0 + kb * 32 + 8 * (i >> 2) + 4 * hw + (i & 3);
        arg = key > qi ? -INFINITY : arg;
      }
      const float pv = fast_exp2(arg);
      ds[kb * 2 + (i >> 3)][i & 7] = (__bf16)(pv * (dpt[kb][i] - drow));
    }
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int t = 0; t < 4; ++t) dq[db] = mfma32(trd(kt, t, db), ds[t], dq[db]);
}

template <int D, bool CAUSAL>
__device__ __forceinline__ void dq_step(int j, int n_tiles, const bf16_t* kt, const bf16_t* vt, bf16_t* kn,
                                        bf16_t* vn, const TileDma<kTile, D, kThreads>& dma,
                                        __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                        const RowRead<D>& rrd, const TrRead<D>& trd, const bf16x8 (&qf)[D / 16],
                                        const bf16x8 (&df)[D / 16], f32x16 (&dq)[D / 32], float lse2, float drow,
                                        const BwdParams& p, int qi, int wq0, int w_last, int lane) {
  const int key0 = j * kTile;
  if (j + 1 < n_tiles) {
    dma.issue(krs, kn, key0 + kTile);
    dma.issue(vrs, vn, key0 + kTile);
  }
  if (wq0 < p.n && (!CAUSAL || key0 <= w_last)) {
    const bool masked = CAUSAL && key0 + kTile - 1 > wq0;
    dq_tile<D, CAUSAL>(kt, vt, rrd, trd, qf, df, dq, lse2, drow, p.c, key0, qi, lane, masked);
  }
  wait_vmem();
  __syncthreads();
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void dq_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) bf16_t k_lds0[kTile * D];
  __shared__ __attribute__((aligned(1024))) bf16_t k_lds1[kTile * D];
  __shared__ __attribute__((aligned(1024))) bf16_t v_lds0[kTile * D];
  __shared__ __attribute__((aligned(1024))) bf16_t v_lds1[kTile * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hw = lane >> 5;
  const int col = lane & 31;
  const int n = p.n;

  const int logical = xcd_logical_block(blockIdx.x, p.nblocks);
  const int head = logical / p.nblk;
  int qblk = logical - head * p.nblk;
  if (CAUSAL) qblk = p.nblk - 1 - qblk;
  const size_t head_off = (size_t)head * n * D;
  const int q_row0 = qblk * kRowsPerBlock;
  const int wq0 = q_row0 + wave * kRowsPerWave;
  const int qi = wq0 + col;

  const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k + head_off, (uint32_t)n * D * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v + head_off, (uint32_t)n * D * 2);
  TileDma<kTile, D, kThreads> dma;
  dma.init(wave, lane);
  dma.issue(krs, k_lds0, 0);
  dma.issue(vrs, v_lds0, 0);

  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 qx = u32x4{0u, 0u, 0u, 0u}, dx = qx;
    if (qi < n) {
      qx = *(const u32x4*)(p.q + head_off + (size_t)qi * D + 16 * ks + 8 * hw);
      dx = *(const u32x4*)(p.dout + head_off + (size_t)qi * D + 16 * ks + 8 * hw);
    }
    qf[ks] = __builtin_bit_cast(bf16x8, qx);
    df[ks] = __builtin_bit_cast(bf16x8, dx);
  }
  float lse2 = 0.f, drow = 0.f;
  if (qi < n) {
    const float* st = p.stats + ((size_t)head * p.n_pad + (qi & ~(kTile - 1))) * 2;
    lse2 = st[qi & (kTile - 1)];
    drow = st[kTile + (qi & (kTile - 1))];
  }
  RowRead<D> rrd;
  rrd.init(lane);
  TrRead<D> trd;
  trd.init(lane);
  f32x16 dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq[db] = f32x16{};

  const int q_last = min(n, q_row0 + kRowsPerBlock) - 1;
  const int n_tiles = CAUSAL ? q_last / kTile + 1 : (n + kTile - 1) / kTile;
  const int w_last = min(n - 1, wq0 + kRowsPerWave - 1);

  wait_vmem();
  __syncthreads();
  for (int j = 0; j < n_tiles; j += 2) {
    dq_step<D, CAUSAL>(j, n_tiles, k_lds0, v_lds0, k_lds1, v_lds1, dma, krs, vrs, rrd, trd, qf, df, dq, lse2, drow, p,
                       qi, wq0, w_last, lane);
    if (j + 1 < n_tiles)
      dq_step<D, CAUSAL>(j + 1, n_tiles, k_lds1, v_lds1, k_lds0, v_lds0, dma, krs, vrs, rrd, trd, qf, df, dq, lse2,
                         drow, p, qi, wq0, w_last, lane);
  }

  if (qi < n) {
    bf16_t* row = p.dq + head_off + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 w;
        w.x = pack_bf16x2(dq[db][4 * g] * p.scale, dq[db][4 * g + 1] * p.scale);
        w.y = pack_bf16x2(dq[db][4 * g + 2] * p.scale, dq[db][4 * g + 3] * p.scale);
        *(uint2*)(row + db * 32 + 8 * g + 4 * hw) = w;
      }
  }
}

template __global__ void dkdv_kernel<64, false>(BwdParams);
template __global__ void dkdv_kernel<64, true>(BwdParams);
template __global__ void dkdv_kernel<128, false>(BwdParams);
template __global__ void dkdv_kernel<128, true>(BwdParams);
template __global__ void dq_kernel<64, false>(BwdParams);
template __global__ void dq_kernel<64, true>(BwdParams);
template __global__ void dq_kernel<128, false>(BwdParams);
template __global__ void dq_kernel<128, true>(BwdParams);
template __global__ void row_stats_kernel<64>(const bf16_t*, const bf16_t*, const float*, float*, int, int, long long);
template __global__ void row_stats_kernel<128>(const bf16_t*, const bf16_t*, const float*, float*, int, int, long long);

template <int D, bool CAUSAL>
hipError_t launch(const BwdArgs& a) {
  BwdParams p;
  p.q = (const bf16_t*)a.q;
  p.k = (const bf16_t*)a.k;
  p.v = (const bf16_t*)a.v;
  p.dout = (const bf16_t*)a.dout;
  p.stats = a.workspace;
  p.dq = (bf16_t*)a.dq;
  p.dk = (bf16_t*)a.dk;
  p.dv = (bf16_t*)a.dv;
  p.n = a.n;
  p.n_pad = (a.n + kTile - 1) / kTile * kTile;
  p.nblk = (a.n + kRowsPerBlock - 1) / kRowsPerBlock;
  p.nblocks = p.nblk * a.bh;
  p.scale = a.scale;
  p.c = a.scale * kLog2e;

  const long long padded_rows = (long long)a.bh * p.n_pad;
  const long long stat_blocks = (padded_rows * (D / 8) + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((row_stats_kernel<D>), dim3((unsigned)stat_blocks), dim3(kThreads), 0, a.stream,
                     (const bf16_t*)a.o, p.dout, a.lse, a.workspace, a.n, p.n_pad, padded_rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dkdv_kernel<D, CAUSAL>), dim3(p.nblocks), dim3(kThreads), 0, a.stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dq_kernel<D, CAUSAL>), dim3(p.nblocks), dim3(kThreads), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(long long bh, int n) {
  return (size_t)bh * (size_t)((n + kTile - 1) / kTile * kTile) * 8;
}

hipError_t launch_bwd_bf16(const BwdArgs& a) {
  if (a.d == 64) return a.causal ? launch<64, true>(a) : launch<64, false>(a);
  return a.causal ? launch<128, true>(a) : launch<128, false>(a);
}

}  // namespace fa
