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
//  1. row_dot_kernel: D_i from O and dO (HBM-bound, one float per row).
//  2. dkdv_kernel: a work-group owns 128 keys (32 per wave, K and V rows held
//     in registers) and loops over 64-row query tiles staged in LDS. Scores
//     are computed as S = Q K^T so each lane holds one key; P and dS then feed
//     dV += P^T dO and dK += dS^T Q directly as A operands, with dO and Q read
//     transposed out of LDS (ds_read_b64_tr_b16).
//  3. dq_kernel: a work-group owns 128 query rows (32 per wave, Q and dO rows
//     in registers) and loops over 64-key tiles staged in LDS. Scores are
//     computed transposed, S^T = K Q^T, so each lane holds one query (its LSE
//     and D are per-lane scalars); dS^T feeds dQ^T += K^T dS^T as the B
//     operand, with K read transposed out of LDS.
// Rows beyond the sequence length are zero-filled in LDS and get LSE = +inf,
// which makes their probabilities exactly zero; only valid rows are stored.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;            // rows per LDS tile
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerBlock = 128;   // keys (dkdv) or queries (dq) per work-group

struct BwdParams {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const bf16_t* dout;
  const float* lse;
  const float* row_dot;
  bf16_t* dq;
  bf16_t* dk;
  bf16_t* dv;
  int n;
  int nblk;      // row blocks per head
  int nblocks;   // work-groups in the grid
  float c;       // scale * log2(e)
  float scale;
};

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

template <int D>
__global__ __launch_bounds__(kThreads) void row_dot_kernel(const bf16_t* o, const bf16_t* dout, float* out,
                                                           long long rows) {
  constexpr int kLanesPerRow = D / 8;
  const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long row = gid / kLanesPerRow;
  const int part = (int)(gid % kLanesPerRow);
  float acc = 0.f;
  if (row < rows) {
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
  if (row < rows && part == 0) out[row] = acc;
}

// Rows [row0, row0 + 64) of a head's LSE (as LSE * log2 e) and D into LDS.
__device__ __forceinline__ void stage_row_stats(const BwdParams& p, size_t head_rows, int row0, int tid,
                                                float* lse_t, float* dot_t) {
  if (tid < kTile) {
    const int r = row0 + tid;
    const bool ok = r < p.n;
    lse_t[tid] = ok ? p.lse[head_rows + r] * kLog2e : INFINITY;
    dot_t[tid] = ok ? p.row_dot[head_rows + r] : 0.f;
  }
}

template <int D, bool CAUSAL, bool MASKED>
__device__ __forceinline__ void dkdv_tile(const bf16_t* qt, const bf16_t* dot_t_rows, const float* lse_t,
                                          const float* dot_t, const bf16x8 (&kf)[D / 16],
                                          const bf16x8 (&vf)[D / 16], f32x16 (&dk)[D / 32],
                                          f32x16 (&dv)[D / 32], const BwdParams& p, int q0, int key,
                                          int lane) {
  const int hw = lane >> 5;
  const int col = lane & 31;
  f32x16 s[2], dp[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    s[qb] = f32x16{};
    dp[qb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      s[qb] = mfma32(lds_row8<D>(qt, qb * 32 + col, 2 * ks + hw), kf[ks], s[qb]);
      dp[qb] = mfma32(lds_row8<D>(dot_t_rows, qb * 32 + col, 2 * ks + hw), vf[ks], dp[qb]);
    }
  }
  // P and dS; lane holds key `key`, register r of block qb holds query
  // q0 + 32 qb + 8 (r / 4) + 4 hw + r % 4.
  float pv[32], dsv[32];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int r0 = qb * 32 + 8 * g + 4 * hw;
      const float4 L = *(const float4*)(lse_t + r0);
      const float4 Dd = *(const float4*)(dot_t + r0);
      const float Lv[4] = {L.x, L.y, L.z, L.w};
      const float Dv[4] = {Dd.x, Dd.y, Dd.z, Dd.w};
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int i = 4 * g + rr;
        float e = fast_exp2(fmaf(s[qb][i], p.c, -Lv[rr]));
        if constexpr (MASKED) {
          if (CAUSAL && key > q0 + r0 + rr) e = 0.f;
        }
        pv[qb * 16 + i] = e;
        dsv[qb * 16 + i] = e * (dp[qb][i] - Dv[rr]);
      }
    }
  bf16x8 pa[4], da[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    pa[t] = pack_bf16x8(&pv[(t >> 1) * 16 + 8 * (t & 1)]);
    da[t] = pack_bf16x8(&dsv[(t >> 1) * 16 + 8 * (t & 1)]);
  }
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      dv[db] = mfma32(pa[t], lds_tr8<D>(dot_t_rows, 16 * t, 32 * db, lane), dv[db]);
      dk[db] = mfma32(da[t], lds_tr8<D>(qt, 16 * t, 32 * db, lane), dk[db]);
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void dkdv_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) bf16_t q_lds[2][kTile * D];
  __shared__ __attribute__((aligned(16))) bf16_t do_lds[2][kTile * D];
  __shared__ __attribute__((aligned(16))) float lse_lds[2][kTile];
  __shared__ __attribute__((aligned(16))) float dot_lds[2][kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hw = lane >> 5;
  const int col = lane & 31;
  const int n = p.n;

  const int logical = xcd_logical_block(blockIdx.x, p.nblocks);
  const int head = logical / p.nblk;
  const int kblk = logical - head * p.nblk;
  const size_t head_rows = (size_t)head * n;
  const size_t head_off = head_rows * D;
  const int key_wg = kblk * kRowsPerBlock;
  const int wk0 = key_wg + wave * kRowsPerWave;
  const int key = wk0 + col;

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
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  const int t_begin = CAUSAL ? key_wg / kTile : 0;
  const int t_end = (n + kTile - 1) / kTile;
  const bf16_t* qbase = p.q + head_off;
  const bf16_t* dbase = p.dout + head_off;
  TileCopy<kTile, D, kThreads> qc, dc;
  qc.load(qbase + (size_t)t_begin * kTile * D, n - t_begin * kTile, tid);
  dc.load(dbase + (size_t)t_begin * kTile * D, n - t_begin * kTile, tid);
  qc.store(q_lds[0], tid);
  dc.store(do_lds[0], tid);
  stage_row_stats(p, head_rows, t_begin * kTile, tid, lse_lds[0], dot_lds[0]);
  __syncthreads();

  for (int t = t_begin; t < t_end; ++t) {
    const int buf = (t - t_begin) & 1;
    const int q0 = t * kTile;
    const bool more = t + 1 < t_end;
    if (more) {
      qc.load(qbase + (size_t)(q0 + kTile) * D, n - q0 - kTile, tid);
      dc.load(dbase + (size_t)(q0 + kTile) * D, n - q0 - kTile, tid);
    }
    const bool active = wk0 < n && (!CAUSAL || q0 + kTile - 1 >= wk0);
    if (active) {
      const bool masked = CAUSAL && q0 < wk0 + kRowsPerWave - 1;
      if (masked)
        dkdv_tile<D, CAUSAL, true>(q_lds[buf], do_lds[buf], lse_lds[buf], dot_lds[buf], kf, vf, dk, dv, p, q0,
                                   key, lane);
      else
        dkdv_tile<D, CAUSAL, false>(q_lds[buf], do_lds[buf], lse_lds[buf], dot_lds[buf], kf, vf, dk, dv, p, q0,
                                    key, lane);
    }
    if (more) {
      qc.store(q_lds[buf ^ 1], tid);
      dc.store(do_lds[buf ^ 1], tid);
      stage_row_stats(p, head_rows, q0 + kTile, tid, lse_lds[buf ^ 1], dot_lds[buf ^ 1]);
    }
    __syncthreads();
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

template <int D, bool CAUSAL, bool MASKED>
__device__ __forceinline__ void dq_tile(const bf16_t* kt, const bf16_t* vt, const bf16x8 (&qf)[D / 16],
                                        const bf16x8 (&df)[D / 16], f32x16 (&dq)[D / 32], float lse2,
                                        float drow, const BwdParams& p, int key0, int qi, int lane) {
  const int hw = lane >> 5;
  const int col = lane & 31;
  f32x16 s[2], dpt[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    s[kb] = f32x16{};
    dpt[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      s[kb] = mfma32(lds_row8<D>(kt, kb * 32 + col, 2 * ks + hw), qf[ks], s[kb]);
      dpt[kb] = mfma32(lds_row8<D>(vt, kb * 32 + col, 2 * ks + hw), df[ks], dpt[kb]);
    }
  }
  float dsv[32];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float e = fast_exp2(fmaf(s[kb][i], p.c, -lse2));
      if constexpr (MASKED) {
        const int key = key0 + kb * 32 + 8 * (i >> 2) + 4 * hw + (i & 3);
        if (CAUSAL && key > qi) e = 0.f;
      }
      dsv[kb * 16 + i] = e * (dpt[kb][i] - drow);
    }
  bf16x8 db8[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) db8[t] = pack_bf16x8(&dsv[(t >> 1) * 16 + 8 * (t & 1)]);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int t = 0; t < 4; ++t) dq[db] = mfma32(lds_tr8<D>(kt, 16 * t, 32 * db, lane), db8[t], dq[db]);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void dq_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) bf16_t k_lds[2][kTile * D];
  __shared__ __attribute__((aligned(16))) bf16_t v_lds[2][kTile * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hw = lane >> 5;
  const int col = lane & 31;
  const int n = p.n;

  const int logical = xcd_logical_block(blockIdx.x, p.nblocks);
  const int head = logical / p.nblk;
  int qblk = logical - head * p.nblk;
  if (CAUSAL) qblk = p.nblk - 1 - qblk;
  const size_t head_rows = (size_t)head * n;
  const size_t head_off = head_rows * D;
  const int q_row0 = qblk * kRowsPerBlock;
  const int wq0 = q_row0 + wave * kRowsPerWave;
  const int qi = wq0 + col;

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
  const float lse2 = qi < n ? p.lse[head_rows + qi] * kLog2e : INFINITY;
  const float drow = qi < n ? p.row_dot[head_rows + qi] : 0.f;

  f32x16 dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq[db] = f32x16{};

  const int q_last = min(n, q_row0 + kRowsPerBlock) - 1;
  const int n_tiles = CAUSAL ? q_last / kTile + 1 : (n + kTile - 1) / kTile;
  const int w_last = min(n - 1, wq0 + kRowsPerWave - 1);
  const bf16_t* kbase = p.k + head_off;
  const bf16_t* vbase = p.v + head_off;
  TileCopy<kTile, D, kThreads> kc, vc;
  kc.load(kbase, n, tid);
  vc.load(vbase, n, tid);
  kc.store(k_lds[0], tid);
  vc.store(v_lds[0], tid);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    const int key0 = j * kTile;
    const bool more = j + 1 < n_tiles;
    if (more) {
      kc.load(kbase + (size_t)(key0 + kTile) * D, n - key0 - kTile, tid);
      vc.load(vbase + (size_t)(key0 + kTile) * D, n - key0 - kTile, tid);
    }
    const bool active = wq0 < n && (!CAUSAL || key0 <= w_last);
    if (active) {
      const bool masked = CAUSAL && key0 + kTile - 1 > wq0;
      if (masked)
        dq_tile<D, CAUSAL, true>(k_lds[buf], v_lds[buf], qf, df, dq, lse2, drow, p, key0, qi, lane);
      else
        dq_tile<D, CAUSAL, false>(k_lds[buf], v_lds[buf], qf, df, dq, lse2, drow, p, key0, qi, lane);
    }
    if (more) {
      kc.store(k_lds[buf ^ 1], tid);
      vc.store(v_lds[buf ^ 1], tid);
    }
    __syncthreads();
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

template <int D, bool CAUSAL>
hipError_t launch(const BwdArgs& a) {
  BwdParams p;
  p.q = (const bf16_t*)a.q;
  p.k = (const bf16_t*)a.k;
  p.v = (const bf16_t*)a.v;
  p.dout = (const bf16_t*)a.dout;
  p.lse = a.lse;
  p.row_dot = a.row_dot;
  p.dq = (bf16_t*)a.dq;
  p.dk = (bf16_t*)a.dk;
  p.dv = (bf16_t*)a.dv;
  p.n = a.n;
  p.nblk = (a.n + kRowsPerBlock - 1) / kRowsPerBlock;
  p.nblocks = p.nblk * a.bh;
  p.scale = a.scale;
  p.c = a.scale * kLog2e;

  const long long rows = (long long)a.bh * a.n;
  const long long dot_blocks = (rows * (D / 8) + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((row_dot_kernel<D>), dim3((unsigned)dot_blocks), dim3(kThreads), 0, a.stream,
                     (const bf16_t*)a.o, p.dout, a.row_dot, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dkdv_kernel<D, CAUSAL>), dim3(p.nblocks), dim3(kThreads), 0, a.stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dq_kernel<D, CAUSAL>), dim3(p.nblocks), dim3(kThreads), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a) {
  if (a.d == 64) return a.causal ? launch<64, true>(a) : launch<64, false>(a);
  return a.causal ? launch<128, true>(a) : launch<128, false>(a);
}

}  // namespace fa
