// Backward attention, bf16 or fp16 in and out, fp32 accumulation, MFMA on gfx950.
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
// Tiles are copied global -> LDS directly (no staging registers). Query rows
// past the end arrive as zeros with zero statistics, so a zero Q / dO row
// contributes exactly nothing to dK and dV; keys past the end are masked on
// the last tile of dq_kernel. Shapes, strides and band masks follow the
// forward pass: query i is aligned with key i + nk - nq, a band keeps keys
// [i + nk - nq - wl, i + nk - nq + wr], each work-group visits only the tiles
// its band touches, and tiles across a band edge set P = 0 on dead pairs. A
// query row that saw no key (LSE = -inf) gets P = 0 on every key. An
// optional fp32 bias enters P's exponent as + log2(e) bias; the bias itself is
// not differentiated.
#include "fa_device.h"
#include "fa_kernels.h"

#include <mutex>

namespace fa {

// Device scratch of the entry point that allocates nothing: the per-row
// statistics live here instead of in a caller's workspace. Each GPU holds its
// own copy from the library's load until the process ends. In host code the
// name is only a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is handed to
// kernels.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_address(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!addr) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = addr;
  }
  *out = g_scratch_addr[dev];
  return hipSuccess;
}

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
  const float* stats;  // per head: nq_pad / 64 tiles of [64 LSE*log2e | 64 D]
  bf16_t* dq;
  bf16_t* dk;
  bf16_t* dv;
  const float* bias;
  long long q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, do_sb, do_sh;  // batch / head strides (elements)
  long long dq_sb, dq_sh, dk_sb, dk_sh, dv_sb, dv_sh, bias_sb, bias_sh;
  int q_sr, k_sr, v_sr, do_sr, dq_sr, dk_sr, dv_sr, bias_sr;  // row strides (elements)
  int heads;
  int nq, nk;
  int nq_pad;    // nq rounded up to a multiple of 64
  int diag;      // nk - nq: the key aligned with query 0
  int wl, wr;    // band (banded kernels only), both >= 0
  int nkb, nqb;  // key blocks (dkdv) and query blocks (dq) per head
  float c;       // scale * log2(e)
  float scale;
};

// Per-head base of a strided tensor.
__device__ __forceinline__ const bf16_t* head_base(const bf16_t* t, long long sb, long long sh, int heads, int head) {
  const int b = head / heads;
  return t + b * sb + (head - b * heads) * sh;
}

// Lanes per query row in row_stats_kernel: D / 8 chunks of 8 elements,
// rounded up to a power of two for the shuffle reduction.
template <int D>
constexpr int row_lanes() {
  return D / 8 <= 4 ? 4 : D / 8 <= 8 ? 8 : D / 8 <= 16 ? 16 : 32;
}

// One group of row_lanes<D>() lanes per padded query row: D_i = dO_i . O_i
// and LSE_i * log2(e). A row that saw no key (LSE = -inf) stores +inf, so the
// kernels' exp2(c s - L) is 0 for it on every key.
template <typename E, int D>
__global__ __launch_bounds__(kThreads) void row_stats_kernel(const bf16_t* o, const bf16_t* dout, const float* lse,
                                                             float* stats, Strides so, Strides sdo, int heads, int nq,
                                                             int nq_pad, long long padded_rows) {
  constexpr int kLanesPerRow = row_lanes<D>();
  const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long prow = gid / kLanesPerRow;
  const int part = (int)(gid % kLanesPerRow);
  const int head = (int)(prow / nq_pad);
  const int r = (int)(prow - (long long)head * nq_pad);
  const bool valid = prow < padded_rows && r < nq;
  float acc = 0.f;
  if (valid && part < D / 8) {
    const int b = head / heads, h = head - b * heads;
    const u32x4 x = *(const u32x4*)(o + b * so.b + h * so.h + r * so.r + part * 8);
    const u32x4 y = *(const u32x4*)(dout + b * sdo.b + h * sdo.h + r * sdo.r + part * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(E::lo(x[i]), E::lo(y[i]), acc);
      acc = fmaf(E::hi(x[i]), E::hi(y[i]), acc);
    }
  }
#pragma unroll
  for (int off = kLanesPerRow / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (prow < padded_rows && part == 0) {
    float* tile = stats + ((long long)head * nq_pad + (r & ~(kTile - 1))) * 2;
    float l2 = 0.f;
    if (valid) {
      const float x = lse[(long long)head * nq + r];
      l2 = x == -INFINITY ? INFINITY : x * kLog2e;
    }
    tile[r & (kTile - 1)] = l2;
    tile[kTile + (r & (kTile - 1))] = acc;
  }
}

// Scheduling groups (see __builtin_amdgcn_sched_group_barrier) for a block of
// N MFMAs that each take R LDS reads: the operands of A MFMAs are read ahead
// of the MFMA that issues, so the matrix core does not wait on LDS latency.
template <int N, int R, int A>
__device__ __forceinline__ void sched_reads_ahead() {
  __builtin_amdgcn_sched_group_barrier(0x100, R * A, 0);
#pragma unroll
  for (int i = 0; i < N - A; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
  }
#pragma unroll
  for (int i = 0; i < A; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
}

// ---------------------------------------------------------------- dK, dV ---

// One 64-query tile against the wave's 32 keys. With a band, `masked` tiles
// (across a band edge) set P = 0 where query row qr is outside this lane's
// [q_lo, q_hi]. Without one the tile holds no masking code at all: query rows
// past the end are zero rows with zero statistics and add nothing.
template <typename E, int D, int MASK, bool BIAS>
__device__ __forceinline__ void dkdv_tile(const bf16_t* qt, const bf16_t* dt, const float* st,
                                          const RowRead<D>& rrd, const TrRead<D>& trd, const bf16x8 (&kf)[D / 16],
                                          const bf16x8 (&vf)[D / 16], f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32],
                                          float c, int q0, int q_lo, int q_hi, int lane, bool masked,
                                          const float* bcol, bool bkey, long long bias_sr, int nq) {
  const int hw = lane >> 5;
  // The tile's bias down this lane's key column, read before the S/dP
  // products so that its latency hides behind them (read next to its use, it
  // stalled every tile on memory latency). d = 256 has no registers for it.
  float bpre[32];
  if constexpr (BIAS && D <= 128) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int qr = q0 + (i >> 4) * 32 + 8 * ((i >> 2) & 3) + 4 * hw + (i & 3);
      // every lane loads (row and column clamped into the bias): no branch
      // per load; rows or keys past the end are zeroed where the value is used
      bpre[i] = bcol[(long long)min(qr, nq - 1) * bias_sr];
    }
  }
  f32x16 s[2], dp[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    s[qb] = f32x16{};
    dp[qb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      s[qb] = E::mfma(rrd(qt, qb, ks), kf[ks], s[qb]);
      dp[qb] = E::mfma(rrd(dt, qb, ks), vf[ks], dp[qb]);
    }
  }
  // lane holds one key; register r of block qb holds query
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
        if constexpr (BIAS) {
          // bias[q][key] down this lane's key column (bkey: the key exists)
          if constexpr (D <= 128) {
            const int qr = q0 + r0 + rr;
            arg = fmaf(kLog2e, (bkey && qr < nq) ? bpre[qb * 16 + i] : 0.f, arg);
          } else {
            const int qr = q0 + r0 + rr;
            const float bv = bcol[(long long)min(qr, nq - 1) * bias_sr];
            if (bkey && qr < nq) arg = fmaf(kLog2e, bv, arg);
          }
        }
        if (MASK != kMaskNone && masked) {
          const int qr = q0 + r0 + rr;
          arg = (qr < q_lo || (MASK == kMaskBand && qr > q_hi)) ? -INFINITY : arg;
        }
        const float pv = fast_exp2(arg);
        const int t = qb * 2 + (g >> 1), e = 4 * (g & 1) + rr;
        pa[t][e] = E::cvt(pv);
        da[t][e] = E::cvt(pv * (dp[qb][i] - Rv[rr]));
      }
    }
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      dv[db] = E::mfma(pa[t], trd(dt, t, db), dv[db]);
      dk[db] = E::mfma(da[t], trd(qt, t, db), dk[db]);
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
  uint32_t q_stride, d_stride;  // bytes between rows of Q and dO
  int wave, lane;
  // query tile starting at row q0 -> LDS
  __device__ __forceinline__ void issue(const QTileBufs& b, int q0) const {
    dma.issue(qrs, b.q, q0, q_stride);
    dma.issue(drs, b.d, q0, d_stride);
    if (wave == 0 && lane < kStatTileBytes / 16) {
      FA_LDS void* dst = (FA_LDS void*)(FA_LDS float*)b.st;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, dst, 16, (uint32_t)(q0 / kTile) * kStatTileBytes + 16 * lane,
                                               0, 0, 0);
    }
  }
};

// One query tile for this wave's keys wk0 .. wk0 + 31. With a band, rows with
// q + diag in [wk0 - wr, wk0 + 31 + wl] see some of the keys and rows with
// q + diag in [wk0 + 31 - wr, wk0 + wl] see all of them.
template <typename E, int D, int MASK, bool BIAS>
__device__ __forceinline__ void dkdv_step(int t, int t_end, const QTileBufs& cur, const QTileBufs& nxt,
                                            const DkdvCopy<D>& cp, const RowRead<D>& rrd, const TrRead<D>& trd,
                                            const bf16x8 (&kf)[D / 16], const bf16x8 (&vf)[D / 16],
                                            f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32], const BwdParams& p,
                                            int wk0, int q_lo, int q_hi, int lane, const float* bcol, bool bkey) {
  const int q0 = t * kTile;
  if (t + 1 < t_end) cp.issue(nxt, q0 + kTile);
  bool live = wk0 < p.nk, masked = false;
  if (MASK != kMaskNone) {
    live = live && q0 + kTile - 1 + p.diag >= wk0 - p.wr;
    masked = q0 + p.diag < wk0 + 31 - p.wr;
    if (MASK == kMaskBand) {
      live = live && q0 + p.diag <= wk0 + 31 + p.wl;
      masked = masked || q0 + kTile - 1 + p.diag > wk0 + p.wl;
    }
  }
  if (live)
    dkdv_tile<E, D, MASK, BIAS>(cur.q, cur.d, cur.st, rrd, trd, kf, vf, dk, dv, p.c, q0, q_lo, q_hi, lane, masked, bcol, bkey,
                                p.bias_sr, p.nq);
  wait_vmem();
  __syncthreads();
}

template <typename E, int D, int MASK, bool BIAS>
__global__ __launch_bounds__(kThreads, 1) void dkdv_kernel(BwdParams p) {
  constexpr int P = lds_pitch<D>();
  __shared__ __attribute__((aligned(1024))) bf16_t q_lds0[kTile * P];
  __shared__ __attribute__((aligned(1024))) bf16_t q_lds1[kTile * P];
  __shared__ __attribute__((aligned(1024))) bf16_t d_lds0[kTile * P];
  __shared__ __attribute__((aligned(1024))) bf16_t d_lds1[kTile * P];
  __shared__ __attribute__((aligned(16))) float s_lds0[2 * kTile];
  __shared__ __attribute__((aligned(16))) float s_lds1[2 * kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hw = lane >> 5;
  const int col = lane & 31;
  const int nq = p.nq, nk = p.nk;

  const int logical = xcd_logical_block(blockIdx.x, (int)gridDim.x);
  const int head = logical / p.nkb;
  const int kblk = logical - head * p.nkb;
  const int key_wg = kblk * kRowsPerBlock;
  const int wk0 = key_wg + wave * kRowsPerWave;
  const int key = wk0 + col;
  // query rows that see this lane's key: [key - diag - wr, key - diag + wl]
  const int q_lo = key - p.diag - p.wr, q_hi = key - p.diag + p.wl;
  // this lane's bias column (the last key's past the end, where bkey is
  // false and the values read are not used)
  const float* bcol = nullptr;
  const bool bkey = key < nk;
  if (BIAS) {
    const int b = head / p.heads;
    bcol = p.bias + b * p.bias_sb + (head - b * p.heads) * p.bias_sh + min(key, nk - 1);
  }

  // query tiles of this work-group's band
  int t_begin = 0, t_end = (nq + kTile - 1) / kTile;
  if (MASK != kMaskNone) {
    const int r_lo = max(0, key_wg - p.diag - p.wr);
    const int r_hi = min(nq - 1, key_wg + kRowsPerBlock - 1 - p.diag + p.wl);
    t_begin = r_lo / kTile;
    t_end = r_hi < r_lo ? t_begin : r_hi / kTile + 1;
  }

  const bf16_t* qh = head_base(p.q, p.q_sb, p.q_sh, p.heads, head);
  const bf16_t* dh = head_base(p.dout, p.do_sb, p.do_sh, p.heads, head);
  const bf16_t* kh = head_base(p.k, p.k_sb, p.k_sh, p.heads, head);
  const bf16_t* vh = head_base(p.v, p.v_sb, p.v_sh, p.heads, head);
  DkdvCopy<D> cp;
  cp.dma.init(wave, lane);
  cp.qrs = rows_rsrc<D>(qh, nq, 2u * p.q_sr);
  cp.drs = rows_rsrc<D>(dh, nq, 2u * p.do_sr);
  cp.srs = make_rsrc(p.stats + (long long)head * p.nq_pad * 2, (uint32_t)p.nq_pad * 8);
  cp.q_stride = 2u * p.q_sr;
  cp.d_stride = 2u * p.do_sr;
  cp.wave = wave;
  cp.lane = lane;
  const QTileBufs b0{q_lds0, d_lds0, s_lds0}, b1{q_lds1, d_lds1, s_lds1};
  if (t_begin < t_end) cp.issue(b0, t_begin * kTile);

  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 kx = u32x4{0u, 0u, 0u, 0u}, vx = kx;
    if (key < nk) {
      kx = *(const u32x4*)(kh + (long long)key * p.k_sr + 16 * ks + 8 * hw);
      vx = *(const u32x4*)(vh + (long long)key * p.v_sr + 16 * ks + 8 * hw);
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
    dkdv_step<E, D, MASK, BIAS>(t, t_end, b0, b1, cp, rrd, trd, kf, vf, dk, dv, p, wk0, q_lo, q_hi, lane, bcol, bkey);
    if (t + 1 < t_end)
      dkdv_step<E, D, MASK, BIAS>(t + 1, t_end, b1, b0, cp, rrd, trd, kf, vf, dk, dv, p, wk0, q_lo, q_hi, lane, bcol, bkey);
  }

  // lane holds d = 32 db + col for keys wk0 + 8 g + 4 hw + rr
  bf16_t* dkh = (bf16_t*)head_base(p.dk, p.dk_sb, p.dk_sh, p.heads, head);
  bf16_t* dvh = (bf16_t*)head_base(p.dv, p.dv_sb, p.dv_sh, p.heads, head);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int kr = wk0 + 8 * g + 4 * hw + rr;
        if (kr < nk) {
          dkh[(long long)kr * p.dk_sr + 32 * db + col] = __builtin_bit_cast(bf16_t, E::cvt(dk[db][4 * g + rr] * p.scale));
          dvh[(long long)kr * p.dv_sr + 32 * db + col] = __builtin_bit_cast(bf16_t, E::cvt(dv[db][4 * g + rr]));
        }
      }
}

// ------------------------------------------- dK, dV split by output ---
//
// The kernel above runs one wave per SIMD (its K/V rows, dK/dV accumulators
// and score tiles take ~340 registers), so its three parts per tile (the S/dP
// products, the vector work forming P and dS, the dV/dK products) run one
// after another and the matrix cores idle through the vector work. This one
// splits the work by output between two waves that share a SIMD, each under
// 256 registers:
//  * group A (waves 0-3) owns dV: it forms S = Q K^T and P = exp2(c S - L),
//    and accumulates dV += P^T dO;
//  * group B (waves 4-7) owns dK: it forms dP = dO V^T and, with A's P handed
//    over through LDS, dS = P (dP - D), and accumulates dK += dS^T Q.
// Waves w and w + 4 own the same 32 keys and run on SIMD w. Their phases
// alternate, so on each SIMD one wave feeds the matrix core while the other
// does vector work; each matrix phase is 2 D / 8 MFMAs:
//   phase 1 of step j:  A: dV += P_{j-1}^T dO_{j-1}, S_j = Q_j K^T | B: dS_{j-1}
//   phase 2 of step j:  A: P_j (registers, and fp32 into LDS for B)  | B: dK += dS_{j-1}^T Q_{j-1}, dP_j = dO_j V^T
// Every product and rounding is the one the kernel above performs, in the
// same order per accumulator, so the two give bit-identical dK and dV.
// Tile j (Q, dO, statistics) is read from phase 1 of step j to phase 2 of
// step j + 1, so tiles are triple-buffered; tile j + 1 goes into the slot
// tile j - 2 left. Both copies are issued outside B's matrix phase: the
// compiler makes LDS reads wait for direct-to-LDS copies it cannot prove
// disjoint, and a copy in flight across B's matrix phase stalled its MFMAs.
//  * A copies Q_{j+1} and its row statistics at the start of its matrix
//    phase of step j and waits for them at the end of step j (A reads them
//    in step j + 1, B's dS and dK one phase later).
//  * B copies dO_{j+1} at the start of its vector phase of step j and waits
//    for it at the end of phase 1 of step j + 1, before its matrix phase
//    reads it; the copy of dO_{j+2}, issued in that phase, stays in flight.

constexpr int kPpThreads = 512;
constexpr int kPpPairs = 4;  // wave pairs (32 keys each) per work-group

struct PpBufs {
  bf16_t* q;
  bf16_t* d;
  float* st;
};

template <int D>
struct PpCopy {
  typedef TileDma<kTile, D, kPpThreads / 2> Dma;  // one group's four waves copy one 64-row tile
  // vector-memory instructions per wave in one dO copy
  static constexpr int kBatch = Dma::kInstr;
  Dma dma;
  __amdgpu_buffer_rsrc_t qrs, drs, srs;
  uint32_t q_stride, d_stride;
  int gwave, lane;
  // Q and the statistics of a tile (group A)
  __device__ __forceinline__ void issue_q(const PpBufs& b, int q0) const {
    dma.issue(qrs, b.q, q0, q_stride);
    if (gwave == 0 && lane < kStatTileBytes / 16) {
      FA_LDS void* dst = (FA_LDS void*)(FA_LDS float*)b.st;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, dst, 16, (uint32_t)(q0 / kTile) * kStatTileBytes + 16 * lane,
                                               0, 0, 0);
    }
  }
  // dO of a tile (group B)
  __device__ __forceinline__ void issue_d(const PpBufs& b, int q0) const { dma.issue(drs, b.d, q0, d_stride); }
};

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt bound out of range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Registers of one wave: its 32 keys' K rows (A) or V rows (B) as B
// operands, its dV (A) or dK (B) accumulators, S (A) or dP (B) of a 64-row
// tile, and P (A) or dS (B) of the previous tile as bf16 A operands.
template <int D>
struct PpState {
  bf16x8 kv[D / 16];
  f32x16 acc[D / 32];
  f32x16 sd[2];
  bf16x8 pd[4];
};

// acc += pd^T T with T read transposed from tile `tt` (rows = queries), then
// sd = R kv^T with R read by rows from tile `rt`. `prev` and `cur` say
// whether the wave's keys see the previous and the current tile.
// Scheduling groups (see __builtin_amdgcn_sched_group_barrier): instruction
// classes the compiler's scheduler must place in the given order. Each block
// of products in the dK/dV kernel keeps kPpAhead LDS operands in flight ahead
// of its MFMAs (the dQ kernel's count is kDqpAhead); unconstrained, the
// scheduler issues every read of the block first and runs out of registers.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kPpAhead = 4;

template <typename E, int D>
__device__ __forceinline__ void pp_matrix(PpState<D>& s, const bf16_t* tt, const bf16_t* rt, bool prev, bool cur,
                                          const RowRead<D>& rrd, const TrRead<D>& trd) {
  constexpr int kN = D / 8;  // MFMAs per block: 4 x D / 32 transposed, 2 x D / 16 by rows
  if (prev) {
    const FA_LDS char* tb = (const FA_LDS char*)(const FA_LDS bf16_t*)tt;
    // output blocks interleaved: no MFMA waits on the one just before it
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) s.acc[db] = E::mfma(s.pd[t], trd.at(tb, t, db), s.acc[db]);
    // two transposed reads per MFMA
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kPpAhead, 0);
#pragma unroll
    for (int i = 0; i < kN - kPpAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
#pragma unroll
    for (int i = 0; i < kPpAhead; ++i) __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
  }
  if (cur) {
    const FA_LDS char* rb = (const FA_LDS char*)(const FA_LDS bf16_t*)rt;
    f32x16 sd[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) sd[qb] = E::mfma(rrd.at(rb, qb, ks), s.kv[ks], sd[qb]);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      s.sd[qb] = sd[qb];
      fence_regs(s.sd[qb]);
    }
    // one row read per MFMA
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kPpAhead, 0);
#pragma unroll
    for (int i = 0; i < kN - kPpAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < kPpAhead; ++i) __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
  }
}

// Group A's vector phase: P of the tile in s.sd (scores S of query rows q0 ..
// q0 + 63 against this lane's key), as bf16 A operands and, in fp32, into the
// pair's LDS slot for group B. With a band, `masked` tiles set P = 0 where
// the query row is outside this lane's [q_lo, q_hi].
template <typename E, int MASK>
__device__ __forceinline__ void pp_probs(bf16x8 (&pd)[4], const f32x16 (&sd)[2], const float* st, f32x4* pslot,
                                         float c, int q0, int q_lo, int q_hi, int lane, bool masked) {
  const int hw = lane >> 5;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int r0 = qb * 32 + 8 * g + 4 * hw;
      const f32x4 Lv = *(const FA_LDS f32x4*)((const FA_LDS float*)st + r0);
      f32x4 pv;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        float arg = fmaf(sd[qb][4 * g + rr], c, -Lv[rr]);
        if (MASK != kMaskNone && masked) {
          const int qr = q0 + r0 + rr;
          arg = (qr < q_lo || (MASK == kMaskBand && qr > q_hi)) ? -INFINITY : arg;
        }
        pv[rr] = fast_exp2(arg);
      }
      *(FA_LDS f32x4*)((FA_LDS f32x4*)pslot + (qb * 4 + g) * 64 + lane) = pv;
      const int t = qb * 2 + (g >> 1);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) pd[t][4 * (g & 1) + rr] = E::cvt(pv[rr]);
    }
#pragma unroll
  for (int t = 0; t < 4; ++t) fence_regs(pd[t]);
}

// Group B's vector phase: dS = P (dP - D) of the previous tile, from group
// A's P in the pair's LDS slot and this wave's dP in s.sd.
template <typename E>
__device__ __forceinline__ void pp_dscores(bf16x8 (&pd)[4], const f32x16 (&sd)[2], const float* st,
                                           const f32x4* pslot, int lane) {
  const int hw = lane >> 5;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int r0 = qb * 32 + 8 * g + 4 * hw;
      const f32x4 Dv = *(const FA_LDS f32x4*)((const FA_LDS float*)st + kTile + r0);
      const f32x4 pv = *(const FA_LDS f32x4*)((const FA_LDS f32x4*)pslot + (qb * 4 + g) * 64 + lane);
      const int t = qb * 2 + (g >> 1);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) pd[t][4 * (g & 1) + rr] = E::cvt(pv[rr] * (sd[qb][4 * g + rr] - Dv[rr]));
    }
#pragma unroll
  for (int t = 0; t < 4; ++t) fence_regs(pd[t]);
}

// Whether the wave's keys wk0 .. wk0 + 31 see query tile q0 .. q0 + 63
// (`live`), and whether some of its pairs are outside the band (`masked`).
template <int MASK>
__device__ __forceinline__ void pp_tile_flags(const BwdParams& p, int q0, int wk0, bool& live, bool& masked) {
  live = wk0 < p.nk;
  masked = false;
  if (MASK != kMaskNone) {
    live = live && q0 + kTile - 1 + p.diag >= wk0 - p.wr;
    masked = q0 + p.diag < wk0 + 31 - p.wr;
    if (MASK == kMaskBand) {
      live = live && q0 + p.diag <= wk0 + 31 + p.wl;
      masked = masked || q0 + kTile - 1 + p.diag > wk0 + p.wl;
    }
  }
}

// Step j of the loop: tile j in `cur`, tile j - 1 in `prv`, tile j + 1 to
// be copied into `nxt`. FIRST: there is no tile j - 1. LAST: j = t_end, there
// is no tile j (only the previous tile's dV, dS and dK remain).
template <typename E, int D, int MASK, bool GROUP_A, bool FIRST, bool LAST>
__device__ __forceinline__ void pp_step(int j, int t_end, const PpBufs& cur, const PpBufs& prv, const PpBufs& nxt,
                                        PpState<D>& s, bool& prev_live, const PpCopy<D>& cp, const RowRead<D>& rrd,
                                        const TrRead<D>& trd, f32x4* pslot, const BwdParams& p, int wk0, int q_lo,
                                        int q_hi, int lane) {
  const int q0 = j * kTile;
  bool live = false, masked = false;
  if (!LAST) pp_tile_flags<MASK>(p, q0, wk0, live, masked);
  const bool prev = !FIRST && prev_live;
  // phase 1: A's matrix phase, B's vector phase
  if constexpr (GROUP_A) {
    if (!LAST && j + 1 < t_end) cp.issue_q(nxt, q0 + kTile);
    pp_matrix<E, D>(s, prv.d, cur.q, prev, live, rrd, trd);
  } else {
    // dO of tile j + 1 into the slot tile j - 2 left
    if (!LAST && j + 1 < t_end) cp.issue_d(nxt, q0 + kTile);
    if (prev) pp_dscores<E>(s.pd, s.sd, prv.st, pslot, lane);
    // tile j's dO, which B reads in the next phase; the copy of tile j + 1
    // may stay in flight
    if (!LAST) {
      if (j + 1 < t_end)
        wait_vmcnt<PpCopy<D>::kBatch>();
      else
        wait_vmem();
    }
  }
  lds_barrier();
  // phase 2: A's vector phase, B's matrix phase
  if constexpr (GROUP_A) {
    if (live) pp_probs<E, MASK>(s.pd, s.sd, cur.st, pslot, p.c, q0, q_lo, q_hi, lane, masked);
    wait_vmem();  // A's copy of Q_{j+1}
  } else {
    pp_matrix<E, D>(s, prv.q, cur.d, prev, live, rrd, trd);
  }
  if (!LAST) lds_barrier();
  prev_live = live;
}

// The whole loop of one group: tile j sits in buffer (j - t_begin) % 3, and
// the loop body is unrolled three times so that each copy of the step names
// fixed buffers.
template <typename E, int D, int MASK, bool GROUP_A>
__device__ __forceinline__ void pp_run(int t_begin, int t_end, const PpBufs& b0, const PpBufs& b1, const PpBufs& b2,
                                       PpState<D>& s, const PpCopy<D>& cp, const RowRead<D>& rrd,
                                       const TrRead<D>& trd, f32x4* pslot, const BwdParams& p, int wk0, int q_lo,
                                       int q_hi, int lane) {
  if (t_begin >= t_end) return;
  bool prev_live = false;
  pp_step<E, D, MASK, GROUP_A, true, false>(t_begin, t_end, b0, b2, b1, s, prev_live, cp, rrd, trd, pslot, p, wk0,
                                            q_lo, q_hi, lane);
  int j = t_begin + 1;
  for (; j + 2 < t_end; j += 3) {
    pp_step<E, D, MASK, GROUP_A, false, false>(j, t_end, b1, b0, b2, s, prev_live, cp, rrd, trd, pslot, p, wk0, q_lo,
                                               q_hi, lane);
    pp_step<E, D, MASK, GROUP_A, false, false>(j + 1, t_end, b2, b1, b0, s, prev_live, cp, rrd, trd, pslot, p, wk0,
                                               q_lo, q_hi, lane);
    pp_step<E, D, MASK, GROUP_A, false, false>(j + 2, t_end, b0, b2, b1, s, prev_live, cp, rrd, trd, pslot, p, wk0,
                                               q_lo, q_hi, lane);
  }
  if (j < t_end) {
    pp_step<E, D, MASK, GROUP_A, false, false>(j, t_end, b1, b0, b2, s, prev_live, cp, rrd, trd, pslot, p, wk0, q_lo,
                                               q_hi, lane);
    ++j;
  }
  if (j < t_end) {
    pp_step<E, D, MASK, GROUP_A, false, false>(j, t_end, b2, b1, b0, s, prev_live, cp, rrd, trd, pslot, p, wk0, q_lo,
                                               q_hi, lane);
    ++j;
  }
  // j = t_end: the last tile's dV, dS and dK; that tile sits in buffer (j - 1 - t_begin) % 3
  const int last = (j - 1 - t_begin) % 3;
  const PpBufs& lb = last == 0 ? b0 : last == 1 ? b1 : b2;
  pp_step<E, D, MASK, GROUP_A, false, true>(j, t_end, b0, lb, b0, s, prev_live, cp, rrd, trd, pslot, p, wk0, q_lo,
                                            q_hi, lane);
}

template <typename E, int D, int MASK>
__global__ __launch_bounds__(kPpThreads, 2) void dkdv_pp_kernel(BwdParams p) {
  constexpr int P = lds_pitch<D>();
  __shared__ __attribute__((aligned(1024))) bf16_t q_lds0[kTile * P];
  __shared__ __attribute__((aligned(1024))) bf16_t q_lds1[kTile * P];
  __shared__ __attribute__((aligned(1024))) bf16_t q_lds2[kTile * P];
  __shared__ __attribute__((aligned(1024))) bf16_t d_lds0[kTile * P];
  __shared__ __attribute__((aligned(1024))) bf16_t d_lds1[kTile * P];
  __shared__ __attribute__((aligned(1024))) bf16_t d_lds2[kTile * P];
  __shared__ __attribute__((aligned(16))) float s_lds0[2 * kTile];
  __shared__ __attribute__((aligned(16))) float s_lds1[2 * kTile];
  __shared__ __attribute__((aligned(16))) float s_lds2[2 * kTile];
  // P of each wave pair's 64 x 32 tile, fp32, one 16-byte chunk per lane per
  // (query block, group of 4 rows)
  __shared__ __attribute__((aligned(1024))) f32x4 p_lds[kPpPairs * 8 * 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool group_a = wave < kPpPairs;
  const int pair = wave & (kPpPairs - 1);
  const int hw = lane >> 5;
  const int col = lane & 31;
  const int nq = p.nq, nk = p.nk;

  const int logical = xcd_logical_block(blockIdx.x, (int)gridDim.x);
  const int head = logical / p.nkb;
  const int kblk = logical - head * p.nkb;
  const int key_wg = kblk * kRowsPerBlock;
  const int wk0 = key_wg + pair * kRowsPerWave;
  const int key = wk0 + col;
  // query rows that see this lane's key: [key - diag - wr, key - diag + wl]
  const int q_lo = key - p.diag - p.wr, q_hi = key - p.diag + p.wl;

  // query tiles of this work-group's band
  int t_begin = 0, t_end = (nq + kTile - 1) / kTile;
  if (MASK != kMaskNone) {
    const int r_lo = max(0, key_wg - p.diag - p.wr);
    const int r_hi = min(nq - 1, key_wg + kRowsPerBlock - 1 - p.diag + p.wl);
    t_begin = r_lo / kTile;
    t_end = r_hi < r_lo ? t_begin : r_hi / kTile + 1;
  }

  const bf16_t* qh = head_base(p.q, p.q_sb, p.q_sh, p.heads, head);
  const bf16_t* dh = head_base(p.dout, p.do_sb, p.do_sh, p.heads, head);
  PpCopy<D> cp;
  cp.dma.init(pair, lane);
  cp.qrs = rows_rsrc<D>(qh, nq, 2u * p.q_sr);
  cp.drs = rows_rsrc<D>(dh, nq, 2u * p.do_sr);
  cp.srs = make_rsrc(p.stats + (long long)head * p.nq_pad * 2, (uint32_t)p.nq_pad * 8);
  cp.q_stride = 2u * p.q_sr;
  cp.d_stride = 2u * p.do_sr;
  cp.gwave = pair;
  cp.lane = lane;
  const PpBufs b0{q_lds0, d_lds0, s_lds0}, b1{q_lds1, d_lds1, s_lds1}, b2{q_lds2, d_lds2, s_lds2};
  // tile t_begin: A copies Q and the statistics, B copies dO
  if (t_begin < t_end) {
    if (group_a) {
      cp.issue_q(b0, t_begin * kTile);
    } else {
      cp.issue_d(b0, t_begin * kTile);
    }
  }

  // A: the K rows of its keys; B: the V rows
  PpState<D> s;
  {
    const bf16_t* src = group_a ? head_base(p.k, p.k_sb, p.k_sh, p.heads, head)
                                : head_base(p.v, p.v_sb, p.v_sh, p.heads, head);
    const long long sr = group_a ? p.k_sr : p.v_sr;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 x = u32x4{0u, 0u, 0u, 0u};
      if (key < nk) x = *(const u32x4*)(src + (long long)key * sr + 16 * ks + 8 * hw);
      s.kv[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }
#pragma unroll
  for (int db = 0; db < D / 32; ++db) s.acc[db] = f32x16{};
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) s.sd[qb] = f32x16{};
#pragma unroll
  for (int t = 0; t < 4; ++t) s.pd[t] = bf16x8{};
  RowRead<D> rrd;
  rrd.init(lane);
  TrRead<D> trd;
  trd.init(lane);
  f32x4* pslot = p_lds + pair * 8 * 64;

  // K / V rows and tile t_begin
  wait_vmem();
  lds_barrier();
  // The two groups run separate copies of the loop (the same sequence of
  // work-group barriers): one loop holding both groups' values at every
  // phase join needs more registers than two waves per SIMD leave.
  if (group_a)
    pp_run<E, D, MASK, true>(t_begin, t_end, b0, b1, b2, s, cp, rrd, trd, pslot, p, wk0, q_lo, q_hi, lane);
  else
    pp_run<E, D, MASK, false>(t_begin, t_end, b0, b1, b2, s, cp, rrd, trd, pslot, p, wk0, q_lo, q_hi, lane);

  // lane holds d = 32 db + col for keys wk0 + 8 g + 4 hw + rr; A stores dV, B stores dK (x scale)
  bf16_t* outh = group_a ? (bf16_t*)head_base(p.dv, p.dv_sb, p.dv_sh, p.heads, head)
                         : (bf16_t*)head_base(p.dk, p.dk_sb, p.dk_sh, p.heads, head);
  const long long osr = group_a ? p.dv_sr : p.dk_sr;
  const float oscale = group_a ? 1.f : p.scale;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int kr = wk0 + 8 * g + 4 * hw + rr;
        if (kr < nk) outh[(long long)kr * osr + 32 * db + col] = __builtin_bit_cast(bf16_t, E::cvt(s.acc[db][4 * g + rr] * oscale));
      }
}

// -------------------------------------------------------------------- dQ ---

// One 64-key tile against the wave's 32 query rows. `masked` tiles set P = 0
// for keys past the end and, with a band, outside this lane's [k_lo, k_hi].
// MASK_CODE says whether the tile carries that code at all: the unmasked main
// loop of a kernel without band has no branch in the middle of its tiles.
template <typename E, int D, int MASK, bool BIAS, bool MASK_CODE>
__device__ __forceinline__ void dq_tile(const bf16_t* kt, const bf16_t* vt, const RowRead<D>& rrd,
                                        const TrRead<D>& trd, const bf16x8 (&qf)[D / 16],
                                        const bf16x8 (&df)[D / 16], f32x16 (&dq)[D / 32], float lse2, float drow,
                                        float c, int key0, int k_lo, int k_hi, int lane, bool masked,
                                        const float* brow, int nk) {
  const int hw = lane >> 5;
  f32x16 s[2], dpt[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    s[kb] = f32x16{};
    dpt[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      s[kb] = E::mfma(rrd(kt, kb, ks), qf[ks], s[kb]);
      dpt[kb] = E::mfma(rrd(vt, kb, ks), df[ks], dpt[kb]);
    }
  }
  // two operands in flight: without a pattern every MFMA waited for its own
  // read (at d = 256 all 192 of them)
  sched_reads_ahead<4 * (D / 16), 1, 2>();
  bf16x8 ds[4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    // bias of this lane's query row for this key block, four consecutive
    // keys per load (one block at a time, to bound the registers it takes)
    f32x4 bv[4];
    if constexpr (BIAS) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int kc = key0 + kb * 32 + 8 * g + 4 * hw;
        bv[g] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (kc + 3 < nk) {
          bv[g] = *(const f32x4*)(brow + kc);
        } else {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            if (kc + rr < nk) bv[g][rr] = brow[kc + rr];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float arg = fmaf(s[kb][i], c, -lse2);
      if constexpr (BIAS) arg = fmaf(kLog2e, bv[i >> 2][i & 3], arg);
      if (MASK_CODE && masked) {
        const int key = key0 + kb * 32 + 8 * (i >> 2) + 4 * hw + (i & 3);
        arg = (key > k_hi || (MASK == kMaskBand && key < k_lo)) ? -INFINITY : arg;
      }
      const float pv = fast_exp2(arg);
      ds[kb * 2 + (i >> 3)][i & 7] = E::cvt(pv * (dpt[kb][i] - drow));
    }
    if constexpr (BIAS) __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int t = 0; t < 4; ++t) dq[db] = E::mfma(trd(kt, t, db), ds[t], dq[db]);
  sched_reads_ahead<4 * (D / 32), 2, 2>();
}

template <typename E, int D, int MASK, bool BIAS, bool MASK_CODE>
__device__ __forceinline__ void dq_step(int j, int n_tiles, int key_base, const bf16_t* kt, const bf16_t* vt,
                                        bf16_t* kn, bf16_t* vn, const TileDma<kTile, D, kThreads>& dma,
                                        __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                        const RowRead<D>& rrd, const TrRead<D>& trd, const bf16x8 (&qf)[D / 16],
                                        const bf16x8 (&df)[D / 16], f32x16 (&dq)[D / 32], float lse2, float drow,
                                        const BwdParams& p, int k_lo, int k_hi, int wq0, int lane, const float* brow) {
  const int key0 = key_base + j * kTile;
  if (j + 1 < n_tiles) {
    dma.issue(krs, kn, key0 + kTile, 2u * p.k_sr);
    dma.issue(vrs, vn, key0 + kTile, 2u * p.v_sr);
  }
  // the wave's rows are wq0 .. wq0 + 31 (rows past nq are never stored)
  bool live = wq0 < p.nq, masked = key0 + kTile > p.nk;
  if (MASK != kMaskNone) {
    live = live && key0 <= wq0 + 31 + p.diag + p.wr;
    masked = masked || key0 + kTile - 1 > wq0 + p.diag + p.wr;
    if (MASK == kMaskBand) {
      live = live && key0 + kTile - 1 >= wq0 + p.diag - p.wl;
      masked = masked || key0 < wq0 + 31 + p.diag - p.wl;
    }
  }
  if (live)
    dq_tile<E, D, MASK, BIAS, MASK_CODE>(kt, vt, rrd, trd, qf, df, dq, lse2, drow, p.c, key0, k_lo, k_hi, lane, masked,
                                         brow, p.nk);
  wait_vmem();
  __syncthreads();
}

// dQ work-groups per CU: two, except at d = 256, whose Q, dO and dQ rows fill
// the registers of one wave per SIMD and whose K/V tiles fill the LDS.
template <int D>
constexpr int dq_blocks_per_cu() {
  return D >= 256 ? 1 : 2;
}

// RAGGED (kernels without a band only): N_k is not a multiple of the 64-key
// tile, so the last tile must mask keys past the end.
template <typename E, int D, int MASK, bool BIAS, bool RAGGED>
__global__ __launch_bounds__(kThreads, dq_blocks_per_cu<D>()) void dq_kernel(BwdParams p) {
  constexpr bool BAND = MASK != kMaskNone;
  constexpr int P = lds_pitch<D>();
  __shared__ __attribute__((aligned(1024))) bf16_t k_lds0[kTile * P];
  __shared__ __attribute__((aligned(1024))) bf16_t k_lds1[kTile * P];
  __shared__ __attribute__((aligned(1024))) bf16_t v_lds0[kTile * P];
  __shared__ __attribute__((aligned(1024))) bf16_t v_lds1[kTile * P];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hw = lane >> 5;
  const int col = lane & 31;
  const int nq = p.nq, nk = p.nk;

  const int logical = xcd_logical_block(blockIdx.x, (int)gridDim.x);
  const int head = logical / p.nqb;
  int qblk = logical - head * p.nqb;
  if (BAND) qblk = p.nqb - 1 - qblk;  // longest rows first under a causal band
  const int q_row0 = qblk * kRowsPerBlock;
  const int wq0 = q_row0 + wave * kRowsPerWave;
  const int qi = wq0 + col;
  // bias row of this lane's query (rows past nq read the last row; unused)
  const float* brow = nullptr;
  if (BIAS) {
    const int b = head / p.heads;
    brow = p.bias + b * p.bias_sb + (head - b * p.heads) * p.bias_sh + (long long)min(qi, nq - 1) * p.bias_sr;
  }
  // live keys of this lane's row: [k_lo, k_hi]
  const int k_lo = BAND ? qi + p.diag - p.wl : 0;
  const int k_hi = BAND ? min(nk - 1, qi + p.diag + p.wr) : nk - 1;

  // key tiles of this work-group's band
  const int q_last = min(nq, q_row0 + kRowsPerBlock) - 1;
  int key_base = 0, n_tiles = (nk + kTile - 1) / kTile;
  if (BAND) {
    const int c_lo = max(0, q_row0 + p.diag - p.wl);
    const int c_hi = min(nk - 1, q_last + p.diag + p.wr);
    key_base = c_lo / kTile * kTile;
    n_tiles = c_hi < c_lo ? 0 : (c_hi - key_base) / kTile + 1;
  }

  const bf16_t* qh = head_base(p.q, p.q_sb, p.q_sh, p.heads, head);
  const bf16_t* dh = head_base(p.dout, p.do_sb, p.do_sh, p.heads, head);
  const bf16_t* kh = head_base(p.k, p.k_sb, p.k_sh, p.heads, head);
  const bf16_t* vh = head_base(p.v, p.v_sb, p.v_sh, p.heads, head);
  const __amdgpu_buffer_rsrc_t krs = rows_rsrc<D>(kh, nk, 2u * p.k_sr);
  const __amdgpu_buffer_rsrc_t vrs = rows_rsrc<D>(vh, nk, 2u * p.v_sr);
  TileDma<kTile, D, kThreads> dma;
  dma.init(wave, lane);
  if (n_tiles > 0) {
    dma.issue(krs, k_lds0, key_base, 2u * p.k_sr);
    dma.issue(vrs, v_lds0, key_base, 2u * p.v_sr);
  }

  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 qx = u32x4{0u, 0u, 0u, 0u}, dx = qx;
    if (qi < nq) {
      qx = *(const u32x4*)(qh + (long long)qi * p.q_sr + 16 * ks + 8 * hw);
      dx = *(const u32x4*)(dh + (long long)qi * p.do_sr + 16 * ks + 8 * hw);
    }
    qf[ks] = __builtin_bit_cast(bf16x8, qx);
    df[ks] = __builtin_bit_cast(bf16x8, dx);
  }
  float lse2 = 0.f, drow = 0.f;
  if (qi < nq) {
    const float* st = p.stats + ((long long)head * p.nq_pad + (qi & ~(kTile - 1))) * 2;
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

  wait_vmem();
  __syncthreads();
  // Tiles carry masking code only where some can need it: with a band, or
  // when the last key tile is ragged (a zero K row past the end would get
  // p = exp2(-LSE log2 e), which overflows for very negative LSE). Without
  // either, the loop has no branch in the middle of its tiles. (A separate
  // masked copy of the step for the ragged tile alone, after the main loop,
  // cost the kernel 12 spilled registers at d = 128.)
  constexpr bool MASK_CODE = BAND || RAGGED;
  for (int j = 0; j < n_tiles; j += 2) {
    dq_step<E, D, MASK, BIAS, MASK_CODE>(j, n_tiles, key_base, k_lds0, v_lds0, k_lds1, v_lds1, dma, krs, vrs, rrd, trd,
                                         qf, df, dq, lse2, drow, p, k_lo, k_hi, wq0, lane, brow);
    if (j + 1 < n_tiles)
      dq_step<E, D, MASK, BIAS, MASK_CODE>(j + 1, n_tiles, key_base, k_lds1, v_lds1, k_lds0, v_lds0, dma, krs, vrs, rrd,
                                           trd, qf, df, dq, lse2, drow, p, k_lo, k_hi, wq0, lane, brow);
  }

  if (qi < nq) {
    bf16_t* row = (bf16_t*)head_base(p.dq, p.dq_sb, p.dq_sh, p.heads, head) + (long long)qi * p.dq_sr;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 w;
        w.x = pack2<E>(dq[db][4 * g] * p.scale, dq[db][4 * g + 1] * p.scale);
        w.y = pack2<E>(dq[db][4 * g + 2] * p.scale, dq[db][4 * g + 3] * p.scale);
        *(uint2*)(row + db * 32 + 8 * g + 4 * hw) = w;
      }
  }
}

// ------------------------------------------------ dQ, two wave groups ---
//
// The kernel above runs two independent work-groups per CU, so whether one
// wave's MFMAs overlap the other wave's vector work on a SIMD is left to
// chance. This one (no bias, d = 96 and 128) runs one work-group of 8 waves (256
// query rows) per CU as two groups of four with the forward pass's
// ping-pong: each wave's work per 64-key tile splits into a matrix phase
// (dQ^T += K_{j-1}^T dS_{j-1}^T for the previous tile, then S^T_j = K_j Q^T
// and dP^T_j = V_j dO^T) and a vector phase (P and dS of tile j), group B
// runs one work-group barrier behind group A, and so on every SIMD one wave
// feeds the matrix core while the other does vector work. Products and
// roundings are the kernel above's, in the same order per accumulator.
// K_j is read in matrix phases j and j + 1, so K and V tiles are
// triple-buffered; group A copies K_{j+1} and V_{j+1} (into the slot of tile
// j - 2) at the start of its matrix phase j and waits for them at the end of
// its vector phase j, before their first reader (its matrix phase j + 1).
// Group B never has a copy in flight.

constexpr int kDqpThreads = 512;
constexpr int kDqpRows = 256;  // query rows per work-group

struct DqpBufs {
  bf16_t* k;
  bf16_t* v;
};

template <int D>
struct DqpState {
  bf16x8 qf[D / 16], df[D / 16];  // this lane's Q and dO rows as B operands
  f32x16 dq[D / 32];              // dQ^T: register r of dq[db] holds d = 32 db + 8 (r / 4) + 4 hw + r % 4
  f32x16 s[2], dpt[2];            // S^T and dP^T of the current tile (lane = query)
  bf16x8 ds[4];                   // dS^T of the previous tile as bf16 B operands
  float lse2, drow;
};

// Operands in flight in the dQ kernel's matrix phase: three, where four
// pushed the causal kernel at d = 128 to 256 registers and the scheduler then
// dropped part of the pattern (43 of 240 MFMAs waited on their own read, 14
// with three).
constexpr int kDqpAhead = 3;

template <typename E, int D>
__device__ __forceinline__ void dqp_matrix(DqpState<D>& st, const bf16_t* kprev, const bf16_t* kcur,
                                           const bf16_t* vcur, bool prev, bool cur, const RowRead<D>& rrd,
                                           const TrRead<D>& trd) {
  constexpr int kN = D / 8;  // transposed dQ MFMAs (4 x D / 32), two reads each
  if (prev) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) st.dq[db] = E::mfma(trd(kprev, t, db), st.ds[t], st.dq[db]);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kDqpAhead, 0);
#pragma unroll
    for (int i = 0; i < kN - kDqpAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
#pragma unroll
    for (int i = 0; i < kDqpAhead; ++i) __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
  }
  if (cur) {
    f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = E::mfma(rrd(kcur, kb, ks), st.qf[ks], s[kb]);
        dp[kb] = E::mfma(rrd(vcur, kb, ks), st.df[ks], dp[kb]);
      }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      st.s[kb] = s[kb];
      st.dpt[kb] = dp[kb];
      fence_regs(st.s[kb]);
      fence_regs(st.dpt[kb]);
    }
    // one row read per MFMA
    constexpr int kR = D / 4;
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kDqpAhead, 0);
#pragma unroll
    for (int i = 0; i < kR - kDqpAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < kDqpAhead; ++i) __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
  }
}

// Vector phase: dS^T = P (dP - D) of the tile in st.s / st.dpt, keys key0 ..
// key0 + 63. `masked` tiles (band edges, ragged end; MASK_CODE kernels only)
// set P = 0 for keys outside this lane's [k_lo, k_hi].
template <typename E, int MASK, bool MASK_CODE>
__device__ __forceinline__ void dqp_vector(bf16x8 (&ds)[4], const f32x16 (&s)[2], const f32x16 (&dpt)[2], float lse2,
                                           float drow, float c, int key0, int k_lo, int k_hi, int lane, bool masked) {
  const int hw = lane >> 5;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float arg = fmaf(s[kb][i], c, -lse2);
      if (MASK_CODE && masked) {
        const int key = key0 + kb * 32 + 8 * (i >> 2) + 4 * hw + (i & 3);
        arg = (key > k_hi || (MASK == kMaskBand && key < k_lo)) ? -INFINITY : arg;
      }
      const float pv = fast_exp2(arg);
      ds[kb * 2 + (i >> 3)][i & 7] = E::cvt(pv * (dpt[kb][i] - drow));
    }
#pragma unroll
  for (int t = 0; t < 4; ++t) fence_regs(ds[t]);
}

// Whether the wave's query rows wq0 .. wq0 + 31 see key tile key0 .. key0 +
// 63 (`live`) and whether the tile needs masking (`masked`).
template <int MASK>
__device__ __forceinline__ void dqp_tile_flags(const BwdParams& p, int key0, int wq0, bool& live, bool& masked) {
  live = wq0 < p.nq;
  masked = key0 + kTile > p.nk;
  if (MASK != kMaskNone) {
    live = live && key0 <= wq0 + 31 + p.diag + p.wr;
    masked = masked || key0 + kTile - 1 > wq0 + p.diag + p.wr;
    if (MASK == kMaskBand) {
      live = live && key0 + kTile - 1 >= wq0 + p.diag - p.wl;
      masked = masked || key0 < wq0 + 31 + p.diag - p.wl;
    }
  }
}

// Iteration j (0 <= j <= n_tiles) of one wave: matrix phase j (tile j - 1 in
// `prv`, tile j in `cur`), a barrier, vector phase j, a barrier. Group A
// copies tile j + 1 into `nxt` at the start of its matrix phase.
template <typename E, int D, int MASK, bool MASK_CODE>
__device__ __forceinline__ void dqp_iteration(int j, int n_tiles, int key_base, bool group_a, const DqpBufs& cur,
                                              const DqpBufs& prv, const DqpBufs& nxt,
                                              const TileDma<kTile, D, kDqpThreads / 2>& dma,
                                              __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                              const RowRead<D>& rrd, const TrRead<D>& trd, DqpState<D>& st,
                                              bool& prev_live, const BwdParams& p, int wq0, int k_lo, int k_hi,
                                              int lane) {
  const int key0 = key_base + j * kTile;
  bool live = false, masked = false;
  if (j < n_tiles) dqp_tile_flags<MASK>(p, key0, wq0, live, masked);
  if (group_a && j + 1 < n_tiles) {
    dma.issue(krs, nxt.k, key0 + kTile, 2u * p.k_sr);
    dma.issue(vrs, nxt.v, key0 + kTile, 2u * p.v_sr);
  }
  dqp_matrix<E, D>(st, prv.k, cur.k, cur.v, j > 0 && prev_live, live, rrd, trd);
  lds_barrier();
  if (live)
    dqp_vector<E, MASK, MASK_CODE>(st.ds, st.s, st.dpt, st.lse2, st.drow, p.c, key0, k_lo, k_hi, lane, masked);
  if (group_a) wait_vmem();  // tile j + 1, read from the next matrix phase on
  lds_barrier();
  prev_live = live;
}

template <typename E, int D, int MASK, bool RAGGED>
__global__ __launch_bounds__(kDqpThreads, 2) void dq_pp_kernel(BwdParams p) {
  constexpr bool BAND = MASK != kMaskNone;
  constexpr bool MASK_CODE = BAND || RAGGED;
  constexpr int P = lds_pitch<D>();
  __shared__ __attribute__((aligned(1024))) bf16_t k_lds0[kTile * P];
  __shared__ __attribute__((aligned(1024))) bf16_t k_lds1[kTile * P];
  __shared__ __attribute__((aligned(1024))) bf16_t k_lds2[kTile * P];
  __shared__ __attribute__((aligned(1024))) bf16_t v_lds0[kTile * P];
  __shared__ __attribute__((aligned(1024))) bf16_t v_lds1[kTile * P];
  __shared__ __attribute__((aligned(1024))) bf16_t v_lds2[kTile * P];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool group_a = wave < 4;
  const int hw = lane >> 5;
  const int col = lane & 31;
  const int nq = p.nq, nk = p.nk;

  const int logical = xcd_logical_block(blockIdx.x, (int)gridDim.x);
  const int head = logical / p.nqb;
  int qblk = logical - head * p.nqb;
  if (BAND) qblk = p.nqb - 1 - qblk;  // longest rows first under a causal band
  const int q_row0 = qblk * kDqpRows;
  const int wq0 = q_row0 + wave * kRowsPerWave;
  const int qi = wq0 + col;
  // live keys of this lane's row: [k_lo, k_hi]
  const int k_lo = BAND ? qi + p.diag - p.wl : 0;
  const int k_hi = BAND ? min(nk - 1, qi + p.diag + p.wr) : nk - 1;

  // key tiles of this work-group's band
  const int q_last = min(nq, q_row0 + kDqpRows) - 1;
  int key_base = 0, n_tiles = (nk + kTile - 1) / kTile;
  if (BAND) {
    const int c_lo = max(0, q_row0 + p.diag - p.wl);
    const int c_hi = min(nk - 1, q_last + p.diag + p.wr);
    key_base = c_lo / kTile * kTile;
    n_tiles = c_hi < c_lo ? 0 : (c_hi - key_base) / kTile + 1;
  }

  const bf16_t* qh = head_base(p.q, p.q_sb, p.q_sh, p.heads, head);
  const bf16_t* dh = head_base(p.dout, p.do_sb, p.do_sh, p.heads, head);
  const bf16_t* kh = head_base(p.k, p.k_sb, p.k_sh, p.heads, head);
  const bf16_t* vh = head_base(p.v, p.v_sb, p.v_sh, p.heads, head);
  const __amdgpu_buffer_rsrc_t krs = rows_rsrc<D>(kh, nk, 2u * p.k_sr);
  const __amdgpu_buffer_rsrc_t vrs = rows_rsrc<D>(vh, nk, 2u * p.v_sr);
  TileDma<kTile, D, kDqpThreads / 2> dma;  // group A's four waves copy every tile
  dma.init(wave & 3, lane);
  const DqpBufs b0{k_lds0, v_lds0}, b1{k_lds1, v_lds1}, b2{k_lds2, v_lds2};
  if (group_a && n_tiles > 0) {
    dma.issue(krs, b0.k, key_base, 2u * p.k_sr);
    dma.issue(vrs, b0.v, key_base, 2u * p.v_sr);
  }

  DqpState<D> st;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 qx = u32x4{0u, 0u, 0u, 0u}, dx = qx;
    if (qi < nq) {
      qx = *(const u32x4*)(qh + (long long)qi * p.q_sr + 16 * ks + 8 * hw);
      dx = *(const u32x4*)(dh + (long long)qi * p.do_sr + 16 * ks + 8 * hw);
    }
    st.qf[ks] = __builtin_bit_cast(bf16x8, qx);
    st.df[ks] = __builtin_bit_cast(bf16x8, dx);
  }
  st.lse2 = 0.f;
  st.drow = 0.f;
  if (qi < nq) {
    const float* sp = p.stats + ((long long)head * p.nq_pad + (qi & ~(kTile - 1))) * 2;
    st.lse2 = sp[qi & (kTile - 1)];
    st.drow = sp[kTile + (qi & (kTile - 1))];
  }
#pragma unroll
  for (int db = 0; db < D / 32; ++db) st.dq[db] = f32x16{};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) st.s[kb] = st.dpt[kb] = f32x16{};
#pragma unroll
  for (int t = 0; t < 4; ++t) st.ds[t] = bf16x8{};
  RowRead<D> rrd;
  rrd.init(lane);
  TrRead<D> trd;
  trd.init(lane);

  wait_vmem();
  lds_barrier();
  // Group B runs one barrier behind group A: while A is in its matrix phase
  // j, B is in its vector phase j - 1, and the other way round.
  if (!group_a) lds_barrier();
  bool prev_live = false;
  // tile j sits in slot j % 3; iteration n_tiles only adds the last tile's dQ
  int j = 0;
  for (; j + 2 <= n_tiles; j += 3) {
    dqp_iteration<E, D, MASK, MASK_CODE>(j, n_tiles, key_base, group_a, b0, b2, b1, dma, krs, vrs, rrd, trd, st,
                                         prev_live, p, wq0, k_lo, k_hi, lane);
    dqp_iteration<E, D, MASK, MASK_CODE>(j + 1, n_tiles, key_base, group_a, b1, b0, b2, dma, krs, vrs, rrd, trd, st,
                                         prev_live, p, wq0, k_lo, k_hi, lane);
    dqp_iteration<E, D, MASK, MASK_CODE>(j + 2, n_tiles, key_base, group_a, b2, b1, b0, dma, krs, vrs, rrd, trd, st,
                                         prev_live, p, wq0, k_lo, k_hi, lane);
  }
  if (j <= n_tiles) {
    dqp_iteration<E, D, MASK, MASK_CODE>(j, n_tiles, key_base, group_a, b0, b2, b1, dma, krs, vrs, rrd, trd, st,
                                         prev_live, p, wq0, k_lo, k_hi, lane);
    ++j;
  }
  if (j <= n_tiles) {
    dqp_iteration<E, D, MASK, MASK_CODE>(j, n_tiles, key_base, group_a, b1, b0, b2, dma, krs, vrs, rrd, trd, st,
                                         prev_live, p, wq0, k_lo, k_hi, lane);
  }
  if (group_a) lds_barrier();

  if (qi < nq) {
    bf16_t* row = (bf16_t*)head_base(p.dq, p.dq_sb, p.dq_sh, p.heads, head) + (long long)qi * p.dq_sr;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 w;
        w.x = pack2<E>(st.dq[db][4 * g] * p.scale, st.dq[db][4 * g + 1] * p.scale);
        w.y = pack2<E>(st.dq[db][4 * g + 2] * p.scale, st.dq[db][4 * g + 3] * p.scale);
        *(uint2*)(row + db * 32 + 8 * g + 4 * hw) = w;
      }
  }
}

// The kernels the launchers below can reach: the single-role dK/dV kernel
// and the one-group dQ kernel with a bias, and without one at d = 256; the
// split dK/dV kernel for d <= 128 without a bias; the two-group dQ kernel for
// d = 96 and 128 without a bias, the one-group one below (ragged dQ variants
// only without a band).
#define FA_BWD_DQ(E, D, B)                                                    \
  template __global__ void dq_kernel<E, D, kMaskNone, B, false>(BwdParams);  \
  template __global__ void dq_kernel<E, D, kMaskNone, B, true>(BwdParams);   \
  template __global__ void dq_kernel<E, D, kMaskUpper, B, false>(BwdParams); \
  template __global__ void dq_kernel<E, D, kMaskBand, B, false>(BwdParams);
#define FA_BWD_COMMON(E, D)                                                                                      \
  template __global__ void dkdv_kernel<E, D, kMaskNone, true>(BwdParams);                                     \
  template __global__ void dkdv_kernel<E, D, kMaskUpper, true>(BwdParams);                                    \
  template __global__ void dkdv_kernel<E, D, kMaskBand, true>(BwdParams);                                     \
  FA_BWD_DQ(E, D, true)                                                                                          \
  template __global__ void row_stats_kernel<E, D>(const bf16_t*, const bf16_t*, const float*, float*, Strides, \
                                                  Strides, int, int, int, long long);
#define FA_BWD_SPLIT(E, D)                                                   \
  FA_BWD_COMMON(E, D)                                                        \
  template __global__ void dkdv_pp_kernel<E, D, kMaskNone>(BwdParams);       \
  template __global__ void dkdv_pp_kernel<E, D, kMaskUpper>(BwdParams);      \
  template __global__ void dkdv_pp_kernel<E, D, kMaskBand>(BwdParams);
#define FA_BWD_DQPP(E, D)                                                    \
  template __global__ void dq_pp_kernel<E, D, kMaskNone, false>(BwdParams);  \
  template __global__ void dq_pp_kernel<E, D, kMaskNone, true>(BwdParams);   \
  template __global__ void dq_pp_kernel<E, D, kMaskUpper, false>(BwdParams); \
  template __global__ void dq_pp_kernel<E, D, kMaskBand, false>(BwdParams);
#define FA_BWD_ALL(E)                                                         \
  FA_BWD_SPLIT(E, 32)                                                         \
  FA_BWD_DQ(E, 32, false)                                                     \
  FA_BWD_SPLIT(E, 64)                                                         \
  FA_BWD_DQ(E, 64, false)                                                     \
  FA_BWD_SPLIT(E, 96)                                                         \
  FA_BWD_DQPP(E, 96)                                                          \
  FA_BWD_SPLIT(E, 128)                                                        \
  FA_BWD_DQPP(E, 128)                                                         \
  FA_BWD_COMMON(E, 256)                                                       \
  FA_BWD_DQ(E, 256, false)                                                    \
  template __global__ void dkdv_kernel<E, 256, kMaskNone, false>(BwdParams);  \
  template __global__ void dkdv_kernel<E, 256, kMaskUpper, false>(BwdParams); \
  template __global__ void dkdv_kernel<E, 256, kMaskBand, false>(BwdParams);
FA_BWD_ALL(Bf16)
FA_BWD_ALL(F16)
#undef FA_BWD_ALL
#undef FA_BWD_SPLIT
#undef FA_BWD_COMMON
#undef FA_BWD_DQ
#undef FA_BWD_DQPP

template <typename E, int D, int MASK, bool BIAS>
hipError_t launch(const BwdArgs& a) {
  const Geometry& g = a.g;
  BwdParams p;
  p.q = (const bf16_t*)a.q;
  p.k = (const bf16_t*)a.k;
  p.v = (const bf16_t*)a.v;
  p.dout = (const bf16_t*)a.dout;
  p.stats = a.workspace;
  p.dq = (bf16_t*)a.dq;
  p.dk = (bf16_t*)a.dk;
  p.dv = (bf16_t*)a.dv;
  p.q_sb = a.sq.b, p.q_sh = a.sq.h, p.q_sr = (int)a.sq.r;
  p.k_sb = a.sk.b, p.k_sh = a.sk.h, p.k_sr = (int)a.sk.r;
  p.v_sb = a.sv.b, p.v_sh = a.sv.h, p.v_sr = (int)a.sv.r;
  p.do_sb = a.sdo.b, p.do_sh = a.sdo.h, p.do_sr = (int)a.sdo.r;
  p.dq_sb = a.sdq.b, p.dq_sh = a.sdq.h, p.dq_sr = (int)a.sdq.r;
  p.dk_sb = a.sdk.b, p.dk_sh = a.sdk.h, p.dk_sr = (int)a.sdk.r;
  p.dv_sb = a.sdv.b, p.dv_sh = a.sdv.h, p.dv_sr = (int)a.sdv.r;
  p.bias = a.bias;
  p.bias_sb = a.sbias.b, p.bias_sh = a.sbias.h, p.bias_sr = (int)a.sbias.r;
  p.heads = g.heads;
  p.nq = g.nq;
  p.nk = g.nk;
  p.nq_pad = (g.nq + kTile - 1) / kTile * kTile;
  p.diag = g.nk - g.nq;
  // an absent bound becomes one no key can reach
  p.wl = g.wl < 0 ? g.nq + g.nk : g.wl;
  p.wr = g.wr < 0 ? g.nq + g.nk : g.wr;
  p.nkb = (g.nk + kRowsPerBlock - 1) / kRowsPerBlock;
  p.nqb = (g.nq + kRowsPerBlock - 1) / kRowsPerBlock;
  p.scale = a.scale;
  p.c = a.scale * kLog2e;
  const long long bh = (long long)g.batch * g.heads;

  // with no query row, dK = dV = 0 and the statistics and dQ launches have
  // no work; with no key, dQ = 0 and dkdv has none
  const long long padded_rows = bh * p.nq_pad;
  if (padded_rows > 0) {
    const long long stat_blocks = (padded_rows * row_lanes<D>() + kThreads - 1) / kThreads;
    hipLaunchKernelGGL((row_stats_kernel<E, D>), dim3((unsigned)stat_blocks), dim3(kThreads), 0, a.stream,
                       (const bf16_t*)a.o, p.dout, a.lse, a.workspace, a.so, a.sdo, g.heads, g.nq, p.nq_pad,
                       padded_rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.nkb > 0) {
    // without a bias and for d <= 128 (whose triple-buffered tiles fit the
    // LDS), the kernel split by output between two waves per SIMD
    if constexpr (!BIAS && D <= 128)
      hipLaunchKernelGGL((dkdv_pp_kernel<E, D, MASK>), dim3((unsigned)(p.nkb * bh)), dim3(kPpThreads), 0, a.stream,
                         p);
    else
      hipLaunchKernelGGL((dkdv_kernel<E, D, MASK, BIAS>), dim3((unsigned)(p.nkb * bh)), dim3(kThreads), 0, a.stream,
                         p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.nqb > 0) {
    if constexpr (!BIAS && D >= 96 && D <= 128) {
      // two wave groups per work-group of 256 query rows (at d <= 64 the
      // one-group kernel fits more waves per SIMD and was faster)
      BwdParams pp = p;
      pp.nqb = (g.nq + kDqpRows - 1) / kDqpRows;
      const dim3 grid((unsigned)(pp.nqb * bh));
      if (MASK == kMaskNone && g.nk % kTile != 0)
        hipLaunchKernelGGL((dq_pp_kernel<E, D, MASK, MASK == kMaskNone>), grid, dim3(kDqpThreads), 0, a.stream, pp);
      else
        hipLaunchKernelGGL((dq_pp_kernel<E, D, MASK, false>), grid, dim3(kDqpThreads), 0, a.stream, pp);
    } else if (MASK == kMaskNone && g.nk % kTile != 0) {
      // without a band, a ragged last key tile needs the masking variant
      hipLaunchKernelGGL((dq_kernel<E, D, MASK, BIAS, MASK == kMaskNone>), dim3((unsigned)(p.nqb * bh)),
                         dim3(kThreads), 0, a.stream, p);
    } else {
      hipLaunchKernelGGL((dq_kernel<E, D, MASK, BIAS, false>), dim3((unsigned)(p.nqb * bh)), dim3(kThreads), 0,
                         a.stream, p);
    }
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename E, int D, bool BIAS>
hipError_t launch_m(const BwdArgs& a) {
  switch (a.g.mask_kind()) {
    case kMaskNone: return launch<E, D, kMaskNone, BIAS>(a);
    case kMaskUpper: return launch<E, D, kMaskUpper, BIAS>(a);
    default: return launch<E, D, kMaskBand, BIAS>(a);
  }
}

template <typename E, int D>
hipError_t launch_b(const BwdArgs& a) {
  return a.bias ? launch_m<E, D, true>(a) : launch_m<E, D, false>(a);
}

template <typename E>
hipError_t launch_d(const BwdArgs& a) {
  switch (a.g.d) {
    case 32: return launch_b<E, 32>(a);
    case 64: return launch_b<E, 64>(a);
    case 96: return launch_b<E, 96>(a);
    case 128: return launch_b<E, 128>(a);
    default: return launch_b<E, 256>(a);
  }
}

}  // namespace

size_t bwd_workspace_bytes(long long bh, int nq) {
  return (size_t)bh * (size_t)((nq + kTile - 1) / kTile * kTile) * 8;
}

hipError_t launch_bwd_mfma(const BwdArgs& a) {
  return a.dtype == kDtypeF16 ? launch_d<F16>(a) : launch_d<Bf16>(a);
}

}  // namespace fa
