// Forward attention, bf16 in / bf16 out, fp32 accumulation, MFMA on gfx950.
//
// Method ('FlashAttention', josueisai.com, section on the softmax trick; the
// kerneldigest.dev glossary entry): a work-group owns a block of query rows of
// one head, streams the K/V tiles of that head through LDS, forms each score
// tile on the matrix cores, folds it into the output with a running row max m
// and running row sum l (rescaling the partial output when m grows), and
// writes only O and LSE = m + ln l. No score or probability tile leaves the
// chip.
//
// Mapping to the hardware:
//  * 4 waves x 32 query rows per work-group; K/V tiles of 64 keys,
//    double-buffered in LDS, one barrier per tile.
//  * Scores are computed transposed, S^T = K Q^T, with Q (the B operand) kept
//    in registers. Each lane then holds one query's scores for 32 keys, so the
//    row max and row sum are in-lane reductions plus one exchange across the
//    two half-waves, and the rescale factor is a per-lane scalar.
//  * O^T = V^T P^T: P leaves the score accumulators as bf16 B operands without
//    any data movement, because its keys come out of the accumulators in an
//    order that the transposed LDS read of V (ds_read_b64_tr_b16) reproduces.
//  * Softmax in base 2: exp(scale*s - scale*m) = exp2(c*s - c*m), c = scale *
//    log2(e), one FMA per score. A negative scale flips the sign bit of Q in
//    registers (exact) so c >= 0 and the running max stays a max.
//  * The reference point m is only moved when a row's max grows by more than
//    8 / c (a factor 2^8 in the exponentials); otherwise the stale m is kept.
//    O / l and m + ln l do not depend on the reference point, so the result is
//    the same up to rounding while most tiles skip the O rescale entirely.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlockM = 32 * kWaves;  // query rows per work-group
constexpr int kBlockN = 64;           // keys per tile

struct FwdParams {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  bf16_t* o;
  float* lse;
  int n;
  int nqb;       // query blocks per head
  int nblocks;   // work-groups in the grid
  float c;       // |scale| * log2(e)
  float scale_abs;
  float thr;     // lazy-rescale threshold in raw score units
  uint32_t qsign;  // 0x80008000 flips two bf16 signs at once when scale < 0
};

template <int D, bool CAUSAL, bool MASKED>
__device__ __forceinline__ void fwd_tile(const bf16_t* kt, const bf16_t* vt, const bf16x8 (&qf)[D / 16],
                                         f32x16 (&acc)[D / 32], float& m, float& l, float& mc,
                                         const FwdParams& p, int key0, int qi, int lane) {
  const int hw = lane >> 5;
  const int col = lane & 31;

  // S^T for keys [key0, key0 + 64) x this wave's 32 queries
  f32x16 s0 = {}, s1 = {};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const bf16x8 a0 = lds_row8<D>(kt, col, 2 * ks + hw);
    const bf16x8 a1 = lds_row8<D>(kt, col + 32, 2 * ks + hw);
    s0 = mfma32(a0, qf[ks], s0);
    s1 = mfma32(a1, qf[ks], s1);
  }
  float sv[32];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    sv[i] = s0[i];
    sv[16 + i] = s1[i];
  }
  if constexpr (MASKED) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int key = key0 + (i >> 4) * 32 + 8 * ((i & 15) >> 2) + 4 * hw + (i & 3);
      const bool dead = key >= p.n || (CAUSAL && key > qi);
      sv[i] = dead ? -INFINITY : sv[i];
    }
  }
  // running max: in-lane over 32 keys, then across the half-wave pair
  float mx = sv[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) mx = fmaxf(mx, sv[i]);
  mx = pair_max(mx);

  const bool need = !(mx <= m + p.thr);
  if (wave_any(need)) {
    const float mnew = fmaxf(m, mx);
    const float ms = (mnew == -INFINITY) ? 0.f : mnew * p.c;
    const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m * p.c - ms);
    l *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    m = mnew;
    mc = ms;
  }

  float rs = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float e = fast_exp2(fmaf(sv[i], p.c, -mc));
    if constexpr (MASKED) e = (sv[i] == -INFINITY) ? 0.f : e;
    sv[i] = e;
    rs += e;
  }
  l += rs;

  bf16x8 pb[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) pb[t] = pack_bf16x8(&sv[(t >> 1) * 16 + 8 * (t & 1)]);

#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[db] = mfma32(lds_tr8<D>(vt, 16 * t, 32 * db, lane), pb[t], acc[db]);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(16))) bf16_t k_lds[2][kBlockN * D];
  __shared__ __attribute__((aligned(16))) bf16_t v_lds[2][kBlockN * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hw = lane >> 5;
  const int col = lane & 31;
  const int n = p.n;

  const int logical = xcd_logical_block(blockIdx.x, p.nblocks);
  const int head = logical / p.nqb;
  int qblk = logical - head * p.nqb;
  if (CAUSAL) qblk = p.nqb - 1 - qblk;  // longest rows first
  const size_t head_off = (size_t)head * n * D;
  const int q_row0 = qblk * kBlockM;
  const int wq0 = q_row0 + wave * 32;
  const int qi = wq0 + col;

  bf16x8 qf[D / 16];
  {
    const bf16_t* qrow = p.q + head_off + (size_t)qi * D + 8 * hw;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (qi < n) x = *(const uint4*)(qrow + 16 * ks);
      x.x ^= p.qsign;
      x.y ^= p.qsign;
      x.z ^= p.qsign;
      x.w ^= p.qsign;
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  const int q_last = min(n, q_row0 + kBlockM) - 1;
  const int n_tiles = CAUSAL ? (q_last / kBlockN + 1) : (n + kBlockN - 1) / kBlockN;
  const int w_last = min(n - 1, wq0 + 31);
  const bool wave_has_rows = wq0 < n;

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  float m = -INFINITY, l = 0.f, mc = 0.f;

  const bf16_t* kbase = p.k + head_off;
  const bf16_t* vbase = p.v + head_off;
  TileCopy<kBlockN, D, kThreads> kc, vc;
  kc.load(kbase, n, tid);
  vc.load(vbase, n, tid);
  kc.store(k_lds[0], tid);
  vc.store(v_lds[0], tid);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    const int key0 = j * kBlockN;
    const bool more = j + 1 < n_tiles;
    if (more) {
      kc.load(kbase + (size_t)(key0 + kBlockN) * D, n - key0 - kBlockN, tid);
      vc.load(vbase + (size_t)(key0 + kBlockN) * D, n - key0 - kBlockN, tid);
    }
    const bool active = wave_has_rows && (!CAUSAL || key0 <= w_last);
    if (active) {
      const bool masked = (key0 + kBlockN > n) || (CAUSAL && key0 + kBlockN - 1 > wq0);
      if (masked)
        fwd_tile<D, CAUSAL, true>(k_lds[buf], v_lds[buf], qf, acc, m, l, mc, p, key0, qi, lane);
      else
        fwd_tile<D, CAUSAL, false>(k_lds[buf], v_lds[buf], qf, acc, m, l, mc, p, key0, qi, lane);
    }
    if (more) {
      kc.store(k_lds[buf ^ 1], tid);
      vc.store(v_lds[buf ^ 1], tid);
    }
    __syncthreads();
  }

  // epilogue: O = acc / l, LSE = m * |scale| + ln l
  const float lt = pair_sum(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qi < n) {
    bf16_t* orow = p.o + head_off + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 w;
        w.x = pack_bf16x2(acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv);
        w.y = pack_bf16x2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv);
        *(uint2*)(orow + db * 32 + 8 * g + 4 * hw) = w;
      }
    if (hw == 0) p.lse[(size_t)head * n + qi] = lt > 0.f ? m * p.scale_abs + __logf(lt) : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a) {
  FwdParams p;
  p.q = (const bf16_t*)a.q;
  p.k = (const bf16_t*)a.k;
  p.v = (const bf16_t*)a.v;
  p.o = (bf16_t*)a.o;
  p.lse = a.lse;
  p.n = a.n;
  p.nqb = (a.n + kBlockM - 1) / kBlockM;
  p.nblocks = p.nqb * a.bh;
  p.scale_abs = fabsf(a.scale);
  p.c = p.scale_abs * kLog2e;
  p.thr = p.c > 0.f ? 8.f / p.c : 3.0e38f;
  p.qsign = a.scale < 0.f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3(p.nblocks), dim3(kThreads), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  if (a.d == 64) return a.causal ? launch<64, true>(a) : launch<64, false>(a);
  return a.causal ? launch<128, true>(a) : launch<128, false>(a);
}

}  // namespace fa
