// Forward attention, bf16 or fp16 in and out, fp32 accumulation, MFMA on gfx950.
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
//  * 8 waves x 32 query rows per work-group, one work-group per CU at d = 128
//    (two at d = 64), so every SIMD runs one wave of group A (waves 0-3) next
//    to one of group B (waves 4-7). K/V tiles hold 128 keys at d = 128 (64 at
//    d = 64): long phases amortise the two barriers per tile and give the
//    softmax more independent work.
//  * Ping-pong: each tile's work splits into a matrix phase (O += P_{j-1} V_{j-1}
//    for the previous tile, then S_j = K_j Q^T) and a softmax phase (max, exp,
//    sum of S_j). Group B runs one phase behind group A and a work-group
//    barrier separates phases, so on every SIMD one wave feeds the matrix core
//    while the other runs the softmax on the vector ALU.
//  * Both groups use K_j and V_{j-1} during iteration j, so the two tiles are
//    kept together as one set, double-buffered in LDS, and copied global ->
//    LDS with buffer_load ... lds (zero-fill past the end). The copies are
//    split between the groups: group A copies K_{j+1} at the start of its
//    matrix phase j (of its softmax phase j at d = 256, whose short phases
//    carry the copy's issue less well); group B copies V_{j+1} into set j's
//    buffer (set j + 2) at the end of its softmax phase j, once both groups
//    have read set j and once group A's K copy of the same phase has drained
//    (issued at the start of the phase, behind that copy, the V copy stalled
//    group B's softmax by about a third). Each copy has at least a whole
//    phase after its issue to land: the barriers wait only for LDS accesses
//    (lds_barrier), and each group waits for its own copy just before the
//    barrier that hands it over.
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
//  * Shapes and masks: queries and keys may differ in number (query i is
//    aligned with key i + nk - nq, so new queries attend over a cache of
//    earlier keys) and a band mask keeps, for each query, the keys from wl
//    before to wr after its aligned key (causal: wr = 0; a sliding window:
//    wl = w). A work-group visits only the K/V tiles its band touches; tiles
//    that straddle a band edge or the end of the keys mask dead scores to
//    -inf. A row that sees no key ends with l = 0: O = 0 and LSE = -inf.
//  * Tensors are addressed through per-tensor batch, head and row strides
//    (d contiguous), so views of other layouts need no copy.
//  * An optional fp32 bias is added to the scaled scores. Its kernels work in
//    log2 units from the start (y = c s + log2(e) bias, one FMA) instead of
//    raw score units, and each lane loads the bias of its query row, four
//    consecutive keys per 16-byte load, at the start of the matrix phase that
//    precedes the softmax phase using it (64-key tiles make room for it in
//    the registers), so the load latency hides behind the MFMAs.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlockM = 32 * kWaves;  // query rows per work-group

// 32-key blocks per K/V tile: 128 keys where the registers allow long
// phases, 64 at small d (two work-groups per CU share the registers) and
// with a bias (whose values for the tile are held in registers through the
// matrix phase), 32 at d = 256 (the O accumulators alone take half the
// registers)
template <int D, bool BIAS>
constexpr int key_blocks() {
  return D >= 256 ? 1 : (D >= 96 && !BIAS) ? 4 : 2;
}

// Whether a bias kernel reads its tile's bias at the start of the matrix
// phase (its latency then hides behind the MFMAs) rather than in the softmax
// phase that adds it; d = 256 has no registers to hold it that long.
template <int D, bool BIAS>
constexpr bool bias_ahead() {
  return BIAS && D < 256;
}

struct FwdParams {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  bf16_t* o;
  float* lse;
  const float* bias;
  long long q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh, bias_sb, bias_sh;  // batch / head strides (elements)
  int q_sr, k_sr, v_sr, o_sr, bias_sr;                                        // row strides (elements)
  int heads;
  int nq, nk;
  int diag;      // nk - nq: the key aligned with query 0
  int wl, wr;    // band (banded kernels only), both >= 0
  int nqb;       // query blocks per head
  int nblocks;   // work-groups in the grid
  float c;       // |scale| * log2(e)
  float scale_abs;
  float thr;     // lazy-rescale threshold in raw score units (kernels without bias)
  uint32_t qsign;  // 0x80008000 flips two bf16 signs at once when scale < 0
};

// Per-wave running state of 32 query rows (one per lane pair l, l ^ 32).
template <int D, int KB>
struct RowState {
  f32x16 acc[D / 32];  // O^T: register r of acc[db] holds d = 32 db + 8 (r / 4) + 4 hw + r % 4
  f32x16 s[KB];        // S^T of the current tile: register r of s[b] holds key 32 b + 8 (r / 4) + 4 hw + r % 4
  bf16x8 pb[2 * KB];   // P of the previous tile as bf16 B operands (pb[2 b + h] = s[b][8 h .. 8 h + 7])
  float m, l, mc;
};

// Scheduling groups (see __builtin_amdgcn_sched_group_barrier): instruction
// classes the compiler's scheduler must place in the given order.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// O += P_{j-1} V_{j-1}. The four output blocks are interleaved, so no MFMA
// waits on the accumulator of the one just before it.
template <typename E, int D, int KB>
__device__ __forceinline__ void pv_mfma(RowState<D, KB>& st, const bf16_t* vt, const TrRead<D>& vrd) {
#pragma unroll
  for (int t = 0; t < 2 * KB; ++t)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) st.acc[db] = E::mfma(vrd(vt, t, db), st.pb[t], st.acc[db]);
}

// Matrix phase of tile j: O += P_{j-1} V_{j-1}, then S_j = K_j Q^T.
// The LDS operand reads run ahead of the MFMAs: at every MFMA about four
// operands are already in flight, so the matrix core does not wait on LDS
// latency (the other wave on the SIMD is in its softmax phase and cannot
// cover it).
template <typename E, int D, int KB>
__device__ __forceinline__ void matrix_phase(RowState<D, KB>& st, const bf16_t* kt, const bf16_t* vt,
                                             const RowRead<D>& krd, const TrRead<D>& vrd,
                                             const bf16x8 (&qf)[D / 16]) {
  pv_mfma<E, D, KB>(st, vt, vrd);
  f32x16 s[KB];
#pragma unroll
  for (int b = 0; b < KB; ++b) s[b] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
    for (int b = 0; b < KB; ++b) s[b] = E::mfma(krd(kt, b, ks), qf[ks], s[b]);
#pragma unroll
  for (int b = 0; b < KB; ++b) {
    st.s[b] = s[b];
    fence_regs(st.s[b]);
  }
  // PV: (D / 32) (2 KB) MFMAs, two transposed reads each; S: KB (D / 16)
  // MFMAs, one read each. At d = 64 (128 registers per lane) and d = 256
  // (128 of the 256 registers hold O) four operands in flight push the phase
  // past the register budget, and the scheduler then drops the pattern
  // altogether (every MFMA waits for its own read); two fit.
  constexpr int kPv = D * KB / 16, kS = KB * D / 16, kAhead = (D == 64 || D == 256) ? 2 : 4;
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kAhead, 0);
#pragma unroll
  for (int i = 0; i < kPv - kAhead; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
  }
#pragma unroll
  for (int i = 0; i < kS; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
  }
#pragma unroll
  for (int i = 0; i < kAhead; ++i) __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
}

// Bias of keys kc .. kc + 3 of this lane's query row (zeros past the last key).
__device__ __forceinline__ f32x4 load_bias4(const float* brow, int kc, int nk) {
  f32x4 bv = f32x4{0.f, 0.f, 0.f, 0.f};
  if (kc + 3 < nk) {
    bv = *(const f32x4*)(brow + kc);
  } else {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      if (kc + rr < nk) bv[rr] = brow[kc + rr];
  }
  return bv;
}

// Maximum of N values as a tree of three-input maxima (v_max3_f32): each
// level turns groups of three into one, so the tree takes about N / 2
// instructions instead of N - 1, with independent instructions side by side.
template <int N>
__device__ __forceinline__ float max_tree(const float* x) {
  if constexpr (N == 1) {
    return x[0];
  } else if constexpr (N == 2) {
    return fmaxf(x[0], x[1]);
  } else {
    constexpr int M = (N + 2) / 3;
    float t[M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const int a = 3 * i;
      t[i] = a + 2 < N ? fmaxf(fmaxf(x[a], x[a + 1]), x[a + 2]) : a + 1 < N ? fmaxf(x[a], x[a + 1]) : x[a];
    }
    return max_tree<M>(t);
  }
}

// Sum of N values as a pairwise tree: independent adds side by side.
template <int N>
__device__ __forceinline__ float sum_tree(const float* x) {
  float t[N / 2];
#pragma unroll
  for (int i = 0; i < N / 2; ++i) t[i] = x[i] + x[i + N / 2];
#pragma unroll
  for (int w = N / 4; w >= 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) t[i] += t[i + w];
  return t[0];
}

// S^T of the wave's tile once more, as the matrix phase formed it but with the
// K rows read from global memory: by the time group B's softmax phase runs,
// group A may already be copying the next tile into the LDS buffer.
template <typename E, int D, int KB>
__device__ __forceinline__ void recompute_scores(float (&x)[16 * KB], const bf16_t* kh, int k_sr, int key0, int nk,
                                                 const bf16x8 (&qf)[D / 16], int lane) {
  const int hw = lane >> 5, col = lane & 31;
  f32x16 acc[KB];
#pragma unroll
  for (int b = 0; b < KB; ++b) acc[b] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      const int kr = key0 + 32 * b + col;
      u32x4 a = u32x4{0u, 0u, 0u, 0u};
      if (kr < nk) a = *(const u32x4*)(kh + (long long)kr * k_sr + 16 * ks + 8 * hw);
      acc[b] = E::mfma(__builtin_bit_cast(bf16x8, a), qf[ks], acc[b]);
      // a rare path: one load at a time, so it takes no registers beyond
      // what the rest of the kernel needs
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
  for (int b = 0; b < KB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) x[16 * b + r] = acc[b][r];
}

// Softmax phase for the tile whose scores are in st.s. With a bias the scores
// become y = c s + log2(e) bias (log2 units) first; `masked` tiles (band
// edges, ragged end) then set the scores of dead keys to -inf.
//
// Without a bias, once a row has a reference point the exponentials are taken
// against it straight away, and the reference is checked afterwards, on the
// sum of the lane's p: a sum of at most kFastSumBound bounds every p by it.
// fp32 has ample room for p that large (O / l and m + ln l do not depend on
// the reference point; the max test below moves it at a factor 2^8 only to
// move it rarely). Only a larger sum (a score far above the reference, or an
// overflow) has the scores formed again and the tile run through the max
// path. That saves the max tree on nearly every tile. The bound is set well
// above 2^8 because a row's first reference can come from a tile with only a
// few live keys (a band edge), and ordinary later tiles then sum to a few
// hundred.
constexpr float kFastSumBound = 65536.f;
template <typename E, int D, int KB, int MASK, bool BIAS>
__device__ __forceinline__ void softmax_phase(RowState<D, KB>& st, const FwdParams& p, int key0, int qi, int lane,
                                              bool masked, const float* brow, const f32x4 (&bpre)[4 * KB],
                                              const bf16_t* kh, const bf16x8 (&qf)[D / 16]) {
  constexpr int kN = 16 * KB;  // scores per lane
  const int hw = lane >> 5;
  // scale of the working units: raw scores without bias, log2 units with one
  const float cu = BIAS ? 1.f : p.c;
  const float thr = BIAS ? 8.f : p.thr;
  float x[kN];
#pragma unroll
  for (int b = 0; b < KB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) x[16 * b + r] = st.s[b][r];
  if constexpr (BIAS) {
#pragma unroll
    for (int b = 0; b < KB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 bv;
        if constexpr (bias_ahead<D, BIAS>())
          bv = bpre[4 * b + g];
        else
          bv = load_bias4(brow, key0 + 32 * b + 8 * g + 4 * hw, p.nk);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) x[16 * b + 4 * g + rr] = fmaf(x[16 * b + 4 * g + rr], p.c, kLog2e * bv[rr]);
        // (loads here at d = 256 only) one key block's loads at a time: the
        // bias must not take more registers beside the scores
        if (g == 3) __builtin_amdgcn_sched_barrier(0);
      }
  }
  auto mask_dead = [&](float (&y)[kN]) {
    // live keys of this row: [lo, hi]
    const int hi = MASK != kMaskNone ? min(qi + p.diag + p.wr, p.nk - 1) : p.nk - 1;
    const int lo = MASK == kMaskBand ? qi + p.diag - p.wl : 0;
    const int k0 = key0 + 4 * hw;
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int b = i >> 4, r = i & 15;
      const int kr = k0 + 32 * b + 8 * (r >> 2) + (r & 3);
      y[i] = (kr > hi || (MASK == kMaskBand && kr < lo)) ? -INFINITY : y[i];
    }
  };
  if (masked) mask_dead(x);

  // moves the reference point to the tile's max where that grows by more
  // than the threshold, rescaling O and l by the same factor
  auto rebase = [&]() {
    // Running max: in-lane as a tree, then across the half-wave pair. The
    // softmax wave has its SIMD's vector ALU to itself during this phase, so
    // only independent instructions hide each other's latency.
    const float mx = pair_max(max_tree<kN>(x));
    if (wave_any(!(mx <= st.m + thr))) {
      const float mnew = fmaxf(st.m, mx);
      const float ms = (mnew == -INFINITY) ? 0.f : mnew * cu;
      const float alpha = (st.m == -INFINITY) ? 0.f : fast_exp2(st.m * cu - ms);
      st.l *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) st.acc[db] *= alpha;
      st.m = mnew;
      st.mc = ms;
    }
  };
  // p = exp2(c s - c m) and the lane's sum of p; c > 0, so dead keys
  // (s = -inf) give exp2(-inf) = 0. FMAs, then exponentials, then a sum tree:
  // independent instructions back to back instead of FMA -> exp -> add chains.
  auto exponentials = [&]() {
    const float nmc = -st.mc;
#pragma unroll
    for (int i = 0; i < kN; ++i) x[i] = fmaf(x[i], cu, nmc);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kN; ++i) x[i] = fast_exp2(x[i]);
    __builtin_amdgcn_sched_barrier(0);
    return sum_tree<kN>(x);
  };

  float ts;
  if constexpr (BIAS) {
    rebase();
    ts = exponentials();
  } else {
    // a row without a reference point yet (no live key so far) takes the
    // tile's max; its O and l are still zero, so nothing is rescaled
    if (wave_any(st.m == -INFINITY)) {
      const float mx = pair_max(max_tree<kN>(x));
      if (st.m == -INFINITY) {
        st.m = mx;
        st.mc = (mx == -INFINITY) ? 0.f : mx * cu;
      }
    }
    ts = exponentials();
    if (wave_any(!(ts <= kFastSumBound))) {
      // rare: a score far above the reference point (or an overflow). The
      // exponentials replaced the scores, so form them again.
      recompute_scores<E, D, KB>(x, kh, p.k_sr, key0, p.nk, qf, lane);
      if (masked) mask_dead(x);
      rebase();
      ts = exponentials();
    }
  }
  st.l += ts;
#pragma unroll
  for (int t = 0; t < 2 * KB; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) st.pb[t][e] = E::cvt(x[8 * t + e]);
#pragma unroll
  for (int t = 0; t < 2 * KB; ++t) fence_regs(st.pb[t]);
  fence_regs(st.l);
}

// One iteration j < n_tiles of the main loop (keys key_base + j * kBlockN
// onwards): matrix(j) on set j (K_j in `kt`, V_{j-1} in `vt`), a barrier,
// softmax(j), a barrier, with the copies placed as described at the top (K_{j+1}
// goes to `kn`; set j + 1's V_j was copied by group B one iteration earlier).
// The buffers are fixed per call (the loop is unrolled by two) so the compiler
// can see that reading set j never depends on a copy into the other set. Every
// wave runs every tile of its work-group: a tile wholly outside a wave's band
// has all scores at -inf, so its p are 0 and it changes nothing.
// Two work-groups share a CU at d = 64, and the issue arbiter favours the
// older one's waves: one would finish in about two thirds of the other's
// time and leave the CU half idle. Each wave lowers its priority as its
// work-group gets through its tiles, so the one behind wins arbitration
// (priority 3, 2, 1, 0 over the four quarters of its tiles). At d = 32 the
// dispatcher's backfilling over many rounds already evens this out.
template <int D, int MASK>
__device__ __forceinline__ void progress_priority(int j, int n_tiles) {
  if constexpr (D == 64 && MASK == kMaskNone) {
    if (j == 0) {
      __builtin_amdgcn_s_setprio(3);
    } else if (4 * j == n_tiles || 4 * j == n_tiles + 1 || 4 * j == n_tiles + 2 || 4 * j == n_tiles + 3) {
      __builtin_amdgcn_s_setprio(2);
    } else if (2 * j == n_tiles || 2 * j == n_tiles + 1) {
      __builtin_amdgcn_s_setprio(1);
    } else if (4 * j == 3 * n_tiles || 4 * j == 3 * n_tiles + 1 || 4 * j == 3 * n_tiles + 2 || 4 * j == 3 * n_tiles + 3) {
      __builtin_amdgcn_s_setprio(0);
    }
  }
}

template <typename E, int D, int KB, int MASK, bool BIAS, bool FULL = true>
__device__ __forceinline__ void fwd_iteration(int j, int n_tiles, int key_base, bool group_b, const bf16_t* kt,
                                              bf16_t* vt,
                                              bf16_t* kn,
                                              const TileDma<32 * KB, D, kThreads / 2>& dma,
                                              __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                              const RowRead<D>& krd, const TrRead<D>& vrd,
                                              const bf16x8 (&qf)[D / 16], RowState<D, KB>& st, const FwdParams& p,
                                              int wq0, int qi, int lane, const float* brow, const bf16_t* kh) {
  constexpr int kBlockN = 32 * KB;
  const int key0 = key_base + j * kBlockN;
  progress_priority<D, MASK>(j, n_tiles);
  // the bias of this tile, for the softmax phase after the matrix phase: read
  // now, so its latency hides behind the matrix phase (and ahead of the tile
  // copy, so waiting for it never waits for the copy)
  f32x4 bpre[4 * KB];
  if constexpr (FULL && bias_ahead<D, BIAS>()) {
    const int hw = lane >> 5;
#pragma unroll
    for (int b = 0; b < KB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) bpre[4 * b + g] = load_bias4(brow, key0 + 32 * b + 8 * g + 4 * hw, p.nk);
  }
  // group A copies K_{j+1} into set j + 1 during its matrix phase (softmax
  // phase at d = 256) and waits for it at the end of its softmax phase; group
  // B copies V_{j+1} into set j's buffer (which becomes set j + 2) at the end
  // of its softmax phase, once both groups have read set j, and waits for it
  // at the end of its next matrix phase.
  // At d = 256 (32-key tiles, short phases) group A issues the copy at the
  // start of its softmax phase instead, where it weighs less on the critical
  // matrix phase; the copy then has one phase to land instead of two. That
  // was 2 % faster at d = 256 and 1-3 % slower at d = 96 and 128.
  constexpr bool kLateK = D >= 256;
  if (!kLateK && !group_b && j + 1 < n_tiles) dma.issue(krs, kn, key0 + kBlockN, 2u * p.k_sr);
  if constexpr (FULL) matrix_phase<E, D, KB>(st, kt, vt, krd, vrd, qf);
  if (group_b) wait_vmem();
  lds_barrier();
  if (kLateK && !group_b && j + 1 < n_tiles) dma.issue(krs, kn, key0 + kBlockN, 2u * p.k_sr);
  // the wave's rows are wq0 .. wq0 + 31: the last has the highest lower
  // bound, the first the lowest upper bound
  const bool masked = (key0 + kBlockN > p.nk) ||
                      (MASK != kMaskNone && key0 + kBlockN - 1 > wq0 + p.diag + p.wr) ||
                      (MASK == kMaskBand && key0 < wq0 + 31 + p.diag - p.wl);
  if constexpr (FULL) softmax_phase<E, D, KB, MASK, BIAS>(st, p, key0, qi, lane, masked, brow, bpre, kh, qf);
  if (group_b && j + 1 < n_tiles) dma.issue(vrs, vt, key0 + kBlockN, 2u * p.v_sr);
  if (!group_b) wait_vmem();
  lds_barrier();
}

// d <= 64 needs few enough registers (at most 128 per lane) for two
// work-groups per CU; larger d runs one.
template <int D>
constexpr int fwd_blocks_per_cu() {
  return D <= 64 ? 2 : 1;
}

// The waves each SIMD must hold (the second __launch_bounds__ argument, which
// caps the registers per lane at 512 / that many): a work-group's 8 waves
// spread over the 4 SIMDs of a CU. Kernels with a bias keep their tile's bias
// in registers and run one work-group per CU.
template <int D, bool BIAS>
constexpr int fwd_waves_per_simd() {
  return (BIAS ? 1 : fwd_blocks_per_cu<D>()) * kWaves / 4;
}

template <typename E, int D, int MASK, bool BIAS>
__global__ __launch_bounds__(kThreads, (fwd_waves_per_simd<D, BIAS>())) void fwd_kernel(FwdParams p) {
  constexpr bool BAND = MASK != kMaskNone;
  constexpr int KB = key_blocks<D, BIAS>();
  constexpr int kBlockN = 32 * KB;  // keys per tile
  constexpr int P = lds_pitch<D>();
  // Two sets of (K tile, V tile), declared as separate objects so the compiler
  // can see that reading one set never depends on the copy filling the other.
  __shared__ __attribute__((aligned(1024))) bf16_t k_lds0[kBlockN * P];
  __shared__ __attribute__((aligned(1024))) bf16_t k_lds1[kBlockN * P];
  __shared__ __attribute__((aligned(1024))) bf16_t v_lds0[kBlockN * P];
  __shared__ __attribute__((aligned(1024))) bf16_t v_lds1[kBlockN * P];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool group_b = wave >= kWaves / 2;
  const int hw = lane >> 5;
  const int col = lane & 31;
  const int nq = p.nq, nk = p.nk;

  const int logical = xcd_logical_block(blockIdx.x, p.nblocks);
  const int head = logical / p.nqb;  // b * heads + h
  int qblk = logical - head * p.nqb;
  if (BAND) qblk = p.nqb - 1 - qblk;  // longest rows first under a causal band
  const int hb = head / p.heads, hh = head - hb * p.heads;
  const bf16_t* qh = p.q + hb * p.q_sb + hh * p.q_sh;
  const bf16_t* kh = p.k + hb * p.k_sb + hh * p.k_sh;
  const bf16_t* vh = p.v + hb * p.v_sb + hh * p.v_sh;
  const int q_row0 = qblk * kBlockM;
  const int wq0 = q_row0 + wave * 32;
  const int qi = wq0 + col;
  // bias row of this lane's query (rows past nq read the last row; unused)
  const float* brow = BIAS ? p.bias + hb * p.bias_sb + hh * p.bias_sh + (long long)min(qi, nq - 1) * p.bias_sr : nullptr;

  // K/V tiles of this work-group's band: [key_base, key_base + n_tiles * kBlockN)
  const int q_last = min(nq, q_row0 + kBlockM) - 1;
  int key_base = 0, n_tiles = (nk + kBlockN - 1) / kBlockN;
  if (BAND) {
    const int k_lo = max(0, q_row0 + p.diag - p.wl);
    const int k_hi = min(nk - 1, q_last + p.diag + p.wr);
    key_base = k_lo / kBlockN * kBlockN;
    n_tiles = k_hi < k_lo ? 0 : (k_hi - key_base) / kBlockN + 1;
  }

  // K/V tiles stream straight into LDS. Group A copies every tile (see the
  // loop below); start the first K tile before loading Q.
  const __amdgpu_buffer_rsrc_t krs = rows_rsrc<D>(kh, nk, 2u * p.k_sr);
  const __amdgpu_buffer_rsrc_t vrs = rows_rsrc<D>(vh, nk, 2u * p.v_sr);
  TileDma<kBlockN, D, kThreads / 2> dma;
  dma.init(wave & (kWaves / 2 - 1), lane);
  RowRead<D> krd;
  krd.init(lane);
  TrRead<D> vrd;
  vrd.init(lane);
  if (!group_b) dma.issue(krs, k_lds0, key_base, 2u * p.k_sr);
  if (group_b && n_tiles > 0) dma.issue(vrs, v_lds1, key_base, 2u * p.v_sr);  // V_0 of set 1

  bf16x8 qf[D / 16];
  {
    const bf16_t* qrow = qh + (long long)qi * p.q_sr + 8 * hw;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 x = u32x4{0u, 0u, 0u, 0u};
      if (qi < nq) x = *(const u32x4*)(qrow + 16 * ks);
      qf[ks] = __builtin_bit_cast(bf16x8, x ^ p.qsign);
    }
  }

  RowState<D, KB> st;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) st.acc[db] = f32x16{};
#pragma unroll
  for (int t = 0; t < 2 * KB; ++t) st.pb[t] = bf16x8{};
  st.m = -INFINITY;
  st.l = 0.f;
  st.mc = 0.f;
  // the first matrix phase multiplies P = 0 by the V buffer of set 0: zero it
  for (int i = tid; i < kBlockN * P / 8; i += kThreads) ((FA_LDS u32x4*)(FA_LDS bf16_t*)v_lds0)[i] = u32x4{};

  wait_vmem();
  lds_barrier();
  // Iteration j uses LDS set j % 2 = {K_j, V_{j-1}}: matrix(j) = O += P_{j-1}
  // V_{j-1} and S_j = K_j Q^T, then softmax(j). Both groups run this same
  // loop, group B one phase (one barrier) behind group A, so while one group
  // is in its matrix phase the other is in its softmax phase. Group A copies
  // set j + 1 during its iteration j (phases 2j and 2j + 1); set j is last
  // read by group B in phase 2j + 1, and set j + 1 is first read by group A in
  // phase 2j + 2.
  if (group_b) lds_barrier();
  // Tiles run in pairs (set 0, then set 1). At d = 64 and 256, whose
  // registers are tightest, an odd last tile runs the first half of a pair
  // inside the loop, and the epilogue forms its lane values again: no tail
  // copy of the iteration follows the loop, and nothing computed before the
  // loop has to survive it (that had cost 1-6 spilled registers and, at
  // d = 256, most of the matrix phase's operand read-ahead). Elsewhere the
  // odd tile runs after the loop, which measured slightly faster.
  constexpr bool kCompact = D == 64 || D == 256;
  int j = 0;
  // (band kernels: the pending P V of the last live tile is done in the tile
  // after it, or after the loop when that is the last tile)
  bool last_pv = true;
  if constexpr (MASK == kMaskBand && D <= 128) {
    // Each wave runs the tiles its own rows see, [ja, je), in full; the tiles
    // before and after them only issue their share of the copies and take
    // part in the barriers. A tile none of its rows sees would change
    // nothing (all its scores -inf); leaving its MFMAs and exponentials out
    // saves energy, which the power-limited clock turns into time (d = 256,
    // which has no registers for the extra loop copies, runs every tile). je - 1 is
    // the tile after the last live one: its matrix phase adds the last live
    // tile's P V, and its own scores are all masked.
    const int klo = max(wq0 + p.diag - p.wl, 0), khi = min(wq0 + 31 + p.diag + p.wr, nk - 1);
    int ja = n_tiles, je = n_tiles;
    if (klo <= khi && wq0 < nq) {
      ja = klo < key_base ? 0 : min((klo - key_base) / kBlockN, n_tiles);
      je = khi < key_base ? 0 : min((khi - key_base) / kBlockN + 2, n_tiles);
      ja = __builtin_amdgcn_readfirstlane(ja);
      je = __builtin_amdgcn_readfirstlane(max(je, ja));
    }
    last_pv = je == n_tiles && ja < je;
    // tiles [a, b) of one kind, each on LDS set j % 2
    auto run = [&](auto full, int a, int b) __attribute__((always_inline)) {
      constexpr bool F = decltype(full)::value;
      int i = a;
      if (i < b && (i & 1)) {
        fwd_iteration<E, D, KB, MASK, BIAS, F>(i, n_tiles, key_base, group_b, k_lds1, v_lds1, k_lds0, dma, krs, vrs,
                                              krd, vrd, qf, st, p, wq0, qi, lane, brow, kh);
        ++i;
      }
      for (; i + 1 < b; i += 2) {
        fwd_iteration<E, D, KB, MASK, BIAS, F>(i, n_tiles, key_base, group_b, k_lds0, v_lds0, k_lds1, dma, krs, vrs,
                                              krd, vrd, qf, st, p, wq0, qi, lane, brow, kh);
        fwd_iteration<E, D, KB, MASK, BIAS, F>(i + 1, n_tiles, key_base, group_b, k_lds1, v_lds1, k_lds0, dma, krs,
                                              vrs, krd, vrd, qf, st, p, wq0, qi, lane, brow, kh);
      }
      if (i < b)
        fwd_iteration<E, D, KB, MASK, BIAS, F>(i, n_tiles, key_base, group_b, k_lds0, v_lds0, k_lds1, dma, krs, vrs,
                                              krd, vrd, qf, st, p, wq0, qi, lane, brow, kh);
    };
    run(std::false_type{}, 0, ja);
    run(std::true_type{}, ja, je);
    run(std::false_type{}, je, n_tiles);
  } else if constexpr (kCompact) {
    for (; j < n_tiles; j += 2) {
      fwd_iteration<E, D, KB, MASK, BIAS>(j, n_tiles, key_base, group_b, k_lds0, v_lds0, k_lds1, dma, krs, vrs, krd,
                                    vrd, qf, st, p, wq0, qi, lane, brow, kh);
      if (j + 1 < n_tiles)
        fwd_iteration<E, D, KB, MASK, BIAS>(j + 1, n_tiles, key_base, group_b, k_lds1, v_lds1, k_lds0, dma, krs,
                                      vrs, krd, vrd, qf, st, p, wq0, qi, lane, brow, kh);
    }
  } else {
    for (; j + 1 < n_tiles; j += 2) {
      fwd_iteration<E, D, KB, MASK, BIAS>(j, n_tiles, key_base, group_b, k_lds0, v_lds0, k_lds1, dma, krs, vrs, krd,
                                    vrd, qf, st, p, wq0, qi, lane, brow, kh);
      fwd_iteration<E, D, KB, MASK, BIAS>(j + 1, n_tiles, key_base, group_b, k_lds1, v_lds1, k_lds0, dma, krs, vrs,
                                    krd, vrd, qf, st, p, wq0, qi, lane, brow, kh);
    }
    if (j < n_tiles)
      fwd_iteration<E, D, KB, MASK, BIAS>(j, n_tiles, key_base, group_b, k_lds0, v_lds0, k_lds1, dma, krs, vrs, krd,
                                    vrd, qf, st, p, wq0, qi, lane, brow, kh);
  }
  // last tile: O += P V of set n_tiles (no copy is in flight any more)
  if (last_pv) pv_mfma<E, D, KB>(st, (n_tiles & 1) ? v_lds1 : v_lds0, vrd);
  if (!group_b) lds_barrier();

  // epilogue: O = acc / l, LSE = m * |scale| + ln l (-inf for a row with no key)
  const float lt = pair_sum(st.l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  // (kCompact: the row and half-wave are formed again from the thread index,
  // laundered so the compiler cannot carry the values from before the loop)
  int qi_e = qi, hw_e = hw;
  if constexpr (kCompact) {
    int te = tid;
    asm volatile("" : "+v"(te));
    qi_e = q_row0 + (te >> 6) * 32 + (te & 31);
    hw_e = (te >> 5) & 1;
  }
  {
    const int qi = qi_e, hw = hw_e;
  if (qi < nq) {
    bf16_t* orow = p.o + hb * p.o_sb + hh * p.o_sh + (long long)qi * p.o_sr;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 w;
        w.x = pack2<E>(st.acc[db][4 * g] * inv, st.acc[db][4 * g + 1] * inv);
        w.y = pack2<E>(st.acc[db][4 * g + 2] * inv, st.acc[db][4 * g + 3] * inv);
        *(uint2*)(orow + db * 32 + 8 * g + 4 * hw) = w;
      }
    // the reference point m is in raw score units (scale |scale|) or, with a
    // bias, in log2 units (scale ln 2)
    const float unit = BIAS ? kLn2 : p.scale_abs;
    if (hw == 0) p.lse[(long long)head * nq + qi] = lt > 0.f ? st.m * unit + __logf(lt) : -INFINITY;
  }
  }
}

#define FA_FWD_INSTANCES_B(E, D, B)                                   \
  template __global__ void fwd_kernel<E, D, kMaskNone, B>(FwdParams);  \
  template __global__ void fwd_kernel<E, D, kMaskUpper, B>(FwdParams); \
  template __global__ void fwd_kernel<E, D, kMaskBand, B>(FwdParams);
#define FA_FWD_INSTANCES(E, D)      \
  FA_FWD_INSTANCES_B(E, D, false) \
  FA_FWD_INSTANCES_B(E, D, true)
#define FA_FWD_INSTANCES_D(E) \
  FA_FWD_INSTANCES(E, 32)     \
  FA_FWD_INSTANCES(E, 64)     \
  FA_FWD_INSTANCES(E, 96)     \
  FA_FWD_INSTANCES(E, 128)    \
  FA_FWD_INSTANCES(E, 256)
FA_FWD_INSTANCES_D(Bf16)
FA_FWD_INSTANCES_D(F16)
#undef FA_FWD_INSTANCES_D
#undef FA_FWD_INSTANCES
#undef FA_FWD_INSTANCES_B

template <typename E, int D, int MASK, bool BIAS>
hipError_t launch(const FwdArgs& a) {
  FwdParams p;
  p.q = (const bf16_t*)a.q;
  p.k = (const bf16_t*)a.k;
  p.v = (const bf16_t*)a.v;
  p.o = (bf16_t*)a.o;
  p.lse = a.lse;
  p.q_sb = a.sq.b, p.q_sh = a.sq.h, p.q_sr = (int)a.sq.r;
  p.k_sb = a.sk.b, p.k_sh = a.sk.h, p.k_sr = (int)a.sk.r;
  p.v_sb = a.sv.b, p.v_sh = a.sv.h, p.v_sr = (int)a.sv.r;
  p.o_sb = a.so.b, p.o_sh = a.so.h, p.o_sr = (int)a.so.r;
  p.bias = a.bias;
  p.bias_sb = a.sbias.b, p.bias_sh = a.sbias.h, p.bias_sr = (int)a.sbias.r;
  p.heads = a.g.heads;
  p.nq = a.g.nq;
  p.nk = a.g.nk;
  p.diag = a.g.nk - a.g.nq;
  // an absent bound becomes one no key can reach
  p.wl = a.g.wl < 0 ? a.g.nq + a.g.nk : a.g.wl;
  p.wr = a.g.wr < 0 ? a.g.nq + a.g.nk : a.g.wr;
  p.nqb = (a.g.nq + kBlockM - 1) / kBlockM;
  p.nblocks = p.nqb * a.g.batch * a.g.heads;
  p.scale_abs = fabsf(a.scale);
  // c is kept strictly positive: with scale = 0 every exp2(c (s - m)) still
  // rounds to exactly 1 (uniform weights) while exp2(c * -inf) stays 0 for
  // masked keys. LSE uses |scale| itself.
  p.c = fmaxf(p.scale_abs * kLog2e, 1e-30f);
  p.thr = p.scale_abs > 0.f ? 8.f / p.c : 3.0e38f;
  p.qsign = a.scale < 0.f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((fwd_kernel<E, D, MASK, BIAS>), dim3(p.nblocks), dim3(kThreads), 0, a.stream, p);
  return hipGetLastError();
}

template <typename E, int D, bool BIAS>
hipError_t launch_m(const FwdArgs& a) {
  switch (a.g.mask_kind()) {
    case kMaskNone: return launch<E, D, kMaskNone, BIAS>(a);
    case kMaskUpper: return launch<E, D, kMaskUpper, BIAS>(a);
    default: return launch<E, D, kMaskBand, BIAS>(a);
  }
}

template <typename E, int D>
hipError_t launch_b(const FwdArgs& a) {
  return a.bias ? launch_m<E, D, true>(a) : launch_m<E, D, false>(a);
}

template <typename E>
hipError_t launch_d(const FwdArgs& a) {
  switch (a.g.d) {
    case 32: return launch_b<E, 32>(a);
    case 64: return launch_b<E, 64>(a);
    case 96: return launch_b<E, 96>(a);
    case 128: return launch_b<E, 128>(a);
    default: return launch_b<E, 256>(a);
  }
}

}  // namespace

hipError_t launch_fwd_mfma(const FwdArgs& a) {
  return a.dtype == kDtypeF16 ? launch_d<F16>(a) : launch_d<Bf16>(a);
}

}  // namespace fa
