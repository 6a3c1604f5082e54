// Device-side building blocks shared by the gfx950 attention kernels.
//
// Lane layouts used throughout (wave64, checked on gfx950 hardware):
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     A: lane l holds A[l % 32][8 * (l / 32) + e], e = 0..7
//     B: lane l holds B[8 * (l / 32) + e][l % 32]
//     D: lane l, register r holds D[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32]
//   ds_read_b64_tr_b16 (per group of 16 lanes): lane i receives element i % 4
//     of the 8 bytes addressed by lane 4 * j + i / 4, for j = 0..3.
//   v_permlane32_swap(x, x): r[1] of lane l < 32 holds x of lane l + 32 and
//     r[0] of lane l >= 32 holds x of lane l - 32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // bfloat16 storage in global memory

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Element types of the 16-bit paths. Tiles and MFMA operands travel as
// 16-byte vectors typed bf16x8 whatever the element type (loads, LDS and
// lane exchanges only move bits); the matrix instruction and the conversions
// to and from fp32 are the only places where the type matters.
struct Bf16 {
  __device__ __forceinline__ static f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) { return mfma32(a, b, c); }
  // fp32 -> element, round to nearest even
  __device__ __forceinline__ static __bf16 cvt(float x) { return (__bf16)x; }
  // element -> fp32 from the low / high half of a 32-bit word
  __device__ __forceinline__ static float lo(uint32_t x) { return __uint_as_float(x << 16); }
  __device__ __forceinline__ static float hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
};

struct F16 {
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  __device__ __forceinline__ static f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
  __device__ __forceinline__ static __bf16 cvt(float x) { return __builtin_bit_cast(__bf16, (_Float16)x); }
  __device__ __forceinline__ static float lo(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xffffu));
  }
  __device__ __forceinline__ static float hi(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
  }
};

// two fp32 -> two elements packed low | high << 16, round to nearest even
template <typename E>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, E::cvt(a)) | ((uint32_t)__builtin_bit_cast(uint16_t, E::cvt(b)) << 16);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// max / sum of x over the lane pair (l, l ^ 32)
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Pins a value at this point of the program: the empty asm claims to read and
// rewrite the registers, so the compiler can neither sink the code that
// produces them past a later barrier nor hoist the code that uses them above
// an earlier one. The kernels use it to keep matrix and vector phases on
// their side of a work-group barrier.
template <typename T>
__device__ __forceinline__ void fence_regs(T& x) {
  asm volatile("" : "+v"(x));
}

__device__ __forceinline__ bool wave_any(bool p) {
  return __builtin_amdgcn_ballot_w64(p) != 0;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// LDS tiles of ROWS x D 16-bit elements, row-major with a row pitch of P =
// lds_pitch<D>() elements, 16-byte chunks XOR-swizzled per row so that both
// read patterns below are free of bank conflicts. gfx950's LDS has 64 banks
// of 4 bytes, so one cycle serves 16 slots of 16 bytes; slot = (row * P / 8 +
// physical chunk) mod 16.
//   * row-operand reads (ds_read_b128): 16 lanes per cycle read 16
//     consecutive rows at one logical chunk c; they need 16 distinct slots.
//   * transposed reads (ds_read_b64_tr_b16): 32 lanes per cycle read 4
//     consecutive rows (aligned to 4) x 4 consecutive chunks (aligned to 4);
//     they need 16 distinct slots.
// physical chunk = c ^ f(row), with f depending on row % 16:
//   16 or more chunks per row (slot = chunk mod 16): f = 4 (row % 4) +
//     (row / 4) % 4 is a permutation of 0..15 (row reads), and 4 aligned rows
//     get distinct f / 4, i.e. distinct aligned groups of 4 chunks
//     (transposed reads).
//   8 chunks (slot = 8 (row % 2) + chunk): f = 4 ((row / 2) % 2) +
//     (row / 4) % 4 is a permutation of 0..7 over the even rows and over the
//     odd rows of any 16, and rows r, r + 2 of an aligned group of 4 get
//     distinct f / 4.
//   4 chunks (slot = 4 (row % 4) + chunk): f = (row / 4) % 4 separates the
//     four rows of any 16 that share row % 4; 4 aligned rows already differ
//     in row % 4.
// D = 96 has 12 chunks, which no XOR pattern keeps in range, so its rows are
// padded to 128 elements and use the 16-chunk pattern (the 4 spare chunks of
// each row hold zeros and are never read).
// ---------------------------------------------------------------------------
template <int D>
constexpr int lds_pitch() {
  return D == 96 ? 128 : D;
}

template <int P>
struct Swz {
  static constexpr int kChunks = P / 8;  // 16-byte chunks per row
  static_assert(kChunks == 4 || kChunks == 8 || kChunks >= 16, "no swizzle for this row pitch");
  __device__ __forceinline__ static int chunk(int row, int c) {
    if constexpr (kChunks >= 16) {
      return c ^ (((row & 3) << 2) | ((row >> 2) & 3));
    } else if constexpr (kChunks == 8) {
      return c ^ ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
    } else {
      return c ^ ((row >> 2) & 3);
    }
  }
  // element offset of (row, col) for a col that is a multiple of 4
  __device__ __forceinline__ static int offset(int row, int col) {
    return row * P + (chunk(row, col >> 3) << 3) + (col & 7);
  }
};

// Per-lane byte offsets of the two LDS read patterns, computed once per kernel
// so the reads in the loop need no address arithmetic (tile base and constant
// row offsets fold into the instruction's immediate offset).
//  RowRead: A/B operand of 8 consecutive elements of row (lane % 32) + 32 kb,
//           columns [16 ks + 8 hw, +8).
//  TrRead:  the transposed operand at rows 16 t + 4 hw + {0..3, 8..11} and
//           column 32 db + lane % 32: with read 0 at rows +{0..3} and read 1
//           at rows +{8..11}, lane l receives a 32x16 A operand whose k index
//           runs over rows in the order the score accumulators hold them.
// With 32 or more chunks per row the swizzle only changes the low four bits
// of a chunk index, so the offsets of chunks 16 .. 31 are those of chunks
// 0 .. 15 plus 256 bytes: only the first 16 chunks' offsets are kept in
// registers (at d = 256 this frees 16 registers per lane), and the rest is a
// constant folded into the instruction.
template <int D>
struct RowRead {
  static constexpr int P = lds_pitch<D>();
  static constexpr int kOff = D / 16 > 8 ? 8 : D / 16;  // operand steps of the first 16 chunks
  uint32_t off[kOff];
  __device__ __forceinline__ void init(int lane) {
    const int row = lane & 31, hw = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < kOff; ++ks) off[ks] = (uint32_t)(row * P + (Swz<P>::chunk(row, 2 * ks + hw) << 3)) * 2;
  }
  __device__ __forceinline__ bf16x8 operator()(const bf16_t* tile, int kb, int ks) const {
    return *(const FA_LDS bf16x8*)((const FA_LDS char*)(const FA_LDS bf16_t*)tile + off[ks % kOff] +
                                   (ks / kOff) * 256 + kb * 32 * P * 2);
  }
  // the same read from a tile given by its LDS byte address
  __device__ __forceinline__ bf16x8 at(const FA_LDS char* base, int kb, int ks) const {
    return *(const FA_LDS bf16x8*)(base + off[ks % kOff] + (ks / kOff) * 256 + kb * 32 * P * 2);
  }
};

template <int D>
struct TrRead {
  static constexpr int P = lds_pitch<D>();
  static constexpr int kOff = D / 32 > 4 ? 4 : D / 32;  // output blocks of the first 16 chunks
  uint32_t off[kOff][2];
  __device__ __forceinline__ void init(int lane) {
    const int s = lane & 15, hw = lane >> 5;
#pragma unroll
    for (int db = 0; db < kOff; ++db)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = 4 * hw + (s >> 2) + 8 * i;
        const int col = 32 * db + ((lane >> 4) & 1) * 16 + 4 * (s & 3);
        off[db][i] = (uint32_t)Swz<P>::offset(row, col) * 2;
      }
  }
  // rows t * 16 + ... (f(row) only depends on row % 16, so +16 rows is a constant)
  __device__ __forceinline__ bf16x8 operator()(const bf16_t* tile, int t, int db) const {
    const FA_LDS char* base = (const FA_LDS char*)(const FA_LDS bf16_t*)tile + t * 16 * P * 2 + (db / kOff) * 256;
    i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(base + off[db % kOff][0]));
    i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(base + off[db % kOff][1]));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 z = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    return __builtin_bit_cast(bf16x8, z);
  }
  // the same read from a tile given by its LDS byte address
  __device__ __forceinline__ bf16x8 at(const FA_LDS char* base, int t, int db) const {
    const FA_LDS char* b = base + t * 16 * P * 2 + (db / kOff) * 256;
    i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(b + off[db % kOff][0]));
    i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(b + off[db % kOff][1]));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 z = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    return __builtin_bit_cast(bf16x8, z);
  }
};


// Direct global -> LDS tile copy (buffer_load ... lds, 16 bytes per lane).
// A ROWS x D tile of 16-bit elements is THREADS/64 waves x kInstr
// instructions; instruction i of wave w fills LDS bytes [(w * kInstr + i) *
// 1024, +1024) of the tile, lane l writing 16 bytes at +16 l, i.e. rows
// lrow + i * kRowsPerInstr of the tile. Each lane fetches the global chunk
// that the swizzled layout stores at its LDS position. Global rows are
// `stride` bytes apart (a multiple of 16, at least one row): the lane's part
// of the offset is lrow * stride plus its swizzled chunk, the rest is a
// wave-uniform row offset. Rows past the end of the buffer resource (see
// rows_rsrc) arrive as zeros, so ragged tails need no branches. No registers
// hold the tile.
template <int ROWS, int D, int THREADS>
struct TileDma {
  static constexpr int P = lds_pitch<D>();
  static constexpr int kRowBytes = P * 2;  // in LDS
  static constexpr int kTileBytes = ROWS * kRowBytes;
  static constexpr int kWaves = THREADS / 64;
  static constexpr int kInstr = kTileBytes / 1024 / kWaves;
  static constexpr int kRowsPerInstr = 1024 / kRowBytes;
  static_assert(kTileBytes % (1024 * kWaves) == 0, "tile must split into whole 1 KB wave copies");
  static_assert(1024 % kRowBytes == 0, "a 1 KB wave copy must hold whole rows");
  // the swizzle depends on row % 16 only, so the chunk offsets repeat after
  // kPeriod instructions
  static constexpr int kPeriod = kInstr < 16 / kRowsPerInstr ? kInstr : 16 / kRowsPerInstr;
  uint32_t chunk_off[kPeriod];  // byte offset of this lane's (swizzled) chunk inside its row
  uint32_t lrow;                // this lane's row in the wave's first instruction
  int lds_off;                  // byte offset of this wave's first 1 KB inside an LDS tile

  __device__ __forceinline__ void init(int wave, int lane) {
    lds_off = wave * kInstr * 1024;
    lrow = (uint32_t)((lds_off + 16 * lane) / kRowBytes);
    const int chunk = ((16 * lane) % kRowBytes) / 16;
#pragma unroll
    for (int i = 0; i < kPeriod; ++i) {
      // the global chunk this LDS position holds; padding chunks of a padded
      // row point past every buffer (offsets stay below 2^31 + 2^31), so they
      // are filled with zeros
      const int g = Swz<P>::chunk(lrow + i * kRowsPerInstr, chunk);
      chunk_off[i] = g < D / 8 ? (uint32_t)(g * 16) : 0x80000000u;
    }
  }
  // Copy rows [row0, row0 + ROWS) of the tensor behind `rsrc` (rows `stride`
  // bytes apart) into `tile`. The whole offset goes in the vector offset: the
  // buffer range check that zero-fills rows past the end does not include the
  // scalar offset.
  // The stride and the LDS destination are laundered through empty asm so the
  // compiler computes the offsets and the kInstr destination addresses here,
  // per copy, instead of hoisting them per tensor and per buffer into
  // registers for the whole loop.
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rsrc, bf16_t* tile, int row0, uint32_t stride) const {
    asm volatile("" : "+s"(stride));
    const uint32_t lane_base = (lrow + (uint32_t)row0) * stride;
    uint32_t dst0 = (uint32_t)(uintptr_t)((FA_LDS char*)(FA_LDS bf16_t*)tile + lds_off);
    asm volatile("" : "+s"(dst0));
#pragma unroll
    for (int i = 0; i < kInstr; ++i) {
      FA_LDS void* dst = (FA_LDS void*)(uintptr_t)(dst0 + i * 1024);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, lane_base + chunk_off[i % kPeriod] + i * kRowsPerInstr * stride, 0,
                                               0, 0);
    }
  }
};

// Buffer resource over `bytes` bytes at `base`; loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Buffer resource over `rows` rows of D 16-bit elements, `stride` bytes
// apart: it ends right after the last element of the last row, so a 16-byte
// load of any row at or past `rows` lies wholly outside and returns zeros.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int rows, uint32_t stride) {
  return make_rsrc(base, rows > 0 ? (uint32_t)(rows - 1) * stride + D * 2 : 0u);
}

// Wait until every vector-memory operation of this wave (including the
// direct-to-LDS copies) has completed: s_waitcnt vmcnt(0).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Work-group barrier for hand-offs through LDS. __syncthreads() also makes
// every wave wait for all of its outstanding global -> LDS copies (its release
// fence counts them as LDS stores), which would cut a copy's time to land to
// the one phase it was issued in. Here the waves wait only for their own LDS
// reads and writes; a copy's consumer waits for it explicitly (wait_vmem in
// the issuing wave before the barrier that hands the tile over). The memory
// clobber keeps the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Work-group id remap so that consecutive logical blocks (the query blocks of
// one head) run on the same XCD and share its L2: hardware hands work-group
// ids to the 8 XCDs round-robin.
__device__ __forceinline__ int xcd_logical_block(int bid, int nblocks) {
  if ((nblocks & 7) != 0) return bid;
  return (bid & 7) * (nblocks >> 3) + (bid >> 3);
}

}  // namespace fa
