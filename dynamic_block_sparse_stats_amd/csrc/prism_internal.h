// prism_internal.h -- types, workspace layout and kernel launchers shared by the
// translation units of libprism.so.  Not installed; the public ABI is include/prism.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/prism.h"

namespace prism {

constexpr int kZone = 8;       // macro-zone edge along T, H, W
constexpr int kZoneTok = 512;  // tokens per zone
constexpr int kUnit = 64;      // tokens per atomic compute unit of the attention kernels
constexpr int kMaxUnits = 65535;  // units per head (block indices fit 16 bits)
constexpr int kTile64 = 1 << 30;  // key tile flag: 64 keys (a 64-token block) instead of 128

// Per-stage tracing: while enabled, records a HIP event pair on the stream around the
// launches of a stage (prism_api.hip).
struct TraceScope {
  TraceScope(int stage, hipStream_t s);
  ~TraceScope();
  int stage;
  hipStream_t stream;
  void *start;
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

struct Dims {
  int T, H, W, heads, D, dtype;
  int Dp;                // row width of the permuted operand copies: 128 for bfloat16 (a
                         //   64-channel head is zero-padded), D for float32
  int N, Z, U, nb_max;   // tokens, zones, 64-token units, max blocks per head (= U)
  int nzt, nzh, nzw;     // zones per axis
  int words;             // 32-bit words per selection bitmask row
  long long cap;         // capacity of one head's CSR (and CSC) lists in block pairs
  size_t elt;            // bytes per token-tensor element
  // element strides of the q, k, v inputs of prism_plan: (token n, head h, channel c) at
  // n * tok_stride + h * head_stride + c (dense [N][heads][D] by default)
  size_t tok_stride, head_stride;
};

// Internal workspace layout: the public arrays of prism_layout plus scratch.
struct Layout {
  prism_layout pub;
  size_t qp, kp, vp;        // permuted copies, row-major [heads][N][D] (float16 for
                            //   bfloat16 inputs, float32 for float32 inputs)
  size_t sel_bits;          // uint32 [heads][nb_max][words]
  size_t csc_bits;          // uint32 [heads][nb_max][words]
  size_t tiles;             // int2 [heads*U]: key tiles, (head, first unit | kTile64)
  size_t btiles;            // int2 [heads*2Z]: query tiles of 256 rows, (head, first unit |
                            //   (log2 B - 6) << 16), two per zone
  size_t counters;          // int32 [16]: [0] = key tiles of 128 keys, [1] = query tiles,
                            //   [2] = key tiles of 256-token blocks (listed first), [3] =
                            //   64-key tiles (listed last, from [0] on)
  // Query tile lists: per query tile, the union of the selection lists of its blocks (one
  // block of 256, two of 128 or four of 64 tokens).  Entries are j | mask << 16: key block j
  // and the bit g set when the tile's block g selects it.  Per head: counts, offsets (as the
  // CSR) and the entries within the pair capacity.
  size_t qt_count, qt_ptr, qt_list;  // int32 [heads][2Z], [heads][2Z+1], [heads][cap]
  size_t dop;               // bwd: gathered dout, row-major [heads][N][D] (as qp)
  size_t o32p;              // fwd: float [heads][N][D] output in permuted order
  size_t lsep;              // fwd: float [heads][N] lse in permuted order
  size_t delta;             // bwd: float [heads][N] in permuted order: rowsum(dO * O)
                            //   (float32 inputs) or -rowsum(dO * O) (bfloat16)
  size_t lse2;              // bwd (bfloat16): float [heads][N] lse * log2(e)
  size_t vmax;              // float [heads]: largest row norm of V (the dS range bound)
  size_t total;
};

prism_status check_config(const prism_config *cfg, Dims *d, const char **why);
Layout make_layout(const Dims &d);

struct Scales {
  float score, softmax;
};
Scales scales_of(const prism_config *cfg, const Dims &d);

// ---------------------------------------------------------------------------- launchers
// plan_kernels.hip
hipError_t launch_audio_stats(const Dims &d, const float *a2v, double *astat, hipStream_t s);
hipError_t launch_zone_stats(const Dims &d, const void *v, int dmode, double *zstat,
                             hipStream_t s);
hipError_t launch_quantize(const Dims &d, const prism_config *cfg, const double *zstat,
                           const double *astat, bool have_audio, uint8_t *ws, const Layout &L,
                           hipStream_t s);
hipError_t launch_gather(const Dims &d, const void *q, const void *k, const void *v,
                         uint8_t *ws, const Layout &L, hipStream_t s);
hipError_t launch_tiles(const Dims &d, uint8_t *ws, const Layout &L, hipStream_t s);
// select_kernels.hip
hipError_t launch_scores_select(const Dims &d, const prism_config *cfg, float score_scale,
                                uint8_t *ws, const Layout &L, hipStream_t s);
// attn_fwd.hip
hipError_t launch_attn_fwd(const Dims &d, float scale, uint8_t *ws, const Layout &L, void *o,
                           float *lse, hipStream_t s);
// attn_bwd.hip
hipError_t launch_attn_bwd(const Dims &d, float scale, uint8_t *ws, const Layout &L,
                           const void *dout, void *dq, void *dk, void *dv, hipStream_t s);

// attn_bwd_dkdv.hip
hipError_t launch_dkdv_bf16(int work_items, hipStream_t s, int N, int U, int nb_max, int heads,
                            const int2 *tiles, const int *counters, const uint16_t *qp,
                            const uint16_t *kp, const uint16_t *vp, const uint16_t *dop,
                            const float *lse2, const float *ndelta, const int *unit_blk,
                            const int *bstart, const int *bsize, const int *tcnt,
                            const int *tptr, const int *trows, long long cap, const int *perm,
                            float scale, float sl2e, int dio, const uint32_t *flags,
                            uint16_t *dk, uint16_t *dv);

// a2v_norm.hip
hipError_t launch_a2v_norm(const void *x, long long n_tokens, int channels, long long ld,
                           int dtype, float *out, hipStream_t s);

// Workgroups of `kernel` (block size `block`) that fit on the current device at once: the
// grid of the persistent attention kernels.
int resident_grid(const void *kernel, int block, int work_items);

// ---------------------------------------------------------------------------- device helpers
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// Round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Row-major [64][128] 16-bit LDS tile: 16 chunks of 16 bytes per row (one row spans the 64
// banks once), chunk c of row r stored at chunk c ^ swz(r), swz(r) = 4 (r % 4) + (r / 4) % 4.
// swz is a bijection on r % 16, so 16-byte reads of one chunk by 16 consecutive rows hit
// 16 different chunk positions; and four consecutive rows (r % 4 = 0..3, same (r / 4) % 4)
// spread a group of four aligned chunks over four different quarters of the banks, which
// keeps the 8-byte transposed reads below (4 rows x 4 chunks x 2 halves per 32 lanes)
// free of bank conflicts too.
// (The address helpers below are __host__ __device__ so that host code can check them.)
__host__ __device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__host__ __device__ __forceinline__ int rm_swz(int r, int c) {
  return r * 256 + ((c ^ swz(r)) << 4);
}

// The A operand of a 32x32x16 float16 MFMA taken transposed from a row-major float16 tile
// X[k][d] with ds_read_b64_tr_b16 (in each 16-lane group, lane i receives element i % 4 of
// the 8-byte pieces addressed by lanes 4j + i / 4, j = 0..3).  Lane l gets, in register e,
// X[kb + 8 (e / 4) + 4 (l / 32) + e % 4][db + l % 32]: row l % 32 of the transposed tile
// and the same key order as a B operand taken from a C tile (register v of a C tile holds
// row (v / 4) * 8 + 4 (l / 32) + v % 4).  kb is a multiple of 16, db of 32.
// Byte offset in the tile of the 8-byte piece lane `lane` addresses in read m (rows 8m ..).
__host__ __device__ __forceinline__ int tr_offset(int kb, int db, int lane, int m) {
  const int g = lane >> 4, s = lane & 15;
  const int col = db + 16 * (g & 1) + 4 * (s & 3);
  const int row = kb + 8 * m + 4 * (g >> 1) + (s >> 2);
  return rm_swz(row, col >> 3) + (col & 7) * 2;
}
__device__ __forceinline__ f16x8 tr_operand(const uint8_t *tile, int kb, int db, int lane) {
  f16x8 r;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const fp16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
        (__attribute__((address_space(3))) fp16x4_t *)(tile + tr_offset(kb, db, lane, m)));
    const f16x4 w = __builtin_bit_cast(f16x4, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) r[4 * m + e] = w[e];
  }
  return r;
}

// The same reads with the per-lane address arithmetic hoisted: in a 256-byte aligned tile the
// swizzle and the chunk index only touch address bits 4-7, so chunk c of row r lies at
// row_base(r) ^ (c << 4); and a transposed piece (kb, db) lies at tr_base ^ (2 db) + 256 kb
// (kb a multiple of 16 leaves swz unchanged, db a multiple of 32 flips chunk bits 2-3 only).
// A wave then keeps one or two base registers per tile instead of one address per read.
// Addresses are 32-bit LDS byte addresses.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
__host__ __device__ __forceinline__ uint32_t row_base(uint32_t tile, int r) {
  return tile + (uint32_t)(r * 256 + (swz(r) << 4));
}
__device__ __forceinline__ f16x8 lds_row16(uint32_t addr) {
  return __builtin_bit_cast(
      f16x8, *(const __attribute__((address_space(3))) u32x4 *)(uintptr_t)addr);
}
struct TrBase {
  uint32_t m0, m1;  // the lane's 8-byte piece of rows 0-7 and 8-15 at kb = 0, db = 0
};
__host__ __device__ __forceinline__ TrBase tr_base(uint32_t tile, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int col = 16 * (g & 1) + 4 * (s & 3);
  const int row = 4 * (g >> 1) + (s >> 2);
  const uint32_t t = tile + (uint32_t)((col & 7) * 2);
  return {t + (uint32_t)rm_swz(row, col >> 3), t + (uint32_t)rm_swz(row + 8, col >> 3)};
}
// The LDS address of read m of tr_operand(tile, kb, db, lane) from tr_base(tile, lane)
__host__ __device__ __forceinline__ uint32_t tr_addr(const TrBase &b, int m, int kb, int db) {
  return ((m ? b.m1 : b.m0) ^ (uint32_t)(2 * db)) + (uint32_t)(256 * kb);
}
// tr_operand(tile, kb, db, lane) from tr_base(tile, lane)
__device__ __forceinline__ f16x8 tr_read(const TrBase &b, int kb, int db) {
  f16x8 r;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const uint32_t a = tr_addr(b, m, kb, db);
    const fp16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
        (__attribute__((address_space(3))) fp16x4_t *)(uintptr_t)a);
    const f16x4 w = __builtin_bit_cast(f16x4, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) r[4 * m + e] = w[e];
  }
  return r;
}

// Typed MFMA wrappers: the builtins accept any 8-element 16-bit vector silently, these do
// not (32x32 output tile, K = 16; C/D layout: lane -> column lane % 32, register v -> row
// (v / 4) * 8 + 4 * (lane / 32) + v % 4).
__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// acc[dt] (C layout: lane = column j, register -> d) += T^T[d][k] X[k][j] over the 64 rows
// k of a row-major [64][128] float16 tile whose transposed-read base is tb; X holds the
// float16 B operands of the four 16-row slices ([half][slice], in the row order of a C
// tile's registers).  Per slice the four d-tiles' accumulators are independent, and the
// next slice's operands are read while one runs.
__device__ __forceinline__ void tr_update(f32x16 (&acc)[4], const TrBase &tb,
                                          const f16x8 (&x)[2][2]) {
  f16x8 ta[2][4];  // [buffer][dt]
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) ta[0][dt] = tr_read(tb, 0, 32 * dt);
#pragma unroll
  for (int sl = 0; sl < 4; ++sl) {
    if (sl < 3)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) ta[(sl + 1) & 1][dt] = tr_read(tb, 16 * (sl + 1), 32 * dt);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      acc[dt] = mfma_f16(ta[sl & 1][dt], x[sl >> 1][sl & 1], acc[dt]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Direct global -> LDS copies (global_load_lds): lane l of one instruction reads 16 (or 4)
// bytes at base + off and writes them at dst + 16 * l (4 * l); base and dst must be
// uniform across the wave (dst is passed in M0).  They are written as inline assembly on
// purpose: the compiler classes the instruction as a flat access that may touch LDS, and
// while one is outstanding on vmcnt (in these kernels: always) it makes every wait for an
// LDS read wait for all of them (lgkmcnt(0)), which stops any LDS read from overlapping
// the MFMAs before it.  The
// hardware counts these copies on vmcnt only.  Hidden from the compiler, they are ordered
// by the kernels themselves: explicit s_waitcnt vmcnt before the barrier that publishes a
// stage, and the "memory" clobber, which keeps the compiler from moving LDS accesses across
// a copy.  (Loads the compiler issues itself stay correct: copies it does not know of only
// make its vmcnt waits stricter.)  M0 is written only here in these kernels.
__device__ __forceinline__ uint32_t lds_dst(void *dst) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)dst);
}
// The copies take the instruction's saddr form: a wave-uniform 64-bit base in SGPRs plus a
// 32-bit per-lane byte offset, so a copy costs no per-lane 64-bit address arithmetic (the
// offsets stay in registers across the whole list walk).
// IMM, the instruction's offset field (0 .. 4095), is added to both addresses: the global
// one (base + off + IMM) and the LDS one (dst + IMM)
template <int IMM = 0>
__device__ __forceinline__ void dma16(const void *base, uint32_t off, void *dst) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%3"
               :
               : "v"(off), "s"(base), "s"(lds_dst(dst)), "i"(IMM)
               : "memory");
}

// A wave's share of a unit copy: rows r0 .. r0 + 15 (r0 a multiple of 16) of a row-major
// [64][128] 16-bit tile, swizzled as in rm_swz, in four 1 KB copies of four rows each.  Lane
// l fetches chunk (l % 16) ^ swz(r) of row r = r0 + 4i + l / 16 in copy i; with r0 a multiple
// of 16, swz(r) = 4 (l / 16) + i, so the lane's source offset in copy i is
// (c0 ^ 16 i) + 1024 i with c0 = copy_offset(r0, l) that of copy 0: one register and a XOR
// per copy, the 1024 i going into the instruction's offset field (which moves the LDS
// destination by the same 1024 i).
__host__ __device__ __forceinline__ uint32_t copy_offset(int r0, int lane) {
  const int r = r0 + (lane >> 4);
  return (uint32_t)(r * 256 + (((lane & 15) ^ swz(r)) << 4));
}
__device__ __forceinline__ void copy_rows16(const void *src, uint32_t c0, uint8_t *dst) {
  dma16<0>(src, c0, dst);
  dma16<1024>(src, c0 ^ 16u, dst);
  dma16<2048>(src, c0 ^ 32u, dst);
  dma16<3072>(src, c0 ^ 48u, dst);
}
__device__ __forceinline__ void dma4(const void *base, uint32_t off, void *dst) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(off), "s"(base), "s"(lds_dst(dst))
               : "memory");
}

// s_waitcnt with the given immediate, then a workgroup barrier.  The compiler fences on
// both sides keep every memory operation of this wave in program order around the pair:
// LDS writes issued before it are covered by the wait (s_barrier itself does not order
// memory for the compiler).
template <int IMM>
__device__ __forceinline__ void wait_and_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(IMM);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8): wait for this wave's vector memory operations down to n outstanding, or for its
// LDS operations
constexpr int vmcnt_imm(int n) { return 0x0f70 | n; }
constexpr int kLgkm0 = 0xc07f;
// every copy of this wave has landed, then a workgroup barrier
__device__ __forceinline__ void wait_copies_and_sync() { wait_and_barrier<vmcnt_imm(0)>(); }
// a workgroup barrier that the compiler may not move memory operations across
__device__ __forceinline__ void workgroup_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// The 64-token units of a list of blocks, in list order (a block of B tokens is B/64
// consecutive units).  With MASKS (the query tiles' lists) entries are j | mask << 16: block
// j and the mask of the tile's blocks that selected it; without (the transposed lists)
// entries are plain block indices.  The list is read 64 entries at a time, one per lane, and
// the current entry is broadcast from its lane: the walk itself issues no memory operation,
// so it never waits behind the direct-to-LDS copies in flight (loads complete in order).
// The members other than the window are the same in every lane.
template <bool MASKS>
struct BlockUnits {
  int base, idx, sub, us, nu, n, lane, self, mask;
  bool empty;
  int win_us, win_nu, win_mask;  // this lane's entry of the window
  const int *list, *bstart, *bsize;
  __device__ void fill() {  // lanes past the end repeat the last entry (never used)
    int j;
    if constexpr (MASKS) {
      const int e = empty ? (self | (0xf << 16)) : list[min(base + lane, n - 1)];
      j = e & 0xffff;
      win_mask = (e >> 16) & 0xf;
    } else {
      j = empty ? self : list[min(base + lane, n - 1)];
    }
    win_us = bstart[j] / kUnit;
    win_nu = bsize[j] / kUnit;
  }
  __device__ void load() {
    us = __builtin_amdgcn_readlane(win_us, idx);
    nu = __builtin_amdgcn_readlane(win_nu, idx);
    if constexpr (MASKS) mask = __builtin_amdgcn_readlane(win_mask, idx);
  }
  // a list of count entries; an empty one (a list a full selection capacity cut to
  // nothing: its head's outputs are NaN) walks the block self_blk instead
  __device__ void init(const int *l, int count, const int *bs, const int *bz, int lane_id,
                       int self_blk) {
    list = l;
    n = __builtin_amdgcn_readfirstlane(count);
    empty = n < 1;
    self = self_blk;
    if (empty) n = 1;
    bstart = bs;
    bsize = bz;
    lane = lane_id;
    base = idx = sub = 0;
    mask = 0xf;
    fill();
    load();
  }
  __device__ int unit() const { return us + sub; }
  // advances; false once the list is exhausted
  __device__ bool next() {
    if (++sub < nu) return true;
    sub = 0;
    if (base + ++idx >= n) return false;
    if (idx == 64) {
      base += 64;
      idx = 0;
      fill();
    }
    load();
    return true;
  }
};

// bfloat16 -> float16 bits (exact inside the float16 range; saturates beyond +-65504).
__device__ __forceinline__ uint16_t bf16_to_f16_bits(uint16_t b) {
  float f = fminf(fmaxf(bf16_to_f32(b), -65504.f), 65504.f);
  _Float16 h = (_Float16)f;
  return __builtin_bit_cast(uint16_t, h);
}

// Softmax weights fed to the f16 MFMA are scaled by 2^10 so that weights down to 2^-24 of
// the row maximum stay normal float16 numbers; the scale cancels in O = sum(p v) / sum(p).
constexpr float kPShift = 10.f;
constexpr float kPScale = 1024.f;
// Lazy rescaling in the forward: the running max is kept until a new maximum exceeds it
// by more than kLazy (log2 units); weights then stay below 2^(kPShift + kLazy) = 2^15.
constexpr float kLazy = 5.f;

// NaN bit patterns for the outputs of a head whose status flags are set (selected and
// stored as integers: the attention kernels are compiled without NaN semantics)
constexpr uint32_t kNaNf32 = 0x7fc00000u;
constexpr uint32_t kNaNbf16x2 = 0x7fc07fc0u;

template <typename T>
__device__ __forceinline__ T *ws_ptr(uint8_t *ws, size_t off) {
  return reinterpret_cast<T *>(ws + off);
}

}  // namespace prism
