// attn_fwd.hip -- exact attention over the selected key blocks (arXiv 2610.05416; nanless
// digest, selection section: every query token of a block against the keys and values of
// the blocks chosen for it, with an online softmax so the score matrix is never stored;
// training section: 64-token atomic units, a 128-token block is 2 units and a 256-token
// block 4, taken in turn; xyznot review, "Метод" item 3).
//
// bfloat16 path, head_dim 128, gfx950 MFMA v_mfma_f32_32x32x16_f16 (the planner stores
// the permuted Q, K, V as float16: exact for bfloat16 values inside the float16 range):
//   * a workgroup (8 waves, two per SIMD) owns one query tile of 256 rows: one block of
//     256, two of 128 or four of 64 tokens, 32 rows per wave; each wave keeps its 32 query
//     rows in registers as the B operand; one workgroup per CU, persistent over the tiles;
//   * the key units of the union of the tile's blocks' selections stream through a
//     four-stage LDS ring (128 KB) filled by direct global->LDS copies, two units ahead of
//     the one being computed (the fourth stage is still being read by the late waves,
//     below): K and V as [64 keys][128] float16, XOR-swizzled by 16-byte chunk; K rows are
//     read directly, V^T with transposing LDS reads (ds_read_b64_tr_b16); each wave
//     computes only the units its own block selected (an entry's mask bit), so with blocks
//     of 64 or 128 tokens every wave still has work;
//   * the two waves of a SIMD run half a unit apart (the late one finishes the previous
//     unit's PV product and forms its scores, then issues its copies, while the early one
//     issues its copies and forms its scores), each wave raises its issue priority while it
//     forms the scores its softmax waits for, and each reads the operands of its next group
//     of MFMAs while the current group runs;
//   * the softmax weights go to the PV product as float16 scaled by 2^10 (11-bit
//     significands where bf16 has 8: at 2K, value rows reach |v| ~ 20 and the PV sums
//     cancel, so bf16 weights cost ~3e-2 absolute); the row sum adds the same float16
//     weights and is kept in float64;
//   * S^T = K Q^T (keys x queries) leaves each query's scores in one lane pair, so the
//     online-softmax max and sum are lane-local plus one exchange across the two half
//     waves; O^T += V^T P^T keeps the output with the same lane-per-query layout, so the
//     rescale by exp(m_old - m_new) is lane-local too;
//   * the epilogue divides by the row sum, writes O to the token's original position
//     (inverse permutation fused) and the natural-log LSE.
// float32 path (small grids): one workgroup per 64-row unit, 4 threads per query row,
// float64 accumulation.
#include "prism_internal.h"

namespace prism {

constexpr int kD = 128;

constexpr int NW = 8;      // waves per workgroup: 8 x 32 = 256 query rows, one block
constexpr int kStages = 4;  // LDS ring depth (copies run 2 units ahead of the one computed)
constexpr int kCpw = 32 / NW;  // 1 KB copies per wave per unit (16 for K, 16 for V)
static_assert(kCpw == 4, "copy_rows16 issues four copies per wave and unit");

// Four LDS stages of 32 KB (distinct objects, named statically by the unrolled unit loop)
// filled by direct global->LDS copies: waves 0-3 copy 16 K rows each, waves 4-7 16 V rows
// each, 4 instructions of 1 KB per wave and unit.
struct FwdStage {
  uint8_t k[16384];  // [64 keys][128] float16, swizzled
  uint8_t v[16384];  // [64 keys][128] float16, swizzled (read transposed)
};
__shared__ __align__(256) FwdStage g_fwd0;
__shared__ __align__(256) FwdStage g_fwd1;
__shared__ __align__(256) FwdStage g_fwd2;
__shared__ __align__(256) FwdStage g_fwd3;
template <int S>
__device__ __forceinline__ FwdStage &fwd_stage() {
  return S == 0 ? g_fwd0 : (S == 1 ? g_fwd1 : (S == 2 ? g_fwd2 : g_fwd3));
}
struct FwdState {
  f16x8 qreg[8];
  f32x16 o[4];
  f16x8 pb[4];  // the current unit's softmax weights, float16 (B operand of the PV product)
  float m, mk;
  double lsum;
};

// S^T = K Q^T for the unit, the online-softmax update (which rescales O) and the unit's
// float16 weights; kt is the LDS address of the unit's K tile
__device__ __forceinline__ void fwd_scores(FwdState &w, uint32_t kt, int lane,
                                           float scale_log2e) {
  const int l32 = lane & 31, hh = lane >> 5;
  // chunk 2kk + hh of key row l32 (a = 0) at kr ^ (kk << 5), of row 32 + l32 8 KB further
  const uint32_t kr = row_base(kt, l32) ^ (uint32_t)(hh << 4);
  // S^T for keys 0-31 (a = 0) and 32-63 (a = 1): lane = query l32, 16 keys per tile.  The
  // operands of the next group of four MFMAs are read while the current group runs.
  f32x16 s[2] = {f32x16{}, f32x16{}};
  f16x8 ka[2][2][2];  // [buffer][a][e]
  auto load = [&](int buf, int grp) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int e = 0; e < 2; ++e)
        ka[buf][a][e] = lds_row16((kr ^ (uint32_t)((2 * grp + e) << 5)) + 8192u * a);
  };
  // the wave issues at a raised priority while it forms the scores its softmax waits for,
  // and at the default one for the exponentials, so that the SIMD's other wave runs its
  // MFMAs under them
  __builtin_amdgcn_s_setprio(1);
  load(0, 0);
#pragma unroll
  for (int grp = 0; grp < 4; ++grp) {
    if (grp < 3) load((grp + 1) & 1, grp + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int a = 0; a < 2; ++a) s[a] = mfma_f16(ka[grp & 1][a][e], w.qreg[2 * grp + e], s[a]);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);
  // online softmax (log2 domain) with lazy rescaling: the running max only moves when a
  // query's new maximum exceeds it by more than 2^kLazy, so the float16 weights
  // 2^(t - m + 10) stay below 2^15
  float tmax = fmaxf(s[0][0], s[0][1]);
#pragma unroll
  for (int v = 2; v < 16; v += 2) tmax = fmaxf(tmax, fmaxf(s[0][v], s[0][v + 1]));
#pragma unroll
  for (int v = 0; v < 16; v += 2) tmax = fmaxf(tmax, fmaxf(s[1][v], s[1][v + 1]));
  {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax),
                                               false, false);
    tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  }
  const float tm = tmax * scale_log2e;
  const bool grow = tm > w.m + kLazy;
  if (__ballot(grow)) {
    const float mnew = grow ? tm : w.m;
    const float alpha = __builtin_amdgcn_exp2f(w.m - mnew);
    w.m = mnew;
    w.mk = mnew - kPShift;
    w.lsum *= (double)alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) w.o[dt][v] *= alpha;
  }
  // the row sum adds the float16 weights the MFMA consumes (two per dot2 instruction), so
  // the normaliser matches the weights exactly
  // (built in a fresh variable: the previous unit's weights are dead from here on)
  float psum = 0.f;
  f16x8 pb[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      pb[g][e] = (_Float16)__builtin_amdgcn_exp2f(
          fmaf(s[g >> 1][8 * (g & 1) + e], scale_log2e, -w.mk));
#pragma unroll
    for (int e = 0; e < 8; e += 2)
      psum = __builtin_amdgcn_fdot2(f16x2{pb[g][e], pb[g][e + 1]}, f16x2{1, 1}, psum, false);
  }
  w.lsum += (double)psum;
#pragma unroll
  for (int g = 0; g < 4; ++g) w.pb[g] = pb[g];
}

// O^T[d][q] += V^T[d][keys] P^T[keys][q] with the weights of the last fwd_scores, V^T read
// transposed from the row-major tile at LDS address vt; per 16-key slice the four d-tiles'
// accumulators are independent
__device__ __forceinline__ void fwd_values(FwdState &w, uint32_t vt, int lane) {
  const TrBase vb = tr_base(vt, lane);
  f16x8 va[2][4];  // [buffer][dt]: the next slice's operands are read while one runs
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) va[0][dt] = tr_read(vb, 0, 32 * dt);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    if (g < 3)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) va[(g + 1) & 1][dt] = tr_read(vb, 16 * (g + 1), 32 * dt);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) w.o[dt] = mfma_f16(va[g & 1][dt], w.pb[g], w.o[dt]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The LDS address of stage S plus an opaque zero: it keeps the compiler from hoisting the
// per-lane addresses of all four stages into registers for the whole loop
template <int S>
__device__ __forceinline__ uint32_t fwd_stage_addr() {
  int z = 0;
  asm volatile("" : "+v"(z));
  return lds_addr(&fwd_stage<S>()) + (uint32_t)z;
}

// s_waitcnt vmcnt(kCpw) (expcnt and lgkmcnt left alone), then a workgroup barrier: every
// wave issues exactly kCpw copies per step, so this wave's copies for the unit one step
// back have landed (vector memory loads complete in order), and after the barrier every
// wave's have.  The count is the same on every path, which also lets the compiler see that
// no further wait is needed before the LDS reads.
__device__ __forceinline__ void wait_unit_one_behind() {
  wait_and_barrier<vmcnt_imm(kCpw)>();
}

// The waves of one role.  The two waves of a SIMD (w and w + 4) run half a unit apart so
// that one's softmax arithmetic overlaps the other's MFMAs: after the barrier of step u the
// early wave (w < 4) forms the scores of unit u, then its PV product; the late wave first
// finishes the PV product of unit u - 1, then forms the scores of unit u, and carries their
// weights across the next barrier.
template <bool LATE>
__device__ __forceinline__ void fwd_waves(
    int wave, int lane, int N, int U, int nb_max, int heads, const int2 *__restrict__ tiles,
    int ntiles, const uint16_t *__restrict__ qp, const uint16_t *__restrict__ kp,
    const uint16_t *__restrict__ vp, const int *__restrict__ unit_blk,
    const int *__restrict__ blk_start, const int *__restrict__ blk_size,
    int Z, const int *__restrict__ qt_count, const int *__restrict__ qt_ptr,
    const int *__restrict__ qt_list, long long cap, const int *__restrict__ perm,
    float scale_log2e, int dio, const uint32_t *__restrict__ flags, uint16_t *__restrict__ out,
    float *__restrict__ lse_out, float *__restrict__ o32p, float *__restrict__ lsep) {
  const int l32 = lane & 31, hh = lane >> 5;
  // copies of this wave: K rows 16w.. (early waves) or V rows 16(w-4).. (late waves)
  const int wq = wave & (NW / 2 - 1);
  const uint8_t *csrc = reinterpret_cast<const uint8_t *>(LATE ? vp : kp);
  const int cdst = (LATE ? 16384 : 0) + wq * 4096;
  const uint32_t c0 = copy_offset(16 * wq, lane);  // this lane's source offset in the unit

  for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int2 tl = tiles[t];
    const int h = __builtin_amdgcn_readfirstlane(tl.x);
    const int ty = __builtin_amdgcn_readfirstlane(tl.y);
    // 256 query rows: one block of 256, two of 128 or four of 64 tokens; the tile's list is
    // the union of its blocks' lists, each entry with the mask of the blocks that selected it
    const int u0 = ty & 0xffff, lb = (ty >> 16) & 3;
    const int g = (32 * wave) >> (6 + lb);  // this wave's block within the tile
    const int qslot = u0 >> 2;
    const int blk = unit_blk[(size_t)h * U + u0];
    const int *bs = blk_start + (size_t)h * nb_max, *bz = blk_size + (size_t)h * nb_max;
    BlockUnits<true> pre;  // the issuing cursor
    pre.init(qt_list + (size_t)h * cap + qt_ptr[(size_t)h * (2 * Z + 1) + qslot],
             qt_count[(size_t)h * 2 * Z + qslot], bs, bz, lane, blk);

    // this wave's 32 query rows as B operands: Q[row][16kk + 8hh .. +8]
    const int row0 = u0 * kUnit + wave * 32;
    FwdState w;
    {
      const uint16_t *qrow = qp + ((size_t)h * N + row0 + l32) * kD + 8 * hh;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        w.qreg[kk] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(qrow + 16 * kk));
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) w.o[dt] = f32x16{};
    w.m = -INFINITY;
    w.mk = -INFINITY;
    w.lsum = 0.0;

    // the Q rows (and the cursor's first window) have landed before any copy is issued,
    // so no later LDS read or MFMA waits behind the copies for them
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    const uint8_t *hbase = csrc + (size_t)h * N * kD * 2;
    int issued = 0;
    bool pending = true;  // pre points at a unit not yet issued
    int smask[kStages];   // the entry mask of the unit in each stage
    // every step issues kCpw copies: past the end of the list they repeat the last unit
    // into a stage no step reads any more (drained before the next tile)
    auto issue = [&](auto stage_tag) {
      constexpr int X = decltype(stage_tag)::value;
      const uint8_t *src = hbase + (size_t)pre.unit() * kUnit * kD * 2;
      copy_rows16(src, c0, reinterpret_cast<uint8_t *>(&fwd_stage<X>()) + cdst);
      smask[X] = pre.mask;
      if (pending) {
        ++issued;
        pending = pre.next();
      }
    };
    // step u (stage S = u mod 4): wait for unit u (unit u + 1 stays in flight), refill the
    // stage of unit u - 2 (no wave reads it any more) with unit u + 2, compute the units
    // this wave's block selected.  One step past the last unit finishes the late wave's PV
    // product.  Returns whether unit u existed.
    auto step = [&](auto stage_tag, int u) {
      constexpr int S = decltype(stage_tag)::value;
      wait_unit_one_behind();
      // issued counts the units up to u + 1 at least, or all of them
      const bool unit_u = u < issued;
      const bool on = unit_u && ((smask[S] >> g) & 1);
      const uint32_t st = fwd_stage_addr<S>();
      if constexpr (LATE) {
        // the late wave issues its copies at the end of its step, so that right after the
        // barrier the early waves' copies and score products go first
        // (the product of a unit this wave skipped, or of none at u = 0, takes zero
        // weights: a conditional product here would make the compiler spill)
        const uint32_t prev = fwd_stage_addr<(S + kStages - 1) % kStages>();
        fwd_values(w, (u == 0 ? st : prev) + 16384, lane);
        if (on) {
          fwd_scores(w, st, lane, scale_log2e);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) w.pb[q] = f16x8{};
        }
        issue(std::integral_constant<int, (S + 2) % kStages>{});
        if (!unit_u) return false;
      } else {
        issue(std::integral_constant<int, (S + 2) % kStages>{});
        if (!unit_u) return false;
        if (on) {
          fwd_scores(w, st, lane, scale_log2e);
          fwd_values(w, st + 16384, lane);
        }
      }
      return true;
    };

#pragma unroll
    for (int q = 0; q < 4; ++q) w.pb[q] = f16x8{};

    workgroup_barrier();  // every wave is done with the previous tile's stages
    issue(std::integral_constant<int, 0>{});
    issue(std::integral_constant<int, 1>{});
    for (int i = 0;; i += kStages) {
      if (!step(std::integral_constant<int, 0>{}, i)) break;
      if (!step(std::integral_constant<int, 1>{}, i + 1)) break;
      if (!step(std::integral_constant<int, 2>{}, i + 2)) break;
      if (!step(std::integral_constant<int, 3>{}, i + 3)) break;
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the trailing repeat copies
    // epilogue
    const double ltot = w.lsum + __shfl_xor(w.lsum, 32, 64);  // the two half waves' keys
    // a head whose operands left the float16 range or whose selection overflowed its
    // lists gets NaN outputs
    const bool poisoned =
        (flags[h] & (PRISM_FLAG_QKV_RANGE | PRISM_FLAG_SELECTION_OVERFLOW)) != 0u;
    const float inv = (float)(1.0 / ltot);
    const int prow = row0 + l32;
    const int token = perm[(size_t)h * N + prow];
    uint16_t *orow = out + ((size_t)token * heads + h) * dio;
    float *frow = o32p + ((size_t)h * N + prow) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int d0 = 32 * dt + 8 * v4 + 4 * hh;
        const float a0 = w.o[dt][4 * v4 + 0] * inv, a1 = w.o[dt][4 * v4 + 1] * inv,
                    a2 = w.o[dt][4 * v4 + 2] * inv, a3 = w.o[dt][4 * v4 + 3] * inv;
        uint32_t lo = (uint32_t)f32_to_bf16(a0) | ((uint32_t)f32_to_bf16(a1) << 16);
        uint32_t hi = (uint32_t)f32_to_bf16(a2) | ((uint32_t)f32_to_bf16(a3) << 16);
        u32x4 fb = __builtin_bit_cast(u32x4, f32x4{a0, a1, a2, a3});
        if (poisoned) {
          lo = hi = kNaNbf16x2;
          fb = u32x4{kNaNf32, kNaNf32, kNaNf32, kNaNf32};
        }
        // a 64-channel head keeps its padded channels (zero) in the float32 copy only
        if (32 * dt < dio) *reinterpret_cast<u32x2 *>(orow + d0) = u32x2{lo, hi};
        *reinterpret_cast<u32x4 *>(frow + d0) = fb;
      }
    const float lse = (float)(((double)w.m - kPShift + log2(ltot)) * 0.69314718055994530942);
    const uint32_t lbits = poisoned ? kNaNf32 : __float_as_uint(lse);
    if (hh == 0) {
      reinterpret_cast<uint32_t *>(lse_out)[(size_t)h * N + token] = lbits;
      reinterpret_cast<uint32_t *>(lsep)[(size_t)h * N + prow] = lbits;
    }
  }
}

// One workgroup (8 waves, one per 32 rows; two waves per SIMD, 128 KB of LDS) per query
// block, persistent over the block list.
__global__ void __launch_bounds__(NW * 64)
    attn_fwd_bf16_kernel(int N, int U, int nb_max, int heads, const int2 *__restrict__ tiles,
                         const int *__restrict__ tile_count, const uint16_t *__restrict__ qp,
                         const uint16_t *__restrict__ kp, const uint16_t *__restrict__ vp,
                         const int *__restrict__ unit_blk, const int *__restrict__ blk_start,
                         const int *__restrict__ blk_size, int Z,
                         const int *__restrict__ qt_count, const int *__restrict__ qt_ptr,
                         const int *__restrict__ qt_list, long long cap,
                         const int *__restrict__ perm, float scale_log2e, int dio,
                         const uint32_t *__restrict__ flags, uint16_t *__restrict__ out,
                         float *__restrict__ lse_out, float *__restrict__ o32p,
                         float *__restrict__ lsep) {
  // the wave index is uniform in the wave: in a scalar register, every branch on it (and on
  // the block-list cursor) is a scalar branch
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int ntiles = *tile_count;
  // the two roles run the same sequence of barriers and copies
  if (wave < NW / 2)
    fwd_waves<false>(wave, lane, N, U, nb_max, heads, tiles, ntiles, qp, kp, vp, unit_blk,
                     blk_start, blk_size, Z, qt_count, qt_ptr, qt_list, cap, perm,
                     scale_log2e, dio, flags, out, lse_out, o32p, lsep);
  else
    fwd_waves<true>(wave, lane, N, U, nb_max, heads, tiles, ntiles, qp, kp, vp, unit_blk,
                    blk_start, blk_size, Z, qt_count, qt_ptr, qt_list, cap, perm,
                    scale_log2e, dio, flags, out, lse_out, o32p, lsep);
}

// ---------------------------------------------------------------------------- float32
// Small grids in float32: one workgroup per 64-row unit, 4 threads per query row, products
// and sums carried in float64 (outputs of magnitude ~10 stay well inside 1e-4 of the exact
// result), with a per-key online softmax.
template <int D>
__global__ void __launch_bounds__(256)
    attn_fwd_f32_kernel(int N, int U, int nb_max, int heads, const float *__restrict__ qp,
                        const float *__restrict__ kp, const float *__restrict__ vp,
                        const int *__restrict__ unit_blk, const int *__restrict__ blk_start,
                        const int *__restrict__ blk_size, const int *__restrict__ sel_count,
                        const int *__restrict__ csr_ptr, const int *__restrict__ csr_col,
                        long long cap, const int *__restrict__ perm, float scale,
                        const uint32_t *__restrict__ flags, float *__restrict__ out,
                        float *__restrict__ lse_out, float *__restrict__ o32p,
                        float *__restrict__ lsep) {
  constexpr int DP = D / 4;  // dims per thread
  __shared__ float ks[kUnit][D], vs[kUnit][D];
  const int u0 = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int r = tid >> 2, part = tid & 3;
  const int blk = unit_blk[(size_t)h * U + u0];
  const int ncols = sel_count[(size_t)h * nb_max + blk];
  const int *cols = csr_col + (size_t)h * cap + csr_ptr[(size_t)h * (nb_max + 1) + blk];
  const int prow = u0 * kUnit + r;
  float qv[DP];
  double ov[DP];
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    qv[e] = qp[((size_t)h * N + prow) * D + part * DP + e];
    ov[e] = 0.0;
  }
  double m = -INFINITY, l = 0.0;
  for (int c = 0; c < ncols; ++c) {
    const int j = cols[c];
    const int us = blk_start[(size_t)h * nb_max + j] / kUnit;
    const int nu = blk_size[(size_t)h * nb_max + j] / kUnit;
    for (int u = us; u < us + nu; ++u) {
      __syncthreads();
      for (int i = tid; i < kUnit * D; i += 256) {
        ks[i / D][i % D] = kp[((size_t)h * N + (size_t)u * kUnit) * D + i];
        vs[i / D][i % D] = vp[((size_t)h * N + (size_t)u * kUnit) * D + i];
      }
      __syncthreads();
      for (int y = 0; y < kUnit; ++y) {
        double a = 0.0;
#pragma unroll
        for (int e = 0; e < DP; ++e) a += (double)qv[e] * (double)ks[y][part * DP + e];
        a += __shfl_xor(a, 1, 64);
        a += __shfl_xor(a, 2, 64);
        const double sc = a * (double)scale;
        if (sc > m) {
          const double cr = exp(m - sc);
          l *= cr;
#pragma unroll
          for (int e = 0; e < DP; ++e) ov[e] *= cr;
          m = sc;
        }
        const double p = exp(sc - m);
        l += p;
#pragma unroll
        for (int e = 0; e < DP; ++e) ov[e] += p * (double)vs[y][part * DP + e];
      }
    }
  }
  const int token = perm[(size_t)h * N + prow];
  // a head whose selection overflowed its lists gets NaN outputs
  const bool poisoned = (flags[h] & PRISM_FLAG_SELECTION_OVERFLOW) != 0u;
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    const uint32_t x = poisoned ? kNaNf32 : __float_as_uint((float)(ov[e] / l));
    reinterpret_cast<uint32_t *>(out)[((size_t)token * heads + h) * D + part * DP + e] = x;
    reinterpret_cast<uint32_t *>(o32p)[((size_t)h * N + prow) * D + part * DP + e] = x;
  }
  if (part == 0) {
    const uint32_t ls = poisoned ? kNaNf32 : __float_as_uint((float)(m + log(l)));
    reinterpret_cast<uint32_t *>(lse_out)[(size_t)h * N + token] = ls;
    reinterpret_cast<uint32_t *>(lsep)[(size_t)h * N + prow] = ls;
  }
}

hipError_t launch_attn_fwd(const Dims &d, float scale, uint8_t *ws, const Layout &L, void *o,
                           float *lse, hipStream_t s) {
  const int *unit_blk = (const int *)(ws + L.pub.unit_block);
  const int *bstart = (const int *)(ws + L.pub.block_start);
  const int *bsize = (const int *)(ws + L.pub.block_size);
  const int *cnt = (const int *)(ws + L.pub.sel_count);
  const int *cptr = (const int *)(ws + L.pub.csr_ptr);
  const int *cols = (const int *)(ws + L.pub.csr_col);
  const int *perm = (const int *)(ws + L.pub.perm);
  const uint32_t *flags = (const uint32_t *)(ws + L.pub.flags);
  float *o32p = (float *)(ws + L.o32p), *lsep = (float *)(ws + L.lsep);
  TraceScope tr(PRISM_STAGE_ATTN_FWD, s);
  if (d.dtype == PRISM_BF16) {
    const int *counters = (const int *)(ws + L.counters);
    const float sl2e = scale * 1.4426950408889634f;
    const int grid = resident_grid((const void *)attn_fwd_bf16_kernel, NW * 64, d.heads * d.U);
    hipLaunchKernelGGL(attn_fwd_bf16_kernel, dim3(grid), dim3(NW * 64), 0, s, d.N, d.U,
                       d.nb_max, d.heads, (const int2 *)(ws + L.btiles), counters + 1,
                       (const uint16_t *)(ws + L.qp), (const uint16_t *)(ws + L.kp),
                       (const uint16_t *)(ws + L.vp), unit_blk, bstart, bsize, d.Z,
                       (const int *)(ws + L.qt_count), (const int *)(ws + L.qt_ptr),
                       (const int *)(ws + L.qt_list), d.cap, perm, sl2e, d.D, flags,
                       (uint16_t *)o, lse, o32p, lsep);
  } else {
    dim3 grid(d.U, d.heads);
    if (d.D == 64)
      hipLaunchKernelGGL((attn_fwd_f32_kernel<64>), grid, dim3(256), 0, s, d.N, d.U, d.nb_max,
                         d.heads, (const float *)(ws + L.qp), (const float *)(ws + L.kp),
                         (const float *)(ws + L.vp), unit_blk, bstart, bsize, cnt, cptr, cols,
                         d.cap, perm, scale, flags, (float *)o, lse, o32p, lsep);
    else
      hipLaunchKernelGGL((attn_fwd_f32_kernel<128>), grid, dim3(256), 0, s, d.N, d.U, d.nb_max,
                         d.heads, (const float *)(ws + L.qp), (const float *)(ws + L.kp),
                         (const float *)(ws + L.vp), unit_blk, bstart, bsize, cnt, cptr, cols,
                         d.cap, perm, scale, flags, (float *)o, lse, o32p, lsep);
  }
  return hipGetLastError();
}

}  // namespace prism
