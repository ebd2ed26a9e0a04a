// attn_bwd.hip -- gradients of the block-sparse attention with the plan held constant
// (arXiv 2610.05416; nanless digest, training section: shape assignment and block
// selection are constants that pass no gradient; gradients flow only through the sparse
// attention over the selected blocks).
//
// With P_xy = exp(scale q_x.k_y - lse_x) over the key tokens y of the blocks selected for
// x's block, delta_x = do_x.o_x and dS_xy = P_xy (do_x.v_y - delta_x):
//   dv_y = sum_x P_xy do_x,  dk_y = scale sum_x dS_xy q_x,  dq_x = scale sum_y dS_xy k_y.
// Three passes, none with atomics (results are bit-reproducible):
//   prep  -- gathers dO into the permuted row-major layout and forms delta from the
//            float32 output the forward kept;
//   dK/dV -- one workgroup per key tile (pairs of waves over 32 keys, K or V rows held in
//            registers), streaming the 64-token query units of every query block that
//            selected the key block (the transposed selection lists);
//   dQ    -- one workgroup per query tile of 256 rows (32 queries per wave, Q and dO in
//            registers), streaming the selected key units as in the forward pass.
// Both MFMA passes recompute P from the stored lse and run on the float16 MFMA: the
// permuted copies are float16, the transposed operands (K^T, Q^T, dO^T) are read from
// the row-major LDS tiles with transposing LDS reads, P is fed scaled by 2^10 (as in the
// forward) and dS unscaled; outputs go straight to the tokens' original positions.
#include "prism_internal.h"

namespace prism {

constexpr int kDB = 128;


// ============================================================================ prep
// dO gathered into the permuted row-major layout (float16 for bfloat16 inputs, the operand
// type of the MFMA passes, in rows of DP = 128 with zero padding for a 64-channel head),
// delta = rowsum(dO * O) from the float32 output the forward kept; for bfloat16, delta is
// stored negated (the dP accumulators start from it) and lse as lse * log2(e) (the exp2
// argument).  For bfloat16 it also sets the head's range flags: a dO value outside the
// float16 range, or a row whose bound |dO_x| (max_y |v_y| + |o_x|) on |dS_xy| =
// |P_xy (dP_xy - delta_x)| reaches 65504 (P <= 1, |dP_xy| <= |dO_x| |v_y|, |delta_x| <=
// |dO_x| |o_x|), where the float16 dS the MFMA passes take could overflow.
template <typename T, int D, bool F16, int DP>
__global__ void __launch_bounds__(256)
    bwd_prep_kernel(int N, int heads, const int *__restrict__ perm, const T *__restrict__ dout,
                    const float *__restrict__ o32p, const float *__restrict__ lsep,
                    T *__restrict__ dop, float *__restrict__ delta, float *__restrict__ lse2,
                    const float *__restrict__ vmax, uint32_t *__restrict__ flags) {
  constexpr int VPC = 16 / (int)sizeof(T);
  constexpr int CH = D / VPC;
  constexpr int RG = 256 / CH;
  constexpr int RPT = kUnit / RG;
  static_assert(DP == D || (F16 && DP == 2 * D), "padding only for float16 copies");
  // heads vary fastest across the grid: the workgroups resident together gather every
  // head's slice of the same zones' token rows
  const int u = blockIdx.x / heads, h = blockIdx.x % heads, tid = threadIdx.x;
  const int c = tid % CH, rg = tid / CH;
  const size_t tstride = (size_t)heads * D;
  bool dout_bad = false, ds_bad = false;
  float vm = 0.f;
  if constexpr (F16) vm = vmax[h];
#pragma unroll
  for (int rr = 0; rr < RPT; ++rr) {
    const int row = rg + RG * rr;
    const size_t p = (size_t)u * kUnit + row;
    const int token = perm[(size_t)h * N + p];
    const u32x4 a =
        *reinterpret_cast<const u32x4 *>(dout + token * tstride + (size_t)h * D + c * VPC);
    const float *orow = o32p + ((size_t)h * N + p) * DP + c * VPC;
    float dot = 0.f, dd = 0.f, oo = 0.f;
    if constexpr (F16) {
      u32x4 hv;
      const f32x4 o0 = *reinterpret_cast<const f32x4 *>(orow);
      const f32x4 o1 = *reinterpret_cast<const f32x4 *>(orow + 4);
      const float ov[8] = {o0[0], o0[1], o0[2], o0[3], o1[0], o1[1], o1[2], o1[3]};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(a[e] << 16), hi = __uint_as_float(a[e] & 0xffff0000u);
        dot += lo * ov[2 * e];
        dot += hi * ov[2 * e + 1];
        dd += lo * lo + hi * hi;
        oo += ov[2 * e] * ov[2 * e] + ov[2 * e + 1] * ov[2 * e + 1];
        dout_bad |= (a[e] & 0x7fffu) >= 0x4780u || ((a[e] >> 16) & 0x7fffu) >= 0x4780u;
        hv[e] = (uint32_t)bf16_to_f16_bits((uint16_t)(a[e] & 0xffffu)) |
                ((uint32_t)bf16_to_f16_bits((uint16_t)(a[e] >> 16)) << 16);
      }
      T *drow = dop + ((size_t)h * N + p) * DP;
      __builtin_nontemporal_store(hv, reinterpret_cast<u32x4 *>(drow + c * VPC));
      if constexpr (DP > D)
        __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u},
                                    reinterpret_cast<u32x4 *>(drow + (c + CH) * VPC));
    } else {
      const f32x4 o0 = *reinterpret_cast<const f32x4 *>(orow);
#pragma unroll
      for (int e = 0; e < 4; ++e) dot += __uint_as_float(a[e]) * o0[e];
      *reinterpret_cast<u32x4 *>(dop + ((size_t)h * N + p) * D + c * VPC) = a;
    }
#pragma unroll
    for (int off = 1; off < CH; off <<= 1) dot += __shfl_xor(dot, off, 64);
    if constexpr (F16) {
#pragma unroll
      for (int off = 1; off < CH; off <<= 1) {
        dd += __shfl_xor(dd, off, 64);
        oo += __shfl_xor(oo, off, 64);
      }
      ds_bad |= sqrtf(dd) * (vm + sqrtf(oo)) >= 65504.f;
    }
    if (c == 0) {
      if constexpr (F16) {
        delta[(size_t)h * N + p] = -dot;
        lse2[(size_t)h * N + p] = lsep[(size_t)h * N + p] * 1.4426950408889634f;
      } else {
        delta[(size_t)h * N + p] = dot;
      }
    }
  }
  if constexpr (F16) {
    const bool any_dout = __any(dout_bad), any_ds = __any(ds_bad);
    if ((tid & 63) == 0 && (any_dout || any_ds))
      atomicOr(flags + h, (any_dout ? (uint32_t)PRISM_FLAG_DOUT_RANGE : 0u) |
                              (any_ds ? (uint32_t)PRISM_FLAG_DS_RANGE : 0u));
  }
}

// The backward's flags (dO range, dS bound) start clear on every backward.
__global__ void clear_bwd_flags_kernel(int heads, uint32_t *__restrict__ flags) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h < heads) flags[h] &= ~(uint32_t)(PRISM_FLAG_DOUT_RANGE | PRISM_FLAG_DS_RANGE);
}

// ============================================================================ dQ (bf16)
// One workgroup of eight waves (two per SIMD) per query tile of 256 rows (32 queries per
// wave, Q and dO rows held as B operands; a wave computes only the units its own block
// selected), streaming the key units of the tile's union list through a four-stage LDS
// ring of direct global->LDS copies, two units ahead of the one being computed: per stage
// K and V row-major [64][128] float16 (32 KB); waves 0-3 copy 16 K rows each, waves 4-7
// 16 V rows, four one-kilobyte copies per wave and unit.  Per unit a wave forms S^T and
// dP^T (K and V rows read directly), dS = P (dP - delta) as float16, and dQ^T += K^T dS^T
// (K^T through transposing reads).  As in the forward, the two waves of a SIMD run half a
// unit apart: the late wave (w >= 4) runs the dQ product of the previous unit (then issues
// its copies) before the scores of the current one, carrying dS across the barrier, so one
// wave's exponentials overlap the other's MFMAs; a wave raises its issue priority while it
// forms S and dP.
constexpr int QW = 8;
constexpr int kQStages = 4;
constexpr int kQCpw = 32 / QW;
static_assert(kQCpw == 4, "copy_rows16 issues four copies per wave and unit");
struct DqStage {
  uint8_t tile[2][16384];  // K, V
};
__shared__ __align__(256) DqStage g_dq0;
__shared__ __align__(256) DqStage g_dq1;
__shared__ __align__(256) DqStage g_dq2;
__shared__ __align__(256) DqStage g_dq3;
template <int S>
__device__ __forceinline__ DqStage &dq_stage() {
  return S == 0 ? g_dq0 : (S == 1 ? g_dq1 : (S == 2 ? g_dq2 : g_dq3));
}
// The LDS address of stage S plus an opaque zero: it keeps the per-lane addresses of all
// stages from being hoisted into registers for the whole loop
template <int S>
__device__ __forceinline__ uint32_t dq_stage_addr() {
  int z = 0;
  asm volatile("" : "+v"(z));
  return lds_addr(&dq_stage<S>()) + (uint32_t)z;
}

struct DqState {
  f16x8 qreg[8], doreg[8];
  f32x16 acc[4];
  f16x8 db[2][2];  // the current unit's dS (float16 B operands) [half][slice]
  float lse2, ndlt;
};

// Keys 32a .. 32a + 31 of the unit at LDS address st: S^T = K Q^T and dP^T = V dO^T (dP
// started at -delta; lane = query l32, register v = key 32a + (v/4)*8 + 4hh + v%4), their
// MFMAs alternating, the next k-step's K and V operands read while one runs; then
// dS = P (dP - delta) rounded to float16
__device__ __forceinline__ void dq_half(const DqState &w, uint32_t st, int a, int lane,
                                        float scale_log2e, f16x8 (&db)[2]) {
  const int l32 = lane & 31, hh = lane >> 5;
  // chunk 2kk + hh of K row 32a + l32 at r ^ (kk << 5); the V row 16 KB further
  const uint32_t r = row_base(st, 32 * a + l32) ^ (uint32_t)(hh << 4);
  f32x16 s = f32x16{}, dp;
#pragma unroll
  for (int v = 0; v < 16; ++v) dp[v] = w.ndlt;
  f16x8 x[2][2];  // [buffer][K, V]: one k-step of 16 dims per group
  auto load = [&](int buf, int kk) {
    const uint32_t ad = r ^ (uint32_t)(kk << 5);
    x[buf][0] = lds_row16(ad);
    x[buf][1] = lds_row16(ad + 16384u);
  };
  // raised issue priority while forming S and dP (the exponentials below wait for them),
  // default priority for the exponentials: the SIMD's other wave runs its MFMAs under them
  __builtin_amdgcn_s_setprio(1);
  load(0, 0);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    if (kk < 7) load((kk + 1) & 1, kk + 1);
    __builtin_amdgcn_sched_barrier(0);
    s = mfma_f16(x[kk & 1][0], w.qreg[kk], s);
    dp = mfma_f16(x[kk & 1][1], w.doreg[kk], dp);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const float p = __builtin_amdgcn_exp2f(fmaf(s[v], scale_log2e, -w.lse2));
    db[v >> 3][v & 7] = (_Float16)(p * dp[v]);
  }
}
// dS of the unit at st (both halves, built fresh: the previous unit's is dead here)
__device__ __forceinline__ void dq_scores(DqState &w, uint32_t st, int lane, float scale_log2e) {
  f16x8 db[2][2];
  dq_half(w, st, 0, lane, scale_log2e, db[0]);
  dq_half(w, st, 1, lane, scale_log2e, db[1]);
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int g = 0; g < 2; ++g) w.db[a][g] = db[a][g];
}
// dQ^T[d][q] += K^T[d][keys] dS^T[keys][q], K^T read transposed from the K tile at st
__device__ __forceinline__ void dq_update(DqState &w, uint32_t st, int lane) {
  tr_update(w.acc, tr_base(st, lane), w.db);
}

// s_waitcnt vmcnt(kQCpw) and a workgroup barrier: every wave issues exactly kQCpw copies
// per step, so the unit one step behind the newest has landed everywhere
__device__ __forceinline__ void dq_wait_one_behind() {
  wait_and_barrier<vmcnt_imm(kQCpw)>();
}

template <bool LATE>
__device__ __forceinline__ void dq_waves(
    int wave, int lane, int N, int U, int nb_max, int heads, const int2 *__restrict__ tiles,
    int ntiles, const uint16_t *__restrict__ qp, const uint16_t *__restrict__ kp,
    const uint16_t *__restrict__ vp, const uint16_t *__restrict__ dop,
    const float *__restrict__ lse2, const float *__restrict__ ndelta,
    const int *__restrict__ unit_blk, const int *__restrict__ blk_start,
    const int *__restrict__ blk_size, int Z, const int *__restrict__ qt_count,
    const int *__restrict__ qt_ptr, const int *__restrict__ qt_list, long long cap,
    const int *__restrict__ perm, float scale, float scale_log2e, int dio,
    const uint32_t *__restrict__ flags, uint16_t *__restrict__ dq) {
  const int l32 = lane & 31, hh = lane >> 5;
  // copies of this wave: K rows 16w.. (early waves) or V rows 16(w-4).. (late waves)
  const int wq = wave & (QW / 2 - 1);
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
    BlockUnits<true> pre;
    pre.init(qt_list + (size_t)h * cap + qt_ptr[(size_t)h * (2 * Z + 1) + qslot],
             qt_count[(size_t)h * 2 * Z + qslot], bs, bz, lane, blk);
    const int row0 = u0 * kUnit + wave * 32;
    DqState w;
    {
      const uint16_t *qr = qp + ((size_t)h * N + row0 + l32) * kDB + 8 * hh;
      const uint16_t *dr = dop + ((size_t)h * N + row0 + l32) * kDB + 8 * hh;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        w.qreg[kk] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(qr + 16 * kk));
        w.doreg[kk] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(dr + 16 * kk));
      }
      w.lse2 = lse2[(size_t)h * N + row0 + l32];
      w.ndlt = ndelta[(size_t)h * N + row0 + l32];
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) w.acc[dt] = f32x16{};
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int q = 0; q < 2; ++q) w.db[a][q] = f16x8{};
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // rows and cursor window in before any copy

    const uint8_t *hbase = csrc + (size_t)h * N * kDB * 2;
    int issued = 0;
    bool pending = true;
    int smask[kQStages];  // the entry mask of the unit in each stage
    // kQCpw copies per step; past the end of the list they repeat the last unit into a
    // stage no step reads any more (drained before the next tile)
    auto issue = [&](auto stage_tag) {
      constexpr int X = decltype(stage_tag)::value;
      const uint8_t *src = hbase + (size_t)pre.unit() * kUnit * kDB * 2;
      copy_rows16(src, c0, reinterpret_cast<uint8_t *>(&dq_stage<X>()) + cdst);
      smask[X] = pre.mask;
      if (pending) {
        ++issued;
        pending = pre.next();
      }
    };
    // step u (stage S = u mod 4): wait for unit u (u + 1 stays in flight), refill the stage
    // of unit u - 2 with unit u + 2, compute the units this wave's block selected.  One step
    // past the last unit finishes the late wave's dQ product.  Returns whether unit u
    // existed.
    auto step = [&](auto stage_tag, int u) {
      constexpr int S = decltype(stage_tag)::value;
      dq_wait_one_behind();
      // issued counts the units up to u + 1 at least, or all of them
      const bool unit_u = u < issued;
      const bool on = unit_u && ((smask[S] >> g) & 1);
      const uint32_t st = dq_stage_addr<S>();
      if constexpr (LATE) {
        // the late wave issues its copies after its dQ product, so that right after the
        // barrier the early waves' copies and score products go first
        // (the product of a unit this wave skipped, or of none at u = 0, takes zero dS: a
        // conditional product here would make the compiler spill)
        const uint32_t prev = dq_stage_addr<(S + kQStages - 1) % kQStages>();
        dq_update(w, u == 0 ? st : prev, lane);
        issue(std::integral_constant<int, (S + 2) % kQStages>{});
        if (!unit_u) return false;
        if (on) {
          dq_scores(w, st, lane, scale_log2e);
        } else {
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int q = 0; q < 2; ++q) w.db[a][q] = f16x8{};
        }
      } else {
        issue(std::integral_constant<int, (S + 2) % kQStages>{});
        if (!unit_u) return false;
        if (on) {
          dq_scores(w, st, lane, scale_log2e);
          dq_update(w, st, lane);
        }
      }
      return true;
    };

    workgroup_barrier();  // every wave is done with the previous tile's stages
    issue(std::integral_constant<int, 0>{});
    issue(std::integral_constant<int, 1>{});
    for (int i = 0;; i += kQStages) {
      if (!step(std::integral_constant<int, 0>{}, i)) break;
      if (!step(std::integral_constant<int, 1>{}, i + 1)) break;
      if (!step(std::integral_constant<int, 2>{}, i + 2)) break;
      if (!step(std::integral_constant<int, 3>{}, i + 3)) break;
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the trailing repeat copies
    const int token = perm[(size_t)h * N + row0 + l32];
    uint16_t *qrow = dq + ((size_t)token * heads + h) * dio;
    // any status flag of the head (operand range, selection overflow, dS bound): NaN
    const bool poisoned = flags[h] != 0u;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int d0 = 32 * dt + 8 * v4 + 4 * hh;
        uint32_t lo = (uint32_t)f32_to_bf16(w.acc[dt][4 * v4] * scale) |
                      ((uint32_t)f32_to_bf16(w.acc[dt][4 * v4 + 1] * scale) << 16);
        uint32_t hi = (uint32_t)f32_to_bf16(w.acc[dt][4 * v4 + 2] * scale) |
                      ((uint32_t)f32_to_bf16(w.acc[dt][4 * v4 + 3] * scale) << 16);
        if (poisoned) lo = hi = kNaNbf16x2;
        if (32 * dt < dio) *reinterpret_cast<u32x2 *>(qrow + d0) = u32x2{lo, hi};
      }
  }
}

__global__ void __launch_bounds__(QW * 64)
    attn_dq_bf16_kernel(int N, int U, int nb_max, int heads, const int2 *__restrict__ tiles,
                        const int *__restrict__ tile_count, const uint16_t *__restrict__ qp,
                        const uint16_t *__restrict__ kp, const uint16_t *__restrict__ vp,
                        const uint16_t *__restrict__ dop, const float *__restrict__ lse2,
                        const float *__restrict__ ndelta, const int *__restrict__ unit_blk,
                        const int *__restrict__ blk_start, const int *__restrict__ blk_size,
                        int Z, const int *__restrict__ qt_count,
                        const int *__restrict__ qt_ptr, const int *__restrict__ qt_list,
                        long long cap, const int *__restrict__ perm, float scale,
                        float scale_log2e, int dio, const uint32_t *__restrict__ flags,
                        uint16_t *__restrict__ dq) {
  // the wave index is uniform in the wave; the two roles run the same sequence of barriers
  // and copies
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int ntiles = *tile_count;
  if (wave < QW / 2)
    dq_waves<false>(wave, lane, N, U, nb_max, heads, tiles, ntiles, qp, kp, vp, dop, lse2,
                    ndelta, unit_blk, blk_start, blk_size, Z, qt_count, qt_ptr, qt_list, cap,
                    perm, scale, scale_log2e, dio, flags, dq);
  else
    dq_waves<true>(wave, lane, N, U, nb_max, heads, tiles, ntiles, qp, kp, vp, dop, lse2,
                   ndelta, unit_blk, blk_start, blk_size, Z, qt_count, qt_ptr, qt_list, cap,
                   perm, scale, scale_log2e, dio, flags, dq);
}

// ============================================================================ float32
// Small grids in float32 (products and sums in float64, as in the forward).
// dQ: one workgroup per 64-row query unit, 4 threads per row.
template <int D>
__global__ void __launch_bounds__(256)
    attn_dq_f32_kernel(int N, int U, int nb_max, int heads, const float *__restrict__ qp,
                       const float *__restrict__ kp, const float *__restrict__ vp,
                       const float *__restrict__ dop, const float *__restrict__ lsep,
                       const float *__restrict__ delta, const int *__restrict__ unit_blk,
                       const int *__restrict__ blk_start, const int *__restrict__ blk_size,
                       const int *__restrict__ sel_count, const int *__restrict__ csr_ptr,
                       const int *__restrict__ csr_col, long long cap,
                       const int *__restrict__ perm, float scale,
                       const uint32_t *__restrict__ flags, float *__restrict__ dq) {
  constexpr int DP = D / 4;
  __shared__ float ks[kUnit][D], vs[kUnit][D];
  const int u0 = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int r = tid >> 2, part = tid & 3;
  const int blk = unit_blk[(size_t)h * U + u0];
  const int ncols = sel_count[(size_t)h * nb_max + blk];
  const int *cols = csr_col + (size_t)h * cap + csr_ptr[(size_t)h * (nb_max + 1) + blk];
  const int prow = u0 * kUnit + r;
  float qv[DP], dov[DP];
  double acc[DP];
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    qv[e] = qp[((size_t)h * N + prow) * D + part * DP + e];
    dov[e] = dop[((size_t)h * N + prow) * D + part * DP + e];
    acc[e] = 0.0;
  }
  const double l = lsep[(size_t)h * N + prow], dl = delta[(size_t)h * N + prow];
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
        double a = 0.0, b = 0.0;
#pragma unroll
        for (int e = 0; e < DP; ++e) {
          a += (double)qv[e] * (double)ks[y][part * DP + e];
          b += (double)dov[e] * (double)vs[y][part * DP + e];
        }
        a += __shfl_xor(a, 1, 64);
        a += __shfl_xor(a, 2, 64);
        b += __shfl_xor(b, 1, 64);
        b += __shfl_xor(b, 2, 64);
        const double p = exp(a * (double)scale - l);
        const double ds = p * (b - dl);
#pragma unroll
        for (int e = 0; e < DP; ++e) acc[e] += ds * (double)ks[y][part * DP + e];
      }
    }
  }
  const int token = perm[(size_t)h * N + prow];
  const bool poisoned = flags[h] != 0u;
#pragma unroll
  for (int e = 0; e < DP; ++e)
    reinterpret_cast<uint32_t *>(dq)[((size_t)token * heads + h) * D + part * DP + e] =
        poisoned ? kNaNf32 : __float_as_uint((float)(acc[e] * scale));
}

// dK/dV: one workgroup per 64-key unit, 4 threads per key row, over the transposed lists.
template <int D>
__global__ void __launch_bounds__(256)
    attn_dkdv_f32_kernel(int N, int U, int nb_max, int heads, const float *__restrict__ qp,
                         const float *__restrict__ kp, const float *__restrict__ vp,
                         const float *__restrict__ dop, const float *__restrict__ lsep,
                         const float *__restrict__ delta, const int *__restrict__ unit_blk,
                         const int *__restrict__ blk_start, const int *__restrict__ blk_size,
                         const int *__restrict__ csc_count, const int *__restrict__ csc_ptr,
                         const int *__restrict__ csc_row, long long cap,
                         const int *__restrict__ perm, float scale,
                         const uint32_t *__restrict__ flags, float *__restrict__ dk,
                         float *__restrict__ dv) {
  constexpr int DP = D / 4;
  __shared__ float qs[kUnit][D], ds_[kUnit][D];
  const int u0 = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int r = tid >> 2, part = tid & 3;
  const int jblk = unit_blk[(size_t)h * U + u0];
  const int nq = csc_count[(size_t)h * nb_max + jblk];
  const int *qlist = csc_row + (size_t)h * cap + csc_ptr[(size_t)h * (nb_max + 1) + jblk];
  const int krow = u0 * kUnit + r;
  float kv[DP], vv[DP];
  double gk[DP], gv[DP];
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    kv[e] = kp[((size_t)h * N + krow) * D + part * DP + e];
    vv[e] = vp[((size_t)h * N + krow) * D + part * DP + e];
    gk[e] = gv[e] = 0.0;
  }
  for (int c = 0; c < nq; ++c) {
    const int i = qlist[c];
    const int us = blk_start[(size_t)h * nb_max + i] / kUnit;
    const int nu = blk_size[(size_t)h * nb_max + i] / kUnit;
    for (int u = us; u < us + nu; ++u) {
      __syncthreads();
      for (int x = tid; x < kUnit * D; x += 256) {
        qs[x / D][x % D] = qp[((size_t)h * N + (size_t)u * kUnit) * D + x];
        ds_[x / D][x % D] = dop[((size_t)h * N + (size_t)u * kUnit) * D + x];
      }
      __syncthreads();
      for (int x = 0; x < kUnit; ++x) {
        const size_t px = (size_t)h * N + (size_t)u * kUnit + x;
        double a = 0.0, b = 0.0;
#pragma unroll
        for (int e = 0; e < DP; ++e) {
          a += (double)kv[e] * (double)qs[x][part * DP + e];
          b += (double)vv[e] * (double)ds_[x][part * DP + e];
        }
        a += __shfl_xor(a, 1, 64);
        a += __shfl_xor(a, 2, 64);
        b += __shfl_xor(b, 1, 64);
        b += __shfl_xor(b, 2, 64);
        const double p = exp(a * (double)scale - (double)lsep[px]);
        const double g = p * (b - (double)delta[px]);
#pragma unroll
        for (int e = 0; e < DP; ++e) {
          gv[e] += p * (double)ds_[x][part * DP + e];
          gk[e] += g * (double)qs[x][part * DP + e];
        }
      }
    }
  }
  const int token = perm[(size_t)h * N + krow];
  const bool poisoned = flags[h] != 0u;
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    const size_t at = ((size_t)token * heads + h) * D + part * DP + e;
    reinterpret_cast<uint32_t *>(dk)[at] =
        poisoned ? kNaNf32 : __float_as_uint((float)(gk[e] * scale));
    reinterpret_cast<uint32_t *>(dv)[at] = poisoned ? kNaNf32 : __float_as_uint((float)gv[e]);
  }
}

// ============================================================================ launcher
hipError_t launch_attn_bwd(const Dims &d, float scale, uint8_t *ws, const Layout &L,
                           const void *dout, void *dq, void *dk, void *dv, hipStream_t s) {
  const int *perm = (const int *)(ws + L.pub.perm);
  const int *unit_blk = (const int *)(ws + L.pub.unit_block);
  const int *bstart = (const int *)(ws + L.pub.block_start);
  const int *bsize = (const int *)(ws + L.pub.block_size);
  const int *cnt = (const int *)(ws + L.pub.sel_count);
  const int *cptr = (const int *)(ws + L.pub.csr_ptr);
  const int *cols = (const int *)(ws + L.pub.csr_col);
  const int *tcnt = (const int *)(ws + L.pub.csc_count);
  const int *tptr = (const int *)(ws + L.pub.csc_ptr);
  const int *trows = (const int *)(ws + L.pub.csc_row);
  uint32_t *flags = (uint32_t *)(ws + L.pub.flags);
  const float *vmax = (const float *)(ws + L.vmax);
  float *delta = (float *)(ws + L.delta), *lse2 = (float *)(ws + L.lse2);
  const float *lsep = (const float *)(ws + L.lsep), *o32p = (const float *)(ws + L.o32p);
  dim3 ugrid(d.U, d.heads);
  dim3 pgrid(d.U * d.heads);  // bwd_prep: one-dimensional, heads fastest
  if (d.dtype == PRISM_BF16) {
    typedef uint16_t T;
    {
      TraceScope tr(PRISM_STAGE_BWD_PREP, s);
      hipLaunchKernelGGL(clear_bwd_flags_kernel, dim3((d.heads + 255) / 256), dim3(256), 0, s,
                         d.heads, flags);
      if (d.D == 64)
        hipLaunchKernelGGL((bwd_prep_kernel<T, 64, true, 128>), pgrid, dim3(256), 0, s, d.N,
                           d.heads, perm, (const T *)dout, o32p, lsep, (T *)(ws + L.dop), delta,
                           lse2, vmax, flags);
      else
        hipLaunchKernelGGL((bwd_prep_kernel<T, 128, true, 128>), pgrid, dim3(256), 0, s, d.N,
                           d.heads, perm, (const T *)dout, o32p, lsep, (T *)(ws + L.dop), delta,
                           lse2, vmax, flags);
    }
    const int *counters = (const int *)(ws + L.counters);
    const float sl2e = scale * 1.4426950408889634f;
    const int maxt = d.heads * d.U;
    const T *qp = (const T *)(ws + L.qp), *kp = (const T *)(ws + L.kp),
            *vp = (const T *)(ws + L.vp), *dop = (const T *)(ws + L.dop);
    const int2 *tiles = (const int2 *)(ws + L.tiles), *btiles = (const int2 *)(ws + L.btiles);
    {
      TraceScope tr(PRISM_STAGE_BWD_DKDV, s);
      (void)launch_dkdv_bf16(maxt, s, d.N, d.U, d.nb_max, d.heads, tiles, counters, qp, kp,
                             vp, dop, lse2, delta, unit_blk, bstart, bsize, tcnt, tptr, trows,
                             d.cap, perm, scale, sl2e, d.D, flags, (T *)dk, (T *)dv);
    }
    {
      TraceScope tr(PRISM_STAGE_BWD_DQ, s);
      const int grid = resident_grid((const void *)attn_dq_bf16_kernel, QW * 64, maxt);
      hipLaunchKernelGGL(attn_dq_bf16_kernel, dim3(grid), dim3(QW * 64), 0, s, d.N, d.U,
                         d.nb_max, d.heads, btiles, counters + 1, qp, kp, vp, dop, lse2, delta,
                         unit_blk, bstart, bsize, d.Z, (const int *)(ws + L.qt_count),
                         (const int *)(ws + L.qt_ptr), (const int *)(ws + L.qt_list), d.cap,
                         perm, scale, sl2e, d.D, flags, (T *)dq);
    }
  } else {
    typedef float T;
    TraceScope tr(PRISM_STAGE_BWD_DKDV, s);
    const T *qp = (const T *)(ws + L.qp), *kp = (const T *)(ws + L.kp),
            *vp = (const T *)(ws + L.vp), *dop = (const T *)(ws + L.dop);
#define PRISM_BWD_F32(D)                                                                      \
  hipLaunchKernelGGL((bwd_prep_kernel<T, D, false, D>), pgrid, dim3(256), 0, s, d.N, d.heads,   \
                     perm, (const T *)dout, o32p, lsep, (T *)(ws + L.dop), delta, nullptr,     \
                     nullptr, flags);                                                          \
  hipLaunchKernelGGL((attn_dq_f32_kernel<D>), ugrid, dim3(256), 0, s, d.N, d.U, d.nb_max,      \
                     d.heads, qp, kp, vp, dop, lsep, delta, unit_blk, bstart, bsize, cnt,      \
                     cptr, cols, d.cap, perm, scale, flags, (T *)dq);                          \
  hipLaunchKernelGGL((attn_dkdv_f32_kernel<D>), ugrid, dim3(256), 0, s, d.N, d.U, d.nb_max,    \
                     d.heads, qp, kp, vp, dop, lsep, delta, unit_blk, bstart, bsize, tcnt,     \
                     tptr, trows, d.cap, perm, scale, flags, (T *)dk, (T *)dv)
    if (d.D == 64) {
      PRISM_BWD_F32(64);
    } else {
      PRISM_BWD_F32(128);
    }
#undef PRISM_BWD_F32
  }
  return hipGetLastError();
}

}  // namespace prism
