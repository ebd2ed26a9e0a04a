// attn_bwd_dkdv.hip -- dK and dV of the block-sparse attention (bfloat16 path), key-major
// over the transposed selection lists.  Same method as attn_bwd.hip (digest, training
// section: the plan is constant; gradients flow only through the selected blocks), in a
// translation unit of its own because its register budget is best served by the default
// MFMA register form.
#include <type_traits>

#include "prism_internal.h"

namespace prism {

namespace {
constexpr int kDB = 128;
}  // namespace

// ============================================================================ dK / dV (bf16)
// One workgroup of eight waves (two per SIMD) per 128-key tile (a 256-key block is two
// tiles), in four pairs; pair w owns keys 32w .. 32w + 31 of the tile.  (The 64-key tiles of
// 64-token blocks run in a second launch in which pair w owns keys 32 (w % 2) .. + 31 and
// one half of each unit's query rows, below.)  Over the 64-token query units of every query
// block that selected the key block:
//   * the P wave (w < 4) holds K as B operand, forms S = Q K^T and P = exp(S - lse),
//     hands P to its partner through LDS (float32) and accumulates dV^T += dO^T P;
//   * the dS wave (w >= 4) holds V as B operand, forms dP = dO V^T and accumulates
//     dK^T += Q^T dS with dS = P (dP - delta).
// The two waves of a pair share a SIMD.  Each unit has two barriers: after the first the
// P wave forms S and P (its lse values read before the S product, so the exponentials never
// wait on LDS) while the dS wave forms dP and then the dK product of the previous unit (the
// first operands of which it reads before dP), so the P wave's exponentials overlap MFMAs;
// after the second (P published) the P wave runs its dV product while the dS wave forms dS,
// which it keeps for the next unit.  One step past the last unit finishes the last dK
// product.
//
// Query units stream through a three-stage LDS ring filled by direct global->LDS copies
// (global_load_lds_dwordx4: lane l of one instruction lands at +16*l, so the XOR swizzle
// is applied by choosing which source chunk each lane fetches).  The copies of unit u + 2
// are issued after the second barrier of unit u, once the dS wave is done with the stage
// of unit u - 1.  Per stage: Q and dO row-major [64][128] float16 (Q^T and dO^T are read
// from them with transposing LDS reads), lse and delta [64].  Waves 0-3 copy 16 Q rows
// each, waves 4-7 16 dO rows (four one-kilobyte copies per unit), waves 0 and 1 also one
// 256-byte vector.
constexpr int NW = 8;
constexpr int kStages = 3;
constexpr uint32_t kDOTile = 16384;  // byte offset of the dO tile in a stage
constexpr uint32_t kVecs = 32768;    // byte offset of the lse and delta vectors

// The stages are distinct LDS objects and the unit loop is unrolled by three, so every
// LDS read names its stage statically.  256-byte alignment lets the swizzled addresses be
// formed by XOR (row_base, tr_base).
struct Stage {
  uint8_t tile[2][16384];  // Q, dO (row-major float16)
  float vec[2][kUnit];     // lse * log2(e), -delta
};
__shared__ __align__(256) Stage g_stage0;
__shared__ __align__(256) Stage g_stage1;
__shared__ __align__(256) Stage g_stage2;
// P (float32) of the current unit per pair, in the P wave's C layout:
// [pair][half][register group of 4][lane]
__shared__ __align__(16) f32x4 g_pex[4][2][4][64];
template <int S>
__device__ __forceinline__ Stage &stage() {
  return S == 0 ? g_stage0 : (S == 1 ? g_stage1 : g_stage2);
}
// The LDS address of stage S plus an opaque zero: it keeps the per-lane addresses of all
// stages from being hoisted into registers for the whole loop
template <int S>
__device__ __forceinline__ uint32_t stage_addr() {
  int z = 0;
  asm volatile("" : "+v"(z));
  return lds_addr(&stage<S>()) + (uint32_t)z;
}
__device__ __forceinline__ f32x4 lds_f32x4(uint32_t addr) {
  return *(const __attribute__((address_space(3))) f32x4 *)(uintptr_t)addr;
}

// acc[a] (C layout: lane = key l32, register v = query 32a + (v/4)*8 + 4hh + v%4) += the
// 32 queries of half a of the row-major [64][128] float16 tile at LDS address t times the
// wave's B operand, for both halves: the two accumulators alternate, and the operands of
// the next group of four MFMAs are read while the current group runs
__device__ __forceinline__ void both_halves_product(f32x16 (&acc)[2], uint32_t t,
                                                    const f16x8 (&b)[8], int l32, int hh) {
  // chunk 2kk + hh of row l32 at r ^ (kk << 5); row 32 + l32 8 KB further
  const uint32_t r = row_base(t, l32) ^ (uint32_t)(hh << 4);
  f16x8 x[2][2][2];  // [buffer][a][e]
  auto load = [&](int buf, int grp) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int e = 0; e < 2; ++e)
        x[buf][a][e] = lds_row16((r ^ (uint32_t)((2 * grp + e) << 5)) + 8192u * a);
  };
  load(0, 0);
#pragma unroll
  for (int grp = 0; grp < 4; ++grp) {
    if (grp < 3) load((grp + 1) & 1, grp + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int a = 0; a < 2; ++a) acc[a] = mfma_f16(x[grp & 1][a][e], b[2 * grp + e], acc[a]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The state of one wave of a pair: its B operand rows (K for the P wave, V for the dS
// wave), its accumulators (dV^T or dK^T) and the values it carries: the P wave P * 2^10
// as float16 (the operand of the dV product) [half][slice]; the dS wave dP - delta in
// float32 [half] and the previous unit's dS as float16 [half][slice].
struct PState {
  f16x8 breg[8];
  f32x16 acc[4];
  f16x8 x[2][2];
};
struct DState {
  f16x8 breg[8];
  f32x16 acc[4];
  f32x16 dp[2];
  f16x8 db[2][2];
};

// P wave, before the mid-unit barrier: S and P for both halves, P published; st is the
// stage's LDS address
__device__ __forceinline__ void p_first(PState &w, uint32_t st, int pair, int lane,
                                        float scale_log2e) {
  const int l32 = lane & 31, hh = lane >> 5;
  // the lse values of the lane's 32 queries are read before the product, so that the
  // exponentials below never wait on LDS
  f32x4 lv[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4)
      lv[a][v4] = lds_f32x4(st + kVecs + 4u * (32 * a + 8 * v4 + 4 * hh));
  f32x16 sacc[2] = {f32x16{}, f32x16{}};
  both_halves_product(sacc, st, w.breg, l32, hh);
  f16x8 x[2][2];  // built fresh: the previous unit's weights are dead here
#pragma unroll
  for (int a = 0; a < 2; ++a) {
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const f32x4 l4 = lv[a][v4];
      f32x4 p4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = 4 * v4 + e;
        p4[e] = __builtin_amdgcn_exp2f(fmaf(sacc[a][v], scale_log2e, -l4[e]));
        x[a][v >> 3][v & 7] = (_Float16)(p4[e] * kPScale);
      }
      g_pex[pair][a][v4][lane] = p4;
    }
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int g = 0; g < 2; ++g) w.x[a][g] = x[a][g];
}
// P wave, after the barrier: dV^T += dO^T (P * 2^10)
__device__ __forceinline__ void p_second(PState &w, uint32_t st, int lane) {
  tr_update(w.acc, tr_base(st + kDOTile, lane), w.x);
}
// dS wave, before the barrier: dP, started at -delta
__device__ __forceinline__ void d_dp(DState &w, uint32_t st, int lane) {
  const int l32 = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const f32x4 d4 = lds_f32x4(st + kVecs + 4u * (kUnit + 32 * a + 8 * v4 + 4 * hh));
#pragma unroll
      for (int e = 0; e < 4; ++e) w.dp[a][4 * v4 + e] = d4[e];
    }
  both_halves_product(w.dp, st + kDOTile, w.breg, l32, hh);
}
// dS wave: the transposed-read base of the Q tile at st and the A operands of the first
// 16-row slice of the dK product, read before the dP product so that the dK product does
// not start on an LDS round trip
__device__ __forceinline__ TrBase d_dk_first(uint32_t st, int lane, f16x8 (&first)[4]) {
  const TrBase tb = tr_base(st, lane);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) first[dt] = tr_read(tb, 0, 32 * dt);
  return tb;
}
// dS wave: dK^T += Q^T dS with the carried dS (Q^T through tb, its first slice in first);
// per slice the four d-tiles' accumulators are independent, and the next slice's operands
// are read while one runs
__device__ __forceinline__ void d_dk(DState &w, const TrBase &tb, const f16x8 (&first)[4]) {
  f16x8 ta[2][4];  // [buffer][dt]
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) ta[0][dt] = first[dt];
#pragma unroll
  for (int sl = 0; sl < 4; ++sl) {
    if (sl < 3)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) ta[(sl + 1) & 1][dt] = tr_read(tb, 16 * (sl + 1), 32 * dt);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      w.acc[dt] = mfma_f16(ta[sl & 1][dt], w.db[sl >> 1][sl & 1], w.acc[dt]);
    __builtin_amdgcn_sched_barrier(0);
  }
}
// dS wave, after the barrier: dS = P (dP - delta) in float32, rounded once to float16
__device__ __forceinline__ void d_ds(DState &w, int pair, int lane) {
  // all eight reads of P are in flight together, then the products
  f32x4 pv[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) pv[a][v4] = g_pex[pair][a][v4][lane];
  __builtin_amdgcn_sched_barrier(0);
  f16x8 db[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const f32x4 p4 = pv[a][v4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = 4 * v4 + e;
        db[a][v >> 3][v & 7] = (_Float16)(p4[e] * w.dp[a][v]);
      }
    }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int g = 0; g < 2; ++g) w.db[a][g] = db[a][g];
}

// ---- 64-key tiles (a launch of their own): the four pairs split the tile into 32 keys x
// one half of each unit's queries.  Pair p owns keys 32 (p % 2) .. + 31 and query half
// a = p / 2 (rows 32a .. 32a + 31 of every unit), so every wave has work; the two pairs of a
// key half add their accumulators at the end of the tile.  A wave keeps one half's values in
// the [0] entries of its state.

// acc (C layout, lane = key l32) += the 32 query rows of the row-major float16 tile at LDS
// address t (the half's first row) times the wave's B operand; the next group's operands
// are read while one runs
__device__ __forceinline__ void half_product(f32x16 &acc, uint32_t t, const f16x8 (&b)[8],
                                             int l32, int hh) {
  const uint32_t r = row_base(t, l32) ^ (uint32_t)(hh << 4);
  f16x8 x[2][2];  // [buffer][e]
  auto load = [&](int buf, int grp) {
#pragma unroll
    for (int e = 0; e < 2; ++e) x[buf][e] = lds_row16(r ^ (uint32_t)((2 * grp + e) << 5));
  };
  load(0, 0);
#pragma unroll
  for (int grp = 0; grp < 4; ++grp) {
    if (grp < 3) load((grp + 1) & 1, grp + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < 2; ++e) acc = mfma_f16(x[grp & 1][e], b[2 * grp + e], acc);
    __builtin_amdgcn_sched_barrier(0);
  }
}
// acc[dt] += T^T[d][k] X[k][j] over the 32 rows k of one half (two 16-row slices) of the
// tile whose transposed-read base is tb (taken at the half's first row); first holds the
// first slice's operands
__device__ __forceinline__ void half_tr_update(f32x16 (&acc)[4], const TrBase &tb,
                                               const f16x8 (&x)[2], const f16x8 (&first)[4]) {
  f16x8 second[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) second[dt] = tr_read(tb, 16, 32 * dt);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = mfma_f16(first[dt], x[0], acc[dt]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = mfma_f16(second[dt], x[1], acc[dt]);
}
// P wave of a 64-key tile, before the barrier: S and P for half a, published
__device__ __forceinline__ void ps_first(PState &w, uint32_t st, int pair, int a, int lane,
                                         float scale_log2e) {
  const int l32 = lane & 31, hh = lane >> 5;
  f32x4 lv[4];
#pragma unroll
  for (int v4 = 0; v4 < 4; ++v4)
    lv[v4] = lds_f32x4(st + kVecs + 4u * (32 * a + 8 * v4 + 4 * hh));
  f32x16 sacc = f32x16{};
  half_product(sacc, st + 8192u * (uint32_t)a, w.breg, l32, hh);
  f16x8 x[2];
#pragma unroll
  for (int v4 = 0; v4 < 4; ++v4) {
    f32x4 p4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = 4 * v4 + e;
      p4[e] = __builtin_amdgcn_exp2f(fmaf(sacc[v], scale_log2e, -lv[v4][e]));
      x[v >> 3][v & 7] = (_Float16)(p4[e] * kPScale);
    }
    g_pex[pair][a][v4][lane] = p4;
  }
  w.x[0][0] = x[0];
  w.x[0][1] = x[1];
}
// P wave of a 64-key tile, after the barrier: dV^T += dO^T (P * 2^10) over half a
__device__ __forceinline__ void ps_second(PState &w, uint32_t st, int a, int lane) {
  const TrBase tb = tr_base(st + kDOTile + 8192u * (uint32_t)a, lane);
  f16x8 first[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) first[dt] = tr_read(tb, 0, 32 * dt);
  half_tr_update(w.acc, tb, w.x[0], first);
}
// dS wave of a 64-key tile: dP for half a, started at -delta
__device__ __forceinline__ void ds_dp(DState &w, uint32_t st, int a, int lane) {
  const int l32 = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int v4 = 0; v4 < 4; ++v4) {
    const f32x4 d4 = lds_f32x4(st + kVecs + 4u * (kUnit + 32 * a + 8 * v4 + 4 * hh));
#pragma unroll
    for (int e = 0; e < 4; ++e) w.dp[0][4 * v4 + e] = d4[e];
  }
  half_product(w.dp[0], st + kDOTile + 8192u * (uint32_t)a, w.breg, l32, hh);
}
// dS wave of a 64-key tile: the transposed-read base of half a of the Q tile at st and the
// first slice's operands of the dK product (read before dP)
__device__ __forceinline__ TrBase ds_dk_first(uint32_t st, int a, int lane,
                                              f16x8 (&first)[4]) {
  const TrBase tb = tr_base(st + 8192u * (uint32_t)a, lane);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) first[dt] = tr_read(tb, 0, 32 * dt);
  return tb;
}
// dS wave of a 64-key tile, after the barrier: dS = P (dP - delta) for half a
__device__ __forceinline__ void ds_ds(DState &w, int pair, int a, int lane) {
  f32x4 pv[4];
#pragma unroll
  for (int v4 = 0; v4 < 4; ++v4) pv[v4] = g_pex[pair][a][v4][lane];
  __builtin_amdgcn_sched_barrier(0);
  f16x8 db[2];
#pragma unroll
  for (int v4 = 0; v4 < 4; ++v4)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = 4 * v4 + e;
      db[v >> 3][v & 7] = (_Float16)(pv[v4][e] * w.dp[0][v]);
    }
  w.db[0][0] = db[0];
  w.db[0][1] = db[1];
}

// P published: the P waves' LDS writes are complete before the barrier
__device__ __forceinline__ void publish_sync() { wait_and_barrier<kLgkm0>(); }

template <bool PW, bool SPLIT>
__device__ __forceinline__ void dkdv_waves(
    int wave, int lane, int N, int U, int nb_max, int heads, const int2 *__restrict__ tiles,
    const int *__restrict__ tile_count, int ntiles, const uint16_t *__restrict__ qp,
    const uint16_t *__restrict__ kp, const uint16_t *__restrict__ vp,
    const uint16_t *__restrict__ dop, const float *__restrict__ lse2,
    const float *__restrict__ ndelta, const int *__restrict__ unit_blk,
    const int *__restrict__ blk_start, const int *__restrict__ blk_size,
    const int *__restrict__ csc_count, const int *__restrict__ csc_ptr,
    const int *__restrict__ csc_row, long long cap, const int *__restrict__ perm, float scale,
    float scale_log2e, int dio, const uint32_t *__restrict__ flags, uint16_t *__restrict__ dk,
    uint16_t *__restrict__ dv) {
  const int l32 = lane & 31, hh = lane >> 5;
  const int pair = wave & 3;
  // copies of this wave: Q rows 16w.. (P waves) or dO rows 16(w-4).. (dS waves); waves 0
  // and 1 also copy the lse and delta vectors
  const uint8_t *tsrc = reinterpret_cast<const uint8_t *>(PW ? qp : dop);
  const int cdst = (PW ? 0 : 16384) + pair * 4096;
  const uint32_t c0 = copy_offset(16 * pair, lane);  // this lane's source offset in the unit
  const bool vcopy = wave < 2;
  const float *vsrc = wave == 1 ? ndelta : lse2;

  // the two halves of a 256-token key block (tiles 2p and 2p + 1 of the first npaired) go
  // to slots j and j + 8 of a group of 16, i.e. to workgroups b and b + 8, which sit on the
  // same XCD (workgroups are dealt to the eight XCDs in turn)
  // (the 64-key tiles follow the others in the list)
  const int npaired = SPLIT ? 0 : __builtin_amdgcn_readfirstlane(tile_count[2]) & ~15;
  const int tbase = SPLIT ? __builtin_amdgcn_readfirstlane(tile_count[0]) : 0;
  for (int slot = blockIdx.x; slot < ntiles; slot += gridDim.x) {
    int t;
    if constexpr (SPLIT) {
      // the eight tiles of a zone (neighbouring key blocks, similar query lists) go to
      // workgroups of one XCD: in each full group of 64, tile 8z + s to slot 8s + z
      const int within = slot & 63;
      t = tbase + (slot < (ntiles & ~63) ? (slot & ~63) + 8 * (within & 7) + (within >> 3)
                                          : slot);
    } else {
      const int j = slot & 15;
      t = slot < npaired ? (slot & ~15) + 2 * (j & 7) + (j >> 3) : slot;
    }
    const int2 tl = tiles[t];
    const int h = __builtin_amdgcn_readfirstlane(tl.x);
    const int ty = __builtin_amdgcn_readfirstlane(tl.y);
    // 128-key tiles (two per 256-key block), 64-key tiles for 64-key blocks
    const int u0 = ty & (kTile64 - 1), rows = (ty & kTile64) ? kUnit : 2 * kUnit;
    const bool active = SPLIT || pair * 32 < rows;
    const int half = SPLIT ? pair >> 1 : 0;  // 64-key tiles: this pair's query half
    const int jblk = unit_blk[(size_t)h * U + u0];
    const int nq = __builtin_amdgcn_readfirstlane(csc_count[(size_t)h * nb_max + jblk]);
    const int *qlist = csc_row + (size_t)h * cap + csc_ptr[(size_t)h * (nb_max + 1) + jblk];
    const int *bs = blk_start + (size_t)h * nb_max, *bz = blk_size + (size_t)h * nb_max;
    // the pair's 32 keys: K^T (P wave) or V^T (dS wave) as B operand (lane = key, 8 dims
    // per k-step)
    const int key0 = u0 * kUnit + (SPLIT ? pair & 1 : pair) * 32;
    std::conditional_t<PW, PState, DState> w;
    if (active) {
      const uint16_t *br = (PW ? kp : vp) + ((size_t)h * N + key0 + l32) * kDB + 8 * hh;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        w.breg[kk] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(br + 16 * kk));
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) w.acc[dt] = f32x16{};
    if constexpr (!PW) {
      // the dK product of the first step multiplies by zero (there is no previous unit)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int g = 0; g < 2; ++g) w.db[a][g] = f16x8{};
    }

    const size_t hb = (size_t)h * N;
    int issued = 0;
    bool pending = true;
    BlockUnits<false> pre;
    // every step issues this wave's copies: past the end of the list they repeat the last
    // unit (finite data) into a stage no step reads any more, or reads only for a result
    // it discards (drained before the next tile)
    auto issue = [&](Stage &st) {
      const int u = pre.unit();
      const uint8_t *src = tsrc + (hb + (size_t)u * kUnit) * kDB * 2;
      copy_rows16(src, c0, reinterpret_cast<uint8_t *>(&st) + cdst);
      if (vcopy) dma4(vsrc + hb + (size_t)u * kUnit, 4u * (uint32_t)lane, st.vec[wave]);
      if (pending) {
        ++issued;
        pending = pre.next();
      }
    };
    // this wave's copies of the unit one step behind the newest have landed everywhere
    auto wait_one_behind = [&]() {
      if (vcopy)
        wait_and_barrier<vmcnt_imm(5)>();
      else
        wait_and_barrier<vmcnt_imm(4)>();
    };
    // step u (stage S = u mod 3): wait for unit u; first half; barrier (P published);
    // refill the stage of unit u - 1 with unit u + 2; second half.  Returns whether unit
    // u existed.  The step after the last unit only runs the dS wave's last dK product
    // (its dP there reads the repeated copy of the last unit and is discarded).
    auto step = [&](auto stage_tag, int u) {
      constexpr int S = decltype(stage_tag)::value;
      wait_one_behind();
      const bool unit_u = u < issued;
      const uint32_t st = stage_addr<S>();
      if constexpr (PW && SPLIT) {
        if (!unit_u) return false;
        ps_first(w, st, pair, half, lane, scale_log2e);
        publish_sync();
        issue(stage<(S + 2) % kStages>());
        ps_second(w, st, half, lane);
      } else if constexpr (SPLIT) {
        {
          const uint32_t prev = stage_addr<(S + kStages - 1) % kStages>();
          f16x8 first[4];
          const TrBase tb = ds_dk_first(u == 0 ? st : prev, half, lane, first);
          ds_dp(w, st, half, lane);
          half_tr_update(w.acc, tb, w.db[0], first);
        }
        if (!unit_u) return false;
        publish_sync();
        issue(stage<(S + 2) % kStages>());
        ds_ds(w, pair, half, lane);
      } else if constexpr (PW) {
        if (!unit_u) return false;
        if (active) p_first(w, st, pair, lane, scale_log2e);
        publish_sync();
        issue(stage<(S + 2) % kStages>());
        if (active) p_second(w, st, lane);
      } else {
        if (active) {
          const uint32_t prev = stage_addr<(S + kStages - 1) % kStages>();
          f16x8 first[4];
          const TrBase tb = d_dk_first(u == 0 ? st : prev, lane, first);
          d_dp(w, st, lane);
          d_dk(w, tb, first);
        }
        if (!unit_u) return false;
        publish_sync();
        issue(stage<(S + 2) % kStages>());
        if (active) d_ds(w, pair, lane);
      }
      return true;
    };

    workgroup_barrier();  // every wave is done with the previous tile's stages
    if (nq > 0) {
      pre.init(qlist, nq, bs, bz, lane, jblk);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // K or V rows and the cursor window are in
      issue(g_stage0);
      issue(g_stage1);
      for (int i = 0;; i += kStages) {
        if (!step(std::integral_constant<int, 0>{}, i)) break;
        if (!step(std::integral_constant<int, 1>{}, i + 1)) break;
        if (!step(std::integral_constant<int, 2>{}, i + 2)) break;
      }
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the trailing repeat copies
    }
    if constexpr (SPLIT) {
      // the pairs of query half 1 hand their accumulators to those of half 0 (same keys)
      // through the stage tiles, which no wave reads or fills any more (every wave's copies
      // have landed before the first barrier)
      workgroup_barrier();
      const int region = (wave & 1) + (PW ? 0 : 2);
      f32x4 *red = reinterpret_cast<f32x4 *>(region < 2 ? g_stage0.tile[region & 1]
                                                        : g_stage1.tile[region & 1]);
      if (half) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4)
            red[(dt * 4 + v4) * 64 + lane] = f32x4{w.acc[dt][4 * v4], w.acc[dt][4 * v4 + 1],
                                                   w.acc[dt][4 * v4 + 2], w.acc[dt][4 * v4 + 3]};
      }
      wait_and_barrier<kLgkm0>();
      if (half) continue;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const f32x4 o = red[(dt * 4 + v4) * 64 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) w.acc[dt][4 * v4 + e] += o[e];
        }
    }
    // epilogue: C layout lane = key l32, register v -> d = 32dt + (v/4)*8 + 4hh + v%4; the
    // P wave writes dV (P carried 2^10), the dS wave dK (times the softmax scale)
    if (!active) continue;
    const int token = perm[(size_t)h * N + key0 + l32];
    uint16_t *orow = (PW ? dv : dk) + ((size_t)token * heads + h) * dio;
    // any status flag of the head (operand range, selection overflow, dS bound): NaN
    const bool poisoned = flags[h] != 0u;
    const float mul = PW ? 1.f / kPScale : scale;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int d0 = 32 * dt + 8 * v4 + 4 * hh;
        const f32x16 &A = w.acc[dt];
        uint32_t x0 = (uint32_t)f32_to_bf16(A[4 * v4] * mul) |
                      ((uint32_t)f32_to_bf16(A[4 * v4 + 1] * mul) << 16);
        uint32_t x1 = (uint32_t)f32_to_bf16(A[4 * v4 + 2] * mul) |
                      ((uint32_t)f32_to_bf16(A[4 * v4 + 3] * mul) << 16);
        if (poisoned) x0 = x1 = kNaNbf16x2;
        if (32 * dt < dio) *reinterpret_cast<u32x2 *>(orow + d0) = u32x2{x0, x1};
      }
  }
}

// The kernel of the 128-key tiles (SPLIT false) and that of the 64-key tiles (SPLIT true);
// the two roles run the same sequence of barriers and copies
template <bool SPLIT>
__device__ __forceinline__ void dkdv_body(
    int N, int U, int nb_max, int heads, const int2 *__restrict__ tiles,
    const int *__restrict__ tile_count, const uint16_t *__restrict__ qp,
    const uint16_t *__restrict__ kp, const uint16_t *__restrict__ vp,
    const uint16_t *__restrict__ dop, const float *__restrict__ lse2,
    const float *__restrict__ ndelta, const int *__restrict__ unit_blk,
    const int *__restrict__ blk_start, const int *__restrict__ blk_size,
    const int *__restrict__ csc_count, const int *__restrict__ csc_ptr,
    const int *__restrict__ csc_row, long long cap, const int *__restrict__ perm, float scale,
    float scale_log2e, int dio, const uint32_t *__restrict__ flags, uint16_t *__restrict__ dk,
    uint16_t *__restrict__ dv) {
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int ntiles = SPLIT ? tile_count[3] : *tile_count;
  if (wave < 4)
    dkdv_waves<true, SPLIT>(wave, lane, N, U, nb_max, heads, tiles, tile_count, ntiles, qp,
                            kp, vp, dop, lse2, ndelta, unit_blk, blk_start, blk_size,
                            csc_count, csc_ptr, csc_row, cap, perm, scale, scale_log2e, dio,
                            flags, dk, dv);
  else
    dkdv_waves<false, SPLIT>(wave, lane, N, U, nb_max, heads, tiles, tile_count, ntiles, qp,
                             kp, vp, dop, lse2, ndelta, unit_blk, blk_start, blk_size,
                             csc_count, csc_ptr, csc_row, cap, perm, scale, scale_log2e, dio,
                             flags, dk, dv);
}

#define PRISM_DKDV_PARAMS                                                                    \
  int N, int U, int nb_max, int heads, const int2 *__restrict__ tiles,                       \
      const int *__restrict__ tile_count, const uint16_t *__restrict__ qp,                   \
      const uint16_t *__restrict__ kp, const uint16_t *__restrict__ vp,                      \
      const uint16_t *__restrict__ dop, const float *__restrict__ lse2,                      \
      const float *__restrict__ ndelta, const int *__restrict__ unit_blk,                    \
      const int *__restrict__ blk_start, const int *__restrict__ blk_size,                   \
      const int *__restrict__ csc_count, const int *__restrict__ csc_ptr,                    \
      const int *__restrict__ csc_row, long long cap, const int *__restrict__ perm,          \
      float scale, float scale_log2e, int dio, const uint32_t *__restrict__ flags,           \
      uint16_t *__restrict__ dk, uint16_t *__restrict__ dv
#define PRISM_DKDV_ARGS                                                                      \
  N, U, nb_max, heads, tiles, tile_count, qp, kp, vp, dop, lse2, ndelta, unit_blk,           \
      blk_start, blk_size, csc_count, csc_ptr, csc_row, cap, perm, scale, scale_log2e, dio,  \
      flags, dk, dv

__global__ void __launch_bounds__(NW * 64) attn_dkdv_bf16_kernel(PRISM_DKDV_PARAMS) {
  dkdv_body<false>(PRISM_DKDV_ARGS);
}
__global__ void __launch_bounds__(NW * 64) attn_dkdv64_bf16_kernel(PRISM_DKDV_PARAMS) {
  dkdv_body<true>(PRISM_DKDV_ARGS);
}

// The 128-key tiles, then the 64-key tiles (each launch persistent over its part of the
// list; the second exits at once when there are none)
hipError_t launch_dkdv_bf16(int work_items, hipStream_t s, int N, int U, int nb_max, int heads,
                            const int2 *tiles, const int *counters, const uint16_t *qp,
                            const uint16_t *kp, const uint16_t *vp, const uint16_t *dop,
                            const float *lse2, const float *ndelta, const int *unit_blk,
                            const int *bstart, const int *bsize, const int *tcnt,
                            const int *tptr, const int *trows, long long cap, const int *perm,
                            float scale, float sl2e, int dio, const uint32_t *flags,
                            uint16_t *dk, uint16_t *dv) {
  const int grid = resident_grid((const void *)attn_dkdv_bf16_kernel, NW * 64, work_items);
  hipLaunchKernelGGL(attn_dkdv_bf16_kernel, dim3(grid), dim3(NW * 64), 0, s, N, U, nb_max,
                     heads, tiles, counters, qp, kp, vp, dop, lse2, ndelta, unit_blk, bstart,
                     bsize, tcnt, tptr, trows, cap, perm, scale, sl2e, dio, flags, dk, dv);
  const int grid64 = resident_grid((const void *)attn_dkdv64_bf16_kernel, NW * 64, work_items);
  hipLaunchKernelGGL(attn_dkdv64_bf16_kernel, dim3(grid64), dim3(NW * 64), 0, s, N, U, nb_max,
                     heads, tiles, counters, qp, kp, vp, dop, lse2, ndelta, unit_blk, bstart,
                     bsize, tcnt, tptr, trows, cap, perm, scale, sl2e, dio, flags, dk, dv);
  return hipGetLastError();
}

#undef PRISM_DKDV_PARAMS
#undef PRISM_DKDV_ARGS

}  // namespace prism
