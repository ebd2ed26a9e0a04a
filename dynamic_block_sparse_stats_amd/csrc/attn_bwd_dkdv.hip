// attn_bwd_dkdv.hip -- dK and dV of the block-sparse attention (bfloat16 path), key-major
// over the transposed selection lists.  Same method as attn_bwd.hip (digest, training
// section: the plan is constant; gradients flow only through the selected blocks), in a
// translation unit of its own because its register budget (K and V rows plus the dK and
// dV accumulators of 32 keys per wave) is best served by the default MFMA register form.
#include "prism_internal.h"

namespace prism {

namespace {
constexpr int kDB = 128;

__device__ __forceinline__ int rm_off(int r, int c) {  // [64][128] bf16 tile, 16 chunks/row
  return r * 256 + ((c ^ (r & 15)) << 4);
}
__device__ __forceinline__ int tr_off(int d, int c) {  // [128][64] f16 tile, 8 chunks/row
  return d * 128 + ((c ^ ((d >> 1) & 7)) << 4);
}
}  // namespace

// ============================================================================ dK / dV (bf16)
// One workgroup of four waves per key tile; each wave owns 32 keys (its K and V rows are
// the B operands, held in registers) and accumulates dK^T and dV^T over the 64-token
// query units of every query block that selected the key block.  A 64-key tile leaves
// waves 2-3 idle in the arithmetic.
//
// Query units stream through a two-stage LDS ring filled by direct global->LDS copies
// (global_load_lds_dwordx4: lane l of one instruction lands at +16*l, so the XOR swizzle
// is applied by choosing which source chunk each lane fetches).  Per stage: Q and dO
// row-major [64][128] bf16, Q^T and dO^T [128][64] f16, lse and delta [64].  Each wave
// copies one of the four tiles (16 instructions) and one 256-byte vector, so every wave
// has the same number of copies in flight; the copy of the next unit is issued right after
// the barrier that publishes the current one and overlaps its 64 MFMAs.
constexpr int NW = 4;

// The two stages are distinct LDS objects and the unit loop is unrolled by two, so every
// LDS read names its stage statically; the compiler can then see that the copies in flight
// (into the other stage) do not feed the reads, and issues no wait for them.
struct Stage {
  uint8_t tile[4][16384];  // Q, dO (row-major bf16), Q^T, dO^T (f16)
  float vec[4][kUnit];     // lse * log2(e) - 10, -delta * 2^-10, unused, unused
};
__shared__ __align__(16) Stage g_stage0;
__shared__ __align__(16) Stage g_stage1;
template <int S>
__device__ __forceinline__ Stage &stage() {
  return S ? g_stage1 : g_stage0;
}

struct DkdvState {
  bf16x8 kreg[8], vreg[8];
  f32x16 dkt[4], dvt[4];
};

template <int S>
__device__ __forceinline__ void dkdv_unit(DkdvState &w, int l32, int hh, float scale_log2e) {
  const Stage &sg = stage<S>();
  f16x8 pb[4], db[4];
#pragma unroll
  for (int a = 0; a < 2; ++a) {  // queries 32a .. 32a + 31 of the unit
    const int r = 32 * a + l32;
    bf16x8 qa[8], da[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      qa[kk] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4 *>(sg.tile[0] + rm_off(r, 2 * kk + hh)));
      da[kk] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4 *>(sg.tile[1] + rm_off(r, 2 * kk + hh)));
    }
    // per query row of the C layout: lse * log2(e) - 10 and -delta * 2^-10
    f32x4 l4[4], d4[4];
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const int q0 = 32 * a + 8 * v4 + 4 * hh;
      l4[v4] = *reinterpret_cast<const f32x4 *>(sg.vec[0] + q0);
      d4[v4] = *reinterpret_cast<const f32x4 *>(sg.vec[1] + q0);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs below
    f32x16 sacc = f32x16{}, dp;
#pragma unroll
    for (int v = 0; v < 16; ++v) dp[v] = d4[v >> 2][v & 3];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      sacc = mfma_bf16(qa[kk], w.kreg[kk], sacc);
      dp = mfma_bf16(da[kk], w.vreg[kk], dp);
    }
    // C layout: lane = key l32, register v = query 32a + (v/4)*8 + 4hh + v%4;  p is
    // P * 2^10 and dp is (dP - delta) * 2^-10
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sacc[v], scale_log2e, -l4[v >> 2][v & 3]));
      const int g = 2 * a + (v >> 3), slot = v & 7;
      pb[g][slot] = (_Float16)p;
      db[g][slot] = (_Float16)(p * dp[v]);
    }
  }
  // dV^T[d][key] += dO^T[d][q] P[q][key];  dK^T[d][key] += Q^T[d][q] dS[q][key]
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int d = 32 * dt + l32;
    f16x8 doa[4], qta[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      doa[g] = __builtin_bit_cast(
          f16x8, *reinterpret_cast<const u32x4 *>(sg.tile[3] + tr_off(d, 2 * g + hh)));
      qta[g] = __builtin_bit_cast(
          f16x8, *reinterpret_cast<const u32x4 *>(sg.tile[2] + tr_off(d, 2 * g + hh)));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      w.dvt[dt] = mfma_f16(doa[g], pb[g], w.dvt[dt]);
      w.dkt[dt] = mfma_f16(qta[g], db[g], w.dkt[dt]);
    }
  }
}

__global__ void __launch_bounds__(NW * 64)
    attn_dkdv_bf16_kernel(int N, int U, int nb_max, int heads, const int2 *__restrict__ tiles,
                          const int *__restrict__ tile_count, const uint16_t *__restrict__ qp,
                          const uint16_t *__restrict__ qpt, const uint16_t *__restrict__ kp,
                          const uint16_t *__restrict__ vp, const uint16_t *__restrict__ dop,
                          const uint16_t *__restrict__ dopt, const float *__restrict__ lse2,
                          const float *__restrict__ delta, const int *__restrict__ unit_blk,
                          const int *__restrict__ blk_start, const int *__restrict__ blk_size,
                          const int *__restrict__ csc_count, const int *__restrict__ csc_row,
                          const int *__restrict__ perm, float scale, float scale_log2e,
                          uint16_t *__restrict__ dk, uint16_t *__restrict__ dv) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int ntiles = *tile_count;
  const uint8_t *tsrc = reinterpret_cast<const uint8_t *>(
      wave == 0 ? qp : (wave == 1 ? dop : (wave == 2 ? qpt : dopt)));
  const float *vsrc = wave == 1 ? delta : lse2;
  // this lane's byte offset inside copy i (1 KB) of its wave's tile: rows 4i.. (row-major
  // tiles) or 8i.. (transposed tiles); the swizzle only depends on the row within 16 / 8
  auto lofs = [&](int i) {
    if (wave < 2) {
      const int r = 4 * i + (lane >> 4);
      return r * 256 + (((lane & 15) ^ (r & 15)) << 4);
    }
    const int d = 8 * i + (lane >> 3);
    return d * 128 + (((lane & 7) ^ ((d >> 1) & 7)) << 4);
  };

  for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int2 tl = tiles[t];
    const int h = tl.x, u0 = tl.y & (kTile64 - 1);
    const bool active = !(tl.y & kTile64) || wave < 2;
    const int jblk = unit_blk[(size_t)h * U + u0];
    const int nq = csc_count[(size_t)h * nb_max + jblk];
    const int *qlist = csc_row + ((size_t)h * nb_max + jblk) * nb_max;
    const int *bs = blk_start + (size_t)h * nb_max, *bz = blk_size + (size_t)h * nb_max;
    // this wave's 32 keys: K^T and V^T as B operands (lane = key, 8 dims per k-step)
    const int key0 = u0 * kUnit + wave * 32;
    DkdvState w;
    if (active) {
      const uint16_t *kr = kp + ((size_t)h * N + key0 + l32) * kDB + 8 * hh;
      const uint16_t *vr = vp + ((size_t)h * N + key0 + l32) * kDB + 8 * hh;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        w.kreg[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(kr + 16 * kk));
        w.vreg[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(vr + 16 * kk));
      }
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) w.dkt[dt] = w.dvt[dt] = f32x16{};

    const size_t hb = (size_t)h * N;
    auto issue0 = [&](int u) {
      const uint8_t *src = tsrc + (hb + (size_t)u * kUnit) * kDB * 2;
#pragma unroll
      for (int i = 0; i < 16; ++i) dma16(src + lofs(i), g_stage0.tile[wave] + 1024 * i);
      dma4(vsrc + hb + (size_t)u * kUnit + lane, g_stage0.vec[wave]);
    };
    auto issue1 = [&](int u) {
      const uint8_t *src = tsrc + (hb + (size_t)u * kUnit) * kDB * 2;
#pragma unroll
      for (int i = 0; i < 16; ++i) dma16(src + lofs(i), g_stage1.tile[wave] + 1024 * i);
      dma4(vsrc + hb + (size_t)u * kUnit + lane, g_stage1.vec[wave]);
    };

    __builtin_amdgcn_s_barrier();  // every wave is done with the previous tile's stages
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (nq > 0) {
      BlockUnits cur;
      cur.init(qlist, nq, bs, bz, lane);
      issue0(cur.unit());
      while (true) {
        bool more = cur.next();
        wait_copies_and_sync();  // stage 0 has landed everywhere; stage 1 is free
        if (more) issue1(cur.unit());
        if (active) dkdv_unit<0>(w, l32, hh, scale_log2e);
        if (!more) break;
        more = cur.next();
        wait_copies_and_sync();  // stage 1 has landed everywhere; stage 0 is free
        if (more) issue0(cur.unit());
        if (active) dkdv_unit<1>(w, l32, hh, scale_log2e);
        if (!more) break;
      }
    }
    // epilogue: C layout lane = key l32, register v -> d = 32dt + (v/4)*8 + 4hh + v%4
    if (!active) continue;
    const int token = perm[(size_t)h * N + key0 + l32];
    uint16_t *krow = dk + ((size_t)token * heads + h) * kDB;
    uint16_t *vrow = dv + ((size_t)token * heads + h) * kDB;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int d0 = 32 * dt + 8 * v4 + 4 * hh;
        const f32x16 &K = w.dkt[dt], &V = w.dvt[dt];
        uint32_t k0 = (uint32_t)f32_to_bf16(K[4 * v4] * scale) |
                      ((uint32_t)f32_to_bf16(K[4 * v4 + 1] * scale) << 16);
        uint32_t k1 = (uint32_t)f32_to_bf16(K[4 * v4 + 2] * scale) |
                      ((uint32_t)f32_to_bf16(K[4 * v4 + 3] * scale) << 16);
        const float vs = 1.f / kPScale;
        uint32_t w0 = (uint32_t)f32_to_bf16(V[4 * v4] * vs) |
                      ((uint32_t)f32_to_bf16(V[4 * v4 + 1] * vs) << 16);
        uint32_t w1 = (uint32_t)f32_to_bf16(V[4 * v4 + 2] * vs) |
                      ((uint32_t)f32_to_bf16(V[4 * v4 + 3] * vs) << 16);
        *reinterpret_cast<u32x2 *>(krow + d0) = u32x2{k0, k1};
        *reinterpret_cast<u32x2 *>(vrow + d0) = u32x2{w0, w1};
      }
  }
}

hipError_t launch_dkdv_bf16(int work_items, hipStream_t s, int N, int U, int nb_max, int heads,
                            const int2 *tiles, const int *counters, const uint16_t *qp,
                            const uint16_t *qpt, const uint16_t *kp, const uint16_t *vp,
                            const uint16_t *dop, const uint16_t *dopt, const float *lse2,
                            const float *delta, const int *unit_blk, const int *bstart,
                            const int *bsize, const int *tcnt, const int *trows,
                            const int *perm, float scale, float sl2e, uint16_t *dk,
                            uint16_t *dv) {
  const int grid = resident_grid((const void *)attn_dkdv_bf16_kernel, NW * 64, work_items);
  hipLaunchKernelGGL(attn_dkdv_bf16_kernel, dim3(grid), dim3(NW * 64), 0, s, N, U, nb_max,
                     heads, tiles, counters, qp, qpt, kp, vp, dop, dopt, lse2, delta, unit_blk,
                     bstart, bsize, tcnt, trows, perm, scale, sl2e, dk, dv);
  return hipGetLastError();
}

}  // namespace prism
