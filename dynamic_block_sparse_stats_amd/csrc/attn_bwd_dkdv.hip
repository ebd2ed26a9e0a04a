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
// Four waves per workgroup; a 64-key tile (a 64-token block) leaves waves 2-3 to help stage
// the query units only.
constexpr int NW = 4;

__global__ void __launch_bounds__(NW * 64)
    attn_dkdv_bf16_kernel(int N, int U, int nb_max, int heads, const int2 *__restrict__ tiles,
                          const int *__restrict__ tile_count, const uint16_t *__restrict__ qp,
                          const uint16_t *__restrict__ qpt, const uint16_t *__restrict__ kp,
                          const uint16_t *__restrict__ vp, const uint16_t *__restrict__ dop,
                          const uint16_t *__restrict__ dopt, const float *__restrict__ lsep,
                          const float *__restrict__ delta, const int *__restrict__ unit_blk,
                          const int *__restrict__ blk_start, const int *__restrict__ blk_size,
                          const int *__restrict__ csc_count, const int *__restrict__ csc_row,
                          const int *__restrict__ perm, float scale, float scale_log2e,
                          uint16_t *__restrict__ dk, uint16_t *__restrict__ dv) {
  constexpr int NT = NW * 64;
  constexpr int CPT = 1024 / NT;
  __shared__ __align__(16) uint8_t lds[4][16384];  // Q, dO (row-major), Q^T, dO^T
  __shared__ __align__(16) float lsd[2][kUnit];    // lse * log2(e), delta of the unit
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int ntiles = *tile_count;
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
    bf16x8 kreg[8], vreg[8];
    if (active) {
      const uint16_t *kr = kp + ((size_t)h * N + key0 + l32) * kDB + 8 * hh;
      const uint16_t *vr = vp + ((size_t)h * N + key0 + l32) * kDB + 8 * hh;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        kreg[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(kr + 16 * kk));
        vreg[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(vr + 16 * kk));
      }
    }
    f32x16 dkt[4], dvt[4];  // [d][key] accumulators, 4 tiles of 32 dims
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) dkt[dt] = dvt[dt] = f32x16{};

    for (int qi = 0; qi < nq; ++qi) {
      const int iblk = qlist[qi];
      const int us = bs[iblk] / kUnit, nu = bz[iblk] / kUnit;
      for (int u = us; u < us + nu; ++u) {
        __syncthreads();
        const size_t ub = ((size_t)h * N + (size_t)u * kUnit) * kDB * 2;  // bytes
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
          const int q = tid + NT * e;
          const uint8_t *g0 = reinterpret_cast<const uint8_t *>(qp) + ub + 16 * q;
          const uint8_t *g1 = reinterpret_cast<const uint8_t *>(dop) + ub + 16 * q;
          const uint8_t *g2 = reinterpret_cast<const uint8_t *>(qpt) + ub + 16 * q;
          const uint8_t *g3 = reinterpret_cast<const uint8_t *>(dopt) + ub + 16 * q;
          *reinterpret_cast<u32x4 *>(&lds[0][rm_off(q >> 4, q & 15)]) =
              *reinterpret_cast<const u32x4 *>(g0);
          *reinterpret_cast<u32x4 *>(&lds[1][rm_off(q >> 4, q & 15)]) =
              *reinterpret_cast<const u32x4 *>(g1);
          *reinterpret_cast<u32x4 *>(&lds[2][tr_off(q >> 3, q & 7)]) =
              *reinterpret_cast<const u32x4 *>(g2);
          *reinterpret_cast<u32x4 *>(&lds[3][tr_off(q >> 3, q & 7)]) =
              *reinterpret_cast<const u32x4 *>(g3);
        }
        if (tid < 2 * kUnit) {
          const size_t pr = (size_t)h * N + (size_t)u * kUnit + (tid & (kUnit - 1));
          lsd[tid >> 6][tid & (kUnit - 1)] =
              tid < kUnit ? lsep[pr] * 1.4426950408889634f : delta[pr];
        }
        __syncthreads();
        if (!active) continue;
        f16x8 pb[4], db[4];
#pragma unroll
        for (int a = 0; a < 2; ++a) {  // queries 32a .. 32a + 31 of the unit
          f32x16 s = f32x16{}, dp = f32x16{};
          const int r = 32 * a + l32;
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) {
            bf16x8 qa = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4 *>(&lds[0][rm_off(r, 2 * kk + hh)]));
            bf16x8 da = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4 *>(&lds[1][rm_off(r, 2 * kk + hh)]));
            s = mfma_bf16(qa, kreg[kk], s);
            dp = mfma_bf16(da, vreg[kk], dp);
          }
          // C layout: lane = key l32, register v = query 32a + (v/4)*8 + 4hh + v%4
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const int q0 = 32 * a + 8 * v4 + 4 * hh;
            const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&lsd[0][q0]);
            const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&lsd[1][q0]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int v = 4 * v4 + e;
              const float p = __builtin_amdgcn_exp2f(fmaf(s[v], scale_log2e, -l4[e]));
              const int g = 2 * a + (v >> 3), slot = v & 7;
              pb[g][slot] = (_Float16)(p * kPScale);
              db[g][slot] = (_Float16)(p * (dp[v] - d4[e]));
            }
          }
        }
        // dV^T[d][key] += dO^T[d][q] P[q][key];  dK^T[d][key] += Q^T[d][q] dS[q][key]
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int d = 32 * dt + l32;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f16x8 doa = __builtin_bit_cast(
                f16x8, *reinterpret_cast<const u32x4 *>(&lds[3][tr_off(d, 2 * g + hh)]));
            f16x8 qta = __builtin_bit_cast(
                f16x8, *reinterpret_cast<const u32x4 *>(&lds[2][tr_off(d, 2 * g + hh)]));
            dvt[dt] = mfma_f16(doa, pb[g], dvt[dt]);
            dkt[dt] = mfma_f16(qta, db[g], dkt[dt]);
          }
        }
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
        const f32x16 &K = dkt[dt], &V = dvt[dt];
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
                            const uint16_t *dop, const uint16_t *dopt, const float *lsep,
                            const float *delta, const int *unit_blk, const int *bstart,
                            const int *bsize, const int *tcnt, const int *trows,
                            const int *perm, float scale, float sl2e, uint16_t *dk,
                            uint16_t *dv) {
  const int grid = resident_grid((const void *)attn_dkdv_bf16_kernel, NW * 64, work_items);
  hipLaunchKernelGGL(attn_dkdv_bf16_kernel, dim3(grid), dim3(NW * 64), 0, s, N, U, nb_max,
                     heads, tiles, counters, qp, qpt, kp, vp, dop, dopt, lsep, delta, unit_blk,
                     bstart, bsize, tcnt, trows, perm, scale, sl2e, dk, dv);
  return hipGetLastError();
}

}  // namespace prism
