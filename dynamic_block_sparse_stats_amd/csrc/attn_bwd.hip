// attn_bwd.hip -- gradients of the block-sparse attention with the plan held constant
// (arXiv 2610.05416; nanless digest, training section: shape assignment and block
// selection are constants that pass no gradient; gradients flow only through the sparse
// attention over the selected blocks).
//
// With P_xy = exp(scale q_x.k_y - lse_x) over the key tokens y of the blocks selected for
// x's block, delta_x = do_x.o_x and dS_xy = P_xy (do_x.v_y - delta_x):
//   dv_y = sum_x P_xy do_x,  dk_y = scale sum_x dS_xy q_x,  dq_x = scale sum_y dS_xy k_y.
// Three passes, none with atomics (results are bit-reproducible):
//   prep  -- gathers dO into the permuted layout (row-major and per-unit transposed) and
//            forms delta from the float32 output the forward kept;  for bfloat16 it also
//            folds the constants of the two MFMA passes into their inputs: the row-major dO
//            copy is scaled by 2^-10 and delta stored as -delta * 2^-10 (so the dP
//            accumulator starts at -delta and ends at (dP - delta) * 2^-10), and lse is
//            stored as lse * log2(e) - 10 (so the exp2 gives P * 2^10 directly);
//   dK/dV -- one workgroup per key tile (32 keys per wave, K and V rows held in registers),
//            streaming the 64-token query units of every query block that selected the
//            key block (the transposed selection lists);
//   dQ    -- one workgroup per query tile (32 queries per wave, Q and dO in registers),
//            streaming the selected key units as in the forward pass.
// Both MFMA passes recompute P from the stored lse; the products with P and dS run on the
// float16 MFMA (P scaled by 2^10, as in the forward) against the float16 transposed copies;
// outputs go straight to the tokens' original positions.
#include "prism_internal.h"

namespace prism {

constexpr int kDB = 128;

__device__ __forceinline__ int rm_off(int r, int c) {  // [64][128] bf16 tile, 16 chunks/row
  return r * 256 + ((c ^ (r & 15)) << 4);
}
__device__ __forceinline__ int tr_off(int d, int c) {  // [128][64] bf16 tile, 8 chunks/row
  return d * 128 + ((c ^ ((d >> 1) & 7)) << 4);
}
__device__ __forceinline__ int swap23b(int e) {
  return (e & ~12) | ((e >> 1) & 4) | ((e << 1) & 8);
}

// ============================================================================ prep
template <typename T, int D, bool TRANSPOSE>
__global__ void __launch_bounds__(256)
    bwd_prep_kernel(int N, int heads, const int *__restrict__ perm, const T *__restrict__ dout,
                    const float *__restrict__ o32p, const float *__restrict__ lsep,
                    T *__restrict__ dop, T *__restrict__ dopt, float *__restrict__ delta,
                    float *__restrict__ lse2) {
  constexpr int VPC = 16 / (int)sizeof(T);
  constexpr int CH = D / VPC;
  constexpr int RG = 256 / CH;
  constexpr int RPT = kUnit / RG;
  const int u = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int c = tid % CH, rg = tid / CH;
  __shared__ __align__(16) uint16_t tile[TRANSPOSE ? kUnit * D : 8];
  const size_t tstride = (size_t)heads * D;
#pragma unroll
  for (int rr = 0; rr < RPT; ++rr) {
    const int row = rg + RG * rr;
    const size_t p = (size_t)u * kUnit + row;
    const int token = perm[(size_t)h * N + p];
    u32x4 a = *reinterpret_cast<const u32x4 *>(dout + token * tstride + (size_t)h * D + c * VPC);
    if constexpr (TRANSPOSE) {
      // dO * 2^-kPShift: an exact power-of-two scaling of each bfloat16
      u32x4 sc;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(a[e] << 16) * (1.f / kPScale);
        const float hi = __uint_as_float(a[e] & 0xffff0000u) * (1.f / kPScale);
        sc[e] = (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
      }
      *reinterpret_cast<u32x4 *>(dop + ((size_t)h * N + p) * D + c * VPC) = sc;
    } else {
      *reinterpret_cast<u32x4 *>(dop + ((size_t)h * N + p) * D + c * VPC) = a;
    }
    const float *orow = o32p + ((size_t)h * N + p) * D + c * VPC;
    float dot = 0.f;
    if constexpr (sizeof(T) == 2) {
      const f32x4 o0 = *reinterpret_cast<const f32x4 *>(orow);
      const f32x4 o1 = *reinterpret_cast<const f32x4 *>(orow + 4);
      const float ov[8] = {o0[0], o0[1], o0[2], o0[3], o1[0], o1[1], o1[2], o1[3]};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dot += __uint_as_float(a[e] << 16) * ov[2 * e];
        dot += __uint_as_float(a[e] & 0xffff0000u) * ov[2 * e + 1];
      }
    } else {
      const f32x4 o0 = *reinterpret_cast<const f32x4 *>(orow);
#pragma unroll
      for (int e = 0; e < 4; ++e) dot += __uint_as_float(a[e]) * o0[e];
    }
#pragma unroll
    for (int off = 1; off < CH; off <<= 1) dot += __shfl_xor(dot, off, 64);
    if (c == 0) {
      if constexpr (TRANSPOSE) {
        delta[(size_t)h * N + p] = -dot * (1.f / kPScale);
        lse2[(size_t)h * N + p] = lsep[(size_t)h * N + p] * 1.4426950408889634f - kPShift;
      } else {
        delta[(size_t)h * N + p] = dot;
      }
    }
    if constexpr (TRANSPOSE) *reinterpret_cast<u32x4 *>(&tile[row * D + c * VPC]) = a;
  }
  if constexpr (TRANSPOSE) {
    __syncthreads();
    const int dd = tid >> 1, half = tid & 1;
    const size_t ubase = ((size_t)h * (N / kUnit) + u) * (size_t)(D * kUnit);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      uint32_t pk[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        int pos0 = 32 * half + 8 * cc + e;
        int key0 = (pos0 & ~15) | swap23b(pos0 & 15);
        int key1 = ((pos0 + 1) & ~15) | swap23b((pos0 + 1) & 15);
        pk[e >> 1] = (uint32_t)bf16_to_f16_bits(tile[key0 * D + dd]) |
                     ((uint32_t)bf16_to_f16_bits(tile[key1 * D + dd]) << 16);
      }
      *reinterpret_cast<u32x4 *>(dopt + ubase + (size_t)dd * kUnit + 32 * half + 8 * cc) =
          u32x4{pk[0], pk[1], pk[2], pk[3]};
    }
  }
}

constexpr int NW = 4;

// ============================================================================ dQ (bf16)
// One workgroup of four waves per query tile (32 queries per wave, Q and dO rows held as B
// operands), streaming the selected key units through a two-stage LDS ring of direct
// global->LDS copies as in the forward: per stage K and V row-major [64][128] bf16 and
// K^T [128][64] f16 (48 KB); each wave issues 12 of the 48 one-kilobyte copies.
struct DqStage {
  uint8_t tile[3][16384];  // K, V, K^T
};
__shared__ __align__(16) DqStage g_dq0;
__shared__ __align__(16) DqStage g_dq1;
template <int S>
__device__ __forceinline__ const DqStage &dq_stage() {
  return S ? g_dq1 : g_dq0;
}

struct DqState {
  bf16x8 qreg[8], doreg[8];
  f32x16 acc[4];
  float lse2, ndlt;
};

template <int S>
__device__ __forceinline__ void dq_unit(DqState &w, int l32, int hh, float scale_log2e) {
  const DqStage &sg = dq_stage<S>();
  f16x8 db[4];
#pragma unroll
  for (int a = 0; a < 2; ++a) {  // keys 32a .. 32a + 31
    const int r = 32 * a + l32;
    bf16x8 ka[8], va[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      ka[kk] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4 *>(sg.tile[0] + rm_off(r, 2 * kk + hh)));
      va[kk] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4 *>(sg.tile[1] + rm_off(r, 2 * kk + hh)));
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s = f32x16{}, dp;
#pragma unroll
    for (int v = 0; v < 16; ++v) dp[v] = w.ndlt;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      s = mfma_bf16(ka[kk], w.qreg[kk], s);
      dp = mfma_bf16(va[kk], w.doreg[kk], dp);
    }
    // lane = query, register v = key 32a + (v/4)*8 + 4hh + v%4;  P * 2^10 times
    // (dP - delta) * 2^-10
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[v], scale_log2e, -w.lse2));
      db[2 * a + (v >> 3)][v & 7] = (_Float16)(p * dp[v]);
    }
  }
  // dQ^T[d][q] += K^T[d][keys] dS^T[keys][q]
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int d = 32 * dt + l32;
    f16x8 kt[4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
      kt[g] = __builtin_bit_cast(
          f16x8, *reinterpret_cast<const u32x4 *>(sg.tile[2] + tr_off(d, 2 * g + hh)));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < 4; ++g) w.acc[dt] = mfma_f16(kt[g], db[g], w.acc[dt]);
  }
}

__global__ void __launch_bounds__(NW * 64)
    attn_dq_bf16_kernel(int N, int U, int nb_max, int heads, const int2 *__restrict__ tiles,
                        const int *__restrict__ tile_count, const uint16_t *__restrict__ qp,
                        const uint16_t *__restrict__ kp, const uint16_t *__restrict__ kpt,
                        const uint16_t *__restrict__ vp, const uint16_t *__restrict__ dop,
                        const float *__restrict__ lse2, const float *__restrict__ ndelta,
                        const int *__restrict__ unit_blk, const int *__restrict__ blk_start,
                        const int *__restrict__ blk_size, const int *__restrict__ sel_count,
                        const int *__restrict__ csr_col, const int *__restrict__ perm,
                        float scale, float scale_log2e, uint16_t *__restrict__ dq) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int ntiles = *tile_count;
  // copy j in 12*wave .. 12*wave + 11 of [K (16), V (16), K^T (16)] one-kilobyte copies
  auto csrc_of = [&](int j) -> const uint8_t * {
    const int tsel = j >> 4;
    return reinterpret_cast<const uint8_t *>(tsel == 0 ? kp : (tsel == 1 ? vp : kpt));
  };
  auto cofs = [&](int j) {
    const int i = j & 15;
    if (j < 32) {
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
    const int blk = unit_blk[(size_t)h * U + u0];
    const int *bs = blk_start + (size_t)h * nb_max, *bz = blk_size + (size_t)h * nb_max;
    BlockUnits cur;
    cur.init(csr_col + ((size_t)h * nb_max + blk) * nb_max,
             sel_count[(size_t)h * nb_max + blk], bs, bz, lane);
    const int row0 = u0 * kUnit + wave * 32;
    DqState w;
    w.lse2 = 0.f;
    w.ndlt = 0.f;
    if (active) {
      const uint16_t *qr = qp + ((size_t)h * N + row0 + l32) * kDB + 8 * hh;
      const uint16_t *dr = dop + ((size_t)h * N + row0 + l32) * kDB + 8 * hh;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        w.qreg[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(qr + 16 * kk));
        w.doreg[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(dr + 16 * kk));
      }
      w.lse2 = lse2[(size_t)h * N + row0 + l32];
      w.ndlt = ndelta[(size_t)h * N + row0 + l32];
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) w.acc[dt] = f32x16{};

    const size_t hb = (size_t)h * N * kDB * 2;
    auto issue0 = [&](int u) {
#pragma unroll
      for (int e = 0; e < 12; ++e) {
        const int j = 12 * wave + e;
        dma16(csrc_of(j) + hb + (size_t)u * kUnit * kDB * 2 + cofs(j),
              g_dq0.tile[j >> 4] + 1024 * (j & 15));
      }
    };
    auto issue1 = [&](int u) {
#pragma unroll
      for (int e = 0; e < 12; ++e) {
        const int j = 12 * wave + e;
        dma16(csrc_of(j) + hb + (size_t)u * kUnit * kDB * 2 + cofs(j),
              g_dq1.tile[j >> 4] + 1024 * (j & 15));
      }
    };

    __builtin_amdgcn_s_barrier();  // every wave is done with the previous tile's stages
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    issue0(cur.unit());
    while (true) {
      bool more = cur.next();
      wait_copies_and_sync();
      if (more) issue1(cur.unit());
      if (active) dq_unit<0>(w, l32, hh, scale_log2e);
      if (!more) break;
      more = cur.next();
      wait_copies_and_sync();
      if (more) issue0(cur.unit());
      if (active) dq_unit<1>(w, l32, hh, scale_log2e);
      if (!more) break;
    }
    if (!active) continue;
    const int token = perm[(size_t)h * N + row0 + l32];
    uint16_t *qrow = dq + ((size_t)token * heads + h) * kDB;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int d0 = 32 * dt + 8 * v4 + 4 * hh;
        uint32_t lo = (uint32_t)f32_to_bf16(w.acc[dt][4 * v4] * scale) |
                      ((uint32_t)f32_to_bf16(w.acc[dt][4 * v4 + 1] * scale) << 16);
        uint32_t hi = (uint32_t)f32_to_bf16(w.acc[dt][4 * v4 + 2] * scale) |
                      ((uint32_t)f32_to_bf16(w.acc[dt][4 * v4 + 3] * scale) << 16);
        *reinterpret_cast<u32x2 *>(qrow + d0) = u32x2{lo, hi};
      }
  }
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
                       const int *__restrict__ sel_count, const int *__restrict__ csr_col,
                       const int *__restrict__ perm, float scale, float *__restrict__ dq) {
  constexpr int DP = D / 4;
  __shared__ float ks[kUnit][D], vs[kUnit][D];
  const int u0 = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int r = tid >> 2, part = tid & 3;
  const int blk = unit_blk[(size_t)h * U + u0];
  const int ncols = sel_count[(size_t)h * nb_max + blk];
  const int *cols = csr_col + ((size_t)h * nb_max + blk) * nb_max;
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
#pragma unroll
  for (int e = 0; e < DP; ++e)
    dq[((size_t)token * heads + h) * D + part * DP + e] = (float)(acc[e] * scale);
}

// dK/dV: one workgroup per 64-key unit, 4 threads per key row, over the transposed lists.
template <int D>
__global__ void __launch_bounds__(256)
    attn_dkdv_f32_kernel(int N, int U, int nb_max, int heads, const float *__restrict__ qp,
                         const float *__restrict__ kp, const float *__restrict__ vp,
                         const float *__restrict__ dop, const float *__restrict__ lsep,
                         const float *__restrict__ delta, const int *__restrict__ unit_blk,
                         const int *__restrict__ blk_start, const int *__restrict__ blk_size,
                         const int *__restrict__ csc_count, const int *__restrict__ csc_row,
                         const int *__restrict__ perm, float scale, float *__restrict__ dk,
                         float *__restrict__ dv) {
  constexpr int DP = D / 4;
  __shared__ float qs[kUnit][D], ds_[kUnit][D];
  const int u0 = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int r = tid >> 2, part = tid & 3;
  const int jblk = unit_blk[(size_t)h * U + u0];
  const int nq = csc_count[(size_t)h * nb_max + jblk];
  const int *qlist = csc_row + ((size_t)h * nb_max + jblk) * nb_max;
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
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    dk[((size_t)token * heads + h) * D + part * DP + e] = (float)(gk[e] * scale);
    dv[((size_t)token * heads + h) * D + part * DP + e] = (float)gv[e];
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
  const int *cols = (const int *)(ws + L.pub.csr_col);
  const int *tcnt = (const int *)(ws + L.pub.csc_count);
  const int *trows = (const int *)(ws + L.pub.csc_row);
  float *delta = (float *)(ws + L.delta), *lse2 = (float *)(ws + L.lse2);
  const float *lsep = (const float *)(ws + L.lsep), *o32p = (const float *)(ws + L.o32p);
  dim3 ugrid(d.U, d.heads);
  if (d.dtype == PRISM_BF16) {
    typedef uint16_t T;
    {
      TraceScope tr(PRISM_STAGE_BWD_PREP, s);
      hipLaunchKernelGGL((bwd_prep_kernel<T, 128, true>), ugrid, dim3(256), 0, s, d.N, d.heads,
                       perm, (const T *)dout, o32p, lsep, (T *)(ws + L.dop),
                       (T *)(ws + L.dopt), delta, lse2);
    }
    const int *counters = (const int *)(ws + L.counters);
    const float sl2e = scale * 1.4426950408889634f;
    const int maxt = d.heads * d.U;
    const T *qp = (const T *)(ws + L.qp), *kp = (const T *)(ws + L.kp),
            *vp = (const T *)(ws + L.vp), *qpt = (const T *)(ws + L.qpt),
            *kpt = (const T *)(ws + L.kpt), *dop = (const T *)(ws + L.dop),
            *dopt = (const T *)(ws + L.dopt);
    const int2 *tiles = (const int2 *)(ws + L.tiles);
    {
      TraceScope tr(PRISM_STAGE_BWD_DKDV, s);
      launch_dkdv_bf16(maxt, s, d.N, d.U, d.nb_max, d.heads, tiles, counters, qp, qpt, kp, vp,
                       dop, dopt, lse2, delta, unit_blk, bstart, bsize, tcnt, trows, perm, scale,
                       sl2e, (T *)dk, (T *)dv);
    }
    {
      TraceScope tr(PRISM_STAGE_BWD_DQ, s);
      const int grid = resident_grid((const void *)attn_dq_bf16_kernel, NW * 64, maxt);
      hipLaunchKernelGGL(attn_dq_bf16_kernel, dim3(grid), dim3(NW * 64), 0, s, d.N, d.U,
                         d.nb_max, d.heads, tiles, counters, qp, kp, kpt, vp, dop, lse2, delta,
                         unit_blk, bstart, bsize, cnt, cols, perm, scale, sl2e, (T *)dq);
    }
  } else {
    typedef float T;
    TraceScope tr(PRISM_STAGE_BWD_DKDV, s);
    const T *qp = (const T *)(ws + L.qp), *kp = (const T *)(ws + L.kp),
            *vp = (const T *)(ws + L.vp), *dop = (const T *)(ws + L.dop);
    if (d.D == 64) {
      hipLaunchKernelGGL((bwd_prep_kernel<T, 64, false>), ugrid, dim3(256), 0, s, d.N, d.heads,
                         perm, (const T *)dout, o32p, lsep, (T *)(ws + L.dop), nullptr, delta,
                         nullptr);
      hipLaunchKernelGGL((attn_dq_f32_kernel<64>), ugrid, dim3(256), 0, s, d.N, d.U, d.nb_max,
                         d.heads, qp, kp, vp, dop, lsep, delta, unit_blk, bstart, bsize, cnt,
                         cols, perm, scale, (T *)dq);
      hipLaunchKernelGGL((attn_dkdv_f32_kernel<64>), ugrid, dim3(256), 0, s, d.N, d.U,
                         d.nb_max, d.heads, qp, kp, vp, dop, lsep, delta, unit_blk, bstart,
                         bsize, tcnt, trows, perm, scale, (T *)dk, (T *)dv);
    } else {
      hipLaunchKernelGGL((bwd_prep_kernel<T, 128, false>), ugrid, dim3(256), 0, s, d.N,
                         d.heads, perm, (const T *)dout, o32p, lsep, (T *)(ws + L.dop),
                         nullptr, delta, nullptr);
      hipLaunchKernelGGL((attn_dq_f32_kernel<128>), ugrid, dim3(256), 0, s, d.N, d.U, d.nb_max,
                         d.heads, qp, kp, vp, dop, lsep, delta, unit_blk, bstart, bsize, cnt,
                         cols, perm, scale, (T *)dq);
      hipLaunchKernelGGL((attn_dkdv_f32_kernel<128>), ugrid, dim3(256), 0, s, d.N, d.U,
                         d.nb_max, d.heads, qp, kp, vp, dop, lsep, delta, unit_blk, bstart,
                         bsize, tcnt, trows, perm, scale, (T *)dk, (T *)dv);
    }
  }
  return hipGetLastError();
}

}  // namespace prism
